"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check
that the pin suite notices every one of them."""
import importlib.util
import os
import types

import pytest

from tests import pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "lora.py")

MUTATIONS = {
    "drop_scale_fwd": ("Y[r0:r1] = Xc @ W + s * (Zc @ Bi)", "Y[r0:r1] = Xc @ W + (Zc @ Bi)"),
    "sign_fwd": ("Y[r0:r1] = Xc @ W + s * (Zc @ Bi)", "Y[r0:r1] = Xc @ W - s * (Zc @ Bi)"),
    "drop_base_fwd": ("Y[r0:r1] = Xc @ W + s * (Zc @ Bi)", "Y[r0:r1] = s * (Zc @ Bi)"),
    "drop_scale_dz": ("dZc = s * (dYc @ Bi.T)", "dZc = (dYc @ Bi.T)"),
    "drop_lora_dx": ("dX[r0:r1] = dYc @ W.T + dZc @ Ai.T", "dX[r0:r1] = dYc @ W.T"),
    "double_scale_dx": ("dX[r0:r1] = dYc @ W.T + dZc @ Ai.T", "dX[r0:r1] = dYc @ W.T + s * (dZc @ Ai.T)"),
    "drop_scale_db": ("gB += s * (Zc.T @ dYc)", "gB += (Zc.T @ dYc)"),
    "double_scale_da": ("gA += Xc.T @ dZc", "gA += s * (Xc.T @ dZc)"),
    "db_from_x": ("gB += s * (Zc.T @ dYc)", "gB += s * ((Xc @ Ai).T @ (Xc @ W))"),
    "segment_shift": ("return [(o[i], o[i + 1]) for i in range(len(o) - 1)]",
                      "return [(o[i] + (1 if 0 < i else 0), o[i + 1]) for i in range(len(o) - 1)]"),
    "wrong_adapter_B": ("Bi = as_f64(B[i], dtype)\n        s = float(scales[i])\n        Zi",
                        "Bi = as_f64(B[i - 1] if B[i - 1].shape == B[i].shape else B[i], dtype)\n"
                        "        s = float(scales[i])\n        Zi"),
    "wrong_scale_index": ("s = float(scales[i])\n        Zi", "s = float(scales[0])\n        Zi"),
    "bf16_decode_shift": ("<< np.uint32(16)", "<< np.uint32(15)"),
    "proj_da_drop_scale": ("out_a.append(s * ga)", "out_a.append(ga)"),
    "proj_db_wrong_vector": ("gb += Xc.T @ (Gc @ v)", "gb += Xc.T @ (Gc @ bu)"),
    "proj_chunk_tail_lost": ("            r1 = min(hi, r0 + chunk)\n            Xc = as_f64(X[r0:r1], dtype)\n            Gc",
                             "            r1 = min(hi - 1, r0 + chunk)\n            Xc = as_f64(X[r0:r1], dtype)\n            Gc"),
    "sampled_z_no_scale": ("zi = s * (x @ Ai)", "zi = (x @ Ai)"),
    "ids_unstable_sort": ('perm = np.argsort(ids, kind="stable")', 'perm = np.argsort(-ids, kind="stable")[::-1]'),
    "ids_offsets_shift": ("offsets[1:] = np.cumsum(np.bincount(ids, minlength=n))",
                          "offsets[1:] = np.cumsum(np.bincount(ids, minlength=n)) - 1"),
    "ids_y_not_unpermuted": ("    Y = np.empty_like(Yg)\n    Y[perm] = Yg", "    Y = np.empty_like(Yg)\n    Y[:] = Yg"),
    "ids_dx_wrong_inverse": ("        dX[perm] = dXg", "        dX[:] = dXg[perm]"),
}


def _mutant(old, new) -> types.ModuleType:
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new, 1)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name):
    old, new = MUTATIONS[name]
    mod = _mutant(old, new)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # AssertionError or a shape error both mean "caught"
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught mutation {name}"
