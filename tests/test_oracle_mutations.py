"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check
that the pin suite notices every one of them."""
import importlib.util
import os
import sys
import types

import pytest

from tests import pins, pins_adamw, pins_multi, pins_mx, pins_plan

ORACLE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")
SRC = os.path.join(ORACLE, "lora.py")
SRC_ADAMW = os.path.join(ORACLE, "adamw.py")
SRC_MULTI = os.path.join(ORACLE, "multi.py")
SRC_MX = os.path.join(ORACLE, "mx.py")
SRC_PLAN = os.path.join(ORACLE, "plan_mirror.py")

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
    "sampled_z_no_scale": ("zi = s * (x @ Ai)", "zi = (x @ Ai)"),
    "ids_unstable_sort": ('perm = np.argsort(ids, kind="stable")', 'perm = np.argsort(-ids, kind="stable")[::-1]'),
    "ids_offsets_shift": ("offsets[1:] = np.cumsum(np.bincount(ids, minlength=n))",
                          "offsets[1:] = np.cumsum(np.bincount(ids, minlength=n)) - 1"),
    "ids_y_not_unpermuted": ("    Y = np.empty_like(Yg)\n    Y[perm] = Yg", "    Y = np.empty_like(Yg)\n    Y[:] = Yg"),
    "ids_dx_wrong_inverse": ("        dX[perm] = dXg", "        dX[:] = dXg[perm]"),
}

ADAMW_MUTATIONS = {
    "no_bias_correction_m": ("m_hat = m / (1.0 - beta1 ** t)", "m_hat = m"),
    "no_bias_correction_v": ("v_hat = v / (1.0 - beta2 ** t)", "v_hat = v"),
    "bias_exponent_off_by_one": ("beta2 ** t)", "beta2 ** (t + 1))"),
    "coupled_decay": ("p = p * (1.0 - lr * weight_decay)", "g = g + weight_decay * p"),
    "decay_not_scaled_by_lr": ("p = p * (1.0 - lr * weight_decay)", "p = p * (1.0 - weight_decay)"),
    "decay_after_update": ("    p = p * (1.0 - lr * weight_decay)\n", "    p0 = p\n"),
    "velocity_of_abs_grad": ("(1.0 - beta2) * g * g", "(1.0 - beta2) * np.abs(g)"),
    "eps_inside_sqrt": ("(np.sqrt(v_hat) + eps)", "np.sqrt(v_hat + eps)"),
    "momentum_betas_swapped": ("beta1 * m + (1.0 - beta1) * g", "(1.0 - beta1) * m + beta1 * g"),
    "step_zero_updates": ("if t <= 0:", "if t < 0:"),
    "sign_of_step": ("p = p - lr * m_hat", "p = p + lr * m_hat"),
    "wrong_adapter_hparams": ('h["lr"], h["beta1"]', 'hparams[0]["lr"], h["beta1"]'),
    "clip_norm_not_square_root": ("norm = np.sqrt(sum(", "norm = (sum("),
    "clip_per_tensor": ("c_i = clip_coef(grads[i], h.get(\"max_grad_norm\", 0.0))", "c_i = clip_coef(grads[i][:1], h.get(\"max_grad_norm\", 0.0))"),
    "clip_can_amplify": ("return min(1.0, mx / (norm + 1e-6))", "return mx / (norm + 1e-6)"),
}


MULTI_MUTATIONS = {
    "fwd_wrong_w0_columns": ("Y[r0:r1, c0:c1] = Xc @ W[:, c0:c1] + s * (Zc @ Bip)",
                             "Y[r0:r1, c0:c1] = Xc @ W[:, :c1 - c0] + s * (Zc @ Bip)"),
    "fwd_drop_scale": ("Y[r0:r1, c0:c1] = Xc @ W[:, c0:c1] + s * (Zc @ Bip)",
                       "Y[r0:r1, c0:c1] = Xc @ W[:, c0:c1] + (Zc @ Bip)"),
    "fwd_scale_of_projection_0": ("            s = float(scales[i][p])\n            Zip = np.zeros((b - a",
                                  "            s = float(scales[i][0])\n            Zip = np.zeros((b - a"),
    "dx_overwrites_projections": ("dX[r0:r1] += Gp @ W[:, c0:c1].T + dZc @ Aip.T",
                                  "dX[r0:r1] = Gp @ W[:, c0:c1].T + dZc @ Aip.T"),
    "dx_drop_lora": ("dX[r0:r1] += Gp @ W[:, c0:c1].T + dZc @ Aip.T", "dX[r0:r1] += Gp @ W[:, c0:c1].T"),
    "dy_columns_of_first_projection": ("Gp = as_f64(dY[r0:r1], dtype)[:, c0:c1]",
                                       "Gp = as_f64(dY[r0:r1], dtype)[:, 0:c1 - c0]"),
    "db_drop_scale": ("gB += s * (Zc.T @ Gp)", "gB += (Zc.T @ Gp)"),
    "columns_off_by_one": ("        c.append(c[-1] + int(d))", "        c.append(c[-1] + int(d) - (1 if len(c) == 2 else 0))"),
    "sampled_dx_overwrites": ("dX[ks] += g[:, c0:c1] @ W[:, c0:c1].T", "dX[ks] = g[:, c0:c1] @ W[:, c0:c1].T"),
}


MX_MUTATIONS = {
    "act_emax_7": ("np.clip(ex - 1 - 8, -127, 127)", "np.clip(ex - 1 - 7, -127, 127)"),
    "act_exponent_rounded_up": ("np.clip(ex - 1 - 8, -127, 127)", "np.clip(ex - 8, -127, 127)"),
    "act_no_clamp": ("np.clip(ex - 1 - 8, -127, 127)", "(ex - 1 - 8)"),
    "act_no_saturation": ("code = np.where(a >= 448.0, 0x7E, code)", "code = code"),
    "act_truncating": ("n = np.rint(np.where(sub, 8.0, a) * np.exp2(3.0 - e))", "n = np.floor(np.where(sub, 8.0, a) * np.exp2(3.0 - e))"),
    "act_subnormal_step": ("np.rint(a * 2.0 ** 9)", "np.rint(a * 2.0 ** 8)"),
    "act_block_along_rows": ("blk = x.reshape(T, K // 32, 32)", "blk = x.T.reshape(K, T // 32, 32).transpose(1, 0, 2).reshape(T, K // 32, 32) if T % 32 == 0 else x.reshape(T, K // 32, 32) * 1.01"),
    "act_lora_on_quantized": ("Zi = Xi @ as_f64(A[i], \"bf16\")", "Zi = Xq[lo:hi] @ as_f64(A[i], \"bf16\")"),
    "act_base_unquantized": ("Y[lo:hi] = Xq[lo:hi] @ W +", "Y[lo:hi] = Xi @ W +"),
    "exponent_bias_6": ("norm = (8 + m) * np.exp2(e - 10.0)", "norm = (8 + m) * np.exp2(e - 9.0)"),
    "subnormal_scale": ("sub = m * 2.0 ** -9", "sub = m * 2.0 ** -10"),
    "subnormal_as_normal": ("v = s * np.where(e == 0, sub, norm)", "v = s * norm"),
    "nan_code_finite": ("return np.where((c & 0x7F) == 0x7F, np.nan, v)", "return v"),
    "scale_bias_126": ("np.exp2(x - 127.0)", "np.exp2(x - 126.0)"),
    "scale_nan_ignored": ("return np.where(x == 255, np.nan, np.exp2(x - 127.0))", "return np.exp2(x - 127.0)"),
    "no_ties_to_even": ("r = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF", "r = ((u + 0x8000) >> 16) & 0xFFFF"),
    "truncate_not_round": ("r = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF", "r = (u >> 16) & 0xFFFF"),
    "block_along_output": ("w = q * np.repeat(sc.T, 32, axis=0)",
                           "w = q * np.repeat(np.repeat(sc.T[:1], d_in, axis=0)[:, :1], d_out, axis=1)"),
    "nk_not_transposed": ("    if layout != \"kn\":\n        q = q.T", "    if layout != \"kn\":\n        q = q.reshape(d_in, d_out)"),
    "sign_dropped": ("s = np.where(c >> 7, -1.0, 1.0)", "s = np.where(c >> 7, 1.0, 1.0)"),
    "e2m1_sign_bit_2": ("s = np.where(c >> 3, -1.0, 1.0)", "s = np.where((c >> 2) & 1, -1.0, 1.0)"),
    "e2m1_bias_2": ("(2 + m) * np.exp2(e - 2.0)", "(2 + m) * np.exp2(e - 3.0)"),
    "e2m1_subnormal_as_one": ("np.where(e == 0, 0.5 * m,", "np.where(e == 0, 1.0 * m,"),
    "e2m1_nibbles_swapped": ("    out[:, 0::2] = b & 15\n    out[:, 1::2] = b >> 4",
                             "    out[:, 0::2] = b >> 4\n    out[:, 1::2] = b & 15"),
    "e2m1_mantissa_weight": ("(2 + m) * np.exp2", "(2 + 2 * m) * np.exp2"),
    "mxfp4_decoded_as_fp8": ("    if fmt == \"mxfp4\":", "    if fmt == \"mxfp4-never\":"),
}


PLAN_MUTATIONS = {
    "rpad_min_16": ("rpad = [max(32, _pow2_at_least(r)) for r in rk]", "rpad = [max(16, _pow2_at_least(r)) for r in rk]"),
    "zoff_without_rows": ("z += cnt[v // P] * rpad[v]", "z += rpad[v]"),
    "roff_unpadded": ("rr += rpad[v]", "rr += rk[v]"),
    "seg_start_by_projection": ("seg_start.append(o[v // P])", "seg_start.append(o[v % P])"),
    "group_floor": ("target = -(-(s * T) // S)  # ceil", "target = (s * T) // S"),
    "group_not_monotone": ("g[s] = max(g[s - 1], a)", "g[s] = a if a < n else g[s - 1]"),
    "bucket_ascending": ("key=lambda v: (-rpad[v], v % P, v // P)", "key=lambda v: (rpad[v], v % P, v // P)"),
    "bucket_adapter_before_projection": ("key=lambda v: (-rpad[v], v % P, v // P)",
                                         "key=lambda v: (-rpad[v], v // P, v % P)"),
    "nano_tail_dropped": ("nb.append((v, r0, min(NB, hi - r0)))", "nb.append((v, r0, NB)) if r0 + NB <= hi else None"),
    "chunk_by_rank_not_rpad": ("opts.chunk_per_rank * rpad[v])", "opts.chunk_per_rank * rk[v])"),
    "chunk_max_ignored": ("kc = min(opts.chunk_max, max(", "kc = (max("),
    "cpref_after": ("cpref.append(cp)\n                cboff.append(cb)\n                cp += rpad[v]",
                    "cp += rpad[v]\n                cpref.append(cp)\n                cboff.append(cb)"),
    "cboff_without_width": ("cb += rpad[v] * wd[v % P]", "cb += rpad[v] * wd[0]"),
    "ext_wrong_projection": ("v = j * P + q", "v = j * P"),
    "ext_k_step_64": ("for k0 in range(0, rpad[v], KSTEP):", "for k0 in range(0, rpad[v], 2 * KSTEP):"),
    "tile_boundary_rounded_up": ("a[s] = max(a[s - 1], G * ((o[g[s]] // BM) // G))",
                                 "a[s] = max(a[s - 1], G * -(-(o[g[s]] // BM) // G))"),
    "tile_boundary_not_aligned": ("G = 16 if ntile >= 32 * S else 1", "G = 1"),
    "tile_alignment_threshold_per_plan": ("G = 16 if ntile >= 32 * S else 1", "G = 16 if ntile >= 32 else 1"),
    "tile_ext_own_group_only": ("                for j in range(n):\n                    lo, hi = max(o[j], t0)",
                                "                for j in range(g[s], g[s + 1]):\n                    lo, hi = max(o[j], t0)"),
    "default_nano_rows_threshold": ("NB = 128 if T * P >= 65536 else", "NB = 128 if T * P > 65536 else"),
    "default_nano_rows_ignores_projections": ("(64 if T * P >= 32768 else 32)", "(64 if T >= 32768 else 32)"),
    "split_k_no_rebalance": ("    return -(-nk // kper)", "    return sp"),
    "split_k_limit_64": ("if tiles <= 0 or tiles >= 128 or nk < 16:", "if tiles <= 0 or tiles >= 64 or nk < 16:"),
    "ids_reverse_within_adapter": ("    for t, a in enumerate(ids):\n        perm[nxt[a]] = t",
                                   "    for t, a in reversed(list(enumerate(ids))):\n        perm[nxt[a]] = t"),
    "ids_prefix_off_by_one": ("        off[a + 1] += 1", "        off[min(a + 2, n)] += 1"),
}


def _mutant(old, new, src_path=SRC) -> types.ModuleType:
    with open(src_path) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new, 1)
    mod = types.ModuleType("oracle.oracle_mutant")
    mod.__package__ = "oracle"
    # dataclasses look their module up in sys.modules while the class body runs
    sys.modules[mod.__name__] = mod
    try:
        exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    finally:
        del sys.modules[mod.__name__]
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


@pytest.mark.parametrize("name", sorted(ADAMW_MUTATIONS))
def test_adamw_pins_catch_planted_mistake(name):
    old, new = ADAMW_MUTATIONS[name]
    mod = _mutant(old, new, SRC_ADAMW)
    caught = []
    for pin in pins_adamw.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught mutation {name}"


@pytest.mark.parametrize("name", sorted(MULTI_MUTATIONS))
def test_multi_pins_catch_planted_mistake(name):
    old, new = MULTI_MUTATIONS[name]
    mod = _mutant(old, new, SRC_MULTI)
    caught = []
    for pin in pins_multi.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught mutation {name}"


@pytest.mark.parametrize("name", sorted(MX_MUTATIONS))
def test_mx_pins_catch_planted_mistake(name):
    old, new = MX_MUTATIONS[name]
    mod = _mutant(old, new, SRC_MX)
    caught = []
    for pin in pins_mx.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught mutation {name}"


@pytest.mark.parametrize("name", sorted(PLAN_MUTATIONS))
def test_plan_pins_catch_planted_mistake(name):
    old, new = PLAN_MUTATIONS[name]
    mod = _mutant(old, new, SRC_PLAN)
    caught = []
    for pin in pins_plan.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught mutation {name}"
