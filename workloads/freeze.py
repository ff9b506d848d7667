"""Write the frozen integer structure of every workload (seeds 0-2).

Run: python -m workloads.freeze
"""
import os

from .configs import WORKLOAD_NAMES, FROZEN_DIR, draw_workload, frozen_path


def main():
    os.makedirs(FROZEN_DIR, exist_ok=True)
    for name in WORKLOAD_NAMES:
        for seed in (0, 1, 2):
            w = draw_workload(name, seed)
            with open(frozen_path(name, seed), "w") as f:
                f.write(w.to_json() + "\n")
            print(name, seed, "T=%d" % w.T, "ranks", w.ranks[:8], "tokens", w.tokens[:8])


if __name__ == "__main__":
    main()
