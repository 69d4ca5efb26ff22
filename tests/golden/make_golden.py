"""Writes tiny_decode.json: a small fixed decode case and the oracle's answer.

Run from the repository root:  python tests/golden/make_golden.py
Inputs are small integers scaled by 1/8 (exact in bf16 and fp32); expected
values come from the CPU oracle only.
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
from oracle import tis_oracle as O  # noqa: E402


def main():
    rng = np.random.default_rng(20261203)
    B, Hkv, G, d, b, L, lv, W = 1, 2, 2, 8, 2, 4, 3, 3
    N = b ** lv * L
    K = (rng.integers(-16, 17, size=(B, Hkv, N, d)) / 8.0).astype(np.float32)
    V = (rng.integers(-16, 17, size=(B, Hkv, N, d)) / 8.0).astype(np.float32)
    Q = (rng.integers(-16, 17, size=(B, Hkv * G, d)) / 8.0).astype(np.float32)
    res = O.decode(Q, K, V, "f32", b, L, lv, W)
    out = {
        "about": "tiny decode case; expected values written by tests/golden/make_golden.py "
                 "from the CPU oracle (fp64, summaries rounded once to fp32)",
        "geometry": {"batch": B, "kv_heads": Hkv, "q_heads": Hkv * G, "head_dim": d,
                     "branching": b, "leaf_block": L, "levels": lv, "beam": W},
        "K": K.tolist(), "V": V.tolist(), "Q": Q.tolist(),
        "summaries": [s.tolist() for s in res["tree"]["stored"]],
        "indices": res["route"]["indices"].tolist(),
        "trace": res["route"]["trace"].tolist(),
        "min_gap": float(np.min(res["route"]["gap"])),
        "out": res["out"].tolist(),
    }
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_decode.json"), "w") as f:
        json.dump(out, f, separators=(",", ":"))
        f.write("\n")


if __name__ == "__main__":
    main()
