"""Plants one plausible mistake in the oracle, on the CPU, and runs the
oracle's pins against it (test infrastructure: a mutant is a check that the
pins would notice the mistake, never a second oracle).

    python tests/oracle_mutants.py NAME     # exit status of the pin run
    python tests/oracle_mutants.py --list

The mutation is a one-place edit of the oracle's source text; the edited
module's functions replace the oracle's in the already imported module, so
the pins (which call the oracle through the module) run against it.  NAME
"none:<module>" runs that module's pins on the oracle as it is.  The pins run here are those
that do not compare with stored oracle outputs (the golden file is left
out): closed forms, exact rational brute force, library routines,
invariants and the tie-measure pins.
"""
from __future__ import annotations

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# name -> (oracle module, text in its source, replacement); each text occurs
# once in its module
MUTANTS = {
    # ---- oracle/tis_oracle.py
    # route
    "tie_order_highest_index": ("tis_oracle", "order = np.lexsort((cand, -sigma))",
                                "order = np.lexsort((-cand, -sigma))"),
    "score_sign": ("tis_oracle", "sigma = summ @ q", "sigma = -(summ @ q)"),
    "child_index_stride": ("tis_oracle", 
        "cand = (kept[:, None] * branching + children[None, :]).ravel()",
        "cand = (kept[:, None] + children[None, :] * branching ** (l - 1)).ravel()"),
    "root_child_missing": ("tis_oracle", "cand = children.copy()", "cand = children[1:].copy()"),
    "level_order_reversed": ("tis_oracle", "summ = stored[l - 1][bi, hk][cand]",
                             "summ = stored[-l][bi, hk][cand]"),
    "route_reads_head_zero": ("tis_oracle", "summ = stored[l - 1][bi, hk][cand]",
                              "summ = stored[l - 1][bi, 0][cand]"),
    "keep_one_fewer_when_all_fit": ("tis_oracle", "n_keep = min(beam, len(cand))",
                                    "n_keep = min(beam, len(cand) - 1)"),
    "gqa_map_route": ("tis_oracle", "hk = hq // G\n            q = q64[bi, hq]",
                      "hk = hq % Hkv\n            q = q64[bi, hq]"),
    # tie measure
    "gap_next_pair": ("tis_oracle", "a, c = sigma[order[n_keep - 1]], sigma[order[n_keep]]",
                      "a, c = sigma[order[n_keep]], sigma[order[min(n_keep + 1, len(cand) - 1)]]"),
    "gap_absolute": ("tis_oracle", "gap[bi, hq, l - 1] = 0.0 if den == 0.0 else (a - c) / den",
                     "gap[bi, hq, l - 1] = a - c"),
    "gap_min_denominator": ("tis_oracle", "den = max(abs(a), abs(c))", "den = min(abs(a), abs(c))"),
    # build
    "sum_not_mean": ("tis_oracle", "means[l - 1][bi, h] = node_sums / M_l", "means[l - 1][bi, h] = node_sums"),
    "fp32_accumulation": ("tis_oracle", 
        "node_sums = k64.reshape(n_l, M_l, d).sum(axis=1)",
        "node_sums = k64.astype(np.float32).reshape(n_l, M_l, d).sum(\n"
        "                    axis=1, dtype=np.float32).astype(np.float64)"),
    "node_keys_interleaved": ("tis_oracle", "node_sums = k64.reshape(n_l, M_l, d).sum(axis=1)",
                              "node_sums = k64.reshape(M_l, n_l, d).sum(axis=0)"),
    "summary_not_rounded": ("tis_oracle", "stored = [round_summary(m, summary_dtype) for m in means]",
                            "stored = [np.asarray(m) for m in means]"),
    # attend
    "gqa_map_attend": ("tis_oracle", "hk = hq // G\n            sel =", "hk = hq % Hkv\n            sel ="),
    "scale_one_over_d": ("tis_oracle", "scale = 1.0 / math.sqrt(d)", "scale = 1.0 / d"),
    "block_row_offset": ("tis_oracle", "rows = (blocks[:, None] * leaf_block",
                         "rows = (blocks[:, None] * (leaf_block - 1)"),
    "repeated_block_twice": ("tis_oracle", "blocks = np.unique(sel[sel >= 0])", "blocks = sel[sel >= 0]"),
    # input widening and summary rounding
    "bf16_read_as_fp16": ("tis_oracle", 
        "hi = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)\n"
        "        return hi.view(np.float32).astype(np.float64)",
        "return np.asarray(x, dtype=np.uint16).view(np.float16).astype(np.float64)"),
    "bf16_ties_away": ("tis_oracle", "y = np.ldexp(np.rint(np.ldexp(ax, -q)), q)",
                       "y = np.ldexp(np.floor(np.ldexp(ax, -q) + 0.5), q)"),
    "bf16_truncate": ("tis_oracle", "y = np.ldexp(np.rint(np.ldexp(ax, -q)), q)",
                      "y = np.ldexp(np.floor(np.ldexp(ax, -q)), q)"),
    "bf16_through_float32": ("tis_oracle", 
        "ax = np.abs(x)\n    _, e = np.frexp(ax)\n    q = np.maximum(e - _BF16_SIG_BITS",
        "ax = np.abs(x).astype(np.float32).astype(np.float64)\n    _, e = np.frexp(ax)\n"
        "    q = np.maximum(e - _BF16_SIG_BITS"),
    "e4m3_ties_away": ("tis_oracle", "return np.copysign(np.ldexp(np.rint(np.ldexp(ax, -q)), q), x)",
                       "return np.copysign(np.ldexp(np.floor(np.ldexp(ax, -q) + 0.5), q), x)"),
    "fp8_scale_boundary": ("tis_oracle", "e = np.where(f <= 0.875, k - 9, k - 8)",
                           "e = np.where(f < 0.875, k - 9, k - 8)"),
    # ---- oracle/tis_grow_oracle.py (growing cache)
    "grow_depth_one_early": ("tis_grow_oracle", "while branching ** lv * leaf_block < n_keys:",
                             "while branching ** lv * leaf_block <= n_keys:"),
    "grow_open_mean_over_full_span": ("tis_grow_oracle", "k64[lo:hi].sum(axis=0) / (hi - lo)",
                                      "k64[lo:hi].sum(axis=0) / M"),
    "grow_open_node_never_scored": ("tis_grow_oracle", "cand = cand[cand < e[l - 1]]",
                                    "cand = cand[cand < e[l - 1] - 1]"),
    "grow_attend_reads_past_n": (
        "tis_grow_oracle",
        "np.arange(j * leaf_block, min((j + 1) * leaf_block, n_keys))",
        "np.arange(j * leaf_block, (j + 1) * leaf_block)"),
    "grow_tie_order": ("tis_grow_oracle", "order = np.lexsort((cand, -sigma))",
                       "order = np.lexsort((-cand, -sigma))"),
    # ---- oracle/tis_sphere_oracle.py (bounding spheres)
    "sphere_mean_not_max": ("tis_sphere_oracle", "(diff * diff).sum(axis=2).max(axis=1)",
                            "(diff * diff).sum(axis=2).mean(axis=1)"),
    "sphere_bound_without_norm": ("tis_sphere_oracle",
                                  "bound = c @ q64[bi, hq] + qn[bi, hq] * r",
                                  "bound = c @ q64[bi, hq] + r"),
    "sphere_bound_r_squared": ("tis_sphere_oracle", "bound = c @ q64[bi, hq] + qn[bi, hq] * r",
                               "bound = c @ q64[bi, hq] + qn[bi, hq] * r * r"),
    "sphere_strict_prune": ("tis_sphere_oracle", "kept = np.sort(cand[bound >= t])",
                            "kept = np.sort(cand[bound > t])"),
    "sphere_strict_key_mask": ("tis_sphere_oracle", "            sel = s >= t\n",
                               "            sel = s > t\n"),
    "sphere_overflow_at_max": ("tis_sphere_oracle", "if len(kept) > max_nodes:",
                               "if len(kept) >= max_nodes:"),
    "sphere_squared_query_norm": ("tis_sphere_oracle", "return np.sqrt((q * q).sum(axis=-1))",
                                  "return (q * q).sum(axis=-1)"),
    "sphere_gqa_map": ("tis_sphere_oracle", "k = widen(K[bi, hq // G, rows], dtype)",
                       "k = widen(K[bi, hq % Hkv, rows], dtype)"),
    # ---- oracle/tis_causal_oracle.py (causal prefill)
    "causal_sees_next_key": ("tis_causal_oracle", "n = int(t) + 1",
                             "n = min(int(t) + 2, N)"),
    "causal_query_of_previous_position": ("tis_causal_oracle",
                                          "q = np.ascontiguousarray(Q[:, :, t])",
                                          "q = np.ascontiguousarray(Q[:, :, max(int(t) - 1, 0)])"),
    "causal_full_leaf_counts": ("tis_causal_oracle",
                                "min(leaf_block, n_keys - j * leaf_block)", "leaf_block"),
    "causal_gap_largest_level": ("tis_causal_oracle", "gap[:, :, i] = g.min(axis=-1)",
                                 "gap[:, :, i] = g.max(axis=-1)"),
}

# the pins run for a mutant of each module
PIN_FILES = {
    "tis_oracle": ["tests/test_oracle_pins.py", "tests/test_tie_measure_pins.py",
                   "tests/test_summary_rounding_pins.py"],
    "tis_grow_oracle": ["tests/test_grow_oracle_pins.py"],
    "tis_sphere_oracle": ["tests/test_sphere_oracle_pins.py"],
    "tis_causal_oracle": ["tests/test_causal_oracle_pins.py"],
}


def apply(name: str) -> list:
    """Replaces the mutated oracle module's functions by those of its edited
    source; returns the pin files to run."""
    import importlib
    if name.startswith("none"):
        module = name.split(":", 1)[1] if ":" in name else "tis_oracle"
        return PIN_FILES[module]
    module, old, new = MUTANTS[name]
    O = importlib.import_module("oracle." + module)
    with open(O.__file__) as f:
        src = f.read()
    if src.count(old) != 1:
        raise SystemExit(f"mutant {name}: its text occurs {src.count(old)} times in {module}")
    ns = {"__name__": O.__name__ + "_mutant", "__file__": O.__file__}
    exec(compile(src.replace(old, new), O.__file__, "exec"), ns)
    for k, v in ns.items():
        if callable(v) and getattr(v, "__module__", None) == ns["__name__"] and hasattr(O, k):
            setattr(O, k, v)
    return PIN_FILES[module]


def main(argv) -> int:
    if argv and argv[0] == "--list":
        print("\n".join([f"none:{m}" for m in PIN_FILES] + sorted(MUTANTS)))
        return 0
    name = argv[0] if argv else "none"
    sys.path.insert(0, ROOT)
    os.chdir(ROOT)
    pins = apply(name)
    import pytest
    rc = pytest.main(pins + ["-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                                  "--hypothesis-seed=0"])
    # 0: every pin passed; 1: a pin failed (a crash inside the oracle counts);
    # anything else is a broken run, not a verdict on the oracle
    print(f"PIN_RUN {name} {'PASSED' if rc == 0 else 'FAILED' if rc == 1 else f'BROKEN {rc}'}",
          flush=True)
    return int(rc)


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
