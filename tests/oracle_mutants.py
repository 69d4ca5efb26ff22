"""Plants one plausible mistake in the oracle, on the CPU, and runs the
oracle's pins against it (test infrastructure: a mutant is a check that the
pins would notice the mistake, never a second oracle).

    python tests/oracle_mutants.py NAME     # exit status of the pin run
    python tests/oracle_mutants.py --list

The mutation is a one-place edit of the oracle's source text; the edited
module's functions replace the oracle's in the already imported module, so
the pins (which call the oracle through the module) run against it.  NAME
"none" runs the pins on the oracle as it is.  The pins run here are those
that do not compare with stored oracle outputs (the golden file is left
out): closed forms, exact rational brute force, library routines,
invariants and the tie-measure pins.
"""
from __future__ import annotations

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# name -> (text in oracle/tis_oracle.py, replacement); each text occurs once
MUTANTS = {
    # route
    "tie_order_highest_index": ("order = np.lexsort((cand, -sigma))",
                                "order = np.lexsort((-cand, -sigma))"),
    "score_sign": ("sigma = summ @ q", "sigma = -(summ @ q)"),
    "child_index_stride": (
        "cand = (kept[:, None] * branching + children[None, :]).ravel()",
        "cand = (kept[:, None] + children[None, :] * branching ** (l - 1)).ravel()"),
    "root_child_missing": ("cand = children.copy()", "cand = children[1:].copy()"),
    "level_order_reversed": ("summ = stored[l - 1][bi, hk][cand]",
                             "summ = stored[-l][bi, hk][cand]"),
    "route_reads_head_zero": ("summ = stored[l - 1][bi, hk][cand]",
                              "summ = stored[l - 1][bi, 0][cand]"),
    "keep_one_fewer_when_all_fit": ("n_keep = min(beam, len(cand))",
                                    "n_keep = min(beam, len(cand) - 1)"),
    "gqa_map_route": ("hk = hq // G\n            q = q64[bi, hq]",
                      "hk = hq % Hkv\n            q = q64[bi, hq]"),
    # tie measure
    "gap_next_pair": ("a, c = sigma[order[n_keep - 1]], sigma[order[n_keep]]",
                      "a, c = sigma[order[n_keep]], sigma[order[min(n_keep + 1, len(cand) - 1)]]"),
    "gap_absolute": ("gap[bi, hq, l - 1] = 0.0 if den == 0.0 else (a - c) / den",
                     "gap[bi, hq, l - 1] = a - c"),
    "gap_min_denominator": ("den = max(abs(a), abs(c))", "den = min(abs(a), abs(c))"),
    # build
    "sum_not_mean": ("means[l - 1][bi, h] = node_sums / M_l", "means[l - 1][bi, h] = node_sums"),
    "fp32_accumulation": (
        "node_sums = k64.reshape(n_l, M_l, d).sum(axis=1)",
        "node_sums = k64.astype(np.float32).reshape(n_l, M_l, d).sum(\n"
        "                    axis=1, dtype=np.float32).astype(np.float64)"),
    "node_keys_interleaved": ("node_sums = k64.reshape(n_l, M_l, d).sum(axis=1)",
                              "node_sums = k64.reshape(M_l, n_l, d).sum(axis=0)"),
    "summary_not_rounded": ("stored = [round_summary(m, summary_dtype) for m in means]",
                            "stored = [np.asarray(m) for m in means]"),
    # attend
    "gqa_map_attend": ("hk = hq // G\n            sel =", "hk = hq % Hkv\n            sel ="),
    "scale_one_over_d": ("scale = 1.0 / math.sqrt(d)", "scale = 1.0 / d"),
    "block_row_offset": ("rows = (blocks[:, None] * leaf_block",
                         "rows = (blocks[:, None] * (leaf_block - 1)"),
    "repeated_block_twice": ("blocks = np.unique(sel[sel >= 0])", "blocks = sel[sel >= 0]"),
    # input widening and summary rounding
    "bf16_read_as_fp16": (
        "hi = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)\n"
        "        return hi.view(np.float32).astype(np.float64)",
        "return np.asarray(x, dtype=np.uint16).view(np.float16).astype(np.float64)"),
    "bf16_ties_away": ("y = np.ldexp(np.rint(np.ldexp(ax, -q)), q)",
                       "y = np.ldexp(np.floor(np.ldexp(ax, -q) + 0.5), q)"),
    "bf16_truncate": ("y = np.ldexp(np.rint(np.ldexp(ax, -q)), q)",
                      "y = np.ldexp(np.floor(np.ldexp(ax, -q)), q)"),
    "bf16_through_float32": (
        "ax = np.abs(x)\n    _, e = np.frexp(ax)\n    q = np.maximum(e - _BF16_SIG_BITS",
        "ax = np.abs(x).astype(np.float32).astype(np.float64)\n    _, e = np.frexp(ax)\n"
        "    q = np.maximum(e - _BF16_SIG_BITS"),
    "e4m3_ties_away": ("return np.copysign(np.ldexp(np.rint(np.ldexp(ax, -q)), q), x)",
                       "return np.copysign(np.ldexp(np.floor(np.ldexp(ax, -q) + 0.5), q), x)"),
    "fp8_scale_boundary": ("e = np.where(f <= 0.875, k - 9, k - 8)",
                           "e = np.where(f < 0.875, k - 9, k - 8)"),
}

PIN_FILES = ["tests/test_oracle_pins.py", "tests/test_tie_measure_pins.py",
             "tests/test_summary_rounding_pins.py"]


def apply(name: str) -> None:
    """Replaces the oracle module's functions by those of the mutated source."""
    from oracle import tis_oracle as O
    if name == "none":
        return
    old, new = MUTANTS[name]
    with open(O.__file__) as f:
        src = f.read()
    if src.count(old) != 1:
        raise SystemExit(f"mutant {name}: its text occurs {src.count(old)} times in the oracle")
    ns = {"__name__": O.__name__ + "_mutant", "__file__": O.__file__}
    exec(compile(src.replace(old, new), O.__file__, "exec"), ns)
    for k, v in ns.items():
        if callable(v) and getattr(v, "__module__", None) == ns["__name__"] and hasattr(O, k):
            setattr(O, k, v)


def main(argv) -> int:
    if argv and argv[0] == "--list":
        print("\n".join(["none"] + sorted(MUTANTS)))
        return 0
    name = argv[0] if argv else "none"
    sys.path.insert(0, ROOT)
    os.chdir(ROOT)
    apply(name)
    import pytest
    rc = pytest.main(PIN_FILES + ["-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                                  "--hypothesis-seed=0"])
    # 0: every pin passed; 1: a pin failed (a crash inside the oracle counts);
    # anything else is a broken run, not a verdict on the oracle
    print(f"PIN_RUN {name} {'PASSED' if rc == 0 else 'FAILED' if rc == 1 else f'BROKEN {rc}'}",
          flush=True)
    return int(rc)


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
