"""Comparison rules between the HIP path and the CPU oracle.

* summaries: equal or at most `max_ulp` units in the last place of the stored
  type (float32 or bfloat16) apart (the oracle rounds the exact mean once; the
  kernel sums in fp64 in another order, so a different rounding needs a
  near-tie of the mean);
* leaf indices: bit-exact, except on queries whose oracle cut gap at some
  level is below 1e-5 relative, which are counted and reported instead; their
  number is bounded (excused_bound: 0 on full-size cases, 0.1% elsewhere);
* attention outputs: max-abs error within the tolerance for the input type
  (1e-4 for fp32 inputs, 2e-2 for bf16 inputs with fp32 accumulation).
"""
from __future__ import annotations

import numpy as np

TIE_GAP = 1e-5
ATTEND_TOL = {"f32": 1e-4, "bf16": 2e-2}


def ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in float32 units in the last place (+0 and -0 count as equal)."""
    def key(x):
        i = np.ascontiguousarray(x, dtype=np.float32).view(np.int32).astype(np.int64)
        return np.where(i < 0, -(i & 0x7FFFFFFF), i)
    return np.abs(key(a) - key(b))


# float32 units in the last place per unit of the stored summary type (a
# bfloat16 drops the low 16 bits of a float32, an e4m3 code keeps 3 fraction
# bits of its 23: a step of a normal code is 2^20 float32 units)
ULP_SCALE = {"f32": 1, "bf16": 1 << 16, "fp8": 1 << 20}


def compare_summaries(gpu_levels, oracle_stored, max_ulp: int = 1, summary_dtype: str = "f32"):
    """Returns (bit_equal, total, worst_ulp), ulps of the stored type; raises
    AssertionError past max_ulp.  gpu_levels hold float32 values (a bfloat16
    summary widened exactly)."""
    scale = ULP_SCALE[summary_dtype]
    equal = total = worst = 0
    for l, (g, o) in enumerate(zip(gpu_levels, oracle_stored), start=1):
        g = np.asarray(g, dtype=np.float32)
        assert g.shape == o.shape, (l, g.shape, o.shape)
        d = -(-ulp_distance(g, o) // scale)   # whole units of the stored type, rounded up
        equal += int(np.count_nonzero(d == 0))
        total += d.size
        worst = max(worst, int(d.max()))
        if d.max() > max_ulp:
            bad = np.argwhere(d > max_ulp)[:5]
            raise AssertionError(f"level {l}: {np.count_nonzero(d > max_ulp)} summaries more than "
                                 f"{max_ulp} ulp from the oracle, e.g. at {bad.tolist()}")
    return equal, total, worst


def excused_bound(n: int) -> int:
    """Most tie-exposed mismatches a parity case over n queries (or
    positions) may excuse: 0.1% of them, so 0 below 1,000.  The kernels
    score in fp64 like the oracle, so a mismatch needs two scores within
    about 1e-15 of each other; the full-size cases pass 0 explicitly."""
    return n // 1000


def check_excused(excused: int, n: int, max_excused=None, what: str = "queries") -> None:
    bound = excused_bound(n) if max_excused is None else max_excused
    assert excused <= bound, (f"{excused} tie-exposed mismatches among {n} {what}, more than "
                              f"the {bound} a case may excuse")


def compare_indices(gpu_idx: np.ndarray, oracle_route: dict, max_excused=None):
    """Returns (exact, tie_exposed_mismatch, n_queries).  Fails on any mismatch
    of a query whose every cut gap is >= TIE_GAP, and when the tie-exposed
    mismatches exceed max_excused (default: excused_bound(n_queries))."""
    want = oracle_route["indices"]
    assert gpu_idx.shape == want.shape, (gpu_idx.shape, want.shape)
    mismatch = np.any(gpu_idx != want, axis=-1)
    tie = np.min(oracle_route["gap"], axis=-1) < TIE_GAP
    hard = mismatch & ~tie
    if np.any(hard):
        where = np.argwhere(hard)[:5].tolist()
        q = tuple(where[0])
        raise AssertionError(f"{int(hard.sum())} queries select other leaves than the oracle "
                             f"with no near-tie, e.g. {where}: gpu {gpu_idx[q].tolist()} "
                             f"oracle {want[q].tolist()} gaps {oracle_route['gap'][q].tolist()}")
    n = int(np.prod(mismatch.shape))
    excused = int((mismatch & tie).sum())
    check_excused(excused, n, max_excused)
    return n - int(mismatch.sum()), excused, n


def compare_trace(gpu_trace: np.ndarray, oracle_route: dict) -> None:
    """Kept set of every level, on queries with no near-tie."""
    tie = np.min(oracle_route["gap"], axis=-1) < TIE_GAP
    want = oracle_route["trace"]
    ok = np.all(gpu_trace == want, axis=(-1, -2)) | tie
    assert np.all(ok), f"trace differs on {int((~ok).sum())} queries"


def compare_outputs(gpu_out: np.ndarray, oracle_out: np.ndarray, dtype: str) -> float:
    tol = ATTEND_TOL[dtype]
    assert gpu_out.shape == oracle_out.shape
    err = float(np.max(np.abs(gpu_out.astype(np.float64) - oracle_out))) if gpu_out.size else 0.0
    assert np.all(np.isfinite(gpu_out)), "non-finite attention output"
    assert err <= tol, f"max-abs error {err:.3g} > {tol}"
    return err
