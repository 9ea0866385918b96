"""Shared helpers of the GPU parity tests (HIP path vs the fp64 oracle)."""
from __future__ import annotations

import numpy as np

import oracle

# Tolerances: fp32 inputs 1e-5 max-abs on out and lse; bf16 inputs (fp32
# accumulation) 2e-2 on out and 1e-3 on lse.
TOL = {"f32": (1e-5, 1e-5), "bf16": (2e-2, 1e-3)}


def sample_rows(index: np.ndarray, cu_rows: np.ndarray, n_random: int, seed: int) -> np.ndarray:
    """Local rows to check at full size: both ends of every sample and of
    every run of consecutive global ids (image, chunk r, chunk 2P-1-r, the
    first pad), plus random rows."""
    R = len(index)
    picks = set()
    starts = [0] + [i for i in range(1, R) if index[i] != index[i - 1] + 1 or index[i] < 0 <= index[i - 1]]
    for s in starts:
        for d in (0, 1, 31, 32, 63, 64):
            if s + d < R:
                picks.add(s + d)
        if s > 0:
            picks.add(s - 1)
    for c in cu_rows:
        for d in (-1, 0):
            if 0 <= c + d < R:
                picks.add(int(c + d))
    rng = np.random.default_rng(seed)
    picks.update(rng.integers(0, R, size=min(n_random, R)).tolist())
    return np.array(sorted(picks), dtype=np.int64)


def compare(out_gpu, lse_gpu, out_ref, lse_ref, dtype: str, what: str):
    """Max-abs parity; pad rows (lse -inf in the oracle) must be exactly 0 / -inf."""
    o = out_gpu.detach().float().cpu().numpy().astype(np.float64)
    l = lse_gpu.detach().float().cpu().numpy().astype(np.float64)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    pad = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(l), pad), f"{what}: -inf lse pattern differs"
    pad_rows = pad.all(axis=0)
    if pad_rows.any():
        assert np.all(o[pad_rows] == 0.0), f"{what}: pad rows not exactly 0"
    tol_o, tol_l = TOL[dtype]
    err_o = float(np.abs(o - out_ref).max()) if o.size else 0.0
    fin = ~pad
    err_l = float(np.abs(l[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    assert err_o <= tol_o, f"{what}: out max-abs {err_o:.3e} > {tol_o}"
    assert err_l <= tol_l, f"{what}: lse max-abs {err_l:.3e} > {tol_l}"
    return err_o, err_l


def oracle_rows(q, k, v, n_img, cu, P, r, rows=None, split="head_tail"):
    return oracle.rank_attention(q, k, v, n_img, cu, P, r, local_rows=rows, split=split)


def pooled_oracle(q, k, v, n_img, cu, P, r, rows=None, heads=None, split="head_tail", stats=None):
    """The oracle's rank rows (all, or the local rows ``rows``) for the query
    heads ``heads`` (all if None), computed by threads of this process over
    (KV group, 128-row) tasks; see oracle.pool."""
    from oracle.pool import rank_attention_pooled

    return rank_attention_pooled(q, k, v, n_img, cu, P, r, local_rows=rows, split=split, heads=heads,
                                 executor="thread", row_chunk=128, stats=stats)
