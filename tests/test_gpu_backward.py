"""GPU parity of the per-rank backward (cp_attn_rank_bwd) against the fp64
oracle's gradients (oracle.rank_attention_backward): small cases for every
rank, workloads 3 and 4 on every element, workloads 4 and 5 on sampled rows
and keys with whole-tensor properties.

Inputs q, k, v and dout are bf16 (the oracle reads the same values); out
and lse come from the library's own forward, as in training. Two bounds:
the max-abs error relative to the largest reference gradient of the tensor,
and, per (row, head) of dq and per (key, KV head) of dk and dv, the max-abs
error relative to that row's or key's own largest reference gradient (with
a floor of 2^-8 of the tensor's, for rows whose gradient is near zero).
"""
import zlib

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
# |g - g_ref|_max <= BWD_RTOL * max(|g_ref|_max, 1). With bf16 inputs the
# forward's out is bf16, so Delta = rowsum(dout * out) carries its rounding
# (unit roundoff u = 2^-8) into dS, dq and dk; bf16 with head_dim 128 also rounds P
# and dS to bf16 for its MFMA products. fp32 inputs run the fp32 FMA
# kernels end to end, so only fp32 rounding remains (BWD_RTOL_F32).
BWD_RTOL = 2e-2
BWD_RTOL_F32 = 1e-4
# Per row / per key: |g_i - ref_i|_max <= ROW_RTOL * (|ref_i|_max + 2^-8 |ref|_max)
# + slack_i. A gradient row is a sum over the row's keys (dq) or rows (dk,
# dv) whose terms carry the bf16 roundings above independently, so that part
# of its error scales with its own magnitude (the floor covers rows whose
# gradient is near zero). dq also moves with Delta's error, which does not
# shrink with dq: Delta_i = sum_d dout_id out_id is taken from the bf16
# forward output, |dDelta_i| <= 2u sum_d |dout_id out_id| (its rounding and
# the forward's own bf16 error), and dq_i = sum_j P_ij (dP_ij - Delta_i) k_j
# / sqrt(D) moves by dDelta_i (P k)_i / sqrt(D) -- the slack (a row whose
# exact dq nearly cancels, such as a two-key row with a peaky softmax, is
# dominated by it). (P k)_i is attention with the keys as values.
U_BF16 = 2.0 ** -8  # unit roundoff of bf16 (8-bit significand)
ROW_RTOL = 2e-2
ROW_RTOL_F32 = 1e-4
ROW_FLOOR = 2.0 ** -8


@pytest.fixture(scope="module")
def cp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_parallelism_amd as m
    return m


def draw(seed, T, H, Hkv, D, R, dtype=torch.bfloat16):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, D), dtype=np.float32)
    k = rng.standard_normal((T, Hkv, D), dtype=np.float32)
    v = rng.standard_normal((T, Hkv, D), dtype=np.float32)
    dout = rng.standard_normal((R, H, D), dtype=np.float32)
    return [torch.from_numpy(a).to(dtype) for a in (q, k, v, dout)]


def rel_err(got, ref):
    g = got.detach().float().cpu().numpy().astype(np.float64)
    scale = max(float(np.abs(ref).max()) if ref.size else 0.0, 1.0)
    return float(np.abs(g - ref).max()) / scale if ref.size else 0.0


def row_err(got, ref, rtol, slack=None):
    """Worst over rows (the last axis is head_dim, every other index one
    row or key and head) of |g - ref|_max / (rtol (|ref_row|_max + floor) +
    slack_row); at most 1 when every row is inside its bound."""
    if ref.size == 0:
        return 0.0
    g = got.detach().float().cpu().numpy().astype(np.float64) if hasattr(got, "detach") else np.asarray(got)
    floor = ROW_FLOOR * max(float(np.abs(ref).max()), 1e-30)
    err = np.abs(g - ref).max(axis=-1)
    bound = rtol * (np.abs(ref).max(axis=-1) + floor)
    if slack is not None:
        bound = bound + slack
    return float((err / bound).max())


def delta_slack(q, k, v, dout, n_img, cu, P, r, split="head_tail", rows=None):
    """Per (row, head) of dq [len(rows) or R, H]: how far the forward output's
    error moves dq_i through Delta (see ROW_RTOL's note), from the oracle:
    |dDelta_i| |(P k)_i|_max / sqrt(D), with |dDelta_i| <= 2u sum_d |dout_id
    out_id| for bf16 inputs and <= 1e-5 sum_d |dout_id| for fp32 inputs (the
    fp32 forward is tested to 1e-5 max-abs)."""
    D = q.shape[2]
    o, _ = oracle.rank_attention(q, k, v, n_img, cu, P, r, local_rows=rows, split=split)
    pk, _ = oracle.rank_attention(q, k, k, n_img, cu, P, r, local_rows=rows, split=split)
    do = dout.double().numpy() if hasattr(dout, "double") else np.asarray(dout, np.float64)
    if rows is not None:
        do = do[np.asarray(rows)]
    if dout.dtype == torch.float32:
        d_delta = 1e-5 * np.abs(do).sum(axis=-1)
    else:
        d_delta = 2 * U_BF16 * np.abs(do * o).sum(axis=-1)
    return d_delta * np.abs(pk).max(axis=-1) / np.sqrt(D)


def run_bwd_case(cp, name, n_img, text, H, Hkv, P, r, split="head_tail", D=128, dtype=torch.bfloat16):
    lens = np.array(n_img) + np.array(text)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    img = np.array(n_img, np.int32)
    idx, _ = oracle.partition_index(T, img, cu, P, r, split)
    q, k, v, dout = draw(zlib.crc32(name.encode()) % 1000 + r, T, H, Hkv, D, len(idx), dtype)
    # pad rows carry no gradient (their forward output is a constant 0)
    dout[torch.from_numpy(idx < 0)] = 0
    print(f"bwd case {name} T={T} H={H} Hkv={Hkv} D={D} {dtype} P={P} r={r} split={split} R={len(idx)}",
          flush=True)
    qd, kd, vd, dd = (t.to(DEV) for t in (q, k, v, dout))
    out, lse = cp.rank_fwd(qd, kd, vd, cp_size=P, cp_rank=r, n_img=img, cu_seqlens=cu, split=split)
    dq, dk, dv = cp.rank_bwd(qd, kd, vd, out, lse, dd, cp_size=P, cp_rank=r, n_img=img, cu_seqlens=cu,
                             split=split)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.rank_attention_backward(q, k, v, dout, img, cu, P, r, split)
    errs = (rel_err(dq, rq), rel_err(dk, rk), rel_err(dv, rv))
    row_tol = ROW_RTOL_F32 if dtype == torch.float32 else ROW_RTOL
    slack = delta_slack(q, k, v, dout, img, cu, P, r, split)
    rows = (row_err(dq, rq, row_tol, slack), row_err(dk, rk, row_tol), row_err(dv, rv, row_tol))
    print(f"  rel max-abs error dq {errs[0]:.2e} dk {errs[1]:.2e} dv {errs[2]:.2e}; per row/key, "
          f"fraction of the bound: dq {rows[0]:.2f} dk {rows[1]:.2f} dv {rows[2]:.2f}", flush=True)
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()
    assert torch.all(dq[torch.from_numpy(idx < 0).to(DEV)] == 0)
    tol = BWD_RTOL_F32 if dtype == torch.float32 else BWD_RTOL
    assert max(errs) <= tol, (name, r, errs)
    assert max(rows) <= 1.0, (name, r, rows)
    return errs


CASES = [
    # (name, n_img, text, H, Hkv, P)
    ("bwd-text-gqa4", [0], [700], 8, 2, 2),
    ("bwd-text-mha", [0], [500], 4, 4, 3),
    ("bwd-image-gqa2", [37], [300], 4, 2, 2),
    ("bwd-packed-gqa3", [12, 0, 5], [200, 77, 130], 6, 2, 4),
    ("bwd-P1", [0], [333], 4, 1, 1),
    ("bwd-P8-short", [3], [100], 4, 4, 8),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_all_ranks(cp, case):
    name, n_img, text, H, Hkv, P = case
    for r in range(P):
        run_bwd_case(cp, name, n_img, text, H, Hkv, P, r)


FMA_CASES = [
    # (name, n_img, text, H, Hkv, P, D, dtype): the fp32 FMA kernels
    ("bwd-f32-d128", [0], [300], 4, 2, 2, 128, torch.float32),
    ("bwd-f32-d64-image", [21], [250], 4, 4, 3, 64, torch.float32),
    ("bwd-f32-d64-packed", [5, 0], [130, 77], 4, 1, 2, 64, torch.float32),
    ("bwd-bf16-d64-gqa2", [9], [400], 8, 4, 4, 64, torch.bfloat16),
]


@pytest.mark.parametrize("case", FMA_CASES, ids=[c[0] for c in FMA_CASES])
def test_backward_fma_path_all_ranks(cp, case):
    name, n_img, text, H, Hkv, P, D, dtype = case
    for r in range(P):
        run_bwd_case(cp, name, n_img, text, H, Hkv, P, r, D=D, dtype=dtype)


def test_backward_contiguous_split(cp):
    for r in range(3):
        run_bwd_case(cp, "bwd-contig", [20], [400], 4, 2, 3, r, split="contiguous")


def test_backward_deterministic(cp):
    T, H, Hkv, D, P, r = 900, 8, 2, 128, 2, 1
    idx, _ = oracle.partition_index(T, None, None, P, r)
    q, k, v, dout = (t.to(DEV) for t in draw(11, T, H, Hkv, D, len(idx)))
    out, lse = cp.rank_fwd(q, k, v, cp_size=P, cp_rank=r)
    bw = cp.RankAttentionBackward(q, k, v, cp_size=P, cp_rank=r)
    a = [t.clone() for t in bw(out, lse, dout)]
    b = bw(out, lse, dout)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))


# ------------------------------------------------ full-size shares, sampled
# At the full workload sizes the oracle computes, one by one, what depends
# on few rows: dq of sampled rank rows (a row's dq depends on that row
# alone), and dk/dv of the last keys of each sample that the rank's rows see
# (only the rows at or after such a key see it). Keys no rank row sees must
# be exactly 0, and sum_keys dv = sum_rows dout per KV head (softmax rows sum
# to 1), within the bf16 rounding of P (unit roundoff 2^-8, doubled).

def _f32(t):
    return t.detach().float().cpu().numpy()


def _exact_dq_rows(q, k, v, dout, idx, cu, rows, H, Hkv):
    D = q.shape[2]
    scale = oracle.softmax_scale(D)
    ids = idx[rows].astype(np.int64)
    smp = np.searchsorted(cu, ids, side="right") - 1
    ref = np.zeros((len(rows), H, D))
    for s in np.unique(smp):
        sel = np.nonzero(smp == s)[0]
        a, b = int(cu[s]), int(cu[s + 1])
        allowed = oracle.visible(np.arange(a, b), ids[sel])
        for h in range(H):
            g = oracle.kv_head_of(h, H, Hkv)
            gq, _, _ = oracle.attend_backward(_f32(q[ids[sel], h]), _f32(k[a:b, g]), _f32(v[a:b, g]), allowed,
                                              scale, _f32(dout[rows[sel], h]))
            ref[sel, h] = gq
    return ref


def _exact_last_keys(q, k, v, dout, idx, cu, s, n_keys, H, Hkv):
    """dk, dv of the last n_keys keys (of sample s) that the rank's rows see."""
    D = q.shape[2]
    scale = oracle.softmax_scale(D)
    a, b = int(cu[s]), int(cu[s + 1])
    ids = idx.astype(np.int64)
    mine = np.nonzero((ids >= a) & (ids < b))[0]
    j0 = max(int(ids[mine].max()) - n_keys + 1, a)
    sel = mine[ids[mine] >= j0]  # every rank row that sees a key >= j0
    allowed = oracle.visible(np.arange(a, b), ids[sel])
    n = int(ids[mine].max()) + 1 - j0
    dk = np.zeros((n, Hkv, D))
    dv = np.zeros_like(dk)
    for h in range(H):
        g = oracle.kv_head_of(h, H, Hkv)
        _, gk, gv = oracle.attend_backward(_f32(q[ids[sel], h]), _f32(k[a:b, g]), _f32(v[a:b, g]), allowed,
                                           scale, _f32(dout[sel, h]))
        dk[:, g] += gk[j0 - a:j0 - a + n]
        dv[:, g] += gv[j0 - a:j0 - a + n]
    return j0, dk, dv


@pytest.mark.parametrize("num", [4, 5])
def test_backward_workload_sampled(cp, num):
    import workloads
    from gpu_common import sample_rows

    w = workloads.get(num)
    q, k, v = workloads.make_inputs(w)
    r = w.ranks[0]
    cu = w.cu_seqlens if w.n_samples > 1 else None
    n_img = w.n_img_array if any(w.n_img) else None
    idx, cu_rows = oracle.partition_index(w.seq_len, n_img, cu, w.cp_size, r)
    H, Hkv, D = w.heads, w.kv_heads, w.head_dim
    rng = np.random.default_rng(w.seed + 7)
    dout = torch.from_numpy(rng.standard_normal((len(idx), H, D), dtype=np.float32)).to(torch.bfloat16)
    dout[torch.from_numpy(idx < 0)] = 0
    print(f"bwd workload {num} rank {r}: R={len(idx)} T={w.seq_len}", flush=True)
    qd, kd, vd, dd = (t.to(DEV) for t in (q, k, v, dout))
    out, lse = cp.rank_fwd(qd, kd, vd, cp_size=w.cp_size, cp_rank=r, n_img=n_img, cu_seqlens=cu)
    bw = cp.RankAttentionBackward(qd, kd, vd, cp_size=w.cp_size, cp_rank=r, n_img=n_img, cu_seqlens=cu)
    dq, dk, dv = (t.clone() for t in bw(out, lse, dd))
    dq2, dk2, dv2 = bw(out, lse, dd)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()
    assert torch.all(dq[torch.from_numpy(idx < 0).to(DEV)] == 0)

    cu64 = np.array([0, w.seq_len], np.int64) if cu is None else np.asarray(cu, np.int64)
    rows = sample_rows(idx, cu_rows, 12, seed=num)
    rows = rows[idx[rows] >= 0]
    ref = _exact_dq_rows(q, k, v, dout, idx, cu64, rows, H, Hkv)
    e = rel_err(dq[torch.as_tensor(rows, device=DEV)], ref)
    slack = delta_slack(q, k, v, dout, n_img, cu, w.cp_size, r, rows=rows)
    e_row = row_err(dq[torch.as_tensor(rows, device=DEV)], ref, ROW_RTOL, slack)
    print(f"  dq on {len(rows)} sampled rows: rel max-abs {e:.2e}, per row {e_row:.2f} of the bound", flush=True)
    assert e <= BWD_RTOL and e_row <= 1.0

    # keys that no rank row sees: exactly zero
    ids = idx.astype(np.int64)
    seen = np.zeros(w.seq_len, bool)
    for s in range(len(cu64) - 1):
        mine = ids[(ids >= cu64[s]) & (ids < cu64[s + 1])]
        if len(mine):
            seen[cu64[s]:mine.max() + 1] = True
    unseen = torch.as_tensor(~seen, device=DEV)
    assert torch.all(dk[unseen] == 0) and torch.all(dv[unseen] == 0)

    for s in range(min(len(cu64) - 1, 3)):
        j0, rk, rv = _exact_last_keys(q, k, v, dout, idx, cu64, s, 24, H, Hkv)
        sl = slice(j0, j0 + rk.shape[0])
        ek, ev = rel_err(dk[sl], rk), rel_err(dv[sl], rv)
        rk_, rv_ = row_err(dk[sl], rk, ROW_RTOL), row_err(dv[sl], rv, ROW_RTOL)
        print(f"  sample {s}: dk/dv of keys [{j0}, {j0 + rk.shape[0]}) rel max-abs {ek:.2e} / {ev:.2e}, "
              f"per key {rk_:.2f} / {rv_:.2f} of the bound", flush=True)
        assert max(ek, ev) <= BWD_RTOL and max(rk_, rv_) <= 1.0

    # sum over keys of dv = sum over the rank's rows of dout, per KV head
    grp = H // Hkv
    do64 = dout.double().numpy().reshape(len(idx), Hkv, grp, D)
    want = do64.sum(axis=(0, 2))
    bound = 2.0 ** -7 * np.abs(do64).sum(axis=(0, 2)) + 1e-3
    got = dv.double().sum(dim=0).cpu().numpy()
    worst = float((np.abs(got - want) / bound).max())
    print(f"  sum_keys dv vs sum_rows dout: worst |diff| / bound {worst:.3f}", flush=True)
    assert worst <= 1.0


@pytest.mark.parametrize("num", [3, 4])
def test_backward_workload_full(cp, num):
    # every element of dq, dk and dv against the oracle's gradients, computed
    # over (KV head, 256-row) tasks in threads (oracle.pool; the row terms of
    # the backward are independent), with the per-tensor and per-row/key
    # bounds of the small cases
    import workloads
    from gpu_common import pooled_oracle
    from oracle.pool import rank_attention_backward_pooled

    w = workloads.get(num)
    q, k, v = workloads.make_inputs(w)
    r = w.ranks[0]
    cu = w.cu_seqlens if w.n_samples > 1 else None
    n_img = w.n_img_array if any(w.n_img) else None
    idx, _ = oracle.partition_index(w.seq_len, n_img, cu, w.cp_size, r)
    H, D = w.heads, w.head_dim
    rng = np.random.default_rng(w.seed + 7)
    dout = torch.from_numpy(rng.standard_normal((len(idx), H, D), dtype=np.float32)).to(torch.bfloat16)
    dout[torch.from_numpy(idx < 0)] = 0
    print(f"bwd workload {num} rank {r}: R={len(idx)} T={w.seq_len}, every element", flush=True)
    qd, kd, vd, dd = (t.to(DEV) for t in (q, k, v, dout))
    out, lse = cp.rank_fwd(qd, kd, vd, cp_size=w.cp_size, cp_rank=r, n_img=n_img, cu_seqlens=cu)
    dq, dk, dv = cp.rank_bwd(qd, kd, vd, out, lse, dd, cp_size=w.cp_size, cp_rank=r, n_img=n_img,
                             cu_seqlens=cu)
    torch.cuda.synchronize()
    rq, rk, rv = rank_attention_backward_pooled(q, k, v, dout, n_img, cu, w.cp_size, r)
    print(f"  oracle gradients done", flush=True)
    # the Delta slack of dq (see ROW_RTOL's note), from the pooled oracle's
    # rows of out and of attention with the keys as values
    o, _ = pooled_oracle(q, k, v, n_img, cu, w.cp_size, r)
    pk, _ = pooled_oracle(q, k, k, n_img, cu, w.cp_size, r)
    do = dout.double().numpy()
    slack = 2 * U_BF16 * np.abs(do * o).sum(axis=-1) * np.abs(pk).max(axis=-1) / np.sqrt(D)
    errs = (rel_err(dq, rq), rel_err(dk, rk), rel_err(dv, rv))
    rows = (row_err(dq, rq, ROW_RTOL, slack), row_err(dk, rk, ROW_RTOL), row_err(dv, rv, ROW_RTOL))
    print(f"  rel max-abs error dq {errs[0]:.2e} dk {errs[1]:.2e} dv {errs[2]:.2e}; per row/key, "
          f"fraction of the bound: dq {rows[0]:.2f} dk {rows[1]:.2f} dv {rows[2]:.2f}", flush=True)
    assert max(errs) <= BWD_RTOL and max(rows) <= 1.0


def test_backward_rank_sum_is_the_unsplit_gradient(cp):
    # The reverse ring / all-reduce over the CP group: summing every rank's
    # dk, dv (the image keys' gradients included) and scattering every
    # rank's dq by its index gives the unsplit sequence's gradients. Image
    # rows are replicated on every rank; their loss gradient is carried by
    # rank 0's copy here, so the sum counts it once.
    T_img, T_txt, H, Hkv, D, P = 40, 600, 4, 2, 128, 4
    T = T_img + T_txt
    img = np.array([T_img], np.int32)
    rng = np.random.default_rng(21)
    q, k, v = (torch.from_numpy(rng.standard_normal((T, h, D), dtype=np.float32)).to(torch.bfloat16)
               for h in (H, Hkv, Hkv))
    dfull = torch.from_numpy(rng.standard_normal((T, H, D), dtype=np.float32)).to(torch.bfloat16)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    dq_sum = torch.zeros(T, H, D, dtype=torch.float64)
    dk_sum = torch.zeros(T, Hkv, D, dtype=torch.float64)
    dv_sum = torch.zeros(T, Hkv, D, dtype=torch.float64)
    for r in range(P):
        idx, _ = oracle.partition_index(T, img, None, P, r)
        ids = torch.from_numpy(np.maximum(idx, 0).astype(np.int64))
        dout = dfull[ids].clone()
        dout[torch.from_numpy(idx < 0)] = 0
        if r > 0:
            dout[:T_img] = 0  # image rows: rank 0's copy carries the gradient
        out, lse = cp.rank_fwd(qd, kd, vd, cp_size=P, cp_rank=r, n_img=img)
        dq, dk, dv = cp.rank_bwd(qd, kd, vd, out, lse, dout.to(DEV), cp_size=P, cp_rank=r, n_img=img)
        torch.cuda.synchronize()
        real = torch.from_numpy(idx >= 0)
        dq_sum.index_add_(0, ids[real], dq.double().cpu()[real])
        dk_sum += dk.double().cpu()
        dv_sum += dv.double().cpu()
    out1, lse1 = cp.rank_fwd(qd, kd, vd, cp_size=1, cp_rank=0, n_img=img)
    g1 = cp.rank_bwd(qd, kd, vd, out1, lse1, dfull.to(DEV), cp_size=1, cp_rank=0, n_img=img)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.rank_attention_backward(q, k, v, dfull, img, None, 1, 0)
    for name, s, one, ref in (("dq", dq_sum, g1[0], rq), ("dk", dk_sum, g1[1], rk), ("dv", dv_sum, g1[2], rv)):
        e_sum = rel_err(s, ref)
        e_one = rel_err(one, ref)
        print(f"  {name}: rank sum vs oracle {e_sum:.2e}, unsplit GPU vs oracle {e_one:.2e}", flush=True)
        assert e_sum <= BWD_RTOL and e_one <= BWD_RTOL
    # the image keys' gradients come from every rank's text rows
    assert float(dk_sum[:T_img].abs().sum()) > 0
