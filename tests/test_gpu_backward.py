"""GPU parity of the per-rank backward (cp_attn_rank_bwd) against the fp64
oracle's gradients (oracle.rank_attention_backward).

Inputs q, k, v and dout are bf16 (the oracle reads the same values); out
and lse come from the library's own forward, as in training. The bound is
max-abs error relative to the largest reference gradient of the tensor.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
# |g - g_ref|_max <= BWD_RTOL * max(|g_ref|_max, 1)
BWD_RTOL = 2e-2


@pytest.fixture(scope="module")
def cp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_parallelism_amd as m
    return m


def draw(seed, T, H, Hkv, D, R):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, D), dtype=np.float32)
    k = rng.standard_normal((T, Hkv, D), dtype=np.float32)
    v = rng.standard_normal((T, Hkv, D), dtype=np.float32)
    dout = rng.standard_normal((R, H, D), dtype=np.float32)
    return [torch.from_numpy(a).to(torch.bfloat16) for a in (q, k, v, dout)]


def rel_err(got, ref):
    g = got.detach().float().cpu().numpy().astype(np.float64)
    scale = max(float(np.abs(ref).max()) if ref.size else 0.0, 1.0)
    return float(np.abs(g - ref).max()) / scale if ref.size else 0.0


def run_bwd_case(cp, name, n_img, text, H, Hkv, P, r, split="head_tail"):
    D = 128
    lens = np.array(n_img) + np.array(text)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    img = np.array(n_img, np.int32)
    idx, _ = oracle.partition_index(T, img, cu, P, r, split)
    q, k, v, dout = draw(zlib.crc32(name.encode()) % 1000 + r, T, H, Hkv, D, len(idx))
    # pad rows carry no gradient (their forward output is a constant 0)
    dout[torch.from_numpy(idx < 0)] = 0
    print(f"bwd case {name} T={T} H={H} Hkv={Hkv} P={P} r={r} split={split} R={len(idx)}", flush=True)
    qd, kd, vd, dd = (t.to(DEV) for t in (q, k, v, dout))
    out, lse = cp.rank_fwd(qd, kd, vd, cp_size=P, cp_rank=r, n_img=img, cu_seqlens=cu, split=split)
    dq, dk, dv = cp.rank_bwd(qd, kd, vd, out, lse, dd, cp_size=P, cp_rank=r, n_img=img, cu_seqlens=cu,
                             split=split)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.rank_attention_backward(q, k, v, dout, img, cu, P, r, split)
    errs = (rel_err(dq, rq), rel_err(dk, rk), rel_err(dv, rv))
    print(f"  rel max-abs error dq {errs[0]:.2e} dk {errs[1]:.2e} dv {errs[2]:.2e}", flush=True)
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()
    assert torch.all(dq[torch.from_numpy(idx < 0).to(DEV)] == 0)
    assert max(errs) <= BWD_RTOL, (name, r, errs)
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
