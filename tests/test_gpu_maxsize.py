"""Maximum-size parity: one rank's share of a 300,007-token sequence whose
Q, K and V tensors each exceed 2 GiB (300,007 tokens x 32 heads x 128 x
bf16 = 2.46 GB), so every global address past 2^31 bytes is exercised. The
length is ragged: at P = 8 the chunks hold 18,751 tokens and the last one
ends in 9 pad rows, which rank 0 holds (chunk 0 and chunk 15, the head-tail
pair of the context-parallel multimodal page, section 1.1).

Inputs are drawn on the device (workloads.draw_on_device). The fp64 oracle
computes sampled rows and keys one by one from slices read back to the host:
forward out/lse of sampled rows for three heads, backward dq of sampled rows
and dk/dv of the last keys for two heads, plus sum_keys dv = sum_rows dout
for every head.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_common import TOL, sample_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
T, H, HKV, D, P, RANK = 300_007, 32, 32, 128, 8, 0
BWD_RTOL = 2e-2  # as for the other bf16 backward tests


@pytest.fixture(scope="module")
def cp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_parallelism_amd as m
    return m


@pytest.fixture(scope="module")
def big(cp):
    q, k, v = workloads.draw_on_device([(T, H, D), (T, HKV, D), (T, HKV, D)], seed=4242)
    assert k.numel() * k.element_size() > 2 ** 31 and q.numel() * q.element_size() > 2 ** 31
    idx, cu_rows = oracle.partition_index(T, None, None, P, RANK)
    assert (idx < 0).sum() == 9 and idx.max() == T - 1
    print(f"max-size problem: T={T} R={len(idx)} K bytes={k.numel() * 2}", flush=True)
    yield q, k, v, idx, cu_rows
    del q, k, v
    torch.cuda.empty_cache()


def _f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def test_maxsize_forward_sampled(cp, big):
    q, k, v, idx, cu_rows = big
    ra = cp.RankAttention(q, k, v, cp_size=P, cp_rank=RANK)
    ra.out.fill_(float("nan"))  # canary: every row must be overwritten
    ra.lse.fill_(float("nan"))
    out, lse = ra()
    torch.cuda.synchronize()
    assert not torch.isnan(out).any() and not torch.isnan(lse).any()
    pads = torch.as_tensor(idx < 0, device=DEV)
    assert torch.all(out[pads] == 0) and torch.all(torch.isneginf(lse[:, pads]))
    assert torch.isfinite(lse[:, ~pads]).all()

    rows = sample_rows(idx, cu_rows, 24, seed=7)
    rows = rows[idx[rows] >= 0]
    ids = idx[rows].astype(np.int64)
    hi = int(ids.max()) + 1
    allowed = oracle.visible(np.arange(hi), ids)
    scale = oracle.softmax_scale(D)
    rt = torch.as_tensor(rows, device=DEV)
    tol_o, tol_l = TOL["bf16"]
    for h in (0, 13, 31):
        g = oracle.kv_head_of(h, H, HKV)
        ro, rl = oracle.attend(_f64(q[torch.as_tensor(ids, device=DEV), h]), _f64(k[:hi, g]), _f64(v[:hi, g]),
                               allowed, scale)
        eo = float(np.abs(_f64(out[rt, h]) - ro).max())
        el = float(np.abs(_f64(lse[h, rt]) - rl).max())
        print(f"  head {h}: {len(rows)} rows, out max-abs {eo:.3e}, lse max-abs {el:.3e}", flush=True)
        assert eo <= tol_o and el <= tol_l


def test_maxsize_backward_sampled(cp, big):
    q, k, v, idx, cu_rows = big
    R = len(idx)
    (dout,) = workloads.draw_on_device([(R, H, D)], seed=4243)
    dout[torch.as_tensor(idx < 0, device=DEV)] = 0
    out, lse = cp.rank_fwd(q, k, v, cp_size=P, cp_rank=RANK)
    bw = cp.RankAttentionBackward(q, k, v, cp_size=P, cp_rank=RANK)
    dq, dk, dv = bw(out, lse, dout)
    torch.cuda.synchronize()
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()
    assert torch.all(dq[torch.as_tensor(idx < 0, device=DEV)] == 0)
    scale = oracle.softmax_scale(D)

    def rel(got, ref):
        return float(np.abs(_f64(got) - ref).max()) / max(float(np.abs(ref).max()), 1.0)

    # dq of sampled rows: a row's dq depends on that row alone
    rows = sample_rows(idx, cu_rows, 8, seed=8)
    rows = rows[idx[rows] >= 0]
    ids = idx[rows].astype(np.int64)
    hi = int(ids.max()) + 1
    allowed = oracle.visible(np.arange(hi), ids)
    rt, it = torch.as_tensor(rows, device=DEV), torch.as_tensor(ids, device=DEV)
    for h in (0, 31):
        g = oracle.kv_head_of(h, H, HKV)
        gq, _, _ = oracle.attend_backward(_f64(q[it, h]), _f64(k[:hi, g]), _f64(v[:hi, g]), allowed, scale,
                                          _f64(dout[rt, h]))
        e = rel(dq[rt, h], gq)
        print(f"  dq head {h}: {len(rows)} rows, rel max-abs {e:.2e}", flush=True)
        assert e <= BWD_RTOL

    # dk, dv of the last 24 keys: only rank rows at or after them see them
    all_ids = idx.astype(np.int64)
    j0 = T - 24
    sel = np.nonzero(all_ids >= j0)[0]
    allowed = oracle.visible(np.arange(T), all_ids[sel])
    st, it = torch.as_tensor(sel, device=DEV), torch.as_tensor(all_ids[sel], device=DEV)
    for h in (0, 31):
        g = oracle.kv_head_of(h, H, HKV)
        _, gk, gv = oracle.attend_backward(_f64(q[it, h]), _f64(k[:, g]), _f64(v[:, g]), allowed, scale,
                                           _f64(dout[st, h]))
        ek, ev = rel(dk[j0:, g], gk[j0:]), rel(dv[j0:, g], gv[j0:])
        print(f"  dk/dv head {h}: keys [{j0}, {T}), rel max-abs {ek:.2e} / {ev:.2e}", flush=True)
        assert max(ek, ev) <= BWD_RTOL

    # softmax rows sum to 1: sum over keys of dv = sum over rows of dout, per head
    want = dout.double().sum(dim=0)
    bound = 2.0 ** -7 * dout.double().abs().sum(dim=0) + 1e-3
    worst = float(((dv.double().sum(dim=0) - want).abs() / bound).max())
    print(f"  sum_keys dv vs sum_rows dout: worst |diff| / bound {worst:.3f}", flush=True)
    assert worst <= 1.0
