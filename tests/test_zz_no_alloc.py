"""cp_attn_rank_fwd_noalloc (a static device scratch instead of a caller
workspace; no allocation) against cp_attn_rank_fwd through the C ABI: two
calls in a row, the second on a smaller problem, for each kernel family;
bit-identical to the workspace entry point under the same schedule, and
within the bf16 / fp32 tolerances of the default one."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_common import TOL

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
I32P = ctypes.POINTER(ctypes.c_int32)


@pytest.fixture(scope="module")
def cp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_parallelism_amd as m
    return m


def problem(seed, n_img, text, H, Hkv, D, dtype):
    n_img = np.asarray(n_img, np.int32)
    cu = np.concatenate([[0], np.cumsum(n_img + np.asarray(text))]).astype(np.int32)
    T = int(cu[-1])
    rng = np.random.default_rng(seed)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(rng.standard_normal((T, h, D), dtype=np.float32)).to(dt).to(DEV)
               for h in (H, Hkv, Hkv))
    return q, k, v, n_img, cu


def noalloc(cp, q, k, v, n_img, cu, P, r):
    T, H, D = q.shape
    Hkv = k.shape[1]
    idx, _ = cp.partition_index(T, n_img, cu, cp_size=P, cp_rank=r)
    R = len(idx)
    out = torch.full((R, H, D), float("nan"), dtype=q.dtype, device=DEV)
    lse = torch.full((H, R), float("nan"), dtype=torch.float32, device=DEV)
    code = cp.CP_DTYPE_BF16 if q.dtype == torch.bfloat16 else cp.CP_DTYPE_F32
    st = cp.cp_attn_rank_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), code, T,
                                     n_img.ctypes.data_as(I32P), cu.ctypes.data_as(I32P), len(cu) - 1, P, r,
                                     H, Hkv, D, out.data_ptr(), lse.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)
    cp.check(st, "cp_attn_rank_fwd_noalloc")
    torch.cuda.synchronize()
    return out, lse


# (name, [(n_img, text, P, r) for the first and the second, smaller call], H, Hkv, D, dtype)
FAMILIES = [
    ("bf16-d128-gqa4", [([300, 0, 41], [5000, 700, 2300], 4, 1), ([17], [900], 2, 0)], 8, 2, 128, "bf16"),
    ("bf16-d128-mha", [([0], [6000], 8, 5), ([0, 9], [300, 200], 3, 2)], 4, 4, 128, "bf16"),
    ("f32-d64", [([20, 0], [900, 333], 3, 2), ([0], [150], 2, 1)], 2, 2, 64, "f32"),
    ("bf16-d64-gqa2", [([64], [1500], 4, 3), ([5], [200], 2, 0)], 4, 2, 64, "bf16"),
]


@pytest.mark.parametrize("fam", FAMILIES, ids=[f[0] for f in FAMILIES])
def test_noalloc_matches_workspace_entry_point(cp, fam):
    name, calls, H, Hkv, D, dtype = fam
    schedule = "row_tile" if (dtype == "bf16" and D == 128) else "per_step"
    for i, (n_img, text, P, r) in enumerate(calls):
        q, k, v, img, cu = problem(100 + i, n_img, text, H, Hkv, D, dtype)
        print(f"noalloc {name} call {i}: T={q.shape[0]} P={P} r={r} schedule={schedule}", flush=True)
        got_o, got_l = noalloc(cp, q, k, v, img, cu, P, r)
        ref_o, ref_l = cp.rank_fwd(q, k, v, cp_size=P, cp_rank=r, n_img=img, cu_seqlens=cu, schedule=schedule)
        torch.cuda.synchronize()
        assert torch.equal(got_o, ref_o) and torch.equal(got_l, ref_l), (name, i)
        # and the default entry point (which may pick the other schedule)
        auto_o, auto_l = cp.rank_fwd(q, k, v, cp_size=P, cp_rank=r, n_img=img, cu_seqlens=cu)
        torch.cuda.synchronize()
        tol_o, tol_l = TOL[dtype]
        fin = torch.isfinite(auto_l)
        assert torch.equal(fin, torch.isfinite(got_l))
        assert (got_o.float() - auto_o.float()).abs().max().item() <= tol_o
        assert (got_l[fin] - auto_l[fin]).abs().max().item() <= tol_l


def test_noalloc_refuses_a_plan_beyond_its_scratch(cp):
    # 3M rank rows need 24 MB of row index and step masks: refused before any
    # device work (the pointers are never read)
    fake = ctypes.c_void_p(4096)
    T = 3_000_000
    st = cp.cp_attn_rank_fwd_noalloc(fake, fake, fake, cp.CP_DTYPE_BF16, T, None, None, 1, 1, 0, 2, 2, 128,
                                     fake, fake, None)
    assert st == cp.CP_ENOSPC
