"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle.

Small problems, and workloads 2-5 at full size (3, 4 and 5 under both
schedules), are compared on every output element. Whole-output properties
are checked too: pad rows exact, no row left unwritten, determinism, image
rows identical across ranks, reassembly over ranks.
"""
import ctypes
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads

from gpu_common import TOL, compare, oracle_rows, pooled_oracle, sample_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def cp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_parallelism_amd as m
    return m


def draw(seed, T, H, Hkv, D, dtype, q_scale=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, D), dtype=np.float32) * np.float32(q_scale)
    k = rng.standard_normal((T, Hkv, D), dtype=np.float32)
    v = rng.standard_normal((T, Hkv, D), dtype=np.float32)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    return [torch.from_numpy(a).to(dt) for a in (q, k, v)]


def run_case(cp, q, k, v, n_img, cu, P, r, dtype, rows=None, what="", split="head_tail",
             schedule="auto"):
    print(f"case {what} T={q.shape[0]} H={q.shape[1]} Hkv={k.shape[1]} D={q.shape[2]} P={P} r={r} "
          f"dtype={dtype} split={split} schedule={schedule}", flush=True)
    out, lse = cp.rank_fwd(q.to(DEV), k.to(DEV), v.to(DEV), cp_size=P, cp_rank=r, n_img=n_img,
                           cu_seqlens=cu, split=split, schedule=schedule)
    torch.cuda.synchronize()
    if rows is None:
        ro, rl = oracle_rows(q, k, v, n_img, cu, P, r, split=split)
        return compare(out, lse, ro, rl, dtype, what)
    ro, rl = oracle_rows(q, k, v, n_img, cu, P, r, rows, split=split)
    return compare(out[torch.as_tensor(rows, device=DEV)], lse[:, torch.as_tensor(rows, device=DEV)],
                   ro, rl, dtype, what)


# --------------------------------------------------------------- gather and merge alone


def test_gather_bitexact(cp):
    for dtype, (T, H, D), cu in (("bf16", (300, 4, 128), [0, 100, 163, 300]),
                                 ("f32", (77, 2, 64), [0, 30, 50, 77])):
        q, _, _ = draw(7, T, H, 1, D, dtype)
        n_img, cu = np.array([5, 0, 17]), np.array(cu)
        idx, _ = oracle.partition_index(T, n_img, cu, 3, 1)
        got = cp.gather_rows(q.to(DEV), idx).cpu()
        want = torch.zeros((len(idx), H, D), dtype=q.dtype)
        want[idx >= 0] = q[idx[idx >= 0]]
        assert torch.equal(got, want)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_merge_vs_oracle(cp, dtype):
    # partials from the oracle over a random split of each row's keys into
    # S blocks (some rows miss some blocks); the merge must give the oracle's
    # full result
    rng = np.random.default_rng(11)
    T, H, D, S = 96, 3, 128, 5
    q, k, v = (rng.standard_normal((T, H, D)) for _ in range(3))
    full_o, full_l = oracle.causal_attention(q, k, v)
    block = rng.integers(0, S, size=T)
    po = np.zeros((S, T, H, D), np.float32)
    pl = np.full((S, H, T), -np.inf, np.float32)
    for s in range(S):
        allowed = oracle.visible(np.arange(T), np.arange(T)) & (block[None, :] == s)
        for h in range(H):
            o, l = oracle.attend(q[:, h], k[:, h], v[:, h], allowed, oracle.softmax_scale(D))
            po[s, :, h] = o
            pl[s, h] = l
    mask = np.zeros(T, np.uint32)
    for s in range(S):
        mask |= (np.isfinite(pl[s]).any(axis=0).astype(np.uint32) << s)
    mask[-3:] = 0  # rows with no partial: 0 / -inf
    full_o[-3:] = 0
    full_l[:, -3:] = -np.inf
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    out, lse = cp.lse_merge(torch.from_numpy(po).to(DEV), torch.from_numpy(pl).to(DEV), mask, dt)
    torch.cuda.synchronize()
    # fp32 partials carry ~1e-7 rounding; the bound is the fp32 one
    compare(out, lse, full_o, full_l, "f32" if dtype == "f32" else "bf16", f"merge {dtype}")


# --------------------------------------------------------------- small problems, every output

SMALL = [
    # (name, n_img, text, H, Hkv, D, P, dtype)
    ("text-one-tile", [0], [40], 2, 2, 64, 2, "f32"),
    ("text-ragged", [0], [1000], 4, 2, 128, 3, "f32"),
    ("image-text", [37], [500], 2, 1, 64, 4, "f32"),
    ("packed", [5, 0, 13, 64], [90, 33, 1, 200], 2, 2, 128, 2, "f32"),
    ("bf16-text", [0], [1000], 4, 4, 128, 3, "bf16"),
    ("bf16-gqa4", [0], [777], 8, 2, 128, 2, "bf16"),
    ("bf16-gqa2", [19], [600], 4, 2, 128, 4, "bf16"),
    ("bf16-gqa8", [0], [513], 8, 1, 128, 1, "bf16"),
    ("bf16-d64", [70], [300], 4, 4, 64, 2, "bf16"),
    ("bf16-packed", [33, 0, 130, 7], [260, 45, 3, 700], 4, 4, 128, 4, "bf16"),
    ("bf16-all-image", [64, 100], [0, 129], 2, 2, 128, 2, "bf16"),
    ("bf16-P8-short", [0, 3], [9, 100], 2, 2, 128, 8, "bf16"),
    ("bf16-P32-gqa4", [0], [3000], 4, 1, 128, 32, "bf16"),
    ("bf16-gqa3", [11], [900], 6, 2, 128, 3, "bf16"),
    # head_dim 64 with 2 and 4 query heads per KV head in one workgroup
    ("bf16-d64-gqa2-image", [23], [700], 4, 2, 64, 3, "bf16"),
    ("bf16-d64-gqa4-image", [50], [400], 4, 1, 64, 4, "bf16"),
    ("bf16-d64-gqa4-packed", [9, 0, 40], [300, 77, 500], 8, 2, 64, 2, "bf16"),
    ("bf16-d64-gqa2-packed", [0, 17], [130, 260], 8, 4, 64, 3, "bf16"),
]


def schedules_of(dtype, head_dim):
    """bf16 head_dim 128 has both schedules (whole row tiles with the merge in
    the kernel, or one ring step per workgroup and a merge pass); the other
    shapes have the per-step kernels only."""
    return ("row_tile", "per_step") if (dtype == "bf16" and head_dim == 128) else ("per_step",)


def with_schedules(cases):
    pairs = [(c, m) for c in cases for m in schedules_of(c[7], c[5])]
    return pairs, [f"{c[0]}-{m}" for c, m in pairs]


SMALL_SCHED, SMALL_IDS = with_schedules(SMALL)


@pytest.mark.parametrize("case,schedule", SMALL_SCHED, ids=SMALL_IDS)
def test_small_all_ranks(cp, case, schedule):
    name, n_img, text, H, Hkv, D, P, dtype = case
    lens = np.array(n_img) + np.array(text)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q, k, v = draw(zlib.crc32(name.encode()) % 1000, T, H, Hkv, D, dtype)
    for r in range(P):
        run_case(cp, q, k, v, np.array(n_img, np.int32), cu, P, r, dtype, what=f"{name} r={r}",
                 schedule=schedule)


CONTIGUOUS = [
    ("contig-f32", [0], [1000], 4, 2, 128, 3, "f32"),
    ("contig-bf16-packed", [21, 0, 40], [700, 90, 333], 8, 2, 128, 4, "bf16"),
    ("contig-bf16-d64", [0], [500], 4, 4, 64, 2, "bf16"),
]
CONTIG_SCHED, CONTIG_IDS = with_schedules(CONTIGUOUS)


@pytest.mark.parametrize("case,schedule", CONTIG_SCHED, ids=CONTIG_IDS)
def test_contiguous_split_all_ranks(cp, case, schedule):
    # the plain P-way split (section 1.1's unbalanced baseline) through the same kernels
    name, n_img, text, H, Hkv, D, P, dtype = case
    lens = np.array(n_img) + np.array(text)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q, k, v = draw(zlib.crc32(name.encode()) % 1000, T, H, Hkv, D, dtype)
    for r in range(P):
        run_case(cp, q, k, v, np.array(n_img, np.int32), cu, P, r, dtype, what=f"{name} r={r}",
                 split="contiguous", schedule=schedule)


@pytest.mark.parametrize("schedule", ["row_tile", "per_step"])
def test_peaky_softmax(cp, schedule):
    q, k, v = draw(5, 700, 4, 4, 128, "bf16", q_scale=8.0)
    for r in range(2):
        run_case(cp, q, k, v, None, None, 2, r, "bf16", what=f"peaky r={r}", schedule=schedule)


def test_row_tile_schedule_is_refused_where_it_does_not_exist(cp):
    q = torch.zeros(64, 2, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(cp.CpError):
        cp.rank_fwd(q, q, q, cp_size=2, cp_rank=0, schedule="row_tile")
    q = torch.zeros(64, 2, 128, dtype=torch.float32, device=DEV)
    with pytest.raises(cp.CpError):
        cp.rank_fwd(q, q, q, cp_size=2, cp_rank=0, schedule="row_tile")


def test_unsuffixed_entry_points_on_device(cp):
    # cp_attn_rank_fwd and cp_attn_rank_fwd_timed (NULL events) called
    # directly with device pointers: every rank of an image + packed GQA
    # problem against the oracle, and bit-identical to the _ex entry point
    # with the default split and schedule
    n_img = np.array([31, 0, 12], np.int32)
    text = [400, 95, 611]
    cu = np.concatenate([[0], np.cumsum(n_img + np.array(text))]).astype(np.int32)
    T, H, Hkv, D, P = int(cu[-1]), 8, 2, 128, 3
    q, k, v = draw(77, T, H, Hkv, D, "bf16")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    I32 = ctypes.POINTER(ctypes.c_int32)
    cu_p, img_p = cu.ctypes.data_as(I32), n_img.ctypes.data_as(I32)
    stream = torch.cuda.current_stream().cuda_stream
    for r in range(P):
        rows = ctypes.c_int64(0)
        cp.check(cp.cp_partition_index(T, img_p, cu_p, 3, P, r, None, 0, ctypes.byref(rows), None),
                 "cp_partition_index")
        R = rows.value
        ws_bytes = ctypes.c_size_t(0)
        cp.check(cp.cp_attn_rank_workspace_size(T, img_p, cu_p, 3, P, r, H, Hkv, D, cp.CP_DTYPE_BF16,
                                                ctypes.byref(ws_bytes)), "cp_attn_rank_workspace_size")
        ws = torch.empty(max(ws_bytes.value, 256), dtype=torch.uint8, device=DEV)
        outs = []
        for fn in ("plain", "timed"):
            out = torch.full((R, H, D), float("nan"), dtype=torch.bfloat16, device=DEV)
            lse = torch.full((H, R), float("nan"), dtype=torch.float32, device=DEV)
            args = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), cp.CP_DTYPE_BF16, T, img_p, cu_p, 3, P, r,
                    H, Hkv, D, out.data_ptr(), lse.data_ptr(), ws.data_ptr(), ws_bytes.value, stream)
            st = cp.cp_attn_rank_fwd(*args) if fn == "plain" else cp.cp_attn_rank_fwd_timed(*args, None)
            cp.check(st, "cp_attn_rank_fwd")
            torch.cuda.synchronize()
            outs.append((out, lse))
        ro, rl = oracle_rows(q, k, v, n_img, cu, P, r)
        compare(outs[0][0], outs[0][1], ro, rl, "bf16", f"cp_attn_rank_fwd r={r}")
        ex_out, ex_lse = cp.rank_fwd(qd, kd, vd, cp_size=P, cp_rank=r, n_img=n_img, cu_seqlens=cu)
        torch.cuda.synchronize()
        for out, lse in outs:
            assert torch.equal(out, ex_out) and torch.equal(lse, ex_lse)


def test_empty_input(cp):
    # no samples, no rows: the call succeeds and returns empty outputs
    q = torch.empty((0, 2, 128), dtype=torch.bfloat16, device=DEV)
    out, lse = cp.rank_fwd(q, q[:, :1].contiguous(), q[:, :1].contiguous(), cp_size=2, cp_rank=1,
                           cu_seqlens=np.array([0], np.int32))
    torch.cuda.synchronize()
    assert out.shape == (0, 2, 128) and lse.shape == (2, 0)


# --------------------------------------------------------------- the five workloads


def workload_inputs(num, device=None):
    w = workloads.get(num)
    return w, workloads.make_inputs(w, device=device)


def test_workload2_both_schedules_agree(cp):
    # the two bf16 head_dim-128 schedules on one full-size share: same rows to
    # within the bf16 bound, pads identical
    w, (q, k, v) = workload_inputs(2)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    res = []
    for schedule in ("row_tile", "per_step"):
        out, lse = cp.rank_fwd(qd, kd, vd, cp_size=w.cp_size, cp_rank=1, schedule=schedule)
        torch.cuda.synchronize()
        res.append((out.float().cpu(), lse.cpu()))
    assert (res[0][0] - res[1][0]).abs().max().item() <= TOL["bf16"][0]
    assert (res[0][1] - res[1][1]).abs().max().item() <= TOL["bf16"][1]


def test_workload1_full(cp):
    w, (q, k, v) = workload_inputs(1)
    for r in range(w.cp_size):
        run_case(cp, q, k, v, None, None, w.cp_size, r, w.dtype, what=f"w1 r={r}")


def run_workload_share(cp, num, r, q, k, v, qd, kd, vd):
    """One rank share of a workload in bench's launch configuration (the
    default split and schedule), with whole-output checks: every row
    written (NaN canary), pad rows exact, bit-identical on repeat."""
    w = workloads.get(num)
    cu = w.cu_seqlens if w.n_samples > 1 else None
    n_img = w.n_img_array if any(w.n_img) else None
    idx, cu_rows = oracle.partition_index(w.seq_len, n_img, cu, w.cp_size, r)
    ra = cp.RankAttention(qd, kd, vd, cp_size=w.cp_size, cp_rank=r, n_img=n_img, cu_seqlens=cu)
    ra.out.fill_(float("nan"))  # canary: every row must be overwritten
    ra.lse.fill_(float("nan"))
    out, lse = ra()
    torch.cuda.synchronize()
    assert not torch.isnan(out).any() and not torch.isnan(lse).any()
    pads = torch.as_tensor(idx < 0, device=DEV)
    if pads.any():
        assert torch.all(out[pads] == 0) and torch.all(torch.isneginf(lse[:, pads]))
    assert torch.isfinite(lse[:, ~pads]).all()
    out1, lse1 = out.clone(), lse.clone()
    out2, lse2 = ra()  # determinism: bit-identical repeat
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)
    return out1, lse1, idx, cu_rows, n_img, cu


@pytest.mark.parametrize("num", [2, 3, 4, 5])
def test_workload_full(cp, num):
    # every row, every head, every element against the fp64 oracle
    w, (q, k, v) = workload_inputs(num)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    for r in w.ranks:
        out, lse, idx, _, n_img, cu = run_workload_share(cp, num, r, q, k, v, qd, kd, vd)
        print(f"workload {num} rank {r}: GPU done, oracle on all {len(idx)} rows x {w.heads} heads",
              flush=True)
        st = {}
        ro, rl = pooled_oracle(q, k, v, n_img, cu, w.cp_size, r, stats=st)
        eo, el = compare(out, lse, ro, rl, w.dtype, f"workload {num} r={r}")
        print(f"workload {num} rank {r}: max-abs out {eo:.3e} lse {el:.3e} "
              f"(oracle {st['wall_s']:.1f} s on {st['workers']} threads)", flush=True)
        if num != 2:
            # the other schedule on the same share (workload 2 takes it by
            # default): one ring step per workgroup, partials and the merge pass
            del out, lse
            out_s, lse_s = cp.rank_fwd(qd, kd, vd, cp_size=w.cp_size, cp_rank=r, n_img=n_img,
                                       cu_seqlens=cu, schedule="per_step")
            torch.cuda.synchronize()
            eo, el = compare(out_s, lse_s, ro, rl, w.dtype, f"workload {num} r={r} per_step")
            print(f"workload {num} rank {r} per_step: max-abs out {eo:.3e} lse {el:.3e}", flush=True)
            del out_s, lse_s


def test_workload3_image_rows_identical_across_ranks(cp):
    # invariant 3 on the HIP path: every rank's image rows are bit-identical
    w, (q, k, v) = workload_inputs(3)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    n = w.n_img[0]
    ref = None
    for r in range(w.cp_size):
        out, lse = cp.rank_fwd(qd, kd, vd, cp_size=w.cp_size, cp_rank=r, n_img=w.n_img_array)
        torch.cuda.synchronize()
        img = (out[:n].clone(), lse[:, :n].clone())
        if ref is None:
            ref = img
        else:
            assert torch.equal(img[0], ref[0]) and torch.equal(img[1], ref[1]), f"rank {r}"


def test_workload2_reassembly_and_equal_work(cp):
    # invariant 1 (every text row once over the ranks) and invariant 2 (equal
    # per-rank pairs) on the library's own partition, checked against rows
    # computed on one rank-1 call (P = 1: the whole sequence, no split)
    w, (q, k, v) = workload_inputs(2)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    T = w.seq_len
    full_o, full_l = cp.rank_fwd(qd, kd, vd, cp_size=1, cp_rank=0)
    torch.cuda.synchronize()
    seen = np.zeros(T, int)
    pairs = set()
    for r in range(w.cp_size):
        idx, _ = cp.partition_index(T, cp_size=w.cp_size, cp_rank=r)
        pairs.add(cp.pair_counts(T, cp_size=w.cp_size, cp_rank=r))
        out, lse = cp.rank_fwd(qd, kd, vd, cp_size=w.cp_size, cp_rank=r)
        torch.cuda.synchronize()
        it = torch.as_tensor(idx, device=DEV, dtype=torch.long)
        d_o = (out.float() - full_o[it].float()).abs().max().item()
        d_l = (lse - full_l[:, it]).abs().max().item()
        assert d_o <= TOL["bf16"][0] and d_l <= TOL["bf16"][1], (r, d_o, d_l)
        seen[idx] += 1
    assert np.all(seen == 1)
    assert len(pairs) == 1


def test_ulysses_share_matches_ring_and_oracle(cp):
    # the Ulysses layout of the same job (after an all-to-all over heads: all
    # tokens, heads/P) is plain causal attention (cp_size 1) on a head
    # subset; its rows must equal the ring rank shares reassembled, and the
    # oracle on sampled rows
    w, (q, k, v) = workload_inputs(2)
    P = w.cp_size
    hq, hk = w.heads // P, w.kv_heads // P
    qu, ku, vu = q[:, :hq].contiguous(), k[:, :hk].contiguous(), v[:, :hk].contiguous()
    ou, lu = cp.rank_fwd(qu.to(DEV), ku.to(DEV), vu.to(DEV), cp_size=1, cp_rank=0)
    torch.cuda.synchronize()
    idx, cu_rows = oracle.partition_index(w.seq_len, None, None, 1, 0)
    rows = sample_rows(idx, cu_rows, 64, seed=77)
    ro, rl = oracle_rows(qu, ku, vu, None, None, 1, 0, rows)
    rt = torch.as_tensor(rows, device=DEV)
    compare(ou[rt], lu[:, rt], ro, rl, "bf16", "ulysses share")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    for r in range(P):
        ridx, _ = cp.partition_index(w.seq_len, cp_size=P, cp_rank=r)
        out, lse = cp.rank_fwd(qd, kd, vd, cp_size=P, cp_rank=r)
        torch.cuda.synchronize()
        it = torch.as_tensor(ridx, device=DEV, dtype=torch.long)
        d_o = (out[:, :hq].float() - ou[it].float()).abs().max().item()
        d_l = (lse[:hq] - lu[:, it]).abs().max().item()
        assert d_o <= TOL["bf16"][0] and d_l <= TOL["bf16"][1], (r, d_o, d_l)


def test_binding_rejects_mismatched_inputs(cp):
    # the binding hands raw pointers to the kernels: a dtype or shape that
    # does not match must be refused on the host, before any launch
    T, H, Hkv, D, P = 300, 4, 2, 128, 2
    q = torch.zeros(T, H, D, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(T, Hkv, D, dtype=torch.bfloat16, device=DEV)
    v = torch.zeros(T, Hkv, D, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(TypeError):
        cp.RankAttentionBackward(q.float(), k, v, cp_size=P, cp_rank=0)
    with pytest.raises(ValueError):
        cp.RankAttentionBackward(q, k[:-1].contiguous(), v, cp_size=P, cp_rank=0)
    with pytest.raises(ValueError):
        cp.RankAttention(q, k, v[:, :1].contiguous(), cp_size=P, cp_rank=0)
    bw = cp.RankAttentionBackward(q, k, v, cp_size=P, cp_rank=0)
    out, lse = cp.rank_fwd(q, k, v, cp_size=P, cp_rank=0)
    with pytest.raises(TypeError):
        bw(out.float(), lse, out)
    with pytest.raises(TypeError):
        bw(out, lse.double(), out)
    with pytest.raises(ValueError):
        cp.gather_rows(q, np.array([0, T], np.int32))
    with pytest.raises(ValueError):
        cp.gather_rows(q, np.array([-2], np.int32))
    po = torch.zeros(2, 8, H, D, device=DEV)
    with pytest.raises(ValueError):
        cp.lse_merge(po, torch.zeros(2, 8, H, device=DEV), np.zeros(8, np.uint32), torch.bfloat16)
    with pytest.raises(ValueError):
        cp.lse_merge(po, torch.zeros(2, H, 8, device=DEV), np.zeros(7, np.uint32), torch.bfloat16)
    torch.cuda.synchronize()
