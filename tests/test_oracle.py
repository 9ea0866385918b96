"""Pins for the fp64 oracle: page example, closed forms, brute force,
library routines, invariants, and planted mistakes that the pins catch.

All CPU; none of these touch the HIP library.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import cp_oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_qkv(rng, T, H, Hkv, D, scale=1.0):
    q = rng.standard_normal((T, H, D)) * scale
    k = rng.standard_normal((T, Hkv, D))
    v = rng.standard_normal((T, Hkv, D))
    return q, k, v


# ---------------------------------------------------------------- pins


def pin_page_example():
    """Max count of mismatched chunks against the page's CP=2 example."""
    doc = json.load(open(os.path.join(GOLDEN, "partition_page_example.json")))
    P = doc["cp_size"]
    bad = 0
    for c in (1, 3, 5):
        L = 2 * P * c
        for r_s, chunks in doc["chunks_per_rank"].items():
            idx, _ = oracle.partition_index(L, None, None, P, int(r_s))
            want = np.concatenate([np.arange(k * c, (k + 1) * c) for k in chunks])
            bad += int(not np.array_equal(idx, want))
    return bad


def brute_force(q, k, v, cu):
    """Scalar loops with math.fsum: the softmax definition, row by row."""
    T, H, D = q.shape
    Hkv = k.shape[1]
    out = np.zeros((T, H, D))
    lse = np.zeros((H, T))
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        for i in range(a, b):
            for h in range(H):
                g = h * Hkv // H
                sc = [math.fsum(q[i, h, d] * k[j, g, d] for d in range(D)) / math.sqrt(D)
                      for j in range(a, i + 1)]
                m = max(sc)
                w = [math.exp(x - m) for x in sc]
                l = math.fsum(w)
                for d in range(D):
                    out[i, h, d] = math.fsum(w[t] * v[a + t, g, d] for t in range(len(w))) / l
                lse[h, i] = m + math.log(l)
    return out, lse


def pin_brute_force(seed=0):
    rng = np.random.default_rng(seed)
    cu = np.array([0, 5, 12, 13])
    q, k, v = rand_qkv(rng, 13, 4, 2, 3)
    o, l = oracle.causal_attention(q, k, v, cu)
    bo, bl = brute_force(q, k, v, cu)
    return max(np.abs(o - bo).max(), np.abs(l - bl).max())


def torch_reference(q, k, v):
    """torch CPU fp64 flash-attention op (causal): out [T,H,D], lse [H,T]."""
    H, Hkv = q.shape[1], k.shape[1]
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2)[None].repeat_interleave(H // Hkv, dim=1)
    tv = torch.from_numpy(v).permute(1, 0, 2)[None].repeat_interleave(H // Hkv, dim=1)
    o, lse = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
        tq.contiguous(), tk.contiguous(), tv.contiguous(), 0.0, True)[:2]
    sdpa = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2)[None], torch.from_numpy(k).permute(1, 0, 2)[None],
        torch.from_numpy(v).permute(1, 0, 2)[None], is_causal=True, enable_gqa=True)
    assert torch.allclose(o, sdpa, atol=1e-12)
    return o[0].permute(1, 0, 2).numpy(), lse[0].numpy()


def pin_torch(seed=1, T=96, H=8, Hkv=2, D=32, scale=1.0):
    rng = np.random.default_rng(seed)
    q, k, v = rand_qkv(rng, T, H, Hkv, D, scale)
    o, l = oracle.causal_attention(q, k, v)
    to, tl = torch_reference(q, k, v)
    return max(np.abs(o - to).max(), np.abs(l - tl).max())


def pin_packed_blockdiag(seed=2):
    """Packed samples against torch SDPA with an explicit block-diagonal causal mask."""
    rng = np.random.default_rng(seed)
    cu = np.array([0, 17, 18, 40, 64])
    T, H, Hkv, D = 64, 4, 4, 16
    q, k, v = rand_qkv(rng, T, H, Hkv, D)
    sample = np.searchsorted(cu, np.arange(T), side="right") - 1
    mask = (sample[:, None] == sample[None, :]) & (np.arange(T)[None, :] <= np.arange(T)[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2), torch.from_numpy(k).permute(1, 0, 2),
        torch.from_numpy(v).permute(1, 0, 2), attn_mask=torch.from_numpy(mask))
    o, _ = oracle.causal_attention(q, k, v, cu)
    return np.abs(o - ref.permute(1, 0, 2).numpy()).max()


def pin_closed_forms(seed=3):
    """Q = 0: out is the mean of the visible V rows and lse = ln(#visible).
    V = const: out = const."""
    rng = np.random.default_rng(seed)
    cu = np.array([0, 7, 30])
    T, H, Hkv, D = 30, 4, 2, 8
    _, k, v = rand_qkv(rng, T, H, Hkv, D)
    q = np.zeros((T, H, D))
    o, l = oracle.causal_attention(q, k, v, cu)
    err = 0.0
    for s in range(2):
        a, b = cu[s], cu[s + 1]
        for i in range(a, b):
            for h in range(H):
                g = h * Hkv // H
                err = max(err, np.abs(o[i, h] - v[a:i + 1, g].mean(axis=0)).max())
                err = max(err, abs(l[h, i] - math.log(i - a + 1)))
    q2 = rng.standard_normal((T, H, D))
    vc = np.broadcast_to(rng.standard_normal(D), (T, Hkv, D)).copy()
    o2, _ = oracle.causal_attention(q2, k, vc, cu)
    err = max(err, np.abs(o2 - vc[:1, :1]).max())
    return err


def pin_merge_identity(seed=4):
    """Split each row's visible keys into random disjoint blocks, attend per
    block with the oracle, merge by lse: the full result comes back."""
    rng = np.random.default_rng(seed)
    T, D = 40, 8
    q, k, v = rand_qkv(rng, T, 1, 1, D)
    rows = np.arange(T)
    full_o, full_l = oracle.causal_attention(q, k, v)
    nb = 4
    block_of = rng.integers(0, nb, size=T)
    outs, lses = [], []
    for b in range(nb):
        allowed = oracle.visible(np.arange(T), rows) & (block_of[None, :] == b)
        o, l = oracle.attend(q[:, 0], k[:, 0], v[:, 0], allowed, oracle.softmax_scale(D))
        outs.append(o)
        lses.append(l)
    mo, ml = oracle.lse_merge(outs, lses)
    return max(np.abs(mo - full_o[:, 0]).max(), np.abs(ml - full_l[0]).max())


def pin_reassembly(seed=5, P_list=(1, 2, 4, 8)):
    """Invariant 1: the union of all ranks' rows is the unsplit output."""
    rng = np.random.default_rng(seed)
    n_img = np.array([3, 0, 5])
    cu = np.array([0, 20, 37, 70])
    T = 70
    q, k, v = rand_qkv(rng, T, 2, 1, 8)
    full_o, full_l = oracle.causal_attention(q, k, v, cu)
    err = 0.0
    for P in P_list:
        seen = np.zeros(T, int)
        for r in range(P):
            idx, _ = oracle.partition_index(T, n_img, cu, P, r)
            o, l = oracle.rank_attention(q, k, v, n_img, cu, P, r)
            real = idx >= 0
            err = max(err, np.abs(o[real] - full_o[idx[real]]).max())
            err = max(err, np.abs(l[:, real] - full_l[:, idx[real]]).max())
            if (~real).any():
                err = max(err, np.abs(o[~real]).max())
                err = max(err, float(np.any(np.isfinite(l[:, ~real]))))
            seen[idx[real]] += 1
        # text tokens exactly once, image tokens once per rank
        img_tok = np.concatenate([np.arange(cu[s], cu[s] + n_img[s]) for s in range(3)])
        want = np.ones(T, int)
        want[img_tok] = P
        err = max(err, float(np.any(seen != want)))
    return err


def pin_image_rows_identical(seed=6, P=4):
    """Invariant 3: every rank outputs the same image-prefix rows, bit-exact."""
    rng = np.random.default_rng(seed)
    n_img, cu, T = np.array([6]), np.array([0, 30]), 30
    q, k, v = rand_qkv(rng, T, 2, 2, 4)
    first = None
    bad = 0
    for r in range(P):
        o, l = oracle.rank_attention(q, k, v, n_img, cu, P, r)
        img = (o[:6], l[:, :6])
        if first is None:
            first = img
        else:
            bad += int(not (np.array_equal(img[0], first[0]) and np.array_equal(img[1], first[1])))
    return bad


def brute_pairs(L, n_img, P, r):
    """Count unmasked pairs from an explicit mask matrix over the padded sample."""
    T = L - n_img
    c = -(-T // (2 * P))
    Lp = n_img + 2 * P * c
    mask = np.tril(np.ones((Lp, Lp), dtype=np.int64))
    rows = list(range(n_img)) + [n_img + t for k in (r, 2 * P - 1 - r) for t in range(k * c, (k + 1) * c)]
    padded = int(mask[rows].sum())
    real_rows = [x for x in rows if x < L]
    real = int(mask[real_rows][:, :L].sum())
    return padded, real


def pin_pair_counts():
    bad = 0
    for P in range(1, 5):
        for n in range(0, 4):
            for T in range(0, 3 * 2 * P + 2):
                if n + T == 0:
                    continue
                for r in range(P):
                    got = oracle.pair_counts(n + T, [n], None, P, r)
                    bad += int(got != brute_pairs(n + T, n, P, r))
                    c = -(-T // (2 * P))
                    closed = 2 * P * c * c + c + n * (n + 1) // 2 + 2 * c * n
                    bad += int(got[0] != closed)
    return bad


def pin_backward_finite_differences(seed=7, n_checks=24, eps=1e-6):
    """Analytic rank-share gradients against central differences of the
    forward oracle's loss sum(out_rank * dout), image prefix and packing."""
    rng = np.random.default_rng(seed)
    n_img, cu = np.array([3, 0]), np.array([0, 9, 16])
    T, H, Hkv, D, P = 16, 4, 2, 4, 2
    q, k, v = rand_qkv(rng, T, H, Hkv, D)
    err = 0.0
    for r in range(P):
        idx, _ = oracle.partition_index(T, n_img, cu, P, r)
        dout = rng.standard_normal((len(idx), H, D))
        dq, dk, dv = oracle.rank_attention_backward(q, k, v, dout, n_img, cu, P, r)

        def loss(qq, kk, vv):
            o, _ = oracle.rank_attention(qq, kk, vv, n_img, cu, P, r)
            return float(np.sum(o * dout))
        for which, arr in (("q", q), ("k", k), ("v", v)):
            for _ in range(n_checks):
                i = tuple(int(rng.integers(0, n)) for n in arr.shape)
                hi, lo = arr.copy(), arr.copy()
                hi[i] += eps
                lo[i] -= eps
                args_hi = {"q": (hi, k, v), "k": (q, hi, v), "v": (q, k, hi)}[which]
                args_lo = {"q": (lo, k, v), "k": (q, lo, v), "v": (q, k, lo)}[which]
                fd = (loss(*args_hi) - loss(*args_lo)) / (2 * eps)
                if which == "q":
                    loc = np.nonzero(idx == i[0])[0]
                    an = dq[loc[0], i[1], i[2]] if len(loc) else 0.0
                else:
                    an = (dk if which == "k" else dv)[i]
                err = max(err, abs(fd - an))
    return err


def pin_backward_torch(seed=8, T=40, H=4, Hkv=2, D=8, P=2):
    """Against torch fp64 autograd of scaled_dot_product_attention with an
    explicit causal mask, on the rank's rows (a library routine)."""
    rng = np.random.default_rng(seed)
    n_img = np.array([5])
    q, k, v = rand_qkv(rng, T, H, Hkv, D)
    err = 0.0
    for r in range(P):
        idx, _ = oracle.partition_index(T, n_img, None, P, r)
        real = idx >= 0
        dout = rng.standard_normal((len(idx), H, D))
        dq, dk, dv = oracle.rank_attention_backward(q, k, v, dout, n_img, None, P, r)
        tq = torch.from_numpy(q).requires_grad_()
        tk = torch.from_numpy(k).requires_grad_()
        tv = torch.from_numpy(v).requires_grad_()
        mask = torch.tril(torch.ones(T, T, dtype=torch.bool))
        o = torch.nn.functional.scaled_dot_product_attention(
            tq.permute(1, 0, 2)[None], tk.permute(1, 0, 2)[None], tv.permute(1, 0, 2)[None],
            attn_mask=mask, enable_gqa=True)[0].permute(1, 0, 2)
        rows = torch.from_numpy(idx[real].astype(np.int64))
        (o[rows] * torch.from_numpy(dout[real])).sum().backward()
        err = max(err, np.abs(tq.grad.numpy()[idx[real]] - dq[real]).max(),
                  np.abs(tk.grad.numpy() - dk).max(), np.abs(tv.grad.numpy() - dv).max())
        assert np.all(dq[~real] == 0)
    return err


def pin_backward_reassembly(seed=9, P_list=(2, 4)):
    """Summing dk, dv over the ranks and scattering dq back by each rank's
    index gives the unsplit sequence's gradients (cp_size 1)."""
    rng = np.random.default_rng(seed)
    n_img, cu = np.array([4, 6]), np.array([0, 30, 57])
    T, H, Hkv, D = 57, 2, 1, 8
    q, k, v = rand_qkv(rng, T, H, Hkv, D)
    dout_full = rng.standard_normal((T, H, D))
    idx1, _ = oracle.partition_index(T, n_img, cu, 1, 0)
    dq1, dk1, dv1 = oracle.rank_attention_backward(q, k, v, np.where((idx1 >= 0)[:, None, None],
                                                                     dout_full[np.maximum(idx1, 0)], 0.0),
                                                   n_img, cu, 1, 0)
    full_dq = np.zeros((T, H, D))
    full_dq[idx1[idx1 >= 0]] = dq1[idx1 >= 0]
    err = 0.0
    for P in P_list:
        dq_sum, dk_sum, dv_sum = np.zeros((T, H, D)), np.zeros((T, Hkv, D)), np.zeros((T, Hkv, D))
        image_rows = [np.arange(int(cu[s]), int(cu[s]) + int(n_img[s])) for s in range(len(n_img))]
        image_ids = np.concatenate(image_rows)
        for r in range(P):
            idx, _ = oracle.partition_index(T, n_img, cu, P, r)
            real = idx >= 0
            # every rank outputs the image rows; the loss takes each token's
            # gradient once, so image rows carry dout on one rank only
            dout = np.zeros((len(idx), H, D))
            keep = real & (~np.isin(idx, image_ids) | (r == 0))
            dout[keep] = dout_full[idx[keep]]
            dq, dk, dv = oracle.rank_attention_backward(q, k, v, dout, n_img, cu, P, r)
            dq_sum[idx[real]] += dq[real]
            dk_sum += dk
            dv_sum += dv
        err = max(err, np.abs(dq_sum - full_dq).max(), np.abs(dk_sum - dk1).max(),
                  np.abs(dv_sum - dv1).max())
    return err


# ---------------------------------------------------------------- tests of the true oracle


def test_page_example():
    assert pin_page_example() == 0


def test_page_index_formula():
    # section 1.1: rank r selects chunks [r, 2P - r - 1]
    for P in (1, 2, 3, 4, 8):
        c = 3
        for r in range(P):
            idx, cu_rows = oracle.partition_index(2 * P * c, None, None, P, r)
            want = np.concatenate([np.arange(r * c, r * c + c),
                                   np.arange((2 * P - r - 1) * c, (2 * P - r) * c)])
            assert np.array_equal(idx, want)
            assert list(cu_rows) == [0, 2 * c]


def test_workload1_rank0_rows():
    w = workloads.get(1)
    idx, _ = oracle.partition_index(w.seq_len, None, None, w.cp_size, 0)
    assert np.array_equal(idx, np.concatenate([np.arange(0, 64), np.arange(192, 256)]))


def test_partition_permutation_and_image_on_every_rank():
    rng = np.random.default_rng(7)
    for trial in range(40):
        n = int(rng.integers(1, 5))
        n_img, cu = workloads.random_meta(rng, n, 7, 30)
        T = int(cu[-1])
        P = int(rng.integers(1, 6))
        count = np.zeros(T, int)
        for r in range(P):
            idx, cu_rows = oracle.partition_index(T, n_img, cu, P, r)
            count[idx[idx >= 0]] += 1
            assert cu_rows[-1] == len(idx)
            for s in range(n):
                local = idx[cu_rows[s]:cu_rows[s + 1]]
                assert np.array_equal(local[:n_img[s]], np.arange(cu[s], cu[s] + n_img[s]))
                c = -(-(cu[s + 1] - cu[s] - n_img[s]) // (2 * P))
                assert len(local) == n_img[s] + 2 * c
        for s in range(n):
            assert np.all(count[cu[s]:cu[s] + n_img[s]] == P)
            assert np.all(count[cu[s] + n_img[s]:cu[s + 1]] == 1)


def test_pads_only_at_text_end():
    idx, _ = oracle.partition_index(11, [2], None, 2, 0)  # text 9 -> c=3, 12 slots, 3 pads
    assert list(idx) == [0, 1, 2, 3, 4, -1, -1, -1]
    idx1, _ = oracle.partition_index(11, [2], None, 2, 1)
    assert list(idx1) == [0, 1, 5, 6, 7, 8, 9, 10]


def owner_partition(seq_len, n_img, cu, P, r):
    """The rank's rows by a second formulation that does not reshape or
    select: text offset t of a sample (pads included, t < 2P*c) lies in
    chunk k = t // c, and head-tail pairing gives chunk k to rank
    min(k, 2P - 1 - k). Rank r keeps the offsets it owns in increasing
    order (its chunk r comes before its chunk 2P-1-r), after the image."""
    ids = []
    for s in range(len(cu) - 1):
        a, b, n = int(cu[s]), int(cu[s + 1]), int(n_img[s])
        T = b - a - n
        c = -(-T // (2 * P))
        ids += list(range(a, a + n))
        for t in range(2 * P * c):
            k = t // c
            if min(k, 2 * P - 1 - k) == r:
                ids.append(a + n + t if t < T else -1)
    return np.array(ids, dtype=np.int64)


def test_partition_equals_owner_formulation():
    # context-parallel multimodal page, section 1.1 (head-tail pairing) and
    # 5.3 (per sample): the reshape-and-select partition equals the owner rule
    rng = np.random.default_rng(17)
    for trial in range(150):
        n = int(rng.integers(1, 5))
        n_img, cu = workloads.random_meta(rng, n, 9, 60)
        T = int(cu[-1])
        P = int(rng.integers(1, 7))
        for r in range(P):
            idx, _ = oracle.partition_index(T, n_img, cu, P, r)
            assert np.array_equal(idx, owner_partition(T, n_img, cu, P, r)), (trial, P, r)
    for w in workloads.WORKLOADS.values():
        idx, _ = oracle.partition_index(w.seq_len, w.n_img_array, w.cu_seqlens, w.cp_size, w.rank)
        assert np.array_equal(idx, owner_partition(w.seq_len, w.n_img_array, w.cu_seqlens, w.cp_size, w.rank))


def test_real_pairs_are_padded_minus_pad_rows():
    # pad rows count n_img + t + 1 pairs in the padded total (t its text
    # offset) and none in the real one; offsets come from the owner rule
    rng = np.random.default_rng(19)
    for trial in range(150):
        n = int(rng.integers(1, 5))
        n_img, cu = workloads.random_meta(rng, n, 9, 60)
        T = int(cu[-1])
        P = int(rng.integers(1, 7))
        for r in range(P):
            padded, real = oracle.pair_counts(T, n_img, cu, P, r)
            pad_terms = 0
            for s in range(n):
                a, b, ni = int(cu[s]), int(cu[s + 1]), int(n_img[s])
                Ts = b - a - ni
                c = -(-Ts // (2 * P))
                for t in range(Ts, 2 * P * c):  # the pads sit at the end of the text
                    k = t // c
                    if min(k, 2 * P - 1 - k) == r:
                        pad_terms += ni + t + 1
            assert real == padded - pad_terms, (trial, P, r)


# Per-head pair counts of the five synthetic workloads, written out as
# integers from the per-sample closed form (image rows n(n+1)/2, text rows
# against the image 2cn, text rows 2Pc^2 + c) -- not from the oracle.
#   1: text 256, P=2, c=64:                 2*2*64^2 + 64            = 16,448
#   2: text 8192, P=4, c=1024:              2*4*1024^2 + 1024        = 8,389,632
#   3: image 2304 + text 16384, P=4, c=2048:
#      2304*2305/2 + 2*2048*2304 + 2*4*2048^2 + 2048                 = 45,649,024
#   4: text 65536, P=8, c=4096:             2*8*4096^2 + 4096        = 268,439,552
#   5: 8 samples (seed 1005), P=4: the sum of the closed form over samples
#      = 60,919,305 padded on every rank; rank 0 holds every pad row, so
#      its real count is lower: 60,648,617.
PAIR_LITERALS = {1: 16_448, 2: 8_389_632, 3: 45_649_024, 4: 268_439_552, 5: 60_919_305}
ROW_LITERALS = {1: 128, 2: 2_048, 3: 6_400, 4: 8_192, 5: 23_094}


def test_pair_count_literals():
    for num, want in PAIR_LITERALS.items():
        w = workloads.get(num)
        for r in range(w.cp_size):
            padded, real = oracle.pair_counts(w.seq_len, w.n_img_array, w.cu_seqlens, w.cp_size, r)
            assert padded == want, (num, r)
            if num != 5 or r != 0:
                assert real == padded, (num, r)
            idx, _ = oracle.partition_index(w.seq_len, w.n_img_array, w.cu_seqlens, w.cp_size, r)
            assert len(idx) == ROW_LITERALS[num], (num, r)
    w = workloads.get(5)
    assert oracle.pair_counts(w.seq_len, w.n_img_array, w.cu_seqlens, w.cp_size, 0)[1] == 60_648_617
    # the workload-5 lengths these literals were worked out for
    assert list(w.n_img) == [1320, 2232, 1445, 1306, 2055, 773, 1169, 1916]
    assert list(w.text_len) == [2553, 7766, 3813, 5971, 7177, 8049, 3044, 5100]
    assert list(w.cu_seqlens) == [0, 3873, 13871, 19129, 26406, 35638, 44460, 48673, 55689]


def test_pair_counts_brute_force_and_closed_form():
    assert pin_pair_counts() == 0


def test_pair_counts_equal_across_ranks():
    # invariant 2, exact integers, on the five workloads (padded counts)
    doc = json.load(open(os.path.join(GOLDEN, "workload_counts.json")))
    for num, w in workloads.WORKLOADS.items():
        vals = set()
        for r in range(w.cp_size):
            got = oracle.pair_counts(w.seq_len, w.n_img_array, w.cu_seqlens, w.cp_size, r)
            g = doc["workloads"][str(num)]["ranks"][str(r)]
            assert got == (g["pairs_padded"], g["pairs_real"])
            vals.add(got[0])
        assert len(vals) == 1


def test_pair_counts_sum_to_full_causal():
    for P in (1, 2, 4, 8):
        L = 2 * P * 5
        tot = sum(oracle.pair_counts(L, None, None, P, r)[1] for r in range(P))
        assert tot == L * (L + 1) // 2


def test_naive_contiguous_split_is_unbalanced():
    # section 1.1: a plain P-way split loads the tail rank most; for P=4 at
    # L=8192 the per-rank pairs grow as 1:3:5:7
    L, P = 8192, 4
    per = L // P
    counts = [sum(p + 1 for p in range(r * per, (r + 1) * per)) for r in range(P)]
    assert len(set(counts)) == P
    base = per * per // 2
    assert [round(c / base) for c in counts] == [1, 3, 5, 7]
    balanced = {oracle.pair_counts(L, None, None, P, r)[1] for r in range(P)}
    assert len(balanced) == 1


def test_contiguous_split_is_the_plain_split():
    # section 1.1's plain split: rank r holds the r-th contiguous P-th of the
    # (padded) text, so concatenating ranks 0..P-1 gives the text in order;
    # the image prefix stays whole on every rank
    for T, n, P in ((8192, 0, 4), (1001, 37, 3), (5, 2, 4)):
        c = -(-T // (2 * P))
        text = [t for t in range(n, n + T)] + [-1] * (2 * P * c - T)
        joined = []
        for r in range(P):
            idx, cu_rows = oracle.partition_index(n + T, [n], None, P, r, split="contiguous")
            assert list(idx[:n]) == list(range(n)) and list(cu_rows) == [0, len(idx)]
            joined += list(idx[n:])
            assert list(idx[n:]) == text[2 * r * c:(2 * r + 2) * c]
        assert joined == text


def test_contiguous_split_pair_counts_skew():
    # per-rank causal pairs of the plain split grow as 1:3:5:7 for P=4
    # (section 1.1: later tokens attend to more tokens); brute force
    L, P = 8192, 4
    per = L // P
    for r in range(P):
        brute = sum(p + 1 for p in range(r * per, (r + 1) * per))
        assert oracle.pair_counts(L, None, None, P, r, split="contiguous") == (brute, brute)
    pairs = [oracle.pair_counts(L, None, None, P, r, split="contiguous")[1] for r in range(P)]
    assert [round(x / (per * per // 2)) for x in pairs] == [1, 3, 5, 7]
    # both splits cover every causal pair once over the ranks
    total = L * (L + 1) // 2
    assert sum(pairs) == total
    assert sum(oracle.pair_counts(L, None, None, P, r)[1] for r in range(P)) == total


def test_backward_finite_differences():
    assert pin_backward_finite_differences() < 1e-6


def test_backward_torch_autograd():
    assert pin_backward_torch() < 1e-12


def test_backward_reassembly():
    assert pin_backward_reassembly() < 1e-12


def test_backward_row_subsets_add_up_and_pool():
    # the row terms of the backward are independent: dq rows of a subset are
    # the full share's, and dk, dv of disjoint subsets sum to the full
    # share's -- so the threaded (KV head, row chunk) pool, which places and
    # adds those pieces, reproduces the single call
    from oracle.pool import rank_attention_backward_pooled

    rng = np.random.default_rng(12)
    n_img = np.array([7, 0, 3], np.int32)
    cu = np.array([0, 60, 101, 190], np.int32)
    T, H, Hkv, D, P, r = 190, 4, 2, 8, 3, 1
    q, k, v = rand_qkv(rng, T, H, Hkv, D)
    idx, _ = oracle.partition_index(T, n_img, cu, P, r)
    dout = rng.standard_normal((len(idx), H, D))
    dout[idx < 0] = 0
    fq, fk, fv = oracle.rank_attention_backward(q, k, v, dout, n_img, cu, P, r)
    half = np.arange(0, len(idx), 2)
    rest = np.arange(1, len(idx), 2)
    aq, ak, av = oracle.rank_attention_backward(q, k, v, dout, n_img, cu, P, r, local_rows=half)
    bq, bk, bv = oracle.rank_attention_backward(q, k, v, dout, n_img, cu, P, r, local_rows=rest)
    assert np.array_equal(aq[half], fq[half]) and np.all(aq[rest] == 0)
    assert np.abs(ak + bk - fk).max() < 1e-12 and np.abs(av + bv - fv).max() < 1e-12
    for chunk in (5, 16, 1000):
        pq, pk, pv = rank_attention_backward_pooled(q, k, v, dout, n_img, cu, P, r, row_chunk=chunk,
                                                    workers=3)
        assert np.abs(pq - fq).max() < 1e-12
        assert np.abs(pk - fk).max() < 1e-12 and np.abs(pv - fv).max() < 1e-12


def test_backward_single_key_row():
    # a row that sees one key has P = 1 and dS = 0: its dq is exactly zero
    rng = np.random.default_rng(10)
    q, k, v = rand_qkv(rng, 8, 2, 2, 4)
    idx, _ = oracle.partition_index(8, None, None, 2, 0)
    dout = rng.standard_normal((len(idx), 2, 4))
    dq, _, dv = oracle.rank_attention_backward(q, k, v, dout, None, None, 2, 0)
    assert idx[0] == 0 and np.all(dq[0] == 0.0)


def test_brute_force():
    assert pin_brute_force() < 1e-12


def test_torch_library():
    assert pin_torch() < 1e-12
    assert pin_torch(seed=11, scale=8.0) < 1e-11  # peaky softmax


def test_packed_blockdiag_mask():
    assert pin_packed_blockdiag() < 1e-12


def test_closed_forms():
    assert pin_closed_forms() < 1e-12


def test_merge_identity():
    assert pin_merge_identity() < 1e-12


def test_merge_all_empty_rows():
    o, l = oracle.lse_merge([np.ones((3, 4)), np.ones((3, 4))], [np.full(3, -np.inf)] * 2)
    assert np.all(o == 0) and np.all(np.isneginf(l))


def test_reassembly_invariant():
    assert pin_reassembly() < 1e-12


def test_image_rows_identical_invariant():
    assert pin_image_rows_identical() == 0


def test_packed_equals_per_sample():
    rng = np.random.default_rng(8)
    cu = np.array([0, 9, 25, 26, 41])
    q, k, v = rand_qkv(rng, 41, 2, 1, 8)
    o, l = oracle.causal_attention(q, k, v, cu)
    for s in range(4):
        a, b = cu[s], cu[s + 1]
        o1, l1 = oracle.causal_attention(q[a:b], k[a:b], v[a:b])
        assert np.array_equal(o[a:b], o1) and np.array_equal(l[:, a:b], l1)


def test_rank_rows_equal_literal():
    rng = np.random.default_rng(9)
    n_img, cu = np.array([4, 0]), np.array([0, 29, 51])
    q, k, v = rand_qkv(rng, 51, 2, 2, 8)
    for r in range(3):
        a = oracle.rank_attention(q, k, v, n_img, cu, 3, r)
        b = oracle.rank_attention(q, k, v, n_img, cu, 3, r, literal=True)
        # same definition, different row blocking: equal up to summation order
        assert np.abs(a[0] - b[0]).max() < 1e-13
        assert np.array_equal(np.isneginf(a[1]), np.isneginf(b[1]))
        fin = np.isfinite(a[1])
        assert np.abs(a[1][fin] - b[1][fin]).max() < 1e-13
        sub = [1, 5, 7]
        c = oracle.rank_attention(q, k, v, n_img, cu, 3, r, local_rows=sub)
        assert np.abs(c[0] - a[0][sub]).max() < 1e-13


def test_all_image_sample_and_tiny_text():
    # a sample that is only image (no text chunks) and text shorter than 2P
    rng = np.random.default_rng(10)
    n_img, cu = np.array([5, 1]), np.array([0, 5, 8])
    q, k, v = rand_qkv(rng, 8, 1, 1, 4)
    full_o, _ = oracle.causal_attention(q, k, v, cu)
    for r in range(4):
        idx, _ = oracle.partition_index(8, n_img, cu, 4, r)
        o, l = oracle.rank_attention(q, k, v, n_img, cu, 4, r)
        real = idx >= 0
        assert np.abs(o[real] - full_o[idx[real]]).max() < 1e-15
        assert np.all(o[~real] == 0) and np.all(np.isneginf(l[:, ~real]))


# ---------------------------------------------------------------- planted mistakes


def test_mutant_exclusive_diagonal_is_caught(monkeypatch):
    monkeypatch.setattr(cp_oracle, "visible", lambda kk, rr: kk[None, :] < rr[:, None])
    assert pin_brute_force() > 1e-3 or np.isnan(pin_brute_force())
    assert not (pin_torch() < 1e-6)


def test_mutant_scale_is_caught(monkeypatch):
    monkeypatch.setattr(cp_oracle, "softmax_scale", lambda d: 1.0 / d)
    assert pin_torch() > 1e-3
    assert pin_brute_force() > 1e-3


def test_mutant_gqa_map_is_caught(monkeypatch):
    monkeypatch.setattr(cp_oracle, "kv_head_of", lambda h, H, Hkv: h % Hkv)
    assert pin_torch() > 1e-3
    assert pin_brute_force() > 1e-3


def test_mutant_dropped_max_shift_in_lse_is_caught(monkeypatch):
    real_attend = cp_oracle.attend

    def bad_attend(q, k, v, allowed, scale):
        o, l = real_attend(q, k, v, allowed, scale)
        s = np.where(allowed, (q @ k.T) * scale, -np.inf)
        return o, l - np.max(s, axis=1)  # forgets to add the max back
    monkeypatch.setattr(cp_oracle, "attend", bad_attend)
    assert pin_torch() > 1e-3


def test_mutant_chunk_order_is_caught(monkeypatch):
    real = cp_oracle.partition_index

    def swapped(seq_len, n_img, cu, P, r):
        idx, cu_rows = real(seq_len, n_img, cu, P, r)
        if cu is None and (n_img is None or np.all(np.asarray(n_img) == 0)) and len(idx) > 1:
            h = len(idx) // 2
            idx = np.concatenate([idx[h:], idx[:h]])
        return idx, cu_rows
    monkeypatch.setattr(oracle, "partition_index", swapped)
    assert pin_page_example() > 0


def test_mutant_split_image_breaks_invariant3(monkeypatch):
    # section 3.1's failure mode: cutting the image together with the text
    real = cp_oracle.partition_index

    def naive(seq_len, n_img, cu, P, r, split="head_tail"):
        return real(seq_len, None, cu, P, r, split)
    monkeypatch.setattr(cp_oracle, "partition_index", naive)
    assert pin_image_rows_identical() > 0 or pin_reassembly() > 0


def test_mutant_pair_count_off_by_one_is_caught(monkeypatch):
    real = cp_oracle.pair_counts

    def bad(*a):
        p, r = real(*a)
        return p - 1, r
    monkeypatch.setattr(oracle, "pair_counts", bad)
    assert pin_pair_counts() > 0


def test_mutant_merge_weights_are_caught(monkeypatch):
    real = cp_oracle.lse_merge

    def bad(outs, lses):
        o, l = real(outs, lses)
        return np.mean(np.stack(outs), axis=0), l  # plain average of partials
    monkeypatch.setattr(oracle, "lse_merge", bad)
    assert pin_merge_identity() > 1e-3


def test_mutant_backward_dropped_delta_is_caught(monkeypatch):
    real = cp_oracle.attend_backward

    def bad(q, k, v, allowed, scale, dout):
        q64, k64, v64, d64 = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
        s_ = np.where(allowed, (q64 @ k64.T) * scale, -np.inf)
        m = np.max(s_, axis=1, initial=-np.inf)
        e = np.where(allowed, np.exp(s_ - np.where(np.isfinite(m), m, 0.0)[:, None]), 0.0)
        p = e / np.maximum(e.sum(axis=1, keepdims=True), 1e-300)
        ds = p * (d64 @ v64.T)  # the row term sum_j P_j dP_j dropped
        return (ds @ k64) * scale, (ds.T @ q64) * scale, p.T @ d64
    monkeypatch.setattr(cp_oracle, "attend_backward", bad)
    assert real is not bad
    assert pin_backward_finite_differences(n_checks=8) > 1e-3


def test_mutant_backward_scale_is_caught(monkeypatch):
    real = cp_oracle.attend_backward

    def bad(q, k, v, allowed, scale, dout):
        gq, gk, gv = real(q, k, v, allowed, scale, dout)
        return gq / scale, gk, gv
    monkeypatch.setattr(cp_oracle, "attend_backward", bad)
    assert pin_backward_finite_differences(n_checks=8) > 1e-3



def test_backward_sampling_helpers_match_full_oracle():
    # the full-size GPU backward test checks sampled dq rows and the last
    # keys of each sample with oracle pieces (attend_backward over a subset of
    # rows); on a small packed case those pieces equal the full oracle
    import importlib.util
    import os

    import torch

    path = os.path.join(os.path.dirname(__file__), "test_gpu_backward.py")
    spec = importlib.util.spec_from_file_location("gpu_backward_helpers", path)
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    T, H, Hkv, D, P, r = 700, 4, 2, 128, 3, 1
    cu = np.array([0, 300, 700], np.int32)
    img = np.array([10, 0], np.int32)
    idx, _ = oracle.partition_index(T, img, cu, P, r)
    q, k, v, dout = m.draw(5, T, H, Hkv, D, len(idx))
    dout[torch.from_numpy(idx < 0)] = 0
    fq, fk, fv = oracle.rank_attention_backward(q, k, v, dout, img, cu, P, r)
    rows = np.nonzero(idx >= 0)[0][::17]
    ref = m._exact_dq_rows(q, k, v, dout, idx, cu.astype(np.int64), rows, H, Hkv)
    assert np.abs(ref - fq[rows]).max() <= 1e-12
    for s in range(2):
        j0, rk, rv = m._exact_last_keys(q, k, v, dout, idx, cu.astype(np.int64), s, 24, H, Hkv)
        assert len(rk) == 24
        assert np.abs(rk - fk[j0:j0 + 24]).max() <= 1e-12
        assert np.abs(rv - fv[j0:j0 + 24]).max() <= 1e-12
    # sum over keys of dv = sum over rows of dout, per KV head
    do64 = dout.double().numpy().reshape(len(idx), Hkv, H // Hkv, D)
    assert np.abs(fv.sum(axis=0) - do64.sum(axis=(0, 2))).max() <= 1e-9
