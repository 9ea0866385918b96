"""fp64 CPU oracle: partition, pair counts and per-rank causal attention.

TEST INFRASTRUCTURE (see the package docstring): plain, slow, obviously
correct, and independent of the HIP library.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "chunk_len",
    "owned_chunks",
    "partition_index",
    "pair_counts",
    "attend",
    "softmax_scale",
    "kv_head_of",
    "visible",
    "causal_attention",
    "rank_attention",
    "attend_backward",
    "rank_attention_backward",
    "lse_merge",
]


def _as_meta(seq_len: int, n_img, cu_seqlens):
    """Normalise (n_img, cu_seqlens): None means one sample / no image."""
    if cu_seqlens is None:
        cu = np.array([0, int(seq_len)], dtype=np.int64)
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
    n = len(cu) - 1
    if n_img is None:
        img = np.zeros(n, dtype=np.int64)
    else:
        img = np.asarray(n_img, dtype=np.int64).reshape(n)
    assert cu[0] == 0 and cu[-1] == seq_len and np.all(np.diff(cu) > 0)
    assert np.all(img >= 0) and np.all(img <= np.diff(cu))
    return img, cu


def chunk_len(text_len: int, cp_size: int) -> int:
    """Tokens per chunk when a sample's text is cut into 2P chunks.

    Context-parallel multimodal page, §1.1: the sequence is cut into 2P
    chunks. Reading for lengths that 2P does not divide: round the chunk
    up and pad the text at its end.
    """
    return -(-int(text_len) // (2 * int(cp_size)))


def owned_chunks(cp_size: int, cp_rank: int, split: str = "head_tail") -> np.ndarray:
    """The two of the 2P text chunks a rank holds, in its local order.

    Context-parallel multimodal page, §1.1: head-tail pairing gives rank r
    chunks [r, 2P - r - 1]. The page contrasts it with the plain split into
    P contiguous pieces, which loads the later ranks more under a causal
    mask; on the same 2P chunks that split gives rank r chunks [2r, 2r + 1]
    ("contiguous").
    """
    P, r = int(cp_size), int(cp_rank)
    if split == "head_tail":
        return np.array([r, 2 * P - r - 1])
    if split == "contiguous":
        return np.array([2 * r, 2 * r + 1])
    raise ValueError(f"unknown split {split!r}")


def partition_index(seq_len: int, n_img, cu_seqlens, cp_size: int, cp_rank: int,
                    split: str = "head_tail") -> Tuple[np.ndarray, np.ndarray]:
    """Global token ids of the rows rank ``cp_rank`` holds, -1 for pads.

    Follows the page's steps literally, per sample:

    * §4.1: the image prefix is kept whole (every rank gets all of it) and
      only the text is split;
    * §1.1: the (padded) text is viewed as 2P chunks and rows
      [cp_rank, 2*cp_size - cp_rank - 1] are index-selected, in that order
      (``split="contiguous"``: rows [2*cp_rank, 2*cp_rank + 1], see
      ``owned_chunks``);
    * §5.3: with packed samples the split is done per sample, using the
      cu_seqlens boundaries; samples keep their order.

    Returns (index int32[R], cu_rows int32[n_samples + 1]), where cu_rows
    are the sample boundaries in the rank-local row order.
    """
    img, cu = _as_meta(seq_len, n_img, cu_seqlens)
    P, r = int(cp_size), int(cp_rank)
    assert P >= 1 and 0 <= r < P
    pieces = []
    cu_rows = [0]
    for s in range(len(cu) - 1):
        a, b, n = int(cu[s]), int(cu[s + 1]), int(img[s])
        image_ids = np.arange(a, a + n, dtype=np.int64)
        text_ids = np.arange(a + n, b, dtype=np.int64)
        c = chunk_len(len(text_ids), P)
        padded = np.full(2 * P * c, -1, dtype=np.int64)
        padded[: len(text_ids)] = text_ids
        chunks = padded.reshape(2 * P, c)
        select = owned_chunks(P, r, split)
        mine = chunks[select].reshape(-1)
        local = np.concatenate([image_ids, mine])
        pieces.append(local)
        cu_rows.append(cu_rows[-1] + len(local))
    index = np.concatenate(pieces) if pieces else np.zeros(0, dtype=np.int64)
    return index.astype(np.int32), np.asarray(cu_rows, dtype=np.int32)


def pair_counts(seq_len: int, n_img, cu_seqlens, cp_size: int, cp_rank: int,
                split: str = "head_tail") -> Tuple[int, int]:
    """Unmasked (query, key) pairs per head on one rank: (padded, real).

    With the causal mask a query at position p inside its sample sees keys
    at positions 0..p of that sample, so it contributes p + 1 pairs
    (§1.1: later tokens attend to more tokens). ``real`` sums this over the
    rank's real rows. ``padded`` also counts each pad row as if it were a
    token at its padded text offset t, i.e. n_img + t + 1 pairs; this is
    the quantity the head-tail pairing equalises exactly.
    """
    img, cu = _as_meta(seq_len, n_img, cu_seqlens)
    P, r = int(cp_size), int(cp_rank)
    padded_total = 0
    real_total = 0
    for s in range(len(cu) - 1):
        a, b, n = int(cu[s]), int(cu[s + 1]), int(img[s])
        T = b - a - n
        c = chunk_len(T, P)
        # positions inside the sample of every row this rank holds,
        # pads included at their padded offsets
        offsets = np.arange(2 * P * c).reshape(2 * P, c)[owned_chunks(P, r, split)].reshape(-1)
        positions = np.concatenate([np.arange(n), n + offsets])
        is_real = np.concatenate([np.ones(n, bool), offsets < T])
        padded_total += int(np.sum(positions + 1))
        real_total += int(np.sum((positions + 1)[is_real]))
    return padded_total, real_total


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, allowed: np.ndarray,
           scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of query rows over the keys each row may see.

    q [n, D], k [m, D], v [m, D], allowed bool [n, m]. Two exact passes per
    row: the max over allowed scores, then sum of exp(score - max). Returns
    out [n, D] = sum_j softmax_j * v_j and lse [n] = max + ln(sum). A row
    with no allowed key gets out 0 and lse -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = (q @ k.T) * scale
    s = np.where(allowed, s, -np.inf)
    m = np.max(s, axis=1, initial=-np.inf)
    any_key = np.isfinite(m)
    m_safe = np.where(any_key, m, 0.0)
    e = np.where(allowed, np.exp(s - m_safe[:, None]), 0.0)
    l = e.sum(axis=1)
    out = np.zeros((q.shape[0], v.shape[1]), dtype=np.float64)
    out[any_key] = (e[any_key] @ v) / l[any_key, None]
    lse = np.full(q.shape[0], -np.inf)
    lse[any_key] = m[any_key] + np.log(l[any_key])
    return out, lse


def softmax_scale(head_dim: int) -> float:
    """Score scale 1/sqrt(head_dim) (reading: the pages give none)."""
    return 1.0 / math.sqrt(head_dim)


def kv_head_of(h: int, heads: int, kv_heads: int) -> int:
    """KV head read by query head h: consecutive query heads share one."""
    return h // (heads // kv_heads)


def visible(key_ids: np.ndarray, row_ids: np.ndarray) -> np.ndarray:
    """Causal visibility with an inclusive diagonal: key j is seen by row i
    iff j <= i (both global ids inside one sample). bool [rows, keys]."""
    return key_ids[None, :] <= row_ids[:, None]


def _to64(x) -> np.ndarray:
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def causal_attention(q, k, v, cu_seqlens=None, rows: Optional[Sequence[int]] = None,
                     block: int = 1024) -> Tuple[np.ndarray, np.ndarray]:
    """Full-sequence causal softmax attention in fp64.

    q [T, H, D], k and v [T, Hkv, D]. Query at global token i of sample
    [a, b) sees keys a..i (inclusive diagonal); samples never see each
    other. Scale 1/sqrt(D); query head h reads KV head h // (H // Hkv).
    ``rows`` restricts the computation to those global token ids (each
    row's result depends on nothing else). Returns out [n, H, D] and
    lse [H, n] for the requested rows (all T rows if ``rows`` is None).
    """
    q, k, v = _to64(q), _to64(k), _to64(v)
    T, H, D = q.shape
    Hkv = k.shape[1]
    assert H % Hkv == 0
    scale = softmax_scale(D)
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int64)
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), H, D))
    lse = np.full((H, len(rows)), -np.inf)
    sample_of = np.searchsorted(cu, rows, side="right") - 1
    for s in np.unique(sample_of):
        a = int(cu[s])
        sel = np.nonzero(sample_of == s)[0]
        for i0 in range(0, len(sel), block):
            part = sel[i0:i0 + block]
            g_rows = rows[part]
            hi = int(g_rows.max()) + 1
            keys = np.arange(a, hi)
            allowed = visible(keys, g_rows)
            for h in range(H):
                kh = kv_head_of(h, H, Hkv)
                o, l_ = attend(q[g_rows, h], k[a:hi, kh], v[a:hi, kh], allowed, scale)
                out[part, h] = o
                lse[h, part] = l_
    return out, lse


def rank_attention(q, k, v, n_img, cu_seqlens, cp_size: int, cp_rank: int,
                   local_rows: Optional[Sequence[int]] = None, literal: bool = False,
                   split: str = "head_tail") -> Tuple[np.ndarray, np.ndarray]:
    """The rows of full-sequence causal attention that one CP rank holds.

    out [R, H, D], lse [H, R] in the rank-local row order of
    ``partition_index``; pad rows are 0 / -inf. With ``literal`` the whole
    sequence is computed first and then index-selected, as the method's
    definition reads; otherwise only the rank's rows (or ``local_rows``, a
    subset of local row numbers) are computed, which gives the same values
    because each row depends only on its own visible keys.
    """
    T, H, D = (int(x) for x in q.shape)
    index, _ = partition_index(T, n_img, cu_seqlens, cp_size, cp_rank, split)
    if local_rows is None:
        local_rows = np.arange(len(index))
    local_rows = np.asarray(local_rows, dtype=np.int64)
    ids = index[local_rows].astype(np.int64)
    real = ids >= 0
    out = np.zeros((len(local_rows), H, D))
    lse = np.full((H, len(local_rows)), -np.inf)
    if real.any():
        if literal:
            full_o, full_l = causal_attention(q, k, v, cu_seqlens)
            out[real] = full_o[ids[real]]
            lse[:, real] = full_l[:, ids[real]]
        else:
            o, l_ = causal_attention(q, k, v, cu_seqlens, rows=ids[real])
            out[real] = o
            lse[:, real] = l_
    return out, lse


def attend_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, allowed: np.ndarray, scale: float,
                    dout: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients of softmax attention (``attend``) for one head.

    With S = q k^T * scale over the allowed keys, P = softmax(S) per row and
    out = P v, a loss with gradient dout w.r.t. out has (chain rule through
    the softmax, written out):
      dV = P^T dout;  dP = dout v^T;  dS = P * (dP - sum_j P_j dP_j);
      dq = dS k * scale;  dk = dS^T q * scale.
    Rows with no allowed key contribute nothing. Returns (dq, dk, dv).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    s = np.where(allowed, (q @ k.T) * scale, -np.inf)
    m = np.max(s, axis=1, initial=-np.inf)
    any_key = np.isfinite(m)
    e = np.where(allowed, np.exp(s - np.where(any_key, m, 0.0)[:, None]), 0.0)
    l = e.sum(axis=1)
    p = np.zeros_like(e)
    p[any_key] = e[any_key] / l[any_key, None]
    dv = p.T @ dout
    dp = dout @ v.T
    ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
    return (ds @ k) * scale, (ds.T @ q) * scale, dv


def rank_attention_backward(q, k, v, dout, n_img, cu_seqlens, cp_size: int, cp_rank: int,
                            split: str = "head_tail", local_rows: Optional[Sequence[int]] = None
                            ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients of one CP rank's share of causal attention.

    The share is the rank's rows of full-sequence causal attention
    (``rank_attention``); ``dout`` [R, H, D] is a loss gradient w.r.t. those
    rows, in the rank-local order. Returns dq [R, H, D] (pad rows 0), and
    dk, dv [T, Hkv, D]: every key's gradient summed over the rank's rows
    and over the query heads that read its KV head. Summing dk, dv over all
    ranks (and scattering every rank's dq back by its index) gives the
    gradients of the whole sequence -- the reduction the reverse ring or an
    all-reduce performs across GPUs.

    With ``local_rows`` (a subset of local row numbers) only those rows'
    terms are taken: their dq rows (the others stay 0), and dk, dv summed
    over them alone. A row's dq and its terms of dk and dv depend on that
    row only (its P, dP and Delta), so the results of disjoint subsets add
    up to the whole share's.
    """
    q, k, v, dout = _to64(q), _to64(k), _to64(v), _to64(dout)
    T, H, D = q.shape
    Hkv = k.shape[1]
    scale = softmax_scale(D)
    index, _ = partition_index(T, n_img, cu_seqlens, cp_size, cp_rank, split)
    cu = np.array([0, T], dtype=np.int64) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    dq = np.zeros((len(index), H, D))
    dk = np.zeros((T, Hkv, D))
    dv = np.zeros((T, Hkv, D))
    ids = index.astype(np.int64)
    sample_of = np.searchsorted(cu, np.maximum(ids, 0), side="right") - 1
    taken = np.ones(len(ids), dtype=bool)
    if local_rows is not None:
        taken[:] = False
        taken[np.asarray(local_rows, dtype=np.int64)] = True
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        sel = np.nonzero((ids >= 0) & (sample_of == s) & taken)[0]
        if len(sel) == 0:
            continue
        rows = ids[sel]
        keys = np.arange(a, b)
        allowed = visible(keys, rows)
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            gq, gk, gv = attend_backward(q[rows, h], k[a:b, g], v[a:b, g], allowed, scale, dout[sel, h])
            dq[sel, h] = gq
            dk[a:b, g] += gk
            dv[a:b, g] += gv
    return dq, dk, dv


def lse_merge(outs: Sequence[np.ndarray], lses: Sequence[np.ndarray]
              ) -> Tuple[np.ndarray, np.ndarray]:
    """Combine partial attention results over disjoint key blocks.

    Each partial b has out_b (softmax over block b's keys applied to V) and
    lse_b. With m = max_b lse_b and w_b = exp(lse_b - m): the combined
    lse = m + ln(sum_b w_b) and out = sum_b w_b out_b / sum_b w_b, which is
    the softmax over the union of the blocks (Ring Attention's blockwise
    combination). Rows where every lse_b is -inf get 0 / -inf.

    outs[b] has shape [..., D], lses[b] the matching shape [...].
    """
    L = np.stack([np.asarray(x, dtype=np.float64) for x in lses])
    O = np.stack([np.asarray(x, dtype=np.float64) for x in outs])
    m = np.max(L, axis=0)
    ok = np.isfinite(m)
    m_safe = np.where(ok, m, 0.0)
    w = np.where(np.isfinite(L), np.exp(L - m_safe[None]), 0.0)
    wsum = w.sum(axis=0)
    out = np.zeros(O.shape[1:])
    num = np.sum(w[..., None] * np.where(np.isfinite(L)[..., None], O, 0.0), axis=0)
    out[ok] = num[ok] / wsum[ok][..., None]
    lse = np.full(m.shape, -np.inf)
    lse[ok] = m[ok] + np.log(wsum[ok])
    return out, lse
