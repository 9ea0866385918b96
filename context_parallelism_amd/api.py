"""Tensor-level helpers over the C ABI.

torch supplies device memory and the current stream; every step of the
computation runs in the HIP library. Inputs must already be GPU tensors:
there is no CPU path.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple

import numpy as np

from . import _lib
from ._lib import (CP_DTYPE_BF16, CP_DTYPE_F32, CP_SCHED_AUTO, CP_SCHED_PER_STEP, CP_SCHED_ROW_TILE,
                   CP_SPLIT_CONTIGUOUS, CP_SPLIT_HEAD_TAIL, check)

_I32P = ctypes.POINTER(ctypes.c_int32)
SPLITS = {"head_tail": CP_SPLIT_HEAD_TAIL, "contiguous": CP_SPLIT_CONTIGUOUS}
SCHEDULES = {"auto": CP_SCHED_AUTO, "row_tile": CP_SCHED_ROW_TILE, "per_step": CP_SCHED_PER_STEP}


def _split_code(split) -> int:
    if split not in SPLITS:
        raise ValueError(f"split must be one of {sorted(SPLITS)}, not {split!r}")
    return SPLITS[split]


def _schedule_code(schedule) -> int:
    if schedule not in SCHEDULES:
        raise ValueError(f"schedule must be one of {sorted(SCHEDULES)}, not {schedule!r}")
    return SCHEDULES[schedule]


def _meta(n_img, cu_seqlens):
    """Host int32 arrays (kept alive by the caller) and their pointers."""
    cu = None if cu_seqlens is None else np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    img = None if n_img is None else np.ascontiguousarray(np.asarray(n_img, dtype=np.int32)).reshape(-1)
    n_samples = 1 if cu is None else len(cu) - 1
    cu_p = None if cu is None else cu.ctypes.data_as(_I32P)
    img_p = None if img is None else img.ctypes.data_as(_I32P)
    return (cu, img), cu_p, img_p, n_samples


def partition_index(seq_len: int, n_img=None, cu_seqlens=None, *, cp_size: int, cp_rank: int,
                    split: str = "head_tail") -> Tuple[np.ndarray, np.ndarray]:
    """(index int32[R], cu_rows int32[n_samples+1]) of one CP rank."""
    keep, cu_p, img_p, n = _meta(n_img, cu_seqlens)
    sp = _split_code(split)
    rows = ctypes.c_int64(0)
    check(_lib.cp_partition_index_ex(seq_len, img_p, cu_p, n, cp_size, cp_rank, sp, None, 0,
                                     ctypes.byref(rows), None), "cp_partition_index_ex")
    index = np.zeros(rows.value, dtype=np.int32)
    cu_rows = np.zeros(n + 1, dtype=np.int32)
    check(_lib.cp_partition_index_ex(seq_len, img_p, cu_p, n, cp_size, cp_rank, sp,
                                     index.ctypes.data_as(_I32P), rows.value, ctypes.byref(rows),
                                     cu_rows.ctypes.data_as(_I32P)), "cp_partition_index_ex")
    return index, cu_rows


def pair_counts(seq_len: int, n_img=None, cu_seqlens=None, *, cp_size: int, cp_rank: int,
                split: str = "head_tail") -> Tuple[int, int]:
    """(padded, real) unmasked pairs per head on one rank."""
    keep, cu_p, img_p, n = _meta(n_img, cu_seqlens)
    padded, real = ctypes.c_int64(0), ctypes.c_int64(0)
    check(_lib.cp_pair_counts_ex(seq_len, img_p, cu_p, n, cp_size, cp_rank, _split_code(split),
                                 ctypes.byref(padded), ctypes.byref(real)), "cp_pair_counts_ex")
    return padded.value, real.value


def workspace_size(seq_len: int, n_img=None, cu_seqlens=None, *, cp_size: int, cp_rank: int,
                   heads: int, kv_heads: int, head_dim: int, dtype: int, split: str = "head_tail",
                   schedule: str = "auto") -> int:
    keep, cu_p, img_p, n = _meta(n_img, cu_seqlens)
    b = ctypes.c_size_t(0)
    check(_lib.cp_attn_rank_workspace_size_ex(seq_len, img_p, cu_p, n, cp_size, cp_rank,
                                              _split_code(split), _schedule_code(schedule), heads,
                                              kv_heads, head_dim, dtype, ctypes.byref(b)),
          "cp_attn_rank_workspace_size_ex")
    return b.value


def plan_stats(seq_len: int, n_img=None, cu_seqlens=None, *, cp_size: int, cp_rank: int,
               heads: int, kv_heads: int, head_dim: int, dtype: int, split: str = "head_tail") -> dict:
    """Work-list diagnostics of one rank (see cp_attn_rank_plan_stats)."""
    keep, cu_p, img_p, n = _meta(n_img, cu_seqlens)
    vals = [ctypes.c_int64(0) for _ in range(4)]
    steps = np.zeros(cp_size, dtype=np.int64)
    check(_lib.cp_attn_rank_plan_stats_ex(seq_len, img_p, cu_p, n, cp_size, cp_rank, _split_code(split),
                                          heads, kv_heads, head_dim, dtype,
                                          *[ctypes.byref(x) for x in vals],
                                          steps.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))),
          "cp_attn_rank_plan_stats_ex")
    return {"tiles": vals[0].value, "entries": vals[1].value, "kv_tiles": vals[2].value,
            "covered_pairs": vals[3].value, "step_pairs": steps.tolist()}


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return CP_DTYPE_BF16
    if t.dtype == torch.float32:
        return CP_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _stream(t) -> int:
    import torch

    return torch.cuda.current_stream(t.device).cuda_stream


def _check_gpu(named, device=None):
    """Every tensor a contiguous GPU tensor on one device (the kernels take
    raw pointers: a mismatch here would be an out-of-bounds read there)."""
    for name, t in named:
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (the HIP library has no CPU path)")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if device is None:
            device = t.device
        elif t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")
    return device


def _check_qkv(q, k, v):
    """q [T,H,D], k and v [T,Hkv,D], one dtype, one device, contiguous (THD)."""
    _check_gpu((("q", q), ("k", k), ("v", v)))
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be 3-D (THD layout)")
    T, H, D = q.shape
    Tk, Hkv, Dk = k.shape
    if tuple(v.shape) != (Tk, Hkv, Dk) or Tk != T or Dk != D:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    return _dtype_code(q), int(T), int(H), int(Hkv), int(D)


class RankAttention:
    """Reusable per-rank forward: sizes the outputs and the workspace once
    and keeps those tensors, so repeated calls (benchmarks) allocate nothing.
    ``schedule``: "auto", "row_tile" or "per_step" (CP_SCHED_*)."""

    def __init__(self, q, k, v, *, cp_size: int, cp_rank: int, n_img=None, cu_seqlens=None,
                 split: str = "head_tail", schedule: str = "auto"):
        import torch

        self.dtype, self.T, self.H, self.Hkv, self.D = _check_qkv(q, k, v)
        self.q, self.k, self.v = q, k, v
        self.cp_size, self.cp_rank = int(cp_size), int(cp_rank)
        self.split = _split_code(split)
        self.schedule = _schedule_code(schedule)
        self._keep, self._cu_p, self._img_p, self.n_samples = _meta(n_img, cu_seqlens)
        rows = ctypes.c_int64(0)
        check(_lib.cp_partition_index_ex(self.T, self._img_p, self._cu_p, self.n_samples, self.cp_size,
                                         self.cp_rank, self.split, None, 0, ctypes.byref(rows), None),
              "cp_partition_index_ex")
        self.R = rows.value
        self.ws_bytes = workspace_size(self.T, self._keep[1], self._keep[0], cp_size=self.cp_size,
                                       cp_rank=self.cp_rank, heads=self.H, kv_heads=self.Hkv,
                                       head_dim=self.D, dtype=self.dtype, split=split,
                                       schedule=schedule)
        dev = q.device
        self.out = torch.empty((self.R, self.H, self.D), dtype=q.dtype, device=dev)
        self.lse = torch.empty((self.H, self.R), dtype=torch.float32, device=dev)
        self.workspace = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=dev)

    def __call__(self, events=None):
        """Run the forward. ``events``: optional sequence of six raw
        hipEvent_t handles recorded at the stage boundaries
        (cp_attn_rank_fwd_timed)."""
        ev = None
        if events is not None:
            if len(events) != 6:
                raise ValueError("cp_attn_rank_fwd_ex records exactly six events")
            ev = (ctypes.c_void_p * 6)(*[ctypes.c_void_p(int(e) if e else None) for e in events])
        check(_lib.cp_attn_rank_fwd_ex(self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), self.dtype,
                                       self.T, self._img_p, self._cu_p, self.n_samples, self.cp_size,
                                       self.cp_rank, self.split, self.schedule, self.H, self.Hkv,
                                       self.D, self.out.data_ptr(), self.lse.data_ptr(), self.workspace.data_ptr(),
                                       self.ws_bytes, _stream(self.q), ev), "cp_attn_rank_fwd_ex")
        return self.out, self.lse


def rank_fwd(q, k, v, *, cp_size: int, cp_rank: int, n_img=None, cu_seqlens=None,
             split: str = "head_tail", schedule: str = "auto"):
    """Per-rank forward attention. Returns (out [R,H,D] in q.dtype, lse fp32 [H,R])."""
    return RankAttention(q, k, v, cp_size=cp_size, cp_rank=cp_rank, n_img=n_img,
                         cu_seqlens=cu_seqlens, split=split, schedule=schedule)()


class RankAttentionBackward:
    """Reusable per-rank backward (cp_attn_rank_bwd): plans the sizes once and
    keeps the gradient and workspace tensors. dq is fp32 [R, H, D] in the
    rank-local row order; dk, dv are fp32 [T, Hkv, D] over every key."""

    def __init__(self, q, k, v, *, cp_size: int, cp_rank: int, n_img=None, cu_seqlens=None,
                 split: str = "head_tail"):
        import torch

        self.dtype, self.T, self.H, self.Hkv, self.D = _check_qkv(q, k, v)
        self.q, self.k, self.v = q, k, v
        self.cp_size, self.cp_rank, self.split = int(cp_size), int(cp_rank), _split_code(split)
        self._keep, self._cu_p, self._img_p, self.n_samples = _meta(n_img, cu_seqlens)
        rows = ctypes.c_int64(0)
        check(_lib.cp_partition_index_ex(self.T, self._img_p, self._cu_p, self.n_samples, self.cp_size,
                                         self.cp_rank, self.split, None, 0, ctypes.byref(rows), None),
              "cp_partition_index_ex")
        self.R = rows.value
        b = ctypes.c_size_t(0)
        check(_lib.cp_attn_rank_bwd_workspace_size(self.T, self._img_p, self._cu_p, self.n_samples,
                                                   self.cp_size, self.cp_rank, self.split, self.H,
                                                   self.Hkv, self.D, self.dtype, ctypes.byref(b)),
              "cp_attn_rank_bwd_workspace_size")
        self.ws_bytes = b.value
        dev = q.device
        self.dq = torch.empty((self.R, self.H, self.D), dtype=torch.float32, device=dev)
        self.dk = torch.empty((self.T, self.Hkv, self.D), dtype=torch.float32, device=dev)
        self.dv = torch.empty_like(self.dk)
        self.workspace = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=dev)

    def __call__(self, out, lse, dout):
        import torch

        _check_gpu((("out", out), ("lse", lse), ("dout", dout)), self.q.device)
        if out.dtype != self.q.dtype or dout.dtype != self.q.dtype:
            raise TypeError(f"out and dout must have q's dtype {self.q.dtype}")
        if lse.dtype != torch.float32:
            raise TypeError("lse must be float32")
        if tuple(out.shape) != (self.R, self.H, self.D) or tuple(dout.shape) != (self.R, self.H, self.D):
            raise ValueError("out and dout must be [R, heads, head_dim] of this rank")
        if tuple(lse.shape) != (self.H, self.R):
            raise ValueError("lse must be [heads, R]")
        check(_lib.cp_attn_rank_bwd(self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), out.data_ptr(),
                                    lse.data_ptr(), dout.data_ptr(), self.dtype, self.T, self._img_p,
                                    self._cu_p, self.n_samples, self.cp_size, self.cp_rank, self.split,
                                    self.H, self.Hkv, self.D, self.dq.data_ptr(), self.dk.data_ptr(),
                                    self.dv.data_ptr(), self.workspace.data_ptr(), self.ws_bytes,
                                    _stream(self.q)), "cp_attn_rank_bwd")
        return self.dq, self.dk, self.dv


def rank_bwd(q, k, v, out, lse, dout, *, cp_size: int, cp_rank: int, n_img=None, cu_seqlens=None,
             split: str = "head_tail"):
    """Gradients of one rank's share: (dq [R,H,D], dk [T,Hkv,D], dv [T,Hkv,D]), fp32."""
    return RankAttentionBackward(q, k, v, cp_size=cp_size, cp_rank=cp_rank, n_img=n_img,
                                 cu_seqlens=cu_seqlens, split=split)(out, lse, dout)


def gather_rows(src, index):
    """dst[i] = src[index[i]] (0 where index is -1); src a GPU tensor [N, ...]."""
    import torch

    _check_gpu((("src", src),))
    index = np.asarray(index)
    if index.size and (int(index.min()) < -1 or int(index.max()) >= src.shape[0]):
        raise ValueError(f"index values must be -1 or in [0, {src.shape[0]})")
    idx = torch.as_tensor(index.astype(np.int32)).to(src.device)
    row_elems = int(np.prod(src.shape[1:])) if src.dim() > 1 else 1
    dst = torch.empty((len(idx),) + tuple(src.shape[1:]), dtype=src.dtype, device=src.device)
    check(_lib.cp_gather_rows(src.data_ptr(), _dtype_code(src), src.shape[0], row_elems, idx.data_ptr(),
                              len(idx), dst.data_ptr(), _stream(src)), "cp_gather_rows")
    return dst


def lse_merge(part_out, part_lse, step_mask, out_dtype):
    """Merge per-step partials: part_out fp32 [S,R,H,D], part_lse fp32 [S,H,R],
    step_mask uint32-compatible int [R]. Returns (out [R,H,D], lse [H,R])."""
    import torch

    _check_gpu((("part_out", part_out), ("part_lse", part_lse)))
    if part_out.dtype != torch.float32 or part_lse.dtype != torch.float32:
        raise TypeError("part_out and part_lse must be float32")
    if part_out.dim() != 4:
        raise ValueError("part_out must be [steps, rows, heads, head_dim]")
    S, R, H, D = part_out.shape
    if tuple(part_lse.shape) != (S, H, R):
        raise ValueError(f"part_lse must be [{S}, {H}, {R}], not {tuple(part_lse.shape)}")
    if len(step_mask) != R:
        raise ValueError(f"step_mask must have {R} entries")
    mask = torch.as_tensor(np.asarray(step_mask, dtype=np.uint32).view(np.int32)).to(part_out.device)
    out = torch.empty((R, H, D), dtype=out_dtype, device=part_out.device)
    lse = torch.empty((H, R), dtype=torch.float32, device=part_out.device)
    check(_lib.cp_lse_merge(part_out.data_ptr(), part_lse.data_ptr(), mask.data_ptr(), S, R, H, D,
                            _dtype_code(out), out.data_ptr(), lse.data_ptr(), _stream(part_out)),
          "cp_lse_merge")
    return out, lse
