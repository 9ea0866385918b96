"""Seeded synthetic workloads for per-rank context-parallel attention.

This module only draws inputs: sequence metadata (sample lengths, image
prefixes) and Q/K/V activations. It holds none of the method's arithmetic
(no partition, no masking, no softmax), so both the fp64 oracle and the HIP
path can take their inputs from here without sharing any computation.

The five workloads follow the shapes the context-parallel multimodal page
describes ("Context Parallelism for multimodal models", sections 1.1, 4.1
and 5.3): text-only causal sequences cut into 2P chunks, an image-token
prefix that every rank keeps whole, and packed samples delimited by
cu_seqlens. Activations are i.i.d. N(0, 1) because the pages use no dataset;
bf16 inputs are the round-to-nearest-even images of the fp32 draws.

Seed convention: numpy ``default_rng(1000 + number)``. For the packed
workload the per-sample lengths are drawn first (image length, then text
length, sample by sample), then Q, K and V in that order, each as
``standard_normal(dtype=float32)``.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get", "make_inputs", "random_meta", "draw_on_device"]


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape of one per-rank attention problem.

    ``n_img`` and ``text_len`` hold one entry per packed sample; a single
    sequence is one sample. ``ranks`` lists the CP ranks whose shares are
    run (in turn, on one GPU).
    """

    number: int
    name: str
    n_img: tuple
    text_len: tuple
    cp_size: int
    ranks: tuple
    heads: int
    kv_heads: int
    head_dim: int
    dtype: str  # "f32" or "bf16"

    @property
    def seed(self) -> int:
        return 1000 + self.number

    @property
    def n_samples(self) -> int:
        return len(self.text_len)

    @property
    def sample_lens(self) -> List[int]:
        return [int(a) + int(b) for a, b in zip(self.n_img, self.text_len)]

    @property
    def seq_len(self) -> int:
        return int(sum(self.sample_lens))

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.sample_lens)]).astype(np.int32)

    @property
    def n_img_array(self) -> np.ndarray:
        return np.asarray(self.n_img, dtype=np.int32)

    @property
    def rank(self) -> int:
        return int(self.ranks[0])


def _packed_lengths(seed: int, n_samples: int):
    rng = np.random.default_rng(seed)
    n_img, text = [], []
    for _ in range(n_samples):
        n_img.append(int(rng.integers(576, 2304, endpoint=True)))
        text.append(int(rng.integers(2048, 8192, endpoint=True)))
    return rng, tuple(n_img), tuple(text)


def _build() -> dict:
    _, n5, t5 = _packed_lengths(1005, 8)
    w = [
        Workload(1, "text L=256 P=2 r=0 H=2 D=64 fp32", (0,), (256,), 2, (0,), 2, 2, 64, "f32"),
        Workload(2, "text L=8192 P=4 all ranks H=16 D=128 bf16", (0,), (8192,), 4, (0, 1, 2, 3),
                 16, 16, 128, "bf16"),
        Workload(3, "image 2304 + text 16384 P=4 r=1 H=32 D=128 bf16", (2304,), (16384,), 4, (1,),
                 32, 32, 128, "bf16"),
        Workload(4, "text L=65536 P=8 r=3 GQA 32/8 D=128 bf16", (0,), (65536,), 8, (3,),
                 32, 8, 128, "bf16"),
        Workload(5, "packed 8 samples image+text P=4 r=2 H=32 D=128 bf16", n5, t5, 4, (2,),
                 32, 32, 128, "bf16"),
    ]
    return {x.number: x for x in w}


WORKLOADS = _build()


def get(number: int) -> Workload:
    return WORKLOADS[number]


def make_inputs(w: Workload, q_scale: float = 1.0, device: Optional[str] = None):
    """Draw Q [T,H,D], K [T,Hkv,D], V [T,Hkv,D] for workload ``w``.

    Returns torch tensors in the workload dtype (float32 or bfloat16),
    contiguous, on ``device`` (CPU if None). ``q_scale`` multiplies Q in
    fp32 before rounding (a peaky-softmax variant).
    """
    import torch

    if w.n_samples > 1:
        rng, n_img, text = _packed_lengths(w.seed, w.n_samples)
        assert n_img == tuple(w.n_img) and text == tuple(w.text_len)
    else:
        rng = np.random.default_rng(w.seed)
    T = w.seq_len
    q = rng.standard_normal((T, w.heads, w.head_dim), dtype=np.float32)
    k = rng.standard_normal((T, w.kv_heads, w.head_dim), dtype=np.float32)
    v = rng.standard_normal((T, w.kv_heads, w.head_dim), dtype=np.float32)
    if q_scale != 1.0:
        q *= np.float32(q_scale)
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    out = []
    for a in (q, k, v):
        t = torch.from_numpy(a).to(dt)
        if device is not None:
            t = t.to(device)
        out.append(t.contiguous())
    return tuple(out)


def random_meta(rng: np.random.Generator, n_samples: int, max_img: int, max_text: int,
                min_len: int = 1):
    """Random packed-sequence metadata for property tests.

    Returns (n_img int32[n], cu_seqlens int32[n+1]); every sample has at
    least ``min_len`` tokens, image prefixes may be empty, and a sample may
    be all image (no text).
    """
    n_img = rng.integers(0, max_img + 1, size=n_samples)
    text = rng.integers(0, max_text + 1, size=n_samples)
    lens = np.maximum(n_img + text, min_len)
    text = lens - n_img
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return n_img.astype(np.int32), cu


def draw_on_device(shapes, seed: int, dtype: str = "bf16", device: str = "cuda:0"):
    """I.i.d. N(0, 1) tensors of the given shapes for problems too large to
    draw on the host (several GB each): drawn on ``device`` by torch's
    generator seeded with ``seed``, in the order given, in fp32, then
    rounded to bf16 (or kept fp32). A checker reads back only the slices it
    needs, so both sides still take the same values from here.
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    out = []
    for shape in shapes:
        t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
        out.append(t.to(dt).contiguous())
        del t
    return tuple(out)
