"""fp64 CPU oracle for the per-rank attention of load-balanced context parallelism.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The HIP
library never calls it, links it or falls back to it, and this package
imports nothing from the HIP library.

Sources (cited by page address and section):

* the context-parallel multimodal page
  (xuesongtap.github.io/2026/03/22/context-parallel-multimodal), §1.1 (cut
  the sequence into 2P chunks, rank r keeps chunks r and 2P-1-r by an
  ``index_select`` on the sequence dimension), §2 and §4.1 (the image-token
  prefix is kept whole on every rank and only the text is split; each rank
  attends over [image, its text chunks]), §5.3 (packed samples carry
  ``cu_seqlens`` boundaries and the balancing is applied per sample);
* Ring Attention (Liu et al., ICLR 2024, cited by that page as [2]): the
  blockwise partial results are combined by their log-sum-exp, which
  reproduces the softmax over the union of the key blocks exactly.

Readings where the pages are silent:

* text not divisible by 2P is padded at its end to a multiple of 2P; pad
  rows are outputs of value 0 with lse = -inf and pad keys are never seen;
* the mask is causal with an inclusive diagonal over [image, text] inside
  one sample and block-diagonal across packed samples;
* softmax scale 1/sqrt(head_dim); lse uses the natural log;
* query head h reads KV head floor(h / (heads / kv_heads)).

Parity unpinned: the pad-row values (0 / -inf) and the pad placement are
conventions of this repository, not fixed by the pages; the tests check
them only against this oracle.
"""
from .cp_oracle import (  # noqa: F401
    chunk_len,
    owned_chunks,
    partition_index,
    pair_counts,
    attend,
    softmax_scale,
    kv_head_of,
    visible,
    causal_attention,
    rank_attention,
    attend_backward,
    rank_attention_backward,
    lse_merge,
)
