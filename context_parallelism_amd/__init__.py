"""MI355X-native per-rank attention of load-balanced context parallelism.

The C ABI (include/cpattn.h) is exposed under the same names
(``cp_partition_index``, ``cp_attn_rank_fwd``, ...); ``rank_fwd`` and
friends are tensor-level helpers over it. Every step of the computation runs
in libcpattn.so (hand-written gfx950 kernels); importing this package fails
if the library has not been built.
"""
from ._lib import (  # noqa: F401
    CP_DTYPE_BF16,
    CP_DTYPE_F32,
    CP_EHIP,
    CP_EINVAL,
    CP_ENOSPC,
    CP_EUNSUPPORTED,
    CP_MAX_CP_SIZE,
    CP_NOALLOC_SCRATCH_BYTES,
    CP_OK,
    CP_SCHED_AUTO,
    CP_SCHED_PER_STEP,
    CP_SCHED_ROW_TILE,
    CP_SPLIT_CONTIGUOUS,
    CP_SPLIT_HEAD_TAIL,
    LIB_PATH,
    SIGNATURES,
    CpError,
    check,
    cp_attn_rank_bwd,
    cp_attn_rank_bwd_workspace_size,
    cp_attn_rank_fwd,
    cp_attn_rank_fwd_ex,
    cp_attn_rank_fwd_noalloc,
    cp_attn_rank_fwd_timed,
    cp_attn_rank_plan_stats,
    cp_attn_rank_plan_stats_ex,
    cp_attn_rank_workspace_size,
    cp_attn_rank_workspace_size_ex,
    cp_gather_rows,
    cp_lse_merge,
    cp_pair_counts,
    cp_pair_counts_ex,
    cp_partition_index,
    cp_partition_index_ex,
    cp_status_string,
    load,
)
from .api import (  # noqa: F401
    SCHEDULES,
    SPLITS,
    RankAttention,
    RankAttentionBackward,
    gather_rows,
    lse_merge,
    pair_counts,
    partition_index,
    plan_stats,
    rank_bwd,
    rank_fwd,
    workspace_size,
)

load()
