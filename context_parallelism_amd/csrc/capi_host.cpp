// Host-only entry points of the C ABI (no HIP): partition, pair counts,
// workspace size, status strings. See include/cpattn.h.
#include <algorithm>
#include <exception>
#include <vector>

#include "cpattn.h"
#include "plan.h"
#include "workspace.h"

using namespace cpattn;

extern "C" {

cp_status cp_partition_index_ex(int64_t seq_len, const int32_t* n_img, const int32_t* cu_seqlens,
                                int32_t n_samples, int32_t cp_size, int32_t cp_rank, int32_t split,
                                int32_t* index, int64_t capacity, int64_t* n_rows,
                                int32_t* cu_rows_local) {
  try {
    Meta m;
    int32_t st = build_meta(seq_len, n_img, cu_seqlens, n_samples, cp_size, cp_rank, m, split);
    if (st != CP_OK) return st;
    if (index != nullptr && capacity < m.rows) return CP_ENOSPC;
    if (n_rows) *n_rows = m.rows;
    fill_index(m, index, cu_rows_local);
    return CP_OK;
  } catch (const std::exception&) {
    return CP_EINVAL;
  }
}

cp_status cp_pair_counts_ex(int64_t seq_len, const int32_t* n_img, const int32_t* cu_seqlens,
                            int32_t n_samples, int32_t cp_size, int32_t cp_rank, int32_t split,
                            int64_t* pairs_padded, int64_t* pairs_real) {
  try {
    Meta m;
    int32_t st = build_meta(seq_len, n_img, cu_seqlens, n_samples, cp_size, cp_rank, m, split);
    if (st != CP_OK) return st;
    pair_counts(m, pairs_padded, pairs_real);
    return CP_OK;
  } catch (const std::exception&) {
    return CP_EINVAL;
  }
}

cp_status cp_attn_rank_workspace_size_ex(int64_t seq_len, const int32_t* n_img,
                                         const int32_t* cu_seqlens, int32_t n_samples,
                                         int32_t cp_size, int32_t cp_rank, int32_t split,
                                         int32_t schedule, int32_t heads, int32_t kv_heads,
                                         int32_t head_dim, int32_t dtype, size_t* bytes) {
  if (bytes == nullptr) return CP_EINVAL;
  try {
    Workspace w;
    int32_t st = prepare_workspace(seq_len, n_img, cu_seqlens, n_samples, cp_size, cp_rank, heads,
                                   kv_heads, head_dim, dtype, w, split, schedule);
    if (st != CP_OK) return st;
    *bytes = w.total;
    return CP_OK;
  } catch (const std::exception&) {
    return CP_EINVAL;
  }
}

cp_status cp_attn_rank_plan_stats_ex(int64_t seq_len, const int32_t* n_img,
                                     const int32_t* cu_seqlens, int32_t n_samples, int32_t cp_size,
                                     int32_t cp_rank, int32_t split, int32_t heads,
                                     int32_t kv_heads, int32_t head_dim, int32_t dtype,
                                     int64_t* n_tiles, int64_t* n_entries, int64_t* kv_tiles,
                                     int64_t* covered_pairs, int64_t* step_pairs) {
  try {
    Workspace w;
    int32_t st = prepare_workspace(seq_len, n_img, cu_seqlens, n_samples, cp_size, cp_rank, heads,
                                   kv_heads, head_dim, dtype, w, split, CP_SCHED_AUTO);
    if (st != CP_OK) return st;
    const Plan& p = w.plan;
    std::vector<int64_t> per_step(size_t(cp_size), 0);
    int64_t total = 0;
    for (const EntryRec& e : p.entries) {
      const TileRec& t = p.tiles[size_t(e.tile)];
      for (int32_t sp = e.span_begin; sp < e.span_end; ++sp) {
        const SpanRec& s = p.spans[size_t(sp)];
        for (int32_t i = 0; i < t.nrows; ++i) {
          const int64_t g = int64_t(t.g0) + i;  // row sees keys <= g
          const int64_t hi = std::min<int64_t>(s.k1, g + 1);
          if (hi > s.k0) {
            per_step[size_t(e.step)] += hi - s.k0;
            total += hi - s.k0;
          }
        }
      }
    }
    if (n_tiles) *n_tiles = int64_t(p.tiles.size());
    if (n_entries) *n_entries = int64_t(p.entries.size());
    if (kv_tiles) *kv_tiles = p.kv_tiles;
    if (covered_pairs) *covered_pairs = total;
    if (step_pairs)
      for (int32_t s = 0; s < cp_size; ++s) step_pairs[s] = per_step[size_t(s)];
    return CP_OK;
  } catch (const std::exception&) {
    return CP_EINVAL;
  }
}

cp_status cp_partition_index(int64_t seq_len, const int32_t* n_img, const int32_t* cu_seqlens,
                             int32_t n_samples, int32_t cp_size, int32_t cp_rank, int32_t* index,
                             int64_t capacity, int64_t* n_rows, int32_t* cu_rows_local) {
  return cp_partition_index_ex(seq_len, n_img, cu_seqlens, n_samples, cp_size, cp_rank,
                               CP_SPLIT_HEAD_TAIL, index, capacity, n_rows, cu_rows_local);
}

cp_status cp_pair_counts(int64_t seq_len, const int32_t* n_img, const int32_t* cu_seqlens,
                         int32_t n_samples, int32_t cp_size, int32_t cp_rank, int64_t* pairs_padded,
                         int64_t* pairs_real) {
  return cp_pair_counts_ex(seq_len, n_img, cu_seqlens, n_samples, cp_size, cp_rank,
                           CP_SPLIT_HEAD_TAIL, pairs_padded, pairs_real);
}

cp_status cp_attn_rank_workspace_size(int64_t seq_len, const int32_t* n_img,
                                      const int32_t* cu_seqlens, int32_t n_samples,
                                      int32_t cp_size, int32_t cp_rank, int32_t heads,
                                      int32_t kv_heads, int32_t head_dim, int32_t dtype,
                                      size_t* bytes) {
  return cp_attn_rank_workspace_size_ex(seq_len, n_img, cu_seqlens, n_samples, cp_size, cp_rank,
                                        CP_SPLIT_HEAD_TAIL, CP_SCHED_AUTO, heads, kv_heads, head_dim,
                                        dtype, bytes);
}

cp_status cp_attn_rank_plan_stats(int64_t seq_len, const int32_t* n_img, const int32_t* cu_seqlens,
                                  int32_t n_samples, int32_t cp_size, int32_t cp_rank,
                                  int32_t heads, int32_t kv_heads, int32_t head_dim, int32_t dtype,
                                  int64_t* n_tiles, int64_t* n_entries, int64_t* kv_tiles,
                                  int64_t* covered_pairs, int64_t* step_pairs) {
  return cp_attn_rank_plan_stats_ex(seq_len, n_img, cu_seqlens, n_samples, cp_size, cp_rank,
                                    CP_SPLIT_HEAD_TAIL, heads, kv_heads, head_dim, dtype, n_tiles,
                                    n_entries, kv_tiles, covered_pairs, step_pairs);
}

cp_status cp_attn_rank_bwd_workspace_size(int64_t seq_len, const int32_t* n_img,
                                          const int32_t* cu_seqlens, int32_t n_samples,
                                          int32_t cp_size, int32_t cp_rank, int32_t split,
                                          int32_t heads, int32_t kv_heads, int32_t head_dim,
                                          int32_t dtype, size_t* bytes) {
  if (bytes == nullptr) return CP_EINVAL;
  try {
    BwdWorkspace w;
    int32_t st = prepare_bwd_workspace(seq_len, n_img, cu_seqlens, n_samples, cp_size, cp_rank, split,
                                       heads, kv_heads, head_dim, dtype, w);
    if (st != CP_OK) return st;
    *bytes = w.total;
    return CP_OK;
  } catch (const std::exception&) {
    return CP_EINVAL;
  }
}

const char* cp_status_string(cp_status s) {
  switch (s) {
    case CP_OK: return "success";
    case CP_EINVAL: return "invalid argument";
    case CP_ENOSPC: return "caller buffer too small";
    case CP_EUNSUPPORTED: return "unsupported argument";
    case CP_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

}  // extern "C"
