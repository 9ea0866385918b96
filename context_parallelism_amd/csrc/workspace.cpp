#include "workspace.h"

#include <cstring>

#include "cpattn.h"
#ifdef CPATTN_CHECK_PLANS
#include "plan_check.h"
#endif

namespace cpattn {

namespace {
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
}  // namespace

int32_t prepare_workspace(int64_t seq_len, const int32_t* n_img, const int32_t* cu_seqlens,
                          int32_t n_samples, int32_t cp_size, int32_t cp_rank, int32_t heads,
                          int32_t kv_heads, int32_t head_dim, int32_t dtype, Workspace& w,
                          int32_t split, int32_t schedule) {
  if (dtype != CP_DTYPE_F32 && dtype != CP_DTYPE_BF16) return CP_EUNSUPPORTED;
  if (heads < 1 || kv_heads < 1 || heads % kv_heads != 0) return CP_EINVAL;
  if (head_dim != 64 && head_dim != 128) return CP_EUNSUPPORTED;
  if (schedule != CP_SCHED_AUTO && schedule != CP_SCHED_ROW_TILE && schedule != CP_SCHED_PER_STEP)
    return CP_EUNSUPPORTED;
  // one online softmax across the steps exists for bf16 head_dim 128 only
  const bool has_row_tile = dtype == CP_DTYPE_BF16 && head_dim == 128;
  if (schedule == CP_SCHED_ROW_TILE && !has_row_tile) return CP_EUNSUPPORTED;
  int32_t st = build_meta(seq_len, n_img, cu_seqlens, n_samples, cp_size, cp_rank, w.meta, split);
  if (st != CP_OK) return st;
  w.heads = heads;
  w.kv_heads = kv_heads;
  w.head_dim = head_dim;
  w.dtype = dtype;
  w.shape = tile_shape(dtype, heads / kv_heads, head_dim);
  build_plan(w.meta, w.shape.rows, kBlockN, w.plan);
  const size_t R = size_t(w.meta.rows);
  size_t off = 0;
  w.off_index = off;
  off = align256(off + R * sizeof(int32_t));
  w.off_mask = off;
  off = align256(off + R * sizeof(uint32_t));
  w.off_tiles = off;
  off = align256(off + w.plan.tiles.size() * sizeof(TileRec));
  w.off_entries = off;
  off = align256(off + w.plan.entries.size() * sizeof(EntryRec));
  w.off_spans = off;
  off = align256(off + w.plan.spans.size() * sizeof(SpanRec));
  w.unit_kernel = has_row_tile;
  if (w.unit_kernel) {
    const int64_t n_hg = heads / w.shape.heads_per_wg;
    w.unit_per_step = schedule == CP_SCHED_PER_STEP ||
                      (schedule == CP_SCHED_AUTO && int64_t(w.plan.units.size()) * n_hg < kUnitMinWorkgroups);
    // one workgroup of the row-tile kernel per compute unit: 32 per XCD
    w.xcd_major = !w.unit_per_step && choose_xcd_major(w.meta, w.plan, int32_t(n_hg), 32);
  }
#ifdef CPATTN_CHECK_PLANS
  st = check_plan(w.meta, w.plan);  // the plan as launched (units in their final order)
  if (st != CP_OK) return st;
#endif
  w.off_tile_entries = off;
  off = align256(off + w.launch_entries().size() * sizeof(EntryRec));
  w.off_units = off;
  off = align256(off + w.launch_units().size() * sizeof(UnitRec));
  w.plan_bytes = off;
  w.off_po = off;
  if (w.unit_kernel && !w.unit_per_step) {
    // one online softmax across all ring steps of a row tile: no partials
    w.off_pl = off;
  } else {
    off = align256(off + size_t(cp_size) * R * size_t(heads) * head_dim * sizeof(float));
    w.off_pl = off;
    off = align256(off + size_t(cp_size) * size_t(heads) * R * sizeof(float));
  }
  w.total = off;
  return CP_OK;
}

void pack_plan(const Workspace& w, uint8_t* dst) {
  std::memset(dst, 0, w.plan_bytes);
  const Plan& p = w.plan;
  if (!p.index.empty()) std::memcpy(dst + w.off_index, p.index.data(), p.index.size() * sizeof(int32_t));
  if (!p.row_mask.empty())
    std::memcpy(dst + w.off_mask, p.row_mask.data(), p.row_mask.size() * sizeof(uint32_t));
  if (!p.tiles.empty()) std::memcpy(dst + w.off_tiles, p.tiles.data(), p.tiles.size() * sizeof(TileRec));
  if (!p.entries.empty())
    std::memcpy(dst + w.off_entries, p.entries.data(), p.entries.size() * sizeof(EntryRec));
  if (!p.spans.empty()) std::memcpy(dst + w.off_spans, p.spans.data(), p.spans.size() * sizeof(SpanRec));
  const std::vector<EntryRec>& e = w.launch_entries();
  if (!e.empty()) std::memcpy(dst + w.off_tile_entries, e.data(), e.size() * sizeof(EntryRec));
  const std::vector<UnitRec>& u = w.launch_units();
  if (!u.empty()) std::memcpy(dst + w.off_units, u.data(), u.size() * sizeof(UnitRec));
}

int32_t prepare_bwd_workspace(int64_t seq_len, const int32_t* n_img, const int32_t* cu_seqlens,
                              int32_t n_samples, int32_t cp_size, int32_t cp_rank, int32_t split,
                              int32_t heads, int32_t kv_heads, int32_t head_dim, int32_t dtype,
                              BwdWorkspace& w) {
  if (dtype != CP_DTYPE_F32 && dtype != CP_DTYPE_BF16) return CP_EUNSUPPORTED;
  if (heads < 1 || kv_heads < 1 || heads % kv_heads != 0) return CP_EINVAL;
  if (head_dim != 64 && head_dim != 128) return CP_EUNSUPPORTED;
  int32_t st = build_meta(seq_len, n_img, cu_seqlens, n_samples, cp_size, cp_rank, w.meta, split);
  if (st != CP_OK) return st;
  w.heads = heads;
  w.kv_heads = kv_heads;
  w.head_dim = head_dim;
  const int32_t group = heads / kv_heads;
  w.mfma = dtype == CP_DTYPE_BF16 && head_dim == 128;
  if (w.mfma) {
    w.heads_per_wg = (group % 4 == 0) ? 4 : (group % 2 == 0) ? 2 : 1;
    w.rows_per_tile = 32 * 4 / w.heads_per_wg;  // dQ: 4 waves of 32 rows
  } else {
    w.heads_per_wg = 1;
    w.rows_per_tile = 256 / (head_dim / 32);  // dQ: 256 threads, head_dim / 32 per row
  }
  w.n_hg = heads / w.heads_per_wg;
  build_bwd_plan(w.meta, w.rows_per_tile, w.plan);
  if (w.mfma) {
    // workgroup orders of the MFMA kernels: dQ runs two workgroups per
    // compute unit (64 per XCD), dK/dV one (32)
    w.q_xcd_major = choose_xcd_major(w.meta, w.plan.rows, w.n_hg, 64);
    std::vector<int64_t> cost(w.plan.ktiles.size());
    std::vector<int32_t> sample(w.plan.ktiles.size());
    for (size_t i = 0; i < cost.size(); ++i) {
      cost[i] = w.plan.ktiles[i].rb1 - w.plan.ktiles[i].rb0;
      sample[i] = w.plan.ktiles[i].s0;  // the sample's first token identifies it
    }
    std::vector<int64_t> order;
    w.kv_xcd_major = xcd_major_order(cost, sample, kv_heads, 32, order);
    if (w.kv_xcd_major) {
      std::vector<KeyTileRec> kt;
      kt.reserve(order.size());
      for (int64_t i : order) kt.push_back(w.plan.ktiles[size_t(i)]);
      w.plan.ktiles.swap(kt);
    }
  }
#ifdef CPATTN_CHECK_PLANS
  st = check_bwd_plan(w.meta, w.plan);  // the plan as launched
  if (st != CP_OK) return st;
#endif
  const Plan& p = w.plan.rows;
  const size_t R = size_t(w.meta.rows);
  size_t off = 0;
  w.off_index = off;
  off = align256(off + R * sizeof(int32_t));
  w.off_tiles = off;
  off = align256(off + p.tiles.size() * sizeof(TileRec));
  w.off_spans = off;
  off = align256(off + p.spans.size() * sizeof(SpanRec));
  w.off_tile_entries = off;  // the units' entries
  off = align256(off + p.unit_entries.size() * sizeof(EntryRec));
  w.off_units = off;
  off = align256(off + p.units.size() * sizeof(UnitRec));
  w.off_ktiles = off;
  off = align256(off + w.plan.ktiles.size() * sizeof(KeyTileRec));
  w.off_row_lo = off;
  off = align256(off + w.plan.row_lo.size() * sizeof(int32_t));
  w.off_blk = off;
  off = align256(off + w.plan.blk.size() * sizeof(int32_t));
  w.plan_bytes = off;
  w.nrb = int32_t((R + kBwdRowBlock - 1) / kBwdRowBlock);
  w.off_qr = off;
  off = align256(off + R * size_t(heads) * head_dim * (dtype == CP_DTYPE_BF16 ? 2 : 4));
  w.off_delta = off;
  off = align256(off + size_t(heads) * R * sizeof(float));
  w.off_rec = off;
  off = align256(off + size_t(heads) * w.nrb * 4 * kBwdRowBlock * sizeof(int32_t));
  w.total = off;
  return CP_OK;
}

void pack_bwd_plan(const BwdWorkspace& w, uint8_t* dst) {
  std::memset(dst, 0, w.plan_bytes);
  const Plan& p = w.plan.rows;
  auto put = [&](size_t off, const void* src, size_t bytes) {
    if (bytes) std::memcpy(dst + off, src, bytes);
  };
  put(w.off_index, p.index.data(), p.index.size() * sizeof(int32_t));
  put(w.off_tiles, p.tiles.data(), p.tiles.size() * sizeof(TileRec));
  put(w.off_spans, p.spans.data(), p.spans.size() * sizeof(SpanRec));
  put(w.off_tile_entries, p.unit_entries.data(), p.unit_entries.size() * sizeof(EntryRec));
  put(w.off_units, p.units.data(), p.units.size() * sizeof(UnitRec));
  put(w.off_ktiles, w.plan.ktiles.data(), w.plan.ktiles.size() * sizeof(KeyTileRec));
  put(w.off_row_lo, w.plan.row_lo.data(), w.plan.row_lo.size() * sizeof(int32_t));
  put(w.off_blk, w.plan.blk.data(), w.plan.blk.size() * sizeof(int32_t));
}

}  // namespace cpattn
