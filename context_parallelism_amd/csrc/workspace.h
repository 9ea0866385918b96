// Workspace layout of cp_attn_rank_fwd (host only, no HIP). The device
// workspace holds, each region 256-byte aligned:
//   plan   : index int32[R], step mask uint32[R], tiles, entries, spans,
//            the launched units' entries (step-ordered entries for step
//            units, unit entries for row-tile units), units (uploaded from
//            the host in one copy);
//   part_o : per-step partial outputs fp32 [P, R, H, D] and
//   part_l : per-step log-sum-exps fp32 [P, H, R], for the per-step kernels
//            and the merge pass. The unit kernel (bf16, head_dim 128, large
//            grids) carries one online softmax across all ring steps of a
//            row tile and needs neither.
#pragma once

#include <cstddef>
#include <cstdint>

#include "plan.h"

namespace cpattn {

struct Workspace {
  Meta meta;
  Plan plan;
  TileShape shape{0, 0};
  int32_t heads = 0, kv_heads = 0, head_dim = 0, dtype = 0;
  size_t off_index = 0, off_mask = 0, off_tiles = 0, off_entries = 0, off_spans = 0;
  size_t off_tile_entries = 0, off_units = 0;
  bool unit_kernel = false;  // bf16 head_dim 128: units, one online softmax across the steps
  bool unit_per_step = false;  // ... but one step per unit and the merge pass (small grids)
  bool xcd_major = false;      // unit kernel, row-tile schedule: XCD-major workgroup order
  const std::vector<UnitRec>& launch_units() const {
    return unit_per_step ? plan.step_units : plan.units;
  }
  // the entries the launched units index
  const std::vector<EntryRec>& launch_entries() const {
    return unit_kernel && !unit_per_step ? plan.unit_entries : plan.tile_entries;
  }
  size_t plan_bytes = 0;
  size_t off_po = 0, off_pl = 0, total = 0;
};

// Under CP_SCHED_AUTO, below this many workgroups the unit kernel takes
// one ring step per unit (more, smaller workgroups) and the steps are
// merged in a separate pass: two workgroups per compute unit of a 256-CU
// MI355X.
constexpr int64_t kUnitMinWorkgroups = 512;

// Checks every argument, builds the plan and the layout. Returns a cp_status.
// schedule: CP_SCHED_AUTO, CP_SCHED_ROW_TILE or CP_SCHED_PER_STEP.
int32_t prepare_workspace(int64_t seq_len, const int32_t* n_img, const int32_t* cu_seqlens,
                          int32_t n_samples, int32_t cp_size, int32_t cp_rank, int32_t heads,
                          int32_t kv_heads, int32_t head_dim, int32_t dtype, Workspace& w,
                          int32_t split, int32_t schedule);

// Backward workspace, each region 256-byte aligned:
//   plan  : index int32[R], dQ row tiles, spans, unit entries, units,
//           dK/dV key tiles, sample start per row int32[R], per 32-row
//           block bounds int32[nrb][2] (uploaded from the host in one copy);
//   qr    : gathered rank-local Q rows [R, H, D] in the input dtype;
//   delta : rowsum(dout * out) fp32 [H, R];
//   rec   : dK/dV row records [H][nrb][4][32] (nrb = ceil(R / 32)): per row
//           lse * log2(e), delta, sample start, global id - sample start.
struct BwdWorkspace {
  Meta meta;
  BwdPlan plan;
  bool mfma = false;  // bf16 with head_dim 128: the MFMA kernels; otherwise the fp32 FMA kernels
  bool q_xcd_major = false, kv_xcd_major = false;  // XCD-major orders of dQ and dK/dV (MFMA kernels)
  int32_t heads = 0, kv_heads = 0, head_dim = 0;
  int32_t heads_per_wg = 1, rows_per_tile = 0, n_hg = 0;
  size_t off_index = 0, off_tiles = 0, off_spans = 0, off_tile_entries = 0, off_units = 0,
         off_ktiles = 0, off_row_lo = 0, off_blk = 0, plan_bytes = 0;
  size_t off_qr = 0, off_delta = 0, off_rec = 0, total = 0;
  int32_t nrb = 0;
};

int32_t prepare_bwd_workspace(int64_t seq_len, const int32_t* n_img, const int32_t* cu_seqlens,
                              int32_t n_samples, int32_t cp_size, int32_t cp_rank, int32_t split,
                              int32_t heads, int32_t kv_heads, int32_t head_dim, int32_t dtype,
                              BwdWorkspace& w);
void pack_bwd_plan(const BwdWorkspace& w, uint8_t* dst);

// Writes the plan region (w.plan_bytes bytes) into dst.
void pack_plan(const Workspace& w, uint8_t* dst);

}  // namespace cpattn
