// Launch interface of the gfx950 kernels (private to the library).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.h"

namespace cpattn {

struct AttnArgs {
  const void* q;         // Q [T, H, D]: a row tile is a run of consecutive global ids, so its
                         // rows are read in place (the rank's gather fused into the Q load)
  const void* k;         // [T, Hkv, D]
  const void* v;         // [T, Hkv, D]
  float* part_o;         // [P, R, H, D] fp32, normalised per step
  float* part_lse;       // [P, H, R] fp32, natural log
  const TileRec* tiles;
  const EntryRec* entries;
  const SpanRec* spans;
  const EntryRec* tile_entries;  // the units' entries: unit entries (row-tile schedule) or
                                 // (tile, step) entries (per-step schedule)
  const UnitRec* units;          // unit kernel work list
  void* out;                     // [R, H, D] in the input dtype (unit kernel)
  float* lse;                    // [H, R] fp32 (unit kernel)
  int32_t per_step;              // unit kernel: units of one step, partials for the merge pass
  int32_t xcd_major;             // unit kernel: XCD-major workgroup order (see xcd_major_pays)
  int32_t n_units;               // unit kernel: units in the launch
  int32_t R, H, Hkv;
  int32_t n_hg;          // head groups (workgroups per entry)
  int32_t group;         // heads / kv_heads
  float scale_log2;      // log2(e) / sqrt(D)
  float scale;           // 1 / sqrt(D)
};

// Backward (bf16, head_dim 128).
struct BwdArgs {
  const void* qr;      // gathered rank-local Q [R, H, 128]
  const void* k;       // [T, Hkv, 128]
  const void* v;       // [T, Hkv, 128]
  const void* dout;    // [R, H, 128]
  const float* lse;    // forward lse [H, R]
  const float* delta;  // rowsum(dout * out) [H, R]
  const int32_t* index;  // global id per rank row, -1 for pads
  const int32_t* rec;  // dK/dV row records [H][nrb][4][32]: lse * log2 e (+inf for pads),
                       // delta, sample start, global id - sample start
  const int32_t* blk;  // per 32-row block {largest sample start, smallest global id}
  float* dq;           // [R, H, 128]
  float* dk;           // [T, Hkv, 128]
  float* dv;           // [T, Hkv, 128]
  const TileRec* tiles;
  const SpanRec* spans;
  const EntryRec* tile_entries;  // the dQ units' entries (each the union of a row tile's step spans)
  const UnitRec* units;
  const KeyTileRec* ktiles;
  int32_t R, H, Hkv, n_hg, group, nrb;
  float scale, scale_log2;
  int32_t q_xcd_major, n_units;     // dQ workgroup order (MFMA kernel; see xcd_major_order)
  int32_t kv_xcd_major, n_ktiles;   // dK/dV workgroup order (MFMA kernel)
};

// delta[h][r] = rowsum(dout * out) for every rank row, and the dK/dV row
// records (rec, nrb 32-row blocks; row_lo: sample start per row).
hipError_t launch_bwd_prep(const void* out, const void* dout, const float* lse, const int32_t* index,
                           const int32_t* row_lo, float* delta, int32_t* rec, int32_t R, int32_t H,
                           int32_t nrb, int32_t dtype, int32_t head_dim, hipStream_t stream);
// dQ for every unit, then dK/dV for every key tile.
hipError_t launch_bwd(const BwdArgs& a, int heads_per_wg, int n_units, int n_ktiles,
                      hipStream_t stream);
// The same gradients with plain fp32 FMA kernels (fp32 inputs, or head_dim
// 64): one workgroup per (row tile, head) for dQ, per (key tile, KV head)
// for dK/dV.
hipError_t launch_bwd_generic(const BwdArgs& a, int32_t dtype, int32_t head_dim, int n_units, int n_ktiles,
                              hipStream_t stream);

hipError_t launch_gather(const void* src, const int32_t* index, void* dst, int64_t n_rows,
                         int64_t row_bytes, hipStream_t stream);

hipError_t launch_attn_bf16(const AttnArgs& a, int head_dim, int heads_per_wg, int n_entries,
                            hipStream_t stream);

// bf16, head_dim 128: one workgroup per (unit, head group), all ring steps
// of the unit's row tile, per-step partials merged in the kernel; writes
// a.out and a.lse for the unit's rows.
hipError_t launch_attn_bf16_units(const AttnArgs& a, int heads_per_wg, int n_units,
                                  hipStream_t stream);

// out[i] = 0 and lse[:, i] = -inf for every rank-local row i with index -1.
hipError_t launch_fill_pad_rows(const int32_t* index, int64_t n_rows, int32_t heads,
                                int32_t head_dim, int32_t dtype, void* out, float* lse,
                                hipStream_t stream);

hipError_t launch_attn_f32(const AttnArgs& a, int head_dim, int n_entries, hipStream_t stream);

hipError_t launch_lse_merge(const float* part_o, const float* part_lse, const uint32_t* mask,
                            int32_t n_steps, int64_t n_rows, int32_t heads, int32_t head_dim, int32_t dtype,
                            void* out, float* lse, hipStream_t stream);

}  // namespace cpattn
