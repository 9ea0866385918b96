// Device entry points of the C ABI: the per-rank forward and the gather and
// merge steps on their own. See include/cpattn.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <exception>
#include <mutex>
#include <vector>

#include "cpattn.h"
#include "kernels.h"
#include "workspace.h"

using namespace cpattn;

namespace {

// Pinned host staging for the plan upload: a ring of kStagingSlots buffers
// per host thread. A slot's copy must have left it before a later call
// rewrites it; an event recorded after each copy guards that, so the host
// waits only when it is kStagingSlots uploads ahead of the device. Never
// freed (process lifetime).
constexpr int kStagingSlots = 4;
struct StagingSlot {
  void* host = nullptr;
  size_t cap = 0;
  hipEvent_t copied = nullptr;
  int device = -1;
  bool pending = false;
};
struct Staging {
  StagingSlot slot[kStagingSlots];
  int next = 0;
};
thread_local Staging t_stage;

template <typename Pack>
hipError_t stage_and_upload(size_t plan_bytes, Pack pack, void* dst, hipStream_t stream) {
  StagingSlot& s = t_stage.slot[t_stage.next];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (s.pending) {
    e = hipEventSynchronize(s.copied);
    if (e != hipSuccess) return e;
    s.pending = false;
  }
  if (s.copied != nullptr && s.device != dev) {
    (void)hipEventDestroy(s.copied);
    s.copied = nullptr;
  }
  if (s.copied == nullptr) {
    e = hipEventCreateWithFlags(&s.copied, hipEventDisableTiming);
    if (e != hipSuccess) return e;
    s.device = dev;
  }
  if (s.cap < plan_bytes) {
    if (s.host) (void)hipHostFree(s.host);
    s.host = nullptr;
    s.cap = 0;
    size_t cap = plan_bytes < (size_t(1) << 20) ? (size_t(1) << 20) : plan_bytes * 2;
    e = hipHostMalloc(&s.host, cap, hipHostMallocPortable);
    if (e != hipSuccess) return e;
    s.cap = cap;
  }
  pack(static_cast<uint8_t*>(s.host));
  e = hipMemcpyAsync(dst, s.host, plan_bytes, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return e;
  e = hipEventRecord(s.copied, stream);
  if (e != hipSuccess) return e;
  s.pending = true;
  t_stage.next = (t_stage.next + 1) % kStagingSlots;
  return hipSuccess;
}

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline hipError_t mark(void* const* events, int i, hipStream_t s) {
  return (events && events[i]) ? hipEventRecord(static_cast<hipEvent_t>(events[i]), s) : hipSuccess;
}

// How the plan reaches the device workspace.
enum class Upload {
  kPinnedStaging,  // the thread's pinned staging buffer, asynchronous
  kHeapWait,       // ordinary host memory, and the call waits for the copy (allocates no pinned memory)
};

// Plan on the host, then copy it into the device workspace `ws` on `s`.
hipError_t upload_plan(const Workspace& w, uint8_t* ws, hipStream_t s, Upload mode) {
  if (mode == Upload::kPinnedStaging)
    return stage_and_upload(w.plan_bytes, [&](uint8_t* dst) { pack_plan(w, dst); }, ws, s);
  std::vector<uint8_t> host(w.plan_bytes);
  pack_plan(w, host.data());
  hipError_t e = hipMemcpyAsync(ws, host.data(), w.plan_bytes, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return e;
  // `host` is freed on return: wait until the copy has read it
  return hipStreamSynchronize(s);
}

// Argument checks shared by the forward entry points (after the plan is
// built); the workspace pointer is checked by the caller.
cp_status check_fwd_pointers(const void* q, const void* k, const void* v, const void* out, const float* lse) {
  if (!q || !k || !v || !out || !lse) return CP_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(lse, 4))
    return CP_EINVAL;
  return CP_OK;
}

// Upload the plan of `w` into `ws` and launch the forward's kernels on `s`.
cp_status run_fwd(const Workspace& w, const void* q, const void* k, const void* v, int32_t dtype,
                  int32_t cp_size, int32_t heads, int32_t kv_heads, int32_t head_dim, void* out,
                  float* lse, uint8_t* ws, hipStream_t s, void* const* events, Upload mode) {
  const int64_t R = w.meta.rows;
  if (mark(events, 0, s) != hipSuccess) return CP_EHIP;
  if (upload_plan(w, ws, s, mode) != hipSuccess) return CP_EHIP;
  if (mark(events, 1, s) != hipSuccess) return CP_EHIP;
  // The attention kernels read each row tile's Q rows in place (a tile is
  // a run of consecutive global ids), so the gather has no pass of its own.
  const int32_t* index = reinterpret_cast<const int32_t*>(ws + w.off_index);
  if (mark(events, 2, s) != hipSuccess) return CP_EHIP;

  AttnArgs a;
  // (no V relayout: the bf16 head_dim-128 kernel reads V tiles row-major
  // and transposes them in its LDS reads)
  if (mark(events, 3, s) != hipSuccess) return CP_EHIP;
  a.q = q;
  a.k = k;
  a.v = v;
  a.part_o = reinterpret_cast<float*>(ws + w.off_po);
  a.part_lse = reinterpret_cast<float*>(ws + w.off_pl);
  a.tiles = reinterpret_cast<const TileRec*>(ws + w.off_tiles);
  a.entries = reinterpret_cast<const EntryRec*>(ws + w.off_entries);
  a.spans = reinterpret_cast<const SpanRec*>(ws + w.off_spans);
  a.tile_entries = reinterpret_cast<const EntryRec*>(ws + w.off_tile_entries);
  a.units = reinterpret_cast<const UnitRec*>(ws + w.off_units);
  a.out = out;
  a.lse = lse;
  a.R = int32_t(R);
  a.H = heads;
  a.Hkv = kv_heads;
  a.group = heads / kv_heads;
  a.n_hg = heads / w.shape.heads_per_wg;
  a.scale = float(1.0 / std::sqrt(double(head_dim)));
  a.scale_log2 = float(1.4426950408889634 / std::sqrt(double(head_dim)));
  const int n_entries = int(w.plan.entries.size());
  a.per_step = w.unit_per_step ? 1 : 0;
  a.xcd_major = w.xcd_major ? 1 : 0;
  a.n_units = int32_t(w.launch_units().size());
  if (w.unit_kernel && !w.unit_per_step) {
    // all ring steps of a row tile in one workgroup, merged in the kernel
    if (launch_attn_bf16_units(a, w.shape.heads_per_wg, int(w.plan.units.size()), s) != hipSuccess)
      return CP_EHIP;
    if (w.plan.pad_rows > 0 &&
        launch_fill_pad_rows(index, R, heads, head_dim, dtype, out, lse, s) != hipSuccess)
      return CP_EHIP;
    if (mark(events, 4, s) != hipSuccess) return CP_EHIP;
    if (mark(events, 5, s) != hipSuccess) return CP_EHIP;
    return CP_OK;
  }
  // per-step partials for the merge pass: small bf16 head_dim-128 grids
  // (unit kernel, one step per unit), head_dim 64, fp32
  hipError_t e = w.unit_kernel
                     ? launch_attn_bf16_units(a, w.shape.heads_per_wg, int(w.plan.step_units.size()), s)
                 : dtype == CP_DTYPE_BF16
                     ? launch_attn_bf16(a, head_dim, w.shape.heads_per_wg, n_entries, s)
                     : launch_attn_f32(a, head_dim, n_entries, s);
  if (e != hipSuccess) return CP_EHIP;
  if (mark(events, 4, s) != hipSuccess) return CP_EHIP;

  const uint32_t* mask = reinterpret_cast<const uint32_t*>(ws + w.off_mask);
  if (launch_lse_merge(a.part_o, a.part_lse, mask, cp_size, R, heads, head_dim, dtype, out, lse, s) !=
      hipSuccess)
    return CP_EHIP;
  if (mark(events, 5, s) != hipSuccess) return CP_EHIP;
  return CP_OK;
}

cp_status rank_fwd(const void* q, const void* k, const void* v, int32_t dtype, int64_t seq_len,
                   const int32_t* n_img, const int32_t* cu_seqlens, int32_t n_samples,
                   int32_t cp_size, int32_t cp_rank, int32_t split, int32_t schedule, int32_t heads,
                   int32_t kv_heads, int32_t head_dim, void* out, float* lse, void* workspace,
                   size_t workspace_bytes, void* stream, void* const* events) {
  try {
    Workspace w;
    int32_t st = prepare_workspace(seq_len, n_img, cu_seqlens, n_samples, cp_size, cp_rank, heads,
                                   kv_heads, head_dim, dtype, w, split, schedule);
    if (st != CP_OK) return st;
    if (w.meta.rows == 0) return CP_OK;
    st = check_fwd_pointers(q, k, v, out, lse);
    if (st != CP_OK) return st;
    if (!workspace || !aligned(workspace, 256)) return CP_EINVAL;
    if (workspace_bytes < w.total) return CP_ENOSPC;
    return run_fwd(w, q, k, v, dtype, cp_size, heads, kv_heads, head_dim, out, lse,
                   static_cast<uint8_t*>(workspace), static_cast<hipStream_t>(stream), events,
                   Upload::kPinnedStaging);
  } catch (const std::exception&) {
    return CP_EINVAL;
  }
}

// ------------------------------------------------ entry point without allocation
// The scratch of cp_attn_rank_fwd_noalloc: one array per GPU, in the code
// object's device memory, held until the process ends. Host code never uses
// its name as an address (on the host it only stands for the symbol): the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[CP_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, looked up on its first use.
hipError_t scratch_on_current_device(uint8_t** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = static_cast<uint8_t*>(g_scratch_ptr[dev]);
  return hipSuccess;
}

cp_status rank_fwd_noalloc(const void* q, const void* k, const void* v, int32_t dtype, int64_t seq_len,
                           const int32_t* n_img, const int32_t* cu_seqlens, int32_t n_samples,
                           int32_t cp_size, int32_t cp_rank, int32_t heads, int32_t kv_heads,
                           int32_t head_dim, void* out, float* lse, void* stream) {
  try {
    // bf16 head_dim 128 carries one online softmax across the steps: the
    // scratch holds the plan only; the other paths also hold the per-step
    // partials
    const int32_t schedule = (dtype == CP_DTYPE_BF16 && head_dim == 128) ? CP_SCHED_ROW_TILE : CP_SCHED_AUTO;
    Workspace w;
    int32_t st = prepare_workspace(seq_len, n_img, cu_seqlens, n_samples, cp_size, cp_rank, heads,
                                   kv_heads, head_dim, dtype, w, CP_SPLIT_HEAD_TAIL, schedule);
    if (st != CP_OK) return st;
    if (w.meta.rows == 0) return CP_OK;
    st = check_fwd_pointers(q, k, v, out, lse);
    if (st != CP_OK) return st;
    if (w.total > CP_NOALLOC_SCRATCH_BYTES) return CP_ENOSPC;
    uint8_t* ws = nullptr;
    if (scratch_on_current_device(&ws) != hipSuccess) return CP_EHIP;
    return run_fwd(w, q, k, v, dtype, cp_size, heads, kv_heads, head_dim, out, lse, ws,
                   static_cast<hipStream_t>(stream), nullptr, Upload::kHeapWait);
  } catch (const std::exception&) {
    return CP_EINVAL;
  }
}

cp_status rank_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
                   const void* dout, int32_t dtype, int64_t seq_len, const int32_t* n_img,
                   const int32_t* cu_seqlens, int32_t n_samples, int32_t cp_size, int32_t cp_rank,
                   int32_t split, int32_t heads, int32_t kv_heads, int32_t head_dim, float* dq,
                   float* dk, float* dv, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    BwdWorkspace w;
    int32_t st = prepare_bwd_workspace(seq_len, n_img, cu_seqlens, n_samples, cp_size, cp_rank, split,
                                       heads, kv_heads, head_dim, dtype, w);
    if (st != CP_OK) return st;
    const int64_t R = w.meta.rows;
    if (seq_len == 0) return CP_OK;  // no keys and no rows
    if (!k || !v || !dk || !dv || !workspace) return CP_EINVAL;
    if (R > 0 && (!q || !out || !lse || !dout || !dq)) return CP_EINVAL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        !aligned(dout, 16) || !aligned(lse, 4) || !aligned(dq, 16) || !aligned(dk, 16) ||
        !aligned(dv, 16) || !aligned(workspace, 256))
      return CP_EINVAL;
    if (workspace_bytes < w.total) return CP_ENOSPC;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    if (stage_and_upload(w.plan_bytes, [&](uint8_t* dst) { pack_bwd_plan(w, dst); }, ws, s) != hipSuccess)
      return CP_EHIP;
    BwdArgs a;
    a.qr = ws + w.off_qr;
    a.k = k;
    a.v = v;
    a.dout = dout;
    a.lse = lse;
    a.delta = reinterpret_cast<const float*>(ws + w.off_delta);
    a.index = reinterpret_cast<const int32_t*>(ws + w.off_index);
    a.rec = reinterpret_cast<const int32_t*>(ws + w.off_rec);
    a.blk = reinterpret_cast<const int32_t*>(ws + w.off_blk);
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.tiles = reinterpret_cast<const TileRec*>(ws + w.off_tiles);
    a.spans = reinterpret_cast<const SpanRec*>(ws + w.off_spans);
    a.tile_entries = reinterpret_cast<const EntryRec*>(ws + w.off_tile_entries);
    a.units = reinterpret_cast<const UnitRec*>(ws + w.off_units);
    a.ktiles = reinterpret_cast<const KeyTileRec*>(ws + w.off_ktiles);
    a.R = int32_t(R);
    a.H = heads;
    a.Hkv = kv_heads;
    a.n_hg = w.n_hg;
    a.group = heads / kv_heads;
    a.nrb = w.nrb;
    a.scale = float(1.0 / std::sqrt(double(head_dim)));
    a.scale_log2 = float(1.4426950408889634 / std::sqrt(double(head_dim)));
    a.q_xcd_major = w.q_xcd_major ? 1 : 0;
    a.n_units = int32_t(w.plan.rows.units.size());
    a.kv_xcd_major = w.kv_xcd_major ? 1 : 0;
    a.n_ktiles = int32_t(w.plan.ktiles.size());
    if (R > 0) {
      const int64_t row_bytes = int64_t(heads) * head_dim * (dtype == CP_DTYPE_BF16 ? 2 : 4);
      if (launch_gather(q, a.index, ws + w.off_qr, R, row_bytes, s) != hipSuccess) return CP_EHIP;
      if (launch_bwd_prep(out, dout, lse, a.index, reinterpret_cast<const int32_t*>(ws + w.off_row_lo),
                          reinterpret_cast<float*>(ws + w.off_delta), reinterpret_cast<int32_t*>(ws + w.off_rec),
                          int32_t(R), heads, w.nrb, dtype, head_dim, s) != hipSuccess)
        return CP_EHIP;
      if (w.plan.rows.pad_rows > 0 &&
          launch_fill_pad_rows(a.index, R, heads, head_dim, CP_DTYPE_F32, dq, nullptr, s) != hipSuccess)
        return CP_EHIP;
    }
    // every key tile of every sample is written (zeros where no rank row sees it)
    const int n_units = R > 0 ? int(w.plan.rows.units.size()) : 0;
    const int n_ktiles = int(w.plan.ktiles.size());
    if ((w.mfma ? launch_bwd(a, w.heads_per_wg, n_units, n_ktiles, s)
                : launch_bwd_generic(a, dtype, head_dim, n_units, n_ktiles, s)) != hipSuccess)
      return CP_EHIP;
    return CP_OK;
  } catch (const std::exception&) {
    return CP_EINVAL;
  }
}

}  // namespace

extern "C" {

cp_status cp_attn_rank_bwd(const void* q, const void* k, const void* v, const void* out,
                           const float* lse, const void* dout, int32_t dtype, int64_t seq_len,
                           const int32_t* n_img, const int32_t* cu_seqlens, int32_t n_samples,
                           int32_t cp_size, int32_t cp_rank, int32_t split, int32_t heads,
                           int32_t kv_heads, int32_t head_dim, float* dq, float* dk, float* dv,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return rank_bwd(q, k, v, out, lse, dout, dtype, seq_len, n_img, cu_seqlens, n_samples, cp_size,
                  cp_rank, split, heads, kv_heads, head_dim, dq, dk, dv, workspace, workspace_bytes,
                  stream);
}


cp_status cp_attn_rank_fwd(const void* q, const void* k, const void* v, int32_t dtype,
                           int64_t seq_len, const int32_t* n_img, const int32_t* cu_seqlens,
                           int32_t n_samples, int32_t cp_size, int32_t cp_rank, int32_t heads,
                           int32_t kv_heads, int32_t head_dim, void* out, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return rank_fwd(q, k, v, dtype, seq_len, n_img, cu_seqlens, n_samples, cp_size, cp_rank,
                  CP_SPLIT_HEAD_TAIL, CP_SCHED_AUTO, heads, kv_heads, head_dim, out, lse, workspace,
                  workspace_bytes, stream, nullptr);
}

cp_status cp_attn_rank_fwd_noalloc(const void* q, const void* k, const void* v, int32_t dtype,
                                   int64_t seq_len, const int32_t* n_img, const int32_t* cu_seqlens,
                                   int32_t n_samples, int32_t cp_size, int32_t cp_rank, int32_t heads,
                                   int32_t kv_heads, int32_t head_dim, void* out, float* lse,
                                   void* stream) {
  return rank_fwd_noalloc(q, k, v, dtype, seq_len, n_img, cu_seqlens, n_samples, cp_size, cp_rank, heads,
                          kv_heads, head_dim, out, lse, stream);
}

cp_status cp_attn_rank_fwd_timed(const void* q, const void* k, const void* v, int32_t dtype,
                                 int64_t seq_len, const int32_t* n_img, const int32_t* cu_seqlens,
                                 int32_t n_samples, int32_t cp_size, int32_t cp_rank,
                                 int32_t heads, int32_t kv_heads, int32_t head_dim, void* out,
                                 float* lse, void* workspace, size_t workspace_bytes,
                                 void* stream, void* const* events) {
  return rank_fwd(q, k, v, dtype, seq_len, n_img, cu_seqlens, n_samples, cp_size, cp_rank,
                  CP_SPLIT_HEAD_TAIL, CP_SCHED_AUTO, heads, kv_heads, head_dim, out, lse, workspace,
                  workspace_bytes, stream, events);
}

cp_status cp_attn_rank_fwd_ex(const void* q, const void* k, const void* v, int32_t dtype,
                              int64_t seq_len, const int32_t* n_img, const int32_t* cu_seqlens,
                              int32_t n_samples, int32_t cp_size, int32_t cp_rank, int32_t split,
                              int32_t schedule, int32_t heads, int32_t kv_heads, int32_t head_dim,
                              void* out, float* lse, void* workspace, size_t workspace_bytes,
                              void* stream, void* const* events) {
  return rank_fwd(q, k, v, dtype, seq_len, n_img, cu_seqlens, n_samples, cp_size, cp_rank, split,
                  schedule, heads, kv_heads, head_dim, out, lse, workspace, workspace_bytes, stream,
                  events);
}

cp_status cp_gather_rows(const void* src, int32_t dtype, int64_t src_rows, int64_t row_elems,
                         const int32_t* index, int64_t n_rows, void* dst, void* stream) {
  if (dtype != CP_DTYPE_F32 && dtype != CP_DTYPE_BF16) return CP_EUNSUPPORTED;
  if (src_rows < 0 || row_elems < 1 || n_rows < 0) return CP_EINVAL;
  const size_t esize = dtype == CP_DTYPE_BF16 ? 2 : 4;
  const int64_t row_bytes = row_elems * int64_t(esize);
  if (row_bytes % 16 != 0) return CP_EUNSUPPORTED;
  if (n_rows == 0) return CP_OK;
  if (!src || !index || !dst || !aligned(src, 16) || !aligned(dst, 16)) return CP_EINVAL;
  if (uint64_t(row_bytes / 16) * uint64_t(n_rows) >= (uint64_t(1) << 32)) return CP_EUNSUPPORTED;
  return launch_gather(src, index, dst, n_rows, row_bytes, static_cast<hipStream_t>(stream)) == hipSuccess
             ? CP_OK
             : CP_EHIP;
}

cp_status cp_lse_merge(const float* part_out, const float* part_lse, const uint32_t* step_mask,
                       int32_t n_steps, int64_t n_rows, int32_t heads, int32_t head_dim,
                       int32_t dtype, void* out, float* lse, void* stream) {
  if (dtype != CP_DTYPE_F32 && dtype != CP_DTYPE_BF16) return CP_EUNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return CP_EUNSUPPORTED;
  if (n_steps < 1 || n_rows < 0 || heads < 1) return CP_EINVAL;
  if (n_steps > CP_MAX_CP_SIZE) return CP_EUNSUPPORTED;
  if (n_rows >= (int64_t(1) << 31)) return CP_EUNSUPPORTED;
  if (n_rows == 0) return CP_OK;
  if (!part_out || !part_lse || !step_mask || !out || !lse || !aligned(part_out, 16) ||
      !aligned(out, 16))
    return CP_EINVAL;
  return launch_lse_merge(part_out, part_lse, step_mask, n_steps, n_rows, heads, head_dim, dtype, out, lse,
                          static_cast<hipStream_t>(stream)) == hipSuccess
             ? CP_OK
             : CP_EHIP;
}

}  // extern "C"
