// Host-side planning for per-rank context-parallel attention: argument
// checks, the rank partition, exact pair counts and the per-step work list
// the attention kernel walks. Integer only; no HIP calls.
#pragma once

#include <cstdint>
#include <vector>

namespace cpattn {

// One packed sample as seen by one rank.
struct SampleGeom {
  int64_t a;        // global id of the sample's first token
  int32_t n_img;    // image-prefix length
  int32_t text;     // real text length T
  int32_t c;        // chunk length ceil(T / 2P)
  int64_t local0;   // first rank-local row of the sample
};

// A run of consecutive rank-local rows whose global ids are consecutive
// real tokens of one sample: the image prefix, or the real part of one of
// the rank's two text chunks.
struct Segment {
  int64_t local0;   // first rank-local row
  int64_t g0;       // global id of that row
  int32_t len;      // rows
  int32_t sample;
  int32_t kind;     // 0 image, 1 first owned chunk, 2 second owned chunk
};

// Tile shapes of the attention kernels. Each bf16 wave owns 32 query rows
// of one head; a bf16 workgroup has kBf16Waves (head_dim 64) or
// kBf16WavesD128 (head_dim 128) waves; K/V stream through LDS kBlockN keys
// at a time.
constexpr int kBlockN = 64;
constexpr int kBf16Waves = 4;
constexpr int kBf16WavesD128 = 8;  // two ping-pong groups of four
constexpr int kF32RowsPerTile = 64;

struct TileShape {
  int32_t rows;          // rows per plan tile (bm)
  int32_t heads_per_wg;  // query heads sharing one KV head in a workgroup
};

// bf16 (dtype 1): heads_per_wg = largest of 4, 2, 1 dividing heads/kv_heads,
// rows = 32 * waves / heads_per_wg. fp32: one head, kF32RowsPerTile.
TileShape tile_shape(int32_t dtype, int32_t group, int32_t head_dim);

struct Meta {
  int64_t seq_len = 0;
  int32_t P = 1, r = 0;
  int32_t split = 0;  // CP_SPLIT_HEAD_TAIL or CP_SPLIT_CONTIGUOUS
  std::vector<SampleGeom> samples;
  int64_t rows = 0;  // R
};

// Checks (seq_len, n_img, cu_seqlens, n_samples, cp_size, cp_rank) and fills
// `m`. Returns a cp_status value.
int32_t build_meta(int64_t seq_len, const int32_t* n_img, const int32_t* cu_seqlens,
                   int32_t n_samples, int32_t cp_size, int32_t cp_rank, Meta& m,
                   int32_t split = 0);

// The two text chunks (of 2P) that rank `rank` holds, in local order:
// head-tail pairing {rank, 2P-1-rank}; contiguous split {2rank, 2rank+1}.
inline void owned_chunks(const Meta& m, int32_t rank, int32_t ks[2]) {
  if (m.split == 1) {
    ks[0] = 2 * rank;
    ks[1] = 2 * rank + 1;
  } else {
    ks[0] = rank;
    ks[1] = 2 * m.P - 1 - rank;
  }
}

void fill_index(const Meta& m, int32_t* index, int32_t* cu_rows_local);
void pair_counts(const Meta& m, int64_t* padded, int64_t* real);
std::vector<Segment> segments(const Meta& m);

// Device-side plan records (plain int32 so the same bytes serve host and GPU).
struct TileRec { int32_t local0, nrows, g0, pad; };          // a row tile
// (tile, step) work; step is -1 in a unit entry, which covers all steps
struct EntryRec { int32_t tile, step, span_begin, span_end; };
struct SpanRec { int32_t k0, k1; };  // global keys [k0, k1)
// Work of one workgroup: entries [e0, e1) of the entry list its launch
// uploads, whose key spans are contiguous in the span list. A row-tile unit
// (`units`) has one unit entry (unit_entries[e0], e1 = e0 + 1): the union
// of the tile's step spans in key order. A step unit (`step_units`) has one
// (tile, step) entry of tile_entries. n_tiles: the key tiles of the plan's
// bn keys a kernel walks over those spans, each span from its start rounded
// down to 8 keys (counted here so the kernel need not walk the spans).
struct UnitRec { int32_t tile, e0, e1, n_tiles; };

struct Plan {
  int32_t bm = 0, bn = 0;
  std::vector<TileRec> tiles;
  std::vector<EntryRec> entries;  // launch order: longest first
  std::vector<EntryRec> tile_entries;  // the same entries in (tile, step) order
  // one per row tile that has entries, in tile order: all of its steps'
  // spans, sorted by key and joined where one ends at the next's start
  std::vector<EntryRec> unit_entries;
  std::vector<UnitRec> units;          // one per row tile, launch order: longest first
  std::vector<UnitRec> step_units;     // one per entry (a single step), longest first
  int64_t pad_rows = 0;                // rank-local rows with index -1
  std::vector<SpanRec> spans;
  std::vector<uint32_t> row_mask;  // per rank-local row: steps with a partial
  std::vector<int32_t> index;      // per rank-local row: global id or -1
  int64_t kv_tiles = 0;            // sum over entries of key tiles (one head group)
};

// Key ranges of ring step s for a rank (source rank j = (r - s) mod P):
// at s = 0 the sample's image prefix and the rank's own two chunks, at
// s > 0 chunks j and 2P-1-j; each clipped to real tokens. Appends to out.
void step_ranges(const Meta& m, int32_t sample, int32_t step, std::vector<SpanRec>& out);

// Row tiles of `bm` rows cut per segment; for each tile and step the key
// spans it can see (clipped to the tile's last row), entries sorted by
// descending key-tile count (`bn` keys per tile); for each tile the union of
// those spans (its unit entry).
void build_plan(const Meta& m, int32_t bm, int32_t bn, Plan& p);

// Workgroup order of the row-tile kernel (and of the backward's dQ and
// dK/dV kernels). Item-major: workgroup b takes item b / n_groups (items
// longest first) and group b % n_groups (head group, or KV head). XCD-major:
// workgroups are dealt round-robin to the 8 XCDs (b % 8), and XCD x takes
// groups x, x + 8, ... one after another, each over all items, with the
// items grouped by sample (samples with the most work first, each sample's
// items longest first). An XCD's compute units then work on one head and a
// few samples at a time, whose K/V (or Q and dO rows) its L2 can share,
// where item-major mixes n_groups / 8 heads and, in cost order, many
// samples. xcd_major_order chooses XCD-major if n_groups is a multiple of 8
// above 8 and its modelled end, on 8 XCDs running `slots` workgroups each
// (every workgroup its cost plus a fixed overhead, dispatched in order to
// the slot of its XCD that frees first), is within kXcdMajorSlack of
// item-major's: with few items per head, XCD-major starts the later heads'
// long items late. It then returns true and the grouped order of the items
// (indices into `cost`). Launches above kXcdModelMaxWorkgroups workgroups
// are not modelled and keep the item-major order.
constexpr int32_t kXcds = 8;
constexpr double kXcdMajorSlack = 1.05;
constexpr int64_t kXcdModelMaxWorkgroups = int64_t(1) << 18;
bool xcd_major_order(const std::vector<int64_t>& cost, const std::vector<int32_t>& sample,
                     int32_t n_groups, int32_t slots, std::vector<int64_t>& order);
// The same for a plan's units (sample of a unit: that of its tile), which it
// reorders when it chooses XCD-major.
bool choose_xcd_major(const Meta& m, Plan& p, int32_t n_groups, int32_t slots);

// ---------------------------------------------------------------- backward
// dK/dV work: keys [k0, k1) of one sample [s0, s1) (k1 <= s1), and the
// 32-row blocks of rank-local rows [32 rb0, 32 rb1) that hold every rank row
// of that sample with a global id >= k0 (other rows of those blocks are
// masked by their index).
constexpr int kBwdRowBlock = 32;   // rank-local rows per dK/dV row block
constexpr int kDqBlockN = 32;      // keys per dQ key tile (the backward plan's bn)
constexpr int kBwdKeyTile = 128;   // keys per dK/dV workgroup (4 waves x 32)
struct KeyTileRec { int32_t k0, k1, rb0, rb1, s0, s1, pad0, pad1; };

struct BwdPlan {
  Plan rows;                        // dQ: row tiles with their ring-step spans and units
  std::vector<KeyTileRec> ktiles;   // dK/dV: every key tile of every sample, longest first
  std::vector<int32_t> row_lo;      // per rank row: global id of its sample's first token (0 for pads)
  // per 32-row block: the largest sample start and the smallest global id
  // over its real rows (INT32_MIN / INT32_MAX when it has none); a key range
  // [k0, k1] is visible to every row of the block when lo_max <= k0 and
  // k1 <= hi_min
  std::vector<int32_t> blk;         // [n_blocks][2] = {lo_max, hi_min}
};

// rows_bm: rows per dQ row tile.
void build_bwd_plan(const Meta& m, int32_t rows_bm, BwdPlan& b);

}  // namespace cpattn
