// Host-side validation of the plans the kernels walk (see plan.h). Built
// into the library only with -DCPATTN_CHECK_PLANS (the sanitizer test
// build): prepare_workspace and prepare_bwd_workspace then check every plan
// they build and return CP_EINVAL if a record could take a kernel outside
// its buffers or miss or repeat a visible pair.
//
// What a valid plan is follows from the partition of the context-parallel
// multimodal page (section 1.1: rank r's rows are chunks r and 2P-1-r of a
// sample's text; section 4.1: the image prefix on every rank; section 5.3:
// samples never see each other) and the ring steps that read source rank
// (r - s) mod P at step s.
#include "plan_check.h"

#include <algorithm>
#include <vector>

#include "cpattn.h"

namespace cpattn {

namespace {

// The sample holding global token g (samples are sorted by start).
int32_t sample_of(const Meta& m, int64_t g) {
  int32_t lo = 0, hi = int32_t(m.samples.size()) - 1;
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) / 2;
    if (m.samples[size_t(mid)].a <= g) lo = mid; else hi = mid - 1;
  }
  return lo;
}

inline int64_t sample_end(const SampleGeom& g) { return g.a + g.n_img + g.text; }

}  // namespace

int32_t check_plan(const Meta& m, const Plan& p) {
  const int64_t R = m.rows;
  if (int64_t(p.index.size()) != R || int64_t(p.row_mask.size()) != R) return CP_EINVAL;
  if (p.bm < 1 || p.bn < 1) return CP_EINVAL;
  // index: ids in [0, seq_len) or -1, no real id twice
  std::vector<uint8_t> seen(size_t(m.seq_len), 0);
  for (int32_t g : p.index) {
    if (g < -1 || g >= m.seq_len) return CP_EINVAL;
    if (g >= 0 && seen[size_t(g)]++) return CP_EINVAL;
  }
  // tiles: runs of consecutive real tokens of one sample, inside [0, R)
  std::vector<int32_t> tile_of_row(size_t(R), -1);
  for (size_t t = 0; t < p.tiles.size(); ++t) {
    const TileRec& tr = p.tiles[t];
    if (tr.nrows < 1 || tr.nrows > p.bm || tr.local0 < 0 || int64_t(tr.local0) + tr.nrows > R)
      return CP_EINVAL;
    if (tr.g0 < 0 || int64_t(tr.g0) + tr.nrows > m.seq_len) return CP_EINVAL;
    const int32_t s = sample_of(m, tr.g0);
    if (int64_t(tr.g0) + tr.nrows > sample_end(m.samples[size_t(s)])) return CP_EINVAL;
    for (int32_t i = 0; i < tr.nrows; ++i) {
      const size_t l = size_t(tr.local0 + i);
      if (p.index[l] != tr.g0 + i) return CP_EINVAL;
      if (tile_of_row[l] != -1) return CP_EINVAL;  // a row in two tiles
      tile_of_row[l] = int32_t(t);
    }
  }
  for (int64_t l = 0; l < R; ++l)  // every real row in a tile, no pad row in one
    if ((p.index[size_t(l)] >= 0) != (tile_of_row[size_t(l)] >= 0)) return CP_EINVAL;

  // entries in (tile, step) order; spans inside the tile's sample, at or
  // below its last row, inside the key ranges of that ring step
  std::vector<SpanRec> ranges;
  std::vector<int64_t> entry_pairs(p.tile_entries.size(), 0);
  for (size_t e = 0; e < p.tile_entries.size(); ++e) {
    const EntryRec& er = p.tile_entries[e];
    if (er.tile < 0 || size_t(er.tile) >= p.tiles.size() || er.step < 0 || er.step >= m.P) return CP_EINVAL;
    if (er.span_begin < 0 || er.span_begin >= er.span_end || size_t(er.span_end) > p.spans.size())
      return CP_EINVAL;
    if (e > 0) {
      const EntryRec& prev = p.tile_entries[e - 1];
      if (prev.tile > er.tile || (prev.tile == er.tile && prev.step >= er.step)) return CP_EINVAL;
    }
    const TileRec& tr = p.tiles[size_t(er.tile)];
    const int32_t s = sample_of(m, tr.g0);
    ranges.clear();
    step_ranges(m, s, er.step, ranges);
    int32_t last_k1 = -1;
    for (int32_t i = er.span_begin; i < er.span_end; ++i) {
      const SpanRec& sp = p.spans[size_t(i)];
      if (sp.k0 >= sp.k1 || sp.k0 < last_k1) return CP_EINVAL;  // empty or overlapping spans
      last_k1 = sp.k1;
      if (int64_t(sp.k1) > int64_t(tr.g0) + tr.nrows) return CP_EINVAL;  // above the tile's last row
      bool inside = false;
      for (const SpanRec& rg : ranges) inside = inside || (rg.k0 <= sp.k0 && sp.k1 <= rg.k1);
      if (!inside) return CP_EINVAL;
      for (int32_t r = 0; r < tr.nrows; ++r) {
        const int64_t g = int64_t(tr.g0) + r;
        const int64_t hi = std::min<int64_t>(sp.k1, g + 1);
        if (hi > sp.k0) entry_pairs[e] += hi - sp.k0;
      }
    }
    // a span is clipped, never dropped: each step range below the tile's
    // last row appears as the span that starts at the range's start
    for (const SpanRec& rg : ranges) {
      if (int64_t(rg.k0) >= int64_t(tr.g0) + tr.nrows) continue;
      bool found = false;
      for (int32_t i = er.span_begin; i < er.span_end; ++i) found = found || p.spans[size_t(i)].k0 == rg.k0;
      if (!found) return CP_EINVAL;
    }
  }
  // every (tile, step) pair that sees a key has exactly one entry, and the
  // row step masks say which
  for (size_t t = 0; t < p.tiles.size(); ++t) {
    const TileRec& tr = p.tiles[t];
    const int32_t s = sample_of(m, tr.g0);
    uint32_t want = 0;
    for (int32_t st = 0; st < m.P; ++st) {
      ranges.clear();
      step_ranges(m, s, st, ranges);
      for (const SpanRec& rg : ranges)
        if (int64_t(rg.k0) < int64_t(tr.g0) + tr.nrows) want |= 1u << st;
    }
    for (int32_t i = 0; i < tr.nrows; ++i)
      if (p.row_mask[size_t(tr.local0 + i)] != want) return CP_EINVAL;
  }
  for (int64_t l = 0; l < R; ++l)
    if (p.index[size_t(l)] < 0 && p.row_mask[size_t(l)] != 0) return CP_EINVAL;

  // entries (launch order) are the tile entries, each once
  if (p.entries.size() != p.tile_entries.size() || p.step_units.size() != p.tile_entries.size())
    return CP_EINVAL;
  {
    auto key = [](const EntryRec& e) { return (int64_t(e.tile) << 32) | uint32_t(e.step); };
    std::vector<int64_t> a, b;
    for (const EntryRec& e : p.entries) a.push_back(key(e));
    for (const EntryRec& e : p.tile_entries) b.push_back(key(e));
    std::sort(a.begin(), a.end());
    if (a != b) return CP_EINVAL;  // tile_entries is sorted by (tile, step) above
  }
  // key tiles of p.bn keys over entries [e0, e1) of `list` (their spans
  // contiguous), each span from its start rounded down to 8
  auto walk_tiles = [&](const std::vector<EntryRec>& list, int32_t e0, int32_t e1) {
    int64_t n = 0;
    for (int32_t i = list[size_t(e0)].span_begin; i < list[size_t(e1 - 1)].span_end; ++i)
      n += (int64_t(p.spans[size_t(i)].k1) - (p.spans[size_t(i)].k0 & ~7) + p.bn - 1) / p.bn;
    return n;
  };
  // units: one per tile that has entries, each with its own unit entry,
  // whose spans are the tile's step spans in key order, joined where one
  // ends at the next's start: sorted, apart, and covered exactly by them
  if (p.unit_entries.size() != p.units.size()) return CP_EINVAL;
  std::vector<uint8_t> unit_seen(p.tiles.size(), 0), ue_seen(p.unit_entries.size(), 0);
  std::vector<SpanRec> tile_spans;
  for (const UnitRec& u : p.units) {
    if (u.tile < 0 || size_t(u.tile) >= p.tiles.size() || unit_seen[size_t(u.tile)]) return CP_EINVAL;
    unit_seen[size_t(u.tile)] = 1;
    if (u.e0 < 0 || u.e1 != u.e0 + 1 || size_t(u.e0) >= p.unit_entries.size() || ue_seen[size_t(u.e0)])
      return CP_EINVAL;
    ue_seen[size_t(u.e0)] = 1;
    const EntryRec& ue = p.unit_entries[size_t(u.e0)];
    if (ue.tile != u.tile || ue.step != -1) return CP_EINVAL;
    if (ue.span_begin < 0 || ue.span_begin >= ue.span_end || size_t(ue.span_end) > p.spans.size())
      return CP_EINVAL;
    if (int64_t(u.n_tiles) != walk_tiles(p.unit_entries, u.e0, u.e1)) return CP_EINVAL;
    tile_spans.clear();
    for (const EntryRec& e : p.tile_entries)
      if (e.tile == u.tile)
        for (int32_t i = e.span_begin; i < e.span_end; ++i) tile_spans.push_back(p.spans[size_t(i)]);
    std::sort(tile_spans.begin(), tile_spans.end(),
              [](const SpanRec& x, const SpanRec& y) { return x.k0 < y.k0; });
    size_t j = 0;
    int64_t prev_k1 = INT64_MIN;
    for (int32_t i = ue.span_begin; i < ue.span_end; ++i) {
      const SpanRec& sp = p.spans[size_t(i)];
      if (sp.k0 >= sp.k1 || int64_t(sp.k0) <= prev_k1) return CP_EINVAL;  // sorted and apart
      prev_k1 = sp.k1;
      int64_t cur = sp.k0;
      while (cur < sp.k1) {
        if (j >= tile_spans.size() || tile_spans[j].k0 != cur) return CP_EINVAL;
        cur = tile_spans[j++].k1;
      }
      if (cur != sp.k1) return CP_EINVAL;
    }
    if (j != tile_spans.size()) return CP_EINVAL;
  }
  for (size_t t = 0; t < p.tiles.size(); ++t)
    if (bool(unit_seen[t]) != (p.row_mask[size_t(p.tiles[t].local0)] != 0)) return CP_EINVAL;
  std::vector<uint8_t> su_seen(p.tile_entries.size(), 0);
  for (const UnitRec& u : p.step_units) {
    if (u.e0 < 0 || u.e1 != u.e0 + 1 || size_t(u.e0) >= p.tile_entries.size() || su_seen[size_t(u.e0)])
      return CP_EINVAL;
    su_seen[size_t(u.e0)] = 1;
    if (p.tile_entries[size_t(u.e0)].tile != u.tile) return CP_EINVAL;
    if (int64_t(u.n_tiles) != walk_tiles(p.tile_entries, u.e0, u.e1)) return CP_EINVAL;
  }

  // the spans expose every visible pair once: the rank's real pair count
  int64_t covered = 0;
  for (int64_t x : entry_pairs) covered += x;
  int64_t padded = 0, real = 0;
  pair_counts(m, &padded, &real);
  if (covered != real) return CP_EINVAL;
  int64_t pads = 0;
  for (int32_t g : p.index) pads += g < 0;
  if (pads != p.pad_rows) return CP_EINVAL;
  return CP_OK;
}

int32_t check_bwd_plan(const Meta& m, const BwdPlan& b) {
  int32_t st = check_plan(m, b.rows);
  if (st != CP_OK) return st;
  const std::vector<int32_t>& index = b.rows.index;
  const int64_t R = m.rows;
  const int64_t nrb = (R + kBwdRowBlock - 1) / kBwdRowBlock;
  if (int64_t(b.row_lo.size()) != R || int64_t(b.blk.size()) != 2 * nrb) return CP_EINVAL;
  for (int64_t l = 0; l < R; ++l) {
    const int32_t g = index[size_t(l)];
    if (g >= 0 && b.row_lo[size_t(l)] != m.samples[size_t(sample_of(m, g))].a) return CP_EINVAL;
  }
  // key tiles: every key of every sample once; the row blocks hold every
  // rank row of the sample that sees a key of the tile
  std::vector<uint8_t> key_seen(size_t(m.seq_len), 0);
  for (const KeyTileRec& t : b.ktiles) {
    if (t.k0 < 0 || t.k0 >= t.k1 || t.k1 - t.k0 > kBwdKeyTile || t.k1 > m.seq_len) return CP_EINVAL;
    const int32_t s = sample_of(m, t.k0);
    const SampleGeom& g = m.samples[size_t(s)];
    if (t.s0 != g.a || t.s1 != sample_end(g) || t.k1 > t.s1) return CP_EINVAL;
    if (t.rb0 < 0 || t.rb0 > t.rb1 || t.rb1 > nrb) return CP_EINVAL;
    for (int32_t k = t.k0; k < t.k1; ++k) {
      if (key_seen[size_t(k)]) return CP_EINVAL;
      key_seen[size_t(k)] = 1;
    }
    for (int64_t l = 0; l < R; ++l) {
      const int32_t gid = index[size_t(l)];
      if (gid < t.k0 || gid >= t.s1) continue;  // pads, earlier rows, other samples
      const int64_t rb = l / kBwdRowBlock;
      if (rb < t.rb0 || rb >= t.rb1) return CP_EINVAL;
    }
  }
  for (int64_t k = 0; k < m.seq_len; ++k)
    if (!key_seen[size_t(k)]) return CP_EINVAL;
  // block bounds: the largest sample start and the smallest id of its rows
  for (int64_t rb = 0; rb < nrb; ++rb) {
    int32_t lo_max = INT32_MIN, hi_min = INT32_MAX;
    for (int64_t l = rb * kBwdRowBlock; l < std::min(R, (rb + 1) * kBwdRowBlock); ++l) {
      if (index[size_t(l)] < 0) continue;
      lo_max = std::max(lo_max, b.row_lo[size_t(l)]);
      hi_min = std::min(hi_min, index[size_t(l)]);
    }
    if (b.blk[size_t(2 * rb)] != lo_max || b.blk[size_t(2 * rb + 1)] != hi_min) return CP_EINVAL;
  }
  return CP_OK;
}

}  // namespace cpattn
