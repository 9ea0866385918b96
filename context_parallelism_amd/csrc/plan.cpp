// Host planning: see plan.h. Partition and pair counts follow the
// context-parallel multimodal page (xuesongtap.github.io/2026/03/22/
// context-parallel-multimodal): section 1.1 (2P chunks, rank r keeps
// chunks r and 2P-1-r), section 4.1 (image prefix kept whole, only text
// split), section 5.3 (packed samples split one by one via cu_seqlens).
#include "plan.h"

#include <algorithm>
#include <functional>
#include <map>
#include <queue>

#include "cpattn.h"

namespace cpattn {

TileShape tile_shape(int32_t dtype, int32_t group, int32_t head_dim) {
  if (dtype != CP_DTYPE_BF16) return {kF32RowsPerTile, 1};
  const int32_t hpw = (group % 4 == 0) ? 4 : (group % 2 == 0) ? 2 : 1;
  const int32_t waves = head_dim == 128 ? kBf16WavesD128 : kBf16Waves;
  return {32 * waves / hpw, hpw};
}

int32_t build_meta(int64_t seq_len, const int32_t* n_img, const int32_t* cu_seqlens,
                   int32_t n_samples, int32_t cp_size, int32_t cp_rank, Meta& m, int32_t split) {
  if (split != 0 && split != 1) return CP_EUNSUPPORTED;
  if (cp_size < 1) return CP_EINVAL;
  if (cp_size > CP_MAX_CP_SIZE) return CP_EUNSUPPORTED;
  if (cp_rank < 0 || cp_rank >= cp_size) return CP_EINVAL;
  if (seq_len < 0 || n_samples < 0) return CP_EINVAL;
  if (seq_len >= (int64_t(1) << 31)) return CP_EUNSUPPORTED;
  if (cu_seqlens == nullptr) {
    if (n_samples != 1 || seq_len < 1) return CP_EINVAL;
  } else {
    if (cu_seqlens[0] != 0) return CP_EINVAL;
    for (int32_t s = 0; s < n_samples; ++s)
      if (cu_seqlens[s + 1] <= cu_seqlens[s]) return CP_EINVAL;
    if (int64_t(cu_seqlens[n_samples]) != seq_len) return CP_EINVAL;
  }
  m = Meta();
  m.split = split;
  m.seq_len = seq_len;
  m.P = cp_size;
  m.r = cp_rank;
  m.samples.resize(n_samples);
  int64_t local = 0;
  for (int32_t s = 0; s < n_samples; ++s) {
    int64_t a = cu_seqlens ? cu_seqlens[s] : 0;
    int64_t b = cu_seqlens ? cu_seqlens[s + 1] : seq_len;
    int64_t n = n_img ? n_img[s] : 0;
    if (n < 0 || n > b - a) return CP_EINVAL;
    SampleGeom& g = m.samples[s];
    g.a = a;
    g.n_img = int32_t(n);
    g.text = int32_t(b - a - n);
    g.c = int32_t((int64_t(g.text) + 2 * cp_size - 1) / (2 * cp_size));
    g.local0 = local;
    local += n + 2 * int64_t(g.c);
  }
  if (local >= (int64_t(1) << 31)) return CP_EUNSUPPORTED;
  m.rows = local;
  return CP_OK;
}

namespace {
// Real tokens of text chunk k of a sample: offsets [k*c, min((k+1)*c, T)).
inline int32_t chunk_real(const SampleGeom& g, int32_t k) {
  int64_t lo = int64_t(k) * g.c;
  int64_t hi = std::min<int64_t>(lo + g.c, g.text);
  return hi > lo ? int32_t(hi - lo) : 0;
}
// Sum of (n_img + t + 1) for t in [lo, lo + cnt): pairs of cnt text rows.
inline int64_t text_pairs(const SampleGeom& g, int64_t lo, int64_t cnt) {
  return cnt * (int64_t(g.n_img) + 1 + lo) + cnt * (cnt - 1) / 2;
}
}  // namespace

void fill_index(const Meta& m, int32_t* index, int32_t* cu_rows_local) {
  const int32_t r = m.r;
  for (size_t s = 0; s < m.samples.size(); ++s) {
    const SampleGeom& g = m.samples[s];
    if (cu_rows_local) cu_rows_local[s] = int32_t(g.local0);
    if (!index) continue;
    int32_t* out = index + g.local0;
    for (int32_t i = 0; i < g.n_img; ++i) *out++ = int32_t(g.a + i);
    int32_t ks[2];
    owned_chunks(m, r, ks);
    for (int32_t k : ks) {
      for (int32_t u = 0; u < g.c; ++u) {
        int64_t t = int64_t(k) * g.c + u;
        *out++ = t < g.text ? int32_t(g.a + g.n_img + t) : -1;
      }
    }
  }
  if (cu_rows_local) cu_rows_local[m.samples.size()] = int32_t(m.rows);
}

void pair_counts(const Meta& m, int64_t* padded, int64_t* real) {
  const int32_t r = m.r;
  int64_t pp = 0, rr = 0;
  for (const SampleGeom& g : m.samples) {
    int64_t img = int64_t(g.n_img) * (g.n_img + 1) / 2;  // image row i sees i + 1 keys
    pp += img;
    rr += img;
    int32_t ks[2];
    owned_chunks(m, r, ks);
    for (int32_t k : ks) {
      int64_t lo = int64_t(k) * g.c;
      pp += text_pairs(g, lo, g.c);
      rr += text_pairs(g, lo, chunk_real(g, k));
    }
  }
  if (padded) *padded = pp;
  if (real) *real = rr;
}

std::vector<Segment> segments(const Meta& m) {
  std::vector<Segment> out;
  const int32_t r = m.r;
  for (size_t s = 0; s < m.samples.size(); ++s) {
    const SampleGeom& g = m.samples[s];
    if (g.n_img > 0) out.push_back({g.local0, g.a, g.n_img, int32_t(s), 0});
    int32_t ks[2];
    owned_chunks(m, r, ks);
    for (int kind = 1; kind <= 2; ++kind) {
      int32_t k = ks[kind - 1];
      int32_t len = chunk_real(g, k);
      if (len == 0) continue;
      int64_t local0 = g.local0 + g.n_img + int64_t(kind - 1) * g.c;
      out.push_back({local0, g.a + g.n_img + int64_t(k) * g.c, len, int32_t(s), kind});
    }
  }
  return out;
}

void step_ranges(const Meta& m, int32_t sample, int32_t step, std::vector<SpanRec>& out) {
  const SampleGeom& g = m.samples[sample];
  const int32_t P = m.P;
  const int32_t j = ((m.r - step) % P + P) % P;  // source rank of this ring step
  if (step == 0 && g.n_img > 0) out.push_back({int32_t(g.a), int32_t(g.a + g.n_img)});
  int32_t ks[2];
  owned_chunks(m, j, ks);
  for (int32_t k : ks) {
    int32_t len = chunk_real(g, k);
    if (len == 0) continue;
    int64_t k0 = g.a + g.n_img + int64_t(k) * g.c;
    out.push_back({int32_t(k0), int32_t(k0 + len)});
  }
}

void build_plan(const Meta& m, int32_t bm, int32_t bn, Plan& p) {
  p = Plan();
  p.bm = bm;
  p.bn = bn;
  p.index.resize(size_t(m.rows));
  p.row_mask.assign(size_t(m.rows), 0u);
  if (m.rows > 0) fill_index(m, p.index.data(), nullptr);
  struct Pending { EntryRec e; int64_t cost; };
  std::vector<Pending> pend;
  std::vector<SpanRec> ranges;
  for (const Segment& seg : segments(m)) {
    for (int32_t off = 0; off < seg.len; off += bm) {
      TileRec t;
      t.local0 = int32_t(seg.local0 + off);
      t.nrows = std::min(bm, seg.len - off);
      t.g0 = int32_t(seg.g0 + off);
      t.pad = 0;
      const int32_t tile_id = int32_t(p.tiles.size());
      p.tiles.push_back(t);
      const int32_t g_hi = t.g0 + t.nrows;  // keys >= g_hi are seen by no row of the tile
      uint32_t mask = 0;
      for (int32_t s = 0; s < m.P; ++s) {
        ranges.clear();
        step_ranges(m, seg.sample, s, ranges);
        EntryRec e{tile_id, s, int32_t(p.spans.size()), 0};
        int64_t cost = 0;
        for (const SpanRec& rg : ranges) {
          int32_t k1 = std::min(rg.k1, g_hi);
          if (k1 <= rg.k0) continue;
          p.spans.push_back({rg.k0, k1});
          // tiles start at multiples of 8 keys (the kernels align them)
          cost += (int64_t(k1) - (rg.k0 & ~7) + bn - 1) / bn;
        }
        e.span_end = int32_t(p.spans.size());
        if (e.span_end == e.span_begin) continue;
        mask |= 1u << s;
        pend.push_back({e, cost});
        p.kv_tiles += cost;
      }
      for (int32_t i = 0; i < t.nrows; ++i) p.row_mask[size_t(t.local0 + i)] = mask;
    }
  }
  // units: every tile's entries in step order (pend is in (tile, step) order)
  struct PendingUnit { UnitRec u; int64_t cost; };
  std::vector<PendingUnit> units;
  p.tile_entries.reserve(pend.size());
  for (size_t i = 0; i < pend.size(); ++i) {
    const int32_t e = int32_t(p.tile_entries.size());
    if (units.empty() || units.back().u.tile != pend[i].e.tile)
      units.push_back({UnitRec{pend[i].e.tile, e, e, 0}, 0});
    p.tile_entries.push_back(pend[i].e);
    units.back().u.e1 = e + 1;
    units.back().cost += pend[i].cost;
  }
  // A row-tile unit carries one online softmax across all ring steps, so it
  // may walk the union of its steps' key ranges in any order: the ranges of
  // different steps are disjoint, and softmax over a union of disjoint key
  // sets is the same whatever order the sets come in. Its unit entry lists
  // the step spans sorted by key and joined where one ends at the next's
  // start, which leaves one range per row tile of a single-sample text share
  // (the sample's start up to the tile's last row) and saves the key-tile
  // rounding at each range end that does not fall on a tile boundary.
  p.unit_entries.reserve(units.size());
  std::vector<SpanRec> steps_spans;
  for (PendingUnit& u : units) {
    const EntryRec& first = p.tile_entries[size_t(u.u.e0)];
    const EntryRec& last = p.tile_entries[size_t(u.u.e1 - 1)];
    steps_spans.assign(p.spans.begin() + first.span_begin, p.spans.begin() + last.span_end);
    std::sort(steps_spans.begin(), steps_spans.end(),
              [](const SpanRec& x, const SpanRec& y) { return x.k0 < y.k0; });
    EntryRec ue{u.u.tile, -1, int32_t(p.spans.size()), 0};
    int64_t cost = 0;
    for (size_t i = 0; i < steps_spans.size();) {
      SpanRec sp = steps_spans[i++];
      while (i < steps_spans.size() && steps_spans[i].k0 == sp.k1) sp.k1 = steps_spans[i++].k1;
      p.spans.push_back(sp);
      cost += (int64_t(sp.k1) - (sp.k0 & ~7) + bn - 1) / bn;
    }
    ue.span_end = int32_t(p.spans.size());
    u.u.e0 = int32_t(p.unit_entries.size());
    u.u.e1 = u.u.e0 + 1;
    u.cost = cost;
    p.unit_entries.push_back(ue);
  }
  std::stable_sort(units.begin(), units.end(),
                   [](const PendingUnit& x, const PendingUnit& y) { return x.cost > y.cost; });
  p.units.reserve(units.size());
  for (PendingUnit& u : units) {
    u.u.n_tiles = int32_t(u.cost);
    p.units.push_back(u.u);
  }
  // step units: every entry alone, same order as the entries below
  {
    std::vector<PendingUnit> su;
    su.reserve(pend.size());
    for (size_t i = 0; i < pend.size(); ++i)
      su.push_back({UnitRec{pend[i].e.tile, int32_t(i), int32_t(i) + 1, int32_t(pend[i].cost)}, pend[i].cost});
    std::stable_sort(su.begin(), su.end(),
                     [](const PendingUnit& x, const PendingUnit& y) { return x.cost > y.cost; });
    p.step_units.reserve(su.size());
    for (const PendingUnit& u : su) p.step_units.push_back(u.u);
  }
  std::stable_sort(pend.begin(), pend.end(),
                   [](const Pending& x, const Pending& y) { return x.cost > y.cost; });
  p.entries.reserve(pend.size());
  for (const Pending& q : pend) p.entries.push_back(q.e);
  for (int32_t g : p.index) p.pad_rows += g < 0;
}

bool xcd_major_order(const std::vector<int64_t>& cost, const std::vector<int32_t>& sample,
                     int32_t n_groups, int32_t slots, std::vector<int64_t>& order) {
  const int64_t n = int64_t(cost.size());
  if (n_groups <= kXcds || n_groups % kXcds != 0 || n == 0 || slots < 1) return false;
  // the model costs a heap operation per workgroup on every call: beyond
  // kXcdModelMaxWorkgroups the order stays item-major
  if (n * n_groups > kXcdModelMaxWorkgroups) return false;
  constexpr double kWorkgroupCost = 4.5;  // a workgroup's fill and drain, in cost units
  // modelled end of a launch of the items in `ord`
  auto finish = [&](const std::vector<int64_t>& ord, bool xcd_major) {
    double end = 0.0;
    for (int32_t x = 0; x < kXcds; ++x) {
      std::priority_queue<double, std::vector<double>, std::greater<double>> free_at;
      for (int32_t c = 0; c < slots; ++c) free_at.push(0.0);
      for (int64_t b = x; b < n * n_groups; b += kXcds) {
        const int64_t i = xcd_major ? (b / kXcds) % n : b / n_groups;
        const double t = free_at.top() + double(cost[size_t(ord[size_t(i)])]) + kWorkgroupCost;
        free_at.pop();
        free_at.push(t);
        end = std::max(end, t);
      }
    }
    return end;
  };
  std::vector<int64_t> given(static_cast<size_t>(n));
  for (int64_t i = 0; i < n; ++i) given[size_t(i)] = i;
  // grouped by sample: samples with the most work first, then the items'
  // own order
  std::map<int32_t, int64_t> total;
  for (int64_t i = 0; i < n; ++i) total[sample[size_t(i)]] += cost[size_t(i)];
  std::vector<int64_t> grouped = given;
  std::stable_sort(grouped.begin(), grouped.end(), [&](int64_t x, int64_t y) {
    const int32_t a = sample[size_t(x)], b = sample[size_t(y)];
    if (a == b) return false;
    const int64_t ta = total[a], tb = total[b];
    return ta != tb ? ta > tb : a < b;
  });
  if (finish(grouped, true) > kXcdMajorSlack * finish(given, false)) return false;
  order.swap(grouped);
  return true;
}

bool choose_xcd_major(const Meta& m, Plan& p, int32_t n_groups, int32_t slots) {
  const size_t n = p.units.size();
  std::vector<int64_t> cost(n);
  std::vector<int32_t> sample(n);
  for (size_t i = 0; i < n; ++i) {
    cost[i] = p.units[i].n_tiles;
    const int64_t g = p.tiles[size_t(p.units[i].tile)].g0;
    int32_t lo = 0, hi = int32_t(m.samples.size()) - 1;
    while (lo < hi) {
      const int32_t mid = (lo + hi + 1) / 2;
      if (m.samples[size_t(mid)].a <= g) lo = mid; else hi = mid - 1;
    }
    sample[i] = lo;
  }
  std::vector<int64_t> order;
  if (!xcd_major_order(cost, sample, n_groups, slots, order)) return false;
  std::vector<UnitRec> units;
  units.reserve(n);
  for (int64_t i : order) units.push_back(p.units[size_t(i)]);
  p.units.swap(units);
  return true;
}

void build_bwd_plan(const Meta& m, int32_t rows_bm, BwdPlan& b) {
  b = BwdPlan();
  build_plan(m, rows_bm, kDqBlockN, b.rows);
  const std::vector<int32_t>& index = b.rows.index;
  struct Pending { KeyTileRec k; int64_t cost; };
  std::vector<Pending> pend;
  for (size_t si = 0; si < m.samples.size(); ++si) {
    const SampleGeom& g = m.samples[si];
    const int64_t s0 = g.a, s1 = g.a + g.n_img + g.text;  // the sample's tokens
    const int64_t l0 = g.local0, l1 = g.local0 + g.n_img + 2 * int64_t(g.c);  // its rank rows
    const int32_t rb1 = int32_t((l1 + kBwdRowBlock - 1) / kBwdRowBlock);
    // rank rows of the sample are in increasing global order apart from pads
    // (-1), so the rows that see key k0 start at the first real row >= k0
    int64_t first = l0;
    for (int64_t k0 = s0; k0 < s1; k0 += kBwdKeyTile) {
      while (first < l1 && (index[size_t(first)] < 0 || index[size_t(first)] < k0)) ++first;
      KeyTileRec t{int32_t(k0), int32_t(std::min<int64_t>(k0 + kBwdKeyTile, s1)), 0, 0,
                   int32_t(s0), int32_t(s1), 0, 0};
      if (first < l1) {
        t.rb0 = int32_t(first / kBwdRowBlock);
        t.rb1 = rb1;
      }
      pend.push_back({t, int64_t(t.rb1 - t.rb0)});
    }
  }
  std::stable_sort(pend.begin(), pend.end(),
                   [](const Pending& x, const Pending& y) { return x.cost > y.cost; });
  b.ktiles.reserve(pend.size());
  for (const Pending& q : pend) b.ktiles.push_back(q.k);

  const int64_t R = m.rows;
  b.row_lo.assign(size_t(R), 0);
  for (const SampleGeom& g : m.samples) {
    const int64_t l1 = g.local0 + g.n_img + 2 * int64_t(g.c);
    for (int64_t l = g.local0; l < l1; ++l) b.row_lo[size_t(l)] = int32_t(g.a);
  }
  const int64_t nrb = (R + kBwdRowBlock - 1) / kBwdRowBlock;
  b.blk.assign(size_t(2 * nrb), 0);
  for (int64_t rb = 0; rb < nrb; ++rb) {
    int32_t lo_max = INT32_MIN, hi_min = INT32_MAX;
    for (int64_t l = rb * kBwdRowBlock; l < std::min(R, (rb + 1) * kBwdRowBlock); ++l) {
      if (index[size_t(l)] < 0) continue;
      lo_max = std::max(lo_max, b.row_lo[size_t(l)]);
      hi_min = std::min(hi_min, index[size_t(l)]);
    }
    b.blk[size_t(2 * rb)] = lo_max;
    b.blk[size_t(2 * rb + 1)] = hi_min;
  }
}

}  // namespace cpattn
