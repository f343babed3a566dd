// Host plan builder: validation of the DFS segment forest and derivation of
// the span / tile lists the kernels walk.  Plain C++, no device code.
#include "plan.hpp"

#include <algorithm>
#include <cstdio>
#include <numeric>
#include <utility>

namespace tree_attn {

namespace {

std::string fmt(const char* f, long long a, long long b = 0, long long c = 0) {
  char buf[256];
  std::snprintf(buf, sizeof(buf), f, a, b, c);
  return buf;
}

}  // namespace

bool build_host_plan(const int32_t* parent, const int32_t* seg_start, const int32_t* seg_len,
                     int32_t S, int32_t q_begin, int32_t q_end, HostPlan& p, std::string& err) {
  if (!parent || !seg_start || !seg_len) {
    err = "null topology pointer";
    return false;
  }
  if (S < 1) {
    err = fmt("num_segments must be >= 1 (got %lld)", S);
    return false;
  }
  // contiguity, lengths, total size
  int64_t T = 0;
  for (int32_t s = 0; s < S; ++s) {
    if (seg_len[s] < 1) {
      err = fmt("segment %lld has length %lld (must be >= 1)", s, seg_len[s]);
      return false;
    }
    if (seg_start[s] != T) {
      err = fmt("segment %lld starts at %lld, expected %lld (segments must be contiguous from 0)", s,
                seg_start[s], T);
      return false;
    }
    T += seg_len[s];
    if (T >= (int64_t(1) << 31)) {
      err = "total tokens must be < 2^31";
      return false;
    }
  }
  // parent links and DFS pre-order: parent[s] is -1 or on the root-to-(s-1) path
  std::vector<int32_t> path;
  p.end.assign(S, 0);
  for (int32_t s = 0; s < S; ++s) {
    const int32_t par = parent[s];
    if (par < -1 || par >= s) {
      err = fmt("segment %lld has parent %lld (must be -1 or an earlier segment)", s, par);
      return false;
    }
    while (!path.empty() && path.back() != par) {
      p.end[path.back()] = seg_start[s];
      path.pop_back();
    }
    if (par >= 0 && path.empty()) {
      err = fmt("segment %lld: parent %lld is not an ancestor of segment %lld (order is not a DFS pre-order)",
                s, par, s - 1);
      return false;
    }
    path.push_back(s);
  }
  for (int32_t s : path) p.end[s] = int32_t(T);
  if (q_end < 0) q_end = int32_t(T);
  if (q_begin < 0 || q_begin >= q_end || q_end > T) {
    err = fmt("query run [%lld, %lld) must be a non-empty range inside [0, %lld)", q_begin, q_end, T);
    return false;
  }

  p.T = int32_t(T);
  p.q_begin = q_begin;
  p.q_end = q_end;
  p.S = S;
  p.parent.assign(parent, parent + S);
  p.start.assign(seg_start, seg_start + S);
  p.len.assign(seg_len, seg_len + S);
  p.depth.assign(S, 0);
  p.prefix.assign(S, 0);
  p.num_roots = 0;
  p.max_depth = 0;
  p.max_path = 0;
  p.pairs = 0;
  for (int32_t s = 0; s < S; ++s) {
    const int32_t par = parent[s];
    if (par < 0) {
      ++p.num_roots;
    } else {
      p.depth[s] = p.depth[par] + 1;
      p.prefix[s] = p.prefix[par] + seg_len[par];
    }
    p.max_depth = std::max(p.max_depth, p.depth[s]);
    const int64_t n = seg_len[s];
    p.max_path = std::max<int64_t>(p.max_path, int64_t(p.prefix[s]) + n);
    // pairs of the run's queries in this segment: offsets [o0, o1)
    const int64_t o0 = std::max<int64_t>(0, q_begin - seg_start[s]), o1 = std::min<int64_t>(n, q_end - seg_start[s]);
    if (o1 > o0) p.pairs += (o1 - o0) * int64_t(p.prefix[s]) + (o1 * (o1 + 1) - o0 * (o0 + 1)) / 2;
  }

  // merged ancestor spans per segment: root ... parent, then the segment
  p.span_ptr.assign(S + 1, 0);
  p.spans.clear();
  std::vector<int32_t> chain;
  for (int32_t s = 0; s < S; ++s) {
    chain.clear();
    for (int32_t a = s; a >= 0; a = parent[a]) chain.push_back(a);
    std::reverse(chain.begin(), chain.end());
    int32_t virt = 0;
    const size_t first = p.spans.size();
    for (int32_t a : chain) {
      if (p.spans.size() > first && p.spans.back().phys + p.spans.back().len == seg_start[a]) {
        p.spans.back().len += seg_len[a];
      } else {
        p.spans.push_back(Span{seg_start[a], seg_len[a], virt, 0});
      }
      virt += seg_len[a];
    }
    p.span_ptr[s + 1] = int32_t(p.spans.size());
    p.max_spans = std::max(p.max_spans, p.span_ptr[s + 1] - p.span_ptr[s]);
  }

  // query tiles per size, longest key range first (stable on ties)
  for (int t = 0; t < kNumQTileSizes; ++t) {
    const int tq = kQTileSizes[t];
    auto& tiles = p.qtiles[t];
    tiles.clear();
    for (int32_t s = 0; s < S; ++s) {
      // the run's tokens of this segment, [o0, o1) from its start; a short
      // tile goes first, where its walk of the ancestor path is shortest
      // (fewer of its rows exist, so fewer wavefronts share the work)
      const int32_t o0 = std::max(0, q_begin - seg_start[s]), o1 = std::min(seg_len[s], q_end - seg_start[s]);
      const Span& f = p.spans[p.span_ptr[s]];
      for (int32_t o = o0; o < o1;) {
        const int32_t n = o == o0 && (o1 - o0) % tq ? (o1 - o0) % tq : tq;
        tiles.push_back(QTile{seg_start[s] + o, n, s, p.prefix[s] + o, p.span_ptr[s], f.phys, f.len, f.virt});
        o += n;
      }
    }
    std::stable_sort(tiles.begin(), tiles.end(), [](const QTile& a, const QTile& b) {
      return int64_t(a.pos0) + a.nq > int64_t(b.pos0) + b.nq;
    });
  }
  // 64-key tiles over every key, most run queries first (stable on ties).
  // The queries that see key tile [k0, k0 + nk) are [k0, qend); the kernels
  // walk their intersection with the run (empty: the tile's keys get zero
  // gradients).
  auto walk = [&](const KTile& t) {
    return int64_t(std::max(0, std::min(t.qend, q_end) - std::max(t.k0, q_begin)));
  };
  p.ktiles.clear();
  for (int32_t s = 0; s < S; ++s)
    for (int32_t o = 0; o < seg_len[s]; o += kKTile)
      p.ktiles.push_back(
          KTile{seg_start[s] + o, std::min(kKTile, seg_len[s] - o), s, p.end[s], seg_start[s] + seg_len[s], {}});
  std::stable_sort(p.ktiles.begin(), p.ktiles.end(), [&](const KTile& a, const KTile& b) { return walk(a) > walk(b); });
  // 128-key tiles; a segment's remainder of at most 64 keys is a 64-key tile
  // (walked at half the cost per step), so no tile is more than half empty.
  // Longest estimated walk first: query steps times 15 (128-key) or 8.
  p.ktiles_wide.clear();
  for (int32_t s = 0; s < S; ++s)
    for (int32_t o = 0; o < seg_len[s]; o += kKTileWide)
      p.ktiles_wide.push_back(
          KTile{seg_start[s] + o, std::min(kKTileWide, seg_len[s] - o), s, p.end[s], seg_start[s] + seg_len[s], {}});
  auto cost = [&](const KTile& t) { return (walk(t) + kKTile - 1) / kKTile * (t.nk > kKTile ? 15 : 8); };
  std::stable_sort(p.ktiles_wide.begin(), p.ktiles_wide.end(),
                   [&](const KTile& a, const KTile& b) { return cost(a) > cost(b); });
  return true;
}

}  // namespace tree_attn
