// Host-side bounds checker for the plan builders, meant to run under
// AddressSanitizer and UndefinedBehaviorSanitizer (built with g++ by
// tests/test_host_sanitizers.py; no device code).
//
// For every forest in the input file it builds the attention plan (whole and
// for a few query runs), the bounded fragments, the Mamba tables and a CSR
// of sampled edges, and checks that every index a kernel derives from those
// tables stays inside the tensors it addresses:
//   * ancestor spans: rows phys .. phys + len - 1 inside [0, T), virtual
//     positions contiguous from 0 up to the segment's path length, and the
//     32-bit byte offsets of K/V row gathers (row * Hkv * row bytes + row
//     bytes) below 2^32 for the shapes the library accepts;
//   * query tiles of every size: inside one segment and the query run,
//     position of the first token equal to its offset on the path, every run
//     token in exactly one tile;
//   * key tiles (64 and 128 keys): inside one segment, query end equal to the
//     end of the segment's subtree, every key in exactly one tile, and the
//     two query ranges of the 128-key walk non-negative and covering exactly
//     the run's queries that see the tile;
//   * the first span copied into each query tile record;
//   * fragments, Mamba predecessors / halo / successors / units, edge CSR.
// Malformed forests must be rejected with an error, never read out of range.
//
// Input: lines "forest <name> <S>" followed by three lines of S integers
// (parent, seg_start, seg_len).  Prints "ALL OK" and exits 0 when every check
// passes; prints the first failure and exits 1 otherwise.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <fstream>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "../../shared_prefix_tree_amd/csrc/edge_plan.hpp"
#include "../../shared_prefix_tree_amd/csrc/fragments.hpp"
#include "../../shared_prefix_tree_amd/csrc/mamba_plan.hpp"
#include "../../shared_prefix_tree_amd/csrc/plan.hpp"

using namespace tree_attn;

namespace {

int g_checks = 0;

#define CHECK(cond, ...)                                                  \
  do {                                                                    \
    ++g_checks;                                                           \
    if (!(cond)) {                                                        \
      std::fprintf(stderr, "FAIL %s:%d: %s: ", __FILE__, __LINE__, #cond); \
      std::fprintf(stderr, __VA_ARGS__);                                  \
      std::fprintf(stderr, "\n");                                         \
      std::exit(1);                                                       \
    }                                                                     \
  } while (0)

struct Forest {
  std::string name;
  std::vector<int32_t> parent, start, len;
};

// Independent derivations from the parent links alone.
std::vector<int32_t> path_of(const Forest& f, int32_t s) {
  std::vector<int32_t> p;
  for (int32_t a = f.parent[s]; a >= 0; a = f.parent[a]) p.insert(p.begin(), a);
  return p;
}

void check_attention_plan(const Forest& f, int32_t qb, int32_t qe) {
  const int32_t S = int32_t(f.parent.size());
  HostPlan p;
  std::string err;
  CHECK(build_host_plan(f.parent.data(), f.start.data(), f.len.data(), S, qb, qe, p, err), "%s: %s",
        f.name.c_str(), err.c_str());
  const int32_t T = p.T;
  if (qe < 0) qe = T;
  CHECK(int32_t(p.span_ptr.size()) == S + 1 && p.span_ptr[0] == 0 && p.span_ptr[S] == int32_t(p.spans.size()),
        "%s: span CSR", f.name.c_str());
  // subtree ends and path lengths from parents
  std::vector<int32_t> end(S), prefix(S, 0);
  for (int32_t s = 0; s < S; ++s) end[s] = f.start[s] + f.len[s];
  for (int32_t s = S - 1; s >= 0; --s)
    if (f.parent[s] >= 0) end[f.parent[s]] = std::max(end[f.parent[s]], end[s]);
  for (int32_t s = 0; s < S; ++s)
    for (int32_t a : path_of(f, s)) prefix[s] += f.len[a];
  int64_t pairs = 0;
  for (int32_t s = 0; s < S; ++s) {
    CHECK(p.end[s] == end[s] && p.prefix[s] == prefix[s], "%s: segment %d end/prefix", f.name.c_str(), s);
    const int32_t a = p.span_ptr[s], b = p.span_ptr[s + 1];
    CHECK(a < b && b - a <= p.max_spans, "%s: segment %d spans", f.name.c_str(), s);
    int32_t virt = 0;
    for (int32_t k = a; k < b; ++k) {
      const Span& sp = p.spans[k];
      CHECK(sp.len >= 1 && sp.phys >= 0 && int64_t(sp.phys) + sp.len <= T, "%s: span rows", f.name.c_str());
      CHECK(sp.virt == virt, "%s: span virtual positions", f.name.c_str());
      virt += sp.len;
    }
    CHECK(virt == prefix[s] + f.len[s], "%s: segment %d path length", f.name.c_str(), s);
    CHECK(p.spans[b - 1].phys + p.spans[b - 1].len == f.start[s] + f.len[s], "%s: own span last", f.name.c_str());
    const int64_t o0 = std::max<int64_t>(0, qb - f.start[s]), o1 = std::min<int64_t>(f.len[s], int64_t(qe) - f.start[s]);
    if (o1 > o0) pairs += (o1 - o0) * int64_t(prefix[s]) + (o1 * (o1 + 1) - o0 * (o0 + 1)) / 2;
  }
  CHECK(p.pairs == pairs, "%s: pairs %lld vs %lld", f.name.c_str(), (long long)p.pairs, (long long)pairs);
  // the K/V gathers of the query-major walks use 32-bit byte offsets
  // row * Hkv * RB + chunk: for the shapes the library accepts (checked at
  // each call: T * Hkv * D * elem < 2^32) the largest row offset fits
  for (int rb : {128, 256}) {
    for (int hkv : {1, 2, 8, 64}) {
      const uint64_t kv_bytes = uint64_t(T) * hkv * rb;
      if (kv_bytes >= (uint64_t(1) << 32)) continue;  // rejected by the call
      CHECK(uint64_t(T - 1) * hkv * rb + rb <= (uint64_t(1) << 32), "%s: 32-bit K/V offsets", f.name.c_str());
    }
  }
  // query tiles of every size
  for (int t = 0; t < kNumQTileSizes; ++t) {
    const int tq = kQTileSizes[t];
    std::vector<int> seen(T, 0);
    for (const QTile& q : p.qtiles[t]) {
      CHECK(q.seg >= 0 && q.seg < S, "%s: tile segment", f.name.c_str());
      const int32_t s = q.seg;
      CHECK(q.nq >= 1 && q.nq <= tq, "%s: tile size", f.name.c_str());
      CHECK(q.q0 >= f.start[s] && int64_t(q.q0) + q.nq <= f.start[s] + f.len[s], "%s: tile inside segment",
            f.name.c_str());
      CHECK(q.q0 >= qb && q.q0 + q.nq <= qe, "%s: tile inside run", f.name.c_str());
      CHECK(q.pos0 == prefix[s] + (q.q0 - f.start[s]), "%s: tile position", f.name.c_str());
      // the walk covers virtual positions [0, pos0 + nq): all on the path
      CHECK(int64_t(q.pos0) + q.nq <= int64_t(prefix[s]) + f.len[s], "%s: walk length", f.name.c_str());
      // the first span, carried in the tile record, is the segment's first
      CHECK(q.span0 == p.span_ptr[s], "%s: tile first span index", f.name.c_str());
      const Span& sp0 = p.spans[size_t(q.span0)];
      CHECK(q.phys0 == sp0.phys && q.len0 == sp0.len && q.virt0 == sp0.virt && q.virt0 == 0,
            "%s: tile first span copy", f.name.c_str());
      for (int32_t i = q.q0; i < q.q0 + q.nq; ++i) ++seen[i];
    }
    for (int32_t i = 0; i < T; ++i)
      CHECK(seen[i] == (i >= qb && i < qe ? 1 : 0), "%s: token %d in %d tiles of %d", f.name.c_str(), i, seen[i],
            tq);
  }
  // key tiles
  for (int wide = 0; wide < 2; ++wide) {
    const auto& tiles = wide ? p.ktiles_wide : p.ktiles;
    const int tk = wide ? kKTileWide : kKTile;
    std::vector<int> seen(T, 0);
    for (const KTile& k : tiles) {
      CHECK(k.seg >= 0 && k.seg < S, "%s: key tile segment", f.name.c_str());
      CHECK(k.nk >= 1 && k.nk <= tk, "%s: key tile size", f.name.c_str());
      CHECK(k.k0 >= f.start[k.seg] && k.k0 + k.nk <= f.start[k.seg] + f.len[k.seg], "%s: key tile inside segment",
            f.name.c_str());
      CHECK(k.qend == end[k.seg] && k.qend <= T && k.qend >= k.k0 + k.nk, "%s: key tile query end",
            f.name.c_str());
      CHECK(k.send == f.start[k.seg] + f.len[k.seg], "%s: key tile segment end", f.name.c_str());
      // The 128-key walk's two query ranges, derived as the kernel derives
      // them: the segment's descendants, then its own queries.  Neither may
      // have a negative length (the copies clamp rows to range end - 1 as an
      // unsigned offset), both lie in [0, T), and together they are exactly
      // the run's queries that see the tile.
      {
        const int32_t qbeg = std::max(k.k0, qb), qend = std::max(std::min(k.qend, qe), qbeg);
        const int32_t split = std::min(std::max(k.send, qbeg), qend);
        const bool first_empty = split >= qend;
        const int32_t lo0 = first_empty ? qbeg : split, hi0 = qend;
        const int32_t lo1 = first_empty ? qend : qbeg, hi1 = first_empty ? qend : split;
        CHECK(lo0 <= hi0 && lo1 <= hi1, "%s: walk range lengths", f.name.c_str());
        CHECK(lo0 >= 0 && hi0 <= T && lo1 >= 0 && hi1 <= T, "%s: walk ranges inside [0, T)", f.name.c_str());
        const int32_t want_lo = std::max(k.k0, qb), want_hi = std::min(k.qend, qe);
        const int64_t want = std::max(0, want_hi - want_lo);
        CHECK(int64_t(hi0 - lo0) + (hi1 - lo1) == want, "%s: walk ranges cover the visible run queries",
              f.name.c_str());
        // [lo1, hi1) then directly [lo0, hi0) when both are non-empty
        if (want > 0)
          CHECK(hi0 == want_hi && (hi1 == lo1 ? lo0 == want_lo : lo1 == want_lo && hi1 == lo0),
                "%s: walk ranges adjacent", f.name.c_str());
      }
      for (int32_t j = k.k0; j < k.k0 + k.nk; ++j) ++seen[j];
    }
    for (int32_t j = 0; j < T; ++j) CHECK(seen[j] == 1, "%s: key %d in %d tiles", f.name.c_str(), j, seen[j]);
  }
}

void check_fragments(const Forest& f, int32_t bound) {
  const int32_t S = int32_t(f.parent.size());
  Fragments fr;
  std::string err;
  HostPlan p;
  CHECK(build_host_plan(f.parent.data(), f.start.data(), f.len.data(), S, 0, -1, p, err), "%s", err.c_str());
  const bool fits = p.max_path <= bound;
  const bool ok = build_fragments(f.parent.data(), f.start.data(), f.len.data(), S, bound, fr, err);
  CHECK(ok == fits, "%s: fragments accepted=%d, longest path %lld, bound %d", f.name.c_str(), ok,
        (long long)p.max_path, bound);
  if (!ok) return;
  const int32_t F = int32_t(fr.frag_seg_ptr.size()) - 1;
  CHECK(F >= 1 && int32_t(fr.frag_token_ptr.size()) == F + 1, "%s: fragment CSR", f.name.c_str());
  std::vector<int> owned(p.T, 0);
  for (int32_t g = 0; g < F; ++g) {
    const int32_t s0 = fr.frag_seg_ptr[g], s1 = fr.frag_seg_ptr[g + 1];
    const int32_t t0 = fr.frag_token_ptr[g], t1 = fr.frag_token_ptr[g + 1];
    CHECK(s0 < s1 && t0 < t1 && t1 - t0 <= bound, "%s: fragment %d size", f.name.c_str(), g);
    std::vector<int32_t> par(fr.seg_parent.begin() + s0, fr.seg_parent.begin() + s1);
    std::vector<int32_t> ln(fr.seg_len.begin() + s0, fr.seg_len.begin() + s1), st(ln.size(), 0);
    int64_t sum = 0;
    for (size_t k = 0; k < ln.size(); ++k) {
      st[k] = int32_t(sum);
      sum += ln[k];
    }
    CHECK(sum == t1 - t0, "%s: fragment %d token count", f.name.c_str(), g);
    HostPlan fp;
    CHECK(build_host_plan(par.data(), st.data(), ln.data(), int32_t(ln.size()), 0, -1, fp, err),
          "%s: fragment %d is not a forest: %s", f.name.c_str(), g, err.c_str());
    for (int32_t t = t0; t < t1; ++t) {
      const int32_t src = fr.token_source[t];
      CHECK(src >= 0 && src < p.T, "%s: token source", f.name.c_str());
      owned[src] += fr.token_owner[t];
    }
  }
  for (int32_t i = 0; i < p.T; ++i) CHECK(owned[i] == 1, "%s: token %d owned %d times", f.name.c_str(), i, owned[i]);
}

void check_mamba(const Forest& f) {
  const int32_t S = int32_t(f.parent.size());
  MambaTables m;
  std::string err;
  CHECK(build_mamba_tables(f.parent.data(), f.start.data(), f.len.data(), S, m, err), "%s", err.c_str());
  const int32_t T = m.T;
  CHECK(int32_t(m.prev.size()) == T && int64_t(m.halo.size()) == int64_t(T) * kConvHalo, "%s: mamba sizes",
        f.name.c_str());
  for (int32_t s = 0; s < S; ++s)
    for (int32_t o = 0; o < f.len[s]; ++o) {
      const int32_t i = f.start[s] + o;
      const int32_t want = o > 0 ? i - 1 : f.parent[s] < 0 ? -1 : f.start[f.parent[s]] + f.len[f.parent[s]] - 1;
      CHECK(m.prev[i] == want, "%s: prev of %d", f.name.c_str(), i);
    }
  for (int32_t i = 0; i < T; ++i) {
    int32_t j = i;
    for (int k = 1; k <= kConvHalo; ++k) {
      j = j < 0 ? -1 : m.prev[j];
      CHECK(m.halo[size_t(i) * kConvHalo + k - 1] == j, "%s: halo", f.name.c_str());
      CHECK(j >= -1 && j < i, "%s: halo range", f.name.c_str());
    }
  }
  CHECK(int32_t(m.csucc_ptr.size()) == T + 1 && m.csucc_ptr[T] == int32_t(m.csucc.size()), "%s: csucc CSR",
        f.name.c_str());
  for (int32_t j = 0; j < T; ++j)
    for (int32_t e = m.csucc_ptr[j]; e < m.csucc_ptr[j + 1]; ++e) {
      const int32_t i = m.csucc[e] >> 2, k = m.csucc[e] & 3;
      CHECK(i > j && i < T && k >= 1 && k <= kConvHalo, "%s: successor range", f.name.c_str());
      CHECK(m.halo[size_t(i) * kConvHalo + k - 1] == j && i != j + k, "%s: successor entry", f.name.c_str());
    }
  CHECK(int32_t(m.unit_start.size()) == m.U && int32_t(m.usucc_ptr.size()) == m.U + 1, "%s: units",
        f.name.c_str());
  std::vector<int> seen(T, 0);
  for (int32_t u = 0; u < m.U; ++u) {
    CHECK(m.unit_len[u] >= 1 && m.unit_len[u] <= kMambaUnit && m.unit_start[u] >= 0 &&
              m.unit_start[u] + m.unit_len[u] <= T,
          "%s: unit range", f.name.c_str());
    CHECK(m.unit_pred[u] >= -1 && m.unit_pred[u] < u, "%s: unit predecessor", f.name.c_str());
    if (m.unit_pred[u] >= 0) {
      const int32_t pu = m.unit_pred[u];
      CHECK(m.prev[m.unit_start[u]] == m.unit_start[pu] + m.unit_len[pu] - 1, "%s: unit link", f.name.c_str());
    }
    for (int32_t i = m.unit_start[u]; i < m.unit_start[u] + m.unit_len[u]; ++i) ++seen[i];
    for (int32_t e = m.usucc_ptr[u]; e < m.usucc_ptr[u + 1]; ++e)
      CHECK(m.usucc[e] > u && m.usucc[e] < m.U && m.unit_pred[m.usucc[e]] == u, "%s: unit successors",
            f.name.c_str());
  }
  for (int32_t i = 0; i < T; ++i) CHECK(seen[i] == 1, "%s: token %d in %d units", f.name.c_str(), i, seen[i]);
}

void check_edges(const Forest& f, uint64_t seed) {
  int32_t T = 0;
  for (int32_t n : f.len) T += n;
  const int32_t V = 1000, E = std::max(1, T / 3);
  std::vector<int32_t> src(E), tgt(E), row_ptr, ids;
  uint64_t x = seed * 6364136223846793005ull + 1442695040888963407ull;
  for (int32_t e = 0; e < E; ++e) {
    x = x * 6364136223846793005ull + 1442695040888963407ull;
    src[e] = int32_t((x >> 33) % uint64_t(T));
    tgt[e] = int32_t((x >> 13) % uint64_t(V));
  }
  std::string err;
  CHECK(build_edge_csr(src.data(), tgt.data(), E, T, V, row_ptr, ids, err), "%s", err.c_str());
  CHECK(int32_t(row_ptr.size()) == T + 1 && row_ptr[T] == E, "%s: edge CSR", f.name.c_str());
  std::vector<int> seen(E, 0);
  for (int32_t t = 0; t < T; ++t)
    for (int32_t k = row_ptr[t]; k < row_ptr[t + 1]; ++k) {
      CHECK(ids[k] >= 0 && ids[k] < E && src[ids[k]] == t, "%s: edge ids", f.name.c_str());
      if (k > row_ptr[t]) CHECK(ids[k] > ids[k - 1], "%s: edge order", f.name.c_str());
      ++seen[ids[k]];
    }
  for (int32_t e = 0; e < E; ++e) CHECK(seen[e] == 1, "%s: edge listed %d times", f.name.c_str(), seen[e]);
  src[E / 2] = T;  // out of range: rejected
  CHECK(!build_edge_csr(src.data(), tgt.data(), E, T, V, row_ptr, ids, err), "%s: bad edge accepted",
        f.name.c_str());
}

// Malformed variants of a forest: each must be rejected by every builder.
void check_rejections(const Forest& f) {
  const int32_t S = int32_t(f.parent.size());
  std::vector<Forest> bad;
  if (S >= 2) {
    Forest g = f;
    g.parent[S - 1] = S - 1;  // parent >= self
    bad.push_back(g);
    g = f;
    g.start[S - 1] += 1;  // gap
    bad.push_back(g);
    g = f;
    g.len[S / 2] = 0;  // empty segment
    bad.push_back(g);
    g = f;
    g.parent[S - 1] = -7;
    bad.push_back(g);
  }
  {
    Forest g = f;
    g.start[0] = 1;  // does not start at 0
    bad.push_back(g);
  }
  // a non-DFS order: a child of segment 0 after a different root
  if (S >= 3) {
    Forest g;
    g.parent = {-1, -1, 0};
    g.start = {0, 4, 8};
    g.len = {4, 4, 4};
    bad.push_back(g);
  }
  for (const Forest& g : bad) {
    HostPlan p;
    Fragments fr;
    MambaTables m;
    std::string err;
    const int32_t n = int32_t(g.parent.size());
    CHECK(!build_host_plan(g.parent.data(), g.start.data(), g.len.data(), n, 0, -1, p, err),
          "%s: malformed forest accepted", f.name.c_str());
    CHECK(!err.empty(), "%s: no error message", f.name.c_str());
    CHECK(!build_fragments(g.parent.data(), g.start.data(), g.len.data(), n, 1 << 20, fr, err),
          "%s: fragments of a malformed forest", f.name.c_str());
    CHECK(!build_mamba_tables(g.parent.data(), g.start.data(), g.len.data(), n, m, err),
          "%s: Mamba tables of a malformed forest", f.name.c_str());
  }
  HostPlan p;
  std::string err;
  CHECK(!build_host_plan(nullptr, f.start.data(), f.len.data(), S, 0, -1, p, err), "null parent accepted");
  CHECK(!build_host_plan(f.parent.data(), f.start.data(), f.len.data(), 0, 0, -1, p, err), "S = 0 accepted");
  int32_t T = 0;
  for (int32_t n : f.len) T += n;
  CHECK(!build_host_plan(f.parent.data(), f.start.data(), f.len.data(), S, T, T + 1, p, err), "empty run accepted");
  CHECK(!build_host_plan(f.parent.data(), f.start.data(), f.len.data(), S, -1, T, p, err), "negative run accepted");
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 2) {
    std::fprintf(stderr, "usage: %s forests.txt\n", argv[0]);
    return 2;
  }
  std::ifstream in(argv[1]);
  std::string word;
  int n_forests = 0;
  while (in >> word) {
    CHECK(word == "forest", "bad input token %s", word.c_str());
    Forest f;
    int32_t S = 0;
    in >> f.name >> S;
    f.parent.resize(S);
    f.start.resize(S);
    f.len.resize(S);
    for (auto* v : {&f.parent, &f.start, &f.len})
      for (int32_t& x : *v) in >> x;
    CHECK(bool(in), "truncated input at %s", f.name.c_str());
    int32_t T = 0;
    for (int32_t n : f.len) T += n;
    check_attention_plan(f, 0, -1);
    if (T >= 4) {
      check_attention_plan(f, T / 4, T / 2 + 1);
      check_attention_plan(f, T - 1, T);
      check_attention_plan(f, 0, 1);
    }
    HostPlan p;
    std::string err;
    build_host_plan(f.parent.data(), f.start.data(), f.len.data(), S, 0, -1, p, err);
    for (int64_t bound : {p.max_path, p.max_path + 17, 2 * p.max_path + 5, int64_t(T), p.max_path - 1})
      if (bound >= 1 && bound < (int64_t(1) << 31)) check_fragments(f, int32_t(bound));
    check_mamba(f);
    check_edges(f, uint64_t(n_forests) + 1);
    check_rejections(f);
    ++n_forests;
  }
  std::printf("ALL OK: %d forests, %d checks\n", n_forests, g_checks);
  return 0;
}
