// Host-side plan of a DFS-linearized segment forest, and the records the
// kernels read from device memory.
//
// The plan turns the packed-sequence metadata (segment starts and lengths,
// parent links; Megatron-LM issue "Shared-prefix training with context
// parallelism for exact agent trajectories", section "Describe the solution
// you'd like") into the lists the kernels walk:
//   * per segment, its ancestor path as merged physical key spans, root
//     first, then the segment itself; span i covers virtual positions
//     [virt, virt + len) of the segment's reconstructed root-to-leaf
//     sequence, so the own-segment causal rule becomes "virtual key
//     position <= query position";
//   * query tiles (32/64/128/256/96 tokens, never crossing a segment) with the
//     position of their first token in that sequence;
//   * key tiles (64 tokens, never crossing a segment) with the end of the
//     contiguous range of queries that see them.  In a DFS pre-order every
//     subtree is a contiguous token range, so the queries that see key j
//     are exactly [j, subtree_end(seg(j))).
// Tile lists are sorted longest-first so the biggest work items start first.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace tree_attn {

struct QTile {
  int32_t q0;    // first query token
  int32_t nq;    // tokens in the tile (<= tile size)
  int32_t seg;   // segment of every token in the tile
  int32_t pos0;  // position of q0 in its reconstructed sequence
  // the segment's first span (its index in the span list, then a copy of
  // phys, len, virt), so a walk starts from this one record
  int32_t span0;
  int32_t phys0, len0, virt0;
};
static_assert(sizeof(QTile) == 32, "one 32-byte record per query tile");

struct KTile {
  int32_t k0;    // first key token
  int32_t nk;    // tokens in the tile (<= 64)
  int32_t seg;   // segment of every key in the tile
  int32_t qend;  // queries that see the tile: [k0, qend)
  int32_t send;  // one past the segment's last token: [send, qend) are its descendants
  int32_t pad[3];
};
static_assert(sizeof(KTile) == 32, "one 32-byte record per key tile");

struct Span {
  int32_t phys;  // first physical token
  int32_t len;   // tokens
  int32_t virt;  // virtual position of `phys` in the segment's sequence
  int32_t pad;
};

constexpr int kNumQTileSizes = 5;
constexpr int kQTileSizes[kNumQTileSizes] = {32, 64, 128, 256, 96};
constexpr int kKTile = 64;       // key tiles of the fp32 dK/dV pass
constexpr int kKTileWide = 128;  // key tiles of the bf16 dK/dV pass

inline int qtile_index(int tq) {
  return tq == 32 ? 0 : tq == 64 ? 1 : tq == 128 ? 2 : tq == 256 ? 3 : tq == 96 ? 4 : -1;
}

struct HostPlan {
  int32_t T = 0, S = 0, num_roots = 0, max_depth = 0, max_spans = 0;
  int32_t q_begin = 0, q_end = 0;  // the query run: tokens whose attention is computed
  int64_t max_path = 0, pairs = 0;
  std::vector<int32_t> parent, start, len, depth, prefix, end;
  std::vector<int32_t> span_ptr;
  std::vector<Span> spans;
  std::vector<QTile> qtiles[kNumQTileSizes];
  std::vector<KTile> ktiles;       // kKTile keys
  std::vector<KTile> ktiles_wide;  // kKTileWide keys
};

// Validates the topology and fills `plan`; on failure returns false and
// sets `err`.
// A query run [q_begin, q_end) restricts the queries (q_end < 0: to the
// last token); the keys are always every token.
bool build_host_plan(const int32_t* parent, const int32_t* seg_start, const int32_t* seg_len,
                     int32_t num_segments, int32_t q_begin, int32_t q_end, HostPlan& plan, std::string& err);

}  // namespace tree_attn
