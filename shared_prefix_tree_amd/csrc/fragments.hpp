// Bounded fragment planning with ancestor repetition (host only).
//
// Issue "Shared-prefix training with context parallelism for exact agent
// trajectories" (section "Describe the solution you'd like"): fragments are
// size-bounded, and ancestor segments may be duplicated in several of them;
// its measured token counts (the issue's own numbers: 3,744,651 tree
// tokens, 3,919,929 after fragmentation) are this step's metric.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace tree_attn {

struct Fragments {
  int32_t max_tokens = 0;
  int64_t source_tokens = 0;
  std::vector<int32_t> frag_seg_ptr;    // [F + 1] into seg_parent / seg_len
  std::vector<int32_t> frag_token_ptr;  // [F + 1] into token_source / token_owner
  std::vector<int32_t> seg_parent;      // parent within the fragment (-1: root)
  std::vector<int32_t> seg_len;
  std::vector<int32_t> token_source;    // source token of each fragment token
  std::vector<int32_t> token_owner;     // 1: the fragment owns the token's loss; 0: a repeated copy
};

// Splits a DFS segment forest into fragments of at most max_tokens tokens.
// Each fragment is a DFS forest of its own in which every token sees exactly
// the tokens it sees in the source forest: a fragment that starts inside a
// tree first repeats the ancestor chain of its first segment, and a segment
// split at a fragment boundary restarts with a repeated copy of its already
// placed part (same segment).  Every source token is owned by exactly one
// fragment.  Fails (false, `err`) on a malformed forest or when a root-to-leaf
// path is longer than max_tokens.
bool build_fragments(const int32_t* parent, const int32_t* seg_start, const int32_t* seg_len, int32_t num_segments,
                     int32_t max_tokens, Fragments& out, std::string& err);

}  // namespace tree_attn
