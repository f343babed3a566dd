// Host tables of the Mamba state-forking path (plain C++, no device code).
//
// Every token continues the sequence of its ancestor path: prev(i) is the
// token before i in its segment, or for a segment's first token the last
// token of the parent segment (-1 at a root); the draft "feat(hybrid): add
// opt-in shared-prefix attention and Mamba execution" (intro) forks the
// recurrent state and the convolution halo at exactly these branch points.
// The tables below are what the convolution and scan kernels walk.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace tree_attn {

constexpr int kMambaUnit = 128;     // tokens per scan unit
constexpr int kConvMaxWidth = 4;    // convolution widths 1..4
constexpr int kConvHalo = kConvMaxWidth - 1;

struct MambaTables {
  int32_t T = 0, S = 0, U = 0, max_depth = 0;
  std::vector<int32_t> prev;                    // [T]
  std::vector<int32_t> halo;                    // [T][kConvHalo]: prev^1 .. prev^kConvHalo (-1: none)
  std::vector<int32_t> csucc_ptr, csucc;        // token j -> entries 4 i + k with prev^k(i) = j, i != j + k
  std::vector<int32_t> unit_start, unit_len, unit_pred;  // [U]
  std::vector<int32_t> usucc_ptr, usucc;        // unit u -> units v with pred(v) = u, ascending
  std::vector<int32_t> uchain;                  // 1: u's only successor is u + 1
};

// Validates the forest (the rules of the attention plan) and fills `m`;
// on failure returns false and sets `err`.
bool build_mamba_tables(const int32_t* parent, const int32_t* seg_start, const int32_t* seg_len, int32_t S,
                        MambaTables& m, std::string& err);

}  // namespace tree_attn
