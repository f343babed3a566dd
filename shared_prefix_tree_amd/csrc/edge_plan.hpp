// Host tables of the sampled-edge loss (plain C++, no device code): the
// edges grouped by source token, so a token's hidden-state gradient is a sum
// over its own edges in a fixed order.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace tree_attn {

// Checks 0 <= src[e] < num_tokens and 0 <= tgt[e] < vocab for every edge and
// builds the CSR by source: row_ptr [num_tokens + 1], ids [num_edges] (edge
// indices, ascending within a token).  Returns false and sets `err` on a bad
// edge or size.
bool build_edge_csr(const int32_t* edge_src, const int32_t* edge_tgt, int32_t num_edges, int32_t num_tokens,
                    int32_t vocab, std::vector<int32_t>& row_ptr, std::vector<int32_t>& ids, std::string& err);

}  // namespace tree_attn
