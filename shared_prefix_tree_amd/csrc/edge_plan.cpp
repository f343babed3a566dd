// Sampled-edge CSR by source token; see edge_plan.hpp.
#include "edge_plan.hpp"

namespace tree_attn {

bool build_edge_csr(const int32_t* edge_src, const int32_t* edge_tgt, int32_t num_edges, int32_t num_tokens,
                    int32_t vocab, std::vector<int32_t>& row_ptr, std::vector<int32_t>& ids, std::string& err) {
  if (num_edges < 1 || num_tokens < 1 || vocab < 1 || !edge_src || !edge_tgt) {
    err = "need >= 1 edge, token and vocabulary row";
    return false;
  }
  for (int32_t e = 0; e < num_edges; ++e) {
    if (edge_src[e] < 0 || edge_src[e] >= num_tokens || edge_tgt[e] < 0 || edge_tgt[e] >= vocab) {
      err = "edge " + std::to_string(e) + " has source " + std::to_string(edge_src[e]) + " / sampled token " +
            std::to_string(edge_tgt[e]) + " outside [0, " + std::to_string(num_tokens) + ") / [0, " +
            std::to_string(vocab) + ")";
      return false;
    }
  }
  row_ptr.assign(size_t(num_tokens) + 1, 0);
  ids.assign(size_t(num_edges), 0);
  for (int32_t e = 0; e < num_edges; ++e) ++row_ptr[size_t(edge_src[e]) + 1];
  for (int32_t t = 0; t < num_tokens; ++t) row_ptr[size_t(t) + 1] += row_ptr[t];
  std::vector<int32_t> fill(row_ptr.begin(), row_ptr.end() - 1);
  for (int32_t e = 0; e < num_edges; ++e) ids[size_t(fill[edge_src[e]]++)] = e;
  return true;
}

}  // namespace tree_attn
