// Mamba host tables: predecessors, convolution halo and successors, scan
// units of a DFS segment forest; see mamba_plan.hpp.
#include "mamba_plan.hpp"

#include <algorithm>

#include "plan.hpp"

namespace tree_attn {

bool build_mamba_tables(const int32_t* parent, const int32_t* seg_start, const int32_t* seg_len, int32_t S,
                        MambaTables& m, std::string& err) {
  HostPlan hp;  // validation of the DFS forest (same rules as the attention plan)
  if (!build_host_plan(parent, seg_start, seg_len, S, 0, -1, hp, err)) return false;
  const int32_t T = hp.T;
  m.T = T;
  m.S = S;
  m.max_depth = hp.max_depth;
  m.prev.resize(T);
  for (int32_t i = 0; i < T; ++i) m.prev[i] = i - 1;
  for (int32_t s = 0; s < S; ++s)
    m.prev[seg_start[s]] = parent[s] < 0 ? -1 : seg_start[parent[s]] + seg_len[parent[s]] - 1;
  m.halo.assign(size_t(T) * kConvHalo, -1);
  std::vector<int32_t> count(size_t(T) + 1, 0);
  for (int32_t i = 0; i < T; ++i) {
    int32_t j = i;
    for (int k = 1; k <= kConvHalo; ++k) {
      j = j < 0 ? -1 : m.prev[j];
      m.halo[size_t(i) * kConvHalo + k - 1] = j;
      if (j >= 0 && j != i - k) ++count[size_t(j) + 1];  // (successors k tokens ahead are read from the halo)
    }
  }
  for (int32_t t = 0; t < T; ++t) count[t + 1] += count[t];
  m.csucc_ptr = count;
  m.csucc.resize(count[T]);
  std::vector<int32_t> fill(count.begin(), count.end() - 1);
  // entries of a token in (k, i) order: for each k, successors ascending
  for (int k = 1; k <= kConvHalo; ++k)
    for (int32_t i = 0; i < T; ++i) {
      const int32_t j = m.halo[size_t(i) * kConvHalo + k - 1];
      if (j >= 0 && j != i - k) m.csucc[fill[j]++] = 4 * i + k;
    }
  // units
  std::vector<int32_t> last_unit(S, -1);
  for (int32_t s = 0; s < S; ++s) {
    for (int32_t off = 0; off < seg_len[s]; off += kMambaUnit) {
      const int32_t u = int32_t(m.unit_start.size());
      m.unit_start.push_back(seg_start[s] + off);
      m.unit_len.push_back(std::min(kMambaUnit, seg_len[s] - off));
      m.unit_pred.push_back(off > 0 ? u - 1 : parent[s] < 0 ? -1 : last_unit[parent[s]]);
      last_unit[s] = u;
    }
  }
  m.U = int32_t(m.unit_start.size());
  m.usucc_ptr.assign(size_t(m.U) + 1, 0);
  for (int32_t u = 0; u < m.U; ++u)
    if (m.unit_pred[u] >= 0) ++m.usucc_ptr[size_t(m.unit_pred[u]) + 1];
  for (int32_t u = 0; u < m.U; ++u) m.usucc_ptr[u + 1] += m.usucc_ptr[u];
  m.usucc.resize(m.usucc_ptr[m.U]);
  std::vector<int32_t> uf(m.usucc_ptr.begin(), m.usucc_ptr.end() - 1);
  for (int32_t u = 0; u < m.U; ++u)
    if (m.unit_pred[u] >= 0) m.usucc[uf[m.unit_pred[u]]++] = u;
  m.uchain.assign(m.U, 0);
  for (int32_t u = 0; u < m.U; ++u)
    m.uchain[u] = (m.usucc_ptr[u + 1] - m.usucc_ptr[u] == 1 && m.usucc[m.usucc_ptr[u]] == u + 1) ? 1 : 0;
  return true;
}

}  // namespace tree_attn
