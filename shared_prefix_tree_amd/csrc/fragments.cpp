// Bounded fragment planning with ancestor repetition (host only); see
// fragments.hpp.
#include "fragments.hpp"

#include <algorithm>

#include "plan.hpp"

namespace tree_attn {

bool build_fragments(const int32_t* parent, const int32_t* seg_start, const int32_t* seg_len, int32_t S,
                     int32_t max_tokens, Fragments& f, std::string& err) {
  HostPlan p;  // validation (DFS pre-order, contiguity) and the path lengths
  if (!build_host_plan(parent, seg_start, seg_len, S, 0, -1, p, err)) return false;
  if (max_tokens < 1) {
    err = "max_tokens must be >= 1";
    return false;
  }
  if (p.max_path > max_tokens) {
    err = "a root-to-leaf path of " + std::to_string(p.max_path) + " tokens does not fit max_tokens = " +
          std::to_string(max_tokens);
    return false;
  }
  f = Fragments{};
  f.max_tokens = max_tokens;
  f.source_tokens = p.T;
  f.frag_seg_ptr.push_back(0);
  f.frag_token_ptr.push_back(0);

  // placed[s]: index of source segment s's piece in the current fragment
  // (valid when stamp[s] == the current fragment's number)
  std::vector<int32_t> placed(S, -1), stamp(S, -1);
  int32_t frag = 0;
  int64_t used = 0;  // tokens in the current fragment
  std::vector<int32_t> chain;

  // appends source tokens [lo, hi) of segment s as one fragment segment whose
  // first `copies` tokens are repeated (not owned)
  auto place = [&](int32_t s, int32_t lo, int32_t hi, int32_t copies) {
    const int32_t par = parent[s] >= 0 && stamp[parent[s]] == frag ? placed[parent[s]] : -1;
    f.seg_parent.push_back(par < 0 ? -1 : par - f.frag_seg_ptr.back());
    f.seg_len.push_back(hi - lo);
    for (int32_t o = lo; o < hi; ++o) {
      f.token_source.push_back(seg_start[s] + o);
      f.token_owner.push_back(o - lo >= copies ? 1 : 0);
    }
    placed[s] = int32_t(f.seg_parent.size()) - 1;
    stamp[s] = frag;
    used += hi - lo;
  };
  auto close = [&]() {
    f.frag_seg_ptr.push_back(int32_t(f.seg_parent.size()));
    f.frag_token_ptr.push_back(int32_t(f.token_source.size()));
    ++frag;
    used = 0;
  };

  for (int32_t s = 0; s < S; ++s) {
    int32_t done = 0;  // tokens of s owned so far
    while (done < seg_len[s]) {
      if (used == 0) {
        // a fresh fragment repeats the ancestor chain, root first
        chain.clear();
        for (int32_t a = parent[s]; a >= 0; a = parent[a]) chain.push_back(a);
        for (auto it = chain.rbegin(); it != chain.rend(); ++it) place(*it, 0, seg_len[*it], seg_len[*it]);
      }
      // the piece [0, hi) restarts with a copy of the part of s owned
      // elsewhere; after a split the whole rest fits (chain + s <= bound)
      const int32_t hi = int32_t(std::min<int64_t>(seg_len[s], max_tokens - used));
      place(s, 0, hi, done);
      done = hi;
      if (used == max_tokens) close();
    }
  }
  if (used > 0) close();
  return true;
}

}  // namespace tree_attn
