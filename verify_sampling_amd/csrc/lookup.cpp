// vs_lookup_tree: prompt-lookup drafting of a token tree.
//
// "One RDNA4 verify pass has slack for about two dozen speculative tokens":
// prompt lookup proposes what followed earlier occurrences of the last
// n-gram of the context (the introduction); instead of only the most recent
// one, the top few matches, ranked by how often they recur, become branches
// of a token tree sharing their common prefixes, inside the ~24-token budget
// of one verify pass ("Spend the budget on a tree", "What I am building
// toward").  Host code: one backward scan of the context per window.

#include <algorithm>
#include <cstdint>
#include <vector>

#include "verify_sampling.h"

namespace {

struct Proposal {
  int start;   // continuation = ctx[start, start + len)
  int len;
  int count;   // matches proposing exactly this continuation
  int recent;  // the most recent of those matches
};

}  // namespace

extern "C" int vs_lookup_tree(const int32_t* ctx, int ctx_len, int n, int branches, int depth,
                              int max_nodes, int32_t* tokens, int32_t* parent) {
  if (!tokens || !parent || (ctx_len > 0 && !ctx)) return VS_ERR_NULL;
  if (ctx_len < 0 || n < 1 || branches < 1 || depth < 1 || max_nodes < 1 ||
      max_nodes > VS_MAX_DRAFTS)
    return VS_ERR_SHAPE;
  if (ctx_len < n + 1) return 0;

  // earlier occurrences of the last n tokens (the first token filters)
  const int32_t* q = ctx + (ctx_len - n);
  const int32_t q0 = q[0];
  std::vector<int> pos;
  for (int p = ctx_len - n - 1; p >= 0; --p)
    if (ctx[p] == q0 && std::equal(q + 1, q + n, ctx + p + 1)) pos.push_back(p);
  if (pos.empty()) return 0;

  // group identical continuations: sort by continuation, most recent first
  // within a group (positions are distinct)
  auto cont_len = [&](int p) { return std::min(depth, ctx_len - (p + n)); };
  std::sort(pos.begin(), pos.end(), [&](int a, int b) {
    const int la = cont_len(a), lb = cont_len(b);
    const int32_t* ca = ctx + a + n;
    const int32_t* cb = ctx + b + n;
    const int m = std::min(la, lb);
    for (int i = 0; i < m; ++i)
      if (ca[i] != cb[i]) return ca[i] < cb[i];
    if (la != lb) return la < lb;
    return a > b;
  });
  std::vector<Proposal> props;
  for (size_t i = 0; i < pos.size();) {
    const int p = pos[i];
    const int len = cont_len(p);
    size_t j = i + 1;
    while (j < pos.size() && cont_len(pos[j]) == len &&
           std::equal(ctx + p + n, ctx + p + n + len, ctx + pos[j] + n))
      ++j;
    props.push_back({p + n, len, static_cast<int>(j - i), p});
    i = j;
  }
  // most recurrent first, then the most recent
  const int keep = std::min(branches, static_cast<int>(props.size()));
  std::partial_sort(props.begin(), props.begin() + keep, props.end(),
                    [](const Proposal& a, const Proposal& b) {
                      return a.count != b.count ? a.count > b.count : a.recent > b.recent;
                    });

  int nodes = 0;
  for (int b = 0; b < keep; ++b) {
    const Proposal& pr = props[b];
    int node = -1;
    for (int i = 0; i < pr.len; ++i) {
      const int32_t t = ctx[pr.start + i];
      int child = -1;
      for (int j = 0; j < nodes; ++j)
        if (parent[j] == node && tokens[j] == t) {
          child = j;
          break;
        }
      if (child < 0) {
        if (nodes == max_nodes) return nodes;
        tokens[nodes] = t;
        parent[nodes] = node;
        child = nodes++;
      }
      node = child;
    }
  }
  return nodes;
}
