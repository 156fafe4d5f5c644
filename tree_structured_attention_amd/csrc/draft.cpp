// Host draft-tree builder: decoupled draft-target matching and prefix-tree
// batching ("HSD: Training-Free Acceleration for Document Parsing
// Vision-Language Models with Hierarchical Speculative Decoding" notes, key
// design 3 (a) and (b)).  Integer work on host arrays; no GPU.
//
// (a) The last `window` accepted tokens are matched at every position of
//     every draft; what follows a match is a candidate continuation.
// (b) The candidates are merged into a prefix tree whose nodes are the
//     distinct prefixes, linearised in creation order, so each node's parent
//     comes before it and the result feeds the verify plan directly.
#include <algorithm>
#include <climits>
#include <cstring>
#include <vector>

#include "ta_internal.h"

using namespace ta;

namespace {

// Trie with first-child / next-sibling links; node ids are creation order.
struct Trie {
  std::vector<int32_t> token, parent, first_child, next_sibling;
  int32_t root_first = -1;

  int32_t find(int32_t cur, int32_t t) const {
    for (int32_t c = cur < 0 ? root_first : first_child[cur]; c >= 0; c = next_sibling[c])
      if (token[c] == t) return c;
    return -1;
  }
  int32_t add(int32_t cur, int32_t t) {
    const int32_t id = int32_t(token.size());
    token.push_back(t);
    parent.push_back(cur);
    first_child.push_back(-1);
    next_sibling.push_back(-1);
    // append at the end of the sibling list so siblings stay in creation order
    int32_t* link = cur < 0 ? &root_first : &first_child[cur];
    while (*link >= 0) link = &next_sibling[*link];
    *link = id;
    return id;
  }
};

}  // namespace

extern "C" int tree_attn_draft_tree(const int32_t* accepted, int32_t n_accepted, const int32_t* drafts,
                                    const int32_t* draft_len, int32_t n_drafts, int32_t window,
                                    int32_t max_nodes, int32_t max_depth, int32_t* tokens, int32_t* parent,
                                    int32_t* n_nodes) try {
  if (!n_nodes) return fail(TA_ERR_INVALID_ARG, "draft_tree: n_nodes is NULL");
  if (n_accepted < 0 || n_drafts < 0) return fail(TA_ERR_INVALID_ARG, "draft_tree: negative count");
  if (window < 1) return fail(TA_ERR_INVALID_ARG, "draft_tree: window must be >= 1");
  if (max_nodes < 0 || max_depth < 0) return fail(TA_ERR_INVALID_ARG, "draft_tree: negative budget");
  if (n_accepted > 0 && !accepted) return fail(TA_ERR_INVALID_ARG, "draft_tree: accepted is NULL");
  if (n_drafts > 0 && !draft_len) return fail(TA_ERR_INVALID_ARG, "draft_tree: draft_len is NULL");
  if (max_nodes > 0 && (!tokens || !parent)) return fail(TA_ERR_INVALID_ARG, "draft_tree: output arrays are NULL");
  int64_t total = 0;
  for (int32_t d = 0; d < n_drafts; ++d) {
    if (draft_len[d] < 0) return fail(TA_ERR_INVALID_ARG, "draft_tree: negative draft length");
    total += draft_len[d];
  }
  if (total > 0 && !drafts) return fail(TA_ERR_INVALID_ARG, "draft_tree: drafts is NULL");

  Trie trie;
  bool full = false;
  if (n_accepted >= window) {
    const int32_t* w = accepted + (n_accepted - window);
    const int32_t depth_cap = max_depth > 0 ? max_depth : INT32_MAX;
    const int32_t* d = drafts;
    for (int32_t di = 0; di < n_drafts && !full; d += draft_len[di], ++di) {
      const int64_t len = draft_len[di];
      // a match at j leaves the continuation d[j + window, len); empty ones are dropped
      for (int64_t j = 0; j + window < len && !full; ++j) {
        if (std::memcmp(d + j, w, sizeof(int32_t) * size_t(window)) != 0) continue;
        const int64_t stop = std::min<int64_t>(len, j + window + int64_t(depth_cap));
        int32_t cur = -1;
        for (int64_t i = j + window; i < stop; ++i) {
          int32_t nxt = trie.find(cur, d[i]);
          if (nxt < 0) {
            if (int32_t(trie.token.size()) >= max_nodes) {
              full = true;  // the node budget ends insertion
              break;
            }
            nxt = trie.add(cur, d[i]);
          }
          cur = nxt;
        }
      }
    }
  }
  const size_t n = trie.token.size();
  if (n) {
    std::memcpy(tokens, trie.token.data(), n * sizeof(int32_t));
    std::memcpy(parent, trie.parent.data(), n * sizeof(int32_t));
  }
  *n_nodes = int32_t(n);
  return TA_OK;
} catch (...) {
  return ta::fail_exception("draft_tree");
}
