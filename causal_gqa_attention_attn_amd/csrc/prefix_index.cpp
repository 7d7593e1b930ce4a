// Host-side prefix index over token ids: which recorded request holds the
// longest reusable prefix of a new request (page "KV Cache 与 Prefill/Decode
// 推理路径", prefix-sharing lesson: reuse needs an exact token-id prefix match;
// two requests that first differ at index m share positions 0..m-1; a prefix
// tree over the requests answers which prefix is reusable and the block table
// where it lives, which kv_cache_fork then shares).
//
// A radix tree: every node holds an edge label (a run of token ids) and the
// ids of the recorded requests whose token sequence runs through the node.
// A match walks the tree as far as the query agrees with it, possibly ending
// inside an edge, and returns the smallest request id below that point.
#include <algorithm>
#include <map>
#include <set>
#include <vector>

#include "gqa.h"

#define GQA_EXPORT extern "C" __attribute__((visibility("default")))

struct gqa_prefix_index {
  struct Node {
    std::vector<int32_t> label;           // token ids on the edge into this node
    std::map<int32_t, int32_t> child;     // first token of a child's label -> node
    std::set<int32_t> seqs;               // recorded requests whose path passes through this node
    int32_t parent = -1;
  };
  std::vector<Node> nodes;                // nodes[0] is the root (empty label)
  std::vector<int32_t> free_nodes;
  std::map<int32_t, std::vector<int32_t>> recorded;   // request id -> its token ids

  gqa_prefix_index() { nodes.emplace_back(); }

  int32_t new_node() {
    if (!free_nodes.empty()) {
      const int32_t i = free_nodes.back();
      free_nodes.pop_back();
      nodes[i] = Node();
      return i;
    }
    nodes.emplace_back();
    return static_cast<int32_t>(nodes.size() - 1);
  }

  // Split node v's edge after k tokens: a new node takes the first k tokens
  // and becomes v's parent.
  int32_t split(int32_t v, size_t k) {
    const int32_t u = new_node();
    Node& nv = nodes[v];
    const int32_t p = nv.parent;
    nodes[u].label.assign(nv.label.begin(), nv.label.begin() + k);
    nodes[u].seqs = nv.seqs;
    nodes[u].parent = p;
    nodes[u].child[nv.label[k]] = v;
    nodes[p].child[nodes[u].label[0]] = u;
    nv.label.erase(nv.label.begin(), nv.label.begin() + k);
    nv.parent = u;
    return u;
  }

  void insert(int32_t seq, const std::vector<int32_t>& t) {
    int32_t v = 0;
    size_t i = 0;
    nodes[0].seqs.insert(seq);
    while (i < t.size()) {
      auto it = nodes[v].child.find(t[i]);
      if (it == nodes[v].child.end()) {
        const int32_t w = new_node();
        nodes[w].label.assign(t.begin() + i, t.end());
        nodes[w].parent = v;
        nodes[w].seqs.insert(seq);
        nodes[v].child[t[i]] = w;
        return;
      }
      int32_t w = it->second;
      const std::vector<int32_t>& lab = nodes[w].label;
      size_t k = 0;
      while (k < lab.size() && i + k < t.size() && lab[k] == t[i + k]) ++k;
      if (k < lab.size()) w = split(w, k);
      nodes[w].seqs.insert(seq);
      i += k;
      v = w;
    }
  }

  void remove(int32_t seq, const std::vector<int32_t>& t) {
    int32_t v = 0;
    size_t i = 0;
    nodes[0].seqs.erase(seq);
    std::vector<int32_t> path;
    while (i < t.size()) {
      const int32_t w = nodes[v].child.at(t[i]);
      nodes[w].seqs.erase(seq);
      path.push_back(w);
      i += nodes[w].label.size();
      v = w;
    }
    // drop nodes no recorded request passes through any more (deepest first)
    for (auto it = path.rbegin(); it != path.rend(); ++it) {
      const int32_t w = *it;
      if (!nodes[w].seqs.empty()) continue;
      nodes[nodes[w].parent].child.erase(nodes[w].label[0]);
      free_nodes.push_back(w);
    }
  }

  void match(const int32_t* t, int32_t n, int32_t* seq_out, int32_t* m_out) const {
    int32_t v = 0, below = 0;             // `below`: node whose requests share the matched run
    int32_t i = 0;
    while (i < n) {
      auto it = nodes[v].child.find(t[i]);
      if (it == nodes[v].child.end()) break;
      const int32_t w = it->second;
      const std::vector<int32_t>& lab = nodes[w].label;
      int32_t k = 0;
      while (k < static_cast<int32_t>(lab.size()) && i + k < n && lab[k] == t[i + k]) ++k;
      i += k;
      below = w;
      if (k < static_cast<int32_t>(lab.size())) break;
      v = w;
    }
    *m_out = i;
    *seq_out = i > 0 ? *nodes[below].seqs.begin() : -1;
  }
};

namespace gqa {
void set_last_error(const char* msg);
}

namespace {
gqa_status prefix_fail(gqa_status s, const char* msg) {
  gqa::set_last_error(msg);
  return s;
}
}  // namespace

GQA_EXPORT gqa_status gqa_prefix_index_create(gqa_prefix_index** out) {
  if (!out) return prefix_fail(GQA_ERR_ARG, "out is null");
  *out = new gqa_prefix_index();
  return GQA_OK;
}

GQA_EXPORT gqa_status gqa_prefix_index_destroy(gqa_prefix_index* ix) {
  delete ix;
  return GQA_OK;
}

GQA_EXPORT gqa_status gqa_prefix_index_insert(gqa_prefix_index* ix, int32_t seq, const int32_t* tokens, int32_t n) {
  if (!ix || seq < 0 || n < 0 || (n > 0 && !tokens)) return prefix_fail(GQA_ERR_ARG, "bad prefix-index insert");
  auto it = ix->recorded.find(seq);
  if (it != ix->recorded.end()) {
    ix->remove(seq, it->second);
    ix->recorded.erase(it);
  }
  std::vector<int32_t> t(tokens, tokens + n);
  ix->insert(seq, t);
  ix->recorded.emplace(seq, std::move(t));
  return GQA_OK;
}

GQA_EXPORT gqa_status gqa_prefix_index_remove(gqa_prefix_index* ix, int32_t seq) {
  if (!ix) return prefix_fail(GQA_ERR_ARG, "index is null");
  auto it = ix->recorded.find(seq);
  if (it == ix->recorded.end()) return GQA_OK;
  ix->remove(seq, it->second);
  ix->recorded.erase(it);
  return GQA_OK;
}

GQA_EXPORT gqa_status gqa_prefix_index_match(const gqa_prefix_index* ix, const int32_t* tokens, int32_t n,
                                             int32_t* seq_out, int32_t* m_out) {
  if (!ix || !seq_out || !m_out || n < 0 || (n > 0 && !tokens))
    return prefix_fail(GQA_ERR_ARG, "bad prefix-index match");
  ix->match(tokens, n, seq_out, m_out);
  return GQA_OK;
}
