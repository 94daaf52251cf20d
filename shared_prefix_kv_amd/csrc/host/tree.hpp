// Host-side KV page pool, resident token-prefix (radix) tree and staged-round
// planner.
//
// Reuse is keyed on the exact token prefix (LLM2Jev shared-prefix page, Radix
// Cache section); candidates that share a prefix are grouped into a tree and
// submitted in rounds so that a shared prefix exists before the candidates that
// reuse it (same page, staged-submission section).  Page size 16 tokens.
//
// Rules (the pages leave them open):
//  * page allocation: lowest free ids first; every node starts on a fresh page;
//  * the candidate tree is a compressed, token-granular trie below each
//    candidate's resident match; a node with children, where no candidate
//    ends, and shorter than one page is dissolved top-down into its children;
//  * round k computes the nodes at depth k; canonical node order is
//    (depth, smallest candidate index through the node);
//  * childless nodes release their pages when their round ends, the plan's
//    other nodes when the call ends.
#pragma once

#include <cstdint>
#include <map>
#include <set>
#include <string>
#include <unordered_map>
#include <vector>

namespace jev {

constexpr int kPage = 16;

inline int32_t pages_for(int64_t n_tokens) { return int32_t((n_tokens + kPage - 1) / kPage); }

class PagePool {
 public:
  explicit PagePool(int32_t n = 0) { reset(n); }
  void reset(int32_t n) {
    n_total_ = n;
    free_.clear();
    for (int32_t i = 0; i < n; ++i) free_.insert(free_.end(), i);
  }
  int32_t n_free() const { return int32_t(free_.size()); }
  int32_t n_total() const { return n_total_; }
  // Takes the n lowest free ids (ascending).  Caller checks n_free() first.
  std::vector<int32_t> alloc(int32_t n) {
    std::vector<int32_t> out;
    out.reserve(n);
    for (int32_t i = 0; i < n; ++i) {
      auto it = free_.begin();
      out.push_back(*it);
      free_.erase(it);
    }
    return out;
  }
  void release(const std::vector<int32_t>& pages) {
    for (int32_t p : pages) free_.insert(p);
  }
  // Marks the given ids as used; false (and no change) if one is not free.
  bool take(const std::vector<int32_t>& pages) {
    for (int32_t p : pages)
      if (!free_.count(p)) return false;
    for (int32_t p : pages) free_.erase(p);
    return true;
  }
  std::set<int32_t> snapshot() const { return free_; }
  void restore(std::set<int32_t> s) { free_ = std::move(s); }

 private:
  int32_t n_total_ = 0;
  std::set<int32_t> free_;
};

struct ResNode {
  int64_t handle = 0;
  int64_t parent = 0;  // 0 = empty root
  std::vector<int32_t> tokens;
  std::vector<int32_t> pages;
  int64_t start = 0;   // logical position of tokens[0]
  int64_t refs = 1;
  uint64_t last_use = 0;           // stamp of the last call that used the node
  std::vector<int64_t> children;  // creation order
};

// One (page, valid token count) entry of a key list.
struct PageRef {
  int32_t page;
  int32_t valid;
};

// Cache policy of unreferenced prefixes (openjev-multimodal performance page,
// repeated-state section: a state's KV is kept for the next request, and
// several states can be kept and used in turn).  With keep() set, a prefix
// whose last caller reference is dropped stays resident as a cached prefix; a
// call that is short of pages evicts cached prefixes that have no children,
// least recently used first (ties: the smallest handle), never one on the
// path of a prefix the call uses.  A node's last use is the stamp of the last
// call that created, re-referenced, scored under or released a prefix whose
// path contains it.
class ResidentTree {
 public:
  explicit ResidentTree(PagePool* pool) : pool_(pool) {}
  // Points a copy of the tree at a copy of its pool (for dry runs).
  void rebind(PagePool* pool) { pool_ = pool; }

  bool has(int64_t h) const { return h == 0 || nodes_.count(h) != 0; }
  const ResNode& node(int64_t h) const { return nodes_.at(h); }
  int64_t end_pos(int64_t h) const;
  int32_t size() const { return int32_t(nodes_.size()); }
  // Pages of the path root..h (root first).
  std::vector<PageRef> path_pages(int64_t h) const;

  struct PrefillItem {
    int64_t parent;
    const int32_t* tok;
    int64_t n;
  };
  // Number of new pages the items need (in-call duplicates counted once).
  int64_t prefill_need(const std::vector<PrefillItem>& items) const;
  // Creates or re-references one node per item; out[i] = handle, created[i] =
  // whether it is new.  Caller has checked prefill_need() against the pool.
  void prefill(const std::vector<PrefillItem>& items, std::vector<int64_t>* out,
               std::vector<char>* created);
  // A new node continuing `parent` with tokens tok[0..n) whose K/V are
  // already in `pages` (free ids, taken from the pool here); one reference.
  // Returns its handle, or 0 if a page is not free.
  int64_t adopt(int64_t parent, const int32_t* tok, int64_t n, const std::vector<int32_t>& pages);
  // Drops one reference; without keep(), frees nodes with no reference and no child.
  void release(int64_t h);
  void set_keep(bool keep) { keep_ = keep; }
  bool keep() const { return keep_; }
  // Marks every node on the root..h path as used at `stamp`.
  void touch_path(int64_t h, uint64_t stamp);
  // Evicts the least recently used cached node without children that is not
  // in `pinned`; returns its handle, or 0 if there is none.
  int64_t evict_one(const std::set<int64_t>& pinned);
  // Evicts node h (a cached node without children).
  void evict(int64_t h);
  int64_t evictions() const { return evictions_; }
  int32_t cached_count() const;
  int32_t cached_pages() const;
  int32_t pages_held() const;
  // The child of `parent` whose segment is exactly tok[0..n), or 0.
  int64_t find_child(int64_t parent, const int32_t* tok, int64_t n) const;
  // Splits node h after its first `at` tokens (a multiple of the page size,
  // inside the node): a new node takes h's place under its parent with the
  // first at / 16 pages and no reference; h keeps its handle, references and
  // children with the rest and becomes the new node's child.  Returns the new
  // handle.
  int64_t split(int64_t h, int64_t at);
  // Anchor of a candidate with reuse inside resident nodes: full-node matches
  // as in match(); where none continues, the child sharing the longest
  // page-aligned run (at least one page, leaving >= 1 token; ties: the
  // earliest created) is split at that page boundary and its first part is
  // the anchor.
  void match_split(const int32_t* seq, int64_t n, int64_t* handle, int64_t* matched);
  // Deepest full-node match leaving >= 1 token.
  void match(const int32_t* seq, int64_t n, int64_t* handle, int64_t* matched) const;

 private:
  const std::vector<int64_t>& children(int64_t parent) const {
    return parent == 0 ? root_children_ : nodes_.at(parent).children;
  }
  std::vector<int64_t>& children_mut(int64_t parent) {
    return parent == 0 ? root_children_ : nodes_.at(parent).children;
  }

  PagePool* pool_;
  std::map<int64_t, ResNode> nodes_;
  std::vector<int64_t> root_children_;
  int64_t next_handle_ = 1;
  bool keep_ = false;
  int64_t evictions_ = 0;
};

struct PlanNode {
  std::vector<int32_t> cands;  // sorted candidate indices through the node
  int64_t a = 0, b = 0;        // segment [a, b) relative to the anchor
  int64_t anchor = 0;          // resident handle the subtree continues
  std::vector<int32_t> readout;
  std::vector<int32_t> children;  // indices into Plan::nodes
  int32_t parent = -1;            // index into Plan::nodes, -1 = anchor
  int32_t depth = 0;
  int32_t id = -1;
  std::vector<int32_t> pages;
  int32_t cand_min() const { return cands[0]; }
};

struct Plan {
  std::vector<PlanNode> nodes;                 // storage (index != id)
  std::vector<std::vector<int32_t>> rounds;    // per round: node storage indices, canonical order
  std::vector<int64_t> anchors;                // per candidate
  std::vector<int64_t> anchor_len;             // per candidate
  std::vector<int32_t> readout_node;           // per candidate: node id
  std::vector<int32_t> id_to_index;            // node id -> storage index
  std::vector<int32_t> serialize() const;
};

// Builds the plan of n candidates (seq i = tok[off[i]..off[i+1])) and assigns
// pages, replaying the rounds on the pool (allocate a round's nodes, release its
// childless nodes, release the rest after the last round).  Returns false (pool
// untouched) if the pool cannot hold the plan.  Either way the pool ends as it
// started: the plan's pages live only for the call, and device work of a later
// call that re-uses them is stream-ordered after this call's.
// Round orders of a candidate plan.  DEPTH: round k computes the nodes at
// tree depth k.  CANDIDATE_FIRST (LLM2Jev shared-prefix page,
// staged-submission section: a real candidate is scored first to build the
// shared prefix, then the candidates that reuse it are submitted; deeper forks
// take further rounds and independent branches share one): each round takes
// every node whose parent is computed; a node without children is computed
// with all its candidates, while a node with children is computed by one
// builder, its smallest candidate, whose whole remaining path down to its own
// read-out node is computed in that round too.  Within a round nodes are in
// (tree depth, smallest candidate) order.
enum class PlanMode { DEPTH = 0, CANDIDATE_FIRST = 1 };

bool plan_candidates(const ResidentTree& tree, PagePool* pool, int32_t n, const int32_t* tok,
                     const int64_t* off, Plan* plan, PlanMode mode = PlanMode::DEPTH);

}  // namespace jev
