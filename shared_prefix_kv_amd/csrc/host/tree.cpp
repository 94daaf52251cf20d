// Resident prefix tree and staged-round planner (rules in tree.hpp).
#include "tree.hpp"

#include <algorithm>
#include <deque>

namespace jev {

int64_t ResidentTree::end_pos(int64_t h) const {
  if (h == 0) return 0;
  const ResNode& n = nodes_.at(h);
  return n.start + int64_t(n.tokens.size());
}

std::vector<PageRef> ResidentTree::path_pages(int64_t h) const {
  std::vector<const ResNode*> chain;
  while (h != 0) {
    const ResNode& n = nodes_.at(h);
    chain.push_back(&n);
    h = n.parent;
  }
  std::vector<PageRef> out;
  for (auto it = chain.rbegin(); it != chain.rend(); ++it) {
    const ResNode& n = **it;
    int64_t L = int64_t(n.tokens.size());
    for (size_t i = 0; i < n.pages.size(); ++i) {
      int64_t v = L - int64_t(kPage) * int64_t(i);
      out.push_back({n.pages[i], int32_t(v < kPage ? v : kPage)});
    }
  }
  return out;
}

int64_t ResidentTree::find_child(int64_t parent, const int32_t* tok, int64_t n) const {
  for (int64_t c : children(parent)) {
    const ResNode& cn = nodes_.at(c);
    if (int64_t(cn.tokens.size()) == n && std::equal(cn.tokens.begin(), cn.tokens.end(), tok))
      return c;
  }
  return 0;
}

int64_t ResidentTree::prefill_need(const std::vector<PrefillItem>& items) const {
  int64_t need = 0;
  for (size_t i = 0; i < items.size(); ++i) {
    const PrefillItem& it = items[i];
    if (find_child(it.parent, it.tok, it.n) != 0) continue;
    bool dup = false;
    for (size_t j = 0; j < i && !dup; ++j) {
      const PrefillItem& o = items[j];
      dup = o.parent == it.parent && o.n == it.n && std::equal(o.tok, o.tok + o.n, it.tok);
    }
    if (!dup) need += pages_for(it.n);
  }
  return need;
}

void ResidentTree::prefill(const std::vector<PrefillItem>& items, std::vector<int64_t>* out,
                           std::vector<char>* created) {
  out->clear();
  created->clear();
  for (const PrefillItem& it : items) {
    int64_t h = find_child(it.parent, it.tok, it.n);
    if (h != 0) {
      nodes_.at(h).refs += 1;
      out->push_back(h);
      created->push_back(0);
      continue;
    }
    h = next_handle_++;
    ResNode n;
    n.handle = h;
    n.parent = it.parent;
    n.tokens.assign(it.tok, it.tok + it.n);
    n.pages = pool_->alloc(pages_for(it.n));
    n.start = end_pos(it.parent);
    nodes_.emplace(h, std::move(n));
    children_mut(it.parent).push_back(h);
    out->push_back(h);
    created->push_back(1);
  }
}

int64_t ResidentTree::adopt(int64_t parent, const int32_t* tok, int64_t n, const std::vector<int32_t>& pages) {
  if (!pool_->take(pages)) return 0;
  const int64_t h = next_handle_++;
  ResNode nd;
  nd.handle = h;
  nd.parent = parent;
  nd.tokens.assign(tok, tok + n);
  nd.pages = pages;
  nd.start = end_pos(parent);
  nodes_.emplace(h, std::move(nd));
  children_mut(parent).push_back(h);
  return h;
}

void ResidentTree::release(int64_t h) {
  ResNode* n = &nodes_.at(h);
  n->refs -= 1;
  if (keep_) return;
  while (n != nullptr && n->refs == 0 && n->children.empty()) {
    pool_->release(n->pages);
    int64_t parent = n->parent;
    auto& sib = children_mut(parent);
    sib.erase(std::find(sib.begin(), sib.end(), n->handle));
    nodes_.erase(n->handle);
    n = parent == 0 ? nullptr : &nodes_.at(parent);
  }
}

int64_t ResidentTree::split(int64_t h, int64_t at) {
  ResNode& tail = nodes_.at(h);
  const int64_t nh = next_handle_++;
  ResNode head;
  head.handle = nh;
  head.parent = tail.parent;
  head.tokens.assign(tail.tokens.begin(), tail.tokens.begin() + at);
  head.pages.assign(tail.pages.begin(), tail.pages.begin() + at / kPage);
  head.start = tail.start;
  head.refs = 0;
  head.last_use = tail.last_use;
  head.children.push_back(h);
  auto& sib = children_mut(tail.parent);
  *std::find(sib.begin(), sib.end(), h) = nh;
  tail.parent = nh;
  tail.tokens.erase(tail.tokens.begin(), tail.tokens.begin() + at);
  tail.pages.erase(tail.pages.begin(), tail.pages.begin() + at / kPage);
  tail.start += at;
  nodes_.emplace(nh, std::move(head));
  return nh;
}

void ResidentTree::match_split(const int32_t* seq, int64_t n, int64_t* handle, int64_t* matched) {
  int64_t h, pos;
  match(seq, n, &h, &pos);
  int64_t best = 0, best_at = 0;
  for (int64_t c : children(h)) {
    const std::vector<int32_t>& t = nodes_.at(c).tokens;
    const int64_t lim = std::min<int64_t>(int64_t(t.size()), n - 1 - pos);
    int64_t l = 0;
    while (l < lim && t[size_t(l)] == seq[pos + l]) ++l;
    const int64_t at = l / kPage * kPage;
    if (at >= kPage && at < int64_t(t.size()) && at > best_at) {
      best = c;
      best_at = at;
    }
  }
  if (best != 0) {
    h = split(best, best_at);
    pos += best_at;
  }
  *handle = h;
  *matched = pos;
}

void ResidentTree::touch_path(int64_t h, uint64_t stamp) {
  for (; h != 0; h = nodes_.at(h).parent) nodes_.at(h).last_use = stamp;
}

int64_t ResidentTree::evict_one(const std::set<int64_t>& pinned) {
  int64_t best = 0;
  uint64_t best_use = 0;
  for (const auto& kv : nodes_) {  // ascending handles: the first of equal stamps wins
    const ResNode& n = kv.second;
    if (n.refs != 0 || !n.children.empty() || pinned.count(n.handle)) continue;
    if (best == 0 || n.last_use < best_use) {
      best = n.handle;
      best_use = n.last_use;
    }
  }
  if (best != 0) evict(best);
  return best;
}

void ResidentTree::evict(int64_t h) {
  ResNode& n = nodes_.at(h);
  pool_->release(n.pages);
  auto& sib = children_mut(n.parent);
  sib.erase(std::find(sib.begin(), sib.end(), h));
  nodes_.erase(h);
  evictions_ += 1;
}

int32_t ResidentTree::cached_count() const {
  int32_t k = 0;
  for (const auto& kv : nodes_) k += kv.second.refs == 0;
  return k;
}

int32_t ResidentTree::cached_pages() const {
  int32_t k = 0;
  for (const auto& kv : nodes_)
    if (kv.second.refs == 0) k += int32_t(kv.second.pages.size());
  return k;
}

int32_t ResidentTree::pages_held() const {
  int32_t k = 0;
  for (const auto& kv : nodes_) k += int32_t(kv.second.pages.size());
  return k;
}

void ResidentTree::match(const int32_t* seq, int64_t n, int64_t* handle, int64_t* matched) const {
  int64_t h = 0, pos = 0;
  for (;;) {
    int64_t best = 0;
    size_t best_len = 0;
    for (int64_t c : children(h)) {
      const std::vector<int32_t>& t = nodes_.at(c).tokens;
      if (pos + int64_t(t.size()) < n && std::equal(t.begin(), t.end(), seq + pos)) {
        if (best == 0 || t.size() > best_len) {
          best = c;
          best_len = t.size();
        }
      }
    }
    if (best == 0) break;
    h = best;
    pos += int64_t(best_len);
  }
  *handle = h;
  *matched = pos;
}

// ---------------------------------------------------------------- planner

namespace {

struct Builder {
  Plan* plan;
  const std::vector<const int32_t*>& rel;
  const std::vector<int64_t>& len;

  // Children of a node whose candidates share tokens [0, a); returns storage indices.
  std::vector<int32_t> build(const std::vector<int32_t>& cands, int64_t a, int64_t anchor) {
    std::vector<int32_t> order_tok;
    std::vector<std::vector<int32_t>> groups;
    for (int32_t c : cands) {
      if (len[c] == a) continue;
      int32_t t = rel[c][a];
      size_t g = 0;
      while (g < order_tok.size() && order_tok[g] != t) ++g;
      if (g == order_tok.size()) {
        order_tok.push_back(t);
        groups.emplace_back();
      }
      groups[g].push_back(c);
    }
    std::vector<int32_t> out;
    for (auto& part : groups) {
      int64_t b = a + 1;
      for (;;) {
        bool ok = true;
        for (int32_t c : part) {
          if (len[c] <= b || rel[c][b] != rel[part[0]][b]) {
            ok = false;
            break;
          }
        }
        if (!ok) break;
        ++b;
      }
      PlanNode node;
      node.cands = part;
      node.a = a;
      node.b = b;
      node.anchor = anchor;
      std::vector<int32_t> deeper;
      for (int32_t c : part) {
        if (len[c] == b)
          node.readout.push_back(c);
        else
          deeper.push_back(c);
      }
      int32_t idx = int32_t(plan->nodes.size());
      plan->nodes.push_back(std::move(node));
      std::vector<int32_t> ch = build(deeper, b, anchor);
      plan->nodes[idx].children = std::move(ch);
      out.push_back(idx);
    }
    return out;
  }

  std::vector<int32_t> dissolve(const std::vector<int32_t>& list) {
    std::vector<int32_t> out;
    std::deque<int32_t> queue(list.begin(), list.end());
    while (!queue.empty()) {
      int32_t i = queue.front();
      queue.pop_front();
      PlanNode& n = plan->nodes[i];
      if (!n.children.empty() && n.readout.empty() && (n.b - n.a) < kPage) {
        for (int32_t c : n.children) plan->nodes[c].a = n.a;
        for (auto it = n.children.rbegin(); it != n.children.rend(); ++it) queue.push_front(*it);
        n.children.clear();
        continue;
      }
      out.push_back(i);
    }
    std::stable_sort(out.begin(), out.end(), [&](int32_t x, int32_t y) {
      return plan->nodes[x].cand_min() < plan->nodes[y].cand_min();
    });
    for (int32_t i : out) {
      std::vector<int32_t> ch = plan->nodes[i].children;
      plan->nodes[i].children = dissolve(ch);
    }
    return out;
  }
};

}  // namespace

bool plan_candidates(const ResidentTree& tree, PagePool* pool, int32_t n, const int32_t* tok,
                     const int64_t* off, Plan* plan, PlanMode mode) {
  *plan = Plan();
  std::vector<const int32_t*> rel(n);
  std::vector<int64_t> len(n);
  plan->anchors.resize(n);
  plan->anchor_len.resize(n);
  for (int32_t c = 0; c < n; ++c) {
    int64_t h, m;
    tree.match(tok + off[c], off[c + 1] - off[c], &h, &m);
    plan->anchors[c] = h;
    plan->anchor_len[c] = m;
    rel[c] = tok + off[c] + m;
    len[c] = off[c + 1] - off[c] - m;
  }
  // group candidates by anchor, anchors in order of first appearance
  std::vector<int64_t> anchor_order;
  std::vector<std::vector<int32_t>> by_anchor;
  for (int32_t c = 0; c < n; ++c) {
    size_t g = 0;
    while (g < anchor_order.size() && anchor_order[g] != plan->anchors[c]) ++g;
    if (g == anchor_order.size()) {
      anchor_order.push_back(plan->anchors[c]);
      by_anchor.emplace_back();
    }
    by_anchor[g].push_back(c);
  }
  Builder B{plan, rel, len};
  std::vector<int32_t> tops;
  for (size_t g = 0; g < by_anchor.size(); ++g) {
    std::vector<int32_t> t = B.dissolve(B.build(by_anchor[g], 0, anchor_order[g]));
    tops.insert(tops.end(), t.begin(), t.end());
  }
  // tree depth and parent links
  auto by_min = [&](int32_t x, int32_t y) {
    return plan->nodes[x].cand_min() < plan->nodes[y].cand_min();
  };
  {
    std::vector<int32_t> level = tops;
    int32_t depth = 1;
    while (!level.empty()) {
      std::vector<int32_t> next;
      for (int32_t i : level) {
        plan->nodes[i].depth = depth;
        for (int32_t c : plan->nodes[i].children) {
          plan->nodes[c].parent = i;
          next.push_back(c);
        }
      }
      level = std::move(next);
      ++depth;
    }
  }
  auto by_depth_min = [&](int32_t x, int32_t y) {
    const PlanNode& a = plan->nodes[x];
    const PlanNode& b = plan->nodes[y];
    return a.depth != b.depth ? a.depth < b.depth : a.cand_min() < b.cand_min();
  };
  std::vector<int32_t> frontier = tops;
  while (!frontier.empty()) {
    std::vector<int32_t> round;
    if (mode == PlanMode::DEPTH) {
      round = frontier;
    } else {
      for (int32_t v : frontier) {
        if (plan->nodes[v].children.empty()) {
          round.push_back(v);
          continue;
        }
        // the builder: the node's smallest candidate, down its own path
        const int32_t bc = plan->nodes[v].cand_min();
        int32_t x = v;
        for (;;) {
          round.push_back(x);
          const PlanNode& nx = plan->nodes[x];
          if (std::find(nx.readout.begin(), nx.readout.end(), bc) != nx.readout.end()) break;
          int32_t down = -1;
          for (int32_t ch : nx.children) {
            const auto& cs = plan->nodes[ch].cands;
            if (std::binary_search(cs.begin(), cs.end(), bc)) {
              down = ch;
              break;
            }
          }
          x = down;
        }
      }
    }
    std::sort(round.begin(), round.end(), by_depth_min);
    // next: children of this round's nodes that it did not compute
    std::vector<char> in_round(plan->nodes.size(), 0);
    for (int32_t i : round) in_round[i] = 1;
    std::vector<int32_t> next;
    for (int32_t i : round)
      for (int32_t c : plan->nodes[i].children)
        if (!in_round[c]) next.push_back(c);
    std::sort(next.begin(), next.end(), by_min);
    plan->rounds.push_back(std::move(round));
    frontier = std::move(next);
  }
  int32_t id = 0;
  for (auto& rnd : plan->rounds)
    for (int32_t i : rnd) {
      plan->nodes[i].id = id++;
      plan->id_to_index.push_back(i);
    }
  // pages: replay the rounds on the pool (all-or-nothing)
  std::set<int32_t> snap = pool->snapshot();
  bool ok = true;
  for (auto& rnd : plan->rounds) {
    for (int32_t i : rnd) {
      PlanNode& x = plan->nodes[i];
      int32_t need = pages_for(x.b - x.a);
      if (need > pool->n_free()) {
        ok = false;
        break;
      }
      x.pages = pool->alloc(need);
    }
    if (!ok) break;
    for (int32_t i : rnd)
      if (plan->nodes[i].children.empty()) pool->release(plan->nodes[i].pages);
  }
  pool->restore(std::move(snap));
  if (!ok) return false;
  plan->readout_node.assign(n, -1);
  for (auto& rnd : plan->rounds)
    for (int32_t i : rnd)
      for (int32_t c : plan->nodes[i].readout) plan->readout_node[c] = plan->nodes[i].id;
  return true;
}

std::vector<int32_t> Plan::serialize() const {
  std::vector<int32_t> out;
  out.push_back(int32_t(rounds.size()));
  for (auto& rnd : rounds) {
    out.push_back(int32_t(rnd.size()));
    for (int32_t i : rnd) {
      const PlanNode& x = nodes[i];
      out.push_back(x.id);
      out.push_back(x.parent >= 0 ? nodes[x.parent].id : -1);
      out.push_back(int32_t(x.anchor));
      out.push_back(x.depth);
      out.push_back(x.cand_min());
      out.push_back(int32_t(x.a));
      out.push_back(int32_t(x.b - x.a));
      out.push_back(int32_t(x.pages.size()));
      out.insert(out.end(), x.pages.begin(), x.pages.end());
      out.push_back(int32_t(x.readout.size()));
      out.insert(out.end(), x.readout.begin(), x.readout.end());
    }
  }
  out.push_back(int32_t(readout_node.size()));
  for (size_t c = 0; c < readout_node.size(); ++c) {
    out.push_back(int32_t(anchors[c]));
    out.push_back(int32_t(anchor_len[c]));
    out.push_back(readout_node[c]);
  }
  return out;
}

}  // namespace jev
