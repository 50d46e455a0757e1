// Extended radix tree of cached states (host only).
//
// Sources, cited by page title and section:
//   [AKV-blog]  "AKV: Cache Engineering for Autonomous Agents ...", section 3
//               (each edge carries the token sequence and the ordered cache
//               operations applied to it; a request walks tokens and
//               operations together, and forks where the operations diverge)
//   [AKV-notes] "Cache Engineering for Agents", section 3 (drop nodes,
//               reposition branches, and the cache reuse matching rules:
//               exact match, retrigger match, lookup order; eviction)
//
// A history is a sequence of events: a token (id, position) or one span of a
// cache operation (drop [b, e), repos [b, e) by delta).  The tree is a trie
// over events; a checkpoint registers the pool sequence whose current state
// is the history's state.  A node can be served by a checkpoint below it when
// the path between them holds tokens only: operations after the node would
// have changed the node's tokens, appended tokens do not (the first k logical
// tokens of the checkpoint's sequence are then the node's state).
//
// Matching a request history (the walk stops at the first event that does
// not match):
//   exact     tokens, positions and operations equal -> reuse as is;
//   retrigger tokens and operations equal, every position shifted by one
//             delta -> reuse after turning the keys by that delta
//             (akv_seq_clone);
// the longest exact prefix is taken first, and a retrigger prefix replaces it
// only when strictly longer.  Among servers of one node the checkpoint
// registered last wins.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <memory>
#include <new>
#include <string>
#include <vector>

#include "../../include/akv.h"
#include "akv_internal.h"

struct akv_tree {
  struct Node {
    akv_event ev{};                 // event on the edge from the parent
    int32_t parent = -1;
    int32_t depth = 0;              // events from the root
    int32_t tokens = 0;             // token events from the root
    std::vector<int32_t> kids;
    int32_t server = -1;            // checkpoint serving this node (latest), or -1
  };
  struct Check {
    int32_t node = -1;
    int32_t seq = -1;
    int64_t stamp = 0;              // last insert or match
    int64_t order = 0;              // insertion order (ties: later wins)
    int32_t pins = 0;
    bool live = false;
  };
  std::vector<Node> nodes;
  std::vector<Check> checks;
  int64_t clock = 0;
  int64_t inserted = 0;
};

namespace {

akv_status tfail(akv_status s, const char* what) {
  akv::set_error(what);
  return s;
}

bool same_event(const akv_event& a, const akv_event& b) {
  return a.kind == b.kind && a.a == b.a && a.b == b.b && a.c == b.c;
}

bool valid_event(const akv_event& e) {
  switch (e.kind) {
    case AKV_EV_TOKEN: return e.b >= 0;
    case AKV_EV_DROP: return e.a >= 0 && e.a <= e.b;
    case AKV_EV_REPOS: return e.a >= 0 && e.a <= e.b;
    default: return false;
  }
}

// Servers of the node a checkpoint sits on: up through token edges only.
void mark_servers(akv_tree* t, int32_t node, int32_t ck) {
  for (int32_t n = node; n >= 0; n = t->nodes[n].parent) {
    t->nodes[n].server = ck;
    if (t->nodes[n].ev.kind != AKV_EV_TOKEN || n == 0) break;
  }
}

// Rebuild every node's server from the live checkpoints, older first, so the
// latest registered checkpoint wins where several serve one node.
void rebuild_servers(akv_tree* t) {
  for (auto& n : t->nodes) n.server = -1;
  std::vector<int32_t> live;
  for (int32_t i = 0; i < (int32_t)t->checks.size(); ++i)
    if (t->checks[i].live) live.push_back(i);
  std::sort(live.begin(), live.end(),
            [&](int32_t a, int32_t b) { return t->checks[a].order < t->checks[b].order; });
  for (int32_t c : live) mark_servers(t, t->checks[c].node, c);
}

struct Best {
  int32_t node = -1;
  int32_t depth = 0;
  int64_t order = -1;
  int64_t delta = 0;
};

// Retrigger walk: tokens by id with one position shift, operations exactly;
// every compatible path (positional versions fork on positions), depth first
// with an explicit stack.
void retrigger_walk(const akv_tree* t, const akv_event* ev, int32_t n_ev, Best& best) {
  struct Frame {
    int32_t node, i;
    bool have_delta;
    int64_t delta;
  };
  std::vector<Frame> stack{{0, 0, false, 0}};
  while (!stack.empty()) {
    const Frame f = stack.back();
    stack.pop_back();
    const akv_tree::Node& nd = t->nodes[f.node];
    if (nd.server >= 0 && f.i > 0) {
      const int64_t ord = t->checks[nd.server].order;
      if (f.i > best.depth || (f.i == best.depth && ord > best.order))
        best = {f.node, f.i, ord, f.have_delta ? f.delta : 0};
    }
    if (f.i == n_ev) continue;
    const akv_event& e = ev[f.i];
    for (int32_t k : nd.kids) {
      const akv_event& c = t->nodes[k].ev;
      if (c.kind != e.kind) continue;
      if (e.kind == AKV_EV_TOKEN) {
        if (c.a != e.a) continue;
        const int64_t d = (int64_t)e.b - c.b;
        if (f.have_delta && d != f.delta) continue;
        stack.push_back({k, f.i + 1, true, d});
      } else if (same_event(c, e)) {
        stack.push_back({k, f.i + 1, f.have_delta, f.delta});
      }
    }
  }
}

}  // namespace

extern "C" {

akv_status akv_tree_create(akv_tree** out) {
  if (!out) return tfail(AKV_EINVAL, "out is NULL");
  try {
    akv_tree* t = new akv_tree();
    t->nodes.emplace_back();   // root
    *out = t;
    return AKV_OK;
  } catch (const std::bad_alloc&) {
    return tfail(AKV_ENOMEM, "host allocation failed");
  }
}

akv_status akv_tree_destroy(akv_tree* t) {
  delete t;
  return AKV_OK;
}

akv_status akv_tree_insert(akv_tree* t, const akv_event* ev, int32_t n, int32_t seq) {
  if (!t) return tfail(AKV_EINVAL, "NULL tree");
  if (n < 1 || !ev) return tfail(AKV_EINVAL, "a checkpoint needs a non-empty history");
  if (seq < 0) return tfail(AKV_EINVAL, "negative sequence id");
  for (int32_t i = 0; i < n; ++i)
    if (!valid_event(ev[i])) return tfail(AKV_EINVAL, "bad event");
  for (const auto& c : t->checks)
    if (c.live && c.seq == seq) return tfail(AKV_EINVAL, "sequence already registered");
  try {
    int32_t cur = 0;
    for (int32_t i = 0; i < n; ++i) {
      int32_t next = -1;
      for (int32_t k : t->nodes[cur].kids)
        if (same_event(t->nodes[k].ev, ev[i])) {
          next = k;
          break;
        }
      if (next < 0) {
        akv_tree::Node nd;
        nd.ev = ev[i];
        nd.parent = cur;
        nd.depth = t->nodes[cur].depth + 1;
        nd.tokens = t->nodes[cur].tokens + (ev[i].kind == AKV_EV_TOKEN ? 1 : 0);
        next = (int32_t)t->nodes.size();
        t->nodes.push_back(nd);
        t->nodes[cur].kids.push_back(next);
      }
      cur = next;
    }
    akv_tree::Check c;
    c.node = cur;
    c.seq = seq;
    c.stamp = ++t->clock;
    c.order = ++t->inserted;
    c.live = true;
    t->checks.push_back(c);
    mark_servers(t, cur, (int32_t)t->checks.size() - 1);
    return AKV_OK;
  } catch (const std::bad_alloc&) {
    return tfail(AKV_ENOMEM, "host allocation failed");
  }
}

akv_status akv_tree_match(akv_tree* t, const akv_event* ev, int32_t n, akv_tree_hit* out) {
  if (!t || !out) return tfail(AKV_EINVAL, "NULL argument");
  if (n < 0 || (n > 0 && !ev)) return tfail(AKV_EINVAL, "bad history");
  for (int32_t i = 0; i < n; ++i)
    if (!valid_event(ev[i])) return tfail(AKV_EINVAL, "bad event");
  *out = akv_tree_hit{-1, 0, 0, 0, 0};
  // exact: one path
  Best ex;
  int32_t cur = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t next = -1;
    for (int32_t k : t->nodes[cur].kids)
      if (same_event(t->nodes[k].ev, ev[i])) {
        next = k;
        break;
      }
    if (next < 0) break;
    cur = next;
    if (t->nodes[cur].server >= 0) ex = {cur, i + 1, t->checks[t->nodes[cur].server].order, 0};
  }
  // retrigger: every path of equal ids and operations under one shift
  Best rt;
  retrigger_walk(t, ev, n, rt);
  const bool take_rt = rt.node >= 0 && rt.depth > ex.depth;
  const Best& b = take_rt ? rt : ex;
  if (b.node < 0) return AKV_OK;
  const int32_t ck = t->nodes[b.node].server;
  akv_tree::Check& c = t->checks[ck];
  c.stamp = ++t->clock;
  out->seq = c.seq;
  out->n_events = b.depth;
  out->n_tokens = t->nodes[b.node].tokens;
  out->exact = take_rt ? 0 : 1;
  out->delta = (int32_t)(take_rt ? b.delta : 0);
  if (take_rt && (b.delta < INT32_MIN || b.delta > INT32_MAX)) return tfail(AKV_ERANGE, "shift out of range");
  return AKV_OK;
}

akv_status akv_tree_pin(akv_tree* t, int32_t seq, int32_t add) {
  if (!t) return tfail(AKV_EINVAL, "NULL tree");
  for (auto& c : t->checks)
    if (c.live && c.seq == seq) {
      if (c.pins + add < 0) return tfail(AKV_EINVAL, "unpinned more than pinned");
      c.pins += add;
      return AKV_OK;
    }
  return tfail(AKV_EINVAL, "sequence not registered");
}

akv_status akv_tree_evict(akv_tree* t, int32_t max_n, int32_t* seqs_out, int32_t* n_out) {
  if (!t || !n_out) return tfail(AKV_EINVAL, "NULL argument");
  if (max_n < 0 || (max_n > 0 && !seqs_out)) return tfail(AKV_EINVAL, "bad output");
  std::vector<int32_t> cand;
  for (int32_t i = 0; i < (int32_t)t->checks.size(); ++i)
    if (t->checks[i].live && t->checks[i].pins == 0) cand.push_back(i);
  std::sort(cand.begin(), cand.end(), [&](int32_t a, int32_t b) {
    return t->checks[a].stamp != t->checks[b].stamp ? t->checks[a].stamp < t->checks[b].stamp
                                                    : t->checks[a].order < t->checks[b].order;
  });
  int32_t k = 0;
  for (; k < (int32_t)cand.size() && k < max_n; ++k) {
    t->checks[cand[k]].live = false;
    seqs_out[k] = t->checks[cand[k]].seq;
  }
  *n_out = k;
  if (k) rebuild_servers(t);
  return AKV_OK;
}

akv_status akv_tree_stats(akv_tree* t, int32_t* n_nodes, int32_t* n_checkpoints) {
  if (!t) return tfail(AKV_EINVAL, "NULL tree");
  if (n_nodes) *n_nodes = (int32_t)t->nodes.size();
  if (n_checkpoints) {
    int32_t c = 0;
    for (const auto& ck : t->checks) c += ck.live ? 1 : 0;
    *n_checkpoints = c;
  }
  return AKV_OK;
}

}  // extern "C"
