// Host-side tile planner (see plan.hpp for the rules and their sources).
#include "plan.hpp"

#include <algorithm>
#include <map>
#include <numeric>
#include <set>

namespace mk {

namespace {

std::array<int, kMaxDims> build_partition(const std::array<int, 3>& grid, const std::array<int, 3>& amap) {
  std::array<int, kMaxDims> part{{1, 1, 1, 1}};
  for (int a = 0; a < 3; ++a)
    if (amap[a] >= 0) part[amap[a]] *= grid[a];
  return part;
}

long lcm_l(long a, long b) { return a / std::gcd(a, b) * b; }

enum Kind { kChain, kFork, kJoin, kMixed };

// Op-specific payload words (instruction words 14..23) of task (x, y, z).
void payload(const GraphOp& op, int x, int y, int z, const std::vector<int32_t>* kv_len, int32_t* w) {
  (void)z;
  const auto& p = op.p;
  switch (op.kind) {
    case kQkv:  // p0 = rows per tile
      w[0] = y * p[0];
      w[1] = p[0];
      break;
    case kAttn: {  // p0 = splits
      int pos = (*kv_len)[x], lo, hi;
      split_range(pos, p[0], z, &lo, &hi);
      w[0] = lo;
      w[1] = hi;
      w[2] = pos;
      break;
    }
    case kCombine:  // p0 = splits
      w[0] = p[0];
      break;
    case kOproj:
    case kLmHead:  // p0 = rows per tile, p1 = total rows
    case kGateUp:  // p0 = outputs per tile, p1 = total outputs
      w[0] = x * p[0];
      w[1] = std::min(p[0], p[1] - x * p[0]);
      break;
    case kDown:  // p0 = rows per tile, p1 = total rows, p2 = K
      w[0] = x * p[0];
      w[1] = std::min(p[0], p[1] - x * p[0]);
      w[2] = 0;
      w[3] = p[2];
      break;
    case kArgmax:  // p0 = LM-head tiles
      w[0] = p[0];
      break;
    case kGA0:
    case kGQaNorm:  // one token row per task
      w[0] = x;
      break;
    case kGQkva:
    case kGIdxk:
    case kGIdxq:  // p0 = output rows
      w[0] = x * kGlmRows;
      w[1] = std::min(kGlmRows, p[0] - x * kGlmRows);
      w[2] = -1;
      break;
    case kGGate:  // p0 = output rows, p1 = 128-column blocks of K; x row tile, y K-split
      w[0] = x * kGlmRows;
      w[1] = std::min(kGlmRows, p[0] - x * kGlmRows);
      w[2] = -1;
      w[3] = y * kGateBlocks;
      w[4] = std::min(kGateBlocks, p[1] - y * kGateBlocks);
      break;
    case kGGateRed:  // p0 = output rows, p1 = K-splits
      w[0] = x * kGlmRows;
      w[1] = std::min(kGlmRows, p[0] - x * kGlmRows);
      w[2] = p[1];
      break;
    case kGQkvb: {  // p0 = head_dim, p1 = nope dims, p2 = rope dims; x head, y tile
      const int base = x * p[0];
      if (y < p[1] / kGlmRows) {
        w[0] = base + y * kGlmRows;
        w[1] = kGlmRows;
        w[2] = -1;
      } else {
        const int j = y - p[1] / kGlmRows, h = kGlmRows / 2;
        w[0] = base + p[1] + j * h;
        w[1] = h;
        w[2] = base + p[1] + p[2] / 2 + j * h;
      }
      break;
    }
    default:
      break;
  }
}

// Place task t in queue t % num_cus at slot t / num_cus and write its words
// (MegaRTP article, section 4 "KernelPlan"); fills the op table too.
void encode(const std::vector<GraphOp>& ops, const std::vector<int32_t>* kv_len, Plan* out) {
  Plan& P = *out;
  const int num_cus = P.num_cus;
  P.max_len = std::max(1, ceil_div(P.num_tasks, num_cus));
  P.queue.assign((size_t)num_cus * P.max_len * kWords, 0);
  for (int t = 0; t < P.num_tasks; ++t) {
    const auto& tk = P.tasks[t];
    const GraphOp& op = ops[tk[0]];
    int32_t* w = &P.queue[((size_t)(t % num_cus) * P.max_len + t / num_cus) * kWords];
    w[kWOpcode] = op.opcode;
    w[kWSpec] = op.spec;
    w[kWOpRow] = tk[0];
    if (P.task_wait[t] >= 0) {
      w[kWWaitCnt] = 1;
      w[kWWaitEv] = P.task_wait[t];
      w[kWWaitTgt] = (int32_t)P.event_target[P.task_wait[t]];
      if (P.task_wait2[t] >= 0) {
        w[kWWaitCnt] = 2;
        w[kWWait2Ev] = P.task_wait2[t];
        w[kWWait2Tgt] = (int32_t)P.event_target[P.task_wait2[t]];
      }
    }
    if (P.task_trigger[t] >= 0) {
      w[kWSigCnt] = 1;
      w[kWSigEv] = P.task_trigger[t];
      w[kWSigInc] = 1;
      if (!P.sig_pub.empty()) w[kWSigPub] = P.sig_pub[t][0];
      if (P.task_trigger2[t] >= 0) {
        w[kWSigCnt] = 2;
        w[kWSig2Ev] = P.task_trigger2[t];
        w[kWSig2Inc] = 1;
        w[kWSig2Pub] = P.sig_pub[t][1];
      }
    }
    w[kWTask] = t;
    w[kWLayer] = op.layer;
    w[kWGx] = tk[1];
    w[kWGy] = tk[2];
    w[kWGz] = tk[3];
    payload(op, tk[1], tk[2], tk[3], kv_len, w + kWPay);
  }
  const int n_ops = (int)ops.size();
  P.op_table.assign((size_t)n_ops * 8, 0);
  for (int o = 0; o < n_ops; ++o) {
    int32_t* r = &P.op_table[(size_t)o * 8];
    r[0] = ops[o].opcode;
    r[1] = ops[o].spec;
    r[2] = ops[o].layer;
    r[3] = ops[o].grid[0];
    r[4] = ops[o].grid[1];
    r[5] = ops[o].grid[2];
    r[6] = ops[o].grid[0] * ops[o].grid[1] * ops[o].grid[2];
  }
}

}  // namespace

std::string plan_graph(const std::vector<GraphOp>& ops, const std::vector<GraphEdge>& edges, int num_cus,
                       const std::vector<int32_t>* kv_len, Plan* out) {
  const int n_ops = (int)ops.size(), n_edges = (int)edges.size();
  if (num_cus <= 0) return "num_cus must be positive";
  for (const auto& op : ops)
    for (int a = 0; a < 3; ++a)
      if (op.grid[a] < 1) return "grid extents must be >= 1";
  for (const auto& e : edges) {
    if (e.prod < 0 || e.cons >= n_ops || e.prod >= e.cons) return "edges must go from a lower to a higher op index";
    for (int a = 0; a < 3; ++a)
      if (e.out_map[a] >= kMaxDims || e.in_map[a] >= kMaxDims || e.out_map[a] < -1 || e.in_map[a] < -1)
        return "map entries must be -1..3";
  }

  // 1. per-edge gcd partition, with the ragged-alignment check
  std::vector<std::array<int, kMaxDims>> evd(n_edges);
  for (int i = 0; i < n_edges; ++i) {
    const auto& e = edges[i];
    auto pp = build_partition(ops[e.prod].grid, e.out_map);
    auto cp = build_partition(ops[e.cons].grid, e.in_map);
    for (int d = 0; d < kMaxDims; ++d) {
      int g = std::gcd(pp[d], cp[d]);
      if (e.has_extent && g > 1) {
        for (int k = 1; k < g; ++k) {
          long bp = std::min<long>((long)k * (pp[d] / g) * e.ptile[d], e.extent[d]);
          long bc = std::min<long>((long)k * (cp[d] / g) * e.ctile[d], e.extent[d]);
          if (bp != bc) {
            g = 1;
            break;
          }
        }
      }
      evd[i][d] = g;
    }
  }
  auto whole = [&](int i) {
    for (int d = 0; d < kMaxDims; ++d)
      if (evd[i][d] != 1) return false;
    return true;
  };

  // 2. residual stripping by full-dependency sets
  std::vector<std::vector<int>> in_edges(n_ops);
  for (int i = 0; i < n_edges; ++i) in_edges[edges[i].cons].push_back(i);
  std::vector<std::set<int>> fd(n_ops);
  std::vector<uint8_t> kept(n_edges, 1);
  for (int c = 0; c < n_ops; ++c) {
    for (int i : in_edges[c]) {
      int p = edges[i].prod;
      for (int j : in_edges[c]) {
        if (j != i && edges[j].prod != p && fd[edges[j].prod].count(p)) {
          kept[i] = 0;
          break;
        }
      }
    }
    for (int i : in_edges[c]) {
      if (!kept[i]) continue;
      int x = edges[i].prod;
      fd[c].insert(fd[x].begin(), fd[x].end());
      if (whole(i)) fd[c].insert(x);
    }
  }

  // 3. components of kept edges (edges sharing a producer or a consumer)
  std::vector<int> parent(n_edges);
  std::iota(parent.begin(), parent.end(), 0);
  auto find = [&](int i) {
    while (parent[i] != i) {
      parent[i] = parent[parent[i]];
      i = parent[i];
    }
    return i;
  };
  std::map<int, std::vector<int>> by_prod, by_cons;
  for (int i = 0; i < n_edges; ++i)
    if (kept[i]) {
      by_prod[edges[i].prod].push_back(i);
      by_cons[edges[i].cons].push_back(i);
    }
  auto unite = [&](const std::vector<int>& grp) {
    for (size_t k = 1; k < grp.size(); ++k) {
      int a = find(grp[0]), b = find(grp[k]);
      if (a != b) parent[std::max(a, b)] = std::min(a, b);
    }
  };
  for (auto& kv : by_prod) unite(kv.second);
  for (auto& kv : by_cons) unite(kv.second);
  std::map<int, std::vector<int>> comps;
  for (int i = 0; i < n_edges; ++i)
    if (kept[i]) comps[find(i)].push_back(i);
  std::map<int, Kind> kind;
  std::vector<int> comp_of_cons(n_ops, -1);
  for (auto& kv : comps) {
    const auto& es = kv.second;
    std::set<int> prods, conss;
    std::set<std::pair<int, int>> pairs;
    for (int i : es) {
      prods.insert(edges[i].prod);
      conss.insert(edges[i].cons);
      pairs.insert({edges[i].prod, edges[i].cons});
    }
    Kind k;
    if (es.size() == 1) {
      k = kChain;
    } else if (pairs.size() != es.size()) {
      k = kMixed;
    } else if (prods.size() == 1 && std::all_of(conss.begin(), conss.end(), [&](int c) { return by_cons[c].size() == 1; })) {
      k = kFork;
    } else if (conss.size() == 1 && std::all_of(prods.begin(), prods.end(), [&](int p) { return by_prod[p].size() == 1; })) {
      k = kJoin;
    } else {
      k = kMixed;
    }
    kind[kv.first] = k;
    if (k == kMixed)
      for (int i : es) evd[i] = {{1, 1, 1, 1}};
    for (int c : conss) comp_of_cons[c] = kv.first;
    if (*prods.rbegin() >= *conss.begin()) return "a component's producers must precede its consumers";
  }

  // 4. fork / join lcm normalization
  for (auto& kv : comps) {
    const auto& es = kv.second;
    Kind k = kind[kv.first];
    if (k != kFork && k != kJoin) continue;
    const GraphOp& O = ops[k == kFork ? edges[es[0]].prod : edges[es[0]].cons];
    for (int a = 0; a < 3; ++a) {
      long Lx = 1;
      for (int i : es) {
        int d = k == kFork ? edges[i].out_map[a] : edges[i].in_map[a];
        int ev = d >= 0 ? evd[i][d] : 1;
        Lx = lcm_l(Lx, O.grid[a] / ev);
      }
      for (int i : es) {
        int d = k == kFork ? edges[i].out_map[a] : edges[i].in_map[a];
        if (d >= 0) evd[i][d] = (O.grid[a] % Lx == 0) ? (int)(O.grid[a] / Lx) : 1;
      }
    }
  }

  // 5. linearization
  Plan& P = *out;
  P = Plan();
  std::map<std::array<int, 4>, int> task_of;
  std::vector<uint8_t> emitted(n_ops, 0);
  auto new_task = [&](int o, int x, int y, int z, int wait_ev) {
    task_of[{{o, x, y, z}}] = (int)P.tasks.size();
    P.tasks.push_back({{o, x, y, z}});
    P.task_trigger.push_back(-1);
    P.task_wait.push_back(wait_ev);
  };
  struct Slice {
    int op;
    std::array<int, 3> lo, hi;
  };
  // per-axis range of an op's tasks in the slice whose event index along tensor dim d is idx[d]
  auto axis_slice = [&](int o, const std::array<int, 3>& amap, const std::array<int, kMaxDims>& ed,
                        const std::array<int, kMaxDims>& idx) {
    Slice s{o, {{0, 0, 0}}, {{0, 0, 0}}};
    for (int a = 0; a < 3; ++a) {
      int d = amap[a];
      if (d >= 0 && ed[d] > 1) {
        int span = ops[o].grid[a] / ed[d];
        s.lo[a] = idx[d] * span;
        s.hi[a] = (idx[d] + 1) * span;
      } else {
        s.lo[a] = 0;
        s.hi[a] = ops[o].grid[a];
      }
    }
    return s;
  };
  std::string err;
  auto emit_event = [&](const std::vector<Slice>& cons, const std::vector<Slice>& prods) {
    int eid = (int)P.event_first.size();
    P.event_first.push_back((int)P.tasks.size());
    for (const auto& s : cons)
      for (int x = s.lo[0]; x < s.hi[0]; ++x)
        for (int y = s.lo[1]; y < s.hi[1]; ++y)
          for (int z = s.lo[2]; z < s.hi[2]; ++z) new_task(s.op, x, y, z, eid);
    P.event_last.push_back((int)P.tasks.size());
    uint32_t n = 0;
    for (const auto& s : prods)
      for (int x = s.lo[0]; x < s.hi[0]; ++x)
        for (int y = s.lo[1]; y < s.hi[1]; ++y)
          for (int z = s.lo[2]; z < s.hi[2]; ++z) {
            int t = task_of.at({{s.op, x, y, z}});
            if (P.task_trigger[t] != -1) err = "a task would trigger two events";
            P.task_trigger[t] = eid;
            ++n;
          }
    P.event_target.push_back(n);
  };

  for (int c = 0; c < n_ops; ++c) {
    if (emitted[c]) continue;
    const GraphOp& C = ops[c];
    if (comp_of_cons[c] < 0) {
      for (int x = 0; x < C.grid[0]; ++x)
        for (int y = 0; y < C.grid[1]; ++y)
          for (int z = 0; z < C.grid[2]; ++z) new_task(c, x, y, z, -1);
      emitted[c] = 1;
      continue;
    }
    int root = comp_of_cons[c];
    const auto& es = comps[root];
    Kind k = kind[root];
    if (k == kChain || k == kJoin) {
      int i0 = es[0];
      std::array<int, 3> nev;
      for (int a = 0; a < 3; ++a) {
        int d = edges[i0].in_map[a];
        nev[a] = d >= 0 ? evd[i0][d] : 1;
      }
      for (int ix = 0; ix < nev[0]; ++ix)
        for (int iy = 0; iy < nev[1]; ++iy)
          for (int iz = 0; iz < nev[2]; ++iz) {
            std::array<int, 3> cidx{{ix, iy, iz}};
            Slice cs{c, {{0, 0, 0}}, {{0, 0, 0}}};
            for (int a = 0; a < 3; ++a) {
              int span = C.grid[a] / nev[a];
              cs.lo[a] = cidx[a] * span;
              cs.hi[a] = (cidx[a] + 1) * span;
            }
            std::vector<Slice> prods;
            for (int i : es) {
              const auto& e = edges[i];
              std::array<int, kMaxDims> idx{{0, 0, 0, 0}};
              for (int a = 0; a < 3; ++a)
                if (e.in_map[a] >= 0) idx[e.in_map[a]] = cidx[a];
              prods.push_back(axis_slice(e.prod, e.out_map, evd[i], idx));
            }
            emit_event({cs}, prods);
          }
      emitted[c] = 1;
    } else if (k == kFork) {
      int p = edges[es[0]].prod;
      const GraphOp& Pop = ops[p];
      std::array<int, 3> nev;
      for (int a = 0; a < 3; ++a) {
        int d = edges[es[0]].out_map[a];
        nev[a] = d >= 0 ? evd[es[0]][d] : 1;
      }
      std::vector<int> order(es.begin(), es.end());
      std::stable_sort(order.begin(), order.end(), [&](int u, int v) { return edges[u].cons < edges[v].cons; });
      for (int ix = 0; ix < nev[0]; ++ix)
        for (int iy = 0; iy < nev[1]; ++iy)
          for (int iz = 0; iz < nev[2]; ++iz) {
            std::array<int, 3> pidx{{ix, iy, iz}};
            Slice ps{p, {{0, 0, 0}}, {{0, 0, 0}}};
            for (int a = 0; a < 3; ++a) {
              int span = Pop.grid[a] / nev[a];
              ps.lo[a] = pidx[a] * span;
              ps.hi[a] = (pidx[a] + 1) * span;
            }
            std::vector<Slice> cons;
            for (int i : order) {
              const auto& e = edges[i];
              std::array<int, kMaxDims> idx{{0, 0, 0, 0}};
              for (int a = 0; a < 3; ++a)
                if (e.out_map[a] >= 0) idx[e.out_map[a]] = pidx[a];
              cons.push_back(axis_slice(e.cons, e.in_map, evd[i], idx));
            }
            emit_event(cons, {ps});
          }
      for (int i : es) emitted[edges[i].cons] = 1;
    } else {
      std::set<int> conss, prods;
      for (int i : es) {
        conss.insert(edges[i].cons);
        prods.insert(edges[i].prod);
      }
      auto full = [&](int o) { return Slice{o, {{0, 0, 0}}, ops[o].grid}; };
      std::vector<Slice> cs, ps;
      for (int o : conss) cs.push_back(full(o));
      for (int o : prods) ps.push_back(full(o));
      emit_event(cs, ps);
      for (int o : conss) emitted[o] = 1;
    }
    if (!err.empty()) return err;
  }

  // 6. placement and encoding
  P.num_cus = num_cus;
  P.num_tasks = (int)P.tasks.size();
  P.num_events = (int)P.event_first.size();
  P.task_wait2.assign(P.num_tasks, -1);
  P.task_trigger2.assign(P.num_tasks, -1);
  encode(ops, kv_len, &P);
  P.edge_kept = kept;
  return "";
}

std::string plan_pairs(const std::vector<GraphOp>& ops, const std::vector<PairPub>& pubs,
                       const std::vector<PairEdge>& edges, int num_cus, const std::vector<int32_t>* kv_len, Plan* out) {
  const int n_ops = (int)ops.size(), n_pubs = (int)pubs.size();
  if (num_cus <= 0) return "num_cus must be positive";
  for (const auto& op : ops)
    for (int a = 0; a < 3; ++a)
      if (op.grid[a] < 1) return "grid extents must be >= 1";
  for (const auto& p : pubs) {
    if (p.op < 0 || p.op >= n_ops) return "publication of an unknown op";
    for (int r = 0; r < 3; ++r)
      if (p.map[r] < -1 || p.map[r] >= 3 || p.div[r] < 1 || p.sel[r] < -1 || (p.sel[r] >= 0 && p.sel[r] >= ops[p.op].grid[r]))
        return "publication map/div/sel out of range";
  }
  for (const auto& e : edges) {
    if (e.pub < 0 || e.pub >= n_pubs || e.cons >= n_ops || !(pubs[e.pub].op < e.cons))
      return "an edge must read a publication of an earlier op";
    if (e.strategy < kPairWhole || e.strategy > kPairTileReduce) return "unknown pairing strategy";
    for (int r = 0; r < 3; ++r)
      if (e.map[r] < -1 || e.map[r] >= 3 || e.div[r] < 1) return "edge map/div out of range";
  }
  auto nregions = [&](const PairPub& p) {
    std::array<int, 3> n{{1, 1, 1}};
    for (int r = 0; r < 3; ++r)
      if (p.map[r] >= 0) n[r] = ceil_div(ops[p.op].grid[p.map[r]], p.div[r]);
    return n;
  };
  auto region = [](const std::array<int, 3>& c, const std::array<int, 3>& map, const std::array<int, 3>& div) {
    std::array<int, 3> r{{0, 0, 0}};
    for (int d = 0; d < 3; ++d)
      if (map[d] >= 0) r[d] = c[map[d]] / div[d];
    return r;
  };
  auto publishes = [](const PairPub& p, const std::array<int, 3>& c) {
    for (int a = 0; a < 3; ++a)
      if (p.sel[a] >= 0 && c[a] != p.sel[a]) return false;
    return true;
  };
  // publishing tiles per (publication, region)
  std::vector<std::map<std::array<int, 3>, int>> count(n_pubs);
  for (int k = 0; k < n_pubs; ++k) {
    const auto& g = ops[pubs[k].op].grid;
    for (int x = 0; x < g[0]; ++x)
      for (int y = 0; y < g[1]; ++y)
        for (int z = 0; z < g[2]; ++z) {
          std::array<int, 3> c{{x, y, z}};
          if (publishes(pubs[k], c)) ++count[k][region(c, pubs[k].map, pubs[k].div)];
        }
  }
  Plan& P = *out;
  P = Plan();
  for (int o = 0; o < n_ops; ++o)
    for (int x = 0; x < ops[o].grid[0]; ++x)
      for (int y = 0; y < ops[o].grid[1]; ++y)
        for (int z = 0; z < ops[o].grid[2]; ++z) P.tasks.push_back({{o, x, y, z}});
  const int T = (int)P.tasks.size();
  std::vector<std::vector<int>> in_edges(n_ops);
  for (int i = 0; i < (int)edges.size(); ++i) in_edges[edges[i].cons].push_back(i);
  std::map<std::pair<int, std::array<int, 3>>, int> ev_of;
  std::map<int, int> reduce_n;
  std::vector<std::vector<int>> ev_tasks;
  P.task_wait.assign(T, -1);
  P.task_wait2.assign(T, -1);
  for (int t = 0; t < T; ++t) {
    const auto& tk = P.tasks[t];
    const std::array<int, 3> c{{tk[1], tk[2], tk[3]}};
    int w[3], nw = 0;
    for (int i : in_edges[tk[0]]) {
      const PairEdge& e = edges[i];
      const PairPub& p = pubs[e.pub];
      const auto r = region(c, e.map, e.div);
      const auto nr = nregions(p);
      for (int d = 0; d < 3; ++d)
        if (r[d] >= nr[d]) return "edge " + std::to_string(i) + ": a consumer tile reads a region outside the publication";
      auto it = count[e.pub].find(r);
      const int n = it == count[e.pub].end() ? 0 : it->second;
      if (n == 0) return "edge " + std::to_string(i) + ": a region has no publishing tile";
      if (e.strategy == kPairWhole && (nr != std::array<int, 3>{{1, 1, 1}} || p.sel != std::array<int, 3>{{-1, -1, -1}}))
        return "edge " + std::to_string(i) + ": 'whole' needs one region that every producer tile publishes";
      if (e.strategy == kPairTile && n != 1) return "edge " + std::to_string(i) + ": 'tile' needs one producer tile per region";
      if (e.strategy == kPairTileReduce && reduce_n.emplace(i, n).first->second != n)
        return "edge " + std::to_string(i) + ": 'tile_reduce' regions must have equal partial counts";
      const auto key = std::make_pair(e.pub, r);
      auto ev = ev_of.find(key);
      if (ev == ev_of.end()) {
        ev = ev_of.emplace(key, (int)P.event_target.size()).first;
        P.event_target.push_back((uint32_t)n);
        ev_tasks.emplace_back();
      }
      bool dup = false;
      for (int j = 0; j < nw; ++j) dup |= w[j] == ev->second;
      if (dup) continue;
      if (nw == 2) return "a task waits on more than two events";
      w[nw++] = ev->second;
      ev_tasks[ev->second].push_back(t);
    }
    if (nw > 0) P.task_wait[t] = w[0];
    if (nw > 1) P.task_wait2[t] = w[1];
  }
  std::vector<std::vector<int>> pubs_of(n_ops);
  for (int k = 0; k < n_pubs; ++k) pubs_of[pubs[k].op].push_back(k);
  P.task_trigger.assign(T, -1);
  P.task_trigger2.assign(T, -1);
  P.sig_pub.assign(T, {{0, 0}});
  for (int t = 0; t < T; ++t) {
    const auto& tk = P.tasks[t];
    const std::array<int, 3> c{{tk[1], tk[2], tk[3]}};
    int ns = 0;
    for (int k : pubs_of[tk[0]]) {
      if (!publishes(pubs[k], c)) continue;
      auto ev = ev_of.find(std::make_pair(k, region(c, pubs[k].map, pubs[k].div)));
      if (ev == ev_of.end()) continue;
      if (ns == 2) return "a task signals more than two events";
      (ns == 0 ? P.task_trigger[t] : P.task_trigger2[t]) = ev->second;
      P.sig_pub[t][ns++] = k;
    }
  }
  P.num_cus = num_cus;
  P.num_tasks = T;
  P.num_events = (int)P.event_target.size();
  for (const auto& ts : ev_tasks) {
    P.event_first.push_back(ts.front());
    P.event_last.push_back(ts.back() + 1);
  }
  encode(ops, kv_len, &P);
  P.edge_kept.assign(edges.size(), 1);
  return "";
}

void model_pairs(const std::vector<GraphOp>& ops, std::vector<PairPub>* pubs_out, std::vector<PairEdge>* edges_out) {
  auto& pubs = *pubs_out;
  auto& edges = *edges_out;
  pubs.clear();
  edges.clear();
  auto pub = [&](int op, std::array<int, 3> map) {
    PairPub p;
    p.op = op;
    p.map = map;
    pubs.push_back(p);
    return (int)pubs.size() - 1;
  };
  auto edge = [&](int p, int c, int strategy, std::array<int, 3> map) {
    PairEdge e;
    e.pub = p;
    e.cons = c;
    e.strategy = strategy;
    e.map = map;
    edges.push_back(e);
  };
  const std::array<int, 3> none{{-1, -1, -1}};
  const int L = ((int)ops.size() - 2) / 6;
  int prev_d = -1;
  for (int l = 0; l < L; ++l) {
    const int q = 6 * l, a = q + 1, c = q + 2, o = q + 3, g = q + 4, d = q + 5;
    const int pq = pub(q, {{0, -1, -1}}), pa = pub(a, {{0, 1, -1}}), pc = pub(c, none), po = pub(o, none),
              pg = pub(g, none);
    if (prev_d >= 0) edge(prev_d, q, kPairWhole, none);
    edge(pq, a, kPairTileCover, {{1, -1, -1}});
    edge(pa, c, kPairTileReduce, {{0, 1, -1}});
    edge(pc, o, kPairWhole, none);
    if (prev_d >= 0) edge(prev_d, o, kPairWhole, none);
    edge(po, g, kPairWhole, none);
    edge(pg, d, kPairWhole, none);
    edge(po, d, kPairWhole, none);
    prev_d = pub(d, none);
  }
  const int lm = 6 * L, am = lm + 1;
  edge(prev_d, lm, kPairWhole, none);
  edge(pub(lm, none), am, kPairWhole, none);
}

void balance_attention(const std::vector<GraphOp>& ops, const std::vector<int32_t>& kv_len, int splits, Plan* out) {
  Plan& P = *out;
  const int C = P.num_cus, T = P.num_tasks;
  auto rows = [&](int t) {
    int lo, hi;
    split_range(kv_len[P.tasks[t][1]], splits, P.tasks[t][3], &lo, &hi);
    return hi - lo;
  };
  std::map<int, std::vector<long>> load;
  for (int t = 0; t < T;) {
    const int o = P.tasks[t][0];
    if (ops[o].opcode != kAttn) {
      ++t;
      continue;
    }
    int e = t + 1;
    while (e < T && P.tasks[e][0] == o && P.task_wait[e] == P.task_wait[t] && P.task_wait2[e] == P.task_wait2[t]) ++e;
    auto& ld = load[o];
    if (ld.empty()) ld.assign(C, 0);
    std::vector<int> order;
    for (int u = t; u < e; ++u) order.push_back(u);
    std::stable_sort(order.begin(), order.end(), [&](int u, int v) { return rows(u) > rows(v); });
    std::vector<int> free_pos(order.size()), from(e - t);
    for (int k = 0; k < e - t; ++k) free_pos[k] = t + k;
    for (int u : order) {
      size_t best = 0;
      for (size_t k = 1; k < free_pos.size(); ++k) {
        const int v = free_pos[k], b = free_pos[best];
        if (ld[v % C] < ld[b % C] || (ld[v % C] == ld[b % C] && v < b)) best = k;
      }
      const int pos = free_pos[best];
      free_pos.erase(free_pos.begin() + best);
      from[pos - t] = u;
      ld[pos % C] += rows(u);
    }
    std::vector<std::array<int, 4>> tk(P.tasks.begin() + t, P.tasks.begin() + e);
    std::vector<int32_t> tr(P.task_trigger.begin() + t, P.task_trigger.begin() + e),
        tr2(P.task_trigger2.begin() + t, P.task_trigger2.begin() + e);
    std::vector<std::array<int32_t, 2>> sp;
    if (!P.sig_pub.empty()) sp.assign(P.sig_pub.begin() + t, P.sig_pub.begin() + e);
    for (int pos = t; pos < e; ++pos) {
      const int k = from[pos - t] - t;
      P.tasks[pos] = tk[k];
      P.task_trigger[pos] = tr[k];
      P.task_trigger2[pos] = tr2[k];
      if (!sp.empty()) P.sig_pub[pos] = sp[k];
    }
    t = e;
  }
  encode(ops, &kv_len, &P);
}

void resolve_opts(const ModelShape& m, const std::vector<int32_t>& kv_len, ModelOpts* o) {
  if (!o->gemv_rows) o->gemv_rows = std::max(4, std::min(16, 32768 / m.hidden));
  if (!o->gateup_outs) o->gateup_outs = std::max(1, o->gemv_rows / 2);
  // batch 1: a down tile is held in the compute waves' registers (64 KiB of
  // weights); batched: read from the 128 KiB page ring, which it may fill (more
  // rows per tile, fewer re-reads of the sequences' activations)
  if (!o->down_rows) o->down_rows = std::max(1, std::min(16, (kv_len.size() == 1 ? 32768 : 65536) / m.ffn));
  if (!o->lm_rows) o->lm_rows = o->gemv_rows;
  if (!o->attn_splits) {
    int n = *std::max_element(kv_len.begin(), kv_len.end()) + 1;
    int S = std::max(1, std::min(32, ceil_div(n, 64)));
    // no more splits than give about two tasks per compute unit over all
    // (sequence, kv head) pairs: every split pays its own q/k/v loads
    const int pairs = (int)kv_len.size() * m.n_kv_heads;
    S = std::min(S, std::max(1, ceil_div(2L * o->num_cus, pairs)));
    // one split's K and V rows within 64 KiB.  While the tasks still fit on the
    // compute units at one each, an eighth of the units are left without one
    // (their rings prefetch the FFN weights through the attention chain), and
    // a split may take the page ring less one 64 KiB tile (9 pages of 16 KiB
    // at batch 1, 8 above): one more split would put a second attention task
    // on some units, which costs the chain more than a larger tile costs the
    // ring.  Batched head_dim-64 tasks stream their rows through the ring and
    // take no cap.
    const bool streams = kv_len.size() > 1 && m.head_dim == 64;
    long cap = 65536;
    if ((long)pairs * S <= o->num_cus) {
      while (S > 1 && (long)pairs * S * 8 > 7L * o->num_cus) --S;
      cap = (kv_len.size() == 1 ? 9L : 8L) * 16384 - 65536;
    }
    while (!streams && (long)ceil_div(n, S) * m.head_dim * 4 > cap) ++S;
    o->attn_splits = S;
  }
}

std::string model_graph(const ModelShape& m, int batch, const std::vector<int32_t>& kv_len, const ModelOpts& o,
                        std::vector<GraphOp>* ops_out, std::vector<GraphEdge>* edges_out) {
  const int H = m.hidden, nq = m.n_q_heads, nkv = m.n_kv_heads, hd = m.head_dim, F = m.ffn, V = m.vocab;
  const int L = m.n_layers, B = batch;
  const int hpg = nq / nkv, RPG = (hpg + 2) * hd;
  const int R = o.gemv_rows, GU = o.gateup_outs, DR = o.down_rows, LR = o.lm_rows, S = o.attn_splits;
  if (R <= 0 || GU <= 0 || DR <= 0 || LR <= 0 || S <= 0) return "tile options must be positive";
  if (RPG % R || hd % R) return "gemv_rows must divide head_dim";
  const int T_qkv = RPG / R, T_o = ceil_div(H, R), T_f = ceil_div(F, GU), T_d = ceil_div(H, DR),
            T_v = ceil_div(V, LR);
  const int spec = B > 4 ? 1 : 0;
  auto& ops = *ops_out;
  auto& edges = *edges_out;
  ops.clear();
  edges.clear();
  auto add = [&](int opcode, std::array<int, 3> grid, int layer, int sp, std::array<int, 8> p) {
    GraphOp op;
    op.opcode = opcode;
    op.kind = opcode;
    op.grid = grid;
    op.layer = layer;
    op.spec = sp;
    op.p = p;
    ops.push_back(op);
    return (int)ops.size() - 1;
  };
  auto edge = [&](int p, int c, std::array<int, 3> om, std::array<int, 3> im, std::array<int, 4> ext,
                  std::array<int, 4> pt, std::array<int, 4> ct) {
    GraphEdge e;
    e.prod = p;
    e.cons = c;
    e.out_map = om;
    e.in_map = im;
    e.has_extent = true;
    e.extent = ext;
    e.ptile = pt;
    e.ctile = ct;
    edges.push_back(e);
  };
  const std::array<int, 3> none{{-1, -1, -1}};
  int prev_down = -1;
  for (int l = 0; l < L; ++l) {
    int q = add(kQkv, {{nkv, T_qkv, 1}}, l, spec, {{R}});
    int a = add(kAttn, {{B, nkv, S}}, l, 0, {{S}});
    int c = add(kCombine, {{B, nkv, 1}}, l, 0, {{S}});
    int op = add(kOproj, {{T_o, 1, 1}}, l, spec, {{R, H}});
    int g = add(kGateUp, {{T_f, 1, 1}}, l, spec, {{GU, F}});
    int d = add(kDown, {{T_d, 1, 1}}, l, spec, {{DR, H, F}});
    if (prev_down >= 0) edge(prev_down, q, {{1, -1, -1}}, none, {{B, H, 1, 1}}, {{1, DR, 1, 1}}, {{1, H, 1, 1}});
    edge(q, a, {{1, 2, -1}}, {{0, 1, -1}}, {{B, nkv, RPG, 1}}, {{B, 1, R, 1}}, {{1, 1, RPG, 1}});
    edge(a, c, {{0, 1, 2}}, {{0, 1, -1}}, {{B, nkv, S, 1}}, {{1, 1, 1, 1}}, {{1, 1, S, 1}});
    edge(c, op, {{0, 1, -1}}, none, {{B, nkv, 1, 1}}, {{1, 1, 1, 1}}, {{B, nkv, 1, 1}});
    if (prev_down >= 0) edge(prev_down, op, {{1, -1, -1}}, none, {{B, H, 1, 1}}, {{1, DR, 1, 1}}, {{1, H, 1, 1}});
    edge(op, g, {{1, -1, -1}}, none, {{B, H, 1, 1}}, {{1, R, 1, 1}}, {{1, H, 1, 1}});
    edge(op, d, {{1, -1, -1}}, none, {{B, H, 1, 1}}, {{1, R, 1, 1}}, {{1, H, 1, 1}});
    edge(g, d, {{1, -1, -1}}, none, {{B, F, 1, 1}}, {{1, GU, 1, 1}}, {{1, F, 1, 1}});
    prev_down = d;
  }
  int lm = add(kLmHead, {{T_v, 1, 1}}, L, spec, {{LR, V}});
  int am = add(kArgmax, {{B, 1, 1}}, L, 0, {{T_v}});
  edge(prev_down, lm, {{1, -1, -1}}, none, {{B, H, 1, 1}}, {{1, DR, 1, 1}}, {{1, H, 1, 1}});
  edge(lm, am, {{1, -1, -1}}, {{0, -1, -1}}, {{B, T_v, 1, 1}}, {{B, 1, 1, 1}}, {{1, T_v, 1, 1}});
  return "";
}

}  // namespace mk

namespace mk {

// GLM-style pre-attention path (MegaRTP article, section 4): A0 and the q-path
// norm work one token row per task; the fp8 GEMMs are cut into 16-row output
// tiles; QKV-B's rope dims come in tiles that pair 8 rows of the first half with
// the 8 rows half the rope width further on.
std::string glm_graph(const GlmShape& g, int M, std::vector<GraphOp>* ops_out, std::vector<GraphEdge>* edges_out) {
  const int R = kGlmRows, nope = g.head_dim - g.rope_dim;
  const int Na = g.q_lora + g.kv_lora + g.rope_dim, Niq = g.n_idx_heads * g.idx_head_dim;
  if (nope <= 0 || nope % R || g.rope_dim % R) return "nope and rope dims must be positive multiples of 16";
  auto& ops = *ops_out;
  auto& edges = *edges_out;
  ops.clear();
  edges.clear();
  auto add = [&](int opcode, std::array<int, 3> grid, std::array<int, 8> p) {
    GraphOp op;
    op.opcode = opcode;
    op.kind = opcode;
    op.grid = grid;
    op.p = p;
    ops.push_back(op);
    return (int)ops.size() - 1;
  };
  auto edge = [&](int p, int c, std::array<int, 3> om, std::array<int, 3> im, std::array<int, 4> ext,
                  std::array<int, 4> pt, std::array<int, 4> ct) {
    GraphEdge e;
    e.prod = p;
    e.cons = c;
    e.out_map = om;
    e.in_map = im;
    e.has_extent = true;
    e.extent = ext;
    e.ptile = pt;
    e.ctile = ct;
    edges.push_back(e);
  };
  const std::array<int, 3> none{{-1, -1, -1}}, d0{{0, -1, -1}}, d1{{1, -1, -1}};
  const int a0 = add(kGA0, {{M, 1, 1}}, {{}});
  const int qa = add(kGQkva, {{ceil_div(Na, R), 1, 1}}, {{Na}});
  // the head gate as K-split partial tiles (one 128-column block per compute
  // wave) and a reduce op that adds the partials of each row tile in split
  // order: the MegaRTP article's tile_reduce pairing (section 4, "TaskGraph")
  const int nkb = g.hidden / 128, gsplits = ceil_div(nkb, kGateBlocks), Tg = ceil_div(g.n_gate, R);
  const int ga = add(kGGate, {{Tg, gsplits, 1}}, {{g.n_gate, nkb}});
  const int ik = add(kGIdxk, {{ceil_div(g.idx_head_dim, R), 1, 1}}, {{g.idx_head_dim}});
  const int gr = add(kGGateRed, {{Tg, 1, 1}}, {{g.n_gate, gsplits}});
  const int qn = add(kGQaNorm, {{M, 1, 1}}, {{}});
  const int qb = add(kGQkvb, {{g.n_heads, (nope + g.rope_dim) / R, 1}}, {{g.head_dim, nope, g.rope_dim}});
  const int iq = add(kGIdxq, {{ceil_div(Niq, R), 1, 1}}, {{Niq}});
  for (int c : {qa, ga, ik}) edge(a0, c, d0, none, {{M, g.hidden, 1, 1}}, {{1, g.hidden, 1, 1}}, {{M, g.hidden, 1, 1}});
  edge(ga, gr, d1, d1, {{M, g.n_gate, 1, 1}}, {{M, R, 1, 1}}, {{M, R, 1, 1}});
  edge(qa, qn, d1, d0, {{M, Na, 1, 1}}, {{M, R, 1, 1}}, {{1, Na, 1, 1}});
  for (int c : {qb, iq}) edge(qn, c, d0, none, {{M, g.q_lora, 1, 1}}, {{1, g.q_lora, 1, 1}}, {{M, g.q_lora, 1, 1}});
  return "";
}

}  // namespace mk
