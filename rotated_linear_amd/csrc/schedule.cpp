// Host-side ordering of the pairs of each stage for bank-conflict-free LDS access.
//
// The pairs of one stage touch disjoint channels, so they may be processed in any
// order, and a pair (i, j, cos, sin) may be stored as (j, i, cos, -sin): both give
// x'_i = c x_i + s x_j and x'_j = c x_j - s x_i ("ParoQuant: pairwise rotations that
// survive deployment", section "A rotation small enough to execute", 2x2 equation).
// The kernels hand pair p to lane p mod 64 and keep channel c at LDS word c*R (R rows
// interleaved), so the bank a lane hits is set by c mod (banks / R). This file picks
// an order in which every aligned run of q consecutive pairs, for q = 64, 32, 16 and
// 8, has pairwise different first channels mod q and pairwise different second
// channels mod q. Then a wave's gather of x_i (or x_j) spreads evenly over the banks
// whatever R is.
//
// Construction (always succeeds when D % 128 == 0):
//   1. residues mod 64 form a multigraph with one edge per pair; every vertex has
//      even degree D/64, so walking closed trails orients the edges with equal in-
//      and out-degree everywhere (an Eulerian orientation); the tail of an edge
//      becomes the pair's first channel;
//   2. the oriented edges form a (D/128)-regular bipartite multigraph (first residue
//      -> second residue), which splits into D/128 perfect matchings (Hall); each
//      matching is a run of 64 pairs with distinct residues mod 64 on both sides;
//   3. a run of 2q pairs with distinct residues mod 2q is split into two runs of q
//      with distinct residues mod q: pairs sharing a first-channel class mod q, or a
//      second-channel class mod q, must be separated; those constraints form disjoint
//      even cycles, so a 2-colouring exists. Recurse down to q = 8.
// The input is canonicalised first (first channel < second channel, sorted), so the
// result depends only on the set of pairs, not on the order they were given in.
#include <algorithm>
#include <array>
#include <vector>

#include "paro_internal.h"

namespace paro {

namespace {

constexpr int Q = 64;

// Kuhn's augmenting-path perfect matching on a 64x64 bipartite support graph.
bool try_kuhn(int u, const std::array<std::array<int, Q>, Q>& cnt, std::array<int, Q>& match_r,
              std::array<char, Q>& seen) {
  for (int v = 0; v < Q; ++v) {
    if (cnt[u][v] <= 0 || seen[v]) continue;
    seen[v] = 1;
    if (match_r[v] < 0 || try_kuhn(match_r[v], cnt, match_r, seen)) {
      match_r[v] = u;
      return true;
    }
  }
  return false;
}

// Split `run` (2q pairs, distinct residues mod 2q on both sides) into two halves of q pairs
// with distinct residues mod q on both sides; recurse down to q = 8.
void split_run(std::vector<StagePair>& run, int q) {
  if (q < 8) return;
  const int n = int(run.size());  // == 2q
  std::vector<int> by_i(q, -1), by_j(q, -1), link_i(n), link_j(n);
  for (int p = 0; p < n; ++p) {
    const int ri = run[p].i % q, rj = run[p].j % q;
    if (by_i[ri] < 0) by_i[ri] = p; else { link_i[p] = by_i[ri]; link_i[by_i[ri]] = p; }
    if (by_j[rj] < 0) by_j[rj] = p; else { link_j[p] = by_j[rj]; link_j[by_j[rj]] = p; }
  }
  std::vector<int> colour(n, -1);
  for (int s = 0; s < n; ++s) {
    if (colour[s] >= 0) continue;
    // walk the alternating cycle s -i- a -j- b -i- ...
    int p = s, c = 0;
    bool use_i = true;
    while (colour[p] < 0) {
      colour[p] = c;
      p = use_i ? link_i[p] : link_j[p];
      use_i = !use_i;
      c ^= 1;
    }
  }
  std::vector<StagePair> lo, hi;
  lo.reserve(q);
  hi.reserve(q);
  for (int p = 0; p < n; ++p) (colour[p] ? hi : lo).push_back(run[p]);
  split_run(lo, q / 2);
  split_run(hi, q / 2);
  std::copy(lo.begin(), lo.end(), run.begin());
  std::copy(hi.begin(), hi.end(), run.begin() + q);
}

}  // namespace

bool schedule_stage(int D, std::vector<StagePair>& pairs) {
  const int P = D / 2;
  if (D % 128 != 0 || int(pairs.size()) != P) return false;
  // canonical form: first channel < second channel, sorted by first channel
  for (auto& pr : pairs)
    if (pr.i > pr.j) {
      std::swap(pr.i, pr.j);
      pr.s = -pr.s;
    }
  std::sort(pairs.begin(), pairs.end(), [](const StagePair& a, const StagePair& b) { return a.i < b.i; });

  // 1. Eulerian orientation of the residue multigraph
  std::vector<std::vector<int>> adj(Q);
  for (int p = 0; p < P; ++p) {
    adj[pairs[p].i % Q].push_back(p);
    if (pairs[p].j % Q != pairs[p].i % Q) adj[pairs[p].j % Q].push_back(p);
  }
  std::vector<char> used(P, 0);
  std::vector<size_t> ptr(Q, 0);
  for (int start = 0; start < Q; ++start) {
    int v = start;
    for (;;) {
      while (ptr[v] < adj[v].size() && used[adj[v][ptr[v]]]) ++ptr[v];
      if (ptr[v] == adj[v].size()) break;  // closed: all degrees are even
      const int p = adj[v][ptr[v]];
      used[p] = 1;
      StagePair& pr = pairs[p];
      if (pr.i % Q != v) {  // orient the edge away from v
        std::swap(pr.i, pr.j);
        pr.s = -pr.s;
      }
      v = pr.j % Q;
    }
  }
  // 2. decompose into perfect matchings of the residue bipartite multigraph
  std::array<std::array<int, Q>, Q> cnt{};
  std::vector<std::vector<int>> bucket(Q * Q);
  for (int p = 0; p < P; ++p) {
    const int a = pairs[p].i % Q, b = pairs[p].j % Q;
    ++cnt[a][b];
    bucket[a * Q + b].push_back(p);
  }
  std::vector<StagePair> out;
  out.reserve(P);
  const int rounds = P / Q;
  for (int r = 0; r < rounds; ++r) {
    std::array<int, Q> match_r;
    match_r.fill(-1);
    for (int u = 0; u < Q; ++u) {
      std::array<char, Q> seen{};
      if (!try_kuhn(u, cnt, match_r, seen)) return false;  // impossible for a regular graph
    }
    std::vector<StagePair> run;
    run.reserve(Q);
    for (int v = 0; v < Q; ++v) {
      const int u = match_r[v];
      --cnt[u][v];
      run.push_back(pairs[bucket[u * Q + v].back()]);
      bucket[u * Q + v].pop_back();
    }
    // 3. recursive halving for q = 32, 16, 8
    split_run(run, Q / 2);
    out.insert(out.end(), run.begin(), run.end());
  }
  pairs.swap(out);
  return true;
}

}  // namespace paro
