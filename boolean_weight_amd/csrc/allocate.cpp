// Kernels per weight under a bit budget, on the host.
//
// "Highly Efficient and Effective LLMs with Multi-Boolean Architectures",
// Italian gist.science summary, section "D. Allocazione Automatica dei
// Kernel": the number of kernels of each weight is allocated for an average
// bit budget, trading the residual approximation error against the weight's
// size.  (The importance term of that section needs data; every weight
// counts the same here.)
//
// Exact optimum by dynamic programming over the weights in order.  A partial
// allocation of weights 0..l is a state (bits used, exact error sum, K
// prefix).  A state is dropped when another one uses no more bits and has no
// larger error (on equal bits and error, the one whose prefix comes first in
// lexicographic order stays): appending the same K values to both keeps that
// order, because the error sums are exact.  So the surviving states always
// contain the allocation a search over every K vector would choose: least
// exact error, then fewest bits, then the first vector in lexicographic order.
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <vector>

#include "../../include/mbok.h"

namespace mbok {
namespace {

// Exact sum of nonnegative float64 values: a fixed-point integer of 36
// 64-bit limbs whose lowest bit is 2^-1127 (a double is mant * 2^(e - 53)
// with e >= -1073 and 53-bit mant, and below 2^1024, so every double lands
// at bit 0 or above, and sums of up to 2^150 values fit).
struct ExactSum {
  static constexpr int kLimbs = 36;
  static constexpr int kLowExp = -1127;
  uint64_t v[kLimbs] = {};

  void add(double x) {
    if (x == 0.0) return;
    int e = 0;
    const double f = std::frexp(x, &e);  // x = f * 2^e, 0.5 <= f < 1
    const uint64_t mant = (uint64_t)std::ldexp(f, 53);  // x = mant * 2^(e - 53)
    const int pos = e - 53 - kLowExp;
    int limb = pos / 64;
    const int sh = pos % 64;
    const unsigned __int128 t = (unsigned __int128)mant << sh;
    uint64_t carry = 0;
    uint64_t part[2] = {(uint64_t)t, (uint64_t)(t >> 64)};
    for (int p = 0; p < 2 || carry; ++p, ++limb) {
      const unsigned __int128 s =
          (unsigned __int128)v[limb] + (p < 2 ? part[p] : 0) + carry;
      v[limb] = (uint64_t)s;
      carry = (uint64_t)(s >> 64);
    }
  }
  void add(const ExactSum& o) {
    uint64_t carry = 0;
    for (int l = 0; l < kLimbs; ++l) {
      const unsigned __int128 s = (unsigned __int128)v[l] + o.v[l] + carry;
      v[l] = (uint64_t)s;
      carry = (uint64_t)(s >> 64);
    }
  }
  // -1, 0, +1
  int cmp(const ExactSum& o) const {
    for (int l = kLimbs - 1; l >= 0; --l)
      if (v[l] != o.v[l]) return v[l] < o.v[l] ? -1 : 1;
    return 0;
  }
};

// A partial allocation of weights 0..l: its bits, its exact error sum, and
// its K prefix as a link to the state of weights 0..l-1 it extends plus its
// own K.  `lex` is the rank of the prefix in lexicographic order among the
// states of the same length: prefixes compare as (rank of the parent prefix,
// K), so ties are broken without copying prefixes.
struct State {
  int64_t bits;
  ExactSum err;
  int32_t parent;
  int32_t lex;
  uint8_t K;
};

// (bits, error, prefix) ascending; plex = ranks of the parents' prefixes
bool state_less(const State& a, const State& b, const std::vector<int32_t>& plex) {
  if (a.bits != b.bits) return a.bits < b.bits;
  const int c = a.err.cmp(b.err);
  if (c != 0) return c < 0;
  if (a.parent != b.parent) return plex[a.parent] < plex[b.parent];
  return a.K < b.K;
}

constexpr size_t kMaxStates = size_t(1) << 22;

}  // namespace

int allocate_kernels(int L, const int64_t* sizes, const double* errors, int kmax, int64_t budget,
                     int32_t* K_out) {
  // suffix[l] = bits of K = 1 for weights l..L-1: the least the rest can use
  std::vector<int64_t> suffix(L + 1, 0);
  for (int l = L - 1; l >= 0; --l) suffix[l] = suffix[l + 1] + sizes[l];
  if (suffix[0] > budget) return MBOK_ERR_INFEASIBLE;
  std::vector<ExactSum> errs((size_t)L * kmax);
  for (size_t t = 0; t < errs.size(); ++t) errs[t].add(errors[t]);

  std::vector<State> front(1);
  front[0].bits = 0;
  front[0].parent = -1;
  front[0].lex = 0;
  front[0].K = 0;
  std::vector<State> cand;
  std::vector<int32_t> plex;
  std::vector<size_t> order;
  // links[l][i]: (parent index in front l-1, K) of state i of front l
  std::vector<std::vector<std::pair<int32_t, uint8_t>>> links(L);
  for (int l = 0; l < L; ++l) {
    cand.clear();
    plex.resize(front.size());
    for (size_t fi = 0; fi < front.size(); ++fi) {
      plex[fi] = front[fi].lex;
      const State& st = front[fi];
      for (int K = 1; K <= kmax; ++K) {
        const int64_t nb = st.bits + (int64_t)K * sizes[l];
        if (nb + suffix[l + 1] > budget) break;  // larger K only uses more
        State s;
        s.bits = nb;
        s.err = st.err;
        s.err.add(errs[(size_t)l * kmax + (K - 1)]);
        s.parent = (int32_t)fi;
        s.lex = 0;
        s.K = (uint8_t)K;
        cand.push_back(s);
      }
    }
    if (cand.size() > kMaxStates) return MBOK_ERR_UNSUPPORTED;
    order.resize(cand.size());
    for (size_t i = 0; i < order.size(); ++i) order[i] = i;
    std::sort(order.begin(), order.end(), [&](size_t a, size_t b) {
      return state_less(cand[a], cand[b], plex);
    });
    front.clear();
    for (size_t i : order) {
      // keep only states with a strictly smaller error than every kept one
      // (those use no more bits, or the same bits and come first)
      if (front.empty() || cand[i].err.cmp(front.back().err) < 0) front.push_back(cand[i]);
    }
    // lexicographic ranks of the kept prefixes: (parent's rank, K)
    order.resize(front.size());
    for (size_t i = 0; i < order.size(); ++i) order[i] = i;
    std::sort(order.begin(), order.end(), [&](size_t a, size_t b) {
      const State &x = front[a], &y = front[b];
      if (x.parent != y.parent) return plex[x.parent] < plex[y.parent];
      return x.K < y.K;
    });
    for (size_t r = 0; r < order.size(); ++r) front[order[r]].lex = (int32_t)r;
    links[l].resize(front.size());
    for (size_t i = 0; i < front.size(); ++i) links[l][i] = {front[i].parent, front[i].K};
  }
  // the front is ordered by bits with strictly falling error: the last state
  // has the least error, and no other state has that error
  int32_t at = (int32_t)front.size() - 1;
  for (int l = L - 1; l >= 0; --l) {
    K_out[l] = links[l][at].second;
    at = links[l][at].first;
  }
  return MBOK_OK;
}

}  // namespace mbok
