// Dynamic (confidence-ranked) candidate tree on gfx950.
//
// Sources: "Multi-Token Prediction: Draft-Model-Free Speculative Decoding", section "2. EAGLE &
// EAGLE-2: Feature-Level Autoregression" (the tree follows the candidates' confidence: deeper
// where the predictions are sure, wider where they are not) and "Production Deployment
// Guidelines", "Dynamic Tree Depth Tuning"; "Medusa Explained: Multi-Head Speculative Decoding
// Guide", "1. Combinatorial Tree Construction" (head k proposes the candidates of depth k).
//
// A node is a path of candidate ranks (r_1 .. r_d), one per head, scored by its joint
// log-probability sum_k log p_k(r_k) (log-probabilities clamped at 0, so no path outscores its
// prefix).  The tree is the N best paths: higher score first, then smaller depth, then smaller
// ranks from the first head on.  Nodes are laid out breadth first with the children of a node
// in rank order, which is the order of (depth, rank tuple).
//
// One wave per sequence selects the N paths best-first: the frontier holds, for every selected
// path, its first child and its next sibling (both score no higher than it), so the best
// frontier entry is always the next path in the order.  Each round is a wave-wide arg-best over
// the frontier (at most N + 1 entries in LDS).  For N <= 64 the frontier is instead kept sorted
// across the lanes, one entry per lane: the best entry is lane 0's, and a round shifts it out
// and inserts the (at most two) new entries at their ranks (a ballot count, then a one-lane
// shift of the lanes behind), with no reduction and no LDS round trip.  An entry ranked at or
// beyond the number of picks still to make can never be picked (every entry ahead of it is
// smaller and is picked first), so 64 lanes hold every entry that matters.  The (depth, ranks)
// key is packed in 64 bits: depth in the top 4 bits, the rank at depth d in bits
// [60 - 4d, 64 - 4d), so depth <= 15 and ranks < 16.

#include <algorithm>

#include "mv_device.h"
#include "mv_host.h"

namespace mv {
namespace {

constexpr int kDynMaxDepth = 15;
constexpr int kDynFrontier = MV_MAX_NODES + 1;

struct DynParams {
  int B, D, s_max, N, W;
  int s[kDynMaxDepth];
  const int32_t* ids;   // [B, D, s_max]
  const float* vals;    // [B, D, s_max]
  const float* lse;     // [B, D] or null
  int32_t* parents;     // [B, N]
  int32_t* depth;       // [B, N]
  int32_t* tokens;      // [B, N]
  uint32_t* anc;        // [B, N, W]
  float* logp;          // [B, N] or null
  int32_t* status;
};

// Selection order as one unsigned 128-bit key (A, K), smallest first: A orders the score from
// high to low (the usual order-preserving map of a double's bits, inverted; -0 counts as +0),
// K is the (depth, ranks) key.
__device__ __forceinline__ uint64_t score_key(double s) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(s + 0.0));
  const uint64_t m = (u >> 63) ? ~u : (u | (static_cast<uint64_t>(1) << 63));
  return ~m;
}

struct SelKey {
  uint64_t a, k;
  uint32_t j;  // frontier slot
};

__device__ __forceinline__ void take_if_less(SelKey& x, uint64_t oa, uint64_t ok, uint32_t oj) {
  const bool c = (oa < x.a) | ((oa == x.a) & (ok < x.k));  // selects, not a branch per lane
  x.a = c ? oa : x.a;
  x.k = c ? ok : x.k;
  x.j = c ? oj : x.j;
}

template <int CTRL>
__device__ __forceinline__ void dpp_step(SelKey& x) {
  const uint64_t oa = (static_cast<uint64_t>(dpp_u32<CTRL>(static_cast<uint32_t>(x.a >> 32))) << 32) |
                      dpp_u32<CTRL>(static_cast<uint32_t>(x.a));
  const uint64_t ok = (static_cast<uint64_t>(dpp_u32<CTRL>(static_cast<uint32_t>(x.k >> 32))) << 32) |
                      dpp_u32<CTRL>(static_cast<uint32_t>(x.k));
  take_if_less(x, oa, ok, dpp_u32<CTRL>(x.j));
}

template <typename Swap>
__device__ __forceinline__ void swap_step(SelKey& x, Swap swap) {
  const LanePair ah = swap(static_cast<uint32_t>(x.a >> 32)), al = swap(static_cast<uint32_t>(x.a));
  const LanePair kh = swap(static_cast<uint32_t>(x.k >> 32)), kl = swap(static_cast<uint32_t>(x.k));
  const LanePair jj = swap(x.j);
  x = {(static_cast<uint64_t>(ah.a) << 32) | al.a, (static_cast<uint64_t>(kh.a) << 32) | kl.a, jj.a};
  take_if_less(x, (static_cast<uint64_t>(ah.b) << 32) | al.b, (static_cast<uint64_t>(kh.b) << 32) | kl.b,
               jj.b);
}

// Wave-wide minimum of distinct keys: a butterfly of lane exchanges; every lane ends with it.
__device__ __forceinline__ void wave_min_key(SelKey& x) {
  dpp_step<kDppXor1>(x);
  dpp_step<kDppXor2>(x);
  dpp_step<kDppHalfMirror>(x);
  dpp_step<kDppMirror>(x);
  swap_step(x, [](uint32_t v) { return swap16(v); });
  swap_step(x, [](uint32_t v) { return swap32(v); });
}

__device__ __forceinline__ int key_depth(uint64_t k) { return static_cast<int>(k >> 60); }
__device__ __forceinline__ int key_rank(uint64_t k, int d) {
  return static_cast<int>((k >> (60 - 4 * d)) & 15u);
}

// whole-wave one-lane shifts (DPP wave_shr:1 / wave_shl:1): lane i takes lane i - 1 (i + 1);
// the lane without a source keeps `fill`
__device__ __forceinline__ uint32_t wave_shr1(uint32_t v, uint32_t fill) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(fill), static_cast<int>(v), 0x138, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t wave_shl1(uint32_t v, uint32_t fill) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(fill), static_cast<int>(v), 0x130, 0xF, 0xF, false));
}

// One frontier entry per lane (sorted mode): selection key (a, k), score, parent's score,
// parent's selection index.  An empty entry has a = k = ~0 and sorts last.
struct DynEntry {
  uint64_t a, k;
  double sc, ps;
  int par;
};

template <bool LEFT>
__device__ __forceinline__ DynEntry wave_shift(const DynEntry& e) {
  auto sh = [](uint32_t v, uint32_t fill) { return LEFT ? wave_shl1(v, fill) : wave_shr1(v, fill); };
  auto sh64 = [&](uint64_t v, uint64_t fill) {
    return (static_cast<uint64_t>(sh(static_cast<uint32_t>(v >> 32), static_cast<uint32_t>(fill >> 32))) << 32) |
           sh(static_cast<uint32_t>(v), static_cast<uint32_t>(fill));
  };
  auto shd = [&](double v) {
    return __longlong_as_double(static_cast<long long>(sh64(static_cast<uint64_t>(__double_as_longlong(v)), 0)));
  };
  return {sh64(e.a, ~static_cast<uint64_t>(0)), sh64(e.k, ~static_cast<uint64_t>(0)), shd(e.sc), shd(e.ps),
          static_cast<int>(sh(static_cast<uint32_t>(e.par), 0xffffffffu))};
}

__device__ __forceinline__ DynEntry pick(bool f, const DynEntry& u, const DynEntry& v) {
  return {f ? u.a : v.a, f ? u.k : v.k, f ? u.sc : v.sc, f ? u.ps : v.ps, f ? u.par : v.par};
}

__device__ __forceinline__ uint64_t first_lane_u64(uint64_t v) {
  return (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v >> 32)))) << 32) |
         static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v)));
}

template <bool SORTED>
__global__ __launch_bounds__(64) void dynamic_tree_kernel(const DynParams p) {
  __shared__ double lp[kDynMaxDepth][MV_MAX_TOPK];
  __shared__ double fs[kDynFrontier], fps[kDynFrontier];  // score, parent's score
  __shared__ uint64_t fk[kDynFrontier];
  __shared__ int fpar[kDynFrontier];                       // parent's selection index
  __shared__ double ss[MV_MAX_NODES];
  __shared__ uint64_t sk[MV_MAX_NODES];
  __shared__ int spar[MV_MAX_NODES], spos[MV_MAX_NODES];
  __shared__ uint32_t mrow[MV_MAX_NODES][(MV_MAX_NODES + 31) / 32];
  __shared__ int fcount, nsel;
  const int b = blockIdx.x, lane = threadIdx.x;
  const int D = p.D, N = p.N;
  for (int i = lane; i < D * MV_MAX_TOPK; i += 64) {
    const int d = i / MV_MAX_TOPK, r = i % MV_MAX_TOPK;
    double v = 0.0;
    if (r < p.s[d]) {
      const size_t o = (static_cast<size_t>(b) * D + d) * p.s_max + r;
      v = static_cast<double>(p.vals[o]);
      if (p.lse) v -= static_cast<double>(p.lse[static_cast<size_t>(b) * D + d]);
      v = fmin(0.0, v);
    }
    lp[d][r] = v;
  }
  __syncthreads();
  int ns_sorted = 0;
  if constexpr (SORTED) {
    DynEntry e = {~static_cast<uint64_t>(0), ~static_cast<uint64_t>(0), 0.0, 0.0, -1};
    if (lane == 0) {
      e.sc = lp[0][0];
      e.k = static_cast<uint64_t>(1) << 60;  // depth 1, rank 0
      e.a = score_key(e.sc);
    }
    // put x at its rank: the lanes behind it move back by one lane
    auto insert = [&](const DynEntry& x) {
      const bool lt = (e.a < x.a) | ((e.a == x.a) & (e.k < x.k));
      const int pos = __popcll(__ballot(lt));
      e = pick(lane == pos, x, pick(lane > pos, wave_shift<false>(e), e));
    };
    for (int n = 0; n < N; ++n) {
      const uint64_t wa = first_lane_u64(e.a), wk = first_lane_u64(e.k);
      // an empty frontier means every path is in the tree; the host has checked that there
      // are at least N paths, so this only guards the loops below
      if (wa == ~static_cast<uint64_t>(0) && wk == ~static_cast<uint64_t>(0)) break;
      const double wsc = __longlong_as_double(static_cast<long long>(first_lane_u64(static_cast<uint64_t>(__double_as_longlong(e.sc)))));
      const double wps = __longlong_as_double(static_cast<long long>(first_lane_u64(static_cast<uint64_t>(__double_as_longlong(e.ps)))));
      const int wpar = __builtin_amdgcn_readfirstlane(e.par);
      const int d = key_depth(wk), r = key_rank(wk, d);
      if (lane == 0) {
        ss[n] = wsc;
        sk[n] = wk;
        spar[n] = wpar;
      }
      e = wave_shift<true>(e);  // the chosen entry leaves
      if (d < D) {  // its first child
        const double c = wsc + lp[d][0];
        insert({score_key(c), (wk & ((static_cast<uint64_t>(1) << 60) - 1)) | (static_cast<uint64_t>(d + 1) << 60),
                c, wsc, n});
      }
      if (r + 1 < p.s[d - 1]) {  // its next sibling
        const double c = wps + lp[d - 1][r + 1];
        insert({score_key(c), wk + (static_cast<uint64_t>(1) << (60 - 4 * d)), c, wps, wpar});
      }
      ns_sorted = n + 1;
    }
    __syncthreads();
  } else {
    if (lane == 0) {
      fs[0] = lp[0][0];
      fps[0] = 0.0;
      fk[0] = static_cast<uint64_t>(1) << 60;  // depth 1, rank 0
      fpar[0] = -1;
      fcount = 1;
      nsel = 0;
    }
    __syncthreads();
    for (int n = 0; n < N; ++n) {
      const int fc = fcount;
      SelKey best = {~static_cast<uint64_t>(0), ~static_cast<uint64_t>(0), 0xffffffffu};
      for (int j = lane; j < fc; j += 64) take_if_less(best, score_key(fs[j]), fk[j], j);
      wave_min_key(best);  // keys are distinct: every lane ends with the same entry
      // an empty frontier means every path is in the tree; the host has checked that there
      // are at least N paths, so this only guards the loops below
      if (best.j == 0xffffffffu) break;
      const int bj = static_cast<int>(best.j);
      const uint64_t bk = best.k;
      if (lane == 0) {
        const double bs = fs[bj];
        const int d = key_depth(bk), r = key_rank(bk, d);
        const int par = fpar[bj];
        const double psc = fps[bj];
        ss[n] = bs;
        sk[n] = bk;
        spar[n] = par;
        int cnt = fc;
        // first child replaces the chosen entry; without one the last entry moves into its slot
        if (d < D) {
          fs[bj] = bs + lp[d][0];
          fps[bj] = bs;
          fk[bj] = (bk & ((static_cast<uint64_t>(1) << 60) - 1)) | (static_cast<uint64_t>(d + 1) << 60);
          fpar[bj] = n;
        } else {
          --cnt;
          if (bj != cnt) {
            fs[bj] = fs[cnt];
            fps[bj] = fps[cnt];
            fk[bj] = fk[cnt];
            fpar[bj] = fpar[cnt];
          }
        }
        if (r + 1 < p.s[d - 1]) {  // next sibling
          fs[cnt] = psc + lp[d - 1][r + 1];
          fps[cnt] = psc;
          fk[cnt] = bk + (static_cast<uint64_t>(1) << (60 - 4 * d));
          fpar[cnt] = par;
          ++cnt;
        }
        fcount = cnt;
        nsel = n + 1;
      }
      __syncthreads();
    }
  }
  const int ns = SORTED ? ns_sorted : nsel;
  // breadth-first position = rank of (depth, ranks) among the selected keys
  for (int i = lane; i < ns; i += 64) {
    const uint64_t k = sk[i];
    int pos = 0;
    for (int m = 0; m < ns; ++m) pos += sk[m] < k;
    spos[i] = pos;
  }
  __syncthreads();
  int flags = ns < N ? MV_DEV_BAD_RANK : 0;
  const int W = p.W;
  for (int i = lane; i < N * W; i += 64) mrow[i / W][i % W] = 0u;
  for (int i = lane + ns; i < N; i += 64) {  // unreachable (see above): empty nodes
    const size_t q = static_cast<size_t>(b) * N + i;
    p.parents[q] = -1;
    p.depth[q] = 0;
    p.tokens[q] = -1;
    if (p.logp) p.logp[q] = 0.f;
  }
  __syncthreads();
  for (int i = lane; i < ns; i += 64) {
    const int o = spos[i];
    const uint64_t k = sk[i];
    const int d = key_depth(k), r = key_rank(k, d);
    for (int m = i; m >= 0; m = spar[m]) mrow[o][spos[m] >> 5] |= 1u << (spos[m] & 31);
    const size_t q = static_cast<size_t>(b) * N + o;
    p.parents[q] = spar[i] < 0 ? -1 : spos[spar[i]];
    p.depth[q] = d;
    const int tok = p.ids[(static_cast<size_t>(b) * D + d - 1) * p.s_max + r];
    if (tok < 0) flags |= MV_DEV_BAD_RANK;
    p.tokens[q] = tok;
    if (p.logp) p.logp[q] = static_cast<float>(ss[i]);
  }
  __syncthreads();
  for (int i = lane; i < N * W; i += 64)
    p.anc[static_cast<size_t>(b) * N * W + i] = mrow[i / W][i % W];
  if (flags && p.status) atomicOr(p.status, flags);
}

}  // namespace
}  // namespace mv

using namespace mv;

extern "C" {

MV_API int mv_build_dynamic_tree(int B, int D, int s_max, const int* s_per_depth, int N,
                                 const int32_t* cand_ids, const float* cand_vals,
                                 const float* cand_lse, int32_t* parents, int32_t* depth,
                                 int32_t* node_tokens, uint32_t* anc_mask, float* node_logp,
                                 int32_t* dev_status, void* stream) {
  if (B < 1 || D < 1 || s_max < 1 || N < 1) return MV_ERR_INVALID_ARG;
  if (!cand_ids || !cand_vals || !parents || !depth || !node_tokens || !anc_mask)
    return MV_ERR_INVALID_ARG;
  if (D > kDynMaxDepth || s_max > MV_MAX_TOPK || N > MV_MAX_NODES) return MV_ERR_UNSUPPORTED;
  DynParams p{};
  // paths available: sum over depths of the product of the widths so far (saturating at N)
  long long total = 0, prod = 1;
  for (int d = 0; d < D; ++d) {
    const int s = s_per_depth ? s_per_depth[d] : s_max;
    if (s < 1 || s > s_max) return MV_ERR_INVALID_ARG;
    p.s[d] = s;
    prod = std::min<long long>(prod * s, N);
    total = std::min<long long>(total + prod, N);
  }
  if (total < N) return MV_ERR_INVALID_ARG;
  p.B = B; p.D = D; p.s_max = s_max; p.N = N; p.W = (N + 31) / 32;
  p.ids = cand_ids; p.vals = cand_vals; p.lse = cand_lse;
  p.parents = parents; p.depth = depth; p.tokens = node_tokens; p.anc = anc_mask;
  p.logp = node_logp; p.status = dev_status;
  if (N <= 64) dynamic_tree_kernel<true><<<B, 64, 0, as_stream(stream)>>>(p);
  else dynamic_tree_kernel<false><<<B, 64, 0, as_stream(stream)>>>(p);
  return launch_status();
}

}  // extern "C"
