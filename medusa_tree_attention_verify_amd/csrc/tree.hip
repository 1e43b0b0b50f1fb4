// Candidate-tree assembly on gfx950: parent array -> depth, sibling rank, ancestor-or-self
// bitmask and the token of every node.
//
// Sources: "Multi-Token Prediction: Draft-Model-Free Speculative Decoding", the verification
// engine's tree format (a parent array; -1 marks a root that hangs off the prefix) and "The
// 2D Tree Attention Mask" (a node sees its ancestors and itself); "Medusa Explained:
// Multi-Head Speculative Decoding Guide", "1. Combinatorial Tree Construction" (the depth-k
// nodes are the top-s_k tokens of the depth-k head).  Each thread collects its node's
// ancestor-or-self set by following parent links until it leaves the tree.
//
// One workgroup, one thread per node.  Every walk checks parents[c] in [-1, c), so it moves
// to strictly smaller indices and ends within N steps even on a malformed array.

#include "mv_device.h"
#include "mv_host.h"

namespace mv {
namespace {

struct DepthWidths {
  int s[MV_MAX_DEPTH];
};

__global__ __launch_bounds__(MV_MAX_NODES) void tree_build_kernel(
    int N, const int32_t* __restrict__ parents, int B, int D, int s_max, DepthWidths sw,
    const int32_t* __restrict__ cand, uint32_t* __restrict__ anc, int32_t* __restrict__ depth_out,
    int32_t* __restrict__ tokens, int32_t* __restrict__ status) {
  __shared__ int par[MV_MAX_NODES];
  const int i = threadIdx.x;
  if (i < N) par[i] = parents[i];
  __syncthreads();
  if (i >= N) return;
  const int W = (N + 31) >> 5;
  uint32_t bits[MV_MAX_NODES / 32];
#pragma unroll
  for (int w = 0; w < MV_MAX_NODES / 32; ++w) bits[w] = 0u;
  int flags = 0, dep = 0, c = i;
  while (c != -1) {
#pragma unroll
    for (int w = 0; w < MV_MAX_NODES / 32; ++w)
      if (w == (c >> 5)) bits[w] |= 1u << (c & 31);
    ++dep;
    const int nx = par[c];
    if (nx < -1 || nx >= c) { flags |= MV_DEV_BAD_PARENT; break; }
    c = nx;
  }
  if (flags) {  // malformed: the node sees only itself
#pragma unroll
    for (int w = 0; w < MV_MAX_NODES / 32; ++w) bits[w] = (w == (i >> 5)) ? (1u << (i & 31)) : 0u;
    dep = 1;
  }
#pragma unroll
  for (int w = 0; w < MV_MAX_NODES / 32; ++w)
    if (w < W) anc[static_cast<size_t>(i) * W + w] = bits[w];
  if (depth_out) depth_out[i] = dep;
  if (cand) {
    const int p = par[i];
    int rank = 0;
    for (int j = 0; j < i; ++j) rank += (par[j] == p);
    int tok_ok = !flags;
    if (dep > D) { flags |= MV_DEV_TOO_DEEP; tok_ok = 0; }
    else if (rank >= sw.s[dep - 1]) { flags |= MV_DEV_BAD_RANK; tok_ok = 0; }
    for (int b = 0; b < B; ++b)
      tokens[static_cast<size_t>(b) * N + i] =
          tok_ok ? cand[(static_cast<size_t>(b) * D + (dep - 1)) * s_max + rank] : -1;
  }
  if (flags && status) atomicOr(status, flags);
}

}  // namespace
}  // namespace mv

using namespace mv;

extern "C" MV_API int mv_build_tree_mask(int N, const int32_t* parents, int B, int D, int s_max,
                                         const int* s_per_depth, const int32_t* cand,
                                         uint32_t* anc_mask, int32_t* depth,
                                         int32_t* node_tokens, int32_t* dev_status,
                                         void* stream) {
  if (N < 1 || !parents || !anc_mask) return MV_ERR_INVALID_ARG;
  if (N > MV_MAX_NODES) return MV_ERR_UNSUPPORTED;
  DepthWidths sw{};
  if (cand) {
    if (!node_tokens || B < 1 || D < 1 || s_max < 1) return MV_ERR_INVALID_ARG;
    if (D > MV_MAX_DEPTH || s_max > MV_MAX_TOPK) return MV_ERR_UNSUPPORTED;
    for (int k = 0; k < D; ++k) {
      sw.s[k] = s_per_depth ? s_per_depth[k] : s_max;
      if (sw.s[k] < 1 || sw.s[k] > s_max) return MV_ERR_INVALID_ARG;
    }
  } else {
    B = 0;
    D = MV_MAX_DEPTH;
  }
  tree_build_kernel<<<1, MV_MAX_NODES, 0, as_stream(stream)>>>(N, parents, B, D, s_max, sw, cand,
                                                                anc_mask, depth, node_tokens,
                                                                dev_status);
  return launch_status();
}
