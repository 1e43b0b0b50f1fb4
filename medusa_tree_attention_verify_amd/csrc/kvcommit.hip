// Commit of the accepted path into the KV cache (the step after acceptance).
//
// Sources: "Multi-Token Prediction: Draft-Model-Free Speculative Decoding", "The 2D Tree
// Attention Mask" (the engine commits the longest accepted path; each node sees its ancestors,
// so a kept path is an ordinary causal continuation of the prefix) and "Production Deployment
// Guidelines" (the KV entries of unselected branches are culled); "Medusa Explained:
// Multi-Head Speculative Decoding Guide", "2. Single-Pass Tree Attention Verification" (the
// tree is verified after the prefix in one pass).
//
// The tree's K/V rows sit at cache rows [L_b, L_b + N) in node order.  Committing the accepted
// path path_nodes[b][0..len) moves row L_b + path_nodes[b][j] to row L_b + j for every KV head
// and then writes prefix_len[b] + len to prefix_out[b], so the next step sees prefix + accepted
// tokens as one contiguous causal prefix.  The copy is in place: a destination row can be a later source
// (path [1, 3] writes row L_b + 1 and reads it), so each workgroup stages all of its source
// rows in LDS before it writes any.  The new prefix lengths go to a separate buffer from the
// copy kernel itself; written in place they need a second launch, after every workgroup has
// read the old ones.

#include "mv_device.h"
#include "mv_host.h"

namespace mv {
namespace {

struct CommitParams {
  int B, Hkv, dh, L_cap, N, D, esz;  // esz: bytes per element
  char* k;
  char* v;
  const int32_t* prefix_len;
  int32_t* prefix_out;        // may equal prefix_len
  const int32_t* path_nodes;  // [B][D]
  const int32_t* accept_len;  // [B]
  int32_t* status;
};

constexpr int kCommitThreads = 256;
constexpr int kMaxRowBytes = 128 * 4;  // dh <= 128, fp32

// Number of rows to commit for sequence b, or 0 with the reason in *flags when the sequence's
// prefix or path is invalid.  Fills src[0..len) with the path's nodes when src is given.
__device__ int commit_len(const CommitParams& p, int b, int* flags, int* src) {
  const int L = p.prefix_len[b];
  const int len = p.accept_len[b];
  if (L < 0 || L + p.N > p.L_cap) {
    *flags |= MV_DEV_BAD_PREFIX;
    return 0;
  }
  if (len < 0 || len > p.D) {
    *flags |= MV_DEV_BAD_PATH;
    return 0;
  }
  for (int j = 0; j < len; ++j) {
    const int node = p.path_nodes[static_cast<size_t>(b) * p.D + j];
    if (node < j || node >= p.N) {  // a node on level j of a root path has index >= j
      *flags |= MV_DEV_BAD_PATH;
      return 0;
    }
    if (src) src[j] = node;
  }
  return len;
}

// One workgroup per (sequence, KV head): stage <= D rows of K and of V, then write them back.
__global__ __launch_bounds__(kCommitThreads) void kv_commit_kernel(const CommitParams p) {
  __shared__ __attribute__((aligned(16))) char stage[2][MV_MAX_DEPTH][kMaxRowBytes];
  __shared__ int src[MV_MAX_DEPTH];
  __shared__ int nrows;
  const int b = blockIdx.x / p.Hkv, g = blockIdx.x % p.Hkv, tid = threadIdx.x;
  if (tid == 0) {
    int flags = 0;
    nrows = commit_len(p, b, &flags, src);
    if (g == 0) {
      if (flags && p.status) atomicOr(p.status, flags);
      // a separate output buffer takes the new prefix here; in place it needs a second launch
      if (p.prefix_out != p.prefix_len) p.prefix_out[b] = p.prefix_len[b] + nrows;
    }
  }
  __syncthreads();
  const int n = nrows;
  if (n == 0) return;
  const int lb = p.prefix_len[b];
  const int row_bytes = p.dh * p.esz;  // a multiple of 16 (dh in {64, 128})
  const int pieces = row_bytes / 16;
  const size_t head = (static_cast<size_t>(b) * p.Hkv + g) * p.L_cap;
  for (int i = tid; i < 2 * n * pieces; i += kCommitThreads) {
    const int which = i / (n * pieces), r = (i / pieces) % n, c = i % pieces;
    const char* base = which ? p.v : p.k;
    const size_t row = head + static_cast<size_t>(lb + src[r]);
    *reinterpret_cast<uint4*>(&stage[which][r][c * 16]) =
        *reinterpret_cast<const uint4*>(base + row * row_bytes + c * 16);
  }
  __syncthreads();
  for (int i = tid; i < 2 * n * pieces; i += kCommitThreads) {
    const int which = i / (n * pieces), r = (i / pieces) % n, c = i % pieces;
    char* base = which ? p.v : p.k;
    const size_t row = head + static_cast<size_t>(lb + r);
    *reinterpret_cast<uint4*>(base + row * row_bytes + c * 16) =
        *reinterpret_cast<const uint4*>(&stage[which][r][c * 16]);
  }
}

// prefix_out[b] = prefix_len[b] + accept_len[b] for a valid sequence, prefix_len[b] otherwise
// (after the copies, which read prefix_len; a separate launch, so prefix_out may alias it).
__global__ void advance_prefix_kernel(const CommitParams p) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= p.B) return;
  int flags = 0;
  const int len = commit_len(p, b, &flags, nullptr);
  p.prefix_out[b] = p.prefix_len[b] + (flags == 0 ? len : 0);
}

}  // namespace
}  // namespace mv

using namespace mv;

extern "C" {

MV_API int mv_kv_commit(int dt, int B, int Hkv, int dh, int L_cap, int N, int D, void* k_cache,
                        void* v_cache, const int32_t* prefix_len, int32_t* prefix_out,
                        const int32_t* path_nodes, const int32_t* accept_len,
                        int32_t* dev_status, void* stream) {
  if (dt != MV_F32 && dt != MV_BF16) return MV_ERR_INVALID_ARG;
  if (B < 1 || Hkv < 1 || N < 1 || D < 1 || L_cap < N) return MV_ERR_INVALID_ARG;
  if (!k_cache || !v_cache || !prefix_len || !prefix_out || !path_nodes || !accept_len)
    return MV_ERR_INVALID_ARG;
  if (dh != 64 && dh != 128) return MV_ERR_UNSUPPORTED;
  if (N > MV_MAX_NODES || D > MV_MAX_DEPTH) return MV_ERR_UNSUPPORTED;
  CommitParams p{};
  p.B = B; p.Hkv = Hkv; p.dh = dh; p.L_cap = L_cap; p.N = N; p.D = D;
  p.esz = dt == MV_BF16 ? 2 : 4;
  p.k = static_cast<char*>(k_cache);
  p.v = static_cast<char*>(v_cache);
  p.prefix_len = prefix_len;
  p.prefix_out = prefix_out;
  p.path_nodes = path_nodes;
  p.accept_len = accept_len;
  p.status = dev_status;
  const long long blocks = static_cast<long long>(B) * Hkv;
  if (blocks > (1LL << 31) - 1) return MV_ERR_UNSUPPORTED;
  hipStream_t st = as_stream(stream);
  kv_commit_kernel<<<static_cast<int>(blocks), kCommitThreads, 0, st>>>(p);
  if (prefix_out != prefix_len) return launch_status();
  MV_TRY(launch_status());
  advance_prefix_kernel<<<ceil_div(B, 256), 256, 0, st>>>(p);
  return launch_status();
}

}  // extern "C"
