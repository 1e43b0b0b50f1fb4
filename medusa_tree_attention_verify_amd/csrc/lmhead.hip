// Target LM head over the verification rows, fused with what acceptance consumes.
//
// Sources: "Medusa Explained: Multi-Head Speculative Decoding Guide", "2. Single-Pass Tree
// Attention Verification" (the target model outputs a distribution for every candidate node,
// and a node is accepted when its token equals the target's greedy prediction);
// "Speculative Decoding & Medusa Tree Attention: Accelerating LLM Inference by 3x Without
// Accuracy Loss", "2. The Acceptance Sampling Rule" (P_target is the softmax of the target's
// logits).
//
// For T rows of final hidden states x (B*(N+1) of them in a verify step: per sequence the last
// prefix position, then the tree nodes): logits[t][v] = sum_j W[v][j] x[t][j].  The call returns
// per row the greedy token argmax_v logits[t][v] (ties: lowest id), optionally that logit and
// LSE[t] = log sum_v exp(logits[t][v]), and never writes the [T][V] logits.
//
// One streaming pass over W: a workgroup owns 64 vocabulary rows and a group of up to 128
// target rows, and its NW waves split d.  Per k-step a lane loads one 16-byte piece of each of
// the 4 row tiles (the A operand of v_mfma_f32_16x16x32_bf16: 16 rows x 32 columns of W) and of
// each of the NCT column tiles of x (the B operand: 16 target rows), so every weight byte
// crosses HBM once and the x pieces come from L2.  The waves reduce one 16-row column tile at a
// time through LDS; for those 16 target rows the epilogue writes per 64-row vocabulary block
// the partial (max, its id, sum exp(logit - max)).  A second kernel merges the ceil(V/64)
// partials of each row.

#include <math.h>

#include <algorithm>

#include "mv_device.h"
#include "mv_host.h"

namespace mv {
namespace {

constexpr int kLmRows = 64;        // vocabulary rows per workgroup
constexpr int kLmMaxCols = 128;    // target rows per workgroup (8 column tiles)
constexpr int kLmMergeThreads = 256;

struct LmParams {
  int T, d, V, KT, nrb, ncols;  // KT = d / 32, nrb = ceil(V / 64), ncols = target rows per group
  const uint16_t* x;            // [T][d] bf16
  const uint16_t* w;            // [V][d] bf16
  float* pm;                    // [T][nrb] partial max
  float* pl;                    // [T][nrb] partial sum exp(logit - max)
  int* pidx;                    // [T][nrb] id of the partial max (lowest on ties)
  int32_t* ids;                 // [T]
  float* maxv;                  // [T] or null
  float* lse;                   // [T] or null
};

template <int NW, int NCT>
__global__ __launch_bounds__(NW * 64) void lm_head_kernel(const LmParams p) {
  constexpr int RT = kLmRows / 16, U = 2;
  __shared__ float red[NW][kLmRows][17];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rb = blockIdx.x, row0 = rb * kLmRows;
  const int col0 = blockIdx.y * p.ncols;
  const int t0 = (w * p.KT) / NW, t1 = ((w + 1) * p.KT) / NW;

  // A operand: lane (row r = lane % 16, k-group g = lane / 16) of row tile rt reads the 16 bytes
  // W[row0 + 16*rt + r][32*t + 8*g .. +8]; rows past V are clamped (their logits are not used).
  const u32x4* ap[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = min(row0 + rt * 16 + (lane & 15), p.V - 1);
    ap[rt] = reinterpret_cast<const u32x4*>(p.w + static_cast<size_t>(r) * p.d) + (lane >> 4) + t0 * 4;
  }
  // B operand: lane (column c = lane % 16, k-group g) of column tile ct reads
  // x[col0 + 16*ct + c][32*t + 8*g .. +8]; columns past T read row T-1 (results not used).
  const u32x4* bp[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int c = min(col0 + ct * 16 + (lane & 15), p.T - 1);
    bp[ct] = reinterpret_cast<const u32x4*>(p.x + static_cast<size_t>(c) * p.d) + (lane >> 4) + t0 * 4;
  }
  f32x4 acc[RT][NCT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto step = [&](const u32x4 (&a)[RT], const u32x4 (&b)[NCT]) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, a[rt]), __builtin_bit_cast(bf16x8, b[ct]), acc[rt][ct], 0, 0, 0);
  };
  int t = t0;
  for (; t + U <= t1; t += U) {
    u32x4 a[U][RT], b[U][NCT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) a[u][rt] = ap[rt][u * 4];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) b[u][ct] = bp[ct][u * 4];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) step(a[u], b[u]);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) ap[rt] += U * 4;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) bp[ct] += U * 4;
  }
  for (; t < t1; ++t) {
    u32x4 a[RT], b[NCT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) a[rt] = ap[rt][0];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) b[ct] = bp[ct][0];
    step(a, b);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) ap[rt] += 4;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) bp[ct] += 4;
  }

  // Per column tile: the waves' partial sums meet in LDS (16x16 D layout: lane holds rows
  // 4*(lane/16) + v, column lane % 16), then each wave takes 16/NW of the tile's target rows;
  // lane = vocabulary row for the (max, id, sum exp) of its 64-row block.
  const int row = row0 + lane;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[w][rt * 16 + (lane >> 4) * 4 + v][lane & 15] = acc[rt][ct][v];
    __syncthreads();
    for (int cc = w; cc < 16; cc += NW) {
      const int tok = col0 + ct * 16 + cc;
      if (tok >= p.T || ct * 16 + cc >= p.ncols) continue;  // wave-uniform
      const bool live = row < p.V;
      float val = -INFINITY;
      if (live) {
        val = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) val += red[ww][lane][cc];
      }
      float bv = val;
      int bi = live ? row : INT_MAX;
      wave_argbest(bv, bi);
      const float l = wave_sum(val == -INFINITY ? 0.f : expf(val - bv));
      if (lane == 0) {
        const size_t q = static_cast<size_t>(tok) * p.nrb + rb;
        p.pm[q] = bv;
        p.pl[q] = l;
        p.pidx[q] = bi;
      }
    }
    __syncthreads();
  }
}

// One workgroup per target row: argmax (lowest id on ties) and LSE from the block partials.
__global__ __launch_bounds__(kLmMergeThreads) void lm_head_merge_kernel(const LmParams p) {
  __shared__ float sv[kLmMergeThreads / 64], sm[kLmMergeThreads / 64], sl[kLmMergeThreads / 64];
  __shared__ int si[kLmMergeThreads / 64];
  const int tok = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const size_t base = static_cast<size_t>(tok) * p.nrb;
  float bv = -INFINITY, m = -INFINITY, l = 0.f;
  int bi = INT_MAX;
  constexpr int BATCH = 4;
  for (int j0 = tid; j0 < p.nrb; j0 += kLmMergeThreads * BATCH) {
    float mv[BATCH], lv[BATCH];
    int iv[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int j = j0 + u * kLmMergeThreads;
      mv[u] = j < p.nrb ? p.pm[base + j] : -INFINITY;
      lv[u] = j < p.nrb ? p.pl[base + j] : 0.f;
      iv[u] = j < p.nrb ? p.pidx[base + j] : INT_MAX;
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      if (kv_better(mv[u], iv[u], bv, bi)) {
        bv = mv[u];
        bi = iv[u];
      }
      ml_merge(m, l, mv[u], lv[u]);
    }
  }
  wave_argbest(bv, bi);
  wave_ml_merge(m, l);
  if (lane == 0) {
    sv[w] = bv;
    si[w] = bi;
    sm[w] = m;
    sl[w] = l;
  }
  __syncthreads();
  if (tid == 0) {
    for (int k = 1; k < kLmMergeThreads / 64; ++k) {
      if (kv_better(sv[k], si[k], bv, bi)) {
        bv = sv[k];
        bi = si[k];
      }
    }
    float M = sm[0], L = sl[0];
    for (int k = 1; k < kLmMergeThreads / 64; ++k) ml_merge(M, L, sm[k], sl[k]);
    p.ids[tok] = bi == INT_MAX ? -1 : bi;
    if (p.maxv) p.maxv[tok] = bv;
    if (p.lse) p.lse[tok] = M + logf(L);
  }
}

struct LmPlan {
  int nrb = 1, ncols = 16, nct = 1, ngrp = 1, nw = 4;
  size_t ws_bytes = 0;
};

LmPlan plan_lm(int T, int d, int V) {
  LmPlan a;
  a.nrb = ceil_div(V, kLmRows);
  const int cols = std::min(T, kLmMaxCols);
  a.nct = ceil_div(cols, 16);
  a.ncols = 16 * a.nct;
  a.ngrp = ceil_div(T, a.ncols);
  a.nw = d / 32 >= 64 ? 8 : 4;
  Carver c(nullptr);
  const size_t np = static_cast<size_t>(T) * a.nrb;
  c.take<float>(np);
  c.take<float>(np);
  c.take<int>(np);
  a.ws_bytes = c.bytes();
  return a;
}

int check_lm(int dt, int T, int d, int V) {
  if (dt != MV_F32 && dt != MV_BF16) return MV_ERR_INVALID_ARG;
  if (T < 1 || d < 1 || V < 1) return MV_ERR_INVALID_ARG;
  if (dt != MV_BF16 || d % 32 != 0) return MV_ERR_UNSUPPORTED;
  return MV_OK;
}

}  // namespace
}  // namespace mv

using namespace mv;

extern "C" {

MV_API size_t mv_lm_head_workspace(int dt, int T, int d, int V) {
  if (check_lm(dt, T, d, V) != MV_OK) return 0;
  return plan_lm(T, d, V).ws_bytes;
}

MV_API int mv_lm_head_argmax(int dt, int T, int d, int V, const void* x, const void* w_lm,
                             int32_t* argmax_ids, float* max_logit, float* lse, void* ws,
                             size_t ws_bytes, void* stream) {
  MV_TRY(check_lm(dt, T, d, V));
  if (!x || !w_lm || !argmax_ids) return MV_ERR_INVALID_ARG;
  const LmPlan a = plan_lm(T, d, V);
  MV_TRY(check_ws(ws, ws_bytes, a.ws_bytes));
  LmParams p{};
  p.T = T; p.d = d; p.V = V; p.KT = d / 32; p.nrb = a.nrb; p.ncols = a.ncols;
  p.x = static_cast<const uint16_t*>(x);
  p.w = static_cast<const uint16_t*>(w_lm);
  Carver c(ws);
  const size_t np = static_cast<size_t>(T) * a.nrb;
  p.pm = c.take<float>(np);
  p.pl = c.take<float>(np);
  p.pidx = c.take<int>(np);
  p.ids = argmax_ids;
  p.maxv = max_logit;
  p.lse = lse;
  hipStream_t st = as_stream(stream);
  const dim3 grid(a.nrb, a.ngrp);
  bool launched = false;
#define MV_LM_CASE(NW_, NCT_) \
  if (a.nw == NW_ && a.nct == NCT_) { lm_head_kernel<NW_, NCT_><<<grid, NW_ * 64, 0, st>>>(p); launched = true; }
  MV_LM_CASE(4, 1) MV_LM_CASE(4, 2) MV_LM_CASE(4, 3) MV_LM_CASE(4, 4)
  MV_LM_CASE(4, 5) MV_LM_CASE(4, 6) MV_LM_CASE(4, 7) MV_LM_CASE(4, 8)
  MV_LM_CASE(8, 1) MV_LM_CASE(8, 2) MV_LM_CASE(8, 3) MV_LM_CASE(8, 4)
  MV_LM_CASE(8, 5) MV_LM_CASE(8, 6) MV_LM_CASE(8, 7) MV_LM_CASE(8, 8)
#undef MV_LM_CASE
  if (!launched) return MV_ERR_UNSUPPORTED;  // no kernel instance for this shape
  MV_TRY(launch_status());
  lm_head_merge_kernel<<<T, kLmMergeThreads, 0, st>>>(p);
  return launch_status();
}

}  // extern "C"
