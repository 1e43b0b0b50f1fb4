// Medusa heads on gfx950: the residual block h_k = SiLU(W_res^(k) h) + h and the vocabulary
// projection logits_k = W_head^(k) h_k with its top-s_k tokens and log-sum-exp.
//
// Source: "Medusa Explained: Multi-Head Speculative Decoding Guide", section "The
// Architectural Blueprint" (residual block without bias, softmax over the projection) and
// "1. Combinatorial Tree Construction" (each head offers its top-s_k tokens).
//
// Both products are matrix-vector products over a handful of batch rows, so they are bound by
// streaming the weights once from HBM.  They run on the bf16 matrix cores anyway: one
// v_mfma_f32_16x16x32_bf16 takes a 16-row x 32-column weight tile straight from the load
// registers and reduces over the 32 columns in hardware, which leaves the vector ALUs free and
// needs no cross-lane reduction in the streaming loop.  The 16 MFMA columns carry the batch:
// columns 0-7 hold the high bf16 part of up to 8 batch vectors and columns 8-15 the bf16
// remainder (x - hi), so an fp32 vector enters the product with ~16 significant bits and the
// sum of the two column halves is the fp32-accurate dot product.  bf16 inputs have a zero
// remainder.  The vector side is pre-arranged in the exact register layout of the MFMA B
// operand ("packed"), so the streaming loop does one coalesced 16-byte load per lane for it.
//
// Each workgroup owns 32 weight rows; its NW waves split the reduction dimension and meet in
// LDS.  The projection's epilogue keeps only a per-workgroup top-s and (max, sum-exp) pair per
// batch row; a small second kernel merges them per (head, batch row), so the logits never
// have to be written.

#include <math.h>

#include <mutex>

#include "mv_device.h"
#include "mv_host.h"

// Scratch of the allocation-free entry point (mv_medusa_heads_noalloc): every GPU the library
// runs on holds one copy for the life of the process.  Host code never passes this name to a
// kernel (on the host it only stands in for the symbol); it uses the per-device address that
// hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[MV_HEADS_NOALLOC_SCRATCH_BYTES];

namespace mv {
namespace {

constexpr int kRows = 32;  // weight rows per workgroup
constexpr int kMaxBatchF32 = 32;  // batch rows of the fp32 heads (a register accumulator each)

// Streaming parameters (measured on MI355X; see the head-projection profile).
#ifndef MV_GEMV_U
#define MV_GEMV_U 2            // k-steps per load batch
#endif
#ifndef MV_GEMV_WAVES
#define MV_GEMV_WAVES 12288    // waves per launch to aim for (1024 SIMDs on the chip)
#endif

struct GemvParams {
  int B, d, R, K, T, nrb;   // R = rows per head, T = d / 32, nrb = ceil(R / kRows)
  const void* W;            // [K][R][d]
  const u32x4* bsrc;        // packed B operand (bf16 path)
  long long bsrc_hstride;   // per-head stride of bsrc in u32x4 units (0 = shared)
  const float* xsrc;        // fp32 path: vector source, [B][xstride] with per-head offset
  long long x_bstride, x_hstride;
  // residual epilogue
  const void* h;
  float* hk_ws;
  float* hk_out;
  uint16_t* bpack_out;
  // projection epilogue
  void* logits;
  float* pval;
  int* pidx;
  float* pm;
  float* pl;
  int32_t* topk_ids;
  float* topk_vals;
  int ld_topk;
  float* lse;
  int s_max;
  int s[MV_MAX_HEADS];
};

__device__ __forceinline__ u32x4 wload(const u32x4* p) { return *p; }

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* base, size_t i) {
  if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t*>(base)[i]);
  else return static_cast<const float*>(base)[i];
}

template <bool BF16>
__device__ __forceinline__ void store_elem(void* base, size_t i, float v) {
  if constexpr (BF16) static_cast<uint16_t*>(base)[i] = f32_to_bf16(v);
  else static_cast<float*>(base)[i] = v;
}

// ---- residual epilogue: h_k = SiLU(u) + h; keep fp32 h_k and (bf16 path) its packed form.
template <bool BF16, int BC>
__device__ void residual_epilogue(const GemvParams& p, int k, int row0, float (*ys)[BC]) {
  const int nct = BC / 8;
  for (int idx = threadIdx.x; idx < kRows * BC; idx += blockDim.x) {
    const int row = idx / BC, b = idx % BC, j = row0 + row;
    if (j >= p.d) continue;
    float v = 0.f;
    if (b < p.B) {
      const float u = ys[row][b];
      const float silu = u / (1.0f + expf(-u));
      v = silu + load_elem<BF16>(p.h, static_cast<size_t>(b) * p.d + j);
      const size_t o = (static_cast<size_t>(b) * p.K + k) * p.d + j;
      p.hk_ws[o] = v;
      if (p.hk_out) p.hk_out[o] = v;
    }
    if constexpr (BF16) {
      const uint16_t hi = (b < p.B) ? f32_to_bf16(v) : 0;
      const uint16_t lo = (b < p.B) ? f32_to_bf16(v - bf16_to_f32(hi)) : 0;
      const int t = j >> 5, g = (j >> 3) & 3, e = j & 7, ct = b >> 3, bb = b & 7;
      const size_t base = ((static_cast<size_t>(k) * p.T + t) * nct + ct) * 64;
      p.bpack_out[(base + g * 16 + bb) * 8 + e] = hi;
      p.bpack_out[(base + g * 16 + 8 + bb) * 8 + e] = lo;
    }
  }
}

// ---- merge of the per-workgroup partials: one workgroup per (head k, batch row b).
// A separate launch: a completion counter inside the projection kernel would need an
// agent-scope release/acquire per workgroup, which on this multi-XCD part writes back and
// invalidates the XCD's L2 for every workgroup.  One pass over the partials with coalesced,
// independent loads: every thread folds its candidates into a sorted register list of SM
// entries (SM >= s_max) and an online (max, sum); each wave then draws its top s_k from the
// list heads and merges its (max, sum) pairs with register butterflies, and after a single
// barrier wave 0 draws the final s_k from the waves' winners.
constexpr int kMergeThreads = 512;
constexpr int kMergeWaves = kMergeThreads / 64;

template <int SM>
__device__ __forceinline__ void list_insert(float (&lv)[SM], int (&li)[SM], float v, int i) {
#pragma unroll
  for (int q = 0; q < SM; ++q) {
    if constexpr (SM > 8) {
      // long lists: a compare-exchange chain of selects (as branches, lanes that disagree
      // run both sides of every step); short ones are faster with the branches
      const bool c = kv_better(v, i, lv[q], li[q]);
      const float tv = lv[q];
      const int ti = li[q];
      lv[q] = c ? v : tv;
      li[q] = c ? i : ti;
      v = c ? tv : v;
      i = c ? ti : i;
    } else if (kv_better(v, i, lv[q], li[q])) {
      const float tv = lv[q];
      const int ti = li[q];
      lv[q] = v;
      li[q] = i;
      v = tv;
      i = ti;
    }
  }
}

template <int SM>
__device__ __forceinline__ void list_pop(float (&lv)[SM], int (&li)[SM]) {
#pragma unroll
  for (int q = 0; q + 1 < SM; ++q) {
    lv[q] = lv[q + 1];
    li[q] = li[q + 1];
  }
  lv[SM - 1] = -INFINITY;
  li[SM - 1] = INT_MAX;
}

// Wave 0's final phase of the merges: the waves' top s (wtv/wti, best first), at most
// kMergeWaves * s <= 128 candidates, two per lane and sorted, give the final s by wave
// arg-bests; the waves' (max, sum) pairs give the LSE.
__device__ __forceinline__ void merge_wave_winners(const GemvParams& p, const float (&wtv)[kMergeWaves][MV_MAX_TOPK],
                                                   const int (&wti)[kMergeWaves][MV_MAX_TOPK],
                                                   const float (&wm)[kMergeWaves], const float (&wl)[kMergeWaves],
                                                   int s, int smax, int b, int k, int lane) {
  float cv[2];
  int ci[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int c = lane + 64 * q;
    const bool ok = c < kMergeWaves * s;
    cv[q] = ok ? wtv[c / max(s, 1)][c % max(s, 1)] : -INFINITY;
    ci[q] = ok ? wti[c / max(s, 1)][c % max(s, 1)] : INT_MAX;
  }
  if (kv_better(cv[1], ci[1], cv[0], ci[0])) {
    const float tv = cv[0];
    const int ti = ci[0];
    cv[0] = cv[1];
    ci[0] = ci[1];
    cv[1] = tv;
    ci[1] = ti;
  }
  for (int r = 0; r < smax; ++r) {
    float bv = r < s ? cv[0] : -INFINITY;
    int bi = r < s ? ci[0] : INT_MAX;
    wave_argbest(bv, bi);
    if (r < s && bi != INT_MAX && ci[0] == bi) {
      cv[0] = cv[1];
      ci[0] = ci[1];
      cv[1] = -INFINITY;
      ci[1] = INT_MAX;
    }
    if (lane == 0) {
      const size_t o = static_cast<size_t>(b) * p.ld_topk + static_cast<size_t>(k) * smax + r;
      const bool ok = r < s && bi != INT_MAX;
      p.topk_ids[o] = ok ? bi : -1;
      p.topk_vals[o] = ok ? bv : -INFINITY;
    }
  }
  float M = lane < kMergeWaves ? wm[lane] : -INFINITY;
  float Ls = lane < kMergeWaves ? wl[lane] : 0.f;
  wave_ml_merge(M, Ls);
  if (lane == 0 && p.lse) p.lse[static_cast<size_t>(b) * p.K + k] = M + logf(Ls);
}

template <int SM>
__global__ __launch_bounds__(kMergeThreads) void heads_merge_kernel(const GemvParams p) {
  __shared__ float wtv[kMergeWaves][MV_MAX_TOPK];
  __shared__ int wti[kMergeWaves][MV_MAX_TOPK];
  __shared__ float wm[kMergeWaves], wl[kMergeWaves];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int k = blockIdx.x % p.K, b = blockIdx.x / p.K;
  const int nrb = p.nrb, s = p.s[k], smax = p.s_max;
  const size_t base = (static_cast<size_t>(k) * p.B + b) * nrb;
  float lv[SM];
  int li[SM];
#pragma unroll
  for (int q = 0; q < SM; ++q) {
    lv[q] = -INFINITY;
    li[q] = INT_MAX;
  }
  const int n = nrb * smax;
  const int* pidx = p.pidx + base * smax;
  const float* pval = p.pval + base * smax;
  // Every candidate and (max, sum) pair a thread merges is requested before any is used: the
  // partials were written from every XCD, so each load is a trip to memory and must not wait
  // for the previous one (with V = 32000 and s_max = 4 one pass of 8 + 2 loads covers all).
  constexpr int BATCH = 8, MBATCH = 2;
  float m = -INFINITY, l = 0.f;
  for (int c0 = tid, j0 = tid; c0 < n || j0 < nrb; c0 += kMergeThreads * BATCH, j0 += kMergeThreads * MBATCH) {
    int ii[BATCH];
    float vv[BATCH], mb[MBATCH], lb[MBATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int c = c0 + u * kMergeThreads;
      ii[u] = c < n ? pidx[c] : -1;
      vv[u] = c < n ? pval[c] : -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < MBATCH; ++u) {
      const int j = j0 + u * kMergeThreads;
      mb[u] = j < nrb ? p.pm[base + j] : -INFINITY;
      lb[u] = j < nrb ? p.pl[base + j] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u)
      if (ii[u] >= 0 && (c0 + u * kMergeThreads) % smax < s) list_insert<SM>(lv, li, vv[u], ii[u]);
#pragma unroll
    for (int u = 0; u < MBATCH; ++u) ml_merge(m, l, mb[u], lb[u]);
  }
  // per wave: top s (token ids are unique, so exactly one lane owns each winner and pops it)
  for (int r = 0; r < s; ++r) {
    float bv = lv[0];
    int bi = li[0];
    wave_argbest(bv, bi);
    if (bi != INT_MAX && li[0] == bi) list_pop<SM>(lv, li);
    if (lane == 0) {
      wtv[w][r] = bv;
      wti[w][r] = bi;
    }
  }
  wave_ml_merge(m, l);
  if (lane == 0) {
    wm[w] = m;
    wl[w] = l;
  }
  __syncthreads();
  if (w != 0) return;
  merge_wave_winners(p, wtv, wti, wm, wl, s, smax, b, k, lane);
}

// ---- merge as a tournament, for lists longer than 8 (up to kMergeThreads * CPT candidates
// per (head, batch row)).  Every candidate stays in registers, unsorted (CPT per thread).  Each
// of the s_k rounds takes the workgroup's best (value, then lower id) with one wave arg-best and
// one LDS exchange between the waves, and the thread holding the winning id drops it.  The LDS
// slots alternate between rounds, so one barrier per round suffices: a wave can only overwrite
// a slot after every wave has passed the barrier that follows its last reader.  At 10
// candidates per head this replaces the 16-slot sorted lists' insertion chains.
template <int CPT>
__global__ __launch_bounds__(kMergeThreads) void heads_tournament_kernel(const GemvParams p) {
  __shared__ float rv[2][kMergeWaves];
  __shared__ int ri[2][kMergeWaves];
  __shared__ float wm[kMergeWaves], wl[kMergeWaves];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int k = blockIdx.x % p.K, b = blockIdx.x / p.K;
  const int nrb = p.nrb, s = p.s[k], smax = p.s_max;
  const size_t base = (static_cast<size_t>(k) * p.B + b) * nrb;
  const int n = nrb * smax;
  const int* pidx = p.pidx + base * smax;
  const float* pval = p.pval + base * smax;
  float cv[CPT];
  int ci[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) {  // all requested before any is used
    const int c = tid + u * kMergeThreads;
    ci[u] = c < n ? pidx[c] : -1;
    cv[u] = c < n ? pval[c] : -INFINITY;
  }
  float m = -INFINITY, l = 0.f;
  for (int j = tid; j < nrb; j += kMergeThreads) ml_merge(m, l, p.pm[base + j], p.pl[base + j]);
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const bool ok = ci[u] >= 0 && (tid + u * kMergeThreads) % smax < s;
    cv[u] = ok ? cv[u] : -INFINITY;
    ci[u] = ok ? ci[u] : INT_MAX;
  }
  wave_ml_merge(m, l);
  if (lane == 0) {
    wm[w] = m;
    wl[w] = l;
  }
  const size_t o = static_cast<size_t>(b) * p.ld_topk + static_cast<size_t>(k) * smax;
  for (int r = 0; r < s; ++r) {
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const bool c = kv_better(cv[u], ci[u], bv, bi);
      bv = c ? cv[u] : bv;
      bi = c ? ci[u] : bi;
    }
    wave_argbest(bv, bi);
    if (lane == 0) {
      rv[r & 1][w] = bv;
      ri[r & 1][w] = bi;
    }
    __syncthreads();
    float gv = rv[r & 1][0];
    int gi = ri[r & 1][0];
#pragma unroll
    for (int q = 1; q < kMergeWaves; ++q) {
      const float ov = rv[r & 1][q];
      const int oi = ri[r & 1][q];
      const bool c = kv_better(ov, oi, gv, gi);
      gv = c ? ov : gv;
      gi = c ? oi : gi;
    }
    if (gi != INT_MAX) {  // token ids are unique: exactly one slot of one thread holds it
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        const bool hit = ci[u] == gi;
        cv[u] = hit ? -INFINITY : cv[u];
        ci[u] = hit ? INT_MAX : ci[u];
      }
    }
    if (tid == 0) {
      p.topk_ids[o + r] = gi != INT_MAX ? gi : -1;
      p.topk_vals[o + r] = gi != INT_MAX ? gv : -INFINITY;
    }
  }
  if (tid == 0)
    for (int r = s; r < smax; ++r) {
      p.topk_ids[o + r] = -1;
      p.topk_vals[o + r] = -INFINITY;
    }
  __syncthreads();
  if (w != 0) return;
  float M = lane < kMergeWaves ? wm[lane] : -INFINITY;
  float Ls = lane < kMergeWaves ? wl[lane] : 0.f;
  wave_ml_merge(M, Ls);
  if (lane == 0 && p.lse) p.lse[static_cast<size_t>(b) * p.K + k] = M + logf(Ls);
}

// Merge of the blocks' sorted lists (each 32-row block's list is its top s, best first): a
// k-way merge over the list heads.  Each thread holds the lists of BPT blocks in registers and
// their current heads; per rank a wave takes the best head among its threads (a wave arg-best)
// and only the thread owning the winner advances that list.  Each wave so draws its own top s
// with no workgroup barrier per rank; after one barrier wave 0 merges the waves' winners.  A
// rank costs a comparison of BPT heads per thread instead of a scan of every candidate the
// thread holds.
template <int BPT, int SMX>
__global__ __launch_bounds__(kMergeThreads) void heads_kmerge_kernel(const GemvParams p) {
  __shared__ float wtv[kMergeWaves][MV_MAX_TOPK];
  __shared__ int wti[kMergeWaves][MV_MAX_TOPK];
  __shared__ float wm[kMergeWaves], wl[kMergeWaves];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int k = blockIdx.x % p.K, b = blockIdx.x / p.K;
  const int nrb = p.nrb, s = p.s[k], smax = p.s_max;
  const size_t base = (static_cast<size_t>(k) * p.B + b) * nrb;
  const int* pidx = p.pidx + base * smax;
  const float* pval = p.pval + base * smax;
  float lv[BPT][SMX];
  int li[BPT][SMX];
#pragma unroll
  for (int q = 0; q < BPT; ++q) {  // all requested before any is used
    const int blk = tid + q * kMergeThreads;
#pragma unroll
    for (int r = 0; r < SMX; ++r) {
      const bool ok = blk < nrb && r < s;
      const int id = ok ? pidx[static_cast<size_t>(blk) * smax + r] : -1;
      const float v = ok ? pval[static_cast<size_t>(blk) * smax + r] : -INFINITY;
      li[q][r] = id >= 0 ? id : INT_MAX;
      lv[q][r] = id >= 0 ? v : -INFINITY;
    }
  }
  float m = -INFINITY, l = 0.f;
  for (int j = tid; j < nrb; j += kMergeThreads) ml_merge(m, l, p.pm[base + j], p.pl[base + j]);
  wave_ml_merge(m, l);
  if (lane == 0) {
    wm[w] = m;
    wl[w] = l;
  }
  int ptr[BPT];
  float hv[BPT];
  int hi[BPT];
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    ptr[q] = 0;
    hv[q] = lv[q][0];
    hi[q] = li[q][0];
  }
  for (int r = 0; r < s; ++r) {
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      const bool c = kv_better(hv[q], hi[q], bv, bi);
      bv = c ? hv[q] : bv;
      bi = c ? hi[q] : bi;
    }
    wave_argbest(bv, bi);
    if (bi != INT_MAX) {  // token ids are unique: exactly one head of one lane holds it
#pragma unroll
      for (int q = 0; q < BPT; ++q) {
        if (hi[q] == bi) {
          const int nx = ++ptr[q];
          float v = -INFINITY;
          int id = INT_MAX;
#pragma unroll
          for (int t = 1; t < SMX; ++t) {
            v = t == nx ? lv[q][t] : v;
            id = t == nx ? li[q][t] : id;
          }
          hv[q] = v;
          hi[q] = id;
        }
      }
    }
    if (lane == 0) {
      wtv[w][r] = bv;
      wti[w][r] = bi;
    }
  }
  __syncthreads();
  if (w != 0) return;
  merge_wave_winners(p, wtv, wti, wm, wl, s, smax, b, k, lane);
}

// ---- projection epilogue: optional logits, per-workgroup top-s and (max, sum exp).
template <bool BF16, int NW, int BC>
__device__ void head_epilogue(const GemvParams& p, int k, int rb, float (*ys)[BC]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int row0 = rb * kRows;
  if (p.logits) {
    for (int idx = threadIdx.x; idx < kRows * BC; idx += blockDim.x) {
      const int row = idx / BC, b = idx % BC, j = row0 + row;
      if (b < p.B && j < p.R)
        store_elem<BF16>(p.logits, (static_cast<size_t>(b) * p.K + k) * p.R + j, ys[row][b]);
    }
  }
  const int s = p.s[k];
  for (int b = w; b < p.B; b += NW) {
    const int j = row0 + lane;
    float val = (lane < kRows && j < p.R) ? ys[lane][b] : -INFINITY;
    const float m = wave_max(val);
    const float l = wave_sum(val == -INFINITY ? 0.f : expf(val - m));
    const size_t q = (static_cast<size_t>(k) * p.B + b) * p.nrb + rb;
    if (lane == 0) {
      p.pm[q] = m;
      p.pl[q] = l;
    }
    for (int r = 0; r < s; ++r) {
      float bv = val;
      int bi = (val == -INFINITY) ? INT_MAX : j;
      wave_argbest(bv, bi);
      if (lane == 0) {
        p.pval[q * p.s_max + r] = bv;
        p.pidx[q * p.s_max + r] = (bi == INT_MAX) ? -1 : bi;
      }
      if (bi == j) val = -INFINITY;
    }
  }
}

// ---- bf16 weights: MFMA streaming loop.
// LDS arrays of gemv_bf16_kernel: the waves' partial sums and the reduced outputs (the
// projection launch pads its LDS request from their sizes).
template <int NW, int NCT> using GemvRed = float[NW][kRows][16 * NCT + 1];
template <int NCT> using GemvYs = float[kRows][8 * NCT];

// Row-segment weight loads (ROWLOAD, the projection).  Loading straight into
// the MFMA operand layout reads 16 rows x 64 bytes per instruction; with d = 8192 those rows are
// 16 KB apart and the 70B-share projection streamed at ~5.1 TB/s.  Reading 2 rows x 512
// contiguous bytes per instruction and going through LDS to the operand layout streams it at
// ~5.8 TB/s (412 -> 363 us; the Llama-3-8B-shaped projection 188 -> 181 us).  Each wave stages
// its own k-range, so the LDS region is private to the wave and needs no workgroup barrier
// (77 KB per 4-wave workgroup).
constexpr int kRlS = 8;                // k-steps per stage of the row-segment loads
constexpr int kRlP = kRlS * 32 + 8;    // LDS row pitch (elements): conflict-free operand reads

template <int NW, int NCT, int MODE, bool ROWLOAD = false>
__global__ __launch_bounds__(NW * 64) void gemv_bf16_kernel(const GemvParams p) {
  constexpr int RT = kRows / 16, BC = 8 * NCT, U = MV_GEMV_U;
  __shared__ GemvRed<NW, NCT> red;
  __shared__ GemvYs<NCT> ys;
  __shared__ __attribute__((aligned(16))) uint16_t wst[ROWLOAD ? NW : 1][ROWLOAD ? kRows : 1][ROWLOAD ? kRlP : 8];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int k = blockIdx.y, rb = blockIdx.x, row0 = rb * kRows;

  const int t0 = (w * p.T) / NW, t1 = ((w + 1) * p.T) / NW;
  // Weight operand: lane (row r = lane % 16, k-group g = lane / 16) of row tile rt reads the
  // 16 bytes W[row0 + 16*rt + r][32*t + 8*g .. +8] at k-step t; rows past R are clamped.
  const uint16_t* Wk = static_cast<const uint16_t*>(p.W) + static_cast<size_t>(k) * p.R * p.d;
  const u32x4* ap[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = min(row0 + rt * 16 + (lane & 15), p.R - 1);
    ap[rt] = reinterpret_cast<const u32x4*>(Wk + static_cast<size_t>(r) * p.d) + (lane >> 4) + t0 * 4;
  }
  // Vector operand.  Projection: the packed h_k, one 16-byte load per lane and k-step.
  // Residual: h itself (bf16, no remainder part): lane (column c, k-group g) of column tile ct
  // reads h[8*ct + c][32*t + 8*g .. +8] for c < 8 and batch rows that exist, zero otherwise.
  const u32x4* bp[NCT];
  bool bvalid[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    if constexpr (MODE == 0) {
      const int c = lane & 15, bb = ct * 8 + (c & 7);
      bvalid[ct] = c < 8 && bb < p.B;
      bp[ct] = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.h) +
                                              static_cast<size_t>(bvalid[ct] ? bb : 0) * p.d) +
               (lane >> 4) + t0 * 4;
    } else {
      bvalid[ct] = true;
      bp[ct] = p.bsrc + k * p.bsrc_hstride + (static_cast<size_t>(t0) * NCT + ct) * 64 + lane;
    }
  }
  constexpr int BSTEP = MODE == 0 ? 4 : NCT * 64;  // u32x4 units per k-step

  f32x4 acc[RT][NCT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  const u32x4 zero = {0u, 0u, 0u, 0u};
  auto step = [&](const u32x4 (&a)[RT], const u32x4 (&bv)[NCT]) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, a[rt]), __builtin_bit_cast(bf16x8, bv[ct]), acc[rt][ct], 0, 0, 0);
  };
  int t = t0;
  if constexpr (ROWLOAD) {
    // Row segments: each instruction reads 2 rows x 512 contiguous bytes (lanes 0-31 one row,
    // 32-63 the next); a stage of kRlS k-steps (32 rows) goes through this wave's own LDS
    // region and is read back in the MFMA operand layout.  Two stages of loads in flight.
    uint16_t (*ws)[kRlP] = wst[w];
    const int lr = lane >> 5, lc = (lane & 31) * 8;
    auto sload = [&](int ts, u32x4 (&r)[kRows / 2]) {
#pragma unroll
      for (int i = 0; i < kRows / 2; ++i) {
        const int row = min(row0 + 2 * i + lr, p.R - 1);
        r[i] = wload(reinterpret_cast<const u32x4*>(Wk + static_cast<size_t>(row) * p.d + ts * 32 + lc));
      }
    };
    auto sstore = [&](const u32x4 (&r)[kRows / 2]) {
#pragma unroll
      for (int i = 0; i < kRows / 2; ++i) *reinterpret_cast<u32x4*>(&ws[2 * i + lr][lc]) = r[i];
    };
    auto scompute = [&]() {
#pragma unroll
      for (int s = 0; s < kRlS; ++s) {
        u32x4 a[RT], bv[NCT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          a[rt] = *reinterpret_cast<const u32x4*>(&ws[rt * 16 + (lane & 15)][s * 32 + (lane >> 4) * 8]);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) bv[ct] = bvalid[ct] ? bp[ct][s * BSTEP] : zero;
        step(a, bv);
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) bp[ct] += kRlS * BSTEP;
    };
    const int nst = (t1 - t0) / kRlS;
    u32x4 r0[kRows / 2], r1[kRows / 2];
    if (nst > 0) sload(t, r0);
    if (nst > 1) sload(t + kRlS, r1);
    int st = 0;
    for (; st + 2 <= nst; st += 2) {
      sstore(r0);
      scompute();
      if (st + 2 < nst) sload(t + (st + 2) * kRlS, r0);
      sstore(r1);
      scompute();
      if (st + 3 < nst) sload(t + (st + 3) * kRlS, r1);
    }
    if (st < nst) {
      sstore(r0);
      scompute();
    }
    t += nst * kRlS;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) ap[rt] += nst * kRlS * 4;
  }
  for (; t + U <= t1; t += U) {
    u32x4 a[U][RT], bv[U][NCT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) a[u][rt] = wload(ap[rt] + u * 4);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) bv[u][ct] = bvalid[ct] ? bp[ct][u * BSTEP] : zero;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) step(a[u], bv[u]);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) ap[rt] += U * 4;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) bp[ct] += U * BSTEP;
  }
  for (; t < t1; ++t) {
    u32x4 a[RT], bv[NCT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) a[rt] = wload(ap[rt]);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) bv[ct] = bvalid[ct] ? bp[ct][0] : zero;
    step(a, bv);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) ap[rt] += 4;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) bp[ct] += BSTEP;
  }
  // D layout of a 16x16 MFMA tile: lane holds rows 4*(lane/16) + v, column lane % 16.
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        red[w][rt * 16 + (lane >> 4) * 4 + v][ct * 16 + (lane & 15)] = acc[rt][ct][v];
  __syncthreads();
  for (int idx = threadIdx.x; idx < kRows * BC; idx += blockDim.x) {
    const int row = idx / BC, b = idx % BC, ct = b >> 3, bb = b & 7;
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) s += red[ww][row][ct * 16 + bb] + red[ww][row][ct * 16 + 8 + bb];
    ys[row][b] = s;
  }
  __syncthreads();
  if constexpr (MODE == 0) residual_epilogue<true, BC>(p, k, row0, ys);
  else head_epilogue<true, NW, BC>(p, k, rb, ys);
}

// ---- fp32 weights: vector-ALU loop, one wave per weight row.
template <int NW, int MODE>
__global__ __launch_bounds__(NW * 64) void gemv_f32_kernel(const GemvParams p) {
  constexpr int BC = kMaxBatchF32;
  __shared__ float ys[kRows][BC];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int k = blockIdx.y, rb = blockIdx.x, row0 = rb * kRows;
  const float* Wk = static_cast<const float*>(p.W) + static_cast<size_t>(k) * p.R * p.d;
  const float* X = p.xsrc + k * p.x_hstride;
  // The wave's rows go in groups of kRG: one 256-column step of every row of a group is
  // requested at once, so the wave waits one round trip per group and step, not per row.
  // Rows past R read row R-1 and are not stored.
  constexpr int kRG = 4;
  for (int r0 = w; r0 < kRows; r0 += NW * kRG) {
    float acc[kRG][BC];
#pragma unroll
    for (int g = 0; g < kRG; ++g)
#pragma unroll
      for (int b = 0; b < BC; ++b) acc[g][b] = 0.f;
    const float* wr[kRG];
#pragma unroll
    for (int g = 0; g < kRG; ++g)
      wr[g] = Wk + static_cast<size_t>(min(row0 + r0 + g * NW, p.R - 1)) * p.d;
    for (int c = lane * 4; c < p.d; c += 256) {
      float4 wv[kRG];
#pragma unroll
      for (int g = 0; g < kRG; ++g) wv[g] = *reinterpret_cast<const float4*>(wr[g] + c);
#pragma unroll
      for (int b = 0; b < BC; ++b) {
        if (b < p.B) {
          const float4 xv = *reinterpret_cast<const float4*>(X + b * p.x_bstride + c);
#pragma unroll
          for (int g = 0; g < kRG; ++g)
            acc[g][b] = fmaf(wv[g].x, xv.x, fmaf(wv[g].y, xv.y, fmaf(wv[g].z, xv.z, fmaf(wv[g].w, xv.w, acc[g][b]))));
        }
      }
    }
#pragma unroll
    for (int g = 0; g < kRG; ++g) {
      const int r = r0 + g * NW;
#pragma unroll
      for (int b = 0; b < BC; ++b) {
        if (b < p.B) {
          const float s = wave_sum(acc[g][b]);
          if (lane == 0 && r < kRows && row0 + r < p.R) ys[r][b] = s;
        }
      }
    }
  }
  __syncthreads();
  if constexpr (MODE == 0) residual_epilogue<false, BC>(p, k, row0, ys);
  else head_epilogue<false, NW, BC>(p, k, rb, ys);
}

// ---- top-s of each row of a logit matrix (one workgroup per row), optionally the row's
// log-sum-exp.  One pass over the row: every thread keeps its S best (value, id) pairs sorted
// in registers and a running (max, sum exp(x - max)) pair; then each wave takes its top s by
// wave arg-bests over the threads' current heads (the owner of each winner popping it), and
// one wave takes the row's top s from the waves' lists.  Rows whose elements are
// 16-byte aligned are read with 16-byte loads.  After each batch of loads the wave takes the
// largest of its lanes' S-th best values: the wave has seen S elements at least that large, so
// an element below it cannot be among the row's S best and skips the insertion (which, with
// every thread seeing only V / threads elements, otherwise ran in some lane of almost every
// step).
template <bool BF16, int S, int kTopkThreads>
__global__ __launch_bounds__(kTopkThreads) void topk_rows_kernel(int V, int s, const void* x, long long ldx,
                                                        int32_t* ids, float* vals, int ld_out,
                                                        float* lse, int vec) {
  constexpr int NW = kTopkThreads / 64;
  __shared__ float cv[NW][S];
  __shared__ int ci[NW][S];
  __shared__ float sm[NW], sl[NW];
  const size_t rowoff = static_cast<size_t>(blockIdx.x) * ldx;
  float lv[S];
  int li[S];
#pragma unroll
  for (int k = 0; k < S; ++k) {
    lv[k] = -INFINITY;
    li[k] = INT_MAX;
  }
  float m = -INFINITY, l = 0.f;
  float wthr = -INFINITY;  // a lower bound on the wave's, so on the row's, S-th best value
  // running (max, sum exp(x - max)) without a branch: one exp of -|v - m| serves both cases
  // (a new maximum rescales the sum, any other value adds its term); -inf adds nothing
  auto lse_take = [&](float v) {
    const bool bigger = v > m;
    const float t = __expf(-fabsf(v - m));
    const float up = fmaf(l, t, 1.f);                    // v is the new maximum
    const float add = l + (v == -INFINITY ? 0.f : t);     // any other value
    l = bigger ? up : add;
    m = bigger ? v : m;
  };
  // insert, keeping the list sorted (after the first few elements almost never taken)
  auto insert = [&](float v, int j) {
    if (v >= lv[S - 1] && v >= wthr && kv_better(v, j, lv[S - 1], li[S - 1])) {
#pragma unroll
      for (int k = S - 1; k > 0; --k) {
        const bool shift = kv_better(v, j, lv[k - 1], li[k - 1]);
        const bool here = !shift && kv_better(v, j, lv[k], li[k]);
        lv[k] = shift ? lv[k - 1] : (here ? v : lv[k]);
        li[k] = shift ? li[k - 1] : (here ? j : li[k]);
      }
      if (kv_better(v, j, lv[0], li[0])) {
        lv[0] = v;
        li[0] = j;
      }
    }
  };
  auto take = [&](float v, int j) {
    if (lse) lse_take(v);
    if (__builtin_expect(v >= lv[S - 1] && v >= wthr, 0)) insert(v, j);
  };
  constexpr int EPV = BF16 ? 8 : 4;  // elements per 16-byte load
  constexpr int U = 8;                // loads in flight per thread
  if (vec) {
    const int nv = V / EPV;
    // buffer loads over the row: a piece past its end reads as zero, so no load sits under a
    // branch and a batch's U loads are in flight together (a conditional load made the
    // compiler wait for each one)
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(static_cast<const char*>(x) + rowoff * (BF16 ? 2 : 4)), 0, nv * 16,
        kBufferRsrcWord3);
    // the trip count is the same in every lane, so the wave-wide maximum below has all lanes
    for (int q0 = threadIdx.x; q0 - static_cast<int>(threadIdx.x) < nv; q0 += kTopkThreads * U) {
      uint4 t4[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int q = q0 + u * kTopkThreads;
        t4[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, q < nv ? 16 * q : kBufferOutOfRange, 0, 0));
      }
      auto unpack = [&](const uint4& t, float (&v)[EPV]) {
        const uint32_t w4[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const uint32_t word = w4[BF16 ? e / 2 : e];
          v[e] = BF16 ? __uint_as_float((e & 1) ? (word & 0xffff0000u) : (word << 16))
                      : __uint_as_float(word);
        }
      };
      if (q0 == static_cast<int>(threadIdx.x)) {
        // First batch: start the wave threshold at the S-th largest of the lanes' maxima over
        // the batch (S distinct elements reach it, so it bounds the wave's S-th best from
        // below).  Without it every lane's list fills from -inf and the insertion runs in some
        // lane of nearly every early step (s = 16 over 128256: 237 us).
        float mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float v[EPV];
          unpack(t4[u], v);
#pragma unroll
          for (int e = 0; e < EPV; ++e) mx = q0 + u * kTopkThreads < nv ? fmaxf(mx, v[e]) : mx;
        }
        float cur = -INFINITY;
        for (int k = 0; k < S; ++k) {
          cur = wave_max(mx);
          const uint64_t hold = __ballot(mx == cur);  // drop one lane holding it
          if (static_cast<int>(threadIdx.x & 63) == __ffsll(static_cast<long long>(hold)) - 1) mx = -INFINITY;
        }
        wthr = cur;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int q = q0 + u * kTopkThreads;
        if (q >= nv) break;
        float v[EPV];
        unpack(t4[u], v);
        if (lse) {
#pragma unroll
          for (int e = 0; e < EPV; ++e) lse_take(v[e]);
        }
        // one branch per 16-byte piece: its largest element against the thresholds
        float g = v[0];
#pragma unroll
        for (int e = 1; e < EPV; ++e) g = fmaxf(g, v[e]);
        if (__builtin_expect(g >= lv[S - 1] && g >= wthr, 0)) {
#pragma unroll
          for (int e = 0; e < EPV; ++e) insert(v[e], q * EPV + e);
        }
      }
      wthr = fmaxf(wthr, wave_max(lv[S - 1]));
    }
  } else {
    for (int j0 = threadIdx.x; j0 - static_cast<int>(threadIdx.x) < V; j0 += kTopkThreads * U) {
      float tv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + u * kTopkThreads;
        tv[u] = j < V ? load_elem<BF16>(x, rowoff + j) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + u * kTopkThreads;
        if (j >= V) break;
        take(tv[u], j);
      }
      wthr = fmaxf(wthr, wave_max(lv[S - 1]));
    }
  }
  if (lse) {
    wave_ml_merge(m, l);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) {
      sm[w] = m;
      sl[w] = l;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int k = 1; k < NW; ++k) ml_merge(m, l, sm[k], sl[k]);
      lse[blockIdx.x] = m + logf(l);
    }
  }
  // Each wave's top s (wave arg-bests over the lanes' list heads, the owner popping each
  // winner; ids are unique per row), then wave 0 takes the row's top s from the waves' lists.
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int r = 0; r < s; ++r) {
    float bv = lv[0];
    int bi = li[0];
    wave_argbest(bv, bi);
    if (lane == 0) {
      cv[w][r] = bv;
      ci[w][r] = bi;
    }
    if (bi != INT_MAX && li[0] == bi) {
#pragma unroll
      for (int k = 0; k < S - 1; ++k) {
        lv[k] = lv[k + 1];
        li[k] = li[k + 1];
      }
      lv[S - 1] = -INFINITY;
      li[S - 1] = INT_MAX;
    }
  }
  __syncthreads();
  if (w != 0) return;
  constexpr int CPL = (NW * S + 63) / 64;  // candidates per lane
  float hv[CPL];
  int hi[CPL];
#pragma unroll
  for (int t = 0; t < CPL; ++t) {
    const int c = lane + 64 * t;
    const bool ok = c < NW * s;
    hv[t] = ok ? cv[c / s][c % s] : -INFINITY;
    hi[t] = ok ? ci[c / s][c % s] : INT_MAX;
  }
  for (int r = 0; r < s; ++r) {
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
      const bool c = kv_better(hv[t], hi[t], bv, bi);
      bv = c ? hv[t] : bv;
      bi = c ? hi[t] : bi;
    }
    wave_argbest(bv, bi);
    if (lane == 0) {
      const size_t o = static_cast<size_t>(blockIdx.x) * ld_out + r;
      ids[o] = bi == INT_MAX ? -1 : bi;
      if (vals) vals[o] = bv;
    }
    if (bi != INT_MAX) {
#pragma unroll
      for (int t = 0; t < CPL; ++t) {
        const bool hit = hi[t] == bi;
        hv[t] = hit ? -INFINITY : hv[t];
        hi[t] = hit ? INT_MAX : hi[t];
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------
int nct_for(int B) { return B <= 8 ? 1 : (B <= 16 ? 2 : (B <= 32 ? 4 : 8)); }

struct HeadsLayout {
  float* hk = nullptr;
  uint16_t* bpack_hk = nullptr;
  float* pval = nullptr;
  int* pidx = nullptr;
  float* pm = nullptr;
  float* pl = nullptr;
  size_t residual_bytes = 0;  // prefix used by the residual call
  size_t bytes = 0;
};

// Workspace layout.  The residual call's buffers come first so that it can check its part
// without knowing V and s_max.
HeadsLayout heads_layout(void* ws, int dt, int B, int d, int V, int K, int s_max) {
  HeadsLayout L;
  Carver c(ws);
  const int nct = nct_for(B);
  const size_t T = static_cast<size_t>(d) / 32;
  L.hk = c.take<float>(static_cast<size_t>(B) * K * d);
  if (dt == MV_BF16) {
    L.bpack_hk = c.take<uint16_t>(static_cast<size_t>(K) * T * nct * 64 * 8);
  }
  L.residual_bytes = c.bytes();
  const size_t nrb = static_cast<size_t>(ceil_div(V, kRows));
  const size_t np = static_cast<size_t>(K) * B * nrb;
  L.pval = c.take<float>(np * s_max);
  L.pidx = c.take<int>(np * s_max);
  L.pm = c.take<float>(np);
  L.pl = c.take<float>(np);
  L.bytes = c.bytes();
  return L;
}

int check_common(int dt, int B, int d, int K) {
  if (dt != MV_F32 && dt != MV_BF16) return MV_ERR_INVALID_ARG;
  if (B < 1 || d < 1 || K < 1) return MV_ERR_INVALID_ARG;
  if (B > MV_MAX_BATCH_HEADS || K > MV_MAX_HEADS) return MV_ERR_UNSUPPORTED;
  if (dt == MV_F32 && B > kMaxBatchF32) return MV_ERR_UNSUPPORTED;
  if (dt == MV_BF16 && d % 32 != 0) return MV_ERR_UNSUPPORTED;
  if (dt == MV_F32 && d % 4 != 0) return MV_ERR_UNSUPPORTED;
  return MV_OK;
}

// Waves per workgroup: the smallest power of two that gives the launch about MV_GEMV_WAVES
// waves (12 per SIMD) to cover HBM latency, while each wave keeps at least 8 k-steps.
int pick_nw(long long nblocks, int T, int cap) {
  int nw = 1;
  while (nw * 2 <= cap && nblocks * nw < MV_GEMV_WAVES && T / (nw * 2) >= 8) nw *= 2;
  return nw;
}

// The projection takes the row-segment loads where the workgroup has at most 4 waves; the
// residual (8-wave workgroups, which would need 154 KB of staging) loads straight into the
// operand layout.
template <int MODE>
int launch_gemv(int dt, const GemvParams& p, int K, hipStream_t st) {
  const dim3 grid(p.nrb, K);
  if (dt == MV_F32) {
    const int nw = pick_nw(static_cast<long long>(p.nrb) * K, 1 << 30, 8);
    switch (nw) {
      case 1: gemv_f32_kernel<1, MODE><<<grid, 64, 0, st>>>(p); break;
      case 2: gemv_f32_kernel<2, MODE><<<grid, 128, 0, st>>>(p); break;
      case 4: gemv_f32_kernel<4, MODE><<<grid, 256, 0, st>>>(p); break;
      default: gemv_f32_kernel<8, MODE><<<grid, 512, 0, st>>>(p); break;
    }
    return launch_status();
  }
  const int nct = nct_for(p.B);
  const int nw = pick_nw(static_cast<long long>(p.nrb) * K, p.T, 16 / nct > 8 ? 8 : 16 / nct);
#define MV_GEMV_CASE(NW_, NCT_)                                                                  \
  if (nw == NW_ && nct == NCT_) {                                                                \
    if (MODE == 1 && NW_ <= 4)                                                                   \
      gemv_bf16_kernel<NW_, NCT_, MODE, MODE == 1 && NW_ <= 4><<<grid, NW_ * 64, 0, st>>>(p);    \
    else                                                                                         \
      gemv_bf16_kernel<NW_, NCT_, MODE, false><<<grid, NW_ * 64, 0, st>>>(p);                    \
    return launch_status();                                                                      \
  }
  MV_GEMV_CASE(1, 1) MV_GEMV_CASE(2, 1) MV_GEMV_CASE(4, 1) MV_GEMV_CASE(8, 1)
  MV_GEMV_CASE(1, 2) MV_GEMV_CASE(2, 2) MV_GEMV_CASE(4, 2) MV_GEMV_CASE(8, 2)
  MV_GEMV_CASE(1, 4) MV_GEMV_CASE(2, 4) MV_GEMV_CASE(4, 4)
  MV_GEMV_CASE(1, 8) MV_GEMV_CASE(2, 8)
#undef MV_GEMV_CASE
  return MV_ERR_UNSUPPORTED;
}

}  // namespace
}  // namespace mv

using namespace mv;

extern "C" {

MV_API size_t mv_medusa_heads_workspace(int dt, int B, int d, int V, int K, int s_max) {
  if (check_common(dt, B, d, K) != MV_OK || V < 1 || s_max < 1) return 0;
  return heads_layout(nullptr, dt, B, d, V, K, s_max).bytes;
}

MV_API int mv_medusa_residual(int dt, int B, int d, int K, const void* h, const void* w_res,
                              float* hk, void* ws, size_t ws_bytes, void* stream) {
  MV_TRY(check_common(dt, B, d, K));
  if (!h || !w_res) return MV_ERR_INVALID_ARG;
  HeadsLayout need = heads_layout(nullptr, dt, B, d, 1, K, 1);
  MV_TRY(check_ws(ws, ws_bytes, need.residual_bytes));
  HeadsLayout L = heads_layout(ws, dt, B, d, 1, K, 1);
  hipStream_t st = as_stream(stream);
  GemvParams p{};
  p.B = B; p.d = d; p.R = d; p.K = K; p.T = d / 32; p.nrb = ceil_div(d, kRows);
  p.W = w_res; p.h = h; p.hk_ws = L.hk; p.hk_out = hk;
  if (dt == MV_BF16) {
    p.bsrc = nullptr;
    p.bsrc_hstride = 0;
    p.bpack_out = L.bpack_hk;
  } else {
    p.xsrc = static_cast<const float*>(h);
    p.x_bstride = d;
    p.x_hstride = 0;
  }
  return launch_gemv<0>(dt, p, K, st);
}

static int check_select(int V, int K, const int* s_per_head, int s_max) {
  if (V < 1 || !s_per_head) return MV_ERR_INVALID_ARG;
  if (s_max < 1 || s_max > MV_MAX_TOPK || s_max > V) return MV_ERR_UNSUPPORTED;
  for (int k = 0; k < K; ++k)
    if (s_per_head[k] < 1 || s_per_head[k] > s_max) return MV_ERR_INVALID_ARG;
  return MV_OK;
}

static GemvParams head_params(int dt, int B, int d, int V, int K, const int* s_per_head,
                              int s_max, const HeadsLayout& L) {
  GemvParams p{};
  p.B = B; p.d = d; p.R = V; p.K = K; p.T = d / 32; p.nrb = ceil_div(V, kRows);
  p.pval = L.pval; p.pidx = L.pidx; p.pm = L.pm; p.pl = L.pl;
  p.s_max = s_max;
  for (int k = 0; k < K; ++k) p.s[k] = s_per_head[k];
  if (dt == MV_BF16) {
    const int nct = nct_for(B);
    p.bsrc = reinterpret_cast<const u32x4*>(L.bpack_hk);
    p.bsrc_hstride = static_cast<long long>(d / 32) * nct * 64;
  } else {
    p.xsrc = L.hk;
    p.x_bstride = static_cast<long long>(K) * d;
    p.x_hstride = d;
  }
  return p;
}

MV_API int mv_medusa_head_project(int dt, int B, int d, int V, int K, const int* s_per_head,
                                  int s_max, const void* w_head, void* logits, void* ws,
                                  size_t ws_bytes, void* stream) {
  MV_TRY(check_common(dt, B, d, K));
  MV_TRY(check_select(V, K, s_per_head, s_max));
  if (!w_head) return MV_ERR_INVALID_ARG;
  MV_TRY(check_ws(ws, ws_bytes, heads_layout(nullptr, dt, B, d, V, K, s_max).bytes));
  const HeadsLayout L = heads_layout(ws, dt, B, d, V, K, s_max);
  GemvParams p = head_params(dt, B, d, V, K, s_per_head, s_max, L);
  p.W = w_head;
  p.logits = logits;
  return launch_gemv<1>(dt, p, K, as_stream(stream));
}

MV_API int mv_medusa_head_select(int dt, int B, int d, int V, int K, const int* s_per_head,
                                 int s_max, int32_t* topk_ids, float* topk_vals, int ld_topk,
                                 float* lse, void* ws, size_t ws_bytes, void* stream) {
  MV_TRY(check_common(dt, B, d, K));
  MV_TRY(check_select(V, K, s_per_head, s_max));
  if (!topk_ids || !topk_vals) return MV_ERR_INVALID_ARG;
  if (ld_topk == 0) ld_topk = K * s_max;
  if (ld_topk < K * s_max) return MV_ERR_INVALID_ARG;
  MV_TRY(check_ws(ws, ws_bytes, heads_layout(nullptr, dt, B, d, V, K, s_max).bytes));
  const HeadsLayout L = heads_layout(ws, dt, B, d, V, K, s_max);
  GemvParams p = head_params(dt, B, d, V, K, s_per_head, s_max, L);
  p.topk_ids = topk_ids;
  p.topk_vals = topk_vals;
  p.ld_topk = ld_topk;
  p.lse = lse;
  hipStream_t st = as_stream(stream);
  // Lists of up to 8 slots: per-thread sorted lists.  Longer (up to 16): a k-way merge of the
  // blocks' lists when every thread holds at most two of them, else a tournament over the
  // candidates held in registers when they fit (up to 32 per thread), else the 16-slot lists.
  const long long n = static_cast<long long>(p.nrb) * s_max;
  if (s_max <= 4) heads_merge_kernel<4><<<K * B, kMergeThreads, 0, st>>>(p);
  else if (s_max <= 8) heads_merge_kernel<8><<<K * B, kMergeThreads, 0, st>>>(p);
  else if (p.nrb <= 2 * kMergeThreads) heads_kmerge_kernel<2, MV_MAX_TOPK><<<K * B, kMergeThreads, 0, st>>>(p);
  else if (n <= 16LL * kMergeThreads) heads_tournament_kernel<16><<<K * B, kMergeThreads, 0, st>>>(p);
  else if (n <= 32LL * kMergeThreads) heads_tournament_kernel<32><<<K * B, kMergeThreads, 0, st>>>(p);
  else heads_merge_kernel<MV_MAX_TOPK><<<K * B, kMergeThreads, 0, st>>>(p);
  return launch_status();
}

MV_API int mv_medusa_heads(int dt, int B, int d, int V, int K, const int* s_per_head, int s_max,
                           const void* h, const void* w_res, const void* w_head, float* hk,
                           void* logits, int32_t* topk_ids, float* topk_vals, int ld_topk,
                           float* lse, void* ws, size_t ws_bytes, void* stream) {
  MV_TRY(check_common(dt, B, d, K));
  if (V < 1 || !s_per_head || !w_head || !topk_ids || !topk_vals) return MV_ERR_INVALID_ARG;
  if (s_max < 1 || s_max > MV_MAX_TOPK || s_max > V) return MV_ERR_UNSUPPORTED;
  for (int k = 0; k < K; ++k)
    if (s_per_head[k] < 1 || s_per_head[k] > s_max) return MV_ERR_INVALID_ARG;
  if (ld_topk != 0 && ld_topk < K * s_max) return MV_ERR_INVALID_ARG;
  MV_TRY(check_ws(ws, ws_bytes, heads_layout(nullptr, dt, B, d, V, K, s_max).bytes));
  MV_TRY(mv_medusa_residual(dt, B, d, K, h, w_res, hk, ws, ws_bytes, stream));
  MV_TRY(mv_medusa_head_project(dt, B, d, V, K, s_per_head, s_max, w_head, logits, ws, ws_bytes,
                                stream));
  return mv_medusa_head_select(dt, B, d, V, K, s_per_head, s_max, topk_ids, topk_vals, ld_topk,
                               lse, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {
constexpr int kScratchMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kScratchMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device (with that
// device current) and kept.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchMaxDevices) return MV_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return MV_ERR_HIP;
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return MV_OK;
}
}  // namespace

extern "C" {

MV_API int mv_medusa_heads_noalloc(int dt, int B, int d, int V, int K, const int* s_per_head,
                                   int s_max, const void* h, const void* w_res,
                                   const void* w_head, float* hk, void* logits,
                                   int32_t* topk_ids, float* topk_vals, int ld_topk, float* lse,
                                   void* stream) {
  MV_TRY(check_common(dt, B, d, K));
  if (V < 1) return MV_ERR_INVALID_ARG;
  if (s_max < 1 || s_max > MV_MAX_TOPK || s_max > V) return MV_ERR_UNSUPPORTED;
  // the size check comes before anything touches the device
  const size_t need = heads_layout(nullptr, dt, B, d, V, K, s_max).bytes;
  if (need > static_cast<size_t>(MV_HEADS_NOALLOC_SCRATCH_BYTES)) return MV_ERR_UNSUPPORTED;
  void* ws = nullptr;
  MV_TRY(scratch_address(&ws));
  // the three kernels write every scratch byte they later read, so nothing is cleared
  return mv_medusa_heads(dt, B, d, V, K, s_per_head, s_max, h, w_res, w_head, hk, logits,
                         topk_ids, topk_vals, ld_topk, lse, ws,
                         static_cast<size_t>(MV_HEADS_NOALLOC_SCRATCH_BYTES), stream);
}

MV_API int mv_topk_rows(int dt, int R, int V, int s, const void* x, long long ldx, int32_t* ids,
                        float* vals, int ld_out, float* lse, void* stream) {
  if (dt != MV_F32 && dt != MV_BF16) return MV_ERR_INVALID_ARG;
  if (R < 1 || V < 1 || !x || !ids) return MV_ERR_INVALID_ARG;
  if (s < 1 || s > MV_MAX_TOPK || s > V) return MV_ERR_UNSUPPORTED;
  if (ldx < V || ld_out < s) return MV_ERR_INVALID_ARG;
  hipStream_t st = as_stream(stream);
  const int epv = dt == MV_BF16 ? 8 : 4;
  // (16-byte pieces through a buffer resource over one row: its bytes must fit the 31-bit offsets)
  const int vec = (V % epv == 0 && ldx % epv == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
                   static_cast<long long>(V) * (dt == MV_BF16 ? 2 : 4) < 0x7fffffffLL) ? 1 : 0;
  // 1024 threads per row for long rows (the Llama-3 vocabulary: 79 us against 137 us with 256
  // for 256 rows), 256 for short ones, where the launch and the final arg-bests dominate
#define MV_TOPK_CASE(S_, NT_)                                                                     \
  if (s <= S_) {                                                                                  \
    if (dt == MV_BF16) topk_rows_kernel<true, S_, NT_><<<R, NT_, 0, st>>>(V, s, x, ldx, ids, vals, ld_out, lse, vec); \
    else topk_rows_kernel<false, S_, NT_><<<R, NT_, 0, st>>>(V, s, x, ldx, ids, vals, ld_out, lse, vec); \
    return launch_status();                                                                       \
  }
  if (V >= 32768) {
    MV_TOPK_CASE(4, 1024) MV_TOPK_CASE(8, 1024) MV_TOPK_CASE(16, 1024)
  } else {
    MV_TOPK_CASE(4, 256) MV_TOPK_CASE(8, 256) MV_TOPK_CASE(16, 256)
  }
#undef MV_TOPK_CASE
  return MV_ERR_UNSUPPORTED;
}

}  // extern "C"
