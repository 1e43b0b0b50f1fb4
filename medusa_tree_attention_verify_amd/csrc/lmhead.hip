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
// Up to 128 target rows: one streaming pass over W per group of rows (lm_head_kernel).  More
// rows: a tiled GEMM over 256-row vocabulary blocks (lm_head_gemm_kernel), which reads W once
// per block of 128 or 256 target rows through LDS.  Both write per (row, vocabulary block)
// partials; a second kernel merges each row's partials into the greedy id and the LSE.

#include <math.h>

#include <algorithm>

#include "mv_device.h"
#include "mv_host.h"

namespace mv {
namespace {

constexpr int kLmMergeThreads = 256;

struct LmParams {
  int T, d, V, KT, nrb;         // KT = d / 32, nrb = vocabulary blocks (of 64, 128 or 256 rows)
  const uint16_t* x;            // [T][d] bf16
  const uint16_t* w;            // [V][d] bf16
  float* pm;                    // [T][nrb] partial max
  float* pl;                    // [T][nrb] partial sum exp(logit - max)
  int* pidx;                    // [T][nrb] id of the partial max (lowest on ties)
  int32_t* ids;                 // [T]
  float* maxv;                  // [T] or null
  float* lse;                   // [T] or null
  // Rows mode (terminal rows of speculative acceptance): target row t is x row
  // t * xrow_mul + xrow[t * xrow_stride] (xrow null: row t), and the kernel writes
  // rows_out[t][v] = exp(logit - lse_in[that row]) instead of partials.
  const int* xrow;
  int xrow_stride, xrow_mul;
  const float* lse_in;
  float* rows_out;              // [T][V]
};

__device__ __forceinline__ int lm_xrow(const LmParams& p, int t) {
  return p.xrow ? t * p.xrow_mul + p.xrow[static_cast<size_t>(t) * p.xrow_stride] : t;
}

// Streaming kernel.  A workgroup owns 64 or 128 vocabulary rows (4 or 8 waves, one 16-row MFMA
// tile per wave) and a group of up to 128 target rows (NCT column tiles of 16).  Each wave
// streams its 16 weight rows over the whole of d as the A operand of v_mfma_f32_16x16x32_bf16
// (one 16-byte load per lane and k-step, U k-steps per batch, the next batch in registers), so
// every weight byte crosses HBM once per target-row group.  The target rows' slice of x for a
// batch is staged in LDS once for all the waves (double-buffered, the next batch in registers)
// and read back as the B operand; an 80-byte row pitch makes those 16-byte reads conflict-free.
// Epilogue per column tile: each wave reduces its 16 rows for every target row in registers
// (lane swaps between the four 16-lane groups), the waves meet in LDS, and the workgroup writes
// per target row the partial (max, its id, sum exp(logit - max)) of its vocabulary block.
constexpr int kLmXPitch = 40;  // bf16 elements per staged target row (32 + 8 padding)
constexpr int kLmUPad = 32;    // bf16 elements between the k-step slices of one x batch

// Waves per workgroup (16 vocabulary rows each): 8 in rows mode, and where a workgroup's x
// buffers exceed 80 KB (8 column tiles with 4-step batches), so that two 4-wave workgroups
// would not fit one CU's 160 KB of LDS; else 4.
constexpr int lm_waves(int nct, int u, bool rows) {
  return rows || 2 * u * (16 * nct * kLmXPitch + kLmUPad) * 2 > 80 * 1024 ? 8 : 4;
}

template <int NCT, int U, bool ROWS>
__global__ __launch_bounds__(64 * lm_waves(NCT, U, ROWS)) void lm_head_kernel(const LmParams p) {
  constexpr int NWV = lm_waves(NCT, U, ROWS), NT = 64 * NWV;
  constexpr int NCOL = 16 * NCT;
  constexpr int XP = NCOL * 4 * U;            // 16-byte pieces of one x batch
  constexpr int XPT = (XP + NT - 1) / NT;     // per thread
  __shared__ __attribute__((aligned(16))) uint16_t Xs[2][U][NCOL * kLmXPitch + kLmUPad];
  __shared__ float em[NWV][NCOL], es[NWV][NCOL];
  __shared__ int ei[NWV][NCOL];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rb = blockIdx.x, row0 = rb * 16 * NWV, col0 = blockIdx.y * NCOL;
  const int nb = p.KT / U;
  // A operand: lane (row r = lane % 16, k-group g = lane / 16) of wave w reads the 16 bytes
  // W[row0 + 16w + r][32t + 8g .. +8] at k-step t; rows past V are clamped (not used).
  const uint16_t* wp = p.w + static_cast<size_t>(min(row0 + 16 * w + (lane & 15), p.V - 1)) * p.d + 8 * (lane >> 4);
  auto wload = [&](int bt, u32x4 (&a)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) a[u] = *reinterpret_cast<const u32x4*>(wp + static_cast<size_t>(bt * U + u) * 32);
  };
  // x batch bt: piece q = (target row c, u, quarter qq) is x[col0 + c][32*(bt*U + u) + 8*qq .. +8],
  // so 4U consecutive lanes read one row's 64U contiguous bytes (16 rows x 64 bytes per load
  // instruction, the previous order, put every piece of an instruction 8 KB apart at d = 4096);
  // target rows past T read row T-1 (their results are not written).
  // a thread's pieces keep their target rows in every batch: their row starts are found once
  // (in rows mode through the gathered row index, a load the batches then do not repeat)
  const uint16_t* xrp[XPT];
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int q = tid + i * NT;
    const int c = q / (4 * U), u = (q / 4) % U, qq = q % 4;
    const int t = min(col0 + c, p.T - 1);
    xrp[i] = p.x + static_cast<size_t>(ROWS ? lm_xrow(p, t) : t) * p.d + 32 * u + 8 * qq;
  }
  auto xload = [&](int bt, u32x4 (&xr)[XPT]) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int q = tid + i * NT;
      if (XP % NT == 0 || q < XP) xr[i] = *reinterpret_cast<const u32x4*>(xrp[i] + 32 * bt * U);
    }
  };
  // (the k-step slices sit kLmUPad elements further apart than their size, 16 banks, so the
  // 16 lanes of one row store to distinct banks)
  auto xstore = [&](int buf, const u32x4 (&xr)[XPT]) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int q = tid + i * NT;
      if (XP % NT == 0 || q < XP) {
        const int c = q / (4 * U), u = (q / 4) % U, qq = q % 4;
        *reinterpret_cast<u32x4*>(&Xs[buf][u][c * kLmXPitch + 8 * qq]) = xr[i];
      }
    }
  };
  f32x4 acc[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf, const u32x4 (&a)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        // B operand: lane (target row c = lane % 16, k-group g) reads x[16ct + c][8g .. +8]
        const u32x4 bop = *reinterpret_cast<const u32x4*>(&Xs[buf][u][(16 * ct + (lane & 15)) * kLmXPitch + 8 * (lane >> 4)]);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[u]),
                                                          __builtin_bit_cast(bf16x8, bop), acc[ct], 0, 0, 0);
      }
  };
  // Batch bt computes from LDS buffer bt & 1 with weights in register set bt & 1; the x batch
  // bt+1 (already in registers) is stored to the other buffer after the compute, then batch
  // bt+2 is requested into the registers just freed.
  u32x4 xr[XPT], wa0[U], wa1[U];
  xload(0, xr);
  wload(0, wa0);
  xstore(0, xr);
  if (nb > 1) {
    xload(1, xr);
    wload(1, wa1);
  }
  __syncthreads();
  for (int bt = 0; bt < nb; bt += 2) {
    compute(0, wa0);
    if (bt + 1 < nb) xstore(1, xr);
    if (bt + 2 < nb) {
      xload(bt + 2, xr);
      wload(bt + 2, wa0);
    }
    __syncthreads();
    if (bt + 1 < nb) {
      compute(1, wa1);
      if (bt + 2 < nb) xstore(0, xr);
      if (bt + 3 < nb) {
        xload(bt + 3, xr);
        wload(bt + 3, wa1);
      }
    }
    __syncthreads();
  }

  // Epilogue.  acc[ct][v]: vocabulary row row0 + 16w + 4*(lane/16) + v, target row
  // col0 + 16ct + lane%16; the four 16-lane groups hold the other rows of the same target rows.
  const int c16 = lane & 15;
  if constexpr (ROWS) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int t = col0 + 16 * ct + c16;
      if (t >= p.T) continue;
      // exp in fp32: the rows are stored in fp32 (the residual sums over them run in fp64)
      const float lse = p.lse_in[lm_xrow(p, t)];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = row0 + 16 * w + 4 * (lane >> 4) + v;
        if (r < p.V) p.rows_out[static_cast<size_t>(t) * p.V + r] = expf(acc[ct][v] - lse);
      }
    }
    return;
  }
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = row0 + 16 * w + 4 * (lane >> 4) + v;
      const float val = r < p.V ? acc[ct][v] : -INFINITY;
      if (kv_better(val, r, bv, bi)) {
        bv = val;
        bi = r;
      }
    }
#pragma unroll
    for (int step = 0; step < 2; ++step) {
      const LanePair tv = step == 0 ? swap16(__float_as_uint(bv)) : swap32(__float_as_uint(bv));
      const LanePair ti = step == 0 ? swap16(static_cast<uint32_t>(bi)) : swap32(static_cast<uint32_t>(bi));
      bv = __uint_as_float(tv.a);
      bi = static_cast<int>(ti.a);
      if (kv_better(__uint_as_float(tv.b), static_cast<int>(ti.b), bv, bi)) {
        bv = __uint_as_float(tv.b);
        bi = static_cast<int>(ti.b);
      }
    }
    float sm = 0.f;
    if (bv != -INFINITY) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = row0 + 16 * w + 4 * (lane >> 4) + v;
        sm += r < p.V ? expf(acc[ct][v] - bv) : 0.f;
      }
    }
    {
      LanePair t2 = swap16(__float_as_uint(sm));
      sm = __uint_as_float(t2.a) + __uint_as_float(t2.b);
      t2 = swap32(__float_as_uint(sm));
      sm = __uint_as_float(t2.a) + __uint_as_float(t2.b);
    }
    if (lane < 16) {
      em[w][16 * ct + c16] = bv;
      ei[w][16 * ct + c16] = bi;
      es[w][16 * ct + c16] = sm;
    }
  }
  __syncthreads();
  for (int c = tid; c < NCOL; c += NT) {
    const int tok = col0 + c;
    if (tok >= p.T) break;
    float m = em[0][c], l = es[0][c], bv = em[0][c];
    int bi = ei[0][c];
#pragma unroll
    for (int q = 1; q < NWV; ++q) {
      if (kv_better(em[q][c], ei[q][c], bv, bi)) {
        bv = em[q][c];
        bi = ei[q][c];
      }
      ml_merge(m, l, em[q][c], es[q][c]);
    }
    const size_t o = static_cast<size_t>(tok) * p.nrb + rb;
    p.pm[o] = m;
    p.pl[o] = l;
    p.pidx[o] = bi;
  }
}

// Tiled kernel for many target rows (batched verify steps).  Streaming W once per 128 rows
// re-reads it ceil(T/128) times; past that the product is a GEMM whose matrix-core work
// (2*T*V*d FLOPs) outweighs the weight bytes, so both operands go through LDS in large tiles.
// A workgroup owns 256 vocabulary rows x BN target rows, split over WM x WN waves (two per
// SIMD, so one wave's MFMAs run while the other waits on its LDS operand reads); each wave owns
// a (256/WM) x (BN/WN) block of v_mfma_f32_32x32x16_bf16 accumulators (A operand: weight rows,
// B operand: target rows, both K-contiguous).  d advances 64 columns per stage through two
// LDS buffers; the global loads run two stages ahead in two register sets.  Loads are buffer
// loads over the workgroup's own weight and target slabs, so rows past V or T read as zeros
// with no load under a branch.  The epilogue writes the same per-(target row, vocabulary
// block) partials as the streaming kernel, with 256-row blocks.  Jobs (vocabulary block,
// target block) are dealt to the 8 XCDs in contiguous runs, in an order chosen so that the
// workgroups resident on one XCD share operand slabs in L2 (below).
constexpr int kLgRows = 256;                 // vocabulary rows per workgroup
constexpr int kLgBK = 64;                    // columns of d per stage
constexpr int kLgPitch = kLgBK + 8;          // LDS row pitch (elements): conflict-free 16-byte reads
constexpr int kXcds = 8;                     // MI355X hands workgroups to its 8 XCDs round-robin
// Job order: strips of 8 vocabulary blocks when the target rows' hidden states exceed 24 MB
// (4160 x 4096: 4195 -> 4046 us, their re-fetches from beyond L2 being the larger stream),
// else target block fastest (520 x 8192, where the 4 MB weight slabs are the operand worth
// sharing: 397 us against 439 us with strips of 8).
constexpr int kLgStrip = 8;
constexpr size_t kLgStripMinXBytes = 24u << 20;

template <int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void lm_head_gemm_kernel(const LmParams p, int ntb, int jobs, int sv) {
  constexpr int NT = WM * WN * 64;
  constexpr int RM = kLgRows / WM, RN = BN / WN;     // rows of a wave's block
  constexpr int NI = RM / 32, NJ = RN / 32;          // 32-row blocks per wave
  constexpr int PA = kLgRows * kLgBK / 8 / NT;       // 16-byte pieces per thread and stage
  constexpr int PB = BN * kLgBK / 8 / NT;
  static_assert(NI >= 1 && NJ >= 1 && PA >= 1 && PB >= 1, "tile shape");
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kLgRows * kLgPitch];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * kLgPitch];
  __shared__ float em[WM][BN], es[WM][BN];
  __shared__ int ei[WM][BN];
  // The accumulators live in the matrix-core register file.
  asm volatile("" ::: "a0");

  const int per = (jobs + kXcds - 1) / kXcds;
  const int job = static_cast<int>(blockIdx.x % kXcds) * per + static_cast<int>(blockIdx.x / kXcds);
  if (job >= jobs) return;
  // strips of sv vocabulary blocks x every target block, vocabulary block fastest: with sv = 8
  // the ~32 workgroups resident on an XCD cover 8 vocabulary x 4 target blocks and share both
  // slabs; sv = 1 is target block fastest (the weight slab shared, the target slabs streamed)
  const int nvb = p.nrb;
  const int strip = job / (sv * ntb), r = job - strip * sv * ntb;
  const int gv = min(sv, nvb - strip * sv);
  const int vb = strip * sv + r % gv, tb = r / gv;
  const int row0 = vb * kLgRows, col0 = tb * BN;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w % WM, wn = w / WM, l32 = lane & 31, half = lane >> 5;

  const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p.w + static_cast<size_t>(row0) * p.d), 0,
      min(kLgRows, p.V - row0) * p.d * 2, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p.x + static_cast<size_t>(col0) * p.d), 0,
      min(BN, p.T - col0) * p.d * 2, kBufferRsrcWord3);
  const int nk = p.d / kLgBK;
  // piece q = tid + NT i: row q / 8, 16-byte chunk q % 8 of the stage's 64 columns.  The two
  // requests past the last stage re-read it (never used), so the loads carry no condition.
  auto gload = [&](int s, u32x4 (&ra)[PA], u32x4 (&rb)[PB]) {
    const int k0 = min(s, nk - 1) * kLgBK;
#pragma unroll
    for (int i = 0; i < PA; ++i) {
      const int q = tid + i * NT;
      const int off = ((q >> 3) * p.d + k0 + (q & 7) * 8) * 2;
      ra[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ars, off, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int q = tid + i * NT;
      const int off = ((q >> 3) * p.d + k0 + (q & 7) * 8) * 2;
      rb[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(brs, off, 0, 0));
    }
  };
  auto swrite = [&](int buf, const u32x4 (&ra)[PA], const u32x4 (&rb)[PB]) {
#pragma unroll
    for (int i = 0; i < PA; ++i) {
      const int q = tid + i * NT;
      *reinterpret_cast<u32x4*>(&As[buf][(q >> 3) * kLgPitch + (q & 7) * 8]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int q = tid + i * NT;
      *reinterpret_cast<u32x4*>(&Bs[buf][(q >> 3) * kLgPitch + (q & 7) * 8]) = rb[i];
    }
  };
  f32x16 acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  // Operands of one 16-column k-step: lane (row l32, column group half) reads 8 consecutive
  // columns of its weight row (A) and of its target row (B).  The next k-step's operands are
  // read while this one's MFMAs run (two fragment sets), one LDS read placed after each MFMA
  // by scheduling groups: 5% over the compiler's own order, which waited on each read just
  // before its first use.
  auto ldf = [&](int buf, int ks, bf16x8 (&a)[NI], bf16x8 (&b)[NJ]) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      a[i] = *reinterpret_cast<const bf16x8*>(&As[buf][(RM * wm + 32 * i + l32) * kLgPitch + ks * 16 + half * 8]);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      b[j] = *reinterpret_cast<const bf16x8*>(&Bs[buf][(RN * wn + 32 * j + l32) * kLgPitch + ks * 16 + half * 8]);
  };
  auto mm = [&](const bf16x8 (&a)[NI], const bf16x8 (&b)[NJ]) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  };
  auto interleave = [&]() {  // DS read / MFMA alternation, then the remaining MFMAs
#pragma unroll
    for (int q = 0; q < NI + NJ; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NI * NJ - (NI + NJ), 0);
  };
  static_assert(NI * NJ >= NI + NJ && (kLgBK / 16) % 2 == 0, "interleave shape");
  auto compute = [&](int buf) {
    bf16x8 a0[NI], b0[NJ], a1[NI], b1[NJ];
    ldf(buf, 0, a0, b0);
#pragma unroll
    for (int ks = 0; ks < kLgBK / 16; ks += 2) {
      ldf(buf, ks + 1, a1, b1);
      mm(a0, b0);
      interleave();
      if (ks + 2 < kLgBK / 16) {
        ldf(buf, ks + 2, a0, b0);
        mm(a1, b1);
        interleave();
      } else {
        mm(a1, b1);
      }
    }
  };
  // Stage s computes from LDS buffer s & 1.  Registers: set 0 holds stage s + 2 (requested at
  // the top of the iteration), set 1 stage s + 1 (arrived), stored once buffer 1 is free.
  u32x4 ra0[PA], rb0[PB], ra1[PA], rb1[PB];
  gload(0, ra0, rb0);
  gload(1, ra1, rb1);
  swrite(0, ra0, rb0);
  __syncthreads();
  for (int s = 0; s < nk; s += 2) {  // nk is even (d % 128 == 0)
    gload(s + 2, ra0, rb0);
    compute(0);
    swrite(1, ra1, rb1);
    __syncthreads();
    gload(s + 3, ra1, rb1);
    compute(1);
    swrite(0, ra0, rb0);
    __syncthreads();
  }

  // Epilogue.  acc[i][j][v]: vocabulary row row0 + RM wm + 32 i + 8 (v / 4) + 4 half + v % 4,
  // target row col0 + RN wn + 32 j + l32; lanes l and l ^ 32 hold the two row halves.
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = row0 + RM * wm + 32 * i + 8 * (v >> 2) + 4 * half + (v & 3);
        const float val = r < p.V ? acc[i][j][v] : -INFINITY;
        if (kv_better(val, r, bv, bi)) {
          bv = val;
          bi = r;
        }
      }
    {
      const LanePair tv = swap32(__float_as_uint(bv)), ti = swap32(static_cast<uint32_t>(bi));
      bv = __uint_as_float(tv.a);
      bi = static_cast<int>(ti.a);
      if (kv_better(__uint_as_float(tv.b), static_cast<int>(ti.b), bv, bi)) {
        bv = __uint_as_float(tv.b);
        bi = static_cast<int>(ti.b);
      }
    }
    float sm = 0.f;
    if (bv != -INFINITY) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = row0 + RM * wm + 32 * i + 8 * (v >> 2) + 4 * half + (v & 3);
          sm += r < p.V ? expf(acc[i][j][v] - bv) : 0.f;
        }
    }
    {
      const LanePair t2 = swap32(__float_as_uint(sm));
      sm = __uint_as_float(t2.a) + __uint_as_float(t2.b);
    }
    if (half == 0) {
      const int c = RN * wn + 32 * j + l32;
      em[wm][c] = bv;
      ei[wm][c] = bi;
      es[wm][c] = sm;
    }
  }
  __syncthreads();
  for (int c = tid; c < BN; c += NT) {
    const int tok = col0 + c;
    if (tok >= p.T) break;
    float m = em[0][c], l = es[0][c], bv = em[0][c];
    int bi = ei[0][c];
#pragma unroll
    for (int q = 1; q < WM; ++q) {
      if (kv_better(em[q][c], ei[q][c], bv, bi)) {
        bv = em[q][c];
        bi = ei[q][c];
      }
      ml_merge(m, l, em[q][c], es[q][c]);
    }
    const size_t o = static_cast<size_t>(tok) * p.nrb + vb;
    p.pm[o] = m;
    p.pl[o] = l;
    p.pidx[o] = bi;
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
  int nrb = 1, nct = 1, ncols = 16, ngrp = 1, u = 1;
  int gemm_bn = 0;  // > 0: the tiled kernel with this many target rows per workgroup
  int ntb = 0, jobs = 0;
  size_t ws_bytes = 0;
};

// Column tiles per workgroup: the smallest instantiated count that covers T, at most 8 (128
// target rows; more rows run as several groups, each streaming W again).  Wider groups were
// measured slower: 32 tiles at 520 target rows took 613 us against 506 us for groups of 128 rows
// with the previous kernel, because every workgroup restages the whole x tile (its 64 weight
// rows reuse it only 64-fold) and the 32-tile kernel runs one wave per SIMD.  k-steps per
// batch: 4 (2 or 1 when d/32 is not a multiple).
constexpr int kLmNct[] = {1, 2, 3, 4, 5, 6, 7, 8};
constexpr int kLmMaxNct = 8;

// Tiled-kernel choices, from a sweep over T = 130..4160 (d = 4096 and 8192): 8 waves (two per
// SIMD) beat 4 waves with one per SIMD by 10-20%, 4 x 2 wave grids beat 2 x 4 by up to 7%, and
// 256-row target tiles only pay once the 128-row tiles' extra weight re-reads outweigh the
// padding of the last tile (equal at 2080 rows, 1.5% ahead at 4160).
#ifndef MV_LG256_WM
#define MV_LG256_WM 4  // wave grid of the tiled kernel: 4 x 2 waves for 256 target rows
#define MV_LG256_WN 2
#endif
#ifndef MV_LG128_WM
#define MV_LG128_WM 4  // ... and for 128
#define MV_LG128_WN 2
#endif
#ifndef MV_LM_GEMM_MIN_T
#define MV_LM_GEMM_MIN_T 129  // target rows from which the tiled kernel runs
#endif
#ifndef MV_LM_GEMM_BN256_MIN_T
#define MV_LM_GEMM_BN256_MIN_T 2049  // ... and from which it takes 256 target rows per workgroup
#endif

LmPlan plan_lm(int T, int d, int V) {
  LmPlan a;
  // (the tiled kernel's buffer ranges cover 256 rows x d bf16, so d stays far below 2^22)
  if (T >= MV_LM_GEMM_MIN_T && d % (2 * kLgBK) == 0 && d <= (1 << 20)) {
    a.gemm_bn = T >= MV_LM_GEMM_BN256_MIN_T ? 256 : 128;
    a.nrb = ceil_div(V, kLgRows);
    a.ntb = ceil_div(T, a.gemm_bn);
    a.jobs = a.nrb * a.ntb;
    Carver c(nullptr);
    const size_t np = static_cast<size_t>(T) * a.nrb;
    c.take<float>(np);
    c.take<float>(np);
    c.take<int>(np);
    a.ws_bytes = c.bytes();
    return a;
  }
  const int need = ceil_div(std::min(T, 16 * kLmMaxNct), 16);
  for (int n : kLmNct)
    if (n >= need) {
      a.nct = n;
      break;
    }
  a.ncols = 16 * a.nct;
  a.ngrp = ceil_div(T, a.ncols);
  const int KT = d / 32;
  a.u = KT % 4 == 0 ? 4 : (KT % 2 == 0 ? 2 : 1);
  a.nrb = ceil_div(V, 16 * lm_waves(a.nct, a.u, false));
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
  p.T = T; p.d = d; p.V = V; p.KT = d / 32; p.nrb = a.nrb;
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
  if (a.gemm_bn > 0) {
    const int grid = ceil_div(a.jobs, kXcds) * kXcds;
    const int sv = static_cast<size_t>(T) * d * 2 > kLgStripMinXBytes ? kLgStrip : 1;
    if (a.gemm_bn == 256)
      lm_head_gemm_kernel<256, MV_LG256_WM, MV_LG256_WN><<<grid, MV_LG256_WM * MV_LG256_WN * 64, 0, st>>>(p, a.ntb, a.jobs, sv);
    else
      lm_head_gemm_kernel<128, MV_LG128_WM, MV_LG128_WN><<<grid, MV_LG128_WM * MV_LG128_WN * 64, 0, st>>>(p, a.ntb, a.jobs, sv);
    MV_TRY(launch_status());
    lm_head_merge_kernel<<<T, kLmMergeThreads, 0, st>>>(p);
    return launch_status();
  }
  const dim3 grid(a.nrb, a.ngrp);
  bool launched = false;
#define MV_LM_CASE(NCT_, U_) \
  if (!launched && a.nct == NCT_ && a.u == U_) { lm_head_kernel<NCT_, U_, false><<<grid, 64 * lm_waves(NCT_, U_, false), 0, st>>>(p); launched = true; }
  MV_LM_CASE(1, 4) MV_LM_CASE(2, 4) MV_LM_CASE(3, 4) MV_LM_CASE(4, 4)
  MV_LM_CASE(5, 4) MV_LM_CASE(6, 4) MV_LM_CASE(7, 4) MV_LM_CASE(8, 4)
  MV_LM_CASE(1, 2) MV_LM_CASE(2, 2) MV_LM_CASE(3, 2) MV_LM_CASE(4, 2)
  MV_LM_CASE(5, 2) MV_LM_CASE(6, 2) MV_LM_CASE(7, 2) MV_LM_CASE(8, 2)
  MV_LM_CASE(1, 1) MV_LM_CASE(2, 1) MV_LM_CASE(3, 1) MV_LM_CASE(4, 1)
  MV_LM_CASE(5, 1) MV_LM_CASE(6, 1) MV_LM_CASE(7, 1) MV_LM_CASE(8, 1)
#undef MV_LM_CASE
  if (!launched) return MV_ERR_UNSUPPORTED;  // no kernel instance for this shape
  MV_TRY(launch_status());
  lm_head_merge_kernel<<<T, kLmMergeThreads, 0, st>>>(p);
  return launch_status();
}

}  // extern "C"

namespace mv {

// Probability rows exp(W x - LSE) of T gathered target rows (one streaming pass over W per
// group of up to 128 rows): the terminal rows of speculative acceptance from the LM head.
int lm_head_prob_rows(int T, int d, int V, const uint16_t* x, const int* xrow, int xrow_stride,
                      int xrow_mul, const float* lse_in, const uint16_t* w, float* rows_out,
                      hipStream_t st) {
  if (T < 1 || V < 1 || d < 32 || d % 32 != 0) return MV_ERR_UNSUPPORTED;
  LmParams p{};
  p.T = T; p.d = d; p.V = V; p.KT = d / 32;
  p.x = x; p.w = w;
  p.xrow = xrow; p.xrow_stride = xrow_stride; p.xrow_mul = xrow_mul;
  p.lse_in = lse_in; p.rows_out = rows_out;
  const int nct = ceil_div(std::min(T, 16 * kLmMaxNct), 16);
  const int u = p.KT % 4 == 0 ? 4 : (p.KT % 2 == 0 ? 2 : 1);
  p.nrb = ceil_div(V, 16 * lm_waves(nct, u, true));
  const dim3 grid(p.nrb, ceil_div(T, 16 * nct));
  bool launched = false;
#define MV_LMR_CASE(NCT_, U_) \
  if (!launched && nct == NCT_ && u == U_) { lm_head_kernel<NCT_, U_, true><<<grid, 64 * lm_waves(NCT_, U_, true), 0, st>>>(p); launched = true; }
  MV_LMR_CASE(1, 4) MV_LMR_CASE(2, 4) MV_LMR_CASE(3, 4) MV_LMR_CASE(4, 4)
  MV_LMR_CASE(5, 4) MV_LMR_CASE(6, 4) MV_LMR_CASE(7, 4) MV_LMR_CASE(8, 4)
  MV_LMR_CASE(1, 2) MV_LMR_CASE(2, 2) MV_LMR_CASE(3, 2) MV_LMR_CASE(4, 2)
  MV_LMR_CASE(5, 2) MV_LMR_CASE(6, 2) MV_LMR_CASE(7, 2) MV_LMR_CASE(8, 2)
  MV_LMR_CASE(1, 1) MV_LMR_CASE(2, 1) MV_LMR_CASE(3, 1) MV_LMR_CASE(4, 1)
  MV_LMR_CASE(5, 1) MV_LMR_CASE(6, 1) MV_LMR_CASE(7, 1) MV_LMR_CASE(8, 1)
#undef MV_LMR_CASE
  if (!launched) return MV_ERR_UNSUPPORTED;
  return launch_status();
}

}  // namespace mv
