// Acceptance on gfx950: greedy longest accepted path, or the speculative rule with residual
// resampling, plus the extra token that follows the committed path.
//
// Sources: "Medusa Explained: Multi-Head Speculative Decoding Guide", "2. Single-Pass Tree
// Attention Verification" (step 3: longest path whose every token equals the target's greedy
// choice); "Speculative Decoding & Medusa Tree Attention", section 2, "The Acceptance
// Sampling Rule" (accept with probability min(1, P_t/P_d), else sample from
// normalize(max(0, P_t - P_d))); "Multi-Token Prediction: Draft-Model-Free Speculative
// Decoding", the verification engine (a node counts only when its whole root path passes;
// among equally long accepted paths the first is kept) and the text box of its Figure 1 (the
// target adds one token after the committed path).
//
// Greedy: the target rows are scanned once by many workgroups (row segments -> partial
// argmax), then one workgroup per sequence merges them and walks the tree.
// Speculative: one workgroup per sequence gathers the 2N probabilities it needs, decides,
// walks and picks the terminal row; the terminal row is then summed in segments by many
// workgroups (fp64) and a last pass per sequence locates the inverse-CDF position.
// Multi-candidate (siblings tested in turn against the running residual): one workgroup per
// sequence walks the tree; each rejection that is followed by another sibling costs one fp64
// reduction over the vocabulary, and the extra token reuses the segment-sum and sample passes.
//
// Decision exactness: u < P_t/P_d is evaluated as u*P_d < P_t in fp64; the product of two
// fp32 numbers is exact in fp64, so the decision is the exact real-number comparison.

#include <math.h>

#include <algorithm>

#include "mv_device.h"
#include "mv_host.h"

namespace mv {
namespace {

__device__ __forceinline__ int ceil_div_dev(int a, int b) { return (a + b - 1) / b; }

struct AcceptParams {
  int B, N, V, D, R, S, segLen;
  int vec4;  // speculative rows may be read as float4 (V, segLen multiples of 4; 16-byte bases)
  const int32_t* pred_ids;  // greedy with precomputed target argmax ids [B][N+1], or null
  const int32_t* parents;
  int pstride;  // entries between two sequences' parent arrays (0: one tree for the batch)
  const int32_t* tokens;
  const void* target;
  const float* draft;
  const float* uniforms;
  int32_t* accept_len;
  int32_t* path_nodes;
  int32_t* out_tokens;
  uint8_t* node_accept;
  float* alpha;
  int32_t* status;
  float* amax_v;  // greedy partials [B*R][S]
  int* amax_i;
  int* term;      // speculative: [B][4] = {terminal row, -, accepted length, -}
  double* term_c; // speculative: [B] residual coefficient c of the terminal row: the extra
                  // token is drawn from max(0, P_t - c P_d) (c = 0: from P_t itself)
  double* seg_r;  // speculative: [B][S] segment sums of the residual / of P_t
  double* seg_t;
  int* seg_lr;    // last index with a positive entry in the segment (-1 if none)
  int* seg_lt;
  // speculative rule fed by the target LM head: per-node P_t(x_i), P_d(x_i) at the parent's row
  // (fp64, [B][N]); the terminal rows are then one row per sequence ([B][V], compact = 1)
  const double* node_pt;
  const double* node_pd;
  int compact;
};

// First element of the terminal row of sequence b in target (or draft).
__device__ __forceinline__ size_t term_row_offset(const AcceptParams& p, int b, int row) {
  return p.compact ? static_cast<size_t>(b) * p.V : (static_cast<size_t>(b) * p.R + row) * p.V;
}

// ---- greedy: partial argmax of one row segment.
template <bool BF16>
__global__ __launch_bounds__(256) void row_argmax_kernel(const AcceptParams p) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int s = blockIdx.x % p.S;
  const size_t row = blockIdx.x / p.S;
  const int j0 = s * p.segLen, j1 = min(p.V, j0 + p.segLen);
  const size_t off = row * p.V;
  float bv = -INFINITY;
  int bi = INT_MAX;
  if constexpr (BF16) {
    const uint16_t* x = static_cast<const uint16_t*>(p.target) + off;
    if ((p.V & 7) == 0) {
      for (int j = j0 + threadIdx.x * 8; j < j1; j += 256 * 8) {
        const uint4 w = load_nt_u4(x + j);
        const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = __uint_as_float((e & 1) ? (wd[e >> 1] & 0xffff0000u) : (wd[e >> 1] << 16));
          if (v > bv) { bv = v; bi = j + e; }
        }
      }
    } else {
      for (int j = j0 + threadIdx.x; j < j1; j += 256) {
        const float v = bf16_to_f32(x[j]);
        if (v > bv) { bv = v; bi = j; }
      }
    }
  } else {
    const float* x = static_cast<const float*>(p.target) + off;
    if ((p.V & 3) == 0) {
      for (int j = j0 + threadIdx.x * 4; j < j1; j += 256 * 4) {
        const float4 w = load_nt_f4(x + j);
        if (w.x > bv) { bv = w.x; bi = j; }
        if (w.y > bv) { bv = w.y; bi = j + 1; }
        if (w.z > bv) { bv = w.z; bi = j + 2; }
        if (w.w > bv) { bv = w.w; bi = j + 3; }
      }
    } else {
      for (int j = j0 + threadIdx.x; j < j1; j += 256) {
        const float v = x[j];
        if (v > bv) { bv = v; bi = j; }
      }
    }
  }
  block_argbest(bv, bi, sv, si);
  if (threadIdx.x == 0) {
    p.amax_v[row * p.S + s] = bv;
    p.amax_i[row * p.S + s] = bi;
  }
}

// ---- per-sequence decisions, accepted set, terminal node, committed path.
template <bool SPEC>
__global__ __launch_bounds__(256) void accept_path_kernel(const AcceptParams p) {
  __shared__ int par[MV_MAX_NODES];
  __shared__ int pred[MV_MAX_NODES + 1];
  __shared__ int pass[MV_MAX_NODES];
  __shared__ int tks[MV_MAX_NODES];  // node tokens, read with the parents (the test and the
                                     // path output then read LDS)
  __shared__ float sv[4];
  __shared__ int si[4];
  const int b = blockIdx.x, tid = threadIdx.x, N = p.N, R = p.R;
  if (tid < N) {
    par[tid] = p.parents[static_cast<size_t>(b) * p.pstride + tid];
    tks[tid] = p.tokens[static_cast<size_t>(b) * N + tid];
  }
  if constexpr (!SPEC) {
    for (int r = tid; r < R && p.pred_ids; r += 256) pred[r] = p.pred_ids[static_cast<size_t>(b) * R + r];
    for (int r = tid; r < R && !p.pred_ids; r += 256) {
      float bv = -INFINITY;
      int bi = INT_MAX;
      const size_t q = (static_cast<size_t>(b) * R + r) * p.S;
      for (int s = 0; s < p.S; ++s) {
        const float v = p.amax_v[q + s];
        const int i = p.amax_i[q + s];
        if (kv_better(v, i, bv, bi)) { bv = v; bi = i; }
      }
      pred[r] = bi;
    }
  }
  __syncthreads();
  int flags = 0;
  if (tid < N) {
    const int pn = par[tid];
    int ok = 0;
    if (pn < -1 || pn >= tid) {
      flags |= MV_DEV_BAD_PARENT;
    } else {
      const int tok = tks[tid];
      if (tok < 0 || tok >= p.V) {
        flags |= MV_DEV_BAD_TOKEN;
        if (SPEC && p.alpha) p.alpha[static_cast<size_t>(b) * N + tid] = 0.f;
      } else if constexpr (SPEC) {
        const size_t o = (static_cast<size_t>(b) * R + (pn + 1)) * p.V + tok;
        const size_t on = static_cast<size_t>(b) * N + tid;
        const double pt = p.node_pt ? p.node_pt[on] : static_cast<double>(static_cast<const float*>(p.target)[o]);
        const double pd = p.node_pd ? p.node_pd[on] : static_cast<double>(p.draft[o]);
        const double u = p.uniforms[static_cast<size_t>(b) * R + tid];
        const double a = pd == 0.0 ? 1.0 : fmin(1.0, pt / pd);
        ok = pd == 0.0 ? (u < 1.0) : (u < 1.0 && u * pd < pt);
        if (p.alpha) p.alpha[static_cast<size_t>(b) * N + tid] = static_cast<float>(a);
      } else {
        ok = tok == pred[pn + 1];
      }
    }
    pass[tid] = ok;
  }
  __syncthreads();
  int accepted = 0, dep = 0;
  if (tid < N) {
    int c = tid, ok = 1;
    while (c != -1) {
      ok &= pass[c];
      ++dep;
      const int nx = par[c];
      if (nx < -1 || nx >= c) { ok = 0; break; }
      c = nx;
    }
    accepted = ok;
    if (p.node_accept) p.node_accept[static_cast<size_t>(b) * N + tid] = static_cast<uint8_t>(ok);
  }
  float bv = accepted ? static_cast<float>(dep) : -INFINITY;
  int bi = accepted ? tid : INT_MAX;
  block_argbest(bv, bi, sv, si);
  const int term = bi == INT_MAX ? -1 : bi;
  const int has_child = __syncthreads_or(tid < N && par[tid] == term);
  if (tid == 0) {
    int len = 0;
    for (int c = term; c != -1 && len <= N; c = par[c]) ++len;
    if (len > p.D) flags |= MV_DEV_TOO_DEEP;
    const int D = p.D;
    int32_t* pn_out = p.path_nodes + static_cast<size_t>(b) * D;
    int32_t* tk_out = p.out_tokens + static_cast<size_t>(b) * (D + 1);
    for (int k = 0; k < D; ++k) pn_out[k] = -1;
    for (int k = 0; k <= D; ++k) tk_out[k] = -1;
    int k = len - 1;
    for (int c = term; c != -1 && k >= 0; c = par[c], --k) {
      if (k < D) {
        pn_out[k] = c;
        tk_out[k] = tks[c];
      }
    }
    const int lc = min(len, D);
    p.accept_len[b] = lc;
    if constexpr (SPEC) {
      p.term[b * 4 + 0] = term + 1;
      p.term[b * 4 + 2] = lc;
      p.term_c[b] = has_child ? 1.0 : 0.0;  // all children of the terminal were rejected
    } else {
      tk_out[lc] = pred[term + 1];
    }
  }
  if (flags && p.status) atomicOr(p.status, flags);
}

// One element of the terminal row: the target probability and the residual max(0, P_t - P_d),
// folded into fp64 segment sums and last-positive indices.
struct SegAcc {
  double sr = 0.0, st = 0.0;
  int lr = -1, lt = -1;
  __device__ __forceinline__ void add(float x, float y, int j, bool resid, double c) {
    const double t = x;
    st += t;
    if (t > 0.0) lt = j;
    if (resid) {
      const double r = fmax(0.0, t - c * static_cast<double>(y));
      sr += r;
      if (r > 0.0) lr = j;
    }
  }
};

// ---- speculative: fp64 segment sums of the terminal row (residual and target).  Each thread
// walks its elements in increasing index order, so its last positive index is the largest.
__global__ __launch_bounds__(256) void residual_segsum_kernel(const AcceptParams p) {
  __shared__ double sd[4];
  __shared__ int smx[4];
  const int s = blockIdx.x % p.S, b = blockIdx.x / p.S;
  const int row = p.term[b * 4 + 0];
  const double cres = p.term_c[b];
  const bool resid = cres > 0.0;
  const size_t off = term_row_offset(p, b, row);
  const float* pt = static_cast<const float*>(p.target) + off;
  const float* pd = p.draft + off;
  const int j0 = s * p.segLen, j1 = min(p.V, j0 + p.segLen);
  SegAcc a;
  if (p.vec4) {
    // 16-byte pieces, two per thread in flight (j0 and j1 are multiples of 4)
    constexpr int U = 2;
    for (int j = j0 + 4 * static_cast<int>(threadIdx.x); j < j1; j += 4 * 256 * U) {
      float4 t4[U], d4[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int jj = j + 4 * 256 * u;
        t4[u] = jj < j1 ? *reinterpret_cast<const float4*>(pt + jj) : make_float4(0.f, 0.f, 0.f, 0.f);
        d4[u] = (resid && jj < j1) ? *reinterpret_cast<const float4*>(pd + jj) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int jj = j + 4 * 256 * u;
        if (jj < j1) {
          a.add(t4[u].x, d4[u].x, jj + 0, resid, cres);
          a.add(t4[u].y, d4[u].y, jj + 1, resid, cres);
          a.add(t4[u].z, d4[u].z, jj + 2, resid, cres);
          a.add(t4[u].w, d4[u].w, jj + 3, resid, cres);
        }
      }
    }
  } else {
    for (int j = j0 + static_cast<int>(threadIdx.x); j < j1; j += 256)
      a.add(pt[j], resid ? pd[j] : 0.f, j, resid, cres);
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  double vals[2] = {a.sr, a.st};
  int idx[2] = {a.lr, a.lt};
  double outv[2];
  int outi[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const double v = wave_sum_f64(vals[q]);
    const int mi = wave_max_i(idx[q]);
    __syncthreads();
    if (lane == 0) { sd[w] = v; smx[w] = mi; }
    __syncthreads();
    outv[q] = sd[0] + sd[1] + sd[2] + sd[3];
    outi[q] = max(max(smx[0], smx[1]), max(smx[2], smx[3]));
  }
  if (threadIdx.x == 0) {
    const size_t q = static_cast<size_t>(b) * p.S + s;
    p.seg_r[q] = outv[0];
    p.seg_t[q] = outv[1];
    p.seg_lr[q] = outi[0];
    p.seg_lt[q] = outi[1];
  }
}

// ---- speculative: inverse-CDF position of u * Z in the chosen distribution.  The segment
// records are staged in LDS by as many threads, thread 0 picks the segment; the 256 threads
// split that segment into contiguous ranges of up to kSampleChunk elements each fetched in one
// batch, an LDS scan gives each range its starting cumulative mass, and the one thread t with
// incl(t-1) <= u*Z < incl(t) walks its range element by element in registers.
constexpr int kSampleChunk = 32;

__global__ __launch_bounds__(256) void residual_sample_kernel(const AcceptParams p) {
  __shared__ double sc[256];
  __shared__ double segm[2][256];
  __shared__ int segl[2][256];
  __shared__ double tval;
  __shared__ int sh[3];
  __shared__ int found;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int row = p.term[b * 4 + 0], len = p.term[b * 4 + 2];
  const double cres = p.term_c[b];
  const int resid = cres > 0.0;
  const size_t off = term_row_offset(p, b, row);
  const float* pt = static_cast<const float*>(p.target) + off;
  const float* pd = p.draft + off;
  const size_t sq = static_cast<size_t>(b) * p.S;
  if (tid < p.S) {  // S <= 256
    segm[0][tid] = p.seg_r[sq + tid];
    segm[1][tid] = p.seg_t[sq + tid];
    segl[0][tid] = p.seg_lr[sq + tid];
    segl[1][tid] = p.seg_lt[sq + tid];
  }
  __syncthreads();
  if (tid == 0) {
    double zr = 0.0;
    for (int s = 0; s < p.S; ++s) zr += segm[0][s];
    const int use_r = resid && zr > 0.0;
    const int q = use_r ? 0 : 1;
    double tot = 0.0;
    for (int s = 0; s < p.S; ++s) tot += segm[q][s];
    const double t = static_cast<double>(p.uniforms[static_cast<size_t>(b) * p.R + p.N]) * tot;
    int sstar = -1, last = -1;
    double acc = 0.0, base = 0.0;
    for (int s = 0; s < p.S; ++s) {
      const double nx = acc + segm[q][s];
      if (sstar < 0 && nx > t) {
        sstar = s;
        base = acc;
      }
      acc = nx;
      last = max(last, segl[q][s]);
    }
    sh[0] = use_r;
    sh[1] = sstar;
    sh[2] = last;
    tval = t - base;  // mass still to cover inside the chosen segment
    found = -1;
  }
  __syncthreads();
  const bool use_r = sh[0] != 0;
  const int sstar = sh[1];
  int token = sh[2];
  if (sstar >= 0) {
    const double t = tval;
    const int j0 = sstar * p.segLen, j1 = min(p.V, j0 + p.segLen);
    const int per = (ceil_div_dev(j1 - j0, 256) + 3) / 4 * 4;  // a multiple of 4: aligned pieces
    const int a0 = min(j1, j0 + tid * per), a1 = min(j1, a0 + per);
    auto rv = [&](float x, float y) -> double {
      return use_r ? fmax(0.0, static_cast<double>(x) - cres * static_cast<double>(y))
                   : static_cast<double>(x);
    };
    float xv[kSampleChunk], yv[kSampleChunk];
    auto fetch = [&](int j) {  // elements j .. j+kSampleChunk-1 of this range (zeros past a1)
      if (p.vec4 && j + kSampleChunk <= a1) {
#pragma unroll
        for (int u = 0; u < kSampleChunk; u += 4) {
          const float4 x4 = *reinterpret_cast<const float4*>(pt + j + u);
          const float4 y4 = use_r ? *reinterpret_cast<const float4*>(pd + j + u) : make_float4(0.f, 0.f, 0.f, 0.f);
          xv[u] = x4.x; xv[u + 1] = x4.y; xv[u + 2] = x4.z; xv[u + 3] = x4.w;
          yv[u] = y4.x; yv[u + 1] = y4.y; yv[u + 2] = y4.z; yv[u + 3] = y4.w;
        }
      } else {
#pragma unroll
        for (int u = 0; u < kSampleChunk; ++u) {
          xv[u] = j + u < a1 ? pt[j + u] : 0.f;
          yv[u] = (use_r && j + u < a1) ? pd[j + u] : 0.f;
        }
      }
    };
    double mine = 0.0;
    for (int j = a0; j < a1; j += kSampleChunk) {
      fetch(j);
#pragma unroll
      for (int u = 0; u < kSampleChunk; ++u) mine += rv(xv[u], yv[u]);
    }
    // inclusive scan of the 256 range masses (Hillis-Steele in LDS)
    sc[tid] = mine;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      const double v = tid >= o ? sc[tid - o] : 0.0;
      __syncthreads();
      sc[tid] += v;
      __syncthreads();
    }
    const double incl = sc[tid];
    const double excl = tid > 0 ? sc[tid - 1] : 0.0;
    if (a0 < a1 && excl <= t && t < incl) {
      double acc = excl;
      int hit = -1;
      for (int j = a0; j < a1 && hit < 0; j += kSampleChunk) {
        if (a1 - a0 > kSampleChunk) fetch(j);  // a single-chunk range is still in registers
#pragma unroll
        for (int u = 0; u < kSampleChunk; ++u) {
          if (hit < 0 && j + u < a1) {
            acc += rv(xv[u], yv[u]);
            if (acc > t) hit = j + u;
          }
        }
      }
      found = hit;
    }
    __syncthreads();
    if (found >= 0) token = found;
    else token = use_r ? segl[0][sstar] : segl[1][sstar];
  }
  if (tid == 0) p.out_tokens[static_cast<size_t>(b) * (p.D + 1) + len] = token;
}

// ---- multi-candidate: the sibling-recursive rule.  At a node with target row P_t and draft
// row Q, the r-th rejection among its children turns the running distribution into
// normalize(max(0, P_r-1 - Q)).  Unrolled, P_r = max(0, P_t - c_r Q) / Z(c_r) with
// Z(c) = sum_v max(0, P_t(v) - c Q(v)), c_1 = 1 and c_r+1 = c_r + Z(c_r), so the walk only
// carries (c, Z(c)) and needs one reduction over the vocabulary per rejection that is
// followed by another sibling.  A zero residual falls back to P_t (c = 0, Z = 1).
constexpr int kWalkThreads = 1024;
#ifndef MV_WALK_U
#define MV_WALK_U 2
#endif
constexpr int kWalkMaxVec4V = 1 << 28;  // the row's byte offsets stay far inside 31 bits

// Z(c) over one row pair, fp64, by the whole workgroup; the same reduction order every time.
// The float4 path reads both rows through buffer resources: a piece past the row reads as
// zeros, whose term max(0, 0 - c * 0) is zero, so no load sits under a branch and the next
// sweep's loads are in flight while this sweep's terms are summed.
__device__ double residual_mass(const AcceptParams& p, const float* pt, const float* pd, double c,
                                double* red) {
  const int tid = threadIdx.x;
  double acc = 0.0;
  if (p.vec4 && p.V <= kWalkMaxVec4V) {
    constexpr int U = MV_WALK_U;                    // 16-byte pieces per row and sweep
    constexpr int kSweep = 16 * kWalkThreads;       // bytes of a row one sweep covers
    const int bytes = 4 * p.V;
    const __amdgpu_buffer_rsrc_t rt =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(pt), 0, bytes, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t rd =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(pd), 0, bytes, kBufferRsrcWord3);
    auto ld = [](__amdgpu_buffer_rsrc_t rs, int off) {
      return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    };
    float4 t4[U], d4[U];
    int off = 16 * tid;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      t4[u] = ld(rt, off + u * kSweep);
      d4[u] = ld(rd, off + u * kSweep);
    }
    for (int base = 0; base < bytes; base += U * kSweep) {
      off += U * kSweep;
      float4 tn[U], dn[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        tn[u] = ld(rt, off + u * kSweep);
        dn[u] = ld(rd, off + u * kSweep);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        acc += fmax(0.0, static_cast<double>(t4[u].x) - c * static_cast<double>(d4[u].x));
        acc += fmax(0.0, static_cast<double>(t4[u].y) - c * static_cast<double>(d4[u].y));
        acc += fmax(0.0, static_cast<double>(t4[u].z) - c * static_cast<double>(d4[u].z));
        acc += fmax(0.0, static_cast<double>(t4[u].w) - c * static_cast<double>(d4[u].w));
        t4[u] = tn[u];
        d4[u] = dn[u];
      }
    }
  } else {
    for (int j = tid; j < p.V; j += kWalkThreads)
      acc += fmax(0.0, static_cast<double>(pt[j]) - c * static_cast<double>(pd[j]));
  }
  const double w = wave_sum_f64(acc);
  if ((tid & 63) == 0) red[tid >> 6] = w;
  __syncthreads();
  double z = 0.0;
#pragma unroll
  for (int i = 0; i < kWalkThreads / 64; ++i) z += red[i];
  __syncthreads();  // red is free again
  return z;
}

__global__ __launch_bounds__(kWalkThreads) void multicand_walk_kernel(const AcceptParams p) {
  __shared__ int par[MV_MAX_NODES];
  __shared__ int first[MV_MAX_NODES + 1];  // first child of node r - 1 (r = 0: the prefix)
  __shared__ int nsib[MV_MAX_NODES];       // next sibling in index order
  __shared__ int path[MV_MAX_NODES];
  __shared__ float alph[MV_MAX_NODES];
  __shared__ float gpt[MV_MAX_NODES], gpd[MV_MAX_NODES], gu[MV_MAX_NODES];  // per-node gathers
  __shared__ int gtok[MV_MAX_NODES];  // node token, -1 if outside [0, V)
  __shared__ uint8_t onpath[MV_MAX_NODES];
  __shared__ double red[kWalkThreads / 64];
  __shared__ int st_child, st_node, st_len, st_reduce;
  __shared__ double st_c, st_z, st_cn;
  const int b = blockIdx.x, tid = threadIdx.x, N = p.N;
  const size_t rb = static_cast<size_t>(b) * p.R;
  const float* PT = static_cast<const float*>(p.target);
  int flags = 0;
  if (tid <= N) first[tid] = N;
  if (tid < N) {
    par[tid] = p.parents[static_cast<size_t>(b) * p.pstride + tid];
    alph[tid] = -1.f;
    onpath[tid] = 0;
  }
  __syncthreads();
  bool valid = false;
  if (tid < N) {  // a node with a malformed parent entry takes no part in the walk
    const int pn = par[tid];
    valid = pn >= -1 && pn < tid;
    if (valid) atomicMin(&first[pn + 1], tid);
    else flags |= MV_DEV_BAD_PARENT;
    // whatever the running residual, node i's test reads P_t and P_d at its parent's row and
    // its own token, and its uniform: gather them all now, in parallel
    const int x = p.tokens[static_cast<size_t>(b) * N + tid];
    const bool ok = valid && x >= 0 && x < p.V;
    if (valid && !ok) flags |= MV_DEV_BAD_TOKEN;
    gtok[tid] = ok ? x : -1;
    if (ok) {
      const size_t o = (rb + pn + 1) * p.V + x;
      gpt[tid] = PT[o];
      gpd[tid] = p.draft[o];
      gu[tid] = p.uniforms[rb + tid];
    }
  }
  __syncthreads();
  if (tid < N) {
    int nx = -1;
    if (valid) {
      const int pn = par[tid];
      for (int j = tid + 1; j < N; ++j) {
        if (par[j] == pn) {
          nx = j;
          break;
        }
      }
    }
    nsib[tid] = nx;
  }
  if (tid <= N && first[tid] >= N) first[tid] = -1;
  __syncthreads();
  if (tid == 0) {
    st_child = first[0];
    st_node = -1;
    st_len = 0;
    st_c = 0.0;
    st_z = 1.0;
  }
  __syncthreads();
  for (;;) {
    const int child = st_child;
    __syncthreads();  // every thread has the state before thread 0 changes it
    if (child < 0) break;
    if (tid == 0) {
      const double c = st_c, z = st_z;
      int reduce = 0;
      if (gtok[child] < 0) {  // not a candidate: rejected, the distribution is unchanged
        alph[child] = 0.f;
        st_child = nsib[child];
      } else {
        const double p0 = gpt[child], q = gpd[child], u = gu[child];
        const double numer = c == 0.0 ? p0 : fmax(0.0, p0 - c * q);  // Z(c) P_r(x)
        const double den = q * z;                                     // Z(c) Q(x)
        int acc;
        double a;
        if (q == 0.0) {
          a = 1.0;
          acc = u < 1.0;
        } else {
          a = fmin(1.0, numer / den);
          acc = u < 1.0 && u * den < numer;
        }
        alph[child] = static_cast<float>(a);
        if (acc) {
          path[st_len] = child;
          onpath[child] = 1;
          st_len = st_len + 1;
          st_node = child;
          st_c = 0.0;
          st_z = 1.0;
          st_child = first[child + 1];
        } else {
          const double cn = c == 0.0 ? 1.0 : c + z;
          const int sib = nsib[child];
          if (sib >= 0) {
            st_cn = cn;
            reduce = 1;
          } else {
            st_c = cn;  // the extra token's pass normalises this last residual
          }
          st_child = sib;
        }
      }
      st_reduce = reduce;
    }
    __syncthreads();
    if (st_reduce) {
      const size_t off = (rb + st_node + 1) * p.V;
      const double zz = residual_mass(p, PT + off, p.draft + off, st_cn, red);
      if (tid == 0) {
        if (zz > 0.0) {
          st_c = st_cn;
          st_z = zz;
        } else {
          st_c = 0.0;
          st_z = 1.0;
        }
      }
    }
    __syncthreads();
  }
  if (tid == 0) {
    const int len = st_len, D = p.D;
    if (len > D) flags |= MV_DEV_TOO_DEEP;
    const int lc = min(len, D);
    int32_t* pn_out = p.path_nodes + static_cast<size_t>(b) * D;
    int32_t* tk_out = p.out_tokens + static_cast<size_t>(b) * (D + 1);
    for (int k = 0; k < D; ++k) pn_out[k] = k < lc ? path[k] : -1;
    for (int k = 0; k <= D; ++k)  // an accepted node's token is in range, so gtok holds it
      tk_out[k] = k < lc ? gtok[path[k]] : -1;
    p.accept_len[b] = lc;
    p.term[b * 4 + 0] = st_node + 1;
    p.term[b * 4 + 2] = lc;
    p.term_c[b] = st_c;
  }
  __syncthreads();
  if (tid < N) {
    if (p.node_accept) p.node_accept[static_cast<size_t>(b) * N + tid] = onpath[tid];
    if (p.alpha) p.alpha[static_cast<size_t>(b) * N + tid] = alph[tid];
  }
  if (flags && p.status) atomicOr(p.status, flags);
}

// ---- speculative rule fed by the target LM head and the Medusa heads' logits ------------------
// The target distribution at row r is softmax(W_lm x_t[r]) and the draft distribution of the
// nodes at depth k is softmax of head k's logits (one row per depth and sequence: the heads
// all read the same hidden state).  Nothing of size [B][N+1][V] exists: a node's P_t(x_i) is one
// dot product W_lm[x_i] . x_t[parent row] against the row's LSE, its P_d(x_i) one entry of the
// draft logits against their LSE, and the terminal's two rows are produced after the walk
// (one GEMV over W_lm for the target row).
struct SpecLmParams {
  int B, N, V, d, D, pstride, draft_bf16;
  const int32_t* parents;
  const int32_t* tokens;
  const uint16_t* x;      // [B][N+1][d] bf16 hidden states of the verify rows
  const uint16_t* w;      // [V][d] bf16 LM head
  const float* lse_t;     // [B][N+1] log-sum-exp of the target logits
  const void* dlog;       // [B][D][V] draft logits (fp32 or bf16)
  const float* dlse;      // [B][D]
  double* node_pt;        // [B][N]
  double* node_pd;
  const int* term;        // [B][4] from the walk: {terminal row, -, accepted length, -}
  const double* term_c;
  float* row_t;           // [B][V] target row of the terminal
  float* row_d;           // [B][V] draft row of the terminal's children (when it has any)
};

__device__ __forceinline__ float dot8_bf16(const uint4 a, const uint4 b, float acc) {
  const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = fmaf(__uint_as_float(av[i] << 16), __uint_as_float(bv[i] << 16), acc);
    acc = fmaf(__uint_as_float(av[i] & 0xffff0000u), __uint_as_float(bv[i] & 0xffff0000u), acc);
  }
  return acc;
}

__device__ __forceinline__ double draft_logit(const SpecLmParams& q, int b, int k, int v) {
  const size_t o = (static_cast<size_t>(b) * q.D + k) * q.V + v;
  return q.draft_bf16 ? static_cast<double>(bf16_to_f32(static_cast<const uint16_t*>(q.dlog)[o]))
                      : static_cast<double>(static_cast<const float*>(q.dlog)[o]);
}

// One wave per node (b, i): P_t(x_i) = exp(W_lm[x_i] . x_t[b][p_i + 1] - LSE_t) and
// P_d(x_i) = exp(draft logit of depth(i) at x_i - its LSE), both in fp64 from the fp32 dot.
// Malformed parents or tokens leave 0 / 0 (the walk flags them).
__global__ __launch_bounds__(256) void spec_lm_nodes_kernel(const SpecLmParams q) {
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wid >= q.B * q.N) return;
  const int b = wid / q.N, i = wid % q.N;
  const int32_t* par = q.parents + static_cast<size_t>(b) * q.pstride;
  const int tok = q.tokens[static_cast<size_t>(b) * q.N + i];
  int dep = 0, c = i;
  bool ok = tok >= 0 && tok < q.V;
  while (c != -1 && ok) {  // strictly decreasing indices: at most N steps
    ++dep;
    const int nx = par[c];
    if (nx < -1 || nx >= c) ok = false;
    c = nx;
  }
  ok = ok && dep <= q.D;
  double pt = 0.0, pd = 0.0;
  if (ok) {
    const int row = par[i] + 1;
    const uint16_t* wr = q.w + static_cast<size_t>(tok) * q.d;
    const uint16_t* xr = q.x + (static_cast<size_t>(b) * (q.N + 1) + row) * q.d;
    float acc = 0.f;
    for (int j = 8 * lane; j < q.d; j += 512)
      acc = dot8_bf16(*reinterpret_cast<const uint4*>(wr + j), *reinterpret_cast<const uint4*>(xr + j), acc);
    const float dotv = wave_sum(acc);
    pt = exp(static_cast<double>(dotv) - static_cast<double>(q.lse_t[static_cast<size_t>(b) * (q.N + 1) + row]));
    pd = exp(draft_logit(q, b, dep - 1, tok) - static_cast<double>(q.dlse[static_cast<size_t>(b) * q.D + dep - 1]));
  }
  if (lane == 0) {
    q.node_pt[wid] = pt;
    q.node_pd[wid] = pd;
  }
}

// Terminal rows after the walk.  The target row row_t[b][v] = exp(W_lm[v] . x_t[b][row_b] -
// LSE_t) comes from the LM head's streaming kernel in its rows mode (one pass over W_lm for up
// to 128 sequences, on the matrix cores).  The draft row, when the terminal has children (they
// were all rejected): row_d[b][v] = exp(draft logit of depth len_b + 1 at v - its LSE), else 0.
__global__ __launch_bounds__(256) void spec_lm_draft_rows_kernel(const SpecLmParams q) {
  const int b = blockIdx.y;
  const int v = blockIdx.x * 256 + threadIdx.x;
  if (v >= q.V) return;
  const bool child = q.term_c[b] > 0.0;
  const int k = q.term[b * 4 + 2];  // depth of the terminal = draft row of its children
  q.row_d[static_cast<size_t>(b) * q.V + v] =
      (child && k < q.D)
          ? expf(static_cast<float>(draft_logit(q, b, k, v)) - q.dlse[static_cast<size_t>(b) * q.D + k])
          : 0.f;
}

struct AcceptPlan {
  int S = 1, segLen = 1;
  size_t ws_bytes = 0;
};

AcceptPlan plan_accept(int mode, int B, int N, int V, void* ws, AcceptParams* p) {
  AcceptPlan a;
  const long long R = N + 1;
  int S;
  if (mode == MV_ACCEPT_GREEDY) {
    S = static_cast<int>(std::max<long long>(1, (1024 + B * R - 1) / (B * R)));
    S = std::min(S, std::max(1, V / 2048));
    a.segLen = (ceil_div(V, S) + 7) / 8 * 8;
  } else {
    S = std::max(1, ceil_div(1024, B));
    S = std::min(S, std::min(256, std::max(1, V / 1024)));
    a.segLen = (ceil_div(V, S) + 3) / 4 * 4;
  }
  a.S = ceil_div(V, a.segLen);
  Carver c(ws);
  if (mode == MV_ACCEPT_GREEDY) {
    float* av = c.take<float>(static_cast<size_t>(B) * R * a.S);
    int* ai = c.take<int>(static_cast<size_t>(B) * R * a.S);
    if (p) { p->amax_v = av; p->amax_i = ai; }
  } else {
    int* tm = c.take<int>(static_cast<size_t>(B) * 4);
    double* tc = c.take<double>(static_cast<size_t>(B));
    double* sr = c.take<double>(static_cast<size_t>(B) * a.S);
    double* st = c.take<double>(static_cast<size_t>(B) * a.S);
    int* lr = c.take<int>(static_cast<size_t>(B) * a.S);
    int* lt = c.take<int>(static_cast<size_t>(B) * a.S);
    if (p) {
      p->term = tm; p->term_c = tc;
      p->seg_r = sr; p->seg_t = st; p->seg_lr = lr; p->seg_lt = lt;
    }
  }
  a.ws_bytes = c.bytes();
  return a;
}

}  // namespace
}  // namespace mv

using namespace mv;

extern "C" {

MV_API size_t mv_accept_paths_workspace(int mode, int B, int N, int V) {
  if ((mode != MV_ACCEPT_GREEDY && mode != MV_ACCEPT_SPECULATIVE && mode != MV_ACCEPT_MULTICAND) ||
      B < 1 || N < 1 || V < 1)
    return 0;
  if (N > MV_MAX_NODES) return 0;
  return plan_accept(mode, B, N, V, nullptr, nullptr).ws_bytes;
}

MV_API int mv_accept_paths(int mode, int target_dt, int B, int N, int V, int D,
                           const int32_t* parents, int parents_stride,
                           const int32_t* node_tokens, const void* target,
                           const float* draft, const float* uniforms, int32_t* accept_len,
                           int32_t* path_nodes, int32_t* out_tokens, uint8_t* node_accept,
                           float* alpha, int32_t* dev_status, void* ws, size_t ws_bytes,
                           void* stream) {
  if (mode != MV_ACCEPT_GREEDY && mode != MV_ACCEPT_SPECULATIVE && mode != MV_ACCEPT_MULTICAND)
    return MV_ERR_INVALID_ARG;
  if (target_dt != MV_F32 && target_dt != MV_BF16 && target_dt != MV_TARGET_IDS) return MV_ERR_INVALID_ARG;
  if (target_dt == MV_TARGET_IDS && mode != MV_ACCEPT_GREEDY) return MV_ERR_INVALID_ARG;
  if (B < 1 || N < 1 || V < 1 || D < 1) return MV_ERR_INVALID_ARG;
  if (parents_stride != 0 && parents_stride < N) return MV_ERR_INVALID_ARG;
  if (N > MV_MAX_NODES || D > MV_MAX_DEPTH) return MV_ERR_UNSUPPORTED;
  if (!parents || !node_tokens || !target || !accept_len || !path_nodes || !out_tokens)
    return MV_ERR_INVALID_ARG;
  if (mode != MV_ACCEPT_GREEDY) {
    if (target_dt != MV_F32) return MV_ERR_UNSUPPORTED;
    if (!draft || !uniforms) return MV_ERR_INVALID_ARG;
  }
  const bool ids = target_dt == MV_TARGET_IDS;
  const AcceptPlan need = plan_accept(mode, B, N, V, nullptr, nullptr);
  if (!ids) MV_TRY(check_ws(ws, ws_bytes, need.ws_bytes));
  AcceptParams p{};
  p.B = B; p.N = N; p.V = V; p.D = D; p.R = N + 1;
  p.parents = parents; p.pstride = parents_stride; p.tokens = node_tokens; p.target = target; p.draft = draft;
  p.uniforms = uniforms; p.accept_len = accept_len; p.path_nodes = path_nodes;
  p.out_tokens = out_tokens; p.node_accept = node_accept; p.alpha = alpha; p.status = dev_status;
  const AcceptPlan a = plan_accept(mode, B, N, V, ids ? nullptr : ws, ids ? nullptr : &p);
  if (ids) p.pred_ids = static_cast<const int32_t*>(target);
  p.S = a.S;
  p.segLen = a.segLen;
  p.vec4 = (V % 4 == 0 && a.segLen % 4 == 0 &&
            ((reinterpret_cast<uintptr_t>(target) | reinterpret_cast<uintptr_t>(draft)) & 15) == 0) ? 1 : 0;
  hipStream_t st = as_stream(stream);
  if (ids) {
    accept_path_kernel<false><<<B, 256, 0, st>>>(p);
    return launch_status();
  }
  if (mode == MV_ACCEPT_GREEDY) {
    const long long blocks = static_cast<long long>(B) * p.R * a.S;
    if (blocks > (1LL << 31) - 1) return MV_ERR_UNSUPPORTED;
    if (target_dt == MV_BF16) row_argmax_kernel<true><<<static_cast<int>(blocks), 256, 0, st>>>(p);
    else row_argmax_kernel<false><<<static_cast<int>(blocks), 256, 0, st>>>(p);
    MV_TRY(launch_status());
    accept_path_kernel<false><<<B, 256, 0, st>>>(p);
    return launch_status();
  }
  if (mode == MV_ACCEPT_MULTICAND) multicand_walk_kernel<<<B, kWalkThreads, 0, st>>>(p);
  else accept_path_kernel<true><<<B, 256, 0, st>>>(p);
  MV_TRY(launch_status());
  residual_segsum_kernel<<<B * a.S, 256, 0, st>>>(p);
  MV_TRY(launch_status());
  residual_sample_kernel<<<B, 256, 0, st>>>(p);
  return launch_status();
}

MV_API size_t mv_accept_speculative_lm_workspace(int B, int N, int V) {
  if (B < 1 || N < 1 || V < 1 || N > MV_MAX_NODES) return 0;
  const AcceptPlan a = plan_accept(MV_ACCEPT_SPECULATIVE, B, N, V, nullptr, nullptr);
  Carver c(nullptr);
  c.take<char>(a.ws_bytes);
  c.take<double>(static_cast<size_t>(B) * N * 2);
  c.take<float>(static_cast<size_t>(B) * V * 2);
  return c.bytes();
}

MV_API int mv_accept_speculative_lm(int draft_dt, int B, int N, int V, int d, int D,
                                    const int32_t* parents, int parents_stride,
                                    const int32_t* node_tokens, const void* x_t,
                                    const void* w_lm, const float* lse_t,
                                    const void* draft_logits, const float* draft_lse,
                                    const float* uniforms, int32_t* accept_len,
                                    int32_t* path_nodes, int32_t* out_tokens,
                                    uint8_t* node_accept, float* alpha, int32_t* dev_status,
                                    void* ws, size_t ws_bytes, void* stream) {
  if (draft_dt != MV_F32 && draft_dt != MV_BF16) return MV_ERR_INVALID_ARG;
  if (B < 1 || N < 1 || V < 1 || D < 1 || d < 8) return MV_ERR_INVALID_ARG;
  if (parents_stride != 0 && parents_stride < N) return MV_ERR_INVALID_ARG;
  if (N > MV_MAX_NODES || D > MV_MAX_DEPTH) return MV_ERR_UNSUPPORTED;
  if (d % 32 != 0) return MV_ERR_UNSUPPORTED;
  if (!parents || !node_tokens || !x_t || !w_lm || !lse_t || !draft_logits || !draft_lse ||
      !uniforms || !accept_len || !path_nodes || !out_tokens)
    return MV_ERR_INVALID_ARG;
  MV_TRY(check_ws(ws, ws_bytes, mv_accept_speculative_lm_workspace(B, N, V)));
  AcceptParams p{};
  p.B = B; p.N = N; p.V = V; p.D = D; p.R = N + 1;
  p.parents = parents; p.pstride = parents_stride; p.tokens = node_tokens;
  p.uniforms = uniforms; p.accept_len = accept_len; p.path_nodes = path_nodes;
  p.out_tokens = out_tokens; p.node_accept = node_accept; p.alpha = alpha; p.status = dev_status;
  const AcceptPlan a = plan_accept(MV_ACCEPT_SPECULATIVE, B, N, V, ws, &p);
  Carver c(ws);
  c.take<char>(a.ws_bytes);
  double* npt = c.take<double>(static_cast<size_t>(B) * N);
  double* npd = c.take<double>(static_cast<size_t>(B) * N);
  float* rt = c.take<float>(static_cast<size_t>(B) * V);
  float* rd = c.take<float>(static_cast<size_t>(B) * V);
  p.node_pt = npt; p.node_pd = npd;
  p.compact = 1;
  p.target = rt; p.draft = rd;
  p.S = a.S;
  p.segLen = a.segLen;
  p.vec4 = (V % 4 == 0 && a.segLen % 4 == 0) ? 1 : 0;  // carved rows are 256-byte aligned
  SpecLmParams q{};
  q.B = B; q.N = N; q.V = V; q.d = d; q.D = D;
  q.pstride = parents_stride; q.draft_bf16 = draft_dt == MV_BF16;
  q.parents = parents; q.tokens = node_tokens;
  q.x = static_cast<const uint16_t*>(x_t); q.w = static_cast<const uint16_t*>(w_lm);
  q.lse_t = lse_t; q.dlog = draft_logits; q.dlse = draft_lse;
  q.node_pt = npt; q.node_pd = npd; q.term = p.term; q.term_c = p.term_c;
  q.row_t = rt; q.row_d = rd;
  hipStream_t st = as_stream(stream);
  spec_lm_nodes_kernel<<<ceil_div(static_cast<long long>(B) * N, 4), 256, 0, st>>>(q);
  MV_TRY(launch_status());
  accept_path_kernel<true><<<B, 256, 0, st>>>(p);
  MV_TRY(launch_status());
  MV_TRY(lm_head_prob_rows(B, d, V, q.x, p.term, 4, N + 1, lse_t, q.w, rt, st));
  spec_lm_draft_rows_kernel<<<dim3(ceil_div(V, 256), B), 256, 0, st>>>(q);
  MV_TRY(launch_status());
  residual_segsum_kernel<<<B * a.S, 256, 0, st>>>(p);
  MV_TRY(launch_status());
  residual_sample_kernel<<<B, 256, 0, st>>>(p);
  return launch_status();
}

}  // extern "C"
