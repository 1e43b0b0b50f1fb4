// Tree-masked GQA attention on gfx950.
//
// Sources: "Medusa Explained: Multi-Head Speculative Decoding Guide", "2. Single-Pass Tree
// Attention Verification" (the candidate tree is packed after the prefix and every node sees
// the whole prefix plus its ancestors; mask M_tree is 0 there and -inf elsewhere);
// "Multi-Token Prediction: Draft-Model-Free Speculative Decoding", "The 2D Tree Attention
// Mask" (ancestor-or-self, so every node also sees itself).
//
// bf16 path.  For one (sequence b, KV head g) the G query heads of the group and the N tree
// nodes form M = N*G query rows that share every key, so they are packed into the MFMA tile:
// a wave owns 32 query rows, a workgroup of 8 waves 256 rows (all of them for a 64-node tree
// with 4 query heads per KV head, so each K/V byte crosses HBM once).  The prefix is split
// into chunks handled by separate workgroups (split-KV); the chunk that ends the prefix also
// takes the N tree keys, where the per-node ancestor bitmask replaces the dense mask.  Per
// 64-key tile:
//   * K and V arrive with coalesced 16-byte loads one tile ahead (registers) and are stored
//     row-major in LDS, each with a padded pitch chosen so that its operand reads are
//     bank-conflict free;
//   * S^T = K Q^T: two 32x32 output tiles of v_mfma_f32_32x32x16_bf16 per wave; in that output
//     layout a lane holds 32 keys of one query, so the softmax max/sum need one cross-lane
//     step (lanes l and l+32);
//   * online softmax: running max in raw score units, p = 2^(s*c - m*c) with c = scale*log2(e)
//     as one FMA and a raw v_exp_f32 per score; the O rescale is skipped when no lane's max
//     moved;
//   * O^T += V^T P^T with P rounded to bf16 (v_cvt_pk_bf16_f32) and fp32 accumulation; the V^T
//     operand comes from the row-major V tile through transposed LDS reads
//     (ds_read_b64_tr_b16, two per operand).
// A second kernel merges the chunk partials with their (max, sum) pairs.
//
// Launch beside other kernels (mv_tree_attn_verify_beside), for a step that runs the attention
// on a second stream beside the bandwidth-bound Medusa heads: the same kernel launched
// persistent on half of the CUs, one workgroup per CU striding over the workgroup indices.  Such
// a workgroup holds nearly all of its CU's registers (two waves of ~250 per SIMD), so the
// heads' workgroups stream their weights on the other half of the chip instead of sharing SIMDs
// with the attention.
//
// fp32 path: a vector-ALU kernel, one wave per query row, no chunking (the fp32 configuration
// is a small check case).

#include <math.h>

#include <algorithm>

#include "mv_device.h"
#include "mv_host.h"

namespace mv {
namespace {

struct AttnParams {
  int B, N, Hq, Hkv, G, M, L_cap, max_L, CK, nchunks, qtiles, W, jobs;
  int vblocks;  // workgroup indices of the launch (a persistent grid strides over them)
  float scale_log2;
  const void* q;
  const void* k;
  const void* v;
  const int32_t* prefix_len;
  const uint32_t* anc;
  int mask_stride;  // words between two sequences' masks (0: one mask for the whole batch)
  void* out;
  float* lse;
  float* part_o;
  float2* part_ml;
  int32_t* status;
  const int32_t* order;  // sequences by decreasing prefix length (null: batch order)
  // Balanced split of a batch (null: every sequence in chunks of CK keys): plan[3b] = chunks
  // of sequence b, plan[3b + 1] = its chunk length, plan[3b + 2] = the chunk-job index of its
  // first chunk; jtab[j] = (b << 16) | chunk for the chunk-jobs j in launch order, kNoJob past
  // the last.  The partials of chunk-job j then sit at chunk slot j (nchunks = slots per
  // (sequence, KV head) otherwise, total slots here).
  const int32_t* plan;
  const uint32_t* jtab;
};

constexpr uint32_t kNoJob = 0xffffffffu;

constexpr int kXcds = 8;  // MI355X: workgroups are handed to the 8 XCDs round-robin

__device__ __forceinline__ int clamp_prefix(const AttnParams& p, int Lb, bool report) {
  const int hi = min(p.max_L, p.L_cap - p.N);
  if (Lb < 0 || Lb > hi) {
    if (report && p.status) atomicOr(p.status, MV_DEV_BAD_PREFIX);
    Lb = max(0, min(Lb, hi));
  }
  return Lb;
}

#ifndef MV_ATTN_TARGET_WG
#define MV_ATTN_TARGET_WG 2048  // split-KV: aim for this many workgroups (one sequence)
#endif
#ifndef MV_ATTN_TARGET_WG_BATCH
#define MV_ATTN_TARGET_WG_BATCH 768  // ... and with several sequences (at most)
#endif
#ifndef MV_ATTN_TARGET_WG_BESIDE
#define MV_ATTN_TARGET_WG_BESIDE 768  // ... for a batch in the launch beside other kernels (indices)
#endif
#ifndef MV_ATTN_BALANCED
#define MV_ATTN_BALANCED 1  // batches that split: chunk plan from the actual lengths
#endif
#ifndef MV_ATTN_MIN_CHUNK
#define MV_ATTN_MIN_CHUNK 256   // but never chunks shorter than this many keys
#endif

constexpr int kKT = 64;  // keys per tile
// Waves per attention workgroup, 32 query rows each (two per SIMD).
constexpr int kNWV = 8;
constexpr float kLazyLog2 = 8.f;  // running-max slack of the online softmax (log2 units)


typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

template <int DH, int NWV, bool PERSIST>
__global__ __launch_bounds__(NWV * 64) __attribute__((amdgpu_waves_per_eu(2, 8)))
void tree_attn_bf16_kernel(const AttnParams p) {
  constexpr int NT = NWV * 64;
  constexpr int KP = DH + 8;    // K tile pitch (elements): conflict-free 16-byte reads
  constexpr int VKP = DH + 32;  // V tile pitch: conflict-free transposed reads (see below)
  constexpr int KS = DH / 16;   // k-steps of one S^T MFMA chain
  constexpr int DB = DH / 32;   // 32-wide blocks of the head dimension
  constexpr int DG = DH / 8;    // 16-byte pieces per key row
  constexpr int PPT = kKT * DG / NT;
  static_assert((kKT * DG) % NT == 0, "tile pieces must split evenly");
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kKT * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][kKT * VKP];

  // Job j = (sequence rank, chunk, KV head), longest sequences first (workgroups are dispatched
  // in index order, so the long jobs do not end up in the tail); jobs are dealt round-robin
  // over the XCDs, and the query tiles of one job stay on one XCD, where they share its K/V.
  // vb is the workgroup index (blockIdx.x, or each index a persistent launch walks).
  auto run = [&](const int vb) {
    const int xcd = vb % kXcds, pos = vb / kXcds;
    const int qt = pos % p.qtiles;
    const int job = (pos / p.qtiles) * kXcds + xcd;
    if (job >= p.jobs) return;
    const int g = job % p.Hkv;
    int b, c, ncb, ck;
    if (p.jtab) {
      const uint32_t e = p.jtab[job / p.Hkv];
      if (e == kNoJob) return;
      b = static_cast<int>(e >> 16);
      c = static_cast<int>(e & 0xffffu);
      ncb = p.plan[3 * b];
      ck = p.plan[3 * b + 1];
    } else {
      c = (job / p.Hkv) % p.nchunks;
      const int rank = job / (p.Hkv * p.nchunks);
      b = p.order ? p.order[rank] : rank;
      ck = p.CK;
      ncb = -1;
    }

    const int Lb = clamp_prefix(p, p.prefix_len[b], threadIdx.x == 0 && qt == 0 && c == 0 && g == 0);
    if (ncb < 0) ncb = max(1, (Lb + p.CK - 1) / p.CK);
    if (c >= ncb) return;
    const int kbeg = c * ck, kend = min(Lb, kbeg + ck);
    const bool last = c == ncb - 1;
    const int ntp = kend > kbeg ? (kend - kbeg + kKT - 1) / kKT : 0;
    const int ntiles = ntp + (last ? (p.N + kKT - 1) / kKT : 0);

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int l32 = lane & 31, half = lane >> 5;
    const int m = qt * (NWV * 32) + wv * 32 + l32;
    const bool qvalid = m < p.M;
    const int node = qvalid ? m / p.G : 0;
    const int h = g * p.G + (qvalid ? m % p.G : 0);

    // Q is the B operand of S^T = K Q^T: lane holds query l32, dims ks*16 + 8*half .. +8.
    bf16x8 qreg[KS];
    {
      const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + (static_cast<size_t>(b * p.N + node) * p.Hq + h) * DH;
  #pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 t4 = qvalid ? *reinterpret_cast<const uint4*>(qrow + ks * 16 + half * 8) : make_uint4(0, 0, 0, 0);
        qreg[ks] = as_bf16x8(t4);
      }
    }
    const size_t kvbase = (static_cast<size_t>(b) * p.Hkv + g) * p.L_cap * DH;
    const uint16_t* Kg = static_cast<const uint16_t*>(p.k) + kvbase;
    const uint16_t* Vg = static_cast<const uint16_t*>(p.v) + kvbase;

    auto tile_rows = [&](int t, int& row0, int& nv) {
      if (t < ntp) {
        row0 = kbeg + t * kKT;
        nv = min(kKT, kend - row0);
      } else {
        const int tt = t - ntp;
        row0 = Lb + tt * kKT;
        nv = min(kKT, p.N - tt * kKT);
      }
    };
    // One register set of prefetched K/V pieces: tile t+1 is requested while tile t computes.
    // Buffer loads over this (sequence, KV head)'s slice of the cache: rows past a partial tile
    // and requests past the last tile get an offset beyond the slice, which the hardware's range
    // check turns into zeros, so no load sits under a branch.
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(Kg), 0, p.L_cap * DH * 2, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(Vg), 0, p.L_cap * DH * 2, kBufferRsrcWord3);
    uint4 kr[PPT], vr[PPT];
    auto gload = [&](int t, uint4 (&kr)[PPT], uint4 (&vr)[PPT]) {
      int row0 = 0, nv = 0;
      if (t < ntiles) tile_rows(t, row0, nv);
  #pragma unroll
      for (int i = 0; i < PPT; ++i) {
        const int pc = tid + i * NT, key = pc / DG, dg = pc % DG;
        const int off = key < nv ? ((row0 + key) * DH + dg * 8) * 2 : kBufferOutOfRange;
        kr[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0));
        vr[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0));
      }
    };
    auto swrite = [&](int buf, const uint4 (&kr)[PPT], const uint4 (&vr)[PPT]) {
  #pragma unroll
      for (int i = 0; i < PPT; ++i) {
        const int pc = tid + i * NT, key = pc / DG, dg = pc % DG;
        *reinterpret_cast<uint4*>(&Ks[buf][key * KP + dg * 8]) = kr[i];
        *reinterpret_cast<uint4*>(&Vs[buf][key * VKP + dg * 8]) = vr[i];
      }
    };

    f32x16 oacc[DB];
  #pragma unroll
    for (int db = 0; db < DB; ++db)
  #pragma unroll
      for (int v = 0; v < 16; ++v) oacc[db][v] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const float lazy = kLazyLog2 / p.scale_log2;  // in raw score units

    auto compute = [&](int t) {
      const int buf = t & 1;
      f32x16 sacc[2];
  #pragma unroll
      for (int st = 0; st < 2; ++st) {
  #pragma unroll
        for (int v = 0; v < 16; ++v) sacc[st][v] = 0.f;
  #pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint4 a = *reinterpret_cast<const uint4*>(&Ks[buf][(st * 32 + l32) * KP + ks * 16 + half * 8]);
          sacc[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), qreg[ks], sacc[st], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      int row0, nv;
      tile_rows(t, row0, nv);
      const bool tree = t >= ntp;
      // 32x32 output layout: lane holds query l32 and keys 32*st + 8*(v/4) + 4*half + v%4.
      f32x16 (&sv)[2] = sacc;  // scores, then probabilities, in place
      // Visibility of the 32 scores this lane holds, bit 16*st + v: all set for a full prefix
      // tile; the tail of a partial tile and non-ancestors of a tree tile are cleared.
      uint32_t vis = 0xffffffffu;
      if (tree || nv < kKT) {
        uint32_t aw[2] = {0xffffffffu, 0xffffffffu};
        if (tree) {
          const int w0 = 2 * (t - ntp);
          const uint32_t* arow = p.anc + static_cast<size_t>(b) * p.mask_stride +
                                 static_cast<size_t>(node) * p.W;
          aw[0] = qvalid ? arow[w0] : 0u;
          aw[1] = (qvalid && w0 + 1 < p.W) ? arow[w0 + 1] : 0u;
        }
        vis = 0u;
  #pragma unroll
        for (int st = 0; st < 2; ++st)
  #pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int kl = 8 * (v >> 2) + 4 * half + (v & 3);
            const bool ok = st * 32 + kl < nv && ((aw[st] >> kl) & 1u);
            vis |= static_cast<uint32_t>(ok) << (16 * st + v);
          }
      }
      // Online softmax; the running max is kept in raw score units and the scale is folded into
      // the exp2 argument: p = 2^(s*c - m*c), c = scale*log2(e), one FMA per score.
      float tmax = -INFINITY;
      if (vis == 0xffffffffu) {
  #pragma unroll
        for (int st = 0; st < 2; ++st)
  #pragma unroll
          for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, sv[st][v]);
      } else {
  #pragma unroll
        for (int st = 0; st < 2; ++st)
  #pragma unroll
          for (int v = 0; v < 16; ++v) {
            sv[st][v] = ((vis >> (16 * st + v)) & 1u) ? sv[st][v] : -INFINITY;
            tmax = fmaxf(tmax, sv[st][v]);
          }
      }
      {  // lanes l and l^32 hold the two key halves of one query
        const LanePair t2 = swap32(__float_as_uint(tmax));
        tmax = fmaxf(__uint_as_float(t2.a), __uint_as_float(t2.b));
      }
      const float c2 = p.scale_log2;
      // Lazy rescaling: the running max moves only when a score passes it by more than
      // kLazyLog2 in log2 units.  Until then the stale max keeps every p <= 2^kLazyLog2, well
      // inside fp32 and bf16 range, and the O rescale below is skipped; (m, l, O) stay an exact
      // log-sum-exp triple for whatever reference max they carry.
      const float m_new = tmax > m_run + lazy ? tmax : m_run;
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * c2);
      const float mc = m_use * c2;
      float lsum = 0.f;
  #pragma unroll
      for (int st = 0; st < 2; ++st)
  #pragma unroll
        for (int v = 0; v < 16; ++v) {
          sv[st][v] = __builtin_amdgcn_exp2f(fmaf(sv[st][v], c2, -mc));
          lsum += sv[st][v];
        }
      {
        const LanePair t2 = swap32(__float_as_uint(lsum));
        lsum = __uint_as_float(t2.a) + __uint_as_float(t2.b);
      }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
      // Keep the P.V operand reads below the softmax: hoisting them above it would keep 16
      // operand registers per lane alive across the exp2 work.
      __builtin_amdgcn_sched_barrier(0);
      if (!__all(alpha == 1.0f)) {  // the running max moved for some query of this wave
  #pragma unroll
        for (int db = 0; db < DB; ++db)
  #pragma unroll
          for (int v = 0; v < 16; ++v) oacc[db][v] *= alpha;
      }
  #pragma unroll
      for (int st = 0; st < 2; ++st)
  #pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int o = 8 * hf;
          const uint4 pw = make_uint4(pack_bf16x2(sv[st][o + 0], sv[st][o + 1]),
                                      pack_bf16x2(sv[st][o + 2], sv[st][o + 3]),
                                      pack_bf16x2(sv[st][o + 4], sv[st][o + 5]),
                                      pack_bf16x2(sv[st][o + 6], sv[st][o + 7]));
  #pragma unroll
          for (int db = 0; db < DB; ++db) {
            // A operand of O^T += V^T P^T: lane (dim 32*db + l32, key group half) needs V[key][dim]
            // for the 8 keys whose probabilities it holds in pw.  Two transposed LDS reads
            // (ds_read_b64_tr_b16): in each 16-lane group, output lane j gets element j%4 of the
            // 4-element read of group lane 4e + j/4, so group lane i reads dims
            // 16*(G&1) + 4*(i&3) .. +3 of key row 4*half + i/4 (and that row + 8).  With the
            // V pitch of DH+32 elements the 4 rows x 4 column chunks of two groups land on 64
            // distinct banks.
            const int G = lane >> 4, il = lane & 15;
            const uint16_t* vp = &Vs[buf][(st * 32 + hf * 16 + 4 * half + (il >> 2)) * VKP + db * 32 + 16 * (G & 1) + 4 * (il & 3)];
            const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vp));
            const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vp + 8 * VKP));
            const v8i16 a16 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            const bf16x8 a = __builtin_bit_cast(bf16x8, a16);
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8(pw), oacc[db], 0, 0, 0);
          }
        }
    };

    // Pipeline: LDS holds tile t (computing) and tile t+1 (stored at the end of iteration t);
    // tile t+1's loads are issued before tile t's compute, which covers their latency.  (A
    // second register set, two tiles ahead, measured no faster and cost 22 registers.)
    gload(0, kr, vr);
    swrite(0, kr, vr);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      gload(t + 1, kr, vr);
      compute(t);
      swrite((t + 1) & 1, kr, vr);
      __syncthreads();
    }

    if (!qvalid) return;
    // Output layout of O^T: lane holds query l32, dims db*32 + 8*(v/4) + 4*half + v%4.
    if (ncb == 1) {
      const float inv = 1.f / l_run;
      uint16_t* orow = static_cast<uint16_t*>(p.out) + (static_cast<size_t>(b * p.N + node) * p.Hq + h) * DH;
  #pragma unroll
      for (int db = 0; db < DB; ++db)
  #pragma unroll
        for (int vq = 0; vq < 4; ++vq) {
          const int d0 = db * 32 + 8 * vq + 4 * half;
          uint2 w2;
          w2.x = pack_bf16x2(oacc[db][vq * 4 + 0] * inv, oacc[db][vq * 4 + 1] * inv);
          w2.y = pack_bf16x2(oacc[db][vq * 4 + 2] * inv, oacc[db][vq * 4 + 3] * inv);
          *reinterpret_cast<uint2*>(orow + d0) = w2;
        }
      if (p.lse && half == 0)
        p.lse[(static_cast<size_t>(b) * p.Hq + h) * p.N + node] = (m_run * p.scale_log2 + log2f(l_run)) * kLn2;
    } else {
      // The partial output goes out in the MFMA register order: one 16 KB block per (job, query
      // tile, wave), float4 (db, vq) of lane l at [(db*4 + vq)*64 + l], so every store
      // instruction writes 1 KB of consecutive bytes (the combine reads it in the same order).
      // chunk slot: per (sequence, KV head) chunk c, or the chunk-job index of a balanced plan
      const size_t rowi = p.plan ? (static_cast<size_t>(job / p.Hkv) * p.Hq + h) * p.N + node
                                 : (static_cast<size_t>(b * p.Hq + h) * p.N + node) * p.nchunks + c;
      const size_t slot = p.plan ? ((static_cast<size_t>(job / p.Hkv) * p.Hkv + g) * p.qtiles + qt) * NWV + wv
                                 : ((static_cast<size_t>(b * p.Hkv + g) * p.nchunks + c) * p.qtiles + qt) * NWV + wv;
      float4* po = reinterpret_cast<float4*>(p.part_o) + slot * (DB * 4 * 64) + lane;
  #pragma unroll
      for (int db = 0; db < DB; ++db)
  #pragma unroll
        for (int vq = 0; vq < 4; ++vq)
          po[(db * 4 + vq) * 64] =
              make_float4(oacc[db][vq * 4 + 0], oacc[db][vq * 4 + 1], oacc[db][vq * 4 + 2], oacc[db][vq * 4 + 3]);
      if (half == 0) p.part_ml[rowi] = make_float2(m_run * p.scale_log2, l_run);
    }
  };
  if constexpr (PERSIST) {
    // Persistent: the grid (a multiple of the XCD count) strides over the workgroup indices,
    // so every index a workgroup takes maps to its own XCD, as in a launch of its own.
    for (int vb = static_cast<int>(blockIdx.x); vb < p.vblocks; vb += static_cast<int>(gridDim.x)) {
      __syncthreads();  // the previous index's last tile may still be read from LDS
      run(vb);
    }
  } else {
    run(static_cast<int>(blockIdx.x));
  }
}

// Merge of the chunk partials: O = sum_c 2^(m_c - m) O_c / sum_c 2^(m_c - m) l_c, as an online
// log-sum-exp over the chunks.  One thread per float4 of the attention kernel's register-order
// partial blocks (the same position in every chunk's block), so each wave reads 1 KB of
// consecutive bytes per chunk; the partials of up to CB chunks are requested before any is
// used (CB covers every chunk of the one-sequence launches: one round trip to memory).
template <int DH, int CB, int NWV>
__global__ __launch_bounds__(256) void attn_combine_kernel(const AttnParams p) {
  constexpr int DB = DH / 32, SLOT = DB * 4 * 64;  // float4 per (job, query tile, wave) block
  const size_t gid = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  const int pos = static_cast<int>(gid % SLOT);
  const size_t slot = gid / SLOT;                   // ((b*Hkv + g)*qtiles + qt)*NWV + wv
  const int wv = static_cast<int>(slot % NWV);
  const int qt = static_cast<int>((slot / NWV) % p.qtiles);
  const size_t bg = slot / (static_cast<size_t>(NWV) * p.qtiles);
  if (bg >= static_cast<size_t>(p.B) * p.Hkv) return;
  const int g = static_cast<int>(bg % p.Hkv), b = static_cast<int>(bg / p.Hkv);
  const int lane = pos % 64, dbvq = pos / 64, l32 = lane & 31, half = lane >> 5;
  const int m = qt * (NWV * 32) + wv * 32 + l32;
  if (m >= p.M) return;
  const int i = m / p.G, h = g * p.G + m % p.G;
  const int d0 = (dbvq / 4) * 32 + 8 * (dbvq % 4) + 4 * half;
  const int Lb = clamp_prefix(p, p.prefix_len[b], false);
  const int ncb = p.plan ? p.plan[3 * b] : max(1, (Lb + p.CK - 1) / p.CK);
  if (ncb == 1) return;  // the attention kernel wrote this row itself
  // chunk c of this row: slot (b, g, c) per sequence, or slot j0 + c of a balanced plan
  size_t mlbase, mlstride, pfirst, cstride;
  if (p.plan) {
    const size_t j0 = static_cast<size_t>(p.plan[3 * b + 2]);
    mlbase = (j0 * p.Hq + h) * p.N + i;
    mlstride = static_cast<size_t>(p.Hq) * p.N;
    pfirst = ((j0 * p.Hkv + g) * p.qtiles + qt) * (static_cast<size_t>(NWV) * SLOT);
    cstride = static_cast<size_t>(p.Hkv) * p.qtiles * NWV * SLOT;
  } else {
    mlbase = (static_cast<size_t>(b * p.Hq + h) * p.N + i) * p.nchunks;
    mlstride = 1;
    pfirst = ((bg * p.nchunks) * p.qtiles + qt) * (static_cast<size_t>(NWV) * SLOT);
    cstride = static_cast<size_t>(p.qtiles) * NWV * SLOT;  // float4 per chunk
  }
  const float4* pbase = reinterpret_cast<const float4*>(p.part_o) + pfirst + static_cast<size_t>(wv) * SLOT + pos;
  float M = -INFINITY, L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c0 = 0; c0 < ncb; c0 += CB) {
    float2 ml[CB];
    float4 po[CB];
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const int c = c0 + u;
      ml[u] = c < ncb ? p.part_ml[mlbase + c * mlstride] : make_float2(-INFINITY, 0.f);
      po[u] = c < ncb ? pbase[c * cstride] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      if (ml[u].x == -INFINITY) continue;
      const float mn = fmaxf(M, ml[u].x);
      const float a = exp2f(M - mn);  // 0 while M is -inf
      const float w = exp2f(ml[u].x - mn);
      acc.x = acc.x * a + w * po[u].x;
      acc.y = acc.y * a + w * po[u].y;
      acc.z = acc.z * a + w * po[u].z;
      acc.w = acc.w * a + w * po[u].w;
      L = L * a + w * ml[u].y;
      M = mn;
    }
  }
  const float inv = 1.f / L;
  uint16_t* orow = static_cast<uint16_t*>(p.out) + (static_cast<size_t>(b * p.N + i) * p.Hq + h) * DH;
  uint2 w2;
  w2.x = pack_bf16x2(acc.x * inv, acc.y * inv);
  w2.y = pack_bf16x2(acc.z * inv, acc.w * inv);
  *reinterpret_cast<uint2*>(orow + d0) = w2;
  if (p.lse && d0 == 0) p.lse[(static_cast<size_t>(b) * p.Hq + h) * p.N + i] = (M + log2f(L)) * kLn2;
}

// fp32: one wave per query row (b, node i, head h); lanes run over keys for the scores and
// over head dimensions for P.V.
template <int DH>
__global__ __launch_bounds__(256) void tree_attn_f32_kernel(const AttnParams p) {
  const int rowid = blockIdx.x * 4 + (threadIdx.x >> 6);  // ((b*N + i)*Hq + h)
  if (rowid >= p.B * p.N * p.Hq) return;
  const int lane = threadIdx.x & 63;
  const int h = rowid % p.Hq, i = (rowid / p.Hq) % p.N, b = rowid / (p.Hq * p.N);
  const int g = h / p.G;
  const int Lb = clamp_prefix(p, p.prefix_len[b], lane == 0 && i == 0 && h == 0);
  const float* qrow = static_cast<const float*>(p.q) + static_cast<size_t>(rowid) * DH;
  float qv[DH];
#pragma unroll
  for (int d = 0; d < DH; d += 4) {
    const float4 t = *reinterpret_cast<const float4*>(qrow + d);
    qv[d] = t.x; qv[d + 1] = t.y; qv[d + 2] = t.z; qv[d + 3] = t.w;
  }
  const size_t kvbase = (static_cast<size_t>(b) * p.Hkv + g) * p.L_cap * DH;
  const float* Kg = static_cast<const float*>(p.k) + kvbase;
  const float* Vg = static_cast<const float*>(p.v) + kvbase;
  const uint32_t* ancrow =
      p.anc + static_cast<size_t>(b) * p.mask_stride + static_cast<size_t>(i) * p.W;
  const int nkeys = Lb + p.N;
  float m_run = -INFINITY, l_run = 0.f, acc[DH / 64];
#pragma unroll
  for (int e = 0; e < DH / 64; ++e) acc[e] = 0.f;
  // P.V takes every chunk as 64 keys in batches of kF whose V rows are requested before any is
  // used; each key's weight is read from its lane with readlane (the key index is uniform).
  // Keys past the last one read its V row (in bounds) and, like masked or underflowed keys,
  // carry weight zero, which adds nothing whatever the row holds.  With dh = 64 the chunk's
  // V rows go out together with its K rows.
  constexpr int kF = DH == 64 ? 64 : 16;
  auto vload = [&](int key, int e) {
    return Vg[static_cast<size_t>(min(key, nkeys - 1)) * DH + lane + 64 * e];
  };
  for (int k0 = 0; k0 < nkeys; k0 += 64) {
    float vv[kF][DH / 64];
    if constexpr (DH == 64) {
#pragma unroll
      for (int u = 0; u < kF; ++u) vv[u][0] = vload(k0 + u, 0);
    }
    const int kk = k0 + lane;
    bool ok = kk < nkeys;
    if (ok && kk >= Lb) {
      const int j = kk - Lb;
      ok = (ancrow[j >> 5] >> (j & 31)) & 1u;
    }
    float s = -INFINITY;
    if (ok) {
      const float* kr = Kg + static_cast<size_t>(kk) * DH;
      float a = 0.f;
#pragma unroll
      for (int d = 0; d < DH; d += 4) {
        const float4 t = *reinterpret_cast<const float4*>(kr + d);
        a = fmaf(qv[d], t.x, a);
        a = fmaf(qv[d + 1], t.y, a);
        a = fmaf(qv[d + 2], t.z, a);
        a = fmaf(qv[d + 3], t.w, a);
      }
      s = a * p.scale_log2;
    }
    const float tmax = wave_max(s);
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    const float pj = exp2f(s - m_use);
    l_run = l_run * alpha + wave_sum(pj);
    m_run = m_new;
#pragma unroll
    for (int e = 0; e < DH / 64; ++e) acc[e] *= alpha;
#pragma unroll
    for (int j = 0; j < 64; j += kF) {
      if constexpr (DH != 64) {
#pragma unroll
        for (int u = 0; u < kF; ++u)
#pragma unroll
          for (int e = 0; e < DH / 64; ++e) vv[u][e] = vload(k0 + j + u, e);
      }
#pragma unroll
      for (int u = 0; u < kF; ++u) {
        const float pb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pj), j + u));
#pragma unroll
        for (int e = 0; e < DH / 64; ++e) acc[e] = pb != 0.f ? fmaf(pb, vv[u][e], acc[e]) : acc[e];
      }
    }
  }
  float* orow = static_cast<float*>(p.out) + static_cast<size_t>(rowid) * DH;
  const float inv = 1.f / l_run;
#pragma unroll
  for (int e = 0; e < DH / 64; ++e) orow[lane + 64 * e] = acc[e] * inv;
  if (p.lse && lane == 0) p.lse[(static_cast<size_t>(b) * p.Hq + h) * p.N + i] = (m_run + log2f(l_run)) * kLn2;
}

// ---------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------

// Sequences ranked by decreasing (clamped) prefix length, ties by index: order[rank] = b.
//
// With `plan` (a batch whose host plan splits the keys): a balanced split from the actual
// lengths.  The host sizes chunks from the longest prefix only, so with uneven lengths the
// chunk count rarely fills whole rounds of the chip (8 sequences of 9.6k-29.8k keys gave 528
// workgroups, two full rounds and 16 in a third).  Here the batch's keys are cut into about
// c_target chunks of near-equal length Lc: each sequence takes floor(L_b / Lc) chunks (at least
// 1, at most the host's per-sequence count), the remaining chunks go to the largest remainders,
// each sequence's chunk length is rounded up to whole key tiles and its count recomputed (so no
// chunk is empty).  The chunk-jobs are tabled longest sequence first, chunks in order.
constexpr int kOrderMaxB = 1024;

__global__ __launch_bounds__(kOrderMaxB) void seq_order_kernel(const AttnParams p, int32_t* order,
                                                               int32_t* plan, uint32_t* jtab,
                                                               int c_target) {
  __shared__ int Ls[kOrderMaxB];
  __shared__ int ns[kOrderMaxB];
  __shared__ int rk[kOrderMaxB];
  __shared__ int shared_lc;
  const int b = threadIdx.x;
  if (b < p.B) Ls[b] = clamp_prefix(p, p.prefix_len[b], false);
  __syncthreads();
  int rank = 0, Lb = 0;
  if (b < p.B) {
    Lb = Ls[b];
    for (int j = 0; j < p.B; ++j) rank += Ls[j] > Lb || (Ls[j] == Lb && j < b);
    order[rank] = b;
    rk[b] = rank;
  }
  if (!plan) return;
  if (b == 0) {
    long long tot = 0;
    for (int j = 0; j < p.B; ++j) tot += Ls[j];
    const long long lc = (tot + c_target - 1) / c_target;
    shared_lc = static_cast<int>(std::max<long long>(MV_ATTN_MIN_CHUNK, std::min<long long>(lc, 1 << 30)));
  }
  __syncthreads();
  const int lc = shared_lc;
  int n = 0, rem = 0;
  if (b < p.B) {
    n = std::max(1, Lb / lc);
    rem = Lb - n * lc;  // > 0 only where a chunk more could go
    ns[b] = n;
  }
  __syncthreads();
  int given = 0;
  for (int j = 0; j < p.B; ++j) given += ns[j];
  const int deficit = c_target - given;
  // +1 chunk for the `deficit` largest remainders (ties by index)
  if (b < p.B && deficit > 0 && rem > 0) {
    int better = 0;
    for (int j = 0; j < p.B; ++j) {
      const int rj = Ls[j] - ns[j] * lc;
      if (rj > 0 && (rj > rem || (rj == rem && j < b))) ++better;
    }
    if (better < deficit) ++n;
  }
  int ck = kKT;
  if (b < p.B) {
    ck = std::max(kKT, (Lb + n - 1) / n);
    ck = (ck + kKT - 1) / kKT * kKT;
    n = Lb > 0 ? (Lb + ck - 1) / ck : 1;
  }
  __syncthreads();
  if (b < p.B) ns[b] = n;
  __syncthreads();
  if (b < p.B) {
    int start = 0;
    for (int j = 0; j < p.B; ++j) start += rk[j] < rank ? ns[j] : 0;
    plan[3 * b] = n;
    plan[3 * b + 1] = ck;
    plan[3 * b + 2] = start;
    for (int c = 0; c < n; ++c) jtab[start + c] = (static_cast<uint32_t>(b) << 16) | static_cast<uint32_t>(c);
  }
  int total = 0;
  for (int j = 0; j < p.B; ++j) total += ns[j];
  // p.nchunks is the total of chunk slots here (c_target + B bounds the chunks)
  for (int j = total + static_cast<int>(threadIdx.x); j < p.nchunks; j += blockDim.x) jtab[j] = kNoJob;
}

struct AttnPlan {
  int qtiles = 1, CK = 256, nchunks = 1;
  bool ordered = false;  // a length ordering of the sequences in the workspace
  bool balanced = false;  // ... and a balanced chunk plan from the actual lengths
  int c_target = 0;       // chunks the balanced plan aims for (whole batch)
  size_t ws_bytes = 0;
};

// Chunking (split-KV): aim for MV_ATTN_TARGET_WG workgroups (MV_ATTN_TARGET_WG_BATCH for a
// batch) so that the chip stays busy, but keep chunks of at least MV_ATTN_MIN_CHUNK keys:
// every chunk writes an fp32 partial output as large as its query block, so short chunks turn
// a K/V-streaming kernel into a partial-output-writing one.  `beside` plans the persistent
// launch on half of the CUs (the targets then count its workgroup indices).
// CUs of the current device (cached per device; 0 if the runtime cannot say)
int current_cus() {
  constexpr int kMaxDev = 64;
  static int cus[kMaxDev] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDev && cus[dev] > 0) return cus[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < kMaxDev) cus[dev] = n;
  return n;
}

AttnPlan plan_attn(int dt, int B, int N, int Hq, int Hkv, int dh, int max_L, bool beside) {
  AttnPlan a;
  if (dt == MV_F32) return a;
  const int M = N * (Hq / Hkv);
  a.qtiles = ceil_div(M, kNWV * 32);
  const long long base = static_cast<long long>(B) * Hkv * a.qtiles;
  // A batch splits only as far as its (sequence, KV head, query tile) jobs stay within the
  // batch target (rounding down): the jobs of a large batch already fill the chip, and every
  // extra chunk writes M x dh partials that the combine reads back.  A small batch of long
  // sequences (a few jobs per CU) does split, so that the longest jobs do not set the tail.
  const long long target = B > 1 ? (beside ? MV_ATTN_TARGET_WG_BESIDE : MV_ATTN_TARGET_WG_BATCH)
                                 : MV_ATTN_TARGET_WG;
  int want = static_cast<int>(B > 1 ? std::max<long long>(1, target / base)
                                    : std::max<long long>(1, (target + base - 1) / base));
  const int cap = std::max(1, ceil_div(max_L, MV_ATTN_MIN_CHUNK));
  want = std::min(want, cap);
  auto chunk_keys = [&](int w) {
    const int c = ceil_div(std::max(max_L, 1), w);
    return std::max(MV_ATTN_MIN_CHUNK, (c + kKT - 1) / kKT * kKT);
  };
  // One sequence in a launch of its own: its workgroups run one per CU (the kernel's registers
  // allow no second), so they go in rounds of the CU count.  Of the chunk counts up to the
  // target's, take the one whose rounds x tiles per chunk is least (fewer chunks on ties):
  // 131072 keys x 8 KV heads x 7 query tiles on 256 CUs took 37 chunks, 8 full rounds and a
  // ninth of 24 workgroups; 32 chunks make 7 rounds of 64 tiles.
  const int ncu = B == 1 && !beside ? current_cus() : 0;
  if (ncu > 0 && base * want > ncu) {
    long long best = -1;
    int bw = want;
    for (int w = want; w >= 1; --w) {
      const int c = chunk_keys(w), nc = std::max(1, ceil_div(max_L, c));
      const long long cost = ceil_div(base * nc, static_cast<long long>(ncu)) * (c / kKT);
      if (best < 0 || cost <= best) {
        best = cost;
        bw = w;
      }
    }
    want = bw;
  }
  const int ck = chunk_keys(want);
  a.CK = ck;
  a.nchunks = std::max(1, ceil_div(max_L, ck));
  a.ordered = B > 1 && B <= kOrderMaxB;
#if MV_ATTN_BALANCED
  a.balanced = a.ordered && a.nchunks > 1;
#endif
  if (a.balanced) {
    // chunks aimed for: the batch's workgroup target (at most the host plan's chunk count);
    // the at-least-one-chunk rule can add up to one per sequence, so slots = target + B
    const long long per_chunk = static_cast<long long>(Hkv) * a.qtiles;  // workgroups per chunk
    a.c_target = static_cast<int>(std::min<long long>(static_cast<long long>(B) * a.nchunks,
                                                      std::max<long long>(B, target / per_chunk)));
    a.nchunks = a.c_target + B;  // total chunk slots (partials, job table)
  }
  // chunk slots of the partials: per (sequence, KV head) nchunks, or nchunks in total
  const size_t cslots = a.balanced ? static_cast<size_t>(a.nchunks) : static_cast<size_t>(B) * a.nchunks;
  Carver c(nullptr);
  if (a.ordered) c.take<int32_t>(B);
  if (a.balanced) {
    c.take<int32_t>(3 * static_cast<size_t>(B));
    c.take<uint32_t>(static_cast<size_t>(a.nchunks));
  }
  if (a.nchunks > 1) {
    const size_t rows = cslots * Hq * N;
    const size_t tile_rows = cslots * Hkv * a.qtiles * kNWV * 32;
    c.take<float>(tile_rows * dh);  // register-order blocks, padded to whole query tiles
    c.take<float2>(rows);
  }
  a.ws_bytes = c.bytes();
  return a;
}

template <int NWV>
void launch_combine(const AttnParams& p, int dh, int nchunks, hipStream_t st) {
  const long long slots = static_cast<long long>(p.B) * p.Hkv * p.qtiles * NWV;
  const dim3 g64(static_cast<unsigned>(ceil_div(slots * (2 * 4 * 64), 256LL))),
      g128(static_cast<unsigned>(ceil_div(slots * (4 * 4 * 64), 256LL)));
  if (nchunks <= 4) {
    if (dh == 64) attn_combine_kernel<64, 4, NWV><<<g64, 256, 0, st>>>(p);
    else attn_combine_kernel<128, 4, NWV><<<g128, 256, 0, st>>>(p);
  } else if (nchunks <= 8) {
    if (dh == 64) attn_combine_kernel<64, 8, NWV><<<g64, 256, 0, st>>>(p);
    else attn_combine_kernel<128, 8, NWV><<<g128, 256, 0, st>>>(p);
  } else {
    if (dh == 64) attn_combine_kernel<64, 16, NWV><<<g64, 256, 0, st>>>(p);
    else attn_combine_kernel<128, 16, NWV><<<g128, 256, 0, st>>>(p);
  }
}

size_t attn_workspace(int dt, int B, int N, int Hq, int Hkv, int dh, int max_L, bool beside) {
  if ((dt != MV_F32 && dt != MV_BF16) || B < 1 || N < 1 || Hq < 1 || Hkv < 1 || max_L < 0) return 0;
  if (Hq % Hkv != 0 || (dh != 64 && dh != 128) || N > MV_MAX_NODES) return 0;
  return plan_attn(dt, B, N, Hq, Hkv, dh, max_L, beside).ws_bytes;
}

int tree_attn(int dt, int B, int N, int Hq, int Hkv, int dh, int L_cap, int max_L, const void* q,
              const void* k_cache, const void* v_cache, const int32_t* prefix_len,
              const uint32_t* anc_mask, int mask_stride, float scale, void* out, float* lse,
              int32_t* dev_status, void* ws, size_t ws_bytes, void* stream, bool beside) {
  if (dt != MV_F32 && dt != MV_BF16) return MV_ERR_INVALID_ARG;
  if (B < 1 || N < 1 || Hq < 1 || Hkv < 1 || max_L < 0 || L_cap < N) return MV_ERR_INVALID_ARG;
  if (!q || !k_cache || !v_cache || !prefix_len || !anc_mask || !out) return MV_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return MV_ERR_INVALID_ARG;
  if (dh != 64 && dh != 128) return MV_ERR_UNSUPPORTED;
  if (N > MV_MAX_NODES) return MV_ERR_UNSUPPORTED;
  if (max_L > L_cap - N) return MV_ERR_INVALID_ARG;
  if (mask_stride != 0 && mask_stride < N * ((N + 31) / 32)) return MV_ERR_INVALID_ARG;
  // bf16 K/V are read through buffer resources over one (sequence, KV head) slice, whose
  // byte size must fit the 31-bit offsets.
  if (dt == MV_BF16 && static_cast<long long>(L_cap) * dh * 2 > 0x7fffffffLL) return MV_ERR_UNSUPPORTED;
  const AttnPlan a = plan_attn(dt, B, N, Hq, Hkv, dh, max_L, beside);
  MV_TRY(check_ws(ws, ws_bytes, a.ws_bytes));
  AttnParams p{};
  p.B = B; p.N = N; p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv; p.M = N * p.G;
  p.L_cap = L_cap; p.max_L = max_L; p.CK = a.CK; p.nchunks = a.nchunks; p.qtiles = a.qtiles;
  p.W = (N + 31) / 32;
  p.scale_log2 = (scale > 0.f ? scale : 1.0f / sqrtf(static_cast<float>(dh))) * kLog2e;
  p.q = q; p.k = k_cache; p.v = v_cache; p.prefix_len = prefix_len; p.anc = anc_mask;
  p.mask_stride = mask_stride;
  p.out = out; p.lse = lse; p.status = dev_status;
  hipStream_t st = as_stream(stream);
  if (dt == MV_F32) {
    const int rows = B * N * Hq;
    const int blocks = (rows + 3) / 4;
    if (dh == 64) tree_attn_f32_kernel<64><<<blocks, 256, 0, st>>>(p);
    else tree_attn_f32_kernel<128><<<blocks, 256, 0, st>>>(p);
    return launch_status();
  }
  // Persistent grid of the launch beside other kernels: one workgroup per CU on half of the
  // CUs (rounded down to whole XCDs), striding over the workgroup indices.  (Measured on the
  // 70B-shaped forked step: 3/8 of the CUs 1194, half 1363, 5/8 1318 steps/s.)
  int pgrid = 0;
  if (beside) {
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return MV_ERR_HIP;
    pgrid = std::max(kXcds, ncu / (2 * kXcds) * kXcds);
  }
  Carver c(ws);
  int32_t* order = a.ordered ? c.take<int32_t>(B) : nullptr;
  int32_t* plan = a.balanced ? c.take<int32_t>(3 * static_cast<size_t>(B)) : nullptr;
  uint32_t* jtab = a.balanced ? c.take<uint32_t>(static_cast<size_t>(a.nchunks)) : nullptr;
  const size_t cslots = a.balanced ? static_cast<size_t>(a.nchunks) : static_cast<size_t>(B) * a.nchunks;
  if (a.nchunks > 1) {
    const size_t rows = cslots * Hq * N;
    const size_t tile_rows = cslots * Hkv * a.qtiles * kNWV * 32;
    p.part_o = c.take<float>(tile_rows * dh);
    p.part_ml = c.take<float2>(rows);
  }
  const long long jobs = static_cast<long long>(cslots) * Hkv;
  const long long grid = (jobs + kXcds - 1) / kXcds * kXcds * a.qtiles;
  if (grid > (1LL << 30)) return MV_ERR_UNSUPPORTED;
  p.jobs = static_cast<int>(jobs);
  p.vblocks = static_cast<int>(grid);
  if (order) {
    // one wave per 64 sequences: a small workgroup is placed at once on a busy chip
    seq_order_kernel<<<1, std::min(kOrderMaxB, ceil_div(B, 64) * 64), 0, st>>>(p, order, plan, jtab, a.c_target);
    MV_TRY(launch_status());
    p.order = order;
    p.plan = plan;
    p.jtab = jtab;
  }
  if (beside) {
    const int g = static_cast<int>(std::min<long long>(grid, pgrid));
    if (dh == 64) tree_attn_bf16_kernel<64, kNWV, true><<<g, kNWV * 64, 0, st>>>(p);
    else tree_attn_bf16_kernel<128, kNWV, true><<<g, kNWV * 64, 0, st>>>(p);
  } else {
    const int g = static_cast<int>(grid);
    if (dh == 64) tree_attn_bf16_kernel<64, kNWV, false><<<g, kNWV * 64, 0, st>>>(p);
    else tree_attn_bf16_kernel<128, kNWV, false><<<g, kNWV * 64, 0, st>>>(p);
  }
  MV_TRY(launch_status());
  if (a.nchunks > 1) {
    launch_combine<kNWV>(p, dh, a.nchunks, st);
    MV_TRY(launch_status());
  }
  return MV_OK;
}

}  // namespace
}  // namespace mv

using namespace mv;

extern "C" {

MV_API size_t mv_tree_attn_verify_workspace(int dt, int B, int N, int Hq, int Hkv, int dh, int max_L) {
  return attn_workspace(dt, B, N, Hq, Hkv, dh, max_L, false);
}

MV_API int mv_tree_attn_verify(int dt, int B, int N, int Hq, int Hkv, int dh, int L_cap, int max_L,
                               const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* prefix_len, const uint32_t* anc_mask,
                               int mask_stride, float scale,
                               void* out, float* lse, int32_t* dev_status, void* ws,
                               size_t ws_bytes, void* stream) {
  return tree_attn(dt, B, N, Hq, Hkv, dh, L_cap, max_L, q, k_cache, v_cache, prefix_len, anc_mask,
                   mask_stride, scale, out, lse, dev_status, ws, ws_bytes, stream, false);
}

MV_API size_t mv_tree_attn_verify_beside_workspace(int dt, int B, int N, int Hq, int Hkv, int dh,
                                                   int max_L) {
  return attn_workspace(dt, B, N, Hq, Hkv, dh, max_L, true);
}

MV_API int mv_tree_attn_verify_beside(int dt, int B, int N, int Hq, int Hkv, int dh, int L_cap,
                                      int max_L, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* prefix_len,
                                      const uint32_t* anc_mask, int mask_stride, float scale,
                                      void* out, float* lse, int32_t* dev_status, void* ws,
                                      size_t ws_bytes, void* stream) {
  return tree_attn(dt, B, N, Hq, Hkv, dh, L_cap, max_L, q, k_cache, v_cache, prefix_len, anc_mask,
                   mask_stride, scale, out, lse, dev_status, ws, ws_bytes, stream, true);
}

}  // extern "C"
