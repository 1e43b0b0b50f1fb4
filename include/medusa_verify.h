/*
 * medusa_verify.h -- C ABI of the MI355X (gfx950) Medusa tree-verification library.
 *
 * One verify step of Medusa decoding, split into the operations below:
 *
 *   (a1) Medusa residual block   h_k = SiLU(W_res^(k) h) + h
 *   (a2) Medusa head projection  logits_k = W_head^(k) h_k, its top-s_k tokens and log-sum-exp
 *   (a3) candidate-tree assembly from a parent array -> per-node ancestor-or-self bitmask
 *   (a4/a5) tree-masked GQA attention of every tree node over the KV prefix plus its ancestors
 *   (a6/a7) acceptance: greedy longest accepted path, or the speculative min(1, P_t/P_d) rule
 *           with residual resampling, plus one extra ("bonus") token.
 *
 * Sources (web pages on the method):
 *   [MX]  "Medusa Explained: Multi-Head Speculative Decoding Guide" (aifetchly blog):
 *         "The Architectural Blueprint" (head equations), "1. Combinatorial Tree Construction",
 *         "2. Single-Pass Tree Attention Verification" (mask M_tree, 5-candidate example,
 *         greedy longest-path rule).
 *   [MTP] "Multi-Token Prediction: Draft-Model-Free Speculative Decoding" (globaltechdigest
 *         blog): "The 2D Tree Attention Mask", "Tree-Structured Attention Verification"
 *         (Figure 1's text box: the target adds one token after the committed path), and the
 *         verification-engine code (parent-array trees with -1 roots; the first of equally
 *         long accepted paths is kept).
 *   [SD]  "Speculative Decoding & Medusa Tree Attention" (akmalkhaniub blog), section 2,
 *         "The Acceptance Sampling Rule" (alpha and the residual distribution).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers are DEVICE pointers (memory of the current HIP device) unless marked "host".
 *   The caller owns every buffer.  The library never allocates, frees or synchronises;
 *   scratch memory comes only through (ws, ws_bytes), sized by the matching *_workspace()
 *   query (0 bytes is a valid answer).  ws must be 256-byte aligned.
 * - stream is a hipStream_t passed as void* (NULL = the default stream).  Every call only
 *   enqueues work on it and returns.
 * - Host-side argument checks run first; on failure nothing is launched and a negative
 *   mv_status is returned.  Data-dependent errors (a malformed parent array, a prefix that
 *   does not fit the cache, a tree deeper than the output) cannot be seen by the host; they
 *   are OR-ed as bit flags (MV_DEV_*) into *dev_status when dev_status is not NULL, and the
 *   kernels still finish with every access in bounds (outputs of the offending item are then
 *   unspecified).  The caller zeroes dev_status before the call.
 * - Layouts are row-major, innermost dimension last.  bf16 tensors hold raw bfloat16 bits.
 * - Thread safety: no mutable global state.  Calls that share one workspace must be ordered
 *   (the same stream does that).
 * - Numerics: every dot product accumulates in fp32; the acceptance decisions and the
 *   residual sampling are taken in fp64.
 */
#ifndef MEDUSA_VERIFY_H
#define MEDUSA_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifndef MV_API
#if defined(__GNUC__) || defined(__clang__)
#define MV_API __attribute__((visibility("default")))
#else
#define MV_API
#endif
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MV_OK = 0,
  MV_ERR_INVALID_ARG = -1,   /* NULL required pointer, non-positive size, bad enum value */
  MV_ERR_INVALID_TREE = -2,  /* reserved for host-validated tree specs (binding level) */
  MV_ERR_UNSUPPORTED = -3,   /* a size or dtype the library does not implement (see each call) */
  MV_ERR_WORKSPACE = -4,     /* ws is NULL/misaligned or ws_bytes is below the query */
  MV_ERR_HIP = -5            /* a HIP launch or runtime call failed */
} mv_status;

typedef enum { MV_F32 = 0, MV_BF16 = 1 } mv_dtype;
typedef enum {
  MV_ACCEPT_GREEDY = 0,
  MV_ACCEPT_SPECULATIVE = 1,
  MV_ACCEPT_MULTICAND = 2
} mv_accept_mode;

/* target_dt of greedy mv_accept_paths when the target rows arrive as argmax ids. */
#define MV_TARGET_IDS 2

/* Device-side error flags (OR-ed into *dev_status). */
#define MV_DEV_BAD_PARENT   0x1  /* parents[i] outside [-1, i) (parents must be topological) */
#define MV_DEV_BAD_RANK     0x2  /* a node's sibling rank is >= the candidate width of its depth */
#define MV_DEV_TOO_DEEP     0x4  /* a node's depth exceeds D */
#define MV_DEV_BAD_PREFIX   0x8  /* prefix_len[b] < 0, > max_L, or prefix_len[b] + N > L_cap */
#define MV_DEV_BAD_TOKEN    0x10 /* a node token is outside [0, V) */
#define MV_DEV_BAD_PATH     0x20 /* a committed path node outside [j, N), or a length outside [0, D] */

/* Limits of the library. */
#define MV_MAX_NODES 256   /* N: tree nodes */
#define MV_MAX_DEPTH 16    /* D: tree depth */
#define MV_MAX_TOPK  16    /* s: candidates per head / per depth */
#define MV_MAX_BATCH_HEADS 64  /* B for the Medusa heads (bf16; fp32 takes up to 32) */
#define MV_MAX_HEADS 16    /* K: Medusa heads */

/* Human-readable text of a mv_status value (static storage). */
MV_API const char* mv_status_string(int status);

/* MV_OK when `device` is a gfx950 GPU, MV_ERR_UNSUPPORTED for another GPU, MV_ERR_HIP when
 * the device cannot be queried. */
MV_API int mv_device_check(int device);

/* Library version, major*10000 + minor*100 + patch. */
MV_API int mv_version(void);

/* ---------------------------------------------------------------------------------------
 * (a1)+(a2) Medusa heads.  [MX] "The Architectural Blueprint": every head k has one residual
 * block without bias, h_k = SiLU(W_res^(k) h) + h, followed by a vocabulary projection whose
 * softmax is the head's distribution; [MX] "1. Combinatorial Tree Construction": each head
 * contributes its top-s_k tokens.  Softmax is monotone, so the top-s_k of the distribution are
 * the top-s_k logits, and lse = log sum_v exp(logit_v) gives the distribution itself.
 *
 *   dt        MV_BF16 (weights, h and logits in bf16) or MV_F32.
 *   B         batch (1..MV_MAX_BATCH_HEADS for bf16, 1..32 for fp32), d model width,
 *             V vocabulary, K heads (1..16).
 *             bf16 needs d % 32 == 0; fp32 needs d % 4 == 0.
 *   h         [B, d] dt.
 *   w_res     [K, d, d] dt, W_res^(k)[out][in] (row-major, out-major).
 *   w_head    [K, V, d] dt.
 *   hk        [B, K, d] fp32 output of the residual block, or NULL.  (It is always kept in ws.)
 *   s_per_head host [K], 1 <= s_k <= s_max <= MV_MAX_TOPK, s_max <= V.
 *   logits    [B, K, V] dt output, or NULL (then the logits are never written to memory).
 *   topk_ids  int32, topk_vals fp32: element (b, k, r) at  b*ld_topk + k*s_max + r, r < s_max;
 *             ld_topk >= K*s_max (0 means K*s_max).  Rank r orders larger logit first, equal
 *             logits by lower token id.  Slots r >= s_k hold id -1 and value -inf.
 *   lse       [B, K] fp32 natural-log log-sum-exp of each head's logits, or NULL.
 *   ws        workspace from mv_medusa_heads_workspace(dt, B, d, V, K, s_max).  The residual
 *             call leaves the head input there for the projection, the projection leaves its
 *             per-block partials there for the selection, so the calls of one step must get
 *             the same ws (mv_medusa_heads does all three).
 * Values are accumulated in fp32.  With bf16 weights, h_k stays fp32: the projection feeds it
 * to the bf16 matrix cores as the sum of two bf16 numbers (high part + remainder), which keeps
 * about 16 significant bits of h_k in every product.
 * ------------------------------------------------------------------------------------- */
MV_API size_t mv_medusa_heads_workspace(int dt, int B, int d, int V, int K, int s_max);

MV_API int mv_medusa_residual(int dt, int B, int d, int K, const void* h, const void* w_res,
                       float* hk, void* ws, size_t ws_bytes, void* stream);

/* The projection (streams W_head once; per-32-row block top-s and (max, sum exp) partials go to
 * ws; logits are written only when `logits` is not NULL) and the selection (merges those
 * partials into topk_ids / topk_vals / lse).  They are two calls so that the weight stream can
 * be timed on its own; both need the same ws, after mv_medusa_residual. */
MV_API int mv_medusa_head_project(int dt, int B, int d, int V, int K, const int* s_per_head,
                                  int s_max, const void* w_head, void* logits, void* ws,
                                  size_t ws_bytes, void* stream);

MV_API int mv_medusa_head_select(int dt, int B, int d, int V, int K, const int* s_per_head,
                                 int s_max, int32_t* topk_ids, float* topk_vals, int ld_topk,
                                 float* lse, void* ws, size_t ws_bytes, void* stream);

MV_API int mv_medusa_heads(int dt, int B, int d, int V, int K, const int* s_per_head, int s_max,
                    const void* h, const void* w_res, const void* w_head, float* hk,
                    void* logits, int32_t* topk_ids, float* topk_vals, int ld_topk, float* lse,
                    void* ws, size_t ws_bytes, void* stream);

/* Allocation-free variant of mv_medusa_heads, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, outputs and results as mv_medusa_heads, without the workspace: its scratch lives
 * in a device array inside the library (MV_HEADS_NOALLOC_SCRATCH_BYTES, 32 MiB), one copy per
 * GPU, held until the process ends.  The first call on a device looks the array's address up
 * on that device (the current one); no call allocates or frees memory.
 *   Sizes whose mv_medusa_heads_workspace(dt, B, d, V, K, s_max) exceeds the array are
 *   rejected with MV_ERR_UNSUPPORTED before anything is launched; argument errors are those
 *   of mv_medusa_heads.
 *   Every call on one GPU shares that GPU's array, which keeps the last call's contents (no
 *   part of it needs clearing: each call writes what it reads).  Calls that overlap on one
 *   GPU (other streams, other host threads) race on it: serialise them. */
#define MV_HEADS_NOALLOC_SCRATCH_BYTES (32 << 20)

MV_API int mv_medusa_heads_noalloc(int dt, int B, int d, int V, int K, const int* s_per_head,
                                   int s_max, const void* h, const void* w_res,
                                   const void* w_head, float* hk, void* logits,
                                   int32_t* topk_ids, float* topk_vals, int ld_topk, float* lse,
                                   void* stream);

/* Top-s entries of each of R rows of a logit matrix (the same selection rule as the heads),
 * for candidates that come from logits the caller already has -- e.g. the base model's own
 * head ("Head 0", which predicts the next token in [MX] "The Architectural Blueprint").
 * Also a draft model's per-depth logits, whose softmax is the draft distribution P_draft of
 * [SD] "The Acceptance Sampling Rule": lse then gives each row's log-sum-exp.
 *   x      row r starts at x + r*ldx elements (dt), V entries per row.
 *   ids    int32, vals fp32 (vals may be NULL): row r at r*ld_out, s entries.
 *   lse    fp32 [R] or NULL: log sum_v exp(x[r][v]), accumulated in fp32.
 * 1 <= s <= MV_MAX_TOPK, s <= V.  No workspace. */
MV_API int mv_topk_rows(int dt, int R, int V, int s, const void* x, long long ldx, int32_t* ids,
                 float* vals, int ld_out, float* lse, void* stream);

/* ---------------------------------------------------------------------------------------
 * (a3) Candidate-tree assembly.  [MTP] verification-engine code: the tree is a parent array,
 * -1 marking a node that hangs directly off the prefix (several such roots form a forest);
 * [MTP] "The 2D Tree Attention Mask": node i may see node j iff j is an ancestor of i or
 * j == i; [MX] "2. Single-Pass Tree Attention Verification" gives the same mask in additive
 * form.  [MX] "1. Combinatorial Tree Construction": the depth-k nodes are the top-s_k tokens
 * of the head for depth k.
 *
 *   N        1..MV_MAX_NODES nodes, parents [N] int32, topological: -1 <= parents[i] < i.
 *   anc_mask [N, W] uint32 output, W = ceil(N/32): bit (j % 32) of word j/32 of row i is set
 *            iff j is an ancestor of i or j == i.
 *   depth    [N] int32 output (1 for a node whose parent is -1), or NULL.
 *   cand     [B, D, s_max] int32 candidate tokens per depth, or NULL (then node_tokens is
 *            not written).  Node i takes cand[b][depth_i - 1][rank_i], rank_i = number of
 *            earlier nodes with the same parent.  s_per_depth (host [D], or NULL = s_max each)
 *            bounds rank_i; D <= MV_MAX_DEPTH.
 *   node_tokens [B, N] int32 output (may be NULL when cand is NULL).
 *   dev_status  MV_DEV_BAD_PARENT / MV_DEV_BAD_RANK / MV_DEV_TOO_DEEP flags, or NULL.
 * ------------------------------------------------------------------------------------- */
MV_API int mv_build_tree_mask(int N, const int32_t* parents, int B, int D, int s_max,
                       const int* s_per_depth, const int32_t* cand, uint32_t* anc_mask,
                       int32_t* depth, int32_t* node_tokens, int32_t* dev_status,
                       void* stream);

/* ---------------------------------------------------------------------------------------
 * Dynamic (confidence-ranked) tree: an alternative to (a3) for per-sequence trees.
 * [MTP] "2. EAGLE & EAGLE-2: Feature-Level Autoregression": the tree follows the candidates'
 * confidence (deeper where the predictions are sure, wider where they are not); [MTP]
 * "Production Deployment Guidelines", "Dynamic Tree Depth Tuning"; [MX] "1. Combinatorial
 * Tree Construction": head k proposes the candidates of depth k.
 *
 * A node is a path of candidate ranks (r_1 .. r_d), scored by sum_k log p_k(r_k) with
 * log p = min(0, cand_vals - cand_lse) summed in fp64 from the first head on.  Each
 * sequence's tree is its N best paths: higher score first, then smaller depth, then smaller
 * ranks from the first head on.  Nodes are laid out breadth first, children of a node in rank
 * order (parents[i] < i).  The outputs feed mv_tree_attn_verify (mask_stride = N *
 * ceil(N/32)) and mv_accept_paths (parents_stride = N).
 *
 *   cand_ids, cand_vals [B, D, s_max]: head k's candidates best first (int32 token ids, fp32
 *            logits), e.g. from mv_medusa_head_select with ld = D * s_max.
 *   cand_lse [B, D] fp32 (each head's log-sum-exp) or NULL when cand_vals are
 *            log-probabilities.
 *   s_per_depth host [D] (1 <= s_k <= s_max) or NULL for s_max everywhere; D <= 15,
 *            s_max <= MV_MAX_TOPK, N <= MV_MAX_NODES, and the number of paths
 *            sum_d prod_{k<=d} s_k must be >= N (else MV_ERR_INVALID_ARG).
 *   parents, depth (1-based), node_tokens [B, N] int32; anc_mask [B, N, ceil(N/32)] uint32
 *            (ancestor-or-self bits, as mv_build_tree_mask); node_logp [B, N] fp32 (the
 *            path's score) or NULL.
 *   dev_status MV_DEV_BAD_RANK when a chosen candidate's id is negative (an empty slot).
 * One 64-lane workgroup per sequence; no workspace.
 * ------------------------------------------------------------------------------------- */
MV_API int mv_build_dynamic_tree(int B, int D, int s_max, const int* s_per_depth, int N,
                                 const int32_t* cand_ids, const float* cand_vals,
                                 const float* cand_lse, int32_t* parents, int32_t* depth,
                                 int32_t* node_tokens, uint32_t* anc_mask, float* node_logp,
                                 int32_t* dev_status, void* stream);

/* ---------------------------------------------------------------------------------------
 * (a4)+(a5) Tree-masked GQA attention.  [MX] "2. Single-Pass Tree Attention Verification":
 * the tree is flattened into one packed sequence after the prefix and each node attends to
 * the whole prefix plus its ancestors (additive mask 0 / -inf); [MTP] "The 2D Tree Attention
 * Mask" adds the node itself.  Scores are scaled dot products, softmax over the visible keys.
 *
 *   dt       MV_BF16 or MV_F32 (q, caches and out share it).  dh in {64, 128}.
 *   q        [B, N, Hq, dh]; query head h reads KV head h / (Hq/Hkv).  Hq % Hkv == 0.
 *   k_cache, v_cache [B, Hkv, L_cap, dh]: rows [0, L_b) of sequence b are the prefix and rows
 *            [L_b, L_b + N) hold the tree's own keys/values in node order; L_b =
 *            prefix_len[b] (device int32 [B]), 0 <= L_b <= max_L, L_b + N <= L_cap.
 *            bf16: one (sequence, KV head) slice must stay below 2 GiB (L_cap * dh * 2 <
 *            2^31, i.e. L_cap < 8388608 at dh = 128), else MV_ERR_UNSUPPORTED.
 *   anc_mask [N, ceil(N/32)] uint32 from mv_build_tree_mask (one tree for the batch,
 *            mask_stride = 0), or one mask per sequence, sequence b's at
 *            anc_mask + b * mask_stride (mask_stride >= N * ceil(N/32) words; e.g. from
 *            mv_build_dynamic_tree).
 *   scale    softmax scale; <= 0 selects 1/sqrt(dh).
 *   out      [B, N, Hq, dh] dt output.  lse [B, Hq, N] fp32 natural-log output, or NULL.
 *   ws       workspace from mv_tree_attn_verify_workspace() with the same sizes: the prefix
 *            is split into chunks processed by separate workgroups and merged afterwards.
 *   dev_status MV_DEV_BAD_PREFIX when a prefix length is out of range (it is then clamped).
 * ------------------------------------------------------------------------------------- */
MV_API size_t mv_tree_attn_verify_workspace(int dt, int B, int N, int Hq, int Hkv, int dh, int max_L);

MV_API int mv_tree_attn_verify(int dt, int B, int N, int Hq, int Hkv, int dh, int L_cap, int max_L,
                        const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* prefix_len, const uint32_t* anc_mask, int mask_stride,
                        float scale, void* out, float* lse, int32_t* dev_status, void* ws,
                        size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * (a4)+(a5) The same tree-masked GQA attention, launched to run beside bandwidth-bound kernels
 * on another stream (the Medusa heads of the same step; the passages above define it).
 * Arguments, layouts, results and errors are those of mv_tree_attn_verify; ws must come from
 * mv_tree_attn_verify_beside_workspace() with the same sizes.  The bf16 path runs as one
 * persistent 8-wave workgroup per CU on half of the CUs; each holds nearly all of its CU's
 * registers, so the other stream's workgroups run on the other half and both progress at once.
 * On its own it is about twice as slow as mv_tree_attn_verify; fp32 runs the same kernel as
 * mv_tree_attn_verify.
 * ------------------------------------------------------------------------------------- */
MV_API size_t mv_tree_attn_verify_beside_workspace(int dt, int B, int N, int Hq, int Hkv, int dh,
                                                   int max_L);

MV_API int mv_tree_attn_verify_beside(int dt, int B, int N, int Hq, int Hkv, int dh, int L_cap,
                                      int max_L, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* prefix_len,
                                      const uint32_t* anc_mask, int mask_stride, float scale,
                                      void* out, float* lse, int32_t* dev_status, void* ws,
                                      size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * Target LM head over the verification rows (the row before acceptance).  [MX] "2. Single-Pass
 * Tree Attention Verification", step 2: the target model outputs a distribution for every
 * candidate node; step 3 compares each node with the target's greedy prediction.  [SD] "The
 * Acceptance Sampling Rule": P_target is the softmax of the target's logits.
 *
 * logits[t][v] = sum_j W[v][j] x[t][j] for T rows of final hidden states (B*(N+1) per verify
 * step: per sequence the last prefix position, then node 0..N-1).  Per row the call returns
 * the greedy token (argmax over v, lowest id on ties) and optionally its logit and
 * LSE = log sum_v exp(logits[t][v]); the [T, V] logits are never written.  The argmax ids feed
 * mv_accept_paths with target_dt = MV_TARGET_IDS; P_target(v) = exp(logit - LSE).
 *
 *   dt         MV_BF16 only (MV_F32 -> MV_ERR_UNSUPPORTED).  d % 32 == 0.
 *   x [T, d], w_lm [V, d] (the LM head weight, one row per vocabulary entry), bf16.
 *   argmax_ids [T] int32; max_logit [T] fp32 or NULL; lse [T] fp32 or NULL.
 *   Accumulation in fp32.  No device flags.
 * ------------------------------------------------------------------------------------- */
MV_API size_t mv_lm_head_workspace(int dt, int T, int d, int V);

MV_API int mv_lm_head_argmax(int dt, int T, int d, int V, const void* x, const void* w_lm,
                             int32_t* argmax_ids, float* max_logit, float* lse, void* ws,
                             size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * (a6)+(a7) Acceptance and the extra token.  Row 0 of target/draft is the distribution after
 * the last prefix token; row i+1 the one after node i.  Each node is tested against the row
 * of its parent, and is accepted when it and all of its ancestors pass.  The committed path ends at the deepest accepted node, the lowest index winning
 * ties (the [MTP] engine code keeps the first of equally long paths); the target then adds
 * one more token after it (the text box of [MTP] Figure 1).
 *
 * MV_ACCEPT_GREEDY ([MX] "2. Single-Pass Tree Attention Verification", step 3): target holds
 *   logits (dt); node i passes iff its token equals the argmax of its parent's row (lowest
 *   index on ties).  The extra token is the argmax of the terminal's row.
 * MV_ACCEPT_SPECULATIVE ([SD] "The Acceptance Sampling Rule"): target, draft hold fp32
 *   probabilities; alpha_i = min(1, P_t(x_i)/P_d(x_i)) at the parent's row (1 when
 *   P_d(x_i) = 0); node i passes iff uniforms[b][i] < alpha_i.  The extra token is drawn
 *   with uniforms[b][N] by inverse CDF (first v whose running sum exceeds u * total, over
 *   token order) from normalize(max(0, P_t - P_d)) of the terminal's row when the terminal
 *   has children (all of them rejected), from P_t when that residual is all zero, and from
 *   P_t of the terminal's row when the terminal is a leaf.  Decisions and sums are in fp64.
 * MV_ACCEPT_MULTICAND ([SD] "The Acceptance Sampling Rule" applied to the siblings in turn;
 *   [MTP] "The 2D Tree Attention Mask": the tree is evaluated by rejection sampling): same
 *   inputs as speculative.  Walking from the prefix with P = P_t of the current row, the
 *   children of the current node are tested in index order: alpha_i = min(1, P(x_i)/P_d(x_i))
 *   at the current (parent) row, accepted iff uniforms[b][i] < alpha_i, and the walk moves to
 *   the first accepted child (P = P_t of its row).  A rejection replaces P by
 *   normalize(max(0, P - P_d)) (P_t when that is all zero) before the next sibling.  The
 *   extra token is drawn with uniforms[b][N] from P where the walk stops.  Lossless when
 *   the siblings are independent draws from the parent row's P_d.  alpha is -1 for nodes
 *   that were never tested; node_accept marks the path.  Each rejection followed by a
 *   further sibling costs one pass over the vocabulary row.
 *
 *   target_dt MV_BF16 or MV_F32 for greedy; must be MV_F32 for the two sampling modes.
 *            Greedy also takes MV_TARGET_IDS: target then holds the target's greedy token per
 *            row, int32 [B, N+1] (e.g. from mv_lm_head_argmax), and needs no workspace.
 *   parents [N] int32 (one tree for the batch, parents_stride = 0) or one parent array per
 *            sequence at parents + b * parents_stride (parents_stride >= N).
 *   node_tokens [B, N] int32; target [B, N+1, V]; draft [B, N+1, V] fp32 and
 *   uniforms [B, N+1] fp32 in [0, 1) (sampling modes only, else NULL).
 *   D        max tree depth (size of the outputs), 1..MV_MAX_DEPTH.
 *   accept_len [B] int32; path_nodes [B, D] int32 (-1 padded); out_tokens [B, D+1] int32
 *            (accepted tokens, then the extra token, then -1).
 *   node_accept [B, N] uint8 (1 = accepted) or NULL; alpha [B, N] fp32 (sampling modes) or
 *            NULL.
 *   dev_status MV_DEV_BAD_PARENT / MV_DEV_TOO_DEEP / MV_DEV_BAD_TOKEN flags, or NULL.
 * ------------------------------------------------------------------------------------- */
MV_API size_t mv_accept_paths_workspace(int mode, int B, int N, int V);

MV_API int mv_accept_paths(int mode, int target_dt, int B, int N, int V, int D,
                    const int32_t* parents, int parents_stride,
                    const int32_t* node_tokens, const void* target, const float* draft,
                    const float* uniforms, int32_t* accept_len, int32_t* path_nodes,
                    int32_t* out_tokens, uint8_t* node_accept, float* alpha,
                    int32_t* dev_status, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * Speculative acceptance fed by the target LM head and the Medusa heads' logits, without any
 * [B][N+1][V] probability tensor.  [SD] "The Acceptance Sampling Rule" (the rule, P_target =
 * softmax of the target's logits); [MX] "2. Single-Pass Tree Attention Verification", step 2
 * (the target outputs a distribution at every candidate node); [MX] "The Architectural
 * Blueprint" (head k's softmax is the draft distribution of the depth-k tokens; every head reads
 * the same hidden state, so all depth-k nodes of a sequence share it).
 *   P_t at row r (row 0 = after the prefix, row i+1 = after node i) = softmax(W_lm x_t[b][r]);
 *   P_d at row r = softmax(draft_logits[b][depth(r)]) with depth(row 0) = 0 and depth(row i+1)
 *   = depth of node i.  Node i's test uses its parent's row: alpha_i = min(1, P_t(x_i)/P_d(x_i))
 *   (1 when P_d(x_i) = 0), accepted iff uniforms[b][i] < alpha_i and every ancestor is accepted.
 *   The path, its tokens and the extra token follow mv_accept_paths(MV_ACCEPT_SPECULATIVE):
 *   the extra token is drawn with uniforms[b][N] from normalize(max(0, P_t - P_d)) at the
 *   terminal's row when it has children (P_t if that is all zero), else from P_t.
 * How it is computed: P_t(x_i) from one dot product W_lm[x_i] . x_t[parent row] (fp32
 * accumulation) against lse_t, P_d(x_i) from one draft logit against draft_lse, both in fp64;
 * after the walk one streaming pass over W_lm (per 128 sequences, on the matrix cores) makes
 * each sequence's terminal target row, the draft logits its draft row, and the fp64 segment
 * sums / inverse CDF of mv_accept_paths
 * draw the extra token.  With fp32 dot products the decisions can differ from an exact one only
 * where |u - alpha| is within the dot product's rounding (~1e-5 relative).
 *   draft_dt      MV_F32 or MV_BF16: type of draft_logits [B][D][V] (row k = depth k+1).
 *   x_t [B][N+1][d] bf16, w_lm [V][d] bf16 (d % 32 == 0); lse_t [B][N+1] fp32 natural-log
 *   log-sum-exp of the target logits (mv_lm_head_argmax gives it); draft_lse [B][D] fp32 the
 *   log-sum-exp of each draft row.  Other arguments, outputs and errors as mv_accept_paths.
 *   ws from mv_accept_speculative_lm_workspace(B, N, V).
 * ------------------------------------------------------------------------------------- */
MV_API size_t mv_accept_speculative_lm_workspace(int B, int N, int V);

MV_API int mv_accept_speculative_lm(int draft_dt, int B, int N, int V, int d, int D,
                                    const int32_t* parents, int parents_stride,
                                    const int32_t* node_tokens, const void* x_t,
                                    const void* w_lm, const float* lse_t,
                                    const void* draft_logits, const float* draft_lse,
                                    const float* uniforms, int32_t* accept_len,
                                    int32_t* path_nodes, int32_t* out_tokens,
                                    uint8_t* node_accept, float* alpha, int32_t* dev_status,
                                    void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * Commit of the accepted path (the step after acceptance).  [MTP] "The 2D Tree Attention
 * Mask": the engine commits the longest accepted path, and a node sees exactly its ancestors,
 * so the kept path is an ordinary causal continuation of the prefix; [MTP] "Production
 * Deployment Guidelines": the KV entries of unselected branches are culled.
 *
 * For every sequence b with L = prefix_len[b] and len = accept_len[b]: cache rows
 * L + path_nodes[b][j] move to rows L + j (j < len) in k_cache and v_cache for every KV head,
 * then prefix_out[b] = L + len.  The next step's attention then sees prefix + accepted tokens as
 * one contiguous prefix.  In place (sources are staged before any write); rows L + len ..
 * L + N - 1 keep stale tree entries and are overwritten by the next step's tree.
 *
 *   dt         MV_BF16 or MV_F32 (the caches' element type).  dh in {64, 128}.
 *   k_cache, v_cache [B, Hkv, L_cap, dh] (modified); prefix_len [B] int32 (read);
 *   prefix_out [B] int32 (written; may be prefix_len itself, for an in-place advance, or a
 *            second buffer so that a replayed step keeps its input prefix);
 *   path_nodes [B, D], accept_len [B] int32 as written by mv_accept_paths.
 *   dev_status MV_DEV_BAD_PREFIX (L + N > L_cap) / MV_DEV_BAD_PATH; such a sequence keeps its
 *            cache rows and prefix_out[b] = prefix_len[b].  No workspace.
 * ------------------------------------------------------------------------------------- */
MV_API int mv_kv_commit(int dt, int B, int Hkv, int dh, int L_cap, int N, int D, void* k_cache,
                        void* v_cache, const int32_t* prefix_len, int32_t* prefix_out,
                        const int32_t* path_nodes, const int32_t* accept_len,
                        int32_t* dev_status, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MEDUSA_VERIFY_H */
