/*
 * qgg.h -- C-ABI of the MI355X (gfx950) quantized MoE grouped-GEMM library.
 *
 * The path (Orbit page, section 时刻细节, "Active-expert-chunked
 * dequantization"): every token activates only the experts its router picks;
 * the picked experts are grouped into fixed-size chunks, each chunk's 4-bit
 * weights are dequantized to BF16 only while the chunk is being computed, the
 * expert projections run as one grouped matrix multiplication, and the
 * high-precision copy is released before the next chunk.  The base stays
 * frozen in its low-precision format (same page, 单节点 Kimi-K2.6 驱散: INT4;
 * 单节点 DeepSeek V4 Flash 驱散: FP4).  The backward computes no gradient for the
 * frozen base (时刻细节, bypass-base-weight-grad GEMM backward).
 *
 * Weight formats (page "超大规模开放权重模型技术解析", 三 微缩放量化的原理:
 * groups of 32 elements share one scale):
 *   QGG_FMT_MXFP4  E2M1 nibbles, one E8M0 exponent byte per 32 elements along K
 *   QGG_FMT_INT4   two's-complement nibbles, one BF16 scale per 32 along K
 *
 * Conventions for every call
 *  - Pointers are DEVICE memory owned by the caller unless marked "host".
 *    The library never allocates device memory: scratch and intermediates
 *    come from the caller's `workspace`, sized by qgg_workspace_bytes().  A
 *    call uses its workspace until its last kernel ends (it also holds the
 *    counters from which the grouped GEMM launches hand out their work), so
 *    calls that may run at the same time need workspaces of their own.
 *  - BF16 tensors are passed as uint16_t bit patterns.  Row-major throughout.
 *  - Calls are asynchronous on `stream` (a hipStream_t; 0 = null stream) and
 *    never synchronize with the host, so a whole call can be captured into a
 *    HIP graph and replayed.  Variant QGG_CHUNKED launches a fixed number of
 *    chunk iterations, ceil(min(E, T*k) / C); the active-expert count and the
 *    per-chunk tile bounds are read on the device, and iterations past the
 *    last live chunk return at once.  No call issues hipMemset.
 *  - Argument errors are detected on the host before any launch and returned
 *    as a status; nothing aborts.  Data errors found on the device (a
 *    non-finite router logit, an expert id outside [0, E)) set *err_flag to a
 *    nonzero value when err_flag is not NULL; the caller zeroes it first.
 *  - Limits: 1 <= k <= 32, k <= E <= 1024, T*k < 2^31; K % 128 == 0 and
 *    N % 64 == 0 for dequant_grouped_gemm, d % 128 == 0 and inter % 128 == 0
 *    for moe_ffn_fwd, d % 256 == 0 and inter % 256 == 0 for moe_dx_bwd; every
 *    BF16 matrix read as a GEMM A operand (the activations and the P x inter
 *    or P x 2 inter intermediates) under 4 GiB.  Sizes outside these return
 *    QGG_ERR_UNSUPPORTED.
 *  - Pair index p = t*k + j names token t's j-th routed expert.  "Sorted
 *    order" lists pairs expert by expert (ascending id), ascending p inside an
 *    expert; row i of a sorted tensor belongs to pair perm[i].
 */
#ifndef QGG_H_
#define QGG_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* qgg_stream_t; /* same type as hipStream_t */
typedef int qgg_status;

#define QGG_OK 0
#define QGG_ERR_INVALID_ARG 1
#define QGG_ERR_UNSUPPORTED 2
#define QGG_ERR_WORKSPACE_TOO_SMALL 3
#define QGG_ERR_HIP 4

#define QGG_FMT_MXFP4 1
#define QGG_FMT_INT4 2

/* variant: CHUNKED dequantizes one chunk of active experts into BF16 scratch
 * and runs a BF16 grouped GEMM over it (the pages' formulation); FUSED decodes
 * nibbles and scales in registers and feeds BF16 MFMA directly (no scratch). */
#define QGG_CHUNKED 0
#define QGG_FUSED 1

/* dequant_grouped_gemm flags */
#define QGG_A_SORTED 0        /* a is [P][K] already in sorted order          */
#define QGG_A_TOKENS 1        /* a is [T][K]; sorted row i reads a[perm[i]/k] */
#define QGG_TRANSPOSE_W 2     /* y = a . W (reduce over N; a is [.][N], y [P][K]) */
#define QGG_DEQUANT_ONLY 4    /* CHUNKED only: write the first chunk's BF16
                                 weights [chunk][N][K] to the start of the
                                 workspace and stop (a test hook)            */

/* workspace queries */
#define QGG_CALL_PERMUTE 1
#define QGG_CALL_GEMM 2
#define QGG_CALL_FFN_FWD 3
#define QGG_CALL_DX_BWD 4
#define QGG_CALL_LORA_BWD 5   /* d = N, N_or_inter = adapter rank */
#define QGG_CALL_FFN_LORA_BWD 6   /* N_or_inter = inter; adapters up to rank 128 */

/* Storage layouts of the packed weights and scales (the bytes are the same,
 * only their order differs):
 * QGG_LAYOUT_ROWS  packed [E][N][K/2]: element k of a row is byte k>>1, low
 *                  nibble for even k; scales [E][N][K/32].
 * QGG_LAYOUT_MFMA  tiles of 32 rows x 64 K: packed [E][N/32][K/64][64][16]
 *                  where slot L = 32*h + c holds the 16 bytes of scale group
 *                  2*j + h of row 32*cb + c (tile (cb, j)), nibble order as
 *                  in a row; scales [E][N/32][K/64][64] in the same slot
 *                  order.  One wavefront reads one K step of 32 rows as a
 *                  single contiguous 1 KiB block.  Produced from ROWS by
 *                  qgg_repack_weights (once, when the frozen base is
 *                  loaded); needs N % 32 == 0 and K % 64 == 0. */
#define QGG_LAYOUT_ROWS 0
#define QGG_LAYOUT_MFMA 1

/* A frozen 4-bit weight tensor of E experts, each [N][K] (out x in).
 * scales hold uint8 E8M0 codes (value 2^(c-127), 255 = NaN) for MXFP4 and
 * uint16 BF16 bits for INT4, in the order `layout` names.  Host struct,
 * device pointers, read only. */
typedef struct {
  int32_t fmt;
  int32_t E, N, K;
  const uint8_t* packed;
  const void* scales;
  int32_t layout;
} qgg_qweight;

/* Routing permutation, all device arrays written by expert_permute.
 * counts[E]      pairs routed to each expert
 * offsets[E+1]   exclusive prefix sum of counts
 * perm[P]        sorted row -> pair index
 * inv_perm[P]    pair index -> sorted row
 * active[E]      ids of experts with counts > 0, ascending; rest are -1
 * n_active[1]    number of active experts
 * perm and inv_perm may be NULL when P = T*k is 0; the others never. */
typedef struct {
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* inv_perm;
  int32_t* active;
  int32_t* n_active;
} qgg_perm;

/* moe_route -- per token, top-k experts of fp32 router logits [T][E] under the
 * key (logit descending, expert id ascending), with gates = softmax over all E
 * renormalised over the k kept experts (equivalently, softmax over the kept
 * logits).  Orbit page, 时刻细节: tokens activate only router-selected experts.
 * Outputs topk_ids [T][k] int32 (slot order = key order) and topk_gates
 * [T][k] fp32 summing to 1 per token.  A non-finite logit sets *err_flag. */
qgg_status moe_route(const float* logits, int T, int E, int k, int32_t* topk_ids,
                     float* topk_gates, int32_t* err_flag, qgg_stream_t stream);

/* expert_permute -- group the T*k (token, expert) pairs by expert: a stable
 * counting sort built from wavefront prefix sums (same passage: the selected
 * experts are grouped into batches before the grouped GEMM).  Fills every
 * array of *p (a host struct of device pointers).  If x and x_perm are both
 * non-NULL it also gathers x_perm[i][:] = x[perm[i]/k][:] (BF16, d columns).
 * Expert ids outside [0, E) set *err_flag and are dropped from the sort.
 * workspace: qgg_workspace_bytes(QGG_CALL_PERMUTE, ...) bytes. */
qgg_status expert_permute(const int32_t* topk_ids, int T, int k, int E, const qgg_perm* p,
                          const uint16_t* x, int d, uint16_t* x_perm, int32_t* err_flag,
                          void* workspace, size_t ws_bytes, qgg_stream_t stream);

/* dequant_grouped_gemm -- one grouped projection over the routed rows
 * (Orbit page, section 时刻细节, "Active-expert-chunked dequantization": the
 * chunk's experts are dequantized for the duration of the chunk and run as
 * one grouped matrix multiplication; the group-32 scales along K follow
 * "超大规模开放权重模型技术解析", 三 微缩放量化的原理):
 * y[i][:] = a_row(i) . W_e^T for every sorted row i of expert e (fp32
 * accumulate, BF16 out), y is [P][N] in sorted order.  With QGG_TRANSPOSE_W
 * the product is a_row(i) . W_e (a is [.][N], y is [P][K]): the transposed
 * access of the input-gradient backward (same Orbit section, the
 * bypass-base-weight-grad GEMM backward).  variant and chunk (experts per
 * chunk, 0 = every expert that can be active, i.e. min(E, T*k) of them) as
 * above; chunking never changes the result.  p must come from
 * expert_permute on the same routing.  QGG_CHUNKED's BF16 scratch is
 * chunk' * N * K * 2 bytes of the workspace, chunk' = chunk or, for 0,
 * min(E, T*k): the host does not know how many experts the routing will
 * activate, so a caller that knows the count passes it as chunk.
 * Exactness: QGG_CHUNKED decodes every code and scale as the format defines
 * (value rounded once to BF16).  QGG_FUSED decodes the same values for every
 * MXFP4 scale code and for INT4 scales that are NaN or finite with
 * magnitude below 2^119; INT4 groups whose scale is +-Inf or has magnitude
 * >= 2^119 are outside its exact domain (qgg_check_weights flags them). */
qgg_status dequant_grouped_gemm(const qgg_qweight* w, const uint16_t* a, int flags,
                                const qgg_perm* p, int T, int k, int variant, int chunk,
                                void* workspace, size_t ws_bytes, uint16_t* y,
                                qgg_stream_t stream);

/* LoRA adapter of one grouped projection (device arrays, BF16 bits):
 * A [E][rank][K] (down), B [E][N][rank] (up); y gains alpha * (a A_e^T) B_e^T.
 * rank is a multiple of 16 in [16, 128]. */
typedef struct {
  int32_t rank;
  float alpha;
  const uint16_t* A;
  const uint16_t* B;
} qgg_lora;

/* lora_grouped_gemm -- dequant_grouped_gemm with a BF16 LoRA adapter on the
 * frozen quantized base: y[i][:] = a_row(i) . W_e^T + u[i] . B_e^T with
 * u[i][:] = alpha * a_row(i) . A_e^T.  Orbit page, opening section: the base
 * stays frozen in its low-precision format and one BF16 adapter on top of it
 * is what trains.  The adapter's form is a reading: the Orbit issue page
 * ("What's the difference between this and the slime framework?") has the
 * maintainers choose orthogonal finetuning (OFT / QOFT) as the default and
 * prefer it to LoRA, which the question raises; the pages give no OFT
 * formula, so the additive low-rank form, the one the pages name and define
 * least ambiguously, is the one built.  u is formed first (fp32 accumulate, stored BF16 in
 * u_out [P][rank], sorted order: the activation the adapter's backward
 * needs); the up projection runs as extra MFMA steps on the same fp32
 * accumulators as the base product, so y is rounded to BF16 once.  Arguments
 * otherwise as dequant_grouped_gemm (same workspace); QGG_TRANSPOSE_W and
 * QGG_DEQUANT_ONLY are rejected (QGG_ERR_INVALID_ARG), a rank outside the
 * limits returns QGG_ERR_UNSUPPORTED. */
qgg_status lora_grouped_gemm(const qgg_qweight* w, const qgg_lora* lora, const uint16_t* a,
                             int flags, const qgg_perm* p, int T, int k, int variant, int chunk,
                             void* workspace, size_t ws_bytes, uint16_t* u_out, uint16_t* y,
                             qgg_stream_t stream);

/* lora_grouped_gemm_bwd -- the adapter's backward for L = <dY, y> of
 * lora_grouped_gemm, the base frozen (Orbit page, 时刻细节: no gradient is
 * formed for the frozen base; the adapter is what trains).  With du_i =
 * dY_i . B_e (fp32, workspace):
 *   dx[i][:]  = alpha du_i . A_e         BF16 [P][K], sorted order: the
 *               adapter's part of the input gradient (the base part is
 *               dequant_grouped_gemm with QGG_TRANSPOSE_W on the same dY);
 *   dA[e]     = alpha sum_i du_i (x) a_row(i)    fp32 [E][rank][K];
 *   dB[e]     = sum_i dY_i (x) u_i               fp32 [E][N][rank];
 * sums over the rows i of expert e in sorted order; experts with no rows get
 * zeros.  dy [P][N] BF16 sorted; u [P][rank] BF16 as lora_grouped_gemm wrote
 * it; a and flags (QGG_A_TOKENS or 0) as in the forward.  Any of dx, dA, dB
 * may be NULL (not all).  workspace: qgg_workspace_bytes(QGG_CALL_LORA_BWD,
 * T, N, E, k, rank, ...) (it holds du and a transposed copy of B).
 * Deterministic. */
qgg_status lora_grouped_gemm_bwd(const qgg_lora* lora, int E, int N, int K, const uint16_t* a,
                                 int flags, const uint16_t* dy, const uint16_t* u,
                                 const qgg_perm* p, int T, int k, void* workspace,
                                 size_t ws_bytes, uint16_t* dx, float* dA, float* dB,
                                 qgg_stream_t stream);

/* moe_ffn_fwd -- the SwiGLU expert FFN for a routed batch (Orbit page,
 * section 时刻细节: routing, active-expert chunks, temporary dequantization
 * and grouped GEMMs; the expert FFN's SwiGLU form, its gate|up concatenation
 * and the gate-weighted scatter-combine are the workload definition this
 * library targets, T=8192 d=7168 E=256 top-8 inter=2048): route, permute,
 * h = x . W_gu^T (rows [0,inter) of W_gu are gate, [inter, 2*inter) up),
 * a = silu(gate) * up, o = a . W_down^T, y[t] = sum_j g[t,j] * o[pair(t,j)]
 * (fp32 sum in ascending j).  w_gate_up: N = 2*inter, K = d; w_down: N = d,
 * K = inter.  Writes topk_ids/topk_gates [T][k], the arrays of *p, y [T][d];
 * if h_save is not NULL also h [P][2*inter] BF16 in sorted order (needed by
 * moe_dx_bwd). */
qgg_status moe_ffn_fwd(const qgg_qweight* w_gate_up, const qgg_qweight* w_down,
                       const uint16_t* x, const float* logits, int T, int d, int E, int k,
                       int inter, int variant, int chunk, int32_t* topk_ids, float* topk_gates,
                       const qgg_perm* p, uint16_t* h_save, int32_t* err_flag, void* workspace,
                       size_t ws_bytes, uint16_t* y, qgg_stream_t stream);

/* moe_ffn_fwd_noalloc -- moe_ffn_fwd for callers that cannot allocate device
 * memory or hand over a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): the same kernels, with
 * the workspace taken from a library-owned static device array of
 * QGG_STATIC_SCRATCH_BYTES (32 MiB) per GPU, kept until the process ends.
 * Arguments and results as moe_ffn_fwd without workspace / ws_bytes.  A call
 * whose qgg_workspace_bytes(QGG_CALL_FFN_FWD, ...) exceeds the array returns
 * QGG_ERR_WORKSPACE_TOO_SMALL before any launch (e.g. the FUSED decode batch
 * T=64, d=7168, E=384, top-8, inter=2048 needs about 10 MiB; a CHUNKED call
 * needs chunk * 2 * inter * d * 2 bytes of scratch on top).  It calls no
 * allocator.  Every call on one GPU shares that GPU's array and leaves its
 * contents behind; every byte a call reads from it is written by the same
 * call first, so no clearing is needed, but calls that overlap on one GPU
 * (different streams or threads) race and must be serialised by the
 * caller. */
#define QGG_STATIC_SCRATCH_BYTES (32u << 20)
qgg_status moe_ffn_fwd_noalloc(const qgg_qweight* w_gate_up, const qgg_qweight* w_down,
                               const uint16_t* x, const float* logits, int T, int d, int E, int k,
                               int inter, int variant, int chunk, int32_t* topk_ids,
                               float* topk_gates, const qgg_perm* p, uint16_t* h_save,
                               int32_t* err_flag, uint16_t* y, qgg_stream_t stream);

/* moe_ffn_fwd_lora -- moe_ffn_fwd with a BF16 LoRA adapter on the gate_up
 * and/or the down projection (either pointer may be NULL, not both): the
 * forward of the base + adapter path that the Orbit page runs in training
 * and in rollout alike (opening section).  h = x W_gu^T + u_gu B_gu^T with
 * u_gu = alpha_gu x A_gu^T (A_gu [E][rank][d], B_gu [E][2*inter][rank]); a as
 * in moe_ffn_fwd; o = a W_dn^T + u_dn B_dn^T with u_dn = alpha_dn a A_dn^T
 * (A_dn [E][rank][inter], B_dn [E][d][rank]).  u_gate_up / u_down receive u
 * ([P][rank] BF16, sorted order) for each given adapter.  Each up projection
 * accumulates into its GEMM's fp32 accumulators (one BF16 rounding).  The
 * CHUNKED variant runs every chunk's gate_up before any chunk's down when a
 * down adapter is given (its u needs all of a); scratch stays one chunk.
 * Same shapes, workspace (QGG_CALL_FFN_FWD) and errors as moe_ffn_fwd; a
 * rank outside [16, 128] or not a multiple of 16 returns
 * QGG_ERR_UNSUPPORTED. */
qgg_status moe_ffn_fwd_lora(const qgg_qweight* w_gate_up, const qgg_qweight* w_down,
                            const qgg_lora* lora_gate_up, const qgg_lora* lora_down,
                            const uint16_t* x, const float* logits, int T, int d, int E, int k,
                            int inter, int variant, int chunk, int32_t* topk_ids,
                            float* topk_gates, const qgg_perm* p, uint16_t* h_save,
                            uint16_t* u_gate_up, uint16_t* u_down, int32_t* err_flag,
                            void* workspace, size_t ws_bytes, uint16_t* y, qgg_stream_t stream);

/* moe_dx_bwd -- input gradient of moe_ffn_fwd with the base frozen (Orbit
 * page, section 时刻细节, the bypass-base-weight-grad GEMM backward: the
 * frozen base gets no weight gradient, so only dX flows through it; the
 * weights are read transposed): no weight gradient and no gate gradient
 * (gates are constants).
 * dA = (g * dY[t]) . W_down, dH = [dA * up * silu'(gate) | dA * silu(gate)]
 * using h_saved from the forward, dXp = dH . W_gu, dx[t] = sum_j dXp[pair(t,j)]
 * (fp32 sum in ascending j).  dy, dx [T][d] BF16; topk_gates [T][k]. */
qgg_status moe_dx_bwd(const qgg_qweight* w_gate_up, const qgg_qweight* w_down,
                      const uint16_t* dy, const float* topk_gates, const qgg_perm* p,
                      const uint16_t* h_saved, int T, int d, int E, int k, int inter, int variant,
                      int chunk, void* workspace, size_t ws_bytes, uint16_t* dx,
                      qgg_stream_t stream);

/* moe_ffn_bwd_lora -- backward of moe_ffn_fwd_lora for L = <dY, y>: the base
 * frozen and the gates constant, the BF16 adapters trained (Orbit page,
 * opening section: the low-precision base stays frozen and the BF16 adapter
 * on top of it is what trains, in training as in rollout; section 时刻细节:
 * the backward forms no gradient for the frozen base).  Per routed pair with
 * gate g, dO = g dY[t]:
 *   down adapter   du = dO . B_dn (fp32); dA_down[e] = alpha_dn sum du (x) a,
 *                  a = silu(h_gate) h_up recomputed from h_saved;
 *                  dB_down[e] = sum dO (x) u_down;
 *                  its share of dA, alpha_dn du . A_dn, is added to
 *                  dO . W_down before the SwiGLU derivative;
 *   dH = [dA * up * silu'(gate) | dA * silu(gate)] from h_saved;
 *   gate_up adapter  du = dH . B_gu (fp32); dA_gate_up[e] = alpha_gu sum du (x)
 *                  x[t]; dB_gate_up[e] = sum dH (x) u_gate_up;
 *                  its share of dXp, alpha_gu du . A_gu, is added to dH . W_gu;
 *   dx[t] = sum_j dXp[pair(t, j)] (fp32, ascending j; the two shares of a
 *   pair added first).
 * Sums over an expert's rows run in sorted order; experts with no rows get
 * zero gradients.  Arguments: the weights and adapters given to
 * moe_ffn_fwd_lora (either adapter NULL, not both), x [T][d] (its input;
 * needed for dA_gate_up), dy [T][d] BF16, topk_gates and p from that call,
 * h_saved [P][2*inter] and u_gate_up / u_down [P][rank] as it wrote them.
 * Outputs, each nullable (at least one): dx [T][d] BF16, dA_gate_up
 * [E][r][d], dB_gate_up [E][2*inter][r], dA_down [E][r][inter], dB_down
 * [E][d][r] fp32 (written in full).  Same shape limits as moe_dx_bwd; ranks
 * as moe_ffn_fwd_lora.  workspace: qgg_workspace_bytes(QGG_CALL_FFN_LORA_BWD,
 * T, d, E, k, inter, variant, chunk).  The CHUNKED variant runs every chunk's
 * down projection before any chunk's gate_up (the gate_up adapter needs all
 * of dH); scratch stays one chunk.  Deterministic. */
qgg_status moe_ffn_bwd_lora(const qgg_qweight* w_gate_up, const qgg_qweight* w_down,
                            const qgg_lora* lora_gate_up, const qgg_lora* lora_down,
                            const uint16_t* x, const uint16_t* dy, const float* topk_gates,
                            const qgg_perm* p, const uint16_t* h_saved,
                            const uint16_t* u_gate_up, const uint16_t* u_down, int T, int d,
                            int E, int k, int inter, int variant, int chunk, void* workspace,
                            size_t ws_bytes, uint16_t* dx, float* dA_gate_up, float* dB_gate_up,
                            float* dA_down, float* dB_down, qgg_stream_t stream);

/* moe_router_bwd -- the gradient a trainable router receives through the
 * frozen base: L = <dY, y> of moe_ffn_fwd differentiated with respect to the
 * gates and the router logits, the routing choice held fixed (top-k selection
 * is piecewise constant in the logits).  The Orbit page (section 时刻细节)
 * freezes the base and trains what sits beside it; the router's own logits
 * stay in high precision ("超大规模开放权重模型技术解析", section 三).
 *   dgates[t][j]  = <dY[t], o[pair(t,j)]>, formed as <dY[t] . W_down, a> in
 *                   the epilogue of the down-projection backward (the same
 *                   value by the adjoint identity), fp32 partial sums over
 *                   256-column pieces added in ascending order;
 *   dlogits[t][e] = g_j (dg_j - sum_i g_i dg_i) when e is token t's j-th
 *                   kept expert, 0 for every other expert (the backward of
 *                   the softmax over the kept logits).
 * Arguments as moe_dx_bwd, plus topk_ids [T][k] (from moe_route) and three
 * outputs: dx [T][d] BF16 as moe_dx_bwd (nullable: then the gate_up backward
 * GEMM is skipped), dgates [T][k] fp32 (nullable), dlogits [T][E] fp32
 * (nullable; every entry written).  At least one of dgates / dlogits must be
 * given.  Same shape limits, workspace (QGG_CALL_DX_BWD) and errors as
 * moe_dx_bwd; deterministic. */
qgg_status moe_router_bwd(const qgg_qweight* w_gate_up, const qgg_qweight* w_down,
                          const uint16_t* dy, const int32_t* topk_ids, const float* topk_gates,
                          const qgg_perm* p, const uint16_t* h_saved, int T, int d, int E, int k,
                          int inter, int variant, int chunk, void* workspace, size_t ws_bytes,
                          uint16_t* dx, float* dgates, float* dlogits, qgg_stream_t stream);

/* qgg_repack_weights -- copy a QGG_LAYOUT_ROWS weight tensor into the
 * QGG_LAYOUT_MFMA order: packed_out gets E*N*K/2 bytes, scales_out E*N*K/32
 * scale entries (device buffers the caller owns, not aliasing the source).
 * A pure permutation of bytes and scale entries; values are untouched. */
qgg_status qgg_repack_weights(const qgg_qweight* src, uint8_t* packed_out, void* scales_out,
                              qgg_stream_t stream);

/* qgg_check_weights -- scan the scales of a frozen weight tensor (either
 * layout) for values the QGG_FUSED decoder does not reproduce exactly, and
 * set bit 4 (value 4) of *err_flag (device int32, which the caller zeroes
 * first) if there is one: an INT4 BF16 scale that is +-Inf or has magnitude
 * >= 2^119 (the fused decode forms q*s as fma(n' 2^-9, 512 s, -8 s) and needs
 * 512 s finite).  NaN scales decode to NaN in both variants; every MXFP4
 * E8M0 code decodes exactly in both.  Meant for load time, beside
 * qgg_repack_weights; QGG_CHUNKED decodes flagged weights exactly.  The
 * group-32 scale formats: "超大规模开放权重模型技术解析", 三 微缩放量化的原理. */
qgg_status qgg_check_weights(const qgg_qweight* w, int32_t* err_flag, qgg_stream_t stream);

/* Workspace bytes a call needs.  N_or_inter is N for QGG_CALL_GEMM (with K =
 * d) and inter for the FFN calls.  *scratch_bytes (nullable) receives the part
 * that holds dequantized BF16 weights (0 for QGG_FUSED): chunk * max(N*K) * 2. */
size_t qgg_workspace_bytes(int call, int T, int d, int E, int k, int N_or_inter, int variant,
                           int chunk, size_t* scratch_bytes);

/* Measurement hook (not part of the path): while `events` is not NULL, each
 * kernel launch the calling thread makes through this library (every launch
 * function: routing, permutation, each grouped GEMM, each chunk's dequant,
 * combine, ...) is bracketed by hipEventRecord(events[2i]) and
 * hipEventRecord(events[2i+1]) on the call's stream, for the first
 * `capacity` launches (at most 4096) after this call; events are hipEvent_t
 * handles the caller created with timing enabled.  qgg_timing_count() gives
 * the number of launches recorded so far and qgg_timing_kind(i) the kind of
 * launch i (QGG_KERNEL_*).  Pass NULL to stop.  Not for use while the stream
 * is being captured into a graph.  Returns QGG_ERR_INVALID_ARG for a
 * capacity outside [1, 4096]. */
#define QGG_KERNEL_ROUTE 1
#define QGG_KERNEL_PERMUTE 2     /* permutation and M-tile plan */
#define QGG_KERNEL_GEMM 3        /* grouped GEMM y = a W^T */
#define QGG_KERNEL_GEMM_T 4      /* transposed grouped GEMM y = a W */
#define QGG_KERNEL_DEQUANT 5     /* one chunk's dequantization (QGG_CHUNKED) */
#define QGG_KERNEL_COMBINE 6     /* gate-weighted combine / scatter-sum */
#define QGG_KERNEL_LORA 7
#define QGG_KERNEL_ROUTER_BWD 8
#define QGG_KERNEL_OTHER 9
qgg_status qgg_set_timing_events(void* const* events, int capacity);
int qgg_timing_count(void);
int qgg_timing_kind(int i);

/* Human-readable name of a status code (static storage). */
const char* qgg_status_string(qgg_status s);

/* Library version string (static storage). */
const char* qgg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QGG_H_ */
