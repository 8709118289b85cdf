// Host-side declarations shared between the C-ABI layer and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace qgg {

struct PermPtrs {
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* inv_perm;
  int32_t* active;
  int32_t* n_active;
};

enum WSource { kSrcBF16 = 0, kSrcMXFP4 = 1, kSrcINT4 = 2 };
enum AMode { kASorted = 0, kATokens = 1 };
enum Epilogue { kEpiStore = 0, kEpiSwiGLU = 1, kEpiSwiGLUBwd = 2 };

// One grouped GEMM launch over the M-tiles [range[0], range[1]) of a plan.
struct GemmArgs {
  // weights: packed 4-bit (with scales) or BF16; W is [N][K] per expert
  int src;                       // WSource
  const uint8_t* packed;
  const void* scales;
  int layout;                    // QGG_LAYOUT_ROWS | QGG_LAYOUT_MFMA (packed/scales)
  const uint16_t* wbf16;         // BF16 weights, MFMA-tiled, [slots] (src == kSrcBF16)
  int N, K;
  int bf16_slot_base;            // BF16 slot of tile = tile.active_index - base
  // rows (A operand)
  const uint16_t* a;
  int lda;
  int64_t a_rows;                // rows of the A matrix (bounds its buffer resource)
  int amode;                     // AMode
  const int32_t* perm;
  int topk;
  // plan
  const int4* tiles;
  const int32_t* range;          // device: first and one-past-last tile
  int32_t* work;                 // device: item counter (zero before a launch;
                                 // the launch leaves it zero)
  int max_tiles;                 // host bound on range[1] - range[0]
  int mt_rows;                   // rows per M-tile (32 * MB)
  // output
  uint16_t* y;
  int ldy;
  int epi;                       // Epilogue
  int inter;                     // SwiGLU width
  uint16_t* h;                   // fwd: optional h save [P][2I]; bwd: saved h
  const float* gates;            // bwd SwiGLU epilogue: topk gates [T*k]
  // optional LoRA up projection folded into the forward (kEpiStore) GEMM:
  // y += u . B_e^T with u [rows][lora_rank] (sorted order, BF16, already
  // scaled by alpha) and B [E][N][lora_rank] BF16; lora_rank % 16 == 0
  int lora_rank;
  const uint16_t* lora_u;
  const uint16_t* lora_b;
  const uint16_t* lora_da;       // bwd SwiGLU epilogue, optional: [P][inter] BF16 sorted,
                                 // added to g * (dY . W_down) before the SwiGLU
                                 // derivative (a down adapter's share of dA)
  float* gpart;                  // bwd SwiGLU epilogue, optional: per sorted row and
                                 // 256-column item, sum over the item of
                                 // (dY . W_down)[c] * silu(gate)[c] * up[c]; [P][inter/256]
};

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* gates,
                        int32_t* err, hipStream_t s);
// Router gradient from the per-pair partials of <dY . W_down, a> (gpart,
// [P][nitems] by sorted row): dgates [T][k] and dlogits [T][E] (either
// nullable; dlogits fully written).
hipError_t launch_router_bwd(const float* gpart, int nitems, const int32_t* inv_perm,
                             const int32_t* ids, const float* gates, int T, int E, int k,
                             float* dgates, float* dlogits, hipStream_t s);
// u[i][j] = alpha * sum_k a[row(i)][k] A_e[j][k] for the sorted rows of the
// tiles [0, *ntiles) (row(i) = perm[i] / topk for kATokens); A [E][rank][K] BF16,
// u [P][rank] BF16; K % 64 == 0, rank <= 128.
hipError_t launch_lora_u(const uint16_t* x, int K, const int32_t* perm, int topk, int amode,
                         const int4* tiles, const int32_t* ntiles, int max_tiles, int MB,
                         const uint16_t* A, int rank, float alpha, uint16_t* u, hipStream_t s);
// Adapter backward (see lora.hip): bt [E][rank][N] BF16 and du [P][rank] fp32
// scratch; dx [P][K] BF16, dA [E][rank][K] fp32, dB [E][N][rank] fp32, each
// nullable.  N % 64 == 0.
hipError_t launch_lora_bwd(const uint16_t* x, int K, int N, int E, const int32_t* perm, int topk,
                           int amode, const int32_t* offsets, const int4* tiles,
                           const int32_t* ntiles, int max_tiles, int MB, const uint16_t* A,
                           const uint16_t* B, int rank, float alpha, const uint16_t* dy,
                           const uint16_t* u, uint16_t* bt, float* du, uint16_t* dx, float* dA,
                           float* dB, hipStream_t s);
size_t permute_ws_bytes(int64_t P, int E);
hipError_t launch_permute(const int32_t* ids, int64_t P, int E, const PermPtrs& pp, int32_t* err,
                          void* ws, hipStream_t s);
hipError_t launch_gather(const uint16_t* x, int d, const PermPtrs& pp, int E, int k, int64_t P,
                         uint16_t* out, hipStream_t s);
// M-tile plan; chunk_first gets E + 2 entries (chunks past the last live one
// are empty)
hipError_t launch_tile_plan(const PermPtrs& pp, int E, int MT, int C, int4* tiles,
                            int32_t* chunk_first, hipStream_t s);
// permutation followed by the M-tile plan (MT > 0); one launch when P is small
hipError_t launch_permute_plan(const int32_t* ids, int64_t P, int E, const PermPtrs& pp,
                               int32_t* err, void* ws, int MT, int C, int4* tiles,
                               int32_t* chunk_first, hipStream_t s);

// y = a . W^T per tile (reduce over K); output columns are W rows.
hipError_t launch_gemm_nt(const GemmArgs& g, int MB, hipStream_t s);
// y = a . W per tile (reduce over N); output columns are W's K index.
hipError_t launch_gemm_tn(const GemmArgs& g, int MB, hipStream_t s);

// BF16 copy of the weights of active experts [first, first + count) of the
// active list: dst[slot][N][K] row-major, or (tiled_out) in the MFMA-tiled
// BF16 order the grouped GEMMs read: tiles of 32 rows x 64 K, 4 KiB each,
// [slot][N/32][K/64][s = 0..3][slot L = 32*h + c][8 elements], holding
// elements 8*s .. 8*s+7 of scale group 2*j + h of row 32*cb + c.
hipError_t launch_dequant(int fmt, const uint8_t* packed, const void* scales, int layout, int N,
                          int K, const int32_t* active, const int32_t* n_active, int first,
                          int count, bool tiled_out, uint16_t* dst, hipStream_t s);

// Sets bit 4 of *err if any of the n scale entries lies outside the fused
// decoder's exact domain (see dequant_combine.hip).
hipError_t launch_check_scales(int fmt, const void* scales, int64_t n, int32_t* err,
                               hipStream_t s);

// ROWS -> MFMA-tiled copy of packed weights and scales.
hipError_t launch_repack(int fmt, const uint8_t* packed, const void* scales, int E, int N, int K,
                         uint8_t* packed_out, void* scales_out, hipStream_t s);

// out[t] = sum_j w_j * rows[inv_perm[t*k+j]] (w_j = gates[t*k+j], or 1 when
// gates is null), fp32 in ascending j, BF16 out; rows2 (nullable) is added to
// rows term by term.
hipError_t launch_combine(const uint16_t* rows, int d, const int32_t* inv_perm,
                          const float* gates, int T, int k, uint16_t* out, hipStream_t s,
                          const uint16_t* rows2 = nullptr);
// a [P][inter] = silu(h_gate) * h_up from h [P][2 inter] (sorted rows below
// offsets[E]).
hipError_t launch_swiglu_act(const uint16_t* h, int inter, const int32_t* offsets, int E,
                             int64_t P, uint16_t* a, hipStream_t s);
// Backward of a down-projection adapter inside the FFN: the upstream gradient
// of sorted row i is gates[perm[i]] * dy[perm[i] / topk] (token-ordered dy);
// the adapter's input is a [P][K] (sorted).  du [P][rank] and us [P][rank]
// fp32 and bt [E][rank][N] BF16 are scratch.  dx [P][K] BF16 (the adapter's
// share of the input gradient), dA [E][rank][K], dB [E][N][rank] fp32, each
// nullable.
hipError_t launch_lora_bwd_gated(const uint16_t* a, int K, int N, int E, const int32_t* perm,
                                 int topk, const float* gates, const int32_t* offsets,
                                 const int4* tiles, const int32_t* ntiles, int max_tiles, int MB,
                                 const uint16_t* A, const uint16_t* B, int rank, float alpha,
                                 const uint16_t* dy, const uint16_t* u, uint16_t* bt, float* du,
                                 float* us, uint16_t* dx, float* dA, float* dB, int64_t P,
                                 hipStream_t s);

int num_cus();

// Measurement hook (qgg_set_timing_events): while the calling thread has
// events registered, each library launch function brackets its kernels with
// a pair of them on its stream.  Scopes nest; only the outermost records.
enum LaunchKind {
  kLRoute = 1, kLPermute = 2, kLGemm = 3, kLGemmT = 4, kLDequant = 5, kLCombine = 6,
  kLLora = 7, kLRouterBwd = 8, kLOther = 9
};
void timing_begin(int kind, hipStream_t s);
void timing_end(hipStream_t s);
struct TimedLaunch {
  hipStream_t s;
  TimedLaunch(int kind, hipStream_t st) : s(st) { timing_begin(kind, s); }
  ~TimedLaunch() { timing_end(s); }
  TimedLaunch(const TimedLaunch&) = delete;
  TimedLaunch& operator=(const TimedLaunch&) = delete;
};

}  // namespace qgg
