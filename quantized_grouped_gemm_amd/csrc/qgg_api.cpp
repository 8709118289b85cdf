// C-ABI entry points: argument validation, workspace layout, chunk loop and
// kernel orchestration.  No device allocation happens here: every buffer is
// the caller's.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>

#include "qgg.h"
#include "qgg_internal.hpp"

namespace qgg {

int num_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxLoraRank = 128;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Bump allocator over the caller's workspace.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <class T>
  T* take(size_t bytes) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += align_up(bytes);
    return p;
  }
};

// Rows per M-tile, from the mean rows per expert (P / E) rounded up to a
// power-of-two number of 32-row MFMA blocks, at most 4.
// Tile height in 32-row blocks.  Top-k routing gives an expert at most one
// row per token, so a batch of T <= 64 tokens fits every expert in one tile of
// ceil(T / 32) blocks and each expert streams its weights once; larger batches
// take the height from the mean rows per expert.
int choose_mb(int64_t P, int E, int64_t T) {
  if (T <= 64) return T <= 32 ? 1 : 2;
  const int64_t mean = E > 0 ? (P + E - 1) / E : P;
  const int64_t blocks = (mean + 31) / 32;
  if (blocks <= 1) return 1;
  if (blocks <= 2) return 2;
  return 4;
}

int64_t tile_capacity(int64_t P, int E, int MT) { return (P + MT - 1) / MT + E + 1; }

struct Plan {
  int4* tiles = nullptr;
  int32_t* chunk_first = nullptr;
  int32_t* work = nullptr;   // the GEMM launches' item and exit counters
  int mb = 1;
  int64_t cap = 0;
};

void carve_plan(Carver& cv, int64_t P, int E, int64_t T, Plan& pl) {
  pl.mb = choose_mb(P, E, T);
  pl.cap = tile_capacity(P, E, 32 * pl.mb);
  pl.tiles = cv.take<int4>(sizeof(int4) * pl.cap);
  // chunk bounds (E + 2 entries), then the GEMM launches' work counters (2)
  pl.chunk_first = cv.take<int32_t>(sizeof(int32_t) * (E + 4));
  pl.work = pl.chunk_first ? pl.chunk_first + E + 2 : nullptr;
}

bool valid_fmt(int f) { return f == QGG_FMT_MXFP4 || f == QGG_FMT_INT4; }

bool valid_layout(int l) { return l == QGG_LAYOUT_ROWS || l == QGG_LAYOUT_MFMA; }

bool valid_weight(const qgg_qweight* w, int E, int N, int K) {
  return w && valid_fmt(w->fmt) && valid_layout(w->layout) && w->E == E && w->N == N &&
         w->K == K && w->packed && w->scales;
}

// perm and inv_perm hold one entry per routed pair, so an empty batch may
// pass them as NULL
bool valid_perm(const qgg_perm* p, int64_t P) {
  return p && p->counts && p->offsets && p->active && p->n_active &&
         (P == 0 || (p->perm && p->inv_perm));
}

bool valid_route_dims(int T, int E, int k) {
  return T >= 0 && E >= 1 && E <= 1024 && k >= 1 && k <= 32 && k <= E &&
         (int64_t)T * k < (int64_t)1 << 31;
}

// The GEMM kernels address each A operand (activations, intermediates)
// through a 32-bit buffer offset.
bool a_fits(int64_t rows, int64_t ld) { return rows * ld * 2 <= (int64_t)0xFFFFFFFF; }

PermPtrs to_ptrs(const qgg_perm* p) {
  return PermPtrs{p->counts, p->offsets, p->perm, p->inv_perm, p->active, p->n_active};
}

#define QGG_HIP(expr)                          \
  do {                                         \
    if ((expr) != hipSuccess) return QGG_ERR_HIP; \
  } while (0)

int src_of(int fmt) { return fmt == QGG_FMT_MXFP4 ? kSrcMXFP4 : kSrcINT4; }

GemmArgs base_args(const qgg_qweight* w, const Plan& pl) {
  GemmArgs g;
  std::memset(&g, 0, sizeof g);
  g.src = src_of(w->fmt);
  g.packed = w->packed;
  g.scales = w->scales;
  g.layout = w->layout;
  g.N = w->N;
  g.K = w->K;
  g.tiles = pl.tiles;
  g.range = pl.chunk_first;
  g.work = pl.work;
  g.max_tiles = (int)pl.cap;
  g.mt_rows = 32 * pl.mb;
  return g;
}

// Chunk iterations of a CHUNKED call: enough for every expert that can be
// active (at most min(E, P)); chunks past the live ones are empty on the
// device and their launches return at once, so no count is read back.
int chunk_iterations(int E, int64_t P, int C) {
  const int64_t most = std::min<int64_t>(E, P);
  return (int)((most + C - 1) / C);
}

}  // namespace
}  // namespace qgg

// Library-owned scratch of the allocation-free entry point: one copy per GPU,
// held until the process ends.  Host code reaches it only through the device
// address hipGetSymbolAddress returns (the array's name is a host-side stand-in
// in host code).
static __device__ __align__(256) uint8_t scratch[QGG_STATIC_SCRATCH_BYTES];

namespace qgg {
namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of `scratch` on the current device, looked up once per device
// (with that device current) and kept.
hipError_t static_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
  });
  *out = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

}  // namespace
}  // namespace qgg

using namespace qgg;

extern "C" {

const char* qgg_status_string(qgg_status s) {
  switch (s) {
    case QGG_OK: return "ok";
    case QGG_ERR_INVALID_ARG: return "invalid argument";
    case QGG_ERR_UNSUPPORTED: return "unsupported shape or option";
    case QGG_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case QGG_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* qgg_version(void) { return "qgg 0.2 gfx950"; }

qgg_status qgg_repack_weights(const qgg_qweight* src, uint8_t* packed_out, void* scales_out,
                              qgg_stream_t stream) {
  if (!src || !valid_fmt(src->fmt) || src->layout != QGG_LAYOUT_ROWS || !src->packed ||
      !src->scales || !packed_out || !scales_out || src->E <= 0 || src->N <= 0 || src->K <= 0)
    return QGG_ERR_INVALID_ARG;
  if (src->N % 32 || src->K % 64) return QGG_ERR_UNSUPPORTED;
  if (static_cast<const void*>(packed_out) == static_cast<const void*>(src->packed) ||
      scales_out == src->scales)
    return QGG_ERR_INVALID_ARG;
  QGG_HIP(launch_repack(src->fmt, src->packed, src->scales, src->E, src->N, src->K, packed_out,
                        scales_out, stream));
  return QGG_OK;
}

qgg_status qgg_check_weights(const qgg_qweight* w, int32_t* err_flag, qgg_stream_t stream) {
  if (!w || !valid_fmt(w->fmt) || !valid_layout(w->layout) || !w->scales || !err_flag ||
      w->E <= 0 || w->N <= 0 || w->K <= 0 || w->K % 32)
    return QGG_ERR_INVALID_ARG;
  const int64_t n = (int64_t)w->E * w->N * (w->K / 32);
  QGG_HIP(launch_check_scales(w->fmt, w->scales, n, err_flag, stream));
  return QGG_OK;
}

// Workspace layout per call (each piece 256-byte aligned, in this order):
//  PERMUTE  segment counts
//  GEMM     plan (tiles, chunk table) | BF16 chunk scratch (CHUNKED)
//  FFN_FWD  segment counts | plan | a [P][inter] | o [P][d] | scratch
//  DX_BWD   plan | dH [P][2*inter] | dXp [P][d] | scratch | gate partials [P][inter/256] fp32
//  LORA_BWD plan | du [P][rank] fp32 | B transposed [E][rank][N] BF16
//  FFN_LORA_BWD  DX_BWD's pieces | a [P][inter] | down adapter's dA share
//           [P][inter] | gate_up adapter's dXp share [P][d] | du, us [P][128] fp32
//           | B transposed [E][128][max(d, 2 inter)] BF16
size_t qgg_workspace_bytes(int call, int T, int d, int E, int k, int N_or_inter, int variant,
                           int chunk, size_t* scratch_bytes) {
  if (scratch_bytes) *scratch_bytes = 0;
  if (!valid_route_dims(T, E, k) || d <= 0 || N_or_inter <= 0 || chunk < 0) return 0;
  const int64_t P = (int64_t)T * k;
  const int64_t C = chunk > 0 ? std::min<int64_t>(chunk, E) : std::min<int64_t>(E, std::max<int64_t>(P, 1));
  Carver cv(nullptr);
  Plan pl;
  size_t scratch = 0;
  switch (call) {
    case QGG_CALL_PERMUTE:
      cv.take<char>(permute_ws_bytes(P, E));
      break;
    case QGG_CALL_GEMM:
      carve_plan(cv, P, E, T, pl);
      if (variant == QGG_CHUNKED) scratch = (size_t)C * N_or_inter * d * 2;
      cv.take<char>(scratch);
      break;
    case QGG_CALL_FFN_FWD: {
      const int64_t I = N_or_inter;
      cv.take<char>(permute_ws_bytes(P, E));
      carve_plan(cv, P, E, T, pl);
      cv.take<char>((size_t)P * I * 2);
      cv.take<char>((size_t)P * d * 2);
      if (variant == QGG_CHUNKED) scratch = (size_t)C * 2 * I * d * 2;
      cv.take<char>(scratch);
      break;
    }
    case QGG_CALL_LORA_BWD:   // d = N (dY width), N_or_inter = adapter rank
      carve_plan(cv, P, E, T, pl);
      cv.take<char>((size_t)P * N_or_inter * 4);
      cv.take<char>((size_t)E * N_or_inter * d * 2);
      break;
    case QGG_CALL_DX_BWD:
    case QGG_CALL_FFN_LORA_BWD: {
      const int64_t I = N_or_inter;
      carve_plan(cv, P, E, T, pl);
      cv.take<char>((size_t)P * 2 * I * 2);
      cv.take<char>((size_t)P * d * 2);
      if (variant == QGG_CHUNKED) scratch = (size_t)C * 2 * I * d * 2;
      cv.take<char>(scratch);
      cv.take<char>((size_t)P * (I / 256 > 0 ? I / 256 : 1) * 4);
      if (call == QGG_CALL_FFN_LORA_BWD) {
        cv.take<char>((size_t)P * I * 2);
        cv.take<char>((size_t)P * I * 2);
        cv.take<char>((size_t)P * d * 2);
        cv.take<char>((size_t)P * kMaxLoraRank * 4);
        cv.take<char>((size_t)P * kMaxLoraRank * 4);
        cv.take<char>((size_t)E * kMaxLoraRank * std::max<int64_t>(d, 2 * I) * 2);
      }
      break;
    }
    default:
      return 0;
  }
  if (scratch_bytes) *scratch_bytes = scratch;
  return std::max<size_t>(cv.off, kAlign);
}

qgg_status moe_route(const float* logits, int T, int E, int k, int32_t* topk_ids,
                     float* topk_gates, int32_t* err_flag, qgg_stream_t stream) {
  if (!valid_route_dims(T, E, k)) return QGG_ERR_INVALID_ARG;
  if (T > 0 && (!logits || !topk_ids || !topk_gates)) return QGG_ERR_INVALID_ARG;
  QGG_HIP(launch_route(logits, T, E, k, topk_ids, topk_gates, err_flag, stream));
  return QGG_OK;
}

qgg_status expert_permute(const int32_t* topk_ids, int T, int k, int E, const qgg_perm* p,
                          const uint16_t* x, int d, uint16_t* x_perm, int32_t* err_flag,
                          void* workspace, size_t ws_bytes, qgg_stream_t stream) {
  if (!valid_route_dims(T, E, k) || !valid_perm(p, (int64_t)T * k)) return QGG_ERR_INVALID_ARG;
  if (T > 0 && !topk_ids) return QGG_ERR_INVALID_ARG;
  const bool gather = x != nullptr && x_perm != nullptr;
  if (gather && (d <= 0 || d % 8)) return QGG_ERR_INVALID_ARG;
  const int64_t P = (int64_t)T * k;
  const size_t need = qgg_workspace_bytes(QGG_CALL_PERMUTE, T, 8, E, k, 1, QGG_FUSED, 0, nullptr);
  if (!workspace || ws_bytes < need) return QGG_ERR_WORKSPACE_TOO_SMALL;
  const PermPtrs pp = to_ptrs(p);
  QGG_HIP(launch_permute(topk_ids, P, E, pp, err_flag, workspace, stream));
  if (gather) QGG_HIP(launch_gather(x, d, pp, E, k, P, x_perm, stream));
  return QGG_OK;
}

// Shared body of dequant_grouped_gemm and lora_grouped_gemm (lora may be null).
static qgg_status grouped_gemm(const qgg_qweight* w, const qgg_lora* lora, const uint16_t* a,
                               int flags, const qgg_perm* p, int T, int k, int variant, int chunk,
                               void* workspace, size_t ws_bytes, uint16_t* u_out, uint16_t* y,
                               qgg_stream_t stream) {
  if (!w || !valid_perm(p, (int64_t)T * k) || !valid_fmt(w->fmt) || !valid_layout(w->layout))
    return QGG_ERR_INVALID_ARG;
  const int E = w->E, N = w->N, K = w->K;
  if (!valid_route_dims(T, E, k) || N <= 0 || K <= 0 || chunk < 0) return QGG_ERR_INVALID_ARG;
  if (!w->packed || !w->scales) return QGG_ERR_INVALID_ARG;
  if (variant != QGG_CHUNKED && variant != QGG_FUSED) return QGG_ERR_INVALID_ARG;
  if (flags & ~(QGG_A_TOKENS | QGG_TRANSPOSE_W | QGG_DEQUANT_ONLY)) return QGG_ERR_INVALID_ARG;
  if (K % 128 || N % 64) return QGG_ERR_UNSUPPORTED;
  const bool trans = flags & QGG_TRANSPOSE_W;
  const bool dq_only = flags & QGG_DEQUANT_ONLY;
  if (dq_only && variant != QGG_CHUNKED) return QGG_ERR_INVALID_ARG;
  if (!dq_only && (!a || !y) && T > 0) return QGG_ERR_INVALID_ARG;
  const int64_t P = (int64_t)T * k;
  if (!a_fits((flags & QGG_A_TOKENS) ? T : P, trans ? N : K)) return QGG_ERR_UNSUPPORTED;
  size_t scratch = 0;
  const size_t need = qgg_workspace_bytes(QGG_CALL_GEMM, T, K, E, k, N, variant, chunk, &scratch);
  if (!workspace || ws_bytes < need) return QGG_ERR_WORKSPACE_TOO_SMALL;
  const int C = chunk > 0 ? std::min(chunk, E) : (int)std::min<int64_t>(E, std::max<int64_t>(P, 1));
  Carver cv(workspace);
  Plan pl;
  carve_plan(cv, P, E, T, pl);
  uint16_t* sbuf = cv.take<uint16_t>(scratch);

  if (dq_only) {
    QGG_HIP(launch_dequant(w->fmt, w->packed, w->scales, w->layout, N, K, p->active, p->n_active,
                           0, C, false, static_cast<uint16_t*>(workspace), stream));
    return QGG_OK;
  }
  if (P == 0) return QGG_OK;
  const PermPtrs pp = to_ptrs(p);
  QGG_HIP(launch_tile_plan(pp, E, 32 * pl.mb, variant == QGG_CHUNKED ? C : 0, pl.tiles,
                           pl.chunk_first, stream));
  GemmArgs g = base_args(w, pl);
  g.a = a;
  g.lda = trans ? N : K;
  g.amode = (flags & QGG_A_TOKENS) ? kATokens : kASorted;
  g.a_rows = g.amode == kATokens ? T : P;
  g.perm = p->perm;
  g.topk = k;
  g.y = y;
  g.ldy = trans ? K : N;
  g.epi = kEpiStore;
  if (lora) {
    QGG_HIP(launch_lora_u(a, K, p->perm, k, g.amode, pl.tiles, pl.chunk_first + E + 1,
                          (int)pl.cap, pl.mb, lora->A, lora->rank, lora->alpha, u_out, stream));
    g.lora_rank = lora->rank;
    g.lora_u = u_out;
    g.lora_b = lora->B;
  }
  if (variant == QGG_FUSED) {
    QGG_HIP(trans ? launch_gemm_tn(g, pl.mb, stream) : launch_gemm_nt(g, pl.mb, stream));
    return QGG_OK;
  }
  const int nch = chunk_iterations(E, P, C);
  g.src = kSrcBF16;
  g.wbf16 = sbuf;
  for (int c = 0; c < nch; ++c) {
    QGG_HIP(launch_dequant(w->fmt, w->packed, w->scales, w->layout, N, K, p->active,
                           p->n_active, c * C, C, true, sbuf, stream));
    g.range = pl.chunk_first + c;
    g.max_tiles = (int)pl.cap;
    g.bf16_slot_base = c * C;
    QGG_HIP(trans ? launch_gemm_tn(g, pl.mb, stream) : launch_gemm_nt(g, pl.mb, stream));
  }
  return QGG_OK;
}

qgg_status dequant_grouped_gemm(const qgg_qweight* w, const uint16_t* a, int flags,
                                const qgg_perm* p, int T, int k, int variant, int chunk,
                                void* workspace, size_t ws_bytes, uint16_t* y,
                                qgg_stream_t stream) {
  return grouped_gemm(w, nullptr, a, flags, p, T, k, variant, chunk, workspace, ws_bytes, nullptr,
                      y, stream);
}

qgg_status lora_grouped_gemm(const qgg_qweight* w, const qgg_lora* lora, const uint16_t* a,
                             int flags, const qgg_perm* p, int T, int k, int variant, int chunk,
                             void* workspace, size_t ws_bytes, uint16_t* u_out, uint16_t* y,
                             qgg_stream_t stream) {
  if (!lora || !w) return QGG_ERR_INVALID_ARG;
  if (lora->rank < 16 || lora->rank > 128 || lora->rank % 16) return QGG_ERR_UNSUPPORTED;
  if (!std::isfinite(lora->alpha)) return QGG_ERR_INVALID_ARG;
  if (flags & (QGG_TRANSPOSE_W | QGG_DEQUANT_ONLY)) return QGG_ERR_INVALID_ARG;
  if (T > 0 && (!lora->A || !lora->B || !u_out)) return QGG_ERR_INVALID_ARG;
  return grouped_gemm(w, lora, a, flags, p, T, k, variant, chunk, workspace, ws_bytes, u_out, y,
                      stream);
}

qgg_status lora_grouped_gemm_bwd(const qgg_lora* lora, int E, int N, int K, const uint16_t* a,
                                 int flags, const uint16_t* dy, const uint16_t* u,
                                 const qgg_perm* p, int T, int k, void* workspace,
                                 size_t ws_bytes, uint16_t* dx, float* dA, float* dB,
                                 qgg_stream_t stream) {
  if (!lora || !valid_perm(p, (int64_t)T * k) || !valid_route_dims(T, E, k) || N <= 0 || K <= 0)
    return QGG_ERR_INVALID_ARG;
  if (lora->rank < 16 || lora->rank > 128 || lora->rank % 16) return QGG_ERR_UNSUPPORTED;
  if (!std::isfinite(lora->alpha)) return QGG_ERR_INVALID_ARG;
  if (flags & ~QGG_A_TOKENS) return QGG_ERR_INVALID_ARG;
  if (K % 128 || N % 64) return QGG_ERR_UNSUPPORTED;
  if (!dx && !dA && !dB) return QGG_ERR_INVALID_ARG;
  if (!lora->A || !lora->B) return QGG_ERR_INVALID_ARG;
  if (T > 0 && (!dy || (dB && !u) || (dA && !a))) return QGG_ERR_INVALID_ARG;
  const int64_t P = (int64_t)T * k;
  const size_t need =
      qgg_workspace_bytes(QGG_CALL_LORA_BWD, T, N, E, k, lora->rank, QGG_FUSED, 0, nullptr);
  if (!workspace || ws_bytes < need) return QGG_ERR_WORKSPACE_TOO_SMALL;
  Carver cv(workspace);
  Plan pl;
  carve_plan(cv, P, E, T, pl);
  float* du = cv.take<float>((size_t)P * lora->rank * 4);
  uint16_t* bt = cv.take<uint16_t>((size_t)E * lora->rank * N * 2);
  const PermPtrs pp = to_ptrs(p);
  if (P > 0)
    QGG_HIP(launch_tile_plan(pp, E, 32 * pl.mb, 0, pl.tiles, pl.chunk_first, stream));
  // with no routed rows every adapter gradient is zero: the kernels still
  // run (empty row ranges) so dA and dB are written in full
  QGG_HIP(launch_lora_bwd(a, K, N, E, p->perm, k, (flags & QGG_A_TOKENS) ? kATokens : kASorted,
                          p->offsets, pl.tiles, pl.chunk_first + E + 1, P > 0 ? (int)pl.cap : 0,
                          pl.mb, lora->A, lora->B, lora->rank, lora->alpha, dy, u, bt, du, dx, dA,
                          dB, stream));
  return QGG_OK;
}

// Shared body of moe_ffn_fwd and moe_ffn_fwd_lora (adapters nullable).
static qgg_status ffn_forward(const qgg_qweight* w_gate_up, const qgg_qweight* w_down,
                              const qgg_lora* lgu, const qgg_lora* ldn, const uint16_t* x,
                              const float* logits, int T, int d, int E, int k, int inter,
                              int variant, int chunk, int32_t* topk_ids, float* topk_gates,
                              const qgg_perm* p, uint16_t* h_save, uint16_t* u_gu, uint16_t* u_dn,
                              int32_t* err_flag, void* workspace, size_t ws_bytes, uint16_t* y,
                              qgg_stream_t stream) {
  if (!valid_route_dims(T, E, k) || d <= 0 || inter <= 0 || chunk < 0) return QGG_ERR_INVALID_ARG;
  if (!valid_weight(w_gate_up, E, 2 * inter, d) || !valid_weight(w_down, E, d, inter))
    return QGG_ERR_INVALID_ARG;
  if (w_gate_up->fmt != w_down->fmt) return QGG_ERR_INVALID_ARG;
  if (variant != QGG_CHUNKED && variant != QGG_FUSED) return QGG_ERR_INVALID_ARG;
  if (!valid_perm(p, (int64_t)T * k)) return QGG_ERR_INVALID_ARG;
  if (T > 0 && (!x || !logits || !topk_ids || !topk_gates || !y)) return QGG_ERR_INVALID_ARG;
  if (d % 128 || inter % 128) return QGG_ERR_UNSUPPORTED;
  const int64_t P = (int64_t)T * k;
  if (!a_fits(T, d) || !a_fits(P, inter)) return QGG_ERR_UNSUPPORTED;
  size_t scratch = 0;
  const size_t need =
      qgg_workspace_bytes(QGG_CALL_FFN_FWD, T, d, E, k, inter, variant, chunk, &scratch);
  if (!workspace || ws_bytes < need) return QGG_ERR_WORKSPACE_TOO_SMALL;
  const int C = chunk > 0 ? std::min(chunk, E) : (int)std::min<int64_t>(E, std::max<int64_t>(P, 1));
  Carver cv(workspace);
  void* pws = cv.take<char>(permute_ws_bytes(P, E));
  Plan pl;
  carve_plan(cv, P, E, T, pl);
  uint16_t* abuf = cv.take<uint16_t>((size_t)P * inter * 2);
  uint16_t* obuf = cv.take<uint16_t>((size_t)P * d * 2);
  uint16_t* sbuf = cv.take<uint16_t>(scratch);
  const PermPtrs pp = to_ptrs(p);

  QGG_HIP(launch_route(logits, T, E, k, topk_ids, topk_gates, err_flag, stream));
  if (P == 0) {
    QGG_HIP(launch_permute(topk_ids, P, E, pp, err_flag, pws, stream));
    return QGG_OK;
  }
  QGG_HIP(launch_permute_plan(topk_ids, P, E, pp, err_flag, pws, 32 * pl.mb,
                              variant == QGG_CHUNKED ? C : 0, pl.tiles, pl.chunk_first, stream));
  const int32_t* ntiles = pl.chunk_first + E + 1;

  GemmArgs gu = base_args(w_gate_up, pl);
  gu.a = x;
  gu.lda = d;
  gu.a_rows = T;
  gu.amode = kATokens;
  gu.perm = p->perm;
  gu.topk = k;
  gu.y = abuf;
  gu.ldy = inter;
  gu.epi = kEpiSwiGLU;
  gu.inter = inter;
  gu.h = h_save;
  GemmArgs dn = base_args(w_down, pl);
  dn.a = abuf;
  dn.lda = inter;
  dn.a_rows = P;
  dn.amode = kASorted;
  dn.perm = p->perm;
  dn.topk = k;
  dn.y = obuf;
  dn.ldy = d;
  dn.epi = kEpiStore;

  // adapter up projections ride on the GEMMs' accumulators; u of the down
  // adapter needs the whole SwiGLU output first
  if (lgu) {
    QGG_HIP(launch_lora_u(x, d, p->perm, k, kATokens, pl.tiles, ntiles, (int)pl.cap, pl.mb,
                          lgu->A, lgu->rank, lgu->alpha, u_gu, stream));
    gu.lora_rank = lgu->rank;
    gu.lora_u = u_gu;
    gu.lora_b = lgu->B;
  }
  if (ldn) {
    dn.lora_rank = ldn->rank;
    dn.lora_u = u_dn;
    dn.lora_b = ldn->B;
  }
  auto down_u = [&]() {
    return launch_lora_u(abuf, inter, p->perm, k, kASorted, pl.tiles, ntiles, (int)pl.cap,
                         pl.mb, ldn->A, ldn->rank, ldn->alpha, u_dn, stream);
  };
  if (variant == QGG_FUSED) {
    QGG_HIP(launch_gemm_nt(gu, pl.mb, stream));
    if (ldn) QGG_HIP(down_u());
    QGG_HIP(launch_gemm_nt(dn, pl.mb, stream));
  } else if (ldn) {
    // every chunk's gate_up first (the down adapter's u reads all of a),
    // then every chunk's down projection, through the same one-chunk scratch
    const int nch = chunk_iterations(E, P, C);
    gu.src = dn.src = kSrcBF16;
    gu.wbf16 = dn.wbf16 = sbuf;
    gu.max_tiles = dn.max_tiles = (int)pl.cap;
    for (int c = 0; c < nch; ++c) {
      gu.range = pl.chunk_first + c;
      gu.bf16_slot_base = c * C;
      QGG_HIP(launch_dequant(w_gate_up->fmt, w_gate_up->packed, w_gate_up->scales,
                             w_gate_up->layout, 2 * inter, d, p->active, p->n_active, c * C, C,
                             true, sbuf, stream));
      QGG_HIP(launch_gemm_nt(gu, pl.mb, stream));
    }
    QGG_HIP(down_u());
    for (int c = 0; c < nch; ++c) {
      dn.range = pl.chunk_first + c;
      dn.bf16_slot_base = c * C;
      QGG_HIP(launch_dequant(w_down->fmt, w_down->packed, w_down->scales, w_down->layout, d,
                             inter, p->active, p->n_active, c * C, C, true, sbuf, stream));
      QGG_HIP(launch_gemm_nt(dn, pl.mb, stream));
    }
  } else {
    const int nch = chunk_iterations(E, P, C);
    gu.src = dn.src = kSrcBF16;
    gu.wbf16 = dn.wbf16 = sbuf;
    for (int c = 0; c < nch; ++c) {
      gu.range = dn.range = pl.chunk_first + c;
      gu.max_tiles = dn.max_tiles = (int)pl.cap;
      gu.bf16_slot_base = dn.bf16_slot_base = c * C;
      QGG_HIP(launch_dequant(w_gate_up->fmt, w_gate_up->packed, w_gate_up->scales,
                             w_gate_up->layout, 2 * inter, d, p->active, p->n_active, c * C, C,
                             true, sbuf, stream));
      QGG_HIP(launch_gemm_nt(gu, pl.mb, stream));
      QGG_HIP(launch_dequant(w_down->fmt, w_down->packed, w_down->scales, w_down->layout, d,
                             inter, p->active, p->n_active, c * C, C, true, sbuf, stream));
      QGG_HIP(launch_gemm_nt(dn, pl.mb, stream));
    }
  }
  QGG_HIP(launch_combine(obuf, d, p->inv_perm, topk_gates, T, k, y, stream));
  return QGG_OK;
}

qgg_status moe_ffn_fwd(const qgg_qweight* w_gate_up, const qgg_qweight* w_down,
                       const uint16_t* x, const float* logits, int T, int d, int E, int k,
                       int inter, int variant, int chunk, int32_t* topk_ids, float* topk_gates,
                       const qgg_perm* p, uint16_t* h_save, int32_t* err_flag, void* workspace,
                       size_t ws_bytes, uint16_t* y, qgg_stream_t stream) {
  return ffn_forward(w_gate_up, w_down, nullptr, nullptr, x, logits, T, d, E, k, inter, variant,
                     chunk, topk_ids, topk_gates, p, h_save, nullptr, nullptr, err_flag,
                     workspace, ws_bytes, y, stream);
}

qgg_status moe_ffn_fwd_noalloc(const qgg_qweight* w_gate_up, const qgg_qweight* w_down,
                               const uint16_t* x, const float* logits, int T, int d, int E, int k,
                               int inter, int variant, int chunk, int32_t* topk_ids,
                               float* topk_gates, const qgg_perm* p, uint16_t* h_save,
                               int32_t* err_flag, uint16_t* y, qgg_stream_t stream) {
  if (!valid_route_dims(T, E, k) || d <= 0 || inter <= 0 || chunk < 0) return QGG_ERR_INVALID_ARG;
  if (variant != QGG_CHUNKED && variant != QGG_FUSED) return QGG_ERR_INVALID_ARG;
  const size_t need =
      qgg_workspace_bytes(QGG_CALL_FFN_FWD, T, d, E, k, inter, variant, chunk, nullptr);
  if (need == 0) return QGG_ERR_INVALID_ARG;
  if (need > QGG_STATIC_SCRATCH_BYTES) return QGG_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  if (static_scratch(&ws) != hipSuccess || !ws) return QGG_ERR_HIP;
  return ffn_forward(w_gate_up, w_down, nullptr, nullptr, x, logits, T, d, E, k, inter, variant,
                     chunk, topk_ids, topk_gates, p, h_save, nullptr, nullptr, err_flag, ws,
                     QGG_STATIC_SCRATCH_BYTES, y, stream);
}

static bool valid_lora_rank(const qgg_lora* l) {
  return !l || (l->rank >= 16 && l->rank <= 128 && l->rank % 16 == 0);
}

qgg_status moe_ffn_fwd_lora(const qgg_qweight* w_gate_up, const qgg_qweight* w_down,
                            const qgg_lora* lora_gate_up, const qgg_lora* lora_down,
                            const uint16_t* x, const float* logits, int T, int d, int E, int k,
                            int inter, int variant, int chunk, int32_t* topk_ids,
                            float* topk_gates, const qgg_perm* p, uint16_t* h_save,
                            uint16_t* u_gate_up, uint16_t* u_down, int32_t* err_flag,
                            void* workspace, size_t ws_bytes, uint16_t* y, qgg_stream_t stream) {
  if (!lora_gate_up && !lora_down) return QGG_ERR_INVALID_ARG;
  if (!valid_lora_rank(lora_gate_up) || !valid_lora_rank(lora_down)) return QGG_ERR_UNSUPPORTED;
  if ((lora_gate_up && !std::isfinite(lora_gate_up->alpha)) ||
      (lora_down && !std::isfinite(lora_down->alpha)))
    return QGG_ERR_INVALID_ARG;
  if (T > 0 && lora_gate_up && (!lora_gate_up->A || !lora_gate_up->B || !u_gate_up))
    return QGG_ERR_INVALID_ARG;
  if (T > 0 && lora_down && (!lora_down->A || !lora_down->B || !u_down))
    return QGG_ERR_INVALID_ARG;
  return ffn_forward(w_gate_up, w_down, lora_gate_up, lora_down, x, logits, T, d, E, k, inter,
                     variant, chunk, topk_ids, topk_gates, p, h_save, u_gate_up, u_down,
                     err_flag, workspace, ws_bytes, y, stream);
}

// Shared body of moe_dx_bwd and moe_router_bwd.  dx == nullptr skips the
// gate_up backward GEMM and the scatter-sum; dgates / dlogits != nullptr add
// the router gradient (partials from the SwiGLU-backward epilogue, then one
// small kernel).
static qgg_status backward(const qgg_qweight* w_gate_up, const qgg_qweight* w_down,
                           const uint16_t* dy, const int32_t* topk_ids, const float* topk_gates,
                           const qgg_perm* p, const uint16_t* h_saved, int T, int d, int E,
                           int k, int inter, int variant, int chunk, void* workspace,
                           size_t ws_bytes, uint16_t* dx, float* dgates, float* dlogits,
                           qgg_stream_t stream) {
  if (!valid_route_dims(T, E, k) || d <= 0 || inter <= 0 || chunk < 0) return QGG_ERR_INVALID_ARG;
  if (!valid_weight(w_gate_up, E, 2 * inter, d) || !valid_weight(w_down, E, d, inter))
    return QGG_ERR_INVALID_ARG;
  if (w_gate_up->fmt != w_down->fmt) return QGG_ERR_INVALID_ARG;
  if (variant != QGG_CHUNKED && variant != QGG_FUSED) return QGG_ERR_INVALID_ARG;
  if (!valid_perm(p, (int64_t)T * k)) return QGG_ERR_INVALID_ARG;
  const bool router = dgates != nullptr || dlogits != nullptr;
  if (T > 0 && (!dy || !topk_gates || !h_saved)) return QGG_ERR_INVALID_ARG;
  if (T > 0 && !dx && !router) return QGG_ERR_INVALID_ARG;
  if (T > 0 && dlogits && !topk_ids) return QGG_ERR_INVALID_ARG;
  if (d % 256 || inter % 256) return QGG_ERR_UNSUPPORTED;
  const int64_t P = (int64_t)T * k;
  if (!a_fits(T, d) || !a_fits(P, 2 * inter)) return QGG_ERR_UNSUPPORTED;
  size_t scratch = 0;
  const size_t need =
      qgg_workspace_bytes(QGG_CALL_DX_BWD, T, d, E, k, inter, variant, chunk, &scratch);
  if (!workspace || ws_bytes < need) return QGG_ERR_WORKSPACE_TOO_SMALL;
  if (P == 0) return QGG_OK;
  const int C = chunk > 0 ? std::min(chunk, E) : (int)std::min<int64_t>(E, std::max<int64_t>(P, 1));
  Carver cv(workspace);
  Plan pl;
  carve_plan(cv, P, E, T, pl);
  uint16_t* dh = cv.take<uint16_t>((size_t)P * 2 * inter * 2);
  uint16_t* dxp = cv.take<uint16_t>((size_t)P * d * 2);
  uint16_t* sbuf = cv.take<uint16_t>(scratch);
  float* gpart = cv.take<float>((size_t)P * (inter / 256) * 4);
  const PermPtrs pp = to_ptrs(p);
  QGG_HIP(launch_tile_plan(pp, E, 32 * pl.mb, variant == QGG_CHUNKED ? C : 0, pl.tiles,
                           pl.chunk_first, stream));

  // dA = (g dY) . W_down, then dH from the SwiGLU derivative (fused epilogue)
  GemmArgs dn = base_args(w_down, pl);
  dn.a = dy;
  dn.lda = d;
  dn.a_rows = T;
  dn.amode = kATokens;
  dn.perm = p->perm;
  dn.topk = k;
  dn.y = dh;
  dn.ldy = 2 * inter;
  dn.epi = kEpiSwiGLUBwd;
  dn.inter = inter;
  dn.h = const_cast<uint16_t*>(h_saved);
  dn.gates = topk_gates;
  dn.gpart = router ? gpart : nullptr;
  // dXp = dH . W_gate_up
  GemmArgs gu = base_args(w_gate_up, pl);
  gu.a = dh;
  gu.lda = 2 * inter;
  gu.a_rows = P;
  gu.amode = kASorted;
  gu.perm = p->perm;
  gu.topk = k;
  gu.y = dxp;
  gu.ldy = d;
  gu.epi = kEpiStore;

  if (variant == QGG_FUSED) {
    QGG_HIP(launch_gemm_tn(dn, pl.mb, stream));
    if (dx) QGG_HIP(launch_gemm_tn(gu, pl.mb, stream));
  } else {
    const int nch = chunk_iterations(E, P, C);
    dn.src = gu.src = kSrcBF16;
    dn.wbf16 = gu.wbf16 = sbuf;
    for (int c = 0; c < nch; ++c) {
      dn.range = gu.range = pl.chunk_first + c;
      dn.max_tiles = gu.max_tiles = (int)pl.cap;
      dn.bf16_slot_base = gu.bf16_slot_base = c * C;
      QGG_HIP(launch_dequant(w_down->fmt, w_down->packed, w_down->scales, w_down->layout, d,
                             inter, p->active, p->n_active, c * C, C, true, sbuf, stream));
      QGG_HIP(launch_gemm_tn(dn, pl.mb, stream));
      if (!dx) continue;
      QGG_HIP(launch_dequant(w_gate_up->fmt, w_gate_up->packed, w_gate_up->scales,
                             w_gate_up->layout, 2 * inter, d, p->active, p->n_active, c * C, C,
                             true, sbuf, stream));
      QGG_HIP(launch_gemm_tn(gu, pl.mb, stream));
    }
  }
  if (dx) QGG_HIP(launch_combine(dxp, d, p->inv_perm, nullptr, T, k, dx, stream));
  if (router)
    QGG_HIP(launch_router_bwd(gpart, inter / 256, p->inv_perm, topk_ids, topk_gates, T, E, k,
                              dgates, dlogits, stream));
  return QGG_OK;
}

qgg_status moe_dx_bwd(const qgg_qweight* w_gate_up, const qgg_qweight* w_down,
                      const uint16_t* dy, const float* topk_gates, const qgg_perm* p,
                      const uint16_t* h_saved, int T, int d, int E, int k, int inter, int variant,
                      int chunk, void* workspace, size_t ws_bytes, uint16_t* dx,
                      qgg_stream_t stream) {
  if (T > 0 && !dx) return QGG_ERR_INVALID_ARG;
  return backward(w_gate_up, w_down, dy, nullptr, topk_gates, p, h_saved, T, d, E, k, inter,
                  variant, chunk, workspace, ws_bytes, dx, nullptr, nullptr, stream);
}

qgg_status moe_router_bwd(const qgg_qweight* w_gate_up, const qgg_qweight* w_down,
                          const uint16_t* dy, const int32_t* topk_ids, const float* topk_gates,
                          const qgg_perm* p, const uint16_t* h_saved, int T, int d, int E, int k,
                          int inter, int variant, int chunk, void* workspace, size_t ws_bytes,
                          uint16_t* dx, float* dgates, float* dlogits, qgg_stream_t stream) {
  if (T > 0 && !dgates && !dlogits) return QGG_ERR_INVALID_ARG;
  return backward(w_gate_up, w_down, dy, topk_ids, topk_gates, p, h_saved, T, d, E, k, inter,
                  variant, chunk, workspace, ws_bytes, dx, dgates, dlogits, stream);
}

qgg_status moe_ffn_bwd_lora(const qgg_qweight* w_gate_up, const qgg_qweight* w_down,
                            const qgg_lora* lora_gate_up, const qgg_lora* lora_down,
                            const uint16_t* x, const uint16_t* dy, const float* topk_gates,
                            const qgg_perm* p, const uint16_t* h_saved,
                            const uint16_t* u_gate_up, const uint16_t* u_down, int T, int d,
                            int E, int k, int inter, int variant, int chunk, void* workspace,
                            size_t ws_bytes, uint16_t* dx, float* dA_gate_up, float* dB_gate_up,
                            float* dA_down, float* dB_down, qgg_stream_t stream) {
  const qgg_lora* lgu = lora_gate_up;
  const qgg_lora* ldn = lora_down;
  if (!lgu && !ldn) return QGG_ERR_INVALID_ARG;
  if (!valid_route_dims(T, E, k) || d <= 0 || inter <= 0 || chunk < 0) return QGG_ERR_INVALID_ARG;
  if (!valid_lora_rank(lgu) || !valid_lora_rank(ldn)) return QGG_ERR_UNSUPPORTED;
  if ((lgu && (!std::isfinite(lgu->alpha) || !lgu->A || !lgu->B)) ||
      (ldn && (!std::isfinite(ldn->alpha) || !ldn->A || !ldn->B)))
    return QGG_ERR_INVALID_ARG;
  if (!valid_weight(w_gate_up, E, 2 * inter, d) || !valid_weight(w_down, E, d, inter))
    return QGG_ERR_INVALID_ARG;
  if (w_gate_up->fmt != w_down->fmt) return QGG_ERR_INVALID_ARG;
  if (variant != QGG_CHUNKED && variant != QGG_FUSED) return QGG_ERR_INVALID_ARG;
  if (!valid_perm(p, (int64_t)T * k)) return QGG_ERR_INVALID_ARG;
  const bool want_gu = lgu && (dA_gate_up || dB_gate_up);
  const bool want_dn = ldn && (dA_down || dB_down);
  if (!dx && !want_gu && !want_dn) return QGG_ERR_INVALID_ARG;
  if (T > 0 && (!dy || !topk_gates || !h_saved)) return QGG_ERR_INVALID_ARG;
  if (T > 0 && lgu && ((dA_gate_up && !x) || (dB_gate_up && !u_gate_up)))
    return QGG_ERR_INVALID_ARG;
  if (T > 0 && ldn && dB_down && !u_down) return QGG_ERR_INVALID_ARG;
  if (d % 256 || inter % 256) return QGG_ERR_UNSUPPORTED;
  const int64_t P = (int64_t)T * k;
  if (!a_fits(T, d) || !a_fits(P, 2 * inter)) return QGG_ERR_UNSUPPORTED;
  size_t scratch = 0;
  const size_t need =
      qgg_workspace_bytes(QGG_CALL_FFN_LORA_BWD, T, d, E, k, inter, variant, chunk, &scratch);
  if (!workspace || ws_bytes < need) return QGG_ERR_WORKSPACE_TOO_SMALL;
  const int C = chunk > 0 ? std::min(chunk, E) : (int)std::min<int64_t>(E, std::max<int64_t>(P, 1));
  Carver cv(workspace);
  Plan pl;
  carve_plan(cv, P, E, T, pl);
  uint16_t* dh = cv.take<uint16_t>((size_t)P * 2 * inter * 2);
  uint16_t* dxp = cv.take<uint16_t>((size_t)P * d * 2);
  uint16_t* sbuf = cv.take<uint16_t>(scratch);
  cv.take<float>((size_t)P * (inter / 256) * 4);
  uint16_t* abuf = cv.take<uint16_t>((size_t)P * inter * 2);
  uint16_t* da_share = cv.take<uint16_t>((size_t)P * inter * 2);
  uint16_t* dx_share = cv.take<uint16_t>((size_t)P * d * 2);
  float* du = cv.take<float>((size_t)P * kMaxLoraRank * 4);
  float* us = cv.take<float>((size_t)P * kMaxLoraRank * 4);
  uint16_t* bt =
      cv.take<uint16_t>((size_t)E * kMaxLoraRank * std::max<int64_t>(d, 2 * inter) * 2);
  const PermPtrs pp = to_ptrs(p);
  const int32_t* ntiles = pl.chunk_first + E + 1;
  if (P > 0)
    QGG_HIP(launch_tile_plan(pp, E, 32 * pl.mb, variant == QGG_CHUNKED ? C : 0, pl.tiles,
                             pl.chunk_first, stream));
  const int mt = P > 0 ? (int)pl.cap : 0;

  // the down adapter's share of dA (and its gradients) first: the SwiGLU
  // derivative in the down GEMM's epilogue needs the whole dA
  if (ldn) {
    if (P > 0) QGG_HIP(launch_swiglu_act(h_saved, inter, p->offsets, E, P, abuf, stream));
    QGG_HIP(launch_lora_bwd_gated(abuf, inter, d, E, p->perm, k, topk_gates, p->offsets,
                                  pl.tiles, ntiles, mt, pl.mb, ldn->A, ldn->B, ldn->rank,
                                  ldn->alpha, dy, u_down, bt, du, us, P > 0 ? da_share : nullptr,
                                  dA_down, dB_down, P, stream));
  }
  GemmArgs dn = base_args(w_down, pl);
  dn.a = dy;
  dn.lda = d;
  dn.a_rows = T;
  dn.amode = kATokens;
  dn.perm = p->perm;
  dn.topk = k;
  dn.y = dh;
  dn.ldy = 2 * inter;
  dn.epi = kEpiSwiGLUBwd;
  dn.inter = inter;
  dn.h = const_cast<uint16_t*>(h_saved);
  dn.gates = topk_gates;
  dn.lora_da = ldn ? da_share : nullptr;
  GemmArgs gu = base_args(w_gate_up, pl);
  gu.a = dh;
  gu.lda = 2 * inter;
  gu.a_rows = P;
  gu.amode = kASorted;
  gu.perm = p->perm;
  gu.topk = k;
  gu.y = dxp;
  gu.ldy = d;
  gu.epi = kEpiStore;
  // the gate_up adapter: du = dH . B_gu, its share of dXp, dA, dB
  auto gate_up_adapter = [&]() {
    return launch_lora_bwd(x, d, 2 * inter, E, p->perm, k, kATokens, p->offsets, pl.tiles,
                           ntiles, mt, pl.mb, lgu->A, lgu->B, lgu->rank, lgu->alpha, dh,
                           u_gate_up, bt, du, dx ? dx_share : nullptr, dA_gate_up, dB_gate_up,
                           stream);
  };
  if (P > 0 && variant == QGG_FUSED) {
    QGG_HIP(launch_gemm_tn(dn, pl.mb, stream));
    if (lgu) QGG_HIP(gate_up_adapter());
    if (dx) QGG_HIP(launch_gemm_tn(gu, pl.mb, stream));
  } else if (P > 0) {
    // every chunk's down projection, then the gate_up adapter (it needs all
    // of dH), then every chunk's gate_up projection; one chunk of scratch
    const int nch = chunk_iterations(E, P, C);
    dn.src = gu.src = kSrcBF16;
    dn.wbf16 = gu.wbf16 = sbuf;
    dn.max_tiles = gu.max_tiles = (int)pl.cap;
    for (int c = 0; c < nch; ++c) {
      dn.range = pl.chunk_first + c;
      dn.bf16_slot_base = c * C;
      QGG_HIP(launch_dequant(w_down->fmt, w_down->packed, w_down->scales, w_down->layout, d,
                             inter, p->active, p->n_active, c * C, C, true, sbuf, stream));
      QGG_HIP(launch_gemm_tn(dn, pl.mb, stream));
    }
    if (lgu) QGG_HIP(gate_up_adapter());
    for (int c = 0; dx && c < nch; ++c) {
      gu.range = pl.chunk_first + c;
      gu.bf16_slot_base = c * C;
      QGG_HIP(launch_dequant(w_gate_up->fmt, w_gate_up->packed, w_gate_up->scales,
                             w_gate_up->layout, 2 * inter, d, p->active, p->n_active, c * C, C,
                             true, sbuf, stream));
      QGG_HIP(launch_gemm_tn(gu, pl.mb, stream));
    }
  } else if (lgu) {
    QGG_HIP(gate_up_adapter());   // no routed rows: zero adapter gradients
  }
  if (dx) QGG_HIP(launch_combine(dxp, d, p->inv_perm, nullptr, T, k, dx, stream,
                                 lgu ? dx_share : nullptr));
  return QGG_OK;
}

}  // extern "C"
