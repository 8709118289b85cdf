// LoRA adapter on the frozen quantized projection: the adapter's down
// projection u = alpha * (x . A_e^T) per routed row.
//
// Orbit page, opening section: the base stays frozen in its low-precision
// format and a BF16 adapter on top of it is what trains; the Orbit
// repository's issue #1 names LoRA as that adapter's common form.  The up
// projection u . B_e^T is folded into the forward grouped GEMM as extra
// MFMA steps after its quantized K loop (same fp32 accumulators, one BF16
// rounding), so only u is formed here.
//
// One wavefront per 32-row block of an M-tile: rank / 32 (rounded up) MFMA
// column blocks of v_mfma_f32_32x32x16_bf16, both operands straight from
// global memory (a lane's 8 K values of an x row and of an A_e row are 16
// contiguous bytes), K / 16 steps, four in flight.
#include "qgg_device.hpp"
#include "qgg_internal.hpp"

namespace qgg {

namespace {

template <int NCB>
__global__ __launch_bounds__(64) void k_lora_u(const uint16_t* __restrict__ x, int K,
                                               const int32_t* __restrict__ perm, int topk,
                                               int amode, const int4* __restrict__ tiles,
                                               const int32_t* __restrict__ ntiles, int MB,
                                               const uint16_t* __restrict__ A, int rank,
                                               float alpha, uint16_t* __restrict__ u) {
  const int t = blockIdx.x / MB;
  const int mb = blockIdx.x % MB;
  if (t >= *ntiles) return;
  const int4 tile = tiles[t];
  const int expert = tile.x, row0 = tile.y, nrows = tile.z;
  if (mb * 32 >= nrows) return;
  const int lane = threadIdx.x;
  const int col = lane & 31, half = lane >> 5;
  // this lane's A-operand row (clamped into the tile) and its source row of x
  const int r = min(mb * 32 + col, nrows - 1);
  const int64_t srow = amode == kATokens ? perm[row0 + r] / topk : (int64_t)(row0 + r);
  const uint16_t* xa = x + srow * K + 8 * half;
  const uint16_t* wb[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int j = min(32 * cb + col, rank - 1);
    wb[cb] = A + ((int64_t)expert * rank + j) * K + 8 * half;
  }
  f32x16_t acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[cb][i] = 0.f;
  for (int k0 = 0; k0 < K; k0 += 64) {
    bf16x8_t a[4], b[4][NCB];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      a[s] = *reinterpret_cast<const bf16x8_t*>(xa + k0 + 16 * s);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        b[s][cb] = *reinterpret_cast<const bf16x8_t*>(wb[cb] + k0 + 16 * s);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], b[s][cb], acc[cb], 0, 0, 0);
  }
  // C layout: lane holds column `col` of rows 8 i + 4 half + j
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int j = 32 * cb + col;
    if (j >= rank) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int rr = mb * 32 + 8 * i + 4 * half + jj;
        if (rr < nrows) u[(int64_t)(row0 + rr) * rank + j] =
              __builtin_bit_cast(uint16_t, (__bf16)(alpha * acc[cb][4 * i + jj]));
      }
  }
}

}  // namespace

hipError_t launch_lora_u(const uint16_t* x, int K, const int32_t* perm, int topk, int amode,
                         const int4* tiles, const int32_t* ntiles, int max_tiles, int MB,
                         const uint16_t* A, int rank, float alpha, uint16_t* u, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  const dim3 grid((unsigned)(max_tiles * MB));
  const int ncb = (rank + 31) / 32;
  if (ncb == 1)
    hipLaunchKernelGGL(k_lora_u<1>, grid, dim3(64), 0, s, x, K, perm, topk, amode, tiles, ntiles, MB, A, rank, alpha, u);
  else if (ncb == 2)
    hipLaunchKernelGGL(k_lora_u<2>, grid, dim3(64), 0, s, x, K, perm, topk, amode, tiles, ntiles, MB, A, rank, alpha, u);
  else if (ncb == 3)
    hipLaunchKernelGGL(k_lora_u<3>, grid, dim3(64), 0, s, x, K, perm, topk, amode, tiles, ntiles, MB, A, rank, alpha, u);
  else
    hipLaunchKernelGGL(k_lora_u<4>, grid, dim3(64), 0, s, x, K, perm, topk, amode, tiles, ntiles, MB, A, rank, alpha, u);
  return hipGetLastError();
}

}  // namespace qgg
