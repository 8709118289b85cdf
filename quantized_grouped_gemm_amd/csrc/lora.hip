// LoRA adapter on the frozen quantized projection: the adapter's down
// projection u = alpha * (x . A_e^T) per routed row.
//
// Orbit page, opening section: the base stays frozen in its low-precision
// format and a BF16 adapter on top of it is what trains.  The adapter form is
// a reading: the Orbit issue page has the maintainers default to orthogonal
// finetuning (OFT / QOFT) over LoRA, which the question raises, and the
// pages give no OFT formula, so the additive low-rank form is built.  The up
// projection u . B_e^T is folded into the forward grouped GEMM as extra
// MFMA steps after its quantized K loop (same fp32 accumulators, one BF16
// rounding), so only u is formed here.
//
// One workgroup per M-tile, one wavefront per 32-row block: rank / 32
// (rounded up) MFMA column blocks of v_mfma_f32_32x32x16_bf16, both operands
// straight from global memory (a lane's 8 K values of an x row and of an A_e
// row are 16 contiguous bytes); the tile's wavefronts read the same A_e rows
// at about the same time, so the expert's adapter is fetched once per tile.
#include "qgg_device.hpp"
#include "qgg_internal.hpp"

#include <type_traits>

namespace qgg {

namespace {

template <int NCB, typename OUT>
__global__ __launch_bounds__(256) void k_lora_u(const uint16_t* __restrict__ x, int K,
                                                const int32_t* __restrict__ perm, int topk,
                                                int amode, const int4* __restrict__ tiles,
                                                const int32_t* __restrict__ ntiles,
                                                const uint16_t* __restrict__ A, int rank,
                                                float alpha, OUT* __restrict__ u) {
  const int t = blockIdx.x;
  const int mb = threadIdx.x >> 6;     // wavefront = 32-row block of the tile
  if (t >= *ntiles) return;
  const int4 tile = tiles[t];
  const int expert = tile.x, row0 = tile.y, nrows = tile.z;
  if (mb * 32 >= nrows) return;
  const int lane = threadIdx.x & 63;
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
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int rr = mb * 32 + 8 * i + 4 * half + jj;
        if (rr < nrows && j < rank) {
          const float v = alpha * acc[cb][4 * i + jj];
          if constexpr (std::is_same<OUT, float>::value)
            u[(int64_t)(row0 + rr) * rank + j] = v;
          else
            u[(int64_t)(row0 + rr) * rank + j] = __builtin_bit_cast(uint16_t, (__bf16)v);
        }
      }
  }
}

// ---------------------------------------------------------------- backward
// Gradients of L = <dY, y> through the adapter term alpha (x A^T) B^T, the
// base frozen: du = dY B_e, dx = alpha du A_e, dA_e = alpha sum_i du_i (x) x_i,
// dB_e = sum_i dY_i (x) u_i.  du is the same row-times-matrix product as u
// (k_lora_u on MFMA, with B_e transposed once to [rank][N]); the other three
// run on MFMA with operands staged in LDS and read back transposed.  Every
// sum runs in a fixed order, so results are deterministic.

// Bt[e][j][n] = B[e][n][j]: a 64-row slab of one expert through LDS
__global__ __launch_bounds__(256) void k_lora_bt(const uint16_t* __restrict__ B, int N, int rank,
                                                 uint16_t* __restrict__ Bt) {
  __shared__ uint16_t t[64][128 + 2];
  const int e = blockIdx.x, n0 = blockIdx.y * 64;
  for (int q = threadIdx.x; q < 64 * rank; q += 256) {
    const int n = q / rank, j = q % rank;
    t[n][j] = B[((int64_t)e * N + n0 + n) * rank + j];
  }
  __syncthreads();
  for (int q = threadIdx.x; q < 64 * rank; q += 256) {
    const int j = q / 64, n = q % 64;
    Bt[((int64_t)e * rank + j) * N + n0 + n] = t[n][j];
  }
}

// dx [P][K] BF16 = alpha du A_e for one 32-row block and 256 columns, on
// MFMA: the expert's A rows for those columns sit row-major in LDS and the
// B operand (8 consecutive rank indices of one column) is read back with
// transposing reads, as in the transposed grouped GEMM; each wavefront owns
// 64 columns.  du (fp32) is rounded to BF16 for the MFMA A operand.
__global__ __launch_bounds__(256) void k_lora_dx(const float* __restrict__ du,
                                                 const int4* __restrict__ tiles,
                                                 const int32_t* __restrict__ ntiles, int MB,
                                                 const uint16_t* __restrict__ A, int rank, int K,
                                                 float alpha, uint16_t* __restrict__ dx) {
  extern __shared__ __attribute__((aligned(16))) uint8_t at[];   // [rank][256] BF16
  const int t = blockIdx.x / MB, mb = blockIdx.x % MB;
  if (t >= *ntiles) return;
  const int4 tile = tiles[t];
  const int expert = tile.x, row0 = tile.y, nrows = tile.z;
  if (mb * 32 >= nrows) return;
  const int tid = threadIdx.x;
  const int c0 = blockIdx.y * 256;
  // stage A_e[0..rank)[c0 .. c0 + 256) (columns past K read as zero)
  for (int pc = tid; pc < rank * 32; pc += 256) {
    const int j = pc >> 5, piece = pc & 31;
    const int col = c0 + 8 * piece;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (col < K) v = *reinterpret_cast<const u32x4_t*>(A + ((int64_t)expert * rank + j) * K + col);
    *reinterpret_cast<u32x4_t*>(at + j * 512 + piece * 16) = v;
  }
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const int G = lane >> 4, p = lane & 15;
  // A operand: this lane's du row (clamped into the block)
  const int r = min(mb * 32 + col, nrows - 1);
  const float* dur = du + (int64_t)(row0 + r) * rank + 8 * half;
  // B operand read offsets (sub-step 0): lane 16 G + p points at rank row
  // 8 (G >> 1) + 4 up + p / 4, column 64 wave + 32 nb + 16 (G & 1) + 4 (p & 3)
  int boff[2][2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int up = 0; up < 2; ++up)
      boff[nb][up] = (8 * (G >> 1) + 4 * up + (p >> 2)) * 512 +
                     (64 * wave + 32 * nb + 16 * (G & 1) + 4 * (p & 3)) * 2;
  f32x16_t acc[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[nb][i] = 0.f;
  for (int j0 = 0; j0 < rank; j0 += 16) {
    const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(dur + j0);
    const f32x4_t hi = *reinterpret_cast<const f32x4_t*>(dur + j0 + 4);
    const bf16x8_t a = __builtin_bit_cast(
        bf16x8_t, u32x4_t{pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                          pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3])});
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const uint2 b0 = lds_tr4(at + j0 * 512 + boff[nb][0]);
      const uint2 b1 = lds_tr4(at + j0 * 512 + boff[nb][1]);
      const bf16x8_t b = __builtin_bit_cast(bf16x8_t, u32x4_t{b0.x, b0.y, b1.x, b1.y});
      acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[nb], 0, 0, 0);
    }
  }
  // C layout: lane holds column `col` of rows 8 i + 4 half + jj
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int k = c0 + 64 * wave + 32 * nb + col;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int rr = mb * 32 + 8 * i + 4 * half + jj;
        if (rr < nrows && k < K)
          dx[(int64_t)(row0 + rr) * K + k] =
              __builtin_bit_cast(uint16_t, (__bf16)(alpha * acc[nb][4 * i + jj]));
      }
  }
}

// Weight gradient of one expert on MFMA, reduced over the expert's rows i
// (ascending, 16 per MFMA step): G[j][c] = scale sum_i L[i][j] R[i][c] for
// dA (L = du, R = the rows' x; stored [rank][C]), or G[c][j] = sum_i R[i][c]
// L[i][j] for dB (L = u, R = dY; stored [C][rank]).  Each step stages 16 rows
// of R (256 columns) and of L (rank, zero-padded to 32s) in LDS, row-major;
// both MFMA operands (8 consecutive rows of one column) come back through
// transposing reads.  Rows past the expert's end are zero.
template <int NJB, typename LT, bool TRANS_OUT>
__global__ __launch_bounds__(256) void k_lora_wgrad(const LT* __restrict__ L, int rank,
                                                    const uint16_t* __restrict__ Rm, int C,
                                                    const int32_t* __restrict__ offsets,
                                                    const int32_t* __restrict__ perm, int topk,
                                                    int amode, float scale,
                                                    float* __restrict__ G) {
  constexpr int LW = 32 * NJB;                     // L tile width (elements)
  __shared__ __attribute__((aligned(16))) uint8_t rt[16 * 512];
  __shared__ __attribute__((aligned(16))) uint8_t lt[16 * LW * 2];
  const int e = blockIdx.x;
  const int c0 = blockIdx.y * 256;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const int Gq = lane >> 4, p = lane & 15;
  const int i0 = offsets[e], i1 = offsets[e + 1];
  // transposing-read offsets: lane 16 Gq + p points at tile row
  // 8 (Gq >> 1) + 4 up + p / 4 and column 16 (Gq & 1) + 4 (p & 3) of its block
  const int trow0 = 8 * (Gq >> 1) + (p >> 2);
  const int tcol = 16 * (Gq & 1) + 4 * (p & 3);
  f32x16_t acc[NJB][2];
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[jb][nb][q] = 0.f;
  for (int b = i0; b < i1; b += 16) {
    __syncthreads();
    for (int pc = tid; pc < 16 * 32; pc += 256) {
      const int r = pc >> 5, piece = pc & 31;
      const int i = b + r;
      const int cc = c0 + 8 * piece;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (i < i1 && cc < C) {
        const int64_t src = amode == kATokens ? perm[i] / topk : (int64_t)i;
        v = *reinterpret_cast<const u32x4_t*>(Rm + src * C + cc);
      }
      *reinterpret_cast<u32x4_t*>(rt + r * 512 + piece * 16) = v;
    }
    for (int q = tid; q < 16 * LW; q += 256) {
      const int r = q / LW, j = q % LW;
      float v = 0.f;
      if (b + r < i1 && j < rank) {
        if constexpr (std::is_same<LT, float>::value) v = L[(int64_t)(b + r) * rank + j];
        else v = bf16_to_f32(L[(int64_t)(b + r) * rank + j]);
      }
      reinterpret_cast<uint16_t*>(lt)[r * LW + j] = __builtin_bit_cast(uint16_t, (__bf16)v);
    }
    __syncthreads();
    bf16x8_t lf[NJB], rf[2];
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) {
      const uint2 a0 = lds_tr4(lt + trow0 * LW * 2 + (32 * jb + tcol) * 2);
      const uint2 a1 = lds_tr4(lt + (trow0 + 4) * LW * 2 + (32 * jb + tcol) * 2);
      lf[jb] = __builtin_bit_cast(bf16x8_t, u32x4_t{a0.x, a0.y, a1.x, a1.y});
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int cb = 64 * wave + 32 * nb + tcol;
      const uint2 b0 = lds_tr4(rt + trow0 * 512 + cb * 2);
      const uint2 b1 = lds_tr4(rt + (trow0 + 4) * 512 + cb * 2);
      rf[nb] = __builtin_bit_cast(bf16x8_t, u32x4_t{b0.x, b0.y, b1.x, b1.y});
    }
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        if constexpr (TRANS_OUT)
          acc[jb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rf[nb], lf[jb], acc[jb][nb], 0, 0, 0);
        else
          acc[jb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lf[jb], rf[nb], acc[jb][nb], 0, 0, 0);
      }
  }
  // C layout: lane holds column `col` of rows 8 q + 4 half + qq of each tile
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int tr = 8 * q + 4 * half + qq;     // tile row
          const float v = scale * acc[jb][nb][4 * q + qq];
          if constexpr (TRANS_OUT) {
            const int n = c0 + 64 * wave + 32 * nb + tr, j = 32 * jb + col;
            if (n < C && j < rank) G[((int64_t)e * C + n) * rank + j] = v;
          } else {
            const int j = 32 * jb + tr, c = c0 + 64 * wave + 32 * nb + col;
            if (j < rank && c < C) G[((int64_t)e * rank + j) * C + c] = v;
          }
        }
}

// du[i][:] *= g_i and us[i][:] = g_i * u[i][:] with g_i = gates[perm[i]], for
// the sorted rows i < offsets[E]: the gate of a pair scales the upstream
// gradient of its down-projection adapter (fp32).
__global__ __launch_bounds__(256) void k_gate_rows(float* __restrict__ du,
                                                   const uint16_t* __restrict__ u,
                                                   float* __restrict__ us, int rank,
                                                   const int32_t* __restrict__ perm,
                                                   const float* __restrict__ gates,
                                                   const int32_t* __restrict__ nrows_p) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t i = q / rank;
  if (i >= *nrows_p) return;
  const float g = gates[perm[i]];
  du[q] *= g;
  if (u) us[q] = g * bf16_to_f32(u[q]);
}

template <typename LT, bool TRANS_OUT>
void launch_wgrad(const LT* L, int rank, const uint16_t* Rm, int C, int E,
                  const int32_t* offsets, const int32_t* perm, int topk, int amode, float scale,
                  float* G, hipStream_t s) {
  const dim3 grid((unsigned)E, (C + 255) / 256);
  const int njb = (rank + 31) / 32;
  if (njb == 1)
    hipLaunchKernelGGL((k_lora_wgrad<1, LT, TRANS_OUT>), grid, dim3(256), 0, s, L, rank, Rm, C, offsets, perm, topk, amode, scale, G);
  else if (njb == 2)
    hipLaunchKernelGGL((k_lora_wgrad<2, LT, TRANS_OUT>), grid, dim3(256), 0, s, L, rank, Rm, C, offsets, perm, topk, amode, scale, G);
  else if (njb == 3)
    hipLaunchKernelGGL((k_lora_wgrad<3, LT, TRANS_OUT>), grid, dim3(256), 0, s, L, rank, Rm, C, offsets, perm, topk, amode, scale, G);
  else
    hipLaunchKernelGGL((k_lora_wgrad<4, LT, TRANS_OUT>), grid, dim3(256), 0, s, L, rank, Rm, C, offsets, perm, topk, amode, scale, G);
}

}  // namespace

template <typename OUT>
static void lora_rows_x_wt(const uint16_t* x, int K, const int32_t* perm, int topk, int amode,
                           const int4* tiles, const int32_t* ntiles, int max_tiles, int MB,
                           const uint16_t* W, int rank, float alpha, OUT* out, hipStream_t s) {
  const dim3 grid((unsigned)max_tiles);
  const int ncb = (rank + 31) / 32;
  if (ncb == 1)
    hipLaunchKernelGGL((k_lora_u<1, OUT>), grid, dim3(64 * MB), 0, s, x, K, perm, topk, amode, tiles, ntiles, W, rank, alpha, out);
  else if (ncb == 2)
    hipLaunchKernelGGL((k_lora_u<2, OUT>), grid, dim3(64 * MB), 0, s, x, K, perm, topk, amode, tiles, ntiles, W, rank, alpha, out);
  else if (ncb == 3)
    hipLaunchKernelGGL((k_lora_u<3, OUT>), grid, dim3(64 * MB), 0, s, x, K, perm, topk, amode, tiles, ntiles, W, rank, alpha, out);
  else
    hipLaunchKernelGGL((k_lora_u<4, OUT>), grid, dim3(64 * MB), 0, s, x, K, perm, topk, amode, tiles, ntiles, W, rank, alpha, out);
}

hipError_t launch_lora_bwd(const uint16_t* x, int K, int N, int E, const int32_t* perm, int topk,
                           int amode, const int32_t* offsets, const int4* tiles,
                           const int32_t* ntiles, int max_tiles, int MB, const uint16_t* A,
                           const uint16_t* B, int rank, float alpha, const uint16_t* dy,
                           const uint16_t* u, uint16_t* bt, float* du, uint16_t* dx, float* dA,
                           float* dB, hipStream_t s) {
  TimedLaunch timed_(kLLora, s);
  if (dx || dA) {
    // du = dY B_e over the sorted rows (zero rows: nothing to form)
    hipLaunchKernelGGL(k_lora_bt, dim3((unsigned)E, N / 64), dim3(256), 0, s, B, N, rank, bt);
    if (max_tiles > 0) {
      lora_rows_x_wt<float>(dy, N, perm, 1, kASorted, tiles, ntiles, max_tiles, MB, bt, rank,
                            1.0f, du, s);
      if (dx)
        hipLaunchKernelGGL(k_lora_dx, dim3((unsigned)(max_tiles * MB), (K + 255) / 256),
                           dim3(256), (size_t)rank * 512, s, du, tiles, ntiles, MB, A, rank, K,
                           alpha, dx);
    }
    if (dA) launch_wgrad<float, false>(du, rank, x, K, E, offsets, perm, topk, amode, alpha, dA, s);
  }
  if (dB) launch_wgrad<uint16_t, true>(u, rank, dy, N, E, offsets, perm, 1, kASorted, 1.0f, dB, s);
  return hipGetLastError();
}

hipError_t launch_lora_bwd_gated(const uint16_t* a, int K, int N, int E, const int32_t* perm,
                                 int topk, const float* gates, const int32_t* offsets,
                                 const int4* tiles, const int32_t* ntiles, int max_tiles, int MB,
                                 const uint16_t* A, const uint16_t* B, int rank, float alpha,
                                 const uint16_t* dy, const uint16_t* u, uint16_t* bt, float* du,
                                 float* us, uint16_t* dx, float* dA, float* dB, int64_t P,
                                 hipStream_t s) {
  TimedLaunch timed_(kLLora, s);
  if (max_tiles > 0) {
    // du = g * (dY[token] . B_e) per sorted row; us = g * u for dB
    hipLaunchKernelGGL(k_lora_bt, dim3((unsigned)E, N / 64), dim3(256), 0, s, B, N, rank, bt);
    lora_rows_x_wt<float>(dy, N, perm, topk, kATokens, tiles, ntiles, max_tiles, MB, bt, rank,
                          1.0f, du, s);
    const int64_t n = P * rank;
    hipLaunchKernelGGL(k_gate_rows, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, du,
                       dB ? u : nullptr, us, rank, perm, gates, offsets + E);
    if (dx)
      hipLaunchKernelGGL(k_lora_dx, dim3((unsigned)(max_tiles * MB), (K + 255) / 256), dim3(256),
                         (size_t)rank * 512, s, du, tiles, ntiles, MB, A, rank, K, alpha, dx);
  }
  // weight gradients: the kernels run even with no routed rows, so dA and dB
  // are written in full (zeros)
  if (dA) launch_wgrad<float, false>(du, rank, a, K, E, offsets, perm, 1, kASorted, alpha, dA, s);
  if (dB) launch_wgrad<float, true>(us, rank, dy, N, E, offsets, perm, topk, kATokens, 1.0f, dB, s);
  return hipGetLastError();
}

hipError_t launch_lora_u(const uint16_t* x, int K, const int32_t* perm, int topk, int amode,
                         const int4* tiles, const int32_t* ntiles, int max_tiles, int MB,
                         const uint16_t* A, int rank, float alpha, uint16_t* u, hipStream_t s) {
  TimedLaunch timed_(kLLora, s);
  if (max_tiles <= 0) return hipSuccess;
  lora_rows_x_wt<uint16_t>(x, K, perm, topk, amode, tiles, ntiles, max_tiles, MB, A, rank, alpha,
                           u, s);
  return hipGetLastError();
}

}  // namespace qgg
