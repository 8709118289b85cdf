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

// ---------------------------------------------------------------- backward
// Gradients of L = <dY, y> through the adapter term alpha (x A^T) B^T, the
// base frozen: du = dY B_e, dx = alpha du A_e, dA_e = alpha sum_i du_i (x) x_i,
// dB_e = sum_i dY_i (x) u_i.  Plain fp32 FMA kernels with LDS staging (the
// adapter is a rank-r update: these are 2 P r (N + 2K) + 2 P N r flops next to
// the base's 2 P N K); every sum runs in a fixed order, so results are
// deterministic.

// du [P][rank] fp32 for one 32-row block of a tile; thread (row = t / 8,
// column group t % 8) owns columns g, g + 8, ...
template <int RQ>
__global__ __launch_bounds__(256) void k_lora_du(const uint16_t* __restrict__ dy, int N,
                                                 const int4* __restrict__ tiles,
                                                 const int32_t* __restrict__ ntiles, int MB,
                                                 const uint16_t* __restrict__ B, int rank,
                                                 float* __restrict__ du) {
  __shared__ __attribute__((aligned(16))) uint16_t dys[32][64 + 8];
  __shared__ __attribute__((aligned(16))) uint16_t bs[64][128 + 8];
  const int t = blockIdx.x / MB, mb = blockIdx.x % MB;
  if (t >= *ntiles) return;
  const int4 tile = tiles[t];
  const int expert = tile.x, row0 = tile.y, nrows = tile.z;
  if (mb * 32 >= nrows) return;
  const int tid = threadIdx.x;
  const int row = tid >> 3, cg = tid & 7;
  const int lrow = min(mb * 32 + row, nrows - 1);
  const int rp = rank / 8;                    // 16-byte pieces per B row
  float acc[RQ];
#pragma unroll
  for (int q = 0; q < RQ; ++q) acc[q] = 0.f;
  for (int n0 = 0; n0 < N; n0 += 64) {
    *reinterpret_cast<u32x4_t*>(&dys[row][8 * cg]) =
        *reinterpret_cast<const u32x4_t*>(dy + (int64_t)(row0 + lrow) * N + n0 + 8 * cg);
    for (int pc = tid; pc < 64 * rp; pc += 256) {
      const int n = pc / rp, jp = pc % rp;
      *reinterpret_cast<u32x4_t*>(&bs[n][8 * jp]) = *reinterpret_cast<const u32x4_t*>(
          B + ((int64_t)expert * N + n0 + n) * rank + 8 * jp);
    }
    __syncthreads();
    for (int n = 0; n < 64; ++n) {
      const float d = bf16_to_f32(dys[row][n]);
#pragma unroll
      for (int q = 0; q < RQ; ++q)
        if (cg + 8 * q < rank) acc[q] = fmaf(d, bf16_to_f32(bs[n][cg + 8 * q]), acc[q]);
    }
    __syncthreads();
  }
  if (mb * 32 + row < nrows) {
#pragma unroll
    for (int q = 0; q < RQ; ++q)
      if (cg + 8 * q < rank) du[(int64_t)(row0 + mb * 32 + row) * rank + cg + 8 * q] = acc[q];
  }
}

// dx [P][K] BF16 = alpha du A_e for one 32-row block and 256 columns
__global__ __launch_bounds__(256) void k_lora_dx(const float* __restrict__ du,
                                                 const int4* __restrict__ tiles,
                                                 const int32_t* __restrict__ ntiles, int MB,
                                                 const uint16_t* __restrict__ A, int rank, int K,
                                                 float alpha, uint16_t* __restrict__ dx) {
  __shared__ float dus[32][128];
  const int t = blockIdx.x / MB, mb = blockIdx.x % MB;
  if (t >= *ntiles) return;
  const int4 tile = tiles[t];
  const int expert = tile.x, row0 = tile.y, nrows = tile.z;
  if (mb * 32 >= nrows) return;
  const int tid = threadIdx.x;
  const int nr = min(32, nrows - mb * 32);
  for (int q = tid; q < 32 * rank; q += 256) {
    const int r = q / rank, j = q % rank;
    dus[r][j] = r < nr ? du[(int64_t)(row0 + mb * 32 + r) * rank + j] : 0.f;
  }
  __syncthreads();
  const int k = blockIdx.y * 256 + tid;
  if (k >= K) return;
  float acc[32];
#pragma unroll
  for (int r = 0; r < 32; ++r) acc[r] = 0.f;
  const uint16_t* a = A + (int64_t)expert * rank * K + k;
  for (int j = 0; j < rank; ++j) {
    const float w = bf16_to_f32(a[(int64_t)j * K]);
#pragma unroll
    for (int r = 0; r < 32; ++r) acc[r] = fmaf(dus[r][j], w, acc[r]);
  }
#pragma unroll
  for (int r = 0; r < 32; ++r)
    if (r < nr)
      dx[(int64_t)(row0 + mb * 32 + r) * K + k] = __builtin_bit_cast(uint16_t, (__bf16)(alpha * acc[r]));
}

// dA [E][rank][K] fp32 = alpha sum over the expert's rows of du_i (x) x_i;
// thread owns column k, rows staged 32 at a time
template <int R>
__global__ __launch_bounds__(256) void k_lora_dA(const float* __restrict__ du,
                                                 const uint16_t* __restrict__ x, int K,
                                                 const int32_t* __restrict__ offsets,
                                                 const int32_t* __restrict__ perm, int topk,
                                                 int amode, int rank, float alpha,
                                                 float* __restrict__ dA) {
  __shared__ float dus[32][128];
  __shared__ int64_t src[32];
  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  const int k = blockIdx.y * 256 + tid;
  const int i0 = offsets[e], i1 = offsets[e + 1];
  float acc[R];
#pragma unroll
  for (int j = 0; j < R; ++j) acc[j] = 0.f;
  for (int b = i0; b < i1; b += 32) {
    const int nr = min(32, i1 - b);
    __syncthreads();
    for (int q = tid; q < 32 * rank; q += 256) {
      const int r = q / rank, j = q % rank;
      dus[r][j] = r < nr ? du[(int64_t)(b + r) * rank + j] : 0.f;
    }
    if (tid < 32) src[tid] = tid < nr ? (amode == kATokens ? perm[b + tid] / topk : (int64_t)(b + tid)) : 0;
    __syncthreads();
    if (k < K) {
      for (int r = 0; r < nr; ++r) {
        const float xv = bf16_to_f32(x[src[r] * K + k]);
#pragma unroll
        for (int j = 0; j < R; ++j)
          if (j < rank) acc[j] = fmaf(dus[r][j], xv, acc[j]);
      }
    }
  }
  if (k < K) {
#pragma unroll
    for (int j = 0; j < R; ++j)
      if (j < rank) dA[((int64_t)e * rank + j) * K + k] = alpha * acc[j];
  }
}

// dB [E][N][rank] fp32 = sum over the expert's rows of dY_i (x) u_i; thread
// owns output row n
template <int R>
__global__ __launch_bounds__(256) void k_lora_dB(const uint16_t* __restrict__ dy, int N,
                                                 const uint16_t* __restrict__ u,
                                                 const int32_t* __restrict__ offsets, int rank,
                                                 float* __restrict__ dB) {
  __shared__ float us[32][128];
  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = blockIdx.y * 256 + tid;
  const int i0 = offsets[e], i1 = offsets[e + 1];
  float acc[R];
#pragma unroll
  for (int j = 0; j < R; ++j) acc[j] = 0.f;
  for (int b = i0; b < i1; b += 32) {
    const int nr = min(32, i1 - b);
    __syncthreads();
    for (int q = tid; q < 32 * rank; q += 256) {
      const int r = q / rank, j = q % rank;
      us[r][j] = r < nr ? bf16_to_f32(u[(int64_t)(b + r) * rank + j]) : 0.f;
    }
    __syncthreads();
    if (n < N) {
      for (int r = 0; r < nr; ++r) {
        const float g = bf16_to_f32(dy[(int64_t)(b + r) * N + n]);
#pragma unroll
        for (int j = 0; j < R; ++j)
          if (j < rank) acc[j] = fmaf(g, us[r][j], acc[j]);
      }
    }
  }
  if (n < N) {
    float* o = dB + ((int64_t)e * N + n) * rank;
#pragma unroll
    for (int j = 0; j < R; ++j)
      if (j < rank) o[j] = acc[j];
  }
}

}  // namespace

hipError_t launch_lora_bwd(const uint16_t* x, int K, int N, int E, const int32_t* perm, int topk,
                           int amode, const int32_t* offsets, const int4* tiles,
                           const int32_t* ntiles, int max_tiles, int MB, const uint16_t* A,
                           const uint16_t* B, int rank, float alpha, const uint16_t* dy,
                           const uint16_t* u, float* du, uint16_t* dx, float* dA, float* dB,
                           hipStream_t s) {
  if (dx || dA) {
    if (max_tiles > 0) {
      const dim3 g1((unsigned)(max_tiles * MB));
      if (rank <= 32)
        hipLaunchKernelGGL(k_lora_du<4>, g1, dim3(256), 0, s, dy, N, tiles, ntiles, MB, B, rank, du);
      else if (rank <= 64)
        hipLaunchKernelGGL(k_lora_du<8>, g1, dim3(256), 0, s, dy, N, tiles, ntiles, MB, B, rank, du);
      else
        hipLaunchKernelGGL(k_lora_du<16>, g1, dim3(256), 0, s, dy, N, tiles, ntiles, MB, B, rank, du);
      if (dx)
        hipLaunchKernelGGL(k_lora_dx, dim3((unsigned)(max_tiles * MB), (K + 255) / 256), dim3(256), 0,
                           s, du, tiles, ntiles, MB, A, rank, K, alpha, dx);
    }
    if (dA) {
      const dim3 g3((unsigned)E, (K + 255) / 256);
      if (rank <= 32)
        hipLaunchKernelGGL(k_lora_dA<32>, g3, dim3(256), 0, s, du, x, K, offsets, perm, topk, amode, rank, alpha, dA);
      else if (rank <= 64)
        hipLaunchKernelGGL(k_lora_dA<64>, g3, dim3(256), 0, s, du, x, K, offsets, perm, topk, amode, rank, alpha, dA);
      else
        hipLaunchKernelGGL(k_lora_dA<128>, g3, dim3(256), 0, s, du, x, K, offsets, perm, topk, amode, rank, alpha, dA);
    }
  }
  if (dB) {
    const dim3 g4((unsigned)E, (N + 255) / 256);
    if (rank <= 32)
      hipLaunchKernelGGL(k_lora_dB<32>, g4, dim3(256), 0, s, dy, N, u, offsets, rank, dB);
    else if (rank <= 64)
      hipLaunchKernelGGL(k_lora_dB<64>, g4, dim3(256), 0, s, dy, N, u, offsets, rank, dB);
    else
      hipLaunchKernelGGL(k_lora_dB<128>, g4, dim3(256), 0, s, dy, N, u, offsets, rank, dB);
  }
  return hipGetLastError();
}

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
