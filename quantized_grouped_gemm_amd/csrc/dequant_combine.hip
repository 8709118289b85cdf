// Chunk dequantization (the chunked variant's scratch fill) and the
// gate-weighted combine / scatter-sum back to token order.
//
// Orbit page, section 时刻细节 ("Active-expert-chunked dequantization"): a
// chunk of router-selected experts is dequantized temporarily and the
// high-precision copy is released after the grouped GEMM; here "release" is
// the next chunk overwriting the same scratch in stream order.  Group-32
// decoding: "超大规模开放权重模型技术解析", 三 微缩放量化的原理.
#include "qgg_device.hpp"
#include "qgg_internal.hpp"

namespace qgg {

namespace {

// fp32 value of each E2M1 code (sign bit 3).
__constant__ float kE2M1Val[16] = {0.0f,  0.5f,  1.0f,  1.5f,  2.0f,  3.0f,  4.0f,  6.0f,
                                   -0.0f, -0.5f, -1.0f, -1.5f, -2.0f, -3.0f, -4.0f, -6.0f};

// Offset, in 16-byte units (and in scale entries), of scale group g of row n
// of expert e: rows layout, or the MFMA-tiled layout (tiles of 32 rows x 64
// K, slot 32 * (g % 2) + n % 32).
__device__ __forceinline__ int64_t group_index(int layout, int64_t e, int64_t n, int64_t g,
                                               int N, int K) {
  if (layout == 1)
    return ((e * (N / 32) + (n >> 5)) * (K / 64) + (g >> 1)) * 64 + (g & 1) * 32 + (n & 31);
  return (e * N + n) * (K / 32) + g;
}

// One thread per 32-element group: 16 packed bytes + 1 scale -> 64 bytes of
// BF16.  The product code value x scale is formed in fp32 (exact unless it
// overflows) and rounded to BF16 to nearest even; an E8M0 code of 255 (NaN)
// yields the quiet NaN 0x7FC0 for the whole group.  Output row-major
// [slot][N][K], or MFMA-tiled BF16 (see launch_dequant).
template <int FMT>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ packed,
                                                 const void* __restrict__ scales, int layout,
                                                 int N, int K, const int32_t* __restrict__ active,
                                                 const int32_t* __restrict__ n_active, int first,
                                                 int count, int tiled_out,
                                                 uint16_t* __restrict__ dst) {
  const int64_t groups_per_expert = (int64_t)N * (K / 32);
  // the chunk's live experts (the active list is read on the device, so an
  // empty chunk costs one short launch)
  const int live = min(count, *n_active - first);
  const int64_t total = live > 0 ? (int64_t)live * groups_per_expert : 0;
  for (int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gid < total;
       gid += (int64_t)gridDim.x * blockDim.x) {
  const int slot = (int)(gid / groups_per_expert);
  const int a = first + slot;
  const int64_t e = active[a];
  const int64_t gi = gid % groups_per_expert;
  int64_t n, g;
  if (tiled_out) {
    // threads walk the tiled order (tile, slot L) so that each wavefront's
    // stores of one piece are one contiguous KiB
    const int L = (int)(gi & 63);
    const int64_t tile = gi >> 6;
    n = (tile / (K / 64)) * 32 + (L & 31);
    g = (tile % (K / 64)) * 2 + (L >> 5);
  } else {
    n = gi / (K / 32);          // row-major order: n * (K/32) + group
    g = gi % (K / 32);
  }
  const int64_t src = group_index(layout, e, n, g, N, K);
  const u32x4_t w = reinterpret_cast<const u32x4_t*>(packed)[src];
  uint32_t out[16];
  if constexpr (FMT == 1) {
    const uint32_t code = static_cast<const uint8_t*>(scales)[src];
    const float s = e8m0_to_f32(code);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t byte = (w[i >> 2] >> (8 * (i & 3))) & 0xFFu;
      uint32_t lo = f32_to_bf16_rne(kE2M1Val[byte & 15] * s);
      uint32_t hi = f32_to_bf16_rne(kE2M1Val[byte >> 4] * s);
      if (code == 255) lo = hi = 0x7FC0u;
      out[i] = lo | (hi << 16);
    }
  } else {
    const float s = bf16_to_f32(static_cast<const uint16_t*>(scales)[src]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t byte = (w[i >> 2] >> (8 * (i & 3))) & 0xFFu;
      const int q0 = (int)(byte & 15u) - ((byte & 8u) ? 16 : 0);
      const int q1 = (int)(byte >> 4) - ((byte & 128u) ? 16 : 0);
      out[i] = f32_to_bf16_rne((float)q0 * s) | (f32_to_bf16_rne((float)q1 * s) << 16);
    }
  }
  if (tiled_out) {
    // piece s of slot L of tile (n / 32, g / 2): 16 bytes at (s * 64 + L) * 16
    uint8_t* tile = reinterpret_cast<uint8_t*>(dst) +
                    (((int64_t)slot * (N / 32) + (n >> 5)) * (K / 64) + (g >> 1)) * 4096;
    const int L = (int)((g & 1) * 32 + (n & 31));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4_t v = {out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]};
      *reinterpret_cast<u32x4_t*>(tile + (i * 64 + L) * 16) = v;
    }
  } else {
    u32x4_t* o = reinterpret_cast<u32x4_t*>(dst + ((int64_t)slot * groups_per_expert + gi) * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4_t v = {out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]};
      o[i] = v;
    }
  }
  }
}

// Rows -> MFMA-tiled copy: one thread per 16-byte group chunk, written in
// tiled order so the stores are contiguous across the wavefront.
template <int SB>
__global__ __launch_bounds__(256) void k_repack(const uint8_t* __restrict__ packed,
                                                const uint8_t* __restrict__ scales, int E, int N,
                                                int K, uint8_t* __restrict__ packed_out,
                                                uint8_t* __restrict__ scales_out) {
  const int64_t total = (int64_t)E * N * (K / 32);
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total) return;
  // t enumerates the tiled order: ((e, cb, j), slot L)
  const int L = (int)(t & 63);
  const int64_t tile = t >> 6;
  const int64_t j = tile % (K / 64);
  const int64_t ecb = tile / (K / 64);
  const int64_t cb = ecb % (N / 32);
  const int64_t e = ecb / (N / 32);
  const int64_t n = cb * 32 + (L & 31);
  const int64_t g = j * 2 + (L >> 5);
  const int64_t src = (e * N + n) * (K / 32) + g;
  reinterpret_cast<u32x4_t*>(packed_out)[t] = reinterpret_cast<const u32x4_t*>(packed)[src];
#pragma unroll
  for (int i = 0; i < SB; ++i) scales_out[t * SB + i] = scales[src * SB + i];
}

// out[t][:] = sum over j ascending of w_j * rows[inv_perm[t*k+j]][:], fp32
// accumulation, BF16 out; with rows2, each term is w_j * (rows + rows2) of
// that sorted row (the two added in fp32 first).  Grid (T, column blocks):
// each thread owns 8 columns of one token and issues its k row loads
// together; a block spans a whole row (up to 1024 threads).
__global__ __launch_bounds__(1024) void k_combine(const uint16_t* __restrict__ rows,
                                                 const uint16_t* __restrict__ rows2, int d,
                                                 const int32_t* __restrict__ inv_perm,
                                                 const float* __restrict__ gates, int k,
                                                 uint16_t* __restrict__ out) {
  const int64_t t = blockIdx.x;
  const int c = blockIdx.y * blockDim.x + threadIdx.x;   // 8-column chunk
  if (c >= d / 8) return;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  constexpr int kB = 8;   // loads in flight per batch
  for (int j0 = 0; j0 < k; j0 += kB) {
    u32x4_t v[kB];
    float w[kB];
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const int j = j0 + b;
      const int src = j < k ? inv_perm[t * k + j] : -1;
      w[b] = src < 0 ? 0.f : (gates ? gates[t * k + j] : 1.0f);
      // each routed row is read once: non-temporal loads keep it out of the caches
      v[b] = src < 0 ? u32x4_t{0u, 0u, 0u, 0u}
                     : __builtin_nontemporal_load(
                           reinterpret_cast<const u32x4_t*>(rows + (int64_t)src * d) + c);
    }
    if (rows2) {
      u32x4_t v2[kB];
#pragma unroll
      for (int b = 0; b < kB; ++b) {
        const int j = j0 + b;
        const int src = j < k ? inv_perm[t * k + j] : -1;
        v2[b] = src < 0 ? u32x4_t{0u, 0u, 0u, 0u}
                        : reinterpret_cast<const u32x4_t*>(rows2 + (int64_t)src * d)[c];
      }
#pragma unroll
      for (int b = 0; b < kB; ++b) {
        if (j0 + b >= k) break;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float lo = bf16_to_f32(v[b][i] & 0xFFFFu) + bf16_to_f32(v2[b][i] & 0xFFFFu);
          const float hi = bf16_to_f32(v[b][i] >> 16) + bf16_to_f32(v2[b][i] >> 16);
          acc[2 * i] = __builtin_fmaf(w[b], lo, acc[2 * i]);
          acc[2 * i + 1] = __builtin_fmaf(w[b], hi, acc[2 * i + 1]);
        }
      }
      continue;
    }
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      if (j0 + b >= k) break;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = __builtin_fmaf(w[b], bf16_to_f32(v[b][i] & 0xFFFFu), acc[2 * i]);
        acc[2 * i + 1] = __builtin_fmaf(w[b], bf16_to_f32(v[b][i] >> 16), acc[2 * i + 1]);
      }
    }
  }
  u32x4_t o = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
               pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
  __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(out + t * d) + c);
}

// Scale validation for the fused decoder: an INT4 group whose BF16 scale is
// +-Inf or has magnitude >= 2^119 (exponent field 246..255 without NaN, i.e.
// |bits| in [0x7B00, 0x7F80]) sets bit 4 of *err.  The fused INT4 decode
// forms q * s as fma(n' 2^-9, 512 s, -8 s), which needs 512 s finite; NaN
// scales decode to NaN on both variants and are not flagged.  MXFP4 scale
// codes all decode exactly on both variants.
__global__ __launch_bounds__(256) void k_check_scales_int4(const uint16_t* __restrict__ scales,
                                                           int64_t n, int32_t* __restrict__ err) {
  bool bad = false;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t m = scales[i] & 0x7FFFu;
    bad |= m >= 0x7B00u && m <= 0x7F80u;
  }
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(err, 4);
}

}  // namespace

hipError_t launch_check_scales(int fmt, const void* scales, int64_t n, int32_t* err,
                               hipStream_t s) {
  TimedLaunch timed_(kLOther, s);
  if (fmt != 2 || n <= 0) return hipSuccess;
  const dim3 grid((unsigned)std::min<int64_t>((n + 255) / 256, (int64_t)num_cus() * 8));
  hipLaunchKernelGGL(k_check_scales_int4, grid, dim3(256), 0, s,
                     static_cast<const uint16_t*>(scales), n, err);
  return hipGetLastError();
}

hipError_t launch_dequant(int fmt, const uint8_t* packed, const void* scales, int layout, int N,
                          int K, const int32_t* active, const int32_t* n_active, int first,
                          int count, bool tiled_out, uint16_t* dst, hipStream_t s) {
  TimedLaunch timed_(kLDequant, s);
  const int64_t groups = (int64_t)count * N * (K / 32);
  if (groups <= 0) return hipSuccess;
  const dim3 grid((unsigned)std::min<int64_t>((groups + 255) / 256, (int64_t)num_cus() * 32));
  if (fmt == 1)
    hipLaunchKernelGGL(k_dequant<1>, grid, dim3(256), 0, s, packed, scales, layout, N, K, active,
                       n_active, first, count, tiled_out ? 1 : 0, dst);
  else
    hipLaunchKernelGGL(k_dequant<2>, grid, dim3(256), 0, s, packed, scales, layout, N, K, active,
                       n_active, first, count, tiled_out ? 1 : 0, dst);
  return hipGetLastError();
}

hipError_t launch_repack(int fmt, const uint8_t* packed, const void* scales, int E, int N, int K,
                         uint8_t* packed_out, void* scales_out, hipStream_t s) {
  TimedLaunch timed_(kLOther, s);
  const int64_t total = (int64_t)E * N * (K / 32);
  if (total <= 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 255) / 256));
  const uint8_t* sc = static_cast<const uint8_t*>(scales);
  uint8_t* so = static_cast<uint8_t*>(scales_out);
  if (fmt == 1)
    hipLaunchKernelGGL(k_repack<1>, grid, dim3(256), 0, s, packed, sc, E, N, K, packed_out, so);
  else
    hipLaunchKernelGGL(k_repack<2>, grid, dim3(256), 0, s, packed, sc, E, N, K, packed_out, so);
  return hipGetLastError();
}

hipError_t launch_combine(const uint16_t* rows, int d, const int32_t* inv_perm,
                          const float* gates, int T, int k, uint16_t* out, hipStream_t s,
                          const uint16_t* rows2) {
  TimedLaunch timed_(kLCombine, s);
  if (T == 0) return hipSuccess;
  const int chunks = d / 8;
  const int ny = (chunks + 1023) / 1024;
  const int threads = ((chunks + ny - 1) / ny + 63) / 64 * 64;
  hipLaunchKernelGGL(k_combine, dim3(T, ny), dim3(threads), 0, s, rows, rows2, d, inv_perm, gates,
                     k, out);
  return hipGetLastError();
}

// a[i][c] = silu(h[i][c]) * h[i][inter + c] for the sorted rows i < offsets[E]
// (BF16 in and out, fp32 arithmetic): the SwiGLU output recomputed from the
// saved h.  One thread per 8 columns.
__global__ __launch_bounds__(256) void k_swiglu_act(const uint16_t* __restrict__ h, int inter,
                                                    const int32_t* __restrict__ nrows_p,
                                                    uint16_t* __restrict__ a) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int per = inter / 8;
  const int64_t i = q / per;
  const int c = (int)(q % per) * 8;
  if (i >= *nrows_p) return;
  const u32x4_t g = *reinterpret_cast<const u32x4_t*>(h + i * 2 * inter + c);
  const u32x4_t u = *reinterpret_cast<const u32x4_t*>(h + i * 2 * inter + inter + c);
  uint32_t o[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float g0 = bf16_to_f32(g[w] & 0xFFFFu), g1 = bf16_to_f32(g[w] >> 16);
    const float u0 = bf16_to_f32(u[w] & 0xFFFFu), u1 = bf16_to_f32(u[w] >> 16);
    o[w] = pack_bf16x2(silu_f32(g0) * u0, silu_f32(g1) * u1);
  }
  *reinterpret_cast<u32x4_t*>(a + i * inter + c) = u32x4_t{o[0], o[1], o[2], o[3]};
}

hipError_t launch_swiglu_act(const uint16_t* h, int inter, const int32_t* offsets, int E,
                             int64_t P, uint16_t* a, hipStream_t s) {
  TimedLaunch timed_(kLOther, s);
  const int64_t n = P * (inter / 8);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_swiglu_act, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, h, inter,
                     offsets + E, a);
  return hipGetLastError();
}

}  // namespace qgg
