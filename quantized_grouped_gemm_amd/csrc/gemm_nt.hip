// Grouped GEMM y = a . W_e^T over the routed rows of each expert, with the
// expert weights either 4-bit (decoded in registers: the fused variant) or
// BF16 (a dequantized chunk in scratch: the chunked variant).
//
// Orbit page, section 时刻细节 ("Active-expert-chunked dequantization"): the
// router-selected experts run as one grouped matrix multiplication over BF16
// weights.  Group-32 scales along K follow "超大规模开放权重模型技术解析",
// 三 微缩放量化的原理.
//
// Work decomposition (gfx950, 64-wide wavefronts, v_mfma_f32_32x32x16_bf16):
//  - a work item is (M-tile of up to 32*MB rows of one expert, 256 output
//    columns); a persistent grid walks the items, split into 8 contiguous
//    ranges so that each XCD (blocks are dealt round-robin to the 8 XCDs)
//    works on neighbouring items that share A rows and weights in its L2;
//  - 4 wavefronts per workgroup, each owning 64 output columns (two 32-column
//    MFMA blocks) for all rows of the tile, so each weight element is loaded
//    and decoded exactly once per tile;
//  - weights go from HBM straight into MFMA B-operand registers: lane (c, h)
//    of a column block loads the 16 bytes of one 32-element scale group of
//    W row c (group 2s+h of a 64-wide K step), decodes 8 elements per MFMA;
//    the K order inside an MFMA is permuted identically for A and B, which
//    leaves each dot product unchanged;
//  - activation rows (gathered through perm when they are token-ordered) are
//    staged through double-buffered LDS, 128 K elements per stage.
#include "qgg_device.hpp"
#include "qgg_internal.hpp"

namespace qgg {

namespace {

constexpr int kKL = 128;                 // K elements per LDS stage
constexpr int kRowB = kKL * 2 + 16;      // padded LDS bytes per A row
constexpr int kCPR = kKL * 2 / 16;       // 16-byte chunks per row per stage

__device__ __forceinline__ uint16_t bf16_hw(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}

template <int SRC>
struct BRegs {
  u32x4_t w[SRC == kSrcBF16 ? 4 : 1];
  float s, neg8s;
};

template <int SRC>
__device__ __forceinline__ void load_b(const GemmArgs& g, const uint8_t* wp, const uint8_t* sp,
                                       const uint16_t* wb, int group, BRegs<SRC>& r) {
  if constexpr (SRC == kSrcBF16) {
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(wb + group * 32);
#pragma unroll
    for (int s = 0; s < 4; ++s) r.w[s] = src[s];
  } else {
    r.w[0] = *reinterpret_cast<const u32x4_t*>(wp + group * 16);
    if constexpr (SRC == kSrcMXFP4) {
      r.s = e8m0_to_f32(sp[group]);
    } else {
      r.s = bf16_to_f32(reinterpret_cast<const uint16_t*>(sp)[group]);
      r.neg8s = -8.0f * r.s;
    }
  }
}

// MFMA B operand for K step s (8 elements) of a loaded group.
template <int SRC>
__device__ __forceinline__ bf16x8_t b_operand(const BRegs<SRC>& r, int s) {
  uint32_t o[4];
  if constexpr (SRC == kSrcBF16) {
    return __builtin_bit_cast(bf16x8_t, r.w[s]);
  } else if constexpr (SRC == kSrcMXFP4) {
    dq8_mxfp4(r.w[0][s], r.s, o);
  } else {
    dq8_int4(r.w[0][s], r.s, r.neg8s, o);
  }
  u32x4_t v = {o[0], o[1], o[2], o[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

template <int SRC, int MB, int EPI, int AMODE>
__global__ __launch_bounds__(256, MB == 4 ? 1 : 2) void k_gemm_nt(GemmArgs g) {
  constexpr int MT = 32 * MB;
  constexpr int NCH = MT * kCPR / 256;   // A chunks per thread per stage
  __shared__ __attribute__((aligned(16))) uint8_t As[2][MT * kRowB];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;
  const int t_begin = g.range[0];
  const int t_end = g.range[1];
  const int n_tiles_n = EPI == kEpiSwiGLU ? (g.inter + 127) / 128 : (g.N + 255) / 256;
  const int items = (t_end - t_begin) * n_tiles_n;
  const int per_xcd = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7;
  const int span = (items + 7) >> 3;
  const int q_end = min(items, (xcd + 1) * span);
  const int nstages = g.K / kKL;
  const int64_t rowbytes = g.K / 2;
  const int64_t rowscales = g.K / 32;

  for (int q = xcd * span + (blockIdx.x >> 3); q < q_end; q += per_xcd) {
    const int4 tile = g.tiles[t_begin + q / n_tiles_n];
    const int nt = q % n_tiles_n;
    const int expert = tile.x, row0 = tile.y, nrows = tile.z;

    // A sources and LDS destinations of this thread's 16-byte chunks
    const uint16_t* asrc[NCH];
    int adst[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + 256 * i;
      const int r = c / kCPR;
      const int cc = c % kCPR;
      const int rr = r < nrows ? r : 0;
      int64_t srow;
      if constexpr (AMODE == kATokens) srow = g.perm[row0 + rr] / g.topk;
      else srow = row0 + rr;
      asrc[i] = g.a + srow * g.lda + cc * 8;
      adst[i] = r * kRowB + cc * 16;
    }

    // this wave's two 32-column blocks (W rows)
    int wrow0, wrow1;
    bool active;
    if constexpr (EPI == kEpiSwiGLU) {
      const int base = nt * 128 + wave * 32;
      active = base < g.inter;
      wrow0 = base + col;
      wrow1 = g.inter + base + col;
    } else {
      const int base = nt * 256 + wave * 64;
      active = base < g.N;
      wrow0 = base + col;
      wrow1 = base + 32 + col;
    }
    const uint8_t *wp0 = nullptr, *wp1 = nullptr, *sp0 = nullptr, *sp1 = nullptr;
    const uint16_t *wb0 = nullptr, *wb1 = nullptr;
    if constexpr (SRC == kSrcBF16) {
      const int64_t slot = tile.w - g.bf16_slot_base;
      wb0 = g.wbf16 + (slot * g.N + wrow0) * (int64_t)g.K;
      wb1 = g.wbf16 + (slot * g.N + wrow1) * (int64_t)g.K;
    } else {
      const int sb = SRC == kSrcMXFP4 ? 1 : 2;
      wp0 = g.packed + ((int64_t)expert * g.N + wrow0) * rowbytes;
      wp1 = g.packed + ((int64_t)expert * g.N + wrow1) * rowbytes;
      sp0 = static_cast<const uint8_t*>(g.scales) + ((int64_t)expert * g.N + wrow0) * rowscales * sb;
      sp1 = static_cast<const uint8_t*>(g.scales) + ((int64_t)expert * g.N + wrow1) * rowscales * sb;
    }

    f32x16_t acc[MB][2];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;
      }
    }

    BRegs<SRC> bcur0, bcur1, bnxt0, bnxt1;
    if (active) {
      load_b<SRC>(g, wp0, sp0, wb0, half, bcur0);
      load_b<SRC>(g, wp1, sp1, wb1, half, bcur1);
    }
    u32x4_t areg[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) areg[i] = *reinterpret_cast<const u32x4_t*>(asrc[i]);
#pragma unroll
    for (int i = 0; i < NCH; ++i) *reinterpret_cast<u32x4_t*>(&As[0][adst[i]]) = areg[i];
    __syncthreads();

    for (int st = 0; st < nstages; ++st) {
      const int buf = st & 1;
      if (st + 1 < nstages) {
#pragma unroll
        for (int i = 0; i < NCH; ++i)
          areg[i] = *reinterpret_cast<const u32x4_t*>(asrc[i] + (st + 1) * kKL);
      }
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const int step = st * 2 + sub;  // 64-wide K step
        if (active) {
          if (step + 1 < nstages * 2) {
            load_b<SRC>(g, wp0, sp0, wb0, (step + 1) * 2 + half, bnxt0);
            load_b<SRC>(g, wp1, sp1, wb1, (step + 1) * 2 + half, bnxt1);
          }
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const bf16x8_t b0 = b_operand<SRC>(bcur0, s);
            const bf16x8_t b1 = b_operand<SRC>(bcur1, s);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
              if (mb * 32 < nrows) {
                const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
                    &As[buf][(mb * 32 + col) * kRowB + (sub * 64 + half * 32 + s * 8) * 2]);
                acc[mb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, acc[mb][0], 0, 0, 0);
                acc[mb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, acc[mb][1], 0, 0, 0);
              }
            }
          }
          bcur0 = bnxt0;
          bcur1 = bnxt1;
        }
      }
      if (st + 1 < nstages) {
#pragma unroll
        for (int i = 0; i < NCH; ++i)
          *reinterpret_cast<u32x4_t*>(&As[buf ^ 1][adst[i]]) = areg[i];
      }
      __syncthreads();
    }

    if (!active) continue;
    // epilogue: lane holds column `col` of rows 8i + 4*half + j of each block
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (mb * 32 >= nrows) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = mb * 32 + 8 * i + 4 * half + j;
          if (r >= nrows) continue;
          const int64_t orow = row0 + r;
          const float v0 = acc[mb][0][i * 4 + j];
          const float v1 = acc[mb][1][i * 4 + j];
          if constexpr (EPI == kEpiSwiGLU) {
            const int c = wrow0;  // gate column in [0, inter)
            g.y[orow * g.ldy + c] = bf16_hw(silu_f32(v0) * v1);
            if (g.h) {
              g.h[orow * 2 * g.inter + c] = bf16_hw(v0);
              g.h[orow * 2 * g.inter + g.inter + c] = bf16_hw(v1);
            }
          } else {
            g.y[orow * g.ldy + wrow0] = bf16_hw(v0);
            g.y[orow * g.ldy + wrow1] = bf16_hw(v1);
          }
        }
      }
    }
  }
}

template <int SRC, int MB, int EPI, int AMODE>
hipError_t launch_nt_t(const GemmArgs& g, hipStream_t s) {
  const int n_tiles_n = EPI == kEpiSwiGLU ? (g.inter + 127) / 128 : (g.N + 255) / 256;
  const int64_t bound = (int64_t)g.max_tiles * n_tiles_n;
  if (bound <= 0) return hipSuccess;
  int64_t grid = std::min<int64_t>(bound, (int64_t)num_cus() * (MB == 4 ? 1 : 2));
  grid = (grid + 7) / 8 * 8;
  hipLaunchKernelGGL((k_gemm_nt<SRC, MB, EPI, AMODE>), dim3((unsigned)grid), dim3(256), 0, s, g);
  return hipGetLastError();
}

template <int SRC, int MB>
hipError_t launch_nt_e(const GemmArgs& g, hipStream_t s) {
  if (g.epi == kEpiSwiGLU) {
    return g.amode == kATokens ? launch_nt_t<SRC, MB, kEpiSwiGLU, kATokens>(g, s)
                               : launch_nt_t<SRC, MB, kEpiSwiGLU, kASorted>(g, s);
  }
  return g.amode == kATokens ? launch_nt_t<SRC, MB, kEpiStore, kATokens>(g, s)
                             : launch_nt_t<SRC, MB, kEpiStore, kASorted>(g, s);
}

template <int SRC>
hipError_t launch_nt_m(const GemmArgs& g, int MB, hipStream_t s) {
  switch (MB) {
    case 1: return launch_nt_e<SRC, 1>(g, s);
    case 2: return launch_nt_e<SRC, 2>(g, s);
    default: return launch_nt_e<SRC, 4>(g, s);
  }
}

}  // namespace

hipError_t launch_gemm_nt(const GemmArgs& g, int MB, hipStream_t s) {
  switch (g.src) {
    case kSrcBF16: return launch_nt_m<kSrcBF16>(g, MB, s);
    case kSrcMXFP4: return launch_nt_m<kSrcMXFP4>(g, MB, s);
    default: return launch_nt_m<kSrcINT4>(g, MB, s);
  }
}

}  // namespace qgg
