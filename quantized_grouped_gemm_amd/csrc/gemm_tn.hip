// Grouped GEMM y = a . W_e over the routed rows of each expert (reduction over
// W's rows), the transposed access that the input-gradient backward needs.
//
// Orbit page, section 时刻细节: the backward through the frozen base forms
// only the input gradient (bypass-base-weight-grad GEMM backward), so the
// weights are read transposed: dA = dO . W_down and dXp = dH . W_gate_up,
// with the group-32 scales running along W's K index (the output columns
// here), not along the reduction.
//
// Work decomposition: as the forward kernel (persistent grid, XCD-contiguous
// item ranges, 4 wavefronts x 64 output columns, v_mfma_f32_32x32x16_bf16),
// but both operands are staged through double-buffered LDS, 32 reduction
// rows per stage.  Each stage's weight tile (32 W rows x 256 columns) is
// loaded once per workgroup with each thread taking two adjacent rows and 16
// columns; the decoded values are paired row-wise with v_perm_b32 and written
// column-major, so a B operand (8 consecutive reduction rows of one column) is
// one 16-byte LDS read.  The SwiGLU-backward epilogue applies the gate and the
// SwiGLU derivative from the saved forward activations.
#include "qgg_device.hpp"
#include "qgg_internal.hpp"

#include <type_traits>

namespace qgg {

namespace {

constexpr int kKR = 32;               // reduction rows per stage
constexpr int kRowBT = kKR * 2 + 16;  // padded LDS bytes per row (A) / column (B)
// B columns get an extra 64 bytes every 16 columns so that the 64 lanes of a
// wavefront writing (row pair, column) words hit 64 distinct banks.
constexpr int kBsBytes = 256 * kRowBT + 16 * 64;
__device__ __forceinline__ int bcol(int c) { return c * kRowBT + (c >> 4) * 64; }

__device__ __forceinline__ uint16_t bf16_hw_t(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}

template <int SRC>
struct BStage {
  // two W rows, 16 columns each
  uint32_t p[SRC == kSrcBF16 ? 16 : 4];
  uint32_t sraw0, sraw1;   // raw scale bits, converted when decoding
};

template <int SRC>
__device__ __forceinline__ void load_bt(const GemmArgs& g, int64_t slot_or_expert, int r,
                                        int c, BStage<SRC>& b) {
  // rows r, r+1 of W (reduction index), columns c..c+15 (W's K index)
  // element (n, k) of an MFMA-tiled tensor: tile (n / 32, k / 64), slot
  // 32 * ((k % 64) / 32) + n % 32; rows r and r + 1 are adjacent slots
  const int64_t cb = r >> 5;
  const int64_t j = c >> 6;
  const int lslot = ((c & 63) >> 5) * 32 + (r & 31);
  const int64_t tile = (slot_or_expert * (g.N / 32) + cb) * (g.K / 64) + j;
  if constexpr (SRC == kSrcBF16) {
    // 16 consecutive k = the pieces s0 and s0 + 1 (8 elements each)
    const int s0 = (c & 31) >> 3;
    const uint8_t* base = reinterpret_cast<const uint8_t*>(g.wbf16) + tile * 4096;
    const u32x4_t x0 = *reinterpret_cast<const u32x4_t*>(base + (s0 * 64 + lslot) * 16);
    const u32x4_t x1 = *reinterpret_cast<const u32x4_t*>(base + ((s0 + 1) * 64 + lslot) * 16);
    const u32x4_t y0 = *reinterpret_cast<const u32x4_t*>(base + (s0 * 64 + lslot + 1) * 16);
    const u32x4_t y1 = *reinterpret_cast<const u32x4_t*>(base + ((s0 + 1) * 64 + lslot + 1) * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      b.p[i] = x0[i];
      b.p[4 + i] = x1[i];
      b.p[8 + i] = y0[i];
      b.p[12 + i] = y1[i];
    }
  } else {
    const int sbytes = SRC == kSrcMXFP4 ? 1 : 2;
    const uint8_t* sp = static_cast<const uint8_t*>(g.scales);
    const uint8_t* w0;
    int64_t wnext, si, snext;
    if (g.layout == 1) {
      w0 = g.packed + (tile * 64 + lslot) * 16 + ((c & 31) >> 1);
      wnext = 16;
      si = tile * 64 + lslot;
      snext = 1;
    } else {
      const int64_t rowbytes = g.K / 2;
      w0 = g.packed + (slot_or_expert * g.N + r) * rowbytes + c / 2;
      wnext = rowbytes;
      si = (slot_or_expert * g.N + r) * (int64_t)(g.K / 32) + c / 32;
      snext = g.K / 32;
    }
    const uint2 x = *reinterpret_cast<const uint2*>(w0);
    const uint2 y = *reinterpret_cast<const uint2*>(w0 + wnext);
    b.p[0] = x.x;
    b.p[1] = x.y;
    b.p[2] = y.x;
    b.p[3] = y.y;
    if constexpr (SRC == kSrcMXFP4) {
      b.sraw0 = sp[si];
      b.sraw1 = sp[si + snext];
    } else {
      const uint16_t* sp16 = reinterpret_cast<const uint16_t*>(sp);
      b.sraw0 = sp16[si];
      b.sraw1 = sp16[si + snext];
    }
    (void)sbytes;
  }
}

// Decode both rows to BF16 pairs, interleave row-wise per column and store
// column-major: Bs[col][r..r+1].
template <int SRC>
__device__ __forceinline__ void store_bt(const BStage<SRC>& b, uint8_t* Bs, int cl, int rp) {
  uint32_t r0[8], r1[8];
  if constexpr (SRC == kSrcBF16) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      r0[i] = b.p[i];
      r1[i] = b.p[8 + i];
    }
  } else if constexpr (SRC == kSrcMXFP4) {
    const float s0 = e8m0_to_f32(b.sraw0), s1 = e8m0_to_f32(b.sraw1);
    dq8_mxfp4(b.p[0], s0, r0);
    dq8_mxfp4(b.p[1], s0, r0 + 4);
    dq8_mxfp4(b.p[2], s1, r1);
    dq8_mxfp4(b.p[3], s1, r1 + 4);
  } else {
    const float s0 = bf16_to_f32(b.sraw0), s1 = bf16_to_f32(b.sraw1);
    const float n0 = -8.0f * s0, n1 = -8.0f * s1;
    const float m0 = 512.0f * s0, m1 = 512.0f * s1;
    dq8_int4(b.p[0], m0, n0, r0);
    dq8_int4(b.p[1], m0, n0, r0 + 4);
    dq8_int4(b.p[2], m1, n1, r1);
    dq8_int4(b.p[3], m1, n1, r1 + 4);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // column 2i: low halves; column 2i+1: high halves
    const uint32_t lo = __builtin_amdgcn_perm(r1[i], r0[i], 0x05040100u);
    const uint32_t hi = __builtin_amdgcn_perm(r1[i], r0[i], 0x07060302u);
    *reinterpret_cast<uint32_t*>(Bs + bcol(cl + 2 * i) + rp * 4) = lo;
    *reinterpret_cast<uint32_t*>(Bs + bcol(cl + 2 * i + 1) + rp * 4) = hi;
  }
}

// One work item: tile (rows [row0, row0 + nrows) of one expert) x 256 output
// columns starting at c0, NMB live 32-row blocks.  Branch-free like the
// forward kernel: out-of-range loads are clamped, the weight stages come
// through a two-deep register ring, the LDS buffer parity is static.
template <int SRC, int MB, int EPI, int AMODE, int NMB>
__device__ __forceinline__ void gemm_tn_item(const GemmArgs& g, uint8_t (*As)[32 * MB * kRowBT],
                                             uint8_t (*Bs)[kBsBytes], int4 tile, int c0) {
  constexpr int MT = 32 * MB;
  constexpr int ACH = MT * 4;                    // 16-byte A chunks per stage
  constexpr int NCH = (ACH + 255) / 256;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;
  const int nstages = g.N / kKR;
  const int row0 = tile.y, nrows = tile.z;
  const int64_t wsel = SRC == kSrcBF16 ? (int64_t)(tile.w - g.bf16_slot_base) : tile.x;
  // B loader role: rows 2*rp, 2*rp+1 of the stage, columns 16*bq .. +15
  // (columns past K are clamped; only idle wavefronts would read them)
  const int rp = tid & 15;
  const int bq = tid >> 4;
  const int bcol0 = min(c0 + 16 * bq, g.K - 16);

  // A chunks: when a stage has fewer chunks than threads (MB == 1), the
  // spare threads repeat a chunk, writing the same bytes to the same place
  const uint16_t* asrc[NCH];
  int adst[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = (tid + 256 * i) % ACH;
    const int r = c >> 2;
    const int cc = c & 3;
    const int rr = r < nrows ? r : 0;
    int64_t srow;
    if constexpr (AMODE == kATokens) srow = g.perm[row0 + rr] / g.topk;
    else srow = row0 + rr;
    asrc[i] = g.a + srow * g.lda + cc * 8;
    adst[i] = r * kRowBT + cc * 16;
  }
  const int wbase = c0 + wave * 64;
  const bool active = wbase < g.K;

  f32x16_t acc[NMB][2];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;

  BStage<SRC> ring[2];
  load_bt<SRC>(g, wsel, 2 * rp, bcol0, ring[0]);
  load_bt<SRC>(g, wsel, (nstages > 1 ? kKR : 0) + 2 * rp, bcol0, ring[1]);
  u32x4_t areg[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) areg[i] = *reinterpret_cast<const u32x4_t*>(asrc[i]);
  store_bt<SRC>(ring[0], Bs[0], 16 * bq, rp);
  load_bt<SRC>(g, wsel, (nstages > 2 ? 2 * kKR : 0) + 2 * rp, bcol0, ring[0]);
#pragma unroll
  for (int i = 0; i < NCH; ++i) *reinterpret_cast<u32x4_t*>(&As[0][adst[i]]) = areg[i];
  __syncthreads();

  // stage st computes from buffer BUF while the ring slot holding stage st+1
  // is decoded into the other buffer and refilled with stage st+3
  auto kstage = [&](int st, BStage<SRC>& nxt, auto buf_c) {
    constexpr int BUF = decltype(buf_c)::value;
    const int s1 = st + 1 < nstages ? st + 1 : st;
#pragma unroll
    for (int i = 0; i < NCH; ++i)
      areg[i] = *reinterpret_cast<const u32x4_t*>(asrc[i] + s1 * kKR);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8_t b0 = *reinterpret_cast<const bf16x8_t*>(
          &Bs[BUF][bcol(wave * 64 + col) + (16 * s + 8 * half) * 2]);
      const bf16x8_t b1 = *reinterpret_cast<const bf16x8_t*>(
          &Bs[BUF][bcol(wave * 64 + 32 + col) + (16 * s + 8 * half) * 2]);
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
            &As[BUF][(mb * 32 + col) * kRowBT + (16 * s + 8 * half) * 2]);
        acc[mb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, acc[mb][0], 0, 0, 0);
        acc[mb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, acc[mb][1], 0, 0, 0);
      }
    }
    store_bt<SRC>(nxt, Bs[BUF ^ 1], 16 * bq, rp);
    {
      const int s3 = st + 3 < nstages ? st + 3 : nstages - 1;
      load_bt<SRC>(g, wsel, s3 * kKR + 2 * rp, bcol0, nxt);
    }
#pragma unroll
    for (int i = 0; i < NCH; ++i) *reinterpret_cast<u32x4_t*>(&As[BUF ^ 1][adst[i]]) = areg[i];
    __syncthreads();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  // on entry ring[1] holds stage 1 and ring[0] stage 2; stage st + 1 lives
  // in ring[(st + 1) & 1]
  int st = 0;
  for (; st + 2 <= nstages; st += 2) {
    kstage(st, ring[1], I0{});
    kstage(st + 1, ring[0], I1{});
  }
  if (st < nstages) kstage(st, ring[1], I0{});

  if (!active) return;
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = mb * 32 + 8 * i + 4 * half + j;
        if (r < nrows) {
          const int64_t orow = row0 + r;
          float gate = 1.f;
          if constexpr (EPI == kEpiSwiGLUBwd) gate = g.gates[g.perm[orow]];
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const int c = wbase + nb * 32 + col;
            const float v = acc[mb][nb][i * 4 + j];
            if constexpr (EPI == kEpiSwiGLUBwd) {
              // v = (dY . W_down)[c]; dA = g * v; h_saved holds [gate | up]
              const float da = gate * v;
              const int64_t hb = orow * 2 * (int64_t)g.inter;
              const float hg = bf16_to_f32(g.h[hb + c]);
              const float hu = bf16_to_f32(g.h[hb + g.inter + c]);
              const float sg = 1.0f / (1.0f + __expf(-hg));
              const float dsilu = sg * (1.0f + hg * (1.0f - sg));
              g.y[orow * g.ldy + c] = bf16_hw_t(da * hu * dsilu);
              g.y[orow * g.ldy + g.inter + c] = bf16_hw_t(da * hg * sg);
            } else {
              g.y[orow * g.ldy + c] = bf16_hw_t(v);
            }
          }
        }
      }
    }
  }
}

template <int SRC, int MB, int EPI, int AMODE>
__global__ __launch_bounds__(256, MB == 4 ? 1 : 2) void k_gemm_tn(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t As[2][32 * MB * kRowBT];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][kBsBytes];
  const int t_begin = g.range[0];
  const int t_end = g.range[1];
  const int n_tiles_n = (g.K + 255) / 256;      // output columns = W's K index
  const int items = (t_end - t_begin) * n_tiles_n;
  const int per_xcd = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7;
  const int span = (items + 7) >> 3;
  const int q_end = min(items, (xcd + 1) * span);
  for (int q = xcd * span + (blockIdx.x >> 3); q < q_end; q += per_xcd) {
    const int4 tile = g.tiles[t_begin + q / n_tiles_n];
    const int c0 = (q % n_tiles_n) * 256;
    const int nmb = (tile.z + 31) / 32;
    if (MB == 1 || nmb <= 1) {
      gemm_tn_item<SRC, MB, EPI, AMODE, 1>(g, As, Bs, tile, c0);
    } else if (MB == 2 || nmb == 2) {
      gemm_tn_item<SRC, MB, EPI, AMODE, (MB >= 2 ? 2 : 1)>(g, As, Bs, tile, c0);
    } else if (nmb == 3) {
      gemm_tn_item<SRC, MB, EPI, AMODE, (MB >= 4 ? 3 : 1)>(g, As, Bs, tile, c0);
    } else {
      gemm_tn_item<SRC, MB, EPI, AMODE, (MB >= 4 ? 4 : 1)>(g, As, Bs, tile, c0);
    }
  }
}

template <int SRC, int MB, int EPI, int AMODE>
hipError_t launch_tn_t(const GemmArgs& g, hipStream_t s) {
  const int n_tiles_n = (g.K + 255) / 256;
  const int64_t bound = (int64_t)g.max_tiles * n_tiles_n;
  if (bound <= 0) return hipSuccess;
  int64_t grid = std::min<int64_t>(bound, (int64_t)num_cus() * (MB == 4 ? 1 : 2));
  grid = (grid + 7) / 8 * 8;
  hipLaunchKernelGGL((k_gemm_tn<SRC, MB, EPI, AMODE>), dim3((unsigned)grid), dim3(256), 0, s, g);
  return hipGetLastError();
}

template <int SRC, int MB>
hipError_t launch_tn_e(const GemmArgs& g, hipStream_t s) {
  if (g.epi == kEpiSwiGLUBwd) {
    return g.amode == kATokens ? launch_tn_t<SRC, MB, kEpiSwiGLUBwd, kATokens>(g, s)
                               : launch_tn_t<SRC, MB, kEpiSwiGLUBwd, kASorted>(g, s);
  }
  return g.amode == kATokens ? launch_tn_t<SRC, MB, kEpiStore, kATokens>(g, s)
                             : launch_tn_t<SRC, MB, kEpiStore, kASorted>(g, s);
}

template <int SRC>
hipError_t launch_tn_m(const GemmArgs& g, int MB, hipStream_t s) {
  switch (MB) {
    case 1: return launch_tn_e<SRC, 1>(g, s);
    case 2: return launch_tn_e<SRC, 2>(g, s);
    default: return launch_tn_e<SRC, 4>(g, s);
  }
}

}  // namespace

hipError_t launch_gemm_tn(const GemmArgs& g, int MB, hipStream_t s) {
  switch (g.src) {
    case kSrcBF16: return launch_tn_m<kSrcBF16>(g, MB, s);
    case kSrcMXFP4: return launch_tn_m<kSrcMXFP4>(g, MB, s);
    default: return launch_tn_m<kSrcINT4>(g, MB, s);
  }
}

}  // namespace qgg
