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
//  - a work item is (M-tile of up to 32*MB rows of one expert, 64*NW output
//    columns); a persistent grid starts on items 0 .. grid - 1 and takes the
//    rest in order from a counter, so the columns of one M-tile run side by
//    side and a workgroup that drew small tiles takes more of them;
//  - NW wavefronts per workgroup (8 for 128-row tiles, else 4), each owning 64
//    output columns (two 32-column MFMA blocks) for all rows of the tile, so
//    each weight element is loaded and decoded exactly once per tile;
//  - weights go from HBM straight into MFMA B-operand registers: lane (c, h)
//    of a column block loads the 16 bytes of one 32-element scale group of
//    W row c (group 2s+h of a 64-wide K step), decodes 8 elements per MFMA;
//    the K order inside an MFMA is permuted identically for A and B, which
//    leaves each dot product unchanged;
//  - activation rows (gathered through perm when they are token-ordered) are
//    staged through a ring of four LDS stage buffers, 64 K elements per stage.
#include "qgg_device.hpp"
#include "qgg_internal.hpp"

#include <type_traits>

namespace qgg {

namespace {

constexpr int kKL = 64;                  // K elements per stage (one K step)
constexpr int kStageRowB = kKL * 2;      // A bytes per tile row per stage
constexpr int kNBuf = 4;                 // stages in the LDS ring of A tiles
// Wavefronts per workgroup (each owns 64 output columns of an item) and
// workgroups per CU.  128-row tiles take 512-column items on eight waves:
// every A stage copied into LDS then feeds twice the columns, which halves
// the L2 -> LDS traffic of A.  Shorter tiles (decode-sized and mid-sized
// expert groups) need fewer registers and take 256-column items on four
// waves, three workgroups per CU for 32-row tiles and two for 64-row tiles,
// which keeps more weight loads in flight.
template <int MB>
constexpr int nt_waves() { return MB == 4 ? 8 : 4; }
template <int MB>
constexpr int nt_occupancy() { return MB == 1 ? 3 : (MB == 2 ? 2 : 1); }
// weight steps in flight per wavefront (BF16 steps are 4x larger)
template <int SRC>
constexpr int ring_depth() { return SRC == kSrcBF16 ? 2 : 4; }
// vector-memory instructions one stage issues to refill the weight ring
template <int SRC>
constexpr int b_loads_per_stage() { return SRC == kSrcBF16 ? 8 : 4; }

// A tiles in LDS: tile row r of a stage is 128 contiguous bytes whose eight
// 16-byte K chunks are permuted, chunk kc at slot kc ^ swz(r), so that an
// MFMA operand read (one chunk of 32 consecutive rows) hits distinct banks.
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

__device__ __forceinline__ uint16_t bf16_hw(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}

template <int SRC>
struct BRegs {
  u32x4_t w[SRC == kSrcBF16 ? 4 : 1];
  uint32_t sraw;   // raw scale bits; converted only when decoding, so a
                   // refill never waits for its own load
};

// Per-lane weight stream: buffer resources over one expert's (or BF16
// slot's) weight and scale bytes, this lane's byte offsets at K step 0, and
// the wave-uniform byte strides from one 64-wide K step to the next (so a
// step's address is a scalar add, and offsets past the slice read zeros).
struct BStream {
  __amdgpu_buffer_rsrc_t w, s;
  uint32_t wv, sv;
  int wstep, sstep;
};

template <int SRC>
__device__ __forceinline__ void load_b(const BStream& b, int step, BRegs<SRC>& r) {
  if constexpr (SRC == kSrcBF16) {
    // tiled BF16: the four 8-element pieces of a lane sit 1 KiB apart
#pragma unroll
    for (int s = 0; s < 4; ++s)
      r.w[s] = __builtin_amdgcn_raw_buffer_load_b128(b.w, b.wv + s * 1024, step * b.wstep, 0);
  } else {
    r.w[0] = __builtin_amdgcn_raw_buffer_load_b128(b.w, b.wv, step * b.wstep, 0);
    if constexpr (SRC == kSrcMXFP4)
      r.sraw = __builtin_amdgcn_raw_buffer_load_b8(b.s, b.sv, step * b.sstep, 0);
    else
      r.sraw = __builtin_amdgcn_raw_buffer_load_b16(b.s, b.sv, step * b.sstep, 0);
  }
}

// Stream of W rows 32 cb .. 32 cb + 31 (cb wave-uniform) for lane
// `lane` = 32 * half + col, which reads row 32 cb + col.
template <int SRC>
__device__ __forceinline__ BStream make_stream(const GemmArgs& g, int64_t expert_or_slot, int cb,
                                               int lane) {
  BStream b;
  const int nkt = g.K / 64;                    // K steps
  const int half = lane >> 5;
  const int col = lane & 31;
  if constexpr (SRC == kSrcBF16) {
    const uint32_t bytes = (uint32_t)g.N * (uint32_t)g.K * 2u;
    b.w = raw_buffer(reinterpret_cast<const uint8_t*>(g.wbf16) + expert_or_slot * bytes, bytes);
    b.s = b.w;
    b.wv = (uint32_t)(cb * nkt) * 4096u + lane * 16;
    b.wstep = 4096;
    b.sv = 0;
    b.sstep = 0;
  } else {
    const int sb = SRC == kSrcMXFP4 ? 1 : 2;
    const uint32_t wbytes = (uint32_t)g.N * (uint32_t)(g.K / 2);
    const uint32_t sbytes = (uint32_t)g.N * (uint32_t)(g.K / 32) * sb;
    b.w = raw_buffer(g.packed + expert_or_slot * wbytes, wbytes);
    b.s = raw_buffer(static_cast<const uint8_t*>(g.scales) + expert_or_slot * sbytes, sbytes);
    if (g.layout == 1) {   // MFMA-tiled: 1 KiB per (32 rows, 64 K) tile
      const uint32_t t0 = (uint32_t)(cb * nkt);
      b.wv = t0 * 1024u + lane * 16;
      b.wstep = 1024;
      b.sv = (t0 * 64u + lane) * sb;
      b.sstep = 64 * sb;
    } else {               // rows
      const uint32_t row = (uint32_t)(cb * 32 + col);
      b.wv = row * (uint32_t)(g.K / 2) + half * 16;
      b.wstep = 32;
      b.sv = (row * (uint32_t)(g.K / 32) + half) * sb;
      b.sstep = 2 * sb;
    }
  }
  return b;
}

// Scale of a loaded group in the form the decoder takes.
template <int SRC>
struct BScale {
  float s, neg8s;
};

template <int SRC>
__device__ __forceinline__ BScale<SRC> b_scale(const BRegs<SRC>& r) {
  BScale<SRC> o{0.f, 0.f};
  if constexpr (SRC == kSrcMXFP4) {
    o.s = e8m0_to_f32(r.sraw);
  } else if constexpr (SRC == kSrcINT4) {
    const float sc = bf16_to_f32(r.sraw);
    o.s = 512.0f * sc;
    o.neg8s = -8.0f * sc;
  }
  return o;
}

// MFMA B operand for K step s (8 elements) of a loaded group.
template <int SRC>
__device__ __forceinline__ bf16x8_t b_operand(const BRegs<SRC>& r, const BScale<SRC>& sc, int s) {
  uint32_t o[4];
  if constexpr (SRC == kSrcBF16) {
    return __builtin_bit_cast(bf16x8_t, r.w[s]);
  } else if constexpr (SRC == kSrcMXFP4) {
    dq8_mxfp4(r.w[0][s], sc.s, o);
  } else {
    dq8_int4(r.w[0][s], sc.s, sc.neg8s, o);
  }
  u32x4_t v = {o[0], o[1], o[2], o[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// One work item: tile (expert, rows [row0, row0 + nrows)) x 64 NW output
// columns, with NMB live 32-row blocks.  The K loop is branch-free: every
// load index is clamped into range instead of guarded, so the compiler keeps
// exact vmcnt counts.  Both operand streams run ahead of the MFMAs: the A
// tile is copied global -> LDS kNBuf - 1 stages ahead into a ring of kNBuf
// stage buffers, the weights ring_depth steps ahead into registers, and the
// stage barrier waits only for the copies of the next stage.
template <int SRC, int MB, int EPI, int AMODE, int NMB>
__device__ __forceinline__ void gemm_nt_item(const GemmArgs& g,
                                             const LdsRing4& As, int4 tile,
                                             int nt, int& next_q) {
  constexpr int kRing = ring_depth<SRC>();
  constexpr int kBL = b_loads_per_stage<SRC>();
  constexpr int NW = nt_waves<MB>();
  constexpr int kNCA = (256 * NMB + 64 * NW - 1) / (64 * NW);   // A copies per thread
  constexpr int kStageLoads = kNCA + kBL;           // vector-memory ops per stage
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;
  const int nsteps = g.K / kKL;
  const int expert = tile.x, row0 = tile.y, nrows = tile.z;

  // A copies: 16-byte slot p = 64 NW i + tid of a stage (i < kNCA; block mb
  // holds tile rows 32 mb .. 32 mb + 31) receives K chunk (p & 7) ^ swz(r) of
  // tile row r = p >> 3; rows past the tile's end copy its first row (with
  // NMB < MB the extra slots stay inside the MB-block stage buffer)
  // (byte offsets into the A buffer; the host keeps A under 4 GiB)
  const __amdgpu_buffer_rsrc_t arsrc = raw_buffer(g.a, (uint32_t)(g.a_rows * g.lda * 2));
  uint32_t aoffs[kNCA];
#pragma unroll
  for (int i = 0; i < kNCA; ++i) {
    const int p = 64 * NW * i + tid;
    const int r = p >> 3;
    const int kc = (p & 7) ^ swz(r);
    const int rr = r < nrows ? r : 0;
    int64_t srow;
    if constexpr (AMODE == kATokens) srow = g.perm[row0 + rr] / g.topk;
    else srow = row0 + rr;
    aoffs[i] = (uint32_t)((srow * g.lda + kc * 8) * 2);
  }
  auto copy_a = [&](int st, auto buf_c) {
    constexpr int BUF = decltype(buf_c)::value;
    const uint32_t soff = (uint32_t)((st < nsteps ? st : nsteps - 1) * kStageRowB);
#pragma unroll
    for (int i = 0; i < kNCA; ++i)
      copy16_to_lds(arsrc, aoffs[i], soff, As.b[BUF] + (64 * NW * i + 64 * wave) * 16);
  };
  // LDS offsets of this lane's A operand chunks (row col of a block, K chunk
  // 4 half + s): the chunk's slot is xb ^ c with c = s ^ 4 (mb & 1)
  const int xb = (half << 2) ^ swz(col);
  int aoff[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) aoff[c] = col * kStageRowB + ((xb ^ c) << 4);

  // this wave's two 32-column blocks (W rows 32 cb0.., 32 cb1..; wave-
  // uniform); a wave past the matrix edge computes on clamped rows and
  // stores nothing
  int cb0, cb1, ocol;
  bool active;
  if constexpr (EPI == kEpiSwiGLU) {
    const int base = nt * 32 * NW + wave * 32;
    active = base < g.inter;
    const int cbase = active ? base : g.inter - 32;
    ocol = cbase + col;
    cb0 = cbase >> 5;                  // gate rows
    cb1 = (g.inter + cbase) >> 5;      // up rows
  } else {
    const int base = nt * 64 * NW + wave * 64;
    active = base < g.N;
    const int cbase = active ? base : g.N - 64;
    ocol = cbase + col;
    cb0 = cbase >> 5;
    cb1 = cb0 + 1;
  }
  const int wrow0 = cb0 * 32 + col, wrow1 = cb1 * 32 + col;
  const int64_t wsel = SRC == kSrcBF16 ? (int64_t)(tile.w - g.bf16_slot_base) : (int64_t)expert;
  const BStream bs0 = make_stream<SRC>(g, wsel, cb0, lane);
  const BStream bs1 = make_stream<SRC>(g, wsel, cb1, lane);

  f32x16_t acc[NMB][2];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  // Prologue: A stages 0, 1, 2, then the weight ring (kRing steps).  The
  // fences pin that issue order: waiting for all but the loads issued after
  // stage 0's copies lands stage 0, and the stage barriers below can count
  // on at least 2 kStageLoads loads being younger than stage 1's or 2's
  // copies.
  BRegs<SRC> ring[kRing][2];
  copy_a(0, I0{});
  compiler_fence();
  copy_a(1, I1{});
  compiler_fence();
  copy_a(2, I2{});
  compiler_fence();
#pragma unroll
  for (int r = 0; r < kRing; ++r) {
    const int st = r < nsteps ? r : nsteps - 1;
    load_b<SRC>(bs0, st, ring[r][0]);
    load_b<SRC>(bs1, st, ring[r][1]);
  }
  static_assert(kRing * kBL >= kStageLoads, "prologue leaves too few younger loads");
  stage_barrier<2 * kNCA + kRing * kBL>();

  // one stage = one 64-wide K step; BUF = stage % kNBuf (compile-time)
  auto kstage = [&](int step, BRegs<SRC>(&slot)[2], auto buf_c) {
    constexpr int BUF = decltype(buf_c)::value;
    copy_a(step + kNBuf - 1, std::integral_constant<int, (BUF + kNBuf - 1) % kNBuf>{});
    const BScale<SRC> sc0 = b_scale<SRC>(slot[0]);
    const BScale<SRC> sc1 = b_scale<SRC>(slot[1]);
    const uint8_t* at = As.b[BUF];
    auto a_op = [&](int mb, int s) {
      return *reinterpret_cast<const bf16x8_t*>(at + mb * 32 * kStageRowB +
                                                aoff[s ^ ((mb & 1) << 2)]);
    };
    // A operands: each block's operand for the next K sub-step is read as
    // soon as its MFMAs for this sub-step have issued, so the read lands
    // behind the other blocks' MFMAs with one register set per block
    bf16x8_t acur[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) acur[mb] = a_op(mb, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8_t b0 = b_operand<SRC>(slot[0], sc0, s);
      const bf16x8_t b1 = b_operand<SRC>(slot[1], sc1, s);
      if (s == 3) {
        const int nx = step + kRing < nsteps ? step + kRing : nsteps - 1;
        load_b<SRC>(bs0, nx, slot[0]);
        load_b<SRC>(bs1, nx, slot[1]);
      }
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        acc[mb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(acur[mb], b0, acc[mb][0], 0, 0, 0);
        acc[mb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(acur[mb], b1, acc[mb][1], 0, 0, 0);
        if (s < 3) acur[mb] = a_op(mb, s + 1);
      }
    }
    if constexpr (SRC != kSrcBF16) {
      // schedule the stage as MFMA, up to kV VALU, MFMA, ... so that the
      // decode of the next sub-step runs on the vector ALU while the matrix
      // core works (the compiler otherwise bunches the decode)
      constexpr int kV = (28 + NMB - 1) / NMB;
#pragma unroll
      for (int i = 0; i < 8 * NMB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kV, 0);
      }
    }
    // the copies of stage step + 1 were issued two stages ago
    stage_barrier<2 * kStageLoads>();
  };

  int base = 0;
  for (; base + 4 <= nsteps; base += 4) {
    kstage(base + 0, ring[0], I0{});
    kstage(base + 1, ring[1 % kRing], I1{});
    kstage(base + 2, ring[2 % kRing], I2{});
    kstage(base + 3, ring[3 % kRing], I3{});
  }
  if (base < nsteps) {                   // two steps left (K % 128 == 0)
    kstage(base + 0, ring[0], I0{});
    kstage(base + 1, ring[1 % kRing], I1{});
  }
  // drain the clamped copies past the last stage before the LDS ring is
  // reused by the next item
  __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(0));
  // claim the workgroup's next item now, so the counter's round trip runs
  // under this item's epilogue
  if (threadIdx.x == 0) next_q = atomicAdd(g.work, 1);

  if (!active) return;
  {
    // LoRA up projection as extra K steps on the same accumulators: A rows
    // from u (this lane's row of each block, clamped into the tile), B rows
    // from the expert's adapter B (this wave's two weight rows: two output
    // column blocks, or the gate and up blocks of a SwiGLU item)
    if (g.lora_rank > 0) {
      const int rk = g.lora_rank;
      const uint16_t* b0p = g.lora_b + ((int64_t)expert * g.N + wrow0) * rk + 8 * half;
      const uint16_t* b1p = g.lora_b + ((int64_t)expert * g.N + wrow1) * rk + 8 * half;
      const uint16_t* up[NMB];
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        const int r = mb * 32 + col < nrows ? mb * 32 + col : nrows - 1;
        up[mb] = g.lora_u + (int64_t)(row0 + r) * rk + 8 * half;
      }
      for (int j = 0; j < rk; j += 16) {
        const bf16x8_t b0 = *reinterpret_cast<const bf16x8_t*>(b0p + j);
        const bf16x8_t b1 = *reinterpret_cast<const bf16x8_t*>(b1p + j);
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(up[mb] + j);
          acc[mb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, acc[mb][0], 0, 0, 0);
          acc[mb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, acc[mb][1], 0, 0, 0);
        }
      }
    }
  }
  // epilogue: lane holds column `col` of rows 8i + 4*half + j of each block
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = mb * 32 + 8 * i + 4 * half + j;
        if (r < nrows) {
          const int64_t orow = row0 + r;
          const float v0 = acc[mb][0][i * 4 + j];
          const float v1 = acc[mb][1][i * 4 + j];
          if constexpr (EPI == kEpiSwiGLU) {
            g.y[orow * g.ldy + ocol] = bf16_hw(silu_f32(v0) * v1);
            if (g.h) {
              g.h[orow * 2 * g.inter + ocol] = bf16_hw(v0);
              g.h[orow * 2 * g.inter + g.inter + ocol] = bf16_hw(v1);
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
__global__ __launch_bounds__(64 * nt_waves<MB>(), nt_occupancy<MB>()) void k_gemm_nt(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t A0[32 * MB * kStageRowB];
  __shared__ __attribute__((aligned(16))) uint8_t A1[32 * MB * kStageRowB];
  __shared__ __attribute__((aligned(16))) uint8_t A2[32 * MB * kStageRowB];
  __shared__ __attribute__((aligned(16))) uint8_t A3[32 * MB * kStageRowB];
  const LdsRing4 As{{A0, A1, A2, A3}};
  static_assert(kNBuf == 4, "four A stage buffers");
  __shared__ int s_next;
  const int t_begin = g.range[0];
  const int t_end = g.range[1];
  constexpr int NW = nt_waves<MB>();
  const int n_tiles_n = EPI == kEpiSwiGLU ? (g.inter + 32 * NW - 1) / (32 * NW)
                                          : (g.N + 64 * NW - 1) / (64 * NW);
  const unsigned items = (unsigned)((t_end - t_begin) * n_tiles_n);
  // Items (M-tile q / n_tiles_n, column tile q % n_tiles_n): workgroup b
  // starts with item b, and every further item comes in order from one
  // counter, so a workgroup that drew small tiles takes more of them (the
  // plan puts the largest tiles first); an empty launch touches no counter.
  int next_q = 0;
  unsigned q = blockIdx.x;
  while (q < items) {
    const int4 tile = g.tiles[t_begin + (int)(q / n_tiles_n)];
    const int nt = (int)(q % n_tiles_n);
    const int nmb = (tile.z + 31) / 32;
    if (MB == 1 || nmb <= 1) {
      gemm_nt_item<SRC, MB, EPI, AMODE, 1>(g, As, tile, nt, next_q);
    } else if (MB == 2 || nmb == 2) {
      gemm_nt_item<SRC, MB, EPI, AMODE, (MB >= 2 ? 2 : 1)>(g, As, tile, nt, next_q);
    } else if (nmb == 3) {
      gemm_nt_item<SRC, MB, EPI, AMODE, (MB >= 4 ? 3 : 1)>(g, As, tile, nt, next_q);
    } else {
      gemm_nt_item<SRC, MB, EPI, AMODE, (MB >= 4 ? 4 : 1)>(g, As, tile, nt, next_q);
    }
    // draws return 0, 1, ... and a launch makes exactly `items` of them (one
    // per item past the grid's first, one failing draw per workgroup that
    // had an item), so the draw of items - 1 is the last: it clears the
    // counter for the next launch
    if (threadIdx.x == 0) {
      s_next = next_q;
      if ((unsigned)next_q == items - 1) atomicExch(g.work, 0);
    }
    stage_barrier<63>();
    q = gridDim.x + (unsigned)__builtin_amdgcn_readfirstlane(s_next);
  }
}

template <int SRC, int MB, int EPI, int AMODE>
hipError_t launch_nt_t(const GemmArgs& g, hipStream_t s) {
  constexpr int NW = nt_waves<MB>();
  const int n_tiles_n = EPI == kEpiSwiGLU ? (g.inter + 32 * NW - 1) / (32 * NW)
                                          : (g.N + 64 * NW - 1) / (64 * NW);
  const int64_t bound = (int64_t)g.max_tiles * n_tiles_n;
  if (bound <= 0) return hipSuccess;
  int64_t grid = std::min<int64_t>(bound, (int64_t)num_cus() * nt_occupancy<MB>());
  grid = (grid + 7) / 8 * 8;
  hipLaunchKernelGGL((k_gemm_nt<SRC, MB, EPI, AMODE>), dim3((unsigned)grid), dim3(64 * NW), 0, s,
                     g);
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
  TimedLaunch timed_(kLGemm, s);
  switch (g.src) {
    case kSrcBF16: return launch_nt_m<kSrcBF16>(g, MB, s);
    case kSrcMXFP4: return launch_nt_m<kSrcMXFP4>(g, MB, s);
    default: return launch_nt_m<kSrcINT4>(g, MB, s);
  }
}

}  // namespace qgg
