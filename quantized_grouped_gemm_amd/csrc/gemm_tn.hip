// Grouped GEMM y = a . W_e over the routed rows of each expert (reduction over
// W's rows), the transposed access that the input-gradient backward needs.
//
// Orbit page, section 时刻细节: the backward through the frozen base forms
// only the input gradient (bypass-base-weight-grad GEMM backward), so the
// weights are read transposed: dA = dO . W_down and dXp = dH . W_gate_up,
// with the group-32 scales running along W's K index (the output columns
// here), not along the reduction.
//
// Work decomposition: as the forward kernel (persistent grid taking items past
// its first in order from a counter, NW wavefronts x 64 output columns,
// v_mfma_f32_32x32x16_bf16),
// with 32 reduction rows (W rows) per stage:
//  - A (rows of the routed activations) is copied global -> LDS three stages
//    ahead into a ring of four stage buffers, as in the forward kernel;
//  - each stage's weight tile (32 W rows x 64 NW columns) is loaded once per
//    workgroup, one 32-element scale group per thread (a single 16-byte load
//    and one scale), decoded to BF16 and stored row-major in LDS one stage
//    ahead of use;
//  - the MFMA B operand (8 consecutive W rows of one column) is read back with
//    two transposing LDS reads (ds_read_b64_tr_b16), so no register shuffle
//    is needed to turn rows into columns.
// The SwiGLU-backward epilogue applies the gate and the SwiGLU derivative
// from the saved forward activations.
#include "qgg_device.hpp"
#include "qgg_internal.hpp"

#include <type_traits>

namespace qgg {

namespace {

constexpr int kKR = 32;                   // reduction rows per stage
constexpr int kNBufA = 4;                 // stages in the LDS ring of A tiles
constexpr int kARowB = kKR * 2;           // A bytes per tile row per stage
// Wavefronts per workgroup (each owns 64 output columns of an item) and
// workgroups per CU: 128-row tiles of the plain-store form take 512-column
// items on eight waves, so that every A stage copied into LDS feeds twice the
// columns.  Shorter tiles, and the SwiGLU-backward form (whose epilogue needs
// registers the eight-wave build would spill), keep 256-column items and two
// workgroups per CU.
template <int MB, int EPI>
constexpr int tn_waves() { return MB == 4 && EPI == kEpiStore ? 8 : 4; }
template <int MB, int EPI>
constexpr int tn_occupancy() { return tn_waves<MB, EPI>() == 8 ? 1 : 2; }
// A stage buffer: MT rows, but at least what one round of 16-byte copies by
// the workgroup's threads fills
template <int MB, int EPI>
constexpr int a_stage_bytes() {
  return 32 * MB * kARowB > 1024 * tn_waves<MB, EPI>() ? 32 * MB * kARowB
                                                        : 1024 * tn_waves<MB, EPI>();
}
// B tile: 32 rows of 64 NW BF16 columns; the 16-byte piece P of row r is
// stored at piece position P ^ swz_b(r).  swz_b takes the 16 values 0..15
// on any 16 consecutive rows, with rows 4q..4q+3 differing in both bit pairs
// [2:1] and [3:2]; this keeps the transposing reads (4 rows x 32 bytes per
// 16 lanes, 4 rows x 64 bytes per 32 lanes) and the row stores (8 or 16 rows
// x 16 bytes) free of bank conflicts whether a bank cycle serves 128 or 256
// bytes.
template <int NW>
constexpr int b_row_bytes() { return 64 * NW * 2; }
template <int NW>
constexpr int b_stage_bytes() { return kKR * b_row_bytes<NW>(); }
__device__ __forceinline__ int swz_b(int r) {
  return ((0xCA60 >> (4 * (r & 3))) & 15) ^ ((r >> 2) & 1) ^ (((r >> 3) & 1) << 1);
}
// weight stages in flight per thread (BF16 stages are 4x larger)
template <int SRC>
constexpr int tn_ring_depth() { return SRC == kSrcBF16 ? 2 : 4; }
// vector-memory instructions one stage issues for the weight ring
template <int SRC>
constexpr int tn_b_loads() { return SRC == kSrcBF16 ? 4 : 2; }

// A chunk slot of tile row r: its four 16-byte K chunks are permuted (chunk
// kc at slot kc ^ swz_a(r)) so that operand reads of 32 consecutive rows hit
// distinct banks (chosen by measuring SQ_LDS_BANK_CONFLICT for candidate
// permutations of this read pattern on the chip; an unswizzled layout costs
// 3x the LDS cycles).
__device__ __forceinline__ int swz_a(int r) { return (r ^ (r >> 2)) & 3; }

__device__ __forceinline__ uint16_t bf16_hw_t(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}

template <int SRC>
struct BGroup {
  u32x4_t w[SRC == kSrcBF16 ? 4 : 1];   // one row's 32 consecutive columns
  uint32_t sraw;                        // raw scale bits
};

// This thread's slice of the weight stream: W row 32 st + jr, columns
// c0 + 32 sg .. + 31, i.e. one 32-element scale group per stage.  Offsets
// are bytes within one expert's (or BF16 slot's) weights; a stage adds the
// wave-uniform wstep / sstep.
struct BStreamT {
  __amdgpu_buffer_rsrc_t w, s;
  uint32_t wv, sv;
  int wstep, sstep;
};

template <int SRC>
__device__ __forceinline__ BStreamT make_stream_t(const GemmArgs& g, int64_t expert_or_slot,
                                                  int jr, int kcol) {
  // kcol: first of the 32 columns (a multiple of 32, may lie past K)
  BStreamT b;
  const int nkt = g.K / 64;
  const uint32_t slot = 32u * ((kcol >> 5) & 1) + jr;   // MFMA-tiled slot of row jr
  if constexpr (SRC == kSrcBF16) {
    const uint32_t bytes = (uint32_t)g.N * (uint32_t)g.K * 2u;
    b.w = raw_buffer(reinterpret_cast<const uint8_t*>(g.wbf16) + expert_or_slot * bytes, bytes);
    b.s = b.w;
    b.wv = (uint32_t)(kcol >> 6) * 4096u + slot * 16u;
    b.wstep = nkt * 4096;
    b.sv = 0;
    b.sstep = 0;
  } else {
    const int sb = SRC == kSrcMXFP4 ? 1 : 2;
    const uint32_t wbytes = (uint32_t)g.N * (uint32_t)(g.K / 2);
    const uint32_t sbytes = (uint32_t)g.N * (uint32_t)(g.K / 32) * sb;
    b.w = raw_buffer(g.packed + expert_or_slot * wbytes, wbytes);
    b.s = raw_buffer(static_cast<const uint8_t*>(g.scales) + expert_or_slot * sbytes, sbytes);
    if (g.layout == 1) {   // MFMA-tiled: tile (row block, 64 columns), slot
      const uint32_t t = (uint32_t)(kcol >> 6);
      b.wv = (t * 64u + slot) * 16u;
      b.wstep = nkt * 1024;
      b.sv = (t * 64u + slot) * sb;
      b.sstep = nkt * 64 * sb;
    } else {               // rows
      b.wv = (uint32_t)jr * (uint32_t)(g.K / 2) + (uint32_t)(kcol / 2);
      b.wstep = 32 * (g.K / 2);
      b.sv = ((uint32_t)jr * (uint32_t)(g.K / 32) + (uint32_t)(kcol / 32)) * sb;
      b.sstep = 32 * (g.K / 32) * sb;
    }
  }
  return b;
}

template <int SRC>
__device__ __forceinline__ void load_bt(const BStreamT& b, int st, BGroup<SRC>& r) {
  if constexpr (SRC == kSrcBF16) {
    // tiled BF16: the four 8-element pieces of a slot sit 1 KiB apart
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r.w[i] = __builtin_amdgcn_raw_buffer_load_b128(b.w, b.wv + i * 1024, st * b.wstep, 0);
  } else {
    r.w[0] = __builtin_amdgcn_raw_buffer_load_b128(b.w, b.wv, st * b.wstep, 0);
    if constexpr (SRC == kSrcMXFP4)
      r.sraw = __builtin_amdgcn_raw_buffer_load_b8(b.s, b.sv, st * b.sstep, 0);
    else
      r.sraw = __builtin_amdgcn_raw_buffer_load_b16(b.s, b.sv, st * b.sstep, 0);
  }
}

// Scale operand of the scaled FP4 conversions for E8M0 code c.  Those
// conversions read only the exponent field of their fp32 scale and take it as
// an E8M0 code (2^(c-127); code 0 gives 2^-127 and 255 NaN, as the format
// defines; measured for every code and every byte of FP4 pairs, identical to
// passing the exact fp32 value of 2^(c-127)), so the code shifted into that
// field is the whole operand and no special case costs VALU here.
__device__ __forceinline__ float e8m0_scale_operand(uint32_t c) { return __uint_as_float(c << 23); }

// Decode one group (32 columns of one W row) to BF16 and store its four
// 16-byte pieces at the given LDS byte offsets.
template <int SRC>
__device__ __forceinline__ void store_bt(const BGroup<SRC>& b, uint8_t* base, const int (&off)[4]) {
  u32x4_t v[4];
  if constexpr (SRC == kSrcBF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = b.w[i];
  } else {
    uint32_t o[16];
    if constexpr (SRC == kSrcMXFP4) {
      const float sc = e8m0_scale_operand(b.sraw);
#pragma unroll
      for (int i = 0; i < 4; ++i) dq8_mxfp4(b.w[0][i], sc, o + 4 * i);
    } else {
      const float sc = bf16_to_f32(b.sraw);
      const float m = 512.0f * sc, n8 = -8.0f * sc;
#pragma unroll
      for (int i = 0; i < 4; ++i) dq8_int4(b.w[0][i], m, n8, o + 4 * i);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = u32x4_t{o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]};
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4_t*>(base + off[i]) = v[i];
}


// One work item: tile (rows [row0, row0 + nrows) of one expert) x 64 NW
// output columns starting at c0, NMB live 32-row blocks.  Branch-free like
// the forward kernel: out-of-range loads are clamped (or read zeros through
// the buffer bounds) and only the stores are guarded.
template <int SRC, int MB, int EPI, int AMODE, int NMB>
__device__ __forceinline__ void gemm_tn_item(const GemmArgs& g, const LdsRing4& As,
                                             uint8_t (*Bs)[b_stage_bytes<tn_waves<MB, EPI>()>()],
                                             float* Gl, int4 tile, int c0, int& next_q) {
  constexpr int NW = tn_waves<MB, EPI>();
  constexpr int NT = 64 * NW;                       // threads
  constexpr int kBRowB = b_row_bytes<NW>();
  constexpr int kRing = tn_ring_depth<SRC>();
  constexpr int kBL = tn_b_loads<SRC>();
  constexpr int kNCA = (128 * NMB + NT - 1) / NT;   // A copies per thread per stage
  constexpr int kStageLoads = kNCA + kBL;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;
  const int nstages = g.N / kKR;
  const int row0 = tile.y, nrows = tile.z;
  const int64_t wsel = SRC == kSrcBF16 ? (int64_t)(tile.w - g.bf16_slot_base) : tile.x;

  // A copies: chunk slot p = NT i + tid of a stage holds K chunk
  // (p & 3) ^ swz_a(r) of tile row r = p >> 2 (slots past the live blocks
  // copy clamped rows that no operand read touches)
  const __amdgpu_buffer_rsrc_t arsrc = raw_buffer(g.a, (uint32_t)(g.a_rows * g.lda * 2));
  uint32_t aoffs[kNCA];
#pragma unroll
  for (int i = 0; i < kNCA; ++i) {
    const int p = NT * i + tid;
    const int r = p >> 2;
    const int kc = (p & 3) ^ swz_a(r);
    const int rr = r < nrows ? r : 0;
    int64_t srow;
    if constexpr (AMODE == kATokens) srow = g.perm[row0 + rr] / g.topk;
    else srow = row0 + rr;
    aoffs[i] = (uint32_t)((srow * g.lda + kc * 8) * 2);
  }
  auto copy_a = [&](int st, auto buf_c) {
    constexpr int BUF = decltype(buf_c)::value;
    const uint32_t soff = (uint32_t)((st < nstages ? st : nstages - 1) * kARowB);
#pragma unroll
    for (int i = 0; i < kNCA; ++i)
      copy16_to_lds(arsrc, aoffs[i], soff, As.b[BUF] + (NT * i + 64 * wave) * 16);
  };
  // A operand offsets: row col of a block, chunk 2 s + half
  int aoff[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) aoff[s] = col * kARowB + (((2 * s + half) ^ swz_a(col)) << 4);

  // B loader role: W row jr of the stage, columns c0 + 32 sg .. + 31 (the
  // row's pieces 4 sg .. 4 sg + 3); lanes 0..31 of a wavefront take 32
  // consecutive rows of one column group
  const int jr = tid & 31;
  const int sg = tid >> 5;
  const BStreamT bst = make_stream_t<SRC>(g, wsel, jr, c0 + 32 * sg);
  int bwoff[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) bwoff[k] = jr * kBRowB + (((4 * sg + k) ^ swz_b(jr)) << 4);
  // B operand reads: lane 16 G + i of the wavefront points at row
  // 16 s + 8 (G >> 1) + 4 up + i / 4 (up: the upper four of the eight rows),
  // column 64 wave + 32 nb + 16 (G & 1) + 4 (i & 3) (the row's swizzle does
  // not depend on s)
  const int bg = lane >> 4, bi = lane & 15;
  int broff[2][2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int up = 0; up < 2; ++up) {
      const int piece = 8 * wave + 4 * nb + 2 * (bg & 1) + ((bi & 3) >> 1);
      const int row = 8 * (bg >> 1) + 4 * up + (bi >> 2);
      broff[nb][up] = row * kBRowB + ((piece ^ swz_b(row)) << 4) + 8 * (bi & 1);
    }

  const int wbase = c0 + wave * 64;
  const bool active = wbase < g.K;
  // SwiGLU-backward epilogue: the gate of tile row tid, loaded now and put
  // in LDS after the K loop, so the epilogue does not wait on perm -> gates
  float gval = 0.f;
  if constexpr (EPI == kEpiSwiGLUBwd) {
    if (tid < 32 * NMB) gval = g.gates[g.perm[row0 + (tid < nrows ? tid : 0)]];
  }

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

  // Prologue: A stages 0, 1, 2 (issue order pinned), weight stages
  // 0 .. kRing - 1; stage 0's weights are decoded into Bs[0] and its ring
  // slot refilled with stage kRing.
  BGroup<SRC> ring[kRing];
  copy_a(0, I0{});
  compiler_fence();
  copy_a(1, I1{});
  compiler_fence();
  copy_a(2, I2{});
  compiler_fence();
#pragma unroll
  for (int r = 0; r < kRing; ++r) load_bt<SRC>(bst, r < nstages ? r : nstages - 1, ring[r]);
  store_bt<SRC>(ring[0], Bs[0], bwoff);
  load_bt<SRC>(bst, kRing < nstages ? kRing : nstages - 1, ring[0]);
  static_assert(kRing * kBL >= kStageLoads, "prologue leaves too few younger loads");
  stage_barrier<2 * kNCA + (kRing + 1) * kBL>();

  // stage st: MFMAs from As[st % 4] and Bs[st % 2]; the weights of stage
  // st + 1 (ring slot (st + 1) % kRing) are decoded into Bs[(st + 1) % 2]
  // and the slot refilled with stage st + 1 + kRing
  auto kstage = [&](int st, auto abuf_c) {
    constexpr int ABUF = decltype(abuf_c)::value;
    constexpr int BBUF = ABUF & 1;
    constexpr int SLOT = (ABUF + 1) % kRing;
    copy_a(st + kNBufA - 1, std::integral_constant<int, (ABUF + kNBufA - 1) % kNBufA>{});
    const uint8_t* at = As.b[ABUF];
    const uint8_t* bt = Bs[BBUF];
    // operand reads in the order the MFMAs consume them: sub-step 0's,
    // then its first MFMA pair, then sub-step 1's reads behind the
    // remaining sub-step 0 MFMAs
    bf16x8_t bop[2][2], aop[2][NMB];
    auto read_ops = [&](int s) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const uint2 lo = lds_tr4(bt + 16 * s * kBRowB + broff[nb][0]);
        const uint2 hi = lds_tr4(bt + 16 * s * kBRowB + broff[nb][1]);
        bop[s][nb] = __builtin_bit_cast(bf16x8_t, u32x4_t{lo.x, lo.y, hi.x, hi.y});
      }
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
        aop[s][mb] = *reinterpret_cast<const bf16x8_t*>(at + mb * 32 * kARowB + aoff[s]);
    };
    auto mfma_pair = [&](int s, int mb) {
      acc[mb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[s][mb], bop[s][0], acc[mb][0], 0, 0, 0);
      acc[mb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[s][mb], bop[s][1], acc[mb][1], 0, 0, 0);
    };
    read_ops(0);
    mfma_pair(0, 0);
    __builtin_amdgcn_sched_barrier(0);
    read_ops(1);
#pragma unroll
    for (int mb = 1; mb < NMB; ++mb) mfma_pair(0, mb);
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) mfma_pair(1, mb);
    store_bt<SRC>(ring[SLOT], Bs[BBUF ^ 1], bwoff);
    {
      const int nx = st + 1 + kRing;
      load_bt<SRC>(bst, nx < nstages ? nx : nstages - 1, ring[SLOT]);
    }
    // A copies of stage st + 1 were issued two stages ago
    stage_barrier<2 * kStageLoads>();
  };

  int st = 0;
  for (; st + 4 <= nstages; st += 4) {
    kstage(st + 0, I0{});
    kstage(st + 1, I1{});
    kstage(st + 2, I2{});
    kstage(st + 3, I3{});
  }
  // tail: nstages is even (N % 64 == 0)
  if (st < nstages) {
    kstage(st + 0, I0{});
    kstage(st + 1, I1{});
  }
  __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(0));
  // claim the workgroup's next item now, so the counter's round trip runs
  // under this item's epilogue
  if (tid == 0) next_q = atomicAdd(g.work, 1);
  if constexpr (EPI == kEpiSwiGLUBwd) {
    if (tid < 32 * NMB) Gl[tid] = gval;
    stage_barrier<63>();
  }

  // Epilogue through LDS, 16 tile rows per round: the wavefronts write their
  // fp32 accumulators (C layout: lane = column, 16 rows per lane) into a
  // 16 x 64 NW tile in Bs[0] (16-byte chunks XOR-permuted by row bit 2), then
  // every thread finishes 16 consecutive columns of one row with 16-byte
  // loads of the saved activations and 16-byte stores.
  (void)active;
  float* tile_f = reinterpret_cast<float*>(Bs[0]);
  auto tidx = [](int row, int c) { return row * NT + (((c >> 2) ^ (((row >> 2) & 1) << 3)) << 2) + (c & 3); };
  const int erow = tid / (4 * NW);      // this thread's row in a round
  const int eseg = tid % (4 * NW);      // its 16 columns: c0 + 16 eseg ..
  const int ecol = c0 + 16 * eseg;
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
    for (int ih = 0; ih < 2; ++ih) {
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            tile_f[tidx(8 * ii + 4 * half + j, wave * 64 + nb * 32 + col)] =
                acc[mb][nb][(2 * ih + ii) * 4 + j];
      stage_barrier<63>();
      const int r = mb * 32 + 16 * ih + erow;
      if (r < nrows && ecol < g.K) {
        const int64_t orow = row0 + r;
        float v[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4_t x = *reinterpret_cast<const f32x4_t*>(&tile_f[tidx(erow, 16 * eseg + 4 * q)]);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[4 * q + e] = x[e];
        }
        if constexpr (EPI == kEpiSwiGLUBwd) {
          // v = (dY . W_down)[c]; dA = g * v (+ the adapter's share when
          // lora_da is given); h_saved holds [gate | up]
          const float gate = Gl[r];
          const int64_t hb = orow * 2 * (int64_t)g.inter + ecol;
          const u32x4_t* hgp = reinterpret_cast<const u32x4_t*>(g.h + hb);
          const u32x4_t* hup = reinterpret_cast<const u32x4_t*>(g.h + hb + g.inter);
          const u32x4_t hg2[2] = {hgp[0], hgp[1]}, hu2[2] = {hup[0], hup[1]};
          u32x4_t ld2[2] = {u32x4_t{0u, 0u, 0u, 0u}, u32x4_t{0u, 0u, 0u, 0u}};
          if (g.lora_da) {
            const u32x4_t* lp = reinterpret_cast<const u32x4_t*>(
                g.lora_da + orow * (int64_t)g.inter + ecol);
            ld2[0] = lp[0];
            ld2[1] = lp[1];
          }
          uint32_t og[8], ou[8];
          float gp = 0.f;   // this thread's 16 terms of <dY . W_down, a>
#pragma unroll
          for (int e = 0; e < 16; e += 2) {
            float rg[2], ru[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              const uint32_t wg = hg2[(e + h2) >> 3][((e + h2) & 7) >> 1];
              const uint32_t wu = hu2[(e + h2) >> 3][((e + h2) & 7) >> 1];
              const float hg = bf16_to_f32(((e + h2) & 1) ? (wg >> 16) : (wg & 0xFFFFu));
              const float hu = bf16_to_f32(((e + h2) & 1) ? (wu >> 16) : (wu & 0xFFFFu));
              const uint32_t wl = ld2[(e + h2) >> 3][((e + h2) & 7) >> 1];
              const float da = gate * v[e + h2] +
                               bf16_to_f32(((e + h2) & 1) ? (wl >> 16) : (wl & 0xFFFFu));
              const float sg = 1.0f / (1.0f + __expf(-hg));
              const float dsilu = sg * (1.0f + hg * (1.0f - sg));
              rg[h2] = da * hu * dsilu;
              ru[h2] = da * hg * sg;
              gp = fmaf(v[e + h2], hg * sg * hu, gp);
            }
            og[e >> 1] = (uint32_t)bf16_hw_t(rg[0]) | ((uint32_t)bf16_hw_t(rg[1]) << 16);
            ou[e >> 1] = (uint32_t)bf16_hw_t(ru[0]) | ((uint32_t)bf16_hw_t(ru[1]) << 16);
          }
          if (g.gpart) {
            // the 16 threads of a row's 256-column part are 16 consecutive
            // lanes: a fixed butterfly gives every one the part's sum, one
            // partial per 256 columns
#pragma unroll
            for (int m = 1; m < 16; m <<= 1) gp += __shfl_xor(gp, m, 16);
            if ((eseg & 15) == 0) g.gpart[orow * (g.inter / 256) + ecol / 256] = gp;
          }
          u32x4_t* yg = reinterpret_cast<u32x4_t*>(g.y + orow * g.ldy + ecol);
          u32x4_t* yu = reinterpret_cast<u32x4_t*>(g.y + orow * g.ldy + g.inter + ecol);
          yg[0] = u32x4_t{og[0], og[1], og[2], og[3]};
          yg[1] = u32x4_t{og[4], og[5], og[6], og[7]};
          yu[0] = u32x4_t{ou[0], ou[1], ou[2], ou[3]};
          yu[1] = u32x4_t{ou[4], ou[5], ou[6], ou[7]};
        } else {
          uint32_t o[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            o[e] = (uint32_t)bf16_hw_t(v[2 * e]) | ((uint32_t)bf16_hw_t(v[2 * e + 1]) << 16);
          u32x4_t* yp = reinterpret_cast<u32x4_t*>(g.y + orow * g.ldy + ecol);
          yp[0] = u32x4_t{o[0], o[1], o[2], o[3]};
          yp[1] = u32x4_t{o[4], o[5], o[6], o[7]};
        }
      }
      stage_barrier<63>();
    }
  }
}

template <int SRC, int MB, int EPI, int AMODE>
__global__ __launch_bounds__((64 * tn_waves<MB, EPI>()), (tn_occupancy<MB, EPI>())) void k_gemm_tn(
    GemmArgs g) {
  constexpr int NW = tn_waves<MB, EPI>();
  __shared__ __attribute__((aligned(16))) uint8_t A0[a_stage_bytes<MB, EPI>()];
  __shared__ __attribute__((aligned(16))) uint8_t A1[a_stage_bytes<MB, EPI>()];
  __shared__ __attribute__((aligned(16))) uint8_t A2[a_stage_bytes<MB, EPI>()];
  __shared__ __attribute__((aligned(16))) uint8_t A3[a_stage_bytes<MB, EPI>()];
  const LdsRing4 As{{A0, A1, A2, A3}};
  static_assert(kNBufA == 4, "four A stage buffers");
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][b_stage_bytes<NW>()];
  __shared__ float Gl[32 * MB];   // per-row gates for the SwiGLU-backward epilogue
  __shared__ int s_next;
  const int t_begin = g.range[0];
  const int t_end = g.range[1];
  const int n_tiles_n = (g.K + 64 * NW - 1) / (64 * NW);   // output columns = W's K index
  const unsigned items = (unsigned)((t_end - t_begin) * n_tiles_n);
  // workgroup b starts with item b, the rest come in order from one counter,
  // as in the forward kernel
  int next_q = 0;
  unsigned q = blockIdx.x;
  while (q < items) {
    const int4 tile = g.tiles[t_begin + (int)(q / n_tiles_n)];
    const int c0 = (int)(q % n_tiles_n) * 64 * NW;
    const int nmb = (tile.z + 31) / 32;
    if (MB == 1 || nmb <= 1) {
      gemm_tn_item<SRC, MB, EPI, AMODE, 1>(g, As, Bs, Gl, tile, c0, next_q);
    } else if (MB == 2 || nmb == 2) {
      gemm_tn_item<SRC, MB, EPI, AMODE, (MB >= 2 ? 2 : 1)>(g, As, Bs, Gl, tile, c0, next_q);
    } else if (nmb == 3) {
      gemm_tn_item<SRC, MB, EPI, AMODE, (MB >= 4 ? 3 : 1)>(g, As, Bs, Gl, tile, c0, next_q);
    } else {
      gemm_tn_item<SRC, MB, EPI, AMODE, (MB >= 4 ? 4 : 1)>(g, As, Bs, Gl, tile, c0, next_q);
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
hipError_t launch_tn_t(const GemmArgs& g, hipStream_t s) {
  constexpr int NW = tn_waves<MB, EPI>();
  const int n_tiles_n = (g.K + 64 * NW - 1) / (64 * NW);
  const int64_t bound = (int64_t)g.max_tiles * n_tiles_n;
  if (bound <= 0) return hipSuccess;
  int64_t grid = std::min<int64_t>(bound, (int64_t)num_cus() * tn_occupancy<MB, EPI>());
  grid = (grid + 7) / 8 * 8;
  hipLaunchKernelGGL((k_gemm_tn<SRC, MB, EPI, AMODE>), dim3((unsigned)grid), dim3(64 * NW), 0, s,
                     g);
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
  TimedLaunch timed_(kLGemmT, s);
  switch (g.src) {
    case kSrcBF16: return launch_tn_m<kSrcBF16>(g, MB, s);
    case kSrcMXFP4: return launch_tn_m<kSrcMXFP4>(g, MB, s);
    default: return launch_tn_m<kSrcINT4>(g, MB, s);
  }
}

}  // namespace qgg
