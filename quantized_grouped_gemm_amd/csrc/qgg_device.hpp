// Device helpers shared by the gfx950 kernels: BF16 conversion, wavefront
// prefix sums, MFMA operand types and the 4-bit decoders.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qgg {

constexpr int kWave = 64;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }

// Round-to-nearest-even fp32 -> BF16 in integer arithmetic; NaN -> quiet NaN
// with the input's upper bits.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 -> packed BF16 pair (v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  bf16x2_t b = __builtin_convertvector(v, bf16x2_t);
  return __builtin_bit_cast(uint32_t, b);
}

// Inclusive prefix sum across the 64 lanes of a wavefront.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int n = __shfl_up(v, off, kWave);
    if (lane >= off) v += n;
  }
  return v;
}

// Exclusive prefix sum over a whole workgroup of `nthreads` threads (a
// multiple of 64, <= 1024); `lds` holds >= 16 ints.  Returns the exclusive
// prefix and writes the total to *total.  All threads must call it.
__device__ __forceinline__ int block_excl_scan(int v, int* lds, int* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nwaves = blockDim.x / kWave;
  const int incl = wave_incl_scan(v);
  if (lane == kWave - 1) lds[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int s = lane < nwaves ? lds[lane] : 0;
    s = wave_incl_scan(s);
    if (lane < nwaves) lds[lane] = s;
  }
  __syncthreads();
  const int before = wave ? lds[wave - 1] : 0;
  *total = lds[nwaves - 1];
  __syncthreads();
  return before + incl - v;
}

// E8M0 exponent code -> fp32 scale 2^(c-127); code 0 is the subnormal 2^-127,
// code 255 is NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t c) {
  const uint32_t bits = c == 0 ? 0x00400000u : (c == 255 ? 0x7FC00000u : (c << 23));
  return __uint_as_float(bits);
}

// Eight MXFP4 codes (one 32-bit word, element 2b in the low nibble of byte b)
// times a power-of-two scale -> eight BF16 values packed in four words
// (v_cvt_scalef32_pk_bf16_fp4; exact while the product is representable).
__device__ __forceinline__ void dq8_mxfp4(uint32_t w, float scale, uint32_t out[4]) {
  out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
  out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
  out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
  out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
}

// Eight two's-complement INT4 codes times a BF16 scale s -> eight BF16 values.
// With n' = q + 8 (the code XOR 8), each n' in 0..15 is moved into a byte;
// read as an FP8 E4M3 code, byte n' is exactly n' * 2^-9 (codes 0..7 are the
// subnormals m * 2^-9, codes 8..15 the first binade (8 + m) * 2^-9), so one
// v_cvt_pk_f32_fp8 yields two exact values.  fma(n' 2^-9, 512 s, -8 s) is
// q * s formed exactly and rounded once; q * s needs at most 12 significant
// bits, so the fp32 value is exact and the BF16 rounding matches
// bf16_rne(q * s).  s512 = 512 s and neg8s = -8 s are exact powers-of-two
// multiples of s (finite for every scale below 2^118).
__device__ __forceinline__ void dq8_int4(uint32_t w, float s512, float neg8s, uint32_t out[4]) {
  // (x ^ 8) & 15 per byte: one three-input bitwise op for each half
  const uint32_t lo = (w ^ 0x08080808u) & 0x0F0F0F0Fu;          // elements 0, 2, 4, 6
  const uint32_t hi = ((w >> 4) ^ 0x08080808u) & 0x0F0F0F0Fu;   // elements 1, 3, 5, 7
  const f32x2_t e02 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
  const f32x2_t e46 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
  const f32x2_t e13 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
  const f32x2_t e57 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
  out[0] = pack_bf16x2(__builtin_fmaf(e02[0], s512, neg8s), __builtin_fmaf(e13[0], s512, neg8s));
  out[1] = pack_bf16x2(__builtin_fmaf(e02[1], s512, neg8s), __builtin_fmaf(e13[1], s512, neg8s));
  out[2] = pack_bf16x2(__builtin_fmaf(e46[0], s512, neg8s), __builtin_fmaf(e57[0], s512, neg8s));
  out[3] = pack_bf16x2(__builtin_fmaf(e46[1], s512, neg8s), __builtin_fmaf(e57[1], s512, neg8s));
}

// 4 BF16 of a B column (rows r .. r + 3) by a transposing LDS read: within
// each 16-lane group, lane i receives element i % 4 of the 8-byte rows that
// lanes i / 4, i / 4 + 4, i / 4 + 8, i / 4 + 12 point at.
__device__ __forceinline__ uint2 lds_tr4(const uint8_t* p) {
  typedef short s16x4_t __attribute__((ext_vector_type(4)));
  const s16x4_t v =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)p);
  return __builtin_bit_cast(uint2, v);
}

// ---- memory pipeline helpers shared by the GEMM kernels

// s_waitcnt immediate: wait until at most n vector-memory operations are
// outstanding and all LDS operations are done (gfx9 encoding: vmcnt in bits
// [3:0] and [15:14], expcnt [6:4] left at its maximum, lgkmcnt [11:8] = 0).
constexpr int vm_lgkm0_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4); }

// Compiler-only fence: no memory access moves across it; emits nothing.
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// 16 bytes from a buffer -> LDS without a register round trip
// (buffer_load_dwordx4 ... lds): lane i of the wavefront writes lds + 16 i,
// so the LDS pointer must be the same for the whole wavefront.  Offsets past
// the buffer's size read zeros.  (The buffer form, unlike the global one, is
// tracked by the compiler as an ordinary in-order vector-memory load, so its
// own waits for register loads keep exact counts.)
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff,
                                              uint32_t soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, soff, 0, 0);
}

// Raw (untyped, unswizzled) buffer resource over [base, base + bytes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Barrier between two pipeline stages.  A wavefront first waits until at
// most N of its vector-memory operations are outstanding (the caller picks N
// as the loads issued after its LDS copies for the next stage, so those have
// landed while the younger copies and weight loads stay in flight) and its
// LDS operations are done, then meets the others.  No memory fence: at
// workgroup scope one would drain every outstanding load, LDS copies
// included.
template <int N>
__device__ __forceinline__ void stage_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  compiler_fence();
  __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(N));
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

// Four LDS stage buffers declared as separate objects (see the kernels):
// with one array the compiler cannot tell an LDS copy into one buffer from a
// read of another, and drains every in-flight copy before each LDS read.
struct LdsRing4 {
  uint8_t* b[4];
};

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

}  // namespace qgg
