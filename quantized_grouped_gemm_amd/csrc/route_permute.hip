// Routing, stable expert permutation, row gather and M-tile planning.
//
// Orbit page, section 时刻细节 ("Active-expert-chunked dequantization"): each
// token activates only the experts its router selects, and the selected
// experts are grouped before the grouped GEMM.  The grouping here is a stable
// counting sort of the (token, expert) pairs by expert id built from
// wavefront prefix sums; every step is deterministic (no order-dependent
// atomics: LDS atomics are used only for counts).
#include "qgg_device.hpp"
#include "qgg_internal.hpp"

namespace qgg {

// ---------------------------------------------------------------- route
// One wavefront per token.  Each lane holds up to 16 logits (E <= 1024); k
// rounds of a wavefront arg-max under the key (logit desc, id asc) pick the
// experts; gates are the softmax over the kept logits.
__global__ __launch_bounds__(256) void k_route(const float* __restrict__ logits, int T, int E,
                                               int k, int32_t* __restrict__ ids,
                                               float* __restrict__ gates,
                                               int32_t* __restrict__ err) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + threadIdx.x / 64;
  if (t >= T) return;
  const float* row = logits + (int64_t)t * E;
  float v[16];
  bool bad = false;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = lane + 64 * i;
    float x = -INFINITY;
    if (e < E) {
      x = row[e];
      if (!__builtin_isfinite(x)) {
        bad = true;
        x = -INFINITY;
      }
    }
    v[i] = x;
  }
  if (__any(bad) && lane == 0 && err) atomicOr(err, 1);
  uint32_t taken = 0;  // bit i: v[i] already selected
  float m = 0.f, sum = 0.f;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u) && (v[i] > bv || bi == 0x7FFFFFFF)) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (j == 0) m = bv;
    const float w = expf(bv - m);
    sum += w;
    if (lane == 0) {
      ids[(int64_t)t * k + j] = bi;
      gates[(int64_t)t * k + j] = w;
    }
  }
  if (lane == 0) {
    for (int j = 0; j < k; ++j) gates[(int64_t)t * k + j] = gates[(int64_t)t * k + j] / sum;
  }
}

// -------------------------------------------------------------- permute
// Pairs are split into segments of kSeg (one workgroup each) and each segment
// into 16 wave sub-segments of kSeg/16.
constexpr int kSeg = 4096;
constexpr int kSub = kSeg / 16;

__device__ __forceinline__ int load_id(const int32_t* ids, int64_t p, int64_t P, int E,
                                       int32_t* err) {
  if (p >= P) return -1;
  const int e = ids[p];
  if (e < 0 || e >= E) {
    if (err) atomicOr(err, 2);
    return -1;
  }
  return e;
}

// blk[b][e] = number of pairs of segment b routed to expert e.
__global__ __launch_bounds__(1024) void k_perm_count(const int32_t* __restrict__ ids, int64_t P,
                                                     int E, int32_t* __restrict__ blk,
                                                     int32_t* __restrict__ err) {
  extern __shared__ int lds_cnt[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) lds_cnt[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kSeg;
  for (int i = threadIdx.x; i < kSeg; i += blockDim.x) {
    const int e = load_id(ids, base + i, P, E, err);
    if (e >= 0) atomicAdd(&lds_cnt[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) blk[(int64_t)blockIdx.x * E + e] = lds_cnt[e];
}

// counts, offsets (exclusive prefix), active list, n_active; blk[b][e] is
// replaced by the first sorted row of segment b's pairs of expert e.
__global__ __launch_bounds__(1024) void k_perm_scan(int nblk, int E, int32_t* __restrict__ blk,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ active,
                                                    int32_t* __restrict__ n_active) {
  __shared__ int scratch[16];
  const int e = threadIdx.x;  // E <= 1024 = blockDim.x
  int run = 0;
  if (e < E) {
    for (int b = 0; b < nblk; ++b) {
      const int c = blk[(int64_t)b * E + e];
      blk[(int64_t)b * E + e] = run;
      run += c;
    }
  }
  int total;
  const int off = block_excl_scan(e < E ? run : 0, scratch, &total);
  if (e < E) {
    counts[e] = run;
    offsets[e] = off;
    for (int b = 0; b < nblk; ++b) blk[(int64_t)b * E + e] += off;
  }
  if (e == 0) offsets[E] = total;
  int nact;
  const int flag = (e < E && run > 0) ? 1 : 0;
  const int pos = block_excl_scan(flag, scratch, &nact);
  if (flag) active[pos] = e;
  if (e < E && e >= nact) active[e] = -1;
  if (e == 0) *n_active = nact;
}

// perm / inv_perm.  Within a wave step of 64 pairs the rank of a pair among
// equal experts comes from a broadcast scan of the step's ids in LDS; across
// steps a per-wave, per-expert cursor in LDS carries the running position.
__global__ __launch_bounds__(1024) void k_perm_scatter(const int32_t* __restrict__ ids, int64_t P,
                                                       int E, const int32_t* __restrict__ blk,
                                                       int32_t* __restrict__ perm,
                                                       int32_t* __restrict__ inv_perm) {
  extern __shared__ int lds[];
  int* cur = lds;                 // [16][E] per-wave cursors
  int* sid = lds + 16 * E;        // [16][64] ids of the current step
  const int wave = threadIdx.x / 64;
  const int lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < 16 * E; i += blockDim.x) cur[i] = 0;
  __syncthreads();
  const int64_t sub0 = (int64_t)blockIdx.x * kSeg + (int64_t)wave * kSub;
  for (int s = 0; s < kSub; s += 64) {
    const int e = load_id(ids, sub0 + s + lane, P, E, nullptr);
    if (e >= 0) atomicAdd(&cur[wave * E + e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = blk[(int64_t)blockIdx.x * E + e];
    for (int w = 0; w < 16; ++w) {
      const int c = cur[w * E + e];
      cur[w * E + e] = run;
      run += c;
    }
  }
  __syncthreads();
  int* mine = sid + wave * 64;
  for (int s = 0; s < kSub; s += 64) {
    const int64_t p = sub0 + s + lane;
    const int e = load_id(ids, p, P, E, nullptr);
    mine[lane] = e >= 0 ? e : -1 - lane;  // invalid slots never match
    __syncthreads();
    int rank = 0;
    bool last = true;
    const int me = mine[lane];
#pragma unroll 8
    for (int i = 0; i < 64; ++i) {
      const int o = mine[i];
      rank += (i < lane && o == me) ? 1 : 0;
      last = last && !(i > lane && o == me);
    }
    int base = 0;
    if (e >= 0) base = cur[wave * E + e];
    __syncthreads();
    if (e >= 0) {
      const int pos = base + rank;
      perm[pos] = (int32_t)p;
      inv_perm[p] = pos;
      if (last) cur[wave * E + e] = pos + 1;
    } else if (p < P) {
      inv_perm[p] = -1;
    }
    __syncthreads();
  }
}

// x_perm[i][:] = x[perm[i] / k][:], one wavefront per row, 16-byte moves.
__global__ __launch_bounds__(256) void k_gather_rows(const uint16_t* __restrict__ x, int d,
                                                     const int32_t* __restrict__ perm,
                                                     const int32_t* __restrict__ offsets, int E,
                                                     int k, uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x & 63;
  if (i >= offsets[E]) return;
  const int64_t t = perm[i] / k;
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + t * d);
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + i * d);
  for (int c = lane; c < d / 8; c += 64) dst[c] = src[c];
}

// M-tile plan: for the active experts in ascending order, tiles of up to MT
// rows.  tiles[j] = {expert, first sorted row, rows, active index};
// chunk_first[c] = first tile of chunk c (chunks of C active experts), and
// chunk_first[nchunks] = number of tiles.
__global__ __launch_bounds__(1024) void k_tile_plan(const int32_t* __restrict__ counts,
                                                    const int32_t* __restrict__ offsets,
                                                    const int32_t* __restrict__ active,
                                                    const int32_t* __restrict__ n_active, int MT,
                                                    int C, int4* __restrict__ tiles,
                                                    int32_t* __restrict__ chunk_first) {
  __shared__ int scratch[16];
  const int a = threadIdx.x;
  const int A = *n_active;
  const int e = a < A ? active[a] : -1;
  const int cnt = e >= 0 ? counts[e] : 0;
  const int nt = (cnt + MT - 1) / MT;
  int total;
  const int first = block_excl_scan(nt, scratch, &total);
  if (e >= 0) {
    const int r0 = offsets[e];
    for (int i = 0; i < nt; ++i) {
      const int rows = min(MT, cnt - i * MT);
      tiles[first + i] = make_int4(e, r0 + i * MT, rows, a);
    }
  }
  const int CC = C > 0 ? C : (A > 0 ? A : 1);
  if (a < A && a % CC == 0) chunk_first[a / CC] = first;
  if (a == 0) {
    const int nch = (A + CC - 1) / CC;
    chunk_first[nch] = total;
    if (nch == 0) chunk_first[0] = 0;
  }
}

// ------------------------------------------------------------- launchers

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* gates,
                        int32_t* err, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(k_route, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, ids, gates,
                     err);
  return hipGetLastError();
}

size_t permute_ws_bytes(int64_t P, int E) {
  const int64_t nblk = (P + kSeg - 1) / kSeg;
  return (size_t)std::max<int64_t>(nblk, 1) * E * sizeof(int32_t);
}

hipError_t launch_permute(const int32_t* ids, int64_t P, int E, const PermPtrs& pp, int32_t* err,
                          void* ws, hipStream_t s) {
  const int nblk = (int)((P + kSeg - 1) / kSeg);
  int32_t* blk = static_cast<int32_t*>(ws);
  if (nblk > 0) {
    hipLaunchKernelGGL(k_perm_count, dim3(nblk), dim3(1024), E * sizeof(int), s, ids, P, E, blk,
                       err);
  }
  hipLaunchKernelGGL(k_perm_scan, dim3(1), dim3(1024), 0, s, nblk, E, blk, pp.counts, pp.offsets,
                     pp.active, pp.n_active);
  if (nblk > 0) {
    const size_t lds = (16 * E + 16 * 64) * sizeof(int);
    if (lds > 65536) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_perm_scatter),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_perm_scatter, dim3(nblk), dim3(1024), lds, s, ids, P, E, blk, pp.perm,
                       pp.inv_perm);
  }
  return hipGetLastError();
}

hipError_t launch_gather(const uint16_t* x, int d, const PermPtrs& pp, int E, int k, int64_t P,
                         uint16_t* out, hipStream_t s) {
  if (P == 0) return hipSuccess;
  hipLaunchKernelGGL(k_gather_rows, dim3((unsigned)((P + 3) / 4)), dim3(256), 0, s, x, d,
                     pp.perm, pp.offsets, E, k, out);
  return hipGetLastError();
}

hipError_t launch_tile_plan(const PermPtrs& pp, int MT, int C, int4* tiles, int32_t* chunk_first,
                            hipStream_t s) {
  hipLaunchKernelGGL(k_tile_plan, dim3(1), dim3(1024), 0, s, pp.counts, pp.offsets, pp.active,
                     pp.n_active, MT, C, tiles, chunk_first);
  return hipGetLastError();
}

}  // namespace qgg
