// Routing, stable expert permutation, row gather and M-tile planning.
//
// Orbit page, section 时刻细节 ("Active-expert-chunked dequantization"): each
// token activates only the experts its router selects, and the selected
// experts are grouped before the grouped GEMM.  The grouping here is a stable
// counting sort of the (token, expert) pairs by expert id: counts, an
// exclusive scan, then placement by ordered wavefront ballots (a pair's rank
// inside its expert is a population count); every step is deterministic (no
// order-dependent atomics: LDS atomics are used only for counts).
#include "qgg_device.hpp"
#include "qgg_internal.hpp"

#include <type_traits>

namespace qgg {

// ---------------------------------------------------------------- route
// Wavefront maximum of a 64-bit key through DPP row/quad moves (no LDS round
// trips); the result is read from lane 63.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
  auto step = [&](auto ctrl_c, auto rmask_c) {
    constexpr int kCtrl = decltype(ctrl_c)::value;
    constexpr int kRow = decltype(rmask_c)::value;
    const uint32_t lo = (uint32_t)k, hi = (uint32_t)(k >> 32);
    const uint32_t olo = __builtin_amdgcn_update_dpp(lo, lo, kCtrl, kRow, 0xF, false);
    const uint32_t ohi = __builtin_amdgcn_update_dpp(hi, hi, kCtrl, kRow, 0xF, false);
    const uint64_t o = ((uint64_t)ohi << 32) | olo;
    k = o > k ? o : k;
  };
  using std::integral_constant;
  step(integral_constant<int, 0xB1>{}, integral_constant<int, 0xF>{});   // quad_perm 1,0,3,2
  step(integral_constant<int, 0x4E>{}, integral_constant<int, 0xF>{});   // quad_perm 2,3,0,1
  step(integral_constant<int, 0x141>{}, integral_constant<int, 0xF>{});  // row_half_mirror
  step(integral_constant<int, 0x140>{}, integral_constant<int, 0xF>{});  // row_mirror
  step(integral_constant<int, 0x142>{}, integral_constant<int, 0xA>{});  // row_bcast:15
  step(integral_constant<int, 0x143>{}, integral_constant<int, 0xC>{});  // row_bcast:31
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)k, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(k >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// fp32 -> uint32 with the same order (larger float, larger key)
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One wavefront per token.  Each lane holds NV logits (experts lane, lane +
// 64, ...; NV * 64 >= E); k rounds of a wavefront arg-max under the key
// (logit desc, id asc) pick the experts, each lane offering its best
// untaken entry (recomputed only by the lane whose entry was just taken);
// gates are the softmax over the kept logits.
template <int NV>
__global__ __launch_bounds__(256) void k_route(const float* __restrict__ logits, int T, int E,
                                               int k, int32_t* __restrict__ ids,
                                               float* __restrict__ gates,
                                               int32_t* __restrict__ err) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + threadIdx.x / 64;
  if (t >= T) return;
  const float* row = logits + (int64_t)t * E;
  float v[NV];
  bool bad = false;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + 64 * i;
    float x = -INFINITY;
    if (e < E) {
      x = row[e];
      if (!__builtin_isfinite(x)) {
        bad = true;
        x = -INFINITY;
      }
    }
    v[i] = x + 0.0f;   // -0 -> +0: equal logits tie on the expert id
  }
  if (__any(bad) && lane == 0 && err) atomicOr(err, 1);
  uint32_t taken = 0;  // bit i: v[i] already selected
  float m = 0.f, sum = 0.f;
  int my_id = 0;       // lane j keeps pick j (k <= 32)
  float my_w = 0.f;
  // this lane's best untaken entry; key 0 = none (a valid entry, even -inf,
  // has a nonzero key)
  auto lane_best = [&]() {
    uint64_t key = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = lane + 64 * i;
      const uint64_t ki = ((uint64_t)order_key(v[i]) << 32) | (uint32_t)~e;
      if (e < E && !((taken >> i) & 1u) && ki > key) key = ki;
    }
    return key;
  };
  uint64_t mine = lane_best();
  for (int j = 0; j < k; ++j) {
    const uint64_t key = wave_max_u64(mine);
    const int bi = (int)~(uint32_t)key;
    const uint32_t ok = (uint32_t)(key >> 32);
    const float best = __uint_as_float((ok & 0x80000000u) ? (ok & 0x7FFFFFFFu) : ~ok);
    if ((bi & 63) == lane) {
      taken |= 1u << (bi >> 6);
      mine = lane_best();
    }
    if (j == 0) m = best;
    const float w = expf(best - m);
    sum += w;
    if (lane == j) {
      my_id = bi;
      my_w = w;
    }
  }
  if (lane < k) {
    ids[(int64_t)t * k + lane] = my_id;
    gates[(int64_t)t * k + lane] = my_w / sum;
  }
}

// ------------------------------------------------------- router backward
// Gradient handed back to the router when the base is frozen and the routing
// choice is held fixed.  One wavefront per token; lane j < k owns pair
// (t, j): dg_j = <dY[t], o[t, j]>, summed from the per-item partials the
// SwiGLU-backward epilogue left in gpart (ascending item).  The gates are
// the softmax of the kept logits, whose backward is
// dl_j = g_j (dg_j - sum_i g_i dg_i); experts not kept get 0.  A pair that
// the permutation dropped (its expert id was outside [0, E), inv_perm -1)
// contributed nothing to the forward output, so its dg is 0 and no logit
// entry belongs to it.
__global__ __launch_bounds__(256) void k_router_bwd(const float* __restrict__ gpart, int nitems,
                                                    const int32_t* __restrict__ inv_perm,
                                                    const int32_t* __restrict__ ids,
                                                    const float* __restrict__ gates, int T, int E,
                                                    int k, float* __restrict__ dgates,
                                                    float* __restrict__ dlogits) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + threadIdx.x / 64;
  if (t >= T) return;
  float dg = 0.f, g = 0.f;
  int id = -1;
  if (lane < k) {
    const int64_t q = (int64_t)t * k + lane;
    const int src = inv_perm[q];
    if (src >= 0) {
      const float* row = gpart + (int64_t)src * nitems;
      for (int c = 0; c < nitems; ++c) dg += row[c];
      id = ids[q];
    }
    g = gates[q];
    if (dgates) dgates[q] = dg;
  }
  if (!dlogits) return;
  // sum_i g_i dg_i in ascending i, the same value in every lane
  const int gdg = __float_as_int(g * dg);
  float sgd = 0.f;
  for (int i = 0; i < k; ++i) sgd += __int_as_float(__builtin_amdgcn_readlane(gdg, i));
  const float dl = g * (dg - sgd);
  const int dli = __float_as_int(dl);
  float* out = dlogits + (int64_t)t * E;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    float v = 0.f;
    for (int i = 0; i < k; ++i)
      if (__builtin_amdgcn_readlane(id, i) == e) v = __int_as_float(__builtin_amdgcn_readlane(dli, i));
    if (e < E) out[e] = v;
  }
}

// -------------------------------------------------------------- permute
// Pairs are split into segments of kSeg (one counting workgroup each).
constexpr int kSeg = 4096;

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

// blk[b][e] = number of pairs of segment b routed to expert e (LDS: E ints).
__device__ __forceinline__ void perm_count_body(const int32_t* __restrict__ ids, int64_t P, int E,
                                                int32_t* __restrict__ blk,
                                                int32_t* __restrict__ err, int* lds_cnt, int b,
                                                int32_t* __restrict__ inv_perm = nullptr) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) lds_cnt[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)b * kSeg;
  for (int i = threadIdx.x; i < kSeg; i += blockDim.x) {
    const int e = load_id(ids, base + i, P, E, err);
    if (e >= 0) atomicAdd(&lds_cnt[e], 1);
    else if (inv_perm && base + i < P) inv_perm[base + i] = -1;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) blk[(int64_t)b * E + e] = lds_cnt[e];
}

__global__ __launch_bounds__(1024) void k_perm_count(const int32_t* __restrict__ ids, int64_t P,
                                                     int E, int32_t* __restrict__ blk,
                                                     int32_t* __restrict__ err,
                                                     int32_t* __restrict__ inv_perm) {
  extern __shared__ int lds_cnt[];
  perm_count_body(ids, P, E, blk, err, lds_cnt, blockIdx.x, inv_perm);
}

// perm / inv_perm for many pairs: one wavefront per (segment b, expert e)
// walks the segment's pair ids in order (eight 64-pair ballots in flight) and
// places its pairs from blk[b][e] (the first sorted row of the segment's
// pairs of e, after the scan) + the population count of earlier hits; pairs
// with invalid ids were marked by the count step.
__global__ __launch_bounds__(256) void k_perm_place(const int32_t* __restrict__ ids, int64_t P,
                                                    int E, const int32_t* __restrict__ blk,
                                                    const int32_t* __restrict__ counts,
                                                    const int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ perm,
                                                    int32_t* __restrict__ inv_perm) {
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  if (e >= E) return;
  int run = blk[(int64_t)b * E + e];
  const int end = (int64_t)(b + 1) * kSeg < P ? blk[(int64_t)(b + 1) * E + e]
                                              : offsets[e] + counts[e];
  if (run == end) return;                      // no pair of e in this segment
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  const int64_t p0 = (int64_t)b * kSeg;
  constexpr int kU = 8;
  for (int c0 = 0; c0 < kSeg; c0 += 64 * kU) {
    int id[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t p = p0 + c0 + 64 * u + lane;
      id[u] = p < P ? ids[p] : -1;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const bool hit = id[u] == e;
      const uint64_t mask = __ballot(hit);
      if (hit) {
        const int64_t p = p0 + c0 + 64 * u + lane;
        const int pos = run + __popcll(mask & below);
        perm[pos] = (int32_t)p;
        inv_perm[p] = pos;
      }
      run += __popcll(mask);
    }
    if (run == end) return;
  }
}

// counts, offsets (exclusive prefix), active list, n_active; blk[b][e] is
// replaced by the first sorted row of segment b's pairs of expert e.
__device__ __forceinline__ void perm_scan_body(int nblk, int E, int32_t* __restrict__ blk,
                                               int32_t* __restrict__ counts,
                                               int32_t* __restrict__ offsets,
                                               int32_t* __restrict__ active,
                                               int32_t* __restrict__ n_active, int* scratch) {
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

__global__ __launch_bounds__(1024) void k_perm_scan(int nblk, int E, int32_t* __restrict__ blk,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ active,
                                                    int32_t* __restrict__ n_active) {
  __shared__ int scratch[16];
  perm_scan_body(nblk, E, blk, counts, offsets, active, n_active, scratch);
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

// M-tile plan: the rows of the active experts cut into tiles of up to MT rows,
// tiles[j] = {expert, first sorted row, rows, active index}, grouped into
// chunks of C active experts: chunk_first[c] = first tile of chunk c and
// chunk_first[nchunks] = number of tiles.  Inside a chunk the tiles are
// ordered by their number of live 32-row blocks, most first (ascending
// expert within a size), so that workgroups taking the items of a launch in
// order from one counter finish on the smallest.  The GEMM launches' two
// work counters (work[0], work[1]) are cleared here, before any launch of the
// call uses them.
__device__ __forceinline__ void tile_plan_body(const int32_t* __restrict__ counts,
                                               const int32_t* __restrict__ offsets,
                                               const int32_t* __restrict__ active,
                                               const int32_t* __restrict__ n_active, int MT,
                                               int C, int4* __restrict__ tiles,
                                               int32_t* __restrict__ chunk_first, int* scratch,
                                               int (*sk)[1025], int E, int32_t* work) {
  const int a = threadIdx.x;
  const int A = *n_active;
  const int e = a < A ? active[a] : -1;
  const int cnt = e >= 0 ? counts[e] : 0;
  const int MB = MT / 32;
  const int nfull = cnt / MT;
  const int rem = cnt - nfull * MT;
  const int rb = (rem + 31) / 32;        // live blocks of the last, partial tile
  // sk[b - 1][i] = tiles with b live blocks of the active experts before i
  // (i = 0 .. A; experts past the last active one add none): the MB
  // exclusive scans of one pass, wavefront scans first, then wavefront b
  // scans the wavefront totals of size b
  const int lane = a & 63, wv = a >> 6, nwv = blockDim.x >> 6;
  int incl[4];
#pragma unroll
  for (int b = 1; b <= 4; ++b) {
    const int nb = b > MB ? 0 : (b == MB ? nfull : 0) + (rb == b ? 1 : 0);
    incl[b - 1] = wave_incl_scan(nb);
    if (lane == 63) scratch[16 * (b - 1) + wv] = incl[b - 1];
    incl[b - 1] -= nb;
  }
  __syncthreads();
  if (wv < MB) {
    const int v = lane < nwv ? scratch[16 * wv + lane] : 0;
    const int w = wave_incl_scan(v);
    if (lane < nwv) scratch[16 * wv + lane] = w;
  }
  __syncthreads();
  int total = 0;
  for (int b = 1; b <= MB; ++b) {
    sk[b - 1][a] = (wv ? scratch[16 * (b - 1) + wv - 1] : 0) + incl[b - 1];
    const int tb = scratch[16 * (b - 1) + nwv - 1];
    if (a == 0) sk[b - 1][1024] = tb;
    total += tb;
  }
  __syncthreads();
  const int CC = C > 0 ? C : (A > 0 ? A : 1);
  if (e >= 0) {
    const int c0 = a / CC * CC;                      // this chunk's experts [c0, c1)
    const int c1 = min(c0 + CC, A);
    int j = 0;                                        // tiles before the chunk
    for (int b = 1; b <= MB; ++b) j += sk[b - 1][c0];
    if (a == c0) chunk_first[a / CC] = j;
    const int r0 = offsets[e];
    for (int b = MB; b >= 1; --b) {
      const int lo = sk[b - 1][c0];
      int t = j + sk[b - 1][a] - lo;
      if (b == MB)
        for (int i = 0; i < nfull; ++i) tiles[t++] = make_int4(e, r0 + i * MT, MT, a);
      if (rb == b) tiles[t] = make_int4(e, r0 + nfull * MT, rem, a);
      j += sk[b - 1][c1] - lo;
    }
  }
  // chunks past the last live one (up to entry E + 1) are empty: their
  // bounds both read `total`, so a chunk loop of fixed length needs no host
  // read-back of the active count
  const int nch = (A + CC - 1) / CC;
  for (int c = nch + a; c <= E + 1; c += blockDim.x) chunk_first[c] = total;
  if (a == 0) {
    work[0] = 0;
    work[1] = 0;
  }
}

__global__ __launch_bounds__(1024) void k_tile_plan(const int32_t* __restrict__ counts,
                                                    const int32_t* __restrict__ offsets,
                                                    const int32_t* __restrict__ active,
                                                    const int32_t* __restrict__ n_active, int MT,
                                                    int C, int4* __restrict__ tiles,
                                                    int32_t* __restrict__ chunk_first, int E,
                                                    int32_t* __restrict__ work) {
  __shared__ int scratch[64];
  __shared__ int sk[4][1025];
  tile_plan_body(counts, offsets, active, n_active, MT, C, tiles, chunk_first, scratch, sk, E,
                 work);
}

// Permutation of at most kTiny pairs in one workgroup without rank loops:
// counts by LDS atomics, then wavefront w places the pairs of active experts
// w, w + 16, ...: every wavefront holds all ids in registers (64 pairs per
// register), so one ballot per 64 pairs finds an expert's pairs in order and
// a pair's rank inside its expert is a population count over the lower lanes
// plus the running count of earlier ballots.
constexpr int kTiny = 1024;

__global__ __launch_bounds__(1024) void k_perm_tiny(const int32_t* __restrict__ ids, int64_t P,
                                                    int E, int32_t* __restrict__ blk,
                                                    PermPtrs pp, int32_t* __restrict__ err,
                                                    int MT, int C, int4* __restrict__ tiles,
                                                    int32_t* __restrict__ chunk_first,
                                                    int32_t* __restrict__ work) {
  extern __shared__ int cnt[];       // [E]
  __shared__ int scratch[64];
  __shared__ int sk[4][1025];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int np = (int)P;
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  int r[kTiny / 64];                 // r[c] = id of pair 64 c + lane (-1: none)
#pragma unroll
  for (int c = 0; c < kTiny / 64; ++c) r[c] = load_id(ids, 64 * c + lane, P, E, nullptr);
  __syncthreads();
  {
    const int i = threadIdx.x;       // this thread's pair (for counts and errors)
    const int e = load_id(ids, i, P, E, err);
    if (e >= 0) atomicAdd(&cnt[e], 1);
    else if (i < np) pp.inv_perm[i] = -1;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) blk[e] = cnt[e];
  __syncthreads();
  perm_scan_body(1, E, blk, pp.counts, pp.offsets, pp.active, pp.n_active, scratch);
  __syncthreads();
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  const int nact = *pp.n_active;
  for (int a = wave; a < nact; a += 16) {
    const int e = pp.active[a];
    int run = pp.offsets[e];
#pragma unroll
    for (int c = 0; c < kTiny / 64; ++c) {
      const bool hit = r[c] == e;
      const uint64_t mask = __ballot(hit);
      if (hit) {
        const int pos = run + __popcll(mask & below);
        pp.perm[pos] = 64 * c + lane;
        pp.inv_perm[64 * c + lane] = pos;
      }
      run += __popcll(mask);
    }
  }
  if (MT > 0) {
    __syncthreads();
    tile_plan_body(pp.counts, pp.offsets, pp.active, pp.n_active, MT, C, tiles, chunk_first,
                   scratch, sk, E, work);
  }
}

// ------------------------------------------------------------- launchers

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* gates,
                        int32_t* err, hipStream_t s) {
  TimedLaunch timed_(kLRoute, s);
  if (T == 0) return hipSuccess;
  const dim3 grid((T + 3) / 4);
  if (E <= 64) hipLaunchKernelGGL(k_route<1>, grid, dim3(256), 0, s, logits, T, E, k, ids, gates, err);
  else if (E <= 128) hipLaunchKernelGGL(k_route<2>, grid, dim3(256), 0, s, logits, T, E, k, ids, gates, err);
  else if (E <= 256) hipLaunchKernelGGL(k_route<4>, grid, dim3(256), 0, s, logits, T, E, k, ids, gates, err);
  else if (E <= 512) hipLaunchKernelGGL(k_route<8>, grid, dim3(256), 0, s, logits, T, E, k, ids, gates, err);
  else hipLaunchKernelGGL(k_route<16>, grid, dim3(256), 0, s, logits, T, E, k, ids, gates, err);
  return hipGetLastError();
}

hipError_t launch_router_bwd(const float* gpart, int nitems, const int32_t* inv_perm,
                             const int32_t* ids, const float* gates, int T, int E, int k,
                             float* dgates, float* dlogits, hipStream_t s) {
  TimedLaunch timed_(kLRouterBwd, s);
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(k_router_bwd, dim3((T + 3) / 4), dim3(256), 0, s, gpart, nitems, inv_perm,
                     ids, gates, T, E, k, dgates, dlogits);
  return hipGetLastError();
}

size_t permute_ws_bytes(int64_t P, int E) {
  const int64_t nblk = (P + kSeg - 1) / kSeg;
  return (size_t)std::max<int64_t>(nblk, 1) * E * sizeof(int32_t);
}

hipError_t launch_permute_plan(const int32_t* ids, int64_t P, int E, const PermPtrs& pp,
                               int32_t* err, void* ws, int MT, int C, int4* tiles,
                               int32_t* chunk_first, hipStream_t s) {
  TimedLaunch timed_(kLPermute, s);
  if (P <= kTiny) {
    hipLaunchKernelGGL(k_perm_tiny, dim3(1), dim3(1024), E * sizeof(int), s, ids, P, E,
                       static_cast<int32_t*>(ws), pp, err, MT, C, tiles, chunk_first,
                       chunk_first ? chunk_first + E + 2 : nullptr);
    return hipGetLastError();
  }
  const int nblk = (int)((P + kSeg - 1) / kSeg);
  int32_t* blk = static_cast<int32_t*>(ws);
  hipLaunchKernelGGL(k_perm_count, dim3(nblk), dim3(1024), E * sizeof(int), s, ids, P, E, blk,
                     err, pp.inv_perm);
  hipLaunchKernelGGL(k_perm_scan, dim3(1), dim3(1024), 0, s, nblk, E, blk, pp.counts, pp.offsets,
                     pp.active, pp.n_active);
  hipLaunchKernelGGL(k_perm_place, dim3((E + 3) / 4, nblk), dim3(256), 0, s, ids, P, E, blk,
                     pp.counts, pp.offsets, pp.perm, pp.inv_perm);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || MT <= 0) return e;
  return launch_tile_plan(pp, E, MT, C, tiles, chunk_first, s);
}

hipError_t launch_permute(const int32_t* ids, int64_t P, int E, const PermPtrs& pp, int32_t* err,
                          void* ws, hipStream_t s) {
  return launch_permute_plan(ids, P, E, pp, err, ws, 0, 0, nullptr, nullptr, s);
}

hipError_t launch_gather(const uint16_t* x, int d, const PermPtrs& pp, int E, int k, int64_t P,
                         uint16_t* out, hipStream_t s) {
  TimedLaunch timed_(kLOther, s);
  if (P == 0) return hipSuccess;
  hipLaunchKernelGGL(k_gather_rows, dim3((unsigned)((P + 3) / 4)), dim3(256), 0, s, x, d,
                     pp.perm, pp.offsets, E, k, out);
  return hipGetLastError();
}

hipError_t launch_tile_plan(const PermPtrs& pp, int E, int MT, int C, int4* tiles,
                            int32_t* chunk_first, hipStream_t s) {
  TimedLaunch timed_(kLPermute, s);
  hipLaunchKernelGGL(k_tile_plan, dim3(1), dim3(1024), 0, s, pp.counts, pp.offsets, pp.active,
                     pp.n_active, MT, C, tiles, chunk_first, E, chunk_first + E + 2);
  return hipGetLastError();
}

}  // namespace qgg
