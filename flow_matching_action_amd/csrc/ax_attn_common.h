// Device-side pieces shared by the split-KV attention kernels (bf16 and fp8 caches):
// launch shape, the LDS hand-off counters, the MFMA operand layouts, and the query
// norm/RoPE helpers. The kernels themselves are in ax_attn.hip and ax_attn_f8.hip.
#pragma once
#include "ax_dev.h"

namespace ax {

constexpr int kBlk = 32;                      // keys per block
constexpr int kQBytes = kQRows * kD * 2;      // 32 KB: the 128 query rows in bf16
constexpr int kComputeWaves = 8;
constexpr int kLoaderWaves = 4;
constexpr int kThreads = 64 * (kComputeWaves + kLoaderWaves);
constexpr int kMaxBlocks = 12;                // blocks per split in any kernel variant
// LDS hand-off counters: queries normed, query fragments read, block b landed, block b
// consumed, merge data of query group q ready
constexpr int kCntQNormed = 0, kCntQRead = 1, kCntBlock = 2;
constexpr int kCntDone = kCntBlock + kMaxBlocks, kCntMerge = kCntDone + kMaxBlocks, kNCnt = kCntMerge + 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescale = 8.0f;              // lazy-rescale threshold (log2 units)
constexpr int kNonTemporal = 2;               // cache-policy operand of a load: nt

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;

// Chunk swizzles (16-byte chunk index within a row: 16 chunks in a bf16 row, 8 in an fp8 row).
// Query rows are read by consecutive lanes from consecutive rows: all 4 row bits.
__device__ __forceinline__ int qswz(int r) { return r & 15; }
// K rows are read by 8-lane groups from rows {0..3, 8..11} + 4j (the MFMA row order pi below):
// bits 0, 1 and 3 of the row make those 8 rows hit 8 distinct 16-byte bank groups. The
// swizzle stays below 8, so chunks c and c + 8 keep their 128-byte distance.
__device__ __forceinline__ int kswz(int r) { return (r & 3) | ((r >> 1) & 4); }
// V rows of a bf16 tile: the swizzle only depends on row & 3, so all transpose reads of a
// lane share two base addresses (t even / odd) plus immediate offsets, and still spread a
// 16-lane group over 8 distinct chunks.
__device__ __forceinline__ int vswz(int r) { return 2 * (r & 3); }
// A lane's value and that of lane ^ 32, in either order: v_permlane32_swap exchanges the upper
// half of one operand with the lower half of the other, so fed the same value twice, each of
// its two results holds one of the pair in every lane. A VALU exchange, unlike ds_bpermute.
__device__ __forceinline__ float2 pair32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return float2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// Row order inside a 32-key block seen by the MFMA: swap bits 2 and 3.
__device__ __forceinline__ int perm_key(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// Head-dim chunk (8 columns) used by k-step kk in lane half h: half h holds columns
// [32h, 32h+32) and [64+32h, 96+32h), so a RoPE pair (j, j+64) stays in one lane.
__device__ __forceinline__ int dcol(int kk, int h) { return (kk < 4) ? 32 * h + 8 * kk : 64 + 32 * h + 8 * (kk - 4); }

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding: vmcnt bits [3:0]
// and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}

// Workgroup barrier for LDS hand-offs: this wave's LDS writes are complete (lgkmcnt), then
// s_barrier; the memory clobber keeps the compiler from moving memory accesses across it.
// Unlike __syncthreads() there is no release fence, which would also drain this wave's
// direct-to-LDS loads of later blocks (callers wait for exactly the loads they need).
// The scheduling fences keep the compiler from hoisting arithmetic (and the waits for its
// operands) above the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// In-workgroup hand-off counters in LDS. A producer wave bumps a counter once its data is
// in LDS; consumers poll it. Unlike s_barrier this never makes a producer wait for its
// consumers, so the cache stream runs ahead of the arithmetic as far as the LDS tiles
// allow (tiles are never reused within a launch, so there is nothing to wait for).
// The increment is written as inline asm: the compiler cannot tell an LDS atomic from the
// direct-to-LDS loads still in flight and would drain them all (vmcnt(0)) before it.
typedef __attribute__((address_space(3))) int lds_int;
__device__ __forceinline__ void arrive(int* cnt, int lane) {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's own LDS writes come first
  if (lane == 0) {
    const unsigned off = (unsigned)(uintptr_t)(lds_int*)cnt;
    asm volatile("ds_add_u32 %0, %1" ::"v"(off), "v"(1) : "memory");
  }
  __builtin_amdgcn_sched_barrier(0);
}

// The wait is bounded (about 30 ms at 2.4 GHz, thousands of times any real wait) so that a
// wave always exits even if a count were wrong. A wave whose wait runs out carries on with
// whatever LDS holds, remembers it in expired, and reports it through the workspace status
// word (report_expired), so a wrong count shows instead of passing as output. The bound is a
// kernel argument: a host-side debug setting can shrink it to force the path without a hang.
__device__ __forceinline__ void await(int* cnt, int n, int limit, bool& expired) {
  __builtin_amdgcn_sched_barrier(0);
  int spin = limit;
#pragma clang loop unroll(disable)
  while (__builtin_amdgcn_readfirstlane(__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) < n) {
    if (--spin <= 0) {
      expired = true;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Workspace status word (the first 4 bytes of every workspace; the first 256 bytes are
// reserved for it): flags OR-ed in by the kernels, never cleared by them.
constexpr int kStatusWaitExpired = 1;
constexpr size_t kStatusBytes = 256;
__device__ __forceinline__ void report_expired(int* status, bool expired, int lane) {
  if (expired && lane == 0) __hip_atomic_fetch_or(status, kStatusWaitExpired, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// RoPE table values of token tok for the 8 frequencies 8 (j16 & 7) .. +7: lanes j16 < 8 load
// the cosines, lanes j16 >= 8 the sines, and the partner lane (j16 ^ 8, same frequencies)
// hands over the other half, so each table byte is requested once per row group.
__device__ __forceinline__ void load_cos_sin_half(const float* cos_t, const float* sin_t, int tok, int j16,
                                                  f32x4& h0, f32x4& h1) {
  const float* src = ((j16 < 8) ? cos_t : sin_t) + tok * 64 + 8 * (j16 & 7);
  h0 = reinterpret_cast<const f32x4*>(src)[0];
  h1 = reinterpret_cast<const f32x4*>(src)[1];
}

__device__ __forceinline__ void split_cos_sin(const f32x4& h0, const f32x4& h1, int j16, float* c, float* s) {
  const bool lo = j16 < 8;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float mine = (e < 4) ? h0[e & 3] : h1[e & 3];
    const float other = row_ror<8>(mine);
    c[e] = lo ? mine : other;
    s[e] = lo ? other : mine;
  }
}

__device__ __forceinline__ void unpack8v(const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ u32x4 pack8v(const float* f) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  return r;
}


// RMSNorm + RoPE in place in LDS of the query rows 32p + r16 (p = 0..3) that this lane's
// 16-lane group holds, in the pair layout (columns 4 j16 .. +3 and 64 + 4 j16 .. +3), rows
// swizzled by qswz. graw: the lane's 8 gammas in that layout; cs[t]: cos, sin of frequencies
// 4 j16 .. +3 of token set t = p & 1. All rows are read before any is written back.
__device__ __forceinline__ void norm_rope_query_rows(uint8_t* qlds, const uint2 (&graw)[2], const f32x4 (&cs)[2][2],
                                                     int j16, int r16, float eps) {
  float qg[8], A[2][8], B[2][8];
  unpack_pair(graw[0], graw[1], qg);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float c[4] = {cs[t][0][0], cs[t][0][1], cs[t][0][2], cs[t][0][3]};
    const float sn[4] = {cs[t][1][0], cs[t][1][1], cs[t][1][2], cs[t][1][3]};
    rope_coef_pair(qg, c, sn, A[t], B[t]);
  }
  uint2 lo[4], hi[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = 32 * p + r16;
    lo[p] = *reinterpret_cast<const uint2*>(qlds + r * 256 + pair_off_lo(j16, qswz(r)));
    hi[p] = *reinterpret_cast<const uint2*>(qlds + r * 256 + pair_off_hi(j16, qswz(r)));
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    float x[8];
    unpack_pair(lo[p], hi[p], x);
    norm_rope_pair(x, A[p & 1], B[p & 1], eps);
    pack_pair(x, lo[p], hi[p]);
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = 32 * p + r16;
    *reinterpret_cast<uint2*>(qlds + r * 256 + pair_off_lo(j16, qswz(r))) = lo[p];
    *reinterpret_cast<uint2*>(qlds + r * 256 + pair_off_hi(j16, qswz(r))) = hi[p];
  }
}


// Split partials in float16. O is stored as O 2^-e per (split, query row), with 2^e the power of
// two just above the row's largest |O| (max |O 2^-e| in [0.5, 1)); e is stored beside the row's
// m and l, which stay float32 and unscaled. The scaling is ldexp, exact for every finite O
// (denormal ones included: e >= -149 and |O 2^-e| < 1), so nothing overflows whatever the
// magnitudes; the combine multiplies the row's weight by 2^e. Float16 then keeps 11 significant
// bits of every element within 2^14 of the row's largest |O| (its normal range), and smaller
// elements an absolute error below 2^-25 of that largest value.
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2 pack_f16x4(float a, float b, float c, float d) {
  const f16x4 v = {(_Float16)a, (_Float16)b, (_Float16)c, (_Float16)d};  // nearest even
  return __builtin_bit_cast(u32x2, v);
}
__device__ __forceinline__ f32x4 unpack_f16x4(const u32x2& u) {
  const f16x4 v = __builtin_bit_cast(f16x4, u);
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

// The fp8 kernel folds the value scales into P with a fixed factor 2^kF8VShift (the products
// p * scale * 2^64 stay in bf16's normal range for every float32 scale from the denormals up to
// 2^25), so its O accumulates in units of 2^-64; the stored exponent takes the factor back out.
constexpr int kF8VShift = 64;

// Store of one wave's partial for query rows 32 qgrp .. +31 (lane (n, h): row n, the half h of
// the accumulator layout): O at po + ((part * 4 + qgrp) * 16 + j) * 64 + lane in 8-byte units
// (slot j = 4t + jj, 4 float16 each, non-temporal: the combine reads it once), m, l and e at
// pm / pl / pe + part * 128 + query row. l_tot is the row's whole sum (both halves); O is in
// units of 2^-kF8VShift, so e - kF8VShift is stored.
__device__ __forceinline__ void store_partial_f16(const f32x16 (&o)[4], float m, float l_tot, int qgrp, int lane,
                                                  float* po_all, float* pm, float* pl, int* pe, long long part) {
  const int n = lane & 31;
  const int h = lane >> 5;
  float amax = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(o[t][i]));
  const float2 ap = pair32(amax);
  const int e = __builtin_amdgcn_frexp_expf(fmaxf(ap.x, ap.y));  // 0 for an all-zero row
  u32x2* po = reinterpret_cast<u32x2*>(po_all) + (part * 4 + qgrp) * (16 * 64) + lane;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      __builtin_nontemporal_store(pack_f16x4(__builtin_ldexpf(o[t][4 * jj], -e), __builtin_ldexpf(o[t][4 * jj + 1], -e),
                                             __builtin_ldexpf(o[t][4 * jj + 2], -e),
                                             __builtin_ldexpf(o[t][4 * jj + 3], -e)),
                                  &po[(4 * t + jj) * 64]);
  if (h == 0) {
    const int qrow = 32 * qgrp + n;
    __builtin_nontemporal_store(m, &pm[part * kQRows + qrow]);
    __builtin_nontemporal_store(l_tot, &pl[part * kQRows + qrow]);
    __builtin_nontemporal_store(e - kF8VShift, &pe[part * kQRows + qrow]);
  }
}

// End of a split: the two parity waves of query group qgrp hold (m, l, O) over disjoint
// blocks. The odd wave hands its O (16 KB: slot j = 4t + jj of the accumulator layout, 1 KB
// per slot, slots 0..7 at xlo and 8..15 at xhi) and (m, l) to the even one through LDS, once
// region_free() says nobody reads those regions any more; the even wave rescales both to
// the larger m and stores the split's partial (store_partial_f16). With a single block
// (two_parities false) the odd wave holds nothing.
template <typename RegionFree>
__device__ __forceinline__ void merge_and_store_partial(f32x16 (&o)[4], float m_run, float l_run,
                                                        bool two_parities, int par, int qgrp, int lane,
                                                        uint8_t* xlo, uint8_t* xhi, RegionFree&& region_free,
                                                        float (*mlx)[2][32], int* cnt, float* po_all,
                                                        float* pm, float* pl, int* pe, long long part,
                                                        int limit, bool& expired) {
  const int n = lane & 31;
  const int h = lane >> 5;
  const float2 l_pair = pair32(l_run);
  const float l_tot = l_pair.x + l_pair.y;
  if (!two_parities) {
    if (par == 1) return;
    store_partial_f16(o, expired ? __builtin_nanf("") : m_run, l_tot, qgrp, lane, po_all, pm, pl, pe, part);
    return;
  }
  auto slot = [&](int j) { return reinterpret_cast<f32x4*>(j < 8 ? xlo + j * 1024 : xhi + (j - 8) * 1024) + lane; };
  if (par == 1) {
    region_free();
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        *slot(4 * t + jj) = f32x4{o[t][4 * jj], o[t][4 * jj + 1], o[t][4 * jj + 2], o[t][4 * jj + 3]};
    if (h == 0) {
      mlx[qgrp][0][n] = m_run;
      mlx[qgrp][1][n] = l_tot;
    }
    arrive(&cnt[kCntMerge + qgrp], lane);
    return;
  }
  await(&cnt[kCntMerge + qgrp], 1, limit, expired);
  const float m_o = mlx[qgrp][0][n];
  const float l_o = mlx[qgrp][1][n];
  const float m_new = fmaxf(m_run, m_o);  // m_run is finite: block 0 holds a visible key
  const float ae = __builtin_amdgcn_exp2f(m_run - m_new);
  const float ao = __builtin_amdgcn_exp2f(m_o - m_new);  // 0 if the odd wave saw no key
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const f32x4 x = *slot(4 * t + jj);
#pragma unroll
      for (int e = 0; e < 4; ++e) o[t][4 * jj + e] = ae * o[t][4 * jj + e] + ao * x[e];
    }
  // an expired wait leaves this row's partial NaN (m), besides the status word
  store_partial_f16(o, expired ? __builtin_nanf("") : m_new, ae * l_tot + ao * l_o, qgrp, lane, po_all, pm, pl, pe,
                    part);
}

}  // namespace ax
