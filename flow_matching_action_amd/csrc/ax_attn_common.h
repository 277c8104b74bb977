// Device-side pieces shared by the attention kernels (the expert step over bf16 and fp8 caches,
// ax_attn.hip; the text-model decode step, ax_decode.hip): the block tiles' swizzles, the LDS
// hand-off counters and bounded waits, the workspace status word, the float16 partial packing and
// the e4m3 conversions.
#pragma once
#include "ax_dev.h"

namespace ax {

constexpr int kBlk = 32;                      // keys per block
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescale = 8.0f;              // lazy-rescale threshold (log2 units)
constexpr int kNonTemporal = 2;               // cache-policy operand of a load: nt

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef int v8i32 __attribute__((ext_vector_type(8)));  // 32 fp8 codes: an f8f6f4 MFMA operand
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;

// Chunk swizzles (16-byte chunk index within a 256-byte bf16 row). Query rows are read by
// consecutive lanes from consecutive rows: all 4 row bits.
__device__ __forceinline__ int qswz(int r) { return r & 15; }
// K and V rows of a 32-key block tile (16 chunks of 16 bytes a row). LDS serves a ds_read_b128
// for 16 lanes per cycle and a ds_read_b64_tr_b16 for 32, all 64 banks at once, so those lanes
// must hit 16 distinct chunks; the swizzles also keep 8-lane (b128) and 16-lane (tr) halves on 8
// distinct chunks of one 128-byte half, the other half taking the other 8.
// K: lanes 0..15 read rows 0..15 (or 16..31) at one chunk c: row r's chunk c sits at c ^ (r & 15).
__device__ __forceinline__ int kswz16(int r) { return r & 15; }
// V: the 32 lanes of two 16-lane transpose groups read rows 0..7 (mod 16) at chunks 2 dt and
// 2 dt + 1: 2 (r & 7) moves the pair to 2 (dt ^ (r & 7)), a distinct pair per row, with rows 0..3
// in one half and rows 4..7 in the other.
__device__ __forceinline__ int vswz16(int r) { return 2 * (r & 7); }
// A lane's value and that of lane ^ 32, in either order: v_permlane32_swap exchanges the upper
// half of one operand with the lower half of the other, so fed the same value twice, each of
// its two results holds one of the pair in every lane. A VALU exchange, unlike ds_bpermute.
__device__ __forceinline__ float2 pair32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return float2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}

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
// allow.
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


typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
// Four floats to float16 (nearest even) in two 32-bit words.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2 pack_f16x4(float a, float b, float c, float d) {
  const f16x4 v = {(_Float16)a, (_Float16)b, (_Float16)c, (_Float16)d};  // nearest even
  return __builtin_bit_cast(u32x2, v);
}
constexpr float kE4m3Max = 448.0f;

// 8 e4m3 codes (bytes of w0, then w1) -> 8 bf16, exactly.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Per-row e4m3 quantisation of a 128-wide row held by a group of 16 lanes (8 values each):
// scale = max |x| / 448 (1 for an all-zero row), codes = nearest-even e4m3 of x / scale,
// saturated to +-448 (v_cvt_pk_fp8_f32 rounds to nearest even and does not saturate, hence
// the clamp). Divisions are float32, correctly rounded. All 16 lanes must call together.
__device__ __forceinline__ uint2 quant_row16(const float* x, float& scale) {
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[e]));
  m = fmaxf(m, row_ror<8>(m));
  m = fmaxf(m, row_ror<4>(m));
  m = fmaxf(m, row_ror<2>(m));
  m = fmaxf(m, row_ror<1>(m));
  scale = m > 0.f ? m / kE4m3Max : 1.0f;
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = fminf(fmaxf(x[e] / scale, -kE4m3Max), kE4m3Max);
  int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w0, true);
  int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], w1, true);
  return make_uint2((uint32_t)w0, (uint32_t)w1);
}

// The fp8-cache kernel folds the value scales into P with a fixed factor 2^kF8VShift (the
// products p * scale * 2^64 stay in bf16's normal range for every float32 scale from the
// denormals up to 2^25), so its O accumulates in units of 2^-64; the stored exponent takes the
// factor back out.
constexpr int kF8VShift = 64;

}  // namespace ax
