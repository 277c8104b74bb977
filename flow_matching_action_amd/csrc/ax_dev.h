// Device-side helpers shared by the gfx950 kernels of libax.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace ax {

constexpr int kHq = 16;       // query heads
constexpr int kHkv = 8;       // kv heads
constexpr int kT = 64;        // expert tokens
constexpr int kD = 128;       // head dim
constexpr int kRep = kHq / kHkv;
constexpr int kQRows = kRep * kT;  // folded query rows per kv head

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Compile-time loop: f(std::integral_constant<int, I>{}) for I = 0 .. N-1, so that
// register arrays indexed by I never need to live in private memory.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float32 -> bf16 bits, nearest-even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair (low = lo), nearest-even: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Unpack 8 bf16 held in a uint4 into floats.
__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ uint4 pack8(const float* f) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                    pack_bf16x2(f[6], f[7]));
}

// Value of lane (i + N) mod 16 within each row of 16 lanes (DPP row_ror, a plain VALU
// move; no LDS round trip).
template <int N>
__device__ __forceinline__ float row_ror(float x) {
  static_assert(N > 0 && N < 16, "row_ror");
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x120 + N, 0xf, 0xf, false));
}

// RMSNorm + rotate_half RoPE of one 128-wide row held by a group of 16 consecutive
// lanes, 8 elements per lane (lane j16 holds columns 8*j16 .. 8*j16+7). The row partner
// of column c +- 64 sits 8 lanes away. All lanes of the wave must call these together.
//
// With y = x * inv * gamma (inv = 1/sqrt(mean(x^2) + eps)), the rotation of column j < 64 is
// y_j cos_j - y_{j+64} sin_j and of column j + 64 is y_{j+64} cos_j + y_j sin_j, so
//   out_e = inv * (x_e * A_e + x'_e * B_e),  A_e = gamma_e cos_e,  B_e = -+ gamma'_e sin_e
// where ' is the partner column; A and B depend only on the token and the gamma vector and
// are formed once per token (rope_coef), the per-row work is norm_rope_row16.
// g: the 8 gammas; c, s: cos/sin for columns (8*j16+e) mod 64.
__device__ __forceinline__ void rope_coef(const float* g, const float* c, const float* s, int j16, float* A,
                                          float* B) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float gp = row_ror<8>(g[e]);
    A[e] = g[e] * c[e];
    B[e] = ((j16 < 8) ? -gp : gp) * s[e];  // lower half: x c - x' s; upper half: x c + x' s
  }
}

// x: the 8 inputs, replaced by the outputs. The sum of squares is a rotate-by-8/4/2/1
// butterfly, which leaves the same bits in all 16 lanes.
__device__ __forceinline__ void norm_rope_row16(float* x, const float* A, const float* B, float eps) {
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
  ss += row_ror<8>(ss);
  ss += row_ror<4>(ss);
  ss += row_ror<2>(ss);
  ss += row_ror<1>(ss);
  const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / kD) + eps);  // v_rsq_f32
  float p[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) p[e] = row_ror<8>(x[e]);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = inv * __builtin_fmaf(p[e], B[e], x[e] * A[e]);
}

// The same RMSNorm + RoPE in the pair layout: lane j16 of a row's 16-lane group holds
// columns 4 j16 .. +3 (x[0..3]) and 64 + 4 j16 .. +3 (x[4..7]), so both members of every
// RoPE pair (j, j + 64) sit in one lane and the rotation needs no lane moves; the RoPE rows
// a lane needs are the 4 frequencies 4 j16 .. +3, one float4 of cosines and one of sines.
// g: the 8 gammas in that layout; c, s: cos/sin of frequencies 4 j16 .. +3.
__device__ __forceinline__ void rope_coef_pair(const float* g, const float* c, const float* s, float* A,
                                               float* B) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    A[e] = g[e] * c[e];              // column j:      x_j c_j - x_{j+64} s_j
    B[e] = (-g[4 + e]) * s[e];
    A[4 + e] = g[4 + e] * c[e];      // column j + 64: x_{j+64} c_j + x_j s_j
    B[4 + e] = g[e] * s[e];
  }
}

// x: the 8 inputs in the pair layout, replaced by the outputs. The sum of squares is a
// rotate-by-8/4/2/1 butterfly over the 16 lanes, which leaves the same bits in all of them.
__device__ __forceinline__ void norm_rope_pair(float* x, const float* A, const float* B, float eps) {
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
  ss += row_ror<8>(ss);
  ss += row_ror<4>(ss);
  ss += row_ror<2>(ss);
  ss += row_ror<1>(ss);
  const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / kD) + eps);  // v_rsq_f32
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = inv * __builtin_fmaf(x[e ^ 4], B[e], x[e] * A[e]);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = y[e];
}

// norm_rope_pair with the result multiplied by post (folded into the row's 1/rms), for a row
// that feeds a product whose scale is applied here instead of on every product.
__device__ __forceinline__ void norm_rope_pair_scaled(float* x, const float* A, const float* B, float eps,
                                                      float post) {
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
  ss += row_ror<8>(ss);
  ss += row_ror<4>(ss);
  ss += row_ror<2>(ss);
  ss += row_ror<1>(ss);
  const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / kD) + eps) * post;
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = inv * __builtin_fmaf(x[e ^ 4], B[e], x[e] * A[e]);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = y[e];
}

// Pair-layout row access: the lane's two 8-byte pieces (4 bf16 each) of a bf16 row.
__device__ __forceinline__ void unpack_pair(const uint2& lo, const uint2& hi, float* x) {
  x[0] = __uint_as_float(lo.x << 16); x[1] = __uint_as_float(lo.x & 0xffff0000u);
  x[2] = __uint_as_float(lo.y << 16); x[3] = __uint_as_float(lo.y & 0xffff0000u);
  x[4] = __uint_as_float(hi.x << 16); x[5] = __uint_as_float(hi.x & 0xffff0000u);
  x[6] = __uint_as_float(hi.y << 16); x[7] = __uint_as_float(hi.y & 0xffff0000u);
}
__device__ __forceinline__ void pack_pair(const float* x, uint2& lo, uint2& hi) {
  lo = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
  hi = make_uint2(pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7]));
}
// Byte offsets of the two pieces in a 256-byte row whose 16-byte chunks are XOR-swizzled by
// sw (chunk c of the row lives at chunk c ^ sw).
__device__ __forceinline__ int pair_off_lo(int j16, int sw) { return 16 * ((j16 >> 1) ^ sw) + 8 * (j16 & 1); }
__device__ __forceinline__ int pair_off_hi(int j16, int sw) { return 16 * ((8 + (j16 >> 1)) ^ sw) + 8 * (j16 & 1); }

}  // namespace ax
