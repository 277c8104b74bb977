// The rest of one action-expert decoder layer around the attention step: the residual
// RMSNorms, the M = 64 projections (qkv, o, the SwiGLU MLP) and their epilogues.
//
// What is computed: page code/alpamayo_tt/EXPERT_NOTES.md, section "Layouts" (the per-layer op
// list and the weight shapes; weights stored input-major, [in, out]) and page
// code/alpamayo_tt/expert.py, TTExpert.layer. Every op hands a bf16 tensor to the next; inside an
// op the arithmetic is float32.
//
// gfx950 mapping
// - Weights are packed once (k_pack_w64) so that each 1 KB block holds, lane by lane, exactly the
//   16-byte W^T operand a lane hands v_mfma_f32_32x32x16_bf16 for one (32-column block, 16-row
//   step).
// - The weights are the stream (M = 64 is far below the ridge). Each wave loads its weight
//   operands straight into registers (one plain 16-byte load per lane and step, non-temporal)
//   while the workgroup's slice of A goes through LDS, runs one 32 x 32 tile of C^T = W^T A^T per
//   step, and the waves that split K inside the workgroup add their tiles through LDS.
// - k_gemm32: one 32-row half of the tokens per workgroup, the two halves of a column tile on one
//   XCD (the second weight read is an L2 hit). With all of K in the workgroup the epilogue runs in
//   place: qkv's head split into q/k/v [heads][64][128], or SiLU(g) * u with the gate and up
//   column blocks in the same workgroup, so no partial leaves it. The o projection takes it with
//   2 splits of K and float32 partials.
// - k_gemm64: all 64 rows per workgroup, K in splits with float32 partials (the down projection,
//   whose 6144 rows of K do not fit one workgroup's LDS, and any other shape).
// - k_reduce_residual_norm: a split sum, the residual add and the norm that follows, in one pass
//   per row (o: x2 and n2; down: x_out and, for a chained layer, the next layer's first norm);
//   k_rmsnorm_rows: the first norm; k_gemm_reduce: the plain split sum of a stand-alone product.
#include "ax_attn_common.h"
#include "ax_launch.h"

namespace ax {

constexpr int kGemmM = 64;      // token rows
constexpr int kNBlk = 32;       // columns of one weight block (the matrix-core tile's n)
constexpr int kMaxSplit = 256;

// Packed weight layout. W [K][N] (input-major) is stored as 1 KB blocks, one per (32-column block
// j, 16-row step s), at block index j * (K / 16) + s: a column block's steps are consecutive. In a
// block, the 16 bytes of lane l are W[16 s + 8 (l / 32) + e][32 j + l % 32], e = 0..7: exactly
// the W^T operand lane l hands v_mfma_f32_32x32x16_bf16, so one plain 16-byte load per lane
// fetches an operand, with no transpose and no LDS.
__global__ __launch_bounds__(256) void k_pack_w64(const uint16_t* W, int K, int N, uint16_t* Wp) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;  // 16-byte chunk of the packed layout
  const long long b = i >> 6;
  const int l = (int)(i & 63);
  const int steps = K / 16;
  const int j = (int)(b / steps), s = (int)(b % steps);
  const uint16_t* src = W + (long long)(16 * s + 8 * (l >> 5)) * N + kNBlk * j + (l & 31);
  uint16_t v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = src[(long long)e * N];
  u32x4 o;
  o[0] = v[0] | (uint32_t)v[1] << 16;
  o[1] = v[2] | (uint32_t)v[3] << 16;
  o[2] = v[4] | (uint32_t)v[5] << 16;
  o[3] = v[6] | (uint32_t)v[7] << 16;
  *reinterpret_cast<u32x4*>(Wp + i * 8) = o;
}

// A element (m, k): row-major [64][lda], or (heads = true) the attention output [16][64][128]
// read as its heads concatenated ([64][2048]: column 128 h + d of row m is head h, token m,
// element d).
__device__ __forceinline__ const uint16_t* a_elem(const uint16_t* A, int lda, int m, int k, bool heads) {
  return heads ? A + ((long long)(k >> 7) * kGemmM + m) * 128 + (k & 127) : A + (long long)m * lda + k;
}

// A slice rows in LDS are KC x 2 bytes; chunk c of row m sits at position c ^ (m & 15) (within its
// aligned group of 16 chunks), so the 16 rows a 16-lane group reads at one chunk hit 16 distinct
// 16-byte bank groups.
__device__ __forceinline__ int aswz(int c, int m) { return c ^ (m & 15); }

// One split of C = A W over NB column blocks of 32. The workgroup has NB x KW waves: wave (nb, kq)
// streams column block nb over its KW-th share of the split's KC = KW x STEPS x 16 rows, straight
// into registers (STEPS 1 KB loads per wave, all issued at the start and consumed in order), while
// the split's 64 x KC slice of A sits in LDS (loaded first, from L2, through registers: a
// direct-to-LDS load would make the compiler drain the whole weight stream before the first LDS
// read). Each wave makes C^T[32 n][64 m] with two matrix-core products per step (m halves); the
// KW waves of a column block then add their tiles in LDS in kq order and the first stores the
// split's float32 partial, part[split][64][N]. A is row-major [64][K].
template <int NB, int KW, int STEPS>
__global__ __launch_bounds__(64 * NB * KW) void k_gemm64(const uint16_t* A, const uint16_t* W, int K, int N,
                                                       float* part) {
  constexpr int KC = KW * STEPS * 16;
  constexpr int kCpr = KC / 8;                     // 16-byte chunks per A row
  static_assert(kCpr % 16 == 0, "A rows of at least 16 chunks");
  constexpr int kALoads = kGemmM * kCpr / 64;      // 1 KB loads of the A slice
  static_assert(kALoads % (NB * KW) == 0, "A slice split evenly over the waves");
  constexpr int kRedBytes = (KW - 1) * NB * 64 * 32 * 4;
  constexpr int kLds = kGemmM * KC * 2 > kRedBytes ? kGemmM * KC * 2 : kRedBytes;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int nb = wave % NB;
  const int kq = wave / NB;
  // consecutive ids take consecutive splits, so (ids landing on XCD id % 8) an XCD holds the same
  // splits of every column tile and reads only their slices of A
  const int n_split = K / KC;
  const int split = blockIdx.x % n_split;
  const int tile = blockIdx.x / n_split;
  const int k0 = split * KC;

  // the A slice first (plain loads into registers; stored to LDS once the weight loads are out):
  // chunk e of the slice, row m = e / kCpr, position e % kCpr, holds chunk aswz(e % kCpr, m)
  constexpr int kAPer = kALoads / (NB * KW);
  u32x4 av[kAPer];
#pragma unroll
  for (int j = 0; j < kAPer; ++j) {
    const int e = 64 * (j * (NB * KW) + wave) + lane;
    const int m = e / kCpr;
    const int c = aswz(e % kCpr, m);
    av[j] = *reinterpret_cast<const u32x4*>(A + (long long)m * K + k0 + 8 * c);
  }
  __builtin_amdgcn_sched_barrier(0);
  // then every weight operand of this wave, from a wave-uniform base
  const int jb = tile * NB + nb;
  const u32x4* wsrc = reinterpret_cast<const u32x4*>(W) + ((long long)jb * (K / 16) + k0 / 16 + kq * STEPS) * 64;
  u32x4 wv[STEPS];
#pragma unroll
  for (int s = 0; s < STEPS; ++s) wv[s] = __builtin_nontemporal_load(wsrc + s * 64 + lane);
  __builtin_amdgcn_sched_barrier(0);
  u32x4* alds = reinterpret_cast<u32x4*>(lds);
#pragma unroll
  for (int j = 0; j < kAPer; ++j) alds[64 * (j * (NB * KW) + wave) + lane] = av[j];
  __syncthreads();

  f32x16 acc[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[h][i] = 0.f;
  const int am0 = lane & 31;
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int c = 2 * (kq * STEPS + s) + (lane >> 5);
    bf16x8 wf;
    __builtin_memcpy(&wf, &wv[s], 16);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int m = 32 * h + am0;
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(lds + m * (KC * 2) + 16 * aswz(c, m));
      acc[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, af, acc[h], 0, 0, 0);
    }
  }

  // the KW waves of column block nb add their tiles in kq order
  if constexpr (KW > 1) {
    __syncthreads();  // every wave is done with the A slice; its LDS now holds the tiles
    f32x4* red = reinterpret_cast<f32x4*>(lds);
    if (kq > 0) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int a = 0; a < 4; ++a)
          red[(((kq - 1) * NB + nb) * 8 + 4 * h + a) * 64 + lane] =
              f32x4{acc[h][4 * a], acc[h][4 * a + 1], acc[h][4 * a + 2], acc[h][4 * a + 3]};
    }
    __syncthreads();
    if (kq > 0) return;
#pragma unroll
    for (int q = 1; q < KW; ++q)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x4 v = red[(((q - 1) * NB + nb) * 8 + 4 * h + a) * 64 + lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[h][4 * a + e] += v[e];
        }
  }
  // lane (m = lane % 32, g = lane / 32) holds C rows 32 h + m, columns 32 jb + 8a + 4g + (0..3)
  const int pcol = kNBlk * jb + 4 * (lane >> 5);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float* dst = part + ((long long)split * kGemmM + 32 * h + am0) * N + pcol;
#pragma unroll
    for (int a = 0; a < 4; ++a)
      __builtin_nontemporal_store(f32x4{acc[h][4 * a], acc[h][4 * a + 1], acc[h][4 * a + 2], acc[h][4 * a + 3]},
                                  reinterpret_cast<f32x4*>(dst + 8 * a));
  }
}

enum GemmEpilogue { kEpiQkvSplit = 1, kEpiSwiGlu = 3, kEpiPartial = 4 };

// One 32-row half of C = A W over the whole of K, with the op's epilogue applied in place, so no
// float32 partial leaves the workgroup. The workgroup has NB x KW waves; wave (nb, kq) streams
// column block nb over rows 16 STEPS kq .. 16 STEPS (kq + 1) of K straight into registers (a ring
// of D 1 KB loads in flight, D = STEPS: all at once) while the half's 32 x K slice of A goes
// through LDS (as in k_gemm64), and makes one 32 x 32 tile C^T[32 n][32 m] per step. The KW
// tiles of a column block are then added in kq order through LDS; epilogue item (p, a) (column
// block or block pair p, columns 8a .. 8a + 7 of it) goes to wave 4p + a.
// Grid: 16 ids per 8 column tiles, the two halves of a tile 8 ids apart, so both run on one XCD
// and the second read of the tile's weights is an L2 hit.
// kEpiQkvSplit: column blocks NB t .. NB t + NB - 1 of W0, bf16(C) into q / k / v
// [heads][64][128].
// kEpiSwiGlu: blocks (NB / 2) t + p of W0 (x w1, waves nb = p) and of W1 (x w3, nb = NB / 2 + p),
// out[m][32 j + c] = bf16(bf16(silu(C1)) * bf16(C3)), silu(g) = g / (1 + e^-g).
// kEpiPartial: K is cut into n_split splits of KC = 16 KW STEPS rows (blockIdx / (2 n_tiles) is the
// split); the split's float32 C goes to part[split][64][N] (summed by k_reduce_residual_norm).
// HEADS: A is the attention output [16][64][128] read as [64][2048] (a_elem).
template <int NB, int KW, int STEPS, int EPI, bool HEADS, int D = STEPS>
__global__ __launch_bounds__(64 * NB * KW) void k_gemm32(const uint16_t* A, const uint16_t* W0, const uint16_t* W1,
                                                       int N, uint16_t* out, uint16_t* out_k, uint16_t* out_v,
                                                       int Ktot, float* part) {
  static_assert(EPI == kEpiQkvSplit || EPI == kEpiSwiGlu || EPI == kEpiPartial, "k_gemm32 epilogue");
  constexpr bool kPairs = EPI == kEpiSwiGlu;
  static_assert(!kPairs || NB % 2 == 0, "SwiGLU takes column blocks in pairs");
  constexpr int kWaves = NB * KW;
  constexpr int kHalf = kPairs ? NB / 2 : NB;  // column blocks of W0 per tile
  constexpr int kItems = 4 * kHalf;
  static_assert(kItems <= kWaves, "one epilogue item per wave");
  static_assert(D >= 1 && D <= STEPS, "ring depth");
  constexpr int K = KW * STEPS * 16;                // rows of K per workgroup (all of K unless kEpiPartial)
  constexpr int kCpr = K / 8;                       // 16-byte chunks per A row
  static_assert(kCpr % 16 == 0, "A rows of at least 16 chunks");
  constexpr int kALoads = 32 * kCpr / 64;           // 1 KB loads of the A half
  static_assert(kALoads % kWaves == 0, "A half split evenly over the waves");
  constexpr int kRedBytes = kWaves * 4 * 64 * 16;  // every wave's tile, 16 floats per lane
  constexpr int kLds = 32 * K * 2 > kRedBytes ? 32 * K * 2 : kRedBytes;
  static_assert(kLds <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int nb = wave % NB;
  const int kq = wave / NB;
  const int n_tiles = N / (kNBlk * kHalf);
  const int split = EPI == kEpiPartial ? blockIdx.x / (2 * n_tiles) : 0;
  const int b = EPI == kEpiPartial ? blockIdx.x % (2 * n_tiles) : blockIdx.x;
  const int tile = (b >> 4) * 8 + (b & 7);
  const int mh = (b >> 3) & 1;
  const int lda = EPI == kEpiPartial ? Ktot : K;
  const int k0 = split * K;

  constexpr int kAPer = kALoads / kWaves;
  u32x4 av[kAPer];
#pragma unroll
  for (int j = 0; j < kAPer; ++j) {
    const int e = 64 * (j * kWaves + wave) + lane;
    const int m = e / kCpr;
    const int c = aswz(e % kCpr, m);
    av[j] = *reinterpret_cast<const u32x4*>(a_elem(A, lda, 32 * mh + m, k0 + 8 * c, HEADS));
  }
  __builtin_amdgcn_sched_barrier(0);
  const uint16_t* W = (kPairs && nb >= kHalf) ? W1 : W0;
  const int jb = tile * kHalf + nb % kHalf;
  const u32x4* wsrc =
      reinterpret_cast<const u32x4*>(W) + ((long long)jb * (lda / 16) + k0 / 16 + kq * STEPS) * 64;
  u32x4 wv[D];
#pragma unroll
  for (int s = 0; s < D; ++s) wv[s] = __builtin_nontemporal_load(wsrc + s * 64 + lane);
  __builtin_amdgcn_sched_barrier(0);
  u32x4* alds = reinterpret_cast<u32x4*>(lds);
#pragma unroll
  for (int j = 0; j < kAPer; ++j) alds[64 * (j * kWaves + wave) + lane] = av[j];
  __syncthreads();

  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  const int am0 = lane & 31;
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int c = 2 * (kq * STEPS + s) + (lane >> 5);
    bf16x8 wf;
    __builtin_memcpy(&wf, &wv[s % D], 16);
    const bf16x8 af = *reinterpret_cast<const bf16x8*>(lds + am0 * (K * 2) + 16 * aswz(c, am0));
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, af, acc, 0, 0, 0);
    if (s + D < STEPS) wv[s % D] = __builtin_nontemporal_load(wsrc + (s + D) * 64 + lane);
  }

  __syncthreads();  // every wave is done with the A half; its LDS now holds the tiles
  f32x4* red = reinterpret_cast<f32x4*>(lds);
#pragma unroll
  for (int a = 0; a < 4; ++a)
    red[(wave * 4 + a) * 64 + lane] = f32x4{acc[4 * a], acc[4 * a + 1], acc[4 * a + 2], acc[4 * a + 3]};
  __syncthreads();
  if (wave >= kItems) return;
  const int a = wave & 3, pi = wave >> 2;
  // lane (m = lane % 32, g = lane / 32) sums C rows 32 mh + m, columns 32 j + 8a + 4g + (0..3) of
  // column block pi (and, for SwiGLU, of its partner NB / 2 + pi)
  constexpr int kSets = kPairs ? 2 : 1;
  f32x4 sv[kSets];
#pragma unroll
  for (int n = 0; n < kSets; ++n) {
    const int bn = pi + n * kHalf;
    sv[n] = red[(bn * 4 + a) * 64 + lane];
#pragma unroll
    for (int q = 1; q < KW; ++q) {
      const f32x4 v = red[((q * NB + bn) * 4 + a) * 64 + lane];
      sv[n][0] += v[0]; sv[n][1] += v[1]; sv[n][2] += v[2]; sv[n][3] += v[3];
    }
  }
  const int m = 32 * mh + am0;
  const int col = kNBlk * (tile * kHalf + pi) + 8 * a + 4 * (lane >> 5);
  if constexpr (EPI == kEpiPartial) {
    __builtin_nontemporal_store(sv[0], reinterpret_cast<f32x4*>(part + ((long long)split * kGemmM + m) * N + col));
    return;
  }
  float r[4];
  uint16_t* dst;
  if constexpr (EPI == kEpiSwiGlu) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float gv = bf16_to_f32(f32_to_bf16(sv[0][e] / (1.0f + __expf(-sv[0][e]))));
      const float uv = bf16_to_f32(f32_to_bf16(sv[1][e]));
      r[e] = gv * uv;
    }
    dst = out + (long long)m * N + col;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = sv[0][e];
    const int head = col >> 7, d = col & 127;
    uint16_t* base = head < kHq ? out : head < kHq + kHkv ? out_k : out_v;
    const int hh = head < kHq ? head : head < kHq + kHkv ? head - kHq : head - kHq - kHkv;
    dst = base + ((long long)hh * kGemmM + m) * 128 + d;
  }
  *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]));
}

// Sum of the splits of C[64, N], rounded to bf16. A workgroup covers one row and 256 columns:
// thread (g, q) sums splits g, g + 4, ... of columns 4q .. 4q + 3 (eight loads in flight), and
// group 0 adds the four group sums in group order, so the result does not depend on timing.
constexpr int kRedGroups = 4, kRedBatch = 8;

__global__ __launch_bounds__(256) void k_gemm_reduce(const float* part, int n_split, int N, uint16_t* out) {
  __shared__ f32x4 red[kRedGroups - 1][64];
  const int g = threadIdx.x >> 6;
  const int q = threadIdx.x & 63;
  const int m = blockIdx.x % kGemmM;
  const int n = (blockIdx.x / kGemmM) * 256 + 4 * q;
  const long long stride = (long long)kGemmM * N / 4;  // float4s per split
  const bool live = n < N;  // the last block of a width that is not a multiple of 256
  const f32x4* p = reinterpret_cast<const f32x4*>(part + (long long)m * N + (live ? n : 0));
  const int ns = live ? n_split : 0;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = g; c0 < ns; c0 += kRedGroups * kRedBatch) {
    f32x4 v[kRedBatch];
#pragma unroll
    for (int b = 0; b < kRedBatch; ++b) {
      const int c = c0 + kRedGroups * b;
      v[b] = c < ns ? p[c * stride] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int b = 0; b < kRedBatch; ++b) {
      s[0] += v[b][0]; s[1] += v[b][1]; s[2] += v[b][2]; s[3] += v[b][3];
    }
  }
  if (g > 0) red[g - 1][q] = s;
  __syncthreads();
  if (g > 0 || !live) return;
#pragma unroll
  for (int k = 0; k < kRedGroups - 1; ++k) {
    const f32x4 v = red[k][q];
    s[0] += v[0]; s[1] += v[1]; s[2] += v[2]; s[3] += v[3];
  }
  *reinterpret_cast<uint2*>(out + (long long)m * N + n) = make_uint2(pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3]));
}

// Residual RMSNorm: out[m] = bf16(gamma * x[m] / sqrt(mean(x[m]^2) + eps)), one workgroup per row,
// 8 columns per thread (width = 8 x blockDim).
__global__ __launch_bounds__(256) void k_rmsnorm_rows(const uint16_t* x, const uint16_t* gamma, float eps, int width,
                                                      uint16_t* out) {
  __shared__ float part[8];
  const int m = blockIdx.x;
  const int t = threadIdx.x;
  const bool live = 8 * t < width;
  float v[8], g[8];
  if (live) {
    unpack8v(*reinterpret_cast<const u32x4*>(x + (long long)m * width + 8 * t), v);
    unpack8v(*reinterpret_cast<const u32x4*>(gamma + 8 * t), g);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = g[e] = 0.f;
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if ((t & 63) == 0) part[t >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) tot += part[w];
  const float inv = 1.0f / sqrtf(tot / (float)width + eps);
  if (!live) return;
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = v[e] * inv * g[e];
  *reinterpret_cast<u32x4*>(out + (long long)m * width + 8 * t) = pack8v(o);
}

// A split sum, the residual add and the next norm in one pass, one workgroup per row:
// y[m] = bf16(x[m] + bf16(sum of the splits of C[m])) and, if gamma is not null, n[m] =
// bf16(gamma * y[m] / sqrt(mean(y[m]^2) + eps)), the same arithmetic and summation order as
// k_rmsnorm_rows on y. Used for the o projection (y = x2, n = n2) and the down projection (y =
// x_out, and for a chained layer n = the next layer's first norm). 8 columns per thread, width = 8
// x blockDim; the splits are added in order 0, 1, ..., all loads of a thread issued before any is
// added.
template <int NSPLIT>
__global__ __launch_bounds__(256) void k_reduce_residual_norm(const float* part, const uint16_t* x,
                                                              const uint16_t* gamma, float eps, int width,
                                                              uint16_t* y, uint16_t* n) {
  __shared__ float red[8];
  const int m = blockIdx.x;
  const int t = threadIdx.x;
  const long long row = (long long)m * width + 8 * t;
  const f32x4* p = reinterpret_cast<const f32x4*>(part + row);
  const long long stride = (long long)kGemmM * width / 4;
  f32x4 v[NSPLIT][2];
#pragma unroll
  for (int c = 0; c < NSPLIT; ++c) {
    v[c][0] = p[c * stride];
    v[c][1] = p[c * stride + 1];
  }
  float xr[8], o[8];
  unpack8v(*reinterpret_cast<const u32x4*>(x + row), xr);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float sum = v[0][e >> 2][e & 3];
#pragma unroll
    for (int c = 1; c < NSPLIT; ++c) sum += v[c][e >> 2][e & 3];
    o[e] = bf16_to_f32(f32_to_bf16(xr[e] + bf16_to_f32(f32_to_bf16(sum))));  // y, as stored
    ss += o[e] * o[e];
  }
  *reinterpret_cast<u32x4*>(y + row) = pack8v(o);
  if (gamma == nullptr) return;
  float g[8];
  unpack8v(*reinterpret_cast<const u32x4*>(gamma + 8 * t), g);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if ((t & 63) == 0) red[t >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) tot += red[w];
  const float inv = 1.0f / sqrtf(tot / (float)width + eps);
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = o[e] * inv * g[e];
  *reinterpret_cast<u32x4*>(n + row) = pack8v(o);
}

// ---- host side -----------------------------------------------------------------------------------

// Projection shapes. A configuration is (NB column blocks, KW waves along k, STEPS 16-row steps per
// wave); a split then covers KC = 16 KW STEPS rows and the grid is (N / (32 NB)) x (K / KC).
struct GemmCfg {
  int nb, kw, steps, depth = 0;  // depth: weight loads in flight per wave (k_gemm32; 0 = all)
};
// the layer's four projections, each the fastest of a sweep over configurations on the cold-weight
// workload: qkv 64 x 4 = 256 workgroups of 2 waves, o 48 x 4 = 192 of 4, gate/up 96 x 2 = 192 of 8,
// down 24 x 8 = 192 of 4
constexpr GemmCfg kCfgDown{2, 2, 24};
constexpr int kDownSplits = kLayerMlp / (16 * kCfgDown.kw * kCfgDown.steps);
// the o projection in the 32-row form with 2 splits of K (2 x 48 x 2 = 192 workgroups of 8 waves)
constexpr GemmCfg kCfgO32{1, 8, 8, 8};
constexpr int kOSplits = kHq * 128 / (16 * kCfgO32.kw * kCfgO32.steps);
// qkv and gate/up take the whole of K per 32-row half (k_gemm32): qkv 2 x 128 = 256 workgroups,
// gate/up 2 x 192 = 384
constexpr GemmCfg kCfgQkv32{1, 8, 12, 12}, kCfgGateUp32{4, 2, 48, 16};
static_assert(16 * kCfgQkv32.kw * kCfgQkv32.steps == kLayerHidden, "qkv takes the whole of K");
static_assert(16 * kCfgGateUp32.kw * kCfgGateUp32.steps == kLayerHidden, "gate/up take the whole of K");
static_assert((kLayerQkv / kNBlk / kCfgQkv32.nb) % 8 == 0 && (kLayerMlp / kNBlk / (kCfgGateUp32.nb / 2)) % 8 == 0,
              "tiles in groups of 8");
// any other shape: 4 waves along k over one column block, the most rows per wave that still gives
// 256 workgroups (else the fewest)
static GemmCfg gemm_cfg_generic(int K, int N) {
  for (int st : {12, 8, 6, 4, 2}) {
    const int kc = 64 * st;
    if (K % kc == 0 && K / kc <= kMaxSplit && (N / kNBlk) * (K / kc) >= 256) return {1, 4, st};
  }
  return (K % 128 == 0 && K / 128 <= kMaxSplit) ? GemmCfg{1, 4, 2} : GemmCfg{0, 0, 0};
}
static int gemm_splits(const GemmCfg& c, int K) { return K / (16 * c.kw * c.steps); }

bool gemm64_shape_ok(int K, int N) {
  return K > 0 && N > 0 && N % 64 == 0 && K % 128 == 0 && gemm_cfg_generic(K, N).nb > 0;
}

size_t gemm64_partials_bytes(int K, int N) {
  const GemmCfg c = gemm_cfg_generic(K, N);
  if (c.nb == 0) return 0;
  return (size_t)gemm_splits(c, K) * kGemmM * N * 4;
}

template <int NB, int KW, int STEPS>
static void launch_gemm_cfg(const uint16_t* A, const uint16_t* W, int K, int N, float* part, hipStream_t st) {
  const int tiles = (N / kNBlk) / NB;
  const int splits = K / (16 * KW * STEPS);
  hipLaunchKernelGGL((k_gemm64<NB, KW, STEPS>), dim3(tiles * splits), dim3(64 * NB * KW), 0, st, A, W, K, N, part);
}

static hipError_t launch_gemm_generic(const uint16_t* A, const uint16_t* W, int K, int N, float* part,
                                      hipStream_t st, int* n_split) {
  const GemmCfg c = gemm_cfg_generic(K, N);
  *n_split = gemm_splits(c, K);
  switch (c.steps) {
    case 12: launch_gemm_cfg<1, 4, 12>(A, W, K, N, part, st); break;
    case 8: launch_gemm_cfg<1, 4, 8>(A, W, K, N, part, st); break;
    case 6: launch_gemm_cfg<1, 4, 6>(A, W, K, N, part, st); break;
    case 4: launch_gemm_cfg<1, 4, 4>(A, W, K, N, part, st); break;
    case 2: launch_gemm_cfg<1, 4, 2>(A, W, K, N, part, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

static hipError_t launch_reduce(const float* part, int n_split, int N, uint16_t* out, hipStream_t st) {
  hipLaunchKernelGGL(k_gemm_reduce, dim3(kGemmM * ((N + 255) / 256)), dim3(256), 0, st, part, n_split, N, out);
  return hipGetLastError();
}

hipError_t launch_pack_w64(const uint16_t* W, int K, int N, uint16_t* Wp, hipStream_t st) {
  const long long chunks = (long long)K * N / 8;
  hipLaunchKernelGGL(k_pack_w64, dim3((unsigned)(chunks / 256)), dim3(256), 0, st, W, K, N, Wp);
  return hipGetLastError();
}

hipError_t launch_linear64(const uint16_t* A, const uint16_t* W, int K, int N, uint16_t* C, void* ws,
                           hipStream_t st) {
  int ns = 0;
  hipError_t e = launch_gemm_generic(A, W, K, N, static_cast<float*>(ws), st, &ns);
  if (e != hipSuccess) return e;
  return launch_reduce(static_cast<float*>(ws), ns, N, C, st);
}

// Layer workspace: activations, then the attention workspace, then the GEMM partials (the
// largest: x w1 and x w3 together).
struct LayerWs {
  uint16_t *n1, *q, *k, *v, *attn, *x2, *n2, *mlp;
  void* attn_ws;
  float* part;
};
static size_t al256(size_t x) { return (x + 255) & ~size_t(255); }
static size_t layer_ws_layout(const AttnPlan& plan, void* ws, LayerWs* l) {
  size_t off = 0;
  char* w = static_cast<char*>(ws);
  auto take = [&](size_t bytes) {
    char* p = w ? w + off : nullptr;
    off += al256(bytes);
    return p;
  };
  // the attention step's workspace first: its status word is the layer workspace's
  void* attn_ws = take(attn_partials_bytes(plan));
  const size_t act = (size_t)kGemmM * kLayerHidden * 2;
  uint16_t* n1 = reinterpret_cast<uint16_t*>(take(act));
  uint16_t* q = reinterpret_cast<uint16_t*>(take((size_t)kHq * kGemmM * 128 * 2));
  uint16_t* k = reinterpret_cast<uint16_t*>(take((size_t)kHkv * kGemmM * 128 * 2));
  uint16_t* v = reinterpret_cast<uint16_t*>(take((size_t)kHkv * kGemmM * 128 * 2));
  uint16_t* attn = reinterpret_cast<uint16_t*>(take((size_t)kHq * kGemmM * 128 * 2));
  uint16_t* x2 = reinterpret_cast<uint16_t*>(take(act));
  uint16_t* n2 = reinterpret_cast<uint16_t*>(take(act));
  uint16_t* mlp = reinterpret_cast<uint16_t*>(take((size_t)kGemmM * kLayerMlp * 2));
  // float32 partials of the larger split projection (qkv and gate/up leave none)
  size_t pmax = 0;
  for (size_t b : {(size_t)kOSplits * kGemmM * kLayerHidden * 4, (size_t)kDownSplits * kGemmM * kLayerHidden * 4})
    pmax = b > pmax ? b : pmax;
  float* part = reinterpret_cast<float*>(take(pmax));
  if (l) *l = LayerWs{n1, q, k, v, attn, x2, n2, mlp, attn_ws, part};
  return off;
}

size_t layer_workspace_bytes(int S, int Smax) { return layer_ws_layout(attn_plan(S, Smax), nullptr, nullptr); }

hipError_t launch_layer(const LayerLaunch& p, hipStream_t st) {
  const AttnPlan plan = attn_plan(p.S, p.Smax);
  LayerWs l;
  layer_ws_layout(plan, p.ws, &l);
  hipError_t e;
#define AX_TRY(x)                \
  do {                           \
    e = (x);                     \
    if (e != hipSuccess) return e; \
  } while (0)
  // the first norm, unless the previous layer's last launch made it (a chained layer)
  const uint16_t* n1 = p.n1_in;
  if (n1 == nullptr) {
    hipLaunchKernelGGL(k_rmsnorm_rows, dim3(kGemmM), dim3(kLayerHidden / 8), 0, st, p.x, p.ln1, p.eps, kLayerHidden,
                       l.n1);
    AX_TRY(hipGetLastError());
    n1 = l.n1;
  }
  hipLaunchKernelGGL((k_gemm32<kCfgQkv32.nb, kCfgQkv32.kw, kCfgQkv32.steps, kEpiQkvSplit, false, kCfgQkv32.depth>),
                     dim3(2 * kLayerQkv / kNBlk / kCfgQkv32.nb), dim3(64 * kCfgQkv32.nb * kCfgQkv32.kw), 0, st, n1,
                     p.wqkv, nullptr, kLayerQkv, l.q, l.k, l.v, kLayerHidden, nullptr);
  AX_TRY(hipGetLastError());
  AttnLaunch a{l.q, p.qn, p.kn, p.cos_t, p.sin_t, p.eps, l.k, l.v, p.Kc, p.Vc, l.attn, l.attn_ws, p.S, p.Smax,
               /*q_norm=*/1};
  AX_TRY(launch_attn(plan, a, st));
  hipLaunchKernelGGL((k_gemm32<kCfgO32.nb, kCfgO32.kw, kCfgO32.steps, kEpiPartial, true, kCfgO32.depth>),
                     dim3(2 * kLayerHidden / kNBlk / kCfgO32.nb * kOSplits), dim3(64 * kCfgO32.nb * kCfgO32.kw), 0, st,
                     l.attn, p.wo, nullptr, kLayerHidden, nullptr, nullptr, nullptr, kHq * 128, l.part);
  AX_TRY(hipGetLastError());
  hipLaunchKernelGGL(k_reduce_residual_norm<kOSplits>, dim3(kGemmM), dim3(kLayerHidden / 8), 0, st, l.part, p.x,
                     p.ln2, p.eps, kLayerHidden, l.x2, l.n2);
  AX_TRY(hipGetLastError());
  hipLaunchKernelGGL((k_gemm32<kCfgGateUp32.nb, kCfgGateUp32.kw, kCfgGateUp32.steps, kEpiSwiGlu, false,
                               kCfgGateUp32.depth>),
                     dim3(2 * kLayerMlp / kNBlk / (kCfgGateUp32.nb / 2)), dim3(64 * kCfgGateUp32.nb * kCfgGateUp32.kw), 0,
                     st, l.n2, p.w1, p.w3, kLayerMlp, l.mlp, nullptr, nullptr, kLayerHidden, nullptr);
  AX_TRY(hipGetLastError());
  launch_gemm_cfg<kCfgDown.nb, kCfgDown.kw, kCfgDown.steps>(l.mlp, p.w2, kLayerMlp, kLayerHidden, l.part, st);
  AX_TRY(hipGetLastError());
  // the split sum + residual, and for a chained layer the next layer's first norm
  hipLaunchKernelGGL(k_reduce_residual_norm<kDownSplits>, dim3(kGemmM), dim3(kLayerHidden / 8), 0, st, l.part, l.x2,
                     p.ln1_next, p.eps, kLayerHidden, p.x_out, p.n1_out);
  AX_TRY(hipGetLastError());
#undef AX_TRY
  return hipSuccess;
}

}  // namespace ax
