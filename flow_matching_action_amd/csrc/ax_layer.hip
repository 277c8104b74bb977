// The rest of one action-expert decoder layer around the attention step: the residual
// RMSNorms, the M = 64 projections (qkv, o, the SwiGLU MLP) and their epilogues.
//
// What is computed: page code/alpamayo_tt/EXPERT_NOTES.md, section "Layouts" (the per-layer op
// list and the weight shapes; weights stored input-major, [in, out]) and page
// code/alpamayo_tt/expert.py, TTExpert.layer. Every op hands a bf16 tensor to the next; inside an
// op the arithmetic is float32.
//
// gfx950 mapping
// - k_gemm64: C[64, N] = A[64, K] W[K, N] for the 64 token rows. The weights are the stream
//   (M = 64 is far below the ridge), so the grid is (N / 64 column tiles) x (K / KC splits) and
//   each workgroup moves one KC x 64 weight tile and the matching 64 x KC slice of A into LDS
//   with direct-to-LDS loads, then four waves each make one 32 x 32 tile of C^T = W^T A^T on
//   v_mfma_f32_32x32x16_bf16: W^T comes from the row-major weight tile through
//   ds_read_tr16_b64 (as V^T in the attention kernel), A^T straight from A's rows. The split's
//   float32 partial goes to the workspace.
// - k_gemm_reduce: sums the splits in a fixed order and applies the op's epilogue: the head
//   split of qkv into q/k/v [heads][64][128], the residual add (o + x, d + x2), or SiLU(g) * u.
// - k_rmsnorm_rows: one workgroup per token row.
#include "ax_attn_common.h"
#include "ax_launch.h"

namespace ax {

constexpr int kGemmM = 64;      // token rows
constexpr int kGemmNT = 64;     // output columns per workgroup
constexpr int kGemmThreads = 256;

// W tile rows are 128 bytes (64 columns): chunk c of row k holds columns 8c' .. 8c'+7 with
// c' = c ^ wswz(k); the transpose read of a 16-lane group takes rows r .. r+3 at one chunk pair.
__device__ __forceinline__ int wswz(int k) { return 2 * (k & 3); }
// A tile rows are KC x 2 bytes: within each aligned group of 8 chunks, chunk c holds chunk
// c ^ (m & 7), so the 32 rows a k-step reads at one column spread over 8 bank groups.
__device__ __forceinline__ int aswz(int c, int m) { return (c & ~7) | ((c & 7) ^ (m & 7)); }

// A element (m, k): row-major [64][lda], or (heads = true) the attention output [16][64][128]
// read as its heads concatenated ([64][2048]: column 128 h + d of row m is head h, token m,
// element d).
__device__ __forceinline__ const uint16_t* a_elem(const uint16_t* A, int lda, int m, int k, bool heads) {
  return heads ? A + ((long long)(k >> 7) * kGemmM + m) * 128 + (k & 127) : A + (long long)m * lda + k;
}

template <int KC, bool HEADS>
__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm64(const uint16_t* A, int lda, const uint16_t* W, int N,
                                                          float* part) {
  static_assert(KC % 64 == 0 && KC <= 512, "k chunk");
  __shared__ __attribute__((aligned(16))) uint8_t wt[KC * kGemmNT * 2];
  __shared__ __attribute__((aligned(16))) uint8_t at[kGemmM * KC * 2];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n_tiles = N / kGemmNT;
  const int tile = blockIdx.x % n_tiles;
  const int split = blockIdx.x / n_tiles;
  const int n0 = tile * kGemmNT;
  const int k0 = split * KC;

  // weight tile: KC rows of 128 bytes, 8 rows per 1 KB load (lane l: row 8i + l / 8, chunk l % 8)
  constexpr int kWLoads = KC / 8;
  static_for<kWLoads / 4>([&](auto ic) {
    constexpr int i0 = decltype(ic)::value;
    const int i = 4 * i0 + wave;
    const int k = 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ wswz(k);
    __builtin_amdgcn_global_load_lds(W + (long long)(k0 + k) * N + n0 + 8 * c, (lds_void*)(wt + i * 1024), 16, 0,
                                     kNonTemporal);
  });
  // A slice: 64 rows of KC x 2 bytes (KC / 8 chunks per row), 1 KB per load
  constexpr int kCpr = KC / 8;
  constexpr int kALoads = kGemmM * kCpr / 64;
  static_for<kALoads / 4>([&](auto ic) {
    constexpr int i0 = decltype(ic)::value;
    const int i = 4 * i0 + wave;
    const int e = 64 * i + lane;      // chunk index in the tile
    const int m = e / kCpr;
    const int c = aswz(e % kCpr, m);  // the A chunk that lands at this position
    __builtin_amdgcn_global_load_lds(a_elem(A, lda, m, k0 + 8 * c, HEADS), (lds_void*)(at + i * 1024), 16, 0, 0);
  });
  wait_vmcnt<0>();
  lds_barrier();

  // wave w: C^T tile (n-sub t = w & 1: columns 32t .. 32t+31) x (m-sub = w >> 1: rows 32ms .. +31)
  const int t = wave & 1;
  const int ms = wave >> 1;
  const int G = lane >> 4, li = lane & 15;
  const int wrow0 = 8 * (G >> 1) + (li >> 2);                  // + 4 hf + 16 kstep
  const int wx = 4 * t + 2 * (G & 1) + ((li & 3) >> 1);        // chunk before the swizzle
  const int woff = wrow0 * 128 + 16 * (wx ^ wswz(wrow0)) + 8 * (li & 1);
  const int am = 32 * ms + (lane & 31);                         // A row of this lane's B operand
  const int ah = lane >> 5;
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll 4
  for (int ks = 0; ks < KC / 16; ++ks) {
    // A operand: W^T rows n = 32t + lane % 32, k = 16 ks + 8 (lane / 32) .. +7 (swizzle depends on k & 3 only)
    const v4i16 w0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(wt + (16 * ks) * 128 + woff));
    const v4i16 w1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(wt + (16 * ks + 4) * 128 + woff));
    const v4i16 both[2] = {w0, w1};
    bf16x8 wf;
    __builtin_memcpy(&wf, both, 16);
    // B operand: A^T, row am, k = 16 ks + 8 ah .. +7
    const int c = 2 * ks + ah;
    const bf16x8 af = *reinterpret_cast<const bf16x8*>(at + am * (KC * 2) + 16 * aswz(c, am));
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, af, acc, 0, 0, 0);
  }
  // lane (m = lane % 32, h) holds C rows 32 ms + m, columns 32t + 8a + 4h + (0..3), a = 0..3
  float* dst = part + ((long long)split * kGemmM + am) * N + n0 + 32 * t + 4 * ah;
#pragma unroll
  for (int a = 0; a < 4; ++a)
    __builtin_nontemporal_store(f32x4{acc[4 * a], acc[4 * a + 1], acc[4 * a + 2], acc[4 * a + 3]},
                                reinterpret_cast<f32x4*>(dst + 8 * a));
}

enum GemmEpilogue { kEpiStore = 0, kEpiQkvSplit = 1, kEpiResidual = 2, kEpiSwiGlu = 3 };

// Sum of the splits of C[64, N] in split order, then the epilogue; thread = 4 consecutive columns.
// kEpiStore: out[m][n] = bf16(C); kEpiQkvSplit: bf16(C) into q / k / v [heads][64][128] (columns
// 0..2047 q heads, 2048..3071 k heads, 3072..4095 v heads); kEpiResidual: out = bf16(res +
// bf16(C)); kEpiSwiGlu: C and C2 are x w1 and x w3, out = bf16(bf16(silu(C)) * bf16(C2)).
template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_reduce(const float* part, const float* part2, int n_split, int N,
                                                     const uint16_t* res, uint16_t* out, uint16_t* out_k,
                                                     uint16_t* out_v) {
  const int i = blockIdx.x * 256 + threadIdx.x;  // quad index
  if (i >= kGemmM * N / 4) return;
  const int m = (4 * i) / N;
  const int n = (4 * i) % N;
  const long long stride = (long long)kGemmM * N / 4;
  const f32x4* p = reinterpret_cast<const f32x4*>(part) + i;
  f32x4 s = p[0];
  for (int c = 1; c < n_split; ++c) {
    const f32x4 v = p[c * stride];
    s[0] += v[0]; s[1] += v[1]; s[2] += v[2]; s[3] += v[3];
  }
  float r[4];
  if constexpr (EPI == kEpiSwiGlu) {
    const f32x4* p2 = reinterpret_cast<const f32x4*>(part2) + i;
    f32x4 s2 = p2[0];
    for (int c = 1; c < n_split; ++c) {
      const f32x4 v = p2[c * stride];
      s2[0] += v[0]; s2[1] += v[1]; s2[2] += v[2]; s2[3] += v[3];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float g = bf16_to_f32(f32_to_bf16(s[e] / (1.0f + __expf(-s[e]))));
      const float u = bf16_to_f32(f32_to_bf16(s2[e]));
      r[e] = g * u;
    }
  } else if constexpr (EPI == kEpiResidual) {
    const uint2 rr = *reinterpret_cast<const uint2*>(res + (long long)m * N + n);
    const float x[4] = {bf16_to_f32(rr.x & 0xffffu), bf16_to_f32(rr.x >> 16), bf16_to_f32(rr.y & 0xffffu),
                        bf16_to_f32(rr.y >> 16)};
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = x[e] + bf16_to_f32(f32_to_bf16(s[e]));
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = s[e];
  }
  const uint2 o2 = make_uint2(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]));
  uint16_t* dst;
  if constexpr (EPI == kEpiQkvSplit) {
    const int head = n >> 7, d = n & 127;
    uint16_t* base = head < kHq ? out : head < kHq + kHkv ? out_k : out_v;
    const int hh = head < kHq ? head : head < kHq + kHkv ? head - kHq : head - kHq - kHkv;
    dst = base + ((long long)hh * kGemmM + m) * 128 + d;
  } else {
    dst = out + (long long)m * N + n;
  }
  *reinterpret_cast<uint2*>(dst) = o2;
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

// ---- host side -----------------------------------------------------------------------------------

// K chunk per workgroup: the largest of 512, 256, 128 that divides K and leaves at least 256
// workgroups, else the one with the most workgroups.
static int gemm_kc(int K, int N) {
  const int tiles = N / kGemmNT;
  int best = 0;
  for (int kc : {512, 256, 128})
    if (K % kc == 0 && tiles * (K / kc) >= 256) return kc;
  for (int kc : {128, 256, 512})
    if (K % kc == 0) { best = kc; break; }
  return best;
}

size_t gemm64_partials_bytes(int K, int N) {
  const int kc = gemm_kc(K, N);
  if (kc == 0) return 0;
  return (size_t)(K / kc) * kGemmM * N * 4;
}

bool gemm64_shape_ok(int K, int N) { return K > 0 && N > 0 && N % kGemmNT == 0 && K % 128 == 0; }

template <bool HEADS>
static hipError_t launch_gemm(const uint16_t* A, int lda, const uint16_t* W, int K, int N, float* part,
                              hipStream_t st, int* n_split) {
  const int kc = gemm_kc(K, N);
  *n_split = K / kc;
  const dim3 grid((N / kGemmNT) * (K / kc));
  if (kc == 512) hipLaunchKernelGGL((k_gemm64<512, HEADS>), grid, dim3(kGemmThreads), 0, st, A, lda, W, N, part);
  else if (kc == 256) hipLaunchKernelGGL((k_gemm64<256, HEADS>), grid, dim3(kGemmThreads), 0, st, A, lda, W, N, part);
  else hipLaunchKernelGGL((k_gemm64<128, HEADS>), grid, dim3(kGemmThreads), 0, st, A, lda, W, N, part);
  return hipGetLastError();
}

template <int EPI>
static hipError_t launch_reduce(const float* part, const float* part2, int n_split, int N, const uint16_t* res,
                                uint16_t* out, uint16_t* out_k, uint16_t* out_v, hipStream_t st) {
  const int quads = kGemmM * N / 4;
  hipLaunchKernelGGL((k_gemm_reduce<EPI>), dim3((quads + 255) / 256), dim3(256), 0, st, part, part2, n_split, N, res,
                     out, out_k, out_v);
  return hipGetLastError();
}

hipError_t launch_linear64(const uint16_t* A, const uint16_t* W, int K, int N, uint16_t* C, void* ws,
                           hipStream_t st) {
  int ns = 0;
  hipError_t e = launch_gemm<false>(A, K, W, K, N, static_cast<float*>(ws), st, &ns);
  if (e != hipSuccess) return e;
  return launch_reduce<kEpiStore>(static_cast<float*>(ws), nullptr, ns, N, nullptr, C, nullptr, nullptr, st);
}

// Layer workspace: activations, then the attention workspace, then the GEMM partials (the
// largest: x w1 and x w3 together).
struct LayerWs {
  uint16_t *n1, *q, *k, *v, *attn, *x2, *n2, *mlp;
  void* attn_ws;
  float *part, *part2;
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
  const size_t act = (size_t)kGemmM * kLayerHidden * 2;
  uint16_t* n1 = reinterpret_cast<uint16_t*>(take(act));
  uint16_t* q = reinterpret_cast<uint16_t*>(take((size_t)kHq * kGemmM * 128 * 2));
  uint16_t* k = reinterpret_cast<uint16_t*>(take((size_t)kHkv * kGemmM * 128 * 2));
  uint16_t* v = reinterpret_cast<uint16_t*>(take((size_t)kHkv * kGemmM * 128 * 2));
  uint16_t* attn = reinterpret_cast<uint16_t*>(take((size_t)kHq * kGemmM * 128 * 2));
  uint16_t* x2 = reinterpret_cast<uint16_t*>(take(act));
  uint16_t* n2 = reinterpret_cast<uint16_t*>(take(act));
  uint16_t* mlp = reinterpret_cast<uint16_t*>(take((size_t)kGemmM * kLayerMlp * 2));
  void* attn_ws = take(attn_partials_bytes(plan));
  const size_t p1 = gemm64_partials_bytes(kLayerHidden, kLayerMlp);
  size_t pmax = p1;
  for (size_t b : {gemm64_partials_bytes(kLayerHidden, kLayerQkv), gemm64_partials_bytes(kHq * 128, kLayerHidden),
                   gemm64_partials_bytes(kLayerMlp, kLayerHidden)})
    pmax = b > pmax ? b : pmax;
  float* part = reinterpret_cast<float*>(take(pmax));
  float* part2 = reinterpret_cast<float*>(take(p1));
  if (l) *l = LayerWs{n1, q, k, v, attn, x2, n2, mlp, attn_ws, part, part2};
  return off;
}

size_t layer_workspace_bytes(int S, int Smax) { return layer_ws_layout(attn_plan(S, Smax), nullptr, nullptr); }

hipError_t launch_layer(const LayerLaunch& p, hipStream_t st) {
  const AttnPlan plan = attn_plan(p.S, p.Smax);
  LayerWs l;
  layer_ws_layout(plan, p.ws, &l);
  hipError_t e;
  int ns = 0;
#define AX_TRY(x)                \
  do {                           \
    e = (x);                     \
    if (e != hipSuccess) return e; \
  } while (0)
  hipLaunchKernelGGL(k_rmsnorm_rows, dim3(kGemmM), dim3(kLayerHidden / 8), 0, st, p.x, p.ln1, p.eps, kLayerHidden,
                     l.n1);
  AX_TRY(hipGetLastError());
  AX_TRY(launch_gemm<false>(l.n1, kLayerHidden, p.wqkv, kLayerHidden, kLayerQkv, l.part, st, &ns));
  AX_TRY(launch_reduce<kEpiQkvSplit>(l.part, nullptr, ns, kLayerQkv, nullptr, l.q, l.k, l.v, st));
  AttnLaunch a{l.q, p.qn, p.kn, p.cos_t, p.sin_t, p.eps, l.k, l.v, p.Kc, p.Vc, l.attn, l.attn_ws, p.S, p.Smax,
               /*q_norm=*/1, /*tail_norm=*/1};
  AX_TRY(launch_attn(plan, a, st));
  AX_TRY(launch_gemm<true>(l.attn, 0, p.wo, kHq * 128, kLayerHidden, l.part, st, &ns));
  AX_TRY(launch_reduce<kEpiResidual>(l.part, nullptr, ns, kLayerHidden, p.x, l.x2, nullptr, nullptr, st));
  hipLaunchKernelGGL(k_rmsnorm_rows, dim3(kGemmM), dim3(kLayerHidden / 8), 0, st, l.x2, p.ln2, p.eps, kLayerHidden,
                     l.n2);
  AX_TRY(hipGetLastError());
  AX_TRY(launch_gemm<false>(l.n2, kLayerHidden, p.w1, kLayerHidden, kLayerMlp, l.part, st, &ns));
  AX_TRY(launch_gemm<false>(l.n2, kLayerHidden, p.w3, kLayerHidden, kLayerMlp, l.part2, st, &ns));
  AX_TRY(launch_reduce<kEpiSwiGlu>(l.part, l.part2, ns, kLayerMlp, nullptr, l.mlp, nullptr, nullptr, st));
  AX_TRY(launch_gemm<false>(l.mlp, kLayerMlp, p.w2, kLayerMlp, kLayerHidden, l.part, st, &ns));
  AX_TRY(launch_reduce<kEpiResidual>(l.part, nullptr, ns, kLayerHidden, l.x2, p.x_out, nullptr, nullptr, st));
#undef AX_TRY
  return hipSuccess;
}

}  // namespace ax
