// Split-KV attention of the 128 folded query rows of each kv head over the visible
// cache rows, and the log-sum-exp combine of the splits.
//
// What is computed: page code/alpamayo_tt/expert.py, TTExpert.attention_core in
// decode mode - per kv head g ("user" g) the 2 q heads x 64 tokens form 128 query
// rows that attend, non-causally and with scale 1/sqrt(128), to cache rows [0, S)
// and [Smax-64, Smax); the additive mask of TTExpert.build_mask hides the rest.
// The pages' kernel splits each head's key sequence over cores and reduces the
// parts (EXPERT_NOTES.md, "masking approach"); the per-split quantities and the
// combine are the usual flash-decode ones:
//   m_c = max_j s_j, l_c = sum_j 2^(s_j - m_c), O_c = sum_j 2^(s_j - m_c) v_j
//   out = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c,  M = max_c m_c
// with s_j = log2(e) * (q . k_j) / sqrt(128) (base-2 exponentials of scaled
// scores, which equal the natural-base softmax).
//
// gfx950 mapping
// - One workgroup (4 waves) per (kv head, key split); workgroup id w -> head w % 8,
//   so all splits of one head are dispatched to the same XCD and share its L2.
// - Keys are processed in blocks of 32. All global loads of a split (K and V,
//   16 bytes per lane, 4 per thread per block) are issued before any compute, so
//   each CU keeps its whole share of the cache in flight; each block lands in its
//   own LDS tile (K row-major, V transposed), no buffer is reused.
// - Wave w owns query rows 32w..32w+31. S^T = K Q^T on v_mfma_f32_32x32x16_bf16:
//   A = K rows (M = keys), B = Q^T (N = query rows) from registers. Each lane then
//   holds one query row's scores, so the softmax statistics need one cross-half
//   exchange. O^T = V^T P^T reuses the S^T accumulator as the B operand directly.
// - Inside a block, MFMA row m reads key pi(m) (bits 2 and 3 of m swapped). With
//   that order the 8 keys a lane contributes to one PV step are consecutive, so the
//   V^T operand is a single 16-byte LDS read.
#include "ax_dev.h"
#include "ax_launch.h"

namespace ax {

constexpr int kBlk = 32;                  // keys per block
constexpr int kMaxNB = 8;                 // blocks per split, upper bound
constexpr int kKRow = kD + 8;             // LDS K row: 272 bytes (rows shift by 4 banks)
constexpr int kVRow = kBlk + 8;           // LDS V^T row (one head-dim column): 80 bytes
constexpr int kKTile = kBlk * kKRow;      // elements
constexpr int kTile = kKTile + kD * kVRow;
constexpr int kTileBytes = kTile * 2;     // 18944
constexpr float kLog2e = 1.4426950408889634f;

struct AttnArgs {
  const uint16_t* q;  // [8][128][128]
  const uint16_t* Kc;
  const uint16_t* Vc;
  float* po;          // [8][n_split][128 d][128 q]
  float* pm;          // [8][n_split][128]
  float* pl;          // [8][n_split][128]
  int S, Smax, n_split, kps;
};

// Visible key index (0 .. S+63) -> cache row.
__device__ __forceinline__ int key_row(int vk, int S, int Smax) { return vk < S ? vk : vk + (Smax - kT - S); }

// Row order inside a 32-key block seen by the MFMA: swap bits 2 and 3.
__device__ __forceinline__ int perm_key(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// Head-dim chunk (8 columns) used by k-step kk in lane half h: half h holds columns
// [32h, 32h+32) and [64+32h, 96+32h).
__device__ __forceinline__ int dcol(int kk, int h) { return (kk < 4) ? 32 * h + 8 * kk : 64 + 32 * h + 8 * (kk - 4); }

// Transposed V tile: row d (one head-dim column) holds the block's 32 keys as 4 groups
// of 8 (16 bytes each); group G of row d is stored at slot G ^ ((d >> 4) & 3), which
// spreads the packed key-pair writes over the banks and keeps every 16-byte read of a
// 16-lane group on distinct banks. Returns the element offset of group G of row d.
__device__ __forceinline__ int vt_off(int d, int G) { return d * kVRow + 8 * (G ^ ((d >> 4) & 3)); }

template <int NB>
__global__ __launch_bounds__(256, 1) void k_attn_split(AttnArgs a) {
  extern __shared__ __align__(16) uint16_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int h = lane >> 5;
  const int g = blockIdx.x % kHkv;
  const int split = blockIdx.x / kHkv;
  const int n_keys = a.S + kT;
  const int k_begin = split * a.kps;
  const int k_end = min(k_begin + a.kps, n_keys);

  const long long head_off = (long long)g * a.Smax * kD;
  const uint16_t* Kg = a.Kc + head_off;
  const uint16_t* Vg = a.Vc + head_off;

  // query fragments (B operand of S^T = K Q^T): row 32*wave + n, columns dcol(kk, h)
  const int qrow = 32 * wave + n;
  const uint16_t* qp = a.q + ((long long)g * kQRows + qrow) * kD;
  bf16x8 qf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qp + dcol(kk, h));

  // Loader roles (every thread, no branches, so all loads issue before any wait):
  //   K: rows (tid >> 4) and (tid >> 4) + 16 of the block, 16-byte chunk tid & 15;
  //   V: rows 2p and 2p+1, p = tid >> 4, chunk tid & 15 (stored transposed, key pairs packed).
  const int lc = tid & 15;
  const int lr = tid >> 4;
  u32x4 st[NB][4];
  static_for<NB>([&](auto bc) {
    constexpr int b = decltype(bc)::value;
    const int kb = k_begin + b * kBlk;
    static_for<4>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int rloc = (i < 2) ? lr + 16 * i : 2 * lr + (i - 2);
      const int vk = kb + rloc;
      const int row = key_row(vk < k_end ? vk : k_begin, a.S, a.Smax);
      const uint16_t* base = (i < 2) ? Kg : Vg;
      st[b][i] = *reinterpret_cast<const u32x4*>(base + (long long)row * kD + 8 * lc);
    });
  });
  // Keep every load above this point: the whole split is in flight before the first wait.
  __builtin_amdgcn_sched_barrier(0);

  f32x16 o[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sscale = kLog2e * 0.08838834764831845f;  // log2(e) / sqrt(128)
  const int krow = perm_key(n);

  // Blocks past the split end (only in a short last split) are fully masked: they add
  // nothing, and block 0 always holds at least one key, so m_run is finite from then on.
  static_for<NB>([&](auto bc) {
    constexpr int b = decltype(bc)::value;
    const int kb = k_begin + b * kBlk;
    uint16_t* tK = lds + b * kTile;
    uint16_t* tV = tK + kKTile;
    const u32x4 z = {0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(tK + lr * kKRow + 8 * lc) = (kb + lr < k_end) ? st[b][0] : z;
    *reinterpret_cast<u32x4*>(tK + (lr + 16) * kKRow + 8 * lc) = (kb + lr + 16 < k_end) ? st[b][1] : z;
    {
      const int r0 = 2 * lr;
      const uint32_t m0 = (kb + r0 < k_end) ? 0x0000ffffu : 0u;
      const uint32_t m1 = (kb + r0 + 1 < k_end) ? 0xffff0000u : 0u;
      const u32x4 w0 = st[b][2], w1 = st[b][3];
      static_for<8>([&](auto ec) {
        constexpr int e = decltype(ec)::value;
        const uint32_t lo = (e & 1) ? (w0[e >> 1] >> 16) : (w0[e >> 1] & 0xffffu);
        const uint32_t hi = (e & 1) ? (w1[e >> 1] & 0xffff0000u) : (w1[e >> 1] << 16);
        const int d = 8 * lc + e;
        *reinterpret_cast<uint32_t*>(tV + vt_off(d, lr >> 2) + 2 * (lr & 3)) = (lo & m0) | (hi & m1);
      });
    }
    __syncthreads();

    // All LDS fragments of the block first (K for S^T, V^T for the PV step), then the MFMAs.
    bf16x8 kf[8], vf[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) kf[kk] = *reinterpret_cast<const bf16x8*>(tK + krow * kKRow + dcol(kk, h));
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        vf[4 * c + t] = *reinterpret_cast<const bf16x8*>(tV + vt_off(32 * t + n, 2 * c + h));
    __builtin_amdgcn_sched_barrier(0);
    // S^T = K Q^T for this block
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[kk], s, 0, 0, 0);
    // scale, mask the keys past the split end, online softmax
    float bmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = perm_key(8 * (i >> 2) + 4 * h + (i & 3));
      s[i] = (kb + key < k_end) ? s[i] * sscale : -INFINITY;
      bmax = fmaxf(bmax, s[i]);
    }
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
    const float m_new = fmaxf(m_run, bmax);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[i] = exp2f(s[i] - m_new);
      psum += s[i];
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
    bf16x8 pb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) pb[c][j] = (__bf16)s[8 * c + j];
    // O^T += V^T P^T
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int t = 0; t < 4; ++t) o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[4 * c + t], pb[c], o[t], 0, 0, 0);
  });

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const long long part = (long long)g * a.n_split + split;
  float* po = a.po + part * (kD * kQRows);
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int d = 32 * t + 8 * (i >> 2) + 4 * h + (i & 3);
      po[d * kQRows + qrow] = o[t][i];
    }
  if (h == 0) {
    a.pm[part * kQRows + qrow] = m_run;
    a.pl[part * kQRows + qrow] = l_tot;
  }
}

// Combine: block -> (head g, 32 query rows, 16 head-dim columns); thread -> (query row, 2 columns).
__global__ __launch_bounds__(256) void k_attn_combine(const float* po, const float* pm, const float* pl,
                                                      uint16_t* out, int n_split) {
  const int g = blockIdx.x % kHkv;
  const int qb = (blockIdx.x / kHkv) & 3;
  const int db = blockIdx.x / (kHkv * 4);
  const int q = 32 * qb + (threadIdx.x & 31);
  const int d = 16 * db + 2 * (threadIdx.x >> 5);
  float M = -INFINITY, L = 0.f, acc0 = 0.f, acc1 = 0.f;
  for (int c = 0; c < n_split; ++c) {
    const long long part = (long long)g * n_split + c;
    const float mc = pm[part * kQRows + q];
    const float lc = pl[part * kQRows + q];
    const float* oc = po + part * (kD * kQRows);
    const float o0 = oc[d * kQRows + q], o1 = oc[(d + 1) * kQRows + q];
    if (mc > M) {
      const float r = exp2f(M - mc);
      acc0 *= r; acc1 *= r; L *= r;
      M = mc;
    }
    const float w = exp2f(mc - M);
    acc0 += w * o0;
    acc1 += w * o1;
    L += w * lc;
  }
  const float inv = 1.0f / L;
  *reinterpret_cast<uint32_t*>(out + ((long long)g * kQRows + q) * kD + d) = pack_bf16x2(acc0 * inv, acc1 * inv);
}

AttnPlan attn_plan(int S, int /*Smax*/) {
  AttnPlan p;
  p.n_keys = S + kT;
  const int target = 32;  // splits per head: 8 heads x 32 = 256 workgroups, one per CU
  int kps = (p.n_keys + target - 1) / target;
  if (kps < kBlk) kps = kBlk;
  if (kps > kBlk * kMaxNB) kps = kBlk * kMaxNB;
  p.keys_per_split = kps;
  p.n_split = (p.n_keys + kps - 1) / kps;
  p.blocks = (kps + kBlk - 1) / kBlk;
  return p;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t attn_partials_bytes(const AttnPlan& p) {
  const size_t parts = (size_t)kHkv * p.n_split;
  return align256(parts * kD * kQRows * 4) + 2 * align256(parts * kQRows * 4);
}

template <int NB>
static hipError_t launch_nb(const AttnArgs& a, hipStream_t st) {
  static bool attr_set[64] = {};
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (dev >= 0 && dev < 64 && !attr_set[dev]) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_split<NB>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, NB * kTileBytes);
    if (e != hipSuccess) return e;
    attr_set[dev] = true;
  }
  hipLaunchKernelGGL(k_attn_split<NB>, dim3(kHkv * a.n_split), dim3(256), NB * kTileBytes, st, a);
  return hipGetLastError();
}

hipError_t launch_attn(const AttnPlan& plan, const AttnLaunch& p, hipStream_t st) {
  AttnArgs a;
  const size_t parts = (size_t)kHkv * plan.n_split;
  char* ws = static_cast<char*>(p.ws);
  a.q = p.q; a.Kc = p.Kc; a.Vc = p.Vc;
  a.po = reinterpret_cast<float*>(ws);
  a.pm = reinterpret_cast<float*>(ws + align256(parts * kD * kQRows * 4));
  a.pl = reinterpret_cast<float*>(ws + align256(parts * kD * kQRows * 4) + align256(parts * kQRows * 4));
  a.S = p.S; a.Smax = p.Smax; a.n_split = plan.n_split; a.kps = plan.keys_per_split;
  hipError_t e;
  switch (plan.blocks) {
    case 1: e = launch_nb<1>(a, st); break;
    case 2: e = launch_nb<2>(a, st); break;
    case 3: e = launch_nb<3>(a, st); break;
    case 4: e = launch_nb<4>(a, st); break;
    case 5: e = launch_nb<5>(a, st); break;
    case 6: e = launch_nb<6>(a, st); break;
    case 7: e = launch_nb<7>(a, st); break;
    default: e = launch_nb<8>(a, st); break;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_attn_combine, dim3(kHkv * 4 * 8), dim3(256), 0, st, a.po, a.pm, a.pl, p.out,
                     plan.n_split);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_copy_words(const uint4* src, uint4* dst, size_t n) {
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n; i += (size_t)gridDim.x * 256ull) dst[i] = src[i];
}

hipError_t launch_copy_words(const void* src, void* dst, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_copy_words, dim3((unsigned)blocks), dim3(256), 0, st, static_cast<const uint4*>(src),
                     static_cast<uint4*>(dst), n);
  return hipGetLastError();
}

}  // namespace ax
