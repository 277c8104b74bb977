// Split-KV attention of the 128 folded query rows of each kv head over the visible
// cache rows (with the q/k RMSNorm + RoPE and the own-K/V tail write folded in), and
// the log-sum-exp combine of the splits.
//
// What is computed: page code/alpamayo_tt/expert.py, TTExpert.layer from the q/k
// norms to attention_core in decode mode - per kv head g ("user" g) the 2 q heads x
// 64 tokens form 128 query rows that attend, non-causally and with scale
// 1/sqrt(128), to cache rows [0, S) and [Smax-64, Smax); the additive mask of
// TTExpert.build_mask hides the rest. The pages' kernel splits each head's key
// sequence over cores and reduces the parts (EXPERT_NOTES.md, "masking approach");
// the per-split quantities and the combine are the flash-decode ones:
//   m_c = max_j s_j, l_c = sum_j 2^(s_j - m_c), O_c = sum_j 2^(s_j - m_c) v_j
//   out = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c,  M = max_c m_c
// with s_j = log2(e) * (q . k_j) / sqrt(128) (base-2 exponentials of scaled scores
// give the same softmax).
//
// gfx950 mapping
// - One workgroup of 8 waves (one compute and one loader wave per SIMD) per (kv head, key
//   split); workgroup id w -> head w % 8, which the dispatcher places on XCD w % 8, so a
//   head's splits share one L2. The cache keys [0, S) are cut into splits of at most 6
//   blocks of 32 keys; the 64 own tokens form one more split of their own.
// - Waves 4..7 (loaders) stream the split's K/V rows into per-block LDS tiles with
//   direct-to-LDS loads (global_load_lds, 16 bytes per lane), a few blocks ahead, and
//   count each landed block in LDS; rows are 256 bytes with the 16-byte chunks
//   XOR-swizzled by row.
// - Waves 0..3 (compute) fetch and norm/rope the 128 query rows in place in LDS (16
//   lanes per row, the same arithmetic as the stand-alone norm/RoPE kernel); in the own
//   split they also norm/rope the own k rows and write the cache tail. Then wave w takes
//   query rows 32w .. +31 over every block of the split: S^T = K Q^T on
//   v_mfma_f32_32x32x16_bf16 (A = K rows, B = Q^T), so each lane holds one query row's
//   scores; O^T = V^T P^T with V^T read straight from row-major V by ds_read_tr16_b64
//   and P^T taken from the S^T accumulator. Inside a block MFMA row m reads key pi(m)
//   (bits 2 and 3 swapped), which makes the 8 keys a lane supplies to one PV step
//   consecutive. The loop is software-pipelined one block deep (scores of block b+1
//   with the softmax of block b, and the PV of block b with the row max of block b+1),
//   and each wave stores its own rows' partial.
#include "ax_attn_common.h"
#include "ax_launch.h"

namespace ax {

constexpr int kMaxNB = 6;                     // blocks per split, upper bound (LDS: 6 x 16 KB + 48 KB)
static_assert(kMaxNB <= kMaxBlocks, "counter layout");
constexpr int kTileBytes = 2 * kBlk * kD * 2; // K 8 KB + V 8 KB
constexpr int kDmaDepth = 3;                  // blocks of a split in flight per loader wave
// Wave roles of the split kernel: one compute wave and one loader wave per SIMD, so that a
// compute wave has 256 registers for its software pipeline.
constexpr int kFCompute = 4;
constexpr int kFLoad = 4;
constexpr int kFThreads = 64 * (kFCompute + kFLoad);

struct FusedArgs {
  const uint16_t* q;       // [16][64][128]: raw q (q_norm) or already roped q
  const uint16_t* gq;
  const uint16_t* gk;
  const float* cos_t;      // [64][64]
  const float* sin_t;
  float eps;
  // Source of the own-token rows of head g: kt_base + g * tail_stride (row-major, 128 per row):
  // the own k/v tensors (raw k if normed here) or, when own_tail is 0, the cache tail itself.
  const uint16_t* kt_base;
  const uint16_t* vt_base;
  long long tail_stride;
  int own_tail;            // own rows come from k/v tensors: norm (if NORM) and write them to the cache tail
  uint16_t* Kc;
  uint16_t* Vc;
  float* po;               // [8][n_split][4 query groups][16 slots][64 lanes]: 4 float16 of O each
  float* pm;               // [8][n_split][128]
  float* pl;
  int S, Smax, n_split, kps;
  int n_cache_split;       // splits over cache keys [0, S); split n_cache_split holds the 64 own tokens
  int q_norm;
};

// The LDS tiles are distinct objects so that the compiler's wait counting can tell the
// direct-to-LDS loads of one block from another block and from the query buffer.
#define AX_TILE(b) __shared__ __attribute__((aligned(16))) uint8_t t##b[kTileBytes]
template <int B>
__device__ __forceinline__ uint8_t* pick(uint8_t* t0, uint8_t* t1, uint8_t* t2, uint8_t* t3, uint8_t* t4,
                                         uint8_t* t5) {
  if constexpr (B == 0) return t0;
  else if constexpr (B == 1) return t1;
  else if constexpr (B == 2) return t2;
  else if constexpr (B == 3) return t3;
  else if constexpr (B == 4) return t4;
  else return t5;
}

// RMSNorm + RoPE in place in LDS of the 8 query rows 32p + 16s + r16 (p = 0..3, s = 0..1)
// that this lane's 16-lane group holds, in the pair layout (columns 4 j16 .. +3 and
// 64 + 4 j16 .. +3); row 32p + 16s + r16 is token 32(p & 1) + 16s + r16, whose RoPE
// coefficients are A/B[2(p & 1) + s]. All rows are read before any is written back. Per row
// the arithmetic is that of the stand-alone kernel.
__device__ __forceinline__ void norm_rope_query_rows8(uint8_t* qlds, const float (&A)[4][8], const float (&B)[4][8],
                                                      int j16, int r16, float eps) {
  uint2 lo[8], hi[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 32 * (i >> 1) + 16 * (i & 1) + r16;
    lo[i] = *reinterpret_cast<const uint2*>(qlds + r * 256 + pair_off_lo(j16, qswz(r)));
    hi[i] = *reinterpret_cast<const uint2*>(qlds + r * 256 + pair_off_hi(j16, qswz(r)));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = 2 * ((i >> 1) & 1) + (i & 1);
    float x[8];
    unpack_pair(lo[i], hi[i], x);
    norm_rope_pair(x, A[t], B[t], eps);
    pack_pair(x, lo[i], hi[i]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 32 * (i >> 1) + 16 * (i & 1) + r16;
    *reinterpret_cast<uint2*>(qlds + r * 256 + pair_off_lo(j16, qswz(r))) = lo[i];
    *reinterpret_cast<uint2*>(qlds + r * 256 + pair_off_hi(j16, qswz(r))) = hi[i];
  }
}

// NORM: q and the own k arrive raw and are normed + roped here (the layer step); otherwise
// both arrive roped (attention only).
//
// Wave roles (8 waves, 2 per SIMD).
// - Waves 4..7 (loaders) only issue direct-to-LDS loads of the split's cache blocks and count
//   each landed block in LDS. Keeping ordinary loads and LDS-DMA loads in different waves
//   keeps each wave's vmcnt in order, so no wave ever has to drain its queue early; the
//   counters (not barriers) let the loads run ahead of the arithmetic.
// - Waves 0..3 (compute) fetch, norm and rope the 128 query rows in place in LDS and handle
//   the own-token rows; then wave w takes query rows 32w .. +31 over every block of the
//   split, software-pipelined: the QK^T of block b+1 runs on the matrix cores while the
//   exponentials of block b run on the vector ALU, and the PV of block b while the max of
//   block b+1. Each wave stores its rows' partial itself.
template <int NB, bool NORM>
__global__ __launch_bounds__(kFThreads, 1) void k_attn_fused(FusedArgs a) {
  AX_TILE(0); AX_TILE(1); AX_TILE(2); AX_TILE(3); AX_TILE(4); AX_TILE(5);
  __shared__ __attribute__((aligned(16))) uint8_t qlds[kQBytes];
  // roped own-token K rows (row tok, chunks swizzled like the tile row they stand in for)
  __shared__ __attribute__((aligned(16))) uint8_t kown[kT * 256];
  // hand-off counters
  __shared__ int cnt[kNCnt];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = blockIdx.x % kHkv;
  const int split = blockIdx.x / kHkv;
  const int n_keys = a.S + kT;
  // Cache splits cover [0, S) in kps-key ranges; the last split holds just the 64 own-token
  // keys, so that its extra work (own k norm, tail write) falls on a short split.
  const bool own_split = split >= a.n_cache_split;
  const int k_begin = own_split ? a.S : split * a.kps;
  const int k_end = own_split ? n_keys : min(k_begin + a.kps, a.S);
  const long long head_off = (long long)g * a.Smax * kD;
  // own rows come from the k/v tensors (normed here if NORM) and go to the cache tail
  const bool own_tail = a.own_tail != 0;

  if (tid < kNCnt) cnt[tid] = 0;
  // Compute-wave lanes: lane group r16 (0..15) norms query rows 32p + 16s + r16 (token
  // 32(p & 1) + 16s + r16) and own-token rows 16u + r16 (u = 0..3): tokens 16u + r16 in both.
  const int j16 = tid & 15;
  const int r16 = tid >> 4;
  const bool has_own = own_tail && own_split;  // this split holds the own-token rows
  uint2 graw[2], gkraw[2], kraw[4][2];  // pair layout: columns 4 j16 .. +3, 64 + 4 j16 .. +3
  u32x4 vraw[4];                        // 16-byte piece j16 (columns 8 j16 .. +7)
  f32x4 cs_h[4][2];                     // cos, sin of frequencies 4 j16 .. +3
  if (wave < kFCompute) {
    // 1. Prologue loads, all issued before the start barrier and so ahead of the cache stream
    //    in the CU's memory queue: the 32 query rows this wave norms (rows 32p + 16s + 4 wave
    //    .. +3; lane l lands at 16 l of the 1 KB, so it fetches the chunk that the row's
    //    swizzle puts there), the gammas, the RoPE table rows and the own-token rows.
    const uint16_t* qh = a.q + (long long)(2 * g) * kT * kD;  // q heads 2g, 2g+1: 128 rows, contiguous
    static_for<8>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int row0 = 32 * (i >> 1) + 16 * (i & 1) + 4 * wave;
      const int row = row0 + (lane >> 4);
      const uint16_t* src = qh + row * kD + 8 * ((lane & 15) ^ qswz(row));
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(qlds + row0 * 256), 16, 0, 0);
    });
    if constexpr (NORM) {
      graw[0] = *reinterpret_cast<const uint2*>(a.gq + 4 * j16);
      graw[1] = *reinterpret_cast<const uint2*>(a.gq + 64 + 4 * j16);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int tok = 16 * u + r16;
        cs_h[u][0] = *reinterpret_cast<const f32x4*>(a.cos_t + tok * 64 + 4 * j16);
        cs_h[u][1] = *reinterpret_cast<const f32x4*>(a.sin_t + tok * 64 + 4 * j16);
      }
    }
    if (has_own) {
      const uint16_t* kt = a.kt_base + g * a.tail_stride;
      const uint16_t* vt = a.vt_base + g * a.tail_stride;
      if constexpr (NORM) {
        gkraw[0] = *reinterpret_cast<const uint2*>(a.gk + 4 * j16);
        gkraw[1] = *reinterpret_cast<const uint2*>(a.gk + 64 + 4 * j16);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint16_t* krow_p = kt + (long long)(16 * u + r16) * kD;
        kraw[u][0] = *reinterpret_cast<const uint2*>(krow_p + 4 * j16);
        kraw[u][1] = *reinterpret_cast<const uint2*>(krow_p + 64 + 4 * j16);
        vraw[u] = *reinterpret_cast<const u32x4*>(vt + (long long)(16 * u + r16) * kD + 8 * j16);
      }
    }
  }
  lds_barrier();  // start: counters cleared (the only workgroup barrier)

  if (wave >= kFCompute) {
    // ---------------- loader waves: of each block the K row groups w and w+4 and the V row
    // groups w and w+4 (4 rows each)
    const int w = wave - kFCompute;
    const uint16_t* kc = a.Kc + head_off;
    const uint16_t* vc = a.Vc + head_off;
    const uint16_t* kt = a.kt_base + g * a.tail_stride;
    const uint16_t* vt = a.vt_base + g * a.tail_stride;
    // DMA of block b: this wave's K row groups w, w+4 and V row groups w, w+4.
    auto issue_block = [&](auto bc) {
      constexpr int b = decltype(bc)::value;
      uint8_t* tile = pick<b>(t0, t1, t2, t3, t4, t5);
      static_for<2>([&](auto hc) {
        constexpr int half = decltype(hc)::value;
        const int grp = w + 4 * half;
        const int rloc = 4 * grp + (lane >> 4);
        int vk = k_begin + b * kBlk + rloc;
        vk = vk < k_end ? vk : k_begin;  // rows past the split end reload a visible row; they are masked
        const bool in_cache = vk < a.S;
        const long long row = in_cache ? vk : vk - a.S;
        const uint16_t* ks = (in_cache ? kc : kt) + row * kD + 8 * ((lane & 15) ^ kswz(rloc));
        const uint16_t* vs = (in_cache ? vc : vt) + row * kD + 8 * ((lane & 15) ^ vswz(rloc));
        // (own-token K rows land here too but are read from kown instead)
        // Ordinary cache policy: with non-temporal loads the launch alone was 1.5-3% faster but
        // the step (with the combine after it) 1.6-3.6% slower, on two boxes.
        __builtin_amdgcn_global_load_lds(ks, (lds_void*)(tile + grp * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vs, (lds_void*)(tile + kTileBytes / 2 + grp * 1024), 16, 0, 0);
      });
    };
    // The CU's memory queue throttles issue, so only kDmaDepth blocks are kept in flight:
    // block b + kDmaDepth is issued right after block b has landed, and no count waits for
    // the issue of loads that are not needed yet.
    constexpr int D = NB < kDmaDepth ? NB : kDmaDepth;
    static_for<D>([&](auto bc) { issue_block(bc); });
    static_for<NB>([&](auto bc) {
      constexpr int b = decltype(bc)::value;
      constexpr int later = (b + D - 1 < NB - 1 ? b + D - 1 : NB - 1) - b;
      wait_vmcnt<4 * later>();  // loads are issued in block order: block b has landed
      arrive(&cnt[kCntBlock + b], lane);
      if constexpr (b + D < NB) issue_block(std::integral_constant<int, b + D>{});
    });
    return;
  }

  // ---------------- compute waves (256 threads)
  // 2. the query rows, normed and roped in place in LDS (unless they came roped)
  wait_vmcnt<0>();  // this wave's query rows and every prologue load have landed
  float qc[4][4], qs[4][4];
  if constexpr (NORM) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qc[u][e] = cs_h[u][0][e];
        qs[u][e] = cs_h[u][1][e];
      }
    float qg[8], A[4][8], B[4][8];
    unpack_pair(graw[0], graw[1], qg);
#pragma unroll
    for (int u = 0; u < 4; ++u) rope_coef_pair(qg, qc[u], qs[u], A[u], B[u]);
    norm_rope_query_rows8(qlds, A, B, j16, r16, a.eps);
  }
  // 3. own-token rows (own split only): K normed + roped (or taken roped) into kown and the
  //    cache tail, V copied to the cache tail (the stores come after every load has been
  //    waited for, so no later wait includes them)
  if (has_own) {
    float gk[8];
    if constexpr (NORM) unpack_pair(gkraw[0], gkraw[1], gk);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int tok = 16 * u + r16;
      uint2 klo = kraw[u][0], khi = kraw[u][1];
      if constexpr (NORM) {
        float x[8], A[8], B[8];
        unpack_pair(klo, khi, x);
        rope_coef_pair(gk, qc[u], qs[u], A, B);
        norm_rope_pair(x, A, B, a.eps);
        pack_pair(x, klo, khi);
      }
      uint8_t* kr = kown + tok * 256;  // swizzled like tile row tok % 32
      *reinterpret_cast<uint2*>(kr + pair_off_lo(j16, kswz(tok & (kBlk - 1)))) = klo;
      *reinterpret_cast<uint2*>(kr + pair_off_hi(j16, kswz(tok & (kBlk - 1)))) = khi;
      const long long dst = head_off + (long long)(a.Smax - kT + tok) * kD;
      *reinterpret_cast<uint2*>(a.Kc + dst + 4 * j16) = klo;
      *reinterpret_cast<uint2*>(a.Kc + dst + 64 + 4 * j16) = khi;
      *reinterpret_cast<u32x4*>(a.Vc + dst + 8 * j16) = vraw[u];
    }
  }
  arrive(&cnt[kCntQNormed], lane);
  await(&cnt[kCntQNormed], kFCompute);  // all 128 query rows and the own-token K rows are in LDS

  const int n = lane & 31;
  const int h = lane >> 5;
  const int qrow = 32 * wave + n;
  bf16x8 qf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    qf[kk] = *reinterpret_cast<const bf16x8*>(qlds + qrow * 256 + 16 * ((dcol(kk, h) >> 3) ^ qswz(qrow)));

  f32x16 o[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
  float l_run = 0.f;  // row sum (this lane's half of the keys)
  const float sc = kLog2e * 0.08838834764831845f;  // log2(e) / sqrt(128)
  const int krow = perm_key(n);
  // Per-lane LDS offsets, fixed for the loop: a block only adds its tile's (constant) base.
  // K fragment kk is chunk dcol(kk, h) / 8 = 4h + (kk & 3) + 8 (kk >> 2) of row krow; the
  // swizzle leaves the + 8, so koff[kk & 3] + 128 (kk >> 2).
  int koff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) koff[j] = krow * 256 + 16 * ((4 * h + j) ^ kswz(krow));
  // V^T operands: lane group G = lane >> 4, li = lane & 15 reads row 16c + 8(G>>1) + 4 hf +
  // li/4 at chunk 4t + 2(G&1) + ((li&3)>>1) (columns 32t + 16(G&1) + 4(li&3) .. +3); the
  // swizzle depends only on row & 3 = (li/4) & 3, so t = 0, 1 have their own offsets and
  // t = 2, 3 add 8 chunks. The transpose read hands lane li of the group column
  // 32t + 16(G&1) + li of 4 consecutive rows.
  const int G = lane >> 4, li = lane & 15;
  const int vrow0 = 8 * (G >> 1) + (li >> 2);
  const int vx = 2 * (G & 1) + ((li & 3) >> 1);
  const int voff[2] = {vrow0 * 256 + 16 * (vx ^ vswz(vrow0)) + 8 * (li & 1),
                       vrow0 * 256 + 16 * ((4 + vx) ^ vswz(vrow0)) + 8 * (li & 1)};

  // Blocks 0 .. nb-1 hold visible keys (only the last can be partial). K of an own-token block
  // (own split with own_tail) is read from kown, swizzled like the tile. The pipeline reads K
  // and forms scores ahead of the softmax; past nb it reads a tile without waiting for it
  // (LDS, in bounds), and nothing computed from such a tile is used: its max takes no part in
  // the rescale test and the loop ends before its exponentials.
  const int nb = (k_end - k_begin + kBlk - 1) / kBlk;
  const bool k_from_own = has_own;
  auto kbase = [&](auto bc) -> const uint8_t* {
    constexpr int b = decltype(bc)::value;
    if constexpr (b * kBlk < kT)
      if (k_from_own) return kown + b * kBlk * 256;
    return pick<b>(t0, t1, t2, t3, t4, t5);
  };
  auto read_k = [&](const uint8_t* base, bf16x8 (&kf)[8]) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) kf[kk] = *reinterpret_cast<const bf16x8*>(base + koff[kk & 3] + 128 * (kk >> 2));
  };
  auto qk = [&](const bf16x8 (&kf)[8]) {
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[kk], s, 0, 0, 0);
    return s;
  };
  // Row max of a block's scores over both lane halves, in log2 units. Rows past the split end
  // hold a copy of the split's first key (see the loaders), a visible key, so the max of a
  // partial block needs no mask.
  auto blk_max = [&](const f32x16& s) {
    float m0 = fmaxf(fmaxf(s[0], s[1]), s[2]);
    float m1 = fmaxf(fmaxf(s[3], s[4]), s[5]);
    float m2 = fmaxf(fmaxf(s[6], s[7]), s[8]);
    float m3 = fmaxf(fmaxf(s[9], s[10]), s[11]);
    float m4 = fmaxf(fmaxf(s[12], s[13]), s[14]);
    const float m = fmaxf(fmaxf(fmaxf(m0, m1), fmaxf(m2, m3)), fmaxf(m4, s[15]));
    const float2 pr = pair32(m);
    return fmaxf(pr.x, pr.y) * sc;
  };

  bf16x8 kf[8];
  // block 0: scores, max; the exponent reference m_run starts at its max (finite: block 0 holds
  // a visible key)
  await(&cnt[kCntBlock + 0], kFLoad);
  read_k(kbase(std::integral_constant<int, 0>{}), kf);
  f32x16 s_cur = qk(kf);
  float m_run = blk_max(s_cur);
  if constexpr (NB > 1) {
    if (nb > 1) {
      await(&cnt[kCntBlock + 1], kFLoad);
      read_k(kbase(std::integral_constant<int, 1>{}), kf);
    }
  }
  const bf16x2_t one2 = {(__bf16)1.0f, (__bf16)1.0f};

  static_for<NB>([&](auto bc) {
    constexpr int b = decltype(bc)::value;
    if (b >= nb) return;
    if constexpr (b + 2 < NB) {
      if (b + 2 < nb) await(&cnt[kCntBlock + b + 2], kFLoad);  // its K is read below
    }
    const int kb = k_begin + b * kBlk;
    if (b == nb - 1 && kb + kBlk > k_end) {
      // the last visible block is partial: keys past the split end get p = 0. Accumulator
      // element i of lane half h is key perm_key(8(i>>2) + 4h + (i&3)) = 8h + kofs(i).
      const int lim = k_end - kb - 8 * h;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kofs = 16 * (i >> 3) + 4 * ((i >> 2) & 1) + (i & 3);
        s_cur[i] = (kofs < lim) ? s_cur[i] : -INFINITY;
      }
    }
    const uint8_t* tv = pick<b>(t0, t1, t2, t3, t4, t5) + kTileBytes / 2;
    // (A) Step by step: the V^T fragment of one PV step of block b, one score MFMA of block
    //     b+1 and two of block b's p = 2^(s sc - m_run) (v_exp_f32 directly: the
    //     arguments are <= kRescale or -inf) with their bf16 pair and its share of l, which
    //     the vector ALU works through while the matrix core computes. The exponent
    //     reference m_run only moves when some row's max exceeds it by more than kRescale
    //     (log2 units): p stays below 2^kRescale, exact for the final normalisation, and the
    //     O rescale (64 multiplies) runs only on such jumps.
    //     l sums the same bf16-rounded p that the PV product uses (v_dot2_f32_bf16 against
    //     (1, 1)), so the output is an exact convex combination of V rows; with the fp32 p a
    //     row dominated by one key would be off by that p's rounding (up to 2^-9 of its V
    //     row), since p of a block after the first may exceed 1.
    //     The scheduling barriers keep this order: left alone, the compiler issues the score
    //     chain back to back with nothing to overlap it.
    v4i16 vt[2][4][2];
    f32x16 s_next;
#pragma unroll
    for (int i = 0; i < 16; ++i) s_next[i] = 0.f;
    bf16x8 pb[2];
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      {
        const int c = i >> 2, t = i & 3;  // the V^T fragment of PV step i, read a step at a time
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
          vt[c][t][hf] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16*)(tv + (16 * c + 4 * hf) * 256 + 128 * (t >> 1) + voff[t & 1]));
      }
      if constexpr (b + 1 < NB) s_next = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[i], s_next, 0, 0, 0);
      const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[2 * i], sc, -m_run));
      const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[2 * i + 1], sc, -m_run));
      const bf16x2_t pr = {(__bf16)e0, (__bf16)e1};
      pb[i >> 2][2 * (i & 3)] = pr[0];
      pb[i >> 2][2 * (i & 3) + 1] = pr[1];
      ps[i & 3] = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, ps[i & 3], false);
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    // (B) Step by step: one K fragment of block b+2 (past the last visible block, of a tile
    //     nobody waits for: its scores are never used), one PV MFMA of block b (O^T += V^T P^T,
    //     two halves of 16 keys, independent accumulators) and a share of block b+1's row
    //     max. Spreading the LDS reads over the steps keeps the wave from stalling on
    //     a full LDS queue with nothing else issued.
    float mx[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (b + 2 < NB) {
        const uint8_t* kbn = kbase(std::integral_constant<int, b + 2>{});
        kf[i] = *reinterpret_cast<const bf16x8*>(kbn + koff[i & 3] + 128 * (i >> 2));
      }
      const int c = i >> 2, t = i & 3;
      const v4i16 both[2] = {vt[c][t][0], vt[c][t][1]};
      bf16x8 vf;
      __builtin_memcpy(&vf, both, 16);
      o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[c], o[t], 0, 0, 0);
      if constexpr (b + 1 < NB) {
        if (i < 4) mx[i] = fmaxf(s_next[2 * i], s_next[2 * i + 1]);
        else mx[i & 3] = fmaxf(fmaxf(mx[i & 3], s_next[2 * i]), s_next[2 * i + 1]);
        asm volatile("" : "+v"(mx[i & 3]));  // computed here, not sunk to its use after the loop
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (b + 1 < NB) {
      if (b + 1 < nb) {
        const float2 pr = pair32(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3])));
        const float m_blk = fmaxf(pr.x, pr.y) * sc;
        if (__any(m_blk > m_run + kRescale)) {
          const float m_new = fmaxf(m_run, m_blk);
          const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
        }
      }
      s_cur = s_next;
    }
  });

  // The wave's partial: O (unnormalised), m and l of query rows 32w .. +31.
  const long long part = (long long)g * a.n_split + split;
  merge_and_store_partial(o, m_run, l_run, false, 0, wave, lane, nullptr, nullptr, [] {}, nullptr, cnt, a.po,
                          a.pm, a.pl, part);
}

// Combine: out = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c, M = max_c m_c.
// Workgroup (head g, rows 8r .. 8r+7, column half hc): 512 threads in 4 split groups of 128
// (8 rows x 16 column quads); group k reduces splits k, k + 4, ..., issuing the loads of up to
// kCombBatch splits before using any of them, so the whole partial set is in flight at once.
// The 8 rows of a (slot, half) of the accumulator layout are one 128-byte line. The groups meet
// in LDS.
constexpr int kCombGroups = 4;
constexpr int kCombBatch = 8;
__global__ __launch_bounds__(512) void k_attn_combine(const float* po, const float* pm, const float* pl,
                                                      uint16_t* out, int n_split) {
  __shared__ float sM[kCombGroups][8], sL[kCombGroups][8];
  __shared__ f32x4 sA[kCombGroups][128];
  const int g = blockIdx.x % kHkv;
  const int rest = blockIdx.x / kHkv;   // 0..31
  const int rblk = rest >> 1;           // rows 8 rblk .. +7
  const int hc = rest & 1;              // column quads 16 hc .. +15
  const int grp = threadIdx.x >> 7;
  const int t = threadIdx.x & 127;
  const int rloc = t >> 4;
  const int quad = 16 * hc + (t & 15);
  const int q = 8 * rblk + rloc;
  const int d0 = 4 * quad;              // = 32 tt + 8 jj + 4 h
  const int tt = d0 >> 5, jj = (d0 >> 3) & 3, h = (d0 >> 2) & 1;
  const int slot = 4 * tt + jj, lane = (q & 31) + 32 * h;
  const float* pmg = pm + (long long)g * n_split * kQRows + q;
  const float* plg = pl + (long long)g * n_split * kQRows + q;
  const u32x2* pog = reinterpret_cast<const u32x2*>(po) + ((long long)g * n_split * 4 + (q >> 5)) * (16 * 64) +
                     slot * 64 + lane;
  const long long pstride = 4 * 16 * 64;  // 4-float16 groups per split partial
  float M = -INFINITY, L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = grp; c0 < n_split; c0 += kCombGroups * kCombBatch) {
    float mv[kCombBatch], lv[kCombBatch];
    f32x4 ov[kCombBatch];
#pragma unroll
    for (int k = 0; k < kCombBatch; ++k) {
      const int c = min(c0 + kCombGroups * k, n_split - 1);  // past the end: a repeat, weighted 0 below
      mv[k] = pmg[(long long)c * kQRows];
      lv[k] = plg[(long long)c * kQRows];
      ov[k] = unpack_f16x4(pog[(long long)c * pstride]);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load of the batch is issued before any is used
    float Mb = M;
#pragma unroll
    for (int k = 0; k < kCombBatch; ++k)
      if (c0 + kCombGroups * k < n_split) Mb = fmaxf(Mb, mv[k]);
    const float r = __builtin_amdgcn_exp2f(M - Mb);  // 0 while M is -inf
    L *= r;
    acc[0] *= r; acc[1] *= r; acc[2] *= r; acc[3] *= r;
    M = Mb;
#pragma unroll
    for (int k = 0; k < kCombBatch; ++k) {
      const float w = (c0 + kCombGroups * k < n_split) ? __builtin_amdgcn_exp2f(mv[k] - M) : 0.f;
      L += w * lv[k];
      acc[0] += w * ov[k][0]; acc[1] += w * ov[k][1]; acc[2] += w * ov[k][2]; acc[3] += w * ov[k][3];
    }
  }
  if ((t & 15) == 0) {
    sM[grp][rloc] = M;
    sL[grp][rloc] = L;
  }
  sA[grp][t] = acc;
  __syncthreads();
  if (grp != 0) return;
  float Mt = sM[0][rloc];  // group 0 holds split 0, so Mt is finite
#pragma unroll
  for (int k = 1; k < kCombGroups; ++k) Mt = fmaxf(Mt, sM[k][rloc]);
  float Lt = 0.f;
  f32x4 At = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < kCombGroups; ++k) {
    const float w = __builtin_amdgcn_exp2f(sM[k][rloc] - Mt);  // 0 for a group without splits
    Lt += w * sL[k][rloc];
    const f32x4 v = sA[k][t];
    At[0] += w * v[0]; At[1] += w * v[1]; At[2] += w * v[2]; At[3] += w * v[3];
  }
  const float inv = 1.0f / Lt;
  uint2 o2;
  o2.x = pack_bf16x2(At[0] * inv, At[1] * inv);
  o2.y = pack_bf16x2(At[2] * inv, At[3] * inv);
  *reinterpret_cast<uint2*>(out + ((long long)g * kQRows + q) * kD + d0) = o2;
}

AttnPlan attn_plan(int S, int /*Smax*/) {
  AttnPlan p;
  p.n_keys = S + kT;
  // 31 cache splits + the own-token split per head: 8 heads x 32 = 256 workgroups, one per CU
  const int target = 31;
  int kps = (S + target - 1) / target;
  if (kps < kBlk) kps = kBlk;
  if (kps > kBlk * kMaxNB) kps = kBlk * kMaxNB;
  p.keys_per_split = kps;
  p.n_cache_split = (S + kps - 1) / kps;
  p.n_split = p.n_cache_split + 1;
  p.blocks = (kps + kBlk - 1) / kBlk;
  if (p.blocks < kT / kBlk) p.blocks = kT / kBlk;
  return p;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t attn_partials_bytes(const AttnPlan& p) {
  const size_t parts = (size_t)kHkv * p.n_split;
  return align256(parts * kD * kQRows * 2) + 2 * align256(parts * kQRows * 4);
}

template <int NB>
static hipError_t launch_nb(const FusedArgs& a, hipStream_t st) {
  if (a.q_norm)
    hipLaunchKernelGGL((k_attn_fused<NB, true>), dim3(kHkv * a.n_split), dim3(kFThreads), 0, st, a);
  else
    hipLaunchKernelGGL((k_attn_fused<NB, false>), dim3(kHkv * a.n_split), dim3(kFThreads), 0, st, a);
  return hipGetLastError();
}

WsLayout ws_layout(const AttnPlan& plan, const void* ws) {
  const size_t parts = (size_t)kHkv * plan.n_split;
  char* w = static_cast<char*>(const_cast<void*>(ws));
  WsLayout l;
  l.po = reinterpret_cast<float*>(w);
  l.pm = reinterpret_cast<float*>(w + align256(parts * kD * kQRows * 2));
  l.pl = reinterpret_cast<float*>(w + align256(parts * kD * kQRows * 2) + align256(parts * kQRows * 4));
  return l;
}

hipError_t launch_attn_combine(const AttnPlan& plan, const void* ws, uint16_t* out, hipStream_t st) {
  const WsLayout l = ws_layout(plan, ws);
  hipLaunchKernelGGL(k_attn_combine, dim3(kHkv * 32), dim3(512), 0, st, l.po, l.pm, l.pl, out, plan.n_split);
  return hipGetLastError();
}

hipError_t launch_attn(const AttnPlan& plan, const AttnLaunch& p, hipStream_t st) {
  const hipError_t e = launch_attn_split(plan, p, st);
  if (e != hipSuccess) return e;
  return launch_attn_combine(plan, p.ws, p.out, st);
}

hipError_t launch_attn_split(const AttnPlan& plan, const AttnLaunch& p, hipStream_t st) {
  FusedArgs a;
  a.q = p.q; a.gq = p.gq; a.gk = p.gk; a.cos_t = p.cos_t; a.sin_t = p.sin_t; a.eps = p.eps;
  a.own_tail = p.k_tail != nullptr;
  if (a.own_tail) {
    a.kt_base = p.k_tail; a.vt_base = p.v_tail; a.tail_stride = (long long)kT * kD;
  } else {
    a.kt_base = p.Kc + (long long)(p.Smax - kT) * kD; a.vt_base = p.Vc + (long long)(p.Smax - kT) * kD;
    a.tail_stride = (long long)p.Smax * kD;
  }
  a.Kc = p.Kc; a.Vc = p.Vc;
  const WsLayout l = ws_layout(plan, p.ws);
  a.po = l.po; a.pm = l.pm; a.pl = l.pl;
  a.S = p.S; a.Smax = p.Smax; a.n_split = plan.n_split; a.kps = plan.keys_per_split;
  a.n_cache_split = plan.n_cache_split;
  a.q_norm = p.q_norm;
  hipError_t e;
  switch (plan.blocks) {
    case 1: e = launch_nb<1>(a, st); break;
    case 2: e = launch_nb<2>(a, st); break;
    case 3: e = launch_nb<3>(a, st); break;
    case 4: e = launch_nb<4>(a, st); break;
    case 5: e = launch_nb<5>(a, st); break;
    default: e = launch_nb<6>(a, st); break;
  }
  return e;
}

__global__ __launch_bounds__(256) void k_copy_words(const u32x4* src, u32x4* dst, size_t n) {
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n; i += (size_t)gridDim.x * 256ull) dst[i] = src[i];
}

hipError_t launch_copy_words(const void* src, void* dst, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_copy_words, dim3((unsigned)blocks), dim3(256), 0, st, static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), n);
  return hipGetLastError();
}

}  // namespace ax
