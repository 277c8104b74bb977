// Split-KV attention over an fp8 KV cache: e4m3 codes with one float32 scale per (kv head,
// row), the same layer step as ax_attn.hip otherwise (q/k RMSNorm + RoPE, own rows into the
// cache tail, attention of the 128 folded query rows of each kv head over [0, S) and the
// tail, log-sum-exp combine).
//
// What is computed: page code/alpamayo_tt/expert.py, TTExpert.layer and attention_core, with
// the 8-bit cache the pages offer as an option (TTExpert.__init__, the kv_cache dtype map;
// page code/alpamayo_tt/EXPERT_NOTES.md, the bfp8-cache row of the decode attention timing).
// The cache value of row j is e4m3(code) * scale_j, so with the same s_j and flash-decode
// quantities as the bf16 kernel:
//   q . k_j = scale_j * (q . e4m3(code_j)),   sum_j p_j v_j = sum_j (p_j vscale_j) e4m3(vcode_j)
// The own rows the layer writes are quantised per row: scale = max |x| / 448, code = the
// nearest-even, saturating e4m3 rounding of x / scale (float32 divisions).
//
// gfx950 mapping (differences from the bf16 kernel)
// - Tiles hold 32 rows of 128 bytes for K and for V (8 KB per block), so a split holds up to
//   12 blocks; the loader waves also move the block's 64 scales into LDS (a 4-byte-per-lane
//   direct-to-LDS load).
// - K fragments are read as bytes and converted exactly to bf16 (v_cvt_scalef32_pk_bf16_fp8
//   with scale 1: every e4m3 value is a bf16 value) for the same bf16 MFMAs; the key scales
//   multiply the scores.
// - V^T operands come from ds_read_b64_tr_b8: in each 16-lane group, result lane j, byte k is
//   byte j & 7 of source lane 2k + (j >> 3), so source lanes that point at 8 rows (two 8-byte
//   halves each) hand every lane 8 consecutive keys of one column - the A operand of
//   v_mfma_f32_32x32x16_bf16 after conversion. The value scales are folded into P.
// - The own split's blocks are filled by the compute waves (quantised own rows), not by DMA.
#include "ax_attn_common.h"
#include "ax_launch.h"

namespace ax {

constexpr int kMaxNB8 = 12;               // blocks per split (LDS: 12 x 8 KB + 32 KB + scales)
static_assert(kMaxNB8 <= kMaxBlocks, "counter layout");
constexpr int kTile8 = 2 * kBlk * kD;     // K 4 KB + V 4 KB
constexpr int kVOff8 = kBlk * kD;         // V half of a tile
constexpr int kDmaDepth8 = 6;             // blocks in flight per loader wave (48 KB per CU)
constexpr float kE4m3Max = 448.0f;

struct F8Args {
  const uint16_t* q;       // [16][64][128]: raw q (NORM) or already roped q
  const uint16_t* gq;
  const uint16_t* gk;
  const float* cos_t;      // [64][64]
  const float* sin_t;
  float eps;
  const uint16_t* k_own;   // own k [8][64][128] (raw if NORM, else roped) or null: tail already in the cache
  const uint16_t* v_own;
  uint8_t* Kc;             // [8][Smax][128] e4m3
  float* Ks;               // [8][Smax]
  uint8_t* Vc;
  float* Vs;
  float* po;
  float* pm;
  float* pl;
  int* pe;
  int* status;             // workspace status word
  int spin_limit;          // polls before a wait gives up
  int S, Smax, n_split, kps, n_cache_split;
};

// V chunk swizzle of an fp8 row (8 chunks of 16 bytes): the transpose read of a 16-lane group
// takes 8 consecutive rows at one chunk, which row & 7 spreads over all 8 chunks.
__device__ __forceinline__ int vswz8(int r) { return r & 7; }

typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i32 lds_v2i32;

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

// Wave roles and hand-offs as in the bf16 kernel (8 compute waves, 4 loader waves, LDS
// counters, one start barrier). NORM: q and the own k arrive raw and are normed + roped here.
template <int NB, bool NORM>
__global__ __launch_bounds__(kThreads, 1) void k_attn_f8(F8Args a) {
  // at least 8 tiles, so that tiles 2q and 2q+1 can take the merge hand-off of query group q
  constexpr int NT = NB < 8 ? 8 : NB;
  __shared__ __attribute__((aligned(16))) uint8_t tiles[NT][kTile8];
  __shared__ __attribute__((aligned(16))) uint8_t qlds[kQBytes];
  // scales of block b: scl[b][w][0..7] = K scales of rows 8w .. 8w+7, scl[b][w][8..15] = V scales
  __shared__ __attribute__((aligned(16))) float scl[NB][4][16];
  __shared__ float mlx[4][2][32];
  __shared__ int cnt[kNCnt];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = blockIdx.x % kHkv;
  const int split = blockIdx.x / kHkv;
  const int n_keys = a.S + kT;
  const bool own_split = split >= a.n_cache_split;
  const int k_begin = own_split ? a.S : split * a.kps;
  const int k_end = own_split ? n_keys : min(k_begin + a.kps, a.S);
  const long long head_row = (long long)g * a.Smax;  // first cache row of head g
  const bool own_tail = a.k_own != nullptr;          // own rows quantised here into tiles and cache tail

  if (tid < kNCnt) cnt[tid] = 0;
  bool expired = false;  // a bounded wait of this wave ran out
  if (wave < kComputeWaves) {
    const uint16_t* qh = a.q + (long long)(2 * g) * kT * kD;
    static_for<4>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      const int row = 32 * p + 4 * wave + (lane >> 4);
      const uint16_t* src = qh + row * kD + 8 * ((lane & 15) ^ qswz(row));
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(qlds + (32 * p + 4 * wave) * 256), 16, 0, 0);
    });
  }
  lds_barrier();  // start: counters cleared (the only workgroup barrier)

  if (wave >= kComputeWaves) {
    // ---------------- loader waves: rows 8w .. 8w+7 of each block (K, V, and their scales)
    const int w = wave - kComputeWaves;
    if (own_split && own_tail) {
      // the compute waves fill the own split's tiles; nothing to load
      static_for<NB>([&](auto bc) { arrive(&cnt[kCntBlock + decltype(bc)::value], lane); });
      return;  // (no waits)
    }
    // cache row of visible key vk (own tokens from the cache tail); rows past the split end
    // reload a visible row, which the compute waves mask
    auto cache_row = [&](int vk) -> long long {
      vk = vk < k_end ? vk : k_begin;
      return head_row + (vk < a.S ? vk : a.Smax - kT + (vk - a.S));
    };
    auto issue_block = [&](auto bc) {
      constexpr int b = decltype(bc)::value;
      const int r = 8 * w + (lane >> 3);
      const long long cr = cache_row(k_begin + b * kBlk + r);
      const uint8_t* ks = a.Kc + cr * kD + 16 * ((lane & 7) ^ kswz(r));
      const uint8_t* vs = a.Vc + cr * kD + 16 * ((lane & 7) ^ vswz8(r));
      // ordinary cache policy, as in the bf16 kernel (non-temporal: launch alone 2% faster, the
      // step with the combine 2% slower)
      __builtin_amdgcn_global_load_lds(ks, (lds_void*)(&tiles[b][0] + w * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vs, (lds_void*)(&tiles[b][kVOff8] + w * 1024), 16, 0, 0);
      // lanes 0..7: K scales of rows 8w .. 8w+7, lanes 8..15: V scales (lane i lands at 4 i)
      if (lane < 16) {
        const long long sr = cache_row(k_begin + b * kBlk + 8 * w + (lane & 7));
        const float* src = (lane < 8 ? a.Ks : a.Vs) + sr;
        __builtin_amdgcn_global_load_lds(src, (lds_void*)&scl[b][w][0], 4, 0, 0);
      }
    };
    constexpr int D = NB < kDmaDepth8 ? NB : kDmaDepth8;
    static_for<D>([&](auto bc) { issue_block(bc); });
    static_for<NB>([&](auto bc) {
      constexpr int b = decltype(bc)::value;
      constexpr int later = (b + D - 1 < NB - 1 ? b + D - 1 : NB - 1) - b;
      wait_vmcnt<3 * later>();  // three loads per block, issued in block order: block b has landed
      arrive(&cnt[kCntBlock + b], lane);
      if constexpr (b + D < NB) issue_block(std::integral_constant<int, b + D>{});
    });
    return;  // (no waits)
  }

  // ---------------- compute waves (512 threads)
  const int j16 = tid & 15;
  const int r16 = tid >> 4;  // 0..31
  const bool has_own = own_tail && own_split;
  // Raw q / own k are held in the pair layout (columns 4 j16 .. +3 and 64 + 4 j16 .. +3) when
  // normed here, the v rows (and a k that arrives roped) as 16-byte pieces j16.
  uint2 graw[2], gkraw[2], kpair[2][2];
  u32x4 kraw[2], vraw[2];
  f32x4 cs_h[2][2];  // cos, sin of frequencies 4 j16 .. +3 of tokens r16 and 32 + r16
  if constexpr (NORM) {
    graw[0] = *reinterpret_cast<const uint2*>(a.gq + 4 * j16);
    graw[1] = *reinterpret_cast<const uint2*>(a.gq + 64 + 4 * j16);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int tok = 32 * p + r16;
      cs_h[p][0] = *reinterpret_cast<const f32x4*>(a.cos_t + tok * 64 + 4 * j16);
      cs_h[p][1] = *reinterpret_cast<const f32x4*>(a.sin_t + tok * 64 + 4 * j16);
    }
  }
  if (has_own) {
    if constexpr (NORM) {
      gkraw[0] = *reinterpret_cast<const uint2*>(a.gk + 4 * j16);
      gkraw[1] = *reinterpret_cast<const uint2*>(a.gk + 64 + 4 * j16);
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const long long tok_off = ((long long)g * kT + 32 * p + r16) * kD;
      if constexpr (NORM) {
        kpair[p][0] = *reinterpret_cast<const uint2*>(a.k_own + tok_off + 4 * j16);
        kpair[p][1] = *reinterpret_cast<const uint2*>(a.k_own + tok_off + 64 + 4 * j16);
      } else {
        kraw[p] = *reinterpret_cast<const u32x4*>(a.k_own + tok_off + 8 * j16);
      }
      vraw[p] = *reinterpret_cast<const u32x4*>(a.v_own + tok_off + 8 * j16);
    }
  }
  wait_vmcnt<0>();  // its query rows and every prologue load have landed
  if constexpr (NORM) norm_rope_query_rows(qlds, graw, cs_h, j16, r16, a.eps);
  // own tokens (the own split only): k normed + roped (or taken roped) and rounded to bf16, v
  // as given; each row quantised into the own blocks' tiles, the scales into LDS, both into
  // the cache tail. Token tok is key tok of the split: block tok / 32, row tok % 32.
  if (has_own) {
    float gk[8];
    if constexpr (NORM) unpack_pair(gkraw[0], gkraw[1], gk);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int tok = 32 * p + r16;
      const int r = tok & (kBlk - 1);
      const long long crow = head_row + a.Smax - kT + tok;
      uint8_t* tile = &tiles[p][0];
      float x[8], sk, sv;
      if constexpr (NORM) {
        // normed and roped in the pair layout, rounded to bf16 (the activation format),
        // quantised; the lane's codes are columns 4 j16 .. +3 and 64 + 4 j16 .. +3
        float A[8], B[8];
        const float c[4] = {cs_h[p][0][0], cs_h[p][0][1], cs_h[p][0][2], cs_h[p][0][3]};
        const float sn[4] = {cs_h[p][1][0], cs_h[p][1][1], cs_h[p][1][2], cs_h[p][1][3]};
        unpack_pair(kpair[p][0], kpair[p][1], x);
        rope_coef_pair(gk, c, sn, A, B);
        norm_rope_pair(x, A, B, a.eps);
        uint2 lo, hi;
        pack_pair(x, lo, hi);
        unpack_pair(lo, hi, x);
        const uint2 ck = quant_row16(x, sk);
        *reinterpret_cast<uint32_t*>(tile + r * kD + 16 * ((j16 >> 2) ^ kswz(r)) + 4 * (j16 & 3)) = ck.x;
        *reinterpret_cast<uint32_t*>(tile + r * kD + 16 * ((4 + (j16 >> 2)) ^ kswz(r)) + 4 * (j16 & 3)) = ck.y;
        *reinterpret_cast<uint32_t*>(a.Kc + crow * kD + 4 * j16) = ck.x;
        *reinterpret_cast<uint32_t*>(a.Kc + crow * kD + 64 + 4 * j16) = ck.y;
      } else {
        unpack8v(kraw[p], x);
        const uint2 ck = quant_row16(x, sk);
        *reinterpret_cast<uint2*>(tile + r * kD + 16 * ((j16 >> 1) ^ kswz(r)) + 8 * (j16 & 1)) = ck;
        *reinterpret_cast<uint2*>(a.Kc + crow * kD + 8 * j16) = ck;
      }
      unpack8v(vraw[p], x);
      const uint2 cv = quant_row16(x, sv);
      *reinterpret_cast<uint2*>(tile + kVOff8 + r * kD + 16 * ((j16 >> 1) ^ vswz8(r)) + 8 * (j16 & 1)) = cv;
      *reinterpret_cast<uint2*>(a.Vc + crow * kD + 8 * j16) = cv;
      if (j16 == 0) {
        scl[p][r >> 3][r & 7] = sk;
        scl[p][r >> 3][8 + (r & 7)] = sv;
        a.Ks[crow] = sk;
        a.Vs[crow] = sv;
      }
    }
  }
  arrive(&cnt[kCntQNormed], lane);
  await(&cnt[kCntQNormed], kComputeWaves, a.spin_limit, expired);  // all 128 query rows (and the own blocks) are in LDS

  const int qgrp = wave & 3;  // query rows 32 qgrp .. +31
  const int par = wave >> 2;  // blocks b with b % 2 == par
  const int n = lane & 31;
  const int h = lane >> 5;
  const int qrow = 32 * qgrp + n;
  bf16x8 qf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    qf[kk] = *reinterpret_cast<const bf16x8*>(qlds + qrow * 256 + 16 * ((dcol(kk, h) >> 3) ^ qswz(qrow)));
  arrive(&cnt[kCntQRead], lane);

  f32x16 o[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sc = kLog2e * 0.08838834764831845f;  // log2(e) / sqrt(128)
  const int krow = perm_key(n);
  // K: k-steps 2m, 2m+1 are the low and high 8 bytes of chunk 2h + m (m < 2) or 4 + 2h + m - 2
  int koff[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) koff[m] = krow * kD + 16 * (((m < 2) ? 2 * h + m : 4 + 2 * h + m - 2) ^ kswz(krow));
  // V^T: 16-lane group G = lane >> 4, lane s = lane & 15 points at row 8 (G >> 1) + (s >> 1) (+ 16
  // for the second half of the block), byte 32 t + 16 (G & 1) + 8 (s & 1)
  const int G = lane >> 4, sl = lane & 15;
  const int vrow0 = 8 * (G >> 1) + (sl >> 1);
  int voff[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) voff[t] = kVOff8 + vrow0 * kD + 16 * ((2 * t + (G & 1)) ^ vswz8(vrow0)) + 8 * (sl & 1);

  static_for<NB>([&](auto bc) {
    constexpr int b = decltype(bc)::value;
    const int kb = k_begin + b * kBlk;
    if ((b & 1) != par) return;
    await(&cnt[kCntBlock + b], kLoaderWaves, a.spin_limit, expired);
    if (kb < k_end) {
      const uint8_t* tile = &tiles[b][0];
      f32x16 s;
      {
        u32x4 kr[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) kr[m] = *reinterpret_cast<const u32x4*>(tile + koff[m]);
        bf16x8 kf[8];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          kf[2 * m] = e4m3x8_to_bf16(kr[m][0], kr[m][1]);
          kf[2 * m + 1] = e4m3x8_to_bf16(kr[m][2], kr[m][3]);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[kk], s, 0, 0, 0);
      }
      // key scales: accumulator element i of lane half h is key 8h + i (i < 8) or 16 + 8h + i - 8
      {
        const f32x4* s0 = reinterpret_cast<const f32x4*>(&scl[b][h][0]);
        const f32x4* s1 = reinterpret_cast<const f32x4*>(&scl[b][2 + h][0]);
        const f32x4 k0 = s0[0], k1 = s0[1], k2 = s1[0], k3 = s1[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[e] *= k0[e];
          s[4 + e] *= k1[e];
          s[8 + e] *= k2[e];
          s[12 + e] *= k3[e];
        }
      }
      if (kb + kBlk > k_end) {
        const int lim = k_end - kb - 8 * h;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kofs = 16 * (i >> 3) + 4 * ((i >> 2) & 1) + (i & 3);
          s[i] = (kofs < lim) ? s[i] : -INFINITY;
        }
      }
      float bmax = s[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) bmax = fmaxf(bmax, s[i]);
      {
        const float2 pr = pair32(bmax);
        bmax = fmaxf(pr.x, pr.y);
      }
      const float m_blk = bmax * sc;
      if constexpr (b < 2) {
        m_run = m_blk;
      } else if (__any(m_blk > m_run + kRescale)) {
        const float m_new = fmaxf(m_run, m_blk);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
      }
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], sc, -m_run));
        psum += s[i];
      }
      l_run += psum;
      // O^T += V^T (P diag(vscale))^T in two halves of 16 keys: half c, element j is key 16c + 8h + j
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const f32x4* vsp = reinterpret_cast<const f32x4*>(&scl[b][2 * c + h][8]);
        const f32x4 va = vsp[0] * 0x1p64f, vb = vsp[1] * 0x1p64f;  // 2^kF8VShift
        bf16x8 pb;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pb[j] = (__bf16)(s[8 * c + j] * va[j]);
          pb[4 + j] = (__bf16)(s[8 * c + 4 + j] * vb[j]);
        }
        v2i32 vt[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          vt[t] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32*)(tile + 16 * c * kD + voff[t]));
#pragma unroll
        for (int t = 0; t < 4; ++t)
          o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(e4m3x8_to_bf16((uint32_t)vt[t][0], (uint32_t)vt[t][1]), pb,
                                                         o[t], 0, 0, 0);
      }
    }
    arrive(&cnt[kCntDone + b], lane);
  });

  // merge hand-off in tiles 2 qgrp and 2 qgrp + 1, once their blocks (if any) are consumed
  auto region_free = [&]() {
    if (2 * qgrp < NB) await(&cnt[kCntDone + 2 * qgrp], 4, a.spin_limit, expired);
    if (2 * qgrp + 1 < NB) await(&cnt[kCntDone + 2 * qgrp + 1], 4, a.spin_limit, expired);
  };
  const long long part = (long long)g * a.n_split + split;
  merge_and_store_partial(o, m_run, l_run, NB >= 2, par, qgrp, lane, &tiles[2 * qgrp][0], &tiles[2 * qgrp + 1][0],
                          region_free, mlx, cnt, a.po, a.pm, a.pl, a.pe, part, a.spin_limit, expired);
  report_expired(a.status, expired, lane);
}

// Stand-alone tail write: row (tensor, head g, token i) of k (roped) and v quantised per row
// into cache row Smax - 64 + i of head g, codes and scale. 16 lanes per row.
__global__ __launch_bounds__(256) void k_tail_quant_f8(const uint16_t* k, const uint16_t* v, uint8_t* Kc, float* Ks,
                                                       uint8_t* Vc, float* Vs, int Smax) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int row = t >> 4;          // 0 .. 1023: k rows, then v rows
  const int j16 = t & 15;
  const bool is_v = row >= kHkv * kT;
  const int r = row & (kHkv * kT - 1);
  const int g = r / kT, tok = r % kT;
  const u32x4 raw = *reinterpret_cast<const u32x4*>((is_v ? v : k) + (long long)r * kD + 8 * j16);
  float x[8];
  unpack8v(raw, x);
  float scale;
  const uint2 codes = quant_row16(x, scale);
  const long long crow = (long long)g * Smax + Smax - kT + tok;
  *reinterpret_cast<uint2*>((is_v ? Vc : Kc) + crow * kD + 8 * j16) = codes;
  if (j16 == 0) (is_v ? Vs : Ks)[crow] = scale;
}

// Combine of the fp8 kernel's partials: out = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c,
// M = max_c m_c, O_c the float16 partial times 2^(e_c). Workgroup (head g, rows 8r .. 8r+7, column half hc): 512 threads in 4 split
// groups of 128 (8 rows x 16 column quads); group k reduces splits k, k + 4, ..., issuing the loads
// of up to kCombBatch splits before using any of them, so the whole partial set is in flight at
// once. The 8 rows of a (slot, half) of the accumulator layout are one 128-byte line. The groups
// meet in LDS.
constexpr int kCombGroups = 4;
constexpr int kCombBatch = 8;
__global__ __launch_bounds__(512) void k_attn_f8_combine(const float* po, const float* pm, const float* pl,
                                                         const int* pe, uint16_t* out, int n_split) {
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
  const int* peg = pe + (long long)g * n_split * kQRows + q;
  const u32x2* pog = reinterpret_cast<const u32x2*>(po) + ((long long)g * n_split * 4 + (q >> 5)) * (16 * 64) +
                     slot * 64 + lane;
  const long long pstride = 4 * 16 * 64;  // 4-float16 groups per split partial
  float M = -INFINITY, L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = grp; c0 < n_split; c0 += kCombGroups * kCombBatch) {
    float mv[kCombBatch], lv[kCombBatch];
    int ev[kCombBatch];
    f32x4 ov[kCombBatch];
#pragma unroll
    for (int k = 0; k < kCombBatch; ++k) {
      const int c = min(c0 + kCombGroups * k, n_split - 1);  // past the end: a repeat, weighted 0 below
      mv[k] = pmg[(long long)c * kQRows];
      lv[k] = plg[(long long)c * kQRows];
      ev[k] = peg[(long long)c * kQRows];
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
      const float wo = __builtin_ldexpf(w, ev[k]);  // O_c = float16 partial x 2^e_c
      acc[0] += wo * ov[k][0]; acc[1] += wo * ov[k][1]; acc[2] += wo * ov[k][2]; acc[3] += wo * ov[k][3];
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

static size_t align256_f8(size_t x) { return (x + 255) & ~size_t(255); }

// The status word, then O, m, l and e, each 256-byte aligned.
size_t attn_partials_bytes_f8(const AttnPlan& p) {
  const size_t parts = (size_t)kHkv * p.n_split;
  return kStatusBytes + align256_f8(parts * kD * kQRows * 2) + 3 * align256_f8(parts * kQRows * 4);
}

WsLayoutF8 ws_layout_f8(const AttnPlan& plan, const void* ws) {
  const size_t parts = (size_t)kHkv * plan.n_split;
  char* w = static_cast<char*>(const_cast<void*>(ws));
  WsLayoutF8 l;
  l.status = reinterpret_cast<int*>(w);
  w += kStatusBytes;
  l.po = reinterpret_cast<float*>(w);
  w += align256_f8(parts * kD * kQRows * 2);
  l.pm = reinterpret_cast<float*>(w);
  w += align256_f8(parts * kQRows * 4);
  l.pl = reinterpret_cast<float*>(w);
  w += align256_f8(parts * kQRows * 4);
  l.pe = reinterpret_cast<int*>(w);
  return l;
}

hipError_t launch_attn_f8_combine(const AttnPlan& plan, const void* ws, uint16_t* out, hipStream_t st) {
  const WsLayoutF8 l = ws_layout_f8(plan, ws);
  hipLaunchKernelGGL(k_attn_f8_combine, dim3(kHkv * 32), dim3(512), 0, st, l.po, l.pm, l.pl, l.pe, out,
                     plan.n_split);
  return hipGetLastError();
}

AttnPlan attn_plan_f8(int S, int /*Smax*/) {
  AttnPlan p;
  p.n_keys = S + kT;
  const int target = 31;  // cache splits per head; with the own split 8 x 32 = 256 workgroups
  int kps = (S + target - 1) / target;
  if (kps < kBlk) kps = kBlk;
  if (kps > kBlk * kMaxNB8) kps = kBlk * kMaxNB8;
  p.keys_per_split = kps;
  p.n_cache_split = (S + kps - 1) / kps;
  p.n_split = p.n_cache_split + 1;
  p.blocks = (kps + kBlk - 1) / kBlk;
  if (p.blocks < kT / kBlk) p.blocks = kT / kBlk;
  return p;
}

template <int NB>
static hipError_t launch_f8_nb(const F8Args& a, bool norm, hipStream_t st) {
  if (norm)
    hipLaunchKernelGGL((k_attn_f8<NB, true>), dim3(kHkv * a.n_split), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((k_attn_f8<NB, false>), dim3(kHkv * a.n_split), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_f8_split(const AttnPlan& plan, const AttnLaunchF8& p, hipStream_t st) {
  const WsLayoutF8 l = ws_layout_f8(plan, p.ws);
  F8Args a;
  a.q = p.q;
  a.gq = p.gq;
  a.gk = p.gk;
  a.cos_t = p.cos_t;
  a.sin_t = p.sin_t;
  a.eps = p.eps;
  a.k_own = p.k_own;
  a.v_own = p.v_own;
  a.Kc = p.Kc;
  a.Ks = p.Ks;
  a.Vc = p.Vc;
  a.Vs = p.Vs;
  a.po = l.po;
  a.pm = l.pm;
  a.pl = l.pl;
  a.pe = l.pe;
  a.status = l.status;
  a.spin_limit = wait_limit();
  a.S = p.S;
  a.Smax = p.Smax;
  a.n_split = plan.n_split;
  a.kps = plan.keys_per_split;
  a.n_cache_split = plan.n_cache_split;
  const bool norm = p.q_norm != 0;
  switch (plan.blocks) {
    case 2: return launch_f8_nb<2>(a, norm, st);
    case 3: return launch_f8_nb<3>(a, norm, st);
    case 4: return launch_f8_nb<4>(a, norm, st);
    case 5: return launch_f8_nb<5>(a, norm, st);
    case 6: return launch_f8_nb<6>(a, norm, st);
    case 7: return launch_f8_nb<7>(a, norm, st);
    case 8: return launch_f8_nb<8>(a, norm, st);
    case 9: return launch_f8_nb<9>(a, norm, st);
    case 10: return launch_f8_nb<10>(a, norm, st);
    case 11: return launch_f8_nb<11>(a, norm, st);
    case 12: return launch_f8_nb<12>(a, norm, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_f8(const AttnPlan& plan, const AttnLaunchF8& p, hipStream_t st) {
  const hipError_t e = launch_attn_f8_split(plan, p, st);
  if (e != hipSuccess) return e;
  return launch_attn_f8_combine(plan, p.ws, p.out, st);
}

hipError_t launch_tail_quant_f8(const uint16_t* k, const uint16_t* v, uint8_t* Kc, float* Ks, uint8_t* Vc,
                                float* Vs, int Smax, hipStream_t st) {
  hipLaunchKernelGGL(k_tail_quant_f8, dim3(2 * kHkv * kT * 16 / 256), dim3(256), 0, st, k, v, Kc, Ks, Vc, Vs, Smax);
  return hipGetLastError();
}

}  // namespace ax
