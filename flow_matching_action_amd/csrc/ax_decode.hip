// Single-token decode attention of the text model: the attention part of one decode step of a
// layer with 64 query heads and 8 kv heads of width 128.
//
// What is computed: page code/alpamayo_tt/text.py, TTTextModel._layer_decode - q and k of the
// new token RMSNormed per head and roped at position pos + rope_delta, the roped k and the v
// written into cache row pos (paged_update_cache), then every query head h attends to rows
// [0, pos] of kv head h / 8 with scale 1/sqrt(128) (scaled_dot_product_attention_decode with
// cur_pos = pos). The key range is split and the splits combined as in the expert step:
//   m_c = max_j s_j, l_c = sum_j 2^(s_j - m_c), O_c = sum_j 2^(s_j - m_c) v_j,
//   out = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c,  s_j = log2(e) (q . k_j) / sqrt(128).
//
// gfx950 mapping
// - One workgroup of 8 waves per (kv head, key split of at most 8 blocks of 32 keys); 32 splits
//   per head when the keys allow, so 256 workgroups stream the cache once.
// - Waves 4..7 (loaders) stream the split's blocks into their own LDS tiles (direct-to-LDS
//   loads, rows 256 bytes, swizzled as in the expert kernel), a few blocks ahead, and count
//   each landed block in LDS. Key pos comes from the new token's raw k / v instead of the
//   cache; the compute wave that consumes its block norms and ropes that k row in the tile
//   and writes both rows to cache row pos.
// - Waves 0..3 (compute): wave 0 norms and ropes the 8 query rows of the kv head into LDS;
//   wave w consumes blocks w, w + 4. The 8 rows are the first 8 of the expert kernel's 16-row
//   MFMA layout and tiles (S^T = K Q^T per 16-key half on v_mfma_f32_16x16x32_bf16, O^T += V^T
//   P^T with P^T straight from the score accumulators and V^T read by ds_read_b64_tr_b16); rows
//   8..15 are zero. (On the 32-row layout, with 24 zero rows, the block arithmetic took ~2.2 us
//   of the step; this layout halves it.)
// - The compute waves merge their (m, l, O) through LDS; wave 0 stores the split's partial
//   (8 rows). k_decode_combine then reduces the splits of each of the 64 output rows.
#include "ax_attn_common.h"
#include "ax_launch.h"

namespace ax {

constexpr int kDecQHeads = 64;
constexpr int kDecRows = kDecQHeads / kHkv;   // 8 query rows (heads) per kv head
constexpr int kDecCompute = 4;                // compute waves
constexpr int kDecLoaders = 4;                // loader waves (8 rows of each block each)
constexpr int kDecThreads = 64 * (kDecCompute + kDecLoaders);
constexpr int kDecDepth = 3;                  // blocks in flight per loader wave
// LDS hand-off counters: query rows normed, block b landed, merge data of the compute waves ready
constexpr int kDcQ = 0, kDcBlock = 1, kDcMerge = kDcBlock + 8, kDcN = kDcMerge + 1;
constexpr int kDecMaxNB = 8;                  // blocks per split (LDS: 8 x 16 KB)
constexpr int kDecTile = 2 * kBlk * kD * 2;   // K 8 KB + V 8 KB

struct DecArgs {
  const uint16_t* q;      // [64][128] raw
  const uint16_t* k;      // [8][128] raw
  const uint16_t* v;      // [8][128]
  const uint16_t* gq;
  const uint16_t* gk;
  const float* cos_t;     // [64]: cos of (pos + rope_delta) * theta^(-2j/128)
  const float* sin_t;
  float eps;
  uint16_t* Kc;           // [8][Smax][128]
  uint16_t* Vc;
  float* po;              // [8][n_split][8 rows][128]
  float* pm;              // [8][n_split][8]
  float* pl;
  int* status;            // workspace status word
  int spin_limit;         // polls before a wait gives up
  int pos, Smax, n_split, kps;
};

template <int NB>
__global__ __launch_bounds__(kDecThreads, 1) void k_decode_attn(DecArgs a) {
  static_assert(NB >= 1 && NB <= kDecMaxNB, "blocks per split");
  __shared__ __attribute__((aligned(16))) uint8_t tiles[NB][kDecTile];
  __shared__ __attribute__((aligned(16))) uint8_t qlds[kDecRows * 256];
  // merge hand-off of compute waves 1..3: O of rows 0..7 (column tile dt, slot (row, group)), m and l
  __shared__ f32x4 mo[kDecCompute - 1][8][32];
  __shared__ float mml[kDecCompute - 1][2][kDecRows];
  __shared__ int cnt[kDcN];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int j16 = lane & 15;
  const int g = blockIdx.x % kHkv;
  const int split = blockIdx.x / kHkv;
  const int n_keys = a.pos + 1;
  const int k_begin = split * a.kps;
  const int k_end = min(k_begin + a.kps, n_keys);
  const long long head_row = (long long)g * a.Smax;

  if (tid < kDcN) cnt[tid] = 0;
  lds_barrier();  // counters cleared (the only workgroup barrier)
  bool expired = false;  // a bounded wait of this wave ran out

  if (wave >= kDecCompute) {
    // ---------------- loader waves: rows 8w .. 8w+7 of each block, K then V (two 1 KB loads each)
    const int w = wave - kDecCompute;
    auto issue_block = [&](auto bc) {
      constexpr int b = decltype(bc)::value;
      uint8_t* tile = &tiles[b][0];
      static_for<2>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const int r = 8 * w + 4 * i + (lane >> 4);
        int kk = k_begin + b * kBlk + r;
        kk = kk < k_end ? kk : k_begin;  // rows past the split end reload a visible row (masked)
        const bool is_new = kk == a.pos;
        const uint16_t* ks = is_new ? a.k + (long long)g * kD : a.Kc + (head_row + kk) * kD;
        const uint16_t* vs = is_new ? a.v + (long long)g * kD : a.Vc + (head_row + kk) * kD;
        // non-temporal: the decode step measured 5% faster than with ordinary reads
        __builtin_amdgcn_global_load_lds(ks + 8 * ((lane & 15) ^ kswz16(r)), (lds_void*)(tile + (8 * w + 4 * i) * 256),
                                         16, 0, kNonTemporal);
        __builtin_amdgcn_global_load_lds(vs + 8 * ((lane & 15) ^ vswz16(r)),
                                         (lds_void*)(tile + kDecTile / 2 + (8 * w + 4 * i) * 256), 16, 0, kNonTemporal);
      });
    };
    constexpr int D = NB < kDecDepth ? NB : kDecDepth;
    static_for<D>([&](auto bc) { issue_block(bc); });
    static_for<NB>([&](auto bc) {
      constexpr int b = decltype(bc)::value;
      constexpr int later = (b + D - 1 < NB - 1 ? b + D - 1 : NB - 1) - b;
      wait_vmcnt<4 * later>();  // four loads per block, in block order: block b has landed
      arrive(&cnt[kDcBlock + b], lane);
      if constexpr (b + D < NB) issue_block(std::integral_constant<int, b + D>{});
    });
    return;
  }

  // ---------------- compute waves
  const u32x4 graw = *reinterpret_cast<const u32x4*>(a.gq + 8 * j16);
  const u32x4 gkraw = *reinterpret_cast<const u32x4*>(a.gk + 8 * j16);
  f32x4 cs_h[2];
  load_cos_sin_half(a.cos_t, a.sin_t, 0, j16, cs_h[0], cs_h[1]);
  if (wave == 0) {
    // the 8 query rows of head g: rows 4i + (lane >> 4), i = 0, 1 (lane l lands at 16 l)
    static_for<2>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int row = 4 * i + (lane >> 4);
      const uint16_t* src = a.q + (long long)(kDecRows * g + row) * kD + 8 * ((lane & 15) ^ qswz(row));
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(qlds + 4 * i * 256), 16, 0, 0);
    });
  }
  float qc[8], qs[8], A[8], B[8];
  split_cos_sin(cs_h[0], cs_h[1], j16, qc, qs);
  wait_vmcnt<0>();
  if (wave == 0) {
    // norm + RoPE of the query rows in place, 16 lanes per row, 4 rows per pass
    float qg[8];
    unpack8v(graw, qg);
    rope_coef(qg, qc, qs, j16, A, B);
    u32x4 qv[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int r = 4 * p + (lane >> 4);
      qv[p] = *reinterpret_cast<const u32x4*>(qlds + r * 256 + 16 * (j16 ^ qswz(r)));
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      float x[8];
      unpack8v(qv[p], x);
      norm_rope_row16(x, A, B, a.eps);
      qv[p] = pack8v(x);
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int r = 4 * p + (lane >> 4);
      *reinterpret_cast<u32x4*>(qlds + r * 256 + 16 * (j16 ^ qswz(r))) = qv[p];
    }
    arrive(&cnt[kDcQ], lane);
  }
  await(&cnt[kDcQ], 1, a.spin_limit, expired);

  // The query rows as MFMA B operands (16 rows of the 16-row layout; rows 8..15 are zero): k-step
  // kk takes columns 32 kk .. 32 kk + 31; lane l holds row l & 15, columns 32 kk + 8 (l >> 4) ..
  const int g4 = lane >> 4;
  bf16x8 qf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    if (j16 < kDecRows) {
      qf[kk] = *reinterpret_cast<const bf16x8*>(qlds + j16 * 256 + 16 * ((4 * kk + g4) ^ qswz(j16)));
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[kk][e] = (__bf16)0.f;
    }
  }

  f32x4 o[8];  // O^T: lane l holds O[row l & 15][16 dt + 4 (l >> 4) + i]
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;  // the lane's row; l_run is the lane's share of its sum
  const float sc = kLog2e * 0.08838834764831845f;  // log2(e) / sqrt(128)
  // K: key row 16 t + j16, chunk 4 kk + g4 (the second half of the keys 4 KB further on)
  int koff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) koff[kk] = j16 * 256 + 16 * ((4 * kk + g4) ^ kswz16(j16));
  // V^T: lane j16 of group g4 supplies key row 4 g4 + (j16 >> 2) (+ 16 for the second read),
  // columns 16 dt + 4 (j16 & 3) .. + 3
  const int vr = 4 * g4 + (j16 >> 2);
  int voff[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
    voff[dt] = kDecTile / 2 + vr * 256 + 16 * ((2 * dt + ((j16 & 3) >> 1)) ^ vswz16(vr)) + 8 * (j16 & 1);

  static_for<NB>([&](auto bc) {
    constexpr int b = decltype(bc)::value;
    if (b % kDecCompute != wave) return;
    const int kb = k_begin + b * kBlk;
    await(&cnt[kDcBlock + b], kDecLoaders, a.spin_limit, expired);
    if (kb >= k_end) return;
    uint8_t* tile = &tiles[b][0];
    // (a split's last block can reach past the split's end: key pos must be one of this split's)
    if (a.pos >= kb && a.pos < min(kb + kBlk, k_end) && lane < 16) {
      // the new token's k row: norm + RoPE in place, then both rows to cache row pos
      const int r = a.pos - kb;
      u32x4* kp = reinterpret_cast<u32x4*>(tile + r * 256 + 16 * (j16 ^ kswz16(r)));
      const u32x4 vraw = *reinterpret_cast<const u32x4*>(tile + kDecTile / 2 + r * 256 + 16 * (j16 ^ vswz16(r)));
      float gkv[8], x[8];
      unpack8v(gkraw, gkv);
      rope_coef(gkv, qc, qs, j16, A, B);
      unpack8v(*kp, x);
      norm_rope_row16(x, A, B, a.eps);
      const u32x4 kr = pack8v(x);
      *kp = kr;
      const long long dst = (head_row + a.pos) * kD + 8 * j16;
      *reinterpret_cast<u32x4*>(a.Kc + dst) = kr;
      *reinterpret_cast<u32x4*>(a.Vc + dst) = vraw;
    }
    // S^T = K Q^T per 16-key half t: lane l holds row j16 against keys 16 t + 4 g4 + i
    f32x4 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      bf16x8 kf[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) kf[kk] = *reinterpret_cast<const bf16x8*>(tile + koff[kk] + 4096 * t);
      s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kk], qf[kk], s[t], 0, 0, 0);
    }
    if (kb + kBlk > k_end) {
      const int lim = k_end - kb - 4 * g4;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[t][i] = (16 * t + i < lim) ? s[t][i] : -INFINITY;
    }
    // the row's block max: the lane's 8 keys, then the four lanes j16 + 16 i of the row
    float bmax = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                       fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    {
      const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(bmax), __float_as_uint(bmax), false, false);
      bmax = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
      const float2 pr = pair32(bmax);
      bmax = fmaxf(pr.x, pr.y);
    }
    const float m_blk = bmax * sc;
    if constexpr (b < kDecCompute) {
      m_run = m_blk;  // the wave's first block holds a visible key
    } else if (__any(m_blk > m_run + kRescale)) {
      const float m_new = fmaxf(m_run, m_blk);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[dt][i] *= alpha;
    }
    // p as P^T straight from the two score accumulators (slots 0..3: keys 4 g4 + i, 4..7: keys
    // 16 + 4 g4 + i); the row sum adds the same bf16-rounded p that the PV product uses, so each
    // output row is an exact convex combination of v rows
    const bf16x2_t one2 = {(__bf16)1.0f, (__bf16)1.0f};
    bf16x8 pb;
    float ps = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const bf16x2_t pr = {(__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[t][i], sc, -m_run)),
                             (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[t][i + 1], sc, -m_run))};
        pb[4 * t + i] = pr[0];
        pb[4 * t + i + 1] = pr[1];
        ps = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, ps, false);
      }
    l_run += ps;
    // O^T += V^T P^T per 16-column tile dt (V^T in the same key order: two ds_read_b64_tr_b16)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const v4i16 both[2] = {__builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(tile + voff[dt])),
                             __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(tile + voff[dt] + 4096))};
      bf16x8 vf;
      __builtin_memcpy(&vf, both, 16);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb, o[dt], 0, 0, 0);
    }
  });

  // merge of the compute waves (rows 0..7: lanes j16 < 8), then the partial
  float l_tot = l_run;  // the row's total: its four lanes' shares
  {
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(l_tot), __float_as_uint(l_tot), false, false);
    l_tot = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    const float2 pr = pair32(l_tot);
    l_tot = pr.x + pr.y;
  }
  const int ml = (lane & 7) + 8 * g4;  // merge slot of lane (row j16 < 8, group g4)
  if (wave > 0) {
    if (j16 < kDecRows) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) mo[wave - 1][dt][ml] = o[dt];
      if (g4 == 0) {
        mml[wave - 1][0][j16] = m_run;
        mml[wave - 1][1][j16] = l_tot;
      }
    }
    arrive(&cnt[kDcMerge], lane);
    report_expired(a.status, expired, lane);
    return;
  }
  await(&cnt[kDcMerge], kDecCompute - 1, a.spin_limit, expired);
  report_expired(a.status, expired, lane);
  if (j16 >= kDecRows) return;
  float m_all = m_run, l_all = l_tot;  // block 0 holds a visible key: m_run is finite
#pragma unroll
  for (int w = 0; w < kDecCompute - 1; ++w) {
    const float m_o = mml[w][0][j16];
    const float l_o = mml[w][1][j16];
    const float m_new = fmaxf(m_all, m_o);
    const float ae = __builtin_amdgcn_exp2f(m_all - m_new);
    const float ao = __builtin_amdgcn_exp2f(m_o - m_new);  // 0 for a wave without blocks (m = -inf)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const f32x4 x = mo[w][dt][ml];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[dt][e] = ae * o[dt][e] + ao * x[e];
    }
    l_all = ae * l_all + ao * l_o;
    m_all = m_new;
  }
  const long long prow = ((long long)g * a.n_split + split) * kDecRows + j16;
  // lane (row j16, group g4) holds columns 16 dt + 4 g4 .. +3 of row j16
  f32x4* po = reinterpret_cast<f32x4*>(a.po + prow * kD);
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) po[4 * dt + g4] = o[dt];
  if (g4 == 0) {
    a.pm[prow] = expired ? __builtin_nanf("") : m_all;
    a.pl[prow] = l_all;
  }
}

// Combine of the splits: workgroup (head g, row r) = output row 8 g + r (query head 8 g + r):
// 512 threads in 4 split groups of 128 columns; group k reduces splits k, k + 4, ..., issuing the
// loads of 8 splits before using any of them, so 32 splits are in flight at once. The groups
// meet in LDS. Fixed order.
constexpr int kDecCombGroups = 4;
constexpr int kDecCombBatch = 8;
__global__ __launch_bounds__(kDecCombGroups * kD) void k_decode_combine(const float* po, const float* pm,
                                                                        const float* pl, uint16_t* out,
                                                                        int n_split) {
  __shared__ float sM[kDecCombGroups], sL[kDecCombGroups];
  __shared__ float sA[kDecCombGroups][kD];
  const int g = blockIdx.x / kDecRows;
  const int r = blockIdx.x % kDecRows;
  const int grp = threadIdx.x / kD;
  const int d = threadIdx.x % kD;
  const long long base = (long long)g * n_split * kDecRows + r;  // row of split c: base + c * 8
  float M = -INFINITY, L = 0.f, acc = 0.f;
  for (int c0 = grp; c0 < n_split; c0 += kDecCombGroups * kDecCombBatch) {
    float mv[kDecCombBatch], lv[kDecCombBatch], xv[kDecCombBatch];
#pragma unroll
    for (int k = 0; k < kDecCombBatch; ++k) {
      const int c = min(c0 + kDecCombGroups * k, n_split - 1);  // past the end: a repeat, weighted 0 below
      const long long row = base + (long long)c * kDecRows;
      mv[k] = pm[row];
      lv[k] = pl[row];
      xv[k] = po[row * kD + d];
    }
    __builtin_amdgcn_sched_barrier(0);  // every load of the batch is issued before any is used
    float Mb = M;
#pragma unroll
    for (int k = 0; k < kDecCombBatch; ++k)
      if (c0 + kDecCombGroups * k < n_split) Mb = fmaxf(Mb, mv[k]);
    const float rs = __builtin_amdgcn_exp2f(M - Mb);  // 0 while M is -inf
    L *= rs;
    acc *= rs;
    M = Mb;
#pragma unroll
    for (int k = 0; k < kDecCombBatch; ++k) {
      const float w = (c0 + kDecCombGroups * k < n_split) ? __builtin_amdgcn_exp2f(mv[k] - M) : 0.f;
      L += w * lv[k];
      acc += w * xv[k];
    }
  }
  if (d == 0) {
    sM[grp] = M;
    sL[grp] = L;
  }
  sA[grp][d] = acc;
  __syncthreads();
  if (grp != 0) return;
  float Mt = sM[0];  // group 0 holds split 0, so Mt is finite
#pragma unroll
  for (int k = 1; k < kDecCombGroups; ++k) Mt = fmaxf(Mt, sM[k]);
  float Lt = 0.f, At = 0.f;
#pragma unroll
  for (int k = 0; k < kDecCombGroups; ++k) {
    const float w = __builtin_amdgcn_exp2f(sM[k] - Mt);  // 0 for a group without splits
    Lt += w * sL[k];
    At += w * sA[k][d];
  }
  out[(long long)blockIdx.x * kD + d] = (uint16_t)f32_to_bf16(At / Lt);
}

AttnPlan decode_plan(int pos) {
  AttnPlan p;
  p.n_keys = pos + 1;
  const int target = 32;  // splits per head: 8 x 32 = 256 workgroups
  int kps = (p.n_keys + target - 1) / target;
  if (kps < kBlk) kps = kBlk;
  if (kps > kBlk * kDecMaxNB) kps = kBlk * kDecMaxNB;
  p.keys_per_split = kps;
  p.n_split = (p.n_keys + kps - 1) / kps;
  p.n_cache_split = p.n_split;
  p.blocks = (kps + kBlk - 1) / kBlk;
  return p;
}

static size_t align256d(size_t x) { return (x + 255) & ~size_t(255); }

// The status word, then O, m and l, each 256-byte aligned.
size_t decode_partials_bytes(const AttnPlan& p) {
  const size_t rows = (size_t)kHkv * p.n_split * kDecRows;
  return kStatusBytes + align256d(rows * kD * 4) + 2 * align256d(rows * 4);
}

template <int NB>
static hipError_t launch_dec_nb(const DecArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((k_decode_attn<NB>), dim3(kHkv * a.n_split), dim3(kDecThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_decode(const AttnPlan& plan, const DecodeLaunch& p, hipStream_t st) {
  const size_t rows = (size_t)kHkv * plan.n_split * kDecRows;
  char* w = static_cast<char*>(p.ws);
  DecArgs a;
  a.status = reinterpret_cast<int*>(w);
  a.spin_limit = wait_limit();
  w += kStatusBytes;
  a.q = p.q; a.k = p.k; a.v = p.v; a.gq = p.gq; a.gk = p.gk; a.cos_t = p.cos_t; a.sin_t = p.sin_t; a.eps = p.eps;
  a.Kc = p.Kc; a.Vc = p.Vc;
  a.po = reinterpret_cast<float*>(w);
  a.pm = reinterpret_cast<float*>(w + align256d(rows * kD * 4));
  a.pl = reinterpret_cast<float*>(w + align256d(rows * kD * 4) + align256d(rows * 4));
  a.pos = p.pos; a.Smax = p.Smax; a.n_split = plan.n_split; a.kps = plan.keys_per_split;
  hipError_t e;
  switch (plan.blocks) {
    case 1: e = launch_dec_nb<1>(a, st); break;
    case 2: e = launch_dec_nb<2>(a, st); break;
    case 3: e = launch_dec_nb<3>(a, st); break;
    case 4: e = launch_dec_nb<4>(a, st); break;
    case 5: e = launch_dec_nb<5>(a, st); break;
    case 6: e = launch_dec_nb<6>(a, st); break;
    case 7: e = launch_dec_nb<7>(a, st); break;
    default: e = launch_dec_nb<8>(a, st); break;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_decode_combine, dim3(kHkv * kDecRows), dim3(kDecCombGroups * kD), 0, st, a.po, a.pm, a.pl,
                     p.out, plan.n_split);
  return hipGetLastError();
}

}  // namespace ax
