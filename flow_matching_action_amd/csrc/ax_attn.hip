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
// - One workgroup of 12 waves per (kv head, key split); workgroup id w -> head w % 8,
//   which the dispatcher places on XCD w % 8, so a head's splits share one L2. The cache
//   keys [0, S) are cut into splits of at most 6 blocks of 32 keys; the 64 own tokens
//   form one more split of their own.
// - Waves 8..11 (loaders) stream the split's K/V rows into per-block LDS tiles with
//   direct-to-LDS loads (global_load_lds, 16 bytes per lane), a few blocks ahead, and
//   count each landed block in LDS; rows are 256 bytes with the 16-byte chunks
//   XOR-swizzled by row.
// - Waves 0..7 (compute) fetch and norm/rope the 128 query rows in place in LDS (16
//   lanes per row, the same arithmetic as the stand-alone norm/RoPE kernel); in the own
//   split they also norm/rope the own k rows and write the cache tail. Then wave w takes
//   query rows 32 (w & 3) .. +31 over the blocks of parity w >> 2: S^T = K Q^T on
//   v_mfma_f32_32x32x16_bf16 (A = K rows, B = Q^T), so each lane holds one query row's
//   scores; O^T = V^T P^T with V^T read straight from row-major V by ds_read_tr16_b64
//   and P^T taken from the S^T accumulator. Inside a block MFMA row m reads key pi(m)
//   (bits 2 and 3 swapped), which makes the 8 keys a lane supplies to one PV step
//   consecutive. The two parity waves of a query group merge through LDS and the even
//   one stores the split's partial.
#include "ax_attn_common.h"
#include "ax_launch.h"

namespace ax {

constexpr int kMaxNB = 6;                     // blocks per split, upper bound (LDS: 6 x 16 KB + 48 KB)
static_assert(kMaxNB <= kMaxBlocks, "counter layout");
constexpr int kTileBytes = 2 * kBlk * kD * 2; // K 8 KB + V 8 KB
constexpr int kDmaDepth = 3;                  // blocks of a split in flight per loader wave

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
  float* po;               // [8][n_split][4 query groups][16 slots][64 lanes]: 4 floats of O each
  float* pm;               // [8][n_split][128]
  float* pl;
  int S, Smax, n_split, kps;
  int n_cache_split;       // splits over cache keys [0, S); split n_cache_split holds the 64 own tokens
  int q_norm, tail_norm;
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

// NORM: q and the own k arrive raw and are normed + roped here (the layer step); otherwise
// both arrive roped (attention only).
//
// Wave roles (12 waves, 3 per SIMD).
// - Waves 8..11 (loaders) only issue direct-to-LDS loads - the 128 query rows of the head,
//   then the cache blocks of the split - and count each landed block in LDS. Keeping
//   ordinary loads and LDS-DMA loads in different waves keeps each wave's vmcnt in order,
//   so no wave ever has to drain its queue early; the counters (not barriers) let the loads
//   run ahead of the arithmetic.
// - Waves 0..7 (compute) norm/rope the queries in place in LDS and handle the own-token
//   rows, then wave w takes query rows 32 (w & 3) .. +31 over the blocks of parity w >> 2.
//   The two waves of a query group share a SIMD, so one's matrix-core work overlaps the
//   other's softmax. At the end the odd-parity wave hands its (m, l, O) to the even one
//   through LDS, which merges them and writes the split's partial.
template <int NB, bool NORM>
__global__ __launch_bounds__(kThreads, 1) void k_attn_fused(FusedArgs a) {
  AX_TILE(0); AX_TILE(1); AX_TILE(2); AX_TILE(3); AX_TILE(4); AX_TILE(5);
  __shared__ __attribute__((aligned(16))) uint8_t qlds[kQBytes];
  // roped own-token K rows (row tok, chunks swizzled like the tile row they stand in for)
  __shared__ __attribute__((aligned(16))) uint8_t kown[kT * 256];
  __shared__ float mlx[4][2][32];  // merge hand-off: (m, l) of the odd-parity waves per query row
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
  // blocks holding own-token rows that need the tail step (norm of k and/or cache tail write)
  const bool own_tail = a.own_tail != 0;

  if (tid < kNCnt) cnt[tid] = 0;
  if (wave < kComputeWaves) {
    // Each compute wave fetches the 16 query rows it norms (rows 32p + 4 wave .. +3, p = 0..3)
    // ahead of the cache stream; lane l lands at 16 l of the 1 KB, so it fetches the chunk
    // that the row's swizzle puts there.
    const uint16_t* qh = a.q + (long long)(2 * g) * kT * kD;  // q heads 2g, 2g+1: 128 rows, contiguous
    static_for<4>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      const int row = 32 * p + 4 * wave + (lane >> 4);
      const uint16_t* src = qh + row * kD + 8 * ((lane & 15) ^ qswz(row));
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(qlds + (32 * p + 4 * wave) * 256), 16, 0, 0);
    });
  }
  lds_barrier();  // start: counters cleared (the only workgroup barrier)

  if (wave >= kComputeWaves) {
    // ---------------- loader waves: of each block the K row groups w and w+4 and the V row
    // groups w and w+4 (4 rows each)
    const int w = wave - kComputeWaves;
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
        // non-temporal: the cache rows are read once per step and should not push other data
        // out of L2
        __builtin_amdgcn_global_load_lds(ks, (lds_void*)(tile + grp * 1024), 16, 0, kNonTemporal);
        __builtin_amdgcn_global_load_lds(vs, (lds_void*)(tile + kTileBytes / 2 + grp * 1024), 16, 0, kNonTemporal);
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

  // ---------------- compute waves (512 threads)
  const int j16 = tid & 15;
  const int r16 = tid >> 4;  // 0..31
  // 1. Prologue loads. Query pass p (0..3) covers folded row 32p + r16 (q head 2g + row/64,
  //    token row % 64), so token set p & 1: token r16 or 32 + r16; own-token row set p (0..1)
  //    is token 32p + r16 and uses the same cos/sin. Wave w's rows are the ones it fetched.
  u32x4 graw, gkraw, kraw[2], vraw[2];
  f32x4 cs_h[2][2];
  if constexpr (NORM) {
    graw = *reinterpret_cast<const u32x4*>(a.gq + 8 * j16);
#pragma unroll
    for (int p = 0; p < 2; ++p) load_cos_sin_half(a.cos_t, a.sin_t, 32 * p + r16, j16, cs_h[p][0], cs_h[p][1]);
  }
  const bool has_own = own_tail && k_end > a.S;  // this split holds own-token rows
  if (has_own) {
    const uint16_t* kt = a.kt_base + g * a.tail_stride;
    const uint16_t* vt = a.vt_base + g * a.tail_stride;
    if constexpr (NORM) gkraw = *reinterpret_cast<const u32x4*>(a.gk + 8 * j16);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int tok = 32 * p + r16;
      kraw[p] = *reinterpret_cast<const u32x4*>(kt + (long long)tok * kD + 8 * j16);
      vraw[p] = *reinterpret_cast<const u32x4*>(vt + (long long)tok * kD + 8 * j16);
    }
  }
  float qc[2][8], qs[2][8];
  if constexpr (NORM) {
#pragma unroll
    for (int p = 0; p < 2; ++p) split_cos_sin(cs_h[p][0], cs_h[p][1], j16, qc[p], qs[p]);
  }
  // 2. this wave's query rows, normed and roped in place in LDS (unless they came roped)
  wait_vmcnt<0>();  // its query rows and every prologue load have landed
  if constexpr (NORM) norm_rope_query_rows(qlds, graw, qc, qs, j16, r16, a.eps);
  // 3. own-token rows of this split: K normed + roped (or taken roped) into kown and the cache
  //    tail, V copied to the cache tail (the stores come after every load has been waited
  //    for, so no later wait includes them)
  if (has_own) {
    float gk[8];
    if constexpr (NORM) unpack8v(gkraw, gk);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int tok = 32 * p + r16;
      const int vk = a.S + tok;
      if (vk >= k_begin && vk < k_end) {
        u32x4 kv = kraw[p];
        if constexpr (NORM) {
          float x[8], A[8], B[8];
          unpack8v(kv, x);
          rope_coef(gk, qc[p], qs[p], j16, A, B);
          norm_rope_row16(x, A, B, a.eps);
          kv = pack8v(x);
        }
        const int rr = (vk - k_begin) & (kBlk - 1);
        *reinterpret_cast<u32x4*>(kown + tok * 256 + 16 * (j16 ^ kswz(rr))) = kv;
        const long long dst = head_off + (long long)(a.Smax - kT + tok) * kD + 8 * j16;
        *reinterpret_cast<u32x4*>(a.Kc + dst) = kv;
        *reinterpret_cast<u32x4*>(a.Vc + dst) = vraw[p];
      }
    }
  }
  arrive(&cnt[kCntQNormed], lane);
  await(&cnt[kCntQNormed], kComputeWaves);  // all 128 query rows and the own-token K rows are in LDS

  const int qgrp = wave & 3;  // query rows 32 qgrp .. +31
  const int par = wave >> 2;  // blocks b with b % 2 == par
  const int n = lane & 31;
  const int h = lane >> 5;
  const int qrow = 32 * qgrp + n;
  bf16x8 qf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    qf[kk] = *reinterpret_cast<const bf16x8*>(qlds + qrow * 256 + 16 * ((dcol(kk, h) >> 3) ^ qswz(qrow)));
  arrive(&cnt[kCntQRead], lane);  // this wave no longer reads qlds

  f32x16 o[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;  // running max in log2 units of the scaled score, row sum
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

  // Blocks of this wave's parity. A block past the split end (only in a short split) is
  // skipped, but still awaited and counted as consumed, so that a consumed tile is never
  // written by a load still in flight; the first block a wave processes holds at least one
  // visible key, so m_run is finite after it.
  static_for<NB>([&](auto bc) {
    constexpr int b = decltype(bc)::value;
    const int kb = k_begin + b * kBlk;
    if ((b & 1) != par) return;
    uint8_t* tile = pick<b>(t0, t1, t2, t3, t4, t5);
    await(&cnt[kCntBlock + b], kLoaderWaves);
    if (kb < k_end) {
      // S^T = K Q^T: K fragments from LDS (own-token rows from kown), then 8 MFMAs.
      f32x16 s;
      {
        bf16x8 kf[8];
        if (!own_tail || kb + kBlk <= a.S) {  // no own-token row in the block
#pragma unroll
          for (int kk = 0; kk < 8; ++kk)
            kf[kk] = *reinterpret_cast<const bf16x8*>(tile + koff[kk & 3] + 128 * (kk >> 2));
        } else {
          // own-token row tok stands in kown at row tok, swizzled like tile row krow
          const int kvk = kb + krow;
          const bool own = kvk >= a.S;
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) {
            const int off = koff[kk & 3] + 128 * (kk >> 2);
            kf[kk] = *reinterpret_cast<const bf16x8*>(own ? kown + (kvk - a.S) * 256 + (off - krow * 256) : tile + off);
          }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[kk], s, 0, 0, 0);
        // Keep four K reads in flight ahead of the dependent MFMA chain: 4 reads, then
        // (MFMA, read) x 4, then the last 4 MFMAs. Left to itself the scheduler waits for
        // each read right before its MFMA, which exposes the LDS latency eight times.
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      }
      if (kb + kBlk > k_end) {  // only a split's last block can be partial
        // accumulator element i of lane half h is key perm_key(8(i>>2) + 4h + (i&3)) = 8h + kofs(i)
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
      // The exponent reference m_run only moves when some row's max exceeds it by more than
      // kRescale (log2 units): p stays below 2^kRescale, exact for the final normalisation,
      // and the O rescale (64 multiplies) runs only on such jumps.
      const float m_blk = bmax * sc;
      if constexpr (b < 2) {
        m_run = m_blk;  // this wave's first block: O and l are still zero
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
      // v_exp_f32 directly: arguments are <= kRescale or -inf (masked)
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], sc, -m_run));
        psum += s[i];
      }
      l_run += psum;
      // O^T += V^T P^T, in two halves of 16 keys (operand layout at voff above).
      const uint8_t* tv = tile + kTileBytes / 2;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        bf16x8 pb;
#pragma unroll
        for (int j = 0; j < 8; ++j) pb[j] = (__bf16)s[8 * c + j];
        v4i16 vt[4][2];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
            vt[t][hf] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4i16*)(tv + (16 * c + 4 * hf) * 256 + 128 * (t >> 1) + voff[t & 1]));
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const v4i16 both[2] = {vt[t][0], vt[t][1]};
          bf16x8 vf;
          __builtin_memcpy(&vf, both, 16);
          o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, o[t], 0, 0, 0);
        }
      }
    }
    arrive(&cnt[kCntDone + b], lane);
  });

  // Merge of the two parities. The odd wave's O goes to a 16 KB region that nobody reads any
  // more: the tile of block qgrp once its four readers are done with it, or for qgrp >= NB a
  // half of the query buffer once every compute wave holds its query fragments.
  uint8_t* region = qlds;
  if constexpr (NB >= 2) {
    if (qgrp < NB) region = qgrp == 0 ? t0 : qgrp == 1 ? t1 : qgrp == 2 ? t2 : t3;
    else region = qlds + (qgrp - NB) * kTileBytes;
  }
  auto region_free = [&]() {
    if (qgrp < NB) await(&cnt[kCntDone + qgrp], 4);
    else await(&cnt[kCntQRead], kComputeWaves);
  };
  const long long part = (long long)g * a.n_split + split;
  merge_and_store_partial(o, m_run, l_run, NB >= 2, par, qgrp, lane, region, region + kTileBytes / 2,
                          region_free, mlx, cnt, a.po, a.pm, a.pl, part);
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
  const f32x4* pog = reinterpret_cast<const f32x4*>(po) + ((long long)g * n_split * 4 + (q >> 5)) * (16 * 64) +
                     slot * 64 + lane;
  const long long pstride = 4 * 16 * 64;  // float4s per split partial
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
      ov[k] = pog[(long long)c * pstride];
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
  return align256(parts * kD * kQRows * 4) + 2 * align256(parts * kQRows * 4);
}

template <int NB>
static hipError_t launch_nb(const FusedArgs& a, hipStream_t st) {
  if (a.q_norm)
    hipLaunchKernelGGL((k_attn_fused<NB, true>), dim3(kHkv * a.n_split), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((k_attn_fused<NB, false>), dim3(kHkv * a.n_split), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

WsLayout ws_layout(const AttnPlan& plan, const void* ws) {
  const size_t parts = (size_t)kHkv * plan.n_split;
  char* w = static_cast<char*>(const_cast<void*>(ws));
  WsLayout l;
  l.po = reinterpret_cast<float*>(w);
  l.pm = reinterpret_cast<float*>(w + align256(parts * kD * kQRows * 4));
  l.pl = reinterpret_cast<float*>(w + align256(parts * kD * kQRows * 4) + align256(parts * kQRows * 4));
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
  a.q_norm = p.q_norm; a.tail_norm = p.tail_norm;
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
