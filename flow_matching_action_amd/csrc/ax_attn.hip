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
// - One workgroup of 16 waves per (kv head, key split); workgroup id w -> head w % 8,
//   which the dispatcher places on XCD w % 8, so a head's splits share one L2.
// - Keys go in blocks of 32 visible keys (visible key v < S is cache row v; v >= S is
//   own token v - S). Every wave issues one 1 KB direct-to-LDS load per block
//   (global_load_lds, 16 bytes per lane) - waves 0..7 the K rows, 8..15 the V rows -
//   for all blocks of the split before anything waits, so a CU keeps its whole share
//   of the cache in flight from 16 waves. Each block has its own LDS tile; rows are
//   256 bytes with the 16-byte chunks XOR-swizzled by row.
// - The 128 query rows are normed and roped by all 1024 threads (16 lanes per row,
//   the same arithmetic as the stand-alone norm/RoPE kernel) into LDS; the rows of
//   own tokens are normed/roped in LDS by the block that holds them, which also
//   writes them to the cache tail.
// - Waves 0..3 compute, wave w owning query rows 32w..32w+31: S^T = K Q^T on
//   v_mfma_f32_32x32x16_bf16 (A = K rows, B = Q^T), so each lane holds one query
//   row's scores; O^T = V^T P^T with V^T read straight from row-major V by
//   ds_read_tr16_b64 and P^T taken from the S^T accumulator. Inside a block MFMA row
//   m reads key pi(m) (bits 2 and 3 swapped), which makes the 8 keys a lane supplies
//   to one PV step consecutive.
#include "ax_dev.h"
#include "ax_launch.h"

namespace ax {

constexpr int kBlk = 32;                      // keys per block
constexpr int kMaxNB = 7;                     // blocks per split, upper bound (LDS: 7 x 16 KB + 32 KB)
constexpr int kTileBytes = 2 * kBlk * kD * 2; // K 8 KB + V 8 KB
constexpr int kQBytes = kQRows * kD * 2;      // 32 KB
constexpr int kThreads = 512;
constexpr int kDmaDepth = 3;                  // blocks of a split in flight per loader wave
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescale = 8.0f;              // lazy-rescale threshold (log2 units)

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
  float* po;               // [8][n_split][128 d][128 q]
  float* pm;               // [8][n_split][128]
  float* pl;
  int S, Smax, n_split, kps;
  int q_norm, tail_norm;
};

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;

// Chunk swizzles (16-byte chunk index within a 256-byte row).
__device__ __forceinline__ int kswz(int r) { return r & 15; }
// V rows: the swizzle only depends on row & 3, so all transpose reads of a lane share two
// base addresses (t even / odd) plus immediate offsets, and still spread a 16-lane group
// over 8 distinct chunks.
__device__ __forceinline__ int vswz(int r) { return 2 * (r & 3); }

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

__device__ __forceinline__ void load_cos_sin(const float* cos_t, const float* sin_t, int tok, int j16, float* c,
                                             float* s) {
  const int f0 = 8 * (j16 & 7);
  const f32x4* cp = reinterpret_cast<const f32x4*>(cos_t + tok * 64 + f0);
  const f32x4* sp = reinterpret_cast<const f32x4*>(sin_t + tok * 64 + f0);
  const f32x4 c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    c[e] = c0[e]; c[4 + e] = c1[e]; s[e] = s0[e]; s[4 + e] = s1[e];
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

// The LDS tiles are distinct objects so that the compiler's wait counting can tell the
// direct-to-LDS loads of one block from another block and from the query buffer.
#define AX_TILE(b) __shared__ __attribute__((aligned(16))) uint8_t t##b[kTileBytes]
template <int B>
__device__ __forceinline__ uint8_t* pick(uint8_t* t0, uint8_t* t1, uint8_t* t2, uint8_t* t3, uint8_t* t4,
                                         uint8_t* t5, uint8_t* t6) {
  if constexpr (B == 0) return t0;
  else if constexpr (B == 1) return t1;
  else if constexpr (B == 2) return t2;
  else if constexpr (B == 3) return t3;
  else if constexpr (B == 4) return t4;
  else if constexpr (B == 5) return t5;
  else return t6;
}

// NORM: q and the own k arrive raw and are normed + roped here (the layer step); otherwise
// both arrive roped (attention only).
//
// Wave roles. Waves 4..7 only issue the direct-to-LDS cache loads and then mark each block
// ready (wait for their own loads, barrier). Waves 0..3 do everything else: the query
// norm/RoPE, the own-token rows, the attention and the partials. Keeping ordinary loads
// and LDS-DMA loads in different waves keeps each wave's vmcnt in order, so no wave ever
// has to drain its queue early.
template <int NB, bool NORM>
__global__ __launch_bounds__(kThreads, 1) void k_attn_fused(FusedArgs a) {
  AX_TILE(0); AX_TILE(1); AX_TILE(2); AX_TILE(3); AX_TILE(4); AX_TILE(5); AX_TILE(6);
  __shared__ __attribute__((aligned(16))) uint8_t qlds[kQBytes];
  // roped own-token K rows (row tok, chunks swizzled like the tile row they stand in for)
  __shared__ __attribute__((aligned(16))) uint8_t kown[kT * 256];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = blockIdx.x % kHkv;
  const int split = blockIdx.x / kHkv;
  const int n_keys = a.S + kT;
  const int k_begin = split * a.kps;
  const int k_end = min(k_begin + a.kps, n_keys);
  const long long head_off = (long long)g * a.Smax * kD;
  // blocks holding own-token rows that need the tail step (norm of k and/or cache tail write)
  const bool own_tail = a.own_tail != 0;

  if (wave >= 4) {
    // ---------------- loader waves: K row groups w and w+4, V row groups w and w+4 (4 rows each)
    const int w = wave - 4;
    lds_barrier();  // the compute waves have issued their query / table loads: they go first
    const uint16_t* kc = a.Kc + head_off;
    const uint16_t* vc = a.Vc + head_off;
    const uint16_t* kt = a.kt_base + g * a.tail_stride;
    const uint16_t* vt = a.vt_base + g * a.tail_stride;
    // DMA of block b: this wave's K row groups w, w+4 and V row groups w, w+4.
    auto issue_block = [&](auto bc) {
      constexpr int b = decltype(bc)::value;
      uint8_t* tile = pick<b>(t0, t1, t2, t3, t4, t5, t6);
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
        __builtin_amdgcn_global_load_lds(ks, (lds_void*)(tile + grp * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vs, (lds_void*)(tile + kTileBytes / 2 + grp * 1024), 16, 0, 0);
      });
    };
    // The CU's memory queue throttles issue, so only kDmaDepth blocks are kept in flight:
    // block b + kDmaDepth is issued right after block b is handed over, and the barriers
    // never wait for the issue of loads that are not needed yet.
    static_for<(NB < kDmaDepth ? NB : kDmaDepth)>([&](auto bc) { issue_block(bc); });
    lds_barrier();  // queries and own-token K rows written by the compute waves
    static_for<NB>([&](auto bc) {
      constexpr int b = decltype(bc)::value;
      constexpr int later = (b + kDmaDepth - 1 < NB - 1 ? b + kDmaDepth - 1 : NB - 1) - b;
      wait_vmcnt<4 * later>();  // loads are issued in block order: block b has landed
      lds_barrier();
      if constexpr (b + kDmaDepth < NB) issue_block(std::integral_constant<int, b + kDmaDepth>{});
    });
    return;
  }

  // ---------------- compute waves (256 threads)
  const int j16 = tid & 15;
  const int r16 = tid >> 4;  // 0..15
  // 1. Issue every load of the prologue, then release the loader waves (start barrier), so
  //    these small loads sit ahead of the cache stream in the CU's memory queue.
  //    Query pass p covers folded row 16p + r16 (q head 2g + row/64, token row % 64), so token
  //    16(p&3) + r16; own-token row tok = 16p + r16 (p < 4) uses the same cos/sin.
  u32x4 qraw[8], graw, gkraw, kraw[4], vraw[4];
  float qc[4][8], qs[4][8];
#pragma unroll
  for (int p = 0; p < 8; ++p)
    qraw[p] = *reinterpret_cast<const u32x4*>(a.q + ((long long)(2 * g) * kT + 16 * p + r16) * kD + 8 * j16);
  if constexpr (NORM) {
    graw = *reinterpret_cast<const u32x4*>(a.gq + 8 * j16);
#pragma unroll
    for (int p = 0; p < 4; ++p) load_cos_sin(a.cos_t, a.sin_t, 16 * p + r16, j16, qc[p], qs[p]);
  }
  const bool has_own = own_tail && k_end > a.S;  // this split holds own-token rows
  if (has_own) {
    const uint16_t* kt = a.kt_base + g * a.tail_stride;
    const uint16_t* vt = a.vt_base + g * a.tail_stride;
    if constexpr (NORM) gkraw = *reinterpret_cast<const u32x4*>(a.gk + 8 * j16);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int tok = 16 * p + r16;
      kraw[p] = *reinterpret_cast<const u32x4*>(kt + (long long)tok * kD + 8 * j16);
      vraw[p] = *reinterpret_cast<const u32x4*>(vt + (long long)tok * kD + 8 * j16);
    }
  }
  lds_barrier();  // start: loader waves begin the cache stream

  // 2. queries -> LDS (normed and roped unless given roped)
  {
    float qg[8];
    if constexpr (NORM) unpack8v(graw, qg);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int r = 16 * p + r16;
      u32x4 v = qraw[p];
      if constexpr (NORM) {
        float x[8];
        unpack8v(v, x);
        norm_rope_row16(x, qg, qc[p & 3], qs[p & 3], a.eps, j16);
        v = pack8v(x);
      }
      *reinterpret_cast<u32x4*>(qlds + r * 256 + 16 * (j16 ^ kswz(r))) = v;
    }
  }
  // 3. own-token rows of this split: K normed + roped (or taken roped) into kown and the cache
  //    tail, V copied to the cache tail
  if (has_own) {
    float gk[8];
    if constexpr (NORM) unpack8v(gkraw, gk);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int tok = 16 * p + r16;
      const int vk = a.S + tok;
      if (vk >= k_begin && vk < k_end) {
        u32x4 kv = kraw[p];
        if constexpr (NORM) {
          float x[8];
          unpack8v(kv, x);
          norm_rope_row16(x, gk, qc[p], qs[p], a.eps, j16);
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
  lds_barrier();  // queries and own-token K rows are in LDS

  const int n = lane & 31;
  const int h = lane >> 5;
  bf16x8 qf[8];
  {
    const int qrow = 32 * wave + n;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qf[kk] = *reinterpret_cast<const bf16x8*>(qlds + qrow * 256 + 16 * ((dcol(kk, h) >> 3) ^ kswz(qrow)));
  }

  f32x16 o[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;  // running max in log2 units of the scaled score, row sum
  const float sc = kLog2e * 0.08838834764831845f;  // log2(e) / sqrt(128)
  const int krow = perm_key(n);

  // S^T = K Q^T of block b: K fragments from LDS (own-token rows from kown), then 8 MFMAs.
  auto issue_qk = [&](auto bc) -> f32x16 {
    constexpr int b = decltype(bc)::value;
    const int kb = k_begin + b * kBlk;
    const uint8_t* tk = pick<b>(t0, t1, t2, t3, t4, t5, t6);
    const int kvk = kb + krow;
    const uint8_t* krow_base = (own_tail && kvk >= a.S) ? kown + (kvk - a.S) * 256 : tk + krow * 256;
    bf16x8 kf[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      kf[kk] = *reinterpret_cast<const bf16x8*>(krow_base + 16 * ((dcol(kk, h) >> 3) ^ kswz(krow)));
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[kk], s, 0, 0, 0);
    return s;
  };

  // Software pipeline over the blocks: while the matrix cores run block b+1's S^T, the wave
  // does block b's softmax; then block b's PV. Blocks past the split end (only in a short
  // last split) are fully masked: they add nothing, and block 0 always holds at least one
  // key, so m_run is finite from block 0 on.
  lds_barrier();  // block 0 is in LDS
  f32x16 s_cur = issue_qk(std::integral_constant<int, 0>{});
  static_for<NB>([&](auto bc) {
    constexpr int b = decltype(bc)::value;
    const int kb = k_begin + b * kBlk;
    const uint8_t* tv = pick<b>(t0, t1, t2, t3, t4, t5, t6) + kTileBytes / 2;
    // V^T operands of block b: lane group G = lane >> 4, i = lane & 15 points at row
    // 16c + 8(G>>1) + 4*half + i/4, columns 32t + 16(G&1) + 4(i&3) .. +3; the transpose
    // read hands lane i of the group column 32t + 16(G&1) + i of 4 consecutive rows.
    v4i16 vt[2][4][2];
    {
      const int G = lane >> 4, i = lane & 15;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const int row = 16 * c + 8 * (G >> 1) + 4 * hf + (i >> 2);
            const int chunk = 4 * t + 2 * (G & 1) + ((i & 3) >> 1);
            vt[c][t][hf] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4i16*)(tv + row * 256 + 16 * (chunk ^ vswz(row)) + 8 * (i & 1)));
          }
    }
    f32x16 s_next;
    if constexpr (b + 1 < NB) {
      lds_barrier();  // block b+1 is in LDS
      s_next = issue_qk(std::integral_constant<int, b + 1>{});
    }
    __builtin_amdgcn_sched_barrier(0);

    f32x16 s = s_cur;
    if (__builtin_expect(kb + kBlk > k_end, 0)) {  // only a split's last block can be partial
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
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
    // The exponent reference m_run only moves when some row's max exceeds it by more than
    // kRescale (log2 units): p stays below 2^kRescale, exact for the final normalisation,
    // and the O rescale (64 multiplies) runs only on such jumps (always on block 0).
    const float m_blk = bmax * sc;
    if (__any(m_blk > m_run + kRescale)) {
      const float m_new = fmaxf(m_run, m_blk);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on block 0
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
    bf16x8 pb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) pb[c][j] = (__bf16)s[8 * c + j];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const v4i16 both[2] = {vt[c][t][0], vt[c][t][1]};
        bf16x8 vf;
        __builtin_memcpy(&vf, both, 16);
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[c], o[t], 0, 0, 0);
      }
    if constexpr (b + 1 < NB) s_cur = s_next;
  });

  const int qrow = 32 * wave + n;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const long long part = (long long)g * a.n_split + split;
  // Partial O in the accumulator layout, lane-major: slot j = 4t + jj holds, for query row
  // 32*wave + n, the 4 columns 32t + 8jj + 4h .. +3 (accumulator elements 4jj .. 4jj+3 of
  // tile t); one store instruction writes 1 KB contiguously.
  f32x4* po = reinterpret_cast<f32x4*>(a.po) + (part * 4 + wave) * (16 * 64) + lane;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const f32x4 v = {o[t][4 * jj], o[t][4 * jj + 1], o[t][4 * jj + 2], o[t][4 * jj + 3]};
      po[(4 * t + jj) * 64] = v;
    }
  if (h == 0) {
    a.pm[part * kQRows + qrow] = m_run;
    a.pl[part * kQRows + qrow] = l_tot;
  }
}

// Combine. Thread -> (head g, query row q, 4 columns d0..d0+3); it reads one float4 of each
// split's partial (slot and lane of the accumulator layout above), then
// out = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c.
// Grid: 8 heads x 16 blocks of 256 threads; block: 32 rows x 8 column quads.
__global__ __launch_bounds__(256) void k_attn_combine(const float* po, const float* pm, const float* pl,
                                                      uint16_t* out, int n_split) {
  const int g = blockIdx.x % kHkv;
  const int rest = blockIdx.x / kHkv;   // 0..15
  const int wave = rest & 3;            // query rows 32*wave .. +31
  const int quad0 = (rest >> 2) * 8;    // column quads quad0 .. quad0+7 of 32
  const int n = threadIdx.x & 31;
  const int quad = quad0 + (threadIdx.x >> 5);
  const int q = 32 * wave + n;
  const int d0 = 4 * quad;              // = 32t + 8jj + 4h
  const int t = d0 >> 5, jj = (d0 >> 3) & 3, h = (d0 >> 2) & 1;
  const int slot = 4 * t + jj, lane = n + 32 * h;
  const float* pmg = pm + (long long)g * n_split * kQRows + q;
  const float* plg = pl + (long long)g * n_split * kQRows + q;
  const f32x4* pog = reinterpret_cast<const f32x4*>(po) + ((long long)g * n_split * 4 + wave) * (16 * 64) +
                     slot * 64 + lane;
  const long long pstride = 4 * 16 * 64;  // float4s per split partial
  float M = -INFINITY;
#pragma unroll 8
  for (int c = 0; c < n_split; ++c) M = fmaxf(M, pmg[(long long)c * kQRows]);
  float L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int c = 0; c < n_split; ++c) {
    const float w = __builtin_amdgcn_exp2f(pmg[(long long)c * kQRows] - M);
    L += w * plg[(long long)c * kQRows];
    const f32x4 v = pog[(long long)c * pstride];
    acc[0] += w * v[0]; acc[1] += w * v[1]; acc[2] += w * v[2]; acc[3] += w * v[3];
  }
  const float inv = 1.0f / L;
  uint2 r;
  r.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  r.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<uint2*>(out + ((long long)g * kQRows + q) * kD + d0) = r;
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
static hipError_t launch_nb(const FusedArgs& a, hipStream_t st) {
  if (a.q_norm)
    hipLaunchKernelGGL((k_attn_fused<NB, true>), dim3(kHkv * a.n_split), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((k_attn_fused<NB, false>), dim3(kHkv * a.n_split), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn(const AttnPlan& plan, const AttnLaunch& p, hipStream_t st) {
  FusedArgs a;
  const size_t parts = (size_t)kHkv * plan.n_split;
  char* ws = static_cast<char*>(p.ws);
  a.q = p.q; a.gq = p.gq; a.gk = p.gk; a.cos_t = p.cos_t; a.sin_t = p.sin_t; a.eps = p.eps;
  a.own_tail = p.k_tail != nullptr;
  if (a.own_tail) {
    a.kt_base = p.k_tail; a.vt_base = p.v_tail; a.tail_stride = (long long)kT * kD;
  } else {
    a.kt_base = p.Kc + (long long)(p.Smax - kT) * kD; a.vt_base = p.Vc + (long long)(p.Smax - kT) * kD;
    a.tail_stride = (long long)p.Smax * kD;
  }
  a.Kc = p.Kc; a.Vc = p.Vc;
  a.po = reinterpret_cast<float*>(ws);
  a.pm = reinterpret_cast<float*>(ws + align256(parts * kD * kQRows * 4));
  a.pl = reinterpret_cast<float*>(ws + align256(parts * kD * kQRows * 4) + align256(parts * kQRows * 4));
  a.S = p.S; a.Smax = p.Smax; a.n_split = plan.n_split; a.kps = plan.keys_per_split;
  a.q_norm = p.q_norm; a.tail_norm = p.tail_norm;
  hipError_t e;
  switch (plan.blocks) {
    case 1: e = launch_nb<1>(a, st); break;
    case 2: e = launch_nb<2>(a, st); break;
    case 3: e = launch_nb<3>(a, st); break;
    case 4: e = launch_nb<4>(a, st); break;
    case 5: e = launch_nb<5>(a, st); break;
    case 6: e = launch_nb<6>(a, st); break;
    default: e = launch_nb<7>(a, st); break;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_attn_combine, dim3(kHkv * 16), dim3(256), 0, st, a.po, a.pm, a.pl, p.out, plan.n_split);
  return hipGetLastError();
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
