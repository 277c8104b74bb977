// Split-KV attention of the folded query rows of each kv head over the visible cache rows
// (with the q/k RMSNorm + RoPE and the own-K/V tail write folded in), and the log-sum-exp
// combine of the splits.
//
// What is computed: page code/alpamayo_tt/expert.py, TTExpert.layer from the q/k norms to
// attention_core in decode mode - per kv head g ("user" g) the 2 q heads x 64 tokens form 128
// query rows that attend, non-causally and with scale 1/sqrt(128), to cache rows [0, S) and
// [Smax-64, Smax); the additive mask of TTExpert.build_mask hides the rest. The pages' kernel
// splits each head's key sequence over cores and reduces the parts (EXPERT_NOTES.md, "masking
// approach"); the per-split quantities and the combine are the flash-decode ones:
//   m_c = max_j s_j, l_c = sum_j 2^(s_j - m_c), O_c = sum_j 2^(s_j - m_c) v_j
//   out = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c,  M = max_c m_c
// with s_j = log2(e) * (q . k_j) / sqrt(128) (base-2 exponentials of scaled scores give the same
// softmax), and m_c any reference at or near the split's maximum.
//
// gfx950 mapping (k_attn_split)
// - One workgroup of 12 waves per (kv head g, key range, q head 2g + hp): 64 query rows. Workgroup
//   id w has head w % 8, which the dispatcher places on XCD w % 8, and the two q heads of a key
//   range are consecutive ids, so the second read of the range's K/V comes from that XCD's L2.
//   The cache keys [0, S) are cut into at most 15 ranges of whole 32-key blocks (at most 10
//   blocks each); the 64 own tokens form one more range of 2 blocks.
// - Waves 0..3 (loaders, one per SIMD) issue direct-to-LDS loads (global_load_lds, 16 bytes per
//   lane): first the query prologue (16 query rows, their RoPE rows and the gammas for the row
//   tile on the same SIMD), then the blocks a few ahead into a ring of 6 tiles, and count each
//   landed block in LDS. A wave whose loads wait for room in the CU's memory pipeline stalls at
//   issue, so the loads are kept away from the arithmetic.
// - Waves 4..11 (compute): wave 4 + w takes row tile t = w & 3 (rows 16 t .. 16 t + 15) over the
//   blocks of parity p = w >> 2, so each SIMD runs one loader and the two compute
//   waves of one row tile: a single wave issues vector instructions at only a fraction of a SIMD's
//   rate, and the per-block exponentials are the larger part of the work. Per block S^T = K Q^T on
//   v_mfma_f32_16x16x32_bf16 (A = K rows, B = Q^T) and O^T += V^T P^T with V^T read by
//   ds_read_b64_tr_b16 and P^T taken straight from the S^T accumulators. The blocks are
//   software-pipelined: the scores of block b run on the matrix cores while the exponentials of
//   the previous block run on the vector ALU, and the PV of the previous block beside the row
//   max of block b.
// - fp8 cache: K stays in e4m3 codes and S^T comes from v_mfma_f32_16x16x128_f8f6f4, with each
//   query row scaled by a power of two and split into two e4m3 parts whose sum is the scaled bf16
//   row exactly for every element down to 2^-10 of the row's largest (below, within 2^-17 of
//   it); the loaders convert only V to bf16. Key scales multiply S, value scales P.
// - The three waves of a SIMD norm and rope their row tile's 16 query rows in LDS first.
// - The two parity waves of a row tile merge (m, l, O) through LDS, each finalising half of the
//   columns, and store the range's partial: O in float16 with a power-of-two exponent per (row,
//   32-column quarter), m and l in float32.
// - Every hand-off is an LDS counter; every wait on one is bounded, and a wave whose wait runs out
//   marks its rows' partial NaN, so that a miscounted hand-off shows in the output.
#include "ax_attn_common.h"
#include "ax_launch.h"

namespace ax {

constexpr int kSRT = 4;                         // row tiles of 16 query rows (one per SIMD)
constexpr int kSC = 8;                          // compute waves: 4 row tiles x 2 block parities
constexpr int kSL = 4;                          // loader waves
constexpr int kSThreads = 64 * (kSC + kSL);
constexpr int kSTile = 2 * kBlk * kD * 2;       // 16 KB: the K rows, then the V rows of a 32-key block
constexpr int kSV = kBlk * kD * 2;              // offset of the V rows in a tile
constexpr int kSRing = 6;                       // tiles; block b uses tile b % kSRing (bf16 cache)
constexpr int kSMaxNB = 10;                     // blocks per key range (bf16 cache)
// fp8 cache: the ring's first 32 KB are four V tiles of the bf16 values the loaders convert (block
// b in V tile b % 4: 32 rows of 256 bytes, the bf16 tiles' V layout), the rest eight raw tiles of
// codes (block b in raw tile b % 8: 32 rows of 128 bytes for K, chunk-swizzled, which the matrix
// cores read as codes, then 32 rows for V). In the own range, blocks 0 and 1 arrive as bf16 rows
// in two bf16 tiles at kSStage8 (raw tiles 2..5, unused there) and are quantised from there.
constexpr int kSRing8 = 4;                      // V tiles
constexpr int kSVTile8 = kBlk * kD * 2;
constexpr int kSRaw8 = 8;                       // raw tiles
constexpr int kSRawTile = 2 * kBlk * kD;
constexpr int kSRawBase = kSRing8 * kSVTile8;
constexpr int kSStage8 = kSRawBase + 2 * kSRawTile;
static_assert(kSRawBase + kSRaw8 * kSRawTile <= kSRing * kSTile, "fp8 rings inside the bf16 ring");
static_assert(kSStage8 + 2 * kSTile <= kSRawBase + kSRaw8 * kSRawTile, "own-range staging inside the raw tiles");
constexpr int kSDoneN = kSRaw8 > kSRing ? kSRaw8 : kSRing;  // tile-use counters
constexpr int kSMaxNB8 = 17;                    // blocks per key range (fp8 cache)
constexpr int kSDepth = 3;                      // blocks in flight per loader wave
constexpr int kSCacheRanges = 15;               // cache key ranges per kv head, at most
constexpr float kSRescale = 16.0f;              // lazy-rescale threshold (log2 units)
constexpr float kScoreScale = kLog2e * 0.08838834764831845f;  // log2(e) / sqrt(128)
// LDS hand-off counters: prologue of row tile t landed, query rows normed, query fragments read,
// block b landed, uses of tile r finished, merge data of row tile t written
constexpr int kCPro = 0, kCNorm = 4, kCFrag = 5, kCLand = 6, kCDone = kCLand + kSMaxNB8, kCMrg = kCDone + kSDoneN,
              kCN = kCMrg + 4;

struct SplitArgs {
  const uint16_t* q;       // [16][64][128]: raw q (NORM) or already roped q
  const uint16_t* gq;
  const uint16_t* gk;
  const float* cos_t;      // [64][64]
  const float* sin_t;
  float eps;
  // Own-token rows of head g at kt_base + g * tail_stride (row-major, 128 per row): the own k/v
  // tensors (raw k if NORM) or, when own_tail is 0, the cache tail itself.
  const uint16_t* kt_base;
  const uint16_t* vt_base;
  long long tail_stride;
  int own_tail;            // own rows come from k/v tensors; q head parity 0 writes them to the cache tail
  uint16_t* Kc;
  uint16_t* Vc;
  // fp8 cache (F8): codes [8][Smax][128] e4m3 and float32 row scales [8][Smax]; own rows, when
  // given, are quantised here into the cache tail (kt_base / vt_base are then the own k / v)
  uint8_t* Kc8;
  uint8_t* Vc8;
  float* Ks;
  float* Vs;
  WsLayout part;            // the status word and the partials
  int spin_limit;           // polls before a wait gives up
  int S, Smax, n_split, kps;
  int n_cache_split;       // ranges over cache keys [0, S); range n_cache_split holds the 64 own tokens
};

// LDS-typed pointers: kept in the LDS address space end to end.
typedef __attribute__((address_space(3))) uint8_t lds_u8;
// (as 32-bit vectors of the same size: HIP's uint2 class cannot be copied out of another address space)
template <typename T>
__device__ __forceinline__ T lds_ld(const lds_u8* p) {
  typedef uint32_t N __attribute__((ext_vector_type(sizeof(T) / 4)));
  return __builtin_bit_cast(T, *reinterpret_cast<const __attribute__((address_space(3))) N*>(p));
}
template <>
__device__ __forceinline__ float lds_ld<float>(const lds_u8* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) float*>(p);
}
template <typename T>
__device__ __forceinline__ void lds_st(lds_u8* p, const T& v) {
  typedef uint32_t N __attribute__((ext_vector_type(sizeof(T) / 4)));
  *reinterpret_cast<__attribute__((address_space(3))) N*>(p) = __builtin_bit_cast(N, v);
}
template <>
__device__ __forceinline__ void lds_st<float>(lds_u8* p, const float& v) {
  *reinterpret_cast<__attribute__((address_space(3))) float*>(p) = v;
}
#define AX_LDS(x) ((lds_u8*)(x))

// Direct-to-LDS loads and the waits for them, written as inline asm. The compiler does not tell
// one LDS object from another for its own direct-to-LDS loads and drains every load in flight
// (vmcnt(0)) before any LDS access that follows one (a loader's counter update included).
// Written here, the loads are invisible to its wait counting and each wave waits, in order, for
// exactly the loads it needs: vm_wait<N>() returns once at most N of this wave's loads are
// outstanding (loads complete in issue order). The "memory" clobbers keep every LDS access on its
// side of the loads and waits. These instructions have no destination registers (the data goes
// to LDS at the M0 base + 16 bytes x lane, or 4 for dma_x1).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is reserved: nothing else in these kernels keeps a value in it
__device__ __forceinline__ void dma_x4(const void* src, const lds_u8* dst) {
  const uint32_t base = (uint32_t)(uintptr_t)dst;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(base) : "memory", "m0");
}
__device__ __forceinline__ void dma_x1(const void* src, const lds_u8* dst) {
  const uint32_t base = (uint32_t)(uintptr_t)dst;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(base) : "memory", "m0");
}
#pragma clang diagnostic pop
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// The split kernel's LDS: the ring of block tiles; the 64 query rows; the RoPE rows (cos, sin) of
// the 64 tokens, which later take the merge's exchange; the gammas; the counters.
__shared__ __attribute__((aligned(16))) uint8_t sRing[kSRing * kSTile];
__shared__ __attribute__((aligned(16))) uint8_t sQ[kT * 256];
__shared__ __attribute__((aligned(16))) uint8_t sRope[2 * kT * 256];
__shared__ __attribute__((aligned(16))) uint8_t sGam[2 * 256];
__shared__ int sCnt[kCN];
// fp8 cache: the row scales of block b, 16 per loader share L: K scales of rows 8 L .. 8 L + 7 at
// [16 L .. 16 L + 7], V scales at [16 L + 8 .. 16 L + 15] (never reused within a launch)
__shared__ __attribute__((aligned(16))) float sScl8[kSMaxNB8][64];

// Bounded waits on the counters: a wave whose wait runs out (by default about 30 ms; thousands of
// times any real wait) carries on and remembers it; its partial is then marked NaN and the
// workspace status word flagged.
// The loop stays rolled: every wave of the workgroup shares one short copy of it in the
// instruction cache.
__device__ __forceinline__ void await_cnt(int i, int n, int limit, bool& expired) {
  __builtin_amdgcn_sched_barrier(0);
  int spin = limit;
#pragma clang loop unroll(disable)
  while (__builtin_amdgcn_readfirstlane(__hip_atomic_load(&sCnt[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) < n) {
    if (--spin <= 0) {
      expired = true;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Per-workgroup facts every wave shares.
struct SplitCtx {
  int g, hp, split, k_begin, k_end, nb, lane;
  bool own;                // the range of the 64 own tokens
  bool pre;                // its blocks are filled in the prologue (own rows given, or the bf16 tail)
  bool partial;            // the last block of the range has keys past k_end
};

// A loader's share of cache block b (keys k_begin + 32 b + r): K and V rows 8 L .. 8 L + 7 (two
// loads of 4 rows each), 16 bytes per lane, chunks swizzled per row. Rows past k_end reload the
// range's first key, a visible key; their scores are masked before the exponentials.
__device__ __forceinline__ void dma_block_share(const uint16_t* kc, const uint16_t* vc, const SplitCtx& c, int L,
                                                int b, lds_u8* tile) {
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int r0 = 8 * L + 4 * h2;
    const int r = r0 + (c.lane >> 4);
    int v = c.k_begin + kBlk * b + r;
    v = v < c.k_end ? v : c.k_begin;
    dma_x4(kc + (long long)v * kD + 8 * ((c.lane & 15) ^ kswz16(r)), tile + r0 * 256);
    dma_x4(vc + (long long)v * kD + 8 * ((c.lane & 15) ^ vswz16(r)), tile + kSV + r0 * 256);
  }
}

// fp8 cache: a loader's share of block b (keys k_begin + 32 b + r, rows r = 8 L .. 8 L + 7) into
// raw tile b % 4: one 1 KB load for the K codes, one for the V codes, row-major 128 bytes a row,
// and (lanes 0..15) the rows' K and V scales into the block's scale record. Keys past the tail
// start are the cache tail's rows; rows past k_end reload the range's first key.
__device__ __forceinline__ long long cache_row8(const SplitArgs& a, const SplitCtx& c, int v) {
  v = v < c.k_end ? v : c.k_begin;
  return (long long)c.g * a.Smax + (v < a.S ? v : a.Smax - kT + (v - a.S));
}
// K codes: chunk c (16 bytes) of row r at c ^ kswz8(r), so that the 16 rows a 16-lane group reads
// at one chunk hit all 64 banks once (rows 128 bytes apart share banks two rows apart).
__device__ __forceinline__ int kswz8(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ void dma_block_f8(const SplitArgs& a, const SplitCtx& c, int L, int b) {
  lds_u8* raw = AX_LDS(sRing) + kSRawBase + (b % kSRaw8) * kSRawTile;
  const int r = 8 * L + (c.lane >> 3);
  const long long row = cache_row8(a, c, c.k_begin + kBlk * b + r);
  dma_x4(a.Kc8 + row * kD + 16 * ((c.lane & 7) ^ kswz8(r)), raw + 8 * L * kD);
  dma_x4(a.Vc8 + row * kD + 16 * (c.lane & 7), raw + kBlk * kD + 8 * L * kD);
  if (c.lane < 16) {
    const long long srow = cache_row8(a, c, c.k_begin + kBlk * b + 8 * L + (c.lane & 7));
    dma_x1((c.lane < 8 ? a.Ks : a.Vs) + srow, AX_LDS(sScl8) + b * 256 + 64 * L);
  }
}
// ... and, once landed, the V rows converted exactly (every e4m3 value is a bf16 value) into the
// block's V tile b % 4 with the bf16 tiles' V swizzle: code chunk c8 of a row (16 bytes) is bf16
// chunks 2 c8 and 2 c8 + 1. (K stays in codes.) The scales are applied in float32 by the compute
// waves. (Scaling V here instead, rounded to bf16, made the launch 4% slower: the loaders share the
// SIMDs with the compute waves.)
__device__ __forceinline__ void convert_block_f8(const SplitCtx& c, int L, int b) {
  const lds_u8* raw = AX_LDS(sRing) + kSRawBase + (b % kSRaw8) * kSRawTile;
  lds_u8* vt = AX_LDS(sRing) + (b % kSRing8) * kSVTile8;
  const int r = 8 * L + (c.lane >> 3), c8 = c.lane & 7;
  const u32x4 vw = lds_ld<u32x4>(raw + kBlk * kD + r * kD + 16 * c8);
  lds_st(vt + r * 256 + 16 * ((2 * c8) ^ vswz16(r)), e4m3x8_to_bf16(vw[0], vw[1]));
  lds_st(vt + r * 256 + 16 * ((2 * c8 + 1) ^ vswz16(r)), e4m3x8_to_bf16(vw[2], vw[3]));
}

__device__ __forceinline__ float fmax_(float a, float b) { return __builtin_elementwise_maximum(a, b); }
// A lane's value and that of lane ^ 16, in either order (v_permlane16_swap, as pair32 for 32).
__device__ __forceinline__ float2 pair16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return float2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
// The lane's largest score of a block (its 8 keys), and the max over the four lanes l & 15 + 16 i
// that hold one query row. The IEEE maximum (v_maximum3_f32 on gfx950) needs no quieting of its
// inputs, unlike fmaxf on MFMA results.
__device__ __forceinline__ float lane_max8(const f32x4* s) {
  return fmax_(fmax_(fmax_(s[0][0], s[0][1]), fmax_(s[0][2], s[0][3])),
               fmax_(fmax_(s[1][0], s[1][1]), fmax_(s[1][2], s[1][3])));
}
__device__ __forceinline__ float row_max4(float x) {
  float2 p = pair16(x);
  x = fmax_(p.x, p.y);
  p = pair32(x);
  return fmax_(p.x, p.y);
}

// The bf16 tile holding own block blk (tokens 32 blk .. 32 blk + 31) in the own range: the ring's
// tiles 0, 1, or with the fp8 cache the staging tiles the quantisation reads.
template <bool F8>
__device__ __forceinline__ lds_u8* own_tile(int blk) {
  return AX_LDS(sRing) + (F8 ? kSStage8 : 0) + blk * kSTile;
}

// Norm + RoPE in place of query rows row0 .. row0 + 4 NP - 1 (NP passes of 4 rows, 16 lanes per
// row: the arithmetic of the stand-alone norm/RoPE kernel, so the bits are the same) and, in the
// own range, of the own k rows of the same tokens (same RoPE rows, gamma k). The 16 rows of a row
// tile are split between the three waves of its SIMD (4 + 4 + 8), since a single wave issues
// vector instructions at only half of a SIMD's rate. Within a pass every LDS read comes first,
// then the arithmetic, then the stores, so that the rows' dependency chains interleave.
template <int NP, bool F8>
__device__ __forceinline__ void norm_rows(const SplitArgs& a, const SplitCtx& c, const int row0) {
  const int lane = c.lane, j16 = lane & 15, r4 = lane >> 4;
  float g8[8];
  unpack_pair(lds_ld<uint2>(AX_LDS(sGam) + 8 * j16), lds_ld<uint2>(AX_LDS(sGam) + 128 + 8 * j16), g8);
  uint2 lo[NP], hi[NP];
  float cc[NP][4], ss[NP][4];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int r = row0 + 4 * i + r4;  // query row = token
    lo[i] = lds_ld<uint2>(AX_LDS(sQ) + r * 256 + pair_off_lo(j16, qswz(r)));
    hi[i] = lds_ld<uint2>(AX_LDS(sQ) + r * 256 + pair_off_hi(j16, qswz(r)));
    const f32x4 cs = lds_ld<f32x4>(AX_LDS(sRope) + (row0 + 4 * i) * 256 + 16 * lane);
    const f32x4 sn = lds_ld<f32x4>(AX_LDS(sRope) + kT * 256 + (row0 + 4 * i) * 256 + 16 * lane);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      cc[i][e] = cs[e];
      ss[i][e] = sn[e];
    }
  }
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    float x[8], A[8], B[8];
    unpack_pair(lo[i], hi[i], x);
    rope_coef_pair(g8, cc[i], ss[i], A, B);
    norm_rope_pair(x, A, B, a.eps);
    pack_pair(x, lo[i], hi[i]);
  }
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int r = row0 + 4 * i + r4;
    lds_st(AX_LDS(sQ) + r * 256 + pair_off_lo(j16, qswz(r)), lo[i]);
    lds_st(AX_LDS(sQ) + r * 256 + pair_off_hi(j16, qswz(r)), hi[i]);
  }
  if (c.own) {
    float gk8[8];
    unpack_pair(lds_ld<uint2>(AX_LDS(sGam) + 256 + 8 * j16), lds_ld<uint2>(AX_LDS(sGam) + 384 + 8 * j16), gk8);
    uint2 klo[NP], khi[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int tr = (row0 + 4 * i + r4) & (kBlk - 1);
      const lds_u8* krow = own_tile<F8>((row0 + 4 * i) >> 5) + tr * 256;
      klo[i] = lds_ld<uint2>(krow + pair_off_lo(j16, kswz16(tr)));
      khi[i] = lds_ld<uint2>(krow + pair_off_hi(j16, kswz16(tr)));
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      float y[8], kA[8], kB[8];
      rope_coef_pair(gk8, cc[i], ss[i], kA, kB);
      unpack_pair(klo[i], khi[i], y);
      norm_rope_pair(y, kA, kB, a.eps);
      pack_pair(y, klo[i], khi[i]);
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int tr = (row0 + 4 * i + r4) & (kBlk - 1);
      lds_u8* krow = own_tile<F8>((row0 + 4 * i) >> 5) + tr * 256;
      lds_st(krow + pair_off_lo(j16, kswz16(tr)), klo[i]);
      lds_st(krow + pair_off_hi(j16, kswz16(tr)), khi[i]);
    }
  }
}

// fp8 cache, own range: the own k rows (normed and roped, or given roped) and the own v rows of
// tokens row0 .. row0 + 4 NP - 1, from the staging tiles, quantised per row (16 lanes per row:
// quant_row16, the definition of the cache format): the K codes into raw tile blk, the V codes'
// values in bf16 into V tile blk and the row scales into the block's scale record, as for a block
// the loaders bring; the codes and scales go to the cache tail here (q head parity 0), while they
// are at hand.
template <int NP>
__device__ __forceinline__ void quant_own_rows(const SplitArgs& a, const SplitCtx& c, const int row0) {
  const int j16 = c.lane & 15, r4 = c.lane >> 4;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int tok = row0 + 4 * i + r4;
    const int tr = tok & (kBlk - 1), blk = tok >> 5;
    const lds_u8* st = own_tile<true>(blk);
    float x[8], y[8], sk, sv;
    unpack8v(lds_ld<u32x4>(st + tr * 256 + 16 * (j16 ^ kswz16(tr))), x);
    unpack8v(lds_ld<u32x4>(st + kSV + tr * 256 + 16 * (j16 ^ vswz16(tr))), y);
    const uint2 ck = quant_row16(x, sk);
    const uint2 cv = quant_row16(y, sv);
    // lane j16's 8 codes are half j16 & 1 of code chunk j16 >> 1
    lds_st(AX_LDS(sRing) + kSRawBase + blk * kSRawTile + tr * kD + 16 * ((j16 >> 1) ^ kswz8(tr)) + 8 * (j16 & 1), ck);
    lds_st(AX_LDS(sRing) + blk * kSVTile8 + tr * 256 + 16 * (j16 ^ vswz16(tr)), e4m3x8_to_bf16(cv.x, cv.y));
    if (j16 == 0) {
      sScl8[blk][16 * (tr >> 3) + (tr & 7)] = sk;
      sScl8[blk][16 * (tr >> 3) + 8 + (tr & 7)] = sv;
    }
    if (c.hp == 0) {
      const long long crow = (long long)c.g * a.Smax + a.Smax - kT + tok;
      __builtin_nontemporal_store(u32x2{ck.x, ck.y}, reinterpret_cast<u32x2*>(a.Kc8 + crow * kD + 8 * j16));
      __builtin_nontemporal_store(u32x2{cv.x, cv.y}, reinterpret_cast<u32x2*>(a.Vc8 + crow * kD + 8 * j16));
      if (j16 == 0) {
        a.Ks[crow] = sk;
        a.Vs[crow] = sv;
      }
    }
  }
}

// ---------------------------------------------------------------------------------- loaders
template <bool NORM, bool F8>
__device__ __forceinline__ void split_loader(const SplitArgs& a, const SplitCtx& c, int L) {
  const int lane = c.lane, j16 = lane & 15, r4 = lane >> 4;
  const long long head_off = (long long)c.g * a.Smax * kD;
  const uint16_t* kc = F8 ? nullptr : a.Kc + head_off;
  const uint16_t* vc = F8 ? nullptr : a.Vc + head_off;
  lds_u8* ring = AX_LDS(sRing);
  // 1. the prologue of row tile L (the two compute waves on this SIMD): query rows 16 L + 4 i + r4
  //    (lane l lands at 16 l of each 1 KB, so it fetches the chunk the row's swizzle puts there),
  //    their RoPE rows, the gammas;
  //    in the own range also own k/v rows 16 L .. 16 L + 15 (blocks 0, 1 in tiles 0, 1; with the
  //    fp8 cache only when the own rows are given, else that range is streamed like any other)
  const uint16_t* qh = a.q + (long long)(2 * c.g + c.hp) * kT * kD;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * L + 4 * i + r4;
    dma_x4(qh + (long long)r * kD + 8 * (j16 ^ qswz(r)), AX_LDS(sQ) + (16 * L + 4 * i) * 256);
  }
  if constexpr (NORM) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = 16 * L + 4 * i + r4;
      dma_x4(a.cos_t + tok * 64 + 4 * j16, AX_LDS(sRope) + (16 * L + 4 * i) * 256);
      dma_x4(a.sin_t + tok * 64 + 4 * j16, AX_LDS(sRope) + kT * 256 + (16 * L + 4 * i) * 256);
    }
    // every loader brings both gamma vectors (the same bytes), so that row tile L's compute
    // waves need no other loader's count
    dma_x1(a.gq + 2 * lane, AX_LDS(sGam));
    dma_x1(a.gk + 2 * lane, AX_LDS(sGam) + 256);
  }
  if (c.pre) {
    const uint16_t* kt = a.kt_base + c.g * a.tail_stride;
    const uint16_t* vt = a.vt_base + c.g * a.tail_stride;
    lds_u8* ot = own_tile<F8>(L >> 1);  // tokens 0..31 in own tile 0, 32..63 in own tile 1
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tr0 = 16 * (L & 1) + 4 * i;
      const int tr = tr0 + r4;
      const int tok = 16 * L + 4 * i + r4;
      dma_x4(kt + (long long)tok * kD + 8 * (j16 ^ kswz16(tr)), ot + tr0 * 256);
      dma_x4(vt + (long long)tok * kD + 8 * (j16 ^ vswz16(tr)), ot + kSV + tr0 * 256);
    }
  }
  lds_barrier();  // counters cleared (the workgroup's only barrier)
  bool expired = false;
  if (c.pre) {
    vm_wait<0>();
    arrive(&sCnt[kCPro + L], lane);
    if constexpr (NORM) norm_rows<2, F8>(a, c, 16 * L + 8);
    if constexpr (F8) quant_own_rows<2>(a, c, 16 * L + 8);
    if constexpr (NORM || F8) arrive(&sCnt[kCNorm], lane);
    return;
  }
  // 2. blocks: kSDepth in flight. bf16: block b goes to tile b % kSRing once all four uses of the
  //    tile's previous block (one per row tile) are finished; 4 loads of this wave. fp8: block b
  //    goes to raw tile b % 8 once the four uses of block b - 8 are finished, 3 loads; once
  //    landed, and once V tile b % 4 is free, this wave converts its V rows into it.
  constexpr int LPB = F8 ? 3 : 4;  // loads per block
  const int nb = c.nb;
  auto issue = [&](int b) {
    if constexpr (F8) {
      // raw tile b % 8: all four uses of its previous block (K codes read by the matrix cores) done
      if (b >= kSRaw8) await_cnt(kCDone + b % kSRaw8, kSRT * (b / kSRaw8), a.spin_limit, expired);
      dma_block_f8(a, c, L, b);
    } else {
      if (b >= kSRing) await_cnt(kCDone + b % kSRing, kSRT * (b / kSRing), a.spin_limit, expired);
      dma_block_share(kc, vc, c, L, b, ring + (b % kSRing) * kSTile);
    }
  };
  const int d0 = nb < kSDepth ? nb : kSDepth;
  // blocks 0 and 1, then the prologue's hand-off (it was issued first: it has landed once at most
  // their loads are outstanding), this wave's share of the norm, then the next block: issuing
  // loads takes the wave long enough that announcing the prologue after all of them would hold
  // up the norm
  issue(0);
  if (d0 > 1) {
    issue(1);
    vm_wait<2 * LPB>();
  } else {
    vm_wait<LPB>();
  }
  arrive(&sCnt[kCPro + L], lane);
  if constexpr (NORM) {
    norm_rows<2, F8>(a, c, 16 * L + 8);
    arrive(&sCnt[kCNorm], lane);
  }
  for (int b = 2; b < d0; ++b) issue(b);
  for (int b = 0; b < nb; ++b) {
    const int later = (b + kSDepth - 1 < nb ? b + kSDepth - 1 : nb - 1) - b;  // blocks issued after b
    if (later >= 2) vm_wait<2 * LPB>(); else if (later == 1) vm_wait<LPB>(); else vm_wait<0>();
    if constexpr (F8) {
      // V tile b % 4: all four uses of block b - 4 done (its uses count at kCDone + (b - 4) % 8)
      if (b >= kSRing8)
        await_cnt(kCDone + (b - kSRing8) % kSRaw8, kSRT * ((b - kSRing8) / kSRaw8 + 1), a.spin_limit, expired);
      convert_block_f8(c, L, b);
    }
    arrive(&sCnt[kCLand + b], lane);
    if (b + kSDepth < nb) issue(b + kSDepth);
  }
  report_expired(a.part.status, expired, lane);
}

// ---------------------------------------------------------------------------------- compute
// Compute wave W (0..7) takes row tile T = W & 3 (query rows 16 T .. 16 T + 15) over the blocks of
// parity P = W >> 2; both waves of row tile T share SIMD T with loader T. T, P and the block
// count are run-time values and the block loop is rolled, so that the eight compute waves run
// one short copy of the code.
//
// MFMA layouts (v_mfma_f32_16x16x32_bf16, D = A B + C with A 16 x 32, B 32 x 16): lane l holds
// A[l & 15][8 (l >> 4) + 0..7], B[8 (l >> 4) + 0..7][l & 15] and D[4 (l >> 4) + i][l & 15].
// - Scores S^T = K Q^T per 16-key half t of a block: A = K rows 16 t .. 16 t + 15, B = Q^T, so
//   lane l holds query row l & 15 against keys 16 t + 4 (l >> 4) + i.
// - O^T += V^T P^T per 16-column tile dt of the head dim: B = P^T straight from the two score
//   accumulators (lane slots 0..3 = keys 4 (l >> 4) + i, slots 4..7 = keys 16 + 4 (l >> 4) + i),
//   A = V^T read in the same key order by two ds_read_b64_tr_b16; lane l then holds
//   O[query row l & 15][16 dt + 4 (l >> 4) + i].
template <bool NORM, bool F8>
__device__ __forceinline__ void split_compute(const SplitArgs& a, const SplitCtx& c, const int W) {
  const int T = W & 3, P = W >> 2;
  const int NB = c.nb > P ? (c.nb - P + 1) / 2 : 0;  // blocks P, P + 2, ... below nb
  const int lane = c.lane, j16 = lane & 15, g4 = lane >> 4;
  const long long head_off = (long long)c.g * a.Smax * kD;
  lds_u8* ring = AX_LDS(sRing);
  bool expired = false;
  lds_barrier();  // counters cleared

  // 1. Norm + RoPE of query rows 16 T + 4 P .. + 3 in place (rows 16 T + 8 .. + 15 are loader T's,
  //    the other four the partner wave's); in the own range also the own k rows of the same
  //    tokens, and with the fp8 cache the own k and v rows quantised. Roped q arrives ready.
  await_cnt(kCPro + T, 1, a.spin_limit, expired);
  if constexpr (NORM) norm_rows<1, F8>(a, c, 16 * T + 4 * P);
  if constexpr (F8) {
    if (c.pre) quant_own_rows<1>(a, c, 16 * T + 4 * P);
  }
  arrive(&sCnt[kCNorm], lane);
  // all 64 query rows (and in the own range the own rows) ready: twelve waves norm them
  await_cnt(kCNorm, (NORM || (F8 && c.pre)) ? kSC + kSL : kSC, a.spin_limit, expired);

  // 2. The query rows of row tile T as MFMA B operands (k-step kk: columns 32 kk .. 32 kk + 31).
  //    fp8 cache: the scores are products of the K codes with q on v_mfma_f32_16x16x128_f8f6f4
  //    (e4m3 x e4m3; lane l holds row l & 15 of either operand, columns 32 (l >> 4) .. + 31, as
  //    32 codes), q in two e4m3 parts: x = q 2^sg with 2^sg putting the row's largest |q| in
  //    [128, 256), hi = e4m3(x), lo = e4m3(x - hi) (both to nearest even; |x| < 256 needs no
  //    saturation): hi + lo = x exactly for |x| >= 1/4 (x keeps bf16's 8 significant bits, and
  //    x - hi is a multiple of x's last bit no larger than 8 of them), and within 2^-10 below,
  //    2^-17 of the row's largest; the score scale takes 2^-sg.
  bf16x8 qf[4];
  v8i32 qh, ql;
  float sscale = kScoreScale;  // log2(e) / sqrt(128), and with the fp8 cache times 2^-sg
  {
    const int r = 16 * T + j16;
    const lds_u8* qrow = AX_LDS(sQ) + r * 256;
    if constexpr (!F8) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) qf[kk] = lds_ld<bf16x8>(qrow + 16 * ((4 * kk + g4) ^ qswz(r)));
    } else {
      float x[32];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) unpack8v(lds_ld<u32x4>(qrow + 16 * ((4 * g4 + cc) ^ qswz(r))), x + 8 * cc);
      float mx = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) mx = fmax_(mx, fabsf(x[e]));
      mx = row_max4(mx);
      const int sg = mx > 0.f ? 8 - __builtin_amdgcn_frexp_expf(mx) : 0;
      sscale = kScoreScale * __builtin_ldexpf(1.0f, -sg);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = __builtin_ldexpf(x[4 * j + e], sg);
        int wh = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
        wh = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], wh, true);
        const auto d01 = __builtin_amdgcn_cvt_pk_f32_fp8(wh, false);
        const auto d23 = __builtin_amdgcn_cvt_pk_f32_fp8(wh, true);
        int wl = __builtin_amdgcn_cvt_pk_fp8_f32(y[0] - d01[0], y[1] - d01[1], 0, false);
        wl = __builtin_amdgcn_cvt_pk_fp8_f32(y[2] - d23[0], y[3] - d23[1], wl, true);
        qh[j] = wh;
        ql[j] = wl;
      }
    }
  }
  arrive(&sCnt[kCFrag], lane);  // (the exchange of step 5 reuses the RoPE rows once all eight have read)

  // 3. The blocks P, P + 2, ..., software-pipelined one block deep.
  // K: key row 16 t + j16, chunk 4 kk + g4; the second half of the keys is 4 KB further on. fp8
  // cache: the codes of key row 16 t + j16, chunks 2 g4 and 2 g4 + 1 (columns 32 g4 .. + 31); the
  // second half 2 KB further on.
  int koff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    koff[kk] = F8 ? (kk < 2 ? j16 * kD + 16 * ((2 * g4 + kk) ^ kswz8(j16)) : 0)
                  : j16 * 256 + 16 * ((4 * kk + g4) ^ kswz16(j16));
  // V: lane j16 of 16-lane group g4 supplies key row 4 g4 + (j16 >> 2) (+ 16 for the second read),
  // columns 16 dt + 4 (j16 & 3) .. + 3: half j16 & 1 of chunk 2 dt + ((j16 & 3) >> 1)
  const int vr = 4 * g4 + (j16 >> 2);
  int voff[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
    voff[dt] = vr * 256 + 16 * ((2 * dt + ((j16 & 3) >> 1)) ^ vswz16(vr)) + 8 * (j16 & 1);
  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;  // exponent reference of the lane's row (log2 units), the same in its 4 lanes
  float l = 0.f;        // this lane's share of the row sum
  f32x4 s[2];           // raw scores q . k of the block being exponentiated
  bf16x8 kf[2][4];
  v8i32 ka[2];  // fp8 cache: the K codes of the two halves
  v4i16 vt[8][2];
  bf16x8 pb;
  const bf16x2_t one2 = {(__bf16)1.0f, (__bf16)1.0f};
  constexpr int RS = F8 ? kSRaw8 : kSRing;  // tile-use counters in turn
  // (b uniform: scalar ops) K rows of block b (fp8: its raw tile's codes) and its V rows
  auto ktile_of = [&](int b) {
    return F8 ? ring + kSRawBase + (b % kSRaw8) * kSRawTile : ring + (b % kSRing) * kSTile;
  };
  auto vtile_of = [&](int b) { return F8 ? ring + (b % kSRing8) * kSVTile8 : ring + (b % kSRing) * kSTile + kSV; };
  auto read_k = [&](const lds_u8* base) {
    if constexpr (F8) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const u32x4 c0 = lds_ld<u32x4>(base + koff[0] + 2048 * t);
        const u32x4 c1 = lds_ld<u32x4>(base + koff[1] + 2048 * t);
        ka[t] = v8i32{(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3], (int)c1[0], (int)c1[1], (int)c1[2], (int)c1[3]};
      }
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) kf[t][kk] = lds_ld<bf16x8>(base + koff[kk] + 4096 * t);
    }
  };
  auto read_v = [&](const lds_u8* base) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        vt[dt][hf] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(base + voff[dt] + 4096 * hf));
  };
  auto qk = [&](f32x4* sd) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sd[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (F8) {
        sd[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka[t], qh, sd[t], 0, 0, 0, 0, 0, 0);
        sd[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka[t], ql, sd[t], 0, 0, 0, 0, 0, 0);
      } else {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          sd[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[t][kk], qf[kk], sd[t], 0, 0, 0);
      }
    }
  };
  // p = 2^(s log2(e) / sqrt(128) - m) (v_exp_f32 directly: the arguments are at most kSRescale, or
  // -inf), their bf16 pairs (the PV operand) and the row sum of the same rounded values, so every
  // output row is an exact convex combination of V rows. fp8 cache (block bx): p 2^kF8VShift
  // from the same exponential, times the key's value scale before the rounding to bf16 (the shift
  // keeps the products of every float32 scale from the denormals up to 2^25 in bf16's normal
  // range; O then accumulates in units of 2^-kF8VShift), and the row sum of the float32 p
  // 2^kF8VShift.
  auto softmax = [&](int bx) {
    float ps[2] = {0.f, 0.f};
    f32x4 vs[2];
    if constexpr (F8) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
        vs[t] = lds_ld<f32x4>(AX_LDS(sScl8) + bx * 256 + 64 * (2 * t + (g4 >> 1)) + 16 * (g4 & 1) + 32);
    }
    const float mo = F8 ? (float)kF8VShift - m : -m;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][2 * i], sscale, mo));
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][2 * i + 1], sscale, mo));
        if constexpr (F8) {
          const bf16x2_t pr = {(__bf16)(e0 * vs[t][2 * i]), (__bf16)(e1 * vs[t][2 * i + 1])};
          pb[4 * t + 2 * i] = pr[0];
          pb[4 * t + 2 * i + 1] = pr[1];
          ps[i] += e0 + e1;
        } else {
          const bf16x2_t pr = {(__bf16)e0, (__bf16)e1};
          pb[4 * t + 2 * i] = pr[0];
          pb[4 * t + 2 * i + 1] = pr[1];
          ps[i] = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, ps[i], false);
        }
      }
    l += ps[0] + ps[1];
  };
  // fp8 cache: the scores of block bx times their keys' scales (the lane's keys 16 t + 4 g4 + i)
  auto kscale = [&](f32x4* sd, int bx) {
    if constexpr (F8) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const f32x4 ks = lds_ld<f32x4>(AX_LDS(sScl8) + bx * 256 + 64 * (2 * t + (g4 >> 1)) + 16 * (g4 & 1));
#pragma unroll
        for (int i = 0; i < 4; ++i) sd[t][i] *= ks[i];
      }
    }
  };
  auto pv = [&]() {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const v4i16 both[2] = {vt[dt][0], vt[dt][1]};
      bf16x8 vf;
      __builtin_memcpy(&vf, both, 16);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb, o[dt], 0, 0, 0);
    }
  };
  // Keys of the range's last block past k_end get p = 0 (after the row max: such rows reload the
  // range's first key, a visible one).
  auto mask_tail = [&](f32x4* sd, int b) {
    const int lim = c.k_end - (c.k_begin + kBlk * b) - 4 * g4;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) sd[t][i] = (16 * t + i < lim) ? sd[t][i] : -INFINITY;
  };
  // Release of block b's tile (all four row tiles count here) right after its V reads are issued,
  // without waiting for them: a wave's LDS operations execute in order, so the increment cannot
  // pass the reads, and a loader that sees it only then starts loads that land far later.
  auto release = [&](int b) {
    if (c.pre) return;
    __builtin_amdgcn_sched_barrier(0);
    if (lane == 0) {
      const unsigned off = (unsigned)(uintptr_t)(lds_int*)&sCnt[kCDone + b % RS];
      asm volatile("ds_add_u32 %0, %1" ::"v"(off), "v"(1) : "memory");
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto landed = [&](int b) {
    if (c.pre) return;  // the own blocks are ready with the normed query rows
    await_cnt(kCLand + b, kSL, a.spin_limit, expired);
  };

  // K of block b + 2 is read at the end of iteration b, and its landed count is read early in
  // the iteration (before the V reads), so that neither the poll nor the K reads wait behind
  // this block's V reads; only a block not yet landed takes the blocking poll.
  // (The blocks go to the two waves by parity, not first come first served, so that every
  // partial sum, and with it the result, is the same from run to run.)
  if (NB > 0) {
    landed(P);
    read_k(ktile_of(P));
    qk(s);
    kscale(s, P);
    read_v(vtile_of(P));
    m = row_max4(lane_max8(s)) * sscale;  // finite: the block holds a visible key
    if (c.partial && P == c.nb - 1) mask_tail(s, P);
    release(P);
    if (NB > 1) {
      landed(P + 2);
      read_k(ktile_of(P + 2));
    }
#pragma clang loop unroll(disable)
    for (int k = 1; k < NB; ++k) {
      const int b = P + 2 * k;
      const bool more = k + 1 < NB;
      // (the count is read behind this block's K reads, which the scores need first anyway)
      const int early = (more && !c.pre)
                            ? __hip_atomic_load(&sCnt[kCLand + b + 2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)
                            : kSL;
      // (A) scores of block b beside the exponentials of block b - 2
      f32x4 sn[2];
      qk(sn);
      softmax(b - 2);
      kscale(sn, b);
      // (B) PV of block b - 2 beside the lane's share of the row max of block b
      pv();
      const float bm = lane_max8(sn) * sscale;
      read_v(vtile_of(b));
      // the reference moves only when the row's block max exceeds it by more than kSRescale:
      // p stays below 2^kSRescale and the O rescale is rare; a lane's share of the row max
      // decides whether any row needs it, and only then are the row's four lanes combined
      if (__builtin_amdgcn_ballot_w64(bm > m + kSRescale) != 0) {
        const float mn = fmax_(m, row_max4(bm));
        const float alpha = __builtin_amdgcn_exp2f(m - mn);
        m = mn;
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[dt][i] *= alpha;
      }
      if (c.partial && b == c.nb - 1) mask_tail(sn, b);
      s[0] = sn[0];
      s[1] = sn[1];
      release(b);
      if (more) {
        if (__builtin_amdgcn_readfirstlane(early) < kSL) landed(b + 2);
        read_k(ktile_of(b + 2));
      }
    }
    softmax(P + 2 * (NB - 1));
    pv();
  }

  // 4. Own range, q head parity 0: the roped own k rows and the own v rows of tokens 16 T + 8 P ..
  //    + 7 to the cache tail (the loaders load nothing into the own range's tiles). (The fp8 cache's
  //    tail was written with the quantisation.)
  if constexpr (!F8) {
    if (c.own && a.own_tail && c.hp == 0) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int tok = 16 * T + 8 * P + 4 * i + g4;
        const int tr = tok & (kBlk - 1);
        const lds_u8* ot = ring + (tok >> 5) * kSTile;
        const long long dst = head_off + (long long)(a.Smax - kT + tok) * kD + 8 * j16;
        const u32x4 kr = lds_ld<u32x4>(ot + tr * 256 + 16 * (j16 ^ kswz16(tr)));
        const u32x4 vr = lds_ld<u32x4>(ot + kSV + tr * 256 + 16 * (j16 ^ vswz16(tr)));
        __builtin_nontemporal_store(kr, reinterpret_cast<u32x4*>(a.Kc + dst));
        __builtin_nontemporal_store(vr, reinterpret_cast<u32x4*>(a.Vc + dst));
      }
    }
  }

  // 5. Merge of the two parity waves of row tile T through the RoPE rows' LDS (free once every
  //    compute wave has read its query fragments): wave (T, P) keeps column tiles 4 P .. 4 P + 3
  //    and hands over the other four (1 KB each) with its m and row total l.
  float lt = l;  // the row's total: its four lanes' shares
  {
    float2 pr = pair16(lt);
    lt = pr.x + pr.y;
    pr = pair32(lt);
    lt = pr.x + pr.y;
  }
  await_cnt(kCFrag, kSC, a.spin_limit, expired);
  lds_u8* xw = AX_LDS(sRope) + (2 * T + P) * 4096;        // written by this wave
  lds_u8* xr = AX_LDS(sRope) + (2 * T + (1 - P)) * 4096;  // written by the partner
  lds_u8* mw = AX_LDS(sQ) + (2 * T + P) * 512;            // this wave's m, then row total l, per lane
  lds_u8* mr = AX_LDS(sQ) + (2 * T + (1 - P)) * 512;      // the partner's
  // o[] is indexed with constants only (a run-time index would move the accumulators through
  // memory): the two parities take two copies of the hand-over and the store
  auto hand_over = [&](auto pc) {
    constexpr int PP = decltype(pc)::value;
#pragma unroll
    for (int j = 0; j < 4; ++j) lds_st(xw + j * 1024 + 16 * lane, o[4 * (1 - PP) + j]);
  };
  if (P == 0) hand_over(std::integral_constant<int, 0>{}); else hand_over(std::integral_constant<int, 1>{});
  lds_st(mw + 4 * lane, m);
  lds_st(mw + 256 + 4 * lane, lt);
  arrive(&sCnt[kCMrg + T], lane);
  await_cnt(kCMrg + T, 2, a.spin_limit, expired);
  const float mo = lds_ld<float>(mr + 4 * lane);
  const float lo_ = lds_ld<float>(mr + 256 + 4 * lane);
  const float M = fmax_(m, mo);  // finite: parity 0 has a block
  const float aw = __builtin_amdgcn_exp2f(m - M);   // 0 for a wave without blocks
  const float ao = __builtin_amdgcn_exp2f(mo - M);
  const float L = aw * lt + ao * lo_;  // stored by parity 0
  const bool bad = __builtin_amdgcn_ballot_w64(expired) != 0;
  const long long part = (long long)c.g * a.n_split + c.split;
  const int row = 64 * c.hp + 16 * T + j16;  // folded row of head g
  // Quarter qd = 2 PP + qq of the row (columns 32 qd .. 32 qd + 31) is column tiles 2 qd and
  // 2 qd + 1; in float16 with a power-of-two exponent per (row, quarter): the largest |value|
  // maps into [0.5, 1) and ldexp scales each element exactly, with no intermediate overflow.
  // Group (part, hp, T, qd) holds the quarter's 16 rows row-major (64 bytes a row), so that the
  // combine reads a row's quarter as one contiguous run; the two stores of a quarter fill its 1 KB.
  // Whole-line results that a later launch reads (these partials, the cache tail, the combine's
  // output) are stored nontemporally: they drain to memory during the launch rather than in the
  // L2 write-back at its end. (The 4- and 8-byte record words stay ordinary stores: as
  // nontemporal partial-line writes they slowed the launch.)
  auto store = [&](auto pc) {
    constexpr int PP = decltype(pc)::value;
    int exq[2];
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      f32x4 acc[2];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const f32x4 x = lds_ld<f32x4>(xr + (2 * qq + jj) * 1024 + 16 * lane);
        const f32x4& mine = o[4 * PP + 2 * qq + jj];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[jj][e] = __builtin_fmaf(ao, x[e], aw * mine[e]);
      }
      float mx = 0.f;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmax_(mx, fabsf(acc[jj][e]));
      mx = row_max4(mx);
      const int ex = __builtin_amdgcn_frexp_expf(mx);  // 0 for an all-zero quarter
      exq[qq] = F8 ? ex - kF8VShift : ex;  // (fp8: O in units of 2^-kF8VShift)
      u32x2 v[2];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        v[jj] = pack_f16x4(__builtin_ldexpf(acc[jj][0], -ex), __builtin_ldexpf(acc[jj][1], -ex),
                           __builtin_ldexpf(acc[jj][2], -ex), __builtin_ldexpf(acc[jj][3], -ex));
      u32x2* po = reinterpret_cast<u32x2*>(a.part.po) + (((part * 2 + c.hp) * 4 + T) * 4 + 2 * PP + qq) * 128 + 8 * j16 + g4;
      __builtin_nontemporal_store(v[0], po);  // columns 4 g4 .. 4 g4 + 3 of the quarter
      __builtin_nontemporal_store(v[1], po + 4);  // columns 16 + 4 g4 .. 16 + 4 g4 + 3
    }
    // the two quarters' exponents as one word of the row's record (e[2 PP], e[2 PP + 1])
    if (g4 == 0)
      reinterpret_cast<uint32_t*>(&a.part.rec[part * kQRows + row])[2 + PP] =
          (uint32_t)(exq[0] & 0xffff) | ((uint32_t)exq[1] << 16);
  };
  if (P == 0) store(std::integral_constant<int, 0>{}); else store(std::integral_constant<int, 1>{});
  if (P == 0 && g4 == 0)
    *reinterpret_cast<float2*>(&a.part.rec[part * kQRows + row]) =
        float2{bad ? __builtin_nanf("") : M, F8 ? L * 0x1p-64f : L};  // (fp8: l in units of 2^-kF8VShift)
  report_expired(a.part.status, expired, lane);
}

// NORM: q and the own k arrive raw and are normed + roped here (the layer step); otherwise both
// arrive roped (attention only).
template <bool NORM, bool F8>
__global__ __launch_bounds__(kSThreads, 1) void k_attn_split(SplitArgs a) {
  SplitCtx c;
  c.lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  c.g = blockIdx.x % kHkv;
  const int j = blockIdx.x / kHkv;
  c.split = j >> 1;
  c.hp = j & 1;
  c.own = c.split >= a.n_cache_split;
  c.pre = c.own && (!F8 || a.own_tail);
  c.k_begin = c.own ? a.S : c.split * a.kps;
  c.k_end = c.own ? a.S + kT : min(c.k_begin + a.kps, a.S);
  c.nb = (c.k_end - c.k_begin + kBlk - 1) / kBlk;
  c.partial = c.nb * kBlk != c.k_end - c.k_begin;
  if (threadIdx.x < kCN) sCnt[threadIdx.x] = 0;  // (wave 0, before its barrier)
  if (wave >= kSL)
    split_compute<NORM, F8>(a, c, wave - kSL);
  else
    split_loader<NORM, F8>(a, c, wave);
}

// Combine: out = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c, M = max_c m_c, with O_c the
// float16 partial times 2^(its quarter's exponent). One wave per output row (kv head g, folded
// row r = 64 hp + 16 T + j), the splits taken 16 at a time: lane 16 qd + k holds split c0 + k's
// (m, l) and its exponent for quarter qd; lane l then sums columns 2 l, 2 l + 1 over the splits in
// a fixed order, rescaling between groups of 16 with the running max. Columns 2 l, 2 l + 1 are
// word l & 15 of row j in the split's 1 KB group (hp, T, qd = l >> 4): one 4-byte load per split,
// 64 contiguous bytes per 16 lanes.
// Workgroup w: head w % 8 (the XCD whose L2 took the head's partials), rows 4 (w / 8) .. +3.
__global__ __launch_bounds__(256) void k_attn_combine(WsLayout p, uint16_t* out, int n_split) {
  const int lane = threadIdx.x & 63;
  const int g = blockIdx.x % kHkv;
  const int r = 4 * (blockIdx.x / kHkv) + (threadIdx.x >> 6);
  const int dt = lane >> 4;  // the quarter qd of the lane's columns
  const long long head = (long long)g * n_split;
  const int grp = (r >> 4) * 4 + dt;  // (hp * 4 + T) * 4 + qd
  const int word = 16 * (r & 15) + (lane & 15);
  const uint32_t* pw = reinterpret_cast<const uint32_t*>(p.po) + (head * 32 + grp) * 256 + word;
  float M = -INFINITY, L = 0.f, acc0 = 0.f, acc1 = 0.f;
  for (int c0 = 0; c0 < n_split; c0 += 16) {
    const int cs = c0 + (lane & 15);
    const bool valid = cs < n_split;
    const int cl = valid ? cs : c0;  // lanes past n_split repeat split c0, weighted 0 below
    const f32x4 rv = *reinterpret_cast<const f32x4*>(p.rec + (head + cl) * kQRows + r);
    const uint32_t ew = __float_as_uint(rv[2 + (dt >> 1)]);
    const int ec = (dt & 1) ? (int)(int16_t)(ew >> 16) : (int)(int16_t)(ew & 0xffff);
    float2 ov[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int ck = c0 + k < n_split ? c0 + k : c0;
      const uint32_t bits = pw[(long long)ck * 32 * 256];
      const _Float16 lo = __builtin_bit_cast(_Float16, (uint16_t)(bits & 0xffffu));
      const _Float16 hi = __builtin_bit_cast(_Float16, (uint16_t)(bits >> 16));
      ov[k] = float2{(float)lo, (float)hi};
    }
    float Mg = valid ? rv[0] : -INFINITY;
    Mg = fmaxf(Mg, row_ror<8>(Mg));
    Mg = fmaxf(Mg, row_ror<4>(Mg));
    Mg = fmaxf(Mg, row_ror<2>(Mg));
    Mg = fmaxf(Mg, row_ror<1>(Mg));  // every lane of a 16-lane row: the group's max
    const float Mn = fmaxf(M, Mg);
    const float rs = __builtin_amdgcn_exp2f(M - Mn);  // 0 while M is -inf
    acc0 *= rs;
    acc1 *= rs;
    L *= rs;
    M = Mn;
    const float w = valid ? __builtin_amdgcn_exp2f(rv[0] - M) : 0.f;
    float wl = w * rv[1];
    wl += row_ror<8>(wl);
    wl += row_ror<4>(wl);
    wl += row_ror<2>(wl);
    wl += row_ror<1>(wl);
    L += wl;
    const float wq = __builtin_ldexpf(w, ec);  // weight of split cs, quarter lane >> 4
    static_for<16>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      // the weight of split c0 + k for this lane's quarter: lane k of the same 16-lane row
      // (DPP row_newbcast)
      const float wk = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(wq), 0x150 + k, 0xf, 0xf, false));
      acc0 = __builtin_fmaf(wk, ov[k].x, acc0);
      acc1 = __builtin_fmaf(wk, ov[k].y, acc1);
    });
  }
  const float inv = 1.0f / L;
  uint32_t* dst = reinterpret_cast<uint32_t*>(out + ((long long)g * kQRows + r) * kD + 2 * lane);
  __builtin_nontemporal_store(pack_bf16x2(acc0 * inv, acc1 * inv), dst);  // (a whole 256-byte row per wave)
}

AttnPlan attn_plan(int S, int /*Smax*/) {
  AttnPlan p;
  p.n_keys = S + kT;
  // at most 15 cache ranges of whole blocks, at most 10 blocks each, plus the own-token range:
  // with two q heads per range, 8 x 16 x 2 = 256 workgroups at S = 4700
  int kps = (S + kSCacheRanges - 1) / kSCacheRanges;
  kps = (kps + kBlk - 1) / kBlk * kBlk;
  if (kps < kBlk) kps = kBlk;
  if (kps > kBlk * kSMaxNB) kps = kBlk * kSMaxNB;
  p.keys_per_split = kps;
  p.n_cache_split = (S + kps - 1) / kps;
  p.n_split = p.n_cache_split + 1;
  p.blocks = kps / kBlk;
  return p;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t attn_partials_bytes(const AttnPlan& p) {
  const size_t rows = (size_t)kHkv * p.n_split * kQRows;
  return kStatusBytes + align256(rows * kD * 2) + align256(rows * sizeof(PartRec));
}

WsLayout ws_layout(const AttnPlan& plan, const void* ws) {
  const size_t rows = (size_t)kHkv * plan.n_split * kQRows;
  char* w = static_cast<char*>(const_cast<void*>(ws));
  WsLayout l;
  l.status = reinterpret_cast<int*>(w);
  w += kStatusBytes;
  l.po = reinterpret_cast<uint16_t*>(w);
  w += align256(rows * kD * 2);
  l.rec = reinterpret_cast<PartRec*>(w);
  return l;
}

hipError_t launch_attn_combine(const AttnPlan& plan, const void* ws, uint16_t* out, hipStream_t st) {
  hipLaunchKernelGGL(k_attn_combine, dim3(kHkv * kQRows / 4), dim3(256), 0, st, ws_layout(plan, ws), out,
                     plan.n_split);
  return hipGetLastError();
}

hipError_t launch_attn(const AttnPlan& plan, const AttnLaunch& p, hipStream_t st) {
  const hipError_t e = launch_attn_split(plan, p, st);
  if (e != hipSuccess) return e;
  return launch_attn_combine(plan, p.ws, p.out, st);
}

hipError_t launch_attn_split(const AttnPlan& plan, const AttnLaunch& p, hipStream_t st) {
  SplitArgs a{};
  a.q = p.q; a.gq = p.gq; a.gk = p.gk; a.cos_t = p.cos_t; a.sin_t = p.sin_t; a.eps = p.eps;
  a.own_tail = p.k_tail != nullptr;
  if (a.own_tail) {
    a.kt_base = p.k_tail; a.vt_base = p.v_tail; a.tail_stride = (long long)kT * kD;
  } else {
    a.kt_base = p.Kc + (long long)(p.Smax - kT) * kD; a.vt_base = p.Vc + (long long)(p.Smax - kT) * kD;
    a.tail_stride = (long long)p.Smax * kD;
  }
  a.Kc = p.Kc; a.Vc = p.Vc;
  a.part = ws_layout(plan, p.ws);
  a.spin_limit = wait_limit();
  a.S = p.S; a.Smax = p.Smax; a.n_split = plan.n_split; a.kps = plan.keys_per_split;
  a.n_cache_split = plan.n_cache_split;
  const dim3 grid(kHkv * plan.n_split * 2);
  if (p.q_norm)
    hipLaunchKernelGGL((k_attn_split<true, false>), grid, dim3(kSThreads), 0, st, a);
  else
    hipLaunchKernelGGL((k_attn_split<false, false>), grid, dim3(kSThreads), 0, st, a);
  return hipGetLastError();
}

// fp8 cache: the same plan with ranges of at most 17 blocks (at S = 8128: 15 ranges of 544 keys,
// 256 workgroups), the same partials and combine.
AttnPlan attn_plan_f8(int S, int /*Smax*/) {
  AttnPlan p;
  p.n_keys = S + kT;
  int kps = (S + kSCacheRanges - 1) / kSCacheRanges;
  kps = (kps + kBlk - 1) / kBlk * kBlk;
  if (kps < kBlk) kps = kBlk;
  if (kps > kBlk * kSMaxNB8) kps = kBlk * kSMaxNB8;
  p.keys_per_split = kps;
  p.n_cache_split = (S + kps - 1) / kps;
  p.n_split = p.n_cache_split + 1;
  p.blocks = kps / kBlk;
  return p;
}

size_t attn_partials_bytes_f8(const AttnPlan& p) { return attn_partials_bytes(p); }

hipError_t launch_attn_f8_combine(const AttnPlan& plan, const void* ws, uint16_t* out, hipStream_t st) {
  return launch_attn_combine(plan, ws, out, st);
}

hipError_t launch_attn_f8_split(const AttnPlan& plan, const AttnLaunchF8& p, hipStream_t st) {
  SplitArgs a{};
  a.q = p.q; a.gq = p.gq; a.gk = p.gk; a.cos_t = p.cos_t; a.sin_t = p.sin_t; a.eps = p.eps;
  a.own_tail = p.k_own != nullptr;
  a.kt_base = p.k_own; a.vt_base = p.v_own; a.tail_stride = (long long)kT * kD;
  a.Kc = nullptr; a.Vc = nullptr;
  a.Kc8 = p.Kc; a.Vc8 = p.Vc; a.Ks = p.Ks; a.Vs = p.Vs;
  a.part = ws_layout(plan, p.ws);
  a.spin_limit = wait_limit();
  a.S = p.S; a.Smax = p.Smax; a.n_split = plan.n_split; a.kps = plan.keys_per_split;
  a.n_cache_split = plan.n_cache_split;
  const dim3 grid(kHkv * plan.n_split * 2);
  if (p.q_norm)
    hipLaunchKernelGGL((k_attn_split<true, true>), grid, dim3(kSThreads), 0, st, a);
  else
    hipLaunchKernelGGL((k_attn_split<false, true>), grid, dim3(kSThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_f8(const AttnPlan& plan, const AttnLaunchF8& p, hipStream_t st) {
  const hipError_t e = launch_attn_f8_split(plan, p, st);
  if (e != hipSuccess) return e;
  return launch_attn_combine(plan, p.ws, p.out, st);
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
