// q/k RMSNorm + rotate_half RoPE, and the own-K/V tail write into the KV cache.
//
// Page code/alpamayo_tt/expert.py, TTExpert.layer: rms_norm of q and k with the
// qn/kn gammas, rotary_embedding_hf on both, then fill_cache of the roped k and
// the raw v at row Smax - 64 of the layer's cache (EXPERT_NOTES.md, "Attention
// over the VLM cache: masking approach").
//
// Layout of the work: a 16-lane group owns one 128-wide row. Rows 0..1023 are q (head
// h = r / 64, token r % 64), rows 1024..1535 are k, rows 1536..2047 are v (copied, not
// normed, one 16-byte piece per lane). A q or k row is held in the pair layout (lane j16:
// columns 4 j16 .. +3 and 64 + 4 j16 .. +3, two 8-byte pieces), the arithmetic the fused
// attention kernels use too, so both paths give the same bits. 256-thread blocks, 16 rows
// each: 128 blocks for a full step.
#include "ax_dev.h"
#include "ax_launch.h"

namespace ax {

struct QkArgs {
  const uint16_t* q_in;
  const uint16_t* k_in;
  const uint16_t* v_in;     // may be null (no v copy)
  const uint16_t* gq;
  const uint16_t* gk;
  const float* cos_t;       // [64][64]
  const float* sin_t;
  float eps;
  uint16_t* q_out;          // [16][64][128]; null: q rows skipped
  uint16_t* k_dst;          // roped k destination base
  uint16_t* v_dst;          // v destination base (null: skip)
  long long kv_head_stride; // elements between kv heads at the destination
  long long kv_row0;        // first destination row of token 0
  int row_begin;            // first row of the job (0: q, 1024: k only, 2048: v only)
  int row_end;
};

constexpr int kQRowsAll = kHq * kT;   // 1024
constexpr int kKRowsAll = kHkv * kT;  // 512

__global__ __launch_bounds__(256) void k_qk_norm_rope(QkArgs a) {
  const int j16 = threadIdx.x & 15;
  const int row = a.row_begin + blockIdx.x * 16 + (threadIdx.x >> 4);
  // Rows past the end still take part in the shuffles of their wave but store nothing.
  const bool live = row < a.row_end;
  const int r = live ? row : a.row_begin;
  const bool is_q = r < kQRowsAll;
  const bool is_k = !is_q && r < kQRowsAll + kKRowsAll;
  const int rr = is_q ? r : (is_k ? r - kQRowsAll : r - kQRowsAll - kKRowsAll);
  const int tok = rr & (kT - 1);
  const int head = rr >> 6;

  const uint16_t* src = (is_q ? a.q_in : (is_k ? a.k_in : a.v_in)) + (long long)rr * kD;
  if (is_q || is_k) {
    float x[8], g[8], A[8], B[8];
    unpack_pair(*reinterpret_cast<const uint2*>(src + 4 * j16), *reinterpret_cast<const uint2*>(src + 64 + 4 * j16),
                x);
    const uint16_t* gam = is_q ? a.gq : a.gk;
    unpack_pair(*reinterpret_cast<const uint2*>(gam + 4 * j16), *reinterpret_cast<const uint2*>(gam + 64 + 4 * j16),
                g);
    const float4 c4 = *reinterpret_cast<const float4*>(a.cos_t + tok * 64 + 4 * j16);
    const float4 s4 = *reinterpret_cast<const float4*>(a.sin_t + tok * 64 + 4 * j16);
    const float c[4] = {c4.x, c4.y, c4.z, c4.w}, s[4] = {s4.x, s4.y, s4.z, s4.w};
    rope_coef_pair(g, c, s, A, B);
    norm_rope_pair(x, A, B, a.eps);
    if (live) {
      uint16_t* dst = is_q ? a.q_out + (long long)rr * kD
                           : a.k_dst + head * a.kv_head_stride + (a.kv_row0 + tok) * kD;
      uint2 lo, hi;
      pack_pair(x, lo, hi);
      *reinterpret_cast<uint2*>(dst + 4 * j16) = lo;
      *reinterpret_cast<uint2*>(dst + 64 + 4 * j16) = hi;
    }
  } else if (live) {
    uint16_t* dst = a.v_dst + head * a.kv_head_stride + (a.kv_row0 + tok) * kD;
    *reinterpret_cast<uint4*>(dst + 8 * j16) = *reinterpret_cast<const uint4*>(src + 8 * j16);
  }
}

// Plain tail copy: 1024 rows (k then v), one 16-byte word per lane.
__global__ __launch_bounds__(256) void k_tail_copy(const uint16_t* k, const uint16_t* v, uint16_t* Kc,
                                                   uint16_t* Vc, long long head_stride, long long row0) {
  const int w = blockIdx.x * 256 + threadIdx.x;  // word index over 2 * 512 rows * 16 words
  const int row = w >> 4, j16 = w & 15;
  if (row >= 2 * kKRowsAll) return;
  const bool is_k = row < kKRowsAll;
  const int rr = is_k ? row : row - kKRowsAll;
  const uint4 x = *reinterpret_cast<const uint4*>((is_k ? k : v) + (long long)rr * kD + 8 * j16);
  uint16_t* dst = (is_k ? Kc : Vc) + (rr >> 6) * head_stride + (row0 + (rr & 63)) * kD;
  *reinterpret_cast<uint4*>(dst + 8 * j16) = x;
}

hipError_t launch_qk_norm_rope(const QkLaunch& p, hipStream_t st) {
  QkArgs a;
  a.q_in = p.q_in; a.k_in = p.k_in; a.v_in = p.v_in; a.gq = p.gq; a.gk = p.gk;
  a.cos_t = p.cos_t; a.sin_t = p.sin_t; a.eps = p.eps; a.q_out = p.q_out;
  a.k_dst = p.k_dst; a.v_dst = p.v_dst;
  if (p.tail_smax > 0) {
    a.kv_head_stride = (long long)p.tail_smax * kD;
    a.kv_row0 = p.tail_smax - kT;
  } else {
    a.kv_head_stride = (long long)kT * kD;
    a.kv_row0 = 0;
  }
  a.row_begin = 0;
  a.row_end = kQRowsAll + kKRowsAll + (p.v_dst ? kKRowsAll : 0);
  const int nblk = (a.row_end - a.row_begin + 15) / 16;
  hipLaunchKernelGGL(k_qk_norm_rope, dim3(nblk), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_tail_copy(const uint16_t* k, const uint16_t* v, uint16_t* Kc, uint16_t* Vc, int Smax,
                            hipStream_t st) {
  const int words = 2 * kKRowsAll * 16;
  hipLaunchKernelGGL(k_tail_copy, dim3((words + 255) / 256), dim3(256), 0, st, k, v, Kc, Vc,
                     (long long)Smax * kD, (long long)(Smax - kT));
  return hipGetLastError();
}

}  // namespace ax
