// q/k RMSNorm + rotate_half RoPE, and the own-K/V tail write into the KV cache.
//
// Page code/alpamayo_tt/expert.py, TTExpert.layer: rms_norm of q and k with the
// qn/kn gammas, rotary_embedding_hf on both, then fill_cache of the roped k and
// the raw v at row Smax - 64 of the layer's cache (EXPERT_NOTES.md, "Attention
// over the VLM cache: masking approach").
//
// Layout of the work: a 16-lane group owns one 128-wide row (8 bf16 per lane,
// one 16-byte load). Rows 0..1023 are q (head h = r / 64, token r % 64), rows
// 1024..1535 are k, rows 1536..2047 are v (copied, not normed). 256-thread
// blocks, 16 rows each: 128 blocks for a full step.
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

  const uint16_t* src = is_q ? a.q_in : (is_k ? a.k_in : a.v_in);
  const uint4 raw = *reinterpret_cast<const uint4*>(src + (long long)rr * kD + 8 * j16);
  if (is_q || is_k) {
    float x[8], g[8], c[8], s[8];
    unpack8(raw, x);
    unpack8(*reinterpret_cast<const uint4*>((is_q ? a.gq : a.gk) + 8 * j16), g);
    const int f0 = 8 * (j16 & 7);
    const float4* cp = reinterpret_cast<const float4*>(a.cos_t + tok * 64 + f0);
    const float4* sp = reinterpret_cast<const float4*>(a.sin_t + tok * 64 + f0);
    const float4 c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
    c[0] = c0.x; c[1] = c0.y; c[2] = c0.z; c[3] = c0.w; c[4] = c1.x; c[5] = c1.y; c[6] = c1.z; c[7] = c1.w;
    s[0] = s0.x; s[1] = s0.y; s[2] = s0.z; s[3] = s0.w; s[4] = s1.x; s[5] = s1.y; s[6] = s1.z; s[7] = s1.w;
    float A[8], B[8];
    rope_coef(g, c, s, j16, A, B);
    norm_rope_row16(x, A, B, a.eps);
    if (live) {
      uint16_t* dst = is_q ? a.q_out + (long long)rr * kD
                           : a.k_dst + head * a.kv_head_stride + (a.kv_row0 + tok) * kD;
      *reinterpret_cast<uint4*>(dst + 8 * j16) = pack8(x);
    }
  } else if (live) {
    uint16_t* dst = a.v_dst + head * a.kv_head_stride + (a.kv_row0 + tok) * kD;
    *reinterpret_cast<uint4*>(dst + 8 * j16) = raw;
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
