// Internal host-side launch interfaces between the C ABI (ax_api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ax {

struct QkLaunch {
  const uint16_t* q_in;
  const uint16_t* k_in;
  const uint16_t* v_in;
  const uint16_t* gq;
  const uint16_t* gk;
  const float* cos_t;
  const float* sin_t;
  float eps;
  uint16_t* q_out;
  uint16_t* k_dst;   // k_out ([8][64][128]) or Kc
  uint16_t* v_dst;   // null, or Vc
  int tail_smax;     // 0: k_dst is a plain [8][64][128] tensor; >0: k_dst/v_dst are caches of this length
};

hipError_t launch_qk_norm_rope(const QkLaunch& p, hipStream_t st);
hipError_t launch_tail_copy(const uint16_t* k, const uint16_t* v, uint16_t* Kc, uint16_t* Vc, int Smax,
                            hipStream_t st);

// Split-KV attention plan for one (S, Smax).
struct AttnPlan {
  int n_keys;        // S + 64 visible keys per kv head
  int n_split;       // key splits per kv head: n_cache_split over [0, S), then one over the own tokens
  int n_cache_split;
  int keys_per_split;  // of the cache splits (the last one may be shorter)
  int blocks;        // 32-key blocks per split (kernel variant), at least the own split's 2
};

AttnPlan attn_plan(int S, int Smax);     // bf16 cache
AttnPlan attn_plan_f8(int S, int Smax);  // fp8 cache (longer key ranges: a block is half the bytes)

// Polls a bounded in-workgroup wait makes before it gives up: the default (about 30 ms of
// polling), or the value set through ax_debug_set_wait_limit.
constexpr int kDefaultWaitLimit = 1 << 20;
int wait_limit();

// Partials inside the workspace (both cache formats), after the status word (the first 256
// bytes), per (kv head g, key range c) = part g * n_split + c: O in float16, scaled by 2^-e per
// (row, 32-column quarter qd), in 1 KB groups (part, q head parity hp, row tile T, qd), each the
// quarter's 16 rows row-major (row 64 hp + 16 T + j at byte 64 j, its column 32 qd + x at
// 64 j + 2 x); then one 16-byte record per (part, folded row): float m, float l, int16 e[4].
// Both regions 256-byte aligned.
struct PartRec {
  float m;
  float l;
  int16_t e[4];
};
static_assert(sizeof(PartRec) == 16, "one 16-byte load per record");
struct WsLayout {
  int* status;
  uint16_t* po;
  PartRec* rec;
};
size_t attn_partials_bytes(const AttnPlan& p);
WsLayout ws_layout(const AttnPlan& plan, const void* ws);

// fp8-cache partials: the same layout as the bf16 cache's
size_t attn_partials_bytes_f8(const AttnPlan& p);

struct AttnLaunch {
  const uint16_t* q;       // [16][64][128] (== folded [8][128][128]): raw if q_norm, else roped
  const uint16_t* gq;      // RMSNorm gammas (used when q_norm)
  const uint16_t* gk;
  const float* cos_t;      // RoPE tables [64][64]
  const float* sin_t;
  float eps;
  const uint16_t* k_tail;  // own k [8][64][128] (raw if q_norm, else roped), or null: tail already in Kc
  const uint16_t* v_tail;  // own v, or null
  uint16_t* Kc;
  uint16_t* Vc;
  uint16_t* out;           // [8][128][128]
  void* ws;                // partials
  int S, Smax;
  int q_norm;              // q and the own k arrive raw and are normed + roped in the kernel
};

// fp8 cache: e4m3 codes [8][Smax][128] with a float32 scale per (kv head, row) [8][Smax].
struct AttnLaunchF8 {
  const uint16_t* q;       // [16][64][128]: raw if q_norm, else roped
  const uint16_t* gq;
  const uint16_t* gk;
  const float* cos_t;
  const float* sin_t;
  float eps;
  const uint16_t* k_own;   // own k [8][64][128] (raw if q_norm, else roped), or null: tail already in the cache
  const uint16_t* v_own;
  uint8_t* Kc;
  float* Ks;
  uint8_t* Vc;
  float* Vs;
  uint16_t* out;
  void* ws;
  int S, Smax;
  int q_norm;
};
hipError_t launch_attn_f8(const AttnPlan& plan, const AttnLaunchF8& p, hipStream_t st);        // both
hipError_t launch_attn_f8_split(const AttnPlan& plan, const AttnLaunchF8& p, hipStream_t st);  // partials
hipError_t launch_attn_f8_combine(const AttnPlan& plan, const void* ws, uint16_t* out, hipStream_t st);
hipError_t launch_tail_quant_f8(const uint16_t* k, const uint16_t* v, uint8_t* Kc, float* Ks, uint8_t* Vc,
                                float* Vs, int Smax, hipStream_t st);

hipError_t launch_attn(const AttnPlan& plan, const AttnLaunch& p, hipStream_t st);        // both
hipError_t launch_attn_split(const AttnPlan& plan, const AttnLaunch& p, hipStream_t st);  // partials
hipError_t launch_attn_combine(const AttnPlan& plan, const void* ws, uint16_t* out, hipStream_t st);

// Text-model decode step: one token at cache row pos, 64 query heads, 8 kv heads.
struct DecodeLaunch {
  const uint16_t* q;      // [64][128] raw
  const uint16_t* k;      // [8][128] raw
  const uint16_t* v;      // [8][128]
  const uint16_t* gq;
  const uint16_t* gk;
  const float* cos_t;     // [64] for position pos + rope_delta
  const float* sin_t;
  float eps;
  uint16_t* Kc;
  uint16_t* Vc;
  uint16_t* out;          // [64][128]
  void* ws;
  int pos, Smax;
};
AttnPlan decode_plan(int pos);
size_t decode_partials_bytes(const AttnPlan& p);
hipError_t launch_decode(const AttnPlan& plan, const DecodeLaunch& p, hipStream_t st);

// One whole expert decoder layer (residual norms, projections, SwiGLU MLP around the attention
// step). Widths of the expert's layer: residual 1536, qkv 4096 (16 + 8 + 8 heads of 128), MLP 6144.
constexpr int kLayerHidden = 1536;
constexpr int kLayerQkv = 4096;
constexpr int kLayerMlp = 6144;
struct LayerLaunch {
  const uint16_t* x;      // [64][1536]
  const uint16_t* ln1;    // [1536]
  const uint16_t* wqkv;   // [1536][4096], packed (launch_pack_w64) like the other four matrices
  const uint16_t* qn;     // [128]
  const uint16_t* kn;
  const uint16_t* wo;     // [2048][1536]
  const uint16_t* ln2;
  const uint16_t* w1;     // [1536][6144]
  const uint16_t* w3;
  const uint16_t* w2;     // [6144][1536]
  const float* cos_t;     // [64][64]
  const float* sin_t;
  float eps;
  uint16_t* Kc;
  uint16_t* Vc;
  int S, Smax;
  uint16_t* x_out;        // [64][1536]
  void* ws;
  // a chained layer: n1_in (if not null) is RMSNorm(x; ln1), made by the previous layer's last
  // launch, and the first norm is skipped; with ln1_next, the last launch also writes n1_out =
  // RMSNorm(x_out; ln1_next) for the next layer
  const uint16_t* n1_in = nullptr;
  const uint16_t* ln1_next = nullptr;
  uint16_t* n1_out = nullptr;
};
size_t layer_workspace_bytes(int S, int Smax);
hipError_t launch_layer(const LayerLaunch& p, hipStream_t st);
// C[64][N] = bf16(A[64][K] W[K][N]) (W input-major, packed); ws: gemm64_partials_bytes(K, N) bytes.
bool gemm64_shape_ok(int K, int N);
// Weights into the packed layout the projection kernel streams (K x N elements, same size).
hipError_t launch_pack_w64(const uint16_t* W, int K, int N, uint16_t* Wp, hipStream_t st);
size_t gemm64_partials_bytes(int K, int N);
hipError_t launch_linear64(const uint16_t* A, const uint16_t* W, int K, int N, uint16_t* C, void* ws,
                           hipStream_t st);

hipError_t launch_copy_words(const void* src, void* dst, size_t n, hipStream_t st);

}  // namespace ax
