// C ABI of libax: argument validation on the host, then launches on the caller's stream.
// Declarations and the contract of every entry point are in include/ax.h.
#include <math.h>
#include <string.h>

#include <atomic>

#include "../../include/ax.h"
#include "ax_launch.h"

namespace {

constexpr int kMaxDev = 64;
// 0 = unknown, 1 = gfx950, -1 = other; atomic because callers on several host threads may fill
// the same entry (all with the same value)
std::atomic<int> g_arch[kMaxDev];

// Is the current device a gfx950? Cached per device (the query is not a stream operation).
int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return AX_E_UNSUPPORTED;
  int arch = g_arch[dev].load(std::memory_order_relaxed);
  if (arch == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return AX_E_UNSUPPORTED;
    arch = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_arch[dev].store(arch, std::memory_order_relaxed);
  }
  return arch == 1 ? AX_OK : AX_E_UNSUPPORTED;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_ptrs(std::initializer_list<const void*> ps, bool allow_null = false) {
  for (const void* p : ps)
    if (p == nullptr && !allow_null) return AX_E_NULL;
  for (const void* p : ps)
    if (p != nullptr && !aligned16(p)) return AX_E_ALIGN;
  return AX_OK;
}

int check_shape(int S, int Smax) {
  if (Smax < AX_N_TOK || Smax > AX_SMAX_LIMIT) return AX_E_SHAPE;
  if (S < 0 || S > Smax - AX_N_TOK) return AX_E_SHAPE;
  return AX_OK;
}

int check_eps(float eps) { return (isfinite(eps) && eps >= 0.f) ? AX_OK : AX_E_ARG; }

int status(hipError_t e) { return e == hipSuccess ? AX_OK : static_cast<int>(e); }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Polls of a bounded in-workgroup wait (0: the default); read at each launch.
std::atomic<int> g_wait_limit{0};

}  // namespace

// Scratch of ax_expert_layer_attn_noalloc: one copy per GPU the library runs on, held until the
// process ends. In host code the array's name is only a stand-in: kernels get the device address
// that hipGetSymbolAddress returns for it on the current device (scratch_ptr).
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

std::atomic<void*> g_scratch[kMaxDev];

// Device address of the current device's scratch, looked up on the device's first call (with
// that device current) and kept per device.
int scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return AX_E_UNSUPPORTED;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return static_cast<int>(e);
    if (p == nullptr) return AX_E_UNSUPPORTED;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return AX_OK;
}

}  // namespace

namespace ax {
int wait_limit() {
  const int v = g_wait_limit.load(std::memory_order_relaxed);
  return v > 0 ? v : kDefaultWaitLimit;
}
}  // namespace ax

extern "C" {

int ax_abi_version(void) { return AX_ABI_VERSION; }

int ax_debug_set_wait_limit(int polls) {
  if (polls < 0) return AX_E_ARG;
  g_wait_limit.store(polls, std::memory_order_relaxed);
  return AX_OK;
}

const char* ax_strerror(int code) {
  switch (code) {
    case AX_OK: return "ok";
    case AX_E_NULL: return "a required pointer is NULL";
    case AX_E_SHAPE: return "invalid shape: need 64 <= Smax <= 2^20 and 0 <= S <= Smax - 64";
    case AX_E_ALIGN: return "a device pointer is not 16-byte aligned";
    case AX_E_WORKSPACE: return "workspace too small or misaligned";
    case AX_E_UNSUPPORTED: return "no gfx950 device is current";
    case AX_E_ARG: return "invalid scalar argument";
    default: return code > 0 ? hipGetErrorString(static_cast<hipError_t>(code)) : "unknown error";
  }
}

int ax_rope_tables(int pos0, int n_tok, int head_dim, double theta, float* cos_h, float* sin_h) {
  if (!cos_h || !sin_h) return AX_E_NULL;
  if (n_tok <= 0 || head_dim <= 0 || (head_dim & 1)) return AX_E_SHAPE;
  if (!(theta > 0.0) || !isfinite(theta) || pos0 < 0) return AX_E_ARG;
  const int half = head_dim / 2;
  for (int j = 0; j < half; ++j) {
    const double inv = pow(theta, -2.0 * j / head_dim);
    for (int i = 0; i < n_tok; ++i) {
      const double ang = (double)(pos0 + i) * inv;
      cos_h[i * half + j] = (float)cos(ang);
      sin_h[i * half + j] = (float)sin(ang);
    }
  }
  return AX_OK;
}

int ax_qk_norm_rope(const uint16_t* q_in, const uint16_t* k_in, const uint16_t* gamma_q,
                    const uint16_t* gamma_k, const float* rope_cos, const float* rope_sin, float eps,
                    uint16_t* q_out, uint16_t* k_out, void* stream) {
  int r = check_ptrs({q_in, k_in, gamma_q, gamma_k, rope_cos, rope_sin, q_out, k_out});
  if (r == AX_OK) r = check_eps(eps);
  if (r == AX_OK) r = check_device();
  if (r != AX_OK) return r;
  ax::QkLaunch p{q_in, k_in, nullptr, gamma_q, gamma_k, rope_cos, rope_sin, eps, q_out, k_out, nullptr, 0};
  return status(ax::launch_qk_norm_rope(p, as_stream(stream)));
}

int ax_cache_tail_write(const uint16_t* k_roped, const uint16_t* v, uint16_t* Kc, uint16_t* Vc, int Smax,
                        void* stream) {
  int r = check_ptrs({k_roped, v, Kc, Vc});
  if (r == AX_OK) r = check_shape(0, Smax);
  if (r == AX_OK) r = check_device();
  if (r != AX_OK) return r;
  return status(ax::launch_tail_copy(k_roped, v, Kc, Vc, Smax, as_stream(stream)));
}

int ax_qk_norm_rope_tail(const uint16_t* q_in, const uint16_t* k_in, const uint16_t* v_in,
                         const uint16_t* gamma_q, const uint16_t* gamma_k, const float* rope_cos,
                         const float* rope_sin, float eps, uint16_t* q_out, uint16_t* Kc, uint16_t* Vc,
                         int Smax, void* stream) {
  int r = check_ptrs({q_in, k_in, v_in, gamma_q, gamma_k, rope_cos, rope_sin, q_out, Kc, Vc});
  if (r == AX_OK) r = check_shape(0, Smax);
  if (r == AX_OK) r = check_eps(eps);
  if (r == AX_OK) r = check_device();
  if (r != AX_OK) return r;
  ax::QkLaunch p{q_in, k_in, v_in, gamma_q, gamma_k, rope_cos, rope_sin, eps, q_out, Kc, Vc, Smax};
  return status(ax::launch_qk_norm_rope(p, as_stream(stream)));
}

size_t ax_expert_attn_workspace_bytes(int S, int Smax) {
  if (check_shape(S, Smax) != AX_OK) return 0;
  return ax::attn_partials_bytes(ax::attn_plan(S, Smax));
}

static int check_ws(const void* ws, size_t ws_bytes, int S, int Smax) {
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return AX_E_WORKSPACE;
  return ws_bytes >= ax_expert_attn_workspace_bytes(S, Smax) ? AX_OK : AX_E_WORKSPACE;
}

int ax_expert_attn(const uint16_t* q_roped, const uint16_t* k_own, const uint16_t* v_own, uint16_t* Kc,
                   uint16_t* Vc, int S, int Smax, uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  int r = check_ptrs({q_roped, Kc, Vc, out, ws});
  if (r == AX_OK && ((k_own == nullptr) != (v_own == nullptr))) r = AX_E_NULL;
  if (r == AX_OK && k_own && (!aligned16(k_own) || !aligned16(v_own))) r = AX_E_ALIGN;
  if (r == AX_OK) r = check_shape(S, Smax);
  if (r == AX_OK) r = check_ws(ws, ws_bytes, S, Smax);
  if (r == AX_OK) r = check_device();
  if (r != AX_OK) return r;
  const ax::AttnPlan plan = ax::attn_plan(S, Smax);
  ax::AttnLaunch p{q_roped, nullptr, nullptr, nullptr, nullptr, 0.f, k_own, v_own, Kc, Vc, out, ws, S, Smax,
                   /*q_norm=*/0};
  return status(ax::launch_attn(plan, p, as_stream(stream)));
}

int ax_expert_layer_attn(const uint16_t* q_in, const uint16_t* k_in, const uint16_t* v_in,
                         const uint16_t* gamma_q, const uint16_t* gamma_k, const float* rope_cos,
                         const float* rope_sin, float eps, uint16_t* Kc, uint16_t* Vc, int S, int Smax,
                         uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  int r = check_ptrs({q_in, k_in, v_in, gamma_q, gamma_k, rope_cos, rope_sin, Kc, Vc, out, ws});
  if (r == AX_OK) r = check_shape(S, Smax);
  if (r == AX_OK) r = check_eps(eps);
  if (r == AX_OK) r = check_ws(ws, ws_bytes, S, Smax);
  if (r == AX_OK) r = check_device();
  if (r != AX_OK) return r;
  const ax::AttnPlan plan = ax::attn_plan(S, Smax);
  ax::AttnLaunch p{q_in, gamma_q, gamma_k, rope_cos, rope_sin, eps, k_in, v_in, Kc, Vc, out, ws, S, Smax,
                   /*q_norm=*/1};
  return status(ax::launch_attn(plan, p, as_stream(stream)));
}

int ax_expert_layer_attn_noalloc(const uint16_t* q_in, const uint16_t* k_in, const uint16_t* v_in,
                                 const uint16_t* gamma_q, const uint16_t* gamma_k, const float* rope_cos,
                                 const float* rope_sin, float eps, uint16_t* Kc, uint16_t* Vc, int S, int Smax,
                                 uint16_t* out, void* stream) {
  int r = check_ptrs({q_in, k_in, v_in, gamma_q, gamma_k, rope_cos, rope_sin, Kc, Vc, out});
  if (r == AX_OK) r = check_shape(S, Smax);
  if (r == AX_OK) r = check_eps(eps);
  if (r == AX_OK && ax_expert_attn_workspace_bytes(S, Smax) > kNoAllocScratchBytes) r = AX_E_WORKSPACE;
  if (r == AX_OK) r = check_device();
  void* ws = nullptr;
  if (r == AX_OK) r = scratch_ptr(&ws);
  if (r != AX_OK) return r;
  const ax::AttnPlan plan = ax::attn_plan(S, Smax);
  ax::AttnLaunch p{q_in, gamma_q, gamma_k, rope_cos, rope_sin, eps, k_in, v_in, Kc, Vc, out, ws, S, Smax,
                   /*q_norm=*/1};
  return status(ax::launch_attn(plan, p, as_stream(stream)));
}

int ax_expert_layer_attn_split(const uint16_t* q_in, const uint16_t* k_in, const uint16_t* v_in,
                               const uint16_t* gamma_q, const uint16_t* gamma_k, const float* rope_cos,
                               const float* rope_sin, float eps, uint16_t* Kc, uint16_t* Vc, int S, int Smax,
                               void* ws, size_t ws_bytes, void* stream) {
  int r = check_ptrs({q_in, k_in, v_in, gamma_q, gamma_k, rope_cos, rope_sin, Kc, Vc, ws});
  if (r == AX_OK) r = check_shape(S, Smax);
  if (r == AX_OK) r = check_eps(eps);
  if (r == AX_OK) r = check_ws(ws, ws_bytes, S, Smax);
  if (r == AX_OK) r = check_device();
  if (r != AX_OK) return r;
  const ax::AttnPlan plan = ax::attn_plan(S, Smax);
  ax::AttnLaunch p{q_in, gamma_q, gamma_k, rope_cos, rope_sin, eps, k_in, v_in, Kc, Vc, nullptr, ws, S, Smax,
                   /*q_norm=*/1};
  return status(ax::launch_attn_split(plan, p, as_stream(stream)));
}

int ax_expert_attn_combine(const void* ws, size_t ws_bytes, int S, int Smax, uint16_t* out, void* stream) {
  int r = check_ptrs({ws, out});
  if (r == AX_OK) r = check_shape(S, Smax);
  if (r == AX_OK) r = check_ws(ws, ws_bytes, S, Smax);
  if (r == AX_OK) r = check_device();
  if (r != AX_OK) return r;
  return status(ax::launch_attn_combine(ax::attn_plan(S, Smax), ws, out, as_stream(stream)));
}

// ---- fp8 cache ------------------------------------------------------------------------------

size_t ax_expert_attn_fp8_workspace_bytes(int S, int Smax) {
  if (check_shape(S, Smax) != AX_OK) return 0;
  return ax::attn_partials_bytes_f8(ax::attn_plan_f8(S, Smax));
}

static int check_ws_f8(const void* ws, size_t ws_bytes, int S, int Smax) {
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return AX_E_WORKSPACE;
  return ws_bytes >= ax_expert_attn_fp8_workspace_bytes(S, Smax) ? AX_OK : AX_E_WORKSPACE;
}

int ax_cache_tail_write_fp8(const uint16_t* k_roped, const uint16_t* v, uint8_t* Kc8, float* Ks, uint8_t* Vc8,
                            float* Vs, int Smax, void* stream) {
  int r = check_ptrs({k_roped, v, Kc8, Ks, Vc8, Vs});
  if (r == AX_OK) r = check_shape(0, Smax);
  if (r == AX_OK) r = check_device();
  if (r != AX_OK) return r;
  return status(ax::launch_tail_quant_f8(k_roped, v, Kc8, Ks, Vc8, Vs, Smax, as_stream(stream)));
}

int ax_expert_attn_fp8(const uint16_t* q_roped, const uint16_t* k_own, const uint16_t* v_own, uint8_t* Kc8,
                       float* Ks, uint8_t* Vc8, float* Vs, int S, int Smax, uint16_t* out, void* ws,
                       size_t ws_bytes, void* stream) {
  int r = check_ptrs({q_roped, Kc8, Ks, Vc8, Vs, out, ws});
  if (r == AX_OK && ((k_own == nullptr) != (v_own == nullptr))) r = AX_E_NULL;
  if (r == AX_OK && k_own && (!aligned16(k_own) || !aligned16(v_own))) r = AX_E_ALIGN;
  if (r == AX_OK) r = check_shape(S, Smax);
  if (r == AX_OK) r = check_ws_f8(ws, ws_bytes, S, Smax);
  if (r == AX_OK) r = check_device();
  if (r != AX_OK) return r;
  const ax::AttnPlan plan = ax::attn_plan_f8(S, Smax);
  ax::AttnLaunchF8 p{q_roped, nullptr, nullptr, nullptr, nullptr, 0.f, k_own, v_own, Kc8, Ks, Vc8, Vs, out, ws,
                     S, Smax, /*q_norm=*/0};
  return status(ax::launch_attn_f8(plan, p, as_stream(stream)));
}

static int check_layer_f8(const uint16_t* q_in, const uint16_t* k_in, const uint16_t* v_in, const uint16_t* gamma_q,
                          const uint16_t* gamma_k, const float* rope_cos, const float* rope_sin, float eps,
                          uint8_t* Kc8, float* Ks, uint8_t* Vc8, float* Vs, int S, int Smax, void* ws,
                          size_t ws_bytes) {
  int r = check_ptrs({q_in, k_in, v_in, gamma_q, gamma_k, rope_cos, rope_sin, Kc8, Ks, Vc8, Vs, ws});
  if (r == AX_OK) r = check_shape(S, Smax);
  if (r == AX_OK) r = check_eps(eps);
  if (r == AX_OK) r = check_ws_f8(ws, ws_bytes, S, Smax);
  if (r == AX_OK) r = check_device();
  return r;
}

int ax_expert_layer_attn_fp8(const uint16_t* q_in, const uint16_t* k_in, const uint16_t* v_in,
                             const uint16_t* gamma_q, const uint16_t* gamma_k, const float* rope_cos,
                             const float* rope_sin, float eps, uint8_t* Kc8, float* Ks, uint8_t* Vc8, float* Vs,
                             int S, int Smax, uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  int r = out == nullptr ? AX_E_NULL : aligned16(out) ? AX_OK : AX_E_ALIGN;
  if (r == AX_OK)
    r = check_layer_f8(q_in, k_in, v_in, gamma_q, gamma_k, rope_cos, rope_sin, eps, Kc8, Ks, Vc8, Vs, S, Smax, ws,
                       ws_bytes);
  if (r != AX_OK) return r;
  const ax::AttnPlan plan = ax::attn_plan_f8(S, Smax);
  ax::AttnLaunchF8 p{q_in, gamma_q, gamma_k, rope_cos, rope_sin, eps, k_in, v_in, Kc8, Ks, Vc8, Vs, out, ws,
                     S, Smax, /*q_norm=*/1};
  return status(ax::launch_attn_f8(plan, p, as_stream(stream)));
}

int ax_expert_layer_attn_fp8_split(const uint16_t* q_in, const uint16_t* k_in, const uint16_t* v_in,
                                   const uint16_t* gamma_q, const uint16_t* gamma_k, const float* rope_cos,
                                   const float* rope_sin, float eps, uint8_t* Kc8, float* Ks, uint8_t* Vc8,
                                   float* Vs, int S, int Smax, void* ws, size_t ws_bytes, void* stream) {
  const int r = check_layer_f8(q_in, k_in, v_in, gamma_q, gamma_k, rope_cos, rope_sin, eps, Kc8, Ks, Vc8, Vs, S,
                               Smax, ws, ws_bytes);
  if (r != AX_OK) return r;
  const ax::AttnPlan plan = ax::attn_plan_f8(S, Smax);
  ax::AttnLaunchF8 p{q_in, gamma_q, gamma_k, rope_cos, rope_sin, eps, k_in, v_in, Kc8, Ks, Vc8, Vs, nullptr, ws,
                     S, Smax, /*q_norm=*/1};
  return status(ax::launch_attn_f8_split(plan, p, as_stream(stream)));
}

int ax_expert_attn_fp8_combine(const void* ws, size_t ws_bytes, int S, int Smax, uint16_t* out, void* stream) {
  int r = check_ptrs({ws, out});
  if (r == AX_OK) r = check_shape(S, Smax);
  if (r == AX_OK) r = check_ws_f8(ws, ws_bytes, S, Smax);
  if (r == AX_OK) r = check_device();
  if (r != AX_OK) return r;
  return status(ax::launch_attn_f8_combine(ax::attn_plan_f8(S, Smax), ws, out, as_stream(stream)));
}

// ---- text-model decode step -------------------------------------------------------------------

size_t ax_text_decode_workspace_bytes(int pos, int Smax) {
  if (Smax < 1 || Smax > AX_SMAX_LIMIT || pos < 0 || pos >= Smax) return 0;
  return ax::decode_partials_bytes(ax::decode_plan(pos));
}

int ax_text_decode_attn(const uint16_t* q_in, const uint16_t* k_in, const uint16_t* v_in, const uint16_t* gamma_q,
                        const uint16_t* gamma_k, const float* rope_cos, const float* rope_sin, float eps,
                        uint16_t* Kc, uint16_t* Vc, int pos, int Smax, uint16_t* out, void* ws, size_t ws_bytes,
                        void* stream) {
  int r = check_ptrs({q_in, k_in, v_in, gamma_q, gamma_k, rope_cos, rope_sin, Kc, Vc, out, ws});
  if (r == AX_OK && (Smax < 1 || Smax > AX_SMAX_LIMIT || pos < 0 || pos >= Smax)) r = AX_E_SHAPE;
  if (r == AX_OK) r = check_eps(eps);
  if (r == AX_OK && ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0 || ws_bytes < ax_text_decode_workspace_bytes(pos, Smax)))
    r = AX_E_WORKSPACE;
  if (r == AX_OK) r = check_device();
  if (r != AX_OK) return r;
  ax::DecodeLaunch p{q_in, k_in, v_in, gamma_q, gamma_k, rope_cos, rope_sin, eps, Kc, Vc, out, ws, pos, Smax};
  return status(ax::launch_decode(ax::decode_plan(pos), p, as_stream(stream)));
}

// ---- the whole expert layer ------------------------------------------------------------------------

int ax_pack_weight_m64(const uint16_t* W, int K, int N, uint16_t* W_packed, void* stream) {
  int r = check_ptrs({W, W_packed});
  if (r == AX_OK && (!ax::gemm64_shape_ok(K, N) || K > (1 << 20) || N > (1 << 20))) r = AX_E_SHAPE;
  if (r == AX_OK) r = check_device();
  if (r != AX_OK) return r;
  return status(ax::launch_pack_w64(W, K, N, W_packed, as_stream(stream)));
}

size_t ax_linear_m64_workspace_bytes(int K, int N) {
  return ax::gemm64_shape_ok(K, N) ? ax::gemm64_partials_bytes(K, N) : 0;
}

int ax_linear_m64(const uint16_t* A, const uint16_t* W, int K, int N, uint16_t* C, void* ws, size_t ws_bytes,
                  void* stream) {
  int r = check_ptrs({A, W, C, ws});
  if (r == AX_OK && (!ax::gemm64_shape_ok(K, N) || K > (1 << 20) || N > (1 << 20))) r = AX_E_SHAPE;
  if (r == AX_OK && ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0 || ws_bytes < ax_linear_m64_workspace_bytes(K, N)))
    r = AX_E_WORKSPACE;
  if (r == AX_OK) r = check_device();
  if (r != AX_OK) return r;
  return status(ax::launch_linear64(A, W, K, N, C, ws, as_stream(stream)));
}

size_t ax_expert_layer_workspace_bytes(int S, int Smax) {
  if (check_shape(S, Smax) != AX_OK) return 0;
  return ax::layer_workspace_bytes(S, Smax);
}

int ax_expert_layer(const uint16_t* x_in, const uint16_t* ln1, const uint16_t* wqkv, const uint16_t* q_norm_w,
                    const uint16_t* k_norm_w, const uint16_t* wo, const uint16_t* ln2, const uint16_t* w1,
                    const uint16_t* w3, const uint16_t* w2, const float* rope_cos, const float* rope_sin, float eps,
                    uint16_t* Kc, uint16_t* Vc, int S, int Smax, uint16_t* x_out, void* ws, size_t ws_bytes,
                    void* stream) {
  int r = check_ptrs({x_in, ln1, wqkv, q_norm_w, k_norm_w, wo, ln2, w1, w3, w2, rope_cos, rope_sin, Kc, Vc, x_out, ws});
  if (r == AX_OK) r = check_shape(S, Smax);
  if (r == AX_OK) r = check_eps(eps);
  if (r == AX_OK && ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0 || ws_bytes < ax_expert_layer_workspace_bytes(S, Smax)))
    r = AX_E_WORKSPACE;
  if (r == AX_OK) r = check_device();
  if (r != AX_OK) return r;
  ax::LayerLaunch p{x_in, ln1, wqkv, q_norm_w, k_norm_w, wo, ln2, w1, w3, w2, rope_cos, rope_sin, eps, Kc, Vc, S, Smax,
                    x_out, ws};
  return status(ax::launch_layer(p, as_stream(stream)));
}

static bool overlap(const void* a, const void* b, size_t n) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return a && b && (x < y ? y - x < n : x - y < n);
}

int ax_expert_layer_chained(const uint16_t* x_in, const uint16_t* n1_in, const uint16_t* ln1, const uint16_t* wqkv,
                            const uint16_t* q_norm_w, const uint16_t* k_norm_w, const uint16_t* wo,
                            const uint16_t* ln2, const uint16_t* w1, const uint16_t* w3, const uint16_t* w2,
                            const float* rope_cos, const float* rope_sin, float eps, uint16_t* Kc, uint16_t* Vc,
                            int S, int Smax, uint16_t* x_out, const uint16_t* ln1_next, uint16_t* n1_out, void* ws,
                            size_t ws_bytes, void* stream) {
  int r = check_ptrs({x_in, wqkv, q_norm_w, k_norm_w, wo, ln2, w1, w3, w2, rope_cos, rope_sin, Kc, Vc, x_out, ws});
  if (r == AX_OK && n1_in == nullptr && ln1 == nullptr) r = AX_E_NULL;  // the first norm needs ln1
  if (r == AX_OK && (ln1_next == nullptr) != (n1_out == nullptr)) r = AX_E_NULL;
  if (r == AX_OK) r = check_ptrs({n1_in, ln1, ln1_next, n1_out}, /*allow_null=*/true);
  if (r == AX_OK) r = check_shape(S, Smax);
  if (r == AX_OK) r = check_eps(eps);
  const size_t act = (size_t)AX_N_TOK * 1536 * 2;
  if (r == AX_OK && (overlap(x_in, x_out, act) || overlap(n1_out, x_in, act) || overlap(n1_out, x_out, act) ||
                     overlap(n1_out, n1_in, act)))
    r = AX_E_ARG;
  if (r == AX_OK && ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0 || ws_bytes < ax_expert_layer_workspace_bytes(S, Smax)))
    r = AX_E_WORKSPACE;
  if (r == AX_OK) r = check_device();
  if (r != AX_OK) return r;
  ax::LayerLaunch p{x_in, ln1, wqkv, q_norm_w, k_norm_w, wo, ln2, w1, w3, w2, rope_cos, rope_sin, eps, Kc, Vc, S, Smax,
                    x_out, ws, n1_in, ln1_next, n1_out};
  return status(ax::launch_layer(p, as_stream(stream)));
}

int ax_copy_words(const void* src, void* dst, size_t n_words16, void* stream) {
  int r = check_ptrs({src, dst});
  if (r == AX_OK) r = check_device();
  if (r != AX_OK) return r;
  return status(ax::launch_copy_words(src, dst, n_words16, as_stream(stream)));
}

}  // extern "C"
