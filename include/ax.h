/*
 * ax.h - C ABI of the MI355X (gfx950) expert-attention library (libax.so).
 *
 * One layer of the Alpamayo2-Super flow-matching action expert's attention
 * step, as described on page code/alpamayo_tt/expert.py (TTExpert.layer and
 * TTExpert.attention_core) and page code/alpamayo_tt/EXPERT_NOTES.md
 * (sections "Layouts" and "Attention over the VLM cache: masking approach"):
 *
 *   64 expert tokens, 16 query heads, 8 GQA kv heads, head_dim 128.
 *   q and the expert's own k get per-head RMSNorm (eps 1e-6) and HF
 *   rotate_half RoPE (theta 5e6, positions S + rope_delta + i); the own roped
 *   K and the raw own V overwrite rows [Smax-64, Smax) of the layer's KV cache;
 *   the 128 folded query rows of each kv head (2 q heads x 64 tokens) attend
 *   non-causally to cache rows [0, S) and [Smax-64, Smax) - the rows an
 *   additive 0/-1e9 mask leaves visible - with scale 1/sqrt(128).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Shapes are fixed by the model: Hq = 16, Hkv = 8, T = 64, D = 128.
 * - bf16 tensors are passed as uint16_t bit patterns. All tensors are dense,
 *   row-major, in device memory owned by the caller, 16-byte aligned:
 *     q        [16][64][128]   (q head h, token i)
 *     k, v     [8][64][128]    (kv head g, token i)
 *     gamma    [128]
 *     Kc, Vc   [8][Smax][128]  (kv head g, cache row j), 256 bytes per row
 *     out      [16][64][128]   per-head attention output before the head concat
 *   Folded view: row r of kv head g is q head 2g + r/64, token r % 64, so q,
 *   out and any [8][128][128] view of them are the same bytes.
 * - RoPE tables are float32 [64][64] in device memory: table[i][j] is
 *   cos (or sin) of (S + rope_delta + i) * theta^(-2j/128); column j serves
 *   both j and j + 64 (rotate_half layout). ax_rope_tables() fills them.
 * - 0 <= S <= Smax - 64 and 64 <= Smax <= AX_SMAX_LIMIT. Rows [S, Smax-64)
 *   are never read: any contents are allowed there.
 * - `stream` is a hipStream_t (NULL = the null stream). Calls only enqueue
 *   work: nothing is synchronised, nothing is allocated, no host memory is
 *   touched except where stated. Launch is asynchronous; faults surface at
 *   the next synchronisation of the stream.
 * - Return value: AX_OK (0) = enqueued; a negative AX_E_* code = the
 *   arguments were rejected on the host before anything was enqueued or
 *   written; a positive value = the hipError_t of a failed launch.
 * - Calls on the same cache/workspace buffers must be ordered on one stream
 *   (or synchronised); the library keeps no state between calls besides a
 *   per-device record of whether the device is a gfx950 and the debug wait
 *   limit (ax_debug_set_wait_limit).
 * - Workspace status word: the first 4 bytes of the workspace of every
 *   attention entry point (bf16 and fp8 cache, decode, whole layer) are an
 *   int32 status word (the first 256 bytes are reserved for it). The kernels OR AX_STATUS_* flags into it and never clear it; the
 *   rest of a workspace holds scratch whose contents on entry do not matter.
 *   A caller that wants the status zeroes the word once and reads it back
 *   after synchronising. AX_STATUS_WAIT_EXPIRED: a workgroup's bounded wait
 *   for an in-workgroup hand-off gave up (by default after about 30 ms of
 *   polling, thousands of times any real wait); the workgroup finishes anyway,
 *   the affected split's result is NaN, and the output must not be trusted.
 */
#ifndef AX_H
#define AX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AX_ABI_VERSION 1

#define AX_N_Q_HEADS 16
#define AX_N_KV_HEADS 8
#define AX_N_TOK 64
#define AX_HEAD_DIM 128
#define AX_SMAX_LIMIT (1 << 20)

enum {
  AX_OK = 0,
  AX_E_NULL = -1,        /* a required pointer is NULL */
  AX_E_SHAPE = -2,       /* S < 0, S > Smax - 64, Smax < 64 or Smax > AX_SMAX_LIMIT, bad n_tok/head_dim */
  AX_E_ALIGN = -3,       /* a device pointer is not 16-byte aligned */
  AX_E_WORKSPACE = -4,   /* workspace smaller than ax_expert_attn_workspace_bytes() */
  AX_E_UNSUPPORTED = -5, /* current device is not a gfx950, or no device */
  AX_E_ARG = -6          /* another invalid scalar (eps < 0 or not finite, theta <= 0, ...) */
};

#define AX_STATUS_WAIT_EXPIRED 1

/* ABI version of the loaded library (AX_ABI_VERSION). */
int ax_abi_version(void);

/*
 * Debug setting, process-wide: the number of polls after which a bounded
 * in-workgroup wait gives up, for launches enqueued after the call
 * (0 = the default). A tiny limit makes waits give up early, so that the
 * AX_STATUS_WAIT_EXPIRED path can be exercised without a hang; results are
 * then wrong by design. AX_E_ARG for polls < 0.
 */
int ax_debug_set_wait_limit(int polls);

/* Static text for a return code of any entry point (never NULL). */
const char* ax_strerror(int code);

/*
 * Host function: RoPE tables for the n_tok positions pos0 + i
 * (pos0 = S + rope_delta; page code/alpamayo_tt/expert.py, TTExpert.set_context,
 * and EXPERT_NOTES.md, table "Layouts", row "cos / sin").
 * cos_h, sin_h: HOST float arrays [n_tok][head_dim/2], written as the float32
 * rounding of values computed in double precision. head_dim must be even and
 * positive, n_tok positive, theta > 0, pos0 >= 0. No device work.
 */
int ax_rope_tables(int pos0, int n_tok, int head_dim, double theta, float* cos_h, float* sin_h);

/*
 * q/k RMSNorm + RoPE (the q_norm, k_norm, rope q and rope k ops of
 * TTExpert.layer, page code/alpamayo_tt/expert.py).
 * q_out[h][i][:] = bf16(rope(gamma_q * q_in / sqrt(mean(q_in^2) + eps)))
 * k_out likewise with gamma_k; arithmetic in float32, one rounding at the
 * store (nearest-even). q_out may equal q_in and k_out may equal k_in
 * (exact aliasing only). Shapes: q [16][64][128], k [8][64][128].
 */
int ax_qk_norm_rope(const uint16_t* q_in, const uint16_t* k_in, const uint16_t* gamma_q,
                    const uint16_t* gamma_k, const float* rope_cos, const float* rope_sin, float eps,
                    uint16_t* q_out, uint16_t* k_out, void* stream);

/*
 * Tail write (the two fill_cache calls of TTExpert.layer at row Smax - 64,
 * page code/alpamayo_tt/expert.py; EXPERT_NOTES.md, "masking approach").
 * Kc[g][Smax-64+i][:] = k_roped[g][i][:], Vc[g][Smax-64+i][:] = v[g][i][:],
 * bit-exact copies; every other cache row is left untouched.
 */
int ax_cache_tail_write(const uint16_t* k_roped, const uint16_t* v, uint16_t* Kc, uint16_t* Vc,
                        int Smax, void* stream);

/*
 * Fused RMSNorm + RoPE + tail write in one launch: q_out as ax_qk_norm_rope,
 * the roped k goes straight into Kc rows [Smax-64, Smax) and v into Vc rows
 * [Smax-64, Smax) (bit-identical to ax_qk_norm_rope followed by
 * ax_cache_tail_write).
 */
int ax_qk_norm_rope_tail(const uint16_t* q_in, const uint16_t* k_in, const uint16_t* v_in,
                         const uint16_t* gamma_q, const uint16_t* gamma_k, const float* rope_cos,
                         const float* rope_sin, float eps, uint16_t* q_out, uint16_t* Kc,
                         uint16_t* Vc, int Smax, void* stream);

/*
 * Bytes of caller-owned device workspace that ax_expert_attn and
 * ax_expert_layer_attn need for (S, Smax): the status word, then the
 * per-split partials (O in float16 scaled by a power of two per row and
 * 32-column quarter, with the exponents; running maxima and row sums in
 * float32). 0 if (S, Smax) is invalid.
 */
size_t ax_expert_attn_workspace_bytes(int S, int Smax);

/*
 * Attention of the 128 folded rows of each kv head over cache rows [0, S)
 * and [Smax-64, Smax) (TTExpert.attention_core in decode mode, page
 * code/alpamayo_tt/expert.py; the mask of TTExpert.build_mask is implied by S
 * and Smax: the hidden rows are skipped, not read).
 * q_roped: [16][64][128] bf16, already normed and roped.
 * If k_own and v_own are both non-NULL, the tail write (k_own is the ROPED
 * own k) is done first; if both are NULL the tail is taken as already
 * written; exactly one NULL is AX_E_NULL.
 * out: [16][64][128] bf16 (nearest-even rounding of the float32 result).
 * Arithmetic: bf16 products on the matrix cores, float32 accumulation,
 * float32 softmax and split combine; the split partials pass through
 * float16 with a power-of-two scale per (row, 32-column quarter), which keeps
 * 11 significant bits of every element within 2^14 of its quarter's largest
 * |value|. ws: workspace of at least ax_expert_attn_workspace_bytes(S, Smax)
 * bytes, 256-byte aligned; apart from the status word its contents on entry
 * do not matter and on return are unspecified.
 */
int ax_expert_attn(const uint16_t* q_roped, const uint16_t* k_own, const uint16_t* v_own,
                   uint16_t* Kc, uint16_t* Vc, int S, int Smax, uint16_t* out, void* ws,
                   size_t ws_bytes, void* stream);

/*
 * The whole attention step of one layer: the result of ax_qk_norm_rope_tail
 * followed by ax_expert_attn on its roped q (k_own = v_own = NULL), bit for
 * bit, in two launches (norm + RoPE + tail write + split attention in one
 * kernel, then the combine). Updates the cache tail of Kc/Vc and writes out
 * [16][64][128]. Inputs as above.
 */
int ax_expert_layer_attn(const uint16_t* q_in, const uint16_t* k_in, const uint16_t* v_in,
                         const uint16_t* gamma_q, const uint16_t* gamma_k, const float* rope_cos,
                         const float* rope_sin, float eps, uint16_t* Kc, uint16_t* Vc, int S,
                         int Smax, uint16_t* out, void* ws, size_t ws_bytes, void* stream);

/*
 * ax_expert_layer_attn for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): no workspace
 * argument, and no allocation of any kind. The partials live in a static
 * 16 MiB device array of the library, one per GPU, held until the process
 * ends, so (S, Smax) whose ax_expert_attn_workspace_bytes exceeds 16 MiB
 * (S > 18880) are AX_E_WORKSPACE. Nothing in that array needs to start at
 * zero: each call writes every partial it reads; its status word is not
 * reported (a wait that gives up still leaves NaN in the output). All calls on
 * one GPU share the array, so calls that overlap on one GPU (on different
 * streams, unordered) race and give wrong results; order them on one stream.
 * Output, cache update and arithmetic are those of ax_expert_layer_attn, bit
 * for bit.
 */
int ax_expert_layer_attn_noalloc(const uint16_t* q_in, const uint16_t* k_in, const uint16_t* v_in,
                                 const uint16_t* gamma_q, const uint16_t* gamma_k,
                                 const float* rope_cos, const float* rope_sin, float eps,
                                 uint16_t* Kc, uint16_t* Vc, int S, int Smax, uint16_t* out,
                                 void* stream);

/*
 * The two launches of ax_expert_layer_attn, for callers that time or order
 * them separately (same pages and passages as above).
 * ax_expert_layer_attn_split: q/k RMSNorm, RoPE, the cache tail write and the
 * split attention; every split's partial (unnormalised O in scaled float16
 * with its exponents, running max and row sum in float32) is left in ws.
 * ax_expert_attn_combine: the log-sum-exp
 * combine of the partials in ws for the same (S, Smax) into out. The two in
 * this order on one stream with the same ws equal ax_expert_layer_attn. The
 * combine reads only ws; it is undefined unless the split call for (S, Smax)
 * ran before it on ws.
 */
int ax_expert_layer_attn_split(const uint16_t* q_in, const uint16_t* k_in, const uint16_t* v_in,
                               const uint16_t* gamma_q, const uint16_t* gamma_k,
                               const float* rope_cos, const float* rope_sin, float eps,
                               uint16_t* Kc, uint16_t* Vc, int S, int Smax, void* ws,
                               size_t ws_bytes, void* stream);
int ax_expert_attn_combine(const void* ws, size_t ws_bytes, int S, int Smax, uint16_t* out,
                           void* stream);

/*
 * fp8 KV cache. The pages offer an 8-bit cache for the same step (page
 * code/alpamayo_tt/expert.py, TTExpert.__init__, the kv_cache dtype map;
 * page code/alpamayo_tt/EXPERT_NOTES.md, the bfp8-cache row of the decode
 * attention timing). Here a cache row is 128 OCP e4m3 codes ("fn": bias 7,
 * no infinities, 0x7F/0xFF NaN, max 448) with one float32 scale:
 *   Kc8, Vc8 [8][Smax][128] uint8 (128 bytes per row), Ks, Vs [8][Smax] float
 *   value of element (g, j, d) = e4m3(Kc8[g][j][d]) * Ks[g][j]
 * Own rows written into the tail are quantised per row:
 *   scale = max_d |x_d| / 448 (1.0 for an all-zero row),
 *   code_d = e4m3 nearest-even, saturating to +-448, of x_d / scale,
 * both divisions in float32; x is the bf16 roped own k, or the bf16 own v.
 * Pointers as for the bf16 cache (16-byte aligned device memory owned by the
 * caller); the other conventions above apply unchanged.
 */

/* Workspace bytes of the fp8 calls for (S, Smax); 0 if invalid. */
size_t ax_expert_attn_fp8_workspace_bytes(int S, int Smax);

/*
 * Tail write into an fp8 cache: rows (g, i) of k_roped and v [8][64][128]
 * bf16 quantised by the rule above into Kc8/Ks and Vc8/Vs row Smax - 64 + i.
 * Every other row and scale is left untouched.
 */
int ax_cache_tail_write_fp8(const uint16_t* k_roped, const uint16_t* v, uint8_t* Kc8, float* Ks,
                            uint8_t* Vc8, float* Vs, int Smax, void* stream);

/*
 * ax_expert_attn over an fp8 cache: if k_own/v_own (roped k, v; bf16) are
 * both non-NULL their quantised rows are written to the tail first, if both
 * are NULL the tail is taken as already written. Scores and the value sum use
 * the dequantised rows: the key codes meet q on the fp8 matrix cores, q as
 * two e4m3 parts whose sum is its bf16 row scaled by a power of two (exact
 * down to 2^-10 of the row's largest element, within 2^-17 of it below); each
 * value code is converted exactly to bf16 for the bf16 matrix cores. The key
 * scales multiply the float32 scores and the value scales (times a fixed
 * 2^64, taken back out in the combine) the float32 softmax weights before
 * they are rounded to bf16; value scales from the float32 denormals up to
 * 2^25 keep those products in bf16's normal range.
 * ws: at least ax_expert_attn_fp8_workspace_bytes(S, Smax) bytes, 256-byte
 * aligned (the status word, then partials in the bf16 cache's layout, with
 * longer key ranges).
 */
int ax_expert_attn_fp8(const uint16_t* q_roped, const uint16_t* k_own, const uint16_t* v_own,
                       uint8_t* Kc8, float* Ks, uint8_t* Vc8, float* Vs, int S, int Smax,
                       uint16_t* out, void* ws, size_t ws_bytes, void* stream);

/*
 * The whole attention step of one layer over an fp8 cache (ax_expert_layer_attn
 * with the tail quantised): q/k RMSNorm + RoPE, the own rows quantised into the
 * tail (k after rounding the roped k to bf16), attention, combine; two launches.
 * The _split / _combine pair are those two launches, as for the bf16 cache.
 */
int ax_expert_layer_attn_fp8(const uint16_t* q_in, const uint16_t* k_in, const uint16_t* v_in,
                             const uint16_t* gamma_q, const uint16_t* gamma_k, const float* rope_cos,
                             const float* rope_sin, float eps, uint8_t* Kc8, float* Ks, uint8_t* Vc8,
                             float* Vs, int S, int Smax, uint16_t* out, void* ws, size_t ws_bytes,
                             void* stream);
int ax_expert_layer_attn_fp8_split(const uint16_t* q_in, const uint16_t* k_in, const uint16_t* v_in,
                                   const uint16_t* gamma_q, const uint16_t* gamma_k,
                                   const float* rope_cos, const float* rope_sin, float eps,
                                   uint8_t* Kc8, float* Ks, uint8_t* Vc8, float* Vs, int S, int Smax,
                                   void* ws, size_t ws_bytes, void* stream);
int ax_expert_attn_fp8_combine(const void* ws, size_t ws_bytes, int S, int Smax, uint16_t* out,
                               void* stream);

/*
 * Text-model decode step (page code/alpamayo_tt/text.py,
 * TTTextModel._layer_decode from the q/k norms to the attention output): the
 * VLM's text layers have 64 query heads and 8 kv heads of width 128. One new
 * token at cache position pos:
 *   q_in [64][128], k_in and v_in [8][128] bf16 (raw, after the qkv
 *   projection); gamma_q, gamma_k [128]; rope_cos, rope_sin float32 [64]:
 *   cos / sin of (pos + rope_delta) * theta^(-2j/128), j = 0..63 (the one-token
 *   table of ax_rope_tables(pos + rope_delta, 1, 128, theta, ...)).
 * q and k are RMSNormed per head (eps) and roped in float32; the roped k
 * (rounded to bf16) and v_in are written into row pos of Kc and Vc
 * [8][Smax][128]; query head h attends to rows [0, pos] of kv head h / 8 with
 * scale 1/sqrt(128); out [64][128] bf16. Rows after pos are never read; every
 * row except pos is left untouched. 0 <= pos < Smax <= AX_SMAX_LIMIT.
 * ws: at least ax_text_decode_workspace_bytes(pos, Smax) bytes, 256-byte
 * aligned; apart from the status word its contents on entry do not matter.
 * Two launches (split attention, combine).
 */
size_t ax_text_decode_workspace_bytes(int pos, int Smax);
int ax_text_decode_attn(const uint16_t* q_in, const uint16_t* k_in, const uint16_t* v_in,
                        const uint16_t* gamma_q, const uint16_t* gamma_k, const float* rope_cos,
                        const float* rope_sin, float eps, uint16_t* Kc, uint16_t* Vc, int pos,
                        int Smax, uint16_t* out, void* ws, size_t ws_bytes, void* stream);

/*
 * One whole action-expert decoder layer, the pages' layer_fn(i, x, K, V) -> x
 * (page code/alpamayo_tt/EXPERT_NOTES.md, section "Layouts": the per-layer op
 * list and the weight shapes; page code/alpamayo_tt/expert.py, TTExpert.layer):
 *   n1 = RMSNorm(x; ln1), qkv = n1 wqkv split into q heads 0..15, k heads 0..7,
 *   v heads 0..7 (columns 128 h .. 128 h + 127 of each block), the attention
 *   step of ax_expert_layer_attn on them (q_norm_w / k_norm_w are its gammas),
 *   heads concatenated, x2 = x + attn wo, n2 = RMSNorm(x2; ln2),
 *   x_out = x2 + (silu(n2 w1) * (n2 w3)) w2.
 * x_in, x_out [64][1536]; ln1, ln2 [1536]; weights input-major (the transpose
 * of the HF layout, as the pages store them): wqkv [1536][4096], wo
 * [2048][1536], w1 and w3 [1536][6144], w2 [6144][1536]; all bf16, each passed
 * through ax_pack_weight_m64 once beforehand. Every op
 * hands a bf16 tensor to the next (rounded to nearest even); inside an op the
 * arithmetic is float32 (products of bf16 on the matrix cores). Updates the
 * cache tail like ax_expert_layer_attn. x_out must not alias x_in. ws: at least
 * ax_expert_layer_workspace_bytes(S, Smax) bytes, 256-byte aligned, starting
 * with the status word. Nine launches.
 */
size_t ax_expert_layer_workspace_bytes(int S, int Smax);
int ax_expert_layer(const uint16_t* x_in, const uint16_t* ln1, const uint16_t* wqkv,
                    const uint16_t* q_norm_w, const uint16_t* k_norm_w, const uint16_t* wo,
                    const uint16_t* ln2, const uint16_t* w1, const uint16_t* w3, const uint16_t* w2,
                    const float* rope_cos, const float* rope_sin, float eps, uint16_t* Kc, uint16_t* Vc,
                    int S, int Smax, uint16_t* x_out, void* ws, size_t ws_bytes, void* stream);

/*
 * ax_expert_layer for layers run one after another, the output residual of
 * one the input of the next (the expert's stack of decoder layers; page
 * code/alpamayo_tt/expert.py, TTExpert, whose forward calls the layer function
 * once per layer). The first norm of a layer then runs in the previous
 * layer's last launch:
 * - n1_in: NULL, or RMSNorm(x_in; ln1) [64][1536] as the previous call wrote it
 *   to its n1_out; the first norm is then skipped and ln1 is not read (it may
 *   be NULL).
 * - ln1_next, n1_out: both NULL, or the next layer's ln1 [1536] and a
 *   [64][1536] buffer that receives RMSNorm(x_out; ln1_next), written by the
 *   launch that writes x_out.
 * Every other argument as for ax_expert_layer. x_out and n1_out are the bits
 * ax_expert_layer gives for the same inputs (and n1_out the bits its first
 * norm gives on x_out). AX_E_NULL if exactly one of ln1_next / n1_out is NULL,
 * or if n1_in and ln1 are both NULL; AX_E_ARG if n1_out overlaps x_in, x_out or
 * n1_in, or x_out overlaps x_in. A caller keeps two n1 buffers and alternates
 * them. Eight launches with n1_in, nine without.
 */
int ax_expert_layer_chained(const uint16_t* x_in, const uint16_t* n1_in, const uint16_t* ln1,
                            const uint16_t* wqkv, const uint16_t* q_norm_w, const uint16_t* k_norm_w,
                            const uint16_t* wo, const uint16_t* ln2, const uint16_t* w1,
                            const uint16_t* w3, const uint16_t* w2, const float* rope_cos,
                            const float* rope_sin, float eps, uint16_t* Kc, uint16_t* Vc, int S,
                            int Smax, uint16_t* x_out, const uint16_t* ln1_next, uint16_t* n1_out,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * Weight packing for the projections: W [K][N] bf16, input-major, into W_packed
 * (same size, a separate buffer) in the layout the projection kernel streams:
 * 4 KB blocks of 32 rows x 64 columns, the blocks of one 64-column tile
 * consecutive, so that each workgroup reads one contiguous range. A one-time
 * step when weights are loaded. K a multiple of 128, N of 64.
 */
int ax_pack_weight_m64(const uint16_t* W, int K, int N, uint16_t* W_packed, void* stream);

/*
 * The layer's projection on its own: C[64][N] = bf16(A[64][K] W[K][N]) for 64
 * rows (bf16 A and W, W input-major and packed by ax_pack_weight_m64, float32
 * accumulation). K a multiple of 128, N of 64. ws:
 * ax_linear_m64_workspace_bytes(K, N) bytes (float32 split partials), 256-byte
 * aligned.
 */
size_t ax_linear_m64_workspace_bytes(int K, int N);
int ax_linear_m64(const uint16_t* A, const uint16_t* W, int K, int N, uint16_t* C, void* ws,
                  size_t ws_bytes, void* stream);

/*
 * Measurement helper: dst[i] = src[i] for n 16-byte words, one plain
 * streaming copy kernel. Used to calibrate hardware byte counters against a
 * transfer of known size. Pointers 16-byte aligned.
 */
int ax_copy_words(const void* src, void* dst, size_t n_words16, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AX_H */
