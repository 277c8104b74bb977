// The fp8 cache's stand-alone tail write: the own k (roped) and v rows quantised per row into the
// cache tail, codes and scales. The fp8 attention step itself is the bf16 split kernel's fp8
// instantiation (ax_attn.hip): its loader waves convert each landed block of codes once into a
// bf16 tile and the compute waves apply the row scales in float32.
//
// What is computed: page code/alpamayo_tt/expert.py, TTExpert.layer with the 8-bit cache the pages
// offer as an option (TTExpert.__init__, the kv_cache dtype map; page
// code/alpamayo_tt/EXPERT_NOTES.md, the bfp8-cache row of the decode attention timing): the cache
// value of row j is e4m3(code) * scale_j, with scale = max |x| / 448 per row and the code the
// nearest-even, saturating e4m3 rounding of x / scale (float32 divisions).
#include "ax_attn_common.h"
#include "ax_launch.h"

namespace ax {

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

hipError_t launch_tail_quant_f8(const uint16_t* k, const uint16_t* v, uint8_t* Kc, float* Ks, uint8_t* Vc,
                                float* Vs, int Smax, hipStream_t st) {
  hipLaunchKernelGGL(k_tail_quant_f8, dim3(2 * kHkv * kT * 16 / 256), dim3(256), 0, st, k, v, Kc, Ks, Vc, Vs, Smax);
  return hipGetLastError();
}

}  // namespace ax
