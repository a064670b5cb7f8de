// ngq_bf16.h -- bf16 conversions shared by the device code of libngq (not
// installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ngq {
namespace dev {

// fp32 -> bf16 bit pattern, rounded to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// bf16 pattern -> fp64, decoded from the fields (no fp32 step, so subnormal
// inputs do not depend on the fp32 denormal mode)
__device__ __forceinline__ double bf16_bits_to_f64(uint32_t b) {
  const uint32_t ex = (b >> 7) & 0xFFu, man = b & 0x7Fu;
  double v;
  if (ex == 0xFFu)
    v = man ? __builtin_nan("") : __builtin_inf();
  else
    v = ex ? ldexp((double)(128u + man), (int)ex - 134) : ldexp((double)man, -133);
  return (b & 0x8000u) ? -v : v;
}

// bf16 nearest-even rounding of an fp64 value, taken directly from fp64 (no
// intermediate fp32 rounding).  With a in [2^E, 2^(E+1)) the bf16 ulp is
// 2^u, u = max(E, -126) - 7 (8 significant bits; below 2^-126 the subnormal
// ulp 2^-133).  m = rint(a / 2^u) is the significand in ulps, rounded with
// ties to even (the scaling is by a power of two, exact); the pattern is then
// ((u + 133) << 7) + m, which also covers m = 256 (carry into the next binade)
// and the subnormals (u = -133).  Inputs here are finite with |v| <= sqrt(N).
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double v) {
  const uint32_t sign = signbit(v) ? 0x8000u : 0u;  // -0 keeps its sign
  const double a = fabs(v);
  if (a == 0.0) return (uint16_t)sign;
  int e;
  (void)frexp(a, &e);  // a = f 2^e with f in [0.5, 1), so E = e - 1
  const int u = max(e - 1, -126) - 7;
  const uint32_t m = (uint32_t)rint(ldexp(a, -u));
  return (uint16_t)((((uint32_t)(u + 133) << 7) + m) | sign);
}

}  // namespace dev
}  // namespace ngq
