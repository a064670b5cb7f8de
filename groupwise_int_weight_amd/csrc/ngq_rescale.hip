// ngq_rescale.hip -- per-token RMS rescale of a bf16 activation block.
//
//   x[t][n] = bf16( z[t][n] / sqrt( (1/N) sum_n z[t][n]^2 ) ),  a zero row -> zeros
//
// It chains the output of one stacked layer into the next at unit scale.  The
// pages do not describe such a step; it carries no epsilon and no learned
// weight.  The arithmetic is fp64 throughout and the result is rounded once,
// to nearest even, from the fp64 quotient, so the only difference from an
// exact evaluation is the summation order of the squares (each square of a
// bf16 value is exact in fp64).  The block is T x N with T <= 8 in the decode
// path, so the kernel is latency bound: one workgroup handles one row, or,
// unless the call is in place, eight workgroups share it.
#include <hip/hip_runtime.h>

#include "ngq_internal.h"

namespace ngq {
namespace dev {

typedef uint32_t r32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowThreads = 256;

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

// One row per workgroup.  VEC: rows start 16-byte aligned (N % 8 == 0), so the
// row is read in 8-element chunks.
template <bool VEC>
__global__ __launch_bounds__(kRowThreads) void rms_rescale_kernel(const uint16_t* z, uint16_t* x, int N) {
  const size_t row = (size_t)blockIdx.x * (size_t)N;
  const uint16_t* zr = z + row;
  uint16_t* xr = x + row;
  double ss = 0.0;
  if constexpr (VEC) {
    const r32x4* z8 = reinterpret_cast<const r32x4*>(zr);
    for (int c = threadIdx.x; c < N / 8; c += kRowThreads) {
      const r32x4 w = z8[c];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const double lo = bf16_bits_to_f64(w[j]), hi = bf16_bits_to_f64(w[j] >> 16);
        ss += lo * lo;
        ss += hi * hi;
      }
    }
  } else {
    for (int n = threadIdx.x; n < N; n += kRowThreads) {
      const double v = bf16_bits_to_f64(zr[n]);
      ss += v * v;
    }
  }
  // fixed-order tree: within the wave by xor shuffles, then the four wave sums
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  __shared__ double wsum[kRowThreads / 64];
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
  __syncthreads();
  const double tot = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  const double r = sqrt(tot / (double)N);
  // All of the row was read before the barrier, so in-place use (x == z) is safe.
  if constexpr (VEC) {
    const r32x4* z8 = reinterpret_cast<const r32x4*>(zr);
    r32x4* x8 = reinterpret_cast<r32x4*>(xr);
    for (int c = threadIdx.x; c < N / 8; c += kRowThreads) {
      const r32x4 w = z8[c];
      r32x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = r > 0.0 ? f64_to_bf16_rne(bf16_bits_to_f64(w[j]) / r) : 0u;
        const uint32_t hi = r > 0.0 ? f64_to_bf16_rne(bf16_bits_to_f64(w[j] >> 16) / r) : 0u;
        o[j] = lo | (hi << 16);
      }
      x8[c] = o;
    }
  } else {
    for (int n = threadIdx.x; n < N; n += kRowThreads)
      xr[n] = r > 0.0 ? f64_to_bf16_rne(bf16_bits_to_f64(zr[n]) / r) : (uint16_t)0;
  }
}

// The same result with each row spread over S workgroups (grid S x T): every
// workgroup reads the whole row and computes the same fixed-order sum of
// squares (so all slices use the same bits of r), then scales only its own
// 1/S of the row.  The per-element work of a row then runs on S CUs instead
// of one.  Not for in-place use: a slice written early could be read by
// another workgroup's first pass.
template <int S>
__global__ __launch_bounds__(kRowThreads) void rms_rescale_split_kernel(const uint16_t* z, uint16_t* x, int N) {
  const size_t row = (size_t)blockIdx.y * (size_t)N;
  const r32x4* z8 = reinterpret_cast<const r32x4*>(z + row);
  r32x4* x8 = reinterpret_cast<r32x4*>(x + row);
  const int nch = N / 8;
  double ss = 0.0;
  for (int c = threadIdx.x; c < nch; c += kRowThreads) {
    const r32x4 w = z8[c];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double lo = bf16_bits_to_f64(w[j]), hi = bf16_bits_to_f64(w[j] >> 16);
      ss += lo * lo;
      ss += hi * hi;
    }
  }
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  __shared__ double wsum[kRowThreads / 64];
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
  __syncthreads();
  const double tot = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  const double r = sqrt(tot / (double)N);
  const int per = (nch + S - 1) / S;
  const int c0 = blockIdx.x * per, c1 = min(c0 + per, nch);
  for (int c = c0 + threadIdx.x; c < c1; c += kRowThreads) {
    const r32x4 w = z8[c];
    r32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = r > 0.0 ? f64_to_bf16_rne(bf16_bits_to_f64(w[j]) / r) : 0u;
      const uint32_t hi = r > 0.0 ? f64_to_bf16_rne(bf16_bits_to_f64(w[j] >> 16) / r) : 0u;
      o[j] = lo | (hi << 16);
    }
    x8[c] = o;
  }
}

}  // namespace dev
}  // namespace ngq

using namespace ngq;

extern "C" int ngq_rms_rescale(int T, int N, const void* z, void* x, void* stream) {
  if (T < 0 || T > 65535 || N < 0 || N > (1 << 24)) return NGQ_ERR_SHAPE;
  if (T == 0 || N == 0) return NGQ_OK;
  int rc;
  if ((rc = check_ptr(z)) != NGQ_OK) return rc;
  if ((rc = check_ptr(x)) != NGQ_OK) return rc;
  const size_t bytes = (size_t)T * (size_t)N * 2u;
  if (bytes >= kMaxBuffer) return NGQ_ERR_UNSUPPORTED;
  if (x != z && overlaps(x, bytes, z, bytes)) return NGQ_ERR_ARG;
  hipStream_t st = (hipStream_t)stream;
  const uint16_t* zi = static_cast<const uint16_t*>(z);
  uint16_t* xo = static_cast<uint16_t*>(x);
  if (N % 8 == 0 && x != z && N >= 8 * 64 * 8)
    hipLaunchKernelGGL(dev::rms_rescale_split_kernel<8>, dim3(8u, (unsigned)T), dim3(dev::kRowThreads), 0, st, zi, xo,
                       N);
  else if (N % 8 == 0)
    hipLaunchKernelGGL(dev::rms_rescale_kernel<true>, dim3((unsigned)T), dim3(dev::kRowThreads), 0, st, zi, xo, N);
  else
    hipLaunchKernelGGL(dev::rms_rescale_kernel<false>, dim3((unsigned)T), dim3(dev::kRowThreads), 0, st, zi, xo, N);
  return hipGetLastError() == hipSuccess ? NGQ_OK : NGQ_ERR_HIP;
}
