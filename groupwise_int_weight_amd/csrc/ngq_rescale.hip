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
// unless the call is in place, eight workgroups share it.  The same row
// kernel also closes a split-K projection (ngq_gemm_rescale): it adds the
// slices' fp32 sums, rounds them to the projection's bf16 output and rescales
// that, in one launch.
#include <hip/hip_runtime.h>

#include "ngq_bf16.h"
#include "ngq_internal.h"

namespace ngq {
namespace dev {

typedef uint32_t r32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowThreads = 256;

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

// Rows spread over several workgroups.  Grid R x T: workgroup (j, t) builds
// the whole of row t as bf16 words in LDS, computing the fixed-order sum of
// squares on the way (so every workgroup of the row gets the same bits of r),
// then writes its own 1/R of the row's chunks, one word (two elements) per
// thread.  Not for in-place use: a slice written early could be read by
// another workgroup's first pass.  The row comes either from a bf16 block z
// (ngq_rms_rescale) or from the fp32 slice sums of a split-K projection, which
// are added in slice order and rounded to bf16 first (the projection's own
// output, written here too): one chunk -> thread mapping and one order of the
// squares serve both, so a fused call gives the bits ngq_rms_rescale gives
// for the same row.
constexpr int kSplitRowThreads = 1024;
constexpr int kRowParts = 8;  // workgroups per row

// squares of the eight bf16 of a 16-byte chunk, in element order
__device__ __forceinline__ void add_squares(const r32x4 w, double& ss) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const double lo = bf16_bits_to_f64(w[j]), hi = bf16_bits_to_f64(w[j] >> 16);
    ss += lo * lo;
    ss += hi * hi;
  }
}

// r = sqrt(mean square) from the per-thread sums: xor-shuffle tree in each
// wave, then the wave sums in wave order.  Contains the workgroup barrier.
__device__ __forceinline__ double row_rms(double ss, int N) {
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  __shared__ double wsum[kSplitRowThreads / 64];
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
  __syncthreads();
  double tot = wsum[0];
#pragma unroll
  for (int i = 1; i < kSplitRowThreads / 64; ++i) tot += wsum[i];
  return sqrt(tot / (double)N);
}

// this workgroup's 1/kRowParts of the row, from the LDS words: x = z / r
// rounded to bf16 (zeros for a zero row), and z itself when y is given
__device__ __forceinline__ void write_part(const uint32_t* zw, int nch, double r, uint32_t* y, uint32_t* x) {
  const int per = (nch + kRowParts - 1) / kRowParts;
  const int c0 = blockIdx.x * per, c1 = min(c0 + per, nch);
  for (int i = 4 * c0 + (int)threadIdx.x; i < 4 * c1; i += kSplitRowThreads) {
    const uint32_t w = zw[i];
    if (y) y[i] = w;
    const uint32_t lo = r > 0.0 ? f64_to_bf16_rne(bf16_bits_to_f64(w) / r) : 0u;
    const uint32_t hi = r > 0.0 ? f64_to_bf16_rne(bf16_bits_to_f64(w >> 16) / r) : 0u;
    x[i] = lo | (hi << 16);
  }
}

// z bf16 [T][N] -> x; N % 8 == 0; 2 N bytes of dynamic LDS
__global__ __launch_bounds__(kSplitRowThreads) void rms_rescale_split_kernel(const uint16_t* z, uint16_t* x, int N) {
  extern __shared__ r32x4 zrow[];
  const size_t row = (size_t)blockIdx.y * (size_t)N;
  const r32x4* z8 = reinterpret_cast<const r32x4*>(z + row);
  const int nch = N / 8;
  double ss = 0.0;
  for (int c = threadIdx.x; c < nch; c += kSplitRowThreads) {
    const r32x4 w = z8[c];
    zrow[c] = w;
    add_squares(w, ss);
  }
  const double r = row_rms(ss, N);
  write_part(reinterpret_cast<const uint32_t*>(zrow), nch, r, nullptr, reinterpret_cast<uint32_t*>(x + row));
}

// partial fp32 [S][T][N] -> y = bf16(partial[0] + ... + partial[S-1]) (slice
// order, as the split-K reduction) and x = the rescale of y; N % 8 == 0; 2 N
// bytes of dynamic LDS.  All S loads of a chunk are issued before the adds.
// RES: the residual r (bf16 [T][N]) is added to the fp32 sum last, before its
// one rounding: y = bf16(partial[0] + ... + partial[S-1] + r).
template <int S, bool RES>
__global__ __launch_bounds__(kSplitRowThreads) void reduce_rescale_kernel(const float* __restrict__ partial,
                                                                          const uint16_t* __restrict__ res, int T,
                                                                          int N, uint16_t* y, uint16_t* x) {
  extern __shared__ r32x4 zrow[];
  const size_t row = (size_t)blockIdx.y * (size_t)N, TN = (size_t)T * (size_t)N;
  const float4* p4 = reinterpret_cast<const float4*>(partial + row);
  const int nch = N / 8;
  double ss = 0.0;
  for (int c = threadIdx.x; c < nch; c += kSplitRowThreads) {
    float4 lo[S], hi[S];
#pragma unroll
    for (int ks = 0; ks < S; ++ks) {
      lo[ks] = p4[ks * (TN / 4) + 2 * c];
      hi[ks] = p4[ks * (TN / 4) + 2 * c + 1];
    }
    r32x4 rv = {0u, 0u, 0u, 0u};
    if constexpr (RES) rv = reinterpret_cast<const r32x4*>(res + row)[c];
    float4 a = lo[0], b = hi[0];
#pragma unroll
    for (int ks = 1; ks < S; ++ks) {
      a.x += lo[ks].x; a.y += lo[ks].y; a.z += lo[ks].z; a.w += lo[ks].w;
      b.x += hi[ks].x; b.y += hi[ks].y; b.z += hi[ks].z; b.w += hi[ks].w;
    }
    if constexpr (RES) {
      // a bf16 value is the upper half of its fp32 value
      a.x += __uint_as_float(rv[0] << 16); a.y += __uint_as_float(rv[0] & 0xFFFF0000u);
      a.z += __uint_as_float(rv[1] << 16); a.w += __uint_as_float(rv[1] & 0xFFFF0000u);
      b.x += __uint_as_float(rv[2] << 16); b.y += __uint_as_float(rv[2] & 0xFFFF0000u);
      b.z += __uint_as_float(rv[3] << 16); b.w += __uint_as_float(rv[3] & 0xFFFF0000u);
    }
    r32x4 w;
    w[0] = f32_to_bf16_rne(a.x) | ((uint32_t)f32_to_bf16_rne(a.y) << 16);
    w[1] = f32_to_bf16_rne(a.z) | ((uint32_t)f32_to_bf16_rne(a.w) << 16);
    w[2] = f32_to_bf16_rne(b.x) | ((uint32_t)f32_to_bf16_rne(b.y) << 16);
    w[3] = f32_to_bf16_rne(b.z) | ((uint32_t)f32_to_bf16_rne(b.w) << 16);
    zrow[c] = w;
    add_squares(w, ss);
  }
  const double r = row_rms(ss, N);
  write_part(reinterpret_cast<const uint32_t*>(zrow), nch, r, reinterpret_cast<uint32_t*>(y + row),
             reinterpret_cast<uint32_t*>(x + row));
}

}  // namespace dev
}  // namespace ngq

namespace ngq {

// Rows long enough to spread over kRowParts workgroups, whose bf16 copy fits
// the LDS a workgroup may take without an attribute change (64 KB, with the
// kernel's own 64 bytes).
static bool split_rows(int N) { return N % 8 == 0 && N >= 4096 && N <= 30720; }

bool reduce_rescale_fits(int N) { return split_rows(N); }

template <int S>
static void launch_rr(const float* partial, const void* res, int T, int N, void* y, void* x, hipStream_t st) {
  const dim3 grid((unsigned)dev::kRowParts, (unsigned)T), block(dev::kSplitRowThreads);
  const uint32_t lds = (uint32_t)N * 2u;
  const uint16_t* r = static_cast<const uint16_t*>(res);
  uint16_t* yy = static_cast<uint16_t*>(y);
  uint16_t* xx = static_cast<uint16_t*>(x);
  if (res != nullptr)
    hipLaunchKernelGGL((dev::reduce_rescale_kernel<S, true>), grid, block, lds, st, partial, r, T, N, yy, xx);
  else
    hipLaunchKernelGGL((dev::reduce_rescale_kernel<S, false>), grid, block, lds, st, partial, r, T, N, yy, xx);
}

int launch_reduce_rescale(const float* partial, int S, int T, int N, void* y, void* x, const void* res,
                          void* stream) {
  if (!split_rows(N)) return NGQ_ERR_UNSUPPORTED;
  hipStream_t st = (hipStream_t)stream;
  switch (S) {
    case 1: launch_rr<1>(partial, res, T, N, y, x, st); break;
    case 2: launch_rr<2>(partial, res, T, N, y, x, st); break;
    case 3: launch_rr<3>(partial, res, T, N, y, x, st); break;
    case 4: launch_rr<4>(partial, res, T, N, y, x, st); break;
    case 5: launch_rr<5>(partial, res, T, N, y, x, st); break;
    case 6: launch_rr<6>(partial, res, T, N, y, x, st); break;
    case 7: launch_rr<7>(partial, res, T, N, y, x, st); break;
    case 8: launch_rr<8>(partial, res, T, N, y, x, st); break;
    default: return NGQ_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? NGQ_OK : NGQ_ERR_HIP;
}

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
  if (split_rows(N) && x != z)
    hipLaunchKernelGGL(dev::rms_rescale_split_kernel, dim3((unsigned)dev::kRowParts, (unsigned)T),
                       dim3(dev::kSplitRowThreads), (uint32_t)N * 2u, st, zi, xo, N);
  else if (N % 8 == 0)
    hipLaunchKernelGGL(dev::rms_rescale_kernel<true>, dim3((unsigned)T), dim3(dev::kRowThreads), 0, st, zi, xo, N);
  else
    hipLaunchKernelGGL(dev::rms_rescale_kernel<false>, dim3((unsigned)T), dim3(dev::kRowThreads), 0, st, zi, xo, N);
  return hipGetLastError() == hipSuccess ? NGQ_OK : NGQ_ERR_HIP;
}
