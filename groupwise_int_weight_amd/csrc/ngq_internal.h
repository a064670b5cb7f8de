// ngq_internal.h -- shared host-side declarations of libngq (not installed).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "ngq.h"

namespace ngq {

constexpr int kGroup = 64;
constexpr size_t kMaxBuffer = (size_t)1 << 31;  // every buffer < 2 GiB (32-bit buffer offsets)

struct Format {
  int bits = 0;          // 4, 5 or 8
  bool scale_bf16 = false;
};

// Parse `bits` (width | NGQ_SCALE_BF16).  Returns NGQ_OK or NGQ_ERR_UNSUPPORTED.
int parse_format(int bits, int group, Format* f);

// Byte sizes of the packed planes for a K x N matrix (valid shapes only).
size_t p0_bytes(int K, int N, int bits);
size_t p1_bytes(int K, int N, int bits);

// Shape check shared by every entry point: K >= 0, K % 64 == 0, N >= 0, N % 4 == 0.
int check_kn(int K, int N);

// 16-byte alignment and non-null.
int check_ptr(const void* p);

// True when [a, a+na) and [b, b+nb) overlap.
bool overlaps(const void* a, size_t na, const void* b, size_t nb);

// The split-K closing kernel of ngq_gemm_rescale (ngq_rescale.hip): y = the
// slice-order sum of the S fp32 slice sums partial[S][T][N] (then + res, the
// bf16 residual [T][N], when res is not null) rounded to bf16, and x = the
// RMS rescale of y, bit for bit as ngq_rms_rescale(T, N, y, x).  Only for
// 1 <= S <= 8 and rows that reduce_rescale_fits (else NGQ_ERR_UNSUPPORTED);
// arguments are not checked further.
bool reduce_rescale_fits(int N);
int launch_reduce_rescale(const float* partial, int S, int T, int N, void* y, void* x, const void* res,
                          void* stream);

}  // namespace ngq
