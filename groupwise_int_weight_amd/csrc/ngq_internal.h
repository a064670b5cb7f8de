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

}  // namespace ngq
