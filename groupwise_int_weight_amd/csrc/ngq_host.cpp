// ngq_host.cpp -- host-only part of libngq: sizes, validation, the bit-plane
// packer and status strings.  Nothing in this file calls the HIP runtime, so
// every function here also works on a machine without a GPU.
#include <string.h>

#include <vector>

#include "ngq_internal.h"

namespace ngq {

int parse_format(int bits, int group, Format* f) {
  if (group != kGroup) return NGQ_ERR_UNSUPPORTED;
  if (bits & ~(0xFF | NGQ_SCALE_BF16)) return NGQ_ERR_UNSUPPORTED;
  int w = bits & 0xFF;
  if (w != 4 && w != 5 && w != 8) return NGQ_ERR_UNSUPPORTED;
  f->bits = w;
  f->scale_bf16 = (bits & NGQ_SCALE_BF16) != 0;
  return NGQ_OK;
}

size_t p0_bytes(int K, int N, int bits) {
  size_t kn = (size_t)K * (size_t)N;
  return bits == 8 ? kn : kn / 2;
}

size_t p1_bytes(int K, int N, int bits) { return bits == 5 ? (size_t)K * (size_t)N / 8 : 0; }

int check_kn(int K, int N) {
  if (K < 0 || N < 0 || K % kGroup != 0 || N % 4 != 0) return NGQ_ERR_SHAPE;
  return NGQ_OK;
}

int check_ptr(const void* p) {
  if (!p) return NGQ_ERR_ARG;
  if (((uintptr_t)p) & 15) return NGQ_ERR_ALIGN;
  return NGQ_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

}  // namespace ngq

using namespace ngq;

extern "C" size_t ngq_packed_bytes(int K, int N, int bits, int group) {
  Format f;
  if (parse_format(bits, group, &f) != NGQ_OK || check_kn(K, N) != NGQ_OK) return 0;
  return p0_bytes(K, N, f.bits) + p1_bytes(K, N, f.bits);
}

extern "C" size_t ngq_scale_bytes(int K, int N, int bits, int group) {
  Format f;
  if (parse_format(bits, group, &f) != NGQ_OK || check_kn(K, N) != NGQ_OK) return 0;
  return (size_t)(K / kGroup) * (size_t)N * 2;
}

// The packer builds one row of words at a time: for a row of P0 (or P1) it
// ORs each of the 8 (4, 32) source code rows into the row of words, so the
// codes are read row-major exactly once.
extern "C" int ngq_pack(int K, int N, int bits, int group, const int8_t* codes, void* wq_out) {
  Format f;
  int rc = parse_format(bits & ~NGQ_SCALE_BF16, group, &f);
  if (rc != NGQ_OK) return rc;
  if ((rc = check_kn(K, N)) != NGQ_OK) return rc;
  size_t total = p0_bytes(K, N, f.bits) + p1_bytes(K, N, f.bits);
  if (total == 0) return NGQ_OK;
  if (!codes || !wq_out) return NGQ_ERR_ARG;
  const int lo = -(1 << (f.bits - 1)), hi = (1 << (f.bits - 1)) - 1;
  const size_t kn = (size_t)K * N;
  for (size_t i = 0; i < kn; ++i)
    if (codes[i] < lo || codes[i] > hi) return NGQ_ERR_ARG;

  uint8_t* out = static_cast<uint8_t*>(wq_out);
  std::vector<uint32_t> row((size_t)N);
  const int per_word = f.bits == 8 ? 4 : 8;  // codes per P0 word along K
  const int field = f.bits == 8 ? 8 : 4;     // bits per P0 field
  const int bias = 1 << (f.bits - 1);
  const uint32_t fmask = f.bits == 8 ? 0xFFu : 0xFu;
  for (int kb = 0; kb < K / per_word; ++kb) {
    std::fill(row.begin(), row.end(), 0u);
    for (int i = 0; i < per_word; ++i) {
      const int8_t* src = codes + (size_t)(kb * per_word + i) * N;
      const int sh = field * i;
      for (int n = 0; n < N; ++n) row[n] |= ((uint32_t)(src[n] + bias) & fmask) << sh;
    }
    memcpy(out + (size_t)kb * N * 4, row.data(), (size_t)N * 4);
  }
  if (f.bits == 5) {
    uint8_t* p1 = out + p0_bytes(K, N, 5);
    for (int kb = 0; kb < K / 32; ++kb) {
      std::fill(row.begin(), row.end(), 0u);
      for (int i = 0; i < 32; ++i) {
        const int8_t* src = codes + (size_t)(kb * 32 + i) * N;
        for (int n = 0; n < N; ++n) row[n] |= (((uint32_t)(src[n] + 16) >> 4) & 1u) << i;
      }
      memcpy(p1 + (size_t)kb * N * 4, row.data(), (size_t)N * 4);
    }
  }
  return NGQ_OK;
}

extern "C" const char* ngq_strerror(int status) {
  switch (status) {
    case NGQ_OK: return "ok";
    case NGQ_ERR_ARG: return "invalid argument (null pointer, overlapping output or code out of range)";
    case NGQ_ERR_SHAPE: return "unsupported shape (T out of range for the call, K % 64 != 0 or N % 4 != 0)";
    case NGQ_ERR_UNSUPPORTED: return "unsupported format (bits 4/5/8, group 64, buffers < 2 GiB)";
    case NGQ_ERR_ALIGN: return "buffer not 16-byte aligned";
    case NGQ_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

extern "C" int ngq_version(void) { return 1; }
