// ngq_gemm.hip -- gfx950 kernels of libngq and their C entry points.
//
// The projection Y[T x N] = X[T x K] . dequant(Wq[K x N]) for T <= 8 tokens
// (the small-batch Q4/Q5 projections whose T=8 routing the NInfer-4090 V3
// topic, section "What V3 did", tunes for the GDN projection, the attention
// Q5 projection and the SwiGLU path).  The pages give the operation and its
// single-operator timings on an RTX 4090 ("Measured data"), not a kernel; the
// design below is written for CDNA4.
//
// Work decomposition.  A workgroup owns a tile of 16*V output columns over the
// whole K (or several such tiles, one after another), so no partial sum ever
// leaves the workgroup and the result is deterministic.  Its waves share K in
// units of 128-k group pairs, either interleaved (wave w takes pairs w, w + W,
// ..., so the waves move through K together) or handed out by an LDS counter,
// and meet once per tile in LDS, where the partials are summed in a fixed
// order.  V (1..4 columns per lane) is picked per shape so that the tiles
// fill the 256 CUs in whole rounds, with tiles of at least 32 columns where N
// allows; consecutive tiles go to the same XCD (workgroup b runs on XCD
// b % 8), so neighbouring columns that share a cache line share an L2.  Two
// kernels implement this: gemm_kernel loads each pair's X with its weights,
// gemm_xres_kernel stages X in LDS once; the host picks one per shape.
//
// Inner step.  The path streams packed weights once from HBM and is bandwidth
// bound, but at T=8 a VALU-only dot product would need ~4.5 VALU lane-ops per
// weight against ~3.7 available at 70 % of HBM peak, so the multiply-add runs
// on the matrix cores: v_mfma_f32_16x16x32_bf16 with A = 16 weight columns x
// 32 k, B = 32 k x 16 "slots".  T <= 8 fills only half of the 16 slots, so
// slot j = t + 8h carries token t restricted to the first (h = 0) or second
// (h = 1) group of a pair of 64-k groups: one MFMA chain then yields separate
// per-group partial sums for two groups at once, which is what the per-group
// scale needs, at no cost in MFMA issue.
//
// Unpack without subtraction.  A code field u (0..31) becomes the bf16 value
// 128 + u by placing u in the low mantissa bits under the exponent byte 0x43.
// The wanted code is c = u - bias, so sum_k x (128 + u) over-counts by
// (128 + bias) sum_k x; that term comes from one extra MFMA per step with a
// constant A = -(128 + bias), which seeds each group's partial sum.  int8
// fields are converted exactly with v_cvt_f32_ubyte and their bias (128) is
// removed the same way.  Each group partial is then scaled in fp32:
// acc += s[g][n] * partial, so no rounded weight*scale product is ever formed.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <deque>
#include <mutex>
#include <queue>
#include <tuple>
#include <type_traits>
#include <utility>
#include <vector>

#include "ngq_bf16.h"
#include "ngq_internal.h"

namespace ngq {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 12 waves (3 per SIMD) with one pair each in flight: measured on MI355X, 12 to
// 16 pairs in flight per CU stream fastest; deeper per-wave pipelines or fewer
// waves congest the memory pipeline or leave it short.
constexpr int kWaves = 12;
constexpr int kThreads = kWaves * 64;
// A buffer offset that is out of range for every buffer (all are < 2 GiB, and
// adding an in-range offset cannot wrap 32 bits).  Out-of-range buffer loads
// return zero without touching memory.
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  // raw buffer (stride 0), 32-bit data format: bounds-checked against `bytes`.
  // Every descriptor is built from kernel arguments, so it is uniform; saying
  // so (readfirstlane) keeps it in scalar registers.  Where the compiler lost
  // track of that it held the descriptor in vector registers and wrapped
  // every load in a loop over the lanes' distinct descriptors.
  // (readfirstlane returns a signed int: each half goes through uint32_t, or
  // the low half would sign-extend into the high one)
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  void* const pu = reinterpret_cast<void*>(((uint64_t)hi << 32) | (uint64_t)lo);
  return __builtin_amdgcn_make_buffer_rsrc(pu, (short)0, __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000);
}

// Cache policy of a buffer load (the instruction's aux bits): 0 default, or
// kNT, the nontemporal hint, for data read once (weights and scales).  On
// MI355X a weights-only stream of the QK tile pattern took 5.76 instead of
// 6.02 us per 22 MB launch with it, the gate/value pattern 9.81 instead of
// 10.06; the coherence-scope bits changed nothing.  In the decode kernels
// (T <= 8) it took 1-7 % off every projection (gate/up + SwiGLU T = 8:
// 26.7 against 27.6 us, split-K down 16.7 against 17.9, the fused launch
// 36.7 against 38.0).
constexpr int kNT = 2;

template <int NW, int AUX = 0>
__device__ __forceinline__ void load_words(uint32_t* d, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (NW == 1) {
    d[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX);
  } else if constexpr (NW == 2) {
    u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX);
    d[0] = v[0]; d[1] = v[1];
  } else if constexpr (NW == 3) {
    u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, AUX);
    d[0] = v[0]; d[1] = v[1]; d[2] = v[2];
  } else if constexpr (NW == 4) {
    u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
    d[0] = v[0]; d[1] = v[1]; d[2] = v[2]; d[3] = v[3];
  } else {
    load_words<4, AUX>(d, r, off);
    load_words<NW - 4, AUX>(d + 4, r, off + 16u);
  }
}

// ---- unpack: one 8-k block of one column -> eight bf16 (128 + u) ----

// Unpack in the interleaved k order: dword j of the result holds k = j (low
// half) and k = j + 4 (high half) of an 8-k block, each as the bf16 value
// 128 + u.  hb: the block's eight 5th bits (bit i for k = i), 0 for int4; they
// are spread to bits 4..7 (k 0..3) and 20..23 (k 4..7) and shifted into
// place with the nibbles.
// The masks come in as values the compiler cannot fold (a kernel argument
// and a vector register): with two literal operands, or two scalar ones, it
// splits each and-or in two, since a three-operand VALU instruction takes no
// literal and at most one scalar operand on this target.
struct UnpackMasks {
  uint32_t nib;   // 0x000F000F
  uint32_t base;  // 0x43004300
  uint32_t hi;    // 0x00100010
};
constexpr UnpackMasks kMasks = {0x000F000Fu, 0x43004300u, 0x00100010u};

__device__ __forceinline__ u32x4 nibbles_to_bf16_il(uint32_t w, const UnpackMasks& mk) {
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = ((w >> (4 * j)) & mk.nib) | mk.base;
  return r;
}

// The 5th bits of k-block b of a high-bit word p1 (its byte b, bit i for
// k = i) spread for nibbles5_to_bf16_il with one byte permute: byte 0 of the
// result is byte b of p1s = p1 << 4 (the block's k 0..3 bits at 4..7), byte 2
// is byte b of p1 (k 4..7 at bits 4..7 of it, so 20..23); bits 0..3 and
// 16..19 carry neighbouring bits that the unpack never reads.  p1s is shared
// by the four blocks of the word; hb_select(b) is the permute's selector.
__host__ __device__ constexpr uint32_t hb_select(uint32_t b) { return b | 0x0C00u | ((4u + b) << 16) | 0x0C000000u; }
__device__ __forceinline__ uint32_t hb_spread(uint32_t p1, uint32_t p1s, uint32_t sel) {
  return __builtin_amdgcn_perm(p1, p1s, sel);
}

// int5: the high bits are first merged into the base pattern, then the
// nibbles; each merge is one three-input bitwise op ((a & b) | c, truth
// table 0xEA), so an output register costs two shifts and two ops.  hs holds
// the block's eight 5th bits spread: k 0..3 at bits 4..7, k 4..7 at bits
// 20..23 (hb_spread); no other bit of it is read.
__device__ __forceinline__ u32x4 nibbles5_to_bf16_il(uint32_t w, uint32_t hs, const UnpackMasks& mk) {
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t hi = __builtin_amdgcn_bitop3_b32(hs >> j, mk.hi, mk.base, 0xEA);
    r[j] = __builtin_amdgcn_bitop3_b32(w >> (4 * j), mk.nib, hi, 0xEA);
  }
  return r;
}

// int8 in the interleaved order: w0 holds k 0..3, w1 k 4..7; each byte u is
// converted exactly (u <= 255 has at most 8 significant bits) and the upper
// halves of the fp32 values are its bf16.
__device__ __forceinline__ u32x4 bytes_to_bf16_il(uint32_t w0, uint32_t w1) {
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo = __float_as_uint((float)((w0 >> (8 * j)) & 0xFFu));
    const uint32_t hi = __float_as_uint((float)((w1 >> (8 * j)) & 0xFFu));
    r[j] = __builtin_amdgcn_perm(hi, lo, 0x07060302u);
  }
  return r;
}

// An X chunk of 8 bf16 (k order 0..7, two per dword) in the interleaved order.
__device__ __forceinline__ u32x4 interleave_x(const uint32_t (&d)[4]) {
  return u32x4{__builtin_amdgcn_perm(d[2], d[0], 0x05040100u), __builtin_amdgcn_perm(d[2], d[0], 0x07060302u),
               __builtin_amdgcn_perm(d[3], d[1], 0x05040100u), __builtin_amdgcn_perm(d[3], d[1], 0x07060302u)};
}

// Two bf16 in a dword.  Taken by value: hipcc turned __builtin_bit_cast of a
// vector element (v[j] of an ext_vector) into a read of element 0.
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2_t, v); }

template <int BITS>
struct Code {
  static constexpr int bias = 1 << (BITS - 1);
  // value of the unpacked bf16 minus the code: 128 + bias for the nibble
  // formats (value 128 + u), bias for int8 (value u)
  static constexpr int offset = BITS == 8 ? bias : 128 + bias;
  // bf16 bit pattern of -offset (exact: 136, 144 and 128 need <= 5 bits)
  static constexpr uint16_t neg_offset_bf16 = BITS == 4 ? 0xC308 : (BITS == 5 ? 0xC310 : 0xC300);
};

__device__ __forceinline__ float scale_to_f32(uint32_t dw, int half, bool bf16) {
  const uint32_t bits = half ? (dw >> 16) : (dw & 0xFFFFu);
  if (bf16) return __uint_as_float(bits << 16);
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

struct GemmArgs {
  const void* x;
  const void* wq;
  const void* scales;
  void* y;
  int T, K;
  int Nout;    // output columns
  int Ncols;   // columns of the packed matrix and of the scales
  int up_off;  // SwiGLU: column offset of the up half (N_ff); 0 otherwise
  int G;       // K / 64
  int pairs;   // ceil(G / 2)
  int ppw;     // pairs per wave
  int ntiles;  // workgroups
  uint32_t p0_bytes, p1_bytes, s_bytes, x_bytes;
  uint32_t mask_nib, mask_base, mask_hi;  // the unpack constants (UnpackMasks)
  // X-resident launches (grid-stride over the tiles): ntiles / grid and
  // ntiles % grid, so that a workgroup's tile count needs no division.  Kept
  // last: inserted after ntiles, they moved the fields above and the
  // per-pair kernel's argument loads with them, which cost 17 % on the
  // gate/value projection (measured).
  int tiles_q, tiles_r;
};

template <int BITS, int V, int NSETS>
struct PairBuf {
  static constexpr int WPK = BITS == 8 ? 2 : 1;  // P0 words per 8-k block and column
  uint32_t a[NSETS][4][V * WPK];                 // [set][step][word]; int8: V words of row 2kb, then 2kb+1
  uint32_t p1[NSETS][2][BITS == 5 ? V : 1];      // int5 high-bit words, one per half pair
  uint32_t x[2][4];                              // X rows of the pair: 2 loads x 16 B per lane
  uint32_t sc[NSETS][2 * V];                     // 4V scales (16-bit) per set
};

// Pairs in flight per wave: one with dynamic assignment (the waves' own count
// supplies the depth), two for the static fallback.
template <bool DYN>
constexpr int pipeline_depth() {
  return DYN ? 1 : 2;
}

// Shared-memory layout of one workgroup: per-wave X staging slots, then (dynamic
// assignment) one partial-sum block per pair and the pair counter, or (static
// assignment) one partial-sum block per wave.
struct Smem {
  // Per-wave staging of the X block of one pair: 8 token rows of 128 k (bf16),
  // rows padded to 272 B against bank conflicts, then a zero block that the
  // lanes of the other group half read at the same step offsets (16 B each at
  // 0, 32, 64, 96), so every lane reads one address without a select.
  static constexpr uint32_t XROW = 272, XZERO = 112, XSLOT = 8 * XROW + XZERO;
  static constexpr uint32_t XS = kWaves * XSLOT;
  // a partial-sum block holds [set][token][column] fp32, token rows padded by
  // 4 floats so the 8 token writes of one column hit distinct banks
  static __host__ __device__ constexpr uint32_t block_floats(int nsets, int tile) {
    return (uint32_t)nsets * 8u * (uint32_t)(tile + 4);
  }
  static __host__ __device__ constexpr uint32_t bytes(bool dyn, int pairs, int nsets, int tile) {
    return XS + (dyn ? (uint32_t)pairs : (uint32_t)kWaves) * block_floats(nsets, tile) * 4u + 16u;
  }
};

template <int BITS, bool SBF16, int V, int NSETS, bool DYN>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs a) {
  constexpr int NB = pipeline_depth<DYN>();
  constexpr int WPK = BITS == 8 ? 2 : 1;
  constexpr int TILE = 16 * V;
  constexpr uint32_t XROW = Smem::XROW, XZERO = Smem::XZERO;
  constexpr uint32_t BLK = Smem::block_floats(NSETS, TILE);
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float* const part = reinterpret_cast<float*>(smem + Smem::XS);
  const int nblk = DYN ? a.pairs : kWaves;
  uint32_t* const counter = reinterpret_cast<uint32_t*>(part + (uint32_t)nblk * BLK);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15;  // operand row / slot index
  const int q = lane >> 4;  // operand k-slot / result row group

  // XCD-aware tile order: XCD x receives workgroups x, x+8, ...; give them
  // consecutive tiles.
  const int b = blockIdx.x;
  const int xcd = b & 7, per = a.ntiles >> 3, rem = a.ntiles & 7;
  const int tile = xcd * per + min(xcd, rem) + (b >> 3);
  const int c0 = tile * TILE;

  const __amdgpu_buffer_rsrc_t rW = make_rsrc(a.wq, a.p0_bytes);
  const __amdgpu_buffer_rsrc_t rP1 = make_rsrc(static_cast<const char*>(a.wq) + a.p0_bytes, a.p1_bytes);
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(a.scales, a.s_bytes);
  // the base pattern lives in a vector register (an empty asm hides its
  // value), so each and-or takes one scalar and one vector constant
  uint32_t vbase = a.mask_base;
  asm volatile("" : "+v"(vbase));
  const UnpackMasks mk{a.mask_nib, vbase, a.mask_hi};

  const uint32_t rowb = (uint32_t)a.Ncols * 4u;  // bytes of one packed row
  // Within a pair (16 k-blocks of 8 k), k-slot q of step s reads k-block
  // 2s + (q & 1) of group (q >> 1): lanes q = 0, 1 serve the first group,
  // q = 2, 3 the second.
  const uint32_t lane_kb = 8u * (uint32_t)(q >> 1) + (uint32_t)(q & 1);
  uint32_t offA[NSETS], offP1[NSETS], offS[NSETS];
  // B slot j = m carries token t = m & 7 for group half h = m >> 3; only the
  // k-slots of that half are non-zero.
  const int t = m & 7, h = m >> 3;
  uint8_t* const xslot = smem + wave * Smem::XSLOT;
#pragma unroll
  for (int s = 0; s < NSETS; ++s) {
    const uint32_t col = (uint32_t)(c0 + s * a.up_off + V * m);
    offA[s] = lane_kb * WPK * rowb + col * 4u;
    offP1[s] = 2u * (uint32_t)(q >> 1) * rowb + col * 4u;
    // result rows 4q..4q+3 of every MFMA -> columns c0 + 4Vq + [0, 4V)
    offS[s] = (uint32_t)h * (uint32_t)a.Ncols * 2u + (uint32_t)(c0 + s * a.up_off + 4 * V * q) * 2u;
  }
  // X block of a pair, read coalesced: load L, lane l -> token 4L + (l >> 4),
  // 8 k at k-block (l & 15) of the pair.  Rows t >= T load nothing (zeros).
  const int xrow = lane >> 4, xkb = lane & 15;
  const uint32_t offX = (uint32_t)xrow * (uint32_t)a.K * 2u + (uint32_t)xkb * 16u;
  const uint32_t rowX4 = 4u * (uint32_t)a.K * 2u;
  const bool x0_on = xrow < a.T, x1_on = xrow + 4 < a.T;
  // B fragment source in the staging slot (the zero block for the other half)
  const bool b_on = (q >> 1) == h;
  const uint32_t bsrc = b_on ? (uint32_t)t * XROW + lane_kb * 16u : 8u * XROW;
  if (lane < XZERO / 16) *reinterpret_cast<u32x4*>(xslot + 8 * XROW + 16u * (uint32_t)lane) = u32x4{0u, 0u, 0u, 0u};
  if constexpr (DYN) {
    if (threadIdx.x == 0) *counter = (uint32_t)(kWaves * NB);
    __syncthreads();
  }

  // Loads of pair p (wave uniform; p >= pairs loads nothing).  Flags are
  // combined bitwise so that no lane-divergent branch appears.
  auto issue = [&](PairBuf<BITS, V, NSETS>& buf, int p) {
    const bool valid = p < a.pairs;
    // last pair of an odd group count: its second group does not exist
    const bool half = (p == a.pairs - 1) & ((a.G & 1) != 0);
    const uint32_t pa = valid ? (uint32_t)p * 16u * WPK * rowb : kOOB;
    const uint32_t pp1 = valid ? (uint32_t)p * 4u * rowb : kOOB;
    const bool xin = valid & !(half & (xkb >= 8));
    const uint32_t px0 = (xin & x0_on) ? (uint32_t)p * 256u + offX : kOOB;
    const uint32_t px1 = (xin & x1_on) ? (uint32_t)p * 256u + offX + rowX4 : kOOB;
    const uint32_t ps = valid ? (uint32_t)p * rowb : kOOB;  // two scale rows of 2-byte entries
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int s = 0; s < NSETS; ++s) {
        const uint32_t o = offA[s] + pa + (uint32_t)st * 2u * WPK * rowb;
        load_words<V, kNT>(&buf.a[s][st][0], rW, o);
        if constexpr (BITS == 8) load_words<V, kNT>(&buf.a[s][st][V], rW, o + rowb);
      }
    }
    load_words<4>(&buf.x[0][0], rX, px0);
    load_words<4>(&buf.x[1][0], rX, px1);
    if constexpr (BITS == 5) {
#pragma unroll
      for (int s = 0; s < NSETS; ++s) {
        load_words<V, kNT>(&buf.p1[s][0][0], rP1, offP1[s] + pp1);
        load_words<V, kNT>(&buf.p1[s][1][0], rP1, offP1[s] + pp1 + rowb);
      }
    }
#pragma unroll
    for (int s = 0; s < NSETS; ++s) load_words<2 * V, kNT>(&buf.sc[s][0], rS, offS[s] + ps);
  };

  f32x4 acc[NSETS][V];
#pragma unroll
  for (int s = 0; s < NSETS; ++s)
#pragma unroll
    for (int i = 0; i < V; ++i) acc[s][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const u32x4 negoff = {Code<BITS>::neg_offset_bf16 * 0x10001u, Code<BITS>::neg_offset_bf16 * 0x10001u,
                        Code<BITS>::neg_offset_bf16 * 0x10001u, Code<BITS>::neg_offset_bf16 * 0x10001u};

  // Slots j and j + 8 hold the two group halves of token j: add them, then the
  // lanes of the first half write the tile block [set][token][column].
  auto store_block = [&](f32x4 (&v)[NSETS][V], float* blk) {
#pragma unroll
    for (int s = 0; s < NSETS; ++s)
#pragma unroll
      for (int i = 0; i < V; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int other = __builtin_amdgcn_mov_dpp(__float_as_int(v[s][i][r]), 0x128 /* row_ror:8 */, 0xF,
                                                     0xF, false);
          v[s][i][r] += __int_as_float(other);
        }
    if (h == 0) {
#pragma unroll
      for (int s = 0; s < NSETS; ++s)
#pragma unroll
        for (int i = 0; i < V; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int col = V * (4 * q + r) + i;
            blk[((uint32_t)s * 8u + (uint32_t)t) * (uint32_t)(TILE + 4) + (uint32_t)col] = v[s][i][r];
          }
    }
  };

  // Multiply one pair.  Dynamic assignment: the pair's scaled partial goes to
  // its own block (the final sum runs over pairs in order, whichever wave did
  // them).  Static assignment: it accumulates into the wave's registers.
  auto compute = [&](const PairBuf<BITS, V, NSETS>& buf, int p) {
    // stage the pair's X rows, then read the four B fragments back (LDS is in
    // order within a wave, so no barrier is needed)
    *reinterpret_cast<u32x4*>(xslot + (uint32_t)xrow * XROW + (uint32_t)xkb * 16u) = interleave_x(buf.x[0]);
    *reinterpret_cast<u32x4*>(xslot + (uint32_t)(xrow + 4) * XROW + (uint32_t)xkb * 16u) = interleave_x(buf.x[1]);
    bf16x8 bfrag[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      bfrag[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xslot + bsrc + (uint32_t)st * 32u));
    }
    // -(128 + bias) * sum_k x over each group half: seeds every partial sum
    f32x4 dx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st)
      dx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, negoff), bfrag[st], dx, 0, 0, 0);
    f32x4 dp[NSETS][V];
#pragma unroll
    for (int s = 0; s < NSETS; ++s)
#pragma unroll
      for (int i = 0; i < V; ++i) dp[s][i] = dx;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int s = 0; s < NSETS; ++s) {
#pragma unroll
        for (int i = 0; i < V; ++i) {
          u32x4 av;
          if constexpr (BITS == 4) {
            av = nibbles_to_bf16_il(buf.a[s][st][i], mk);
          } else if constexpr (BITS == 5) {
            // k-block 2 st + (q & 1) of a 32-k P1 word group: byte 2 (st & 1) + (q & 1)
            const uint32_t p1 = buf.p1[s][st >> 1][i];
            const uint32_t hs = hb_spread(p1, p1 << 4, hb_select(2u * (uint32_t)(st & 1) + (uint32_t)(q & 1)));
            av = nibbles5_to_bf16_il(buf.a[s][st][i], hs, mk);
          } else {
            av = bytes_to_bf16_il(buf.a[s][st][i], buf.a[s][st][V + i]);
          }
          dp[s][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), bfrag[st],
                                                             dp[s][i], 0, 0, 0);
        }
      }
    }
    if constexpr (DYN) {
      f32x4 pv[NSETS][V];
#pragma unroll
      for (int s = 0; s < NSETS; ++s)
#pragma unroll
        for (int i = 0; i < V; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int e = V * r + i;
            pv[s][i][r] = scale_to_f32(buf.sc[s][e >> 1], e & 1, SBF16) * dp[s][i][r];
          }
      store_block(pv, part + (uint32_t)p * BLK);
    } else {
#pragma unroll
      for (int s = 0; s < NSETS; ++s)
#pragma unroll
        for (int i = 0; i < V; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int e = V * r + i;
            const float sc = scale_to_f32(buf.sc[s][e >> 1], e & 1, SBF16);
            acc[s][i][r] = __builtin_fmaf(sc, dp[s][i][r], acc[s][i][r]);
          }
    }
  };

  // NB pairs in flight per wave.  Loads are issued without a branch (a pair
  // past the end loads nothing), so no branch separates a load from its use
  // and the counter wait before each compute covers exactly that pair's loads;
  // the scheduling barriers keep the pairs' loads in issue order.
  PairBuf<BITS, V, NSETS> buf[NB];
  if constexpr (DYN) {
    // Pairs are handed out by a workgroup counter, so waves that get their data
    // sooner (the older waves of each SIMD win issue arbitration) take more of
    // them.  The first NB pairs of each wave are fixed (wave w starts with pairs
    // w, w + 12, ...), the counter hands out the rest.  A wave's pairs come in
    // increasing order and are computed in issue order, so the first
    // out-of-range pair ends the wave's work.
    auto grab = [&](uint32_t n) -> int {
      uint32_t v = 0;
      if (lane == 0) v = __hip_atomic_fetch_add(counter, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      return (int)__builtin_amdgcn_readfirstlane(v);
    };
    int pidx[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      pidx[u] = wave + kWaves * u;
      issue(buf[u], pidx[u]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Only the compute and the counter grab sit under (wave-uniform) branches;
    // the loads do not, or the counter waits would lose their depth.  Once a
    // wave's pairs run out, its remaining slots issue out-of-range loads.
    do {
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const bool live = pidx[u] < a.pairs;
        if (live) compute(buf[u], pidx[u]);
        __builtin_amdgcn_sched_barrier(0);
        pidx[u] = live ? grab(1u) : a.pairs;
        issue(buf[u], pidx[u]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } while (pidx[0] < a.pairs);
  } else {
    // Wave w takes pairs w, w + 12, w + 24, ...: the waves move through K
    // together, so the chip streams a narrow band of weight rows at a time.
    // A slot past the last pair loads nothing and adds zero.
    auto pair_of = [&](int i) { return wave + kWaves * i; };
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      issue(buf[u], pair_of(u));
      __builtin_amdgcn_sched_barrier(0);
    }
    int it = 0;
    for (; it + NB < a.ppw; it += NB) {
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        compute(buf[u], pair_of(it + u));
        __builtin_amdgcn_sched_barrier(0);
        issue(buf[u], pair_of(it + u + NB));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // the last (up to NB) pairs are already in flight: no more loads
#pragma unroll
    for (int u = 0; u < NB; ++u)
      if (it + u < a.ppw && pair_of(it + u) < a.pairs) compute(buf[u], pair_of(it + u));
    store_block(acc, part + (uint32_t)wave * BLK);
  }
  __syncthreads();

  // Sum the blocks (pairs, or waves) in a fixed order, round, store
  // (consecutive threads write consecutive columns of one token row).
  uint16_t* y = static_cast<uint16_t*>(a.y);
  for (int idx = threadIdx.x; idx < 8 * TILE; idx += kThreads) {
    const int tt = idx / TILE, col = idx % TILE;
    if (tt >= a.T || c0 + col >= a.Nout) continue;
    float v[NSETS];
#pragma unroll
    for (int s = 0; s < NSETS; ++s) {
      const float* src = part + ((uint32_t)s * 8u + (uint32_t)tt) * (uint32_t)(TILE + 4) + (uint32_t)col;
      float sum = 0.f;
      for (int k = 0; k < nblk; ++k) sum += src[(uint32_t)k * BLK];
      v[s] = sum;
    }
    float out;
    if constexpr (NSETS == 2) {
      out = v[0] * v[1] / (1.0f + expf(-v[0]));  // SiLU(gate) * up
    } else {
      out = v[0];
    }
    y[(size_t)tt * a.Nout + c0 + col] = f32_to_bf16_rne(out);
  }
}

// ---- X-resident kernel ------------------------------------------------------
//
// The activations X (T x K bf16, at most 80 KB for K = 5120) are staged in LDS
// once per workgroup, so the loop over group pairs issues only weight and
// scale loads.  X is stored with each 8-k block in the order k = 0, 4, 1, 5,
// 2, 6, 3, 7, the order in which the unpack produces weights.
//
// A workgroup may own several tiles (tile r, r + G, ... for its rank r among
// G workgroups); X stays resident across them and the pair stream runs on
// across a tile boundary, so the next tile's first loads are in flight while
// a tile is reduced and stored.  Wave w takes pairs w, w + W, w + 2W, ... of
// every tile, NB of them in flight, so the waves of a workgroup move through K
// together; each wave accumulates its pairs in registers and the waves'
// partials are summed in wave order, so results do not depend on timing.

// LDS of the X-resident kernel: a zero block (bytes 0..127, read by the lanes
// whose B slot belongs to the other group half or to a token >= T), the token
// rows of X (row stride 2K + 16 bytes, so the 8 rows of one k offset fall in
// distinct banks), then one partial-sum block per wave.
struct XSmem {
  static constexpr uint32_t ZERO = 128;
  static __host__ __device__ constexpr uint32_t xrow(int K) { return 2u * (uint32_t)K + 16u; }
  static __host__ __device__ constexpr uint32_t x_end(int T, int K) { return ZERO + (uint32_t)T * xrow(K); }
  static __host__ __device__ constexpr uint32_t bytes(int T, int K, int waves, int nsets, int tile) {
    return x_end(T, K) + (uint32_t)waves * Smem::block_floats(nsets, tile) * 4u;
  }
};

// Workgroup barrier that orders LDS only.  __syncthreads() also makes the
// wave's earlier global stores visible, which on this target waits for every
// outstanding vector memory operation, loads included; the weight loads in
// flight across a tile boundary must not be drained that way.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int BITS, int V, int NSETS>
struct WBuf {
  static constexpr int WPK = BITS == 8 ? 2 : 1;
  uint32_t a[NSETS][4][V * WPK];
  uint32_t p1[NSETS][2][BITS == 5 ? V : 1];
  uint32_t sc[NSETS][2 * V];
};

// The per-lane constants of an X-resident workgroup: operand row m and k-slot
// q, B slot token t and group half h, whether that slot is live, and where in
// LDS its B fragments start.
struct XresLane {
  int wave, m, q, t, h;
  uint32_t lane_kb;
  bool b_on;
  uint32_t bsrc;
  UnpackMasks mk;
};

// One projection as the tile runner sees it.
struct ProjView {
  const void* wq;
  const void* scales;
  void* y;
  uint32_t p0_bytes, p1_bytes, s_bytes;
  int Nout, Ncols, up_off;
};

// Shape constants shared by every projection of a launch.  K is the length
// of the X rows in LDS: the whole K, or a K slice of pairs p0 .. pend - 1
// (split K); G and pairs count the groups and pairs of the whole K.
struct XresShape {
  int T, K, G, pairs, ppw, p0, pend;
};

__device__ __forceinline__ XresLane xres_lane(int T, int K, uint32_t mask_nib, uint32_t mask_base, uint32_t mask_hi) {
  XresLane ln;
  const int lane = threadIdx.x & 63;
  ln.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  ln.m = lane & 15;
  ln.q = lane >> 4;
  ln.t = ln.m & 7;
  ln.h = ln.m >> 3;
  ln.lane_kb = 8u * (uint32_t)(ln.q >> 1) + (uint32_t)(ln.q & 1);
  // B fragment source: this lane's token row at its k-slot, or the zero block
  ln.b_on = ((ln.q >> 1) == ln.h) & (ln.t < T);
  ln.bsrc = XSmem::ZERO + (uint32_t)ln.t * XSmem::xrow(K) + ln.lane_kb * 16u;
  // the base pattern lives in a vector register (an empty asm hides its
  // value), so each and-or takes one scalar and one vector constant
  uint32_t vbase = mask_base;
  asm volatile("" : "+v"(vbase));
  ln.mk = UnpackMasks{mask_nib, vbase, mask_hi};
  return ln;
}

// Row and column (tt, kc) of this thread's 16-byte chunks c_j = tid + 64 W j
// of a [rows][rowch] array of chunks, with one division for the first chunk
// and none after: a step of 64 W chunks is q0 rows and r0 chunks, r0 <
// rowch, so each step carries at most one row.  (A division per chunk, of a
// value known only at run time, costs ~25 VALU instructions.)  rowch <= 0
// gives zeros.
template <int XL, int W>
__device__ __forceinline__ void chunk_coords(int rowch, int (&tt)[XL], int (&kc)[XL]) {
  constexpr int S = W * 64;
  const int d = rowch > 0 ? rowch : 1;
  int t = (int)threadIdx.x / d, k = (int)threadIdx.x - t * d;
  const int q0 = S / d, r0 = S - q0 * d;
#pragma unroll
  for (int j = 0; j < XL; ++j) {
    tt[j] = t;
    kc[j] = k;
    k += r0;
    t += q0;
    if (k >= d) {
      k -= d;
      ++t;
    }
  }
}

// The X prologue: XL 16-byte chunks of X per thread, loaded before any weight
// (x_stage writes them to LDS once the first pairs' loads are issued).
template <int XL, int W>
__device__ __forceinline__ void x_load(uint32_t (&xv)[XL][4], const void* x, uint32_t x_bytes, int T, int K) {
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(x, x_bytes);
  const int nch = T * (K >> 3);
#pragma unroll
  for (int j = 0; j < XL; ++j) {
    const int c = threadIdx.x + W * 64 * j;
    const uint32_t off = c < nch ? (uint32_t)c * 16u : kOOB;  // X rows are contiguous in memory
    load_words<4>(xv[j], rX, off);
  }
}

// X into LDS in the interleaved order (waits for the X loads only), the zero
// block, barrier.
template <int XL, int W>
__device__ __forceinline__ void x_stage(uint8_t* smem, const uint32_t (&xv)[XL][4], int T, int K) {
  const int nch = T * (K >> 3), rowch = K >> 3;
  const uint32_t XROW = XSmem::xrow(K);
  // the LDS addresses depend on no loaded value: computed first, while the
  // loads are in flight (the barrier keeps them ahead of the first wait)
  int tt[XL], kc[XL];
  chunk_coords<XL, W>(rowch, tt, kc);
  uint32_t dst[XL];
#pragma unroll
  for (int j = 0; j < XL; ++j) dst[j] = XSmem::ZERO + (uint32_t)tt[j] * XROW + (uint32_t)kc[j] * 16u;
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < XL; ++j) {
    const int c = threadIdx.x + W * 64 * j;
    // an empty asm makes the chunk a value of this point: where staging sits
    // in a loop, the interleave is not hoisted above the first weight loads
    // (it would wait for X before they are issued)
    uint32_t d[4] = {xv[j][0], xv[j][1], xv[j][2], xv[j][3]};
    asm volatile("" : "+v"(d[0]), "+v"(d[1]), "+v"(d[2]), "+v"(d[3]));
    if (c < nch) *reinterpret_cast<u32x4*>(smem + dst[j]) = interleave_x(d);
  }
  if (threadIdx.x < XSmem::ZERO / 16) *reinterpret_cast<u32x4*>(smem + 16u * threadIdx.x) = u32x4{0u, 0u, 0u, 0u};
  lds_barrier();
}

// The loads of one pair of a column tile: P0 (two rows per 8-k block for
// int8), the int5 high bits and the scales, bounds-checked (an invalid pair
// reads out of range: nothing).  The lane's offsets within a tile are
// computed once.
template <int BITS, int V, int NSETS>
struct PairLoads {
  static constexpr int WPK = BITS == 8 ? 2 : 1;
  __amdgpu_buffer_rsrc_t rW, rP1, rS;
  uint32_t rowb, offA[NSETS], offP1[NSETS], offS[NSETS];

  __device__ __forceinline__ PairLoads(const ProjView& pv, const XresLane& ln) {
    rW = make_rsrc(pv.wq, pv.p0_bytes);
    rP1 = make_rsrc(static_cast<const char*>(pv.wq) + pv.p0_bytes, pv.p1_bytes);
    rS = make_rsrc(pv.scales, pv.s_bytes);
    rowb = (uint32_t)pv.Ncols * 4u;
#pragma unroll
    for (int s = 0; s < NSETS; ++s) {
      const uint32_t col = (uint32_t)(s * pv.up_off + V * ln.m);
      offA[s] = ln.lane_kb * WPK * rowb + col * 4u;
      offP1[s] = 2u * (uint32_t)(ln.q >> 1) * rowb + col * 4u;
      offS[s] = (uint32_t)ln.h * (uint32_t)pv.Ncols * 2u + (uint32_t)(s * pv.up_off + 4 * V * ln.q) * 2u;
    }
  }

  // pair p of the tile at column c0 (flags combined bitwise, so that no
  // lane-divergent branch appears)
  template <class Buf>
  __device__ __forceinline__ void issue(Buf& buf, uint32_t c0, int p, bool valid) const {
    const uint32_t pa = valid ? (uint32_t)p * 16u * WPK * rowb + c0 * 4u : kOOB;
    const uint32_t pp1 = valid ? (uint32_t)p * 4u * rowb + c0 * 4u : kOOB;
    const uint32_t ps = valid ? (uint32_t)p * rowb + c0 * 2u : kOOB;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int s = 0; s < NSETS; ++s) {
        const uint32_t o = offA[s] + pa + (uint32_t)st * 2u * WPK * rowb;
        load_words<V, kNT>(&buf.a[s][st][0], rW, o);
        if constexpr (BITS == 8) load_words<V, kNT>(&buf.a[s][st][V], rW, o + rowb);
      }
    }
    if constexpr (BITS == 5) {
#pragma unroll
      for (int s = 0; s < NSETS; ++s) {
        load_words<V, kNT>(&buf.p1[s][0][0], rP1, offP1[s] + pp1);
        load_words<V, kNT>(&buf.p1[s][1][0], rP1, offP1[s] + pp1 + rowb);
      }
    }
#pragma unroll
    for (int s = 0; s < NSETS; ++s) load_words<2 * V, kNT>(&buf.sc[s][0], rS, offS[s] + ps);
  }
};

// Per-group partial sums of pair p of a tile, before scaling: the pair's
// weight words in `buf` against X in LDS, each lane's B slot being token t of
// group half h.  The -(128 + bias) sum_k x term seeds every partial.
template <int BITS, int V, int NSETS, class Buf>
__device__ __forceinline__ void pair_partials(const Buf& buf, int p, const XresShape& sh, const XresLane& ln,
                                              const uint8_t* smem, f32x4 (&dp)[NSETS][V]) {
  const u32x4 negoff = {Code<BITS>::neg_offset_bf16 * 0x10001u, Code<BITS>::neg_offset_bf16 * 0x10001u,
                        Code<BITS>::neg_offset_bf16 * 0x10001u, Code<BITS>::neg_offset_bf16 * 0x10001u};
  // the second group of the last pair of an odd group count does not exist:
  // its lanes read zeros
  const bool half = (p == sh.pairs - 1) & ((sh.G & 1) != 0);
  const bool on = ln.b_on & !(half & (ln.h == 1));
  const uint32_t src = on ? ln.bsrc + (uint32_t)(p - sh.p0) * 256u : 0u;
  bf16x8 bfrag[4];
#pragma unroll
  for (int st = 0; st < 4; ++st)
    bfrag[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(smem + src + (uint32_t)st * 32u));
  f32x4 dx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < 4; ++st)
    dx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, negoff), bfrag[st], dx, 0, 0, 0);
#pragma unroll
  for (int s = 0; s < NSETS; ++s)
#pragma unroll
    for (int i = 0; i < V; ++i) dp[s][i] = dx;
#pragma unroll
  for (int st = 0; st < 4; ++st) {
#pragma unroll
    for (int s = 0; s < NSETS; ++s) {
#pragma unroll
      for (int i = 0; i < V; ++i) {
        u32x4 av;
        if constexpr (BITS == 4) {
          av = nibbles_to_bf16_il(buf.a[s][st][i], ln.mk);
        } else if constexpr (BITS == 5) {
          // k-block 2 st + (q & 1) of a 32-k P1 word group: byte 2 (st & 1) + (q & 1)
          const uint32_t p1 = buf.p1[s][st >> 1][i];
          const uint32_t hs = hb_spread(p1, p1 << 4, hb_select(2u * (uint32_t)(st & 1) + (uint32_t)(ln.q & 1)));
          av = nibbles5_to_bf16_il(buf.a[s][st][i], hs, ln.mk);
        } else {
          av = bytes_to_bf16_il(buf.a[s][st][i], buf.a[s][st][V + i]);
        }
        dp[s][i] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), bfrag[st], dp[s][i], 0, 0, 0);
      }
    }
  }
}

// acc += s * partial for every output of the pair (its scales in `buf`)
template <int V, int NSETS, class Buf>
__device__ __forceinline__ void scale_accumulate(const Buf& buf, bool sbf16, const f32x4 (&dp)[NSETS][V],
                                                 f32x4 (&acc)[NSETS][V]) {
#pragma unroll
  for (int s = 0; s < NSETS; ++s)
#pragma unroll
    for (int i = 0; i < V; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = V * r + i;
        acc[s][i][r] = __builtin_fmaf(scale_to_f32(buf.sc[s][e >> 1], e & 1, sbf16), dp[s][i][r], acc[s][i][r]);
      }
}

// A wave's partial block of a tile into LDS: slots j and j + 8 hold the two
// group halves of token j, added here; the lanes of the first half write the
// block [set][token][column].
template <int V, int NSETS>
__device__ __forceinline__ void store_partials(const f32x4 (&v)[NSETS][V], const XresLane& ln, float* blk) {
  constexpr int TILE = 16 * V;
#pragma unroll
  for (int s = 0; s < NSETS; ++s)
#pragma unroll
    for (int i = 0; i < V; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int other =
            __builtin_amdgcn_mov_dpp(__float_as_int(v[s][i][r]), 0x128 /* row_ror:8 */, 0xF, 0xF, false);
        const float sum = v[s][i][r] + __int_as_float(other);
        if (ln.h == 0)
          blk[((uint32_t)s * 8u + (uint32_t)ln.t) * (uint32_t)(TILE + 4) + (uint32_t)(V * (4 * ln.q + r) + i)] = sum;
      }
}

// The outputs of the tile at column c0: the W wave blocks summed in wave
// order, SwiGLU or plain, rounded to bf16.
template <int V, int NSETS, int W>
__device__ __forceinline__ void finish_outputs(const float* part, const ProjView& pv, int T, int c0) {
  constexpr int TILE = 16 * V;
  constexpr uint32_t BLK = Smem::block_floats(NSETS, TILE);
  uint16_t* y = static_cast<uint16_t*>(pv.y);
  for (int idx = threadIdx.x; idx < 8 * TILE; idx += W * 64) {
    const int tt = idx / TILE, col = idx % TILE;
    if (tt >= T || c0 + col >= pv.Nout) continue;
    float v[NSETS];
#pragma unroll
    for (int s = 0; s < NSETS; ++s) {
      const float* src = part + ((uint32_t)s * 8u + (uint32_t)tt) * (uint32_t)(TILE + 4) + (uint32_t)col;
      float sum = 0.f;
#pragma unroll
      for (int k = 0; k < W; ++k) sum += src[(uint32_t)k * BLK];
      v[s] = sum;
    }
    float out;
    if constexpr (NSETS == 2) {
      out = v[0] * v[1] / (1.0f + expf(-v[0]));  // SiLU(gate) * up
    } else {
      out = v[0];
    }
    y[(size_t)tt * pv.Nout + c0 + col] = f32_to_bf16_rne(out);
  }
}

// The tile loop of the X-resident kernels: `ntiles` column tiles of one
// projection, tile i being tile tbase + tstride * i of 16 V columns, with the
// pair pipeline running on across tile boundaries.  `buf` holds NB pairs in
// flight; when `primed`, the first NB pairs were issued into it before the
// call.  `stage` runs once, right after the first pairs' loads are issued (the
// X staging of the prologue, or nothing when X is already in LDS).  In the
// last NB slots of the last tile, `drain(buf[u], u)` issues what follows the
// loop into the freed buffers (the next segment's first pairs, or nothing).
// `finish(part, c0)` turns the wave blocks of the tile at column c0 into its
// outputs.  The LDS partial-sum region is free on entry and on return.
template <int BITS, bool SBF16, int V, int NSETS, int W, int NB, class Buf, class Stage, class Drain, class Finish>
__device__ __forceinline__ void xres_tiles(const ProjView& pv, const XresShape& sh, const XresLane& ln, uint8_t* smem,
                                           int tbase, int tstride, int ntiles, Buf (&buf)[NB], bool primed,
                                           Stage&& stage, Drain&& drain, Finish&& finish) {
  constexpr int TILE = 16 * V;
  constexpr uint32_t BLK = Smem::block_floats(NSETS, TILE);
  float* const part = reinterpret_cast<float*>(smem + XSmem::x_end(sh.T, sh.K));
  const int wave = ln.wave;

  const PairLoads<BITS, V, NSETS> ld(pv, ln);
  // loads of pair p of tile i (nothing when either is out of range)
  auto issue_at = [&](Buf& buf, int ti, int p) {
    ld.issue(buf, (uint32_t)((tbase + tstride * ti) * TILE), p, (ti < ntiles) & (p < sh.pend));
  };

  // item (tile i, slot k) is pair wave + W k of tile i; every tile has ppw
  // slots (the same for all waves, a multiple of NB), of which the first cnt
  // are real pairs
  const int npairs = sh.pend - sh.p0;
  const int cnt = npairs > wave ? (npairs - wave + W - 1) / W : 0;
  const int cntp = sh.ppw;
  int is_tile = 0, is_k = 0;  // next item to issue
  auto issue_next = [&](Buf& b, bool do_issue) {
    if (do_issue) issue_at(b, is_tile, is_k < cnt ? sh.p0 + wave + W * is_k : sh.pend);
    if (++is_k == cntp) {
      is_k = 0;
      ++is_tile;
    }
  };

#pragma unroll
  for (int u = 0; u < NB; ++u) {
    issue_next(buf[u], !primed);
    __builtin_amdgcn_sched_barrier(0);
  }
  stage();

  f32x4 acc[NSETS][V];
  auto clear_acc = [&]() {
#pragma unroll
    for (int s = 0; s < NSETS; ++s)
#pragma unroll
      for (int i = 0; i < V; ++i) acc[s][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  clear_acc();

  // one slot block: each buffer's pair computed and scaled, then refilled
  // (by the next item, or, in the final block, by `drain`)
  auto run_block = [&](int kk, bool final_block) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      if (kk + u < cnt) {
        f32x4 dp[NSETS][V];
        pair_partials<BITS, V, NSETS>(buf[u], sh.p0 + wave + W * (kk + u), sh, ln, smem, dp);
        scale_accumulate<V, NSETS>(buf[u], SBF16, dp, acc);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (final_block)
        drain(buf[u], u);
      else
        issue_next(buf[u], true);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  for (int ti = 0; ti < ntiles; ++ti) {
    // the final block of the last tile is peeled off: only there does
    // `drain` refill the buffers
    const bool last = ti == ntiles - 1 && cntp > 0;
    const int kk_end = last ? cntp - NB : cntp;
    for (int kk = 0; kk < kk_end; kk += NB) run_block(kk, false);
    if (last) run_block(cntp - NB, true);
    store_partials<V, NSETS>(acc, ln, part + (uint32_t)wave * BLK);
    clear_acc();
    lds_barrier();
    finish(part, (tbase + tstride * ti) * TILE);
    lds_barrier();
  }
}

// XL: X chunks (16 bytes) per thread in the prologue; W waves; NB pairs in
// flight per wave.
template <int BITS, bool SBF16, int V, int NSETS, int W, int NB, int XL>
__global__ __launch_bounds__(W * 64) void gemm_xres_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const XresLane ln = xres_lane(a.T, a.K, a.mask_nib, a.mask_base, a.mask_hi);
  // rank of this workgroup with the workgroups of one XCD (b % 8) numbered
  // consecutively, so that one XCD works on neighbouring tiles at a time
  const int G = gridDim.x, b = blockIdx.x, xcd = b & 7;
  const int rank = xcd * (G >> 3) + min(xcd, G & 7) + (b >> 3);
  const int my_tiles = a.tiles_q + (rank < a.tiles_r ? 1 : 0);  // tiles rank, rank + G, ... < ntiles

  // -- prologue: X loads first, then the first pairs' weights; the X wait in
  // x_stage then leaves those weights in flight.
  uint32_t xv[XL][4];
  x_load<XL, W>(xv, a.x, a.x_bytes, a.T, a.K);
  __builtin_amdgcn_sched_barrier(0);
  const ProjView pv{a.wq, a.scales, a.y, a.p0_bytes, a.p1_bytes, a.s_bytes, a.Nout, a.Ncols, a.up_off};
  const XresShape sh{a.T, a.K, a.G, a.pairs, a.ppw, 0, a.pairs};
  WBuf<BITS, V, NSETS> buf[NB];
  xres_tiles<BITS, SBF16, V, NSETS, W, NB>(
      pv, sh, ln, smem, rank, G, my_tiles, buf, false, [&]() { x_stage<XL, W>(smem, xv, a.T, a.K); },
      [](WBuf<BITS, V, NSETS>&, int) {},
      [&](const float* part, int c0) { finish_outputs<V, NSETS, W>(part, pv, a.T, c0); });
}

// ---- one round of tiles: each wave streams its own pairs ------------------------
//
// For shapes whose column tiles fill the CUs once (the QK projection: 256
// tiles of 32 columns), a workgroup owns one tile and every group pair of it
// is read by exactly one wave, so X needs no sharing between waves: wave w
// takes pairs w, w + W, ... and loads each pair's X band (T rows of 128 k)
// with the pair's weights and scales.  No workgroup-wide X prologue or
// barrier stands before the weight stream, which starts with the kernel's
// first loads.
//
// One pair is in flight per wave, and the next is requested as soon as the
// current one has landed, before it is computed, so the compute of a pair
// overlaps the next pair's round trip.  Measured on MI355X with the loads
// alone, about 20-32 KB in flight per CU streams fastest (W = 10 pairs of
// QK, 8 of gate/value; more in flight was slower), so the wave count, not a
// deeper per-wave pipeline, sets the depth.  Weights and scales are read
// with the nontemporal hint.
//
// X bands are loaded with as few lanes and bytes as T needs (each load's
// lanes return data through the same path whether in range or not, and in
// a load-only probe every X load added to the launch: 0.45 us for a single
// 16-lane load per pair at T = 1):
//   T = 1: one dword per lane (k 2l, 2l + 1 of the band);
//   T = 2: two dwords per lane (token l / 32, k 4 (l % 32) .. + 3);
//   T = 3, 4: one 16-byte load (token l / 16, k-block l % 16);
//   T > 4: two 16-byte loads.
// The band is written to a per-wave LDS slot in the interleaved k order of
// the unpack: 16-bit stores to their places for T <= 2, one permute per
// 4 bytes and 16-byte stores otherwise.
template <int BITS, int V, int NSETS>
struct StreamBuf {
  static constexpr int WPK = BITS == 8 ? 2 : 1;
  uint32_t a[NSETS][4][V * WPK];             // [set][step][word]; int8: V words of row 2kb, then 2kb+1
  uint32_t p1[NSETS][2][BITS == 5 ? V : 1];  // int5 high-bit words, one per group of the pair
  uint32_t sc[NSETS][2 * V];                 // 4V scales (16-bit)
  uint32_t x[2][4];                          // the pair's X band
};

// LDS of the streaming kernel: one X staging slot per wave (gemm_kernel's
// layout), then one partial-sum block per wave.
template <int W>
struct StreamSmem {
  static __host__ __device__ constexpr uint32_t bytes(int tile, int nsets = 1) {
    return (uint32_t)W * Smem::XSLOT + (uint32_t)W * Smem::block_floats(nsets, tile) * 4u;
  }
};

// Workgroup b of a launch over ntiles tiles takes this tile: consecutive
// tiles on one XCD (workgroup b runs on XCD b % 8).
__device__ __forceinline__ int xcd_tile(int b, int ntiles) {
  const int xcd = b & 7, per = ntiles >> 3, rem = ntiles & 7;
  return xcd * per + min(xcd, rem) + (b >> 3);
}

// LDS byte offset of element k (0..127) of a band's token row in the
// interleaved order: each 8-k block holds k = 0, 4, 1, 5, 2, 6, 3, 7.
__device__ __forceinline__ uint32_t il_offset(uint32_t k) {
  return (k >> 3) * 16u + (2u * (k & 3u) + ((k >> 2) & 1u)) * 2u;
}

// XM: the X load class, 1 (T = 1), 2 (T = 2), 4 (T = 3, 4) or 8 (T > 4); a
// template parameter so that no load sits under a branch (where the compiler
// waits for it, and with it every older load, before the join)
// NSETS = 2: the SwiGLU gate/up projection, the tile's columns of both
// halves (gate at c, up at up_off + c) in each pair.
// A K slice of a tile (split K): pairs pbase .. pbase + npairs - 1, ppw pair
// slots per wave, and the slice's fp32 output block [T][Nout].
struct StreamSlice {
  int pbase, npairs, ppw;
  float* partial;
};

// SLICE: the tile over one K slice, its wave blocks summed in wave order into
// the slice's fp32 block instead of rounded into y.
template <int BITS, bool SBF16, int V, int W, int XM, int NSETS, bool SLICE = false>
__device__ __forceinline__ void stream_tile(const GemmArgs& a, int tile, uint8_t* smem,
                                            const StreamSlice& sl = StreamSlice{0, 0, 0, nullptr}) {
  constexpr int WPK = BITS == 8 ? 2 : 1;
  constexpr int TILE = 16 * V;
  constexpr uint32_t XROW = Smem::XROW, XZERO = Smem::XZERO;
  constexpr uint32_t BLK = Smem::block_floats(NSETS, TILE);
  float* const part = reinterpret_cast<float*>(smem + (uint32_t)W * Smem::XSLOT);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15, q = lane >> 4;
  const int t = m & 7, h = m >> 3;  // B slot m: token t of group half h
  const uint32_t c0 = (uint32_t)(tile * TILE);

  const __amdgpu_buffer_rsrc_t rW = make_rsrc(a.wq, a.p0_bytes);
  const __amdgpu_buffer_rsrc_t rP1 = make_rsrc(static_cast<const char*>(a.wq) + a.p0_bytes, a.p1_bytes);
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(a.scales, a.s_bytes);
  uint32_t vbase = a.mask_base;
  asm volatile("" : "+v"(vbase));
  const UnpackMasks mk{a.mask_nib, vbase, a.mask_hi};

  const uint32_t rowb = (uint32_t)a.Ncols * 4u;
  // k-slot q of step st reads k-block 2 st + (q & 1) of group (q >> 1)
  const uint32_t lane_kb = 8u * (uint32_t)(q >> 1) + (uint32_t)(q & 1);
  uint32_t offA[NSETS], offP1[NSETS], offS[NSETS];
#pragma unroll
  for (int s = 0; s < NSETS; ++s) {
    const uint32_t cs = c0 + (uint32_t)(s * a.up_off);
    const uint32_t col = cs + (uint32_t)(V * m);
    offA[s] = lane_kb * WPK * rowb + col * 4u;
    offP1[s] = 2u * (uint32_t)(q >> 1) * rowb + col * 4u;
    // result rows 4q..4q+3 of every MFMA -> columns c0 + 4Vq + [0, 4V)
    offS[s] = (uint32_t)h * (uint32_t)a.Ncols * 2u + (cs + (uint32_t)(4 * V * q)) * 2u;
  }

  // This lane's share of a band: token row xt, first element xk (of the
  // band's 128), xe elements; chunk loads (T > 2) take 8 elements from rows
  // xt and xt + 4.
  const int T = a.T;
  constexpr int xmode = XM;
  const int xt = xmode == 1 ? 0 : (xmode == 2 ? lane >> 5 : lane >> 4);
  const int xk = xmode == 1 ? 2 * lane : (xmode == 2 ? 4 * (lane & 31) : 8 * (lane & 15));
  const uint32_t offX = (uint32_t)xt * (uint32_t)a.K * 2u + (uint32_t)xk * 2u;
  const uint32_t rowX4 = 4u * (uint32_t)a.K * 2u;
  const bool x0_on = xt < T, x1_on = xt + 4 < T;
  uint8_t* const xslot = smem + (uint32_t)wave * Smem::XSLOT;
  const uint32_t xdst = (uint32_t)xt * XROW + il_offset((uint32_t)xk);  // T <= 2: first element
  // B fragment source in the slot: this lane's token row at its k-slot, or
  // the zero block
  const bool b_on = (q >> 1) == h;
  const uint32_t bsrc = b_on ? (uint32_t)t * XROW + lane_kb * 16u : 8u * XROW;
  if (lane < XZERO / 16) *reinterpret_cast<u32x4*>(xslot + 8 * XROW + 16u * (uint32_t)lane) = u32x4{0u, 0u, 0u, 0u};
  // rows t >= T of the slot are read by the lanes of those tokens and must
  // hold zeros; rows no load covers (T <= 2: rows T..7, T <= 4: rows 4..7)
  // are cleared once here, the others are written with every band
  if constexpr (xmode <= 4) {
    for (int r = T; r < 8; ++r) *reinterpret_cast<uint32_t*>(xslot + (uint32_t)r * XROW + 4u * (uint32_t)lane) = 0u;
  }

  auto pair_of = [&](int i) { return wave + W * i; };
  // the pairs this tile covers: all of K, or the slice's
  const int pbase = SLICE ? sl.pbase : 0;
  const int npairs = SLICE ? sl.npairs : a.pairs;
  const int ppw = SLICE ? sl.ppw : a.ppw;

  // the loads of pair pbase + j (j >= npairs: out of range, nothing moves);
  // flags are combined bitwise so that no lane-divergent branch appears
  auto issue = [&](StreamBuf<BITS, V, NSETS>& buf, int j) {
    const bool valid = j < npairs;
    const int p = pbase + j;
    const uint32_t pa = valid ? (uint32_t)p * 16u * WPK * rowb : kOOB;
    const uint32_t pp1 = valid ? (uint32_t)p * 4u * rowb : kOOB;
    const uint32_t ps = valid ? (uint32_t)p * rowb : kOOB;  // two scale rows of 2-byte entries
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int s = 0; s < NSETS; ++s) {
        const uint32_t o = offA[s] + pa + (uint32_t)st * 2u * WPK * rowb;
        load_words<V, kNT>(&buf.a[s][st][0], rW, o);
        if constexpr (BITS == 8) load_words<V, kNT>(&buf.a[s][st][V], rW, o + rowb);
      }
    }
#pragma unroll
    for (int s = 0; s < NSETS; ++s) {
      if constexpr (BITS == 5) {
        load_words<V, kNT>(&buf.p1[s][0][0], rP1, offP1[s] + pp1);
        load_words<V, kNT>(&buf.p1[s][1][0], rP1, offP1[s] + pp1 + rowb);
      }
      load_words<2 * V, kNT>(&buf.sc[s][0], rS, offS[s] + ps);
    }
    // the band: the second group of the last pair of an odd group count
    // does not exist (elements 64..127 of its band read nothing)
    const bool half = (p == a.pairs - 1) & ((a.G & 1) != 0);
    const bool xin = valid & !(half & (xk >= 64));
    const uint32_t px0 = (xin & x0_on) ? (uint32_t)p * 256u + offX : kOOB;
    if constexpr (xmode == 1) {
      load_words<1>(&buf.x[0][0], rX, px0);
    } else if constexpr (xmode == 2) {
      load_words<2>(&buf.x[0][0], rX, px0);
    } else {
      load_words<4>(&buf.x[0][0], rX, px0);
      if constexpr (xmode == 8)
        load_words<4>(&buf.x[1][0], rX, (xin & x1_on) ? (uint32_t)p * 256u + offX + rowX4 : kOOB);
    }
  };

  // the landed band of a pair into the slot (the previous pair's B fragments
  // have been read: LDS is in order within a wave)
  auto stage_x = [&](const StreamBuf<BITS, V, NSETS>& buf) {
    if constexpr (xmode <= 2) {
      uint16_t* const d = reinterpret_cast<uint16_t*>(xslot + xdst);
      // element xk + e sits il_offset(xk + e) - il_offset(xk) bytes on: xk is
      // a multiple of 2 (T = 1) or 4 (T = 2) within an 8-k block
      d[0] = (uint16_t)buf.x[0][0];
      d[2] = (uint16_t)(buf.x[0][0] >> 16);
      if constexpr (xmode == 2) {
        d[4] = (uint16_t)buf.x[0][1];
        d[6] = (uint16_t)(buf.x[0][1] >> 16);
      }
    } else {
      *reinterpret_cast<u32x4*>(xslot + (uint32_t)xt * XROW + (uint32_t)(xk >> 3) * 16u) = interleave_x(buf.x[0]);
      if constexpr (xmode == 8)
        *reinterpret_cast<u32x4*>(xslot + (uint32_t)(xt + 4) * XROW + (uint32_t)(xk >> 3) * 16u) =
            interleave_x(buf.x[1]);
    }
  };

  f32x4 acc[NSETS][V];
#pragma unroll
  for (int s = 0; s < NSETS; ++s)
#pragma unroll
    for (int i = 0; i < V; ++i) acc[s][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const u32x4 negoff = {Code<BITS>::neg_offset_bf16 * 0x10001u, Code<BITS>::neg_offset_bf16 * 0x10001u,
                        Code<BITS>::neg_offset_bf16 * 0x10001u, Code<BITS>::neg_offset_bf16 * 0x10001u};

  // one pair: its B fragments from the slot, multiply, scale into the
  // accumulators
  auto compute = [&](const StreamBuf<BITS, V, NSETS>& buf) {
    bf16x8 bfrag[4];
#pragma unroll
    for (int st = 0; st < 4; ++st)
      bfrag[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xslot + bsrc + (uint32_t)st * 32u));
    f32x4 dx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st)
      dx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, negoff), bfrag[st], dx, 0, 0, 0);
    f32x4 dp[NSETS][V];
#pragma unroll
    for (int s = 0; s < NSETS; ++s)
#pragma unroll
      for (int i = 0; i < V; ++i) dp[s][i] = dx;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int s = 0; s < NSETS; ++s) {
#pragma unroll
        for (int i = 0; i < V; ++i) {
          u32x4 av;
          if constexpr (BITS == 4) {
            av = nibbles_to_bf16_il(buf.a[s][st][i], mk);
          } else if constexpr (BITS == 5) {
            // k-block 2 st + (q & 1) of a 32-k P1 word group: byte 2 (st & 1) + (q & 1)
            const uint32_t p1 = buf.p1[s][st >> 1][i];
            const uint32_t hs = hb_spread(p1, p1 << 4, hb_select(2u * (uint32_t)(st & 1) + (uint32_t)(q & 1)));
            av = nibbles5_to_bf16_il(buf.a[s][st][i], hs, mk);
          } else {
            av = bytes_to_bf16_il(buf.a[s][st][i], buf.a[s][st][V + i]);
          }
          dp[s][i] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), bfrag[st], dp[s][i], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int s = 0; s < NSETS; ++s)
#pragma unroll
      for (int i = 0; i < V; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = V * r + i;
          acc[s][i][r] = __builtin_fmaf(scale_to_f32(buf.sc[s][e >> 1], e & 1, SBF16), dp[s][i][r], acc[s][i][r]);
        }
  };

  // Pair slot i of this wave is pair wave + W i.  Two buffers: once slot i
  // has landed, slot i + 1 is requested, then slot i is computed.  A slot
  // past the last pair loads nothing and is not computed.
  StreamBuf<BITS, V, NSETS> buf[2];
  issue(buf[0], pair_of(0));
  __builtin_amdgcn_sched_barrier(0);
  for (int i = 0; i < ppw; i += 2) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    stage_x(buf[0]);
    issue(buf[1], pair_of(i + 1));
    __builtin_amdgcn_sched_barrier(0);
    if (pair_of(i) < npairs) compute(buf[0]);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    stage_x(buf[1]);
    issue(buf[0], pair_of(i + 2));
    __builtin_amdgcn_sched_barrier(0);
    if (pair_of(i + 1) < npairs) compute(buf[1]);
    __builtin_amdgcn_sched_barrier(0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // the two group halves of each token (slots j, j + 8), then the wave
  // blocks summed in wave order
  XresLane ln;
  ln.t = t;
  ln.q = q;
  ln.h = h;
  store_partials<V, NSETS>(acc, ln, part + (uint32_t)wave * BLK);
  lds_barrier();
  if constexpr (SLICE) {
    static_assert(NSETS == 1, "a K slice has one output set");
    for (int idx = threadIdx.x; idx < 8 * TILE; idx += W * 64) {
      const int tt = idx / TILE, col = idx % TILE;
      if (tt >= a.T || (int)c0 + col >= a.Nout) continue;
      const float* src = part + (uint32_t)tt * (uint32_t)(TILE + 4) + (uint32_t)col;
      float sum = 0.f;
#pragma unroll
      for (int k = 0; k < W; ++k) sum += src[(uint32_t)k * BLK];
      sl.partial[(size_t)tt * a.Nout + c0 + col] = sum;
    }
  } else {
    const ProjView pv{a.wq, a.scales, a.y, a.p0_bytes, a.p1_bytes, a.s_bytes, a.Nout, a.Ncols, a.up_off};
    finish_outputs<V, NSETS, W>(part, pv, a.T, (int)c0);
  }
}

template <int BITS, bool SBF16, int V, int W, int XM, int NSETS>
__global__ __launch_bounds__(W * 64) void gemm_stream_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  stream_tile<BITS, SBF16, V, W, XM, NSETS>(a, xcd_tile(blockIdx.x, a.ntiles), smem);
}

// ---- the same stream with a VALU inner step ---------------------------------
//
// gemm_dot_kernel is gemm_stream_kernel's pipeline (one 32-column tile per
// workgroup, pair w + W i on wave w, one pair in flight per wave, X band per
// pair) with the multiply-add on the vector ALU instead of the matrix cores:
// lane (c, g) owns column c0 + c and group g of every pair, unpacks its 8
// words per pair into bf16 pairs (the value 128 + u) and accumulates
// v_dot2_f32_bf16 products against X read from LDS (one address per half
// wave: a broadcast).  The offset (128 + bias) sum x of each group and token
// is reduced from the pair's X band across the lanes that hold it (DPP row
// shifts) and subtracted before scaling.  Measured against the MFMA step on
// the same pipeline, it is the faster of the two only at T = 1 for int4 and
// int8 (the projection's rows then cost one dot2 per two weights; from T = 2
// the VALU issue grows with T while the MFMA step's does not), where the
// library routes to it, and for the int4 SwiGLU projection at T = 1.
// NSETS = 2: the SwiGLU gate/up projection; the lane also owns column
// up_off + c0 + c (the up half), and each X element read from LDS serves
// both columns.
template <int W, int XM, int NSETS>
struct DotSmem {
  static constexpr uint32_t SLOT = (uint32_t)XM * Smem::XROW;  // per wave: the pair's X band, XM token rows
  static constexpr uint32_t SX = 16u * 4u;  // per wave: sums of x per (token, group) or per 16-lane row
  static __host__ __device__ constexpr uint32_t sx_off() { return (uint32_t)W * SLOT; }
  static __host__ __device__ constexpr uint32_t part_off() { return sx_off() + (uint32_t)W * SX; }
  // partial sums [wave][set][group][token][column]
  static __host__ __device__ constexpr uint32_t bytes() {
    return part_off() + (uint32_t)W * (uint32_t)NSETS * 2u * (uint32_t)XM * 32u * 4u;
  }
};

template <int BITS, int NSETS>
struct DotBuf {
  static constexpr int WPK = BITS == 8 ? 2 : 1;
  uint32_t a[NSETS][8 * WPK];  // one word per k-block of the lane's group (int8: two)
  uint32_t p1[NSETS][BITS == 5 ? 2 : 1];
  uint32_t sc[NSETS];          // the lane's scales (16-bit)
  uint32_t x[2][4];            // the pair's X band (the streaming kernel's load classes)
};

// One 32-column tile of one projection (the body of gemm_dot_kernel, also
// run by gemm_multi_dot_kernel).
template <int BITS, bool SBF16, int W, int XM, int NSETS>
__device__ __forceinline__ void dot_tile(const GemmArgs& a, int tile, uint8_t* smem) {
  constexpr int WPK = BITS == 8 ? 2 : 1;
  constexpr uint32_t XROW = Smem::XROW;
  using Lds = DotSmem<W, XM, NSETS>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 31, g = lane >> 5;  // column of the tile, group of the pair
  const uint32_t c0 = (uint32_t)(tile * 32);

  const __amdgpu_buffer_rsrc_t rW = make_rsrc(a.wq, a.p0_bytes);
  const __amdgpu_buffer_rsrc_t rP1 = make_rsrc(static_cast<const char*>(a.wq) + a.p0_bytes, a.p1_bytes);
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(a.scales, a.s_bytes);
  uint32_t vbase = a.mask_base;
  asm volatile("" : "+v"(vbase));
  const UnpackMasks mk{a.mask_nib, vbase, a.mask_hi};

  const uint32_t rowb = (uint32_t)a.Ncols * 4u;
  uint32_t offW[NSETS], offP1[NSETS], offS[NSETS];
#pragma unroll
  for (int s = 0; s < NSETS; ++s) {
    const uint32_t col = c0 + (uint32_t)(s * a.up_off) + (uint32_t)c;
    offW[s] = 8u * (uint32_t)g * WPK * rowb + col * 4u;  // k-block 0 of the lane's group
    offP1[s] = 2u * (uint32_t)g * rowb + col * 4u;
    offS[s] = (uint32_t)g * (uint32_t)a.Ncols * 2u + col * 2u;
  }

  // the X band, as in gemm_stream_kernel
  const int T = a.T;
  constexpr int xmode = XM;
  const int xt = xmode == 1 ? 0 : (xmode == 2 ? lane >> 5 : lane >> 4);
  const int xk = xmode == 1 ? 2 * lane : (xmode == 2 ? 4 * (lane & 31) : 8 * (lane & 15));
  const uint32_t offX = (uint32_t)xt * (uint32_t)a.K * 2u + (uint32_t)xk * 2u;
  const uint32_t rowX4 = 4u * (uint32_t)a.K * 2u;
  const bool x0_on = xt < T, x1_on = xt + 4 < T;
  uint8_t* const xslot = smem + (uint32_t)wave * Lds::SLOT;
  float* const sxw = reinterpret_cast<float*>(smem + Lds::sx_off() + (uint32_t)wave * Lds::SX);
  const uint32_t xdst = (uint32_t)xt * XROW + il_offset((uint32_t)xk);

  auto pair_of = [&](int i) { return wave + W * i; };

  auto issue = [&](DotBuf<BITS, NSETS>& buf, int p) {
    const bool valid = p < a.pairs;
    const bool half = (p == a.pairs - 1) & ((a.G & 1) != 0);
    const bool gin = valid & !(half & (g == 1));  // the lane's group exists
#pragma unroll
    for (int s = 0; s < NSETS; ++s) {
      const uint32_t pa = gin ? (uint32_t)p * 16u * WPK * rowb + offW[s] : kOOB;
#pragma unroll
      for (int kb = 0; kb < 8 * WPK; ++kb) load_words<1, kNT>(&buf.a[s][kb], rW, pa + (uint32_t)kb * rowb);
      if constexpr (BITS == 5) {
        const uint32_t pp1 = gin ? (uint32_t)p * 4u * rowb + offP1[s] : kOOB;
        load_words<1, kNT>(&buf.p1[s][0], rP1, pp1);
        load_words<1, kNT>(&buf.p1[s][1], rP1, pp1 + rowb);
      }
      buf.sc[s] = __builtin_amdgcn_raw_buffer_load_b16(rS, gin ? (uint32_t)p * rowb + offS[s] : kOOB, 0, kNT);
    }
    const bool xin = valid & !(half & (xk >= 64));
    const uint32_t px0 = (xin & x0_on) ? (uint32_t)p * 256u + offX : kOOB;
    if constexpr (xmode == 1) {
      load_words<1>(&buf.x[0][0], rX, px0);
    } else if constexpr (xmode == 2) {
      load_words<2>(&buf.x[0][0], rX, px0);
    } else {
      load_words<4>(&buf.x[0][0], rX, px0);
      if constexpr (xmode == 8)
        load_words<4>(&buf.x[1][0], rX, (xin & x1_on) ? (uint32_t)p * 256u + offX + rowX4 : kOOB);
    }
  };

  // the landed band into the slot, and the sums of x per (token, group):
  // each lane's share, then a segmented sum over the lanes of one (token,
  // group) with DPP row shifts (8 lanes a segment for 16-byte chunks, 16 for
  // T = 2; for T = 1 the two 16-lane rows of a group are added by the reader)
  const uint32_t ones = 0x3F803F80u;  // bf16 (1, 1)
  auto stage_x = [&](const DotBuf<BITS, NSETS>& buf) {
    float s0 = 0.f, s1 = 0.f;
    if constexpr (xmode <= 2) {
      uint16_t* const d = reinterpret_cast<uint16_t*>(xslot + xdst);
      d[0] = (uint16_t)buf.x[0][0];
      d[2] = (uint16_t)(buf.x[0][0] >> 16);
      s0 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(buf.x[0][0]),
                                            as_bf16x2(ones), 0.f, false);
      if constexpr (xmode == 2) {
        d[4] = (uint16_t)buf.x[0][1];
        d[6] = (uint16_t)(buf.x[0][1] >> 16);
        s0 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(buf.x[0][1]),
                                              as_bf16x2(ones), s0, false);
      }
    } else {
      *reinterpret_cast<u32x4*>(xslot + (uint32_t)xt * XROW + (uint32_t)(xk >> 3) * 16u) = interleave_x(buf.x[0]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        s0 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(buf.x[0][j]),
                                              as_bf16x2(ones), s0, false);
      if constexpr (xmode == 8) {
        *reinterpret_cast<u32x4*>(xslot + (uint32_t)(xt + 4) * XROW + (uint32_t)(xk >> 3) * 16u) =
            interleave_x(buf.x[1]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          s1 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(buf.x[1][j]),
                                                as_bf16x2(ones), s1, false);
      }
    }
    constexpr int seg = xmode >= 4 ? 8 : 16;
    // row_shr:1, 2, 4 (and 8): lane i then holds the sum of lanes i - seg + 1 .. i of its row
    s0 += __builtin_amdgcn_update_dpp(0.f, s0, 0x111, 0xF, 0xF, true);
    s0 += __builtin_amdgcn_update_dpp(0.f, s0, 0x112, 0xF, 0xF, true);
    s0 += __builtin_amdgcn_update_dpp(0.f, s0, 0x114, 0xF, 0xF, true);
    if constexpr (seg == 16) s0 += __builtin_amdgcn_update_dpp(0.f, s0, 0x118, 0xF, 0xF, true);
    if constexpr (xmode == 8) {
      s1 += __builtin_amdgcn_update_dpp(0.f, s1, 0x111, 0xF, 0xF, true);
      s1 += __builtin_amdgcn_update_dpp(0.f, s1, 0x112, 0xF, 0xF, true);
      s1 += __builtin_amdgcn_update_dpp(0.f, s1, 0x114, 0xF, 0xF, true);
    }
    if ((lane & (seg - 1)) == seg - 1) {
      if constexpr (xmode >= 4) {
        const int gg = (lane >> 3) & 1;  // lanes 0..7 of a row: group 0
        sxw[xt * 2 + gg] = s0;
        if constexpr (xmode == 8) sxw[(xt + 4) * 2 + gg] = s1;
      } else {
        sxw[lane >> 4] = s0;  // row r: T = 2 token r / 2, group r % 2; T = 1 group r / 2
      }
    }
  };
  auto sum_x = [&](int t) -> float {
    if constexpr (xmode == 1) return sxw[2 * g] + sxw[2 * g + 1];
    return sxw[t * 2 + g];
  };

  float acc[NSETS][XM];
#pragma unroll
  for (int s = 0; s < NSETS; ++s)
#pragma unroll
    for (int t = 0; t < XM; ++t) acc[s][t] = 0.f;

  auto compute = [&](const DotBuf<BITS, NSETS>& buf) {
    float pacc[NSETS][XM];
#pragma unroll
    for (int s = 0; s < NSETS; ++s)
#pragma unroll
      for (int t = 0; t < XM; ++t) pacc[s][t] = 0.f;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      u32x4 w[NSETS];
#pragma unroll
      for (int s = 0; s < NSETS; ++s) {
        if constexpr (BITS == 4) {
          w[s] = nibbles_to_bf16_il(buf.a[s][kb], mk);
        } else if constexpr (BITS == 5) {
          const uint32_t p1 = buf.p1[s][kb >> 2];
          w[s] = nibbles5_to_bf16_il(buf.a[s][kb], hb_spread(p1, p1 << 4, hb_select((uint32_t)(kb & 3))), mk);
        } else {
          w[s] = bytes_to_bf16_il(buf.a[s][2 * kb], buf.a[s][2 * kb + 1]);
        }
      }
#pragma unroll
      for (int t = 0; t < XM; ++t) {
        if (t < T) {
          const u32x4 xr = *reinterpret_cast<const u32x4*>(xslot + (uint32_t)t * XROW + (uint32_t)(8 * g + kb) * 16u);
#pragma unroll
          for (int s = 0; s < NSETS; ++s)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              pacc[s][t] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w[s][j]), as_bf16x2(xr[j]), pacc[s][t], false);
        }
      }
    }
#pragma unroll
    for (int s = 0; s < NSETS; ++s) {
      const float sc = scale_to_f32(buf.sc[s], 0, SBF16);
#pragma unroll
      for (int t = 0; t < XM; ++t)
        if (t < T) acc[s][t] = __builtin_fmaf(sc, pacc[s][t] - (float)Code<BITS>::offset * sum_x(t), acc[s][t]);
    }
  };

  DotBuf<BITS, NSETS> buf[2];
  issue(buf[0], pair_of(0));
  __builtin_amdgcn_sched_barrier(0);
  for (int i = 0; i < a.ppw; i += 2) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    stage_x(buf[0]);
    issue(buf[1], pair_of(i + 1));
    __builtin_amdgcn_sched_barrier(0);
    if (pair_of(i) < a.pairs) compute(buf[0]);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    stage_x(buf[1]);
    issue(buf[0], pair_of(i + 2));
    __builtin_amdgcn_sched_barrier(0);
    if (pair_of(i + 1) < a.pairs) compute(buf[1]);
    __builtin_amdgcn_sched_barrier(0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // partial sums [wave][set][group][token][column], added in wave then group
  // order; SwiGLU as in finish_outputs
  float* const part = reinterpret_cast<float*>(smem + Lds::part_off());
  auto slot = [](int w, int s, int gg, int t, int cc) -> uint32_t {
    return (((((uint32_t)w * NSETS + (uint32_t)s) * 2u + (uint32_t)gg) * XM + (uint32_t)t) * 32u) + (uint32_t)cc;
  };
#pragma unroll
  for (int s = 0; s < NSETS; ++s)
#pragma unroll
    for (int t = 0; t < XM; ++t)
      if (t < T) part[slot(wave, s, g, t, c)] = acc[s][t];
  lds_barrier();
  uint16_t* y = static_cast<uint16_t*>(a.y);
  for (int idx = threadIdx.x; idx < XM * 32; idx += W * 64) {
    const int tt = idx >> 5, cc = idx & 31;
    if (tt >= T || c0 + (uint32_t)cc >= (uint32_t)a.Nout) continue;
    float v[NSETS];
#pragma unroll
    for (int s = 0; s < NSETS; ++s) {
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        sum += part[slot(w, s, 0, tt, cc)];
        sum += part[slot(w, s, 1, tt, cc)];
      }
      v[s] = sum;
    }
    float out;
    if constexpr (NSETS == 2) {
      out = v[0] * v[1] / (1.0f + expf(-v[0]));  // SiLU(gate) * up
    } else {
      out = v[0];
    }
    y[(size_t)tt * a.Nout + c0 + cc] = f32_to_bf16_rne(out);
  }
}

template <int BITS, bool SBF16, int W, int XM, int NSETS>
__global__ __launch_bounds__(W * 64) void gemm_dot_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  dot_tile<BITS, SBF16, W, XM, NSETS>(a, xcd_tile(blockIdx.x, a.ntiles), smem);
}

// ---- several projections of one X in one launch ----------------------------
//
// The projections of a layer that read the same activations (QK, gate/value
// and gate/up) run as one launch.  Where every projection is int4 or plain
// int5 / int8 that launch is one workgroup per tile (gemm_multi_dot_kernel,
// gemm_multi_stream_kernel, below); otherwise it is this persistent kernel:
// X is staged once per workgroup, and the tiles of all projections are
// spread over the workgroups by cost (host-planned, longest tiles first to
// the least loaded workgroup), which also evens out projections whose tile
// count is not a multiple of the CU count.  Workgroup r owns a contiguous
// range of each projection's tiles and runs them projection by projection
// with the X-resident tile loop, the pair pipeline running on from one
// projection into the next.

constexpr int kMultiMaxProj = 4;
constexpr int kMultiMaxWg = 256;
constexpr int kMultiW = 8, kMultiNB = 2, kMultiXL = 10;

// Tile runner of a projection: bit width, scale type and output sets.
__host__ __device__ constexpr int multi_kind(int bits, bool sbf16, int nsets) {
  return (bits == 4 ? 0 : bits == 5 ? 1 : 2) * 4 + (sbf16 ? 2 : 0) + (nsets - 1);
}
// Tile width (columns per lane) of each runner: 32-column tiles, except int8
// with two output sets, which needs 16 to stay within registers.
__host__ __device__ constexpr int multi_v(int bits, int nsets) { return bits == 8 && nsets == 2 ? 1 : 2; }

struct MultiProj {
  const void* wq;
  const void* scales;
  void* y;
  uint32_t p0_bytes, p1_bytes, s_bytes;
  int Nout, Ncols, up_off;
  int kind;
};

struct MultiArgs {
  const void* x;
  uint32_t x_bytes;
  int T, K, G, pairs, ppw;
  uint32_t mask_nib, mask_base, mask_hi;
  MultiProj proj[kMultiMaxProj];
  // workgroup b owns tiles first[b][p] .. first[b][p] + count[b][p] - 1 of
  // projection p (two scalar loads give a workgroup all its ranges); the host
  // places neighbouring ranges on one XCD, so the scale cache lines that two
  // neighbouring tiles share are fetched into one L2
  uint16_t first[kMultiMaxWg][kMultiMaxProj];
  uint8_t count[kMultiMaxWg][kMultiMaxProj];
};

// X into LDS when it exceeds XL chunks per thread (long K at large T): the
// zero block, then X in rounds of XL chunks per thread, and the barrier.  Run
// before any weight load is issued (its loop would otherwise leave the
// compiler unable to tell which loads are in flight).
template <int XL, int W>
__device__ __forceinline__ void x_stage_rounds(uint8_t* smem, const void* x, uint32_t x_bytes, int T, int K) {
  const int nch = T * (K >> 3), rowch = K >> 3;
  const uint32_t XROW = XSmem::xrow(K);
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(x, x_bytes);
  if (threadIdx.x < XSmem::ZERO / 16) *reinterpret_cast<u32x4*>(smem + 16u * threadIdx.x) = u32x4{0u, 0u, 0u, 0u};
  // round r's chunk j is chunk r XL + j of the thread's sequence
  int tt[XL], kc[XL];
  chunk_coords<XL, W>(rowch, tt, kc);
  const int RS = XL * W * 64;
  const int dq = RS / (rowch > 0 ? rowch : 1), dr = RS - dq * (rowch > 0 ? rowch : 1);
  for (int base = 0; base < nch; base += RS) {
    uint32_t xr[XL][4];
#pragma unroll
    for (int j = 0; j < XL; ++j) {
      const int c = base + threadIdx.x + W * 64 * j;
      load_words<4>(xr[j], rX, c < nch ? (uint32_t)c * 16u : kOOB);
    }
#pragma unroll
    for (int j = 0; j < XL; ++j) {
      const int c = base + threadIdx.x + W * 64 * j;
      if (c < nch)
        *reinterpret_cast<u32x4*>(smem + XSmem::ZERO + (uint32_t)tt[j] * XROW + (uint32_t)kc[j] * 16u) =
            interleave_x(xr[j]);
      // the same chunk of the next round
      kc[j] += dr;
      tt[j] += dq;
      if (kc[j] >= rowch) {
        kc[j] -= rowch;
        ++tt[j];
      }
    }
  }
  lds_barrier();
}

// This workgroup's tile ranges (its row of the table) and the range of
// projection p in them.
struct MultiRanges {
  uint32_t f01, f23, cnt;
  __device__ int get(int p, int& f) const {
    f = (int)(((p < 2 ? f01 : f23) >> (16u * (uint32_t)(p & 1))) & 0xFFFFu);
    return (int)((cnt >> (8u * (uint32_t)p)) & 0xFFu);
  }
  // the next projection after `from` with tiles here (kMultiMaxProj: none)
  __device__ int next(int from, int& f, int& n) const {
    int q = from + 1;
    while (q < kMultiMaxProj && (n = get(q, f)) == 0) ++q;
    return q;
  }
};

__device__ __forceinline__ ProjView multi_view(const MultiProj& mp) {
  return ProjView{mp.wq, mp.scales, mp.y, mp.p0_bytes, mp.p1_bytes, mp.s_bytes, mp.Nout, mp.Ncols, mp.up_off};
}

// The start of a fused launch: every argument needed before the first weight
// loads is read with no read depending on another, so that the scalar loads
// go out together (each dependent argument read would add a round trip before
// the weights are issued): the tile ranges, projection 0's buffers (the host
// lists first a projection every workgroup has tiles of, when one exists) and
// the shape.  The other descriptors' kinds are read too, which brings every
// descriptor's cache line into the scalar cache for later segments.
__device__ __forceinline__ MultiRanges multi_start(const MultiArgs& a, ProjView& pv0, int& kind0) {
  const uint32_t* row = reinterpret_cast<const uint32_t*>(&a.first[blockIdx.x][0]);
  const MultiRanges rg{row[0], row[1], *reinterpret_cast<const uint32_t*>(&a.count[blockIdx.x][0])};
  pv0 = multi_view(a.proj[0]);
  kind0 = a.proj[0].kind;
  // empty asm statements that use the values keep their loads in this first
  // round trip (the compiler would otherwise sink them below the X loads)
  asm volatile("" ::"s"(rg.f01), "s"(rg.f23), "s"(rg.cnt), "s"(pv0.wq), "s"(pv0.scales), "s"(pv0.y),
               "s"(pv0.p0_bytes), "s"(pv0.p1_bytes), "s"(pv0.s_bytes), "s"(pv0.Nout), "s"(pv0.Ncols),
               "s"(pv0.up_off), "s"(kind0));
  asm volatile("" ::"s"(a.x), "s"(a.x_bytes), "s"(a.T), "s"(a.K), "s"(a.G), "s"(a.pairs), "s"(a.ppw),
               "s"(a.mask_nib), "s"(a.mask_base), "s"(a.mask_hi), "s"(a.proj[1].kind), "s"(a.proj[2].kind),
               "s"(a.proj[3].kind));
  return rg;
}

// BIGX: X exceeds the prologue's XL chunks per thread and is staged in rounds
// before the first weight loads; otherwise the first projection's first
// pairs are issued before X is staged, and the two loads overlap.
template <bool BIGX>
__global__ __launch_bounds__(kMultiW * 64) void gemm_multi_kernel(MultiArgs a) {
  constexpr int W = kMultiW, NB = kMultiNB, XL = kMultiXL;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  ProjView pv0;
  int kind0;
  const MultiRanges rg = multi_start(a, pv0, kind0);
  const XresLane ln = xres_lane(a.T, a.K, a.mask_nib, a.mask_base, a.mask_hi);
  const XresShape sh{a.T, a.K, a.G, a.pairs, a.ppw, 0, a.pairs};

  uint32_t xv[BIGX ? 1 : XL][4];
  if constexpr (BIGX)
    x_stage_rounds<XL, W>(smem, a.x, a.x_bytes, a.T, a.K);
  else
    x_load<XL, W>(xv, a.x, a.x_bytes, a.T, a.K);
  __builtin_amdgcn_sched_barrier(0);

  bool staged = BIGX;
  auto stage = [&]() {
    if constexpr (!BIGX) {
      if (!staged) x_stage<XL, W>(smem, xv, a.T, a.K);
    }
    staged = true;
  };
  auto no_drain = [](auto&, int) {};
  for (int p = 0; p < kMultiMaxProj; ++p) {
    int f = 0;
    const int n = rg.get(p, f);
    if (n == 0) continue;
    const ProjView pv = p == 0 ? pv0 : multi_view(a.proj[p]);
    switch (p == 0 ? kind0 : a.proj[p].kind) {
#define NGQ_MULTI_CASE(BITS, SBF16, NSETS)                                                                       \
  case multi_kind(BITS, SBF16, NSETS): {                                                                         \
    WBuf<BITS, multi_v(BITS, NSETS), NSETS> buf[NB];                                                             \
    xres_tiles<BITS, SBF16, multi_v(BITS, NSETS), NSETS, W, NB>(                                                 \
        pv, sh, ln, smem, f, 1, n, buf, false, stage, no_drain, [&](const float* part, int c0) {                  \
          finish_outputs<multi_v(BITS, NSETS), NSETS, W>(part, pv, a.T, c0);                                      \
        });                                                                                                      \
    break;                                                                                                       \
  }
      NGQ_MULTI_CASE(4, false, 1) NGQ_MULTI_CASE(4, false, 2) NGQ_MULTI_CASE(4, true, 1) NGQ_MULTI_CASE(4, true, 2)
      NGQ_MULTI_CASE(5, false, 1) NGQ_MULTI_CASE(5, false, 2) NGQ_MULTI_CASE(5, true, 1) NGQ_MULTI_CASE(5, true, 2)
      NGQ_MULTI_CASE(8, false, 1) NGQ_MULTI_CASE(8, false, 2) NGQ_MULTI_CASE(8, true, 1) NGQ_MULTI_CASE(8, true, 2)
#undef NGQ_MULTI_CASE
      default:
        break;
    }
  }
}

// ---- several projections, one tile per workgroup -----------------------------
//
// The projections of one x run as one launch of independent workgroups, one
// per 32-column tile of any projection: at T = 1 each runs the VALU-step tile
// of gemm_dot_kernel with kMultiDotW waves (three workgroups a CU), at T =
// 2..8 the MFMA-step tile of gemm_stream_kernel with kMultiStreamW waves (four
// a CU).  Segment p of the grid holds projection p's tiles (the heaviest
// tiles first, so the light ones fill the end), and the hardware hands out
// workgroups as others finish, which evens out the unequal tiles with no
// plan.  The kinds served are those whose tile keeps that many workgroups on
// a CU (int4 with or without SwiGLU, int5 and int8 plain).
constexpr int kMultiDotW = 7;

struct MultiTileArgs {
  GemmArgs proj[kMultiMaxProj];
  int end[kMultiMaxProj];   // one past projection p's last workgroup
  int kind[kMultiMaxProj];  // multi_kind of projection p
};

__host__ __device__ constexpr bool multi_tile_kind(int kind) {
  return kind == multi_kind(4, false, 1) || kind == multi_kind(4, true, 1) || kind == multi_kind(4, false, 2) ||
         kind == multi_kind(4, true, 2) || kind == multi_kind(5, false, 1) || kind == multi_kind(5, true, 1) ||
         kind == multi_kind(8, false, 1) || kind == multi_kind(8, true, 1);
}

__global__ __launch_bounds__(kMultiDotW * 64) void gemm_multi_dot_kernel(MultiTileArgs m) {
  constexpr int W = kMultiDotW;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int b = blockIdx.x;
  int p = 0;
#pragma unroll
  for (int i = 0; i < kMultiMaxProj - 1; ++i) p += b >= m.end[i] ? 1 : 0;
  const int b0 = p == 0 ? 0 : m.end[p - 1];
  const int tile = xcd_tile(b - b0, m.end[p] - b0);
  const GemmArgs& a = m.proj[p];
  switch (m.kind[p]) {
    case multi_kind(4, false, 1): dot_tile<4, false, W, 1, 1>(a, tile, smem); break;
    case multi_kind(4, true, 1): dot_tile<4, true, W, 1, 1>(a, tile, smem); break;
    case multi_kind(4, false, 2): dot_tile<4, false, W, 1, 2>(a, tile, smem); break;
    case multi_kind(4, true, 2): dot_tile<4, true, W, 1, 2>(a, tile, smem); break;
    case multi_kind(5, false, 1): dot_tile<5, false, W, 1, 1>(a, tile, smem); break;
    case multi_kind(5, true, 1): dot_tile<5, true, W, 1, 1>(a, tile, smem); break;
    case multi_kind(8, false, 1): dot_tile<8, false, W, 1, 1>(a, tile, smem); break;
    case multi_kind(8, true, 1): dot_tile<8, true, W, 1, 1>(a, tile, smem); break;
    default: break;
  }
}

constexpr int kMultiStreamW = 4;

// Columns of a tile (of each half, for SwiGLU) in gemm_multi_stream_kernel:
// 64 at T >= 5, where a tile's X bands (80 KB per workgroup at T = 8) are
// worth sharing over more columns, else 32.  Stacked layer at T = 8: 37.4 us
// with 32-column tiles, 36.1 with 64-column plain tiles, 34.9-35.1 with
// 64-column SwiGLU tiles too (200 VGPRs: two 4-wave workgroups a CU; 2, 3,
// 6 or 8 waves 7-11 % slower); at T <= 4 wider tiles gain nothing.
__host__ __device__ constexpr int multi_tile_cols(int T) { return T >= 5 ? 64 : 32; }

template <int XM>
__global__ __launch_bounds__(kMultiStreamW * 64) void gemm_multi_stream_kernel(MultiTileArgs m) {
  constexpr int W = kMultiStreamW;
  constexpr int VP = multi_tile_cols(XM) / 16;  // XM = 8 stands for T = 5..8
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int b = blockIdx.x;
  int p = 0;
#pragma unroll
  for (int i = 0; i < kMultiMaxProj - 1; ++i) p += b >= m.end[i] ? 1 : 0;
  const int b0 = p == 0 ? 0 : m.end[p - 1];
  const int tile = xcd_tile(b - b0, m.end[p] - b0);
  const GemmArgs& a = m.proj[p];
  switch (m.kind[p]) {
    case multi_kind(4, false, 1): stream_tile<4, false, VP, W, XM, 1>(a, tile, smem); break;
    case multi_kind(4, true, 1): stream_tile<4, true, VP, W, XM, 1>(a, tile, smem); break;
    case multi_kind(4, false, 2): stream_tile<4, false, VP, W, XM, 2>(a, tile, smem); break;
    case multi_kind(4, true, 2): stream_tile<4, true, VP, W, XM, 2>(a, tile, smem); break;
    case multi_kind(5, false, 1): stream_tile<5, false, VP, W, XM, 1>(a, tile, smem); break;
    case multi_kind(5, true, 1): stream_tile<5, true, VP, W, XM, 1>(a, tile, smem); break;
    case multi_kind(8, false, 1): stream_tile<8, false, VP, W, XM, 1>(a, tile, smem); break;
    case multi_kind(8, true, 1): stream_tile<8, true, VP, W, XM, 1>(a, tile, smem); break;
    default: break;
  }
}

// ---- split K: long K over few column tiles ----------------------------------
//
// A projection with long K and few 32-column tiles (the down projection: K =
// 17408, 160 tiles) leaves CUs idle with one workgroup per tile.  Here K is
// cut into S slices of whole group pairs and each workgroup streams one
// 64-column tile over one slice on the streaming kernel's pipeline (X band
// per pair, one pair in flight per wave), workgroup b taking tile b / S of
// slice b % S; S is chosen so that the S x (tiles of 64 columns) workgroups
// fill the CUs about once (down: 3 slices x 80 tiles).  Each unit's fp32 sum
// goes to partial[slice][t][n] in a caller's workspace, and a second kernel
// adds the S partials of every output in slice order and rounds to bf16, so
// the result is deterministic.

constexpr int kSplitWaves = 8;
constexpr int kSplitV = 4;  // 64-column tiles

struct SplitArgs {
  GemmArgs g;  // the projection; g.pairs counts the pairs of the whole K
  float* partial;  // [S][T][N]
  int S, pps;  // slices, pairs per slice (the last may have fewer)
};

template <int BITS, bool SBF16, int XM>
__global__ __launch_bounds__(kSplitWaves * 64) void gemm_splitk_kernel(SplitArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int b = blockIdx.x, ks = b % a.S;
  const int pb = ks * a.pps, np = max(0, min(a.pps, a.g.pairs - pb));
  const StreamSlice sl{pb, np, (np + kSplitWaves - 1) / kSplitWaves,
                       a.partial + (size_t)ks * (size_t)a.g.T * (size_t)a.g.Nout};
  stream_tile<BITS, SBF16, kSplitV, kSplitWaves, XM, 1, true>(a.g, xcd_tile(b / a.S, a.g.ntiles), smem, sl);
}

// y[e] = bf16(partial[0][e] + partial[1][e] + ... + partial[S-1][e]), in slice
// order; e runs over the T N outputs, four per thread (N % 4 == 0).
// With a residual r (bf16, same layout as y), r[e] is added last, before the
// rounding.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partial, int S, int TN,
                                                            uint16_t* __restrict__ y,
                                                            const uint16_t* __restrict__ res) {
  const int e = 4 * (blockIdx.x * 256 + threadIdx.x);
  if (e >= TN) return;
  float4 acc = *reinterpret_cast<const float4*>(partial + e);
  for (int ks = 1; ks < S; ++ks) {
    const float4 v = *reinterpret_cast<const float4*>(partial + (size_t)ks * TN + e);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  if (res != nullptr) {
    const u32x2 r = *reinterpret_cast<const u32x2*>(res + e);
    acc.x += __uint_as_float(r[0] << 16);
    acc.y += __uint_as_float(r[0] & 0xFFFF0000u);
    acc.z += __uint_as_float(r[1] << 16);
    acc.w += __uint_as_float(r[1] & 0xFFFF0000u);
  }
  const uint32_t lo = f32_to_bf16_rne(acc.x) | ((uint32_t)f32_to_bf16_rne(acc.y) << 16);
  const uint32_t hi = f32_to_bf16_rne(acc.z) | ((uint32_t)f32_to_bf16_rne(acc.w) << 16);
  *reinterpret_cast<u32x2*>(y + e) = u32x2{lo, hi};
}

// ---- many tokens: several requests verified together, 8 < T <= 64 -----------
//
// Requests verified together (T = requests x (drafts + 1), up to 64) still
// stream every weight once.  By default this kernel serves 8 < T <= 32; from
// 33 tokens the token x column kernels below are faster (it still serves up
// to 64 when forced).  The tokens run in blocks of 16 as the B
// operand's 16 columns (no slot sharing), so each MFMA step covers 32 k of
// one group: step st of a pair reads k-blocks 4 st .. 4 st + 3 (group st / 2),
// k-slot q of a lane taking k-block 4 st + q.  X is too large for LDS (640 KB
// at T = 64, K = 5120), so every wave reads its pair's X slice from memory
// (L2, after the first workgroup of an XCD has fetched it) straight into B
// fragments: lane m of k-slot q takes the 8 k of token 16 tb + m, put into
// the interleaved k order of the unpack in registers.  A pair's unpacked
// weights serve all token blocks, and the -(128 + bias) sum_k x term of each
// group comes from one MFMA chain per token block shared by all columns.  A
// workgroup of kWideWaves waves takes one tile of 16 V columns (V = 3 where
// that makes one tile per CU, as for N = 12288); wave w takes pairs w, w + W,
// ... with two in flight, and the wave sums are added in wave order through
// LDS, 16 tokens at a time.

constexpr int kWideWaves = 4;

struct WideArgs {
  const void* x;
  const void* wq;
  const void* scales;
  void* y;
  int T, K, Nout, Ncols, up_off, G, pairs, ntiles;
  uint32_t p0_bytes, p1_bytes, s_bytes, x_bytes;
  uint32_t mask_nib, mask_base, mask_hi;
};

template <int BITS, int V, int NSETS, int TB>
struct WideBuf {
  static constexpr int WPK = BITS == 8 ? 2 : 1;
  uint32_t a[NSETS][4][V * WPK];             // [set][step][word]; int8: row 2kb words, then 2kb+1
  uint32_t p1[NSETS][4][BITS == 5 ? V : 1];  // int5: the 32-k high-bit word of each step
  uint32_t x[TB][4][4];                      // [token block][step][dword]
  uint32_t sc[NSETS][2][2 * V];              // [set][group][4V 16-bit scales]
};

// LDS of the wave-sum exchange: per wave [set][16 tokens][16 V + 4 columns] fp32
__host__ __device__ constexpr uint32_t wide_block_floats(int nsets, int v) {
  return (uint32_t)nsets * 16u * (16u * (uint32_t)v + 4u);
}

template <int BITS, bool SBF16, int V, int NSETS, int TB>
__global__ __launch_bounds__(kWideWaves * 64) void gemm_wide_kernel(WideArgs a) {
  constexpr int W = kWideWaves, TILE = 16 * V, WPK = BITS == 8 ? 2 : 1, NB = 2;
  constexpr uint32_t BLK = wide_block_floats(NSETS, V), ROW = TILE + 4;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float* const part = reinterpret_cast<float*>(smem);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15, q = lane >> 4;
  // XCD-aware tile order, as in gemm_kernel
  const int b = blockIdx.x, xcd = b & 7, per = a.ntiles >> 3, rem = a.ntiles & 7;
  const int tile = xcd * per + min(xcd, rem) + (b >> 3);
  const int c0 = tile * TILE;
  // Every workgroup reads the same X.  Starting each tile at a different pair
  // (the pair order rotated by the tile index) keeps the workgroups of an XCD
  // on different X lines at any moment instead of all queueing for the same
  // few L2 lines.
  const int rot = a.pairs > 0 ? tile % a.pairs : 0;

  const __amdgpu_buffer_rsrc_t rW = make_rsrc(a.wq, a.p0_bytes);
  const __amdgpu_buffer_rsrc_t rP1 = make_rsrc(static_cast<const char*>(a.wq) + a.p0_bytes, a.p1_bytes);
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(a.scales, a.s_bytes);
  uint32_t vbase = a.mask_base;
  asm volatile("" : "+v"(vbase));
  const UnpackMasks mk{a.mask_nib, vbase, a.mask_hi};

  const uint32_t rowb = (uint32_t)a.Ncols * 4u;
  uint32_t offA[NSETS], offC[NSETS], offS[NSETS];
#pragma unroll
  for (int s = 0; s < NSETS; ++s) {
    offC[s] = (uint32_t)(c0 + s * a.up_off + V * m) * 4u;
    offA[s] = (uint32_t)q * WPK * rowb + offC[s];
    offS[s] = (uint32_t)(c0 + s * a.up_off + 4 * V * q) * 2u;
  }
  uint32_t offX[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int t = 16 * tb + m;
    offX[tb] = t < a.T ? (uint32_t)t * (uint32_t)a.K * 2u + (uint32_t)q * 16u : kOOB;
  }

  // loads of the v-th pair of the rotated order (wave uniform; v >= pairs
  // loads nothing)
  auto issue = [&](WideBuf<BITS, V, NSETS, TB>& buf, int v) {
    const bool valid = v < a.pairs;
    const int p = v + rot < a.pairs ? v + rot : v + rot - a.pairs;
    // last pair of an odd group count: its second group does not exist (its
    // weight, high-bit and scale rows lie past their buffers, but its X
    // offsets would run into the next token's row, so they are cut here)
    const bool half = (p == a.pairs - 1) & ((a.G & 1) != 0);
    const uint32_t pa = valid ? (uint32_t)p * 16u * WPK * rowb : kOOB;
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int s = 0; s < NSETS; ++s) {
        const uint32_t o = offA[s] + pa + (uint32_t)st * 4u * WPK * rowb;
        load_words<V, kNT>(&buf.a[s][st][0], rW, o);
        if constexpr (BITS == 8) load_words<V, kNT>(&buf.a[s][st][V], rW, o + rowb);
      }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const bool on = valid & !(half & (st >= 2));
        load_words<4>(&buf.x[tb][st][0], rX, on ? offX[tb] + (uint32_t)p * 256u + (uint32_t)st * 64u : kOOB);
      }
    if constexpr (BITS == 5) {
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int s = 0; s < NSETS; ++s)
          load_words<V>(&buf.p1[s][st][0], rP1, valid ? (uint32_t)(4 * p + st) * rowb + offC[s] : kOOB);
    }
#pragma unroll
    for (int s = 0; s < NSETS; ++s)
#pragma unroll
      for (int g = 0; g < 2; ++g)
        load_words<2 * V>(&buf.sc[s][g][0], rS,
                          valid ? (uint32_t)(2 * p + g) * (uint32_t)a.Ncols * 2u + offS[s] : kOOB);
  };

  f32x4 acc[TB][NSETS][V];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int s = 0; s < NSETS; ++s)
#pragma unroll
      for (int i = 0; i < V; ++i) acc[tb][s][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const u32x4 negoff = {Code<BITS>::neg_offset_bf16 * 0x10001u, Code<BITS>::neg_offset_bf16 * 0x10001u,
                        Code<BITS>::neg_offset_bf16 * 0x10001u, Code<BITS>::neg_offset_bf16 * 0x10001u};

  auto compute = [&](const WideBuf<BITS, V, NSETS, TB>& buf) {
    u32x4 av[4][NSETS][V];
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int s = 0; s < NSETS; ++s)
#pragma unroll
        for (int i = 0; i < V; ++i) {
          if constexpr (BITS == 4) {
            av[st][s][i] = nibbles_to_bf16_il(buf.a[s][st][i], mk);
          } else if constexpr (BITS == 5) {
            // k-block 4 st + q is byte q of the step's 32-k high-bit word
            const uint32_t p1 = buf.p1[s][st][i];
            av[st][s][i] = nibbles5_to_bf16_il(buf.a[s][st][i], hb_spread(p1, p1 << 4, hb_select((uint32_t)q)), mk);
          } else {
            av[st][s][i] = bytes_to_bf16_il(buf.a[s][st][i], buf.a[s][st][V + i]);
          }
        }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      bf16x8 bfrag[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) bfrag[st] = __builtin_bit_cast(bf16x8, interleave_x(buf.x[tb][st]));
#pragma unroll
      for (int gr = 0; gr < 2; ++gr) {
        f32x4 dx = {0.f, 0.f, 0.f, 0.f};
        dx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, negoff), bfrag[2 * gr], dx, 0, 0, 0);
        dx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, negoff), bfrag[2 * gr + 1], dx, 0, 0,
                                                     0);
#pragma unroll
        for (int s = 0; s < NSETS; ++s)
#pragma unroll
          for (int i = 0; i < V; ++i) {
            f32x4 dp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[2 * gr][s][i]),
                                                               bfrag[2 * gr], dx, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[2 * gr + 1][s][i]),
                                                         bfrag[2 * gr + 1], dp, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int e = V * r + i;
              const float sc = scale_to_f32(buf.sc[s][gr][e >> 1], e & 1, SBF16);
              acc[tb][s][i][r] = __builtin_fmaf(sc, dp[r], acc[tb][s][i][r]);
            }
          }
      }
    }
  };

  // two pairs in flight per wave; loads are issued without a branch (a pair
  // past the end loads nothing), and the scheduling barriers keep the pairs'
  // loads in issue order, so each compute waits for exactly its own pair
  WideBuf<BITS, V, NSETS, TB> buf[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    issue(buf[u], wave + W * u);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int k = wave; k < a.pairs; k += NB * W) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int p = k + W * u;
      if (p < a.pairs) compute(buf[u]);
      __builtin_amdgcn_sched_barrier(0);
      issue(buf[u], p + NB * W);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // the wave sums, 16 tokens at a time: each wave writes its block, then the
  // outputs add the W blocks in wave order
  uint16_t* const y = static_cast<uint16_t*>(a.y);
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    if (tb > 0) __syncthreads();  // the previous round's blocks are read
    float* const blk = part + (uint32_t)wave * BLK;
#pragma unroll
    for (int s = 0; s < NSETS; ++s)
#pragma unroll
      for (int i = 0; i < V; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          blk[((uint32_t)s * 16u + (uint32_t)m) * ROW + (uint32_t)(V * (4 * q + r) + i)] = acc[tb][s][i][r];
    __syncthreads();
    for (int idx = threadIdx.x; idx < 16 * TILE; idx += W * 64) {
      const int tt = idx / TILE, col = idx % TILE, t = 16 * tb + tt;
      if (t >= a.T || c0 + col >= a.Nout) continue;
      float v[NSETS];
#pragma unroll
      for (int s = 0; s < NSETS; ++s) {
        const float* src = part + ((uint32_t)s * 16u + (uint32_t)tt) * ROW + (uint32_t)col;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) sum += src[(uint32_t)w * BLK];
        v[s] = sum;
      }
      float out;
      if constexpr (NSETS == 2) {
        out = v[0] * v[1] / (1.0f + expf(-v[0]));  // SiLU(gate) * up
      } else {
        out = v[0];
      }
      y[(size_t)t * a.Nout + c0 + col] = f32_to_bf16_rne(out);
    }
  }
}

// ---- prefill-size T: token x column tiles ----------------------------------
//
// A prefill chunk (hundreds to thousands of tokens, the engine's
// `--prefill-chunk` on the NInfer-4090 V3 topic) reuses every weight across
// many tokens, so the work is a dense contraction and the MFMA units, not
// the weight stream, set the pace.  One workgroup owns a tile of 64 weight
// columns (64 output columns, or 32 gate + 32 up columns with the SwiGLU
// epilogue) by 64 tokens; its 4 waves split K, wave w taking the groups
// g = w, w + 4, ...  Per group a wave unpacks its 64 columns once (two 32-k
// steps, the interleaved order of the decode kernels) and multiplies them
// with 4 token blocks of 16: 32 MFMAs plus 8 for the -(128 + bias) sum_k x
// term, then acc += s * partial per group.  Weights, scales and X go from
// memory straight into registers, NB groups ahead.  The 4 wave sums meet in
// LDS and are added in wave order (deterministic, no atomics).  Where 64
// columns per tile leave CUs idle (tens of tokens, or few columns) a plain
// projection's tiles narrow to 32 or 16 columns (V = 2 or 1 per lane): less
// unpack and MFMA work per group and wave, more workgroups.

constexpr int kTiledWaves = 4;
constexpr int kTiledTok = 64;   // tokens per tile: 4 MFMA token blocks
constexpr int kTiledCols = 64;  // weight columns per tile: 16 lanes x 4

struct TiledArgs {
  const void* x;
  const void* wq;
  const void* scales;
  void* y;
  int T, K, Nout, Ncols, up_off, G, tiles_n, tiles;
  uint32_t p0_bytes, p1_bytes, s_bytes, x_bytes;
  uint32_t mask_nib, mask_base, mask_hi;
};

// LDS of the wave-sum exchange: per wave 64 values per lane
// (e accumulators per lane: 16 NSETS V, at most 64)
__host__ __device__ constexpr uint32_t tiled_lds_bytes(int e) {
  return (uint32_t)kTiledWaves * (uint32_t)e * 64u * 4u;
}

template <int BITS, int NSETS, int V_ = 4 / NSETS>
struct TiledBuf {
  static constexpr int V = V_, WPK = BITS == 8 ? 2 : 1;
  uint32_t a[NSETS][2][V * WPK];             // [set][32-k step][word]; int8: row 2kb words, then 2kb+1
  uint32_t p1[NSETS][2][BITS == 5 ? V : 1];  // int5: the step's 32-k high-bit word
  uint32_t sc[NSETS][2 * V];                 // 4V 16-bit scales per set
  uint32_t x[4][2][4];                       // [token block][step][dword]
};

// The weight side of a wave's 16 V NSETS columns (64 unless the K-split
// kernel narrows its tiles) in the token x column kernels:
// lane (m, q) loads, per set s and 32-k step, V adjacent P0 words of columns
// c0 + s up_off + V m .. at 8-k block 8 g + 4 ks + q (two rows for int8),
// the int5 high-bit words of the same columns, and the 4V scales of columns
// c0 + s up_off + 4 V q ...  Columns past the matrix read the next row or
// nothing: only their own (discarded) outputs see them.
template <int BITS, int NSETS, int V_ = 4 / NSETS>
struct TileWeights {
  static constexpr int V = V_, WPK = BITS == 8 ? 2 : 1;
  __amdgpu_buffer_rsrc_t rW, rP1, rS;
  uint32_t rowb, srow, offA[NSETS], offP1[NSETS], offS[NSETS];

  __device__ __forceinline__ TileWeights(const TiledArgs& a, int c0, int m, int q) {
    rW = make_rsrc(a.wq, a.p0_bytes);
    rP1 = make_rsrc(static_cast<const char*>(a.wq) + a.p0_bytes, a.p1_bytes);
    rS = make_rsrc(a.scales, a.s_bytes);
    rowb = (uint32_t)a.Ncols * 4u;
    srow = (uint32_t)a.Ncols * 2u;
#pragma unroll
    for (int s = 0; s < NSETS; ++s) {
      const uint32_t col = (uint32_t)(c0 + s * a.up_off + V * m);
      offA[s] = (uint32_t)q * WPK * rowb + col * 4u;
      offP1[s] = col * 4u;
      offS[s] = (uint32_t)(c0 + s * a.up_off + 4 * V * q) * 2u;
    }
  }

  // group g's words and scales into `buf` (nothing when !valid)
  template <class Buf>
  __device__ __forceinline__ void issue(Buf& buf, int g, bool valid) const {
    const uint32_t ga = valid ? (uint32_t)g * 8u * WPK * rowb : kOOB;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int s = 0; s < NSETS; ++s) {
        const uint32_t o = offA[s] + ga + (uint32_t)ks * 4u * WPK * rowb;
        load_words<V>(&buf.a[s][ks][0], rW, o);
        if constexpr (BITS == 8) load_words<V>(&buf.a[s][ks][V], rW, o + rowb);
      }
    if constexpr (BITS == 5) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int s = 0; s < NSETS; ++s)
          load_words<V>(&buf.p1[s][ks][0], rP1, valid ? (uint32_t)(2 * g + ks) * rowb + offP1[s] : kOOB);
    }
#pragma unroll
    for (int s = 0; s < NSETS; ++s)
      load_words<2 * V>(&buf.sc[s][0], rS, valid ? (uint32_t)g * srow + offS[s] : kOOB);
  }
};

// One group (64 k) of a token x column tile for one wave: the offset chain
// -(128 + bias) sum_k x per token block, then per weight column the two
// 32-k steps unpacked once and multiplied with the 4 token blocks' B
// fragments `bfr`, each group's partial scaled into acc.  Lane (m, q): A row
// m = weight column V m + i of set s, k-slot q.  `buf` holds the group's
// P0 words, int5 high-bit words and scales (TiledBuf or SxBuf).
template <int BITS, bool SBF16, int NSETS, int V, class Buf>
__device__ __forceinline__ void tile_group(const Buf& buf, const bf16x8 (&bfr)[4][2], const UnpackMasks& mk, int q,
                                           f32x4 (&acc)[NSETS][V][4]) {
  const u32x4 negoff = {Code<BITS>::neg_offset_bf16 * 0x10001u, Code<BITS>::neg_offset_bf16 * 0x10001u,
                        Code<BITS>::neg_offset_bf16 * 0x10001u, Code<BITS>::neg_offset_bf16 * 0x10001u};
  f32x4 dx[4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    dx[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, negoff), bfr[tb][0],
                                                     f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    dx[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, negoff), bfr[tb][1], dx[tb], 0, 0, 0);
  }
#pragma unroll
  for (int s = 0; s < NSETS; ++s)
#pragma unroll
    for (int i = 0; i < V; ++i) {
      u32x4 av[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if constexpr (BITS == 4) {
          av[ks] = nibbles_to_bf16_il(buf.a[s][ks][i], mk);
        } else if constexpr (BITS == 5) {
          // k-block 4 ks + q is byte q of the step's 32-k high-bit word
          const uint32_t p1 = buf.p1[s][ks][i];
          av[ks] = nibbles5_to_bf16_il(buf.a[s][ks][i], hb_spread(p1, p1 << 4, hb_select((uint32_t)q)), mk);
        } else {
          av[ks] = bytes_to_bf16_il(buf.a[s][ks][i], buf.a[s][ks][V + i]);
        }
      }
      float sc[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = V * r + i;
        sc[r] = scale_to_f32(buf.sc[s][e >> 1], e & 1, SBF16);
      }
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        f32x4 dp =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[0]), bfr[tb][0], dx[tb], 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[1]), bfr[tb][1], dp, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[s][i][tb][r] = __builtin_fmaf(sc[r], dp[r], acc[s][i][tb][r]);
      }
    }
}

template <int BITS, bool SBF16, int NSETS, int NB, int V>
__global__ __launch_bounds__(kTiledWaves * 64) void gemm_tiled_kernel(TiledArgs a) {
  static_assert(NSETS == 2 ? V == 2 : V == 4 || V == 2 || V == 1, "column tile");
  constexpr int W = kTiledWaves;
  constexpr int OCOLS = 16 * V;     // output columns per tile
  constexpr int E = NSETS * V * 16;  // accumulators per lane (16-64)
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float* const part = reinterpret_cast<float*>(smem);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15, q = lane >> 4;
  // XCD-aware order: each XCD (block b runs on XCD b % 8) takes a contiguous
  // range of tiles, token tile slowest, so the workgroups of one XCD share
  // the X rows of a token tile in its L2
  const int b = blockIdx.x, xcd = b & 7, per = a.tiles >> 3, rem = a.tiles & 7;
  const int tile = xcd * per + min(xcd, rem) + (b >> 3);
  const int tt = tile / a.tiles_n, tn = tile - tt * a.tiles_n;
  const int t0 = tt * kTiledTok, c0 = tn * OCOLS;

  const __amdgpu_buffer_rsrc_t rX = make_rsrc(a.x, a.x_bytes);
  uint32_t vbase = a.mask_base;
  asm volatile("" : "+v"(vbase));
  const UnpackMasks mk{a.mask_nib, vbase, a.mask_hi};

  // Lane (m, q) supplies, for set s and column i < V, operand row m of the
  // A block (weight column c0 + s up_off + V m + i) at the 8 k of slot q, and
  // token 16 tb + m of the B block; its results are rows 4q + r (weight
  // columns c0 + s up_off + V (4q + r) + i) for token 16 tb + m.
  const TileWeights<BITS, NSETS, V> tw(a, c0, m, q);
  uint32_t offX[4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    const int t = t0 + 16 * tb + m;
    offX[tb] = t < a.T ? (uint32_t)t * (uint32_t)a.K * 2u + (uint32_t)q * 16u : kOOB;
  }

  // loads of group g (g >= G loads nothing)
  auto issue = [&](TiledBuf<BITS, NSETS, V>& buf, int g) {
    const bool valid = g < a.G;
    tw.issue(buf, g, valid);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        load_words<4>(&buf.x[tb][ks][0], rX, valid ? offX[tb] + (uint32_t)g * 128u + (uint32_t)ks * 64u : kOOB);
  };

  f32x4 acc[NSETS][V][4];
#pragma unroll
  for (int s = 0; s < NSETS; ++s)
#pragma unroll
    for (int i = 0; i < V; ++i)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) acc[s][i][tb] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const TiledBuf<BITS, NSETS, V>& buf) {
    bf16x8 bfr[4][2];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) bfr[tb][ks] = __builtin_bit_cast(bf16x8, interleave_x(buf.x[tb][ks]));
    tile_group<BITS, SBF16, NSETS>(buf, bfr, mk, q, acc);
  };

  // NB groups in flight per wave; loads are issued without a branch (a group
  // past the end loads nothing), and the scheduling barriers keep the groups'
  // loads in issue order, so each compute waits for exactly its own group
  TiledBuf<BITS, NSETS, V> buf[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    issue(buf[u], wave + W * u);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int g = wave; g < a.G; g += NB * W) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int gg = g + W * u;
      if (gg < a.G) compute(buf[u]);
      __builtin_amdgcn_sched_barrier(0);
      issue(buf[u], gg + NB * W);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // the wave sums: value e of lane l of wave w at part[(w E + e) 64 + l]
#pragma unroll
  for (int s = 0; s < NSETS; ++s)
#pragma unroll
    for (int i = 0; i < V; ++i)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = ((s * V + i) * 4 + tb) * 4 + r;
          part[((uint32_t)wave * E + (uint32_t)e) * 64u + (uint32_t)lane] = acc[s][i][tb][r];
        }
  __syncthreads();
  // wave w finishes token block w: the four wave sums in wave order, then
  // SwiGLU or plain, V consecutive output columns per store (V even, or a
  // single column: N % 4 == 0 keeps every store aligned and inside its row)
  const int tb = wave, t = t0 + 16 * tb + m;
  uint16_t* const y = static_cast<uint16_t*>(a.y);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int col = c0 + V * (4 * q + r);
    if (t >= a.T || col >= a.Nout) continue;
    float v[NSETS][V];
#pragma unroll
    for (int s = 0; s < NSETS; ++s)
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const int e = ((s * V + i) * 4 + tb) * 4 + r;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) sum += part[((uint32_t)w * E + (uint32_t)e) * 64u + (uint32_t)lane];
        v[s][i] = sum;
      }
    uint16_t* const dst = y + (size_t)t * a.Nout + col;
    if constexpr (V == 1) {  // plain projections only
      *dst = f32_to_bf16_rne(v[0][0]);
    } else {
      uint32_t pk[V / 2];
#pragma unroll
      for (int i = 0; i < V; i += 2) {
        float o0, o1;
        if constexpr (NSETS == 2) {
          o0 = v[0][i] * v[1][i] / (1.0f + expf(-v[0][i]));  // SiLU(gate) * up
          o1 = v[0][i + 1] * v[1][i + 1] / (1.0f + expf(-v[0][i + 1]));
        } else {
          o0 = v[0][i];
          o1 = v[0][i + 1];
        }
        pk[i / 2] = (uint32_t)f32_to_bf16_rne(o0) | ((uint32_t)f32_to_bf16_rne(o1) << 16);
      }
      if constexpr (V == 4)
        *reinterpret_cast<u32x2*>(dst) = u32x2{pk[0], pk[1]};
      else
        *reinterpret_cast<uint32_t*>(dst) = pk[0];
    }
  }
}

// Large T: the 4 waves of a workgroup split the columns instead of K.  The
// workgroup owns 256 weight columns (wave w: columns 64 w .. 64 w + 63) by
// 64 tokens and walks every group; the group's X tile (64 tokens x 64 k) is
// loaded once per workgroup, written to LDS in the interleaved k order
// (double-buffered, one barrier per group) and read by all 4 waves, so each
// byte of X fetched from L2 feeds 4x the MFMA work of the K-split kernel.
// Each wave's sums are whole: outputs go from registers straight to memory.

constexpr int kSxCols = 4 * kTiledCols;            // weight columns per workgroup
constexpr int kSxBand = 4;                         // token tiles per band of the tile order
constexpr uint32_t kSxRow = 2u * 64u + 16u;        // LDS bytes per token row of an X tile (padded)
// LDS bytes of one group's X tile of 16 TB token rows
__host__ __device__ constexpr uint32_t sx_buf_bytes(int tb) { return 16u * (uint32_t)tb * kSxRow; }

__host__ __device__ constexpr uint32_t tiled_sx_lds_bytes(int tb) { return 2u * sx_buf_bytes(tb); }

template <int BITS, int NSETS, int TB>
struct SxBuf {
  static constexpr int V = 4 / NSETS, WPK = BITS == 8 ? 2 : 1;
  uint32_t a[NSETS][2][V * WPK];             // as TiledBuf
  uint32_t p1[NSETS][2][BITS == 5 ? V : 1];
  uint32_t sc[NSETS][2 * V];
  uint32_t x[TB / 2][4];                     // this thread's 16-byte chunks of the X tile
};

// tile_group with the token blocks outermost, for the 96- and 128-token
// tiles: the A fragments and scales of all columns first, then per token
// block its B fragments (read by `rb`), its offset chain and its MFMAs, so
// that one block's B fragments live at a time and the kernel keeps two waves
// per SIMD.  The same arithmetic in the same order per output as tile_group.
template <int BITS, bool SBF16, int NSETS, int TB, class Buf, class ReadB>
__device__ __forceinline__ void tile_group_tbo(const Buf& buf, ReadB&& rb, const UnpackMasks& mk, int q,
                                               f32x4 (&acc)[NSETS][4 / NSETS][TB]) {
  constexpr int V = 4 / NSETS;
  const u32x4 negoff = {Code<BITS>::neg_offset_bf16 * 0x10001u, Code<BITS>::neg_offset_bf16 * 0x10001u,
                        Code<BITS>::neg_offset_bf16 * 0x10001u, Code<BITS>::neg_offset_bf16 * 0x10001u};
  u32x4 av[NSETS][V][2];
  float sc[NSETS][V][4];
#pragma unroll
  for (int s = 0; s < NSETS; ++s)
#pragma unroll
    for (int i = 0; i < V; ++i) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if constexpr (BITS == 4) {
          av[s][i][ks] = nibbles_to_bf16_il(buf.a[s][ks][i], mk);
        } else if constexpr (BITS == 5) {
          // k-block 4 ks + q is byte q of the step's 32-k high-bit word
          const uint32_t p1 = buf.p1[s][ks][i];
          av[s][i][ks] = nibbles5_to_bf16_il(buf.a[s][ks][i], hb_spread(p1, p1 << 4, hb_select((uint32_t)q)), mk);
        } else {
          av[s][i][ks] = bytes_to_bf16_il(buf.a[s][ks][i], buf.a[s][ks][V + i]);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = V * r + i;
        sc[s][i][r] = scale_to_f32(buf.sc[s][e >> 1], e & 1, SBF16);
      }
    }
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    bf16x8 b[2];
    rb(b, tb);
    f32x4 dx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, negoff), b[0],
                                                       f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    dx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, negoff), b[1], dx, 0, 0, 0);
#pragma unroll
    for (int s = 0; s < NSETS; ++s)
#pragma unroll
      for (int i = 0; i < V; ++i) {
        f32x4 dp =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[s][i][0]), b[0], dx, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[s][i][1]), b[1], dp, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[s][i][tb][r] = __builtin_fmaf(sc[s][i][r], dp[r], acc[s][i][tb][r]);
      }
  }
}

// TB token blocks of 16 per tile (64, 96 or 128 tokens): more tokens reuse
// each unpacked weight word for more MFMAs; which size fills the CUs best
// depends on the shape (chosen on the host).
template <int BITS, bool SBF16, int NSETS, int NB, int TB>
__global__ __launch_bounds__(kTiledWaves * 64) void gemm_tiled_sx_kernel(TiledArgs a) {
  constexpr int V = 4 / NSETS, XC = TB / 2;  // X chunks per thread and group
  constexpr uint32_t XBUF = sx_buf_bytes(TB);
  constexpr int OCOLS = kSxCols / NSETS;  // output columns per workgroup
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15, q = lane >> 4;
  // XCD-aware order (each XCD a contiguous range of tiles), the range walked
  // in bands of kSxBand token tiles, token tile fastest: the workgroups one
  // XCD runs at a time then share a few token tiles' X and a few column
  // tiles' weights in its L2, instead of one token tile and every column
  // tile's weights
  const int b = blockIdx.x, xcd = b & 7, per = a.tiles >> 3, rem = a.tiles & 7;
  const int tile = xcd * per + min(xcd, rem) + (b >> 3);
  const int tiles_t = a.tiles / a.tiles_n, band = tile / (kSxBand * a.tiles_n);
  const int in_band = tile - band * (kSxBand * a.tiles_n), bt = min(kSxBand, tiles_t - band * kSxBand);
  const int tt = band * kSxBand + in_band % bt, tn = in_band / bt;
  const int t0 = tt * 16 * TB;
  const int c0 = tn * OCOLS + wave * (OCOLS / kTiledWaves);  // this wave's first output column

  const __amdgpu_buffer_rsrc_t rX = make_rsrc(a.x, a.x_bytes);
  uint32_t vbase = a.mask_base;
  asm volatile("" : "+v"(vbase));
  const UnpackMasks mk{a.mask_nib, vbase, a.mask_hi};

  // operand roles of lane (m, q) as in gemm_tiled_kernel, for this wave's columns
  const TileWeights<BITS, NSETS> tw(a, c0, m, q);
  // X tile chunks of this thread: chunk j = tid + 256 u is token row j / 8,
  // 16-byte k chunk j % 8 of the group
  uint32_t offX[XC], ldsX[XC];
#pragma unroll
  for (int u = 0; u < XC; ++u) {
    const int j = (int)threadIdx.x + 256 * u, row = j >> 3, kc = j & 7, t = t0 + row;
    offX[u] = t < a.T ? (uint32_t)t * (uint32_t)a.K * 2u + (uint32_t)kc * 16u : kOOB;
    ldsX[u] = (uint32_t)row * kSxRow + (uint32_t)kc * 16u;
  }
  // B fragment of token block tb, step ks: row 16 tb + m, k chunk 4 ks + q
  const uint32_t ldsB = (uint32_t)m * kSxRow + (uint32_t)q * 16u;

  auto issue = [&](SxBuf<BITS, NSETS, TB>& buf, int g) {
    const bool valid = g < a.G;
    tw.issue(buf, g, valid);
#pragma unroll
    for (int u = 0; u < XC; ++u) load_words<4>(&buf.x[u][0], rX, valid ? offX[u] + (uint32_t)g * 128u : kOOB);
  };

  f32x4 acc[NSETS][V][TB];
#pragma unroll
  for (int s = 0; s < NSETS; ++s)
#pragma unroll
    for (int i = 0; i < V; ++i)
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) acc[s][i][tb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // group g: its X chunks into LDS buffer g % 2, barrier, then the wave's MFMAs
  auto compute = [&](const SxBuf<BITS, NSETS, TB>& buf, int g) {
    uint8_t* const xb = smem + (uint32_t)(g & 1) * XBUF;
#pragma unroll
    for (int u = 0; u < XC; ++u) *reinterpret_cast<u32x4*>(xb + ldsX[u]) = interleave_x(buf.x[u]);
    lds_barrier();
    auto read_b = [&](bf16x8 (&b)[2], int tb) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        b[ks] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(xb + ldsB + (uint32_t)tb * 16u * kSxRow + (uint32_t)ks * 64u));
    };
    if constexpr (TB == 4) {
      bf16x8 bfr[4][2];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) read_b(bfr[tb], tb);
      tile_group<BITS, SBF16, NSETS>(buf, bfr, mk, q, acc);
    } else {
      tile_group_tbo<BITS, SBF16, NSETS, TB>(buf, read_b, mk, q, acc);
    }
  };

  // NB groups in flight; every wave walks every group (the barrier inside
  // compute is reached the same number of times by all waves)
  SxBuf<BITS, NSETS, TB> buf[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    issue(buf[u], u);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int g = 0; g < a.G; g += NB) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      if (g + u < a.G) compute(buf[u], g + u);
      __builtin_amdgcn_sched_barrier(0);
      issue(buf[u], g + u + NB);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // outputs from registers: token t0 + 16 tb + m, V consecutive columns
  // c0 + V (4q + r) .. per (tb, r)
  uint16_t* const y = static_cast<uint16_t*>(a.y);
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int t = t0 + 16 * tb + m;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int col = c0 + V * (4 * q + r);
      if (t >= a.T || col >= a.Nout) continue;
      uint32_t pk[V / 2];
#pragma unroll
      for (int i = 0; i < V; i += 2) {
        float o0, o1;
        if constexpr (NSETS == 2) {
          const float g0 = acc[0][i][tb][r], g1 = acc[0][i + 1][tb][r];
          o0 = g0 * acc[1][i][tb][r] / (1.0f + expf(-g0));  // SiLU(gate) * up
          o1 = g1 * acc[1][i + 1][tb][r] / (1.0f + expf(-g1));
        } else {
          o0 = acc[0][i][tb][r];
          o1 = acc[0][i + 1][tb][r];
        }
        pk[i / 2] = (uint32_t)f32_to_bf16_rne(o0) | ((uint32_t)f32_to_bf16_rne(o1) << 16);
      }
      uint16_t* dst = y + (size_t)t * a.Nout + col;
      if constexpr (V == 4)
        *reinterpret_cast<u32x2*>(dst) = u32x2{pk[0], pk[1]};
      else
        *reinterpret_cast<uint32_t*>(dst) = pk[0];
    }
  }
}

// ---- debug kernels: the GEMM's unpack and scale decoding, materialised ----

template <int BITS, bool SBF16, bool DEQUANT>
__global__ __launch_bounds__(256) void unpack_kernel(const void* wq, uint32_t p0_bytes, const void* scales,
                                                     int K, int N, void* out) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int kb = blockIdx.y;  // 8-k block
  if (n >= N) return;
  const uint32_t* p0 = static_cast<const uint32_t*>(wq);
  u32x4 v;
  if constexpr (BITS == 4) {
    v = nibbles_to_bf16_il(p0[(size_t)kb * N + n], kMasks);
  } else if constexpr (BITS == 5) {
    const uint32_t* p1 = reinterpret_cast<const uint32_t*>(static_cast<const char*>(wq) + p0_bytes);
    const uint32_t hw = p1[(size_t)(kb >> 2) * N + n];
    v = nibbles5_to_bf16_il(p0[(size_t)kb * N + n], hb_spread(hw, hw << 4, hb_select((uint32_t)(kb & 3))), kMasks);
  } else {
    v = bytes_to_bf16_il(p0[(size_t)(2 * kb) * N + n], p0[(size_t)(2 * kb + 1) * N + n]);
  }
  float sc = 1.0f;
  if constexpr (DEQUANT) {
    const uint32_t* s32 = static_cast<const uint32_t*>(scales);
    const size_t si = (size_t)(kb / 8) * N + n;
    sc = scale_to_f32(s32[si >> 1], (int)(si & 1), SBF16);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    // element e of the interleaved block is k = (e >> 1) + 4 (e & 1)
    const uint32_t bits16 = (v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
    const float val = __uint_as_float(bits16 << 16) - (float)Code<BITS>::offset;  // the code, exact
    const size_t o = (size_t)(8 * kb + (e >> 1) + 4 * (e & 1)) * N + n;
    if constexpr (DEQUANT)
      static_cast<float*>(out)[o] = val * sc;
    else
      static_cast<int8_t*>(out)[o] = (int8_t)(int)val;
  }
}

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ buf, size_t n16,
                                                          uint32_t* sink) {
  uint32_t x = 0;
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a0 = __builtin_nontemporal_load(&buf[i]);
    const u32x4 a1 = __builtin_nontemporal_load(&buf[i + stride]);
    const u32x4 a2 = __builtin_nontemporal_load(&buf[i + 2 * stride]);
    const u32x4 a3 = __builtin_nontemporal_load(&buf[i + 3 * stride]);
    x ^= a0[0] ^ a0[1] ^ a0[2] ^ a0[3] ^ a1[0] ^ a1[1] ^ a1[2] ^ a1[3];
    x ^= a2[0] ^ a2[1] ^ a2[2] ^ a2[3] ^ a3[0] ^ a3[1] ^ a3[2] ^ a3[3];
  }
  for (; i < n16; i += stride) {
    const u32x4 a0 = buf[i];
    x ^= a0[0] ^ a0[1] ^ a0[2] ^ a0[3];
  }
  // one word per workgroup: xor-reduce through LDS
  __shared__ uint32_t part[256];
  part[threadIdx.x] = x;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) part[threadIdx.x] ^= part[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0];
}

// The partial-sum area of ngq_gemm_splitk_static: a fixed array in device
// memory (each device the library runs on holds its own copy for the life of
// the process), for callers that cannot allocate.  Host code never passes its
// name to a kernel: the device address comes from hipGetSymbolAddress.
constexpr size_t kStaticScratchBytes = NGQ_STATIC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

// The weight stream of gemm_stream_kernel alone: the same tiles, waves, pair
// order and loads (weights, int5 high bits, scales; nontemporal), one pair in
// flight per wave and the next requested as soon as it lands, but no X, no
// compute and no output beyond a checksum.  Its time per launch is the
// attainable time of the projection's weight stream in this access pattern,
// which the bench reports beside the 8 TB/s peak.  sink[block] = XOR of the
// packed P0 words the workgroup read (each read once);
// sink[gridDim + block] = a sum over the other words (keeps their loads).
template <int BITS, int V, int W>
__global__ __launch_bounds__(W * 64) void stream_tiles_kernel(GemmArgs a, uint32_t* sink) {
  constexpr int WPK = BITS == 8 ? 2 : 1;
  constexpr int TILE = 16 * V;
  __shared__ uint32_t red[2][W];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15, q = lane >> 4, h = m >> 3;
  const int b = blockIdx.x;
  const int xcd = b & 7, per = a.ntiles >> 3, rem = a.ntiles & 7;
  const int tile = xcd * per + min(xcd, rem) + (b >> 3);
  const uint32_t c0 = (uint32_t)(tile * TILE);
  const __amdgpu_buffer_rsrc_t rW = make_rsrc(a.wq, a.p0_bytes);
  const __amdgpu_buffer_rsrc_t rP1 = make_rsrc(static_cast<const char*>(a.wq) + a.p0_bytes, a.p1_bytes);
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(a.scales, a.s_bytes);
  const uint32_t rowb = (uint32_t)a.Ncols * 4u;
  const uint32_t lane_kb = 8u * (uint32_t)(q >> 1) + (uint32_t)(q & 1);
  const uint32_t col = c0 + (uint32_t)(V * m);
  const uint32_t offA = lane_kb * WPK * rowb + col * 4u;
  const uint32_t offP1 = 2u * (uint32_t)(q >> 1) * rowb + col * 4u;
  const uint32_t offS = (uint32_t)h * (uint32_t)a.Ncols * 2u + (c0 + (uint32_t)(4 * V * q)) * 2u;
  struct Buf {
    uint32_t a[4][V * WPK];
    uint32_t p1[2][BITS == 5 ? V : 1];
    uint32_t sc[2 * V];
  };
  auto issue = [&](Buf& buf, int p) {
    const bool valid = p < a.pairs;
    const uint32_t pa = valid ? (uint32_t)p * 16u * WPK * rowb : kOOB;
    const uint32_t pp1 = valid ? (uint32_t)p * 4u * rowb : kOOB;
    const uint32_t ps = valid ? (uint32_t)p * rowb : kOOB;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const uint32_t o = offA + pa + (uint32_t)st * 2u * WPK * rowb;
      load_words<V, kNT>(&buf.a[st][0], rW, o);
      if constexpr (BITS == 8) load_words<V, kNT>(&buf.a[st][V], rW, o + rowb);
    }
    if constexpr (BITS == 5) {
      load_words<V, kNT>(&buf.p1[0][0], rP1, offP1 + pp1);
      load_words<V, kNT>(&buf.p1[1][0], rP1, offP1 + pp1 + rowb);
    }
    load_words<2 * V, kNT>(&buf.sc[0], rS, offS + ps);
  };
  uint32_t x = 0, other = 0;
  auto consume = [&](const Buf& buf) {
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int i = 0; i < V * WPK; ++i) x ^= buf.a[st][i];
    if constexpr (BITS == 5) {
#pragma unroll
      for (int i = 0; i < V; ++i) other += buf.p1[0][i] + buf.p1[1][i];
    }
#pragma unroll
    for (int i = 0; i < 2 * V; ++i) other += buf.sc[i];
  };
  Buf buf[2];
  auto pair_of = [&](int i) { return wave + W * i; };
  issue(buf[0], pair_of(0));
  __builtin_amdgcn_sched_barrier(0);
  for (int i = 0; i < a.ppw; i += 2) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    issue(buf[1], pair_of(i + 1));
    __builtin_amdgcn_sched_barrier(0);
    consume(buf[0]);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    issue(buf[0], pair_of(i + 2));
    __builtin_amdgcn_sched_barrier(0);
    consume(buf[1]);
    __builtin_amdgcn_sched_barrier(0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // lanes, then waves (an out-of-range pair loaded zeros: no effect)
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    x ^= __shfl_xor(x, off);
    other += __shfl_xor(other, off);
  }
  if (lane == 0) {
    red[0][wave] = x;
    red[1][wave] = other;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t rx = 0, ro = 0;
    for (int w = 0; w < W; ++w) {
      rx ^= red[0][w];
      ro += red[1][w];
    }
    sink[blockIdx.x] = rx;
    sink[gridDim.x + blockIdx.x] = ro;
  }
}

}  // namespace dev

// ---- host side: configuration and launch ------------------------------------

namespace {

constexpr uint32_t kMaxLds = 160u * 1024u;  // LDS of one CDNA4 workgroup

// Kernel path forced by ngq_debug_force_kernel (NGQ_KERNEL_AUTO: the library
// chooses per shape).
std::atomic<int> kernel_override{NGQ_KERNEL_AUTO};

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  static std::atomic<int> cache[64];  // zero-initialised (static storage); 0 = not yet read
  const bool cached = dev >= 0 && dev < 64;
  if (cached) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (cached) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Raises a kernel's dynamic LDS limit from the default 64 KiB to the 160 KiB
// of a CDNA4 workgroup on the current device.  A function attribute belongs
// to a device, so `done` (one per kernel) keeps a bit per device index; two
// threads that both see the bit clear both make the call, which is
// idempotent.
hipError_t raise_lds(const void* kern, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev >= 0 && dev < 64 ? 1ull << dev : 0ull;
  if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
  if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_release);
  return e;
}

// Columns per lane V in [vmin, vmax]: the tile count should fill the CUs in
// whole rounds (one workgroup per CU at a time).  Efficiency = tiles / (rounds
// * CUs); on a tie prefer the larger V when the rounds are full (fewer, longer
// tiles), else the smaller V (more CUs busy in the last round).
int choose_v(int N, int cus, int vmin, int vmax) {
  vmin = std::min(vmin, vmax);
  int best_v = vmin;
  double best_eff = -1.0;
  for (int v = vmax; v >= vmin; --v) {
    const long tiles = (N + 16L * v - 1) / (16L * v);
    const long rounds = (tiles + cus - 1) / cus;
    const double eff = (double)tiles / (double)(rounds * cus);
    const bool full = eff > 0.999;
    if (eff > best_eff + 1e-9 || (!full && eff > best_eff - 1e-9)) {
      best_eff = eff;
      best_v = v;
    }
  }
  return best_v;
}

// One instantiation.  Its LDS (X staging + partial-sum blocks) can exceed the
// default 64 KiB dynamic limit, which is then raised (raise_lds).
template <int BITS, bool SBF16, int V, int NSETS, bool DYN>
hipError_t launch_one(const dev::GemmArgs& a, uint32_t lds, hipStream_t st) {
  auto kern = dev::gemm_kernel<BITS, SBF16, V, NSETS, DYN>;
  static std::atomic<uint64_t> raised{0};
  if (lds > 64u * 1024u) {
    const hipError_t e = raise_lds(reinterpret_cast<const void*>(kern), raised);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)a.ntiles), dim3(dev::kThreads), lds, st, a);
  return hipGetLastError();
}

// X-resident kernel configurations (measured on MI355X): 14 waves with one
// pair in flight each for a single round of 32-column tiles, 8 waves with two
// pairs each otherwise.  XL covers T K <= XL * W * 512.
struct XCfg {
  int W, NB, XL;
};
constexpr XCfg kX14 = {14, 1, 6}, kX8a = {8, 2, 10}, kX8b = {8, 2, 18};

// Token x column tiles: groups in flight per wave, and the smallest T routed
// to them rather than to the 8 < T <= 64 kernel.
constexpr int kTiledNB = 2, kSxNB = 2;  // 3 in flight measured 2-4 % slower for the shared-X kernel
// The K-split kernel's plain tiles narrow from 64 to 32 and 16 columns (V =
// 4, 2, 1) while the wider tiles would leave CUs without a workgroup and
// the narrower ones fit one round; this is the narrowest allowed.
constexpr int kTiledMinV = 1;
// shared-X tiles once there are at least 0.6 per CU (measured crossover:
// QK at T = 256, 0.5 per CU, is faster K-split; down at T = 512, 0.63 per CU,
// shared)
constexpr int kSxMinTiles10PerCu = 6;
constexpr int kTiledFromT = 33;  // measured: from 33 tokens on, its 64-token tiles beat the 64-row verify kernel

// Widest tile (columns per lane) that compiles without register spills.
constexpr int xres_vmax(int bits, int nsets, int xl) {
  if (nsets == 2) return bits == 8 ? 1 : 2;
  return bits == 8 ? 2 : (bits == 5 && xl == kX8b.XL ? 3 : 4);
}

template <int BITS, bool SBF16, int V, int NSETS, int W, int NB, int XL>
hipError_t launch_xres_one(const dev::GemmArgs& a, int grid, uint32_t lds, hipStream_t st) {
  auto kern = dev::gemm_xres_kernel<BITS, SBF16, V, NSETS, W, NB, XL>;
  static std::atomic<uint64_t> raised{0};
  if (lds > 64u * 1024u) {
    const hipError_t e = raise_lds(reinterpret_cast<const void*>(kern), raised);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(W * 64), lds, st, a);
  return hipGetLastError();
}

// v is at most xres_vmax(BITS, NSETS, XL) (the caller chose it so); only those
// widths are instantiated.
template <int BITS, bool SBF16, int NSETS, int W, int NB, int XL>
hipError_t launch_xres_vx(int v, const dev::GemmArgs& a, int grid, uint32_t lds, hipStream_t st) {
  constexpr int VM = xres_vmax(BITS, NSETS, XL);
  if constexpr (VM >= 4) {
    if (v >= 4) return launch_xres_one<BITS, SBF16, 4, NSETS, W, NB, XL>(a, grid, lds, st);
  }
  if constexpr (VM >= 3) {
    if (v == 3) return launch_xres_one<BITS, SBF16, 3, NSETS, W, NB, XL>(a, grid, lds, st);
  }
  if constexpr (VM >= 2) {
    if (v == 2) return launch_xres_one<BITS, SBF16, 2, NSETS, W, NB, XL>(a, grid, lds, st);
  }
  return launch_xres_one<BITS, SBF16, 1, NSETS, W, NB, XL>(a, grid, lds, st);
}

template <int BITS, bool SBF16, int NSETS>
hipError_t launch_xres_v(const XCfg& c, int v, const dev::GemmArgs& a, int grid, uint32_t lds, hipStream_t st) {
  if (c.W == kX14.W) {
    if constexpr (NSETS == 1) return launch_xres_vx<BITS, SBF16, 1, kX14.W, kX14.NB, kX14.XL>(v, a, grid, lds, st);
  }
  if (c.XL == kX8a.XL) return launch_xres_vx<BITS, SBF16, NSETS, kX8a.W, kX8a.NB, kX8a.XL>(v, a, grid, lds, st);
  return launch_xres_vx<BITS, SBF16, NSETS, kX8b.W, kX8b.NB, kX8b.XL>(v, a, grid, lds, st);
}

template <int NSETS>
hipError_t launch_xres(const Format& f, const XCfg& c, int v, const dev::GemmArgs& a, int grid, uint32_t lds,
                       hipStream_t st) {
  if (f.bits == 4)
    return f.scale_bf16 ? launch_xres_v<4, true, NSETS>(c, v, a, grid, lds, st)
                        : launch_xres_v<4, false, NSETS>(c, v, a, grid, lds, st);
  if (f.bits == 5)
    return f.scale_bf16 ? launch_xres_v<5, true, NSETS>(c, v, a, grid, lds, st)
                        : launch_xres_v<5, false, NSETS>(c, v, a, grid, lds, st);
  return f.scale_bf16 ? launch_xres_v<8, true, NSETS>(c, v, a, grid, lds, st)
                      : launch_xres_v<8, false, NSETS>(c, v, a, grid, lds, st);
}

template <int BITS, bool SBF16, int NSETS, bool DYN>
hipError_t launch_v(int v, const dev::GemmArgs& a, uint32_t lds, hipStream_t st) {
  if constexpr (NSETS == 1) {
    switch (v) {
      case 1: return launch_one<BITS, SBF16, 1, 1, DYN>(a, lds, st);
      case 2: return launch_one<BITS, SBF16, 2, 1, DYN>(a, lds, st);
      case 3: return launch_one<BITS, SBF16, 3, 1, DYN>(a, lds, st);
      default: return launch_one<BITS, SBF16, 4, 1, DYN>(a, lds, st);
    }
  } else {
    switch (v) {
      case 1: return launch_one<BITS, SBF16, 1, 2, DYN>(a, lds, st);
      default: return launch_one<BITS, SBF16, 2, 2, DYN>(a, lds, st);
    }
  }
}

template <int NSETS, bool DYN>
hipError_t launch_fmt(const Format& f, int v, const dev::GemmArgs& a, uint32_t lds, hipStream_t st) {
  if (f.bits == 4)
    return f.scale_bf16 ? launch_v<4, true, NSETS, DYN>(v, a, lds, st) : launch_v<4, false, NSETS, DYN>(v, a, lds, st);
  if (f.bits == 5)
    return f.scale_bf16 ? launch_v<5, true, NSETS, DYN>(v, a, lds, st) : launch_v<5, false, NSETS, DYN>(v, a, lds, st);
  return f.scale_bf16 ? launch_v<8, true, NSETS, DYN>(v, a, lds, st) : launch_v<8, false, NSETS, DYN>(v, a, lds, st);
}

// The streaming single-round kernels: one workgroup per tile of 32 columns
// (16 where N is narrower), LDS under 64 KiB, the X load class following T.
// Waves per workgroup: 10 for int4 and int5; for int8, whose pair of a
// 32-column tile is twice as large, 5 (MFMA step) and 8 (VALU step).  A
// weights-only stream of the int8 QK-shape tiles took 9.78 us with 5 waves,
// 10.11 with 6, 10.28 with 8 and 10.32 with 10 (int4: 10 waves best, 6.08 us
// against 6.52 with 12 and 6.66 with 8); in an interleaved A/B of the whole
// kernels, int8 with 5 streaming waves took 10.41, 10.31, 10.90 us at T = 2,
// 4, 8 against 10.66, 10.70, 11.13 for the 14-wave X-resident kernel, and
// the VALU step with 7 waves 10.00 at T = 1 against 10.23-10.26 with 8, 10.24
// with 6, 10.75 with 9 and 10.77 with 10.
constexpr int kStreamW = 10;
constexpr int kStreamW8 = 5;
constexpr int kStreamW2 = 5;  // SwiGLU (two output sets), whose pairs are twice as large
constexpr int kStreamSwigluMaxT = 4;
constexpr int kDotW8 = 7;
constexpr int kDotW2 = 7;  // SwiGLU (two output sets): three workgroups a CU at 81 VGPRs
// int8 at T >= 2 on the streaming kernel (else the 14-wave X-resident one)
constexpr bool kInt8Stream = true;
constexpr int stream_waves(int bits, int nsets = 1) {
  return nsets == 2 ? kStreamW2 : (bits == 8 ? kStreamW8 : kStreamW);
}
constexpr int dot_waves(int bits, int nsets = 1) { return nsets == 2 ? kDotW2 : (bits == 8 ? kDotW8 : kStreamW); }

template <int BITS, bool SBF16, int V, int NSETS>
hipError_t launch_stream_v(const dev::GemmArgs& a, hipStream_t st) {
  constexpr int W = stream_waves(BITS, NSETS);
  auto one = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)a.ntiles), dim3(W * 64), dev::StreamSmem<W>::bytes(16 * V, NSETS), st,
                       a);
    return hipGetLastError();
  };
  if (a.T == 1) return one(dev::gemm_stream_kernel<BITS, SBF16, V, W, 1, NSETS>);
  if (a.T == 2) return one(dev::gemm_stream_kernel<BITS, SBF16, V, W, 2, NSETS>);
  if (a.T <= 4) return one(dev::gemm_stream_kernel<BITS, SBF16, V, W, 4, NSETS>);
  return one(dev::gemm_stream_kernel<BITS, SBF16, V, W, 8, NSETS>);
}
static_assert(dev::StreamSmem<kStreamW>::bytes(32) <= 64u * 1024u && dev::StreamSmem<kStreamW8>::bytes(32) <= 64u * 1024u &&
                  dev::StreamSmem<kStreamW2>::bytes(32, 2) <= 64u * 1024u,
              "the streaming kernel's LDS stays under the default 64 KiB limit");

template <int BITS, bool SBF16, int NSETS>
hipError_t launch_stream_b(int v, const dev::GemmArgs& a, hipStream_t st) {
  return v >= 2 ? launch_stream_v<BITS, SBF16, 2, NSETS>(a, st) : launch_stream_v<BITS, SBF16, 1, NSETS>(a, st);
}

template <int NSETS>
hipError_t launch_stream(const Format& f, int v, const dev::GemmArgs& a, hipStream_t st) {
  if (f.bits == 4)
    return f.scale_bf16 ? launch_stream_b<4, true, NSETS>(v, a, st) : launch_stream_b<4, false, NSETS>(v, a, st);
  if (f.bits == 5)
    return f.scale_bf16 ? launch_stream_b<5, true, NSETS>(v, a, st) : launch_stream_b<5, false, NSETS>(v, a, st);
  return f.scale_bf16 ? launch_stream_b<8, true, NSETS>(v, a, st) : launch_stream_b<8, false, NSETS>(v, a, st);
}

// The VALU-inner-step kernel: the streaming kernel's pipeline and tiles (32
// columns; 10 waves, 7 for int8 and for SwiGLU).
template <int BITS, bool SBF16, int NSETS>
hipError_t launch_dot_b(const dev::GemmArgs& a, hipStream_t st) {
  constexpr int W = dot_waves(BITS, NSETS);
  auto one = [&](auto kern, uint32_t lds) {
    hipLaunchKernelGGL(kern, dim3((unsigned)a.ntiles), dim3(W * 64), lds, st, a);
    return hipGetLastError();
  };
  if (a.T == 1) return one(dev::gemm_dot_kernel<BITS, SBF16, W, 1, NSETS>, dev::DotSmem<W, 1, NSETS>::bytes());
  if (a.T == 2) return one(dev::gemm_dot_kernel<BITS, SBF16, W, 2, NSETS>, dev::DotSmem<W, 2, NSETS>::bytes());
  if (a.T <= 4) return one(dev::gemm_dot_kernel<BITS, SBF16, W, 4, NSETS>, dev::DotSmem<W, 4, NSETS>::bytes());
  return one(dev::gemm_dot_kernel<BITS, SBF16, W, 8, NSETS>, dev::DotSmem<W, 8, NSETS>::bytes());
}
static_assert(dev::DotSmem<kStreamW, 8, 1>::bytes() <= 64u * 1024u && dev::DotSmem<kDotW8, 8, 1>::bytes() <= 64u * 1024u &&
                  dev::DotSmem<kDotW2, 8, 2>::bytes() <= 64u * 1024u,
              "the VALU kernel's LDS stays under 64 KiB");

template <int NSETS>
hipError_t launch_dot(const Format& f, const dev::GemmArgs& a, hipStream_t st) {
  if (f.bits == 4) return f.scale_bf16 ? launch_dot_b<4, true, NSETS>(a, st) : launch_dot_b<4, false, NSETS>(a, st);
  if (f.bits == 5) return f.scale_bf16 ? launch_dot_b<5, true, NSETS>(a, st) : launch_dot_b<5, false, NSETS>(a, st);
  return f.scale_bf16 ? launch_dot_b<8, true, NSETS>(a, st) : launch_dot_b<8, false, NSETS>(a, st);
}

// Shared validation and launch of ngq_gemm (nsets 1) and ngq_swiglu_gemm (2).
// ---- many tokens (host) ----

template <int BITS, bool SBF16, int NSETS>
hipError_t launch_wide_b(int v, int tb, const dev::WideArgs& a, uint32_t lds, hipStream_t st) {
  auto one = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)a.ntiles), dim3(dev::kWideWaves * 64), lds, st, a);
    return hipGetLastError();
  };
  if constexpr (NSETS == 1) {
    if (v == 3) return tb == 1 ? one(dev::gemm_wide_kernel<BITS, SBF16, 3, 1, 1>)
                               : one(dev::gemm_wide_kernel<BITS, SBF16, 3, 1, 2>);
  }
  if (tb == 1) return one(dev::gemm_wide_kernel<BITS, SBF16, 2, NSETS, 1>);
  if (tb == 2) return one(dev::gemm_wide_kernel<BITS, SBF16, 2, NSETS, 2>);
  return one(dev::gemm_wide_kernel<BITS, SBF16, 2, NSETS, 4>);
}

template <int NSETS>
hipError_t launch_wide(const Format& f, int v, int tb, const dev::WideArgs& a, uint32_t lds, hipStream_t st) {
  if (f.bits == 4)
    return f.scale_bf16 ? launch_wide_b<4, true, NSETS>(v, tb, a, lds, st)
                        : launch_wide_b<4, false, NSETS>(v, tb, a, lds, st);
  if (f.bits == 5)
    return f.scale_bf16 ? launch_wide_b<5, true, NSETS>(v, tb, a, lds, st)
                        : launch_wide_b<5, false, NSETS>(v, tb, a, lds, st);
  return f.scale_bf16 ? launch_wide_b<8, true, NSETS>(v, tb, a, lds, st)
                      : launch_wide_b<8, false, NSETS>(v, tb, a, lds, st);
}

// 8 < T <= 64 (by default up to 32), arguments already checked: one workgroup per tile of 32
// columns, or 48 where that gives one tile per CU (plain projections at
// T <= 32, whose registers allow it); 16 (T <= 16), 32 or 64 token rows per
// workgroup.
int run_wide(int nsets, int T, int K, int Nout, int Ncols, const Format& f, const void* x, const void* wq,
             const void* scales, void* y, size_t wb0, size_t wb1, size_t sb, size_t xb, void* stream) {
  dev::WideArgs a;
  a.x = x; a.wq = wq; a.scales = scales; a.y = y;
  a.T = T; a.K = K; a.Nout = Nout; a.Ncols = Ncols; a.up_off = nsets == 2 ? Nout : 0;
  a.G = K / kGroup;
  a.pairs = (a.G + 1) / 2;
  const int tb = T <= 16 ? 1 : T <= 32 ? 2 : 4;
  const int v = nsets == 1 && tb <= 2 && Nout >= 32 ? choose_v(Nout, cu_count(), 2, 3) : 2;
  a.ntiles = (Nout + 16 * v - 1) / (16 * v);
  a.p0_bytes = (uint32_t)wb0; a.p1_bytes = (uint32_t)wb1; a.s_bytes = (uint32_t)sb; a.x_bytes = (uint32_t)xb;
  a.mask_nib = dev::kMasks.nib; a.mask_base = dev::kMasks.base; a.mask_hi = dev::kMasks.hi;
  const uint32_t lds = dev::kWideWaves * dev::wide_block_floats(nsets, v) * 4u;
  const hipError_t e = nsets == 1 ? launch_wide<1>(f, v, tb, a, lds, (hipStream_t)stream)
                                  : launch_wide<2>(f, v, tb, a, lds, (hipStream_t)stream);
  return e == hipSuccess ? NGQ_OK : NGQ_ERR_HIP;
}

template <int BITS, bool SBF16, int NSETS>
hipError_t launch_tiled_b(int v, const dev::TiledArgs& a, uint32_t lds, hipStream_t st) {
  // lds <= 64 KB (tiled_lds_bytes of at most 64 accumulators per lane)
  auto one = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)a.tiles), dim3(dev::kTiledWaves * 64), lds, st, a);
    return hipGetLastError();
  };
  if constexpr (NSETS == 1) {
    if (v == 2) return one(dev::gemm_tiled_kernel<BITS, SBF16, 1, kTiledNB, 2>);
    if (v == 1) return one(dev::gemm_tiled_kernel<BITS, SBF16, 1, kTiledNB, 1>);
  }
  return one(dev::gemm_tiled_kernel<BITS, SBF16, NSETS, kTiledNB, 4 / NSETS>);
}

// 96- and 128-token tiles for int4 only: the int5 and int8 variants need
// more than 256 VGPRs there (one wave per SIMD).
template <int BITS, bool SBF16, int NSETS>
hipError_t launch_tiled_sx_b(int tb, const dev::TiledArgs& a, uint32_t lds, hipStream_t st) {
  auto one = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)a.tiles), dim3(dev::kTiledWaves * 64), lds, st, a);
    return hipGetLastError();
  };
  if constexpr (BITS == 4) {
    if (tb == 8) return one(dev::gemm_tiled_sx_kernel<BITS, SBF16, NSETS, kSxNB, 8>);
    if (tb == 6) return one(dev::gemm_tiled_sx_kernel<BITS, SBF16, NSETS, kSxNB, 6>);
  }
  return one(dev::gemm_tiled_sx_kernel<BITS, SBF16, NSETS, kSxNB, 4>);
}

// Token tile of the shared-X kernel (token blocks of 16): the one whose tile
// count best fills rounds of two workgroups per CU, the larger on a tie
// (measured: QK T = 2048 runs 128-token tiles 8 % faster, down T = 2048
// 96-token tiles 13 % faster, QK T = 1024 and int8 64-token tiles).
int sx_token_blocks(int bits, long sx_cols, int T, int cus) {
  if (bits != 4) return 4;
  int best = 4;
  double best_eff = -1.0;
  for (int tb : {8, 6, 4}) {
    const long tiles = sx_cols * ((T + 16L * tb - 1) / (16L * tb));
    const long slots = 2L * cus;
    const double eff = (double)tiles / (double)(((tiles + slots - 1) / slots) * slots);
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = tb;
    }
  }
  return best;
}

// sel: token blocks per tile (shared-X kernel) or columns per lane and set,
// V (K-split kernel)
template <int NSETS, bool SX>
hipError_t launch_tiled(const Format& f, int sel, const dev::TiledArgs& a, uint32_t lds, hipStream_t st) {
  if constexpr (SX) {
    if (f.bits == 4)
      return f.scale_bf16 ? launch_tiled_sx_b<4, true, NSETS>(sel, a, lds, st)
                          : launch_tiled_sx_b<4, false, NSETS>(sel, a, lds, st);
    if (f.bits == 5)
      return f.scale_bf16 ? launch_tiled_sx_b<5, true, NSETS>(sel, a, lds, st)
                          : launch_tiled_sx_b<5, false, NSETS>(sel, a, lds, st);
    return f.scale_bf16 ? launch_tiled_sx_b<8, true, NSETS>(sel, a, lds, st)
                        : launch_tiled_sx_b<8, false, NSETS>(sel, a, lds, st);
  } else {
    if (f.bits == 4)
      return f.scale_bf16 ? launch_tiled_b<4, true, NSETS>(sel, a, lds, st)
                          : launch_tiled_b<4, false, NSETS>(sel, a, lds, st);
    if (f.bits == 5)
      return f.scale_bf16 ? launch_tiled_b<5, true, NSETS>(sel, a, lds, st)
                          : launch_tiled_b<5, false, NSETS>(sel, a, lds, st);
    return f.scale_bf16 ? launch_tiled_b<8, true, NSETS>(sel, a, lds, st)
                        : launch_tiled_b<8, false, NSETS>(sel, a, lds, st);
  }
}

// Token x column tiles (prefill-size T; any T >= 1 when forced), arguments
// already checked: 64 tokens by 64 weight columns per workgroup (32 or 16
// for a plain projection whose 64-column tiles would leave CUs idle) with K
// split over its waves, or (sx) 64, 96 or 128 tokens by 256 weight columns sharing
// each X tile, which needs 4x as many tokens to fill the CUs.  `path` is
// NGQ_KERNEL_TILED or NGQ_KERNEL_TILED_SX (64 tokens), _SX96 or _SX128 (int4)
// to force one, anything else to choose.
int run_tiled(int path, int nsets, int T, int K, int Nout, int Ncols, const Format& f, const void* x,
              const void* wq, const void* scales, void* y, size_t wb0, size_t wb1, size_t sb, size_t xb,
              void* stream) {
  dev::TiledArgs a;
  a.x = x; a.wq = wq; a.scales = scales; a.y = y;
  a.T = T; a.K = K; a.Nout = Nout; a.Ncols = Ncols; a.up_off = nsets == 2 ? Nout : 0;
  a.G = K / kGroup;
  const long sx_cols = (Nout + dev::kSxCols / nsets - 1) / (dev::kSxCols / nsets);
  const long sx_tiles = sx_cols * ((T + dev::kTiledTok - 1) / dev::kTiledTok);
  if ((path == NGQ_KERNEL_TILED_SX96 || path == NGQ_KERNEL_TILED_SX128) && f.bits != 4) return NGQ_ERR_UNSUPPORTED;
  const bool sx = path == NGQ_KERNEL_TILED_SX || path == NGQ_KERNEL_TILED_SX96 || path == NGQ_KERNEL_TILED_SX128 ||
                  (path != NGQ_KERNEL_TILED && 10 * sx_tiles >= (long)kSxMinTiles10PerCu * cu_count());
  const int tb = !sx                                 ? 4
                 : path == NGQ_KERNEL_TILED_SX       ? 4
                 : path == NGQ_KERNEL_TILED_SX96     ? 6
                 : path == NGQ_KERNEL_TILED_SX128    ? 8
                                                     : sx_token_blocks(f.bits, sx_cols, T, cu_count());
  const long ttiles = (T + 16L * tb - 1) / (16L * tb);
  // K-split tiles of 16 v output columns per set: a plain projection halves
  // v while its tiles leave CUs without a workgroup and the halved tiles
  // still fit one round (a CU running two narrow tiles finishes last: QK at
  // 64 tokens on 32-column tiles, 256 of them, takes 23.2 us against 24.8
  // on 64; GV on 32, 384 tiles, 47 against 27)
  const long cus = cu_count();
  auto ktiles = [&](int vv) { return (long)((Nout + 16 * vv - 1) / (16 * vv)) * ttiles; };
  int v = 4 / nsets;
  while (!sx && nsets == 1 && v > kTiledMinV && ktiles(v) < cus && ktiles(v / 2) <= cus) v /= 2;
  const int ocols = sx ? dev::kSxCols / nsets : 16 * v;
  a.tiles_n = (Nout + ocols - 1) / ocols;
  const long tiles = (long)a.tiles_n * ttiles;
  if (tiles > 0x7FFFFFFFL) return NGQ_ERR_SHAPE;
  a.tiles = (int)tiles;
  a.p0_bytes = (uint32_t)wb0; a.p1_bytes = (uint32_t)wb1; a.s_bytes = (uint32_t)sb; a.x_bytes = (uint32_t)xb;
  a.mask_nib = dev::kMasks.nib; a.mask_base = dev::kMasks.base; a.mask_hi = dev::kMasks.hi;
  hipError_t e;
  if (sx) {
    const uint32_t lds = dev::tiled_sx_lds_bytes(tb);
    e = nsets == 1 ? launch_tiled<1, true>(f, tb, a, lds, (hipStream_t)stream)
                   : launch_tiled<2, true>(f, tb, a, lds, (hipStream_t)stream);
  } else {
    const uint32_t lds = dev::tiled_lds_bytes(16 * nsets * v);
    e = nsets == 1 ? launch_tiled<1, false>(f, v, a, lds, (hipStream_t)stream)
                   : launch_tiled<2, false>(f, v, a, lds, (hipStream_t)stream);
  }
  return e == hipSuccess ? NGQ_OK : NGQ_ERR_HIP;
}

int run_gemm(int nsets, int T, int K, int Nout, int bits, int group, const void* x, const void* wq,
             const void* scales, void* y, void* stream) {
  Format f;
  int rc = parse_format(bits, group, &f);
  if (rc != NGQ_OK) return rc;
  if (T < 0 || T > NGQ_MAX_T_PREFILL) return NGQ_ERR_SHAPE;
  if ((rc = check_kn(K, Nout)) != NGQ_OK) return rc;
  const long ncols_l = (long)Nout * nsets;
  if (ncols_l > (1L << 30)) return NGQ_ERR_SHAPE;
  const int Ncols = (int)ncols_l;
  if (T == 0 || Nout == 0) return NGQ_OK;
  const size_t xb = (size_t)T * K * 2, yb = (size_t)T * Nout * 2;
  const size_t wb0 = p0_bytes(K, Ncols, f.bits), wb1 = p1_bytes(K, Ncols, f.bits);
  const size_t sb = (size_t)(K / kGroup) * Ncols * 2;
  if ((rc = check_ptr(y)) != NGQ_OK) return rc;
  if (K > 0) {
    if ((rc = check_ptr(x)) != NGQ_OK) return rc;
    if ((rc = check_ptr(wq)) != NGQ_OK) return rc;
    if ((rc = check_ptr(scales)) != NGQ_OK) return rc;
  }
  if (xb >= kMaxBuffer || yb >= kMaxBuffer || wb0 + wb1 >= kMaxBuffer || sb >= kMaxBuffer)
    return NGQ_ERR_UNSUPPORTED;
  if (overlaps(y, yb, x, xb) || overlaps(y, yb, wq, wb0 + wb1) || overlaps(y, yb, scales, sb)) return NGQ_ERR_ARG;
  const int forced = kernel_override.load(std::memory_order_relaxed);
  if (forced == NGQ_KERNEL_TILED || forced == NGQ_KERNEL_TILED_SX || forced == NGQ_KERNEL_TILED_SX96 ||
      forced == NGQ_KERNEL_TILED_SX128)
    return run_tiled(forced, nsets, T, K, Nout, Ncols, f, x, wq, scales, y, wb0, wb1, sb, xb, stream);
  if (forced == NGQ_KERNEL_WIDE && (T <= NGQ_MAX_T || T > NGQ_MAX_T_VERIFY)) return NGQ_ERR_UNSUPPORTED;
  if (T > NGQ_MAX_T) {
    if (forced != NGQ_KERNEL_WIDE && T >= kTiledFromT)
      return run_tiled(NGQ_KERNEL_AUTO, nsets, T, K, Nout, Ncols, f, x, wq, scales, y, wb0, wb1, sb, xb, stream);
    return run_wide(nsets, T, K, Nout, Ncols, f, x, wq, scales, y, wb0, wb1, sb, xb, stream);
  }

  const int cus = cu_count();
  // Tiles of at least 32 columns where N allows: a 16-column tile reads 64 of
  // every 128 weight bytes of a row per cache line, and streams at about half
  // the rate (measured).
  const int vmin = Nout >= 32 ? 2 : 1;
  const long xchunks = (long)T * K / 8;
  const int pairs = (K / kGroup + 1) / 2;
  const int v_pp = choose_v(Nout, cus, vmin, nsets == 1 ? 4 : 2);  // per-pair-X kernel
  const long tiles_pp = (Nout + 16L * v_pp - 1) / (16L * v_pp);
  const bool pp_dyn_fits = dev::Smem::bytes(true, pairs, nsets, 16 * v_pp) <= kMaxLds;
  // An X-resident configuration for this shape: its tile width and LDS, or
  // false when X does not fit or the prologue does not cover it.
  auto xres_fits = [&](const XCfg& c, int& vx, uint32_t& lx) -> bool {
    if (K == 0 || (nsets == 2 && c.W == kX14.W) || xchunks > (long)c.XL * c.W * 64) return false;
    vx = c.W == kX14.W ? std::min(v_pp, xres_vmax(f.bits, nsets, c.XL))
                       : choose_v(Nout, cus, vmin, xres_vmax(f.bits, nsets, c.XL));
    lx = dev::XSmem::bytes(T, K, c.W, nsets, 16 * vx);
    return lx <= kMaxLds;
  };
  const XCfg x8 = xchunks <= (long)kX8a.XL * kX8a.W * 64 ? kX8a : kX8b;
  // Kernel choice (measured on MI355X):
  //  - one round of 32-column tiles and one output set: at T = 1 the VALU
  //    inner step for int4 and int8 (QK shape: 6.39 against 6.52 us with the
  //    MFMA step, int8 10.71 against 10.92; from T = 2 the MFMA step wins,
  //    by 12-22 % at T = 2 and 2-2.7x at T = 8), otherwise the streaming
  //    kernel (QK, T = 2..8: 6.5-7.4 us against 7.4-7.9 for the 14-wave
  //    X-resident kernel; int8 with 5 waves, 2-4 % ahead of the X-resident
  //    kernel); other one-round shapes: per-pair X with dynamic pair
  //    assignment (gate/value: 48-column tiles, where the streaming kernel's
  //    int5 unpack did not keep up);
  //  - SwiGLU at T = 1, int4: the VALU step with 7 waves, one workgroup
  //    per 32-column tile (gate/up, 544 tiles: 21.0 us against 23.1 for the
  //    streaming kernel; three of its workgroups fit on a CU, so all 544 are
  //    resident at once: with 9 or 10 waves only two fit, and 25.7 / 23.9);
  //  - SwiGLU at T <= 4 otherwise: the streaming kernel with 5 waves and one
  //    workgroup per 32-column tile (gate/up, 544 tiles: 23.5 us against 27.0
  //    for the persistent X-resident kernel, whose 2.125 rounds of tiles end
  //    in a round on 32 CUs; 3, 4, 6, 8 waves: 24.7-27.3; at T = 8 the X
  //    bands make it 3 % slower than the X-resident kernel);
  //  - otherwise the X-resident kernel with 8 waves when X fits in LDS;
  //  - otherwise per-pair X (dynamic, or static ranges for very long K).
  int path = forced;
  XCfg xc = x8;
  int v = v_pp, vx = 0;
  uint32_t lx = 0;
  if (path == NGQ_KERNEL_AUTO) {
    const bool one_round_tiles = nsets == 1 && tiles_pp <= cus;
    const bool one_round = one_round_tiles && pp_dyn_fits;
    // the streaming kernels need no per-pair LDS blocks: long K (the down
    // projection, 160 tiles) takes them too up to T = 4 (measured there:
    // T = 1 VALU step 14.2 us against 15.3 X-resident, T = 2 and 4 MFMA step
    // 2 % ahead; at T = 8 the per-pair kernel stays 2 % ahead)
    const bool streams = one_round_tiles && v_pp == 2 && K > 0 && (pp_dyn_fits || T <= 4);
    if (streams && T == 1 && f.bits != 5)
      path = NGQ_KERNEL_DOT;
    else if (streams && (f.bits != 8 || kInt8Stream))
      path = NGQ_KERNEL_STREAM;
    else if (nsets == 2 && T == 1 && f.bits == 4 && K > 0)
      path = NGQ_KERNEL_DOT;
    else if (nsets == 2 && T <= kStreamSwigluMaxT && f.bits != 8 && K > 0)
      path = NGQ_KERNEL_STREAM;
    else if (one_round && v_pp == 2 && xres_fits(kX14, vx, lx))
      path = NGQ_KERNEL_XRES14;
    else if (!one_round && xres_fits(x8, vx, lx))
      path = NGQ_KERNEL_XRES8;
    else
      path = pp_dyn_fits ? NGQ_KERNEL_PERPAIR_DYN : NGQ_KERNEL_PERPAIR_STATIC;
  } else if (path == NGQ_KERNEL_XRES14 || path == NGQ_KERNEL_XRES8) {
    if (!xres_fits(path == NGQ_KERNEL_XRES14 ? kX14 : x8, vx, lx)) return NGQ_ERR_UNSUPPORTED;
  } else if (path == NGQ_KERNEL_PERPAIR_DYN && !pp_dyn_fits) {
    return NGQ_ERR_UNSUPPORTED;
  }
  const bool xres = path == NGQ_KERNEL_XRES14 || path == NGQ_KERNEL_XRES8;
  if (xres) {
    xc = path == NGQ_KERNEL_XRES14 ? kX14 : x8;
    v = vx;
  }
  dev::GemmArgs a;
  a.x = x; a.wq = wq; a.scales = scales; a.y = y;
  a.T = T; a.K = K; a.Nout = Nout; a.Ncols = Ncols; a.up_off = nsets == 2 ? Nout : 0;
  a.G = K / kGroup;
  a.pairs = pairs;
  a.ppw = (a.pairs + dev::kWaves - 1) / dev::kWaves;
  a.tiles_q = a.tiles_r = 0;  // set for the X-resident launch below
  a.ntiles = (Nout + 16 * v - 1) / (16 * v);
  a.p0_bytes = (uint32_t)wb0; a.p1_bytes = (uint32_t)wb1; a.s_bytes = (uint32_t)sb; a.x_bytes = (uint32_t)xb;
  a.mask_nib = dev::kMasks.nib; a.mask_base = dev::kMasks.base; a.mask_hi = dev::kMasks.hi;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (path == NGQ_KERNEL_DOT) {
    a.ntiles = (Nout + 31) / 32;
    a.ppw = (a.pairs + dot_waves(f.bits, nsets) - 1) / dot_waves(f.bits, nsets);
    e = nsets == 1 ? launch_dot<1>(f, a, st) : launch_dot<2>(f, a, st);
    return e == hipSuccess ? NGQ_OK : NGQ_ERR_HIP;
  }
  if (path == NGQ_KERNEL_STREAM) {
    const int vs = Nout >= 32 ? 2 : 1;
    a.ntiles = (Nout + 16 * vs - 1) / (16 * vs);
    const int ws = stream_waves(f.bits, nsets);
    a.ppw = (a.pairs + ws - 1) / ws;
    e = nsets == 1 ? launch_stream<1>(f, vs, a, st) : launch_stream<2>(f, vs, a, st);
    return e == hipSuccess ? NGQ_OK : NGQ_ERR_HIP;
  }
  if (xres) {
    const int per = (a.pairs + xc.W - 1) / xc.W;
    a.ppw = (per + xc.NB - 1) / xc.NB * xc.NB;
    const int grid = std::min(a.ntiles, cus);
    a.tiles_q = a.ntiles / grid;
    a.tiles_r = a.ntiles % grid;
    e = nsets == 1 ? launch_xres<1>(f, xc, v, a, grid, lx, st) : launch_xres<2>(f, xc, v, a, grid, lx, st);
    return e == hipSuccess ? NGQ_OK : NGQ_ERR_HIP;
  }
  // Dynamic pair assignment needs one partial-sum block per pair in LDS; very
  // long K uses static ranges (one block per wave).
  const bool dyn = path == NGQ_KERNEL_PERPAIR_DYN;
  const uint32_t lds = dev::Smem::bytes(dyn, a.pairs, nsets, 16 * v);
  if (nsets == 1)
    e = dyn ? launch_fmt<1, true>(f, v, a, lds, st) : launch_fmt<1, false>(f, v, a, lds, st);
  else
    e = dyn ? launch_fmt<2, true>(f, v, a, lds, st) : launch_fmt<2, false>(f, v, a, lds, st);
  return e == hipSuccess ? NGQ_OK : NGQ_ERR_HIP;
}

template <bool DEQUANT>
int run_unpack(int K, int N, int bits, int group, const void* wq, const void* scales, void* out, void* stream) {
  Format f;
  int rc = parse_format(bits, group, &f);
  if (rc != NGQ_OK) return rc;
  if ((rc = check_kn(K, N)) != NGQ_OK) return rc;
  if (K == 0 || N == 0) return NGQ_OK;
  if ((rc = check_ptr(wq)) != NGQ_OK) return rc;
  if ((rc = check_ptr(out)) != NGQ_OK) return rc;
  if (DEQUANT && (rc = check_ptr(scales)) != NGQ_OK) return rc;
  const size_t wb = p0_bytes(K, N, f.bits) + p1_bytes(K, N, f.bits);
  const size_t ob = (size_t)K * N * (DEQUANT ? 4 : 1);
  if (wb >= kMaxBuffer) return NGQ_ERR_UNSUPPORTED;
  if (overlaps(out, ob, wq, wb)) return NGQ_ERR_ARG;
  const dim3 grid((unsigned)((N + 255) / 256), (unsigned)(K / 8)), block(256);
  const uint32_t p0b = (uint32_t)p0_bytes(K, N, f.bits);
  hipStream_t st = (hipStream_t)stream;
#define NGQ_UNPACK(B, S) hipLaunchKernelGGL((dev::unpack_kernel<B, S, DEQUANT>), grid, block, 0, st, wq, p0b, scales, K, N, out)
  if (f.bits == 4) { if (f.scale_bf16) NGQ_UNPACK(4, true); else NGQ_UNPACK(4, false); }
  else if (f.bits == 5) { if (f.scale_bf16) NGQ_UNPACK(5, true); else NGQ_UNPACK(5, false); }
  else { if (f.scale_bf16) NGQ_UNPACK(8, true); else NGQ_UNPACK(8, false); }
#undef NGQ_UNPACK
  return hipGetLastError() == hipSuccess ? NGQ_OK : NGQ_ERR_HIP;
}


// ---- several projections of one X in one launch (host) ----

// Shapes whose plans are kept; the oldest is dropped beyond that.
constexpr size_t kPlanCacheSize = 16;

// Tiles per projection and workgroup for one shape (see gemm_multi_kernel).
struct MultiPlan {
  int key[3 + 2 * dev::kMultiMaxProj];  // grid bound, K, nproj, then (kind, Nout) per projection
  int grid;
  uint16_t first[dev::kMultiMaxWg][dev::kMultiMaxProj];
  uint8_t count[dev::kMultiMaxWg][dev::kMultiMaxProj];
};

// Longest tiles first, each to the least loaded workgroup (lowest rank on a
// tie).  The cost of a tile is its weight and scale bytes.  Ranks own
// contiguous tile ranges and are placed on blocks XCD-grouped (block b runs
// on XCD b % 8; ranks r, r + 1, ... of one XCD are its blocks in order).
// Returns false when a projection has more tiles than the table holds.
bool make_plan(int K, int nproj, const int* kind, const int* nout, int wg_max, MultiPlan& pl) {
  struct P {
    double cost;
    int p, tiles;
  } ps[dev::kMultiMaxProj];
  long total = 0;
  for (int p = 0; p < nproj; ++p) {
    const int kd = kind[p], bits = kd / 4 == 0 ? 4 : (kd / 4 == 1 ? 5 : 8), nsets = kd % 2 + 1;
    const int cols = 16 * dev::multi_v(bits, nsets);
    ps[p].p = p;
    ps[p].tiles = (nout[p] + cols - 1) / cols;
    ps[p].cost = (double)cols * nsets * K * ((double)bits / 8.0 + 2.0 / kGroup);
    if (ps[p].tiles > 65535) return false;  // the first-tile table holds 16 bits
    total += ps[p].tiles;
  }
  pl.grid = (int)std::min<long>(total, wg_max);
  std::memset(pl.first, 0, sizeof(pl.first));
  std::memset(pl.count, 0, sizeof(pl.count));
  if (pl.grid == 0) return true;
  int cnt[dev::kMultiMaxProj][dev::kMultiMaxWg] = {};
  std::stable_sort(ps, ps + nproj, [](const P& a, const P& b) { return a.cost > b.cost; });
  // (load, tie order, rank); on equal loads the tie order takes one rank of
  // each XCD in turn, so the more loaded ranks spread over the XCDs
  const int G = pl.grid, per_xcd = (G + 7) / 8;
  using Slot = std::tuple<double, int, int>;
  std::priority_queue<Slot, std::vector<Slot>, std::greater<Slot>> heap;
  for (int r = 0; r < G; ++r) heap.push({0.0, (r % per_xcd) * 8 + r / per_xcd, r});
  for (int i = 0; i < nproj; ++i) {
    for (int k = 0; k < ps[i].tiles; ++k) {
      Slot s = heap.top();
      heap.pop();
      ++cnt[ps[i].p][std::get<2>(s)];
      std::get<0>(s) += ps[i].cost;
      heap.push(s);
    }
  }
  int start[dev::kMultiMaxProj][dev::kMultiMaxWg];  // first tile of each rank
  for (int p = 0; p < nproj; ++p) {
    int acc = 0;
    for (int r = 0; r < G; ++r) {
      if (cnt[p][r] > 255) return false;  // the count table holds 8 bits
      start[p][r] = acc;
      acc += cnt[p][r];
    }
  }
  for (int b = 0; b < G; ++b) {
    const int xcd = b & 7, r = xcd * (G >> 3) + std::min(xcd, G & 7) + (b >> 3);
    for (int p = 0; p < nproj; ++p) {
      pl.first[b][p] = (uint16_t)start[p][r];
      pl.count[b][p] = (uint8_t)cnt[p][r];
    }
  }
  return true;
}

// The plan of a shape, computed once and kept (a few shapes per process),
// copied into the launch arguments while the cache's lock is held: a plan
// may be evicted (and freed) by another thread as soon as the lock is
// released, so no pointer into the cache leaves this function.  Returns the
// grid, or -1 when the shape has no plan.
int load_plan(int K, int nproj, const int* kind, const int* nout, int wg_max, dev::MultiArgs& a) {
  static std::mutex mu;
  static std::deque<MultiPlan> plans;
  int key[3 + 2 * dev::kMultiMaxProj] = {wg_max, K, nproj};
  for (int p = 0; p < nproj; ++p) {
    key[3 + 2 * p] = kind[p];
    key[4 + 2 * p] = nout[p];
  }
  std::lock_guard<std::mutex> lock(mu);
  const MultiPlan* found = nullptr;
  for (const MultiPlan& pl : plans)
    if (std::memcmp(pl.key, key, sizeof(key)) == 0) found = &pl;
  if (found == nullptr) {
    MultiPlan pl;
    std::memcpy(pl.key, key, sizeof(key));
    if (!make_plan(K, nproj, kind, nout, wg_max, pl)) return -1;
    if (plans.size() == kPlanCacheSize) plans.pop_front();
    plans.push_back(pl);
    found = &plans.back();
  }
  static_assert(sizeof(a.first) == sizeof(found->first) && sizeof(a.count) == sizeof(found->count),
                "plan tables and launch arguments differ");
  std::memcpy(a.first, found->first, sizeof(a.first));
  std::memcpy(a.count, found->count, sizeof(a.count));
  return found->grid;
}

// ngq_multi_gemm as one workgroup per tile (gemm_multi_dot_kernel at T = 1,
// gemm_multi_stream_kernel above): the validated projections (descriptors in
// a.proj, kinds in kind) as segments of one grid, the heaviest tiles (weight
// and scale bytes per tile) first.  Measured against the persistent kernel
// (QK + gate/value + gate/up): T = 1 32.7 against 37.8 us, T = 2 32.7
// against 37.2-38.2, T = 4 33.5 against 37.4-37.9, T = 8 34.9-35.1 (37.2-37.4
// with 32-column tiles) against 37.9-39.0; with 2, 3, 5, 6 or 8 waves a tile
// at T >= 2: 2-11 % slower than 4.
constexpr int kMultiStreamMaxT = 8;

int run_multi_tiles(int T, int K, const void* x, size_t xb, const dev::MultiArgs& a, const int* kind, int n,
                  void* stream) {
  int order[NGQ_MAX_PROJ];
  long tile_bytes[NGQ_MAX_PROJ];
  for (int i = 0; i < n; ++i) {
    const dev::MultiProj& mp = a.proj[i];
    const int tc = dev::multi_tile_cols(T);
    tile_bytes[i] = ((long)mp.p0_bytes + mp.p1_bytes + mp.s_bytes) / ((mp.Nout + tc - 1) / tc);
    order[i] = i;
  }
  std::stable_sort(order, order + n, [&](int i, int j) { return tile_bytes[i] > tile_bytes[j]; });
  dev::MultiTileArgs m;
  std::memset(&m, 0, sizeof(m));
  const int G = K / kGroup, pairs = (G + 1) / 2;
  long grid = 0;
  for (int i = 0; i < dev::kMultiMaxProj; ++i) m.end[i] = INT32_MAX;
  for (int i = 0; i < n; ++i) {
    const dev::MultiProj& mp = a.proj[order[i]];
    dev::GemmArgs& g = m.proj[i];
    g.x = x; g.wq = mp.wq; g.scales = mp.scales; g.y = mp.y;
    const int w = T == 1 ? dev::kMultiDotW : dev::kMultiStreamW;
    g.T = T; g.K = K; g.Nout = mp.Nout; g.Ncols = mp.Ncols; g.up_off = mp.up_off;
    g.G = G; g.pairs = pairs;
    g.ppw = (pairs + w - 1) / w;
    const int tc = dev::multi_tile_cols(T);
    g.ntiles = (mp.Nout + tc - 1) / tc;
    g.p0_bytes = mp.p0_bytes; g.p1_bytes = mp.p1_bytes; g.s_bytes = mp.s_bytes; g.x_bytes = (uint32_t)xb;
    g.mask_nib = dev::kMasks.nib; g.mask_base = dev::kMasks.base; g.mask_hi = dev::kMasks.hi;
    g.tiles_q = g.tiles_r = 0;
    grid += g.ntiles;
    m.end[i] = (int)grid;
    m.kind[i] = kind[order[i]];
  }
  if (grid > INT32_MAX / 2) return NGQ_ERR_UNSUPPORTED;
  hipStream_t st = (hipStream_t)stream;
  if (T == 1) {
    const uint32_t lds = dev::DotSmem<dev::kMultiDotW, 1, 2>::bytes();
    hipLaunchKernelGGL(dev::gemm_multi_dot_kernel, dim3((unsigned)grid), dim3(dev::kMultiDotW * 64), lds, st, m);
  } else {
    const uint32_t lds = dev::StreamSmem<dev::kMultiStreamW>::bytes(64, 2);
    const dim3 g((unsigned)grid), blk(dev::kMultiStreamW * 64);
    if (T == 2)
      hipLaunchKernelGGL(dev::gemm_multi_stream_kernel<2>, g, blk, lds, st, m);
    else if (T <= 4)
      hipLaunchKernelGGL(dev::gemm_multi_stream_kernel<4>, g, blk, lds, st, m);
    else
      hipLaunchKernelGGL(dev::gemm_multi_stream_kernel<8>, g, blk, lds, st, m);
  }
  return hipGetLastError() == hipSuccess ? NGQ_OK : NGQ_ERR_HIP;
}

int run_multi(int T, int K, int group, const void* x, const ngq_proj* projs, int nproj, void* stream) {
  if (projs == nullptr || nproj < 1 || nproj > NGQ_MAX_PROJ) return NGQ_ERR_ARG;
  if (T < 0 || T > NGQ_MAX_T) return NGQ_ERR_SHAPE;
  Format f[NGQ_MAX_PROJ];
  int rc;
  for (int p = 0; p < nproj; ++p) {
    if ((rc = parse_format(projs[p].bits, group, &f[p])) != NGQ_OK) return rc;
    if ((projs[p].swiglu != 0 && projs[p].swiglu != 1) || projs[p].reserved != 0) return NGQ_ERR_ARG;
    if ((rc = check_kn(K, projs[p].n)) != NGQ_OK) return rc;
    if ((long)projs[p].n * (projs[p].swiglu + 1) > (1L << 30)) return NGQ_ERR_SHAPE;
  }
  if (T == 0) return NGQ_OK;
  const size_t xb = (size_t)T * K * 2;
  if (xb >= kMaxBuffer) return NGQ_ERR_UNSUPPORTED;
  if (K > 0 && (rc = check_ptr(x)) != NGQ_OK) return rc;
  // the projections with work, their buffers and sizes
  dev::MultiArgs a;
  std::memset(&a, 0, sizeof(a));
  int kind[NGQ_MAX_PROJ], nout[NGQ_MAX_PROJ];
  size_t wbytes[NGQ_MAX_PROJ], sbytes[NGQ_MAX_PROJ], ybytes[NGQ_MAX_PROJ];
  const ngq_proj* live[NGQ_MAX_PROJ];
  int n = 0, nsets_max = 1, v_max = 1;
  for (int p = 0; p < nproj; ++p) {
    const ngq_proj& pr = projs[p];
    if (pr.n == 0) continue;
    const int nsets = pr.swiglu + 1, Ncols = pr.n * nsets;
    const size_t wb0 = p0_bytes(K, Ncols, f[p].bits), wb1 = p1_bytes(K, Ncols, f[p].bits);
    const size_t sb = (size_t)(K / kGroup) * Ncols * 2, yb = (size_t)T * pr.n * 2;
    if ((rc = check_ptr(pr.y)) != NGQ_OK) return rc;
    if (K > 0) {
      if ((rc = check_ptr(pr.wq)) != NGQ_OK) return rc;
      if ((rc = check_ptr(pr.scales)) != NGQ_OK) return rc;
    }
    if (yb >= kMaxBuffer || wb0 + wb1 >= kMaxBuffer || sb >= kMaxBuffer) return NGQ_ERR_UNSUPPORTED;
    live[n] = &pr;
    wbytes[n] = wb0 + wb1;
    sbytes[n] = sb;
    ybytes[n] = yb;
    kind[n] = dev::multi_kind(f[p].bits, f[p].scale_bf16, nsets);
    nout[n] = pr.n;
    nsets_max = std::max(nsets_max, nsets);
    v_max = std::max(v_max, dev::multi_v(f[p].bits, nsets));
    dev::MultiProj& mp = a.proj[n];
    mp.wq = pr.wq;
    mp.scales = pr.scales;
    mp.y = pr.y;
    mp.p0_bytes = (uint32_t)wb0;
    mp.p1_bytes = (uint32_t)wb1;
    mp.s_bytes = (uint32_t)sb;
    mp.Nout = pr.n;
    mp.Ncols = Ncols;
    mp.up_off = nsets == 2 ? pr.n : 0;
    mp.kind = kind[n];
    ++n;
  }
  // every output overlaps no input and no other output
  for (int i = 0; i < n; ++i) {
    if (K > 0 && overlaps(live[i]->y, ybytes[i], x, xb)) return NGQ_ERR_ARG;
    for (int j = 0; j < n; ++j) {
      if (K > 0 && (overlaps(live[i]->y, ybytes[i], live[j]->wq, wbytes[j]) ||
                    overlaps(live[i]->y, ybytes[i], live[j]->scales, sbytes[j])))
        return NGQ_ERR_ARG;
      if (j != i && overlaps(live[i]->y, ybytes[i], live[j]->y, ybytes[j])) return NGQ_ERR_ARG;
    }
  }
  if (n == 0) return NGQ_OK;
  if (T <= kMultiStreamMaxT && K > 0 && std::all_of(kind, kind + n, [](int k) { return dev::multi_tile_kind(k); }))
    return run_multi_tiles(T, K, x, xb, a, kind, n, stream);
  const uint32_t lds = dev::XSmem::bytes(T, K, dev::kMultiW, 1, 0) +
                       (uint32_t)dev::kMultiW * dev::Smem::block_floats(nsets_max, 16 * v_max) * 4u;
  if (lds > kMaxLds) return NGQ_ERR_UNSUPPORTED;
  // The projection with the most tiles first: every workgroup has tiles of it
  // (when any projection has as many tiles as workgroups), so each one finds
  // its first segment without scanning.
  {
    int order[NGQ_MAX_PROJ];
    for (int i = 0; i < n; ++i) order[i] = i;
    std::stable_sort(order, order + n, [&](int i, int j) {
      return (nout[i] + 31) / 32 > (nout[j] + 31) / 32;
    });
    dev::MultiProj mp[NGQ_MAX_PROJ];
    int kd[NGQ_MAX_PROJ], no[NGQ_MAX_PROJ];
    for (int i = 0; i < n; ++i) {
      mp[i] = a.proj[order[i]];
      kd[i] = kind[order[i]];
      no[i] = nout[order[i]];
    }
    for (int i = 0; i < n; ++i) {
      a.proj[i] = mp[i];
      kind[i] = kd[i];
      nout[i] = no[i];
    }
  }
  const int grid = load_plan(K, n, kind, nout, std::min(cu_count(), dev::kMultiMaxWg), a);
  if (grid < 0) return NGQ_ERR_UNSUPPORTED;
  a.x = x;
  a.x_bytes = (uint32_t)xb;
  a.T = T;
  a.K = K;
  a.G = K / kGroup;
  a.pairs = (a.G + 1) / 2;
  const int per = (a.pairs + dev::kMultiW - 1) / dev::kMultiW;
  a.ppw = (per + dev::kMultiNB - 1) / dev::kMultiNB * dev::kMultiNB;
  a.mask_nib = dev::kMasks.nib;
  a.mask_base = dev::kMasks.base;
  a.mask_hi = dev::kMasks.hi;
  using Kern = void (*)(dev::MultiArgs);
  static const Kern kernels[2] = {dev::gemm_multi_kernel<false>, dev::gemm_multi_kernel<true>};
  static std::atomic<uint64_t> raised[2] = {{0}, {0}};
  const bool big_x = (long)T * (K / 8) > (long)dev::kMultiXL * dev::kMultiW * 64;
  if (raise_lds(reinterpret_cast<const void*>(kernels[big_x ? 1 : 0]), raised[big_x ? 1 : 0]) != hipSuccess)
    return NGQ_ERR_HIP;
  if (grid == 0) return NGQ_OK;
  hipLaunchKernelGGL(kernels[big_x ? 1 : 0], dim3((unsigned)grid), dim3(dev::kMultiW * 64), lds,
                     (hipStream_t)stream, a);
  return hipGetLastError() == hipSuccess ? NGQ_OK : NGQ_ERR_HIP;
}


// ---- split K (host) ----

constexpr int kSplitMax = 8;  // slices; the workspace is sized for this many

// Workspace bytes of the split-K call: the fp32 partials of kSplitMax slices
// at NGQ_MAX_T tokens.
size_t splitk_workspace_bytes(int N) { return (size_t)kSplitMax * NGQ_MAX_T * (size_t)N * 4u; }

// Slices for a shape whose 32-column tiles leave CUs idle: as many as let
// S x (64-column tiles) fill the CUs once, with at least 8 pairs a slice, at
// most kSplitMax; 1 means no split.  The down projection (K = 17408, N = 5120)
// gets 3 slices x 80 tiles.  Measured on MI355X (interleaved A/B, the split
// and its closing kernel): 12.2, 12.7, 12.8, 13.5 us at T = 1, 2, 4, 8
// against 14.2, 15.1, 16.1 for the unsplit streaming kernels and 16.1 for
// the earlier 8-slice X-resident split at T = 8; with the closing rescale
// 15.0 / 16.3 us at T = 1 / 8 against 18.3 / 19.9.  2 slices (160
// workgroups) or 4 (320), and 32-column tiles, were slower.
int split_count(int K, int N, int cus) {
  const int pairs = (K / kGroup + 1) / 2, tiles64 = (N + 63) / 64;
  if ((N + 31) / 32 >= cus || tiles64 == 0) return 1;
  return std::max(1, std::min(kSplitMax, std::min(cus / tiles64, pairs / 8)));
}

// The split kernel: S x (64-column tiles) workgroups.
template <int BITS, bool SBF16>
hipError_t launch_splitk_b(const dev::SplitArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)(a.S * a.g.ntiles)), blk(dev::kSplitWaves * 64);
  const uint32_t lds = dev::StreamSmem<dev::kSplitWaves>::bytes(16 * dev::kSplitV, 1);
  if (a.g.T == 1)
    hipLaunchKernelGGL((dev::gemm_splitk_kernel<BITS, SBF16, 1>), grid, blk, lds, st, a);
  else if (a.g.T == 2)
    hipLaunchKernelGGL((dev::gemm_splitk_kernel<BITS, SBF16, 2>), grid, blk, lds, st, a);
  else if (a.g.T <= 4)
    hipLaunchKernelGGL((dev::gemm_splitk_kernel<BITS, SBF16, 4>), grid, blk, lds, st, a);
  else
    hipLaunchKernelGGL((dev::gemm_splitk_kernel<BITS, SBF16, 8>), grid, blk, lds, st, a);
  return hipGetLastError();
}
static_assert(dev::StreamSmem<dev::kSplitWaves>::bytes(16 * dev::kSplitV, 1) <= 64u * 1024u,
              "the split kernel's LDS stays under the default 64 KiB limit");

// x_next == nullptr: ngq_gemm_splitk.  Otherwise ngq_gemm_rescale: the same
// projection and split, then x_next = the RMS rescale of y; where K is split
// the closing kernel also does the rescale, so the split's second launch
// replaces the rescale's own.  With a residual (ngq_gemm_residual_rescale) K
// is always split (split_count's slices, or one), so that the residual meets
// the fp32 sum in the closing kernel and y is rounded once.
int run_splitk(int T, int K, int N, int bits, int group, const void* x, const void* wq, const void* scales, void* y,
               void* x_next, const void* residual, void* workspace, size_t workspace_bytes, void* stream) {
  Format f;
  int rc = parse_format(bits, group, &f);
  if (rc != NGQ_OK) return rc;
  if (T < 0 || T > NGQ_MAX_T) return NGQ_ERR_SHAPE;
  if ((rc = check_kn(K, N)) != NGQ_OK) return rc;
  const bool fuse = x_next != nullptr, res = residual != nullptr;
  if (res && !fuse) return NGQ_ERR_ARG;
  const int pairs = (K / kGroup + 1) / 2;
  const int S = split_count(K, N, cu_count());
  const bool split = S > 1 || res;  // the split kernel and a closing kernel
  const size_t xb = (size_t)T * K * 2, yb = (size_t)T * N * 2;
  const size_t wb0 = p0_bytes(K, N, f.bits), wb1 = p1_bytes(K, N, f.bits), sb = (size_t)(K / kGroup) * N * 2;
  if (fuse && T > 0 && N > 0) {
    if ((rc = check_ptr(x_next)) != NGQ_OK) return rc;
    if (yb >= kMaxBuffer) return NGQ_ERR_UNSUPPORTED;
    if (overlaps(x_next, yb, x, xb) || overlaps(x_next, yb, wq, wb0 + wb1) || overlaps(x_next, yb, scales, sb) ||
        overlaps(x_next, yb, y, yb) || (split && overlaps(x_next, yb, workspace, (size_t)S * T * N * 4)))
      return NGQ_ERR_ARG;
  }
  if (res && T > 0 && N > 0) {
    // read while other workgroups write y and x_next: no overlap with either
    if ((rc = check_ptr(residual)) != NGQ_OK) return rc;
    if (overlaps(residual, yb, y, yb) || overlaps(residual, yb, x_next, yb) ||
        overlaps(residual, yb, workspace, (size_t)S * T * N * 4))
      return NGQ_ERR_ARG;
  }
  if (!split) {
    rc = run_gemm(1, T, K, N, bits, group, x, wq, scales, y, stream);
    if (rc != NGQ_OK || !fuse) return rc;
    return ngq_rms_rescale(T, N, y, x_next, stream);
  }
  if (T == 0 || N == 0) return NGQ_OK;
  const size_t pb = (size_t)S * T * N * 4;
  if ((rc = check_ptr(y)) != NGQ_OK || (rc = check_ptr(x)) != NGQ_OK || (rc = check_ptr(wq)) != NGQ_OK ||
      (rc = check_ptr(scales)) != NGQ_OK || (rc = check_ptr(workspace)) != NGQ_OK)
    return rc;
  if (workspace_bytes < pb) return NGQ_ERR_ARG;
  if (xb >= kMaxBuffer || yb >= kMaxBuffer || wb0 + wb1 >= kMaxBuffer || sb >= kMaxBuffer || pb >= kMaxBuffer)
    return NGQ_ERR_UNSUPPORTED;
  if (overlaps(y, yb, x, xb) || overlaps(y, yb, wq, wb0 + wb1) || overlaps(y, yb, scales, sb) ||
      overlaps(workspace, pb, x, xb) || overlaps(workspace, pb, wq, wb0 + wb1) ||
      overlaps(workspace, pb, scales, sb) || overlaps(workspace, pb, y, yb))
    return NGQ_ERR_ARG;
  dev::SplitArgs a;
  dev::GemmArgs& g = a.g;
  g.x = x; g.wq = wq; g.scales = scales; g.y = y;
  g.T = T; g.K = K; g.Nout = N; g.Ncols = N; g.up_off = 0;
  g.G = K / kGroup; g.pairs = pairs; g.ppw = 0;  // the slices set their own
  g.ntiles = (N + 16 * dev::kSplitV - 1) / (16 * dev::kSplitV);
  g.p0_bytes = (uint32_t)wb0; g.p1_bytes = (uint32_t)wb1; g.s_bytes = (uint32_t)sb; g.x_bytes = (uint32_t)xb;
  g.mask_nib = dev::kMasks.nib; g.mask_base = dev::kMasks.base; g.mask_hi = dev::kMasks.hi;
  g.tiles_q = g.tiles_r = 0;
  a.partial = static_cast<float*>(workspace);
  a.S = S;
  a.pps = (pairs + S - 1) / S;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (f.bits == 4)
    e = f.scale_bf16 ? launch_splitk_b<4, true>(a, st) : launch_splitk_b<4, false>(a, st);
  else if (f.bits == 5)
    e = f.scale_bf16 ? launch_splitk_b<5, true>(a, st) : launch_splitk_b<5, false>(a, st);
  else
    e = f.scale_bf16 ? launch_splitk_b<8, true>(a, st) : launch_splitk_b<8, false>(a, st);
  if (e != hipSuccess) return NGQ_ERR_HIP;
  if (fuse && reduce_rescale_fits(N))
    return launch_reduce_rescale(static_cast<const float*>(workspace), S, T, N, y, x_next, residual, stream);
  const int TN = T * N;
  hipLaunchKernelGGL(dev::splitk_reduce_kernel, dim3((unsigned)((TN / 4 + 255) / 256)), dim3(256), 0, st,
                     static_cast<const float*>(workspace), S, TN, static_cast<uint16_t*>(y),
                     static_cast<const uint16_t*>(residual));
  if (hipGetLastError() != hipSuccess) return NGQ_ERR_HIP;
  return fuse ? ngq_rms_rescale(T, N, y, x_next, stream) : NGQ_OK;
}

// Device address of the static scratch array on the current device, looked up
// once per device (with that device current) and kept; nullptr and the HIP
// status on failure.
void* static_scratch(hipError_t& err) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> ptrs[kMaxDevices];
  static std::mutex mu;
  int dev = 0;
  err = hipGetDevice(&dev);
  if (err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    err = hipErrorInvalidDevice;
    return nullptr;
  }
  void* p = ptrs[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(mu);
  p = ptrs[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(dev::scratch));
    if (err != hipSuccess) return nullptr;
    ptrs[dev].store(p, std::memory_order_release);
  }
  return p;
}

int run_splitk_static(int T, int K, int N, int bits, int group, const void* x, const void* wq, const void* scales,
                      void* y, void* stream) {
  Format f;
  int rc = parse_format(bits, group, &f);
  if (rc != NGQ_OK) return rc;
  if (T < 0 || T > NGQ_MAX_T) return NGQ_ERR_SHAPE;
  if ((rc = check_kn(K, N)) != NGQ_OK) return rc;
  if (T == 0 || N == 0) return NGQ_OK;
  // the same split as ngq_gemm_splitk; the partial sums must fit the array
  const int S = split_count(K, N, cu_count());
  const size_t need = S > 1 ? (size_t)S * T * N * 4u : 0;
  if (need > dev::kStaticScratchBytes) return NGQ_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (S > 1) {
    hipError_t e;
    ws = static_scratch(e);
    if (ws == nullptr) return NGQ_ERR_HIP;
  }
  return run_splitk(T, K, N, bits, group, x, wq, scales, y, nullptr, nullptr, ws,
                    S > 1 ? dev::kStaticScratchBytes : 0, stream);
}

}  // namespace
}  // namespace ngq

using namespace ngq;

extern "C" int ngq_gemm(int T, int K, int N, int bits, int group, const void* x, const void* wq,
                        const void* scales, void* y, void* stream) {
  return run_gemm(1, T, K, N, bits, group, x, wq, scales, y, stream);
}

extern "C" int ngq_swiglu_gemm(int T, int K, int N_ff, int bits, int group, const void* x,
                               const void* wq_gate_up, const void* scales_gate_up, void* h, void* stream) {
  return run_gemm(2, T, K, N_ff, bits, group, x, wq_gate_up, scales_gate_up, h, stream);
}

extern "C" int ngq_multi_gemm(int T, int K, int group, const void* x, const ngq_proj* projs, int nproj,
                              void* stream) {
  return run_multi(T, K, group, x, projs, nproj, stream);
}

extern "C" size_t ngq_splitk_workspace_bytes(int K, int N, int bits, int group) {
  Format f;
  if (parse_format(bits, group, &f) != NGQ_OK || check_kn(K, N) != NGQ_OK) return 0;
  return splitk_workspace_bytes(N);
}

extern "C" int ngq_gemm_splitk(int T, int K, int N, int bits, int group, const void* x, const void* wq,
                               const void* scales, void* y, void* workspace, size_t workspace_bytes, void* stream) {
  return run_splitk(T, K, N, bits, group, x, wq, scales, y, nullptr, nullptr, workspace, workspace_bytes, stream);
}

extern "C" int ngq_gemm_splitk_static(int T, int K, int N, int bits, int group, const void* x, const void* wq,
                                      const void* scales, void* y, void* stream) {
  return run_splitk_static(T, K, N, bits, group, x, wq, scales, y, stream);
}

extern "C" int ngq_gemm_rescale(int T, int K, int N, int bits, int group, const void* x, const void* wq,
                                const void* scales, void* y, void* x_next, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (x_next == nullptr) return NGQ_ERR_ARG;
  return run_splitk(T, K, N, bits, group, x, wq, scales, y, x_next, nullptr, workspace, workspace_bytes, stream);
}

extern "C" int ngq_gemm_residual_rescale(int T, int K, int N, int bits, int group, const void* x, const void* wq,
                                         const void* scales, const void* residual, void* y, void* x_next,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  if (x_next == nullptr || residual == nullptr) return NGQ_ERR_ARG;
  return run_splitk(T, K, N, bits, group, x, wq, scales, y, x_next, residual, workspace, workspace_bytes, stream);
}

extern "C" int ngq_unpack_codes(int K, int N, int bits, int group, const void* wq, int8_t* codes, void* stream) {
  return run_unpack<false>(K, N, bits, group, wq, nullptr, codes, stream);
}

extern "C" int ngq_dequant_f32(int K, int N, int bits, int group, const void* wq, const void* scales, float* w,
                               void* stream) {
  return run_unpack<true>(K, N, bits, group, wq, scales, w, stream);
}

extern "C" int ngq_stream_read(const void* buf, size_t bytes, void* sink, void* stream) {
  if (bytes % 16) return NGQ_ERR_SHAPE;
  if (bytes == 0) return NGQ_OK;
  int rc;
  if ((rc = check_ptr(buf)) != NGQ_OK) return rc;
  if ((rc = check_ptr(sink)) != NGQ_OK) return rc;
  const size_t n16 = bytes / 16;
  size_t blocks = (n16 + 255) / 256;
  blocks = std::min<size_t>(blocks, 4096);
  hipLaunchKernelGGL(dev::stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const dev::u32x4*>(buf), n16, static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? NGQ_OK : NGQ_ERR_HIP;
}

extern "C" int ngq_stream_tiles(int K, int N, int bits, int group, int cols, const void* wq, const void* scales,
                                void* sink, void* stream) {
  Format f;
  int rc = parse_format(bits, group, &f);
  if (rc != NGQ_OK) return rc;
  if ((rc = check_kn(K, N)) != NGQ_OK) return rc;
  if (cols != 32 && cols != 48) return NGQ_ERR_UNSUPPORTED;
  if (N % cols != 0) return NGQ_ERR_SHAPE;  // whole tiles only
  if (K == 0 || N == 0) return NGQ_OK;
  if ((rc = check_ptr(wq)) != NGQ_OK || (rc = check_ptr(scales)) != NGQ_OK || (rc = check_ptr(sink)) != NGQ_OK)
    return rc;
  const size_t wb0 = p0_bytes(K, N, f.bits), wb1 = p1_bytes(K, N, f.bits), sb = (size_t)(K / kGroup) * N * 2;
  if (wb0 + wb1 >= kMaxBuffer || sb >= kMaxBuffer) return NGQ_ERR_UNSUPPORTED;
  const int ntiles = (N + cols - 1) / cols;
  if (ntiles > 2048) return NGQ_ERR_SHAPE;  // the sink holds two words per workgroup
  dev::GemmArgs a;
  std::memset(&a, 0, sizeof(a));
  a.wq = wq; a.scales = scales;
  a.K = K; a.Nout = N; a.Ncols = N;
  a.G = K / kGroup;
  a.pairs = (a.G + 1) / 2;
  a.ntiles = ntiles;
  a.p0_bytes = (uint32_t)wb0; a.p1_bytes = (uint32_t)wb1; a.s_bytes = (uint32_t)sb;
  const int W = cols == 32 ? stream_waves(f.bits) : 8;
  a.ppw = (a.pairs + W - 1) / W;
  uint32_t* sk = static_cast<uint32_t*>(sink);
  hipStream_t st = (hipStream_t)stream;
  auto go = [&](auto kern, int w) {
    hipLaunchKernelGGL(kern, dim3((unsigned)ntiles), dim3(w * 64), 0, st, a, sk);
    return hipGetLastError() == hipSuccess ? NGQ_OK : NGQ_ERR_HIP;
  };
  if (f.bits == 4) return cols == 32 ? go(dev::stream_tiles_kernel<4, 2, 10>, 10) : go(dev::stream_tiles_kernel<4, 3, 8>, 8);
  if (f.bits == 5) return cols == 32 ? go(dev::stream_tiles_kernel<5, 2, 10>, 10) : go(dev::stream_tiles_kernel<5, 3, 8>, 8);
  return cols == 32 ? go(dev::stream_tiles_kernel<8, 2, kStreamW8>, kStreamW8) : go(dev::stream_tiles_kernel<8, 3, 8>, 8);
}

extern "C" int ngq_debug_force_kernel(int path) {
  if (path < NGQ_KERNEL_AUTO || path > NGQ_KERNEL_DOT) return NGQ_ERR_ARG;
  return kernel_override.exchange(path);
}
