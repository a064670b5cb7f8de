/*
 * ngq.h -- C ABI of libngq: small-T groupwise-int projections on MI355X (gfx950).
 *
 * The operation.  A decode or speculative-verify step of a groupwise-int
 * quantised model multiplies T <= 8 token activations (up to 64 when
 * several requests are verified together) by each quantised projection matrix:
 *
 *     Y[T x N] = X[T x K] . dequant(Wq[K x N]),   dequant: w[k][n] = c[k][n] * s[k/64][n]
 *
 * The NInfer-4090 V3 topic (lcz.me/topic/2047), section "What V3 did", tunes
 * the T=8 routing of small-batch Q4/Q5 projections for the GDN projection, the
 * attention Q5 projection and the SwiGLU path, and its "Measured data"
 * section times the T=8 attention Q5 gate/value and GDN QK Q4 projections as
 * single operators.  The ninfer-ext README, "Comparison with upstream NInfer",
 * credits a Q5 K-split path aimed at the verify rounds of speculative decoding
 * (T = drafts + 1).  The pages fix neither the layout nor the arithmetic;
 * this library takes symmetric codes with one scale per 64 consecutive k and
 * column, fp32 accumulation and bf16 output.
 *
 * Conventions (all entry points):
 *  - Every buffer is allocated by the caller.  Device pointers are HIP device
 *    memory on the current device; host pointers are ordinary host memory.
 *    The library keeps no pointer after a call returns and allocates nothing.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  GPU
 *    entry points enqueue work and return without synchronising; a device
 *    fault surfaces at the caller's next synchronisation.
 *  - Arguments are validated before any HIP call; on error nothing is
 *    enqueued and a negative NGQ_ERR_* status is returned.  No C++ exception
 *    crosses this boundary.  Entry points are reentrant and thread-safe.
 *  - Results are deterministic: the same inputs on the same device give
 *    bit-identical outputs (no atomics, fixed reduction order).
 *  - Every buffer must be 16-byte aligned and smaller than 2 GiB.
 *
 * Packed weight layout (little-endian 32-bit words, row-major, column fastest;
 * u is the offset-binary field, c the signed code):
 *   int4 (bits 4): P0 = u32[K/8][N]; bits 4i..4i+3 of word (kb, n) hold
 *                  u = c + 8 for k = 8 kb + i.  c in [-8, 7].
 *   int5 (bits 5): P0 as int4 holding u & 15 with u = c + 16, then directly
 *                  after it P1 = u32[K/32][N]; bit i of word (kb, n) holds
 *                  u >> 4 for k = 32 kb + i.  c in [-16, 15].
 *   int8 (bits 8): P0 = u32[K/4][N]; byte i of word (kb, n) holds u = c + 128
 *                  for k = 4 kb + i.  c in [-128, 127].
 *   scales:        [K/64][N] fp16 (default) or bf16 (bits | NGQ_SCALE_BF16).
 *   x:             [T][K] bf16, row-major.   y: [T][N] bf16, row-major.
 */
#ifndef NGQ_H
#define NGQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define NGQ_OK 0
#define NGQ_ERR_ARG (-1)         /* null pointer, aliasing output, code out of range */
#define NGQ_ERR_SHAPE (-2)       /* T, K or N outside the supported shapes */
#define NGQ_ERR_UNSUPPORTED (-3) /* bit width, scale flag, group size or buffer size */
#define NGQ_ERR_ALIGN (-4)       /* a buffer is not 16-byte aligned */
#define NGQ_ERR_HIP (-5)         /* the HIP runtime reported an error */

/* Bit widths, and the flag selecting bf16 scales (OR it into `bits`). */
#define NGQ_INT4 4
#define NGQ_INT5 5
#define NGQ_INT8 8
#define NGQ_SCALE_BF16 0x100
#define NGQ_GROUP 64 /* the only supported group size */
#define NGQ_MAX_T 8  /* tokens per call: plain decode (1) up to 7 drafts + 1 */
#define NGQ_MAX_T_VERIFY 64 /* several requests verified in one call: up to 8 requests x 8 tokens */
#define NGQ_MAX_T_PREFILL 16384 /* ngq_gemm / ngq_swiglu_gemm: prefill chunks */

/* Bytes of the packed weight buffer (P0, plus P1 for int5) for a K x N
 * matrix; 0 when the arguments are invalid.  Host only, no HIP call. */
size_t ngq_packed_bytes(int K, int N, int bits, int group);

/* Bytes of the scale buffer, (K/64) * N * 2; 0 when invalid.  Host only. */
size_t ngq_scale_bytes(int K, int N, int bits, int group);

/* Pack signed codes into the layout above.  Host only, no HIP call.
 *   codes  : host int8 [K][N], row-major, each within the range of `bits`
 *   wq_out : host buffer of ngq_packed_bytes(K, N, bits, group) bytes
 * K % 64 == 0, N % 4 == 0.  Returns NGQ_ERR_ARG for a code out of range (the
 * output is then unspecified), NGQ_ERR_SHAPE / NGQ_ERR_UNSUPPORTED as above.
 * The NGQ_SCALE_BF16 flag is ignored here. */
int ngq_pack(int K, int N, int bits, int group, const int8_t* codes, void* wq_out);

/* Y = X . dequant(Wq) for 0 <= T <= 16384 tokens.  T <= 8 is one request's
 * decode or verify step (the projection of the "What V3 did" T-routing,
 * NInfer-4090 V3 topic).  8 < T <= 64 is the verify rounds of several
 * requests stacked into one call, so that the weights stream once for all of
 * them: an engine serves up to 8 active requests (HotRepo page on
 * Neroued/ninfer, "Constraints"), each verifying up to 7 drafts + 1 (the
 * ninfer-ext README, "Recommended settings"; the V3 topic's "Measured data"
 * runs 2, 4 and 8 requests with 7 drafts).  T > 64 is a prefill chunk (the
 * V3 topic's quick start runs chunks of 1024 tokens), computed in token x
 * column tiles.
 *   x      : device bf16 [T][K]
 *   wq     : device, ngq_pack layout for K x N
 *   scales : device fp16|bf16 [K/64][N]
 *   y      : device bf16 [T][N], overwritten; must not overlap the inputs
 * K % 64 == 0 (K = 0 writes zeros), N % 4 == 0; T == 0 or N == 0 is a no-op.
 * Accumulates in fp32 and rounds to bf16 to nearest even. */
int ngq_gemm(int T, int K, int N, int bits, int group, const void* x, const void* wq,
             const void* scales, void* y, void* stream);

/* Fused gate/up projection with the SiLU-times-up epilogue of a SwiGLU MLP
 * (the "SwiGLU path" of the NInfer-4090 V3 topic, section "What V3 did"):
 *   h[t][j] = bf16( SiLU(g) * u ),  g = (X . W)[t][j],  u = (X . W)[t][N_ff + j]
 * with SiLU(g) = g / (1 + e^-g), g and u kept in fp32.
 *   x              : device bf16 [T][K]
 *   wq_gate_up     : device, ngq_pack layout of the K x (2 N_ff) matrix whose
 *                    columns [0, N_ff) are the gate and [N_ff, 2 N_ff) the up
 *                    projection
 *   scales_gate_up : device fp16|bf16 [K/64][2 N_ff]
 *   h              : device bf16 [T][N_ff], overwritten; must not overlap inputs
 * T as for ngq_gemm (0..16384).  The down projection is a plain ngq_gemm with
 * K = N_ff and x = h. */
int ngq_swiglu_gemm(int T, int K, int N_ff, int bits, int group, const void* x,
                    const void* wq_gate_up, const void* scales_gate_up, void* h, void* stream);

/* Bytes of the workspace ngq_gemm_splitk needs for a K x N projection at any
 * T <= 8 (fp32 partial sums of up to 8 K slices); 0 when the arguments are
 * invalid.  Host only, no HIP call. */
size_t ngq_splitk_workspace_bytes(int K, int N, int bits, int group);

/* ngq_gemm for long K and few 32-column tiles (a down projection: K = 17408,
 * N = 5120), with K split into slices of whole group pairs so that every CU
 * has work: one workgroup per 64-column tile and slice, each streaming its
 * slice's pairs with their X bands.  Each slice's fp32 sum goes to
 * `workspace`, and a second kernel on the same stream adds the slices' sums
 * in slice order and rounds to bf16.
 *   workspace : device, at least ngq_splitk_workspace_bytes(K, N, bits, group)
 *               bytes, 16-byte aligned; no initial contents are needed; it
 *               must not overlap the other buffers, and calls that may run
 *               at the same time must not share it (too small: NGQ_ERR_ARG)
 * Shapes, formats and status codes as ngq_gemm.  K is split, at any T, where
 * the 32-column tiles alone leave CUs idle, into as many slices (at most 8)
 * as let the slices' 64-column tiles fill the CUs once with at least 8 pairs
 * each (the down projection: 3); where that leaves one slice the call runs
 * as ngq_gemm and the workspace is not used.
 * The fp32 sums are grouped differently from ngq_gemm's, so the two can
 * differ in the last bit; each is deterministic. */
int ngq_gemm_splitk(int T, int K, int N, int bits, int group, const void* x, const void* wq,
                    const void* scales, void* y, void* workspace, size_t workspace_bytes, void* stream);

/* ngq_gemm_splitk for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels, split and result bit for bit, with the fp32 partial sums
 * in a fixed array of NGQ_STATIC_SCRATCH_BYTES in device memory that the
 * library holds on each device it runs on until the process ends.  The call
 * allocates nothing; the caller passes inputs and outputs as for
 * ngq_gemm_splitk.
 *  - The array's device address is looked up on a device's first call (a
 *    HIP runtime query, no allocation).
 *  - Where K is split into S slices, the partial sums take S * T * N * 4
 *    bytes (S <= 8); beyond NGQ_STATIC_SCRATCH_BYTES the call returns
 *    NGQ_ERR_UNSUPPORTED before any launch.  Unsplit calls need no scratch.
 *  - Every call on one device shares that device's array: calls that may run
 *    at the same time on one device (other streams, other threads) race and
 *    must be ordered by the caller.  Nothing in the array needs to start at
 *    zero: the split kernels write every partial sum they read.
 * Shapes, formats and other status codes as ngq_gemm_splitk. */
#define NGQ_STATIC_SCRATCH_BYTES (4u << 20)
int ngq_gemm_splitk_static(int T, int K, int N, int bits, int group, const void* x, const void* wq,
                           const void* scales, void* y, void* stream);

/* Several projections of the same activations in one launch.  The
 * projections of a layer that read one x (in the stacked sweep: QK,
 * gate/value and the gate/up pair) are computed as one kernel, so the launch
 * is paid once and the tiles of all of them are spread over the CUs
 * together.  Each projection computes exactly what ngq_gemm (swiglu = 0) or
 * ngq_swiglu_gemm (swiglu = 1) computes for it: the same formula, fp32
 * accumulation and bf16 rounding.
 *   x     : device bf16 [T][K], shared by every projection
 *   projs : host array of nproj (1..NGQ_MAX_PROJ) descriptions, read during
 *           the call only:
 *     bits   : NGQ_INT4 | NGQ_INT5 | NGQ_INT8, optionally | NGQ_SCALE_BF16
 *     n      : output columns (N, or N_ff with swiglu); n % 4 == 0; 0 = skip
 *     swiglu : 0 plain, 1 gate/up with the SiLU(gate) * up epilogue
 *     reserved : must be 0
 *     wq, scales : device, as for ngq_gemm over n (plain) or 2 n (swiglu)
 *                  columns
 *     y      : device bf16 [T][n], overwritten; no output may overlap x, any
 *              projection's wq or scales, or another output
 * K % 64 == 0; T == 0 is a no-op.  X and the partial sums must fit in the
 * workgroup's LDS (T * (2 K + 16) + 128 bytes for X: K up to ~9000 at T = 8),
 * otherwise NGQ_ERR_UNSUPPORTED.  Any mix of bit widths, scale types and
 * plain / SwiGLU projections may share a call.  When every projection is
 * int4 (plain or SwiGLU) or plain int5 / int8, the call runs instead one
 * workgroup per 32-column tile of any projection (the VALU step with 7 waves
 * at T = 1, the MFMA step with 4 waves above; the hardware spreads the
 * unequal tiles), with no LDS limit on K. */
#define NGQ_MAX_PROJ 4
typedef struct ngq_proj {
  int bits;
  int n;
  int swiglu;
  int reserved;
  const void* wq;
  const void* scales;
  void* y;
} ngq_proj;
int ngq_multi_gemm(int T, int K, int group, const void* x, const ngq_proj* projs, int nproj, void* stream);

/* Per-token RMS rescale of a bf16 block (not a step the pages describe: it
 * chains the output of one stacked layer into the next at unit scale):
 *   x[t][n] = bf16( z[t][n] / sqrt((1/N) sum_n z[t][n]^2) ),  all-zero row -> zeros
 * No epsilon, no learned weight.  Evaluated in fp64 and rounded once, to
 * nearest even, from the fp64 quotient.
 *   z : device bf16 [T][N];  x : device bf16 [T][N], overwritten.  x == z
 *       (in place) is allowed; any other overlap is NGQ_ERR_ARG.
 * 0 <= T <= 65535, 0 <= N <= 2^24; T == 0 or N == 0 is a no-op. */
int ngq_rms_rescale(int T, int N, const void* z, void* x, void* stream);

/* The last projection of a stacked layer with the rescale that closes it:
 *   y      = X . dequant(Wq) in bf16, as ngq_gemm_splitk computes it, and
 *   x_next = the per-token RMS rescale of y, as ngq_rms_rescale(T, N, y, x_next)
 * computes it (bit for bit, given the same y).  K is split as
 * ngq_gemm_splitk splits it (the down projection: K = 17408, N = 5120, 3
 * slices at every T), and the kernel that adds the slices' fp32 sums also
 * rescales the rows, so the pair of results costs two launches; where no
 * split applies the call is ngq_gemm followed by ngq_rms_rescale.  y equals
 * ngq_gemm_splitk's y bit for bit.
 *   x_next    : device bf16 [T][N], overwritten; must not overlap x, wq,
 *               scales, y or the workspace (NGQ_ERR_ARG); null: NGQ_ERR_ARG
 *   workspace : as for ngq_gemm_splitk (ngq_splitk_workspace_bytes bytes)
 * Other arguments, shapes and status codes as ngq_gemm_splitk. */
int ngq_gemm_rescale(int T, int K, int N, int bits, int group, const void* x, const void* wq,
                     const void* scales, void* y, void* x_next, void* workspace, size_t workspace_bytes,
                     void* stream);

/* The same closing step with the residual connection added in the epilogue
 * (not a step the pages describe: the residual stream of the stacked layer,
 * added where the last projection's sums are closed, so that the block
 * needs no separate pass):
 *   y      = bf16( X . dequant(Wq) + residual ): the residual (bf16) is added
 *            to the projection's fp32 sum, which is rounded once
 *   x_next = the per-token RMS rescale of y, as ngq_rms_rescale(T, N, y, x_next)
 * K is always split here (ngq_gemm_splitk's slices, or one slice where it
 * does not split), and the kernel that adds the slices' fp32 sums in slice
 * order adds the residual last; the sums are grouped as in ngq_gemm_rescale
 * wherever that one splits, and y can differ from ngq_gemm_rescale's y +
 * residual in the last bit (one rounding here, two there).
 *   residual : device bf16 [T][N]; must not overlap y, x_next or the
 *              workspace (NGQ_ERR_ARG: other workgroups write those while it
 *              is read); null: NGQ_ERR_ARG
 *   workspace: device, at least ngq_splitk_workspace_bytes(K, N, bits, group)
 *              bytes, for every T (it is always used)
 * Other arguments, shapes and status codes as ngq_gemm_rescale. */
int ngq_gemm_residual_rescale(int T, int K, int N, int bits, int group, const void* x, const void* wq,
                              const void* scales, const void* residual, void* y, void* x_next, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Debug export: the signed codes as the GEMM kernels unpack them.
 *   wq : device, ngq_pack layout;  codes : device int8 [K][N], overwritten. */
int ngq_unpack_codes(int K, int N, int bits, int group, const void* wq, int8_t* codes, void* stream);

/* Debug export: w[k][n] = c[k][n] * s[k/64][n] in fp32 (exact), with the
 * GEMM kernels' unpack and scale decoding.  w : device float [K][N]. */
int ngq_dequant_f32(int K, int N, int bits, int group, const void* wq, const void* scales, float* w,
                    void* stream);

/* Debug export: force the kernel path of ngq_gemm / ngq_swiglu_gemm for every
 * later call in the process (tests use it to run each path on the same
 * shapes).  NGQ_KERNEL_AUTO restores the per-shape choice.  Paths 1..4, 10
 * and 11 are the T <= 8 kernels (larger T keeps the library's choice under them);
 * NGQ_KERNEL_WIDE serves 8 < T <= 64; the token x column paths serve any T
 * (the 96- and 128-token ones int4 only).  A forced path that cannot serve a shape (X or the partial sums do not
 * fit in LDS, the 14-wave kernel with the SwiGLU epilogue, NGQ_KERNEL_WIDE
 * outside its T range) makes those calls return NGQ_ERR_UNSUPPORTED.
 * Returns the previous setting, or NGQ_ERR_ARG for an unknown path.  Not
 * thread-safe with respect to calls that are running. */
#define NGQ_KERNEL_AUTO 0
#define NGQ_KERNEL_PERPAIR_DYN 1    /* X per pair, pairs handed out dynamically */
#define NGQ_KERNEL_PERPAIR_STATIC 2 /* X per pair, static pair ranges per wave */
#define NGQ_KERNEL_XRES14 3         /* X resident in LDS, 14 waves, one pair each */
#define NGQ_KERNEL_XRES8 4          /* X resident in LDS, 8 waves, two pairs each */
#define NGQ_KERNEL_WIDE 5           /* 8 < T <= 64: token blocks of 16, X per pair */
#define NGQ_KERNEL_TILED 6          /* token x column tiles (prefill), K split over waves, any T */
#define NGQ_KERNEL_TILED_SX 7       /* token x column tiles, X tile shared by the waves, any T */
#define NGQ_KERNEL_TILED_SX96 8     /* the same with 96-token tiles (int4 only) */
#define NGQ_KERNEL_TILED_SX128 9    /* the same with 128-token tiles (int4 only) */
#define NGQ_KERNEL_STREAM 10        /* T <= 8, one workgroup per column tile, each wave streams its
                                       pairs with their X band (plain or SwiGLU) */
#define NGQ_KERNEL_DOT 11           /* the same pipeline with the multiply-add on the VALU (bf16 dot2);
                                       the library's choice at T = 1 for int4 and int8 (plain
                                       or SwiGLU int4) */
int ngq_debug_force_kernel(int path);

/* Bandwidth calibration: stream `bytes` (a multiple of 16) from device memory
 * `buf` with 128-bit loads and write one word per workgroup to `sink`
 * (device, at least 16384 bytes) so the reads cannot be elided.  Used by the
 * bench to measure the attainable HBM read rate of the device. */
int ngq_stream_read(const void* buf, size_t bytes, void* sink, void* stream);

/* Calibration: the weight stream of a K x N projection in the access pattern
 * of the streaming decode kernel (NGQ_KERNEL_STREAM), alone: the same column
 * tiles (cols = 32 with that kernel's waves per workgroup: 10, or 5 for
 * int8; or cols = 48, 8 waves), pair order and loads of the
 * packed words and scales, with no X, no arithmetic and no output.  Its
 * launch time is what this pattern can attain for the projection's weight
 * bytes, which the bench reports beside the HBM peak.
 *   wq, scales : device, as for ngq_gemm
 *   sink       : device, at least 16384 bytes; word b (b < number of tiles)
 *                receives the XOR of the packed P0 words tile b read (each
 *                once; a check of the pattern), word tiles + b a sum of the
 *                other words it read
 * Status codes as ngq_gemm; cols other than 32 or 48: NGQ_ERR_UNSUPPORTED;
 * N not a multiple of cols (whole tiles only) or more than 2048 tiles:
 * NGQ_ERR_SHAPE. */
int ngq_stream_tiles(int K, int N, int bits, int group, int cols, const void* wq, const void* scales, void* sink,
                     void* stream);

/* Static description of a status code. */
const char* ngq_strerror(int status);

/* Layout/ABI version of this library (increments when either changes). */
int ngq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NGQ_H */
