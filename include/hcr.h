/*
 * hcr.h -- C ABI of the BF16 hyper-connection read (HC read) for MI355X (gfx950).
 *
 * The operation (Strata PR #2812, "sycl: STRATA_GR_FUSED=1, the two-kernel
 * BF16 hyper-connection read (opt-in)", sections Summary and What changed;
 * Strata PR #2070, Turing kernels for the hyper-connection read, first
 * comment): for each of T tokens of a speculative-decode verify window, the
 * S = 4 residual streams of d = 2560 values are RMS-normalised per stream,
 * projected down to R = 320 values (lo, plus an optional injection),
 * projected back up to S x d values, and finished by the epilogue (an
 * optional pending write, a sigmoid gate per stream, the stream mean).
 * Per token t, stream s, column c, down row r, up row j = s*d + c:
 *
 *   rs[t,s]    = 1 / sqrt(mean_c x[t,s,c]^2 + 1e-6)
 *   lo[t,r]    = sum_s rs[t,s] * sum_c W_down[r, s*d+c] * x[t,s,c] * w_norm[s,c]  (+ inj[t,r])
 *   u[t,j]     = sum_k W_up[j,k] * lo[t,k]
 *   out[t,s,c] = pending[t,s,c] (or 0) + sigmoid(lo[t,s]) * u[t, s*d+c]
 *   mean[t,c]  = (1/4) * sum_s out[t,s,c]
 *
 * T may be 0..16 (the pages' windows are 1..8 tokens; 9..16 serve larger windows).
 * Arithmetic is FP32 (BF16 weights are widened exactly; the up projection of
 * BF16 weights runs on the matrix cores with lo split into BF16 high and low
 * parts); summation orders are fixed, so a call is bitwise reproducible, also
 * as a replayed HIP graph.  A token's results are the same bit for bit
 * whatever the other tokens of the window within one range of T: BF16 weights
 * T = 1..8 and T = 9..16, Q8_0 copies T = 1..2, 3..8 and 9..16.
 *
 * Memory. Every pointer is a device pointer the caller owns (the library
 * allocates nothing on the device and never frees caller memory).  Layouts
 * are contiguous, token-major, fixed strides:
 *   x, pending, out : float [T][4][2560]
 *   mean            : float [T][2560]
 *   inj             : float [T][320]
 *   w_down          : BF16  [320][10240]  row-major, column block s = stream s
 *   w_up            : BF16  [10240][320]  row-major, row s*2560 + c
 *   w_norm          : float [4][2560]
 *   scratch         : hcr_scratch_bytes() bytes, 256-byte aligned, one per handle
 * Every pointer but scratch must be 16-byte aligned.
 *
 * Errors. Functions return HCR_OK (0) or a negative code; hcr_strerror()
 * names it.  All argument checks run on the host before any HIP call, so a
 * rejected call has no effect on the device.  There is no fallback path.
 */
#ifndef HCR_H
#define HCR_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HCR_STREAMS 4      /* residual streams S */
#define HCR_STREAM_D 2560  /* values per stream d */
#define HCR_RANK 320       /* down-projection rows R (up-projection K) */
#define HCR_T_MAX 16       /* tokens per read */

enum {
  HCR_OK = 0,
  HCR_EINVAL = -1,   /* null handle/pointer, or T outside 0..HCR_T_MAX */
  HCR_EALIGN = -2,   /* a pointer is not 16-byte (scratch: 256-byte) aligned */
  HCR_ESCRATCH = -3, /* scratch smaller than hcr_scratch_bytes() */
  HCR_EALIAS = -4,   /* buffers overlap in a way the read does not allow */
  HCR_EHIP = -5      /* a HIP launch failed (hipGetLastError after the launches) */
};

typedef struct hcr_handle* hcr_t;

/* Bytes of device scratch one handle needs (partial sums, sums of squares, lo, rs).
 * Basis: Strata PR #2812, Title (the two-kernel read reuses the argument struct,
 * scratch and helpers of the Q8_0 read it builds on); What changed (the down
 * kernel's partial sums and the lo / injection / rs it writes live there). */
size_t hcr_scratch_bytes(void);

/* Byte offsets, inside a handle's scratch, of the last read's lo (float [T][320])
 * and rs (float [T][4]); valid after the read's kernels complete.  Basis: Strata
 * PR #2812, What changed (the finish writes lo / the injection and rs) and Summary
 * (lo / rs / mixed are the outputs compared with the default read). */
int hcr_scratch_layout(size_t* lo_offset, size_t* rs_offset);

/* Geometry compiled into the library (any argument may be NULL).  Basis: Strata
 * PR #2812, What changed (a 1,280-column slab is half a stream; 16 columns x 4
 * streams per up work-group; K = 320); larger T serve Strata PR #2070's larger
 * windows (first comment). */
int hcr_geometry(int* streams, int* stream_d, int* rank, int* t_max);

/* Create a handle for one weight set (one layer half: w_down, w_up, w_norm) and
 * its scratch.  Basis: Strata PR #2812, Title (the argument struct and scratch the
 * read keeps per layer half) and Summary (same BF16 weights, no extra VRAM).
 * Host-only: records pointers, makes no HIP call.  The weights and
 * the scratch must stay valid until hcr_destroy.  Errors: HCR_EINVAL (a NULL
 * pointer), HCR_EALIGN, HCR_ESCRATCH, HCR_EALIAS (scratch overlaps a weight). */
int hcr_create(const void* w_down, const void* w_up, const float* w_norm,
               void* scratch, size_t scratch_bytes, hcr_t* out);

/* Q8_0 copies (Strata PR #2812, Summary: the sibling read of PR #2810 runs the
 * same two kernels on Q8_0 copies of the two projections, kept in VRAM beside
 * the BF16 weights).  The pages do not define the block; this library reads it
 * as GGML's Q8_0: 32 consecutive weights of a row form a block with one IEEE
 * binary16 scale d and 32 int8 codes q, a weight being d * q.  Quantisation,
 * in IEEE binary32: amax = max |w| over the block, d = amax / 127,
 * q = round(w * (1 / d)) with ties away from zero (q = 0 when d = 0), and the
 * stored scale is d rounded to binary16 (nearest, ties to even).
 * Storage is split so that every load stays aligned:
 *   codes  : int8   [rows][cols]        row-major
 *   scales : uint16 [rows][cols / 32]   binary16 bit patterns, row-major
 *
 * hcr_quantize_q8_0: make the Q8_0 copy of a row-major BF16 matrix w
 * [rows][cols] (cols a multiple of 32; weights finite) on the device,
 * asynchronously on `stream` (one kernel; no allocation).  Finite scales need
 * every block's largest |w| to be at most 127 * 65504 = 8,319,008 (65504 is
 * binary16's largest finite value): beyond it d rounds to +inf in binary16, the
 * call still returns HCR_OK, and a read on such copies has non-finite outputs.  The codes and the
 * scales are bitwise those of the rule above.  For the read, W_down is
 * [320][10240] and W_up is [10240][320].  Pointers are device pointers the
 * caller owns, 16-byte aligned, and codes, scales and w must not overlap.
 * Errors: HCR_EINVAL (NULL, rows or cols <= 0, cols % 32 != 0, too large),
 * HCR_EALIGN, HCR_EALIAS (all before any HIP call), HCR_EHIP. */
int hcr_quantize_q8_0(const void* w, int rows, int cols, void* codes, void* scales, void* stream);

/* Create a handle that reads the Q8_0 copies of one weight set: W_down codes
 * [320][10240] and scales [320][320], W_up codes [10240][320] and scales
 * [10240][10], w_norm float [4][2560].  Host-only, as hcr_create; hcr_read
 * then runs the same read on the decoded weights d * q.  Every pointer must
 * be 16-byte aligned (scratch 256).  Errors as hcr_create. */
int hcr_create_q8_0(const void* down_codes, const void* down_scales, const void* up_codes,
                    const void* up_scales, const float* w_norm, void* scratch, size_t scratch_bytes,
                    hcr_t* out);

/* Skinny BF16 matrix-vector product, the second workload of the pages' decode
 * window (Strata PR #2221, first comment: the attn_q projection, 2,560 inputs to
 * 12,288 outputs, at one to four columns, cold weights; the pages' Q2_0 format is
 * not defined there, so the weights here are BF16):
 *   y[t][n] = sum_k W[n][k] * x[t][k],   t < T, n < rows, k < cols
 *   w : BF16 [rows][cols] row-major      x : float [T][cols]      y : float [T][rows]
 * Asynchronous on `stream` (one kernel; no allocation, no memset).  FP32
 * accumulation in a fixed order (bitwise reproducible).  rows >= 1, cols a
 * multiple of 8 and at most 3072, T in 0..4 (T = 0 enqueues nothing); w and x
 * finite.  Device pointers the caller owns, 16-byte aligned; y must not overlap
 * w or x.
 * Errors: HCR_EINVAL, HCR_EALIGN, HCR_EALIAS (all before any HIP call), HCR_EHIP. */
int hcr_matvec_bf16(const void* w, int rows, int cols, int T, const float* x, float* y, void* stream);

/* One HC read of T tokens, asynchronous on `stream` (a hipStream_t; NULL is the
 * null stream).  Basis: Strata PR #2812, Summary (the norm, the down projection
 * and its partial reduction in one kernel, the up projection in a second) and
 * What changed (the up kernel's epilogue: pending write, gate, stream mean).
 * Enqueues two kernels and returns; no host synchronisation,
 * allocation or memset, so it can be captured into a HIP graph.
 *   x        [T][4][2560]  read only
 *   pending  [T][4][2560]  or NULL (no pending write)
 *   inj      [T][320]      or NULL (no injection)
 *   out      [T][4][2560]  written; may be exactly x or exactly pending,
 *                          otherwise must not overlap any other buffer
 *   mean     [T][2560]     written; must not overlap any other buffer
 * T = 0 is an empty read: nothing is enqueued.  Reads on one handle share its
 * scratch and must be ordered on one stream; distinct handles are independent.
 * The handle's weights may be BF16 (hcr_create) or Q8_0 copies (hcr_create_q8_0).
 * Errors: HCR_EINVAL, HCR_EALIGN, HCR_EALIAS (all before any HIP call), HCR_EHIP. */
int hcr_read(hcr_t h, int T, const float* x, const float* pending, const float* inj,
             float* out, float* mean, void* stream);

/* The read of hcr_read on BF16 weights, for callers that cannot allocate device
 * memory or keep a scratch buffer per weight set (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): no handle and no
 * caller scratch.  The partial sums, lo and rs live in the library's own device
 * array of hcr_scratch_bytes() bytes, one per GPU, held from the first call on
 * that GPU until the process ends; the first call on a GPU looks its address up
 * (hipGetSymbolAddress), later calls make no allocation, free or memset.
 * Every call on one GPU shares that GPU's array: calls whose kernels overlap in
 * time on one GPU race, so order them (e.g. on one stream).  The read runs on
 * the device of `stream` (the current device for NULL).
 *   w_down, w_up, w_norm : as hcr_create (BF16 weights, device pointers, 16-byte aligned)
 *   T, x, pending, inj, out, mean, stream : as hcr_read
 * T may be 0..HCR_T_MAX (the array holds HCR_T_MAX tokens; larger T is rejected).
 * Results are bitwise those of hcr_read on a handle of the same weights.
 * Errors: HCR_EINVAL (T out of range, a NULL weight, x, out or mean),
 * HCR_EALIGN, HCR_EALIAS (all before any HIP call), HCR_EHIP (the address
 * lookup or a launch failed). */
int hcr_read_static(const void* w_down, const void* w_up, const float* w_norm, int T, const float* x,
                    const float* pending, const float* inj, float* out, float* mean, void* stream);

/* Free the host-side handle (never the caller's device memory).  NULL is a no-op.
 * Basis: Strata PR #2812, Title (the handle is the read's argument struct; the
 * weights and the scratch stay the caller's). */
void hcr_destroy(hcr_t h);

/* Static text naming an error code.  Basis: Strata PR #2812, What changed
 * (arguments not at the callers' fixed strides fall back to the default read
 * with one line on stderr; this library has one code path, so such a call
 * returns an error code, and this is its line of text). */
const char* hcr_strerror(int rc);

#ifdef __cplusplus
}
#endif

#endif /* HCR_H */
