/*
 * hcr_calib.h -- C ABI of the calibration kernels of the BF16 hyper-connection
 * read (libhcr_calib.so).  Measurement only: nothing here computes the read.
 *
 * The read (include/hcr.h; Strata PR #2812, "sycl: STRATA_GR_FUSED=1, the
 * two-kernel BF16 hyper-connection read (opt-in)", What changed: one kernel for
 * the norm, the down projection and its split-reduction finish, a second for the
 * up projection and the epilogue) costs two dependent launches that each stream
 * one 6.55 MB BF16 matrix.  These kernels give the floor of that structure on
 * the machine at hand, per T:
 *
 *   HCRC_EMPTY  two empty kernels with the grids and work-group sizes of the
 *               read's two launches at T;
 *   HCRC_LOADS  two kernels with the same grids and work-group sizes that issue
 *               exactly the read's global loads at T, in the same order and with
 *               the same cache policy (down: the stream's x for the T tokens,
 *               w_norm, then the work-group's 5 rows of W_down; up: the 4 stream
 *               partials of lo, then the work-group's 40 rows of W_up, for
 *               T = 1..12 straight into LDS as the read loads them), wait for
 *               every loaded value and discard it: no arithmetic, no other LDS
 *               access, no barrier, no store.
 *
 *   HCRC_LOADS_STORE  HCRC_LOADS with one 4-byte store per down work-group,
 *               issued before its loads (into scratch's lo slot): the fixed
 *               cost of a kernel that writes memory at all.
 *
 * The difference between the read and HCRC_LOADS is what the read's arithmetic,
 * reductions, LDS staging, barriers and stores add to its bare memory traffic.
 *
 * hcrc_read_floor: enqueue the pair `kind` for T tokens (1..HCR_T_MAX) on
 * `stream` (a hipStream_t; NULL is the null stream).  The pointers are those of
 * a read (include/hcr.h layouts): w_down and w_up BF16, w_norm float [4][2560],
 * scratch of hcr_scratch_bytes() bytes (its partials are loaded; only
 * HCRC_LOADS_STORE writes, 256 floats into its lo slot), x float [T][4][2560];
 * all device pointers, 16-byte aligned (scratch 256), otherwise only read.
 * HCRC_EMPTY ignores them (they may be NULL).  No allocation, no
 * memset; graph-capturable.
 * Errors: HCR_EINVAL (unknown kind, T out of range, a NULL pointer for
 * HCRC_LOADS), HCR_EALIGN (both before any HIP call), HCR_EHIP.
 */
#ifndef HCR_CALIB_H
#define HCR_CALIB_H

#ifdef __cplusplus
extern "C" {
#endif

enum { HCRC_EMPTY = 0, HCRC_LOADS = 1, HCRC_LOADS_STORE = 2 };

int hcrc_read_floor(int kind, int T, const void* w_down, const void* w_up, const float* w_norm, void* scratch,
                    const float* x, void* stream);

/*
 * hcrc_up_kernel: enqueue one of the library's two up-projection kernels alone,
 * for T tokens (1..HCR_T_MAX), BF16 weights, no pending write or injection, so
 * that the two can be timed against each other at every T (the read dispatches
 * the matrix-core kernel at every T for BF16 weights, the vector-ALU one serves
 * Q8_0 copies at T = 1..3; Strata PR #2812's up kernel is the basis of both,
 * What changed):
 *   HCRC_UP_VALU  hc_up (v_dot2_f32_bf16 on lo split into BF16 high and low parts)
 *   HCRC_UP_MFMA  hc_up_mfma (v_mfma_f32_16x16x32_bf16, the same split)
 * w_up: BF16 [10240][320]; scratch: a handle's scratch (hcr_scratch_bytes()
 * bytes, 256-byte aligned), whose stream partials are read as the up kernel
 * reads them after a down kernel and whose lo slot is written; out float
 * [T][4][2560] and mean float [T][2560] are written.  All device pointers,
 * 16-byte aligned, none overlapping.  The values computed are those of a read
 * whose down kernel left the scratch's partials; the call is for timing.
 * Errors: HCR_EINVAL (unknown kind, T out of range, a NULL pointer), HCR_EALIGN
 * (both before any HIP call), HCR_EHIP.
 */
enum { HCRC_UP_VALU = 0, HCRC_UP_MFMA = 1 };

int hcrc_up_kernel(int kind, int T, const void* w_up, void* scratch, float* out, float* mean, void* stream);

/*
 * hcrc_slab_pair: the load pattern of Strata PR #2812's down kernel (What
 * changed: a work-group of rows over a 1,280-column slab, half a stream, and
 * the last work-group of a row group to arrive finishing the split reduction;
 * Extra Notes: the (2, 80) shape) on MI355X, to price its finish against the
 * read's design.  Down: 256 work-groups of 10 rows x one 1,280-column slab
 * (the 8 slabs of a row group on one XCD, work-group b % 8 = row group % 8),
 * 4 waves, every lane 4 + 1 columns, loading x (T tokens), w_norm and its 10
 * weight rows; up: the read's up grid loading lo only (not 4 stream partials)
 * and its W_up tile.  No arithmetic; loaded values are discarded.
 *   HCRC_SLAB_LOADS   the loads only;
 *   HCRC_SLAB_STORES  + every down work-group stores its 10 T partials and T
 *                     sums of squares;
 *   HCRC_SLAB_FINISH  + the finish: after its stores a work-group increments
 *                     its row group's counter (one agent-scope acquire-release
 *                     atomic, no spinning); the 8th to arrive reads the 8
 *                     slabs' partials and sums of squares, writes lo and
 *                     resets the counter.
 * slab_scratch: HCRC_SLAB_SCRATCH_BYTES bytes, 256-byte aligned, zero-filled
 * before the first call (the counters; the finish leaves them at zero), used
 * by one stream at a time.  w_down, w_up (BF16), w_norm, x: as for
 * hcrc_read_floor.  T in 1..8.  Errors: HCR_EINVAL, HCR_EALIGN (before any HIP
 * call), HCR_EHIP.
 */
enum { HCRC_SLAB_LOADS = 0, HCRC_SLAB_STORES = 1, HCRC_SLAB_FINISH = 2 };
#define HCRC_SLAB_SCRATCH_BYTES (256u * 1024u)

int hcrc_slab_pair(int kind, int T, const void* w_down, const void* w_up, const float* w_norm, void* slab_scratch,
                   const float* x, void* stream);

/*
 * hcrc_slab_read: the whole read in the pages' shape, with its arithmetic
 * (Strata PR #2812, What changed: the down kernel stages x * w_norm unscaled
 * with the slab's sums of squares; the last work-group of a row group to
 * arrive applies rs per stream, writes lo, the injection and rs, and resets
 * the counter; the up kernel reads lo).  Down: the work-groups, lanes and
 * loads of hcrc_slab_pair, each computing its slab's T sums of squares and
 * its 10 rows' unscaled partials (one FP32 FMA chain per row and token over
 * the exactly widened weights, then the wave and the 4 waves in a fixed
 * order), then one agent-scope acquire-release arrival; the 8th arrival of a
 * row group computes rs[t][s] = 1 / sqrt(mean of squares + 1e-6) from the
 * stream's two slabs, lo[t][r] = sum over s of rs * (its two slab partials),
 * plus inj[t][r] when inj is given, writes lo (and, for row group 0, rs) and
 * sets the counter back to zero; nobody waits.  Up: libhcr.so's up kernel
 * (hc_up_mfma's body) reading lo alone instead of 4 stream partials, with the
 * pending write when pending is given, then the gate and the stream mean.
 * Results: out [T][4][2560] and mean [T][2560] as hcr_read's, within the
 * same tolerance of the reference (the sums run in another order, so not
 * bitwise hcr_read's); lo [T][320] and rs [T][4] at HCRC_SLAB_OFF_LO and
 * HCRC_SLAB_OFF_RS bytes into slab_scratch.  Measurement only: it prices the
 * pages' finish on MI355X with the arithmetic in place.
 * slab_scratch: HCRC_SLAB_SCRATCH_BYTES bytes, 256-byte aligned, zero-filled
 * before the first call (each call leaves its counters at zero), used by one
 * stream at a time.  w_down, w_up (BF16), w_norm, x: as for hcrc_read_floor;
 * pending [T][4][2560] and inj [T][320] fp32 may be NULL (off).  Every
 * pointer 16-byte aligned.  T in 1..8.  out must not overlap x, pending or
 * the scratch.  Errors: HCR_EINVAL, HCR_EALIGN (before any HIP call),
 * HCR_EHIP.
 */
#define HCRC_SLAB_OFF_LO 164864u
#define HCRC_SLAB_OFF_RS 185344u
int hcrc_slab_read(int T, const void* w_down, const void* w_up, const float* w_norm, void* slab_scratch,
                   const float* x, const float* pending, const float* inj, float* out, float* mean, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HCR_CALIB_H */
