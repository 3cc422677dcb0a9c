// Compile-time geometry, tiling and scratch layout shared by the kernels and the
// C ABI (the BF16 hyper-connection read, its Q8_0 copies, the skinny matvec).
// Host and device code include it.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "hcr.h"

namespace hcr {

constexpr int S = HCR_STREAMS;     // residual streams
constexpr int D = HCR_STREAM_D;    // values per stream
constexpr int R = HCR_RANK;        // down rows = up K
constexpr int TMAX = HCR_T_MAX;    // tokens per read
constexpr int DD = S * D;          // 10240: down K = up rows

// ---- work-group b runs on XCD b mod XCDS (each XCD has its own L2): the tiles of one XCD are kept
// contiguous, so that the 128-byte lines the work-groups share (rows of partials; pending, out and mean)
// stay in one L2
constexpr int XCDS = 8;
// ---- down kernel: one work-group = one stream (2,560 columns) x 5 rows of W_down, with down_waves(T)
// waves: lane l of wave w owns stream columns [(2048 / W) w + CA l, +CA) and 2048 + (512 / W) w + CB l
// (W = 4: 8 and 2 columns, one wave per SIMD; W = 8: 4 and 1 columns, two waves per SIMD)
constexpr int DOWN_ROWS = 5;
constexpr int DOWN_WGS = S * (R / DOWN_ROWS);  // 256
// down work-group b: stream b mod 4 (XCDs k and k + 4 serve stream k), row group g; XCD k takes row groups
// 0 .. 31 of its stream and XCD k + 4 row groups 32 .. 63
constexpr int down_stream(int b) { return b % S; }
constexpr int down_group(int b) { return ((b % XCDS) / S) * (DOWN_WGS / XCDS) + b / XCDS; }
// Four waves up to 8 tokens, eight from 9 (T = 9..16 share one width, so that a token's result does not
// depend on T within that range).  Measured on MI355X (whole read, one process, alternating, 3 rounds):
// four waves were 0.04-0.15 us faster per read at every T = 1..8 (BF16 mean 7.56 against 7.66 us, Q8_0
// 7.74 against 7.82 us) and 0.2-0.6 us slower at T = 11..16
constexpr int down_waves(int T) { return T <= 8 ? 4 : 8; }
constexpr int down_threads(int T) { return 64 * down_waves(T); }
constexpr int down_ca(int T) { return 32 / down_waves(T); }  // a lane's columns per row: CA at ca, CB at cb
constexpr int down_cb(int T) { return 8 / down_waves(T); }
constexpr bool down_tiles_ok() {
  for (int T = 1; T <= TMAX; ++T) {
    const int w = down_waves(T);
    if ((w != 4 && w != 8) || down_ca(T) * 64 * w != 2048 || down_cb(T) * 64 * w != 512) return false;
  }
  return true;
}
static_assert(down_tiles_ok(), "the down kernel's column runs must tile the stream");
// ---- up kernel: one work-group = 10 columns x 4 streams = 40 rows of W_up, 4 waves of 10 rows;
// a row is reduced by the 32 lanes of a half-wave, lane q owning K [8q, 8q+8) and [256 + 2q, +2)
constexpr int UP_COLS = 10;
constexpr int UP_WGS = D / UP_COLS;                          // 256
// column tile of up work-group b: XCD k = b mod 8 takes tiles 32k .. 32k + 31
constexpr int up_tile(int b) { return (b % XCDS) * (UP_WGS / XCDS) + b / XCDS; }
constexpr int UP_THREADS = 256;
constexpr int UP_ROWS = UP_COLS * S;                         // 40
constexpr int UP_WAVE_ROWS = UP_ROWS / (UP_THREADS / 64);    // 10
constexpr int UP_ITERS = UP_WAVE_ROWS / 2;                   // 5 (two rows per iteration, one per half-wave)
constexpr int UP_MFMA_FROM = 1;  // BF16 up projection on the matrix cores at every T (measured faster at T = 1 too)
// the same for Q8_0 copies from T = 3 (their codes are widened per K step).  Measured on MI355X (bench.py --ab
// --ab-q8, one process, alternating builds, 4 rounds): 0.23 us faster per read at T = 3 than the vector-ALU
// kernel, 0.15 us slower at T = 2
constexpr int UP_MFMA_FROM_Q8 = 3;

// ---- scratch (bytes) ----
constexpr size_t align256(size_t v) { return (v + 255) & ~size_t(255); }
constexpr size_t OFF_PART = 0;                                          // float [S][TMAX][R], rs-scaled
constexpr size_t OFF_LO = align256(OFF_PART + size_t(S) * TMAX * R * 4);  // float [TMAX][R]
constexpr size_t OFF_RS = align256(OFF_LO + size_t(TMAX) * R * 4);             // float [TMAX][S]
constexpr size_t SCRATCH_BYTES = align256(OFF_RS + size_t(TMAX) * S * 4);

static_assert(S == 4 && D == 4 * 512 + 4 * 128 && R % DOWN_ROWS == 0, "down tiling must divide the geometry");
static_assert(XCDS % S == 0 && DOWN_WGS % XCDS == 0 && UP_WGS % XCDS == 0 && XCDS * (DOWN_WGS / XCDS) == DOWN_WGS,
              "work-groups spread evenly over the XCDs");

// the work-group maps, checked at compile time: each tile once, and the tiles of one XCD contiguous
constexpr bool up_tiles_ok() {
  bool seen[UP_WGS] = {};
  for (int b = 0; b < UP_WGS; ++b) {
    const int t = up_tile(b), k = b % XCDS;
    if (t < 0 || t >= UP_WGS || seen[t] || t / (UP_WGS / XCDS) != k) return false;
    seen[t] = true;
  }
  return true;
}
constexpr bool down_groups_ok() {
  bool seen[S][R / DOWN_ROWS] = {};
  for (int b = 0; b < DOWN_WGS; ++b) {
    const int s = down_stream(b), g = down_group(b), k = b % XCDS;
    if (s != k % S || g < 0 || g >= R / DOWN_ROWS || seen[s][g] || g / (DOWN_WGS / XCDS) != k / S) return false;
    seen[s][g] = true;
  }
  return true;
}
static_assert(up_tiles_ok() && down_groups_ok(), "the work-group maps must cover every tile once, per XCD contiguous");
static_assert(R == 32 * 8 + 32 * 2 && D % UP_COLS == 0 && UP_WAVE_ROWS % 2 == 0, "up tiling must divide the geometry");

// ---- weight formats: BF16, or Q8_0 copies (int8 codes + one binary16 scale per 32 weights of a row)
enum : int { FMT_BF16 = 0, FMT_Q8_0 = 1 };

// matrix-core up kernel: one 16-row tile of the 40 rows per wave (3 waves), plus a 4th wave with no tile when it
// takes a round off the lo staging (T * R / 4 items, one per thread and round): from T = 10, and below where it
// saves a round (T = 3, 5, 6, 8, 9).  BF16 (its weights go straight into LDS, so the 4th wave loads none):
// measured 0.17 us faster per read at T = 8 and 0.02-0.03 at T = 3, 5, 6; at T = 4 and 7, where the rounds stay
// the same, 0.15 and 0.22 us slower.  More staging waves, although they take further rounds off, were slower:
// 5 waves at T = 7 / 8 by 0.65 / 0.39 us, 8 waves at T = 6 by 0.63 us.  Q8_0 copies (the 4th wave re-loads the
// third tile's codes): 0.08-0.13 us faster per read at T = 5, 6, 8 and 0.2 us at T = 9 (bench.py --ab --ab-q8,
// one process, alternating builds, 3 rounds)
constexpr int staging_rounds(int T, int threads) { return (T * (R / 4) + threads - 1) / threads; }
constexpr int upm_threads(int T, int /* fmt: the same rule for both formats */) {
  return T >= 10 || staging_rounds(T, 256) < staging_rounds(T, 192) ? 256 : 192;
}
static_assert(upm_threads(3, FMT_BF16) == 256 && upm_threads(4, FMT_BF16) == 192 && upm_threads(7, FMT_BF16) == 192 &&
                  upm_threads(8, FMT_BF16) == 256 && upm_threads(9, FMT_Q8_0) == 256 && upm_threads(4, FMT_Q8_0) == 192,
              "the 4th wave where it saves a staging round");
// BF16 up weights straight into LDS (global_load_lds_dwordx4, whole 128-byte lines) at every T; Q8_0 codes go
// into registers in the matrix-core operand layout.  Measured on MI355X (bench.py --ab, one process, alternating
// builds, 4 rounds, the results bitwise the same), against the operand layout in registers: the LDS path
// 0.08-0.10 us faster per read at T = 10..12, and, once every step's B operand is read ahead of the first weight
// wait, 0.07-0.14 us faster at T = 13..16 as well (slower by 0.08-0.12 there before)
constexpr bool up_weights_lds(int /* T: the same at every T */, int fmt) { return fmt == FMT_BF16; }
constexpr int Q8_BLOCK = 32;
static_assert(D % Q8_BLOCK == 0 && R % Q8_BLOCK == 0 && 256 % Q8_BLOCK == 0 && Q8_BLOCK % down_ca(1) == 0 &&
                  Q8_BLOCK % down_ca(TMAX) == 0 && Q8_BLOCK % 8 == 0,
              "each of a lane's column runs (down: down_ca and down_cb columns; up: 8 and 2) must sit inside one "
              "Q8_0 block");

// Enqueue the two kernels of one read (T in 1..TMAX; arguments already validated).  For
// FMT_BF16 the scale pointers are unused.
int launch_read(int fmt, int T, const void* w_down, const uint16_t* s_down, const void* w_up, const uint16_t* s_up,
                const float* w_norm, void* scratch, const float* x, const float* pending, const float* inj,
                float* out, float* mean, void* stream);

// The device address of the library's own scratch (SCRATCH_BYTES, 256-byte aligned) on the device of
// `stream` (the current device for the null stream), found once per device; HCR_OK or HCR_EHIP.
int static_scratch(void* stream, void** out);

// ---- skinny BF16 matvec: a wave takes one group of MV_ROWS_PER_WAVE rows
constexpr int MV_THREADS = 256;
constexpr int MV_ROWS_PER_WAVE = 4;
constexpr int MV_MAX_WGS = 65536;  // beyond it (rows > 1M) the waves walk the matrix in steps
constexpr int MV_T_MAX = 4;      // columns per call
constexpr int MV_KCH_MAX = 6;    // 16-byte chunks per lane and row: cols <= 64 * 8 * 6 = 3072 (no register spills at T = 4)

// Enqueue y = W x for T columns (arguments already validated: cols % 8 == 0, cols <= 3072, T in 1..4).
int launch_matvec_bf16(const void* w, int rows, int cols, int T, const float* x, float* y, void* stream);

// Enqueue the Q8_0 quantisation of n_blocks 32-weight blocks (arguments already validated).
int launch_quantize_q8_0(const void* w, size_t n_blocks, void* codes, void* scales, void* stream);

}  // namespace hcr
