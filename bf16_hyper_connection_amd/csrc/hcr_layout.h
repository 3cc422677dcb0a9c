// Compile-time geometry, tiling and scratch layout shared by the kernels and the
// C ABI of the BF16 hyper-connection read.  Host and device code include it.
#pragma once

#include <stddef.h>

#include "hcr.h"

namespace hcr {

constexpr int S = HCR_STREAMS;     // residual streams
constexpr int D = HCR_STREAM_D;    // values per stream
constexpr int R = HCR_RANK;        // down rows = up K
constexpr int TMAX = HCR_T_MAX;    // tokens per read
constexpr int DD = S * D;          // 10240: down K = up rows

// ---- down kernel: one work-group = 16 rows (one MFMA row block) x one slab ----
constexpr int SLAB = 1280;                 // columns per slab (half a stream)
constexpr int NSLAB = DD / SLAB;           // 8
constexpr int SLABS_PER_STREAM = D / SLAB; // 2
constexpr int ROWS_WG = 16;
constexpr int NRB = R / ROWS_WG;           // 20 row blocks
constexpr int DOWN_WAVES = 4;
constexpr int DOWN_WAVE_COLS = SLAB / DOWN_WAVES;   // 320 columns per wave
constexpr int DOWN_LANE_COLS = DOWN_WAVE_COLS / 4;  // 80 columns per lane (its row, its k-group)
constexpr int DOWN_CHUNKS = DOWN_LANE_COLS / 8;     // 10 x 16-byte chunks = 10 MFMAs per wave
constexpr int DOWN_WGS = NRB * NSLAB;               // 160

// ---- up kernel: one wave = 4 columns x 4 streams = 16 rows of W_up; 4 waves per work-group ----
constexpr int UP_WAVE_COLS = 4;
constexpr int UP_WAVES = 4;
constexpr int UP_WG_COLS = UP_WAVE_COLS * UP_WAVES;  // 16
constexpr int UP_WGS = D / UP_WG_COLS;               // 160
constexpr int UP_LANE_K = R / 4;                     // 80 K values per lane
constexpr int UP_CHUNKS = UP_LANE_K / 8;             // 10 MFMAs per wave

constexpr int THREADS = 256;

// ---- scratch (bytes) ----
constexpr size_t align256(size_t v) { return (v + 255) & ~size_t(255); }
constexpr size_t OFF_PART = 0;                                     // float [NSLAB][TMAX][R]
constexpr size_t OFF_SSQ = align256(OFF_PART + size_t(NSLAB) * TMAX * R * 4);  // float [NSLAB][TMAX]
constexpr size_t OFF_LO = align256(OFF_SSQ + size_t(NSLAB) * TMAX * 4);        // float [TMAX][R]
constexpr size_t OFF_RS = align256(OFF_LO + size_t(TMAX) * R * 4);             // float [TMAX][S]
constexpr size_t SCRATCH_BYTES = align256(OFF_RS + size_t(TMAX) * S * 4);

static_assert(D % SLAB == 0 && R % ROWS_WG == 0 && D % UP_WG_COLS == 0, "tiling must divide the geometry");
static_assert(DOWN_LANE_COLS % 8 == 0 && UP_LANE_K % 8 == 0, "lanes load whole 16-byte chunks");
static_assert(S == 4 && UP_WAVE_COLS * S == 16, "an up wave's 16 rows are 4 columns of the 4 streams");

// Enqueue the two kernels of one read (T in 1..TMAX; arguments already validated).
int launch_read(int T, const void* w_down, const void* w_up, const float* w_norm, void* scratch,
                const float* x, const float* pending, const float* inj, float* out, float* mean,
                void* stream);

}  // namespace hcr
