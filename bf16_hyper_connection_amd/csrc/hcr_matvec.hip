// Skinny BF16 matrix-vector product for gfx950 (MI355X): y[t][n] = sum_k W[n][k] x[t][k]
// for 1..4 columns t, the decode window's projections (Strata PR #2221, first comment:
// attn_q, 2,560 inputs to 12,288 outputs, one to four columns, cold weights).
//
// The pages give each row four warps on Turing (the exact layout) and then four rows to
// one warp, so that a row's reduction is one warp reduction.  On a wave64 machine the
// same idea becomes: a wave takes a group of 4 rows, lane l owns the 16-byte chunks
// l, l + 64, ... of every row (one coalesced 1 KB load per chunk index), multiplies
// them by the x values of the same columns, which the work-group stages once in LDS in
// each lane's chunk order as BF16 high and low parts (v_dot2_f32_bf16 on the weights'
// BF16 pairs as loaded: no widening; the two parts keep ~2^-17 of each x value), and the
// 4 x T per-lane sums are added over the wave in one multi-value reduction
// (v_permlane32/16_swap halving, then DPP inside rows of 16).
//
// One row group per wave, many waves per CU: on MI355X a streaming kernel reaches HBM
// bandwidth only with many resident waves each holding a few loads in flight (measured: a
// plain 63 MB read ran at 3.4 TB/s with 4 waves per CU and 5.2 TB/s with 16 or more), so
// the kernel keeps its registers low (x is staged once per work-group in LDS) and lets the
// hardware overlap one wave's arithmetic with the others' loads.  Weights are read exactly
// once.  Every sum has a fixed order.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hcr_device.h"
#include "hcr_layout.h"

namespace hcr {

// the rows of group g: the lane's chunks lane + 64 j.  The loads are unconditional (no branch):
// rows past the matrix read its last row (their results are not stored), and chunks past a row
// read the row's last chunk, whose x values are zeros in LDS (the weights being finite, those
// products add exact zeros).
template <int KCH>
__device__ __forceinline__ void load_group(const uint4* __restrict__ w, int rows, int chunks, int g, int lane,
                                           uint4 (&wv)[MV_ROWS_PER_WAVE][KCH]) {
#pragma unroll
  for (int j = 0; j < KCH; ++j) {  // chunk by chunk, the order the products use them
    const int c = min(lane + 64 * j, chunks - 1);
#pragma unroll
    for (int r = 0; r < MV_ROWS_PER_WAVE; ++r) {
      const int row = min(g * MV_ROWS_PER_WAVE + r, rows - 1);
      wv[r][j] = ldw16(w + (size_t)row * chunks + c);
    }
  }
}

// the group's rows x T tokens: per chunk, the 4 BF16 weight pairs times the x values' BF16 high parts, then
// times their low parts (v_dot2_f32_bf16, one chain per row and token; x from LDS, chunk by chunk), the wave
// sum, and the stores of y
template <int T, int KCH, int XPAD>
__device__ __forceinline__ void group_result(const uint4 (&wv)[MV_ROWS_PER_WAVE][KCH], const uint4 (*xs)[XPAD],
                                             int rows, int g, int lane, float* __restrict__ y) {
  constexpr int N = round4(MV_ROWS_PER_WAVE * T);  // zeros pad the values to a multiple of 4
  float v[N];
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = 0.f;
#pragma unroll
  for (int j = 0; j < KCH; ++j) {
    uint4 xh[T], xl[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      xh[t] = xs[0][(t * KCH + j) * 64 + lane];
      xl[t] = xs[1][(t * KCH + j) * 64 + lane];
    }
#pragma unroll
    for (int r = 0; r < MV_ROWS_PER_WAVE; ++r) {
      const uint32_t u[4] = {wv[r][j].x, wv[r][j].y, wv[r][j].z, wv[r][j].w};
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const uint32_t hh[4] = {xh[t].x, xh[t].y, xh[t].z, xh[t].w};
        const uint32_t ll[4] = {xl[t].x, xl[t].y, xl[t].z, xl[t].w};
        float acc = v[r * T + t];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, u[e]), __builtin_bit_cast(bf16x2v, hh[e]), acc, false);
          acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, u[e]), __builtin_bit_cast(bf16x2v, ll[e]), acc, false);
        }
        v[r * T + t] = acc;
      }
    }
    // one chunk's x values live at a time (the scheduler would otherwise load all chunks' x values
    // up front and hold them, which at T = 4 costs a wave of occupancy)
    __builtin_amdgcn_sched_barrier(0);
  }
  // value k = r * T + t (row r of the group, token t); after the sum, the lanes of row q (of 16)
  // hold values q * N/4 + i, i < N/4, in v[i]
  wave_sum<N>(v);
  const int q = lane >> 4, i = lane & 15;
  const int k = q * (N / 4) + i;
  const int row = g * MV_ROWS_PER_WAVE + k / T;
  float out = v[0];
#pragma unroll
  for (int m = 1; m < N / 4; ++m) out = i == m ? v[m] : out;
  if (i < N / 4 && k < MV_ROWS_PER_WAVE * T && row < rows) y[(size_t)(k % T) * rows + row] = out;
}

template <int T, int KCH>
__global__ __launch_bounds__(MV_THREADS) void mv_bf16(const uint4* __restrict__ w, int rows, int chunks,
                                                      const float* __restrict__ x, float* __restrict__ y) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int gw = blockIdx.x * (MV_THREADS / 64) + wave;
  const int nw = gridDim.x * (MV_THREADS / 64);
  const int groups = (rows + MV_ROWS_PER_WAVE - 1) / MV_ROWS_PER_WAVE;
  const int cols = chunks * 8;

  // x once per work-group into LDS, in each lane's chunk order: entry e = (t * KCH + j) * 64 + l of
  // xs[0] (xs[1]) holds the BF16 high (low) parts of x[t] at columns 8(l + 64 j) .. +8 (zeros past the
  // row), so lane l of every wave reads 16 consecutive bytes.  A thread issues its x loads first, then the wave's weight loads,
  // and writes LDS once the x loads (the older ones) are back; the LDS array is padded to whole
  // passes of the work-group so that no write needs a branch.
  constexpr int XS = T * KCH * 64;
  constexpr int XIT = (XS + MV_THREADS - 1) / MV_THREADS;
  __shared__ uint4 xs[2][XIT * MV_THREADS];  // BF16 high parts, low parts
  f32x4 xl[XIT][2];
  bool xin[XIT];
#pragma unroll
  for (int it = 0; it < XIT; ++it) {
    const int e = threadIdx.x + it * MV_THREADS;
    const int t = min(e / (KCH * 64), T - 1), j = (e / 64) % KCH, l = e % 64;
    xin[it] = e < XS && l + 64 * j < chunks;
    const int c = min(l + 64 * j, chunks - 1);
    xl[it][0] = ld4(x + (size_t)t * cols + 8 * c);
    xl[it][1] = ld4(x + (size_t)t * cols + 8 * c + 4);
  }

  // the wave's first row group.  A wave past the last group takes the last group again: the same
  // rows, the same results, stored again to the same addresses (no branch here, so that the
  // compiler keeps these loads ahead of the LDS staging instead of sinking them to their use).
  uint4 wv[MV_ROWS_PER_WAVE][KCH];
  int g = gw < groups ? gw : groups - 1;
  __builtin_amdgcn_sched_barrier(0);  // x loads first, then the weights, then the LDS writes
  load_group<KCH>(w, rows, chunks, g, lane, wv);
  __builtin_amdgcn_sched_barrier(0);

  // (x finite: multiplying by 0 or 1 keeps every load's value in use, so none is made conditional)
#pragma unroll
  for (int it = 0; it < XIT; ++it) {
    const float keep = xin[it] ? 1.f : 0.f;
    float v8[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v8[e] = xl[it][0][e] * keep;
      v8[4 + e] = xl[it][1][e] * keep;
    }
    uint4 hi, lo;
    split_hi_lo(v8, hi, lo);
    xs[0][threadIdx.x + it * MV_THREADS] = hi;
    xs[1][threadIdx.x + it * MV_THREADS] = lo;
  }
  __syncthreads();

  // one row group per wave; a grid smaller than the matrix (very tall matrices) walks it in steps
  while (true) {
    group_result<T, KCH, XIT * MV_THREADS>(wv, xs, rows, g, lane, y);
    if (gw >= groups) break;
    g += nw;
    if (g >= groups) break;
    load_group<KCH>(w, rows, chunks, g, lane, wv);
  }
}

typedef void (*mv_fn)(const uint4*, int, int, const float*, float*);
#define HCR_MV_ROW(T) {mv_bf16<T, 1>, mv_bf16<T, 2>, mv_bf16<T, 3>, mv_bf16<T, 4>, mv_bf16<T, 5>, mv_bf16<T, 6>}
static_assert(MV_KCH_MAX == 6 && MV_T_MAX == 4, "the table below lists every instantiation");
static const mv_fn kMv[MV_T_MAX][MV_KCH_MAX] = {HCR_MV_ROW(1), HCR_MV_ROW(2), HCR_MV_ROW(3), HCR_MV_ROW(4)};
#undef HCR_MV_ROW

int launch_matvec_bf16(const void* w, int rows, int cols, int T, const float* x, float* y, void* stream) {
  const int chunks = cols / 8;
  const int kch = (chunks + 63) / 64;
  const int groups = (rows + MV_ROWS_PER_WAVE - 1) / MV_ROWS_PER_WAVE;
  const int waves_per_wg = MV_THREADS / 64;
  int wgs = (groups + waves_per_wg - 1) / waves_per_wg;
  if (wgs > MV_MAX_WGS) wgs = MV_MAX_WGS;
  (void)hipGetLastError();
  hipLaunchKernelGGL(kMv[T - 1][kch - 1], dim3(wgs), dim3(MV_THREADS), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(w), rows, chunks, x, y);
  return hipGetLastError() == hipSuccess ? HCR_OK : HCR_EHIP;
}

}  // namespace hcr
