// HIP kernels of the BF16 hyper-connection read for gfx950 (MI355X).
//
// The read (Strata PR #2812, two-kernel BF16 hyper-connection read, What
// changed; Strata PR #2070, Turing hyper-connection read kernels) is split in
// two launches that each stream one 6.55 MB BF16 matrix once for all T tokens:
//
//   hc_down<T>: norm statistics + down projection.  A work-group owns 16 rows
//     of W_down and one 1,280-column slab (half a stream).  It stages the T
//     tokens' weighted stream values x*w_norm unscaled in LDS, already split
//     into BF16 high and low parts in MFMA operand order, and the slab's sums
//     of squares; each wave multiplies its 16 x 320 weight tile with
//     v_mfma_f32_16x16x32_bf16, where the 16 MFMA columns are the 8 tokens'
//     high parts and their 8 low parts.  The four waves' tiles are added in a
//     fixed order and the slab partial sums (unscaled) are written to scratch.
//   hc_up<T>: split-reduction finish + up projection + epilogue.  Every
//     work-group first issues its W_up loads, then finishes the down reduction
//     itself from the 8 slab partials (rs per stream from the slab sums of
//     squares, the injection added), which are small and L2-resident, then
//     multiplies 16 W_up rows per wave (4 columns of each of the 4 streams)
//     with lo, split the same way, and applies the epilogue: pending write,
//     sigmoid gate of lo[t][s], stream mean.
//
// Why BF16 high/low operands: the activations are FP32.  Rounding them to
// BF16 once loses ~2^-9 relative, far above the read's 1e-4 tolerance; the
// high part plus the BF16-rounded remainder keep ~2^-17, and BF16 x BF16
// products are exact in the FP32 accumulator.
//
// Why no atomics: the pages finish the split reduction in the last
// work-group to arrive at a counter.  On MI355X an agent-scope arrival
// counter plus the finisher's reads cost several microseconds per launch
// (cross-XCD release/acquire), more than reading the 8 partials again in the
// next launch, whose weight loads are in flight meanwhile.
//
// Determinism: every sum has a fixed order (MFMA accumulation over fixed
// chunks, waves added 0+1+2+3, slabs added per stream in order), so repeated
// calls and graph replays are bitwise identical.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hcr_layout.h"

namespace hcr {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

__device__ __forceinline__ f32x4 mfma16x16x32(const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                 c, 0, 0, 0);
}

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Split 8 FP32 values into BF16 high parts (round to nearest even) and the
// BF16-rounded remainders; returns the packed high (hi) and low (lo) words.
__device__ __forceinline__ void split_hi_lo(const float (&v)[8], uint4& hi, uint4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const f32x2 a = {v[2 * e], v[2 * e + 1]};
    const bf16x2 bh = __builtin_convertvector(a, bf16x2);
    const f32x2 r = a - __builtin_convertvector(bh, f32x2);  // exact
    const bf16x2 bl = __builtin_convertvector(r, bf16x2);
    h[e] = __builtin_bit_cast(uint32_t, bh);
    l[e] = __builtin_bit_cast(uint32_t, bl);
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }

__device__ __forceinline__ f32x4 shfl_xor4(f32x4 v, int m) {
  f32x4 r;
#pragma unroll
  for (int q = 0; q < 4; ++q) r[q] = __shfl_xor(v[q], m, 64);
  return r;
}

// ---------------------------------------------------------------------------
// down: partial sums of one (16-row block, 1,280-column slab) tile
// ---------------------------------------------------------------------------
template <int T>
__global__ __launch_bounds__(THREADS) void hc_down(const uint4* __restrict__ w_down, const float* __restrict__ x,
                                                   const float* __restrict__ w_norm, float* __restrict__ part,
                                                   float* __restrict__ ssq) {
  // Work-group b takes slab b % 8: consecutive work-groups go to consecutive
  // XCDs, so all row blocks of one slab share an XCD's L2 for x and w_norm.
  const int slab = blockIdx.x % NSLAB;
  const int rb = blockIdx.x / NSLAB;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int stream = slab / SLABS_PER_STREAM;
  const int scol0 = (slab % SLABS_PER_STREAM) * SLAB;  // first column of the slab inside its stream

  // Vector-memory loads complete in issue order, so the small loads the staging
  // needs (x, w_norm) are issued first and the weight tile after them: the
  // staging then waits only for its own data while the weights stream in.
  constexpr int ITEMS = T * (SLAB / 8);  // (token, 8-column chunk) staging items
  constexpr int NI = (ITEMS + THREADS - 1) / THREADS;
  f32x4 xv[NI][2], nv[NI][2];
#pragma unroll
  for (int n = 0; n < NI; ++n) {
    const int q = tid + n * THREADS;
    if (q < ITEMS) {
      const int t = q / (SLAB / 8), c8 = q % (SLAB / 8);
      const float* xp = x + ((size_t)t * S + stream) * D + scol0 + 8 * c8;
      const float* np = w_norm + stream * D + scol0 + 8 * c8;
      xv[n][0] = ld4(xp);
      xv[n][1] = ld4(xp + 4);
      nv[n][0] = ld4(np);
      nv[n][1] = ld4(np + 4);
    }
  }

  // 1. the tile's weights: lane (li, lg) holds row 16*rb + li, 80 contiguous columns
  const uint4* wp = w_down + ((size_t)(rb * ROWS_WG + li) * DD + slab * SLAB + wave * DOWN_WAVE_COLS +
                              lg * DOWN_LANE_COLS) / 8;
  uint4 a[DOWN_CHUNKS];
#pragma unroll
  for (int m = 0; m < DOWN_CHUNKS; ++m) a[m] = wp[m];

  // 2. stage x*w_norm (unscaled) as BF16 high/low MFMA operands, and sums of squares
  //    bop[w][m][g][j]: the 16 bytes lane (j, g) of wave w feeds MFMA m
  __shared__ uint4 bop[DOWN_WAVES][DOWN_CHUNKS][4][16];
  __shared__ float ss_part[TMAX][SLAB / 8];
  __shared__ f32x4 ctile[DOWN_WAVES][64];
  // operands of absent tokens (T..7) are zero
  for (int q = tid; q < (TMAX - T) * (SLAB / 8); q += THREADS) {
    const int t = T + q / (SLAB / 8), c8 = q % (SLAB / 8);
    const int w = c8 / (DOWN_CHUNKS * 4), g = (c8 / DOWN_CHUNKS) % 4, m = c8 % DOWN_CHUNKS;
    bop[w][m][g][t] = make_uint4(0, 0, 0, 0);
    bop[w][m][g][t + 8] = make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int n = 0; n < NI; ++n) {
    const int q = tid + n * THREADS;
    if (q < ITEMS) {
      const int t = q / (SLAB / 8), c8 = q % (SLAB / 8);
      const int w = c8 / (DOWN_CHUNKS * 4), g = (c8 / DOWN_CHUNKS) % 4, m = c8 % DOWN_CHUNKS;
      float v[8];
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = xv[n][0][e] * nv[n][0][e];
        v[4 + e] = xv[n][1][e] * nv[n][1][e];
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) ss = __builtin_fmaf(xv[n][h][e], xv[n][h][e], ss);
      uint4 hi, lo;
      split_hi_lo(v, hi, lo);
      bop[w][m][g][t] = hi;
      bop[w][m][g][t + 8] = lo;
      ss_part[t][c8] = ss;
    }
  }
  __syncthreads();

  // 3. 16 rows x 320 columns per wave on the matrix cores
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < DOWN_CHUNKS; ++m) acc = mfma16x16x32(a[m], bop[wave][m][lg][li], acc);
  // lane (li, lg) holds rows 4*lg .. 4*lg+3 of the block for MFMA column li
  ctile[wave][lane] = acc;
  __syncthreads();

  if (wave == 0) {
    // 4. waves added in a fixed order, then high + low parts of each token
    f32x4 c = ((ctile[0][lane] + ctile[1][lane]) + ctile[2][lane]) + ctile[3][lane];
    const f32x4 other = shfl_xor4(c, 8);
    if (li < T) st4(part + ((size_t)slab * TMAX + li) * R + rb * ROWS_WG + 4 * lg, c + other);
  } else if (wave == 1 && rb == 0) {
    // 5. the slab's sum of squares per token (one row block writes it):
    //    lane = 8*t + p sums columns chunks [20p, 20p+20), then p is reduced by a fixed tree
    const int t = lane >> 3, p = lane & 7;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < (SLAB / 8) / 8; ++i) s += ss_part[t][p * ((SLAB / 8) / 8) + i];
    s += __shfl_xor(s, 4, 64);
    s += __shfl_xor(s, 2, 64);
    s += __shfl_xor(s, 1, 64);
    if (p == 0 && t < T) ssq[slab * TMAX + t] = s;
  }
}

// ---------------------------------------------------------------------------
// up: finish the down reduction, up projection, epilogue
// ---------------------------------------------------------------------------
template <int T, bool INJ, bool PEND>
__global__ __launch_bounds__(THREADS) void hc_up(const uint4* __restrict__ w_up, const float* __restrict__ part,
                                                 const float* __restrict__ ssq, const float* __restrict__ inj,
                                                 const float* pending, float* out, float* __restrict__ mean,
                                                 float* __restrict__ lo_out, float* __restrict__ rs_out) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int c0 = blockIdx.x * UP_WG_COLS + wave * UP_WAVE_COLS;  // this wave's 4 columns

  // Vector-memory loads complete in issue order: the small inputs of the
  // prologue and the epilogue (sums of squares, slab partials, injection,
  // pending write) are issued before the weights so that the prologue waits
  // only for them while W_up streams in.
  constexpr int ITEMS = T * (R / 4);  // (token, 4 K values) items of lo
  constexpr int NI = (ITEMS + THREADS - 1) / THREADS;
  float ssv[SLABS_PER_STREAM] = {};
  if (tid < T * S) {
    const int t = tid / S, s = tid % S;
#pragma unroll
    for (int k = 0; k < SLABS_PER_STREAM; ++k) ssv[k] = ssq[(s * SLABS_PER_STREAM + k) * TMAX + t];
  }
  f32x4 pv[NI][NSLAB], iv[NI];
#pragma unroll
  for (int n = 0; n < NI; ++n) {
    const int q = tid + n * THREADS;
    if (q < ITEMS) {
      const int t = q / (R / 4), k = 4 * (q % (R / 4));
#pragma unroll
      for (int sl = 0; sl < NSLAB; ++sl) pv[n][sl] = ld4(part + ((size_t)sl * TMAX + t) * R + k);
      if (INJ) iv[n] = ld4(inj + (size_t)t * R + k);
    }
  }
  const int te = li;  // the epilogue token of this lane
  f32x4 pend = {0.f, 0.f, 0.f, 0.f};
  if (PEND && te < T) pend = ld4(pending + ((size_t)te * S + lg) * D + c0);

  // 1. the wave's 16 W_up rows: row li = stream li/4, column c0 + li%4; lane group lg holds K [80lg, 80lg+80)
  const uint4* wp = w_up + ((size_t)((li >> 2) * D + c0 + (li & 3)) * R + lg * UP_LANE_K) / 8;
  uint4 a[UP_CHUNKS];
#pragma unroll
  for (int m = 0; m < UP_CHUNKS; ++m) a[m] = wp[m];

  __shared__ float rs_sm[TMAX][S];
  __shared__ float lo_sm[TMAX][R];
  __shared__ uint4 bop[UP_CHUNKS][4][16];

  // 2. rs per (token, stream) from the slab sums of squares
  if (tid < T * S) {
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < SLABS_PER_STREAM; ++k) ss += ssv[k];
    rs_sm[tid / S][tid % S] = 1.0f / __builtin_sqrtf(ss * (1.0f / D) + 1e-6f);
  }
  __syncthreads();

  // 3. lo[t][k] = sum_s rs[t][s] * (slab partials of stream s, in order) + inj[t][k]
#pragma unroll
  for (int n = 0; n < NI; ++n) {
    const int q = tid + n * THREADS;
    if (q < ITEMS) {
      const int t = q / (R / 4), k = 4 * (q % (R / 4));
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < S; ++s) {
        f32x4 ps = pv[n][s * SLABS_PER_STREAM];
#pragma unroll
        for (int kk = 1; kk < SLABS_PER_STREAM; ++kk) ps += pv[n][s * SLABS_PER_STREAM + kk];
        v += rs_sm[t][s] * ps;
      }
      if (INJ) v += iv[n];
      *reinterpret_cast<f32x4*>(&lo_sm[t][k]) = v;
    }
  }
  __syncthreads();

  // 4. lo as BF16 high/low MFMA operands: bop[m][g][j] = part j of K [80g + 8m, +8)
  for (int q = tid; q < UP_CHUNKS * 4 * 16; q += THREADS) {
    const int j = q & 15, g = (q >> 4) & 3, m = q >> 6;
    const int t = j & 7;
    uint4 hi = make_uint4(0, 0, 0, 0), lo = hi;
    if (t < T) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = lo_sm[t][g * UP_LANE_K + 8 * m + e];
      split_hi_lo(v, hi, lo);
    }
    const bool high = j < 8;
    bop[m][g][j] = make_uint4(high ? hi.x : lo.x, high ? hi.y : lo.y, high ? hi.z : lo.z, high ? hi.w : lo.w);
  }
  __syncthreads();

  // 5. 16 rows x 320 K on the matrix cores
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < UP_CHUNKS; ++m) acc = mfma16x16x32(a[m], bop[m][lg][li], acc);
  // lane (li, lg): column li (token li%8, high or low part), rows 4lg..4lg+3 = stream lg, columns c0..c0+3
  const f32x4 u = acc + shfl_xor4(acc, 8);

  // 6. epilogue: out = pending + sigmoid(lo[t][s]) * u; mean over the 4 streams in a fixed order
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  if (te < T) {
    const float gate = 1.0f / (1.0f + expf(-lo_sm[te][lg]));
    o = gate * u;
    if (PEND) o += pend;
    st4(out + ((size_t)te * S + lg) * D + c0, o);
  }
  const f32x4 m1 = o + shfl_xor4(o, 16);    // streams (0+1) and (2+3)
  const f32x4 m2 = m1 + shfl_xor4(m1, 32);  // (0+1) + (2+3)
  if (te < T && lg == 0) st4(mean + (size_t)te * D + c0, 0.25f * m2);

  // 7. the read's lo and rs, kept in the scratch for inspection (one work-group)
  if (blockIdx.x == 0) {
    for (int q = tid; q < T * R; q += THREADS) lo_out[q] = lo_sm[q / R][q % R];
    if (tid < T * S) rs_out[tid] = rs_sm[tid / S][tid % S];
  }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
typedef void (*down_fn)(const uint4*, const float*, const float*, float*, float*);
typedef void (*up_fn)(const uint4*, const float*, const float*, const float*, const float*, float*, float*,
                      float*, float*);

static const down_fn kDown[TMAX] = {hc_down<1>, hc_down<2>, hc_down<3>, hc_down<4>,
                                    hc_down<5>, hc_down<6>, hc_down<7>, hc_down<8>};
#define HCR_UP_ROW(T) {{hc_up<T, false, false>, hc_up<T, false, true>}, {hc_up<T, true, false>, hc_up<T, true, true>}}
static const up_fn kUp[TMAX][2][2] = {HCR_UP_ROW(1), HCR_UP_ROW(2), HCR_UP_ROW(3), HCR_UP_ROW(4),
                                      HCR_UP_ROW(5), HCR_UP_ROW(6), HCR_UP_ROW(7), HCR_UP_ROW(8)};
#undef HCR_UP_ROW

int launch_read(int T, const void* w_down, const void* w_up, const float* w_norm, void* scratch,
                const float* x, const float* pending, const float* inj, float* out, float* mean,
                void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* sc = static_cast<char*>(scratch);
  float* part = reinterpret_cast<float*>(sc + OFF_PART);
  float* ssq = reinterpret_cast<float*>(sc + OFF_SSQ);
  float* lo = reinterpret_cast<float*>(sc + OFF_LO);
  float* rs = reinterpret_cast<float*>(sc + OFF_RS);
  (void)hipGetLastError();  // clear a stale error left by unrelated earlier calls
  hipLaunchKernelGGL(kDown[T - 1], dim3(DOWN_WGS), dim3(THREADS), 0, st, static_cast<const uint4*>(w_down), x,
                     w_norm, part, ssq);
  hipLaunchKernelGGL(kUp[T - 1][inj != nullptr][pending != nullptr], dim3(UP_WGS), dim3(THREADS), 0, st, static_cast<const uint4*>(w_up), part, ssq,
                     inj, pending, out, mean, lo, rs);
  return hipGetLastError() == hipSuccess ? HCR_OK : HCR_EHIP;
}

}  // namespace hcr
