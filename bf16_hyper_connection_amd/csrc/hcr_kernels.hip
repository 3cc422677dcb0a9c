// HIP kernels of the BF16 hyper-connection read for gfx950 (MI355X), and of
// its sibling on Q8_0 copies of the two projections.
//
// The read (Strata PR #2812, two-kernel BF16 hyper-connection read, What
// changed; Strata PR #2070, Turing hyper-connection read kernels) is split in
// two launches that each stream one 6.55 MB BF16 matrix once for all T tokens:
//
//   hc_down<T>: norm statistics + down projection + split-reduction finish.
//     A work-group owns one whole stream (2,560 columns) of 5 W_down rows, so
//     it can apply rs itself: 4 waves up to 8 tokens, every lane owning 10
//     columns (a 16-byte and a 4-byte piece of each row), and 8 waves from 9
//     tokens (two per SIMD, so that one wave's arithmetic overlaps the other's
//     waits), every lane owning 5 columns (an 8-byte and a 2-byte piece), all
//     pieces coalesced across the wave;
//     the lane computes x*w_norm and the sums of squares of its columns for
//     the T tokens, and one FP32 FMA chain per (row, token) over the exactly
//     widened BF16 weights.  The 6T per-lane values are summed over the wave
//     (halving with v_permlane32/16_swap, then DPP; each group of four values
//     as soon as its row is done) and over the waves (LDS, fixed order); the
//     work-group writes rs[t][s] * (row sums), one partial per stream.
//   hc_up_mfma<T, INJ, PEND> (BF16 weights from T = 2, Q8_0 copies from T = 4):
//     lo[t][k] = the 4 stream
//     partials (+ injection), then 40 rows of W_up (10 columns x 4 streams) per
//     work-group as three 16-row tiles on the matrix cores
//     (v_mfma_f32_16x16x32_bf16), lo split into BF16 high and low parts as the
//     B operand.  Up to 8 tokens the high parts fill B columns 0..7 and the low
//     parts columns 8..15, one product per K step; from 9 tokens each part has
//     its own product.  Epilogue in the lane: pending write, sigmoid gate of
//     lo[t][s], stream mean.
//   hc_up<T, INJ, PEND>: the same tile on the vector ALUs (BF16 at T = 1,
//     Q8_0 at T = 1..3).  Each row is reduced by the 32 lanes of a half-wave;
//     lane q owns K [8q, 8q+8) and [256+2q, +2) and multiplies with
//     v_dot2_f32_bf16 against the high and low parts of lo.  Epilogue: pending
//     write, sigmoid gate, stream mean of 4 adjacent outputs (DPP quad).
//
// Why the high/low split of lo: the activations are FP32.  Rounding lo to
// BF16 once loses ~2^-9 relative, above the read's 1e-4 tolerance; the high
// part plus the BF16-rounded remainder keep ~2^-17.  The down projection uses
// FMA on widened weights instead: its activations change every row group, and
// the split would cost more VALU than the widening.
//
// Why the matrix cores for the up projection from T = 2: the v_dot2 kernel
// issues ~100 VALU instructions per token per wave, which the loads cannot
// hide with one wave per SIMD; the matrix-core kernel's 10 or 20 MFMAs per
// wave cost the same at every T.  Measured on MI355X, whole read: T = 1
// 6.45 us (v_dot2) against 6.82 (matrix cores); when the matrix-core kernel
// was introduced, T = 2 7.60 against 7.56 and T = 8 10.42 against 9.28.
//
// T = 10..16: the down kernel takes the tokens in groups of 8 (the next
// group's x loads overlap the current group's FMAs); up to 9 in one group.  A token's result is the
// same bit for bit at every T of one range: T = 2..8 and T = 9..16 (the two
// B layouts round differently); a token read alone (T = 1, v_dot2) rounds
// differently again.
//
// Why no atomics: the pages finish the split reduction in the last
// work-group to arrive at a counter.  On MI355X an agent-scope arrival
// counter plus the finisher's reads cost several microseconds per launch
// (cross-XCD release/acquire).  Here the down work-group covers a whole
// stream, and the up kernel adds the 4 stream partials itself while its
// weight loads are in flight.
//
// Loads: vector-memory loads complete in issue order, so every kernel issues
// its small inputs first (x, w_norm; partials, injection, pending) and its
// weight tile after them, all before any arithmetic; the weights go in the
// order the arithmetic uses them (row by row in hc_down, K step by K step in
// hc_up_mfma), and arithmetic that needs only the small inputs is kept ahead
// of every use of the weights, so that it runs while they are in flight.
//
// Work-group b runs on XCD b mod 8, each XCD with its own L2: the tiles of one
// XCD are contiguous (up_tile, down_group), so that the 128-byte lines that
// neighbouring tiles share (partials; pending, out and mean) stay in one L2.
//
// Q8_0 copies (Strata PR #2812, Summary: the sibling read of #2810 on Q8_0
// copies of the projections; the block is read as GGML's Q8_0: 32 weights of
// a row share one binary16 scale d, each weight is d times an int8 code).
// The same two kernels, templated on the weight format, read int8 codes (half
// the bytes of BF16) and two scales per lane and row; each of a lane's two
// column runs sits inside one block, so the lane multiplies each run's FMA sum
// by its block's scale (the down kernel from 4 tokens: the codes times their
// scale first, exact in FP32, once per row).
// The vector-ALU up kernel takes lo in FP32 from LDS (no BF16 split): the
// codes widen exactly to FP32; the matrix-core one widens them exactly to BF16
// and scales each block's product.  q8_quantize makes the copies on the device: 4 lanes per
// block, the block maximum over the quad by DPP, then d = amax / 127,
// codes = round(w * (1 / d)) with ties away from zero, all in IEEE binary32,
// and d stored rounded to binary16.
//
// Determinism: every sum has a fixed order, so repeated calls and graph
// replays are bitwise identical, and each token's result does not depend on T
// within T = 2..8 or within T = 9..16 (BF16), or within T = 1..3, 4..8 or
// 9..16 (Q8_0).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "hcr_device.h"
#include "hcr_layout.h"

namespace hcr {

// down: one stream x 5 rows per work-group; rs applied here (the work-group sees the whole stream)
// x (or w_norm) values of a lane's two column runs: CA columns at ca and CB at cb
template <int CA, int CB>
struct Cols {
  float a[CA], b[CB];
  __device__ __forceinline__ void load(const float* p, int ca, int cb) {
#pragma unroll
    for (int e = 0; e < CA; e += 4) {
      const f32x4 v = ld4(p + ca + e);
      a[e] = v[0], a[e + 1] = v[1], a[e + 2] = v[2], a[e + 3] = v[3];
    }
    if constexpr (CB == 2) {
      const f32x2 v = ld2(p + cb);
      b[0] = v[0], b[1] = v[1];
    } else {
      b[0] = p[cb];
    }
  }
};

template <int T, int FMT>
__global__ __launch_bounds__(down_threads(T)) void hc_down(const void* __restrict__ w_down,
                                                           const uint16_t* __restrict__ s_down,
                                                           const float* __restrict__ x,
                                                           const float* __restrict__ w_norm,
                                                           float* __restrict__ part, float* __restrict__ rs_out) {
  // consecutive work-groups take consecutive streams: the XCD of work-group b (b mod 8) sees one stream, and
  // half of its row groups, contiguous
  const int s = down_stream(blockIdx.x);
  const int g = down_group(blockIdx.x);  // rows DOWN_ROWS*g ..
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  constexpr int WAVES = down_waves(T), CA = down_ca(T), CB = down_cb(T), NC = CA + CB;
  const int ca = (2048 / WAVES) * wave + CA * lane;        // CA columns: one 2*CA-byte chunk per row
  const int cb = 2048 + (512 / WAVES) * wave + CB * lane;  // CB columns

  // Up to 9 tokens are taken in one group (every x load issued up front); from 10 tokens in groups of 8 (x of
  // one group in registers at a time, the next group's loads under this group's FMAs).  Measured on MI355X
  // (whole read, one process, alternating): groups of 8 are 0.08 / 0.04 / 0 / 0.22 us faster than one group
  // at T = 10 / 11 / 12 / 13 for BF16 weights, and up to 0.15 us for the Q8_0 copies.
  constexpr int TG = T <= 9 ? T : 8;
  constexpr int NG = (T + TG - 1) / TG;
  Cols<CA, CB> xv[TG];
  auto load_x = [&](int grp) {
#pragma unroll
    for (int i = 0; i < TG; ++i) {
      const int t = grp * TG + i;
      if (t < T) xv[i].load(x + ((size_t)t * S + s) * D, ca, cb);
    }
  };

  // 1. x of the first group and w_norm first (vector loads complete in issue order), then the 5 weight rows
  load_x(0);
  Cols<CA, CB> nv;
  nv.load(w_norm + s * D, ca, cb);
  uint32_t wa[DOWN_ROWS][CA / 2];  // BF16: CA weights at ca (packed pairs); Q8_0: CA codes (packed quads)
  uint32_t wb[DOWN_ROWS];          // BF16 / Q8_0: the CB weights or codes at cb
  uint32_t sa[DOWN_ROWS], sb[DOWN_ROWS];  // Q8_0: scales of the blocks holding ca and cb
  if constexpr (FMT == FMT_BF16) {
    const uint16_t* wr = static_cast<const uint16_t*>(w_down) + (size_t)(DOWN_ROWS * g) * DD + (size_t)s * D;
#pragma unroll
    for (int r = 0; r < DOWN_ROWS; ++r) {
      if constexpr (CA == 8) {
        const uint4 v = ldw16(wr + (size_t)r * DD + ca);
        wa[r][0] = v.x, wa[r][1] = v.y, wa[r][2] = v.z, wa[r][3] = v.w;
      } else {
        const uint2 v = ldw8(wr + (size_t)r * DD + ca);
        wa[r][0] = v.x, wa[r][1] = v.y;
      }
      if constexpr (CB == 2)
        wb[r] = ldw4(wr + (size_t)r * DD + cb);
      else
        wb[r] = ldw2(wr + (size_t)r * DD + cb);  // widened at its use: a shift here would wait for the load
      __builtin_amdgcn_sched_barrier(0);  // rows in order: row r's loads complete before row r + 1's
    }
  } else {
    const int8_t* wr = static_cast<const int8_t*>(w_down) + (size_t)(DOWN_ROWS * g) * DD + (size_t)s * D;
    const uint16_t* sr = s_down + (size_t)(DOWN_ROWS * g) * (DD / Q8_BLOCK) + (size_t)s * (D / Q8_BLOCK);
#pragma unroll
    for (int r = 0; r < DOWN_ROWS; ++r) {
      if constexpr (CA == 8) {
        const uint2 v = ldw8(wr + (size_t)r * DD + ca);
        wa[r][0] = v.x, wa[r][1] = v.y;
      } else {
        wa[r][0] = ldw4(wr + (size_t)r * DD + ca);
      }
      if constexpr (CB == 2)
        wb[r] = ldw2(wr + (size_t)r * DD + cb);
      else
        wb[r] = ldw1(wr + (size_t)r * DD + cb);
      sa[r] = ldw2(sr + (size_t)r * (DD / Q8_BLOCK) + ca / Q8_BLOCK);
      sb[r] = ldw2(sr + (size_t)r * (DD / Q8_BLOCK) + cb / Q8_BLOCK);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // The lane's 6T values, in the order they become known: the T sums of squares (value t), then the rows
  // (value (r + 1) T + t), then padding; value k sits at quad_pos(k, N), so that the wave reduction of each
  // quadruple can start as soon as its four values are known (with one token group: the sums of squares
  // under the weight loads, each row's quadruples while the next rows' weights arrive)
  constexpr int N = round4((DOWN_ROWS + 1) * T);
  constexpr bool EARLY = NG == 1;
  // quadruples whose values are all known once the sums of squares (c = 0) and rows 0 .. c - 1 are
  constexpr auto quads_known = [](int c) { return c >= DOWN_ROWS ? N / 4 : ((c + 1) * T) / 4; };
  float v[N];
#pragma unroll
  for (int k = (DOWN_ROWS + 1) * T; k < N; ++k) v[quad_pos(k, N)] = 0.f;
#pragma unroll
  for (int grp = 0; grp < NG; ++grp) {
    // 2. activations x*w_norm (unscaled) and the lane's sums of squares of this group's tokens
    float act[TG][NC];
#pragma unroll
    for (int i = 0; i < TG; ++i) {
      const int t = grp * TG + i;
      if (t < T) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < CA; ++e) act[i][e] = xv[i].a[e] * nv.a[e];
#pragma unroll
        for (int e = 0; e < CB; ++e) act[i][CA + e] = xv[i].b[e] * nv.b[e];
#pragma unroll
        for (int e = 0; e < CA; ++e) ss = __builtin_fmaf(xv[i].a[e], xv[i].a[e], ss);
#pragma unroll
        for (int e = 0; e < CB; ++e) ss = __builtin_fmaf(xv[i].b[e], xv[i].b[e], ss);
        v[quad_pos(t, N)] = ss;
      }
    }
    if constexpr (EARLY) {
#pragma unroll
      for (int q = 0; q < quads_known(0); ++q) wave_quad_sum<N>(v, q);
    }
    // the next group's x streams in while this group computes.  The activations and sums of squares need
    // only x and w_norm: kept ahead of every use of the weights, so that they run while the weight loads are
    // in flight (the compiler would otherwise widen the 2-byte weight loads first, and so wait for them)
    if (grp + 1 < NG) load_x(grp + 1);
    __builtin_amdgcn_sched_barrier(0);
    // 3. per row: the weights widened exactly to FP32, one FMA chain per token.  Q8_0: below 4 tokens one
    //    chain per block chunk, each times its block's scale; from 4 tokens the codes are first decoded to
    //    d * q (exact in FP32: 11 + 7 significant bits), once per row, and then take the BF16 path's chain
    constexpr bool DECODE = FMT == FMT_Q8_0 && T >= 4;
#pragma unroll
    for (int r = 0; r < DOWN_ROWS; ++r) {
      float wv[NC];
      if constexpr (FMT == FMT_BF16) {
#pragma unroll
        for (int e = 0; e < CA / 2; ++e) {
          wv[2 * e] = __uint_as_float(wa[r][e] << 16);
          wv[2 * e + 1] = __uint_as_float(wa[r][e] & 0xffff0000u);
        }
        if constexpr (CB == 2) {
          wv[CA] = __uint_as_float(wb[r] << 16);
          wv[CA + 1] = __uint_as_float(wb[r] & 0xffff0000u);
        } else {
          wv[CA] = __uint_as_float(wb[r] << 16);
        }
      } else {
#pragma unroll
        for (int e = 0; e < CA; ++e) wv[e] = code(wa[r][e / 4], e % 4);
#pragma unroll
        for (int e = 0; e < CB; ++e) wv[CA + e] = code(wb[r], e);
        if constexpr (DECODE) {
          const float da = half_bits_to_float(sa[r]), db = half_bits_to_float(sb[r]);
#pragma unroll
          for (int e = 0; e < CA; ++e) wv[e] *= da;
#pragma unroll
          for (int e = 0; e < CB; ++e) wv[CA + e] *= db;
        }
      }
#pragma unroll
      for (int i = 0; i < TG; ++i) {
        const int t = grp * TG + i;
        if (t < T) {
          if constexpr (FMT == FMT_BF16 || DECODE) {
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < NC; ++e) acc = __builtin_fmaf(wv[e], act[i][e], acc);
            v[quad_pos((r + 1) * T + t, N)] = acc;
          } else {
            float a8 = 0.f;
#pragma unroll
            for (int e = 0; e < CA; ++e) a8 = __builtin_fmaf(wv[e], act[i][e], a8);
            float a2 = wv[CA] * act[i][CA];
#pragma unroll
            for (int e = 1; e < CB; ++e) a2 = __builtin_fmaf(wv[CA + e], act[i][CA + e], a2);
            v[quad_pos((r + 1) * T + t, N)] = __builtin_fmaf(half_bits_to_float(sa[r]), a8, half_bits_to_float(sb[r]) * a2);
          }
        }
      }
      // row by row: without this barrier the compiler merged the waits for several rows' loads (four waves
      // at T = 5..7, eight waves with token groups), so that early rows' FMAs waited for later rows' weights.
      // Measured (one process, alternating, 3 rounds): 0.2-0.3 us faster per read at T = 5..7 with four
      // waves, 0.05-0.16 us at T = 10..15 with eight, level at T = 9 and 16
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (EARLY) {  // 4. sums over the wave of the quadruples this row completes
#pragma unroll
        for (int q = quads_known(r); q < quads_known(r + 1); ++q) wave_quad_sum<N>(v, q);
      }
    }
  }

  // 4. sums over the wave (several token groups: all at the end), then over the waves in a fixed order
  if constexpr (!EARLY) wave_sum<N>(v);
  __shared__ float wsum[WAVES][N];
  if ((lane & 15) == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) wsum[wave][(lane >> 4) * (N / 4) + i] = v[i];
  }
  __syncthreads();

  // 5. rs of this stream per token, and the rs-scaled partial sums of the 5 rows: thread (r, t) adds its
  //    value and its token's sum of squares over the waves itself (no second barrier)
  if (tid < DOWN_ROWS * T) {
    const int r = tid / T, t = tid % T;
    const int pr = quad_pos((r + 1) * T + t, N), pq = quad_pos(t, N);
    float a = wsum[0][pr], q = wsum[0][pq];
#pragma unroll
    for (int k = 1; k < WAVES; ++k) {
      a += wsum[k][pr];
      q += wsum[k][pq];
    }
    // rs by the hardware reciprocal square root (within 1 ulp; the argument is at least 1e-6, never
    // subnormal): shorter than a rounded square root and division at the end of the kernel.  The partials
    // are stored coherent at device scope (sc1): the up kernel reads them from the other XCDs' work-groups.
    // Measured on MI355X (cold read, one process, alternating, 3 rounds): 0.07 us (rsq) and 0.09 us (sc1
    // stores) less per read on the mean over T = 1..8
    const float rs = __builtin_amdgcn_rsqf(q * (1.0f / D) + 1e-6f);
    __hip_atomic_store(&part[((size_t)s * TMAX + t) * R + DOWN_ROWS * g + r], rs * a, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    if (g == 0 && r == 0) __hip_atomic_store(&rs_out[t * S + s], rs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}


// The up kernels' first loads: the 4 stream partials (and the injection) of lo, 4 K values of one token
// per item, items tid + n * NT (NT threads).  Neither the loads nor the stores of lo are conditional: items
// past the end load the last item again (store_lo puts those repeats in junk slots).  A branch among the loads
// makes the compiler wait for every load issued so far, and a branch around their only use lets it sink
// them below the weight loads; either would serialise them with the weight stream.
template <int T, bool INJ, int NI, int NT>
__device__ __forceinline__ void load_partials(int tid, const float* __restrict__ part,
                                              const float* __restrict__ inj, f32x4 (&pv)[NI][S],
                                              f32x4 (&iv)[NI]) {
  constexpr int ITEMS = T * (R / 4);
#pragma unroll
  for (int n = 0; n < NI; ++n) {
    const int it = min(tid + n * NT, ITEMS - 1);
    const int t = it / (R / 4), k = 4 * (it % (R / 4));
#pragma unroll
    for (int ss = 0; ss < S; ++ss) pv[n][ss] = ld4(part + ((size_t)ss * TMAX + t) * R + k);
    if (INJ) iv[n] = ld4(inj + (size_t)t * R + k);
  }
}

// lo[t][k] = ((p0 + p1) + p2) + p3 (+ inj) into LDS, for the items load_partials loaded.  lo_sm holds
// T * R + LO_JUNK floats: a lane past the last item stores its repeat into its own slot after lo (the
// address is selected, not branched on), so that no two lanes of a wave write one LDS address.
constexpr int LO_JUNK = 64 * 4;
template <int T, bool INJ, int NI, int NT>
__device__ __forceinline__ void store_lo(int tid, const f32x4 (&pv)[NI][S], const f32x4 (&iv)[NI],
                                         float* lo_sm) {
  constexpr int ITEMS = T * (R / 4);
#pragma unroll
  for (int n = 0; n < NI; ++n) {
    const int it = min(tid + n * NT, ITEMS - 1);
    const int t = it / (R / 4), k = 4 * (it % (R / 4));
    f32x4 vv = ((pv[n][0] + pv[n][1]) + pv[n][2]) + pv[n][3];
    if (INJ) vv += iv[n];
    const int at = tid + n * NT < ITEMS ? t * R + k : T * R + 4 * (tid & 63);
    *reinterpret_cast<f32x4*>(lo_sm + at) = vv;
  }
}

// up on the vector ALUs (BF16 at T = 1, Q8_0 at T = 1..3): lo = sum of the 4 stream partials (+ injection);
// 40 rows of W_up (10 columns x 4 streams) per work-group
template <int T, bool INJ, bool PEND, int FMT>
__global__ __launch_bounds__(UP_THREADS) void hc_up(const void* __restrict__ w_up,
                                                         const uint16_t* __restrict__ s_up,
                                                         const float* __restrict__ part,
                                                         const float* __restrict__ inj, const float* pending,
                                                         float* out, float* __restrict__ mean,
                                                         float* __restrict__ lo_out) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, q = lane & 31;  // half-wave (row of the iteration), K lane
  const int c0 = up_tile(blockIdx.x) * UP_COLS;  // an XCD's tiles are contiguous

  // 1. small loads first (vector loads complete in issue order): stream partials and injection
  //    for lo, pending for the epilogue
  constexpr int ITEMS = T * (R / 4);  // (token, 4 K values)
  constexpr int NI = (ITEMS + UP_THREADS - 1) / UP_THREADS;
  f32x4 pv[NI][S], iv[NI];
  load_partials<T, INJ, NI, UP_THREADS>(tid, part, inj, pv, iv);
  // epilogue: output o = (t * UP_COLS + cc) * 4 + s, the 4 streams of a column in an aligned quad of lanes
  constexpr int NO = (T * UP_ROWS + UP_THREADS - 1) / UP_THREADS;
  float pend[NO];
#pragma unroll
  for (int n = 0; n < NO; ++n) {
    const int o = min(tid + n * UP_THREADS, T * UP_ROWS - 1);  // clamped: no branch among the loads
    const int t = o / UP_ROWS, cc = (o / S) % UP_COLS, s = o % S;
    pend[n] = PEND ? pending[((size_t)t * S + s) * D + c0 + cc] : 0.f;
  }
  __builtin_amdgcn_sched_barrier(0);  // keeps every small load ahead of the weight loads

  // 2. weights: iteration m, half h -> row rw = 10*wave + 2m + h (column rw >> 2, stream rw & 3);
  //    lane q owns K [8q, 8q+8) (one 16-byte chunk) and [256 + 2q, 256 + 2q + 2) (one dword)
  uint4 wa[UP_ITERS];     // BF16: K [8q, 8q+8)
  uint32_t wb[UP_ITERS];  // BF16: K [256+2q, +2); Q8_0: the 2 codes there
  uint2 qa[UP_ITERS];     // Q8_0: codes at K [8q, 8q+8)
  uint32_t sa[UP_ITERS], sb[UP_ITERS];  // Q8_0: scales of blocks q/4 and 8 + q/16 of the row
#pragma unroll
  for (int m = 0; m < UP_ITERS; ++m) {
    const int rw = UP_WAVE_ROWS * wave + 2 * m + h;
    const size_t j = (size_t)(rw & 3) * D + c0 + (rw >> 2);
    if constexpr (FMT == FMT_BF16) {
      const uint16_t* row = static_cast<const uint16_t*>(w_up) + j * R;
      wa[m] = ldw16(row + 8 * q);
      wb[m] = ldw4(row + 256 + 2 * q);
    } else {
      const int8_t* row = static_cast<const int8_t*>(w_up) + j * R;
      qa[m] = ldw8(row + 8 * q);
      wb[m] = ldw2(row + 256 + 2 * q);
      sa[m] = ldw2(s_up + j * (R / Q8_BLOCK) + q / 4);
      sb[m] = ldw2(s_up + j * (R / Q8_BLOCK) + 8 + q / 16);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  __shared__ __attribute__((aligned(16))) float lo_sm[T * R + LO_JUNK];
  constexpr int TS = FMT == FMT_BF16 ? T : 1;  // the BF16 split of lo; Q8_0 reads lo itself
  __shared__ uint4 acta_sm[2][TS][32];  // K [8q, 8q+8): high, low parts
  __shared__ uint2 actb_sm[TS][32];     // K [256+2q, +2): (high, low)
  __shared__ float gate_sm[T][S];
  __shared__ float u_sm[T][UP_ROWS];

  // 3. lo[t][k] = ((p0 + p1) + p2) + p3 (+ inj)
  store_lo<T, INJ, NI, UP_THREADS>(tid, pv, iv, lo_sm);
  __syncthreads();
  // 4. lo as BF16 high/low v_dot2 operands, in each lane's K order; gates; lo for inspection
  for (int i = tid; FMT == FMT_BF16 && i < T * 32; i += UP_THREADS) {
    const int t = i >> 5, qq = i & 31;
    float va[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) va[e] = lo_sm[t * R + 8 * qq + e];
    uint4 hi, lo;
    split_hi_lo(va, hi, lo);
    acta_sm[0][t][qq] = hi;
    acta_sm[1][t][qq] = lo;
    const f32x2 vb = {lo_sm[t * R + 256 + 2 * qq], lo_sm[t * R + 256 + 2 * qq + 1]};
    const bf16x2 bh = __builtin_convertvector(vb, bf16x2);
    const bf16x2 bl = __builtin_convertvector(vb - __builtin_convertvector(bh, f32x2), bf16x2);
    actb_sm[t][qq] = make_uint2(__builtin_bit_cast(uint32_t, bh), __builtin_bit_cast(uint32_t, bl));
  }
  if (tid < T * S) gate_sm[tid / S][tid % S] = 1.0f / (1.0f + expf(-lo_sm[(tid / S) * R + (tid % S)]));
  if (blockIdx.x == 0)
    for (int i = tid; i < T * R; i += UP_THREADS) lo_out[i] = lo_sm[i];
  __syncthreads();

  // 5. dot products: per (iteration, token) the lane's 10 K values, high then low part of lo
  //    (Q8_0: FP32 lo times the widened codes, one chain per block chunk, times its scale)
  constexpr int N = round2(UP_ITERS * T);
  float v[N];
#pragma unroll
  for (int i = UP_ITERS * T; i < N; ++i) v[i] = 0.f;
  if constexpr (FMT == FMT_Q8_0) {
    float wv[UP_ITERS][10], da[UP_ITERS], db[UP_ITERS];
#pragma unroll
    for (int m = 0; m < UP_ITERS; ++m) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        wv[m][e] = code(qa[m].x, e);
        wv[m][4 + e] = code(qa[m].y, e);
      }
      wv[m][8] = code(wb[m], 0);
      wv[m][9] = code(wb[m], 1);
      da[m] = half_bits_to_float(sa[m]);
      db[m] = half_bits_to_float(sb[m]);
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const f32x4 l0 = *reinterpret_cast<const f32x4*>(lo_sm + t * R + 8 * q);
      const f32x4 l1 = *reinterpret_cast<const f32x4*>(lo_sm + t * R + 8 * q + 4);
      const f32x2 l2 = *reinterpret_cast<const f32x2*>(lo_sm + t * R + 256 + 2 * q);
      const float lv[10] = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3], l2[0], l2[1]};
#pragma unroll
      for (int m = 0; m < UP_ITERS; ++m) {
        float a8 = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) a8 = __builtin_fmaf(wv[m][e], lv[e], a8);
        const float a2 = __builtin_fmaf(wv[m][9], lv[9], wv[m][8] * lv[8]);
        v[m * T + t] = __builtin_fmaf(da[m], a8, db[m] * a2);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < (FMT == FMT_BF16 ? T : 0); ++t) {
    const uint4 ah = acta_sm[0][t][q], al = acta_sm[1][t][q];
    const uint2 ab = actb_sm[t][q];
    const uint32_t hh[5] = {ah.x, ah.y, ah.z, ah.w, ab.x};
    const uint32_t ll[5] = {al.x, al.y, al.z, al.w, ab.y};
#pragma unroll
    for (int m = 0; m < UP_ITERS; ++m) {
      const uint32_t w[5] = {wa[m].x, wa[m].y, wa[m].z, wa[m].w, wb[m]};
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < 5; ++d) {
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, w[d]), __builtin_bit_cast(bf16x2v, hh[d]), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, w[d]), __builtin_bit_cast(bf16x2v, ll[d]), acc, false);
      }
      v[m * T + t] = acc;
    }
  }

  // 6. each row over its half-wave; row (lane >> 4) & 1 of the half holds values [((lane >> 4) & 1) * N/2, +N/2)
  half_wave_sum<N>(v);
  if ((lane & 15) == 0) {
    const int base = ((lane >> 4) & 1) * (N / 2);
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const int j = base + i;  // value j = m * T + t of row 10*wave + 2m + h
      if (j < UP_ITERS * T) u_sm[j % T][UP_WAVE_ROWS * wave + 2 * (j / T) + h] = v[i];
    }
  }
  __syncthreads();

  // 7. epilogue: out = pending + sigmoid(lo[t][s]) * u; stream mean over the quad (fixed order)
#pragma unroll
  for (int n = 0; n < NO; ++n) {
    const int o = tid + n * UP_THREADS;
    const bool has = o < T * UP_ROWS;
    const int t = has ? o / UP_ROWS : 0, cc = (o / S) % UP_COLS, s = o % S;
    float val = 0.f;
    if (has) {
      val = gate_sm[t][s] * u_sm[t][S * cc + s];
      if (PEND) val += pend[n];
      out[((size_t)t * S + s) * D + c0 + cc] = val;
    }
    const float m1 = val + dpp<0xB1>(val);  // streams (0+1), (2+3)
    const float m2 = m1 + dpp<0x4E>(m1);    // (0+1) + (2+3)
    if (has && s == 0) mean[(size_t)t * D + c0 + cc] = 0.25f * m2;
  }
}

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

// Q8_0 copies on the matrix cores: an MFMA K step of 32 is exactly one Q8_0 block, so the A operand is the
// block's codes widened exactly to BF16 (|q| <= 127 needs 8 significant bits), each step's product goes to a
// fresh accumulator, and its 4 rows are scaled by their block scales (4 FMAs per lane and step).  The WG's
// 40 rows x 10 block scales (800 bytes) are staged in LDS as floats, sc_sm[column][block][stream].
__device__ __forceinline__ bf16x8 codes_bf16(uint2 q) {
  uint32_t p[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t u = e < 2 ? q.x : q.y;
    const f32x2 f = {code(u, 2 * (e & 1)), code(u, 2 * (e & 1) + 1)};
    p[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));  // exact
  }
  return __builtin_bit_cast(bf16x8, make_uint4(p[0], p[1], p[2], p[3]));
}
constexpr int SC_WORDS = S * UP_COLS * (R / Q8_BLOCK) / 2;  // 200 dwords of binary16 scales per work-group

// up on the matrix cores (BF16 weights from T = UP_MFMA_FROM, Q8_0 copies from T = UP_MFMA_FROM_Q8).  The
// same work-group tile as hc_up (10 columns x 4 streams = 40 rows of W_up), as 3 tiles of 16 rows (waves
// 0..2; rows 40..47 repeat row 39 and are not stored) times v_mfma_f32_16x16x32_bf16: A = 16 rows x 32 K
// of W_up, B = 32 K x 16 columns
// of lo split into BF16 high and low parts.  T <= 8: column t holds token t's high parts and column
// 8 + t its low parts (one MFMA per K step); T > 8: one B matrix of high parts and one of low parts
// (two MFMAs per K step, high then low, into the same accumulator).  Lane (li, lg) then holds column li
// of rows 4 lg .. 4 lg + 3 of its tile: the 4 streams of one output column, so the epilogue and the
// stream mean stay in the lane (T <= 8: after adding column li + 8 by a row rotation).
template <int T, bool INJ, bool PEND, int FMT>
__global__ __launch_bounds__(256) void hc_up_mfma(const void* __restrict__ w_up, const uint16_t* __restrict__ s_up,
                                                  const float* __restrict__ part, const float* __restrict__ inj,
                                                  const float* pending, float* out, float* __restrict__ mean,
                                                  float* __restrict__ lo_out) {
  constexpr int UPM_THREADS = upm_threads(T);
  static_assert(T <= 16 && R % 32 == 0 && UP_ROWS > 32 && UP_ROWS <= 48 && (UPM_THREADS == 192 || UPM_THREADS == 256),
                "3 tiles of 16 rows (waves 0..2), 16 token columns");
  static_assert(Q8_BLOCK == 32 && (R / Q8_BLOCK) % 2 == 0, "one Q8_0 block per MFMA K step; scale rows of whole dwords");
  constexpr bool Q8 = FMT == FMT_Q8_0;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c0 = up_tile(blockIdx.x) * UP_COLS;  // an XCD's tiles are contiguous
  const int li = lane & 15, lg = lane >> 4;
  // 1. small loads first: stream partials and injection for lo, pending for the epilogue, and (Q8_0)
  //    the work-group's block scales: per stream s, rows s*2560 + c0 .. + 9 hold 200 contiguous bytes
  constexpr int ITEMS = T * (R / 4);
  constexpr int NI = (ITEMS + UPM_THREADS - 1) / UPM_THREADS;
  f32x4 pv[NI][S], iv[NI];
  load_partials<T, INJ, NI, UPM_THREADS>(tid, part, inj, pv, iv);
  constexpr int NSC = Q8 ? (SC_WORDS + UPM_THREADS - 1) / UPM_THREADS : 0;
  uint32_t scw[NSC > 0 ? NSC : 1];
#pragma unroll
  for (int n = 0; n < NSC; ++n) {
    const int it = min(tid + n * UPM_THREADS, SC_WORDS - 1), ss = it / (SC_WORDS / S);
    scw[n] = ldw4(reinterpret_cast<const uint32_t*>(s_up + ((size_t)ss * D + c0) * (R / Q8_BLOCK)) + it % (SC_WORDS / S));
  }
  // epilogue lane: token li, column cc = 4 * wave + lg (valid when wave < 3, cc < 10 and li < T); the
  // pending loads are clamped to a valid (token, column), so that no branch separates the loads
  const int cc = 4 * wave + lg;
  const bool eok = wave < 3 && cc < UP_COLS && li < T;
  float pend[S];
#pragma unroll
  for (int s = 0; s < S; ++s)
    pend[s] = PEND ? pending[((size_t)min(li, T - 1) * S + s) * D + c0 + min(cc, UP_COLS - 1)] : 0.f;
  __builtin_amdgcn_sched_barrier(0);  // keeps every small load ahead of the weight loads
  // 2. weights (A operand): tile = wave, row rw = 16 * wave + li, K 32 m + 8 lg.  No load is conditional:
  //    rows 40..47 of the third tile re-load row 39, and a 4th wave (T >= 10) re-loads the third tile's
  //    rows, cache hits whose results are never stored.  A branch around loads, even a wave-uniform one,
  //    makes the compiler wait for them before the first barrier, serialising the weight stream with the
  //    lo staging.
  const int rw = min(16 * min(wave, 2) + li, UP_ROWS - 1);
  // non-temporal weight loads (ldw*), except with a 4th wave: its repeats of the third tile's rows are separate
  // load instructions, which then missed in L2 (measured 0.1-0.17 us slower per read at T = 10..16)
  constexpr bool NTW = UPM_THREADS == 192;
  const size_t j = (size_t)(rw & 3) * D + c0 + (rw >> 2);
  uint4 a[Q8 ? 1 : R / 32];   // BF16: 8 weights per step
  uint2 qa[Q8 ? R / 32 : 1];  // Q8_0: 8 codes per step
#pragma unroll
  for (int m = 0; m < R / 32; ++m) {
    if constexpr (Q8)
      qa[m] = NTW ? ldw8(static_cast<const int8_t*>(w_up) + j * R + 32 * m + 8 * lg)
                  : *reinterpret_cast<const uint2*>(static_cast<const int8_t*>(w_up) + j * R + 32 * m + 8 * lg);
    else
      a[m] = NTW ? ldw16(static_cast<const uint16_t*>(w_up) + j * R + 32 * m + 8 * lg)
                 : *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(w_up) + j * R + 32 * m + 8 * lg);
  }
  __builtin_amdgcn_sched_barrier(0);

  // 3. lo = the 4 stream partials (+ inj), then its BF16 high/low parts in B operand order.
  //    T <= 8 (PACK): one B matrix, column t < 8 = high parts of token t, column 8 + t = its low parts:
  //      bh[m][g][n] = parts of lo[n & 7][32 m + 8 g .. + 8]
  //    T > 8: bh[m][g][t] and bl[m][g][t] = high and low parts of lo[t][32 m + 8 g .. + 8].
  //    Only the T tokens' columns are staged: a column of B reaches only the same column of the
  //    product, and the columns of tokens >= T are never stored.
  constexpr bool PACK = T <= 8;
  __shared__ __attribute__((aligned(16))) float lo_sm[T * R + LO_JUNK];
  __shared__ uint4 bh[R / 32][4][16], bl[PACK ? 1 : R / 32][4][16];
  __shared__ float gate_sm[T][S];
  __shared__ __attribute__((aligned(16))) float sc_sm[Q8 ? 2 * SC_WORDS + 2 * 64 : 4];
  store_lo<T, INJ, NI, UPM_THREADS>(tid, pv, iv, lo_sm);
#pragma unroll
  for (int n = 0; n < NSC; ++n) {  // scale u of stream ss: row c0 + u / 10, block u % 10; repeats to a junk slot
    const int it0 = tid + n * UPM_THREADS, it = min(it0, SC_WORDS - 1), ss = it / (SC_WORDS / S);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int u = 2 * (it % (SC_WORDS / S)) + h, col = u / (R / Q8_BLOCK), blk = u % (R / Q8_BLOCK);
      const int at = it0 < SC_WORDS ? (col * (R / Q8_BLOCK) + blk) * S + ss : 2 * SC_WORDS + 2 * (tid & 63) + h;
      sc_sm[at] = half_bits_to_float(scw[n] >> (16 * h));
    }
  }
  __syncthreads();
  for (int i = tid; i < (R / 32) * 4 * T; i += UPM_THREADS) {
    const int t = i % T, g = (i / T) & 3, m = i / (4 * T);
    float v8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v8[e] = lo_sm[t * R + 32 * m + 8 * g + e];
    uint4 hi, lo;
    split_hi_lo(v8, hi, lo);
    bh[m][g][t] = hi;
    if constexpr (PACK)
      bh[m][g][8 + t] = lo;
    else
      bl[m][g][t] = lo;
  }
  if (tid < T * S) gate_sm[tid / S][tid % S] = 1.0f / (1.0f + expf(-lo_sm[(tid / S) * R + (tid % S)]));
  if (blockIdx.x == 0)
    for (int i = tid; i < T * R; i += UPM_THREADS) lo_out[i] = lo_sm[i];
  __syncthreads();
  if (wave >= 3) return;
  // 4. the tile on the matrix cores, K in order (T > 8: high part then low part of each step, into the
  //    same accumulator; T <= 8: one product per step, then token t's high-part sum (column t) plus its
  //    low-part sum (column 8 + t, brought over by a rotation of the 16-lane row by 8).  Q8_0: each step
  //    (one block) into a fresh accumulator, added times the block scales of the lane's 4 rows.
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < R / 32; ++m) {
    const bf16x8 am = Q8 ? codes_bf16(qa[m]) : __builtin_bit_cast(bf16x8, a[Q8 ? 0 : m]);
    f32x4 pm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, __builtin_bit_cast(bf16x8, bh[m][lg][li]), Q8 ? zero : acc, 0, 0, 0);
    if constexpr (!PACK)
      pm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, __builtin_bit_cast(bf16x8, bl[m][lg][li]), pm, 0, 0, 0);
    if constexpr (Q8) {
      const f32x4 dm = *reinterpret_cast<const f32x4*>(sc_sm + (min(cc, UP_COLS - 1) * (R / Q8_BLOCK) + m) * S);
#pragma unroll
      for (int s = 0; s < S; ++s) acc[s] = __builtin_fmaf(dm[s], pm[s], acc[s]);
    } else {
      acc = pm;
    }
  }
  if constexpr (PACK) {
#pragma unroll
    for (int s = 0; s < S; ++s) acc[s] += dpp<0x128>(acc[s]);  // row_ror:8
  }
  // 5. epilogue: lane = token li, rows 16 wave + 4 lg + s = stream s of column 4 wave + lg; the stream
  //    mean in the v_dot2 kernel's order ((s0 + s1) + (s2 + s3))
  if (eok) {
    float o[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      o[s] = gate_sm[li][s] * acc[s];
      if (PEND) o[s] += pend[s];
      out[((size_t)li * S + s) * D + c0 + cc] = o[s];
    }
    mean[(size_t)li * D + c0 + cc] = 0.25f * ((o[0] + o[1]) + (o[2] + o[3]));
  }
}


// ---------------------------------------------------------------------------
// Q8_0 copies on the device: 4 lanes per 32-weight block (8 BF16 weights each);
// each lane takes Q8_CHUNKS chunks a grid-stride apart, all loads issued first (one chunk: see below)
// ---------------------------------------------------------------------------
// One 16-byte chunk per lane: 1,600 work-groups per matrix of the read (~25 waves per CU).  Measured on
// MI355X (320 x 10240, 64 rotated matrices): 4.45 us per matrix, against 4.89 / 5.30 / 5.92 us with
// 2 / 4 / 8 chunks per lane.
constexpr int Q8_CHUNKS = 1;

__global__ __launch_bounds__(256) void q8_quantize(const uint4* __restrict__ w, size_t n_blocks,
                                                   uint2* __restrict__ codes, uint16_t* __restrict__ scales) {
  const size_t stride = (size_t)gridDim.x * 256;  // a multiple of 4: a quad stays one block
  const size_t i0 = (size_t)blockIdx.x * 256 + threadIdx.x;
  uint4 u[Q8_CHUNKS];
#pragma unroll
  for (int k = 0; k < Q8_CHUNKS; ++k) {
    const size_t i = i0 + k * stride;  // chunk i = block i/4, weights 8(i%4) ..
    u[k] = (i >> 2) < n_blocks ? ldw16(w + i) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int k = 0; k < Q8_CHUNKS; ++k) {
    const size_t i = i0 + k * stride;
    const uint32_t uu[4] = {u[k].x, u[k].y, u[k].z, u[k].w};
    float f[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = __uint_as_float(uu[e] << 16);
      f[2 * e + 1] = __uint_as_float(uu[e] & 0xffff0000u);
    }
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(f[e]));
    amax = fmaxf(amax, dpp<0xB1>(amax));  // quad_perm [1,0,3,2]
    amax = fmaxf(amax, dpp<0x4E>(amax));  // quad_perm [2,3,0,1]
    const float d = amax / 127.0f;        // IEEE binary32 division (correctly rounded)
    const float id = d != 0.f ? 1.0f / d : 0.f;
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int qv = static_cast<int>(__builtin_roundf(f[e] * id));  // ties away from zero
      packed[e >> 2] |= (static_cast<uint32_t>(qv) & 0xffu) << (8 * (e & 3));
    }
    if ((i >> 2) < n_blocks) {  // a quad is entirely in or out
      codes[i] = make_uint2(packed[0], packed[1]);
      if ((i & 3) == 0) scales[i >> 2] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(d));
    }
  }
}

int launch_quantize_q8_0(const void* w, size_t n_blocks, void* codes, void* scales, void* stream) {
  const size_t chunks = n_blocks * 4;
  const size_t wgs = (chunks + 256 * Q8_CHUNKS - 1) / (256 * Q8_CHUNKS);
  (void)hipGetLastError();
  hipLaunchKernelGGL(q8_quantize, dim3(static_cast<unsigned>(wgs)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const uint4*>(w), n_blocks,
                     static_cast<uint2*>(codes), static_cast<uint16_t*>(scales));
  return hipGetLastError() == hipSuccess ? HCR_OK : HCR_EHIP;
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
typedef void (*down_fn)(const void*, const uint16_t*, const float*, const float*, float*, float*);
typedef void (*up_fn)(const void*, const uint16_t*, const float*, const float*, const float*, float*, float*,
                      float*);

#define HCR_DOWN_ROW(F) \
  {hc_down<1, F>,  hc_down<2, F>,  hc_down<3, F>,  hc_down<4, F>,  hc_down<5, F>,  hc_down<6, F>,  \
   hc_down<7, F>,  hc_down<8, F>,  hc_down<9, F>,  hc_down<10, F>, hc_down<11, F>, hc_down<12, F>, \
   hc_down<13, F>, hc_down<14, F>, hc_down<15, F>, hc_down<16, F>}
static const down_fn kDown[2][TMAX] = {HCR_DOWN_ROW(FMT_BF16), HCR_DOWN_ROW(FMT_Q8_0)};
#undef HCR_DOWN_ROW
#define HCR_UP_T(T, F) {{hc_up<T, false, false, F>, hc_up<T, false, true, F>}, {hc_up<T, true, false, F>, hc_up<T, true, true, F>}}
#define HCR_UP_ROW(F)                                                                              \
  {HCR_UP_T(1, F),  HCR_UP_T(2, F),  HCR_UP_T(3, F),  HCR_UP_T(4, F),  HCR_UP_T(5, F),  HCR_UP_T(6, F),  \
   HCR_UP_T(7, F),  HCR_UP_T(8, F),  HCR_UP_T(9, F),  HCR_UP_T(10, F), HCR_UP_T(11, F), HCR_UP_T(12, F), \
   HCR_UP_T(13, F), HCR_UP_T(14, F), HCR_UP_T(15, F), HCR_UP_T(16, F)}
static const up_fn kUp[2][TMAX][2][2] = {HCR_UP_ROW(FMT_BF16), HCR_UP_ROW(FMT_Q8_0)};
#undef HCR_UP_ROW
#undef HCR_UP_T

#define HCR_UPM_T(T, F) {{hc_up_mfma<T, false, false, F>, hc_up_mfma<T, false, true, F>}, \
                         {hc_up_mfma<T, true, false, F>, hc_up_mfma<T, true, true, F>}}
#define HCR_UPM_ROW(F)                                                                             \
  {HCR_UPM_T(1, F),  HCR_UPM_T(2, F),  HCR_UPM_T(3, F),  HCR_UPM_T(4, F),  HCR_UPM_T(5, F),       \
   HCR_UPM_T(6, F),  HCR_UPM_T(7, F),  HCR_UPM_T(8, F),  HCR_UPM_T(9, F),  HCR_UPM_T(10, F),      \
   HCR_UPM_T(11, F), HCR_UPM_T(12, F), HCR_UPM_T(13, F), HCR_UPM_T(14, F), HCR_UPM_T(15, F),      \
   HCR_UPM_T(16, F)}
static_assert(TMAX == 16, "the table below lists T = 1..16");
static const up_fn kUpM[2][TMAX][2][2] = {HCR_UPM_ROW(FMT_BF16), HCR_UPM_ROW(FMT_Q8_0)};
#undef HCR_UPM_ROW
#undef HCR_UPM_T

int launch_read(int fmt, int T, const void* w_down, const uint16_t* s_down, const void* w_up, const uint16_t* s_up,
                const float* w_norm, void* scratch, const float* x, const float* pending, const float* inj,
                float* out, float* mean, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* sc = static_cast<char*>(scratch);
  float* part = reinterpret_cast<float*>(sc + OFF_PART);
  float* lo = reinterpret_cast<float*>(sc + OFF_LO);
  float* rs = reinterpret_cast<float*>(sc + OFF_RS);
  (void)hipGetLastError();  // clear a stale error left by unrelated earlier calls
  hipLaunchKernelGGL(kDown[fmt][T - 1], dim3(DOWN_WGS), dim3(down_threads(T)), 0, st, w_down, s_down, x, w_norm, part,
                     rs);
  const bool mfma = T >= (fmt == FMT_BF16 ? UP_MFMA_FROM : UP_MFMA_FROM_Q8);
  const up_fn up = mfma ? kUpM[fmt][T - 1][inj != nullptr][pending != nullptr]
                        : kUp[fmt][T - 1][inj != nullptr][pending != nullptr];
  hipLaunchKernelGGL(up, dim3(UP_WGS), dim3(mfma ? upm_threads(T) : UP_THREADS), 0, st, w_up, s_up, part, inj,
                     pending, out, mean, lo);
  return hipGetLastError() == hipSuccess ? HCR_OK : HCR_EHIP;
}

// ---------------------------------------------------------------------------
// the library's own scratch (hcr_read_static): one array per GPU, held until the process ends
// ---------------------------------------------------------------------------
// In host code `scratch` names a host-side stand-in, not a device address: the kernels get the address
// hipGetSymbolAddress gives for the device the read runs on, found once per device with that device
// current.  Every call on one GPU shares its array, so calls that overlap in time on one GPU race (the
// caller orders them, e.g. on one stream).  Nothing in it needs to start at zero: each read writes every
// partial, lo and rs value before reading it.
static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::atomic<void*> g_scratch_ptr[MAX_DEVICES];
std::mutex g_scratch_mu;
}  // namespace

int static_scratch(void* stream, void** out) {
  *out = nullptr;
  int cur = -1, dev = -1;
  if (hipGetDevice(&cur) != hipSuccess) return HCR_EHIP;
  dev = cur;
  if (stream && hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &dev) != hipSuccess) return HCR_EHIP;
  if (dev < 0 || dev >= MAX_DEVICES) return HCR_EHIP;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (dev != cur && hipSetDevice(dev) != hipSuccess) return HCR_EHIP;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (dev != cur && hipSetDevice(cur) != hipSuccess) return HCR_EHIP;
      if (e != hipSuccess || !p) return HCR_EHIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return HCR_OK;
}

}  // namespace hcr
