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
//   hc_up_mfma<T, INJ, PEND> (BF16 weights at every T, Q8_0 copies from T = 4):
//     lo[t][k] = the 4 stream
//     partials (+ injection), then 40 rows of W_up (10 columns x 4 streams) per
//     work-group as three 16-row tiles on the matrix cores
//     (v_mfma_f32_16x16x32_bf16), lo split into BF16 high and low parts as the
//     B operand.  Up to 8 tokens the high parts fill B columns 0..7 and the low
//     parts columns 8..15, one product per K step; from 9 tokens each part has
//     its own product.  Epilogue in the lane: pending write, sigmoid gate of
//     lo[t][s], stream mean.
//   hc_up<T, INJ, PEND>: the same tile on the vector ALUs (Q8_0 at T = 1..3;
//     for BF16 only the calibration library runs it, to time it against the other).  Each row is reduced by the 32 lanes of a half-wave;
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
// Why the matrix cores for the BF16 up projection: the v_dot2 kernel issues
// ~100 VALU instructions per token per wave, which the loads cannot hide with
// one wave per SIMD; the matrix-core kernel's 10 or 20 MFMAs per wave cost the
// same at every T.  With its weights loaded straight into LDS in whole lines it
// is faster at T = 1 too: 6.18 against 6.25 us per read (whole read, one
// process, alternating builds, 3 rounds).
//
// T = 10..16: the down kernel takes the tokens in groups of 8 (the next
// group's x loads overlap the current group's FMAs); up to 9 in one group.  A token's result is the
// same bit for bit at every T of one range: T = 1..8 and T = 9..16 (the two
// B layouts round differently).
//
// Why no atomics: the pages finish the split reduction in the last
// work-group to arrive at a counter.  On MI355X an agent-scope arrival
// counter plus the finisher's reads cost several microseconds per launch
// (cross-XCD release/acquire).  Here the down work-group covers a whole
// stream, and the up kernel adds the 4 stream partials itself while its
// weight loads are in flight.
//
// Loads: vector-memory loads complete in issue order, so every kernel issues
// the small inputs its arithmetic needs first (x, w_norm; partials,
// injection) and its weight tile after them, all before any arithmetic (the
// pending values, which only the epilogue needs, go behind the weights where
// the up kernel waits for its loads itself); the weights go in the
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
// within T = 1..8 or within T = 9..16 (BF16), or within T = 1..3, 4..8 or
// 9..16 (Q8_0).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "hcr_device.h"
#include "hcr_layout.h"
#include "hcr_up.h"

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
    // per row the two block scales first, then the codes: the decoded path multiplies every code by its
    // scale, so a row's products wait for its last load either way, and that is a code.  Measured on MI355X
    // (bench.py --ab --ab-q8, one process, alternating builds, 4 rounds): 0.03 us less per read at T = 4..8
#pragma unroll
    for (int r = 0; r < DOWN_ROWS; ++r) {
      sa[r] = ldw2(sr + (size_t)r * (DD / Q8_BLOCK) + ca / Q8_BLOCK);
      sb[r] = ldw2(sr + (size_t)r * (DD / Q8_BLOCK) + cb / Q8_BLOCK);
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
        // pinned here: the compiler had sunk some tokens' sums of squares below the first wait for the
        // weights (T = 3, 6, 7: 20-30 VALU instructions).  Measured on MI355X (bench.py --ab, one process,
        // alternating builds, 6 rounds): the 96-read window 707.6 against 710.0 us; the sweep level
        vm_pin(v[quad_pos(t, N)]);
#pragma unroll
        for (int e = 0; e < NC; ++e) vm_pin(act[i][e]);
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
    // 3. per row: the weights widened exactly to FP32, one FMA chain per token.  Q8_0: below UP_MFMA_FROM_Q8
    //    tokens one chain per block chunk, each times its block's scale; from there the codes are first
    //    decoded to d * q (exact in FP32: 11 + 7 significant bits), once per row, and then take the BF16 path's
    //    chain.  The switch sits where the up kernel switches, so that within each range of T one pair of
    //    kernels serves, a token's result does not depend on T
    constexpr bool DECODE = FMT == FMT_Q8_0 && T >= UP_MFMA_FROM_Q8;
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
      if constexpr (FMT == FMT_BF16 || DECODE) {
        // every token's chain over the CA columns of the row's first load, then (after a scheduling barrier)
        // over the CB columns of its second: each chain keeps its order, and the wait for the second load
        // comes after every product of the first.  The compiler had placed it after the first token's CA
        // products, so that at T = 6 / 8, 53 / 73 FMAs of the last row waited for the last load instead of
        // 12 / 16.  Measured on MI355X (bench.py --ab, one process, alternating builds, 5-6 rounds, the results
        // bitwise the same): the 96-read window 701.8 against 705.6 us, 0.03 us less per read at T = 6..8,
        // level at T = 1..5 and for the Q8_0 copies
        float acc[TG];
#pragma unroll
        for (int i = 0; i < TG; ++i) {
          acc[i] = 0.f;
#pragma unroll
          for (int e = 0; e < CA; ++e) acc[i] = __builtin_fmaf(wv[e], act[i][e], acc[i]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < TG; ++i) {
          const int t = grp * TG + i;
          if (t < T) {
#pragma unroll
            for (int e = CA; e < NC; ++e) acc[i] = __builtin_fmaf(wv[e], act[i][e], acc[i]);
            v[quad_pos((r + 1) * T + t, N)] = acc[i];
          }
        }
      } else {  // Q8_0 below 4 tokens: one chain per block chunk, each times its block's scale
#pragma unroll
        for (int i = 0; i < TG; ++i) {
          const int t = grp * TG + i;
          if (t < T) {
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
  hipLaunchKernelGGL(up, dim3(UP_WGS), dim3(mfma ? upm_threads(T, fmt) : UP_THREADS), 0, st, w_up, s_up, part, inj,
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
