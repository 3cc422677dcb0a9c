// The up kernels of the BF16 hyper-connection read (and of its Q8_0 sibling) for gfx950: hc_up (vector
// ALUs) and hc_up_mfma (matrix cores), with their helpers.  Header-only templates: hcr_kernels.hip
// dispatches them in the read; the calibration library (hcr_calib.hip) launches either one alone, to time
// the two against each other at every T.  The design of both is described in hcr_kernels.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hcr_device.h"
#include "hcr_layout.h"

namespace hcr {

// The up kernels' first loads: the 4 stream partials (and the injection) of lo, 4 K values of one token
// per item, items tid + n * NT (NT threads).  Neither the loads nor the stores of lo are conditional: items
// past the end load the last item again (store_lo puts those repeats in junk slots).  A branch among the loads
// makes the compiler wait for every load issued so far, and a branch around their only use lets it sink
// them below the weight loads; either would serialise them with the weight stream.
template <int T, bool INJ, int NI, int NT, int NSRC = S>
__device__ __forceinline__ void load_partials(int tid, const float* __restrict__ part,
                                              const float* __restrict__ inj, f32x4 (&pv)[NI][S],
                                              f32x4 (&iv)[NI]) {
  constexpr int ITEMS = T * (R / 4);
#pragma unroll
  for (int n = 0; n < NI; ++n) {
    const int it = min(tid + n * NT, ITEMS - 1);
    const int t = it / (R / 4), k = 4 * (it % (R / 4));
#pragma unroll
    for (int ss = 0; ss < NSRC; ++ss) pv[n][ss] = ld4(part + ((size_t)ss * TMAX + t) * R + k);
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
__device__ __forceinline__ void hc_up_body(const void* __restrict__ w_up,
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

// The BF16 weight loads of hc_up_mfma (described there) for tile `wave` of the work-group at column c0:
// 10 loads straight into the wave's LDS region at a_sm, untracked (the kernel waits for them itself).
// Load i of a wave lands at byte i * A_LOAD_STRIDE of its region: 1024 bytes, then 128 of padding, so that
// odd loads start 128 bytes into a 256-byte LDS row and even loads at its start.
constexpr int A_LOAD_STRIDE = 1024 + 128;
template <int A_REGION>
__device__ __forceinline__ void load_a_lds(const uint16_t* __restrict__ w_up, uint32_t a_sm, int wave, int lane,
                                           int c0) {
  const int rho = lane >> 3, e = lane & 7;
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const int p = i >> 1, h = i & 1;
    int rw = 16 * wave + 8 * h + rho;
    rw = rw < UP_ROWS ? rw : rw - 8;
    const size_t j = (size_t)(rw & 3) * D + c0 + (rw >> 2);
    ldw16_lds_untracked(w_up + j * R + 8 * (8 * p + (e ^ rho)), a_sm + wave * A_REGION + i * A_LOAD_STRIDE);
  }
}

// up on the matrix cores (BF16 weights from T = UP_MFMA_FROM, Q8_0 copies from T = UP_MFMA_FROM_Q8).  The
// same work-group tile as hc_up (10 columns x 4 streams = 40 rows of W_up), as 3 tiles of 16 rows (waves
// 0..2; rows 40..47 repeat rows 32..39 and are not stored; a 4th wave, where upm_threads gives one, only
// stages lo) times v_mfma_f32_16x16x32_bf16: A = 16 rows x 32 K
// of W_up, B = 32 K x 16 columns
// of lo split into BF16 high and low parts.  T <= 8: column t holds token t's high parts and column
// 8 + t its low parts (one MFMA per K step); T > 8: one B matrix of high parts and one of low parts
// (two MFMAs per K step, high then low, into the same accumulator).  Lane (li, lg) then holds column li
// of rows 4 lg .. 4 lg + 3 of its tile: the 4 streams of one output column, so the epilogue and the
// stream mean stay in the lane (T <= 8: after adding column li + 8 by a row rotation).  NSRC: the number of
// partial sources summed into lo, the 4 stream partials in the read; 1 where lo itself is given (the
// calibration library's read in the pages' shape, whose down kernel finishes lo).
template <int T, bool INJ, bool PEND, int FMT, int NSRC = S>
__device__ __forceinline__ void hc_up_mfma_body(const void* __restrict__ w_up, const uint16_t* __restrict__ s_up,
                                                  const float* __restrict__ part, const float* __restrict__ inj,
                                                  const float* pending, float* out, float* __restrict__ mean,
                                                  float* __restrict__ lo_out) {
  constexpr int UPM_THREADS = upm_threads(T, FMT);
  static_assert(T <= 16 && R % 32 == 0 && UP_ROWS > 32 && UP_ROWS <= 48 && UPM_THREADS % 64 == 0 && UPM_THREADS >= 192 &&
                    UPM_THREADS <= 512,
                "3 tiles of 16 rows (waves 0..2; further waves stage lo only), 16 token columns");
  static_assert(Q8_BLOCK == 32 && (R / Q8_BLOCK) % 2 == 0, "one Q8_0 block per MFMA K step; scale rows of whole dwords");
  static_assert(NSRC == S || NSRC == 1, "lo from the 4 stream partials, or lo itself");
  constexpr bool Q8 = FMT == FMT_Q8_0;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c0 = up_tile(blockIdx.x) * UP_COLS;  // an XCD's tiles are contiguous
  const int li = lane & 15, lg = lane >> 4;
  // 1. small loads first: stream partials and injection for lo, pending for the epilogue (on the LDS path
  //    after the weights instead, step 2), and (Q8_0) the work-group's block scales: per stream s, rows
  //    s*2560 + c0 .. + 9 hold 200 contiguous bytes
  //    BF16 (ALDS, up_weights_lds): every load of the kernel is untracked (ld*_untracked: the
  //    weights go straight into LDS, step 2) and waited for explicitly; otherwise ordinary loads.  A 4th wave
  //    (upm_threads: from T = 10, and below where it takes a round off the staging) has no tile: with ALDS it
  //    loads no weights.
  constexpr bool NTW = UPM_THREADS == 192;
  constexpr bool ALDS = up_weights_lds(T, FMT);
  constexpr bool EXTRA = UPM_THREADS > 192;  // waves beyond the 3 tiles: no tile, they stage lo only
  constexpr int ITEMS = T * (R / 4);
  constexpr int NI = (ITEMS + UPM_THREADS - 1) / UPM_THREADS;
  f32x4 pv[NI][S], iv[NI];
  if constexpr (ALDS) {
    static_assert(!ALDS || UPM_THREADS <= 256, "at most one staging-only wave on the LDS path");
    const int wv = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
    for (int n = 0; n < NI; ++n) {  // load_partials' items and order
      const int it = min(tid + n * UPM_THREADS, ITEMS - 1);
      const int t = it / (R / 4), k = 4 * (it % (R / 4));
      // The staging-only 4th wave skips a round whose items all lie past the end (T = 5, 8, 10..12), where
      // it would load the last item 4 times over for nothing (its wait counts only the younger pending loads,
      // so it stays exact).  Measured on MI355X (bench.py --ab, one process, alternating builds, 5 rounds):
      // 0.17 us faster per read at T = 8, level at the other T.  The tile waves keep their repeats: skipping
      // them as well (whole waves, or lane by lane) was 0.05-0.2 us slower at T = 1, 2, 4 and 10..11
      if (!(EXTRA && 192 + n * UPM_THREADS >= ITEMS && wv >= 3)) {
#pragma unroll
        for (int ss = 0; ss < NSRC; ++ss) pv[n][ss] = ld4_untracked(part + ((size_t)ss * TMAX + t) * R + k);
        if (INJ) iv[n] = ld4_untracked(inj + (size_t)t * R + k);
      }
    }
  } else {
    load_partials<T, INJ, NI, UPM_THREADS, NSRC>(tid, part, inj, pv, iv);
  }
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
  // A staging-only 4th wave on the LDS path has no epilogue lanes and loads no pending values (its loads are
  // untracked, so the branch adds no wait).  Measured on MI355X (bench.py --ab --ab-window, one process,
  // alternating builds, 6 rounds): the 96-read window (T = 6, pending on) from 721.3 to 712.6 us; skipping the
  // tile waves' lanes outside the epilogue as well gave 715.3 us.  On the LDS path the pending values are
  // loaded after the weights (step 2): only the epilogue uses them, and loads complete in issue order, so they
  // arrive right behind the last weights instead of holding the weights back (the window 706.7 against
  // 710.8 us, the same A/B)
  float pend[S];
  const bool pload = !(ALDS && EXTRA) || __builtin_amdgcn_readfirstlane(wave) < 3;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const float* pp = pending + ((size_t)min(li, T - 1) * S + s) * D + c0 + min(cc, UP_COLS - 1);
    pend[s] = 0.f;
    if (PEND && !ALDS) pend[s] = *pp;
  }
  __builtin_amdgcn_sched_barrier(0);  // keeps every small load ahead of the weight loads
  // 2. weights (A operand), tile = wave: row rw = 16 * wave + li of the work-group's 40 (rw & 3 = stream,
  //    rw >> 2 = column), K chunk (8 values) 4 m + lg at step m.
  //    ALDS: straight into LDS (global_load_lds_dwordx4, non-temporal), each wave into a region of its own
  //    that only it reads back, so no barrier guards it.  Load i = 2 p + h of a wave covers tile rows
  //    8 h .. 8 h + 7 and line p (K 64 p .. 64 p + 63) of each: lane 8 rho + e takes chunk 8 p + (e ^ rho) of
  //    row 8 h + rho, so every 16 lanes read two whole 128-byte lines (in the operand layout every 16 lanes
  //    touch 16 rows, 16 bytes each: twice the requests, measured 0.3-0.4 us slower per read).  Load i lands
  //    at byte i * 1152 of the region (A_LOAD_STRIDE), so the 8 rows of load 2 p sit at 0 and those of load
  //    2 p + 1 at 128 modulo 256: the read-back of one chunk's 16 rows meets 16 distinct LDS bank groups.  The
  //    third tile's rows 40..47 load rows 32..39 again (their products are not stored).
  //    Q8_0 codes in the operand layout, into registers: lane (li, lg) loads the 8 codes of row rw at
  //    K 32 m + 8 lg.  No load is conditional: rows 40..47 of the third tile re-load row 39, and a 4th wave
  //    re-loads the third tile's rows, cache hits whose results are never stored (a branch around loads, even
  //    a wave-uniform one, makes the compiler wait for them before the first barrier).  Non-temporal, except
  //    with a 4th wave: its repeats of the third tile's rows are separate load instructions, which then
  //    missed in L2 (measured with BF16 weights on this path: 0.1-0.17 us slower per read at T = 10..16).
  constexpr int A_REGION = 10 * A_LOAD_STRIDE;
  static_assert(R == 320, "5 lines of 128 bytes per BF16 row, 10 loads per wave");
  __shared__ __attribute__((aligned(16))) unsigned char a_sm[ALDS ? 3 * A_REGION : 16];
  static_assert(ALDS || Q8, "BF16 weights always go straight into LDS (up_weights_lds)");
  uint2 qa[Q8 ? R / 32 : 1];  // Q8_0: 8 codes per step
  if constexpr (ALDS) {
    if (!EXTRA || wave < 3)
      load_a_lds<A_REGION>(static_cast<const uint16_t*>(w_up), lds_addr(a_sm), __builtin_amdgcn_readfirstlane(wave),
                           lane, c0);
    if (PEND && pload) {  // the pending values, behind the weights
#pragma unroll
      for (int s = 0; s < S; ++s)
        pend[s] = ld1_untracked(pending + ((size_t)min(li, T - 1) * S + s) * D + c0 + min(cc, UP_COLS - 1));
    }
  } else {
    const int rw = min(16 * min(wave, 2) + li, UP_ROWS - 1);
    const size_t j = (size_t)(rw & 3) * D + c0 + (rw >> 2);
#pragma unroll
    for (int m = 0; m < R / 32; ++m)
      qa[m] = NTW ? ldw8(static_cast<const int8_t*>(w_up) + j * R + 32 * m + 8 * lg)
                  : *reinterpret_cast<const uint2*>(static_cast<const int8_t*>(w_up) + j * R + 32 * m + 8 * lg);
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (ALDS) {  // the partials (and injection): all but the 10 weight loads and the pending loads
    if (!EXTRA || wave < 3)
      vm_wait<(PEND ? S : 0) + 10>();
    else
      vm_wait<0>();  // a wave with no tile loads no weights, and no pending values
#pragma unroll
    for (int n = 0; n < NI; ++n) {
#pragma unroll
      for (int ss = 0; ss < NSRC; ++ss) vm_pin(pv[n][ss]);
      if (INJ) vm_pin(iv[n]);
    }
  }

  // 3. lo = the 4 stream partials (+ inj), item by item (the 4 K values of one token that load_partials'
  //    order gives each thread), and its BF16 high and low parts straight into B operand order, 8 bytes
  //    each (no round trip of lo through LDS):
  //    T <= 8 (PACK): one B matrix, column t < 8 = high parts of token t, column 8 + t = its low parts:
  //      bh[m][g][n ^ sw] = parts of lo[n & 7][32 m + 8 g .. + 8]
  //    T > 8: bh[m][g][t ^ sw] and bl[m][g][t ^ sw] = high and low parts of lo[t][32 m + 8 g .. + 8];
  //    sw = (4 m + g) % 16.  A wave's items are consecutive K of one token: swizzled, each 32 of them write
  //    32 distinct 8-byte slots of a 256-byte LDS row (unswizzled, every 16 would meet the same banks), and
  //    the operand read of one (m, g) still takes 16 distinct 16-byte slots.  Only the T tokens' columns
  //    are staged: a column of B reaches only the same column of the product, and the columns of tokens
  //    >= T are never stored.  Items past the end (repeats of the last) write a junk slot of their thread.
  constexpr bool PACK = T <= 8;
  __shared__ uint4 bh[R / 32][4][16], bl[PACK ? 1 : R / 32][4][16];
  __shared__ uint2 b_junk[2 * UPM_THREADS];
  __shared__ f32x4 lo4_sm[T];
  __shared__ __attribute__((aligned(16))) float sc_sm[Q8 ? 2 * SC_WORDS + 2 * 64 : 4];
#pragma unroll
  for (int n = 0; n < NI; ++n) {
    const int it0 = tid + n * UPM_THREADS, it = min(it0, ITEMS - 1);
    const int t = it / (R / 4), k = 4 * (it % (R / 4));
    f32x4 vv = NSRC == S ? ((pv[n][0] + pv[n][1]) + pv[n][2]) + pv[n][3] : pv[n][0];
    if (INJ) vv += iv[n];
    uint2 hi, lo;
    split_hi_lo4(vv, hi, lo);
    const int m = k >> 5, g = (k >> 3) & 3, half = (k >> 2) & 1, sw = (4 * m + g) & 15;
    const bool real = it0 < ITEMS;
    uint2* dh = real ? reinterpret_cast<uint2*>(&bh[m][g][t ^ sw]) + half : &b_junk[2 * tid];
    uint2* dl = real ? reinterpret_cast<uint2*>(PACK ? &bh[m][g][(8 + t) ^ sw] : &bl[m][g][t ^ sw]) + half
                     : &b_junk[2 * tid + 1];
    *dh = hi;
    *dl = lo;
    if (real && k == 0) lo4_sm[t] = vv;  // lo[t][0 .. S), whose sigmoids are the gates
    if (real && blockIdx.x == 0) *reinterpret_cast<f32x4*>(lo_out + t * R + k) = vv;
  }
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
  if (wave >= 3) return;
  // the gates of the lane's token, sigmoid of lo[li][0 .. S), computed here while the weights still arrive
  // (in the staging above, the few lanes holding K 0 of a token would hold up their whole waves)
  float gate[S];
  {
    const f32x4 l4 = lo4_sm[min(li, T - 1)];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      gate[s] = 1.0f / (1.0f + expf(-l4[s]));
      vm_pin(gate[s]);  // computed here, ahead of the first wait for the weights, not sunk into the epilogue
    }
  }
  // 4. the tile on the matrix cores, K in order (T > 8: high part then low part of each step, into the
  //    same accumulator; T <= 8: one product per step, then token t's high-part sum (column t) plus its
  //    low-part sum (column 8 + t, brought over by a rotation of the 16-lane row by 8).  Q8_0: each step
  //    (one block) into a fresh accumulator, added times the block scales of the lane's 4 rows.
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  // every step's B operand read from LDS ahead of the first wait for the weights, so that a step waits only
  // for its A read once its weights are in.  Measured on MI355X (bench.py --ab, one process, alternating
  // builds, 4 rounds): 0.04-0.08 us less per read at T = 1..8, 0.19 us at T = 9..12, 0.03-0.05 us at
  // T = 13..16 (weights then in registers), 0.06-0.12 us for the Q8_0 copies from T = 4; the results the same
  // bit for bit
  uint4 bpre[R / 32], lpre[PACK ? 1 : R / 32];
#pragma unroll
  for (int m = 0; m < R / 32; ++m) {
    bpre[m] = bh[m][lg][li ^ ((4 * m + lg) & 15)];  // column li of B, swizzled as staged
    if constexpr (!PACK) lpre[m] = bl[m][lg][li ^ ((4 * m + lg) & 15)];
  }
#pragma unroll
  for (int m = 0; m < R / 32; ++m) {
    bf16x8 am;
    if constexpr (Q8) {
      am = codes_bf16(qa[m]);
    } else {
      // chunk 4 m + lg of tile row li: line p = m / 2, load 2 p + li / 8, lane 8 (li % 8) + (chunk % 8) ^ (li % 8);
      // line p's two loads are done once no more than the 8 - 2 p weight loads after them (and the pending
      // loads behind those) are in flight
      if (m % 2 == 0) vm_wait_n(8 - m + (PEND ? S : 0));
      const int h = li >> 3, r8 = li & 7, ep = (4 * m + lg) & 7;
      am = *reinterpret_cast<const bf16x8*>(a_sm + wave * A_REGION + (2 * (m >> 1) + h) * A_LOAD_STRIDE +
                                            16 * (8 * r8 + (ep ^ r8)));
    }
    f32x4 pm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, __builtin_bit_cast(bf16x8, bpre[m]), Q8 ? zero : acc, 0, 0, 0);
    if constexpr (!PACK)
      pm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, __builtin_bit_cast(bf16x8, lpre[m]), pm, 0, 0, 0);
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
  if constexpr (ALDS && PEND) {  // the pending loads, the youngest of the kernel
    vm_wait<0>();
#pragma unroll
    for (int s = 0; s < S; ++s) vm_pin(pend[s]);
  }
  // 5. epilogue: lane = token li, rows 16 wave + 4 lg + s = stream s of column 4 wave + lg; the stream
  //    mean in the v_dot2 kernel's order ((s0 + s1) + (s2 + s3))
  if (eok) {
    float o[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      o[s] = gate[s] * acc[s];
      if (PEND) o[s] += pend[s];
      out[((size_t)li * S + s) * D + c0 + cc] = o[s];
    }
    mean[(size_t)li * D + c0 + cc] = 0.25f * ((o[0] + o[1]) + (o[2] + o[3]));
  }
}


// the kernels (their bodies above are also launched alone, under other kernel names, by the calibration
// library)
template <int T, bool INJ, bool PEND, int FMT>
__global__ __launch_bounds__(UP_THREADS) void hc_up(const void* __restrict__ w_up, const uint16_t* __restrict__ s_up,
                                                     const float* __restrict__ part, const float* __restrict__ inj,
                                                     const float* pending, float* out, float* __restrict__ mean,
                                                     float* __restrict__ lo_out) {
  hc_up_body<T, INJ, PEND, FMT>(w_up, s_up, part, inj, pending, out, mean, lo_out);
}
template <int T, bool INJ, bool PEND, int FMT>
__global__ __launch_bounds__(upm_threads(T, FMT)) void hc_up_mfma(const void* __restrict__ w_up, const uint16_t* __restrict__ s_up,
                                                  const float* __restrict__ part, const float* __restrict__ inj,
                                                  const float* pending, float* out, float* __restrict__ mean,
                                                  float* __restrict__ lo_out) {
  hc_up_mfma_body<T, INJ, PEND, FMT>(w_up, s_up, part, inj, pending, out, mean, lo_out);
}

}  // namespace hcr
