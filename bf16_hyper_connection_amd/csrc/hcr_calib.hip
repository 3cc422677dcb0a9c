// Calibration kernels of the BF16 hyper-connection read (libhcr_calib.so, include/hcr_calib.h):
// the read's two launches with nothing in them (HCRC_EMPTY), and with only their global loads
// (HCRC_LOADS).  Measurement only.
//
// The load kernels repeat the index arithmetic of hc_down<T, FMT_BF16> and of the up kernel the read
// dispatches for BF16 weights (hc_up_mfma at every T) in hcr_kernels.hip: the same work-group
// maps (down_stream / down_group, up_tile), lane ownership, load widths, load order and cache policy
// (non-temporal weight loads; hc_up_mfma's weights straight into LDS with 3 waves).  Every loaded register
// is handed to an empty asm statement, so the compiler keeps the load and waits for it, and nothing else is
// done with it.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hcr_calib.h"
#include "hcr_device.h"
#include "hcr_layout.h"
#include "hcr_up.h"

namespace hcr {
namespace {

__device__ __forceinline__ void use(uint32_t v) { asm volatile("" ::"v"(v)); }
__device__ __forceinline__ void use(float v) { asm volatile("" ::"v"(v)); }
__device__ __forceinline__ void use(f32x4 v) {
  use(v[0]), use(v[1]), use(v[2]), use(v[3]);
}
__device__ __forceinline__ void use(uint4 v) { use(v.x), use(v.y), use(v.z), use(v.w); }
__device__ __forceinline__ void use(uint2 v) { use(v.x), use(v.y); }

__global__ void cal_empty() {}

// hc_down<T>'s loads: the stream's x (token groups of 8 from T = 10, the next group's loads issued
// before the current group is consumed), w_norm, then the 5 weight rows
template <int CA, int CB>
struct ColsRaw {
  f32x4 a[CA / 4];
  float b[CB];
  __device__ __forceinline__ void load(const float* p, int ca, int cb) {
#pragma unroll
    for (int e = 0; e < CA / 4; ++e) a[e] = ld4(p + ca + 4 * e);
    if constexpr (CB == 2) {
      const f32x2 v = ld2(p + cb);
      b[0] = v[0], b[1] = v[1];
    } else {
      b[0] = p[cb];
    }
  }
  __device__ __forceinline__ void consume() const {
#pragma unroll
    for (int e = 0; e < CA / 4; ++e) use(a[e]);
#pragma unroll
    for (int e = 0; e < CB; ++e) use(b[e]);
  }
};

template <int T, bool STORE>
__global__ __launch_bounds__(down_threads(T)) void cal_down_loads(const uint16_t* __restrict__ w_down,
                                                                  const float* __restrict__ x,
                                                                  const float* __restrict__ w_norm,
                                                                  float* __restrict__ dst) {
  const int s = down_stream(blockIdx.x), g = down_group(blockIdx.x);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (STORE && tid == 0) dst[blockIdx.x] = 1.0f;  // one store per work-group, before the loads
  constexpr int WAVES = down_waves(T), CA = down_ca(T), CB = down_cb(T);
  const int ca = (2048 / WAVES) * wave + CA * lane;
  const int cb = 2048 + (512 / WAVES) * wave + CB * lane;
  constexpr int TG = T <= 9 ? T : 8;
  constexpr int NG = (T + TG - 1) / TG;
  ColsRaw<CA, CB> xv[TG];
  auto load_x = [&](int grp) {
#pragma unroll
    for (int i = 0; i < TG; ++i) {
      const int t = grp * TG + i;
      if (t < T) xv[i].load(x + ((size_t)t * S + s) * D, ca, cb);
    }
  };
  load_x(0);
  ColsRaw<CA, CB> nv;
  nv.load(w_norm + s * D, ca, cb);
  uint32_t wa[DOWN_ROWS][CA / 2], wb[DOWN_ROWS];
  const uint16_t* wr = w_down + (size_t)(DOWN_ROWS * g) * DD + (size_t)s * D;
#pragma unroll
  for (int r = 0; r < DOWN_ROWS; ++r) {
    if constexpr (CA == 8) {
      const uint4 v = ldw16(wr + (size_t)r * DD + ca);
      wa[r][0] = v.x, wa[r][1] = v.y, wa[r][2] = v.z, wa[r][3] = v.w;
    } else {
      const uint2 v = ldw8(wr + (size_t)r * DD + ca);
      wa[r][0] = v.x, wa[r][1] = v.y;
    }
    wb[r] = CB == 2 ? ldw4(wr + (size_t)r * DD + cb) : ldw2(wr + (size_t)r * DD + cb);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int grp = 0; grp < NG; ++grp) {
#pragma unroll
    for (int i = 0; i < TG; ++i)
      if (grp * TG + i < T) xv[i].consume();
    if (grp == 0) nv.consume();
    if (grp + 1 < NG) load_x(grp + 1);
    __builtin_amdgcn_sched_barrier(0);
    if (grp == 0) {
#pragma unroll
      for (int r = 0; r < DOWN_ROWS; ++r) {
#pragma unroll
        for (int e = 0; e < CA / 2; ++e) use(wa[r][e]);
        use(wb[r]);
      }
    }
  }
}

// hc_up_mfma<T>'s loads: partials, then one 16-row tile of W_up per wave.  The BF16 weights go straight into
// LDS through load_a_lds, the read's own function (10 loads per wave; a 4th wave loads none).
template <int T>
__global__ __launch_bounds__(upm_threads(T, FMT_BF16)) void cal_up_mfma_loads(const uint16_t* __restrict__ w_up,
                                                         const float* __restrict__ part) {
  constexpr int NT = upm_threads(T, FMT_BF16);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c0 = up_tile(blockIdx.x) * UP_COLS;
  static_assert(up_weights_lds(T, FMT_BF16), "the read's BF16 up weights go straight into LDS");
  // the partials first (issued before the weights, consumed after them, as in the read)
  constexpr int ITEMS = T * (R / 4);
  constexpr int NI = (ITEMS + NT - 1) / NT;
  f32x4 pv[NI][S];
#pragma unroll
  for (int n = 0; n < NI; ++n) {
    const int it = min(tid + n * NT, ITEMS - 1);
    const int t = it / (R / 4), k = 4 * (it % (R / 4));
#pragma unroll
    for (int ss = 0; ss < S; ++ss)
      pv[n][ss] = ld4_untracked(part + ((size_t)ss * TMAX + t) * R + k);
  }
  __builtin_amdgcn_sched_barrier(0);
  constexpr int A_REGION = 10 * A_LOAD_STRIDE;
  __shared__ __attribute__((aligned(16))) unsigned char a_sm[3 * A_REGION];
  if (NT == 192 || wave < 3) load_a_lds<A_REGION>(w_up, lds_addr(a_sm), __builtin_amdgcn_readfirstlane(wave), lane, c0);
  vm_wait<0>();
#pragma unroll
  for (int n = 0; n < NI; ++n)
#pragma unroll
    for (int ss = 0; ss < S; ++ss) vm_pin(pv[n][ss]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int n = 0; n < NI; ++n)
#pragma unroll
    for (int ss = 0; ss < S; ++ss) use(pv[n][ss]);
}

// ---- the pages' down-kernel shape and finish, as loads (and stores, and the finish) only
// slab scratch: partials [8 slabs][TMAX][R] at 0, sums of squares [8][TMAX] at SLAB_OFF_SS, counters [32 row
// groups] at SLAB_OFF_CTR, lo [TMAX][R] at SLAB_OFF_LO
constexpr int SLABS = 8, SLAB_COLS = DD / SLABS, SLAB_ROWS = 10, SLAB_GROUPS = R / SLAB_ROWS;
constexpr size_t SLAB_OFF_SS = size_t(SLABS) * TMAX * R * 4;
constexpr size_t SLAB_OFF_CTR = SLAB_OFF_SS + size_t(SLABS) * TMAX * 4 + 256;
constexpr size_t SLAB_OFF_LO = SLAB_OFF_CTR + 256;
static_assert(SLAB_COLS == 1280 && SLABS * SLAB_GROUPS == 256 && SLAB_COLS == 256 * 4 + 256 &&
                  SLAB_OFF_LO + size_t(TMAX) * R * 4 <= HCRC_SLAB_SCRATCH_BYTES,
              "8 slabs x 32 row groups of 10 rows; lanes own 4 + 1 columns; the slab scratch holds everything");

template <int T, int KIND>
__global__ __launch_bounds__(256) void cal_slab_down(const uint16_t* __restrict__ w_down, const float* __restrict__ x,
                                                     const float* __restrict__ w_norm, char* scratch) {
  const int b = blockIdx.x;
  const int sl = (b / XCDS) % SLABS, g = b % XCDS + XCDS * (b / (XCDS * SLABS));  // XCD b % 8 = row group % 8
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ca = sl * SLAB_COLS + 256 * wave + 4 * lane, cb = sl * SLAB_COLS + 1024 + 64 * wave + lane;
  float* part = reinterpret_cast<float*>(scratch);
  float* ssb = reinterpret_cast<float*>(scratch + SLAB_OFF_SS);
  unsigned* ctr = reinterpret_cast<unsigned*>(scratch + SLAB_OFF_CTR);
  float* lo = reinterpret_cast<float*>(scratch + SLAB_OFF_LO);
  f32x4 xa[T];
  float xb[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    xa[t] = ld4(x + (size_t)t * DD + ca);
    xb[t] = x[(size_t)t * DD + cb];
  }
  const f32x4 na = ld4(w_norm + ca);
  const float nb = w_norm[cb];
  uint2 wa[SLAB_ROWS];
  uint32_t wb[SLAB_ROWS];
#pragma unroll
  for (int r = 0; r < SLAB_ROWS; ++r) {
    wa[r] = ldw8(w_down + (size_t)(SLAB_ROWS * g + r) * DD + ca);
    wb[r] = ldw2(w_down + (size_t)(SLAB_ROWS * g + r) * DD + cb);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < T; ++t) use(xa[t]), use(xb[t]);
  use(na), use(nb);
#pragma unroll
  for (int r = 0; r < SLAB_ROWS; ++r) use(wa[r]), use(wb[r]);
  if constexpr (KIND == HCRC_SLAB_LOADS) return;
  // the work-group's 10 T partials and T sums of squares, one per thread (values arbitrary)
  if (tid < SLAB_ROWS * T)
    part[((size_t)sl * TMAX + tid / SLAB_ROWS) * R + SLAB_ROWS * g + tid % SLAB_ROWS] = (float)tid;
  else if (tid < (SLAB_ROWS + 1) * T)
    ssb[sl * TMAX + tid - SLAB_ROWS * T] = 1.0f;
  if constexpr (KIND == HCRC_SLAB_FINISH) {
    __shared__ int last;
    __syncthreads();  // every thread's stores precede thread 0's release
    if (tid == 0) {
      const unsigned old = __hip_atomic_fetch_add(ctr + g, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      last = old == SLABS - 1;
    }
    __syncthreads();
    if (last) {  // the 8th work-group of the row group: lo of its 10 rows, then the counter back to zero
      if (tid < SLAB_ROWS * T) {
        const int t = tid / SLAB_ROWS, r = SLAB_ROWS * g + tid % SLAB_ROWS;
        float a = 0.f;
#pragma unroll
        for (int q = 0; q < SLABS; ++q) a += part[((size_t)q * TMAX + t) * R + r] * ssb[q * TMAX + t];
        lo[t * R + r] = a;
      }
      if (tid == 0) __hip_atomic_store(ctr + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// the up grid of the read (hc_up_mfma's lanes and W_up tile) loading lo, T x R floats, instead of 4 partials
template <int T>
__global__ __launch_bounds__(upm_threads(T < 2 ? 2 : T, FMT_BF16)) void cal_slab_up(const uint16_t* __restrict__ w_up, const char* scratch) {
  constexpr int NT = upm_threads(T < 2 ? 2 : T, FMT_BF16);
  const float* lo = reinterpret_cast<const float*>(scratch + SLAB_OFF_LO);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c0 = up_tile(blockIdx.x) * UP_COLS;
  const int li = lane & 15, lg = lane >> 4;
  const int rw = min(16 * min(wave, 2) + li, UP_ROWS - 1);
  const size_t j = (size_t)(rw & 3) * D + c0 + (rw >> 2);
  constexpr int ITEMS = T * (R / 4);
  constexpr int NI = (ITEMS + NT - 1) / NT;
  f32x4 pv[NI];
#pragma unroll
  for (int n = 0; n < NI; ++n) pv[n] = ld4(lo + 4 * min(tid + n * NT, ITEMS - 1));
  __builtin_amdgcn_sched_barrier(0);
  uint4 a[R / 32];
#pragma unroll
  for (int m = 0; m < R / 32; ++m) a[m] = ldw16(w_up + j * R + 32 * m + 8 * lg);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int n = 0; n < NI; ++n) use(pv[n]);
#pragma unroll
  for (int m = 0; m < R / 32; ++m) use(a[m]);
}

// ---- the pages' read with its arithmetic (hcrc_slab_read): the slab down kernel computes a = x * w_norm
// (unscaled), the slab's sums of squares and its 10 rows' partials; the last work-group of a row group to
// arrive applies rs per stream, adds the injection, writes lo (and rs) and resets the counter; the read's own
// up kernel then reads lo alone (NSRC = 1).  Scratch: the slab layout above, plus rs [TMAX][S] and a region
// that takes the up kernel's copy of lo (unused here).
constexpr size_t SLAB_OFF_RS = SLAB_OFF_LO + size_t(TMAX) * R * 4;
constexpr size_t SLAB_OFF_JUNK = SLAB_OFF_RS + size_t(TMAX) * S * 4;
static_assert(SLAB_OFF_JUNK + size_t(TMAX) * R * 4 <= HCRC_SLAB_SCRATCH_BYTES && SLAB_OFF_LO == HCRC_SLAB_OFF_LO &&
                  SLAB_OFF_RS == HCRC_SLAB_OFF_RS,
              "the slab scratch holds the read too, at the offsets the header states");

template <int T, bool INJ>
__global__ __launch_bounds__(256) void cal_slab_read_down(const uint16_t* __restrict__ w_down, const float* __restrict__ x,
                                                          const float* __restrict__ w_norm, const float* __restrict__ inj,
                                                          char* scratch) {
  const int b = blockIdx.x;
  const int sl = (b / XCDS) % SLABS, g = b % XCDS + XCDS * (b / (XCDS * SLABS));  // as cal_slab_down
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ca = sl * SLAB_COLS + 256 * wave + 4 * lane, cb = sl * SLAB_COLS + 1024 + 64 * wave + lane;
  float* part = reinterpret_cast<float*>(scratch);
  float* ssb = reinterpret_cast<float*>(scratch + SLAB_OFF_SS);
  unsigned* ctr = reinterpret_cast<unsigned*>(scratch + SLAB_OFF_CTR);
  float* lo = reinterpret_cast<float*>(scratch + SLAB_OFF_LO);
  float* rs_out = reinterpret_cast<float*>(scratch + SLAB_OFF_RS);
  // loads: x of the T tokens and w_norm at the lane's 4 + 1 columns, then the 10 weight rows
  f32x4 xa[T];
  float xb[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    xa[t] = ld4(x + (size_t)t * DD + ca);
    xb[t] = x[(size_t)t * DD + cb];
  }
  const f32x4 na = ld4(w_norm + ca);
  const float nb = w_norm[cb];
  uint2 wa[SLAB_ROWS];
  uint32_t wb[SLAB_ROWS];
#pragma unroll
  for (int r = 0; r < SLAB_ROWS; ++r) {
    wa[r] = ldw8(w_down + (size_t)(SLAB_ROWS * g + r) * DD + ca);
    wb[r] = ldw2(w_down + (size_t)(SLAB_ROWS * g + r) * DD + cb);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_sched_barrier(0);
  // the lane's values: the T sums of squares (value t), then row r, token t (value T + r T + t)
  constexpr int NV = (SLAB_ROWS + 1) * T, N = round4(NV);
  float v[N];
#pragma unroll
  for (int k = NV; k < N; ++k) v[k] = 0.f;
  float act[T][5];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      act[t][e] = xa[t][e] * na[e];
      ss = __builtin_fmaf(xa[t][e], xa[t][e], ss);
    }
    act[t][4] = xb[t] * nb;
    v[t] = __builtin_fmaf(xb[t], xb[t], ss);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < SLAB_ROWS; ++r) {
    const float wv[5] = {__uint_as_float(wa[r].x << 16), __uint_as_float(wa[r].x & 0xffff0000u),
                         __uint_as_float(wa[r].y << 16), __uint_as_float(wa[r].y & 0xffff0000u),
                         __uint_as_float(wb[r] << 16)};
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 5; ++e) acc = __builtin_fmaf(wv[e], act[t][e], acc);
      v[T + r * T + t] = acc;
    }
  }
  // sums over the wave, then over the 4 waves in a fixed order; the slab's unscaled partials and its sums
  // of squares go to the scratch
  wave_sum<N>(v);
  __shared__ float wsum[4][N];
  if ((lane & 15) == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) wsum[wave][(lane >> 4) * (N / 4) + i] = v[i];
  }
  __syncthreads();
  if (tid < NV) {
    const float a = ((wsum[0][tid] + wsum[1][tid]) + wsum[2][tid]) + wsum[3][tid];
    if (tid < T)
      ssb[sl * TMAX + tid] = a;
    else
      part[((size_t)sl * TMAX + (tid - T) % T) * R + SLAB_ROWS * g + (tid - T) / T] = a;
  }
  // the finish: one agent-scope acquire-release arrival per work-group (every thread's stores precede it
  // through the barrier); the 8th work-group of the row group reads the 8 slabs, nobody waits
  __shared__ int last;
  __syncthreads();
  if (tid == 0) {
    const unsigned old = __hip_atomic_fetch_add(ctr + g, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    last = old == SLABS - 1;
  }
  __syncthreads();
  if (!last) return;
  // rs[t][s] = 1 / sqrt((ss of the stream's 2 slabs) / D + 1e-6); lo[t][r] = sum_s rs * (its 2 slab partials)
  // (+ inj), streams in order
  if (tid < SLAB_ROWS * T) {
    const int t = tid / SLAB_ROWS, r = SLAB_ROWS * g + tid % SLAB_ROWS;
    float acc = 0.f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const float ms = (ssb[(2 * s) * TMAX + t] + ssb[(2 * s + 1) * TMAX + t]) * (1.0f / D);
      const float rs = 1.0f / sqrtf(ms + 1e-6f);
      acc = __builtin_fmaf(rs, part[((size_t)(2 * s) * TMAX + t) * R + r] + part[((size_t)(2 * s + 1) * TMAX + t) * R + r], acc);
    }
    if (INJ) acc += inj[(size_t)t * R + r];
    lo[(size_t)t * R + r] = acc;
  }
  if (g == 0 && tid < S * T) {
    const int t = tid / S, s = tid % S;
    const float ms = (ssb[(2 * s) * TMAX + t] + ssb[(2 * s + 1) * TMAX + t]) * (1.0f / D);
    rs_out[t * S + s] = 1.0f / sqrtf(ms + 1e-6f);
  }
  if (tid == 0) __hip_atomic_store(ctr + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// the read's up kernel on lo alone (its staging reads one source: NSRC = 1); the injection is already in lo
template <int T, bool PEND>
__global__ __launch_bounds__(upm_threads(T, FMT_BF16)) void cal_slab_read_up(const void* w_up, const float* lo,
                                                                             const float* pending, float* out,
                                                                             float* mean, float* junk) {
  hc_up_mfma_body<T, false, PEND, FMT_BF16, 1>(w_up, nullptr, lo, nullptr, pending, out, mean, junk);
}

typedef void (*slab_read_down_fn)(const uint16_t*, const float*, const float*, const float*, char*);
typedef void (*slab_read_up_fn)(const void*, const float*, const float*, float*, float*, float*);
#define HCRC_SRD(T) {cal_slab_read_down<T, false>, cal_slab_read_down<T, true>}
const slab_read_down_fn kSlabReadDown[8][2] = {HCRC_SRD(1), HCRC_SRD(2), HCRC_SRD(3), HCRC_SRD(4),
                                               HCRC_SRD(5), HCRC_SRD(6), HCRC_SRD(7), HCRC_SRD(8)};
#undef HCRC_SRD
#define HCRC_SRU(T) {cal_slab_read_up<T, false>, cal_slab_read_up<T, true>}
const slab_read_up_fn kSlabReadUp[8][2] = {HCRC_SRU(1), HCRC_SRU(2), HCRC_SRU(3), HCRC_SRU(4),
                                           HCRC_SRU(5), HCRC_SRU(6), HCRC_SRU(7), HCRC_SRU(8)};
#undef HCRC_SRU

typedef void (*slab_down_fn)(const uint16_t*, const float*, const float*, char*);
typedef void (*slab_up_fn)(const uint16_t*, const char*);
#define HCRC_SLAB_ROW(K) {cal_slab_down<1, K>, cal_slab_down<2, K>, cal_slab_down<3, K>, cal_slab_down<4, K>, \
                          cal_slab_down<5, K>, cal_slab_down<6, K>, cal_slab_down<7, K>, cal_slab_down<8, K>}
const slab_down_fn kSlabDown[3][8] = {HCRC_SLAB_ROW(HCRC_SLAB_LOADS), HCRC_SLAB_ROW(HCRC_SLAB_STORES),
                                      HCRC_SLAB_ROW(HCRC_SLAB_FINISH)};
#undef HCRC_SLAB_ROW
const slab_up_fn kSlabUp[8] = {cal_slab_up<1>, cal_slab_up<2>, cal_slab_up<3>, cal_slab_up<4>,
                               cal_slab_up<5>, cal_slab_up<6>, cal_slab_up<7>, cal_slab_up<8>};

typedef void (*cal_down_fn)(const uint16_t*, const float*, const float*, float*);
typedef void (*cal_up_fn)(const uint16_t*, const float*);
static_assert(TMAX == 16, "the tables below list T = 1..16");
#define HCRC_DOWN_ROW(F)                                                                                       \
  {cal_down_loads<1, F>,  cal_down_loads<2, F>,  cal_down_loads<3, F>,  cal_down_loads<4, F>,  cal_down_loads<5, F>,  \
   cal_down_loads<6, F>,  cal_down_loads<7, F>,  cal_down_loads<8, F>,  cal_down_loads<9, F>,  cal_down_loads<10, F>, \
   cal_down_loads<11, F>, cal_down_loads<12, F>, cal_down_loads<13, F>, cal_down_loads<14, F>, cal_down_loads<15, F>, \
   cal_down_loads<16, F>}
const cal_down_fn kCalDown[2][TMAX] = {HCRC_DOWN_ROW(false), HCRC_DOWN_ROW(true)};
#undef HCRC_DOWN_ROW
const cal_up_fn kCalUp[TMAX] = {cal_up_mfma_loads<1>,   cal_up_mfma_loads<2>,  cal_up_mfma_loads<3>,
                                cal_up_mfma_loads<4>,   cal_up_mfma_loads<5>,  cal_up_mfma_loads<6>,
                                cal_up_mfma_loads<7>,   cal_up_mfma_loads<8>,  cal_up_mfma_loads<9>,
                                cal_up_mfma_loads<10>,  cal_up_mfma_loads<11>, cal_up_mfma_loads<12>,
                                cal_up_mfma_loads<13>,  cal_up_mfma_loads<14>, cal_up_mfma_loads<15>,
                                cal_up_mfma_loads<16>};
static_assert(UP_MFMA_FROM == 1, "the read dispatches hc_up_mfma at every T for BF16 weights");

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

typedef void (*up_fn)(const void*, const uint16_t*, const float*, const float*, const float*, float*, float*,
                      float*);
// the read's two up kernels under names of their own (the same bodies, BF16 weights, no pending write or
// injection), so that a kernel trace tells them from the read's dispatches
template <int T>
__global__ __launch_bounds__(UP_THREADS) void cal_up_valu(const void* w_up, const uint16_t* s_up, const float* part,
                                                          const float* inj, const float* pending, float* out,
                                                          float* mean, float* lo_out) {
  hc_up_body<T, false, false, FMT_BF16>(w_up, s_up, part, inj, pending, out, mean, lo_out);
}
template <int T>
__global__ __launch_bounds__(upm_threads(T, FMT_BF16)) void cal_up_mfma(const void* w_up, const uint16_t* s_up, const float* part,
                                                   const float* inj, const float* pending, float* out, float* mean,
                                                   float* lo_out) {
  hc_up_mfma_body<T, false, false, FMT_BF16>(w_up, s_up, part, inj, pending, out, mean, lo_out);
}
#define HCRC_UP_T(K, T) K<T>
const up_fn kUpValu[TMAX] = {HCRC_UP_T(cal_up_valu, 1),  HCRC_UP_T(cal_up_valu, 2),  HCRC_UP_T(cal_up_valu, 3),  HCRC_UP_T(cal_up_valu, 4),
                             HCRC_UP_T(cal_up_valu, 5),  HCRC_UP_T(cal_up_valu, 6),  HCRC_UP_T(cal_up_valu, 7),  HCRC_UP_T(cal_up_valu, 8),
                             HCRC_UP_T(cal_up_valu, 9),  HCRC_UP_T(cal_up_valu, 10), HCRC_UP_T(cal_up_valu, 11), HCRC_UP_T(cal_up_valu, 12),
                             HCRC_UP_T(cal_up_valu, 13), HCRC_UP_T(cal_up_valu, 14), HCRC_UP_T(cal_up_valu, 15), HCRC_UP_T(cal_up_valu, 16)};
const up_fn kUpMfma[TMAX] = {
    HCRC_UP_T(cal_up_mfma, 1),  HCRC_UP_T(cal_up_mfma, 2),  HCRC_UP_T(cal_up_mfma, 3),  HCRC_UP_T(cal_up_mfma, 4),
    HCRC_UP_T(cal_up_mfma, 5),  HCRC_UP_T(cal_up_mfma, 6),  HCRC_UP_T(cal_up_mfma, 7),  HCRC_UP_T(cal_up_mfma, 8),
    HCRC_UP_T(cal_up_mfma, 9),  HCRC_UP_T(cal_up_mfma, 10), HCRC_UP_T(cal_up_mfma, 11), HCRC_UP_T(cal_up_mfma, 12),
    HCRC_UP_T(cal_up_mfma, 13), HCRC_UP_T(cal_up_mfma, 14), HCRC_UP_T(cal_up_mfma, 15), HCRC_UP_T(cal_up_mfma, 16)};
#undef HCRC_UP_T

}  // namespace
}  // namespace hcr

extern "C" int hcrc_read_floor(int kind, int T, const void* w_down, const void* w_up, const float* w_norm,
                               void* scratch, const float* x, void* stream) {
  using namespace hcr;
  if ((kind != HCRC_EMPTY && kind != HCRC_LOADS && kind != HCRC_LOADS_STORE) || T < 1 || T > TMAX) return HCR_EINVAL;
  if (kind != HCRC_EMPTY) {
    if (!w_down || !w_up || !w_norm || !scratch || !x) return HCR_EINVAL;
    if (!aligned(w_down, 16) || !aligned(w_up, 16) || !aligned(w_norm, 16) || !aligned(scratch, 256) ||
        !aligned(x, 16))
      return HCR_EALIGN;
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const unsigned up_threads = T >= UP_MFMA_FROM ? upm_threads(T, FMT_BF16) : UP_THREADS;
  (void)hipGetLastError();
  if (kind == HCRC_EMPTY) {
    hipLaunchKernelGGL(cal_empty, dim3(DOWN_WGS), dim3(down_threads(T)), 0, st);
    hipLaunchKernelGGL(cal_empty, dim3(UP_WGS), dim3(up_threads), 0, st);
  } else {
    const float* part = reinterpret_cast<const float*>(static_cast<const char*>(scratch) + OFF_PART);
    float* lo = reinterpret_cast<float*>(static_cast<char*>(scratch) + OFF_LO);
    static_assert(DOWN_WGS <= TMAX * R, "one store per down work-group fits the lo slot");
    hipLaunchKernelGGL(kCalDown[kind == HCRC_LOADS_STORE][T - 1], dim3(DOWN_WGS), dim3(down_threads(T)), 0, st,
                       static_cast<const uint16_t*>(w_down), x, w_norm, lo);
    hipLaunchKernelGGL(kCalUp[T - 1], dim3(UP_WGS), dim3(up_threads), 0, st, static_cast<const uint16_t*>(w_up),
                       part);
  }
  return hipGetLastError() == hipSuccess ? HCR_OK : HCR_EHIP;
}

extern "C" int hcrc_up_kernel(int kind, int T, const void* w_up, void* scratch, float* out, float* mean,
                              void* stream) {
  using namespace hcr;
  if ((kind != HCRC_UP_VALU && kind != HCRC_UP_MFMA) || T < 1 || T > TMAX) return HCR_EINVAL;
  if (!w_up || !scratch || !out || !mean) return HCR_EINVAL;
  if (!aligned(w_up, 16) || !aligned(scratch, 256) || !aligned(out, 16) || !aligned(mean, 16)) return HCR_EALIGN;
  char* sc = static_cast<char*>(scratch);
  const float* part = reinterpret_cast<const float*>(sc + OFF_PART);
  float* lo = reinterpret_cast<float*>(sc + OFF_LO);
  (void)hipGetLastError();
  if (kind == HCRC_UP_VALU)
    hipLaunchKernelGGL(kUpValu[T - 1], dim3(UP_WGS), dim3(UP_THREADS), 0, reinterpret_cast<hipStream_t>(stream), w_up,
                       nullptr, part, nullptr, nullptr, out, mean, lo);
  else
    hipLaunchKernelGGL(kUpMfma[T - 1], dim3(UP_WGS), dim3(upm_threads(T, FMT_BF16)), 0, reinterpret_cast<hipStream_t>(stream),
                       w_up, nullptr, part, nullptr, nullptr, out, mean, lo);
  return hipGetLastError() == hipSuccess ? HCR_OK : HCR_EHIP;
}

extern "C" int hcrc_slab_pair(int kind, int T, const void* w_down, const void* w_up, const float* w_norm,
                              void* slab_scratch, const float* x, void* stream) {
  using namespace hcr;
  if ((kind != HCRC_SLAB_LOADS && kind != HCRC_SLAB_STORES && kind != HCRC_SLAB_FINISH) || T < 1 || T > 8)
    return HCR_EINVAL;
  if (!w_down || !w_up || !w_norm || !slab_scratch || !x) return HCR_EINVAL;
  if (!aligned(w_down, 16) || !aligned(w_up, 16) || !aligned(w_norm, 16) || !aligned(slab_scratch, 256) ||
      !aligned(x, 16))
    return HCR_EALIGN;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* sc = static_cast<char*>(slab_scratch);
  (void)hipGetLastError();
  hipLaunchKernelGGL(kSlabDown[kind][T - 1], dim3(SLABS * SLAB_GROUPS), dim3(256), 0, st,
                     static_cast<const uint16_t*>(w_down), x, w_norm, sc);
  hipLaunchKernelGGL(kSlabUp[T - 1], dim3(UP_WGS), dim3(upm_threads(T < 2 ? 2 : T, FMT_BF16)), 0, st,
                     static_cast<const uint16_t*>(w_up), static_cast<const char*>(sc));
  return hipGetLastError() == hipSuccess ? HCR_OK : HCR_EHIP;
}

extern "C" int hcrc_slab_read(int T, const void* w_down, const void* w_up, const float* w_norm, void* slab_scratch,
                              const float* x, const float* pending, const float* inj, float* out, float* mean,
                              void* stream) {
  using namespace hcr;
  if (T < 1 || T > 8) return HCR_EINVAL;
  if (!w_down || !w_up || !w_norm || !slab_scratch || !x || !out || !mean) return HCR_EINVAL;
  if (!aligned(w_down, 16) || !aligned(w_up, 16) || !aligned(w_norm, 16) || !aligned(slab_scratch, 256) ||
      !aligned(x, 16) || !aligned(out, 16) || !aligned(mean, 16) || (pending && !aligned(pending, 16)) ||
      (inj && !aligned(inj, 16)))
    return HCR_EALIGN;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* sc = static_cast<char*>(slab_scratch);
  (void)hipGetLastError();
  hipLaunchKernelGGL(kSlabReadDown[T - 1][inj != nullptr], dim3(SLABS * SLAB_GROUPS), dim3(256), 0, st,
                     static_cast<const uint16_t*>(w_down), x, w_norm, inj, sc);
  hipLaunchKernelGGL(kSlabReadUp[T - 1][pending != nullptr], dim3(UP_WGS), dim3(upm_threads(T, FMT_BF16)), 0, st,
                     w_up, reinterpret_cast<const float*>(sc + SLAB_OFF_LO), pending, out, mean,
                     reinterpret_cast<float*>(sc + SLAB_OFF_JUNK));
  return hipGetLastError() == hipSuccess ? HCR_OK : HCR_EHIP;
}
