// Device helpers shared by the HIP kernels of this library (gfx950, wave64):
// vector types, exact BF16 / binary16 / int8 widening, the BF16 high/low split,
// DPP lane moves and the fixed-order multi-value wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hcr {

typedef __attribute__((ext_vector_type(4))) float f32x4;

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

// byte k of u as a signed 8-bit code, widened exactly to FP32
__device__ __forceinline__ float code(uint32_t u, int k) {
  return static_cast<float>(static_cast<int8_t>(static_cast<uint8_t>(u >> (8 * k))));
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
// the same split of 4 values
__device__ __forceinline__ void split_hi_lo4(const f32x4& v, uint2& hi, uint2& lo) {
  uint32_t h[2], l[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const f32x2 a = {v[2 * e], v[2 * e + 1]};
    const bf16x2 bh = __builtin_convertvector(a, bf16x2);
    const f32x2 r = a - __builtin_convertvector(bh, f32x2);  // exact
    const bf16x2 bl = __builtin_convertvector(r, bf16x2);
    h[e] = __builtin_bit_cast(uint32_t, bh);
    l[e] = __builtin_bit_cast(uint32_t, bl);
  }
  hi = make_uint2(h[0], h[1]);
  lo = make_uint2(l[0], l[1]);
}

__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// Weight loads: every weight is read once per call, so the loads are non-temporal (the nt bit).  Measured on
// MI355X (cold BF16 read, one process, alternating with ordinary loads): 0.26-0.33 us faster per read on the
// mean over T = 1..8 on two boxes (on a third only T = 1 gained, 0.29 us), 10 % for the skinny matvec.
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
__device__ __forceinline__ uint4 ldw16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ldw8(const void* p) {
  const u32x2_t v = __builtin_nontemporal_load(static_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t ldw4(const void* p) { return __builtin_nontemporal_load(static_cast<const uint32_t*>(p)); }
__device__ __forceinline__ uint32_t ldw2(const void* p) { return __builtin_nontemporal_load(static_cast<const uint16_t*>(p)); }
__device__ __forceinline__ uint32_t ldw1(const void* p) { return __builtin_nontemporal_load(static_cast<const uint8_t*>(p)); }

// Loads whose completion the compiler does not track, for a kernel that waits for them itself (vm_wait).
// The compiler's wait insertion gives up on in-order completion as soon as a load straight into LDS is in
// flight: the first use of any older load then waits for every load, LDS ones included.  A kernel that
// streams its weights into LDS while it works on earlier loads issues all of its vector-memory loads
// through these instead, in a fixed order and number, and places each wait itself (vmcnt counts loads in
// issue order: vmcnt(n) leaves only the n youngest in flight).  The results are plain asm outputs: a caller
// pins them (vm_pin) after the wait that covers them, so that no use moves above it.
__device__ __forceinline__ f32x4 ld4_untracked(const float* p) {
  f32x4 v;
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}
__device__ __forceinline__ float ld1_untracked(const float* p) {
  float v;
  asm volatile("global_load_dword %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}
// A non-temporal 16-byte load straight into LDS (global_load_lds_dwordx4, no registers): lane l's 16 bytes
// land at LDS byte address lds + 16 l; lds is one value for the whole wave, passed in M0 (an input of the asm,
// so the compiler sets M0 and knows it; the load needs one wait state after that write).
__device__ __forceinline__ void ldw16_lds_untracked(const void* p, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(p), "{m0}"(lds) : "memory");
}
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
// vm_wait<n> for an n that is a constant only after unrolling (0 <= n <= 15)
__device__ __forceinline__ void vm_wait_n(int n) {
  switch (n) {
    case 0: vm_wait<0>(); break;   case 1: vm_wait<1>(); break;   case 2: vm_wait<2>(); break;
    case 3: vm_wait<3>(); break;   case 4: vm_wait<4>(); break;   case 5: vm_wait<5>(); break;
    case 6: vm_wait<6>(); break;   case 7: vm_wait<7>(); break;   case 8: vm_wait<8>(); break;
    case 9: vm_wait<9>(); break;   case 10: vm_wait<10>(); break; case 11: vm_wait<11>(); break;
    case 12: vm_wait<12>(); break; case 13: vm_wait<13>(); break; case 14: vm_wait<14>(); break;
    default: vm_wait<0>(); break;  // n > 14: the strictest wait
  }
}
template <typename V>
__device__ __forceinline__ void vm_pin(V& v) { asm volatile("" : "+v"(v)); }
// the LDS byte address of a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p));
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2v;

__device__ __forceinline__ f32x2 ld2(const float* p) { return *reinterpret_cast<const f32x2*>(p); }

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum N values per lane over the 64 lanes of a wave (N a multiple of 4).  Two
// halving steps (v_permlane32_swap, v_permlane16_swap) then a butterfly inside
// each row of 16 lanes; afterwards every lane l holds, in v[0 .. N/4), the
// totals of values (l >> 4) * N/4 + i.  The order of the additions is fixed.
//
// The steps of value i touch only the quadruple of positions i mod N/4 + {0, 1, 2, 3} * N/4, and every value
// meets the same lane pairings (l ^ 32, l ^ 16, then the butterfly), so its total does not depend on its
// position: wave_quad_sum reduces one quadruple, and a caller may reduce the quadruples in any order (for
// instance each as soon as its four values are known) with the same results as wave_sum.
template <int N>
__device__ __forceinline__ void wave_quad_sum(float (&v)[N], int q) {
  static_assert(N % 4 == 0, "wave_sum needs a multiple of 4 values");
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = q + h * (N / 4);
    const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + N / 2]), false, false);
    v[i] = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);  // lanes < 32: value i; lanes >= 32: value i + N/2
  }
  const auto pr = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[q]), __float_as_uint(v[q + N / 4]), false, false);
  v[q] = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);  // even rows: value q; odd rows: value q + N/4
  v[q] += dpp<0xB1>(v[q]);   // quad_perm [1,0,3,2]
  v[q] += dpp<0x4E>(v[q]);   // quad_perm [2,3,0,1]
  v[q] += dpp<0x141>(v[q]);  // row_half_mirror
  v[q] += dpp<0x140>(v[q]);  // row_mirror
}

template <int N>
__device__ __forceinline__ void wave_sum(float (&v)[N]) {
#pragma unroll
  for (int q = 0; q < N / 4; ++q) wave_quad_sum<N>(v, q);
}

// Position in a wave_sum array of N values of the k-th value in the order the values become known: the
// k-th value goes to quadruple k / 4, so that values known early complete their quadruples early.
constexpr int quad_pos(int k, int n) { return k / 4 + (k % 4) * (n / 4); }
constexpr bool quad_pos_ok() {  // a permutation of 0 .. n - 1 that puts value k in quadruple k / 4
  for (int n = 4; n <= 128; n += 4) {
    bool seen[128] = {};
    for (int k = 0; k < n; ++k) {
      const int p = quad_pos(k, n);
      if (p < 0 || p >= n || seen[p] || p % (n / 4) != k / 4) return false;
      seen[p] = true;
    }
  }
  return true;
}
static_assert(quad_pos_ok(), "quad_pos must permute the positions by quadruple");

constexpr int round4(int n) { return (n + 3) & ~3; }

// Sum N values per lane over the 32 lanes of each half-wave (N even): one halving
// step (v_permlane16_swap) then a butterfly inside each row of 16 lanes.  Lanes
// of row (l >> 4) & 1 then hold, in v[0 .. N/2), the half-wave totals of values
// ((l >> 4) & 1) * N/2 + i.
template <int N>
__device__ __forceinline__ void half_wave_sum(float (&v)[N]) {
  static_assert(N % 2 == 0, "half_wave_sum needs an even number of values");
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const auto pr = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + N / 2]), false, false);
    v[i] = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
  }
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    v[i] += dpp<0xB1>(v[i]);
    v[i] += dpp<0x4E>(v[i]);
    v[i] += dpp<0x141>(v[i]);
    v[i] += dpp<0x140>(v[i]);
  }
}

constexpr int round2(int n) { return (n + 1) & ~1; }

}  // namespace hcr
