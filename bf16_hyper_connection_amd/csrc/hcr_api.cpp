// C ABI of the BF16 hyper-connection read: argument validation and the handle.
// Every check runs on the host before any HIP call.

#include <stdint.h>
#include <stdlib.h>

#include "hcr_layout.h"

struct hcr_handle {
  const void* w_down;
  const void* w_up;
  const float* w_norm;
  void* scratch;
};

namespace {

struct Span {
  uintptr_t lo, hi;  // [lo, hi)
  bool present() const { return hi > lo; }
};

Span span(const void* p, size_t bytes) {
  uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return p ? Span{a, a + bytes} : Span{0, 0};
}

bool overlap(Span a, Span b) { return a.present() && b.present() && a.lo < b.hi && b.lo < a.hi; }
bool same(Span a, Span b) { return a.present() && a.lo == b.lo && a.hi == b.hi; }
bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

constexpr size_t W_BYTES = size_t(hcr::R) * hcr::DD * 2;  // each projection, BF16
constexpr size_t WNORM_BYTES = size_t(hcr::S) * hcr::D * 4;

}  // namespace

extern "C" {

size_t hcr_scratch_bytes(void) { return hcr::SCRATCH_BYTES; }

int hcr_scratch_layout(size_t* lo_offset, size_t* rs_offset) {
  if (!lo_offset || !rs_offset) return HCR_EINVAL;
  *lo_offset = hcr::OFF_LO;
  *rs_offset = hcr::OFF_RS;
  return HCR_OK;
}

int hcr_geometry(int* streams, int* stream_d, int* rank, int* t_max) {
  if (streams) *streams = hcr::S;
  if (stream_d) *stream_d = hcr::D;
  if (rank) *rank = hcr::R;
  if (t_max) *t_max = hcr::TMAX;
  return HCR_OK;
}

int hcr_create(const void* w_down, const void* w_up, const float* w_norm, void* scratch, size_t scratch_bytes,
               hcr_t* out) {
  if (!out) return HCR_EINVAL;
  *out = nullptr;
  if (!w_down || !w_up || !w_norm || !scratch) return HCR_EINVAL;
  if (!aligned(w_down, 16) || !aligned(w_up, 16) || !aligned(w_norm, 16) || !aligned(scratch, 256))
    return HCR_EALIGN;
  if (scratch_bytes < hcr::SCRATCH_BYTES) return HCR_ESCRATCH;
  const Span sc = span(scratch, hcr::SCRATCH_BYTES);
  if (overlap(sc, span(w_down, W_BYTES)) || overlap(sc, span(w_up, W_BYTES)) ||
      overlap(sc, span(w_norm, WNORM_BYTES)))
    return HCR_EALIAS;
  hcr_handle* h = static_cast<hcr_handle*>(malloc(sizeof(hcr_handle)));
  if (!h) return HCR_EINVAL;
  h->w_down = w_down;
  h->w_up = w_up;
  h->w_norm = w_norm;
  h->scratch = scratch;
  *out = h;
  return HCR_OK;
}

int hcr_read(hcr_t h, int T, const float* x, const float* pending, const float* inj, float* out, float* mean,
             void* stream) {
  if (!h || T < 0 || T > hcr::TMAX) return HCR_EINVAL;
  if (T == 0) return HCR_OK;
  if (!x || !out || !mean) return HCR_EINVAL;
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(mean, 16) || (pending && !aligned(pending, 16)) ||
      (inj && !aligned(inj, 16)))
    return HCR_EALIGN;

  const size_t stream_bytes = size_t(T) * hcr::S * hcr::D * 4;
  const Span sx = span(x, stream_bytes), sp = span(pending, stream_bytes), so = span(out, stream_bytes);
  const Span sm = span(mean, size_t(T) * hcr::D * 4), si = span(inj, size_t(T) * hcr::R * 4);
  const Span sc = span(h->scratch, hcr::SCRATCH_BYTES);
  const Span sw[3] = {span(h->w_down, W_BYTES), span(h->w_up, W_BYTES), span(h->w_norm, WNORM_BYTES)};

  // out: exactly x, exactly pending, or disjoint from both; never overlapping anything else
  if (overlap(so, sx) && !same(so, sx)) return HCR_EALIAS;
  if (overlap(so, sp) && !same(so, sp)) return HCR_EALIAS;
  if (overlap(so, si) || overlap(so, sm) || overlap(so, sc)) return HCR_EALIAS;
  // mean and scratch are written: they overlap nothing
  const Span inputs[] = {sx, sp, si, sc};
  for (const Span& s : inputs)
    if (overlap(sm, s)) return HCR_EALIAS;
  if (overlap(sc, sx) || overlap(sc, sp) || overlap(sc, si)) return HCR_EALIAS;
  for (const Span& w : sw)
    if (overlap(so, w) || overlap(sm, w)) return HCR_EALIAS;

  return hcr::launch_read(T, h->w_down, h->w_up, h->w_norm, h->scratch, x, pending, inj, out, mean, stream);
}

void hcr_destroy(hcr_t h) { free(h); }

const char* hcr_strerror(int rc) {
  switch (rc) {
    case HCR_OK: return "ok";
    case HCR_EINVAL: return "invalid argument (null handle or pointer, or T outside 0..HCR_T_MAX)";
    case HCR_EALIGN: return "misaligned pointer (16 bytes; scratch 256 bytes)";
    case HCR_ESCRATCH: return "scratch smaller than hcr_scratch_bytes()";
    case HCR_EALIAS: return "buffers overlap in a way the read does not allow";
    case HCR_EHIP: return "HIP kernel launch failed";
    default: return "unknown error code";
  }
}

}  // extern "C"
