// C ABI of the BF16 hyper-connection read, its Q8_0 copies and the skinny BF16 matvec: argument
// validation and the handle.  Every check runs on the host before any HIP call.

#include <stdint.h>
#include <stdlib.h>

#include "hcr_layout.h"

struct hcr_handle {
  int fmt;                 // hcr::FMT_BF16 or hcr::FMT_Q8_0
  const void* w_down;      // BF16 weights or int8 codes
  const void* w_up;
  const uint16_t* s_down;  // Q8_0 scales (binary16), else null
  const uint16_t* s_up;
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
constexpr size_t Q8_CODE_BYTES = size_t(hcr::R) * hcr::DD;                     // each projection, int8
constexpr size_t Q8_SCALE_BYTES = size_t(hcr::R) * hcr::DD / hcr::Q8_BLOCK * 2;  // each projection, binary16
constexpr size_t WNORM_BYTES = size_t(hcr::S) * hcr::D * 4;

// the spans of a handle's weights (absent ones empty)
void weight_spans(const hcr_handle* h, Span (&sw)[5]) {
  const size_t wb = h->fmt == hcr::FMT_BF16 ? W_BYTES : Q8_CODE_BYTES;
  sw[0] = span(h->w_down, wb);
  sw[1] = span(h->w_up, wb);
  sw[2] = span(h->w_norm, WNORM_BYTES);
  sw[3] = span(h->s_down, Q8_SCALE_BYTES);
  sw[4] = span(h->s_up, Q8_SCALE_BYTES);
}

int make_handle(hcr_handle proto, size_t scratch_bytes, hcr_t* out) {
  if (!out) return HCR_EINVAL;
  *out = nullptr;
  if (!proto.w_down || !proto.w_up || !proto.w_norm || !proto.scratch) return HCR_EINVAL;
  if (proto.fmt == hcr::FMT_Q8_0 && (!proto.s_down || !proto.s_up)) return HCR_EINVAL;
  if (!aligned(proto.w_down, 16) || !aligned(proto.w_up, 16) || !aligned(proto.w_norm, 16) ||
      !aligned(proto.scratch, 256) || !aligned(proto.s_down, 16) || !aligned(proto.s_up, 16))
    return HCR_EALIGN;
  if (scratch_bytes < hcr::SCRATCH_BYTES) return HCR_ESCRATCH;
  const Span sc = span(proto.scratch, hcr::SCRATCH_BYTES);
  Span sw[5];
  weight_spans(&proto, sw);
  for (const Span& w : sw)
    if (overlap(sc, w)) return HCR_EALIAS;
  hcr_handle* h = static_cast<hcr_handle*>(malloc(sizeof(hcr_handle)));
  if (!h) return HCR_EINVAL;
  *h = proto;
  *out = h;
  return HCR_OK;
}

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
  return make_handle(hcr_handle{hcr::FMT_BF16, w_down, w_up, nullptr, nullptr, w_norm, scratch}, scratch_bytes, out);
}

int hcr_create_q8_0(const void* down_codes, const void* down_scales, const void* up_codes, const void* up_scales,
                    const float* w_norm, void* scratch, size_t scratch_bytes, hcr_t* out) {
  return make_handle(hcr_handle{hcr::FMT_Q8_0, down_codes, up_codes, static_cast<const uint16_t*>(down_scales),
                                static_cast<const uint16_t*>(up_scales), w_norm, scratch},
                     scratch_bytes, out);
}

int hcr_quantize_q8_0(const void* w, int rows, int cols, void* codes, void* scales, void* stream) {
  if (!w || !codes || !scales || rows <= 0 || cols <= 0 || cols % hcr::Q8_BLOCK) return HCR_EINVAL;
  const size_t n = size_t(rows) * size_t(cols);
  if (n / hcr::Q8_BLOCK * 4 / 256 >= (size_t(1) << 31)) return HCR_EINVAL;  // grid size
  if (!aligned(w, 16) || !aligned(codes, 16) || !aligned(scales, 16)) return HCR_EALIGN;
  const Span sw = span(w, n * 2), sq = span(codes, n), ss = span(scales, n / hcr::Q8_BLOCK * 2);
  if (overlap(sw, sq) || overlap(sw, ss) || overlap(sq, ss)) return HCR_EALIAS;
  return hcr::launch_quantize_q8_0(w, n / hcr::Q8_BLOCK, codes, scales, stream);
}

int hcr_matvec_bf16(const void* w, int rows, int cols, int T, const float* x, float* y, void* stream) {
  if (T == 0) return HCR_OK;
  if (!w || !x || !y || rows <= 0 || cols <= 0 || cols % 8 || cols > 64 * 8 * hcr::MV_KCH_MAX || T < 0 ||
      T > hcr::MV_T_MAX)
    return HCR_EINVAL;
  if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 16)) return HCR_EALIGN;
  const Span sw = span(w, size_t(rows) * size_t(cols) * 2), sx = span(x, size_t(T) * cols * 4),
             sy = span(y, size_t(T) * rows * 4);
  if (overlap(sy, sw) || overlap(sy, sx)) return HCR_EALIAS;
  return hcr::launch_matvec_bf16(w, rows, cols, T, x, y, stream);
}

}  // extern "C"

namespace {

// The argument checks of a read on h's weights (h.scratch null: the library's own scratch, which no caller
// buffer can overlap); HCR_OK when the read may be enqueued.
int check_read(const hcr_handle* h, int T, const float* x, const float* pending, const float* inj, float* out,
               float* mean) {
  if (!x || !out || !mean) return HCR_EINVAL;
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(mean, 16) || (pending && !aligned(pending, 16)) ||
      (inj && !aligned(inj, 16)))
    return HCR_EALIGN;

  const size_t stream_bytes = size_t(T) * hcr::S * hcr::D * 4;
  const Span sx = span(x, stream_bytes), sp = span(pending, stream_bytes), so = span(out, stream_bytes);
  const Span sm = span(mean, size_t(T) * hcr::D * 4), si = span(inj, size_t(T) * hcr::R * 4);
  const Span sc = span(h->scratch, hcr::SCRATCH_BYTES);
  Span sw[5];
  weight_spans(h, sw);

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
  return HCR_OK;
}

}  // namespace

extern "C" {

int hcr_read(hcr_t h, int T, const float* x, const float* pending, const float* inj, float* out, float* mean,
             void* stream) {
  if (!h || T < 0 || T > hcr::TMAX) return HCR_EINVAL;
  if (T == 0) return HCR_OK;
  const int rc = check_read(h, T, x, pending, inj, out, mean);
  if (rc != HCR_OK) return rc;
  return hcr::launch_read(h->fmt, T, h->w_down, h->s_down, h->w_up, h->s_up, h->w_norm, h->scratch, x, pending, inj,
                          out, mean, stream);
}

int hcr_read_static(const void* w_down, const void* w_up, const float* w_norm, int T, const float* x,
                    const float* pending, const float* inj, float* out, float* mean, void* stream) {
  if (T < 0 || T > hcr::TMAX) return HCR_EINVAL;
  if (T == 0) return HCR_OK;
  if (!w_down || !w_up || !w_norm) return HCR_EINVAL;
  if (!aligned(w_down, 16) || !aligned(w_up, 16) || !aligned(w_norm, 16)) return HCR_EALIGN;
  const hcr_handle h{hcr::FMT_BF16, w_down, w_up, nullptr, nullptr, w_norm, nullptr};
  int rc = check_read(&h, T, x, pending, inj, out, mean);
  if (rc != HCR_OK) return rc;
  void* sc = nullptr;
  rc = hcr::static_scratch(stream, &sc);
  if (rc != HCR_OK) return rc;
  return hcr::launch_read(hcr::FMT_BF16, T, w_down, nullptr, w_up, nullptr, w_norm, sc, x, pending, inj, out, mean,
                          stream);
}

void hcr_destroy(hcr_t h) { free(h); }

const char* hcr_strerror(int rc) {
  switch (rc) {
    case HCR_OK: return "ok";
    case HCR_EINVAL: return "invalid argument (null handle or pointer, T outside 0..HCR_T_MAX, or a bad matrix shape)";
    case HCR_EALIGN: return "misaligned pointer (16 bytes; scratch 256 bytes)";
    case HCR_ESCRATCH: return "scratch smaller than hcr_scratch_bytes()";
    case HCR_EALIAS: return "buffers overlap in a way the read does not allow";
    case HCR_EHIP: return "HIP kernel launch failed";
    default: return "unknown error code";
  }
}

}  // extern "C"
