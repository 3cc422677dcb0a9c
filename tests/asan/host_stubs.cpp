// Host-only stand-ins for the library's launchers, so that the C ABI's argument checks (hcr_api.cpp) can be
// built with the host compiler under AddressSanitizer and UndefinedBehaviorSanitizer and exercised without a
// GPU.  The ABI tests make only calls that the checks reject (or T = 0 no-ops): reaching any of these means a
// check let a call through, and it returns HCR_EHIP so the test sees a wrong code.
#include "hcr_layout.h"

namespace hcr {

int launch_read(int, int, const void*, const uint16_t*, const void*, const uint16_t*, const float*, void*,
                const float*, const float*, const float*, float*, float*, void*) {
  return HCR_EHIP;
}
int launch_matvec_bf16(const void*, int, int, int, const float*, float*, void*) { return HCR_EHIP; }
int launch_quantize_q8_0(const void*, size_t, void*, void*, void*) { return HCR_EHIP; }
int static_scratch(void*, void** out) {
  *out = nullptr;
  return HCR_EHIP;
}

}  // namespace hcr
