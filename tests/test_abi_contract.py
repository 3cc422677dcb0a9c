"""Property test of hcr_read's argument checks against a model of the contract include/hcr.h states.

Random placements of x, pending, inj, out and mean (and of the handle's weights and scratch) in a fake address
space: the model decides from the header's rules alone whether the call is invalid (HCR_EINVAL), misaligned
(HCR_EALIGN), aliased (HCR_EALIAS) or valid.  Only calls the model rejects are made: a rejected call returns
before any HIP call, so the fake addresses are never touched.  The library must return the model's code.
Runs only where no GPU is visible, so that a checking bug could never launch a kernel on fake pointers."""

import pytest

torch = pytest.importorskip("torch")
hypothesis = pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

from bf16_hyper_connection_amd import hcr  # noqa: E402
from tests.libhcr_util import ensure_built  # noqa: E402

pytestmark = pytest.mark.skipif(torch.cuda.is_available(), reason="fake device addresses: run where no GPU is visible")

S, D, R, TMAX = 4, 2560, 320, 16
W_BYTES = R * S * D * 2          # each BF16 projection
WN_BYTES = S * D * 4
BASE = 1 << 36                   # the fake address space starts here, 64 GiB up
SLOT = 1 << 24                   # 16 MiB between the "home" slots of the buffers


def spans_for(T, place):
    """{name: (lo, hi) or None} of the call's buffers, from the placements (address or None)."""
    nbytes = {"x": T * S * D * 4, "pending": T * S * D * 4, "out": T * S * D * 4, "mean": T * D * 4,
              "inj": T * R * 4}
    return {k: None if place[k] is None else (place[k], place[k] + nbytes[k]) for k in nbytes}


def overlap(a, b):
    return a is not None and b is not None and a[0] < b[1] and b[0] < a[1]


def model(T, place, handle_spans):
    """The header's rules for hcr_read (h valid): HCR_EINVAL, HCR_EALIGN, HCR_EALIAS or HCR_OK."""
    if T < 0 or T > TMAX:
        return hcr.HCR_EINVAL
    if T == 0:
        return hcr.HCR_OK
    if place["x"] is None or place["out"] is None or place["mean"] is None:
        return hcr.HCR_EINVAL
    if any(p is not None and p % 16 for p in place.values()):
        return hcr.HCR_EALIGN
    sp = spans_for(T, place)
    x, pend, inj, out, mean = sp["x"], sp["pending"], sp["inj"], sp["out"], sp["mean"]
    scratch, weights = handle_spans["scratch"], handle_spans["weights"]
    # out: exactly x, exactly pending, or disjoint from both; otherwise it overlaps nothing
    if overlap(out, x) and out != x:
        return hcr.HCR_EALIAS
    if overlap(out, pend) and out != pend:
        return hcr.HCR_EALIAS
    if any(overlap(out, b) for b in (inj, mean, scratch, *weights)):
        return hcr.HCR_EALIAS
    # mean overlaps nothing; the scratch (written by the read) overlaps no input
    if any(overlap(mean, b) for b in (x, pend, inj, scratch, *weights)):
        return hcr.HCR_EALIAS
    if any(overlap(scratch, b) for b in (x, pend, inj)):
        return hcr.HCR_EALIAS
    return hcr.HCR_OK


# a buffer's placement: absent, in its own slot, or on top of (or inside) another buffer's slot
NAMES = ["x", "pending", "inj", "out", "mean"]
HOME = {"x": 0, "pending": 1, "inj": 2, "out": 3, "mean": 4, "w_down": 5, "w_up": 6, "w_norm": 7, "scratch": 8}


@st.composite
def placements(draw):
    place = {}
    for n in NAMES:
        kind = draw(st.sampled_from(["home", "home", "home", "other", "none"] if n in ("pending", "inj")
                                    else ["home", "home", "home", "other", "none"]))
        if kind == "none":
            place[n] = None
            continue
        slot = HOME[n] if kind == "home" else HOME[draw(st.sampled_from(list(HOME)))]
        offset = draw(st.sampled_from([0, 0, 0, 16, 4, 4096, 81920, 327680, 2 * 327680]))
        place[n] = BASE + slot * SLOT + offset
    T = draw(st.sampled_from([-1, 0, 1, 2, 3, 8, 9, 16, 17]))
    return T, place


@pytest.fixture(scope="module")
def handle():
    ensure_built()
    addr = {k: BASE + HOME[k] * SLOT for k in ("w_down", "w_up", "w_norm", "scratch")}
    h = hcr.hcr_create(addr["w_down"], addr["w_up"], addr["w_norm"], addr["scratch"], hcr.hcr_scratch_bytes())
    spans = {"scratch": (addr["scratch"], addr["scratch"] + hcr.hcr_scratch_bytes()),
             "weights": [(addr["w_down"], addr["w_down"] + W_BYTES), (addr["w_up"], addr["w_up"] + W_BYTES),
                         (addr["w_norm"], addr["w_norm"] + WN_BYTES)]}
    yield h, spans
    hcr.hcr_destroy(h)


@settings(max_examples=3000, deadline=None, suppress_health_check=[HealthCheck.function_scoped_fixture])
@given(case=placements())
def test_read_checks_match_the_contract(handle, case):
    h, spans = handle
    T, place = case
    want = model(T, place, spans)
    if want == hcr.HCR_OK and T != 0:
        return  # a valid call would launch the kernels: not made here (the GPU tests cover valid calls)
    got = hcr.hcr_read(h, T, place["x"], place["pending"], place["inj"], place["out"], place["mean"], None)
    assert got == want, (T, {k: None if v is None else hex(v) for k, v in place.items()}, hcr.hcr_strerror(got))


def test_the_model_sees_every_outcome(handle):
    """The strategy reaches every code the model can give (so the property test exercises each rule)."""
    _, spans = handle
    seen = set()

    @settings(max_examples=2000, deadline=None)
    @given(case=placements())
    def collect(case):
        seen.add(model(case[0], case[1], spans))

    collect()
    assert {hcr.HCR_OK, hcr.HCR_EINVAL, hcr.HCR_EALIGN, hcr.HCR_EALIAS} <= seen
