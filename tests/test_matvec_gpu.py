"""The skinny BF16 matvec on the GPU (through the C ABI) against the FP64 reference.

Every element of y is compared with the reference within 1e-4 of max |y|.
FP32 accumulation over K <= 3072 products of BF16 weights and FP32 inputs
gives ~1e-6 of max |y| here; a wrong row, column or chunk gives O(1).
"""

import numpy as np
import pytest
import torch

import oracle
from bf16_hyper_connection_amd import hcr
from bf16_hyper_connection_amd import inputs as gen
from tests.gpu_util import max_rel, to_dev
from tests.libhcr_util import ensure_built

pytestmark = pytest.mark.gpu
TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


@pytest.fixture(scope="module")
def full_w():
    w = gen.matvec_weights(20)
    return w, to_dev(w)


@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_matvec_full_size(full_w, T):
    """The pages' shape, 12288 x 2560, every output element."""
    w, wd = full_w
    x = gen.matvec_x(20, T, index=T)
    y = hcr.matvec_bf16(wd, to_dev(x))
    torch.cuda.synchronize()
    e = max_rel(y, oracle.matvec_bf16(w, x))
    assert e <= TOL, f"T={T}: error {e:.3e} of max |y|"


@pytest.mark.parametrize("rows,cols", [(1, 8), (3, 72), (5, 520), (4099, 2560), (777, 3000), (64, 3072),
                                        (1030, 512), (2, 2568)])
@pytest.mark.parametrize("T", [1, 4])
def test_matvec_ragged_shapes(rows, cols, T):
    """Row counts that are not multiples of 4 or of the grid, and column counts with partial chunks per lane."""
    w = gen.matvec_weights(21, rows=rows, cols=cols)
    x = gen.matvec_x(21, T, cols=cols)
    y = hcr.matvec_bf16(to_dev(w), to_dev(x))
    torch.cuda.synchronize()
    e = max_rel(y, oracle.matvec_bf16(w, x))
    assert e <= TOL, f"{rows}x{cols} T={T}: error {e:.3e}"


def test_matvec_leaves_rest_of_y_alone(full_w):
    """y is written exactly at [T][rows]: a guard band after it keeps its contents."""
    w, wd = full_w
    x = to_dev(gen.matvec_x(22, 3))
    buf = torch.full((3 * 12288 + 64,), 7.0, device="cuda")
    y = buf[:3 * 12288].view(3, 12288)
    hcr.matvec_bf16(wd, x, y=y)
    torch.cuda.synchronize()
    assert torch.all(buf[3 * 12288:] == 7.0)


def test_matvec_columns_do_not_depend_on_T(full_w):
    """Each column's result is the same, bit for bit, alone or among 4."""
    _, wd = full_w
    x = to_dev(gen.matvec_x(23, 4))
    y4 = hcr.matvec_bf16(wd, x).clone()
    for t in range(4):
        y1 = hcr.matvec_bf16(wd, x[t:t + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(y1[0], y4[t]), f"column {t}"


def test_matvec_graph_replay_bitwise(full_w):
    _, wd = full_w
    x = to_dev(gen.matvec_x(24, 4))
    direct = hcr.matvec_bf16(wd, x).clone()
    y = torch.empty_like(direct)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            hcr.matvec_bf16(wd, x, y=y)
    torch.cuda.current_stream().wait_stream(s)
    for i in range(4):
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, direct), f"replay {i}"


@pytest.mark.parametrize("rows", [1_048_577, 1_100_003])
def test_matvec_tall_matrix_walks_the_grid_in_steps(rows):
    """More row groups than the grid's 65,536 work-groups of 4 waves hold (262,144 groups of 4 rows): the
    waves take a second step (1,048,577 rows: exactly one group in the second step)."""
    cols, T = 8, 2
    w = gen.matvec_int_weights(25, rows, cols)
    x = gen.matvec_x(25, T, cols=cols)
    y = hcr.matvec_bf16(to_dev(w), to_dev(x))
    torch.cuda.synchronize()
    e = max_rel(y, oracle.matvec_bf16(w, x))
    assert e <= TOL, f"tall matrix: error {e:.3e}"
