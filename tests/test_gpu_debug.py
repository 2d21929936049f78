"""Debug mode on the GPU: plans are copied to the host and checked before the
calls that read them.

With debug mode on, a consistent plan gives bit-identical results to the
plain calls; a damaged plan is refused with BSA_ERR_BAD_PLAN before any
kernel runs.  The damage planted here keeps every entry inside its range
(two columns of a row swapped, a tile moved to another column), so the
kernels would stay inside their buffers even if a check missed it.
"""

import numpy as np
import pytest
import torch

import block_sparse_attention_plan_amd as bsa
from block_sparse_attention_plan_amd import workloads as W

from test_gpu_parity import say

pytestmark = pytest.mark.gpu

BAD_PLAN = -7


@pytest.fixture
def debug_mode():
    prev = bsa.set_debug(True)
    yield
    bsa.set_debug(prev)


def _inputs(gpu, seed=5):
    bs, d, H, Mb = 64, 64, 3, 6
    x = W.make_bsa("debug", B=2, H=H, S=Mb * bs, bs=bs, d=d, dtype="bf16", layout="random", p=0.4,
                   seed=seed)
    lay = np.asarray(x.layout, np.int32)
    lay[:, :, 0] = 1
    lay[:, :, Mb - 1] = 1   # every row lists at least two columns
    return x, lay, bs


def test_debug_mode_keeps_results(gpu, debug_mode):
    x, lay, bs = _inputs(gpu)
    say("[debug] consistent plan: forward and backward with and without checks")
    plan = bsa.bsa_plan(torch.from_numpy(lay).to(gpu))
    cols = bsa.bsa_plan_cols(torch.from_numpy(lay).to(gpu))
    bsa.bsa_plan_check(plan, cols)
    q, k, v = x.q.to(gpu), x.k.to(gpu), x.v.to(gpu)
    out, lse = bsa.bsa_forward(q, k, v, plan, x.scale)
    g = torch.randn_like(out)
    grads = bsa.bsa_backward(q, k, v, out, g, lse, plan, cols, x.scale)
    bsa.set_debug(False)
    out2, lse2 = bsa.bsa_forward(q, k, v, plan, x.scale)
    grads2 = bsa.bsa_backward(q, k, v, out2, g, lse2, plan, cols, x.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    for a, b in zip(grads[:3], grads2[:3]):
        assert torch.equal(a, b)


def test_damaged_plan_is_refused(gpu, debug_mode):
    x, lay, bs = _inputs(gpu, seed=6)
    say("[debug] two columns of a row swapped: forward refused")
    plan = bsa.bsa_plan(torch.from_numpy(lay).to(gpu))
    q, k, v = x.q.to(gpu), x.k.to(gpu), x.v.to(gpu)
    col = plan.col_idx()
    row_ptr = plan.row_ptr.cpu().numpy()
    t = int(row_ptr[np.nonzero(np.diff(row_ptr) >= 2)[0][0]])
    a, b = col[t].item(), col[t + 1].item()
    col[t], col[t + 1] = b, a
    with pytest.raises(bsa.BsaError) as e:
        bsa.bsa_forward(q, k, v, plan, x.scale)
    assert e.value.status == BAD_PLAN and "ascending" in str(e.value)
    with pytest.raises(bsa.BsaError) as e:
        bsa.bsa_plan_check(plan)
    assert e.value.status == BAD_PLAN


def test_column_plan_of_another_layout_is_refused(gpu, debug_mode):
    x, lay, bs = _inputs(gpu, seed=7)
    other = lay.copy()
    h, m = 1, 2
    live = np.nonzero(other[h, m])[0]
    dead = np.nonzero(other[h, m] == 0)[0]
    if dead.size == 0:
        pytest.skip("row has no free column")
    other[h, m, live[-1]], other[h, m, dead[0]] = 0, 1
    say("[debug] column plan of a layout with one tile moved: backward refused")
    plan = bsa.bsa_plan(torch.from_numpy(lay).to(gpu))
    cols = bsa.bsa_plan_cols(torch.from_numpy(other).to(gpu))
    bsa.bsa_plan_check(plan)
    bsa.bsa_plan_check(plan_cols=cols)
    q, k, v = x.q.to(gpu), x.k.to(gpu), x.v.to(gpu)
    out, lse = bsa.bsa_forward(q, k, v, plan, x.scale)
    with pytest.raises(bsa.BsaError) as e:
        bsa.bsa_backward(q, k, v, out, torch.ones_like(out), lse, plan, cols, x.scale)
    assert e.value.status == BAD_PLAN and "missing from the column plan" in str(e.value)
