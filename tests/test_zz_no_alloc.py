"""rm_block_bwd_static, the backward for callers that cannot allocate device
memory, through the C ABI: it must give rm_block_bwd's results for the same
saved forward state (the same kernels in the same order, so bit for bit; the
tolerance of the parity tests is checked as well), on consecutive calls with
different shapes sharing the one static scratch buffer."""
import ctypes

import numpy as np
import pytest

from rankmixer_inputs import WORKLOADS, make_case, make_custom
from rm_gpu import GRAD_KEYS, TOL, DeviceCase, compare, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import transformer_block_norm0_amd as rb
    rb.library()


def saved_prefix_bytes(rb, cd):
    off, nb = rb.ws_region(cd, rb.rmblock.RM_WS_STATS)
    return off + nb


def check_static_matches(case, kernels="auto"):
    import torch
    import transformer_block_norm0_amd as rb
    label = f"{case['name']} ({kernels} kernels)"
    say(f"static backward {label}: forward and workspace backward")
    dc = DeviceCase(case, kernels=kernels)
    dc.run()
    ref_bits = dc.raw_bits()
    ref = dc.results()
    # poison the workspace's own scratch area and the outputs: the static variant must use neither
    saved = saved_prefix_bytes(rb, dc.cd)
    dc.ws[saved:].fill_(0xFF)
    for t in [dc.dx] + list(dc.grads.values()):
        t.fill_(float("nan"))
    torch.cuda.synchronize()
    say(f"static backward {label}: rm_block_bwd_static")
    rb.block_bwd_static(dc.cd, dc.params, dc.x, dc.dy, dc.ws, dc.dx, dc.grads, ws_bytes=saved)
    torch.cuda.synchronize()
    got_bits = dc.raw_bits()
    compare(dc.results(), ref, list(GRAD_KEYS), TOL[case["dtype"]], f"static vs workspace backward {label}")
    for k in ref_bits:
        if k == "y":
            continue
        assert np.array_equal(ref_bits[k], got_bits[k]), (label, k)


def test_static_backward_two_calls_second_smaller():
    """Two calls in a row on the shared static buffer: the fp32 B256 T16 D256 k3 workload, then the
    smaller public bf16 shape (whose backward runs the small-batch kernels)."""
    check_static_matches(make_case(WORKLOADS["B256_T16_D256_k3_f32"]))
    check_static_matches(make_case(WORKLOADS["B4_T16_D128_k2_bf16_public"]))


def test_static_backward_main_kernels_and_ragged_shape():
    check_static_matches(make_case(WORKLOADS["B4_T16_D128_k2_f16_public"]), kernels="main")
    check_static_matches(make_custom(67, 16, 256, 2, "bf16", seed=41, ln_affine="random"))


def test_static_backward_rejects_scratch_beyond_its_buffer():
    """The production shape's scratch exceeds the static buffer: RM_E_SCRATCH, nothing launched."""
    import transformer_block_norm0_amd as rb
    lib = rb.library()
    d = rb.dims(1024, 64, 1280, 2, "bf16")
    params = rb.rmblock.CParams(*([256] * 14))
    grads = rb.rmblock.CGrads(*([512] * 14))
    by = ctypes.byref
    st = lib.rm_block_bwd_static(by(d), by(params), 1024, 1024, 4096, 1 << 40, 2048, by(grads), None)
    assert st == 8, st
