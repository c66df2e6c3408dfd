"""The kernel-timing hook of the C ABI (cp_timing_begin / cp_timing_end) on
the GPU: every launch up to the capacity is recorded, in launch order, with a
positive duration, and timing does not change results."""
import pytest
import torch

import prefix_sum_causal_amd as cp

pytestmark = pytest.mark.gpu


def test_timing_records_each_launch_in_order():
    torch.manual_seed(0)
    q = torch.rand(2, 3, 300, 64, device="cuda").bfloat16()
    k = torch.rand(2, 3, 300, 64, device="cuda").bfloat16()
    v = torch.randn(2, 3, 300, 32, device="cuda").bfloat16()
    g = torch.randn(2, 3, 300, 32, device="cuda").bfloat16()
    ref = cp.causal_product_fwd(q, k, v)
    cp.timing_begin(3)
    out = cp.causal_product_fwd(q, k, v)
    cp.causal_product_bwd(q, k, v, g)
    cp.causal_product_fwd(q, k, v)
    cp.causal_product_fwd(q, k, v)  # past the capacity: runs, not timed
    ms = cp.timing_end()
    torch.cuda.synchronize()
    assert len(ms) == 3
    assert all(0.0 < t < 1000.0 for t in ms)
    assert torch.equal(out, ref)


def test_timing_end_without_begin_is_an_error():
    with pytest.raises(cp.CausalProductError):
        cp.timing_end()
