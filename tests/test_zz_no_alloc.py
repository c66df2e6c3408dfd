"""causal_product_fwd_noalloc through the C ABI: the forward for callers that
cannot allocate must give exactly the output and final state of
causal_product_fwd (same kernels) and pass the forward's parity bar against
the fp64 oracle, on two calls in a row (the second smaller, so that it runs
on the scratch the first left behind), both over sequence segments."""
import numpy as np
import pytest
import torch

import oracle
import prefix_sum_causal_amd as cp
import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 2.5e-3}
TDT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _run(shape, dtype, seed):
    N, H, L, E, M = shape
    w = W.Workload("noalloc", "fwd", dtype, N, H, L, E, M, seed=seed)
    d = W.generate(w, need_do=False)
    dev = {k: torch.from_numpy(v).cuda().to(TDT[dtype]) for k, v in d.items()}
    q, k, v = dev["Q"], dev["K"], dev["V"]
    out_ref = torch.empty_like(v)
    st_ref = torch.empty((N, H, E, M), device="cuda", dtype=torch.float32)
    cp.causal_product_fwd(q, k, v, out=out_ref, state_out=st_ref)
    out = torch.full_like(v, float("nan"))
    st = torch.full((N, H, E, M), float("nan"), device="cuda", dtype=torch.float32)
    cp.causal_product_fwd_noalloc(q, k, v, out=out, state_out=st)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref)
    assert torch.equal(st, st_ref)
    ref, sref = oracle.default().fwd(d["Q"], d["K"], d["V"], return_state=True)
    got = out.float().cpu().numpy()
    assert oracle.max_rel_err(got, ref) <= TOL[dtype]
    assert oracle.max_rel_err(st.cpu().numpy(), sref) <= 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
def test_noalloc_forward_two_calls(dtype):
    # few slices and long sequences: both calls run as sequence segments
    _run((1, 3, 3000, 64, 64), dtype, seed=21)
    _run((1, 1, 1000, 32, 64), dtype, seed=22)


def test_noalloc_forward_without_segments():
    # enough slices to fill the GPU: no scratch at all
    _run((4, 64, 300, 64, 64), "bf16", seed=23)
