"""Caller workspaces on the GPU, through the C ABI.

A call over few slices runs as sequence segments and needs scratch for the
segments' increments.  The same call must give the same bits whether that
scratch is the caller's workspace (exactly the size cp_workspace_size
reports, filled with NaN bytes first: its contents need not be initialised;
or a larger buffer at an offset) or the library's own stream-ordered
allocation (workspace NULL).  A workspace smaller than the call needs is
refused with CP_ERR_SCRATCH before anything is enqueued.  Correctness of the
segmented results themselves against the oracle is covered by the parity
tests; here every variant is compared with the library's own allocation.
"""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

# few slices, long enough to be split into segments; E != M and a ragged tail
SHAPES = [(1, 2, 3000, 64, 64), (2, 1, 2085, 32, 128)]
SCRATCH = 7


@pytest.fixture(scope="module")
def cp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import prefix_sum_causal_amd as cp
    return cp


def tensors(shape, dtype, seed):
    N, H, L, E, M = shape
    d = W.generate(W.Workload("ws", "fwd+bwd", dtype, N, H, L, E, M, seed=seed, qk="raw"), need_do=True)
    t = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to("cuda").to(t) for k, v in d.items()}


def p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def workspaces(cp, op, shape, dtype_code):
    """[None (the library allocates), exact NaN-filled, larger at an offset]"""
    need = cp.workspace_size(op, *shape, dtype_code)
    assert need > 0, "the shape must run as sequence segments"
    exact = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    big = torch.full((need + 4096,), 0xFF, dtype=torch.uint8, device="cuda")[256:]
    return need, [None, exact, big]


def call(cp, op, d, shape, dtype_code, ws, nbytes=None):
    """One call of op through the C ABI; returns its outputs (host copies)."""
    N, H, L, E, M = shape
    q, k, v, g = d["Q"], d["K"], d["V"], d["dO"]
    wb = 0 if ws is None else (ws.numel() if nbytes is None else nbytes)
    f32 = dict(device="cuda", dtype=torch.float32)
    if op == cp.CP_OP_CAUSAL_FWD:
        out, st = torch.empty_like(v), torch.empty((N, H, E, M), **f32)
        r = cp.lib.causal_product_fwd(p(q), p(k), p(v), p(out), None, p(st), N, H, L, E, M, dtype_code, p(ws), wb,
                                      stream())
        res = (out, st)
    elif op == cp.CP_OP_CAUSAL_BWD:
        dq, dk, dv, ds0 = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty((N, H, E, M), **f32)
        r = cp.lib.causal_product_bwd(p(q), p(k), p(v), p(g), None, None, p(dq), p(dk), p(dv), p(ds0), N, H, L, E, M,
                                      dtype_code, p(ws), wb, stream())
        res = (dq, dk, dv, ds0)
    elif op == cp.CP_OP_LINATTN_FWD:
        out, st, zt, den = (torch.empty_like(v), torch.empty((N, H, E, M), **f32), torch.empty((N, H, E), **f32),
                            torch.empty((N, H, L), **f32))
        r = cp.lib.linear_attn_fwd(p(q), p(k), p(v), p(out), None, None, p(st), p(zt), p(den), N, H, L, E, M, 1e-6, 1,
                                   dtype_code, p(ws), wb, stream())
        res = (out, st, zt, den)
    else:
        out, st, zt, den = (torch.empty_like(v), torch.empty((N, H, E, M), **f32), torch.empty((N, H, E), **f32),
                            torch.empty((N, H, L), **f32))
        assert cp.lib.linear_attn_fwd(p(q), p(k), p(v), p(out), None, None, p(st), p(zt), p(den), N, H, L, E, M, 1e-6,
                                      1, dtype_code, None, 0, stream()) == 0
        dq, dk, dv, ds0, dz0 = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
                                torch.empty((N, H, E, M), **f32), torch.empty((N, H, E), **f32))
        r = cp.lib.linear_attn_bwd(p(q), p(k), p(v), p(out), p(g), p(den), None, None, p(st), p(zt), p(dq), p(dk),
                                   p(dv), p(ds0), p(dz0), N, H, L, E, M, 1, dtype_code, p(ws), wb, stream())
        res = (dq, dk, dv, ds0, dz0)
    torch.cuda.synchronize()
    return r, [t.cpu() for t in res]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("op", [0, 1, 2, 3])
def test_workspace_gives_the_same_bits(cp, op, dtype, shape):
    code = {"f32": cp.CP_F32, "bf16": cp.CP_BF16}[dtype]
    print(f"workspace op {op} {dtype} {shape}", flush=True)
    d = tensors(shape, dtype, seed=40 + op)
    need, wss = workspaces(cp, op, shape, code)
    ref = None
    for i, ws in enumerate(wss):
        r, res = call(cp, op, d, shape, code, ws)
        assert r == 0, (i, cp.lib.cp_status_string(r))
        if ref is None:
            ref = res
            continue
        for a, b in zip(ref, res):
            assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.uint8) if b.dtype == torch.bfloat16 else b), i
    # a workspace one 16-byte piece short is refused before anything runs
    r, _ = call(cp, op, d, shape, code, wss[1], nbytes=need - 16)
    assert r == SCRATCH


def test_binding_takes_a_workspace(cp):
    shape = SHAPES[0]
    d = tensors(shape, "bf16", seed=7)
    need = cp.workspace_size(cp.CP_OP_CAUSAL_FWD, *shape, cp.CP_BF16)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    a = cp.causal_product_fwd(d["Q"], d["K"], d["V"], workspace=ws)
    b = cp.causal_product_fwd(d["Q"], d["K"], d["V"])
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.uint16), b.view(torch.uint16))
    with pytest.raises(cp.CausalProductError, match="CP_ERR_SCRATCH"):
        cp.causal_product_fwd(d["Q"], d["K"], d["V"], workspace=ws[:need - 16])
