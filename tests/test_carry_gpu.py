"""Parity of the carried state (initial S0 and z0 in, final S and z out, the
gradient of S0) on the GPU against the fp64 oracle, through the C ABI.

Same metric and bars as the other parity tests (max|gpu - ref| / max|ref|,
1e-4 for fp32 I/O, 2e-2 for bf16 I/O).  Shapes include a few slices with a
long sequence, which the forward runs as sequence segments, so the carried-in
state also passes through the segment path.  A sequence processed in two
pieces, the second starting from the first's final state, must agree with
the one-piece result.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
TORCH = {"f32": torch.float32, "bf16": torch.bfloat16}

# (N, H, L, E, M): ragged tails, E != M, and two slices over 1500 rows
# (the forward then splits the sequence into segments)
SHAPES = [(2, 3, 150, 64, 32), (1, 2, 77, 32, 128), (1, 2, 1500, 64, 64), (2, 1, 200, 128, 16)]


@pytest.fixture(scope="module")
def cp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import prefix_sum_causal_amd as cp
    return cp


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


def dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(TORCH[dtype])


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def inputs(shape, dtype, seed, qk="elu1"):
    N, H, L, E, M = shape
    d = W.generate(W.Workload("carry", "fwd+bwd", dtype, N, H, L, E, M, seed=seed, qk=qk), need_do=True)
    r = np.random.default_rng(seed + 1000)
    # initial states of the size the sums reach after a few hundred rows
    d["S0"] = (r.standard_normal((N, H, E, M)) * 20).astype(np.float32)
    d["z0"] = (r.random((N, H, E)) * 100 + 1).astype(np.float32)
    return d


def fstate(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")


def check(got, ref, dtype, what):
    err = oracle.max_rel_err(got, ref)
    print(f"{what}: max rel err {err:.3e}", flush=True)
    assert err <= TOL[dtype], what


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_fwd_from_state(cp, orc, dtype, shape):
    N, H, L, E, M = shape
    d = inputs(shape, dtype, seed=11)
    q, k, v = dev(d["Q"], dtype), dev(d["K"], dtype), dev(d["V"], dtype)
    st = torch.empty((N, H, E, M), device="cuda")
    out = cp.causal_product_fwd(q, k, v, state_in=fstate(d["S0"]), state_out=st)
    torch.cuda.synchronize()
    ref, Sref = orc.fwd(d["Q"], d["K"], d["V"], S0=d["S0"], return_state=True)
    check(host(out), ref, dtype, f"fwd from S0 {dtype} {shape}")
    check(host(st), Sref, "f32", f"final state from S0 {dtype} {shape}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fwd_in_two_pieces(cp, orc, dtype):
    """Pieces carried through the fp32 state equal the one-piece call."""
    shape = (2, 2, 700, 64, 64)
    N, H, L, E, M = shape
    d = inputs(shape, dtype, seed=12)
    q, k, v = dev(d["Q"], dtype), dev(d["K"], dtype), dev(d["V"], dtype)
    full = cp.causal_product_fwd(q, k, v)
    for cut in (1, 64, 333):
        sa = torch.empty((N, H, E, M), device="cuda")
        sb = torch.empty_like(sa)
        a = cp.causal_product_fwd(q[:, :, :cut].contiguous(), k[:, :, :cut].contiguous(),
                                  v[:, :, :cut].contiguous(), state_out=sa)
        b = cp.causal_product_fwd(q[:, :, cut:].contiguous(), k[:, :, cut:].contiguous(),
                                  v[:, :, cut:].contiguous(), state_in=sa, state_out=sb)
        torch.cuda.synchronize()
        check(host(torch.cat([a, b], dim=2)), host(full), dtype, f"two pieces at {cut} {dtype}")
        check(host(sb), orc.state(d["K"], d["V"]), "f32", f"final state of the pieces at {cut} {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_bwd_from_state(cp, orc, dtype, shape):
    """With the initial state: the query gradient uses S0 (through the
    forward's final state, or through the kernel's own pre-pass from S0), and
    the gradient of S0 is sum_i q_i dO_i^T."""
    N, H, L, E, M = shape
    d = inputs(shape, dtype, seed=13)
    q, k, v, g = (dev(d[n], dtype) for n in ("Q", "K", "V", "dO"))
    s0 = fstate(d["S0"])
    st = torch.empty((N, H, E, M), device="cuda")
    cp.causal_product_fwd(q, k, v, state_in=s0, state_out=st)
    ref = orc.bwd(d["Q"], d["K"], d["V"], d["dO"], S0=d["S0"], with_dS0=True)
    for label, kw in (("final state", dict(state_final=st)), ("pre-pass from S0", dict(state_in=s0))):
        ds0 = torch.empty((N, H, E, M), device="cuda")
        got = cp.causal_product_bwd(q, k, v, g, dstate_in=ds0, **kw)
        torch.cuda.synchronize()
        for t, r, name in zip(list(got) + [ds0], ref, ("dq", "dk", "dv", "dS0")):
            check(host(t), r, dtype, f"{name} ({label}) {dtype} {shape}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("fm", [0, 1])
@pytest.mark.parametrize("shape", [(2, 3, 150, 64, 32), (1, 2, 1500, 128, 128)], ids=["small", "segments"])
def test_linattn_from_state(cp, orc, dtype, fm, shape):
    N, H, L, E, M = shape
    d = inputs(shape, dtype, seed=14, qk="raw" if fm else "elu1")
    q, k, v = dev(d["Q"], dtype), dev(d["K"], dtype), dev(d["V"], dtype)
    st = torch.empty((N, H, E, M), device="cuda")
    zt = torch.empty((N, H, E), device="cuda")
    out = cp.linear_attn_fwd(q, k, v, 1e-6, fm, state_in=fstate(d["S0"]), z_in=fstate(d["z0"]),
                             state_out=st, z_out=zt)
    torch.cuda.synchronize()
    ref, Sref, zref = orc.linattn(d["Q"], d["K"], d["V"], 1e-6, fm, S0=d["S0"], z0=d["z0"], return_state=True)
    check(host(out), ref, dtype, f"linattn from (S0, z0) fm={fm} {dtype} {shape}")
    # phi(k) enters the sums rounded to the I/O type, as in the output
    check(host(st), Sref, dtype, f"linattn final S fm={fm} {dtype}")
    check(host(zt), zref, dtype, f"linattn final z fm={fm} {dtype}")


def test_linattn_in_two_pieces(cp, orc):
    shape = (2, 2, 600, 64, 64)
    N, H, L, E, M = shape
    d = inputs(shape, "bf16", seed=15, qk="raw")
    q, k, v = dev(d["Q"], "bf16"), dev(d["K"], "bf16"), dev(d["V"], "bf16")
    full = cp.linear_attn_fwd(q, k, v, 1e-6, 1)
    sa = torch.empty((N, H, E, M), device="cuda")
    za = torch.empty((N, H, E), device="cuda")
    a = cp.linear_attn_fwd(q[:, :, :250].contiguous(), k[:, :, :250].contiguous(), v[:, :, :250].contiguous(),
                           1e-6, 1, state_out=sa, z_out=za)
    b = cp.linear_attn_fwd(q[:, :, 250:].contiguous(), k[:, :, 250:].contiguous(), v[:, :, 250:].contiguous(),
                           1e-6, 1, state_in=sa, z_in=za)
    torch.cuda.synchronize()
    check(host(torch.cat([a, b], dim=2)), host(full), "bf16", "linattn in two pieces")


def test_autograd_initial_state(cp, orc):
    shape = (1, 2, 300, 32, 64)
    N, H, L, E, M = shape
    d = inputs(shape, "f32", seed=16)
    q, k, v, g = (dev(d[n], "f32").requires_grad_(n != "dO") for n in ("Q", "K", "V", "dO"))
    s0 = fstate(d["S0"]).requires_grad_(True)
    out = cp.causal_product(q, k, v, s0)
    out.backward(g)
    torch.cuda.synchronize()
    ref = orc.bwd(d["Q"], d["K"], d["V"], d["dO"], S0=d["S0"], with_dS0=True)
    for t, r, name in zip((q.grad, k.grad, v.grad, s0.grad), ref, ("dq", "dk", "dv", "dS0")):
        check(host(t), r, "f32", f"autograd {name}")
