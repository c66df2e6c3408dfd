"""Head sizes other than the kernel tiles {16, 32, 64, 128}, on the GPU,
against the fp64 oracle, through the C ABI.

A head of E (or M) features runs on the smallest tile that holds it: its
rows are loaded with the padding columns as zero and only its own columns
are stored.  Checked here for every entry point, every dtype, with carried
states and their gradients, a ragged tail and a sequence long enough for the
segmented forward; bitwise on small integers; and guard bands around the
outputs, which a store into a padding column would overwrite.  Same metric
and bars as the other parity tests (max|gpu - ref| / max|ref|: fp32 1e-4,
bf16 2e-2, fp16 2.5e-3).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 2.5e-3}
TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
# rows of whole 16-byte pieces: multiples of 8 (16-bit types) or 4 (fp32)
HEADS16 = [(8, 8), (24, 40), (48, 80), (96, 112), (120, 72), (40, 128), (128, 48), (8, 128), (112, 16)]
HEADS32 = [(4, 12), (20, 36), (48, 80), (100, 60), (128, 44), (12, 128)]
CASES = [("bf16", e, m) for e, m in HEADS16] + [("f16", e, m) for e, m in HEADS16[:5]] + \
        [("f32", e, m) for e, m in HEADS32]


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


def fstate(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def inputs(N, H, L, E, M, dtype, seed, qk="elu1"):
    d = W.generate(W.Workload("heads", "fwd+bwd", dtype, N, H, L, E, M, seed=seed, qk=qk), need_do=True)
    r = np.random.default_rng(seed + 1000)
    d["S0"] = (r.standard_normal((N, H, E, M)) * 20).astype(np.float32)
    d["z0"] = (r.random((N, H, E)) * 100 + 1).astype(np.float32)
    return d


def check(got, ref, tol, what):
    err = oracle.max_rel_err(got, ref)
    print(f"{what}: max rel err {err:.3e}", flush=True)
    assert err <= tol, what


@pytest.mark.parametrize("dtype,E,M", CASES, ids=[f"{d}-E{e}-M{m}" for d, e, m in CASES])
def test_padded_heads_fwd_bwd(cp, orc, dtype, E, M):
    N, H, L = 2, 3, 75
    print(f"padded heads {dtype} E={E} M={M} L={L}", flush=True)
    d = inputs(N, H, L, E, M, dtype, seed=E * 1000 + M)
    q, k, v, g = (dev(d[n], dtype) for n in ("Q", "K", "V", "dO"))
    s0 = fstate(d["S0"])
    st = torch.empty((N, H, E, M), device="cuda")
    out = cp.causal_product_fwd(q, k, v, state_in=s0, state_out=st)
    torch.cuda.synchronize()
    ref, Sref = orc.fwd(d["Q"], d["K"], d["V"], S0=d["S0"], return_state=True)
    check(host(out), ref, TOL[dtype], "out")
    check(host(st), Sref, min(TOL[dtype], 1e-4), "final state")
    bref = orc.bwd(d["Q"], d["K"], d["V"], d["dO"], S0=d["S0"], with_dS0=True)
    for label, kw in (("final state", dict(state_final=st)), ("pre-pass", dict(state_in=s0))):
        ds0 = torch.empty((N, H, E, M), device="cuda")
        got = cp.causal_product_bwd(q, k, v, g, dstate_in=ds0, **kw)
        torch.cuda.synchronize()
        for t, r, name in zip(list(got) + [ds0], bref, ("dq", "dk", "dv", "dS0")):
            check(host(t), r, TOL[dtype] if name != "dS0" else min(TOL[dtype], 1e-4), f"{name} ({label})")


@pytest.mark.parametrize("dtype,E,M", [("bf16", 48, 80), ("bf16", 24, 120), ("f16", 40, 96), ("f32", 20, 36),
                                       ("f32", 100, 60)])
@pytest.mark.parametrize("fm", [0, 1])
def test_padded_heads_linattn(cp, orc, dtype, E, M, fm):
    """Normalised forward and (bf16, fp32) backward: phi(0) = 1 must not leak
    into the padding features of q and k."""
    N, H, L = 2, 2, 97
    print(f"padded linattn {dtype} E={E} M={M} fm={fm}", flush=True)
    d = inputs(N, H, L, E, M, dtype, seed=E + M + fm, qk="raw" if fm else "elu1")
    q, k, v, g = (dev(d[n], dtype) for n in ("Q", "K", "V", "dO"))
    s0, z0 = fstate(d["S0"]), fstate(d["z0"])
    st = torch.empty((N, H, E, M), device="cuda")
    zt = torch.empty((N, H, E), device="cuda")
    den = torch.empty((N, H, L), device="cuda")
    out = cp.linear_attn_fwd(q, k, v, 1e-6, fm, state_in=s0, z_in=z0, state_out=st, z_out=zt, den_out=den)
    torch.cuda.synchronize()
    ref, Sref, zref = orc.linattn(d["Q"], d["K"], d["V"], 1e-6, fm, S0=d["S0"], z0=d["z0"], return_state=True)
    check(host(out), ref, TOL[dtype], "out")
    check(host(st), Sref, TOL[dtype], "final S")
    check(host(zt), zref, TOL[dtype], "final z")
    if dtype == "f16":
        return  # no fp16 normalised backward
    ds0 = torch.empty((N, H, E, M), device="cuda")
    dz0 = torch.empty((N, H, E), device="cuda")
    got = cp.linear_attn_bwd(q, k, v, out, g, den, fm, state_in=s0, z_in=z0, state_final=st, z_final=zt,
                             dstate_in=ds0,
                             dz_in=dz0)
    torch.cuda.synchronize()
    bref = orc.linattn_bwd(d["Q"], d["K"], d["V"], d["dO"], 1e-6, fm, S0=d["S0"], z0=d["z0"])
    for t, r, name in zip(list(got) + [ds0, dz0], bref, ("dq", "dk", "dv", "dS0", "dz0")):
        check(host(t), r, TOL[dtype], name)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_padded_heads_segments(cp, orc, dtype):
    """Two slices over 1500 rows (the forward runs as sequence segments)."""
    E, M = (48, 80) if dtype == "bf16" else (20, 36)
    d = inputs(1, 2, 1500, E, M, dtype, seed=31, qk="raw")
    q, k, v = (dev(d[n], dtype) for n in "QKV")
    out = cp.causal_product_fwd(q, k, v)
    lo = cp.linear_attn_fwd(q, k, v, 1e-6, 1)
    torch.cuda.synchronize()
    # causal product of the raw draws: signed inputs, still the same definition
    check(host(out), orc.fwd(d["Q"], d["K"], d["V"]), TOL[dtype], "segments fwd")
    check(host(lo), orc.linattn(d["Q"], d["K"], d["V"], 1e-6, 1), TOL[dtype], "segments linattn")


@pytest.mark.parametrize("dtype,E,M", [("bf16", 24, 40), ("f16", 8, 56), ("f32", 20, 12)])
def test_padded_heads_integer_bitwise(cp, orc, dtype, E, M):
    """q, k in {0, 1}, v, dO in {0, 1, 2}, L = 6: every product and partial
    sum exact; the exact result is rounded to the I/O type once on both
    sides."""
    d = W.integer_inputs(2, 2, 6, E, M, seed=5, lo=0, hi=2)
    d["Q"] = np.minimum(d["Q"], 1.0).astype(np.float32)
    d["K"] = np.minimum(d["K"], 1.0).astype(np.float32)
    q, k, v, g = (dev(d[n], dtype) for n in ("Q", "K", "V", "dO"))
    out = cp.causal_product_fwd(q, k, v)
    grads = cp.causal_product_bwd(q, k, v, g)
    torch.cuda.synchronize()
    rnd = {"f32": lambda x: x, "bf16": lambda x: W.round_bf16(x.astype(np.float32)).astype(np.float64),
           "f16": lambda x: x.astype(np.float16).astype(np.float64)}[dtype]
    assert np.array_equal(host(out), rnd(orc.fwd(d["Q"], d["K"], d["V"])))
    for t, r in zip(grads, orc.bwd(d["Q"], d["K"], d["V"], d["dO"])):
        assert np.array_equal(host(t), rnd(r))


def _guarded(shape, dtype, pad=4096):
    n = int(np.prod(shape))
    big = torch.full((n + 2 * pad,), 7.0, device="cuda", dtype=TORCH[dtype])
    return big, big[pad:pad + n].view(shape), pad, n


@pytest.mark.parametrize("dtype,E,M", [("bf16", 40, 24), ("f32", 12, 20)])
def test_padded_heads_guard_bands(cp, dtype, E, M):
    """Outputs placed inside larger buffers: nothing is written outside them
    (the padding columns of the last rows would land past the end)."""
    N, H, L = 1, 2, 37
    d = inputs(N, H, L, E, M, dtype, seed=3)
    q, k, v, g = (dev(d[n], dtype) for n in ("Q", "K", "V", "dO"))
    bo, out, pad, n = _guarded((N, H, L, M), dtype)
    cp.causal_product_fwd(q, k, v, out=out)
    bufs = [_guarded((N, H, L, E), dtype), _guarded((N, H, L, E), dtype), _guarded((N, H, L, M), dtype)]
    cp.causal_product_bwd(q, k, v, g, dq=bufs[0][1], dk=bufs[1][1], dv=bufs[2][1])
    torch.cuda.synchronize()
    for big, _, p, m in [(bo, out, pad, n)] + bufs:
        assert torch.all(big[:p] == 7.0) and torch.all(big[p + m:] == 7.0)
    assert torch.equal(out, cp.causal_product_fwd(q, k, v))
    for (_, t, _, _), r in zip(bufs, cp.causal_product_bwd(q, k, v, g)):
        assert torch.equal(t, r)
