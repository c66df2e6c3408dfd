"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Metric: max|gpu - ref| / max|ref| per output tensor, fp64.  Bars: 1e-4 for
fp32 I/O, 2e-2 for bf16 I/O; bitwise equality on small-integer inputs whose
every partial sum and every value rounded to the I/O or operand precision is
exact.  Shapes span several chunks plus a ragged tail, every supported head
size, the five workloads at full size, and L = 1.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

# fp16: the bf16 bar scaled by the ratio of the unit roundoffs (2^-11 / 2^-8)
TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 2.5e-3}
TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


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
    """float32 numpy (values exact in dtype) -> contiguous device tensor."""
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(TORCH[dtype])


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def rand_inputs(N, H, L, E, M, dtype, seed, qk="elu1"):
    w = W.Workload("t", "fwd+bwd", dtype, N, H, L, E, M, seed=seed, qk=qk)
    return W.generate(w, need_do=True)


def say(msg):
    print(msg, flush=True)


HEADS = [(e, m) for e in (16, 32, 64, 128) for m in (16, 32, 64, 128)]


# -- forward -------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("E,M", HEADS)
def test_fwd_all_heads(cp, orc, dtype, E, M):
    say(f"fwd {dtype} E={E} M={M} L=75")
    d = rand_inputs(2, 3, 75, E, M, dtype, seed=E * 1000 + M)
    q, k, v = (dev(d[n], dtype) for n in "QKV")
    st = torch.empty((2, 3, E, M), device="cuda", dtype=torch.float32)
    out = cp.causal_product_fwd(q, k, v, state_out=st)
    torch.cuda.synchronize()
    ref = orc.fwd(d["Q"], d["K"], d["V"])
    assert oracle.max_rel_err(host(out), ref) <= TOL[dtype]
    assert oracle.max_rel_err(host(st), orc.state(d["K"], d["V"])) <= 1e-5


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("L", [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 200])
def test_fwd_lengths(cp, orc, dtype, L):
    say(f"fwd {dtype} L={L}")
    d = rand_inputs(1, 2, L, 64, 32, dtype, seed=L)
    q, k, v = (dev(d[n], dtype) for n in "QKV")
    out = cp.causal_product_fwd(q, k, v)
    torch.cuda.synchronize()
    ref = orc.fwd(d["Q"], d["K"], d["V"])
    assert oracle.max_rel_err(host(out), ref) <= TOL[dtype]
    if L <= 64:
        assert oracle.max_rel_err(host(out), orc.fwd_brute(d["Q"], d["K"], d["V"])) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fwd_l1_closed_form(cp, dtype):
    """L = 1: out_0 = (q_0 . k_0) v_0, bitwise on small integers."""
    say(f"fwd L=1 closed form {dtype}")
    rng = np.random.default_rng(5)
    # q.k <= 64 and |out| <= 192: exact as bf16 operands and outputs
    Q, K = (rng.integers(0, 2, size=(3, 2, 1, 64)).astype(np.float32) for _ in range(2))
    V = rng.integers(-3, 4, size=(3, 2, 1, 128)).astype(np.float32)
    out = cp.causal_product_fwd(dev(Q, dtype), dev(K, dtype), dev(V, dtype))
    exp = np.sum(Q.astype(np.float64) * K, -1, keepdims=True) * V
    assert np.array_equal(host(out), exp)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("E,M", [(16, 16), (64, 64), (32, 128), (128, 32)])
def test_fwd_integer_bitwise(cp, orc, dtype, E, M):
    """Small integers.  fp32: q, k, v in {0,1,2}, L = 40 -- scores <= 512,
    states <= 160, outputs <= 40960, all exact in fp32.  bf16: q, k in {0,1},
    v in {0,1,2}, L = 6 -- scores <= 128 and states <= 12 are exact bf16
    operands, and the exact fp32 result is rounded to bf16 once on both
    sides."""
    say(f"fwd integer bitwise {dtype} E={E} M={M}")
    L = 40 if dtype == "f32" else 6
    d = W.integer_inputs(2, 2, L, E, M, seed=3, lo=0, hi=2)
    if dtype == "bf16":
        d["Q"] = np.minimum(d["Q"], 1.0).astype(np.float32)
        d["K"] = np.minimum(d["K"], 1.0).astype(np.float32)
    out = cp.causal_product_fwd(dev(d["Q"], dtype), dev(d["K"], dtype), dev(d["V"], dtype))
    ref = orc.fwd(d["Q"], d["K"], d["V"])
    if dtype == "bf16":
        ref = W.round_bf16(ref.astype(np.float32)).astype(np.float64)
    assert np.array_equal(host(out), ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fwd_causality(cp, dtype):
    """Changing rows j > i of K and V leaves rows <= i bitwise unchanged."""
    say(f"fwd causality {dtype}")
    d = rand_inputs(1, 4, 130, 64, 64, dtype, seed=9)
    q, k, v = (dev(d[n], dtype) for n in "QKV")
    out1 = cp.causal_product_fwd(q, k, v)
    k2, v2 = k.clone(), v.clone()
    k2[:, :, 70:] *= 3
    v2[:, :, 70:] = -v2[:, :, 70:]
    out2 = cp.causal_product_fwd(q, k2, v2)
    torch.cuda.synchronize()
    assert torch.equal(out1[:, :, :70], out2[:, :, :70])
    assert not torch.equal(out1[:, :, 70:], out2[:, :, 70:])


# Few slices over a long sequence: the forward splits each slice into
# sequence segments (a state-increment pass, then sweeps that start from the
# sum of the earlier segments' increments).
SEG_SHAPES = [(1, 2, 2085, 64, 64), (1, 1, 4133, 128, 128), (2, 1, 3001, 32, 128)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SEG_SHAPES, ids=[str(s) for s in SEG_SHAPES])
def test_segmented_fwd_integer_bitwise(cp, orc, dtype, shape):
    """One-hot Q, K rows and V in {0, 1}: scores are 0 or 1, states count
    rows (a few dozen), outputs stay below 2^24, so every partial sum and
    every operand is exact; the output matches the oracle rounded once to the
    I/O type, the final state matches exactly."""
    say(f"segmented fwd integer bitwise {dtype} {shape}")
    N, H, L, E, M = shape
    d = W.onehot_inputs(N, H, L, E, M, seed=L, need_do=False)
    st = torch.empty((N, H, E, M), device="cuda", dtype=torch.float32)
    out = cp.causal_product_fwd(dev(d["Q"], dtype), dev(d["K"], dtype), dev(d["V"], dtype), state_out=st)
    torch.cuda.synchronize()
    ref, Sref = orc.fwd(d["Q"], d["K"], d["V"], return_state=True)
    assert Sref.max() <= 256  # exact as a bf16 operand
    if dtype == "bf16":
        ref = W.round_bf16(ref.astype(np.float32)).astype(np.float64)
    assert np.array_equal(host(out), ref)
    assert np.array_equal(host(st), Sref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("norm", [False, True])
def test_segmented_fwd_causality(cp, dtype, norm):
    """Few slices, long rows (segmented): changing rows j > i of K and V
    leaves rows <= i bitwise unchanged, across segment boundaries."""
    say(f"segmented fwd causality {dtype} norm={norm}")
    d = rand_inputs(1, 2, 3000, 64, 64, dtype, seed=19, qk="raw" if norm else "elu1")
    q, k, v = (dev(d[n], dtype) for n in "QKV")
    run = (lambda k_, v_: cp.linear_attn_fwd(q, k_, v_, 1e-6, 1)) if norm else \
        (lambda k_, v_: cp.causal_product_fwd(q, k_, v_))
    out1 = run(k, v)
    k2, v2 = k.clone(), v.clone()
    k2[:, :, 1501:] *= 3
    v2[:, :, 1501:] = -v2[:, :, 1501:]
    out2 = run(k2, v2)
    torch.cuda.synchronize()
    assert torch.equal(out1[:, :, :1501], out2[:, :, :1501])
    assert not torch.equal(out1[:, :, 1501:], out2[:, :, 1501:])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SEG_SHAPES[:2], ids=[str(s) for s in SEG_SHAPES[:2]])
def test_bwd_integer_bitwise_long(cp, orc, dtype, shape):
    """One-hot Q, K and V, dO in {0, 1} over a long sequence: prefix and
    suffix states count rows, every product and partial sum is a small exact
    integer, so dQ, dK, dV match the oracle rounded once to the I/O type
    (from the forward's final state and through the pre-pass)."""
    say(f"bwd integer bitwise long {dtype} {shape}")
    N, H, L, E, M = shape
    d = W.onehot_inputs(N, H, L, E, M, seed=L + 1)
    q, k, v, g = (dev(d[n], dtype) for n in ("Q", "K", "V", "dO"))
    st = torch.empty((N, H, E, M), device="cuda", dtype=torch.float32)
    cp.causal_product_fwd(q, k, v, state_out=st)
    ref = orc.bwd(d["Q"], d["K"], d["V"], d["dO"])
    if dtype == "bf16":
        ref = [W.round_bf16(r.astype(np.float32)).astype(np.float64) for r in ref]
    for use in (st, None):
        got = cp.causal_product_bwd(q, k, v, g, state_final=use)
        torch.cuda.synchronize()
        for t, r, name in zip(got, ref, ("dq", "dk", "dv")):
            assert np.array_equal(host(t), r), f"{name} state_final={use is not None}"


SEG_BWD_SHAPES = [(1, 2, 3001, 64, 64), (2, 1, 2500, 32, 128), (1, 1, 5000, 128, 128), (1, 3, 700, 64, 32)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SEG_BWD_SHAPES, ids=[str(s) for s in SEG_BWD_SHAPES])
def test_segmented_bwd(cp, orc, dtype, shape):
    """Few slices over long rows: the backward runs over sequence segments
    (segment increments of both carried states, then per-segment sweeps),
    from an initial state, with and without the forward's final state; dQ,
    dK, dV and the initial state's gradient against the oracle."""
    say(f"segmented bwd {dtype} {shape}")
    N, H, L, E, M = shape
    d = rand_inputs(N, H, L, E, M, dtype, seed=L + E)
    S0 = (np.random.default_rng(L).standard_normal((N, H, E, M)) * 3).astype(np.float32)
    q, k, v, g = (dev(d[n], dtype) for n in ("Q", "K", "V", "dO"))
    s0 = torch.from_numpy(S0).cuda()
    st = torch.empty((N, H, E, M), device="cuda", dtype=torch.float32)
    cp.causal_product_fwd(q, k, v, state_in=s0, state_out=st)
    ref = orc.bwd(d["Q"], d["K"], d["V"], d["dO"], S0=S0, with_dS0=True)
    for use in (st, None):
        ds0 = torch.empty_like(st)
        got = cp.causal_product_bwd(q, k, v, g, state_final=use, state_in=s0, dstate_in=ds0)
        torch.cuda.synchronize()
        for t, r, name in zip(list(got) + [ds0], ref, ("dq", "dk", "dv", "dS0")):
            err = oracle.max_rel_err(host(t), r)
            say(f"  {name} state_final={use is not None}: {err:.3e}")
            assert err <= TOL[dtype], name


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fwd_zero_state(cp, dtype):
    """V = 0 or K = 0 gives exactly zero (the zero-state probe)."""
    d = rand_inputs(1, 2, 50, 32, 32, dtype, seed=4)
    q, k, v = (dev(d[n], dtype) for n in "QKV")
    assert not cp.causal_product_fwd(q * 100, k, torch.zeros_like(v)).any()
    assert not cp.causal_product_fwd(q * 100, torch.zeros_like(k), v).any()


def test_fwd_guard_bands_and_stream(cp, orc):
    """Outputs written in place inside a larger buffer: the bytes around them
    stay untouched; the call runs on a non-default stream."""
    say("fwd guard bands")
    d = rand_inputs(2, 2, 77, 64, 64, "bf16", seed=12)
    q, k, v = (dev(d[n], "bf16") for n in "QKV")
    n = v.numel()
    big = torch.full((n + 4096,), 7.0, device="cuda", dtype=torch.bfloat16)
    out = big[2048:2048 + n].view(v.shape)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        cp.causal_product_fwd(q, k, v, out=out)
    s.synchronize()
    assert torch.all(big[:2048] == 7.0) and torch.all(big[2048 + n:] == 7.0)
    assert oracle.max_rel_err(host(out), orc.fwd(d["Q"], d["K"], d["V"])) <= 2e-2


# -- backward --------------------------------------------------------------------

def _bwd_check(cp, orc, d, dtype, use_state, tol=None):
    q, k, v, g = (dev(d[n], dtype) for n in ("Q", "K", "V", "dO"))
    st = None
    if use_state:
        N, H, L, E = q.shape
        st = torch.empty((N, H, E, v.shape[-1]), device="cuda", dtype=torch.float32)
        cp.causal_product_fwd(q, k, v, state_out=st)
    dq, dk, dv = cp.causal_product_bwd(q, k, v, g, state_final=st)
    torch.cuda.synchronize()
    ref = orc.bwd(d["Q"], d["K"], d["V"], d["dO"])
    errs = [oracle.max_rel_err(host(a), b) for a, b in zip((dq, dk, dv), ref)]
    assert max(errs) <= (tol or TOL[dtype]), errs
    return dq, dk, dv


@pytest.mark.parametrize("use_state", [True, False])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("E,M", HEADS)
def test_bwd_all_heads(cp, orc, dtype, E, M, use_state):
    say(f"bwd {dtype} E={E} M={M} state={use_state}")
    d = rand_inputs(2, 2, 70, E, M, dtype, seed=E * 7 + M)
    _bwd_check(cp, orc, d, dtype, use_state)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("L", [1, 2, 16, 31, 33, 64, 97])
def test_bwd_lengths(cp, orc, dtype, L):
    say(f"bwd {dtype} L={L}")
    d = rand_inputs(1, 3, L, 32, 64, dtype, seed=100 + L)
    _bwd_check(cp, orc, d, dtype, True)
    _bwd_check(cp, orc, d, dtype, False)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_integer_bitwise(cp, orc, dtype):
    """Integers in {0,1,2}: the gradients are exact (bf16 I/O uses L = 4 so
    that every output is exact in bf16)."""
    say(f"bwd integer bitwise {dtype}")
    L = 40 if dtype == "f32" else 4
    d = W.integer_inputs(1, 3, L, 32, 64, seed=8, lo=0, hi=2)
    q, k, v, g = (dev(d[n], dtype) for n in ("Q", "K", "V", "dO"))
    st = torch.empty((1, 3, 32, 64), device="cuda", dtype=torch.float32)
    cp.causal_product_fwd(q, k, v, state_out=st)
    ref = orc.bwd(d["Q"], d["K"], d["V"], d["dO"])
    for state in (st, None):
        got = cp.causal_product_bwd(q, k, v, g, state_final=state)
        for a, b in zip(got, ref):
            if dtype == "bf16":
                b = W.round_bf16(b.astype(np.float32)).astype(np.float64)
            assert np.array_equal(host(a), b)


def test_bwd_homogeneity_on_gpu(cp):
    """<dO, out> = <Q, dQ> = <K, dK> = <V, dV> on the GPU's own results."""
    d = rand_inputs(2, 2, 300, 64, 64, "f32", seed=21)
    q, k, v, g = (dev(d[n], "f32") for n in ("Q", "K", "V", "dO"))
    out = cp.causal_product_fwd(q, k, v)
    dq, dk, dv = cp.causal_product_bwd(q, k, v, g)
    f = float((out.double() * g.double()).sum())
    for x, gx in ((q, dq), (k, dk), (v, dv)):
        assert abs(float((x.double() * gx.double()).sum()) - f) <= 1e-5 * abs(f)


def test_autograd_wrapper(cp, orc):
    d = rand_inputs(1, 2, 90, 64, 64, "bf16", seed=31)
    q, k, v = (dev(d[n], "bf16").requires_grad_(True) for n in "QKV")
    g = dev(d["dO"], "bf16")
    out = cp.causal_product(q, k, v)
    out.backward(g)
    ref = orc.bwd(d["Q"], d["K"], d["V"], d["dO"])
    assert oracle.max_rel_err(host(out.detach()), orc.fwd(d["Q"], d["K"], d["V"])) <= 2e-2
    for t, r in zip((q, k, v), ref):
        assert oracle.max_rel_err(host(t.grad), r) <= 2e-2


# -- normalised forward -------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("E,M", [(16, 16), (32, 128), (64, 64), (128, 128), (128, 16)])
@pytest.mark.parametrize("fm", [1, 0])
def test_linattn(cp, orc, dtype, E, M, fm):
    say(f"linattn {dtype} E={E} M={M} fm={fm}")
    d = rand_inputs(2, 2, 83, E, M, dtype, seed=E + M + fm, qk="raw" if fm else "elu1")
    q, k, v = (dev(d[n], dtype) for n in "QKV")
    out = cp.linear_attn_fwd(q, k, v, 1e-6, fm)
    torch.cuda.synchronize()
    ref = orc.linattn(d["Q"], d["K"], d["V"], 1e-6, fm)
    assert oracle.max_rel_err(host(out), ref) <= TOL[dtype]


@pytest.mark.parametrize("L", [1, 17, 32, 95])
def test_linattn_lengths_and_brute(cp, orc, L):
    d = rand_inputs(1, 2, L, 64, 32, "f32", seed=L, qk="raw")
    q, k, v = (dev(d[n], "f32") for n in "QKV")
    out = host(cp.linear_attn_fwd(q, k, v, 1e-6, 1))
    assert oracle.max_rel_err(out, orc.linattn(d["Q"], d["K"], d["V"], 1e-6, 1)) <= 1e-4
    assert oracle.max_rel_err(out, orc.linattn_brute(d["Q"], d["K"], d["V"], 1e-6, 1)) <= 1e-4


def test_linattn_constant_v(cp):
    """v_j = c: out_i = c (q.z)/(q.z + eps), i.e. c up to eps / den."""
    rng = np.random.default_rng(2)
    Q = rng.standard_normal((1, 2, 60, 32)).astype(np.float32)
    K = rng.standard_normal((1, 2, 60, 32)).astype(np.float32)
    V = np.full((1, 2, 60, 16), 1.5, np.float32)
    out = host(cp.linear_attn_fwd(dev(Q, "f32"), dev(K, "f32"), dev(V, "f32"), 1e-6, 1))
    assert np.max(np.abs(out - 1.5)) <= 1e-5


# -- the workloads at full size -----------------------------------------------------------

@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_workload_full_size(cp, orc, name):
    w = W.WORKLOADS[name]
    say(f"workload {name} {w}")
    d = W.generate(w)
    q, k, v = (dev(d[n], w.dtype) for n in "QKV")
    tol = TOL[w.dtype]
    if w.op.startswith("linattn"):
        st = torch.empty((w.N, w.H, w.E, w.M), device="cuda", dtype=torch.float32)
        zt = torch.empty((w.N, w.H, w.E), device="cuda", dtype=torch.float32)
        den = torch.empty((w.N, w.H, w.L), device="cuda", dtype=torch.float32)
        out = cp.linear_attn_fwd(q, k, v, 1e-6, 1, state_out=st, z_out=zt, den_out=den)
        torch.cuda.synchronize()
        err = oracle.max_rel_err(host(out), orc.linattn(d["Q"], d["K"], d["V"], 1e-6, 1))
        say(f"  linattn err {err:.3e}")
        assert err <= tol
        if w.op == "linattn+bwd":
            g = dev(d["dO"], w.dtype)
            got = cp.linear_attn_bwd(q, k, v, out, g, den, 1, state_final=st, z_final=zt)
            torch.cuda.synchronize()
            ref = orc.linattn_bwd(d["Q"], d["K"], d["V"], d["dO"], 1e-6, 1)
            errs = [oracle.max_rel_err(host(a), b) for a, b in zip(got, ref)]
            say(f"  linattn bwd errs {errs}")
            assert max(errs) <= tol
        return
    st = torch.empty((w.N, w.H, w.E, w.M), device="cuda", dtype=torch.float32)
    out = cp.causal_product_fwd(q, k, v, state_out=st)
    torch.cuda.synchronize()
    err = oracle.max_rel_err(host(out), orc.fwd(d["Q"], d["K"], d["V"]))
    say(f"  fwd err {err:.3e}")
    assert err <= tol
    if w.L <= 64:
        assert oracle.max_rel_err(host(out), orc.fwd_brute(d["Q"], d["K"], d["V"])) <= tol
    if w.op == "fwd+bwd":
        g = dev(d["dO"], w.dtype)
        dq, dk, dv = cp.causal_product_bwd(q, k, v, g, state_final=st)
        torch.cuda.synchronize()
        ref = orc.bwd(d["Q"], d["K"], d["V"], d["dO"])
        errs = [oracle.max_rel_err(host(a), b) for a, b in zip((dq, dk, dv), ref)]
        say(f"  bwd errs {errs}")
        assert max(errs) <= tol
