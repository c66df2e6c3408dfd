"""fp16 (IEEE half) I/O of the HIP path against the fp64 oracle, through the
C ABI.

Metric as for the other dtypes: max|gpu - ref| / max|ref| per output tensor.
Bar: 2.5e-3 -- the bf16 bar (2e-2) scaled by the ratio of the two types' unit
roundoffs (2^-11 / 2^-8): the kernels compute fp16 exactly as bf16 (fp32
accumulation, states and score tiles rounded once to the I/O type as matrix
operands), so their error scales with the operand rounding.  Bitwise
equality on small integers whose every partial sum and operand is exact.
The normalised backward refuses fp16 (CP_ERR_UNSUPPORTED).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL = 2.5e-3
HEADS = [(e, m) for e in (16, 32, 64, 128) for m in (16, 32, 64, 128)]


@pytest.fixture(scope="module")
def cp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import prefix_sum_causal_amd as cp
    return cp


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(torch.float16)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def inputs(N, H, L, E, M, seed, qk="elu1"):
    return W.generate(W.Workload("t", "fwd+bwd", "f16", N, H, L, E, M, seed=seed, qk=qk), need_do=True)


def say(msg):
    print(msg, flush=True)


def test_workload_rounding_is_half():
    d = inputs(1, 1, 8, 16, 16, seed=1)
    for x in d.values():
        assert np.array_equal(x, x.astype(np.float16).astype(np.float32))


@pytest.mark.parametrize("E,M", HEADS)
def test_f16_fwd_bwd_all_heads(cp, orc, E, M):
    say(f"f16 fwd+bwd E={E} M={M} L=75")
    d = inputs(2, 3, 75, E, M, seed=E * 100 + M)
    q, k, v, g = (dev(d[n]) for n in ("Q", "K", "V", "dO"))
    st = torch.empty((2, 3, E, M), device="cuda", dtype=torch.float32)
    out = cp.causal_product_fwd(q, k, v, state_out=st)
    grads_saved = cp.causal_product_bwd(q, k, v, g, state_final=st)
    grads_prepass = cp.causal_product_bwd(q, k, v, g)
    torch.cuda.synchronize()
    assert oracle.max_rel_err(host(out), orc.fwd(d["Q"], d["K"], d["V"])) <= TOL
    assert oracle.max_rel_err(host(st), orc.state(d["K"], d["V"])) <= 1e-5
    refs = orc.bwd(d["Q"], d["K"], d["V"], d["dO"])
    for grads in (grads_saved, grads_prepass):
        for name, t, ref in zip(("dq", "dk", "dv"), grads, refs):
            assert oracle.max_rel_err(host(t), ref) <= TOL, name


@pytest.mark.parametrize("L", [1, 16, 17, 33, 63, 65, 97, 200])
def test_f16_lengths(cp, orc, L):
    say(f"f16 lengths L={L}")
    d = inputs(1, 2, L, 64, 32, seed=L)
    q, k, v, g = (dev(d[n]) for n in ("Q", "K", "V", "dO"))
    out = cp.causal_product_fwd(q, k, v)
    grads = cp.causal_product_bwd(q, k, v, g)
    torch.cuda.synchronize()
    assert oracle.max_rel_err(host(out), orc.fwd(d["Q"], d["K"], d["V"])) <= TOL
    if L <= 64:
        assert oracle.max_rel_err(host(out), orc.fwd_brute(d["Q"], d["K"], d["V"])) <= TOL
    for t, ref in zip(grads, orc.bwd(d["Q"], d["K"], d["V"], d["dO"])):
        assert oracle.max_rel_err(host(t), ref) <= TOL


@pytest.mark.parametrize("E,M", [(16, 16), (64, 64), (32, 128), (128, 32)])
def test_f16_integer_bitwise(cp, orc, E, M):
    """q, k in {0, 1}, v, dO in {0, 1, 2}, L = 12: scores <= 128, states and
    suffix sums <= 24 and every fp32 partial sum are exact half operands and
    exact fp32; the exact result is rounded to half once on both sides."""
    say(f"f16 integer bitwise E={E} M={M}")
    d = W.integer_inputs(2, 2, 12, E, M, seed=7, lo=0, hi=2)
    d["Q"] = np.minimum(d["Q"], 1.0).astype(np.float32)
    d["K"] = np.minimum(d["K"], 1.0).astype(np.float32)
    q, k, v, g = (dev(d[n]) for n in ("Q", "K", "V", "dO"))
    out = cp.causal_product_fwd(q, k, v)
    grads = cp.causal_product_bwd(q, k, v, g)
    torch.cuda.synchronize()
    half = lambda x: x.astype(np.float16).astype(np.float64)
    assert np.array_equal(host(out), half(orc.fwd(d["Q"], d["K"], d["V"])))
    for t, ref in zip(grads, orc.bwd(d["Q"], d["K"], d["V"], d["dO"])):
        assert np.array_equal(host(t), half(ref))


@pytest.mark.parametrize("E,M", [(16, 64), (64, 64), (128, 128), (32, 16)])
@pytest.mark.parametrize("fm", [0, 1])
def test_f16_linattn_fwd(cp, orc, E, M, fm):
    say(f"f16 linattn E={E} M={M} fm={fm}")
    d = inputs(2, 2, 150, E, M, seed=E + M + fm, qk="raw" if fm else "elu1")
    den = torch.empty((2, 2, 150), device="cuda", dtype=torch.float32)
    out = cp.linear_attn_fwd(*(dev(d[n]) for n in "QKV"), 1e-6, fm, den_out=den)
    torch.cuda.synchronize()
    assert oracle.max_rel_err(host(out), orc.linattn(d["Q"], d["K"], d["V"], 1e-6, fm)) <= TOL


def test_f16_linattn_segments(cp, orc):
    """Two slices over 1500 rows: the forward runs as sequence segments."""
    say("f16 linattn segments")
    d = inputs(1, 2, 1500, 64, 64, seed=15, qk="raw")
    out = cp.linear_attn_fwd(*(dev(d[n]) for n in "QKV"), 1e-6, 1)
    torch.cuda.synchronize()
    assert oracle.max_rel_err(host(out), orc.linattn(d["Q"], d["K"], d["V"], 1e-6, 1)) <= TOL


def test_f16_linattn_bwd_refused(cp):
    d = inputs(1, 1, 32, 32, 32, seed=2, qk="raw")
    q, k, v, g = (dev(d[n]) for n in ("Q", "K", "V", "dO"))
    den = torch.ones((1, 1, 32), device="cuda", dtype=torch.float32)
    with pytest.raises(cp.CausalProductError) as e:
        cp.linear_attn_bwd(q, k, v, v.clone(), g, den, 1)
    assert e.value.status == 3


def test_f16_autograd(cp, orc):
    say("f16 autograd")
    d = inputs(2, 2, 90, 32, 64, seed=21)
    q, k, v = (dev(d[n]).requires_grad_(True) for n in "QKV")
    out = cp.causal_product(q, k, v)
    out.backward(dev(d["dO"]))
    torch.cuda.synchronize()
    assert out.dtype == torch.float16
    assert oracle.max_rel_err(host(out), orc.fwd(d["Q"], d["K"], d["V"])) <= TOL
    for t, ref in zip((q, k, v), orc.bwd(d["Q"], d["K"], d["V"], d["dO"])):
        assert oracle.max_rel_err(host(t.grad), ref) <= TOL
