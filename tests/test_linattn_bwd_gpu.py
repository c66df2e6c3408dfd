"""Parity of the backward of the normalised form (linear_attn_bwd) and of
the forward's denominators on the GPU against the fp64 oracle, through the C
ABI and through the autograd wrapper.

Same metric and bars as the other parity tests (max|gpu - ref| / max|ref| per
tensor, 1e-4 for fp32 I/O, 2e-2 for bf16 I/O).  Raw Q, K are N(0,1), so both
branches of phi = elu + 1 are used; shapes have ragged tails, E != M, a wide
head and two slices over 1500 rows.  The backward runs from the forward's
final states (S and z) and, separately, from the initial states through its
own forward pre-pass (also taken when only S is given).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
TORCH = {"f32": torch.float32, "bf16": torch.bfloat16}
SHAPES = [(2, 3, 150, 64, 32), (1, 2, 77, 32, 128), (1, 2, 1500, 64, 64), (2, 1, 100, 128, 128)]


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


def fdev(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(got, ref, dtype, what):
    err = oracle.max_rel_err(got, ref)
    print(f"{what}: max rel err {err:.3e}", flush=True)
    assert err <= TOL[dtype], what


def inputs(shape, dtype, seed, fm, carry):
    N, H, L, E, M = shape
    w = W.Workload("linbwd", "fwd+bwd", dtype, N, H, L, E, M, seed=seed, qk="raw" if fm else "elu1")
    d = W.generate(w, need_do=True)
    if carry:
        r = np.random.default_rng(seed + 2000)
        d["S0"] = (r.standard_normal((N, H, E, M)) * 5).astype(np.float32)
        d["z0"] = (r.random((N, H, E)) * 20 + 1).astype(np.float32)
    else:
        d["S0"] = d["z0"] = None
    return d


def forward(cp, d, dtype, fm):
    q, k, v = dev(d["Q"], dtype), dev(d["K"], dtype), dev(d["V"], dtype)
    N, H, L, E = q.shape
    M = v.shape[-1]
    st = torch.empty((N, H, E, M), device="cuda")
    zt = torch.empty((N, H, E), device="cuda")
    den = torch.empty((N, H, L), device="cuda")
    s0 = fdev(d["S0"]) if d["S0"] is not None else None
    z0 = fdev(d["z0"]) if d["z0"] is not None else None
    out = cp.linear_attn_fwd(q, k, v, 1e-6, fm, state_in=s0, z_in=z0, state_out=st, z_out=zt, den_out=den)
    return q, k, v, out, st, zt, den, s0, z0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("fm", [1, 0])
@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_linattn_bwd(cp, orc, dtype, fm, shape):
    carry = shape[2] != 1500
    d = inputs(shape, dtype, seed=21, fm=fm, carry=carry)
    q, k, v, out, st, zt, den, s0, z0 = forward(cp, d, dtype, fm)
    g = dev(d["dO"], dtype)
    ref = orc.linattn_bwd(d["Q"], d["K"], d["V"], d["dO"], 1e-6, fm, S0=d["S0"], z0=d["z0"])
    for label, kw in (("final states", dict(state_final=st, z_final=zt, state_in=s0, z_in=z0)),
                      ("pre-pass", dict(state_in=s0, z_in=z0)),
                      ("S only", dict(state_final=st, state_in=s0, z_in=z0))):
        ds0 = torch.empty_like(st)
        dz0 = torch.empty_like(zt)
        got = cp.linear_attn_bwd(q, k, v, out, g, den, fm, dstate_in=ds0, dz_in=dz0, **kw)
        torch.cuda.synchronize()
        for t, r, name in zip(list(got) + [ds0, dz0], ref, ("dq", "dk", "dv", "dS0", "dz0")):
            check(host(t), r, dtype, f"{name} ({label}) fm={fm} {dtype} {shape}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_denominators(cp, orc, dtype):
    """den_out_i = phi(q_i) . (z0 + sum_{j<=i} phi(k_j)) + eps."""
    shape = (2, 2, 333, 64, 32)
    d = inputs(shape, dtype, seed=22, fm=1, carry=True)
    _, _, _, _, _, _, den, _, _ = forward(cp, d, dtype, 1)
    torch.cuda.synchronize()
    phi = lambda x: np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))
    c, f = phi(d["Q"].astype(np.float64)), phi(d["K"].astype(np.float64))
    z = d["z0"][..., None, :].astype(np.float64) + np.cumsum(f, axis=-2)
    ref = (c * z).sum(-1) + 1e-6
    check(host(den), ref, dtype, f"denominators {dtype}")


def test_autograd(cp, orc):
    shape = (1, 2, 260, 32, 64)
    d = inputs(shape, "f32", seed=23, fm=1, carry=False)
    q, k, v = (dev(d[n], "f32").requires_grad_(True) for n in ("Q", "K", "V"))
    out = cp.linear_attention(q, k, v)
    out.backward(dev(d["dO"], "f32"))
    torch.cuda.synchronize()
    check(host(out), orc.linattn(d["Q"], d["K"], d["V"], 1e-6, 1), "f32", "autograd forward")
    ref = orc.linattn_bwd(d["Q"], d["K"], d["V"], d["dO"], 1e-6, 1)
    for t, r, name in zip((q.grad, k.grad, v.grad), ref, ("dq", "dk", "dv")):
        check(host(t), r, "f32", f"autograd {name}")


def _both_paths(cp, d, dtype, fm, ref, label):
    q, k, v, out, st, zt, den, s0, z0 = forward(cp, d, dtype, fm)
    g = dev(d["dO"], dtype)
    for path, kw in (("final states", dict(state_final=st, z_final=zt)), ("pre-pass", {})):
        got = cp.linear_attn_bwd(q, k, v, out, g, den, fm, state_in=s0, z_in=z0, **kw)
        torch.cuda.synchronize()
        for t, r, name in zip(got, ref, ("dq", "dk", "dv")):
            check(host(t), r, dtype, f"{name} ({path}) {label}")


def test_linattn_bwd_long_f32(cp, orc):
    """fp32 I/O over 4133 rows: the query gradient peaks at the first rows,
    where the states recovered backwards are smallest next to it."""
    shape = (1, 2, 4133, 64, 64)
    d = inputs(shape, "f32", seed=24, fm=1, carry=False)
    ref = orc.linattn_bwd(d["Q"], d["K"], d["V"], d["dO"], 1e-6, 1)
    _both_paths(cp, d, "f32", 1, ref, f"f32 {shape}")


def dq_summand_scale(d, eps=1e-6, rows=1024):
    """Per row i and feature e, the magnitude of the terms whose sum is dq
    (fp64, feature map elu + 1):
        T_ie = phi'(q_ie) (sum_m |S_i[e, m]| |dn_im| + z_ie sum_m |dO_im| |out_im| / d_i),
    the scale that bounds the rounding error of that sum (each term enters
    with a few roundings of the I/O type), whatever the cancellation between
    S_i dn_i and dd_i z_i."""
    phi = lambda x: np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))
    Q, K, V, dO = (d[n].astype(np.float64) for n in ("Q", "K", "V", "dO"))
    N, H, L, E = Q.shape
    M = V.shape[-1]
    T = np.empty((N, H, L, E))
    for n in range(N):
        for h in range(H):
            c, f, v, g = phi(Q[n, h]), phi(K[n, h]), V[n, h], dO[n, h]
            S, Sa, z = np.zeros((E, M)), np.zeros((E, M)), np.zeros(E)
            for r0 in range(0, L, rows):
                sl = slice(r0, min(L, r0 + rows))
                fv = f[sl, :, None] * v[sl, None, :]
                Si = S + np.cumsum(fv, 0)                 # S_i, inclusive
                zi = z + np.cumsum(f[sl], 0)
                den = np.einsum("ie,ie->i", c[sl], zi) + eps
                out = np.einsum("ie,iem->im", c[sl], Si) / den[:, None]
                dn = np.abs(g[sl]) / den[:, None]
                T[n, h, sl] = (np.einsum("iem,im->ie", np.abs(Si), dn)
                               + zi * (np.abs(g[sl]) * np.abs(out)).sum(1)[:, None] / den[:, None]) \
                    * np.minimum(c[sl], 1.0)
                S, z = Si[-1], zi[-1]
    return T


def test_linattn_bwd_long_bf16_nonnegative_v(cp, orc):
    """bf16 I/O over 16384 rows with V >= 0: the final S grows like L (no
    cancellation between rows), the worst case for recovering early states
    by subtraction from the forward's final states.  There dq = S_i dn_i +
    dd_i z_i is a near cancellation of terms some 40 times larger than dq:
    even exact arithmetic on the bf16 forward output Out leaves an error of
    about 1.7e-2 of max|dq|, so dq is held to the bf16 rounding of its
    summands, row by row (|err_i| <= 2^-7 T_i, see dq_summand_scale), and
    the final-states path must do as well as the pre-pass path."""
    shape = (1, 1, 16384, 64, 64)
    d = inputs(shape, "bf16", seed=25, fm=1, carry=False)
    d["V"] = np.abs(d["V"])
    ref = orc.linattn_bwd(d["Q"], d["K"], d["V"], d["dO"], 1e-6, 1)
    T = dq_summand_scale(d).max(-1)
    q, k, v, out, st, zt, den, s0, z0 = forward(cp, d, "bf16", 1)
    g = dev(d["dO"], "bf16")
    errs = {}
    for path, kw in (("final states", dict(state_final=st, z_final=zt)), ("pre-pass", {})):
        got = cp.linear_attn_bwd(q, k, v, out, g, den, 1, **kw)
        torch.cuda.synchronize()
        dq = host(got[0])
        row = np.abs(dq - ref[0]).max(-1) / T
        errs[path] = oracle.max_rel_err(dq, ref[0])
        print(f"dq ({path}): max rel err {errs[path]:.3e}, worst row err / T {row.max():.3e} "
              f"at row {int(row.argmax(-1).max())}", flush=True)
        assert row.max() <= 2.0 ** -7, path
        for t, r, name in zip(got[1:], ref[1:], ("dk", "dv")):
            check(host(t), r, "bf16", f"{name} ({path}) bf16 V>=0 {shape}")
    assert errs["final states"] <= 1.1 * errs["pre-pass"] + 1e-3


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_row_error_profile(cp, orc, dtype):
    """Error of the normalised output and of dq in the first and last 10% of
    the rows (reported; gated only by the global bar).  Per band: max|err| /
    max|ref| over the band, and the worst row's max|err| relative to that
    row's scale: max|ref row| for the output, the summand scale T_i of
    dq_summand_scale for dq (dq itself vanishes at the first row)."""
    shape = (1, 2, 4096, 64, 64)
    d = inputs(shape, dtype, seed=26, fm=1, carry=False)
    q, k, v, out, st, zt, den, s0, z0 = forward(cp, d, dtype, 1)
    g = dev(d["dO"], dtype)
    dq, _, _ = cp.linear_attn_bwd(q, k, v, out, g, den, 1, state_final=st, z_final=zt)
    torch.cuda.synchronize()
    ref_out = orc.linattn(d["Q"], d["K"], d["V"], 1e-6, 1)
    ref_dq = orc.linattn_bwd(d["Q"], d["K"], d["V"], d["dO"], 1e-6, 1)[0]
    scale = {"out": np.abs(ref_out).max(-1), "dq": dq_summand_scale(d).max(-1)}
    L = shape[2]
    n = L // 10
    for name, got, ref in (("out", host(out), ref_out), ("dq", host(dq), ref_dq)):
        err = np.abs(got - ref)
        for band, sl in (("first 10%", slice(0, n)), ("last 10%", slice(L - n, L))):
            e, r = err[..., sl, :], np.abs(ref[..., sl, :])
            row = e.max(-1) / scale[name][..., sl]
            print(f"ROWERR {dtype} {name} {band}: band {e.max() / r.max():.2e} worst row {row.max():.2e}",
                  flush=True)
        check(got, ref, dtype, f"{name} {dtype}")


SEG_SHAPES = [(1, 2, 3001, 64, 64, "f32"), (1, 2, 3001, 64, 64, "bf16"), (2, 1, 2500, 32, 128, "bf16"),
              (1, 1, 4133, 128, 128, "bf16"), (1, 3, 700, 64, 32, "f32")]


@pytest.mark.parametrize("shape", SEG_SHAPES, ids=[str(s) for s in SEG_SHAPES])
def test_linattn_bwd_segmented(cp, orc, shape):
    """Few slices over long rows: the normalised backward runs over sequence
    segments (segment increments of S, z and of R, r, then per-segment
    sweeps), from initial states, with the final states and through the
    pre-pass; all gradients against the oracle."""
    N, H, L, E, M, dtype = shape
    d = inputs((N, H, L, E, M), dtype, seed=27 + L, fm=1, carry=True)
    q, k, v, out, st, zt, den, s0, z0 = forward(cp, d, dtype, 1)
    g = dev(d["dO"], dtype)
    ref = orc.linattn_bwd(d["Q"], d["K"], d["V"], d["dO"], 1e-6, 1, S0=d["S0"], z0=d["z0"])
    for label, kw in (("final states", dict(state_final=st, z_final=zt)), ("pre-pass", {})):
        ds0, dz0 = torch.empty_like(st), torch.empty_like(zt)
        got = cp.linear_attn_bwd(q, k, v, out, g, den, 1, state_in=s0, z_in=z0, dstate_in=ds0, dz_in=dz0, **kw)
        torch.cuda.synchronize()
        for t, r, name in zip(list(got) + [ds0, dz0], ref, ("dq", "dk", "dv", "dS0", "dz0")):
            check(host(t), r, dtype, f"{name} ({label}) {shape}")
