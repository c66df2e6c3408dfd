"""Pins of the fp64 oracle: checks against what the definition and the
mathematics fix, independent of the oracle's own code.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees.  They run against the real oracle (test_oracle_pins.py) and
against copies of it with planted mistakes (test_oracle_mutants.py), which
shows that a plausible slip anywhere in it fails at least one pin.

Definition pinned: the causal dot product of "Transformers are RNNs",
Algorithm 1, as named in the opening post of "Dot Product Computes Wrong
Values" (triton-lang/triton issue 217), inclusive of the current token as in
the loop excerpt later on that page; its normalised form with phi = elu + 1;
and the gradient of <dO, out>.
"""
from __future__ import annotations

import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TIGHT = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _rand(rng, *shape, positive=False):
    x = rng.standard_normal(shape).astype(np.float32)
    if positive:
        x = np.abs(x) + np.float32(0.25)
    return x


def _close(a, b, tol=TIGHT, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    den = max(float(np.max(np.abs(b))) if b.size else 0.0, 1e-300)
    err = float(np.max(np.abs(a - b))) / den if a.size else 0.0
    assert err <= tol, f"{what}: rel err {err:.3e} > {tol:.1e}"


SHAPES = [(1, 1, 1, 3, 2), (1, 2, 2, 2, 3), (2, 1, 7, 3, 5), (1, 1, 17, 4, 1), (1, 1, 33, 5, 6)]


# -- library routines: torch in float64 ---------------------------------------

def _t(x):
    return torch.from_numpy(np.asarray(x, np.float64))


def torch_fwd(Q, K, V):
    q, k, v = _t(Q), _t(K), _t(V)
    return torch.tril(q @ k.transpose(-1, -2)) @ v


def torch_phi(x):
    x = x if isinstance(x, torch.Tensor) else _t(x)
    return torch.nn.functional.elu(x, alpha=1.0) + 1.0


def torch_linattn(Q, K, V, eps, feature_map):
    q = torch_phi(Q) if feature_map else _t(Q)
    k = torch_phi(K) if feature_map else _t(K)
    a = torch.tril(q @ k.transpose(-1, -2))
    return (a @ _t(V)) / (a.sum(-1, keepdim=True) + eps)


def torch_grads(Q, K, V, dO):
    q, k, v = (_t(x).requires_grad_(True) for x in (Q, K, V))
    out = torch.tril(q @ k.transpose(-1, -2)) @ v
    (out * _t(dO)).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


# -- forward --------------------------------------------------------------------

def pin_fwd_library(o):
    """Recurrence and brute force equal tril(Q K^T) V computed by torch (fp64)."""
    for n, (N, H, L, E, M) in enumerate(SHAPES):
        r = _rng(100 + n)
        Q, K, V = _rand(r, N, H, L, E), _rand(r, N, H, L, E), _rand(r, N, H, L, M)
        ref = torch_fwd(Q, K, V).numpy()
        _close(o.fwd(Q, K, V), ref, what=f"fwd {N,H,L,E,M}")
        _close(o.fwd_brute(Q, K, V), ref, what=f"fwd_brute {N,H,L,E,M}")


def pin_fwd_recurrence_vs_brute(o):
    r = _rng(7)
    Q, K, V = _rand(r, 2, 2, 40, 8, positive=True), _rand(r, 2, 2, 40, 8, positive=True), _rand(r, 2, 2, 40, 3)
    _close(o.fwd(Q, K, V), o.fwd_brute(Q, K, V), what="O(L) vs O(L^2)")


def pin_fwd_l1_closed_form(o):
    """L = 1: out_0 = (q_0 . k_0) v_0, bitwise on exact inputs, tight on random."""
    r = _rng(11)
    Q = r.integers(-3, 4, size=(3, 1, 1, 5)).astype(np.float32)
    K = r.integers(-3, 4, size=(3, 1, 1, 5)).astype(np.float32)
    V = r.integers(-3, 4, size=(3, 1, 1, 4)).astype(np.float32)
    exp = np.einsum("nhle,nhle->nhl", Q.astype(np.float64), K.astype(np.float64))[..., None] * V
    for fn in (o.fwd, o.fwd_brute):
        got = fn(Q, K, V)
        assert np.array_equal(got, exp), "L=1 closed form (integers) not bitwise"
    Q, K, V = _rand(r, 2, 1, 1, 16), _rand(r, 2, 1, 1, 16), _rand(r, 2, 1, 1, 16)
    qk = np.sum(Q.astype(np.float64) * K.astype(np.float64), axis=-1, keepdims=True)
    bound = 4 * 16 * 2.0 ** -53 * np.sum(np.abs(Q.astype(np.float64) * K), -1, keepdims=True) * np.abs(V)
    for fn in (o.fwd, o.fwd_brute):
        assert np.all(np.abs(fn(Q, K, V) - qk * V) <= bound + 1e-300), "L=1 closed form bound"


def pin_fwd_prefix_sum(o):
    """E = 1, q = k = 1: the causal product reduces to the plain prefix sum of V."""
    r = _rng(12)
    for L, M in ((1, 3), (9, 4), (64, 2)):
        V = _rand(r, 2, 1, L, M)
        ones = np.ones((2, 1, L, 1), np.float32)
        _close(o.fwd(ones, ones, V), np.cumsum(V.astype(np.float64), axis=2), what="cumsum")
        _close(o.fwd_brute(ones, ones, V), np.cumsum(V.astype(np.float64), axis=2), what="cumsum brute")


def pin_fwd_zero(o):
    """Zero state or zero query gives zero output (the page's state*0 probe)."""
    r = _rng(13)
    Q, K, V = _rand(r, 1, 2, 9, 4), _rand(r, 1, 2, 9, 4), _rand(r, 1, 2, 9, 3)
    z4, z3 = np.zeros_like(Q), np.zeros_like(V)
    for fn in (o.fwd, o.fwd_brute):
        for args in ((Q, K, z3), (Q, z4, V), (z4, K, V)):
            assert not np.any(fn(*args)), "zero invariant"


def pin_fwd_worked_example(o):
    g = load_worked()
    _close(o.fwd(g["q"], g["k"], g["v"]), g["out"], 0.0, "worked out (recurrence)")
    _close(o.fwd_brute(g["q"], g["k"], g["v"]), g["out"], 0.0, "worked out (brute)")


def pin_fwd_integer_exact(o):
    """Small integers: exact equality with Python-integer brute force."""
    r = _rng(14)
    L, E, M = 6, 3, 2
    Q = r.integers(-2, 3, size=(1, 1, L, E))
    K = r.integers(-2, 3, size=(1, 1, L, E))
    V = r.integers(-2, 3, size=(1, 1, L, M))
    exp = np.zeros((1, 1, L, M))
    for i in range(L):
        for m in range(M):
            exp[0, 0, i, m] = sum(
                sum(int(Q[0, 0, i, e]) * int(K[0, 0, j, e]) for e in range(E)) * int(V[0, 0, j, m])
                for j in range(i + 1))
    f = np.float32
    assert np.array_equal(o.fwd(Q.astype(f), K.astype(f), V.astype(f)), exp)
    assert np.array_equal(o.fwd_brute(Q.astype(f), K.astype(f), V.astype(f)), exp)


def pin_fwd_causal_and_linear(o):
    """A prefix of the sequence gives the same rows; linear in each of Q, K, V."""
    r = _rng(15)
    Q, K, V = _rand(r, 1, 1, 20, 4), _rand(r, 1, 1, 20, 4), _rand(r, 1, 1, 20, 3)
    full = o.fwd(Q, K, V)
    _close(o.fwd(Q[:, :, :7], K[:, :, :7], V[:, :, :7]), full[:, :, :7], what="causality")
    # dyadic values so that 2 V - 3 V2 is exact in fp32
    V = (np.round(V * 64) / 64).astype(np.float32)
    V2 = (np.round(_rand(r, 1, 1, 20, 3) * 64) / 64).astype(np.float32)
    full = o.fwd(Q, K, V)
    lhs = o.fwd(Q, K, (2.0 * V - 3.0 * V2).astype(np.float32))
    _close(lhs, 2.0 * full - 3.0 * o.fwd(Q, K, V2), 1e-11, "linear in V")


def pin_state(o):
    """Final state = sum_j k_j v_j^T (einsum), and reading it with unit queries
    at the last token gives its rows."""
    r = _rng(16)
    K, V = _rand(r, 2, 1, 11, 3), _rand(r, 2, 1, 11, 4)
    S = o.state(K, V)
    _close(S, np.einsum("nhle,nhlm->nhem", K.astype(np.float64), V.astype(np.float64)), what="state")
    for e in range(3):
        Q = np.zeros_like(K)
        Q[..., e] = 1.0
        _close(o.fwd(Q, K, V)[:, :, -1, :], S[:, :, e, :], what="state row")


# -- normalised forward ---------------------------------------------------------

def pin_linattn_library(o):
    for n, (N, H, L, E, M) in enumerate(SHAPES):
        r = _rng(200 + n)
        Q, K, V = _rand(r, N, H, L, E), _rand(r, N, H, L, E), _rand(r, N, H, L, M)
        for fm in (1,):
            ref = torch_linattn(Q, K, V, 1e-6, fm).numpy()
            _close(o.linattn(Q, K, V, 1e-6, fm), ref, 1e-11, f"linattn fm={fm}")
            _close(o.linattn_brute(Q, K, V, 1e-6, fm), ref, 1e-11, f"linattn_brute fm={fm}")
        Qp, Kp = np.abs(Q) + 0.1, np.abs(K) + 0.1
        ref = torch_linattn(Qp, Kp, V, 1e-6, 0).numpy()
        _close(o.linattn(Qp, Kp, V, 1e-6, 0), ref, 1e-11, "linattn fm=0")
        _close(o.linattn_brute(Qp, Kp, V, 1e-6, 0), ref, 1e-11, "linattn_brute fm=0")


def pin_linattn_constant_v(o):
    """v_j = c for all j: out_i = c (q_i.z_i)/(q_i.z_i + eps).  Small inputs make
    eps matter."""
    r = _rng(21)
    L, E, M = 12, 3, 2
    Q = (np.abs(_rand(r, 1, 1, L, E)) * 1e-4).astype(np.float32)
    K = (np.abs(_rand(r, 1, 1, L, E)) * 1e-4).astype(np.float32)
    c = np.array([1.5, -2.0], np.float32)
    V = np.broadcast_to(c, (1, 1, L, M)).astype(np.float32)
    q, k = Q.astype(np.float64), K.astype(np.float64)
    z = np.cumsum(k, axis=2)
    a = np.sum(q * z, axis=-1, keepdims=True)
    exp = c.astype(np.float64) * a / (a + 1e-6)
    _close(o.linattn(Q, K, V, 1e-6, 0), exp, 1e-12, "constant V")
    _close(o.linattn_brute(Q, K, V, 1e-6, 0), exp, 1e-12, "constant V brute")


def pin_linattn_running_mean(o):
    """E = 1, q = k = 1 (identity map): out_i = cumsum(V)_i / (i + 1 + eps)."""
    r = _rng(22)
    L = 30
    V = _rand(r, 1, 1, L, 3)
    ones = np.ones((1, 1, L, 1), np.float32)
    eps = 1e-3
    exp = np.cumsum(V.astype(np.float64), axis=2) / (np.arange(1, L + 1, dtype=np.float64)[:, None] + eps)
    _close(o.linattn(ones, ones, V, eps, 0), exp, what="running mean")
    _close(o.linattn_brute(ones, ones, V, eps, 0), exp, what="running mean brute")


def pin_linattn_feature_map(o):
    """phi(0) = 1 and phi(x) = x + 1 for x > 0 make the elu+1 map on raw
    inputs in {0} U (0, inf) equal the identity map on the shifted values;
    exp(x) for x <= 0 follows from the torch elu comparison."""
    r = _rng(23)
    L, E, M = 10, 4, 3
    raw = np.where(r.random((1, 1, L, E)) < 0.3, 0.0, r.integers(1, 5, size=(1, 1, L, E))).astype(np.float32)
    rawk = np.where(r.random((1, 1, L, E)) < 0.3, 0.0, r.integers(1, 5, size=(1, 1, L, E))).astype(np.float32)
    V = _rand(r, 1, 1, L, M)
    _close(o.linattn(raw, rawk, V, 1e-6, 1), o.linattn(raw + 1, rawk + 1, V, 1e-6, 0), 1e-13, "phi shift")
    neg = -np.abs(_rand(r, 1, 1, L, E)) - 0.5
    negk = -np.abs(_rand(r, 1, 1, L, E)) - 0.5
    _close(o.linattn(neg, negk, V, 1e-6, 1), torch_linattn(neg, negk, V, 1e-6, 1).numpy(), 1e-11,
           "phi negative branch")


def pin_linattn_worked_example(o):
    g = load_worked()
    exp = g["out"] / g["den"][:, None]
    _close(o.linattn(g["q"], g["k"], g["v"], 0.0, 0), exp, 1e-15, "worked normalised")
    _close(o.linattn_brute(g["q"], g["k"], g["v"], 0.0, 0), exp, 1e-15, "worked normalised brute")


# -- backward ---------------------------------------------------------------------

def pin_bwd_autograd(o):
    for n, (N, H, L, E, M) in enumerate(SHAPES):
        r = _rng(300 + n)
        Q, K, V, dO = (_rand(r, N, H, L, E), _rand(r, N, H, L, E), _rand(r, N, H, L, M),
                       _rand(r, N, H, L, M))
        ref = torch_grads(Q, K, V, dO)
        for fn in (o.bwd, o.bwd_brute):
            got = fn(Q, K, V, dO)
            for name, g, e in zip(("dQ", "dK", "dV"), got, ref):
                _close(g, e, what=f"{fn.__name__} {name} {N,H,L,E,M}")


def pin_bwd_directional(o):
    """<dO, out> is linear in each argument, so f(X + D) - f(X) = <dX, D> exactly
    (no step-size error), checked with the forward oracle."""
    r = _rng(31)
    Q, K, V, dO = (_rand(r, 1, 2, 13, 4), _rand(r, 1, 2, 13, 4), _rand(r, 1, 2, 13, 3),
                   _rand(r, 1, 2, 13, 3))
    dQ, dK, dV = o.bwd(Q, K, V, dO)
    f = lambda q, k, v: float(np.sum(o.fwd(q, k, v) * dO))
    base = f(Q, K, V)
    for i, (d, D) in enumerate(((dQ, _rand(r, *Q.shape)), (dK, _rand(r, *K.shape)), (dV, _rand(r, *V.shape)))):
        args = [Q, K, V]
        args[i] = (args[i].astype(np.float64) + D).astype(np.float32)
        Dx = args[i].astype(np.float64) - [Q, K, V][i]
        delta = f(*args) - base
        pred = float(np.sum(d * Dx))
        assert abs(delta - pred) <= 1e-9 * max(1.0, abs(pred)), f"directional derivative arg {i}"


def pin_bwd_homogeneity(o):
    """<dO,out> = <Q,dQ> = <K,dK> = <V,dV> (f is homogeneous of degree 1 in each)."""
    r = _rng(32)
    Q, K, V, dO = (_rand(r, 2, 1, 21, 5), _rand(r, 2, 1, 21, 5), _rand(r, 2, 1, 21, 2),
                   _rand(r, 2, 1, 21, 2))
    f = float(np.sum(o.fwd(Q, K, V) * dO))
    for fn in (o.bwd, o.bwd_brute):
        dQ, dK, dV = fn(Q, K, V, dO)
        for x, g in ((Q, dQ), (K, dK), (V, dV)):
            assert abs(float(np.sum(x * g)) - f) <= 1e-11 * max(1.0, abs(f)), "homogeneity"


def pin_bwd_l1_closed_form(o):
    """L = 1: dq = (dO.v) k, dk = (dO.v) q, dv = (q.k) dO, bitwise on integers."""
    r = _rng(33)
    Q, K = (r.integers(-3, 4, size=(2, 1, 1, 4)).astype(np.float32) for _ in range(2))
    V, dO = (r.integers(-3, 4, size=(2, 1, 1, 3)).astype(np.float32) for _ in range(2))
    gv = np.sum(dO.astype(np.float64) * V, -1, keepdims=True)
    qk = np.sum(Q.astype(np.float64) * K, -1, keepdims=True)
    for fn in (o.bwd, o.bwd_brute):
        dQ, dK, dV = fn(Q, K, V, dO)
        assert np.array_equal(dQ, gv * K) and np.array_equal(dK, gv * Q) and np.array_equal(dV, qk * dO)


def pin_bwd_worked_example(o):
    g = load_worked()
    for fn in (o.bwd, o.bwd_brute):
        dQ, dK, dV = fn(g["q"], g["k"], g["v"], g["dO"])
        _close(dQ, g["dq"], 0.0, "worked dq")
        _close(dK, g["dk"], 0.0, "worked dk")
        _close(dV, g["dv"], 0.0, "worked dv")


def pin_bwd_recurrence_vs_brute(o):
    r = _rng(34)
    Q, K, V, dO = (_rand(r, 1, 3, 37, 6, positive=True), _rand(r, 1, 3, 37, 6, positive=True),
                   _rand(r, 1, 3, 37, 5), _rand(r, 1, 3, 37, 5))
    for a, b, name in zip(o.bwd(Q, K, V, dO), o.bwd_brute(Q, K, V, dO), "QKV"):
        _close(a, b, what=f"d{name} O(L) vs O(L^2)")


# -- carried state: S0 (and z0) as the state before the first row ----------------

def _carry_inputs(seed, shape=(2, 1, 11, 3, 4)):
    r = _rng(seed)
    N, H, L, E, M = shape
    Q, K = _rand(r, N, H, L, E, positive=True), _rand(r, N, H, L, E, positive=True)
    V, dO = _rand(r, N, H, L, M), _rand(r, N, H, L, M)
    S0, z0 = _rand(r, N, H, E, M), _rand(r, N, H, E, positive=True)
    return Q, K, V, dO, S0, z0


def pin_carry_fwd_library(o):
    """out = Q S0 + tril(Q K^T) V and S_{L-1} = S0 + K^T V (torch, float64)."""
    Q, K, V, _, S0, _ = _carry_inputs(40)
    q, k, v, s0 = _t(Q), _t(K), _t(V), _t(S0)
    out, Sf = o.fwd(Q, K, V, S0=S0, return_state=True)
    _close(out, (q @ s0 + torch.tril(q @ k.transpose(-1, -2)) @ v).numpy(), what="fwd with S0")
    _close(Sf, (s0 + k.transpose(-1, -2) @ v).numpy(), what="final state with S0")
    _close(o.fwd_brute(Q, K, V, S0=S0), out, what="brute with S0")


def pin_carry_fwd_composition(o):
    """Running the rows in two pieces, the second from the first's final
    state, gives the one-piece result (outputs and final state)."""
    Q, K, V, _, S0, _ = _carry_inputs(41, (1, 2, 19, 4, 3))
    full, Sf = o.fwd(Q, K, V, S0=S0, return_state=True)
    for cut in (1, 7, 18):
        a, Sa = o.fwd(Q[..., :cut, :], K[..., :cut, :], V[..., :cut, :], S0=S0, return_state=True)
        b, Sb = o.fwd(Q[..., cut:, :], K[..., cut:, :], V[..., cut:, :], S0=Sa.astype(np.float32),
                      return_state=True)
        # the carried state passes through float32 (the boundary's type)
        _close(np.concatenate([a, b], axis=-2), full, tol=1e-6, what=f"pieces at {cut}")
        _close(Sb, Sf, tol=1e-6, what=f"final state, pieces at {cut}")


def pin_carry_linattn_library(o):
    """Normalised form from (S0, z0): numerator c_i^T S0 + sum a_ij v_j,
    denominator c_i.z0 + sum a_ij + eps, final S and z (torch, float64)."""
    Q, K, V, _, S0, z0 = _carry_inputs(42)
    for fm in (0, 1):
        c = torch_phi(_t(Q)) if fm else _t(Q)
        f = torch_phi(_t(K)) if fm else _t(K)
        a = torch.tril(c @ f.transpose(-1, -2))
        num = c @ _t(S0) + a @ _t(V)
        den = (c * _t(z0)[..., None, :]).sum(-1) + a.sum(-1) + 1e-6
        out, Sf, zf = o.linattn(Q, K, V, 1e-6, fm, S0=S0, z0=z0, return_state=True)
        _close(out, (num / den[..., None]).numpy(), what=f"linattn with S0, z0 (fm {fm})")
        _close(Sf, (_t(S0) + f.transpose(-1, -2) @ _t(V)).numpy(), what="final S")
        _close(zf, (_t(z0) + f.sum(-2)).numpy(), what="final z")
        _close(o.linattn_brute(Q, K, V, 1e-6, fm, S0=S0, z0=z0), out, what="brute with S0, z0")


def pin_carry_linattn_composition(o):
    Q, K, V, _, S0, z0 = _carry_inputs(43, (1, 1, 23, 5, 2))
    full = o.linattn(Q, K, V, 1e-6, 1, S0=S0, z0=z0)
    a, Sa, za = o.linattn(Q[..., :9, :], K[..., :9, :], V[..., :9, :], 1e-6, 1, S0=S0, z0=z0, return_state=True)
    b = o.linattn(Q[..., 9:, :], K[..., 9:, :], V[..., 9:, :], 1e-6, 1, S0=Sa.astype(np.float32),
                  z0=za.astype(np.float32))
    _close(np.concatenate([a, b], axis=-2), full, tol=1e-6, what="linattn pieces")


def pin_carry_bwd_autograd(o):
    """Gradients of sum(out * dO) with out = Q S0 + tril(Q K^T) V by torch
    autograd in float64, among them the initial state's sum_i q_i dO_i^T."""
    Q, K, V, dO, S0, _ = _carry_inputs(44)
    ts = [_t(x).requires_grad_(True) for x in (Q, K, V, S0)]
    q, k, v, s0 = ts
    f = ((q @ s0 + torch.tril(q @ k.transpose(-1, -2)) @ v) * _t(dO)).sum()
    f.backward()
    want = [t.grad.numpy() for t in ts]
    for got in (o.bwd(Q, K, V, dO, S0=S0, with_dS0=True), o.bwd_brute(Q, K, V, dO, S0=S0, with_dS0=True)):
        for a, b, name in zip(got, want, ("dQ", "dK", "dV", "dS0")):
            _close(a, b, what=f"{name} with S0")


# -- backward of the normalised form ------------------------------------------------

def pin_linattn_bwd_autograd(o):
    """Gradients of sum(out * dO) for the normalised form, through phi and
    from (S0, z0), by torch autograd in float64 on the brute-force formula;
    raw Q, K with both signs so that both branches of phi are used."""
    for fm, seed in ((1, 45), (0, 46)):
        r = _rng(seed)
        N, H, L, E, M = 2, 1, 13, 3, 4
        Q, K = _rand(r, N, H, L, E, positive=not fm), _rand(r, N, H, L, E, positive=not fm)
        V, dO = _rand(r, N, H, L, M), _rand(r, N, H, L, M)
        S0, z0 = _rand(r, N, H, E, M), _rand(r, N, H, E, positive=True)
        ts = [_t(x).requires_grad_(True) for x in (Q, K, V, S0, z0)]
        q, k, v, s0, z0t = ts
        c = torch_phi(q) if fm else q
        f = torch_phi(k) if fm else k
        a = torch.tril(c @ f.transpose(-1, -2))
        num = c @ s0 + a @ v
        den = (c * z0t[..., None, :]).sum(-1) + a.sum(-1) + 1e-6
        ((num / den[..., None]) * _t(dO)).sum().backward()
        got = o.linattn_bwd(Q, K, V, dO, 1e-6, fm, S0=S0, z0=z0)
        for g_, t, name in zip(got, ts, ("dQ", "dK", "dV", "dS0", "dz0")):
            _close(g_, t.grad.numpy(), what=f"normalised backward {name} (fm {fm})")


def pin_linattn_bwd_reduces_to_causal_product(o):
    """The denominator does not depend on V, so the value gradient of the
    normalised form equals the causal product's value gradient for the
    upstream gradient dO_i / d_i (identity feature map, eps = 0, z0 = 0:
    d_i is the causal row sum of q_i . k_j)."""
    r = _rng(47)
    N, H, L, E, M = 1, 2, 9, 4, 3
    Q, K = _rand(r, N, H, L, E, positive=True), _rand(r, N, H, L, E, positive=True)
    V, dO = _rand(r, N, H, L, M), _rand(r, N, H, L, M)
    den = (torch.tril(_t(Q) @ _t(K).transpose(-1, -2))).sum(-1).numpy()
    scaled = (dO / den[..., None]).astype(np.float32)
    _, _, dV = o.bwd(Q, K, V, scaled)
    got = o.linattn_bwd(Q, K, V, dO, 0.0, 0)[2]
    # dO / d is rounded to float32 on the way into the causal-product oracle
    _close(got, dV, tol=1e-6, what="dV of the normalised form vs causal product of dO / d")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


def load_worked():
    """The hand-worked L=3, E=2, M=2 example in golden/worked_l3_e2_m2.txt."""
    rows = {}
    with open(os.path.join(GOLDEN, "worked_l3_e2_m2.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, *vals = line.split()
            rows[name] = np.array([float(x) for x in vals])
    g = {}
    for name in ("q", "k", "v", "dO"):
        g[name] = rows[name].reshape(1, 1, 3, 2).astype(np.float32)
    for name in ("out", "dq", "dk", "dv"):
        g[name] = rows[name].reshape(1, 1, 3, 2)
    g["den"] = rows["den"]
    return g
