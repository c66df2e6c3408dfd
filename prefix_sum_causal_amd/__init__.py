"""MI355X (gfx950) causal dot product of linear attention.

Thin Python binding of the C ABI in ``include/causalprod.h`` (library
``libcausalprod.so`` built next to this file by ``build.py``).  Every step of
the computation runs in the HIP kernels behind that ABI; this module only
checks tensors, allocates outputs (and, over few slices, the calls'
workspaces) through PyTorch and passes raw device pointers and the current
HIP stream.  There is no fallback: if the library is missing the import
fails.

Functions with the ABI's names (optional tensors and outputs are keyword-only;
each of the four operations also takes an optional ``workspace`` tensor):
    causal_product_fwd(q, k, v, *, out=None, state_in=None, state_out=None)
    causal_product_fwd_noalloc(q, k, v, *, out, state_in=None, state_out=None)
    causal_product_bwd(q, k, v, dout, *, state_final=None, state_in=None,
                       dq=None, dk=None, dv=None, dstate_in=None)
    linear_attn_fwd(q, k, v, eps=1e-6, feature_map=1, *, out=None, state_in=None,
                    z_in=None, state_out=None, z_out=None, den_out=None)
    linear_attn_bwd(q, k, v, out, dout, den, feature_map=1, *, state_in=None,
                    z_in=None, state_final=None, z_final=None, dq=None,
                    dk=None, dv=None, dstate_in=None, dz_in=None)
    workspace_size(op, N, H, L, E, M, dtype)   (cp_workspace_size)
and autograd wrappers ``causal_product(q, k, v, state0=None)`` and
``linear_attention(q, k, v, eps=1e-6, feature_map="elu+1")``.

Tensors are [N, H, L, E] (q, k) and [N, H, L, M] (v), contiguous, on the GPU,
all float32, all bfloat16 or all float16 (float16: not for the normalised
backward), with head sizes E, M <= 128 whose rows are whole 16-byte pieces
(multiples of 8 for the 16-bit types, of 4 for float32).
"""
from __future__ import annotations

import ctypes
import functools
import os
import threading

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# CAUSALPROD_LIB selects another build of the same library (e.g. one built
# with other tuning parameters by build.build(out=..., defines=...)).
LIB_PATH = os.environ.get("CAUSALPROD_LIB") or os.path.join(HERE, "libcausalprod.so")

CP_F32, CP_BF16, CP_F16 = 0, 1, 2
CP_OP_CAUSAL_FWD, CP_OP_CAUSAL_BWD, CP_OP_LINATTN_FWD, CP_OP_LINATTN_BWD = 0, 1, 2, 3
STATUS = {0: "CP_OK", 1: "CP_ERR_NULL", 2: "CP_ERR_DIM", 3: "CP_ERR_UNSUPPORTED", 4: "CP_ERR_ALIGN",
          5: "CP_ERR_ALIAS", 6: "CP_ERR_HIP", 7: "CP_ERR_SCRATCH"}
# Kernel tile sizes: a head of E (or M) features runs on the smallest tile >= E,
# its padding columns read as zero and never stored.
TILE_SIZES = (16, 32, 64, 128)

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m prefix_sum_causal_amd.build`")
lib = ctypes.CDLL(LIB_PATH)

_vp, _i64, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
lib.causal_product_fwd.argtypes = [_vp] * 6 + [_i64] * 5 + [_int, _vp, _i64, _vp]
lib.causal_product_fwd.restype = _int
lib.causal_product_fwd_noalloc.argtypes = [_vp] * 6 + [_i64] * 5 + [_int, _vp]
lib.causal_product_fwd_noalloc.restype = _int
lib.causal_product_bwd.argtypes = [_vp] * 10 + [_i64] * 5 + [_int, _vp, _i64, _vp]
lib.causal_product_bwd.restype = _int
lib.linear_attn_fwd.argtypes = [_vp] * 9 + [_i64] * 5 + [ctypes.c_float, _int, _int, _vp, _i64, _vp]
lib.linear_attn_bwd.argtypes = [_vp] * 15 + [_i64] * 5 + [_int, _int, _vp, _i64, _vp]
lib.linear_attn_bwd.restype = _int
lib.linear_attn_fwd.restype = _int
lib.cp_workspace_size.argtypes = [_int] + [_i64] * 5 + [_int, ctypes.POINTER(_i64)]
lib.cp_workspace_size.restype = _int
lib.cp_status_string.argtypes = [_int]
lib.cp_status_string.restype = ctypes.c_char_p
lib.cp_abi_version.argtypes = []
lib.cp_abi_version.restype = _int
lib.cp_timing_begin.argtypes = [_int]
lib.cp_timing_begin.restype = _int
lib.cp_timing_end.argtypes = [ctypes.POINTER(ctypes.c_float), _int, ctypes.POINTER(_int)]
lib.cp_timing_end.restype = _int


class CausalProductError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib.cp_status_string(status).decode()
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {msg}")
        self.status = status


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise CausalProductError(fn, status)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return CP_F32
    if t.dtype == torch.bfloat16:
        return CP_BF16
    if t.dtype == torch.float16:
        return CP_F16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32, bfloat16 or float16")


def _dims(q: torch.Tensor, v: torch.Tensor):
    if q.dim() != 4 or v.dim() != 4 or q.shape[:3] != v.shape[:3]:
        raise ValueError(f"expected q [N,H,L,E] and v [N,H,L,M], got {tuple(q.shape)} and {tuple(v.shape)}")
    N, H, L, E = q.shape
    return N, H, L, E, v.shape[3]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_tensors(*ts):
    dev, dt = ts[0].device, ts[0].dtype
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if t.device != dev or t.dtype != dt:
            raise ValueError("all tensors must share one device and one dtype")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def timing_begin(capacity: int) -> None:
    """Record the start and end of each of the next ``capacity`` kernel
    launches made by this thread (their dispatch timestamps)."""
    _check("cp_timing_begin", lib.cp_timing_begin(int(capacity)))
    _timing.capacity = int(capacity)


def timing_end() -> list:
    """Wait for the launches recorded since this thread's timing_begin and
    return their durations in milliseconds, in launch order."""
    cap = max(1, getattr(_timing, "capacity", 0))
    buf = (ctypes.c_float * cap)()
    n = _int(0)
    _check("cp_timing_end", lib.cp_timing_end(buf, cap, ctypes.byref(n)))
    _timing.capacity = 0
    return [buf[i] for i in range(n.value)]


# the capacity of this thread's timing (the library keeps its timing state per thread)
_timing = threading.local()


@functools.lru_cache(maxsize=256)
def workspace_size(op: int, N: int, H: int, L: int, E: int, M: int, dtype: int) -> int:
    """Bytes of workspace operation ``op`` (CP_OP_*) needs for these sizes
    and dtype code (0: none); host arithmetic in the library."""
    n = _i64(0)
    _check("cp_workspace_size", lib.cp_workspace_size(op, N, H, L, E, M, dtype, ctypes.byref(n)))
    return n.value


_ws_bytes = {}  # (op, sizes, dtype) -> workspace_size, without the cache wrapper's cost per call


def _workspace(op, q, N, H, L, E, M, workspace):
    """(pointer, bytes, tensor) of the workspace of a call: the caller's
    tensor, or one from PyTorch's allocator on the current stream when the
    call needs one (it stays valid for the work enqueued on that stream)."""
    if workspace is not None:
        if not workspace.is_cuda or not workspace.is_contiguous() or workspace.device != q.device:
            raise ValueError("workspace must be a contiguous tensor on q's device")
        return ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(), workspace
    key = (op, N, H, L, E, M, q.dtype)
    n = _ws_bytes.get(key)
    if n is None:
        n = _ws_bytes[key] = workspace_size(op, N, H, L, E, M, _dtype_code(q))
    if n == 0:
        return None, 0, None
    t = torch.empty(n, dtype=torch.uint8, device=q.device)
    return ctypes.c_void_p(t.data_ptr()), n, t


def _check_state(name, t, shape, device):
    """An optional fp32 state tensor (None passes)."""
    if t is not None and (t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != shape
                          or t.device != device):
        raise ValueError(f"{name} must be a contiguous float32 {list(shape)} tensor on q's device")


def causal_product_fwd(q, k, v, *, out=None, state_in=None, state_out=None, workspace=None):
    """out_i = q_i^T S_i with S_i = S0 + sum_{j<=i} k_j v_j^T.  ``state_in``
    (fp32 [N,H,E,M], optional, None = zero) is S0; ``state_out`` (optional)
    receives the final state S_{L-1}.  ``workspace`` (optional): a device
    tensor of at least workspace_size(CP_OP_CAUSAL_FWD, ...) bytes; by default
    one comes from PyTorch's allocator when the call needs it."""
    N, H, L, E, M = _dims(q, v)
    if k.shape != q.shape:
        raise ValueError("k must have q's shape")
    if out is None:
        out = torch.empty_like(v)
    _check_tensors(q, k, v, out)
    _check_state("state_in", state_in, (N, H, E, M), q.device)
    _check_state("state_out", state_out, (N, H, E, M), q.device)
    wp, wn, _wt = _workspace(CP_OP_CAUSAL_FWD, q, N, H, L, E, M, workspace)
    _check("causal_product_fwd", lib.causal_product_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(state_in), _ptr(state_out), N, H, L, E, M, _dtype_code(q),
        wp, wn, _stream(q.device)))
    return out


def causal_product_fwd_noalloc(q, k, v, *, out, state_in=None, state_out=None):
    """causal_product_fwd for callers that cannot allocate: the caller passes
    ``out`` (and the optional states); the library allocates nothing and keeps
    the scratch of a forward over few slices in a static 16 MiB device buffer
    shared by every call on the GPU (calls that may overlap on one GPU must
    be serialised)."""
    N, H, L, E, M = _dims(q, v)
    if k.shape != q.shape or out.shape != v.shape:
        raise ValueError("k must have q's shape and out v's shape")
    _check_tensors(q, k, v, out)
    _check_state("state_in", state_in, (N, H, E, M), q.device)
    _check_state("state_out", state_out, (N, H, E, M), q.device)
    _check("causal_product_fwd_noalloc", lib.causal_product_fwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(state_in), _ptr(state_out), N, H, L, E, M, _dtype_code(q),
        _stream(q.device)))
    return out


def causal_product_bwd(q, k, v, dout, *, state_final=None, state_in=None, dq=None, dk=None, dv=None,
                       dstate_in=None, workspace=None):
    """Gradients (dq, dk, dv) of sum(out * dout) for out = causal_product_fwd(q, k, v, state_in=S0).
    ``state_final``: optional final state from causal_product_fwd's state_out;
    ``state_in``: the S0 the forward started from (read only without
    state_final); ``dstate_in`` (optional fp32 [N,H,E,M]) receives the
    gradient of S0, sum_i q_i dout_i^T.  ``workspace``: as for
    causal_product_fwd (CP_OP_CAUSAL_BWD)."""
    N, H, L, E, M = _dims(q, v)
    if k.shape != q.shape or dout.shape != v.shape:
        raise ValueError("k must have q's shape and dout v's shape")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_tensors(q, k, v, dout, dq, dk, dv)
    for name, t in (("state_final", state_final), ("state_in", state_in), ("dstate_in", dstate_in)):
        _check_state(name, t, (N, H, E, M), q.device)
    wp, wn, _wt = _workspace(CP_OP_CAUSAL_BWD, q, N, H, L, E, M, workspace)
    _check("causal_product_bwd", lib.causal_product_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(state_in), _ptr(state_final), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(dstate_in), N, H, L, E, M, _dtype_code(q), wp, wn, _stream(q.device)))
    return dq, dk, dv


def linear_attn_fwd(q, k, v, eps: float = 1e-6, feature_map: int = 1, *, out=None, state_in=None, z_in=None,
                    state_out=None, z_out=None, den_out=None, workspace=None):
    """out_i = phi(q_i)^T S_i / (phi(q_i) . z_i + eps) with phi = elu + 1
    (feature_map=1) or the identity (feature_map=0) applied to the raw q, k.
    Optional fp32 states: state_in [N,H,E,M] and z_in [N,H,E] before the
    first row (None = zero); state_out, z_out receive the final S and z;
    den_out [N,H,L] receives the denominators (for linear_attn_bwd).
    ``workspace``: as for causal_product_fwd (CP_OP_LINATTN_FWD)."""
    N, H, L, E, M = _dims(q, v)
    if k.shape != q.shape:
        raise ValueError("k must have q's shape")
    if out is None:
        out = torch.empty_like(v)
    _check_tensors(q, k, v, out)
    for name, t, shape in (("state_in", state_in, (N, H, E, M)), ("z_in", z_in, (N, H, E)),
                           ("state_out", state_out, (N, H, E, M)), ("z_out", z_out, (N, H, E)),
                           ("den_out", den_out, (N, H, L))):
        _check_state(name, t, shape, q.device)
    wp, wn, _wt = _workspace(CP_OP_LINATTN_FWD, q, N, H, L, E, M, workspace)
    _check("linear_attn_fwd", lib.linear_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(state_in), _ptr(z_in), _ptr(state_out), _ptr(z_out),
        _ptr(den_out), N, H, L, E, M, float(eps), int(feature_map), _dtype_code(q), wp, wn, _stream(q.device)))
    return out


def linear_attn_bwd(q, k, v, out, dout, den, feature_map: int = 1, *, state_in=None, z_in=None, state_final=None,
                    z_final=None, dq=None, dk=None, dv=None, dstate_in=None, dz_in=None, workspace=None):
    """Gradients (dq, dk, dv) of sum(out * dout) for out = linear_attn_fwd(q, k, v, ...),
    with respect to the raw q, k (through phi), v; ``den`` is the forward's
    den_out.  state_in / z_in: the initial states the forward started from
    (pass them whenever it had them); state_final, z_final: the forward's
    final S and z (its state_out and z_out), an optional shortcut taken as a
    pair (read for bf16 only); dstate_in [N,H,E,M] and dz_in [N,H,E] receive
    the gradients of the initial states.  ``workspace``: as for
    causal_product_fwd (CP_OP_LINATTN_BWD)."""
    N, H, L, E, M = _dims(q, v)
    if k.shape != q.shape or dout.shape != v.shape or out.shape != v.shape:
        raise ValueError("k must have q's shape, out and dout v's shape")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_tensors(q, k, v, out, dout, dq, dk, dv)
    for name, t, shape in (("den", den, (N, H, L)), ("state_in", state_in, (N, H, E, M)), ("z_in", z_in, (N, H, E)),
                           ("state_final", state_final, (N, H, E, M)), ("z_final", z_final, (N, H, E)),
                           ("dstate_in", dstate_in, (N, H, E, M)), ("dz_in", dz_in, (N, H, E))):
        _check_state(name, t, shape, q.device)
    if den is None:
        raise ValueError("den (the forward's den_out) is required")
    wp, wn, _wt = _workspace(CP_OP_LINATTN_BWD, q, N, H, L, E, M, workspace)
    _check("linear_attn_bwd", lib.linear_attn_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(den), _ptr(state_in), _ptr(z_in), _ptr(state_final),
        _ptr(z_final), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dstate_in), _ptr(dz_in), N, H, L, E, M, int(feature_map),
        _dtype_code(q), wp, wn, _stream(q.device)))
    return dq, dk, dv


class CausalProduct(torch.autograd.Function):
    """Autograd wrapper: the forward keeps the final state so that the
    backward runs its query gradient in the same reverse sweep as the others.
    An initial state (fp32 [N,H,E,M]) may be given and receives a gradient."""

    @staticmethod
    def forward(ctx, q, k, v, state0):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        s0 = state0.contiguous() if state0 is not None else None
        N, H, L, E, M = _dims(q, v)
        state = torch.empty((N, H, E, M), device=q.device, dtype=torch.float32)
        out = causal_product_fwd(q, k, v, state_in=s0, state_out=state)
        ctx.save_for_backward(q, k, v, state)
        ctx.has_state0 = s0 is not None
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, state = ctx.saved_tensors
        ds0 = torch.empty_like(state) if ctx.has_state0 and ctx.needs_input_grad[3] else None
        dq, dk, dv = causal_product_bwd(q, k, v, dout.contiguous(), state_final=state, dstate_in=ds0)
        return dq, dk, dv, ds0


def causal_product(q, k, v, state0=None):
    """Differentiable causal dot product (q, k already feature-mapped),
    optionally from an initial state state0 (fp32 [N,H,E,M])."""
    return CausalProduct.apply(q, k, v, state0)


class LinearAttention(torch.autograd.Function):
    """Autograd wrapper of the normalised form: the forward keeps its output,
    denominators and final states for the backward's single reverse sweep."""

    @staticmethod
    def forward(ctx, q, k, v, eps, feature_map):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        N, H, L, E, M = _dims(q, v)
        st = torch.empty((N, H, E, M), device=q.device, dtype=torch.float32)
        zf = torch.empty((N, H, E), device=q.device, dtype=torch.float32)
        den = torch.empty((N, H, L), device=q.device, dtype=torch.float32)
        out = linear_attn_fwd(q, k, v, eps, feature_map, state_out=st, z_out=zf, den_out=den)
        ctx.save_for_backward(q, k, v, out, den, st, zf)
        ctx.feature_map = feature_map
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, den, st, zf = ctx.saved_tensors
        dq, dk, dv = linear_attn_bwd(q, k, v, out, dout.contiguous(), den, ctx.feature_map, state_final=st,
                                     z_final=zf)
        return dq, dk, dv, None, None


def linear_attention(q, k, v, eps: float = 1e-6, feature_map: str = "elu+1"):
    """Normalised causal linear attention; feature_map "elu+1" or "identity"."""
    fm = {"elu+1": 1, "identity": 0}[feature_map]
    return LinearAttention.apply(q, k, v, eps, fm)


__all__ = ["causal_product_fwd", "causal_product_fwd_noalloc", "causal_product_bwd", "linear_attn_fwd", "linear_attn_bwd", "workspace_size", "causal_product", "linear_attention",
           "CausalProductError", "lib", "LIB_PATH", "timing_begin", "timing_end"]
