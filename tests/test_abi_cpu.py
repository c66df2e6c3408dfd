"""The C ABI on the CPU: the library loads, exports every function that
include/causalprod.h declares, and rejects invalid arguments with the
documented status before touching a device (fake, never dereferenced
addresses; every case here fails validation)."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "causalprod.h")
LIB = os.path.join(ROOT, "prefix_sum_causal_amd", "libcausalprod.so")

OK, NULL, DIM, UNSUP, ALIGN, ALIAS, HIP, SCRATCH = range(8)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libcausalprod.so not built")
    lib = ctypes.CDLL(LIB)
    vp, i64, i = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.causal_product_fwd.argtypes = [vp] * 6 + [i64] * 5 + [i, vp, i64, vp]
    lib.causal_product_fwd_noalloc.argtypes = [vp] * 6 + [i64] * 5 + [i, vp]
    lib.causal_product_bwd.argtypes = [vp] * 10 + [i64] * 5 + [i, vp, i64, vp]
    lib.linear_attn_fwd.argtypes = [vp] * 9 + [i64] * 5 + [ctypes.c_float, i, i, vp, i64, vp]
    lib.linear_attn_bwd.argtypes = [vp] * 15 + [i64] * 5 + [i, i, vp, i64, vp]
    lib.cp_workspace_size.argtypes = [i] + [i64] * 5 + [i, ctypes.POINTER(i64)]
    lib.cp_status_string.restype = ctypes.c_char_p
    return lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(
        ["causal_product_fwd", "causal_product_fwd_noalloc", "causal_product_bwd", "linear_attn_fwd",
         "linear_attn_bwd", "cp_workspace_size", "cp_status_string", "cp_abi_version", "cp_timing_begin",
         "cp_timing_end"])


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version(lib):
    seen = set()
    for s in range(8):
        msg = lib.cp_status_string(s).decode()
        assert msg and msg not in seen
        seen.add(msg)
    assert lib.cp_status_string(99).decode() == "unknown status"
    assert lib.cp_abi_version() == (6 << 16) | 0


def test_timing_rejects_bad_arguments_before_any_device_call(lib):
    lib.cp_timing_begin.argtypes = [ctypes.c_int]
    lib.cp_timing_end.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    assert lib.cp_timing_begin(0) == DIM
    assert lib.cp_timing_begin(-3) == DIM
    assert lib.cp_timing_begin(65537) == DIM
    ms = (ctypes.c_float * 4)()
    n = ctypes.c_int(7)
    assert lib.cp_timing_end(None, 4, ctypes.byref(n)) == NULL
    assert lib.cp_timing_end(ms, 4, None) == NULL
    assert lib.cp_timing_end(ms, 4, ctypes.byref(n)) == NULL  # nothing begun


# fake, 16-byte aligned, disjoint addresses (never dereferenced)
A = [0x10_0000_0000 + n * 0x1_0000_0000 for n in range(12)]
SHAPE = (2, 3, 100, 64, 32)


def fwd(lib, q=A[0], k=A[1], v=A[2], o=A[3], s0=None, st=None, shape=SHAPE, dtype=1, ws=None, wsb=0):
    return lib.causal_product_fwd(q, k, v, o, s0, st, *shape, dtype, ws, wsb, None)


def bwd(lib, q=A[0], k=A[1], v=A[2], g=A[3], s0=None, st=None, dq=A[4], dk=A[5], dv=A[6], ds0=None,
        shape=SHAPE, dtype=1, ws=None, wsb=0):
    return lib.causal_product_bwd(q, k, v, g, s0, st, dq, dk, dv, ds0, *shape, dtype, ws, wsb, None)


def lin(lib, q=A[0], k=A[1], v=A[2], o=A[3], s0=None, z0=None, st=None, zt=None, den=None, shape=SHAPE, eps=1e-6,
        fm=1, dtype=1, ws=None, wsb=0):
    return lib.linear_attn_fwd(q, k, v, o, s0, z0, st, zt, den, *shape, eps, fm, dtype, ws, wsb, None)


def linb(lib, q=A[0], k=A[1], v=A[2], o=A[3], g=A[4], den=A[5], s0=None, z0=None, st=None, zt=None, dq=A[6],
         dk=A[7], dv=A[8], ds0=None, dz0=None, shape=SHAPE, fm=1, dtype=1, ws=None, wsb=0):
    return lib.linear_attn_bwd(q, k, v, o, g, den, s0, z0, st, zt, dq, dk, dv, ds0, dz0, *shape, fm, dtype, ws, wsb,
                               None)


@pytest.mark.parametrize("which", range(4))
def test_null_pointers(lib, which):
    args = dict(q=A[0], k=A[1], v=A[2], o=A[3])
    args[list(args)[which]] = None
    assert fwd(lib, **args) == NULL
    assert lin(lib, **args) == NULL


def test_null_backward_pointers(lib):
    for name in ("q", "k", "v", "g", "dq", "dk", "dv"):
        assert bwd(lib, **{name: None}) == NULL, name


@pytest.mark.parametrize("shape", [(0, 3, 100, 64, 32), (2, -1, 100, 64, 32), (2, 3, 0, 64, 32),
                                   (2, 3, 100, 0, 32), (2, 3, 100, 64, -16), (1, 1, 2 ** 31, 64, 64),
                                   (2 ** 40, 2 ** 30, 4, 16, 16)])
def test_bad_dims(lib, shape):
    assert fwd(lib, shape=shape) == DIM
    assert bwd(lib, shape=shape) == DIM
    assert lin(lib, shape=shape) == DIM


# Head sizes up to 128 whose rows are whole 16-byte pieces: multiples of 8
# for the 16-bit types, of 4 for fp32.
@pytest.mark.parametrize("E,M", [(256, 64), (64, 17), (12, 64), (64, 4), (136, 64), (64, 130)])
def test_unsupported_head_sizes(lib, E, M):
    shape = (2, 3, 100, E, M)
    for dt in (1, 2):
        assert fwd(lib, shape=shape, dtype=dt) == UNSUP
        assert bwd(lib, shape=shape, dtype=dt) == UNSUP
        assert lin(lib, shape=shape, dtype=dt) == UNSUP


@pytest.mark.parametrize("E,M", [(256, 64), (64, 17), (6, 64), (64, 2), (132, 64), (64, 130)])
def test_unsupported_head_sizes_f32(lib, E, M):
    shape = (2, 3, 100, E, M)
    assert fwd(lib, shape=shape, dtype=0) == UNSUP
    assert bwd(lib, shape=shape, dtype=0) == UNSUP
    assert lin(lib, shape=shape, dtype=0) == UNSUP


def test_unsupported_dtype_flag_eps(lib):
    assert fwd(lib, dtype=3) == UNSUP
    assert bwd(lib, dtype=-1) == UNSUP
    assert lin(lib, fm=2) == UNSUP
    assert lin(lib, eps=-1e-3) == UNSUP
    assert lin(lib, eps=math.nan) == UNSUP
    assert lin(lib, eps=math.inf) == UNSUP


def test_misaligned(lib):
    assert fwd(lib, v=A[2] + 8) == ALIGN
    assert fwd(lib, st=A[4] + 4) == ALIGN
    assert fwd(lib, s0=A[5] + 4) == ALIGN
    assert bwd(lib, dk=A[5] + 2) == ALIGN
    assert bwd(lib, st=A[7] + 8) == ALIGN
    assert bwd(lib, s0=A[8] + 8) == ALIGN
    assert bwd(lib, ds0=A[9] + 4) == ALIGN
    assert lin(lib, o=A[3] + 8) == ALIGN
    assert lin(lib, z0=A[6] + 4) == ALIGN
    assert lin(lib, zt=A[7] + 8) == ALIGN


def test_aliasing(lib):
    # SHAPE bf16: q, k are 2*3*100*64*2 = 76800 bytes; v, out 38400 bytes
    assert fwd(lib, o=A[0]) == ALIAS
    assert fwd(lib, o=A[1] + 76800 - 16) == ALIAS
    assert fwd(lib, st=A[3]) == ALIAS            # state_out overlaps out
    assert fwd(lib, st=A[2] + 16) == ALIAS       # state_out overlaps v
    assert bwd(lib, dq=A[5]) == ALIAS            # dq == dk
    assert bwd(lib, dv=A[3]) == ALIAS            # dv == dout
    assert bwd(lib, st=A[4]) == ALIAS            # state_final overlaps dq
    assert bwd(lib, s0=A[7], ds0=A[7] + 16) == ALIAS  # dstate_in overlaps state_in
    assert bwd(lib, ds0=A[6]) == ALIAS           # dstate_in overlaps dv
    assert fwd(lib, s0=A[5], st=A[5]) == ALIAS   # no in-place state update
    assert fwd(lib, s0=A[3]) == ALIAS            # state_in overlaps out
    assert lin(lib, o=A[2]) == ALIAS
    assert lin(lib, z0=A[5], zt=A[5]) == ALIAS
    assert lin(lib, st=A[5], zt=A[5] + 64) == ALIAS  # z_out inside state_out


def test_linear_attn_bwd_validation(lib):
    for name in ("q", "k", "v", "o", "g", "den", "dq", "dk", "dv"):
        assert linb(lib, **{name: None}) == NULL, name
    assert linb(lib, shape=(2, 3, 0, 64, 32)) == DIM
    assert linb(lib, shape=(2, 3, 100, 44, 32)) == UNSUP
    assert linb(lib, fm=3) == UNSUP
    assert linb(lib, dtype=5) == UNSUP
    assert linb(lib, dtype=2) == UNSUP            # no fp16 normalised backward
    assert linb(lib, den=A[5] + 4) == ALIGN
    assert linb(lib, dz0=A[9] + 8) == ALIGN
    assert linb(lib, dq=A[0]) == ALIAS            # dq overlaps q
    assert linb(lib, dv=A[5]) == ALIAS            # dv overlaps den
    assert linb(lib, ds0=A[9], s0=A[9]) == ALIAS  # gradient over its own state
    assert linb(lib, zt=A[9] + 4) == ALIGN
    assert linb(lib, dz0=A[9], zt=A[9]) == ALIAS  # gradient over the final z
    assert lin(lib, den=A[3]) == ALIAS            # den_out overlaps out
    assert lin(lib, den=A[5] + 4) == ALIGN


def test_f16_aliasing_uses_two_byte_elements(lib):
    # SHAPE fp16: q is 2*3*100*64*2 = 76800 bytes, as bf16
    assert fwd(lib, o=A[1] + 76800 - 16, dtype=2) == ALIAS
    assert bwd(lib, dq=A[5], dtype=2) == ALIAS


def fwd_na(lib, q=A[0], k=A[1], v=A[2], o=A[3], s0=None, st=None, shape=SHAPE, dtype=1):
    return lib.causal_product_fwd_noalloc(q, k, v, o, s0, st, *shape, dtype, None)


def test_noalloc_forward_validates_like_the_forward(lib):
    assert fwd_na(lib, q=None) == NULL
    assert fwd_na(lib, shape=(2, 3, 0, 64, 32)) == DIM
    assert fwd_na(lib, shape=(2, 3, 100, 256, 32)) == UNSUP
    assert fwd_na(lib, dtype=4) == UNSUP
    assert fwd_na(lib, v=A[2] + 8) == ALIGN
    assert fwd_na(lib, o=A[0]) == ALIAS
    assert fwd_na(lib, s0=A[5], st=A[5]) == ALIAS


@pytest.mark.parametrize("dtype", [0, 1, 2])
def test_noalloc_forward_rejects_more_scratch_than_it_holds(lib, dtype):
    # 16 slices of 16384 rows with 128-wide heads run as sequence segments
    # whose increments need 16 slices x 16 segments x (128*128 + 128) floats,
    # 16.1 MiB > 16 MiB: refused before anything is enqueued (no device here)
    assert fwd_na(lib, shape=(2, 8, 16384, 128, 128), dtype=dtype) == SCRATCH
    assert "16 MiB" in lib.cp_status_string(SCRATCH).decode()


# ---- workspaces (cp_workspace_size and the workspace arguments) ----

FEW = (2, 8, 16384, 128, 128)  # 16 slices of 16384 rows: run as sequence segments


def wsize(lib, op, shape, dtype=1):
    n = ctypes.c_int64(-1)
    st = lib.cp_workspace_size(op, *shape, dtype, ctypes.byref(n))
    return st, n.value


def test_workspace_size_rejects_bad_arguments(lib):
    assert lib.cp_workspace_size(0, *SHAPE, 1, None) == NULL
    assert wsize(lib, 4, SHAPE)[0] == UNSUP
    assert wsize(lib, -1, SHAPE)[0] == UNSUP
    assert wsize(lib, 0, (2, 3, 0, 64, 32))[0] == DIM
    assert wsize(lib, 1, (2, 3, 100, 256, 32))[0] == UNSUP
    assert wsize(lib, 0, SHAPE, dtype=5)[0] == UNSUP
    assert wsize(lib, 3, SHAPE, dtype=2)[0] == UNSUP  # no fp16 normalised backward


@pytest.mark.parametrize("op", range(4))
def test_workspace_size_zero_when_the_slices_fill_the_gpu(lib, op):
    # 128 slices of 4096 rows: one launch per call, no segments, no scratch
    assert wsize(lib, op, (8, 16, 4096, 64, 64)) == (OK, 0)
    assert wsize(lib, op, SHAPE) == (OK, 0)  # 100 rows: too short to split


@pytest.mark.parametrize("op", range(4))
def test_workspace_size_of_segmented_calls(lib, op):
    st, n = wsize(lib, op, FEW)
    assert st == OK and n > 0
    per_seg = 16 * (128 * 128 + 128) * 4  # one increment per slice and segment
    # forward: one increment per segment; backward: prefix and suffix ones
    unit = per_seg * (1 if op in (0, 2) else 2)
    assert n % unit == 0 and 2 <= n // unit <= 64
    if op == 0:  # the figure the no-allocation forward refuses (16.1 MiB)
        assert n == 16 * 16 * (128 * 128 + 128) * 4
    # the same for the 16-bit types, and fp32 is planned on its own tiles
    if op != 3:
        assert wsize(lib, op, FEW, dtype=2) == (OK, n)
    assert wsize(lib, op, FEW, dtype=0)[0] == OK


def test_workspace_arguments_are_validated_before_any_device_call(lib):
    # misaligned, overlapping an input or an output: refused by validation
    assert fwd(lib, ws=A[11] + 8, wsb=1 << 20) == ALIGN
    assert fwd(lib, ws=A[0], wsb=1 << 20) == ALIAS
    assert bwd(lib, ws=A[4] + 16, wsb=64) == ALIAS
    assert lin(lib, ws=A[2], wsb=16) == ALIAS
    assert linb(lib, ws=A[8], wsb=16) == ALIAS
    # too small for a segmented call: refused on the host (no device here)
    for f, op in ((fwd, 0), (bwd, 1), (lin, 2), (linb, 3)):
        need = wsize(lib, op, FEW)[1]
        assert f(lib, shape=FEW, ws=A[11], wsb=need - 16) == SCRATCH, op
        assert f(lib, shape=FEW, ws=A[11], wsb=-1) == SCRATCH, op
    assert "cp_workspace_size" in lib.cp_status_string(SCRATCH).decode()
