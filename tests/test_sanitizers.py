"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The C ABI's argument checks (prefix_sum_causal_amd/csrc/cp_validate.hpp),
  compiled with g++ -fsanitize=address,undefined into a driver
  (tests/sanitize/validate_driver.cpp) that runs valid and invalid calls,
  extreme sizes and aliasing cases; any sanitizer report aborts it.
* The fp64 oracle (oracle/oracle.c), compiled with the same sanitizers into a
  separate library and run in a child process (the sanitizer runtime
  preloaded) on small random inputs through every function, carried states
  included; its results must equal those of the ordinary build.
"""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def _libasan():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_abi_validation_under_sanitizers(tmp_path):
    exe = tmp_path / "validate_driver"
    subprocess.check_call(["g++", "-std=c++17", "-O1", *SAN, "-I", os.path.join(ROOT, "include"), "-I",
                           os.path.join(ROOT, "prefix_sum_causal_amd", "csrc"),
                           os.path.join(ROOT, "tests", "sanitize", "validate_driver.cpp"), "-o", str(exe)])
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout


CHILD = textwrap.dedent("""
    import sys
    import numpy as np
    sys.path.insert(0, {root!r})
    import oracle
    san = oracle.Oracle({lib!r})
    ref = oracle.default()
    rng = np.random.default_rng(11)
    for (N, H, L, E, M) in ((1, 1, 1, 4, 4), (2, 3, 37, 8, 5), (1, 2, 65, 16, 16)):
        Q = rng.standard_normal((N, H, L, E)).astype(np.float32)
        K = rng.standard_normal((N, H, L, E)).astype(np.float32)
        V = rng.standard_normal((N, H, L, M)).astype(np.float32)
        dO = rng.standard_normal((N, H, L, M)).astype(np.float32)
        S0 = rng.standard_normal((N, H, E, M)).astype(np.float32)
        z0 = rng.uniform(1, 2, (N, H, E)).astype(np.float32)
        Qp, Kp = np.exp(Q), np.exp(K)
        pairs = [
            (san.fwd(Qp, Kp, V, S0, return_state=True), ref.fwd(Qp, Kp, V, S0, return_state=True)),
            (san.fwd_brute(Qp, Kp, V, S0), ref.fwd_brute(Qp, Kp, V, S0)),
            (san.bwd(Qp, Kp, V, dO, S0, with_dS0=True), ref.bwd(Qp, Kp, V, dO, S0, with_dS0=True)),
            (san.bwd_brute(Qp, Kp, V, dO, S0, with_dS0=True), ref.bwd_brute(Qp, Kp, V, dO, S0, with_dS0=True)),
            (san.linattn(Q, K, V, 1e-6, 1, S0, z0, return_state=True), ref.linattn(Q, K, V, 1e-6, 1, S0, z0, return_state=True)),
            (san.linattn_brute(Q, K, V, 1e-6, 0, S0, z0), ref.linattn_brute(Q, K, V, 1e-6, 0, S0, z0)),
            (san.linattn_bwd(Q, K, V, dO, 1e-6, 1, S0, z0), ref.linattn_bwd(Q, K, V, dO, 1e-6, 1, S0, z0)),
            (san.state(Kp, V), ref.state(Kp, V)),
        ]
        for a, b in pairs:
            a = a if isinstance(a, tuple) else (a,)
            b = b if isinstance(b, tuple) else (b,)
            for x, y in zip(a, b):
                assert x.shape == y.shape and np.array_equal(x, y), (N, H, L, E, M)
    print("sanitized oracle ok")
""")


def test_oracle_under_sanitizers(tmp_path):
    asan = _libasan()
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = tmp_path / "liboracle_san.so"
    subprocess.check_call(["gcc", "-std=c99", "-O1", *SAN, "-fPIC", "-shared", "-fopenmp",
                           os.path.join(ROOT, "oracle", "oracle.c"), "-o", str(lib), "-lm"])
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, lib=str(lib))], capture_output=True,
                       text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "sanitized oracle ok" in r.stdout
