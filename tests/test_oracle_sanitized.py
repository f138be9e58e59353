"""The oracle (test infrastructure, plain C) under AddressSanitizer and
UndefinedBehaviorSanitizer, host code only: the same cases run through an
instrumented build in a child process (with the ASan runtime preloaded, since
Python itself is not instrumented) must raise no report and give the same
results as the ordinary build.  The cases cover ragged and empty packed
sequences, T = 0, tiny and full head dims, with and without initial states."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import sys
import numpy as np
import oracle

def bf16(a):
    return (np.asarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)

plain = oracle.Oracle()
san = oracle.Oracle(sys.argv[1])
rng = np.random.default_rng(11)
cases = [(2, 70, 3, 8, 8, None, True), (1, 150, 2, 16, 8, [0, 64, 1, 85], True),
         (1, 0, 2, 4, 4, None, True), (1, 3, 1, 4, 4, [0, 0, 3], False), (1, 130, 1, 128, 128, None, False)]
for (B, T, H, K, V, lens, init) in cases:
    q, k, g = (bf16(rng.standard_normal((B, T, H, K))) for _ in range(3))
    v = bf16(rng.standard_normal((B, T, H, V)))
    beta = bf16(rng.standard_normal((B, T, H)))
    A_log = np.log(rng.uniform(1, 16, size=H)).astype(np.float32)
    dt_bias = (0.1 * rng.standard_normal((H, K))).astype(np.float32)
    cu = None if lens is None else np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    N = B if cu is None else len(lens)
    h0 = (0.1 * rng.standard_normal((N, H, K, V))) if init else None
    args = (q, k, v, g, beta, 0.125, A_log, dt_bias, -5.0)
    o1, f1 = plain.fwd(*args, initial_state=h0, cu_seqlens=cu, num_threads=2)
    o2, f2 = san.fwd(*args, initial_state=h0, cu_seqlens=cu, num_threads=2)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2), (B, T, H, K, V, lens)
print("sanitized oracle ok", flush=True)
'''


def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    libasan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    if not os.path.isabs(libasan) or not os.path.exists(libasan):
        pytest.skip("gcc has no AddressSanitizer runtime here")
    oracle.build()
    so = str(tmp_path / "libkda_oracle_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
                           "-ffp-contract=off", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=undefined", oracle._SRC, "-o", so, "-lm"])
    env = dict(os.environ, LD_PRELOAD=libasan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="2",
               PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-c", CHILD, so], env=env, cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and "sanitized oracle ok" in r.stdout, r.stdout[-3000:] + r.stderr[-3000:]
