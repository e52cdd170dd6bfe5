"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer, and its
independence of the OpenMP thread count.

oracle/sanitize_driver.c includes the oracle source and calls every entry
point once on small random inputs (N = 2^6, 6 + 2 primes, dnum 3); it is
built with gcc and both sanitizers (any report aborts the run) and run as a
separate process.  The thread-count check compares whole outputs word for
word at 1 and at 4 threads."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import ckks_synth as S
from helpers import config_params

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = tmp_path / "orc_san"
    src = os.path.join(ROOT, "oracle", "sanitize_driver.c")
    subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", "-fopenmp", "-std=gnu11", "-I", os.path.join(ROOT, "oracle"),
                           src, "-lm", "-o", str(exe)])
    env = dict(os.environ, OMP_NUM_THREADS="2")
    r = subprocess.run([str(exe)], env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr
    assert "sanitized oracle run: ok" in r.stdout


def test_oracle_words_do_not_depend_on_thread_count(orc):
    P = config_params(orc, "C3", log_n=10)
    level = 23
    cts = S.uniform_limbs(S.stream(21, "thr/ct"), P.q, P.N, lead=(3, 2))
    keys = [S.uniform_limbs(S.stream(21 + b, "thr/k"), P.mods, P.N, lead=(P.dnum, 2)) for b in range(3)]
    gs = [P.galois(k) for k in (1, 77, 300)]
    threads = orc.num_threads()
    try:
        orc.set_num_threads(1)
        one = orc.rotate_batch(P, level, cts, gs, keys)
        mrr1 = orc.mul_relin_rescale(P, level, cts[:2], cts[1:], keys[0])
        orc.set_num_threads(4)
        four = orc.rotate_batch(P, level, cts, gs, keys)
        mrr4 = orc.mul_relin_rescale(P, level, cts[:2], cts[1:], keys[0])
    finally:
        orc.set_num_threads(threads)
    assert np.array_equal(one, four)
    assert np.array_equal(mrr1, mrr4)
