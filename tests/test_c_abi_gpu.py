"""The library used from plain C++ through include/rts.h and the HIP runtime
alone -- no Python binding, no torch (tests/c_abi_consumer.cpp, built next to
the library by __graft_entry__.build()) -- against the CPU oracle, to the bar
of tests/parity.py."""
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle.oracle as O
from request_token_sampling_amd import workloads as W
from request_token_sampling_amd.build_lib import CONSUMER

from parity import LP_ATOL, assert_flagged_row, say

pytestmark = pytest.mark.gpu

TOP_N = 5


def consumer_params(B):
    """The parameters the consumer hard-codes: even rows sampled, odd greedy."""
    return [W.row_params(temperature=0.8, top_k=8, top_p=0.9, min_p=0.05, seed=42, counter=r)
            if r % 2 == 0 else W.row_params() for r in range(B)]


@pytest.mark.parametrize("B,V", [(6, 70001), (3, 248320)])
def test_c_consumer_matches_the_oracle(B, V):
    assert os.path.exists(CONSUMER), "tests/_build/c_abi_consumer is not built"
    say("case c consumer", B, V)
    x = np.random.default_rng(50 + B).normal(0, 3, (B, V)).astype(np.float32)
    with tempfile.TemporaryDirectory() as d:
        fin, fout = os.path.join(d, "in.bin"), os.path.join(d, "out.bin")
        with open(fin, "wb") as f:
            np.array([B, V], np.int32).tofile(f)
            x.tofile(f)
        run = subprocess.run([CONSUMER, fin, fout], capture_output=True, text=True, timeout=120)
        assert run.returncode == 0, run.stderr
        raw = open(fout, "rb").read()
    off = 0

    def take(dtype, n):
        nonlocal off
        a = np.frombuffer(raw, dtype=dtype, count=n, offset=off)
        off += 4 * n
        return a

    tok = take(np.int32, B)
    counts = take(np.int32, 3 * B).reshape(B, 3)
    kept = take(np.int32, 64 * B).reshape(B, 64)
    lp = take(np.float32, B)
    top_ids = take(np.int32, TOP_N * B).reshape(B, TOP_N)
    top_lp = take(np.float32, TOP_N * B).reshape(B, TOP_N)
    assert off == len(raw)

    o = O.sample_tokens(x, consumer_params(B))
    ol = O.token_logprobs(x, o["token"], TOP_N)
    for r in range(B):
        where = f"c consumer row {r}"
        assert np.array_equal(kept[r], o["kept_ids"][r]), where
        assert np.array_equal(counts[r, :2], o["counts"][r, :2]), where
        if o["flags"][r]:
            assert_flagged_row(o, r, int(counts[r, 2]), int(tok[r]), where)
            continue
        assert counts[r, 2] == o["counts"][r, 2] and tok[r] == o["token"][r], where
        assert abs(float(lp[r]) - ol["token_lp"][r]) <= LP_ATOL, where
        assert np.array_equal(top_ids[r], ol["top_ids"][r]), where
        assert np.all(np.abs(top_lp[r].astype(np.float64) - ol["top_lp"][r]) <= LP_ATOL), where
