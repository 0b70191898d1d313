"""GPU parity of the logprobs a sampling call computes in its own pass over
the logits (rts_logprob_request): tokens and kept sequences to the sampling
bar, logprobs to the logprob bar (tests/parity.py), against the CPU oracle.

Cases cover both ways the kernel gets the raw top entries: from the kept
list itself (no penalties and top_k >= top_n) and from a second selection
over the raw values (penalties on, or top_k < top_n, greedy rows), plus the
raw selection's overflow path, ragged and unaligned rows and many launches."""
import numpy as np
import pytest

import request_token_sampling_amd as R
from request_token_sampling_amd import workloads as W

from parity import (compare_fused_logprobs, compare_sample, gpu_sample, oracle_sample, say,
                    to_dev)

pytestmark = pytest.mark.gpu

V = W.V_FULL


def sampled(**kw):
    d = dict(temperature=1.0, top_k=64, top_p=1.0, min_p=0.0, seed=11, counter=0)
    d.update(kw)
    return W.row_params(**d)


def check(x, params, top_n, history=None, hist_len=None, tag="", logits_dev=None):
    say("case fused", tag, np.asarray(x).shape, "top_n", top_n)
    g = gpu_sample(x, params, history, hist_len, logits_dev=logits_dev, logprobs=top_n)
    o = oracle_sample(x, params, history, hist_len)
    compare_sample(g, o, tag)
    compare_fused_logprobs(g, o, x, top_n, tag)
    return g, o


def test_stress_rows_share_the_kept_list():
    w = W.logprobs_stress()
    check(w["logits"], w["params"], w["top_n"], tag="stress fused")


@pytest.mark.parametrize("top_n", [20, 5, 0])
def test_batch_with_penalties_takes_a_raw_selection(top_n):
    w = W.batch_slots()
    check(w["logits"], w["params"], top_n, w["history"], w["hist_len"], tag=f"batch fused")


def test_single_stream_and_greedy():
    w = W.single_stream()
    check(w["logits"], w["sampled"], 20, tag="single fused")
    check(w["logits"], w["greedy"], 20, tag="single greedy fused")   # k = 1 < top_n
    check(w["logits"], w["greedy"], 1, tag="single greedy top1")     # k = 1 = top_n


def test_mixed_top_k_around_top_n():
    rng = np.random.default_rng(21)
    x = rng.normal(0, 3, (8, V)).astype(np.float32)
    params = [sampled(top_k=k, counter=i, top_p=0.95, min_p=0.01)
              for i, k in enumerate((1, 5, 19, 20, 21, 64))] + [W.row_params(), W.row_params()]
    check(x, params, 20, tag="top_k around top_n")


@pytest.mark.parametrize("Vx", [1, 7, 1025, 8193, 65537])
def test_ragged_vocab(Vx):
    rng = np.random.default_rng(Vx + 3)
    x = rng.normal(0, 3, (3, Vx)).astype(np.float32)
    params = [sampled(top_k=64, top_p=0.9, counter=1), sampled(top_k=3, seed=4), W.row_params()]
    check(x, params, 20, tag=f"fused V={Vx}")


def test_special_values_and_overflow_paths():
    """Rows of equal values overflow every chunk's candidate regions (both
    selections) and the row merges; NaN and +inf take their mapped values."""
    rng = np.random.default_rng(22)
    x = rng.normal(0, 3, (5, V)).astype(np.float32)
    x[0] = 0.0
    x[1] = -np.inf
    x[1, 99] = np.nan
    x[2, ::7] = np.nan
    x[2, 5000:5040] = np.inf
    x[3] = 1.0
    x[3, 200000] = 3.0
    H = np.arange(0, 256, dtype=np.int32).reshape(1, 256)
    params = [sampled(top_k=8, counter=1, penalty_repeat=1.2, penalty_last_n=-1, history_row=0),
              sampled(top_k=64, counter=2),
              sampled(top_k=30, counter=3, penalty_freq=0.3, penalty_last_n=-1, history_row=0),
              W.row_params(penalty_repeat=1.5, penalty_last_n=-1, history_row=0),
              sampled(top_k=4, counter=5)]
    check(x, params, 20, H, [256], tag="special fused")


def test_unaligned_rows():
    rng = np.random.default_rng(23)
    B, Vx, ld = 3, 10007, 10013
    buf = rng.normal(0, 3, B * ld + 1).astype(np.float32)
    dev = to_dev(buf)
    params = [sampled(top_k=10, counter=r) for r in range(B)]
    for off in (0, 1):
        view = dev[off:off + B * ld].view(B, ld)[:, :Vx]
        host = np.ascontiguousarray(buf[off:off + B * ld].reshape(B, ld)[:, :Vx])
        check(host, params, 20, tag=f"unaligned off={off}", logits_dev=view)


def test_many_launches():
    rng = np.random.default_rng(24)
    B, Vx = 140, 3000
    x = rng.normal(0, 2, (B, Vx)).astype(np.float32)
    params = [W.row_params() if r % 4 == 0 else
              sampled(top_k=int(rng.integers(1, 65)), seed=r, counter=r) for r in range(B)]
    check(x, params, 7, tag="fused 140 rows")


def test_fused_matches_separate_call():
    """The fused logprobs equal those of rts_token_logprobs on the sampled
    tokens (same partial sums and merge order), to the logprob bar."""
    w = W.batch_slots()
    xd = to_dev(w["logits"])
    hd = to_dev(w["history"])
    fused = R.sample_tokens(xd, w["params"], hd, w["hist_len"], logprobs=20)
    sep = R.token_logprobs(xd, fused["token"], 20)
    for k in ("top_ids",):
        assert np.array_equal(fused[k].cpu().numpy(), sep[k].cpu().numpy())
    for k in ("token_lp", "top_lp"):
        a, b = fused[k].cpu().numpy(), sep[k].cpu().numpy()
        assert np.all(np.abs(a - b) <= 1e-5), k
