"""GPU draw statistics.  Over many Philox counters the sampled ids follow
the temperature-scaled probabilities of the candidates that survive the
cuts (page "#19 serve: per-request temperature/top_p/top_k/min_p/penalties
sampling", "What changed": temperature, then a draw over the kept set keyed
by (seed, counter)).  Parity against the oracle pins each draw; this pins
the distribution the draws come from, with the GPU alone drawing."""
import numpy as np
import pytest
import scipy.stats
import torch

import oracle.oracle as O
import request_token_sampling_amd as R
from request_token_sampling_amd import workloads as W

from parity import say, to_dev

pytestmark = pytest.mark.gpu


def _flat_row():
    x = np.random.default_rng(77).normal(0.0, 1.0, (1, 50_000)).astype(np.float32)
    p = W.row_params(temperature=1.3, top_k=64, top_p=1.0, min_p=0.05, seed=2024, counter=0)
    return x, p


def _single_stream_row():
    w = W.single_stream()
    return w["logits"], w["sampled"][0]


@pytest.mark.parametrize("case", ["single_stream", "flat_k64"])
def test_draws_follow_tempered_probabilities(case):
    x, p = _single_stream_row() if case == "single_stream" else _flat_row()
    rows, calls = 64, 4096  # 262,144 draws: 64 parameter rows over the one logits row
    say("case draw statistics", case, rows * calls)
    ctr = torch.arange(rows, dtype=torch.int64, device="cuda")
    call = R.SampleCall(to_dev(x).expand(rows, -1), [p] * rows, counters=ctr,
                        counter_stride=rows)
    out = torch.empty((calls, rows), dtype=torch.int32, device="cuda")
    for i in range(calls):
        call()
        out[i].copy_(call.token)
    torch.cuda.synchronize()
    tok = out.cpu().numpy().ravel()
    assert int(ctr[0].item()) == rows * calls  # every call advanced the counters

    # the survivors and their tempered weights do not depend on the counter
    o = O.sample_row(x[0], p)
    n = int(o["counts"][2])
    ids = o["kept_ids"][:n]
    y = o["kept_logits"][:n].astype(np.float64)
    prob = np.exp((y - y[0]) / float(np.float32(p["temperature"])))
    prob /= prob.sum()
    assert n > 1, "the case must leave a choice"
    assert np.isin(tok, ids).all(), "a draw outside the survivors"
    picks = np.array([(tok == i).sum() for i in ids], np.int64)
    chi2, pv = scipy.stats.chisquare(picks, prob * tok.size)
    say("  survivors", n, "chi2", round(float(chi2), 1), "p", float(pv))
    assert pv > 1e-4, (picks, prob * tok.size)
