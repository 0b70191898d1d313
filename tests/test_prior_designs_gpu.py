"""GPU parity of the pages' earlier sampler designs (rts_sample_tokens_prior:
one thread per row with k full-vocabulary rescans, one workgroup per row with
k argmax rounds, and the latter with the per-candidate penalty recount)
against the CPU oracle, to the same bar as the single-pass kernel
(tests/parity.py).  They exist as measured ablations; their outputs must
still be the chain's."""
import numpy as np
import pytest
import torch

import request_token_sampling_amd as R
from request_token_sampling_amd import workloads as W

from parity import compare_sample, oracle_sample, say, to_dev

pytestmark = pytest.mark.gpu

DESIGNS = [R.PRIOR_THREAD, R.PRIOR_BLOCK, R.PRIOR_RECOUNT]


def gpu_prior(design, x, params, history=None, hist_len=None):
    h = None if history is None else to_dev(np.asarray(history, np.int32))
    call = R.PriorCall(design, to_dev(np.asarray(x, np.float32)), params, h, hist_len)()
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in call.results().items()}


@pytest.mark.parametrize("design", DESIGNS)
def test_tiny_and_greedy(design):
    w = W.tiny()
    say("case prior tiny", design)
    compare_sample(gpu_prior(design, w["logits"], w["sampled"]),
                   oracle_sample(w["logits"], w["sampled"]), f"prior {design} tiny")
    compare_sample(gpu_prior(design, w["logits"], w["greedy"]),
                   oracle_sample(w["logits"], w["greedy"]), f"prior {design} greedy")


@pytest.mark.parametrize("design", DESIGNS)
def test_single_stream_full_vocab(design):
    w = W.single_stream()
    say("case prior single", design)
    compare_sample(gpu_prior(design, w["logits"], w["sampled"]),
                   oracle_sample(w["logits"], w["sampled"]), f"prior {design} single")


@pytest.mark.parametrize("design", DESIGNS)
def test_verify_window_with_visible_penalties(design):
    vw = W.VerifyWindows()
    hist = vw.history.reshape(1, -1)
    x = W.boost_history(vw.next_logits(), vw.history, 12.0)
    p = vw.params(0)
    say("case prior window", design)
    compare_sample(gpu_prior(design, x, p, hist, [64]), oracle_sample(x, p, hist, [64]),
                   f"prior {design} window")


@pytest.mark.parametrize("design", [R.PRIOR_BLOCK, R.PRIOR_RECOUNT])
def test_ties_specials_and_many_rows(design):
    rng = np.random.default_rng(41)
    B, Vx = 70, 4099
    x = rng.integers(-6, 6, (B, Vx)).astype(np.float32)
    x[1, :] = -np.inf
    x[2, ::3] = np.nan
    x[3, 10:20] = np.inf
    hist = rng.integers(0, Vx, (1, 300)).astype(np.int32)
    params = [W.row_params(temperature=float(np.float32(0.5 + (r % 5) * 0.3)),
                           top_k=1 + (r * 7) % 64, top_p=0.9, min_p=0.01, seed=r, counter=r,
                           penalty_repeat=1.2, penalty_freq=0.1, penalty_last_n=100,
                           history_row=0 if r % 2 else -1)
              for r in range(B)]
    say("case prior ties", design)
    compare_sample(gpu_prior(design, x, params, hist, [300]), oracle_sample(x, params, hist, [300]),
                   f"prior {design} ties")
