"""rts_sample_tokens_noalloc (the library's static scratch, for callers that
cannot allocate) against rts_sample_tokens with a caller workspace: the same
kernels run, so every output must be the same bit for bit, on two calls in
a row, the second with a smaller input (the scratch keeps the first call's
contents), and on a call after many other calls in the same process."""
import numpy as np
import pytest
import torch

import request_token_sampling_amd as R
from request_token_sampling_amd import workloads as W

from parity import say

pytestmark = pytest.mark.gpu


def bits(t):
    """Bit patterns of an output tensor (floats compared as their bits)."""
    if t.dtype == torch.float32:
        t = t.view(torch.int32)
    return t.cpu().numpy()


def assert_same(a, b, tag):
    assert a.keys() == b.keys(), tag
    for k in a:
        assert np.array_equal(bits(a[k]), bits(b[k])), (tag, k)


def both(x, params, hist=None, hist_len=None, **kw):
    """The two entry points on the same inputs, each with its own
    device-resident counters starting at the rows' counters."""
    ctr = [p.get("counter", 0) for p in params]
    ca = torch.tensor(ctr, dtype=torch.int64, device="cuda")
    cb = ca.clone()
    a = R.sample_tokens(x, params, hist, hist_len, counters=ca, counter_stride=len(params), **kw)
    b = R.sample_tokens_noalloc(x, params, hist, hist_len, counters=cb,
                                counter_stride=len(params), **kw)
    torch.cuda.synchronize()
    assert torch.equal(ca, cb)
    return a, b


def big_call():
    """40 rows of V = 248,320: the batch-slot rows with penalties over shared
    history rows, raw top-20 logprobs and lists renormalising them."""
    w = W.batch_slots()
    x = torch.from_numpy(w["logits"]).cuda()
    h = torch.from_numpy(np.asarray(w["history"], np.int32)).cuda()
    rng = np.random.default_rng(5)
    lists = [rng.choice(W.V_FULL, 1000, replace=False).astype(np.int32) for _ in range(40)]
    ids, off = W.pack_allowed(lists)
    return both(x, w["params"], h, w["hist_len"], logprobs=20,
                logprob_allowed=torch.from_numpy(ids).cuda(), logprob_allowed_off=off)


def small_call():
    """3 rows of V = 5,003 (ragged last chunk): a sampled row, a greedy row
    and a masked sampled row."""
    rng = np.random.default_rng(6)
    V = 5003
    x = torch.from_numpy(rng.normal(0, 2, (3, V)).astype(np.float32)).cuda()
    params = [W.row_params(temperature=0.8, top_k=33, top_p=0.9, min_p=0.02, seed=9, counter=4),
              W.row_params(),
              W.row_params(temperature=1.2, top_k=64, seed=9, counter=5)]
    allowed = [np.zeros(0, np.int32), np.zeros(0, np.int32),
               rng.choice(V, 100, replace=False).astype(np.int32)]
    ids, off = W.pack_allowed(allowed)
    return both(x, params, logprobs=5, allowed=torch.from_numpy(ids).cuda(), allowed_off=off)


def test_noalloc_equals_the_workspace_call():
    say("noalloc: 40 rows, V = 248,320, penalties, logprobs, renormalising lists")
    a, b = big_call()
    assert_same(a, b, "40 rows")
    say("noalloc: then 3 rows, V = 5,003, masked row")
    a, b = small_call()
    assert_same(a, b, "3 rows")
    say("noalloc: the 40 rows again")
    a, b = big_call()
    assert_same(a, b, "40 rows again")


def test_noalloc_refuses_more_than_its_scratch():
    cap = R.noalloc_scratch_bytes()
    assert R.workspace_bytes(64, 400_000) > cap
    x = torch.zeros((1, 400_000), dtype=torch.float32, device="cuda").expand(64, -1)
    with pytest.raises(R.RTSError) as e:
        R.sample_tokens_noalloc(x, [W.row_params()] * 64)
    assert e.value.code == R.RTS_ENOSPC and "static scratch" in str(e.value)
