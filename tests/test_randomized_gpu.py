"""Seeded random configurations through the whole call surface at once:
random B, V, logit distributions (normal, integer ties, bf16 grids, special
values), per-row parameters (greedy and sampled, penalties over random
windows with foreign ids, masks), fused logprobs, broadcast rows (ld = 0) and
device counters, each against the oracle (page "#19 serve: per-request
temperature/top_p/top_k/min_p/penalties sampling", "What changed"; page
"#3200 [Engine] OpenAI logprobs / top_logprobs / allowed_token_ids for the
CUDA/HIP engine", "Approach")."""
import numpy as np
import pytest
import torch

import oracle.oracle as O
import request_token_sampling_amd as R
from request_token_sampling_amd import workloads as W

from parity import (compare_fused_logprobs, compare_logprobs, compare_renormalised,
                    compare_sample, say, to_dev)

pytestmark = pytest.mark.gpu


def _logits(rng, B, V):
    kind = rng.integers(0, 4)
    if kind == 0:
        x = rng.normal(0, rng.uniform(0.5, 4), (B, V))
    elif kind == 1:
        x = rng.integers(-8, 9, (B, V))
    elif kind == 2:
        x = rng.normal(0, 3, (B, V)).astype(np.float32)
        x = (x.view(np.uint32) & 0xFFFF0000).view(np.float32)
    else:
        x = rng.normal(0, 2, (B, V))
        for r in range(B):
            pos = rng.choice(V, min(V, 12), replace=False)
            x[r, pos[:3]] = np.nan
            x[r, pos[3:5]] = np.inf
            x[r, pos[5:8]] = -np.inf
    return np.asarray(x, np.float32), int(kind)


def _params(rng, B, H, V):
    out = []
    for r in range(B):
        if rng.random() < 0.2:
            p = W.row_params()
        else:
            p = W.row_params(temperature=float(rng.uniform(0.1, 2.0)), top_k=int(rng.integers(1, 65)),
                             top_p=float(rng.uniform(0.3, 1.0)) if rng.random() < 0.7 else 1.0,
                             min_p=float(rng.uniform(0, 0.3)) if rng.random() < 0.5 else 0.0,
                             seed=int(rng.integers(0, 1 << 62)), counter=int(rng.integers(0, 1 << 40)))
        if H and rng.random() < 0.5:
            p.update(penalty_repeat=float(rng.uniform(0.7, 1.6)),
                     penalty_freq=float(rng.uniform(-0.3, 0.6)),
                     penalty_present=float(rng.uniform(-0.3, 0.6)),
                     penalty_last_n=int(rng.choice([-1, 0, 1, 8, 64, 300])),
                     history_row=int(rng.integers(0, H)))
        out.append(p)
    return out


@pytest.mark.parametrize("seed", range(48))
def test_random_configuration(seed):
    rng = np.random.default_rng(7000 + seed)
    B = int(rng.choice([1, 2, 3, 5, 17, 40, 70]))
    V = int(rng.choice([1, 7, 100, 1023, 4097, 30011, 65536, 120000]))
    broadcast = B > 1 and rng.random() < 0.25
    x, kind = _logits(rng, 1 if broadcast else B, V)
    xs = np.repeat(x, B, axis=0) if broadcast else x
    H = int(rng.integers(0, 3))
    hist = rng.integers(-2, V + 2, (H, 200)).astype(np.int32) if H else None
    hist_len = [int(rng.integers(0, 201)) for _ in range(H)] if H else None
    params = _params(rng, B, H, V)
    masked = rng.random() < 0.3
    lists = [None] * B
    if masked:
        for r in range(B):
            if rng.random() < 0.5:
                lists[r] = rng.integers(-3, V + 3, int(rng.integers(0, 40))).astype(np.int32)
    top_n = int(rng.choice([0, 1, 5, 20])) if rng.random() < 0.5 else None
    say("case random", seed, dict(B=B, V=V, kind=kind, broadcast=broadcast, H=H, masked=masked,
                                  top_n=top_n))

    xd = to_dev(x)
    view = xd.expand(B, -1) if broadcast else xd
    hd = None if hist is None else to_dev(hist)
    ctr = to_dev(np.array([p["counter"] for p in params], np.int64))
    kw = {}
    if masked:
        ids, off = W.pack_allowed(lists)
        kw = dict(allowed=to_dev(ids) if ids.size else torch.zeros(1, dtype=torch.int32,
                                                                     device="cuda"),
                  allowed_off=off)
    out = R.sample_tokens(view, params, hd, hist_len, counters=ctr, counter_stride=3,
                          logprobs=top_n, **kw)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in out.items()}
    if masked:
        o = O.sample_tokens_masked(xs, params, lists, hist, hist_len)
    else:
        o = O.sample_tokens(xs, params, hist, hist_len)
    compare_sample(g, o, f"random {seed}")
    if top_n is not None:
        compare_fused_logprobs(g, o, xs, top_n, f"random {seed} logprobs")
    assert np.array_equal(ctr.cpu().numpy(), [p["counter"] + 3 for p in params])


@pytest.mark.parametrize("seed", range(24))
def test_random_logprob_configuration(seed):
    """rts_token_logprobs on seeded random inputs: unrestricted rows, short
    allowed lists (gathered into registers) and long ones (walked in the
    bitmap), duplicates, foreign ids and out-of-range tokens."""
    rng = np.random.default_rng(9000 + seed)
    B = int(rng.choice([1, 3, 17, 40, 70]))
    V = int(rng.choice([1, 9, 1000, 4097, 30011, 120000]))
    x, kind = _logits(rng, B, V)
    top_n = int(rng.choice([0, 1, 7, 20]))
    tokens = rng.integers(-2, V + 2, B).astype(np.int32)
    lists = None
    if rng.random() < 0.6:
        lists = []
        for r in range(B):
            u = rng.random()
            if u < 0.3:
                lists.append(None)
            elif u < 0.8:
                lists.append(rng.integers(-3, V + 3, int(rng.integers(0, 300))).astype(np.int32))
            else:
                lists.append(rng.integers(-3, V + 3, int(rng.integers(4097, 6000))).astype(np.int32))
            if lists[-1] is not None and lists[-1].size and rng.random() < 0.5:
                tokens[r] = lists[-1][0]            # a listed token (maybe foreign)
    say("case random logprobs", seed, dict(B=B, V=V, kind=kind, top_n=top_n,
                                           allowed=lists is not None))
    xd = to_dev(x)
    t = to_dev(tokens)
    if lists is not None:
        ids, off = W.pack_allowed(lists)
        out = R.token_logprobs(xd, t, top_n, to_dev(ids) if ids.size else
                               torch.zeros(1, dtype=torch.int32, device="cuda"), off)
    else:
        out = R.token_logprobs(xd, t, top_n)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in out.items()}
    o = O.token_logprobs(x, tokens, top_n, lists)
    compare_logprobs(g, o, f"random logprobs {seed}")


@pytest.mark.parametrize("seed", range(24))
def test_random_renormalised_configuration(seed):
    """Sampling calls that also renormalise their logprobs over allowed
    lists: lists of random length (past 2,048 ids some rows take the
    separate pass), repeats and foreign ids, sometimes with candidate masks
    on other rows (separate pass), penalties, broadcast rows."""
    rng = np.random.default_rng(11000 + seed)
    B = int(rng.choice([1, 2, 5, 17, 40, 70]))
    V = int(rng.choice([7, 100, 1023, 4097, 30011, 120000]))
    broadcast = B > 1 and rng.random() < 0.25
    x, kind = _logits(rng, 1 if broadcast else B, V)
    xs = np.repeat(x, B, axis=0) if broadcast else x
    H = int(rng.integers(0, 3))
    hist = rng.integers(-2, V + 2, (H, 200)).astype(np.int32) if H else None
    hist_len = [int(rng.integers(0, 201)) for _ in range(H)] if H else None
    params = _params(rng, B, H, V)
    top_n = int(rng.choice([0, 1, 5, 20]))
    lists = []
    for r in range(B):
        u = rng.random()
        if u < 0.2:
            lists.append(None)
        elif u < 0.85:
            lists.append(rng.integers(-3, V + 3, int(rng.integers(0, 700))).astype(np.int32))
        else:
            lists.append(rng.integers(-3, V + 3, int(rng.integers(1900, 2300))).astype(np.int32))
    masks = None
    if rng.random() < 0.2:
        masks = [None] * B
        masks[int(rng.integers(0, B))] = rng.integers(0, V, 30).astype(np.int32)
    say("case random renorm", seed, dict(B=B, V=V, kind=kind, broadcast=broadcast, H=H,
                                         top_n=top_n, masks=masks is not None,
                                         longest=max((0 if a is None else a.size) for a in lists)))
    xd = to_dev(x)
    view = xd.expand(B, -1) if broadcast else xd
    hd = None if hist is None else to_dev(hist)
    ids, off = W.pack_allowed(lists)
    kw = dict(logprob_allowed=to_dev(ids) if ids.size else torch.zeros(1, dtype=torch.int32,
                                                                       device="cuda"),
              logprob_allowed_off=off)
    if masks is not None:
        mids, moff = W.pack_allowed(masks)
        kw.update(allowed=to_dev(mids), allowed_off=moff)
    out = R.sample_tokens(view, params, hd, hist_len, logprobs=top_n, **kw)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in out.items()}
    if masks is not None:
        o = O.sample_tokens_masked(xs, params, masks, hist, hist_len)
    else:
        o = O.sample_tokens(xs, params, hist, hist_len)
    compare_sample(g, o, f"random renorm {seed}")
    compare_fused_logprobs(g, o, xs, top_n, f"random renorm {seed} logprobs")
    compare_renormalised(g, o, xs, top_n, lists, f"random renorm {seed} renormalised")


@pytest.mark.parametrize("seed", range(12))
def test_random_verify_windows(seed):
    """Verify windows on seeded random inputs: random window sizes and
    penalties, drafts that match a random number of leading rows; the
    accepted counts equal the oracle's for its own tokens."""
    rng = np.random.default_rng(11000 + seed)
    window = int(rng.choice([1, 2, 3, 5, 8]))
    B = window * int(rng.integers(1, 70 // window + 1))
    V = int(rng.choice([1000, 30011, 120000]))
    x, kind = _logits(rng, B, V)
    hist = rng.integers(-2, V + 2, (1, 100)).astype(np.int32)
    params = _params(rng, B, 1, V)
    o = O.sample_tokens(x, params, hist, [100])
    drafts = np.array(o["token"], np.int32)
    for w in range(B // window):
        keep = int(rng.integers(0, window + 1))
        for j in range(keep, window):
            drafts[w * window + j] = (drafts[w * window + j] + 1) % V
    say("case random windows", seed, dict(B=B, V=V, window=window, kind=kind))
    out = R.sample_tokens(to_dev(x), params, to_dev(hist), [100], window=window,
                          draft=to_dev(drafts))
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in out.items()}
    compare_sample(g, o, f"random windows {seed}")
    exp = O.accept_windows(o["token"], window, drafts)
    for w in range(B // window):
        rows = slice(w * window, (w + 1) * window)
        if np.array_equal(g["token"][rows], o["token"][rows]):
            assert g["accepted"][w] == exp[w], (seed, w)
