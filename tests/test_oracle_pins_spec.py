"""Pins of the oracle's masked sampling (reading R11) and verify-window
acceptance (reading R12).

Masked sampling is pinned to the oracle's unrestricted chain on the sub-row
of allowed ids (ids mapped back through the sorted allowed set, history ids
outside it made foreign), which the other pin files tie to numpy, scipy and
rocRAND; acceptance to hand-worked windows.  Pages, cited by title/section:
  #19  "serve: per-request temperature/top_p/top_k/min_p/penalties sampling",
       "What changed" (emitted tokens are the target's own samples)
  #559 "Several conversations at once: batch slots, ...", "Not done (yet)"
       (a sampled row is accepted when its pick equals the draft)
  #3200 "OpenAI logprobs / top_logprobs / allowed_token_ids ...", "Problem and
       result" (allowed_token_ids names exactly the ids of the distribution)
"""
import numpy as np
import pytest

from request_token_sampling_amd import workloads as W


def sampled(**kw):
    d = dict(temperature=0.9, top_k=20, top_p=0.9, min_p=0.02, seed=5, counter=11)
    d.update(kw)
    return W.row_params(**d)


def sub_row(O, x, p, hist, D):
    """The unrestricted chain on x[D], its ids mapped back through D."""
    D = np.asarray(D, np.int64)
    pos = -np.ones(x.size + 1, np.int64)
    pos[D] = np.arange(D.size)
    h = None
    if hist is not None:
        hh = np.asarray(hist, np.int64)
        h = np.where((hh >= 0) & (hh < x.size), pos[np.clip(hh, 0, x.size)], -1)
        h = h.astype(np.int32)
    o = O.sample_row(x[D], p, h)
    ids = o["kept_ids"].copy()
    ids[ids >= 0] = D[ids[ids >= 0]]
    return dict(o, kept_ids=ids, token=int(D[o["token"]]) if o["token"] >= 0 else -1)


CASES = [
    ("sampled", sampled()),
    ("k above domain", sampled(top_k=64)),
    ("greedy", W.row_params()),
    ("penalties", sampled(penalty_repeat=1.4, penalty_freq=0.3, penalty_present=0.2,
                          penalty_last_n=-1, history_row=0)),
    ("min_p", sampled(min_p=0.5, top_p=1.0)),
]


@pytest.mark.parametrize("name,p", CASES)
@pytest.mark.parametrize("size", [1, 7, 40, 1500])
def test_masked_equals_chain_on_the_allowed_subrow(oracle_mod, name, p, size):
    O = oracle_mod
    rng = np.random.default_rng(size)
    V = 4000
    x = W.bf16_grid(rng.normal(0, 3, V).astype(np.float32))   # ties across ids
    D = np.sort(rng.choice(V, size, replace=False))
    hist = np.concatenate([D[: min(size, 30)], rng.integers(0, V, 50)]).astype(np.int32)
    h = hist if p.get("history_row", -1) >= 0 else None
    # duplicates and foreign ids in the list do not change the domain
    lst = np.concatenate([D, D[: size // 2], [-3, V, V + 17]]).astype(np.int32)
    rng.shuffle(lst)
    m = O.sample_row(x, p, h, allowed=lst)
    ref = sub_row(O, x, p, h, D)
    for k in ("token", "x0", "flags"):
        assert m[k] == ref[k], (name, k, m[k], ref[k])
    for k in ("counts", "kept_ids", "kept_logits"):
        assert np.array_equal(m[k], ref[k]), (name, k, m[k], ref[k])
    assert set(m["kept_ids"][m["kept_ids"] >= 0]) <= set(D.tolist())
    assert m["counts"][0] == min(1 if name == "greedy" else p["top_k"], size)


def test_empty_list_means_unrestricted(oracle_mod):
    O = oracle_mod
    x = np.random.default_rng(1).normal(0, 3, 3000).astype(np.float32)
    p = sampled()
    a, b = O.sample_row(x, p), O.sample_row(x, p, allowed=np.zeros(0, np.int32))
    for k in ("token", "x0"):
        assert a[k] == b[k]
    assert np.array_equal(a["kept_ids"], b["kept_ids"])


@pytest.mark.parametrize("p", [sampled(), W.row_params()])
def test_no_allowed_id_in_range_samples_nothing(oracle_mod, p):
    O = oracle_mod
    x = np.random.default_rng(2).normal(0, 3, 500).astype(np.float32)
    m = O.sample_row(x, p, allowed=np.array([-1, 500, 9999], np.int32))
    assert m["token"] == -1
    assert list(m["counts"]) == [0, 0, 0]
    assert np.all(m["kept_ids"] == -1)
    # the draw word is still the row's (seed, counter) word
    assert m["x0"] == O.sample_row(x, p)["x0"]


def test_masked_greedy_is_argmax_over_the_list(oracle_mod):
    O = oracle_mod
    rng = np.random.default_rng(3)
    x = rng.integers(-5, 5, 2000).astype(np.float32)           # many ties
    D = rng.choice(2000, 300, replace=False)
    m = O.sample_row(x, W.row_params(), allowed=D)
    best = D[np.argmax(x[D])]
    first = np.min(D[x[D] == x[best]])                          # ties: lowest id
    assert m["token"] == first


# ---------------------------------------------------------------- acceptance
@pytest.mark.parametrize("tokens,drafts,window,expected", [
    ([5, 6, 7, 8, 9], [5, 6, 7, 8, 0], 5, [5]),      # every draft matched: all 5 emitted
    ([5, 6, 7, 8, 9], [4, 6, 7, 8, 9], 5, [1]),      # first draft rejected: the head only
    ([5, 6, 7, 8, 9], [5, 6, 0, 8, 9], 5, [3]),      # later matches do not count
    ([5, 6, 7, 8, 9], [5, 6, 7, 8, 9], 5, [5]),      # the last row's draft is never read
    ([1, 2, 3, 4], [1, 9, 0, 4], 2, [2, 1]),         # two windows of two rows
    ([7, 7, 7], [7, 7, 7], 1, [1, 1, 1]),            # no drafts: one token per row
])
def test_accepted_prefix_by_hand(oracle_mod, tokens, drafts, window, expected):
    assert list(oracle_mod.accept_windows(tokens, window, drafts)) == expected


def test_acceptance_refuses_ragged_windows(oracle_mod):
    with pytest.raises(ValueError):
        oracle_mod.accept_windows([1, 2, 3], 2, [1, 2, 3])
