"""GPU parity of logprobs renormalised over allowed lists inside a sampling
call (rts_logprob_request.allowed): the sampled tokens and kept sequences to
the sampling bar, the unrestricted and the renormalised logprobs to the
logprob bar (tests/parity.py), against the CPU oracle.

Lists of up to 2,048 ids on rows without a candidate mask are renormalised by
extra workgroups of the sampling launch, which meet each row's merging
workgroup through one exchange on a per-row word; longer lists, and rows that
also carry a mask, take the allowed-id logprob kernels after the launch.
Cases cover both, repeated and out-of-range ids, empty lists, tokens outside
the list, lists whose members are all -inf, several launches, broadcast rows
(ld = 0) and graph replays."""
import numpy as np
import pytest
import torch

import oracle.oracle as O
import request_token_sampling_amd as R
from request_token_sampling_amd import workloads as W

from parity import compare_fused_logprobs, compare_renormalised, compare_sample, say, to_dev

pytestmark = pytest.mark.gpu

V = W.V_FULL


def sampled(**kw):
    d = dict(temperature=1.0, top_k=64, top_p=1.0, min_p=0.0, seed=13, counter=0)
    d.update(kw)
    return W.row_params(**d)


def dev_lists(lists):
    ids, off = W.pack_allowed(lists)
    d = to_dev(ids) if ids.size else torch.zeros(1, dtype=torch.int32, device="cuda")
    return d, off


def gpu_call(xd, params, top_n, lists, mask_lists=None, **kw):
    ids, off = dev_lists(lists)
    if mask_lists is not None:
        mids, moff = dev_lists(mask_lists)
        kw.update(allowed=mids, allowed_off=moff)
    out = R.sample_tokens(xd, params, logprobs=top_n, logprob_allowed=ids,
                          logprob_allowed_off=off, **kw)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def check(x, params, top_n, lists, tag, mask_lists=None, xd=None, history=None, hist_len=None,
          **kw):
    say("case renorm", tag, np.asarray(x).shape, "top_n", top_n)
    xd = to_dev(np.asarray(x, np.float32)) if xd is None else xd
    if history is not None:
        kw.update(history=to_dev(np.asarray(history, np.int32)), history_len=hist_len)
    g = gpu_call(xd, params, top_n, lists, mask_lists, **kw)
    if mask_lists is None:
        o = O.sample_tokens(np.asarray(x, np.float32), params, history, hist_len)
    else:
        o = O.sample_tokens_masked(np.asarray(x, np.float32), params, mask_lists, history,
                                   hist_len)
    compare_sample(g, o, tag)
    compare_fused_logprobs(g, o, x, top_n, tag + " unrestricted")
    compare_renormalised(g, o, x, top_n, lists, tag + " renormalised")
    return g, o


def mixed_lists(rng, Vx, B, token_hint=None):
    """Cycling kinds: random distinct ids, repeats with foreign ids, a list
    without the row's argmax, one id, empty (unrestricted), 2,048 ids with
    repeats."""
    out = []
    for r in range(B):
        c = r % 6
        if c == 0:
            out.append(rng.choice(Vx, min(1000, Vx), replace=False).astype(np.int32))
        elif c == 1:
            a = rng.integers(0, Vx, 300).astype(np.int32)
            out.append(np.concatenate([a, a[:50], [-1, Vx, Vx + 77, -9]]).astype(np.int32))
        elif c == 2:
            a = rng.choice(Vx, min(500, Vx), replace=False).astype(np.int32)
            if token_hint is not None:
                a = a[a != token_hint[r]]
            out.append(a)
        elif c == 3:
            out.append(np.array([int(rng.integers(0, Vx))], np.int32))
        elif c == 4:
            out.append(np.zeros(0, np.int32))
        else:
            out.append(rng.integers(0, Vx, 2048).astype(np.int32))
    return out


def test_stress_lists_in_the_sampling_launch():
    w = W.logprobs_stress()
    check(w["logits"], w["params"], w["top_n"], w["allowed"], "stress renorm")


@pytest.mark.parametrize("top_n", [20, 3, 0])
def test_mixed_lists(top_n):
    rng = np.random.default_rng(31 + top_n)
    B = 12
    x = rng.normal(0, 3, (B, V)).astype(np.float32)
    params = [sampled(top_k=int(k), counter=r, top_p=0.9, min_p=0.01)
              for r, k in enumerate(rng.integers(1, 65, B))]
    lists = mixed_lists(rng, V, B, token_hint=np.argmax(x, axis=1))
    check(x, params, top_n, lists, f"mixed top_n={top_n}")


def test_list_holding_the_sampled_token_only_and_uniform_members():
    """A greedy row whose list is its argmax alone (logprob 0); a row whose
    members are all -inf (each gets -log n); a list of ids outside [0, V)
    only (no member: -inf everywhere)."""
    rng = np.random.default_rng(33)
    x = rng.normal(0, 3, (3, V)).astype(np.float32)
    x[1, 1000:1100] = -np.inf
    params = [W.row_params(), sampled(top_k=5), sampled(top_k=5)]
    lists = [np.array([int(np.argmax(x[0]))], np.int32),
             np.arange(1000, 1100, dtype=np.int32),
             np.array([-3, V, V + 5], np.int32)]
    g, _ = check(x, params, 20, lists, "degenerate lists")
    assert g["allowed_token_lp"][0] == 0.0
    assert np.all(g["allowed_top_ids"][2] == -1) and g["allowed_token_lp"][2] == -np.inf


@pytest.mark.parametrize("n", [2048, 2049])
def test_longest_fused_list_and_the_first_longer_one(n):
    """2,048 ids are renormalised in the sampling launch; 2,049 take the
    allowed-id logprob kernels after it: both to the same bar."""
    rng = np.random.default_rng(n)
    x = rng.normal(0, 3, (4, V)).astype(np.float32)
    params = [sampled(top_k=20, counter=r) for r in range(4)]
    lists = [rng.choice(V, n, replace=False).astype(np.int32) for _ in range(4)]
    lists[2] = np.zeros(0, np.int32)
    check(x, params, 20, lists, f"list of {n}")


def test_vocabulary_past_the_standalone_limit():
    """Lists renormalised inside the sampling call need no vocabulary bitmap,
    so V may exceed 2^19 (the limit of the bitmap kernels that longer lists
    take)."""
    rng = np.random.default_rng(41)
    Vx = 1_100_003
    x = rng.normal(0, 3, (2, Vx)).astype(np.float32)
    params = [sampled(top_k=20, counter=0), W.row_params()]
    lists = [rng.choice(Vx, 1500, replace=False).astype(np.int32),
             np.concatenate([[int(np.argmax(x[1]))], rng.integers(0, Vx, 600)]).astype(np.int32)]
    check(x, params, 20, lists, "V past 2^19")


def test_penalised_rows():
    """Penalties force the second (raw) selection, merged in the same tail
    that meets the renormalising workgroup."""
    w = W.batch_slots()
    rng = np.random.default_rng(39)
    lists = mixed_lists(rng, V, len(w["params"]))
    check(w["logits"], w["params"], 20, lists, "penalised renorm", history=w["history"],
          hist_len=w["hist_len"])


def test_verify_windows():
    """Windows of five rows with drafts: acceptance and renormalised logprobs
    from one launch."""
    rng = np.random.default_rng(40)
    B, window = 10, 5
    x = rng.normal(0, 3, (B, V)).astype(np.float32)
    params = [sampled(top_k=40, top_p=0.95, counter=r) for r in range(B)]
    o = O.sample_tokens(x, params)
    drafts = o["token"].astype(np.int32).copy()
    drafts[2] = (drafts[2] + 1) % V          # window 0 accepts two rows
    lists = mixed_lists(rng, V, B)
    g, o2 = check(x, params, 20, lists, "windows renorm", window=window, draft=to_dev(drafts))
    want = O.accept_windows(o2["token"], window, drafts)
    for w in range(B // window):
        rows = slice(w * window, (w + 1) * window)
        if np.array_equal(g["token"][rows], o2["token"][rows]):
            assert g["accepted"][w] == want[w], (w, g["accepted"][w], want[w])


def test_masked_rows_take_the_separate_pass():
    rng = np.random.default_rng(35)
    x = rng.normal(0, 3, (4, V)).astype(np.float32)
    params = [sampled(top_k=30, counter=r) for r in range(4)]
    masks = [np.arange(0, V, 3, dtype=np.int32), None, None, rng.integers(0, V, 400).astype(np.int32)]
    lists = [rng.choice(V, 700, replace=False).astype(np.int32) for _ in range(4)]
    lists[0] = np.concatenate([lists[0], masks[0][:50]]).astype(np.int32)
    check(x, params, 20, lists, "masked + renorm", mask_lists=masks)


def test_masked_rows_past_the_bitmap_limit():
    """Rows with a candidate mask renormalise their lists after the launch; at
    V = 1,100,003 (past 2^19, where no vocabulary bitmap fits in LDS) that pass
    takes the hash-set kernel, which handles 64 rows a launch: 66 restricted
    rows make two launches.  Lists of up to 2,048 ids with repeats and foreign
    ids, a list whose members are all -inf, an empty list, and top_n 20 and 0."""
    rng = np.random.default_rng(43)
    Vx, B = 1_100_003, 66
    x = rng.normal(0, 3, (B, Vx)).astype(np.float32)
    params = [W.row_params() if r % 11 == 0 else
              sampled(top_k=int(rng.integers(1, 65)), counter=r, top_p=0.9)
              for r in range(B)]
    masks, lists = [], []
    for r in range(B):
        m = rng.choice(Vx, 3000, replace=False).astype(np.int32)
        masks.append(m)
        c = r % 4
        if c == 0:    # members from the mask and outside it, repeats, foreign ids
            a = np.concatenate([m[:700], rng.integers(0, Vx, 600), m[:40], [-1, Vx, Vx + 9]])
        elif c == 1:  # the longest list renormalised in one pass
            a = rng.integers(0, Vx, 2048)
        elif c == 2:
            a = rng.choice(Vx, 900, replace=False)
        else:
            a = np.zeros(0, np.int64) if r % 8 == 3 else m[::3]
        lists.append(np.asarray(a, np.int32))
    # row 5: every member of its list is -inf (each gets -log of the member count)
    lists[5] = rng.choice(Vx, 400, replace=False).astype(np.int32)
    x[5, lists[5]] = -np.inf
    check(x, params, 20, lists, "masked renorm V past 2^19", mask_lists=masks)
    check(x[:4], params[:4], 0, lists[:4], "masked renorm V past 2^19, top_n 0",
          mask_lists=masks[:4])


def test_small_rows_many_launches():
    """70 rows of 1,024 ids (two launches, one chunk per row): the sampling
    side often finishes before the renormalising workgroup."""
    rng = np.random.default_rng(36)
    B, Vx = 70, 1024
    x = rng.normal(0, 2, (B, Vx)).astype(np.float32)
    params = [W.row_params() if r % 5 == 0 else sampled(top_k=int(rng.integers(1, 65)), counter=r)
              for r in range(B)]
    lists = mixed_lists(rng, Vx, B)
    check(x, params, 7, lists, "70 small rows")


def test_broadcast_rows():
    """Several parameter rows over one logits row (ld = 0), each with its own list."""
    rng = np.random.default_rng(37)
    x1 = rng.normal(0, 3, (1, V)).astype(np.float32)
    params = [sampled(top_k=20, counter=r, seed=r) for r in range(3)] + [W.row_params()]
    lists = [rng.choice(V, 900, replace=False).astype(np.int32) for _ in range(4)]
    lists[3] = np.concatenate([lists[3], [int(np.argmax(x1[0]))]]).astype(np.int32)
    xd = to_dev(x1).expand(4, -1)
    check(np.repeat(x1, 4, axis=0), params, 20, lists, "broadcast renorm", xd=xd)


def test_fused_equals_the_separate_call_bitwise():
    """The launch's renormalised values equal rts_token_logprobs' for the same
    lists and the sampled tokens, bit for bit (same member set, same exact
    fixed-point sum, same ranking)."""
    w = W.logprobs_stress()
    xd = to_dev(w["logits"])
    ids, off = dev_lists(w["allowed"])
    g = R.sample_tokens(xd, w["params"], logprobs=20, logprob_allowed=ids, logprob_allowed_off=off)
    sep = R.token_logprobs(xd, g["token"], 20, ids, off)
    torch.cuda.synchronize()
    for a, b in (("allowed_token_lp", "token_lp"), ("allowed_top_ids", "top_ids"),
                 ("allowed_top_lp", "top_lp")):
        assert np.array_equal(g[a].cpu().numpy(), sep[b].cpu().numpy()), a


def test_graph_replays():
    """One captured call replayed three times with eager work between: the
    per-row exchange words return to zero after every launch."""
    rng = np.random.default_rng(38)
    B, top_n = 24, 20
    x = rng.normal(0, 3, (B, V)).astype(np.float32)
    params = [sampled(top_k=int(rng.integers(1, 65)), counter=r, top_p=0.95) for r in range(B)]
    lists = mixed_lists(rng, V, B)
    ids, off = dev_lists(lists)
    xd = to_dev(x)
    c0 = np.array([p["counter"] for p in params], np.int64)
    ctr = to_dev(c0)
    call = R.SampleCall(xd, params, counters=ctr, counter_stride=1, logprobs=top_n,
                        logprob_allowed=ids, logprob_allowed_off=off)
    call()
    torch.cuda.synchronize()
    ctr.copy_(to_dev(c0))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        say("case renorm graph replay", rep)
        graph.replay()
        torch.cuda.synchronize()
        g = {k: v.cpu().numpy().copy() for k, v in call.results().items()}
        want = [dict(p, counter=int(c0[r]) + rep) for r, p in enumerate(params)]
        o = O.sample_tokens(x, want)
        compare_sample(g, o, f"renorm replay {rep}")
        compare_renormalised(g, o, x, top_n, lists, f"renorm replay {rep}")
        float((xd * 2.0).sum().item())
        torch.cuda.synchronize()
    assert np.array_equal(ctr.cpu().numpy(), c0 + 3)
