"""GPU parity of the sampler's verify-window acceptance (reading R12) and of
sampling restricted to allowed ids (reading R11), through the C ABI, against
the CPU oracle; the bar is stated in tests/parity.py."""
import numpy as np
import pytest
import torch

import oracle.oracle as O
import request_token_sampling_amd as R
from request_token_sampling_amd import workloads as W

from parity import compare_fused_logprobs, compare_sample, say, to_dev

pytestmark = pytest.mark.gpu

V = W.V_FULL


def sampled(**kw):
    d = dict(temperature=1.0, top_k=40, top_p=0.95, min_p=0.02, seed=9, counter=0)
    d.update(kw)
    return W.row_params(**d)


def gpu_masked(x, params, lists, history=None, hist_len=None, logprobs=None, **kw):
    ids, off = W.pack_allowed(lists)
    dev_ids = to_dev(ids) if ids.size else torch.zeros(1, dtype=torch.int32, device="cuda")
    h = None if history is None else to_dev(np.asarray(history, np.int32))
    out = R.sample_tokens(to_dev(np.asarray(x, np.float32)), params, h, hist_len,
                          allowed=dev_ids, allowed_off=off, logprobs=logprobs, **kw)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def masked_lists(rng, Vx, B):
    """One row per kind of list, cycling: short, fewer ids than top_k, long,
    duplicates with foreign ids, nothing in range, empty (unrestricted)."""
    kinds = []
    for r in range(B):
        c = r % 6
        if c == 0:
            kinds.append(rng.choice(Vx, 8, replace=False).astype(np.int32))
        elif c == 1:
            kinds.append(rng.choice(Vx, 5, replace=False).astype(np.int32))
        elif c == 2:
            kinds.append(rng.choice(Vx, min(1000, Vx), replace=False).astype(np.int32))
        elif c == 3:
            a = rng.choice(Vx, 30, replace=False)
            kinds.append(np.concatenate([a, a[:10], [-5, Vx, Vx + 3]]).astype(np.int32))
        elif c == 4:
            kinds.append(np.array([-1, Vx, 2 ** 31 - 1], np.int32))
        else:
            kinds.append(np.zeros(0, np.int32))
    return kinds


@pytest.mark.parametrize("Vx", [V, 1025, 70001])
def test_masked_rows_full_and_ragged(Vx):
    rng = np.random.default_rng(Vx)
    B = 12
    x = W.bf16_grid(rng.normal(0, 3, (B, Vx)).astype(np.float32))
    x[3, :50] = np.nan
    x[9, 7] = np.inf
    lists = masked_lists(rng, Vx, B)
    lists[3] = np.concatenate([np.arange(50, dtype=np.int32), lists[3]])   # NaN members
    params = [sampled(counter=r, top_k=[20, 40, 64, 8][r % 4]) for r in range(B)]
    params[6] = W.row_params()                      # a greedy masked row
    say("case masked V", Vx)
    g = gpu_masked(x, params, lists)
    o = O.sample_tokens_masked(x, params, lists)
    compare_sample(g, o, f"masked V={Vx}")
    assert g["token"][4] == -1 and g["token"][10] == -1          # nothing in range
    assert int(g["counts"][1, 0]) == 5                           # fewer ids than top_k


def test_masked_rows_with_penalties_and_fused_logprobs():
    rng = np.random.default_rng(31)
    B = 12
    x = rng.normal(0, 3, (B, V)).astype(np.float32)
    hist = rng.integers(0, 3000, (2, 200)).astype(np.int32)
    lists = masked_lists(rng, 3000, B)              # ids below 3000 meet the history
    x = W.boost_history(x, hist.ravel(), 8.0)
    params = [sampled(counter=r, penalty_repeat=1.3, penalty_freq=0.2, penalty_present=0.3,
                      penalty_last_n=-1, history_row=r % 2) for r in range(B)]
    say("case masked penalties + logprobs")
    g = gpu_masked(x, params, lists, hist, [200, 200], logprobs=20)
    o = O.sample_tokens_masked(x, params, lists, hist, [200, 200])
    compare_sample(g, o, "masked penalties")
    # the reported logprobs stay those of the unrestricted raw logits
    compare_fused_logprobs(g, o, x, 20, "masked lp")


def windows_case(B, window, seed):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 3, (B, V)).astype(np.float32)
    params = [sampled(counter=5 * (r // window) + r % window) for r in range(B)]
    o = O.sample_tokens(x, params)
    # drafts: each window accepts a chosen number of rows, then one mismatch
    drafts = np.empty(B, np.int32)
    for w in range(B // window):
        want = int(rng.integers(0, window))
        for j in range(window):
            r = w * window + j
            t = int(o["token"][r])
            drafts[r] = t if j < want else (t + 1) % V
    return x, params, o, drafts


@pytest.mark.parametrize("B,window", [(5, 5), (75, 5), (12, 1), (64, 64), (30, 3), (66, 33),
                                      (68, 34)])
def test_verify_window_acceptance(B, window):
    x, params, o, drafts = windows_case(B, window, B * 100 + window)
    say("case windows", B, window)
    out = R.sample_tokens(to_dev(x), params, window=window, draft=to_dev(drafts))
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in out.items()}
    compare_sample(g, o, f"windows B={B} w={window}")
    expected = O.accept_windows(o["token"], window, drafts)
    for w in range(B // window):
        rows = slice(w * window, (w + 1) * window)
        if np.array_equal(g["token"][rows], o["token"][rows]):
            assert int(g["accepted"][w]) == int(expected[w]), (w, g["accepted"][w], expected[w])
        else:                                       # a flagged row drew another kept id
            assert 1 <= int(g["accepted"][w]) <= window
    if window > 1 and B // window > 1:
        assert len(set(expected.tolist())) > 1                  # the drafts vary the outcome


def test_windows_with_masks_and_device_counters_repeat():
    """Windows, masks and device counters together, called twice on one
    workspace: window tickets return to zero between calls."""
    B, window = 10, 5
    x, params, o, drafts = windows_case(B, window, 77)
    lists = [None] * B
    lists[2] = np.arange(0, V, 7, dtype=np.int32)
    ids, off = W.pack_allowed(lists)
    xd, dd = to_dev(x), to_dev(drafts)
    ws = R.make_workspace(B, V)
    for rep in range(2):
        ctr = torch.tensor([p["counter"] for p in params], dtype=torch.int64, device="cuda")
        call = R.SampleCall(xd, params, workspace=ws, counters=ctr, counter_stride=1,
                            window=window, draft=dd, allowed=to_dev(ids), allowed_off=off)
        g = {k: v.cpu().numpy() for k, v in call().results().items()}
        om = O.sample_tokens_masked(x, params, lists)
        compare_sample(g, om, f"windows+mask rep {rep}")
        exp = O.accept_windows(om["token"], window, drafts)
        if np.array_equal(g["token"], om["token"]):
            assert np.array_equal(g["accepted"], exp)


def test_graph_replays_of_windows_masks_and_fused_logprobs():
    """One captured call with every feature at once -- two launches (70 rows
    in windows of 5), masks on two rows, fused logprobs, device counters --
    replayed three times with eager work between replays: each replay draws
    with the advanced counters and the self-resetting tickets (row, logprob
    and window) start from zero every time."""
    B, window, top_n = 70, 5, 20
    x, params, _, drafts = windows_case(B, window, 91)
    lists = [None] * B
    lists[3] = np.arange(0, V, 11, dtype=np.int32)
    lists[64] = np.array([5, 17, 17, 123456, V - 1, -4, V + 9], np.int32)
    ids, off = W.pack_allowed(lists)
    xd = to_dev(x)
    c0 = np.array([p["counter"] for p in params], np.int64)
    ctr = to_dev(c0)
    call = R.SampleCall(xd, params, counters=ctr, counter_stride=1, logprobs=top_n,
                        window=window, draft=to_dev(drafts), allowed=to_dev(ids), allowed_off=off)
    call()                                     # eager warm-up: loads the kernels
    torch.cuda.synchronize()
    ctr.copy_(to_dev(c0))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        say("case graph replay, all features", rep)
        graph.replay()
        torch.cuda.synchronize()
        g = {k: v.cpu().numpy().copy() for k, v in call.results().items()}
        want = [dict(p, counter=int(c0[r]) + rep) for r, p in enumerate(params)]
        om = O.sample_tokens_masked(x, want, lists)
        compare_sample(g, om, f"graph replay {rep}")
        compare_fused_logprobs(g, om, x, top_n, f"graph replay {rep} logprobs")
        exp = O.accept_windows(om["token"], window, drafts)
        for w in range(B // window):
            rows = slice(w * window, (w + 1) * window)
            if np.array_equal(g["token"][rows], om["token"][rows]):
                assert g["accepted"][w] == exp[w], (rep, w)
        float((xd * 2.0).sum().item())         # eager work between replays
        torch.cuda.synchronize()
    assert np.array_equal(ctr.cpu().numpy(), c0 + 3)
