"""GPU parity: the HIP library through its C ABI against the CPU oracle on the
same seeded inputs (five workloads at full size, plus ragged, degenerate and
adversarial cases).  The bar is stated in tests/parity.py."""
import numpy as np
import pytest
import torch

import oracle.oracle as O
import request_token_sampling_amd as R
from request_token_sampling_amd import workloads as W

from parity import (compare_logprobs, compare_sample, gpu_logprobs, gpu_sample, oracle_sample,
                     say, to_dev)

pytestmark = pytest.mark.gpu

V = W.V_FULL


def sampled(**kw):
    d = dict(temperature=1.0, top_k=64, top_p=1.0, min_p=0.0, seed=11, counter=0)
    d.update(kw)
    return W.row_params(**d)


def check(logits, params, history=None, hist_len=None, tag=""):
    say("case", tag, np.asarray(logits).shape)
    g = gpu_sample(logits, params, history, hist_len)
    o = oracle_sample(logits, params, history, hist_len)
    return compare_sample(g, o, tag), g, o


# ---------------------------------------------------------------- workloads
def test_tiny_sampled_and_greedy():
    w = W.tiny()
    check(w["logits"], w["sampled"], tag="tiny sampled")
    _, g, _ = check(w["logits"], w["greedy"], tag="tiny greedy")
    assert np.array_equal(g["token"], np.argmax(w["logits"], axis=1))


def test_single_stream_full_vocab():
    w = W.single_stream()
    check(w["logits"], w["sampled"], tag="single sampled")
    _, g, _ = check(w["logits"], w["greedy"], tag="single greedy")
    assert g["token"][0] == int(np.argmax(w["logits"][0]))


def test_verify_windows_counter_persists():
    vw = W.VerifyWindows()
    for w in range(vw.windows):
        x = vw.next_logits()
        p = vw.params(w)
        hist = vw.history.reshape(1, -1)
        _, g, o = check(x, p, hist, [hist.shape[1]], tag=f"window {w}")
        vw.feed_back(int(o["token"][0]))          # the oracle's head token


def test_verify_windows_with_visible_penalties():
    vw = W.VerifyWindows()
    hist = vw.history.reshape(1, -1)
    x = W.boost_history(vw.next_logits(), vw.history, 12.0)
    p = vw.params(0)
    _, g, o = check(x, p, hist, [64], tag="boosted window")
    off = oracle_sample(x, [dict(q, history_row=-1) for q in p])
    assert not np.array_equal(off["kept_ids"], o["kept_ids"]), "penalties must be visible"


def test_batch_slots():
    w = W.batch_slots()
    flagged, _, _ = check(w["logits"], w["params"], w["history"], w["hist_len"], tag="batch")
    say("flagged rows", flagged)


def test_logprobs_stress_sample_and_logprobs():
    w = W.logprobs_stress()
    x = w["logits"]
    _, g, o = check(x, w["params"], tag="stress sample")
    tokens = o["token"]
    xd = to_dev(x)
    gl = gpu_logprobs(x, tokens, w["top_n"], logits_dev=xd)
    ol = O.token_logprobs(x, tokens, w["top_n"])
    compare_logprobs(gl, ol, "stress lp")
    ga = gpu_logprobs(x, tokens, w["top_n"], w["allowed"], logits_dev=xd)
    oa = O.token_logprobs(x, tokens, w["top_n"], w["allowed"])
    compare_logprobs(ga, oa, "stress allowed lp")
    # most sampled tokens are outside a random 1,000-id list: -inf there
    assert np.sum(np.isinf(oa["token_lp"])) > 0


# ---------------------------------------------------------------- edge cases
@pytest.mark.parametrize("Vx", [1, 2, 3, 63, 64, 65, 1023, 1024, 1025, 4097, 8191, 8193,
                                20007, 65537])
def test_ragged_vocab(Vx):
    rng = np.random.default_rng(Vx)
    x = rng.normal(0, 3, (3, Vx)).astype(np.float32)
    params = [sampled(top_k=64, top_p=0.9, min_p=0.02, counter=1),
              sampled(top_k=7, temperature=0.5, seed=3),
              W.row_params()]
    check(x, params, tag=f"V={Vx}")


def test_padded_rows_and_unaligned_base():
    rng = np.random.default_rng(5)
    B, Vx, ld = 4, 10007, 10016
    buf = rng.normal(0, 3, B * ld + 1).astype(np.float32)
    for r in range(B):
        buf[r * ld + Vx:r * ld + ld] = 1e30          # padding must be ignored
    dev = to_dev(buf)
    params = [sampled(top_k=20, counter=r) for r in range(B)]
    for off in (0, 1):                               # 1: rows not 16-byte aligned
        view = dev[off:off + B * ld].view(B, ld)[:, :Vx]
        host = buf[off:off + B * ld].reshape(B, ld)[:, :Vx]
        say("case padded off", off)
        g = gpu_sample(None, params, logits_dev=view)
        compare_sample(g, oracle_sample(host, params), f"padded off={off}")


def test_special_values():
    rng = np.random.default_rng(6)
    x = rng.normal(0, 3, (4, 30000)).astype(np.float32)
    for r in range(4):
        pos = rng.choice(30000, 40, replace=False)
        x[r, pos[:10]] = np.nan
        x[r, pos[10:14]] = np.inf
        x[r, pos[14:18]] = np.float32(3.4028235e38)
        x[r, pos[18:30]] = -np.inf
        x[r, pos[30:35]] = 0.0
        x[r, pos[35:40]] = -0.0
    params = [sampled(top_k=16, counter=r) for r in range(4)]
    check(x, params, tag="special")


@pytest.mark.parametrize("Vx", [1030, 20000, V])
def test_nan_lanes_beside_flt_max(Vx):
    """Lanes whose values are all NaN (or past V) next to lanes holding
    FLT_MAX / +inf: NaN counts as -inf and never takes part in a maximum;
    greedy rows and sampled rows both."""
    rng = np.random.default_rng(Vx + 3)
    x = rng.normal(0, 3, (4, Vx)).astype(np.float32)
    x[0, :700] = np.nan
    x[0, 5] = np.inf
    x[0, 900 % Vx] = np.float32(3.4028235e38)
    x[1, ::2] = np.nan
    x[1, 1::97] = np.inf
    x[2] = np.nan
    x[2, -1] = -np.inf
    x[3] = -np.inf
    x[3, ::5] = np.nan
    params = [W.row_params(), sampled(top_k=3, counter=1), W.row_params(),
              sampled(top_k=64, counter=2)]
    check(x, params, tag=f"nan lanes V={Vx}")
    check(x, [sampled(top_k=1, counter=r) for r in range(4)], tag=f"nan lanes k=1 V={Vx}")


def test_all_equal_rows_force_fallbacks():
    """Every logit equal: each chunk's candidate buffer overflows (k rounds
    over registers) and so does the row merge (k rounds over the list)."""
    x = np.zeros((3, V), np.float32)
    x[1] = -np.inf
    x[2] = 1.0
    x[2, 123456] = 2.0
    params = [sampled(top_k=64, counter=1), sampled(top_k=5), W.row_params()]
    _, g, _ = check(x, params, tag="all equal")
    assert list(g["kept_ids"][0][:64]) == list(range(64))


@pytest.mark.parametrize("B,Vx", [(2, 600_000), (1, 2_200_000)])
def test_long_rows_many_chunks(B, Vx):
    """Rows of more than 64 chunks (the row merge reads the chunk lists as
    sorted streams) and of more than 256 (each merging thread owns several
    streams), with top_k on both sides of the bitonic-tree cut-over."""
    rng = np.random.default_rng(Vx)
    x = rng.normal(0, 3, (B, Vx)).astype(np.float32)
    x[:, rng.choice(Vx, 200, replace=False)] = np.float32(12.5)  # 200 tied ids above the rest
    for ks in ((64, 20), (50, 47)):
        params = [sampled(top_k=ks[r % 2], counter=r, top_p=0.95, min_p=0.01) for r in range(B)]
        check(x, params, tag=f"long rows V={Vx} k={ks}")


@pytest.mark.parametrize("B", [20, 21, 64])
def test_chunk_size_boundaries_full_vocab(B):
    """At V = 248,320 a launch of up to 20 rows takes 4,096-element chunks
    and from 21 rows 8,192 (the chunk is the smallest with at most 64 chunks
    per row whose grid fits one resident round); 64 rows of 8,192-element
    chunks make 1,984 workgroups, more than fit at once.  Penalised rows
    sharing history rows of different lengths, mixed top_k."""
    rng = np.random.default_rng(700 + B)
    H, ldh = 3, 256
    hist = rng.integers(0, V, (H, ldh)).astype(np.int32)
    hist_len = np.array([256, 100, 0], np.int32)
    # history ids lifted into the head, so the penalties decide kept sets
    x = W.boost_history(rng.normal(0, 3, (B, V)).astype(np.float32), hist[:2].ravel(), 9.0)
    params = []
    for r in range(B):
        kw = dict(top_k=int(rng.integers(1, 65)), counter=r, seed=r + 5, top_p=0.9, min_p=0.02,
                  temperature=float(np.float32(rng.uniform(0.3, 1.5))))
        if r % 3 != 2:
            kw.update(penalty_repeat=1.1, penalty_freq=0.5, penalty_present=0.5,
                      penalty_last_n=64 + 32 * (r % 4), history_row=r % H)
        params.append(sampled(**kw))
    check(x, params, hist, hist_len, tag=f"{B} rows at full V")


def test_integer_grid_ties_full_vocab():
    rng = np.random.default_rng(8)
    x = rng.integers(-20, 21, (6, V)).astype(np.float32)
    params = [sampled(top_k=k, counter=k, top_p=0.9) for k in (1, 2, 17, 33, 63, 64)]
    check(x, params, tag="integer ties")


def test_mixed_rows_many_launches():
    """B > 64 rows: several launches, greedy and sampled rows mixed, top_k
    larger than V on some rows."""
    rng = np.random.default_rng(9)
    B, Vx = 150, 3000
    x = rng.normal(0, 2, (B, Vx)).astype(np.float32)
    params = []
    for r in range(B):
        if r % 5 == 0:
            params.append(W.row_params())
        else:
            params.append(sampled(top_k=int(rng.integers(1, 65)),
                                  temperature=float(np.float32(rng.uniform(0.2, 2))),
                                  top_p=float(np.float32(rng.uniform(0.3, 1))),
                                  min_p=float(np.float32(rng.uniform(0, 0.3))),
                                  seed=r, counter=r * 7))
    check(x, params, tag="mixed 150")


def test_penalty_windows_and_foreign_ids():
    rng = np.random.default_rng(10)
    Vx = 50000
    H, ldh = 3, 300
    hist = rng.integers(0, 2000, (H, ldh)).astype(np.int32)
    hist[1, :20] = [-1, Vx, Vx + 5, 2**31 - 1] * 5            # ignored ids
    hist_len = np.array([300, 150, 0], np.int32)
    x = W.boost_history(rng.normal(0, 2, (6, Vx)).astype(np.float32), hist[:2].ravel(), 6.0)
    params = [
        sampled(top_k=40, penalty_repeat=1.3, penalty_freq=0.2, penalty_present=0.4,
                penalty_last_n=64, history_row=0),
        sampled(top_k=40, penalty_repeat=0.8, penalty_freq=-0.1, penalty_present=0.0,
                penalty_last_n=-1, history_row=0, counter=1),
        sampled(top_k=40, penalty_repeat=1.5, penalty_last_n=500, history_row=1, counter=2),
        sampled(top_k=40, penalty_repeat=1.5, penalty_last_n=8, history_row=2, counter=3),
        W.row_params(penalty_repeat=2.0, penalty_last_n=-1, history_row=0),   # greedy
        sampled(top_k=40, penalty_last_n=-1, history_row=0, counter=5),      # neutral
    ]
    check(x, params, hist, hist_len, tag="penalty windows")


def test_ignored_ids_are_counted():
    """The optional status word counts the device ids a call read and
    ignored: history ids outside [0, V) inside the windows of rows whose
    penalties apply, and allowed ids outside [0, V) of masked rows, once
    per occurrence and row; outputs equal the same call without it."""
    rng = np.random.default_rng(12)
    Vx = 50000
    hist = rng.integers(0, 2000, (2, 300)).astype(np.int32)
    hist[0, 250:262] = [-1, Vx, Vx + 5, 2**31 - 1, -7, Vx] * 2     # 12 bad ids, last 64 window
    hist[1, :20] = [-3, Vx] * 10                                    # 20 bad, outside an 8-id window
    hist_len = [300, 300]
    x = rng.normal(0, 2, (5, Vx)).astype(np.float32)
    params = [
        sampled(top_k=20, penalty_repeat=1.3, penalty_last_n=64, history_row=0),
        sampled(top_k=20, penalty_repeat=1.3, penalty_last_n=-1, history_row=1, counter=1),
        sampled(top_k=20, penalty_last_n=-1, history_row=0, counter=2),  # neutral: not read
        sampled(top_k=20, penalty_repeat=1.1, penalty_last_n=8, history_row=1, counter=3),
        sampled(top_k=20, counter=4),                                   # masked below
    ]
    lists = [None, None, None, None, np.array([5, -1, Vx, 17, Vx + 1, 40000], np.int32)]
    ids, off = W.pack_allowed(lists)
    # rows 0 and 1 read 12 and 20 bad history ids (row 3's window holds none);
    # row 4 reads 3 bad allowed ids
    expected = 12 + 20 + 3
    xd, hd, idd = to_dev(x), to_dev(hist), to_dev(ids)
    say("case ignored ids", expected)
    ign = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = R.sample_tokens(xd, params, hd, hist_len, allowed=idd, allowed_off=off, ignored=ign)
    ref = R.sample_tokens(xd, params, hd, hist_len, allowed=idd, allowed_off=off)
    torch.cuda.synchronize()
    assert int(ign.item()) == expected
    for k in out:
        assert torch.equal(out[k], ref[k]), k
    R.sample_tokens(xd, params, hd, hist_len, allowed=idd, allowed_off=off, ignored=ign)
    torch.cuda.synchronize()
    assert int(ign.item()) == 2 * expected        # the word accumulates over calls


def test_determinism_and_row_independence():
    w = W.batch_slots()
    x, p = w["logits"], w["params"]
    g1 = gpu_sample(x, p, w["history"], w["hist_len"])
    g2 = gpu_sample(x, p, w["history"], w["hist_len"])
    for k in g1:
        assert g1[k].tobytes() == g2[k].tobytes(), k
    # one row alone equals the same row inside the batch
    for r in (0, 17, 39):
        solo = gpu_sample(x[r:r + 1], [p[r]], w["history"], w["hist_len"])
        for k in g1:
            assert solo[k][0].tobytes() == g1[k][r].tobytes(), (r, k)


def test_logprob_edges():
    rng = np.random.default_rng(12)
    Vx = 40000
    x = rng.normal(0, 3, (6, Vx)).astype(np.float32)
    x[1] = -np.inf
    x[1, 7] = np.nan
    x[2, :100] = np.inf
    tokens = np.array([5, 3, 50, -4, Vx + 2, 39999], np.int32)
    for top_n in (0, 1, 20):
        say("case logprob edges top_n", top_n)
        compare_logprobs(gpu_logprobs(x, tokens, top_n), O.token_logprobs(x, tokens, top_n),
                         f"edges top_n={top_n}")
    lists = [np.array([5, 5, 5, 9, -1, Vx], np.int32), None, np.arange(0, Vx, 3, dtype=np.int32),
             np.array([Vx + 1], np.int32), np.zeros(0, np.int32),
             rng.choice(Vx, 3000, replace=True).astype(np.int32)]
    say("case logprob allowed edges")
    compare_logprobs(gpu_logprobs(x, tokens, 20, lists), O.token_logprobs(x, tokens, 20, lists),
                     "edges allowed")


def test_logprob_small_and_ragged():
    for Vx in (1, 5, 1023, 1025, 9001):
        rng = np.random.default_rng(Vx + 1)
        x = W.bf16_grid(rng.normal(0, 3, (3, Vx)).astype(np.float32))
        tokens = rng.integers(0, Vx, 3).astype(np.int32)
        say("case logprob V", Vx)
        compare_logprobs(gpu_logprobs(x, tokens, 20), O.token_logprobs(x, tokens, 20),
                         f"lp V={Vx}")


def test_workspace_reuse_across_calls():
    """Tickets return to zero: consecutive calls on one workspace agree."""
    w = W.tiny()
    xd = to_dev(w["logits"])
    ws = R.make_workspace(4, 1024)
    outs = []
    for _ in range(3):
        out = R.sample_tokens(xd, w["sampled"], workspace=ws)
        lp = R.token_logprobs(xd, out["token"], 5, workspace=ws)
        torch.cuda.synchronize()
        outs.append((out["token"].cpu().numpy().copy(), lp["token_lp"].cpu().numpy().copy()))
    for a, b in outs[1:]:
        assert np.array_equal(a, outs[0][0]) and np.array_equal(b, outs[0][1])
    assert int(ws[:512].view(torch.int32).abs().sum().item()) == 0


# ------------------------------------------------- device-resident counters
def test_device_counters_advance_per_call():
    """With device counters, call i draws with c0 + i*stride and the call
    leaves c0 + (i+1)*stride behind (the caller's counter, in HBM)."""
    w = W.tiny()
    x, params = w["logits"], w["sampled"]
    c0 = np.array([5, 9, 2**40 + 7, 0], np.int64)
    ctr = to_dev(c0)
    xd = to_dev(x)
    stride = 3
    for call in range(3):
        say("case device counters call", call)
        out = R.sample_tokens(xd, params, counters=ctr, counter_stride=stride)
        torch.cuda.synchronize()
        g = {k: v.cpu().numpy() for k, v in out.items()}
        want = [dict(p, counter=int(c0[r]) + call * stride) for r, p in enumerate(params)]
        compare_sample(g, oracle_sample(x, want), f"device counters call {call}")
    assert np.array_equal(ctr.cpu().numpy(), c0 + 3 * stride)


def test_graph_replay_draws_fresh_numbers():
    """A captured call replayed three times (eager work and a sync between
    replays) draws with the advancing device counters every time."""
    rng = np.random.default_rng(21)
    Vx = 50000
    x = rng.normal(0, 2, (3, Vx)).astype(np.float32)
    params = [sampled(top_k=40, top_p=0.9, temperature=1.3, seed=77),
              sampled(top_k=7, temperature=0.6, seed=78),
              W.row_params()]
    c0 = np.array([100, 200, 300], np.int64)
    xd = to_dev(x)
    ctr = to_dev(c0)
    call = R.SampleCall(xd, params, counters=ctr, counter_stride=1)
    call()                                     # eager warm-up: loads the kernel
    torch.cuda.synchronize()
    ctr.copy_(to_dev(c0))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    assert np.array_equal(ctr.cpu().numpy(), c0), "capture must not run the call"
    seen = set()
    for rep in range(3):
        say("case graph replay", rep)
        graph.replay()
        torch.cuda.synchronize()
        g = {k: v.cpu().numpy().copy() for k, v in call.results().items()}
        want = [dict(p, counter=int(c0[r]) + rep) for r, p in enumerate(params)]
        compare_sample(g, oracle_sample(x, want), f"graph replay {rep}")
        seen.add(int(g["philox_x0"].view(np.uint32)[0]))
        float((xd * 2.0).sum().item())         # eager work between replays
        torch.cuda.synchronize()
    assert len(seen) == 3, "every replay must draw a fresh number"
    assert np.array_equal(ctr.cpu().numpy(), c0 + 3)


@pytest.mark.parametrize("B,Vx", [(1, V), (40, V), (3, 10007)])
def test_read_rows_measuring_stick(B, Vx):
    """The streaming-read kernel bench.py times as the bandwidth floor reads
    every element once: its chunk maxima are the rows' maxima, exactly."""
    rng = np.random.default_rng(B + Vx)
    x = rng.normal(0, 3, (B, Vx)).astype(np.float32)
    say("case read rows", B, Vx)
    call = R.ReadCall(to_dev(x))()
    torch.cuda.synchronize()
    cm = call.chunk_max.cpu().numpy()
    nch = int(np.sum(~np.isnan(cm[0])))             # entries past the chunk count stay NaN
    assert nch >= 1
    assert np.array_equal(np.max(cm[:, :nch], axis=1), np.max(x, axis=1))


def test_allowed_logprobs_are_deterministic_with_duplicates():
    """Which thread owns a duplicated id depends on timing; the outputs must
    not: repeated calls agree bit for bit and with the oracle."""
    rng = np.random.default_rng(13)
    Vx = 50000
    x = rng.normal(0, 3, (8, Vx)).astype(np.float32)
    base = [rng.choice(Vx, 300, replace=False).astype(np.int32) for _ in range(8)]
    lists = [np.concatenate([b, b, b[:100], b[::-1]]) for b in base]      # 1,000 listed ids
    tokens = np.array([int(b[0]) for b in base], np.int32)
    say("case allowed determinism")
    first = gpu_logprobs(x, tokens, 20, lists)
    for _ in range(3):
        again = gpu_logprobs(x, tokens, 20, lists)
        for k in first:
            assert first[k].tobytes() == again[k].tobytes(), k
    compare_logprobs(first, O.token_logprobs(x, tokens, 20, lists), "allowed dup")


def test_allowed_logprobs_past_the_bitmap_vocabulary_limit():
    """Lists of up to 2,048 ids take the hash-set kernel, which needs no
    vocabulary bitmap: V = 1,100,003 here (longer lists need V <= 2^19)."""
    rng = np.random.default_rng(14)
    Vx = 1_100_003
    x = rng.normal(0, 3, (3, Vx)).astype(np.float32)
    lists = [rng.choice(Vx, 2048, replace=False).astype(np.int32),
             np.concatenate([[7, 7, -1, Vx], rng.integers(0, Vx, 500)]).astype(np.int32), None]
    tokens = np.array([int(lists[0][5]), 7, 123], np.int32)
    say("case allowed logprobs V past 2^19")
    compare_logprobs(gpu_logprobs(x, tokens, 20, lists), O.token_logprobs(x, tokens, 20, lists),
                     "allowed V past 2^19")


def _mixed_params(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for r in range(n):
        if r % 7 == 3:
            out.append(W.row_params())  # greedy
        else:
            out.append(sampled(temperature=float(rng.uniform(0.2, 1.5)),
                               top_k=int(rng.integers(1, 65)), top_p=float(rng.uniform(0.5, 1.0)),
                               min_p=float(rng.uniform(0.0, 0.2)), seed=int(rng.integers(1, 1 << 40)),
                               counter=r))
    return out


@pytest.mark.parametrize("case", ["pair", "five", "max_rows", "two_launches", "ragged_10007",
                                  "ragged_70001"])
def test_broadcast_rows_share_one_logits_row(case):
    """ld = 0: several parameter rows (a sampled and a greedy pass, several
    samples) over one logits row equal the same rows over copies of it.
    Covers the chunk-major placement on two XCDs (two rows) and on eight,
    chunk counts that do not divide evenly, and more rows than one launch."""
    w = W.single_stream()
    x1 = w["logits"]
    if case == "pair":
        params = w["sampled"] + w["greedy"]
    elif case == "five":
        params = w["sampled"] + w["greedy"] + [sampled(top_k=5, counter=c, seed=3) for c in range(3)]
    elif case == "max_rows":
        params = _mixed_params(64, 5)
    elif case == "two_launches":
        params = _mixed_params(70, 6)
    else:
        Vx = int(case.split("_")[1])
        x1 = np.random.default_rng(Vx).normal(0.0, 3.0, (1, Vx)).astype(np.float32)
        params = _mixed_params(3 if Vx < 20000 else 2, Vx)
    B = len(params)
    say("case broadcast rows", case, B, x1.shape[1])
    out = R.sample_tokens(to_dev(x1).expand(B, -1), params)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in out.items()}
    compare_sample(g, oracle_sample(np.repeat(x1, B, axis=0), params), "broadcast " + case)
