"""C-ABI boundary on the CPU: the library loads, exports every function that
include/*.h declares, and refuses bad arguments before touching the GPU.

Pointers passed here are fake non-NULL addresses: every call below fails in
host validation, which runs before anything is enqueued, so no HIP call is
made and nothing is dereferenced."""
import ctypes
import glob
import os
import re

import pytest

import request_token_sampling_amd as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(4096)
BIG_WS = 1 << 40


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w\s\*]*?\b(rts_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"rts_sample_tokens", "rts_token_logprobs", "rts_workspace_bytes",
            "rts_workspace_init", "rts_strerror", "rts_last_error"} <= names
    L = R.lib()
    for n in names:
        assert hasattr(L, n), n


def test_struct_layout_matches_header():
    text = open(os.path.join(ROOT, "include", "rts.h")).read()
    body = text[text.index("typedef struct rts_row_params"):text.index("} rts_row_params;")]
    fields = re.findall(r"^\s*(?:float|int32_t|uint64_t)\s+(\w+);", body, flags=re.M)
    assert fields == [f for f, _ in R.RowParams._fields_]
    assert ctypes.sizeof(R.RowParams) == 56
    body = text[text.index("typedef struct rts_logprob_request"):
                text.index("} rts_logprob_request;")]
    fields = re.findall(r"^\s*(?:const\s+)?(?:float|int32_t|int64_t)\s*\*?\s*(\w+);", body,
                        flags=re.M)
    assert fields == [f for f, _ in R.LogprobRequest._fields_]
    assert ctypes.sizeof(R.LogprobRequest) == 72
    body = text[text.index("typedef struct rts_sample_extras"):text.index("} rts_sample_extras;")]
    fields = re.findall(r"^\s*(?:const\s+)?(?:int32_t|int64_t|uint32_t)\s*\*?\s*(\w+);", body, flags=re.M)
    assert fields == [f for f, _ in R.SampleExtras._fields_]
    assert ctypes.sizeof(R.SampleExtras) == 48


def sample(params, B=None, V=1000, ld=None, logits=FAKE, token=FAKE, ws=FAKE, ws_bytes=BIG_WS,
           history=None, H=0, ldh=0, hist_len=None, lp=None, ex=None):
    L = R.lib()
    arr = R.row_params(params)
    B = len(params) if B is None else B
    hl = None
    if hist_len is not None:
        hl = (ctypes.c_int32 * len(hist_len))(*hist_len)
    return L.rts_sample_tokens(logits, B, V, V if ld is None else ld, arr, history, H, ldh, hl,
                               token, None, None, None, None, None, 0,
                               None if lp is None else ctypes.byref(lp),
                               None if ex is None else ctypes.byref(ex), ws, ws_bytes, None)


SAMPLED = dict(temperature=0.7, top_k=20, top_p=0.9, min_p=0.05, seed=1, counter=0)


def last_error():
    return R.lib().rts_last_error().decode()


@pytest.mark.parametrize("bad,field", [
    (dict(top_k=0), "top_k"),
    (dict(top_k=65), "top_k"),
    (dict(top_k=-3), "top_k"),
    (dict(temperature=float("nan")), "temperature"),
    (dict(temperature=float("inf")), "temperature"),
    (dict(top_p=0.0), "top_p"),
    (dict(top_p=1.5), "top_p"),
    (dict(top_p=float("nan")), "top_p"),
    (dict(min_p=-0.1), "min_p"),
    (dict(min_p=1.01), "min_p"),
    (dict(penalty_repeat=0.0), "penalty_repeat"),
    (dict(penalty_repeat=-1.0), "penalty_repeat"),
    (dict(penalty_repeat=float("inf")), "penalty_repeat"),
    (dict(penalty_freq=float("nan")), "penalty_freq"),
    (dict(penalty_present=float("inf")), "penalty_present"),
    (dict(penalty_last_n=-2), "penalty_last_n"),
    (dict(history_row=-2), "history_row"),
    (dict(history_row=0), "history"),
    (dict(reserved=1), "reserved"),
])
def test_bad_row_is_refused_and_named(bad, field):
    rows = [dict(SAMPLED) for _ in range(5)]
    rows[3].update(bad)
    assert sample(rows) == R.RTS_EINVAL
    msg = last_error()
    assert "row 3" in msg and field in msg, msg


def test_greedy_rows_ignore_top_k():
    # a greedy row with top_k = 0 is valid: the failure comes from a later row
    rows = [dict(temperature=0.0, top_k=0), dict(SAMPLED, top_k=0)]
    assert sample(rows) == R.RTS_EINVAL
    assert "row 1" in last_error()


def test_bad_shapes_and_pointers():
    rows = [dict(SAMPLED)]
    assert sample(rows, B=-1) == R.RTS_EINVAL
    assert sample(rows, V=0) == R.RTS_EINVAL
    assert sample(rows, V=2**31) == R.RTS_EINVAL
    assert sample(rows, V=2**30 + 1) == R.RTS_EINVAL and "2^30" in last_error()
    # the largest vocabulary passes the shape checks (and then needs a larger workspace)
    assert sample(rows, V=2**30, ld=2**30, ws_bytes=4096) == R.RTS_ENOSPC
    assert sample(rows, ld=999) == R.RTS_EINVAL and "ld" in last_error()
    assert sample(rows, ld=1) == R.RTS_EINVAL and "ld" in last_error()
    assert sample(rows, logits=None) == R.RTS_EINVAL and "logits" in last_error()
    assert sample(rows, token=None) == R.RTS_EINVAL and "token" in last_error()
    assert sample(rows, ws=None) == R.RTS_EINVAL


@pytest.mark.parametrize("req,word", [
    (dict(top_n=21), "top_n"),
    (dict(top_n=-1), "top_n"),
    (dict(reserved=2), "reserved"),
    (dict(token_lp=None), "token_lp"),
    (dict(top_ids=None), "top_ids"),
    (dict(top_lp=None), "top_lp"),
])
def test_bad_logprob_request_is_refused(req, word):
    full = dict(top_n=5, reserved=0, token_lp=4096, top_ids=4096, top_lp=4096)
    full.update(req)
    lp = R.LogprobRequest(**full)
    assert sample([dict(SAMPLED)], lp=lp) == R.RTS_EINVAL
    assert word in last_error(), last_error()


def test_logprob_request_without_top_entries_needs_no_top_buffers():
    # top_n = 0: NULL top buffers are fine; the call then fails later, on the
    # bad row, which shows the request itself passed validation.
    lp = R.LogprobRequest(top_n=0, reserved=0, token_lp=4096, top_ids=None, top_lp=None)
    assert sample([dict(SAMPLED, top_k=0)], lp=lp) == R.RTS_EINVAL
    assert "top_k" in last_error()


def lp_allowed_request(off, **kw):
    d = dict(top_n=5, reserved=0, token_lp=4096, top_ids=4096, top_lp=4096, allowed=4096,
             allowed_off=None if off is None else ctypes.cast(off, ctypes.c_void_p),
             allowed_token_lp=4096, allowed_top_ids=4096, allowed_top_lp=4096)
    d.update(kw)
    return R.LogprobRequest(**d)


def test_bad_renormalising_logprob_request_is_refused():
    rows = [dict(SAMPLED) for _ in range(4)]
    off_ok = (ctypes.c_int64 * 5)(0, 3, 3, 10, 12)
    off_down = (ctypes.c_int64 * 5)(0, 3, 2, 10, 12)
    off_neg = (ctypes.c_int64 * 5)(-1, 3, 3, 10, 12)
    cases = [
        (lp_allowed_request(None), "allowed_off"),
        (lp_allowed_request(off_ok, allowed_token_lp=None), "allowed_token_lp"),
        (lp_allowed_request(off_ok, allowed_top_ids=None), "allowed_top_ids"),
        (lp_allowed_request(off_ok, allowed_top_lp=None), "allowed_top_lp"),
        (lp_allowed_request(off_down), "decreases"),
        (lp_allowed_request(off_neg), "[0]"),
        (lp_allowed_request(off_ok, allowed=None), "without lp->allowed"),
    ]
    for lp, word in cases:
        assert sample(rows, lp=lp) == R.RTS_EINVAL, word
        assert word in last_error(), (word, last_error())
    # top_n = 0 needs no top buffers; the bad row then names itself
    lp = lp_allowed_request(off_ok, top_n=0, top_ids=None, top_lp=None, allowed_top_ids=None,
                            allowed_top_lp=None)
    assert sample(rows[:3] + [dict(SAMPLED, top_k=0)], lp=lp) == R.RTS_EINVAL
    assert "row 3" in last_error(), last_error()


def test_long_renormalising_lists_need_small_vocabularies():
    """Lists longer than 2,048 ids take the bitmap kernels, whose vocabulary
    bitmap needs V <= 2^19: refused before anything is enqueued.  Shorter
    lists have no such limit, in the sampling launch or after it (rows that
    also carry a mask): they pass validation and the call fails on the bad
    row."""
    V = 2 ** 20
    rows = [dict(SAMPLED), dict(SAMPLED, top_k=0)]
    long_off = (ctypes.c_int64 * 3)(0, 2049, 2049)
    short_off = (ctypes.c_int64 * 3)(0, 2048, 2048)
    assert sample(rows, V=V, lp=lp_allowed_request(long_off)) == R.RTS_EINVAL
    assert "2^19" in last_error(), last_error()
    assert sample(rows, V=V, lp=lp_allowed_request(short_off)) == R.RTS_EINVAL
    assert "row 1" in last_error(), last_error()
    mask_off = (ctypes.c_int64 * 3)(0, 1, 1)
    ex = extras(allowed=4096, allowed_off=ctypes.cast(mask_off, ctypes.c_void_p))
    assert sample(rows, V=V, lp=lp_allowed_request(short_off), ex=ex) == R.RTS_EINVAL
    assert "row 1" in last_error(), last_error()
    assert sample(rows, V=V, lp=lp_allowed_request(long_off), ex=ex) == R.RTS_EINVAL
    assert "2^19" in last_error(), last_error()


def test_standalone_long_lists_need_small_vocabularies():
    V = 2 ** 20
    off = (ctypes.c_int64 * 2)(0, 2049)
    rc = R.lib().rts_token_logprobs(FAKE, 1, V, V, FAKE, 5, FAKE, ctypes.cast(off, ctypes.c_void_p),
                                    FAKE, FAKE, FAKE, FAKE, BIG_WS, None)
    assert rc == R.RTS_EINVAL and "2^19" in last_error(), last_error()


def extras(**kw):
    d = dict(window=0, reserved=0, draft=None, accepted=None, allowed=None, allowed_off=None)
    d.update(kw)
    return R.SampleExtras(**d)


def test_bad_extras_are_refused():
    rows = [dict(SAMPLED) for _ in range(10)]
    off_ok = (ctypes.c_int64 * 11)(*range(11))
    off_down = (ctypes.c_int64 * 11)(*([0, 5] + [3] * 9))
    off_neg = (ctypes.c_int64 * 11)(*([-1] + list(range(10))))
    off_big = (ctypes.c_int64 * 11)(*([0] * 10 + [2 ** 31]))
    cases = [
        (extras(reserved=1), "reserved"),
        (extras(window=65, draft=4096, accepted=4096), "window"),
        (extras(window=-1), "window"),
        (extras(window=3, draft=4096, accepted=4096), "multiple"),
        (extras(window=5, accepted=4096), "draft"),
        (extras(window=5, draft=4096), "accepted"),
        (extras(allowed=4096), "allowed_off"),
        (extras(allowed=4096, allowed_off=ctypes.cast(off_down, ctypes.c_void_p)), "decreases"),
        (extras(allowed=4096, allowed_off=ctypes.cast(off_neg, ctypes.c_void_p)), "allowed_off[0]"),
        (extras(allowed=4096, allowed_off=ctypes.cast(off_big, ctypes.c_void_p)), "2^31"),
    ]
    for ex, word in cases:
        assert sample(rows, ex=ex) == R.RTS_EINVAL, word
        assert word in last_error(), (word, last_error())
    # a valid window and list pass validation: the bad row then names itself
    bad = [dict(SAMPLED) for _ in range(9)] + [dict(SAMPLED, top_k=0)]
    ex = extras(window=5, draft=4096, accepted=4096, allowed=4096,
                allowed_off=ctypes.cast(off_ok, ctypes.c_void_p))
    assert sample(bad, ex=ex) == R.RTS_EINVAL and "row 9" in last_error()


def test_history_offsets_beyond_int32_are_refused():
    rows = [dict(SAMPLED, history_row=2, penalty_last_n=-1, penalty_repeat=1.1)]
    assert sample(rows, history=FAKE, H=3, ldh=2 ** 30, hist_len=[0, 0, 5]) == R.RTS_EINVAL
    assert "2^31" in last_error()


def test_short_workspace():
    need = R.workspace_bytes(1, 1000)
    assert sample([dict(SAMPLED)], ws_bytes=need - 1) == R.RTS_ENOSPC
    assert "workspace" in last_error()


def test_empty_batch_is_a_noop():
    assert sample([dict(SAMPLED)], B=0) == R.RTS_OK
    assert last_error() == ""


def test_history_checks():
    hist = FAKE
    rows = [dict(SAMPLED, history_row=1, penalty_last_n=64, penalty_repeat=1.1)]
    assert sample(rows, history=hist, H=1, ldh=64, hist_len=[64]) == R.RTS_EINVAL
    assert "history_row" in last_error()
    rows = [dict(SAMPLED, history_row=0, penalty_last_n=-1, penalty_repeat=1.1)]
    assert sample(rows, history=hist, H=1, ldh=64, hist_len=[65]) == R.RTS_EINVAL
    assert "length" in last_error()
    assert sample(rows, history=hist, H=1, ldh=70000, hist_len=[66000]) == R.RTS_EINVAL
    assert "window" in last_error()


def test_workspace_bytes():
    a = R.workspace_bytes(1, 248_320)
    b = R.workspace_bytes(40, 248_320)
    c = R.workspace_bytes(64, 248_320)
    d = R.workspace_bytes(1000, 248_320)
    assert 0 < a < b < c == d        # launches of up to 64 rows reuse one region
    assert R.workspace_bytes(64, 1024) % 256 == 0
    n = ctypes.c_size_t(0)
    assert R.lib().rts_workspace_bytes(-1, 10, ctypes.byref(n)) == R.RTS_EINVAL
    assert R.lib().rts_workspace_bytes(1, 0, ctypes.byref(n)) == R.RTS_EINVAL


def logprobs(B=2, V=1000, ld=None, tokens=FAKE, top_n=5, allowed=None, off=None, lp=FAKE,
             ids=FAKE, tlp=FAKE, ws_bytes=BIG_WS):
    offa = None if off is None else (ctypes.c_int64 * len(off))(*off)
    return R.lib().rts_token_logprobs(FAKE, B, V, V if ld is None else ld, tokens, top_n,
                                      allowed, offa, lp, ids, tlp, FAKE, ws_bytes, None)


def test_logprob_argument_checks():
    assert logprobs(top_n=21) == R.RTS_EINVAL and "top_n" in last_error()
    assert logprobs(top_n=-1) == R.RTS_EINVAL
    assert logprobs(ids=None) == R.RTS_EINVAL
    assert logprobs(tokens=None) == R.RTS_EINVAL
    assert logprobs(lp=None) == R.RTS_EINVAL
    assert logprobs(ld=10) == R.RTS_EINVAL
    assert logprobs(allowed=FAKE, off=None) == R.RTS_EINVAL
    assert logprobs(allowed=FAKE, off=[0, 5, 3]) == R.RTS_EINVAL and "decreases" in last_error()
    assert logprobs(allowed=FAKE, off=[-1, 5, 6]) == R.RTS_EINVAL
    # lists longer than 2,048 ids need the vocabulary bitmap (V <= 2^19)
    assert logprobs(V=(1 << 19) + 1, allowed=FAKE, off=[0, 2049, 2050]) == R.RTS_EINVAL
    assert "2^19" in last_error()
    assert logprobs(ws_bytes=100) == R.RTS_ENOSPC
    assert logprobs(B=0) == R.RTS_OK


def test_strerror():
    L = R.lib()
    for code in (0, -1, -2, -3, 7):
        assert L.rts_strerror(code)


def test_read_rows_refusals():
    L = R.lib()
    assert L.rts_read_rows(FAKE, -1, 100, 100, FAKE, None) == R.RTS_EINVAL
    assert L.rts_read_rows(FAKE, 0, 100, 100, FAKE, None) == R.RTS_OK
    assert L.rts_read_rows(FAKE, 1, 0, 100, FAKE, None) == R.RTS_EINVAL
    assert L.rts_read_rows(FAKE, 1, 100, 99, FAKE, None) == R.RTS_EINVAL and "ld" in last_error()
    assert L.rts_read_rows(None, 1, 100, 100, FAKE, None) == R.RTS_EINVAL
    assert L.rts_read_rows(FAKE, 1, 100, 100, None, None) == R.RTS_EINVAL


def test_prior_designs_refusals():
    L = R.lib()
    arr = R.row_params([dict(SAMPLED)])

    def call(design=2, B=1, V=1000, ld=1000, rows=arr):
        return L.rts_sample_tokens_prior(design, FAKE, B, V, ld, rows, None, 0, 0, None, FAKE,
                                         None, None, None, None, FAKE, BIG_WS, None)
    assert call(design=0) == R.RTS_EINVAL and "design" in last_error()
    assert call(design=4) == R.RTS_EINVAL
    assert call(V=(1 << 20) + 1, ld=(1 << 20) + 1) == R.RTS_EINVAL
    assert call(ld=10) == R.RTS_EINVAL
    assert call(B=0) == R.RTS_OK
    assert call(rows=R.row_params([dict(SAMPLED, top_k=65)])) == R.RTS_EINVAL
    assert "top_k" in last_error()
