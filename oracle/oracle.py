"""ctypes wrapper of the plain C oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg; the product path never imports it.  It shares no
code with the HIP library.  Build it with ``build()`` (gcc, -ffp-contract=off).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
LIB_NATIVE = os.path.join(HERE, "liboracle_native.so")

FLAG_TOP_P_EDGE = 1
FLAG_DRAW_EDGE = 2


class RowParams(ctypes.Structure):
    _fields_ = [
        ("temperature", ctypes.c_float),
        ("top_k", ctypes.c_int32),
        ("top_p", ctypes.c_float),
        ("min_p", ctypes.c_float),
        ("penalty_repeat", ctypes.c_float),
        ("penalty_freq", ctypes.c_float),
        ("penalty_present", ctypes.c_float),
        ("penalty_last_n", ctypes.c_int32),
        ("history_row", ctypes.c_int32),
        ("pad_", ctypes.c_int32),
        ("seed", ctypes.c_uint64),
        ("counter", ctypes.c_uint64),
    ]


def build(force: bool = True, native: bool = False) -> str:
    """Compile oracle.c into liboracle.so next to it.  With `native`, the same
    source with -O3 -march=native into liboracle_native.so: the host-speed
    build the benchmark times (still -ffp-contract=off and no fast-math, so
    every result is the one the -O2 build gives)."""
    out = LIB_NATIVE if native else LIB
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(SRC):
        tmp = out + ".tmp"
        opt = ["-O3", "-march=native"] if native else ["-O2"]
        subprocess.check_call(
            ["gcc", *opt, "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math", "-Wall", "-o", tmp, SRC, "-lm"])
        os.replace(tmp, out)
    return out


_lib = None
_lib_native = None


def _bind(L):
    P = ctypes.c_void_p
    L.oracle_philox4x32_10.argtypes = [P, P, P]
    L.oracle_philox4x32_10.restype = None
    L.oracle_sample_row.argtypes = [P, ctypes.c_int64, P, P, ctypes.c_int64,
                                    P, P, P, P, P, P, P]
    L.oracle_penalised_row.argtypes = [P, ctypes.c_int64, P, P, ctypes.c_int64, P]
    L.oracle_sample_tokens.argtypes = [P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                       P, P, ctypes.c_int64, ctypes.c_int64, P,
                                       P, P, P, P, P, P, P]
    L.oracle_token_logprobs_row.argtypes = [P, ctypes.c_int64, ctypes.c_int32,
                                            ctypes.c_int32, P, ctypes.c_int64, P, P, P]
    L.oracle_sample_row_masked.argtypes = [P, ctypes.c_int64, P, P, ctypes.c_int64,
                                           P, ctypes.c_int64, P, P, P, P, P, P, P]
    L.oracle_accept_windows.argtypes = [P, ctypes.c_int64, ctypes.c_int32, P, P]
    L.oracle_draw_on_prefix.argtypes = [P, ctypes.c_int, ctypes.c_float, ctypes.c_double, P]
    for f in ("oracle_draw_on_prefix", "oracle_sample_row", "oracle_penalised_row",
              "oracle_sample_tokens", "oracle_token_logprobs_row", "oracle_sample_row_masked",
              "oracle_accept_windows"):
        getattr(L, f).restype = ctypes.c_int
    return L


def lib():
    global _lib
    if _lib_native is not None:
        return _lib_native
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build(force=True)
        _lib = _bind(ctypes.CDLL(LIB))
    return _lib


def use_native_build(on: bool = True) -> None:
    """Route every wrapper below through the -O3 -march=native build of the
    same source (built on first use), or back to the -O2 build.  The calls
    release the GIL, so host threads can run rows side by side."""
    global _lib_native
    if on and _lib_native is None:
        _lib_native = _bind(ctypes.CDLL(build(force=True, native=True)))
    elif not on:
        _lib_native = None


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def make_params(d: dict) -> RowParams:
    p = RowParams()
    p.temperature = d.get("temperature", 0.0)
    p.top_k = d.get("top_k", 0)
    p.top_p = d.get("top_p", 1.0)
    p.min_p = d.get("min_p", 0.0)
    p.penalty_repeat = d.get("penalty_repeat", 1.0)
    p.penalty_freq = d.get("penalty_freq", 0.0)
    p.penalty_present = d.get("penalty_present", 0.0)
    p.penalty_last_n = d.get("penalty_last_n", 0)
    p.history_row = d.get("history_row", -1)
    p.seed = d.get("seed", 0)
    p.counter = d.get("counter", 0)
    return p


def philox4x32_10(ctr, key):
    """Philox4x32-10 of one (counter[4], key[2]) block -> 4 uint32 words."""
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def draw_on_prefix(kept_logits, temperature: float, u: float):
    """The draw alone over the kept logits given (temperature, then the
    inverse CDF at u): (picked position, positions j whose CDF value lies
    within 1e-6 of u)."""
    y = np.ascontiguousarray(kept_logits, dtype=np.float32)
    if not 1 <= y.size <= 64:
        raise ValueError("draw_on_prefix takes 1..64 logits")
    edges = np.zeros(1, np.uint64)
    pick = lib().oracle_draw_on_prefix(_ptr(y), int(y.size), float(temperature), float(u),
                                       _ptr(edges))
    e = int(edges[0])
    return int(pick), [j for j in range(64) if (e >> j) & 1]


def penalised_row(x, params: dict, hist=None):
    x = np.ascontiguousarray(x, dtype=np.float32)
    h = None if hist is None else np.ascontiguousarray(hist, dtype=np.int32)
    y = np.empty_like(x)
    p = make_params(params)
    rc = lib().oracle_penalised_row(_ptr(x), x.size, ctypes.byref(p), _ptr(h),
                                    0 if h is None else h.size, _ptr(y))
    if rc != 0:
        raise ValueError("oracle_penalised_row refused its input")
    return y


def sample_row(x, params: dict, hist=None, allowed=None) -> dict:
    """The whole chain on one row; returns a dict of every output.  With a
    non-empty `allowed`, the candidates are its distinct in-range ids."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    h = None if hist is None else np.ascontiguousarray(hist, dtype=np.int32)
    a = None if allowed is None else np.ascontiguousarray(allowed, dtype=np.int32)
    p = make_params(params)
    tok = np.zeros(1, np.int32)
    counts = np.zeros(3, np.int32)
    kid = np.zeros(64, np.int32)
    klg = np.zeros(64, np.float32)
    x0 = np.zeros(1, np.uint32)
    u = np.zeros(1, np.float64)
    fl = np.zeros(1, np.int32)
    rc = lib().oracle_sample_row_masked(_ptr(x), x.size, ctypes.byref(p), _ptr(h),
                                        0 if h is None else h.size, _ptr(a),
                                        0 if a is None else a.size, _ptr(tok), _ptr(counts),
                                        _ptr(kid), _ptr(klg), _ptr(x0), _ptr(u), _ptr(fl))
    if rc != 0:
        raise ValueError("oracle_sample_row refused its input")
    return dict(token=int(tok[0]), counts=counts, kept_ids=kid, kept_logits=klg,
                x0=int(x0[0]), u=float(u[0]), flags=int(fl[0]),
                temperature=float(p.temperature))


def sample_tokens(logits, params: list, history=None, hist_len=None) -> dict:
    """B rows: logits [B][V] float32, history [H][ldh] int32 with hist_len [H]."""
    x = np.ascontiguousarray(logits, dtype=np.float32)
    B, V = x.shape
    arr = (RowParams * max(B, 1))(*[make_params(d) for d in params])
    if history is not None:
        h = np.ascontiguousarray(history, dtype=np.int32)
        H, ldh = h.shape
        hl = np.ascontiguousarray(hist_len, dtype=np.int32)
    else:
        h, H, ldh, hl = None, 0, 0, None
    tok = np.zeros(B, np.int32)
    counts = np.zeros((B, 3), np.int32)
    kid = np.zeros((B, 64), np.int32)
    klg = np.zeros((B, 64), np.float32)
    x0 = np.zeros(B, np.uint32)
    u = np.zeros(B, np.float64)
    fl = np.zeros(B, np.int32)
    rc = lib().oracle_sample_tokens(_ptr(x), B, V, V, arr, _ptr(h), H, ldh, _ptr(hl),
                                    _ptr(tok), _ptr(counts), _ptr(kid), _ptr(klg),
                                    _ptr(x0), _ptr(u), _ptr(fl))
    if rc != 0:
        raise ValueError("oracle_sample_tokens refused its input")
    return dict(token=tok, counts=counts, kept_ids=kid, kept_logits=klg, x0=x0, u=u,
                flags=fl, temperature=np.array([a.temperature for a in arr[:B]], np.float32))


def token_logprobs_row(x, token: int, top_n: int, allowed=None) -> dict:
    x = np.ascontiguousarray(x, dtype=np.float32)
    a = None if allowed is None else np.ascontiguousarray(allowed, dtype=np.int32)
    lp = np.zeros(1, np.float64)
    tid = np.zeros(max(top_n, 1), np.int32)
    tlp = np.zeros(max(top_n, 1), np.float64)
    rc = lib().oracle_token_logprobs_row(_ptr(x), x.size, int(token), int(top_n), _ptr(a),
                                         0 if a is None else a.size, _ptr(lp), _ptr(tid),
                                         _ptr(tlp))
    if rc != 0:
        raise ValueError("oracle_token_logprobs_row refused its input")
    return dict(token_lp=float(lp[0]), top_ids=tid[:top_n].copy(), top_lp=tlp[:top_n].copy())


def token_logprobs(logits, tokens, top_n: int, allowed_lists=None) -> dict:
    x = np.ascontiguousarray(logits, dtype=np.float32)
    B = x.shape[0]
    lp = np.zeros(B, np.float64)
    tid = np.zeros((B, top_n), np.int32)
    tlp = np.zeros((B, top_n), np.float64)
    for r in range(B):
        a = None if allowed_lists is None else allowed_lists[r]
        o = token_logprobs_row(x[r], int(tokens[r]), top_n, a)
        lp[r] = o["token_lp"]
        tid[r] = o["top_ids"]
        tlp[r] = o["top_lp"]
    return dict(token_lp=lp, top_ids=tid, top_lp=tlp)


def sample_tokens_masked(logits, params: list, allowed_lists, history=None,
                         hist_len=None) -> dict:
    """B rows, each restricted to its allowed list (None or empty: no
    restriction); same outputs as sample_tokens."""
    x = np.ascontiguousarray(logits, dtype=np.float32)
    B, V = x.shape
    outs = []
    for r in range(B):
        h = None
        p = params[r]
        if history is not None and p.get("history_row", -1) >= 0:
            h = np.asarray(history, np.int32)[p["history_row"]][:int(hist_len[p["history_row"]])]
        a = allowed_lists[r] if allowed_lists is not None else None
        outs.append(sample_row(x[r], p, h, a))
    return dict(token=np.array([o["token"] for o in outs], np.int32),
                counts=np.stack([o["counts"] for o in outs]),
                kept_ids=np.stack([o["kept_ids"] for o in outs]),
                kept_logits=np.stack([o["kept_logits"] for o in outs]),
                x0=np.array([o["x0"] for o in outs], np.uint32),
                u=np.array([o["u"] for o in outs], np.float64),
                flags=np.array([o["flags"] for o in outs], np.int32),
                temperature=np.array([o["temperature"] for o in outs], np.float32))


def accept_windows(tokens, window: int, drafts) -> np.ndarray:
    """Tokens emitted per verify window of `window` consecutive rows."""
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    d = np.ascontiguousarray(drafts, dtype=np.int32)
    out = np.zeros(t.size // window, np.int32)
    rc = lib().oracle_accept_windows(_ptr(t), t.size, int(window), _ptr(d), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_accept_windows refused its input")
    return out
