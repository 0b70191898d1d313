"""Seeded synthetic inputs for the sampler's workloads.

This module only draws inputs (logit rows, history rows, per-row parameters,
allowed-id lists).  It holds none of the sampling method's arithmetic, so the
HIP path and the CPU oracle can both be fed from it.

The shapes follow the pages' own workloads: a vocabulary of 248,320 head
logits in fp32 (#19, "What changed", the min_p/penalties paragraph), a verify
window of one head row plus four draft rows (#3200 "Validation" and #1916
"Extra Notes" run with --spec 4), up to eight batch slots (#559, item 1),
penalty windows of 64 ids (#19, the server.py paragraph) and injected
duplicate logits (#19, "Verification").  No trained model is involved: the
logits are Gaussian, N(0, sigma) with sigma the standard deviation.
"""
from __future__ import annotations

import numpy as np

V_FULL = 248_320

NEUTRAL = dict(temperature=0.0, top_k=0, top_p=1.0, min_p=0.0, penalty_repeat=1.0,
               penalty_freq=0.0, penalty_present=0.0, penalty_last_n=0, history_row=-1,
               seed=0, counter=0)


def row_params(**kw) -> dict:
    d = dict(NEUTRAL)
    d.update(kw)
    return d


def tiny(V: int = 1024):
    """Four rows of N(0, 2) logits over a small vocabulary; a sampled pass and
    a greedy pass with neutral parameters over the same rows."""
    x = np.random.default_rng(0).normal(0.0, 2.0, (4, V)).astype(np.float32)
    sampled = [row_params(temperature=0.8, top_k=8, top_p=0.9, min_p=0.05, seed=42, counter=r)
               for r in range(4)]
    greedy = [row_params() for _ in range(4)]
    return dict(logits=x, sampled=sampled, greedy=greedy)


def single_stream(V: int = V_FULL):
    """One row of N(0, 3) logits with three spiked heads (+12, +10, +9 added at
    three distinct random ids drawn after the row); top_k 20 sampled and a
    greedy pass over the same row."""
    rng = np.random.default_rng(1)
    x = rng.normal(0.0, 3.0, V).astype(np.float32)
    ids = rng.choice(V, 3, replace=False)
    x[ids] += np.array([12.0, 10.0, 9.0], dtype=np.float32)
    sampled = [row_params(temperature=0.7, top_k=20, top_p=0.8, min_p=0.0, seed=42, counter=0)]
    greedy = [row_params()]
    return dict(logits=x.reshape(1, V), sampled=sampled, greedy=greedy, spikes=ids)


class VerifyWindows:
    """Ten speculative verify windows of five rows (four drafts plus the head).

    Each window draws fresh N(0, 3) rows from one stream.  All five rows share
    one history row of 64 ids: 48 distinct uniform ids plus 16 repeats of them,
    shuffled (25 % repeats).  After a window the caller feeds back row 0's
    token: it is appended and the oldest id dropped.  The Philox counter of
    row r in window w is 5w + r, so it persists across the windows."""

    ROWS = 5
    HLEN = 64

    def __init__(self, V: int = V_FULL, windows: int = 10):
        self.V = V
        self.windows = windows
        self._logit_rng = np.random.default_rng(2)
        hrng = np.random.default_rng(20)
        uniq = hrng.choice(V, 48, replace=False)
        rep = hrng.choice(uniq, 16, replace=True)
        h = np.concatenate([uniq, rep]).astype(np.int32)
        hrng.shuffle(h)
        self.history = h
        self.w = 0

    def params(self, w: int):
        return [row_params(temperature=1.0, top_k=40, top_p=0.95, min_p=0.05,
                           penalty_repeat=1.1, penalty_freq=0.5, penalty_present=0.5,
                           penalty_last_n=64, history_row=0, seed=42,
                           counter=self.ROWS * w + r) for r in range(self.ROWS)]

    def next_logits(self) -> np.ndarray:
        return self._logit_rng.normal(0.0, 3.0, (self.ROWS, self.V)).astype(np.float32)

    def feed_back(self, token: int) -> None:
        self.history = np.concatenate([self.history[1:], np.array([token], np.int32)])


def boost_history(x: np.ndarray, history: np.ndarray, boost: float) -> np.ndarray:
    """Copy of a logit row with the history ids raised by `boost`, as a model
    that keeps predicting its recent tokens would; it makes penalties visible
    in the kept sequence."""
    y = np.array(x, dtype=np.float32, copy=True)
    ids = np.unique(history[(history >= 0) & (history < y.shape[-1])])
    y[..., ids] += np.float32(boost)
    return y


def batch_slots(V: int = V_FULL, slots: int = 8, rows_per_slot: int = 5, hlen: int = 256):
    """Eight slots of five window rows (40 rows) of N(0, 3) logits.  Each slot
    has its own history row of 256 Zipf(1.1) ids (values above V rejected,
    id = z - 1, so most land in low ids).  Per-row parameters are drawn from
    one seeded stream: temperature U[0.2, 1.5], top_k U{1..64}, top_p
    U[0.5, 1], min_p U[0, 0.2]; penalties 1.1 / 0.5 / 0.5 over the last 256
    ids; seed 1000 + slot, counter = the row's place in its slot."""
    B = slots * rows_per_slot
    x = np.random.default_rng(3).normal(0.0, 3.0, (B, V)).astype(np.float32)
    hist = np.zeros((slots, hlen), np.int32)
    for s in range(slots):
        rng = np.random.default_rng(30 + s)
        got = []
        while len(got) < hlen:
            z = rng.zipf(1.1, 4 * hlen)
            got.extend(int(v) - 1 for v in z if v <= V)
        hist[s] = np.array(got[:hlen], np.int32)
    prng = np.random.default_rng(33)
    T = prng.uniform(0.2, 1.5, B)
    K = prng.integers(1, 65, B)
    P = prng.uniform(0.5, 1.0, B)
    M = prng.uniform(0.0, 0.2, B)
    params = []
    for r in range(B):
        s = r // rows_per_slot
        params.append(row_params(temperature=float(np.float32(T[r])), top_k=int(K[r]),
                                 top_p=float(np.float32(P[r])), min_p=float(np.float32(M[r])),
                                 penalty_repeat=1.1, penalty_freq=0.5, penalty_present=0.5,
                                 penalty_last_n=hlen, history_row=s, seed=1000 + s,
                                 counter=r % rows_per_slot))
    hist_len = np.full(slots, hlen, np.int32)
    return dict(logits=x, params=params, history=hist, hist_len=hist_len)


def bf16_grid(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 value (ties to even) and return
    them as fp32: an input transform that makes equal logits common."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16) << 16
    return (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32)


def logprobs_stress(V: int = V_FULL, B: int = 40, n_allowed: int = 1000):
    """40 rows of N(0, 3) logits on the bf16 grid (many equal values); top_k
    64, min_p 0.1, temperature 1; then top-20 logprobs, unrestricted and over
    1,000 distinct random allowed ids per row."""
    x = bf16_grid(np.random.default_rng(4).normal(0.0, 3.0, (B, V)).astype(np.float32))
    params = [row_params(temperature=1.0, top_k=64, min_p=0.1, top_p=1.0, seed=42, counter=r)
              for r in range(B)]
    arng = np.random.default_rng(44)
    allowed = [arng.choice(V, n_allowed, replace=False).astype(np.int32) for _ in range(B)]
    return dict(logits=x, params=params, allowed=allowed, top_n=20)


def pack_allowed(lists):
    """Concatenate per-row id lists into (ids int32[sum], offsets int64[B+1])."""
    off = np.zeros(len(lists) + 1, np.int64)
    for i, a in enumerate(lists):
        off[i + 1] = off[i] + (0 if a is None else len(a))
    ids = np.concatenate([np.asarray(a, np.int32) for a in lists if a is not None and len(a)]) \
        if off[-1] > 0 else np.zeros(0, np.int32)
    return ids.astype(np.int32), off
