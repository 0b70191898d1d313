"""Per-token sampling chain and raw-logit logprobs on MI355X (gfx950).

A thin ctypes binding of the C ABI in include/rts.h (librts.so, built in-tree
by ``python -m request_token_sampling_amd.build_lib``).  It only marshals
arguments: torch provides device memory and the current stream, every step of
the chain runs in the library's HIP kernels, and the library itself checks
every argument.  There is no CPU fallback: if the library is missing, import
of the entry points fails loudly.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librts.so")

RTS_OK, RTS_EINVAL, RTS_ENOSPC, RTS_EDEVICE = 0, -1, -2, -3
MAX_TOP_K = 64
KEPT = 64
MAX_TOP_N = 20
PRIOR_THREAD, PRIOR_BLOCK, PRIOR_RECOUNT = 1, 2, 3


class RTSError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"rts error {code}: {msg}")
        self.code = code


class RowParams(ctypes.Structure):
    """Mirror of rts_row_params (56 bytes)."""
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
        ("reserved", ctypes.c_int32),
        ("seed", ctypes.c_uint64),
        ("counter", ctypes.c_uint64),
    ]


assert ctypes.sizeof(RowParams) == 56


class LogprobRequest(ctypes.Structure):
    """Mirror of rts_logprob_request: raw-logit logprobs of the sampled tokens
    computed in the sampling call's own pass over the logits, optionally also
    renormalised over per-row allowed lists."""
    _fields_ = [
        ("top_n", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("token_lp", ctypes.c_void_p),
        ("top_ids", ctypes.c_void_p),
        ("top_lp", ctypes.c_void_p),
        ("allowed", ctypes.c_void_p),
        ("allowed_off", ctypes.c_void_p),
        ("allowed_token_lp", ctypes.c_void_p),
        ("allowed_top_ids", ctypes.c_void_p),
        ("allowed_top_lp", ctypes.c_void_p),
    ]


assert ctypes.sizeof(LogprobRequest) == 72


class SampleExtras(ctypes.Structure):
    """Mirror of rts_sample_extras: verify windows with drafts, and allowed-id
    lists that restrict a row's candidates."""
    _fields_ = [
        ("window", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("draft", ctypes.c_void_p),
        ("accepted", ctypes.c_void_p),
        ("allowed", ctypes.c_void_p),
        ("allowed_off", ctypes.c_void_p),
        ("ignored_ids", ctypes.c_void_p),
    ]


assert ctypes.sizeof(SampleExtras) == 48

_DEFAULTS = dict(temperature=0.0, top_k=0, top_p=1.0, min_p=0.0, penalty_repeat=1.0,
                 penalty_freq=0.0, penalty_present=0.0, penalty_last_n=0, history_row=-1,
                 reserved=0, seed=0, counter=0)

_lib = None


def lib() -> ctypes.CDLL:
    """Load librts.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "python -m request_token_sampling_amd.build_lib")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        L.rts_workspace_bytes.argtypes = [I64, I64, ctypes.POINTER(ctypes.c_size_t)]
        L.rts_workspace_init.argtypes = [P, SZ, P]
        L.rts_sample_tokens.argtypes = [P, I64, I64, I64, P, P, I64, I64, P, P, P, P, P, P, P,
                                        I64, P, P, P, SZ, P]
        L.rts_token_logprobs.argtypes = [P, I64, I64, I64, P, I32, P, P, P, P, P, P, SZ, P]
        L.rts_read_rows.argtypes = [P, I64, I64, I64, P, P]
        L.rts_sample_tokens_prior.argtypes = [I32, P, I64, I64, I64, P, P, I64, I64, P, P, P, P,
                                              P, P, P, SZ, P]
        L.rts_sample_tokens_noalloc.argtypes = [P, I64, I64, I64, P, P, I64, I64, P, P, P, P, P,
                                                P, P, I64, P, P, P]
        L.rts_noalloc_scratch_bytes.argtypes = []
        L.rts_noalloc_scratch_bytes.restype = ctypes.c_size_t
        for f in ("rts_workspace_bytes", "rts_workspace_init", "rts_sample_tokens",
                  "rts_token_logprobs", "rts_read_rows", "rts_sample_tokens_prior",
                  "rts_sample_tokens_noalloc"):
            getattr(L, f).restype = ctypes.c_int
        L.rts_strerror.argtypes = [ctypes.c_int]
        L.rts_strerror.restype = ctypes.c_char_p
        L.rts_last_error.argtypes = []
        L.rts_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(rc: int) -> None:
    if rc != RTS_OK:
        msg = lib().rts_last_error().decode() or lib().rts_strerror(rc).decode()
        raise RTSError(rc, msg)


def row_params(rows) -> ctypes.Array:
    """A list of dicts (missing keys neutral) -> rts_row_params[B]."""
    arr = (RowParams * max(len(rows), 1))()
    for i, d in enumerate(rows):
        full = dict(_DEFAULTS)
        full.update(d)
        for k, v in full.items():
            setattr(arr[i], k, v)
    return arr


def workspace_bytes(B: int, V: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().rts_workspace_bytes(B, V, ctypes.byref(n)))
    return int(n.value)


def make_workspace(B: int, V: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace (zero counters need no rts_workspace_init)."""
    return torch.zeros(workspace_bytes(B, V), dtype=torch.uint8, device=device)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _rows_view(logits: torch.Tensor):
    if logits.dim() == 1:
        logits = logits.unsqueeze(0)
    if logits.dim() != 2 or logits.dtype != torch.float32 or not logits.is_cuda:
        raise ValueError("logits must be a 2-D float32 CUDA tensor")
    if logits.stride(1) != 1:
        raise ValueError("logits rows must be contiguous")
    B, V = logits.shape
    return logits, B, V, logits.stride(0) if B > 1 else V


class SampleCall:
    """One prepared call of rts_sample_tokens: outputs, workspace and ctypes
    arguments are built once, so repeated calls (benchmarks, decode loops over
    fixed buffers) pay only the C call.  Params may be replaced between calls
    with ``set_params``."""

    def __init__(self, logits, params, history=None, history_len=None, workspace=None,
                 stream=None, counters=None, counter_stride=0, logprobs=None, window=0,
                 draft=None, allowed=None, allowed_off=None, ignored=None,
                 logprob_allowed=None, logprob_allowed_off=None, noalloc=False):
        self.logits, self.B, self.V, self.ld = _rows_view(logits)
        dev = self.logits.device
        # noalloc: call rts_sample_tokens_noalloc (the library's static scratch)
        self.noalloc = bool(noalloc)
        if self.noalloc and workspace is not None:
            raise ValueError("noalloc calls take no workspace")
        self.token = torch.empty(self.B, dtype=torch.int32, device=dev)
        self.counts = torch.empty((self.B, 3), dtype=torch.int32, device=dev)
        self.kept_ids = torch.empty((self.B, KEPT), dtype=torch.int32, device=dev)
        self.kept_logits = torch.empty((self.B, KEPT), dtype=torch.float32, device=dev)
        self.philox_x0 = torch.empty(self.B, dtype=torch.int32, device=dev)
        self.workspace = (None if self.noalloc else
                          workspace if workspace is not None else make_workspace(self.B, self.V, dev))
        self.history = history
        if history is not None:
            if history.dtype != torch.int32 or history.dim() != 2 or history.stride(1) != 1:
                raise ValueError("history must be a 2-D int32 tensor with contiguous rows")
            self.H, self.ldh = history.shape[0], history.stride(0)
            self.hist_len = np.ascontiguousarray(history_len, dtype=np.int32)
        else:
            self.H, self.ldh, self.hist_len = 0, 0, None
        if counters is not None:
            if counters.dtype != torch.int64 or not counters.is_cuda or counters.numel() < self.B:
                raise ValueError("counters must be a CUDA int64 tensor with one entry per row")
        self.counters = counters
        self.counter_stride = int(counter_stride)
        # logprobs=top_n (0..20): raw-logit logprobs of the sampled tokens in the same pass
        self.lp = None
        self.lp_allowed = None
        if logprobs is not None:
            n = int(logprobs)
            self.token_lp = torch.empty(self.B, dtype=torch.float32, device=dev)
            self.top_ids = torch.empty((self.B, max(n, 0)), dtype=torch.int32, device=dev)
            self.top_lp = torch.empty((self.B, max(n, 0)), dtype=torch.float32, device=dev)
            self.lp = LogprobRequest(n, 0, self.token_lp.data_ptr(),
                                     self.top_ids.data_ptr() if n > 0 else None,
                                     self.top_lp.data_ptr() if n > 0 else None)
            # the same, renormalised over per-row allowed lists (not a mask)
            self.lp_allowed = logprob_allowed
            if logprob_allowed is not None:
                if logprob_allowed.dtype != torch.int32 or not logprob_allowed.is_cuda:
                    raise ValueError("logprob_allowed must be a CUDA int32 tensor")
                self.lp_allowed_off = np.ascontiguousarray(logprob_allowed_off, dtype=np.int64)
                self.a_token_lp = torch.empty(self.B, dtype=torch.float32, device=dev)
                self.a_top_ids = torch.empty((self.B, max(n, 0)), dtype=torch.int32, device=dev)
                self.a_top_lp = torch.empty((self.B, max(n, 0)), dtype=torch.float32, device=dev)
                self.lp.allowed = logprob_allowed.data_ptr()
                self.lp.allowed_off = self.lp_allowed_off.ctypes.data_as(ctypes.c_void_p)
                self.lp.allowed_token_lp = self.a_token_lp.data_ptr()
                self.lp.allowed_top_ids = self.a_top_ids.data_ptr() if n > 0 else None
                self.lp.allowed_top_lp = self.a_top_lp.data_ptr() if n > 0 else None
        elif logprob_allowed is not None:
            raise ValueError("logprob_allowed needs logprobs=top_n")
        # verify windows (window rows each, drafts per row) and allowed-id masks
        self.ex = None
        self.accepted = None
        if ignored is not None and (ignored.dtype != torch.int32 or not ignored.is_cuda):
            raise ValueError("ignored must be a CUDA int32 tensor (one counter word)")
        self.ignored = ignored
        if window or allowed is not None or ignored is not None:
            if window:
                if draft is None or draft.dtype != torch.int32 or not draft.is_cuda:
                    raise ValueError("window needs draft: a CUDA int32 tensor of B ids")
                self.accepted = torch.empty(max(self.B // int(window), 1), dtype=torch.int32,
                                            device=dev)
            self.draft = draft
            self.allowed = allowed
            self.allowed_off = (None if allowed is None
                                else np.ascontiguousarray(allowed_off, dtype=np.int64))
            self.ex = SampleExtras(int(window), 0, None if draft is None else draft.data_ptr(),
                                   None if self.accepted is None else self.accepted.data_ptr(),
                                   None if allowed is None else allowed.data_ptr(),
                                   None if allowed is None
                                   else self.allowed_off.ctypes.data_as(ctypes.c_void_p),
                                   None if ignored is None else ignored.data_ptr())
        self.set_params(params)
        self.stream = stream

    def set_params(self, params):
        self.params = params if isinstance(params, ctypes.Array) else row_params(params)
        self._args = None

    def _build_args(self):
        self._args = [
            None, self.B, self.V, self.ld, self.params,
            _ptr(self.history), self.H, self.ldh,
            None if self.hist_len is None else self.hist_len.ctypes.data_as(ctypes.c_void_p),
            _ptr(self.token), _ptr(self.counts), _ptr(self.kept_ids), _ptr(self.kept_logits),
            _ptr(self.philox_x0), _ptr(self.counters), self.counter_stride,
            None if self.lp is None else ctypes.byref(self.lp),
            None if self.ex is None else ctypes.byref(self.ex),
            _ptr(self.workspace), 0 if self.workspace is None else self.workspace.numel(), None]

    def __call__(self):
        if self._args is None:
            self._build_args()
        a = self._args
        a[0] = self.logits.data_ptr()
        a[20] = _stream_handle(self.stream)
        if self.noalloc:
            # rts_sample_tokens_noalloc: the same arguments without the workspace
            _check(lib().rts_sample_tokens_noalloc(*a[:18], a[20]))
        else:
            _check(lib().rts_sample_tokens(*a))
        return self

    def results(self) -> dict:
        """Device tensors; philox_x0 holds the uint32 words' bits as int32."""
        r = dict(token=self.token, counts=self.counts, kept_ids=self.kept_ids,
                 kept_logits=self.kept_logits, philox_x0=self.philox_x0)
        if self.lp is not None:
            r.update(token_lp=self.token_lp, top_ids=self.top_ids, top_lp=self.top_lp)
            if self.lp_allowed is not None:
                r.update(allowed_token_lp=self.a_token_lp, allowed_top_ids=self.a_top_ids,
                         allowed_top_lp=self.a_top_lp)
        if self.accepted is not None:
            r.update(accepted=self.accepted)
        return r


def sample_tokens(logits, params, history=None, history_len=None, workspace=None,
                  stream=None, counters=None, counter_stride=0, logprobs=None, window=0,
                  draft=None, allowed=None, allowed_off=None, ignored=None,
                  logprob_allowed=None, logprob_allowed_off=None) -> dict:
    """Run the sampling chain over the rows of `logits` (CUDA float32 [B][V]).

    params: list of per-row dicts (keys of rts_row_params; missing keys neutral).
    history: CUDA int32 [H][ldh] with host lengths history_len[H], or None.
    Returns device tensors token[B], counts[B][3], kept_ids[B][64],
    kept_logits[B][64], philox_x0[B].  counters: optional CUDA int64 [B]
    device-resident Philox counters, advanced by counter_stride per call.
    logprobs: None, or top_n in 0..20 to add token_lp[B], top_ids[B][top_n]
    and top_lp[B][top_n], the raw-logit logprobs of the sampled tokens,
    computed in the same pass over the logits.
    window, draft: verify windows of `window` rows with a CUDA int32 draft id
    per row; adds accepted[B / window], the tokens each window emits.
    allowed, allowed_off: CUDA int32 ids with host int64 offsets [B+1]; a row
    with a non-empty list samples only among those ids.
    ignored: optional CUDA int32 [1] counter; the call adds the number of
    device ids it read and ignored (outside [0, V)).
    logprob_allowed, logprob_allowed_off (with logprobs): CUDA int32 ids with
    host int64 offsets [B+1]; adds allowed_token_lp[B], allowed_top_ids and
    allowed_top_lp[B][top_n], the logprobs renormalised over each row's list
    (an empty list: the unrestricted values).  The lists do not restrict
    sampling."""
    return SampleCall(logits, params, history, history_len, workspace, stream, counters,
                      counter_stride, logprobs, window, draft, allowed, allowed_off,
                      ignored, logprob_allowed, logprob_allowed_off)().results()


def sample_tokens_noalloc(logits, params, history=None, history_len=None, stream=None,
                          counters=None, counter_stride=0, logprobs=None, window=0, draft=None,
                          allowed=None, allowed_off=None, ignored=None, logprob_allowed=None,
                          logprob_allowed_off=None) -> dict:
    """sample_tokens through rts_sample_tokens_noalloc: no workspace, the
    library's static scratch instead (see include/rts.h)."""
    return SampleCall(logits, params, history, history_len, None, stream, counters,
                      counter_stride, logprobs, window, draft, allowed, allowed_off, ignored,
                      logprob_allowed, logprob_allowed_off, noalloc=True)().results()


def noalloc_scratch_bytes() -> int:
    return int(lib().rts_noalloc_scratch_bytes())


class LogprobCall:
    """One prepared call of rts_token_logprobs (outputs, workspace and ctypes
    arguments built once; the tokens tensor is read at each call)."""

    def __init__(self, logits, tokens, top_n: int, allowed=None, allowed_off=None,
                 workspace=None, stream=None):
        self.logits, self.B, self.V, self.ld = _rows_view(logits)
        dev = self.logits.device
        if tokens.dtype != torch.int32 or not tokens.is_cuda:
            raise ValueError("tokens must be a CUDA int32 tensor")
        self.tokens = tokens
        self.top_n = int(top_n)
        self.token_lp = torch.empty(self.B, dtype=torch.float32, device=dev)
        self.top_ids = torch.empty((self.B, max(self.top_n, 0)), dtype=torch.int32, device=dev)
        self.top_lp = torch.empty((self.B, max(self.top_n, 0)), dtype=torch.float32, device=dev)
        self.workspace = workspace if workspace is not None else make_workspace(self.B, self.V,
                                                                                dev)
        self.allowed = allowed
        self.off = None if allowed is None else np.ascontiguousarray(allowed_off, dtype=np.int64)
        self.stream = stream
        self._args = None

    def __call__(self):
        if self._args is None:
            self._args = [
                None, self.B, self.V, self.ld, None, self.top_n, _ptr(self.allowed),
                None if self.off is None else self.off.ctypes.data_as(ctypes.c_void_p),
                _ptr(self.token_lp), _ptr(self.top_ids) if self.top_n > 0 else None,
                _ptr(self.top_lp) if self.top_n > 0 else None, _ptr(self.workspace),
                self.workspace.numel(), None]
        a = self._args
        a[0] = self.logits.data_ptr()
        a[4] = self.tokens.data_ptr()
        a[13] = _stream_handle(self.stream)
        _check(lib().rts_token_logprobs(*a))
        return self

    def results(self) -> dict:
        return dict(token_lp=self.token_lp, top_ids=self.top_ids, top_lp=self.top_lp)


def token_logprobs(logits, tokens, top_n: int, allowed=None, allowed_off=None,
                   workspace=None, stream=None) -> dict:
    """Raw-logit log-softmax per row: token_lp[B], top_ids[B][top_n],
    top_lp[B][top_n].  allowed: CUDA int32 ids with host int64 offsets [B+1]."""
    return LogprobCall(logits, tokens, top_n, allowed, allowed_off, workspace,
                       stream)().results()


class PriorCall(SampleCall):
    """One prepared call of rts_sample_tokens_prior: the pages' earlier designs
    (PRIOR_THREAD, PRIOR_BLOCK, PRIOR_RECOUNT) over the same arguments, with
    the same outputs as SampleCall, for measurement against it."""

    def __init__(self, design, logits, params, history=None, history_len=None, workspace=None,
                 stream=None):
        super().__init__(logits, params, history, history_len, workspace, stream)
        self.design = int(design)

    def __call__(self):
        hl = None if self.hist_len is None else self.hist_len.ctypes.data_as(ctypes.c_void_p)
        _check(lib().rts_sample_tokens_prior(
            self.design, self.logits.data_ptr(), self.B, self.V, self.ld, self.params,
            _ptr(self.history), self.H, self.ldh, hl, _ptr(self.token), _ptr(self.counts),
            _ptr(self.kept_ids), _ptr(self.kept_logits), _ptr(self.philox_x0),
            _ptr(self.workspace), self.workspace.numel(), _stream_handle(self.stream)))
        return self


class ReadCall:
    """One prepared call of rts_read_rows, the plain streaming read of the
    rows used as the sampler's bandwidth measuring stick."""

    def __init__(self, logits, stream=None):
        self.logits, self.B, self.V, self.ld = _rows_view(logits)
        self.chunk_max = torch.full((self.B, (self.V + 1023) // 1024), float("nan"),
                                    dtype=torch.float32, device=self.logits.device)
        self.stream = stream

    def __call__(self):
        _check(lib().rts_read_rows(self.logits.data_ptr(), self.B, self.V, self.ld,
                                   self.chunk_max.data_ptr(), _stream_handle(self.stream)))
        return self


__all__ = ["sample_tokens", "sample_tokens_noalloc", "noalloc_scratch_bytes", "token_logprobs", "SampleCall", "LogprobCall", "workspace_bytes",
           "make_workspace", "row_params", "RowParams", "LogprobRequest", "SampleExtras", "ReadCall",
           "PriorCall",
           "RTSError",
           "lib"]
