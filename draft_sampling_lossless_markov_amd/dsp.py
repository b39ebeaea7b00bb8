"""ctypes binding of libdsp.so -- argument marshalling only.

The functions carry the C-ABI names (include/dsp.h).  They take torch tensors
that already live on the GPU, pass their data pointers and the current HIP
stream, and raise DspError on a non-OK status.  Every step of the path runs in
the HIP kernels of libdsp.so; there is no fallback: if the library is missing
the first call raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdsp.so")

(DSP_OK, DSP_ERR_INVALID_ARG, DSP_ERR_UNSUPPORTED, DSP_ERR_WORKSPACE, DSP_ERR_HIP,
 DSP_ERR_TIMEOUT) = range(6)
_STATUS_NAMES = ("DSP_OK", "DSP_ERR_INVALID_ARG", "DSP_ERR_UNSUPPORTED", "DSP_ERR_WORKSPACE",
                 "DSP_ERR_HIP", "DSP_ERR_TIMEOUT")
DSP_F32, DSP_BF16 = 0, 1
DSP_WS_DRAFT, DSP_WS_VERIFY, DSP_WS_TV, DSP_WS_STS, DSP_WS_ECE = 0, 1, 2, 3, 4
DSP_PATH_AUTO, DSP_PATH_STREAMING, DSP_PATH_PERSISTENT = 0, 1, 2
DSP_FLAG_TEST_GIVE_UP = 0x100

EXPORTED = ("dsp_status_string", "dsp_last_error", "dsp_version", "dsp_workspace_size",
            "dsp_workspace_status", "dsp_draft_step", "dsp_draft_step_noalloc", "dsp_confidence",
            "dsp_schedule", "dsp_schedule_async", "dsp_verify", "dsp_tv_accept",
            "dsp_confidence_logit", "dsp_sts_fit", "dsp_ece", "dsp_draft_step_rnn",
            "dsp_verify_rnn", "dsp_tv_accept_rnn")

_lib = None


class DspError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_status_name(status)}: {detail}")
        self.status = status


def _status_name(s):
    return _STATUS_NAMES[s] if 0 <= s < len(_STATUS_NAMES) else f"status {s}"


def lib():
    """Load libdsp.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m draft_sampling_lossless_markov_amd.build`")
    L = C.CDLL(LIB_PATH)
    P, I, U64, U32, F, D, SZ = (C.c_void_p, C.c_int, C.c_uint64, C.c_uint32, C.c_float,
                                C.c_double, C.c_size_t)
    L.dsp_status_string.argtypes = [I]
    L.dsp_status_string.restype = C.c_char_p
    L.dsp_last_error.argtypes = []
    L.dsp_last_error.restype = C.c_char_p
    L.dsp_version.restype = I
    L.dsp_workspace_size.argtypes = [I, I, I, I, I]
    L.dsp_workspace_size.restype = SZ
    L.dsp_workspace_status.argtypes = [I, P, SZ, I, I, I, I, P]
    L.dsp_workspace_status.restype = I
    I64 = C.c_int64
    L.dsp_draft_step.argtypes = [P, I, I64, I64, P, P, P, P, P, P, I, I, I, I, I, I, U32, F, U64,
                                 U32, P, SZ, P]
    L.dsp_draft_step_noalloc.argtypes = [P, I, I64, I64, P, P, P, P, P, P, I, I, I, I, I, I, U32,
                                         F, U64, U32, P]
    L.dsp_confidence.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, P]
    L.dsp_schedule.argtypes = [P, P, I, D, I, P, P, P, I, I, P]
    L.dsp_verify.argtypes = [P, I64, I64, P, I64, I64, I, P, P, P, P, P, P, P, P, P, P, P, I, I,
                             I, I, U32, F, U64, U32, P, SZ, P]
    L.dsp_schedule_async.argtypes = [P, P, P, I, D, P, P, P, P, I, I, P]
    L.dsp_tv_accept.argtypes = [P, I64, I64, P, I64, I64, I, P, P, P, P, P, P, I, I, I, I, F, P, SZ, P]
    L.dsp_confidence_logit.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, P]
    L.dsp_draft_step_rnn.argtypes = [P, I, I64, I64, P, P, P, P, P, P, P, P, I, I, I, I, I, I, U32,
                                     F, U64, U32, P, SZ, P]
    L.dsp_verify_rnn.argtypes = [P, I64, I64, P, I64, I64, I, P, P, P, P, P, P, P, P, P, P, P, P,
                                 I, I, I, I, U32, F, U64, U32, P, SZ, P]
    L.dsp_tv_accept_rnn.argtypes = [P, I64, I64, P, I64, I64, I, P, P, P, P, P, P, P, I, I, I, I, F,
                                    P, SZ, P]
    L.dsp_sts_fit.argtypes = [P, P, I, I, F, F, P, P, P, SZ, P]
    L.dsp_ece.argtypes = [P, P, P, I, I, I, P, P, SZ, P]
    for f in ("dsp_draft_step", "dsp_draft_step_noalloc", "dsp_confidence", "dsp_schedule",
              "dsp_schedule_async", "dsp_verify", "dsp_tv_accept", "dsp_confidence_logit",
              "dsp_sts_fit", "dsp_ece", "dsp_draft_step_rnn", "dsp_verify_rnn",
              "dsp_tv_accept_rnn"):
        getattr(L, f).restype = I
    _lib = L
    return L


def _check(status):
    if status != DSP_OK:
        raise DspError(status, lib().dsp_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DSP_F32
    if t.dtype == torch.bfloat16:
        return DSP_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _rows(t: torch.Tensor, name: str):
    """(request stride, position stride) of a logit tensor viewed as [R, positions, V]."""
    if t.dim() != 3 or (t.shape[2] > 1 and t.stride(2) != 1):
        raise ValueError(f"{name} must be a 3-D [R, positions, V] view with contiguous rows")
    return t.stride(0), t.stride(1)


def dsp_workspace_size(which: int, R: int, gamma: int, V: int, r: int) -> int:
    return int(lib().dsp_workspace_size(which, R, gamma, V, r))


def dsp_workspace_status(which: int, ws, R: int, gamma: int, V: int, r: int, stream=None):
    """Wait for the stream; raise DspError(DSP_ERR_TIMEOUT) if a bounded wait of the
    last call on workspace ws gave up (its outputs are then undefined)."""
    _check(lib().dsp_workspace_status(int(which), _ptr(ws), ws.numel() * ws.element_size(), R,
                                      gamma, V, r, _stream(stream)))


def dsp_draft_step(base, E, W2, anchor, tok, q, stats, k, temperature, seed, round_, ws,
                   stream=None, n_steps=1, flags=DSP_PATH_AUTO):
    """Draft positions k .. k + n_steps - 1 of every request; flags selects the
    implementation (DSP_PATH_AUTO, DSP_PATH_STREAMING or DSP_PATH_PERSISTENT)."""
    R, gamma, V = base.shape
    r = E.shape[1]
    rs, ps = _rows(base, "base")
    _check(lib().dsp_draft_step(_ptr(base), _dtype(base), rs, ps, _ptr(E), _ptr(W2), _ptr(anchor),
                                _ptr(tok), _ptr(q), _ptr(stats), R, gamma, V, r, int(k),
                                int(n_steps), int(flags), float(temperature), int(seed), int(round_),
                                _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def dsp_draft_step_rnn(base, E, W2, A, anchor, tok, q, stats, S, k, temperature, seed, round_, ws,
                       stream=None, n_steps=1, flags=DSP_PATH_AUTO):
    """dsp_draft_step with the recurrent head: A [r, r] bf16, states S [R, gamma, r] bf16."""
    R, gamma, V = base.shape
    r = E.shape[1]
    rs, ps = _rows(base, "base")
    _check(lib().dsp_draft_step_rnn(_ptr(base), _dtype(base), rs, ps, _ptr(E), _ptr(W2), _ptr(A),
                                    _ptr(anchor), _ptr(tok), _ptr(q), _ptr(stats), _ptr(S), R, gamma,
                                    V, r, int(k), int(n_steps), int(flags), float(temperature),
                                    int(seed), int(round_), _ptr(ws), ws.numel() * ws.element_size(),
                                    _stream(stream)))


def dsp_draft_step_noalloc(base, E, W2, anchor, tok, q, stats, k, temperature, seed, round_,
                           stream=None, n_steps=1, flags=DSP_PATH_AUTO):
    """dsp_draft_step without a workspace (the library's static per-device scratch)."""
    R, gamma, V = base.shape
    r = E.shape[1]
    rs, ps = _rows(base, "base")
    _check(lib().dsp_draft_step_noalloc(_ptr(base), _dtype(base), rs, ps, _ptr(E), _ptr(W2),
                                        _ptr(anchor), _ptr(tok), _ptr(q), _ptr(stats), R, gamma, V,
                                        r, int(k), int(n_steps), int(flags), float(temperature),
                                        int(seed), int(round_), _stream(stream)))


def dsp_confidence(h, E, anchor, tok, w, T, offset, c, stream=None):
    R, gamma, d = h.shape
    V, r = E.shape
    _check(lib().dsp_confidence(_ptr(h), _ptr(E), _ptr(anchor), _ptr(tok), _ptr(w), _ptr(T),
                                _ptr(offset), _ptr(c), R, gamma, d, V, r, _stream(stream)))


def dsp_confidence_logit(h, E, anchor, tok, w, offset, y, stream=None):
    R, gamma, d = h.shape
    V, r = E.shape
    _check(lib().dsp_confidence_logit(_ptr(h), _ptr(E), _ptr(anchor), _ptr(tok), _ptr(w),
                                      _ptr(offset), _ptr(y), R, gamma, d, V, r, _stream(stream)))


def dsp_sts_fit(z, n_acc, t_lo, t_hi, T, nll, ws, stream=None):
    """z [N, gamma] f32, n_acc [N] int32 -> T [gamma] f32, nll [gamma] f64 (or None)."""
    N, gamma = z.shape
    _check(lib().dsp_sts_fit(_ptr(z), _ptr(n_acc), N, gamma, float(t_lo), float(t_hi), _ptr(T),
                             _ptr(nll), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def dsp_ece(z, n_acc, T, n_bins, ece, ws, stream=None):
    """Calibration error of the cumulative survival into ece [1] f64 (T None: all 1)."""
    N, gamma = z.shape
    _check(lib().dsp_ece(_ptr(z), _ptr(n_acc), _ptr(T), N, gamma, int(n_bins), _ptr(ece),
                         _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def dsp_schedule(c, sps, B_max, tau0, mode, length, a, B, stream=None):
    R, gamma = c.shape
    _check(lib().dsp_schedule(_ptr(c), _ptr(sps), int(B_max), float(tau0), int(mode),
                              _ptr(length), _ptr(a), _ptr(B), R, gamma, _stream(stream)))


def dsp_schedule_async(c, c_hist, sps, B_max, tau0, length, a, B, K, stream=None):
    R, gamma = c.shape
    _check(lib().dsp_schedule_async(_ptr(c), _ptr(c_hist), _ptr(sps), int(B_max), float(tau0),
                                    _ptr(length), _ptr(a), _ptr(B), _ptr(K), R, gamma,
                                    _stream(stream)))


def dsp_verify(target, base, E, W2, anchor, tok, q, stats, length, accept, n_accept, y, p,
               temperature, seed, round_, ws, stream=None, flags=DSP_PATH_AUTO):
    R, g1, V = target.shape
    r = E.shape[1]
    trs, tps = _rows(target, "target")
    brs, bps = _rows(base, "base")
    if base.dtype != target.dtype:
        raise TypeError("base and target logits must share a dtype")
    _check(lib().dsp_verify(_ptr(target), trs, tps, _ptr(base), brs, bps, _dtype(target),
                            _ptr(E), _ptr(W2),
                            _ptr(anchor), _ptr(tok), _ptr(q), _ptr(stats), _ptr(length),
                            _ptr(accept), _ptr(n_accept), _ptr(y), _ptr(p), R, g1 - 1, V, r,
                            int(flags), float(temperature), int(seed), int(round_), _ptr(ws),
                            ws.numel() * ws.element_size(), _stream(stream)))


def dsp_verify_rnn(target, base, E, W2, S, anchor, tok, q, stats, length, accept, n_accept, y, p,
                   temperature, seed, round_, ws, stream=None, flags=DSP_PATH_AUTO):
    """dsp_verify after dsp_draft_step_rnn (S [R, gamma, r] bf16: the draft's states)."""
    R, g1, V = target.shape
    r = E.shape[1]
    trs, tps = _rows(target, "target")
    brs, bps = _rows(base, "base")
    if base.dtype != target.dtype:
        raise TypeError("base and target logits must share a dtype")
    _check(lib().dsp_verify_rnn(_ptr(target), trs, tps, _ptr(base), brs, bps, _dtype(target),
                                _ptr(E), _ptr(W2), _ptr(S), _ptr(anchor), _ptr(tok), _ptr(q),
                                _ptr(stats), _ptr(length), _ptr(accept), _ptr(n_accept), _ptr(y),
                                _ptr(p), R, g1 - 1, V, r, int(flags), float(temperature), int(seed),
                                int(round_), _ptr(ws), ws.numel() * ws.element_size(),
                                _stream(stream)))


def dsp_tv_accept_rnn(target, base, E, W2, S, anchor, tok, stats, alpha, temperature, ws,
                      stream=None):
    """dsp_tv_accept for the recurrent head's draft (S: its states)."""
    R, g1, V = target.shape
    r = E.shape[1]
    trs, tps = _rows(target, "target")
    brs, bps = _rows(base, "base")
    if base.dtype != target.dtype:
        raise TypeError("base and target logits must share a dtype")
    _check(lib().dsp_tv_accept_rnn(_ptr(target), trs, tps, _ptr(base), brs, bps, _dtype(target),
                                   _ptr(E), _ptr(W2), _ptr(S), _ptr(anchor), _ptr(tok), _ptr(stats),
                                   _ptr(alpha), R, g1 - 1, V, r, float(temperature), _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(stream)))


def dsp_tv_accept(target, base, E, W2, anchor, tok, stats, alpha, temperature, ws, stream=None):
    """alpha [R, gamma] (f64): sum_v min(q_k, p_k) of every draft position."""
    R, g1, V = target.shape
    r = E.shape[1]
    trs, tps = _rows(target, "target")
    brs, bps = _rows(base, "base")
    if base.dtype != target.dtype:
        raise TypeError("base and target logits must share a dtype")
    _check(lib().dsp_tv_accept(_ptr(target), trs, tps, _ptr(base), brs, bps, _dtype(target),
                               _ptr(E), _ptr(W2), _ptr(anchor), _ptr(tok), _ptr(stats), _ptr(alpha),
                               R, g1 - 1, V, r, float(temperature), _ptr(ws),
                               ws.numel() * ws.element_size(), _stream(stream)))
