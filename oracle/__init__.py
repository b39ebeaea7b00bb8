"""CPU oracle for the DSpark draft / confidence / schedule / verify path.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
CPU-baseline leg of bench.py, never by the product package.  It shares no
code with the HIP library.  The arithmetic lives in dsp_oracle.c (plain C,
fp64, single thread); this module only marshals numpy arrays through ctypes.

Every function takes compact per-request arrays (n requests) plus `req_id`,
the request index that keys the Philox counter, so a sample of requests of a
large workload can be checked one by one.
"""
from __future__ import annotations

import ctypes as C

import numpy as np

from .build import ensure_built

_lib = None

DT_F32, DT_BF16 = 0, 1


def lib():
    global _lib
    if _lib is None:
        _lib = C.CDLL(ensure_built())
        P = C.c_void_p
        _lib.orc_philox4x32_10.argtypes = [P, P, P]
        _lib.orc_uniform.argtypes = [C.c_uint64, C.c_uint32, C.c_uint32, C.c_uint32, C.c_uint32]
        _lib.orc_uniform.restype = C.c_double
        _lib.orc_markov_logits.argtypes = [C.c_int, C.c_int, P, C.c_int, P, P, C.c_int, P, P]
        _lib.orc_softmax.argtypes = [C.c_int, P, C.c_double, P, P]
        _lib.orc_inverse_cdf.argtypes = [C.c_int, P, C.c_double, C.c_double, P]
        _lib.orc_draft.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, P, C.c_int, P, P, P, P,
                                   C.c_double, C.c_uint64, C.c_uint32, P, P, P, P, P, P, P, P]
        _lib.orc_confidence.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, P, P, P, P,
                                        P, P, P, P, P]
        _lib.orc_schedule.argtypes = [C.c_int, C.c_int, P, P, C.c_int, C.c_double, C.c_int,
                                      P, P, P, P]
        _lib.orc_verify.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, P, P, C.c_int, P, P,
                                    P, P, P, P, P, C.c_double, C.c_uint64, C.c_uint32,
                                    P, P, P, P, P, P, P, P]
        _lib.orc_schedule_async.argtypes = [C.c_int, C.c_int, P, P, P, C.c_int, C.c_double, P, P,
                                            P, P]
        _lib.orc_tv_accept.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, P, P, C.c_int, P, P, P,
                                       P, C.c_double, P, P]
        _lib.orc_rnn_state.argtypes = [C.c_int, C.c_int, P, P, C.c_int, P, P, P]
        _lib.orc_confidence_logit.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, P, P,
                                              P, P, P, P, P]
        _lib.orc_sts_fit.argtypes = [C.c_int, C.c_int, P, P, C.c_double, C.c_double, C.c_int, P,
                                     P, P]
        _lib.orc_ece.argtypes = [C.c_int, C.c_int, P, P, P, C.c_int, P, P]
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _logits(a):
    """Logit arrays: float32 as is, bf16 passed as its uint16 bit patterns."""
    if a.dtype == np.float32:
        return np.ascontiguousarray(a), DT_F32
    if a.dtype == np.uint16:
        return np.ascontiguousarray(a), DT_BF16
    raise TypeError(f"logits must be float32 or bf16 bits (uint16), got {a.dtype}")


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def philox4x32_10(ctr, key):
    ctr = _c(ctr, np.uint32)
    key = _c(key, np.uint32)
    out = np.zeros(4, np.uint32)
    lib().orc_philox4x32_10(_p(ctr), _p(key), _p(out))
    return out


def uniform(seed, rnd, req, pos, purpose) -> float:
    return lib().orc_uniform(seed, rnd, req, pos, purpose)


def markov_logits(base_row, E, W2, prev):
    base_row, dt = _logits(base_row)
    E = _c(E, np.uint16)
    W2 = _c(W2, np.uint16)
    V, r = E.shape
    out = np.zeros(V, np.float32)
    absdot = np.zeros(V, np.float64)
    _check(lib().orc_markov_logits(V, r, _p(base_row), dt, _p(E), _p(W2), int(prev),
                                   _p(out), _p(absdot)), "markov_logits")
    return out, absdot


def softmax(logit, temperature):
    logit = _c(logit, np.float32)
    prob = np.zeros(logit.shape[0], np.float64)
    stats = np.zeros(2, np.float64)
    _check(lib().orc_softmax(logit.shape[0], _p(logit), float(temperature), _p(prob),
                             _p(stats)), "softmax")
    return prob, stats


def inverse_cdf(w, u, window=1e-6):
    w = _c(w, np.float64)
    near = C.c_int(0)
    x = lib().orc_inverse_cdf(w.shape[0], _p(w), float(u), float(window), C.byref(near))
    return x, bool(near.value)


def draft(base, E, W2, anchor, req_id, temperature, seed, rnd, force=None, A=None):
    """base [n, gamma, V] (float32 or bf16 bits).  Returns tok, q, stats, flag.
    force [n, gamma] int32 (optional): tokens >= 0 taken instead of the oracle's
    own draw at those positions (teacher forcing at a flagged decision).
    A [r, r] bf16 bits (optional): the recurrent head with that matrix; the
    result then also holds the states S [n, gamma, r] (bf16 bits) and sflag
    [n, gamma] (a state element near a bf16 rounding midpoint)."""
    base, dt = _logits(base)
    n, gamma, V = base.shape
    E = _c(E, np.uint16)
    W2 = _c(W2, np.uint16)
    r = E.shape[1]
    anchor = _c(anchor, np.int32)
    req_id = _c(req_id, np.int32)
    tok = np.zeros((n, gamma), np.int32)
    q = np.zeros((n, gamma), np.float64)
    stats = np.zeros((n, gamma, 2), np.float64)
    flag = np.zeros((n, gamma), np.int8)
    force = None if force is None else _c(force, np.int32)
    S = sflag = None
    if A is not None:
        A = _c(A, np.uint16)
        assert A.shape == (r, r)
        S = np.zeros((n, gamma, r), np.uint16)
        sflag = np.zeros((n, gamma), np.int8)
    _check(lib().orc_draft(n, gamma, V, r, _p(base), dt, _p(E), _p(W2), _p(anchor), _p(req_id),
                           float(temperature), int(seed), int(rnd), _p(tok), _p(q), _p(stats),
                           _p(flag), _p(force), _p(A), _p(S), _p(sflag)), "draft")
    if A is not None:
        return tok, q, stats, flag, S, sflag
    return tok, q, stats, flag


def rnn_state(A, E, prev, s_prev=None):
    """One step of the recurrent head: bf16(tanh(A s_prev + E[prev])); (state, flag)."""
    A = _c(A, np.uint16)
    E = _c(E, np.uint16)
    V, r = E.shape
    out = np.zeros(r, np.uint16)
    fl = np.zeros(1, np.int8)
    _check(lib().orc_rnn_state(V, r, _p(A), _p(E), int(prev),
                               _p(None if s_prev is None else _c(s_prev, np.uint16)), _p(out),
                               _p(fl)), "rnn_state")
    return out, bool(fl[0])


def confidence(h, E, anchor, tok, w, T, offset=None):
    h = _c(h, np.uint16)
    n, gamma, d = h.shape
    E = _c(E, np.uint16)
    V, r = E.shape
    anchor = _c(anchor, np.int32)
    tok = _c(tok, np.int32)
    w = _c(w, np.float32)
    T = _c(T, np.float32)
    offset = None if offset is None else _c(offset, np.float32)
    c = np.zeros((n, gamma), np.float64)
    flag = np.zeros((n, gamma), np.int8)
    _check(lib().orc_confidence(n, gamma, d, V, r, _p(h), _p(E), _p(anchor), _p(tok), _p(w),
                                _p(T), _p(offset), _p(c), _p(flag)), "confidence")
    return c, flag


def confidence_logit(h, E, anchor, tok, w, offset=None):
    """y [n, gamma] fp64: the confidence head's sigmoid argument before temperature."""
    h = _c(h, np.uint16)
    n, gamma, d = h.shape
    E = _c(E, np.uint16)
    V, r = E.shape
    y = np.zeros((n, gamma), np.float64)
    _check(lib().orc_confidence_logit(n, gamma, d, V, r, _p(h), _p(E), _p(_c(anchor, np.int32)),
                                      _p(_c(tok, np.int32)), _p(_c(w, np.float32)),
                                      _p(None if offset is None else _c(offset, np.float32)),
                                      _p(y)), "confidence_logit")
    return y


STS_GRID = 256


def sts_fit(z, acc, t_lo=1.0 / 16, t_hi=16.0, G=STS_GRID):
    """Sequential temperature scaling on held-out (z [N, gamma] f32, acc [N]).

    t_lo and t_hi bound the temperature grid; a comparison with a caller that
    receives them as fp32 passes the fp32-rounded values.  Returns beta [gamma]
    (fp64 grid points), T = fp32(1 / beta), the final objective nll [gamma] and
    the relative objective gaps [gamma, 2] between the best and second-best
    point of each grid stage."""
    z = _c(z, np.float32)
    N, gamma = z.shape
    acc = _c(acc, np.int32)
    beta = np.zeros(gamma, np.float64)
    nll = np.zeros(gamma, np.float64)
    gap = np.zeros((gamma, 2), np.float64)
    _check(lib().orc_sts_fit(N, gamma, _p(z), _p(acc), float(t_lo), float(t_hi), int(G), _p(beta),
                             _p(nll), _p(gap)), "sts_fit")
    T = (1.0 / beta).astype(np.float32)
    return beta, T, nll, gap


def ece(z, acc, T=None, M=15):
    """Expected calibration error of the cumulative survival; returns (ece, n_edge)."""
    z = _c(z, np.float32)
    N, gamma = z.shape
    out = np.zeros(1, np.float64)
    edge = np.zeros(1, np.int32)
    _check(lib().orc_ece(N, gamma, _p(z), _p(_c(acc, np.int32)),
                         _p(None if T is None else _c(T, np.float32)), int(M), _p(out), _p(edge)),
           "ece")
    return float(out[0]), int(edge[0])


def schedule(c32, sps, B_max, tau0, mode):
    """c32 [R, gamma] float32.  Returns len [R], a [R, gamma] float32, B, evals."""
    c32 = _c(c32, np.float32)
    R, gamma = c32.shape
    sps = _c(sps, np.float32)
    length = np.zeros(R, np.int32)
    a = np.zeros((R, gamma), np.float32)
    B = np.zeros(1, np.int32)
    ev = np.zeros(1, np.int32)
    _check(lib().orc_schedule(R, gamma, _p(c32), _p(sps), int(B_max), float(tau0), int(mode),
                              _p(length), _p(a), _p(B), _p(ev)), "schedule")
    return length, a, int(B[0]), int(ev[0])


def schedule_async(c32, c_hist32, sps, B_max, tau0):
    """Capacity K from the earlier round's confidences (global maximum of Theta, no
    early stop), the first K of the current candidates admitted.  Returns len [R],
    a [R, gamma] (current survival), B, K."""
    c32 = _c(c32, np.float32)
    ch = _c(c_hist32, np.float32)
    R, gamma = c32.shape
    sps = _c(sps, np.float32)
    length = np.zeros(R, np.int32)
    a = np.zeros((R, gamma), np.float32)
    B = np.zeros(1, np.int32)
    K = np.zeros(1, np.int32)
    _check(lib().orc_schedule_async(R, gamma, _p(c32), _p(ch), _p(sps), int(B_max), float(tau0),
                                    _p(length), _p(a), _p(B), _p(K)), "schedule_async")
    return length, a, int(B[0]), int(K[0])


def verify(target, base, E, W2, anchor, tok, q, length, req_id, temperature, seed, rnd,
           force_acc=None, S=None):
    """force_acc [n, gamma] int8 (optional): 0/1 adopted as the accept decision at
    those positions, -1 elsewhere (teacher forcing at a flagged accept test).
    S [n, gamma, r] bf16 bits (optional): the recurrent head's states, whose row
    gives the draft law at a rejection instead of E[prev]."""
    target, dt = _logits(target)
    base, dt2 = _logits(base)
    assert dt == dt2
    n, g1, V = target.shape
    gamma = g1 - 1
    E = _c(E, np.uint16)
    W2 = _c(W2, np.uint16)
    r = E.shape[1]
    anchor = _c(anchor, np.int32)
    tok = _c(tok, np.int32)
    q = _c(q, np.float64)
    length = _c(length, np.int32)
    req_id = _c(req_id, np.int32)
    accept = np.zeros((n, gamma), np.int8)
    n_acc = np.zeros(n, np.int32)
    y = np.zeros(n, np.int32)
    p = np.zeros((n, gamma), np.float64)
    fa = np.zeros((n, gamma), np.int8)
    fy = np.zeros(n, np.int8)
    force_acc = None if force_acc is None else _c(force_acc, np.int8)
    _check(lib().orc_verify(n, gamma, V, r, _p(target), _p(base), dt, _p(E), _p(W2),
                            _p(anchor), _p(tok), _p(q), _p(length), _p(req_id),
                            float(temperature), int(seed), int(rnd), _p(accept), _p(n_acc),
                            _p(y), _p(p), _p(fa), _p(fy), _p(force_acc),
                            _p(None if S is None else _c(S, np.uint16))), "verify")
    return dict(accept=accept, n_accept=n_acc, y=y, p=p, flag_acc=fa, flag_y=fy)


def tv_accept(target, base, E, W2, anchor, tok, temperature, S=None):
    """alpha [n, gamma]: the exact acceptance probability sum_v min(q_k, p_k) of
    every draft position (target [n, gamma+1, V], base [n, gamma, V])."""
    target, dt = _logits(target)
    base, dt2 = _logits(base)
    assert dt == dt2
    n, g1, V = target.shape
    gamma = g1 - 1
    E = _c(E, np.uint16)
    W2 = _c(W2, np.uint16)
    r = E.shape[1]
    anchor = _c(anchor, np.int32)
    tok = _c(tok, np.int32)
    alpha = np.zeros((n, gamma), np.float64)
    _check(lib().orc_tv_accept(n, gamma, V, r, _p(target), _p(base), dt, _p(E), _p(W2),
                               _p(anchor), _p(tok), float(temperature), _p(alpha),
                               _p(None if S is None else _c(S, np.uint16))), "tv_accept")
    return alpha


def bf16_bits(t):
    """uint16 view of a torch bf16 tensor (any device), as a host numpy array."""
    import torch
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def host_logits(t):
    import torch
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    return t.detach().to("cpu").contiguous().numpy().astype(np.float32, copy=False)


def run_round(inp: dict, temperature: float, seed: int, rnd: int, mode=None, tau0=None):
    """The whole path for one round over every request of a (small) input set."""
    R = inp["R"]
    req = np.arange(R, dtype=np.int32)
    base = host_logits(inp["base"])
    target = host_logits(inp["target"])
    E = bf16_bits(inp["E"])
    W2 = bf16_bits(inp["W2"])
    anchor = inp["anchor"].cpu().numpy()
    tok, q, stats, fdraft = draft(base, E, W2, anchor, req, temperature, seed, rnd)
    off = None if inp["offset"] is None else inp["offset"].cpu().numpy()
    c, fconf = confidence(bf16_bits(inp["h"]), E, anchor, tok, inp["w"].cpu().numpy(),
                          inp["T"].cpu().numpy(), off)
    c32 = c.astype(np.float32)
    mode = inp["mode"] if mode is None else mode
    tau0 = inp["tau0"] if tau0 is None else tau0
    length, a, B, _ = schedule(c32, inp["sps"].cpu().numpy(), inp["B_max"], tau0, mode)
    ver = verify(target, base, E, W2, anchor, tok, q, length, req, temperature, seed, rnd)
    return dict(tok=tok, q=q, stats=stats, flag_draft=fdraft, c=c, c32=c32, flag_conf=fconf,
                len=length, a=a, B=B, **ver)
