"""Element-by-element comparison of HIP-path outputs with the oracle's.

TEST INFRASTRUCTURE ONLY (tests/, the smoke check).  Parity rules:
  - integer outputs (tokens, accept bits, lengths, B) identical, except at a
    decision the oracle flags as within rounding reach of a boundary (u within
    1e-6 of a boundary of its fp64 CDF, |u - p/q| < 1e-6, a greedy near-tie, a
    confidence next to an fp32 rounding midpoint).  A differing decision outside
    that window is an error; inside it, it is a counted mismatch, and the rest of
    that request's chain is not compared;
  - probabilities (q, p) and normalisers within 1e-5 relative (fp32 path vs fp64
    oracle); confidences bit-identical after fp32 rounding unless flagged.
Tally counts decisions, flagged decisions (the window, a property of the
oracle's CDF and u alone) and mismatches (flagged decisions that differ).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

RTOL = 1e-5


@dataclass
class Tally:
    decisions: int = 0
    flagged: int = 0
    diverged: int = 0      # mismatched decisions (all inside the window)
    skipped: int = 0       # comparisons skipped downstream of a mismatch
    errors: list = field(default_factory=list)

    def add(self, other: "Tally"):
        self.decisions += other.decisions
        self.flagged += other.flagged
        self.diverged += other.diverged
        self.skipped += other.skipped
        self.errors += other.errors
        return self

    def ok(self):
        return not self.errors

    def flag_rate(self):
        return self.flagged / max(1, self.decisions)

    def mismatch_rate(self):
        return self.diverged / max(1, self.decisions)

    def summary(self):
        return (f"decisions={self.decisions} flagged={self.flagged} mismatched={self.diverged} "
                f"skipped={self.skipped} errors={len(self.errors)} first={self.errors[:5]}")


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.abs(a - b) / np.maximum(np.abs(b), 1e-30)


def compare_draft(g_tok, g_q, g_stats, o_tok, o_q, o_stats, o_flag, greedy, req_ids=None):
    """Walk each request's chain; returns (Tally, diverged_at[n]) where
    diverged_at[i] is the first position whose token differs (gamma if none)."""
    t = Tally()
    n, gamma = o_tok.shape
    diverged_at = np.full(n, gamma, np.int64)
    rid = np.arange(n) if req_ids is None else np.asarray(req_ids)
    for i in range(n):
        for k in range(gamma):
            t.decisions += 1
            t.flagged += int(o_flag[i, k])
            if g_tok[i, k] != o_tok[i, k]:
                if o_flag[i, k]:
                    t.diverged += 1
                    diverged_at[i] = k
                    break
                t.errors.append(("draft token", int(rid[i]), k, int(g_tok[i, k]), int(o_tok[i, k])))
                diverged_at[i] = k
                break
            if greedy:
                if g_q[i, k] != 1.0:
                    t.errors.append(("greedy q", int(rid[i]), k, float(g_q[i, k])))
            else:
                if _rel(g_q[i, k], o_q[i, k]) > RTOL:
                    t.errors.append(("q", int(rid[i]), k, float(g_q[i, k]), float(o_q[i, k])))
                if _rel(g_stats[i, k, 1], o_stats[i, k, 1]) > RTOL:
                    t.errors.append(("Z", int(rid[i]), k, float(g_stats[i, k, 1]),
                                     float(o_stats[i, k, 1])))
            if abs(float(g_stats[i, k, 0]) - o_stats[i, k, 0]) > RTOL * max(1.0, abs(o_stats[i, k, 0])):
                t.errors.append(("M", int(rid[i]), k, float(g_stats[i, k, 0]), float(o_stats[i, k, 0])))
    return t, diverged_at


def compare_confidence(g_c, o_c, o_flag, valid=None):
    """g_c float32; o_c float64.  Bit-identical after rounding unless flagged."""
    t = Tally()
    o32 = o_c.astype(np.float32)
    mask = np.ones(o_c.shape, bool) if valid is None else valid
    t.decisions = int(mask.sum())
    t.flagged = int((o_flag.astype(bool) & mask).sum())
    bad = (g_c.view(np.uint32) != o32.view(np.uint32)) & mask & ~o_flag.astype(bool)
    for i, k in zip(*np.nonzero(bad)):
        t.errors.append(("c", int(i), int(k), float(g_c[i, k]), float(o_c[i, k])))
    return t


def compare_schedule(g_len, g_a, g_B, o_len, o_a, o_B):
    t = Tally(decisions=len(o_len))
    if not np.array_equal(g_a.view(np.uint32), o_a.view(np.uint32)):
        idx = np.argwhere(g_a.view(np.uint32) != o_a.view(np.uint32))[:3]
        t.errors.append(("a", idx.tolist()))
    if not np.array_equal(g_len, o_len):
        idx = np.nonzero(g_len != o_len)[0][:5]
        t.errors.append(("len", idx.tolist(), g_len[idx].tolist(), o_len[idx].tolist()))
    if int(g_B) != int(o_B):
        t.errors.append(("B", int(g_B), int(o_B)))
    return t


def compare_verify(g, o, length, greedy, req_ids=None, skip=None):
    """g, o: dicts with accept [n, gamma], n_accept [n], y [n], p [n, gamma] (and the
    oracle's flag_acc, flag_y)."""
    t = Tally()
    n, gamma = o["accept"].shape
    rid = np.arange(n) if req_ids is None else np.asarray(req_ids)
    for i in range(n):
        if skip is not None and skip[i]:
            continue
        l = int(length[i])
        divergent = False
        for j in range(gamma):
            if j >= l:
                if g["accept"][i, j] != -1 or g["p"][i, j] != 0.0:
                    t.errors.append(("unverified slot", int(rid[i]), j))
                continue
            t.decisions += 1
            fl = bool(o["flag_acc"][i, j])
            t.flagged += int(fl)
            if g["accept"][i, j] != o["accept"][i, j]:
                if fl:
                    if j <= o["n_accept"][i]:
                        divergent = True
                else:
                    t.errors.append(("accept", int(rid[i]), j, int(g["accept"][i, j]),
                                     int(o["accept"][i, j])))
            if greedy:
                if g["p"][i, j] != o["p"][i, j]:
                    t.errors.append(("greedy p", int(rid[i]), j))
            elif _rel(g["p"][i, j], o["p"][i, j]) > RTOL:
                t.errors.append(("p", int(rid[i]), j, float(g["p"][i, j]), float(o["p"][i, j])))
        if divergent:
            t.diverged += 1
            continue
        if g["n_accept"][i] != o["n_accept"][i]:
            t.errors.append(("n_accept", int(rid[i]), int(g["n_accept"][i]), int(o["n_accept"][i])))
            continue
        t.decisions += 1
        fy = bool(o["flag_y"][i])
        t.flagged += int(fy)
        if g["y"][i] != o["y"][i]:
            if fy:
                t.diverged += 1
            else:
                t.errors.append(("y", int(rid[i]), int(g["y"][i]), int(o["y"][i]),
                                 int(o["n_accept"][i]), l))
    return t
