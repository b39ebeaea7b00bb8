"""Element-by-element comparison of HIP-path outputs with the oracle's.

TEST INFRASTRUCTURE ONLY (tests/, the smoke check).  Parity rules:
  - greedy tokens, accept bits and lengths identical, with no exception;
  - sampling: tokens and accept bits identical, except at a decision the oracle
    flags as within rounding reach of a boundary (u within 1e-6 of a boundary of
    its fp64 CDF, |u - p/q| < 1e-6) or a confidence next to an fp32 rounding
    midpoint.  A differing decision outside that window is an error; inside it,
    it is a counted mismatch, and the oracle then adopts the GPU's choice
    (teacher forcing) so that the rest of the chain is still compared;
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
                if o_flag[i, k] and not greedy:
                    t.diverged += 1
                    diverged_at[i] = k
                    break
                if greedy:
                    t.errors.append(("greedy token", int(rid[i]), k, int(g_tok[i, k]),
                                     int(o_tok[i, k]), bool(o_flag[i, k])))
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
    oracle's flag_acc, flag_y).  t.force lists the flagged, differing accept tests
    (row i, position j, the GPU's decision) for a teacher-forced re-run."""
    t = Tally()
    t.force = []
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
                if fl and not greedy:
                    if j <= o["n_accept"][i]:
                        divergent = True
                        t.force.append((i, j, int(g["accept"][i, j])))
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
            if fy and not greedy:
                t.diverged += 1
            else:
                t.errors.append(("y", int(rid[i]), int(g["y"][i]), int(o["y"][i]),
                                 int(o["n_accept"][i]), l))
    return t


# ---------------------------------------------------------------------------
# whole-round parity with teacher forcing
# ---------------------------------------------------------------------------

def _pmap(fn, items, threads):
    if threads <= 1 or len(items) <= 1:
        return [fn(x) for x in items]
    import concurrent.futures as cf
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(fn, items))


def draft_forced(g_tok, g_q, g_stats, oracle_rows, greedy, req_ids, threads=1):
    """Compare a GPU draft with the oracle's, request by request.  oracle_rows(i,
    force_row) runs the oracle draft for compact row i (force_row: [gamma] int32 or
    None) and returns (tok, q, stats, flag) of that row.  At a flagged sampling
    divergence the oracle is re-run with the GPU's token forced there, until the
    chain agrees or an unflagged difference is found.  Returns (Tally, o_tok, o_q,
    o_stats, o_flag) of the final (forced) oracle chain."""
    n, gamma = g_tok.shape
    rows = _pmap(lambda i: oracle_rows(i, None), list(range(n)), threads)
    force = np.full((n, gamma), -1, np.int32)
    forced = 0
    for _ in range(gamma):
        o_tok = np.stack([r[0] for r in rows])
        o_flag = np.stack([r[3] for r in rows])
        redo = []
        for i in range(n):
            for k in range(gamma):
                if g_tok[i, k] != o_tok[i, k]:
                    if o_flag[i, k] and not greedy and force[i, k] < 0:
                        force[i, k] = g_tok[i, k]
                        forced += 1
                        redo.append(i)
                    break
        if not redo:
            break
        new = _pmap(lambda i: oracle_rows(i, force[i]), redo, threads)
        for i, r in zip(redo, new):
            rows[i] = r
    o_tok = np.stack([r[0] for r in rows])
    o_q = np.stack([r[1] for r in rows])
    o_stats = np.stack([r[2] for r in rows])
    o_flag = np.stack([r[3] for r in rows])
    t, _ = compare_draft(g_tok, g_q, g_stats, o_tok, o_q, o_stats, o_flag, greedy, req_ids)
    t.diverged += forced
    return t, o_tok, o_q, o_stats, o_flag


def verify_forced(g, oracle_rows, length, greedy, req_ids, threads=1):
    """Compare a GPU verification with the oracle's.  oracle_rows(i, force_acc_row)
    runs the oracle's verification of compact row i and returns a dict of that
    row (accept, n_accept, y, p, flag_acc, flag_y); at a flagged accept test that
    differs, the oracle is re-run with the GPU's decision adopted there."""
    n = len(length)
    rows = _pmap(lambda i: oracle_rows(i, None), list(range(n)), threads)

    def stack(rs):
        return {k: np.stack([np.asarray(r[k]) for r in rs]) for k in rs[0]}

    gamma = g["accept"].shape[1]
    force = np.full((n, gamma), -1, np.int8)
    forced = 0
    for _ in range(gamma + 1):
        t = compare_verify(g, stack(rows), length, greedy, req_ids)
        redo = sorted({i for i, j, a in t.force if force[i, j] < 0})
        if not redo:
            break
        for i, j, a in t.force:
            if force[i, j] < 0:
                force[i, j] = a
                forced += 1
        new = _pmap(lambda i: oracle_rows(i, force[i]), redo, threads)
        for i, r in zip(redo, new):
            rows[i] = r
    t = compare_verify(g, stack(rows), length, greedy, req_ids)
    t.diverged += forced
    return t, stack(rows)


def confidence_forced(g_c, o_c, o_flag, valid=None):
    """Bit-identical confidences unless flagged; the scheduler's input on the oracle
    side then takes the GPU's value at a flagged difference (teacher forcing)."""
    t = compare_confidence(g_c, o_c, o_flag, valid)
    c32 = o_c.astype(np.float32)
    differ = (g_c.view(np.uint32) != c32.view(np.uint32)) & o_flag.astype(bool)
    t.diverged += int(differ.sum())
    c32[differ] = g_c[differ]
    return t, c32


def round_parity(g, inp, temperature, seed, rnd, subset=None, threads=1):
    """One whole round of the GPU path against the oracle, chained stage by stage.

    g: the GPU's outputs of the round as host arrays (tok, q, stats, c, len, a, B,
    accept, n_accept, y, p), over all R requests.  inp: the round's inputs (host
    or device tensors).  subset: the requests whose draft and verification the
    oracle recomputes (all when None); the confidence head and the scheduler are
    compared over every request, on the oracle's (teacher-forced) draft chain for
    the subset and the GPU's tokens elsewhere, so the scheduler sees exactly the
    round the GPU scheduled.  Returns a dict of Tallies by stage and the total."""
    import oracle as orc
    R, gamma = inp["R"], inp["gamma"]
    greedy = temperature == 0.0
    S = np.arange(R, dtype=np.int32) if subset is None else np.asarray(subset, np.int32)
    idx = S.astype(np.int64)

    def rows_of(t):
        if isinstance(t, np.ndarray):
            return t[idx]
        import torch
        return t[torch.as_tensor(idx, device=t.device)]

    E = orc.bf16_bits(inp["E"])
    W2 = orc.bf16_bits(inp["W2"])
    anchor = np.asarray(inp["anchor"].cpu().numpy(), np.int32)
    base_S = orc.host_logits(rows_of(inp["base"]))
    tgt_S = orc.host_logits(rows_of(inp["target"]))

    def d_rows(i, force_row):
        f = None if force_row is None else force_row[None]
        tok, q, st, fl = orc.draft(base_S[i:i + 1], E, W2, anchor[S[i:i + 1]], S[i:i + 1],
                                   temperature, seed, rnd, force=f)
        return tok[0], q[0], st[0], fl[0]

    t_d, o_tok, o_q, o_stats, o_flag = draft_forced(g["tok"][idx], g["q"][idx], g["stats"][idx],
                                                    d_rows, greedy, S, threads)
    tok_all = np.array(g["tok"], np.int32, copy=True)
    tok_all[idx] = o_tok
    off = None if inp["offset"] is None else inp["offset"].cpu().numpy()
    o_c, o_cf = orc.confidence(orc.bf16_bits(inp["h"]), E, anchor, tok_all, inp["w"].cpu().numpy(),
                               inp["T"].cpu().numpy(), off)
    t_c, c32 = confidence_forced(g["c"], o_c, o_cf)
    o_len, o_a, o_B, _ = orc.schedule(c32, inp["sps"].cpu().numpy(), inp["B_max"], inp["tau0"],
                                      inp["mode"])
    t_s = compare_schedule(g["len"], g["a"], np.asarray(g["B"]).reshape(-1)[0], o_len, o_a, o_B)
    len_S = o_len[idx]

    def v_rows(i, force_row):
        f = None if force_row is None else force_row[None]
        v = orc.verify(tgt_S[i:i + 1], base_S[i:i + 1], E, W2, anchor[S[i:i + 1]], o_tok[i:i + 1],
                       o_q[i:i + 1], len_S[i:i + 1], S[i:i + 1], temperature, seed, rnd,
                       force_acc=f)
        return {k: v[k][0] for k in v}

    g_v = {k: np.asarray(g[k])[idx] for k in ("accept", "n_accept", "y", "p")}
    t_v, _ = verify_forced(g_v, v_rows, len_S, greedy, S, threads)
    total = Tally().add(t_d).add(t_c).add(t_s).add(t_v)
    return {"draft": t_d, "confidence": t_c, "schedule": t_s, "verify": t_v, "total": total,
            "len_sum": int(o_len.sum()), "B": int(o_B)}
