"""Pins of the CPU oracle against what the DSpark pages and the mathematics fix.

These run without a GPU.  Each test checks the oracle against something other
than itself: a value the pages print for a worked example (tests/golden/), a
closed form, an identity of the lossless-verification proof, a library routine
the step reduces to, or brute force on tiny inputs.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch
from scipy import stats as sst
from scipy.special import logsumexp
from scipy.special import softmax as sp_softmax

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            rows.setdefault(key, []).append(vals)
    return rows


def bf16(x):
    """Round float64 values to bf16 and return their uint16 bit patterns."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_val(bits):
    return torch.from_numpy(np.asarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16).double().numpy()


def chi2_ok(counts, probs, alpha):
    counts = np.asarray(counts, np.float64)
    n = counts.sum()
    keep = probs * n > 0
    res = sst.chisquare(counts[keep], probs[keep] * n / probs[keep].sum())
    return res.pvalue > alpha, res.pvalue


# ---------------------------------------------------------------------------
# Philox4x32-10
# ---------------------------------------------------------------------------

def test_philox_known_answers(orc):
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        lines = [l.split() for l in f if l.strip() and not l.startswith("#")]
    assert len(lines) == 3
    for cols in lines:
        ints = [int(c, 16) for c in cols]
        out = orc.philox4x32_10(ints[:4], ints[4:6])
        assert [int(x) for x in out] == ints[6:10]


def test_philox_matches_rocrand_header(orc, tmp_path):
    """Independent implementation: rocRAND's open-source Philox header, compiled
    for the host.  Checks the counter/key word order the oracle relies on."""
    import shutil
    import subprocess
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    hdr = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"
    if not os.path.exists(hdr) or not os.path.exists(hipcc):
        pytest.skip("rocRAND header or hipcc not available")
    src = tmp_path / "p.cpp"
    src.write_text(r'''
#include <cstdio>
#include <rocrand/rocrand_philox4x32_10.h>
struct probe : rocrand_device::philox4x32_10_engine {
  uint4 run(uint4 c, uint2 k) { return ten_rounds(c, k); }
};
int main() {
  probe p; unsigned s = 12345u;
  for (int i = 0; i < 64; ++i) {
    uint4 c; uint2 k;
    s = s * 1664525u + 1013904223u; c.x = s; s = s * 1664525u + 1013904223u; c.y = s;
    s = s * 1664525u + 1013904223u; c.z = s; s = s * 1664525u + 1013904223u; c.w = s;
    s = s * 1664525u + 1013904223u; k.x = s; s = s * 1664525u + 1013904223u; k.y = s;
    uint4 o = p.run(c, k);
    printf("%u %u %u %u %u %u %u %u %u %u\n", c.x, c.y, c.z, c.w, k.x, k.y, o.x, o.y, o.z, o.w);
  }
}
''')
    exe = tmp_path / "p"
    r = subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("rocRAND header did not compile for the host: " + r.stderr[-300:])
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    n = 0
    for line in out.strip().splitlines():
        v = [int(x) for x in line.split()]
        got = orc.philox4x32_10(v[:4], v[4:6])
        assert [int(x) for x in got] == v[6:10]
        n += 1
    assert n == 64


def test_uniform_mapping_and_ks(orc):
    # u = top 24 bits of word 0 / 2^24, counter = (round, req, pos, purpose), key = seed
    seed = 0x0123456789ABCDEF
    w = orc.philox4x32_10([7, 3, 2, 1], [seed & 0xFFFFFFFF, seed >> 32])
    assert orc.uniform(seed, 7, 3, 2, 1) == (int(w[0]) >> 8) / 2.0 ** 24
    us = np.array([orc.uniform(0, rnd, req, pos, pur)
                   for rnd in range(5) for req in range(40) for pos in range(10) for pur in range(3)])
    assert us.min() >= 0.0 and us.max() < 1.0
    assert sst.kstest(us, "uniform").pvalue > 1e-4
    # distinct purposes give distinct streams
    assert orc.uniform(0, 0, 0, 0, 0) != orc.uniform(0, 0, 0, 0, 1)


# ---------------------------------------------------------------------------
# Markov head: the pages' worked example (base 0, 0 plus ln 9: 50% -> 90%)
# ---------------------------------------------------------------------------

def _ln9_split():
    g = _golden("markov_example.txt")
    bias = float(g["bias"][0][0])
    assert abs(bias - math.log(9.0)) < 1e-15
    terms, rest = [], bias
    for _ in range(3):
        t = float(bf16_val(bf16([rest]))[0])
        terms.append(t)
        rest -= t
    return bias, terms


def test_markov_worked_example(orc):
    g = _golden("markov_example.txt")
    before = [float(x) for x in g["prob_before"][0]]
    after = [float(x) for x in g["prob_after"][0]]
    base = np.zeros(2, np.float32)
    # rank-3 factorisation of "add ln 9 to token 0": E[prev] = (1, 1, 1),
    # column 0 of W2 = a three-term bf16 expansion of ln 9, column 1 = 0.
    _, terms = _ln9_split()
    E = bf16([[1.0, 1.0, 1.0], [0.0, 0.0, 0.0]])
    W2 = np.stack([bf16(terms), bf16([0.0, 0.0, 0.0])])
    logit0, _ = orc.markov_logits(base, E, W2, prev=-1)
    p0, _ = orc.softmax(logit0, 1.0)
    np.testing.assert_allclose(p0, before, atol=1e-15)
    logit1, _ = orc.markov_logits(base, E, W2, prev=0)
    p1, _ = orc.softmax(logit1, 1.0)
    np.testing.assert_allclose(p1, after, atol=1e-8)
    # negative control: keeping only the leading bf16 term misses 90% by > 1e-4,
    # so the check above sees every term of the rank-r contraction
    W2c = np.stack([bf16([terms[0], 0.0, 0.0]), bf16([0.0, 0.0, 0.0])])
    lc, _ = orc.markov_logits(base, E, W2c, prev=0)
    pc, _ = orc.softmax(lc, 1.0)
    assert abs(pc[0] - after[0]) > 1e-4
    # greedy draft picks the favoured token
    tok, q, _, fl = orc.draft(np.zeros((1, 1, 2), np.float32), E, W2, np.array([0]), np.array([0]),
                              0.0, 0, 0)
    assert tok[0, 0] == 0 and fl[0, 0] == 0


def test_markov_example_sampling_frequency(orc):
    """10^7 sampled drafts of the worked example: frequency 0.9 within 5 sigma."""
    _, terms = _ln9_split()
    E = bf16([[1.0, 1.0, 1.0], [0.0, 0.0, 0.0]])
    W2 = np.stack([bf16(terms), bf16([0.0, 0.0, 0.0])])
    n = 10_000_000
    base = np.zeros((n, 1, 2), np.float32)
    tok, q, _, _ = orc.draft(base, E, W2, np.zeros(n, np.int32), np.arange(n, dtype=np.int32),
                             1.0, 0, 0)
    freq = float((tok[:, 0] == 0).mean())
    sigma = math.sqrt(0.9 * 0.1 / n)
    assert abs(freq - 0.9) < 5 * sigma
    np.testing.assert_allclose(q[tok[:, 0] == 0, 0][:10], 0.9, atol=1e-8)


def test_markov_bias_is_rank_r_contraction(orc):
    """bias_v = sum_i E[prev, i] W2(i, v): with one-hot E rows the bias is a single
    W2 entry, which catches transposed or mis-indexed operands."""
    rng = np.random.default_rng(1)
    V, r = 7, 5
    W2 = bf16(rng.normal(0, 0.5, (V, r)))
    base = rng.normal(0, 1, V).astype(np.float32)
    for i in range(r):
        Erow = np.zeros((V, r))
        Erow[3, i] = 1.0
        E = bf16(Erow)
        lg, _ = orc.markov_logits(base, E, W2, prev=3)
        expect = (base.astype(np.float64) + bf16_val(W2)[:, i]).astype(np.float32)
        np.testing.assert_array_equal(lg, expect)


def test_markov_out_of_vocabulary_prev_is_no_bias(orc):
    """A previous token outside [0, V) selects no embedding row: its logits are the
    base logits, bit for bit, as for prev = -1 (and the confidence head drops the
    E term); a valid prev does add its bias."""
    rng = np.random.default_rng(2)
    V, r = 9, 8
    E = bf16(rng.normal(0, 0.5, (V, r)))
    W2 = bf16(rng.normal(0, 0.5, (V, r)))
    base = rng.normal(0, 1, V).astype(np.float32)
    for prev in (-1, -7, V, V + 3, 2 ** 30):
        lg, ad = orc.markov_logits(base, E, W2, prev=prev)
        np.testing.assert_array_equal(lg, base)
        assert np.all(ad == 0.0)
    lg, _ = orc.markov_logits(base, E, W2, prev=V - 1)
    assert not np.array_equal(lg, base)


# ---------------------------------------------------------------------------
# Token selection: reductions to library routines
# ---------------------------------------------------------------------------

def test_softmax_matches_scipy(orc):
    rng = np.random.default_rng(2)
    for T in (1.0, 0.7, 1.3):
        x = (rng.normal(0, 3, 1000)).astype(np.float32)
        p, st = orc.softmax(x, T)
        ref = sp_softmax(x.astype(np.float64) / T)
        np.testing.assert_allclose(p, ref, rtol=1e-13, atol=1e-300)
        xd = x.astype(np.float64)
        assert st[0] == xd.max()
        assert abs(st[0] / T + np.log(st[1]) - logsumexp(xd / T)) < 1e-12


def test_inverse_cdf_matches_searchsorted(orc):
    rng = np.random.default_rng(3)
    for _ in range(200):
        V = int(rng.integers(1, 50))
        w = rng.random(V) * (rng.random(V) < 0.7)
        if w.sum() == 0:
            w[0] = 1.0
        u = float(rng.integers(0, 2 ** 24)) / 2 ** 24
        x, _ = orc.inverse_cdf(w, u)
        ref = int(np.searchsorted(np.cumsum(w), u * w.sum(), side="right"))
        assert x == min(ref, V - 1) or (ref == V and w[x] > 0)
        assert w[x] > 0


def test_plain_categorical_when_no_markov_bias(orc):
    """W2 = 0 reduces the draft to categorical sampling from softmax(base / T)."""
    rng = np.random.default_rng(4)
    V, r, n, T = 8, 4, 2_000_000, 0.8
    row = rng.normal(0, 1.0, V).astype(np.float32)
    base = np.broadcast_to(row, (n, 1, V)).copy()
    E = bf16(rng.normal(0, 1, (V, r)))
    W2 = bf16(np.zeros((V, r)))
    tok, q, st, _ = orc.draft(base, E, W2, np.zeros(n, np.int32), np.arange(n, dtype=np.int32), T, 5, 9)
    p = sp_softmax(row.astype(np.float64) / T)
    ok, pv = chi2_ok(np.bincount(tok[:, 0], minlength=V), p, 1e-4)
    assert ok, pv
    np.testing.assert_allclose(q[:, 0], p[tok[:, 0]], rtol=1e-12)


def test_greedy_is_argmax_and_low_temperature_limit(orc):
    rng = np.random.default_rng(5)
    V, r, g = 64, 8, 5
    n = 50
    base = rng.normal(0, 2, (n, g, V)).astype(np.float32)
    E = bf16(rng.normal(0, 0.1, (V, r)))
    W2 = bf16(rng.normal(0, 0.1, (V, r)))
    anchor = rng.integers(0, V, n).astype(np.int32)
    tok, _, _, fl = orc.draft(base, E, W2, anchor, np.arange(n, dtype=np.int32), 0.0, 0, 0)
    # recompute the chain with numpy argmax over the oracle's own logits
    for i in range(n):
        prev = anchor[i]
        for k in range(g):
            lg, _ = orc.markov_logits(base[i, k], E, W2, prev)
            assert tok[i, k] == int(np.argmax(lg))
            prev = tok[i, k]
    # a very low temperature samples the argmax whenever the top gap is large
    tok_c, _, _, _ = orc.draft(base, E, W2, anchor, np.arange(n, dtype=np.int32), 1e-4, 0, 0)
    assert (tok_c == tok).mean() > 0.99


# ---------------------------------------------------------------------------
# Confidence head and sequential temperature scaling
# ---------------------------------------------------------------------------

def test_confidence_concatenation_and_temperature(orc):
    rng = np.random.default_rng(6)
    n, g, d, V, r = 5, 4, 12, 20, 6
    h = bf16(rng.normal(0, 1, (n, g, d)))
    E = bf16(rng.normal(0, 0.3, (V, r)))
    w = rng.normal(0, 0.2, d + r).astype(np.float32)
    T = np.array([1.0, 1.2, 0.8, 2.0], np.float32)
    anchor = rng.integers(0, V, n).astype(np.int32)
    tok = rng.integers(0, V, (n, g)).astype(np.int32)
    c, _ = orc.confidence(h, E, anchor, tok, w, T)
    # [h_k; E[x_{k-1}]] as one hidden vector of width d + r with no E term
    prev = np.concatenate([anchor[:, None], tok[:, :-1]], axis=1)
    h2 = np.concatenate([h, E[prev]], axis=2)
    c2, _ = orc.confidence(h2, E, np.full(n, -1, np.int32), np.full((n, g), -1, np.int32), w, T)
    np.testing.assert_allclose(c, c2, rtol=1e-14)
    # T_k divides the logit: logit(c) * T_k is the same for every T
    c1, _ = orc.confidence(h, E, anchor, tok, w, np.ones(g, np.float32))
    lg = np.log(c / (1 - c)) * T[None, :]
    lg1 = np.log(c1 / (1 - c1))
    np.testing.assert_allclose(lg, lg1, rtol=1e-9, atol=1e-9)
    # negating w mirrors the sigmoid; w = 0 gives exactly 1/2
    cn, _ = orc.confidence(h, E, anchor, tok, -w, T)
    np.testing.assert_allclose(cn, 1 - c, atol=1e-15)
    c0, _ = orc.confidence(h, E, anchor, tok, 0 * w, T)
    assert np.all(c0 == 0.5)
    # a per-request offset shifts the logit before scaling
    off = np.linspace(-2, 2, n).astype(np.float32)
    co, _ = orc.confidence(h, E, anchor, tok, w, np.ones(g, np.float32), off)
    np.testing.assert_allclose(np.log(co / (1 - co)), lg1 + off[:, None].astype(np.float64),
                               rtol=1e-9, atol=1e-9)


def test_confidence_is_a_linear_layer_and_sigmoid(orc):
    """The head of page "DeepSeek联合北大最新文章DSpark" section 2.1 as the library
    layers it is made of: torch's Linear (no bias) over the concatenation
    [h_k; W1[x_{k-1}]] in float64, the offset added, divided by T_k, torch's
    sigmoid.  Every (request, position) has its own hidden row and its own
    previous token, so reading another row, another request's token or the
    token of another position changes the result."""
    rng = np.random.default_rng(16)
    n, g, d, V, r = 7, 5, 24, 40, 8
    h = bf16(rng.normal(0, 1, (n, g, d)))
    E = bf16(rng.normal(0, 0.5, (V, r)))
    w = rng.normal(0, 0.3, d + r).astype(np.float32)
    T = np.array([1.0, 1.3, 0.7, 2.0, 1.1], np.float32)
    off = rng.uniform(-2, 2, n).astype(np.float32)
    anchor = rng.integers(0, V, n).astype(np.int32)
    anchor[2] = -1
    tok = rng.integers(0, V, (n, g)).astype(np.int32)
    c, _ = orc.confidence(h, E, anchor, tok, w, T, off)
    lin = torch.nn.Linear(d + r, 1, bias=False).double()
    with torch.no_grad():
        lin.weight.copy_(torch.from_numpy(w.astype(np.float64))[None, :])
    ref = np.zeros((n, g))
    for i in range(n):
        for k in range(g):
            prev = anchor[i] if k == 0 else tok[i, k - 1]
            e = bf16_val(E[prev]) if prev >= 0 else np.zeros(r)
            x = torch.from_numpy(np.concatenate([bf16_val(h[i, k]), e]))
            with torch.no_grad():
                y = lin(x[None, :])[0, 0] + float(off[i])
                ref[i, k] = torch.sigmoid(y / float(T[k])).item()
    np.testing.assert_allclose(c, ref, rtol=1e-13, atol=0)
    # closed form: a one-hot w reads a single hidden coordinate of row (i, k)
    for idx in (0, 5, d - 1):
        w1 = np.zeros(d + r, np.float32)
        w1[idx] = 1.0
        c1, _ = orc.confidence(h, E, anchor, tok, w1, T)
        hv = bf16_val(h[:, :, idx])
        np.testing.assert_allclose(c1, 1.0 / (1.0 + np.exp(-hv / T[None, :].astype(np.float64))),
                                   rtol=1e-15)
    # one-hot on an embedding coordinate reads E of the previous token
    w1 = np.zeros(d + r, np.float32)
    w1[d + 3] = 1.0
    c1, _ = orc.confidence(h, E, anchor, tok, w1, np.ones(g, np.float32))
    prev = np.concatenate([anchor[:, None], tok[:, :-1]], axis=1)
    ev = np.where(prev >= 0, bf16_val(E[np.maximum(prev, 0), 3]), 0.0)
    np.testing.assert_allclose(c1, 1.0 / (1.0 + np.exp(-ev)), rtol=1e-15)


def test_confidence_flag_marks_fp32_rounding_midpoints(orc):
    """c = sigma(y): y = 2^-23 puts c at 1/2 + 2^-25 (to within 1e-21), the
    midpoint between the fp32 neighbours 1/2 and 1/2 + 2^-24, so the flag fires;
    y = 2^-22 puts c at 1/2 + 2^-24 (less 2e-21), an fp32 value, so it does not."""
    d, V, r = 1, 4, 8
    E = bf16(np.zeros((V, r)))
    h = bf16(np.ones((1, 2, d)))
    anchor = np.array([-1], np.int32)
    tok = np.array([[-1, -1]], np.int32)
    T = np.ones(2, np.float32)
    for y, want in ((2.0 ** -23, 1), (2.0 ** -22, 0)):
        w = np.zeros(d + r, np.float32)
        w[0] = y
        c, fl = orc.confidence(h, E, anchor, tok, w, T)
        assert abs(c[0, 0] - (0.5 + y / 4)) < 1e-20
        assert list(fl[0]) == [want, want], (y, fl)
    # generic values are not flagged
    rng = np.random.default_rng(17)
    h = bf16(rng.normal(0, 1, (50, 4, 16)))
    E = bf16(rng.normal(0, 0.1, (V, r)))
    w = rng.normal(0, 0.1, 16 + r).astype(np.float32)
    _, fl = orc.confidence(h, E, rng.integers(0, V, 50).astype(np.int32),
                           rng.integers(0, V, (50, 4)).astype(np.int32), w, np.ones(4, np.float32))
    assert fl.sum() == 0


# ---------------------------------------------------------------------------
# Near-boundary flags: where a differing decision is allowed
# ---------------------------------------------------------------------------

def _two_logit_row(p0):
    """fp32 logits (0, l1) whose fp64 softmax puts mass close to p0 on token 0, and
    that mass exactly as the oracle's fp64 softmax computes it."""
    l1 = np.float32(np.log(1.0 / p0 - 1.0))
    row = np.array([0.0, l1], np.float32)
    p0_exact = 1.0 / (1.0 + np.exp(np.float64(l1)))
    return row, p0_exact


def test_sampling_flag_window(orc):
    """A draft draw is flagged exactly when u lies within 1e-6 of a boundary of the
    fp64 CDF: rows built so that the boundary after token 0 sits at known
    distances from the draw's u."""
    E = bf16(np.zeros((2, 8)))
    W2 = bf16(np.zeros((2, 8)))
    seed, rnd = 3, 4
    checked = 0
    for req in range(40):
        u = orc.uniform(seed, rnd, req, 0, 0)
        if not 0.05 < u < 0.95:
            continue
        for dist in (-3e-6, -1.5e-6, -0.6e-6, -0.2e-6, 0.2e-6, 0.6e-6, 1.5e-6, 3e-6):
            row, p0 = _two_logit_row(u + dist)
            gap = p0 - u                      # the boundary's actual distance from u
            if abs(abs(gap) - 1e-6) < 5e-8:
                continue                      # too close to the window's edge to call
            tok, _, _, fl = orc.draft(row[None, None, :], E, W2, np.array([-1], np.int32),
                                      np.array([req], np.int32), 1.0, seed, rnd)
            assert tok[0, 0] == (0 if u < p0 else 1)
            assert fl[0, 0] == (abs(gap) < 1e-6), (req, dist, gap)
            checked += 1
    assert checked > 100


def test_greedy_near_tie_flag(orc):
    """Greedy flag: the top-2 gap is within 2 ulp of the maximum plus the bound on
    the bias's summation order.  Without a bias the bound is 2 ulp: gaps of 0, 1
    and 2 ulp at 1.5 (ulp 2^-23) are flagged, 3 and more are not; with a bias the
    window widens by (r + 1) 2^-24 times the two columns' sums of |E W2|."""
    ulp = 2.0 ** -23
    E = bf16(np.zeros((3, 8)))
    W2 = bf16(np.zeros((3, 8)))
    for k_ulp, want in ((0, 1), (1, 1), (2, 1), (3, 0), (40, 0)):
        row = np.array([-5.0, 1.5 - k_ulp * ulp, 1.5], np.float32)
        tok, q, _, fl = orc.draft(row[None, None, :], E, W2, np.array([-1], np.int32),
                                  np.array([0], np.int32), 0.0, 0, 0)
        assert tok[0, 0] == (1 if k_ulp == 0 else 2) and q[0, 0] == 1.0   # ties: lowest index
        assert fl[0, 0] == want, k_ulp
    # with a bias: E[0] = 1 everywhere, W2 columns of +-1/8: |bias| sums of 1 per column
    r = 8
    E = bf16(np.ones((3, r)))
    W2 = bf16(np.concatenate([np.zeros((1, r)), np.full((1, r), 0.125), np.full((1, r), -0.125)]))
    # biases: column 1 +1, column 2 -1; window = 2 ulp + 9 * 2^-24 * 2 = 2 ulp(2.5) + 1.07e-6
    for gap, want in ((0.5e-6, 1), (1.4e-6, 1), (4e-6, 0)):
        row = np.array([-5.0, 1.5, np.float32(3.5 + gap)], np.float32)
        lg, absdot = orc.markov_logits(row, E, W2, 0)
        real_gap = float(lg[2]) - float(lg[1])
        bound = 2 * 2.0 ** -22 + 9 * 2.0 ** -24 * (absdot[1] + absdot[2])
        tok, _, _, fl = orc.draft(row[None, None, :], E, W2, np.array([0], np.int32),
                                  np.array([0], np.int32), 0.0, 0, 0)
        assert fl[0, 0] == (real_gap <= bound) == bool(want), (gap, real_gap, bound)


def test_accept_flag_window(orc):
    """An accept test is flagged exactly when |u - p/q| < 1e-6: q chosen so that the
    ratio p/q sits at known distances from the test's u."""
    E = bf16(np.zeros((2, 8)))
    W2 = bf16(np.zeros((2, 8)))
    seed, rnd = 1, 2
    target = np.array([[[0.3, -0.4], [0.0, 0.0]]], np.float32)
    p0 = sp_softmax(target[0, 0].astype(np.float64))[0]
    base = np.zeros((1, 1, 2), np.float32)
    checked = 0
    for req in range(30):
        u = orc.uniform(seed, rnd, req, 0, 1)
        if not 0.05 < u < 0.95:
            continue
        for dist in (-4e-6, -0.5e-6, 0.5e-6, 4e-6):
            q = np.array([[p0 / (u + dist)]])
            ratio = p0 / q[0, 0]
            v = orc.verify(target, base, E, W2, np.array([-1], np.int32),
                           np.array([[0]], np.int32), q, np.array([1], np.int32),
                           np.array([req], np.int32), 1.0, seed, rnd)
            assert v["accept"][0, 0] == int(u <= ratio)
            assert v["flag_acc"][0, 0] == (abs(u - ratio) < 1e-6), (req, dist)
            checked += 1
    assert checked > 40


def test_teacher_forcing_hooks(orc):
    """The comparison hooks: a forced draft token is the chain's token from then on
    (the next position's bias and draw use it), and a forced accept decision is
    the one the first rejection follows."""
    rng = np.random.default_rng(18)
    V, r, g = 30, 8, 3
    base = rng.normal(0, 1, (1, g, V)).astype(np.float32)
    E = bf16(rng.normal(0, 0.3, (V, r)))
    W2 = bf16(rng.normal(0, 0.3, (V, r)))
    anchor = np.array([4], np.int32)
    req = np.array([9], np.int32)
    tok, q, _, _ = orc.draft(base, E, W2, anchor, req, 1.0, 0, 5)
    forced = (tok[0, 0] + 7) % V
    force = np.array([[forced, -1, -1]], np.int32)
    tf, qf, _, _ = orc.draft(base, E, W2, anchor, req, 1.0, 0, 5, force=force)
    assert tf[0, 0] == forced
    lg0, _ = orc.markov_logits(base[0, 0], E, W2, 4)
    p0, _ = orc.softmax(lg0, 1.0)
    assert qf[0, 0] == p0[forced]
    lg1, _ = orc.markov_logits(base[0, 1], E, W2, forced)
    p1, _ = orc.softmax(lg1, 1.0)
    x1, _ = orc.inverse_cdf(p1, orc.uniform(0, 5, 9, 1, 0))
    assert tf[0, 1] == x1 and qf[0, 1] == p1[x1]
    # accept forcing: force a rejection at position 1 of a fully accepted block
    tgt = np.concatenate([base, base[:, :1]], axis=1)   # p = q: every test accepts
    v = orc.verify(tgt, base, E, W2, anchor, tok, q, np.array([g], np.int32), req, 1.0, 0, 5)
    assert v["n_accept"][0] == g
    fa = np.array([[-1, 0, -1]], np.int8)
    v2 = orc.verify(tgt, base, E, W2, anchor, tok, q, np.array([g], np.int32), req, 1.0, 0, 5,
                    force_acc=fa)
    assert v2["n_accept"][0] == 1 and v2["accept"][0, 1] == 0


# ---------------------------------------------------------------------------
# Prefix scheduler
# ---------------------------------------------------------------------------

def test_survival_worked_example(orc):
    g = _golden("survival_example.txt")
    cond = [float(x) for x in g["conditional_after_first"][0]]
    ratio = [float(x) for x in g["ratio"][0]]
    for c1 in (1.0, 0.9, 0.5, 0.123):
        c = np.array([[c1] + cond], np.float32)
        length, a, B, _ = orc.schedule(c, np.ones(6, np.float32), 6, 0.0, 1)
        expect = c1 * np.array(ratio)
        ulp = np.spacing(np.abs(expect).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(a[0].astype(np.float64) - expect) <= 2 * ulp)
        assert np.all(np.diff(a[0]) <= 0)
        # with a constant SPS the objective rises with every positive a: all admitted
        assert length[0] == 5 and B == 6


def _prefix_curve(a, sps, R, tau0, B_max):
    """Theta after admitting the n best candidates, n = 0..N (fp64, numpy sort)."""
    Rg = a.shape
    flat = a.ravel().astype(np.float64)
    rr = np.repeat(np.arange(a.shape[0]), a.shape[1])
    jj = np.tile(np.arange(a.shape[1]), a.shape[0])
    order = np.lexsort((jj, rr, -flat))
    theta = [tau0 * sps[R - 1]]
    s = tau0
    for n, idx in enumerate(order, start=1):
        if R + n > B_max:
            break
        s += flat[idx]
        theta.append(s * sps[R + n - 1])
    return np.array(theta), order, rr, jj


def test_scheduler_brute_force(orc):
    """Exhaustive search over every length vector on tiny instances (R <= 3,
    gamma <= 4): the best prefix of the global sort is the global optimum, and
    the early stop gives the first local maximum of the prefix curve, which is the
    global one whenever that curve is unimodal."""
    rng = np.random.default_rng(7)
    kinds = {"unimodal": 0, "multimodal": 0}
    for trial in range(400):
        R = int(rng.integers(1, 4))
        gamma = int(rng.integers(1, 5))
        c = rng.uniform(0.05, 1.0, (R, gamma)).astype(np.float32)
        B_full = R * (gamma + 1)
        B_max = int(rng.integers(R, B_full + 1))
        if trial % 3 == 0:
            # jagged cost curve (non-monotone SPS) to produce multimodal objectives
            sps = rng.uniform(0.2, 1.0, B_max).astype(np.float32)
        else:
            k1, k2 = rng.uniform(0.01, 3.0), rng.uniform(0.0, 0.5)
            Bs = np.arange(1, B_max + 1, dtype=np.float64)
            sps = (1.0 / (1.0 + k1 * Bs + k2 * Bs * Bs)).astype(np.float32)
        tau0 = float(rng.choice([0.0, float(R)]))
        length, a, B, _ = orc.schedule(c, sps, B_max, tau0, 1)
        spsd = sps.astype(np.float64)
        # exhaustive optimum over every l vector
        best = -1.0
        for lv in itertools.product(range(gamma + 1), repeat=R):
            Bv = R + sum(lv)
            if Bv > B_max:
                continue
            tau = tau0 + sum(float(a[r_, :lv[r_]].astype(np.float64).sum()) for r_ in range(R))
            best = max(best, tau * spsd[Bv - 1])
        theta, order, rr, jj = _prefix_curve(a, spsd, R, tau0, B_max)
        assert abs(theta.max() - best) <= 1e-12 * max(best, 1e-300)
        # early stop = first n with theta_{n+1} <= theta_n
        n_star = 0
        while n_star + 1 < len(theta) and theta[n_star + 1] > theta[n_star] * (1 + 1e-12):
            n_star += 1
        assert B == R + n_star, (trial, B, R, n_star)
        expect_len = np.bincount(rr[order[:n_star]], minlength=R)
        np.testing.assert_array_equal(length, expect_len)
        # admitted sets are prefixes of each request's block
        unimodal = all(theta[i + 1] <= theta[i] for i in range(n_star, len(theta) - 1))
        if unimodal:
            kinds["unimodal"] += 1
            assert abs(theta[n_star] - best) <= 1e-12 * max(best, 1e-300)
        else:
            kinds["multimodal"] += 1
    assert kinds["unimodal"] > 50 and kinds["multimodal"] > 5, kinds


def test_scheduler_causality(orc):
    """Whether position j of request r is verified must not depend on x_{r,j} or
    later tokens, i.e. on c_{r,j+1..}: perturbing those keeps min(l_r, j+1)."""
    rng = np.random.default_rng(8)
    for _ in range(300):
        R, gamma = int(rng.integers(1, 6)), int(rng.integers(2, 7))
        c = rng.uniform(0.3, 1.0, (R, gamma)).astype(np.float32)
        Bs = np.arange(1, R * (gamma + 1) + 1, dtype=np.float64)
        sps = (1.0 / (12 + 0.1 * Bs + 0.0008 * Bs ** 2 * rng.uniform(1, 200))).astype(np.float32)
        l0, _, _, _ = orc.schedule(c, sps, R * (gamma + 1), 0.0, 1)
        r = int(rng.integers(0, R))
        j = int(rng.integers(0, gamma - 1))
        c2 = c.copy()
        c2[r, j + 1:] = rng.uniform(0.0, 1.0, gamma - j - 1).astype(np.float32)
        l1, _, _, _ = orc.schedule(c2, sps, R * (gamma + 1), 0.0, 1)
        assert min(l0[r], j + 1) == min(l1[r], j + 1)


def test_scheduler_off_and_limits(orc):
    c = np.full((3, 4), 0.9, np.float32)
    length, a, B, _ = orc.schedule(c, np.ones(15, np.float32), 15, 0.0, 0)
    assert list(length) == [4, 4, 4] and B == 15
    # B_max = R admits nothing
    length, _, B, _ = orc.schedule(c, np.ones(3, np.float32), 3, 0.0, 1)
    assert list(length) == [0, 0, 0] and B == 3
    # a = 0 never raises the objective
    length, _, B, _ = orc.schedule(np.zeros((2, 3), np.float32), np.ones(8, np.float32), 8, 0.0, 1)
    assert list(length) == [0, 0] and B == 2


# ---------------------------------------------------------------------------
# Lossless verification: identities of the proof and the pages' examples
# ---------------------------------------------------------------------------

def _tiny_single_position(rng, V, r, skew=None):
    base_row = rng.normal(0, 1.5, V).astype(np.float32)
    E = bf16(rng.normal(0, 0.4, (V, r)))
    W2 = bf16(rng.normal(0, 0.4, (V, r)))
    target_rows = rng.normal(0, 1.5, (2, V)).astype(np.float32)
    return base_row, E, W2, target_rows


def test_total_acceptance_is_sum_min_and_residual_law(orc):
    """Page 5's proof: acceptance probability sum_x min(p, q); rejection
    probability sum max(0, p - q); after rejection y ~ max(0, p - q) normalised.
    10^7 trials at one position, V = 6."""
    rng = np.random.default_rng(9)
    V, r, n, T = 6, 4, 10_000_000, 1.0
    base_row, E, W2, trows = _tiny_single_position(rng, V, r)
    anchor = 2
    base = np.broadcast_to(base_row, (n, 1, V)).copy()
    target = np.broadcast_to(trows, (n, 2, V)).copy()
    req = np.arange(n, dtype=np.int32)
    anc = np.full(n, anchor, np.int32)
    tok, q, _, _ = orc.draft(base, E, W2, anc, req, T, 11, 3)
    res = orc.verify(target, base, E, W2, anc, tok, q, np.ones(n, np.int32), req, T, 11, 3)
    lg, _ = orc.markov_logits(base_row, E, W2, anchor)
    qd, _ = orc.softmax(lg, T)
    p, _ = orc.softmax(trows[0], T)
    acc_rate = float((res["accept"][:, 0] == 1).mean())
    smin = float(np.minimum(p, qd).sum())
    assert abs(acc_rate - smin) < 5 * math.sqrt(smin * (1 - smin) / n)
    rej = res["n_accept"] == 0
    rho = np.maximum(0.0, p - qd)
    assert abs(rej.mean() - rho.sum()) < 5 * math.sqrt(rho.sum() * (1 - rho.sum()) / n)
    ok, pv = chi2_ok(np.bincount(res["y"][rej], minlength=V), rho / rho.sum(), 1e-4)
    assert ok, pv
    # emitted token at position 0 ~ p (lossless)
    emitted = np.where(rej, res["y"], tok[:, 0])
    ok, pv = chi2_ok(np.bincount(emitted, minlength=V), p, 1e-4)
    assert ok, pv


def test_two_token_example(orc):
    """Target wants A 60% / B 40%; a draft skewed either way leaves the output
    law at 60/40 (10^7 trials per skew)."""
    tgt = np.array([float(x) for x in _golden("two_token_example.txt")["target"][0]])
    n = 10_000_000
    E = bf16([[0.0], [0.0]])
    W2 = bf16([[0.0], [0.0]])
    tl = np.log(tgt).astype(np.float32)
    p, _ = orc.softmax(tl, 1.0)
    for qa in (0.95, 0.05, 0.6):
        ql = np.log(np.array([qa, 1 - qa])).astype(np.float32)
        base = np.broadcast_to(ql, (n, 1, 2)).copy()
        target = np.broadcast_to(np.stack([tl, tl]), (n, 2, 2)).copy()
        req = np.arange(n, dtype=np.int32)
        anc = np.full(n, -1, np.int32)
        tok, q, _, _ = orc.draft(base, E, W2, anc, req, 1.0, 21, 0)
        res = orc.verify(target, base, E, W2, anc, tok, q, np.ones(n, np.int32), req, 1.0, 21, 0)
        emitted = np.where(res["n_accept"] == 0, res["y"], tok[:, 0])
        fa = float((emitted == 0).mean())
        assert abs(fa - p[0]) < 5 * math.sqrt(p[0] * p[1] / n), (qa, fa)


def test_reductions_p_equals_q_and_zero_length(orc):
    rng = np.random.default_rng(10)
    V, r, g, n, T = 16, 4, 3, 20000, 0.9
    base = rng.normal(0, 1, (n, g, V)).astype(np.float32)
    E = bf16(rng.normal(0, 0.2, (V, r)))
    W2 = bf16(np.zeros((V, r)))
    anc = rng.integers(0, V, n).astype(np.int32)
    req = np.arange(n, dtype=np.int32)
    tok, q, _, _ = orc.draft(base, E, W2, anc, req, T, 1, 1)
    # target equal to the draft logits (no bias since W2 = 0): p = q, all accepted
    target = np.concatenate([base, rng.normal(0, 1, (n, 1, V)).astype(np.float32)], axis=1)
    res = orc.verify(target, base, E, W2, anc, tok, q, np.full(n, g, np.int32), req, T, 1, 1)
    assert np.all(res["n_accept"] == g) and np.all(res["accept"] == 1)
    np.testing.assert_allclose(res["p"], q, rtol=1e-12)
    # l = 0: verification is one draw from target row 0 (the bonus of an empty block)
    n2 = 2_000_000
    row = rng.normal(0, 1, V).astype(np.float32)
    tgt2 = np.broadcast_to(np.stack([row] * (g + 1)), (n2, g + 1, V)).copy()
    b2 = np.zeros((n2, g, V), np.float32)
    res2 = orc.verify(tgt2, b2, E, W2, np.zeros(n2, np.int32), np.zeros((n2, g), np.int32),
                      np.ones((n2, g)), np.zeros(n2, np.int32), np.arange(n2, dtype=np.int32), T, 4, 4)
    assert np.all(res2["n_accept"] == 0) and np.all(res2["accept"] == -1)
    ok, pv = chi2_ok(np.bincount(res2["y"], minlength=V), sp_softmax(row.astype(np.float64) / T), 1e-4)
    assert ok, pv


def test_greedy_verification_is_exact_match(orc):
    rng = np.random.default_rng(12)
    V, r, g, n = 40, 4, 4, 300
    base = rng.normal(0, 2, (n, g, V)).astype(np.float32)
    E = bf16(rng.normal(0, 0.2, (V, r)))
    W2 = bf16(rng.normal(0, 0.2, (V, r)))
    anc = rng.integers(0, V, n).astype(np.int32)
    req = np.arange(n, dtype=np.int32)
    tok, q, _, _ = orc.draft(base, E, W2, anc, req, 0.0, 0, 0)
    target = rng.normal(0, 2, (n, g + 1, V)).astype(np.float32)
    # make the target agree with the draft on a random prefix
    for i in range(n):
        m = int(rng.integers(0, g + 1))
        for j in range(m):
            target[i, j, tok[i, j]] = target[i, j].max() + 1.0
    length = rng.integers(0, g + 1, n).astype(np.int32)
    res = orc.verify(target, base, E, W2, anc, tok, q, length, req, 0.0, 0, 0)
    for i in range(n):
        am = target[i].argmax(axis=1)
        nacc = 0
        while nacc < length[i] and tok[i, nacc] == am[nacc]:
            nacc += 1
        assert res["n_accept"][i] == nacc
        assert res["y"][i] == am[nacc]


@pytest.mark.slow
def test_whole_path_output_law_chi2(orc):
    """Whole round with the scheduler on, V = 6, gamma = 3: over 10^7 request
    trials, the token emitted at every reached position j follows p_j, because
    whether j is verified depends only on x_{<j}."""
    rng = np.random.default_rng(13)
    V, r, g, d, T = 6, 4, 3, 8, 1.0
    R, rounds = 1000, 10_000
    base_row = rng.normal(0, 1.0, (g, V)).astype(np.float32)
    trows = (np.concatenate([base_row, rng.normal(0, 1.0, (1, V))]) +
             rng.normal(0, 0.8, (g + 1, V))).astype(np.float32)
    E = bf16(rng.normal(0, 0.5, (V, r)))
    W2 = bf16(rng.normal(0, 0.5, (V, r)))
    h = bf16(rng.normal(0, 1, (g, d)))
    w = rng.normal(0, 0.5, d + r).astype(np.float32)
    Tk = np.array([1.0, 1.2, 1.4], np.float32)
    Bs = np.arange(1, R * (g + 1) + 1, dtype=np.float64)
    # a cost curve flat enough that every length 0..gamma occurs
    sps = (1.0 / (12 + 0.3 * Bs + 2e-5 * Bs * Bs)).astype(np.float32)
    base = np.broadcast_to(base_row, (R, g, V)).copy()
    target = np.broadcast_to(trows, (R, g + 1, V)).copy()
    hh = np.broadcast_to(h, (R, g, d)).copy()
    anc = rng.integers(0, V, R).astype(np.int32)
    req = np.arange(R, dtype=np.int32)
    counts = np.zeros((g + 1, V), np.int64)
    lens = np.zeros(g + 1, np.int64)
    for rnd in range(rounds):
        tok, q, _, _ = orc.draft(base, E, W2, anc, req, T, 77, rnd)
        c, _ = orc.confidence(hh, E, anc, tok, w, Tk)
        length, _, _, _ = orc.schedule(c.astype(np.float32), sps, R * (g + 1), 0.0, 1)
        res = orc.verify(target, base, E, W2, anc, tok, q, length, req, T, 77, rnd)
        nacc = res["n_accept"]
        lens += np.bincount(length, minlength=g + 1)
        for j in range(g + 1):
            reached = nacc >= j
            em = np.where(nacc[reached] == j, res["y"][reached],
                          tok[reached, min(j, g - 1)] if j < g else res["y"][reached])
            counts[j] += np.bincount(em, minlength=V)
    assert np.all(lens > 0.03 * lens.sum()), lens  # ragged lengths actually occur
    for j in range(g + 1):
        p, _ = orc.softmax(trows[j], T)
        ok, pv = chi2_ok(counts[j], p, 1e-4 / (g + 1))
        assert ok, (j, pv, counts[j])


def test_oracle_is_deterministic(orc):
    from draft_sampling_lossless_markov_amd.workloads import WORKLOADS, make_inputs
    inp = make_inputs(WORKLOADS[0], 3)
    a = orc.run_round(inp, 1.0, 0, 5)
    b = orc.run_round(inp, 1.0, 0, 5)
    for k in ("tok", "q", "c", "len", "y", "n_accept", "accept"):
        np.testing.assert_array_equal(a[k], b[k])
    c = orc.run_round(inp, 1.0, 0, 6)
    assert not np.array_equal(a["tok"], c["tok"]) or not np.array_equal(a["y"], c["y"])


# ---------------------------------------------------------------------------
# Exact acceptance probability (total-variation target)
# ---------------------------------------------------------------------------

def test_tv_accept_identities(orc):
    """alpha = sum_v min(q, p) (page "为什么DSpark 可以加速推理？", section on the
    mathematics of speculative decoding: the total acceptance probability) equals
    1 - TV(q, p) (page "DeepSeek联合北大最新文章DSpark", section 2.1: the confidence
    head's target is one minus the total-variation distance).  Without a Markov
    bias the draft law is scipy's softmax of the base row, so the identity is
    checked against laws the oracle did not compute; p = q gives 1; disjoint
    supports (masked logits) give 0; the pages' two-token example (target 60/40)
    gives min(qa, 0.6) + min(1 - qa, 0.4)."""
    rng = np.random.default_rng(30)
    n, g, V, r = 5, 3, 40, 8
    base = rng.normal(0, 2, (n, g, V)).astype(np.float32)
    target = rng.normal(0, 2, (n, g + 1, V)).astype(np.float32)
    E = bf16(rng.normal(0, 0.3, (V, r)))
    W0 = bf16(np.zeros((V, r)))
    anchor = rng.integers(0, V, n).astype(np.int32)
    tok = rng.integers(0, V, (n, g)).astype(np.int32)
    for T in (1.0, 0.7):
        a = orc.tv_accept(target, base, E, W0, anchor, tok, T)
        q = sp_softmax(base.astype(np.float64) / T, axis=-1)
        p = sp_softmax(target[:, :g].astype(np.float64) / T, axis=-1)
        np.testing.assert_allclose(a, 1 - 0.5 * np.abs(q - p).sum(-1), rtol=0, atol=1e-14)
    # p = q
    same = np.concatenate([base, base[:, :1]], axis=1)
    np.testing.assert_allclose(orc.tv_accept(same, base, E, W0, anchor, tok, 1.0), 1.0, atol=1e-14)
    # disjoint supports
    b2 = np.full((1, 1, 4), -np.inf, np.float32)
    b2[0, 0, :2] = 0.0
    t2 = np.full((1, 2, 4), -np.inf, np.float32)
    t2[0, :, 2:] = 0.0
    assert orc.tv_accept(t2, b2, bf16(np.zeros((4, 8))), bf16(np.zeros((4, 8))),
                         np.array([-1], np.int32), np.zeros((1, 1), np.int32), 1.0)[0, 0] == 0.0
    # the two-token example
    tgt = np.array([float(x) for x in _golden("two_token_example.txt")["target"][0]])
    tl = np.log(tgt).astype(np.float32)
    p2 = sp_softmax(tl.astype(np.float64))
    for qa in (0.95, 0.05, 0.6, 0.3):
        ql = np.log(np.array([qa, 1 - qa])).astype(np.float32)
        q2 = sp_softmax(ql.astype(np.float64))
        a = orc.tv_accept(np.stack([tl, tl])[None], ql[None, None], bf16(np.zeros((2, 1))),
                          bf16(np.zeros((2, 1))), np.array([-1], np.int32), np.zeros((1, 1), np.int32),
                          1.0)
        assert abs(a[0, 0] - np.minimum(q2, p2).sum()) < 1e-15


def test_tv_accept_is_the_verification_accept_rate(orc):
    """With the Markov bias on, alpha of a position equals the rate at which the
    oracle's own lossless verification accepts draws at it: 4e5 draws of one
    request's first position (distinct Philox request ids), accept rate within
    5 sigma of alpha."""
    rng = np.random.default_rng(31)
    V, r, N = 6, 4, 400_000
    row = rng.normal(0, 1.2, V).astype(np.float32)
    trow = (row + rng.normal(0, 1.0, V)).astype(np.float32)
    E = bf16(rng.normal(0, 0.5, (V, r)))
    W2 = bf16(rng.normal(0, 0.5, (V, r)))
    prev = 3
    base = np.broadcast_to(row, (N, 1, V)).copy()
    target = np.broadcast_to(np.stack([trow, trow]), (N, 2, V)).copy()
    anc = np.full(N, prev, np.int32)
    req = np.arange(N, dtype=np.int32)
    tok, q, _, _ = orc.draft(base, E, W2, anc, req, 1.0, 8, 2)
    res = orc.verify(target, base, E, W2, anc, tok, q, np.ones(N, np.int32), req, 1.0, 8, 2)
    rate = float((res["accept"][:, 0] == 1).mean())
    a = orc.tv_accept(target[:1], base[:1], E, W2, anc[:1], tok[:1], 1.0)[0, 0]
    assert 0.05 < a < 0.95
    assert abs(rate - a) < 5 * math.sqrt(a * (1 - a) / N), (rate, a)


# ---------------------------------------------------------------------------
# Asynchronous scheduler with a capacity barrier
# ---------------------------------------------------------------------------

def _survival_order(c):
    """Survival products (fp32, left to right) and the order a desc, r asc, j asc."""
    a = np.cumprod(c.astype(np.float32), axis=1, dtype=np.float32)
    R, g = a.shape
    rr, jj = np.meshgrid(np.arange(R), np.arange(g), indexing="ij")
    order = np.lexsort((jj.ravel(), rr.ravel(), -a.ravel().astype(np.float64)))
    return a, order, rr.ravel(), jj.ravel()


def test_async_schedule_capacity_is_the_global_optimum(orc):
    """Page "DeepSeek联合北大最新文章DSpark", 挑战2: the capacity comes from an earlier
    round's confidences by a global search without early stop.  Against brute force
    over every length vector of that round (tiny R, gamma, jagged and smooth SPS):
    Theta at the capacity is the exhaustive optimum and the capacity is the smallest
    such n; the admitted set is the first K candidates of the current round's order
    (numpy's cumprod and lexsort)."""
    rng = np.random.default_rng(40)
    for trial in range(300):
        R = int(rng.integers(1, 4))
        gamma = int(rng.integers(1, 5))
        ch = rng.uniform(0.05, 1.0, (R, gamma)).astype(np.float32)
        c = rng.uniform(0.05, 1.0, (R, gamma)).astype(np.float32)
        B_max = int(rng.integers(R, R * (gamma + 1) + 1))
        if trial % 2 == 0:
            sps = rng.uniform(0.2, 1.0, B_max).astype(np.float32)
        else:
            Bs = np.arange(1, B_max + 1, dtype=np.float64)
            sps = (1.0 / (1.0 + rng.uniform(0.01, 3) * Bs + rng.uniform(0, .5) * Bs ** 2)).astype(np.float32)
        tau0 = float(rng.choice([0.0, 0.5]))
        length, a, B, K = orc.schedule_async(c, ch, sps, B_max, tau0)
        ah, _, _, _ = _survival_order(ch)
        spsd = sps.astype(np.float64)
        thetas = {}
        for lv in itertools.product(range(gamma + 1), repeat=R):
            Bv = R + sum(lv)
            if Bv > B_max:
                continue
            tau = tau0 + sum(float(ah[r_, :lv[r_]].astype(np.float64).sum()) for r_ in range(R))
            thetas[Bv - R] = max(thetas.get(Bv - R, -1.0), tau * spsd[Bv - 1])
        best = max(thetas.values())
        assert abs(thetas[K] - best) <= 1e-12 * max(best, 1e-300), (trial, K, thetas)
        assert all(thetas[n] < best * (1 - 1e-12) for n in thetas if n < K), (trial, K, thetas)
        assert B == R + K
        an, order, rr, jj = _survival_order(c)
        np.testing.assert_array_equal(a, an)
        np.testing.assert_array_equal(length, np.bincount(rr[order[:K]], minlength=R))


def test_async_schedule_matches_early_stop_on_unimodal_curves_and_beats_it_on_sawtooth(orc):
    """With the earlier round's confidences equal to the current ones and a smooth
    cost curve, the global search and the synchronous early stop agree.  On a
    sawtooth SPS table (the pages: real hardware curves are jagged and the naive
    early stop gets stuck in a local optimum) the capacity goes past the early stop
    and reaches a strictly higher Theta."""
    rng = np.random.default_rng(41)
    R, gamma = 64, 7
    c = rng.uniform(0.6, 0.98, (R, gamma)).astype(np.float32)
    B_max = R * (gamma + 1)
    Bs = np.arange(1, B_max + 1, dtype=np.float64)
    smooth = (1.0 / (12 + 0.1 * Bs + 0.0008 * Bs * Bs)).astype(np.float32)
    l_s, a_s, B_s, _ = orc.schedule(c, smooth, B_max, 0.0, 1)
    l_a, a_a, B_a, K = orc.schedule_async(c, c, smooth, B_max, 0.0)
    np.testing.assert_array_equal(l_s, l_a)
    assert B_s == B_a == R + K
    # sawtooth: throughput drops right after every multiple of 64 (a kernel-tile edge)
    saw = (1.0 / (12 + 0.02 * Bs) * np.where((Bs % 64) < 8, 0.9, 1.0)).astype(np.float32)
    l_e, _, B_e, _ = orc.schedule(c, saw, B_max, 0.0, 1)
    l_g, _, B_g, K = orc.schedule_async(c, c, saw, B_max, 0.0)
    a, order, _, _ = _survival_order(c)
    cum = np.concatenate([[0.0], np.cumsum(a.ravel()[order].astype(np.float64))])
    theta = lambda B: cum[B - R] * float(saw[B - 1])
    assert B_g > B_e and theta(B_g) > theta(B_e) * 1.01, (B_e, B_g)


def test_async_schedule_causality_and_why_the_barrier_matters(orc):
    """With the capacity fixed from the earlier round, whether position j of
    request r is verified does not depend on x_{r,j} or later tokens (c_{r,j+1..}).
    A global search over the current round's own confidences (the earlier round
    replaced by the current one) does depend on them in some instances -- the
    anticipation the capacity barrier removes (page "DSpark.让每一轮计算，多走几步",
    causality paragraph)."""
    rng = np.random.default_rng(42)
    violations = 0
    for _ in range(2000):
        R, gamma = int(rng.integers(1, 6)), int(rng.integers(2, 7))
        c = rng.uniform(0.3, 1.0, (R, gamma)).astype(np.float32)
        ch = rng.uniform(0.3, 1.0, (R, gamma)).astype(np.float32)
        B_max = R * (gamma + 1)
        sps = rng.uniform(0.2, 1.0, B_max).astype(np.float32)
        r = int(rng.integers(0, R))
        j = int(rng.integers(0, gamma - 1))
        c2 = c.copy()
        c2[r, j + 1:] = rng.uniform(0.0, 1.0, gamma - j - 1).astype(np.float32)
        l0, _, _, _ = orc.schedule_async(c, ch, sps, B_max, 0.0)
        l1, _, _, _ = orc.schedule_async(c2, ch, sps, B_max, 0.0)
        assert min(l0[r], j + 1) == min(l1[r], j + 1)
        g0, _, _, _ = orc.schedule_async(c, c, sps, B_max, 0.0)
        g1, _, _, _ = orc.schedule_async(c2, c2, sps, B_max, 0.0)
        violations += min(g0[r], j + 1) != min(g1[r], j + 1)
    assert violations > 0


# ---------------------------------------------------------------------------
# Sequential temperature scaling and ECE (page "DeepSeek联合北大最新文章DSpark",
# section 2.1: temperatures calibrated position by position, left to right,
# and the calibration error they reduce).
# ---------------------------------------------------------------------------
def _calib(N, gamma, seed, t_true=None):
    from draft_sampling_lossless_markov_amd.workloads import calibration_set
    z, acc = calibration_set(N, gamma, seed, t_true)
    return z.numpy(), acc.numpy()


def test_ece_hand_example_bins_and_cumulative_survival():
    import oracle
    l19 = math.log(19.0)
    # one position: predictions 0.05 (bin 0 of 10) accepted, 0.95 (bin 9) rejected
    z = np.array([[-l19], [l19]], np.float32)
    e, edge = oracle.ece(z, np.array([1, 0], np.int32), M=10)
    assert edge == 0
    assert e == pytest.approx((abs(1 - 0.05) + abs(0 - 0.95)) / 2, abs=1e-6)
    # two positions, cumulative survival 0.95 then 0.9025, accepted length 1:
    # both in bin 9, outcomes 1 then 0
    z = np.array([[l19, l19]], np.float32)
    e, _ = oracle.ece(z, np.array([1], np.int32), M=10)
    assert e == pytest.approx(abs((1 - 0.95) + (0 - 0.9025)) / 2, abs=1e-6)
    # temperatures divide the logits: T = 2 at the first position of sigma(2 ln 19)
    z = np.array([[2 * l19]], np.float32)
    e, _ = oracle.ece(z, np.array([1], np.int32), T=np.array([2.0], np.float32), M=10)
    assert e == pytest.approx(0.05, abs=1e-6)


def test_ece_one_bin_is_the_mean_gap():
    # with a single bin ECE reduces to |mean accept - mean prediction| over all
    # (sample, position) pairs; the predictions by scipy's logistic function
    import oracle
    from scipy.special import expit
    z, acc = _calib(3000, 4, seed=11)
    T = np.array([1.2, 1.7, 0.9, 2.5], np.float32)
    a = np.cumprod(expit(z.astype(np.float64) / T.astype(np.float64)), axis=1)
    s = (acc[:, None] > np.arange(4)[None, :]).astype(np.float64)
    e, _ = oracle.ece(z, acc, T=T, M=1)
    assert e == pytest.approx(abs(s.mean() - a.mean()), rel=1e-12, abs=1e-15)


def test_ece_separates_calibrated_from_overconfident():
    import oracle
    t_true = np.array([1.0, 1.0, 1.0])
    z, acc = _calib(40000, 3, seed=5, t_true=t_true)
    e_cal, _ = oracle.ece(z, acc, M=15)
    assert e_cal < 0.01
    z2, acc2 = _calib(40000, 3, seed=5, t_true=np.array([2.5, 2.5, 2.5]))
    e_over, _ = oracle.ece(z2, acc2, M=15)
    assert e_over > 0.05


def test_sts_first_position_is_a_logistic_fit_without_intercept():
    # at the first position the survival is sigma(beta z) itself: the objective
    # is the logistic log loss, minimised here by scipy's bounded search
    import oracle
    from scipy.optimize import minimize_scalar
    from scipy.special import log_expit
    z, acc = _calib(5000, 2, seed=3)
    beta, T, nll, gap = oracle.sts_fit(z, acc)
    x = z[:, 0].astype(np.float64)
    s = (acc > 0).astype(np.float64)

    def loss(b):
        return -np.sum(s * log_expit(b * x) + (1 - s) * log_expit(-b * x))

    lo, hi = 1.0 / 16, 16.0
    res = minimize_scalar(loss, bounds=(lo, hi), method="bounded", options={"xatol": 1e-10})
    step1 = (hi - lo) / 255
    step2 = 2 * step1 / 255
    assert abs(beta[0] - res.x) <= step2
    assert nll[0] == pytest.approx(loss(beta[0]), rel=1e-12)
    assert nll[0] >= res.fun - 1e-9


def test_sts_recovers_generating_temperatures():
    import oracle
    t_true = np.array([1.5, 2.0, 1.2, 1.8])
    z, acc = _calib(20000, 4, seed=7, t_true=t_true)
    beta, T, nll, gap = oracle.sts_fit(z, acc)
    assert np.all(np.abs(T / t_true - 1) < 0.08), (T, t_true)
    e_before, _ = oracle.ece(z, acc)
    e_after, _ = oracle.ece(z, acc, T=T)
    assert e_after < 0.5 * e_before


def test_sts_fit_is_sequential_and_on_grid():
    import oracle
    z, acc = _calib(2000, 3, seed=9)
    beta, T, nll, gap = oracle.sts_fit(z, acc)
    z2 = z.copy()
    z2[:, 2] = -z2[:, 2] + 0.5
    beta2, _, _, _ = oracle.sts_fit(z2, acc)
    # a later position's logits cannot move an earlier temperature
    assert beta2[0] == beta[0] and beta2[1] == beta[1]
    assert beta2[2] != beta[2]
    # every fitted beta is a point of its second grid, inside [1/16, 16]
    assert np.all((beta >= 1.0 / 16) & (beta <= 16.0))
    assert np.all(gap >= 0)


def test_sts_degenerate_all_zero_logits_take_the_first_grid_point():
    import oracle
    z = np.zeros((100, 2), np.float32)
    acc = np.full(100, 1, np.int32)
    beta, T, nll, gap = oracle.sts_fit(z, acc, t_lo=0.25, t_hi=4.0)
    # sigma(beta 0) = 1/2 for every beta: a tie everywhere, the lowest index wins
    assert np.all(beta == 0.25) and np.all(T == 4.0)
    assert nll[0] == pytest.approx(100 * math.log(2.0), rel=1e-15)


def test_confidence_logit_is_the_sigmoid_argument():
    import oracle
    rng = np.random.default_rng(2)
    n, gamma, d, V, r = 3, 4, 16, 32, 8
    h = bf16(rng.normal(0, 1, (n, gamma, d)))
    E = bf16(rng.normal(0, 0.1, (V, r)))
    anchor = rng.integers(0, V, n).astype(np.int32)
    tok = rng.integers(0, V, (n, gamma)).astype(np.int32)
    w = rng.normal(0, 0.1, d + r).astype(np.float32)
    T = np.array([1.0, 1.3, 0.7, 2.0], np.float32)
    off = rng.normal(0, 1, n).astype(np.float32)
    y = oracle.confidence_logit(h, E, anchor, tok, w, off)
    c, _ = oracle.confidence(h, E, anchor, tok, w, T, off)
    from scipy.special import expit
    np.testing.assert_allclose(c, expit(y / T[None, :].astype(np.float64)), rtol=1e-14)


# ---------------------------------------------------------------------------
# Recurrent sequential head (page "DeepSeek联合北大最新文章DSpark", 第二阶段轻量
# 顺序头: an RNN head that keeps a recurrent state; its form is this library's
# reading, an Elman recurrence s_k = bf16(tanh(A s_{k-1} + E[x_{k-1}]))).
# ---------------------------------------------------------------------------
def _rnn_setup(V, r, seed, a_scale=0.3):
    rng = np.random.default_rng(seed)
    E = bf16(rng.normal(0, 0.8, (V, r)))
    W2 = bf16(rng.normal(0, 0.5, (V, r)))
    A = bf16(rng.normal(0, a_scale / math.sqrt(r), (r, r)))
    return E, W2, A


def test_rnn_state_is_an_elman_cell():
    # torch's RNN cell with identity input weights, no biases and tanh is the
    # recurrence; the oracle rounds every state to bf16 (nearest even) and
    # feeds the rounded state forward, so each step is compared from the
    # oracle's previous state
    import oracle
    V, r = 40, 24
    E, W2, A = _rnn_setup(V, r, 1)
    cell = torch.nn.RNNCell(r, r, bias=False, nonlinearity="tanh").double()
    with torch.no_grad():
        cell.weight_ih.copy_(torch.eye(r, dtype=torch.float64))
        cell.weight_hh.copy_(torch.as_tensor(bf16_val(A), dtype=torch.float64))
    s = None
    exact = total = 0
    for x in [3, 17, 0, 39, 17, 5, -1, 8]:
        out, fl = oracle.rnn_state(A, E, x, s)
        assert not fl
        h = torch.zeros(1, r, dtype=torch.float64) if s is None else \
            torch.as_tensor(bf16_val(s), dtype=torch.float64)[None]
        e = torch.zeros(1, r, dtype=torch.float64) if x < 0 else \
            torch.as_tensor(bf16_val(E[x]), dtype=torch.float64)[None]
        with torch.no_grad():
            ref = cell(e, h)[0].numpy()
        got = bf16_val(out).astype(np.float64)
        ulp = np.spacing(np.abs(ref).astype(np.float32)) * 65536.0   # one bf16 ulp
        assert np.all(np.abs(got - ref) <= 0.5 * ulp * (1 + 1e-9))
        exact += int(np.sum(got == torch.as_tensor(ref).to(torch.bfloat16).double().numpy()))
        total += r
        s = out
    assert exact >= total - 2


def test_rnn_with_zero_recurrence_is_the_markov_head_on_its_state_table():
    import oracle
    V, r, gamma, n = 64, 16, 5, 6
    E, W2, _ = _rnn_setup(V, r, 2)
    A0 = np.zeros((r, r), np.uint16)
    Et = np.stack([oracle.rnn_state(A0, E, v)[0] for v in range(V)])
    rng = np.random.default_rng(3)
    base = rng.normal(0, 2, (n, gamma, V)).astype(np.float32)
    anchor = rng.integers(0, V, n).astype(np.int32)
    req = np.arange(n, dtype=np.int32)
    for temp in (1.0, 0.0):
        t1, q1, s1, f1, S, sf = oracle.draft(base, E, W2, anchor, req, temp, 7, 1, A=A0)
        t2, q2, s2, f2 = oracle.draft(base, Et, W2, anchor, req, temp, 7, 1)
        assert np.array_equal(t1, t2) and np.array_equal(q1, q2) and np.array_equal(s1, s2)
        prev = np.concatenate([anchor[:, None], t1[:, :-1]], axis=1)
        assert np.array_equal(S, Et[prev])


def test_rnn_state_remembers_beyond_one_token():
    # with the previous token forced equal, the state of position 1 still sees
    # the anchor through A; without recurrence it does not
    import oracle
    V, r, gamma = 32, 16, 3
    E, W2, A = _rnn_setup(V, r, 4, a_scale=1.0)
    base = np.zeros((2, gamma, V), np.float32)
    anchor = np.array([1, 2], np.int32)
    req = np.array([0, 0], np.int32)
    force = np.full((2, gamma), -1, np.int32)
    force[:, 0] = 5
    _, _, _, _, S, _ = oracle.draft(base, E, W2, anchor, req, 1.0, 0, 0, force=force, A=A)
    assert not np.array_equal(S[0, 1], S[1, 1])
    _, _, _, _, S0, _ = oracle.draft(base, E, W2, anchor, req, 1.0, 0, 0, force=force,
                                     A=np.zeros_like(A))
    assert np.array_equal(S0[0, 1], S0[1, 1])


def test_rnn_draft_verification_is_lossless():
    # the first emitted token (accepted draft token or the correction / bonus
    # draw) follows the target law p_0 whatever the draft law: chi-square over a
    # 6-token vocabulary with a recurrent draft
    import oracle
    V, r, gamma, n = 6, 8, 2, 60000
    E, W2, A = _rnn_setup(V, r, 5, a_scale=1.0)
    rng = np.random.default_rng(6)
    base1 = rng.normal(0, 1.5, (gamma, V)).astype(np.float32)
    tgt1 = rng.normal(0, 1.5, (gamma + 1, V)).astype(np.float32)
    base = np.broadcast_to(base1, (n, gamma, V)).copy()
    target = np.broadcast_to(tgt1, (n, gamma + 1, V)).copy()
    anchor = np.full(n, 2, np.int32)
    req = np.arange(n, dtype=np.int32)
    tok, q, st, fl, S, sf = oracle.draft(base, E, W2, anchor, req, 1.0, 11, 3, A=A)
    v = oracle.verify(target, base, E, W2, anchor, tok, q, np.full(n, gamma, np.int32), req, 1.0,
                      11, 3, S=S)
    first = np.where(v["n_accept"] > 0, tok[:, 0], v["y"])
    p0 = sp_softmax(tgt1[0].astype(np.float64))
    counts = np.bincount(first, minlength=V)
    stat, pval = sst.chisquare(counts, n * p0)
    assert pval > 1e-4, (counts, n * p0)
    # and the draft law itself differs from p_0 (the test is not vacuous)
    counts_d = np.bincount(tok[:, 0], minlength=V)
    assert sst.chisquare(counts_d, n * p0)[1] < 1e-6
