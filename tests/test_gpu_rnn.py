"""The recurrent sequential head on the GPU vs the CPU oracle, through the C-ABI.

Draft (dsp_draft_step_rnn), verification (dsp_verify_rnn) and the exact
acceptance probability (dsp_tv_accept_rnn) with the recurrent head.  The states
must be bit-identical (bf16) except where the oracle flags a tanh value next to
a bf16 rounding midpoint; tokens, probabilities and accept decisions follow the
parity rules of the Markov head (teacher forcing at a flagged sampling
decision); the verification and the acceptance probabilities are computed on
both sides from the GPU's states.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from oracle.compare import Tally, draft_forced, verify_forced
from draft_sampling_lossless_markov_amd import dsp
from draft_sampling_lossless_markov_amd.workloads import (Workload, _cost_q12, make_inputs,
                                                          place_logits, rnn_matrix)

pytestmark = pytest.mark.gpu

SEED = 0
AGG = Tally()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("the gpu tests need a GPU")
    dsp.lib()


def _wl(R, gamma, V, r, dtype, temperature):
    return Workload(95, f"rnn-R{R}-g{gamma}-V{V}-r{r}", R, gamma, V, r, 8, dtype, 2.0,
                    lambda j, g: 0.7, 0.3, "const:1.0", None, _cost_q12, R * (gamma + 1), 0,
                    temperature)


def _ws(kind, R, gamma, V, r):
    return torch.zeros(dsp.dsp_workspace_size(kind, R, gamma, V, r), dtype=torch.uint8,
                       device="cuda")


def gpu_draft(inp, A, temp, rnd, chunks=None, layout="request"):
    R, gamma, V, r = inp["R"], inp["gamma"], inp["V"], inp["r"]
    base = place_logits(inp["base"], layout, "cuda")
    E, W2, anchor = inp["E"].cuda(), inp["W2"].cuda(), inp["anchor"].cuda()
    tok = torch.zeros(R, gamma, dtype=torch.int32, device="cuda")
    q = torch.zeros(R, gamma, dtype=torch.float32, device="cuda")
    stats = torch.zeros(R, gamma, 2, dtype=torch.float64, device="cuda")
    S = torch.full((R, gamma, r), 0x7fc0, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ws = _ws(dsp.DSP_WS_DRAFT, R, gamma, V, r)
    k = 0
    for n in (chunks or [gamma]):
        dsp.dsp_draft_step_rnn(base, E, W2, A.cuda(), anchor, tok, q, stats, S, k, temp, SEED, rnd,
                               ws, n_steps=n)
        k += n
    torch.cuda.synchronize()
    return base, tok, q, stats, S


def oracle_draft(inp, A, g_tok, g_q, g_stats, temp, rnd, subset):
    E = orc.bf16_bits(inp["E"])
    W2 = orc.bf16_bits(inp["W2"])
    Ab = orc.bf16_bits(A)
    anchor = inp["anchor"].numpy()
    base = orc.host_logits(inp["base"])[subset]
    S_o = {}

    def rows(i, force_row):
        f = None if force_row is None else force_row[None]
        n = subset[i:i + 1]
        tok, q, st, fl, S, sf = orc.draft(base[i:i + 1], E, W2, anchor[n], n, temp, SEED, rnd,
                                          force=f, A=Ab)
        S_o[i] = (S[0], sf[0])
        return tok[0], q[0], st[0], fl[0]

    t, o_tok, o_q, o_stats, o_flag = draft_forced(g_tok[subset], g_q[subset], g_stats[subset],
                                                  rows, temp == 0.0, subset, threads=8)
    # the states of the final (forced) chains
    S = np.stack([S_o[i][0] for i in range(len(subset))])
    sflag = np.stack([S_o[i][1] for i in range(len(subset))])
    return t, o_tok, o_q, S, sflag


def check_states(g_S, o_S, sflag, o_tok, g_tok):
    """Bit-identical states up to the first token the chains disagree on (states
    after it follow different tokens), unless the oracle flags the state."""
    n, gamma, r = o_S.shape
    for i in range(n):
        for k in range(gamma):
            if not np.array_equal(g_S[i, k], o_S[i, k]):
                assert sflag[i, k], (i, k, np.nonzero(g_S[i, k] != o_S[i, k])[0][:5])
            if g_tok[i, k] != o_tok[i, k]:
                break


CASES = [
    # (R, gamma, V, r, dtype, temperature, chunks)
    (4, 4, 32, 8, torch.float32, 1.0, None),
    (4, 4, 32, 8, torch.float32, 0.0, [1, 3]),
    (33, 3, 1003, 24, torch.float32, 0.8, None),          # ragged V: element-wise passes
    (70, 5, 1000, 24, torch.bfloat16, 1.0, [2, 2, 1]),
    (64, 4, 4096, 64, torch.bfloat16, 1.0, None),         # 16-byte rows: the pipelined pass
    (64, 4, 4096, 64, torch.bfloat16, 0.0, None),
    (130, 3, 2048, 256, torch.bfloat16, 1.3, [3]),        # several request blocks, full rank
    (1, 1, 1, 8, torch.float32, 1.0, None),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"R{c[0]}g{c[1]}V{c[2]}r{c[3]}T{c[5]}")
def test_rnn_round_vs_oracle(case):
    R, gamma, V, r, dtype, temp, chunks = case
    inp = make_inputs(_wl(R, gamma, V, r, dtype, temp), 0, "cpu")
    A = rnn_matrix(r, seed=R + V)
    rnd = 3
    base, tok, q, stats, S = gpu_draft(inp, A, temp, rnd, chunks)
    g_tok, g_q, g_stats = tok.cpu().numpy(), q.cpu().numpy(), stats.cpu().numpy()
    g_S = S.cpu().view(torch.int16).numpy().view(np.uint16)
    subset = np.arange(R, dtype=np.int32)
    t, o_tok, o_q, o_S, sflag = oracle_draft(inp, A, g_tok, g_q, g_stats, temp, rnd, subset)
    assert t.ok(), t.summary()
    if temp == 0.0:
        assert t.diverged == 0, t.summary()
    check_states(g_S, o_S, sflag, o_tok, g_tok)
    AGG.add(Tally(decisions=t.decisions, flagged=t.flagged, diverged=t.diverged))

    # verification of ragged prefixes with the GPU's states, against the oracle's
    gen = torch.Generator().manual_seed(R)
    length = torch.randint(0, gamma + 1, (R,), generator=gen, dtype=torch.int32)
    target = place_logits(inp["target"], "request", "cuda", pad_target=True)
    acc = torch.zeros(R, gamma, dtype=torch.int8, device="cuda")
    n_acc = torch.zeros(R, dtype=torch.int32, device="cuda")
    y = torch.zeros(R, dtype=torch.int32, device="cuda")
    p = torch.zeros(R, gamma, dtype=torch.float32, device="cuda")
    ws = _ws(dsp.DSP_WS_VERIFY, R, gamma, V, r)
    dsp.dsp_verify_rnn(target, base, inp["E"].cuda(), inp["W2"].cuda(), S, inp["anchor"].cuda(),
                       tok, q, stats, length.cuda(), acc, n_acc, y, p, temp, SEED, rnd, ws)
    torch.cuda.synchronize()
    g_v = {"accept": acc.cpu().numpy(), "n_accept": n_acc.cpu().numpy(), "y": y.cpu().numpy(),
           "p": p.cpu().numpy()}
    E_h, W2_h = orc.bf16_bits(inp["E"]), orc.bf16_bits(inp["W2"])
    tgt_h, base_h = orc.host_logits(inp["target"]), orc.host_logits(inp["base"])
    anchor = inp["anchor"].numpy()
    lens = length.numpy()

    def v_rows(i, force_row):
        f = None if force_row is None else force_row[None]
        v = orc.verify(tgt_h[i:i + 1], base_h[i:i + 1], E_h, W2_h, anchor[i:i + 1], g_tok[i:i + 1],
                       g_q[i:i + 1].astype(np.float64), lens[i:i + 1], subset[i:i + 1], temp, SEED,
                       rnd, force_acc=f, S=g_S[i:i + 1])
        return {k: v[k][0] for k in v}

    tv, _ = verify_forced(g_v, v_rows, lens, temp == 0.0, subset, threads=8)
    assert tv.ok(), tv.summary()
    if temp == 0.0:
        assert tv.diverged == 0, tv.summary()
    AGG.add(Tally(decisions=tv.decisions, flagged=tv.flagged, diverged=tv.diverged))

    # the exact acceptance probability of every position, from the same states
    if temp > 0.0:
        alpha = torch.zeros(R, gamma, dtype=torch.float64, device="cuda")
        wst = _ws(dsp.DSP_WS_TV, R, gamma, V, r)
        dsp.dsp_tv_accept_rnn(target, base, inp["E"].cuda(), inp["W2"].cuda(), S,
                              inp["anchor"].cuda(), tok, stats, alpha, temp, wst)
        torch.cuda.synchronize()
        o = orc.tv_accept(tgt_h, base_h, E_h, W2_h, anchor, g_tok, temp, S=g_S)
        np.testing.assert_allclose(alpha.cpu().numpy(), o, rtol=1e-5, atol=1e-7)


def test_rnn_zero_recurrence_matches_the_markov_entry_on_the_state_table():
    # A = 0: the recurrent draft is the Markov draft on bf16(tanh(E)) -- both on
    # the GPU, bit for bit (same passes, same picks)
    R, gamma, V, r = 64, 4, 4096, 64
    inp = make_inputs(_wl(R, gamma, V, r, torch.bfloat16, 1.0), 1, "cpu")
    A0 = torch.zeros(r, r, dtype=torch.bfloat16)
    base, tok, q, stats, S = gpu_draft(inp, A0, 1.0, 4)
    Et = torch.tanh(inp["E"].double())
    E_bits = orc.bf16_bits(inp["E"])
    # the table as the oracle rounds it (tanh in fp64, nearest even)
    Et_bits = np.stack([orc.rnn_state(np.zeros((r, r), np.uint16), E_bits, v)[0] for v in range(V)])
    Et_t = torch.as_tensor(Et_bits.view(np.int16)).view(torch.bfloat16)
    tok2 = torch.zeros_like(tok)
    q2 = torch.zeros_like(q)
    st2 = torch.zeros_like(stats)
    ws = _ws(dsp.DSP_WS_DRAFT, R, gamma, V, r)
    dsp.dsp_draft_step(base, Et_t.cuda(), inp["W2"].cuda(), inp["anchor"].cuda(), tok2, q2, st2, 0,
                       1.0, SEED, 4, ws, n_steps=gamma, flags=dsp.DSP_PATH_STREAMING)
    torch.cuda.synchronize()
    assert torch.equal(tok, tok2) and torch.equal(q, q2) and torch.equal(stats, st2)
    del Et


def test_rnn_persistent_path_is_refused():
    R, gamma, V, r = 4, 2, 64, 8
    inp = make_inputs(_wl(R, gamma, V, r, torch.bfloat16, 1.0), 0, "cpu")
    A = rnn_matrix(r, 1)
    with pytest.raises(dsp.DspError) as e:
        base = inp["base"].cuda()
        tok = torch.zeros(R, gamma, dtype=torch.int32, device="cuda")
        q = torch.zeros(R, gamma, dtype=torch.float32, device="cuda")
        st = torch.zeros(R, gamma, 2, dtype=torch.float64, device="cuda")
        S = torch.zeros(R, gamma, r, dtype=torch.bfloat16, device="cuda")
        dsp.dsp_draft_step_rnn(base, inp["E"].cuda(), inp["W2"].cuda(), A.cuda(),
                               inp["anchor"].cuda(), tok, q, st, S, 0, 1.0, SEED, 0,
                               _ws(dsp.DSP_WS_DRAFT, R, gamma, V, r), n_steps=gamma,
                               flags=dsp.DSP_PATH_PERSISTENT)
    assert e.value.status == dsp.DSP_ERR_UNSUPPORTED


def test_zz_rnn_mismatch_rate_over_the_module():
    print(f"  recurrent head, all cases: {AGG.summary()}", flush=True)
    assert AGG.ok()
    assert AGG.mismatch_rate() <= 1e-4 or AGG.diverged <= 2
