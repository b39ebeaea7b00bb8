"""dsp_draft_step_noalloc (the allocation-free draft entry point, its scratch a
static per-device array of the library) against dsp_draft_step with a caller
workspace: identical tokens, q and (M, Z) statistics, on two calls in a row, the
second with a smaller input, for the persistent and the streaming draft paths."""
import numpy as np
import pytest
import torch

from draft_sampling_lossless_markov_amd import dsp
from draft_sampling_lossless_markov_amd.engine import Round
from draft_sampling_lossless_markov_amd.workloads import Workload, _cost_q12, make_inputs, place_logits

pytestmark = pytest.mark.gpu


def _case(R, gamma, V, r, idx):
    wl = Workload(idx, f"noalloc-R{R}-g{gamma}-V{V}", R, gamma, V, r, 8, torch.bfloat16, 2.0,
                  lambda j, g: 0.7, 0.1, "const:1.0", None, _cost_q12, R * (gamma + 1), 1, 1.0)
    inp = make_inputs(wl, 0, layout="position")
    out = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    out["base"] = place_logits(inp["base"], "position", "cuda")
    return out


def _outputs(rd):
    torch.cuda.synchronize()
    return [t.cpu().numpy().copy() for t in (rd.tok, rd.q, rd.stats)]


@pytest.mark.parametrize("flags", [dsp.DSP_PATH_AUTO, dsp.DSP_PATH_STREAMING])
@pytest.mark.parametrize("temp", [1.0, 0.0])
def test_noalloc_matches_workspace_entry_point(flags, temp):
    for (R, gamma, V, r), rnd in (((100, 3, 110000, 256), 3), ((33, 2, 40000, 64), 4)):
        print(f"noalloc vs workspace draft: R{R} g{gamma} V{V} r{r} flags {flags} T {temp}", flush=True)
        inp = _case(R, gamma, V, r, 95)
        rd = Round(R, gamma, V, r)
        args = (inp["base"], inp["E"], inp["W2"], inp["anchor"], rd.tok, rd.q, rd.stats, 0, temp, 0,
                rnd)
        rd.tok.fill_(-5)
        dsp.dsp_draft_step(*args, rd.ws_draft, n_steps=gamma, flags=flags)
        ref = _outputs(rd)
        rd.check()
        rd.tok.fill_(-5)
        rd.q.fill_(-1.0)
        rd.stats.fill_(-1.0)
        dsp.dsp_draft_step_noalloc(*args, n_steps=gamma, flags=flags)
        got = _outputs(rd)
        for a, b in zip(ref, got):
            assert np.array_equal(a, b, equal_nan=False)
        assert np.all((ref[0] >= 0) & (ref[0] < V))
        del rd, inp
    torch.cuda.empty_cache()


def test_noalloc_rejects_sizes_beyond_its_scratch():
    R, gamma, V, r = 2048, 2, 262144, 256
    assert dsp.dsp_workspace_size(dsp.DSP_WS_DRAFT, R, gamma, V, r) > 16 << 20
    base = torch.zeros((R, gamma, V), dtype=torch.bfloat16, device="cuda")
    E = torch.zeros((V, r), dtype=torch.bfloat16, device="cuda")
    rd = Round(4, gamma, 32, 8)
    anchor = torch.zeros(R, dtype=torch.int32, device="cuda")
    tok = torch.zeros((R, gamma), dtype=torch.int32, device="cuda")
    with pytest.raises(dsp.DspError) as ei:
        dsp.dsp_draft_step_noalloc(base, E, E, anchor, tok, rd.q, rd.stats, 0, 1.0, 0, 0,
                                   n_steps=gamma)
    assert ei.value.status == dsp.DSP_ERR_WORKSPACE
