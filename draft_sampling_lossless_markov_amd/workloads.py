"""Seeded synthetic workloads for the DSpark sampling / verification path.

This module only draws random tensors and builds lookup tables; it holds none
of the method's arithmetic.  Both the HIP path and the CPU oracle take their
inputs from here, so the two sides always see identical bytes.

Shapes and value laws follow the workloads described for DSpark (DSpark
paper summaries: page "DeepSeek联合北大最新文章DSpark", section 2.2 for the
SPS(B) table and the scheduler; page "DSpark.让每一轮计算，多走几步" for the
toy cost curve T(B) = 12 + (0.06 + 0.04 L) B + 0.0008 L B^2 ms, here with
L = 1).  The backbone and target models are not run: their outputs are drawn
as Gaussian logits of the stated shapes.

Layouts (row-major, last index contiguous):
  base    [R, gamma,   V]  draft base logits (fp32 or bf16); a view whose
                           storage is [R, gamma, V] (layout "request"),
                           [gamma, R, V] ("position": each draft position one
                           contiguous [R, V] slab) or [R, gamma, V + 64]
                           ("padded": rows of base and target padded by 64);
                           the values do not depend on the layout
  target  [R, gamma+1, V]  target logits; row j is the law of draft position j,
                           row gamma is the bonus row
  E       [V, r]  bf16     Markov embedding (W1 on the pages)
  W2      [V, r]  bf16     the low-rank output factor, stored transposed:
                           element (i, v) of the pages' r x V matrix is W2[v, i]
  h       [R, gamma, d] bf16  backbone hidden states
  w       [d + r] fp32     confidence-head weight
  T       [gamma] fp32     sequential temperature-scaling divisors
  offset  [R] fp32 or None per-request confidence-logit offset
  sps     [B_max] fp32     sps[B-1] = SPS(B)
  anchor  [R] int32        last token emitted by the target
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Optional

import torch


def _cost_q12(B: torch.Tensor) -> torch.Tensor:
    # Toy step cost of the interactive explainer with its slider at L = 1.
    return 12.0 + 0.1 * B + 0.0008 * B * B


def _cost_cfg3(B: torch.Tensor) -> torch.Tensor:
    return 12.0 + 0.05 * B + 0.0004 * B * B


@dataclass(frozen=True)
class Workload:
    idx: int
    name: str
    R: int
    gamma: int
    V: int
    r: int
    d: int
    logit_dtype: torch.dtype
    base_std: float
    noise_std: Callable[[int, int], float]  # (row j, gamma) -> sigma of target noise
    emb_std: float
    T_law: str              # "const:<x>" or "uniform:<lo>:<hi>"
    offset_range: Optional[float]
    cost: Callable[[torch.Tensor], torch.Tensor]
    B_max: int
    mode: int               # 0 scheduler off (every position verified), 1 greedy early stop
    temperature: float
    modes: tuple = ("sampling",)
    rounds: int = 100
    tau0: float = 0.0


WORKLOADS = {
    0: Workload(0, "tiny-R4-g4-V32-r8-d16-fp32", 4, 4, 32, 8, 16, torch.float32, 2.0,
                lambda j, g: 0.5, 0.1, "const:1.2", None, _cost_q12, 20, 1, 1.0,
                modes=("greedy", "sampling"), rounds=1000),
    1: Workload(1, "qwen3-4b-R64-g7-V151936-r256-d2560-bf16", 64, 7, 151936, 256, 2560,
                torch.bfloat16, 3.0, lambda j, g: 1.0, 0.02, "const:1.0", None,
                _cost_q12, 64 * 8, 0, 1.0, rounds=100),
    2: Workload(2, "long-block-R256-g16-V151936-r256-d4096-bf16", 256, 16, 151936, 256, 4096,
                torch.bfloat16, 3.0,
                lambda j, g: 0.5 + 1.5 * min(j, g - 1) / (g - 1) if j < g else 2.0,
                0.02, "uniform:1.0:1.5", None, _cost_q12, 4352, 1, 1.0, rounds=100),
    3: Workload(3, "ragged-R512-g7-V129280-r256-d7168-bf16", 512, 7, 129280, 256, 7168,
                torch.bfloat16, 3.0, lambda j, g: 1.0, 0.02, "const:1.0", 2.0,
                _cost_cfg3, 4096, 1, 1.0, rounds=100),
    4: Workload(4, "large-R2048-g8-V262144-r256-d3840-bf16", 2048, 8, 262144, 256, 3840,
                torch.bfloat16, 3.0, lambda j, g: 1.0, 0.02, "const:1.0", None,
                _cost_q12, 18432, 1, 1.0, modes=("greedy", "sampling"), rounds=200),
}


def sps_table(cost: Callable[[torch.Tensor], torch.Tensor], B_max: int) -> torch.Tensor:
    """SPS(B) = 1 / T(B) for B = 1..B_max, evaluated in fp64 and stored as fp32."""
    B = torch.arange(1, B_max + 1, dtype=torch.float64)
    return (1.0 / cost(B)).to(torch.float32)


def _temps(law: str, gamma: int, g: torch.Generator, device) -> torch.Tensor:
    kind, *args = law.split(":")
    if kind == "const":
        return torch.full((gamma,), float(args[0]), dtype=torch.float32, device=device)
    lo, hi = float(args[0]), float(args[1])
    u = torch.rand(gamma, generator=g, device=device, dtype=torch.float32)
    return lo + (hi - lo) * u


BASE_LAYOUTS = ("request", "position", "padded")
# The layout of the measured configuration: the draft base logits position-major,
# so that each draft step streams one contiguous [R, V] slab.
BENCH_LAYOUT = "position"


def empty_logits(R: int, P: int, V: int, dtype, device, layout: str, pad_target=False):
    """An uninitialised [R, P, V] logit view whose storage follows `layout`
    (for the target tensor only "padded" changes the storage)."""
    if layout == "position" and not pad_target:
        return torch.empty((P, R, V), dtype=dtype, device=device).permute(1, 0, 2)
    if layout == "padded":
        return torch.empty((R, P, V + 64), dtype=dtype, device=device)[:, :, :V]
    return torch.empty((R, P, V), dtype=dtype, device=device)


def place_logits(t: torch.Tensor, layout: str, device, pad_target=False) -> torch.Tensor:
    """A copy of the [R, P, V] logit tensor t on `device`, stored as `layout`."""
    R, P, V = t.shape
    out = empty_logits(R, P, V, t.dtype, device, layout, pad_target)
    out.copy_(t)
    return out


def make_inputs(wl: Workload, set_idx: int = 0, device="cpu", *, seed_base: int = 0,
                R: Optional[int] = None, V: Optional[int] = None,
                layout: str = "request") -> dict:
    """Draw one seeded input set.  `R`/`V` override the workload's sizes (smaller
    parity cases keep the laws but shrink the shape); `layout` places the base
    logits in memory (one of BASE_LAYOUTS) without changing a value."""
    if layout not in BASE_LAYOUTS:
        raise ValueError(f"layout must be one of {BASE_LAYOUTS}, got {layout!r}")
    R = wl.R if R is None else R
    V = wl.V if V is None else V
    gamma, r, d = wl.gamma, wl.r, wl.d
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed_base + 1000 * wl.idx + set_idx)
    ldt = wl.logit_dtype

    def randn(shape, std, dtype):
        return (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * std).to(dtype)

    # Target row j = draft base row j + noise; one extra base-law row feeds the
    # bonus row gamma of the target.
    base = empty_logits(R, gamma, V, ldt, dev, layout)
    target = empty_logits(R, gamma + 1, V, ldt, dev, layout, pad_target=True)
    for j in range(gamma + 1):
        b = (torch.randn((R, V), generator=g, device=dev, dtype=torch.float32)
             * wl.base_std).to(ldt)
        if j < gamma:
            base[:, j] = b
        nz = torch.randn((R, V), generator=g, device=dev, dtype=torch.float32)
        target[:, j] = (b.float() + nz * wl.noise_std(j, gamma)).to(ldt)
        del b, nz

    E = randn((V, r), wl.emb_std, torch.bfloat16)
    W2 = randn((V, r), wl.emb_std, torch.bfloat16)
    h = randn((R, gamma, d), 1.0, torch.bfloat16)
    w = randn((d + r,), 0.1, torch.float32)
    T = _temps(wl.T_law, gamma, g, dev)
    offset = None
    if wl.offset_range is not None:
        u = torch.rand(R, generator=g, device=dev, dtype=torch.float32)
        offset = (2.0 * u - 1.0) * wl.offset_range
    anchor = torch.randint(0, V, (R,), generator=g, device=dev, dtype=torch.int32)
    B_max = min(wl.B_max, R * (gamma + 1)) if R != wl.R else wl.B_max
    sps = sps_table(wl.cost, B_max).to(dev)
    return dict(base=base, target=target, E=E, W2=W2, h=h, w=w, T=T, offset=offset,
                anchor=anchor, sps=sps, R=R, gamma=gamma, V=V, r=r, d=d, B_max=B_max,
                mode=wl.mode, tau0=wl.tau0, temperature=wl.temperature, layout=layout)


def calibration_set(N: int, gamma: int, seed: int, t_true=None, mu: float = 1.5,
                    sd: float = 1.5, device="cpu"):
    """Held-out calibration data for sequential temperature scaling.

    z [N, gamma] fp32 raw confidence logits ~ N(mu, sd^2); acc [N] int32 the
    number of leading draft positions accepted, drawn position by position:
    given positions 0 .. k-1 accepted, position k is accepted with probability
    1 / (1 + exp(-z[n, k] / t_true[k])).  t_true > 1 makes the raw logits
    overconfident, as the pages describe the uncalibrated head.  This is the
    data law of the synthetic labels, not a step of the method.
    """
    g = torch.Generator().manual_seed(int(seed))
    if t_true is None:
        t_true = torch.linspace(1.3, 2.2, gamma, dtype=torch.float64)
    t_true = torch.as_tensor(t_true, dtype=torch.float64)
    z = (mu + sd * torch.randn(N, gamma, generator=g, dtype=torch.float64)).to(torch.float32)
    u = torch.rand(N, gamma, generator=g, dtype=torch.float64)
    p = torch.sigmoid(z.double() / t_true)
    ok = (u < p).to(torch.int32)
    acc = torch.cumprod(ok, dim=1).sum(dim=1).to(torch.int32)
    return z.to(device), acc.to(device)


def rnn_matrix(r: int, seed: int, scale: float = 0.5, device="cpu") -> torch.Tensor:
    """Recurrent matrix of the recurrent sequential head: [r, r] bf16 with
    entries ~ N(0, scale^2 / r), so that A s keeps the state's scale for a
    unit-scale s (spectral radius about `scale`)."""
    g = torch.Generator().manual_seed(int(seed))
    A = torch.randn(r, r, generator=g, dtype=torch.float32) * (scale / r ** 0.5)
    return A.to(torch.bfloat16).to(device)
