"""Seeded synthetic inputs for one layer of a workload.

Recipe (all draws from one torch.Generator seeded per (workload, layer, seed)):

* q, k, v ~ N(0, 1) in fp32, shape [batch, heads, N, d] with N = P + T.
* Structure, added to the keys in fp32 before rounding:
  - "dirs4": 4 directions per layer, each a N(0, I) vector rescaled to norm
    sqrt(d); floor(frac * N) positions per sequence are drawn uniformly
    without replacement and each gets 3 x one of the 4 directions (chosen
    uniformly).  The logit shift q.(3u)/sqrt(d) then has standard deviation 3,
    so attention is sparse.
  - "zipf_dir": one direction per (layer, head) with norm sqrt(d);
    floor(frac * N) positions per sequence are drawn without replacement with
    weights proportional to (i + 1)^-1.1, and every head of that sequence adds
    3 x its direction at those positions.
  - "clusters": 8 centres per (layer, head) ~ N(0, I); every (sequence, head,
    position) gets a uniform cluster a and k = z + c_a, q = z' + c_a.
* Rounding to the storage dtype is round-to-nearest-even (torch's cast); both
  the oracle and the GPU consume these same rounded values.
* Token ids (FastGen): Zipf(1.1) ranks over the vocabulary, id = rank - 1.
* HashEvict projection: one [d, bits] N(0, 1) matrix per layer, rounded to bf16.

The generator runs on any torch device; on the GPU it fills HBM directly.  The
CPU and GPU random streams differ for the same seed, so a test that needs the
same values on both sides generates once and copies.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np
import torch

from .configs import Workload

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass
class LayerInputs:
    """Inputs of one layer, already in the layouts the library expects.

    prompt_q/k/v: [batch, heads, P, d] storage dtype, contiguous.
    dec_q/k/v:    [T, batch, heads, d] storage dtype, contiguous (step-major).
    ids:          [batch, N] int32 or None.
    proj:         [d, bits] bfloat16 or None.
    """
    prompt_q: torch.Tensor
    prompt_k: torch.Tensor
    prompt_v: torch.Tensor
    dec_q: torch.Tensor
    dec_k: torch.Tensor
    dec_v: torch.Tensor
    ids: Optional[torch.Tensor]
    proj: Optional[torch.Tensor]

    def to(self, device) -> "LayerInputs":
        f = lambda x: None if x is None else x.to(device)
        return LayerInputs(*(f(getattr(self, n)) for n in
                             ("prompt_q", "prompt_k", "prompt_v", "dec_q", "dec_k", "dec_v", "ids", "proj")))


def layer_seed(w: Workload, layer: int, seed: int = 0) -> int:
    return (1000 + w.index) * 1_000_003 + layer * 7919 + seed * 104_729


def _unit_dirs(gen, n: int, d: int, device) -> torch.Tensor:
    u = torch.randn((n, d), generator=gen, device=device, dtype=torch.float32)
    return u * (d ** 0.5) / u.norm(dim=-1, keepdim=True)


def _zipf_ids(w: Workload, gen, Bt: int, N: int, device) -> torch.Tensor:
    """Token ids [Bt, N]: Zipf(1.1) ranks over the vocabulary, id = rank - 1."""
    ranks = torch.arange(1, w.vocab + 1, device=device, dtype=torch.float64) ** -1.1
    return torch.multinomial(ranks.expand(Bt, -1), N, replacement=True, generator=gen).to(torch.int32)


HEAD_KINDS = ("special", "punct", "local", "frequent", "broad")


def head_kinds(w: Workload, layer: int = 0):
    """Kind of each head of a layer under the "head_kinds" structure: a
    balanced assignment of the five kinds, shuffled with a seed per layer."""
    rng = np.random.default_rng([w.index, 11, layer])
    base = [HEAD_KINDS[i % len(HEAD_KINDS)] for i in range(w.heads)]
    return [base[i] for i in rng.permutation(w.heads)]


def _add_head_kinds(w: Workload, gen, q, k, ids, n_pos: int, device, layer: int = 0) -> None:
    """Per-head attention structures after the FastGen page's Figure 1: heads
    drawn to special tokens, to special and punctuation tokens, to the recent
    past, to a few frequently attended positions, or to everything."""
    Bt, H, N, d = q.shape
    dirs = _unit_dirs(gen, H, d, device)
    special = torch.tensor(list(w.special_ids), device=device)
    sp_punct = torch.tensor(list(w.special_ids) + list(w.punct_ids), device=device)
    weights = (torch.arange(N, device=device, dtype=torch.float64) + 1.0) ** -1.1
    pos_angle = 2.0 * np.pi * torch.arange(N, device=device, dtype=torch.float32) / (2.0 * N)
    for h, kind in enumerate(head_kinds(w, layer)):
        u = dirs[h]
        if kind in ("special", "punct"):
            keep = torch.isin(ids, special if kind == "special" else sp_punct)      # [Bt, N]
            k[:, h] += 1.5 * keep.unsqueeze(-1).float() * u
            q[:, h] += 0.5 * u
        elif kind == "local":
            # a slowly turning 2-d phase: q_i . k_j grows as |i - j| shrinks
            amp = 11.0
            k[:, h, :, 0] += amp * torch.cos(pos_angle)
            k[:, h, :, 1] += amp * torch.sin(pos_angle)
            q[:, h, :, 0] += amp * torch.cos(pos_angle)
            q[:, h, :, 1] += amp * torch.sin(pos_angle)
        elif kind == "frequent":
            for b in range(Bt):
                pos = torch.multinomial(weights, max(1, n_pos), replacement=False, generator=gen)
                k[b, h, pos] += 1.5 * u
            q[:, h] += 0.5 * u


def generate_layer(w: Workload, layer: int = 0, device="cpu", seed: int = 0) -> LayerInputs:
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(layer_seed(w, layer, seed))
    Bt, H, P, T, d = w.batch, w.heads, w.prompt, w.steps, w.head_dim
    N = P + T
    sd = TORCH_DTYPES[w.dtype]
    shape = (Bt, H, N, d)

    def randn():
        return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)

    ids = None
    proj = None
    if w.structure == "clusters":
        centres = torch.randn((H, 8, d), generator=gen, device=device, dtype=torch.float32)
        assign = torch.randint(0, 8, (Bt, H, N), generator=gen, device=device)
        hidx = torch.arange(H, device=device).view(1, H, 1).expand(Bt, H, N)
        c = centres[hidx, assign]                        # [Bt, H, N, d]
        k = randn() + c
        q = randn() + c
        del c
        v = randn()
    else:
        q = randn()
        k = randn()
        v = randn()
        n_pos = int(w.heavy_frac_positions * N)
        if w.structure == "dirs4":
            dirs = _unit_dirs(gen, 4, d, device)
            for b in range(Bt):
                pos = torch.randperm(N, generator=gen, device=device)[:n_pos]
                which = torch.randint(0, 4, (n_pos,), generator=gen, device=device)
                k[b, :, pos, :] += 3.0 * dirs[which].unsqueeze(0)
        elif w.structure == "zipf_dir":
            dirs = _unit_dirs(gen, H, d, device)            # one per head
            weights = (torch.arange(N, device=device, dtype=torch.float64) + 1.0) ** -1.1
            for b in range(Bt if n_pos > 0 else 0):         # sequences too short to carry one
                pos = torch.multinomial(weights, n_pos, replacement=False, generator=gen)
                k[b, :, pos, :] += 3.0 * dirs.unsqueeze(1)
        elif w.structure == "head_kinds":
            ids = _zipf_ids(w, gen, Bt, N, device)
            _add_head_kinds(w, gen, q, k, ids, n_pos, device)
        else:
            raise ValueError(w.structure)
    if w.family == "fastgen" or (w.family == "adaptive" and ids is None):
        ids = _zipf_ids(w, gen, Bt, N, device)
    if w.family == "hash":
        proj = torch.randn((d, w.sketch_bits), generator=gen, device=device,
                           dtype=torch.float32).to(torch.bfloat16)

    def split(x):
        x = x.to(sd)
        return x[:, :, :P, :].contiguous(), x[:, :, P:, :].permute(2, 0, 1, 3).contiguous()

    pq, dq = split(q); del q
    pk, dk = split(k); del k
    pv, dv = split(v); del v
    return LayerInputs(pq, pk, pv, dq, dk, dv, ids, proj)


def unit_sequence(inp: LayerInputs, b: int, h: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Full-length (P + T) q, k, v of one unit as float64 numpy arrays [N, d].

    Values are the storage-dtype values upcast exactly.
    """
    def cat(p, dd):
        return torch.cat([p[b, h].float(), dd[:, b, h].float()], dim=0).cpu().double().numpy()
    return (cat(inp.prompt_q, inp.dec_q), cat(inp.prompt_k, inp.dec_k), cat(inp.prompt_v, inp.dec_v))


def unit_ids(inp: LayerInputs, b: int) -> Optional[np.ndarray]:
    return None if inp.ids is None else inp.ids[b].cpu().numpy().astype(np.int64)
