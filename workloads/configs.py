"""The five synthetic workloads, with their sizes and cache budgets.

Budgets given as a percentage are taken of the prompt length and floored per
part (the cache is compressed when it is built from the prompt and then kept
at that size): a 20% H2O budget is floor(0.1 P) heavy-hitter slots plus
floor(0.1 P) recent slots; the FastGen local window is floor(0.25 P) and its
frequency part floor(0.1 P); the HashEvict budget of 50% is floor(0.5 P).

Policy codes match the C header: FULL=0, H2O=1, LOCAL=2, SPECIAL=3, HASH=4,
PERSIST=5.

Beside the five workloads, ``opt30b_decode_persist`` runs the OPT-30B-shaped
decode under the persistence-count rule (the Scissorhands reading) with the
same 20% budget, so the two scoring rules are measured on one shape;
``llama65b_fastgen_profiled`` lets FastGen's profile choose each unit's
composite; ``opt30b_decode_h2o_q4`` and ``hashevict_lsh_q4`` are the
OPT-30B-shaped H2O decode and the HashEvict workload with 4-bit cache slots
(eviction combined with quantisation).
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Dict, List, Tuple

FULL, H2O, LOCAL, SPECIAL, HASH, PERSIST, ADAPTIVE = 0, 1, 2, 3, 4, 5, 6
POLICY_NAMES = {FULL: "full", H2O: "h2o", LOCAL: "local", SPECIAL: "special", HASH: "hash",
                PERSIST: "persist", ADAPTIVE: "adaptive"}


@dataclass(frozen=True)
class Workload:
    name: str
    index: int                 # 1-based position in the workload list; seeds derive from it
    layers: int
    batch: int
    heads: int
    head_dim: int
    dtype: str                 # storage dtype of q/k/v: "f32" | "f16" | "bf16"
    prompt: int                # P
    steps: int                 # T decode steps
    family: str                # "h2o" | "fastgen" | "hash" | "persist" | "adaptive"
    structure: str             # "dirs4" | "zipf_dir" | "clusters" | "head_kinds"
    heavy: int = 0             # H2O heavy-hitter slots (family h2o)
    recent: int = 0            # H2O recent window (family h2o)
    local_window: int = 0      # FastGen LOCAL window W (also the FREQ+LOCAL recent part)
    freq_heavy: int = 0        # FastGen FREQ+LOCAL heavy part
    hash_budget: int = 0       # HashEvict budget B
    history_window: int = 0    # persistence heads: steps of pivotal history counted (1..64)
    profile_rows: int = 0      # profiled heads: prompt rows the profile reads
    profile_threshold: float = 0.0   # profiled heads: attention share a composite must recover
    sketch_bits: int = 32
    cache_bits: int = 0        # cached K/V: 0 = the storage dtype, 4 = 4-bit slots
    vocab: int = 32000
    special_ids: Tuple[int, ...] = (0, 1, 2, 3)
    punct_ids: Tuple[int, ...] = tuple(range(4, 14))
    heavy_frac_positions: float = 0.05   # share of the N positions that carry a heavy direction
    description: str = ""

    @property
    def context(self) -> int:
        return self.prompt + self.steps

    @property
    def units_per_layer(self) -> int:
        return self.batch * self.heads

    @property
    def units(self) -> int:
        return self.layers * self.units_per_layer

    def policy_table(self, layer: int = 0) -> Tuple[List[int], List[int], List[int]]:
        """(policy, heavy, recent) per head of one layer.

        H2O family: heavy = hh, recent = r.  LOCAL: heavy = 0, recent = W.
        HASH: heavy = B (the budget ranked by sketch distance), recent = 0.
        FULL and SPECIAL: 0, 0 (their capacity is the context length).
        FastGen heads get a balanced assignment of the four policies, shuffled
        with a seed per layer.
        """
        H = self.heads
        if self.family == "h2o":
            return [H2O] * H, [self.heavy] * H, [self.recent] * H
        if self.family == "persist":
            return [PERSIST] * H, [self.heavy] * H, [self.recent] * H
        if self.family == "adaptive":
            return [ADAPTIVE] * H, [self.freq_heavy] * H, [self.local_window] * H
        if self.family == "hash":
            return [HASH] * H, [self.hash_budget] * H, [0] * H
        if self.family == "fastgen":
            import numpy as np
            kinds = [FULL, LOCAL, SPECIAL, H2O]
            base = [kinds[i % 4] for i in range(H)]
            rng = np.random.default_rng([self.index, 7, layer])
            order = rng.permutation(H)
            pol = [base[i] for i in order]
            heavy, recent = [], []
            for p in pol:
                if p == H2O:
                    heavy.append(self.freq_heavy); recent.append(self.local_window)
                elif p == LOCAL:
                    heavy.append(0); recent.append(self.local_window)
                else:
                    heavy.append(0); recent.append(0)
            return pol, heavy, recent
        raise ValueError(self.family)

    def window_table(self, layer: int = 0) -> List[int]:
        """History window per head of one layer (persistence heads; 0 elsewhere)."""
        pol = self.policy_table(layer)[0]
        return [self.history_window if p == PERSIST else 0 for p in pol]

    def keep_ids(self) -> List[int]:
        return sorted(set(self.special_ids) | set(self.punct_ids))


def _h2o20(P: int) -> Dict[str, int]:
    return {"heavy": int(0.1 * P), "recent": int(0.1 * P)}


def _fastgen(P: int) -> Dict[str, int]:
    return {"local_window": int(0.25 * P), "freq_heavy": int(0.1 * P)}


def _hash(P: int) -> Dict[str, int]:
    return {"hash_budget": int(0.5 * P)}


WORKLOADS: Dict[str, Workload] = {}


def _add(w: Workload) -> None:
    WORKLOADS[w.name] = w


_add(Workload(
    name="tiny_h2o", index=1, layers=1, batch=1, heads=2, head_dim=64, dtype="f32",
    prompt=64, steps=64, family="h2o", structure="dirs4", heavy=16, recent=16,
    heavy_frac_positions=0.10,
    description="1 layer, batch 1, 2 heads, d=64, fp32, P=64, T=64, budget 16 heavy + 16 recent"))
_add(Workload(
    name="opt6.7b_layer_h2o", index=2, layers=1, batch=64, heads=32, head_dim=128, dtype="f16",
    prompt=512, steps=512, family="h2o", structure="zipf_dir", **_h2o20(512),
    description="OPT-6.7B-shaped attention layer: batch 64, 32 heads, d=128, fp16, P=T=512, H2O 20%"))
_add(Workload(
    name="opt30b_decode_h2o", index=3, layers=48, batch=32, heads=56, head_dim=128, dtype="bf16",
    prompt=2048, steps=256, family="h2o", structure="zipf_dir", **_h2o20(2048),
    description="OPT-30B-shaped decode: 48 layers, batch 32, 56 heads, d=128, bf16, P=2048, T=256, H2O 20%"))
_add(Workload(
    name="llama65b_fastgen", index=4, layers=1, batch=8, heads=64, head_dim=128, dtype="bf16",
    prompt=4096, steps=512, family="fastgen", structure="zipf_dir", **_fastgen(4096),
    description="Llama-65B-shaped FastGen per-head policies: batch 8, 64 heads, d=128, bf16, P=4096, T=512"))
_add(Workload(
    name="hashevict_lsh", index=5, layers=1, batch=16, heads=32, head_dim=128, dtype="bf16",
    prompt=8192, steps=1024, family="hash", structure="clusters", **_hash(8192),
    description="HashEvict: batch 16, 32 heads, d=128, bf16, P=8192, T=1024, budget 50%, 32-bit sketches"))

_add(Workload(
    name="opt30b_decode_persist", index=6, layers=48, batch=32, heads=56, head_dim=128, dtype="bf16",
    prompt=2048, steps=256, family="persist", structure="zipf_dir", history_window=64, **_h2o20(2048),
    description="OPT-30B-shaped decode under the persistence-count rule: 48 layers, batch 32, 56 heads, "
                "d=128, bf16, P=2048, T=256, 20% budget (204 + 204), 64-step history"))

_add(Workload(
    name="llama65b_fastgen_profiled", index=7, layers=1, batch=8, heads=64, head_dim=128, dtype="bf16",
    prompt=4096, steps=512, family="adaptive", structure="head_kinds", profile_rows=64,
    profile_threshold=0.95, heavy_frac_positions=0.01, **_fastgen(4096),
    description="Llama-65B-shaped FastGen with profiling: batch 8, 64 heads of five attention kinds, d=128, "
                "bf16, P=4096, T=512; composites special / +punctuation / +409 frequent / +1024 local / full, "
                "chosen per (sequence, head) at 95% recovered attention over the last 64 prompt rows"))

_add(Workload(
    name="opt30b_decode_h2o_q4", index=8, layers=48, batch=32, heads=56, head_dim=128, dtype="bf16",
    prompt=2048, steps=256, family="h2o", structure="zipf_dir", cache_bits=4, **_h2o20(2048),
    description="OPT-30B-shaped H2O decode with 4-bit cache slots: 48 layers, batch 32, 56 heads, d=128, "
                "bf16 inputs, P=2048, T=256, 20% budget (204 + 204); K/V rows in groups of 32 with a "
                "float32 scale and 4-bit codes"))

_add(Workload(
    name="hashevict_lsh_q4", index=9, layers=1, batch=16, heads=32, head_dim=128, dtype="bf16",
    prompt=8192, steps=1024, family="hash", structure="clusters", cache_bits=4, **_hash(8192),
    description="HashEvict with 4-bit cache slots: batch 16, 32 heads, d=128, bf16 inputs, P=8192, T=1024, "
                "budget 50%, 32-bit sketches from the full-precision inputs"))

ORDER = ["tiny_h2o", "opt6.7b_layer_h2o", "opt30b_decode_h2o", "llama65b_fastgen", "hashevict_lsh"]
NEXT = ["opt30b_decode_persist", "llama65b_fastgen_profiled", "opt30b_decode_h2o_q4", "hashevict_lsh_q4"]


def get(name: str) -> Workload:
    return WORKLOADS[name]


def scaled(name: str, **over) -> Workload:
    """A smaller variant of a named workload for tests.

    Budgets that the full workload derives from P are re-derived from the new
    P with the same floor rule unless given explicitly.
    """
    w = WORKLOADS[name]
    P = over.get("prompt", w.prompt)
    derived: Dict[str, int] = {}
    if w.family in ("h2o", "persist") and w.name != "tiny_h2o":
        derived = _h2o20(P)
    elif w.family in ("fastgen", "adaptive"):
        derived = _fastgen(P)
    elif w.family == "hash":
        derived = _hash(P)
    for k, v in derived.items():
        over.setdefault(k, v)
    over.setdefault("name", w.name + "_scaled")
    return dataclasses.replace(w, **over)
