"""GPU parity over seeded random configurations.

Each case draws a workload family (H2O, persistence, FastGen per-head, profiled
FastGen, HashEvict, or a mixed layer of several policies), a dtype, a head
dimension, prompt and decode lengths, per-head budgets, 4-bit slots where the
library builds them, a sketch width and a decode path (fused, or split with
chunks of 16 to 256 slots), and runs a layer through the C ABI in lockstep
with the float64 oracle: kept sets exact up to the 1e-6 near-tie band, scores
within 1e-5, outputs within 2e-3 of the largest output element, plus the
invariants every unit must satisfy.  Configurations the library rejects at
creation (its documented limits) are counted and skipped; the test requires
most draws to run.  The draws are fixed by the seed, so a failure names a
reproducible case."""

import os

import numpy as np
import pytest
import torch
import dataclasses

from tests import harness
from workloads import configs
from workloads.configs import ADAPTIVE, FULL, H2O, HASH, LOCAL, PERSIST, SPECIAL
from workloads.generate import _zipf_ids, generate_layer

pytestmark = pytest.mark.gpu

BASE = {"h2o": "opt30b_decode_h2o", "h2o16": "opt6.7b_layer_h2o", "persist": "opt30b_decode_persist",
        "fastgen": "llama65b_fastgen", "adaptive": "llama65b_fastgen_profiled", "hash": "hashevict_lsh"}
FAMILIES = ["h2o", "h2o16", "persist", "fastgen", "adaptive", "hash", "mixed"]


def draw(rng, medium=False):
    """One random configuration: (family, workload, policy, heavy, recent, history, path, chunk).
    medium: prompts of 700 to 3,999 tokens, budgets up to 6,000 slots, few steps."""
    fam = str(rng.choice(FAMILIES))
    q4 = bool(rng.random() < 0.3) and fam in ("h2o", "h2o16", "persist", "hash", "mixed")
    if medium:
        P, T = int(rng.integers(700, 4000)), int(rng.integers(1, 20))
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    else:
        P, T = int(rng.integers(1, 700)), int(rng.integers(1, 70))
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 5))
    hmax, rmax, bmax = (1500, 700, 6000) if medium else (90, 70, 1300)
    w = configs.scaled(BASE["h2o" if fam == "mixed" else fam], batch=B, heads=H, prompt=P, steps=T)
    w = dataclasses.replace(w, head_dim=int(rng.choice([64, 128])), dtype=str(rng.choice(["f32", "f16", "bf16"])),
                            cache_bits=4 if q4 else 0)
    ctx = P + T

    def hr():
        h, r = int(rng.integers(0, hmax)), int(rng.integers(0, rmax))
        while h + r > ctx:
            h, r = h // 2, r // 2
        return h, r

    hist = None
    if fam in ("h2o", "h2o16", "persist"):
        pol = [PERSIST if fam == "persist" else H2O] * H
        hv, rc = (list(x) for x in zip(*[hr() for _ in range(H)]))
        if fam == "persist":
            hist = [int(rng.integers(1, 65)) for _ in range(H)]
    elif fam == "fastgen":
        pol = [int(rng.choice([FULL, LOCAL, SPECIAL, H2O])) for _ in range(H)]
        hv, rc = [], []
        for p in pol:
            h, r = hr()
            hv.append(h if p == H2O else 0)
            rc.append(r if p in (H2O, LOCAL) else 0)
    elif fam == "adaptive":
        h, r = hr()
        pol, hv, rc = [ADAPTIVE] * H, [max(h, 1)] * H, [max(r, 1)] * H
        w = dataclasses.replace(w, profile_threshold=float(rng.choice([0.0, 0.5, 0.9, 0.99, 2.0])),
                                profile_rows=int(rng.integers(1, 64)))
    elif fam == "hash":
        pol = [HASH] * H
        hv = [int(rng.integers(1, min(ctx, bmax) + 1)) for _ in range(H)]
        rc = [0] * H
        w = dataclasses.replace(w, sketch_bits=int(rng.choice([16, 32, 64])))
    else:
        pol = [int(rng.choice([H2O, PERSIST, LOCAL, FULL, SPECIAL, HASH])) for _ in range(H)]
        hv, rc = [], []
        for p in pol:
            h, r = hr()
            if p == HASH:
                hv.append(int(rng.integers(1, min(ctx, bmax) + 1))); rc.append(0)
            elif p in (H2O, PERSIST):
                hv.append(h); rc.append(r)
            elif p == LOCAL:
                hv.append(0); rc.append(max(r, 1))
            else:
                hv.append(0); rc.append(0)
        hist = [int(rng.integers(1, 65)) if p == PERSIST else 0 for p in pol]
    path = str(rng.choice(["fused", "split"]))
    chunk = int(rng.choice([16, 32, 64, 256]))
    return fam, w, pol, hv, rc, hist, path, chunk


def run_random(seed, cases, medium):
    """Runs `cases` draws in lockstep with the oracle; returns (checked, rejected)."""
    rng = np.random.default_rng(seed)
    ran = rejected = 0
    saved = {k: os.environ.get(k) for k in ("KVEVICT_SPLIT_ABOVE", "KVEVICT_SPLIT_CHUNK")}
    try:
        for i in range(cases):
            fam, w, pol, hv, rc, hist, path, chunk = draw(rng, medium)
            seed = int(rng.integers(0, 1 << 30))
            if path == "split":
                os.environ["KVEVICT_SPLIT_ABOVE"] = "0"
                os.environ["KVEVICT_SPLIT_CHUNK"] = str(chunk)
            else:
                os.environ.pop("KVEVICT_SPLIT_ABOVE", None)
                os.environ.pop("KVEVICT_SPLIT_CHUNK", None)
            inp = generate_layer(w, 0, "cpu", seed)
            g = torch.Generator().manual_seed(seed)
            if (SPECIAL in pol or ADAPTIVE in pol) and inp.ids is None:
                inp.ids = _zipf_ids(w, g, w.batch, w.prompt + w.steps, "cpu")
            if HASH in pol and inp.proj is None:
                inp.proj = torch.randn((w.head_dim, w.sketch_bits), generator=g).to(torch.bfloat16)
            desc = (f"case {i}: {fam} {path}/{chunk} B={w.batch} H={w.heads} d={w.head_dim} {w.dtype} "
                    f"q4={w.cache_bits == 4} P={w.prompt} T={w.steps} pol={pol} hv={hv} rc={rc} hist={hist} "
                    f"bits={w.sketch_bits} seed={seed}")
            try:
                kv = harness.make_cache(w, inp, pol, hv, rc, history=hist)
            except Exception:                      # outside the library's documented limits
                rejected += 1
                continue
            print(f"\n[random] {desc}", flush=True)
            r = harness.run_layer(kv, inp.to("cuda"))
            rep = harness.check_all(w, inp, r, None, policy=pol, heavy=hv, recent=rc, history=hist)
            bad = harness.check_invariants(w, r, inp.prompt_q.shape[2], pol, hv, rc, hist)
            kv.close()
            assert rep.ok, (desc, rep.failures[:10])
            assert not bad, (desc, bad[:10])
            ran += 1
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    print(f"\n[random] {ran} configurations checked, {rejected} rejected by the library", flush=True)
    return ran, rejected


def test_random_configurations():
    ran, _ = run_random(20261203, 160, medium=False)
    assert ran >= 120


def test_random_configurations_medium():
    """Longer prompts and larger budgets: HashEvict budgets past the register
    replay's 1,024-slot step, split layers of many chunks, FastGen FULL heads
    holding thousands of positions."""
    ran, _ = run_random(4031, 24, medium=True)
    assert ran >= 16
