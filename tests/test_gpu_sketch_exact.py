"""HashEvict sketches whose projections cancel below float64 resolution.

Keys and queries at chosen positions are (2^30, +/-2^-30, -2^30, 0, ...), and
the projection's first three rows are 1: every bit's exact sum is +/-2^-30,
while a float64 sum taken left to right gives 0.  Only the exact fallback of
the sign computation gets these bits right, and the test first checks on the
CPU that naive signs would change the replay's decisions.  The logits of such
keys are huge, so outputs are not compared; kept sets and evictions are.
"""

import dataclasses

import numpy as np
import pytest
import torch

from oracle import hashevict
from tests import harness
from workloads import configs
from workloads.generate import generate_layer, unit_sequence

pytestmark = pytest.mark.gpu

P, T, BUDGET = 160, 48, 64


def crafted_inputs(seed=0, bits=32):
    w = dataclasses.replace(configs.scaled("hashevict_lsh", batch=1, heads=2, prompt=P, steps=T), sketch_bits=bits)
    inp = generate_layer(w, 0, "cpu", seed)
    rng = np.random.default_rng(seed)
    proj = inp.proj.clone()
    proj[:3, :] = 1.0
    inp.proj = proj
    big, tiny = 2.0 ** 30, 2.0 ** -30

    def craft(n, sign):
        x = torch.zeros((n, 128))
        x[:, 0] = big
        x[:, 1] = sign * tiny
        x[:, 2] = -big
        return x.to(torch.bfloat16)

    for h in range(2):
        for which, tensor_p, tensor_d in (("k", inp.prompt_k, inp.dec_k), ("q", inp.prompt_q, inp.dec_q)):
            pos = rng.choice(P + T, 24, replace=False)
            signs = rng.choice([-1.0, 1.0], 24)
            rows = craft(24, torch.tensor(signs, dtype=torch.float32))
            for i, p in enumerate(pos):
                if p < P:
                    tensor_p[0, h, p] = rows[i]
                else:
                    tensor_d[p - P, 0, h] = rows[i]
    return w, inp


def naive_sketches(X, W):
    """Left-to-right float64 sums (what the exact fallback must not be)."""
    out = np.zeros(len(X), dtype=np.uint64)
    for b in range(W.shape[1]):
        s = np.zeros(len(X))
        for i in range(X.shape[1]):
            s = s + X[:, i] * W[i, b]
        out |= (s > 0).astype(np.uint64) << np.uint64(b)
    return out


@pytest.mark.parametrize("bits", [16, 32, 64])
def test_cancelling_projections_take_the_exact_sign(bits):
    w, inp = crafted_inputs(bits=bits)
    Wp = inp.proj.float().double().numpy()
    # the crafted rows really need the exact path, and it changes decisions
    Q, K, V = unit_sequence(inp, 0, 0)
    exact_k = hashevict.sketches(K, Wp)
    naive_k = naive_sketches(K, Wp)
    assert (exact_k != naive_k).sum() >= 10
    exact_q = hashevict.sketches(Q, Wp)
    naive_q = naive_sketches(Q, Wp)
    kept_exact = hashevict.replay_prompt(exact_q, exact_k, P, BUDGET)
    kept_naive = hashevict.replay_prompt(naive_q, naive_k, P, BUDGET)
    assert set(kept_exact.tolist()) != set(kept_naive.tolist())

    kv = harness.make_cache(w, inp, policy=[4, 4], heavy=[BUDGET, BUDGET], recent=[0, 0])
    r = harness.run_layer(kv, inp.to("cuda"))
    kv.close()
    for h in range(2):
        Q, K, V = unit_sequence(inp, 0, h)
        tr = hashevict.run_unit(Q, K, V, Wp, P, BUDGET, 1 / np.sqrt(128), steps=T)
        g0 = np.sort(r.prefill_pos[0, h, :int(r.prefill_cnt[0, h])])
        g1 = np.sort(r.final_pos[0, h, :int(r.final_cnt[0, h])])
        assert np.array_equal(g0, np.sort(tr.prefill_kept)), h
        assert np.array_equal(r.evicted[:, 0, h], tr.evicted), h
        assert np.array_equal(g1, tr.final_kept), h


def scaled_inputs(seed, bits):
    """Prompt and step rows of both heads scaled by 2^e, e drawn from
    {-133, -126, -120, -100, 100, 110, 124}: bf16 subnormals, sums of
    magnitudes that overflow float32 (e = 124: 128 products near 2^124), and
    everything between.  The sign of a projection does not depend on the scale, so the
    exact sketches -- and the replay's decisions -- stay well defined."""
    w = dataclasses.replace(configs.scaled("hashevict_lsh", batch=1, heads=2, prompt=P, steps=T), sketch_bits=bits)
    inp = generate_layer(w, 0, "cpu", seed)
    rng = np.random.default_rng(seed + 100)
    exps = np.array([-133, -126, -120, -100, 100, 110, 124])
    for h in range(2):
        for tensor_p, tensor_d in ((inp.prompt_k, inp.dec_k), (inp.prompt_q, inp.dec_q)):
            for p in rng.choice(P + T, 60, replace=False):
                f = float(2.0 ** int(rng.choice(exps)))
                if p < P:
                    tensor_p[0, h, p] = (tensor_p[0, h, p].float() * f).to(torch.bfloat16)
                else:
                    tensor_d[p - P, 0, h] = (tensor_d[p - P, 0, h].float() * f).to(torch.bfloat16)
    return w, inp


@pytest.mark.parametrize("bits", [16, 32, 64])
def test_extreme_row_scales_take_the_exact_sign(bits):
    """bf16 rows are sketched on the matrix cores, in float32; rows whose
    sums overflow or underflow float32 must fall back to the exact sign."""
    w, inp = scaled_inputs(seed=7, bits=bits)
    Wp = inp.proj.float().double().numpy()
    assert inp.prompt_k.dtype == torch.bfloat16
    kv = harness.make_cache(w, inp, policy=[4, 4], heavy=[BUDGET, BUDGET], recent=[0, 0])
    r = harness.run_layer(kv, inp.to("cuda"))
    kv.close()
    for h in range(2):
        Q, K, V = unit_sequence(inp, 0, h)
        assert np.isfinite(K).all() and np.isfinite(Q).all()
        tr = hashevict.run_unit(Q, K, V, Wp, P, BUDGET, 1 / np.sqrt(128), steps=T)
        g0 = np.sort(r.prefill_pos[0, h, :int(r.prefill_cnt[0, h])])
        g1 = np.sort(r.final_pos[0, h, :int(r.final_cnt[0, h])])
        assert np.array_equal(g0, np.sort(tr.prefill_kept)), h
        assert np.array_equal(r.evicted[:, 0, h], tr.evicted), h
        assert np.array_equal(g1, tr.final_kept), h
