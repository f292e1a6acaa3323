"""One handle holding several layers with different per-layer policy tables,
driven in model order (every layer's decode step, then the next step), and
the call-order errors a GPU handle reports."""

import numpy as np
import pytest
import torch

from budgeted_decode_attention_amd import KVCache, KVEvictError, binding
from oracle import lockstep
from tests import harness
from workloads import configs
from workloads.configs import FULL, H2O, LOCAL, SPECIAL
from workloads.generate import generate_layer, unit_ids, unit_sequence

pytestmark = pytest.mark.gpu


def test_three_layers_interleaved():
    w = configs.scaled("llama65b_fastgen", batch=2, heads=4, prompt=300, steps=40)
    L = 3
    # layer 0: all H2O; layer 1: FastGen mix; layer 2: local + full
    tables = [
        ([H2O] * 4, [30, 30, 20, 10], [30, 20, 30, 40]),
        ([FULL, LOCAL, SPECIAL, H2O], [0, 0, 0, 30], [0, 75, 0, 75]),
        ([LOCAL, LOCAL, FULL, FULL], [0, 0, 0, 0], [10, 60, 0, 0]),
    ]
    pol = np.concatenate([t[0] for t in tables]).astype(np.int32)
    hv = np.concatenate([t[1] for t in tables]).astype(np.int32)
    rc = np.concatenate([t[2] for t in tables]).astype(np.int32)
    ins = [generate_layer(w, l, "cpu", 5) for l in range(L)]
    gins = [x.to("cuda") for x in ins]
    kv = KVCache(L, w.batch, w.heads, w.head_dim, w.context, torch.bfloat16, pol, hv, rc,
                 keep_ids=w.keep_ids(), vocab=w.vocab)
    P, T, d = w.prompt, w.steps, w.head_dim
    for l in range(L):
        x = gins[l]
        kv.prefill(l, x.prompt_q, x.prompt_k, x.prompt_v, x.ids[:, :P].contiguous())
    pre = [kv.kept_indices(l) for l in range(L)]
    pre = [tuple(t.cpu().numpy() for t in p) for p in pre]
    out = torch.empty((L, T, w.batch, w.heads, d), dtype=torch.float32, device="cuda")
    ev = torch.empty((L, T, w.batch, w.heads), dtype=torch.int32, device="cuda")
    for s in range(T):
        for l in range(L):
            x = gins[l]
            kv.decode_step(l, x.dec_q[s], x.dec_k[s], x.dec_v[s], x.ids[:, P + s].contiguous(), out[l, s], ev[l, s])
    fin = [tuple(t.cpu().numpy() for t in kv.kept_indices(l)) for l in range(L)]
    torch.cuda.synchronize()
    assert all(kv.position(l) == P + T for l in range(L))
    scale = 1 / np.sqrt(d)
    for l in range(L):
        for b in range(w.batch):
            for h in range(w.heads):
                n0, n1 = int(pre[l][1][b, h]), int(fin[l][1][b, h])
                g = lockstep.GpuUnit(prefill_pos=pre[l][0][b, h, :n0], evicted=ev[l, :, b, h].cpu().numpy(),
                                     out=out[l, :, b, h].cpu().numpy(), final_pos=fin[l][0][b, h, :n1],
                                     prefill_S=pre[l][2][b, h, :n0], final_S=fin[l][2][b, h, :n1])
                Q, K, V = unit_sequence(ins[l], b, h)
                p_, a_, r_ = tables[l][0][h], tables[l][1][h], tables[l][2][h]
                rep = lockstep.check_fastgen(p_, Q, K, V, P, scale, g, heavy=a_, recent=r_,
                                             ids=unit_ids(ins[l], b), keep_ids=w.keep_ids())
                assert rep.ok, (l, b, h, rep.failures[:5])
    kv.close()


def test_call_order_errors():
    w = configs.scaled("opt6.7b_layer_h2o", batch=1, heads=2, prompt=20, steps=3)
    x = generate_layer(w, 0, "cuda", 0)
    kv = harness.make_cache(w, x, max_context=22)
    with pytest.raises(KVEvictError) as e:
        kv.decode_step(0, x.dec_q[0], x.dec_k[0], x.dec_v[0])
    assert e.value.status == binding.KVE_ESTATE
    with pytest.raises(KVEvictError) as e:
        kv.kept_indices(0)
    assert e.value.status == binding.KVE_ESTATE
    kv.prefill(0, x.prompt_q, x.prompt_k, x.prompt_v)
    kv.decode_step(0, x.dec_q[0], x.dec_k[0], x.dec_v[0])
    kv.decode_step(0, x.dec_q[1], x.dec_k[1], x.dec_v[1])
    with pytest.raises(KVEvictError) as e:          # position 22 == max_context
        kv.decode_step(0, x.dec_q[2], x.dec_k[2], x.dec_v[2])
    assert e.value.status == binding.KVE_ESTATE
    with pytest.raises(KVEvictError) as e:
        kv.prefill(1, x.prompt_q, x.prompt_k, x.prompt_v)
    assert e.value.status == binding.KVE_EINVAL
    with pytest.raises(ValueError):                 # wrong dtype caught by the binding's checks
        kv.decode_step(0, x.dec_q[0].float(), x.dec_k[0], x.dec_v[0])
    assert kv.position(0) == 22
    # a fresh prefill resets the layer
    kv.prefill(0, x.prompt_q, x.prompt_k, x.prompt_v)
    assert kv.position(0) == 20
    torch.cuda.synchronize()
    kv.close()
