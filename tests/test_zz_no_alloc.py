"""The allocation-free decode entry point matches the regular one (GPU).

Two handles with the same configuration are prefilled with the same inputs;
one steps with kvevict_decode_step, the other with
kvevict_decode_step_noalloc.  Layers with more than 1,024 slots per unit use
the split decode, whose partials and logits the no-alloc call keeps in the
library's static per-GPU array.  Both must give bit-identical outputs,
eviction logs, kept sets and scores, on two calls in a row, the second with a
smaller layer (so the array still holds the first call's contents).
"""

import numpy as np
import pytest
import torch

from budgeted_decode_attention_amd import KVCache, KVEvictError
from budgeted_decode_attention_amd import binding
from workloads import configs
from workloads.generate import generate_layer

pytestmark = pytest.mark.gpu

H2O, FULL, LOCAL = 1, 0, 2


def _pair(w, policy, heavy, recent, dtype):
    mk = lambda: KVCache(1, w.batch, w.heads, w.head_dim, w.context, dtype,
                         np.array(policy, np.int32), np.array(heavy, np.int32), np.array(recent, np.int32),
                         device="cuda")
    return mk(), mk()


def _run(w, policy, heavy, recent, seed):
    print(f"[no_alloc] batch={w.batch} heads={w.heads} P={w.prompt} T={w.steps} policy={policy} "
          f"heavy={heavy} recent={recent}", flush=True)
    inp = generate_layer(w, 0, "cuda", seed)
    a, b = _pair(w, policy, heavy, recent, inp.prompt_q.dtype)
    assert a.capacity(0) > 1024, "the layer must take the split decode"
    outs = []
    for kv, noalloc in ((a, False), (b, True)):
        kv.prefill(0, inp.prompt_q, inp.prompt_k, inp.prompt_v)
        out = torch.empty((w.steps, w.batch, w.heads, w.head_dim), dtype=torch.float32, device="cuda")
        ev = torch.empty((w.steps, w.batch, w.heads), dtype=torch.int32, device="cuda")
        for s in range(w.steps):
            kv.decode_step(0, inp.dec_q[s], inp.dec_k[s], inp.dec_v[s], None, out[s], ev[s], noalloc=noalloc)
        pos, cnt, sc = kv.kept_indices(0)
        torch.cuda.synchronize()
        outs.append((out.cpu(), ev.cpu(), pos.cpu(), cnt.cpu(), sc.cpu()))
    for x, y, name in zip(outs[0], outs[1], ("out", "evicted", "pos", "count", "scores")):
        assert torch.equal(x, y), name
    assert (outs[0][1] >= 0).any(), "the steps should evict"
    a.close()
    b.close()


def test_noalloc_matches_decode_step_twice_second_smaller():
    # call 1: 3 x 4 units, H2O heads of up to 1,100 + 200 slots and a full-cache
    # head (slot stride 1,398: 256-slot chunks)
    w1 = configs.scaled("opt30b_decode_h2o", batch=3, heads=4, prompt=1390, steps=8)
    _run(w1, [H2O, H2O, FULL, H2O], [1100, 900, 0, 1000], [200, 150, 0, 250], seed=3)
    # call 2, smaller: 2 x 2 units, an H2O head of 700 + 350 slots and a local
    # window of 1,060 (stride 1,060), evicting at the prompt and every step
    w2 = configs.scaled("opt30b_decode_h2o", batch=2, heads=2, prompt=1080, steps=5)
    _run(w2, [H2O, LOCAL], [700, 0], [350, 1060], seed=4)


def test_noalloc_rejects_a_layer_beyond_the_static_scratch():
    # 128 x 32 full-cache units with a stride of 2,100 slots (two 1,280-slot
    # chunks): 4,096 x (2 x 130 + 2,100) x 4 B = 38.7 MB > 32 MiB
    w = configs.scaled("opt30b_decode_h2o", batch=128, heads=32, prompt=40, steps=1)
    kv = KVCache(1, w.batch, w.heads, w.head_dim, 2100, torch.bfloat16, np.array([FULL] * 32, np.int32),
                 np.zeros(32, np.int32), np.zeros(32, np.int32), device="cuda")
    inp = generate_layer(w, 0, "cuda", 5)
    kv.prefill(0, inp.prompt_q, inp.prompt_k, inp.prompt_v)
    out = torch.empty((w.batch, w.heads, w.head_dim), dtype=torch.float32, device="cuda")
    with pytest.raises(KVEvictError) as e:
        kv.decode_step(0, inp.dec_q[0], inp.dec_k[0], inp.dec_v[0], None, out, noalloc=True)
    assert e.value.status == binding.KVE_EUNSUPPORTED and "static scratch" in str(e.value)
    assert kv.position(0) == 40                # nothing was enqueued, the position did not move
    kv.decode_step(0, inp.dec_q[0], inp.dec_k[0], inp.dec_v[0], None, out)   # the regular call still works
    torch.cuda.synchronize()
    assert kv.position(0) == 41 and torch.isfinite(out).all()
    kv.close()
