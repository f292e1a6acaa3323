"""Benchmark: decode tokens/s with H2O eviction at a 20% KV budget, and the
fused decode kernel's achieved HBM bandwidth against MI355X peak.

One step is the whole hot path over one batch: prefill (scoring, selection,
gather) of every layer, then every decode step of every layer, in model
order (layer-major within a step).  Inputs are synthetic, seeded, generated
on the GPU and resident in HBM before timing starts.

Prints one JSON line.  `value` = batch * T / step time (prefill included).
The roofline object covers the fused decode kernel: algorithmic bytes per
launch (kept K/V read, score/position metadata, the step's q/k/v, the victim
write and the fp32 output) divided by its average launch time, measured with
HIP events around sampled decode steps (each a back-to-back group of one
launch per layer, no other kernel in between) on the stream the kernel runs on.
The CPU baseline times the float64 oracle on a bounded sample of units of the
same workload, before the GPU is initialised, and scales it to the job.
"""

from __future__ import annotations

import argparse
import json
import multiprocessing as mp
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode tokens/sec with H2O eviction at 20% budget; achieved HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "opt30b_decode_h2o"


# ---------------------------------------------------------------- CPU baseline (oracle)

def _hash_recovered_share(tr, Q, K, P: int, scale: float) -> float:
    """Mean over decode steps of the share of the full causal softmax (keys
    0..t) that lands on the HashEvict cache attended at step t -- the quality
    side of the sketch-width trade-off.  Rebuilt from the oracle's eviction
    log; not part of the timed oracle run."""
    import numpy as np
    cache = list(int(j) for j in tr.prefill_kept)
    shares = []
    for s_, t in enumerate(range(P, P + len(tr.evicted))):
        e = int(tr.evicted[s_])
        if e >= 0:
            cache[cache.index(e)] = t
        else:
            cache.append(t)
        lg = (K[: t + 1] @ Q[t]) * scale
        p = np.exp(lg - lg.max())
        p /= p.sum()
        shares.append(float(p[np.array(cache)].sum()))
    return float(np.mean(shares))


def _q4_output_error(tr_q4, Q, K, V, P: int, a: int, b: int, scale: float) -> float:
    """Mean over decode steps of ||o_4bit - o|| / ||o||: the same unit with
    cache rows in the storage dtype gives o.  Not part of the timed oracle run."""
    import numpy as np
    from oracle import h2o
    ref = h2o.run_unit(Q, K, V, P, a, b, scale).out
    return float(np.mean(np.linalg.norm(tr_q4.out - ref, axis=1) / np.linalg.norm(ref, axis=1)))


def _oracle_run(kind, Q, K, V, P, a, b, scale, extra, steps=None):
    """One call of the oracle's own per-unit entry point for `kind`; with
    steps=0 it runs the prefill only (scoring and selection of the prompt)."""
    import numpy as np
    from oracle import adaptive, fastgen, h2o, hashevict, persistence, quant
    if kind == "h2o_q4":
        return h2o.run_unit(Q, K, V, P, a, b, scale, steps=steps, Kc=quant.roundtrip(K), Vc=quant.roundtrip(V))
    if kind == "h2o":
        return h2o.run_unit(Q, K, V, P, a, b, scale, steps=steps)
    if kind == "persist":
        return persistence.run_unit(Q, K, V, P, a, b, extra, scale, steps=steps)
    if kind == "adaptive":
        ids, special, punct, rows, thr = extra
        return adaptive.run_unit(Q, K, V, ids, P, special, punct, a, b, scale, rows, thr, steps=steps)
    if kind in ("hash", "hash_q4"):
        cc = dict(Kc=quant.roundtrip(K), Vc=quant.roundtrip(V)) if kind == "hash_q4" else {}
        return hashevict.run_unit(Q, K, V, np.asarray(extra, dtype=np.float64), P, a, scale, steps=steps, **cc)
    pol, ids, keep = extra
    return fastgen.run_unit(pol, Q, K, V, P, scale, heavy=a, recent=b, ids=ids, keep_ids=keep, steps=steps)


def _oracle_unit(args):
    """One unit through the float64 oracle: the prefill alone (timed), then
    prefill + every decode step (timed).  Returns (prefill s, whole-unit s,
    extra) -- extra: the HashEvict cache's recovered share, or for 4-bit slots
    (on the units asked for) the output error against the storage-dtype cache."""
    import numpy as np
    from oracle import adaptive, fastgen, h2o, hashevict, persistence, quant  # noqa: F401  (imported before timing)
    kind, Q, K, V, P, a, b, scale, extra, want_extra = args
    Q, K, V = (np.asarray(x, dtype=np.float64) for x in (Q, K, V))
    t0 = time.perf_counter()
    _oracle_run(kind, Q, K, V, P, a, b, scale, extra, steps=0)
    t1 = time.perf_counter()
    tr = _oracle_run(kind, Q, K, V, P, a, b, scale, extra)
    t2 = time.perf_counter()
    out = None
    if want_extra and kind == "h2o_q4":
        out = _q4_output_error(tr, Q, K, V, P, a, b, scale)
    elif want_extra and kind in ("hash", "hash_q4"):
        out = _hash_recovered_share(tr, Q, K, P, scale)
    return t1 - t0, t2 - t1, out


def _oracle_warmup(task):
    """Pool initializer: the sample's first unit through the oracle's prefill
    and one decode step, untimed, so each worker's one-time library start-up
    (allocator, BLAS) stays out of the timed calls."""
    import numpy as np
    from oracle import adaptive, fastgen, h2o, hashevict, persistence, quant  # noqa: F401
    kind, Q, K, V, P, a, b, scale, extra, _ = task
    Q, K, V = (np.asarray(x, dtype=np.float64) for x in (Q, K, V))
    _oracle_run(kind, Q, K, V, P, a, b, scale, extra, steps=1)


def sample_units(w, n_units: int):
    """Seeded sample of units (layer, sequence, head): half from the first and
    half from the last layer (one layer if the workload has one), drawn
    without replacement over every (sequence, head) of that layer."""
    import numpy as np
    rng = np.random.default_rng([1000 + w.index, 47])
    layers = [0, w.layers - 1] if w.layers > 1 else [0]
    units = []
    for i, layer in enumerate(layers):
        m = min(n_units // len(layers) + (1 if i < n_units % len(layers) else 0), w.batch * w.heads)
        for f in sorted(rng.choice(w.batch * w.heads, m, replace=False).tolist()):
            units.append((layer, f // w.heads, f % w.heads))
    return units


def cpu_baseline(w, n_units: int, workers: int, one_core_units: int = 16):
    """Times the oracle on a seeded sample of `n_units` units of workload `w`
    (inputs generated on the CPU with the same recipe, the first and the last
    layer, every sequence eligible) with `workers` processes, and the first
    `one_core_units` of the sample again in one process.  Prefill and decode
    are timed separately.  Returns the dict for the JSON line.  Must run
    before anything initialises the GPU."""
    import numpy as np
    from workloads.generate import generate_layer, unit_ids, unit_sequence
    pol, hv, rc = w.policy_table(0)
    scale = 1.0 / np.sqrt(w.head_dim)
    units = sample_units(w, n_units)
    tasks = []
    t_gen = time.perf_counter()
    for layer in sorted(set(u[0] for u in units)):
        inp = generate_layer(w, layer, "cpu", 1)
        for (_, b, h) in [u for u in units if u[0] == layer]:
            Q, K, V = (x.astype(np.float32) for x in unit_sequence(inp, b, h))
            want = len(tasks) < 16
            if w.family == "h2o" and w.cache_bits == 4:
                tasks.append(("h2o_q4", Q, K, V, w.prompt, hv[h], rc[h], scale, None, want))
            elif w.family == "h2o":
                tasks.append(("h2o", Q, K, V, w.prompt, hv[h], rc[h], scale, None, False))
            elif w.family == "persist":
                tasks.append(("persist", Q, K, V, w.prompt, hv[h], rc[h], scale, w.window_table(0)[h], False))
            elif w.family == "adaptive":
                tasks.append(("adaptive", Q, K, V, w.prompt, hv[h], rc[h], scale,
                              (unit_ids(inp, b), list(w.special_ids), list(w.punct_ids), w.profile_rows,
                               w.profile_threshold), False))
            elif w.family == "hash":
                tasks.append(("hash_q4" if w.cache_bits == 4 else "hash", Q, K, V, w.prompt, hv[h], 0, scale,
                              inp.proj.float().numpy(), True))
            else:
                tasks.append(("fastgen", Q, K, V, w.prompt, hv[h], rc[h], scale,
                              (pol[h], unit_ids(inp, b), w.keep_ids()), False))
        del inp
    gen_s = time.perf_counter() - t_gen
    os.environ["OMP_NUM_THREADS"] = "1"
    os.environ["OPENBLAS_NUM_THREADS"] = "1"
    os.environ["MKL_NUM_THREADS"] = "1"
    ctx = mp.get_context("spawn")
    t0 = time.perf_counter()
    with ctx.Pool(workers, initializer=_oracle_warmup, initargs=(tasks[0],)) as pool:
        res = pool.map(_oracle_unit, tasks, chunksize=1)
    wall = time.perf_counter() - t0
    one = min(one_core_units, len(tasks))
    t1 = time.perf_counter()
    with ctx.Pool(1, initializer=_oracle_warmup, initargs=(tasks[0],)) as pool:
        res1 = pool.map(_oracle_unit, [t[:-1] + (False,) for t in tasks[:one]], chunksize=1)
    wall1 = time.perf_counter() - t1
    pre = sum(r[0] for r in res)
    tot = sum(r[1] for r in res)
    extra = [r[2] for r in res if r[2] is not None]
    # the parallel wall covers both timed calls of every unit; split it by the
    # per-unit shares and scale it to the job's units
    job_s = wall * (tot / (tot + pre)) * w.units / len(tasks)
    job_pre_s = job_s * pre / tot
    tokens = w.batch * w.steps
    layers = sorted(set(u[0] for u in units))
    return {
        "value": tokens / job_s, "unit": "tokens/s", "cores": workers, "kind": "oracle",
        "sample": f"{len(tasks)} of {w.units} units (full P={w.prompt}, T={w.steps}) drawn with a fixed seed "
                  f"from layer{'s' if len(layers) > 1 else ''} {' and '.join(map(str, layers))} over all "
                  f"{w.batch} sequences x {w.heads} heads; float64 numpy, {workers} processes x 1 BLAS thread, "
                  f"wall {wall:.2f} s; job time scaled by units (extrapolated: {job_s:.0f} s for the whole job)",
        "prefill_s_job": job_pre_s, "decode_s_job": job_s - job_pre_s,
        "decode_only_tokens_per_s": tokens / (job_s - job_pre_s),
        "per_unit_s": {"prefill": pre / len(tasks), "decode": (tot - pre) / len(tasks)},
        "one_core": {"units": one, "wall_s": wall1, "prefill_s": sum(r[0] for r in res1),
                     "decode_s": sum(r[1] - r[0] for r in res1),
                     "tokens_per_s_extrapolated": tokens / (wall1 * (sum(r[1] for r in res1) /
                                                             sum(r[0] + r[1] for r in res1)) * w.units / one)},
        "input_generation_s": gen_s,
        "hash_recovered_share": float(np.mean(extra)) if extra and w.family == "hash" else None,
        "q4_output_rel_err": float(np.mean(extra)) if extra and w.cache_bits == 4 and w.family != "hash" else None,
        "q4_units": len(extra) if w.cache_bits == 4 and w.family != "hash" else 0,
    }


# ---------------------------------------------------------------- GPU

def adaptive_bytes_per_layer_step(w, ids, choice) -> float:
    """As decode_bytes_per_layer_step for profiled units, from each unit's
    chosen composite: special (1) or special + punctuation (2) ids kept so far;
    frequent (3) / + local (4): the protected ids so far plus the unprotected
    part up to its budget (score and position metadata per slot); full (5): t."""
    import numpy as np
    s = {"f32": 4, "f16": 2, "bf16": 2}[w.dtype]
    d = w.head_dim
    io = 3 * d * s + 2 * d * s + 4 * d
    P, T = w.prompt, w.steps
    ids = np.asarray(ids)
    sp = np.isin(ids, np.array(w.special_ids))
    spp = np.isin(ids, np.array(list(w.special_ids) + list(w.punct_ids)))
    before = lambda m: np.cumsum(m, axis=1) - m                       # counts strictly before t
    sp_b, spp_b, free_b = before(sp), before(spp), before(~spp)
    total = 0.0
    for b in range(w.batch):
        for h in range(w.heads):
            k = int(choice[b, h])
            for st in range(T):
                t = P + st
                if k == 1:
                    n, meta = int(sp_b[b, t]), 0
                elif k == 2:
                    n, meta = int(spp_b[b, t]), 0
                elif k in (3, 4):
                    budget = w.freq_heavy + (w.local_window if k == 4 else 0)
                    n, meta = int(spp_b[b, t]) + min(budget, int(free_b[b, t])), 12
                else:
                    n, meta = t, 0
                total += n * d * s * 2 + n * meta + io
    return total / T


def decode_bytes_per_layer_step(w, ids=None) -> float:
    """Algorithmic bytes of one layer's decode step, averaged over the T steps:
    per unit, the kept K and V rows read (n slots x d x s x 2; 4-bit slots:
    d / 2 code bytes and d / 32 float32 scales per row), the per-slot
    metadata the policy needs (H2O: score read and write at the 4-byte float32
    minimum plus the position, 12 B; persistence counts: the 64-bit history
    read and written plus the position, 20 B; HashEvict: sketch and position, 8 B), the
    step's q, k, v, the new token's K/V write and the fp32 output.  n is the
    unit's kept count at that step: B for H2O and HashEvict, W for the local
    window, t for the full cache, and for the special policy the number of
    earlier positions whose id is kept (counted from the ids)."""
    s = {"f32": 4, "f16": 2, "bf16": 2}[w.dtype]
    d = w.head_dim
    row = d // 2 + 4 * (d // 32) if w.cache_bits == 4 else d * s    # bytes of one cached row
    io = 3 * d * s + 2 * row + 4 * d
    pol, hv, rc = w.policy_table(0)
    if w.family == "h2o":
        B = w.heavy + w.recent
        return w.units_per_layer * (B * row * 2 + B * 12 + io)
    if w.family == "persist":
        B = w.heavy + w.recent
        return w.units_per_layer * (B * row * 2 + B * 20 + io)
    if w.family == "hash":
        B = w.hash_budget
        word = 8 if w.sketch_bits == 64 else 4                        # sketch word per slot
        return w.units_per_layer * (B * row * 2 + B * (word + 4) + io + word)
    import numpy as np
    P, T = w.prompt, w.steps
    keep = np.isin(np.asarray(ids), np.array(w.keep_ids()))           # [batch, N]
    kept_before = np.cumsum(keep, axis=1) - keep                       # kept ids strictly before t
    total = 0.0
    for h in range(w.heads):
        for b in range(w.batch):
            for st in range(T):
                t = P + st
                if pol[h] == 1:
                    n, meta = hv[h] + rc[h], 12
                elif pol[h] == 2:
                    n, meta = min(t, rc[h]), 0
                elif pol[h] == 0:
                    n, meta = t, 0
                else:
                    n, meta = int(kept_before[b, t]), 0
                total += n * d * s * 2 + n * meta + io
    return total / T


def _counter_records(workload: str):
    """The committed counter records (profiles/counters_*.txt) whose
    `workload:` matches and whose kernel sources still hash to the value
    recorded with them, as dicts of their machine-readable lines."""
    import glob
    import hashlib
    out = []
    for p in sorted(glob.glob(os.path.join(ROOT, "profiles", "counters_*.txt"))):
        rec = {}
        for line in open(p):
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
        if rec.get("workload") != workload:
            continue
        h = hashlib.sha256()
        for f in rec.get("kernel_sources", "").split():
            with open(os.path.join(ROOT, f), "rb") as fh:
                h.update(fh.read())
        if h.hexdigest()[:16] == rec.get("kernel_sources_sha256"):
            out.append(rec)
    return out


def prefill_counters(workload: str):
    """Matrix-core busy share (rocprofv3's MfmaUtil) and vector-ALU busy share
    of the prefill scoring kernels from a committed counter record, or None."""
    for rec in _counter_records(workload):
        if "rowstats_mfma_util" in rec:
            return {k: float(rec[k]) for k in ("rowstats_mfma_util", "colsum_mfma_util",
                                                "rowstats_valu_busy", "colsum_valu_busy")}
    return None


def counter_traffic(workload: str):
    """HBM bytes per launch of the decode kernel from a committed counter record
    (profiles/counters_*.txt whose `workload:` matches: FETCH_SIZE and
    WRITE_SIZE passes scaled by a plain copy of known size), or None if there
    is none or the kernel sources have changed since it was taken."""
    for rec in _counter_records(workload):
        if "traffic_bytes_per_launch" in rec:
            return float(rec["traffic_bytes_per_launch"])
    return None


def prefill_flops_per_layer(w, prompt_out: bool):
    """Matrix flops of one layer's prefill, as (algorithmic, issued).

    Algorithmic (what the method needs): one causal Q K^T (2 d flops per
    query-key pair with key <= query) per unit whose policy scores the prompt
    (H2O and profiled heads: every row; persistence heads: their last `window`
    rows), and with the prompt output one causal Q K^T plus one P V for every
    unit (the scores then come from that same softmax).  Issued (what the
    kernels run): the column sums recompute Q K^T in a second pass, and the
    prompt output's P V runs twice (each weight enters as a 16-bit (hi, lo)
    pair); the difference is implementation overhead."""
    pairs = w.prompt * (w.prompt + 1) / 2
    pol = w.policy_table(0)[0]
    per = 2.0 * w.head_dim * pairs
    scored = w.batch * sum(1 for p in pol if p in (1, 6))
    units = w.batch * w.heads
    tail = 0.0
    for p, win in zip(pol, w.window_table(0)):
        if p == 5:
            rows = min(win, w.prompt)
            tail += w.batch * 2.0 * w.head_dim * (rows * w.prompt - rows * (rows - 1) / 2)
    if prompt_out:
        algo = 2 * per * units
        issued = 3 * per * units + per * scored + tail
    else:
        algo = per * scored + tail
        issued = 2 * per * scored + 2 * tail
    return algo, issued


def run_gpu(w, steps: int, warmup: int, sample_every: int, calib_mib: int = 0, cold: bool = False,
            prompt_out: bool = False):
    import numpy as np
    import torch
    from budgeted_decode_attention_amd import KVCache
    from workloads.generate import generate_layer

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if calib_mib:
        # a plain copy of known size, for scaling hardware byte counters
        a = torch.ones(calib_mib << 18, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    t0 = time.perf_counter()
    inputs = [generate_layer(w, l, dev, 0) for l in range(w.layers)]
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t0
    pol, hv, rc = w.policy_table(0)
    tabs = [np.tile(np.array(x, dtype=np.int32), w.layers) for x in (pol, hv, rc)]
    kw = {}
    if 3 in pol:
        kw.update(keep_ids=w.keep_ids(), vocab=w.vocab)
    if 4 in pol:
        kw.update(proj=inputs[0].proj)
    if 5 in pol:
        kw.update(history=np.tile(np.array(w.window_table(0), dtype=np.int32), w.layers))
    if 6 in pol:
        kw.update(special_ids=list(w.special_ids), punct_ids=list(w.punct_ids), vocab=w.vocab,
                  profile_rows=w.profile_rows, profile_threshold=w.profile_threshold)
    kv = KVCache(w.layers, w.batch, w.heads, w.head_dim, w.context, inputs[0].prompt_q.dtype,
                 *tabs, cache_bits=w.cache_bits, device=dev, **kw)
    ids = [x.ids for x in inputs]
    pids = [x[:, :w.prompt].contiguous() if x is not None else None for x in ids]
    dids = [[x[:, w.prompt + s].contiguous() for s in range(w.steps)] if x is not None else None for x in ids]
    out = torch.empty((w.layers, w.batch, w.heads, w.head_dim), dtype=torch.float32, device=dev)
    ev = torch.empty((w.layers, w.batch, w.heads), dtype=torch.int32, device=dev)
    # the optional prompt attention output, one layer's worth, rewritten by every layer
    pout = (torch.empty((w.batch, w.heads, w.prompt, w.head_dim), dtype=torch.float32, device=dev)
            if prompt_out else None)
    stream = torch.cuda.current_stream()

    samples = []
    # a sampled group holds at least 8 launches: a pair of events around a
    # single launch adds about 2 us of its own (measured: 25.0 against 23.2 us
    # per launch on the one-layer OPT-6.7B shape)
    group = max(1, -(-8 // w.layers))
    period = max(sample_every, group)

    def step(timed: bool):
        for l in range(w.layers):
            x = inputs[l]
            kv.prefill(l, x.prompt_q, x.prompt_k, x.prompt_v, pids[l], pout)
        e0 = e1 = None
        for s in range(w.steps):
            if timed and s % period == 0:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                n_in = 0
            for l in range(w.layers):
                x = inputs[l]
                tid = dids[l][s] if dids[l] is not None else None
                kv.decode_step(l, x.dec_q[s], x.dec_k[s], x.dec_v[s], tid, out[l], ev[l])
            if e0 is not None:
                n_in += w.layers
                if s % period == group - 1 or s == w.steps - 1:
                    e1.record(stream)
                    samples.append((e0, e1, n_in))
                    e0 = None

    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    # phase split of one untimed step (prefill vs decode), for the report
    p0, p1, p2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    p0.record(stream)
    for l in range(w.layers):
        x = inputs[l]
        kv.prefill(l, x.prompt_q, x.prompt_k, x.prompt_v, pids[l], pout)
    p1.record(stream)
    for s in range(w.steps):
        for l in range(w.layers):
            x = inputs[l]
            tid = dids[l][s] if dids[l] is not None else None
            kv.decode_step(l, x.dec_q[s], x.dec_k[s], x.dec_v[s], tid, out[l], ev[l])
    p2.record(stream)
    torch.cuda.synchronize()
    prefill_ms, decode_ms = p0.elapsed_time(p1), p1.elapsed_time(p2)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    cold_us = None
    if cold:
        # one more pass in which every sampled step group starts after a 1 GiB
        # read of another buffer (outside the timed group), so neither the L2
        # nor the 256 MB Infinity Cache holds the cache's rows; a read leaves
        # no dirty lines whose write-back would compete with the timed launch
        fl = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        sink = torch.empty((), dtype=torch.float32, device=dev)
        cold_samples = []
        for l in range(w.layers):
            x = inputs[l]
            kv.prefill(l, x.prompt_q, x.prompt_k, x.prompt_v, pids[l], pout)
        for s in range(w.steps):
            sample = s % sample_every == 0
            if sample:
                torch.sum(fl, dim=None, out=sink)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            for l in range(w.layers):
                x = inputs[l]
                tid = dids[l][s] if dids[l] is not None else None
                kv.decode_step(l, x.dec_q[s], x.dec_k[s], x.dec_v[s], tid, out[l], ev[l])
            if sample:
                e1.record(stream)
                cold_samples.append((e0, e1))
        torch.cuda.synchronize()
        cold_us = 1e3 * sum(a.elapsed_time(b) for a, b in cold_samples) / (len(cold_samples) * w.layers)
        del fl
    ids0 = inputs[0].ids.cpu().numpy() if inputs[0].ids is not None else None
    choice0 = kv.unit_policies(0).cpu().numpy() if 6 in pol else None
    group_ms = sum(a.elapsed_time(b) for a, b, _ in samples)
    n_launch = sum(n for _, _, n in samples)
    kernel_us = 1e3 * group_ms / n_launch
    return {"wall_s": wall, "gen_s": gen_s, "prefill_ms": prefill_ms, "decode_ms": decode_ms,
            "kernel_us": kernel_us, "n_samples": n_launch,
            "finite": bool(torch.isfinite(out).all().item()) and (pout is None or bool(torch.isfinite(pout).all().item())),
            "ids0": ids0,
            "split": kv.capacity(0) > 1024, "cold_us": cold_us, "choice0": choice0}


def stream_read_ceiling(nbytes: float, reps: int = 24, regions: int = 4):
    """Streaming-read reference on this GPU for one decode launch's bytes:
    libkvevict's plain read (the decode kernels' 16-byte non-temporal loads)
    of `nbytes` bytes, cycling over `regions` distinct buffers so that no
    launch finds its bytes in the Infinity Cache (as the decode's launches
    cycle over layers), timed with HIP events on the current stream.
    Returns (GB/s, microseconds per launch)."""
    import torch
    from budgeted_decode_attention_amd import binding
    n4 = (int(nbytes) + 15) // 16 * 4                      # int32 elements per region
    buf = torch.ones(regions * n4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    views = [buf[i * n4:(i + 1) * n4] for i in range(regions)]
    stream = torch.cuda.current_stream()
    for v in views:
        binding.kvevict_stream_read(v, sink, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for r in range(reps):
        binding.kvevict_stream_read(views[r % regions], sink, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / reps
    del buf
    return n4 * 4 / (us * 1e-6) / 1e9, us


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-units", type=int, default=0,
                    help="oracle sample size for the CPU baseline (0: per-workload default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold", action="store_true",
                    help="also time decode launches that start with the L2 and Infinity Cache flushed")
    ap.add_argument("--layers", type=int, default=0,
                    help="hardware-counter passes only: keep just the first N layers resident (the per-launch "
                         "shape is unchanged); the printed line then describes that reduced job")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (counter calibration)")
    ap.add_argument("--sketch-bits", type=int, default=0,
                    help="HashEvict workloads: sketch width 16, 32 or 64 (0: the workload's own, 32)")
    ap.add_argument("--prompt-out", action="store_true",
                    help="also produce the prompt attention output in every prefill")
    ap.add_argument("--sample-every", type=int, default=4,
                    help="event-time the per-layer decode launches of every k-th decode step")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {a.gpus}); the units shard across GPUs with no "
              f"exchange, so a multi-GPU figure is N x the one-GPU value", file=sys.stderr)
        sys.exit(2)
    from workloads import configs
    import dataclasses
    w = configs.get(a.workload)
    if a.layers:
        w = dataclasses.replace(w, layers=min(a.layers, w.layers))
    if a.sketch_bits:
        w = dataclasses.replace(w, sketch_bits=a.sketch_bits)

    cpu = None
    if not a.no_cpu_baseline:
        workers = min(16, len(os.sched_getaffinity(0)))
        n_units = a.cpu_units or {"h2o": 256, "persist": 256, "fastgen": 64, "hash": 32, "adaptive": 32}[w.family]
        cpu = cpu_baseline(w, n_units, workers)
        print(f"[bench] cpu baseline: {cpu['sample']}", file=sys.stderr, flush=True)

    r = run_gpu(w, a.steps, a.warmup, a.sample_every, a.calibration_copy_mib, a.cold, a.prompt_out)
    pf_algo, pf_issued = (x * w.layers for x in prefill_flops_per_layer(w, a.prompt_out))
    ms = 1e3 * r["wall_s"] / a.steps
    tokens = w.batch * w.steps
    if w.family == "adaptive":
        bytes_launch = adaptive_bytes_per_layer_step(w, r["ids0"], r["choice0"])
    else:
        bytes_launch = decode_bytes_per_layer_step(w, r["ids0"])
    achieved = bytes_launch / (r["kernel_us"] * 1e-6) / 1e9
    ceiling_gbs, ceiling_us = stream_read_ceiling(bytes_launch)
    kernel = ("decode_partial_kernel + decode_combine_kernel" if r["split"] else "decode_fused_kernel")
    if w.family == "hash":
        kernel = "hash_evict_kernel + " + kernel
    line = {
        "metric": METRIC, "value": tokens / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "layers": w.layers, "batch": w.batch, "heads": w.heads,
                   "head_dim": w.head_dim, "prompt": w.prompt, "decode_steps": w.steps,
                   "cached_kv": "4-bit slots (groups of 32, float32 scale)" if w.cache_bits == 4 else w.dtype,
                   "budget": {"h2o": f"{w.heavy} heavy + {w.recent} recent",
                              "fastgen": f"per head: full / local {w.local_window} / special+punct / "
                                         f"{w.freq_heavy} frequency + {w.local_window} local",
                              "hash": f"{w.hash_budget} slots, {w.sketch_bits}-bit sketches",
                              "persist": f"{w.heavy} heavy + {w.recent} recent by persistence count over "
                                         f"{w.history_window} steps",
                              "adaptive": f"profiled per (sequence, head): special / +punctuation / "
                                          f"+{w.freq_heavy} frequent / +{w.local_window} local / full at "
                                          f"{w.profile_threshold:.0%} of the last {w.profile_rows} rows' attention"}[w.family]},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": counter_traffic(w.name),
                     "kernel": kernel, "bytes_per_launch": bytes_launch,
                     "kernel_us": r["kernel_us"], "launches_timed": r["n_samples"],
                     "read_ceiling_gbs": ceiling_gbs, "read_ceiling_us": ceiling_us,
                     "frac_of_read_ceiling": achieved / ceiling_gbs},
        "cpu_baseline": cpu,
        "detail": {"prefill_ms_per_step": r["prefill_ms"], "decode_ms_per_step": r["decode_ms"],
                   "decode_only_tokens_per_s": tokens / (r["decode_ms"] * 1e-3),
                   "prompt_out": a.prompt_out,
                   "sketch_bits": w.sketch_bits if w.family == "hash" else None,
                   "hash_recovered_share": cpu.get("hash_recovered_share") if cpu else None,
                   "q4_output_rel_err_vs_storage_dtype_cache": cpu.get("q4_output_rel_err") if cpu else None,
                   "q4_error_units": cpu.get("q4_units") if cpu else None,
                   "composites_chosen": ({str(k): int((r["choice0"] == k).sum()) for k in range(1, 6)}
                                         if r["choice0"] is not None else None),
                   # FastGen's profile: one float32 per (unit, token) against the
                   # layer's uncompressed K/V bytes (the page reports 0.78 %)
                   "profile_memory": ({"bytes_per_layer": w.units_per_layer * w.context * 4,
                                       "kv_bytes_per_layer": w.units_per_layer * w.context * w.head_dim * 2 *
                                       {"f32": 4, "f16": 2, "bf16": 2}[w.dtype],
                                       "frac_of_kv": 4.0 / (2 * w.head_dim * {"f32": 4, "f16": 2, "bf16": 2}[w.dtype])}
                                      if w.family == "adaptive" else None),
                   "prefill_algorithmic_tflops": pf_algo / (r["prefill_ms"] * 1e-3) / 1e12,
                   "prefill_frac_of_dense_16bit_mfma_peak": pf_algo / (r["prefill_ms"] * 1e-3) / 2.5e15,
                   "prefill_issued_matrix_tflops": pf_issued / (r["prefill_ms"] * 1e-3) / 1e12,
                   "prefill_recompute_overhead": pf_issued / pf_algo - 1.0 if pf_algo else None,
                   "prefill_counters": prefill_counters(w.name),
                   "input_generation_s": r["gen_s"], "outputs_finite": r["finite"],
                   "cold_kernel_us": r["cold_us"],
                   # each cold sample is one step after the flush; with fewer
                   # than 8 layers its event pair adds about 2 us per launch
                   "cold_launches_per_sample": w.layers if r["cold_us"] else None,
                   "cold_frac": (bytes_launch / (r["cold_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS) if r["cold_us"] else None},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
