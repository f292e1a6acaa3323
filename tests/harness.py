"""Drives one layer of a workload through libkvevict and checks it against the
oracle in lockstep.  Used by the GPU parity tests and the smoke check."""

from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Iterable, List, Optional, Tuple

import numpy as np
import torch

from budgeted_decode_attention_amd import KVCache
from oracle import lockstep, quant
from workloads import configs
from workloads.configs import ADAPTIVE, FULL, H2O, HASH, LOCAL, PERSIST, SPECIAL, Workload
from workloads.generate import LayerInputs, generate_layer, unit_ids, unit_sequence


def make_cache(w: Workload, inp: LayerInputs, policy=None, heavy=None, recent=None, max_context=None,
               layers: int = 1, history=None) -> KVCache:
    pol, hv, rc = w.policy_table(0)
    pol = pol if policy is None else policy
    hv = hv if heavy is None else heavy
    rc = rc if recent is None else recent
    tables = [np.array(x, dtype=np.int32) for x in (pol, hv, rc)]
    tables = [np.tile(t, layers) for t in tables]
    kw = {}
    if SPECIAL in list(pol):
        kw.update(keep_ids=w.keep_ids(), vocab=w.vocab)
    if HASH in list(pol):
        kw.update(proj=inp.proj)
    if ADAPTIVE in list(pol):
        kw.update(special_ids=list(w.special_ids), punct_ids=list(w.punct_ids), vocab=w.vocab,
                  profile_rows=w.profile_rows, profile_threshold=w.profile_threshold)
    if PERSIST in list(pol):
        hw = [w.history_window if p == PERSIST else 0 for p in pol] if history is None else history
        kw.update(history=np.tile(np.array(hw, dtype=np.int32), layers))
    return KVCache(layers, w.batch, w.heads, w.head_dim, max_context or w.context,
                   inp.prompt_q.dtype, tables[0], tables[1], tables[2], cache_bits=w.cache_bits, **kw)


@dataclass
class GpuLayerRun:
    prefill_pos: np.ndarray      # [B, H, cap]
    prefill_cnt: np.ndarray
    prefill_S: np.ndarray
    final_pos: np.ndarray
    final_cnt: np.ndarray
    final_S: np.ndarray
    out: np.ndarray              # [T, B, H, d]
    evicted: np.ndarray          # [T, B, H]
    prompt_out: Optional[np.ndarray]
    choice: Optional[np.ndarray] = None  # [B, H] composite chosen by profiled units (0: not profiled)


def run_layer(kv: KVCache, inp: LayerInputs, layer: int = 0, steps: Optional[int] = None,
              want_prompt_out: bool = False) -> GpuLayerRun:
    """Prefill + `steps` decode steps on the GPU; logs copied to the host."""
    P = inp.prompt_q.shape[2]
    T = inp.dec_q.shape[0] if steps is None else steps
    Bt, H, d = kv.batch, kv.heads, kv.head_dim
    dev = kv.device
    ids = inp.ids.to(dev) if inp.ids is not None else None
    po = torch.empty((Bt, H, P, d), dtype=torch.float32, device=dev) if want_prompt_out else None
    kv.prefill(layer, inp.prompt_q, inp.prompt_k, inp.prompt_v,
               ids[:, :P].contiguous() if ids is not None else None, po)
    p0, c0, s0 = kv.kept_indices(layer)
    p0, c0, s0 = p0.cpu(), c0.cpu(), s0.cpu()
    choice = kv.unit_policies(layer).cpu().numpy()
    out = torch.empty((T, Bt, H, d), dtype=torch.float32, device=dev)
    ev = torch.empty((T, Bt, H), dtype=torch.int32, device=dev)
    for s in range(T):
        tid = ids[:, P + s].contiguous() if ids is not None else None
        kv.decode_step(layer, inp.dec_q[s], inp.dec_k[s], inp.dec_v[s], tid, out[s], ev[s])
    p1, c1, s1 = kv.kept_indices(layer)
    torch.cuda.synchronize()
    return GpuLayerRun(p0.numpy(), c0.numpy(), s0.numpy(), p1.cpu().numpy(), c1.cpu().numpy(), s1.cpu().numpy(),
                  out.cpu().numpy(), ev.cpu().numpy(), po.cpu().numpy() if po is not None else None, choice)


def gpu_unit(r: GpuLayerRun, b: int, h: int) -> lockstep.GpuUnit:
    n0, n1 = int(r.prefill_cnt[b, h]), int(r.final_cnt[b, h])
    return lockstep.GpuUnit(
        prefill_pos=r.prefill_pos[b, h, :n0].astype(np.int64), evicted=r.evicted[:, b, h].astype(np.int64),
        out=r.out[:, b, h], final_pos=r.final_pos[b, h, :n1].astype(np.int64),
        prefill_S=r.prefill_S[b, h, :n0], final_S=r.final_S[b, h, :n1],
        prompt_out=r.prompt_out[b, h] if r.prompt_out is not None else None)


def check_unit(w: Workload, inp_cpu: LayerInputs, r: GpuLayerRun, b: int, h: int, policy=None, heavy=None,
               recent=None, scale=None, history=None) -> lockstep.UnitReport:
    pol, hv, rc = w.policy_table(0)
    p = pol[h] if policy is None else policy[h]
    hh = hv[h] if heavy is None else heavy[h]
    rr = rc[h] if recent is None else recent[h]
    sc = (1.0 / np.sqrt(w.head_dim)) if scale is None else scale
    Q, K, V = unit_sequence(inp_cpu, b, h)
    P = inp_cpu.prompt_q.shape[2]
    T = r.out.shape[0]
    g = gpu_unit(r, b, h)
    # 4-bit slots: cached rows read back what the format holds
    Kc, Vc = (quant.roundtrip(K), quant.roundtrip(V)) if w.cache_bits == 4 else (None, None)
    if p == H2O:
        rep = lockstep.check_h2o(Q, K, V, P, hh, rr, sc, g, steps=T, Kc=Kc, Vc=Vc)
    elif p == HASH:
        Wp = inp_cpu.proj.float().double().cpu().numpy()
        rep = lockstep.check_hash(Q, K, V, Wp, P, hh, sc, g, steps=T, Kc=Kc, Vc=Vc)
    elif p == PERSIST:
        win = w.history_window if history is None else history[h]
        rep = lockstep.check_persist(Q, K, V, P, hh, rr, win, sc, g, steps=T, Kc=Kc, Vc=Vc)
    elif p == ADAPTIVE:
        rep = lockstep.check_adaptive(Q, K, V, unit_ids(inp_cpu, b), P, list(w.special_ids), list(w.punct_ids),
                                      hh, rr, sc, w.profile_rows, w.profile_threshold, g, int(r.choice[b, h]),
                                      steps=T)
    else:
        rep = lockstep.check_fastgen(p, Q, K, V, P, sc, g, heavy=hh, recent=rr,
                                     ids=unit_ids(inp_cpu, b), keep_ids=w.keep_ids(), steps=T)
    return rep


def check_all(w: Workload, inp_cpu: LayerInputs, r: GpuLayerRun, units: Optional[Iterable[Tuple[int, int]]] = None,
              **kw) -> lockstep.UnitReport:
    total = lockstep.UnitReport()
    if units is None:
        units = [(b, h) for b in range(w.batch) for h in range(w.heads)]
    for b, h in units:
        total.merge(check_unit(w, inp_cpu, r, b, h, **kw), tag=f"[b={b} h={h}] ")
    return total


def check_invariants(w: Workload, r: GpuLayerRun, P: int, policy=None, heavy=None, recent=None,
                     history=None) -> List[str]:
    """Properties that hold at any size: budgets, recent windows, unique in-range positions."""
    pol, hv, rc = w.policy_table(0)
    pol = pol if policy is None else policy
    hv = hv if heavy is None else heavy
    rc = rc if recent is None else recent
    T = r.out.shape[0]
    t_last = P + T - 1
    bad = []
    for b in range(w.batch):
        for h in range(w.heads):
            n = int(r.final_cnt[b, h])
            pos = r.final_pos[b, h, :n]
            if len(set(pos.tolist())) != n or (pos < 0).any() or (pos > t_last).any():
                bad.append(f"b={b} h={h}: positions not unique/in range")
            if (r.final_pos[b, h, n:] != -1).any():
                bad.append(f"b={b} h={h}: slots past count not empty")
            p = pol[h]
            if p == H2O:
                if n > hv[h] + rc[h]:
                    bad.append(f"b={b} h={h}: over budget")
                win = set(range(max(0, t_last - rc[h] + 1), t_last + 1))
                if not win <= set(pos.tolist()):
                    bad.append(f"b={b} h={h}: recent window not kept")
                if not (r.final_S[b, h, :n] > 0).all():
                    bad.append(f"b={b} h={h}: non-positive score")
            elif p == PERSIST:
                win = w.history_window if history is None else history[h]
                if n > hv[h] + rc[h]:
                    bad.append(f"b={b} h={h}: over budget")
                win_r = set(range(max(0, t_last - rc[h] + 1), t_last + 1))
                if not win_r <= set(pos.tolist()):
                    bad.append(f"b={b} h={h}: recent window not kept")
                bits = np.ascontiguousarray(r.final_S[b, h, :n]).view(np.uint64)
                if win < 64 and (bits >> np.uint64(win)).any():
                    bad.append(f"b={b} h={h}: history bits beyond the window")
            elif p == LOCAL:
                if sorted(pos.tolist()) != list(range(max(0, t_last - rc[h] + 1), t_last + 1)):
                    bad.append(f"b={b} h={h}: local window wrong")
            elif p == HASH:
                if n > hv[h] or t_last not in set(pos.tolist()):
                    bad.append(f"b={b} h={h}: hash cache wrong")
            if not np.isfinite(r.out[:, b, h]).all():
                bad.append(f"b={b} h={h}: non-finite output")
    return bad
