"""The seeded generators: shapes, determinism, rounding, structure (CPU only)."""

import ast
import os

import numpy as np
import torch

import workloads
from workloads import configs
from workloads.generate import generate_layer, unit_sequence

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_five_workloads_and_budgets():
    w = [configs.get(n) for n in configs.ORDER]
    assert [x.index for x in w] == [1, 2, 3, 4, 5]
    assert (w[0].heavy, w[0].recent) == (16, 16)
    assert (w[1].heavy, w[1].recent) == (51, 51)
    assert (w[2].heavy, w[2].recent, w[2].units) == (204, 204, 86016)
    assert (w[3].local_window, w[3].freq_heavy) == (1024, 409)
    assert w[4].hash_budget == 4096
    pol, hv, rc = w[3].policy_table(0)
    assert sorted(pol) == sorted([0, 1, 2, 3] * 16)
    for p, a, b in zip(pol, hv, rc):
        assert (a, b) == {0: (0, 0), 1: (409, 1024), 2: (0, 1024), 3: (0, 0)}[p]


def test_generation_is_deterministic_and_rounded():
    w = configs.scaled("opt6.7b_layer_h2o", batch=2, heads=3, prompt=40, steps=10)
    a = generate_layer(w, 0)
    b = generate_layer(w, 0)
    assert torch.equal(a.prompt_k, b.prompt_k) and torch.equal(a.dec_v, b.dec_v)
    assert a.prompt_q.dtype == torch.float16 and a.prompt_q.shape == (2, 3, 40, 128)
    assert a.dec_q.shape == (10, 2, 3, 128)
    c = generate_layer(w, 1)
    assert not torch.equal(a.prompt_k, c.prompt_k)
    Q, K, V = unit_sequence(a, 1, 2)
    assert Q.shape == (50, 128) and Q.dtype == np.float64
    assert np.array_equal(K[40:], a.dec_k[:, 1, 2].double().numpy())
    assert np.array_equal(K.astype(np.float16).astype(np.float64), K)


def test_heavy_direction_structure_present():
    w = configs.scaled("opt6.7b_layer_h2o", batch=1, heads=2, prompt=200, steps=0)
    x = generate_layer(w, 0)
    k = x.prompt_k[0].float()
    n = k.norm(dim=-1)                    # heavy keys have norm ~ sqrt(d) * sqrt(1 + 9)
    assert (n > 20).sum().item() >= 2 * int(0.05 * 200) * 0.8


def test_fastgen_ids_and_hash_projection():
    w = configs.scaled("llama65b_fastgen", batch=2, heads=4, prompt=64, steps=8)
    x = generate_layer(w, 0)
    assert x.ids.shape == (2, 72) and x.ids.dtype == torch.int32
    assert int(x.ids.min()) >= 0 and int(x.ids.max()) < 32000
    w = configs.scaled("hashevict_lsh", batch=1, heads=2, prompt=64, steps=8)
    x = generate_layer(w, 0)
    assert x.proj.shape == (128, 32) and x.proj.dtype == torch.bfloat16


def _imports(path):
    tree = ast.parse(open(path).read())
    out = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            out |= {a.name.split(".")[0] for a in node.names}
        elif isinstance(node, ast.ImportFrom) and node.module and node.level == 0:
            out.add(node.module.split(".")[0])
    return out


def test_oracle_and_gpu_path_share_no_code():
    """The oracle imports only numpy and the standard library; the workloads import
    neither side; the GPU package never imports the oracle."""
    allowed = {"numpy", "math", "dataclasses", "typing", "__future__", "itertools", "fractions"}
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith(".py"):
            assert _imports(os.path.join(ROOT, "oracle", f)) <= allowed, f
    for f in os.listdir(os.path.join(ROOT, "workloads")):
        if f.endswith(".py"):
            assert not ({"oracle", "budgeted_decode_attention_amd"} & _imports(os.path.join(ROOT, "workloads", f)))
    pkg = os.path.join(ROOT, "budgeted_decode_attention_amd")
    for dp, _, fs in os.walk(pkg):
        for f in fs:
            if f.endswith(".py"):
                assert "oracle" not in _imports(os.path.join(dp, f)), f
