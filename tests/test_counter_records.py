"""The committed hardware-counter records that bench.py reads (CPU only):
each machine-readable section parses, its kernel sources exist, the decode
traffic equals the record's own FETCH_SIZE / WRITE_SIZE arithmetic, and a
record is ignored once its sources no longer hash to the recorded value."""

import glob
import hashlib
import os
import re

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def records():
    out = {}
    for p in sorted(glob.glob(os.path.join(ROOT, "profiles", "counters_*.txt"))):
        rec = {}
        for line in open(p):
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
        out[os.path.basename(p)] = (rec, open(p).read())
    return out


def test_every_record_names_existing_sources_and_a_workload():
    recs = records()
    assert recs
    for name, (rec, _) in recs.items():
        assert rec.get("workload"), name
        srcs = rec.get("kernel_sources", "").split()
        assert srcs, name
        for f in srcs:
            assert os.path.exists(os.path.join(ROOT, f)), (name, f)
        assert re.fullmatch(r"[0-9a-f]{16}", rec.get("kernel_sources_sha256", "")), name


def test_decode_traffic_is_the_scaled_counter_sum():
    for name, (rec, text) in records().items():
        if "traffic_bytes_per_launch" not in rec:
            continue
        m = re.search(r"Traffic per launch = ([\d.]+) x ([\d.]+) KiB \+ ([\d.]+) x ([\d.]+) KiB = (\d+) KiB", text)
        assert m, name
        ff, fetch, wf, write, total = (float(x) for x in m.groups())
        assert abs(ff * fetch + wf * write - total) <= 1.0, name
        assert int(rec["traffic_bytes_per_launch"]) == int(total) * 1024, name


def _source_hash(rec):
    h = hashlib.sha256()
    for f in rec["kernel_sources"].split():
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def test_records_are_read_only_while_their_sources_match(monkeypatch):
    for name, (rec, _) in records().items():
        live = bench._counter_records(rec["workload"])
        assert (rec in live) == (_source_hash(rec) == rec["kernel_sources_sha256"]), name
    real_open = open

    def changed_sources(path, mode="r", *a, **k):
        f = real_open(path, mode, *a, **k)
        if "b" in mode and path.endswith((".hip", ".hpp")):
            data = f.read() + b"\n// changed\n"
            f.close()
            import io
            return io.BytesIO(data)
        return f

    monkeypatch.setattr("builtins.open", changed_sources)
    assert bench.counter_traffic("opt30b_decode_h2o") is None
    assert bench.prefill_counters("opt30b_decode_h2o") is None


def test_every_kernel_trace_names_its_sources_and_their_hash():
    """Each kernel-trace summary carries the sources it was taken with and
    their hash, so a reader can tell whether it still describes the code."""
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "kernels_*.md")))
    assert paths
    for p in paths:
        text = open(p).read()
        m = re.search(r"^kernel_sources: (.+)$", text, re.M)
        assert m, p
        for f in m.group(1).split():
            assert os.path.exists(os.path.join(ROOT, f)), (p, f)
        assert re.search(r"^kernel_sources_sha256: [0-9a-f]{16}$", text, re.M), p
        assert "rocprofv3 --kernel-trace --stats" in text, p
