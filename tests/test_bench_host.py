"""CPU: host-side pieces of bench.py that decide what is measured.

* chunk_addresses lists exactly the KV chunks a decode step reads: per
  (sequence, KV head) its visible pages in order, K then V, at the cache's
  strides; empty sequences and keys before a sliding window contribute none.
* traffic_for reports stored HBM traffic only while the stored kernel hash
  matches the sources.
* bench.py refuses more than one GPU with a message.
* the cold-cache rotation: a replica is read again only after four times the
  last-level caches of other replicas' K/V, for every workload, at any step
  count (a flush also runs before each measured phase).
"""
import json
import os
import subprocess
import sys

import torch

import bench
from paged_kv_decode_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_chunk_addresses_follow_the_visible_pages():
    w = W.custom(batch=3, num_q_heads=4, num_kv_heads=2, head_dim=64, dtype=torch.float16,
                 context_lens=[40, 0, 70], seed=11, window=30)
    p = W.generate(w)
    k, v, pt = p.k_cache, p.v_cache, p.page_table
    got = bench.chunk_addresses(p, k, v, pt).tolist()
    eb = k.element_size()
    want = []
    for b, n in enumerate(p.context_lens.tolist()):
        lo = max(0, n - 30)
        if n == lo:
            continue
        for h in range(2):
            for j in range(lo // 16, (n + 15) // 16):
                off = (int(pt[b, j]) * k.stride(0) + h * k.stride(1)) * eb
                want += [k.data_ptr() + off, v.data_ptr() + off]
    assert got == want
    # sequence 0 sees keys [10, 40): pages 0..2; sequence 2 sees [40, 70): pages 2..4
    assert len(got) == 2 * 2 * (3 + 3)


def test_traffic_is_reported_only_for_the_current_kernel_sources(tmp_path, monkeypatch):
    current = bench.kernel_hash()
    assert len(current) == 16 and current == bench.kernel_hash()
    stored = {"kernel_hash": current,
              "workloads": {"llama1b_ctx3060_f16": {"bytes_per_launch": 123}}}
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic.json").write_text(json.dumps(stored))
    monkeypatch.setattr(bench, "kernel_hash", lambda: current)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_for("llama1b_ctx3060_f16", None) == 123
    assert bench.traffic_for("ctx100k_gqa6_f16", None) is None
    stored["kernel_hash"] = "0" * 16
    (prof / "traffic.json").write_text(json.dumps(stored))
    assert bench.traffic_for("llama1b_ctx3060_f16", None) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 2
    assert "single" in r.stderr and "--gpus 2" not in r.stdout


def test_replica_rotation_rereads_only_after_four_cache_sizes():
    for name in W.CONFIG_ORDER:
        p = W.generate(W.CONFIGS[name])
        kv = p.kv_bytes()
        pool = 2 * p.k_cache.numel() * p.k_cache.element_size()
        for layers in (1, 16):
            R = bench.replica_count(kv, pool, layers)
            assert R % layers == 0 and R >= 2 * layers
            if R * pool < (64 << 30) - pool:       # not capped by the 64 GiB of pools
                assert (R - 1) * kv >= 4 * bench.CACHE_BYTES, (name, layers, R)
    assert bench.FLUSH_BYTES >= 4 * (256 << 20)
    assert bench.replica_count(1 << 20, 1 << 20, 1, replicas=7) == 7
    assert bench.replica_count(1 << 20, 1 << 20, 4, replicas=7) == 8


def test_percentiles():
    r = bench.percentiles([float(x) for x in range(1, 101)])
    assert r["n"] == 100 and r["min"] == 1 and r["max"] == 100
    assert r["p10"] == 11 and r["median"] == 51 and r["p90"] == 90
    assert bench.percentiles([]) is None
