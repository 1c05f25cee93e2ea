"""Host logic of bench.py, on the CPU: the algorithmic byte count that the
step's GB/s and the scorer's roofline rest on (closed forms at the headline
shape), the HBM traffic lookup keyed to the scorer's sources, and the refusal
of more than one GPU."""
import json
import subprocess
import sys

import numpy as np

import bench
import workloads as W


def test_algorithmic_bytes_headline_closed_form():
    inp = W.make_inputs(W.WORKLOADS["headline"])
    wl = inp.wl
    assert (wl.B, wl.q, wl.H, wl.H_I, wl.topk) == (4, 8, 16, 4, 32)
    t = np.full((4, 8, 32), -1, dtype=np.int64)
    t[:, :, :30] = np.arange(30)                       # 30 blocks per row, -1 padded
    t[0, 1, :30] = np.arange(10, 40)                   # sequence 0: rows select {0..29} and {10..39}
    ab = bench.algorithmic_bytes(inp, t)
    assert ab["index_pages"] == 4 * 2048 * 8704 == 71_303_168     # every index page once
    assert ab["kv_pages"] == 2 * (40 + 3 * 30) * 8704              # distinct K and V pages per sequence
    rows = 32
    assert bench.query_bytes(wl) == 4                              # the fp32 query read (its e4m3 codes: an intermediate)
    other = (3 * rows * 128 * 4                  # new K, V, index rows in (fp32)
             + 3 * rows * (64 + 4)               # the three stored MXFP4 rows out
             + rows * 16 * 128 * 4               # query
             + rows * 4 * 128 * 2 + rows * 4 * 4  # index query (bf16), weights
             + 4 * 2048 * 4 + 4 * 4              # page table, context lengths
             + rows * 16 * 128 * 2 + rows * 16 * 4)  # output (bf16), lse
    assert ab["other"] == other == 517_008
    assert ab["total"] == ab["index_pages"] + ab["kv_pages"] + ab["other"]


def test_traffic_follows_the_scorer_sources(monkeypatch):
    with open(bench.TRAFFIC_FILE.format("headline")) as fh:
        js = json.load(fh)
    if js["scorer_sources_sha256"] == bench.scorer_source_hash():
        assert bench.measured_traffic("headline") == js["fetch_bytes_per_launch"] + js["write_bytes_per_launch"]
    monkeypatch.setattr(bench, "scorer_source_hash", lambda: "0" * 64)
    assert bench.measured_traffic("headline") is None              # the kernel changed since the counters
    assert bench.measured_traffic("no_such_workload") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_cache_replicas_exceed_the_infinity_cache():
    """The timed steps rotate over enough cache replicas that they touch at
    least 512 MB (twice the 256 MB Infinity Cache), and never fewer than asked."""
    import bench
    assert bench.cache_replicas(88_131_472) == 6            # the 256K workload: 6 x 88 MB = 529 MB
    assert bench.cache_replicas(16_030_160) == 32           # the 16K FP8 workload: 32 x 16 MB
    assert bench.cache_replicas(76_650_368) == 7            # 6 x 76.7 MB would be 460 MB
    assert bench.cache_replicas(401_518_848) == 6           # large steps keep the minimum
    assert bench.cache_replicas(401_518_848, at_least=2) == 2
    for b in (1, 10**6, 3 * 10**7, 10**9):
        r = bench.cache_replicas(b)
        assert r * b >= bench.ROTATION_BYTES and r >= 6
