"""Host logic of bench.py: algorithmic byte and flop counts, and the lookup of
profiled HBM traffic (reported only while the kernel sources are unchanged)."""
import importlib.util
import math
import os
import shutil

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_decode_bytes_brute_force():
    b = _bench()
    ctx, bs, hq, hkv, d = [0, 1, 17, 300], 16, 16, 8, 128
    for window in (0, 5, 256):
        kv = tbl = 0
        for L in ctx:
            keys = [j for j in range(L) if window == 0 or L - 1 - j < window]
            kv += len(keys) * hkv * d * 2 * 2
            tbl += 4 * len({j // bs for j in keys})
        want = kv + tbl + 2 * len(ctx) * hq * d * 2 + 4 * len(ctx)
        assert b.decode_bytes(ctx, bs, hq, hkv, d, window) == want


def test_prefill_flops_brute_force():
    b = _bench()
    lq, lk = [3, 1, 5], [3, 7, 9]
    for window in (0, 2):
        pairs = 0
        for q_len, k_len in zip(lq, lk):
            p = k_len - q_len
            for i in range(q_len):
                pairs += sum(1 for j in range(k_len)
                             if j <= p + i and (window == 0 or p + i - j < window))
        assert b.prefill_flops(lq, lk, 16, 128, window) == 4 * 128 * pairs * 16


def test_profiled_traffic_records_parse_and_track_sources(tmp_path, monkeypatch):
    b = _bench()
    with open(b.TRAFFIC_PROFILE) as fh:
        records = [l for l in fh.read().splitlines() if l.startswith("traffic-record:")]
    assert {"decode_c64_fused", "prefill_prefix"} <= {r.split()[1] for r in records}
    for r in records:
        fields = dict(f.split("=", 1) for f in r.split()[2:])
        assert float(fields["fetch_kib"]) > 0 and len(fields["sources"]) == 16
    # A changed kernel source no longer matches the recorded hash: traffic is None.
    csrc = tmp_path / "csrc"
    shutil.copytree(b.CSRC, csrc)
    with open(csrc / "paged_decode.hip", "a") as fh:
        fh.write("\n// changed\n")
    monkeypatch.setattr(b, "CSRC", str(csrc))
    assert b.profiled_traffic("decode_c64_fused", "paged_decode.hip") is None
    assert b.profiled_traffic("no_such_record", "paged_decode.hip") is None
