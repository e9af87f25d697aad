"""The library's calls under HIP graph capture: each graph is replayed several
times with eager work and synchronisations between the replays, and every
replay must give the eager result bit for bit (the kernels are deterministic,
the stores idempotent), and every replay's outputs are also checked against
the CPU oracle (max-abs 2e-2, mean-abs 2e-3).  Covers the fused decode step the bench replays, a
split-K decode (partitions merged in the same launch, workspace), the fused prefill
store and the mixed batch split by kind."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from workloads import to_torch

pytestmark = pytest.mark.gpu

REPLAYS = 3
MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def close_to(ref):
    """A check of one output tensor against an oracle result (float64)."""
    def check(got):
        g = got.float().cpu().numpy().astype(np.float64)
        assert np.isfinite(g).all()
        err = np.abs(g - ref)
        assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (float(err.max()), float(err.mean()))
    return check


def replay_matches(fn, outs, keep=(), refs=()):
    """Run fn eagerly, capture it, replay REPLAYS times; each replay's outputs
    must equal the eager ones, and refs[i] (a check against the oracle) must
    accept outs[i] after every replay.  `outs` are overwritten between
    replays, `keep` (caches the call writes) are only compared."""
    fn()
    torch.cuda.synchronize()
    checked = list(outs) + list(keep)
    eager = [o.clone() for o in checked]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm the capture stream
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    noise = torch.randn(1 << 20, device="cuda")
    for _ in range(REPLAYS):
        for o in outs:
            o.fill_(3.0)                     # eager work between replays
        noise.mul_(1.0001)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(checked, eager):
            assert torch.equal(o.view(torch.int16), e.view(torch.int16))
        for o, check in zip(outs, refs):
            check(o)


def test_graph_fused_decode_layers(gpu_lib):
    """Three layers of the c = 64 step (store + attend per layer), as the bench
    captures them (the stored token is the same each time, so the caches are
    only compared)."""
    pk = gpu_lib
    layers = []
    for l in range(3):
        x = W.deep_decode_layer(l)
        t = to_torch(x, "cuda")
        t["out"] = torch.empty_like(t["q"])
        layers.append((x, t))
    mcl = layers[0][0].max_context_len

    def step():
        for x, t in layers:
            pk.paged_decode_store(t["q"], t["key"], t["value"], t["k_cache"], t["v_cache"],
                                  t["block_tables"], t["context_lens"], x.scale,
                                  max_context_len=mcl, out=t["out"])
    refs = []
    for x, _ in layers:
        kc, vc = oracle.kv_store(x.k_cache, x.v_cache, x.key, x.value, x.slot_mapping)
        refs.append(close_to(oracle.paged_decode(x.q, kc, vc, x.block_tables, x.context_lens,
                                                 x.scale)))
    replay_matches(step, [t["out"] for _, t in layers],
                   keep=[c for _, t in layers for c in (t["k_cache"], t["v_cache"])], refs=refs)


def test_graph_split_decode(gpu_lib):
    """Few long sequences: split into partitions whose partials (in the
    workspace) are merged in the same launch through the merge counters, which
    every replay reuses."""
    pk = gpu_lib
    rng = np.random.default_rng(71)
    lens = np.array([4000, 2500, 3100, 17], np.int32)
    bs = 64
    mb = int(np.ceil(lens.max() / bs))
    nb = len(lens) * mb
    tables = rng.permutation(nb).reshape(len(lens), mb).astype(np.int32)
    x = W.PagedInputs(q=W.normal_bf16(rng, (4, 16, 128)), k_cache=W.normal_bf16(rng, (nb, bs, 8, 128)),
                      v_cache=W.normal_bf16(rng, (nb, bs, 8, 128)), block_tables=tables,
                      context_lens=lens, block_size=bs, scale=1 / np.sqrt(128))
    t = to_torch(x, "cuda")
    assert pk.decode_plan(4, 8, int(lens.max()))[1] > 1
    out = torch.empty_like(t["q"])
    ws = torch.empty(pk.decode_workspace_size(4, 16, 8, 128, int(lens.max())), dtype=torch.uint8,
                     device="cuda")
    replay_matches(lambda: pk.paged_decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                                           t["context_lens"], x.scale,
                                           max_context_len=int(lens.max()), out=out, workspace=ws),
                   [out], refs=[close_to(oracle.paged_decode(x.q, x.k_cache, x.v_cache, tables, lens,
                                                             x.scale))])


def test_graph_prefill_store_and_mixed(gpu_lib):
    pk = gpu_lib
    x = W.prefix_prefill()
    t = to_torch(x, "cuda")
    out = torch.empty_like(t["q"])
    msq = int(np.diff(x.cu_seqlens_q).max())
    kc, vc = oracle.kv_store(x.k_cache, x.v_cache, x.key, x.value, x.slot_mapping)
    ref = oracle.paged_prefill(x.q, kc, vc, x.block_tables, x.cu_seqlens_q, x.cu_seqlens_k, x.scale)
    replay_matches(lambda: pk.paged_prefill_store(t["q"], t["key"], t["value"], t["k_cache"],
                                                  t["v_cache"], t["block_tables"], t["cu_seqlens_q"],
                                                  t["cu_seqlens_k"], x.scale, max_seqlen_q=msq,
                                                  out=out),
                   [out], keep=[t["k_cache"], t["v_cache"]], refs=[close_to(ref)])
    y = W.mixed_batch()
    u = to_torch(y, "cuda")
    pk.kv_store(u["key"], u["value"], u["slot_mapping"], u["k_cache"], u["v_cache"])
    lq = np.diff(y.cu_seqlens_q)
    lk = np.diff(y.cu_seqlens_k)
    nd = int(np.sum(lq == 1))
    kc2, vc2 = oracle.kv_store(y.k_cache, y.v_cache, y.key, y.value, y.slot_mapping)
    ref2 = oracle.paged_prefill(y.q, kc2, vc2, y.block_tables, y.cu_seqlens_q, y.cu_seqlens_k,
                                y.scale)
    out2 = torch.empty_like(u["q"])
    ws = torch.empty(max(pk.decode_workspace_size(nd, 16, 8, 128, int(lk[:nd].max())), 1),
                     dtype=torch.uint8, device="cuda")
    replay_matches(lambda: pk.paged_prefill_decode(u["q"], u["k_cache"], u["v_cache"], u["block_tables"],
                                                   u["cu_seqlens_q"], u["cu_seqlens_k"], y.scale,
                                                   num_decode_seqs=nd, max_seqlen_q=int(lq[nd:].max()),
                                                   max_decode_context_len=int(lk[:nd].max()),
                                                   out=out2, workspace=ws),
                   [out2], refs=[close_to(ref2)])
