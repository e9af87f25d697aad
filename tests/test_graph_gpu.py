"""The library's calls under HIP graph capture: each graph is replayed several
times with eager work and synchronisations between the replays, and every
replay must give the eager result bit for bit (the kernels are deterministic,
the stores idempotent).  Covers the fused decode step the bench replays, a
split-K decode (partition + combine kernels, workspace), the fused prefill
store and the mixed batch split by kind."""
import numpy as np
import pytest
import torch

import workloads as W
from workloads import to_torch

pytestmark = pytest.mark.gpu

REPLAYS = 3


def replay_matches(fn, outs, keep=()):
    """Run fn eagerly, capture it, replay REPLAYS times; each replay's outputs
    must equal the eager ones.  `outs` are overwritten between replays,
    `keep` (caches the call writes) are only compared."""
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
    replay_matches(step, [t["out"] for _, t in layers],
                   keep=[c for _, t in layers for c in (t["k_cache"], t["v_cache"])])


def test_graph_split_decode(gpu_lib):
    """Few long sequences: split into partitions, merged by the combine kernel
    through the workspace."""
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
                   [out])


def test_graph_prefill_store_and_mixed(gpu_lib):
    pk = gpu_lib
    x = W.prefix_prefill()
    t = to_torch(x, "cuda")
    out = torch.empty_like(t["q"])
    msq = int(np.diff(x.cu_seqlens_q).max())
    replay_matches(lambda: pk.paged_prefill_store(t["q"], t["key"], t["value"], t["k_cache"],
                                                  t["v_cache"], t["block_tables"], t["cu_seqlens_q"],
                                                  t["cu_seqlens_k"], x.scale, max_seqlen_q=msq,
                                                  out=out),
                   [out], keep=[t["k_cache"], t["v_cache"]])
    y = W.mixed_batch()
    u = to_torch(y, "cuda")
    pk.kv_store(u["key"], u["value"], u["slot_mapping"], u["k_cache"], u["v_cache"])
    lq = np.diff(y.cu_seqlens_q)
    lk = np.diff(y.cu_seqlens_k)
    nd = int(np.sum(lq == 1))
    out2 = torch.empty_like(u["q"])
    ws = torch.empty(max(pk.decode_workspace_size(nd, 16, 8, 128, int(lk[:nd].max())), 1),
                     dtype=torch.uint8, device="cuda")
    replay_matches(lambda: pk.paged_prefill_decode(u["q"], u["k_cache"], u["v_cache"], u["block_tables"],
                                                   u["cu_seqlens_q"], u["cu_seqlens_k"], y.scale,
                                                   num_decode_seqs=nd, max_seqlen_q=int(lq[nd:].max()),
                                                   max_decode_context_len=int(lk[:nd].max()),
                                                   out=out2, workspace=ws),
                   [out2])
