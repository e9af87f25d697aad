"""Split decode merges its partitions in the same launch: each (sequence, KV
head) counts its finished partitions on a counter taken from a per-GPU pool of
2^20, in turn, and the partition that completes the count merges and sets the
counter back to zero.  Repeating one split call past the end of the pool (so
its counters wrap around onto ones every earlier call has used) must keep
giving the same output, bit for bit, and the oracle's result."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from workloads import to_torch

pytestmark = pytest.mark.gpu

POOL = 1 << 20


def test_merge_counters_survive_pool_wrap(gpu_lib):
    pk = gpu_lib
    # 255 sequences x 1 KV head (2 query heads): fewer pairs than CUs, so the
    # planner splits their 200..300-key contexts (several partitions each).
    x = W.decode_inputs(9301, 255, 200, 300, 16, heads=(2, 1, 128))
    t = to_torch(x, "cuda")
    mcl = int(x.context_lens.max())
    ps, nparts = pk.decode_plan(255, 1, mcl)
    assert nparts > 1
    ws = torch.empty(max(pk.decode_workspace_size(255, 2, 1, 128, mcl), 1), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(t["q"])

    def call():
        pk.paged_decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                        x.scale, max_context_len=mcl, out=out, workspace=ws)

    call()
    first = out.clone()
    pairs = 255
    calls = POOL // pairs + 100          # past the end of the pool whatever its cursor
    for i in range(calls):
        call()
        if i % 1000 == 999:
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), first.view(torch.int16)), i
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), first.view(torch.int16))
    ref = oracle.paged_decode(x.q, x.k_cache, x.v_cache, x.block_tables, x.context_lens, x.scale)
    g = out.float().cpu().numpy().astype(np.float64)
    err = np.abs(g - ref)
    assert np.isfinite(g).all() and err.max() <= 2e-2 and err.mean() <= 2e-3, (err.max(), err.mean())
