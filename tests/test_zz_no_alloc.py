"""pk_paged_decode_noalloc (the decode entry that allocates nothing: its
split-K partials live in the library's static per-GPU scratch) against
pk_paged_decode with a caller workspace, through the C ABI: bit-identical
outputs, and within the attention bar of the oracle, on two calls in a row,
the second with a smaller input (the scratch keeps the first call's
contents).  Plans that need more than the scratch are refused on the host."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from workloads import to_torch

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def _case(seed, lens, bs, window=0):
    rng = np.random.default_rng(seed)
    mb = max(1, max(math.ceil(L / bs) for L in lens))
    nb = len(lens) * mb + 2
    tables = rng.permutation(nb)[:len(lens) * mb].reshape(len(lens), mb).astype(np.int32)
    return W.PagedInputs(q=W.normal_bf16(rng, (len(lens), 16, 128)),
                         k_cache=W.normal_bf16(rng, (nb, bs, 8, 128)),
                         v_cache=W.normal_bf16(rng, (nb, bs, 8, 128)),
                         block_tables=tables, context_lens=np.array(lens, np.int32),
                         block_size=bs, scale=1 / math.sqrt(128), sliding_window=window)


def _both(pk, x, partition_size=0):
    t = to_torch(x, "cuda")
    mcl = x.max_context_len
    ref = pk.paged_decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                          x.scale, sliding_window=x.sliding_window, max_context_len=mcl,
                          partition_size=partition_size)
    out = torch.full_like(t["q"], 7.0)
    got = pk.paged_decode_noalloc(t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                                  t["context_lens"], x.scale, max_context_len=mcl, out=out,
                                  sliding_window=x.sliding_window, partition_size=partition_size)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    g = got.float().cpu().numpy().astype(np.float64)
    err = np.abs(g - oracle.paged_decode(x.q, x.k_cache, x.v_cache, x.block_tables,
                                         x.context_lens, x.scale, x.sliding_window))
    assert np.isfinite(g).all() and err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, \
        (float(err.max()), float(err.mean()))


def test_noalloc_two_calls_second_smaller(gpu_lib):
    pk = gpu_lib
    big = _case(91, [3000, 17, 2500, 4096, 1, 777, 2048, 3999], bs=64)
    small = _case(92, [1500, 300, 5], bs=32)
    assert pk.decode_plan(8, 8, big.max_context_len)[1] > 1          # split: uses the scratch
    assert pk.decode_plan(3, 8, small.max_context_len)[1] > 1
    assert small.num_seqs < big.num_seqs and small.max_context_len < big.max_context_len
    assert pk.decode_workspace_size(3, 16, 8, 128, small.max_context_len) > 0
    _both(pk, big)
    _both(pk, small)


def test_noalloc_window_and_single_partition(gpu_lib):
    pk = gpu_lib
    _both(pk, _case(93, [5000, 300, 260, 1], bs=128, window=256), partition_size=64)  # windowed split
    _both(pk, _case(94, [64, 10, 120], bs=16))                         # one partition, no scratch
    _both(pk, _case(95, [900, 1200], bs=64), partition_size=64)        # many partitions


def test_noalloc_refuses_plans_beyond_the_scratch(gpu_lib):
    pk = gpu_lib
    nseq, mcl = 64, 8192
    assert pk.decode_workspace_size(nseq, 16, 8, 128, mcl, 0, 64) > pk.NOALLOC_SCRATCH_BYTES
    q = torch.zeros(nseq, 16, 128, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(2, 64, 8, 128, dtype=torch.bfloat16, device="cuda")
    tables = torch.zeros(nseq, 128, dtype=torch.int32, device="cuda")
    lens = torch.full((nseq,), mcl, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(pk.PagedKVError, match="WORKSPACE"):
        pk.paged_decode_noalloc(q, kc, kc, tables, lens, 1.0, max_context_len=mcl, out=out,
                                partition_size=64)
