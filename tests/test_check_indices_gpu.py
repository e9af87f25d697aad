"""Checked mode (pk_check_indices) on the GPU: clean inputs count nothing,
planted violations are counted exactly (host arithmetic gives the expected
counts), and table entries past a sequence's used range are never judged."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


def cuda_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def test_clean_workloads_count_nothing(gpu_lib):
    for x in (W.small_decode(), W.store_decode(), W.prefix_prefill(), W.mixed_batch()):
        t = W.to_torch(x, "cuda")
        kw = dict(block_tables=t["block_tables"])
        if x.cu_seqlens_q is not None:
            kw.update(cu_seqlens_q=t["cu_seqlens_q"], cu_seqlens_k=t["cu_seqlens_k"])
        else:
            kw.update(context_lens=t["context_lens"])
        if x.slot_mapping is not None:
            kw.update(slot_mapping=t["slot_mapping"])
        assert gpu_lib.check_indices(t["k_cache"], **kw) == dict.fromkeys(gpu_lib.CHECK_FIELDS, 0)


def test_planted_violations_are_counted(gpu_lib):
    rng = np.random.default_rng(61)
    nb, bs = 40, 16
    k_cache = torch.zeros(nb, bs, 1, 128, dtype=torch.bfloat16, device="cuda")
    slots = rng.permutation(nb * bs)[:300].astype(np.int64)
    slots[:5] = [-1, -1, nb * bs, -2, 10 ** 6]          # 2 padding, 3 out of range
    slots[5:12] = slots[20]                              # 7 repeats of one slot
    slots[12] = slots[21]                                # 1 more repeat
    lens = np.array([1, 17, 33, 0, 48, 64], np.int32)
    mb = 4
    tables = rng.integers(0, nb, size=(6, mb)).astype(np.int32)
    tables[1, 1] = nb              # in range of L = 17 (blocks 0..1): counted
    tables[1, 2] = -1              # past the used range: not read, not counted
    tables[3, 0] = 99              # L = 0: nothing used
    tables[4, 2] = -5              # L = 48 uses blocks 0..2: counted
    tables[5, 3] = nb + 1          # L = 64 uses all four: counted
    res = gpu_lib.check_indices(k_cache, slot_mapping=cuda_i32(slots), block_tables=cuda_i32(tables),
                                context_lens=cuda_i32(lens), raise_on_error=False)
    valid = slots[(slots >= 0) & (slots < nb * bs)]
    assert res["slots_out_of_range"] == 3
    assert res["repeated_slots"] == len(valid) - len(np.unique(valid)) == 8
    assert res["bad_table_entries"] == 3
    assert res["bad_lengths"] == 0
    with pytest.raises(gpu_lib.PagedKVError, match="PK_ERR_INDEX"):
        gpu_lib.check_indices(k_cache, slot_mapping=cuda_i32(slots))


def test_length_violations(gpu_lib):
    k_cache = torch.zeros(8, 16, 1, 128, dtype=torch.bfloat16, device="cuda")
    tables = cuda_i32(np.zeros((4, 2), np.int32))
    # context lengths: negative, beyond 2 blocks x 16, fine, fine
    res = gpu_lib.check_indices(k_cache, block_tables=tables,
                                context_lens=cuda_i32([-1, 33, 32, 0]), raise_on_error=False)
    assert res["bad_lengths"] == 2 and res["bad_table_entries"] == 0
    # varlen: a decreasing prefix sum, and fewer keys than queries
    cq = cuda_i32([0, 5, 4, 10, 12])
    ck = cuda_i32([0, 10, 20, 25, 40])
    res = gpu_lib.check_indices(k_cache, block_tables=tables, cu_seqlens_q=cq, cu_seqlens_k=ck,
                                raise_on_error=False)
    # seq 1: Lq = -1; seq 2: Lq 6 > Lk 5; seq 3: Lk 15 fine
    assert res["bad_lengths"] == 2
