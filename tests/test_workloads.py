"""The seeded generator produces the shapes, structure and value recipe it promises."""
import math

import numpy as np
import pytest
import torch

from paged_kv_cache_286_amd import workloads as W
import oracle


def test_generation_is_deterministic():
    a = W.generate(W.make_plan("tiny_decode"))
    b = W.generate(W.make_plan("tiny_decode"))
    assert np.array_equal(a.q, b.q)
    assert np.array_equal(a.k.blocks, b.k.blocks) and np.array_equal(a.v.blocks, b.v.blocks)
    assert np.array_equal(a.plan.block_tables, b.plan.block_tables)


def test_tiny_decode_structure():
    p = W.make_plan("tiny_decode")
    assert p.context_lens.tolist() == [10, 40, 20, 80]
    assert p.query_lens.tolist() == [1, 1, 1, 1]
    used = np.concatenate([p.block_tables[i, :-(-int(L) // 16)] for i, L in enumerate(p.context_lens)])
    assert len(used) == 1 + 3 + 2 + 5 == len(set(used.tolist()))
    assert used.min() >= 0 and used.max() < 64
    assert W.algorithmic_kv_bytes(p)["unique"] == 150 * 2 * 4 * 64 * 2 == 153600


def test_tails_are_poisoned_and_values_standard_normal():
    wl = W.generate(W.make_plan("decode_7b"))
    p = wl.plan
    i = int(np.argmax(p.context_lens % 16 != 0))
    L = int(p.context_lens[i])
    last = int(p.block_tables[i, (L - 1) // 16])
    blk = wl.k[np.array([last])][0]
    assert np.all(blk[:, L % 16:, :] == W.POISON[W.BF16])
    vals = oracle.decode_bits(wl.k.blocks[:200, :, :8, :], W.BF16).ravel()
    vals = vals[np.isfinite(vals)]
    assert abs(vals.mean()) < 0.01 and abs(vals.std() - 1) < 0.01


def test_decode_7b_shape():
    p = W.make_plan("decode_7b")
    assert p.num_seqs == 64 and p.context_lens.min() >= 128 and p.context_lens.max() <= 4096
    t = p.block_tables[p.block_tables >= 0]
    assert len(t) == len(np.unique(t)) and t.max() < 16384


def test_long_tail_shared_prefix():
    p = W.make_plan("long_tail")
    assert p.num_seqs == 256 and p.context_lens.max() <= 32768
    sh = p.shared_seqs
    assert len(sh) == 32 and p.shared_prefix_blocks == 94
    for i in sh:
        assert np.array_equal(p.block_tables[i, :94], p.block_tables[sh[0], :94])
        assert 1504 + 50 <= p.context_lens[i] <= 1504 + 500
    others = np.setdiff1d(np.arange(256), sh)
    assert abs(p.context_lens[others].mean() - 600) < 150          # geometric, mean 600
    b = W.algorithmic_kv_bytes(p)
    assert b["logical"] - b["unique"] == 31 * 1504 * 16384
    # the pool is a 40 GiB budget for this layer's K and V
    assert p.cfg.num_blocks * W.kv_bytes_per_token(p.cfg) * 16 == 40 * 2 ** 30


def test_mixed_prefill_shape():
    p = W.make_plan("mixed_prefill")
    assert p.num_seqs == 129 and p.query_lens[-1] == 512 and p.context_lens[-1] == 2560
    assert np.all(p.query_lens[:128] == 1) and p.total_q_tokens == 640
    assert p.context_lens[:128].min() >= 256 and p.context_lens[:128].max() <= 4096


def test_fp8_scale_recipe():
    cfg = W.Config("f", "f", 8, 2, 64, 16, 32, W.FP8, W.BF16, 9)
    wl = W.generate(W.custom_plan(cfg, [40, 7, 16], [1, 1, 1], 9))
    # the largest valid magnitude of every (block, head) decodes to +-448 * scale / scale
    for u, blk in enumerate(wl.k.used_ids):
        for h in range(2):
            vals = oracle.decode_bits(wl.k.blocks[u, h], W.FP8)
            finite = vals[np.isfinite(vals)]
            assert np.max(np.abs(finite)) == 448.0
            assert wl.k_scale[blk, h] > 0
    # quantised values track the N(0,1) draws they came from within fp8 resolution
    deq = oracle.dequant_fp8(wl.k.blocks[0, 0], wl.k_scale[wl.k.used_ids[0], 0])
    assert np.nanmax(np.abs(deq)) < 6


def test_appended_rows_are_the_last_positions():
    wl = W.generate(W.make_plan("mixed_prefill"))
    p = wl.plan
    assert len(wl.slot_mapping) == 640
    # the chunk's rows land at positions 2048..2559 of the last sequence
    t = p.block_tables[128]
    exp = np.array([t[pos // 16] * 16 + pos % 16 for pos in range(2048, 2560)])
    assert np.array_equal(wl.slot_mapping[128:], exp)
    assert len(np.unique(wl.slot_mapping)) == 640


def test_pre_append_pool_poisons_only_the_appended_slots():
    wl = W.generate(W.make_plan("tiny_decode"))
    pre = wl.pre_append("k").dense()
    post = wl.k.dense()
    diff = np.any(pre != post, axis=(1, 3))            # [NB][bs]
    assert diff.sum() == 4
    out = oracle.kv_append(pre, wl.k_new, wl.slot_mapping, 16)
    assert np.array_equal(out, post)


def test_kv_pools_share_one_allocation_with_a_gap():
    from paged_kv_cache_286_amd.device import KV_POOL_GAP_BYTES, alloc_kv_pools
    shape = (64, 4, 16, 64)
    for dtype in (torch.bfloat16, torch.uint8):
        k, v = alloc_kv_pools(shape, dtype, "cpu", 7)
        assert k.shape == v.shape == shape and k.is_contiguous() and v.is_contiguous()
        nbytes = k.numel() * k.element_size()
        assert v.data_ptr() - k.data_ptr() == nbytes + KV_POOL_GAP_BYTES
        assert KV_POOL_GAP_BYTES % 4096 == 0 and (KV_POOL_GAP_BYTES // 4096) % 2 == 1
        assert int(k.min()) == int(k.max()) == 7 and int(v.min()) == 7
        k.fill_(1)                      # the pools do not overlap
        assert int(v.max()) == 7
