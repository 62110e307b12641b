"""GPU parity: libpagedkv (through its C ABI) against the float64 CPU oracle.

Small steps are compared element by element over every output.  The
full-size step workloads (the launch configurations the benchmark times) are
compared on every sequence and head the oracle can compute in seconds: all
of them for the 16-bit decode and mixed steps, every sequence at a query head
of every kv head (and every head of the longest sequence) for the fp8
grouped-query step, three heads of every prompt row for the prefill step.
Appends are compared bit for bit over whole pools.
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_286_amd import workloads as W

pytestmark = pytest.mark.gpu

# |gpu - ref| <= atol + rtol * |ref| per element (16-bit KV); fp8 KV: |gpu - ref| <= 5e-2
TOL = {W.F16: (2e-3, 1e-2), W.BF16: (2e-3, 1e-2), W.FP8: (5e-2, 0.0)}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture
def plan():
    """Sets the library's plan override for one test and restores the defaults after it."""
    from paged_kv_cache_286_amd import pagedkv as pk
    yield pk.pkv_set_plan_override
    pk.pkv_set_plan_override()


def _device_step(wl):
    from paged_kv_cache_286_amd.device import DeviceStep
    return DeviceStep(wl)


def _run(wl, label):
    p = wl.plan
    _say(f"[gpu] {label}: seqs={p.num_seqs} rows={p.total_q_tokens} max_ctx={p.max_context_len} "
         f"Hq={p.cfg.num_q_heads} Hkv={p.cfg.num_kv_heads} D={p.cfg.head_dim} kv={p.cfg.kv_dtype}")
    ds = _device_step(wl)
    ds.step()
    torch.cuda.synchronize()
    return ds


def _check(wl, ds, seqs=None, heads=None):
    p = wl.plan
    cfg = p.cfg
    ref = oracle.paged_attention(wl.q, wl.k, wl.v, p.block_tables, p.context_lens, p.query_lens,
                                 wl.scale, cfg.block_size, cfg.kv_dtype, cfg.q_dtype,
                                 wl.k_scale, wl.v_scale, seqs=seqs, heads=heads)
    got = oracle.decode_bits(ds.out_bits(), cfg.q_dtype)
    starts = np.concatenate([[0], np.cumsum(p.query_lens.astype(np.int64))])
    atol, rtol = TOL[cfg.kv_dtype]
    worst_abs = worst_rel = 0.0
    for i, r in ref.items():
        g = got[starts[i]:starts[i + 1]]
        if heads is not None:
            g, r = g[:, heads], r[:, heads]
        err = np.abs(g - r)
        worst_abs = max(worst_abs, float(np.nanmax(err)) if np.isfinite(err).all() else np.inf)
        worst_rel = max(worst_rel, float(np.max(err / np.maximum(np.abs(r), 1e-6))))
        ok = oracle.tolerance_ok(g, r, atol, rtol)
        if not ok.all():
            bad = np.argwhere(~ok)[0]
            raise AssertionError(f"seq {i} (L={p.context_lens[i]}, Q={p.query_lens[i]}) row/head/dim "
                                 f"{tuple(bad)}: gpu {g[tuple(bad)]} ref {r[tuple(bad)]}; "
                                 f"{(~ok).sum()} of {ok.size} elements out of tolerance")
    _say(f"    max|err| {worst_abs:.3g}  max rel {worst_rel:.3g}")
    return worst_abs


def _small(Hq, Hkv, D, kv, qd, lens, qlens=None, seed=0, extra_blocks=17):
    nb = sum(-(-int(L) // 16) for L in lens) + extra_blocks
    cfg = W.Config("small", "small", Hq, Hkv, D, 16, nb, kv, qd, seed)
    return W.generate(W.custom_plan(cfg, lens, qlens if qlens is not None else [1] * len(lens), seed))


_rng = np.random.default_rng(2024)
SMALL = {
    "mha_bf16_d128_ragged": dict(Hq=8, Hkv=8, D=128, kv=W.BF16, qd=W.BF16,
                                 lens=[1, 15, 16, 17, 100, 511, 512, 513, 1024, 1500, 2049]),
    "gqa4_bf16_d128": dict(Hq=16, Hkv=4, D=128, kv=W.BF16, qd=W.BF16,
                           lens=_rng.integers(1, 3000, 10).tolist()),
    "gqa16_bf16_d128": dict(Hq=32, Hkv=2, D=128, kv=W.BF16, qd=W.BF16, lens=[5, 700, 1601]),
    "gqa6_bf16_d64": dict(Hq=12, Hkv=2, D=64, kv=W.BF16, qd=W.BF16, lens=[33, 400, 1000]),
    "mha_f16_d64": dict(Hq=4, Hkv=4, D=64, kv=W.F16, qd=W.F16, lens=[10, 40, 20, 80, 1, 999]),
    "gqa2_f16_d128": dict(Hq=8, Hkv=4, D=128, kv=W.F16, qd=W.F16, lens=[64, 65, 2000]),
    "fp8_gqa8_bf16q_d128": dict(Hq=16, Hkv=2, D=128, kv=W.FP8, qd=W.BF16,
                                lens=_rng.integers(1, 5000, 8).tolist()),
    "fp8_mha_f16q_d64": dict(Hq=4, Hkv=4, D=64, kv=W.FP8, qd=W.F16, lens=[3, 16, 17, 300, 1200]),
    "fp8_gqa8_f16q_d128": dict(Hq=16, Hkv=2, D=128, kv=W.FP8, qd=W.F16, lens=[1, 40, 700, 2600]),
    "fp8_gqa4_bf16q_d64": dict(Hq=8, Hkv=2, D=64, kv=W.FP8, qd=W.BF16, lens=[1, 31, 777]),
    "chunk_bf16_d128": dict(Hq=4, Hkv=4, D=128, kv=W.BF16, qd=W.BF16, lens=[40, 300, 700, 33],
                            qlens=[1, 37, 129, 33]),
    "chunk_gqa4_fp8_d128": dict(Hq=8, Hkv=2, D=128, kv=W.FP8, qd=W.BF16, lens=[90, 1000, 20],
                                qlens=[90, 64, 1]),
    "chunk_f16_d64": dict(Hq=4, Hkv=2, D=64, kv=W.F16, qd=W.F16, lens=[17, 600], qlens=[16, 200]),
    # single-row sequences beside chunks: decode rows as two-head VALU workgroups in the step kernel
    "chunk_gqa2_bf16_d128_decodes": dict(Hq=8, Hkv=4, D=128, kv=W.BF16, qd=W.BF16,
                                         lens=[50, 700, 1300, 90, 2500, 16],
                                         qlens=[1, 1, 300, 1, 1, 16]),
    # fp8 prefill items at head_dim 64 (one 16-byte copy per thread and stage)
    "chunk_fp8_mha_f16q_d64": dict(Hq=4, Hkv=4, D=64, kv=W.FP8, qd=W.F16, lens=[200, 900, 35, 64],
                                   qlens=[200, 1, 35, 3]),
    # several query rows per sequence, as a speculative-decoding step verifies
    "specdec_mha_bf16_d128": dict(Hq=8, Hkv=8, D=128, kv=W.BF16, qd=W.BF16,
                                  lens=_rng.integers(50, 3000, 10).tolist(),
                                  qlens=[1, 2, 3, 4, 5, 6, 2, 3, 8, 1]),
    "specdec_gqa4_fp8_d128": dict(Hq=8, Hkv=2, D=128, kv=W.FP8, qd=W.BF16,
                                  lens=[40, 900, 1700, 300, 64], qlens=[4, 3, 2, 9, 1]),
    "specdec_gqa8_bf16_d64": dict(Hq=16, Hkv=2, D=64, kv=W.BF16, qd=W.BF16,
                                  lens=[33, 500, 2100], qlens=[2, 3, 1]),
    # one kv head for 32 query heads: a decode row fills two 16-column tiles
    "mqa32_bf16_d128": dict(Hq=32, Hkv=1, D=128, kv=W.BF16, qd=W.BF16, lens=[1, 17, 900, 2600]),
    "mqa32_fp8_d128": dict(Hq=32, Hkv=1, D=128, kv=W.FP8, qd=W.BF16, lens=[3, 1000, 4100]),
    # prefill rows at 16 query heads per kv head (a chunk entry covers 8 rows x 16 heads)
    "chunk_gqa16_bf16_d64": dict(Hq=32, Hkv=2, D=64, kv=W.BF16, qd=W.BF16, lens=[70, 600, 9],
                                 qlens=[70, 33, 1]),
    "chunk_mqa8_f16_d128": dict(Hq=8, Hkv=1, D=128, kv=W.F16, qd=W.F16, lens=[300, 45, 1000],
                                qlens=[129, 45, 2]),
    # a 16-column tile holds half of one row's 32 query heads
    "chunk_mqa32_bf16_d128": dict(Hq=32, Hkv=1, D=128, kv=W.BF16, qd=W.BF16, lens=[150, 600, 20],
                                  qlens=[150, 7, 1]),
}


def test_tiny_decode_all_outputs():
    wl = W.generate(W.make_plan("tiny_decode"))
    ds = _run(wl, "tiny_decode")
    _check(wl, ds)


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_steps_all_outputs(name):
    wl = _small(seed=sorted(SMALL).index(name) + 100, **SMALL[name])
    ds = _run(wl, name)
    _check(wl, ds)


def _random_case(seed):
    """A seeded random small step: head layout, dtypes, lengths and query rows
    (decodes, speculative-verify rows, prefill chunks, whole prompts) drawn
    over what the library accepts."""
    rng = np.random.default_rng(seed)
    D = int(rng.choice([64, 128]))
    kv = [W.BF16, W.F16, W.FP8][seed % 3]
    qd = (W.BF16 if rng.integers(2) else W.F16) if kv == W.FP8 else kv
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 3, 4, 6, 8, 16]))
    S = int(rng.integers(1, 10))
    lens, qlens = [], []
    for _ in range(S):
        L = int(rng.choice([rng.integers(1, 64), rng.integers(64, 1200), rng.integers(1200, 5000)]))
        kind = rng.integers(6)
        if kind <= 2:
            Q = 1
        elif kind == 3:
            Q = int(rng.integers(2, 9))           # verify rows
        elif kind == 4:
            Q = int(rng.integers(9, 200))         # a prefill chunk
        else:
            Q = L if L <= 200 else 1              # a whole short prompt
        lens.append(L)
        qlens.append(min(Q, L))
    return dict(Hq=Hkv * G, Hkv=Hkv, D=D, kv=kv, qd=qd, lens=lens, qlens=qlens)


@pytest.mark.parametrize("seed", range(1000, 1024))
def test_random_steps_all_outputs(seed):
    case = _random_case(seed)
    wl = _small(seed=seed, **case)
    _check(wl, _run(wl, f"random step seed={seed} G={case['Hq'] // case['Hkv']} qlens={case['qlens']}"))


@pytest.mark.parametrize("part_tokens", [16, 64, 256, 4096])
def test_partition_sizes(part_tokens, plan):
    plan(part_tokens=part_tokens)
    wl = _small(seed=7, **SMALL["mha_bf16_d128_ragged"])
    ds = _run(wl, f"mha_bf16 part_tokens={part_tokens}")
    _check(wl, ds)
    wl8 = _small(seed=8, **SMALL["fp8_gqa8_bf16q_d128"])
    _check(wl8, _run(wl8, f"fp8_gqa8 part_tokens={part_tokens}"))


@pytest.mark.parametrize("path", ["0", "1"])
@pytest.mark.parametrize("name", ["mha_bf16_d128_ragged", "gqa4_bf16_d128", "fp8_gqa8_bf16q_d128",
                                  "mha_f16_d64", "fp8_mha_f16q_d64", "gqa16_bf16_d128"])
def test_decode_paths_forced(name, path, plan):
    # "0": the VALU decode kernel, "1": the MFMA tile kernel, for the same inputs
    plan(decode_on_mfma=int(path))
    wl = _small(seed=sorted(SMALL).index(name) + 300, **SMALL[name])
    _check(wl, _run(wl, f"{name} decode_mfma={path}"))


@pytest.mark.parametrize("small_q", ["1", "2"])
def test_multi_row_routing_forced(small_q, plan):
    # sequences with <= small_q rows run as decode items, longer ones as chunk entries
    plan(small_q=int(small_q))
    for name in ("specdec_mha_bf16_d128", "specdec_gqa4_fp8_d128", "chunk_bf16_d128"):
        wl = _small(seed=sorted(SMALL).index(name) + 500, **SMALL[name])
        _check(wl, _run(wl, f"{name} small_q={small_q}"))


@pytest.mark.parametrize("kv", [W.BF16, W.FP8])
def test_mixed_step_decode_verify_and_prefill_rows(kv):
    # one step with single decode rows, short verify rows, a whole 300-token
    # prompt and a 129-row chunk, at lengths around block and partition edges
    lens = [1, 17, 300, 2000, 90, 513, 4000, 64]
    qlens = [1, 1, 300, 1, 5, 1, 129, 1]
    cfg = W.Config("mixed", "mixed", 8, 8 if kv == W.BF16 else 2, 128, 16, 900, kv, W.BF16, 31)
    wl = W.generate(W.custom_plan(cfg, lens, qlens, 31))
    _check(wl, _run(wl, f"mixed rows kv={kv}"))


@pytest.mark.parametrize("chunk_pt", ["0", "64"])
def test_uniform_prompt_steps(chunk_pt, plan):
    # every sequence a whole prompt (or one chunk) of the same length: the merge
    # launch is skipped only when no chunk row is split ("0": the library's own
    # partition; "64": forced splits, so partitions must be merged)
    plan(chunk_part_tokens=int(chunk_pt))
    for lens, qlens in (([700, 700], [700, 700]), ([2560], [512]), ([300, 300, 300], [300, 300, 300])):
        cfg = W.Config("uni", "uni", 8, 8, 128, 16, 400, W.BF16, W.BF16, 17)
        wl = W.generate(W.custom_plan(cfg, lens, qlens, 17))
        _check(wl, _run(wl, f"uniform prompts {lens}/{qlens} chunk_pt={chunk_pt}"))


@pytest.mark.parametrize("chunk_pt", [64, 256, 1024])
def test_chunk_partition_sizes(chunk_pt, plan):
    plan(chunk_part_tokens=chunk_pt)
    for name in ("chunk_bf16_d128", "chunk_gqa4_fp8_d128", "chunk_f16_d64"):
        wl = _small(seed=sorted(SMALL).index(name) + 400, **SMALL[name])
        _check(wl, _run(wl, f"{name} chunk_part_tokens={chunk_pt}"))


def test_single_token_and_full_table_edges():
    # L = 1 everywhere, and L equal to the whole table (max_blocks * 16)
    wl = _small(Hq=4, Hkv=4, D=128, kv=W.BF16, qd=W.BF16, lens=[1, 1, 1], seed=3)
    _check(wl, _run(wl, "all L=1"))
    cfg = W.Config("edge", "edge", 8, 8, 128, 16, 300, W.BF16, W.BF16, 4)
    wl = W.generate(W.custom_plan(cfg, [4096, 16], [1, 1], 4, max_blocks_per_seq=256))
    _check(wl, _run(wl, "L = max_blocks * 16"))


# ----------------------------------------------------------------------------
# invariances (bitwise on the GPU: the kernel's arithmetic order does not depend on them)
# ----------------------------------------------------------------------------
def test_gpu_physical_relabelling_bitwise():
    wl = _small(seed=11, **SMALL["gqa4_bf16_d128"])
    a = _run(wl, "relabel base").out_bits()
    p = wl.plan
    pi = np.random.default_rng(5).permutation(p.cfg.num_blocks)
    new_ids = pi[wl.k.used_ids]
    order = np.argsort(new_ids)
    k2 = W.BlockStore(new_ids[order], wl.k.blocks[order], p.cfg.num_blocks, wl.k.poison)
    v2 = W.BlockStore(new_ids[order], wl.v.blocks[order], p.cfg.num_blocks, wl.v.poison)
    t2 = np.where(p.block_tables >= 0, pi[np.maximum(p.block_tables, 0)], -1).astype(np.int32)
    p2 = W.Plan(p.cfg, p.context_lens, p.query_lens, t2, p.max_blocks_per_seq)
    wl2 = W.Workload(p2, wl.q, k2, v2, None, None, (pi[wl.append_block] * 16 + wl.append_offset).astype(np.int32),
                     wl.k_new, wl.v_new, wl.scale, pi[wl.append_block], wl.append_offset)
    b = _run(wl2, "relabel moved").out_bits()
    assert np.array_equal(a, b)


def test_gpu_batch_order_bitwise():
    wl = _small(seed=12, **SMALL["mha_bf16_d128_ragged"])
    a = _run(wl, "order base").out_bits()
    p = wl.plan
    perm = np.random.default_rng(6).permutation(p.num_seqs)
    p2 = W.Plan(p.cfg, p.context_lens[perm], p.query_lens[perm], p.block_tables[perm],
                p.max_blocks_per_seq)
    wl2 = W.Workload(p2, wl.q[perm], wl.k, wl.v, None, None, wl.slot_mapping[perm], wl.k_new[perm],
                     wl.v_new[perm], wl.scale, wl.append_block[perm], wl.append_offset[perm])
    b = _run(wl2, "order permuted").out_bits()
    assert np.array_equal(a[perm], b)


def test_gpu_shared_prefix_equals_copies_bitwise():
    cfg = W.Config("sh", "sh", 8, 8, 128, 16, 400, W.BF16, W.BF16, 13)
    wl = W.generate(W.custom_plan(cfg, [200, 300, 90, 177], [1, 1, 1, 1], 13,
                                  shared_prefix_blocks=5, shared_seqs=(0, 1, 3)))
    ds = _run(wl, "shared prefix")
    _check(wl, ds)
    a = ds.out_bits()
    p = wl.plan
    t = p.block_tables.copy()
    free = sorted(set(range(cfg.num_blocks)) - set(t[t >= 0].tolist()))
    ids, kb, vb = list(wl.k.used_ids), list(wl.k.blocks), list(wl.v.blocks)
    for j in range(5):
        src = int(t[1, j])
        new = free[j]
        u = int(np.searchsorted(wl.k.used_ids, src))
        ids.append(new)
        kb.append(wl.k.blocks[u].copy())
        vb.append(wl.v.blocks[u].copy())
        t[1, j] = new
    order = np.argsort(ids)
    k2 = W.BlockStore(np.array(ids)[order], np.stack(kb)[order], cfg.num_blocks, wl.k.poison)
    v2 = W.BlockStore(np.array(ids)[order], np.stack(vb)[order], cfg.num_blocks, wl.v.poison)
    p2 = W.Plan(cfg, p.context_lens, p.query_lens, t, p.max_blocks_per_seq)
    wl2 = W.Workload(p2, wl.q, k2, v2, None, None, wl.slot_mapping, wl.k_new, wl.v_new, wl.scale,
                     wl.append_block, wl.append_offset)
    assert t[1, 0] != t[0, 0]
    b = _run(wl2, "copied prefix").out_bits()
    assert np.array_equal(a, b)


@pytest.mark.parametrize("case", ["mha_bf16_valu", "gqa8_fp8_mfma", "mixed_step"])
def test_gpu_shared_hint_only_changes_the_load_policy(case):
    # the shared_blocks hint picks cached or streaming loads, and whether it is
    # passed at all picks the order the decode launch deals the split
    # partitions in; whatever it says (right, absent, negative, past the
    # table) the output bits stay the same
    Hq, Hkv, kv, qd = {"mha_bf16_valu": (8, 8, W.BF16, W.BF16),
                       "gqa8_fp8_mfma": (16, 2, W.FP8, W.BF16),
                       "mixed_step": (8, 8, W.BF16, W.BF16)}[case]
    lens = [1500, 2600, 700, 40, 2100]
    qlens = [1, 1, 1, 1, 1] if case != "mixed_step" else [1, 1, 300, 1, 17]
    cfg = W.Config("hint", "hint", Hq, Hkv, 128, 16, 800, kv, qd, 21)
    wl = W.generate(W.custom_plan(cfg, lens, qlens, 21, shared_prefix_blocks=40,
                                  shared_seqs=(0, 1, 4)))
    ds = _run(wl, f"shared hint {case}")
    _check(wl, ds)
    assert ds.shared_blocks is not None
    assert ds.shared_blocks.cpu().tolist() == [40, 40, 0, 0, 40]
    # (the step may have taken its append into the attention launches, which
    # attends to the new rows in another order: compare attention calls only)
    ds.out.zero_()
    ds.attend()
    torch.cuda.synchronize()
    want = ds.out_bits()
    S = len(lens)
    dev = ds.shared_blocks.device
    for hint in (None, [0] * S, [-5, 10**6, 3, 2**31 - 1, 17], [200] * S):
        ds.shared_blocks = None if hint is None else torch.tensor(hint, dtype=torch.int32, device=dev)
        ds.out.zero_()
        ds.attend()
        torch.cuda.synchronize()
        assert np.array_equal(ds.out_bits(), want), f"hint {hint}"


# ----------------------------------------------------------------------------
# the append and the step in one call
# ----------------------------------------------------------------------------
FUSE_CASES = {
    # name: (Hq, Hkv, D, kv, q dtype, context lens, query lens, append kernel launches)
    "tiny_f16_d64": (4, 4, 64, W.F16, W.F16, [10, 40, 20, 80], [1, 1, 1, 1], 0),
    "mha_bf16_ragged_split": (8, 8, 128, W.BF16, W.BF16, [1, 16, 17, 1024, 1025, 3001, 4096, 2047],
                              [1] * 8, 0),
    "g2_bf16": (16, 8, 128, W.BF16, W.BF16, [33, 700, 2049, 1], [1] * 4, 0),
    "mha_bf16_large": (8, 8, 128, W.BF16, W.BF16, [4096, 17, 2500, 1] * 4, [1] * 16, 0),
    # steps with prefill chunks store the rows from their prologue launch
    "mixed_step": (8, 8, 128, W.BF16, W.BF16, [50, 700, 1300, 90], [1, 1, 300, 1], 0),
    "mixed_f16_d64": (4, 2, 64, W.F16, W.F16, [37, 513, 16, 260], [1, 40, 16, 1], 0),
    # split decode steps on the MFMA kernel: the merge launch adds the new key
    # (a length-1 sequence has nothing else) and stores the rows
    "gqa4_bf16_mfma": (16, 4, 128, W.BF16, W.BF16, [33, 700, 2049, 1], [1] * 4, 0),
    "fp8_gqa8": (16, 2, 128, W.FP8, W.BF16, [3000, 200, 2047, 1, 17], [1] * 5, 0),
    "fp8_gqa8_f16q_d64": (16, 2, 64, W.FP8, W.F16, [900, 1, 4000, 65], [1] * 4, 0),
    "gqa4_f16_d64": (8, 2, 64, W.F16, W.F16, [100, 1, 2500, 777, 16, 17], [1] * 6, 0),
    # unsplit MFMA decode steps and fp8 steps with prefill chunks enqueue the append kernel
    "gqa4_unsplit": (16, 4, 128, W.BF16, W.BF16, [10, 40, 100], [1] * 3, 1),
    "fp8_mixed": (16, 2, 128, W.FP8, W.BF16, [50, 700, 1300], [1, 200, 1], 1),
}
# cases whose attention reads every row from the pool: the output equals the
# separate calls' bit for bit
FUSE_EXACT = {"mixed_step", "mixed_f16_d64", "gqa4_unsplit", "fp8_mixed"}


@pytest.mark.parametrize("case", sorted(FUSE_CASES))
def test_append_and_step_in_one_call(case):
    # paged_append_attn_step: decode steps on the VALU kernel take the append
    # into their launches (no append kernel runs; the appended row is attended
    # after the pool's blocks, so the last bits may differ; the merge launch
    # stores the rows of split steps, the decode launch those of the others);
    # split decode steps on the MFMA kernel leave the new key to the merge
    # launch, which also stores the rows; 16-bit steps with prefill chunks
    # store the rows from their prologue launch; every other step enqueues the
    # append kernel first.  Where the
    # attention reads every row from the pool the output is the two calls',
    # bit for bit.  Either way both whole pools equal paged_kv_append's and
    # the output passes the oracle.
    from paged_kv_cache_286_amd import pagedkv as pk
    Hq, Hkv, D, kv, qd, lens, qlens, appends = FUSE_CASES[case]
    nb = sum(-(-L // 16) for L in lens) + 9
    wl = W.generate(W.custom_plan(W.Config("fuse", "fuse", Hq, Hkv, D, 16, nb, kv, qd, 61),
                                  lens, qlens, 61))
    _say(f"[gpu] append and step in one call: {case}")
    ds = _device_step(wl)
    assert ds.fusable
    ds.step_separate()
    torch.cuda.synchronize()
    want = (ds.out_bits().copy(), ds.k_pool.cpu().numpy(), ds.v_pool.cpu().numpy())
    ds.poison_appended_slots()
    ds.out.fill_(0x1234)
    pk.pkv_timing_enable(64)
    try:
        ds.step()
        torch.cuda.synchronize()
        pk.pkv_timing_collect()
        launched = pk.pkv_timing_get(pk.PKV_KERNEL_APPEND)[1]
    finally:
        pk.pkv_timing_disable()
    assert launched == appends
    if case in FUSE_EXACT:
        assert np.array_equal(ds.out_bits(), want[0])
    else:
        qd_ = wl.plan.cfg.q_dtype
        assert oracle.tolerance_ok(oracle.decode_bits(ds.out_bits(), qd_),
                                   oracle.decode_bits(want[0], qd_), 2e-3, 1e-2).all()
    assert np.array_equal(ds.k_pool.cpu().numpy(), want[1])
    assert np.array_equal(ds.v_pool.cpu().numpy(), want[2])
    _check(wl, ds)


# ----------------------------------------------------------------------------
# the append, bit for bit over whole pools
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("kv", [W.BF16, W.F16, W.FP8])
def test_append_bit_exact_whole_pool(kv):
    from paged_kv_cache_286_amd import pagedkv as pk
    rng = np.random.default_rng(31)
    NB, H, bs, D = 40, 4, 16, 128
    store = W.STORAGE[kv]
    hi = 256 if store == np.uint8 else 65536
    pool_k = rng.integers(0, hi, size=(NB, H, bs, D)).astype(store)
    pool_v = rng.integers(0, hi, size=(NB, H, bs, D)).astype(store)
    T = 300
    slots = rng.choice(NB * bs, size=T, replace=False).astype(np.int32)
    slots[rng.random(T) < 0.1] = -1                      # skipped rows
    slots[:3] = [NB * bs, NB * bs + 5, -7]               # out of the pool: skipped too
    k_new = rng.integers(0, hi, size=(T, H, D)).astype(store)
    v_new = rng.integers(0, hi, size=(T, H, D)).astype(store)
    dev = torch.device("cuda:0")
    tt = (lambda a: torch.from_numpy(a.view(np.int16)).to(dev)) if store == np.uint16 else \
         (lambda a: torch.from_numpy(a).to(dev))
    gk, gv, nk, nv = tt(pool_k), tt(pool_v), tt(k_new), tt(v_new)
    gs = torch.from_numpy(slots).to(dev)
    _say(f"[gpu] append {kv}: {T} rows into {NB} blocks")
    pk.paged_kv_append(pk.make_pool(NB, bs, H, D, kv), gk, gv, nk, nv, pk.DTYPE_CODES[kv], gs, T,
                       torch.cuda.current_stream())
    torch.cuda.synchronize()
    valid = slots.astype(np.int64)
    valid = np.where(valid >= NB * bs, -1, valid)
    ref_k = oracle.kv_append(pool_k, k_new, valid, bs)
    ref_v = oracle.kv_append(pool_v, v_new, valid, bs)
    got_k = gk.cpu().numpy().view(store)
    got_v = gv.cpu().numpy().view(store)
    assert np.array_equal(got_k, ref_k)
    assert np.array_equal(got_v, ref_v)


def test_append_tiny_decode_matches_oracle_whole_pool():
    wl = W.generate(W.make_plan("tiny_decode"))
    ds = _device_step(wl)
    _say("[gpu] tiny_decode append")
    ds.append()
    torch.cuda.synchronize()
    ref = oracle.kv_append(wl.pre_append("k").dense(), wl.k_new, wl.slot_mapping, 16)
    assert np.array_equal(ds.k_pool.cpu().numpy().view(np.uint16), ref)
    ref = oracle.kv_append(wl.pre_append("v").dense(), wl.v_new, wl.slot_mapping, 16)
    assert np.array_equal(ds.v_pool.cpu().numpy().view(np.uint16), ref)


# ----------------------------------------------------------------------------
# full-size step workloads, sampled
# ----------------------------------------------------------------------------
def _sample_seqs(p, n=6, seed=0):
    rng = np.random.default_rng(seed)
    lens = p.context_lens
    pick = {int(np.argmax(lens)), int(np.argmin(lens)), int(np.argmax(p.query_lens))}
    if p.shared_seqs is not None:
        pick.update(int(x) for x in p.shared_seqs[:2])
    while len(pick) < min(n + 3, p.num_seqs):
        pick.add(int(rng.integers(0, p.num_seqs)))
    return sorted(pick)


def _check_appended(wl, ds, n=64):
    """The appended slots hold the new rows bit for bit; some untouched blocks still hold poison."""
    rows = np.arange(min(n, len(wl.slot_mapping)))
    blk = torch.from_numpy(wl.append_block[rows]).cuda()
    off = torch.from_numpy(wl.append_offset[rows]).cuda()
    got = ds.k_pool[blk, :, off, :].cpu().numpy()
    assert np.array_equal(got.view(W.STORAGE[wl.cfg.kv_dtype]), wl.k_new[rows])
    got = ds.v_pool[blk, :, off, :].cpu().numpy()
    assert np.array_equal(got.view(W.STORAGE[wl.cfg.kv_dtype]), wl.v_new[rows])
    unused = np.setdiff1d(np.arange(wl.cfg.num_blocks), wl.k.used_ids)[:: max(1, wl.cfg.num_blocks // 97)]
    if len(unused):
        u = ds.k_pool[torch.from_numpy(unused).cuda()].cpu().numpy().view(W.STORAGE[wl.cfg.kv_dtype])
        assert np.all(u == wl.k.poison)


@pytest.mark.parametrize("name", ["decode_7b", "long_tail", "mixed_prefill", "fp8_gqa_long",
                                  "prefill_chunks", "gqa_decode"])
def test_full_size_workload_sampled(name):
    _say(f"[gpu] generating {name}")
    wl = W.generate(W.make_plan(name))
    ds = _run(wl, name)
    _check_appended(wl, ds)
    p = wl.plan
    seqs = list(range(p.num_seqs))          # every sequence of the step
    heads = None
    if name == "fp8_gqa_long":
        # every sequence at one query head in each of the 8 kv heads' groups
        # (q head h reads kv head h // 8), then all 64 heads of the longest one
        heads = [0, 9, 18, 27, 36, 45, 54, 63]
        assert sorted({h // (p.cfg.num_q_heads // p.cfg.num_kv_heads) for h in heads}) == \
            list(range(p.cfg.num_kv_heads))
        _check(wl, ds, seqs=[int(np.argmax(p.context_lens))])
    if name == "prefill_chunks":            # every row of all four prompts, three heads
        heads = [0, 13, 31]
    _check(wl, ds, seqs=seqs, heads=heads)
    # every output of the step is finite
    out = oracle.decode_bits(ds.out_bits(), wl.cfg.q_dtype)
    assert np.isfinite(out).all()


@pytest.mark.parametrize("new_dtype", [W.BF16, W.F16])
def test_append_quant_bit_exact_whole_pool(new_dtype):
    from paged_kv_cache_286_amd import pagedkv as pk
    rng = np.random.default_rng(41)
    NB, H, bs, D = 24, 4, 16, 128
    pool_k = rng.integers(0, 0x7E, size=(NB, H, bs, D)).astype(np.uint8)
    pool_v = rng.integers(0, 0x7E, size=(NB, H, bs, D)).astype(np.uint8)
    ks = rng.uniform(0.01, 2.0, size=(NB, H)).astype(np.float32)
    vs = rng.uniform(0.01, 2.0, size=(NB, H)).astype(np.float32)
    T = 150
    fixed = np.array([0, 16, 32, 48, 17, 33])          # new blocks 0..3 and rows after them
    rest = rng.choice(np.setdiff1d(np.arange(NB * bs), fixed), size=T - len(fixed), replace=False)
    slots = np.concatenate([fixed, rest]).astype(np.int32)   # distinct, as the append requires
    slots[rng.random(T) < 0.05] = -1
    assert len(np.unique(slots[slots >= 0])) == (slots >= 0).sum()
    mags = np.exp(rng.uniform(-12, 9, size=(T, H, 1)))
    x = (rng.standard_normal((T, H, D)) * mags).astype(np.float32)
    x[0, 0, :4] = [1e6, -1e6, 0.0, -0.0]
    bits = W.round_to_bits(x, new_dtype)
    kbits, vbits = bits, W.round_to_bits(-x * 0.5, new_dtype)
    init_k = rng.uniform(0.05, 1.0, size=H).astype(np.float32)
    init_v = rng.uniform(0.05, 1.0, size=H).astype(np.float32)
    dev = torch.device("cuda:0")
    g = lambda a: torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)
    gk, gv, gks, gvs = g(pool_k), g(pool_v), g(ks), g(vs)
    _say(f"[gpu] append_quant {new_dtype}: {T} rows")
    pk.paged_kv_append_quant(pk.make_pool(NB, bs, H, D, W.FP8), gk, gv, gks, gvs, g(kbits), g(vbits),
                             pk.DTYPE_CODES[new_dtype], g(init_k), g(init_v), g(slots), T,
                             torch.cuda.current_stream())
    torch.cuda.synchronize()
    rk, rks = oracle.kv_append_quant(pool_k, ks, kbits, new_dtype, slots, bs, init_k)
    rv, rvs = oracle.kv_append_quant(pool_v, vs, vbits, new_dtype, slots, bs, init_v)
    assert np.array_equal(gks.cpu().numpy(), rks) and np.array_equal(gvs.cpu().numpy(), rvs)
    gotk, gotv = gk.cpu().numpy(), gv.cpu().numpy()
    bad = np.argwhere(gotk != rk)
    assert len(bad) == 0, f"{len(bad)} K bytes differ, first at {bad[0]}: {gotk[tuple(bad[0])]:#x} vs {rk[tuple(bad[0])]:#x}"
    assert np.array_equal(gotv, rv)
    # without new-block scales every row uses the stored scale
    gk2 = g(pool_k)
    pk.paged_kv_append_quant(pk.make_pool(NB, bs, H, D, W.FP8), gk2, g(pool_v), g(ks), g(vs),
                             g(kbits), g(vbits), pk.DTYPE_CODES[new_dtype], None, None, g(slots), T,
                             torch.cuda.current_stream())
    torch.cuda.synchronize()
    rk2, _ = oracle.kv_append_quant(pool_k, ks, kbits, new_dtype, slots, bs, None)
    assert np.array_equal(gk2.cpu().numpy(), rk2)


def _guarded_step(wl, label, one_call):
    # the step writes only its output rows and the first paged_attn_workspace_bytes
    # bytes of the workspace: guard bytes after both stay as they were (with
    # the append and the attention as two calls, or as paged_append_attn_step)
    ds = _device_step(wl)
    guard = 1 << 16
    n = ds.ws_bytes
    ws = torch.full((n + guard,), 0xAB, dtype=torch.uint8, device="cuda:0")
    ds.workspace = ws[:n] if n else None
    out_full = torch.full((ds.out.shape[0] + 4,) + tuple(ds.out.shape[1:]), 0x5A5A,
                          dtype=ds.out.dtype, device="cuda:0")
    ds.out = out_full[:ds.out.shape[0]]
    _say(f"[gpu] guard bytes {label} one_call={one_call}: workspace {n} B, {ds.out.shape[0]} rows")
    if one_call:
        assert ds.fusable
        ds.bind_step(torch.cuda.current_stream())()
    else:
        ds.append()
        ds.attend()
    torch.cuda.synchronize()
    assert bool((ws[n:] == 0xAB).all()), "a write past the workspace"
    assert bool((out_full[ds.out.shape[0]:] == 0x5A5A).all()), "a write past the output rows"
    _check(wl, ds)


@pytest.mark.parametrize("one_call", [False, True])
@pytest.mark.parametrize("seed", [1003, 1007, 1013, 1014, 1020])
def test_no_writes_outside_workspace_and_output(seed, one_call):
    _guarded_step(_small(seed=seed, **_random_case(seed)), f"seed={seed}", one_call)


@pytest.mark.parametrize("name", ["mha_bf16_d128_ragged", "gqa4_bf16_d128", "fp8_gqa8_bf16q_d128"])
def test_decode_steps_in_one_call_write_nothing_outside(name):
    # decode-only steps whose append goes into the attention launches (the
    # VALU decode, the MFMA decode of grouped-query and fp8 KV)
    _guarded_step(_small(seed=sorted(SMALL).index(name) + 900, **SMALL[name]), name, True)


@pytest.mark.parametrize("name", ["gqa_decode", "decode_7b", "fp8_gqa_long"])
def test_repeated_steps_bit_identical(name):
    # the same step run again gives the same bits: every reduction has a fixed
    # order (the decode items' K regrouping through LDS included), and the
    # merge launch combines a split row's partitions in partition order
    wl = W.generate(W.make_plan(name))
    ds = _run(wl, f"{name} repeated")
    first = ds.out.clone()
    for r in range(4):
        ds.out.fill_(0)
        ds.step()
        torch.cuda.synchronize()
        assert torch.equal(ds.out, first), f"run {r + 2} differs from the first"


def test_more_rows_than_a_grid_y_dimension_holds(plan):
    # Rows and sequences sit in one-dimensional grids: 70,000 decode sequences
    # (16-token partitions forced, so the merge kernel runs over all of them)
    # and one 66,000-row prompt, both past 65,535.
    rng = np.random.default_rng(5)
    lens = rng.integers(1, 49, 70000).tolist()
    wl = _small(Hq=1, Hkv=1, D=64, kv=W.F16, qd=W.F16, lens=lens, seed=81, extra_blocks=9)
    plan(part_tokens=16)
    ds = _run(wl, "70,000 decode sequences, 16-token partitions")
    p = wl.plan
    assert p.num_seqs > 65535
    seqs = sorted({0, 1, 65534, 65535, 65536, 69999} | set(rng.integers(0, 70000, 40).tolist()))
    _check(wl, ds, seqs=seqs)
    out = oracle.decode_bits(ds.out_bits(), W.F16)
    assert np.isfinite(out).all()
    plan()
    cfg = W.Config("rows", "rows", 1, 1, 64, 16, 66000 // 16 + 9, W.BF16, W.BF16, 82)
    wl = W.generate(W.custom_plan(cfg, [66000], [66000], 82))
    ds = _run(wl, "one 66,000-row prompt")
    got = oracle.decode_bits(ds.out_bits(), W.BF16)
    assert np.isfinite(got).all()
    # row r of the prompt sees keys 0..r: the oracle's decode over the first r + 1 tokens
    rows = sorted({0, 15, 16, 4095, 4096, 65534, 65535, 65536, 65999} |
                  set(rng.integers(0, 66000, 24).tolist()))
    t = wl.plan.block_tables
    for r in rows:
        ref = oracle.paged_attention(wl.q[r:r + 1], wl.k, wl.v, t, np.array([r + 1]), np.array([1]),
                                     wl.scale, 16, W.BF16, W.BF16)[0]
        ok = oracle.tolerance_ok(got[r:r + 1], ref, *TOL[W.BF16])
        assert ok.all(), f"row {r}: {(~ok).sum()} elements out of tolerance"


@pytest.mark.parametrize("qd", [W.BF16, W.F16])
def test_fp8_scores_with_query_dims_over_five_decades(qd):
    # fp8 scores at head_dim 128 run on the fp8 MFMA with each query column
    # scaled by a power of two and split into two fp8 parts; query dims whose
    # magnitudes span 1e-3 .. 1e2 within one column (and columns of very
    # different sizes) still match the oracle, in decode and prefill rows
    rng = np.random.default_rng(77)
    lens, qlens = [900, 33, 2100, 300], [1, 33, 1, 120]
    cfg = W.Config("wide", "wide", 16, 2, 128, 16, 260, W.FP8, qd, 77)
    wl = W.generate(W.custom_plan(cfg, lens, qlens, 77))
    q = oracle.decode_bits(wl.q, qd).astype(np.float32)
    q *= (10.0 ** rng.uniform(-3, 2, size=(1, 1, 128))).astype(np.float32)
    q *= (10.0 ** rng.uniform(-1, 1, size=(q.shape[0], q.shape[1], 1))).astype(np.float32)
    if qd == W.BF16:
        q[:, 3, :] *= np.float32(1e-39 / 4)     # one head's queries subnormal (bf16 keeps them)
    wl.q = W.round_to_bits(q, qd)
    _check(wl, _run(wl, f"fp8 scores, wide-range {qd} queries"))


def _spread_magnitudes(wl, seed, k_decades, v_decades):
    """K/V of a generated step with magnitudes spread over decades: factors
    10^U(lo, hi) per (block, head, slot) on 16-bit pools (rounded again), per
    (block, head) on fp8 pools' scales (bytes kept).  The step's appended rows
    are re-read from the pools."""
    rng = np.random.default_rng(seed)
    cfg = wl.cfg
    for store, scales, (lo, hi) in ((wl.k, wl.k_scale, k_decades), (wl.v, wl.v_scale, v_decades)):
        if cfg.kv_dtype == W.FP8:
            scales *= (10.0 ** rng.uniform(lo, hi, scales.shape)).astype(np.float32)
            continue
        x = oracle.decode_bits(store.blocks, cfg.kv_dtype).astype(np.float32)
        f = (10.0 ** rng.uniform(lo, hi, x.shape[:3] + (1,))).astype(np.float32)
        bits = W.round_to_bits(x * f, cfg.kv_dtype)
        store.blocks[...] = np.where(store.blocks == store.poison, store.blocks, bits)
    rows = np.searchsorted(wl.k.used_ids, wl.append_block)
    wl.k_new = np.ascontiguousarray(wl.k.blocks[rows, :, wl.append_offset, :])
    wl.v_new = np.ascontiguousarray(wl.v.blocks[rows, :, wl.append_offset, :])
    return wl


@pytest.mark.parametrize("kv", [W.BF16, W.F16, W.FP8])
@pytest.mark.parametrize("scale_mul", [1.0, 20.0, 1e-3, 0.0])
def test_kv_magnitudes_over_decades_and_extreme_softmax_scales(kv, scale_mul):
    # keys and values whose sizes vary over decades (16-bit: K and V per token
    # over 4; fp8: K per block scale over 6, V scales at most their generated
    # size over 3 -- the fp8 tolerance is absolute, and a bf16 output near 40
    # is already 0.125 from its neighbours), with the softmax scale as given,
    # 20x (nearly one-hot weights), 1/1000 (nearly flat) or 0 (every visible key
    # weighs the same): decode, verify and prefill rows, MHA 16-bit and 8:1 fp8,
    # against the oracle
    lens, qlens = [700, 90, 2300, 400, 1500, 64], [1, 90, 1, 5, 1, 64]
    Hq, Hkv = (16, 2) if kv == W.FP8 else (8, 8)
    nb = sum(-(-L // 16) for L in lens) + 13
    cfg = W.Config("mag", "mag", Hq, Hkv, 128, 16, nb, kv, W.F16 if kv == W.F16 else W.BF16, 91)
    wl = _spread_magnitudes(W.generate(W.custom_plan(cfg, lens, qlens, 91)), 92,
                            (-3, 3) if kv == W.FP8 else (-2, 2), (-3, 0) if kv == W.FP8 else (-2, 2))
    wl.scale = np.float32(wl.scale * scale_mul)
    _check(wl, _run(wl, f"magnitudes over decades kv={kv} scale x{scale_mul}"))
