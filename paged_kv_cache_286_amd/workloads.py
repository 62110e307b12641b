"""Seeded synthetic workloads for one scheduler step over a paged KV cache.

This module only draws random numbers, places blocks in a pool and stores the
result; it holds none of the attention or append arithmetic.  Both the HIP
path (through the test and bench harnesses) and the CPU oracle take their
inputs from here, so it imports neither of them.

Vocabulary follows "Serving LLMs with vLLM: Continuous Batching and
PagedAttention Explained" (section "Blocks and Block Tables"): the KV cache is
cut into fixed-size blocks of ``block_size`` tokens in one shared physical
pool; each sequence owns a block table listing the physical block that holds
each of its logical blocks; blocks need not be neighbours.

Storage conventions (shared by every consumer):

* K and V pools: ``[num_blocks][num_kv_heads][block_size][head_dim]`` raw
  element bits (uint16 for fp16/bf16, uint8 for fp8-e4m3).
* fp8 scales: ``float32[num_blocks][num_kv_heads]``, one array for K and one
  for V; a stored byte ``b`` of block ``blk`` / head ``h`` means
  ``e4m3(b) * scale[blk, h]``.
* q / out: ``[total_q_tokens][num_q_heads][head_dim]``; the query rows of
  sequence ``i`` follow those of sequence ``i - 1``.
* ``context_lens[i]`` counts every token of sequence ``i`` that this step's
  attention sees, including the rows appended in the same step;
  ``query_lens[i]`` is the number of query rows (1 for a decode), and those
  rows sit at positions ``context_lens[i] - query_lens[i] ...
  context_lens[i] - 1``.
* Slots of a block past the end of its sequence, blocks no table uses, and
  the slots this step's append will fill are "poisoned" with NaN bit
  patterns, so a kernel that reads them without masking shows it.

Value recipe: q, K and V are N(0, 1) float32 draws (numpy PCG64), rounded to
the stored type with round-to-nearest-even.  fp8 K/V use OCP E4M3FN with one
float32 scale per (block, kv_head): ``scale = max(amax, 2**-20) / 448`` over
the block's valid slots, then ``x / scale`` rounded and saturated to +-448.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import math
import os
from typing import Dict, List, Optional

import numpy as np

# ----------------------------------------------------------------------------
# element types
# ----------------------------------------------------------------------------
F16, BF16, FP8 = "f16", "bf16", "fp8_e4m3"
DTYPE_CODES = {F16: 0, BF16: 1, FP8: 2}          # mirror of pkv_dtype in the C header
STORAGE = {F16: np.uint16, BF16: np.uint16, FP8: np.uint8}
ELEM_BYTES = {F16: 2, BF16: 2, FP8: 1}
# quiet-NaN bit patterns used to poison slots nobody may read
POISON = {F16: 0x7E00, BF16: 0x7FC0, FP8: 0x7F}


def round_to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 array -> stored bit pattern of ``dtype`` (RNE), via library casts."""
    import torch

    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == F16:
        return x.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dtype == FP8:
        t = torch.from_numpy(np.clip(x, -448.0, 448.0))
        return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# configurations
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    description: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    kv_dtype: str
    q_dtype: str
    seed: int


CONFIGS: Dict[str, Config] = {
    "tiny_decode": Config(
        "tiny_decode",
        "4 seqs (ctx 10/40/20/80, 1 query each), 4 heads x 64, fp16, block 16, pool 64 blocks",
        4, 4, 64, 16, 64, F16, F16, 1),
    "decode_7b": Config(
        "decode_7b",
        "64 decode seqs, ctx U[128,4096], 32 heads x 128, bf16, block 16, pool for 64x4096 tokens",
        32, 32, 128, 16, 16384, BF16, BF16, 2),
    "long_tail": Config(
        "long_tail",
        "256 seqs, ctx Geometric(mean 600) clipped 32768, 32 share a 1504-token prefix (94 blocks) "
        "+ 50..500 own tokens, 32 heads x 128, bf16, 40 GiB K+V pool",
        32, 32, 128, 16, 163840, BF16, BF16, 3),
    "mixed_prefill": Config(
        "mixed_prefill",
        "128 decodes (ctx U[256,4096]) + a 512-token prefill chunk at offset 2048 of a 4000-token "
        "prompt, 32 heads x 128, bf16",
        32, 32, 128, 16, 33024, BF16, BF16, 4),
    "fp8_gqa_long": Config(
        "fp8_gqa_long",
        "64 decode seqs, ctx U[8192,32768], 64 q heads / 8 kv heads x 128, fp8-e4m3 K/V with a "
        "float32 scale per (block, kv head), bf16 q",
        64, 8, 128, 16, 131072, FP8, BF16, 5),
    # not one of the five steps the metric is quoted on: the 7B decode step's lengths
    # at a grouped-query head layout (32 query / 8 kv heads), which runs the 16-bit
    # MFMA decode items
    "gqa_decode": Config(
        "gqa_decode",
        "64 decode seqs, ctx U[128,4096], 32 q heads / 8 kv heads x 128, bf16, block 16, pool for "
        "64x4096 tokens",
        32, 8, 128, 16, 16384, BF16, BF16, 7),
    # not one of the five steps the metric is quoted on: the prefill tile alone, so
    # that its MFMA rate can be measured without decode rows hiding it
    "prefill_chunks": Config(
        "prefill_chunks",
        "4 whole prompts of 2048 tokens each as query chunks (no decode rows), 32 heads x 128, "
        "bf16, block 16",
        32, 32, 128, 16, 576, BF16, BF16, 6),
}


# ----------------------------------------------------------------------------
# the sequences of a step and where their blocks live
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class Plan:
    """Host-side description of one step: lengths, tables, appended slots."""
    cfg: Config
    context_lens: np.ndarray       # int32 [S]
    query_lens: np.ndarray         # int32 [S]
    block_tables: np.ndarray       # int32 [S][max_blocks], -1 padded
    max_blocks_per_seq: int
    shared_prefix_blocks: int = 0  # >0: seqs in shared_seqs begin with the same physical blocks
    shared_seqs: Optional[np.ndarray] = None

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def total_q_tokens(self) -> int:
        return int(self.query_lens.sum())

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max())

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max())


def _take_tables(lens, pool_order, bs, max_blocks, prefix=None, prefix_seqs=()):
    """Give each sequence ceil(len/bs) blocks from ``pool_order`` in sequence order."""
    S = len(lens)
    tables = np.full((S, max_blocks), -1, dtype=np.int32)
    cursor = 0
    pref = set(int(i) for i in prefix_seqs)
    for i, L in enumerate(lens):
        n = -(-int(L) // bs)
        start = 0
        if prefix is not None and i in pref:
            tables[i, :len(prefix)] = prefix
            start = len(prefix)
        need = n - start
        tables[i, start:n] = pool_order[cursor:cursor + need]
        cursor += need
    if cursor > len(pool_order):
        raise ValueError("pool too small for the step")
    return tables


def make_plan(name: str) -> Plan:
    cfg = CONFIGS[name]
    rng = np.random.default_rng([cfg.seed, 0])
    bs, NB = cfg.block_size, cfg.num_blocks
    if name == "tiny_decode":
        lens = np.array([10, 40, 20, 80], dtype=np.int64)
        qlens = np.ones(4, dtype=np.int64)
        order = rng.permutation(NB)
        tables = _take_tables(lens, order, bs, 80 // bs)
        return Plan(cfg, lens.astype(np.int32), qlens.astype(np.int32), tables, 80 // bs)
    if name == "decode_7b":
        lens = rng.integers(128, 4096, size=64, endpoint=True)
        qlens = np.ones(64, dtype=np.int64)
        order = rng.permutation(NB)
        mb = 4096 // bs
        return Plan(cfg, lens.astype(np.int32), qlens.astype(np.int32),
                    _take_tables(lens, order, bs, mb), mb)
    if name == "gqa_decode":
        lens = rng.integers(128, 4096, size=64, endpoint=True)
        qlens = np.ones(64, dtype=np.int64)
        order = rng.permutation(NB)
        mb = 4096 // bs
        return Plan(cfg, lens.astype(np.int32), qlens.astype(np.int32),
                    _take_tables(lens, order, bs, mb), mb)
    if name == "long_tail":
        S, n_shared, pre_tok = 256, 32, 1504
        lens = np.minimum(rng.geometric(1.0 / 600.0, size=S), 32768)
        shared = np.sort(rng.choice(S, size=n_shared, replace=False))
        lens[shared] = pre_tok + rng.integers(50, 500, size=n_shared, endpoint=True)
        qlens = np.ones(S, dtype=np.int64)
        order = rng.permutation(NB)
        n_pre = pre_tok // bs
        prefix = order[:n_pre]
        mb = 32768 // bs
        tables = _take_tables(lens, order[n_pre:], bs, mb, prefix=prefix, prefix_seqs=shared)
        return Plan(cfg, lens.astype(np.int32), qlens.astype(np.int32), tables, mb,
                    shared_prefix_blocks=n_pre, shared_seqs=shared.astype(np.int32))
    if name == "mixed_prefill":
        n_dec = 128
        lens = np.concatenate([rng.integers(256, 4096, size=n_dec, endpoint=True), [2048 + 512]])
        qlens = np.concatenate([np.ones(n_dec, dtype=np.int64), [512]])
        order = rng.permutation(NB)
        mb = 4096 // bs
        return Plan(cfg, lens.astype(np.int32), qlens.astype(np.int32),
                    _take_tables(lens, order, bs, mb), mb)
    if name == "prefill_chunks":
        lens = np.full(4, 2048, dtype=np.int64)
        order = rng.permutation(NB)
        mb = 2048 // bs
        return Plan(cfg, lens.astype(np.int32), lens.astype(np.int32), _take_tables(lens, order, bs, mb), mb)
    if name == "fp8_gqa_long":
        lens = rng.integers(8192, 32768, size=64, endpoint=True)
        qlens = np.ones(64, dtype=np.int64)
        order = rng.permutation(NB)
        mb = 32768 // bs
        return Plan(cfg, lens.astype(np.int32), qlens.astype(np.int32),
                    _take_tables(lens, order, bs, mb), mb)
    raise KeyError(name)


def custom_plan(cfg: Config, context_lens, query_lens, seed: int,
                max_blocks_per_seq: Optional[int] = None, shared_prefix_blocks: int = 0,
                shared_seqs=()) -> Plan:
    """A plan for arbitrary lengths (tests): random placement without replacement."""
    bs = cfg.block_size
    lens = np.asarray(context_lens, dtype=np.int64)
    qlens = np.asarray(query_lens, dtype=np.int64)
    mb = max_blocks_per_seq or max(1, int(-(-lens.max() // bs)))
    rng = np.random.default_rng([seed, 0])
    order = rng.permutation(cfg.num_blocks)
    prefix = None
    if shared_prefix_blocks:
        prefix = order[:shared_prefix_blocks]
        order = order[shared_prefix_blocks:]
    tables = _take_tables(lens, order, bs, mb, prefix=prefix, prefix_seqs=shared_seqs)
    return Plan(cfg, lens.astype(np.int32), qlens.astype(np.int32), tables, mb,
                shared_prefix_blocks=shared_prefix_blocks,
                shared_seqs=np.asarray(shared_seqs, dtype=np.int32) if shared_prefix_blocks else None)


# ----------------------------------------------------------------------------
# block contents
# ----------------------------------------------------------------------------
class BlockStore:
    """Sparse stand-in for a K or V pool: only the blocks some table uses.

    ``store[ids]`` (an integer array of physical ids) returns
    ``[len(ids)][Hkv][bs][D]`` raw bits like a dense pool would;
    ``store[blk, :, off, :] = row`` writes one slot of one block.
    """

    def __init__(self, used_ids: np.ndarray, blocks: np.ndarray, num_blocks: int, poison: int):
        self.used_ids = used_ids
        self.blocks = blocks
        self.num_blocks = num_blocks
        self.poison = poison
        self.shape = (num_blocks,) + blocks.shape[1:]
        self.dtype = blocks.dtype

    def _rows(self, ids):
        ids = np.asarray(ids, dtype=np.int64)
        pos = np.searchsorted(self.used_ids, ids)
        pos = np.minimum(pos, len(self.used_ids) - 1)
        if not np.all(self.used_ids[pos] == ids):
            raise KeyError("block id not in use")
        return pos

    def __getitem__(self, key):
        if isinstance(key, tuple):
            return self.blocks[(self._rows([key[0]])[0],) + key[1:]]
        return self.blocks[self._rows(key)]

    def __setitem__(self, key, value):
        if not isinstance(key, tuple):
            raise TypeError("write one block at a time")
        self.blocks[(self._rows([key[0]])[0],) + key[1:]] = value

    def copy(self) -> "BlockStore":
        return BlockStore(self.used_ids, self.blocks.copy(), self.num_blocks, self.poison)

    def dense(self) -> np.ndarray:
        """Materialise the whole pool (small pools only); unused blocks are poisoned."""
        out = np.full(self.shape, self.poison, dtype=self.dtype)
        out[self.used_ids] = self.blocks
        return out


@dataclasses.dataclass
class Workload:
    plan: Plan
    q: np.ndarray                  # [Tq][Hq][D] bits
    k: BlockStore                  # post-append contents of every used block
    v: BlockStore
    k_scale: Optional[np.ndarray]  # float32 [NB][Hkv] (fp8 only)
    v_scale: Optional[np.ndarray]
    slot_mapping: np.ndarray       # int32 [T_new]
    k_new: np.ndarray              # [T_new][Hkv][D] bits
    v_new: np.ndarray
    scale: np.float32              # softmax scale 1/sqrt(D) as float32
    append_block: np.ndarray       # int64 [T_new] physical block of each appended row
    append_offset: np.ndarray      # int64 [T_new] slot offset inside that block

    @property
    def cfg(self) -> Config:
        return self.plan.cfg

    def pre_append(self, which: str) -> BlockStore:
        """The pool as it stands before this step's append (appended slots poisoned)."""
        src = self.k if which == "k" else self.v
        out = src.copy()
        for blk, off in zip(self.append_block, self.append_offset):
            out[int(blk), :, int(off), :] = src.poison
        return out


def _valid_tokens_per_block(plan: Plan, used_ids: np.ndarray) -> np.ndarray:
    bs = plan.cfg.block_size
    valid = np.zeros(len(used_ids), dtype=np.int64)
    for i in range(plan.num_seqs):
        L = int(plan.context_lens[i])
        n = -(-L // bs)
        ids = plan.block_tables[i, :n].astype(np.int64)
        cnt = np.full(n, bs, dtype=np.int64)
        cnt[-1] = L - (n - 1) * bs
        pos = np.searchsorted(used_ids, ids)
        valid[pos] = np.maximum(valid[pos], cnt)
    return valid


def _fill_chunk(args):
    (seed, tag, lo, hi, shape, dtype, valid, poison) = args
    rng = np.random.default_rng([seed, tag, lo])
    x = rng.standard_normal((hi - lo,) + shape, dtype=np.float32)
    bs = shape[1]
    mask = np.arange(bs)[None, :] < valid[lo:hi, None]            # [n][bs]
    if dtype == FP8:
        amax = np.where(mask[:, None, :, None], np.abs(x), 0.0).max(axis=(2, 3))   # [n][Hkv]
        sc = (np.maximum(amax, np.float32(2.0 ** -20)) / np.float32(448.0)).astype(np.float32)
        bits = round_to_bits(x / sc[:, :, None, None], FP8)
    else:
        sc = None
        bits = round_to_bits(x, dtype)
    bits[~np.broadcast_to(mask[:, None, :, None], bits.shape)] = poison
    return lo, bits, sc


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def generate(plan: Plan, chunk_blocks: int = 512) -> Workload:
    """Draw q/K/V for ``plan`` (deterministic for a given plan and seed)."""
    cfg = plan.cfg
    bs, Hkv, D, Hq = cfg.block_size, cfg.num_kv_heads, cfg.head_dim, cfg.num_q_heads
    used = [plan.block_tables[i, :-(-int(L) // bs)] for i, L in enumerate(plan.context_lens)]
    used_ids = np.unique(np.concatenate(used).astype(np.int64))
    valid = _valid_tokens_per_block(plan, used_ids)
    U = len(used_ids)
    shape = (Hkv, bs, D)
    store_dt = STORAGE[cfg.kv_dtype]
    poison = POISON[cfg.kv_dtype]
    k_blocks = np.empty((U,) + shape, dtype=store_dt)
    v_blocks = np.empty((U,) + shape, dtype=store_dt)
    k_sc = np.ones((cfg.num_blocks, Hkv), dtype=np.float32) if cfg.kv_dtype == FP8 else None
    v_sc = np.ones((cfg.num_blocks, Hkv), dtype=np.float32) if cfg.kv_dtype == FP8 else None
    jobs = []
    for tag, dst in ((1, k_blocks), (2, v_blocks)):
        for lo in range(0, U, chunk_blocks):
            jobs.append((tag, dst, (cfg.seed, tag, lo, min(U, lo + chunk_blocks), shape,
                                    cfg.kv_dtype, valid, poison)))
    with _cf.ThreadPoolExecutor(_workers()) as ex:
        futs = [(tag, dst, ex.submit(_fill_chunk, a)) for tag, dst, a in jobs]
        for tag, dst, f in futs:
            lo, bits, sc = f.result()
            dst[lo:lo + len(bits)] = bits
            if sc is not None:
                (k_sc if tag == 1 else v_sc)[used_ids[lo:lo + len(bits)]] = sc
    q_rng = np.random.default_rng([cfg.seed, 3])
    q = round_to_bits(q_rng.standard_normal((plan.total_q_tokens, Hq, D), dtype=np.float32),
                      cfg.q_dtype)
    k_store = BlockStore(used_ids, k_blocks, cfg.num_blocks, poison)
    v_store = BlockStore(used_ids, v_blocks, cfg.num_blocks, poison)

    # rows appended this step: every query position of every sequence
    slots, a_blk, a_off = [], [], []
    for i in range(plan.num_seqs):
        L, Q = int(plan.context_lens[i]), int(plan.query_lens[i])
        for pos in range(L - Q, L):
            blk = int(plan.block_tables[i, pos // bs])
            a_blk.append(blk)
            a_off.append(pos % bs)
            slots.append(blk * bs + pos % bs)
    a_blk = np.asarray(a_blk, dtype=np.int64)
    a_off = np.asarray(a_off, dtype=np.int64)
    rows = np.searchsorted(used_ids, a_blk)
    k_new = np.ascontiguousarray(k_blocks[rows, :, a_off, :])
    v_new = np.ascontiguousarray(v_blocks[rows, :, a_off, :])
    return Workload(plan, q, k_store, v_store, k_sc, v_sc,
                    np.asarray(slots, dtype=np.int32), k_new, v_new,
                    np.float32(1.0 / math.sqrt(D)), a_blk, a_off)


def kv_bytes_per_token(cfg: Config) -> int:
    """K plus V bytes one token occupies in one layer's pools."""
    return 2 * cfg.num_kv_heads * cfg.head_dim * ELEM_BYTES[cfg.kv_dtype]


def algorithmic_kv_bytes(plan: Plan) -> Dict[str, int]:
    """Bytes the step must read: each distinct physical (block, token) row once.

    Shared prefix blocks count once ("unique"); ``logical`` counts them per
    reader.  fp8 adds the two float32 scales of every distinct (block, head).
    """
    cfg = plan.cfg
    bs = cfg.block_size
    per_tok = kv_bytes_per_token(cfg)
    logical_tokens = int(plan.context_lens.astype(np.int64).sum())
    seen: Dict[int, int] = {}
    for i, L in enumerate(plan.context_lens):
        L = int(L)
        n = -(-L // bs)
        for j in range(n):
            blk = int(plan.block_tables[i, j])
            cnt = min(bs, L - j * bs)
            seen[blk] = max(seen.get(blk, 0), cnt)
    unique_tokens = sum(seen.values())
    extra = 0
    if cfg.kv_dtype == FP8:
        extra = len(seen) * cfg.num_kv_heads * 2 * 4
    return {"unique": unique_tokens * per_tok + extra,
            "logical": logical_tokens * per_tok + (extra if cfg.kv_dtype == FP8 else 0),
            "unique_tokens": unique_tokens, "logical_tokens": logical_tokens,
            "distinct_blocks": len(seen)}
