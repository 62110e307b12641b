"""Put a synthetic step on the GPU and drive it through the C ABI.

Torch is used only to allocate device memory, upload the seeded inputs and
name the stream; both computations (append and attention) are calls into
libpagedkv through :mod:`paged_kv_cache_286_amd.pagedkv`.
"""
from __future__ import annotations

import numpy as np
import torch

from . import pagedkv as pk
from .workloads import FP8, STORAGE, Workload

_TORCH_STORE = {np.uint16: torch.int16, np.uint8: torch.uint8}


def _bits_tensor(a: np.ndarray, device) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device)
    return torch.from_numpy(a).to(device)


def _poison_value(bits: int, store):
    if store == torch.int16:
        return int(np.array([bits], dtype=np.uint16).view(np.int16)[0])
    return int(bits)


def shared_prefix_blocks(tables: np.ndarray, context_lens: np.ndarray) -> np.ndarray:
    """Per sequence, the leading table entries whose block also appears in another
    sequence's table (the cache-policy hint of paged_attn_step)."""
    lens = np.asarray(context_lens, np.int64)
    nblk = (lens + 15) // 16
    cols = np.arange(tables.shape[1])[None, :]
    used = cols < nblk[:, None]
    ids = tables[used]
    counts = np.bincount(ids[ids >= 0], minlength=1) if ids.size else np.zeros(1, np.int64)
    shared = np.zeros(tables.shape, bool)
    valid = used & (tables >= 0)
    shared[valid] = counts[tables[valid]] > 1
    # length of the leading run of shared entries
    run = np.cumprod(shared, axis=1).sum(axis=1)
    return run.astype(np.int32)


def check_slots_injective(slot_mapping, num_slots: int) -> None:
    """Raise ValueError unless the in-pool slots of an append are distinct.

    Page "Serving LLMs with vLLM", section "Growing During Decode": each new
    token takes a slot of its own.  Two rows aimed at one slot would race in
    the append kernel (whichever lands last wins), so the host refuses such a
    step before anything is enqueued.  Negative slots and slots past the pool
    are skipped rows and may repeat."""
    s = np.asarray(slot_mapping, dtype=np.int64)
    s = s[(s >= 0) & (s < int(num_slots))]
    if s.size != np.unique(s).size:
        vals, counts = np.unique(s, return_counts=True)
        raise ValueError(f"slot_mapping names slot {int(vals[counts > 1][0])} more than once")


def append_fusable(tables: np.ndarray, context_lens, query_lens, slot_mapping) -> bool:
    """True when a step meets paged_append_attn_step's contract: every appended
    row's slot is the one its table names for that row's position, and no block
    holding an appended slot is read by another sequence (the state
    copy-on-write keeps a step in).  Linear in the step's table entries: this
    runs on the host before every engine step."""
    tables = np.asarray(tables)
    lens = np.asarray(context_lens, np.int64)
    qlens = np.asarray(query_lens, np.int64)
    slots = np.asarray(slot_mapping, np.int64)
    S = len(lens)
    seq = np.repeat(np.arange(S), qlens)
    if len(seq) != len(slots) or len(seq) == 0:
        return False
    # position of every row: L - Q .. L - 1 of its sequence
    first = np.repeat(np.cumsum(qlens) - qlens, qlens)
    pos = np.repeat(lens - qlens, qlens) + (np.arange(len(seq)) - first)
    if pos.min() < 0 or (pos // 16).max() >= tables.shape[1]:
        return False
    blk = tables[seq, pos // 16].astype(np.int64)
    if blk.min() < 0 or not np.array_equal(slots, blk * 16 + pos % 16):
        return False
    # every table entry a sequence reads, with its reader
    nblk = (lens + 15) // 16
    if nblk.max() > tables.shape[1]:
        return False
    starts = np.repeat(np.cumsum(nblk) - nblk, nblk)
    col = np.arange(int(nblk.sum())) - starts
    reader = np.repeat(np.arange(S), nblk)
    used = tables.ravel()[reader * tables.shape[1] + col].astype(np.int64)
    if used.min() < 0:
        return False
    # the sequence appending into each appended block; a block appended by two
    # sequences, or read by a sequence other than its appender, breaks it
    owner = np.full(int(max(used.max(), blk.max())) + 1, -1, np.int32)
    owner[blk] = seq
    if not np.array_equal(owner[blk], seq):
        return False
    o = owner[used]
    return bool(((o < 0) | (o == reader)).all())


# Gap between the K and the V pool when both come from one allocation.  Two
# separate large allocations put block b's K and V slices at the same address
# modulo 2 MiB, where they contend for the same HBM banks; starting V 4 KiB
# past the end of K moved the 7B decode step (64 sequences, 2 GiB pools) from
# 373 to 363 us on an MI355X (odd multiples of 4 KiB alike; 2 KiB changed
# nothing, and the other workloads moved by under 1%).
KV_POOL_GAP_BYTES = 4096


def alloc_kv_pools(shape, dtype, device, fill=0):
    """K and V pools of `shape` from one allocation, V starting
    KV_POOL_GAP_BYTES past the end of K (views; each pool contiguous)."""
    n = 1
    for d in shape:
        n *= int(d)
    esize = torch.empty(0, dtype=dtype).element_size()
    gap = KV_POOL_GAP_BYTES // esize
    buf = torch.full((2 * n + gap,), fill, dtype=dtype, device=device)
    return buf[:n].view(shape), buf[n + gap:].view(shape)


class DeviceStep:
    """Device buffers of one step plus the two ABI calls that run it."""

    # buffers whose addresses the bound calls of step() hold: assigning any of
    # them drops the bound calls, so the next step() converts the new addresses
    _BOUND_BUFFERS = frozenset((
        "k_pool", "v_pool", "k_scale", "v_scale", "block_tables", "context_lens", "query_lens",
        "shared_blocks", "q", "out", "k_new", "v_new", "slot_mapping", "workspace", "ws_bytes",
        "pool"))

    def __setattr__(self, name, value):
        if name in DeviceStep._BOUND_BUFFERS:
            object.__setattr__(self, "_bound", None)
            object.__setattr__(self, "_bound_key", None)
        object.__setattr__(self, name, value)

    def __init__(self, wl: Workload, device: str = "cuda:0", upload_chunk_blocks: int = 8192):
        self.wl = wl
        cfg, plan = wl.cfg, wl.plan
        self.device = torch.device(device)
        store = _TORCH_STORE[STORAGE[cfg.kv_dtype]]
        shape = (cfg.num_blocks, cfg.num_kv_heads, cfg.block_size, cfg.head_dim)
        poison = _poison_value(wl.k.poison, store)
        self.k_pool, self.v_pool = alloc_kv_pools(shape, store, self.device, poison)
        ids = torch.from_numpy(wl.k.used_ids).to(self.device)
        for lo in range(0, len(wl.k.used_ids), upload_chunk_blocks):
            hi = min(len(wl.k.used_ids), lo + upload_chunk_blocks)
            self.k_pool.index_copy_(0, ids[lo:hi], _bits_tensor(wl.k.blocks[lo:hi], self.device))
            self.v_pool.index_copy_(0, ids[lo:hi], _bits_tensor(wl.v.blocks[lo:hi], self.device))
        self.poison_appended_slots()
        if cfg.kv_dtype == FP8:
            self.k_scale = torch.from_numpy(wl.k_scale).to(self.device)
            self.v_scale = torch.from_numpy(wl.v_scale).to(self.device)
        else:
            self.k_scale = self.v_scale = None
        self.block_tables = torch.from_numpy(plan.block_tables).to(self.device)
        self.context_lens = torch.from_numpy(plan.context_lens).to(self.device)
        self.query_lens = torch.from_numpy(plan.query_lens).to(self.device)
        shared = shared_prefix_blocks(plan.block_tables, plan.context_lens)
        self.shared_blocks = (torch.from_numpy(shared).to(self.device) if shared.any() else None)
        self.q = _bits_tensor(wl.q, self.device)
        self.out = torch.full_like(self.q, _poison_value(0x7FC0 if cfg.q_dtype == "bf16" else 0x7E00,
                                                         torch.int16))
        check_slots_injective(wl.slot_mapping, cfg.num_blocks * cfg.block_size)
        self.k_new = _bits_tensor(wl.k_new, self.device)
        self.v_new = _bits_tensor(wl.v_new, self.device)
        self.slot_mapping = torch.from_numpy(wl.slot_mapping).to(self.device)
        self.pool = pk.make_pool(cfg.num_blocks, cfg.block_size, cfg.num_kv_heads, cfg.head_dim,
                                 cfg.kv_dtype)
        self.q_dtype = pk.DTYPE_CODES[cfg.q_dtype]
        self.kv_dtype = pk.DTYPE_CODES[cfg.kv_dtype]
        self.ws_bytes = pk.paged_attn_workspace_bytes(
            self.pool, plan.num_seqs, cfg.num_q_heads, plan.total_q_tokens, plan.max_context_len,
            plan.max_query_len)
        self.workspace = (torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
                          if self.ws_bytes else None)
        self.fusable = append_fusable(plan.block_tables, plan.context_lens, plan.query_lens,
                                      wl.slot_mapping)
        self._bound, self._bound_key = None, None

    def poison_appended_slots(self) -> None:
        """Put the pools back in their pre-append state (appended slots hold NaN bits)."""
        wl = self.wl
        if len(wl.append_block) == 0:
            return
        blk = torch.from_numpy(wl.append_block).to(self.device)
        off = torch.from_numpy(wl.append_offset).to(self.device)
        val = _poison_value(wl.k.poison, self.k_pool.dtype)
        self.k_pool[blk, :, off, :] = val
        self.v_pool[blk, :, off, :] = val

    def append(self, stream=None) -> None:
        pk.paged_kv_append(self.pool, self.k_pool, self.v_pool, self.k_new, self.v_new,
                           self.kv_dtype, self.slot_mapping, len(self.wl.slot_mapping),
                           stream if stream is not None else torch.cuda.current_stream(self.device))

    def attend(self, stream=None) -> None:
        plan, cfg = self.wl.plan, self.wl.cfg
        pk.paged_attn_step(
            self.pool, self.q, self.q_dtype, cfg.num_q_heads, self.k_pool, self.v_pool,
            self.k_scale, self.v_scale, self.block_tables, plan.max_blocks_per_seq,
            self.context_lens, self.query_lens, plan.num_seqs, plan.total_q_tokens,
            plan.max_context_len, plan.max_query_len, float(self.wl.scale), self.out,
            self.workspace, self.ws_bytes,
            stream if stream is not None else torch.cuda.current_stream(self.device),
            shared_blocks=self.shared_blocks)

    def step(self, stream=None) -> None:
        """The whole step, append and attention: one paged_append_attn_step call
        where its contract holds (append_fusable), else paged_kv_append then
        paged_attn_step; the arguments are converted once per stream (replacing
        a buffer attribute drops the converted calls)."""
        s = stream if stream is not None else torch.cuda.current_stream(self.device)
        key = int(s.cuda_stream) if not isinstance(s, int) else s
        if self._bound_key != key:
            self._bound = ((self.bind_step(s),) if self.fusable
                           else (self.bind_append(s), self.bind_attend(s)))
            self._bound_key = key
        for call in self._bound:
            call()

    def step_separate(self, stream=None) -> None:
        """The same step as two calls: paged_kv_append, then paged_attn_step."""
        self.append(stream)
        self.attend(stream)

    def bind_step(self, stream):
        plan, cfg = self.wl.plan, self.wl.cfg
        return pk.bind_paged_append_attn_step(
            self.pool, self.k_pool, self.v_pool, self.k_new, self.v_new, self.slot_mapping,
            self.q, self.q_dtype, cfg.num_q_heads, self.k_scale, self.v_scale, self.block_tables,
            plan.max_blocks_per_seq, self.context_lens, self.query_lens, plan.num_seqs,
            plan.total_q_tokens, plan.max_context_len, plan.max_query_len, float(self.wl.scale),
            self.out, self.workspace, self.ws_bytes, stream, shared_blocks=self.shared_blocks)

    def rebind(self) -> None:
        self._bound, self._bound_key = None, None

    def bind_append(self, stream):
        return pk.bind_paged_kv_append(self.pool, self.k_pool, self.v_pool, self.k_new, self.v_new,
                                       self.kv_dtype, self.slot_mapping, len(self.wl.slot_mapping),
                                       stream)

    def bind_attend(self, stream):
        plan, cfg = self.wl.plan, self.wl.cfg
        return pk.bind_paged_attn_step(
            self.pool, self.q, self.q_dtype, cfg.num_q_heads, self.k_pool, self.v_pool,
            self.k_scale, self.v_scale, self.block_tables, plan.max_blocks_per_seq,
            self.context_lens, self.query_lens, plan.num_seqs, plan.total_q_tokens,
            plan.max_context_len, plan.max_query_len, float(self.wl.scale), self.out,
            self.workspace, self.ws_bytes, stream, shared_blocks=self.shared_blocks)

    def out_bits(self) -> np.ndarray:
        return self.out.cpu().numpy().view(np.uint16)
