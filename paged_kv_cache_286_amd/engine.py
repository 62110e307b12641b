"""Continuous batching over the paged KV cache: the host step loop.

Page "Why a Second Kind of Engine", section "Continuous batching" (the
five-step iteration) and page "Serving LLMs with vLLM: Continuous Batching and
PagedAttention Explained", sections "Schedule Per Step", "What the Scheduler
Does", "Chunked Prefill", "Growing During Decode", "Shared Prefixes" and
"Copy-on-Write".  Every step:

1. arrived requests join the waiting queue;
2. the batch is formed from the running sequences (one query token each while
   decoding, the next prompt chunk while prefilling) plus as many waiting
   requests as the free slots, the token budget and the free KV blocks allow;
3. if the blocks for the step's tokens are short, the most recently admitted
   sequence is preempted (its blocks released; it is recomputed later);
4. the step runs: copy-on-write block copies, the KV append of the step's new
   rows, then attention for every query row (``paged_kv_copy_blocks``, then
   ``paged_append_attn_step``, or ``paged_kv_append`` / ``paged_kv_append_quant``
   and ``paged_attn_step``);
5. finished sequences leave and release their blocks in the same step.

Only the attention layer is modelled: queries, keys and values of the step's
tokens are seeded random numbers (there are no model weights), so the loop
measures the scheduler and the paged-KV kernels, not a language model.

Readings: a slot freed by a sequence that finishes in step s is filled in step
s+1; a request needs ``prompt`` prefill tokens, then emits its first output
token at the end of its last prefill chunk and one more per decode step, so it
runs ``output - 1`` decode steps; a preempted request restarts its prefill.
"""
from __future__ import annotations

import dataclasses
from collections import deque
from typing import Dict, List, Optional

import numpy as np

from . import pagedkv as pk
from .device import append_fusable, check_slots_injective


@dataclasses.dataclass
class Request:
    rid: int
    prompt: int                  # prompt tokens
    output: int                  # output tokens to generate (>= 1)
    arrival: int = 0             # step at which it arrives
    parent: int = -1             # request whose first `shared` tokens it shares (prefix sharing)
    shared: int = 0
    tokens: Optional[np.ndarray] = None   # token ids: the prompt's, optionally followed by the output's


@dataclasses.dataclass
class _Seq:
    req: Request
    computed: int = 0            # prompt tokens whose K/V is in the cache
    generated: int = 0           # output tokens emitted
    admitted_step: int = -1
    first_token_step: int = -1
    token_steps: List[int] = dataclasses.field(default_factory=list)
    keyed: bool = False          # added with its token ids (the prefix cache can key its blocks)
    cached: int = 0              # prompt tokens found in the prefix cache at admission

    @property
    def prefilling(self) -> bool:
        return self.computed < self.req.prompt

    @property
    def kv_len(self) -> int:
        return self.computed + max(0, self.generated - 1)


@dataclasses.dataclass
class StepBatch:
    """What one step computes: rows in sequence order, ready for the ABI."""
    step: int
    seq_ids: np.ndarray          # int64 [S]
    query_lens: np.ndarray       # int32 [S]
    context_lens: np.ndarray     # int32 [S]
    block_tables: np.ndarray     # int32 [S][max_blocks]
    slot_mapping: np.ndarray     # int32 [sum(query_lens)]
    copies: np.ndarray           # int32 [k][2] copy-on-write (source, destination)
    finished: List[int]
    preempted: List[int]
    shared_blocks: np.ndarray = None  # int32 [S] leading blocks held by several sequences
    positions: np.ndarray = None  # int32 [rows] position of each new row in its sequence
    token_ids: np.ndarray = None  # int32 [rows] its token id, -1 where the request gave none


class ContinuousBatcher:
    """Per-step batch formation over a pkv_bm block manager (host only)."""

    def __init__(self, num_blocks: int, block_size: int = 16, max_seqs: int = 256,
                 token_budget: int = 2048, max_blocks_per_seq: int = 2048,
                 policy: str = "continuous", prefix_cache: bool = False):
        if policy not in ("continuous", "static"):
            raise ValueError(policy)
        self.bm = pk.BlockManager(num_blocks, block_size, prefix_cache=prefix_cache)
        self.block_size = block_size
        self.max_seqs = max_seqs
        self.budget = token_budget
        self.max_blocks = max_blocks_per_seq
        self.policy = policy
        self.pending: List[Request] = []
        self.waiting: deque = deque()
        self.running: List[_Seq] = []
        self.done: Dict[int, _Seq] = {}
        self.step_no = 0
        self.slot_steps = 0          # sum over steps of batch slots (static batching reckoning)
        self.useful = 0              # output tokens produced
        self.preemptions = 0
        self.cow_copies = 0
        self.prefill_computed = 0    # prompt tokens whose K/V the steps computed
        self.prefill_cached = 0      # prompt tokens taken from the prefix cache instead
        self._release: List[int] = []   # finished in the previous step, blocks not yet returned

    # -- requests ---------------------------------------------------------
    def submit(self, req: Request) -> None:
        if req.output < 1 or req.prompt < 1:
            raise ValueError("a request needs a prompt and at least one output token")
        if req.tokens is not None and len(req.tokens) < req.prompt:
            raise ValueError("token ids, when given, cover at least the prompt")
        self.pending.append(req)

    def idle(self) -> bool:
        return not (self.pending or self.waiting or self.running)

    def run_to_completion(self, max_steps: int = 1_000_000, on_step=None) -> int:
        """Plan steps until every request has finished; returns the number of steps."""
        while not self.idle() and self.step_no < max_steps:
            batch = self.plan()
            if on_step is not None:
                on_step(batch)
        self.flush()
        return self.step_no

    def flush(self) -> None:
        """Return the blocks of sequences that finished in the last planned step."""
        for rid in self._release:
            self.bm.release(rid)
        self._release = []

    # -- one step -----------------------------------------------------------
    def _tokens_for(self, s: _Seq, budget_left: int) -> int:
        if s.prefilling:
            return min(s.req.prompt - s.computed, budget_left)
        return 1

    def _shared_parent_alive(self, req: Request) -> bool:
        return req.parent >= 0 and any(r.req.rid == req.parent for r in self.running)

    def plan(self) -> StepBatch:
        """Form the next step's batch and reserve its KV slots (host only)."""
        # Sequences that finished in the previous step return their blocks now: the
        # previous step's kernels are already enqueued, and stream order puts
        # their reads before this step's writes into reused blocks.
        self.flush()
        self.step_no += 1
        step = self.step_no
        arrived = [r for r in self.pending if r.arrival <= step]
        self.pending = [r for r in self.pending if r.arrival > step]
        self.waiting.extend(sorted(arrived, key=lambda r: (r.arrival, r.rid)))

        preempted: List[int] = []
        while True:
            budget = self.budget
            plan: List[tuple] = []
            for s in self.running:
                n = self._tokens_for(s, budget)
                if n > 0:
                    plan.append((s, n))
                    budget -= n
            seqs = [s.req.rid for s, _ in plan]
            counts = [n for _, n in plan]
            need = self.bm.blocks_needed(seqs, counts) if seqs else 0
            if need <= self.bm.free_blocks:
                break
            victim = self.running.pop()                 # most recently admitted
            self.bm.release(victim.req.rid)
            preempted.append(victim.req.rid)
            self.preemptions += 1
            victim.computed, victim.generated = 0, 0
            victim.token_steps.clear()
            self.waiting.appendleft(victim.req)

        # Continuous batching admits while this step's token budget lasts.  A static
        # batch is formed only when the previous one has drained, and then fills
        # every slot at once; prompts beyond this step's budget are prefilled in
        # the following steps.
        static = self.policy == "static"
        may_admit = not static or not self.running
        while (may_admit and self.waiting and len(self.running) < self.max_seqs
               and (budget > 0 or static)):
            req = self.waiting[0]
            keyed = req.tokens is not None
            if keyed:
                # the prefix cache (when on) supplies the leading full blocks it holds
                shared = self.bm.add_prompt(req.rid, req.tokens[:req.prompt])
            else:
                parent = req.parent if self._shared_parent_alive(req) else -1
                shared = req.shared if parent >= 0 else 0
                if parent >= 0:
                    shared = min(shared, self.bm.length(parent), req.prompt - 1)
                self.bm.add(req.rid, parent, shared)
            first = min(req.prompt - shared, max(budget, 0))
            if self.bm.blocks_needed(seqs + [req.rid], counts + [first]) > self.bm.free_blocks:
                self.bm.release(req.rid)
                break
            self.waiting.popleft()
            s = _Seq(req, computed=shared, admitted_step=step, keyed=keyed,
                     cached=shared if keyed else 0)
            self.prefill_cached += s.cached
            self.running.append(s)
            if first > 0:
                plan.append((s, first))
                seqs.append(req.rid)
                counts.append(first)
                budget -= first

        slots, copies = self.bm.append(seqs, counts) if seqs else (np.zeros(0, np.int32),
                                                                    np.zeros((0, 2), np.int32))
        self.cow_copies += len(copies)
        positions = np.concatenate([np.arange(s.kv_len, s.kv_len + n, dtype=np.int32)
                                    for s, n in plan]) if plan else np.zeros(0, np.int32)
        token_ids = np.full(len(positions), -1, np.int32)
        r = 0
        for s, n in plan:
            t = s.req.tokens
            if t is not None:
                lo = s.kv_len
                hi = min(lo + n, len(t))
                if hi > lo:
                    token_ids[r:r + hi - lo] = t[lo:hi]
                # a decode row's id reaches the prefix cache once its row is written
                if s.keyed and not s.prefilling and hi > lo:
                    self.bm.extend_tokens(s.req.rid, t[lo:hi])
            if s.prefilling:
                self.prefill_computed += n
            r += n
        tables, lens = self.bm.tables(seqs, self.max_blocks) if seqs else (
            np.zeros((0, self.max_blocks), np.int32), np.zeros(0, np.int32))
        shared_blocks = self.bm.shared_prefix(seqs) if seqs else np.zeros(0, np.int32)
        self.slot_steps += self.max_seqs if self.policy == "static" else len(plan)

        # advance the host state as the step will leave it
        finished: List[int] = []
        for s, n in plan:
            if s.prefilling:
                s.computed += n
                if not s.prefilling:
                    s.generated = 1
                    s.first_token_step = step
                    s.token_steps.append(step)
            else:
                s.generated += 1
                s.token_steps.append(step)
            if s.generated >= s.req.output:
                finished.append(s.req.rid)
        self.useful += sum(1 for s, _ in plan if s.token_steps and s.token_steps[-1] == step)
        for rid in finished:
            s = next(x for x in self.running if x.req.rid == rid)
            self.running.remove(s)
            self.done[rid] = s
        self._release = list(finished)
        return StepBatch(step, np.asarray(seqs, np.int64), np.asarray(counts, np.int32),
                         lens.astype(np.int32), tables, slots.astype(np.int32), copies,
                         finished, preempted, shared_blocks, positions, token_ids)


KV_TABLE_ROWS = 4096


def kv_row_index(token_ids: np.ndarray, positions: np.ndarray) -> np.ndarray:
    """Row of the synthetic K/V tables that a token at a position writes: a fixed
    function of (token id, position), so equal prefixes give equal K/V."""
    t = np.asarray(token_ids, np.int64)
    p = np.asarray(positions, np.int64)
    return (t * 7919 + p * 104729) % KV_TABLE_ROWS


class DeviceEngine:
    """Runs planned steps on the GPU through the C ABI (synthetic q / K / V).

    kv_from_tokens=False: each new K/V row is fresh random numbers.  True: every
    request carries token ids and a row is picked from fixed seeded tables by
    kv_row_index(token, position), so K/V depend on the token prefix only, as a
    model's do -- the condition under which a prefix-cache hit can stand in for
    a prefill.  The tables (bf16 / f16 bits) are kept in ``self.kv_tables``.
    """

    # fp8 pools: the scale a block takes when its first row is written, per kv
    # head (a fixed scale: N(0,1) rows reach the E4M3 limit of 448 only past 7)
    FP8_BLOCK_SCALE = 1.0 / 64.0

    def __init__(self, batcher: ContinuousBatcher, num_q_heads: int, num_kv_heads: int,
                 head_dim: int, dtype: str = "bf16", seed: int = 0, device: str = "cuda:0",
                 kv_from_tokens: bool = False,
                 kv_dtype: Optional[str] = None):
        """dtype: the query / new-row type (bf16 or f16).  kv_dtype: the pools'
        type, dtype (default) or "fp8_e4m3" (rows quantised on append with a
        scale per (block, kv head))."""
        import torch
        from .device import alloc_kv_pools
        self.torch = torch
        self.b = batcher
        self.Hq, self.Hkv, self.D = num_q_heads, num_kv_heads, head_dim
        self.dtype = dtype
        self.kv_dtype = kv_dtype or dtype
        self.fp8 = self.kv_dtype == "fp8_e4m3"
        if self.kv_dtype not in (dtype, "fp8_e4m3"):
            raise ValueError(f"kv_dtype {self.kv_dtype} with rows of {dtype}")
        self.dev = torch.device(device)
        nb, bs = batcher.bm.num_blocks, batcher.block_size
        tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
        self.tdt = tdt
        self.k_pool, self.v_pool = alloc_kv_pools((nb, num_kv_heads, bs, head_dim),
                                                  torch.uint8 if self.fp8 else tdt, self.dev)
        self.pool = pk.make_pool(nb, bs, num_kv_heads, head_dim, self.kv_dtype)
        self.code = pk.DTYPE_CODES[dtype]
        self.k_scale = self.v_scale = self.new_block_scale = None
        if self.fp8:
            self.k_scale = torch.ones((nb, num_kv_heads), dtype=torch.float32, device=self.dev)
            self.v_scale = torch.ones_like(self.k_scale)
            self.new_block_scale = torch.full((num_kv_heads,), self.FP8_BLOCK_SCALE,
                                              dtype=torch.float32, device=self.dev)
        self.gen = torch.Generator(device=self.dev)
        self.gen.manual_seed(seed)
        self.scale = float(np.float32(1.0 / np.sqrt(head_dim)))
        self.kv_tables = None
        if kv_from_tokens:
            g = torch.Generator().manual_seed(seed + 1)
            shape = (KV_TABLE_ROWS, num_kv_heads, head_dim)
            ek, ev = (torch.randn(shape, generator=g).to(tdt) for _ in range(2))
            self.kv_tables = (ek.view(torch.int16).numpy().view(np.uint16),
                              ev.view(torch.int16).numpy().view(np.uint16))
            self._ek, self._ev = ek.to(self.dev), ev.to(self.dev)
        self.last = None

    def run(self, batch: StepBatch, stream=None):
        """Enqueue one step; returns (q, out) device tensors of the step's rows."""
        torch = self.torch
        stream = stream if stream is not None else torch.cuda.current_stream(self.dev)
        S = len(batch.seq_ids)
        if S == 0:
            return None
        rows = int(batch.query_lens.sum())
        q = torch.randn((rows, self.Hq, self.D), generator=self.gen, device=self.dev).to(self.tdt)
        if self.kv_tables is not None:
            if (batch.token_ids < 0).any():
                raise ValueError("kv_from_tokens needs the token id of every row")
            idx = torch.from_numpy(kv_row_index(batch.token_ids, batch.positions)).to(self.dev)
            k_new = self._ek.index_select(0, idx)
            v_new = self._ev.index_select(0, idx)
        else:
            k_new = torch.randn((rows, self.Hkv, self.D), generator=self.gen,
                                device=self.dev).to(self.tdt)
            v_new = torch.randn((rows, self.Hkv, self.D), generator=self.gen,
                                device=self.dev).to(self.tdt)
        out = torch.empty_like(q)
        if len(batch.copies):
            pairs = torch.from_numpy(np.ascontiguousarray(batch.copies)).to(self.dev)
            pk.paged_kv_copy_blocks(self.pool, self.k_pool, self.v_pool, self.k_scale,
                                    self.v_scale, pairs, len(batch.copies), stream)
        check_slots_injective(batch.slot_mapping, self.b.bm.num_blocks * self.b.block_size)
        slots = torch.from_numpy(batch.slot_mapping).to(self.dev)
        tables = torch.from_numpy(batch.block_tables).to(self.dev)
        ctx = torch.from_numpy(batch.context_lens).to(self.dev)
        ql = torch.from_numpy(batch.query_lens).to(self.dev)
        max_ctx, max_q = int(batch.context_lens.max()), int(batch.query_lens.max())
        ws_bytes = pk.paged_attn_workspace_bytes(self.pool, S, self.Hq, rows, max_ctx, max_q)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=self.dev)
        shared = None
        if batch.shared_blocks is not None and batch.shared_blocks.any():
            shared = torch.from_numpy(batch.shared_blocks).to(self.dev)
        if not self.fp8 and append_fusable(batch.block_tables, batch.context_lens,
                                           batch.query_lens, batch.slot_mapping):
            # copy-on-write left every appended slot private: append and step in one call
            pk.paged_append_attn_step(self.pool, self.k_pool, self.v_pool, k_new, v_new, slots, q,
                                      self.code, self.Hq, self.k_scale, self.v_scale, tables,
                                      self.b.max_blocks, ctx, ql, S, rows, max_ctx, max_q,
                                      self.scale, out, ws, ws_bytes, stream, shared_blocks=shared)
        else:
            if self.fp8:
                pk.paged_kv_append_quant(self.pool, self.k_pool, self.v_pool, self.k_scale,
                                         self.v_scale, k_new, v_new, self.code,
                                         self.new_block_scale, self.new_block_scale, slots, rows,
                                         stream)
            else:
                pk.paged_kv_append(self.pool, self.k_pool, self.v_pool, k_new, v_new, self.code,
                                   slots, rows, stream)
            pk.paged_attn_step(self.pool, q, self.code, self.Hq, self.k_pool, self.v_pool,
                               self.k_scale, self.v_scale, tables, self.b.max_blocks, ctx, ql, S,
                               rows, max_ctx, max_q, self.scale, out, ws, ws_bytes, stream,
                               shared_blocks=shared)
        self.last = (q, out, ws, k_new, v_new)
        return q, out
