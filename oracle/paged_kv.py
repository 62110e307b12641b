"""CPU oracle for one scheduler step over a paged KV cache (float64, numpy).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the ``smoke()`` entry point and the CPU
baseline leg of the benchmark use it.  It shares no code with the HIP library
and imports nothing from the package: its inputs are plain numpy arrays (raw
element bits, int32 tables and lengths) or any object that returns blocks of
raw bits when indexed with an array of physical block ids.

What it computes, and where each step comes from:

* Page "Serving LLMs with vLLM: Continuous Batching and PagedAttention
  Explained", section "Attention Over Scattered Blocks": the paged kernel takes
  the block table, fetches every block from wherever it lives in the pool and
  scores block by block, yet the result is plain attention -- a softmax of the
  query against all earlier keys, weighting the values.  The oracle therefore
  first gathers a sequence's K and V through its table into contiguous arrays
  and then runs textbook softmax attention on them (gather-then-softmax).
* Same page, section "Blocks and Block Tables": the cache is cut into
  fixed-size blocks (16 tokens in the example); a per-sequence table lists the
  physical block behind each logical block, and blocks need not be adjacent.
  Logical token ``t`` of a sequence lives in physical block
  ``table[t // block_size]`` at offset ``t % block_size``.
* Same page, section "Growing During Decode": each decode step writes its new
  token into the next free slot of the sequence's last block.  The append
  oracle copies raw rows into the slots named by ``slot_mapping``
  (``slot = block * block_size + offset``; negative = skip).
* Same page, sections "Prefill Versus Decode" and "Chunked Prefill", and page
  "Why a Second Kind of Engine", section "Continuous batching": one step mixes
  decodes (one query row) with a piece of a long prompt.  A sequence with
  ``Q`` query rows and ``L`` visible tokens has its rows at positions
  ``L-Q .. L-1``; row ``r`` sees keys ``0 .. L-Q+r`` (causal).
* Page "Why a Second Kind of Engine", section "The memory that concurrency
  actually costs", and the "Static or continuous" section of the
  serving-many-users chapter: an 8-bit KV cache.  Read as OCP FP8 E4M3FN with
  one float32 scale per (block, kv head); a stored value is
  ``float32(e4m3(byte) * scale)``.
* Same sections, quantising on the way in: a 16-bit row appended to an fp8
  pool is divided by its block's scale and rounded to the nearest E4M3FN value
  (ties to even, saturating at +-448); a block whose first slot is written
  takes the caller's per-head scale.
* Page "Serving LLMs with vLLM ...", section "The KV Cache Is Big": per-token
  KV bytes = 2 x layers x hidden x bytes-per-value.
* Splitting a long context into partitions and merging their partial softmax
  states is not on the pages; ``partition_partials``/``lse_merge`` write out
  the standard log-sum-exp merge so that split kernels can be checked
  against the unsplit definition.

Readings where the pages are silent: K and V pools are laid out
``[num_blocks][num_kv_heads][block_size][head_dim]``; with more query heads
than kv heads, query head ``h`` reads kv head ``h // (Hq // Hkv)``; the
softmax scale arrives as float32 and is widened exactly.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

F16, BF16, FP8 = "f16", "bf16", "fp8_e4m3"


# ----------------------------------------------------------------------------
# element decoding (exact widening to float64)
# ----------------------------------------------------------------------------
def _fp8_e4m3fn_table() -> np.ndarray:
    """Value of every byte under OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa.

    Exponent 0 is subnormal (m * 2**-9); byte 0x7F / 0xFF is NaN; no infinities,
    so the largest finite magnitude is 1.75 * 2**8 = 448.
    """
    vals = np.empty(256, dtype=np.float64)
    for b in range(256):
        sign = -1.0 if (b >> 7) & 1 else 1.0
        e = (b >> 3) & 0xF
        m = b & 0x7
        if e == 0xF and m == 0x7:
            vals[b] = np.nan
        elif e == 0:
            vals[b] = sign * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            vals[b] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_FP8_TABLE = _fp8_e4m3fn_table()


def decode_bits(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Raw element bits -> float64, exactly."""
    bits = np.asarray(bits)
    if dtype == F16:
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    if dtype == BF16:
        # a bfloat16 is the upper half of a float32
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == FP8:
        return _FP8_TABLE[bits.astype(np.uint8)]
    raise ValueError(dtype)


def dequant_fp8(bits: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """fp8 bits times their float32 scale, the product rounded to float32."""
    v = decode_bits(bits, FP8).astype(np.float32)        # exact: e4m3 fits in float32
    return (v * np.asarray(scale, dtype=np.float32)).astype(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# paging
# ----------------------------------------------------------------------------
def gather_sequence(pool, table_row: np.ndarray, L: int, block_size: int) -> np.ndarray:
    """Contiguous [L][Hkv][D] raw rows of one sequence, read through its table."""
    n = -(-L // block_size)
    ids = np.asarray(table_row[:n], dtype=np.int64)
    blocks = np.asarray(pool[ids])                           # [n][Hkv][bs][D]
    rows = blocks.transpose(0, 2, 1, 3).reshape(n * block_size, blocks.shape[1], blocks.shape[3])
    return rows[:L]


def gather_scales(scales: np.ndarray, table_row: np.ndarray, L: int, block_size: int) -> np.ndarray:
    """Per-token [L][Hkv] float32 scale of an fp8 sequence."""
    n = -(-L // block_size)
    ids = np.asarray(table_row[:n], dtype=np.int64)
    per_block = np.asarray(scales)[ids]                      # [n][Hkv]
    return np.repeat(per_block, block_size, axis=0)[:L]


def sequence_kv(pool, scales, table_row, L, block_size, kv_dtype) -> np.ndarray:
    raw = gather_sequence(pool, table_row, L, block_size)
    if kv_dtype == FP8:
        sc = gather_scales(scales, table_row, L, block_size)
        return dequant_fp8(raw, sc[:, :, None])
    return decode_bits(raw, kv_dtype)


# ----------------------------------------------------------------------------
# attention on contiguous history
# ----------------------------------------------------------------------------
def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
           return_weights: bool = False):
    """Softmax attention of Q query rows that sit at the END of an L-token history.

    q: [Q][Hq][D]; K, V: [L][Hkv][D] (float64).  Row r is at position
    L - Q + r and sees keys 0 .. L - Q + r.  Returns out [Q][Hq][D] (and the
    weights [Q][Hq][L], zero where masked, if asked).
    """
    Q, Hq, D = q.shape
    L, Hkv, _ = K.shape
    G = Hq // Hkv
    out = np.zeros((Q, Hq, D), dtype=np.float64)
    weights = np.zeros((Q, Hq, L), dtype=np.float64) if return_weights else None
    for r in range(Q):
        pos = L - Q + r
        for h in range(Hq):
            g = h // G
            s = scale * (K[:pos + 1, g, :] @ q[r, h, :])     # [pos+1]
            m = s.max()
            w = np.exp(s - m)
            out[r, h, :] = (w @ V[:pos + 1, g, :]) / w.sum()
            if return_weights:
                weights[r, h, :pos + 1] = w / w.sum()
    return (out, weights) if return_weights else out


def paged_attention(q_bits: np.ndarray, k_pool, v_pool, block_tables: np.ndarray,
                    context_lens: np.ndarray, query_lens: np.ndarray, scale,
                    block_size: int, kv_dtype: str, q_dtype: str,
                    k_scale: Optional[np.ndarray] = None, v_scale: Optional[np.ndarray] = None,
                    seqs: Optional[Iterable[int]] = None,
                    heads: Optional[Sequence[int]] = None) -> Dict[int, np.ndarray]:
    """Output rows of the selected sequences: {seq: [Q_i][Hq][D] float64}.

    ``heads`` restricts the work to some query heads (the other heads of the
    returned array are NaN).
    """
    starts = np.concatenate([[0], np.cumsum(np.asarray(query_lens, dtype=np.int64))])
    scale64 = float(np.float32(scale))
    sel = range(len(context_lens)) if seqs is None else seqs
    result = {}
    for i in sel:
        L, Q = int(context_lens[i]), int(query_lens[i])
        K = sequence_kv(k_pool, k_scale, block_tables[i], L, block_size, kv_dtype)
        V = sequence_kv(v_pool, v_scale, block_tables[i], L, block_size, kv_dtype)
        qi = decode_bits(q_bits[starts[i]:starts[i] + Q], q_dtype)
        if heads is None:
            result[i] = attend(qi, K, V, scale64)
        else:
            Hq, Hkv = qi.shape[1], K.shape[1]
            G = Hq // Hkv
            o = np.full(qi.shape, np.nan)
            for h in heads:
                g = h // G
                o[:, h:h + 1] = attend(qi[:, h:h + 1], K[:, g:g + 1], V[:, g:g + 1], scale64)
            result[i] = o
    return result


# ----------------------------------------------------------------------------
# the append
# ----------------------------------------------------------------------------
def kv_append(pool, new_rows: np.ndarray, slot_mapping: np.ndarray, block_size: int):
    """Write raw row ``new_rows[r]`` ([Hkv][D]) into slot ``slot_mapping[r]`` of a copy of ``pool``.

    Slot s names block s // block_size, offset s % block_size; s < 0 skips the row.
    """
    out = pool.copy()
    for r, s in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if s < 0:
            continue
        out[int(s // block_size), :, int(s % block_size), :] = new_rows[r]
    return out


# ----------------------------------------------------------------------------
# fp8 quantisation on append
# ----------------------------------------------------------------------------
def quantize_e4m3(x) -> np.ndarray:
    """float32 values -> OCP E4M3FN bytes: nearest representable value, ties to the
    even code (even mantissa), magnitudes beyond 448 saturate to +-448, NaN -> 0x7F."""
    x = np.asarray(x, dtype=np.float32)
    codes = np.arange(0x7F)                                   # finite non-negative codes
    vals = _FP8_TABLE[codes].astype(np.float64)               # increasing
    a = np.abs(x.astype(np.float64)).ravel()
    hi = np.searchsorted(vals, a, side="left")                # first value >= a
    hi = np.minimum(hi, len(vals) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(codes[lo] % 2 == 0, lo, hi)))
    pick = np.where(vals[hi] == a, hi, pick)
    pick = np.where(a >= 448.0, 0x7E, pick)
    out = codes[pick].astype(np.uint8)
    out = np.where(np.signbit(x.ravel()), out | 0x80, out).astype(np.uint8)
    out = np.where(np.isnan(x.ravel()), np.uint8(0x7F), out)
    return out.reshape(x.shape)


def kv_append_quant(pool, scales, new_rows: np.ndarray, new_dtype: str,
                    slot_mapping: np.ndarray, block_size: int, new_block_scale=None):
    """Append 16-bit rows into an fp8 pool (copies of pool and scales are returned).

    First, every block whose slot 0 is written takes ``new_block_scale[h]`` as its
    scale (if given).  Then each row r with slot s >= 0 is divided, in float32, by
    the scale of its block and head and quantised with :func:`quantize_e4m3`.
    """
    out = pool.copy()
    sc = np.array(scales, dtype=np.float32, copy=True)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    if new_block_scale is not None:
        init = np.asarray(new_block_scale, dtype=np.float32)
        for s in slots:
            if s >= 0 and s % block_size == 0:
                sc[s // block_size, :] = init
    for r, s in enumerate(slots):
        if s < 0:
            continue
        blk, off = int(s // block_size), int(s % block_size)
        x = decode_bits(new_rows[r], new_dtype).astype(np.float32)          # [Hkv][D], exact
        q = (x / sc[blk][:, None]).astype(np.float32)                         # float32 division
        out[blk, :, off, :] = quantize_e4m3(q)
    return out, sc


# ----------------------------------------------------------------------------
# split-context partitions and their merge
# ----------------------------------------------------------------------------
def partition_partials(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                       part_tokens: int) -> List[Tuple[np.ndarray, np.ndarray, np.ndarray]]:
    """Decode (one query row) over each run of ``part_tokens`` keys separately.

    Returns, per partition, (m [Hq], l [Hq], o_unnormalised [Hq][D]) with
    m = max score, l = sum exp(s - m), o = sum exp(s - m) * v.
    """
    Hq, D = q.shape
    L, Hkv, _ = K.shape
    G = Hq // Hkv
    parts = []
    for start in range(0, L, part_tokens):
        stop = min(L, start + part_tokens)
        m = np.empty(Hq)
        l = np.empty(Hq)
        o = np.empty((Hq, D))
        for h in range(Hq):
            g = h // G
            s = scale * (K[start:stop, g, :] @ q[h])
            m[h] = s.max()
            w = np.exp(s - m[h])
            l[h] = w.sum()
            o[h] = w @ V[start:stop, g, :]
        parts.append((m, l, o))
    return parts


def lse_merge(parts) -> np.ndarray:
    """Combine partition states: M = max m_p; out = sum e^(m_p-M) o_p / sum e^(m_p-M) l_p."""
    M = np.max(np.stack([p[0] for p in parts]), axis=0)
    num = sum(np.exp(p[0] - M)[:, None] * p[2] for p in parts)
    den = sum(np.exp(p[0] - M) * p[1] for p in parts)
    return num / den[:, None]


# ----------------------------------------------------------------------------
# KV sizing
# ----------------------------------------------------------------------------
def kv_bytes_per_token(layers: int, hidden: int, bytes_per_value: int) -> int:
    """One key and one value of ``hidden`` numbers in every layer."""
    return 2 * layers * hidden * bytes_per_value


def tolerance_ok(got: np.ndarray, ref: np.ndarray, atol: float, rtol: float) -> np.ndarray:
    """Element-wise pass mask |got - ref| <= atol + rtol * |ref| (NaN fails)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return np.abs(got - ref) <= atol + rtol * np.abs(ref)
