"""CPU oracle for paged GQA decode attention over compressed pages plus a BF16 tail.

TEST INFRASTRUCTURE ONLY (see oracle/codec.py for who may import it).

What it follows:
  * "GAAC: ...", section "Attention with On-the-Fly Decompression": attention reads compressed
    blocks and rebuilds the BF16 values; compressed blocks and the uncompressed tail take part
    in one and the same softmax, so the result is the original attention formula;
  * "GAAC: ...", section "Block-Wise Compression Scheduling": new tokens live in an uncompressed
    BF16 tail until their page completes;
  * "ZipFusion: ...", "How it works": the stored BF16 values are rebuilt exactly.
The attention itself is the plain definition, computed in float64:
    s_t = sm_scale * sum_d q[h, d] * K[t, g, d],   g = h // (Hq / Hkv),
    o[h, :] = sum_t exp(s_t - max s) V[t, g, :] / sum_t exp(s_t - max s).

Readings: query head h uses KV head h // (Hq/Hkv); the scale is passed in;
tokens 0 .. 16*n_comp-1 come from compressed pages via the block table, the remaining
seq_len - 16*n_comp (0..16) from the tail; a sequence of length 0 gives an all-zero output row.
NaN and Inf are carried by IEEE float64 arithmetic.

Pins (tests/test_oracle_attention.py): pure-Python brute force on tiny inputs, torch's
scaled_dot_product_attention in float64 on CPU, and closed forms (q = 0 gives the mean of V,
constant V gives that V, one dominant logit gives that token's V, one token gives its V).
softmax_weights_fp64 (the weights alone, used to report how many keys a test's softmax really
spreads over) is pinned by closed forms (q = 0 gives 1/T each, a dominant logit gives one-hot)
and by the brute-force weights.
"""
from __future__ import annotations

import numpy as np

from . import codec


def attention_fp64(q_bits, k_bits, v_bits, sm_scale: float) -> np.ndarray:
    """One sequence.  q_bits [Hq, D], k_bits/v_bits [T, Hkv, D] (BF16 bit patterns).

    Returns float64 [Hq, D]."""
    q = codec.bf16_bits_to_f64(q_bits)
    k = codec.bf16_bits_to_f64(k_bits)
    v = codec.bf16_bits_to_f64(v_bits)
    return attention_values_fp64(q, k, v, sm_scale)


def attention_values_fp64(q, k, v, sm_scale: float) -> np.ndarray:
    """The same definition on values: q [Hq, D], k/v [T, Hkv, D] float64.  Returns [Hq, D]."""
    hq, d = q.shape
    t, hkv, _ = k.shape
    out = np.zeros((hq, d), dtype=np.float64)
    if t == 0:
        return out
    group = hq // hkv
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        for h in range(hq):
            g = h // group
            s = sm_scale * (k[:, g, :] @ q[h])          # [T]
            m = np.max(s)
            p = np.exp(s - m)
            out[h] = (p @ v[:, g, :]) / np.sum(p)
    return out


def softmax_weights_fp64(q_bits, k_bits, sm_scale: float) -> np.ndarray:
    """The softmax weights of one sequence: q_bits [Hq, D], k_bits [T, Hkv, D] (BF16 bit
    patterns) -> float64 [Hq, T], w[h, t] = exp(s_t - max s) / sum_t exp(s_t - max s) with the
    scores s_t of the definition above."""
    q = codec.bf16_bits_to_f64(q_bits)
    k = codec.bf16_bits_to_f64(k_bits)
    hq = q.shape[0]
    t, hkv, _ = k.shape
    w = np.zeros((hq, t), dtype=np.float64)
    if t == 0:
        return w
    group = hq // hkv
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        for h in range(hq):
            s = sm_scale * (k[:, h // group, :] @ q[h])
            p = np.exp(s - np.max(s))
            w[h] = p / np.sum(p)
    return w


def gather_sequence(arena, meta_table, block_table_row, n_comp: int, tail_b, n_tail: int):
    """K and V of one sequence in token order, as BF16 bit patterns [T, Hkv, 128].

    meta_table[phys][g][kind] = (off, tags).  tail_b: uint16 [2, Hkv, 16, 128] or None.
    """
    hkv = len(meta_table[0]) if len(meta_table) else tail_b.shape[1]
    t_total = codec.PAGE_TOKENS * n_comp + n_tail
    k = np.zeros((t_total, hkv, codec.HEAD_DIM), dtype=np.uint16)
    v = np.zeros_like(k)
    for p in range(n_comp):
        phys = int(block_table_row[p])
        rows = slice(codec.PAGE_TOKENS * p, codec.PAGE_TOKENS * (p + 1))
        for g in range(hkv):
            off_k, tags_k = meta_table[phys][g][codec.KIND_K]
            off_v, tags_v = meta_table[phys][g][codec.KIND_V]
            k[rows, g, :] = codec.decode_group(arena, off_k, tags_k, codec.KIND_K)
            v[rows, g, :] = codec.decode_group(arena, off_v, tags_v, codec.KIND_V)
    if n_tail:
        base = codec.PAGE_TOKENS * n_comp
        k[base:, :, :] = np.transpose(tail_b[0, :, :n_tail, :], (1, 0, 2))
        v[base:, :, :] = np.transpose(tail_b[1, :, :n_tail, :], (1, 0, 2))
    return k, v


def decode_attention(q_bits, arena, meta_table, block_table, seq_lens, n_comp_pages, tail,
                     sm_scale: float, batch_indices=None) -> np.ndarray:
    """Batched decode attention.  q_bits [B, Hq, 128]; block_table [B, max_pages];
    tail uint16 [B, 2, Hkv, 16, 128] or None.  Returns float64 [B, Hq, 128] (rows of batch
    entries not in batch_indices stay zero)."""
    q_bits = np.asarray(q_bits, dtype=np.uint16)
    bsz = q_bits.shape[0]
    out = np.zeros(q_bits.shape, dtype=np.float64)
    for b in (range(bsz) if batch_indices is None else batch_indices):
        n_comp = int(n_comp_pages[b])
        n_tail = int(seq_lens[b]) - codec.PAGE_TOKENS * n_comp
        if not 0 <= n_tail <= codec.PAGE_TOKENS:
            raise ValueError("seq_len - 16*n_comp_pages must lie in [0, 16]")
        if n_tail and tail is None:
            raise ValueError("tokens past the compressed pages need a tail")
        k, v = gather_sequence(arena, meta_table, block_table[b], n_comp,
                               None if tail is None else tail[b], n_tail)
        out[b] = attention_fp64(q_bits[b], k, v, sm_scale)
    return out
