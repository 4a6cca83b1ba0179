"""Plain float64 CPU oracle for single-token decode attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: it is used by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``, and by nothing else.  It shares
no code, tables or helpers with the HIP library; both sides only see the same
seeded inputs.

What it computes (every function is the plain definition, written out):

* Decode attention for one new query per sequence: every query head reads the
  whole accumulated K/V of its sequence and returns softmax(scale * q K^T) V
  ("Why prefill and decode are opposite problems" on the page "The
  signature-dish specialist: vLLM's attention backend"; the attention kernel of
  §2.2 "Scaling Long-Context Decoding" in the KernelFlume paper,
  academ.us/article/2606.29207).
* The K/V rows are not contiguous: logical block i of a sequence holds tokens
  16i .. 16i+15 and lives in whatever physical frame the block table names;
  the kernel gathers over the physical blocks ("Distributed Paged KV-Cache
  Tiering and Memory Layout" and "Physical Memory Block Layout" on the page
  "Disaggregated Inference Architecture: Paged KV-Cache Tiering, Chunked
  Prefill, and Asynchronous Overlap"; "How the backend reads the paged KV" on
  the vLLM attention-backend page).
* Grouped-query attention: several query heads share one KV head (KernelFlume
  paper §6.3, the Q32:KV8 style ratios, and H_kv in §4.2).
* Partials over contiguous token ranges of one sequence, returned as a
  normalised output and a log-sum-exp, and their merge by the associative
  online-softmax reduction, which equals attention over the full range
  (KernelFlume paper §3.1 "Kernel-level Disaggregation", §3.2 "Workflow of
  Elastic Decoding", §5.1 "Query-First Attention"; the (m, l, O) update
  equations of "Mathematical Formulation of Chunked Attention" on the
  disaggregated-inference page).

Readings where the pages leave a step open (each one is listed with its reason
in the design notes of the repository):

* Pool layout ``[num_blocks, block_size, H_kv, D]`` with D contiguous, separate
  K and V pools: the block-stride formula B_size * H_KV * D * sizeof(dtype) of
  "Physical Memory Block Layout" makes a block hold all KV heads of its tokens.
* Query head h uses KV head h // G with G = H_q / H_kv (contiguous groups).
* ``context_lens[b]`` counts every cached token, the one being decoded
  included (the tail node appends (K_new, V_new) before it attends).
* ``scale`` is an fp32 value multiplying the raw dot product; the oracle uses
  its exact float64 value.  Exponentials are natural; ``lse`` is in nats.
* A partial is (o, lse) with o normalised; an empty range gives o = 0 and
  lse = -inf, and the merge ignores such partials.
* Split-K partition p of a sequence with n tokens covers tokens
  [p*P, min((p+1)*P, n)).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "token_location",
    "gather_sequence",
    "attend",
    "kv_head_of",
    "paged_decode_attention",
    "partial_attention",
    "merge_partials",
    "partition_ranges",
    "split_k_partials",
    "kv_append",
    "fp8_e4m3_value",
    "fp8_e4m3_decode",
    "fp8_e4m3_encode",
    "kv_append_fp8",
    "paged_decode_attention_fp8",
    "kv_cache_bytes",
]


def token_location(block_table_row, t, block_size=16):
    """Physical (frame, slot) of logical token ``t`` of one sequence.

    Logical block i holds tokens i*block_size .. i*block_size+block_size-1 and
    maps to the physical frame ``block_table_row[i]`` (figure "Virtual
    Sequence Address Space" in "Distributed Paged KV-Cache Tiering and Memory
    Layout", disaggregated-inference page).
    """
    return int(block_table_row[t // block_size]), int(t % block_size)


def blocks_needed(n_tokens, block_size=16):
    """Number of blocks a sequence of ``n_tokens`` occupies: ceil(n / bs).

    Same count as the allocator listing in "Physical Memory Block Layout"
    (disaggregated-inference page) uses when it reserves frames.
    """
    return -(-int(n_tokens) // int(block_size))


def gather_sequence(pool, block_table_row, n_tokens, kv_head, block_size=16):
    """Rows 0..n_tokens-1 of one KV head of one sequence, in logical order.

    ``pool`` is ``[num_blocks, block_size, H_kv, D]`` (fp16 or any float);
    returns float64 ``[n_tokens, D]``.  Token t is read from frame
    ``block_table_row[t // bs]`` at slot ``t % bs``; nothing past the last valid
    token of the last block is read.
    """
    D = pool.shape[3]
    out = np.empty((int(n_tokens), D), dtype=np.float64)
    for t in range(int(n_tokens)):
        frame, slot = token_location(block_table_row, t, block_size)
        out[t] = pool[frame, slot, kv_head, :]
    return out


def _gather_sequence_blocks(pool, block_table_row, n_tokens, kv_head, block_size):
    """Same rows as ``gather_sequence``, copied one whole block at a time.

    Used for long sequences where a per-token Python loop is too slow; the
    equality of the two is itself one of the oracle's self-checks.
    """
    D = pool.shape[3]
    n_tokens = int(n_tokens)
    out = np.empty((n_tokens, D), dtype=np.float64)
    for i in range(blocks_needed(n_tokens, block_size)):
        lo = i * block_size
        hi = min(lo + block_size, n_tokens)
        out[lo:hi] = pool[int(block_table_row[i]), : hi - lo, kv_head, :]
    return out


def attend(q_rows, K, V, scale):
    """softmax(scale * q K^T) V for each row of ``q_rows``, in float64.

    q_rows ``[G, D]``, K and V ``[n, D]``.  Returns (o ``[G, D]``, lse ``[G]``)
    with lse = m + ln(sum_t exp(s_t - m)), the natural log-sum-exp of the
    scaled scores.  n = 0 gives o = 0 and lse = -inf.  Two passes: all scores
    first, then max, exponentials, sum and the weighted sum of V.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    G, D = q_rows.shape
    if K.shape[0] == 0:
        return np.zeros((G, D)), np.full(G, -np.inf)
    s = float(np.float32(scale)) * (q_rows @ K.T)          # [G, n]
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    l = w.sum(axis=1, keepdims=True)
    o = (w @ V) / l
    lse = m[:, 0] + np.log(l[:, 0])
    return o, lse


def kv_head_of(h, n_q_heads, n_kv_heads):
    """KV head read by query head h: contiguous groups of G = H_q / H_kv."""
    return h // (n_q_heads // n_kv_heads)


def paged_decode_attention(q, k_pool, v_pool, block_table, context_lens, scale,
                           block_size=16, per_block_gather=True):
    """Decode attention of every sequence over its paged K/V.

    q ``[B, H_q, D]``; k_pool, v_pool ``[num_blocks, block_size, H_kv, D]``;
    block_table int ``[B, >= ceil(max ctx / bs)]``; context_lens int ``[B]``.
    Returns (out float64 ``[B, H_q, D]``, lse float64 ``[B, H_q]``).
    Query head h attends with KV head ``kv_head_of(h, H_q, H_kv)``.
    """
    q = np.asarray(q)
    B, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    assert Hq % Hkv == 0, "H_q must be a multiple of H_kv"
    gather = _gather_sequence_blocks if per_block_gather else gather_sequence
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        n = int(context_lens[b])
        kv = {}
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            if g not in kv:
                kv[g] = (gather(k_pool, block_table[b], n, g, block_size),
                         gather(v_pool, block_table[b], n, g, block_size))
            K, V = kv[g]
            o, l = attend(q[b, h:h + 1], K, V, scale)
            out[b, h], lse[b, h] = o[0], l[0]
    return out, lse


def partial_attention(q, k_pool, v_pool, block_table_slice, range_lens, scale,
                      block_size=16):
    """(o, lse) over one contiguous token range of each sequence.

    The range is described the way a node that owns it would see it: the
    columns of the block table that cover the range and the number of tokens
    in it (KernelFlume paper §3.1 and §3.2: a node computes local attention
    over the token range it stores and returns its partial).  Because o is
    normalised, this is attention over the range itself.
    """
    return paged_decode_attention(q, k_pool, v_pool, block_table_slice, range_lens,
                                  scale, block_size)


def merge_partials(o_parts, lse_parts):
    """Merge R partials (o_r normalised, lse_r) into attention over their union.

    o_parts ``[R, ..., D]``, lse_parts ``[R, ...]``.  With L = max_r lse_r and
    w_r = exp(lse_r - L): lse = L + ln(sum_r w_r) and o = sum_r w_r o_r /
    sum_r w_r.  This is the online-softmax merge of the (m, l, O) equations
    in "Mathematical Formulation of Chunked Attention" (disaggregated-inference
    page) written for normalised partials, and the merge of (o_i, m_i, l_i)
    on the weight node (KernelFlume paper §3.2, §5.1).  Partials with
    lse = -inf (empty ranges) carry no weight; if all are empty the result is
    o = 0, lse = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    L = lse_parts.max(axis=0)
    empty = np.isneginf(L)
    L_safe = np.where(empty, 0.0, L)
    w = np.exp(lse_parts - L_safe[None])                      # exp(-inf) = 0
    wsum = w.sum(axis=0)
    wsum_safe = np.where(empty, 1.0, wsum)
    o = (w[..., None] * o_parts).sum(axis=0) / wsum_safe[..., None]
    lse = np.where(empty, -np.inf, L_safe + np.log(wsum_safe))
    o = np.where(empty[..., None], 0.0, o)
    return o, lse


def partition_ranges(n_tokens, partition_tokens):
    """Split-K partitions of one sequence: [p*P, min((p+1)*P, n)) for p < ceil(n/P).

    The KV of a sequence is cut into contiguous token ranges that are computed
    independently (KernelFlume paper §3.1, and §8 where KV is partitioned by
    sequence ranges).
    """
    n = int(n_tokens)
    P = int(partition_tokens)
    return [(p * P, min((p + 1) * P, n)) for p in range(-(-n // P))]


def split_k_partials(q, k_pool, v_pool, block_table, context_lens, scale,
                     partition_tokens, block_size=16):
    """Per-partition partials of every (sequence, query head).

    Returns (o ``[B, H_q, max_parts, D]``, lse ``[B, H_q, max_parts]``), where
    max_parts = max_b ceil(ctx_b / P); partitions past a sequence's end are
    o = 0, lse = -inf.  Partition boundaries are integers and exact.
    """
    q = np.asarray(q)
    B, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    P = int(partition_tokens)
    assert P % block_size == 0
    max_parts = max([len(partition_ranges(int(n), P)) for n in context_lens] + [0])
    o = np.zeros((B, Hq, max_parts, D))
    lse = np.full((B, Hq, max_parts), -np.inf)
    for b in range(B):
        n = int(context_lens[b])
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            K = _gather_sequence_blocks(k_pool, block_table[b], n, g, block_size)
            V = _gather_sequence_blocks(v_pool, block_table[b], n, g, block_size)
            for p, (lo, hi) in enumerate(partition_ranges(n, P)):
                op, lp = attend(q[b, h:h + 1], K[lo:hi], V[lo:hi], scale)
                o[b, h, p], lse[b, h, p] = op[0], lp[0]
    return o, lse


def kv_append(k_pool, v_pool, k_new, v_new, block_table, context_lens, block_size=16):
    """Write each sequence's newest token into its paged K/V cache.

    ``context_lens[b]`` already counts the new token, so it is token
    t = ctx_b - 1, stored in frame ``block_table[b, t // bs]`` at slot
    ``t % bs``: the tail node appends (K_new, V_new) before attending
    (KernelFlume paper §3.2, §5.1; logical block -> frame mapping of
    "Distributed Paged KV-Cache Tiering and Memory Layout" on the
    disaggregated-inference page).  k_new, v_new: ``[B, H_kv, D]``.
    Sequences with ctx_b = 0 are left alone.  Returns new pools (copies).
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    for b, n in enumerate(context_lens):
        n = int(n)
        if n <= 0:
            continue
        frame, slot = token_location(block_table[b], n - 1, block_size)
        k_out[frame, slot] = k_new[b]
        v_out[frame, slot] = v_new[b]
    return k_out, v_out


def fp8_e4m3_value(code):
    """Value of one FP8 E4M3 code (the OCP 8-bit format: 1 sign bit, 4
    exponent bits with bias 7, 3 mantissa bits; exponent 0 is subnormal,
    m * 2^-9; the codes S.1111.111 are NaN; there are no infinities).

    The FP8 KV cache of "4. Quantised KV cache" in "Optimising decode in vLLM"
    (and the kv_cache_dtype knob of the vLLM attention-backend page) stores
    one such code per element next to a per-tensor scale.
    """
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def fp8_e4m3_decode(codes):
    """Element-wise fp8_e4m3_value of a uint8 array, as float64."""
    table = np.array([fp8_e4m3_value(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def fp8_e4m3_encode(x):
    """E4M3 code (uint8) of each value: the nearest finite E4M3 value, ties to
    the even code (the one whose mantissa ends in 0, as in round-to-nearest-
    even); the sign of zero is kept; NaN gives 0x7F with its sign; magnitudes
    at or above the largest finite value, 448, saturate to +-448.

    Saturation is a reading: the format leaves out-of-range conversion open,
    and a NaN written into a KV cache would poison every attention over it.
    """
    x = np.asarray(x, dtype=np.float64)
    pos = fp8_e4m3_decode(np.arange(0x7F))          # codes 0x00 .. 0x7E: 0 .. 448, increasing
    a = np.abs(x)
    i = np.clip(np.searchsorted(pos, a), 1, 0x7E)    # pos[i-1] < a <= pos[i] inside the range
    lo, hi = pos[i - 1], pos[i]
    up = (hi - a < a - lo) | ((hi - a == a - lo) & (i % 2 == 0))
    code = np.where(up, i, i - 1)
    code = np.where(a >= 448.0, 0x7E, code)
    sign = np.signbit(x).astype(np.int64) << 7
    code = np.where(np.isnan(x), 0x7F, code) | sign
    return code.astype(np.uint8)


def kv_append_fp8(k_codes, v_codes, k_new, v_new, block_table, context_lens, k_scale, v_scale,
                  block_size=16):
    """kv_append into FP8 E4M3 pools: the new rows are quantised to
    fp8_e4m3_encode(fp32(x) * fp32(1 / scale)) with the tensor's scale (the
    product and the reciprocal rounded to fp32), so that scale * value(code)
    is the stored approximation of x (the FP8 KV cache of "4. Quantised KV
    cache" in "Optimising decode in vLLM", one scale per tensor)."""
    inv_k = np.float32(1.0) / np.float32(k_scale)
    inv_v = np.float32(1.0) / np.float32(v_scale)
    kq = fp8_e4m3_encode(np.asarray(k_new, dtype=np.float32) * inv_k)
    vq = fp8_e4m3_encode(np.asarray(v_new, dtype=np.float32) * inv_v)
    return kv_append(k_codes, v_codes, kq, vq, block_table, context_lens, block_size)


def paged_decode_attention_fp8(q, k_codes, v_codes, block_table, context_lens, scale, k_scale,
                               v_scale, block_size=16):
    """Decode attention over an FP8 E4M3 paged cache with per-tensor scales.

    Stored code c of K means k_scale * value(c), of V v_scale * value(c).  Each
    sequence's rows are gathered through the block table, decoded and scaled in
    float64, then attended exactly as in paged_decode_attention.
    """
    q = np.asarray(q)
    B, Hq, D = q.shape
    Hkv = k_codes.shape[2]
    assert Hq % Hkv == 0
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        n = int(context_lens[b])
        kv = {}
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            if g not in kv:
                kc = _gather_sequence_blocks(k_codes, block_table[b], n, g, block_size)
                vc = _gather_sequence_blocks(v_codes, block_table[b], n, g, block_size)
                kv[g] = (float(k_scale) * fp8_e4m3_decode(kc.astype(np.uint8)),
                         float(v_scale) * fp8_e4m3_decode(vc.astype(np.uint8)))
            K, V = kv[g]
            o, l = attend(q[b, h:h + 1], K, V, scale)
            out[b, h], lse[b, h] = o[0], l[0]
    return out, lse


def kv_cache_bytes(seq_lens, n_kv_heads, head_dim, n_layers, bytes_per_elem=2):
    """KV footprint sum_i 2 * s_i * H_kv * d_h * L * bytes (KernelFlume paper §4.2).

    The same count gives M_KV = 2 * N_L * H_KV * S * D * 1 B for one FP8
    request ("Anatomy of Prefill-Decode Disaggregation", disaggregated-inference
    page).
    """
    return sum(2 * int(s) * n_kv_heads * head_dim * n_layers * bytes_per_elem
               for s in seq_lens)
