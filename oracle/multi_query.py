"""Plain float64 CPU oracle for multi-query and shared-prefix (cascade) attention
over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: it is used by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``, and by nothing else.  It shares
no code with the HIP library.

What it computes (each function is the plain definition, written out):

* Several query tokens of one sequence attending to its paged K/V at once: a
  prefill chunk, whose queries see every earlier chunk without a mask and the
  current chunk through a causal mask ("Mathematical Formulation of Chunked
  Attention" on the page "Disaggregated Inference Architecture: Paged
  KV-Cache Tiering, Chunked Prefill, and Asynchronous Overlap"), or the tokens
  a draft model proposed, which the verifier checks in one forward pass
  (knob 3, speculative decoding, of the post "Optimising decode in vLLM:
  squeezing every token out of small hardware").
* Cascade attention for requests that share a prefix: attention over the
  shared prefix once for all of them, then over each request's own suffix,
  the two combined; the result is attention over prefix + suffix ("What
  FlashInfer brings: JIT and cascade attention" on the page "The
  signature-dish specialist: vLLM's attention backend").

Readings where the pages leave a step open:

* The queries of sequence s are rows ``query_start[s] .. query_start[s+1]-1``
  of q, in position order, and they are the LAST n_q tokens of the sequence:
  ``context_lens[s]`` = n counts them (their K/V are already in the cache, as
  for single-token decode).  With the causal mask, query i (0-based) sits at
  position n - n_q + i and sees tokens 0 .. n - n_q + i.  For chunk k of a
  prompt cut into chunks of C tokens this is the page's split: tokens of
  earlier chunks unmasked, tokens of the current chunk up to and including
  the query's own position.  Without the mask every query sees all n tokens.
* n_q > n leaves the first n_q - n queries with nothing to see: their output
  is 0 and their lse is -inf (the convention for empty ranges).
* A cascade group is a run of adjacent requests: requests
  ``group_start[r] .. group_start[r+1]-1`` share prefix r, which is
  ``prefix_lens[r]`` tokens of block-table row r; request b continues with
  ``suffix_lens[b]`` tokens of its own suffix block table.
"""
from __future__ import annotations

import numpy as np

from .paged_attention import _gather_sequence_blocks, attend, kv_head_of

__all__ = [
    "visible_tokens",
    "multi_query_attention",
    "cascade_attention",
    "cascade_read_tokens",
]


def visible_tokens(n_tokens, n_queries, i, causal):
    """How many leading tokens query i of the last n_queries of a sequence sees."""
    if not causal:
        return int(n_tokens)
    return max(0, int(n_tokens) - int(n_queries) + int(i) + 1)


def multi_query_attention(q, k_pool, v_pool, block_table, context_lens, query_start, scale,
                          causal=True, block_size=16):
    """Attention of every query token of every sequence over its paged K/V.

    q ``[T, H_q, D]`` (T = query_start[-1]); k_pool, v_pool
    ``[num_blocks, block_size, H_kv, D]``; block_table int ``[S, width]``;
    context_lens int ``[S]``; query_start int ``[S + 1]``, non-decreasing from
    0.  Returns (out float64 ``[T, H_q, D]``, lse float64 ``[T, H_q]``).
    """
    q = np.asarray(q)
    T, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    S = len(context_lens)
    assert int(query_start[0]) == 0 and int(query_start[S]) == T
    out = np.zeros((T, Hq, D))
    lse = np.full((T, Hq), -np.inf)
    for s in range(S):
        n = int(context_lens[s])
        q0, q1 = int(query_start[s]), int(query_start[s + 1])
        n_q = q1 - q0
        if n_q == 0:
            continue
        for g in range(Hkv):
            K = _gather_sequence_blocks(k_pool, block_table[s], n, g, block_size)
            V = _gather_sequence_blocks(v_pool, block_table[s], n, g, block_size)
            heads = [h for h in range(Hq) if kv_head_of(h, Hq, Hkv) == g]
            for i in range(n_q):
                vis = visible_tokens(n, n_q, i, causal)
                o, l = attend(q[q0 + i, heads], K[:vis], V[:vis], scale)
                out[q0 + i, heads], lse[q0 + i, heads] = o, l
    return out, lse


def cascade_attention(q, k_pool, v_pool, prefix_table, prefix_lens, group_start, suffix_table,
                      suffix_lens, scale, block_size=16):
    """Decode attention of requests whose context is a shared prefix then a suffix.

    q ``[B, H_q, D]``: one decode query per request; prefix_table int
    ``[R, width]``, prefix_lens ``[R]``; group_start ``[R + 1]`` (requests of
    group r are group_start[r] .. group_start[r+1]-1, group_start[R] = B);
    suffix_table ``[B, width]``, suffix_lens ``[B]``.  Request b attends over
    the prefix tokens of its group followed by its own suffix tokens.  Returns
    (out ``[B, H_q, D]``, lse ``[B, H_q]``).
    """
    q = np.asarray(q)
    B, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    R = len(prefix_lens)
    assert int(group_start[0]) == 0 and int(group_start[R]) == B
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for r in range(R):
        for b in range(int(group_start[r]), int(group_start[r + 1])):
            for g in range(Hkv):
                K = np.concatenate([
                    _gather_sequence_blocks(k_pool, prefix_table[r], prefix_lens[r], g, block_size),
                    _gather_sequence_blocks(k_pool, suffix_table[b], suffix_lens[b], g, block_size)])
                V = np.concatenate([
                    _gather_sequence_blocks(v_pool, prefix_table[r], prefix_lens[r], g, block_size),
                    _gather_sequence_blocks(v_pool, suffix_table[b], suffix_lens[b], g, block_size)])
                heads = [h for h in range(Hq) if kv_head_of(h, Hq, Hkv) == g]
                o, l = attend(q[b, heads], K, V, scale)
                out[b, heads], lse[b, heads] = o, l
    return out, lse


def cascade_read_tokens(prefix_len, suffix_lens):
    """Tokens of K/V read: (naive, cascade) for R requests sharing one prefix.

    Naive attention reads the prefix once per request, R * P + sum(s_i);
    cascade attention reads it once, P + sum(s_i) (the read counts of "What
    FlashInfer brings: JIT and cascade attention").
    """
    R = len(suffix_lens)
    s = int(sum(int(x) for x in suffix_lens))
    return R * int(prefix_len) + s, int(prefix_len) + s
