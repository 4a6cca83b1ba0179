"""Checks that pin the multi-query and cascade oracle to facts other than its own code.

Each ``pin_*`` takes the multi-query oracle module (or a patched copy) and the
decode oracle module, and raises AssertionError when the oracle disagrees
with something the pages or plain mathematics fix:

* the chunk positions of the chunked-attention formulation (chunk k of C
  tokens spans k*C .. (k+1)*C - 1) and the cascade read counts of the
  worked example R = 50, P = 1000 (golden fixtures with their citations);
* a dense, textbook causal attention: the full score matrix with a
  lower-triangular mask, softmax and log-sum-exp by scipy;
* the page's (m, l, O) update equations, combining attention over the earlier
  chunks (no mask) with the causal attention inside the current chunk;
* brute force with 50-digit arithmetic on a tiny causal case;
* a single query per sequence is plain decode attention; queries past the
  context see nothing;
* cascade attention equals decode attention over a block table that
  concatenates the prefix's frames and the suffix's frames, and equals the
  merge of a prefix partial and a suffix partial.
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TOL = 1e-12


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def mq_case(rng, lens, n_queries, Hq, Hkv, D, bs=16, extra_blocks=3):
    """Shuffled pool, -1 padded tables, and n_queries[s] query rows per sequence."""
    nblk = [-(-int(n) // bs) for n in lens]
    pool = sum(nblk) + extra_blocks
    perm = rng.permutation(pool)
    width = max(nblk + [1]) + 2
    table = np.full((len(lens), width), -1, dtype=np.int64)
    off = 0
    for s, k in enumerate(nblk):
        table[s, :k] = perm[off:off + k]
        off += k
    qs = np.concatenate([[0], np.cumsum(n_queries)]).astype(np.int64)
    q = rng.standard_normal((int(qs[-1]), Hq, D)).astype(np.float16)
    k = rng.standard_normal((pool, bs, Hkv, D)).astype(np.float16)
    v = rng.standard_normal((pool, bs, Hkv, D)).astype(np.float16)
    return q, k, v, table, np.asarray(lens), qs


def dense_kv(pool, table_row, n, g, bs=16):
    """Rows 0..n-1 of KV head g by fancy indexing (frame = row[t // bs], slot = t % bs)."""
    t = np.arange(int(n))
    return pool[np.asarray(table_row)[t // bs], t % bs, g, :].astype(np.float64)


def pin_chunk_positions(MQ, O):
    ex = _golden("chunked_prefill_positions.json")
    C, k = ex["chunk_tokens"], ex["chunk_index"]
    n = (k + 1) * C                                  # the chunk's K/V are cached too
    assert k * C == ex["first_query_position"] and (k + 1) * C - 1 == ex["last_query_position"]
    assert MQ.visible_tokens(n, C, 0, True) == ex["tokens_seen_by_first_query"]
    assert MQ.visible_tokens(n, C, C - 1, True) == ex["tokens_seen_by_last_query"]
    for i in (0, 1, C // 2, C - 1):
        assert MQ.visible_tokens(n, C, i, True) == k * C + i + 1
        assert MQ.visible_tokens(n, C, i, False) == n


def pin_dense_textbook(MQ, O):
    from scipy.special import logsumexp, softmax
    rng = np.random.default_rng(31)
    lens, nq = [5, 40, 70, 33], [3, 17, 1, 33]
    Hq, Hkv, D = 4, 2, 16
    q, k, v, table, lens, qs = mq_case(rng, lens, nq, Hq, Hkv, D)
    scale = 0.3
    for causal in (True, False):
        out, lse = MQ.multi_query_attention(q, k, v, table, lens, qs, scale, causal=causal)
        for s, n in enumerate(lens):
            n_q = int(qs[s + 1] - qs[s])
            pos = n - n_q + np.arange(n_q)
            mask = np.arange(n)[None, :] <= pos[:, None] if causal else np.ones((n_q, n), bool)
            for h in range(Hq):
                g = h // (Hq // Hkv)
                K, V = dense_kv(k, table[s], n, g), dense_kv(v, table[s], n, g)
                Q = q[qs[s]:qs[s + 1], h].astype(np.float64)
                Sc = float(np.float32(scale)) * Q @ K.T
                Sc = np.where(mask, Sc, -np.inf)
                P = softmax(Sc, axis=1)
                assert np.abs(out[qs[s]:qs[s + 1], h] - P @ V).max() <= TOL
                assert np.abs(lse[qs[s]:qs[s + 1], h] - logsumexp(Sc, axis=1)).max() <= TOL


def _unnormalised(Sc, V):
    """(m, l, O) of one score row without normalisation; an empty row gives (-inf, 0, 0)."""
    if Sc.size == 0:
        return -np.inf, 0.0, np.zeros(V.shape[1])
    m = Sc.max()
    w = np.exp(Sc - m)
    return m, w.sum(), w @ V


def pin_page_chunk_update(MQ, O):
    rng = np.random.default_rng(32)
    C, Hq, Hkv, D = 24, 2, 1, 8
    scale = 0.25
    for k_idx in (0, 3):
        n = (k_idx + 1) * C
        q, kp, vp, table, lens, qs = mq_case(rng, [n], [C], Hq, Hkv, D)
        out, lse = MQ.multi_query_attention(q, kp, vp, table, lens, qs, scale, causal=True)
        K, V = dense_kv(kp, table[0], n, 0), dense_kv(vp, table[0], n, 0)
        for i in range(C):
            for h in range(Hq):
                s_all = float(np.float32(scale)) * (q[i, h].astype(np.float64) @ K.T)
                m_p, l_p, O_p = _unnormalised(s_all[:k_idx * C], V[:k_idx * C])          # earlier chunks
                m_c, l_c, O_c = _unnormalised(s_all[k_idx * C:k_idx * C + i + 1],
                                              V[k_idx * C:k_idx * C + i + 1])            # causal, own chunk
                m_n = max(m_p, m_c)
                a_p, a_c = np.exp(m_p - m_n), np.exp(m_c - m_n)
                l_n = a_p * l_p + a_c * l_c
                O_n = a_p * O_p + a_c * O_c
                assert np.abs(out[i, h] - O_n / l_n).max() <= TOL
                assert abs(lse[i, h] - (m_n + np.log(l_n))) <= TOL


def pin_mpmath_causal(MQ, O):
    import mpmath
    mpmath.mp.dps = 50
    rng = np.random.default_rng(33)
    n, n_q, Hq, Hkv, D = 7, 3, 2, 1, 4
    q, k, v, table, lens, qs = mq_case(rng, [n], [n_q], Hq, Hkv, D)
    scale = 0.7
    out, lse = MQ.multi_query_attention(q, k, v, table, lens, qs, scale, causal=True)
    for i in range(n_q):
        vis = n - n_q + i + 1
        for h in range(Hq):
            rows = [(int(table[0, t // 16]), t % 16) for t in range(vis)]
            s = [mpmath.mpf(float(np.float32(scale))) *
                 mpmath.fsum(mpmath.mpf(float(q[i, h, d])) * mpmath.mpf(float(k[f, sl, 0, d]))
                             for d in range(D)) for f, sl in rows]
            w = [mpmath.exp(x) for x in s]
            den = mpmath.fsum(w)
            assert abs(float(mpmath.log(den)) - lse[i, h]) <= 1e-13
            for d in range(D):
                ref = mpmath.fsum(wi * mpmath.mpf(float(v[f, sl, 0, d]))
                                  for wi, (f, sl) in zip(w, rows)) / den
                assert abs(float(ref) - out[i, h, d]) <= 1e-13


def pin_single_query_is_decode(MQ, O):
    rng = np.random.default_rng(34)
    lens = [1, 16, 17, 100]
    q, k, v, table, lens, qs = mq_case(rng, lens, [1] * 4, 8, 2, 16)
    ref, ref_lse = O.paged_decode_attention(q, k, v, table, lens, 0.2)
    for causal in (True, False):
        out, lse = MQ.multi_query_attention(q, k, v, table, lens, qs, 0.2, causal=causal)
        assert np.abs(out - ref).max() <= TOL and np.abs(lse - ref_lse).max() <= TOL


def pin_queries_past_context(MQ, O):
    rng = np.random.default_rng(35)
    q, k, v, table, lens, qs = mq_case(rng, [3, 0, 20], [5, 2, 0], 2, 1, 8)
    out, lse = MQ.multi_query_attention(q, k, v, table, lens, qs, 0.5, causal=True)
    # sequence 0: 3 tokens, 5 queries -> the first two see nothing, the last sees all 3
    assert np.all(out[0:2] == 0) and np.all(np.isneginf(lse[0:2]))
    assert np.all(np.isfinite(lse[2:5]))
    last, last_lse = O.attend(q[4].astype(np.float64), dense_kv(k, table[0], 3, 0),
                              dense_kv(v, table[0], 3, 0), 0.5)
    assert np.abs(out[4] - last).max() <= TOL
    # sequence 1: no tokens at all
    assert np.all(out[5:7] == 0) and np.all(np.isneginf(lse[5:7]))


def cascade_case(rng, prefix_lens, group_sizes, suffix_lens, Hq, Hkv, D, bs=16):
    """Prefix tables [R, w], suffix tables [B, w] over one shuffled pool."""
    R, B = len(prefix_lens), len(suffix_lens)
    pre_blk = [-(-int(n) // bs) for n in prefix_lens]
    suf_blk = [-(-int(n) // bs) for n in suffix_lens]
    pool = sum(pre_blk) + sum(suf_blk) + 2
    perm = list(rng.permutation(pool))
    w = max(pre_blk + suf_blk + [1]) + 1
    pt = np.full((R, w), -1, dtype=np.int64)
    st = np.full((B, w), -1, dtype=np.int64)
    for r, nb in enumerate(pre_blk):
        pt[r, :nb] = [perm.pop() for _ in range(nb)]
    for b, nb in enumerate(suf_blk):
        st[b, :nb] = [perm.pop() for _ in range(nb)]
    gs = np.concatenate([[0], np.cumsum(group_sizes)]).astype(np.int64)
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    k = rng.standard_normal((pool, bs, Hkv, D)).astype(np.float16)
    v = rng.standard_normal((pool, bs, Hkv, D)).astype(np.float16)
    return q, k, v, pt, np.asarray(prefix_lens), gs, st, np.asarray(suffix_lens)


def pin_cascade_concatenated_table(MQ, O):
    rng = np.random.default_rng(36)
    pre, sizes, suf = [32, 64, 0], [3, 1, 2], [5, 0, 17, 16, 1, 40]
    q, k, v, pt, pl, gs, st, sl = cascade_case(rng, pre, sizes, suf, 8, 2, 16)
    out, lse = MQ.cascade_attention(q, k, v, pt, pl, gs, st, sl, 0.3)
    # every prefix here is whole blocks, so prefix frames + suffix frames form a block table
    B = len(suf)
    table = np.full((B, 16), -1, dtype=np.int64)
    lens = np.zeros(B, dtype=np.int64)
    for r in range(len(pre)):
        for b in range(gs[r], gs[r + 1]):
            frames = list(pt[r, :pre[r] // 16]) + list(st[b, :-(-suf[b] // 16)])
            table[b, :len(frames)] = frames
            lens[b] = pre[r] + suf[b]
    ref, ref_lse = O.paged_decode_attention(q, k, v, table, lens, 0.3)
    assert np.abs(out - ref).max() <= TOL and np.abs(lse - ref_lse).max() <= TOL


def pin_cascade_merge(MQ, O):
    rng = np.random.default_rng(37)
    pre, sizes, suf = [21, 50], [4, 2], [3, 0, 30, 7, 16, 0]
    q, k, v, pt, pl, gs, st, sl = cascade_case(rng, pre, sizes, suf, 4, 1, 8)
    out, lse = MQ.cascade_attention(q, k, v, pt, pl, gs, st, sl, 0.4)
    # prefix pass: the requests of group r are the queries of prefix r, no mask
    o_pre, l_pre = MQ.multi_query_attention(q, k, v, pt, pl, gs, 0.4, causal=False)
    o_suf, l_suf = O.partial_attention(q, k, v, st, sl, 0.4)
    o_m, l_m = O.merge_partials(np.stack([o_pre, o_suf]), np.stack([l_pre, l_suf]))
    assert np.abs(out - o_m).max() <= TOL and np.abs(lse - l_m).max() <= TOL


def pin_cascade_reads(MQ, O):
    ex = _golden("cascade_reads.json")
    naive, cascade = MQ.cascade_read_tokens(ex["prefix_tokens"], [0] * ex["requests"])
    assert naive == ex["naive_prefix_token_reads"] and cascade == ex["cascade_prefix_token_reads"]
    naive, cascade = MQ.cascade_read_tokens(1000, [3, 5])
    assert naive == 2 * 1000 + 8 and cascade == 1000 + 8


ALL_PINS = [
    pin_chunk_positions,
    pin_dense_textbook,
    pin_page_chunk_update,
    pin_mpmath_causal,
    pin_single_query_is_decode,
    pin_queries_past_context,
    pin_cascade_concatenated_table,
    pin_cascade_merge,
    pin_cascade_reads,
]
