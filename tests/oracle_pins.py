"""Checks that pin the float64 oracle to facts other than its own code.

Each ``pin_*`` takes the oracle module (or a patched copy of it) and raises
AssertionError when the oracle disagrees with something the pages or plain
mathematics fix:

* the page's worked example of a block table (three logical blocks mapped to
  frames 42, 9 and 88) and its block-stride and KV-size figures;
* a paged layout equals the contiguous layout, and permuting physical frames
  changes nothing (bitwise);
* closed forms: with scale 0 the output is the exact mean of V and the lse is
  ln n; one token returns its V row exactly;
* brute force with 50-digit arithmetic on tiny inputs;
* linearity in V, and equal query rows in a group give equal outputs;
* merging partials over any split equals attention over the whole range, the
  merge is associative with -inf partials as identity, and it agrees with the
  (m, l, O) update equations printed on the disaggregated-inference page;
* poisoned slots (unused frames, tails of last blocks) are never read.

``test_oracle.py`` runs every pin on the oracle, and runs them again on
planted mistakes to show that each mistake is caught.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def small_paged(rng, lens, Hq, Hkv, D, bs=16, extra_blocks=3, dtype=np.float16):
    """Random q, a shuffled pool with spare frames, and block tables (width + 2, -1 padded)."""
    lens = [int(n) for n in lens]
    nblk = [-(-n // bs) for n in lens]
    pool_blocks = sum(nblk) + extra_blocks
    perm = rng.permutation(pool_blocks)
    width = max(nblk + [1]) + 2
    table = np.full((len(lens), width), -1, dtype=np.int64)
    off = 0
    for b, k in enumerate(nblk):
        table[b, :k] = perm[off:off + k]
        off += k
    q = rng.standard_normal((len(lens), Hq, D)).astype(dtype)
    k = rng.standard_normal((pool_blocks, bs, Hkv, D)).astype(dtype)
    v = rng.standard_normal((pool_blocks, bs, Hkv, D)).astype(dtype)
    return q, k, v, table, np.asarray(lens)


def pin_page_layout_example(O):
    ex = _golden("paged_layout_example.json")
    bs = ex["block_size"]
    row = [blk["physical_frame"] for blk in ex["logical_blocks"]]
    for blk in ex["logical_blocks"]:
        for t in (blk["first_token"], blk["last_token"]):
            frame, slot = O.token_location(row, t, bs)
            assert frame == blk["physical_frame"], (t, frame)
            assert slot == t - blk["first_token"], (t, slot)
    # a pool whose rows spell out their own (frame, slot) address
    pool = np.zeros((100, bs, 1, 2))
    for f in range(100):
        for s in range(bs):
            pool[f, s, 0] = (f, s)
    got = O.gather_sequence(pool, row, 48, 0, bs)
    want = [(blk["physical_frame"], s) for blk in ex["logical_blocks"] for s in range(bs)]
    assert np.array_equal(got, np.array(want, dtype=np.float64))


def pin_block_stride(O):
    ex = _golden("kv_sizing.json")["block_stride_example"]
    pool = np.zeros((3, ex["block_size"], ex["n_kv_heads"], ex["head_dim"]), dtype=np.float16)
    assert pool.strides[0] == ex["bytes"]
    # the same figure read back from the KV-size formula: one block of one cache
    assert O.kv_cache_bytes([ex["block_size"]], ex["n_kv_heads"], ex["head_dim"], 1,
                            ex["bytes_per_elem"]) == 2 * ex["bytes"]


def pin_kv_sizes(O):
    g = _golden("kv_sizing.json")
    m = g["m_kv_70b_fp8"]
    got = O.kv_cache_bytes([m["tokens"]], m["n_kv_heads"], m["head_dim"], m["n_layers"],
                           m["bytes_per_elem"])
    assert abs(got / 1e6 - m["printed_megabytes"]) < 0.01, got     # the page prints it truncated
    a = g["a6000_capacity"]
    per_token = O.kv_cache_bytes([1], a["n_kv_heads"], a["head_dim"], a["n_layers"], 2)
    assert per_token == 128 * 1024
    tokens = (a["gpu_bytes"] - a["params"] * a["bytes_per_param"]) / (a["batch"] * per_token)
    assert 0.85 * a["printed_tokens_per_request"] < tokens < 1.1 * a["printed_tokens_per_request"]


def pin_gather_modes_agree(O):
    rng = np.random.default_rng(11)
    q, k, v, table, lens = small_paged(rng, [1, 15, 16, 17, 40], 4, 2, 8)
    for b, n in enumerate(lens):
        for g in range(2):
            a = O.gather_sequence(k, table[b], n, g, 16)
            c = O._gather_sequence_blocks(k, table[b], n, g, 16)
            assert np.array_equal(a, c)
    out1, lse1 = O.paged_decode_attention(q, k, v, table, lens, 0.3, per_block_gather=False)
    out2, lse2 = O.paged_decode_attention(q, k, v, table, lens, 0.3, per_block_gather=True)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


def _scatter_contiguous(rng, K_seq, V_seq, bs, extra=4):
    """Put per-sequence contiguous [n, Hkv, D] rows into a shuffled pool."""
    Hkv, D = K_seq[0].shape[1:]
    nblk = [-(-len(Kb) // bs) for Kb in K_seq]
    pool_blocks = sum(nblk) + extra
    perm = rng.permutation(pool_blocks)
    kp = np.full((pool_blocks, bs, Hkv, D), np.nan)
    vp = np.full((pool_blocks, bs, Hkv, D), np.nan)
    table = np.full((len(K_seq), max(nblk) + 1), -1, dtype=np.int64)
    off = 0
    for b, (Kb, Vb) in enumerate(zip(K_seq, V_seq)):
        for i in range(nblk[b]):
            f = perm[off + i]
            table[b, i] = f
            rows = Kb[i * bs:(i + 1) * bs]
            kp[f, :len(rows)] = rows
            vp[f, :len(rows)] = Vb[i * bs:(i + 1) * bs]
        off += nblk[b]
    return kp, vp, table


def pin_paged_equals_contiguous(O):
    rng = np.random.default_rng(12)
    lens = [3, 16, 33, 70]
    Hq, Hkv, D, bs = 6, 2, 8, 16
    G = Hq // Hkv
    K_seq = [rng.standard_normal((n, Hkv, D)).astype(np.float16).astype(np.float64) for n in lens]
    V_seq = [rng.standard_normal((n, Hkv, D)).astype(np.float16).astype(np.float64) for n in lens]
    q = rng.standard_normal((len(lens), Hq, D)).astype(np.float16)
    kp, vp, table = _scatter_contiguous(rng, K_seq, V_seq, bs)
    out, lse = O.paged_decode_attention(q, kp, vp, table, lens, 0.35)
    for b in range(len(lens)):
        for h in range(Hq):
            g = h // G                 # contiguous query-head groups
            o, l = O.attend(q[b, h:h + 1], K_seq[b][:, g], V_seq[b][:, g], 0.35)
            assert np.array_equal(out[b, h], o[0]), (b, h)
            assert np.array_equal(lse[b, h], l[0]), (b, h)


def pin_block_permutation_invariance(O):
    rng = np.random.default_rng(13)
    q, k, v, table, lens = small_paged(rng, [5, 32, 49], 4, 1, 8, extra_blocks=5)
    out, lse = O.paged_decode_attention(q, k, v, table, lens, 0.4)
    sigma = rng.permutation(k.shape[0])          # new frame of old frame f is sigma[f]
    k2 = np.empty_like(k)
    v2 = np.empty_like(v)
    k2[sigma] = k
    v2[sigma] = v
    table2 = np.where(table >= 0, sigma[np.maximum(table, 0)], -1)
    out2, lse2 = O.paged_decode_attention(q, k2, v2, table2, lens, 0.4)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def scale0_values(t, d, g):
    """Exact-in-fp16 V entry for logical token t, dim d, KV head g: k * 2^-11, k < 2048."""
    return ((t + 7 * d + 13 * g) % 2048) / 2048.0


def place_logical_values(table, lens, pool, fn):
    """Write fn(t, d, g) at the physical slot of every logical token."""
    bs, Hkv, D = pool.shape[1:]
    for b, n in enumerate(lens):
        for t in range(int(n)):
            f, s = int(table[b][t // bs]), t % bs
            for g in range(Hkv):
                pool[f, s, g] = [fn(t, d, g) for d in range(D)]


def pin_scale0_closed_form(O):
    rng = np.random.default_rng(14)
    q, k, v, table, lens = small_paged(rng, [1, 7, 16, 37, 100], 4, 2, 8)
    place_logical_values(table, lens, v, scale0_values)
    out, lse = O.paged_decode_attention(q, k, v, table, lens, 0.0)
    for b, n in enumerate(lens):
        n = int(n)
        for h in range(4):
            g = h // 2
            assert abs(lse[b, h] - math.log(n)) <= 1e-15 * max(1.0, math.log(n)), (b, h)
            for d in range(8):
                exact = sum(Fraction(scale0_values(t, d, g)) for t in range(n)) / n
                assert abs(Fraction(out[b, h, d]) - exact) <= Fraction(1, 2 ** 52), (b, h, d)


def pin_mpmath_bruteforce(O):
    import mpmath
    mpmath.mp.dps = 50
    rng = np.random.default_rng(15)
    Hq, Hkv, D = 4, 2, 8
    q, k, v, table, lens = small_paged(rng, [1, 2, 17, 40], Hq, Hkv, D)
    scale = float(np.float32(0.5))
    out, lse = O.paged_decode_attention(q, k, v, table, lens, scale)
    for b, n in enumerate(lens):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            rows = [(int(table[b][t // 16]), t % 16) for t in range(int(n))]
            s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(float(q[b, h, d])) *
                                                 mpmath.mpf(float(k[f, sl, g, d]))
                                                 for d in range(D)) for f, sl in rows]
            w = [mpmath.exp(x) for x in s]
            den = mpmath.fsum(w)
            lse_ref = mpmath.log(den)
            assert abs(lse[b, h] - float(lse_ref)) <= 1e-13 * max(1.0, abs(float(lse_ref)))
            for d in range(D):
                ref = mpmath.fsum(wi * mpmath.mpf(float(v[f, sl, g, d]))
                                  for wi, (f, sl) in zip(w, rows)) / den
                assert abs(out[b, h, d] - float(ref)) <= 1e-13 * max(1.0, abs(float(ref))), (b, h, d)


def pin_ctx1_returns_v(O):
    rng = np.random.default_rng(16)
    q, k, v, table, lens = small_paged(rng, [1, 1, 1], 8, 2, 8)
    out, lse = O.paged_decode_attention(q, k, v, table, lens, 0.7)
    for b in range(3):
        f = int(table[b, 0])
        for h in range(8):
            assert np.array_equal(out[b, h], v[f, 0, h // 4].astype(np.float64))
            s = float(np.float32(0.7)) * float(np.dot(q[b, h].astype(np.float64),
                                                     k[f, 0, h // 4].astype(np.float64)))
            assert abs(lse[b, h] - s) <= 1e-15 * max(1.0, abs(s))


def pin_linearity_and_equal_rows(O):
    rng = np.random.default_rng(17)
    q, k, v1, table, lens = small_paged(rng, [9, 40], 4, 2, 8)
    v2 = rng.standard_normal(v1.shape)
    a, c = 0.75, -1.5
    o1, _ = O.paged_decode_attention(q, k, v1, table, lens, 0.3)
    o2, _ = O.paged_decode_attention(q, k, v2, table, lens, 0.3)
    o3, _ = O.paged_decode_attention(q, k, a * v1.astype(np.float64) + c * v2, table, lens, 0.3)
    assert np.allclose(o3, a * o1 + c * o2, rtol=0, atol=1e-12)
    qe = q.copy()
    qe[:, 1] = qe[:, 0]
    qe[:, 3] = qe[:, 2]
    oe, le = O.paged_decode_attention(qe, k, v1, table, lens, 0.3)
    assert np.array_equal(oe[:, 1], oe[:, 0]) and np.array_equal(oe[:, 3], oe[:, 2])
    assert np.array_equal(le[:, 1], le[:, 0])
    assert not np.allclose(oe[:, 1], oe[:, 2])     # different KV heads differ


def pin_merge_equals_full(O):
    rng = np.random.default_rng(18)
    D = 8
    for trial in range(10):
        n = int(rng.integers(2, 60))
        K = rng.standard_normal((n, D))
        V = rng.standard_normal((n, D))
        qr = rng.standard_normal((3, D))
        o_full, l_full = O.attend(qr, K, V, 0.6)
        cuts = sorted(rng.integers(0, n + 1, size=int(rng.integers(1, 5))).tolist())
        bounds = [0] + cuts + [n]                     # may contain empty ranges
        parts = [O.attend(qr, K[lo:hi], V[lo:hi], 0.6) for lo, hi in zip(bounds[:-1], bounds[1:])]
        o_m, l_m = O.merge_partials(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
        assert np.allclose(o_m, o_full, rtol=0, atol=1e-12)
        assert np.allclose(l_m, l_full, rtol=1e-13, atol=0)
    # associativity and the empty partial as identity
    os_ = rng.standard_normal((3, 4, D))
    ls_ = rng.standard_normal((3, 4)) * 5
    ab = O.merge_partials(os_[:2], ls_[:2])
    left = O.merge_partials(np.stack([ab[0], os_[2]]), np.stack([ab[1], ls_[2]]))
    bc = O.merge_partials(os_[1:], ls_[1:])
    right = O.merge_partials(np.stack([os_[0], bc[0]]), np.stack([ls_[0], bc[1]]))
    allm = O.merge_partials(os_, ls_)
    for x in (left, right):
        assert np.allclose(x[0], allm[0], atol=1e-12) and np.allclose(x[1], allm[1], atol=1e-12)
    ident = O.merge_partials(np.stack([os_[0], np.zeros((4, D))]),
                             np.stack([ls_[0], np.full(4, -np.inf)]))
    assert np.array_equal(ident[0], os_[0]) and np.array_equal(ident[1], ls_[0])
    empty = O.merge_partials(np.zeros((2, 4, D)), np.full((2, 4), -np.inf))
    assert np.array_equal(empty[0], np.zeros((4, D))) and np.all(np.isneginf(empty[1]))


def pin_merge_page_equations(O):
    """Fold unnormalised (m, l, O) partials with the page's update equations."""
    rng = np.random.default_rng(19)
    D, n = 8, 50
    K = rng.standard_normal((n, D))
    V = rng.standard_normal((n, D))
    qr = rng.standard_normal((1, D))
    s = 0.45 * (K @ qr[0])
    bounds = [0, 7, 8, 31, 50]
    m_prev, l_prev, O_prev = -np.inf, 0.0, np.zeros(D)
    o_parts, lse_parts = [], []
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        m_cur = s[lo:hi].max()
        l_cur = np.exp(s[lo:hi] - m_cur).sum()
        O_cur = (np.exp(s[lo:hi] - m_cur)[:, None] * V[lo:hi]).sum(axis=0)
        m_new = max(m_prev, m_cur)
        l_prev = np.exp(m_prev - m_new) * l_prev + np.exp(m_cur - m_new) * l_cur
        O_prev = np.exp(m_prev - m_new) * O_prev + np.exp(m_cur - m_new) * O_cur
        m_prev = m_new
        o_parts.append(O_cur / l_cur)
        lse_parts.append(m_cur + np.log(l_cur))
    o_m, l_m = O.merge_partials(np.array(o_parts)[:, None], np.array(lse_parts)[:, None])
    assert np.allclose(o_m[0], O_prev / l_prev, rtol=0, atol=1e-13)
    assert abs(l_m[0] - (m_prev + np.log(l_prev))) <= 1e-13


def pin_partitions(O):
    for n in (0, 1, 15, 16, 17, 511, 512, 513, 2000):
        for P in (16, 32, 512):
            r = O.partition_ranges(n, P)
            assert len(r) == -(-n // P)
            assert all(hi - lo == P for lo, hi in r[:-1])
            if r:
                assert r[0][0] == 0 and r[-1][1] == n and 0 < r[-1][1] - r[-1][0] <= P
            assert all(r[i][1] == r[i + 1][0] for i in range(len(r) - 1))
    rng = np.random.default_rng(20)
    q, k, v, table, lens = small_paged(rng, [1, 31, 32, 33, 95], 4, 2, 8)
    o_p, l_p = O.split_k_partials(q, k, v, table, lens, 0.5, 32)
    out, lse = O.paged_decode_attention(q, k, v, table, lens, 0.5)
    o_m, l_m = O.merge_partials(np.moveaxis(o_p, 2, 0), np.moveaxis(l_p, 2, 0))
    assert np.allclose(o_m, out, rtol=0, atol=1e-12) and np.allclose(l_m, lse, atol=1e-12)
    # the second partition of the 33-token sequence is the single token 32
    b = 3
    f, s = int(table[b, 2]), 0
    assert np.array_equal(o_p[b, 0, 1], v[f, s, 0].astype(np.float64))


def pin_poison_not_read(O):
    rng = np.random.default_rng(21)
    q, k, v, table, lens = small_paged(rng, [5, 21, 32], 4, 2, 8, extra_blocks=4)
    used = {(int(table[b, t // 16]), t % 16) for b, n in enumerate(lens) for t in range(int(n))}
    k1, v1, k2, v2 = k.copy(), v.copy(), k.copy(), v.copy()
    for f in range(k.shape[0]):
        for s in range(16):
            if (f, s) not in used:
                k1[f, s], v1[f, s] = 6e4, np.nan
                k2[f, s], v2[f, s] = 0.0, 0.0
    o1, l1 = O.paged_decode_attention(q, k1, v1, table, lens, 0.3)
    o2, l2 = O.paged_decode_attention(q, k2, v2, table, lens, 0.3)
    assert np.all(np.isfinite(o1)) and np.array_equal(o1, o2) and np.array_equal(l1, l2)


def pin_kv_append(O):
    ex = _golden("paged_layout_example.json")
    row = [blk["physical_frame"] for blk in ex["logical_blocks"]]
    # the figure's request: token 47 is the last slot of logical block 2 (frame 88),
    # token 16 the first slot of logical block 1 (frame 9)
    for ctx, frame, slot in ((48, 88, 15), (17, 9, 0), (1, 42, 0)):
        k = np.zeros((100, 16, 1, 2))
        v = np.zeros((100, 16, 1, 2))
        kn = np.array([[[1.0, 2.0]]])
        k2, v2 = O.kv_append(k, v, kn, -kn, [row], [ctx])
        changed = np.argwhere(np.any(k2 != k, axis=(2, 3)))
        assert changed.tolist() == [[frame, slot]], (ctx, changed.tolist())
        assert np.array_equal(k2[frame, slot], kn[0]) and np.array_equal(v2[frame, slot], -kn[0])
    # append then attend == attention over the old rows plus the new one, contiguous
    rng = np.random.default_rng(23)
    lens_old = [0, 15, 16, 40]
    lens = [n + 1 for n in lens_old]
    q, k, v, table, _ = small_paged(rng, lens, 4, 2, 8)
    kn = rng.standard_normal((4, 2, 8)).astype(np.float16)
    vn = rng.standard_normal((4, 2, 8)).astype(np.float16)
    k2, v2 = O.kv_append(k, v, kn, vn, table, lens)
    out, lse = O.paged_decode_attention(q, k2, v2, table, lens, 0.3)
    for b, n in enumerate(lens_old):
        for h in range(4):
            g = h // 2
            K = np.concatenate([O.gather_sequence(k, table[b], n, g), kn[b, g][None].astype(np.float64)])
            V = np.concatenate([O.gather_sequence(v, table[b], n, g), vn[b, g][None].astype(np.float64)])
            o, l = O.attend(q[b, h:h + 1], K, V, 0.3)
            assert np.array_equal(out[b, h], o[0]) and np.array_equal(lse[b, h], l[0])
    # ctx = 0 appends nothing
    k3, _ = O.kv_append(k, v, kn, vn, table, [0, 0, 0, 0])
    assert np.array_equal(k3, k)


def pin_fp8_decode(O):
    g = _golden("fp8_e4m3_codes.json")
    for code, want in g["codes"].items():
        got = O.fp8_e4m3_value(int(code, 16))
        if want == "nan":
            assert math.isnan(got), code
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), (code, got)
    # an independent decoder of the same format: torch's float8_e4m3fn, all 256 codes
    import torch
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = ref.to(torch.float64).numpy()
    got = O.fp8_e4m3_decode(np.arange(256))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def pin_fp8_encode(O):
    codes = np.arange(256)
    finite = (codes & 0x7F) != 0x7F
    # the encoder inverts the decoder on every finite code (-0 included)
    assert np.array_equal(O.fp8_e4m3_encode(O.fp8_e4m3_decode(codes[finite])), codes[finite])
    # midpoints of adjacent codes go to the even one (exact in float32: 5 bits)
    pos = O.fp8_e4m3_decode(np.arange(0x7F))
    mid = (pos[:-1] + pos[1:]) / 2
    up = np.arange(1, 0x7F)
    want = np.where(up % 2 == 0, up, up - 1)
    assert np.array_equal(O.fp8_e4m3_encode(mid), want)
    assert np.array_equal(O.fp8_e4m3_encode(-mid), want | 0x80)
    # just off a midpoint goes to the nearer code
    assert np.array_equal(O.fp8_e4m3_encode(np.nextafter(mid, np.inf)), up)
    assert np.array_equal(O.fp8_e4m3_encode(np.nextafter(mid, -np.inf)), up - 1)
    # saturation, infinities, NaN
    assert O.fp8_e4m3_encode([448.0, 463.9, 464.0, 1e30, np.inf, -np.inf, -1e30]).tolist() == \
        [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert int(O.fp8_e4m3_encode([np.nan])[0]) & 0x7F == 0x7F
    # an independent encoder of the same format: torch's float8_e4m3fn
    # conversion (round to nearest even), below 464 where it does not overflow
    import torch
    rng = np.random.default_rng(25)
    x = rng.standard_normal(4000) * 10.0 ** rng.uniform(-4, 2.6, 4000)
    x = np.concatenate([x, mid, -mid, [0.0, -0.0, 2.0 ** -10, 2.0 ** -9 * 1.5]]).astype(np.float32)
    x = x[np.abs(x) < 464]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.fp8_e4m3_encode(x), ref)


def pin_kv_append_fp8(O):
    rng = np.random.default_rng(26)
    Hkv, D = 2, 8
    lens = [0, 1, 16, 17, 40]
    _, _, _, table, _ = small_paged(rng, lens, 2, Hkv, D)
    pool = int(table.max()) + 1
    k = rng.integers(0, 0x7F, size=(pool, 16, Hkv, D)).astype(np.uint8)
    v = rng.integers(0, 0x7F, size=(pool, 16, Hkv, D)).astype(np.uint8)
    kn = (rng.standard_normal((len(lens), Hkv, D)) * 3).astype(np.float16)
    vn = (rng.standard_normal((len(lens), Hkv, D)) * 0.2).astype(np.float16)
    ks = float(np.abs(kn.astype(np.float64)).max()) / 400      # in range: no saturation
    vs = float(np.abs(vn.astype(np.float64)).max()) / 400
    k2, v2 = O.kv_append_fp8(k, v, kn, vn, table, lens, ks, vs)
    changed = set()
    for b, n in enumerate(lens):
        if n <= 0:
            continue
        fr, sl = int(table[b][(n - 1) // 16]), (n - 1) % 16
        changed.add((fr, sl))
        for src, codes, s_ in ((kn, k2, ks), (vn, v2, vs)):
            back = s_ * O.fp8_e4m3_decode(codes[fr, sl])
            x = src[b].astype(np.float64)
            # E4M3 keeps 3 mantissa bits: within half a step, 2^-4 relative, or
            # half the smallest step 2^-10 * scale near zero
            assert np.all(np.abs(back - x) <= np.maximum(np.abs(x) * 2.0 ** -4, s_ * 2.0 ** -10)
                          * (1 + 1e-6)), (b, s_)
    for fr in range(pool):
        for sl in range(16):
            if (fr, sl) not in changed:
                assert np.array_equal(k2[fr, sl], k[fr, sl]) and np.array_equal(v2[fr, sl], v[fr, sl])
    # beyond the range the codes saturate to +-448
    big = np.full_like(kn, 1000.0)
    big[:, :, 1::2] = -1000.0
    k3, _ = O.kv_append_fp8(k, v, big, vn, table, lens, 1.0, vs)
    fr, sl = int(table[4][39 // 16]), 39 % 16
    assert set(k3[fr, sl].ravel().tolist()) == {0x7E, 0xFE}


def pin_fp8_attention(O):
    rng = np.random.default_rng(24)
    Hq, Hkv, D = 4, 2, 8
    lens = [1, 9, 40]
    _, _, _, table, _ = small_paged(rng, lens, Hq, Hkv, D)
    pool = table.max() + 1
    codes = rng.integers(0, 256, size=(pool, 16, Hkv, D)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38                     # no NaN codes in owned slots
    vcodes = rng.integers(0, 256, size=(pool, 16, Hkv, D)).astype(np.uint8)
    vcodes[(vcodes & 0x7F) == 0x7F] = 0x3C
    q = rng.standard_normal((len(lens), Hq, D)).astype(np.float16)
    ks, vs = 0.0125, 0.5
    out, lse = O.paged_decode_attention_fp8(q, codes, vcodes, table, lens, 0.3, ks, vs)
    # one token: out = v_scale * value(code), exactly
    f, sl = int(table[0, 0]), 0
    for h in range(Hq):
        want = vs * np.array([O.fp8_e4m3_value(c) for c in vcodes[f, sl, h // 2]])
        assert np.array_equal(out[0, h], want)
    # paged fp8 == attention on the decoded contiguous rows, bitwise
    for b, n in enumerate(lens):
        for h in range(Hq):
            g = h // 2
            rows = [(int(table[b][t // 16]), t % 16) for t in range(n)]
            K = np.array([[ks * O.fp8_e4m3_value(c) for c in codes[fr, s_, g]] for fr, s_ in rows])
            V = np.array([[vs * O.fp8_e4m3_value(c) for c in vcodes[fr, s_, g]] for fr, s_ in rows])
            o, l = O.attend(q[b, h:h + 1], K, V, 0.3)
            assert np.array_equal(out[b, h], o[0]) and np.array_equal(lse[b, h], l[0])
    # scale 0: the mean of the decoded, scaled V rows
    out0, lse0 = O.paged_decode_attention_fp8(q, codes, vcodes, table, lens, 0.0, ks, vs)
    b, n = 2, lens[2]
    for h in range(Hq):
        vals = [[Fraction(O.fp8_e4m3_value(c)) for c in vcodes[int(table[b][t // 16]), t % 16, h // 2]]
                for t in range(n)]
        for d in range(D):
            exact = Fraction(vs) * sum(v[d] for v in vals) / n
            assert abs(Fraction(out0[b, h, d]) - exact) <= Fraction(1, 2 ** 50)
        assert abs(lse0[b, h] - math.log(n)) <= 1e-15 * math.log(n)


ALL_PINS = [
    pin_page_layout_example,
    pin_block_stride,
    pin_kv_sizes,
    pin_gather_modes_agree,
    pin_paged_equals_contiguous,
    pin_block_permutation_invariance,
    pin_scale0_closed_form,
    pin_mpmath_bruteforce,
    pin_ctx1_returns_v,
    pin_linearity_and_equal_rows,
    pin_merge_equals_full,
    pin_merge_page_equations,
    pin_partitions,
    pin_poison_not_read,
    pin_kv_append,
    pin_fp8_decode,
    pin_fp8_encode,
    pin_kv_append_fp8,
    pin_fp8_attention,
]
