"""HIP path against the float64 oracle, element by element, on seeded inputs.

Every call goes through the C ABI (ctypes binding).  Small cases are checked in
full; the full-size workloads too, every sequence, which the oracle computes
one at a time from a host copy of its own blocks, in the launch configuration
the benchmark times.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import decode_attention_paged_attn_amd as pda
from decode_attention_paged_attn_amd import workloads as W
import oracle.paged_attention as O
from tests.schedule import workspace_segments
from tests.parity import (ROW_REL_TOL, compare_lse, compare_out, compare_ulps, p_rounding_bound,
                          to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pda.load_library()          # raises if the HIP library is missing
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _say(msg):
    print(msg, flush=True)


def run(case, partition_tokens=0, **kw):
    _say(f"[run] {case.name} B={case.B} Hq={case.Hq} Hkv={case.Hkv} P={partition_tokens} "
         f"kv={case.kv_dtype}")
    out, lse = pda.paged_decode_attn(case.q, case.k_cache, case.v_cache, case.block_table,
                                     case.context_lens, case.scale, return_lse=True,
                                     partition_tokens=partition_tokens, **case.attn_kwargs(),
                                     **kw)
    torch.cuda.synchronize()
    return out, lse


def oracle_of(case, q, k, v, table, lens):
    """The oracle's attention for this case's cache format on host copies."""
    if case.kv_dtype == "fp8":
        return O.paged_decode_attention_fp8(q, k, v, table, lens, case.scale, case.k_scale,
                                            case.v_scale)
    return O.paged_decode_attention(q, k, v, table, lens, case.scale)


def oracle_full(case):
    return oracle_of(case, *W.host_full(case))


# --- small cases, checked in full ----------------------------------------------

@pytest.mark.parametrize("P", [0, 16, 64, 128, 512, 1024, 4096])
def test_tiny_workload(P):
    case = W.tiny(device="cuda")
    out, lse = run(case, P)
    ref, ref_lse = oracle_full(case)
    compare_out(to_np(out), ref)
    compare_lse(to_np(lse), ref_lse)


RAGGED = [1, 2, 15, 16, 17, 31, 33, 100, 255, 256, 257, 511, 512, 513, 1000, 1537]


# Group sizes and KV-head counts: the pages' GQA shapes Q32:KV8, Q48:KV8 and
# Q64:KV8 (G = 4, 6, 8 at 8 KV heads) and MHA Q32:KV32, Q40:KV40, Q48:KV48,
# plus small and odd KV-head counts (work-groups of 1 to 4 KV heads).
SHAPES = [(1, 2), (2, 2), (4, 2), (8, 1), (4, 8), (6, 8), (8, 8), (6, 1), (1, 32), (1, 40),
          (1, 48), (4, 3), (2, 5), (1, 6), (8, 7), (6, 5)]


@pytest.mark.parametrize("G,Hkv", SHAPES)
@pytest.mark.parametrize("P", [0, 32, 256])
def test_ragged_lengths_all_group_sizes(G, Hkv, P):
    case = W.build_case(RAGGED, G * Hkv, Hkv, pool_blocks=sum(-(-n // 16) for n in RAGGED) + 7,
                        seed=100 + G, device="cuda", name=f"ragged_G{G}")
    out, lse = run(case, P)
    ref, ref_lse = oracle_full(case)
    compare_out(to_np(out), ref)
    compare_lse(to_np(lse), ref_lse)


def test_empty_contexts():
    case = W.build_case([0, 5, 0, 17], 8, 2, seed=3, device="cuda", width=2)
    out, lse = run(case)
    o, l = to_np(out), to_np(lse)
    assert np.all(o[[0, 2]] == 0) and np.all(np.isneginf(l[[0, 2]]))
    ref, ref_lse = oracle_full(case)
    compare_out(o, ref)
    compare_lse(l, ref_lse)


def test_one_token_returns_v_exactly():
    case = W.build_case([1] * 6, 32, 8, seed=4, device="cuda")
    out, _ = run(case)
    o = out.cpu().numpy()
    v = case.v_cache.cpu().numpy()
    for b in range(6):
        f = int(case.block_table_host[b, 0])
        for h in range(32):
            assert np.array_equal(o[b, h], v[f, 0, h // 4]), (b, h)


def test_scale_zero_gives_exact_mean():
    lens = [1, 7, 16, 37, 300, 1025]
    case = W.build_case(lens, 8, 2, seed=5, device="cuda")
    v = case.v_cache.cpu().numpy()
    t = np.arange(16)
    for b, n in enumerate(lens):
        for i in range(-(-n // 16)):
            f = int(case.block_table_host[b, i])
            tok = 16 * i + t
            for g in range(2):
                d = np.arange(128)
                v[f, :, g, :] = ((tok[:, None] + 7 * d[None, :] + 13 * g) % 2048) / 2048.0
    case.v_cache.copy_(torch.from_numpy(v))
    case.scale = 0.0
    out, lse = run(case)
    o, l = to_np(out), to_np(lse)
    for b, n in enumerate(lens):
        for g in range(2):
            exact = [float(sum(Fraction((tt + 7 * d + 13 * g) % 2048, 2048) for tt in range(n)) / n)
                     for d in range(128)]
            for h in range(4 * g, 4 * g + 4):
                compare_out(o[b, h][None], np.array(exact)[None])
                assert abs(l[b, h] - math.log(n)) <= 1e-5


def test_frame_permutation_changes_nothing():
    need = sum(-(-n // 16) for n in RAGGED)
    case = W.build_case(RAGGED, 16, 4, seed=6, device="cuda", pool_blocks=need + 20)
    out1, lse1 = run(case)
    sigma = torch.randperm(case.num_blocks, generator=torch.Generator().manual_seed(1))
    k2 = torch.empty_like(case.k_cache)
    v2 = torch.empty_like(case.v_cache)
    k2[sigma.cuda()] = case.k_cache
    v2[sigma.cuda()] = case.v_cache
    bt = case.block_table.long()
    bt2 = torch.where(bt >= 0, sigma.cuda()[bt.clamp(min=0)], bt).int()
    case.k_cache, case.v_cache, case.block_table = k2, v2, bt2.contiguous()
    out2, lse2 = run(case)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_bitwise_deterministic():
    case = W.build_case(RAGGED * 2, 32, 8, seed=7, device="cuda")
    a, la = run(case, 64)
    b, lb = run(case, 64)
    assert torch.equal(a, b) and torch.equal(la, lb)


@pytest.mark.parametrize("P", [0, 64, 2048])
def test_split_partials_in_workspace(P):
    """Every stored partial equals the oracle's attention over the same token range."""
    lens = [1, 63, 64, 65, 200, 777, 5000, 9000, 3000]
    case = W.build_case(lens, 8, 2, seed=8, device="cuda")
    width = case.block_table.shape[1]
    lay = pda.workspace_layout(case.B, case.Hq, case.Hkv, width, P, kv_fp8=False)
    ws = torch.zeros(pda.workspace_size(case.B, case.Hq, case.Hkv, width, P), dtype=torch.uint8,
                     device="cuda")
    assert ws.numel() >= lay["total_bytes"]
    out, lse = run(case, P, workspace=ws)
    raw = ws.cpu()
    nsl, Hq = lay["n_slots"], case.Hq
    hdr = raw[:4 * (4 + case.B)].view(torch.int32).numpy()
    l_ws = raw[lay["lse_offset"]:lay["lse_offset"] + 4 * nsl * Hq].view(torch.float32)
    o_ws = raw[lay["o_offset"]:lay["o_offset"] + 4 * nsl * Hq * 128].view(torch.float32)
    l_ws = l_ws.reshape(nsl, Hq).numpy()
    o_ws = o_ws.reshape(nsl, Hq, 128).numpy()
    segs = workspace_segments(lens, lay["unit_tokens"], lay["n_runs"])
    nu = [-(-n // lay["unit_tokens"]) for n in lens]
    assert hdr[1] == sum(nu) and hdr[2] == lay["n_runs"] and hdr[3] == lay["unit_tokens"]
    assert list(hdr[4:]) == [sum(nu[:b]) for b in range(case.B)]
    q, k, v, table, ln = W.host_full(case)
    kv = {}
    split = 0
    for w, b, lo, hi in segs:
        if lo == 0 and hi == lens[b]:
            continue                               # whole sequence: written to out directly
        split += 1
        for g in range(case.Hkv):
            if (b, g) not in kv:
                kv[b, g] = (O._gather_sequence_blocks(k, table[b], lens[b], g, 16),
                            O._gather_sequence_blocks(v, table[b], lens[b], g, 16))
            K, V = kv[b, g][0][lo:hi], kv[b, g][1][lo:hi]
            heads = slice(g * 4, g * 4 + 4)
            o_ref, l_ref = O.attend(q[b, heads], K, V, case.scale)
            compare_lse(l_ws[w + b, heads], l_ref, what=f"lse w={w} b={b} [{lo},{hi})")
            compare_out(o_ws[w + b, heads], o_ref, abs_tol=p_rounding_bound(V),
                        row_rel_tol=ROW_REL_TOL,
                        what=f"o w={w} b={b} [{lo},{hi})")
    assert split > 0, "the case should split at least one sequence"
    ref, ref_lse = O.paged_decode_attention(q, k, v, table, ln, case.scale)
    compare_out(to_np(out), ref)
    compare_lse(to_np(lse), ref_lse)


@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (48, 8), (64, 8), (40, 40)])
def test_partial_api_and_merge(Hq, Hkv):
    R, per = 4, 256
    lens = [R * per] * 3
    case = W.build_case(lens, Hq, Hkv, seed=9, device="cuda")
    cols = per // 16
    o_parts, l_parts = [], []
    for r in range(R):
        bt = case.block_table[:, r * cols:(r + 1) * cols]
        ln = torch.full((case.B,), per, dtype=torch.int32, device="cuda")
        o, l = pda.paged_decode_attn_partial(case.q, case.k_cache, case.v_cache, bt, ln,
                                             case.scale)
        o_parts.append(o)
        l_parts.append(l)
    merged, mlse = pda.merge_partials(torch.stack(o_parts).contiguous(),
                                      torch.stack(l_parts).contiguous())
    single, slse = run(case)
    # p enters the PV product rounded to fp16 relative to each range's own
    # running max, so the two schedules agree to fp16 ulps of each row's scale
    compare_ulps(to_np(merged), to_np(single), ulps=2, rowwise=True)
    q, k, v, table, ln = W.host_full(case)
    ref, ref_lse = O.paged_decode_attention(q, k, v, table, ln, case.scale)
    compare_out(to_np(merged), ref)
    compare_lse(to_np(mlse), ref_lse)
    # each partial against the oracle's partial over the same range
    for r in range(R):
        o_ref, l_ref = O.partial_attention(q, k, v, table[:, r * cols:(r + 1) * cols],
                                           [per] * 3, case.scale)
        compare_out(to_np(o_parts[r]), o_ref, abs_tol=p_rounding_bound(v),
                    row_rel_tol=ROW_REL_TOL)
        compare_lse(to_np(l_parts[r]), l_ref)


def test_merge_partials_edge_cases():
    g = torch.Generator(device="cuda").manual_seed(10)
    o = torch.randn((3, 2, 4, 128), generator=g, device="cuda")
    lse = torch.randn((3, 2, 4), generator=g, device="cuda") * 4
    lse[1] = -float("inf")                      # an empty range everywhere
    lse[2, 1] = -float("inf")
    lse[:, 0, 3] = -float("inf")                # (b=0, h=3): every range empty
    out, mlse = pda.merge_partials(o, lse)
    ref_o, ref_l = O.merge_partials(to_np(o), to_np(lse))
    compare_out(to_np(out), ref_o)
    compare_lse(to_np(mlse), ref_l)
    assert np.all(to_np(out)[0, 3] == 0) and np.isneginf(to_np(mlse)[0, 3])


def test_graph_capture_replays_match_eager():
    case = W.build_case(RAGGED, 32, 8, seed=11, device="cuda")
    ws = torch.empty(pda.workspace_size(case.B, 32, 8, case.block_table.shape[1]),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((case.B, 32, 128), dtype=torch.float16, device="cuda")
    lse = torch.empty((case.B, 32), dtype=torch.float32, device="cuda")
    args = (case.q, case.k_cache, case.v_cache, case.block_table, case.context_lens, case.scale)
    pda.paged_decode_attn(*args, out=out, lse_out=lse, workspace=ws)
    torch.cuda.synchronize()
    eager, eager_lse = out.clone(), lse.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            pda.paged_decode_attn(*args, out=out, lse_out=lse, workspace=ws)
    torch.cuda.synchronize()
    for i in range(4):
        out.fill_(7.0)
        lse.fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager) and torch.equal(lse, eager_lse), f"replay {i}"
        _ = (case.q.float() * 2).sum().item()    # eager work between replays


# --- full-size workloads, every sequence ---------------------------------------

def _check_every_sequence(case, results, chunk_tokens=1 << 18):
    """Each (label, out, lse) over the whole batch against the oracle, on every
    sequence.  The oracle reads host copies of the blocks of a few sequences at
    a time (up to ``chunk_tokens`` tokens, or one longer sequence), so host
    memory stays bounded whatever the batch."""
    got = [(label, to_np(o), to_np(l)) for label, o, l in results]
    b0, done = 0, 0
    while b0 < case.B:
        b1, tok = b0 + 1, int(case.lens[b0])
        while b1 < case.B and tok + int(case.lens[b1]) <= chunk_tokens:
            tok += int(case.lens[b1])
            b1 += 1
        ids = list(range(b0, b1))
        q, k, v, table, lens = W.host_sequences(case, ids)
        ref, ref_lse = oracle_of(case, q, k, v, table, lens)
        for label, o, l in got:
            compare_out(o[b0:b1], ref, what=f"{case.name} {label} seqs {b0}..{b1 - 1}")
            compare_lse(l[b0:b1], ref_lse, what=f"{case.name} {label} seqs {b0}..{b1 - 1}")
        del q, k, v
        b0 = b1
        if b0 - done >= 32 or b0 == case.B:
            done = b0
            _say(f"[oracle] {case.name}: {b0} of {case.B} sequences checked")


@pytest.mark.parametrize("kv_dtype", ["fp16", "fp8"])
@pytest.mark.parametrize("name,P", [("llama8b_4k", 0), ("agentic_80k", 512), ("agentic_80k", 0),
                                    ("ragged_mixed", 0), ("agentic_80k_q48kv8", 512),
                                    ("agentic_80k_q40kv40", 512)])
def test_full_size_workload(name, P, kv_dtype):
    case = W.CONFIGS[name](device="cuda", kv_dtype=kv_dtype)
    out, lse = run(case, P)
    assert torch.isfinite(out.float()).all()
    # a rerun is bitwise identical
    out2, lse2 = run(case, P)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    del out2, lse2
    _check_every_sequence(case, [(f"P={P}", out, lse)])
    del case
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kv_dtype", ["fp16", "fp8"])
def test_full_size_partial_merge(kv_dtype):
    """32 sequences of 128K tokens as 4 range partials + merge_partials, and the
    single pass over the whole sequences: both against the oracle on every
    sequence, and against each other to fp16 ulps."""
    case = W.disagg_merge(device="cuda", kv_dtype=kv_dtype)
    views = W.range_views(case, case.ranges)
    o_parts = torch.empty((case.ranges, case.B, case.Hq, 128), dtype=torch.float32, device="cuda")
    l_parts = torch.empty((case.ranges, case.B, case.Hq), dtype=torch.float32, device="cuda")
    for r, (bt, ln) in enumerate(views):
        _say(f"[run] {case.name} range {r}")
        pda.paged_decode_attn_partial(case.q, case.k_cache, case.v_cache, bt, ln, case.scale,
                                      o=o_parts[r], lse=l_parts[r], **case.attn_kwargs())
    merged, mlse = pda.merge_partials(o_parts, l_parts)
    single, slse = run(case)
    compare_ulps(to_np(merged), to_np(single), ulps=2, rowwise=True)
    del o_parts, l_parts
    _check_every_sequence(case, [("4 partials + merge", merged, mlse),
                                 ("single pass", single, slse)])
    del case
    torch.cuda.empty_cache()


# --- KV append of the decoded token --------------------------------------------

def _bits(a):
    return np.ascontiguousarray(a).view(np.uint16)


@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (8, 2)])
def test_kv_append_then_attend(Hq, Hkv):
    lens = [0, 1, 2, 15, 16, 17, 31, 32, 33, 100, 256, 257]   # counts the appended token
    case = W.build_case(lens, Hq, Hkv, seed=12, device="cuda",
                        pool_blocks=sum(-(-n // 16) for n in lens) + 5)
    g = torch.Generator(device="cuda").manual_seed(13)
    kn = torch.randn((case.B, Hkv, 128), generator=g, device="cuda").half()
    vn = torch.randn((case.B, Hkv, 128), generator=g, device="cuda").half()
    q, k, v, table, ln = W.host_full(case)
    k_ref, v_ref = O.kv_append(k, v, kn.cpu().numpy(), vn.cpu().numpy(), table, ln)
    _say(f"[append] B={case.B} Hkv={Hkv}")
    pda.paged_kv_append(case.k_cache, case.v_cache, kn, vn, case.block_table, case.context_lens)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(case.k_cache.cpu().numpy()), _bits(k_ref))
    assert np.array_equal(_bits(case.v_cache.cpu().numpy()), _bits(v_ref))
    out, lse = run(case)
    ref, ref_lse = O.paged_decode_attention(q, k_ref, v_ref, table, ln, case.scale)
    compare_out(to_np(out), ref)
    compare_lse(to_np(lse), ref_lse)


def test_kv_append_full_size():
    case = W.llama8b_4k(device="cuda")
    g = torch.Generator(device="cuda").manual_seed(14)
    kn = torch.randn((case.B, 8, 128), generator=g, device="cuda").half()
    vn = torch.randn((case.B, 8, 128), generator=g, device="cuda").half()
    before = case.k_cache[::97].clone()
    pda.paged_kv_append(case.k_cache, case.v_cache, kn, vn, case.block_table, case.context_lens)
    torch.cuda.synchronize()
    last = torch.from_numpy(case.block_table_host[:, 255]).cuda()
    assert torch.equal(case.k_cache[last, 15], kn) and torch.equal(case.v_cache[last, 15], vn)
    touched = set(case.block_table_host[:, 255].tolist())
    rows = [i for i in range(0, case.num_blocks, 97) if i not in touched]
    assert torch.equal(case.k_cache[rows], before[[r // 97 for r in rows]])
    out, lse = run(case)
    _check_every_sequence(case, [("after append", out, lse)])
    del case
    torch.cuda.empty_cache()


@pytest.mark.parametrize("scale", [-0.0883883476, 0.5, 1e-3])
def test_scale_sign_and_size(scale):
    case = W.build_case(RAGGED, 32, 8, seed=15, device="cuda")
    case.scale = float(np.float32(scale))
    out, lse = run(case)
    ref, ref_lse = oracle_full(case)
    compare_out(to_np(out), ref)
    compare_lse(to_np(lse), ref_lse)


# --- FP8 (E4M3) KV cache --------------------------------------------------------

@pytest.mark.parametrize("P", [0, 64, 512])
def test_fp8_tiny_workload(P):
    case = W.tiny(device="cuda", kv_dtype="fp8")
    out, lse = run(case, P)
    ref, ref_lse = oracle_full(case)
    compare_out(to_np(out), ref)
    compare_lse(to_np(lse), ref_lse)


@pytest.mark.parametrize("G,Hkv", SHAPES)
def test_fp8_ragged_lengths(G, Hkv):
    case = W.build_case(RAGGED, G * Hkv, Hkv, pool_blocks=sum(-(-n // 16) for n in RAGGED) + 7,
                        seed=200 + G, device="cuda", name=f"ragged_fp8_G{G}", kv_dtype="fp8")
    out, lse = run(case)
    ref, ref_lse = oracle_full(case)
    compare_out(to_np(out), ref)
    compare_lse(to_np(lse), ref_lse)


def test_fp8_every_code_decodes_exactly():
    """One token per sequence: out = v_scale * value(code), for every finite code."""
    case = W.build_case([1] * 4, 32, 8, seed=16, device="cuda", kv_dtype="fp8")
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    v = case.v_cache.cpu().numpy()
    allc = np.resize(codes, 4 * 8 * 128).reshape(4, 8, 128)
    for b in range(4):
        v[int(case.block_table_host[b, 0]), 0] = allc[b]
    case.v_cache.copy_(torch.from_numpy(v))
    case.v_scale = 0.5                                   # a power of two keeps fp16 exact
    out, _ = run(case)
    want = (0.5 * O.fp8_e4m3_decode(allc)).astype(np.float16)
    for b in range(4):
        for h in range(32):
            assert np.array_equal(out[b, h].cpu().numpy(), want[b, h // 4]), (b, h)


def test_fp8_partial_api_and_merge():
    R, per = 4, 512
    case = W.build_case([R * per] * 3, 32, 8, seed=17, device="cuda", kv_dtype="fp8")
    cols = per // 16
    o_parts, l_parts = [], []
    for r in range(R):
        bt = case.block_table[:, r * cols:(r + 1) * cols]
        ln = torch.full((case.B,), per, dtype=torch.int32, device="cuda")
        o, l = pda.paged_decode_attn_partial(case.q, case.k_cache, case.v_cache, bt, ln,
                                             case.scale, **case.attn_kwargs())
        o_parts.append(o)
        l_parts.append(l)
    merged, mlse = pda.merge_partials(torch.stack(o_parts).contiguous(),
                                      torch.stack(l_parts).contiguous())
    single, _ = run(case)
    # p enters the FP8 PV products rounded to fp16, so the two schedules agree to
    # fp16 ulps of each row's scale (element-wise near zero they may differ more)
    compare_ulps(to_np(merged), to_np(single), ulps=2, rowwise=True)
    ref, ref_lse = oracle_full(case)
    compare_out(to_np(merged), ref)
    compare_lse(to_np(mlse), ref_lse)


# --- the largest sizes tested ------------------------------------------------------

def test_longest_context_one_million_tokens():
    """One sequence of 2^20 tokens (4 GiB of fp16 K/V, the whole GPU's runs
    splitting it, hundreds of partials per row for the merge).  The oracle
    checks two of the eight KV heads (it gathers 2^20 rows per head)."""
    case = W.build_case([1 << 20], 32, 8, seed=22, device="cuda", rng_backend="torch",
                        name="ctx_1m")
    out, lse = run(case)
    assert torch.isfinite(out.float()).all()
    q, k, v, table, lens = W.host_sequences(case, [0])
    kv_heads = [0, 7]
    q_heads = [h for g in kv_heads for h in range(4 * g, 4 * g + 4)]
    ref, ref_lse = O.paged_decode_attention(q[:, q_heads], k[:, :, kv_heads], v[:, :, kv_heads],
                                            table, lens, case.scale)
    compare_out(to_np(out)[0, q_heads], ref[0], what="ctx 2^20")
    compare_lse(to_np(lse)[0, q_heads], ref_lse[0], what="ctx 2^20")
    del case, k, v
    torch.cuda.empty_cache()


def test_many_sequences():
    """8192 sequences of 0 .. 299 tokens (every 97th empty) in one call."""
    rng = np.random.default_rng(23)
    lens = rng.integers(0, 300, size=8192)
    lens[::97] = 0
    case = W.build_case(lens, 32, 8, seed=23, device="cuda", rng_backend="torch", name="b8192")
    out, lse = run(case)
    o, l = to_np(out), to_np(lse)
    empty = np.flatnonzero(case.lens == 0)
    assert np.all(o[empty] == 0) and np.all(np.isneginf(l[empty]))
    _check_every_sequence(case, [("b8192", out, lse)])
    del case
    torch.cuda.empty_cache()


def test_binding_rejects_bad_buffers_before_a_launch():
    case = W.tiny(device="cuda")
    args = (case.q, case.k_cache, case.v_cache, case.block_table, case.context_lens, case.scale)
    B, Hq = case.B, case.Hq
    bad = [
        dict(out=torch.empty((B, Hq, 64), dtype=torch.float16, device="cuda")),
        dict(out=torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")),
        dict(out=torch.empty((B, Hq, 128), dtype=torch.float16)),                 # host memory
        dict(lse_out=torch.empty((B, Hq + 1), dtype=torch.float32, device="cuda")),
        dict(workspace=torch.empty(16, dtype=torch.uint8, device="cuda")),         # too small
        dict(workspace=torch.empty(1 << 20, dtype=torch.uint8)),                   # host memory
    ]
    for kw in bad:
        with pytest.raises(ValueError):
            pda.paged_decode_attn(*args, **kw)
    o = torch.zeros((2, B, Hq, 128), dtype=torch.float32, device="cuda")
    l = torch.zeros((2, B, Hq), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        pda.merge_partials(o, l, lse_out=torch.empty((B,), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        pda.merge_partials(o, l, out=torch.empty((B, Hq, 128), dtype=torch.float32,
                                                 device="cuda"))
    torch.cuda.synchronize()


# --- append fused into the attention call --------------------------------------------

def _new_rows(case, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    kn = torch.randn((case.B, case.Hkv, 128), generator=g, device="cuda").half()
    vn = torch.randn((case.B, case.Hkv, 128), generator=g, device="cuda").half()
    return kn, vn


def _fused_vs_separate(case, kn, vn, P=0, **kw):
    """paged_decode_attn_append on a copy of the caches against paged_kv_append +
    paged_decode_attn on the original: results and whole pools bit for bit."""
    k2, v2 = case.k_cache.clone(), case.v_cache.clone()
    sc = case.attn_kwargs()
    _say(f"[fused append] {case.name} B={case.B} Hq={case.Hq} Hkv={case.Hkv} P={P} "
         f"kv={case.kv_dtype} {kw}")
    out_f, lse_f = pda.paged_decode_attn_append(case.q, kn, vn, k2, v2, case.block_table,
                                                case.context_lens, case.scale, return_lse=True,
                                                partition_tokens=P, **sc, **kw)
    pda.paged_kv_append(case.k_cache, case.v_cache, kn, vn, case.block_table, case.context_lens,
                        **sc, **kw)
    out_s, lse_s = pda.paged_decode_attn(case.q, case.k_cache, case.v_cache, case.block_table,
                                         case.context_lens, case.scale, return_lse=True,
                                         partition_tokens=P, **sc, **kw)
    torch.cuda.synchronize()
    # bitwise (the pools' unowned slots hold NaN): compare the stored words
    word = torch.int16 if case.k_cache.element_size() == 2 else torch.uint8
    assert torch.equal(k2.view(word), case.k_cache.view(word))
    assert torch.equal(v2.view(word), case.v_cache.view(word))
    assert torch.equal(out_f, out_s) and torch.equal(lse_f, lse_s)
    return out_f, lse_f


@pytest.mark.parametrize("G,Hkv", [(1, 2), (2, 2), (4, 2), (8, 1), (4, 8), (6, 8), (1, 40),
                                   (2, 5)])
@pytest.mark.parametrize("P", [0, 32, 512])
def test_fused_append_equals_append_then_attend(G, Hkv, P):
    lens = [0, 1, 2, 15, 16, 17, 31, 32, 33, 100, 256, 257, 1000]
    case = W.build_case(lens, G * Hkv, Hkv, seed=300 + G, device="cuda",
                        pool_blocks=sum(-(-n // 16) for n in lens) + 5)
    kn, vn = _new_rows(case, 301 + G)
    q, k, v, table, ln = W.host_full(case)
    out, lse = _fused_vs_separate(case, kn, vn, P)
    k_ref, v_ref = O.kv_append(k, v, kn.cpu().numpy(), vn.cpu().numpy(), table, ln)
    ref, ref_lse = O.paged_decode_attention(q, k_ref, v_ref, table, ln, case.scale)
    compare_out(to_np(out), ref)
    compare_lse(to_np(lse), ref_lse)


def test_fused_append_skips_what_append_skips():
    # max_blocks_per_seq = 2 clamps the 40- and 33-token sequences (no append,
    # 32 tokens attended); sequence 3's tail frame lies outside the pool
    case = W.build_case([40, 5, 33, 20], 8, 2, seed=310, device="cuda")
    bt = case.block_table.clone()
    bt[3, 1] = case.k_cache.shape[0] + 7
    case.block_table = bt
    kn, vn = _new_rows(case, 311)
    _fused_vs_separate(case, kn, vn, 0, max_blocks_per_seq=2)


def test_fused_append_full_size():
    case = W.llama8b_4k(device="cuda")
    kn, vn = _new_rows(case, 312)
    _fused_vs_separate(case, kn, vn)
    del case
    torch.cuda.empty_cache()


@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (8, 2)])
def test_fp8_kv_append_then_attend(Hq, Hkv):
    lens = [0, 1, 2, 15, 16, 17, 31, 32, 33, 100, 256, 257]   # counts the appended token
    case = W.build_case(lens, Hq, Hkv, seed=320, device="cuda", kv_dtype="fp8",
                        pool_blocks=sum(-(-n // 16) for n in lens) + 5)
    g = torch.Generator(device="cuda").manual_seed(321)
    kn = torch.randn((case.B, Hkv, 128), generator=g, device="cuda").half()
    vn = torch.randn((case.B, Hkv, 128), generator=g, device="cuda").half()
    kn[3, 0, :4] = torch.tensor([1e4, -1e4, 60000.0, -0.0], dtype=torch.float16)   # saturate, -0
    vn[5, 1, :2] = torch.tensor([float("inf"), float("-inf")], dtype=torch.float16)
    k_host, v_host = case.k_cache.cpu().numpy(), case.v_cache.cpu().numpy()
    table, ln = case.block_table_host.copy(), case.lens.copy()
    k_ref, v_ref = O.kv_append_fp8(k_host, v_host, kn.cpu().numpy(), vn.cpu().numpy(), table, ln,
                                   case.k_scale, case.v_scale)
    _say(f"[append fp8] B={case.B} Hkv={Hkv}")
    pda.paged_kv_append(case.k_cache, case.v_cache, kn, vn, case.block_table, case.context_lens,
                        **case.attn_kwargs())
    torch.cuda.synchronize()
    assert np.array_equal(case.k_cache.cpu().numpy(), k_ref)     # every byte of both pools
    assert np.array_equal(case.v_cache.cpu().numpy(), v_ref)
    # attention over the appended cache (sequences whose new V row holds +-inf excluded)
    out, lse = run(case)
    q = case.q.cpu().numpy()
    ref, ref_lse = O.paged_decode_attention_fp8(q, k_ref, v_ref, table, ln, case.scale,
                                                case.k_scale, case.v_scale)
    keep = [b for b in range(case.B) if b != 5]
    compare_out(to_np(out)[keep], ref[keep])
    compare_lse(to_np(lse)[keep], ref_lse[keep])


@pytest.mark.parametrize("G,Hkv", [(1, 2), (4, 2), (8, 1), (4, 8), (6, 8), (1, 48), (4, 3)])
@pytest.mark.parametrize("P", [0, 64])
def test_fp8_fused_append_equals_append_then_attend(G, Hkv, P):
    lens = [0, 1, 2, 15, 16, 17, 31, 32, 33, 100, 256, 257, 1000]
    case = W.build_case(lens, G * Hkv, Hkv, seed=330 + G, device="cuda", kv_dtype="fp8",
                        pool_blocks=sum(-(-n // 16) for n in lens) + 5)
    kn, vn = _new_rows(case, 331 + G)
    kn[2, 0, :3] = torch.tensor([1e4, -1e4, -0.0], dtype=torch.float16)     # saturate, -0
    q, k, v, table, ln = W.host_full(case)
    out, lse = _fused_vs_separate(case, kn, vn, P)
    k_ref, v_ref = O.kv_append_fp8(k, v, kn.cpu().numpy(), vn.cpu().numpy(), table, ln,
                                   case.k_scale, case.v_scale)
    ref, ref_lse = O.paged_decode_attention_fp8(q, k_ref, v_ref, table, ln, case.scale,
                                                case.k_scale, case.v_scale)
    compare_out(to_np(out), ref)
    compare_lse(to_np(lse), ref_lse)


# FP8 calls whose block table allows contexts past 8192 tokens take up to 8 KV
# heads per work-group (4 otherwise): small ragged batches at a table 1024
# blocks wide, at the tuned occupancy, plain and with the fused append.
@pytest.mark.parametrize("G,Hkv", [(4, 8), (8, 8), (1, 32), (1, 40), (2, 16), (4, 2), (6, 5)])
@pytest.mark.parametrize("P", [0, 64, 512])
def test_fp8_wide_table_head_groups(G, Hkv, P):
    lens = [0, 1, 2, 17, 100, 257, 1000, 3000, 40]
    case = W.build_case(lens, G * Hkv, Hkv, seed=340 + G + Hkv, device="cuda", kv_dtype="fp8",
                        pool_blocks=sum(-(-n // 16) for n in lens) + 5, width=1024)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    lay = pda.workspace_layout(case.B, case.Hq, Hkv, 1024, P, kv_fp8=True)
    assert lay["n_runs"] == cus * 4 * 2 // Hkv
    out, lse = run(case, P)
    ref, ref_lse = oracle_full(case)
    compare_out(to_np(out), ref)
    compare_lse(to_np(lse), ref_lse)
    kn, vn = _new_rows(case, 341 + G)
    q, k, v, table, ln = W.host_full(case)
    out, lse = _fused_vs_separate(case, kn, vn, P)
    k_ref, v_ref = O.kv_append_fp8(k, v, kn.cpu().numpy(), vn.cpu().numpy(), table, ln,
                                   case.k_scale, case.v_scale)
    ref, ref_lse = O.paged_decode_attention_fp8(q, k_ref, v_ref, table, ln, case.scale,
                                                case.k_scale, case.v_scale)
    compare_out(to_np(out), ref)
    compare_lse(to_np(lse), ref_lse)


def test_fp8_fused_append_full_size():
    case = W.llama8b_4k(device="cuda", kv_dtype="fp8")
    kn, vn = _new_rows(case, 332)
    _fused_vs_separate(case, kn, vn)
    del case
    torch.cuda.empty_cache()


@pytest.mark.gpu
@pytest.mark.parametrize("nbytes", [16, 4096, (3 << 20) + 48])
def test_stream_read_reads_without_writing(nbytes):
    """The diagnostic streaming read (the bench's read ceiling) runs on odd sizes
    and leaves its sink alone: it writes nothing for an ordinary buffer."""
    buf = torch.arange(nbytes, dtype=torch.int32, device="cuda").to(torch.uint8)
    sink = torch.full((1,), -5, dtype=torch.int32, device="cuda")
    for nt in (False, True):
        pda.stream_read(buf, sink, nt)
    torch.cuda.synchronize()
    assert int(sink.item()) == -5


def _lds_probe_sums(form, iters):
    """Host model of pda_lds_probe: the wrapping sum each lane of a wave gets.

    Stage word i is i * 2654435761 mod 2^32; read r of a pass covers 64 lane
    shares of the form's width from r times 64 shares.  The transposed form
    (ds_read_b64_tr_b16) hands lane 4a + e of each 16-lane group, as its
    16-bit element b, element e of the 8-byte piece addressed by lane a + 4b of
    the group."""
    words = (np.arange(16384, dtype=np.uint64) * 2654435761) & 0xFFFFFFFF
    width = {0: 16, 1: 8, 2: 8, 3: 4}[form]
    sums = np.zeros(64, dtype=np.uint64)
    for r in range(16):
        for lane in range(64):
            if form == 2:
                grp, a, e = lane // 16 * 16, (lane % 16) // 4, lane % 4
                h = []
                for b in range(4):
                    addr = r * 64 * 8 + 8 * (grp + a + 4 * b) + 2 * e
                    h.append((int(words[addr // 4]) >> (16 * ((addr % 4) // 2))) & 0xFFFF)
                got = (h[0] | h[1] << 16) + (h[2] | h[3] << 16)
            else:
                first = (r * 64 * width + width * lane) // 4
                got = int(words[first:first + width // 4].sum())
            sums[lane] += got
    return (sums * iters) & 0xFFFFFFFF


@pytest.mark.gpu
@pytest.mark.parametrize("form", [0, 1, 2, 3])
def test_lds_probe_sums_what_each_form_reads(form):
    """The LDS read probe (the bench's calibration of the LDS counter) reads
    what its description says: every thread's sum matches the host model, for
    each of the 4 waves of each work-group."""
    iters, wgs = 3, 5
    out = torch.full((wgs * 256,), -1, dtype=torch.int32, device="cuda")
    pda.lds_probe(form, out, iters)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.int64) & 0xFFFFFFFF
    want = np.tile(_lds_probe_sums(form, iters).astype(np.int64), 4 * wgs)
    np.testing.assert_array_equal(got, want)


@pytest.mark.gpu
@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("G", [1, 2, 4, 6, 8])
@pytest.mark.parametrize("Hkv", [1, 2, 4, 8, 32, 40, 48])
def test_split_kernel_runs_at_the_tuned_occupancy(fp8, G, Hkv):
    """The schedule fills every CU with exactly the tuned waves per SIMD (the
    launch pads LDS when a kernel's registers would let more in): 1 for fp16
    with G <= 4, else 2; w waves per SIMD on 4 SIMDs give CUs * 4w / Hkv runs."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    w = 1 if (not fp8 and G <= 4) else 2
    lay = pda.workspace_layout(16, G * Hkv, Hkv, 64, 0, kv_fp8=fp8)
    assert lay["n_runs"] == cus * 4 * w // Hkv


@pytest.mark.parametrize("kv", ["fp16", "fp8"])
@pytest.mark.parametrize("nblk", list(range(1, 9)))
@pytest.mark.parametrize("last", [1, 7, 16])
def test_every_segment_length_of_the_ring(kv, nblk, last):
    """Sequence 0's partition is its whole context, so its single segment has
    nblk blocks (1..8 covers the ring's prologue, whole turns and last partial
    turn for rings of 2 to 4) and a last block with `last` valid tokens; the
    fused append on the same shapes matches append-then-attend bit for bit."""
    n = 16 * (nblk - 1) + last
    lens = [n, 3 * n + 5]
    case = W.build_case(lens, 8, 2, seed=900 + 10 * nblk + last, device="cuda", kv_dtype=kv,
                        pool_blocks=sum(-(-x // 16) for x in lens) + 4)
    P = 16 * nblk
    q, k, v, table, ln = W.host_full(case)
    out, lse = run(case, P)
    if kv == "fp8":
        ref, ref_lse = O.paged_decode_attention_fp8(q, k, v, table, ln, case.scale, case.k_scale,
                                                    case.v_scale)
    else:
        ref, ref_lse = O.paged_decode_attention(q, k, v, table, ln, case.scale)
    compare_out(to_np(out), ref)
    compare_lse(to_np(lse), ref_lse)
    kn, vn = _new_rows(case, 950 + nblk)
    _fused_vs_separate(case, kn, vn, P)
