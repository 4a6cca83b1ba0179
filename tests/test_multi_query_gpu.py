"""Multi-query and cascade attention on the GPU against the float64 oracle.

Every call goes through the C ABI (ctypes binding).  Small cases are checked
in full, and so are the full-size workloads (every query row, every request), in
the launch configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import decode_attention_paged_attn_amd as pda
from decode_attention_paged_attn_amd import workloads as W
import oracle.multi_query as MQ
import oracle.paged_attention as O
from tests.parity import compare_lse, compare_out, p_rounding_bound, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pda.load_library()
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _say(msg):
    print(msg, flush=True)


def run_mq(case, P=0, **kw):
    _say(f"[mq] {case.name} S={case.S} T={case.T} Hq={case.Hq} Hkv={case.Hkv} "
         f"causal={case.causal} P={P} kv={case.kv_dtype}")
    out, lse = pda.paged_multi_query_attn(case.q, case.k_cache, case.v_cache, case.block_table,
                                          case.context_lens, case.query_start, case.scale,
                                          causal=case.causal, return_lse=True,
                                          partition_tokens=P, **case.attn_kwargs(), **kw)
    torch.cuda.synchronize()
    return out, lse


def host_kv(case, k, v):
    """Host copies of (a gather of) the pools as the values they hold: an FP8
    pool's codes decoded by the oracle and multiplied by the tensor's scale."""
    k, v = k.cpu().numpy(), v.cpu().numpy()
    if case.kv_dtype == "fp8":
        return (case.k_scale * O.fp8_e4m3_decode(k), case.v_scale * O.fp8_e4m3_decode(v))
    return k, v


def host_mq(case):
    k, v = host_kv(case, case.k_cache, case.v_cache)
    return (case.q.cpu().numpy(), k, v, case.block_table_host.copy(), case.lens.copy(),
            case.query_start.cpu().numpy().astype(np.int64))


def oracle_mq(case):
    q, k, v, table, lens, qs = host_mq(case)
    return MQ.multi_query_attention(q, k, v, table, lens, qs, case.scale, causal=case.causal)


SMALL_LENS = [0, 1, 5, 16, 17, 40, 100, 257, 600, 33]
SMALL_NQ = [2, 1, 8, 3, 0, 17, 5, 33, 64, 1]


# the pages' GQA and MHA head shapes (Q32:KV8, Q48:KV8, Q64:KV8; Q32:KV32,
# Q40:KV40, Q48:KV48) and small or odd KV-head counts
SHAPES = [(1, 2), (2, 2), (4, 2), (8, 1), (4, 8), (6, 8), (8, 8), (6, 1), (1, 32), (1, 40),
          (1, 48), (4, 3), (2, 5), (1, 6), (8, 7), (6, 5)]


@pytest.mark.parametrize("G,Hkv", SHAPES)
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("P", [0, 32, 256])
def test_small_all_group_sizes(G, Hkv, causal, P):
    case = W.build_mq_case(SMALL_LENS, SMALL_NQ, G * Hkv, Hkv, causal=causal, seed=40 + G,
                           device="cuda", name=f"mq_small_G{G}")
    out, lse = run_mq(case, P)
    ref, ref_lse = oracle_mq(case)
    compare_out(to_np(out), ref)
    compare_lse(to_np(lse), ref_lse)


# The library picks its tile kernel from the average query rows per sequence
# (query tokens x G): up to 16 and 32 rows the register kernel with one or two
# 16-row blocks per wave, up to 64 the shared kernel with 64-row tiles, above
# that 128-row tiles (the wide kernel).  Each pattern lands in one of the four,
# at every group size.
VARIANT_ROWS = {"register16": 12, "register32": 28, "shared64": 48, "wide128": 200,
                "wide128_part": 100}   # 100 rows: the last wave of a tile is partly used


@pytest.mark.parametrize("G,Hkv", [(1, 2), (2, 2), (4, 2), (8, 1), (6, 8), (6, 1), (1, 40)])
@pytest.mark.parametrize("variant", sorted(VARIANT_ROWS))
@pytest.mark.parametrize("causal", [True, False])
def test_tile_kernel_variants(G, Hkv, variant, causal):
    per_seq = max(1, VARIANT_ROWS[variant] // G)
    lens = [per_seq + 3, 700, 95, per_seq]            # some sequences barely hold their queries
    nq = [per_seq] * len(lens)
    case = W.build_mq_case(lens, nq, G * Hkv, Hkv, causal=causal, seed=60 + G, device="cuda",
                           name=f"mq_{variant}_G{G}")
    for P in (0, 48):
        out, lse = run_mq(case, P)
        ref, ref_lse = oracle_mq(case)
        compare_out(to_np(out), ref)
        compare_lse(to_np(lse), ref_lse)


def test_single_query_is_decode():
    lens = [1, 2, 15, 16, 17, 100, 511, 1537]
    case = W.build_mq_case(lens, [1] * len(lens), 32, 8, causal=True, seed=41, device="cuda",
                           name="mq_one_query")
    out, lse = run_mq(case)
    dec, dlse = pda.paged_decode_attn(case.q, case.k_cache, case.v_cache, case.block_table,
                                      case.context_lens, case.scale, return_lse=True)
    q, k, v, table, ln, qs = host_mq(case)
    ref, ref_lse = O.paged_decode_attention(q, k, v, table, ln, case.scale)
    compare_out(to_np(out), ref)
    compare_out(to_np(dec), ref)
    compare_lse(to_np(lse), ref_lse)


def test_queries_past_context_and_empty():
    case = W.build_mq_case([3, 0, 20, 16], [5, 2, 0, 16], 8, 2, causal=True, seed=42,
                           device="cuda", name="mq_degenerate")
    out, lse = run_mq(case)
    o, l = to_np(out), to_np(lse)
    assert np.all(o[0:2] == 0) and np.all(np.isneginf(l[0:2]))      # see nothing
    assert np.all(o[5:7] == 0) and np.all(np.isneginf(l[5:7]))      # empty context
    ref, ref_lse = oracle_mq(case)
    compare_out(o, ref)
    compare_lse(l, ref_lse)


# One long sequence makes the runs of the wide kernel long (tens of units), so
# a run sweeps across many short tiles, some with no token to see (context 0,
# or every query before the first cached token), and a run's segments are
# visited last tile first: cut tiles with several partials, empty tiles and
# whole tiles all in one call.
@pytest.mark.parametrize("kv_dtype", ["fp16", "fp8"])
@pytest.mark.parametrize("causal", [True, False])
def test_wide_runs_across_many_tiles(kv_dtype, causal):
    rng = np.random.default_rng(7)
    short = [int(x) for x in rng.integers(1, 90, size=29)]
    lens = [60000] + short[:10] + [0] + short[10:20] + [3] + short[20:]
    nq = [40] * len(lens)                                  # 160 rows per sequence at G = 4
    case = W.build_mq_case(lens, nq, 8, 2, causal=causal, seed=91, device="cuda",
                           name=f"mq_wide_many_tiles_{kv_dtype}", kv_dtype=kv_dtype)
    ref, ref_lse = oracle_mq(case)
    for P in (0, 64):
        out, lse = run_mq(case, P)
        compare_out(to_np(out), ref)
        compare_lse(to_np(lse), ref_lse)


# The register kernel folds each run in two halves (two waves per KV head) and
# combines them through LDS when the split falls inside one tile.  That needs
# runs of two or more units: one long sequence makes them long, and a few short
# ones (at most 32 rows each, so the register kernel is picked) sit around it.
@pytest.mark.parametrize("kv_dtype", ["fp16", "fp8"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("G,Hkv", [(4, 1), (2, 2), (4, 3), (4, 8), (6, 5)])
def test_register_kernel_halves_combined(kv_dtype, causal, G, Hkv):
    rows = 32 if G != 6 else 30
    nq_long = rows // G
    lens = [7, 20000, 40, 3, 900]
    nq = [1, nq_long, 2, 3, max(1, nq_long - 1)]
    case = W.build_mq_case(lens, nq, G * Hkv, Hkv, causal=causal, seed=95 + G + Hkv,
                           device="cuda", name=f"mq_reg_halves_G{G}_{Hkv}", kv_dtype=kv_dtype)
    ws = torch.zeros(pda.multi_query_workspace_size(case.S, case.T, case.Hq, case.Hkv,
                                                    case.block_table.shape[1], 16),
                     dtype=torch.uint8, device="cuda")
    out, lse = run_mq(case, 16, workspace=ws)
    hdr = ws[:32].cpu().view(torch.int32).numpy()
    assert hdr[0] >= 2, f"runs of {hdr[0]} units: the two halves never share a tile"
    ref, ref_lse = oracle_mq(case)
    compare_out(to_np(out), ref)
    compare_lse(to_np(lse), ref_lse)


# Register-sized tiles (up to 32 rows) over an fp16 cache in a call with at
# least one (sequence, KV head) pair per CU and contexts of at most 8192 tokens
# go to the whole-tile kernel: one work-group per (tile, KV head), 8 waves over
# parts of the tile, combined in LDS; no plan, no merge, the workspace
# untouched.  FP8 calls of the same shape keep the planned path.  Ragged
# contexts (empty, shorter than the 8 parts, one block, several), query
# counts 0, 1 and more than one tile per sequence.
def _whole_tile_case(G, Hkv, rows, causal, kv_dtype, seed, S=None):
    rng = np.random.default_rng(seed)
    S = S or max(256 // Hkv + 5, 8)
    per_seq = max(1, rows // G)
    lens = rng.integers(0, 2500, size=S)
    lens[:6] = [0, 1, 15, 16, 17, 127]
    nq = rng.integers(1, per_seq + 1, size=S)
    nq[:4] = [0, per_seq, 1, 3 * per_seq + 1]       # none, one full tile, one query, 4 tiles
    lens[3] = max(lens[3], nq[3])
    return W.build_mq_case(lens.tolist(), nq.tolist(), G * Hkv, Hkv, causal=causal, seed=seed,
                           device="cuda", name=f"mq_whole_G{G}_{Hkv}_r{rows}", kv_dtype=kv_dtype)


def _untouched(ws):
    return bool((ws[:4096] == 0xAB).all())


@pytest.mark.parametrize("G,Hkv", [(4, 8), (8, 8), (2, 8), (1, 8), (6, 8), (4, 5), (1, 32)])
@pytest.mark.parametrize("rows", [12, 28])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("kv_dtype", ["fp16", "fp8"])
def test_whole_tile_kernel(G, Hkv, rows, causal, kv_dtype):
    case = _whole_tile_case(G, Hkv, rows, causal, kv_dtype, seed=300 + 7 * G + Hkv + rows)
    ws = torch.full((pda.multi_query_workspace_size(case.S, case.T, case.Hq, case.Hkv,
                                                    case.block_table.shape[1], 0),),
                    0xAB, dtype=torch.uint8, device="cuda")
    out, lse = run_mq(case, 0, workspace=ws)
    whole = kv_dtype == "fp16"
    assert _untouched(ws) == whole, f"expected the {'whole-tile' if whole else 'planned'} path"
    ref, ref_lse = oracle_mq(case)
    compare_out(to_np(out), ref)
    compare_lse(to_np(lse), ref_lse)


def test_whole_tile_partial_entry_point():
    case = _whole_tile_case(4, 8, 24, True, "fp16", seed=331)
    o, lse = pda.paged_multi_query_attn_partial(case.q, case.k_cache, case.v_cache,
                                                case.block_table, case.context_lens,
                                                case.query_start, case.scale, causal=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_mq(case)
    v = case.v_cache.cpu().numpy()
    compare_out(to_np(o), ref, abs_tol=p_rounding_bound(v))
    compare_lse(to_np(lse), ref_lse)


def test_planned_path_below_one_pair_per_cu():
    """Fewer (sequence, KV head) pairs than CUs keep the balanced run schedule."""
    case = _whole_tile_case(4, 8, 24, True, "fp16", seed=332, S=20)
    ws = torch.full((pda.multi_query_workspace_size(case.S, case.T, case.Hq, case.Hkv,
                                                    case.block_table.shape[1], 0),),
                    0xAB, dtype=torch.uint8, device="cuda")
    out, lse = run_mq(case, 0, workspace=ws)
    assert not _untouched(ws), "the plan kernel did not run"
    ref, ref_lse = oracle_mq(case)
    compare_out(to_np(out), ref)
    compare_lse(to_np(lse), ref_lse)


@pytest.mark.parametrize("P", [0, 64])
def test_partial_entry_point(P):
    case = W.build_mq_case(SMALL_LENS, SMALL_NQ, 16, 4, causal=True, seed=43, device="cuda",
                           name="mq_partial")
    o, lse = pda.paged_multi_query_attn_partial(case.q, case.k_cache, case.v_cache,
                                                case.block_table, case.context_lens,
                                                case.query_start, case.scale, causal=True,
                                                partition_tokens=P)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_mq(case)
    v = case.v_cache.cpu().numpy()
    compare_out(to_np(o), ref, abs_tol=p_rounding_bound(v))
    compare_lse(to_np(lse), ref_lse)


def test_bitwise_deterministic():
    case = W.build_mq_case(SMALL_LENS * 3, SMALL_NQ * 3, 32, 8, causal=True, seed=44,
                           device="cuda", name="mq_det")
    a, la = run_mq(case, 32)
    b, lb = run_mq(case, 32)
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_scale_sign_and_zero():
    case = W.build_mq_case([37, 300], [4, 9], 8, 2, causal=True, seed=45, device="cuda",
                           name="mq_scale")
    q, k, v, table, lens, qs = host_mq(case)
    for scale in (-0.2, 0.0):
        case.scale = scale
        out, lse = run_mq(case)
        ref, ref_lse = MQ.multi_query_attention(q, k, v, table, lens, qs, scale, causal=True)
        compare_out(to_np(out), ref)
        compare_lse(to_np(lse), ref_lse)


@pytest.mark.parametrize("kv_dtype", ["fp16", "fp8"])
@pytest.mark.parametrize("causal", [True, False])
def test_wide_scale_sign_and_zero(kv_dtype, causal):
    # 60 queries x G = 4 = 240 rows per sequence: the wide tile kernel, whose fold
    # takes exp2 of a masked (-inf) score times the kernels' score scale as 0.
    # Scale 0 gives the uniform softmax over each query's visible tokens, a
    # negative scale flips every score; P = 48 also cuts tiles between runs.
    case = W.build_mq_case([300, 70, 1100], [60, 60, 60], 8, 2, causal=causal, seed=47,
                           device="cuda", name=f"mq_wide_scale_{kv_dtype}", kv_dtype=kv_dtype)
    q, k, v, table, lens, qs = host_mq(case)
    for scale in (-0.2, 0.0):
        case.scale = scale
        ref, ref_lse = MQ.multi_query_attention(q, k, v, table, lens, qs, scale, causal=causal)
        for P in (0, 48):
            out, lse = run_mq(case, P)
            compare_out(to_np(out), ref)
            compare_lse(to_np(lse), ref_lse)


def test_graph_capture_replays_match_eager():
    case = W.build_mq_case(SMALL_LENS, SMALL_NQ, 32, 8, causal=True, seed=46, device="cuda",
                           name="mq_graph")
    ws = torch.empty(pda.multi_query_workspace_size(case.S, case.T, 32, 8,
                                                    case.block_table.shape[1]),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((case.T, 32, 128), dtype=torch.float16, device="cuda")
    lse = torch.empty((case.T, 32), dtype=torch.float32, device="cuda")
    eager, eager_lse = run_mq(case, workspace=ws)
    eager, eager_lse = eager.clone(), eager_lse.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            pda.paged_multi_query_attn(case.q, case.k_cache, case.v_cache, case.block_table,
                                       case.context_lens, case.query_start, case.scale,
                                       causal=True, out=out, lse_out=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    for i in range(3):
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager) and torch.equal(lse, eager_lse), f"replay {i}"


# --- FP8 (E4M3) cache -------------------------------------------------------------

@pytest.mark.parametrize("G,Hkv", SHAPES)
@pytest.mark.parametrize("causal", [True, False])
def test_fp8_small_all_group_sizes(G, Hkv, causal):
    case = W.build_mq_case(SMALL_LENS, SMALL_NQ, G * Hkv, Hkv, causal=causal, seed=140 + G,
                           device="cuda", name=f"mq_small_fp8_G{G}", kv_dtype="fp8")
    for P in (0, 32):
        out, lse = run_mq(case, P)
        ref, ref_lse = oracle_mq(case)
        compare_out(to_np(out), ref)
        compare_lse(to_np(lse), ref_lse)


@pytest.mark.parametrize("G,Hkv", [(1, 2), (4, 2), (8, 1), (6, 8), (6, 1)])
@pytest.mark.parametrize("variant", sorted(VARIANT_ROWS))
def test_fp8_tile_kernel_variants(G, Hkv, variant):
    per_seq = max(1, VARIANT_ROWS[variant] // G)
    lens = [per_seq + 3, 700, 95, per_seq]
    case = W.build_mq_case(lens, [per_seq] * len(lens), G * Hkv, Hkv, causal=True,
                           seed=160 + G, device="cuda", name=f"mq_{variant}_fp8_G{G}",
                           kv_dtype="fp8")
    for P in (0, 48):
        out, lse = run_mq(case, P)
        ref, ref_lse = oracle_mq(case)
        compare_out(to_np(out), ref)
        compare_lse(to_np(lse), ref_lse)


def test_fp8_partial_and_one_query_is_decode():
    lens = [1, 2, 15, 16, 17, 100, 511, 1537]
    case = W.build_mq_case(lens, [1] * len(lens), 32, 8, causal=True, seed=141, device="cuda",
                           name="mq_one_query_fp8", kv_dtype="fp8")
    out, lse = run_mq(case)
    o, l = pda.paged_multi_query_attn_partial(case.q, case.k_cache, case.v_cache,
                                              case.block_table, case.context_lens,
                                              case.query_start, case.scale, causal=True,
                                              **case.attn_kwargs())
    dec = pda.paged_decode_attn(case.q, case.k_cache, case.v_cache, case.block_table,
                                case.context_lens, case.scale, **case.attn_kwargs())
    torch.cuda.synchronize()
    ref, ref_lse = oracle_mq(case)
    compare_out(to_np(out), ref)
    compare_out(to_np(dec), ref)
    compare_lse(to_np(lse), ref_lse)
    _, _, v, *_ = host_mq(case)
    compare_out(to_np(o), ref, abs_tol=p_rounding_bound(v))
    compare_lse(to_np(l), ref_lse)


def test_fp8_needs_scales():
    case = W.build_mq_case([40], [2], 8, 2, seed=142, device="cuda", kv_dtype="fp8")
    with pytest.raises(ValueError):
        pda.paged_multi_query_attn(case.q, case.k_cache, case.v_cache, case.block_table,
                                   case.context_lens, case.query_start, case.scale)


# --- cascade (shared prefix) ----------------------------------------------------

def host_cascade(c):
    k, v = host_kv(c, c.k_cache, c.v_cache)
    return (c.q.cpu().numpy(), k, v, c.prefix_table_host, c.prefix_lens_host, c.group_start_host,
            c.suffix_table_host, c.suffix_lens_host)


def run_cascade(c):
    _say(f"[cascade] {c.name} B={c.B} groups={len(c.prefix_lens_host)} kv={c.kv_dtype}")
    out, lse = pda.cascade_decode_attn(c.q, c.k_cache, c.v_cache, c.prefix_table, c.prefix_lens,
                                       c.group_start, c.suffix_table, c.suffix_lens, c.scale,
                                       return_lse=True, **c.attn_kwargs())
    torch.cuda.synchronize()
    return out, lse


def test_cascade_page_example_shape():
    """50 requests sharing a 1000-token prefix, as in the page's worked example."""
    rng = np.random.default_rng(47)
    suffix = rng.integers(0, 200, size=50)
    c = W.build_cascade_case([1000], [50], suffix, 32, 8, seed=47, device="cuda",
                             name="cascade_r50_p1000")
    out, lse = run_cascade(c)
    ref, ref_lse = MQ.cascade_attention(*host_cascade(c), c.scale)
    compare_out(to_np(out), ref)
    compare_lse(to_np(lse), ref_lse)


@pytest.mark.parametrize("G,Hkv", [(1, 2), (4, 2), (8, 1), (6, 8), (1, 40)])
def test_cascade_groups_and_edges(G, Hkv):
    # group 2 has an empty prefix; some requests have no suffix
    c = W.build_cascade_case([64, 37, 0, 16], [3, 5, 2, 1], [5, 0, 17, 16, 1, 40, 0, 3, 9, 0, 2],
                             G * Hkv, Hkv, seed=48 + G, device="cuda", name=f"cascade_G{G}")
    out, lse = run_cascade(c)
    ref, ref_lse = MQ.cascade_attention(*host_cascade(c), c.scale)
    compare_out(to_np(out), ref)
    compare_lse(to_np(lse), ref_lse)


@pytest.mark.parametrize("G,Hkv", [(1, 2), (4, 2), (8, 1), (6, 8)])
def test_cascade_fp8(G, Hkv):
    c = W.build_cascade_case([64, 37, 0, 16], [3, 5, 2, 1], [5, 0, 17, 16, 1, 40, 0, 3, 9, 0, 2],
                             G * Hkv, Hkv, seed=148 + G, device="cuda",
                             name=f"cascade_fp8_G{G}", kv_dtype="fp8")
    out, lse = run_cascade(c)
    ref, ref_lse = MQ.cascade_attention(*host_cascade(c), c.scale)
    compare_out(to_np(out), ref)
    compare_lse(to_np(lse), ref_lse)


def test_cascade_equals_naive_decode():
    c = W.build_cascade_case([256, 512], [6, 4], list(range(1, 200, 20)), 32, 8, seed=50,
                             device="cuda", name="cascade_vs_naive")
    out, _ = run_cascade(c)
    table, lens = c.naive_table()
    naive = pda.paged_decode_attn(c.q, c.k_cache, c.v_cache, table, lens, c.scale)
    torch.cuda.synchronize()
    ref, _ = MQ.cascade_attention(*host_cascade(c), c.scale)
    compare_out(to_np(out), ref)
    compare_out(to_np(naive), ref)


# --- full-size workloads, every row --------------------------------------------

@pytest.mark.parametrize("kv_dtype", ["fp16", "fp8"])
@pytest.mark.parametrize("config", ["spec_verify", "chunked_prefill"])
def test_full_size_every_row(config, kv_dtype):
    """Every query row of the full-size workload against the oracle."""
    case = W.MQ_CONFIGS[config](device="cuda", kv_dtype=kv_dtype)
    out, lse = run_mq(case)
    o, l = to_np(out), to_np(lse)
    assert np.all(np.isfinite(o))
    ref, ref_lse = oracle_mq(case)
    _say(f"[oracle] {case.name}: {case.T} query rows")
    compare_out(o, ref, what=case.name)
    compare_lse(l, ref_lse, what=case.name)
    del case
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kv_dtype", ["fp16", "fp8"])
def test_full_size_cascade_every_request(kv_dtype):
    """All 200 requests of the shared-prefix workload against the oracle's
    attention over each request's prefix followed by its suffix."""
    c = W.shared_prefix(device="cuda", kv_dtype=kv_dtype)
    out, lse = run_cascade(c)
    o, l = to_np(out), to_np(lse)
    assert np.all(np.isfinite(o))
    ref, ref_lse = MQ.cascade_attention(*host_cascade(c), c.scale)
    _say(f"[oracle] {c.name}: {c.B} requests")
    compare_out(o, ref, what=c.name)
    compare_lse(l, ref_lse, what=c.name)
    del c
    torch.cuda.empty_cache()


def test_most_sequences_per_call():
    """4000 sequences, the most one call takes, with 0 .. 4 causal queries each."""
    rng = np.random.default_rng(53)
    S = 4000
    lens = rng.integers(1, 200, size=S)
    nq = np.minimum(rng.integers(0, 5, size=S), lens)
    case = W.build_mq_case(lens, nq, 8, 2, causal=True, seed=53, device="cuda",
                           rng_backend="torch", name="mq_s4000")
    out, lse = run_mq(case)
    o, l = to_np(out), to_np(lse)
    assert np.all(np.isfinite(o))
    ref, ref_lse = oracle_mq(case)
    compare_out(o, ref, what="4000 sequences")
    compare_lse(l, ref_lse, what="4000 sequences")


def test_binding_rejects_bad_buffers_before_a_launch():
    case = W.build_mq_case([40, 9], [3, 2], 8, 2, seed=54, device="cuda")
    args = (case.q, case.k_cache, case.v_cache, case.block_table, case.context_lens,
            case.query_start, case.scale)
    T, Hq = case.T, case.Hq
    bad = [
        dict(out=torch.empty((T + 1, Hq, 128), dtype=torch.float16, device="cuda")),
        dict(out=torch.empty((T, Hq, 128), dtype=torch.float16)),                  # host memory
        dict(lse_out=torch.empty((T, Hq), dtype=torch.float16, device="cuda")),
        dict(workspace=torch.empty(16, dtype=torch.uint8, device="cuda")),          # too small
        dict(workspace=torch.empty(1 << 22, dtype=torch.uint8)),                    # host memory
    ]
    for kw in bad:
        with pytest.raises(ValueError):
            pda.paged_multi_query_attn(*args, **kw)
    torch.cuda.synchronize()
