"""paged_decode_attn_noalloc (the library's fixed device scratch as the split-K
workspace) against paged_decode_attn with a caller workspace, through the C ABI.

Two calls in a row, the second on a smaller batch, each bitwise equal to the
entry point with a workspace and within the decode tolerance of the oracle;
then a shape whose workspace exceeds the scratch is rejected before a launch.
"""
import numpy as np
import pytest
import torch

import decode_attention_paged_attn_amd as pda
from decode_attention_paged_attn_amd import workloads as W
import oracle.paged_attention as O
from tests.parity import compare_lse, compare_out, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pda.load_library()
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _both(case, P):
    print(f"[noalloc] {case.name} B={case.B} Hq={case.Hq} Hkv={case.Hkv} P={P}", flush=True)
    out = torch.full((case.B, case.Hq, 128), 7.0, dtype=torch.float16, device="cuda")
    lse = torch.full((case.B, case.Hq), 7.0, dtype=torch.float32, device="cuda")
    pda.paged_decode_attn_noalloc(case.q, case.k_cache, case.v_cache, case.block_table,
                                  case.context_lens, case.scale, out, lse_out=lse,
                                  partition_tokens=P)
    ref_out, ref_lse = pda.paged_decode_attn(case.q, case.k_cache, case.v_cache, case.block_table,
                                             case.context_lens, case.scale, return_lse=True,
                                             partition_tokens=P)
    torch.cuda.synchronize()
    return out, lse, ref_out, ref_lse


def test_two_calls_second_smaller_match_the_workspace_entry_point():
    big = W.build_case([9000, 1, 4096, 20000, 333, 77777, 16, 5000], 32, 8, seed=71,
                       device="cuda", rng_backend="torch", name="noalloc_big")
    out, lse, ref_out, ref_lse = _both(big, 256)
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    q, k, v, table, lens = W.host_sequences(big, list(range(big.B)))
    ref, rl = O.paged_decode_attention(q, k, v, table, lens, big.scale)
    compare_out(to_np(out), ref)
    compare_lse(to_np(lse), rl)
    del big, k, v
    # the second call: fewer sequences, fewer heads, another unit length; the
    # scratch still holds the first call's partials
    small = W.build_case([37, 512, 1500], 8, 2, seed=72, device="cuda", name="noalloc_small")
    out, lse, ref_out, ref_lse = _both(small, 64)
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    ref, rl = O.paged_decode_attention(*W.host_full(small), small.scale)
    compare_out(to_np(out), ref)
    compare_lse(to_np(lse), rl)


def test_too_large_for_the_scratch_is_rejected():
    # 4096 sequences x 32 heads: the partial slots alone need more than 32 MiB
    B = 4096
    lens = np.full(B, 16)
    case = W.build_case(lens, 32, 8, seed=73, device="cuda", rng_backend="torch",
                        poison=False, name="noalloc_too_big")
    need = pda.workspace_size(B, 32, 8, case.block_table.shape[1])
    assert need > (32 << 20)
    out = torch.full((B, 32, 128), 7.0, dtype=torch.float16, device="cuda")
    with pytest.raises(pda.PdaError) as e:
        pda.paged_decode_attn_noalloc(case.q, case.k_cache, case.v_cache, case.block_table,
                                      case.context_lens, case.scale, out)
    assert e.value.code == 2 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())           # nothing was launched
