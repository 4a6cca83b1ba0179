"""Seeded synthetic decode-attention workloads over a paged KV cache.

This module only draws inputs: context lengths, a shuffled physical block pool
dealt out as block tables, and N(0, 1) fp16 queries, keys and values.  It holds
none of the attention arithmetic, so both the HIP path and the float64 checker
can be fed from it.

Shapes follow the pages' workloads:

* Llama-3.1-8B attention: 32 query heads, 8 KV heads, head dim 128, fp16 KV
  (KernelFlume paper §6.1 "Implementation and Setup"; the batch-64, ~4K-token
  capacity example in §1 "Introduction").
* 16-token blocks (16 tokens per block by default in "Optimising decode in
  vLLM", section 1; B_size = 16 in "Physical Memory Block Layout" of the
  disaggregated-inference page).
* Agentic long-context sessions with a median of roughly 80K tokens and tails
  above 200K (KernelFlume paper §1 and §2.1).  The trace itself is not used;
  a clipped log-normal with that median stands in for it.

Draw order for a seed: context lengths, then the pool permutation, then Q,
then the K pool, then the V pool.  Small cases draw everything with numpy's
PCG64; large pools draw Q/K/V with a torch generator on the target device
(the lengths and tables still come from PCG64), so multi-GiB pools never pass
through host memory.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

BLOCK_SIZE = 16
HEAD_DIM = 128
K_POISON = 6.0e4        # would dominate any softmax it leaked into
V_POISON = float("nan")  # would turn any output it leaked into into NaN
FP8_POISON = 0x7F        # the E4M3 NaN code, for both FP8 pools
FP8_MAX = 448.0          # largest finite E4M3 value


@dataclasses.dataclass
class Case:
    """One decode-attention batch: device tensors plus the host-side recipe."""
    name: str
    q: torch.Tensor              # [B, Hq, D] fp16
    k_cache: torch.Tensor        # [num_blocks, bs, Hkv, D] fp16
    v_cache: torch.Tensor        # [num_blocks, bs, Hkv, D] fp16
    block_table: torch.Tensor    # [B, width] int32, -1 past each sequence's blocks
    context_lens: torch.Tensor   # [B] int32
    scale: float                 # fp32-representable 1/sqrt(D)
    lens: np.ndarray             # host copy of context_lens (int64)
    block_table_host: np.ndarray  # host copy of block_table (int64)
    seed: int
    rng_backend: str
    partition_tokens: int = 0    # 0 = let the library choose
    ranges: int = 0              # token ranges for the partial + merge workload
    kv_dtype: str = "fp16"       # "fp16", or "fp8": E4M3 codes (uint8) with per-tensor scales
    k_scale: float = 1.0
    v_scale: float = 1.0

    @property
    def kv_bytes_per_elem(self):
        return 1 if self.kv_dtype == "fp8" else 2

    def attn_kwargs(self):
        """The scale arguments paged_decode_attn needs for this cache."""
        return {"k_scale": self.k_scale, "v_scale": self.v_scale} if self.kv_dtype == "fp8" else {}

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def Hq(self):
        return self.q.shape[1]

    @property
    def Hkv(self):
        return self.k_cache.shape[2]

    @property
    def D(self):
        return self.q.shape[2]

    @property
    def num_blocks(self):
        return self.k_cache.shape[0]


def fp32_scale(head_dim: int) -> float:
    """1/sqrt(D) rounded to fp32, the value passed to the kernels."""
    return float(np.float32(1.0 / math.sqrt(head_dim)))


def _deal_blocks(lens, pool_blocks, width, perm, bs):
    nblk = [-(-int(n) // bs) for n in lens]
    if sum(nblk) > pool_blocks:
        raise ValueError("pool too small for the requested lengths")
    table = np.full((len(lens), width), -1, dtype=np.int64)
    off = 0
    for b, k in enumerate(nblk):
        table[b, :k] = perm[off:off + k]
        off += k
    return table, off


def build_case(lens, Hq, Hkv, *, D=HEAD_DIM, bs=BLOCK_SIZE, pool_blocks=None,
               width=None, seed=0, device="cpu", poison=True,
               rng_backend="numpy", name="custom", rng=None,
               partition_tokens=0, ranges=0, kv_dtype="fp16") -> Case:
    """Draw Q, a shuffled K/V pool and block tables for the given lengths.

    ``pool_blocks`` defaults to exactly the blocks the lengths need; extra pool
    blocks are unused and, like the slots past each sequence's last token,
    filled with K = +-6e4 and V = NaN when ``poison`` is set.

    ``kv_dtype="fp8"``: the N(0, 1) pools are quantised to E4M3 codes with one
    scale per pool, amax / 448 (the per-tensor scales of an FP8 KV cache), by
    torch's float8_e4m3fn conversion (round to nearest even); unowned slots
    then hold the NaN code in both pools.
    """
    lens = np.asarray(lens, dtype=np.int64)
    B = len(lens)
    nblk = -(-lens // bs)
    need = int(nblk.sum())
    pool_blocks = need if pool_blocks is None else int(pool_blocks)
    pool_blocks = max(pool_blocks, 1)
    width = max(int(nblk.max()) if B else 1, 1) if width is None else int(width)
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    perm = rng.permutation(pool_blocks)
    table, used = _deal_blocks(lens, pool_blocks, width, perm, bs)

    if rng_backend == "numpy":
        q = rng.standard_normal((B, Hq, D), dtype=np.float32).astype(np.float16)
        k = rng.standard_normal((pool_blocks, bs, Hkv, D), dtype=np.float32).astype(np.float16)
        v = rng.standard_normal((pool_blocks, bs, Hkv, D), dtype=np.float32).astype(np.float16)
        q_t = torch.from_numpy(q).to(device)
        k_t = torch.from_numpy(k).to(device)
        v_t = torch.from_numpy(v).to(device)
    elif rng_backend == "torch":
        gen = torch.Generator(device=device)
        gen.manual_seed(int(seed))
        q_t = torch.randn((B, Hq, D), generator=gen, device=device,
                          dtype=torch.float32).to(torch.float16)
        k_t = torch.empty((pool_blocks, bs, Hkv, D), dtype=torch.float16, device=device)
        v_t = torch.empty_like(k_t)
        chunk = max(1, (1 << 26) // (bs * Hkv * D))
        for dst in (k_t, v_t):
            for lo in range(0, pool_blocks, chunk):
                hi = min(lo + chunk, pool_blocks)
                dst[lo:hi] = torch.randn((hi - lo, bs, Hkv, D), generator=gen,
                                         device=device, dtype=torch.float32)
    else:
        raise ValueError(rng_backend)

    k_scale = v_scale = 1.0
    if kv_dtype == "fp8":
        k_t, k_scale = _to_fp8(k_t)
        v_t, v_scale = _to_fp8(v_t)
    elif kv_dtype != "fp16":
        raise ValueError(kv_dtype)

    if poison:
        _poison(k_t, v_t, lens, table, perm[used:], bs, rng)

    return Case(name=name, q=q_t, k_cache=k_t, v_cache=v_t, kv_dtype=kv_dtype,
                k_scale=k_scale, v_scale=v_scale,
                block_table=torch.from_numpy(table.astype(np.int32)).to(device),
                context_lens=torch.from_numpy(lens.astype(np.int32)).to(device),
                scale=fp32_scale(D), lens=lens, block_table_host=table, seed=seed,
                rng_backend=rng_backend, partition_tokens=partition_tokens,
                ranges=ranges)


def _to_fp8(pool):
    """E4M3 codes (uint8) of pool / s and the per-tensor scale s = amax / 448."""
    amax = max(float(pool.abs().max()), 1e-12)
    scale = float(np.float32(amax / FP8_MAX))
    codes = torch.empty(pool.shape, dtype=torch.uint8, device=pool.device)
    chunk = max(1, (1 << 26) // max(1, pool[0].numel()))
    for lo in range(0, pool.shape[0], chunk):
        x = pool[lo:lo + chunk].float() / scale
        codes[lo:lo + chunk] = x.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale


def _poison(k_t, v_t, lens, table, unused_blocks, bs, rng):
    """Fill every slot no sequence owns: unused blocks and last-block tails."""
    Hkv, D = k_t.shape[2], k_t.shape[3]
    dev = k_t.device
    if k_t.dtype == torch.uint8:                   # FP8 codes: the NaN code everywhere
        blk, slot = _unowned_slots(lens, table, bs)
        if len(unused_blocks):
            idx = torch.from_numpy(np.asarray(unused_blocks, dtype=np.int64)).to(dev)
            k_t[idx] = FP8_POISON
            v_t[idx] = FP8_POISON
        if blk:
            bi = torch.tensor(blk, dtype=torch.int64, device=dev)
            si = torch.tensor(slot, dtype=torch.int64, device=dev)
            k_t[bi, si] = FP8_POISON
            v_t[bi, si] = FP8_POISON
        return
    if len(unused_blocks):
        idx = torch.from_numpy(np.asarray(unused_blocks, dtype=np.int64)).to(dev)
        sign = torch.from_numpy(rng.choice([-1.0, 1.0], size=(len(unused_blocks), bs, Hkv, D))
                                .astype(np.float16)).to(dev)
        k_t[idx] = sign * K_POISON
        v_t[idx] = V_POISON
    blk, slot = _unowned_slots(lens, table, bs)
    if blk:
        bi = torch.tensor(blk, dtype=torch.int64, device=dev)
        si = torch.tensor(slot, dtype=torch.int64, device=dev)
        k_t[bi, si] = K_POISON
        v_t[bi, si] = V_POISON


def _unowned_slots(lens, table, bs):
    """(frame, slot) lists of the slots past each sequence's last token."""
    blk, slot = [], []
    for b, n in enumerate(lens):
        n = int(n)
        if n % bs:
            last = int(table[b, (n - 1) // bs])
            for s in range(n % bs, bs):
                blk.append(last)
                slot.append(s)
    return blk, slot


# --- the pages' workloads -----------------------------------------------------

K1 = 1024   # "K" token counts are binary: 8K = 8192, 128K = 131072


def _suffix(kv_dtype):
    return "" if kv_dtype == "fp16" else "_" + kv_dtype


def tiny(seed=0, device="cpu", poison=True, kv_dtype="fp16"):
    """Batch 2, 8 query / 2 KV heads, context {37, 512}, 35 of a 128-block pool."""
    return build_case([37, 512], 8, 2, pool_blocks=128, seed=seed, device=device,
                      poison=poison, rng_backend="numpy", kv_dtype=kv_dtype,
                      name="tiny_b2_ctx37_512" + _suffix(kv_dtype))


def llama8b_4k(seed=0, device="cpu", rng_backend="torch", kv_dtype="fp16"):
    """Llama-3.1-8B layer: batch 64, 32/8 heads, every context 4096 tokens."""
    return build_case([4096] * 64, 32, 8, seed=seed, device=device, kv_dtype=kv_dtype,
                      rng_backend=rng_backend, name="llama8b_b64_ctx4096" + _suffix(kv_dtype))


def agentic_lengths(rng, B=16, median=80 * K1, sigma=0.42, lo=8 * K1, hi=200 * K1):
    """Clipped log-normal context lengths with the trace's ~80K median.

    sigma = 0.42 puts the expected maximum of ~610 sessions near the ~273K tail
    quoted for the trace: ln(273/80) / Phi^-1(1 - 1/610) = 1.2275 / 2.94.
    """
    z = rng.standard_normal(B)
    return np.clip(np.rint(np.exp(math.log(median) + sigma * z)), lo, hi).astype(np.int64)


def agentic_80k(seed=0, device="cpu", rng_backend="torch", kv_dtype="fp16", heads=(32, 8)):
    """Long-context agentic decode: batch 16, 32/8 heads, P = 512 partitions.

    ``heads`` = (Hq, Hkv) gives the other head shapes the KernelFlume paper
    evaluates (§6.3): GQA Q48:KV8, Q64:KV8 and MHA Q32:KV32, Q40:KV40,
    Q48:KV48, on the same lengths.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = agentic_lengths(rng)
    Hq, Hkv = heads
    shape = "" if (Hq, Hkv) == (32, 8) else f"_q{Hq}kv{Hkv}"
    return build_case(lens, Hq, Hkv, seed=seed, device=device, rng=rng, kv_dtype=kv_dtype,
                      rng_backend=rng_backend,
                      name="agentic_b16_median80k" + shape + _suffix(kv_dtype),
                      partition_tokens=512)


def ragged_lengths(rng, B=256):
    """Uniform on [1, 32K], then 10% of sequences set to 1 and 5% to 128K."""
    lens = rng.integers(1, 32 * K1, size=B, endpoint=True).astype(np.int64)
    order = rng.permutation(B)
    n_one, n_long = round(0.10 * B), round(0.05 * B)
    lens[order[:n_one]] = 1
    lens[order[n_one:n_one + n_long]] = 128 * K1
    return lens


def ragged_mixed(seed=0, device="cpu", rng_backend="torch", kv_dtype="fp16"):
    """Mixed ragged batch: 256 sequences, 32/8 heads."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = ragged_lengths(rng)
    return build_case(lens, 32, 8, seed=seed, device=device, rng=rng, kv_dtype=kv_dtype,
                      rng_backend=rng_backend, name="ragged_b256_u32k" + _suffix(kv_dtype))


def disagg_merge(seed=0, device="cpu", rng_backend="torch", kv_dtype="fp16"):
    """Batch 32, 32/8 heads, 128K tokens each, split into 4 token ranges."""
    return build_case([128 * K1] * 32, 32, 8, seed=seed, device=device, kv_dtype=kv_dtype,
                      rng_backend=rng_backend, name="disagg_b32_ctx128k_r4" + _suffix(kv_dtype),
                      ranges=4)


def range_views(case: Case, R: int):
    """Block-table column slices and lengths of R equal contiguous token ranges.

    Each range must be a whole number of blocks of every sequence; the slices
    are strided views of the one table, as a node owning the range would see.
    """
    width = case.block_table.shape[1]
    if width % R:
        raise ValueError("table width must split into R equal ranges")
    cols = width // R
    toks = cols * BLOCK_SIZE
    if not np.all(case.lens == case.lens[0]) or case.lens[0] != toks * R:
        raise ValueError("range_views expects every sequence to fill the table")
    views = []
    for r in range(R):
        bt = case.block_table[:, r * cols:(r + 1) * cols]
        ln = torch.full((case.B,), toks, dtype=torch.int32, device=case.block_table.device)
        views.append((bt, ln))
    return views


def host_sequences(case: Case, seq_ids):
    """Host copies of Q and of the blocks of the chosen sequences.

    Returns (q [n, Hq, D] fp16, k_pool, v_pool [sum blocks, bs, Hkv, D] fp16,
    block_table [n, width] int64, lens [n]); the blocks are renumbered in the
    order they are copied, so the returned table indexes the returned pools.
    """
    seq_ids = [int(b) for b in seq_ids]
    lens = case.lens[seq_ids]
    nblk = -(-lens // BLOCK_SIZE)
    width = max(int(nblk.max()), 1)
    table = np.full((len(seq_ids), width), -1, dtype=np.int64)
    frames = []
    off = 0
    for i, b in enumerate(seq_ids):
        k = int(nblk[i])
        frames.extend(int(x) for x in case.block_table_host[b, :k])
        table[i, :k] = np.arange(off, off + k)
        off += k
    idx = torch.tensor(frames, dtype=torch.int64, device=case.k_cache.device)
    k_pool = case.k_cache.index_select(0, idx).cpu().numpy()
    v_pool = case.v_cache.index_select(0, idx).cpu().numpy()
    q = case.q[torch.tensor(seq_ids, device=case.q.device)].cpu().numpy()
    return q, k_pool, v_pool, table, lens


def host_full(case: Case):
    """Host copies of the whole case (small cases only): q, pools, table, lens."""
    return (case.q.cpu().numpy(), case.k_cache.cpu().numpy(), case.v_cache.cpu().numpy(),
            case.block_table_host.copy(), case.lens.copy())


# --- several query tokens per sequence, and shared prefixes ---------------------

@dataclasses.dataclass
class MqCase:
    """A multi-query batch: the last n_q tokens of each sequence are queries."""
    name: str
    q: torch.Tensor              # [T, Hq, D] fp16
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor    # [S, width] int32
    context_lens: torch.Tensor   # [S] int32, the query tokens included
    query_start: torch.Tensor    # [S + 1] int32
    scale: float
    lens: np.ndarray
    n_queries: np.ndarray
    block_table_host: np.ndarray
    causal: bool
    seed: int
    kv_dtype: str = "fp16"       # "fp16", or "fp8": E4M3 codes (uint8) with per-tensor scales
    k_scale: float = 1.0
    v_scale: float = 1.0

    def attn_kwargs(self):
        """The scale arguments the attention calls need for this cache."""
        return {"k_scale": self.k_scale, "v_scale": self.v_scale} if self.kv_dtype == "fp8" else {}

    @property
    def S(self):
        return self.context_lens.shape[0]

    @property
    def T(self):
        return self.q.shape[0]

    @property
    def Hq(self):
        return self.q.shape[1]

    @property
    def Hkv(self):
        return self.k_cache.shape[2]


def _queries(T, Hq, D, seed, device):
    """N(0, 1) fp16 query rows, drawn after the pool (seed + 1, torch on the device)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) + 1)
    return torch.randn((T, Hq, D), generator=gen, device=device,
                       dtype=torch.float32).to(torch.float16)


def build_mq_case(lens, n_queries, Hq, Hkv, *, causal=True, seed=0, device="cpu",
                  rng_backend="numpy", name="mq_custom", pool_blocks=None,
                  kv_dtype="fp16") -> MqCase:
    """Pool and tables as build_case draws them, then sum(n_queries) query rows."""
    base = build_case(lens, Hq, Hkv, seed=seed, device=device, rng_backend=rng_backend,
                      name=name, pool_blocks=pool_blocks, kv_dtype=kv_dtype)
    n_queries = np.asarray(n_queries, dtype=np.int64)
    qs = np.concatenate([[0], np.cumsum(n_queries)]).astype(np.int32)
    q = _queries(int(qs[-1]), Hq, base.D, seed, device)
    return MqCase(name=name, q=q, k_cache=base.k_cache, v_cache=base.v_cache,
                  block_table=base.block_table, context_lens=base.context_lens,
                  query_start=torch.from_numpy(qs).to(device), scale=base.scale,
                  lens=base.lens, n_queries=n_queries, block_table_host=base.block_table_host,
                  causal=causal, seed=seed, kv_dtype=kv_dtype, k_scale=base.k_scale,
                  v_scale=base.v_scale)


def spec_verify(seed=0, device="cpu", rng_backend="torch", kv_dtype="fp16"):
    """Speculative verification: 32 sequences of 4096 tokens, 6 query tokens each.

    The 5 proposed tokens of a draft model (5 to 6 in the speculative-decoding
    knob of "Optimising decode in vLLM") plus the last accepted token are
    checked causally in one pass; batches above ~32 requests gain little there.
    """
    return build_mq_case([4096] * 32, [6] * 32, 32, 8, causal=True, seed=seed, device=device,
                         rng_backend=rng_backend, kv_dtype=kv_dtype,
                         name="spec_verify_b32_ctx4096_q6" + _suffix(kv_dtype))


def chunked_prefill(seed=0, device="cpu", rng_backend="torch", kv_dtype="fp16"):
    """Chunked prefill: 4 prompts, each at a 1024-token chunk (chunks 1, 3, 7, 15).

    The chunk attends to the earlier chunks unmasked and to itself causally
    ("Mathematical Formulation of Chunked Attention"; 1024-token chunks in
    the chunk schedule figure of the same section).
    """
    chunks = [1, 3, 7, 15]
    lens = [(c + 1) * K1 for c in chunks]
    return build_mq_case(lens, [K1] * 4, 32, 8, causal=True, seed=seed, device=device,
                         rng_backend=rng_backend, kv_dtype=kv_dtype,
                         name="prefill_s4_chunk1024_at_1_3_7_15" + _suffix(kv_dtype))


@dataclasses.dataclass
class CascadeCase:
    """Decode requests in groups that share a prefix (cascade attention)."""
    name: str
    q: torch.Tensor              # [B, Hq, D]
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    prefix_table: torch.Tensor   # [R, width]
    prefix_lens: torch.Tensor    # [R]
    group_start: torch.Tensor    # [R + 1]
    suffix_table: torch.Tensor   # [B, width]
    suffix_lens: torch.Tensor    # [B]
    scale: float
    prefix_lens_host: np.ndarray
    group_start_host: np.ndarray
    suffix_lens_host: np.ndarray
    prefix_table_host: np.ndarray
    suffix_table_host: np.ndarray
    seed: int
    kv_dtype: str = "fp16"
    k_scale: float = 1.0
    v_scale: float = 1.0

    def attn_kwargs(self):
        """The scale arguments the attention calls need for this cache."""
        return {"k_scale": self.k_scale, "v_scale": self.v_scale} if self.kv_dtype == "fp8" else {}

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def Hq(self):
        return self.q.shape[1]

    @property
    def Hkv(self):
        return self.k_cache.shape[2]

    def naive_table(self):
        """Per request: prefix frames then suffix frames (prefixes of whole blocks only)."""
        pl = self.prefix_lens_host
        if np.any(pl % BLOCK_SIZE):
            raise ValueError("a prefix that ends inside a block has no single-table form")
        rows, lens = [], []
        for r in range(len(pl)):
            for b in range(int(self.group_start_host[r]), int(self.group_start_host[r + 1])):
                nb = -(-int(self.suffix_lens_host[b]) // BLOCK_SIZE)
                rows.append(list(self.prefix_table_host[r, :pl[r] // BLOCK_SIZE]) +
                            list(self.suffix_table_host[b, :nb]))
                lens.append(int(pl[r]) + int(self.suffix_lens_host[b]))
        width = max(max(len(x) for x in rows), 1)
        table = np.full((len(rows), width), -1, dtype=np.int64)
        for i, x in enumerate(rows):
            table[i, :len(x)] = x
        dev = self.q.device
        return (torch.from_numpy(table.astype(np.int32)).to(dev),
                torch.from_numpy(np.asarray(lens, dtype=np.int32)).to(dev))


def build_cascade_case(prefix_lens, group_sizes, suffix_lens, Hq, Hkv, *, seed=0, device="cpu",
                       rng_backend="numpy", name="cascade_custom",
                       kv_dtype="fp16") -> CascadeCase:
    """One pool dealt to R prefix rows then B suffix rows, then B query rows."""
    prefix_lens = np.asarray(prefix_lens, dtype=np.int64)
    suffix_lens = np.asarray(suffix_lens, dtype=np.int64)
    R = len(prefix_lens)
    base = build_case(np.concatenate([prefix_lens, suffix_lens]), Hq, Hkv, seed=seed,
                      device=device, rng_backend=rng_backend, name=name, kv_dtype=kv_dtype)
    gs = np.concatenate([[0], np.cumsum(group_sizes)]).astype(np.int64)
    B = int(gs[-1])
    assert B == len(suffix_lens)
    q = _queries(B, Hq, base.D, seed, device)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a).astype(np.int32)).to(device)
    return CascadeCase(name=name, q=q, k_cache=base.k_cache, v_cache=base.v_cache,
                       prefix_table=i32(base.block_table_host[:R]), prefix_lens=i32(prefix_lens),
                       group_start=i32(gs), suffix_table=i32(base.block_table_host[R:]),
                       suffix_lens=i32(suffix_lens), scale=base.scale,
                       prefix_lens_host=prefix_lens, group_start_host=gs,
                       suffix_lens_host=suffix_lens,
                       prefix_table_host=base.block_table_host[:R].copy(),
                       suffix_table_host=base.block_table_host[R:].copy(), seed=seed,
                       kv_dtype=kv_dtype, k_scale=base.k_scale, v_scale=base.v_scale)


def shared_prefix(seed=0, device="cpu", rng_backend="torch", kv_dtype="fp16"):
    """Cascade decode: 4 groups of 50 requests, each group sharing a 16K-token prefix.

    50 requests per shared prefix as in the worked example of "What
    FlashInfer brings: JIT and cascade attention"; the prefix is 16K tokens
    (a long shared system prompt or document) and each request's own suffix
    is uniform on [1, 1024] tokens.  32/8 heads.
    """
    rng = np.random.Generator(np.random.PCG64(seed + 7))
    suffix = rng.integers(1, K1, size=200, endpoint=True)
    return build_cascade_case([16 * K1] * 4, [50] * 4, suffix, 32, 8, seed=seed, device=device,
                              rng_backend=rng_backend, kv_dtype=kv_dtype,
                              name="cascade_g4x50_prefix16k_suffix1k" + _suffix(kv_dtype))


def _agentic_heads(Hq, Hkv):
    def make(seed=0, device="cpu", rng_backend="torch", kv_dtype="fp16"):
        return agentic_80k(seed, device, rng_backend, kv_dtype, heads=(Hq, Hkv))
    make.__doc__ = f"The agentic batch at Q{Hq}:KV{Hkv} heads."
    return make


CONFIGS = {
    "tiny": tiny,
    "llama8b_4k": llama8b_4k,
    "agentic_80k": agentic_80k,
    "agentic_80k_q48kv8": _agentic_heads(48, 8),
    "agentic_80k_q64kv8": _agentic_heads(64, 8),
    "agentic_80k_q32kv32": _agentic_heads(32, 32),
    "agentic_80k_q40kv40": _agentic_heads(40, 40),
    "agentic_80k_q48kv48": _agentic_heads(48, 48),
    "ragged_mixed": ragged_mixed,
    "disagg_merge": disagg_merge,
}

MQ_CONFIGS = {
    "spec_verify": spec_verify,
    "chunked_prefill": chunked_prefill,
}

CASCADE_CONFIGS = {
    "shared_prefix": shared_prefix,
}
