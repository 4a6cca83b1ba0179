// Multi-query attention over a paged KV cache for MI355X (gfx950): the last
// n_q tokens of a sequence attend to its cached K/V in one pass, with or
// without a causal mask.
//
// The math: a prefill chunk's queries see the earlier chunks unmasked and the
// current chunk causally ("Mathematical Formulation of Chunked Attention" on
// the page "Disaggregated Inference Architecture: Paged KV-Cache Tiering,
// Chunked Prefill, and Asynchronous Overlap"); the tokens a draft model
// proposed are checked by the verifier in one forward pass (knob 3,
// speculative decoding, of the post "Optimising decode in vLLM: squeezing
// every token out of small hardware"); the shared prefix of cascade attention
// is attended once for all requests that share it, unmasked ("What
// FlashInfer brings: JIT and cascade attention" on the page "The
// signature-dish specialist: vLLM's attention backend").  Query i of the
// last n_q tokens of a sequence of n tokens sits at position n - n_q + i; with
// the causal mask it sees tokens 0 .. n - n_q + i, without it all n.
//
// Work decomposition.  The queries of a sequence are cut into tiles of Qt
// query tokens whose Qt x G (query, head) rows fill MFMA row blocks of 16: row
// m is query m / G, head m % G.  Every tile reads its sequence's K/V up to the
// furthest position one of its queries sees, in units of P tokens.  A one-wave
// plan kernel lists the tiles, their units and the prefix sums of the units;
// the units of all tiles, in order, form one stream cut into n_runs equal runs
// (as for single-token decode).  A tile that lies inside one run writes its
// output directly; a tile cut by run boundaries writes normalised partials
// (slot w + its rank among the cut tiles, so at most 2 * n_runs slots) that
// the merge kernel combines by log-sum-exp, one wave per row.  Tiles that see
// no token are written as 0 with lse -inf by the merge kernel.
//
// Three tile kernels, picked by the average query rows per sequence:
//   * register kernel (up to 32 rows): one work-group per (run, group of up to
//     4 KV heads), two waves per KV head (each half of the run, combined in LDS
//     at the end), a tile of one or two 16-row blocks per wave; each wave
//     streams its own K/V through a ring of register buffers, as the decode
//     kernel does;
//   * shared kernel (up to 64 rows): one work-group of 4 waves per (run, KV
//     head) and a 64-row tile, 16 rows per wave; the 256 threads load each
//     16-token block of K and V once (16 bytes of each per thread, a few blocks
//     ahead in registers) into a double-buffered LDS stage, and every wave
//     folds its rows from there, so the tile's K/V is read once for all its
//     rows;
//   * wide kernel (more rows): the shared kernel's staging with 128-row tiles,
//     32 rows per wave on 32x32 MFMAs and 32 tokens per step (64 for FP8).
// The running max and sum of the softmax are per row, each row has its own
// last visible token, and steps every row sees in full skip the mask.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cfloat>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "paged_attn.h"
#include "pda_common.h"

namespace {

using namespace pda;

constexpr int kMqWaves = 4;           // waves per work-group (KV heads, or row groups)
constexpr int kMqMaxKvHeads = 64;
constexpr int kMqMaxSeqs = 4000;      // sequences per call: their facts live in the plan's LDS
constexpr int kMqHdrInts = 8;         // k, U, n_runs, P, n_tiles, n_fix
constexpr int kMqTileArrays = 8;      // seq, q0, nq, base, ntok, ub, rank, fix
constexpr int kMqMaxPartition = 1 << 20;
constexpr int kRegRing = 2;           // register kernel: K/V buffers per wave (blocks in flight + 1)
constexpr int kShPrefetch = 4;        // shared kernel: blocks each thread holds (in flight + 1)
// shared kernel: bytes per token row of one KV head in LDS (the row, 256 bytes
// fp16 or 128 FP8, plus 16 bytes of padding: conflict-free operand reads)
template <bool kFp8>
constexpr int lds_row() { return 128 * KvFmt<kFp8>::kElemBytes + 16; }
constexpr int kNoMask = -(1 << 30);   // causal base of a tile without the causal mask
constexpr float kLazyMax = 8.0f;      // log2 headroom of p over a row's reference max

#ifndef PDA_MQ_NT_REG
#define PDA_MQ_NT_REG 1
#endif
#ifndef PDA_WIDE_REVERSE
#define PDA_WIDE_REVERSE 1
#endif
#ifndef PDA_MQ_NT_STAGE
#define PDA_MQ_NT_STAGE 0
#endif
// K/V loads: non-temporal where a tile streams its own V (register kernel),
// or ordinary where tiles of one sequence read the same K/V again.  K loads
// are ordinary everywhere: each reads half of a token row's lines and the next
// the other half, which a non-temporal first half would let go (8-10% slower
// over FP8).
template <bool kNt, typename T>
__device__ __forceinline__ T kv_load(const char* p) {
  if constexpr (kNt) return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
  else return *reinterpret_cast<const T*>(p);
}

struct MqParams {
  const _Float16* q;        // [T, Hq, D]
  const int32_t* qs;        // [S + 1]: queries of sequence s are rows qs[s] .. qs[s+1]-1
  const void* k;            // [num_blocks, 16, Hkv, D] fp16, or FP8 E4M3 codes
  const void* v;
  const int32_t* bt;        // [S, bt_stride]
  const int32_t* ctx;       // [S] cached tokens, the queries' own included
  long long bt_stride;
  long long num_blocks;     // block ids are clamped into [0, num_blocks)
  int S, T, Hq, Hkv;
  int max_tokens;           // max_blocks_per_seq * 16; longer contexts are clamped
  int P;                    // unit length in tokens
  int n_runs;
  int hg;                   // KV heads per work-group; Hkv / hg head groups
  int causal;
  float qk_scale;           // |scale * k_scale| * log2(e)
  unsigned q_sign;          // 0x80008000 to negate q (scale < 0), else 0
  int32_t* hdr;             // [kMqHdrInts]
  // per tile (tiles_max entries each)
  int32_t* t_seq;           // sequence
  int32_t* t_q0;            // first query row of the tile
  int32_t* t_nq;            // queries in the tile (1 .. Qt)
  int32_t* t_base;          // causal: query qi of the tile sees base + qi tokens (clamped)
  int32_t* t_ntok;          // tokens the tile reads: what its furthest query sees
  int32_t* t_ub;            // units of all earlier tiles
  int32_t* t_rank;          // rank among the tiles cut by run boundaries, else -1
  int32_t* t_fix;           // [n_fix] tiles the merge kernel writes: cut ones and empty ones
  float* ws_o;              // [2 * n_runs, Qt, Hq, D] normalised partials
  float* ws_lse;            // [2 * n_runs, Qt, Hq]
  void* out;                // [T, Hq, D] fp16, or fp32 for the partial entry point
  float* lse_out;           // [T, Hq] or null
  int out_f16;
  // last: inserted before the pointers above, it changed the generated code of
  // the fp16 kernels (up to 30 more VGPRs and spills at 2 row blocks per wave)
  float v_scale;            // multiplies the output (FP8 V scale; 1 for fp16)
  // the merge's view of fix tile f (16-byte aligned): first query row, queries,
  // first partial slot, partials (0 for a tile that sees no token)
  int32_t* t_rec;           // [tiles_max][4]
  int tiles_max;
};

__device__ __forceinline__ int mq_seq_len(const MqParams& p, int s) {
  return min(max(p.ctx[s], 0), p.max_tokens);
}
// query rows of sequence s, clamped into [0, T] so that a malformed
// query_start cannot send a load or store outside q, out or lse_out
__device__ __forceinline__ int mq_q_begin(const MqParams& p, int s) {
  return min(max(p.qs[s], 0), p.T);
}
__device__ __forceinline__ int mq_q_end(const MqParams& p, int s) {
  return min(max(p.qs[s + 1], mq_q_begin(p, s)), p.T);
}

// ---------------------------------------------------------------------------
// plan: the tiles, their units and the run schedule (one wave)

template <int Qt>
__global__ __launch_bounds__(kWave) void mq_plan_kernel(MqParams p) {
  // per sequence: first tile, first query row, query count, cached tokens
  __shared__ int toff[kMqMaxSeqs + 1];
  __shared__ int sqb[kMqMaxSeqs];
  __shared__ int snq[kMqMaxSeqs];
  __shared__ int sn[kMqMaxSeqs];
  const int lane = threadIdx.x;

  int carry = 0;
  for (int s0 = 0; s0 < p.S; s0 += kWave) {
    const int s = s0 + lane;
    int nt = 0;
    if (s < p.S) {
      const int qb = mq_q_begin(p, s);
      const int nq = mq_q_end(p, s) - qb;
      sqb[s] = qb;
      snq[s] = nq;
      sn[s] = mq_seq_len(p, s);
      nt = (nq + Qt - 1) / Qt;
    }
    const int incl = carry + wave_inclusive_scan_i32(nt, lane);
    if (s < p.S) toff[s] = incl - nt;
    carry = __builtin_amdgcn_readlane(incl, kWave - 1);
  }
  const int n_tiles = carry;
  __syncthreads();

  // facts of tile i: the sequence holding it is the last one whose first tile
  // is <= i (sequences without queries own no tile)
  auto facts = [&](int i, int& s, int& q0, int& nq, int& base, int& ntok) {
    int lo = 0, hi = p.S - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (toff[mid] <= i) lo = mid; else hi = mid - 1;
    }
    s = lo;
    const int j = i - toff[s];
    const int nq_seq = snq[s];
    q0 = sqb[s] + j * Qt;
    nq = min(Qt, nq_seq - j * Qt);
    const int n = sn[s];
    if (p.causal) {
      base = n - nq_seq + j * Qt + 1;
      ntok = min(max(base + nq - 1, 0), n);
    } else {
      base = n;
      ntok = n;
    }
  };

  int U = 0;
  for (int i0 = 0; i0 < n_tiles; i0 += kWave) {
    const int i = i0 + lane;
    int nu = 0;
    if (i < n_tiles) {
      int s, q0, nq, base, ntok;
      facts(i, s, q0, nq, base, ntok);
      nu = (ntok + p.P - 1) / p.P;
    }
    U += wave_sum_i32(nu);
  }
  const int k = U > 0 ? (U + p.n_runs - 1) / p.n_runs : 1;

  int ucarry = 0, rcarry = 0, fcarry = 0;
  for (int i0 = 0; i0 < n_tiles; i0 += kWave) {
    const int i = i0 + lane;
    int s = 0, q0 = 0, nq = 0, base = 0, ntok = 0, nu = 0;
    if (i < n_tiles) {
      facts(i, s, q0, nq, base, ntok);
      nu = (ntok + p.P - 1) / p.P;
    }
    const int incl = ucarry + wave_inclusive_scan_i32(nu, lane);
    const int ub = incl - nu;
    const int cut = (nu > 0 && ub / k != (ub + nu - 1) / k) ? 1 : 0;
    const int fix = (i < n_tiles && (cut || nu == 0)) ? 1 : 0;
    const int rincl = rcarry + wave_inclusive_scan_i32(cut, lane);
    const int fincl = fcarry + wave_inclusive_scan_i32(fix, lane);
    if (i < n_tiles) {
      p.t_seq[i] = s;
      p.t_q0[i] = q0;
      p.t_nq[i] = nq;
      p.t_base[i] = base;
      p.t_ntok[i] = ntok;
      p.t_ub[i] = ub;
      p.t_rank[i] = cut ? rincl - 1 : -1;
      if (fix) {
        p.t_fix[fincl - 1] = i;
        const int nseg = nu > 0 ? (ub + nu - 1) / k - ub / k + 1 : 0;
        const int slot0 = nu > 0 ? ub / k + rincl - 1 : 0;    // a listed tile with nu > 0 is cut
        *reinterpret_cast<int4*>(p.t_rec + 4 * (fincl - 1)) = int4{q0, nq, slot0, nseg};
      }
    }
    ucarry = __builtin_amdgcn_readlane(incl, kWave - 1);
    rcarry = __builtin_amdgcn_readlane(rincl, kWave - 1);
    fcarry = __builtin_amdgcn_readlane(fincl, kWave - 1);
  }
  if (lane == 0) {
    p.hdr[0] = k;
    p.hdr[1] = U;
    p.hdr[2] = p.n_runs;
    p.hdr[3] = p.P;
    p.hdr[4] = n_tiles;
    p.hdr[5] = fcarry;
  }
}

// The tile holding unit u: the last tile whose first unit is <= u.
__device__ __forceinline__ int tile_of_unit(const MqParams& p, int u, int n_tiles) {
  int lo = 0, hi = n_tiles - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.t_ub[mid] <= u) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The segments of run w: (tile i, tokens [tok_lo, tok_hi), whole tile?,
// partial slot), in tile order, or last tile first when kReverse.  Uniform over
// the work-group.  Last tile first, a run that covers about one tile starts at
// token 0 of its later tile and reaches the end of the earlier one about when
// the other runs of the sequence reach theirs, so the runs resident together
// read the same K/V blocks at about the same time.
template <bool kReverse, typename F>
__device__ __forceinline__ void for_each_segment_in(const MqParams& p, int w, int u_lo, int u_hi,
                                                    F&& fn) {
  const int U = p.hdr[1], n_tiles = p.hdr[4];
  if (u_lo >= u_hi || n_tiles <= 0) return;
  auto segment = [&](int i) {
    const int before = p.t_ub[i];
    const int nu = (i + 1 < n_tiles ? p.t_ub[i + 1] : U) - before;
    const int p_lo = max(u_lo - before, 0);
    const int p_hi = min(u_hi - before, nu);
    if (p_hi > p_lo)
      fn(i, p_lo * p.P, min(p_hi * p.P, p.t_ntok[i]), p_lo == 0 && p_hi == nu, w + p.t_rank[i]);
  };
  const int first = tile_of_unit(p, u_lo, n_tiles);
  if constexpr (kReverse) {
    const int last = tile_of_unit(p, u_hi - 1, n_tiles);
    for (int i = last; i >= first; --i) segment(i);
  } else {
    for (int i = first; i < n_tiles && p.t_ub[i] < u_hi; ++i) segment(i);
  }
}
template <bool kReverse = false, typename F>
__device__ __forceinline__ void for_each_segment(const MqParams& p, int w, F&& fn) {
  const int k = p.hdr[0], U = p.hdr[1];
  const int u_lo = w * k;
  for_each_segment_in<kReverse>(p, w, u_lo, min(u_lo + k, U), fn);
}

// ---------------------------------------------------------------------------
// per-wave fold of 16-token blocks

// Softmax state of NT row blocks of 16 rows.  The scores are computed
// transposed, S^T = K Q^T, so lane (c, n) (c = lane >> 4, n = lane & 15) holds
// row row0 + 16b + n at tokens 4c .. 4c+3 of a block: the running max and sum
// are one value per lane for its row (the sum over the lane's own tokens).  The
// p.V output holds rows row0 + 16b + 4c + r at lane (c, n), register r.
template <int NT>
struct MqSeg {
  float m[NT];              // running max of row n (base 2)
  float lp[NT];             // running sum of p over this lane's tokens of row n
  f32x4 acc[NT][8];         // p.V tiles: lane (c, n), tile u, reg r = row 4c + r, dim 8n + u
};

template <int NT>
__device__ __forceinline__ void mq_seg_init(MqSeg<NT>& st) {
#pragma unroll
  for (int b = 0; b < NT; ++b) {
    st.m[b] = -INFINITY;
    st.lp[b] = 0.0f;
#pragma unroll
    for (int u = 0; u < 8; ++u) st.acc[b][u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
}

// B operands of the 8 p.V MFMA tiles (v_mfma_f32_16x16x16_f16) from one
// block's V rows, shared by the NT row blocks: tile u covers dims 8n + u, and
// the contraction index 4c + i is token 4c + i, so lane (c, n) takes element u
// of its own V rows 4c .. 4c+3 (loaded as dims 8n .. 8n+7; FP8 codes are
// transposed 4x4 by bytes and decoded exactly to fp16).  Tokens at or past
// nvalid are exact zero rows (selected, so a NaN in an unowned slot cannot
// leak through 0 * NaN).
template <bool kMasked, bool kFp8>
__device__ __forceinline__ void mq_v_operands(const typename KvFmt<kFp8>::VRow (&vr)[4], int c,
                                              int nvalid, half4_t (&vb)[8]) {
  if constexpr (kFp8) {
    u32x2 vv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      vv[i] = (!kMasked || 4 * c + i < nvalid) ? vr[i] : u32x2{0u, 0u};   // code 0 = +0
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      // dims 8n + 4w + e of tokens 4c .. 4c+3: byte e of each token's word w
      const unsigned ab_lo = __builtin_amdgcn_perm(vv[1][w], vv[0][w], 0x05010400u);
      const unsigned ab_hi = __builtin_amdgcn_perm(vv[1][w], vv[0][w], 0x07030602u);
      const unsigned cd_lo = __builtin_amdgcn_perm(vv[3][w], vv[2][w], 0x05010400u);
      const unsigned cd_hi = __builtin_amdgcn_perm(vv[3][w], vv[2][w], 0x07030602u);
      const unsigned tcol[4] = {__builtin_amdgcn_perm(cd_lo, ab_lo, 0x05040100u),
                                __builtin_amdgcn_perm(cd_lo, ab_lo, 0x07060302u),
                                __builtin_amdgcn_perm(cd_hi, ab_hi, 0x05040100u),
                                __builtin_amdgcn_perm(cd_hi, ab_hi, 0x07060302u)};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const half2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(tcol[e], 1.0f, false);
        const half2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(tcol[e], 1.0f, true);
        vb[4 * w + e] = half4_t{lo[0], lo[1], hi[0], hi[1]};
      }
    }
  } else {
    u32x4 vv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      vv[i] = (!kMasked || 4 * c + i < nvalid) ? vr[i] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int w = u / 2;
      const unsigned sel = (u & 1) ? 0x07060302u : 0x05040100u;   // high or low halves
      const unsigned d01 = __builtin_amdgcn_perm(vv[1][w], vv[0][w], sel);
      const unsigned d23 = __builtin_amdgcn_perm(vv[3][w], vv[2][w], sel);
      vb[u] = __builtin_bit_cast(half4_t, u32x2{d01, d23});
    }
  }
}

// One 16-token block starting at token t0, one row block at a time.
//   kr: K token n, 16 bytes at 16c + 64i; vr: V tokens 4c + i, dims 8n .. 8n+7.
//   S^T = K Q^T: the K operands are the A side and the query rows the B side
//   of four v_mfma_f32_16x16x32_f16, so lane (c, n) gets row n at tokens
//   4c + r, which is also the lane's A operand of p.V (row n, contraction
//   indices 4c .. 4c+3): p goes from the score registers to the p.V MFMAs
//   without a transpose.
// In a masked block, row row0 + 16b + n (query qi of the tile) sees tokens
// before min(base + qi, n_seq, tok_hi) when causal, before tok_hi otherwise;
// rows past the tile's queries see everything and are never stored.  Tokens at
// or past t0 + nvalid are exact zeros.
// Where a fold finds the Q operands of row block b, chunk i: registers, or an
// LDS copy [b][i][lane] shared by the waves of a work-group (read at every
// block, so that only one row block's operands are live at a time).
template <int NT>
struct MqQRegs {
  const half8_t (&qa)[NT][4];
  __device__ __forceinline__ half8_t get(int b, int i) const { return qa[b][i]; }
};
typedef __attribute__((address_space(3))) u32x4 LdsU32x4;
struct MqQLds {
  const LdsU32x4* base;
  int lane;
  __device__ __forceinline__ half8_t get(int b, int i) const {
    return __builtin_bit_cast(half8_t, base[(b * 4 + i) * kWave + lane]);
  }
};

template <int G, int NT, bool kMasked, bool kFp8, typename QSrc>
__device__ __forceinline__ void mq_fold(MqSeg<NT>& st, const QSrc& qa,
                                        const u32x4 (&kr)[KvFmt<kFp8>::kKLoads],
                                        const typename KvFmt<kFp8>::VRow (&vr)[4],
                                        float qk_scale, int lane, int row0, int t0, int nvalid,
                                        int causal_base, int n_seq, int nq, int tok_hi) {
  const int n = lane & 15;
  const int c = lane >> 4;
  half8_t kop[4];
  k_operands<kFp8>(kr, kop);
  half4_t vb[8];
  mq_v_operands<kMasked, kFp8>(vr, c, nvalid, vb);
#pragma unroll
  for (int b = 0; b < NT; ++b) {
    f32x4 sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[i], qa.get(b, i), sc, 0, 0, 0);
    float sv[4];
    if (kMasked) {
      const int qi = (row0 + 16 * b + n) / G;
      int e = tok_hi;
      if (qi < nq && causal_base != kNoMask) e = min(min(max(causal_base + qi, 0), n_seq), tok_hi);
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[r] = t0 + 4 * c + r < e ? sc[r] : -INFINITY;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[r] = sc[r];
    }
    // The reference m of a row only has to be the same for all its tokens:
    // it moves when a score exceeds it by more than kLazyMax (so p <= 2^kLazyMax
    // in between), and then to the exact running max.  The check takes the
    // lane's own 4 tokens; the max over the 4 lane groups only when it fires.
    const float xl = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    if (__ballot(xl * qk_scale > st.m[b] + kLazyMax) != 0) {   // uniform branch
      float x = fmaxf(xl, __shfl_xor(xl, 16, kWave));
      x = fmaxf(x, __shfl_xor(x, 32, kWave));
      float mb = x * qk_scale;
      if (kMasked) mb = x == -INFINITY ? -INFINITY : mb;   // a fully masked row stays -inf
      const float mn = fmaxf(st.m[b], mb);
      const float a = mn == st.m[b] ? 1.0f : fast_exp2(st.m[b] - mn);   // 0 on a first token
      st.m[b] = mn;
      st.lp[b] *= a;
      // the p.V output rows of this lane are 4c + r: their factors live in
      // lanes 4c + r of lane group 0
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(a, 4 * c + r, kWave);
#pragma unroll
        for (int u = 0; u < 8; ++u) st.acc[b][u][r] *= ar;
      }
    }
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[r] = fast_exp2(fmaf(sv[r], qk_scale, -st.m[b]));
      if (kMasked) pr[r] = sv[r] == -INFINITY ? 0.0f : pr[r];   // -inf - (-inf) would be NaN
    }
    st.lp[b] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
    const half4_t pa = {static_cast<_Float16>(pr[0]), static_cast<_Float16>(pr[1]),
                        static_cast<_Float16>(pr[2]), static_cast<_Float16>(pr[3])};
#pragma unroll
    for (int u = 0; u < 8; ++u)
      st.acc[b][u] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, vb[u], st.acc[b][u], 0, 0, 0);
  }
}

// Q as the MFMA A operands of rows row0 .. row0 + 16 NT - 1 of a tile: row m
// is query m / G, head g*G + m % G; rows past the tile's queries load its last
// query and are zeroed.
template <int G, int NT, bool kFp8>
__device__ __forceinline__ void mq_load_q(const MqParams& p, int g, int q0, int nq, int row0,
                                          int lane, half8_t (&qa)[NT][4]) {
  const int c = lane >> 4, t = lane & 15;
#pragma unroll
  for (int b = 0; b < NT; ++b) {
    const int m = row0 + 16 * b + t;
    const int qi = m / G, j = m % G;
    const int row = q0 + min(qi, nq - 1);
    const _Float16* qrow = p.q + ((long long)row * p.Hq + (long long)g * G + j) * kD;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      u32x4 x = *reinterpret_cast<const u32x4*>(qrow + KvFmt<kFp8>::q_dim(ii, c)) ^ p.q_sign;
      if (qi >= nq) x = u32x4{0u, 0u, 0u, 0u};
      qa[b][ii] = __builtin_bit_cast(half8_t, x);
    }
  }
}

// Normalise and store rows row0 .. of the wave: lane (c, n) holds rows
// row0 + 16b + 4c + r, dims 8n .. 8n+7.  A whole tile writes the output; a
// segment of a cut tile writes its partial to slot `slot`.
template <int G, int NT, int Qt, bool kFp8>
__device__ __forceinline__ void mq_store(const MqParams& p, MqSeg<NT>& st, int g, int q0, int nq,
                                         int row0, int lane, bool whole, int slot) {
  const int c = lane >> 4, t = lane & 15;
#pragma unroll
  for (int b = 0; b < NT; ++b) {
    // sum of row n over the 4 lane groups; then the values of the output rows
    // 4c + r from lanes 4c + r
    float lrow = st.lp[b];
    lrow += __shfl_xor(lrow, 16, kWave);
    lrow += __shfl_xor(lrow, 32, kWave);
    float lr[4], mr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      lr[r] = __shfl(lrow, 4 * c + r, kWave);
      mr[r] = __shfl(st.m[b], 4 * c + r, kWave);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float l = lr[r];
      const int row = row0 + 16 * b + 4 * c + r;
      const int qi = row / G, j = row % G;
      if (qi >= nq) continue;
      float inv = l > 0.0f ? 1.0f / l : 0.0f;
      if constexpr (kFp8) inv *= p.v_scale;
      const float lse = l > 0.0f ? (mr[r] + __builtin_log2f(l)) * kLn2 : -INFINITY;
      float o[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) o[u] = st.acc[b][u][r] * inv;
      const int h = g * G + j;
      if (whole) {
        const long long dst = ((long long)(q0 + qi) * p.Hq + h) * kD + 8 * t;
        if (p.out_f16) {
          half8_t hv;
#pragma unroll
          for (int e = 0; e < 8; ++e) hv[e] = static_cast<_Float16>(o[e]);
          *reinterpret_cast<half8_t*>(static_cast<_Float16*>(p.out) + dst) = hv;
        } else {
          float* d = static_cast<float*>(p.out) + dst;
          *reinterpret_cast<f32x4*>(d) = f32x4{o[0], o[1], o[2], o[3]};
          *reinterpret_cast<f32x4*>(d + 4) = f32x4{o[4], o[5], o[6], o[7]};
        }
        if (p.lse_out && t == 0) p.lse_out[(long long)(q0 + qi) * p.Hq + h] = lse;
      } else {
        const long long sl = ((long long)slot * Qt + qi) * p.Hq + h;
        float* d = p.ws_o + sl * kD + 8 * t;
        *reinterpret_cast<f32x4*>(d) = f32x4{o[0], o[1], o[2], o[3]};
        *reinterpret_cast<f32x4*>(d + 4) = f32x4{o[4], o[5], o[6], o[7]};
        if (t == 0) p.ws_lse[sl] = lse;
      }
    }
  }
}

// The block-table window of a segment: lane i holds the id of block (window
// base + i); ids outside the pool are clamped (a broken table gives wrong
// numbers, not a fault).
struct BlockWindow {
  const int32_t* row;
  int nblk, lane, ids;
  long long num_blocks, block_bytes;
  __device__ BlockWindow(const int32_t* r, int nb, int ln, long long nblocks, long long bbytes)
      : row(r), nblk(nb), lane(ln), num_blocks(nblocks), block_bytes(bbytes) {
    ids = lane < nblk ? row[lane] : 0;
  }
  __device__ __forceinline__ long long offset(int kb) {
    if ((kb & 63) == 0 && kb > 0) {
      const int idx = kb + lane;
      ids = idx < nblk ? row[idx] : 0;
    }
    const unsigned raw = (unsigned)__builtin_amdgcn_readlane(ids, kb & 63);
    const long long blk = raw < (unsigned long long)num_blocks ? (long long)raw : 0;
    return blk * block_bytes;
  }
};

// ---------------------------------------------------------------------------
// register kernel: two waves per KV head (halves of the run), a tile of one
// or two 16-row blocks per wave

// Folds tokens [tok_lo, tok_hi) of sequence s into st for the tile of nq
// queries from row q0 (causal: query qi sees base + qi tokens), KV head g.
// With qlds (the tile's Q operands in LDS, [b][i][lane]) the operands are read
// there at every block instead of held in registers.
template <int G, int NT, bool kFp8, bool kQLds = false>
__device__ __forceinline__ void mq_reg_fold(const MqParams& p, int lane, int g, int s, int q0,
                                            int nq, int base, int tok_lo, int tok_hi,
                                            MqSeg<NT>& st, const LdsU32x4* qlds = nullptr) {
  using Fmt = KvFmt<kFp8>;
  using VRow = typename Fmt::VRow;
  constexpr int E = Fmt::kElemBytes;
  constexpr int KL = Fmt::kKLoads;
  const int c = lane >> 4, t = lane & 15;
  const int n = mq_seq_len(p, s);
  half8_t qa[NT][4];
  if constexpr (!kQLds) mq_load_q<G, NT, kFp8>(p, g, q0, nq, 0, lane, qa);
  unsigned qoff = 0;
  // blocks wholly before the tile's first query's end skip the mask
  const int causal_base = p.causal ? base : kNoMask;
  const int full_end = p.causal ? min(min(max(base, 0), n), tok_hi) : tok_hi;

  const unsigned row_bytes = (unsigned)(p.Hkv * kD * E);
  const unsigned k_lane = (unsigned)((t * p.Hkv + g) * kD * E + 16 * c);
  const unsigned v_lane = (unsigned)((4 * c * p.Hkv + g) * kD * E + 8 * E * t);   // tokens 4c + i
  const char* kbytes = reinterpret_cast<const char*>(p.k);
  const char* vbytes = reinterpret_cast<const char*>(p.v);
  const int nblk = (tok_hi - tok_lo + kBS - 1) / kBS;
  BlockWindow win(p.bt + (long long)s * p.bt_stride + tok_lo / kBS, nblk, lane, p.num_blocks,
                  (long long)kBS * row_bytes);

  mq_seg_init(st);
  auto load = [&](long long off, u32x4 (&kr)[KL], VRow (&vr)[4]) {
#pragma unroll
    for (int ii = 0; ii < KL; ++ii)
      kr[ii] = kv_load<false, u32x4>(kbytes + off + k_lane + 64 * ii);
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
      vr[ii] = kv_load<PDA_MQ_NT_REG != 0, VRow>(vbytes + off + v_lane + ii * row_bytes);
  };
  constexpr int NB = kRegRing;
  u32x4 kbuf[NB][KL];
  VRow vbuf[NB][4];
#pragma unroll
  for (int ii = 0; ii < NB - 1; ++ii)
    if (ii < nblk) load(win.offset(ii), kbuf[ii], vbuf[ii]);
  for (int kb0 = 0; kb0 < nblk; kb0 += NB) {
#pragma unroll
    for (int sl = 0; sl < NB; ++sl) {
      const int cur = kb0 + sl;
      if (cur >= nblk) break;
      const int nxt = cur + NB - 1;
      if (nxt < nblk) load(win.offset(nxt), kbuf[(sl + NB - 1) % NB], vbuf[(sl + NB - 1) % NB]);
      const int t0 = tok_lo + cur * kBS;
      auto fold = [&](const auto& qsrc) {
        if (t0 + kBS > full_end)
          mq_fold<G, NT, true, kFp8>(st, qsrc, kbuf[sl], vbuf[sl], p.qk_scale, lane, 0, t0,
                                     tok_hi - t0, causal_base, n, nq, tok_hi);
        else
          mq_fold<G, NT, false, kFp8>(st, qsrc, kbuf[sl], vbuf[sl], p.qk_scale, lane, 0, t0,
                                      kBS, causal_base, n, nq, tok_hi);
      };
      // opaque: LDS reads of Q stay in the loop, not hoisted into registers
      if constexpr (kQLds) asm volatile("" : "+v"(qoff));
      if constexpr (kQLds) {
        fold(MqQLds{(const LdsU32x4*)((const __attribute__((address_space(3))) char*)qlds + qoff),
                    lane});
      } else {
        fold(MqQRegs<NT>{qa});
      }
    }
  }
}

template <int G, int NT, bool kFp8>
__device__ __forceinline__ void mq_reg_segment(const MqParams& p, int lane, int g, int i, int tok_lo, int tok_hi,
                               bool whole, int slot, MqSeg<NT>& st, bool defer) {
  constexpr int Qt = 16 * NT / G;
  const int q0 = p.t_q0[i], nq = p.t_nq[i];
  mq_reg_fold<G, NT, kFp8>(p, lane, g, p.t_seq[i], q0, nq, p.t_base[i], tok_lo, tok_hi, st);
  if (!defer) mq_store<G, NT, Qt, kFp8>(p, st, g, q0, nq, 0, lane, whole, slot);
}

// One work-group per (run, group of hg KV heads) with two waves per KV head:
// wave (half, head) folds half `half` of the run's units, the first half in
// tile order and the second last tile first, so the tile holding the split
// (if the split falls inside one) is the last each of the two folds.  The
// second writes its state (max, sum, accumulators) to LDS, and after the one
// barrier the first rescales both to the common max, adds them and stores the
// tile's segment of the whole run: a run twice as long at the same occupancy,
// half the partials to write and merge.
template <int G, int NT, bool kFp8>
__global__ __launch_bounds__(2 * kWave * kMqWaves) __attribute__((amdgpu_waves_per_eu(2)))
void mq_reg_kernel(MqParams p) {
  constexpr int kState = NT * (2 + 32);                  // floats per lane
  const int lane = threadIdx.x & (kWave - 1);
  // [hg][kState][kWave]: one state per KV head of the group, sized at launch
  extern __shared__ float xs_dyn[];
  auto xs = [&](int head, int i) -> float& { return xs_dyn[(head * kState + i) * kWave + lane]; };
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int hg = p.hg;
  const int half = wave >= hg ? 1 : 0;
  const int gl = wave - half * hg;
  const int n_hgroups = p.Hkv / hg;
  const int w = blockIdx.x / n_hgroups;                  // run of the unit stream
  const int g = (blockIdx.x % n_hgroups) * hg + gl;      // KV head
  const int k = p.hdr[0], U = p.hdr[1], n_tiles = p.hdr[4];
  const int u_lo = w * k, u_hi = min(u_lo + k, U);
  const int mid = u_lo + max(u_hi - u_lo + 1, 0) / 2;
  int shared_tile = -1;                                  // uniform over the work-group
  if (n_tiles > 0 && u_lo < mid && mid < u_hi) {
    const int i0 = tile_of_unit(p, mid - 1, n_tiles);
    if (i0 == tile_of_unit(p, mid, n_tiles)) shared_tile = i0;
  }
  MqSeg<NT> st;
  auto seg = [&](int i, int tok_lo, int tok_hi, bool whole, int slot) {
    mq_reg_segment<G, NT, kFp8>(p, lane, g, i, tok_lo, tok_hi, whole, slot, st, i == shared_tile);
  };
  if (half == 0) for_each_segment_in<false>(p, w, u_lo, mid, seg);
  else for_each_segment_in<true>(p, w, mid, u_hi, seg);
  if (shared_tile >= 0 && half == 1) {
#pragma unroll
    for (int b = 0; b < NT; ++b) {
      xs(gl, b) = st.m[b];
      xs(gl, NT + b) = st.lp[b];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) xs(gl, 2 * NT + 32 * b + 4 * u + r) = st.acc[b][u][r];
    }
  }
  __syncthreads();
  if (shared_tile >= 0 && half == 0) {
    const int c = lane >> 4;
#pragma unroll
    for (int b = 0; b < NT; ++b) {
      const float mb = xs(gl, b);
      const float m = fmaxf(st.m[b], mb);
      const float aa = st.m[b] == m ? 1.0f : fast_exp2(st.m[b] - m);   // 0 for an empty side
      const float ab = mb == m ? 1.0f : fast_exp2(mb - m);
      st.lp[b] = st.lp[b] * aa + xs(gl, NT + b) * ab;
      st.m[b] = m;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(aa, 4 * c + r, kWave), br = __shfl(ab, 4 * c + r, kWave);
#pragma unroll
        for (int u = 0; u < 8; ++u)
          st.acc[b][u][r] = st.acc[b][u][r] * ar + xs(gl, 2 * NT + 32 * b + 4 * u + r) * br;
      }
    }
    const int i = shared_tile;
    const int before = p.t_ub[i];
    const int nu = (i + 1 < n_tiles ? p.t_ub[i + 1] : U) - before;
    const bool whole = u_lo <= before && u_hi >= before + nu;
    constexpr int Qt = 16 * NT / G;
    mq_store<G, NT, Qt, kFp8>(p, st, g, p.t_q0[i], p.t_nq[i], 0, lane, whole, w + p.t_rank[i]);
  }
}

// ---------------------------------------------------------------------------
// whole-tile register kernel (fp16 cache): one work-group of kTileParts waves
// per (tile, KV head).  Wave j folds part j of the tile's blocks (as the
// register kernel folds a run), the parts' softmax states meet in LDS, and the
// work-group finishes the rows and writes them: no plan, no partials, no
// merge.  The work-group finds its tile itself from query_start.

constexpr int kTileParts = 8;
constexpr int kTileMaxTokens = 8192;  // longest context the host sends this way
constexpr int kTileMaxGroups = 1 << 20;

// dynamic LDS of a whole-tile launch: each part's accumulators (NT x 4
// registers x 64 lanes x 8 floats), then its row max and sum (NT x 2 x 16),
// then the tile's Q operands (NT x 4 chunks x 64 lanes x 16 bytes)
constexpr size_t mq_tile_state_floats(int NT) {
  return (size_t)kTileParts * NT * (4 * kWave * 8 + 2 * 16);
}
constexpr size_t mq_tile_lds(int NT) {
  return mq_tile_state_floats(NT) * sizeof(float) + (size_t)NT * 4 * kWave * 16;
}

// Tile i of the call (sequence s owns tiles toff[s] .. toff[s] + nt_s - 1,
// nt_s = ceil(queries of s / Qt)): its sequence and its rank in it, found by
// one pass of the work-group over query_start.  False when the call has no
// tile i.  sh: 10 ints of LDS.  Every thread calls it.
template <int Qt>
__device__ bool mq_find_tile(const MqParams& p, int i, int* sh, int& s_out, int& j_out) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  constexpr int kThreads = kWave * kTileParts;
  if (tid == 0) sh[kTileParts] = -1;
  int carry = 0;                                   // tiles of the earlier chunks
  for (int s0 = 0; s0 < p.S; s0 += kThreads) {
    const int s = s0 + tid;
    const int nt = s < p.S ? (mq_q_end(p, s) - mq_q_begin(p, s) + Qt - 1) / Qt : 0;
    const int incl = wave_inclusive_scan_i32(nt, lane);
    if (lane == kWave - 1) sh[wave] = incl;        // wave totals
    __syncthreads();
    int before = carry, total = 0;
#pragma unroll
    for (int w = 0; w < kTileParts; ++w) {
      const int x = sh[w];
      before += w < wave ? x : 0;
      total += x;
    }
    const int excl = before + incl - nt;
    if (nt > 0 && excl <= i && i < excl + nt) {
      sh[kTileParts] = s;
      sh[kTileParts + 1] = i - excl;
    }
    carry += total;
    __syncthreads();                               // before the totals are rewritten
  }
  __syncthreads();                                 // (S = 0: the initial -1)
  // the same in every lane: said so, the caller's branch and its token loop
  // stay uniform (scalar) control flow
  s_out = __builtin_amdgcn_readfirstlane(sh[kTileParts]);
  j_out = __builtin_amdgcn_readfirstlane(sh[kTileParts + 1]);
  return s_out >= 0;
}

typedef __attribute__((address_space(3))) float LdsF32;
typedef const __attribute__((address_space(4))) MqParams ConstMqParams;

// Rows 4c + r of row block b (lane (c, n): head dims 8n .. 8n+7) from the
// parts' states in LDS: rescaled to their common max, summed, normalised and
// stored.  Kept out of line, reading the parameters from the kernel-argument
// segment: inlined, or with the fields passed as arguments, the caller kept
// them live through its token loop and went past the register budget of two
// waves per SIMD (spills inside the loop); a reference to the kernel's
// parameter copy put the copy on the stack, and the K/V loads through its
// pointers became flat loads.
template <int G, int NT, bool kFp8>
__device__ __attribute__((noinline)) void mq_tile_finish(ConstMqParams* pp, const LdsF32* lds,
                                                         int b, int r, int lane, int g, int q0,
                                                         int nq) {
  ConstMqParams& p = *pp;
  const int c = lane >> 4, t = lane & 15;
  const int Hq = p.Hq;
  const LdsF32* lacc = lds;
  const LdsF32* lml = lds + kTileParts * NT * 4 * kWave * 8;
  const int row = 4 * c + r;
  float mp[kTileParts];
  float M = -INFINITY;
#pragma unroll
  for (int q = 0; q < kTileParts; ++q) {
    mp[q] = lml[((q * NT + b) * 2 + 0) * 16 + row];
    M = fmaxf(M, mp[q]);
  }
  float L = 0.0f;
  float o[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int q = 0; q < kTileParts; ++q) {
    const float w = mp[q] == -INFINITY ? 0.0f : fast_exp2(mp[q] - M);   // an empty part adds 0
    L += w * lml[((q * NT + b) * 2 + 1) * 16 + row];
    const LdsF32* a = lacc + (((q * NT + b) * 4 + r) * kWave + lane) * 8;
#pragma unroll
    for (int u = 0; u < 8; ++u) o[u] += w * a[u];
  }
  const int m = 16 * b + row;
  const int qi = m / G, jh = m % G;
  if (qi >= nq) return;
  float inv = L > 0.0f ? 1.0f / L : 0.0f;
  if constexpr (kFp8) inv *= p.v_scale;
  const float lse = L > 0.0f ? (M + __builtin_log2f(L)) * kLn2 : -INFINITY;
  const int h = g * G + jh;
  const long long dst = ((long long)(q0 + qi) * Hq + h) * kD + 8 * t;
  if (p.out_f16) {
    half8_t hv;
#pragma unroll
    for (int e = 0; e < 8; ++e) hv[e] = static_cast<_Float16>(o[e] * inv);
    *reinterpret_cast<half8_t*>(static_cast<_Float16*>(p.out) + dst) = hv;
  } else {
    float* d = static_cast<float*>(p.out) + dst;
    *reinterpret_cast<f32x4*>(d) = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
    *reinterpret_cast<f32x4*>(d + 4) = f32x4{o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv};
  }
  if (p.lse_out && t == 0) p.lse_out[(long long)(q0 + qi) * Hq + h] = lse;
}

template <int G, int NT, bool kFp8>
__global__ __launch_bounds__(kWave * kTileParts) __attribute__((amdgpu_waves_per_eu(2)))
void mq_tile_kernel(MqParams p) {
  constexpr int Qt = 16 * NT / G;
  extern __shared__ float tile_lds[];
  __shared__ int scan[kTileParts + 2];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int i = blockIdx.x / p.Hkv;                // tile
  const int g = blockIdx.x % p.Hkv;                // KV head
  int s, j;
  if (!mq_find_tile<Qt>(p, i, scan, s, j)) return; // uniform over the work-group
  const int qb = mq_q_begin(p, s), nq_seq = mq_q_end(p, s) - qb;
  const int q0 = qb + j * Qt, nq = min(Qt, nq_seq - j * Qt);
  const int n = mq_seq_len(p, s);
  int base, ntok;
  if (p.causal) {
    base = n - nq_seq + j * Qt + 1;
    ntok = min(max(base + nq - 1, 0), n);
  } else {
    base = n;
    ntok = n;
  }
  // part `wave`: blocks [wave * nblk / 8, (wave + 1) * nblk / 8)
  const int nblk = (ntok + kBS - 1) / kBS;
  const int tok_lo = __builtin_amdgcn_readfirstlane(min(wave * nblk / kTileParts * kBS, ntok));
  const int tok_hi = __builtin_amdgcn_readfirstlane(min((wave + 1) * nblk / kTileParts * kBS, ntok));
  // the tile's Q operands into LDS once for the 8 waves (wave 4b + i stores
  // chunk i of row block b, what mq_load_q gives lane (c, t) of a wave), read
  // back at every block: held in registers they put the token loop past the
  // register budget of two waves per SIMD
  LdsU32x4* qlds = (LdsU32x4*)(tile_lds + mq_tile_state_floats(NT));
  if (wave < 4 * NT) {
    const int b = wave >> 2, ii = wave & 3;
    const int c = lane >> 4, t = lane & 15;
    const int m = 16 * b + t;
    const int qi = m / G, jh = m % G;
    const int row = q0 + min(qi, nq - 1);
    const _Float16* qrow = p.q + ((long long)row * p.Hq + (long long)g * G + jh) * kD;
    u32x4 x = *reinterpret_cast<const u32x4*>(qrow + KvFmt<kFp8>::q_dim(ii, c)) ^ p.q_sign;
    if (qi >= nq) x = u32x4{0u, 0u, 0u, 0u};
    qlds[(b * 4 + ii) * kWave + lane] = x;
  }
  __syncthreads();
  MqSeg<NT> st;
  mq_reg_fold<G, NT, kFp8, true>(p, lane, g, s, q0, nq, base, tok_lo, tok_hi, st, qlds);

  // the part's state: accumulators [part][b][r][lane][u], then per row of
  // each block the reference max and the sum over the part's tokens
  const int c = lane >> 4, t = lane & 15;
  float* lacc = tile_lds;
  float* lml = tile_lds + kTileParts * NT * 4 * kWave * 8;
#pragma unroll
  for (int b = 0; b < NT; ++b) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float* d = lacc + (((wave * NT + b) * 4 + r) * kWave + lane) * 8;
      *reinterpret_cast<f32x4*>(d) =
          f32x4{st.acc[b][0][r], st.acc[b][1][r], st.acc[b][2][r], st.acc[b][3][r]};
      *reinterpret_cast<f32x4*>(d + 4) =
          f32x4{st.acc[b][4][r], st.acc[b][5][r], st.acc[b][6][r], st.acc[b][7][r]};
    }
    float l = st.lp[b];
    l += __shfl_xor(l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    if (c == 0) {
      lml[((wave * NT + b) * 2 + 0) * 16 + t] = st.m[b];
      lml[((wave * NT + b) * 2 + 1) * 16 + t] = l;
    }
  }
  __syncthreads();
  // wave 4b + r finishes rows 4c + r of block b
  if (wave < 4 * NT)
    // the kernel's one explicit argument sits at the start of its argument segment
    mq_tile_finish<G, NT, kFp8>((ConstMqParams*)__builtin_amdgcn_kernarg_segment_ptr(),
                                (const LdsF32*)tile_lds, wave >> 2, wave & 3, lane, g, q0, nq);
}

// ---------------------------------------------------------------------------
// shared kernel: 4 waves per KV head share each K/V block through LDS

template <int G, int NT, bool kFp8>
__device__ __forceinline__ void mq_shared_segment(const MqParams& p, char* kv, int lane, int wave, int g, int i,
                                  int tok_lo, int tok_hi, bool whole, int slot) {
  using Fmt = KvFmt<kFp8>;
  using VRow = typename Fmt::VRow;
  using Chunk = VRow;                               // 8 elements: 16 bytes fp16, 8 bytes FP8
  constexpr int E = Fmt::kElemBytes;
  constexpr int KL = Fmt::kKLoads;
  constexpr int kRow = lds_row<kFp8>();
  constexpr int Qt = 64 * NT / G;
  constexpr int kStage = 2 * kBS * kRow;            // K rows then V rows of one block
  const int c = lane >> 4, t = lane & 15;
  const int s = p.t_seq[i], q0 = p.t_q0[i], nq = p.t_nq[i], base = p.t_base[i];
  const int n = mq_seq_len(p, s);
  const int row0 = wave * 16 * NT;                  // this wave's first row of the tile
  const bool idle = row0 / G >= nq;                 // none of the tile's queries (uniform)
  half8_t qa[NT][4];
  mq_load_q<G, NT, kFp8>(p, g, q0, nq, row0, lane, qa);
  const int causal_base = p.causal ? base : kNoMask;
  const int full_end = p.causal ? min(min(max(base + row0 / G, 0), n), tok_hi) : tok_hi;

  // thread (wave, lane) moves 8 elements of K and of V of each block: token
  // tid / 16, elements 8 * (tid % 16) of the row of KV head g
  const int tid = wave * kWave + lane;
  const int ltok = tid >> 4, lchunk = tid & 15;
  const unsigned row_bytes = (unsigned)(p.Hkv * kD * E);
  const unsigned g_off = (unsigned)((ltok * p.Hkv + g) * kD * E + 8 * E * lchunk);
  const int s_off = ltok * kRow + 8 * E * lchunk;
  const char* kbytes = reinterpret_cast<const char*>(p.k);
  const char* vbytes = reinterpret_cast<const char*>(p.v);
  const int nblk = (tok_hi - tok_lo + kBS - 1) / kBS;
  BlockWindow win(p.bt + (long long)s * p.bt_stride + tok_lo / kBS, nblk, lane, p.num_blocks,
                  (long long)kBS * row_bytes);

  MqSeg<NT> st;
  mq_seg_init(st);
  constexpr int NB = kShPrefetch;                  // even: stage = block parity = slot parity
  Chunk pk[NB], pv[NB];
#pragma unroll
  for (int ii = 0; ii < NB - 1; ++ii)
    if (ii < nblk) {
      const long long off = win.offset(ii);
      pk[ii] = kv_load<PDA_MQ_NT_STAGE != 0, Chunk>(kbytes + off + g_off);
      pv[ii] = kv_load<PDA_MQ_NT_STAGE != 0, Chunk>(vbytes + off + g_off);
    }
  for (int kb0 = 0; kb0 < nblk; kb0 += NB) {
#pragma unroll
    for (int sl = 0; sl < NB; ++sl) {
      const int cur = kb0 + sl;
      if (cur >= nblk) break;
      const int nxt = cur + NB - 1;
      if (nxt < nblk) {
        const long long off = win.offset(nxt);
        pk[(sl + NB - 1) % NB] = kv_load<PDA_MQ_NT_STAGE != 0, Chunk>(kbytes + off + g_off);
        pv[(sl + NB - 1) % NB] = kv_load<PDA_MQ_NT_STAGE != 0, Chunk>(vbytes + off + g_off);
      }
      // stage block cur; every wave finished the block that last used this
      // stage before the previous barrier
      char* stage = kv + (sl & 1) * kStage;
      *reinterpret_cast<Chunk*>(stage + s_off) = pk[sl];
      *reinterpret_cast<Chunk*>(stage + kBS * kRow + s_off) = pv[sl];
      __syncthreads();
      if (!idle) {
        u32x4 kr[KL];
        VRow vr[4];
#pragma unroll
        for (int ii = 0; ii < KL; ++ii)
          kr[ii] = *reinterpret_cast<const u32x4*>(stage + t * kRow + 16 * c + 64 * ii);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          vr[ii] = *reinterpret_cast<const VRow*>(stage + kBS * kRow + (4 * c + ii) * kRow +
                                                  8 * E * t);
        const int t0 = tok_lo + cur * kBS;
        if (t0 + kBS > full_end)
          mq_fold<G, NT, true, kFp8>(st, MqQRegs<NT>{qa}, kr, vr, p.qk_scale, lane, row0, t0, tok_hi - t0,
                                     causal_base, n, nq, tok_hi);
        else
          mq_fold<G, NT, false, kFp8>(st, MqQRegs<NT>{qa}, kr, vr, p.qk_scale, lane, row0, t0, kBS,
                                      causal_base, n, nq, tok_hi);
      }
    }
  }
  __syncthreads();                                  // the stages are free for the next segment
  if (!idle) mq_store<G, NT, Qt, kFp8>(p, st, g, q0, nq, row0, lane, whole, slot);
}

template <int G, int NT, bool kFp8>
__global__ __launch_bounds__(kWave * kMqWaves) __attribute__((amdgpu_waves_per_eu(2)))
void mq_shared_kernel(MqParams p) {
  __shared__ __attribute__((aligned(16))) char kv[2 * 2 * kBS * lds_row<kFp8>()];   // 2 stages: K, V
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int w = blockIdx.x / p.Hkv;                 // run of the unit stream
  const int g = blockIdx.x % p.Hkv;                 // KV head
  for_each_segment(p, w, [&](int i, int tok_lo, int tok_hi, bool whole, int slot) {
    mq_shared_segment<G, NT, kFp8>(p, kv, lane, wave, g, i, tok_lo, tok_hi, whole, slot);
  });
}

// ---------------------------------------------------------------------------
// wide kernel: 4 waves x 32 rows per tile on v_mfma_f32_32x32x16_f16, two
// blocks (32 tokens) per sub-step, one or two sub-steps per step
//
// On gfx950 a 32x32x16 f16 MFMA does twice the work of a 16x16x32 one and four
// times that of a 16x16x16 one in about the same issue time (measured: 2.28,
// 1.26 and 0.66 PFLOP/s with independent accumulators), so a tile of 32 rows x
// 32 tokens takes 16 MFMAs here where 16-row blocks over 16-token blocks take 48.
//   * S^T = K Q^T: A = K (32 tokens x 16 dims), B = Q^T, 8 MFMAs over D = 128.
//     Lane l (half hf = l >> 5, n = l & 31) holds query row n at tokens
//     8j + 4hf + i of the step (register 4j + i).  MFMA chunk kk covers head
//     dims 64hf + 8kk .. 64hf + 8kk + 7 in both operands.
//   * p.V: A = p (32 rows x 16 tokens), the lane's registers 8c .. 8c+7 for
//     token chunk c, whose contraction index 8hf + t maps to token
//     16c + 8(t >> 2) + 4hf + (t & 3); B = V at those tokens.  Output tile u
//     holds, in register r of lane l, row 8(r >> 2) + 4hf + (r & 3) at head dim
//     32u + n: the transposed LDS reads (16-bit elements over fp16, bytes over
//     FP8) hand lane l its 8 tokens of that dim (see wide_v_operands).

constexpr int kWideRows = 32;         // query rows per wave
// 32-token sub-steps per staged step (one barrier per step): four over FP8
// (its 128-token stages fit two work-groups per CU: chunked prefill 0.658 ->
// 0.653 ms, cascade 183 -> 178 us against two), two over fp16 (four would not
// fit; two spilled while its K/V went through registers)
#ifndef PDA_WIDE_NS_FP16
#define PDA_WIDE_NS_FP16 2
#endif
#ifndef PDA_WIDE_NS_FP8
#define PDA_WIDE_NS_FP8 4
#endif
#ifndef PDA_WIDE_STAGES
#define PDA_WIDE_STAGES 2             // LDS stages of K/V: steps in flight + 1
#endif
template <bool kFp8>
constexpr int wide_ns() { return kFp8 ? PDA_WIDE_NS_FP8 : PDA_WIDE_NS_FP16; }
constexpr int kWideStages = PDA_WIDE_STAGES;
static_assert(kWideStages >= 2 && kWideStages <= 4, "wide kernel stages");
// waits until at most n of this wave's vector memory operations are outstanding
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// 32-token sub-steps per online-softmax update: two for FP8 (chunked prefill
// 0.84 -> 0.75 ms against one), one for fp16 (two spill)
template <bool kFp8>
constexpr int wide_fold_ns() { return kFp8 ? 2 : 1; }
template <bool kFp8>
constexpr int wide_step() { return 2 * kBS * wide_ns<kFp8>(); }   // tokens per step
// A wide-kernel stage holds whole token rows of one KV head, 256 bytes fp16
// and 128 FP8, unpadded (the layout the direct global-to-LDS loads write).
// Token t sits in row slot wide_prow(t), and its 16-byte chunk c in chunk slot
// c ^ wide_swz(row slot), chosen so that the operand reads find their bytes in
// distinct banks of the 64 x 4-byte LDS (zero bank-conflict cycles counted):
//  - fp16 K (ds_read_b128, 16 lanes a cycle: one chunk of 16 rows): the swizzle
//    is a bijection of the row's low 4 bits;
//  - fp16 V (ds_read_b64_tr_b16, 32 lanes a cycle: chunks 4u .. 4u+3 of 4
//    consecutive rows): the swizzle's bits 2-3 take 4 values over the 4 rows
//    (swapping the row's 2-bit halves does both; row ^ chunk put the 4 rows on
//    the same banks: chunked prefill 0.699 -> 0.672 ms);
//  - FP8 K (16 lanes: one chunk of 16 rows): the swizzle is a bijection over
//    the 8 row slots of either parity (bits 1-3 of the slot, bits 0 and 1 of
//    that swapped);
//  - FP8 V (ds_read_b64_tr_b8, 32 lanes: chunks 2u, 2u + 1 of tokens 4hf + 0..3
//    and 8 + 4hf + 0..3 of a 16-token chunk): the swizzle's bits 1-2 differ
//    over the 4 row slots of either parity among them.
//    Rows 4..7 of each 8 trade places in pairs over FP8 (a layout made for
//    whole-row dword reads of V; the transposed reads find distinct banks with
//    it too).
template <bool kFp8>
constexpr int wide_row_bytes() { return kD * KvFmt<kFp8>::kElemBytes; }
// FP8 V operands by transposed byte reads (ds_read_b64_tr_b8), tile u at
// dims 32u + n as over fp16; else by whole-row dword reads and a byte
// transpose in registers, tile u at dims 4n + u
#ifndef PDA_WIDE_FP8_TR
#define PDA_WIDE_FP8_TR 1
#endif
constexpr bool kWideFp8Tr = PDA_WIDE_FP8_TR != 0;
template <bool kFp8>
__device__ __forceinline__ int wide_prow(int t) {       // an involution
  if constexpr (kFp8) return t ^ ((t >> 2) & 1);
  return t;
}
template <bool kFp8>
__device__ __forceinline__ int wide_swz(int pr) {
  if constexpr (kFp8) {
    const int i = (pr >> 1) & 7;
    if constexpr (kWideFp8Tr) return (i & 4) | ((i & 1) << 1) | ((i >> 1) & 1);
    return i;
  }
  return ((pr & 3) << 2) | ((pr >> 2) & 3);
}
template <bool kFp8>
__device__ __forceinline__ int wide_at(int t, int c) {
  const int pr = wide_prow<kFp8>(t);
  return pr * wide_row_bytes<kFp8>() + 16 * (c ^ wide_swz<kFp8>(pr));
}

__device__ __forceinline__ int wide_row(int r, int hf) { return 8 * (r >> 2) + 4 * hf + (r & 3); }

// A wave issues its QK^T MFMAs at raised priority (s_setprio 1), so that of the
// two waves on a SIMD the one with matrix work ready goes first while the other
// runs its softmax; over FP8 also its p.V MFMAs, whose operands it decodes in
// between.  Measured in one A/B run (chunked prefill / cascade): fp16 598 -> 594
// us / 201 -> 197 us with QK^T only, 602 / 199 us with both; FP8 578 -> 568 us
// with both, cascade unchanged.
template <bool kFp8>
constexpr bool wide_prio_pv() { return kFp8; }

typedef float f32x16 __attribute__((ext_vector_type(16)));

struct WideSeg {
  float m;                  // running reference max of row n (base 2), same in both halves
  float lp;                 // running sum of p over this lane's tokens of row n
  f32x16 acc[4];            // p.V tiles u = 0..3
};

// Q^T as the B operands of the wave's 32 rows: lane l loads row row0 + n, head
// dims 64hf .. 64hf + 63; rows past the tile's queries are zero.
template <int G>
__device__ __forceinline__ void wide_load_q(const MqParams& p, int g, int q0, int nq, int row0,
                                            int lane, half8_t (&qb)[8]) {
  const int n = lane & 31, hf = lane >> 5;
  const int m = row0 + n;
  const int qi = m / G, j = m % G;
  const int row = q0 + min(qi, nq - 1);
  const _Float16* qrow = p.q + ((long long)row * p.Hq + (long long)g * G + j) * kD + 64 * hf;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    u32x4 x = *reinterpret_cast<const u32x4*>(qrow + 8 * kk) ^ p.q_sign;
    if (qi >= nq) x = u32x4{0u, 0u, 0u, 0u};
    qb[kk] = __builtin_bit_cast(half8_t, x);
  }
}

// Per-lane byte offsets, within a stage and for token chunk c = 0, of the V
// reads of wide_v_operands (chunk c adds 16 rows, a constant: the row swizzle
// depends on a row's low 4 bits only).  fp16: entry 2u + r is the 8-byte
// transposed-read piece of tile u, token row 8r + 4hf + b; FP8 by transposed
// byte reads: entry u (repeated at u + 4) is the 8-byte piece of tile u; FP8
// by dword reads: entry 4jj + i is the 4 bytes (dims 4n .. 4n+3) of token row
// 8jj + 4hf + i.  Computed once per segment and kept opaque, so that every
// read is one of these registers plus an immediate offset (the stage, the
// sub-step and c), with no address arithmetic in the token loop.
template <bool kFp8>
__device__ __forceinline__ void wide_v_offsets(int lane, unsigned (&voff)[8]) {
  const int n = lane & 31, hf = lane >> 5;
  if constexpr (kFp8 && kWideFp8Tr) {
    // entry u: the 8-byte piece this lane addresses for tile u's transposed
    // read; in each 16-lane group lane 16q + 8h + e receives, as byte k, byte
    // e of the piece lane 16q + h + 2k addresses (probed on the device), so
    // lane 16q + a addresses dims 32u + 16(q & 1) + 8(a & 1) .. +7 of the
    // token that byte a / 2 of the P operand stands for
    const int q = lane >> 4, a = lane & 15, k = a >> 1;
    const int t = 8 * (k >> 2) + 4 * (q >> 1) + (k & 3);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      voff[u] = (unsigned)(wide_at<true>(t, 2 * u + (q & 1)) + 8 * (a & 1));
      voff[u + 4] = voff[u];
    }
  } else if constexpr (kFp8) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        voff[4 * jj + i] = (unsigned)(wide_at<true>(8 * jj + 4 * hf + i, n >> 2) + 4 * (n & 3));
  } else {
    const int a = n & 3, b = (n >> 2) & 3, g16 = n >> 4;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < 2; ++r)
        voff[2 * u + r] = (unsigned)(wide_at<false>(8 * r + 4 * hf + b, 4 * u + 2 * g16 + (a >> 1)) +
                                     8 * (a & 1));
  }
#pragma unroll
  for (int x = 0; x < 8; ++x) asm volatile("" : "+v"(voff[x]));
}

// B operands of the 4 p.V tiles for token chunk c from the step's V rows in
// LDS (row stride kRow; voff from wide_v_offsets).  Tokens at or past `valid`
// (relative to the step) are exact zeros, selected so that stale or poisoned
// rows cannot leak NaN.
template <bool kMasked, bool kFp8>
__device__ __forceinline__ void wide_v_operands(const char* vstage, const unsigned (&voff)[8],
                                                int c, int hf, int valid, half8_t (&vb)[4]) {
  constexpr int kRow = wide_row_bytes<kFp8>();
  const char* vc = vstage + 16 * c * kRow;
  if constexpr (kFp8 && kWideFp8Tr) {
    // byte k of a lane's read is token 16c + 8(k / 4) + 4hf + k % 4 of dim
    // 32u + n: the P operand's order.  Bytes of tokens at or past `valid`
    // become code 0 (+0).
    typedef int v2i __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(3))) v2i LdsV2i;
    unsigned m0 = ~0u, m1 = ~0u;
    if (kMasked) {
      auto keep = [](int nb) { return nb >= 4 ? ~0u : nb <= 0 ? 0u : (1u << (8 * nb)) - 1u; };
      const int r0 = valid - 16 * c - 4 * hf;      // bytes 0..3: tokens 16c + 4hf + 0..3
      m0 = keep(r0);
      m1 = keep(r0 - 8);                           // bytes 4..7: 8 tokens later
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LdsV2i*)(vc + voff[u]));
      const unsigned w0 = (unsigned)x[0] & m0, w1 = (unsigned)x[1] & m1;
      const half2_t a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
      const half2_t a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
      const half2_t b0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
      const half2_t b1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
      vb[u] = half8_t{a0[0], a0[1], a1[0], a1[1], b0[0], b0[1], b1[0], b1[1]};
    }
  } else if constexpr (kFp8) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      unsigned w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = 16 * c + 8 * jj + 4 * hf + i;
        w[i] = *reinterpret_cast<const unsigned*>(vc + voff[4 * jj + i]);
        if (kMasked && tok >= valid) w[i] = 0u;                      // code 0 = +0
      }
      // 4x4 byte transpose: col[u] = byte u (dim 4n + u) of the 4 tokens
      const unsigned ab_lo = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);
      const unsigned ab_hi = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);
      const unsigned cd_lo = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
      const unsigned cd_hi = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
      const unsigned col[4] = {__builtin_amdgcn_perm(cd_lo, ab_lo, 0x05040100u),
                               __builtin_amdgcn_perm(cd_lo, ab_lo, 0x07060302u),
                               __builtin_amdgcn_perm(cd_hi, ab_hi, 0x05040100u),
                               __builtin_amdgcn_perm(cd_hi, ab_hi, 0x07060302u)};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const half2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(col[u], 1.0f, false);
        const half2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(col[u], 1.0f, true);
        vb[u][4 * jj + 0] = lo[0];
        vb[u][4 * jj + 1] = lo[1];
        vb[u][4 * jj + 2] = hi[0];
        vb[u][4 * jj + 3] = hi[1];
      }
    }
  } else {
    // Transposed LDS reads (ds_read_b64_tr_b16): in each 16-lane group, lane
    // 4a + e receives element e of the 8-byte pieces that lanes a, a + 4,
    // a + 8, a + 12 of the group address.  Lane a + 4b addresses dims
    // 32u + 16 (n / 16) + 4a .. +3 of token 16c + 8r + 4hf + b, so lane n gets
    // dim 32u + n of the four tokens k = 8hf + 4r + b: tile u covers dims
    // 32u .. 32u + 31, column n dim 32u + n.
    typedef __fp16 fp16x4 __attribute__((vector_size(8)));    // the builtin's element type
    typedef __attribute__((address_space(3))) fp16x4 LdsHalf4;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const char* src = vc + voff[2 * u + r];
        half4_t x = __builtin_bit_cast(half4_t, __builtin_amdgcn_ds_read_tr16_b64_v4f16((LdsHalf4*)src));
        if (kMasked) {
#pragma unroll
          for (int e = 0; e < 4; ++e)   // element e came from token 16c + 8r + 4hf + e
            if (16 * c + 8 * r + 4 * hf + e >= valid) x[e] = static_cast<_Float16>(0.0f);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) vb[u][4 * r + e] = x[e];
      }
  }
}

// S^T of one step for the wave's 32 rows: the K rows of the step from LDS
// against the query rows held as B operands.
template <bool kFp8>
__device__ __forceinline__ f32x16 wide_qk(const half8_t (&qb)[8], const char* kstage, int lane) {
  const int n = lane & 31, hf = lane >> 5;
  f32x16 sc;
#pragma unroll
  for (int r = 0; r < 16; ++r) sc[r] = 0.0f;
  // every K read of the sub-step goes out before the first MFMA, so the LDS
  // latency is paid once (fp16 chunked prefill -1%)
  if constexpr (kFp8) {
    u32x4 kw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      kw[j] = *reinterpret_cast<const u32x4*>(kstage + wide_at<true>(n, 4 * hf + j));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 w = kw[j];
      half8_t kop[2];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const half2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[e], 1.0f, false);
        const half2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[e], 1.0f, true);
        kop[e / 2][4 * (e % 2) + 0] = lo[0];
        kop[e / 2][4 * (e % 2) + 1] = lo[1];
        kop[e / 2][4 * (e % 2) + 2] = hi[0];
        kop[e / 2][4 * (e % 2) + 3] = hi[1];
      }
      sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(kop[0], qb[2 * j], sc, 0, 0, 0);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(kop[1], qb[2 * j + 1], sc, 0, 0, 0);
    }
  } else {
    half8_t kop[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      kop[kk] = *reinterpret_cast<const half8_t*>(kstage + wide_at<false>(n, 8 * hf + kk));
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(kop[kk], qb[kk], sc, 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // the 8 LDS reads, then
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);   // the 8 MFMAs
  }
  return sc;
}

// The rest of a step of 32 tokens from t0 once its scores sc are known: the
// online softmax and p.V with the step's V rows from LDS.  In a masked step
// row row0 + n (query qi of the tile) sees tokens before min(base + qi, n_seq,
// tok_hi) when causal, before tok_hi otherwise; rows past the tile's queries
// see everything and are never stored.
template <int G, bool kMasked, bool kFp8, int kNS>
__device__ __forceinline__ void wide_tail(WideSeg& st, const f32x16 (&sc)[kNS],
                                          const char* vstage, const unsigned (&voff)[8],
                                          float qk_scale, int lane, int row0,
                                          int t0, int causal_base, int n_seq, int nq,
                                          int tok_hi) {
  constexpr int kRow = wide_row_bytes<kFp8>();
  const int n = lane & 31, hf = lane >> 5;
  float sv[kNS][16];
  if (kMasked) {
    const int qi = (row0 + n) / G;
    int e = tok_hi;
    if (qi < nq && causal_base != kNoMask) e = min(min(max(causal_base + qi, 0), n_seq), tok_hi);
#pragma unroll
    for (int j = 0; j < kNS; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sv[j][r] = t0 + 32 * j + wide_row(r, hf) < e ? sc[j][r] : -INFINITY;
  } else {
#pragma unroll
    for (int j = 0; j < kNS; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[j][r] = sc[j][r];
  }
  // lazy reference max, as in the 16-row fold: the 2 halves of a row combine
  // only when a score exceeds the reference by more than kLazyMax
  float xl = sv[0][0];
#pragma unroll
  for (int j = 0; j < kNS; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) xl = fmaxf(xl, sv[j][r]);
  if (__ballot(xl * qk_scale > st.m + kLazyMax) != 0) {   // uniform branch
    const float x = fmaxf(xl, __shfl_xor(xl, 32, kWave));
    float mb = x * qk_scale;
    if (kMasked) mb = x == -INFINITY ? -INFINITY : mb;   // a fully masked row stays -inf
    const float mn = fmaxf(st.m, mb);
    const float a = mn == st.m ? 1.0f : fast_exp2(st.m - mn);   // 0 on a first token
    st.m = mn;
    st.lp *= a;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float ar = __shfl(a, wide_row(r, hf), kWave);
#pragma unroll
      for (int u = 0; u < 4; ++u) st.acc[u][r] *= ar;
    }
  }
  float ps = 0.0f;
#pragma unroll
  for (int j = 0; j < kNS; ++j) {
    const int valid = tok_hi - t0 - 32 * j;
    // fp16: both chunks' V operands first, their LDS reads overlapping the
    // exponentials (chunked prefill 616 -> 586 us); FP8 decodes its operands
    // with VALU work of its own and reads them per chunk (574 vs 556 us)
    half8_t vb[2][4];
    if constexpr (!kFp8) {
#pragma unroll
      for (int c = 0; c < 2; ++c)
        wide_v_operands<kMasked, kFp8>(vstage + 32 * j * kRow, voff, c, hf, valid, vb[c]);
    }
    float pr[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pr[r] = fast_exp2(fmaf(sv[j][r], qk_scale, -st.m));
      if (kMasked) pr[r] = sv[j][r] == -INFINITY ? 0.0f : pr[r];   // -inf - (-inf) would be NaN
    }
#pragma unroll
    for (int r = 0; r < 16; r += 4) ps += (pr[r] + pr[r + 1]) + (pr[r + 2] + pr[r + 3]);
    if constexpr (wide_prio_pv<kFp8>()) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      half8_t pa;
#pragma unroll
      for (int t = 0; t < 8; ++t) pa[t] = static_cast<_Float16>(pr[8 * c + t]);
      if constexpr (kFp8) wide_v_operands<kMasked, kFp8>(vstage + 32 * j * kRow, voff, c, hf, valid, vb[c]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        st.acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa, vb[c][u], st.acc[u], 0, 0, 0);
    }
    if constexpr (wide_prio_pv<kFp8>()) __builtin_amdgcn_s_setprio(0);
  }
  st.lp += ps;
}

// Normalise and store the wave's rows: register r of lane l holds row
// row0 + wide_row(r, hf) at head dims n, 32 + n, 64 + n, 96 + n (tiles 0..3),
// or over an FP8 cache read without the transposed byte reads, at dims
// 4n .. 4n+3.
template <int G, bool kFp8>
__device__ __forceinline__ void wide_store(const MqParams& p, WideSeg& st, int g, int q0, int nq,
                                           int row0, int lane, bool whole, int slot) {
  constexpr int Qt = kMqWaves * kWideRows / G;
  const int n = lane & 31;
  int hf = lane >> 5;
  // opaque: otherwise the row indices below are hoisted out of the token loop
  // and their registers spill
  asm volatile("" : "+v"(hf));
  const float lrow = st.lp + __shfl_xor(st.lp, 32, kWave);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int R = wide_row(r, hf);
    const float l = __shfl(lrow, R, kWave);
    const float mr = __shfl(st.m, R, kWave);
    const int row = row0 + R;
    const int qi = row / G, j = row % G;
    if (qi >= nq) continue;
    float inv = l > 0.0f ? 1.0f / l : 0.0f;
    if constexpr (kFp8) inv *= p.v_scale;
    const float lse = l > 0.0f ? (mr + __builtin_log2f(l)) * kLn2 : -INFINITY;
    const f32x4 o = {st.acc[0][r] * inv, st.acc[1][r] * inv, st.acc[2][r] * inv,
                     st.acc[3][r] * inv};
    const int h = g * G + j;
    if constexpr (!kFp8 || kWideFp8Tr) {          // tile u at dims 32u + n
      if (whole) {
        const long long dst = ((long long)(q0 + qi) * p.Hq + h) * kD + n;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (p.out_f16)
            static_cast<_Float16*>(p.out)[dst + 32 * u] = static_cast<_Float16>(o[u]);
          else
            static_cast<float*>(p.out)[dst + 32 * u] = o[u];
        }
        if (p.lse_out && n == 0) p.lse_out[(long long)(q0 + qi) * p.Hq + h] = lse;
      } else {
        const long long sl = ((long long)slot * Qt + qi) * p.Hq + h;
#pragma unroll
        for (int u = 0; u < 4; ++u) p.ws_o[sl * kD + 32 * u + n] = o[u];
        if (n == 0) p.ws_lse[sl] = lse;
      }
      continue;
    }
    if (whole) {
      const long long dst = ((long long)(q0 + qi) * p.Hq + h) * kD + 4 * n;
      if (p.out_f16) {
        const half4_t hv = {static_cast<_Float16>(o[0]), static_cast<_Float16>(o[1]),
                            static_cast<_Float16>(o[2]), static_cast<_Float16>(o[3])};
        *reinterpret_cast<half4_t*>(static_cast<_Float16*>(p.out) + dst) = hv;
      } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + dst) = o;
      }
      if (p.lse_out && n == 0) p.lse_out[(long long)(q0 + qi) * p.Hq + h] = lse;
    } else {
      const long long sl = ((long long)slot * Qt + qi) * p.Hq + h;
      *reinterpret_cast<f32x4*>(p.ws_o + sl * kD + 4 * n) = o;
      if (n == 0) p.ws_lse[sl] = lse;
    }
  }
}

template <int G, bool kFp8>
__device__ __forceinline__ void mq_wide_segment(const MqParams& p,
                                                char* const (&stage)[kWideStages][2],
                                                int lane, int wave, int g, int i, int tok_lo,
                                                int tok_hi, bool whole, int slot) {
  constexpr int E = KvFmt<kFp8>::kElemBytes;
  constexpr int kRow = wide_row_bytes<kFp8>();
  constexpr int kNS = wide_ns<kFp8>();
  constexpr int kStepTok = wide_step<kFp8>();
  const int s = __builtin_amdgcn_readfirstlane(p.t_seq[i]);
  const int q0 = p.t_q0[i], nq = p.t_nq[i], base = p.t_base[i];
  tok_lo = __builtin_amdgcn_readfirstlane(tok_lo);
  tok_hi = __builtin_amdgcn_readfirstlane(tok_hi);
  const int n_seq = mq_seq_len(p, s);
  const int row0 = wave * kWideRows;
  const bool idle = row0 / G >= nq;                 // none of the tile's queries (uniform)
  half8_t qb[8];
  wide_load_q<G>(p, g, q0, nq, row0, lane, qb);
  const int causal_base = p.causal ? base : kNoMask;
  const int full_end = p.causal ? min(min(max(base + row0 / G, 0), n_seq), tok_hi) : tok_hi;

  const unsigned row_bytes = (unsigned)(p.Hkv * kD * E);
  const char* kbytes = reinterpret_cast<const char*>(p.k);
  const char* vbytes = reinterpret_cast<const char*>(p.v);
  const int nblk = (tok_hi - tok_lo + kBS - 1) / kBS;
  const int nstep = (nblk + 2 * kNS - 1) / (2 * kNS);
  // block ids by scalar loads (the table is not written while the kernel runs)
  ConstI32* bt_s = (ConstI32*)(p.bt + (long long)s * p.bt_stride + tok_lo / kBS);
  const long long block_bytes = (long long)kBS * row_bytes;

  WideSeg st;
  st.m = -INFINITY;
  st.lp = 0.0f;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.acc[u][r] = 0.0f;

  unsigned voff[8];
  wide_v_offsets<kFp8>(lane, voff);
  // the step's sub-steps, kFS at a time; a group wholly past tok_hi would
  // add exact zeros and is skipped
  constexpr int kFS = wide_fold_ns<kFp8>();
  auto fold_step = [&](int cur, const char* kstage, const char* vstage) {
#pragma unroll
    for (int j0 = 0; j0 < kNS; j0 += kFS) {
      const int t0 = tok_lo + cur * kStepTok + 32 * j0;
      if (j0 > 0 && t0 >= tok_hi) break;
      f32x16 sc[kFS];
      __builtin_amdgcn_s_setprio(1);               // see wide_prio_pv
#pragma unroll
      for (int j = 0; j < kFS; ++j)
        sc[j] = wide_qk<kFp8>(qb, kstage + 32 * (j0 + j) * kRow, lane);
      __builtin_amdgcn_s_setprio(0);
      const char* vs = vstage + 32 * j0 * kRow;
      if (t0 + 32 * kFS > full_end)
        wide_tail<G, true, kFp8, kFS>(st, sc, vs, voff, p.qk_scale, lane, row0, t0, causal_base, n_seq,
                                      nq, tok_hi);
      else
        wide_tail<G, false, kFp8, kFS>(st, sc, vs, voff, p.qk_scale, lane, row0, t0, causal_base,
                                       n_seq, nq, tok_hi);
    }
  };
  // Direct global-to-LDS staging (global_load_lds_dwordx4, probed on the
  // device: lane l's 16 bytes land at the wave's LDS base + 16 l).  A step's
  // K (or V) rows are kLoads pieces of 1024 bytes, kR row slots each; wave w
  // moves pieces w, w + 4, ..., lane l chunk slot l % kC of row slot l / kC of
  // its piece, so it fetches chunk (l % kC) ^ wide_swz(row slot) of the token
  // wide_prow(row slot).  With S stages, steps cur + 1 .. cur + S - 2 are in
  // flight while step cur is folded: the loads of step cur + S - 1 go out
  // right after the barrier of step cur into the stage step cur - 1 used
  // (which every wave has finished), and before each barrier a wave waits for
  // its own loads of that step only (every step issues the same loads, so
  // the count of later ones outstanding is known).  Rows past the segment's
  // end get its last block again: they lie past tok_hi, where the softmax
  // masks them and their V rows are selected to zero.  The stages are
  // separate LDS arrays and the step loop is unrolled by S, so that the
  // compiler can tell a step's operand reads from the loads in flight into
  // the other stages and puts no wait for those before them.
  typedef __attribute__((address_space(3))) void LdsVoid;
  typedef const __attribute__((address_space(1))) void GlobalVoid;
  constexpr int kC = kRow / 16;                     // 16-byte chunks per row
  constexpr int kR = kWave / kC;                    // rows per piece
  constexpr int kLoads = kStepTok / kR / kMqWaves;  // pieces per wave, K and V each
  static_assert(kBS % kR == 0 && (kStepTok / kR) % kMqWaves == 0 && (kMqWaves * kR) % kBS == 0,
                "piece mapping");
  const int prow = (wave * kR) % kBS + lane / kC;   // row slot within its block, every piece
  const int trow = wide_prow<kFp8>(prow);           // the token it holds
  const unsigned src_off =
      (unsigned)((trow * p.Hkv + g) * kD * E + 16 * ((lane % kC) ^ wide_swz<kFp8>(prow)));
  constexpr int kStepLoads = 2 * kLoads;            // a wave's loads of one step
  constexpr int S = kWideStages;
  // The block ids of the next step to issue are read one step ahead of their
  // use (scalar loads, waited for only where the addresses need them): read
  // just before the loads, each id's latency sat between the barrier and the
  // loads it releases.  An id past the segment's last step is clamped to its
  // last block, so every read stays inside the segment's part of the table.
  const unsigned nb32 = (unsigned)min(p.num_blocks, 0xFFFFFFFFll);
  unsigned ids[kLoads];
  auto load_ids = [&](int step) {
#pragma unroll
    for (int l = 0; l < kLoads; ++l)
      ids[l] = (unsigned)bt_s[min(2 * kNS * step + (wave + kMqWaves * l) * kR / kBS, nblk - 1)];
  };
  auto issue = [&](char* kst, char* vst) {
#pragma unroll
    for (int l = 0; l < kLoads; ++l) {
      const int piece = wave + kMqWaves * l;
      const long long off = (long long)(ids[l] < nb32 ? ids[l] : 0u) * block_bytes;
      __builtin_amdgcn_global_load_lds((GlobalVoid*)(kbytes + off + src_off),
                                       (LdsVoid*)(kst + piece * kWave * 16), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((GlobalVoid*)(vbytes + off + src_off),
                                       (LdsVoid*)(vst + piece * kWave * 16), 16, 0, 0);
    }
  };
  wait_vmcnt<0>();                                  // the previous segment's stores
#pragma unroll
  for (int k = 0; k < S - 1; ++k)
    if (k < nstep) {
      load_ids(k);
      issue(stage[k][0], stage[k][1]);
    }
  if (S - 1 < nstep) load_ids(S - 1);
  for (int cur = 0; cur < nstep; cur += S) {
#pragma unroll
    for (int sl = 0; sl < S; ++sl) {
      const int c = cur + sl;
      if (c >= nstep) break;
      // this wave's loads of step c: the loads of steps c + 1 .. c + S - 2
      // (those issued) went out after them
      const int later = min(S - 2, nstep - 1 - c);
      if (later >= 2) wait_vmcnt<2 * kStepLoads>();
      else if (later == 1) wait_vmcnt<kStepLoads>();
      else wait_vmcnt<0>();
      // a bare barrier: a fence with it would wait for every load in flight.
      // Each wave has waited for its loads of step c above, and its LDS reads
      // of the stage the next loads overwrite were consumed by its MFMAs of
      // step c - 1 before it got here.
      __builtin_amdgcn_s_barrier();
      if (c + S - 1 < nstep) {
        issue(stage[(sl + S - 1) % S][0], stage[(sl + S - 1) % S][1]);
        load_ids(c + S);
      }
      if (!idle) fold_step(c, stage[sl][0], stage[sl][1]);
    }
  }
  __syncthreads();                                  // the stages are free for the next segment
  if (!idle) wide_store<G, kFp8>(p, st, g, q0, nq, row0, lane, whole, slot);
}

// ---------------------------------------------------------------------------
// fp16 wide fold, software-pipelined over 32-token sub-steps: the QK^T MFMAs
// of sub-step t + 1 are issued between the exponentials of sub-step t, and
// its p.V MFMAs follow, so that one wave's matrix and vector work overlap
// (in wide_tail a sub-step's softmax waits for its own QK^T chain, and its
// p.V for the softmax).  Same arithmetic per sub-step as wide_tail with one
// sub-step at a time.

// The lazy reference max check of a sub-step's scores (masked ones are -inf),
// with the rescale when a score passes the reference.
__device__ __forceinline__ void wide_pipe_check(WideSeg& st, const f32x16& sc, float qk_scale,
                                                int lane) {
  const int hf = lane >> 5;
  float xl = sc[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) xl = fmaxf(xl, sc[r]);
  if (__ballot(xl * qk_scale > st.m + kLazyMax) != 0) {   // uniform branch
    const float x = fmaxf(xl, __shfl_xor(xl, 32, kWave));
    const float mn = fmaxf(st.m, x * qk_scale);           // qk_scale > 0: -inf stays -inf
    const float a = mn == st.m ? 1.0f : fast_exp2(st.m - mn);
    st.m = mn;
    st.lp *= a;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float ar = __shfl(a, wide_row(r, hf), kWave);
#pragma unroll
      for (int u = 0; u < 4; ++u) st.acc[u][r] *= ar;
    }
  }
}

// p of the checked scores sc (masked ones -inf) with the QK^T MFMAs of the
// next sub-step (K rows at knext) issued in between, then the p.V MFMAs; sc
// becomes the next sub-step's scores.  The exponent's reference is kept
// finite, so that with qk_scale > 0 a masked score gives exp2(-inf) = 0 even
// in a row that has seen no token yet.
__device__ __forceinline__ void wide_pipe_fold(WideSeg& st, f32x16& sc, const half8_t (&qb)[8],
                                               const char* knext, const half8_t (&vb)[2][4],
                                               float qk_scale, int lane) {
  const int n = lane & 31, hf = lane >> 5;
  f32x16 sn;
#pragma unroll
  for (int r = 0; r < 16; ++r) sn[r] = 0.0f;
  const float m = fmaxf(st.m, -3.0e38f);
  float ps[2];
  half8_t pa[2];
  // the next sub-step's K operands in two halves of 4 registers, each half's
  // 4 MFMAs between the exponentials of 8 of this sub-step's rows
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    half8_t kop[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      kop[k] = *reinterpret_cast<const half8_t*>(knext + wide_at<false>(n, 8 * hf + 4 * h + k));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      sn = __builtin_amdgcn_mfma_f32_32x32x16_f16(kop[k], qb[4 * h + k], sn, 0, 0, 0);
      const int r = 8 * h + 2 * k;
      const float p0 = fast_exp2(fmaf(sc[r], qk_scale, -m));
      const float p1 = fast_exp2(fmaf(sc[r + 1], qk_scale, -m));
      pa[h][2 * k] = static_cast<_Float16>(p0);
      pa[h][2 * k + 1] = static_cast<_Float16>(p1);
      ps[h] = k == 0 ? p0 + p1 : ps[h] + (p0 + p1);
    }
  }
  st.lp += ps[0] + ps[1];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int u = 0; u < 4; ++u)
      st.acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa[c], vb[c][u], st.acc[u], 0, 0, 0);
  sc = sn;
}

template <int G>
__device__ __forceinline__ void mq_wide_segment_pipe(const MqParams& p,
                                                     char* const (&stage)[kWideStages][2],
                                                     int lane, int wave, int g, int i, int tok_lo,
                                                     int tok_hi, bool whole, int slot) {
  static_assert(kWideStages == 2 && wide_ns<false>() == 2, "pipelined fold: 2 stages of 2 sub-steps");
  constexpr int E = 2;
  constexpr int kRow = wide_row_bytes<false>();
  constexpr int kNS = 2;
  const int s = __builtin_amdgcn_readfirstlane(p.t_seq[i]);
  // uniform per tile: scalar, so that the branches on them are scalar too
  const int q0 = __builtin_amdgcn_readfirstlane(p.t_q0[i]);
  const int nq = __builtin_amdgcn_readfirstlane(p.t_nq[i]);
  const int base = __builtin_amdgcn_readfirstlane(p.t_base[i]);
  tok_lo = __builtin_amdgcn_readfirstlane(tok_lo);
  tok_hi = __builtin_amdgcn_readfirstlane(tok_hi);
  const int n_seq = mq_seq_len(p, s);
  const int row0 = wave * kWideRows;
  const int hf = lane >> 5;
  const bool idle = row0 / G >= nq;                 // none of the tile's queries (uniform)
  half8_t qb[8];
  wide_load_q<G>(p, g, q0, nq, row0, lane, qb);
  const int causal_base = p.causal ? base : kNoMask;
  const int full_end = p.causal ? min(min(max(base + row0 / G, 0), n_seq), tok_hi) : tok_hi;

  const unsigned row_bytes = (unsigned)(p.Hkv * kD * E);
  const char* kbytes = reinterpret_cast<const char*>(p.k);
  const char* vbytes = reinterpret_cast<const char*>(p.v);
  const int nblk = (tok_hi - tok_lo + kBS - 1) / kBS;
  const int nstep = (nblk + 2 * kNS - 1) / (2 * kNS);
  const int nsub = (tok_hi - tok_lo + 31) / 32;     // sub-steps holding tokens
  ConstI32* bt_s = (ConstI32*)(p.bt + (long long)s * p.bt_stride + tok_lo / kBS);
  const long long block_bytes = (long long)kBS * row_bytes;

  WideSeg st;
  st.m = -INFINITY;
  st.lp = 0.0f;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.acc[u][r] = 0.0f;
  unsigned voff[8];
  wide_v_offsets<false>(lane, voff);

  // staging as in mq_wide_segment (2 stages; the loads of step k go out
  // after the barrier that opens step k - 1)
  typedef __attribute__((address_space(3))) void LdsVoid;
  typedef const __attribute__((address_space(1))) void GlobalVoid;
  constexpr int kC = kRow / 16;
  constexpr int kR = kWave / kC;
  constexpr int kLoads = wide_step<false>() / kR / kMqWaves;
  static_assert(kBS % kR == 0 && (wide_step<false>() / kR) % kMqWaves == 0 && (kMqWaves * kR) % kBS == 0,
                "piece mapping");
  const int prow = (wave * kR) % kBS + lane / kC;
  const int trow = wide_prow<false>(prow);
  const unsigned src_off =
      (unsigned)((trow * p.Hkv + g) * kD * E + 16 * ((lane % kC) ^ wide_swz<false>(prow)));
  const unsigned nb32 = (unsigned)min(p.num_blocks, 0xFFFFFFFFll);
  unsigned ids[kLoads];
  auto load_ids = [&](int step) {
#pragma unroll
    for (int l = 0; l < kLoads; ++l)
      ids[l] = (unsigned)bt_s[min(2 * kNS * step + (wave + kMqWaves * l) * kR / kBS, nblk - 1)];
  };
  auto issue = [&](char* kst, char* vst) {
#pragma unroll
    for (int l = 0; l < kLoads; ++l) {
      const int piece = wave + kMqWaves * l;
      const long long off = (long long)(ids[l] < nb32 ? ids[l] : 0u) * block_bytes;
      __builtin_amdgcn_global_load_lds((GlobalVoid*)(kbytes + off + src_off),
                                       (LdsVoid*)(kst + piece * kWave * 16), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((GlobalVoid*)(vbytes + off + src_off),
                                       (LdsVoid*)(vst + piece * kWave * 16), 16, 0, 0);
    }
  };

  wait_vmcnt<0>();                                  // the previous segment's stores
  if (nstep > 0) {
    load_ids(0);
    issue(stage[0][0], stage[0][1]);
  }
  if (nstep > 1) load_ids(1);
  __syncthreads();                                  // step 0's rows are in
  if (nstep > 1) {
    issue(stage[1][0], stage[1][1]);
    load_ids(2);
  }
  f32x16 sc;
  if (!idle && nsub > 0) sc = wide_qk<false>(qb, stage[0][0], lane);
  half8_t vb[2][4];
  for (int cur = 0; cur < nstep; cur += 2) {
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      const int c = cur + sl;
      if (c >= nstep) break;
      char* const kcur = stage[sl][0];
      char* const vcur = stage[sl][1];
      const char* knxt = stage[sl ^ 1][0];
      // sub-step t: its mask and max check, then its V operands (registers)
      auto prepare = [&](int t, const char* vsub) {
        const int t0 = tok_lo + 32 * t;
        if (t0 + 32 > full_end) {                   // causal diagonal or segment end
          const int qi = (row0 + (lane & 31)) / G;
          int e = tok_hi;
          if (qi < nq && causal_base != kNoMask) e = min(min(max(causal_base + qi, 0), n_seq), tok_hi);
#pragma unroll
          for (int r = 0; r < 16; ++r) sc[r] = t0 + wide_row(r, hf) < e ? sc[r] : -INFINITY;
        }
        wide_pipe_check(st, sc, p.qk_scale, lane);
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) wide_v_operands<false, false>(vsub, voff, cc, hf, 0, vb[cc]);
        if (t0 + 32 > tok_hi) {                     // rows past the segment: exact zeros
          const int valid = tok_hi - t0;
#pragma unroll
          for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
              for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int e = 0; e < 4; ++e)     // element 4r + e: token 16cc + 8r + 4hf + e
                  if (16 * cc + 8 * r + 4 * hf + e >= valid) vb[cc][u][4 * r + e] = static_cast<_Float16>(0.0f);
        }
      };
      const bool work0 = !idle;                     // sub-step 2c holds tokens (c < nstep)
      const bool work1 = !idle && kNS * c + 1 < nsub;
      if (work0) {
        prepare(kNS * c, vcur);
        wide_pipe_fold(st, sc, qb, kcur + 32 * kRow, vb, p.qk_scale, lane);
      }
      if (work1) prepare(kNS * c + 1, vcur + 32 * kRow);
      // the next step's rows are in once every wave's loads of it are (the
      // fenced barrier waits for this wave's loads and LDS reads); this
      // stage's reads have then returned, so the loads of step c + 2 may
      // refill it.  A fence the compiler models, on every step: with a bare
      // barrier and a wait of our own it still waited for the loads in
      // flight before later reads of the other stage.
      __syncthreads();
      if (c + 2 < nstep) {
        issue(kcur, vcur);
        load_ids(c + 3);
      }
      // the next sub-step's K rows come from the next stage; past the
      // segment's last sub-step they are stale rows, read and then unused
      if (work1) wide_pipe_fold(st, sc, qb, knxt, vb, p.qk_scale, lane);
    }
  }
  __syncthreads();                                  // the stages are free for the next segment
  if (!idle) wide_store<G, false>(p, st, g, q0, nq, row0, lane, whole, slot);
}

#ifndef PDA_WIDE_PIPE
#define PDA_WIDE_PIPE 1               // fp16: the software-pipelined fold
#endif

template <int G, bool kFp8>
__global__ __launch_bounds__(kWave * kMqWaves) __attribute__((amdgpu_waves_per_eu(2)))
void mq_wide_kernel(MqParams p) {
  // the stages of K and V rows, each its own array
  constexpr int kHalf = wide_step<kFp8>() * wide_row_bytes<kFp8>();
  __shared__ __attribute__((aligned(16))) char k0[kHalf], v0[kHalf], k1[kHalf], v1[kHalf];
#if PDA_WIDE_STAGES >= 3
  __shared__ __attribute__((aligned(16))) char k2[kHalf], v2[kHalf];
#endif
#if PDA_WIDE_STAGES >= 4
  __shared__ __attribute__((aligned(16))) char k3[kHalf], v3[kHalf];
#endif
  char* const stage[kWideStages][2] = {{k0, v0}, {k1, v1}
#if PDA_WIDE_STAGES >= 3
                                       , {k2, v2}
#endif
#if PDA_WIDE_STAGES >= 4
                                       , {k3, v3}
#endif
  };
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int w = blockIdx.x / p.Hkv;                 // run of the unit stream
  const int g = blockIdx.x % p.Hkv;                 // KV head
  for_each_segment<PDA_WIDE_REVERSE != 0>(p, w, [&](int i, int tok_lo, int tok_hi, bool whole,
                                                     int slot) {
    if constexpr (!kFp8 && PDA_WIDE_PIPE != 0)
      mq_wide_segment_pipe<G>(p, stage, lane, wave, g, i, tok_lo, tok_hi, whole, slot);
    else
      mq_wide_segment<G, kFp8>(p, stage, lane, wave, g, i, tok_lo, tok_hi, whole, slot);
  });
}

// ---------------------------------------------------------------------------
// merge: the rows of tiles cut by run boundaries, and of tiles that see no
// token; one wave per (listed tile, row), spread over the grid

// R consecutive rows of one listed tile, all with nseg <= kSmallSeg partials
// in slots slot0 .. slot0 + nseg - 1: every load of the R rows is issued at
// once (the lse values as broadcast loads), and each lane merges its two
// dims of every row on its own (the same arithmetic as merge_row, with the
// weights summed in each lane).
constexpr int kMergeRows = 4;
constexpr int kSmallSeg = 8;
__device__ __forceinline__ void merge_rows_small(const float* o, const float* lse, long long slot0,
                                                 int nseg, long long rows, long long row0,
                                                 int lane, f32x2 (&res)[kMergeRows],
                                                 float (&lse_res)[kMergeRows]) {
  float lv[kMergeRows][kSmallSeg];
  f32x2 ov[kMergeRows][kSmallSeg];
#pragma unroll
  for (int r = 0; r < kMergeRows; ++r)
#pragma unroll
    for (int sg = 0; sg < kSmallSeg; ++sg) {
      // rows past the tile's last row (rows need not be a multiple of
      // kMergeRows) re-read the last one; they are never stored
      const long long at = (slot0 + sg) * rows + min(row0 + r, rows - 1);
      lv[r][sg] = sg < nseg ? lse[at] : -INFINITY;
      ov[r][sg] = sg < nseg ? *reinterpret_cast<const f32x2*>(o + at * kD + 2 * lane)
                            : f32x2{0.0f, 0.0f};
    }
#pragma unroll
  for (int r = 0; r < kMergeRows; ++r) {
    float L = lv[r][0];
#pragma unroll
    for (int sg = 1; sg < kSmallSeg; ++sg) L = fmaxf(L, lv[r][sg]);
    res[r] = f32x2{0.0f, 0.0f};
    lse_res[r] = -INFINITY;
    if (L == -INFINITY) continue;
    float wsum = 0.0f;
    f32x2 acc = {0.0f, 0.0f};
#pragma unroll
    for (int sg = 0; sg < kSmallSeg; ++sg) {
      const float w = sg < nseg ? fast_exp2((lv[r][sg] - L) * kLog2e) : 0.0f;
      wsum += w;
      acc.x = fmaf(w, ov[r][sg].x, acc.x);
      acc.y = fmaf(w, ov[r][sg].y, acc.y);
    }
    const float inv = 1.0f / wsum;
    res[r] = f32x2{acc.x * inv, acc.y * inv};
    lse_res[r] = L + __builtin_logf(wsum);
  }
}

template <int Qt>
__global__ __launch_bounds__(256) void mq_merge_kernel(MqParams p) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  // rows of a tile: Qt * Hq, in groups of kMergeRows (the last one may be short)
  const long long rows = (long long)Qt * p.Hq;
  const long long groups = (rows + kMergeRows - 1) / kMergeRows;
  const int n_fix = p.hdr[5];
  for (long long idx = (long long)blockIdx.x * 4 + wave;; idx += (long long)gridDim.x * 4) {
    const int f = (int)min(idx / groups, (long long)p.tiles_max - 1);
    const long long row0 = (idx % groups) * kMergeRows;
    // read with the header, before the bound is known (the index is clamped)
    const int4 rec = *reinterpret_cast<const int4*>(p.t_rec + 4 * f);
    if (idx >= (long long)n_fix * groups) break;
    const int q0 = rec.x, nq = rec.y, nseg = rec.w;
    const long long slot0 = rec.z;
    if (row0 / p.Hq >= nq) continue;                 // every row past the tile's queries
    f32x2 res[kMergeRows];
    float lse_res[kMergeRows];
    if (nseg <= kSmallSeg) {
      merge_rows_small(p.ws_o, p.ws_lse, slot0, nseg, rows, row0, lane, res, lse_res);
    } else {
#pragma unroll
      for (int r = 0; r < kMergeRows; ++r)
        merge_row(p.ws_o, p.ws_lse, slot0, 1, nseg, rows, min(row0 + r, rows - 1), lane, res[r],
                  lse_res[r]);
    }
#pragma unroll
    for (int r = 0; r < kMergeRows; ++r) {
      const long long row = row0 + r;
      const int qi = (int)(row / p.Hq), h = (int)(row % p.Hq);
      if (row >= rows || qi >= nq) continue;
      const long long dst = ((long long)(q0 + qi) * p.Hq + h) * kD + 2 * lane;
      if (p.out_f16) {
        half2_t hv = {static_cast<_Float16>(res[r].x), static_cast<_Float16>(res[r].y)};
        *reinterpret_cast<half2_t*>(static_cast<_Float16*>(p.out) + dst) = hv;
      } else {
        *reinterpret_cast<f32x2*>(static_cast<float*>(p.out) + dst) = res[r];
      }
      if (p.lse_out && lane == 0) p.lse_out[(long long)(q0 + qi) * p.Hq + h] = lse_res[r];
    }
  }
}

// ---------------------------------------------------------------------------
// host side

constexpr int kMaxDevices = 64;
// tile kernel variants: 0, 1 = register kernel with NT = 1, 2 (16- and 32-row
// tiles); 2 = shared kernel (64-row tiles); 3 = wide kernel (128-row tiles)
constexpr int kMqVariants = 4;
// query heads per KV head the kernels are built for, and their table index
constexpr int kMqGroups = 5;
constexpr int kMqGroupSizes[kMqGroups] = {1, 2, 4, 6, 8};
struct MqDeviceFacts {
  std::once_flag once;
  int cus = 0;
  int wg_per_cu[kMqGroups][kMqVariants][2][2 * kMqWaves + 1] = {};   // [G index][variant][fp8][waves]
};
MqDeviceFacts g_mq_dev[kMaxDevices];

int mq_gidx(int G) { return G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : G == 6 ? 3 : 4; }

template <int G, bool kFp8>
const void* mq_kernel_ptr_g(int variant) {
  switch (variant) {
    case 0: return reinterpret_cast<const void*>(&mq_reg_kernel<G, 1, kFp8>);
    case 1: return reinterpret_cast<const void*>(&mq_reg_kernel<G, 2, kFp8>);
    case 2: return reinterpret_cast<const void*>(&mq_shared_kernel<G, 1, kFp8>);
    default: return reinterpret_cast<const void*>(&mq_wide_kernel<G, kFp8>);
  }
}

template <bool kFp8>
const void* mq_kernel_ptr_f(int G, int variant) {
  switch (G) {
    case 1: return mq_kernel_ptr_g<1, kFp8>(variant);
    case 2: return mq_kernel_ptr_g<2, kFp8>(variant);
    case 4: return mq_kernel_ptr_g<4, kFp8>(variant);
    case 6: return mq_kernel_ptr_g<6, kFp8>(variant);
    default: return mq_kernel_ptr_g<8, kFp8>(variant);
  }
}

const void* mq_kernel_ptr(int G, int variant, bool fp8) {
  return fp8 ? mq_kernel_ptr_f<true>(G, variant) : mq_kernel_ptr_f<false>(G, variant);
}

int mq_head_group(int Hkv) {
  for (int hg = kMqWaves; hg > 1; --hg)
    if (Hkv % hg == 0) return hg;
  return 1;
}

#ifndef PDA_MQ_MAX_VARIANT
#define PDA_MQ_MAX_VARIANT 3      // largest tile kernel variant the host picks
#endif

// Tile kernel for the average query rows per sequence (query tokens x G): the
// register kernel with one or two 16-row blocks per wave up to 16 or 32 rows
// (no barrier per block; each wave streams its own K/V), the shared kernel
// with 64-row tiles up to 64 rows, above that the wide kernel with 128-row
// tiles, so that a sequence's K/V is read by few tiles.  Measured on MI355X: a
// 24-row workload (speculative verification) ran faster on 16-row register
// tiles than on one shared 64-row tile (144 vs 218 us); chunked prefill (4096
// rows per sequence) took 1.72 ms with 128-row shared tiles, 1.84 ms with
// 64-row ones and 3.76 ms with 16-row register tiles (before the
// transposed-score fold), 0.80 ms on the wide kernel.
int mq_variant(int S, int T, int G) {
  const long long rows = (long long)((T + S - 1) / std::max(S, 1)) * G;
  const int v = rows <= 16 ? 0 : rows <= 32 ? 1 : rows <= 64 ? 2 : 3;
  return std::min(v, PDA_MQ_MAX_VARIANT);
}

int mq_tile_queries(int variant, int G) { return (16 << variant) / G; }

bool mq_is_shared(int variant) { return variant >= 2; }

// Dynamic LDS of a register-kernel launch with `waves` waves (two per KV head
// of its group): the state one wave of each pair hands to the other.
size_t mq_dyn_lds(int variant, int waves) {
  if (mq_is_shared(variant)) return 0;
  const int NT = variant + 1;
  return (size_t)(waves / 2) * NT * (2 + 32) * kWave * sizeof(float);
}

// Runs of the unit stream: as many work-groups as fit on all CUs at once,
// divided by the work-groups one run has (its head groups, or its KV heads).
int mq_run_count(int G, int variant, int Hkv, bool fp8) {
  // register kernel: two waves per KV head of its head group
  const int waves = mq_is_shared(variant) ? kMqWaves : 2 * mq_head_group(Hkv);
  const int per_run = mq_is_shared(variant) ? Hkv : Hkv / mq_head_group(Hkv);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 1024 / per_run;
  MqDeviceFacts& f = g_mq_dev[dev];
  std::call_once(f.once, [&f, dev] {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    f.cus = cus;
    for (int lg = 0; lg < kMqGroups; ++lg)
      for (int v = 0; v < kMqVariants; ++v)
        for (int f8 = 0; f8 < 2; ++f8)
          for (int w = 1; w <= 2 * kMqWaves; ++w) {
            int n = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                    &n, mq_kernel_ptr(kMqGroupSizes[lg], v, f8 != 0), w * kWave,
                    mq_dyn_lds(v, w)) != hipSuccess ||
                n <= 0)
              n = 1;
            f.wg_per_cu[lg][v][f8][w] = n;
          }
  });
  return std::max(1, f.cus * f.wg_per_cu[mq_gidx(G)][variant][fp8 ? 1 : 0][waves] / per_run);
}

// The whole-tile kernel serves a register variant over an fp16 cache when the
// call has at least one (sequence, KV head) pair per CU and no context longer
// than kTileMaxTokens: every work-group then holds one tile of at most
// kTileMaxTokens / 8 tokens per wave, the hardware hands work-groups to CUs as
// they free up, and the plan, the partials and the merge are not needed.
// Longer contexts (one tile could outlast the rest of the call) and smaller
// calls keep the balanced run schedule.  Measured on MI355X (speculative
// verification, 32 x 4096, 6 queries): fp16 call 98.6 -> 89.4 us.  FP8 keeps
// the run schedule: its fold is short enough per block that the LDS reads of
// Q cost the whole-tile kernel 40%, and with Q in registers its token loop
// spilled.
bool mq_whole_tiles(int S, int Hkv, int variant, int max_tokens, int tiles_max) {
  if (mq_is_shared(variant) || max_tokens > kTileMaxTokens) return false;
  if ((long long)tiles_max * Hkv > kTileMaxGroups) return false;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) {
    MqDeviceFacts& f = g_mq_dev[dev];
    if (f.cus > 0) cus = f.cus;
  }
  return (long long)S * Hkv >= cus;
}

struct MqPlan {
  int variant = 0, Qt = 0, P = 0, n_runs = 0, hg = 0, max_tokens = 0, tiles_max = 0, n_slots = 0;
  bool whole_tiles = false;   // register variants: the whole-tile kernel alone
  size_t hdr_offset = 0, tiles_offset = 0, rec_offset = 0, lse_offset = 0, o_offset = 0,
         total = 0;
};

int mq_check(int S, int T, int Hq, int Hkv, int D, int block_size, int max_blocks,
             int partition_tokens) {
  if (S < 0 || T < 0) return fail(PDA_EINVAL, "S and num_queries must be >= 0 (got %d, %d)", S, T);
  if (S > kMqMaxSeqs)
    return fail(PDA_EUNSUPPORTED, "S = %d sequences above the maximum %d", S, kMqMaxSeqs);
  if (Hq <= 0 || Hkv <= 0) return fail(PDA_EINVAL, "Hq and Hkv must be > 0 (got %d, %d)", Hq, Hkv);
  if (Hq % Hkv != 0) return fail(PDA_EINVAL, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 6 && G != 8)
    return fail(PDA_EUNSUPPORTED, "Hq/Hkv = %d not built (1, 2, 4, 6, 8 are)", G);
  if (Hkv > kMqMaxKvHeads)
    return fail(PDA_EUNSUPPORTED, "Hkv = %d above the maximum %d", Hkv, kMqMaxKvHeads);
  if (D != kD) return fail(PDA_EUNSUPPORTED, "head dim %d not built (128 is)", D);
  if (block_size != kBS) return fail(PDA_EUNSUPPORTED, "block size %d not built (16 is)", block_size);
  if (max_blocks < 0 || max_blocks > (1 << 26))
    return fail(PDA_EINVAL, "max_blocks_per_seq must be in [0, 2^26] (got %d)", max_blocks);
  if ((long long)S * max_blocks >= (1LL << 31))
    return fail(PDA_EUNSUPPORTED, "S * max_blocks_per_seq must stay below 2^31");
  if ((long long)T + S >= (1LL << 30))
    return fail(PDA_EUNSUPPORTED, "num_queries + S must stay below 2^30");
  if (partition_tokens < 0 || partition_tokens % kBS != 0)
    return fail(PDA_EINVAL, "partition_tokens (%d) must be 0 or a positive multiple of %d",
                partition_tokens, kBS);
  if (partition_tokens > kMqMaxPartition)
    return fail(PDA_EUNSUPPORTED, "partition_tokens %d above the maximum %d", partition_tokens,
                kMqMaxPartition);
  return PDA_OK;
}

MqPlan mq_make_plan(int S, int T, int Hq, int Hkv, int max_blocks, int partition_tokens,
                    bool fp8) {
  MqPlan pl;
  const int G = Hq / Hkv;
  pl.variant = mq_variant(S, T, G);
  pl.Qt = mq_tile_queries(pl.variant, G);
  pl.P = partition_tokens > 0 ? partition_tokens : kBS;
  pl.n_runs = mq_run_count(G, pl.variant, Hkv, fp8);
  pl.hg = mq_head_group(Hkv);
  pl.max_tokens = max_blocks * kBS;
  pl.tiles_max = (T + pl.Qt - 1) / pl.Qt + S;
  pl.whole_tiles = !fp8 && mq_whole_tiles(S, Hkv, pl.variant, pl.max_tokens, pl.tiles_max);
  pl.n_slots = 2 * pl.n_runs;
  pl.hdr_offset = 0;
  pl.tiles_offset = align256(sizeof(int32_t) * kMqHdrInts);
  pl.rec_offset =
      pl.tiles_offset + align256(sizeof(int32_t) * (size_t)kMqTileArrays * pl.tiles_max);
  pl.lse_offset = pl.rec_offset + align256(sizeof(int32_t) * 4 * (size_t)pl.tiles_max);
  pl.o_offset = pl.lse_offset + align256(sizeof(float) * (size_t)pl.n_slots * pl.Qt * Hq);
  pl.total = pl.o_offset + align256(sizeof(float) * (size_t)pl.n_slots * pl.Qt * Hq * kD);
  return pl;
}

template <int Qt>
void mq_launch_aux(bool plan, const MqParams& mp, const MqPlan& pl, hipStream_t stream) {
  if (plan) {
    hipLaunchKernelGGL((mq_plan_kernel<Qt>), dim3(1), dim3(kWave), 0, stream, mp);
    return;
  }
  // one wave per kMergeRows rows of the at most n_runs - 1 cut tiles (the rows
  // of empty tiles, rare, are covered by the grid-stride loop)
  const long long merge_groups =
      ((long long)std::max(pl.n_runs - 1, 1) * Qt * mp.Hq + kMergeRows - 1) / kMergeRows;
  hipLaunchKernelGGL((mq_merge_kernel<Qt>),
                     dim3((unsigned)std::min<long long>((merge_groups + 3) / 4, 1 << 20)),
                     dim3(256), 0, stream, mp);
}

template <int G, int V, bool kFp8>
void mq_launch_v(const MqParams& mp, const MqPlan& pl, hipStream_t stream) {
  constexpr int Qt = (16 << V) / G;
  if constexpr (V <= 1 && !kFp8) {
    if (pl.whole_tiles) {
      hipLaunchKernelGGL((mq_tile_kernel<G, V + 1, kFp8>),
                         dim3((unsigned)((long long)pl.tiles_max * mp.Hkv)),
                         dim3(kWave * kTileParts), (unsigned)mq_tile_lds(V + 1), stream, mp);
      return;
    }
  }
  mq_launch_aux<Qt>(true, mp, pl, stream);
  if constexpr (V == 3) {
    hipLaunchKernelGGL((mq_wide_kernel<G, kFp8>), dim3((unsigned)(pl.n_runs * mp.Hkv)),
                       dim3(kMqWaves * kWave), 0, stream, mp);
  } else if constexpr (V == 2) {
    hipLaunchKernelGGL((mq_shared_kernel<G, 1, kFp8>), dim3((unsigned)(pl.n_runs * mp.Hkv)),
                       dim3(kMqWaves * kWave), 0, stream, mp);
  } else {
    hipLaunchKernelGGL((mq_reg_kernel<G, V + 1, kFp8>),
                       dim3((unsigned)(pl.n_runs * (mp.Hkv / pl.hg))),
                       dim3((unsigned)(2 * pl.hg * kWave)), (unsigned)mq_dyn_lds(V, 2 * pl.hg),
                       stream, mp);
  }
  mq_launch_aux<Qt>(false, mp, pl, stream);
}

template <int G, bool kFp8>
void mq_launch(const MqParams& mp, const MqPlan& pl, hipStream_t stream) {
  switch (pl.variant) {
    case 0: mq_launch_v<G, 0, kFp8>(mp, pl, stream); break;
    case 1: mq_launch_v<G, 1, kFp8>(mp, pl, stream); break;
    case 2: mq_launch_v<G, 2, kFp8>(mp, pl, stream); break;
    default: mq_launch_v<G, 3, kFp8>(mp, pl, stream); break;
  }
}

template <bool kFp8>
void mq_launch_f(int G, const MqParams& mp, const MqPlan& pl, hipStream_t stream) {
  switch (G) {
    case 1: mq_launch<1, kFp8>(mp, pl, stream); break;
    case 2: mq_launch<2, kFp8>(mp, pl, stream); break;
    case 4: mq_launch<4, kFp8>(mp, pl, stream); break;
    case 6: mq_launch<6, kFp8>(mp, pl, stream); break;
    default: mq_launch<8, kFp8>(mp, pl, stream); break;
  }
}

int run_multi_query(bool out_f16, void* out, float* lse_out, const void* q,
                    const int32_t* query_start, int T, const void* k_cache, const void* v_cache,
                    const int32_t* bt, int64_t bt_stride, const int32_t* ctx, int S, int Hq,
                    int Hkv, int D, int block_size, int64_t num_blocks, int max_blocks,
                    float scale, bool fp8, float k_scale, float v_scale, int causal,
                    int partition_tokens, void* workspace, size_t workspace_bytes,
                    void* stream_ptr) {
  int rc = mq_check(S, T, Hq, Hkv, D, block_size, max_blocks, partition_tokens);
  if (rc != PDA_OK) return rc;
  if (S == 0 || T == 0) return ok();
  if (!out || !q || !query_start || !k_cache || !v_cache || !bt || !ctx)
    return fail(PDA_EINVAL, "null input or output pointer");
  if (bt_stride < max_blocks)
    return fail(PDA_EINVAL, "block_table_stride (%lld) < max_blocks_per_seq (%d)",
                (long long)bt_stride, max_blocks);
  if (num_blocks <= 0) return fail(PDA_EINVAL, "num_blocks must be > 0");
  if (!finite_f32(scale) || !finite_f32(k_scale) || !finite_f32(v_scale))
    return fail(PDA_EINVAL, "scale, k_scale and v_scale must be finite");
  if (!workspace) return fail(PDA_EINVAL, "workspace is null");
  const MqPlan pl = mq_make_plan(S, T, Hq, Hkv, max_blocks, partition_tokens, fp8);
  if (workspace_bytes < pl.total)
    return fail(PDA_EINVAL, "workspace of %zu bytes is below the %zu needed", workspace_bytes,
                pl.total);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(PDA_EINVAL, "workspace must be 256-byte aligned");

  char* ws = static_cast<char*>(workspace);
  int32_t* tiles = reinterpret_cast<int32_t*>(ws + pl.tiles_offset);
  MqParams mp;
  mp.q = static_cast<const _Float16*>(q);
  mp.qs = query_start;
  mp.k = k_cache;
  mp.v = v_cache;
  mp.bt = bt;
  mp.ctx = ctx;
  mp.bt_stride = bt_stride;
  mp.num_blocks = num_blocks;
  mp.S = S;
  mp.T = T;
  mp.Hq = Hq;
  mp.Hkv = Hkv;
  mp.max_tokens = pl.max_tokens;
  mp.P = pl.P;
  mp.n_runs = pl.n_runs;
  mp.hg = pl.hg;
  mp.causal = causal ? 1 : 0;
  const float score_scale = scale * k_scale;      // k = k_scale * decoded code for FP8
  // at least the least normal float: the kernels take exp2 of -inf * qk_scale
  // as 0 (a masked score); for scale 0 the softmax stays uniform
  mp.qk_scale = std::max(std::fabs(score_scale) * kLog2e, FLT_MIN);
  mp.q_sign = std::signbit(score_scale) ? 0x80008000u : 0u;
  mp.v_scale = v_scale;
  mp.hdr = reinterpret_cast<int32_t*>(ws + pl.hdr_offset);
  mp.t_seq = tiles;
  mp.t_q0 = tiles + 1 * (size_t)pl.tiles_max;
  mp.t_nq = tiles + 2 * (size_t)pl.tiles_max;
  mp.t_base = tiles + 3 * (size_t)pl.tiles_max;
  mp.t_ntok = tiles + 4 * (size_t)pl.tiles_max;
  mp.t_ub = tiles + 5 * (size_t)pl.tiles_max;
  mp.t_rank = tiles + 6 * (size_t)pl.tiles_max;
  mp.t_fix = tiles + 7 * (size_t)pl.tiles_max;
  mp.t_rec = reinterpret_cast<int32_t*>(ws + pl.rec_offset);
  mp.tiles_max = pl.tiles_max;
  mp.ws_o = reinterpret_cast<float*>(ws + pl.o_offset);
  mp.ws_lse = reinterpret_cast<float*>(ws + pl.lse_offset);
  mp.out = out;
  mp.lse_out = lse_out;
  mp.out_f16 = out_f16 ? 1 : 0;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  if (fp8)
    mq_launch_f<true>(Hq / Hkv, mp, pl, stream);
  else
    mq_launch_f<false>(Hq / Hkv, mp, pl, stream);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PDA_EHIP, "multi-query launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int pda_multi_query_workspace_size(int S, int num_queries, int Hq, int Hkv, int D, int block_size,
                                   int max_blocks_per_seq, int partition_tokens, size_t* bytes) {
  if (!bytes) return fail(PDA_EINVAL, "bytes is null");
  int rc = mq_check(S, num_queries, Hq, Hkv, D, block_size, max_blocks_per_seq, partition_tokens);
  if (rc != PDA_OK) return rc;
  *bytes = (S == 0 || num_queries == 0)
               ? 0
               : std::max(mq_make_plan(S, num_queries, Hq, Hkv, max_blocks_per_seq,
                                       partition_tokens, false).total,
                          mq_make_plan(S, num_queries, Hq, Hkv, max_blocks_per_seq,
                                       partition_tokens, true).total);
  return ok();
}

int paged_multi_query_attn(void* out, float* lse_out, const void* q, const int32_t* query_start,
                           int num_queries, const void* k_cache, const void* v_cache,
                           const int32_t* block_table, int64_t block_table_stride,
                           const int32_t* context_lens, int S, int Hq, int Hkv, int D,
                           int block_size, int64_t num_blocks, int max_blocks_per_seq,
                           float scale, int causal, int partition_tokens, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return run_multi_query(true, out, lse_out, q, query_start, num_queries, k_cache, v_cache,
                         block_table, block_table_stride, context_lens, S, Hq, Hkv, D, block_size,
                         num_blocks, max_blocks_per_seq, scale, false, 1.0f, 1.0f, causal,
                         partition_tokens, workspace, workspace_bytes, stream);
}

int paged_multi_query_attn_partial(float* o, float* lse, const void* q,
                                   const int32_t* query_start, int num_queries,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, int64_t block_table_stride,
                                   const int32_t* context_lens, int S, int Hq, int Hkv, int D,
                                   int block_size, int64_t num_blocks, int max_blocks_per_seq,
                                   float scale, int causal, int partition_tokens, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (S > 0 && num_queries > 0 && !lse) return fail(PDA_EINVAL, "lse is null");
  return run_multi_query(false, o, lse, q, query_start, num_queries, k_cache, v_cache,
                         block_table, block_table_stride, context_lens, S, Hq, Hkv, D, block_size,
                         num_blocks, max_blocks_per_seq, scale, false, 1.0f, 1.0f, causal,
                         partition_tokens, workspace, workspace_bytes, stream);
}

int paged_multi_query_attn_fp8(void* out, float* lse_out, const void* q,
                               const int32_t* query_start, int num_queries, const void* k_cache,
                               const void* v_cache, const int32_t* block_table,
                               int64_t block_table_stride, const int32_t* context_lens, int S,
                               int Hq, int Hkv, int D, int block_size, int64_t num_blocks,
                               int max_blocks_per_seq, float scale, float k_scale, float v_scale,
                               int causal, int partition_tokens, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return run_multi_query(true, out, lse_out, q, query_start, num_queries, k_cache, v_cache,
                         block_table, block_table_stride, context_lens, S, Hq, Hkv, D, block_size,
                         num_blocks, max_blocks_per_seq, scale, true, k_scale, v_scale, causal,
                         partition_tokens, workspace, workspace_bytes, stream);
}

int paged_multi_query_attn_partial_fp8(float* o, float* lse, const void* q,
                                       const int32_t* query_start, int num_queries,
                                       const void* k_cache, const void* v_cache,
                                       const int32_t* block_table, int64_t block_table_stride,
                                       const int32_t* context_lens, int S, int Hq, int Hkv, int D,
                                       int block_size, int64_t num_blocks, int max_blocks_per_seq,
                                       float scale, float k_scale, float v_scale, int causal,
                                       int partition_tokens, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  if (S > 0 && num_queries > 0 && !lse) return fail(PDA_EINVAL, "lse is null");
  return run_multi_query(false, o, lse, q, query_start, num_queries, k_cache, v_cache,
                         block_table, block_table_stride, context_lens, S, Hq, Hkv, D, block_size,
                         num_blocks, max_blocks_per_seq, scale, true, k_scale, v_scale, causal,
                         partition_tokens, workspace, workspace_bytes, stream);
}

}  // extern "C"
