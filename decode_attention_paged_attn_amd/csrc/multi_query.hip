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
// Work decomposition.  The queries of a sequence are cut into tiles of
// 16 / G query tokens, so that a tile's G query heads per KV head fill the 16
// rows of the MFMA tiles: row m is query m / G, head m % G.  Every tile reads
// its sequence's K/V up to the furthest position one of its queries sees, in
// units of P tokens.  A one-wave plan kernel lists the tiles, their units and
// the prefix sums of the units; the units of all tiles, in order, form one
// stream cut into n_runs equal runs (as for single-token decode), and the
// persistent grid has one work-group per (run, group of up to 4 KV heads),
// one wave per KV head.  A tile that lies inside one run writes its output
// directly; a tile cut by run boundaries writes normalised partials (slot
// w + its rank among the cut tiles, so at most 2 * n_runs slots) that the
// merge kernel combines by log-sum-exp.  Tiles that see no token at all are
// written as 0 with lse -inf by the merge kernel.
//
// Per segment a wave walks the 16-token blocks through the block table as the
// decode kernel does (the same K/V loads, QK^T and p.V MFMAs), but the
// running max and sum of the softmax are per row and live in the lanes that
// hold the row (lane group c holds rows 4c .. 4c+3), and each row has its own
// last visible token; blocks that every row sees in full skip the mask.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "paged_attn.h"
#include "pda_common.h"

namespace {

using namespace pda;

constexpr int kMqWaves = 4;           // KV heads (waves) per work-group, at most
constexpr int kMqMaxKvHeads = 8;
constexpr int kMqMaxSeqs = 8192;      // sequences per call: their tile offsets live in LDS
constexpr int kMqHdrInts = 8;         // k, U, n_runs, P, n_tiles, n_fix
constexpr int kMqTileArrays = 8;      // seq, q0, nq, base, ntok, ub, rank, fix
constexpr int kMqMaxPartition = 1 << 20;
constexpr int kMqRing = 2;            // K/V register buffers per wave (blocks in flight + 1)

struct MqParams {
  const _Float16* q;        // [T, Hq, D]
  const int32_t* qs;        // [S + 1]: queries of sequence s are rows qs[s] .. qs[s+1]-1
  const _Float16* k;        // [num_blocks, 16, Hkv, D]
  const _Float16* v;
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
  float qk_scale;           // |scale| * log2(e)
  unsigned q_sign;          // 0x80008000 to negate q (scale < 0), else 0
  int32_t* hdr;             // [kMqHdrInts]
  // per tile (tiles_max entries each)
  int32_t* t_seq;           // sequence
  int32_t* t_q0;            // first query row of the tile
  int32_t* t_nq;            // queries in the tile (1 .. 16 / G)
  int32_t* t_base;          // causal: query qi of the tile sees base + qi tokens (clamped)
  int32_t* t_ntok;          // tokens the tile reads: what its furthest query sees
  int32_t* t_ub;            // units of all earlier tiles
  int32_t* t_rank;          // rank among the tiles cut by run boundaries, else -1
  int32_t* t_fix;           // [n_fix] tiles the merge kernel writes: cut ones and empty ones
  float* ws_o;              // [2 * n_runs, 16 / G, Hq, D] normalised partials
  float* ws_lse;            // [2 * n_runs, 16 / G, Hq]
  void* out;                // [T, Hq, D] fp16, or fp32 for the partial entry point
  float* lse_out;           // [T, Hq] or null
  int out_f16;
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

template <int G>
__global__ __launch_bounds__(kWave) void mq_plan_kernel(MqParams p) {
  constexpr int Qt = 16 / G;
  __shared__ int toff[kMqMaxSeqs + 1];             // first tile of each sequence
  const int lane = threadIdx.x;

  int carry = 0;
  for (int s0 = 0; s0 < p.S; s0 += kWave) {
    const int s = s0 + lane;
    int nt = 0;
    if (s < p.S) nt = (mq_q_end(p, s) - mq_q_begin(p, s) + Qt - 1) / Qt;
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
    const int qb = mq_q_begin(p, s);
    const int nq_seq = mq_q_end(p, s) - qb;
    q0 = qb + j * Qt;
    nq = min(Qt, nq_seq - j * Qt);
    const int n = mq_seq_len(p, s);
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
      if (fix) p.t_fix[fincl - 1] = i;
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

// ---------------------------------------------------------------------------
// tile kernel

// Per-wave softmax state of one segment: rows 4c + r (r = 0..3) in lane group c.
struct MqSeg {
  float m[4];               // running max of the row (base 2)
  float lp[4];              // running sum of p of this lane's token slot
  f32x4 acc[8];             // p.V tiles: lane (c, n), tile u, reg r = row 4c + r, dim 8n + u
};

// One 16-token block starting at token t0.  rend[r]: the row's visible tokens
// end (exclusive) inside this segment; nvalid: tokens of the block before the
// segment's end.
template <bool kMasked>
__device__ __forceinline__ void mq_fold(MqSeg& st, const half8_t (&qa)[4], const u32x4 (&kr)[4],
                                        const u32x4 (&vr)[4], float* lds_p, float qk_scale,
                                        int lane, int t0, const int (&rend)[4], int nvalid) {
  const int t = lane & 15;
  const int c = lane >> 4;
  half8_t kop[4];
  k_operands<false>(kr, kop);
  f32x4 sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[i], kop[i], sc, 0, 0, 0);

  bool valid[4];
  float s[4], mb[4];
  bool grow = false;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    valid[r] = !kMasked || t0 + t < rend[r];
    s[r] = valid[r] ? sc[r] : -INFINITY;
    const float x = row16_max(s[r]);
    mb[r] = x == -INFINITY ? -INFINITY : x * qk_scale;   // a fully masked row stays -inf
    grow |= mb[r] > st.m[r];
  }
  if (__ballot(grow) != 0) {        // uniform branch: some row's running max moved
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float mn = fmaxf(st.m[r], mb[r]);
      const float a = mn == st.m[r] ? 1.0f : fast_exp2(st.m[r] - mn);   // 0 on a row's first token
      st.m[r] = mn;
      st.lp[r] *= a;
#pragma unroll
      for (int u = 0; u < 8; ++u) st.acc[u][r] *= a;
    }
  }
  float pr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    pr[r] = fast_exp2(fmaf(s[r], qk_scale, -st.m[r]));
    if (kMasked) pr[r] = valid[r] ? pr[r] : 0.0f;        // -inf - (-inf) would be NaN
    st.lp[r] += pr[r];
  }
  // P as the A operand of the p.V MFMAs through a 16x16 fp16 LDS tile laid
  // out [row][c][i] = p[row][token 4i + c]
  _Float16* tile = reinterpret_cast<_Float16*>(lds_p);
#pragma unroll
  for (int r = 0; r < 4; ++r)
    tile[(4 * c + r) * 16 + (t & 3) * 4 + (t >> 2)] = static_cast<_Float16>(pr[r]);
  const half4_t pa = *reinterpret_cast<const half4_t*>(tile + t * 16 + c * 4);
  pv_mfma<kMasked, false>(st.acc, pa, vr, c, nvalid);
}

// One wave: KV head g of tile i over tokens [tok_lo, tok_hi).
template <int G>
__device__ void mq_segment(const MqParams& p, float* lds_p, int lane, int g, int i, int tok_lo,
                           int tok_hi, bool whole, int slot) {
  constexpr int Qt = 16 / G;
  const int c = lane >> 4, t = lane & 15;
  const int s = p.t_seq[i], q0 = p.t_q0[i], nq = p.t_nq[i], base = p.t_base[i];
  const int n = mq_seq_len(p, s);

  // Q as the MFMA A operand: row t is query t / G, head g*G + t % G
  // (rows past the tile's queries load the tile's last query and are zeroed)
  half8_t qa[4];
  {
    const int qi = t / G, j = t % G;
    const int row = q0 + min(qi, nq - 1);
    const _Float16* qrow = p.q + ((long long)row * p.Hq + (long long)g * G + j) * kD;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      u32x4 x = *reinterpret_cast<const u32x4*>(qrow + KvFmt<false>::q_dim(ii, c)) ^ p.q_sign;
      if (qi >= nq) x = u32x4{0u, 0u, 0u, 0u};
      qa[ii] = __builtin_bit_cast(half8_t, x);
    }
  }
  // where each of this lane group's rows stops seeing tokens in this segment;
  // rows past the tile's queries are never stored and see everything
  int rend[4];
  int row_min = tok_hi;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int qi = (4 * c + r) / G;
    int e = tok_hi;
    if (qi < nq && p.causal) e = min(min(max(base + qi, 0), n), tok_hi);
    rend[r] = e;
    row_min = min(row_min, e);
  }
  // blocks wholly before every row's end skip the mask (uniform over the wave)
  for (int m = 16; m < kWave; m <<= 1) row_min = min(row_min, __shfl_xor(row_min, m, kWave));
  const int full_end = __builtin_amdgcn_readfirstlane(row_min);

  const unsigned row_bytes = (unsigned)(p.Hkv * kD * 2);
  const long long block_bytes = (long long)kBS * row_bytes;
  const unsigned k_lane = (unsigned)((t * p.Hkv + g) * kD * 2 + 16 * c);
  const unsigned v_lane = (unsigned)((c * p.Hkv + g) * kD * 2 + 16 * t);
  const char* kbytes = reinterpret_cast<const char*>(p.k);
  const char* vbytes = reinterpret_cast<const char*>(p.v);
  const int32_t* bt_row = p.bt + (long long)s * p.bt_stride + tok_lo / kBS;
  const int ntok = tok_hi - tok_lo;
  const int nblk = (ntok + kBS - 1) / kBS;

  MqSeg st;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    st.m[r] = -INFINITY;
    st.lp[r] = 0.0f;
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) st.acc[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  int window = lane < nblk ? bt_row[lane] : 0;
  auto block_off = [&](int kb) -> long long {
    if ((kb & 63) == 0 && kb > 0) {
      const int idx = kb + lane;
      window = idx < nblk ? bt_row[idx] : 0;
    }
    const unsigned raw = (unsigned)__builtin_amdgcn_readlane(window, kb & 63);
    const long long blk = raw < (unsigned long long)p.num_blocks ? (long long)raw : 0;
    return blk * block_bytes;
  };
  auto load = [&](long long off, u32x4 (&kr)[4], u32x4 (&vr)[4]) {
    const char* kb = kbytes + off;
    const char* vb = vbytes + off;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
      kr[ii] = *reinterpret_cast<const u32x4*>(kb + k_lane + 64 * ii);
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
      vr[ii] = *reinterpret_cast<const u32x4*>(vb + v_lane + 4 * ii * row_bytes);
  };
  auto fold = [&](const u32x4 (&kr)[4], const u32x4 (&vr)[4], int kb) {
    const int t0 = tok_lo + kb * kBS;
    if (t0 + kBS > full_end)
      mq_fold<true>(st, qa, kr, vr, lds_p, p.qk_scale, lane, t0, rend, tok_hi - t0);
    else
      mq_fold<false>(st, qa, kr, vr, lds_p, p.qk_scale, lane, t0, rend, kBS);
  };

  constexpr int NB = kMqRing;
  u32x4 kbuf[NB][4], vbuf[NB][4];
#pragma unroll
  for (int ii = 0; ii < NB - 1; ++ii)
    if (ii < nblk) load(block_off(ii), kbuf[ii], vbuf[ii]);
  for (int kb0 = 0; kb0 < nblk; kb0 += NB) {
#pragma unroll
    for (int sl = 0; sl < NB; ++sl) {
      const int cur = kb0 + sl;
      if (cur >= nblk) break;
      const int nxt = cur + NB - 1;
      if (nxt < nblk) load(block_off(nxt), kbuf[(sl + NB - 1) % NB], vbuf[(sl + NB - 1) % NB]);
      fold(kbuf[sl], vbuf[sl], cur);
    }
  }

  // epilogue: lane (c, n) holds rows 4c + r, dims 8n .. 8n+7
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float l = row16_sum(st.lp[r]);
    const int row = 4 * c + r;
    const int qi = row / G, j = row % G;
    if (qi >= nq) continue;
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const float lse = l > 0.0f ? (st.m[r] + __builtin_log2f(l)) * kLn2 : -INFINITY;
    float o[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) o[u] = st.acc[u][r] * inv;
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

template <int G>
__global__ __launch_bounds__(kWave * kMqWaves) __attribute__((amdgpu_waves_per_eu(2)))
void mq_kernel(MqParams p) {
  __shared__ float lds[kMqWaves][kBS * 16 / 2];    // one 16x16 fp16 P tile per wave
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int n_hgroups = p.Hkv / p.hg;
  const int w = blockIdx.x / n_hgroups;                  // run of the unit stream
  const int g = (blockIdx.x % n_hgroups) * p.hg + wave;  // KV head
  const int k = p.hdr[0], U = p.hdr[1], n_tiles = p.hdr[4];
  const int u_lo = w * k;
  const int u_hi = min(u_lo + k, U);
  if (u_lo >= u_hi || n_tiles <= 0) return;

  // the tile holding unit u_lo: the last tile whose first unit is <= u_lo
  int lo = 0, hi = n_tiles - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.t_ub[mid] <= u_lo) lo = mid; else hi = mid - 1;
  }
  int u = u_lo;
  for (int i = lo; i < n_tiles && u < u_hi; ++i) {
    const int before = p.t_ub[i];
    const int nu = (i + 1 < n_tiles ? p.t_ub[i + 1] : U) - before;
    const int p_lo = u - before;
    const int p_hi = min(u_hi - before, nu);
    if (p_hi <= p_lo) continue;
    const int tok_lo = p_lo * p.P;
    const int tok_hi = min(p_hi * p.P, p.t_ntok[i]);
    mq_segment<G>(p, lds[wave], lane, g, i, tok_lo, tok_hi, p_lo == 0 && p_hi == nu,
                  w + p.t_rank[i]);
    u = before + p_hi;
  }
}

// ---------------------------------------------------------------------------
// merge: tiles cut by run boundaries, and tiles that see no token

template <int G>
__global__ __launch_bounds__(256) void mq_merge_kernel(MqParams p) {
  constexpr int Qt = 16 / G;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int k = p.hdr[0], U = p.hdr[1], n_tiles = p.hdr[4], n_fix = p.hdr[5];
  for (int f = blockIdx.x; f < n_fix; f += gridDim.x) {
    const int i = p.t_fix[f];
    const int ub = p.t_ub[i];
    const int nu = (i + 1 < n_tiles ? p.t_ub[i + 1] : U) - ub;
    int nseg = 0;
    long long slot0 = 0;
    if (nu > 0) {
      const int w0 = ub / k, w1 = (ub + nu - 1) / k;
      nseg = w1 - w0 + 1;
      slot0 = (long long)w0 + p.t_rank[i];
    }
    const int q0 = p.t_q0[i], nq = p.t_nq[i];
    for (int row = wave; row < nq * p.Hq; row += 4) {
      const int qi = row / p.Hq, h = row % p.Hq;
      f32x2 res;
      float lse_res;
      merge_row(p.ws_o, p.ws_lse, slot0, 1, nseg, (long long)Qt * p.Hq, row, lane, res, lse_res);
      const long long dst = ((long long)(q0 + qi) * p.Hq + h) * kD + 2 * lane;
      if (p.out_f16) {
        half2_t hv = {static_cast<_Float16>(res.x), static_cast<_Float16>(res.y)};
        *reinterpret_cast<half2_t*>(static_cast<_Float16*>(p.out) + dst) = hv;
      } else {
        *reinterpret_cast<f32x2*>(static_cast<float*>(p.out) + dst) = res;
      }
      if (p.lse_out && lane == 0) p.lse_out[(long long)(q0 + qi) * p.Hq + h] = lse_res;
    }
  }
}

// ---------------------------------------------------------------------------
// host side

constexpr int kMaxDevices = 64;
struct MqDeviceFacts {
  std::once_flag once;
  int cus = 0;
  int wg_per_cu[4][kMqWaves + 1] = {};   // [log2 G][waves per work-group]
};
MqDeviceFacts g_mq_dev[kMaxDevices];

const void* mq_kernel_ptr(int G) {
  switch (G) {
    case 1: return reinterpret_cast<const void*>(&mq_kernel<1>);
    case 2: return reinterpret_cast<const void*>(&mq_kernel<2>);
    case 4: return reinterpret_cast<const void*>(&mq_kernel<4>);
    default: return reinterpret_cast<const void*>(&mq_kernel<8>);
  }
}

int mq_log2(int G) { return G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : 3; }

int mq_head_group(int Hkv) {
  for (int hg = kMqWaves; hg > 1; --hg)
    if (Hkv % hg == 0) return hg;
  return 1;
}

// Runs of the unit stream: as many work-groups as fit on all CUs at once,
// divided by the head groups.
int mq_run_count(int G, int Hkv) {
  const int hg = mq_head_group(Hkv);
  const int n_hgroups = Hkv / hg;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 1024 / n_hgroups;
  MqDeviceFacts& f = g_mq_dev[dev];
  std::call_once(f.once, [&f, dev] {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    f.cus = cus;
    for (int lg = 0; lg < 4; ++lg)
      for (int w = 1; w <= kMqWaves; ++w) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, mq_kernel_ptr(1 << lg), w * kWave, 0) !=
                hipSuccess ||
            n <= 0)
          n = 1;
        f.wg_per_cu[lg][w] = n;
      }
  });
  return std::max(1, f.cus * f.wg_per_cu[mq_log2(G)][hg] / n_hgroups);
}

struct MqPlan {
  int Qt = 0, P = 0, n_runs = 0, hg = 0, max_tokens = 0, tiles_max = 0, n_slots = 0;
  size_t hdr_offset = 0, tiles_offset = 0, lse_offset = 0, o_offset = 0, total = 0;
};

int mq_check(int S, int T, int Hq, int Hkv, int D, int block_size, int max_blocks,
             int partition_tokens) {
  if (S < 0 || T < 0) return fail(PDA_EINVAL, "S and num_queries must be >= 0 (got %d, %d)", S, T);
  if (S > kMqMaxSeqs)
    return fail(PDA_EUNSUPPORTED, "S = %d sequences above the maximum %d", S, kMqMaxSeqs);
  if (Hq <= 0 || Hkv <= 0) return fail(PDA_EINVAL, "Hq and Hkv must be > 0 (got %d, %d)", Hq, Hkv);
  if (Hq % Hkv != 0) return fail(PDA_EINVAL, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(PDA_EUNSUPPORTED, "Hq/Hkv = %d not built (1, 2, 4, 8 are)", G);
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

MqPlan mq_make_plan(int S, int T, int Hq, int Hkv, int max_blocks, int partition_tokens) {
  MqPlan pl;
  const int G = Hq / Hkv;
  pl.Qt = 16 / G;
  pl.P = partition_tokens > 0 ? partition_tokens : kBS;
  pl.n_runs = mq_run_count(G, Hkv);
  pl.hg = mq_head_group(Hkv);
  pl.max_tokens = max_blocks * kBS;
  pl.tiles_max = (T + pl.Qt - 1) / pl.Qt + S;
  pl.n_slots = 2 * pl.n_runs;
  pl.hdr_offset = 0;
  pl.tiles_offset = align256(sizeof(int32_t) * kMqHdrInts);
  pl.lse_offset =
      pl.tiles_offset + align256(sizeof(int32_t) * (size_t)kMqTileArrays * pl.tiles_max);
  pl.o_offset = pl.lse_offset + align256(sizeof(float) * (size_t)pl.n_slots * pl.Qt * Hq);
  pl.total = pl.o_offset + align256(sizeof(float) * (size_t)pl.n_slots * pl.Qt * Hq * kD);
  return pl;
}

template <int G>
void mq_launch(const MqParams& mp, const MqPlan& pl, hipStream_t stream) {
  hipLaunchKernelGGL((mq_plan_kernel<G>), dim3(1), dim3(kWave), 0, stream, mp);
  const dim3 grid((unsigned)(pl.n_runs * (mp.Hkv / pl.hg))), block((unsigned)(pl.hg * kWave));
  hipLaunchKernelGGL((mq_kernel<G>), grid, block, 0, stream, mp);
  hipLaunchKernelGGL((mq_merge_kernel<G>), dim3((unsigned)pl.n_runs), dim3(256), 0, stream, mp);
}

int run_multi_query(bool out_f16, void* out, float* lse_out, const void* q,
                    const int32_t* query_start, int T, const void* k_cache, const void* v_cache,
                    const int32_t* bt, int64_t bt_stride, const int32_t* ctx, int S, int Hq,
                    int Hkv, int D, int block_size, int64_t num_blocks, int max_blocks,
                    float scale, int causal, int partition_tokens, void* workspace,
                    size_t workspace_bytes, void* stream_ptr) {
  int rc = mq_check(S, T, Hq, Hkv, D, block_size, max_blocks, partition_tokens);
  if (rc != PDA_OK) return rc;
  if (S == 0 || T == 0) return ok();
  if (!out || !q || !query_start || !k_cache || !v_cache || !bt || !ctx)
    return fail(PDA_EINVAL, "null input or output pointer");
  if (bt_stride < max_blocks)
    return fail(PDA_EINVAL, "block_table_stride (%lld) < max_blocks_per_seq (%d)",
                (long long)bt_stride, max_blocks);
  if (num_blocks <= 0) return fail(PDA_EINVAL, "num_blocks must be > 0");
  if (!finite_f32(scale)) return fail(PDA_EINVAL, "scale must be finite");
  if (!workspace) return fail(PDA_EINVAL, "workspace is null");
  const MqPlan pl = mq_make_plan(S, T, Hq, Hkv, max_blocks, partition_tokens);
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
  mp.k = static_cast<const _Float16*>(k_cache);
  mp.v = static_cast<const _Float16*>(v_cache);
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
  mp.qk_scale = std::fabs(scale) * kLog2e;
  mp.q_sign = std::signbit(scale) ? 0x80008000u : 0u;
  mp.hdr = reinterpret_cast<int32_t*>(ws + pl.hdr_offset);
  mp.t_seq = tiles;
  mp.t_q0 = tiles + 1 * (size_t)pl.tiles_max;
  mp.t_nq = tiles + 2 * (size_t)pl.tiles_max;
  mp.t_base = tiles + 3 * (size_t)pl.tiles_max;
  mp.t_ntok = tiles + 4 * (size_t)pl.tiles_max;
  mp.t_ub = tiles + 5 * (size_t)pl.tiles_max;
  mp.t_rank = tiles + 6 * (size_t)pl.tiles_max;
  mp.t_fix = tiles + 7 * (size_t)pl.tiles_max;
  mp.ws_o = reinterpret_cast<float*>(ws + pl.o_offset);
  mp.ws_lse = reinterpret_cast<float*>(ws + pl.lse_offset);
  mp.out = out;
  mp.lse_out = lse_out;
  mp.out_f16 = out_f16 ? 1 : 0;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  switch (Hq / Hkv) {
    case 1: mq_launch<1>(mp, pl, stream); break;
    case 2: mq_launch<2>(mp, pl, stream); break;
    case 4: mq_launch<4>(mp, pl, stream); break;
    default: mq_launch<8>(mp, pl, stream); break;
  }
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
               : mq_make_plan(S, num_queries, Hq, Hkv, max_blocks_per_seq, partition_tokens).total;
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
                         num_blocks, max_blocks_per_seq, scale, causal, partition_tokens,
                         workspace, workspace_bytes, stream);
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
                         num_blocks, max_blocks_per_seq, scale, causal, partition_tokens,
                         workspace, workspace_bytes, stream);
}

}  // extern "C"
