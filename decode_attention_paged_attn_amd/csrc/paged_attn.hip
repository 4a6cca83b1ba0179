// Single-token decode attention over a paged KV cache for MI355X (gfx950).
//
// The math: attention of one decode query per sequence over its whole cached
// K/V, which is bound by HBM bandwidth ("Why prefill and decode are opposite
// problems" on the page "The signature-dish specialist: vLLM's attention
// backend"); K/V rows gathered through a block table ("How the backend reads
// the paged KV", same page; "Physical Memory Block Layout" on the page
// "Disaggregated Inference Architecture: Paged KV-Cache Tiering, Chunked
// Prefill, and Asynchronous Overlap"); partials over contiguous token ranges
// merged by the associative online-softmax reduction (KernelFlume paper,
// academ.us/article/2606.29207, §3.1, §3.2 and §5.1; the (m, l, O)
// equations of "Mathematical Formulation of Chunked Attention" on the
// disaggregated-inference page).
//
// Work decomposition.  Each sequence's tokens are cut into units of P tokens
// (P a multiple of the 16-token block).  The units of all sequences, taken in
// order, form one stream of U units, cut into n_runs equal contiguous runs
// [w*k, (w+1)*k) with k = ceil(U / n_runs), so every run holds the same
// amount of KV whatever the mix of context lengths.  A run covers one or a
// few consecutive token ranges ("segments") of sequences.  The persistent
// grid has one work-group per (run, head group): a work-group of hg waves
// handles KV heads [h*hg, (h+1)*hg) of its run, one wave per head, and the
// work-groups of one run are adjacent in dispatch order, so the waves that
// read one 16-token block (all KV heads of a block are one contiguous frame)
// run at about the same time.
//
// Per segment, a wave keeps the G = Hq/Hkv query rows of its KV head as MFMA
// operands and walks the blocks through the block table:
//   * K: per block, 4 loads of 16 bytes per lane (each load instruction reads
//     64 contiguous bytes of all 16 token rows); QK^T of the 16 tokens and G
//     heads is 4 v_mfma_f32_16x16x32_f16 (fp16 products, fp32 sums);
//   * softmax: fp32 online softmax with a running max per head; scores are in
//     base-2 units (the scale is folded with log2(e)); p is rounded to fp16
//     and reaches the A-operand layout of the PV product through a 16x16 LDS
//     tile;
//   * V: per block, 4 loads of 16 bytes per lane (each load instruction reads
//     4 whole 256-byte token rows); p.V is 8 v_mfma_f32_16x16x16_f16 whose B
//     operands are byte permutes of the lane's own V loads (fp32 sums).
// A segment that is a whole sequence writes the final output; otherwise its
// normalised partial and log-sum-exp go to workspace slot w + b, and the
// merge kernel combines the slots of each (sequence, query head).

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "paged_attn.h"
#include "pda_common.h"

namespace pda {

thread_local std::string t_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  t_last_error = buf;
  return code;
}

int ok() {
  t_last_error.clear();
  return PDA_OK;
}

}  // namespace pda

// Fixed device scratch of paged_decode_attn_noalloc (see below).
static __device__ __align__(256) unsigned char scratch[PDA_NOALLOC_SCRATCH_BYTES];

namespace {

using namespace pda;

constexpr int kMaxKvHeads = 64;       // one wave per KV head, head groups per work-group
// KV heads (waves) of one work-group at most: 4 over fp16, whose kernel runs
// one wave per SIMD (1, 2, 4 and 8 measured; 4 best); over FP8 8 where a
// context may exceed kLongTokens, else 4 (split kernel, 8 against 4: agentic
// batch 396.2 -> 385.1 us, ragged 1684 -> 1665 us, but Llama 4K 83.4 -> 84.9 us)
#ifndef PDA_MAX_WAVES_PER_WG_FP16
#define PDA_MAX_WAVES_PER_WG_FP16 4
#endif
#ifndef PDA_MAX_WAVES_PER_WG_FP8
#define PDA_MAX_WAVES_PER_WG_FP8 8
#endif
constexpr int max_waves_per_wg(bool fp8) {
  return fp8 ? PDA_MAX_WAVES_PER_WG_FP8 : PDA_MAX_WAVES_PER_WG_FP16;
}
constexpr int kMaxWavesPerWG = max_waves_per_wg(false) > max_waves_per_wg(true)
                                   ? max_waves_per_wg(false) : max_waves_per_wg(true);
constexpr int kLongTokens = 8192;
constexpr float kLazyMax = 8.0f;      // log2 headroom of p over a head's running max
// Occupancy target of the split kernel, held by LDS padding when its registers
// would allow more, and the depth of its ring of K/V register buffers (blocks
// in flight + 1).  Measured on MI355X, ring 3 for both: fp16 (G <= 4) runs
// best at 1 wave per SIMD (0.3-1% over 2; rings 4 and 5 equal), FP8 at 2
// (1 wave is 11% slower on the agentic batch, 3 waves 2-6% slower; rings 4
// and 6 0.7-2% slower).
#ifndef PDA_WAVES_PER_EU_FP8
#define PDA_WAVES_PER_EU_FP8 2
#endif
#ifndef PDA_RING_FP16
#define PDA_RING_FP16 3
#endif
#ifndef PDA_RING_FP8
#define PDA_RING_FP8 3
#endif
#ifndef PDA_WAVES_PER_EU_FP16
#define PDA_WAVES_PER_EU_FP16 1
#endif
constexpr int waves_per_eu(int G, bool fp8) {
  return fp8 && G <= 4 ? PDA_WAVES_PER_EU_FP8 : G <= 4 ? PDA_WAVES_PER_EU_FP16 : 2;
}
constexpr int kMaxPartition = 1 << 20;
constexpr int kHdrInts = 4;           // k, U, n_runs, P, then units_before[b]

// E4M3 code of an fp32 value: the nearest finite E4M3 value, ties to the even
// code (round to nearest even on the 3-bit mantissa), the sign of zero kept;
// NaN gives 0x7F with its sign; magnitudes at or above 448, the largest
// finite value, saturate to +-448 (a NaN written into the cache would poison
// every attention over it).  Computed exactly: every step below is a scaling
// by a power of two or a round to integer.
__device__ __forceinline__ unsigned e4m3_encode(float x) {
  const unsigned bits = __float_as_uint(x);
  const unsigned sign = (bits >> 24) & 0x80u;
  const unsigned mag = bits & 0x7FFFFFFFu;
  if (mag > 0x7F800000u) return sign | 0x7Fu;                         // NaN
  const float a = __uint_as_float(mag);
  if (a >= 448.0f) return sign | 0x7Eu;                               // saturate
  if (a < 0.015625f) return sign | (unsigned)rintf(a * 512.0f);       // m * 2^-9, m = 0 .. 8
  const int e = (int)(mag >> 23) - 127;                               // 2^e <= a < 2^(e+1)
  const unsigned q = (unsigned)rintf((ldexpf(a, -e) - 1.0f) * 8.0f);  // 0 .. 8 (8 carries)
  return sign | min(((unsigned)(e + 7) << 3) + q, 0x7Eu);
}

// ---------------------------------------------------------------------------
// split kernel

struct SplitParams {
  const _Float16* q;        // [B, Hq, D]
  const void* k;            // [num_blocks, 16, Hkv, D] fp16, or FP8 E4M3 codes
  const void* v;
  const int32_t* bt;        // [B, bt_stride]
  const int32_t* ctx;       // [B]
  long long bt_stride;
  long long num_blocks;     // block ids are clamped into [0, num_blocks)
  int B, Hq, Hkv;
  int max_tokens;           // max_blocks_per_seq * 16; longer contexts are clamped
  int P;                    // unit length in tokens
  int n_runs;               // runs of the unit stream (one per work-group and head group)
  int hg;                   // KV heads (waves) per work-group; Hkv / hg head groups
  float qk_scale;           // |scale| * log2(e): scores in base-2 units
  unsigned q_sign;          // 0x80008000 to negate q (scale < 0), else 0
  float v_scale;            // multiplies the output (FP8 V scale; 1 for fp16)
  float* ws_o;              // [n_runs + B, Hq, D] normalised partials
  float* ws_lse;            // [n_runs + B, Hq] natural-log lse of each partial
  int32_t* ws_hdr;          // [4 + B]: k, U, n_runs, P, units before sequence b
  void* out;                // final output of whole-sequence segments
  float* lse_out;           // may be null
  int out_f16;              // out is fp16 (else fp32)
  // fused append: the newest token's K/V rows [B, Hkv, D] fp16, or null; an
  // FP8 cache stores e4m3_encode(x * inv) with these reciprocals of its scales
  const _Float16* k_new;
  const _Float16* v_new;
  float k_inv, v_inv;
};

__device__ __forceinline__ int seq_len(const SplitParams& p, int b) {
  return min(max(p.ctx[b], 0), p.max_tokens);
}

// Per-wave state of one segment for KV head g and its G query heads.
template <int G>
struct Seg {
  float m[G];               // running max per head (base 2), uniform
  float lp[4];              // running sum of p of this lane's token slot, heads 4c+r
  f32x4 acc[8];             // PV MFMA tiles: lane (c, n), tile u, reg r = head 4c+r, dim 8n+u
};

template <int G, bool kMasked, bool kFp8>
__device__ __forceinline__ void fold_block(Seg<G>& st, const half8_t (&qa)[4],
                                           const u32x4 (&kr)[KvFmt<kFp8>::kKLoads],
                                           const typename KvFmt<kFp8>::VRow (&vr)[4], float* lds_p,
                                           float qk_scale, int lane, int nvalid) {
  const int t = lane & 15;        // MFMA column: token of the block
  const int c = lane >> 4;        // MFMA row group: heads 4c .. 4c+3
  const int tg = lane >> 4;       // V layout: token row 4i + tg

  // K as MFMA B operands: lane (c, t) holds token t, dims KvFmt::q_dim(i, c) + 0..7
  half8_t kop[4];
  k_operands<kFp8>(kr, kop);

  // scores: D[head][token] = sum_d q[head][d] k[token][d]
  f32x4 sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[i], kop[i], sc, 0, 0, 0);
  constexpr int kR = G < 4 ? G : 4;   // score registers that hold real heads
  const bool tok_valid = !kMasked || t < nvalid;
  float s[kR];                        // raw q.k; the scale is applied inside the exponent
#pragma unroll
  for (int r = 0; r < kR; ++r) s[r] = tok_valid ? sc[r] : -INFINITY;

  // Lazy reference max: the running max m of a head moves only when one of
  // its scores (base-2 units) exceeds m by more than kLazyMax, so p stays
  // below 2^kLazyMax; only then is the exact block max taken (a DPP row
  // reduction).  The first block always takes it (m = -inf).  Lanes of rows
  // >= G (zero q rows) take no part.
  float ts[kR];
  bool over = false;
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    float m = st.m[r];
#pragma unroll
    for (int cc = 1; cc * 4 + r < G; ++cc) m = c == cc ? st.m[cc * 4 + r] : m;
    ts[r] = s[r] * qk_scale;          // NaN for a masked token when scale' = 0: never "over"
    over |= 4 * c + r < G && ts[r] > m + kLazyMax;
  }
  if (__ballot(over) != 0) {        // uniform branch: the running max moves
    // block max of every head (base-2 units), uniform over the wave
    float mb[G];
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const float x = row16_max(s[r]);
#pragma unroll
      for (int cc = 0; cc * 4 + r < G; ++cc) mb[cc * 4 + r] = uniform_f32(x, 16 * cc) * qk_scale;
    }
    float alpha[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float mn = fmaxf(st.m[j], mb[j]);
      alpha[j] = mn == st.m[j] ? 1.0f : fast_exp2(st.m[j] - mn);   // 0 on the first block
      st.m[j] = mn;
    }
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      float a = alpha[r];
#pragma unroll
      for (int cc = 1; cc * 4 + r < G; ++cc) a = c == cc ? alpha[cc * 4 + r] : a;
      st.lp[r] *= a;
    }
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      float a = alpha[r];
#pragma unroll
      for (int cc = 1; cc * 4 + r < G; ++cc) a = c == cc ? alpha[cc * 4 + r] : a;
#pragma unroll
      for (int u = 0; u < 8; ++u) st.acc[u][r] *= a;
    }
  }

  // p = exp2(scale' * s - m); lane (c, t) owns p of heads 4c + r for token t.
  // A token past the end gets p = 0 by select (scale' may be 0, and -inf * 0
  // would be NaN).
  float pr[kR];
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    float m = st.m[r];
#pragma unroll
    for (int cc = 1; cc * 4 + r < G; ++cc) m = c == cc ? st.m[cc * 4 + r] : m;
    pr[r] = fast_exp2(ts[r] - m);
    if (kMasked) pr[r] = tok_valid ? pr[r] : 0.0f;
    st.lp[r] += pr[r];
  }
  // P as the A operand of the PV MFMAs (16x16x16, fp16): lane (c, m) holds
  // p[head m][tokens c, 4+c, 8+c, 12+c].  It goes through a 16x16 fp16 LDS tile
  // laid out [head][c][i] = p[head][4i + c]; p is rounded to fp16 for the product.
  {
    _Float16* tile = reinterpret_cast<_Float16*>(lds_p);
    if (4 * c < G) {
#pragma unroll
      for (int r = 0; r < kR; ++r)
        tile[(4 * c + r) * 16 + (t & 3) * 4 + (t >> 2)] = static_cast<_Float16>(pr[r]);
    }
  }
  half4_t pa = {0, 0, 0, 0};
  if (t < G) pa = *reinterpret_cast<const half4_t*>(reinterpret_cast<const _Float16*>(lds_p) +
                                                   t * 16 + c * 4);

  pv_mfma<kMasked, kFp8>(st.acc, pa, vr, tg, nvalid);
}

// One wave: KV head g of sequence b over tokens [tok_lo, tok_hi).
// Forced inline: a call would pass the parameters through the stack.
template <int G, bool kFp8, bool kAppend>
__device__ __forceinline__ void run_segment(const SplitParams& p, float* lds_p, int lane, int g,
                                            int b, int tok_lo, int tok_hi, bool whole, int slot) {
  const int c = lane >> 4, t = lane & 15;
  const int tg = lane >> 4, ds = lane & 15;

  using Fmt = KvFmt<kFp8>;
  // Q rows as the MFMA A operand: lane (c, t) holds head t, dims Fmt::q_dim(i, c) + 0..7
  half8_t qa[4];
  {
    const _Float16* qrow = p.q + ((long long)b * p.Hq + (long long)g * G + t) * kD;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (t < G)
        qa[i] = __builtin_bit_cast(
            half8_t, *reinterpret_cast<const u32x4*>(qrow + Fmt::q_dim(i, c)) ^ p.q_sign);
      else
        qa[i] = __builtin_bit_cast(half8_t, u32x4{0u, 0u, 0u, 0u});
    }
  }

  constexpr int E = Fmt::kElemBytes;
  const unsigned row_bytes = (unsigned)(p.Hkv * kD * E);   // between tokens of a block
  const long long block_bytes = (long long)kBS * row_bytes;
  // byte offsets inside a block (the block base is uniform): K lane (c, t)
  // reads token t, 16 bytes at 16c + 64i; V lane (tg, ds) reads token 4i + tg,
  // dims 8ds .. 8ds+7
  const unsigned k_lane = (unsigned)((t * p.Hkv + g) * kD * E + 16 * c);
  const unsigned v_lane = (unsigned)((tg * p.Hkv + g) * kD * E + 8 * E * ds);
  const char* kbytes = reinterpret_cast<const char*>(p.k);
  const char* vbytes = reinterpret_cast<const char*>(p.v);
  const int32_t* bt_row = p.bt + (long long)b * p.bt_stride + tok_lo / kBS;
  const int ntok = tok_hi - tok_lo;
  const int nblk = (ntok + kBS - 1) / kBS;
  const int last_valid = ntok - (nblk - 1) * kBS;

  Seg<G> st;
#pragma unroll
  for (int j = 0; j < G; ++j) st.m[j] = -INFINITY;
#pragma unroll
  for (int u = 0; u < 8; ++u) st.acc[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int r = 0; r < 4; ++r) st.lp[r] = 0.0f;

  // Block ids are uniform: each is one scalar load (the table is read-only
  // here), which the K/V loads in flight never have to wait for.
  ConstI32* bt_s = (ConstI32*)bt_row;
  auto block_off = [&](int raw_id) -> long long {
    // ids outside the pool are clamped: a broken table gives wrong numbers, not a fault
    const unsigned raw = (unsigned)raw_id;
    const long long blk = raw < (unsigned long long)p.num_blocks ? (long long)raw : 0;
    return blk * block_bytes;
  };
  // K/V are read once per call: streaming V non-temporally keeps it from
  // displacing the block table, q and the partials in the caches
  using VRow = typename Fmt::VRow;
  constexpr int KL = Fmt::kKLoads;
  // Fused append: the segment that holds the sequence's newest token writes
  // k_new / v_new into that token's cache slot and uses them in place of what
  // its own loads of the slot returned, under the conditions of
  // paged_kv_append (1 <= ctx <= max tokens, the frame inside the pool).  The
  // slot lies in the segment's last block (tok_hi == ctx), which no other
  // segment of the call reads.
  bool append_here = false;
  int slot_new = 0;
  if constexpr (kAppend) {
    if (p.k_new != nullptr) {
      const int ctx_b = p.ctx[b];
      if (ctx_b > 0 && ctx_b <= p.max_tokens && tok_hi == ctx_b) {
        const unsigned frame = (unsigned)p.bt[(long long)b * p.bt_stride + (ctx_b - 1) / kBS];
        append_here = frame < (unsigned long long)p.num_blocks;
        slot_new = (ctx_b - 1) % kBS;
      }
    }
  }
  // one block's K and V into registers; a load past the segment's end (its
  // data never used) reads a single line for the whole wave
  auto load_id = [&](int id, bool past_end, u32x4 (&kr)[KL], VRow (&vr)[4]) {
    const long long off = block_off(id);
    const char* kb = kbytes + off;
    const char* vb = vbytes + off;
    const unsigned kl = past_end ? 0u : k_lane, vl = past_end ? 0u : v_lane;
    // K: each instruction reads 64 of a token row's bytes and the next the
    // rest of the same lines, so K loads are ordinary (non-temporal ones let
    // the line go between the halves: 1.5% refetched in FP8, up to 9% slower);
    // V loads read whole lines and stream non-temporally
#pragma unroll
    for (int i = 0; i < KL; ++i) kr[i] = *reinterpret_cast<const u32x4*>(kb + kl + 64 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      vr[i] = __builtin_nontemporal_load(
          reinterpret_cast<const VRow*>(vb + vl + 4 * i * row_bytes));
  };
  auto load = [&](int kbi, u32x4 (&kr)[KL], VRow (&vr)[4]) {
    load_id(bt_s[kbi], false, kr, vr);
  };
  // the newest token's rows into the last block's registers and its cache slot
  auto append_new = [&](u32x4 (&kr)[KL], VRow (&vr)[4]) {
    const long long off = block_off(bt_s[nblk - 1]);
    char* kb = const_cast<char*>(kbytes) + off;
    char* vb = const_cast<char*>(vbytes) + off;
    const long long row = ((long long)b * p.Hkv + g) * kD;   // element index in k_new
    if (t == slot_new) {
#pragma unroll
      for (int i = 0; i < KL; ++i) {
        u32x4 x;
        if constexpr (kFp8) {                    // elements 16c + 64i .. +15 as codes
          const half8_t h0 = *reinterpret_cast<const half8_t*>(p.k_new + row + 16 * c + 64 * i);
          const half8_t h1 = *reinterpret_cast<const half8_t*>(p.k_new + row + 16 * c + 64 * i + 8);
          x = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            x[e / 4] |= e4m3_encode(static_cast<float>(h0[e]) * p.k_inv) << (8 * (e % 4));
            x[2 + e / 4] |= e4m3_encode(static_cast<float>(h1[e]) * p.k_inv) << (8 * (e % 4));
          }
        } else {
          x = *reinterpret_cast<const u32x4*>(p.k_new + row + 8 * c + 32 * i);
        }
        kr[i] = x;
        *reinterpret_cast<u32x4*>(kb + k_lane + 64 * i) = x;
      }
    }
    if (tg == (slot_new & 3)) {
      VRow x;
      if constexpr (kFp8) {                      // elements 8ds .. 8ds+7 as codes
        const half8_t h = *reinterpret_cast<const half8_t*>(p.v_new + row + 8 * ds);
        x = VRow{0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          x[e / 4] |= e4m3_encode(static_cast<float>(h[e]) * p.v_inv) << (8 * (e % 4));
      } else {
        x = *reinterpret_cast<const VRow*>(p.v_new + row + 8 * ds);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)                // a constant index keeps vr in registers
        if (r == (slot_new >> 2)) vr[r] = x;
      *reinterpret_cast<VRow*>(vb + v_lane + 4 * (slot_new >> 2) * row_bytes) = x;
    }
  };
  auto fold = [&](const u32x4 (&kr)[KL], const VRow (&vr)[4], int kb) {
    if (kb == nblk - 1 && last_valid < kBS)
      fold_block<G, true, kFp8>(st, qa, kr, vr, lds_p, p.qk_scale, lane, last_valid);
    else
      fold_block<G, false, kFp8>(st, qa, kr, vr, lds_p, p.qk_scale, lane, kBS);
  };
  auto fold_full = [&](const u32x4 (&kr)[KL], const VRow (&vr)[4]) {
    fold_block<G, false, kFp8>(st, qa, kr, vr, lds_p, p.qk_scale, lane, kBS);
  };

  // A ring of NB register buffers (block kb in buffer kb % NB): blocks kb+1 ..
  // kb+NB-1 are in flight while block kb is folded.  The main loop runs whole
  // turns of the ring with no exit inside, and every step issues its loads (a
  // step past the last block reads one line of it for the whole wave): with
  // the same loads on every path, the wait before a fold covers that block's
  // loads only, not the ones behind it.  The main loop never holds the last
  // block, the only one that may be partial, so it folds whole blocks only;
  // each turn reads the table entries of the next turn's loads up front, so no
  // load waits on its id.
  constexpr int NB = kFp8 ? PDA_RING_FP8 : PDA_RING_FP16;
  u32x4 kbuf[NB][KL];
  VRow vbuf[NB][4];
#pragma unroll
  for (int i = 0; i < NB - 1; ++i) load_id(bt_s[min(i, nblk - 1)], i >= nblk, kbuf[i], vbuf[i]);
  int kb0 = 0;
  int ids[NB];
#pragma unroll
  for (int s = 0; s < NB; ++s) ids[s] = bt_s[min(s + NB - 1, nblk - 1)];
  for (; kb0 + NB < nblk; kb0 += NB) {
    int next_ids[NB];
#pragma unroll
    for (int s = 0; s < NB; ++s) next_ids[s] = bt_s[min(kb0 + NB + s + NB - 1, nblk - 1)];
#pragma unroll
    for (int s = 0; s < NB; ++s) {
      load_id(ids[s], kb0 + s + NB - 1 >= nblk, kbuf[(s + NB - 1) % NB], vbuf[(s + NB - 1) % NB]);
      fold_full(kbuf[s], vbuf[s]);
    }
#pragma unroll
    for (int s = 0; s < NB; ++s) ids[s] = next_ids[s];
  }
  // at most NB blocks left, the first NB - 1 of them in flight
#pragma unroll
  for (int s = 0; s < NB; ++s) {
    if (kb0 + s >= nblk) break;
    if (s == NB - 1) load(nblk - 1, kbuf[s], vbuf[s]);
    if constexpr (kAppend)
      if (append_here && kb0 + s == nblk - 1) append_new(kbuf[s], vbuf[s]);
    fold(kbuf[s], vbuf[s], kb0 + s);
  }

  // epilogue: totals over token slots and token rows, normalise, store
  constexpr int kR = G < 4 ? G : 4;
  float l_tot[G];
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const float x = row16_sum(st.lp[r]);
#pragma unroll
    for (int cc = 0; cc * 4 + r < G; ++cc) l_tot[cc * 4 + r] = uniform_f32(x, 16 * cc);
  }
  // lane (c, n) holds head 4c + r, dims 8n .. 8n+7 in tiles 0..7, register r
  const int hq0 = g * G;
#pragma unroll
  for (int r = 0; r < kR; ++r) {
#pragma unroll
    for (int cc = 0; cc * 4 + r < G; ++cc) {
      if (c != cc) continue;
      const int j = cc * 4 + r;
      const float inv = p.v_scale / l_tot[j];
      const float lse = (st.m[j] + __builtin_log2f(l_tot[j])) * kLn2;
      float o[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) o[u] = st.acc[u][r] * inv;
      if (whole) {
        const long long dst = ((long long)b * p.Hq + hq0 + j) * kD + 8 * ds;
        if (p.out_f16) {
          half8_t h;
#pragma unroll
          for (int e = 0; e < 8; ++e) h[e] = static_cast<_Float16>(o[e]);
          *reinterpret_cast<half8_t*>(static_cast<_Float16*>(p.out) + dst) = h;
        } else {
          float* d = static_cast<float*>(p.out) + dst;
          *reinterpret_cast<f32x4*>(d) = f32x4{o[0], o[1], o[2], o[3]};
          *reinterpret_cast<f32x4*>(d + 4) = f32x4{o[4], o[5], o[6], o[7]};
        }
        if (p.lse_out && ds == 0) p.lse_out[(long long)b * p.Hq + hq0 + j] = lse;
      } else {
        const long long sl = (long long)slot * p.Hq + hq0 + j;
        float* d = p.ws_o + sl * kD + 8 * ds;
        *reinterpret_cast<f32x4*>(d) = f32x4{o[0], o[1], o[2], o[3]};
        *reinterpret_cast<f32x4*>(d + 4) = f32x4{o[4], o[5], o[6], o[7]};
        if (ds == 0) p.ws_lse[sl] = lse;
      }
    }
  }
}

template <int G, bool kFp8, bool kAppend = false>
__global__ __launch_bounds__(kWave * max_waves_per_wg(kFp8))
__attribute__((amdgpu_waves_per_eu(waves_per_eu(G, kFp8))))
void split_kernel(SplitParams p) {
  __shared__ float lds[max_waves_per_wg(kFp8)][kBS * 16 / 2];   // one 16x16 fp16 P tile per wave
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int n_hgroups = p.Hkv / p.hg;
  const int w = blockIdx.x / n_hgroups;                  // run of the unit stream
  const int g = (blockIdx.x % n_hgroups) * p.hg + wave;  // KV head
  const bool writer = (blockIdx.x == 0 && wave == 0);

  // units of sequence b: ceil(len / P); U = total; k = units per work-group
  int U = 0;
  for (int b0 = 0; b0 < p.B; b0 += kWave) {
    const int b = b0 + lane;
    const int nu = b < p.B ? (seq_len(p, b) + p.P - 1) / p.P : 0;
    U += __builtin_amdgcn_readfirstlane(wave_sum_i32(nu));   // equal in every lane
  }
  const int k = U > 0 ? (U + p.n_runs - 1) / p.n_runs : 1;
  const int u_lo = w * k;
  const int u_hi = min(u_lo + k, U);

  // locate the sequence holding unit u_lo; work-group 0 records the schedule
  int b_start = -1, before_start = 0, carry = 0;
  for (int b0 = 0; b0 < p.B; b0 += kWave) {
    const int b = b0 + lane;
    const int nu = b < p.B ? (seq_len(p, b) + p.P - 1) / p.P : 0;
    const int incl = carry + wave_inclusive_scan_i32(nu, lane);
    const int excl = incl - nu;
    if (writer && b < p.B) p.ws_hdr[kHdrInts + b] = excl;
    const unsigned long long hit = __ballot(b < p.B && excl <= u_lo && u_lo < incl);
    if (b_start < 0 && hit) {
      const int idx = __builtin_ctzll(hit);
      b_start = b0 + idx;
      before_start = __builtin_amdgcn_readlane(excl, idx);
    }
    carry = __builtin_amdgcn_readlane(incl, kWave - 1);
    if (b_start >= 0 && !writer) break;
  }
  if (writer && lane == 0) {
    p.ws_hdr[0] = k;
    p.ws_hdr[1] = U;
    p.ws_hdr[2] = p.n_runs;
    p.ws_hdr[3] = p.P;
  }
  if (u_lo >= u_hi || b_start < 0) return;

  float* lds_p = lds[wave];
  int u = u_lo, b = b_start, before = before_start;
  while (u < u_hi && b < p.B) {
    // uniform by construction; said so, everything derived from it (the block
    // index, the table row) stays in scalar registers
    const int n = __builtin_amdgcn_readfirstlane(seq_len(p, b));
    const int nu = (n + p.P - 1) / p.P;
    const int p_lo = u - before;
    const int p_hi = min(u_hi - before, nu);
    if (p_hi > p_lo) {
      const int tok_lo = p_lo * p.P;
      const int tok_hi = min(p_hi * p.P, n);
      run_segment<G, kFp8, kAppend>(p, lds_p, lane, g, b, tok_lo, tok_hi, p_lo == 0 && p_hi == nu,
                           w + b);
      u = before + p_hi;
    }
    before += nu;
    ++b;
  }
}

// ---------------------------------------------------------------------------
// log-sum-exp merge

struct MergeParams {
  // partial s (0 <= s < nseg) of (b, h): o + (slot * Hq + h) * D, lse + slot * Hq + h
  const float* o;
  const float* lse;
  const int32_t* hdr;      // non-null: the split kernel's schedule (slot = w0 + s + b)
  const int32_t* ctx;      // with hdr
  int max_tokens;
  int R;                   // without hdr: slot = s * B + b, nseg = R
  int B, Hq;
  void* out;               // fp16 or fp32 [B, Hq, D]
  float* lse_out;          // [B, Hq] or null
  int out_f16;
};

__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const long long unit = (long long)blockIdx.x * 4 + wave;
  if (unit >= (long long)p.B * p.Hq) return;
  const int b = (int)(unit / p.Hq);
  const int h = (int)(unit % p.Hq);

  long long slot0, slot_step;
  int nseg;
  if (p.hdr) {
    const int k = p.hdr[0], P = p.hdr[3];
    const int n = min(max(p.ctx[b], 0), p.max_tokens);
    const int nu = (n + P - 1) / P;
    const int before = p.hdr[kHdrInts + b];
    if (nu > 0) {
      const int w0 = before / k, w1 = (before + nu - 1) / k;
      nseg = w1 - w0 + 1;
      if (nseg == 1) return;                 // written by the split kernel
      slot0 = (long long)w0 + b;
    } else {
      nseg = 0;
      slot0 = 0;
    }
    slot_step = 1;
  } else {
    nseg = p.R;
    slot0 = b;
    slot_step = p.B;
  }

  f32x2 res;
  float lse_res;
  merge_row(p.o, p.lse, slot0, slot_step, nseg, p.Hq, h, lane, res, lse_res);
  const long long dst = ((long long)b * p.Hq + h) * kD + 2 * lane;
  if (p.out_f16) {
    half2_t hv = {static_cast<_Float16>(res.x), static_cast<_Float16>(res.y)};
    *reinterpret_cast<half2_t*>(static_cast<_Float16*>(p.out) + dst) = hv;
  } else {
    *reinterpret_cast<f32x2*>(static_cast<float*>(p.out) + dst) = res;
  }
  if (p.lse_out && lane == 0) p.lse_out[(long long)b * p.Hq + h] = lse_res;
}

// ---------------------------------------------------------------------------
// KV append: the newest token of each sequence into its tail slot

struct AppendParams {
  void* k;                  // [num_blocks, 16, Hkv, D] fp16 or E4M3 codes, written in place
  void* v;
  const _Float16* kn;       // [B, Hkv, D]
  const _Float16* vn;
  const int32_t* bt;
  const int32_t* ctx;       // counts the new token
  long long bt_stride;
  long long num_blocks;
  int B, Hkv;
  int max_tokens;
  float k_inv, v_inv;       // FP8: the codes are e4m3_encode(x * (1 / scale))
};


// One thread per 16-byte chunk of the Hkv * D row of K and of V.
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  const int chunks = p.Hkv * (kD / 8);
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)p.B * chunks) return;
  const int b = (int)(i / chunks);
  const int c = (int)(i % chunks);
  const int n = p.ctx[b];
  if (n <= 0 || n > p.max_tokens) return;           // nothing to append / outside the table
  const int t = n - 1;
  const unsigned frame = (unsigned)p.bt[(long long)b * p.bt_stride + t / kBS];
  if (frame >= (unsigned long long)p.num_blocks) return;
  const long long dst = ((long long)frame * kBS + t % kBS) * p.Hkv * kD + (long long)c * 8;
  const long long src = (long long)b * p.Hkv * kD + (long long)c * 8;
  *reinterpret_cast<u32x4*>(static_cast<_Float16*>(p.k) + dst) =
      *reinterpret_cast<const u32x4*>(p.kn + src);
  *reinterpret_cast<u32x4*>(static_cast<_Float16*>(p.v) + dst) =
      *reinterpret_cast<const u32x4*>(p.vn + src);
}

// FP8 pools: one thread per 8 elements (16 bytes of the fp16 row in, 8 bytes
// of E4M3 codes out) of K and of V.
__global__ __launch_bounds__(256) void append_fp8_kernel(AppendParams p) {
  const int chunks = p.Hkv * (kD / 8);
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)p.B * chunks) return;
  const int b = (int)(i / chunks);
  const int c = (int)(i % chunks);
  const int n = p.ctx[b];
  if (n <= 0 || n > p.max_tokens) return;           // nothing to append / outside the table
  const int t = n - 1;
  const unsigned frame = (unsigned)p.bt[(long long)b * p.bt_stride + t / kBS];
  if (frame >= (unsigned long long)p.num_blocks) return;
  const long long dst = ((long long)frame * kBS + t % kBS) * p.Hkv * kD + (long long)c * 8;
  const long long src = (long long)b * p.Hkv * kD + (long long)c * 8;
  const half8_t kx = *reinterpret_cast<const half8_t*>(p.kn + src);
  const half8_t vx = *reinterpret_cast<const half8_t*>(p.vn + src);
  u32x2 kc = {0u, 0u}, vc = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    kc[e / 4] |= e4m3_encode(static_cast<float>(kx[e]) * p.k_inv) << (8 * (e % 4));
    vc[e / 4] |= e4m3_encode(static_cast<float>(vx[e]) * p.v_inv) << (8 * (e % 4));
  }
  *reinterpret_cast<u32x2*>(static_cast<uint8_t*>(p.k) + dst) = kc;
  *reinterpret_cast<u32x2*>(static_cast<uint8_t*>(p.v) + dst) = vc;
}

// ---------------------------------------------------------------------------
// host side

// Per-device launch facts, filled once: CU count and how many split-kernel
// work-groups of each (G, kernel kind, waves per work-group) shape fit on a CU.
// Kernel kinds: 0 = fp16, 1 = FP8, 2 = fp16 and 3 = FP8 with the fused append.
constexpr int kMaxDevices = 64;
constexpr int kKinds = 4;
constexpr int kGroups = 5;
struct DeviceFacts {
  std::once_flag once;
  int cus = 0;
  int wg_per_cu[kGroups][kKinds][kMaxWavesPerWG + 1] = {};   // [group index][kind][waves per WG]
  int lds_pad[kGroups][kKinds][kMaxWavesPerWG + 1] = {};     // dynamic LDS bytes per launch
};
DeviceFacts g_dev[kMaxDevices];

// The query heads per KV head the split kernel is built for, and their index
// in the per-device tables.
constexpr int kGroupSizes[kGroups] = {1, 2, 4, 6, 8};
int group_index(int G) { return G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : G == 6 ? 3 : 4; }
bool group_built(int G) { return G == 1 || G == 2 || G == 4 || G == 6 || G == 8; }

int kernel_kind(bool fp8, bool append) { return (fp8 ? 1 : 0) + (append ? 2 : 0); }

const void* split_kernel_ptr(int G, int kind) {
  if (kind == 3) {
    switch (G) {
      case 1: return reinterpret_cast<const void*>(&split_kernel<1, true, true>);
      case 2: return reinterpret_cast<const void*>(&split_kernel<2, true, true>);
      case 4: return reinterpret_cast<const void*>(&split_kernel<4, true, true>);
      case 6: return reinterpret_cast<const void*>(&split_kernel<6, true, true>);
      default: return reinterpret_cast<const void*>(&split_kernel<8, true, true>);
    }
  }
  if (kind == 2) {
    switch (G) {
      case 1: return reinterpret_cast<const void*>(&split_kernel<1, false, true>);
      case 2: return reinterpret_cast<const void*>(&split_kernel<2, false, true>);
      case 4: return reinterpret_cast<const void*>(&split_kernel<4, false, true>);
      case 6: return reinterpret_cast<const void*>(&split_kernel<6, false, true>);
      default: return reinterpret_cast<const void*>(&split_kernel<8, false, true>);
    }
  }
  if (kind == 1) {
    switch (G) {
      case 1: return reinterpret_cast<const void*>(&split_kernel<1, true>);
      case 2: return reinterpret_cast<const void*>(&split_kernel<2, true>);
      case 4: return reinterpret_cast<const void*>(&split_kernel<4, true>);
      case 6: return reinterpret_cast<const void*>(&split_kernel<6, true>);
      default: return reinterpret_cast<const void*>(&split_kernel<8, true>);
    }
  }
  switch (G) {
    case 1: return reinterpret_cast<const void*>(&split_kernel<1, false>);
    case 2: return reinterpret_cast<const void*>(&split_kernel<2, false>);
    case 4: return reinterpret_cast<const void*>(&split_kernel<4, false>);
    case 6: return reinterpret_cast<const void*>(&split_kernel<6, false>);
    default: return reinterpret_cast<const void*>(&split_kernel<8, false>);
  }
}

// KV heads (waves) per work-group: 8 over FP8 when contexts may exceed
// kLongTokens and 8 divides Hkv, else the largest divisor of Hkv up to 4
// (a work-group of 5 to 7 waves would leave wave slots of its CU empty).
int head_group(int Hkv, bool fp8, int max_tokens) {
  if (fp8 && max_tokens > kLongTokens && Hkv % 8 == 0 && max_waves_per_wg(true) >= 8) return 8;
  for (int hg = std::min(4, max_waves_per_wg(fp8)); hg > 1; --hg)
    if (Hkv % hg == 0) return hg;
  return 1;
}

// Runs of the unit stream for (G, Hkv, kernel kind) on the current device: as
// many work-groups as fit on all CUs at once, divided by the head groups.
// Dynamic LDS that holds a split kernel to its measured best occupancy
// (waves_per_eu waves per SIMD) when its registers would allow more: each
// work-group takes just over 1 / (target + 1) of the CU's LDS.  0 when the
// registers already limit it or the padding would not fit.
int occupancy_pad(int G, int kind, int hg, int lds_cu, int lds_wg_max, int regs_wgs) {
  const int target = waves_per_eu(G, kind & 1) * 4 / hg;    // 4 SIMDs per CU
  if (target <= 0 || regs_wgs <= target || lds_cu <= 0) return 0;
  const int static_lds = (int)sizeof(float) * max_waves_per_wg(kind & 1) * kBS * 8;
  const int per_wg = (lds_cu / (target + 1) + 1 + 511) / 512 * 512;
  if (per_wg * target > lds_cu || per_wg > lds_wg_max) return 0;
  return std::max(0, per_wg - static_lds);
}

void device_facts(DeviceFacts& f, int dev) {
  int cus = 0, lds_cu = 0, lds_wg = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  if (hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
      hipSuccess)
    lds_cu = 0;
  if (hipDeviceGetAttribute(&lds_wg, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
      hipSuccess)
    lds_wg = 0;
  f.cus = cus;
  for (int lg = 0; lg < kGroups; ++lg)
    for (int kd = 0; kd < kKinds; ++kd)
      for (int w = 1; w <= max_waves_per_wg(kd & 1); ++w) {
        const void* fn = split_kernel_ptr(kGroupSizes[lg], kd);
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, w * kWave, 0) != hipSuccess ||
            n <= 0)
          n = 1;
        const int pad = occupancy_pad(kGroupSizes[lg], kd, w, lds_cu, lds_wg, n);
        if (pad > 0) {
          int m = 0;
          if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&m, fn, w * kWave, pad) == hipSuccess &&
              m > 0) {
            n = m;
            f.lds_pad[lg][kd][w] = pad;
          }
        }
        f.wg_per_cu[lg][kd][w] = n;
      }
}

DeviceFacts* facts() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  DeviceFacts& f = g_dev[dev];
  std::call_once(f.once, [&f, dev] { device_facts(f, dev); });
  return &f;
}

int run_count(int G, int Hkv, int kind, int hg) {
  const int n_hgroups = Hkv / hg;
  const DeviceFacts* f = facts();
  // no device: the tuned occupancy on 256 CUs keeps sizing queries usable
  if (!f) return std::max(1, 256 * 4 * waves_per_eu(G, kind & 1) / Hkv);
  return std::max(1, f->cus * f->wg_per_cu[group_index(G)][kind][hg] / n_hgroups);
}

int lds_pad(int G, int kind, int hg) {
  const DeviceFacts* f = facts();
  return f ? f->lds_pad[group_index(G)][kind][hg] : 0;
}

struct Plan {
  int P = 0;                 // unit length in tokens
  int n_runs = 0;
  int hg = 0;                // waves (KV heads) per work-group
  int max_tokens = 0;
  int n_slots = 0;
  size_t hdr_offset = 0, lse_offset = 0, o_offset = 0, total = 0;
};

int check_shape(int B, int Hq, int Hkv, int D, int block_size, int max_blocks, int partition_tokens) {
  if (B < 0) return fail(PDA_EINVAL, "B must be >= 0 (got %d)", B);
  if (Hq <= 0 || Hkv <= 0) return fail(PDA_EINVAL, "Hq and Hkv must be > 0 (got %d, %d)", Hq, Hkv);
  if (Hq % Hkv != 0) return fail(PDA_EINVAL, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  const int G = Hq / Hkv;
  if (!group_built(G))
    return fail(PDA_EUNSUPPORTED, "Hq/Hkv = %d not built (1, 2, 4, 6, 8 are)", G);
  if (Hkv > kMaxKvHeads)
    return fail(PDA_EUNSUPPORTED, "Hkv = %d above the maximum %d", Hkv, kMaxKvHeads);
  if (D != kD) return fail(PDA_EUNSUPPORTED, "head dim %d not built (128 is)", D);
  if (block_size != kBS) return fail(PDA_EUNSUPPORTED, "block size %d not built (16 is)", block_size);
  if (max_blocks < 0 || max_blocks > (1 << 26))
    return fail(PDA_EINVAL, "max_blocks_per_seq must be in [0, 2^26] (got %d)", max_blocks);
  if ((long long)B * max_blocks >= (1LL << 31))
    return fail(PDA_EUNSUPPORTED, "B * max_blocks_per_seq must stay below 2^31");
  if (partition_tokens < 0 || partition_tokens % kBS != 0)
    return fail(PDA_EINVAL, "partition_tokens (%d) must be 0 or a positive multiple of %d",
                partition_tokens, kBS);
  if (partition_tokens > kMaxPartition)
    return fail(PDA_EUNSUPPORTED, "partition_tokens %d above the maximum %d", partition_tokens,
                kMaxPartition);
  return PDA_OK;
}

Plan make_plan(int B, int Hq, int Hkv, int max_blocks, int partition_tokens, int kind) {
  Plan pl;
  pl.P = partition_tokens > 0 ? partition_tokens : kBS;
  pl.hg = head_group(Hkv, kind & 1, max_blocks * kBS);
  pl.n_runs = run_count(Hq / Hkv, Hkv, kind, pl.hg);
  pl.max_tokens = max_blocks * kBS;
  pl.n_slots = pl.n_runs + B;
  pl.hdr_offset = 0;
  pl.lse_offset = align256(sizeof(int32_t) * (kHdrInts + (size_t)B));
  pl.o_offset = pl.lse_offset + align256(sizeof(float) * (size_t)pl.n_slots * Hq);
  pl.total = pl.o_offset + align256(sizeof(float) * (size_t)pl.n_slots * Hq * kD);
  return pl;
}

int debug_validate(const int32_t* bt, long long bt_stride, const int32_t* ctx, int B,
                   long long num_blocks, int max_blocks, hipStream_t stream) {
  const char* env = getenv("PDA_DEBUG_VALIDATE");
  if (!env || env[0] == '\0' || env[0] == '0') return PDA_OK;
  std::vector<int32_t> h_ctx(B);
  if (hipMemcpyAsync(h_ctx.data(), ctx, sizeof(int32_t) * B, hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return fail(PDA_EHIP, "debug validation: copying context_lens failed");
  std::vector<int32_t> row(max_blocks > 0 ? max_blocks : 1);
  for (int b = 0; b < B; ++b) {
    const long long n = h_ctx[b];
    if (n < 0 || n > (long long)max_blocks * kBS)
      return fail(PDA_EINVAL, "debug validation: context_lens[%d] = %lld outside [0, %lld]", b, n,
                  (long long)max_blocks * kBS);
    const int nb = (int)((n + kBS - 1) / kBS);
    if (nb == 0) continue;
    if (hipMemcpy(row.data(), bt + (long long)b * bt_stride, sizeof(int32_t) * nb,
                  hipMemcpyDeviceToHost) != hipSuccess)
      return fail(PDA_EHIP, "debug validation: copying block_table failed");
    for (int i = 0; i < nb; ++i)
      if (row[i] < 0 || row[i] >= num_blocks)
        return fail(PDA_EINVAL, "debug validation: block_table[%d][%d] = %d outside [0, %lld)", b, i,
                    row[i], num_blocks);
  }
  return PDA_OK;
}

// Shared body of paged_decode_attn and paged_decode_attn_partial.
int run_attention(bool out_f16, void* out, float* lse_out, const void* q, const void* k_cache,
                  const void* v_cache, const int32_t* bt, int64_t bt_stride, const int32_t* ctx,
                  int B, int Hq, int Hkv, int D, int block_size, int64_t num_blocks,
                  int max_blocks, float scale, bool fp8, float k_scale, float v_scale,
                  int partition_tokens, void* workspace, size_t workspace_bytes,
                  void* stream_ptr, const void* k_new = nullptr, const void* v_new = nullptr) {
  int rc = check_shape(B, Hq, Hkv, D, block_size, max_blocks, partition_tokens);
  if (rc != PDA_OK) return rc;
  if (B == 0) return ok();
  if (!out || !q || !k_cache || !v_cache || !bt || !ctx)
    return fail(PDA_EINVAL, "null input or output pointer");
  if (bt_stride < max_blocks)
    return fail(PDA_EINVAL, "block_table_stride (%lld) < max_blocks_per_seq (%d)",
                (long long)bt_stride, max_blocks);
  if (num_blocks <= 0) return fail(PDA_EINVAL, "num_blocks must be > 0");
  if (!finite_f32(scale) || !finite_f32(k_scale) || !finite_f32(v_scale))
    return fail(PDA_EINVAL, "scale, k_scale and v_scale must be finite");
  if (!workspace) return fail(PDA_EINVAL, "workspace is null");
  const bool append = k_new != nullptr;
  if (append && (k_scale == 0.0f || v_scale == 0.0f))
    return fail(PDA_EINVAL, "the fused append needs non-zero k_scale and v_scale");
  const Plan pl = make_plan(B, Hq, Hkv, max_blocks, partition_tokens, kernel_kind(fp8, append));
  if (workspace_bytes < pl.total)
    return fail(PDA_EINVAL, "workspace of %zu bytes is below the %zu needed", workspace_bytes,
                pl.total);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(PDA_EINVAL, "workspace must be 256-byte aligned");
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  rc = debug_validate(bt, bt_stride, ctx, B, num_blocks, max_blocks, stream);
  if (rc != PDA_OK) return rc;

  char* ws = static_cast<char*>(workspace);
  SplitParams sp;
  sp.q = static_cast<const _Float16*>(q);
  sp.k = k_cache;
  sp.v = v_cache;
  sp.bt = bt;
  sp.ctx = ctx;
  sp.bt_stride = bt_stride;
  sp.num_blocks = num_blocks;
  sp.B = B;
  sp.Hq = Hq;
  sp.Hkv = Hkv;
  sp.max_tokens = pl.max_tokens;
  sp.P = pl.P;
  sp.n_runs = pl.n_runs;
  sp.hg = pl.hg;
  const float score_scale = scale * k_scale;      // k = k_scale * decoded code for FP8
  sp.qk_scale = std::fabs(score_scale) * kLog2e;
  sp.q_sign = std::signbit(score_scale) ? 0x80008000u : 0u;
  sp.v_scale = v_scale;
  sp.ws_o = reinterpret_cast<float*>(ws + pl.o_offset);
  sp.ws_lse = reinterpret_cast<float*>(ws + pl.lse_offset);
  sp.ws_hdr = reinterpret_cast<int32_t*>(ws + pl.hdr_offset);
  sp.out = out;
  sp.lse_out = lse_out;
  sp.out_f16 = out_f16 ? 1 : 0;
  sp.k_new = static_cast<const _Float16*>(k_new);
  sp.v_new = static_cast<const _Float16*>(v_new);
  sp.k_inv = 1.0f / k_scale;
  sp.v_inv = 1.0f / v_scale;
  const dim3 grid((unsigned)(pl.n_runs * (Hkv / pl.hg))), block((unsigned)(pl.hg * kWave));
  const unsigned pad = (unsigned)lds_pad(Hq / Hkv, kernel_kind(fp8, append), pl.hg);
  if (fp8 && append) {
    switch (Hq / Hkv) {
      case 1: hipLaunchKernelGGL((split_kernel<1, true, true>), grid, block, pad, stream, sp); break;
      case 2: hipLaunchKernelGGL((split_kernel<2, true, true>), grid, block, pad, stream, sp); break;
      case 4: hipLaunchKernelGGL((split_kernel<4, true, true>), grid, block, pad, stream, sp); break;
      case 6: hipLaunchKernelGGL((split_kernel<6, true, true>), grid, block, pad, stream, sp); break;
      default: hipLaunchKernelGGL((split_kernel<8, true, true>), grid, block, pad, stream, sp); break;
    }
  } else if (fp8) {
    switch (Hq / Hkv) {
      case 1: hipLaunchKernelGGL((split_kernel<1, true>), grid, block, pad, stream, sp); break;
      case 2: hipLaunchKernelGGL((split_kernel<2, true>), grid, block, pad, stream, sp); break;
      case 4: hipLaunchKernelGGL((split_kernel<4, true>), grid, block, pad, stream, sp); break;
      case 6: hipLaunchKernelGGL((split_kernel<6, true>), grid, block, pad, stream, sp); break;
      default: hipLaunchKernelGGL((split_kernel<8, true>), grid, block, pad, stream, sp); break;
    }
  } else if (append) {
    switch (Hq / Hkv) {
      case 1: hipLaunchKernelGGL((split_kernel<1, false, true>), grid, block, pad, stream, sp); break;
      case 2: hipLaunchKernelGGL((split_kernel<2, false, true>), grid, block, pad, stream, sp); break;
      case 4: hipLaunchKernelGGL((split_kernel<4, false, true>), grid, block, pad, stream, sp); break;
      case 6: hipLaunchKernelGGL((split_kernel<6, false, true>), grid, block, pad, stream, sp); break;
      default: hipLaunchKernelGGL((split_kernel<8, false, true>), grid, block, pad, stream, sp); break;
    }
  } else {
    switch (Hq / Hkv) {
      case 1: hipLaunchKernelGGL((split_kernel<1, false>), grid, block, pad, stream, sp); break;
      case 2: hipLaunchKernelGGL((split_kernel<2, false>), grid, block, pad, stream, sp); break;
      case 4: hipLaunchKernelGGL((split_kernel<4, false>), grid, block, pad, stream, sp); break;
      case 6: hipLaunchKernelGGL((split_kernel<6, false>), grid, block, pad, stream, sp); break;
      default: hipLaunchKernelGGL((split_kernel<8, false>), grid, block, pad, stream, sp); break;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PDA_EHIP, "split kernel launch: %s", hipGetErrorString(e));

  MergeParams mp{};
  mp.o = sp.ws_o;
  mp.lse = sp.ws_lse;
  mp.hdr = sp.ws_hdr;
  mp.ctx = ctx;
  mp.max_tokens = pl.max_tokens;
  mp.R = 0;
  mp.B = B;
  mp.Hq = Hq;
  mp.out = out;
  mp.lse_out = lse_out;
  mp.out_f16 = sp.out_f16;
  const long long units = (long long)B * Hq;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, stream, mp);
  e = hipGetLastError();
  if (e != hipSuccess) return fail(PDA_EHIP, "merge kernel launch: %s", hipGetErrorString(e));
  return ok();
}

// Shared body of paged_kv_append and paged_kv_append_fp8.
int run_append(bool fp8, void* k_cache, void* v_cache, const void* k_new, const void* v_new,
               const int32_t* block_table, int64_t block_table_stride,
               const int32_t* context_lens, int B, int Hkv, int D, int block_size,
               int64_t num_blocks, int max_blocks_per_seq, float k_scale, float v_scale,
               void* stream) {
  if (B < 0 || Hkv <= 0) return fail(PDA_EINVAL, "B must be >= 0 and Hkv > 0");
  if (D != kD) return fail(PDA_EUNSUPPORTED, "head dim %d not built (128 is)", D);
  if (block_size != kBS) return fail(PDA_EUNSUPPORTED, "block size %d not built (16 is)", block_size);
  if (max_blocks_per_seq < 0 || max_blocks_per_seq > (1 << 26))
    return fail(PDA_EINVAL, "max_blocks_per_seq must be in [0, 2^26]");
  if (fp8 && (!finite_f32(k_scale) || !finite_f32(v_scale) || k_scale == 0.0f ||
              v_scale == 0.0f))
    return fail(PDA_EINVAL, "k_scale and v_scale must be finite and non-zero");
  if (B == 0 || max_blocks_per_seq == 0) return ok();
  if (!k_cache || !v_cache || !k_new || !v_new || !block_table || !context_lens)
    return fail(PDA_EINVAL, "null pointer");
  if (block_table_stride < max_blocks_per_seq)
    return fail(PDA_EINVAL, "block_table_stride (%lld) < max_blocks_per_seq (%d)",
                (long long)block_table_stride, max_blocks_per_seq);
  if (num_blocks <= 0) return fail(PDA_EINVAL, "num_blocks must be > 0");
  AppendParams ap;
  ap.k = k_cache;
  ap.v = v_cache;
  ap.kn = static_cast<const _Float16*>(k_new);
  ap.vn = static_cast<const _Float16*>(v_new);
  ap.bt = block_table;
  ap.ctx = context_lens;
  ap.bt_stride = block_table_stride;
  ap.num_blocks = num_blocks;
  ap.B = B;
  ap.Hkv = Hkv;
  ap.max_tokens = max_blocks_per_seq * kBS;
  ap.k_inv = 1.0f / k_scale;
  ap.v_inv = 1.0f / v_scale;
  const long long threads = (long long)B * Hkv * (kD / 8);
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (fp8)
    hipLaunchKernelGGL(append_fp8_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream), ap);
  else
    hipLaunchKernelGGL(append_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream), ap);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PDA_EHIP, "append kernel launch: %s", hipGetErrorString(e));
  return ok();
}

// ---------------------------------------------------------------------------
// Fixed device scratch for paged_decode_attn_noalloc: the split-K workspace of
// a call that may not allocate.  Every device the library runs on holds its
// own copy for the life of the process.  Host code never uses the array's
// name as an address: its device address is looked up once per device.

struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// Device address of the current device's scratch (null with *err set if the
// lookup failed); looked up on the first call on each device, that device
// being current.
void* scratch_ptr(hipError_t* err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  ScratchSlot& s = g_scratch[dev];
  std::call_once(s.once, [&s] {
    void* p = nullptr;
    s.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    s.ptr = s.err == hipSuccess ? p : nullptr;
  });
  *err = s.err;
  return s.ptr;
}

}  // namespace

extern "C" {

int pda_workspace_size(int B, int Hq, int Hkv, int D, int block_size, int max_blocks_per_seq,
                       int partition_tokens, size_t* bytes) {
  if (!bytes) return fail(PDA_EINVAL, "bytes is null");
  int rc = check_shape(B, Hq, Hkv, D, block_size, max_blocks_per_seq, partition_tokens);
  if (rc != PDA_OK) return rc;
  size_t need = 0;
  for (int kind = 0; B > 0 && kind < kKinds; ++kind)   // one size serves every entry point
    need = std::max(need, make_plan(B, Hq, Hkv, max_blocks_per_seq, partition_tokens, kind).total);
  *bytes = need;
  return ok();
}

int paged_decode_attn_workspace_size(int B, int Hq, int D, int block_size,
                                     int max_blocks_per_seq, int partition_tokens,
                                     size_t* bytes) {
  if (!bytes) return fail(PDA_EINVAL, "bytes is null");
  if (Hq <= 0) return fail(PDA_EINVAL, "Hq must be > 0 (got %d)", Hq);
  // the largest need over every KV-head count the call may come with; if no
  // count is accepted, the last one's error stands
  size_t need = 0;
  int rc = PDA_EINVAL;
  bool any = false;
  for (int Hkv = 1; Hkv <= Hq; ++Hkv) {
    if (Hq % Hkv != 0) continue;
    size_t n = 0;
    rc = pda_workspace_size(B, Hq, Hkv, D, block_size, max_blocks_per_seq, partition_tokens, &n);
    if (rc == PDA_OK) {
      need = std::max(need, n);
      any = true;
    }
  }
  if (!any) return rc;
  *bytes = need;
  return ok();
}

int pda_workspace_layout(int B, int Hq, int Hkv, int D, int block_size, int max_blocks_per_seq,
                         int partition_tokens, int kv_fp8, pda_layout* layout) {
  if (!layout) return fail(PDA_EINVAL, "layout is null");
  int rc = check_shape(B, Hq, Hkv, D, block_size, max_blocks_per_seq, partition_tokens);
  if (rc != PDA_OK) return rc;
  const Plan pl = make_plan(B, Hq, Hkv, max_blocks_per_seq, partition_tokens,
                            kernel_kind(kv_fp8 != 0, false));
  layout->header_offset = pl.hdr_offset;
  layout->lse_offset = pl.lse_offset;
  layout->o_offset = pl.o_offset;
  layout->total_bytes = pl.total;
  layout->n_runs = pl.n_runs;
  layout->n_slots = pl.n_slots;
  layout->unit_tokens = pl.P;
  return ok();
}

int paged_decode_attn(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, int64_t block_table_stride,
                      const int32_t* context_lens, int B, int Hq, int Hkv, int D, int block_size,
                      int64_t num_blocks, int max_blocks_per_seq, float scale,
                      int partition_tokens, float* lse_out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return run_attention(true, out, lse_out, q, k_cache, v_cache, block_table, block_table_stride,
                       context_lens, B, Hq, Hkv, D, block_size, num_blocks, max_blocks_per_seq,
                       scale, false, 1.0f, 1.0f, partition_tokens, workspace, workspace_bytes,
                       stream);
}

int paged_decode_attn_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, int64_t block_table_stride,
                              const int32_t* context_lens, int B, int Hq, int Hkv, int D,
                              int block_size, int64_t num_blocks, int max_blocks_per_seq,
                              float scale, int partition_tokens, float* lse_out, void* stream) {
  int rc = check_shape(B, Hq, Hkv, D, block_size, max_blocks_per_seq, partition_tokens);
  if (rc != PDA_OK) return rc;
  if (B == 0) return ok();
  const Plan pl = make_plan(B, Hq, Hkv, max_blocks_per_seq, partition_tokens, kernel_kind(false, false));
  if (pl.total > (size_t)PDA_NOALLOC_SCRATCH_BYTES)
    return fail(PDA_EUNSUPPORTED,
                "this call needs %zu bytes of split-K workspace, above the %zu bytes of fixed "
                "scratch; use paged_decode_attn with a caller workspace",
                pl.total, (size_t)PDA_NOALLOC_SCRATCH_BYTES);
  hipError_t e = hipSuccess;
  void* ws = scratch_ptr(&e);
  if (!ws) return fail(PDA_EHIP, "device scratch lookup failed: %s", hipGetErrorString(e));
  return run_attention(true, out, lse_out, q, k_cache, v_cache, block_table, block_table_stride,
                       context_lens, B, Hq, Hkv, D, block_size, num_blocks, max_blocks_per_seq,
                       scale, false, 1.0f, 1.0f, partition_tokens, ws,
                       (size_t)PDA_NOALLOC_SCRATCH_BYTES, stream);
}

int paged_decode_attn_append(void* out, const void* q, const void* k_new, const void* v_new,
                             void* k_cache, void* v_cache, const int32_t* block_table,
                             int64_t block_table_stride, const int32_t* context_lens, int B,
                             int Hq, int Hkv, int D, int block_size, int64_t num_blocks,
                             int max_blocks_per_seq, float scale, int partition_tokens,
                             float* lse_out, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (B > 0 && (!k_new || !v_new)) return fail(PDA_EINVAL, "k_new or v_new is null");
  return run_attention(true, out, lse_out, q, k_cache, v_cache, block_table, block_table_stride,
                       context_lens, B, Hq, Hkv, D, block_size, num_blocks, max_blocks_per_seq,
                       scale, false, 1.0f, 1.0f, partition_tokens, workspace, workspace_bytes,
                       stream, k_new, v_new);
}

int paged_decode_attn_append_fp8(void* out, const void* q, const void* k_new, const void* v_new,
                                 void* k_cache, void* v_cache, const int32_t* block_table,
                                 int64_t block_table_stride, const int32_t* context_lens, int B,
                                 int Hq, int Hkv, int D, int block_size, int64_t num_blocks,
                                 int max_blocks_per_seq, float scale, float k_scale,
                                 float v_scale, int partition_tokens, float* lse_out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (B > 0 && (!k_new || !v_new)) return fail(PDA_EINVAL, "k_new or v_new is null");
  return run_attention(true, out, lse_out, q, k_cache, v_cache, block_table, block_table_stride,
                       context_lens, B, Hq, Hkv, D, block_size, num_blocks, max_blocks_per_seq,
                       scale, true, k_scale, v_scale, partition_tokens, workspace,
                       workspace_bytes, stream, k_new, v_new);
}

int paged_decode_attn_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, int64_t block_table_stride,
                          const int32_t* context_lens, int B, int Hq, int Hkv, int D,
                          int block_size, int64_t num_blocks, int max_blocks_per_seq, float scale,
                          float k_scale, float v_scale, int partition_tokens, float* lse_out,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return run_attention(true, out, lse_out, q, k_cache, v_cache, block_table, block_table_stride,
                       context_lens, B, Hq, Hkv, D, block_size, num_blocks, max_blocks_per_seq,
                       scale, true, k_scale, v_scale, partition_tokens, workspace,
                       workspace_bytes, stream);
}

int paged_decode_attn_partial(float* o, float* lse, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_table,
                              int64_t block_table_stride, const int32_t* context_lens, int B,
                              int Hq, int Hkv, int D, int block_size, int64_t num_blocks,
                              int max_blocks_per_seq, float scale, int partition_tokens,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (B > 0 && !lse) return fail(PDA_EINVAL, "lse is null");
  return run_attention(false, o, lse, q, k_cache, v_cache, block_table, block_table_stride,
                       context_lens, B, Hq, Hkv, D, block_size, num_blocks, max_blocks_per_seq,
                       scale, false, 1.0f, 1.0f, partition_tokens, workspace, workspace_bytes,
                       stream);
}

int paged_decode_attn_partial_fp8(float* o, float* lse, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_table,
                                  int64_t block_table_stride, const int32_t* context_lens, int B,
                                  int Hq, int Hkv, int D, int block_size, int64_t num_blocks,
                                  int max_blocks_per_seq, float scale, float k_scale,
                                  float v_scale, int partition_tokens, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (B > 0 && !lse) return fail(PDA_EINVAL, "lse is null");
  return run_attention(false, o, lse, q, k_cache, v_cache, block_table, block_table_stride,
                       context_lens, B, Hq, Hkv, D, block_size, num_blocks, max_blocks_per_seq,
                       scale, true, k_scale, v_scale, partition_tokens, workspace,
                       workspace_bytes, stream);
}

int merge_partials(void* out, float* lse_out, const float* o_parts, const float* lse_parts, int R,
                   int B, int Hq, int D, void* stream) {
  if (B < 0 || Hq <= 0) return fail(PDA_EINVAL, "B must be >= 0 and Hq > 0");
  if (R < 1) return fail(PDA_EINVAL, "R must be >= 1 (got %d)", R);
  if (D != kD) return fail(PDA_EUNSUPPORTED, "head dim %d not built (128 is)", D);
  if (B == 0) return ok();
  if (!out || !o_parts || !lse_parts) return fail(PDA_EINVAL, "null pointer");
  MergeParams mp{};
  mp.o = o_parts;
  mp.lse = lse_parts;
  mp.hdr = nullptr;
  mp.ctx = nullptr;
  mp.R = R;
  mp.B = B;
  mp.Hq = Hq;
  mp.out = out;
  mp.lse_out = lse_out;
  mp.out_f16 = 1;
  const long long units = (long long)B * Hq;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((units + 3) / 4)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), mp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PDA_EHIP, "merge kernel launch: %s", hipGetErrorString(e));
  return ok();
}

int paged_kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                    const int32_t* block_table, int64_t block_table_stride,
                    const int32_t* context_lens, int B, int Hkv, int D, int block_size,
                    int64_t num_blocks, int max_blocks_per_seq, void* stream) {
  return run_append(false, k_cache, v_cache, k_new, v_new, block_table, block_table_stride,
                    context_lens, B, Hkv, D, block_size, num_blocks, max_blocks_per_seq, 1.0f,
                    1.0f, stream);
}

int paged_kv_append_fp8(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                        const int32_t* block_table, int64_t block_table_stride,
                        const int32_t* context_lens, int B, int Hkv, int D, int block_size,
                        int64_t num_blocks, int max_blocks_per_seq, float k_scale,
                        float v_scale, void* stream) {
  return run_append(true, k_cache, v_cache, k_new, v_new, block_table, block_table_stride,
                    context_lens, B, Hkv, D, block_size, num_blocks, max_blocks_per_seq, k_scale,
                    v_scale, stream);
}

const char* pda_last_error(void) { return pda::t_last_error.c_str(); }

const char* pda_version(void) { return "paged-decode-attn gfx950 0.2"; }

}  // extern "C"
