// Single-token decode attention over a paged KV cache for MI355X (gfx950).
//
// Two kernels on the caller's stream:
//
//  1. split_kernel: one wavefront per (sequence, KV head, split-K partition).
//     The wave keeps the G = Hq/Hkv query rows of its KV head in registers,
//     walks the partition's 16-token blocks through the block table, and
//     for each block issues 16-byte K and V loads (one 256-byte row of one
//     token and head is read by 16 lanes; a load instruction covers 4
//     tokens), computes the G scores of every token with packed fp16 dot
//     products accumulated in fp32, and folds them into an fp32 online
//     softmax (running max m, running sum l, rescaled accumulator).  Every
//     K/V byte is read once for all G query heads.  The result per
//     partition is a normalised partial o and its log-sum-exp.
//  2. merge_kernel: one wavefront per (sequence, query head) combines the
//     partials of all partitions by log-sum-exp into the fp16 output.
//
// The math: attention of one decode query over the whole cached K/V, which
// is memory-bound ("Why prefill and decode are opposite problems" on the
// page "The signature-dish specialist: vLLM's attention backend"); the paged
// gather through a block table ("How the backend reads the paged KV", same
// page; "Physical Memory Block Layout" on the page "Disaggregated Inference
// Architecture: Paged KV-Cache Tiering, Chunked Prefill, and Asynchronous
// Overlap"); partials over contiguous token ranges merged by the associative
// online-softmax reduction (KernelFlume paper, academ.us/article/2606.29207,
// §3.1, §3.2 and §5.1; the (m, l, O) equations of "Mathematical Formulation
// of Chunked Attention" on the disaggregated-inference page).

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "paged_attn.h"

namespace {

constexpr int kD = 128;             // head dim
constexpr int kBS = 16;             // tokens per block
constexpr int kWave = 64;
constexpr int kWavesPerWG = 4;
constexpr int kThreads = kWave * kWavesPerWG;
constexpr int kMaxPartition = 1024;  // 64 block ids: one per lane of the window
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// cross-lane helpers

template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl,
                                         0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the sum.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  x += dpp_f32<0x141>(x);  // row_half_mirror: other quad of the half row
  x += dpp_f32<0x140>(x);  // row_mirror: other half of the row
  return x;
}

__device__ __forceinline__ float xor_lanes(float x, int m) {
  return __shfl_xor(x, m, kWave);
}

// Sum / max over the four rows of the wave (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float across_rows_sum(float x) {
  x += xor_lanes(x, 16);
  x += xor_lanes(x, 32);
  return x;
}
__device__ __forceinline__ float across_rows_max(float x) {
  x = fmaxf(x, xor_lanes(x, 16));
  x = fmaxf(x, xor_lanes(x, 32));
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
  for (int m = 1; m < kWave; m <<= 1) x = fmaxf(x, xor_lanes(x, m));
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) {  // v_exp_f32; exp2(-inf) = 0
  return __builtin_amdgcn_exp2f(x);
}

// ---------------------------------------------------------------------------
// split-K partial kernel

struct SplitParams {
  const _Float16* q;        // [B, Hq, D]
  const _Float16* k;        // [num_blocks, 16, Hkv, D]
  const _Float16* v;
  const int32_t* bt;        // [B, bt_stride]
  const int32_t* ctx;       // [B]
  long long bt_stride;
  long long n_units;        // B * max_parts * Hkv
  long long num_blocks;     // pool rows; block ids are clamped into [0, num_blocks)
  int max_tokens;           // max_blocks_per_seq * 16; longer contexts are clamped
  int B, Hq, Hkv;
  int P;                    // partition length, tokens
  int max_parts;
  float qk_scale;           // scale * log2(e): scores in base-2 units
  float* ws_o;              // [B, max_parts, Hq, D]
  float* ws_lse;            // [B, max_parts, Hq], natural log
};

template <int G>
struct WaveState {
  float m[G];               // running max, base-2 units; uniform over the wave
  float l[G];               // running sum over this lane's row of tokens
  float acc[G][8];          // running output of d = 8*ds .. 8*ds+7, this row
};

// Fold one 16-token block into the running state.  Lane (tg, ds) holds, for
// i = 0..3, token 4i+tg of the block, dims 8ds..8ds+7, of K (kr) and V (vr).
// kMasked: only tokens < nvalid of this block exist.
template <int G, bool kMasked>
__device__ __forceinline__ void fold_block(WaveState<G>& st, const u32x4 (&qv)[G],
                                           const u32x4 (&kr)[4], const u32x4 (&vr)[4],
                                           float qk_scale, int tg, int nvalid) {
  float s[G][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half2_t* kh = reinterpret_cast<const half2_t*>(&kr[i]);
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const half2_t* qh = reinterpret_cast<const half2_t*>(&qv[j]);
      float a = 0.0f;
#pragma unroll
      for (int c = 0; c < 4; ++c) a = __builtin_amdgcn_fdot2(qh[c], kh[c], a, false);
      s[j][i] = row16_sum(a) * qk_scale;
    }
  }
  bool valid[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) valid[i] = !kMasked || (4 * i + tg < nvalid);
  if (kMasked) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < G; ++j) s[j][i] = valid[i] ? s[j][i] : -INFINITY;
  }

  // online softmax: s becomes p = exp2(s - m_new); acc and l are rescaled
#pragma unroll
  for (int j = 0; j < G; ++j) {
    float mx = fmaxf(fmaxf(s[j][0], s[j][1]), fmaxf(s[j][2], s[j][3]));
    mx = across_rows_max(mx);
    const float m_new = fmaxf(st.m[j], mx);      // finite: a block has >= 1 token
    const float alpha = fast_exp2(st.m[j] - m_new);
    st.m[j] = m_new;
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[j][i] = fast_exp2(s[j][i] - m_new);
      psum += s[j][i];
    }
    st.l[j] = st.l[j] * alpha + psum;
#pragma unroll
    for (int e = 0; e < 8; ++e) st.acc[j][e] *= alpha;
  }

  // acc += p V; a token that does not exist contributes an exact zero row
  // (selected, so a NaN in an unused slot cannot leak through 0 * NaN)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const _Float16* vh = reinterpret_cast<const _Float16*>(&vr[i]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = static_cast<float>(vh[e]);
      if (kMasked) x = valid[i] ? x : 0.0f;
#pragma unroll
      for (int j = 0; j < G; ++j) st.acc[j][e] = fmaf(s[j][i], x, st.acc[j][e]);
    }
  }
}

template <int G>
__global__ __launch_bounds__(kThreads) void split_kernel(SplitParams p) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const long long unit = (long long)blockIdx.x * kWavesPerWG + wave;
  if (unit >= p.n_units) return;
  const int g = (int)(unit % p.Hkv);
  const long long rest = unit / p.Hkv;
  const int part = (int)(rest % p.max_parts);
  const int b = (int)(rest / p.max_parts);
  const int n = min(max(p.ctx[b], 0), p.max_tokens);
  const int start = part * p.P;
  if (start >= n) return;                        // empty partition: nothing to write
  const int ntok = min(p.P, n - start);
  const int nblk = (ntok + kBS - 1) / kBS;       // <= 64
  const int tg = lane >> 4;                      // token within a group of 4
  const int ds = lane & 15;                      // 16-byte slice of the 256-byte row

  // Block-table window of the partition: lane i holds the id of block i.
  const int32_t* bt_row = p.bt + (long long)b * p.bt_stride + start / kBS;
  const int my_block = lane < nblk ? bt_row[lane] : 0;

  u32x4 qv[G];
  const _Float16* qrow = p.q + ((long long)b * p.Hq + (long long)g * G) * kD + ds * 8;
#pragma unroll
  for (int j = 0; j < G; ++j) qv[j] = *reinterpret_cast<const u32x4*>(qrow + j * kD);

  const int row_stride = p.Hkv * kD;             // elements between tokens in a block
  const long long block_stride = (long long)kBS * row_stride;
  const int lane_off = (tg * p.Hkv + g) * kD + ds * 8;
  const _Float16* kbase = p.k + lane_off;
  const _Float16* vbase = p.v + lane_off;

  auto load = [&](int kb, u32x4 (&kr)[4], u32x4 (&vr)[4]) {
    // ids outside the pool are clamped: a broken table gives wrong numbers, not a fault
    const unsigned raw = (unsigned)__builtin_amdgcn_readlane(my_block, kb);
    const long long blk = raw < (unsigned long long)p.num_blocks ? (long long)raw : 0;
    const _Float16* kp = kbase + blk * block_stride;
    const _Float16* vp = vbase + blk * block_stride;
#pragma unroll
    for (int i = 0; i < 4; ++i) kr[i] = *reinterpret_cast<const u32x4*>(kp + i * 4 * row_stride);
#pragma unroll
    for (int i = 0; i < 4; ++i) vr[i] = *reinterpret_cast<const u32x4*>(vp + i * 4 * row_stride);
  };

  WaveState<G> st;
#pragma unroll
  for (int j = 0; j < G; ++j) {
    st.m[j] = -INFINITY;
    st.l[j] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) st.acc[j][e] = 0.0f;
  }

  const int last_valid = ntok - (nblk - 1) * kBS;  // 1..16 tokens in the last block
  auto fold_last = [&](const u32x4 (&kr)[4], const u32x4 (&vr)[4]) {
    if (last_valid == kBS)
      fold_block<G, false>(st, qv, kr, vr, p.qk_scale, tg, kBS);
    else
      fold_block<G, true>(st, qv, kr, vr, p.qk_scale, tg, last_valid);
  };

  // Two register buffers: the next block's loads are in flight while the
  // current block is folded.
  u32x4 ka[4], va[4], kb_[4], vb[4];
  load(0, ka, va);
  int blk = 0;
  while (true) {
    if (blk + 1 < nblk) load(blk + 1, kb_, vb);
    if (blk == nblk - 1) { fold_last(ka, va); break; }
    fold_block<G, false>(st, qv, ka, va, p.qk_scale, tg, kBS);
    ++blk;
    if (blk + 1 < nblk) load(blk + 1, ka, va);
    if (blk == nblk - 1) { fold_last(kb_, vb); break; }
    fold_block<G, false>(st, qv, kb_, vb, p.qk_scale, tg, kBS);
    ++blk;
  }

  // Combine the four token rows, normalise, write the partial.
  const long long slot = ((long long)b * p.max_parts + part) * p.Hq + (long long)g * G;
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float l = across_rows_sum(st.l[j]);
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = across_rows_sum(st.acc[j][e]);
    if ((j & 3) == tg) {
      const float inv = 1.0f / l;
      float* dst = p.ws_o + (slot + j) * kD + ds * 8;
      f32x4 lo = {o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
      f32x4 hi = {o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv};
      *reinterpret_cast<f32x4*>(dst) = lo;
      *reinterpret_cast<f32x4*>(dst + 4) = hi;
      if (ds == 0) p.ws_lse[slot + j] = (st.m[j] + __builtin_log2f(l)) * kLn2;
    }
  }
}

// ---------------------------------------------------------------------------
// log-sum-exp merge

struct MergeParams {
  const float* o;          // partial r of (b, h): o + ((b*sb + r*sr) * Hq + h) * D
  const float* lse;        // lse + (b*sb + r*sr) * Hq + h
  long long sb, sr;
  const int32_t* ctx;      // non-null: sequence b has ceil(ctx[b] / P) partials
  int P;
  int max_parts;           // partials per sequence at most (with ctx)
  int R;                   // used when ctx is null
  int B, Hq;
  void* out;               // fp16 [B, Hq, D] or fp32 [B, Hq, D]
  float* lse_out;          // [B, Hq] or null
};

template <bool kOutF16>
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeParams p) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const long long unit = (long long)blockIdx.x * kWavesPerWG + wave;
  if (unit >= (long long)p.B * p.Hq) return;
  const int b = (int)(unit / p.Hq);
  const int h = (int)(unit % p.Hq);
  const int nparts =
      p.ctx ? min((max(p.ctx[b], 0) + p.P - 1) / p.P, p.max_parts) : p.R;

  const float* lse_b = p.lse + (long long)b * p.sb * p.Hq + h;
  const float* o_b = p.o + ((long long)b * p.sb * p.Hq + h) * kD + 2 * lane;
  const long long lse_step = p.sr * p.Hq;
  const long long o_step = p.sr * p.Hq * kD;

  float L = -INFINITY;
  for (int r = lane; r < nparts; r += kWave) L = fmaxf(L, lse_b[r * lse_step]);
  L = wave_max(L);

  f32x2 res = {0.0f, 0.0f};
  float lse_res = -INFINITY;
  if (L != -INFINITY) {
    float wsum = 0.0f;
    f32x2 acc = {0.0f, 0.0f};
    for (int r = 0; r < nparts; ++r) {
      const float w = fast_exp2((lse_b[r * lse_step] - L) * kLog2e);  // 0 for -inf
      const f32x2 o = *reinterpret_cast<const f32x2*>(o_b + r * o_step);
      wsum += w;
      acc.x = fmaf(w, o.x, acc.x);
      acc.y = fmaf(w, o.y, acc.y);
    }
    const float inv = 1.0f / wsum;
    res.x = acc.x * inv;
    res.y = acc.y * inv;
    lse_res = L + __builtin_logf(wsum);
  }
  const long long dst = ((long long)b * p.Hq + h) * kD + 2 * lane;
  if (kOutF16) {
    half2_t hv = {static_cast<_Float16>(res.x), static_cast<_Float16>(res.y)};
    *reinterpret_cast<half2_t*>(static_cast<_Float16*>(p.out) + dst) = hv;
  } else {
    *reinterpret_cast<f32x2*>(static_cast<float*>(p.out) + dst) = res;
  }
  if (p.lse_out && lane == 0) p.lse_out[(long long)b * p.Hq + h] = lse_res;
}

// ---------------------------------------------------------------------------
// host side

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

constexpr int kMaxDevices = 64;
std::once_flag g_cu_once[kMaxDevices];
int g_cu_count[kMaxDevices];

int cu_count(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return 256;
  std::call_once(g_cu_once[dev], [dev] {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    g_cu_count[dev] = cus;
  });
  return g_cu_count[dev];
}

int current_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  return cu_count(dev);
}

struct Plan {
  int P = 0;
  int max_parts = 0;
  int max_tokens = 0;
  size_t o_bytes = 0, lse_bytes = 0, o_offset = 0, lse_offset = 0, total = 0;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Partition length: the requested one, or 512 tokens shrunk (down to 128)
// until the launch has at least ~16 waves per CU of work.
int pick_partition(int B, int Hkv, int max_blocks, int requested, int cus) {
  if (requested > 0) return requested;
  const long long max_tokens = (long long)max_blocks * kBS;
  int P = 512;
  auto units = [&](int P) { return (long long)B * Hkv * ((max_tokens + P - 1) / P); };
  while (P > 128 && units(P) < 16LL * cus) P /= 2;
  return P;
}

int check_shape(int B, int Hq, int Hkv, int D, int block_size, int max_blocks, int partition_tokens) {
  if (B < 0) return fail(PDA_EINVAL, "B must be >= 0 (got %d)", B);
  if (Hq <= 0 || Hkv <= 0) return fail(PDA_EINVAL, "Hq and Hkv must be > 0 (got %d, %d)", Hq, Hkv);
  if (Hq % Hkv != 0) return fail(PDA_EINVAL, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(PDA_EUNSUPPORTED, "Hq/Hkv = %d not built (1, 2, 4, 8 are)", G);
  if (D != kD) return fail(PDA_EUNSUPPORTED, "head dim %d not built (128 is)", D);
  if (block_size != kBS) return fail(PDA_EUNSUPPORTED, "block size %d not built (16 is)", block_size);
  if (max_blocks < 0 || max_blocks > (1 << 26))
    return fail(PDA_EINVAL, "max_blocks_per_seq must be in [0, 2^26] (got %d)", max_blocks);
  if (partition_tokens < 0 || partition_tokens % kBS != 0)
    return fail(PDA_EINVAL, "partition_tokens (%d) must be 0 or a positive multiple of %d",
                partition_tokens, kBS);
  if (partition_tokens > kMaxPartition)
    return fail(PDA_EUNSUPPORTED, "partition_tokens %d above the maximum %d", partition_tokens,
                kMaxPartition);
  return PDA_OK;
}

Plan make_plan(int B, int Hq, int Hkv, int max_blocks, int partition_tokens, int cus) {
  Plan pl;
  pl.P = pick_partition(B, Hkv, max_blocks, partition_tokens, cus);
  const long long max_tokens = (long long)max_blocks * kBS;
  pl.max_tokens = (int)max_tokens;
  pl.max_parts = (int)((max_tokens + pl.P - 1) / pl.P);
  const size_t slots = (size_t)B * pl.max_parts * Hq;
  pl.o_bytes = slots * kD * sizeof(float);
  pl.lse_bytes = slots * sizeof(float);
  pl.o_offset = 0;
  pl.lse_offset = align256(pl.o_bytes);
  pl.total = pl.lse_offset + align256(pl.lse_bytes);
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

int launch_split(const void* q, const void* k_cache, const void* v_cache, const int32_t* bt,
                 long long bt_stride, const int32_t* ctx, int B, int Hq, int Hkv,
                 long long num_blocks, float scale,
                 const Plan& pl, void* workspace, hipStream_t stream) {
  SplitParams sp;
  sp.q = static_cast<const _Float16*>(q);
  sp.k = static_cast<const _Float16*>(k_cache);
  sp.v = static_cast<const _Float16*>(v_cache);
  sp.bt = bt;
  sp.ctx = ctx;
  sp.bt_stride = bt_stride;
  sp.B = B;
  sp.Hq = Hq;
  sp.Hkv = Hkv;
  sp.P = pl.P;
  sp.max_parts = pl.max_parts;
  sp.n_units = (long long)B * pl.max_parts * Hkv;
  sp.num_blocks = num_blocks;
  sp.max_tokens = pl.max_tokens;
  sp.qk_scale = scale * kLog2e;
  sp.ws_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.o_offset);
  sp.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.lse_offset);
  if (sp.n_units == 0) return PDA_OK;
  const long long grid = (sp.n_units + kWavesPerWG - 1) / kWavesPerWG;
  if (grid > 0x7fffffffLL) return fail(PDA_EUNSUPPORTED, "launch of %lld work-groups too large", grid);
  const int G = Hq / Hkv;
  switch (G) {
    case 1: hipLaunchKernelGGL(split_kernel<1>, dim3((unsigned)grid), dim3(kThreads), 0, stream, sp); break;
    case 2: hipLaunchKernelGGL(split_kernel<2>, dim3((unsigned)grid), dim3(kThreads), 0, stream, sp); break;
    case 4: hipLaunchKernelGGL(split_kernel<4>, dim3((unsigned)grid), dim3(kThreads), 0, stream, sp); break;
    case 8: hipLaunchKernelGGL(split_kernel<8>, dim3((unsigned)grid), dim3(kThreads), 0, stream, sp); break;
    default: return fail(PDA_EUNSUPPORTED, "Hq/Hkv = %d not built", G);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PDA_EHIP, "split kernel launch: %s", hipGetErrorString(e));
  return PDA_OK;
}

int launch_merge(bool out_f16, void* out, float* lse_out, const MergeParams& base, hipStream_t stream) {
  MergeParams mp = base;
  mp.out = out;
  mp.lse_out = lse_out;
  const long long units = (long long)mp.B * mp.Hq;
  if (units == 0) return PDA_OK;
  const long long grid = (units + kWavesPerWG - 1) / kWavesPerWG;
  if (out_f16)
    hipLaunchKernelGGL(merge_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0, stream, mp);
  else
    hipLaunchKernelGGL(merge_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0, stream, mp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PDA_EHIP, "merge kernel launch: %s", hipGetErrorString(e));
  return PDA_OK;
}

// Shared body of paged_decode_attn and paged_decode_attn_partial.
int run_attention(bool out_f16, void* out, float* lse_out, const void* q, const void* k_cache,
                  const void* v_cache, const int32_t* bt, int64_t bt_stride, const int32_t* ctx,
                  int B, int Hq, int Hkv, int D, int block_size, int64_t num_blocks,
                  int max_blocks, float scale, int partition_tokens, void* workspace,
                  size_t workspace_bytes, void* stream_ptr) {
  int rc = check_shape(B, Hq, Hkv, D, block_size, max_blocks, partition_tokens);
  if (rc != PDA_OK) return rc;
  if (B == 0) return ok();
  if (!out || !q || !k_cache || !v_cache || !bt || !ctx)
    return fail(PDA_EINVAL, "null input or output pointer");
  if (bt_stride < max_blocks)
    return fail(PDA_EINVAL, "block_table_stride (%lld) < max_blocks_per_seq (%d)",
                (long long)bt_stride, max_blocks);
  if (num_blocks <= 0) return fail(PDA_EINVAL, "num_blocks must be > 0");
  if (!std::isfinite(scale)) return fail(PDA_EINVAL, "scale must be finite");
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const Plan pl = make_plan(B, Hq, Hkv, max_blocks, partition_tokens, current_cu_count());
  if (pl.max_parts > 0) {
    if (!workspace) return fail(PDA_EINVAL, "workspace is null");
    if (workspace_bytes < pl.total)
      return fail(PDA_EINVAL, "workspace of %zu bytes is below the %zu needed", workspace_bytes,
                  pl.total);
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
      return fail(PDA_EINVAL, "workspace must be 256-byte aligned");
  }
  rc = debug_validate(bt, bt_stride, ctx, B, num_blocks, max_blocks, stream);
  if (rc != PDA_OK) return rc;
  rc = launch_split(q, k_cache, v_cache, bt, bt_stride, ctx, B, Hq, Hkv, num_blocks, scale, pl,
                    workspace, stream);
  if (rc != PDA_OK) return rc;
  MergeParams mp{};
  mp.o = reinterpret_cast<const float*>(static_cast<char*>(workspace) + pl.o_offset);
  mp.lse = reinterpret_cast<const float*>(static_cast<char*>(workspace) + pl.lse_offset);
  mp.sb = pl.max_parts;
  mp.sr = 1;
  mp.ctx = ctx;
  mp.P = pl.P;
  mp.max_parts = pl.max_parts;
  mp.R = 0;
  mp.B = B;
  mp.Hq = Hq;
  rc = launch_merge(out_f16, out, lse_out, mp, stream);
  if (rc != PDA_OK) return rc;
  return ok();
}

}  // namespace

extern "C" {

int pda_workspace_size(int B, int Hq, int Hkv, int D, int block_size, int max_blocks_per_seq,
                       int partition_tokens, size_t* bytes) {
  if (!bytes) return fail(PDA_EINVAL, "bytes is null");
  int rc = check_shape(B, Hq, Hkv, D, block_size, max_blocks_per_seq, partition_tokens);
  if (rc != PDA_OK) return rc;
  *bytes = make_plan(B, Hq, Hkv, max_blocks_per_seq, partition_tokens, current_cu_count()).total;
  return ok();
}

int pda_workspace_layout(int B, int Hq, int Hkv, int D, int block_size, int max_blocks_per_seq,
                         int partition_tokens, size_t* o_offset, size_t* lse_offset,
                         int* max_parts, int* partition_tokens_out) {
  if (!o_offset || !lse_offset || !max_parts || !partition_tokens_out)
    return fail(PDA_EINVAL, "null output pointer");
  int rc = check_shape(B, Hq, Hkv, D, block_size, max_blocks_per_seq, partition_tokens);
  if (rc != PDA_OK) return rc;
  const Plan pl = make_plan(B, Hq, Hkv, max_blocks_per_seq, partition_tokens, current_cu_count());
  *o_offset = pl.o_offset;
  *lse_offset = pl.lse_offset;
  *max_parts = pl.max_parts;
  *partition_tokens_out = pl.P;
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
                       scale, partition_tokens, workspace, workspace_bytes, stream);
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
                       scale, partition_tokens, workspace, workspace_bytes, stream);
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
  mp.sb = 1;
  mp.sr = B;
  mp.ctx = nullptr;
  mp.P = 1;
  mp.R = R;
  mp.B = B;
  mp.Hq = Hq;
  int rc = launch_merge(true, out, lse_out, mp, static_cast<hipStream_t>(stream));
  if (rc != PDA_OK) return rc;
  return ok();
}

const char* pda_last_error(void) { return t_last_error.c_str(); }

const char* pda_version(void) { return "paged-decode-attn gfx950 0.1"; }

}  // extern "C"
