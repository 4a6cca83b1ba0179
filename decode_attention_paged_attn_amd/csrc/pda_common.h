// Pieces shared by the paged attention kernels for gfx950 (MI355X): sizes,
// vector types, cross-lane reductions, the K/V element formats with their
// MFMA operand layouts, and the host-side error reporting of the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <type_traits>

namespace pda {

constexpr int kD = 128;               // head dim
constexpr int kBS = 16;               // tokens per block
constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// int32 in the constant address space: a load through it with a uniform
// address is a scalar load (for tables the kernel never writes)
typedef const int32_t __attribute__((address_space(4))) ConstI32;

// ---------------------------------------------------------------------------
// cross-lane helpers

template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, false));
}

// All-reduce over the 16 lanes of a DPP row: every lane of the row ends with
// the result.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  x += dpp_f32<0x141>(x);  // row_half_mirror: other quad of the half row
  x += dpp_f32<0x140>(x);  // row_mirror: other half of the row
  return x;
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f32<0xB1>(x));
  x = fmaxf(x, dpp_f32<0x4E>(x));
  x = fmaxf(x, dpp_f32<0x141>(x));
  x = fmaxf(x, dpp_f32<0x140>(x));
  return x;
}

__device__ __forceinline__ int wave_sum_i32(int x) {
  for (int m = 1; m < kWave; m <<= 1) x += __shfl_xor(x, m, kWave);
  return x;
}
__device__ __forceinline__ int wave_inclusive_scan_i32(int x, int lane) {
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(x, o, kWave);
    if (lane >= o) x += t;
  }
  return x;
}
__device__ __forceinline__ float wave_max_f32(float x) {
  for (int m = 1; m < kWave; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, kWave));
  return x;
}
__device__ __forceinline__ float wave_sum_f32(float x) {
  for (int m = 1; m < kWave; m <<= 1) x += __shfl_xor(x, m, kWave);
  return x;
}

__device__ __forceinline__ float uniform_f32(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

__device__ __forceinline__ float fast_exp2(float x) {  // v_exp_f32; exp2(-inf) = 0
  return __builtin_amdgcn_exp2f(x);
}

// ---------------------------------------------------------------------------
// K/V element storage and the MFMA operands built from it.
//
// fp16 elements are used as stored.  FP8 elements are E4M3 codes, decoded
// exactly (every E4M3 value is an fp16 value) to fp16 MFMA operands; the
// per-tensor scales are folded into the softmax scale and the output
// normalisation by the callers.
//
// Per 16-token block and KV head, lane (c, t) of a wave (c = lane >> 4,
// t = lane & 15) loads
//   * K: token t, kKLoads loads of 16 bytes at byte 16c + 64i of the row; the
//     QK^T product is 4 v_mfma_f32_16x16x32_f16 whose chunk i covers head
//     dims q_dim(i, c) + 0..7 in lane group c;
//   * V: tokens 4i + c (i = 0..3), dims 8t .. 8t+7.
template <bool kFp8>
struct KvFmt {
  static constexpr int kElemBytes = kFp8 ? 1 : 2;
  static constexpr int kKLoads = kFp8 ? 2 : 4;     // 16-byte K loads per lane per block
  using VRow = typename std::conditional<kFp8, u32x2, u32x4>::type;   // 8 V elements
  __device__ static constexpr int q_dim(int i, int c) {
    return kFp8 ? 64 * (i / 2) + 16 * c + 8 * (i % 2) : 32 * i + 8 * c;
  }
};

// The K operands of the 4 QK^T MFMAs from one block's K loads.
template <bool kFp8>
__device__ __forceinline__ void k_operands(const u32x4 (&kr)[KvFmt<kFp8>::kKLoads],
                                           half8_t (&kop)[4]) {
  if constexpr (kFp8) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const half2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(kr[j][w], 1.0f, false);
        const half2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(kr[j][w], 1.0f, true);
        half8_t& dst = kop[2 * j + w / 2];
        dst[4 * (w % 2) + 0] = lo[0];
        dst[4 * (w % 2) + 1] = lo[1];
        dst[4 * (w % 2) + 2] = hi[0];
        dst[4 * (w % 2) + 3] = hi[1];
      }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) kop[i] = __builtin_bit_cast(half8_t, kr[i]);
  }
}

// p . V as eight v_mfma_f32_16x16x16_f16 tiles.  Tile u covers head dims
// 8n + u (n = lane & 15); the contraction index 4c + i stands for token
// 4i + c, so lane (c, n) needs v[token 4i + c][8n + u], i = 0..3, which is
// element u of its own four V loads.  pa is the A operand (p of row lane & 15
// at tokens c, 4+c, 8+c, 12+c).  Tokens at or past nvalid are exact zero rows
// (selected, so a NaN in an unused slot cannot leak through 0 * NaN).
template <bool kMasked, bool kFp8>
__device__ __forceinline__ void pv_mfma(f32x4 (&acc)[8], half4_t pa,
                                        const typename KvFmt<kFp8>::VRow (&vr)[4], int c,
                                        int nvalid) {
  if constexpr (kFp8) {
    u32x2 vv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      vv[i] = (!kMasked || 4 * i + c < nvalid) ? vr[i] : u32x2{0u, 0u};   // code 0 = +0
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      // 4x4 byte transpose of the four tokens' codes of dims 4w .. 4w+3
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
        const half4_t vb = {lo[0], lo[1], hi[0], hi[1]};
        acc[4 * w + e] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, vb, acc[4 * w + e], 0, 0, 0);
      }
    }
  } else {
    u32x4 vv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      vv[i] = (!kMasked || 4 * i + c < nvalid) ? vr[i] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int w = u / 2;
      const unsigned sel = (u & 1) ? 0x07060302u : 0x05040100u;   // high or low halves
      const unsigned d01 = __builtin_amdgcn_perm(vv[1][w], vv[0][w], sel);
      const unsigned d23 = __builtin_amdgcn_perm(vv[3][w], vv[2][w], sel);
      const half4_t vb = __builtin_bit_cast(half4_t, u32x2{d01, d23});
      acc[u] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, vb, acc[u], 0, 0, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// log-sum-exp merge of one output row over nseg normalised partials
//
// Partial s of the row sits at o + (slot(s) * rows + row) * D and
// lse + slot(s) * rows + row, with slot(s) = slot0 + s * slot_step.  With
// L = max_s lse_s and w_s = exp(lse_s - L): out = sum_s w_s o_s / sum_s w_s
// and lse = L + ln(sum_s w_s).  Partials with lse = -inf weigh nothing; if
// every partial is empty the row is 0 with lse -inf.  One wave per row; lane
// l returns dims 2l and 2l + 1.
// Rows with at most N partials: every load of the row in one round (the lse
// of partial `lane` and, for each partial u < N, this lane's two dims; a slot
// past the last re-reads the last with weight 0).
template <int N>
__device__ __forceinline__ void merge_row_batch(const float* o, const float* lse, long long slot0,
                                                long long slot_step, int nseg, long long rows,
                                                long long row, int lane, f32x2& res,
                                                float& lse_res) {
  const int last = max(nseg - 1, 0);
  const float lv =
      lane < nseg ? lse[(slot0 + (long long)lane * slot_step) * rows + row] : -INFINITY;
  f32x2 ov[N];
#pragma unroll
  for (int u = 0; u < N; ++u)
    ov[u] = *reinterpret_cast<const f32x2*>(
        o + ((slot0 + (long long)min(u, last) * slot_step) * rows + row) * kD + 2 * lane);
  const float L = wave_max_f32(lv);
  res = f32x2{0.0f, 0.0f};
  lse_res = -INFINITY;
  if (nseg == 0 || L == -INFINITY) return;
  const float wl = lane < nseg ? fast_exp2((lv - L) * kLog2e) : 0.0f;
  const float wsum = wave_sum_f32(wl);
  f32x2 acc = {0.0f, 0.0f};
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const float wj = uniform_f32(wl, u);
    acc.x = fmaf(wj, ov[u].x, acc.x);
    acc.y = fmaf(wj, ov[u].y, acc.y);
  }
  const float inv = 1.0f / wsum;
  res = f32x2{acc.x * inv, acc.y * inv};
  lse_res = L + __builtin_logf(wsum);
}

__device__ __forceinline__ void merge_row(const float* o, const float* lse, long long slot0,
                                          long long slot_step, int nseg, long long rows,
                                          long long row, int lane, f32x2& res, float& lse_res) {
  // nseg is uniform: one round of loads sized to the row
  if (nseg <= 4)
    return merge_row_batch<4>(o, lse, slot0, slot_step, nseg, rows, row, lane, res, lse_res);
  if (nseg <= 8)
    return merge_row_batch<8>(o, lse, slot0, slot_step, nseg, rows, row, lane, res, lse_res);
  if (nseg <= 16)
    return merge_row_batch<16>(o, lse, slot0, slot_step, nseg, rows, row, lane, res, lse_res);
  float L = -INFINITY;
  for (int s = lane; s < nseg; s += kWave) L = fmaxf(L, lse[(slot0 + s * slot_step) * rows + row]);
  L = wave_max_f32(L);
  res = f32x2{0.0f, 0.0f};
  lse_res = -INFINITY;
  if (L == -INFINITY) return;
  float wsum = 0.0f;
  f32x2 acc = {0.0f, 0.0f};
  const long long ostep = slot_step * rows * kD;
  for (int s0 = 0; s0 < nseg; s0 += kWave) {
    const int s = s0 + lane;
    const float wl =
        s < nseg ? fast_exp2((lse[(slot0 + s * slot_step) * rows + row] - L) * kLog2e) : 0.0f;
    wsum += wl;
    const int cnt = min(kWave, nseg - s0);
    const float* ob = o + ((slot0 + (long long)s0 * slot_step) * rows + row) * kD + 2 * lane;
    int j = 0;
    for (; j + 8 <= cnt; j += 8) {
      f32x2 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const f32x2*>(ob + (j + u) * ostep);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wj = uniform_f32(wl, j + u);
        acc.x = fmaf(wj, v[u].x, acc.x);
        acc.y = fmaf(wj, v[u].y, acc.y);
      }
    }
    for (; j < cnt; ++j) {
      const f32x2 v = *reinterpret_cast<const f32x2*>(ob + j * ostep);
      const float wj = uniform_f32(wl, j);
      acc.x = fmaf(wj, v.x, acc.x);
      acc.y = fmaf(wj, v.y, acc.y);
    }
  }
  wsum = wave_sum_f32(wsum);
  const float inv = 1.0f / wsum;
  res.x = acc.x * inv;
  res.y = acc.y * inv;
  lse_res = L + __builtin_logf(wsum);
}

// ---------------------------------------------------------------------------
// host side: the thread-local message behind pda_last_error()

__attribute__((visibility("hidden"))) int fail(int code, const char* fmt, ...)
    __attribute__((format(printf, 2, 3)));
__attribute__((visibility("hidden"))) int ok();

inline bool finite_f32(float x) {
  uint32_t bits;
  __builtin_memcpy(&bits, &x, sizeof(bits));
  return (bits & 0x7F800000u) != 0x7F800000u;
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace pda
