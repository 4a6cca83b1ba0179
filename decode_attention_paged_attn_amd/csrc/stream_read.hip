// A diagnostic streaming read for MI355X (gfx950): how fast a plain kernel
// reads HBM with the same 16-byte load forms the attention kernels use.  It
// gives the decode kernels' KV-read rate a ceiling measured on the device
// itself, next to the 8 TB/s peak; it is no part of the attention path.
//
// Every thread reads four 16-byte words per step (a grid-stride loop over the
// buffer, loads issued together; 256 work-groups of 256 threads per CU) and
// folds them into an xor.  The result is
// stored only if it equals a value the buffer would have to be built for, so
// in practice nothing is written, while the loads cannot be dropped.
//
// A second diagnostic times the LDS read forms of the multi-query kernels
// (ds_read_b128, ds_read_b64, ds_read_b64_tr_b16, ds_read_b32): every wave of
// a 256-thread work-group reads a 64 KiB stage over and over with
// conflict-free addresses and sums what it gets, so that the SQ_LDS_IDX_ACTIVE
// count of those kernels can be set against what each form costs and against
// a kernel that does nothing else.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "paged_attn.h"
#include "pda_common.h"

namespace {

using namespace pda;

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 4;
constexpr unsigned kNeverXor = 0x9E3779B9u;   // stored only if the xor of a thread's words is this

template <bool kNt>
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4* p, long long n16,
                                                                  unsigned* sink) {
  const long long stride = (long long)gridDim.x * kReadThreads;
  long long i = (long long)blockIdx.x * kReadThreads + threadIdx.x;
  unsigned acc = 0;
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    u32x4 w[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      if constexpr (kNt) w[u] = __builtin_nontemporal_load(p + i + u * stride);
      else w[u] = p[i + u * stride];
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= w[u].x ^ w[u].y ^ w[u].z ^ w[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 w = kNt ? __builtin_nontemporal_load(p + i) : p[i];
    acc ^= w.x ^ w.y ^ w.z ^ w.w;
  }
  if (acc == kNeverXor) sink[0] = acc;
}

constexpr int kLdsProbeThreads = 256;
constexpr int kLdsProbeWords = 16384;          // 64 KiB of stage
constexpr int kLdsProbeReads = 16;             // reads per wave and pass

// Word i of the stage, the pattern the host recomputes to check the sums.
__device__ __forceinline__ unsigned lds_probe_word(int i) { return (unsigned)i * 2654435761u; }

// Form 0: ds_read_b128 (1 KiB per wave-wide read), 1: ds_read_b64 (512 B),
// 2: ds_read_b64_tr_b16 (512 B), 3: ds_read_b32 (256 B).  Read r of a pass
// covers a contiguous window of the stage at r times its size, lane l at l
// times the lane's share: no bank conflicts.  Thread t of work-group b stores
// the wrapping sum of the 32-bit words it received at out[256 b + t].
template <int kForm>
__global__ __launch_bounds__(kLdsProbeThreads) void lds_probe_kernel(unsigned* out, int iters) {
  __shared__ __attribute__((aligned(16))) unsigned stage[kLdsProbeWords];
  typedef __attribute__((address_space(3))) char LdsChar;
  typedef __fp16 fp16x4 __attribute__((vector_size(8)));      // the builtin's element type
  typedef __attribute__((address_space(3))) fp16x4 LdsHalf4;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  for (int i = tid; i < kLdsProbeWords; i += kLdsProbeThreads) stage[i] = lds_probe_word(i);
  __syncthreads();
  const LdsChar* base = (const LdsChar*)stage;
  unsigned acc = 0;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < kLdsProbeReads; ++r) {
      constexpr int kBytes = kForm == 0 ? 16 : kForm == 3 ? 4 : 8;
      unsigned a = (unsigned)(r * kWave * kBytes + kBytes * lane);
      // opaque per read: no hoisting out of the pass, no pairing into read2
      asm volatile("" : "+v"(a));
      if constexpr (kForm == 0) {
        const u32x4 x = *(const __attribute__((address_space(3))) u32x4*)(base + a);
        acc += (x.x + x.y) + (x.z + x.w);
      } else if constexpr (kForm == 1) {
        const u32x2 x = *(const __attribute__((address_space(3))) u32x2*)(base + a);
        acc += x.x + x.y;
      } else if constexpr (kForm == 2) {
        const u32x2 x =
            __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4f16((LdsHalf4*)(base + a)));
        acc += x.x + x.y;
      } else {
        acc += *(const __attribute__((address_space(3))) unsigned*)(base + a);
      }
    }
  }
  out[(long long)blockIdx.x * kLdsProbeThreads + tid] = acc;
}

}  // namespace

extern "C" {

int pda_stream_read(const void* src, size_t bytes, unsigned* sink, int nontemporal,
                    void* stream_ptr) {
  if (bytes == 0) return pda::ok();
  if (!src || !sink) return pda::fail(PDA_EINVAL, "src and sink must not be null");
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || bytes % 16 != 0)
    return pda::fail(PDA_EINVAL, "src and bytes must be multiples of 16");
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  const long long n16 = (long long)(bytes / 16);
  const long long want = (n16 + kReadThreads * kReadUnroll - 1) / (kReadThreads * kReadUnroll);
  // 256 work-groups per CU read fastest on MI355X (4 GiB: 64 per CU 6.64 TB/s
  // non-temporal, 256 per CU 6.97, one pass per thread with no cap 6.46)
  const long long cap = 256LL * cus;
  const unsigned grid = (unsigned)std::max<long long>(1, std::min<long long>(want, cap));
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const u32x4* p = static_cast<const u32x4*>(src);
  if (nontemporal)
    hipLaunchKernelGGL(stream_read_kernel<true>, dim3(grid), dim3(kReadThreads), 0, stream, p,
                       n16, sink);
  else
    hipLaunchKernelGGL(stream_read_kernel<false>, dim3(grid), dim3(kReadThreads), 0, stream, p,
                       n16, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pda::fail(PDA_EHIP, "stream read launch: %s", hipGetErrorString(e));
  return pda::ok();
}

int pda_lds_probe(int form, unsigned* out, int work_groups, int iters, void* stream_ptr) {
  if (form < 0 || form > 3) return pda::fail(PDA_EINVAL, "form must be 0..3");
  if (work_groups < 0 || iters < 0) return pda::fail(PDA_EINVAL, "negative size");
  if (work_groups == 0) return pda::ok();
  if (!out) return pda::fail(PDA_EINVAL, "out must not be null");
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const dim3 grid((unsigned)work_groups), block(kLdsProbeThreads);
  switch (form) {
    case 0: hipLaunchKernelGGL(lds_probe_kernel<0>, grid, block, 0, stream, out, iters); break;
    case 1: hipLaunchKernelGGL(lds_probe_kernel<1>, grid, block, 0, stream, out, iters); break;
    case 2: hipLaunchKernelGGL(lds_probe_kernel<2>, grid, block, 0, stream, out, iters); break;
    default: hipLaunchKernelGGL(lds_probe_kernel<3>, grid, block, 0, stream, out, iters); break;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pda::fail(PDA_EHIP, "LDS probe launch: %s", hipGetErrorString(e));
  return pda::ok();
}

}  // extern "C"
