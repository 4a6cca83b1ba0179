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

}  // extern "C"
