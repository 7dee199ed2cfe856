// Plain streaming read (gfx950): a measurement helper, not part of the q4 library.  It gives
// the practical HBM read ceiling that the decode kernels are compared with: every lane reads
// 16-byte chunks of a buffer, eight loads in flight, grid-striding over the whole buffer, and
// folds them with XOR so that no load is dead; each wave writes one dword.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kBlock = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kBlock) void stream_read_kernel(const u32x4* __restrict__ p, uint64_t n16,
                                                            uint32_t* __restrict__ out) {
  const uint64_t stride = (uint64_t)gridDim.x * kBlock;
  uint64_t i = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) out[(blockIdx.x * kBlock + threadIdx.x) >> 6] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16) from device pointer p (16-byte aligned) with `blocks` blocks of
// 256 threads; out receives blocks * 4 dwords.  Returns 0, or -1 for bad arguments, or the HIP
// error of the launch.
extern "C" int q4b_stream_read(const void* p, int64_t bytes, void* out, int blocks, void* stream) {
  if (!p || !out || bytes <= 0 || bytes % 16 != 0 || blocks <= 0 ||
      (reinterpret_cast<uintptr_t>(p) & 15) != 0)
    return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kBlock), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(p),
                     (uint64_t)bytes / 16, static_cast<uint32_t*>(out));
  return (int)hipGetLastError();
}
