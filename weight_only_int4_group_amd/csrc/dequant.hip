// Standalone dequantisation of packed group-wise INT4 weights to bf16 or fp16 (gfx950).
//
// Method: x_hat = scale * (q - z) per element ("DL S067 · Quantization — INT8, INT4, GPTQ,
// AWQ", §1 "The core math"), with one scale and zero-point per group of g consecutive
// weights along K ("Model Quantization" §1 "Group-wise Quantization").  Symmetric codes are
// 4-bit two's complement with z = 0.
//
// Exactness: the scale is an fp16 value (11 significant bits) and q - z an integer in
// [-15, 15], so scale * (q - z) is exact in fp32; it is formed as fma(q, s, -s z) (s z is
// exact as well, and the fma rounds the exact, representable result once), then rounded to
// the output type to nearest even.  The output therefore equals the exact dequantised value
// rounded once to bf16 / fp16 (fp16 overflows to infinity as IEEE rounding says).
//
// Layout: packed is a flat stream of dwords.  Dword d holds the codes of the flat elements
// 8d .. 8d + 7 (even element in the low nibble), and their outputs are the 16 bytes at
// out + 16 d.  K % g == 0, so groups tile the flat array: dword d belongs to group d / (g / 8),
// which is also the flat index into scales[N, K/g] and zeros[N, K/g].
//
// Access pattern (HBM-bound: 4 bytes of codes in, 16 bytes out per dword).  A wave works on
// chunks of 256 consecutive dwords; in step j (0..3) lane l takes dword 64 j + l, so every
// code load reads 256 contiguous bytes and every 16-byte store writes 1 KiB contiguous.
// Waves stride over the chunks (persistent grid) and request the next chunk's codes and
// group parameters before converting the current one.
#include "q4_device.h"
#include "q4_internal.h"

namespace q4 {
namespace {

constexpr int kChunk = 4 * kWave;     // dwords per wave chunk
constexpr int kBlock = 256;

// Unsigned division of 32-bit n by an invariant divisor through one multiply-high
// (Granlund and Montgomery, "Division by Invariant Integers using Multiplication", 1994,
// §4, the round-up method for N = 32): exact for every 0 <= n < 2^32.
struct DivMagic {
  uint32_t mul;
  uint32_t sh1, sh2;
};

__device__ __forceinline__ uint32_t div_magic(uint32_t n, DivMagic m) {
  const uint32_t t = __umulhi(m.mul, n);
  return (t + ((n - t) >> m.sh1)) >> m.sh2;
}

DivMagic make_div_magic(uint32_t d) {
  uint32_t l = 0;
  while ((uint64_t{1} << l) < d) ++l;             // l = ceil(log2 d)
  DivMagic m;
  m.mul = (uint32_t)(((uint64_t{1} << 32) * ((uint64_t{1} << l) - d)) / d + 1);
  m.sh1 = l < 1 ? l : 1;
  m.sh2 = l > 0 ? l - 1 : 0;
  return m;
}

struct Chunk {
  uint32_t w[4];      // eight codes per dword
  uint16_t s[4];      // fp16 group scale bits
  uint8_t z[4];       // zero-point
};

template <typename Out>
__device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <>
__device__ __forceinline__ uint32_t pack2<__bf16>(float lo, float hi) { return pack_bf16x2(lo, hi); }
template <>
__device__ __forceinline__ uint32_t pack2<_Float16>(float lo, float hi) {
  const f16x2 v = {(_Float16)lo, (_Float16)hi};
  return as_u32(v);
}

// Eight codes of one dword -> 16 bytes of Out.  Symmetric codes are offset by 8 (XOR of the
// sign bit), which turns the int4 value q into q + 8 with zero-point 8.
template <typename Out>
__device__ __forceinline__ u32x4 convert8(uint32_t w, float s, float sz) {
  const uint32_t even = w & 0x0f0f0f0fu, odd = (w >> 4) & 0x0f0f0f0fu;
  float v[8];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    v[2 * b] = __builtin_fmaf((float)((even >> (8 * b)) & 0xffu), s, -sz);
    v[2 * b + 1] = __builtin_fmaf((float)((odd >> (8 * b)) & 0xffu), s, -sz);
  }
  u32x4 r;
  r[0] = pack2<Out>(v[0], v[1]);
  r[1] = pack2<Out>(v[2], v[3]);
  r[2] = pack2<Out>(v[4], v[5]);
  r[3] = pack2<Out>(v[6], v[7]);
  return r;
}

// POW2: the group size in dwords is 2^gshift.  Otherwise chunk starts advance by a fixed
// stride, whose quotient and remainder by the group size are carried from chunk to chunk,
// and the lane's offset inside the chunk is divided through DivMagic.
//
// Every access goes through a buffer resource that starts at the chunk (codes, output) or
// at the chunk's first group (scales, zeros) and ends at the array's end, so lanes past the
// end read zeros and their stores are dropped by the hardware: no per-lane branch.
template <bool SYM, bool POW2, typename Out>
__global__ __launch_bounds__(kBlock) void dequant_kernel(
    const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    const uint8_t* __restrict__ zeros, u32x4* __restrict__ out, uint64_t D, uint64_t groups,
    uint64_t nchunks, uint32_t gd, uint32_t gshift, DivMagic magic, uint64_t stride_q,
    uint32_t stride_r) {
  const uint32_t lane = threadIdx.x & (kWave - 1);
  const uint64_t waves = (uint64_t)gridDim.x * (kBlock / kWave);
  // Chunk bookkeeping is wave-uniform (scalar registers, scalar branches).
  uint64_t c = (uint64_t)blockIdx.x * (kBlock / kWave) +
               (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (c >= nchunks) return;
  // Group of the first dword of chunk c is q0, and that dword is r0 dwords into it.
  uint64_t q0;
  uint32_t r0;
  if (POW2) {
    q0 = (c * kChunk) >> gshift;
    r0 = (uint32_t)(c * kChunk - (q0 << gshift));
  } else {
    q0 = c * kChunk / gd;
    r0 = (uint32_t)(c * kChunk - q0 * gd);
  }

  auto clamp_bytes = [](uint64_t n) { return (uint32_t)(n < (1u << 30) ? n : (1u << 30)); };
  auto load = [&](uint64_t cc, uint64_t qq, uint32_t rr) {
    const uint64_t d0 = cc * kChunk;
    const auto rc = buffer_over(codes + d0, clamp_bytes((D - d0) * 4));
    const auto rs = buffer_over(scales + qq, clamp_bytes((groups - qq) * 2));
    const auto rz = buffer_over(SYM ? nullptr : zeros + qq, SYM ? 0u : clamp_bytes(groups - qq));
    Chunk k;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t o = rr + j * kWave + lane;        // dwords from the start of group qq
      const uint32_t gl = POW2 ? o >> gshift : div_magic(o, magic);
      k.w[j] = __builtin_amdgcn_raw_buffer_load_b32(rc, 4 * (j * kWave + lane), 0, kBufferNT);
      k.s[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, 2 * gl, 0, 0);
      if (!SYM) k.z[j] = __builtin_amdgcn_raw_buffer_load_b8(rz, gl, 0, 0);
    }
    return k;
  };
  // Start of the chunk a wave takes after chunk (cc, qq, rr).
  auto advance = [&](uint64_t& cc, uint64_t& qq, uint32_t& rr) {
    cc += waves;
    qq += stride_q;
    rr += stride_r;
    if (rr >= gd) {
      rr -= gd;
      ++qq;
    }
  };
  auto convert_store = [&](const Chunk& k, uint64_t cc) {
    const uint64_t d0 = cc * kChunk;
    const auto ro = buffer_over(out + d0, clamp_bytes((D - d0) * 16));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = SYM ? k.w[j] ^ 0x88888888u : k.w[j];
      const float sf = (float)__builtin_bit_cast(_Float16, k.s[j]);
      const float zf = SYM ? 8.0f : (float)k.z[j];
      const u32x4 v = convert8<Out>(w, sf, sf * zf);
      // streamed: every output byte is written once (70B-shaped weight: 112.2 -> 106.9 us)
      __builtin_amdgcn_raw_buffer_store_b128(v, ro, 16 * (j * kWave + lane), 0, kBufferNT);
    }
  };

  // A chunk loaded for nothing on the way out is still "used" there, so the compiler cannot
  // sink its loads below the conversion of the previous chunk.
  auto keep = [](const Chunk& k) {
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" ::"v"(k.w[j]), "v"((uint32_t)k.s[j]), "v"((uint32_t)k.z[j]));
  };

  // Two chunks alternate between the register sets a and b, so the loads of one are in
  // flight while the other is converted and stored, with no copy between them (a copy
  // would wait for the loads, and on this ISA the wait counter also covers the stores).
  // A wave past its last chunk reloads its current chunk, so every load stays in bounds.
  Chunk a = load(c, q0, r0);
  while (true) {
    uint64_t c1 = c, q1 = q0;
    uint32_t r1 = r0;
    advance(c1, q1, r1);
    const bool more1 = c1 < nchunks;
    const Chunk b = load(more1 ? c1 : c, more1 ? q1 : q0, more1 ? r1 : r0);
    __builtin_amdgcn_sched_barrier(0);     // keep the phases in this order
    convert_store(a, c);
    __builtin_amdgcn_sched_barrier(0);
    if (!more1) {
      keep(b);
      break;
    }
    uint64_t c2 = c1, q2 = q1;
    uint32_t r2 = r1;
    advance(c2, q2, r2);
    const bool more2 = c2 < nchunks;
    a = load(more2 ? c2 : c1, more2 ? q2 : q1, more2 ? r2 : r1);
    __builtin_amdgcn_sched_barrier(0);
    convert_store(b, c1);
    __builtin_amdgcn_sched_barrier(0);
    if (!more2) {
      keep(a);
      break;
    }
    c = c2;
    q0 = q2;
    r0 = r2;
  }
}

template <bool SYM, typename Out>
hipError_t launch_out(const void* packed, const void* scales, const void* zeros, void* out,
                      uint64_t D, int g, int num_cus, hipStream_t stream) {
  const uint64_t nchunks = (D + kChunk - 1) / kChunk;
  constexpr int kWavesPerBlock = kBlock / kWave;
  uint64_t blocks = (nchunks + kWavesPerBlock - 1) / kWavesPerBlock;
  const uint64_t cap = (uint64_t)num_cus * 8;
  if (blocks > cap) blocks = cap;
  const uint32_t gd = (uint32_t)(g / 8);
  const uint64_t stride = blocks * kWavesPerBlock * kChunk;     // dwords between a wave's chunks
  const DivMagic magic = make_div_magic(gd);
  const bool pow2 = (gd & (gd - 1)) == 0;
  uint32_t gshift = 0;
  while ((1u << gshift) < gd) ++gshift;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kBlock), 0, stream,
                       (const uint32_t*)packed, (const uint16_t*)scales, (const uint8_t*)zeros,
                       (u32x4*)out, D, D / gd, nchunks, gd, gshift, magic, stride / gd,
                       (uint32_t)(stride % gd));
    return hipGetLastError();
  };
  return pow2 ? go(dequant_kernel<SYM, true, Out>) : go(dequant_kernel<SYM, false, Out>);
}

}  // namespace

hipError_t launch_dequantize(const void* packed, const void* scales, const void* zeros, int64_t N,
                             int64_t K, int g, bool sym, void* out, bool f16_out, int num_cus,
                             hipStream_t stream) {
  const uint64_t D = (uint64_t)N * (uint64_t)K / 8;
  if (sym)
    return f16_out ? launch_out<true, _Float16>(packed, scales, zeros, out, D, g, num_cus, stream)
                   : launch_out<true, __bf16>(packed, scales, zeros, out, D, g, num_cus, stream);
  return f16_out ? launch_out<false, _Float16>(packed, scales, zeros, out, D, g, num_cus, stream)
                 : launch_out<false, __bf16>(packed, scales, zeros, out, D, g, num_cus, stream);
}

}  // namespace q4
