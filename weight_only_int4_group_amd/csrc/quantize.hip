// Group-wise INT4 round-to-nearest quantization and nibble packing (gfx950).
//
// Method: "DL S067 · Quantization — INT8, INT4, GPTQ, AWQ", §1 "The core math" (asymmetric
// scale (beta - alpha) / (q_max - q_min), z = round(q_min - alpha / scale),
// q = clip(round(x / scale) + z); symmetric scale max|x| / q_max), applied per group of g
// consecutive weights along K ("DL S067" §2; "Model Quantization" §1 "Group-wise
// Quantization").  The exact rules (fp32 arithmetic, fp16 scale, round half to even,
// alpha/beta extended to include 0, nibble order) are those stated in include/q4.h.
//
// Bit-exactness without an IEEE divide per element.  For a bf16 x and an fp16 scale s the
// exact quotient x / s is either exactly a half-integer or at least 2^-12 away from one, so
// rint of the IEEE fp32 quotient equals rint of the exact quotient.  Each code is therefore
// computed as t = x * r (r ~ 1/s), one residual correction t' = t + fl(x - t s) * r (two
// fmas), and rint(t'): the corrected value is within 2^-40 of x / s, equals it exactly at
// ties, and never crosses a half-integer the exact quotient does not cross.
//
// The per-group scale needs the IEEE quotient itself: fl32(d / 15) (or d / 7) is computed
// as q0 = d * RN(1/15), r = fma(-q0, 15, d) (exact), fl = fma(r, RN(1/15), q0).  A quotient
// by 15 or 7 is never a rounding midpoint and stays at least ulp/30 from one, while the
// sequence is within 2^-24 ulp of it, so the rounding is the IEEE one.
//
// Layout: the weight matrix is processed as a flat array of 8-element chunks (16 bytes of
// bf16 -> 4 bytes of nibbles).  Groups never straddle rows (K % g == 0), so the flat group
// index is also the index into scales[N, K/g] and zeros[N, K/g].
#include "q4_device.h"
#include "q4_internal.h"

namespace q4 {
namespace {

struct GroupParams {
  float sf;       // fp32 value of the stored fp16 scale
  float rcp;      // ~1/sf (any value within 2^-22 relative works, see above)
  float zf;       // zero-point as float (0 in symmetric mode)
  uint16_t s16;   // stored scale bits
};

// alpha <= 0 <= beta already; returns the stored scale, its reciprocal and the zero-point.
// B = 4: codes [0, 15] / [-8, 7], scale d / 15 or d / 7 through the exact-division sequence
// below; B = 8 (W8A16): codes [0, 255] / [-127, 127], scale d / 255 or d / 127 by an IEEE
// division (once per group).  The caps keep d finite and are far above 65504 * k.
template <bool SYM, int B = 4>
__device__ __forceinline__ GroupParams group_params(float alpha, float beta_or_absmax) {
  if constexpr (B == 8) {
    const float d = SYM ? fminf(beta_or_absmax, 1.0e7f) : fminf(beta_or_absmax - alpha, 3.0e7f);
    const float s32 = fminf(d / (SYM ? 127.0f : 255.0f), 65504.0f);
    _Float16 h = (_Float16)s32;
    if (h == (_Float16)0.0f) h = (_Float16)1.0f;
    GroupParams p;
    p.sf = (float)h;
    p.s16 = __builtin_bit_cast(uint16_t, h);
    p.rcp = __builtin_amdgcn_rcpf(p.sf);
    if (SYM) {
      p.zf = 0.0f;
    } else {
      const float t = alpha * p.rcp;
      const float res = __builtin_fmaf(-t, p.sf, alpha);
      const float tq = __builtin_fmaf(res, p.rcp, t);
      p.zf = fminf(fmaxf(-rintf(tq), 0.0f), 255.0f);
    }
    return p;
  }
  float d, c, k;
  if (SYM) {
    d = fminf(beta_or_absmax, 1.0e6f);       // >= 65504 * 7 saturates either way
    k = 7.0f;
    c = 1.0f / 7.0f;
  } else {
    d = fminf(beta_or_absmax - alpha, 2.0e6f);   // one IEEE subtraction; cap keeps it finite
    k = 15.0f;
    c = 1.0f / 15.0f;
  }
  const float q0 = d * c;
  const float r = __builtin_fmaf(-q0, k, d);
  float s32 = __builtin_fmaf(r, c, q0);          // == fl32(d / k)
  s32 = fminf(s32, 65504.0f);
  _Float16 h = (_Float16)s32;                    // round to nearest even
  if (h == (_Float16)0.0f) h = (_Float16)1.0f;
  GroupParams p;
  p.sf = (float)h;
  p.s16 = __builtin_bit_cast(uint16_t, h);
  p.rcp = __builtin_amdgcn_rcpf(p.sf);
  if (SYM) {
    p.zf = 0.0f;
  } else {
    const float t = alpha * p.rcp;
    const float res = __builtin_fmaf(-t, p.sf, alpha);
    const float tq = __builtin_fmaf(res, p.rcp, t);          // ~ alpha / s
    p.zf = fminf(fmaxf(-rintf(tq), 0.0f), 15.0f);           // rint(0 - alpha/s), clamped
  }
  return p;
}

template <bool SYM, int B = 4>
__device__ __forceinline__ uint32_t code_of(float x, const GroupParams& p) {
  const float t = x * p.rcp;
  const float res = __builtin_fmaf(-t, p.sf, x);
  const float tq = __builtin_fmaf(res, p.rcp, t);            // ~ x / s
  const float c = rintf(tq);
  constexpr float kLo = B == 8 ? -127.0f : -8.0f, kHi = B == 8 ? 127.0f : 7.0f;
  constexpr float kTop = B == 8 ? 255.0f : 15.0f;
  constexpr uint32_t kMask = B == 8 ? 0xFFu : 0xFu;
  if (SYM) {
    const float v = fminf(fmaxf(c, kLo), kHi);
    return (uint32_t)(int)v & kMask;                          // B-bit two's complement
  } else {
    const float v = fminf(fmaxf(c + p.zf, 0.0f), kTop);
    return (uint32_t)v;
  }
}

// Unpack a 16-byte chunk of 8 bf16 values.
__device__ __forceinline__ void unpack8(const u32x4 v, float x[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_lo(v[i]);
    x[2 * i + 1] = bf16_hi(v[i]);
  }
}

// Optional per-column scale applied before quantization (AWQ-style scaling): the weight
// quantized is bf16(fl32(w * s_j)), one IEEE fp32 product rounded to nearest even to bf16.
// c8 = K / 8 chunks per row; `row64` says c8 is a multiple of 64, so the 64 consecutive
// chunks of a wave step never straddle a row and their columns follow from one wave-uniform
// remainder; `small` says every flat chunk index fits 32 bits.
struct ColScale {
  const float* s;
  int64_t c8;
  bool row64, small;
};

// Column chunk of flat chunk `chunk` whose wave step starts at flat chunk `wave_base`.
__device__ __forceinline__ uint32_t col_chunk(const ColScale& cs, int64_t wave_base, int64_t chunk) {
  if (cs.row64) {
    const int64_t b = __builtin_amdgcn_readfirstlane((int)(uint32_t)wave_base) |
                      ((int64_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(wave_base >> 32)) << 32);
    return (uint32_t)(b % cs.c8) + (uint32_t)(chunk - wave_base);
  }
  return cs.small ? (uint32_t)chunk % (uint32_t)cs.c8 : (uint32_t)(chunk % cs.c8);
}

__device__ __forceinline__ void apply_colscale(const ColScale& cs, uint32_t cc, float x[8]) {
  const float4* sp = reinterpret_cast<const float4*>(cs.s + 8 * (size_t)cc);
  const float4 a = sp[0], b = sp[1];
  const float sv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (float)(__bf16)(x[i] * sv[i]);
}

template <bool SYM>
__device__ __forceinline__ uint32_t pack8(const float x[8], const GroupParams& p) {
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) w |= code_of<SYM>(x[i], p) << (4 * i);
  return w;
}

// Eight 8-bit codes, element i in byte i.
template <bool SYM>
__device__ __forceinline__ u32x2 pack8_bytes(const float x[8], const GroupParams& p) {
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo |= code_of<SYM, 8>(x[i], p) << (8 * i);
    hi |= code_of<SYM, 8>(x[i + 4], p) << (8 * i);
  }
  return u32x2{lo, hi};
}

// Store the codes of chunk c (8 weights): a dword of nibbles (B = 4) or two dwords of bytes.
template <bool SYM, int B>
__device__ __forceinline__ void store_codes(void* codes, int64_t c, const float x[8], const GroupParams& p) {
  // The codes are written once and not read back by this kernel: streaming stores keep them
  // from displacing the weight stream in the caches.
  if constexpr (B == 8) {
    __builtin_nontemporal_store(pack8_bytes<SYM>(x, p), reinterpret_cast<u32x2*>(codes) + c);
  } else {
    __builtin_nontemporal_store(pack8<SYM>(x, p), reinterpret_cast<uint32_t*>(codes) + c);
  }
}

// Min or max over each aligned group of L lanes (L a power of two, 4..64), the result in every
// lane.  Inside a 16-lane row the partners come from DPP (quad permutes, then the half-row and
// row mirrors: after each step every lane holds the result of a twice larger group, in any
// order, which min and max do not mind), with no LDS traffic; wider groups add lane exchanges
// across rows.
template <int L, typename Op>
__device__ __forceinline__ float lanes_reduce(float v, Op op) {
  v = op(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  if constexpr (L >= 4) v = op(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  if constexpr (L >= 8) v = op(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
  if constexpr (L >= 16) v = op(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
#pragma unroll
  for (int o = 16; o < L; o <<= 1) v = op(v, __shfl_xor(v, o));
  return v;
}

template <int L>
__device__ __forceinline__ float lanes_min(float v) {
  return lanes_reduce<L>(v, [](float a, float b) { return fminf(a, b); });
}
template <int L>
__device__ __forceinline__ float lanes_max(float v) {
  return lanes_reduce<L>(v, [](float a, float b) { return fmaxf(a, b); });
}

// g in {32, 64, 128, 256, 512}: a group is L = g/8 consecutive lanes, each holding one chunk.
// A wave covers 64 consecutive chunks (512 weights) per step; U steps are loaded together.
template <int L, bool SYM, int U, bool SC, int B>
__global__ __launch_bounds__(256) void quantize_lanes_kernel(
    const u32x4* __restrict__ W, int64_t nchunks, void* __restrict__ packed,
    uint16_t* __restrict__ scales, uint8_t* __restrict__ zeros, ColScale cs) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) / kWave;
  for (int64_t base = wave * U; base * kWave < nchunks; base += nwaves * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = (base + u) * kWave + lane;
      v[u] = c < nchunks ? __builtin_nontemporal_load(W + c) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = (base + u) * kWave + lane;
      float x[8];
      unpack8(v[u], x);
      if (SC) apply_colscale(cs, c < nchunks ? col_chunk(cs, (base + u) * kWave, c) : 0u, x);
      float lo = 0.0f, hi = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (SYM) {
          hi = fmaxf(hi, fabsf(x[i]));
        } else {
          lo = fminf(lo, x[i]);
          hi = fmaxf(hi, x[i]);
        }
      }
      if (!SYM) lo = lanes_min<L>(lo);
      hi = lanes_max<L>(hi);
      const GroupParams p = group_params<SYM, B>(lo, hi);
      if (c < nchunks) {
        store_codes<SYM, B>(packed, c, x, p);
        if ((lane & (L - 1)) == 0) {
          const int64_t grp = c / L;
          scales[grp] = p.s16;
          zeros[grp] = (uint8_t)p.zf;
        }
      }
    }
  }
}

// Column-scaled form (AWQ-style) when a row holds a whole number of 64-chunk strips: a wave
// owns one strip (one chunk, eight columns, per lane) of `rows` consecutive rows, so a lane
// loads the eight column scales of its chunk once and applies them to every row it walks,
// instead of re-reading 32 bytes of scales per 16 bytes of weights.  Rows are taken U at a
// time, their loads issued together.  g = 8 L with L | 64, so groups never straddle a strip.
template <int L, bool SYM, int U, int B>
__global__ __launch_bounds__(256) void quantize_cols_kernel(
    const u32x4* __restrict__ W, int64_t N, int64_t c8, int64_t rows, void* __restrict__ packed,
    uint16_t* __restrict__ scales, uint8_t* __restrict__ zeros, const float* __restrict__ colscale) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const int64_t strips = c8 / kWave;
  const int64_t strip = wave % strips;
  const int64_t r0 = (wave / strips) * rows;
  const int64_t r1 = min(N, r0 + rows);
  const int64_t cc = strip * kWave + lane;                       // this lane's column chunk
  const float4* sp = reinterpret_cast<const float4*>(colscale + 8 * cc);
  const float4 sa = sp[0], sb = sp[1];
  const float sv[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
  for (int64_t r = r0; r < r1; r += U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = r + u < r1 ? __builtin_nontemporal_load(W + (r + u) * c8 + cc) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (r + u >= r1) break;                                      // wave-uniform
      const int64_t c = (r + u) * c8 + cc;
      float x[8];
      unpack8(v[u], x);
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = (float)(__bf16)(x[i] * sv[i]);
      float lo = 0.0f, hi = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (SYM) {
          hi = fmaxf(hi, fabsf(x[i]));
        } else {
          lo = fminf(lo, x[i]);
          hi = fmaxf(hi, x[i]);
        }
      }
      if (!SYM) lo = lanes_min<L>(lo);
      hi = lanes_max<L>(hi);
      const GroupParams p = group_params<SYM, B>(lo, hi);
      store_codes<SYM, B>(packed, c, x, p);
      if ((lane & (L - 1)) == 0) {
        const int64_t grp = c / L;
        scales[grp] = p.s16;
        zeros[grp] = (uint8_t)p.zf;
      }
    }
  }
}

// Any g (multiple of 32): one wave per group, two passes over the group's chunks
// (range, then codes); the second pass re-reads the group, normally from cache.
template <bool SYM, bool SC, int B>
__global__ __launch_bounds__(256) void quantize_wave_kernel(
    const u32x4* __restrict__ W, int64_t ngroups, int cpg, void* __restrict__ packed,
    uint16_t* __restrict__ scales, uint8_t* __restrict__ zeros, ColScale cs) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) / kWave;
  for (int64_t grp = wave; grp < ngroups; grp += nwaves) {
    const int64_t c0 = grp * cpg;
    float lo = 0.0f, hi = 0.0f;
    // the group's first column chunk (groups never straddle rows)
    const uint32_t gc = SC ? (uint32_t)((grp % (cs.c8 / cpg)) * cpg) : 0u;
    for (int j = lane; j < cpg; j += kWave) {
      float x[8];
      unpack8(W[c0 + j], x);
      if (SC) apply_colscale(cs, gc + (uint32_t)j, x);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (SYM) {
          hi = fmaxf(hi, fabsf(x[i]));
        } else {
          lo = fminf(lo, x[i]);
          hi = fmaxf(hi, x[i]);
        }
      }
    }
    if (!SYM) lo = lanes_min<kWave>(lo);
    hi = lanes_max<kWave>(hi);
    const GroupParams p = group_params<SYM, B>(lo, hi);
    for (int j = lane; j < cpg; j += kWave) {
      float x[8];
      unpack8(W[c0 + j], x);
      if (SC) apply_colscale(cs, gc + (uint32_t)j, x);
      store_codes<SYM, B>(packed, c0 + j, x, p);
    }
    if (lane == 0) {
      scales[grp] = p.s16;
      zeros[grp] = (uint8_t)p.zf;
    }
  }
}

template <int L, bool SYM, int B>
hipError_t launch_lanes(const void* W, int64_t nchunks, void* packed, void* scales, void* zeros,
                        const ColScale& cs, int num_cus, hipStream_t stream) {
  constexpr int U = 4;
  if (cs.s && cs.row64) {
    // Column strips: 8 rows per wave (two rounds of U loads) while that leaves at least 16
    // waves per compute unit, else fewer (W[8192, 8192] at g = 128: 47.6 -> 38.9 us).
    const int64_t N = nchunks / cs.c8, strips = cs.c8 / kWave;
    int64_t rows = 2 * U;
    while (rows > 1 && strips * ((N + rows - 1) / rows) < (int64_t)num_cus * 16) rows >>= 1;
    const int64_t waves = strips * ((N + rows - 1) / rows);
    const int64_t blocks = (waves + 3) / 4;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((quantize_cols_kernel<L, SYM, U, B>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const u32x4*)W, N, cs.c8, rows, packed, (uint16_t*)scales, (uint8_t*)zeros, cs.s);
    return hipGetLastError();
  }
  const int64_t steps = (nchunks + kWave * U - 1) / (kWave * U);   // wave-steps needed
  const int64_t waves_wanted = steps;
  int64_t blocks = (waves_wanted + 3) / 4;
  // Up to 64 blocks per CU: enough waves in flight to keep HBM busy while each wave waits on
  // its loads (8 per CU left the stream at about 55 % of peak).
  const int64_t cap = (int64_t)num_cus * 64;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const u32x4*)W, nchunks,
                       packed, (uint16_t*)scales, (uint8_t*)zeros, cs);
    return hipGetLastError();
  };
  return cs.s ? go(quantize_lanes_kernel<L, SYM, U, true, B>) : go(quantize_lanes_kernel<L, SYM, U, false, B>);
}

template <bool SYM, int B>
hipError_t launch_mode(const void* W, int64_t N, int64_t K, int g, void* packed, void* scales,
                       void* zeros, const ColScale& cs, int num_cus, hipStream_t stream) {
  const int64_t nchunks = N * K / 8;
  switch (g) {
    case 32: return launch_lanes<4, SYM, B>(W, nchunks, packed, scales, zeros, cs, num_cus, stream);
    case 64: return launch_lanes<8, SYM, B>(W, nchunks, packed, scales, zeros, cs, num_cus, stream);
    case 128: return launch_lanes<16, SYM, B>(W, nchunks, packed, scales, zeros, cs, num_cus, stream);
    case 256: return launch_lanes<32, SYM, B>(W, nchunks, packed, scales, zeros, cs, num_cus, stream);
    case 512: return launch_lanes<64, SYM, B>(W, nchunks, packed, scales, zeros, cs, num_cus, stream);
    default: {
      const int64_t ngroups = N * (K / g);
      int64_t blocks = (ngroups + 3) / 4;
      const int64_t cap = (int64_t)num_cus * 8;
      if (blocks > cap) blocks = cap;
      auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const u32x4*)W, ngroups,
                           g / 8, packed, (uint16_t*)scales, (uint8_t*)zeros, cs);
        return hipGetLastError();
      };
      return cs.s ? go(quantize_wave_kernel<SYM, true, B>) : go(quantize_wave_kernel<SYM, false, B>);
    }
  }
}

}  // namespace

hipError_t launch_quantize(const void* W, int64_t N, int64_t K, int g, bool sym, void* packed,
                           void* scales, void* zeros, int num_cus, hipStream_t stream,
                           const float* colscale) {
  const ColScale cs{colscale, K / 8, (K / 8) % kWave == 0, N * K / 8 <= (int64_t)0xffffffff};
  return sym ? launch_mode<true, 4>(W, N, K, g, packed, scales, zeros, cs, num_cus, stream)
             : launch_mode<false, 4>(W, N, K, g, packed, scales, zeros, cs, num_cus, stream);
}

hipError_t launch_quantize8(const void* W, int64_t N, int64_t K, int g, bool sym, void* codes,
                            void* scales, void* zeros, int num_cus, hipStream_t stream) {
  const ColScale cs{nullptr, K / 8, false, true};
  return sym ? launch_mode<true, 8>(W, N, K, g, codes, scales, zeros, cs, num_cus, stream)
             : launch_mode<false, 8>(W, N, K, g, codes, scales, zeros, cs, num_cus, stream);
}

}  // namespace q4
