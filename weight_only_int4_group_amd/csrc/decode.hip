// W4A16 decode for 1 <= M <= 16 on the fp16 matrix cores of gfx950
// (v_mfma_f32_16x16x32_f16).
//
// W4A16: 4-bit weights dequantised inside the kernel, products on 16-bit operands
// ("LLM Weight Quantization - GPTQ, AWQ, SmoothQuant, FP8 & INT4/INT8 Trade-offs",
// "The vocabulary"); decode reads every weight once and is bound by HBM ("Overview").
// Dequantisation x_hat = scale * (q - z) ("DL S067 · Quantization", §1).
//
// Arithmetic (exact up to fp32 summation and the final bf16 rounding):
//   * (q - z) is formed exactly in fp16 (nibble OR-ed into the mantissa of 1024.0, minus
//     1024 + z; nibbles in bits 4..7 give 16 (q - z));
//   * X is converted to fp16 exactly after scaling each (row m, k tile) by a power of two 2^e
//     that puts its largest |x| in [2^14, 2^15); the positions that meet a 16 (q - z) weight
//     carry 2^(e-4);
//   * the MFMA sums the products of one tile (exact products, fp32 accumulation); each tile's
//     partial is multiplied by scale * 2^-e in fp32 and accumulated.
// Roles: D[m][n] = sum_k X[m][k] W[n][k], A = X (rows m, zero beyond M), B = dequantised W
// (16 rows n).  A tile is TK = min(g, 128) weights wide along K, so it never straddles a group.
// In tile t, lane (j, q) = (lane % 16, lane / 16) owns the TK/4 weights that start at
// k = t TK + q TK/4 in row n0 + j (TK/32 dwords); slice u of the tile is the u-th dword of every
// lane, i.e. one MFMA.  K inside a tile is permuted identically for both operands.
//
// Work split.  A block holds up to 8 waves and stays resident: it stages X once, then walks
// groups of RB blocks of 16 output rows.  Each row block is shared by KS waves that split K
// into KS contiguous ranges of tiles (RB x KS waves per block); with KS > 1 the partial sums
// meet in LDS and one wave stores.  A wave keeps 32 dwords of packed weights per lane in
// flight.  Scales and zero points: with one group per tile (g <= 128) a lane loads the scales
// and zeros of a whole window of tiles at once, one window ahead, instead of two small loads
// per tile.
#include "q4_device.h"
#include "q4_internal.h"

namespace q4 {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kMaxWaves = 8;        // waves sharing one row block at most (K split), and
                                    // LDS slots for their partial sums
constexpr int kWideWaves = 16;      // waves per block of the lean (window) variant

// Four 32-bit registers of fp16 pairs (q - z) (x16 for odd positions) from 8 nibbles: a
// nibble OR-ed into the mantissa of fp16 1024.0 reads 1024 + q, and subtracting 1024 + z
// (1024 + 16 z for nibbles in bits 4..7) leaves q - z (16 (q - z)) exactly, so a weight whose
// code equals its zero point contributes exactly 0.  Slot order (k0, k4, k1, k5, k2, k6, k3,
// k7); X is staged in the same order with the factor 2^-4 on the slots that meet 16 (q - z).
template <bool SYM>
__device__ __forceinline__ f16x8 dequant_q_minus_z(uint32_t dw, uint32_t bias, f16x2 b1, f16x2 b16) {
  if (SYM) dw ^= 0x88888888u;                         // two's complement nibble -> q + 8
  const uint32_t d8 = dw >> 8;
  const f16x2 h0 = as_f16x2((dw & 0x000F000Fu) | bias) - b1;    // k0, k4
  const f16x2 h1 = as_f16x2((dw & 0x00F000F0u) | bias) - b16;   // k1, k5 (x16)
  const f16x2 h2 = as_f16x2((d8 & 0x000F000Fu) | bias) - b1;    // k2, k6
  const f16x2 h3 = as_f16x2((d8 & 0x00F000F0u) | bias) - b16;   // k3, k7 (x16)
  return f16x8{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// Maximum over each aligned group of L lanes (L = 4, 8 or 16, inside one 16-lane DPP row),
// returned to every lane of the group: DPP moves, no LDS round trips.
template <int L>
__device__ __forceinline__ float group_max(float v) {
  static_assert(L == 4 || L == 8 || L == 16, "4, 8 or 16 lanes");
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));   // quad_perm 1,0,3,2
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));   // quad_perm 2,3,0,1
  if (L >= 8) v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));  // row_half_mirror
  if (L >= 16) v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));  // row_mirror
  return v;
}

// The weights are read 64 bytes per row at a time, the rest of each line one tile later:
// plain loads keep the line in the cache for that second half.
template <int DPT>
__device__ __forceinline__ void load_dwords(uint32_t (&d)[DPT], const uint8_t* p) {
  if constexpr (DPT == 4) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
    d[0] = v[0]; d[1] = v[1]; d[2] = v[2]; d[3] = v[3];
  } else if constexpr (DPT == 2) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    d[0] = v[0]; d[1] = v[1];
  } else {
    d[0] = *reinterpret_cast<const uint32_t*>(p);
  }
}

size_t lds_tail(int64_t K, int g);
size_t lds_bytes(int64_t M, int64_t K, int g) { return (size_t)(2 * M * K) + lds_tail(K, g); }

// Bytes of LDS after the staged X: the 2^-e factors and the K-split partial sums.
size_t lds_tail(int64_t K, int g) {
  const int64_t TK = g < 128 ? g : 128;
  return (size_t)(64 * (K / TK)) + (size_t)kMaxWaves * kWave * 16;
}

// WIN: one group per tile, window loads of scales / zeros (needs aligned windows, see launch).
// MAXW: waves per block at most (the lean WIN variant fits 16 waves' registers).
template <int DPT, bool SYM, bool WIN, int MAXW>
__global__ __launch_bounds__(MAXW * kWave) void decode_kernel(
    const uint16_t* __restrict__ X, int M, int N, int K, int g,
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
    const uint8_t* __restrict__ zeros, uint16_t* __restrict__ Y, int RB, int KS) {
  constexpr int TK = 32 * DPT;
  constexpr int P = 32 / DPT;                   // tiles in flight per wave (32 dwords per lane)
  extern __shared__ u32x4 lds4[];
  const int T = K / TK;                         // tiles along K
  const int G = K / g;
  const int TPG = g / TK;                       // tiles per group
  const int MP = M;
  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int j = lane & 15, q = lane >> 4;
  const int NB = (N + 15) >> 4;

  u32x4* xs = lds4;                                                       // [T][DPT][4][MP]
  float* fx = reinterpret_cast<float*>(lds4 + (size_t)T * DPT * 4 * MP);  // [T][16]: 2^-e
  f32x4* red = reinterpret_cast<f32x4*>(fx + (size_t)T * 16);             // [waves][64]

  // This wave: row-block slot r of each group of RB row blocks, tiles [t_beg, t_end) of K.
  const int r = w / KS, part = w - r * KS;
  const int TPP = (T + KS - 1) / KS;
  const int t_beg = min(part * TPP, T), t_end = min(t_beg + TPP, T);
  const int NT = t_end - t_beg;
  const int NGR = (NB + RB - 1) / RB;
  const size_t rowbytes = (size_t)K >> 1;

  // Ring of P tiles.  Loads are unconditional, from clamped tiles (t <= t_end - 1): a load
  // under a branch would make the compiler wait for every load in flight before the next use.
  uint32_t wb[P][DPT];
  uint32_t sb[P], zb[P];
  const uint8_t* pr = packed;
  const uint16_t* sr = scales;
  const uint8_t* zr = zeros;
  int lt = 0, lg = 0, lgi = 0;
  auto load_next = [&](int i) {
    const int t = min(lt, t_end - 1);
    load_dwords<DPT>(wb[i], pr + (size_t)t * (TK / 2));
    if (!WIN) {
      const int gg = lt < t_end ? lg : (t_end - 1) / TPG;
      sb[i] = sr[gg];
      if (!SYM) zb[i] = zr[gg];
    }
    ++lt;
    if (++lgi == TPG) { lgi = 0; ++lg; }
  };
  // Windows (WIN): the scales / zeros of the P tiles (= P groups) of one chunk; the next
  // chunk's window is loaded at the start of the current one.
  constexpr int SW = WIN ? P / 2 : 1, ZW = WIN ? P / 4 : 1;
  uint32_t cs[SW], cz[ZW], ns[SW], nz[ZW];
  auto load_window = [&](uint32_t (&ds)[SW], uint32_t (&dz)[ZW], int c) {
    const int t = min(t_beg + c * P, t_end - P);
    const uint32_t* s4 = reinterpret_cast<const uint32_t*>(sr + t);
#pragma unroll
    for (int v = 0; v < SW; v += 4) {
      const u32x4 x4 = *reinterpret_cast<const u32x4*>(s4 + v);
      ds[v] = x4[0]; ds[v + 1] = x4[1]; ds[v + 2] = x4[2]; ds[v + 3] = x4[3];
    }
    if (!SYM) {
      const uint32_t* z4 = reinterpret_cast<const uint32_t*>(zr + t);
      if constexpr (ZW == 2) {
        const u32x2 x2 = *reinterpret_cast<const u32x2*>(z4);
        dz[0] = x2[0]; dz[1] = x2[1];
      } else {
#pragma unroll
        for (int v = 0; v < ZW; v += 4) {
          const u32x4 x4 = *reinterpret_cast<const u32x4*>(z4 + v);
          dz[v] = x4[0]; dz[v + 1] = x4[1]; dz[v + 2] = x4[2]; dz[v + 3] = x4[3];
        }
      }
    }
  };
  // Point the ring at row block nb = gi RB + r and request its first P tiles (wave-uniform).
  auto begin_group = [&](int gi) {
    const int nb = gi * RB + r;
    if (nb < NB && NT > 0) {
      // Rows past N (ragged last block) read row N - 1; their outputs are not stored.
      const int n = min(nb * 16 + j, N - 1);
      pr = packed + (size_t)n * rowbytes + q * (TK / 8);
      sr = scales + (size_t)n * G;
      zr = zeros + (size_t)n * G;
      lt = t_beg;
      lg = t_beg / TPG;
      lgi = t_beg - lg * TPG;
      if (WIN) load_window(cs, cz, 0);
#pragma unroll
      for (int i = 0; i < P; ++i) load_next(i);
    }
  };

  // The first group's weights are requested before X is staged, so that HBM latency overlaps
  // the staging.
  if (blockIdx.x < NGR) begin_group(blockIdx.x);

  // ---- X -> LDS: TK/8 threads per (m, tile) of the M rows, one octet of 8 values each, four
  // octets per thread in flight; rows M..15 get the factor 0. ----
  constexpr int OPT = TK / 8;                 // octets per tile
  for (int u0 = tid; u0 < T * (16 - MP); u0 += nthreads) fx[(u0 % T) * 16 + MP + u0 / T] = 0.0f;
  const int total = MP * T * OPT;             // a multiple of OPT: lanes leave the loop in whole groups
  for (int base = tid; base < total; base += 4 * nthreads) {
    u32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u0 = min(base + i * nthreads, total - 1);
      const int o = u0 & (OPT - 1);
      const int mt = u0 / OPT;
      const int m = mt / T, t = mt - m * T;
      v[i] = *reinterpret_cast<const u32x4*>(X + (size_t)m * K + (size_t)t * TK + 8 * o);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u0 = base + i * nthreads;     // uniform per aligned group of OPT lanes
      const int o = u0 & (OPT - 1);           // octet o = q DPT + u covers k = t TK + 8 o
      const int mt = u0 / OPT;
      const int m = mt / T, t = mt - m * T;
      float amax = 0.0f;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(v[i][c])), fabsf(bf16_hi(v[i][c]))));
      amax = group_max<OPT>(amax);            // aligned groups of OPT lanes = one (m, tile)
      int e = 0;
      if (amax > 0.0f) {
        int E;
        frexpf(amax, &E);
        e = min(15 - E, 100);                 // amax * 2^e in [2^14, 2^15)
      }
      if (u0 < total) {
        const u32x4 w = v[i];
        const f16x2 p0 = {(_Float16)ldexpf(bf16_lo(w[0]), e), (_Float16)ldexpf(bf16_lo(w[2]), e)};
        const f16x2 p1 = {(_Float16)ldexpf(bf16_hi(w[0]), e - 4), (_Float16)ldexpf(bf16_hi(w[2]), e - 4)};
        const f16x2 p2 = {(_Float16)ldexpf(bf16_lo(w[1]), e), (_Float16)ldexpf(bf16_lo(w[3]), e)};
        const f16x2 p3 = {(_Float16)ldexpf(bf16_hi(w[1]), e - 4), (_Float16)ldexpf(bf16_hi(w[3]), e - 4)};
        const int kq = o / DPT, u = o - kq * DPT;
        xs[((size_t)(t * DPT + u) * 4 + kq) * MP + m] = u32x4{as_u32(p0), as_u32(p1), as_u32(p2), as_u32(p3)};
        if (o == 0) fx[t * 16 + m] = ldexpf(1.0f, -e);
      }
    }
  }
  __syncthreads();

  uint32_t bias = 0x64006400u;
  asm volatile("" : "+v"(bias));   // keep in a VGPR: (x & mask) | bias -> one v_and_or_b32
  const int jx = min(j, MP - 1);

  for (int gi = blockIdx.x; gi < NGR; gi += gridDim.x) {            // block-uniform
    if (gi != (int)blockIdx.x) begin_group(gi);
    const int nb = gi * RB + r;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (nb < NB && NT > 0) {                                          // wave-uniform
      for (int t0 = 0; t0 < NT; t0 += P) {
        if (WIN) load_window(ns, nz, t0 / P + 1);
#pragma unroll
        for (int i = 0; i < P; ++i) {
          const int t = t_beg + t0 + i;
          if (WIN || t < t_end) {             // wave-uniform; WIN: NT is a multiple of P
            uint32_t z, sbits;
            if (WIN) {
              sbits = (cs[i >> 1] >> (16 * (i & 1))) & 0xffffu;
              z = SYM ? 8u : (cz[i >> 2] >> (8 * (i & 3))) & 0xffu;
            } else {
              sbits = sb[i];
              z = SYM ? 8u : zb[i];
            }
            const f16x2 b1 = as_f16x2((0x6400u + z) * 0x00010001u);
            const f16x2 b16 = as_f16x2((0x6400u + 16u * z) * 0x00010001u);
            f32x4 pacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < DPT; ++u) {
              const f16x8 bw = dequant_q_minus_z<SYM>(wb[i][u], bias, b1, b16);
              // rows j >= M read row M - 1: their results land in rows that are never stored
              const f16x8 ax = __builtin_bit_cast(f16x8, xs[((size_t)(t * DPT + u) * 4 + q) * MP + jx]);
              pacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ax, bw, pacc, 0, 0, 0);
            }
            const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)sbits);
            const f32x4 f = *reinterpret_cast<const f32x4*>(fx + t * 16 + 4 * q);   // 2^-e, rows 4q..4q+3
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) acc[rr] = __builtin_fmaf(pacc[rr], s * f[rr], acc[rr]);
          }
          load_next(i);
        }
        if (WIN) {
#pragma unroll
          for (int v = 0; v < SW; ++v) cs[v] = ns[v];
#pragma unroll
          for (int v = 0; v < ZW; ++v) cz[v] = nz[v];
        }
      }
    }
    if (KS > 1) {                                                     // block-uniform
      // Parts 1..KS-1 of row-block slot r leave their sums in slots r (KS - 1) + part - 1
      // (RB (KS - 1) <= kMaxWaves of them); part 0 adds them in part order.
      if (part > 0) red[(r * (KS - 1) + part - 1) * kWave + lane] = acc;
      __syncthreads();
      if (part == 0) {
#pragma unroll 1
        for (int pp = 1; pp < KS; ++pp) acc += red[(r * (KS - 1) + pp - 1) * kWave + lane];
      }
      __syncthreads();
    }
    // lane (j, q): rows m = 4 q + rr of output column 16 nb + j
    const int ncol = nb * 16 + j;
    if (part == 0 && nb < NB && ncol < N) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int m = 4 * q + rr;
        if (m < MP) Y[(size_t)m * N + ncol] = f32_to_bf16_bits(acc[rr]);
      }
    }
  }
}

template <int DPT, bool SYM>
hipError_t launch_cfg(const void* X, int M, int64_t N, int64_t K, int g, const void* packed,
                      const void* scales, const void* zeros, void* Y, int num_cus, hipStream_t stream) {
  constexpr int TK = 32 * DPT, P = 32 / DPT;
  const size_t lds = lds_bytes(M, K, g);
  // More than 64 KiB of dynamic LDS has to be enabled per kernel (thread-safe one-time init).
  static const hipError_t attr = [] {
    const void* kernels[] = {reinterpret_cast<const void*>(&decode_kernel<DPT, SYM, true, kWideWaves>),
                             reinterpret_cast<const void*>(&decode_kernel<DPT, SYM, true, kMaxWaves>),
                             reinterpret_cast<const void*>(&decode_kernel<DPT, SYM, false, kMaxWaves>)};
    for (const void* k : kernels) {
      const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }();
  if (attr != hipSuccess) return attr;
  const int64_t NB = (N + 15) / 16;
  const int64_t T = K / TK;
  const int64_t G = K / g;
  // Row blocks per resident block (RB) and waves splitting each one's K (KS), for a block of at
  // most maxw waves: with fewer row blocks than waves, the spare waves split K, at most
  // kMaxWaves ways, with at most kMaxWaves partial sums in LDS.
  auto split = [&](int maxw, int& RB, int& KS) {
    const int64_t rb = (NB + num_cus - 1) / num_cus;
    if (rb >= maxw) {
      RB = maxw;
      KS = 1;
      return;
    }
    RB = (int)rb;
    KS = min(maxw / RB, kMaxWaves);
    while (KS > 1 && (T % KS != 0 || T / KS < 2 || RB * (KS - 1) > kMaxWaves)) --KS;
  };
  // Window loads: one group per tile, every wave's tile range a whole number of windows, and
  // 4-byte-aligned windows of scales and zeros in every row.
  auto windows = [&](int KS) {
    return (g == TK) && ((T / KS) % P == 0) && (T % KS == 0) && (G % (P < 16 ? P : 16) == 0);
  };
  int RB, KS;
  split(kWideWaves, RB, KS);
  const bool wide = windows(KS);
  if (!wide) split(kMaxWaves, RB, KS);
  const bool win = wide || windows(KS);
  const int64_t groups = (NB + RB - 1) / RB;
  const int64_t blocks = groups < num_cus ? groups : num_cus;
  const int threads = RB * KS * kWave;
#define Q4_DECODE_LAUNCH(WINV, MAXWV)                                                              \
  hipLaunchKernelGGL((decode_kernel<DPT, SYM, WINV, MAXWV>), dim3((unsigned)blocks), dim3((unsigned)threads), \
                     lds, stream, (const uint16_t*)X, M, (int)N, (int)K, g, (const uint8_t*)packed,          \
                     (const uint16_t*)scales, (const uint8_t*)zeros, (uint16_t*)Y, RB, KS)
  if (wide) Q4_DECODE_LAUNCH(true, kWideWaves);
  else if (win) Q4_DECODE_LAUNCH(true, kMaxWaves);
  else Q4_DECODE_LAUNCH(false, kMaxWaves);
#undef Q4_DECODE_LAUNCH
  return hipGetLastError();
}

template <bool SYM>
hipError_t launch_mode(const void* X, int M, int64_t N, int64_t K, int g, const void* packed,
                       const void* scales, const void* zeros, void* Y, int num_cus, hipStream_t stream) {
  if (g == 32) return launch_cfg<1, SYM>(X, M, N, K, g, packed, scales, zeros, Y, num_cus, stream);
  if (g == 64) return launch_cfg<2, SYM>(X, M, N, K, g, packed, scales, zeros, Y, num_cus, stream);
  return launch_cfg<4, SYM>(X, M, N, K, g, packed, scales, zeros, Y, num_cus, stream);
}

}  // namespace

size_t decode_lds_bytes(int64_t M, int64_t K, int g) { return lds_bytes(M, K, g); }

bool decode_fits(int64_t M, int64_t N, int64_t K, int g) {
  (void)N;
  if (M < 1 || M > 16) return false;
  if (!(g == 32 || g == 64 || g % 128 == 0)) return false;
  return decode_lds_bytes(M, K, g) <= 160 * 1024;
}

hipError_t launch_decode(const void* X, int M, int64_t N, int64_t K, int g, bool sym,
                         const void* packed, const void* scales, const void* zeros, void* Y,
                         int num_cus, hipStream_t stream) {
  return sym ? launch_mode<true>(X, M, N, K, g, packed, scales, zeros, Y, num_cus, stream)
             : launch_mode<false>(X, M, N, K, g, packed, scales, zeros, Y, num_cus, stream);
}

}  // namespace q4
