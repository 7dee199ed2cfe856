// W4A16 decode for 1 <= M <= 16 on the matrix cores of gfx950 (v_mfma_f32_16x16x32).
//
// W4A16: 4-bit weights dequantised inside the kernel, products on 16-bit operands
// ("LLM Weight Quantization - GPTQ, AWQ, SmoothQuant, FP8 & INT4/INT8 Trade-offs",
// "The vocabulary"); decode reads every weight once and is bound by HBM ("Overview").
// Dequantisation x_hat = scale * (q - z) ("DL S067 · Quantization", §1), groups of g weights
// along K ("Model Quantization", §1).
//
// Roles.  D[m][n] = sum_k A[m][k] B[k][n] with A = X (16 token slots m) and B = (q - z) of 16 W
// rows n.  Lane l holds A row m = l % 16 and B column n = l % 16, eight k values of the
// quarter kq = l / 16, and D rows 4 (l / 16) .. + 3 of column n.
//
// Work split.  A workgroup (one per compute unit, persistent) walks 16-row blocks of W.  Its WS
// waves split K: wave w owns the K range [v KR, (v + 1) KR), v = (w + workgroup) mod WS.  A
// wave keeps its X range in registers for the whole kernel (the A operand of every row block)
// and streams its W range of each row block through LDS; the WS partial sums of a row block
// meet in LDS in wave order.  The X range arrives through the wave's own stage area before any
// stage is requested: 1 KiB copies of whole lines, then one LDS read per slice, instead of lane
// loads that request every line four times (70B-shaped layer at M = 4 / 8 / 16: 27.2 / 29.1 /
// 32.9 -> 25.8 / 26.6 / 30.0 us; 4096 x 4096 at M = 16: 8.7 -> 7.1 us).
// With M <= 8 (or <= 4) tokens, the 16 token slots carry P = 2 (or 4) parts of the wave's
// K range: slot m holds token m % (16 / P) of part m / (16 / P), and part p's weights go to
// their own accumulator, whose rows of part p are the only ones kept.  So the same registers
// cover a P times longer K range.
//
// Loads.  Each 1 KiB LDS-DMA instruction reads 4 rows x 256 contiguous bytes of codes
// (requests of whole cache lines and more per row: as fast as contiguous streaming), written
// to LDS with the 16-byte chunk c of row r at position (c ^ r) within its row, so that the
// fragment reads of 16 rows at one chunk hit 16 distinct bank groups.  A wave keeps S stages
// in flight and waits for the oldest with an explicit vmcnt: every global load of the main
// loop is one of these LDS-DMA copies.
// Scales and zero-points: each wave copies its groups of the stage's 16 rows into the stage
// (one dword per lane, 16 rows x a few bytes: small scattered requests).  SH form, when a
// workgroup has two row blocks or more and the LDS allows: a row block's scales and
// zero-points are one contiguous range of each array (16 rows x K/g groups), and the
// workgroup copies the whole range into an LDS slot shared by its waves, wave w the w-th of
// WS equal pieces, instead.  The copies for a row block ride with the stage of the row block
// before it, so the barrier that ends that row block (every wave has waited for its stage by
// then) makes the whole range visible; S + 2 slots cover the row blocks in flight.  (70B-shaped
// layer, M = 4 / 8 / 16: 28.1-28.8 / 29.8-30.1 / 33.8-34.1 -> 26.9 / 29.2-29.7 / 32.9-33.3 us;
// with one row block per workgroup, as in the 4096 x 4096 layer, the first range's barrier
// cost more than it saved: 8.7 -> 9.4 us.)
//
// Arithmetic (fast path, exact up to fp32 summation and the final bf16 rounding):
//   * (q - z) is formed exactly in fp16: the nibble OR-ed into the mantissa of 1024.0, minus
//     1024 + z (nibbles in bits 4..7 give 16 (q - z));
//   * X is converted to fp16 exactly after scaling each (token, part) by a power of two 2^e
//     that puts its largest |x| in [2^14, 2^15); the positions that meet a 16 (q - z) weight
//     carry 2^(e - 4);
//   * the MFMA takes exact products and sums them in fp32; each tile's sum is multiplied by its
//     group's scale and accumulated in fp32; 2^-e is applied once per row block.
// The fp16 conversion is exact only while every nonzero |x| 2^(e-4) of the part is at least
// 2^-14 (the matrix cores flush fp16 subnormal inputs).  A wave whose X range has a smaller
// element (a dynamic range above about 2^24 inside one part) runs the exact path instead:
// X and (q - z) as bf16 (exact: bf16 holds 8 significant bits, (q - z) needs 4, 16 (q - z) 8),
// the bf16 matrix instruction, and no power-of-two scaling.
#include <utility>

#include "q4_device.h"
#include "q4_internal.h"

namespace q4 {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxWaves = 8;
constexpr size_t kLdsMax = 160 * 1024;
constexpr int kRedBytes = 1024;          // one f32x4 per lane: a wave's partial of a row block

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most k * L of this wave's vector memory operations are outstanding (k <= 3;
// the launch keeps (S - 1) L <= 63, the counter's range).
template <int L>
__device__ __forceinline__ void wait_stages(int k) {
  constexpr int L2 = 2 * L <= 63 ? 2 * L : 63, L3 = 3 * L <= 63 ? 3 * L : 63;
  if (k <= 0) wait_vm<0>();
  else if (k == 1) wait_vm<L>();
  else if (k == 2) wait_vm<L2>();
  else wait_vm<L3>();
}

// f(0), f(1), ..., f(N - 1) with compile-time arguments: straight-line code that does not
// depend on the unroller's size limits.
template <typename F, int... I>
__device__ __forceinline__ void for_each_index(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS-DMA copies through a buffer resource (an offset at or past the resource's end reads 0):
// 16 bytes per lane, non-temporal, lane i writing LDS bytes [lds + 16 i, + 16); or 4 bytes per
// lane, lane i writing [lds + 4 i, + 4).  The address is the resource base + voff + soff.
__device__ __forceinline__ void dma16(u32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen nt lds" ::"v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds)
               : "memory");
}
// The same without the non-temporal hint, for X (which every workgroup reads).
__device__ __forceinline__ void dma16x(u32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds)
               : "memory");
}
__device__ __forceinline__ void dma4(u32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("buffer_load_dword %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds)
               : "memory");
}

__device__ __forceinline__ u32x4 buffer_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes), (uint32_t)kBufferFlags};
}

// Eight fp16 (q - z) from 8 nibbles (one dword of codes): nibble OR-ed into 1024.0 minus
// 1024 + z (1024 + 16 z for nibbles in bits 4..7).  Slot order (k0, k4, k1, k5, k2, k6, k3,
// k7); the odd k carry 16 (q - z).
template <bool SYM>
__device__ __forceinline__ f16x8 dequant_f16(uint32_t dw, uint32_t bias, f16x2 b1, f16x2 b16) {
  if (SYM) dw ^= 0x88888888u;                         // two's complement nibble -> q + 8
  const uint32_t d8 = dw >> 8;
  const f16x2 h0 = as_f16x2((dw & 0x000F000Fu) | bias) - b1;
  const f16x2 h1 = as_f16x2((dw & 0x00F000F0u) | bias) - b16;
  const f16x2 h2 = as_f16x2((d8 & 0x000F000Fu) | bias) - b1;
  const f16x2 h3 = as_f16x2((d8 & 0x00F000F0u) | bias) - b16;
  return f16x8{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// The same eight values as bf16 (small integers: exact).
__device__ __forceinline__ bf16x8 to_bf16(f16x8 h) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)(float)h[i];
  return r;
}

// Stage geometry of one wave: 16 rows of KR weights (codes), and either its groups' scales
// and zero-points of those rows or (SH) its piece of the next row block's (KR / g groups of
// 16 rows: the range's WS-th part, copied to the shared slot).
template <int P, int NSL, int TK, bool SYM, bool SH>
struct Geo {
  static constexpr int MP = 16 / P;                  // token slots per part
  static constexpr int PW = NSL * 32;                // k per part
  static constexpr int KR = P * PW;                  // k per wave
  static constexpr int RBY = KR / 2;                 // code bytes per row per stage
  static constexpr int SEG = RBY / 256;              // 256-byte segments per row
  static constexpr int NCI = 4 * SEG;                // 1 KiB code copies per stage
  static constexpr int NG = KR / TK;                 // groups (= tiles) per row per stage
  static constexpr int NSI = (8 * NG + 63) / 64;     // scale dword copies (64 dwords each)
  static constexpr int NZI = SYM ? 0 : (4 * NG + 63) / 64;
  static constexpr int L = NCI + NSI + NZI;          // vector memory operations per stage
  static constexpr uint32_t SOFF = 16u * RBY;        // scales inside the stage (not SH)
  static constexpr uint32_t ZOFF = SOFF + 256u * NSI;
  static constexpr uint32_t STAGE = SH ? SOFF : ZOFF + 256u * NZI;   // LDS bytes of one stage
  static constexpr int DPT = TK / 32;                // dwords per lane per tile
  static constexpr int TPP = PW / TK;                // tiles per part
  static_assert(RBY % 256 == 0, "whole 256-byte segments per row");
  static_assert(NG >= 4 && (NG & (NG - 1)) == 0, "at least four groups per stage");
  static_assert(L <= 63, "one stage's copies fit vmcnt");
};

// At most 8 waves per workgroup: two waves per SIMD, 256 registers each (the X range takes 64).
template <int P, int NSL, int TK, bool SYM, bool SH>
__global__ __launch_bounds__(8 * 64) void decode_kernel(
    const uint16_t* __restrict__ X, int M, int N, int K, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros, uint16_t* __restrict__ Y,
    int S) {
  using Gm = Geo<P, NSL, TK, SYM, SH>;
  constexpr int MP = Gm::MP, DPT = Gm::DPT, KR = Gm::KR, NG = Gm::NG;
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int WS = blockDim.x / kWave;
  const int m = lane & 15, kq = lane >> 4;           // A row / B column, k quarter
  const int G = K / TK;                              // groups per row (g = TK)
  const int NB = (N + 15) >> 4;
  // the waves' K ranges rotate with the workgroup, so that the workgroups starting together on
  // one chip region request different parts of X first
  const int K0 = ((w + (int)blockIdx.x) % WS) * KR;
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  const uint32_t my_stages = lds0 + (uint32_t)(w * S) * Gm::STAGE;
  // SH: shared slots of a row block's scales (32 G bytes) then zero-points (16 G), S + 2 of them
  const uint32_t slot_bytes = 32u * (uint32_t)G + (SYM ? 0u : 16u * (uint32_t)G);
  const int NSLOT = SH ? S + 2 : 0;
  const uint32_t sh0 = (uint32_t)(WS * S) * Gm::STAGE;                // offset in lds
  const uint32_t red0 = lds0 + sh0 + (uint32_t)NSLOT * slot_bytes;

  // ---- X range -> registers: slot m = (part, token), slices s = (tile, dword) ----
  const int part = m / MP, tok = m % MP;
  const __amdgpu_buffer_rsrc_t rx = buffer_over(X, (uint32_t)M * (uint32_t)K * 2u);
  u32x4 xr[NSL];
  // X goes through the wave's own stage area before it holds a stage: 1 KiB copies of whole
  // lines, then one LDS read per slice.  The 16 token slots (part, token) of HS = min(NSL, 16)
  // slices each, 64 HS bytes a slot, are copied at a time (a copy covers 1024 / (64 HS)
  // slots; the chunk at position p of slot r's row holds chunk p ^ (r % 16) of its X, so that
  // 16 slots' reads of one chunk hit distinct banks).  Loaded straight into registers, each
  // 16-byte lane load would touch two lines per token and every line would be requested by four
  // instructions.
  constexpr int HS = NSL < 16 ? NSL : 16;               // slices per pass
  constexpr uint32_t RB = 64u * HS;                      // bytes of one slot per pass
  bool xlds = false;
  if constexpr (HS >= 8) xlds = (uint32_t)S * Gm::STAGE >= 16u * RB;   // wave-uniform
  if (xlds) {
    if constexpr (HS >= 8) {
      const u32x4 rxw = buffer_words(X, (uint32_t)M * (uint32_t)K * 2u);
#pragma unroll
      for (int h = 0; h < NSL / HS; ++h) {
        if (h > 0) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the area's reads are done
#pragma unroll
        for (int i = 0; i < (int)(16 * RB / 1024); ++i) {
          const uint32_t at = 1024u * (uint32_t)i + 16u * (uint32_t)lane;   // this lane's bytes
          const uint32_t r = at / RB, p = (at % RB) / 16u;                  // slot, chunk position
          const uint32_t tk = r % (uint32_t)MP, pt = r / (uint32_t)MP;
          dma16x(rxw, 2u * (tk * (uint32_t)K + (uint32_t)K0 + pt * (uint32_t)Gm::PW + (uint32_t)(HS * 32 * h)) +
                          16u * (p ^ (r & 15u)), 0u, my_stages + 1024u * (uint32_t)i);
        }
        wait_vm<0>();
#pragma unroll
        for (int s2 = 0; s2 < HS; ++s2) {
          const int j = s2 / DPT, u = s2 % DPT;
          const int c = j * (TK / 8) + kq * (TK / 32) + u;                 // chunk of the pass
          xr[HS * h + s2] = *reinterpret_cast<const u32x4*>(lds + (my_stages - lds0) + RB * (uint32_t)m +
                                                            16u * (uint32_t)(c ^ m));
        }
      }
      if constexpr (P > 1) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // before the first stage
    }
  } else {
#pragma unroll
    for (int s = 0; s < NSL; ++s) {
      const int j = s / DPT, u = s % DPT;
      const int k = K0 + part * Gm::PW + j * TK + kq * (TK / 4) + 8 * u;
      xr[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rx, 2u * ((uint32_t)tok * (uint32_t)K + (uint32_t)k), 0, 0));
    }
  }
  // ---- stage copies ----
  // Each row block's copies go through resources based at its first row and this wave's K
  // range, holding the bytes up to the end of the matrix: rows past N then lie past the
  // resource's end and read as 0.  The range check covers the vector offset only, so every
  // row offset goes there; the scalar offset carries the 256-byte segment inside the row.
  // Codes: copy i covers rows 4 (i % 4) + lane / 16 and the 256-byte segment i / 4; lane l
  // reads chunk (l % 16) ^ row of it, i.e. the chunk bits XOR 64 (i % 4) bytes (rows are a
  // multiple of 256 bytes long).
  const uint32_t rowbytes = (uint32_t)K / 2u;
  const uint32_t code_lane = (uint32_t)(lane >> 4) * rowbytes + 16u * (uint32_t)((lane & 15) ^ (lane >> 4));
  uint32_t cv[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) cv[q] = (code_lane ^ (64u * (uint32_t)q)) + 4u * (uint32_t)q * rowbytes;
  // not SH: scales: dword d = 64 q + l of the stage is dword d % (NG / 2) of row d / (NG / 2);
  // zeros: dword d % (NG / 4) of row d / (NG / 4) (rows past 15 are padding and land past the
  // stage's 16 rows in LDS)
  uint32_t sv[Gm::NSI], zv[Gm::NZI > 0 ? Gm::NZI : 1];
  if constexpr (!SH) {
#pragma unroll
    for (int q = 0; q < Gm::NSI; ++q)
      sv[q] = (uint32_t)(q * (128 / NG) + lane / (NG / 2)) * (uint32_t)G * 2u + 4u * (uint32_t)(lane % (NG / 2));
#pragma unroll
    for (int q = 0; q < Gm::NZI; ++q)
      zv[q] = (uint32_t)(q * (256 / NG) + lane / (NG / 4)) * (uint32_t)G + 4u * (uint32_t)(lane % (NG / 4));
  }
  // SH: scales and zero-points of row block rb into shared slot j: this wave's piece, 32 NG bytes
  // of scales and 16 NG of zero-points at piece w of each range (lanes past the piece idle, so
  // that no lane writes into another wave's piece; every copy keeps its first 16 lanes).
  // Pieces past the end of the arrays read as 0 (resources end at the arrays' ends; none for
  // rb >= NB, whose slot is never read: the copy is still issued, so that every stage holds L
  // copies).
  auto issue_sz = [&](int rb, int j) {
    const uint32_t total = (uint32_t)N * (uint32_t)G;                // groups in the arrays
    const uint32_t gp = (uint32_t)min(rb, NB) * 16u * (uint32_t)G + (uint32_t)(w * 16 * NG);   // piece start
    const uint32_t left = gp < total ? total - gp : 0u;
    const uint32_t dst = lds0 + sh0 + (uint32_t)j * slot_bytes;
    const u32x4 rs = buffer_words(scales + (gp < total ? gp : 0u), min(left, 16u * (uint32_t)NG) * 2u);
#pragma unroll
    for (int q = 0; q < Gm::NSI; ++q)
      if (256 * q + 4 * lane < 32 * NG) dma4(rs, 256u * (uint32_t)q + 4u * (uint32_t)lane, 0u, dst + (uint32_t)(w * 32 * NG + 256 * q));
    if constexpr (!SYM) {
      const u32x4 rz = buffer_words(zeros + (gp < total ? gp : 0u), min(left, 16u * (uint32_t)NG));
#pragma unroll
      for (int q = 0; q < Gm::NZI; ++q)
        if (256 * q + 4 * lane < 16 * NG)
          dma4(rz, 256u * (uint32_t)q + 4u * (uint32_t)lane, 0u, dst + 32u * (uint32_t)G + (uint32_t)(w * 16 * NG + 256 * q));
    }
  };
  // stage j (row block rb, the j-th of this workgroup): codes, then the row block's scales and
  // zero-points of this wave's groups (SH: the next row block's piece)
  auto issue = [&](int slot, int rb, int j) {
    const uint32_t st = my_stages + (uint32_t)slot * Gm::STAGE;
    const uint32_t n0 = (uint32_t)rb * 16u;                          // rb < NB
    const u32x4 rw = buffer_words(packed + (size_t)n0 * rowbytes + (size_t)(K0 / 2),
                                  ((uint32_t)N - n0) * rowbytes - (uint32_t)(K0 / 2));
#pragma unroll
    for (int i = 0; i < Gm::NCI; ++i) dma16(rw, cv[i & 3], 256u * (uint32_t)(i >> 2), st + 1024u * (uint32_t)i);
    if constexpr (SH) {
      issue_sz(rb + (int)gridDim.x, (j + 1) % NSLOT);
    } else {
      const uint32_t g0 = n0 * (uint32_t)G + (uint32_t)(K0 / TK);    // first group of the range
      const u32x4 rs = buffer_words(scales + g0, ((uint32_t)N * (uint32_t)G - g0) * 2u);
      const u32x4 rz = buffer_words(zeros + g0, SYM ? 0u : (uint32_t)N * (uint32_t)G - g0);
#pragma unroll
      for (int q = 0; q < Gm::NSI; ++q) dma4(rs, sv[q], 0u, st + Gm::SOFF + 256u * (uint32_t)q);
#pragma unroll
      for (int q = 0; q < Gm::NZI; ++q) dma4(rz, zv[q], 0u, st + Gm::ZOFF + 256u * (uint32_t)q);
    }
  };

  // With two or four parts the first stage is requested right behind X (the conversion of X
  // below waits for it too: loads complete in order) and the others after the conversion;
  // with one part (M > 8, whose X range is 32 or 64 KB per wave) every stage once X has
  // arrived: X does not queue behind them (70B-shaped layer, M = 4 / 8 / 16: 29.0 / 31.9 /
  // 42.5 -> 28.3 / 30.0 / 37.8-39.1 us, config 3 9.9 -> 9.2 us)
  const int stride = gridDim.x;
  constexpr int EARLY = P == 1 ? 0 : 1;
  // SH: the first row block's scales and zero-points ahead of its stage (loads complete in
  // order)
  if constexpr (SH && EARLY > 0) issue_sz((int)blockIdx.x, 0);
  for (int s = 0; s < min(S, EARLY); ++s)
    if ((int)blockIdx.x + s * stride < NB) issue(s, (int)blockIdx.x + s * stride, s);

  // The range of |x| is taken on the bf16 bit patterns (their order as unsigned 16-bit integers
  // is the order of the values), two at a time; the smallest nonzero one as the smallest of
  // bits - 1 (zero wraps to the largest).
  u16x2 hi = {0, 0}, lo = {0xffff, 0xffff};
#pragma unroll
  for (int s = 0; s < NSL; ++s)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u16x2 a = __builtin_bit_cast(u16x2, xr[s][c] & 0x7fff7fffu);
      hi = __builtin_elementwise_max(hi, a);
      lo = __builtin_elementwise_min(lo, a - u16x2{1, 1});
    }
  int amax_b = hi[0] > hi[1] ? hi[0] : hi[1];
  int amin_b1 = lo[0] < lo[1] ? lo[0] : lo[1];                     // 0xffff: no nonzero x
  // the part of one token is spread over the four quarters kq: lanes m, m + 16, m + 32, m + 48
  amax_b = max(amax_b, __shfl_xor(amax_b, 16));
  amax_b = max(amax_b, __shfl_xor(amax_b, 32));
  amin_b1 = min(amin_b1, __shfl_xor(amin_b1, 16));
  amin_b1 = min(amin_b1, __shfl_xor(amin_b1, 32));
  const float amax = __uint_as_float((uint32_t)amax_b << 16);
  int e = 0;
  if (amax > 0.0f) e = min(15 - __builtin_amdgcn_frexp_expf(amax), 126);   // amax 2^e in [2^14, 2^15)
  // exact in fp16 (normal, as the matrix cores need) iff every nonzero |x| 2^(e-4) >= 2^-14
  const bool lossy = amin_b1 != 0xffff && __builtin_ldexpf(__uint_as_float((uint32_t)(amin_b1 + 1) << 16), e) < 0x1p-10f;
  const bool exact = __builtin_amdgcn_ballot_w64(lossy) != 0;              // wave-uniform
  const float my_fac = exact ? 1.0f : __builtin_ldexpf(1.0f, -e);
  // one part: the stages are requested now that X is here, so that the conversion below
  // overlaps their latency (M = 16: 35.0 -> 33.9 us; config 3 8.8 -> 8.7 us)
  if constexpr (P == 1) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // X's reads of the stage area are done
    if constexpr (SH) issue_sz((int)blockIdx.x, 0);
    for (int s = 0; s < S; ++s)
      if ((int)blockIdx.x + s * stride < NB) issue(s, (int)blockIdx.x + s * stride, s);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int s = 0; s < NSL; ++s) {
    const u32x4 v = xr[s];
    // k0..k7 = lo/hi halves of v[0..3]; slots (k0, k4, k1, k5, k2, k6, k3, k7), odd k x 2^-4
    const float x[8] = {bf16_lo(v[0]), bf16_hi(v[0]), bf16_lo(v[1]), bf16_hi(v[1]),
                        bf16_lo(v[2]), bf16_hi(v[2]), bf16_lo(v[3]), bf16_hi(v[3])};
    const int ord[8] = {0, 4, 1, 5, 2, 6, 3, 7};
    uint32_t o[4];
    if (!exact) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k0 = ord[2 * q], k1 = ord[2 * q + 1];
        const f16x2 h = {(_Float16)__builtin_ldexpf(x[k0], (k0 & 1) ? e - 4 : e),
                         (_Float16)__builtin_ldexpf(x[k1], (k1 & 1) ? e - 4 : e)};
        o[q] = as_u32(h);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k0 = ord[2 * q], k1 = ord[2 * q + 1];
        o[q] = pack_bf16x2((k0 & 1) ? x[k0] * 0.0625f : x[k0], (k1 & 1) ? x[k1] * 0.0625f : x[k1]);
      }
    }
    xr[s] = u32x4{o[0], o[1], o[2], o[3]};
  }

  if constexpr (P > 1)
    for (int s = EARLY; s < S; ++s)
      if ((int)blockIdx.x + s * stride < NB) issue(s, (int)blockIdx.x + s * stride, s);

  // fragment reads: B column n = m (row of the block), quarter kq
  const int n = m;
  uint32_t bias = 0x64006400u;
  asm volatile("" : "+v"(bias));   // keep in a VGPR: (x & mask) | bias -> one v_and_or_b32

  auto run = [&](auto exact_tag) {
    constexpr bool EX = decltype(exact_tag)::value;
    int it = 0;
    for (int rb = blockIdx.x; rb < NB; rb += stride, ++it) {          // block-uniform
      const int slot = it % S;
      const int later = min(S - 1, (NB - 1 - rb) / stride);           // stages issued after this one
      wait_stages<Gm::L>(later);
      // SH: the first row block's scales and zero-points came before any stage: once every
      // wave has waited for its first stage they are all in LDS (later ones: the previous row
      // block's closing barrier)
      if (SH && it == 0) lds_barrier();
      const uint32_t st = my_stages + (uint32_t)slot * Gm::STAGE;
      // this row block's scales and zero-points: row n's groups from the wave's first one
      const uint32_t shs = sh0 + (uint32_t)(it % NSLOT) * slot_bytes;
      const uint32_t gn = (uint32_t)(n * G + K0 / TK);
      // One part at a time: its accumulator collects the part's tiles, then the lanes whose D rows
      // belong to that part (4 kq / MP == p) keep it.  The tiles are generated at compile time
      // (a fold over an index sequence), so every X register index is a constant.
      f32x4 res = {0.f, 0.f, 0.f, 0.f};
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      auto tile = [&](auto tc) {
        constexpr int t = decltype(tc)::value;
        constexpr int p = t / Gm::TPP, j = t % Gm::TPP;
        if constexpr (j == 0) acc = f32x4{0.f, 0.f, 0.f, 0.f};
        // codes of tile t, row n, quarter kq: bytes t TK/2 + kq TK/8 of the row's stage range
        const int byte = t * (TK / 2) + kq * (TK / 8);
        const int c = byte >> 4;
        const uint32_t pos = (uint32_t)((c >> 4) * 256 + n * 16 + ((c & 15) ^ n));
        const uint32_t off = (st - lds0) + 16u * pos + (uint32_t)(byte & 15);
        uint32_t dw[DPT];
        if constexpr (DPT == 4) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(lds + off);
          dw[0] = v[0]; dw[1] = v[1]; dw[2] = v[2]; dw[3] = v[3];
        } else if constexpr (DPT == 2) {
          const u32x2 v = *reinterpret_cast<const u32x2*>(lds + off);
          dw[0] = v[0]; dw[1] = v[1];
        } else {
          dw[0] = *reinterpret_cast<const uint32_t*>(lds + off);
        }
        uint32_t sbits, z;
        if constexpr (SH) {
          sbits = *reinterpret_cast<const uint16_t*>(lds + shs + 2u * (gn + (uint32_t)t));
          z = SYM ? 8u : (uint32_t)lds[shs + 32u * (uint32_t)G + gn + (uint32_t)t];
        } else {
          sbits = *reinterpret_cast<const uint16_t*>(lds + (st - lds0) + Gm::SOFF + 2 * (n * NG + t));
          z = SYM ? 8u : (uint32_t)lds[(st - lds0) + Gm::ZOFF + n * NG + t];
        }
        const f16x2 b1 = as_f16x2((0x6400u + z) * 0x00010001u);
        const f16x2 b16 = as_f16x2((0x6400u + 16u * z) * 0x00010001u);
        f32x4 pacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < DPT; ++u) {
          const f16x8 bw = dequant_f16<SYM>(dw[u], bias, b1, b16);
          const u32x4 a = xr[j * DPT + u];
          if constexpr (EX)
            pacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), to_bf16(bw), pacc, 0, 0, 0);
          else
            pacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), bw, pacc, 0, 0, 0);
        }
        const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)sbits);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(pacc[r], sc, acc[r]);
        if constexpr (j == Gm::TPP - 1) {
          if ((4 * kq) / MP == p) res = acc;
        }
      };
      for_each_index(tile, std::make_integer_sequence<int, P * Gm::TPP>{});
      // this slot's LDS reads are done: refill it with the row block S strides ahead
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (rb + S * stride < NB) issue(slot, rb + S * stride, it + S);

      // factor of output rows 4 kq + r (token slots of this lane's D fragment)
#pragma unroll
      for (int r = 0; r < 4; ++r) res[r] *= __shfl(my_fac, 4 * kq + r);
      // add the parts: slot 4 kq + r is token (4 kq + r) % MP of part (4 kq + r) / MP
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (P == 4) res[r] += __shfl_xor(res[r], 16);
        if constexpr (P >= 2) res[r] += __shfl_xor(res[r], 32);
      }
      // the waves' partials meet in LDS (two buffers, alternating row blocks)
      const uint32_t red = red0 + (uint32_t)(it & 1) * (uint32_t)(WS * kRedBytes);
      *reinterpret_cast<f32x4*>(lds + (red - lds0) + w * kRedBytes + 16 * lane) = res;
      lds_barrier();
      if (w == it % WS && kq < MP / 4) {                              // wave-uniform / lane mask
        f32x4 sum = *reinterpret_cast<const f32x4*>(lds + (red - lds0) + 16 * lane);
        for (int ww = 1; ww < WS; ++ww)
          sum += *reinterpret_cast<const f32x4*>(lds + (red - lds0) + ww * kRedBytes + 16 * lane);
        const int row = rb * 16 + n;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tk = 4 * kq + r;
          if (row < N && tk < M) Y[(size_t)tk * N + row] = f32_to_bf16_bits(sum[r]);
        }
      }
    }
  };
  if (exact) run(std::true_type{});
  else run(std::false_type{});
}

// Launch geometry of a shape: parts P, slices NSL, waves WS and stages S; sh: the shared
// scale and zero-point slots.
struct Plan {
  int P = 0, NSL = 0, WS = 0, S = 0;
  bool sh = false;
  size_t lds = 0;
};

// Bytes of one stage and vector memory operations per stage (as Geo computes them).
size_t stage_bytes(int P, int NSL, int g, bool sym, bool sh, int* ops) {
  const int KR = P * NSL * 32, NG = KR / g;
  const int NSI = (8 * NG + 63) / 64, NZI = sym ? 0 : (4 * NG + 63) / 64;
  *ops = 4 * (KR / 512) + NSI + NZI;
  return (size_t)16 * (KR / 2) + (sh ? 0u : 256u * NSI + 256u * NZI);
}

Plan plan_for(int64_t M, int64_t N, int64_t K, int g, bool sym, bool sh) {
  Plan pl;
  if (M < 1 || M > 16 || !(g == 32 || g == 64 || g == 128)) return pl;
  if (N * (K / 2) >= ((int64_t)1 << 32) || M * K * 2 >= ((int64_t)1 << 32)) return pl;
  const int P = M <= 4 ? 4 : (M <= 8 ? 2 : 1);
  // slices per part: 16 (64 registers of X), fewer for small groups at several parts (their
  // many tiles per stage would not fit the registers), fewer again when K is short, so that
  // a workgroup has four waves where K allows
  int NSL = 16;
  if ((g == 32 && P >= 2) || (g == 64 && P == 4)) NSL = 8;
  // four parts: 8 slices wherever that gives at most 8 ranges of 1024, i.e. two waves per SIMD
  // (the 70B-shaped layer at M = 4: 31.1 -> 29.2 us)
  if (P == 4 && K % 1024 == 0 && K / 1024 <= kMaxWaves) NSL = 8;
  while (NSL > 4 && P * (NSL / 2) >= 16 && (K % (P * NSL * 32) != 0 || K / (P * NSL * 32) < 4)) NSL /= 2;
  // one part (M > 8) and more than 8 ranges of 512: 32 slices (a 1024 range per wave, 128
  // registers of X) for g = 64 and 128
  if (P == 1 && g >= 64 && K / 512 > kMaxWaves && K % 1024 == 0) NSL = 32;
  const int64_t KR = (int64_t)P * NSL * 32;
  if (K % KR != 0 || KR < 512 || KR / g < 4) return pl;
  const int64_t WS = K / KR;
  if (WS < 1 || WS > kMaxWaves) return pl;
  int ops = 0;
  const size_t st = stage_bytes(P, NSL, g, sym, sh, &ops);
  const size_t red = (size_t)2 * WS * kRedBytes;
  const size_t slot = sh ? (size_t)(K / g) * (sym ? 32 : 48) : 0;   // a row block's scales and zero-points
  if (kLdsMax < red + 2 * slot) return pl;
  int S = (int)((kLdsMax - red - 2 * slot) / ((size_t)WS * st + slot));   // S stages, S + 2 slots
  if (S > 4) S = 4;
  while (S > 2 && (S - 1) * ops > 63) --S;             // the stage waits fit the counter
  if (S < 2) return pl;
  pl.P = P; pl.NSL = NSL; pl.WS = (int)WS; pl.S = S; pl.sh = sh;
  pl.lds = (size_t)WS * S * st + (size_t)(S + 2) * slot + red;
  return pl;
}

template <int P, int NSL, int TK, bool SYM>
hipError_t launch_one(const Plan& pl, const void* X, int M, int64_t N, int64_t K, const void* packed,
                      const void* scales, const void* zeros, void* Y, int num_cus, hipStream_t stream) {
  const auto kernel = pl.sh ? decode_kernel<P, NSL, TK, SYM, true> : decode_kernel<P, NSL, TK, SYM, false>;
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(decode_kernel<P, NSL, TK, SYM, true>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsMax) != hipSuccess
          ? hipErrorInvalidValue
          : hipFuncSetAttribute(reinterpret_cast<const void*>(decode_kernel<P, NSL, TK, SYM, false>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsMax);
  if (attr != hipSuccess) return attr;
  const int64_t NB = (N + 15) / 16;
  const int64_t blocks = NB < num_cus ? NB : num_cus;
  hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3((unsigned)(pl.WS * kWave)), pl.lds, stream,
                     (const uint16_t*)X, M, (int)N, (int)K, (const uint8_t*)packed, (const uint16_t*)scales,
                     (const uint8_t*)zeros, (uint16_t*)Y, pl.S);
  return hipGetLastError();
}

// (plan_for never picks 16 slices for g = 32 at two or four parts, or for g = 64 at four parts,
// nor 32 slices for g = 32)
template <int P, int NSL, bool SYM>
hipError_t launch_tk(const Plan& pl, int g, const void* X, int M, int64_t N, int64_t K, const void* packed,
                     const void* scales, const void* zeros, void* Y, int num_cus, hipStream_t stream) {
  if constexpr (!(NSL == 16 && P >= 2) && NSL != 32)
    if (g == 32) return launch_one<P, NSL, 32, SYM>(pl, X, M, N, K, packed, scales, zeros, Y, num_cus, stream);
  if constexpr (!(NSL == 16 && P == 4))
    if (g == 64) return launch_one<P, NSL, 64, SYM>(pl, X, M, N, K, packed, scales, zeros, Y, num_cus, stream);
  if (g == 128) return launch_one<P, NSL, 128, SYM>(pl, X, M, N, K, packed, scales, zeros, Y, num_cus, stream);
  return hipErrorInvalidValue;
}

template <bool SYM>
hipError_t launch_mode(const Plan& pl, int g, const void* X, int M, int64_t N, int64_t K, const void* packed,
                       const void* scales, const void* zeros, void* Y, int num_cus, hipStream_t stream) {
#define Q4_DECODE(PV, NV)                                                                                    \
  if (pl.P == PV && pl.NSL == NV)                                                                            \
    return launch_tk<PV, NV, SYM>(pl, g, X, M, N, K, packed, scales, zeros, Y, num_cus, stream);
  Q4_DECODE(1, 16)
  Q4_DECODE(1, 32)
  Q4_DECODE(2, 16)
  Q4_DECODE(2, 8)
  Q4_DECODE(4, 16)
  Q4_DECODE(4, 8)
  Q4_DECODE(4, 4)
#undef Q4_DECODE
  return hipErrorInvalidValue;
}

}  // namespace

bool decode_fits(int64_t M, int64_t N, int64_t K, int g) {
  // the symmetric format needs fewer bytes per stage, so an asymmetric fit covers both; the
  // shared slots are taken only where they fit as well
  return plan_for(M, N, K, g, false, false).P != 0;
}

hipError_t launch_decode(const void* X, int M, int64_t N, int64_t K, int g, bool sym,
                         const void* packed, const void* scales, const void* zeros, void* Y,
                         int num_cus, hipStream_t stream) {
  // shared scale slots when every workgroup has two row blocks or more and they fit
  const Plan psh = (N + 15) / 16 >= 2 * (int64_t)num_cus ? plan_for(M, N, K, g, sym, true) : Plan{};
  const Plan pl = psh.P != 0 ? psh : plan_for(M, N, K, g, sym, false);
  if (pl.P == 0) return hipErrorInvalidValue;
  return sym ? launch_mode<true>(pl, g, X, M, N, K, packed, scales, zeros, Y, num_cus, stream)
             : launch_mode<false>(pl, g, X, M, N, K, packed, scales, zeros, Y, num_cus, stream);
}

}  // namespace q4
