// W4A16 prefill GEMM for large M on the bf16 matrix cores of gfx950 (v_mfma_f32_16x16x32_bf16).
//
// The weights stay 4-bit in HBM and are dequantised inside the kernel; the product runs on
// 16-bit operands ("LLM Weight Quantization - GPTQ, AWQ, SmoothQuant, FP8 & INT4/INT8
// Trade-offs", "The vocabulary" and "format notes").  The dequantised weight is
// x_hat = scale * (q - z) ("DL S067 · Quantization", §1), formed exactly in fp32 by one
// mixed-precision fma per weight and rounded once to bf16.
//
// Block = 4 waves, tile = 256 (or 128) rows of X x 256 rows of W, k walked in steps of 128;
// shapes with too few such tiles to fill every compute unit take 128 x 128 tiles instead, and
// those with at most one of these per compute unit 128 x 64.
//   * X: the block's 256 x 128 bf16 slice of each step is copied global -> LDS by the
//     direct-to-LDS loads of gfx950 (no registers), double-buffered: the copy for step s + 1
//     is issued at the start of step s.  Rows are XOR-swizzled in 16-byte chunks so that the
//     MFMA fragment reads hit 16 different bank groups.
//   * W: each wave owns 64 W rows; a lane loads the 32 codes (16 bytes) it needs per row and
//     step ahead of use (one step ahead in the 128-row tile; in the 256-row tile each 16-row
//     block's codes are requested as soon as its register slot is free, most of two steps
//     ahead), and dequantises them in registers straight into MFMA operands, so every weight
//     of the tile is dequantised exactly once per block.
//   * One barrier per step, after the step's loads have landed.
// The k order inside a step is permuted identically for both operands (lane group q takes the
// 32 contiguous k of its codes), which leaves each output sum unchanged.
// W8A16 ("LLM Weight Quantization ...", "Granularity and outliers") uses the same kernel with
// 8-bit codes (B = 8): a lane loads its 32 codes per row and step as two 16-byte loads, a code
// byte placed under the fp16 exponent byte 0x64 reads as 1024 + q (v_perm_b32, two per
// instruction), and fma(1024 + q, s, -s (1024 + z)) = s (q - z) exactly.
// MFMA: D[n][m] = sum_k W[n][k] X[m][k]; a lane's four accumulators are four consecutive n of
// one m, written as one 8-byte store into row-major Y.  Blocks are numbered so that each XCD
// (one L2) works on a rectangle of tiles that share X and W slices.
#include <type_traits>
#include <utility>

#include "q4_device.h"
#include "q4_internal.h"

namespace q4 {
namespace {

constexpr int kStepK = 128;                            // k per step
constexpr int kTileN = 256;                            // W rows per block (64 per wave)
constexpr uint32_t kRowBytes = kStepK * 2;             // one X row of a step in LDS
constexpr uint32_t kSzStage = 4 * (512 + 256);          // scale / zero words per stage
// X rows per block (TM): 128 (two blocks per compute unit) or 256 (one block; every
// dequantised weight then serves twice the X rows).
constexpr int kTileMSmall = 128, kTileMLarge = 256;

// Dequantise 8 codes (one dword, code k in bits 4k..4k+3) into 8 bf16 MFMA operand values.
// A nibble at bits 0..3 OR-ed into fp16 1024.0 (0x6400) reads as 1024 + q; a nibble at bits
// 4..7 OR-ed into fp16 64.0 (0x5400, ulp 1/16) reads as 64 + q.  With c1 = -s (1024 + z) and
// c64 = -s (64 + z), fma(1024 + q, s, c1) = fma(64 + q, s, c64) = s (q - z) exactly in fp32
// (fp16 scale x 5-bit integer), then rounded once to bf16.
// The work is split so that it can be spread between matrix instructions: deq_prep forms the
// four biased fp16 pairs of a dword, deq_pair(i) the i-th packed bf16 pair of the result
// (k = 2i, 2i + 1 in the permuted order k0 k1 | k2 k3 | k4 k5 | k6 k7).
struct Biased {
  f16x2 q0, q1, q2, q3;    // (k0, k4) and (k2, k6) as 1024 + q; (k1, k5) and (k3, k7) as 64 + q
};
// (x & mask) | bias as one v_and_or_b32: the compiler otherwise emits an AND and an OR, each
// with a literal, for every biased pair.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t bias) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(bias));
  return r;
}
template <bool SYM>
__device__ __forceinline__ Biased deq_prep(uint32_t dw) {
  if (SYM) dw ^= 0x88888888u;                     // two's complement nibble -> q + 8, z = 8
  const uint32_t d8 = dw >> 8;
  return Biased{as_f16x2(and_or(dw, 0x000F000Fu, 0x64006400u)), as_f16x2(and_or(dw, 0x00F000F0u, 0x54005400u)),
                as_f16x2(and_or(d8, 0x000F000Fu, 0x64006400u)), as_f16x2(and_or(d8, 0x00F000F0u, 0x54005400u))};
}
// The two fp32 values of pair i (exact), then the pair packed to bf16.
__device__ __forceinline__ void deq_fmas(const Biased& b, int i, float s, float c1, float c64, float& w0, float& w1) {
  const f16x2 lo = (i & 1) ? b.q2 : b.q0;
  const f16x2 hi = (i & 1) ? b.q3 : b.q1;
  const int h = i >> 1;
  w0 = __builtin_fmaf((float)lo[h], s, c1);
  w1 = __builtin_fmaf((float)hi[h], s, c64);
}
__device__ __forceinline__ uint32_t deq_pair(const Biased& b, int i, float s, float c1, float c64) {
  float w0, w1;
  deq_fmas(b, i, s, c1, c64, w0, w1);
  return pack_bf16x2(w0, w1);
}
template <bool SYM>
__device__ __forceinline__ u32x4 dequant8(uint32_t dw, float s, float c1, float c64) {
  const Biased b = deq_prep<SYM>(dw);
  return u32x4{deq_pair(b, 0, s, c1, c64), deq_pair(b, 1, s, c1, c64), deq_pair(b, 2, s, c1, c64),
               deq_pair(b, 3, s, c1, c64)};
}

// 8-bit codes: the eight codes of a sub-step (k0..k7, one byte each) in two dwords.  Pair i of
// the result is (k 2i, k 2i + 1); as 1024 + q in fp16: q0 = (k0, k1), q1 = (k2, k3) from the first
// dword, q2, q3 from the second.  Symmetric codes (int8) are offset by 128, z = 128.
template <bool SYM>
__device__ __forceinline__ Biased deq_prep_b(uint32_t d0, uint32_t d1) {
  if (SYM) {
    d0 ^= 0x80808080u;
    d1 ^= 0x80808080u;
  }
  return Biased{as_f16x2(__builtin_amdgcn_perm(0x64646464u, d0, 0x04010400u)),
                as_f16x2(__builtin_amdgcn_perm(0x64646464u, d0, 0x04030402u)),
                as_f16x2(__builtin_amdgcn_perm(0x64646464u, d1, 0x04010400u)),
                as_f16x2(__builtin_amdgcn_perm(0x64646464u, d1, 0x04030402u))};
}
__device__ __forceinline__ void deq_fmas_b(const Biased& b, int i, float s, float c1, float& w0, float& w1) {
  const f16x2 q = i == 0 ? b.q0 : (i == 1 ? b.q1 : (i == 2 ? b.q2 : b.q3));
  w0 = __builtin_fmaf((float)q[0], s, c1);
  w1 = __builtin_fmaf((float)q[1], s, c1);
}
// One sub-step's MFMA operand (8 bf16) from the code dwords of either width.
template <bool SYM, int B>
__device__ __forceinline__ u32x4 dequant_sub(uint32_t d0, uint32_t d1, float s, float c1, float c64) {
  if constexpr (B == 8) {
    const Biased b = deq_prep_b<SYM>(d0, d1);
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float w0, w1;
      deq_fmas_b(b, i, s, c1, w0, w1);
      r[i] = pack_bf16x2(w0, w1);
    }
    return r;
  } else {
    (void)d1;
    return dequant8<SYM>(d0, s, c1, c64);
  }
}

// acc += a b on the matrix core with the accumulator tied to its AGPRs, so that a wave's 256
// accumulators stay in place (the builtin lets the register allocator move them between
// AGPRs and VGPRs around every MFMA).  The compiler does not look inside the asm, so the
// caller owns the hazards: the vector instruction that writes a (or b) must come at least
// three instructions before the MFMA that reads it, the accumulator must not be rewritten by
// anything but this MFMA, and drain_mfma() must run before the accumulators are read.
__device__ __forceinline__ void mfma_acc(f32x4& acc, const u32x4& a, const bf16x8& b) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void drain_mfma() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// 16 bytes per lane, global -> LDS: lane i writes LDS bytes [lds + 16 i, lds + 16 i + 16).
// `base` and `lds` are wave-uniform; the instruction has no register result.
__device__ __forceinline__ void copy_to_lds(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1 sc1" ::"v"(voff), "s"(base), "{m0}"(lds) : "memory");
}

// 4 bytes per lane, global -> LDS through a buffer resource: lane i writes LDS bytes
// [lds + 4 i, lds + 4 i + 4); a dword at or past the resource's end reads as 0.
__device__ __forceinline__ void copy_dword_to_lds(u32x4 rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("buffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds) : "memory");
}

// Raw-buffer descriptor words for inline asm (same format as buffer_over).
__device__ __forceinline__ u32x4 buffer_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes), (uint32_t)kBufferFlags};
}

// Wait for this wave's LDS traffic, then meet the other waves.  The global loads the next
// step reads (the LDS copies included) have been waited for just before, by the compiler's
// own wait for registers loaded after them.
__device__ __forceinline__ void step_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <int R>
using Slot = std::integral_constant<int, R>;

// f(0), f(1), ..., f(N - 1) with compile-time arguments: straight-line code that does not
// depend on the unroller's size limits.
template <typename F, int... I>
__device__ __forceinline__ void for_each_index(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}

// EDGE = false: every tile of the launch is full (TN W rows, TM X rows in range), so the
// per-lane parts of all addresses are the same for every row group and the rest is
// wave-uniform.  EDGE = true: the last row and / or column of tiles of a ragged shape; X rows
// past M are clamped to row M - 1 and W rows past N read as 0 (their outputs are dropped).
//
// NBW: 16-row blocks of W per wave (4: 256-row W tiles; 2: 128-row tiles, for shapes whose
// 256-row tiles would leave compute units idle; 1: 64-row tiles, when 128-row tiles would give
// a compute unit at most one block, so that two blocks' loads and work overlap).
// B: code width, 4 (W4A16) or 8 (W8A16).
template <int TM, int NBW, bool SYM, bool EDGE, int B>
__global__ __launch_bounds__(256, TM == kTileMSmall ? 2 : 1) void prefill_kernel(
    const uint16_t* __restrict__ X, int M, int N, int K, int lg,
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
    const uint8_t* __restrict__ zeros, uint16_t* __restrict__ Y, int tiles_m, int tiles_n,
    int edge_row, int vec_store) {
  static_assert(TM == kTileMSmall || TM == kTileMLarge, "tile of 128 or 256 X rows");
  constexpr int MB = TM / 16;                          // 16-row blocks of X
  static_assert(NBW == 4 || ((NBW == 2 || NBW == 1) && TM == kTileMSmall), "256-row W tiles, or 128- or 64-row with 128 X rows");
  constexpr int NB = NBW;                              // 16-row blocks of W per wave
  constexpr int TN = 64 * NBW;                         // W rows per block
  constexpr int RPW = 16 * NBW;                        // W rows per wave
  // Scales and zero-points reach registers by per-lane loads issued with the codes (edge
  // tiles and narrow tiles), or through LDS words copied one step ahead (full 256-row tiles,
  // whose copy instructions cover 64 rows per wave).
  constexpr bool REGSZ = EDGE || NBW != 4;
  constexpr int RW = TM / 4;                           // X rows each wave copies per step
  constexpr uint32_t kStageBytes = TM * kRowBytes;     // 32 or 64 KiB
  constexpr uint32_t kWaveDma = kStageBytes / 4;       // bytes each wave copies per step
  constexpr int kDmaOps = kWaveDma / 1024;             // 1 KiB copy instructions per wave
  static_assert(B == 4 || B == 8, "4- or 8-bit codes");
  constexpr int CW = B / 4;                            // 16-byte code loads per row and step
  constexpr uint32_t kZsym = B == 8 ? 128u : 8u;       // symmetric codes are offset by this

  // Two X stages, then (full tiles) two stages of the scale and zero-point words of the
  // block's W rows: per stage and wave, 64 rows x 8 bytes of scales and 64 rows x 4 bytes of
  // zeros, each row's words starting at the 4-byte boundary at or below its first group.
  __shared__ __attribute__((aligned(1024))) uint8_t xl[2 * kStageBytes + 2 * kSzStage];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int li = lane & 15, lq = lane >> 4;

  // Tile of this block.  Full launch: tiles_m x tiles_n full tiles, numbered so that the
  // tiles sharing X rows land on one XCD.  Edge launch: first the bottom row of tiles
  // (edge_row: M is ragged), then the right column above it.
  int bm, bn;
  const int b = blockIdx.x;
  if (EDGE) {
    const int first = edge_row ? tiles_n : 0;
    if (b < first) { bm = tiles_m - 1; bn = b; }
    else { bm = b - first; bn = tiles_n - 1; }
  } else {
    const int tiles = tiles_m * tiles_n;
    // Blocks are dealt to the XCDs round-robin (b & 7).  With an even number of tile rows and
    // tile columns a multiple of 4, XCD x takes the rectangle of half the tile rows by a
    // quarter of the tile columns, so its concurrent tiles share X and W slices in its L2
    // (per step it fetches half the X slices and a quarter of the W slices of the launch);
    // otherwise the tiles sharing X rows go to one XCD.
    if ((tiles_m & 1) == 0 && (tiles_n & 3) == 0) {
      const int x = b & 7, i = b >> 3;
      const int rm = tiles_m >> 1, rn = tiles_n >> 2;
      bm = rm * (x & 1) + i / rn;
      bn = rn * (x >> 1) + i % rn;
    } else {
      const int t = (tiles & 7) == 0 ? (b & 7) * (tiles >> 3) + (b >> 3) : b;
      bm = t / tiles_n;
      bn = t - bm * tiles_n;
    }
  }
  const int m0 = bm * TM, n0 = bn * TN;
  const int KT = K / kStepK;
  const int G = K >> lg;
  const uint32_t xrow_bytes = (uint32_t)K * 2u;

  // X copy: this wave's instruction i fills LDS rows r = RW wave + 4 i + lane / 16 at chunk
  // position lane % 16, which holds chunk (lane % 16) ^ (r % 16) of the row.  r % 16 depends
  // on i only through i % 4, so full tiles need four lane offsets.
  // For full tiles the chunk term is (lane % 16) ^ (lane / 16) ^ 4 (i % 4): one lane offset,
  // XOR-ed with 64 (i % 4) (bits 6..7, clear of the row term, a multiple of 256).
  const uint16_t* xblk = X + (size_t)m0 * K;
  constexpr int ND = EDGE ? kDmaOps : 1;
  uint32_t dma_off[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) {
    const int r = RW * wave + 4 * i + (lane >> 4);
    const int c = (lane & 15) ^ (r & 15);
    const int rr = EDGE ? min(m0 + r, M - 1) - m0 : (lane >> 4);
    dma_off[i] = (uint32_t)rr * xrow_bytes + 16u * (uint32_t)c;
  }
  const uint32_t lds_wave = (uint32_t)(uintptr_t)xl + (uint32_t)wave * kWaveDma;

  // B fragment of k-chunk (4 lq + ks) of row 16 mb + li sits at chunk position
  // (4 lq + ks) ^ li = ((4 lq) ^ li) ^ ks.
  const uint32_t rd_off = (uint32_t)li * kRowBytes + 16u * (uint32_t)((4 * lq) ^ li);

  // W codes, scales and zeros of this block's rows through buffer resources ending at row N
  // (rows past N read as 0).  The group of k = 128 kt + 32 lq is (128 kt >> lg) + (32 lq >> lg)
  // for every power-of-two g >= 32.  Full tiles: one lane offset (row li of a 16-row block)
  // plus a wave-uniform offset for the block and step; edge tiles: a lane offset per block,
  // so that a row past N is out of range on its own.
  const uint32_t rows_left = (uint32_t)min(N - n0, TN);
  const uint32_t wrow = (uint32_t)K * B / 8;           // code bytes per W row
  const __amdgpu_buffer_rsrc_t rw = buffer_over(packed + (size_t)n0 * (size_t)wrow, rows_left * wrow);
  const __amdgpu_buffer_rsrc_t rs = buffer_over(scales + (size_t)n0 * G, rows_left * (uint32_t)G * 2u);
  const __amdgpu_buffer_rsrc_t rz = buffer_over(zeros + (size_t)n0 * G, rows_left * (uint32_t)G);
  const uint32_t gl = (uint32_t)((32 * lq) >> lg);
  constexpr int NV = EDGE ? NB : 1;
  uint32_t voff_w[NV], voff_s[NV], voff_z[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const uint32_t r = EDGE ? (uint32_t)(RPW * wave + 16 * v + li) : (uint32_t)li;
    voff_w[v] = r * wrow + 16u * CW * (uint32_t)lq;
    voff_z[v] = r * (uint32_t)G + gl;
    voff_s[v] = 2u * voff_z[v];
  }

  // Scale / zero words of the full path.  Copy: scale instruction j covers the wave's rows
  // 32 j + lane / 2 (dword lane % 2 of the 8-byte window), the zero instruction row lane.
  // Read: row 16 nb + li; all row offsets 16 nb G are multiples of 4, so the position inside
  // the window is the same for every nb.
  const u32x4 sz_s = buffer_words(scales + (size_t)n0 * G, (uint32_t)kTileN * (uint32_t)G * 2u);
  const u32x4 sz_z = buffer_words(zeros + (size_t)n0 * G, (uint32_t)kTileN * (uint32_t)G);
  const uint32_t rg_s = (uint32_t)(64 * wave + (lane >> 1)) * (uint32_t)G * 2u;
  const uint32_t rg_z = (uint32_t)(64 * wave + lane) * (uint32_t)G;
  const uint32_t rg_r = (uint32_t)li * (uint32_t)G;
  const uint32_t sz_lds = (uint32_t)(uintptr_t)xl + 2u * kStageBytes;

  f32x4 acc[NB][MB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 wq[2][NB][CW];              // codes: k = 32 lq .. 32 lq + 31 of the step, per W row
  uint32_t ws[2][NB], wz[2][NB];    // raw scale bits / zero point of that 32-k chunk

  auto copy_x = [&](int buf, int kt) {
    const uint16_t* src = xblk + (size_t)min(kt, KT - 1) * kStepK;
    const uint32_t dst = lds_wave + (uint32_t)buf * kStageBytes;
#pragma unroll
    for (int i = 0; i < kDmaOps; ++i) {
      if (EDGE) copy_to_lds(src, dma_off[i], dst + 1024u * i);
      else copy_to_lds(src + (size_t)(RW * wave + 4 * i) * K, dma_off[0] ^ (64u * (i & 3)), dst + 1024u * i);
    }
  };
  auto copy_x_piece = [&](int buf, int kt, int i) {
    const uint16_t* src = xblk + (size_t)min(kt, KT - 1) * kStepK;
    const uint32_t dst = lds_wave + (uint32_t)buf * kStageBytes;
    if (EDGE) copy_to_lds(src, dma_off[i], dst + 1024u * i);
    else copy_to_lds(src + (size_t)(RW * wave + 4 * i) * K, dma_off[0] ^ (64u * (i & 3)), dst + 1024u * i);
  };
  auto copy_sz = [&](int buf, int kt) {
    const uint32_t gs = (uint32_t)((min(kt, KT - 1) * kStepK) >> lg);
    const uint32_t dst = sz_lds + (uint32_t)buf * kSzStage + (uint32_t)wave * 512u;
    const uint32_t v0 = ((rg_s + 2u * gs) & ~3u) + 4u * (uint32_t)(lane & 1);
    copy_dword_to_lds(sz_s, v0, dst);
    copy_dword_to_lds(sz_s, v0 + 64u * (uint32_t)G, dst + 256u);
    if (!SYM) copy_dword_to_lds(sz_z, (rg_z + gs) & ~3u, sz_lds + (uint32_t)buf * kSzStage + 2048u + (uint32_t)wave * 256u);
  };
  auto load_w = [&](auto S, int kt) {
    constexpr int R = decltype(S)::value;
    const int ktc = min(kt, KT - 1);
    const int gs = (ktc * kStepK) >> lg;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int v = EDGE ? nb : 0;
      const int rb = EDGE ? 0 : RPW * wave + 16 * nb;   // wave-uniform row of the block
#pragma unroll
      for (int c = 0; c < CW; ++c)
        wq[R][nb][c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
            rw, voff_w[v] + 16u * c, rb * (int)wrow + ktc * (kStepK * B / 8), 0));
      if (REGSZ) {
        ws[R][nb] = __builtin_amdgcn_raw_buffer_load_b16(rs, voff_s[v], 2 * (rb * G + gs), 0);
        wz[R][nb] = SYM ? kZsym : (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rz, voff_z[v], rb * G + gs, 0);
      }
    }
  };

  // One 16-row block's codes (and, edge tiles, its scale and zero-point) of step kt into
  // slot R: the large tile requests each block as soon as its codes in the slot are dead.
  auto load_w_nb = [&](auto S, int kt, auto NBC) {
    constexpr int R = decltype(S)::value;
    constexpr int nb = decltype(NBC)::value;
    const int ktc = min(kt, KT - 1);
    const int gs = (ktc * kStepK) >> lg;
    const int v = EDGE ? nb : 0;
    const int rb = EDGE ? 0 : RPW * wave + 16 * nb;
#pragma unroll
    for (int c = 0; c < CW; ++c)
      wq[R][nb][c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
          rw, voff_w[v] + 16u * c, rb * (int)wrow + ktc * (kStepK * B / 8), 0));
    if (REGSZ) {
      ws[R][nb] = __builtin_amdgcn_raw_buffer_load_b16(rs, voff_s[v], 2 * (rb * G + gs), 0);
      wz[R][nb] = SYM ? kZsym : (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rz, voff_z[v], rb * G + gs, 0);
    }
  };

  // Name the W registers of slot R (codes, and scales / zeros when they come by register):
  // the compiler then waits for those loads here, and for nothing issued after them.
  // (One asm statement per kind, so that the compiler emits one wait for the whole set.)
  auto keep_w = [&wq, &ws, &wz](auto S) {
    constexpr int R = decltype(S)::value;
    if constexpr (NB == 4 && CW == 1) {
      asm volatile("" ::"v"(wq[R][0][0]), "v"(wq[R][1][0]), "v"(wq[R][2][0]), "v"(wq[R][3][0]));
    } else if constexpr (NB == 4) {
      asm volatile("" ::"v"(wq[R][0][0]), "v"(wq[R][0][1]), "v"(wq[R][1][0]), "v"(wq[R][1][1]), "v"(wq[R][2][0]),
                   "v"(wq[R][2][1]), "v"(wq[R][3][0]), "v"(wq[R][3][1]));
    } else if constexpr (NB == 1 && CW == 1) {
      asm volatile("" ::"v"(wq[R][0][0]));
    } else if constexpr (NB == 1) {
      asm volatile("" ::"v"(wq[R][0][0]), "v"(wq[R][0][1]));
    } else if constexpr (CW == 1) {
      asm volatile("" ::"v"(wq[R][0][0]), "v"(wq[R][1][0]));
    } else {
      asm volatile("" ::"v"(wq[R][0][0]), "v"(wq[R][0][1]), "v"(wq[R][1][0]), "v"(wq[R][1][1]));
    }
    if constexpr (REGSZ) {
      if constexpr (NB == 4) {
        asm volatile("" ::"v"(ws[R][0]), "v"(ws[R][1]), "v"(ws[R][2]), "v"(ws[R][3]));
        if constexpr (!SYM) asm volatile("" ::"v"(wz[R][0]), "v"(wz[R][1]), "v"(wz[R][2]), "v"(wz[R][3]));
      } else if constexpr (NB == 1) {
        asm volatile("" ::"v"(ws[R][0]));
        if constexpr (!SYM) asm volatile("" ::"v"(wz[R][0]));
      } else {
        asm volatile("" ::"v"(ws[R][0]), "v"(ws[R][1]));
        if constexpr (!SYM) asm volatile("" ::"v"(wz[R][0]), "v"(wz[R][1]));
      }
    }
  };
  // The two dwords of sub-step ks's codes in a row's slot (the second is unused for 4-bit).
  auto sub_d0 = [](const u32x4* w, int ks) { return B == 8 ? w[ks >> 1][2 * (ks & 1)] : w[0][ks]; };
  auto sub_d1 = [](const u32x4* w, int ks) { return B == 8 ? w[ks >> 1][2 * (ks & 1) + 1] : 0u; };

  // One step: copy X of step kt + 1 into the other buffer, load W codes of step kt + 1 into
  // the other slot, multiply step kt.
  auto step = [&](auto S, int kt) {
    constexpr int R = decltype(S)::value;
    // The previous barrier already waited for these registers; naming them here, before any
    // new load is issued, keeps the compiler's own wait for them from covering the new loads.
    keep_w(S);
    // This step's scale / zero words (copied during the previous step) -> registers.
    uint32_t sb[NB], zb[NB];
    if (!REGSZ) {
      const uint32_t gs = (uint32_t)((kt * kStepK) >> lg);
      const uint32_t par = rg_r + gs;
      const uint8_t* st = xl + 2u * kStageBytes + (uint32_t)R * kSzStage;
      const uint8_t* srow = st + (uint32_t)wave * 512u + (uint32_t)li * 8u + 2u * gl + 2u * (par & 1u);
      const uint8_t* zrow = st + 2048u + (uint32_t)wave * 256u + (uint32_t)li * 4u + gl + (par & 3u);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        sb[nb] = *reinterpret_cast<const uint16_t*>(srow + 128 * nb);
        zb[nb] = SYM ? kZsym : (uint32_t)zrow[64 * nb];
      }
    }
    copy_x(R ^ 1, kt + 1);
    if (!REGSZ) copy_sz(R ^ 1, kt + 1);
    load_w(Slot<R ^ 1>{}, kt + 1);
    // Keep the loads here: left alone, the scheduler sinks them to the end of the step to
    // shorten register lifetimes, which exposes their whole latency at the barrier.
    __builtin_amdgcn_sched_barrier(0);

    float s[NB], c1[NB], c64[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      s[nb] = (float)__builtin_bit_cast(_Float16, (uint16_t)(REGSZ ? ws[R][nb] : sb[nb]));
      const float zf = (float)(REGSZ ? wz[R][nb] : zb[nb]);
      c1[nb] = -s[nb] * (1024.0f + zf);
      c64[nb] = B == 8 ? c1[nb] : -s[nb] * (64.0f + zf);
    }
    const uint8_t* xs = xl + (uint32_t)R * kStageBytes;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 a[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        a[nb] = __builtin_bit_cast(bf16x8, dequant_sub<SYM, B>(sub_d0(wq[R][nb], ks), sub_d1(wq[R][nb], ks), s[nb],
                                                               c1[nb], c64[nb]));
      const uint32_t ro = rd_off ^ (16u * ks);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const bf16x8 bx = *reinterpret_cast<const bf16x8*>(xs + mb * 16 * kRowBytes + ro);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[nb], bx, acc[nb][mb], 0, 0, 0);
      }
    }
    // Wait for the next step's W registers, and so for everything issued before them (the X
    // and scale / zero copies), before the barrier.
    keep_w(Slot<R ^ 1>{});
    step_barrier();
  };

  if constexpr (TM == kTileMSmall) {
    copy_x(0, 0);
    if (!REGSZ) copy_sz(0, 0);
    load_w(Slot<0>{}, 0);
    keep_w(Slot<0>{});
    step_barrier();

    // Straight-line body of two steps (one per buffer / register slot); an odd last step follows.
    int kt = 0;
    for (; kt + 2 <= KT; kt += 2) {
      step(Slot<0>{}, kt);
      step(Slot<1>{}, kt + 1);
    }
    if (kt < KT) step(Slot<0>{}, kt);
  } else {
    // One wave per SIMD.  A step is 64 groups g = (ks, mb), each four MFMAs (X rows 16 mb..
    // x the wave's 64 W rows, sub-step ks) followed by a quarter of a dequantisation for the
    // next sub-step (for ks = 3: sub-step 0 of the next step, whose codes and scales this wave
    // loaded itself) and the LDS read of the X fragment two groups ahead.  sched_barrier keeps
    // the groups in order, which is what makes the MFMA asm safe: an operand written in group
    // g is first read in group g + 1 or later, behind at least three MFMAs, and every
    // accumulator is rewritten only by its own MFMA, 16 groups later.
    // LDS byte offsets of this lane's X fragment for (stage R, sub-step ks), kept in registers
    // (opaque to the compiler) so that each read's remaining row-block offset, at most
    // 15 x 4 KiB, is the instruction's immediate
    uint32_t xoff[2][4];
#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        xoff[rr][kk] = (uint32_t)rr * kStageBytes + (rd_off ^ (16u * kk));
        asm volatile("" : "+v"(xoff[rr][kk]));
      }
    u32x4 a[2][NB];                          // operands of sub-step ks (slot ks & 1)
    float sc[2][NB], cc1[2][NB], cc64[2][NB];   // per step slot: scale, -s (1024 + z), -s (64 + z)

    auto prep_scales = [&](auto S, int kt) {
      constexpr int R = decltype(S)::value;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        uint32_t sbits, zbits;
        if (REGSZ) {
          sbits = ws[R][nb];
          zbits = wz[R][nb];
        } else {
          const uint32_t gs = (uint32_t)((kt * kStepK) >> lg);
          const uint32_t par = rg_r + gs;
          const uint8_t* st = xl + 2u * kStageBytes + (uint32_t)R * kSzStage;
          sbits = *reinterpret_cast<const uint16_t*>(st + (uint32_t)wave * 512u + (uint32_t)li * 8u + 2u * gl +
                                                     2u * (par & 1u) + 128u * nb);
          zbits = SYM ? kZsym : (uint32_t)st[2048u + (uint32_t)wave * 256u + (uint32_t)li * 4u + gl + (par & 3u) + 64u * nb];
        }
        sc[R][nb] = (float)__builtin_bit_cast(_Float16, (uint16_t)sbits);
        const float zf = (float)zbits;
        cc1[R][nb] = -sc[R][nb] * (1024.0f + zf);
        cc64[R][nb] = B == 8 ? cc1[R][nb] : -sc[R][nb] * (64.0f + zf);
      }
    };
    // Wait for this wave's loads of the step in slot R (codes; everything issued before them).
    auto wait_codes = [&](auto S) { keep_w(S); };

    auto step_large = [&](auto S, int kt) {
      constexpr int R = decltype(S)::value;
      constexpr int NG = 4 * MB;          // groups per step
      constexpr int XA = 2;               // X fragments read this many groups ahead
      auto xfrag = [&](int g) {
        return *reinterpret_cast<const bf16x8*>(xl + xoff[R][g / MB] + (g % MB) * 16 * kRowBytes);
      };
      bf16x8 bx[XA + 1];
#pragma unroll
      for (int g = 0; g < XA; ++g) bx[g] = xfrag(g);
      Biased bq;
      for_each_index([&](auto GC) {
        constexpr int g = decltype(GC)::value;
        constexpr int ks = g / MB, mb = g % MB;
        constexpr int nbw = mb >> 2, piece = mb & 3;
        constexpr bool next = ks == 3;                 // dequantising sub-step 0 of the next step
        constexpr int dst = next ? 0 : (ks + 1) & 1;
        constexpr int S2 = next ? (R ^ 1) : R;         // step slot of the codes and scales
        const bf16x8 b = bx[g % (XA + 1)];
        // Four slots, each one MFMA and then a little other work, so that the wave issues the
        // other work while the MFMA executes.  Slot 0: this group's LDS read two groups ahead
        // and, in the first groups, one of the next step's copies (one X copy per group, then
        // the scale / zero words); in groups 34..46, the codes of the step after next.
        mfma_acc(acc[0][mb], a[ks & 1][0], b);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (g + XA < NG) bx[(g + XA) % (XA + 1)] = xfrag(g + XA);
        // block nb of slot R was last read in group 33 + 4 nb (sub-step 3 of this step): the
        // block's codes of step kt + 2 are requested into it in group 34 + 4 nb, which gives
        // them until group 47 of the next step (against groups 0 -> 47 of one step when a
        // slot was refilled at the start of the step it feeds: 207 -> 202 us at g = 128, and
        // 237 -> 201 us for 8-bit codes, whose loads are twice as large)
        if constexpr (g >= 34 && g <= 46 && (g - 34) % 4 == 0)
          load_w_nb(Slot<R>{}, kt + 2, std::integral_constant<int, (g - 34) / 4>{});
        if constexpr (g < kDmaOps) copy_x_piece(R ^ 1, kt + 1, g);
        if constexpr (g == kDmaOps) { if (!REGSZ) copy_sz(R ^ 1, kt + 1); }
        __builtin_amdgcn_sched_barrier(0);
        // Slot 1: half of the biased fp16 pairs of a new code dword (the other half one group
        // later, which evens out the vector work between groups).
        mfma_acc(acc[1][mb], a[ks & 1][1], b);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (B == 8) {
          if constexpr (piece == 0) {
            constexpr int kn = next ? 0 : ks + 1;                   // the sub-step dequantised
            const u32x4* wsrc = next ? wq[R ^ 1][nbw] : wq[R][nbw];
            bq = deq_prep_b<SYM>(sub_d0(wsrc, kn), sub_d1(wsrc, kn));
          }
        } else if constexpr (piece <= 1) {
          // the four biased pairs of the dword in two halves: (k0, k4), (k1, k5) for pieces 0 and
          // 2 here, (k2, k6), (k3, k7) for pieces 1 and 3 one group later
          constexpr int kn = next ? 0 : ks + 1;
          const u32x4* wsrc = next ? wq[R ^ 1][nbw] : wq[R][nbw];
          uint32_t dw = sub_d0(wsrc, kn);
          if (SYM) dw ^= 0x88888888u;
          if constexpr (piece == 0) {
            bq.q0 = as_f16x2(and_or(dw, 0x000F000Fu, 0x64006400u));
            bq.q1 = as_f16x2(and_or(dw, 0x00F000F0u, 0x54005400u));
          } else {
            const uint32_t d8 = dw >> 8;
            bq.q2 = as_f16x2(and_or(d8, 0x000F000Fu, 0x64006400u));
            bq.q3 = as_f16x2(and_or(d8, 0x00F000F0u, 0x54005400u));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        // Slot 2: the two exact products of this group's pair.
        mfma_acc(acc[2][mb], a[ks & 1][2], b);
        __builtin_amdgcn_sched_barrier(0);
        float w0, w1;
        if constexpr (B == 8) deq_fmas_b(bq, piece, sc[S2][nbw], cc1[S2][nbw], w0, w1);
        else deq_fmas(bq, piece, sc[S2][nbw], cc1[S2][nbw], cc64[S2][nbw], w0, w1);
        __builtin_amdgcn_sched_barrier(0);
        // Slot 3: the pair packed into the operand; before sub-step 3, this wave's next codes
        // are waited for and the next step's scales formed.
        mfma_acc(acc[3][mb], a[ks & 1][3], b);
        __builtin_amdgcn_sched_barrier(0);
        a[dst][nbw][piece] = pack_bf16x2(w0, w1);
        if constexpr (ks == 2 && mb == MB - 1) {
          wait_codes(Slot<R ^ 1>{});
          prep_scales(Slot<R ^ 1>{}, kt + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }, std::make_integer_sequence<int, NG>{});
      step_barrier();
    };

    copy_x(0, 0);
    if (!REGSZ) copy_sz(0, 0);
    load_w(Slot<0>{}, 0);
    wait_codes(Slot<0>{});
    load_w(Slot<1>{}, 1);                    // the codes of step 1 (slot 1), two steps ahead
    prep_scales(Slot<0>{}, 0);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      a[0][nb] = dequant_sub<SYM, B>(sub_d0(wq[0][nb], 0), sub_d1(wq[0][nb], 0), sc[0][nb], cc1[0][nb], cc64[0][nb]);
    step_barrier();

    int kt = 0;
    for (; kt + 2 <= KT; kt += 2) {
      step_large(Slot<0>{}, kt);
      step_large(Slot<1>{}, kt + 1);
    }
    if (kt < KT) step_large(Slot<0>{}, kt);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the last steps' look-ahead loads (unused)
    drain_mfma();
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) asm volatile("" : "+a"(acc[nb][mb]));
  }

  // D[n][m]: lane (li, lq) holds n = 4 lq + e (e = 0..3) of column m = li.
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = m0 + mb * 16 + li;
      const int nbase = n0 + RPW * wave + nb * 16 + 4 * lq;
      if (m < M) {
        const f32x4 v = acc[nb][mb];
        uint16_t* yrow = Y + (size_t)m * N;
        if (vec_store && nbase + 3 < N) {
          *reinterpret_cast<u32x2*>(yrow + nbase) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (nbase + e < N) yrow[nbase + e] = f32_to_bf16_bits(v[e]);
        }
      }
    }
  }
}

template <int TM, int NBW, bool SYM, int B>
hipError_t launch_tm(const void* X, int64_t M, int64_t N, int64_t K, int lg, const void* packed,
                     const void* scales, const void* zeros, void* Y, hipStream_t stream) {
  constexpr int TN = 64 * NBW;
  const int full_m = (int)(M / TM), full_n = (int)(N / TN);
  const int tiles_m = (int)((M + TM - 1) / TM);
  const int tiles_n = (int)((N + TN - 1) / TN);
  const int vec = (N % 4 == 0) && ((reinterpret_cast<uintptr_t>(Y) & 7) == 0);
  const int64_t full_blocks = (int64_t)full_m * full_n;
  if ((int64_t)tiles_m * tiles_n > 0x7fffffff) return hipErrorInvalidValue;
  if (full_blocks > 0) {
    hipLaunchKernelGGL((prefill_kernel<TM, NBW, SYM, false, B>), dim3((unsigned)full_blocks), dim3(256), 0, stream,
                       (const uint16_t*)X, (int)M, (int)N, (int)K, lg, (const uint8_t*)packed,
                       (const uint16_t*)scales, (const uint8_t*)zeros, (uint16_t*)Y, full_m, full_n, 0, vec);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // Ragged edge: the bottom row of tiles (if M is ragged) and the right column above it (if N
  // is ragged).
  const int edge_row = tiles_m != full_m;
  const int64_t edge_blocks = (edge_row ? tiles_n : 0) + (tiles_n != full_n ? full_m : 0);
  if (edge_blocks > 0) {
    hipLaunchKernelGGL((prefill_kernel<TM, NBW, SYM, true, B>), dim3((unsigned)edge_blocks), dim3(256), 0, stream,
                       (const uint16_t*)X, (int)M, (int)N, (int)K, lg, (const uint8_t*)packed,
                       (const uint16_t*)scales, (const uint8_t*)zeros, (uint16_t*)Y, tiles_m, tiles_n,
                       edge_row, vec);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <bool SYM, int B>
hipError_t launch_sym(const void* X, int64_t M, int64_t N, int64_t K, int lg, const void* packed,
                      const void* scales, const void* zeros, void* Y, int num_cus, hipStream_t stream) {
  // The 256-row tile runs one block per compute unit: take it when its tiles fill every unit.
  const int64_t large_tiles = ((M + kTileMLarge - 1) / kTileMLarge) * ((N + kTileN - 1) / kTileN);
  if (large_tiles >= num_cus)
    return launch_tm<kTileMLarge, 4, SYM, B>(X, M, N, K, lg, packed, scales, zeros, Y, stream);
  // 128 X rows: 256-row W tiles when they fill both block slots of every unit, else twice as
  // many 128-row tiles (M=1024 at 8192^2: 180 -> 157 us).
  // (8-bit codes: the 128 x 256 tile would spill its doubled code registers, so they go
  // straight to 128 x 128.)
  const int64_t small_tiles = ((M + kTileMSmall - 1) / kTileMSmall) * ((N + kTileN - 1) / kTileN);
  if (B == 4 && small_tiles >= 2 * (int64_t)num_cus)
    return launch_tm<kTileMSmall, 4, SYM, B>(X, M, N, K, lg, packed, scales, zeros, Y, stream);
  // At most one 128 x 128 tile per compute unit (small M: a block's time is its K loop, bound by
  // its loads' latency): 128 x 64 tiles, twice as many blocks, two sharing a unit and all
  // resident at once (70B-shaped layer M = 64 / 128: 96.8 / 102.6 -> 88.0 / 94.7 us; 8192^2
  // M = 128 / 256 / 384 / 512: 95.7 / 95.6 / 96.7 / 96.8 -> 71.0 / 71.5 / 79.9 / 94.8 us).  With
  // more, the 128 x 64 blocks would run in more than one round: 8192^2 M = 768 125.8 -> 160.7 us,
  // the 70B-shaped layer M = 256 162.6 -> 185.7 us.
  const int64_t half_tiles = ((M + kTileMSmall - 1) / kTileMSmall) * ((N + 127) / 128);
  if (half_tiles <= (int64_t)num_cus)
    return launch_tm<kTileMSmall, 1, SYM, B>(X, M, N, K, lg, packed, scales, zeros, Y, stream);
  return launch_tm<kTileMSmall, 2, SYM, B>(X, M, N, K, lg, packed, scales, zeros, Y, stream);
}

}  // namespace

bool prefill_fits(int64_t M, int64_t N, int64_t K, int g, int bits) {
  // 32-bit offsets: a block's X rows and the W codes / scales behind one buffer resource
  // must span < 2 GiB.
  const int64_t lim = int64_t(1) << 31;
  return M >= kPrefillMinM && K % kStepK == 0 && g >= 32 && (g & (g - 1)) == 0 &&
         (int64_t)kTileMLarge * K * 2 < lim && N * (K * bits / 8) < lim && N * (K / g) * 2 < lim;
}

hipError_t launch_prefill(const void* X, int64_t M, int64_t N, int64_t K, int g, bool sym,
                          const void* packed, const void* scales, const void* zeros, void* Y,
                          int num_cus, hipStream_t stream) {
  int lg = 0;
  while ((1 << lg) < g) ++lg;
  return sym ? launch_sym<true, 4>(X, M, N, K, lg, packed, scales, zeros, Y, num_cus, stream)
             : launch_sym<false, 4>(X, M, N, K, lg, packed, scales, zeros, Y, num_cus, stream);
}

hipError_t launch_prefill8(const void* X, int64_t M, int64_t N, int64_t K, int g, bool sym,
                           const void* codes, const void* scales, const void* zeros, void* Y,
                           int num_cus, hipStream_t stream) {
  int lg = 0;
  while ((1 << lg) < g) ++lg;
  return sym ? launch_sym<true, 8>(X, M, N, K, lg, codes, scales, zeros, Y, num_cus, stream)
             : launch_sym<false, 8>(X, M, N, K, lg, codes, scales, zeros, Y, num_cus, stream);
}

}  // namespace q4
