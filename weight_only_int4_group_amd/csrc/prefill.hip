// W4A16 prefill GEMM for large M on the bf16 matrix cores of gfx950 (v_mfma_f32_16x16x32_bf16).
//
// The weights stay 4-bit in HBM and are dequantised inside the kernel; the product runs on
// 16-bit operands ("LLM Weight Quantization - GPTQ, AWQ, SmoothQuant, FP8 & INT4/INT8
// Trade-offs", "The vocabulary" and "format notes").  The dequantised weight is
// x_hat = scale * (q - z) ("DL S067 · Quantization", §1), formed exactly in fp32 by one
// mixed-precision fma per weight and rounded once to bf16.
//
// Block = 4 waves, tile = 256 rows of X x 256 rows of W, k walked in steps of 128.
//   * X: the block's 256 x 128 bf16 slice of each step is copied global -> LDS by the
//     direct-to-LDS loads of gfx950 (no registers), double-buffered: the copy for step s + 1
//     is issued at the start of step s.  Rows are XOR-swizzled in 16-byte chunks so that the
//     MFMA fragment reads hit 16 different bank groups.
//   * W: each wave owns 64 W rows; a lane loads the 32 codes (16 bytes) it needs per row and
//     step, one step ahead, and dequantises them in registers straight into MFMA operands, so
//     every weight of the tile is dequantised exactly once per block.
//   * One barrier per step, after the step's loads have landed.
// The k order inside a step is permuted identically for both operands (lane group q takes the
// 32 contiguous k of its codes), which leaves each output sum unchanged.
// MFMA: D[n][m] = sum_k W[n][k] X[m][k]; a lane's four accumulators are four consecutive n of
// one m, written as one 8-byte store into row-major Y.  Blocks are numbered so the tiles that
// share X rows land on one XCD (one L2).
#include <type_traits>

#include "q4_device.h"
#include "q4_internal.h"

namespace q4 {
namespace {

constexpr int kStepK = 128;                            // k per step
constexpr int kTileM = 128;                            // X rows per block
constexpr int kTileN = 256;                            // W rows per block (64 per wave)
constexpr uint32_t kRowBytes = kStepK * 2;             // one X row of a step in LDS
constexpr uint32_t kStageBytes = kTileM * kRowBytes;   // 32 KiB
constexpr uint32_t kWaveDma = kStageBytes / 4;         // bytes each wave copies per step
constexpr int kDmaOps = kWaveDma / 1024;               // 1 KiB copy instructions per wave
constexpr uint32_t kSzStage = 4 * (512 + 256);          // scale / zero words per stage

// Dequantise 8 codes (one dword, code k in bits 4k..4k+3) into 8 bf16 MFMA operand values.
// A nibble at bits 0..3 OR-ed into fp16 1024.0 (0x6400) reads as 1024 + q; a nibble at bits
// 4..7 OR-ed into fp16 64.0 (0x5400, ulp 1/16) reads as 64 + q.  With c1 = -s (1024 + z) and
// c64 = -s (64 + z), fma(1024 + q, s, c1) = fma(64 + q, s, c64) = s (q - z) exactly in fp32
// (fp16 scale x 5-bit integer), then rounded once to bf16.
template <bool SYM>
__device__ __forceinline__ u32x4 dequant8(uint32_t dw, float s, float c1, float c64) {
  if (SYM) dw ^= 0x88888888u;                     // two's complement nibble -> q + 8, z = 8
  const uint32_t d8 = dw >> 8;
  const f16x2 q0 = as_f16x2((dw & 0x000F000Fu) | 0x64006400u);   // k0, k4
  const f16x2 q1 = as_f16x2((dw & 0x00F000F0u) | 0x54005400u);   // k1, k5
  const f16x2 q2 = as_f16x2((d8 & 0x000F000Fu) | 0x64006400u);   // k2, k6
  const f16x2 q3 = as_f16x2((d8 & 0x00F000F0u) | 0x54005400u);   // k3, k7
  const float w0 = __builtin_fmaf((float)q0[0], s, c1);
  const float w4 = __builtin_fmaf((float)q0[1], s, c1);
  const float w1 = __builtin_fmaf((float)q1[0], s, c64);
  const float w5 = __builtin_fmaf((float)q1[1], s, c64);
  const float w2 = __builtin_fmaf((float)q2[0], s, c1);
  const float w6 = __builtin_fmaf((float)q2[1], s, c1);
  const float w3 = __builtin_fmaf((float)q3[0], s, c64);
  const float w7 = __builtin_fmaf((float)q3[1], s, c64);
  return u32x4{pack_bf16x2(w0, w1), pack_bf16x2(w2, w3), pack_bf16x2(w4, w5), pack_bf16x2(w6, w7)};
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

// EDGE = false: every tile of the launch is full (256 W rows, 128 X rows in range), so the
// per-lane parts of all addresses are the same for every row group and the rest is
// wave-uniform.  EDGE = true: the last row and / or column of tiles of a ragged shape; X rows
// past M are clamped to row M - 1 and W rows past N read as 0 (their outputs are dropped).
template <bool SYM, bool EDGE>
__global__ __launch_bounds__(256, 2) void prefill_kernel(
    const uint16_t* __restrict__ X, int M, int N, int K, int lg,
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
    const uint8_t* __restrict__ zeros, uint16_t* __restrict__ Y, int tiles_m, int tiles_n,
    int edge_row, int vec_store) {
  constexpr int MB = kTileM / 16;    // 16-row blocks of X
  constexpr int NB = 4;              // 16-row blocks of W per wave
  constexpr int RW = kTileM / 4;     // X rows each wave copies per step

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
    const int t = (tiles & 7) == 0 ? (b & 7) * (tiles >> 3) + (b >> 3) : b;
    bm = t / tiles_n;
    bn = t - bm * tiles_n;
  }
  const int m0 = bm * kTileM, n0 = bn * kTileN;
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
  const uint32_t rows_left = (uint32_t)min(N - n0, kTileN);
  const __amdgpu_buffer_rsrc_t rw = buffer_over(packed + (size_t)n0 * (size_t)(K / 2), rows_left * (uint32_t)(K / 2));
  const __amdgpu_buffer_rsrc_t rs = buffer_over(scales + (size_t)n0 * G, rows_left * (uint32_t)G * 2u);
  const __amdgpu_buffer_rsrc_t rz = buffer_over(zeros + (size_t)n0 * G, rows_left * (uint32_t)G);
  const uint32_t gl = (uint32_t)((32 * lq) >> lg);
  constexpr int NV = EDGE ? NB : 1;
  uint32_t voff_w[NV], voff_s[NV], voff_z[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const uint32_t r = EDGE ? (uint32_t)(64 * wave + 16 * v + li) : (uint32_t)li;
    voff_w[v] = r * (uint32_t)(K / 2) + 16u * (uint32_t)lq;
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

  u32x4 wq[2][NB];                  // codes: k = 32 lq .. 32 lq + 31 of the step, per W row
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
      const int rb = EDGE ? 0 : 64 * wave + 16 * nb;    // wave-uniform row of the block
      wq[R][nb] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
          rw, voff_w[v], rb * (K / 2) + ktc * (kStepK / 2), 0));
      if (EDGE) {
        ws[R][nb] = __builtin_amdgcn_raw_buffer_load_b16(rs, voff_s[v], 2 * (rb * G + gs), 0);
        wz[R][nb] = SYM ? 8u : (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rz, voff_z[v], rb * G + gs, 0);
      }
    }
  };

  // One step: copy X of step kt + 1 into the other buffer, load W codes of step kt + 1 into
  // the other slot, multiply step kt.
  auto step = [&](auto S, int kt) {
    constexpr int R = decltype(S)::value;
    // The previous barrier already waited for these registers; naming them here, before any
    // new load is issued, keeps the compiler's own wait for them from covering the new loads.
    asm volatile("" ::"v"(wq[R][0]), "v"(wq[R][1]), "v"(wq[R][2]), "v"(wq[R][3]));
    if (EDGE) {
      asm volatile("" ::"v"(ws[R][0]), "v"(ws[R][1]), "v"(ws[R][2]), "v"(ws[R][3]));
      if (!SYM) asm volatile("" ::"v"(wz[R][0]), "v"(wz[R][1]), "v"(wz[R][2]), "v"(wz[R][3]));
    }
    // This step's scale / zero words (copied during the previous step) -> registers.
    uint32_t sb[NB], zb[NB];
    if (!EDGE) {
      const uint32_t gs = (uint32_t)((kt * kStepK) >> lg);
      const uint32_t par = rg_r + gs;
      const uint8_t* st = xl + 2u * kStageBytes + (uint32_t)R * kSzStage;
      const uint8_t* srow = st + (uint32_t)wave * 512u + (uint32_t)li * 8u + 2u * gl + 2u * (par & 1u);
      const uint8_t* zrow = st + 2048u + (uint32_t)wave * 256u + (uint32_t)li * 4u + gl + (par & 3u);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        sb[nb] = *reinterpret_cast<const uint16_t*>(srow + 128 * nb);
        zb[nb] = SYM ? 8u : (uint32_t)zrow[64 * nb];
      }
    }
    copy_x(R ^ 1, kt + 1);
    if (!EDGE) copy_sz(R ^ 1, kt + 1);
    load_w(Slot<R ^ 1>{}, kt + 1);
    // Keep the loads here: left alone, the scheduler sinks them to the end of the step to
    // shorten register lifetimes, which exposes their whole latency at the barrier.
    __builtin_amdgcn_sched_barrier(0);

    float s[NB], c1[NB], c64[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      s[nb] = (float)__builtin_bit_cast(_Float16, (uint16_t)(EDGE ? ws[R][nb] : sb[nb]));
      const float zf = (float)(EDGE ? wz[R][nb] : zb[nb]);
      c1[nb] = -s[nb] * (1024.0f + zf);
      c64[nb] = -s[nb] * (64.0f + zf);
    }
    const uint8_t* xs = xl + (uint32_t)R * kStageBytes;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 a[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        a[nb] = __builtin_bit_cast(bf16x8, dequant8<SYM>(wq[R][nb][ks], s[nb], c1[nb], c64[nb]));
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
    asm volatile("" ::"v"(wq[R ^ 1][0]), "v"(wq[R ^ 1][1]), "v"(wq[R ^ 1][2]), "v"(wq[R ^ 1][3]));
    if (EDGE) {
      asm volatile("" ::"v"(ws[R ^ 1][0]), "v"(ws[R ^ 1][1]), "v"(ws[R ^ 1][2]), "v"(ws[R ^ 1][3]));
      if (!SYM) asm volatile("" ::"v"(wz[R ^ 1][0]), "v"(wz[R ^ 1][1]), "v"(wz[R ^ 1][2]), "v"(wz[R ^ 1][3]));
    }
    step_barrier();
  };

  copy_x(0, 0);
  if (!EDGE) copy_sz(0, 0);
  load_w(Slot<0>{}, 0);
  asm volatile("" ::"v"(wq[0][0]), "v"(wq[0][1]), "v"(wq[0][2]), "v"(wq[0][3]));
  if (EDGE) {
    asm volatile("" ::"v"(ws[0][0]), "v"(ws[0][1]), "v"(ws[0][2]), "v"(ws[0][3]));
    if (!SYM) asm volatile("" ::"v"(wz[0][0]), "v"(wz[0][1]), "v"(wz[0][2]), "v"(wz[0][3]));
  }
  step_barrier();

  // Straight-line body of two steps (one per buffer / register slot); an odd last step follows.
  int kt = 0;
  for (; kt + 2 <= KT; kt += 2) {
    step(Slot<0>{}, kt);
    step(Slot<1>{}, kt + 1);
  }
  if (kt < KT) step(Slot<0>{}, kt);

  // D[n][m]: lane (li, lq) holds n = 4 lq + e (e = 0..3) of column m = li.
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = m0 + mb * 16 + li;
      const int nbase = n0 + 64 * wave + nb * 16 + 4 * lq;
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

template <bool SYM>
hipError_t launch_sym(const void* X, int64_t M, int64_t N, int64_t K, int lg, const void* packed,
                      const void* scales, const void* zeros, void* Y, hipStream_t stream) {
  const int full_m = (int)(M / kTileM), full_n = (int)(N / kTileN);
  const int tiles_m = (int)((M + kTileM - 1) / kTileM);
  const int tiles_n = (int)((N + kTileN - 1) / kTileN);
  const int vec = (N % 4 == 0) && ((reinterpret_cast<uintptr_t>(Y) & 7) == 0);
  const int64_t full_blocks = (int64_t)full_m * full_n;
  if ((int64_t)tiles_m * tiles_n > 0x7fffffff) return hipErrorInvalidValue;
  if (full_blocks > 0) {
    hipLaunchKernelGGL((prefill_kernel<SYM, false>), dim3((unsigned)full_blocks), dim3(256), 0, stream,
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
    hipLaunchKernelGGL((prefill_kernel<SYM, true>), dim3((unsigned)edge_blocks), dim3(256), 0, stream,
                       (const uint16_t*)X, (int)M, (int)N, (int)K, lg, (const uint8_t*)packed,
                       (const uint16_t*)scales, (const uint8_t*)zeros, (uint16_t*)Y, tiles_m, tiles_n,
                       edge_row, vec);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

bool prefill_fits(int64_t M, int64_t N, int64_t K, int g) {
  // 32-bit offsets: a block's X rows and the W codes / scales behind one buffer resource
  // must span < 2 GiB.
  const int64_t lim = int64_t(1) << 31;
  return M >= kPrefillMinM && K % kStepK == 0 && g >= 32 && (g & (g - 1)) == 0 &&
         (int64_t)kTileM * K * 2 < lim && N * (K / 2) < lim && N * (K / g) * 2 < lim;
}

hipError_t launch_prefill(const void* X, int64_t M, int64_t N, int64_t K, int g, bool sym,
                          const void* packed, const void* scales, const void* zeros, void* Y,
                          hipStream_t stream) {
  int lg = 0;
  while ((1 << lg) < g) ++lg;
  return sym ? launch_sym<true>(X, M, N, K, lg, packed, scales, zeros, Y, stream)
             : launch_sym<false>(X, M, N, K, lg, packed, scales, zeros, Y, stream);
}

}  // namespace q4
