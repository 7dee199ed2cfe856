// C ABI of the q4 library: argument validation (no HIP call before it passes), kernel
// selection and launch on the caller's stream.  See include/q4.h for the contract.
#include "../../include/q4.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <initializer_list>

#include "q4_internal.h"

namespace {

constexpr int64_t kMaxDim = 0x7fffffff;

struct Range {
  uintptr_t lo, hi;
};

Range range_of(const void* p, int64_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + static_cast<uintptr_t>(bytes)};
}

bool overlap(const Range& a, const Range& b) {
  return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_shape(int64_t N, int64_t K, int32_t g, int32_t mode) {
  if (N < 1 || K < 1 || N > kMaxDim || K > kMaxDim) return Q4_ERR_SHAPE;
  if (g < 32 || g % 32 != 0 || K % g != 0) return Q4_ERR_GROUP;
  if (mode != Q4_ASYM && mode != Q4_SYM) return Q4_ERR_MODE;
  return Q4_OK;
}

// Compute units of the current device, cached per device id.
int num_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

bool gemv_fits(int64_t M, int64_t K) {
  return (M == 1 && K <= q4::kGemvMaxK) || (M == 2 && K <= q4::kGemvMaxK2);
}

// Q4_KERNEL_DECODE above 16 rows runs as launches of 16 rows (the last one M mod 16): every
// chunk's shape must fit the decode kernel.
bool decode_rows_fit(int64_t M, int64_t N, int64_t K, int32_t g) {
  if (M <= 16) return q4::decode_fits(M, N, K, g);
  return q4::decode_fits(16, N, K, g) && (M % 16 == 0 || q4::decode_fits(M % 16, N, K, g));
}

// Up to how many rows Q4_KERNEL_AUTO takes the decode kernel in 16-row launches, each of which
// reads W once, rather than the GEMM.  Below a few hundred rows the GEMM's time hardly depends
// on M: its blocks walk all of K, about 0.0117 us per k on MI355X (47.5 us at K = 4096, 93-96 us
// at K = 8192, M = 17 ... 384).  A decode launch is costed at 4.4 us, plus 0.001 us per k (its X
// start-up), plus its weight bytes at 4.5 TB/s, which is at or above what was measured (7.1 us
// for 4096 x 4096, 11.3 for 11008 x 4096, 16 for 8192 x 8192, 30 for 28672 x 8192).  So as many
// launches as fit in the GEMM's time, at least three and at most six: 4096 x 4096 and 8192 x
// 8192 at M = 64 take 28.4 and 63.8 us against 47.5 and 93.4 for the GEMM; 28672 x 8192 at
// M = 32 / 48 59 / 90 us against 96.
int64_t decode_max_rows(int64_t N, int64_t K, int32_t g) {
  const double bytes = (double)N * (double)K * (0.5 + 3.0 / (double)g);
  const double t_launch = 4.4 + 0.001 * (double)K + bytes / 4.5e6, t_gemm = 0.0117 * (double)K;   // us
  int64_t n = (int64_t)(t_gemm / t_launch);
  n = n < 3 ? 3 : (n > 6 ? 6 : n);
  return 16 * n;
}

// Q4_KERNEL_AUTO: the decode kernels for small M, the GEMM otherwise.
int auto_kernel(int64_t M, int64_t N, int64_t K, int32_t g) {
  if (M == 1 && gemv_fits(M, K)) return Q4_KERNEL_GEMV;
  if (q4::decode_fits(M, N, K, g)) return Q4_KERNEL_DECODE;
  if (gemv_fits(M, K)) return Q4_KERNEL_GEMV;
  if (M <= decode_max_rows(N, K, g) && decode_rows_fit(M, N, K, g)) return Q4_KERNEL_DECODE;
  return Q4_KERNEL_GEMM;
}

// bits: code width, 4 (packed [N, K/2]) or 8 (codes [N, K]).
int validate_matmul(const void* X, int64_t M, int64_t N, int64_t K, int32_t g, int32_t mode,
                    const void* packed, const void* scales, const void* zeros, const void* Y,
                    int bits = 4) {
  int st = check_shape(N, K, g, mode);
  if (st != Q4_OK) return st;
  if (M < 0 || M > kMaxDim) return Q4_ERR_SHAPE;
  if (M == 0) return Q4_OK;
  if (!X || !packed || !scales || !Y || (mode == Q4_ASYM && !zeros)) return Q4_ERR_NULL;
  if (!aligned(X, 16) || !aligned(packed, 16) || !aligned(scales, 2) || !aligned(Y, 2))
    return Q4_ERR_ALIGN;
  const int64_t G = K / g;
  const Range y = range_of(Y, M * N * 2);
  if (overlap(y, range_of(X, M * K * 2)) || overlap(y, range_of(packed, N * K * bits / 8)) ||
      overlap(y, range_of(scales, N * G * 2)) ||
      (mode == Q4_ASYM && overlap(y, range_of(zeros, N * G))))
    return Q4_ERR_ALIAS;
  return Q4_OK;
}

// Quantizer arguments: W [N, K] bf16 in, codes of `bits` bits, scales and zeros out.
int validate_quantize(const void* W, int64_t N, int64_t K, int32_t g, int32_t mode, const void* packed,
                      const void* scales, const void* zeros, int bits) {
  int st = check_shape(N, K, g, mode);
  if (st != Q4_OK) return st;
  if (!W || !packed || !scales || !zeros) return Q4_ERR_NULL;
  if (!aligned(W, 16) || !aligned(packed, 16) || !aligned(scales, 2)) return Q4_ERR_ALIGN;
  const int64_t G = K / g;
  const Range w = range_of(W, N * K * 2), p = range_of(packed, N * K * bits / 8),
              s = range_of(scales, N * G * 2), z = range_of(zeros, N * G);
  if (overlap(w, p) || overlap(w, s) || overlap(w, z) || overlap(p, s) || overlap(p, z) ||
      overlap(s, z))
    return Q4_ERR_ALIAS;
  return Q4_OK;
}

int finish(hipError_t e) { return e == hipSuccess ? Q4_OK : Q4_ERR_HIP; }

// True if any two of the ranges overlap.
bool any_overlap(std::initializer_list<Range> rs) {
  for (auto a = rs.begin(); a != rs.end(); ++a)
    for (auto b = a + 1; b != rs.end(); ++b)
      if (overlap(*a, *b)) return true;
  return false;
}

constexpr int kMaxAlphas = 64;

}  // namespace

extern "C" {

int q4_version(void) { return Q4_VERSION; }

const char* q4_status_string(int status) {
  switch (status) {
    case Q4_OK: return "ok";
    case Q4_ERR_NULL: return "a required pointer is NULL";
    case Q4_ERR_SHAPE: return "invalid shape: need N >= 1, K >= 1, M >= 0, all <= 2^31-1";
    case Q4_ERR_GROUP: return "invalid group size: need g >= 32, g % 32 == 0 and K % g == 0";
    case Q4_ERR_MODE: return "invalid mode, kernel selector or output type";
    case Q4_ERR_ALIGN:
      return "misaligned pointer: W, X, packed and dequantize's out need 16 bytes; scales, Y need 2";
    case Q4_ERR_HIP: return "the HIP runtime rejected a kernel launch";
    case Q4_ERR_ALIAS: return "an output buffer overlaps an input or another output";
    case Q4_ERR_UNSUPPORTED: return "the chosen kernel does not support this shape";
    case Q4_ERR_WORKSPACE: return "workspace smaller than the matching *_workspace_bytes() requires";
    case Q4_ERR_VALUE: return "a numeric parameter is out of range (e.g. GPTQ damping not finite and >= 0)";
    case Q4_ERR_SCRATCH: return "the sizes need more scratch than the library's static buffer holds";
    default: return "unknown status";
  }
}

int q4_quantize_rtn(const void* W, int64_t N, int64_t K, int32_t g, int32_t mode, void* packed,
                    void* scales, void* zeros, void* stream) {
  const int st = validate_quantize(W, N, K, g, mode, packed, scales, zeros, 4);
  if (st != Q4_OK) return st;
  return finish(q4::launch_quantize(W, N, K, g, mode == Q4_SYM, packed, scales, zeros, num_cus(),
                                    static_cast<hipStream_t>(stream)));
}

int q4_select_kernel(int64_t M, int64_t N, int64_t K, int32_t g) {
  int st = check_shape(N, K, g, Q4_ASYM);
  if (st != Q4_OK) return st;
  if (M < 0 || M > kMaxDim) return Q4_ERR_SHAPE;
  if (M == 0) return Q4_KERNEL_GEMM;
  return auto_kernel(M, N, K, g);
}

int q4_matmul_kernel(const void* X, int64_t M, int64_t N, int64_t K, int32_t g, int32_t mode,
                     const void* packed, const void* scales, const void* zeros, void* Y,
                     int32_t kernel, void* stream) {
  if (kernel < Q4_KERNEL_AUTO || kernel > Q4_KERNEL_DECODE) return Q4_ERR_MODE;
  int st = validate_matmul(X, M, N, K, g, mode, packed, scales, zeros, Y);
  if (st != Q4_OK) return st;
  if (M == 0) return Q4_OK;
  if (kernel == Q4_KERNEL_AUTO) kernel = auto_kernel(M, N, K, g);
  if (kernel == Q4_KERNEL_GEMV && !gemv_fits(M, K)) return Q4_ERR_UNSUPPORTED;
  if (kernel == Q4_KERNEL_DECODE && !decode_rows_fit(M, N, K, g)) return Q4_ERR_UNSUPPORTED;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool sym = mode == Q4_SYM;
  if (kernel == Q4_KERNEL_GEMV)
    return finish(q4::launch_gemv(X, (int)M, N, K, g, sym, packed, scales, zeros, Y, num_cus(), s));
  if (kernel == Q4_KERNEL_DECODE) {
    // 16 rows of X and Y per launch (row-major: a chunk is a contiguous block of each)
    for (int64_t r = 0; r < M; r += 16) {
      const hipError_t e = q4::launch_decode(static_cast<const uint16_t*>(X) + r * K, (int)(M - r < 16 ? M - r : 16),
                                             N, K, g, sym, packed, scales, zeros,
                                             static_cast<uint16_t*>(Y) + r * N, num_cus(), s);
      if (e != hipSuccess) return finish(e);
    }
    return Q4_OK;
  }
  if (q4::prefill_fits(M, N, K, g))
    return finish(q4::launch_prefill(X, M, N, K, g, sym, packed, scales, zeros, Y, num_cus(), s));
  return finish(q4::launch_gemm(X, M, N, K, g, sym, packed, scales, zeros, Y, num_cus(), s));
}

int q4_quantize_rtn_scaled(const void* W, const void* s, int64_t N, int64_t K, int32_t g, int32_t mode,
                           void* packed, void* scales, void* zeros, void* stream) {
  int st = check_shape(N, K, g, mode);
  if (st != Q4_OK) return st;
  if (!W || !s || !packed || !scales || !zeros) return Q4_ERR_NULL;
  if (!aligned(W, 16) || !aligned(s, 16) || !aligned(packed, 16) || !aligned(scales, 2)) return Q4_ERR_ALIGN;
  const int64_t G = K / g;
  const Range w = range_of(W, N * K * 2), sc = range_of(s, K * 4), p = range_of(packed, N * K / 2),
              sg = range_of(scales, N * G * 2), z = range_of(zeros, N * G);
  if (any_overlap({p, sg, z}) || any_overlap({w, p}) || any_overlap({w, sg}) || any_overlap({w, z}) ||
      any_overlap({sc, p}) || any_overlap({sc, sg}) || any_overlap({sc, z}))
    return Q4_ERR_ALIAS;
  return finish(q4::launch_quantize(W, N, K, g, mode == Q4_SYM, packed, scales, zeros, num_cus(),
                                    static_cast<hipStream_t>(stream), static_cast<const float*>(s)));
}

int q4_scale_columns(const void* A, int64_t rows, int64_t cols, const void* s, int32_t op, void* out,
                     void* stream) {
  if (rows < 0 || rows > kMaxDim || cols < 8 || cols > kMaxDim) return Q4_ERR_SHAPE;
  if (cols % 8 != 0) return Q4_ERR_SHAPE;
  if (op != Q4_SCALE_MUL && op != Q4_SCALE_DIV) return Q4_ERR_MODE;
  if (rows == 0) return Q4_OK;
  if (!A || !s || !out) return Q4_ERR_NULL;
  if (!aligned(A, 16) || !aligned(s, 16) || !aligned(out, 16)) return Q4_ERR_ALIGN;
  const Range a = range_of(A, rows * cols * 2), o = range_of(out, rows * cols * 2), sc = range_of(s, cols * 4);
  if ((A != out && overlap(a, o)) || overlap(sc, o)) return Q4_ERR_ALIAS;
  return finish(q4::launch_scale_columns(A, rows, cols, s, op == Q4_SCALE_DIV, out, num_cus(),
                                         static_cast<hipStream_t>(stream)));
}

int64_t q4_awq_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t g, int32_t n_alpha) {
  int st = check_shape(N, K, g, Q4_ASYM);
  if (st != Q4_OK) return st;
  if (M < 1 || M > kMaxDim || n_alpha < 1 || n_alpha > kMaxAlphas) return Q4_ERR_SHAPE;
  return (int64_t)q4::awq_layout(M, N, K, g, n_alpha).bytes;
}

int q4_awq_search(const void* X, int64_t M, const void* Yref, const void* W, int64_t N, int64_t K,
                  int32_t g, int32_t mode, int32_t n_alpha, void* workspace, int64_t workspace_bytes,
                  void* s_out, void* packed, void* scales, void* zeros, void* errors, void* best,
                  void* stream) {
  int st = check_shape(N, K, g, mode);
  if (st != Q4_OK) return st;
  if (M < 1 || M > kMaxDim || n_alpha < 1 || n_alpha > kMaxAlphas) return Q4_ERR_SHAPE;
  if (!X || !Yref || !W || !workspace || !s_out || !packed || !scales || !zeros || !errors || !best)
    return Q4_ERR_NULL;
  if (!aligned(X, 16) || !aligned(W, 16) || !aligned(Yref, 2) || !aligned(workspace, 256) ||
      !aligned(s_out, 16) || !aligned(packed, 16) || !aligned(scales, 2) || !aligned(errors, 8) ||
      !aligned(best, 4))
    return Q4_ERR_ALIGN;
  const q4::AwqLayout L = q4::awq_layout(M, N, K, g, n_alpha);
  if (workspace_bytes < (int64_t)L.bytes) return Q4_ERR_WORKSPACE;
  const int64_t G = K / g;
  const Range x = range_of(X, M * K * 2), yr = range_of(Yref, M * N * 2), w = range_of(W, N * K * 2),
              ws = range_of(workspace, (int64_t)L.bytes), so = range_of(s_out, K * 4),
              p = range_of(packed, N * K / 2), sg = range_of(scales, N * G * 2), z = range_of(zeros, N * G),
              e = range_of(errors, (int64_t)n_alpha * 8), b = range_of(best, 4);
  for (const Range& out : {ws, so, p, sg, z, e, b})
    if (overlap(out, x) || overlap(out, yr) || overlap(out, w)) return Q4_ERR_ALIAS;
  if (any_overlap({ws, so, p, sg, z, e, b})) return Q4_ERR_ALIAS;

  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const bool sym = mode == Q4_SYM;
  char* base = static_cast<char*>(workspace);
  float* s_all = reinterpret_cast<float*>(base + L.scales_all);
  hipError_t he = q4::launch_absmean(X, M, K, base + L.partial, base + L.absmean, hs);
  if (he == hipSuccess) he = q4::launch_awq_scales(base + L.absmean, K, n_alpha, s_all, hs);
  for (int i = 0; i < n_alpha && he == hipSuccess; ++i) {
    const float* si = s_all + (size_t)i * K;
    he = q4::launch_quantize(W, N, K, g, sym, base + L.packed, base + L.qscales, base + L.qzeros, num_cus(),
                             hs, si);
    if (he == hipSuccess) he = q4::launch_scale_columns(X, M, K, si, true, base + L.xs, num_cus(), hs);
    if (he == hipSuccess) {
      const int mst = q4_matmul(base + L.xs, M, N, K, g, mode, base + L.packed, base + L.qscales,
                                base + L.qzeros, base + L.y, stream);
      if (mst != Q4_OK) return mst;
    }
    if (he == hipSuccess)
      he = q4::launch_sq_err(base + L.y, Yref, M * N, base + L.err_partial,
                             static_cast<double*>(errors) + i, hs);
  }
  if (he == hipSuccess) he = q4::launch_awq_select(errors, n_alpha, s_all, K, best, s_out, hs);
  if (he == hipSuccess)
    he = q4::launch_quantize(W, N, K, g, sym, packed, scales, zeros, num_cus(), hs,
                             static_cast<const float*>(s_out));
  return finish(he);
}

int q4_dequantize(int64_t N, int64_t K, int32_t g, int32_t mode, const void* packed,
                  const void* scales, const void* zeros, void* out, int32_t out_dtype,
                  void* stream) {
  int st = check_shape(N, K, g, mode);
  if (st != Q4_OK) return st;
  if (out_dtype != Q4_DTYPE_BF16 && out_dtype != Q4_DTYPE_F16) return Q4_ERR_MODE;
  if (!packed || !scales || !out || (mode == Q4_ASYM && !zeros)) return Q4_ERR_NULL;
  if (!aligned(packed, 16) || !aligned(scales, 2) || !aligned(out, 16)) return Q4_ERR_ALIGN;
  const int64_t G = K / g;
  const Range o = range_of(out, N * K * 2);
  if (overlap(o, range_of(packed, N * K / 2)) || overlap(o, range_of(scales, N * G * 2)) ||
      (mode == Q4_ASYM && overlap(o, range_of(zeros, N * G))))
    return Q4_ERR_ALIAS;
  return finish(q4::launch_dequantize(packed, scales, zeros, N, K, g, mode == Q4_SYM, out,
                                      out_dtype == Q4_DTYPE_F16, num_cus(),
                                      static_cast<hipStream_t>(stream)));
}

int q4_matmul(const void* X, int64_t M, int64_t N, int64_t K, int32_t g, int32_t mode,
              const void* packed, const void* scales, const void* zeros, void* Y, void* stream) {
  return q4_matmul_kernel(X, M, N, K, g, mode, packed, scales, zeros, Y, Q4_KERNEL_AUTO, stream);
}

int q4_quantize_rtn8(const void* W, int64_t N, int64_t K, int32_t g, int32_t mode, void* codes,
                     void* scales, void* zeros, void* stream) {
  const int st = validate_quantize(W, N, K, g, mode, codes, scales, zeros, 8);
  if (st != Q4_OK) return st;
  return finish(q4::launch_quantize8(W, N, K, g, mode == Q4_SYM, codes, scales, zeros, num_cus(),
                                     static_cast<hipStream_t>(stream)));
}

int q4_select_kernel_w8(int64_t M, int64_t N, int64_t K, int32_t g) {
  int st = check_shape(N, K, g, Q4_ASYM);
  if (st != Q4_OK) return st;
  if (M < 0 || M > kMaxDim) return Q4_ERR_SHAPE;
  return (M >= 1 && q4::gemv8_fits(M, K)) ? Q4_KERNEL_GEMV : Q4_KERNEL_GEMM;
}

int q4_matmul_w8(const void* X, int64_t M, int64_t N, int64_t K, int32_t g, int32_t mode,
                 const void* codes, const void* scales, const void* zeros, void* Y, int32_t kernel,
                 void* stream) {
  if (kernel < Q4_KERNEL_AUTO || kernel > Q4_KERNEL_DECODE) return Q4_ERR_MODE;
  int st = validate_matmul(X, M, N, K, g, mode, codes, scales, zeros, Y, 8);
  if (st != Q4_OK) return st;
  if (M == 0) return Q4_OK;
  if (kernel == Q4_KERNEL_AUTO) kernel = q4_select_kernel_w8(M, N, K, g);
  if (kernel == Q4_KERNEL_DECODE || (kernel == Q4_KERNEL_GEMV && !q4::gemv8_fits(M, K)))
    return Q4_ERR_UNSUPPORTED;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool sym = mode == Q4_SYM;
  if (kernel == Q4_KERNEL_GEMV)
    return finish(q4::launch_gemv8(X, (int)M, N, K, g, sym, codes, scales, zeros, Y, num_cus(), s));
  if (q4::prefill_fits(M, N, K, g, 8))
    return finish(q4::launch_prefill8(X, M, N, K, g, sym, codes, scales, zeros, Y, num_cus(), s));
  return finish(q4::launch_gemm8(X, M, N, K, g, sym, codes, scales, zeros, Y, num_cus(), s));
}

int64_t q4_gptq_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t g) {
  int st = check_shape(N, K, g, Q4_ASYM);
  if (st != Q4_OK) return st;
  if (M < 1 || M > kMaxDim || K > q4::kGptqMaxK) return Q4_ERR_SHAPE;
  return q4::gptq_layout(N, K).bytes;
}

int q4_gptq(const void* X, int64_t M, const void* W, int64_t N, int64_t K, int32_t g, int32_t mode, float damp,
            void* workspace, int64_t workspace_bytes, void* packed, void* scales, void* zeros, void* info,
            void* stream) {
  int st = check_shape(N, K, g, mode);
  if (st != Q4_OK) return st;
  if (M < 1 || M > kMaxDim || K > q4::kGptqMaxK) return Q4_ERR_SHAPE;
  if (!std::isfinite(damp) || damp < 0.0f) return Q4_ERR_VALUE;
  if (!X || !W || !workspace || !packed || !scales || !zeros || !info) return Q4_ERR_NULL;
  if (!aligned(X, 16) || !aligned(W, 16) || !aligned(packed, 16) || !aligned(scales, 2) ||
      !aligned(workspace, 256) || !aligned(info, 4))
    return Q4_ERR_ALIGN;
  const q4::GptqLayout L = q4::gptq_layout(N, K);
  if (workspace_bytes < L.bytes) return Q4_ERR_WORKSPACE;
  const int64_t G = K / g;
  const Range x = range_of(X, M * K * 2), w = range_of(W, N * K * 2), ws = range_of(workspace, L.bytes),
              p = range_of(packed, N * K / 2), s = range_of(scales, N * G * 2), z = range_of(zeros, N * G),
              in = range_of(info, 4);
  for (const Range& o : {ws, p, s, z, in})
    if (overlap(o, x) || overlap(o, w)) return Q4_ERR_ALIAS;
  if (any_overlap({ws, p, s, z, in})) return Q4_ERR_ALIAS;
  return finish(q4::launch_gptq(X, M, W, N, K, g, mode == Q4_SYM, damp, workspace, packed, scales, zeros,
                                static_cast<int*>(info), num_cus(), static_cast<hipStream_t>(stream)));
}

}  // extern "C"
