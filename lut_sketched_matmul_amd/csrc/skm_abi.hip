// C ABI of the sketched-weight matmul: argument checks and kernel selection.
// The formulas, layouts and error rules are documented in sketch_matmul.h.
#include "sketch_matmul.h"

#include <cmath>
#include <mutex>

#include "skm_common.h"
#include "skm_launch.h"

// Scratch of sketch_matmul_bwd_noalloc: one array per GPU, held until the
// process ends. Host code never uses this name as a device address: the
// address comes from hipGetSymbolAddress, looked up once per device (see
// noalloc_scratch below).
constexpr size_t kScratchBytes = size_t(8) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

using skm::Problem;

constexpr int kVersion = 100;  // 0.1.0
constexpr int64_t kMaxFactorD = int64_t(1) << 16;  // sketch_hessian_factor: the tile grid stays below 2^31 blocks

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(int dt) { return dt == SKM_F32 ? 4 : 2; }

bool valid_dtype(int dt) { return dt == SKM_F32 || dt == SKM_F16 || dt == SKM_BF16; }

// (activation dtype, table dtype) pairs with a kernel
bool supported_pair(int x_dt, int lut_dt) {
  if (!valid_dtype(x_dt) || !valid_dtype(lut_dt)) return false;
  if (x_dt == SKM_F32 || lut_dt == SKM_F32) return x_dt == SKM_F32 && lut_dt == SKM_F32;
  return true;
}

int check_shape(int64_t m, int64_t n, int64_t d, int b, int gpr) {
  if (b < 2 || b > 4) return SKM_EINVAL;
  if (m < 0 || n < 1 || d < 32 || gpr < 1) return SKM_EINVAL;
  if (d % gpr != 0) return SKM_EINVAL;
  if ((d / gpr) % 32 != 0) return SKM_EINVAL;
  // indices of one launch are addressed with 32-bit table offsets and 64-bit
  // element offsets; keep every dimension well inside those ranges
  if (n > (int64_t(1) << 31) || d > (int64_t(1) << 31) || m > (int64_t(1) << 31)) return SKM_EINVAL;
  return SKM_OK;
}

struct Range {
  const void* p;
  int64_t bytes;
};

bool overlap(Range a, Range b) {
  if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + (uintptr_t)b.bytes && b0 < a0 + (uintptr_t)a.bytes;
}

int status_of(hipError_t e) { return e == hipSuccess ? SKM_OK : SKM_EHIP; }

// finite and at least lo
bool finite_in(float v, float lo) { return std::isfinite(v) && v >= lo; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// bf16 activations with f16 tables: the matrix-core operands are f16, and
// the activations (forward) or output gradients (dX) are prescaled per row
bool prescaled_pair(int x_dt, int lut_dt) { return x_dt == SKM_BF16 && lut_dt == SKM_F16; }

// whether a forward call of these sizes reads row exponents of X from the
// workspace (the GEMM, and the decode when it does not stage its activations)
bool fwd_reads_rexp(const Problem& p, int x_dt, int lut_dt) {
  if (!prescaled_pair(x_dt, lut_dt) || p.m < 1) return false;
  if (skm::decode_supported(p)) return !skm::decode_stages_activations(p, false, 1, true);
  return true;
}

}  // namespace

extern "C" {

int sketch_version(void) { return kVersion; }

const char* sketch_status_str(int status) {
  switch (status) {
    case SKM_OK: return "ok";
    case SKM_EINVAL: return "invalid argument (size, bit width, group count or NULL pointer)";
    case SKM_EUNSUPPORTED: return "unsupported dtype combination";
    case SKM_EALIGN: return "pointer not 16-byte aligned";
    case SKM_EWORKSPACE: return "workspace too small";
    case SKM_EHIP: return "HIP runtime error at launch";
    case SKM_EALIAS: return "output buffer overlaps an input buffer";
    default: return "unknown status";
  }
}

int sketch_unpack_indices(const uint8_t* idx_packed, int64_t n, int64_t d, int b, uint8_t* idx,
                          hipStream_t stream) {
  int st = check_shape(0, n, d, b, 1);
  if (st != SKM_OK) return st;
  if (!idx_packed || !idx) return SKM_EINVAL;
  if (!aligned16(idx_packed) || !aligned16(idx)) return SKM_EALIGN;
  if (overlap({idx, n * d}, {idx_packed, n * d * b / 8})) return SKM_EALIAS;
  const Problem p{0, n, d, b, 1};
  return status_of(skm::launch_unpack(idx_packed, p, idx, stream));
}

int sketch_dequant(const uint8_t* idx_packed, const void* lut, int lut_dtype, int64_t n, int64_t d, int b, int gpr,
                   void* W, hipStream_t stream) {
  int st = check_shape(0, n, d, b, gpr);
  if (st != SKM_OK) return st;
  if (!valid_dtype(lut_dtype)) return SKM_EUNSUPPORTED;
  if (!idx_packed || !lut || !W) return SKM_EINVAL;
  if (!aligned16(idx_packed) || !aligned16(lut) || !aligned16(W)) return SKM_EALIGN;
  const int es = elem_bytes(lut_dtype);
  const Range out{W, n * d * es};
  if (overlap(out, {idx_packed, n * d * b / 8}) || overlap(out, {lut, n * gpr * (int64_t(1) << b) * es}))
    return SKM_EALIAS;
  const Problem p{0, n, d, b, gpr};
  return status_of(skm::launch_dequant(idx_packed, lut, lut_dtype, p, W, stream));
}

size_t sketch_matmul_fwd_workspace(int64_t m, int64_t n, int64_t d, int b, int gpr, int x_dtype, int lut_dtype) {
  if (check_shape(m, n, d, b, gpr) != SKM_OK || !supported_pair(x_dtype, lut_dtype)) return 0;
  const Problem p{m, n, d, b, gpr};
  return fwd_reads_rexp(p, x_dtype, lut_dtype) ? align256((size_t)m * 4) : 0;
}

int sketch_matmul_fwd(const void* X, int x_dtype, const uint8_t* idx_packed, const void* lut, int lut_dtype,
                      int64_t m, int64_t n, int64_t d, int b, int gpr, void* Y, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  int st = check_shape(m, n, d, b, gpr);
  if (st != SKM_OK) return st;
  if (!supported_pair(x_dtype, lut_dtype)) return SKM_EUNSUPPORTED;
  if (!idx_packed || !lut) return SKM_EINVAL;
  if (m > 0 && (!X || !Y)) return SKM_EINVAL;
  if (!aligned16(idx_packed) || !aligned16(lut) || (X && !aligned16(X)) || (Y && !aligned16(Y)) ||
      (workspace && !aligned16(workspace)))
    return SKM_EALIGN;
  const size_t ws_need = sketch_matmul_fwd_workspace(m, n, d, b, gpr, x_dtype, lut_dtype);
  if (workspace_bytes < ws_need || (ws_need && !workspace)) return SKM_EWORKSPACE;
  const int xs = elem_bytes(x_dtype), ls = elem_bytes(lut_dtype);
  const Range out{Y, m * n * xs}, ws{workspace, (int64_t)ws_need};
  const Range ins[3] = {{X, m * d * xs}, {idx_packed, n * d * b / 8}, {lut, n * gpr * (int64_t(1) << b) * ls}};
  for (const Range& r : ins)
    if (overlap(out, r) || overlap(ws, r)) return SKM_EALIAS;
  if (overlap(out, ws)) return SKM_EALIAS;
  if (m == 0) return SKM_OK;
  const Problem p{m, n, d, b, gpr};
  if (x_dtype == SKM_F32)
    return status_of(skm::launch_fwd_f32((const float*)X, idx_packed, (const float*)lut, p, (float*)Y, stream));
  int32_t* rexp = nullptr;
  if (ws_need) {
    rexp = static_cast<int32_t*>(workspace);
    st = status_of(skm::launch_row_exp(X, m, d, rexp, stream));
    if (st != SKM_OK) return st;
  }
  if (skm::decode_supported(p))
    return status_of(skm::launch_decode(X, x_dtype, idx_packed, lut, lut_dtype, p, Y, rexp, stream));
  if (skm::gemm_fwd_supported(p))
    return status_of(skm::launch_gemm_fwd(X, x_dtype, idx_packed, lut, lut_dtype, p, Y, rexp, stream));
  return SKM_EUNSUPPORTED;
}

int sketch_matmul_fwd_multi(const void* X, int x_dtype, const uint8_t* idx_packed, const void* luts, int lut_dtype,
                            const int32_t* lut_set, int n_sets, int64_t m, int64_t n, int64_t d, int b, int gpr,
                            void* Y, hipStream_t stream) {
  int st = check_shape(m, n, d, b, gpr);
  if (st != SKM_OK) return st;
  if (!supported_pair(x_dtype, lut_dtype)) return SKM_EUNSUPPORTED;
  if (!idx_packed || !luts || n_sets < 1) return SKM_EINVAL;
  if (m > 0 && (!X || !Y || !lut_set)) return SKM_EINVAL;
  if (!aligned16(idx_packed) || !aligned16(luts) || (X && !aligned16(X)) || (Y && !aligned16(Y)) ||
      ((uintptr_t)lut_set & 3u) != 0)
    return SKM_EALIGN;
  const int xs = elem_bytes(x_dtype), ls = elem_bytes(lut_dtype);
  const Range out{Y, m * n * xs};
  if (overlap(out, {X, m * d * xs}) || overlap(out, {idx_packed, n * d * b / 8}) ||
      overlap(out, {luts, (int64_t)n_sets * n * gpr * (int64_t(1) << b) * ls}) || overlap(out, {lut_set, m * 4}))
    return SKM_EALIAS;
  if (m == 0) return SKM_OK;
  const Problem p{m, n, d, b, gpr};
  if (x_dtype == SKM_F32 || !skm::decode_multi_supported(p, prescaled_pair(x_dtype, lut_dtype)))
    return SKM_EUNSUPPORTED;
  return status_of(skm::launch_decode_multi(X, x_dtype, idx_packed, luts, lut_dtype, lut_set, n_sets, p, Y, stream));
}

// Backward workspace: [row exponents of dY: m int32, 256-byte aligned]
// (bf16 dY with f16 tables, read by dX), then [partial dLUT tables of the
// token ranges] (16-bit path, when the table gradient is split over tokens)
size_t bwd_rexp_bytes(int64_t m, int io_dtype, int lut_dtype) {
  return prescaled_pair(io_dtype, lut_dtype) && m > 0 ? align256((size_t)m * 4) : 0;
}

size_t sketch_matmul_bwd_workspace(int64_t m, int64_t n, int64_t d, int b, int gpr, int io_dtype, int lut_dtype) {
  if (check_shape(m, n, d, b, gpr) != SKM_OK || !supported_pair(io_dtype, lut_dtype)) return 0;
  const Problem p{m, n, d, b, gpr};
  const size_t part = io_dtype == SKM_F32 || m < 1 ? 0 : skm::dlut_partial_bytes(p);
  return bwd_rexp_bytes(m, io_dtype, lut_dtype) + part;
}

int sketch_matmul_bwd(const void* dY, const void* X, int io_dtype, const uint8_t* idx_packed, const void* lut,
                      int lut_dtype, int64_t m, int64_t n, int64_t d, int b, int gpr, float* dX, float* dLUT,
                      int accumulate, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_shape(m, n, d, b, gpr);
  if (st != SKM_OK) return st;
  if (!supported_pair(io_dtype, lut_dtype)) return SKM_EUNSUPPORTED;
  if (!idx_packed || !lut) return SKM_EINVAL;
  if (accumulate != 0 && accumulate != 1) return SKM_EINVAL;
  if (m > 0 && !dY && (dX || dLUT)) return SKM_EINVAL;
  if (m > 0 && dLUT && !X) return SKM_EINVAL;
  if (!aligned16(idx_packed) || !aligned16(lut) || (dY && !aligned16(dY)) || (X && !aligned16(X)) ||
      (dX && !aligned16(dX)) || (dLUT && !aligned16(dLUT)) || (workspace && !aligned16(workspace)))
    return SKM_EALIGN;
  const size_t ws_need = sketch_matmul_bwd_workspace(m, n, d, b, gpr, io_dtype, lut_dtype);
  if (workspace_bytes < ws_need || (ws_need && !workspace)) return SKM_EWORKSPACE;
  const int xs = elem_bytes(io_dtype), ls = elem_bytes(lut_dtype);
  const int64_t K = int64_t(1) << b;
  const Range ins[4] = {{dY, m * n * xs}, {X, m * d * xs}, {idx_packed, n * d * b / 8}, {lut, n * gpr * K * ls}};
  const Range odx{dX, m * d * 4}, odl{dLUT, n * gpr * K * 4}, ows{workspace, (int64_t)ws_need};
  for (const Range& r : ins)
    if (overlap(odx, r) || overlap(odl, r) || overlap(ows, r)) return SKM_EALIAS;
  if (overlap(odx, odl) || overlap(odx, ows) || overlap(odl, ows)) return SKM_EALIAS;

  const Problem p{m, n, d, b, gpr};
  if (m == 0) {
    if (dLUT && !accumulate) return status_of(skm::launch_zero_f32(dLUT, n * gpr * K, stream));
    return SKM_OK;
  }
  if (io_dtype == SKM_F32) {
    if (dX) {
      st = status_of(skm::launch_dx_f32((const float*)dY, idx_packed, (const float*)lut, p, dX, stream));
      if (st != SKM_OK) return st;
    }
    if (dLUT)
      return status_of(skm::launch_dlut_f32((const float*)dY, (const float*)X, idx_packed, p, dLUT, accumulate,
                                            stream));
    return SKM_OK;
  }
  if (!skm::gemm_bwd_supported(p)) return SKM_EUNSUPPORTED;
  if (dX) {
    int32_t* rexp = nullptr;
    if (prescaled_pair(io_dtype, lut_dtype)) {
      rexp = static_cast<int32_t*>(workspace);
      st = status_of(skm::launch_row_exp(dY, m, n, rexp, stream));
      if (st != SKM_OK) return st;
    }
    st = status_of(skm::launch_gemm_dx(dY, io_dtype, idx_packed, lut, lut_dtype, p, dX, rexp, stream));
    if (st != SKM_OK) return st;
  }
  if (dLUT) {
    float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + bwd_rexp_bytes(m, io_dtype, lut_dtype));
    return status_of(skm::launch_gemm_dlut(dY, X, io_dtype, idx_packed, p, dLUT, accumulate, part, stream));
  }
  return SKM_OK;
}

// Device address of this GPU's scratch array (the current device), looked up
// with that device current on its first use and kept per device; nullptr on
// failure.
static void* noalloc_scratch() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

int sketch_matmul_bwd_noalloc(const void* dY, const void* X, int io_dtype, const uint8_t* idx_packed,
                              const void* lut, int lut_dtype, int64_t m, int64_t n, int64_t d, int b, int gpr,
                              float* dX, float* dLUT, int accumulate, hipStream_t stream) {
  // (invalid arguments give a size of 0 and are rejected by sketch_matmul_bwd)
  const size_t need = sketch_matmul_bwd_workspace(m, n, d, b, gpr, io_dtype, lut_dtype);
  if (need > kScratchBytes) return SKM_EWORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    ws = noalloc_scratch();
    if (!ws) return SKM_EHIP;
  }
  return sketch_matmul_bwd(dY, X, io_dtype, idx_packed, lut, lut_dtype, m, n, d, b, gpr, dX, dLUT, accumulate, ws,
                           ws ? kScratchBytes : 0, stream);
}

int sketch_column_weights(const float* U, int64_t d, float* h, hipStream_t stream) {
  if (d < 1 || d > (int64_t(1) << 20)) return SKM_EINVAL;
  if (!U || !h) return SKM_EINVAL;
  if (!aligned16(U) || !aligned16(h)) return SKM_EALIGN;
  if (overlap({h, d * 4}, {U, d * d * 4})) return SKM_EALIAS;
  return status_of(skm::launch_col_weights(U, d, h, stream));
}

int sketch_lloyd(const float* W, const float* h, int64_t n, int64_t d, int b, int gpr, int iters, void* lut,
                 int lut_dtype, hipStream_t stream) {
  int st = check_shape(0, n, d, b, gpr);
  if (st) return st;
  if (iters < 0) return SKM_EINVAL;
  if (!valid_dtype(lut_dtype)) return SKM_EUNSUPPORTED;
  if (!W || !h || !lut) return SKM_EINVAL;
  if (!aligned16(W) || !aligned16(h) || !aligned16(lut)) return SKM_EALIGN;
  const Range o{lut, n * gpr * (int64_t(1) << b) * elem_bytes(lut_dtype)};
  if (overlap(o, {W, n * d * 4}) || overlap(o, {h, d * 4})) return SKM_EALIAS;
  const Problem p{0, n, d, b, gpr};
  return status_of(skm::launch_lloyd(W, h, p, iters, lut, lut_dtype, stream));
}

size_t sketch_hessian_factor_workspace(int64_t d) {
  return d >= 1 && d <= kMaxFactorD ? skm::hessian_factor_workspace_bytes(d) : 0;
}

int sketch_hessian_factor(const double* H, int64_t d, double damp, float* U, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  if (d < 1 || d > kMaxFactorD) return SKM_EINVAL;
  if (!(damp >= 0.0) || !std::isfinite(damp)) return SKM_EINVAL;
  if (!H || !U || !workspace) return SKM_EINVAL;
  if (!aligned16(H) || !aligned16(U) || !aligned16(workspace)) return SKM_EALIGN;
  const size_t need = skm::hessian_factor_workspace_bytes(d);
  if (workspace_bytes < need) return SKM_EWORKSPACE;
  const Range h{H, d * d * 8}, u{U, d * d * 4}, w{workspace, (int64_t)need};
  if (overlap(u, h) || overlap(w, h) || overlap(u, w)) return SKM_EALIAS;
  return status_of(skm::launch_hessian_factor(H, d, damp, U, workspace, stream));
}

size_t sketch_map_workspace(int64_t n) { return n > 0 ? skm::map_workspace_bytes(n) : 0; }

int sketch_map(float* W, const float* U, const void* lut, int lut_dtype, int64_t n, int64_t d, int b, int gpr,
               uint8_t* idx_packed, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_shape(0, n, d, b, gpr);
  if (st) return st;
  // the trailing update's grid has ceil(n / 64) rows of blocks
  if (d > (int64_t(1) << 20) || n > (int64_t(1) << 22)) return SKM_EINVAL;
  if (!valid_dtype(lut_dtype)) return SKM_EUNSUPPORTED;
  if (!W || !U || !lut || !idx_packed || !workspace) return SKM_EINVAL;
  if (!aligned16(W) || !aligned16(U) || !aligned16(lut) || !aligned16(idx_packed) || !aligned16(workspace))
    return SKM_EALIGN;
  if (workspace_bytes < skm::map_workspace_bytes(n)) return SKM_EWORKSPACE;
  const Range w[3] = {{W, n * d * 4}, {idx_packed, n * d * b / 8}, {workspace, (int64_t)skm::map_workspace_bytes(n)}};
  const Range r[2] = {{U, d * d * 4}, {lut, n * gpr * (int64_t(1) << b) * elem_bytes(lut_dtype)}};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 2; ++j)
      if (overlap(w[i], r[j])) return SKM_EALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(w[i], w[j])) return SKM_EALIAS;
  }
  const Problem p{0, n, d, b, gpr};
  return status_of(skm::launch_map(W, U, lut, lut_dtype, p, idx_packed, (float*)workspace, stream));
}

int sketch_lut_adam_step(float* master, void* lut, int lut_dtype, const float* grad, float* exp_avg,
                         float* exp_avg_sq, int64_t count, int64_t step, float lr, float beta1, float beta2,
                         float eps, float weight_decay, float grad_scale, hipStream_t stream) {
  if (count < 0 || step < 1) return SKM_EINVAL;
  if (!finite_in(lr, 0.f) || !finite_in(eps, 0.f) || !finite_in(weight_decay, 0.f) || !std::isfinite(grad_scale))
    return SKM_EINVAL;
  if (!(beta1 >= 0.f && beta1 < 1.f) || !(beta2 >= 0.f && beta2 < 1.f)) return SKM_EINVAL;
  if (lut && lut_dtype != SKM_F16 && lut_dtype != SKM_BF16) return SKM_EUNSUPPORTED;
  if (count == 0) return SKM_OK;
  if (!master || !grad || !exp_avg || !exp_avg_sq) return SKM_EINVAL;
  if (!aligned16(master) || !aligned16(grad) || !aligned16(exp_avg) || !aligned16(exp_avg_sq) ||
      (lut && !aligned16(lut)))
    return SKM_EALIGN;
  const Range w[4] = {{master, count * 4}, {exp_avg, count * 4}, {exp_avg_sq, count * 4}, {lut, count * 2}};
  for (int i = 0; i < 4; ++i) {
    if (overlap(w[i], {grad, count * 4})) return SKM_EALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(w[i], w[j])) return SKM_EALIAS;
  }
  // bias corrections in double on the host, handed to the kernel in fp32
  const double bc1 = 1.0 - std::pow((double)beta1, (double)step);
  const double bc2 = 1.0 - std::pow((double)beta2, (double)step);
  if (!(bc1 > 0.0) || !(bc2 > 0.0)) return SKM_EINVAL;
  skm::AdamArgs a;
  a.beta1 = beta1;
  a.beta2 = beta2;
  a.one_minus_beta1 = (float)(1.0 - (double)beta1);
  a.one_minus_beta2 = (float)(1.0 - (double)beta2);
  a.eps = eps;
  a.decay = (float)(1.0 - (double)lr * (double)weight_decay);
  a.step_size = (float)((double)lr / bc1);
  a.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(bc2));
  a.grad_scale = grad_scale;
  return status_of(skm::launch_lut_adam(master, lut, lut_dtype, grad, exp_avg, exp_avg_sq, count, a, stream));
}

int sketch_lut_sgd_step(float* master, void* lut, int lut_dtype, const float* grad, float* momentum_buf,
                        int64_t count, float lr, float momentum, float weight_decay, float grad_scale,
                        hipStream_t stream) {
  if (count < 0) return SKM_EINVAL;
  if (!finite_in(lr, 0.f) || !finite_in(momentum, 0.f) || !finite_in(weight_decay, 0.f) ||
      !std::isfinite(grad_scale))
    return SKM_EINVAL;
  if (lut && lut_dtype != SKM_F16 && lut_dtype != SKM_BF16) return SKM_EUNSUPPORTED;
  if (count == 0) return SKM_OK;
  if (!master || !grad || (momentum != 0.f && !momentum_buf)) return SKM_EINVAL;
  float* buf = momentum != 0.f ? momentum_buf : nullptr;
  if (!aligned16(master) || !aligned16(grad) || (buf && !aligned16(buf)) || (lut && !aligned16(lut)))
    return SKM_EALIGN;
  const Range w[3] = {{master, count * 4}, {buf, count * 4}, {lut, count * 2}};
  for (int i = 0; i < 3; ++i) {
    if (overlap(w[i], {grad, count * 4})) return SKM_EALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(w[i], w[j])) return SKM_EALIAS;
  }
  const skm::SgdArgs a{lr, momentum, weight_decay, grad_scale};
  return status_of(skm::launch_lut_sgd(master, lut, lut_dtype, grad, buf, count, a, stream));
}

}  // extern "C"
