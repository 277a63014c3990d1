// Host-side launchers of the sketched-matmul kernels. Internal to the library:
// the public surface is the C ABI in include/sketch_matmul.h. Every launcher
// assumes the arguments were validated by the ABI layer and only enqueues
// work on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace skm {

// The tiled kernels allocate only dynamic LDS and address it with absolute
// byte offsets, which holds only when the dynamic LDS starts at address 0,
// i.e. when the kernel has no static LDS. prepare_kernel checks that on the
// host (hipFuncGetAttributes) and raises the kernel's dynamic LDS limit when
// it needs more than 64 KB; callers run it once per kernel and return its
// error instead of launching.
inline hipError_t prepare_kernel(const void* kern, size_t dyn_lds) {
  hipFuncAttributes a;
  hipError_t e = hipFuncGetAttributes(&a, kern);
  if (e != hipSuccess) return e;
  if (a.sharedSizeBytes != 0) return hipErrorInvalidConfiguration;
  if (dyn_lds > 65536) e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn_lds);
  return e;
}

struct Problem {
  int64_t m, n, d;
  int b, gpr;
  int k() const { return 1 << b; }
  int64_t group_cols() const { return d / gpr; }
  int64_t units() const { return d / 32; }
  int64_t row_bytes() const { return d * b / 8; }
};

// checking aids
hipError_t launch_unpack(const uint8_t* idx_packed, const Problem& p, uint8_t* idx, hipStream_t s);
hipError_t launch_dequant(const uint8_t* idx_packed, const void* lut, int lut_dtype, const Problem& p, void* W,
                          hipStream_t s);

// fp32 path (fp32 activations and fp32 tables)
hipError_t launch_fwd_f32(const float* X, const uint8_t* idx, const float* lut, const Problem& p, float* Y,
                          hipStream_t s);
hipError_t launch_dx_f32(const float* dY, const uint8_t* idx, const float* lut, const Problem& p, float* dX,
                         hipStream_t s);
hipError_t launch_dlut_f32(const float* dY, const float* X, const uint8_t* idx, const Problem& p, float* dLUT,
                           int accumulate, hipStream_t s);

// fill `count` floats with zero (used instead of hipMemsetAsync so that a
// captured graph holds only kernel nodes)
hipError_t launch_zero_f32(float* dst, int64_t count, hipStream_t s);

// matrix-core paths (16-bit operands, fp32 accumulation)
// decode: m <= decode_max_m(), tables of one 16-row block must fit in LDS
int decode_max_m();
bool decode_supported(const Problem& p);
// whether the decode stages the activations in LDS (then, for bf16
// activations with f16 tables, it finds the row exponents itself; otherwise
// it reads them from rexp)
bool decode_stages_activations(const Problem& p, bool multi, int n_sets, bool scaled);
bool decode_multi_supported(const Problem& p, bool scaled);
hipError_t launch_decode(const void* X, int x_dtype, const uint8_t* idx, const void* lut, int lut_dtype,
                         const Problem& p, void* Y, const int32_t* rexp, hipStream_t s);
// decode with one table set per token: luts [n_sets][n][gpr][2^b], lut_set [m]
hipError_t launch_decode_multi(const void* X, int x_dtype, const uint8_t* idx, const void* luts, int lut_dtype,
                               const int32_t* lut_set, int n_sets, const Problem& p, void* Y, hipStream_t s);
// the same with set-interleaved tables (one LDS read looks up a weight for up
// to 8 sets; at most 16 sets in use); not for the prescaled (BF16, F16) pair
bool decode_sets_supported(const Problem& p, int n_sets, bool scaled);
hipError_t launch_decode_sets(const void* X, int x_dtype, const uint8_t* idx, const void* luts, int lut_dtype,
                              const int32_t* lut_set, int n_sets, const Problem& p, void* Y, hipStream_t s);

// per-row exponents of the bf16 -> f16 operand prescale (skm_common.h) of a
// bf16 matrix A [rows][cols] into e [rows]
hipError_t launch_row_exp(const void* A, int64_t rows, int64_t cols, int32_t* e, hipStream_t s);

// prefill / training forward: m > 16, tiled matrix-core GEMM. rexp: the row
// exponents of X (read only for bf16 activations with f16 tables)
bool gemm_fwd_supported(const Problem& p);
hipError_t launch_gemm_fwd(const void* X, int x_dtype, const uint8_t* idx, const void* lut, int lut_dtype,
                           const Problem& p, void* Y, const int32_t* rexp, hipStream_t s);

// backward on the matrix cores (16-bit operands, fp32 results)
bool gemm_bwd_supported(const Problem& p);
hipError_t launch_gemm_dx(const void* dY, int io_dtype, const uint8_t* idx, const void* lut, int lut_dtype,
                          const Problem& p, float* dX, const int32_t* rexp, hipStream_t s);
// dLUT; when the (128-row block, group) grid is small the tokens are split
// into ranges whose partial tables (dlut_partial_bytes(p) bytes, 0 when not
// split) go to `part` and are then added in range order
size_t dlut_partial_bytes(const Problem& p);
hipError_t launch_gemm_dlut(const void* dY, const void* X, int io_dtype, const uint8_t* idx, const Problem& p,
                            float* dLUT, int accumulate, float* part, hipStream_t s);

// sketch construction: column weights 1 / [H^-1]_jj from the factor U, the
// weighted Lloyd tables, and the error-compensated mapping (Wc is overwritten;
// E holds map_workspace_bytes(n))
hipError_t launch_col_weights(const float* U, int64_t d, float* h, hipStream_t s);
hipError_t launch_lloyd(const float* W, const float* h, const Problem& p, int iters, void* lut, int lut_dtype,
                        hipStream_t s);
size_t map_workspace_bytes(int64_t n);
// the factor U of the damped inverse Hessian (skm_factor.hip); the workspace
// holds hessian_factor_workspace_bytes(d)
size_t hessian_factor_workspace_bytes(int64_t d);
hipError_t launch_hessian_factor(const double* H, int64_t d, double damp, float* U, void* workspace, hipStream_t s);
hipError_t launch_map(float* Wc, const float* U, const void* lut, int lut_dtype, const Problem& p, uint8_t* idx,
                      float* E, hipStream_t s);

// fused table optimizer steps (fp32 master, optional 16-bit compute copy;
// lut == nullptr skips the copy)
struct AdamArgs {
  float beta1, beta2, one_minus_beta1, one_minus_beta2;
  float eps;
  float decay;         // 1 - lr * weight_decay (decoupled decay)
  float step_size;     // lr / (1 - beta1^step)
  float inv_sqrt_bc2;  // 1 / sqrt(1 - beta2^step)
  float grad_scale;
};
struct SgdArgs {
  float lr, momentum, weight_decay, grad_scale;
};
hipError_t launch_lut_adam(float* master, void* lut, int lut_dtype, const float* grad, float* exp_avg,
                           float* exp_avg_sq, int64_t count, const AdamArgs& a, hipStream_t s);
hipError_t launch_lut_sgd(float* master, void* lut, int lut_dtype, const float* grad, float* buf, int64_t count,
                          const SgdArgs& a, hipStream_t s);

}  // namespace skm
