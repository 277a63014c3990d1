// Fused optimizer steps for the trainable tables.
//
// Fine-tuning updates only the table values; the mapping stays frozen (SpaLLM
// section 2.3). The tables are kept as an fp32 master copy, and the matmul
// kernels read a 16-bit compute copy. One pass over the entries reads the
// master, the gradient and the optimizer state, writes the new master and
// state, and writes the rounded 16-bit copy, so no separate conversion pass is
// needed. The pages do not name an optimizer; these are Adam with decoupled
// weight decay (Kingma & Ba, Adam, Algorithm 1; Loshchilov & Hutter, AdamW)
// and plain SGD with heavy-ball momentum, in the forms torch.optim uses.
//
// The pass is bound by HBM bandwidth: Adam moves 30 bytes per entry (reads
// master, gradient and both moments, writes master, both moments and the copy).
// Each thread takes eight consecutive entries with 16-byte loads and stores.
#include "skm_common.h"
#include "skm_launch.h"

namespace skm {

namespace {

constexpr int OPT_PER_THREAD = 8;
constexpr int OPT_THREADS = 256;

__device__ __forceinline__ void adam_one(const AdamArgs& a, float& p, float g, float& m1, float& m2) {
  g *= a.grad_scale;
  p *= a.decay;
  m1 = a.beta1 * m1 + a.one_minus_beta1 * g;
  m2 = a.beta2 * m2 + a.one_minus_beta2 * (g * g);
  const float den = sqrtf(m2) * a.inv_sqrt_bc2 + a.eps;
  p -= a.step_size * (m1 / den);
}

template <bool MOM>
__device__ __forceinline__ void sgd_one(const SgdArgs& a, float& p, float g, float& buf) {
  g = g * a.grad_scale + a.weight_decay * p;
  if (MOM) {
    buf = a.momentum * buf + g;
    g = buf;
  }
  p -= a.lr * g;
}

// The copy is the stored fp32 master rounded to 16 bits. Without the empty asm
// the compiler fuses the update's last fma with the f16 conversion
// (v_fma_mixlo_f16), which rounds the exact result once: at fp32 values that
// are ties in f16 that picks a different neighbour than rounding the master.
template <typename TL>
__device__ __forceinline__ TL round_master(float p) {
  asm volatile("" : "+v"(p));
  return from_f32<TL>(p);
}

template <typename TL>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return (uint32_t)bits16(round_master<TL>(lo)) | ((uint32_t)bits16(round_master<TL>(hi)) << 16);
}

template <typename TL>
__device__ __forceinline__ void store_copy8(TL* lut, int64_t e0, const f32x4& p0, const f32x4& p1) {
  const u32x4 v = {pack2<TL>(p0[0], p0[1]), pack2<TL>(p0[2], p0[3]), pack2<TL>(p1[0], p1[1]),
                   pack2<TL>(p1[2], p1[3])};
  *reinterpret_cast<u32x4*>(lut + e0) = v;
}

template <typename TL>
__device__ __forceinline__ void store_copy1(TL* lut, int64_t e, float p) {
  lut[e] = round_master<TL>(p);
}

// TL: dtype of the compute copy (ignored when COPY is false)
template <typename TL, bool COPY>
__global__ void __launch_bounds__(OPT_THREADS)
    k_lut_adam(float* __restrict__ master, TL* __restrict__ lut, const float* __restrict__ grad,
               float* __restrict__ exp_avg, float* __restrict__ exp_avg_sq, int64_t count, AdamArgs a) {
  const int64_t e0 = ((int64_t)blockIdx.x * OPT_THREADS + threadIdx.x) * OPT_PER_THREAD;
  if (e0 >= count) return;
  if (e0 + OPT_PER_THREAD <= count) {
    const f32x4* pp = reinterpret_cast<const f32x4*>(master + e0);
    const f32x4* gp = reinterpret_cast<const f32x4*>(grad + e0);
    const f32x4* mp = reinterpret_cast<const f32x4*>(exp_avg + e0);
    const f32x4* vp = reinterpret_cast<const f32x4*>(exp_avg_sq + e0);
    f32x4 p[2] = {pp[0], pp[1]}, g[2] = {gp[0], gp[1]}, m1[2] = {mp[0], mp[1]}, m2[2] = {vp[0], vp[1]};
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float pr = p[h][r], mr = m1[h][r], vr = m2[h][r];
        adam_one(a, pr, g[h][r], mr, vr);
        p[h][r] = pr;
        m1[h][r] = mr;
        m2[h][r] = vr;
      }
    f32x4* po = reinterpret_cast<f32x4*>(master + e0);
    f32x4* mo = reinterpret_cast<f32x4*>(exp_avg + e0);
    f32x4* vo = reinterpret_cast<f32x4*>(exp_avg_sq + e0);
    po[0] = p[0];
    po[1] = p[1];
    mo[0] = m1[0];
    mo[1] = m1[1];
    vo[0] = m2[0];
    vo[1] = m2[1];
    if (COPY) store_copy8<TL>(lut, e0, p[0], p[1]);
  } else {
    // ragged tail: fewer than eight entries left
    for (int64_t e = e0; e < count; ++e) {
      float p = master[e], mr = exp_avg[e], vr = exp_avg_sq[e];
      adam_one(a, p, grad[e], mr, vr);
      master[e] = p;
      exp_avg[e] = mr;
      exp_avg_sq[e] = vr;
      if (COPY) store_copy1<TL>(lut, e, p);
    }
  }
}

template <typename TL, bool COPY, bool MOM>
__global__ void __launch_bounds__(OPT_THREADS)
    k_lut_sgd(float* __restrict__ master, TL* __restrict__ lut, const float* __restrict__ grad,
              float* __restrict__ buf, int64_t count, SgdArgs a) {
  const int64_t e0 = ((int64_t)blockIdx.x * OPT_THREADS + threadIdx.x) * OPT_PER_THREAD;
  if (e0 >= count) return;
  if (e0 + OPT_PER_THREAD <= count) {
    const f32x4* pp = reinterpret_cast<const f32x4*>(master + e0);
    const f32x4* gp = reinterpret_cast<const f32x4*>(grad + e0);
    f32x4 p[2] = {pp[0], pp[1]}, g[2] = {gp[0], gp[1]}, bb[2] = {};
    if (MOM) {
      const f32x4* bp = reinterpret_cast<const f32x4*>(buf + e0);
      bb[0] = bp[0];
      bb[1] = bp[1];
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float pr = p[h][r], br = bb[h][r];
        sgd_one<MOM>(a, pr, g[h][r], br);
        p[h][r] = pr;
        bb[h][r] = br;
      }
    f32x4* po = reinterpret_cast<f32x4*>(master + e0);
    po[0] = p[0];
    po[1] = p[1];
    if (MOM) {
      f32x4* bo = reinterpret_cast<f32x4*>(buf + e0);
      bo[0] = bb[0];
      bo[1] = bb[1];
    }
    if (COPY) store_copy8<TL>(lut, e0, p[0], p[1]);
  } else {
    for (int64_t e = e0; e < count; ++e) {
      float p = master[e], br = MOM ? buf[e] : 0.f;
      sgd_one<MOM>(a, p, grad[e], br);
      master[e] = p;
      if (MOM) buf[e] = br;
      if (COPY) store_copy1<TL>(lut, e, p);
    }
  }
}

dim3 opt_grid(int64_t count) {
  const int64_t threads = (count + OPT_PER_THREAD - 1) / OPT_PER_THREAD;
  return dim3((unsigned)((threads + OPT_THREADS - 1) / OPT_THREADS));
}

}  // namespace

hipError_t launch_lut_adam(float* master, void* lut, int lut_dtype, const float* grad, float* exp_avg,
                           float* exp_avg_sq, int64_t count, const AdamArgs& a, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  const dim3 grid = opt_grid(count), block(OPT_THREADS);
  if (!lut)
    hipLaunchKernelGGL((k_lut_adam<half_t, false>), grid, block, 0, s, master, nullptr, grad, exp_avg, exp_avg_sq,
                       count, a);
  else if (lut_dtype == DT_F16)
    hipLaunchKernelGGL((k_lut_adam<half_t, true>), grid, block, 0, s, master, (half_t*)lut, grad, exp_avg,
                       exp_avg_sq, count, a);
  else
    hipLaunchKernelGGL((k_lut_adam<bf16_t, true>), grid, block, 0, s, master, (bf16_t*)lut, grad, exp_avg,
                       exp_avg_sq, count, a);
  return hipGetLastError();
}

hipError_t launch_lut_sgd(float* master, void* lut, int lut_dtype, const float* grad, float* buf, int64_t count,
                          const SgdArgs& a, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  const dim3 grid = opt_grid(count), block(OPT_THREADS);
  const bool mom = a.momentum != 0.f;
#define SKM_SGD(TL, COPY, MOM) \
  hipLaunchKernelGGL((k_lut_sgd<TL, COPY, MOM>), grid, block, 0, s, master, (TL*)lut, grad, buf, count, a)
  if (!lut) {
    if (mom) SKM_SGD(half_t, false, true);
    else SKM_SGD(half_t, false, false);
  } else if (lut_dtype == DT_F16) {
    if (mom) SKM_SGD(half_t, true, true);
    else SKM_SGD(half_t, true, false);
  } else {
    if (mom) SKM_SGD(bf16_t, true, true);
    else SKM_SGD(bf16_t, true, false);
  }
#undef SKM_SGD
  return hipGetLastError();
}

}  // namespace skm
