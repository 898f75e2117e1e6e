// AdamW step on the LoRA adapters, and their optimizer state paged between
// HBM and pinned host memory (numbered list items (4) and (5) of "DL0087
// QLoRA: 4-bit Quantized LoRA": only the adapters train, and the optimizer
// states are paged to host RAM during transient memory spikes; "Memory
// Management Details" of "QLoRA: Quantized Low Rank Adaptation at Extreme
// Scale": paged optimizers offload their states to CPU memory when needed).
//
// The step streams bf16 parameters and gradients and fp32 moments m, v once
// (22 bytes per parameter) and is bound by the memory the moments live in:
// HBM when the state is resident, the host link when it is paged out, in
// which case the kernel reads and writes the pinned host copy directly.
// Paging is explicit (no demand paging without XNACK): page-out copies the
// moments to their pinned host home and frees the HBM copy, returning that
// memory for the spike; page-in copies them back.  Where the moments live
// never changes the arithmetic: results are bit-identical either way.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>

#include "device_common.hpp"
#include "kernels.hpp"
#include "qlora_nf4.h"

namespace qnf4 {

namespace {

constexpr int kAdamThreads = 256;

struct AdamArgs {
  float decay;      // 1 - lr wd
  float beta1, one_minus_beta1, beta2, one_minus_beta2;
  float step_size;  // lr / (1 - beta1^t)
  float inv_bc2;    // 1 / sqrt(1 - beta2^t)
  float eps;
};

__device__ __forceinline__ void adam_one(float& p, float g, float& m, float& v,
                                         const AdamArgs& a) {
  p *= a.decay;
  m = a.beta1 * m + a.one_minus_beta1 * g;
  v = a.beta2 * v + a.one_minus_beta2 * (g * g);
  const float denom = sqrtf(v) * a.inv_bc2 + a.eps;
  p -= a.step_size * (m / denom);
}

// Thread i of the grid-stride loop takes 8 consecutive parameters: 16 bytes
// of p and g, 32 of m and v.  The n % 8 tail is taken by the first threads.
__global__ __launch_bounds__(kAdamThreads) void k_adamw(uint16_t* __restrict__ p,
                                                        const uint16_t* __restrict__ g,
                                                        float* __restrict__ m,
                                                        float* __restrict__ v, int64_t n,
                                                        AdamArgs a) {
  const int64_t n8 = n / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n8; i += stride) {
    const u32x4 pw = *reinterpret_cast<const u32x4*>(p + 8 * i);
    const u32x4 gw = *reinterpret_cast<const u32x4*>(g + 8 * i);
    f32x4 m0 = *reinterpret_cast<const f32x4*>(m + 8 * i);
    f32x4 m1 = *reinterpret_cast<const f32x4*>(m + 8 * i + 4);
    f32x4 v0 = *reinterpret_cast<const f32x4*>(v + 8 * i);
    f32x4 v1 = *reinterpret_cast<const f32x4*>(v + 8 * i + 4);
    float pf[8], gf[8], mf[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w},
                        vf[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t pj = pw[j], gj = gw[j];
      pf[2 * j] = bf16_lo_to_f32(pj);
      pf[2 * j + 1] = bf16_hi_to_f32(pj);
      gf[2 * j] = bf16_lo_to_f32(gj);
      gf[2 * j + 1] = bf16_hi_to_f32(gj);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) adam_one(pf[j], gf[j], mf[j], vf[j], a);
    u32x4 po;
#pragma unroll
    for (int j = 0; j < 4; ++j) po[j] = pack_bf16x2(pf[2 * j], pf[2 * j + 1]);
    *reinterpret_cast<u32x4*>(p + 8 * i) = po;
    *reinterpret_cast<f32x4*>(m + 8 * i) = f32x4{mf[0], mf[1], mf[2], mf[3]};
    *reinterpret_cast<f32x4*>(m + 8 * i + 4) = f32x4{mf[4], mf[5], mf[6], mf[7]};
    *reinterpret_cast<f32x4*>(v + 8 * i) = f32x4{vf[0], vf[1], vf[2], vf[3]};
    *reinterpret_cast<f32x4*>(v + 8 * i + 4) = f32x4{vf[4], vf[5], vf[6], vf[7]};
  }
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (t < n - 8 * n8) {
    const int64_t k = 8 * n8 + t;
    float pf = bf16_lo_to_f32(p[k]), mf = m[k], vf = v[k];
    adam_one(pf, bf16_lo_to_f32(g[k]), mf, vf, a);
    p[k] = static_cast<uint16_t>(pack_bf16x2(pf, 0.f) & 0xFFFFu);
    m[k] = mf;
    v[k] = vf;
  }
}

}  // namespace

hipError_t launch_adamw(uint16_t* p, const uint16_t* g, float* m, float* v, int64_t n,
                        float lr, float beta1, float beta2, float eps, float weight_decay,
                        int64_t step, hipStream_t stream) {
  AdamArgs a;
  a.decay = static_cast<float>(1.0 - static_cast<double>(lr) * weight_decay);
  a.beta1 = beta1;
  a.one_minus_beta1 = static_cast<float>(1.0 - beta1);
  a.beta2 = beta2;
  a.one_minus_beta2 = static_cast<float>(1.0 - beta2);
  a.step_size = static_cast<float>(lr / (1.0 - std::pow(static_cast<double>(beta1), step)));
  a.inv_bc2 = static_cast<float>(1.0 / std::sqrt(1.0 - std::pow(static_cast<double>(beta2), step)));
  a.eps = eps;
  const int64_t n8 = n / 8;
  int64_t grid = (std::max<int64_t>(n8, 8) + kAdamThreads - 1) / kAdamThreads;
  if (grid > 4096) grid = 4096;
  prof_begin(5, stream);
  hipLaunchKernelGGL(k_adamw, dim3(static_cast<unsigned>(grid)), dim3(kAdamThreads), 0, stream,
                     p, g, m, v, n, a);
  prof_end(5, stream);
  return hipGetLastError();
}

}  // namespace qnf4

// ---------------------------------------------------------------------------
// Paged optimizer state: m and v ([n] fp32 each, v starting at a 256-byte
// boundary after m) in HBM while resident, with a pinned host home they are
// paged to.
// ---------------------------------------------------------------------------

struct qlora_paged_state {
  int64_t n = 0;
  int64_t ld = 0;           // v starts ld floats after m (n rounded up to 64: 256-byte aligned)
  int device = -1;          // the GPU whose HBM holds the resident copy
  float* dev = nullptr;     // [2 ld] in HBM, or null when paged out
  float* host = nullptr;    // [2 ld] pinned host home (allocated on first page-out)
  float* host_dev = nullptr;   // the device-visible address of `host`
};

namespace {

bool aligned16p(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_st(hipError_t e) { return e == hipSuccess ? QLORA_OK : QLORA_ERR_HIP; }

int ensure_host(qlora_paged_state* st) {
  if (st->host) return QLORA_OK;
  void* h = nullptr;
  if (hipHostMalloc(&h, static_cast<size_t>(st->ld) * 2 * sizeof(float), hipHostMallocDefault) !=
      hipSuccess)
    return QLORA_ERR_HIP;
  void* d = nullptr;
  if (hipHostGetDevicePointer(&d, h, 0) != hipSuccess) {
    (void)hipHostFree(h);
    return QLORA_ERR_HIP;
  }
  st->host = static_cast<float*>(h);
  st->host_dev = static_cast<float*>(d);
  return QLORA_OK;
}

}  // namespace

extern "C" {

int qlora_paged_state_create(int64_t n, int on_host, qlora_paged_state** out) {
  if (!out) return QLORA_ERR_NULL;
  *out = nullptr;
  if (n < 1 || n > (int64_t(1) << 40)) return QLORA_ERR_SHAPE;
  auto* st = new qlora_paged_state;
  st->n = n;
  st->ld = (n + 63) / 64 * 64;
  const size_t bytes = static_cast<size_t>(st->ld) * 2 * sizeof(float);
  int rc = QLORA_OK;
  if (hipGetDevice(&st->device) != hipSuccess) rc = QLORA_ERR_HIP;
  if (rc == QLORA_OK && on_host) {
    rc = ensure_host(st);
    if (rc == QLORA_OK) std::memset(st->host, 0, bytes);
  } else if (rc == QLORA_OK) {
    void* d = nullptr;
    rc = hip_st(hipMalloc(&d, bytes));
    if (rc == QLORA_OK) {
      st->dev = static_cast<float*>(d);
      rc = hip_st(hipMemset(st->dev, 0, bytes));
    }
  }
  if (rc != QLORA_OK) {
    qlora_paged_state_destroy(st);
    return rc;
  }
  *out = st;
  return QLORA_OK;
}

int qlora_paged_state_destroy(qlora_paged_state* st) {
  if (!st) return QLORA_OK;
  int rc = QLORA_OK;
  if (st->dev && hipFree(st->dev) != hipSuccess) rc = QLORA_ERR_HIP;
  if (st->host && hipHostFree(st->host) != hipSuccess) rc = QLORA_ERR_HIP;
  delete st;
  return rc;
}

int qlora_paged_state_resident(const qlora_paged_state* st) {
  return st && st->dev ? 1 : 0;
}

int qlora_paged_state_pointers(const qlora_paged_state* st, float** m, float** v) {
  if (!st || !m || !v) return QLORA_ERR_NULL;
  float* base = st->dev ? st->dev : st->host_dev;
  *m = base;
  *v = base + st->ld;
  return QLORA_OK;
}

// The page calls allocate and free on the state's own device.
static int on_state_device(const qlora_paged_state* st) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return QLORA_ERR_HIP;
  return cur == st->device ? QLORA_OK : QLORA_ERR_SHAPE;
}

int qlora_paged_state_page_out(qlora_paged_state* st, qlora_stream_t stream) {
  if (!st) return QLORA_ERR_NULL;
  if (!st->dev) return QLORA_OK;
  if (const int rc = on_state_device(st)) return rc;
  int rc = ensure_host(st);
  if (rc) return rc;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const size_t bytes = static_cast<size_t>(st->ld) * 2 * sizeof(float);
  if (hipMemcpyAsync(st->host, st->dev, bytes, hipMemcpyDeviceToHost, hs) != hipSuccess ||
      hipStreamSynchronize(hs) != hipSuccess)
    return QLORA_ERR_HIP;
  if (hipFree(st->dev) != hipSuccess) return QLORA_ERR_HIP;
  st->dev = nullptr;
  return QLORA_OK;
}

int qlora_paged_state_page_in(qlora_paged_state* st, qlora_stream_t stream) {
  if (!st) return QLORA_ERR_NULL;
  if (st->dev) return QLORA_OK;
  if (const int rc = on_state_device(st)) return rc;
  const size_t bytes = static_cast<size_t>(st->ld) * 2 * sizeof(float);
  void* d = nullptr;
  if (hipMalloc(&d, bytes) != hipSuccess) return QLORA_ERR_HIP;   // stays on the host
  if (hipMemcpyAsync(d, st->host, bytes, hipMemcpyHostToDevice,
                     static_cast<hipStream_t>(stream)) != hipSuccess) {
    (void)hipFree(d);
    return QLORA_ERR_HIP;
  }
  st->dev = static_cast<float*>(d);
  return QLORA_OK;
}

// m and v to or from caller memory laid out as [2][n]
int qlora_paged_state_read(const qlora_paged_state* st, float* dst, qlora_stream_t stream) {
  if (!st || !dst) return QLORA_ERR_NULL;
  const float* src = st->dev ? st->dev : st->host;
  const size_t bytes = static_cast<size_t>(st->n) * sizeof(float);
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(dst, src, bytes, hipMemcpyDefault, hs) != hipSuccess) return QLORA_ERR_HIP;
  return hip_st(hipMemcpyAsync(dst + st->n, src + st->ld, bytes, hipMemcpyDefault, hs));
}

int qlora_paged_state_write(qlora_paged_state* st, const float* src, qlora_stream_t stream) {
  if (!st || !src) return QLORA_ERR_NULL;
  float* dst = st->dev ? st->dev : st->host;
  const size_t bytes = static_cast<size_t>(st->n) * sizeof(float);
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(dst, src, bytes, hipMemcpyDefault, hs) != hipSuccess) return QLORA_ERR_HIP;
  return hip_st(hipMemcpyAsync(dst + st->ld, src + st->n, bytes, hipMemcpyDefault, hs));
}

int qlora_adamw_step(uint16_t* param, const uint16_t* grad, float* exp_avg, float* exp_avg_sq,
                     int64_t n, const qlora_adamw_config* cfg, int64_t step,
                     qlora_stream_t stream) {
  if (!param || !grad || !exp_avg || !exp_avg_sq || !cfg) return QLORA_ERR_NULL;
  if (n < 1 || step < 1) return QLORA_ERR_SHAPE;
  if (!(cfg->beta1 >= 0.f && cfg->beta1 < 1.f && cfg->beta2 >= 0.f && cfg->beta2 < 1.f &&
        cfg->eps > 0.f && cfg->lr >= 0.f && cfg->weight_decay >= 0.f))
    return QLORA_ERR_SHAPE;
  if (!aligned16p(param) || !aligned16p(grad) || !aligned16p(exp_avg) || !aligned16p(exp_avg_sq))
    return QLORA_ERR_ALIGN;
  return hip_st(qnf4::launch_adamw(param, grad, exp_avg, exp_avg_sq, n, cfg->lr, cfg->beta1,
                                   cfg->beta2, cfg->eps, cfg->weight_decay, step,
                                   static_cast<hipStream_t>(stream)));
}

}  // extern "C"
