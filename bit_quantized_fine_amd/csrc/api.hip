// C ABI of the QLoRA NF4 linear layer (declared in include/qlora_nf4.h):
// argument validation, the NF4 level and threshold tables, workspace
// carving, dispatch to the kernel launchers, and event-based kernel timing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "device_common.hpp"
#include "kernels.hpp"
#include "qlora_nf4.h"

namespace qnf4 {
namespace {

// ---------------------------------------------------------------------------
// NF4 level table ("4-bit NormalFloat" of "QLoRA: Finetuning 65B Models on a
// Single GPU"; Mathematical Formulation of "DL0087 QLoRA").  Levels sit at the
// normal quantiles of the probability centres of equal-mass bins: 8 bins of
// mass 1/16 above the median, 7 of mass 1/14 below it, plus an exact zero;
// each side divided by its extreme quantile.  The quantile is found by
// Newton's method on Phi(z) = erfc(-z/sqrt 2)/2 in long double.
// ---------------------------------------------------------------------------

long double normal_quantile(long double p) {
  const long double rt2 = sqrtl(2.0L);
  const long double inv_rt2pi = 1.0L / sqrtl(2.0L * 3.14159265358979323846264338327950288L);
  long double z = 1.6L * logl(p / (1.0L - p)) / 2.0L;  // logistic starting point
  for (int it = 0; it < 200; ++it) {
    const long double f = 0.5L * erfcl(-z / rt2) - p;
    const long double dens = inv_rt2pi * expl(-0.5L * z * z);
    const long double step = f / dens;
    z -= step;
    if (fabsl(step) <= 1e-18L * (1.0L + fabsl(z))) break;
  }
  return z;
}

struct Tables {
  Nf4Tables t;
  Tables() {
    long double pos[8], neg[7];
    for (int j = 1; j <= 8; ++j) pos[j - 1] = normal_quantile(0.5L + (j - 0.5L) / 16.0L);
    for (int j = 1; j <= 7; ++j) neg[j - 1] = normal_quantile(0.5L + (j - 0.5L) / 14.0L);
    // ascending: -neg[6]/neg[6] ... -neg[0]/neg[6], 0, pos[0]/pos[7] ... 1
    for (int i = 0; i < 7; ++i) t.q[i] = static_cast<float>(-neg[6 - i] / neg[6]);
    t.q[7] = 0.0f;
    for (int i = 0; i < 8; ++i) t.q[8 + i] = static_cast<float>(pos[i] / pos[7]);
    // thresholds: largest fp32 <= exact midpoint (the fp64 sum of two fp32 is exact)
    for (int j = 0; j < 15; ++j) {
      const double mid = (static_cast<double>(t.q[j]) + static_cast<double>(t.q[j + 1])) * 0.5;
      float th = static_cast<float>(mid);
      if (static_cast<double>(th) > mid) th = std::nextafter(th, -INFINITY);
      t.t[j] = th;
    }
  }
};

const Nf4Tables& tables() {
  static const Tables tb;
  return tb.t;
}

// ---------------------------------------------------------------------------
// Validation helpers
// ---------------------------------------------------------------------------

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// The GEMM kernels address a 256-token tile of X or dY, and the code
// stream, with 32-bit byte offsets.
constexpr int64_t kMaxK = int64_t(1) << 22;        // weight columns (in features)
constexpr int64_t kMaxN = int64_t(1) << 22;        // weight rows (out features)
constexpr int64_t kMaxElems = int64_t(1) << 32;    // N * K of one weight

int check_weight(const qlora_nf4_weight* w) {
  if (!w || !w->codes || !w->absmax_q || !w->absmax_scale) return QLORA_ERR_NULL;
  if (w->N < 1 || w->K < kBlock || w->K % kBlock != 0) return QLORA_ERR_SHAPE;
  // kernels address the code stream with 32-bit byte offsets
  if (w->K > kMaxK || w->N > kMaxN || w->N > kMaxElems / w->K) return QLORA_ERR_SHAPE;
  if (!aligned16(w->codes) || (reinterpret_cast<uintptr_t>(w->absmax_scale) & 3u))
    return QLORA_ERR_ALIGN;
  return QLORA_OK;
}

int check_rank(int r) {
  if (r < 0 || r > 256 || r % 8 != 0) return QLORA_ERR_RANK;
  return QLORA_OK;
}

Nf4View view(const qlora_nf4_weight* w) {
  return Nf4View{w->codes, w->absmax_q, w->absmax_scale, w->N, w->K};
}

int hip_status(hipError_t e) { return e == hipSuccess ? QLORA_OK : QLORA_ERR_HIP; }

// Forward workspace: the split-reduction partials of T, then (reusing the
// same bytes once T is final) those of the GEMM when it splits its reduction.
size_t fwd_ws_bytes(int64_t M, int64_t N, int64_t K, int r) {
  size_t f = r > 0 ? rank_ws_floats(M, N, K, r) : 0;
  if (!decode_fits(M, K)) {
    const GemmSplit sp = fwd_gemm_split(M, N, K);
    if (sp.splits > 1) f = std::max<size_t>(f, (size_t)sp.splits * M * N);
  }
  return round_up(f * sizeof(float), 256);
}

// Backward workspace: G [M][r] and the recomputed T [M][r] (r > 0), then the
// partials of the rank products, whose bytes the dX GEMM's partials reuse.
size_t bwd_ws_bytes(int64_t M, int64_t N, int64_t K, int r) {
  const size_t mr = r > 0 ? round_up((size_t)M * r * sizeof(float), 256) : 0;
  size_t f = r > 0 ? rank_ws_floats(M, N, K, r) : 0;
  const GemmSplit sp = dx_gemm_split(M, N, K);
  if (sp.splits > 1) f = std::max<size_t>(f, (size_t)sp.splits * M * K);
  return 2 * mr + round_up(f * sizeof(float), 256);
}

// ---------------------------------------------------------------------------
// Kernel timing: event pairs around launches, accumulated per family.
// ---------------------------------------------------------------------------

constexpr int kFamilies = 5;

struct Profiler {
  std::mutex mu;
  bool enabled = false;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  std::vector<std::pair<int, size_t>> pending;   // (family, index of start event)
  hipEvent_t open[kFamilies] = {};
  size_t open_idx[kFamilies] = {};
  double total_ms[kFamilies] = {};
  int64_t count[kFamilies] = {};

  hipEvent_t take(size_t& idx) {
    if (used == pool.size()) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      pool.push_back(e);
    }
    idx = used;
    return pool[used++];
  }
  void drain() {
    for (auto& pr : pending) {
      float ms = 0.f;
      if (hipEventSynchronize(pool[pr.second + 1]) == hipSuccess &&
          hipEventElapsedTime(&ms, pool[pr.second], pool[pr.second + 1]) == hipSuccess) {
        total_ms[pr.first] += ms;
        count[pr.first] += 1;
      }
    }
    pending.clear();
    used = 0;
  }
};

Profiler& profiler() {
  static Profiler p;
  return p;
}

}  // namespace

void prof_begin(int family, hipStream_t stream) {
  Profiler& p = profiler();
  if (!p.enabled) return;
  std::lock_guard<std::mutex> lk(p.mu);
  if (p.used + 2 > 8192) p.drain();
  size_t i0, i1;
  hipEvent_t a = p.take(i0);
  hipEvent_t b = p.take(i1);
  if (!a || !b || i1 != i0 + 1) return;
  p.open[family] = a;
  p.open_idx[family] = i0;
  hipEventRecord(a, stream);
}

void prof_end(int family, hipStream_t stream) {
  Profiler& p = profiler();
  if (!p.enabled) return;
  std::lock_guard<std::mutex> lk(p.mu);
  if (!p.open[family]) return;
  const size_t i0 = p.open_idx[family];
  hipEventRecord(p.pool[i0 + 1], stream);
  p.pending.emplace_back(family, i0);
  p.open[family] = nullptr;
}

}  // namespace qnf4

using namespace qnf4;

extern "C" {

const char* qlora_status_string(int status) {
  switch (status) {
    case QLORA_OK: return "ok";
    case QLORA_ERR_NULL: return "a required pointer is NULL";
    case QLORA_ERR_SHAPE: return "invalid shape (need M>=1, N>=1, N%8==0, K>=64, K%64==0)";
    case QLORA_ERR_RANK: return "invalid rank (need 0<=r<=256, r%8==0)";
    case QLORA_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case QLORA_ERR_HIP: return "HIP runtime error or kernel launch failure";
    case QLORA_ERR_WORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

const char* qlora_version(void) { return "1.0.0"; }

int qlora_nf4_levels(float* out16) {
  if (!out16) return QLORA_ERR_NULL;
  std::memcpy(out16, tables().q, sizeof(float) * 16);
  return QLORA_OK;
}

int qlora_nf4_thresholds(float* out15) {
  if (!out15) return QLORA_ERR_NULL;
  std::memcpy(out15, tables().t, sizeof(float) * 15);
  return QLORA_OK;
}

size_t qlora_nf4_codes_bytes(int64_t N, int64_t K) {
  if (N < 0 || K < 0 || K % kBlock) return 0;
  return static_cast<size_t>(N) * static_cast<size_t>(K) / 2;
}

size_t qlora_nf4_absmax_q_bytes(int64_t N, int64_t K) {
  if (N < 0 || K < 0 || K % kBlock) return 0;
  return static_cast<size_t>(N) * static_cast<size_t>(K) / kBlock;
}

size_t qlora_nf4_scale_count(int64_t N, int64_t K) {
  if (N < 0 || K < 0 || K % kBlock) return 0;
  const size_t nb = static_cast<size_t>(N) * static_cast<size_t>(K) / kBlock;
  return (nb + kGroup - 1) / kGroup;
}

int qlora_nf4_quantize(const float* W, int64_t N, int64_t K, uint8_t* codes,
                       uint8_t* absmax_q, float* absmax_scale, qlora_stream_t stream) {
  if (!W || !codes || !absmax_q || !absmax_scale) return QLORA_ERR_NULL;
  if (N < 1 || K < kBlock || K % kBlock != 0) return QLORA_ERR_SHAPE;
  if (K > kMaxK || N > kMaxN || N > kMaxElems / K) return QLORA_ERR_SHAPE;
  if (!aligned16(W) || !aligned16(codes) || (reinterpret_cast<uintptr_t>(absmax_scale) & 3u))
    return QLORA_ERR_ALIGN;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  prof_begin(3, st);
  const hipError_t e = launch_quantize(W, N, K, codes, absmax_q, absmax_scale, tables(), st);
  prof_end(3, st);
  return hip_status(e);
}

int qlora_nf4_dequantize(const qlora_nf4_weight* w, uint16_t* W_bf16, qlora_stream_t stream) {
  int st = check_weight(w);
  if (st) return st;
  if (!W_bf16) return QLORA_ERR_NULL;
  if (!aligned16(W_bf16)) return QLORA_ERR_ALIGN;
  return hip_status(launch_dequantize(w->codes, w->absmax_q, w->absmax_scale, w->N, w->K,
                                      W_bf16, tables(), static_cast<hipStream_t>(stream)));
}

size_t qlora_linear_fwd_workspace_bytes(int64_t M, int64_t N, int64_t K, int r) {
  if (M < 1 || N < 1 || K < 1) return 0;
  return fwd_ws_bytes(M, N, K, r);
}

size_t qlora_linear_bwd_workspace_bytes(int64_t M, int64_t N, int64_t K, int r) {
  if (M < 1 || N < 1 || K < 1) return 0;
  return bwd_ws_bytes(M, N, K, r);
}

int qlora_linear_fwd(const uint16_t* X, int64_t M, const qlora_nf4_weight* w,
                     const uint16_t* A, const uint16_t* B, int r, float s, uint16_t* Y,
                     float* T, void* workspace, size_t workspace_bytes,
                     qlora_stream_t stream) {
  int st = check_weight(w);
  if (st) return st;
  if ((st = check_rank(r))) return st;
  if (!X || !Y) return QLORA_ERR_NULL;
  if (r > 0 && (!A || !B || !T)) return QLORA_ERR_NULL;
  if (M < 1 || w->N % 8 != 0) return QLORA_ERR_SHAPE;
  if (!aligned16(X) || !aligned16(Y) || (r > 0 && (!aligned16(A) || !aligned16(B) || !aligned16(T))))
    return QLORA_ERR_ALIGN;
  const size_t need = fwd_ws_bytes(M, w->N, w->K, r);
  if (need > 0 && (!workspace || workspace_bytes < need)) return QLORA_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return QLORA_ERR_ALIGN;

  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const Nf4View v = view(w);
  hipError_t e = hipSuccess;
  float* ws = static_cast<float*>(workspace);
  const bool decode = decode_fits(M, w->K);
  if (decode && decode_folds_t(M, r)) {
    // T's partial sums are added up inside the decode kernel (no reduction
    // launch); its workgroup 0 writes T.
    int nz = 0;
    e = launch_lora_down_partials(X, M, w->K, A, r, decode_max_t_partials(M, w->K, r), ws, &nz,
                                  hs);
    if (e == hipSuccess) e = launch_fwd_decode(X, M, v, ws, nz, T, B, r, s, Y, tables(), hs);
    return hip_status(e);
  }
  if (r > 0) e = launch_lora_down(X, M, w->K, A, r, T, ws, hs);
  if (e != hipSuccess) return QLORA_ERR_HIP;
  if (decode)
    e = launch_fwd_decode(X, M, v, T, 0, nullptr, B, r, s, Y, tables(), hs);
  else
    e = launch_fwd_gemm(X, M, v, T, B, r, s, Y, ws, tables(), hs);
  return hip_status(e);
}

int qlora_linear_bwd(const uint16_t* dY, const uint16_t* X, int64_t M,
                     const qlora_nf4_weight* w, const uint16_t* A, const uint16_t* B, int r,
                     float s, const float* T_saved, uint16_t* dX, uint16_t* dA, uint16_t* dB,
                     void* workspace, size_t workspace_bytes, qlora_stream_t stream) {
  int st = check_weight(w);
  if (st) return st;
  if ((st = check_rank(r))) return st;
  if (!dY || !X) return QLORA_ERR_NULL;
  if (r > 0 && (!A || !B || !dA || !dB)) return QLORA_ERR_NULL;
  if (M < 1 || w->N % 8 != 0) return QLORA_ERR_SHAPE;
  if (!aligned16(dY) || !aligned16(X) || (dX && !aligned16(dX)) ||
      (r > 0 && (!aligned16(A) || !aligned16(B) || !aligned16(dA) || !aligned16(dB) ||
                 (T_saved && !aligned16(T_saved)))))
    return QLORA_ERR_ALIGN;
  const size_t need = bwd_ws_bytes(M, w->N, w->K, r);
  if (need > 0 && (!workspace || workspace_bytes < need)) return QLORA_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return QLORA_ERR_ALIGN;

  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const Nf4View v = view(w);
  hipError_t e = hipSuccess;
  float* G = nullptr;
  char* base = static_cast<char*>(workspace);
  const size_t mr = r > 0 ? round_up((size_t)M * r * sizeof(float), 256) : 0;
  float* part = base ? reinterpret_cast<float*>(base + 2 * mr) : nullptr;
  if (r > 0) {
    G = reinterpret_cast<float*>(base);
    float* Tr = reinterpret_cast<float*>(base + mr);
    const float* T = T_saved;
    if (!T) {
      e = launch_lora_down(X, M, w->K, A, r, Tr, part, hs);
      T = Tr;
    }
    if (e == hipSuccess) e = launch_grad_in_and_b(dY, M, w->N, B, T, r, s, G, dB, part, hs);
    if (e == hipSuccess) e = launch_grad_a(X, M, w->K, G, r, s, dA, part, hs);
    if (e != hipSuccess) return QLORA_ERR_HIP;
  }
  if (dX) e = launch_dx_gemm(dY, M, v, G, A, r, s, dX, part, tables(), hs);
  return hip_status(e);
}

int qlora_profile_enable(int enable) {
  Profiler& p = profiler();
  std::lock_guard<std::mutex> lk(p.mu);
  p.enabled = enable != 0;
  return QLORA_OK;
}

int qlora_profile_read(int family, double* total_ms, int64_t* launches) {
  if (family < 0 || family >= kFamilies) return QLORA_ERR_SHAPE;
  Profiler& p = profiler();
  std::lock_guard<std::mutex> lk(p.mu);
  p.drain();
  if (total_ms) *total_ms = p.total_ms[family];
  if (launches) *launches = p.count[family];
  return QLORA_OK;
}

int qlora_profile_reset(void) {
  Profiler& p = profiler();
  std::lock_guard<std::mutex> lk(p.mu);
  p.drain();
  for (int f = 0; f < kFamilies; ++f) {
    p.total_ms[f] = 0.0;
    p.count[f] = 0;
  }
  return QLORA_OK;
}

}  // extern "C"
