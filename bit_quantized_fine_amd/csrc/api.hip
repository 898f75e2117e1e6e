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

// Thresholds of a level table for the quantizer's rule code = #{j : x > t_j}:
// the code of x is the nearest level, ties to the lower index, so t_j is the
// largest fp32 not above the midpoint of level j and the next larger distinct
// level (a level equal to the one before it is never chosen: FP4's -0).  The
// fp64 sum of two fp32 levels is exact.
void fill_thresholds(Nf4Tables& t) {
  for (int j = 0; j < 15; ++j) {
    int n = j + 1;
    while (n < 15 && !(t.q[n] > t.q[j])) ++n;
    const double mid = (static_cast<double>(t.q[j]) + static_cast<double>(t.q[n])) * 0.5;
    float th = static_cast<float>(mid);
    if (static_cast<double>(th) > mid) th = std::nextafter(th, -INFINITY);
    t.t[j] = th;
  }
}

// The 4-bit types "4-bit NormalFloat" of "QLoRA: Finetuning 65B Models on a
// Single GPU" sets against each other: NF4 above; INT4 with sixteen levels
// spaced uniformly over [-1, 1], (2k - 15) / 15; FP4 as the sixteen E2M1
// values (sign, 2 exponent bits with bias 1, 1 mantissa bit) over their
// largest magnitude 6, ascending with +0 before -0.
struct Tables {
  Nf4Tables t[3];
  Tables() {
    long double pos[8], neg[7];
    for (int j = 1; j <= 8; ++j) pos[j - 1] = normal_quantile(0.5L + (j - 0.5L) / 16.0L);
    for (int j = 1; j <= 7; ++j) neg[j - 1] = normal_quantile(0.5L + (j - 0.5L) / 14.0L);
    // ascending: -neg[6]/neg[6] ... -neg[0]/neg[6], 0, pos[0]/pos[7] ... 1
    Nf4Tables& nf = t[QLORA_CODEBOOK_NF4];
    for (int i = 0; i < 7; ++i) nf.q[i] = static_cast<float>(-neg[6 - i] / neg[6]);
    nf.q[7] = 0.0f;
    for (int i = 0; i < 8; ++i) nf.q[8 + i] = static_cast<float>(pos[i] / pos[7]);

    Nf4Tables& in = t[QLORA_CODEBOOK_INT4];
    for (int k = 0; k < 16; ++k) in.q[k] = static_cast<float>((2.0 * k - 15.0) / 15.0);

    // E2M1 magnitudes of the bit patterns 0..7: 0, 0.5 (subnormal), then
    // 2^(e-1) (1 + m/2) for exponent fields e = 1..3
    double mag[8];
    for (int b = 0; b < 8; ++b) {
      const int e = b >> 1, m = b & 1;
      mag[b] = e == 0 ? 0.5 * m : std::ldexp(1.0 + 0.5 * m, e - 1);
    }
    Nf4Tables& fp = t[QLORA_CODEBOOK_FP4];
    for (int i = 0; i < 7; ++i) fp.q[i] = static_cast<float>(-mag[7 - i] / 6.0);
    fp.q[7] = 0.0f;
    fp.q[8] = -0.0f;
    for (int i = 1; i < 8; ++i) fp.q[8 + i] = static_cast<float>(mag[i] / 6.0);

    for (Nf4Tables& x : t) fill_thresholds(x);
  }
};

const Nf4Tables& tables(int codebook = QLORA_CODEBOOK_NF4) {
  static const Tables tb;
  return tb.t[codebook];
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
  size_t f = lora_down_ws_floats(M, K, r);
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

// Forward arguments other than the weight (N: the weight's rows).
int check_fwd_rest(const uint16_t* X, int64_t M, int64_t N, const uint16_t* A, const uint16_t* B,
                   int r, const uint16_t* Y, const float* T) {
  int st = check_rank(r);
  if (st) return st;
  if (!X || !Y) return QLORA_ERR_NULL;
  if (r > 0 && (!A || !B || !T)) return QLORA_ERR_NULL;
  if (M < 1 || N % 8 != 0) return QLORA_ERR_SHAPE;
  if (!aligned16(X) || !aligned16(Y) || (r > 0 && (!aligned16(A) || !aligned16(B) || !aligned16(T))))
    return QLORA_ERR_ALIGN;
  return QLORA_OK;
}

int check_fwd_args(const uint16_t* X, int64_t M, const qlora_nf4_weight* w, const uint16_t* A,
                   const uint16_t* B, int r, const uint16_t* Y, const float* T) {
  const int st = check_weight(w);
  return st ? st : check_fwd_rest(X, M, w->N, A, B, r, Y, T);
}

// A 4-bit weight of any codebook and constant format.
int check_q4_weight(const qlora_q4_weight* w) {
  if (!w) return QLORA_ERR_NULL;
  if (w->codebook < QLORA_CODEBOOK_NF4 || w->codebook > QLORA_CODEBOOK_FP4 ||
      (w->double_quant != 0 && w->double_quant != 1))
    return QLORA_ERR_FORMAT;
  if (!w->codes || !w->absmax_scale || (w->double_quant && !w->absmax_q)) return QLORA_ERR_NULL;
  if (w->N < 1 || w->K < kBlock || w->K % kBlock != 0) return QLORA_ERR_SHAPE;
  if (w->K > kMaxK || w->N > kMaxN || w->N > kMaxElems / w->K) return QLORA_ERR_SHAPE;
  // fp32 constants are read 16 bytes at a time by the streaming kernel
  if (!aligned16(w->codes) || (reinterpret_cast<uintptr_t>(w->absmax_scale) &
                               (w->double_quant ? 3u : 15u)))
    return QLORA_ERR_ALIGN;
  return QLORA_OK;
}

Nf4View q4_view(const qlora_q4_weight* w) {
  Nf4View v{w->codes, w->absmax_q, w->absmax_scale, w->N, w->K};
  v.dq = w->double_quant != 0;
  return v;
}

// ---------------------------------------------------------------------------
// Fixed scratch of the allocation-free forward.  A file-scope device array:
// each GPU the library runs on holds its own copy, at its own address, until
// the process ends.  Host code never passes the array's name to a kernel (on
// the host it is only a stand-in for the symbol); the device address is
// looked up once per device with hipGetSymbolAddress, with that device
// current, and kept.
// ---------------------------------------------------------------------------

constexpr size_t kScratchBytes = QLORA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_for_current_device(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QLORA_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QLORA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<float*>(g_scratch_ptr[dev]);
  return QLORA_OK;
}

// The forward once its arguments are checked; ws holds at least
// fwd_ws_bytes(M, N, K, r) bytes.
int fwd_impl(const uint16_t* X, int64_t M, const Nf4View& v, const Nf4Tables& tb,
             const uint16_t* A, const uint16_t* B, int r, float s, uint16_t* Y, float* T,
             float* ws, hipStream_t hs) {
  hipError_t e = hipSuccess;
  const bool decode = decode_fits(M, v.K);
  if (decode && decode_folds_t(M, r)) {
    // T's partial sums are added up inside the decode kernel (no reduction
    // launch); its workgroup 0 writes T.
    int nz = 0;
    e = launch_lora_down_partials(X, M, v.K, A, r, kMaxDownPartials, ws, &nz, hs);
    if (e == hipSuccess) e = launch_fwd_decode(X, M, v, ws, nz, T, B, r, s, Y, tb, hs);
    return hip_status(e);
  }
  if (r > 0) e = launch_lora_down(X, M, v.K, A, r, T, ws, hs);
  if (e != hipSuccess) return QLORA_ERR_HIP;
  if (decode)
    e = launch_fwd_decode(X, M, v, T, 0, nullptr, B, r, s, Y, tb, hs);
  else
    e = launch_fwd_gemm(X, M, v, T, B, r, s, Y, ws, tb, hs);
  return hip_status(e);
}

// The backward once the weight is checked (either form); ws as bwd_ws_bytes.
int bwd_impl(const uint16_t* dY, const uint16_t* X, int64_t M, const Nf4View& v,
             const Nf4Tables& tb, const uint16_t* A, const uint16_t* B, int r, float s, const float* T_saved,
             uint16_t* dX, uint16_t* dA, uint16_t* dB, void* workspace, size_t workspace_bytes,
             hipStream_t hs) {
  int st = check_rank(r);
  if (st) return st;
  if (!dY || !X) return QLORA_ERR_NULL;
  if (r > 0 && (!A || !B || !dA || !dB)) return QLORA_ERR_NULL;
  if (M < 1 || v.N % 8 != 0) return QLORA_ERR_SHAPE;
  if (!aligned16(dY) || !aligned16(X) || (dX && !aligned16(dX)) ||
      (r > 0 && (!aligned16(A) || !aligned16(B) || !aligned16(dA) || !aligned16(dB) ||
                 (T_saved && !aligned16(T_saved)))))
    return QLORA_ERR_ALIGN;
  const size_t need = bwd_ws_bytes(M, v.N, v.K, r);
  if (need > 0 && (!workspace || workspace_bytes < need)) return QLORA_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return QLORA_ERR_ALIGN;

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
      e = launch_lora_down(X, M, v.K, A, r, Tr, part, hs);
      T = Tr;
    }
    if (e == hipSuccess) e = launch_grad_in_and_b(dY, M, v.N, B, T, r, s, G, dB, part, hs);
    if (e == hipSuccess) e = launch_grad_a(X, M, v.K, G, r, s, dA, part, hs);
    if (e != hipSuccess) return QLORA_ERR_HIP;
  }
  if (dX) e = launch_dx_gemm(dY, M, v, G, A, r, s, dX, part, tb, hs);
  return hip_status(e);
}

// ---------------------------------------------------------------------------
// 16-bit LoRA: the same kernels over a bf16 weight [N, K] (no quantization),
// the baseline QLoRA's speed is set against.
// ---------------------------------------------------------------------------

// The kernels address the bf16 weight with 32-bit byte offsets below 2^31.
constexpr int64_t kMaxDenseElems = int64_t(1) << 30;

int check_dense(const uint16_t* W, int64_t N, int64_t K) {
  if (!W) return QLORA_ERR_NULL;
  if (N < 1 || N % 8 != 0 || K < kBlock || K % kBlock != 0) return QLORA_ERR_SHAPE;
  if (K > kMaxK || N > kMaxN || N > kMaxDenseElems / K) return QLORA_ERR_SHAPE;
  if (!aligned16(W)) return QLORA_ERR_ALIGN;
  return QLORA_OK;
}

Nf4View dense_view(const uint16_t* W, int64_t N, int64_t K) {
  Nf4View v{nullptr, nullptr, nullptr, N, K};
  v.dense = W;
  return v;
}

// The tiled GEMM at every M (no streaming path for the bf16 weight).
size_t dense_fwd_ws_bytes(int64_t M, int64_t N, int64_t K, int r) {
  size_t f = lora_down_ws_floats(M, K, r);
  const GemmSplit sp = fwd_gemm_split(M, N, K);
  if (sp.splits > 1) f = std::max<size_t>(f, (size_t)sp.splits * M * N);
  return round_up(f * sizeof(float), 256);
}

// ---------------------------------------------------------------------------
// Fused multi-projection block: S projections that share their input, stored
// as one NF4 weight of S * nseg rows with their adapters side by side.
// ---------------------------------------------------------------------------

// Limits of the block layout: segments aligned to the GEMM's 128-row tiles and
// to whole groups of 256 block constants (so a segment is a weight of its
// own), and a combined rank S r the rank products and the dX term take.
int check_block(const qlora_nf4_weight* w, int S, int r) {
  if (S < 1 || w->N % S != 0) return QLORA_ERR_SHAPE;
  const int64_t nseg = w->N / S;
  if (nseg % 128 != 0 || (nseg * w->K / kBlock) % kGroup != 0) return QLORA_ERR_SHAPE;
  if (r < 1 || int64_t(S) * r > 256) return QLORA_ERR_RANK;
  return QLORA_OK;
}

size_t block_fwd_ws_bytes(int64_t M, int S, int64_t nseg, int64_t K, int r) {
  size_t f = lora_down_ws_floats(M, K, S * r);
  if (!decode_fits(M, K)) {
    const GemmSplit sp = fwd_gemm_split(M, S * nseg, K);
    if (sp.splits > 1) f = std::max<size_t>(f, (size_t)sp.splits * M * S * nseg);
  }
  return round_up(f * sizeof(float), 256);
}

size_t block_bwd_ws_bytes(int64_t M, int S, int64_t nseg, int64_t K, int r) {
  const size_t mr = round_up((size_t)M * S * r * sizeof(float), 256);
  size_t f = std::max(rank_ws_floats(M, nseg, K, r), rank_ws_floats(M, S * nseg, K, S * r));
  const GemmSplit sp = dx_gemm_split(M, S * nseg, K);
  if (sp.splits > 1) f = std::max<size_t>(f, (size_t)sp.splits * M * K);
  return 2 * mr + round_up(f * sizeof(float), 256);
}

// ---------------------------------------------------------------------------
// Kernel timing: event pairs around launches, accumulated per family.
// ---------------------------------------------------------------------------

constexpr int kFamilies = 6;

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
    case QLORA_ERR_SHAPE:
      return "invalid shape (need M>=1, N>=1, N%8==0, K>=64, K%64==0, N<=2^22, K<=2^22, "
             "N*K<=2^32)";
    case QLORA_ERR_RANK: return "invalid rank (need 0<=r<=256, r%8==0)";
    case QLORA_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case QLORA_ERR_HIP: return "HIP runtime error or kernel launch failure";
    case QLORA_ERR_WORKSPACE: return "workspace too small";
    case QLORA_ERR_SCRATCH:
      return "the call needs more workspace than the fixed scratch of qlora_linear_fwd_noalloc "
             "(QLORA_NOALLOC_SCRATCH_BYTES)";
    case QLORA_ERR_FORMAT:
      return "unknown codebook or constant format (codebook 0..2, double_quant 0 or 1)";
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
  int st = check_fwd_args(X, M, w, A, B, r, Y, T);
  if (st) return st;
  const size_t need = fwd_ws_bytes(M, w->N, w->K, r);
  if (need > 0 && (!workspace || workspace_bytes < need)) return QLORA_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return QLORA_ERR_ALIGN;
  return fwd_impl(X, M, view(w), tables(), A, B, r, s, Y, T, static_cast<float*>(workspace),
                  static_cast<hipStream_t>(stream));
}

int qlora_linear_fwd_noalloc(const uint16_t* X, int64_t M, const qlora_nf4_weight* w,
                             const uint16_t* A, const uint16_t* B, int r, float s, uint16_t* Y,
                             float* T, qlora_stream_t stream) {
  int st = check_fwd_args(X, M, w, A, B, r, Y, T);
  if (st) return st;
  if (fwd_ws_bytes(M, w->N, w->K, r) > kScratchBytes) return QLORA_ERR_SCRATCH;
  float* ws = nullptr;
  if ((st = scratch_for_current_device(&ws))) return st;
  return fwd_impl(X, M, view(w), tables(), A, B, r, s, Y, T, ws,
                  static_cast<hipStream_t>(stream));
}

int qlora_linear_bwd(const uint16_t* dY, const uint16_t* X, int64_t M,
                     const qlora_nf4_weight* w, const uint16_t* A, const uint16_t* B, int r,
                     float s, const float* T_saved, uint16_t* dX, uint16_t* dA, uint16_t* dB,
                     void* workspace, size_t workspace_bytes, qlora_stream_t stream) {
  const int st = check_weight(w);
  if (st) return st;
  return bwd_impl(dY, X, M, view(w), tables(), A, B, r, s, T_saved, dX, dA, dB, workspace,
                  workspace_bytes, static_cast<hipStream_t>(stream));
}

size_t qlora_lora16_fwd_workspace_bytes(int64_t M, int64_t N, int64_t K, int r) {
  if (M < 1 || N < 1 || K < 1 || r < 0) return 0;
  return dense_fwd_ws_bytes(M, N, K, r);
}

size_t qlora_lora16_bwd_workspace_bytes(int64_t M, int64_t N, int64_t K, int r) {
  if (M < 1 || N < 1 || K < 1 || r < 0) return 0;
  return bwd_ws_bytes(M, N, K, r);
}

int qlora_lora16_fwd(const uint16_t* X, int64_t M, const uint16_t* W, int64_t N, int64_t K,
                     const uint16_t* A, const uint16_t* B, int r, float s, uint16_t* Y,
                     float* T, void* workspace, size_t workspace_bytes,
                     qlora_stream_t stream) {
  int st = check_dense(W, N, K);
  if (st) return st;
  if ((st = check_rank(r))) return st;
  if (!X || !Y) return QLORA_ERR_NULL;
  if (r > 0 && (!A || !B || !T)) return QLORA_ERR_NULL;
  if (M < 1) return QLORA_ERR_SHAPE;
  if (!aligned16(X) || !aligned16(Y) || (r > 0 && (!aligned16(A) || !aligned16(B) || !aligned16(T))))
    return QLORA_ERR_ALIGN;
  const size_t need = dense_fwd_ws_bytes(M, N, K, r);
  if (need > 0 && (!workspace || workspace_bytes < need)) return QLORA_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return QLORA_ERR_ALIGN;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  float* ws = static_cast<float*>(workspace);
  hipError_t e = hipSuccess;
  if (r > 0) e = launch_lora_down(X, M, K, A, r, T, ws, hs);
  if (e == hipSuccess) e = launch_fwd_gemm(X, M, dense_view(W, N, K), T, B, r, s, Y, ws, tables(), hs);
  return hip_status(e);
}

int qlora_lora16_bwd(const uint16_t* dY, const uint16_t* X, int64_t M, const uint16_t* W,
                     int64_t N, int64_t K, const uint16_t* A, const uint16_t* B, int r, float s,
                     const float* T_saved, uint16_t* dX, uint16_t* dA, uint16_t* dB,
                     void* workspace, size_t workspace_bytes, qlora_stream_t stream) {
  const int st = check_dense(W, N, K);
  if (st) return st;
  return bwd_impl(dY, X, M, dense_view(W, N, K), tables(), A, B, r, s, T_saved, dX, dA, dB,
                  workspace,
                  workspace_bytes, static_cast<hipStream_t>(stream));
}

int qlora_q4_levels(int codebook, float* out16) {
  if (!out16) return QLORA_ERR_NULL;
  if (codebook < QLORA_CODEBOOK_NF4 || codebook > QLORA_CODEBOOK_FP4) return QLORA_ERR_FORMAT;
  std::memcpy(out16, tables(codebook).q, sizeof(float) * 16);
  return QLORA_OK;
}

int qlora_q4_thresholds(int codebook, float* out15) {
  if (!out15) return QLORA_ERR_NULL;
  if (codebook < QLORA_CODEBOOK_NF4 || codebook > QLORA_CODEBOOK_FP4) return QLORA_ERR_FORMAT;
  std::memcpy(out15, tables(codebook).t, sizeof(float) * 15);
  return QLORA_OK;
}

size_t qlora_q4_scale_count(int64_t N, int64_t K, int double_quant) {
  if (N < 0 || K < 0 || K % kBlock) return 0;
  const size_t nb = static_cast<size_t>(N) * static_cast<size_t>(K) / kBlock;
  return double_quant ? (nb + kGroup - 1) / kGroup : nb;
}

int qlora_q4_quantize(const float* W, int64_t N, int64_t K, int codebook, int double_quant,
                      uint8_t* codes, uint8_t* absmax_q, float* absmax_scale,
                      qlora_stream_t stream) {
  if (codebook < QLORA_CODEBOOK_NF4 || codebook > QLORA_CODEBOOK_FP4 ||
      (double_quant != 0 && double_quant != 1))
    return QLORA_ERR_FORMAT;
  if (!W || !codes || !absmax_scale || (double_quant && !absmax_q)) return QLORA_ERR_NULL;
  if (N < 1 || K < kBlock || K % kBlock != 0) return QLORA_ERR_SHAPE;
  if (K > kMaxK || N > kMaxN || N > kMaxElems / K) return QLORA_ERR_SHAPE;
  if (!aligned16(W) || !aligned16(codes) ||
      (reinterpret_cast<uintptr_t>(absmax_scale) & (double_quant ? 3u : 15u)))
    return QLORA_ERR_ALIGN;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  prof_begin(3, st);
  const hipError_t e = launch_quantize(W, N, K, codes, absmax_q, absmax_scale, tables(codebook),
                                       st, double_quant != 0);
  prof_end(3, st);
  return hip_status(e);
}

int qlora_q4_dequantize(const qlora_q4_weight* w, uint16_t* W_bf16, qlora_stream_t stream) {
  const int st = check_q4_weight(w);
  if (st) return st;
  if (!W_bf16) return QLORA_ERR_NULL;
  if (!aligned16(W_bf16)) return QLORA_ERR_ALIGN;
  return hip_status(launch_dequantize(w->codes, w->absmax_q, w->absmax_scale, w->N, w->K,
                                      W_bf16, tables(w->codebook),
                                      static_cast<hipStream_t>(stream), w->double_quant != 0));
}

int qlora_q4_linear_fwd(const uint16_t* X, int64_t M, const qlora_q4_weight* w,
                        const uint16_t* A, const uint16_t* B, int r, float s, uint16_t* Y,
                        float* T, void* workspace, size_t workspace_bytes,
                        qlora_stream_t stream) {
  int st = check_q4_weight(w);
  if (st) return st;
  if ((st = check_fwd_rest(X, M, w->N, A, B, r, Y, T))) return st;
  const size_t need = fwd_ws_bytes(M, w->N, w->K, r);
  if (need > 0 && (!workspace || workspace_bytes < need)) return QLORA_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return QLORA_ERR_ALIGN;
  return fwd_impl(X, M, q4_view(w), tables(w->codebook), A, B, r, s, Y, T,
                  static_cast<float*>(workspace), static_cast<hipStream_t>(stream));
}

int qlora_q4_linear_bwd(const uint16_t* dY, const uint16_t* X, int64_t M,
                        const qlora_q4_weight* w, const uint16_t* A, const uint16_t* B, int r,
                        float s, const float* T_saved, uint16_t* dX, uint16_t* dA, uint16_t* dB,
                        void* workspace, size_t workspace_bytes, qlora_stream_t stream) {
  const int st = check_q4_weight(w);
  if (st) return st;
  return bwd_impl(dY, X, M, q4_view(w), tables(w->codebook), A, B, r, s, T_saved, dX, dA, dB,
                  workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

size_t qlora_block_fwd_workspace_bytes(int64_t M, int S, int64_t nseg, int64_t K, int r) {
  if (M < 1 || S < 1 || nseg < 1 || K < 1 || r < 1) return 0;
  return block_fwd_ws_bytes(M, S, nseg, K, r);
}

size_t qlora_block_bwd_workspace_bytes(int64_t M, int S, int64_t nseg, int64_t K, int r) {
  if (M < 1 || S < 1 || nseg < 1 || K < 1 || r < 1) return 0;
  return block_bwd_ws_bytes(M, S, nseg, K, r);
}

int qlora_block_fwd(const uint16_t* X, int64_t M, const qlora_nf4_weight* w, int S,
                    const uint16_t* A, const uint16_t* B, int r, float s, uint16_t* Y, float* T,
                    void* workspace, size_t workspace_bytes, qlora_stream_t stream) {
  int st = check_fwd_args(X, M, w, A, B, r, Y, T);
  if (st) return st;
  if (r == 0) return QLORA_ERR_RANK;
  if ((st = check_block(w, S, r))) return st;
  const int64_t nseg = w->N / S;
  const int rt = S * r;
  const size_t need = block_fwd_ws_bytes(M, S, nseg, w->K, r);
  if (!workspace || workspace_bytes < need) return QLORA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return QLORA_ERR_ALIGN;

  const hipStream_t hs = static_cast<hipStream_t>(stream);
  float* ws = static_cast<float*>(workspace);
  // T = X . [A_0 .. A_{S-1}] for all projections in one product
  hipError_t e = launch_lora_down(X, M, w->K, A, rt, T, ws, hs);
  if (e != hipSuccess) return QLORA_ERR_HIP;
  if (!decode_fits(M, w->K)) {
    // one GEMM over all S nseg rows; each row tile adds its own adapter
    e = launch_fwd_gemm(X, M, view(w), T, B, r, s, Y, ws, tables(), hs, rt, nseg);
    return hip_status(e);
  }
  // few tokens: the streaming kernel per projection (a segment is a whole
  // weight: its codes, constants and group scales start at group boundaries)
  const int64_t seg_codes = nseg * w->K / 2, seg_blocks = nseg * w->K / kBlock;
  for (int j = 0; j < S && e == hipSuccess; ++j) {
    const Nf4View v{w->codes + j * seg_codes, w->absmax_q + j * seg_blocks,
                    w->absmax_scale + j * seg_blocks / kGroup, nseg, w->K};
    // (each projection writes its own columns of Y, row stride S nseg)
    e = launch_fwd_decode(X, M, v, T + j * r, 0, nullptr, B + j * nseg, r, s, Y + j * nseg,
                          tables(), hs, rt, w->N, w->N);
  }
  return hip_status(e);
}

int qlora_block_bwd(const uint16_t* dY, const uint16_t* X, int64_t M, const qlora_nf4_weight* w,
                    int S, const uint16_t* A, const uint16_t* B, int r, float s,
                    const float* T_saved, uint16_t* dX, uint16_t* dA, uint16_t* dB,
                    void* workspace, size_t workspace_bytes, qlora_stream_t stream) {
  int st = check_weight(w);
  if (st) return st;
  if ((st = check_rank(r))) return st;
  if (r == 0) return QLORA_ERR_RANK;
  if ((st = check_block(w, S, r))) return st;
  if (!dY || !X || !A || !B || !dA || !dB) return QLORA_ERR_NULL;
  if (M < 1) return QLORA_ERR_SHAPE;
  if (!aligned16(dY) || !aligned16(X) || (dX && !aligned16(dX)) || !aligned16(A) ||
      !aligned16(B) || !aligned16(dA) || !aligned16(dB) || (T_saved && !aligned16(T_saved)))
    return QLORA_ERR_ALIGN;
  const int64_t nseg = w->N / S;
  const int rt = S * r;
  const size_t need = block_bwd_ws_bytes(M, S, nseg, w->K, r);
  if (!workspace || workspace_bytes < need) return QLORA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return QLORA_ERR_ALIGN;

  const hipStream_t hs = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(workspace);
  const size_t mr = round_up((size_t)M * rt * sizeof(float), 256);
  float* G = reinterpret_cast<float*>(base);            // [M][S r]
  float* Tr = reinterpret_cast<float*>(base + mr);      // [M][S r]
  float* part = reinterpret_cast<float*>(base + 2 * mr);
  hipError_t e = hipSuccess;
  const float* T = T_saved;
  if (!T) {
    e = launch_lora_down(X, M, w->K, A, rt, Tr, part, hs);
    T = Tr;
  }
  // per projection: G_j = dY_j . B_j^T and dB_j = s . T_j^T . dY_j, on the
  // segments' columns of dY, B, dB and the segments' ranks of T and G
  for (int j = 0; j < S && e == hipSuccess; ++j)
    e = launch_grad_in_and_b(dY + j * nseg, M, nseg, B + j * nseg, T + j * r, r, s, G + j * r,
                             dB + j * nseg, part, hs, w->N, w->N, rt);
  // dA = s . X^T . G for all projections in one product
  if (e == hipSuccess) e = launch_grad_a(X, M, w->K, G, rt, s, dA, part, hs);
  // dX = sum_j dY_j . deq(W_j) + s . G_j . A_j^T: one GEMM over all S nseg rows
  if (e == hipSuccess && dX)
    e = launch_dx_gemm(dY, M, view(w), G, A, rt, s, dX, part, tables(), hs);
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
