// Host-callable launchers of the gfx950 kernels.  Every launcher enqueues on
// `stream`, allocates nothing and returns hipGetLastError() of its launches.
// Shapes are validated by the caller (the C ABI layer).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qnf4 {

struct Nf4Tables;

// dq: double-quantized constants (absmax_q [nb] bytes, absmax_scale one fp32
// per 256 blocks), else absmax_scale holds each block's fp32 absmax.
hipError_t launch_quantize(const float* W, int64_t N, int64_t K, uint8_t* codes,
                           uint8_t* absmax_q, float* absmax_scale,
                           const Nf4Tables& tb, hipStream_t stream, bool dq = true);

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* absmax_q,
                             const float* absmax_scale, int64_t N, int64_t K,
                             uint16_t* out, const Nf4Tables& tb, hipStream_t stream,
                             bool dq = true);

struct Nf4View {
  const uint8_t* codes;
  const uint8_t* absmax_q;
  const float* absmax_scale;
  int64_t N, K;
  // When set, the GEMM launchers read this bf16 weight [N, K] instead of the
  // NF4 fields (the 16-bit LoRA baseline); N K 2 must stay below 2^31 bytes.
  const uint16_t* dense = nullptr;
  // false: fp32 block constants in absmax_scale [N K / 64], absmax_q unused.
  bool dq = true;
};

// Profiling hook: the launchers call these around the launches of one
// kernel family (no-ops unless profiling is enabled).
void prof_begin(int family, hipStream_t stream);
void prof_end(int family, hipStream_t stream);

// Split reduction of a dequantizing GEMM whose tiles would leave most of
// the CUs idle: `splits` workgroups per tile, each over `cps` consecutive
// chunks of the reduction, write fp32 partials that a second kernel adds up
// in split order (deterministic) and rounds to bf16.
struct GemmSplit {
  int splits, cps;
};
GemmSplit gemm_split(int64_t tiles, int64_t nchunks);
hipError_t launch_split_reduce_bf16(const float* part, int splits, int64_t count, uint16_t* out,
                                    hipStream_t stream);

// Y[M,N] = bf16( X . deq(W)^T + s . T . B ), large-M MFMA path with the
// dequantized weight tiles staged in LDS.  T [M, r] fp32 (may be null when
// r == 0).  part: fwd_gemm_split(M, N, K).splits * M * N floats when that is
// above 1 (else unused).  Segments (seg_rows > 0, a multiple of 128): rows
// [j seg_rows, (j + 1) seg_rows) of W carry adapter j, whose T is columns
// [j r, (j + 1) r) of T (row stride ldt) and whose B is columns of the same
// rows of B [r, N]; by default one segment, ldt = r.
GemmSplit fwd_gemm_split(int64_t M, int64_t N, int64_t K);
hipError_t launch_fwd_gemm(const uint16_t* X, int64_t M, const Nf4View& w,
                           const float* T, const uint16_t* B, int r, float s,
                           uint16_t* Y, float* part, const Nf4Tables& tb, hipStream_t stream,
                           int ldt = 0, int64_t seg_rows = 0);

// Same result, small-M streaming path, for shapes with decode_fits(M, K).
// decode_folds_t(M, r): the kernel can add up T's partial sums itself.
bool decode_fits(int64_t M, int64_t K);
bool decode_folds_t(int64_t M, int r);
// With nz > 0, T holds nz partial sums [nz][M][r] of X . A which the kernel
// adds up itself (workgroup 0 also writes the total to Tout); with nz == 0, T
// is the final [M][r] with row stride ldt (default r) and Tout is unused.  B
// and Y have row strides ldb and ldy (default N).
hipError_t launch_fwd_decode(const uint16_t* X, int64_t M, const Nf4View& w,
                             const float* T, int nz, float* Tout, const uint16_t* B, int r,
                             float s, uint16_t* Y, const Nf4Tables& tb, hipStream_t stream,
                             int ldt = 0, int64_t ldb = 0, int64_t ldy = 0);

// dX[M,K] = bf16( dY . deq(W) + s . G . A^T ), MFMA path with the
// dequantized weight tiles staged in LDS and read back transposed.
GemmSplit dx_gemm_split(int64_t M, int64_t N, int64_t K);
hipError_t launch_dx_gemm(const uint16_t* dY, int64_t M, const Nf4View& w,
                          const float* G, const uint16_t* A, int r, float s,
                          uint16_t* dX, float* part, const Nf4Tables& tb, hipStream_t stream);

// Rank-r products with a split reduction; partials go to `ws`.
size_t rank_ws_floats(int64_t M, int64_t N, int64_t K, int r);
// The partials of T = X . A alone (the forward's rank product).
size_t lora_down_ws_floats(int64_t M, int64_t K, int r);

// Few-token LoRA down-projection: nz <= maxp fp32 partial sums [nz][M][r]
// of T = X . A go to ws (nz returned); M <= 16, maxp <= kMaxDownPartials.
constexpr int kMaxDownPartials = 64;
int lora_down_partial_count(int64_t K, int maxp);
hipError_t launch_lora_down_partials(const uint16_t* X, int64_t M, int64_t K, const uint16_t* A,
                                     int r, int maxp, float* ws, int* nz, hipStream_t stream);

// T[M,r] = X . A (fp32 out).
hipError_t launch_lora_down(const uint16_t* X, int64_t M, int64_t K,
                            const uint16_t* A, int r, float* T, float* ws,
                            hipStream_t stream);
// G[M,r] = dY . B^T (fp32 out) and dB[r,N] = bf16( s . T^T . dY ), both
// products in one launch and both split reductions in one more.  Row strides
// (0 = dense): ldy of dY, ldb of B and of dB, ldt of T and of G.
hipError_t launch_grad_in_and_b(const uint16_t* dY, int64_t M, int64_t N, const uint16_t* B,
                                const float* T, int r, float s, float* G, uint16_t* dB,
                                float* ws, hipStream_t stream, int64_t ldy = 0, int64_t ldb = 0,
                                int ldt = 0);
// dA[K,r] = bf16( s . X^T . G ).
hipError_t launch_grad_a(const uint16_t* X, int64_t M, int64_t K, const float* G,
                         int r, float s, uint16_t* dA, float* ws, hipStream_t stream);

// One AdamW step over n parameters (bf16 p, g; fp32 m, v, device or
// device-visible pinned host memory, 16-byte aligned), bias corrections for
// step `step` (>= 1).
hipError_t launch_adamw(uint16_t* p, const uint16_t* g, float* m, float* v, int64_t n,
                        float lr, float beta1, float beta2, float eps, float weight_decay,
                        int64_t step, hipStream_t stream);

}  // namespace qnf4
