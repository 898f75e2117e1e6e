/*
 * qlora_nf4.h -- C ABI of the QLoRA frozen-base NF4 linear layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (Mathematical Formulation and Figure 1 of "DL0087 QLoRA: 4-bit
 * Quantized LoRA"; the formula was lost when that page was extracted and is
 * rebuilt here from its bullets):
 *
 *     Y = X . deq(W)^T + s . (X . A) . B
 *
 *   X  [M, K]  bf16 activations (tokens x in-features), row-major
 *   W  [N, K]  frozen base weight, out x in (the layout of a linear layer),
 *              stored as NF4 codes with double-quantized block constants
 *   A  [K, r]  bf16 LoRA down-projection, row-major
 *   B  [r, N]  bf16 LoRA up-projection, row-major
 *   s          LoRA scale (alpha / r)
 *   Y  [M, N]  bf16 output, row-major
 *
 * Storage format of W (list items (2) and (3) of "DL0087 QLoRA"; "Double
 * Quantization and Paged Optimizers" of "QLoRA: Finetuning 65B Models on a
 * Single GPU"):
 *   - blocks of 64 consecutive weights of the row-major flattening of W
 *     (K must be a multiple of 64, so a block lies inside one row);
 *   - codes: 4-bit index into the 16 NF4 levels, two per byte, the even
 *     element in the low nibble: N*K/2 bytes;
 *   - absmax_q: one 8-bit constant per block: N*K/64 bytes;
 *   - absmax_scale: one fp32 second-level scale per 256 consecutive blocks
 *     (the last group may be short): ceil(N*K/64/256) floats.
 *   Block b's constant is c_hat = fl32(absmax_q[b] * absmax_scale[b/256])
 *   and its weights are bf16_rne(fl32(level[code] * c_hat)).
 *
 * Conventions for every entry point:
 *   - Pointers named as device pointers are device memory owned by the
 *     caller; the library never allocates, frees or keeps them.
 *   - Device buffers must be 16-byte aligned, contiguous, row-major.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *     No entry point synchronises the host.
 *   - Arguments are validated before anything is enqueued; on error nothing
 *     is enqueued and a nonzero qlora_status is returned.  A failed kernel
 *     launch returns QLORA_ERR_HIP.  Faults inside kernels surface at the
 *     caller's next synchronisation.
 *   - A workspace is scratch for the duration of one call: calls that may
 *     run concurrently (on different streams) need separate workspaces, and
 *     outputs must not overlap inputs or the workspace.
 *   - The NF4 weight buffers are read-only for fwd/bwd: the base is frozen
 *     ("The Quantization Layer" of "QLoRA: Quantized Low Rank Adaptation at
 *     Extreme Scale").
 *   - r = 0 (A and B may then be NULL) selects the base-only layer.
 */
#ifndef QLORA_NF4_H
#define QLORA_NF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QLORA_OK = 0,
  QLORA_ERR_NULL = 1,       /* a required pointer is NULL */
  QLORA_ERR_SHAPE = 2,      /* M, N or K out of range, or K % 64 != 0 */
  QLORA_ERR_RANK = 3,       /* r outside [0, 256] */
  QLORA_ERR_ALIGN = 4,      /* a device pointer is not 16-byte aligned */
  QLORA_ERR_HIP = 5,        /* a HIP runtime call or kernel launch failed */
  QLORA_ERR_WORKSPACE = 6   /* workspace too small */
} qlora_status;

/* A hipStream_t, passed as an opaque pointer so this header needs no HIP. */
typedef void* qlora_stream_t;

/* Read-only view of an NF4 weight W [N, K] in device memory. */
typedef struct {
  const uint8_t* codes;        /* N*K/2 bytes */
  const uint8_t* absmax_q;     /* N*K/64 bytes */
  const float* absmax_scale;   /* ceil(N*K/64/256) floats */
  int64_t N;
  int64_t K;
} qlora_nf4_weight;

/* Human-readable name of a status code (static string, never NULL). */
const char* qlora_status_string(int status);

/* Library version as "major.minor.patch" (static string). */
const char* qlora_version(void);

/*
 * The 16 NF4 levels, ascending, into host memory `out16` ("4-bit
 * NormalFloat" of "QLoRA: Finetuning 65B Models on a Single GPU": levels at
 * normal quantiles, each covering equal probability mass; Mathematical
 * Formulation of "DL0087 QLoRA": rescaled to [-1, 1] with an exact zero).
 * Construction: 8 positive levels at Phi^-1(1/2 + (j - 1/2)/16), j = 1..8,
 * and 7 negative levels at -Phi^-1(1/2 + (j - 1/2)/14), j = 1..7, each side
 * divided by its extreme value, plus 0; computed once on the host in
 * extended precision and rounded to fp32.  Returns QLORA_ERR_NULL if
 * out16 is NULL.
 */
int qlora_nf4_levels(float* out16);

/*
 * The 15 decision thresholds of nearest-level encoding, into host memory:
 * t[j] is the largest fp32 not above the exact midpoint of levels j and j+1,
 * so the code of a normalised x is the number of t[j] with x > t[j]
 * (ties go to the lower level).
 */
int qlora_nf4_thresholds(float* out15);

/* Sizes of the three buffers of an N x K NF4 weight (0 if K % 64 != 0). */
size_t qlora_nf4_codes_bytes(int64_t N, int64_t K);
size_t qlora_nf4_absmax_q_bytes(int64_t N, int64_t K);
size_t qlora_nf4_scale_count(int64_t N, int64_t K);

/*
 * Quantize a float32 weight W [N, K] (device) to NF4 with double
 * quantization (list items (1)-(3) of "DL0087 QLoRA").
 * Per block: c = max|w|, x = fl32(w / c) (IEEE divide), code = nearest
 * level (lower on ties); an all-zero block gets c = 0 and code 7.
 * Per group of 256 blocks: d = fl32(max c / 255), e = rint_even(fl32(c / d))
 * clamped to [0, 255] (e = 0 when d = 0).  The codes use the unquantized c.
 * Outputs (device): codes [N*K/2], absmax_q [N*K/64], absmax_scale
 * [ceil(N*K/16384)].  W must be finite.  N >= 1, K >= 64, K % 64 == 0,
 * N <= 2^22, K <= 2^22 and N*K <= 2^32 (the kernels address a weight's
 * codes, and a 256-token tile of X or dY, with 32-bit byte offsets); the
 * same limits apply to every qlora_nf4_weight.
 */
int qlora_nf4_quantize(const float* W, int64_t N, int64_t K, uint8_t* codes,
                       uint8_t* absmax_q, float* absmax_scale,
                       qlora_stream_t stream);

/*
 * Dequantize W to bf16 (a standalone op; Mathematical Formulation of
 * "DL0087 QLoRA").  W_bf16 [N, K] (device, bf16 bit patterns) receives
 * bf16_rne(fl32(level[code] * fl32(e * d))).  The training path never
 * materialises this tensor; this entry point exists for inspection.
 */
int qlora_nf4_dequantize(const qlora_nf4_weight* w, uint16_t* W_bf16,
                         qlora_stream_t stream);

/*
 * Workspace bytes qlora_linear_fwd needs for these sizes: split-reduction
 * partials of the LoRA down-projection, and those of the dequantizing GEMM
 * when its tiles are too few for the GPU (small M; then also for r = 0).
 * Contents need no initialisation.
 */
size_t qlora_linear_fwd_workspace_bytes(int64_t M, int64_t N, int64_t K, int r);

/*
 * Forward (Mathematical Formulation and Figure 1 of "DL0087 QLoRA";
 * "The Quantization Layer" of "QLoRA: Quantized Low Rank Adaptation at
 * Extreme Scale": dequantize to bf16 on the fly, matmul, add the LoRA update).
 *   X  [M, K] bf16 (device)          Y [M, N] bf16 (device, output)
 *   A  [K, r], B [r, N] bf16 (device; may be NULL when r == 0)
 *   T  [M, r] fp32 (device, output; required when r > 0): T = X . A,
 *      kept for the backward pass.
 *   workspace: device, at least qlora_linear_fwd_workspace_bytes() bytes
 *      (may be NULL when that is 0).
 * Accumulation is fp32; Y is rounded to bf16 once.  M >= 1.
 */
int qlora_linear_fwd(const uint16_t* X, int64_t M, const qlora_nf4_weight* w,
                     const uint16_t* A, const uint16_t* B, int r, float s,
                     uint16_t* Y, float* T, void* workspace,
                     size_t workspace_bytes, qlora_stream_t stream);

/*
 * Workspace bytes qlora_linear_bwd needs (G = dY . B^T, the recomputed T
 * when none is passed, and split-reduction partials of the rank-r products
 * and, for small M, of the dX GEMM).  No initialisation needed.
 */
size_t qlora_linear_bwd_workspace_bytes(int64_t M, int64_t N, int64_t K, int r);

/*
 * Backward (list item (4) of "DL0087 QLoRA": gradients pass through
 * the frozen 4-bit weights and are stored only for the adapters; the
 * backward dequantizes again; "The Efficient Symphony of the QLoRA
 * Workflow" of "QLoRA (Quantized Low-Rank Adaptation)").
 *   G  = dY . B^T                       (workspace, fp32)
 *   dX = dY . deq(W) + s . G . A^T      [M, K] bf16, skipped if dX == NULL
 *   dA = s . X^T . G                    [K, r] bf16
 *   dB = s . T^T . dY                   [r, N] bf16
 * T_saved [M, r] fp32 is the T of the forward pass; NULL recomputes
 * T = X . A (the gradient-checkpointing form).  No gradient is formed for W
 * or its constants.  dA and dB may be NULL only when r == 0.
 */
int qlora_linear_bwd(const uint16_t* dY, const uint16_t* X, int64_t M,
                     const qlora_nf4_weight* w, const uint16_t* A,
                     const uint16_t* B, int r, float s, const float* T_saved,
                     uint16_t* dX, uint16_t* dA, uint16_t* dB, void* workspace,
                     size_t workspace_bytes, qlora_stream_t stream);

/*
 * Kernel timing for measurement.  When enabled (enable != 0), the library
 * records a pair of HIP events on the launch stream around every launch of
 * the kernel families below and accumulates their elapsed times; reading
 * synchronises on the recorded events.  Disabled by default; enabling adds
 * two event records per timed launch.
 *   family 0: dequantizing GEMM (forward, M > 16)
 *   family 1: dequantizing GEMM (backward dX)
 *   family 2: decode GEMV (forward, M <= 16)
 *   family 3: quantize
 *   family 4: small rank-r GEMMs and reductions (T, G, dA, dB)
 * qlora_profile_read writes the total milliseconds and launch count of a
 * family (either pointer may be NULL) and returns QLORA_ERR_SHAPE for an
 * unknown family.  qlora_profile_reset clears all totals.
 */
int qlora_profile_enable(int enable);
int qlora_profile_read(int family, double* total_ms, int64_t* launches);
int qlora_profile_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_NF4_H */
