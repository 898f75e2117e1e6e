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
 *   - Limits: K % 64 == 0 (a block lies inside one row), r % 8 == 0 and
 *     r <= 256, N % 8 == 0 for qlora_linear_fwd / qlora_linear_bwd (the
 *     kernels write 8-byte groups of 4 outputs and read 16-byte pieces of
 *     B), N <= 2^22, K <= 2^22 and N*K <= 2^32 (32-bit buffer offsets).
 *   - Path selection (results follow the same definition on both paths):
 *     qlora_linear_fwd streams the weight with the few-token kernel when
 *     M <= 16 and K <= 32768, and runs the tiled MFMA GEMM otherwise.
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
  QLORA_ERR_SHAPE = 2,      /* M < 1, N < 1, K < 64, K % 64 != 0, N % 8 != 0
                               (fwd/bwd), N > 2^22, K > 2^22 or N*K > 2^32 */
  QLORA_ERR_RANK = 3,       /* r outside [0, 256] or r % 8 != 0 */
  QLORA_ERR_ALIGN = 4,      /* a device pointer is not 16-byte aligned */
  QLORA_ERR_HIP = 5,        /* a HIP runtime call or kernel launch failed */
  QLORA_ERR_WORKSPACE = 6,  /* workspace too small */
  QLORA_ERR_SCRATCH = 7,    /* qlora_linear_fwd_noalloc: the call needs more than
                               QLORA_NOALLOC_SCRATCH_BYTES of workspace */
  QLORA_ERR_FORMAT = 8      /* qlora_q4_*: unknown codebook, or double_quant
                               not 0 or 1 */
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

/*
 * 16-entry codebooks of the qlora_q4_* calls: the 4-bit types "4-bit
 * NormalFloat" of "QLoRA: Finetuning 65B Models on a Single GPU" sets against
 * each other (NF4 is information-theoretically optimal for normally
 * distributed weights and beats INT4 and FP4).  Each is 16 fp32 levels over
 * [-1, 1], ascending; the code of a normalised weight is its nearest level,
 * ties to the lower index.
 *   NF4:  the NF4 levels (as qlora_nf4_levels).
 *   INT4: sixteen levels spaced uniformly, (2k - 15) / 15 for k = 0..15 (no
 *         zero level).
 *   FP4:  the sixteen E2M1 floats (sign, 2 exponent bits with bias 1, 1
 *         mantissa bit) divided by their largest magnitude 6; +0 is code 7,
 *         -0 code 8 (never produced by quantization).
 */
typedef enum {
  QLORA_CODEBOOK_NF4 = 0,
  QLORA_CODEBOOK_INT4 = 1,
  QLORA_CODEBOOK_FP4 = 2
} qlora_codebook;

/*
 * Read-only view of a 4-bit weight W [N, K] of any codebook and constant
 * format.  double_quant = 1: the NF4 format's constants (absmax_q N*K/64
 * bytes, absmax_scale ceil(N*K/64/256) floats, 4-byte aligned).
 * double_quant = 0: one fp32 absmax per 64-block in absmax_scale (N*K/64
 * floats, 16-byte aligned; absmax_q unused and may be NULL): the 0.5
 * bits-per-parameter format double quantization improves on (list item (3)
 * of "DL0087 QLoRA": 0.5 to about 0.127 bits).
 */
typedef struct {
  const uint8_t* codes;        /* N*K/2 bytes, 16-byte aligned */
  const uint8_t* absmax_q;
  const float* absmax_scale;
  int64_t N;
  int64_t K;
  int32_t codebook;            /* qlora_codebook */
  int32_t double_quant;        /* 1 or 0 */
} qlora_q4_weight;

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
 * Accumulation is fp32; Y is rounded to bf16 once.  M >= 1, N % 8 == 0,
 * r % 8 == 0 (QLORA_ERR_SHAPE / QLORA_ERR_RANK otherwise).
 */
int qlora_linear_fwd(const uint16_t* X, int64_t M, const qlora_nf4_weight* w,
                     const uint16_t* A, const uint16_t* B, int r, float s,
                     uint16_t* Y, float* T, void* workspace,
                     size_t workspace_bytes, qlora_stream_t stream);

/*
 * The forward of qlora_linear_fwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments and results, bit for bit, without the
 * workspace arguments.  The workspace is instead a fixed device array of
 * QLORA_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until
 * the process ends; no call allocates or frees anything.
 *   - A call whose workspace (qlora_linear_fwd_workspace_bytes) exceeds that
 *     size returns QLORA_ERR_SCRATCH before enqueueing anything.  The GEMM's
 *     split-reduction partials never exceed 32 MiB, and T's partial sums
 *     exceed it only when M . r > 2^23, so every call with M . r <= 2^23
 *     (M <= 32768 at r = 256, M <= 131072 at r = 64) fits.
 *   - The first call on a device looks up the array's device address
 *     (hipGetSymbolAddress, with that device current); make it outside
 *     graph capture.
 *   - Every call on one GPU uses that GPU's array: calls that overlap on
 *     one GPU (on different streams, or from several threads) race, and
 *     must be serialised by the caller.  The array's contents need no
 *     initialisation and keep whatever the last call left.
 */
#define QLORA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int qlora_linear_fwd_noalloc(const uint16_t* X, int64_t M,
                             const qlora_nf4_weight* w, const uint16_t* A,
                             const uint16_t* B, int r, float s, uint16_t* Y,
                             float* T, qlora_stream_t stream);

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
 * Fused multi-projection block ("LoRA placement: adapters at every layer" of
 * "QLoRA: Finetuning 65B Models on a Single GPU": adapters on every linear
 * layer, the query, key and value projections and the MLP's gate and up
 * projections among them; the rank bullet of the Mathematical Formulation of
 * "DL0087 QLoRA").  S projections that read the same input X,
 *     Y_j = X . deq(W_j)^T + s . (X . A_j) . B_j,   j = 0 .. S-1,
 * computed together: one product T = X . [A_0 .. A_{S-1}] and, for M > 16,
 * one dequantizing GEMM over all S * nseg weight rows, each row tile adding
 * its own projection's adapter.
 *   w  [S*nseg, K]: the S weights stacked along N (nseg = w->N / S), quantized
 *      as one NF4 weight.  nseg % 128 == 0 and nseg*K % 16384 == 0 (each
 *      projection starts at a group of 256 block constants, so it equals the
 *      projection quantized on its own); QLORA_ERR_SHAPE otherwise.
 *   A  [K, S*r] bf16: A_j in columns j*r .. j*r+r-1.
 *   B  [r, S*nseg] bf16: B_j in columns j*nseg .. j*nseg+nseg-1.
 *   Y  [M, S*nseg] bf16 (output): Y_j in the same columns as B_j.
 *   T  [M, S*r] fp32 (output): T_j = X . A_j in the columns of A_j.
 *   1 <= r and S*r <= 256, r % 8 == 0 (QLORA_ERR_RANK otherwise).
 * Workspace: qlora_block_fwd_workspace_bytes(M, S, nseg, K, r) bytes.
 */
size_t qlora_block_fwd_workspace_bytes(int64_t M, int S, int64_t nseg, int64_t K, int r);
int qlora_block_fwd(const uint16_t* X, int64_t M, const qlora_nf4_weight* w, int S,
                    const uint16_t* A, const uint16_t* B, int r, float s, uint16_t* Y,
                    float* T, void* workspace, size_t workspace_bytes,
                    qlora_stream_t stream);

/*
 * Backward of the fused block (list item (4) of "DL0087 QLoRA"): with dY
 * [M, S*nseg] holding dY_j in the columns of Y_j,
 *   G_j = dY_j . B_j^T, dB_j = s . T_j^T . dY_j   (dB [r, S*nseg], like B)
 *   dA  = s . X^T . [G_0 .. G_{S-1}]              (dA [K, S*r], like A)
 *   dX  = sum_j dY_j . deq(W_j) + s . G_j . A_j^T (one GEMM over all rows;
 *         skipped if dX == NULL)
 * T_saved is the forward's T [M, S*r], or NULL to recompute it.  Shapes,
 * limits and errors as for qlora_block_fwd; workspace:
 * qlora_block_bwd_workspace_bytes(M, S, nseg, K, r) bytes.
 */
size_t qlora_block_bwd_workspace_bytes(int64_t M, int S, int64_t nseg, int64_t K, int r);
int qlora_block_bwd(const uint16_t* dY, const uint16_t* X, int64_t M,
                    const qlora_nf4_weight* w, int S, const uint16_t* A,
                    const uint16_t* B, int r, float s, const float* T_saved,
                    uint16_t* dX, uint16_t* dA, uint16_t* dB, void* workspace,
                    size_t workspace_bytes, qlora_stream_t stream);

/*
 * 16-bit LoRA on the same kernels: the layer with a bf16 base weight instead
 * of an NF4 one, the baseline QLoRA is set against ("Performance Reality" of
 * "QLoRA: Quantized Low Rank Adaptation at Extreme Scale": QLoRA compared
 * with full 16-bit LoRA; the opening of "DL0087 QLoRA").  It runs the tiled
 * GEMMs of qlora_linear_fwd / qlora_linear_bwd with the weight tile loaded
 * instead of dequantized, and the same rank products and LoRA epilogue, so
 * the two forms differ only in the weight's bytes and the dequantization:
 *   Y  = X . W^T + s . T . B,  T = X . A
 *   dX = dY . W + s . G . A^T, dA = s . X^T . G, dB = s . T^T . dY, G = dY . B^T
 *   W  [N, K] bf16 (device, read-only), row-major, 16-byte aligned;
 *      N % 8 == 0, K % 64 == 0, N, K <= 2^22 and N*K <= 2^30
 *      (QLORA_ERR_SHAPE otherwise: the kernels address W with 32-bit byte
 *      offsets below 2^31).
 * Every other argument, output, limit and error is that of
 * qlora_linear_fwd / qlora_linear_bwd.  The tiled GEMM runs at every M
 * (there is no streaming path for M <= 16).  Workspace:
 * qlora_lora16_fwd_workspace_bytes / qlora_lora16_bwd_workspace_bytes.
 */
size_t qlora_lora16_fwd_workspace_bytes(int64_t M, int64_t N, int64_t K, int r);
size_t qlora_lora16_bwd_workspace_bytes(int64_t M, int64_t N, int64_t K, int r);
int qlora_lora16_fwd(const uint16_t* X, int64_t M, const uint16_t* W, int64_t N, int64_t K,
                     const uint16_t* A, const uint16_t* B, int r, float s, uint16_t* Y,
                     float* T, void* workspace, size_t workspace_bytes,
                     qlora_stream_t stream);
int qlora_lora16_bwd(const uint16_t* dY, const uint16_t* X, int64_t M, const uint16_t* W,
                     int64_t N, int64_t K, const uint16_t* A, const uint16_t* B, int r,
                     float s, const float* T_saved, uint16_t* dX, uint16_t* dA,
                     uint16_t* dB, void* workspace, size_t workspace_bytes,
                     qlora_stream_t stream);

/*
 * The NF4 calls for any codebook and constant format (qlora_q4_weight): the
 * same kernels with the codebook's level and threshold tables and, without
 * double quantization, fp32 block constants.  Dequantization is
 * bf16_rne(fl32(q[code] * c)) with c = fl32(e * d) (double_quant = 1) or the
 * stored fp32 absmax (double_quant = 0).
 *   qlora_q4_levels / qlora_q4_thresholds: a codebook's 16 levels and the 15
 *     fp32 thresholds t_j of its quantizer (code = #{j : x > t_j}), into host
 *     memory.
 *   qlora_q4_scale_count: floats of absmax_scale for the format.
 *   qlora_q4_quantize: as qlora_nf4_quantize, with absmax_q written only when
 *     double_quant = 1 (may be NULL otherwise).
 *   qlora_q4_dequantize, qlora_q4_linear_fwd, qlora_q4_linear_bwd: as the
 *     qlora_nf4 / qlora_linear calls, with the same arguments, limits, path
 *     selection and workspace sizes (qlora_linear_fwd_workspace_bytes,
 *     qlora_linear_bwd_workspace_bytes).
 * Errors: as those calls, plus QLORA_ERR_FORMAT for an unknown codebook or
 * a double_quant other than 0 or 1.
 */
int qlora_q4_levels(int codebook, float* out16);
int qlora_q4_thresholds(int codebook, float* out15);
size_t qlora_q4_scale_count(int64_t N, int64_t K, int double_quant);
int qlora_q4_quantize(const float* W, int64_t N, int64_t K, int codebook, int double_quant,
                      uint8_t* codes, uint8_t* absmax_q, float* absmax_scale,
                      qlora_stream_t stream);
int qlora_q4_dequantize(const qlora_q4_weight* w, uint16_t* W_bf16, qlora_stream_t stream);
int qlora_q4_linear_fwd(const uint16_t* X, int64_t M, const qlora_q4_weight* w,
                        const uint16_t* A, const uint16_t* B, int r, float s, uint16_t* Y,
                        float* T, void* workspace, size_t workspace_bytes,
                        qlora_stream_t stream);
int qlora_q4_linear_bwd(const uint16_t* dY, const uint16_t* X, int64_t M,
                        const qlora_q4_weight* w, const uint16_t* A, const uint16_t* B, int r,
                        float s, const float* T_saved, uint16_t* dX, uint16_t* dA,
                        uint16_t* dB, void* workspace, size_t workspace_bytes,
                        qlora_stream_t stream);

/*
 * Optimizer step on the adapters, and its state paged between HBM and host
 * memory (numbered list items (4) and (5) of "DL0087 QLoRA": only the
 * adapters train, so optimizer state scales with the adapter rank, and the
 * optimizer states are paged to host RAM during transient memory spikes;
 * "Memory Management Details" of "QLoRA: Quantized Low Rank Adaptation at
 * Extreme Scale": paged optimizers offload their states to CPU memory).
 *
 * qlora_adamw_step: one AdamW step (decoupled weight decay) over n
 * parameters, step = 1, 2, ...:
 *     p <- p (1 - lr wd);  m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2
 *     p <- p - lr (m / (1 - b1^step)) / (sqrt(v / (1 - b2^step)) + eps)
 * computed in fp32.  param [n] bf16 (updated in place), grad [n] bf16, the
 * moments exp_avg, exp_avg_sq [n] fp32 (updated in place) -- HBM or the
 * device-visible address of pinned host memory (qlora_paged_state_pointers
 * gives either).  All four 16-byte aligned.  Adapters kept in one flat
 * buffer (A and B of every layer as slices) take one call per step.
 * Errors: QLORA_ERR_NULL, QLORA_ERR_ALIGN, QLORA_ERR_SHAPE (n < 1, step < 1,
 * betas outside [0, 1), eps <= 0, lr or weight_decay < 0), QLORA_ERR_HIP.
 */
typedef struct {
  float lr;
  float beta1;
  float beta2;
  float eps;
  float weight_decay;
} qlora_adamw_config;

int qlora_adamw_step(uint16_t* param, const uint16_t* grad, float* exp_avg, float* exp_avg_sq,
                     int64_t n, const qlora_adamw_config* cfg, int64_t step,
                     qlora_stream_t stream);

/*
 * Paged optimizer state: the moments m and v of n parameters (fp32, zero at
 * creation), owned by the library.  Resident, they live in HBM of the device
 * current at creation; paged out, in a pinned host home that the GPU reads
 * and writes directly (a step on paged-out state runs at the host link's
 * rate, with the same results bit for bit).  Paging is explicit: there is no
 * demand paging.
 *   qlora_paged_state_create: n >= 1; on_host != 0 starts paged out.
 *   qlora_paged_state_page_out: copies the moments to the host home
 *     (allocated on first use), waits for the copy on `stream`, frees the HBM
 *     copy.  A no-op when already paged out.
 *   qlora_paged_state_page_in: allocates HBM and copies the moments back
 *     (ordered on `stream`).  If the allocation fails the state stays paged
 *     out, usable, and QLORA_ERR_HIP is returned.  A no-op when resident.
 *   qlora_paged_state_pointers: the current m and v (device-visible), to
 *     pass to qlora_adamw_step; they change with every page-out and page-in.
 *   qlora_paged_state_resident: 1 when the moments are in HBM, else 0.
 *   qlora_paged_state_read / _write: copy the moments, as [2][n] fp32 (m
 *     then v), to or from caller memory (device or host; ordered on
 *     `stream`), e.g. to checkpoint and restore them.
 * The page calls allocate or free memory, so they stay outside HIP graph
 * capture, and run with the creation device current (QLORA_ERR_SHAPE
 * otherwise); work that uses the state must be ordered before a page-out on
 * `stream`, which page-out synchronizes.
 */
typedef struct qlora_paged_state qlora_paged_state;

int qlora_paged_state_create(int64_t n, int on_host, qlora_paged_state** out);
int qlora_paged_state_destroy(qlora_paged_state* st);
int qlora_paged_state_page_out(qlora_paged_state* st, qlora_stream_t stream);
int qlora_paged_state_page_in(qlora_paged_state* st, qlora_stream_t stream);
int qlora_paged_state_pointers(const qlora_paged_state* st, float** exp_avg,
                               float** exp_avg_sq);
int qlora_paged_state_resident(const qlora_paged_state* st);
int qlora_paged_state_read(const qlora_paged_state* st, float* dst, qlora_stream_t stream);
int qlora_paged_state_write(qlora_paged_state* st, const float* src, qlora_stream_t stream);

/*
 * Kernel timing for measurement.  When enabled (enable != 0), the library
 * records a pair of HIP events on the launch stream around every launch of
 * the kernel families below and accumulates their elapsed times; reading
 * synchronises on the recorded events.  Disabled by default; enabling adds
 * two event records per timed launch.
 *   family 0: tiled forward GEMM (dequantizing at M > 16; also the bf16
 *             weight of qlora_lora16_fwd)
 *   family 1: tiled dX GEMM (dequantizing; also qlora_lora16_bwd)
 *   family 2: decode GEMV (forward, M <= 16)
 *   family 3: quantize
 *   family 4: small rank-r GEMMs and reductions (T, G, dA, dB)
 *   family 5: AdamW step (qlora_adamw_step)
 * qlora_profile_read writes the total milliseconds and launch count of a
 * family (either pointer may be NULL) and returns QLORA_ERR_SHAPE for an
 * unknown family.  qlora_profile_reset clears all totals.
 */
int qlora_profile_enable(int enable);
int qlora_profile_read(int family, double* total_ms, int64_t* launches);
int qlora_profile_reset(void);

/*
 * Peak probes (measurement only; not part of the layer).  They give the
 * rates this GPU reaches, against which kernel rates are also reported.
 *   qlora_probe_hbm_read: `workgroups` workgroups of 256 threads read the
 *     `bytes` (a multiple of 16, buf 16-byte aligned) of device buffer buf
 *     once with 16-byte non-temporal loads.  The caller times the launch;
 *     use a buffer far larger than the last-level cache (e.g. 4 GiB).
 *   qlora_probe_mfma_bf16: `workgroups` workgroups of 4 waves; every wave
 *     issues iters x 8 independent v_mfma_f32_32x32x16_bf16 on register
 *     operands: workgroups x 4 x iters x 8 x 32768 flops.
 * sink: device memory of at least `workgroups` uint32, written only in a
 * case that does not occur (it keeps the work from being removed).
 * Errors: QLORA_ERR_NULL, QLORA_ERR_ALIGN, QLORA_ERR_SHAPE (workgroups or
 * iters < 1), QLORA_ERR_HIP on a failed launch.
 */
int qlora_probe_hbm_read(const void* buf, size_t bytes, uint32_t* sink, int workgroups,
                         qlora_stream_t stream);
int qlora_probe_mfma_bf16(int64_t iters, int workgroups, uint32_t* sink,
                          qlora_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_NF4_H */
