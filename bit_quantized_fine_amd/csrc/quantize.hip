// NF4 quantization with double quantization, and standalone
// dequantization to bf16 (an op of its own).
//
// Format (list items (2) and (3) of "DL0087 QLoRA: 4-bit Quantized LoRA";
// "Double Quantization and Paged Optimizers" of "QLoRA: Finetuning 65B Models
// on a Single GPU"): blocks of 64 weights with one absmax each; the absmax
// constants quantized to 8 bits with one fp32 scale per 256 of them.  The
// level and threshold tables come in as arguments (NF4, or the INT4 / FP4
// tables of "4-bit NormalFloat" in the same page), and with dq == 0 each
// block keeps its fp32 absmax instead (the format double quantization
// improves on).
#include <cmath>
#include <cstring>

#include "device_common.hpp"
#include "kernels.hpp"

namespace qnf4 {

// Buckets of the quantizer's code search (k_quantize): 34 per sign.
constexpr int kBucketsPerSign = 34;
constexpr int kBuckets = 2 * kBucketsPerSign;
constexpr int kBucketBias = 221;   // one below bits 30..22 of 2^-16 (222)
struct QuantBuckets {
  uint32_t base[kBuckets];   // thresholds below the whole bucket
  uint32_t ta[kBuckets];     // fp32 bits of the thresholds inside it (+inf if none)
  uint32_t tb[kBuckets];
};

// The code of a normalised weight x in [-1, 1] is #{j : x > t_j} over the
// 15 thresholds.  Instead of 15 comparisons, x's bucket -- its sign, its
// binary exponent and its top mantissa bit (half an octave), with every
// |x| < 2^-16 in one bucket per sign -- selects a table entry holding the
// count of thresholds below the whole bucket and the (at most two)
// thresholds inside it; the code is that count plus two comparisons.  The
// host builds the entries from the threshold table (QuantBuckets below).
constexpr int kBucketCopies = 16;   // lane l reads copy l % 16: no bank conflicts

__device__ __forceinline__ uint32_t bucket_code(const u32x4* btab, float x, int copy) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  // (clamped at both ends: a weight that is not finite, which the format
  // excludes, still reads inside the table)
  const int b =
      min(max(static_cast<int>((u >> 22) & 0x1FFu) - kBucketBias, 0), kBucketsPerSign - 1);
  const int idx = b + static_cast<int>(u >> 31) * kBucketsPerSign;
  const u32x4 e = btab[idx * kBucketCopies + copy];
  // (elements copied to plain values first: this compiler bit-casts element
  // 0 when __builtin_bit_cast is given a vector element)
  const uint32_t base = e.x, ta = e.y, tb = e.z;
  return base + (x > __builtin_bit_cast(float, ta) ? 1u : 0u) +
         (x > __builtin_bit_cast(float, tb) ? 1u : 0u);
}

// One workgroup per double-quantization group of 256 blocks (16384 weights).
// 256 threads; each iteration covers 16 blocks, one block per 16 lanes, each
// lane holding 4 consecutive weights (one 16-byte load).  The block absmax is
// reduced across the 16 lanes and kept in LDS; the first-level constants
// never reach HBM.
__global__ __launch_bounds__(256) void k_quantize(
    const float* __restrict__ W, int64_t nblocks, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ absmax_q, float* __restrict__ absmax_scale,
    QuantBuckets bk, int dq) {
  __shared__ float cs[kGroup];
  __shared__ float wmax[4];
  __shared__ u32x4 btab[kBuckets * kBucketCopies];
  const int tid = threadIdx.x;
  for (int i = tid; i < kBuckets * kBucketCopies; i += 256) {
    const int e = i / kBucketCopies;
    btab[i] = u32x4{bk.base[e], bk.ta[e], bk.tb[e], 0u};
  }
  __syncthreads();
  const int copy = tid & (kBucketCopies - 1);
  const int64_t g = blockIdx.x;
  const int64_t b0 = g * kGroup;
  const int nblk = static_cast<int>(min<int64_t>(kGroup, nblocks - b0));
  const int sub = tid & 15;   // lane within the block's 16

#pragma unroll 4
  for (int it = 0; it < kGroup / 16; ++it) {
    const int bl = it * 16 + (tid >> 4);
    if (bl < nblk) {
      const int64_t elem = (b0 + bl) * kBlock + sub * 4;
      const float4 v = *reinterpret_cast<const float4*>(W + elem);
      float m = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
      // max over the block's 16 lanes (a DPP row): pairs, quads, the row's
      // halves (half mirror), then both halves (mirror)
      m = fmaxf(m, dpp_f32<0xB1>(m));
      m = fmaxf(m, dpp_f32<0x4E>(m));
      m = fmaxf(m, dpp_f32<0x141>(m));
      m = fmaxf(m, dpp_f32<0x140>(m));
      // x = fl32(w / c); an all-zero block divides zeros by 1 (code 7).
      const float c = m > 0.f ? m : 1.f;
      float x[4];
      if (c >= 0x1p-96f && c <= 0x1p125f) {
        // Markstein's quotient: with y = RN(1/c) and q = RN(w y), the
        // remainder r = w - q c is a float that an fma forms exactly, and
        // RN(q + r y) = RN(w / c).  The range of c keeps y normal and keeps
        // r clear of the subnormal range for |q| >= 2^-6, below the
        // smallest nonzero threshold of the three tables (NF4's, 0.021).
        // Between 2^-120 and 2^-6 only the sign of x decides the code, and
        // q has the quotient's sign; below 2^-120 the quotient may round to
        // zero, which decides the code where a table has a threshold at
        // zero (INT4's), so those weights take the IEEE divide.
        const float y = 1.0f / c;
        const float w[4] = {v.x, v.y, v.z, v.w};
        float qmin = 1.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float q = w[i] * y;
          x[i] = __builtin_fmaf(__builtin_fmaf(-q, c, w[i]), y, q);
          qmin = fminf(qmin, fabsf(q));
        }
        if (qmin < 0x1p-120f) {
#pragma unroll
          for (int i = 0; i < 4; ++i) x[i] = w[i] / c;
        }
      } else {   // IEEE divide
        x[0] = v.x / c;
        x[1] = v.y / c;
        x[2] = v.z / c;
        x[3] = v.w / c;
      }
      uint32_t packed = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) packed |= bucket_code(btab, x[i], copy) << (4 * i);
      *reinterpret_cast<uint16_t*>(codes + elem / 2) = static_cast<uint16_t>(packed);
      if (sub == 0) cs[bl] = m;
    }
  }
  __syncthreads();

  const float c = tid < nblk ? cs[tid] : 0.f;
  if (!dq) {   // fp32 constants: the absmax of every block as it is
    if (tid < nblk) absmax_scale[b0 + tid] = c;
    return;
  }
  // Second level: group max, d = fl32(max / 255), e = rint(fl32(c / d)).
  float m = c;
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((tid & 63) == 0) wmax[tid >> 6] = m;
  __syncthreads();
  const float s = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float d = s / 255.0f;
  if (tid < nblk) {
    uint8_t e = 0;
    if (d > 0.f) {
      const float r = __builtin_rintf(c / d);
      e = static_cast<uint8_t>(fminf(fmaxf(r, 0.f), 255.f));
    }
    absmax_q[b0 + tid] = e;
  }
  if (tid == 0) absmax_scale[g] = d;
}

// Standalone dequantization: each thread expands 16 code bytes (32 weights,
// half a block) into 32 bf16 values, with the block's 16 dequantized values
// formed in registers and selected by byte permutes (the same routine the
// tiled forward GEMM uses).
__global__ __launch_bounds__(256) void k_dequantize(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ absmax_q,
    const float* __restrict__ absmax_scale, int64_t nchunks,
    uint16_t* __restrict__ out, Nf4Tables tb, int dq) {
  const Levels lv = load_levels(tb);
  for (int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; c < nchunks;
       c += (int64_t)gridDim.x * blockDim.x) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(codes + c * 16);
    const Bf16Planes t = block_planes(lv, block_scale(absmax_q, absmax_scale, c >> 1, dq));
    u32x4* dst = reinterpret_cast<u32x4*>(out + c * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = dequant8_planes(w[i], t);
  }
}

// Bucket entries from the threshold table.  Bucket b of a sign holds the
// x of that sign whose bits 30..22 (exponent, top mantissa bit) are b + 221
// (b >= 1: |x| in [2^e (1 + m/2), 2^e (1 + (m + 1)/2)) with e >= -16), or
// below 222 (b = 0: |x| < 2^-16, zero and subnormals included).  For the
// bucket's least and greatest members lo <= hi, a threshold t < lo counts for
// every member, one with t >= hi for none, and one in [lo, hi) is compared
// (x > t); unused comparison slots hold +inf.  Returns false if a bucket
// would need more than two comparisons (no 4-bit table here does).
bool build_quant_buckets(const float* t, QuantBuckets& out) {
  auto f32 = [](uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; };
  auto bits = [](float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; };
  for (int sign = 0; sign < 2; ++sign) {
    for (int b = 0; b < kBucketsPerSign; ++b) {
      uint32_t lo_u, hi_u;   // magnitudes of the bucket's extreme members
      if (b == 0) {
        lo_u = 0u;
        hi_u = (static_cast<uint32_t>(kBucketBias + 1) << 22) - 1u;
      } else {
        lo_u = static_cast<uint32_t>(b + kBucketBias) << 22;
        hi_u = lo_u + (1u << 22) - 1u;
        if (hi_u > 0x3F800000u) hi_u = 0x3F800000u;   // |x| <= 1
      }
      const float lo = sign ? -f32(hi_u) : f32(lo_u);
      const float hi = sign ? -f32(lo_u) : f32(hi_u);
      uint32_t base = 0, nc = 0;
      float cmp[2] = {INFINITY, INFINITY};
      for (int j = 0; j < 15; ++j) {
        if (t[j] < lo) {
          ++base;
        } else if (t[j] < hi) {
          if (nc == 2) return false;
          cmp[nc++] = t[j];
        }
      }
      const int e = b + sign * kBucketsPerSign;
      out.base[e] = base;
      out.ta[e] = bits(cmp[0]);
      out.tb[e] = bits(cmp[1]);
    }
  }
  return true;
}

hipError_t launch_quantize(const float* W, int64_t N, int64_t K, uint8_t* codes,
                           uint8_t* absmax_q, float* absmax_scale,
                           const Nf4Tables& tb, hipStream_t stream, bool dq) {
  QuantBuckets bk;
  if (!build_quant_buckets(tb.t, bk)) return hipErrorInvalidValue;
  const int64_t nblocks = N * K / kBlock;
  const int64_t ngroups = (nblocks + kGroup - 1) / kGroup;
  hipLaunchKernelGGL(k_quantize, dim3(static_cast<unsigned>(ngroups)), dim3(256), 0,
                     stream, W, nblocks, codes, absmax_q, absmax_scale, bk, dq ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* absmax_q,
                             const float* absmax_scale, int64_t N, int64_t K,
                             uint16_t* out, const Nf4Tables& tb,
                             hipStream_t stream, bool dq) {
  const int64_t nchunks = N * K / 32;
  int64_t grid = (nchunks + 255) / 256;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(k_dequantize, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                     stream, codes, absmax_q, absmax_scale, nchunks, out, tb, dq ? 1 : 0);
  return hipGetLastError();
}

}  // namespace qnf4
