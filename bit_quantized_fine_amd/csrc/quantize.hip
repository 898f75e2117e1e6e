// NF4 quantization with double quantization, and standalone
// dequantization to bf16 (an op of its own).
//
// Format (list items (2) and (3) of "DL0087 QLoRA: 4-bit Quantized LoRA";
// "Double Quantization and Paged Optimizers" of "QLoRA: Finetuning 65B Models
// on a Single GPU"): blocks of 64 weights with one absmax each; the absmax
// constants quantized to 8 bits with one fp32 scale per 256 of them.
#include "device_common.hpp"
#include "kernels.hpp"

namespace qnf4 {

// One workgroup per double-quantization group of 256 blocks (16384 weights).
// 256 threads; each iteration covers 16 blocks, one block per 16 lanes, each
// lane holding 4 consecutive weights (one 16-byte load).  The block absmax is
// reduced across the 16 lanes and kept in LDS; the first-level constants
// never reach HBM.
__global__ __launch_bounds__(256) void k_quantize(
    const float* __restrict__ W, int64_t nblocks, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ absmax_q, float* __restrict__ absmax_scale,
    Nf4Tables tb) {
  __shared__ float cs[kGroup];
  __shared__ float wmax[4];
  const int tid = threadIdx.x;
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
      m = fmaxf(m, __shfl_xor(m, 8, 16));
      m = fmaxf(m, __shfl_xor(m, 4, 16));
      m = fmaxf(m, __shfl_xor(m, 2, 16));
      m = fmaxf(m, __shfl_xor(m, 1, 16));
      // IEEE divide; an all-zero block divides zeros by 1 (code 7).
      const float c = m > 0.f ? m : 1.f;
      const float x[4] = {v.x / c, v.y / c, v.z / c, v.w / c};
      uint32_t packed = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t code = 0;
#pragma unroll
        for (int j = 0; j < 15; ++j) code += (x[i] > tb.t[j]) ? 1u : 0u;
        packed |= code << (4 * i);
      }
      *reinterpret_cast<uint16_t*>(codes + elem / 2) = static_cast<uint16_t>(packed);
      if (sub == 0) cs[bl] = m;
    }
  }
  __syncthreads();

  // Second level: group max, d = fl32(max / 255), e = rint(fl32(c / d)).
  const float c = tid < nblk ? cs[tid] : 0.f;
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
// half a block) into 32 bf16 values.
__global__ __launch_bounds__(256) void k_dequantize(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ absmax_q,
    const float* __restrict__ absmax_scale, int64_t nchunks,
    uint16_t* __restrict__ out, Nf4Tables tb) {
  __shared__ float2 tab[256];
  build_pair_table(tab, tb, threadIdx.x, blockDim.x);
  __syncthreads();
  for (int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; c < nchunks;
       c += (int64_t)gridDim.x * blockDim.x) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(codes + c * 16);
    const float chat = block_scale(absmax_q, absmax_scale, c >> 1);
    u32x4* dst = reinterpret_cast<u32x4*>(out + c * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = dequant8(w[i], chat, tab);
  }
}

hipError_t launch_quantize(const float* W, int64_t N, int64_t K, uint8_t* codes,
                           uint8_t* absmax_q, float* absmax_scale,
                           const Nf4Tables& tb, hipStream_t stream) {
  const int64_t nblocks = N * K / kBlock;
  const int64_t ngroups = (nblocks + kGroup - 1) / kGroup;
  hipLaunchKernelGGL(k_quantize, dim3(static_cast<unsigned>(ngroups)), dim3(256), 0,
                     stream, W, nblocks, codes, absmax_q, absmax_scale, tb);
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* absmax_q,
                             const float* absmax_scale, int64_t N, int64_t K,
                             uint16_t* out, const Nf4Tables& tb,
                             hipStream_t stream) {
  const int64_t nchunks = N * K / 32;
  int64_t grid = (nchunks + 255) / 256;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(k_dequantize, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                     stream, codes, absmax_q, absmax_scale, nchunks, out, tb);
  return hipGetLastError();
}

}  // namespace qnf4
