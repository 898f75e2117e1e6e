// Forward for few tokens (M <= 16): the bandwidth-bound decode path.
//
// Y = X . deq(W)^T + s . T . B with T = X . A computed beforehand.  At small
// M the layer is a stream over the NF4 weight (0.516 bytes per weight), so
// the kernel is organised around the code stream: every lane issues 16-byte
// loads of 32 consecutive codes, dequantizes them in registers (Mathematical
// Formulation of "DL0087 QLoRA": the bf16 tile is rebuilt just before the
// matmul and discarded) and feeds them straight to v_mfma_f32_16x16x32_bf16
// with the token dimension padded to 16.
//
// Workgroup = 4 waves on 16 weight rows.  Chunk c covers k in [128c, 128c+128);
// wave w takes chunks w, w+4, ...; lane l works on row n0 + (l % 16) and the
// 32 k starting at 128c + 32(l / 16).  The four waves' partial sums meet in
// LDS; the LoRA update is added as extra MFMA steps over the rank, spread
// over the waves.
#include "device_common.hpp"
#include "kernels.hpp"

namespace qnf4 {

constexpr int kDecRows = 16;
constexpr int kDecXLdsBytes = 64 * 1024;   // X staged in LDS when M*K*2 fits

// XLDS: X [M, K] is copied once into LDS and the MFMA B fragments are read
// from there; otherwise each lane loads its X fragments from global memory.
// DB: chunks per load batch; two batches are in flight per wave.
template <bool XLDS, int DB>
__global__ __launch_bounds__(256) void k_fwd_decode(
    const uint16_t* __restrict__ X, int M, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ absmax_q, const float* __restrict__ absmax_scale,
    int64_t N, int64_t K, const float* __restrict__ T, int nz, float* __restrict__ Tout,
    const uint16_t* __restrict__ Bl, int r, float s, uint16_t* __restrict__ Y,
    Nf4Tables tb) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xlds[];
  __shared__ float2 tab[256];
  __shared__ f32x4 red[4][64];
  __shared__ __attribute__((aligned(16))) uint16_t xzero[8];   // read by lanes past M
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * kDecRows;
  const int64_t n = n0 + li;
  const bool n_ok = n < N;
  const bool m_ok = li < M;
  const int nchunks = static_cast<int>((K + 127) / 128);
  const uint16_t* xrow = X + (int64_t)li * K;
  const int64_t brow = n * (K / kBlock);

  // Buffer descriptors: rows n >= N fall outside the code / constant buffers
  // and read as zero; a chunk past K (half of the last chunk when K % 128 is
  // 64, or past the wave's range) gets a zero block scale, so whatever code
  // bytes it reads contribute zero.
  const uint32_t nb = static_cast<uint32_t>(N * K / kBlock);
  const BufRes rc = make_bufres(codes, static_cast<uint32_t>(N * K / 2));
  const BufRes re = make_bufres(absmax_q, nb);
  const BufRes rd = make_bufres(absmax_scale, ((nb + kGroup - 1) / kGroup) * 4u);
  const uint32_t cbase = static_cast<uint32_t>(n * (K / 2)) + 64u * wave + 16u * g;
  const uint32_t ebase = static_cast<uint32_t>(brow) + 2u * wave + (g >> 1);

  // Chunks of this wave: c = wave + 4t, t < nmine.
  const int nmine = nchunks > wave ? (nchunks - wave + 3) / 4 : 0;
  u32x4 cw[2][DB];
  uint32_t ce[2][DB];
  float cd[2][DB];
  uint32_t okm[2];   // bit u: chunk u of the batch lies inside K (applied at use)
  u32x4 xv[XLDS ? 1 : 2][XLDS ? 1 : DB][4];
  const int K32 = static_cast<int>(K);
  auto load_batch = [&](int t0, int st) {
    const uint32_t co = cbase + 256u * t0, eo = ebase + 8u * t0;
    uint32_t m = 0;
#pragma unroll
    for (int u = 0; u < DB; ++u) {
      const int t = t0 + u;
      const int k0 = (wave + 4 * t) * 128 + 32 * g;
      const bool ok = t < nmine && k0 < K32;
      m |= ok ? (1u << u) : 0u;
      cw[st][u] = buf_load16(rc, co + 256u * u);
      ce[st][u] = buf_load_u8(re, eo + 8u * u);
      cd[st][u] = buf_load_f32(rd, ((eo + 8u * u) >> 8) * 4u);
      if constexpr (!XLDS) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          xv[st][u][i] = (m_ok && ok) ? *reinterpret_cast<const u32x4*>(xrow + k0 + 8 * i)
                                      : u32x4{0, 0, 0, 0};
      }
    }
    okm[st] = m;
  };
  // Code loads first (the HBM stream), then the small X staging and the
  // level table while they are in flight.
  if (nmine > 0) load_batch(0, 0);
  if (nmine > DB) load_batch(DB, 1);

  // LoRA update as extra MFMA steps: P[n, j] = B[j, n], Q[m, j] = s*T[m, j]
  // split into bf16 hi and lo.  Step q = (j0 / 32) pairs with both halves;
  // the 32-rank steps are dealt round-robin to the waves, and the first
  // step's operands are loaded now so the tail waits on no fresh loads.
  const int nlsteps = (r + 31) / 32;
  auto lora_load = [&](int q, uint32_t* bw, f32x4* tq) {
    const int j = 32 * q + 8 * g;
    const bool j_ok = j < r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lo = 0, hi = 0;
      if (n_ok && j_ok) {
        lo = Bl[(int64_t)(j + 2 * i) * N + n];
        hi = Bl[(int64_t)(j + 2 * i + 1) * N + n];
      }
      bw[i] = lo | (hi << 16);
    }
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    tq[0] = z;
    tq[1] = z;
    if (m_ok && j_ok) {
      if (nz == 0) {
        tq[0] = *reinterpret_cast<const f32x4*>(T + (int64_t)li * r + j);
        tq[1] = *reinterpret_cast<const f32x4*>(T + (int64_t)li * r + j + 4);
      } else {
        // add up the partial sums of T: eight independent streams so the
        // loads overlap, combined in a fixed order (deterministic)
        f32x4 a0[8], a1[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) a0[u] = a1[u] = z;
        for (int z0 = 0; z0 < nz; z0 += 8) {
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            if (z0 + u < nz) {
              const float* p = T + ((int64_t)(z0 + u) * M + li) * r + j;
              a0[u] += *reinterpret_cast<const f32x4*>(p);
              a1[u] += *reinterpret_cast<const f32x4*>(p + 4);
            }
          }
        }
        tq[0] = ((a0[0] + a0[1]) + (a0[2] + a0[3])) + ((a0[4] + a0[5]) + (a0[6] + a0[7]));
        tq[1] = ((a1[0] + a1[1]) + (a1[2] + a1[3])) + ((a1[4] + a1[5]) + (a1[6] + a1[7]));
        if (blockIdx.x == 0) {
          *reinterpret_cast<f32x4*>(Tout + (int64_t)li * r + j) = tq[0];
          *reinterpret_cast<f32x4*>(Tout + (int64_t)li * r + j + 4) = tq[1];
        }
      }
    }
  };
  uint32_t lb[4];
  f32x4 lt[2];
  if (wave < nlsteps) lora_load(wave, lb, lt);
  if (tid == 0) *reinterpret_cast<u32x4*>(xzero) = u32x4{0, 0, 0, 0};
  if constexpr (XLDS) {
    const int64_t nx = (int64_t)M * K / 8;
    for (int64_t i = tid; i < nx; i += 256)
      reinterpret_cast<u32x4*>(xlds)[i] = reinterpret_cast<const u32x4*>(X)[i];
  }
  build_pair_table(tab, tb, tid, 256);
  __syncthreads();

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto mul_batch = [&](int t0, int st) {
#pragma unroll
    for (int u = 0; u < DB; ++u) {
      const bool ok = (okm[st] >> u) & 1u;
      const float chat = ok ? static_cast<float>(ce[st][u]) * cd[st][u] : 0.f;
      const int k0 = (wave + 4 * (t0 + u)) * 128 + 32 * g;
      const bool xok = m_ok && ok;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x4 b;
        if constexpr (XLDS)   // lanes without data read the zero slot (no branch)
          b = *reinterpret_cast<const u32x4*>(xok ? xlds + li * K32 + k0 + 8 * i : xzero);
        else
          b = xv[st][u][i];
        acc = mfma16(dequant8(cw[st][u][i], chat, tab), b, acc);
      }
    }
  };
  for (int t0 = 0; t0 < nmine; t0 += 2 * DB) {
    mul_batch(t0, 0);
    if (t0 + 2 * DB < nmine) load_batch(t0 + 2 * DB, 0);
    if (t0 + DB >= nmine) break;
    mul_batch(t0 + DB, 1);
    if (t0 + 3 * DB < nmine) load_batch(t0 + 3 * DB, 1);
  }

  for (int q = wave; q < nlsteps; q += 4) {
    if (q != wave) lora_load(q, lb, lt);
    const float v[8] = {lt[0].x * s, lt[0].y * s, lt[0].z * s, lt[0].w * s,
                        lt[1].x * s, lt[1].y * s, lt[1].z * s, lt[1].w * s};
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split_bf16x2(v[2 * i], v[2 * i + 1], h[i], l[i]);
    const u32x4 bw = {lb[0], lb[1], lb[2], lb[3]};
    acc = mfma16(bw, u32x4{h[0], h[1], h[2], h[3]}, acc);
    acc = mfma16(bw, u32x4{l[0], l[1], l[2], l[3]}, acc);
  }

  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    const f32x4 t = red[0][lane] + red[1][lane] + red[2][lane] + red[3][lane];
    const int64_t nout = n0 + 4 * g;   // 4 consecutive outputs of token li
    if (li < M && nout < N) {
      *reinterpret_cast<u32x2*>(Y + (int64_t)li * N + nout) =
          u32x2{pack_bf16x2(t.x, t.y), pack_bf16x2(t.z, t.w)};
    }
  }
}

hipError_t launch_fwd_decode(const uint16_t* X, int64_t M, const Nf4View& w,
                             const float* T, int nz, float* Tout, const uint16_t* B, int r,
                             float s, uint16_t* Y, const Nf4Tables& tb, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>((w.N + kDecRows - 1) / kDecRows);
  const size_t xbytes = static_cast<size_t>(M) * w.K * 2;
  // allow the X staging buffer beyond the default dynamic-LDS limit (once)
  static const bool xlds_ok =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&k_fwd_decode<true, 8>),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          kDecXLdsBytes) == hipSuccess;
  prof_begin(2, stream);
  if (xlds_ok && xbytes <= kDecXLdsBytes) {
    hipLaunchKernelGGL((k_fwd_decode<true, 8>), dim3(grid), dim3(256), xbytes, stream, X,
                       (int)M, w.codes, w.absmax_q, w.absmax_scale, w.N, w.K, T, nz, Tout, B, r,
                       s, Y, tb);
  } else {
    hipLaunchKernelGGL((k_fwd_decode<false, 2>), dim3(grid), dim3(256), 0, stream, X, (int)M,
                       w.codes, w.absmax_q, w.absmax_scale, w.N, w.K, T, nz, Tout, B, r, s, Y,
                       tb);
  }
  prof_end(2, stream);
  return hipGetLastError();
}

}  // namespace qnf4
