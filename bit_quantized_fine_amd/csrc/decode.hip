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
// LDS; wave 0 also adds the LoRA update as extra MFMA steps over the rank.
#include "device_common.hpp"
#include "kernels.hpp"

namespace qnf4 {

constexpr int kDecRows = 16;

__global__ __launch_bounds__(256) void k_fwd_decode(
    const uint16_t* __restrict__ X, int M, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ absmax_q, const float* __restrict__ absmax_scale,
    int64_t N, int64_t K, const float* __restrict__ T,
    const uint16_t* __restrict__ Bl, int r, float s, uint16_t* __restrict__ Y,
    Nf4Tables tb) {
  __shared__ float2 tab[256];
  __shared__ f32x4 red[4][64];
  const int tid = threadIdx.x;
  build_pair_table(tab, tb, tid, 256);
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * kDecRows;
  const int64_t n = n0 + li;
  const bool n_ok = n < N;
  const bool m_ok = li < M;
  const int nchunks = static_cast<int>((K + 127) / 128);
  const uint8_t* crow = codes + n * (K / 2);
  const uint16_t* xrow = X + (int64_t)li * K;
  const int64_t brow = n * (K / kBlock);

  // Chunks of this wave: c = wave + 4t.  Loads are issued a batch of DB
  // chunks at a time, one batch ahead of the batch being multiplied, so each
  // wave keeps 2 x DB 16-byte code loads (and their X fragments) in flight.
  constexpr int DB = 4;
  const int nmine = nchunks > wave ? (nchunks - wave + 3) / 4 : 0;
  u32x4 cw[2][DB];
  uint32_t ce[2][DB];
  float cd[2][DB];
  u32x4 xv[2][DB][4];
  auto load_batch = [&](int t0, int st) {
#pragma unroll
    for (int u = 0; u < DB; ++u) {
      const int t = t0 + u;
      const int64_t k0 = (int64_t)(wave + 4 * t) * 128 + 32 * g;
      const bool ok = t < nmine && k0 < K;
      cw[st][u] = u32x4{0, 0, 0, 0};
      ce[st][u] = 0;
      cd[st][u] = 0.f;
      if (n_ok && ok) {
        const int64_t blk = brow + k0 / kBlock;
        cw[st][u] = *reinterpret_cast<const u32x4*>(crow + k0 / 2);
        ce[st][u] = absmax_q[blk];
        cd[st][u] = absmax_scale[blk >> 8];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xv[st][u][i] = (m_ok && ok) ? *reinterpret_cast<const u32x4*>(xrow + k0 + 8 * i)
                                    : u32x4{0, 0, 0, 0};
    }
  };
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto mul_batch = [&](int st) {
#pragma unroll
    for (int u = 0; u < DB; ++u) {
      const float chat = static_cast<float>(ce[st][u]) * cd[st][u];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = mfma16(dequant8(cw[st][u][i], chat, tab), xv[st][u][i], acc);
    }
  };
  if (nmine > 0) load_batch(0, 0);
  for (int t0 = 0; t0 < nmine; t0 += 2 * DB) {
    if (t0 + DB < nmine) load_batch(t0 + DB, 1);
    mul_batch(0);
    if (t0 + DB >= nmine) break;
    if (t0 + 2 * DB < nmine) load_batch(t0 + 2 * DB, 0);
    mul_batch(1);
  }

  if (wave == 0 && r > 0) {
    // LoRA update: P[n, j] = B[j, n], Q[m, j] = s * T[m, j] (hi, then lo).
    for (int pass = 0; pass < 2; ++pass) {
      for (int j0 = 0; j0 < r; j0 += 32) {
        const int j = j0 + 8 * g;
        const bool j_ok = j < r;
        uint32_t bw[4] = {0, 0, 0, 0};
        if (n_ok && j_ok) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t lo = Bl[(int64_t)(j + 2 * i) * N + n];
            const uint32_t hi = Bl[(int64_t)(j + 2 * i + 1) * N + n];
            bw[i] = lo | (hi << 16);
          }
        }
        u32x4 tq = {0, 0, 0, 0};
        if (m_ok && j_ok) {
          const f32x4 t0 = *reinterpret_cast<const f32x4*>(T + (int64_t)li * r + j);
          const f32x4 t1 = *reinterpret_cast<const f32x4*>(T + (int64_t)li * r + j + 4);
          const float v[8] = {t0.x * s, t0.y * s, t0.z * s, t0.w * s,
                              t1.x * s, t1.y * s, t1.z * s, t1.w * s};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            uint32_t h, l;
            split_bf16x2(v[2 * i], v[2 * i + 1], h, l);
            tq[i] = pass ? l : h;
          }
        }
        acc = mfma16(u32x4{bw[0], bw[1], bw[2], bw[3]}, tq, acc);
      }
    }
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
                             const float* T, const uint16_t* B, int r, float s,
                             uint16_t* Y, const Nf4Tables& tb, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>((w.N + kDecRows - 1) / kDecRows);
  prof_begin(2, stream);
  hipLaunchKernelGGL(k_fwd_decode, dim3(grid), dim3(256), 0, stream, X, (int)M, w.codes,
                     w.absmax_q, w.absmax_scale, w.N, w.K, T, B, r, s, Y, tb);
  prof_end(2, stream);
  return hipGetLastError();
}

}  // namespace qnf4
