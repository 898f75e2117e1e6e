// Backward dX = dY . deq(W) + s . G . A^T on bf16 MFMA (list item (4) of
// "DL0087 QLoRA: 4-bit Quantized LoRA": gradients pass through the frozen
// 4-bit weights; the backward pass dequantizes again).
//
// Here the reduction runs over the weight's rows n while its 64-blocks run
// along k, so the dequantized weight is needed "transposed".  Workgroup tile:
// 256 output columns k x 128 tokens; 8 waves each own 32 consecutive k.  In
// one 32-n MFMA step, lane (rho = l % 16, g = l / 16) loads one code byte --
// the two codes of columns k = kw + 2 rho + {0, 1} -- from each of the 8 rows
// n = n0 + 8g + t, t = 0..7, and dequantizes them into the A operands of two
// 16-row MFMA subtiles (subtile e holds column kw + 2 rho + e in row rho):
// the 8 values along n for a fixed k are exactly one A fragment.  The
// dequantized weight never leaves registers.  dY is shared through LDS; the
// block constants of a chunk (one per row n and 64-column block) are
// multiplied out once per workgroup into LDS.
//
// Output: lane l of a wave ends with columns kw + 8(l/16) .. +7 of token
// (l % 16) of each 16-token subtile, i.e. one contiguous 16-byte store.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace qnf4 {

namespace {

constexpr int DP = 256;          // output columns k per workgroup
constexpr int DQ = 128;          // tokens per workgroup
constexpr int DN = 64;           // reduction (n) per chunk (two 32-n MFMA steps)
constexpr int DNW = 8;           // waves
constexpr int DRW = DP / DNW;    // k per wave (32)
constexpr int DT = 256 * 2;      // threads
constexpr int YS = 128 + 8;      // LDS row stride of the dY tile (also the LoRA tile)
constexpr int CB = DP / kBlock;  // 64-column blocks per tile (4)

__device__ __forceinline__ int xcd_remap_dx(int b, int total) {
  const int n8 = total >> 3, rem = total & 7;
  const int x = b & 7, i = b >> 3;
  return x * n8 + min(x, rem) + i;
}

}  // namespace

__global__ __launch_bounds__(DT) void k_dx_gemm2(
    const uint16_t* __restrict__ dY, int64_t M, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ absmax_q, const float* __restrict__ absmax_scale,
    int64_t N, int64_t K, const float* __restrict__ G, const uint16_t* __restrict__ Al,
    int r, float s, uint16_t* __restrict__ dX, int ptiles, int qtiles, Nf4Tables tb) {
  constexpr int TB = DQ / 16;                 // token subtiles
  constexpr int YCH = DQ * DN / 8 / DT;       // 16-byte dY chunks per thread per chunk (2)
  __shared__ __attribute__((aligned(16))) uint16_t ys[2][DQ * YS];   // dY uses 64 of 136 columns
  __shared__ __attribute__((aligned(16))) float cs[2][CB * DN];   // block constants [blk][n]
  __shared__ float2 tab[256];

  const int tid = threadIdx.x;
  const int wave = wave_id(), lane = tid & 63;
  const int li = lane & 15, g = lane >> 4;
  build_pair_table(tab, tb, tid, DT);

  const int tile = xcd_remap_dx(blockIdx.x, ptiles * qtiles);
  const int qt = tile / ptiles, pt = tile - qt * ptiles;
  const int64_t p0 = (int64_t)pt * DP, q0 = (int64_t)qt * DQ;
  const int nchunks = static_cast<int>((N + DN - 1) / DN);
  const int64_t kw = p0 + wave * DRW;                 // this wave's first column
  const int wblk = (wave * DRW) / kBlock;             // its block within the tile

  const uint32_t rowb = static_cast<uint32_t>(K / 2);
  const BufRes rc = make_bufres(codes, static_cast<uint32_t>(N * K / 2));
  // byte of columns kw + 2 li, kw + 2 li + 1 in row 0; rows add rowb each.
  // Columns past K (possible only in the last tile) get a zero block
  // constant below, so the bytes read there do not matter.
  const uint32_t cbase = static_cast<uint32_t>(kw / 2) + li;

  f32x4 acc[2][TB];
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int b = 0; b < TB; ++b) acc[e][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- staging of dY (registers, two chunks deep) and block constants ----
  u32x4 yr[2][YCH];
  uint32_t ce[2];    // each thread: one (block, row) constant per chunk
  float cd[2];
  auto load_y = [&](int c, int st) {
#pragma unroll
    for (int j = 0; j < YCH; ++j) {
      const int idx = tid + j * DT;
      const int row = idx >> 3, col = idx & 7;
      const int64_t m = q0 + row, n = (int64_t)c * DN + col * 8;
      yr[st][j] = (m < M && n < N) ? *reinterpret_cast<const u32x4*>(dY + m * N + n)
                                   : u32x4{0, 0, 0, 0};
    }
    // constants: thread t < 256 -> block t / 64 of the tile, row n0 + t % 64
    const int cb = (tid >> 6) & 3, cr = tid & 63;
    const int64_t n = (int64_t)c * DN + cr;
    const int64_t kb = (p0 / kBlock) + cb;
    if (n < N && kb * kBlock < K) {
      const int64_t blk = n * (K / kBlock) + kb;
      ce[st] = absmax_q[blk];
      cd[st] = absmax_scale[blk >> 8];
    } else {
      ce[st] = 0;
      cd[st] = 0.f;
    }
  };
  auto store_y = [&](int buf, int st) {
#pragma unroll
    for (int j = 0; j < YCH; ++j) {
      const int idx = tid + j * DT;
      *reinterpret_cast<u32x4*>(&ys[buf][(idx >> 3) * YS + (idx & 7) * 8]) = yr[st][j];
    }
    if (tid < CB * DN) cs[buf][tid] = static_cast<float>(ce[st]) * cd[st];   // fl32(e * d)
  };

  // ---- code bytes of one chunk: 2 steps x 8 rows, one byte each ----
  uint32_t cb8[2][2][8];
  auto load_codes = [&](int c, int st) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t row = static_cast<uint32_t>(c * DN + 32 * i + 8 * g + t);
        cb8[st][i][t] = buf_load_u8(rc, cbase + row * rowb);
      }
  };

  // dY and its constants are staged two chunks ahead, the code bytes one
  // chunk ahead (each in stage c & 1).
  load_y(0, 0);
  load_codes(0, 0);
  if (nchunks > 1) load_y(1, 1);
  __syncthreads();   // pair table
  store_y(0, 0);
  __syncthreads();

  auto step = [&](int c, auto stc) {
    constexpr int ST = decltype(stc)::value;
    if (c + 1 < nchunks) load_codes(c + 1, ST ^ 1);
    if (c + 2 < nchunks) load_y(c + 2, ST);
    const auto& cur = cb8[ST];
    const uint16_t* yt = ys[ST];
    const float* ct = cs[ST] + wblk * DN;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      // block constants of rows n0 + 32i + 8g + t, t = 0..7
      const f32x4 c0 = *reinterpret_cast<const f32x4*>(ct + 32 * i + 8 * g);
      const f32x4 c1 = *reinterpret_cast<const f32x4*>(ct + 32 * i + 8 * g + 4);
      const float chat[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      float v[8][2];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float2 q = tab[cur[i][t] & 0xFFu];
        v[t][0] = q.x * chat[t];
        v[t][1] = q.y * chat[t];
      }
      u32x4 A[2];
#pragma unroll
      for (int e = 0; e < 2; ++e)
        A[e] = u32x4{pack_bf16x2(v[0][e], v[1][e]), pack_bf16x2(v[2][e], v[3][e]),
                     pack_bf16x2(v[4][e], v[5][e]), pack_bf16x2(v[6][e], v[7][e])};
#pragma unroll
      for (int b = 0; b < TB; ++b) {
        const u32x4 Bf = *reinterpret_cast<const u32x4*>(yt + (16 * b + li) * YS + 32 * i + 8 * g);
        acc[0][b] = mfma16(A[0], Bf, acc[0][b]);
        acc[1][b] = mfma16(A[1], Bf, acc[1][b]);
      }
    }
    if (c + 1 < nchunks) store_y(ST ^ 1, ST ^ 1);
    __syncthreads();
  };
  for (int c = 0; c < nchunks; c += 2) {
    step(c, std::integral_constant<int, 0>{});
    if (c + 1 < nchunks) step(c + 1, std::integral_constant<int, 1>{});
  }

  // ---- LoRA term s . G . A^T: extra chunks over the rank.  Columns 0..63
  // of the staged tile carry bf16(s.G) (hi), 64..127 the remainder (lo); the
  // A operand row of subtile e, lane rho is A[kw + 2 rho + e][j .. j + 7]. ----
  if (r > 0) {
    uint16_t* gt = ys[0];
    for (int j0 = 0; j0 < r; j0 += 64) {
      for (int idx = tid; idx < DQ * 8; idx += DT) {
        const int row = idx >> 3, col = idx & 7;
        const int64_t m = q0 + row;
        const int j = j0 + col * 8;
        uint32_t hi[4] = {0, 0, 0, 0}, lo[4] = {0, 0, 0, 0};
        if (m < M && j < r) {
          const f32x4 t0 = *reinterpret_cast<const f32x4*>(G + m * r + j);
          const f32x4 t1 = *reinterpret_cast<const f32x4*>(G + m * r + j + 4);
          const float vv[8] = {t0.x * s, t0.y * s, t0.z * s, t0.w * s,
                               t1.x * s, t1.y * s, t1.z * s, t1.w * s};
#pragma unroll
          for (int e = 0; e < 4; ++e) split_bf16x2(vv[2 * e], vv[2 * e + 1], hi[e], lo[e]);
        }
        *reinterpret_cast<u32x4*>(gt + row * YS + col * 8) = u32x4{hi[0], hi[1], hi[2], hi[3]};
        *reinterpret_cast<u32x4*>(gt + row * YS + 64 + col * 8) =
            u32x4{lo[0], lo[1], lo[2], lo[3]};
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = 32 * i + 8 * g;           // column of the staged tile
        const int j = j0 + (kk & 63);
        u32x4 A[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int64_t k = kw + 2 * li + e;
          A[e] = (k < K && j < r) ? *reinterpret_cast<const u32x4*>(Al + k * r + j)
                                  : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int b = 0; b < TB; ++b) {
          const u32x4 Bf = *reinterpret_cast<const u32x4*>(gt + (16 * b + li) * YS + kk);
          acc[0][b] = mfma16(A[0], Bf, acc[0][b]);
          acc[1][b] = mfma16(A[1], Bf, acc[1][b]);
        }
      }
      __syncthreads();
    }
  }

  // ---- store: lane holds columns kw + 8g + 2 rr + e (rr = 0..3, e = 0..1) ----
  const int64_t k8 = kw + 8 * g;
#pragma unroll
  for (int b = 0; b < TB; ++b) {
    const int64_t m = q0 + 16 * b + li;
    if (m < M && k8 < K) {
      const f32x4 a0 = acc[0][b], a1 = acc[1][b];
      *reinterpret_cast<u32x4*>(dX + m * K + k8) =
          u32x4{pack_bf16x2(a0.x, a1.x), pack_bf16x2(a0.y, a1.y), pack_bf16x2(a0.z, a1.z),
                pack_bf16x2(a0.w, a1.w)};
    }
  }
}

hipError_t launch_dx_gemm(const uint16_t* dY, int64_t M, const Nf4View& w,
                          const float* G, const uint16_t* A, int r, float s,
                          uint16_t* dX, const Nf4Tables& tb, hipStream_t stream) {
  const int ptiles = static_cast<int>((w.K + DP - 1) / DP);
  const int qtiles = static_cast<int>((M + DQ - 1) / DQ);
  prof_begin(1, stream);
  hipLaunchKernelGGL(k_dx_gemm2, dim3(ptiles * qtiles), dim3(DT), 0, stream, dY, M, w.codes,
                     w.absmax_q, w.absmax_scale, w.N, w.K, G, A, r, s, dX, ptiles, qtiles, tb);
  prof_end(1, stream);
  return hipGetLastError();
}

}  // namespace qnf4
