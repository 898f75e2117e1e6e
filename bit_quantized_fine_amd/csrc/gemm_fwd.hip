// Forward for many tokens: Y = X . deq(W)^T + s . T . B on bf16 MFMA.
//
// Workgroup tile: 256 weight rows (n) x 128 tokens (m), reduction in chunks
// of 128 k.  The token tile of X is shared through LDS; the weight rows are
// split between the waves (each wave owns 256/NW consecutive rows), so each
// NF4 code is loaded and dequantized exactly once per workgroup, straight
// from a 16-byte global load into the A-operand registers of
// v_mfma_f32_16x16x32_bf16 (the bf16 tile of the Mathematical Formulation
// of "DL0087 QLoRA" lives only in registers).
//
// Reduction order inside a chunk: lane group g = lane/16 of a wave holds the
// 32 codes k0+32g .. k0+32g+31 of its row (one 16-byte load); MFMA step i
// consumes k0 + 32g + 8i + (0..7) from every lane group.  The X fragment is
// read from LDS with the same k mapping, so the sum is over every k once.
//
// The LoRA update is appended as extra reduction chunks over the rank:
// columns 0..63 of such a chunk carry bf16(s.T) (hi part), columns 64..127
// the bf16 remainder (lo part), both against B^T staged through LDS.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace qnf4 {

namespace {

constexpr int FP = 256;          // weight rows per workgroup
constexpr int FQ = 128;          // tokens per workgroup
constexpr int FK = 128;          // reduction elements per chunk
constexpr int XS = FK + 8;       // LDS row stride of the token tile (272 B)
constexpr int BTS = 64 + 8;      // LDS row stride of the B^T tile (144 B)
constexpr int SMEM_ELEMS = 2 * FQ * XS > FP * BTS + FQ * XS ? 2 * FQ * XS : FP * BTS + FQ * XS;

// Tile id of workgroup b when consecutive workgroups go round-robin to the 8
// XCDs: every XCD gets a contiguous run of tile ids, so workgroups sharing a
// token tile (consecutive ids, token-major order) share an L2.
__device__ __forceinline__ int xcd_remap(int b, int total) {
  const int n8 = total >> 3, rem = total & 7;
  const int x = b & 7, i = b >> 3;
  return x * n8 + min(x, rem) + i;
}

}  // namespace

template <int NW>
__global__ __launch_bounds__(64 * NW) void k_fwd_gemm2(
    const uint16_t* __restrict__ X, int64_t M, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ absmax_q, const float* __restrict__ absmax_scale,
    int64_t N, int64_t K, const float* __restrict__ T, const uint16_t* __restrict__ Bl,
    int r, float s, uint16_t* __restrict__ Y, int ptiles, int qtiles, Nf4Tables tb) {
  constexpr int NT_ = 64 * NW;
  constexpr int RW = FP / NW;        // weight rows per wave
  constexpr int TA = RW / 16;        // 16-row subtiles per wave
  constexpr int TB = FQ / 16;        // 16-token subtiles
  constexpr int XCH = FQ * FK / 8 / NT_;   // 16-byte X chunks per thread per chunk
  static_assert(FQ * FK / 8 % NT_ == 0, "X tile split");

  __shared__ __attribute__((aligned(16))) uint16_t smem[SMEM_ELEMS];
  __shared__ float2 tab[256];

  const int tid = threadIdx.x;
  const int wave = wave_id(), lane = tid & 63;
  const int li = lane & 15, g = lane >> 4;
  build_pair_table(tab, tb, tid, NT_);

  const int tile = xcd_remap(blockIdx.x, ptiles * qtiles);
  const int qt = tile / ptiles, pt = tile - qt * ptiles;
  const int64_t p0 = (int64_t)pt * FP, q0 = (int64_t)qt * FQ;
  const int nchunks = static_cast<int>((K + FK - 1) / FK);

  // weight rows of this lane
  const uint8_t* crow[TA];
  int64_t brow[TA];
  bool nok[TA];
#pragma unroll
  for (int a = 0; a < TA; ++a) {
    const int64_t n = p0 + wave * RW + 16 * a + li;
    nok[a] = n < N;
    const int64_t nn = nok[a] ? n : 0;
    crow[a] = codes + nn * (K / 2) + 16 * g;
    brow[a] = nn * (K / kBlock) + (g >> 1);
  }

  f32x4 acc[TA][TB];
#pragma unroll
  for (int a = 0; a < TA; ++a)
#pragma unroll
    for (int b = 0; b < TB; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Register staging, two chunks deep: X(c) and the codes of chunk c live in
  // stage c & 1 from the start of iteration c-2 until they are consumed.
  u32x4 xr[2][XCH];
  u32x4 cw[2][TA];
  uint32_t ce[2][TA];   // 8-bit block constant, as loaded
  float cd[2][TA];      // its fp32 group scale, as loaded

  auto load_x = [&](int c, int st) {
#pragma unroll
    for (int j = 0; j < XCH; ++j) {
      const int idx = tid + j * NT_;
      const int row = idx >> 4, col = idx & 15;
      const int64_t m = q0 + row, k = (int64_t)c * FK + col * 8;
      xr[st][j] = (m < M && k < K) ? *reinterpret_cast<const u32x4*>(X + m * K + k)
                                   : u32x4{0, 0, 0, 0};
    }
  };
  auto store_x = [&](int buf, int st) {
    uint16_t* xs = smem + buf * FQ * XS;
#pragma unroll
    for (int j = 0; j < XCH; ++j) {
      const int idx = tid + j * NT_;
      *reinterpret_cast<u32x4*>(xs + (idx >> 4) * XS + (idx & 15) * 8) = xr[st][j];
    }
  };
  auto load_w = [&](int c, int st) {
    const bool kok = (int64_t)c * FK + 32 * g < K;
#pragma unroll
    for (int a = 0; a < TA; ++a) {
      // The block constant is multiplied out only when the chunk is used,
      // so these loads are not waited for here.
      if (nok[a] && kok) {
        const int64_t blk = brow[a] + 2 * c;
        cw[st][a] = *reinterpret_cast<const u32x4*>(crow[a] + (int64_t)c * (FK / 2));
        ce[st][a] = absmax_q[blk];
        cd[st][a] = absmax_scale[blk >> 8];
      } else {
        cw[st][a] = u32x4{0, 0, 0, 0};
        ce[st][a] = 0;
        cd[st][a] = 0.f;
      }
    }
  };

  load_x(0, 0);
  load_w(0, 0);
  if (nchunks > 1) {
    load_x(1, 1);
    load_w(1, 1);
  }
  __syncthreads();          // pair table ready
  store_x(0, 0);
  __syncthreads();

  // One chunk: take this chunk's codes out of their stage, refill the stage
  // with chunk c+2 (codes and X), multiply chunk c from LDS buffer c & 1,
  // then stage X(c+1) into the other LDS buffer.
  auto step = [&](int c, auto stc) {
    constexpr int ST = decltype(stc)::value;
    u32x4 cur[TA];
    float cch[TA];
#pragma unroll
    for (int a = 0; a < TA; ++a) {
      cur[a] = cw[ST][a];
      cch[a] = static_cast<float>(ce[ST][a]) * cd[ST][a];   // fl32(e * d)
    }
    if (c + 2 < nchunks) {
      load_w(c + 2, ST);
      load_x(c + 2, ST);
    }
    const uint16_t* xs = smem + ST * FQ * XS;
    // Software pipeline over the four 32-k steps: the X fragments and the
    // level-table lookups of step i+1 are issued before the MFMAs of step i.
    u32x4 bf[2][TB];
    float2 lk[2][TA][4];
    auto issue = [&](int i, int sb) {
#pragma unroll
      for (int b = 0; b < TB; ++b)
        bf[sb][b] = *reinterpret_cast<const u32x4*>(xs + (16 * b + li) * XS + (4 * g + i) * 8);
#pragma unroll
      for (int a = 0; a < TA; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) lk[sb][a][q] = tab[(cur[a][i] >> (8 * q)) & 0xFFu];
    };
    issue(0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sb = i & 1;
      if (i < 3) issue(i + 1, sb ^ 1);
      u32x4 A[TA];
#pragma unroll
      for (int a = 0; a < TA; ++a) {
        const float cc = cch[a];
        A[a] = u32x4{pack_bf16x2(lk[sb][a][0].x * cc, lk[sb][a][0].y * cc),
                     pack_bf16x2(lk[sb][a][1].x * cc, lk[sb][a][1].y * cc),
                     pack_bf16x2(lk[sb][a][2].x * cc, lk[sb][a][2].y * cc),
                     pack_bf16x2(lk[sb][a][3].x * cc, lk[sb][a][3].y * cc)};
      }
#pragma unroll
      for (int b = 0; b < TB; ++b)
#pragma unroll
        for (int a = 0; a < TA; ++a) acc[a][b] = mfma16(A[a], bf[sb][b], acc[a][b]);
    }
    if (c + 1 < nchunks) store_x(ST ^ 1, ST ^ 1);
    __syncthreads();
  };
  for (int c = 0; c < nchunks; c += 2) {
    step(c, std::integral_constant<int, 0>{});
    if (c + 1 < nchunks) step(c + 1, std::integral_constant<int, 1>{});
  }

  // LoRA update: extra chunks over the rank, hi and lo halves of s.T.
  if (r > 0) {
    uint16_t* bt = smem;                 // [FP][BTS]: B^T rows n, 64 ranks
    uint16_t* tt = smem + FP * BTS;      // [FQ][XS]: s.T hi (0..63) | lo (64..127)
    for (int j0 = 0; j0 < r; j0 += 64) {
      // B^T tile: 8x8 patches, (FP/8) x 8 of them
      for (int p = tid; p < FP; p += NT_) {
        const int rp = p % (FP / 8), kp = p / (FP / 8);
        const int64_t n = p0 + rp * 8;
        u32x4 rows[8], cols[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int j = j0 + kp * 8 + t;
          rows[t] = (n < N && j < r) ? *reinterpret_cast<const u32x4*>(Bl + (int64_t)j * N + n)
                                     : u32x4{0, 0, 0, 0};
        }
        transpose8x8_b16(rows, cols);
#pragma unroll
        for (int t = 0; t < 8; ++t)
          *reinterpret_cast<u32x4*>(bt + (rp * 8 + t) * BTS + kp * 8) = cols[t];
      }
      // s.T tile split into bf16 hi / lo
      for (int idx = tid; idx < FQ * 8; idx += NT_) {
        const int row = idx >> 3, col = idx & 7;
        const int64_t m = q0 + row;
        const int j = j0 + col * 8;
        uint32_t hi[4] = {0, 0, 0, 0}, lo[4] = {0, 0, 0, 0};
        if (m < M && j < r) {
          const f32x4 t0 = *reinterpret_cast<const f32x4*>(T + m * r + j);
          const f32x4 t1 = *reinterpret_cast<const f32x4*>(T + m * r + j + 4);
          const float v[8] = {t0.x * s, t0.y * s, t0.z * s, t0.w * s,
                              t1.x * s, t1.y * s, t1.z * s, t1.w * s};
#pragma unroll
          for (int e = 0; e < 4; ++e) split_bf16x2(v[2 * e], v[2 * e + 1], hi[e], lo[e]);
        }
        *reinterpret_cast<u32x4*>(tt + row * XS + col * 8) = u32x4{hi[0], hi[1], hi[2], hi[3]};
        *reinterpret_cast<u32x4*>(tt + row * XS + 64 + col * 8) = u32x4{lo[0], lo[1], lo[2], lo[3]};
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = 32 * g + 8 * i;
        u32x4 A[TA];
#pragma unroll
        for (int a = 0; a < TA; ++a)
          A[a] = *reinterpret_cast<const u32x4*>(bt + (wave * RW + 16 * a + li) * BTS + (kk & 63));
#pragma unroll
        for (int b = 0; b < TB; ++b) {
          const u32x4 Bf = *reinterpret_cast<const u32x4*>(tt + (16 * b + li) * XS + kk);
#pragma unroll
          for (int a = 0; a < TA; ++a) acc[a][b] = mfma16(A[a], Bf, acc[a][b]);
        }
      }
      __syncthreads();
    }
  }

  // Y[m, n..n+3] for the lane's 4 consecutive rows n of each subtile
#pragma unroll
  for (int a = 0; a < TA; ++a) {
    const int64_t n = p0 + wave * RW + 16 * a + 4 * g;
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      const int64_t m = q0 + 16 * b + li;
      if (m < M && n < N) {
        const f32x4 v = acc[a][b];
        *reinterpret_cast<u32x2*>(Y + m * N + n) =
            u32x2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
      }
    }
  }
}

hipError_t launch_fwd_gemm(const uint16_t* X, int64_t M, const Nf4View& w,
                           const float* T, const uint16_t* B, int r, float s,
                           uint16_t* Y, const Nf4Tables& tb, hipStream_t stream) {
  constexpr int NW = 8;
  const int ptiles = static_cast<int>((w.N + FP - 1) / FP);
  const int qtiles = static_cast<int>((M + FQ - 1) / FQ);
  prof_begin(0, stream);
  hipLaunchKernelGGL(k_fwd_gemm2<NW>, dim3(ptiles * qtiles), dim3(64 * NW), 0, stream, X, M,
                     w.codes, w.absmax_q, w.absmax_scale, w.N, w.K, T, B, r, s, Y, ptiles,
                     qtiles, tb);
  prof_end(0, stream);
  return hipGetLastError();
}

}  // namespace qnf4
