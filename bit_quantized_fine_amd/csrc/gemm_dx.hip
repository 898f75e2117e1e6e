// Backward dX = dY . deq(W) + s . G . A^T on bf16 MFMA (list item (4) of
// "DL0087 QLoRA: 4-bit Quantized LoRA": gradients pass through the frozen
// 4-bit weights; the backward pass dequantizes again), with the dequantized
// weight tile staged in LDS.
//
// Here the reduction runs over the weight's rows n while its 64-blocks run
// along k, so the weight enters the MFMA "transposed".  Workgroup = 8 waves,
// tile = 128 output columns (k) x 256 tokens (m), reduction in chunks of 64
// rows n.  Every chunk the 512 threads dequantize the tile's 64 x 128
// weights once -- thread t takes 16 codes of row t/8 -- into one of two LDS
// buffers in their natural row-major order, and the waves read their A
// fragments (16 columns k x 32 rows n) with ds_read_b64_tr_b16, which
// transposes 4 x 16 blocks of 16-bit elements across each group of 16 lanes.
// dY is staged through LDS by coalesced loads.  Wave w owns tokens
// 64 (w % 4) .. +63, all 128 columns, and the 32-row half (w / 4) of every
// chunk; the two halves' accumulators are added through LDS at the end.
//
// LDS layouts: a weight row n holds its 128 k as sixteen 16-byte pieces,
// piece p at slot p ^ ((n % 2) ^ 2 (n % 4) ^ 8 ((n / 8) % 2)): the rows a
// transposing read touches use distinct 32-byte slot pairs, and the two rows
// of a 16-lane dequantizing store use opposite slot parities.  A dY token row
// holds its 64 n as eight pieces, piece q at slot q ^ ((m / 2) % 8).
//
// The LoRA term s . G . A^T is appended as extra reduction steps over the
// rank: A^T fragments come straight from A [K, r], s.G enters as bf16 hi and
// lo halves.
//
// kFormDense instantiates the same kernel over a bf16 weight [N, K] (the 16-bit
// LoRA baseline): each thread loads its 16 weights of row t/8 (32 bytes) and
// stores them where the dequantized values would go.  kFormNoDq reads one
// fp32 constant per block (codes without double quantization).
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace qnf4 {

namespace {

constexpr int XP = 128;          // output columns k per workgroup
constexpr int XQ = 256;          // tokens per workgroup
constexpr int XN = 64;           // weight rows n per chunk
constexpr int XWT = 4;           // token groups
constexpr int XKS = 2;           // waves splitting a chunk's two 32-n steps
constexpr int XW = XWT * XKS;    // waves
constexpr int XT = 64 * XW;      // threads
constexpr int XAS = XP;          // LDS row stride of the weight tile (256 B, swizzled)
constexpr int XYS = XN;          // LDS row stride of the dY tile (128 B, swizzled)
constexpr int XTA = XP / 16;     // 16-column subtiles (8)
constexpr int XTB = XQ / XWT / 16;   // 16-token subtiles per wave (4)
constexpr int kXA = XN * XAS;    // elements of one weight tile buffer
constexpr int kXY = XQ * XYS;    // elements of one dY tile buffer
constexpr int kDxLds = kRepTabBytes + 2 * kXA * 2 + 2 * kXY * 2;
constexpr int XYPT = XQ * XN / 8 / XT;   // 16-byte dY pieces a thread stages per chunk (4)

__device__ __forceinline__ int xcd_remap_dx(int b, int total) {
  const int n8 = total >> 3, rem = total & 7;
  const int x = b & 7, i = b >> 3;
  return x * n8 + min(x, rem) + i;
}

// Slot of 16-byte piece p of weight-tile row n.
__device__ __forceinline__ int wslot(int n, int p) {
  return p ^ ((n & 1) ^ (2 * (n & 3)) ^ (8 * ((n >> 3) & 1)));
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 LdsV4i16;

}  // namespace

template <int kForm>
__global__ __launch_bounds__(XT) void k_dx_gemm(
    const uint16_t* __restrict__ dY, int64_t M, const uint16_t* __restrict__ Wd,
    const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ absmax_q, const float* __restrict__ absmax_scale,
    int64_t N, int64_t K, const float* __restrict__ G, const uint16_t* __restrict__ Al,
    int r, float s, uint16_t* __restrict__ dX, int ptiles, int qtiles, int cps,
    float* __restrict__ part, Nf4Tables tb) {
  // Dynamic LDS only (the level table sits at address 0): the replicated
  // table, two weight tiles, two dY tiles; the table's bytes hold the
  // accumulator exchange after the main loop.
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  char* tab = reinterpret_cast<char*>(dyn);
  uint16_t* Ws = reinterpret_cast<uint16_t*>(dyn + kRepTabBytes);   // [2][XN][XAS]
  uint16_t* Ys = Ws + 2 * kXA;                                       // [2][XQ][XYS]

  const int tid = threadIdx.x;
  const int wave = wave_id(), lane = tid & 63;
  const int li = lane & 15, g = lane >> 4;
  const int wt = wave % XWT, ks = wave / XWT;
  if constexpr (kForm != kFormDense) build_rep_pair_table<XT>(tab, load_levels(tb), tid);

  // With a split reduction (few tiles), workgroup b takes row chunks
  // [z cps, (z + 1) cps) of its tile and writes fp32 partial sums.
  const int ntiles = ptiles * qtiles;
  const int lin = xcd_remap_dx(blockIdx.x, static_cast<int>(gridDim.x));
  const int z = lin / ntiles, tile = lin - z * ntiles;
  const int qt = tile / ptiles, pt = tile - qt * ptiles;
  const int64_t k0 = (int64_t)pt * XP, q0 = (int64_t)qt * XQ;
  const int c0 = z * cps;
  // end of this split's row chunks
  const int nchunks = min(static_cast<int>((N + XN - 1) / XN), c0 + cps);
  const int KB = static_cast<int>(K / kBlock);

  // Buffer descriptors: rows n >= N and tokens m >= M read as zero.
  const uint32_t nb = static_cast<uint32_t>(N * K / kBlock);
  const BufRes rc = make_bufres(codes, static_cast<uint32_t>(N * K / 2));
  const BufRes re = make_bufres(absmax_q, nb);
  // second-level scales, or one fp32 constant per block (kFormNoDq)
  const BufRes rd = make_bufres(
      absmax_scale, (kForm == kFormNoDq ? nb : (nb + kGroup - 1) / kGroup) * 4u);
  // the bf16 weight (kFormDense; N K 2 < 2^31 bytes)
  const BufRes rw = make_bufres(Wd, static_cast<uint32_t>(kForm == kFormDense ? N * K * 2 : 0));
  // dY is addressed from the tile's first token (its 256 rows span less
  // than 2^31 bytes for N <= 2^22).  (A plain conditional, not min(): the
  // 64-bit min is opaque to the compiler's uniformity analysis and would put
  // the descriptor in vector registers.)
  const int64_t tile_rows = M - q0 < XQ ? M - q0 : XQ;
  const BufRes ry = make_bufres(dY + q0 * N, static_cast<uint32_t>(tile_rows * N * 2));

  // Dequantization role: row dr of the chunk, columns k0 + 16 dp .. +15.
  // Columns past K (a half tile when K % 128 == 64) get a zero constant.
  const int dr = tid >> 3, dp = tid & 7;
  const bool dkok = k0 + 16 * dp < K;
  const uint32_t dcode = static_cast<uint32_t>(dr * (K / 2) + k0 / 2 + 8 * dp);   // + c 64 K/2
  const uint32_t dblk = static_cast<uint32_t>(dr * KB + (k0 + 16 * dp) / kBlock);   // + c 64 KB
  // kFormDense: the same 16 weights as bf16, byte offset (+ c 64 K 2)
  const uint32_t dw = static_cast<uint32_t>((dr * K + k0 + 16 * dp) * 2);
  u32x2 cw[2];
  uint32_t ce[2];
  float cd[2];
  u32x4 ww[2][2];
  auto load_codes = [&](int c, int st) {
    const bool live = c < nchunks && dkok;
    if constexpr (kForm == kFormDense) {
      const uint32_t o = dw + static_cast<uint32_t>(c * XN) * static_cast<uint32_t>(K * 2);
      ww[st][0] = buf_load16(rw, live ? o : 0x80000000u);
      ww[st][1] = buf_load16(rw, live ? o + 16u : 0x80000000u);
    } else {
      const uint32_t blk = dblk + static_cast<uint32_t>(c * XN * KB);
      cw[st] = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                     rc, live ? dcode + static_cast<uint32_t>(c * XN) * static_cast<uint32_t>(K / 2)
                              : 0x80000000u, 0, 0));
      if constexpr (kForm == kFormNoDq) {   // e = 1, d = the block's absmax
        ce[st] = 1u;
        cd[st] = buf_load_f32(rd, live ? blk * 4u : 0x80000000u);
      } else {
        ce[st] = buf_load_u8(re, live ? blk : 0x80000000u);
        cd[st] = buf_load_f32(rd, live ? (blk / kGroup) * 4u : 0x80000000u);
      }
    }
  };
  uint32_t ta[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) ta[b] = rep_lane_base(lane);
  auto dequant = [&](int st, int buf) {
    uint16_t* dst = Ws + buf * kXA + dr * XAS;
    if constexpr (kForm == kFormDense) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        *reinterpret_cast<u32x4*>(dst + 8 * wslot(dr, 2 * dp + i)) = ww[st][i];
      return;
    }
    const float chat = static_cast<float>(ce[st]) * cd[st];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t w = cw[st][i];
      const f32x2 v0 = rep_lookup<0>(ta[0], w);
      const f32x2 v1 = rep_lookup<1>(ta[1], w);
      const f32x2 v2 = rep_lookup<2>(ta[2], w);
      const f32x2 v3 = rep_lookup<3>(ta[3], w);
      *reinterpret_cast<u32x4*>(dst + 8 * wslot(dr, 2 * dp + i)) =
          u32x4{pack_bf16x2(v0.x * chat, v0.y * chat), pack_bf16x2(v1.x * chat, v1.y * chat),
                pack_bf16x2(v2.x * chat, v2.y * chat), pack_bf16x2(v3.x * chat, v3.y * chat)};
    }
  };

  // dY staging role: piece j of thread tid is token row yr + 64 j (yr = tid / 8)
  // of the tile, 16-byte piece tid % 8 of its 128-byte chunk row.
  const int yr = tid >> 3, yq = tid & 7;
  const uint32_t ysrc = static_cast<uint32_t>((yr * N + 8 * yq) * 2);   // + 128 c
  u32x4 yw[2][XYPT];
  auto load_y = [&](int c, int st) {
    const bool live = c < nchunks && c * XN + 8 * yq < N;
#pragma unroll
    for (int j = 0; j < XYPT; ++j)
      yw[st][j] = buf_load16(
          ry, live ? ysrc + static_cast<uint32_t>((64 * j * N + c * XN) * 2) : 0x80000000u);
  };
  auto store_y = [&](int st, int buf) {
#pragma unroll
    for (int j = 0; j < XYPT; ++j) {
      const int row = yr + 64 * j;
      *reinterpret_cast<u32x4*>(Ys + buf * kXY + row * XYS + 8 * (yq ^ ((row >> 1) & 7))) =
          yw[st][j];
    }
  };

  f32x4 acc[XTA][XTB];
#pragma unroll
  for (int a = 0; a < XTA; ++a)
#pragma unroll
    for (int b = 0; b < XTB; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A fragment (columns 16 a + li, rows 32 ks + 8 g .. +7): two transposing
  // reads of rows nb4 + t/4, columns 16 a + 4 (t % 4) (t = li).
  // Operands of one 32-n step are read into registers first; the MFMAs then
  // touch no memory, so the compiler can interleave them with the staging
  // work of the next chunk.
  u32x4 af[XTA], bf[XTB];
  // Transposing-read address of rows 32 ks + 8 g + 4 e + li / 4, columns
  // 16 a + 4 (li % 4): rbase[e] + 16 (a ^ rsw[e]) + ... in elements, where
  // rsw[e] is the row's XOR on the 16-column group.
  int rbase[2], rsw[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int n = 32 * ks + 8 * g + 4 * e + (li >> 2);
    const int x = (n & 1) ^ (2 * (n & 3)) ^ (8 * ((n >> 3) & 1));   // slot XOR
    rbase[e] = n * XAS + 8 * (((li & 3) >> 1) ^ (x & 1)) + 4 * (li & 1);
    rsw[e] = x >> 1;
  }
  auto read_frags = [&](int buf) {
    const uint16_t* yt = Ys + buf * kXY + (64 * wt + li) * XYS + 8 * ((g + 4 * ks) ^ (li >> 1));
#pragma unroll
    for (int b = 0; b < XTB; ++b) bf[b] = *reinterpret_cast<const u32x4*>(yt + 16 * b * XYS);
    const uint16_t* wt0 = Ws + buf * kXA;
    // Recomputing the 16 addresses each chunk (one VALU op each) is cheaper
    // than holding them in registers across the loop.
    int sw[2] = {rsw[0], rsw[1]};
    asm volatile("" : "+v"(sw[0]), "+v"(sw[1]));
#pragma unroll
    for (int a = 0; a < XTA; ++a) {
      v4i16 h[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint16_t* src = wt0 + rbase[e] + 16 * (a ^ sw[e]);
        h[e] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LdsV4i16*)(src));
      }
      const u32x2 h0 = __builtin_bit_cast(u32x2, h[0]), h1 = __builtin_bit_cast(u32x2, h[1]);
      af[a] = u32x4{h0[0], h0[1], h1[0], h1[1]};
    }
  };
  auto mma = [&]() {
#pragma unroll
    for (int a = 0; a < XTA; ++a)
#pragma unroll
      for (int b = 0; b < XTB; ++b) acc[a][b] = mfma16(af[a], bf[b], acc[a][b]);
  };

  load_codes(c0, 0);
  load_codes(c0 + 1, 1);
  load_y(c0, 0);
  load_y(c0 + 1, 1);
  __syncthreads();   // level table
  dequant(0, 0);
  store_y(0, 0);
  load_codes(c0 + 2, 0);
  load_y(c0 + 2, 0);
  __syncthreads();
  // iteration c: read the operands of chunk c from buffers c&1; stage chunk
  // c+1 into buffers (c+1)&1 -- dequantize its codes and store its dY, both
  // loaded two iterations ago -- and refill those register stages with chunk
  // c+3; multiply chunk c.
  auto iter = [&](int c, auto stc) {
    constexpr int ST = decltype(stc)::value;
    read_frags(ST);
    dequant(ST ^ 1, ST ^ 1);
    store_y(ST ^ 1, ST ^ 1);
    load_codes(c + 3, ST ^ 1);
    load_y(c + 3, ST ^ 1);
    mma();
    __syncthreads();
  };
  // Iterations run in pairs with no exit between them, so the compiler's
  // load counting sees one path and waits only for the stage it consumes.
  // An odd chunk count adds one pass over a chunk past the end, whose codes,
  // constants and activations all read as zero: it adds zeros.
  for (int c = c0; c < nchunks; c += 2) {
    iter(c, std::integral_constant<int, 0>{});
    iter(c + 1, std::integral_constant<int, 1>{});
  }

  // LoRA term (the first split only): extra steps over the rank, 32 at a
  // time, alternating between the two halves before their accumulators are
  // added.
  for (int j0 = 32 * ks; z == 0 && j0 < r; j0 += 64) {
    const int j = j0 + 8 * g;
    u32x4 gh[XTB], gl[XTB];
#pragma unroll
    for (int b = 0; b < XTB; ++b) {
      const int64_t m = q0 + 64 * wt + 16 * b + li;
      uint32_t hi[4] = {0, 0, 0, 0}, lo[4] = {0, 0, 0, 0};
      if (m < M && j < r) {
        const f32x4 t0 = *reinterpret_cast<const f32x4*>(G + m * r + j);
        const f32x4 t1 = *reinterpret_cast<const f32x4*>(G + m * r + j + 4);
        const float v[8] = {t0.x * s, t0.y * s, t0.z * s, t0.w * s,
                            t1.x * s, t1.y * s, t1.z * s, t1.w * s};
#pragma unroll
        for (int e = 0; e < 4; ++e) split_bf16x2(v[2 * e], v[2 * e + 1], hi[e], lo[e]);
      }
      gh[b] = u32x4{hi[0], hi[1], hi[2], hi[3]};
      gl[b] = u32x4{lo[0], lo[1], lo[2], lo[3]};
    }
#pragma unroll
    for (int a = 0; a < XTA; ++a) {
      const int64_t k = k0 + 16 * a + li;
      const u32x4 af = (k < K && j < r) ? *reinterpret_cast<const u32x4*>(Al + k * r + j)
                                        : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int b = 0; b < XTB; ++b) {
        acc[a][b] = mfma16(af, gh[b], acc[a][b]);
        acc[a][b] = mfma16(af, gl[b], acc[a][b]);
      }
    }
  }

  // Add the second n half into the first through LDS, half of the column
  // subtiles at a time.
  f32x4* xch = reinterpret_cast<f32x4*>(dyn);   // [XWT][XTA/2][XTB][64]
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (ks == 1) {
#pragma unroll
      for (int a = 0; a < XTA / 2; ++a)
#pragma unroll
        for (int b = 0; b < XTB; ++b)
          xch[((wt * (XTA / 2) + a) * XTB + b) * 64 + lane] = acc[h * (XTA / 2) + a][b];
    }
    __syncthreads();
    if (ks == 0) {
#pragma unroll
      for (int a = 0; a < XTA / 2; ++a)
#pragma unroll
        for (int b = 0; b < XTB; ++b)
          acc[h * (XTA / 2) + a][b] += xch[((wt * (XTA / 2) + a) * XTB + b) * 64 + lane];
    }
    __syncthreads();
  }
  if (ks != 0) return;

  // dX[m, k..k+3] for the lane's 4 consecutive columns k of each subtile
  // (bf16), or this split's fp32 partial sums part[z][m][k..k+3]
#pragma unroll
  for (int a = 0; a < XTA; ++a) {
    const int64_t k = k0 + 16 * a + 4 * g;
#pragma unroll
    for (int b = 0; b < XTB; ++b) {
      const int64_t m = q0 + 64 * wt + 16 * b + li;
      if (m < M && k < K) {
        const f32x4 v = acc[a][b];
        if (part) {
          *reinterpret_cast<f32x4*>(part + ((int64_t)z * M + m) * K + k) = v;
        } else {
          *reinterpret_cast<u32x2*>(dX + m * K + k) =
              u32x2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
        }
      }
    }
  }
}

GemmSplit dx_gemm_split(int64_t M, int64_t N, int64_t K) {
  return gemm_split((K + XP - 1) / XP * ((M + XQ - 1) / XQ), (N + XN - 1) / XN);
}

hipError_t launch_dx_gemm(const uint16_t* dY, int64_t M, const Nf4View& w,
                          const float* G, const uint16_t* A, int r, float s,
                          uint16_t* dX, float* part, const Nf4Tables& tb, hipStream_t stream) {
  static const hipError_t attr[3] = {
      hipFuncSetAttribute(reinterpret_cast<const void*>(&k_dx_gemm<kFormDq>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kDxLds),
      hipFuncSetAttribute(reinterpret_cast<const void*>(&k_dx_gemm<kFormNoDq>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kDxLds),
      hipFuncSetAttribute(reinterpret_cast<const void*>(&k_dx_gemm<kFormDense>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kDxLds)};
  const int form = w.dense ? kFormDense : (w.dq ? kFormDq : kFormNoDq);
  if (attr[form] != hipSuccess) return attr[form];
  decltype(&k_dx_gemm<kFormDq>) kern =
      form == kFormDense ? k_dx_gemm<kFormDense> : (form == kFormNoDq ? k_dx_gemm<kFormNoDq> : k_dx_gemm<kFormDq>);
  const int ptiles = static_cast<int>((w.K + XP - 1) / XP);
  const int qtiles = static_cast<int>((M + XQ - 1) / XQ);
  const GemmSplit sp = dx_gemm_split(M, w.N, w.K);
  if (sp.splits > 1 && !part) return hipErrorInvalidValue;
  prof_begin(1, stream);
  hipLaunchKernelGGL(kern,
                     dim3(ptiles * qtiles * sp.splits), dim3(XT), kDxLds, stream, dY, M, w.dense,
                     w.codes, w.absmax_q, w.absmax_scale, w.N, w.K, G, A, r, s, dX, ptiles,
                     qtiles, sp.cps, sp.splits > 1 ? part : nullptr, tb);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && sp.splits > 1)
    e = launch_split_reduce_bf16(part, sp.splits, M * w.K, dX, stream);
  prof_end(1, stream);
  return e;
}

}  // namespace qnf4
