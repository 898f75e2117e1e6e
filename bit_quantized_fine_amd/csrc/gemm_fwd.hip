// Forward for many tokens: Y = X . deq(W)^T + s . T . B on bf16 MFMA, with the
// dequantized weight tile staged in LDS (Mathematical Formulation and
// Figure 1 of "DL0087 QLoRA": a bf16 tile of W is rebuilt just before the
// matmul and discarded).
//
// Workgroup = 8 waves, tile = 128 weight rows (n) x 256 tokens (m), reduction
// in chunks of 64 k (one NF4 block per row).  Every chunk the 512 threads
// dequantize the tile's 128 x 64 weights once into one of two LDS buffers,
// while the waves multiply the other buffer.  Wave w owns tokens
// 64 (w % 4) .. +63 and all 128 rows, and the 32-k half (w / 4) of every
// chunk; the two halves' accumulators are added through LDS at the end, each
// half receiving and storing four of the eight row subtiles.
// Splitting the chunk's two 32-k steps between two waves puts two waves on
// every SIMD (128 accumulator registers each).
//
// The dequantized tile is stored fragment-major: the 16 x 32 MFMA operand of
// row subtile a and k half s is 1 KB in lane order (lane l = 16 g + i holds
// row 16 a + i, k 32 s + 8 g .. +7), so a wave reads each operand with one
// contiguous 1 KB access.  Thread t of wave w produces two of those 16-byte
// pieces from 16 codes of row 16 w + t % 16.  X reaches LDS through
// coalesced 16-byte loads (eight lanes per 128-byte token row) issued two
// chunks ahead, its rows' 16-byte pieces XOR-swizzled by (row / 2) % 8.
//
// The LoRA update is appended as extra reduction steps over the rank: B^T is
// staged in LDS through 8x8 transposes, s.T enters as bf16 hi and lo halves.
//
// kFormDense instantiates the same kernel over a bf16 weight [N, K] (16-bit LoRA,
// the baseline of "Performance Reality" in "QLoRA: Quantized Low Rank
// Adaptation at Extreme Scale"): each thread loads its 16 weights (32 bytes)
// instead of 16 codes and stores them into the same operand pieces, so the
// two forms differ only in the weight's bytes and the dequantization.
// kFormNoDq reads one fp32 constant per block in place of the 8-bit constant
// and its group's scale (4-bit codes without double quantization); the level
// table is an argument (NF4, INT4 or FP4).
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace qnf4 {

namespace {

constexpr int GP = 128;          // weight rows per workgroup
constexpr int GQ = 256;          // tokens per workgroup
constexpr int GK = 64;           // reduction elements per chunk (one block per row)
constexpr int GWT = 4;           // token groups
constexpr int GKS = 2;           // waves splitting a chunk's two 32-k steps
constexpr int GW = GWT * GKS;    // waves
constexpr int GT = 64 * GW;      // threads
constexpr int GTA = GP / 16;     // 16-row subtiles (8)
constexpr int GTB = GQ / GWT / 16;   // 16-token subtiles per wave (4)
constexpr int BTS = 64 + 8;     // LDS row stride of the B^T tile
constexpr int kAFrag = 64 * 8;   // bf16 elements of one 16 x 32 operand (1 KB)
constexpr int kATile = GTA * GKS * kAFrag;   // one dequantized 128 x 64 tile (16 KB)
constexpr int XTS = GK;          // LDS row stride of the X tile (128 B, XOR-swizzled)
constexpr int kXTile = GQ * XTS;   // elements of one X tile buffer
constexpr int XPT = GQ * GK / 8 / GT;   // 16-byte X pieces a thread stages per chunk (4)
constexpr int kFwdLds = kRepTabBytes + 2 * kATile * 2 + 2 * kXTile * 2;

__device__ __forceinline__ int xcd_remap(int b, int total) {
  const int n8 = total >> 3, rem = total & 7;
  const int x = b & 7, i = b >> 3;
  return x * n8 + min(x, rem) + i;
}

}  // namespace

template <int kForm>
__global__ __launch_bounds__(GT) void k_fwd_gemm(
    const uint16_t* __restrict__ X, int64_t M, const uint16_t* __restrict__ Wd,
    const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ absmax_q, const float* __restrict__ absmax_scale,
    int64_t N, int64_t K, const float* __restrict__ T, const uint16_t* __restrict__ Bl,
    int r, float s, uint16_t* __restrict__ Y, int ptiles, int qtiles, int cps,
    float* __restrict__ part, Nf4Tables tb, int ldt, int seg_rows) {
  // Dynamic LDS only (so the table sits at address 0): the replicated level
  // table, then two A tile buffers; after the main loop the same bytes hold
  // the accumulator exchange and the B^T tile of the LoRA update.
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  char* tab = reinterpret_cast<char*>(dyn);
  uint16_t* As = reinterpret_cast<uint16_t*>(dyn + kRepTabBytes);   // [2][kATile]
  uint16_t* Xs = As + 2 * kATile;   // two X tile buffers [GQ][XTS]

  const int tid = threadIdx.x;
  const int wave = wave_id(), lane = tid & 63;
  const int li = lane & 15, g = lane >> 4;
  const int wt = wave % GWT, ks = wave / GWT;
  if constexpr (kForm != kFormDense) build_rep_pair_table<GT>(tab, load_levels(tb), tid);

  // With a split reduction (few tiles), workgroup b takes chunks
  // [z cps, (z + 1) cps) of its tile and writes fp32 partial sums.
  const int ntiles = ptiles * qtiles;
  const int lin = xcd_remap(blockIdx.x, static_cast<int>(gridDim.x));
  const int z = lin / ntiles, tile = lin - z * ntiles;
  const int qt = tile / ptiles, pt = tile - qt * ptiles;
  const int64_t p0 = (int64_t)pt * GP, q0 = (int64_t)qt * GQ;
  const int c0 = z * cps;
  const int nchunks = min(static_cast<int>(K / GK), c0 + cps);   // end of this split's chunks
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
  // X is addressed from the tile's first token (its 256 rows span less
  // than 2^31 bytes for K <= 2^22).  (A plain conditional, not min(): the
  // 64-bit min is opaque to the compiler's uniformity analysis and would put
  // the descriptor in vector registers.)
  const int64_t tile_rows = M - q0 < GQ ? M - q0 : GQ;
  const BufRes rx = make_bufres(X + q0 * K, static_cast<uint32_t>(tile_rows * K * 2));

  // Dequantization role: row 16 wave + li of the tile, codes 32 sd + 16 h ..
  // +15 of the chunk (sd = lane / 32, h = (lane / 16) % 2): pieces 2 h and
  // 2 h + 1 of the operand (row subtile wave, k half sd).
  const int sd = lane >> 5, h = (lane >> 4) & 1;
  const int64_t dn = p0 + 16 * wave + li;
  const uint32_t dcode = static_cast<uint32_t>(dn * (K / 2)) + 16u * sd + 8u * h;   // + 32 c
  const uint32_t dblk = static_cast<uint32_t>(dn * KB);                           // + c
  // kFormDense: the same 16 weights as bf16, byte offset (+ 128 c)
  const uint32_t dw = static_cast<uint32_t>(dn * K * 2) + 64u * sd + 32u * h;
  u32x2 cw[2];
  uint32_t ce[2];
  float cd[2];
  u32x4 ww[2][2];
  auto load_codes = [&](int c, int st) {
    const bool live = c < nchunks;
    if constexpr (kForm == kFormDense) {
      const uint32_t o = live ? dw + 128u * c : 0x80000000u;
      ww[st][0] = buf_load16(rw, o);
      ww[st][1] = buf_load16(rw, live ? o + 16u : 0x80000000u);
    } else {
      const uint32_t blk = dblk + static_cast<uint32_t>(c);
      cw[st] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                             rc, live ? dcode + 32u * c : 0x80000000u, 0, 0));
      if constexpr (kForm == kFormNoDq) {   // e = 1, d = the block's absmax
        ce[st] = 1u;
        cd[st] = buf_load_f32(rd, live ? blk * 4u : 0x80000000u);
      } else {
        ce[st] = buf_load_u8(re, live ? blk : 0x80000000u);
        cd[st] = buf_load_f32(rd, live ? (blk / kGroup) * 4u : 0x80000000u);
      }
    }
  };
  // bf16_rne(fl32(level * fl32(e * d))) of 16 codes -> two operand pieces
  uint32_t ta[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) ta[b] = rep_lane_base(lane);
  uint16_t* const dpiece = As + (2 * wave + sd) * kAFrag + (32 * h + li) * 8;
  auto dequant = [&](int st, int buf) {
    if constexpr (kForm == kFormDense) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        *reinterpret_cast<u32x4*>(dpiece + buf * kATile + 16 * 8 * i) = ww[st][i];
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
      *reinterpret_cast<u32x4*>(dpiece + buf * kATile + 16 * 8 * i) =
          u32x4{pack_bf16x2(v0.x * chat, v0.y * chat), pack_bf16x2(v1.x * chat, v1.y * chat),
                pack_bf16x2(v2.x * chat, v2.y * chat), pack_bf16x2(v3.x * chat, v3.y * chat)};
    }
  };

  // X staging role: piece j of thread tid is token row xr + 64 j (xr = tid / 8)
  // of the tile, 16-byte piece tid % 8 of its 128-byte chunk row, stored at
  // slot (tid % 8) ^ ((row / 2) % 8).
  const int xr = tid >> 3, xq = tid & 7;
  const uint32_t xsrc = static_cast<uint32_t>((xr * K + 8 * xq) * 2);   // + 128 c
  u32x4 xw[2][XPT];
  auto load_x = [&](int c, int st) {
    const bool live = c < nchunks;
#pragma unroll
    for (int j = 0; j < XPT; ++j)
      xw[st][j] = buf_load16(
          rx, live ? xsrc + static_cast<uint32_t>((64 * j * K + c * GK) * 2) : 0x80000000u);
  };
  auto store_x = [&](int st, int buf) {
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int row = xr + 64 * j;
      *reinterpret_cast<u32x4*>(Xs + buf * kXTile + row * XTS + 8 * (xq ^ ((row >> 1) & 7))) =
          xw[st][j];
    }
  };

  f32x4 acc[GTA][GTB];
#pragma unroll
  for (int a = 0; a < GTA; ++a)
#pragma unroll
    for (int b = 0; b < GTB; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A operand (row subtile a, k half ks): one contiguous 1 KB read; B
  // operand: token 64 wt + 16 b + li, piece g + 4 ks (swizzle (li / 2) % 8)
  const uint16_t* const apiece = As + ks * kAFrag + lane * 8;
  const uint16_t* const xpiece = Xs + (64 * wt + li) * XTS + 8 * ((g + 4 * ks) ^ (li >> 1));
  // Operands of one 32-k step are read into registers first; the MFMAs then
  // touch no memory, so the compiler can interleave them with the staging
  // work of the next chunk (LDS reads and writes it cannot otherwise move
  // across, not knowing the two buffers are disjoint).
  u32x4 af[GTA], bf[GTB];
  auto read_frags = [&](int buf) {
#pragma unroll
    for (int b = 0; b < GTB; ++b)
      bf[b] = *reinterpret_cast<const u32x4*>(xpiece + buf * kXTile + 16 * b * XTS);
#pragma unroll
    for (int a = 0; a < GTA; ++a)
      af[a] = *reinterpret_cast<const u32x4*>(apiece + buf * kATile + 2 * a * kAFrag);
  };
  auto mma = [&]() {
#pragma unroll
    for (int a = 0; a < GTA; ++a)
#pragma unroll
      for (int b = 0; b < GTB; ++b) acc[a][b] = mfma16(af[a], bf[b], acc[a][b]);
  };

  load_codes(c0, 0);
  load_codes(c0 + 1, 1);
  load_x(c0, 0);
  load_x(c0 + 1, 1);
  __syncthreads();   // level table
  dequant(0, 0);
  store_x(0, 0);
  load_codes(c0 + 2, 0);
  load_x(c0 + 2, 0);
  __syncthreads();
  // iteration c: read the operands of chunk c from buffers c&1; stage chunk
  // c+1 into buffers (c+1)&1 -- dequantize its codes and store its X, both
  // loaded two iterations ago -- and refill those register stages with chunk
  // c+3; multiply chunk c.
  auto iter = [&](int c, auto stc) {
    constexpr int ST = decltype(stc)::value;
    read_frags(ST);
    dequant(ST ^ 1, ST ^ 1);
    store_x(ST ^ 1, ST ^ 1);
    load_codes(c + 3, ST ^ 1);
    load_x(c + 3, ST ^ 1);
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

  // LoRA update: 64 ranks at a time, B^T tile [128 rows][64 ranks] in LDS,
  // s.T hi / lo halves per lane from global memory.  Each k half takes one
  // of the chunk's two 32-rank steps, before the halves are added.
  if (r > 0 && z == 0) {   // the first split adds the LoRA update
    // T columns of this tile's segment: rows [j seg_rows, (j + 1) seg_rows)
    // of W belong to adapter j, whose T occupies columns j r .. of T (row
    // stride ldt); a single segment is the plain layer.
    const float* Tt = T + (p0 / seg_rows) * r;
    uint16_t* bt = As;
    for (int j0 = 0; j0 < r; j0 += 64) {
      // this wave's s.T operands, loaded before the B^T staging so that the
      // two loads' latencies overlap
      const int jt = j0 + 32 * ks + 8 * g;
      f32x4 traw[GTB][2];
      bool tok[GTB];
#pragma unroll
      for (int b = 0; b < GTB; ++b) {
        const int64_t m = q0 + 64 * wt + 16 * b + li;
        const bool ok = m < M && jt < r;
        tok[b] = ok;
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        traw[b][0] = ok ? *reinterpret_cast<const f32x4*>(Tt + m * ldt + jt) : zero;
        traw[b][1] = ok ? *reinterpret_cast<const f32x4*>(Tt + m * ldt + jt + 4) : zero;
      }
      if (tid < GP) {   // patch tid: rows 8 (tid % 16) .., ranks j0 + 8 (tid / 16) ..
        const int rp = tid % (GP / 8), kp = tid / (GP / 8);
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
      __syncthreads();
      {
        const int i = ks;
        {
          u32x4 th[GTB], tl[GTB];
#pragma unroll
          for (int b = 0; b < GTB; ++b) {
            uint32_t hi[4] = {0, 0, 0, 0}, lo[4] = {0, 0, 0, 0};
            if (tok[b]) {
              const f32x4 t0 = traw[b][0], t1 = traw[b][1];
              const float v[8] = {t0.x * s, t0.y * s, t0.z * s, t0.w * s,
                                  t1.x * s, t1.y * s, t1.z * s, t1.w * s};
#pragma unroll
              for (int e = 0; e < 4; ++e) split_bf16x2(v[2 * e], v[2 * e + 1], hi[e], lo[e]);
            }
            th[b] = u32x4{hi[0], hi[1], hi[2], hi[3]};
            tl[b] = u32x4{lo[0], lo[1], lo[2], lo[3]};
          }
#pragma unroll
          for (int a = 0; a < GTA; ++a) {
            const u32x4 af =
                *reinterpret_cast<const u32x4*>(bt + (16 * a + li) * BTS + 32 * i + 8 * g);
#pragma unroll
            for (int b = 0; b < GTB; ++b) {
              acc[a][b] = mfma16(af, th[b], acc[a][b]);
              acc[a][b] = mfma16(af, tl[b], acc[a][b]);
            }
          }
        }
      }
      __syncthreads();
    }
  }

  // Add the two k halves: wave ks keeps row subtiles 4 ks .. 4 ks + 3 and
  // receives them from its partner (the other ks, same token group) through
  // LDS, in one round; each half then stores its own row subtiles.
  f32x4* xch = reinterpret_cast<f32x4*>(dyn);   // [2][GWT][GTA/2][GTB][64]
  {
    // (compile-time accumulator indices on both sides of a scalar branch)
    auto hand = [&](auto kc) {
      constexpr int K0 = decltype(kc)::value, GIVE = 1 - K0;
#pragma unroll
      for (int a = 0; a < GTA / 2; ++a)
#pragma unroll
        for (int b = 0; b < GTB; ++b)
          xch[(((GIVE * GWT + wt) * (GTA / 2) + a) * GTB + b) * 64 + lane] =
              acc[GIVE * (GTA / 2) + a][b];
    };
    auto take = [&](auto kc) {
      constexpr int K0 = decltype(kc)::value;
#pragma unroll
      for (int a = 0; a < GTA / 2; ++a)
#pragma unroll
        for (int b = 0; b < GTB; ++b)
          acc[K0 * (GTA / 2) + a][b] +=
              xch[(((K0 * GWT + wt) * (GTA / 2) + a) * GTB + b) * 64 + lane];
    };
    if (ks == 0) hand(std::integral_constant<int, 0>{}); else hand(std::integral_constant<int, 1>{});
    __syncthreads();
    if (ks == 0) take(std::integral_constant<int, 0>{}); else take(std::integral_constant<int, 1>{});
  }

  // Y[m, n..n+3] for the lane's 4 consecutive rows n of each subtile (bf16),
  // or this split's fp32 partial sums part[z][m][n..n+3]
  auto store = [&](auto kc) {
    constexpr int K0 = decltype(kc)::value;
#pragma unroll
    for (int a0 = 0; a0 < GTA / 2; ++a0) {
      const int a = K0 * (GTA / 2) + a0;
      const int64_t n = p0 + 16 * a + 4 * g;
#pragma unroll
      for (int b = 0; b < GTB; ++b) {
        const int64_t m = q0 + 64 * wt + 16 * b + li;
        if (m < M && n < N) {
          const f32x4 v = acc[a][b];
          if (part) {
            *reinterpret_cast<f32x4*>(part + ((int64_t)z * M + m) * N + n) = v;
          } else {
            *reinterpret_cast<u32x2*>(Y + m * N + n) =
                u32x2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
          }
        }
      }
    }
  };
  if (ks == 0) store(std::integral_constant<int, 0>{}); else store(std::integral_constant<int, 1>{});
}

GemmSplit fwd_gemm_split(int64_t M, int64_t N, int64_t K) {
  return gemm_split((N + GP - 1) / GP * ((M + GQ - 1) / GQ), K / GK);
}

hipError_t launch_fwd_gemm(const uint16_t* X, int64_t M, const Nf4View& w,
                            const float* T, const uint16_t* B, int r, float s,
                            uint16_t* Y, float* part, const Nf4Tables& tb, hipStream_t stream,
                            int ldt, int64_t seg_rows) {
  static const hipError_t attr[3] = {
      hipFuncSetAttribute(reinterpret_cast<const void*>(&k_fwd_gemm<kFormDq>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kFwdLds),
      hipFuncSetAttribute(reinterpret_cast<const void*>(&k_fwd_gemm<kFormNoDq>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kFwdLds),
      hipFuncSetAttribute(reinterpret_cast<const void*>(&k_fwd_gemm<kFormDense>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kFwdLds)};
  const int form = w.dense ? kFormDense : (w.dq ? kFormDq : kFormNoDq);
  if (attr[form] != hipSuccess) return attr[form];
  decltype(&k_fwd_gemm<kFormDq>) kern =
      form == kFormDense ? k_fwd_gemm<kFormDense> : (form == kFormNoDq ? k_fwd_gemm<kFormNoDq> : k_fwd_gemm<kFormDq>);
  const int ptiles = static_cast<int>((w.N + GP - 1) / GP);
  const int qtiles = static_cast<int>((M + GQ - 1) / GQ);
  const GemmSplit sp = fwd_gemm_split(M, w.N, w.K);
  if (sp.splits > 1 && !part) return hipErrorInvalidValue;
  prof_begin(0, stream);
  hipLaunchKernelGGL(kern,
                     dim3(ptiles * qtiles * sp.splits), dim3(GT), kFwdLds, stream, X, M, w.dense,
                     w.codes, w.absmax_q, w.absmax_scale, w.N, w.K, T, B, r, s, Y, ptiles,
                     qtiles, sp.cps, sp.splits > 1 ? part : nullptr, tb, ldt > 0 ? ldt : r,
                     static_cast<int>(seg_rows > 0 ? seg_rows : w.N));
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && sp.splits > 1)
    e = launch_split_reduce_bf16(part, sp.splits, M * w.N, Y, stream);
  prof_end(0, stream);
  return e;
}

}  // namespace qnf4
