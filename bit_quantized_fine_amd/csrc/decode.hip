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
// Workgroup = 8 waves on R fragments of 16 weight rows.  The reduction runs
// in chunks of 128 k; wave w takes chunks w, w+8, w+16, ... of every row
// fragment.  Lane l works on row (l % 16) of each fragment and the 32 k
// starting at 32 (l / 16) inside the chunk.  The code loads are the only
// vector-memory traffic of the main loop: they run D chunks ahead in a
// register ring, while the 8-bit block constants and fp32 group scales of the
// workgroup's rows, and X itself when it is small, are staged in LDS once at
// the start.  The waves' partial sums meet in LDS; the LoRA update is added
// as extra MFMA steps over the rank, dealt to the waves before that
// reduction.
#include "device_common.hpp"
#include "kernels.hpp"

namespace qnf4 {

namespace {

constexpr int kDecWaves = 8;
constexpr int kDecThreads = kDecWaves * 64;
// A buffer offset past the end of every buffer the kernel reads (weights are
// limited to N*K <= 2^32, so their code buffers hold at most 2^31 bytes).
constexpr uint32_t kDecOffNone = 0x80000000u;
constexpr int kDecR = 1;                   // row fragments per workgroup
constexpr int kDecMaxK = 32768;            // block constants of the rows fit in LDS
constexpr int kDecXLdsBytes = 64 * 1024;   // X staged in LDS up to this size
constexpr int kDecXPieces = kDecXLdsBytes / 16 / kDecThreads;   // 16-byte X pieces a thread
// T partial sums: quad q = (token m, ranks 4jq..4jq+3) is summed by
// kDecThreads / (M r / 4) threads with kDecTSumLoads loads each, which covers
// the at most kMaxDownPartials partials when M r <= kDecTSumMaxMR.
constexpr int kDecTSumLoads = 8;
constexpr int kDecTSumMaxMR = 4 * kDecThreads * kDecTSumLoads / kMaxDownPartials;

int round16(int64_t v) { return static_cast<int>((v + 15) / 16 * 16); }

// Dynamic LDS of one workgroup: the 8-bit block constants [16R][K/64] and
// group scales [dmax] as loaded, the block scales c_hat = e * d they make,
// transposed to [K/64 + 1][16R] fp32 (the extra column is zero), and (XLDS)
// X [M][K] bf16 followed by 128 zero bytes.
struct DecLds {
  int ebytes, dmax, dbytes, cbytes, xbytes;
  DecLds(int R, int64_t M, int64_t K, bool xlds) {
    const int64_t kb = K / kBlock;
    ebytes = round16(16 * R * kb);
    dmax = static_cast<int>(16 * R * kb / kGroup + 2);
    dbytes = round16(4 * dmax);
    cbytes = round16(4 * 16 * R * (kb + 1));
    xbytes = xlds ? round16(M * K * 2) + 128 : 0;
  }
  int total() const { return ebytes + dbytes + cbytes + xbytes; }
};

}  // namespace

// LDS byte address of the byte-pair table entry for byte `B` of w: one SDWA
// shift that reads the byte in place (the table base goes into the LDS
// instruction's offset field).
template <int B>
__device__ __forceinline__ uint32_t pair_addr(uint32_t w) {
  uint32_t a;
  if constexpr (B == 0)
    asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD "
        "src1_sel:BYTE_0" : "=v"(a) : "v"(w));
  else if constexpr (B == 1)
    asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD "
        "src1_sel:BYTE_1" : "=v"(a) : "v"(w));
  else if constexpr (B == 2)
    asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD "
        "src1_sel:BYTE_2" : "=v"(a) : "v"(w));
  else
    asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD "
        "src1_sel:BYTE_3" : "=v"(a) : "v"(w));
  return a;
}

template <int R, int D, bool XLDS, int WPE>
__global__ __launch_bounds__(kDecThreads, WPE) void k_fwd_decode(
    const uint16_t* __restrict__ X, int M, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ absmax_q, const float* __restrict__ absmax_scale,
    int64_t N, int64_t K, const float* __restrict__ T, int nz, float* __restrict__ Tout,
    const uint16_t* __restrict__ Bl, int r, float s, uint16_t* __restrict__ Y,
    Nf4Tables tb, int ebytes, int dmax, int dbytes, int cbytes) {
  constexpr int NW = kDecWaves, ROWS = 16 * R;
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  __shared__ float2 tab[256];
  // partial sums of T at the start, the waves' partial outputs at the end
  constexpr int kRedSlots = NW * R * 64 > kDecThreads ? NW * R * 64 : kDecThreads;
  __shared__ f32x4 red_tsum[kRedSlots];
  __shared__ f32x4 tfin[kDecTSumMaxMR / 4];
  f32x4* tsum = red_tsum;                                           // [kDecThreads]
  auto red = [&](int w, int p) -> f32x4* { return red_tsum + (w * R + p) * 64; };
  const int tid = threadIdx.x;
  const int wave = wave_id(), lane = tid & 63;
  const int li = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * ROWS;
  const int K32 = static_cast<int>(K);
  const int KB = K32 / kBlock;
  const int nchunks = (K32 + 127) / 128;
  const int nmine = nchunks > wave ? (nchunks - wave + NW - 1) / NW : 0;
  uint8_t* es = dyn;                                               // [ROWS][KB]
  float* dsc = reinterpret_cast<float*>(dyn + ebytes);             // [dmax]
  float* cs = reinterpret_cast<float*>(dyn + ebytes + dbytes);     // [KB + 1][ROWS]
  uint16_t* xs = reinterpret_cast<uint16_t*>(dyn + ebytes + dbytes + cbytes);   // [M][K], zeros

  // Buffer descriptors: rows n >= N fall outside the code / constant buffers
  // and read as zero, and so do token rows li >= M of X.  The second half of
  // a chunk past K (K % 128 == 64) gets a zero block scale instead, so the
  // code bytes it reads from the next row contribute nothing.
  const uint32_t nb = static_cast<uint32_t>(N * K / kBlock);
  const BufRes rc = make_bufres(codes, static_cast<uint32_t>(N * K / 2));
  const BufRes re = make_bufres(absmax_q, nb);
  const BufRes rd = make_bufres(absmax_scale, ((nb + kGroup - 1) / kGroup) * 4u);
  const BufRes rx = make_bufres(X, static_cast<uint32_t>(M) * static_cast<uint32_t>(K) * 2u);

  // Staging loads first, a fixed number per thread, so that waiting for them
  // does not wait for the code stream issued after them: the block constants
  // of the workgroup's rows (one contiguous byte range), their group scales,
  // X, and the partial sums of T.
  const uint32_t e0 = static_cast<uint32_t>(n0) * KB;   // first block of the workgroup
  const uint32_t g0 = e0 / kGroup;
  const int erange = ROWS * KB;
  u32x4 ev[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int idx = tid + i * kDecThreads;
    ev[i] = buf_load16(re, 16 * idx < erange ? e0 + 16u * idx : kDecOffNone);
  }
  const float dv = buf_load_f32(rd, tid < dmax ? (g0 + tid) * 4u : kDecOffNone);
  u32x4 xw[XLDS ? kDecXPieces : 1];
  const int xrange = M * K32 * 2;
  if constexpr (XLDS) {
#pragma unroll
    for (int i = 0; i < kDecXPieces; ++i) {
      const int idx = tid + i * kDecThreads;
      xw[i] = buf_load16(rx, 16 * idx < xrange ? 16u * idx : kDecOffNone);
    }
  }
  // (nz > 0 only with M r <= kDecTSumMaxMR, so tpq * kDecTSumLoads >= nz.)
  const int nq = M * r / 4;
  const int tpq = nz > 0 ? kDecThreads / nq : 1;
  const int myq = tid / tpq, sub = tid % tpq;
  f32x4 tp = {0.f, 0.f, 0.f, 0.f};
  if (nz > 0) {
    const BufRes rt = make_bufres(T, static_cast<uint32_t>(nz * M * r) * 4u);
    const int m = myq / (r / 4), jq = myq % (r / 4);
#pragma unroll
    for (int i = 0; i < kDecTSumLoads; ++i) {
      const int z = sub + tpq * i;
      const bool ok = myq < nq && z < nz;
      tp += __builtin_bit_cast(
          f32x4, buf_load16(rt, ok ? static_cast<uint32_t>(((z * M + m) * r + 4 * jq) * 4)
                                   : kDecOffNone));
    }
  }

  // The code ring: every call issues the same loads, so the compiler can
  // count them and wait for exactly one chunk at a time; chunks past the
  // wave's last one get an offset beyond every buffer and read zeros without
  // memory traffic.
  uint32_t cb[R];
#pragma unroll
  for (int p = 0; p < R; ++p)
    cb[p] = static_cast<uint32_t>((n0 + 16 * p + li) * (K / 2)) + 64u * wave + 16u * g;
  const uint32_t xb = (static_cast<uint32_t>(li) * K32 + 128u * wave + 32u * g) * 2u;
  u32x4 cw[D][R];
  u32x4 xv[XLDS ? 1 : D][4];
  auto load = [&](int t, int st) {
    const bool live = t < nmine;
#pragma unroll
    for (int p = 0; p < R; ++p)
      cw[st][p] = buf_load16(rc, live ? cb[p] + 64u * NW * t : kDecOffNone);
    if constexpr (!XLDS) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xv[st][i] = buf_load16(rx, live ? xb + 256u * NW * t + 16u * i : kDecOffNone);
    }
  };
#pragma unroll
  for (int u = 0; u < D; ++u) load(u, u);

  // LoRA update: pair q = (fragment p, 32-rank step) contributes
  // P[n, j] = B[j, n] times Q[m, j] = s*T[m, j] split into bf16 hi and lo.
  // Pairs are dealt round-robin to the waves; the first pair's B operand is
  // loaded now so the tail waits on no fresh loads.
  const int nsteps = (r + 31) / 32;
  const int npairs = R * nsteps;
  auto load_b = [&](int q, uint32_t* bw) {
    const int p = q / nsteps, j = 32 * (q % nsteps) + 8 * g;
    const int64_t n = n0 + 16 * p + li;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lo = 0, hi = 0;
      if (n < N && j < r) {
        lo = Bl[(int64_t)(j + 2 * i) * N + n];
        hi = Bl[(int64_t)(j + 2 * i + 1) * N + n];
      }
      bw[i] = lo | (hi << 16);
    }
  };
  uint32_t lb[4];
  if (wave < npairs) load_b(wave, lb);

  // Stage into LDS.
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int idx = tid + i * kDecThreads;
    if (16 * idx < erange) *reinterpret_cast<u32x4*>(es + 16 * idx) = ev[i];
  }
  if (tid < dmax) dsc[tid] = dv;
  if constexpr (XLDS) {
#pragma unroll
    for (int i = 0; i < kDecXPieces; ++i) {
      const int idx = tid + i * kDecThreads;
      if (16 * idx < xrange) *reinterpret_cast<u32x4*>(xs + 8 * idx) = xw[i];
    }
    if (tid < 8) *reinterpret_cast<u32x4*>(xs + M * K32 + 8 * tid) = u32x4{0, 0, 0, 0};
  }
  tsum[tid] = tp;
  if (tid < 256) {
    float lo = 0.f, hi = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      lo = ((tid & 15) == j) ? tb.q[j] : lo;
      hi = ((tid >> 4) == j) ? tb.q[j] : hi;
    }
    tab[tid] = make_float2(lo, hi);
  }
  __syncthreads();
  // Block scales, transposed so that the 16 rows of a fragment read 16
  // consecutive words; column KB stays zero for the half chunk past K.
  for (int i = tid; i < ROWS * (KB + 1); i += kDecThreads) {
    const int col = i / ROWS, row = i % ROWS;
    float v = 0.f;
    if (col < KB) {
      const uint32_t blk = e0 + static_cast<uint32_t>(row * KB + col);
      v = static_cast<float>(es[row * KB + col]) * dsc[blk / kGroup - g0];
    }
    cs[i] = v;
  }
  if (nz > 0) {
    if (tid < nq) {   // fixed order: deterministic
      f32x4 t = tsum[tid * tpq];
      for (int u = 1; u < tpq; ++u) t += tsum[tid * tpq + u];
      tfin[tid] = t;
      if (blockIdx.x == 0) *reinterpret_cast<f32x4*>(Tout + 4 * tid) = t;   // [M][r]
    }
  }
  __syncthreads();
  const char* tabb = reinterpret_cast<const char*>(tab);

  f32x4 acc[R];
#pragma unroll
  for (int p = 0; p < R; ++p) acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
  // All LDS reads of a chunk (constants, table lookups, X) are issued before
  // any of their products, so one LDS round trip serves the chunk's 4R MFMAs.
  // Lanes past M read X from the zero slot with stride 0; past K (the second
  // half of a chunk when K % 128 == 64) they meet the zero block scale, and
  // their X reads stay inside the next token row or the zero slot.
  const uint16_t* xlane = li < M ? xs + li * K32 + 32 * g : xs + M * K32;
  const int xstep = li < M ? 128 : 0;
  const float* clane = cs + (g >> 1) * ROWS + li;
  auto compute = [&](int t, int st) {
    const int c = wave + NW * t;
    float chat[R];
#pragma unroll
    for (int p = 0; p < R; ++p) chat[p] = clane[2 * c * ROWS + 16 * p];
    float2 lk[R][4][4];
#pragma unroll
    for (int p = 0; p < R; ++p)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = cw[st][p][i];
        lk[p][i][0] = *reinterpret_cast<const float2*>(tabb + pair_addr<0>(w));
        lk[p][i][1] = *reinterpret_cast<const float2*>(tabb + pair_addr<1>(w));
        lk[p][i][2] = *reinterpret_cast<const float2*>(tabb + pair_addr<2>(w));
        lk[p][i][3] = *reinterpret_cast<const float2*>(tabb + pair_addr<3>(w));
      }
    u32x4 xf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (XLDS)
        xf[i] = *reinterpret_cast<const u32x4*>(xlane + c * xstep + 8 * i);
      else
        xf[i] = xv[st][i];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int p = 0; p < R; ++p) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x4 a;
#pragma unroll
        for (int b = 0; b < 4; ++b)
          a[b] = pack_bf16x2(lk[p][i][b].x * chat[p], lk[p][i][b].y * chat[p]);
        acc[p] = mfma16(a, xf[i], acc[p]);
      }
    }
  };
  for (int t0 = 0; t0 < nmine; t0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int t = t0 + u;
      if (t < nmine) compute(t, u);
      load(t + D, u);
    }
  }

  for (int q = wave; q < npairs; q += NW) {
    if (q != wave) load_b(q, lb);
    const int p = q / nsteps, j = 32 * (q % nsteps) + 8 * g;
    f32x4 t0 = {0.f, 0.f, 0.f, 0.f}, t1 = t0;
    if (li < M && j < r) {
      if (nz > 0) {
        t0 = tfin[(li * r + j) / 4];
        t1 = tfin[(li * r + j) / 4 + 1];
      } else {
        t0 = *reinterpret_cast<const f32x4*>(T + (int64_t)li * r + j);
        t1 = *reinterpret_cast<const f32x4*>(T + (int64_t)li * r + j + 4);
      }
    }
    const float v[8] = {t0.x * s, t0.y * s, t0.z * s, t0.w * s,
                        t1.x * s, t1.y * s, t1.z * s, t1.w * s};
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split_bf16x2(v[2 * i], v[2 * i + 1], h[i], l[i]);
    const u32x4 bw = {lb[0], lb[1], lb[2], lb[3]};
#pragma unroll
    for (int pp = 0; pp < R; ++pp) {   // compile-time register index; p is wave-uniform
      if (pp == p) {
        acc[pp] = mfma16(bw, u32x4{h[0], h[1], h[2], h[3]}, acc[pp]);
        acc[pp] = mfma16(bw, u32x4{l[0], l[1], l[2], l[3]}, acc[pp]);
      }
    }
  }

#pragma unroll
  for (int p = 0; p < R; ++p) red(wave, p)[lane] = acc[p];
  __syncthreads();
  for (int p = wave; p < R; p += NW) {
    f32x4 t = red(0, p)[lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) t += red(w, p)[lane];
    const int64_t nout = n0 + 16 * p + 4 * g;   // 4 consecutive outputs of token li
    if (li < M && nout < N) {
      *reinterpret_cast<u32x2*>(Y + (int64_t)li * N + nout) =
          u32x2{pack_bf16x2(t.x, t.y), pack_bf16x2(t.z, t.w)};
    }
  }
}

namespace {

template <int R, int D, bool XLDS, int WPE>
hipError_t launch_decode_variant(const uint16_t* X, int64_t M, const Nf4View& w, const float* T,
                                 int nz, float* Tout, const uint16_t* B, int r, float s,
                                 uint16_t* Y, const Nf4Tables& tb, hipStream_t stream) {
  // allow the largest dynamic LDS this variant takes (once per variant)
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&k_fwd_decode<R, D, XLDS, WPE>),
      hipFuncAttributeMaxDynamicSharedMemorySize,
      DecLds(R, 1, kDecMaxK, false).total() + (XLDS ? kDecXLdsBytes + 128 : 0));
  if (attr != hipSuccess) return attr;
  const DecLds L(R, M, w.K, XLDS);
  const unsigned grid = static_cast<unsigned>((w.N + 16 * R - 1) / (16 * R));
  hipLaunchKernelGGL((k_fwd_decode<R, D, XLDS, WPE>), dim3(grid), dim3(kDecThreads), L.total(),
                     stream, X, (int)M, w.codes, w.absmax_q, w.absmax_scale, w.N, w.K, T, nz,
                     Tout, B, r, s, Y, tb, L.ebytes, L.dmax, L.dbytes, L.cbytes);
  return hipGetLastError();
}

}  // namespace

bool decode_fits(int64_t M, int64_t K) { return M <= 16 && K <= kDecMaxK; }

bool decode_folds_t(int64_t M, int r) {
  return r > 0 && M <= 4 && M * r <= kDecTSumMaxMR;
}

hipError_t launch_fwd_decode(const uint16_t* X, int64_t M, const Nf4View& w,
                             const float* T, int nz, float* Tout, const uint16_t* B, int r,
                             float s, uint16_t* Y, const Nf4Tables& tb, hipStream_t stream) {
  prof_begin(2, stream);
  hipError_t e;
  if (M * w.K * 2 <= kDecXLdsBytes)
    e = launch_decode_variant<kDecR, 4, true, 4>(X, M, w, T, nz, Tout, B, r, s, Y, tb, stream);
  else
    e = launch_decode_variant<kDecR, 4, false, 2>(X, M, w, T, nz, Tout, B, r, s, Y, tb, stream);
  prof_end(2, stream);
  return e;
}

}  // namespace qnf4
