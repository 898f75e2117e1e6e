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
// Workgroup = 16 waves on two fragments of 16 weight rows; eight waves share
// a fragment and split its reduction dimension in chunks of 128 k (wave kw
// takes chunks kw, kw+8, ...).  Lane l works on row (l % 16) and on the 32 k
// starting at 32 (l / 16) inside each chunk.  The code loads are the only
// vector-memory traffic of the main loop; they run D chunks ahead in a
// register ring.  The 8-bit block constants and fp32 group scales of the
// workgroup's rows, and X itself when it is small, are staged in LDS once.
// The byte-pair level table sits in LDS as 32 copies interleaved at 8-byte
// steps in 256-byte rows, so lane l reads copy (l % 32) and a lookup never
// meets a bank conflict; its address is one SDWA byte move.  The waves'
// partial sums meet in LDS; the LoRA update is added as extra MFMA steps
// over the rank before that reduction.
#include "device_common.hpp"
#include "kernels.hpp"

namespace qnf4 {

namespace {

constexpr int kDecR = 2;                       // row fragments per workgroup
constexpr int kDecKSlots = 8;                  // waves on one fragment
constexpr int kDecWaves = kDecR * kDecKSlots;
constexpr int kDecThreads = kDecWaves * 64;
constexpr int kDecRows = 16 * kDecR;
// A buffer offset past the end of every buffer the kernel reads (weights are
// limited to N*K <= 2^32, so their code buffers hold at most 2^31 bytes).
constexpr uint32_t kDecOffNone = 0x80000000u;
constexpr int kDecMaxK = 32768;                // block constants of the rows fit in LDS
constexpr int kDecXLdsBytes = 64 * 1024;       // X staged in LDS up to this size
constexpr int kDecLdsMax = 160 * 1024;         // LDS of one workgroup
constexpr int kDecXPieces = kDecXLdsBytes / 16 / kDecThreads;   // 16-byte X pieces a thread
// T partial sums: quad q = (token m, ranks 4jq..4jq+3) is summed by
// ceil(nz / kDecTSumLoads) threads with kDecTSumLoads loads each; M r <=
// kDecTSumMaxMR keeps that within the workgroup for the at most
// kMaxDownPartials partials.
constexpr int kDecTSumLoads = 8;
constexpr int kDecTSumMaxMR = 4 * kDecThreads * kDecTSumLoads / kMaxDownPartials;
constexpr int kDecEPieces = (kDecRows * kDecMaxK / kBlock / 4 + kDecThreads - 1) / kDecThreads;

int round16(int64_t v) { return static_cast<int>((v + 15) / 16 * 16); }

// Dynamic LDS of one workgroup, in order: the level table, the waves'
// partial sums (first the partial sums of T), the summed T, the block
// constants transposed to [K/64 + 1][32] bytes (the extra column is zero),
// the group scales [dmax] of the workgroup's blocks, and (XLDS) X [M][K]
// followed by 128 zero bytes.
struct DecLds {
  int eoff, doff, xoff, dmax, total;
  DecLds(int64_t M, int64_t K, bool xlds) {
    const int64_t kb = K / kBlock;
    eoff = kRepTabBytes + kDecThreads * 16 + kDecTSumMaxMR * 4;
    doff = eoff + round16(kDecRows * (kb + 1));
    dmax = static_cast<int>(kDecRows * kb / kGroup + 2);
    xoff = doff + round16(4 * dmax);
    total = xoff + (xlds ? round16(M * K * 2) + 128 : 0);
  }
};

}  // namespace

template <int D, bool XLDS>
__global__ __launch_bounds__(kDecThreads) void k_fwd_decode(
    const uint16_t* __restrict__ X, int M, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ absmax_q, const float* __restrict__ absmax_scale,
    int64_t N, int64_t K, const float* __restrict__ T, int nz, float* __restrict__ Tout,
    const uint16_t* __restrict__ Bl, int r, float s, uint16_t* __restrict__ Y,
    Nf4Tables tb, int eoff, int doff, int xoff, int dmax, float inv_kb) {
  constexpr int ROWS = kDecRows;
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  char* tab = reinterpret_cast<char*>(dyn);                          // level pairs
  f32x4* red = reinterpret_cast<f32x4*>(dyn + kRepTabBytes);            // [kDecThreads]
  f32x4* tfin = red + kDecThreads;                                   // [kDecTSumMaxMR / 4]
  uint8_t* et = dyn + eoff;                                          // [KB + 1][ROWS]
  float* dsc = reinterpret_cast<float*>(dyn + doff);                 // [dmax]
  uint16_t* xs = reinterpret_cast<uint16_t*>(dyn + xoff);            // [M][K], zeros
  const int tid = threadIdx.x;
  const int wave = wave_id(), lane = tid & 63;
  const int p = wave / kDecKSlots, kw = wave % kDecKSlots;           // fragment, K slot
  const int li = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * ROWS;
  const int K32 = static_cast<int>(K);
  const int KB = K32 / kBlock;
  const int nchunks = (K32 + 127) / 128;
  const int nmine = nchunks > kw ? (nchunks - kw + kDecKSlots - 1) / kDecKSlots : 0;

  // Buffer descriptors: rows n >= N fall outside the code / constant buffers
  // and read as zero, and so do token rows li >= M of X.  The second half of
  // a chunk past K (K % 128 == 64) gets a zero block constant instead, so the
  // code bytes it reads from the next row contribute nothing.
  const uint32_t nb = static_cast<uint32_t>(N * K / kBlock);
  const BufRes rc = make_bufres(codes, static_cast<uint32_t>(N * K / 2));
  const BufRes re = make_bufres(absmax_q, nb);
  const BufRes rd = make_bufres(absmax_scale, ((nb + kGroup - 1) / kGroup) * 4u);
  const BufRes rx = make_bufres(X, static_cast<uint32_t>(M) * static_cast<uint32_t>(K) * 2u);

  // Staging loads first, a fixed number per thread, so that waiting for them
  // does not wait for the code stream issued after them: the block constants
  // of the workgroup's rows (one contiguous byte range, read as dwords), their
  // group scales, X, and the partial sums of T.
  const uint32_t e0 = static_cast<uint32_t>(n0) * KB;   // first block of the workgroup
  const uint32_t g0 = e0 / kGroup;
  const int erange = ROWS * KB;                         // bytes, a multiple of 4
  uint32_t ev[kDecEPieces];
#pragma unroll
  for (int i = 0; i < kDecEPieces; ++i) {
    const int idx = tid + i * kDecThreads;
    ev[i] = __builtin_amdgcn_raw_buffer_load_b32(re, 4 * idx < erange ? e0 + 4u * idx
                                                                      : kDecOffNone, 0, 0);
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
  // Quad q is summed by tpq threads (kDecTSumLoads partials each, in
  // registers), then by one thread over those tpq (nz > 0 only with
  // M r <= kDecTSumMaxMR, so nq * tpq <= kDecThreads).
  const int nq = M * r / 4;
  const int tpq = nz > 0 ? (nz + kDecTSumLoads - 1) / kDecTSumLoads : 1;
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
  const uint32_t cb = static_cast<uint32_t>((n0 + 16 * p + li) * (K / 2)) + 64u * kw + 16u * g;
  const uint32_t xb = (static_cast<uint32_t>(li) * K32 + 128u * kw + 32u * g) * 2u;
  u32x4 cw[D];
  u32x4 xv[XLDS ? 1 : D][4];
  auto load = [&](int t, int st) {
    const bool live = t < nmine;
    cw[st] = buf_load16(rc, live ? cb + 64u * kDecKSlots * t : kDecOffNone);
    if constexpr (!XLDS) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xv[st][i] = buf_load16(rx, live ? xb + 256u * kDecKSlots * t + 16u * i : kDecOffNone);
    }
  };
#pragma unroll
  for (int u = 0; u < D; ++u) load(u, u);

  // LoRA update: step q of this wave's fragment (wave kw takes step kw)
  // contributes P[n, j] = B[j, n] times Q[m, j] = s*T[m, j] split into bf16
  // hi and lo; its B operand is loaded now so the tail waits on no fresh load.
  const int nsteps = (r + 31) / 32;
  const int64_t nrow = n0 + 16 * p + li;
  uint32_t lb[4] = {0, 0, 0, 0};
  if (kw < nsteps) {
    const int j = 32 * kw + 8 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lo = 0, hi = 0;
      if (nrow < N && j < r) {
        lo = Bl[(int64_t)(j + 2 * i) * N + nrow];
        hi = Bl[(int64_t)(j + 2 * i + 1) * N + nrow];
      }
      lb[i] = lo | (hi << 16);
    }
  }

  // Stage into LDS: level table, X, the T partial sums.
  build_rep_pair_table(tab, tb, tid);
  if constexpr (XLDS) {
#pragma unroll
    for (int i = 0; i < kDecXPieces; ++i) {
      const int idx = tid + i * kDecThreads;
      if (16 * idx < xrange) *reinterpret_cast<u32x4*>(xs + 8 * idx) = xw[i];
    }
    if (tid < 8) *reinterpret_cast<u32x4*>(xs + M * K32 + 8 * tid) = u32x4{0, 0, 0, 0};
  }
  red[tid] = tp;
  // Block constants, transposed so that a fragment's 16 rows read 16
  // consecutive bytes; column KB is zero for the half chunk past K.
#pragma unroll
  for (int i = 0; i < kDecEPieces; ++i) {
    const int idx = tid + i * kDecThreads;
    if (4 * idx < erange) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int f = 4 * idx + b;   // row-major index: row f / KB, column f % KB
        const int row = static_cast<int>((static_cast<float>(f) + 0.5f) * inv_kb);
        et[(f - row * KB) * ROWS + row] = static_cast<uint8_t>(ev[i] >> (8 * b));
      }
    }
  }
  if (tid < ROWS) et[KB * ROWS + tid] = 0;
  if (tid < dmax) dsc[tid] = dv;

  // Lanes past M read X from the zero slot with stride 0; past K (the second
  // half of a chunk when K % 128 == 64) they meet the zero block constant,
  // and their X reads stay inside the next token row or the zero slot.
  const uint16_t* xlane = li < M ? xs + li * K32 + 32 * g : xs + M * K32;
  const int xstep = li < M ? 128 : 0;
  const int row = 16 * p + li;
  // Table addresses: copy (lane % 32) in byte 0, entry in byte 1.  The
  // kernel declares no static LDS, so the dynamic block, and the table at its
  // start, begins at LDS address 0 and the address needs no base added.
  uint32_t ta[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) ta[b] = rep_lane_base(lane);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // All LDS reads of a chunk (constant, table lookups, X) are issued before
  // any of their products, so one LDS round trip serves the chunk's MFMAs.
  auto compute = [&](int t, int st) {
    const int c = kw + kDecKSlots * t;
    const int j = 2 * c + (g >> 1);   // block of the lane inside its row (KB: zero)
    const float e = static_cast<float>(et[j * ROWS + row]);
    const float d = dsc[(e0 + static_cast<uint32_t>(row * KB + j)) / kGroup - g0];
    f32x2 lk[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = cw[st][i];
      lk[i][0] = rep_lookup<0>(ta[0], w);
      lk[i][1] = rep_lookup<1>(ta[1], w);
      lk[i][2] = rep_lookup<2>(ta[2], w);
      lk[i][3] = rep_lookup<3>(ta[3], w);
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
    const float chat = e * d;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4 a;
#pragma unroll
      for (int b = 0; b < 4; ++b) a[b] = pack_bf16x2(lk[i][b].x * chat, lk[i][b].y * chat);
      acc = mfma16(a, xf[i], acc);
    }
  };
  __syncthreads();
  for (int t0 = 0; t0 < nmine; t0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int t = t0 + u;
      if (t < nmine) compute(t, u);
      load(t + D, u);
    }
  }

  // T's partial sums are added after the main loop, off its critical path.
  __syncthreads();
  if (nz > 0 && tid < nq) {   // fixed order: deterministic
    f32x4 t = red[tid * tpq];
    for (int u = 1; u < tpq; ++u) t += red[tid * tpq + u];
    tfin[tid] = t;
    if (blockIdx.x == 0) *reinterpret_cast<f32x4*>(Tout + 4 * tid) = t;   // [M][r]
  }
  __syncthreads();

  if (kw < nsteps) {
    const int j = 32 * kw + 8 * g;
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
    acc = mfma16(bw, u32x4{h[0], h[1], h[2], h[3]}, acc);
    acc = mfma16(bw, u32x4{l[0], l[1], l[2], l[3]}, acc);
  }

  red[wave * 64 + lane] = acc;   // the T partial sums in red were read before the barrier above
  __syncthreads();
  if (kw == 0) {
    f32x4 t = red[(p * kDecKSlots) * 64 + lane];
#pragma unroll
    for (int w = 1; w < kDecKSlots; ++w) t += red[(p * kDecKSlots + w) * 64 + lane];
    const int64_t nout = n0 + 16 * p + 4 * g;   // 4 consecutive outputs of token li
    if (li < M && nout < N) {
      *reinterpret_cast<u32x2*>(Y + (int64_t)li * N + nout) =
          u32x2{pack_bf16x2(t.x, t.y), pack_bf16x2(t.z, t.w)};
    }
  }
}

namespace {

template <int D, bool XLDS>
hipError_t launch_decode_variant(const uint16_t* X, int64_t M, const Nf4View& w, const float* T,
                                 int nz, float* Tout, const uint16_t* B, int r, float s,
                                 uint16_t* Y, const Nf4Tables& tb, hipStream_t stream) {
  // allow the largest dynamic LDS this variant takes (once per variant)
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&k_fwd_decode<D, XLDS>),
      hipFuncAttributeMaxDynamicSharedMemorySize,
      XLDS ? kDecLdsMax : DecLds(1, kDecMaxK, false).total);
  if (attr != hipSuccess) return attr;
  const DecLds L(M, w.K, XLDS);
  const unsigned grid = static_cast<unsigned>((w.N + kDecRows - 1) / kDecRows);
  const float inv_kb = 1.0f / static_cast<float>(w.K / kBlock);
  hipLaunchKernelGGL((k_fwd_decode<D, XLDS>), dim3(grid), dim3(kDecThreads), L.total, stream,
                     X, (int)M, w.codes, w.absmax_q, w.absmax_scale, w.N, w.K, T, nz, Tout, B,
                     r, s, Y, tb, L.eoff, L.doff, L.xoff, L.dmax, inv_kb);
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
  // Two chunks in flight per wave: with all 16 waves of every CU streaming,
  // deeper rings (measured up to 8) only delay the first products.
  hipError_t e;
  // X goes to LDS when it fits next to the rest (M = 1 always; M = 4 up to
  // K = 8192); otherwise each wave reads its X fragments from global memory.
  if (M * w.K * 2 <= kDecXLdsBytes && DecLds(M, w.K, true).total <= kDecLdsMax)
    e = launch_decode_variant<2, true>(X, M, w, T, nz, Tout, B, r, s, Y, tb, stream);
  else
    e = launch_decode_variant<2, false>(X, M, w, T, nz, Tout, B, r, s, Y, tb, stream);
  prof_end(2, stream);
  return e;
}

}  // namespace qnf4
