// Forward for few tokens (M <= 16): the bandwidth-bound decode path.
//
// Y = X . deq(W)^T + s . T . B with T = X . A computed beforehand.  At small
// M the layer is a stream over the NF4 weight (0.516 bytes per weight), so
// the kernel is organised around the code stream: every lane issues 16-byte
// loads of 32 consecutive codes, turns them into bf16 levels in registers
// and feeds them straight to v_mfma_f32_16x16x32_bf16 with the token
// dimension padded to 16.
//
// The weight of a code is c_b . q (Mathematical Formulation of "DL0087
// QLoRA": the block constant dequantized from the 8-bit constant and its
// group scale, times the NF4 level).  Since c_b is shared by the 64 weights
// of a block, this kernel multiplies the levels by X first and the block's
// partial sum by c_b after: every MFMA covers the codes of one block only,
// and four FMAs per block apply its scale to the lane's four outputs.  The
// per-weight work is then one table lookup, with no multiply and no
// conversion (the levels are rounded to bf16 once, in the table).
//
// Workgroup = 16 waves on two fragments of 16 weight rows; eight waves share
// a fragment and split its reduction dimension in chunks of 128 k (wave kw
// takes chunks kw, kw+8, ...).  A chunk is two blocks.  Lane l loads the 16
// bytes at 16 (l / 16) of row (l % 16)'s 64-byte chunk segment: lanes 0-31
// hold the first block, lanes 32-63 the second.  One cross-half swap of two
// of the four dwords (v_permlane32_swap) leaves every lane with two dwords of
// each block; MFMA s of a block takes dword s of each lane, and X is read at
// the matching k.  The code loads are the only vector-memory traffic of the
// main loop; they run D chunks ahead in a register ring.
//
// Staged in LDS once: the bf16 level-pair table (64 copies, one per lane, so
// lookups never meet a bank conflict), the block scales c_b of the
// workgroup's rows as fp32 [K/64 + 1][32] (the extra column is zero), the
// workgroup's columns of B, and X itself when it fits.  The waves' partial
// sums meet in LDS; the LoRA update is added as extra MFMA steps over the
// rank before that reduction.
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
constexpr int kDecMaxK = 32768;                // block scales of the rows fit in LDS
constexpr int kDecMaxR = 256;
constexpr int kDecXLdsBytes = 64 * 1024;       // X staged in LDS up to this size
constexpr int kDecLdsMax = 160 * 1024;         // LDS of one workgroup
constexpr int kDecXPieces = kDecXLdsBytes / 16 / kDecThreads;   // at most 4 16-byte X pieces a thread
constexpr int kDecXZero = 256;                 // zero bytes after X (lanes past M read there)
constexpr int kDecXPad = 8;                    // X rows in LDS are K + 8 elements apart
// T partial sums are added up by rows of 16 lanes: row h takes the quad (4
// ranks of one token) h, its lane z the partials z + 16 i, i < TQ.  M r <=
// kDecTSumMaxMR keeps that within one quad per row.  A kernel with X in LDS
// takes up to 64 partials (TQ = 4); the one reading X from global memory, 32
// (TQ = 2, registers are short there).  With a final T, the lanes of the
// LoRA waves use the first two loads for their 8 values.
constexpr int dec_tq(int fr) { return fr == 1 ? 4 : 2; }
constexpr int kDecTSumMaxMR = 4 * (kDecThreads / 16);
static_assert(kMaxDownPartials <= dec_tq(1) * 16, "partials per lane of a 16-lane row");
static_assert(kMaxDownPartials / 2 <= dec_tq(2) * 16, "partials per lane of a 16-lane row");
// Block constants of the workgroup's rows, read as 8-byte pieces.
constexpr int kDecEPieces = (kDecRows * kDecMaxK / kBlock / 8 + kDecThreads - 1) / kDecThreads;

int round16(int64_t v) { return static_cast<int>((v + 15) / 16 * 16); }

// Dynamic LDS of one workgroup, in order: the level table, B's columns
// [r][32], the summed T, the block scales [K/64 + 1][32] fp32, and (XLDS) X
// [M][K + kDecXPad] (the padding puts the rows' equal columns in different
// banks) followed by kDecXZero zero bytes.  After the main loop the waves'
// partial sums [kDecThreads] f32x4 reuse the bytes from the block scales on.
struct DecLds {
  int boff, toff, coff, xoff, total;
  DecLds(int64_t M, int64_t K, int r, bool xlds, int fr = 1) {
    const int64_t kb = K / kBlock;
    boff = kRepTabBytes;
    toff = boff + round16(int64_t(64) * r);
    coff = toff + kDecTSumMaxMR * 4;
    xoff = coff + round16(kDecRows * (kb + 1) * 4);
    const int end = xoff + (xlds ? round16(M * (K + kDecXPad) * 2) + kDecXZero : 0);
    total = end > coff + kDecThreads * 16 * fr ? end : coff + kDecThreads * 16 * fr;
  }
};

}  // namespace

template <int D, int XP, int FR>
__global__ __launch_bounds__(kDecThreads) void k_fwd_decode(
    const uint16_t* __restrict__ X, int M, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ absmax_q, const float* __restrict__ absmax_scale,
    int64_t N, int64_t K, const float* __restrict__ T, int nz, float* __restrict__ Tout,
    const uint16_t* __restrict__ Bl, int r, float s, uint16_t* __restrict__ Y,
    Nf4Tables tb, int boff, int toff, int coff, int xoff, float inv_kb) {
  constexpr int ROWS = kDecRows;
  constexpr bool XLDS = XP > 0;   // X staged in LDS, XP 16-byte pieces per thread
  // FR = 1: eight waves per fragment; FR = 2: every wave works on both
  // fragments, and 16 waves split K (each X piece then serves 32 rows).
  constexpr int KS = kDecKSlots * FR;   // waves splitting K
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  char* tab = reinterpret_cast<char*>(dyn);                          // bf16 level pairs
  uint16_t* bst = reinterpret_cast<uint16_t*>(dyn + boff);           // B columns [r][ROWS]
  f32x4* tfin = reinterpret_cast<f32x4*>(dyn + toff);                // [kDecTSumMaxMR / 4]
  float* csc = reinterpret_cast<float*>(dyn + coff);                 // [KB + 1][ROWS]
  f32x4* red = reinterpret_cast<f32x4*>(dyn + coff);                 // after the main loop
  uint16_t* xs = reinterpret_cast<uint16_t*>(dyn + xoff);            // [M][K + pad], zeros
  const Levels lv = load_levels(tb);
  const int tid = threadIdx.x;
  const int wave = wave_id(), lane = tid & 63;
  const int p = FR == 1 ? wave / kDecKSlots : 0, kw = wave % KS;      // fragment, K slot
  const int li = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * ROWS;
  const int K32 = static_cast<int>(K);
  const int KB = K32 / kBlock;
  const int nchunks = (K32 + 127) / 128;
  const int nmine = nchunks > kw ? (nchunks - kw + KS - 1) / KS : 0;
  auto frag = [&](int f) { return FR == 1 ? p : f; };   // fragment of the wave's slot f

  // Buffer descriptors: rows n >= N fall outside the code / constant buffers
  // and read as zero, and so do token rows li >= M of X.  The second block of
  // a chunk past K (K % 128 == 64) reads the next row's codes; its products
  // are dropped.
  const uint32_t nb = static_cast<uint32_t>(N * K / kBlock);
  const BufRes rc = make_bufres(codes, static_cast<uint32_t>(N * K / 2));
  const BufRes re = make_bufres(absmax_q, nb);
  const BufRes rd = make_bufres(absmax_scale, ((nb + kGroup - 1) / kGroup) * 4u);
  const BufRes rx = make_bufres(X, static_cast<uint32_t>(M) * static_cast<uint32_t>(K) * 2u);

  // Staging loads first, a fixed number per thread, so that waiting for them
  // does not wait for the code stream issued after them: the block constants
  // of the workgroup's rows (one contiguous byte range, in 8-byte pieces) and
  // the group scale of each piece (a piece never straddles two groups: both
  // the range start and the group size are multiples of 8), X, and for the
  // LoRA update (used only after the main loop) the partial sums of T and
  // the workgroup's columns of B.
  const uint32_t e0 = static_cast<uint32_t>(n0) * KB;   // first block of the workgroup
  const int erange = ROWS * KB;                         // bytes, a multiple of 8
  u32x2 ev[kDecEPieces];
  float dv[kDecEPieces];
#pragma unroll
  for (int i = 0; i < kDecEPieces; ++i) {
    const int idx = tid + i * kDecThreads;
    const bool ok = 8 * idx < erange;
    ev[i] = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_raw_buffer_load_b64(re, ok ? e0 + 8u * idx : kDecOffNone, 0, 0));
    dv[i] = buf_load_f32(rd, ok ? ((e0 + 8u * idx) / kGroup) * 4u : kDecOffNone);
  }
  // X: XP pieces per thread, as many as M K 2 bytes need (a load whose lanes
  // all fall outside the range still occupies the address unit, and at kernel
  // start the staging loads of 16 waves queue there ahead of the code stream)
  u32x4 xw[XLDS ? XP : 1];
  const int xrange = M * K32 * 2;
  if constexpr (XLDS) {
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int idx = tid + i * kDecThreads;
      xw[i] = buf_load16(rx, 16 * idx < xrange ? 16u * idx : kDecOffNone);
    }
  }
  // T for the LoRA update, used only after the main loop.  With nz > 0, the
  // 16-lane row h sums quad h (4 ranks of one token) over the partials, lane
  // z loading partials z + 16 i; with nz == 0 T is final and the lanes of the
  // LoRA waves load their own 8 values of it (the first two loads).
  const int nsteps = (r + 31) / 32;
  const int nq = M * r / 4;
  const int hr = tid >> 4, hl = tid & 15;
  constexpr int TQ = dec_tq(FR);
  f32x4 tq[TQ];
  {
    // (one load sequence for both cases: a branch here would make the
    // compiler wait for the loads of one side before those of the other)
    const BufRes rt = make_bufres(T, static_cast<uint32_t>((nz > 0 ? nz : 1) * M * r) * 4u);
    const int j = 32 * kw + 8 * g;
    const bool lora_lane = kw < nsteps && li < M && j < r;
#pragma unroll
    for (int i = 0; i < TQ; ++i) {
      const int z = hl + 16 * i;
      const bool ok = nz > 0 ? (hr < nq && z < nz) : (lora_lane && i < 2);
      const int idx = nz > 0 ? z * M * r + 4 * hr : li * r + j + 4 * i;
      tq[i] = __builtin_bit_cast(
          f32x4, buf_load16(rt, ok ? static_cast<uint32_t>(idx * 4) : kDecOffNone));
    }
  }
  // The workgroup's 32 columns of B [r][N] (one 16-byte piece per thread for
  // r <= 256), staged in LDS for the LoRA update after the main loop.
  u32x4 bpiece;
  {
    const BufRes rbl = make_bufres(Bl, static_cast<uint32_t>(r) * static_cast<uint32_t>(N) * 2u);
    const int j = tid >> 2, c = tid & 3;
    const bool ok = j < r && n0 + 8 * c < N;
    bpiece = buf_load16(rbl, ok ? static_cast<uint32_t>((j * N + n0 + 8 * c) * 2) : kDecOffNone);
  }

  // The code ring: every call issues the same loads, so the compiler can
  // count them and wait for exactly one chunk at a time; chunks past the
  // wave's last one get an offset beyond every buffer and read zeros without
  // memory traffic.  Without X in LDS, each lane also loads the X pieces its
  // four MFMAs take.
  uint32_t cb[FR];
#pragma unroll
  for (int f = 0; f < FR; ++f)
    cb[f] = static_cast<uint32_t>((n0 + 16 * frag(f) + li) * (K / 2)) + 64u * kw + 16u * g;
  // k offset (inside a block) of the 8 codes that lane group g supplies to
  // step 0 of a block after the swap (dword 4 (g % 2) + 2 (g / 2); step 1
  // takes the next dword).
  const int xo0 = 8 * (4 * (g & 1) + 2 * (g >> 1));
  const uint32_t xb = (static_cast<uint32_t>(li) * K32 + 128u * kw + xo0) * 2u;
  u32x4 cw[D][FR];
  u32x4 xv[XLDS ? 1 : D][4];
  auto load = [&](int t, int st) {
    const bool live = t < nmine;
#pragma unroll
    for (int f = 0; f < FR; ++f)
      cw[st][f] = buf_load16(rc, live ? cb[f] + 64u * KS * t : kDecOffNone);
    if constexpr (!XLDS) {
#pragma unroll
      for (int i = 0; i < 4; ++i)   // block i / 2, step i % 2
        xv[st][i] = buf_load16(
            rx, live ? xb + 256u * KS * t + 128u * (i >> 1) + 16u * (i & 1) : kDecOffNone);
    }
  };
#pragma unroll
  for (int u = 0; u < D; ++u) load(u, u);

  // Stage into LDS: level table, X, block scales, B.
  build_rep_bf16_pair_table<kDecThreads>(tab, lv, tid);
  if constexpr (XLDS) {
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int idx = tid + i * kDecThreads;
      const int row = idx / (K32 / 8);   // piece idx holds elements 8 idx .. of X [M][K]
      if (16 * idx < xrange) *reinterpret_cast<u32x4*>(xs + 8 * idx + kDecXPad * row) = xw[i];
    }
    if (tid < kDecXZero / 16)
      *reinterpret_cast<u32x4*>(xs + M * (K32 + kDecXPad) + 8 * tid) = u32x4{0, 0, 0, 0};
    if (tid < M)   // the row padding, which the half chunk past K reads
      *reinterpret_cast<u32x4*>(xs + tid * (K32 + kDecXPad) + K32) = u32x4{0, 0, 0, 0};
  }
  // Block scales c = e . d, transposed so that the four rows of a lane's
  // outputs read 16 consecutive bytes; column KB is zero.
#pragma unroll
  for (int i = 0; i < kDecEPieces; ++i) {
    const int idx = tid + i * kDecThreads;
    if (8 * idx < erange) {
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const int f = 8 * idx + b;   // row-major index: row f / KB, column f % KB
        const int row = static_cast<int>((static_cast<float>(f) + 0.5f) * inv_kb);
        const uint32_t w = b < 4 ? ev[i].x : ev[i].y;
        const float e = static_cast<float>((w >> (8 * (b % 4))) & 0xFFu);
        csc[(f - row * KB) * ROWS + row] = e * dv[i];
      }
    }
  }
  if (tid < ROWS) csc[KB * ROWS + tid] = 0.f;
  if ((tid >> 2) < r) reinterpret_cast<u32x4*>(bst)[tid] = bpiece;

  // Lanes past M read X from the zero bytes with stride 0; past K (the second
  // block of a chunk when K % 128 == 64) their X reads stay inside the row
  // padding, the next token row or the zero bytes, and the products are
  // dropped.
  const int xrow = K32 + kDecXPad;
  const uint16_t* xlane = li < M ? xs + li * xrow + xo0 : xs + M * xrow + xo0;
  const int xstep = li < M ? 128 : 0;
  const float* clane = csc + 4 * g;   // + 16 fragment: scales of the lane's output rows
  // Table addresses: the lane's copy offset in byte 0, entry in byte 1.  The
  // kernel declares no static LDS, so the dynamic block, and the table at its
  // start, begins at LDS address 0 and the address needs no base added.
  const uint32_t ta = static_cast<uint32_t>(lane) << 2;

  f32x4 acc[FR];
#pragma unroll
  for (int f = 0; f < FR; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
  // All LDS reads of a chunk (scales, table lookups, X) are issued before any
  // of their products, so one LDS round trip serves the chunk's MFMAs.
  auto compute = [&](int t, int st) {
    const int c = kw + KS * t;
    u32x4 a[FR][4], xf[4];
    f32x4 cA[FR], cB[FR];
#pragma unroll
    for (int f = 0; f < FR; ++f) {
      // Regroup: dwords 0, 1 of lanes 0-31 and 2, 3 of lanes 32-63 stay; the
      // others trade places across the two halves.  After it, dwords 0, 1
      // hold codes of the first block and 2, 3 of the second, in every lane.
      uint32_t d[4] = {cw[st][f].x, cw[st][f].y, cw[st][f].z, cw[st][f].w};
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const auto sw = __builtin_amdgcn_permlane32_swap(d[u], d[2 + u], false, false);
        d[u] = sw[0];
        d[2 + u] = sw[1];
      }
      cA[f] = *reinterpret_cast<const f32x4*>(clane + 16 * frag(f) + (2 * c) * ROWS);
      cB[f] = *reinterpret_cast<const f32x4*>(clane + 16 * frag(f) + (2 * c + 1) * ROWS);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[f][i][0] = rep_bf16_lookup<0>(ta, d[i]);
        a[f][i][1] = rep_bf16_lookup<1>(ta, d[i]);
        a[f][i][2] = rep_bf16_lookup<2>(ta, d[i]);
        a[f][i][3] = rep_bf16_lookup<3>(ta, d[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (XLDS)
        xf[i] = *reinterpret_cast<const u32x4*>(xlane + c * xstep + 64 * (i >> 1) + 8 * (i & 1));
      else
        xf[i] = xv[st][i];
    }
    __builtin_amdgcn_sched_barrier(0);
    // (the second block of a chunk past K, when K % 128 == 64, is dropped
    // rather than scaled by zero: its products may hold anything)
    const bool second = 2 * c + 1 < KB;   // wave-uniform
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int f = 0; f < FR; ++f) {
      f32x4 pA = mfma16(a[f][0], xf[0], zero);
      pA = mfma16(a[f][1], xf[1], pA);
      f32x4 pB = mfma16(a[f][2], xf[2], zero);
      pB = mfma16(a[f][3], xf[3], pB);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[f][j] = __builtin_fmaf(cA[f][j], pA[j], acc[f][j]);
        if (second) acc[f][j] = __builtin_fmaf(cB[f][j], pB[j], acc[f][j]);
      }
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

  // The LoRA step's B operand, B[j .. j+7, n] for the lane's row n.
  u32x4 bw[FR];
#pragma unroll
  for (int f = 0; f < FR; ++f) {
    bw[f] = u32x4{0, 0, 0, 0};
    if (kw < nsteps) {
      const int j = 32 * kw + 8 * g, row = 16 * frag(f) + li;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = j + 2 * i < r ? bst[(j + 2 * i) * ROWS + row] : 0u;
        const uint32_t hi = j + 2 * i + 1 < r ? bst[(j + 2 * i + 1) * ROWS + row] : 0u;
        bw[f][i] = lo | (hi << 16);
      }
    }
  }

  // T's partial sums are added after the main loop, off its critical path:
  // the lane's four partials, then a butterfly over its 16-lane row with DPP
  // moves (xor 1, xor 2, rotate 4, rotate 8), in a fixed order
  // (deterministic).
  if (nz > 0) {
    f32x4 v = tq[0] + tq[1];
    if constexpr (TQ == 4) v = (tq[0] + tq[1]) + (tq[2] + tq[3]);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v[c] += dpp_f32<0xB1>(v[c]);    // quad_perm [1, 0, 3, 2]
      v[c] += dpp_f32<0x4E>(v[c]);    // quad_perm [2, 3, 0, 1]
      v[c] += dpp_f32<0x124>(v[c]);   // row_ror 4
      v[c] += dpp_f32<0x128>(v[c]);   // row_ror 8
    }
    if (hl == 0 && hr < nq) {
      tfin[hr] = v;
      if (blockIdx.x == 0) *reinterpret_cast<f32x4*>(Tout + 4 * hr) = v;   // [M][r]
    }
  }
  __syncthreads();

  // LoRA update: step kw of the fragment (rank block 32 kw .. 32 kw + 31)
  // adds P[n, j] = B[j, n] times Q[m, j] = s T[m, j], with Q split into bf16
  // hi and lo halves.
  if (kw < nsteps) {
    const int j = 32 * kw + 8 * g;
    f32x4 t0 = tq[0], t1 = tq[1];
    if (nz > 0) {
      const bool ok = li < M && j < r;
      t0 = ok ? tfin[(li * r + j) / 4] : f32x4{0.f, 0.f, 0.f, 0.f};
      t1 = ok ? tfin[(li * r + j) / 4 + 1] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float v[8] = {t0.x * s, t0.y * s, t0.z * s, t0.w * s,
                        t1.x * s, t1.y * s, t1.z * s, t1.w * s};
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split_bf16x2(v[2 * i], v[2 * i + 1], h[i], l[i]);
#pragma unroll
    for (int f = 0; f < FR; ++f) {
      acc[f] = mfma16(bw[f], u32x4{h[0], h[1], h[2], h[3]}, acc[f]);
      acc[f] = mfma16(bw[f], u32x4{l[0], l[1], l[2], l[3]}, acc[f]);
    }
  }

  // the block scales and X are no longer read: red [wave][FR][64]
#pragma unroll
  for (int f = 0; f < FR; ++f) red[(wave * FR + f) * 64 + lane] = acc[f];
  __syncthreads();
  // fragment po is summed over its KS slots by one wave: the first wave of
  // the fragment (FR = 1), or wave po (FR = 2)
  const int po = FR == 1 ? p : wave;
  if (FR == 1 ? kw == 0 : wave < kDecR) {
    auto part = [&](int w) {   // slot w of fragment po
      return FR == 1 ? red[(po * kDecKSlots + w) * 64 + lane] : red[(w * FR + po) * 64 + lane];
    };
    f32x4 t = part(0);
#pragma unroll
    for (int w = 1; w < KS; ++w) t += part(w);
    const int64_t nout = n0 + 16 * po + 4 * g;   // 4 consecutive outputs of token li
    if (li < M && nout < N) {
      *reinterpret_cast<u32x2*>(Y + (int64_t)li * N + nout) =
          u32x2{pack_bf16x2(t.x, t.y), pack_bf16x2(t.z, t.w)};
    }
  }
}

namespace {

template <int D, int XP, int FR>
hipError_t launch_decode_variant(const uint16_t* X, int64_t M, const Nf4View& w, const float* T,
                                 int nz, float* Tout, const uint16_t* B, int r, float s,
                                 uint16_t* Y, const Nf4Tables& tb, hipStream_t stream) {
  // allow the largest dynamic LDS (once per variant)
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&k_fwd_decode<D, XP, FR>),
      hipFuncAttributeMaxDynamicSharedMemorySize, kDecLdsMax);
  if (attr != hipSuccess) return attr;
  const DecLds L(M, w.K, r, XP > 0, FR);
  if (L.total > kDecLdsMax || nz > 16 * dec_tq(FR)) return hipErrorInvalidValue;
  const unsigned grid = static_cast<unsigned>((w.N + kDecRows - 1) / kDecRows);
  const float inv_kb = 1.0f / static_cast<float>(w.K / kBlock);
  hipLaunchKernelGGL((k_fwd_decode<D, XP, FR>), dim3(grid), dim3(kDecThreads), L.total, stream,
                     X, (int)M, w.codes, w.absmax_q, w.absmax_scale, w.N, w.K, T, nz, Tout, B,
                     r, s, Y, tb, L.boff, L.toff, L.coff, L.xoff, inv_kb);
  return hipGetLastError();
}

bool decode_x_in_lds(int64_t M, int64_t K, int r) {
  return M * K * 2 <= kDecXLdsBytes && DecLds(M, K, r, true).total <= kDecLdsMax;
}

}  // namespace

bool decode_fits(int64_t M, int64_t K) { return M <= 16 && K <= kDecMaxK; }

// Up to 64 partials when one token's T is at most 64 values and X sits in LDS
// (each workgroup reads all nz M r of them), else 32.
int decode_max_t_partials(int64_t M, int64_t K, int r) {
  return M * r <= 64 && decode_x_in_lds(M, K, r) ? kMaxDownPartials : kMaxDownPartials / 2;
}

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
  // X goes to LDS when it fits next to the rest (M = 1 up to K = 22016 with
  // r <= 64; M = 4 up to K = 8192), in as few 16-byte pieces per thread as it
  // needs; otherwise each wave reads its X pieces from global memory.
  if (decode_x_in_lds(M, w.K, r)) {
    const int64_t xbytes = M * w.K * 2;
    const int64_t per_piece = 16 * kDecThreads;
    if (xbytes <= per_piece)
      e = launch_decode_variant<2, 1, 1>(X, M, w, T, nz, Tout, B, r, s, Y, tb, stream);
    else if (xbytes <= 2 * per_piece)
      e = launch_decode_variant<2, 2, 1>(X, M, w, T, nz, Tout, B, r, s, Y, tb, stream);
    else
      e = launch_decode_variant<2, kDecXPieces, 1>(X, M, w, T, nz, Tout, B, r, s, Y, tb, stream);
  } else {
    // X from global memory: each wave works on both fragments, so each X
    // piece it loads serves 32 rows.
    e = launch_decode_variant<2, 0, 2>(X, M, w, T, nz, Tout, B, r, s, Y, tb, stream);
  }
  prof_end(2, stream);
  return e;
}

static_assert(kRepTabBytes + 64 * kDecMaxR + kDecTSumMaxMR * 4 +
                      kDecRows * (kDecMaxK / kBlock + 1) * 4 <= kDecLdsMax,
              "block scales of the largest K fit next to the table without X");

}  // namespace qnf4
