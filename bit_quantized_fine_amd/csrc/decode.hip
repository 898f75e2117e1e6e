// Forward for few tokens (M <= 16): the bandwidth-bound decode path.
//
// Y = X . deq(W)^T + s . T . B with T = X . A computed beforehand.  At small
// M the layer is a stream over the NF4 weight (0.516 bytes per weight), so
// the kernel is organised around the code stream: every lane issues 16-byte
// loads of 32 consecutive codes, dequantizes them in registers and feeds them
// straight to v_mfma_f32_16x16x32_bf16 with the token dimension padded to 16.
//
// Every weight entering the MFMA is the defined dequantized value
// bf16_rne(fl32(q[code] . c_b)) with c_b = fl32(e_b . d_g) (Mathematical
// Formulation of "DL0087 QLoRA": the bf16 tile is rebuilt just before the
// matmul).  A code byte selects an fp32 level pair from a table in LDS; the
// pair is multiplied by the block constant and rounded to a bf16 pair.
//
// Workgroup = 16 waves on two fragments of 16 weight rows; eight waves share
// a fragment and split its reduction dimension in chunks of 128 k (wave kw
// takes chunks kw, kw+8, ...).  A chunk is two blocks.  Lane l loads the 16
// bytes at 16 (l / 16) of row (l % 16)'s 64-byte chunk segment, i.e. the 32 k
// starting at 32 (l / 16): lanes 0-31 hold the first block, lanes 32-63 the
// second, so each lane needs one block constant per chunk.  MFMA i of a chunk
// takes dword i of every lane (k = 32 (l / 16) + 8 i .. +7), and X is read at
// the same k.  The code loads are the only vector-memory traffic of the main
// loop; they run D chunks ahead in a register ring.
//
// Staged in LDS once: the fp32 level-pair table (32 copies, lane l reading
// copy l % 32, so a half-wave's lookups never meet a bank conflict), the
// block constants c_b of the workgroup's rows as fp32 [K/64 + 1][32] (the
// extra column is zero), the workgroup's columns of B, and X itself when it
// fits.  The waves' partial sums meet in LDS; the LoRA update is added as
// extra MFMA steps over the rank before that reduction.
//
// When X does not fit whole and has more than 8 token rows, the SL
// instantiations stage it in K-slices of 1024 columns (32 KB at 16 tokens),
// together with that slice's block constants, in two LDS copies used in
// turn: every wave takes one chunk of every slice, one workgroup barrier
// ends each slice, and the slice after next is stored into the copy just
// freed while the waves work on the other, from registers loaded two slices
// ahead.  The code ring runs on across the boundaries.
//
// The level table is an argument (NF4, or the INT4 / FP4 tables of "4-bit
// NormalFloat" in "QLoRA: Finetuning 65B Models on a Single GPU"), and the
// NODQ instantiation stages fp32 block constants c_b (no double
// quantization) in place of e_b . d_g.
#include <type_traits>

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
// holds up to 64 partials so (TQ = 4); the others, 32 (TQ = 2, registers are
// short there).  With a final T, the lanes of the LoRA waves use the first
// two loads for their 8 values.
constexpr int dec_tq(int fr, int sl = 0) { return fr == 1 && sl == 0 ? 4 : 2; }
constexpr int kDecTSumMaxMR = 4 * (kDecThreads / 16);
// More T values than that (up to one per thread: M r <= kDecTFinMaxMR), or
// more partials than the registers hold, are summed after the main loop
// instead, one value per thread over the partials in order, without
// registers held through the loop.
constexpr int kDecTFinMaxMR = kDecThreads;
int dec_tfin_floats(int64_t M, int r) {
  return M * r > kDecTSumMaxMR && M * r <= kDecTFinMaxMR ? static_cast<int>(M * r)
                                                         : kDecTSumMaxMR;
}
static_assert(kMaxDownPartials <= dec_tq(1) * 16, "partials per lane of a 16-lane row");
static_assert(kMaxDownPartials / 2 <= dec_tq(2) * 16, "partials per lane of a 16-lane row");
// Block constants of the workgroup's rows, read as 8-byte pieces.
constexpr int kDecEPieces = (kDecRows * kDecMaxK / kBlock / 8 + kDecThreads - 1) / kDecThreads;

int round16(int64_t v) { return static_cast<int>((v + 15) / 16 * 16); }

// Dynamic LDS of one workgroup, in order: the level table, B's columns
// [r][32], the summed T, the block scales [K/64 + 1][32] fp32, and (XLDS) X
// [M][K + kDecXPad] (the padding puts the rows' equal columns in different
// banks) followed by kDecXZero zero bytes.  With K-slices of ksl columns the
// scales and X hold one slice: K is replaced by ksl.  After the main loop the
// waves' partial sums [kDecThreads] f32x4 reuse the bytes from the block
// scales on.
struct DecLds {
  int boff, toff, coff, xoff, total;
  DecLds(int64_t M, int64_t K, int r, bool xlds, int fr = 1, int ksl = 0, int nbuf = 1) {
    const int64_t kx = ksl > 0 ? ksl : K;
    const int64_t kb = kx / kBlock;
    boff = kRepTabBytes;
    toff = boff + round16(int64_t(64) * r);
    coff = toff + round16(int64_t(4) * dec_tfin_floats(M, r));
    xoff = coff + nbuf * round16(kDecRows * (kb + 1) * 4);
    const int end = xoff + (xlds ? nbuf * round16(M * (kx + kDecXPad) * 2) + kDecXZero : 0);
    total = end > coff + kDecThreads * 16 * fr ? end : coff + kDecThreads * 16 * fr;
  }
};

}  // namespace

template <int D, int XP, int FR, bool NODQ, bool SL>
__global__ __launch_bounds__(kDecThreads) void k_fwd_decode(
    const uint16_t* __restrict__ X, int M, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ absmax_q, const float* __restrict__ absmax_scale,
    int64_t N, int64_t K, const float* __restrict__ T, int nz, float* __restrict__ Tout,
    const uint16_t* __restrict__ Bl, int r, float s, uint16_t* __restrict__ Y,
    Nf4Tables tb, int boff, int toff, int coff, int xoff, float inv_kb, int ldt, int ldb,
    int ldy, int ksl) {
  constexpr int ROWS = kDecRows;
  constexpr bool XLDS = XP > 0;   // X staged in LDS, XP 16-byte pieces per thread
  // SL: X and the block constants staged in K-slices of ksl = 1024 columns
  // (one chunk of each of the eight waves of a fragment), in two LDS copies
  // and two register sets used in turn; slice t sits in copy t % 2, which is
  // also the code ring's slot of chunk t.
  static_assert(!SL || (XP == 2 && FR == 1 && D == 2), "sliced form");
  constexpr int NB = SL ? 2 : 1;   // LDS copies of X and of the block constants
  // FR = 1: eight waves per fragment; FR = 2: every wave works on both
  // fragments, and 16 waves split K (each X piece then serves 32 rows).
  constexpr int KS = kDecKSlots * FR;   // waves splitting K
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  char* tab = reinterpret_cast<char*>(dyn);                          // fp32 level pairs
  uint16_t* bst = reinterpret_cast<uint16_t*>(dyn + boff);           // B columns [r][ROWS]
  f32x4* tfin = reinterpret_cast<f32x4*>(dyn + toff);   // the summed T [M r / 4]
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
  const int KX = SL ? ksl : K32;   // columns of X and of the block scales in LDS
  const int KXB = KX / kBlock;
  const int nslices = (K32 + KX - 1) / KX;

  // Buffer descriptors: rows n >= N fall outside the code / constant buffers
  // and read as zero, and so do token rows li >= M of X.  The second block of
  // a chunk past K (K % 128 == 64) reads the next row's codes; its weights
  // are zero (block constant from the zero column KB).
  const uint32_t nb = static_cast<uint32_t>(N * K / kBlock);
  const BufRes rc = make_bufres(codes, static_cast<uint32_t>(N * K / 2));
  const BufRes re = make_bufres(absmax_q, nb);
  // second-level scales, or (NODQ) one fp32 constant per block
  const BufRes rd =
      make_bufres(absmax_scale, (NODQ ? nb : (nb + kGroup - 1) / kGroup) * 4u);
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
  u32x4 cv[NODQ ? kDecEPieces : 1][2];   // NODQ: the 8 blocks' fp32 constants
  if constexpr (!SL) {
#pragma unroll
    for (int i = 0; i < kDecEPieces; ++i) {
      const int idx = tid + i * kDecThreads;
      const bool ok = 8 * idx < erange;
      if constexpr (NODQ) {
        const uint32_t o = (e0 + 8u * idx) * 4u;
        cv[i][0] = buf_load16(rd, ok ? o : kDecOffNone);
        cv[i][1] = buf_load16(rd, ok ? o + 16u : kDecOffNone);
      } else {
        ev[i] = __builtin_bit_cast(
            u32x2,
            __builtin_amdgcn_raw_buffer_load_b64(re, ok ? e0 + 8u * idx : kDecOffNone, 0, 0));
        dv[i] = buf_load_f32(rd, ok ? ((e0 + 8u * idx) / kGroup) * 4u : kDecOffNone);
      }
    }
  }
  // X: XP pieces per thread, as many as M K 2 bytes need (a load whose lanes
  // all fall outside the range still occupies the address unit, and at kernel
  // start the staging loads of 16 waves queue there ahead of the code stream)
  u32x4 xw[XLDS ? XP : 1];
  const int xrange = M * K32 * 2;
  if constexpr (XLDS && !SL) {
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int idx = tid + i * kDecThreads;
      xw[i] = buf_load16(rx, 16 * idx < xrange ? 16u * idx : kDecOffNone);
    }
  }
  // One K-slice (SL): X piece idx holds columns 8 (idx % (KX / 8)) .. + 7 of
  // token row idx / (KX / 8); constant entry f (one per thread) is block
  // f / ROWS of the slice in row f % ROWS (its place in the transposed LDS
  // layout).  Columns and blocks past K read zero, so the half chunk past K
  // multiplies zeros.
  u32x4 xn[SL ? XP : 1];   // the second register set for X
  uint32_t se[NB];         // e bytes
  float sd[NB];            // their group scales d, or (NODQ) the fp32 constants
  const int lgp = SL ? __builtin_ctz(static_cast<unsigned>(KX / 8)) : 0;
  // one slice's X and constants in LDS: elements / floats per copy
  const int xcopy = M * (KX + kDecXPad), ccopy = ROWS * (KXB + 1);
  auto slice_load = [&](int set, int sg) {
    const bool any = sg < nslices;
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int idx = tid + i * kDecThreads;
      const int row = idx >> lgp, col = 8 * (idx & ((1 << lgp) - 1));
      const int gk = sg * KX + col;
      const bool ok = any && row < M && gk < K32;
      const u32x4 v = buf_load16(rx, ok ? static_cast<uint32_t>(row * K32 + gk) * 2u : kDecOffNone);
      if (set == 0) xw[i] = v; else xn[SL ? i : 0] = v;
    }
    const int row = tid % ROWS, blk = tid / ROWS;
    const int gb = sg * KXB + blk;
    const bool ok = any && blk < KXB && gb < KB;
    const uint32_t b = static_cast<uint32_t>(n0 + row) * KB + gb;   // rows past N: zeros
    if constexpr (NODQ) {
      sd[set] = buf_load_f32(rd, ok ? b * 4u : kDecOffNone);
    } else {
      se[set] = buf_load_u8(re, ok ? b : kDecOffNone);
      sd[set] = buf_load_f32(rd, ok ? (b / kGroup) * 4u : kDecOffNone);
    }
  };
  auto slice_store = [&](int set, int copy) {
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int idx = tid + i * kDecThreads;
      const int row = idx >> lgp, col = 8 * (idx & ((1 << lgp) - 1));
      if (row < M)
        *reinterpret_cast<u32x4*>(xs + copy * xcopy + row * (KX + kDecXPad) + col) =
            set == 0 ? xw[i] : xn[SL ? i : 0];
    }
    if (tid < ROWS * KXB)
      csc[copy * ccopy + tid] = NODQ ? sd[set] : static_cast<float>(se[set]) * sd[set];
  };
  if constexpr (SL) slice_load(0, 0);
  // T for the LoRA update, used only after the main loop.  With nz > 0, the
  // 16-lane row h sums quad h (4 ranks of one token) over the partials, lane
  // z loading partials z + 16 i; with nz == 0 T is final and the lanes of the
  // LoRA waves load their own 8 values of it (the first two loads).
  const int nsteps = (r + 31) / 32;
  const int nq = M * r / 4;
  // summed after the main loop: more T values than the 16-lane rows take,
  // or more partials than their registers hold
  const bool late_fold = nz > 0 && (M * r > kDecTSumMaxMR || nz > 16 * dec_tq(FR, SL));
  const int hr = tid >> 4, hl = tid & 15;
  constexpr int TQ = dec_tq(FR, SL);
  f32x4 tq[TQ];
  {
    // (one load sequence for both cases: a branch here would make the
    // compiler wait for the loads of one side before those of the other)
    const BufRes rt =
        make_bufres(T, static_cast<uint32_t>(nz > 0 ? nz * M * r : M * ldt) * 4u);
    const int j = 32 * kw + 8 * g;
    const bool lora_lane = kw < nsteps && li < M && j < r;
#pragma unroll
    for (int i = 0; i < TQ; ++i) {
      const int z = hl + 16 * i;
      const bool ok = nz > 0 ? (!late_fold && hr < nq && z < nz) : (lora_lane && i < 2);
      const int idx = nz > 0 ? z * M * r + 4 * hr : li * ldt + j + 4 * i;
      tq[i] = __builtin_bit_cast(
          f32x4, buf_load16(rt, ok ? static_cast<uint32_t>(idx * 4) : kDecOffNone));
    }
  }
  // The workgroup's 32 columns of B [r][N] (one 16-byte piece per thread for
  // r <= 256), staged in LDS for the LoRA update after the main loop.
  u32x4 bpiece;
  {
    const BufRes rbl = make_bufres(Bl, static_cast<uint32_t>(r) * static_cast<uint32_t>(ldb) * 2u);
    const int j = tid >> 2, c = tid & 3;
    const bool ok = j < r && n0 + 8 * c < N;
    bpiece = buf_load16(rbl, ok ? static_cast<uint32_t>((j * ldb + n0 + 8 * c) * 2) : kDecOffNone);
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
  // k offset (inside a chunk) of the 8 codes lane group g supplies to MFMA 0
  // of a chunk (MFMA i takes the 8 after 8 i more).
  const int xo0 = 32 * g;
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
        xv[st][i] = buf_load16(rx, live ? xb + 256u * KS * t + 16u * i : kDecOffNone);
    }
  };
#pragma unroll
  for (int u = 0; u < D; ++u) load(u, u);

  // Stage into LDS: level table, X, block scales, B.
  build_rep_pair_table<kDecThreads>(tab, lv, tid);
  if constexpr (SL) {
    slice_store(0, 0);
    if (tid < kDecXZero / 16)
      *reinterpret_cast<u32x4*>(xs + NB * xcopy + 8 * tid) = u32x4{0, 0, 0, 0};
    if (tid < NB * M)   // row padding of each copy
      *reinterpret_cast<u32x4*>(xs + (tid / M) * xcopy + (tid % M) * (KX + kDecXPad) + KX) =
          u32x4{0, 0, 0, 0};
    if (tid < NB * ROWS) csc[(tid / ROWS) * ccopy + KXB * ROWS + tid % ROWS] = 0.f;
    slice_load(1, 1);   // slices 1 and 2 in flight (sets 1 and 0)
    slice_load(0, 2);
  } else if constexpr (XLDS) {
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
  for (int i = 0; i < (SL ? 0 : kDecEPieces); ++i) {
    const int idx = tid + i * kDecThreads;
    if (8 * idx < erange) {
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const int f = 8 * idx + b;   // row-major index: row f / KB, column f % KB
        const int row = static_cast<int>((static_cast<float>(f) + 0.5f) * inv_kb);
        float c;
        if constexpr (NODQ) {
          // (the element is converted to a plain value first: this compiler
          // reads element 0 when __builtin_bit_cast is given a vector
          // element directly)
          c = __builtin_bit_cast(float, static_cast<uint32_t>(cv[NODQ ? i : 0][b / 4][b % 4]));
        } else {
          const uint32_t w = b < 4 ? ev[i].x : ev[i].y;
          c = static_cast<float>((w >> (8 * (b % 4))) & 0xFFu) * dv[i];
        }
        csc[(f - row * KB) * ROWS + row] = c;
      }
    }
  }
  if (!SL && tid < ROWS) csc[KB * ROWS + tid] = 0.f;
  if ((tid >> 2) < r) reinterpret_cast<u32x4*>(bst)[tid] = bpiece;

  // Lanes past M read X from the zero bytes with stride 0.  Past K (the
  // second block of a chunk when K % 128 == 64) the X reads of lanes 32-63
  // stay inside the next token row or the zero bytes, and their weights are
  // zero: their block constant is the zero column KB.
  const int xrow = KX + kDecXPad;
  const uint16_t* xlane = li < M ? xs + li * xrow + xo0 : xs + NB * M * xrow + xo0;
  const int xstep = li < M ? 128 : 0;
  const int xcstep = li < M ? xcopy : 0;   // (SL) to the second LDS copy
  // block constant of the lane's row li and block 2 c + g / 2: + 16 fragment
  const float* clane = csc + (g >> 1) * ROWS + li;
  // Table addresses: the lane's copy offset in byte 0, entry in byte 1.  The
  // kernel declares no static LDS, so the dynamic block, and the table at its
  // start, begins at LDS address 0 and the address needs no base added.
  const uint32_t ta = rep_lane_base(lane);

  f32x4 acc[FR];
#pragma unroll
  for (int f = 0; f < FR; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
  // All LDS reads of a fragment's chunk (block constant, table lookups, X)
  // are issued before any of their products, so one LDS round trip serves
  // its MFMAs; with two fragments a wave (X from global memory) takes them
  // one after the other, which keeps the lookups of one in registers.
  int cbase = 0;   // (SL) first chunk of the slice
  auto compute = [&](int t, int st) {
    const int c = kw + KS * t - cbase;   // chunk, counted from the first in LDS
    const int cp = SL ? st : 0;          // (SL) LDS copy: slice t in copy t % 2
    u32x4 xf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (XLDS)
        xf[i] = *reinterpret_cast<const u32x4*>(xlane + cp * xcstep + c * xstep + 8 * i);
      else
        xf[i] = xv[st][i];
    }
#pragma unroll
    for (int f = 0; f < FR; ++f) {
      const float ch = clane[cp * ccopy + 16 * frag(f) + 2 * c * ROWS];
      f32x2 v[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = cw[st][f][i];
        v[i][0] = rep_lookup<0>(ta, w);
        v[i][1] = rep_lookup<1>(ta, w);
        v[i][2] = rep_lookup<2>(ta, w);
        v[i][3] = rep_lookup<3>(ta, w);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x4 a;
#pragma unroll
        for (int b = 0; b < 4; ++b) a[b] = pack_bf16x2(v[i][b].x * ch, v[i][b].y * ch);
        acc[f] = mfma16(a, xf[i], acc[f]);
      }
    }
  };
  __syncthreads();
  if constexpr (SL) {
    // Slice t (chunk t of every wave) is read from copy t % 2.  After the
    // barrier that ends slice t - 1, slice t + 1 (in registers since two
    // slices ago) is stored into the other copy, which slice t - 1 used,
    // and slice t + 3 is loaded into the freed registers.
    for (int sg = 0; sg < nslices; sg += 2) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int t = sg + u;
        if (t > 0) __syncthreads();
        if (t + 1 < nslices) slice_store(1 - u, 1 - u);
        slice_load(1 - u, t + 3);
        cbase = t * KS;
        if (t < nmine) compute(t, u);
        load(t + D, u);
      }
    }
  } else {
    for (int t0 = 0; t0 < nmine; t0 += D) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        const int t = t0 + u;
        if (t < nmine) compute(t, u);
        load(t + D, u);
      }
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
  if (late_fold) {
    // one T value per thread, its nz partials added in partial order
    // (deterministic)
    const int mr = M * r;
    const BufRes rt = make_bufres(T, static_cast<uint32_t>(nz * mr) * 4u);
    if (tid < mr) {
      // 16 loads in flight at a time; partials past nz read as zero, and
      // adding zero leaves the sum (never -0 here) as it was
      float t = 0.f;
      for (int z0 = 0; z0 < nz; z0 += 16) {
        float pz[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
          pz[i] = buf_load_f32(rt, z0 + i < nz ? static_cast<uint32_t>((z0 + i) * mr + tid) * 4u
                                               : kDecOffNone);
#pragma unroll
        for (int i = 0; i < 16; ++i) t += pz[i];
      }
      reinterpret_cast<float*>(tfin)[tid] = t;
      if (blockIdx.x == 0) Tout[tid] = t;   // [M][r]
    }
  } else if (nz > 0) {
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
      *reinterpret_cast<u32x2*>(Y + (int64_t)li * ldy + nout) =
          u32x2{pack_bf16x2(t.x, t.y), pack_bf16x2(t.z, t.w)};
    }
  }
}

namespace {

template <int D, int XP, int FR, bool NODQ, bool SL = false>
hipError_t launch_decode_variant(const uint16_t* X, int64_t M, const Nf4View& w, const float* T,
                                 int nz, float* Tout, const uint16_t* B, int r, float s,
                                 uint16_t* Y, const Nf4Tables& tb, hipStream_t stream, int ldt,
                                 int ldb, int ldy, int ksl = 0) {
  // allow the largest dynamic LDS (once per variant)
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&k_fwd_decode<D, XP, FR, NODQ, SL>),
      hipFuncAttributeMaxDynamicSharedMemorySize, kDecLdsMax);
  if (attr != hipSuccess) return attr;
  if (SL && ksl != 1024) return hipErrorInvalidValue;
  const DecLds L(M, w.K, r, XP > 0, FR, ksl, SL ? 2 : 1);
  if (L.total > kDecLdsMax || nz > kMaxDownPartials) return hipErrorInvalidValue;
  const unsigned grid = static_cast<unsigned>((w.N + kDecRows - 1) / kDecRows);
  const float inv_kb = 1.0f / static_cast<float>(w.K / kBlock);
  hipLaunchKernelGGL((k_fwd_decode<D, XP, FR, NODQ, SL>), dim3(grid), dim3(kDecThreads), L.total,
                     stream, X, (int)M, w.codes, w.absmax_q, w.absmax_scale, w.N, w.K, T, nz, Tout,
                     B, r, s, Y, tb, L.boff, L.toff, L.coff, L.xoff, inv_kb, ldt, ldb, ldy, ksl);
  return hipGetLastError();
}

bool decode_x_in_lds(int64_t M, int64_t K, int r) {
  return M * K * 2 <= kDecXLdsBytes && DecLds(M, K, r, true).total <= kDecLdsMax;
}

// Slice width for X in K-slices: 1024 columns in two LDS copies when they
// fit (always, for M <= 16), else 0.
int decode_slice(int64_t M, int64_t K, int r) {
  constexpr int ksl = 1024;
  return M * ksl * 2 <= kDecXLdsBytes / 2 && DecLds(M, K, r, true, 1, ksl, 2).total <= kDecLdsMax
             ? ksl : 0;
}

}  // namespace

bool decode_fits(int64_t M, int64_t K) { return M <= 16 && K <= kDecMaxK; }

bool decode_folds_t(int64_t M, int r) {
  return r > 0 && M * r <= kDecTFinMaxMR;
}

hipError_t launch_fwd_decode(const uint16_t* X, int64_t M, const Nf4View& w,
                             const float* T, int nz, float* Tout, const uint16_t* B, int r,
                             float s, uint16_t* Y, const Nf4Tables& tb, hipStream_t stream,
                             int ldt, int64_t ldb, int64_t ldy) {
  if (ldt <= 0) ldt = r;
  if (ldb <= 0) ldb = w.N;
  if (ldy <= 0) ldy = w.N;
  prof_begin(2, stream);
  // Two chunks in flight per wave: with all 16 waves of every CU streaming,
  // deeper rings (measured up to 8) only delay the first products.
  // X goes to LDS when it fits next to the rest (M = 1 up to K = 22016 with
  // r <= 64; M = 4 up to K = 8192), in as few 16-byte pieces per thread as it
  // needs.  Otherwise, for more than 8 tokens, in K-slices: each wave's X
  // loads from global memory touch one cache line per token, and at M = 16
  // the sliced form runs 36 against 46 us at 8192 x 22016; with 4 tokens
  // (single-copy 4096-column slices) it was the slower one (37 against 34 us).
  auto run = [&](auto nodq) {
    constexpr bool ND = decltype(nodq)::value;
    const int lb = static_cast<int>(ldb), ly = static_cast<int>(ldy);
    if (decode_x_in_lds(M, w.K, r)) {
      const int64_t xbytes = M * w.K * 2;
      const int64_t per_piece = 16 * kDecThreads;
      if (xbytes <= per_piece)
        return launch_decode_variant<2, 1, 1, ND>(X, M, w, T, nz, Tout, B, r, s, Y, tb, stream,
                                                  ldt, lb, ly);
      if (xbytes <= 2 * per_piece)
        return launch_decode_variant<2, 2, 1, ND>(X, M, w, T, nz, Tout, B, r, s, Y, tb, stream,
                                                  ldt, lb, ly);
      return launch_decode_variant<2, kDecXPieces, 1, ND>(X, M, w, T, nz, Tout, B, r, s, Y, tb,
                                                          stream, ldt, lb, ly);
    }
    if (M > 8 && decode_slice(M, w.K, r) == 1024)
      return launch_decode_variant<2, 2, 1, ND, true>(X, M, w, T, nz, Tout, B, r, s, Y, tb, stream,
                                                      ldt, lb, ly, 1024);
    // X from global memory: each wave works on both fragments, so each X
    // piece it loads serves 32 rows.
    return launch_decode_variant<2, 0, 2, ND>(X, M, w, T, nz, Tout, B, r, s, Y, tb, stream, ldt,
                                              lb, ly);
  };
  const hipError_t e =
      w.dq ? run(std::false_type{}) : run(std::true_type{});
  prof_end(2, stream);
  return e;
}

static_assert(kRepTabBytes + 64 * kDecMaxR + kDecTFinMaxMR * 4 +
                      kDecRows * (kDecMaxK / kBlock + 1) * 4 <= kDecLdsMax,
              "block scales of the largest K fit next to the table without X");

}  // namespace qnf4
