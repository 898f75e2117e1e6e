// MFMA GEMMs of the QLoRA NF4 linear layer on gfx950.
//
// The rank-r products (T = X.A, G = dY.B^T, dA, dB) have the form C[q, p] = sum_k P[p, k] . Q[q, k]: the
// workgroup stages a P tile (BP rows x 64 reduction elements) and a Q tile
// (BQ x 64) in LDS, and four waves (2 x 2) accumulate their (BP/2 x BQ/2)
// share with v_mfma_f32_16x16x32_bf16.  Each loader fixes its tile's LDS
// layout and how a lane reads its 8 reduction elements from it:
//   Bf16Nat  bf16 rows, reduction contiguous (X and dY of T and G, B as [r,N])
//   Bf16RedMajor / F32RedMajor  reduction-major tiles kept as they lie in
//            memory and read with transposing LDS reads (A as [K,r]; X, dY,
//            G, T of dA and dB); fp32 sources are split into bf16 hi and lo
//            passes, so the fp32 factor keeps ~16 bits through the bf16 MFMA
// The weight-streaming GEMMs (forward and dX) have kernels of their own.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace qnf4 {

constexpr int BK = 64;              // reduction elements per tile
constexpr int LDS_STRIDE = BK + 8;  // bf16 per LDS row: 144 B, spreads rows over banks
constexpr int NT = 256;             // threads per workgroup (4 waves)

struct OpParams {
  const void* ptr;
  int64_t ld;      // leading dimension of the source array (elements)
  int64_t nrows;   // extent of the tile-row index
  int64_t nred;    // extent of the reduction index
  float scale;     // fp32 sources: value = scale * src
};

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st_lds16(uint16_t* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// ---------------------------------------------------------------------------
// Loaders.  load(kt) fetches reduction tile kt into registers; store(lds)
// writes the tile [ROWS][LDS_STRIDE] to LDS; elements outside the operand
// are zero.
// ---------------------------------------------------------------------------

template <int ROWS>
struct Bf16Nat {   // element (row, k) = src[row * ld + k]
  static constexpr int TILE = ROWS * LDS_STRIDE;
  __device__ static u32x4 frag(const uint16_t* tile, int c0, int ks, int lane) {
    return *reinterpret_cast<const u32x4*>(tile + (c0 + (lane & 15)) * LDS_STRIDE + 32 * ks +
                                           8 * (lane >> 4));
  }
  static constexpr int CH = ROWS * BK / 8;              // 16-byte chunks
  static constexpr int CPT = (CH + NT - 1) / NT;
  OpParams o;
  int64_t row0;
  u32x4 r[CPT];
  __device__ void load(int kt, int tid) {
    const uint16_t* src = static_cast<const uint16_t*>(o.ptr);
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + c * NT;
      const int row = idx >> 3, kc = idx & 7;
      const int64_t gr = row0 + row, gk = (int64_t)kt * BK + kc * 8;
      r[c] = (idx < CH && gr < o.nrows && gk < o.nred) ? ld16(src + gr * o.ld + gk)
                                                        : u32x4{0, 0, 0, 0};
    }
  }
  __device__ void store(uint16_t* lds, int tid) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + c * NT;
      if (idx < CH) st_lds16(lds + (idx >> 3) * LDS_STRIDE + (idx & 7) * 8, r[c]);
    }
  }
};

// ---------------------------------------------------------------------------
// Reduction-major operands (element (row, k) = src[k * ld + row]: X^T, dY^T,
// and the fp32 G^T, T^T of the adapter gradients).  The tile is stored as it
// lies in memory, [BK reduction rows][COLS] (coalesced 16-byte loads, no
// register transposes), and the MFMA fragment -- 8 consecutive reduction
// elements of one row per lane -- is read with ds_read_b64_tr_b16, which
// transposes 4 x 16 blocks of 16-bit elements across each 16-lane group.
// 16-byte pieces are XOR-swizzled in 32-byte units so the 8 tile rows of a
// half-wave transposing read (rows 8g + 4e + i, g = 0, 1) hit distinct banks.
// ---------------------------------------------------------------------------

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 LdsV4i16;

template <int COLS>
__device__ __forceinline__ int rm_slot(int row, int piece) {
  static_assert(COLS == 64 || COLS == 128, "tile width");
  const int f = COLS == 64 ? (((row >> 1) & 1) | (((row >> 3) & 1) << 1))   // 128-byte rows
                           : ((row & 3) | (((row >> 3) & 1) << 2));          // 256-byte rows
  return piece ^ (2 * f);
}

// Fragment of tile rows (columns) c0 .. c0+15, reduction step ks.
template <int COLS>
__device__ __forceinline__ u32x4 rm_frag(const uint16_t* tile, int c0, int ks, int lane) {
  const int li = lane & 15, g = lane >> 4;
  const int col = c0 + 4 * (li & 3);
  u32x2 h[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int red = 32 * ks + 8 * g + 4 * e + (li >> 2);
    const uint16_t* p = tile + red * COLS + 8 * rm_slot<COLS>(red, col >> 3) + (col & 7);
    h[e] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LdsV4i16*)(p)));
  }
  return u32x4{h[0][0], h[0][1], h[1][0], h[1][1]};
}

template <int COLS>
struct Bf16RedMajor {   // element (row, k) = src[k * ld + row], bf16
  static constexpr int TILE = BK * COLS;
  static constexpr int PCS = COLS / 8;                 // 16-byte pieces per tile row
  static constexpr int CPT = BK * PCS / NT;            // pieces a thread
  OpParams o;
  int64_t row0;
  u32x4 r[CPT];
  __device__ void load(int kt, int tid) {
    const uint16_t* src = static_cast<const uint16_t*>(o.ptr);
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + c * NT, red = idx / PCS, pc = idx % PCS;
      const int64_t gk = (int64_t)kt * BK + red, gr = row0 + 8 * pc;
      r[c] = (gk < o.nred && gr < o.nrows) ? ld16(src + gk * o.ld + gr) : u32x4{0, 0, 0, 0};
    }
  }
  __device__ void store(uint16_t* lds, int tid) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + c * NT, red = idx / PCS, pc = idx % PCS;
      st_lds16(lds + red * COLS + 8 * rm_slot<COLS>(red, pc), r[c]);
    }
  }
  __device__ static u32x4 frag(const uint16_t* tile, int c0, int ks, int lane) {
    return rm_frag<COLS>(tile, c0, ks, lane);
  }
};

template <int COLS>
struct F32RedMajor {    // element (row, k) = scale * src[k * ld + row], fp32 -> bf16 hi, lo
  static constexpr int TILE = BK * COLS;
  static constexpr int QCS = COLS / 4;                 // 4-float pieces per tile row
  static constexpr int CPT = BK * QCS / NT;
  OpParams o;
  int64_t row0;
  f32x4 r[CPT];
  __device__ void load(int kt, int tid) {
    const float* src = static_cast<const float*>(o.ptr);
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + c * NT, red = idx / QCS, qc = idx % QCS;
      const int64_t gk = (int64_t)kt * BK + red, gr = row0 + 4 * qc;
      r[c] = (gk < o.nred && gr < o.nrows) ? *reinterpret_cast<const f32x4*>(src + gk * o.ld + gr)
                                           : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  __device__ void store2(uint16_t* hi, uint16_t* lo, int tid) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + c * NT, red = idx / QCS, qc = idx % QCS;
      uint32_t h0, l0, h1, l1;
      split_bf16x2(r[c].x * o.scale, r[c].y * o.scale, h0, l0);
      split_bf16x2(r[c].z * o.scale, r[c].w * o.scale, h1, l1);
      const int off = red * COLS + 8 * rm_slot<COLS>(red, qc >> 1) + 4 * (qc & 1);
      *reinterpret_cast<u32x2*>(hi + off) = u32x2{h0, h1};
      *reinterpret_cast<u32x2*>(lo + off) = u32x2{l0, l1};
    }
  }
  __device__ static u32x4 frag(const uint16_t* tile, int c0, int ks, int lane) {
    return rm_frag<COLS>(tile, c0, ks, lane);
  }
};

// ---------------------------------------------------------------------------
// MFMA tile step and the double-buffered tile loop
// ---------------------------------------------------------------------------

template <int BP, int BQ>
struct Mma {
  static constexpr int TP = BP / 32, TQ = BQ / 32;   // 16x16 tiles per wave
  f32x4 acc[TP][TQ];
  __device__ void zero() {
#pragma unroll
    for (int i = 0; i < TP; ++i)
#pragma unroll
      for (int j = 0; j < TQ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // FP, FQ: the operands' tile layouts (their loaders' frag readers)
  template <class FP, class FQ>
  __device__ void step(const uint16_t* ldsP, const uint16_t* ldsQ, int wave, int lane) {
    const int wp = (wave & 1) * (BP / 2), wq = (wave >> 1) * (BQ / 2);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      u32x4 a[TP], b[TQ];
#pragma unroll
      for (int i = 0; i < TP; ++i) a[i] = FP::frag(ldsP, wp + 16 * i, ks, lane);
#pragma unroll
      for (int j = 0; j < TQ; ++j) b[j] = FQ::frag(ldsQ, wq + 16 * j, ks, lane);
#pragma unroll
      for (int i = 0; i < TP; ++i)
#pragma unroll
        for (int j = 0; j < TQ; ++j) acc[i][j] = mfma16(a[i], b[j], acc[i][j]);
    }
  }
};

// Runs reduction tiles [kt0, kt1) through two LDS buffers with a ring of D
// register stages (tiles are loaded D ahead; a depth of 4 measured no faster
// than 2 for these memory-light tiles).  HL selects
// an fp32 operand split into bf16 hi and lo halves (1: P, 2: Q): both halves
// are staged per tile and multiplied against the other operand, which is
// loaded once.  Buffer layout: [P or P_hi][Q or Q_hi][second half].
template <int BP, int BQ, int HL, int D, class LP, class LQ>
__device__ void run_tiles(const LP& lp0, const LQ& lq0, int kt0, int kt1, Mma<BP, BQ>& mma,
                          uint16_t* lds, int tid) {
  static_assert(D % 2 == 0, "the ring depth keeps the LDS buffer of a slot fixed");
  if (kt0 >= kt1) return;
  constexpr int XT = HL == 0 ? 0 : (HL == 1 ? LP::TILE : LQ::TILE);   // the extra (lo) tile
  constexpr int BUF = LP::TILE + LQ::TILE + XT;
  const int wave = wave_id(), lane = tid & 63;
  LP lp[D];
  LQ lq[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    lp[d] = lp0;
    lq[d] = lq0;
  }
  auto P = [&](int b) { return lds + b * BUF; };
  auto Q = [&](int b) { return lds + b * BUF + LP::TILE; };
  auto X = [&](int b) { return lds + b * BUF + LP::TILE + LQ::TILE; };
  auto load = [&](int t, int d) {
    if (t < kt1) {
      lp[d].load(t, tid);
      lq[d].load(t, tid);
    }
  };
  auto store = [&](int d, int b) {
    if constexpr (HL == 0) {
      lp[d].store(P(b), tid);
      lq[d].store(Q(b), tid);
    } else if constexpr (HL == 1) {
      lp[d].store2(P(b), X(b), tid);
      lq[d].store(Q(b), tid);
    } else {
      lp[d].store(P(b), tid);
      lq[d].store2(Q(b), X(b), tid);
    }
  };
  auto step = [&](int b) {
    mma.template step<LP, LQ>(P(b), Q(b), wave, lane);
    if constexpr (HL == 1) mma.template step<LP, LQ>(X(b), Q(b), wave, lane);
    if constexpr (HL == 2) mma.template step<LP, LQ>(P(b), X(b), wave, lane);
  };
  // tile t lives in register slot (t - kt0) % D and LDS buffer (t - kt0) % 2
#pragma unroll
  for (int d = 0; d < D; ++d) load(kt0 + d, d);
  store(0, 0);
  load(kt0 + D, 0);
  __syncthreads();
  for (int kt = kt0; kt < kt1; kt += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int t = kt + u;
      if (t < kt1) {
        step(u & 1);
        if (t + 1 < kt1) {
          store((u + 1) % D, (u & 1) ^ 1);
          load(t + 1 + D, (u + 1) % D);
        }
        __syncthreads();
      }
    }
  }
}

// Stores C[q, p] as bf16 (lane holds 4 consecutive p of one q per tile).
template <int BP, int BQ>
__device__ void store_bf16(const Mma<BP, BQ>& mma, uint16_t* out, int64_t ldo,
                           int64_t p0, int64_t q0, int64_t P, int64_t Q, int tid) {
  const int wave = wave_id(), lane = tid & 63;
  const int64_t wp = p0 + (wave & 1) * (BP / 2) + 4 * (lane >> 4);
  const int64_t wq = q0 + (wave >> 1) * (BQ / 2) + (lane & 15);
#pragma unroll
  for (int i = 0; i < Mma<BP, BQ>::TP; ++i)
#pragma unroll
    for (int j = 0; j < Mma<BP, BQ>::TQ; ++j) {
      const int64_t p = wp + 16 * i, q = wq + 16 * j;
      if (p < P && q < Q) {   // P % 4 == 0, so the 4 values are all in range
        const f32x4 v = mma.acc[i][j];
        *reinterpret_cast<u32x2*>(out + q * ldo + p) =
            u32x2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
      }
    }
}

template <int BP, int BQ>
__device__ void store_f32(const Mma<BP, BQ>& mma, float* out, int64_t ldo,
                          int64_t p0, int64_t q0, int64_t P, int64_t Q, int tid) {
  const int wave = wave_id(), lane = tid & 63;
  const int64_t wp = p0 + (wave & 1) * (BP / 2) + 4 * (lane >> 4);
  const int64_t wq = q0 + (wave >> 1) * (BQ / 2) + (lane & 15);
#pragma unroll
  for (int i = 0; i < Mma<BP, BQ>::TP; ++i)
#pragma unroll
    for (int j = 0; j < Mma<BP, BQ>::TQ; ++j) {
      const int64_t p = wp + 16 * i, q = wq + 16 * j;
      if (p < P && q < Q) *reinterpret_cast<f32x4*>(out + q * ldo + p) = mma.acc[i][j];
    }
}

// ---------------------------------------------------------------------------
// Rank-r products with a split reduction: partial sums of C[q, p] for
// reduction tiles [z*tps, (z+1)*tps) go to ws[z][q][p]; a second kernel sums
// the partials in split order (deterministic) and writes the result.
// ---------------------------------------------------------------------------

// HL: 0 = both operands bf16; 1 = P is fp32 (hi/lo); 2 = Q is fp32 (hi/lo).
template <int BP, int BQ, class LP, class LQ, int HL>
struct RankKind {
  static constexpr int XT = HL == 0 ? 0 : (HL == 1 ? LP::TILE : LQ::TILE);
  static constexpr int LDS = 2 * (LP::TILE + LQ::TILE + XT);   // bf16 elements
};

// One product: tile (x, y) of C and reduction split z.
struct RankJob {
  OpParams po, qo;
  int ntiles, tps;
  float* ws;
  int64_t P, Q;
  int px, qy, nblk;   // tiles along P and Q; workgroups (px qy splits)
};

template <int BP, int BQ, class LP, class LQ, int HL>
__device__ __forceinline__ void rank_tile(const RankJob& j, int x, int y, int z, uint16_t* lds,
                                          int tid) {
  const int64_t p0 = (int64_t)x * BP, q0 = (int64_t)y * BQ;
  const int kt0 = z * j.tps, kt1 = min(j.ntiles, kt0 + j.tps);
  Mma<BP, BQ> mma;
  mma.zero();
  LP lp{j.po, p0};
  LQ lq{j.qo, q0};
  run_tiles<BP, BQ, HL, 2>(lp, lq, kt0, kt1, mma, lds, tid);
  store_f32(mma, j.ws + (int64_t)z * j.P * j.Q, j.P, p0, q0, j.P, j.Q, tid);
}

template <int BP, int BQ, class LP, class LQ, int HL>
__global__ __launch_bounds__(NT) void k_rank(RankJob j) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[RankKind<BP, BQ, LP, LQ, HL>::LDS];
  rank_tile<BP, BQ, LP, LQ, HL>(j, blockIdx.x, blockIdx.y, blockIdx.z, lds, threadIdx.x);
}

// Two independent products in one launch (workgroups [0, a.nblk) run the
// first, the rest the second), so they share the machine instead of running
// one after the other.
template <int BPA, int BQA, class LPA, class LQA, int HLA, int BPB, int BQB, class LPB, class LQB,
          int HLB>
__global__ __launch_bounds__(NT) void k_rank_pair(RankJob a, RankJob b) {
  constexpr int LA = RankKind<BPA, BQA, LPA, LQA, HLA>::LDS;
  constexpr int LB = RankKind<BPB, BQB, LPB, LQB, HLB>::LDS;
  __shared__ __attribute__((aligned(16))) uint16_t lds[LA > LB ? LA : LB];
  int blk = blockIdx.x;   // uniform: the branch is a scalar one
  if (blk < a.nblk) {
    rank_tile<BPA, BQA, LPA, LQA, HLA>(a, blk % a.px, (blk / a.px) % a.qy, blk / (a.px * a.qy),
                                       lds, threadIdx.x);
  } else {
    blk -= a.nblk;
    rank_tile<BPB, BQB, LPB, LQB, HLB>(b, blk % b.px, (blk / b.px) % b.qy, blk / (b.px * b.qy),
                                       lds, threadIdx.x);
  }
}

// out[i] = scale * sum_z ws[z][i]; fp32 or bf16 output; 4 elements a thread.
template <bool BF16_OUT>
__global__ __launch_bounds__(256) void k_split_reduce(const float* ws, int splits,
                                                      int64_t count, float scale,
                                                      void* out) {
  const int64_t i = 4 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x);
  if (i >= count) return;
  // four independent partial sums so the loads of several splits overlap;
  // the combination order is fixed, so results are deterministic
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0, s2 = s0, s3 = s0;
  int z = 0;
  for (; z + 4 <= splits; z += 4) {
    s0 += *reinterpret_cast<const f32x4*>(ws + (int64_t)(z + 0) * count + i);
    s1 += *reinterpret_cast<const f32x4*>(ws + (int64_t)(z + 1) * count + i);
    s2 += *reinterpret_cast<const f32x4*>(ws + (int64_t)(z + 2) * count + i);
    s3 += *reinterpret_cast<const f32x4*>(ws + (int64_t)(z + 3) * count + i);
  }
  for (; z < splits; ++z) s0 += *reinterpret_cast<const f32x4*>(ws + (int64_t)z * count + i);
  f32x4 s = (s0 + s1) + (s2 + s3);
  s *= scale;
  if constexpr (BF16_OUT) {
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + i) =
        u32x2{pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w)};
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + i) = s;
  }
}

// Two split reductions in one launch: blocks [0, ga) reduce the first.
struct ReduceJob {
  const float* ws;
  int splits;
  int64_t count;
  float scale;
  void* out;
  int64_t prow;   // elements per output row (a multiple of 4)
  int64_t ldo;    // output row stride (prow for a dense output)
};

template <bool BF16_A, bool BF16_B>
__global__ __launch_bounds__(256) void k_split_reduce_pair(ReduceJob a, ReduceJob b, int ga) {
  const bool first = static_cast<int>(blockIdx.x) < ga;
  const ReduceJob& j = first ? a : b;
  const int64_t i = 4 * ((int64_t)(first ? blockIdx.x : blockIdx.x - ga) * blockDim.x + threadIdx.x);
  if (i >= j.count) return;
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0, s2 = s0, s3 = s0;
  int z = 0;
  for (; z + 4 <= j.splits; z += 4) {
    s0 += *reinterpret_cast<const f32x4*>(j.ws + (int64_t)(z + 0) * j.count + i);
    s1 += *reinterpret_cast<const f32x4*>(j.ws + (int64_t)(z + 1) * j.count + i);
    s2 += *reinterpret_cast<const f32x4*>(j.ws + (int64_t)(z + 2) * j.count + i);
    s3 += *reinterpret_cast<const f32x4*>(j.ws + (int64_t)(z + 3) * j.count + i);
  }
  for (; z < j.splits; ++z) s0 += *reinterpret_cast<const f32x4*>(j.ws + (int64_t)z * j.count + i);
  f32x4 s = (s0 + s1) + (s2 + s3);
  s *= j.scale;
  const int64_t row = i / j.prow, o = row * j.ldo + (i - row * j.prow);
  if (first ? BF16_A : BF16_B) {
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(j.out) + o) =
        u32x2{pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w)};
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(j.out) + o) = s;
  }
}

// ---------------------------------------------------------------------------
// LoRA down-projection for few tokens (M <= 16): workgroup z covers spw
// consecutive slices of 128 k; partial[z][m][j] = sum over them of
// X[m, k] A[k, j].  Each A slice is transposed through LDS in 8x8 patches
// (16 KB a slice, staged by the first 128 threads), 64 ranks at a time; wave
// w multiplies ranks 16w..16w+15 of the 64 against the token fragments,
// which come straight from global memory.  128-k slices give 64 workgroups
// at K = 8192 where 256-k slices gave 32; the kernel is a short latency
// chain, so more of them in parallel end sooner (about 0.3 us per call).
// ---------------------------------------------------------------------------

constexpr int LDS_K = 128;             // k per slice
constexpr int LDS_KS = LDS_K + 8;      // LDS row stride (elements)

__global__ __launch_bounds__(256) void k_lora_down_small(const uint16_t* __restrict__ X, int M,
                                                         int64_t K, const uint16_t* __restrict__ A,
                                                         int r, int spw, float* __restrict__ ws) {
  __shared__ __attribute__((aligned(16))) uint16_t at[64 * LDS_KS];
  const int tid = threadIdx.x;
  const int wave = wave_id(), lane = tid & 63;
  const int li = lane & 15, g = lane >> 4;
  const bool m_ok = li < M;
  const int jp = tid & 7, kp = tid >> 3;   // A patch: ranks j0 + 8 jp .., k rows 8 kp ..
  const int K32 = static_cast<int>(K);     // K <= 2^22 and M K, K r < 2^30 here
  const BufRes rx = make_bufres(X, static_cast<uint32_t>(M * K32 * 2));
  const BufRes ra = make_bufres(A, static_cast<uint32_t>(K32 * r * 2));
  // Slices run as a two-stage pipeline: the loads of slice sub + 1 are in
  // flight while slice sub is transposed and multiplied.
  u32x4 xf[2][LDS_K / 32];   // token fragments for the k32 steps of a slice
  u32x4 rows[2][8];   // this thread's 8x8 patch of the slice's A rows
  for (int j0 = 0; j0 < r; j0 += 64) {
    // (buffer loads with out-of-range offsets instead of branches, so the
    // compiler can wait for one stage while the other is in flight)
    auto load = [&](int sub, int b) {   // past the workgroup's slices: reads nothing
      const int k0 = sub < spw ? (blockIdx.x * spw + sub) * LDS_K : K32;
#pragma unroll
      for (int st = 0; st < LDS_K / 32; ++st) {
        const int k = k0 + 32 * st + 8 * g;
        xf[b][st] = buf_load16(rx, m_ok && k < K ? static_cast<uint32_t>((li * K32 + k) * 2)
                                                 : 0x80000000u);
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int k = k0 + kp * 8 + t;
        const int j = j0 + jp * 8;
        const bool ok = kp * 8 < LDS_K && k < K && j < r;   // 16 threads of rows a slice
        rows[b][t] = buf_load16(ra, ok ? static_cast<uint32_t>((k * r + j) * 2) : 0x80000000u);
      }
    };
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    auto step = [&](int sub, auto bc) {
      constexpr int b = decltype(bc)::value;
      if (sub >= spw) return;   // uniform
      load(sub + 1, b ^ 1);
      u32x4 cols[8];
      transpose8x8_b16(rows[b], cols);
      if (kp * 8 < LDS_K) {   // threads past the slice's rows hold zeros
#pragma unroll
        for (int t = 0; t < 8; ++t)
          *reinterpret_cast<u32x4*>(at + (jp * 8 + t) * LDS_KS + kp * 8) = cols[t];
      }
      __syncthreads();
#pragma unroll
      for (int st = 0; st < LDS_K / 32; ++st) {
        const u32x4 af =
            *reinterpret_cast<const u32x4*>(at + (16 * wave + li) * LDS_KS + 32 * st + 8 * g);
        acc = mfma16(af, xf[b][st], acc);
      }
      __syncthreads();
    };
    load(0, 0);
    for (int sub = 0; sub < spw; sub += 2) {
      step(sub, std::integral_constant<int, 0>{});
      step(sub + 1, std::integral_constant<int, 1>{});
    }
    const int j = j0 + 16 * wave + 4 * g;
    if (m_ok && j < r)
      *reinterpret_cast<f32x4*>(ws + ((int64_t)blockIdx.x * M + li) * r + j) = acc;
  }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------

namespace {

OpParams op(const void* p, int64_t ld, int64_t nrows, int64_t nred, float scale = 1.f) {
  OpParams o{};
  o.ptr = p;
  o.ld = ld;
  o.nrows = nrows;
  o.nred = nred;
  o.scale = scale;
  return o;
}

unsigned cdiv(int64_t a, int64_t b) { return static_cast<unsigned>((a + b - 1) / b); }

struct Split {
  int ntiles, tps, splits;
};

// Split the reduction so that the grid has about one workgroup per CU, with
// at least four reduction tiles per split (fewer, larger splits keep the fp32
// partial sums small next to the operands they reduce).
Split choose_split(int64_t nred, int64_t ptiles, int64_t qtiles) {
  Split s;
  s.ntiles = static_cast<int>((nred + BK - 1) / BK);
  const int64_t want = std::max<int64_t>(1, 256 / std::max<int64_t>(1, ptiles * qtiles));
  s.tps = static_cast<int>(std::max<int64_t>(4, (s.ntiles + want - 1) / want));
  s.splits = (s.ntiles + s.tps - 1) / s.tps;
  return s;
}

RankJob job(const OpParams& po, const OpParams& qo, const Split& sp, float* ws, int64_t P,
            int64_t Q, int64_t px, int64_t qy) {
  RankJob j;
  j.po = po;
  j.qo = qo;
  j.ntiles = sp.ntiles;
  j.tps = sp.tps;
  j.ws = ws;
  j.P = P;
  j.Q = Q;
  j.px = static_cast<int>(px);
  j.qy = static_cast<int>(qy);
  j.nblk = static_cast<int>(px * qy * sp.splits);
  return j;
}

template <bool BF16>
hipError_t reduce(const float* ws, int splits, int64_t count, float scale, void* out,
                  hipStream_t stream) {
  const unsigned grid = cdiv(count / 4, 256);
  hipLaunchKernelGGL(k_split_reduce<BF16>, dim3(grid), dim3(256), 0, stream, ws, splits,
                     count, scale, out);
  return hipGetLastError();
}

constexpr int RB_R = 64;     // tile of the rank dimension
constexpr int RB_X = 128;    // tile of the long dimension

}  // namespace

GemmSplit gemm_split(int64_t tiles, int64_t nchunks) {
  GemmSplit g{1, static_cast<int>(nchunks)};
  // Only when the tiles would fill under three quarters of the 256 CUs, and
  // with at least 8 chunks per split (the partials cost a pass of their own).
  if (tiles >= 192 || nchunks < 16) return g;
  const int64_t want = std::min<int64_t>(256 / tiles, nchunks / 8);
  if (want < 2) return g;
  int64_t cps = (nchunks + want - 1) / want;
  cps += cps & 1;   // whole pairs of chunks
  g.splits = static_cast<int>((nchunks + cps - 1) / cps);
  g.cps = static_cast<int>(cps);
  return g;
}

hipError_t launch_split_reduce_bf16(const float* part, int splits, int64_t count, uint16_t* out,
                                    hipStream_t stream) {
  return reduce<true>(part, splits, count, 1.f, out, stream);
}

size_t rank_ws_floats(int64_t M, int64_t N, int64_t K, int r) {
  if (r <= 0) return 0;
  if (M <= 16)
    return (size_t)lora_down_partial_count(K, kMaxDownPartials) * M * r +
           rank_ws_floats(17, N, K, r);
  const int64_t rt = (r + RB_R - 1) / RB_R;
  const Split t = choose_split(K, rt, (M + RB_X - 1) / RB_X);
  const Split g = choose_split(N, rt, (M + RB_X - 1) / RB_X);
  const Split a = choose_split(M, rt, (K + RB_X - 1) / RB_X);
  const Split b = choose_split(M, (N + RB_X - 1) / RB_X, rt);
  size_t m = 0;
  m = std::max<size_t>(m, (size_t)t.splits * M * r);
  m = std::max<size_t>(m, (size_t)g.splits * M * r + (size_t)b.splits * r * N);   // together
  m = std::max<size_t>(m, (size_t)a.splits * K * r);
  return m;
}

size_t lora_down_ws_floats(int64_t M, int64_t K, int r) {
  if (r <= 0) return 0;
  if (M <= 16) return (size_t)lora_down_partial_count(K, kMaxDownPartials) * M * r;
  const Split t = choose_split(K, (r + RB_R - 1) / RB_R, (M + RB_X - 1) / RB_X);
  return (size_t)t.splits * M * r;
}

int lora_down_partial_count(int64_t K, int maxp) {
  const int64_t slices = (K + LDS_K - 1) / LDS_K;
  const int64_t spw = (slices + maxp - 1) / maxp;
  return static_cast<int>((slices + spw - 1) / spw);
}

hipError_t launch_lora_down_partials(const uint16_t* X, int64_t M, int64_t K, const uint16_t* A,
                                     int r, int maxp, float* ws, int* nz, hipStream_t stream) {
  if (maxp < 1 || maxp > kMaxDownPartials) return hipErrorInvalidValue;
  const int64_t slices = (K + LDS_K - 1) / LDS_K;
  const int spw = static_cast<int>((slices + maxp - 1) / maxp);
  *nz = lora_down_partial_count(K, maxp);
  prof_begin(4, stream);
  hipLaunchKernelGGL(k_lora_down_small, dim3(*nz), dim3(256), 0, stream, X, (int)M, K, A, r, spw,
                     ws);
  prof_end(4, stream);
  return hipGetLastError();
}

hipError_t launch_lora_down(const uint16_t* X, int64_t M, int64_t K, const uint16_t* A,
                            int r, float* T, float* ws, hipStream_t stream) {
  if (M <= 16) {
    int nz = 0;
    hipError_t e = launch_lora_down_partials(X, M, K, A, r, kMaxDownPartials / 2, ws, &nz, stream);
    if (e == hipSuccess) {
      prof_begin(4, stream);
      e = reduce<false>(ws, nz, M * r, 1.f, T, stream);
      prof_end(4, stream);
    }
    return e;
  }
  const int64_t pt = (r + RB_R - 1) / RB_R, qt = (M + RB_X - 1) / RB_X;
  const Split sp = choose_split(K, pt, qt);
  prof_begin(4, stream);
  hipLaunchKernelGGL((k_rank<RB_R, RB_X, Bf16RedMajor<RB_R>, Bf16Nat<RB_X>, 0>),
                     dim3(pt, qt, sp.splits), dim3(NT), 0, stream,
                     job(op(A, r, r, K), op(X, K, M, K), sp, ws, r, M, pt, qt));
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = reduce<false>(ws, sp.splits, M * r, 1.f, T, stream);
  prof_end(4, stream);
  return e;
}

hipError_t launch_grad_in_and_b(const uint16_t* dY, int64_t M, int64_t N, const uint16_t* B,
                                const float* T, int r, float s, float* G, uint16_t* dB,
                                float* ws, hipStream_t stream, int64_t ldy, int64_t ldb,
                                int ldt) {
  if (ldy <= 0) ldy = N;
  if (ldb <= 0) ldb = N;
  if (ldt <= 0) ldt = r;
  // G = dY . B^T: tiles (ranks, tokens), split over N
  const int64_t gpt = (r + RB_R - 1) / RB_R, gqt = (M + RB_X - 1) / RB_X;
  const Split gs = choose_split(N, gpt, gqt);
  // dB partials: tiles (N, ranks), split over M; after G's partials in ws
  const int64_t bpt = (N + RB_X - 1) / RB_X, bqt = (r + RB_R - 1) / RB_R;
  const Split bs = choose_split(M, bpt, bqt);
  float* wsb = ws + (size_t)gs.splits * M * r;
  const RankJob jg = job(op(B, ldb, r, N), op(dY, ldy, M, N), gs, ws, r, M, gpt, gqt);
  const RankJob jb = job(op(dY, ldy, N, M), op(T, ldt, r, M), bs, wsb, N, r, bpt, bqt);
  prof_begin(4, stream);
  hipLaunchKernelGGL((k_rank_pair<RB_R, RB_X, Bf16Nat<RB_R>, Bf16Nat<RB_X>, 0, RB_X, RB_R,
                                  Bf16RedMajor<RB_X>, F32RedMajor<RB_R>, 2>),
                     dim3(jg.nblk + jb.nblk), dim3(NT), 0, stream, jg, jb);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) {
    const ReduceJob rg{ws, gs.splits, M * r, 1.f, G, r, ldt};
    const ReduceJob rb{wsb, bs.splits, r * N, s, dB, N, ldb};
    const unsigned ga = cdiv(rg.count / 4, 256), gb = cdiv(rb.count / 4, 256);
    hipLaunchKernelGGL((k_split_reduce_pair<false, true>), dim3(ga + gb), dim3(256), 0, stream,
                       rg, rb, static_cast<int>(ga));
    e = hipGetLastError();
  }
  prof_end(4, stream);
  return e;
}

hipError_t launch_grad_a(const uint16_t* X, int64_t M, int64_t K, const float* G,
                         int r, float s, uint16_t* dA, float* ws, hipStream_t stream) {
  const int64_t pt = (r + RB_R - 1) / RB_R, qt = (K + RB_X - 1) / RB_X;
  const Split sp = choose_split(M, pt, qt);
  prof_begin(4, stream);
  hipLaunchKernelGGL((k_rank<RB_R, RB_X, F32RedMajor<RB_R>, Bf16RedMajor<RB_X>, 1>),
                     dim3(pt, qt, sp.splits), dim3(NT), 0, stream,
                     job(op(G, r, r, M), op(X, K, K, M), sp, ws, r, K, pt, qt));
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = reduce<true>(ws, sp.splits, K * r, s, dA, stream);
  prof_end(4, stream);
  return e;
}

}  // namespace qnf4
