// Device-side building blocks shared by the gfx950 kernels of the QLoRA NF4
// linear layer: vector types, bf16 packing, the NF4 level-pair lookup tables,
// dequantization in registers, and the 16x16x32 bf16 MFMA wrapper.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qnf4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// The 16 NF4 levels and the 15 nearest-level decision thresholds, passed to
// kernels by value (they land in scalar registers / the kernarg segment).
struct Nf4Tables {
  float q[16];
  float t[15];
};

constexpr int kBlock = 64;    // weights per absmax constant
constexpr int kGroup = 256;   // constants per fp32 second-level scale

// Index of the calling wave in its workgroup, as a wave-uniform (scalar)
// value: branches on it are scalar branches, never EXEC-masked ones.  An MFMA
// placed under an EXEC-masked branch still runs for a wave whose mask is
// empty, so MFMAs may only sit under conditions the compiler sees as uniform.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
}

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
// `a` lands in the low half (the lower-addressed element).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 h = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t packed) {
  return __builtin_bit_cast(float, packed << 16);
}
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t packed) {
  return __builtin_bit_cast(float, packed & 0xFFFF0000u);
}

// Split fp32 values a, b into bf16 hi parts and bf16 lo parts (v - hi),
// so that hi + lo carries ~16 significant bits of v.
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi,
                                             uint32_t& lo) {
  hi = pack_bf16x2(a, b);
  lo = pack_bf16x2(a - bf16_lo_to_f32(hi), b - bf16_hi_to_f32(hi));
}

// Byte-pair table replicated for conflict-free lookups: 32 copies of the 256
// entries, entry b of copy c at byte 256 b + 8 c, so lane l reads copy
// (l % 32) and the 32 lanes of a half-wave always hit distinct bank pairs
// whatever the codes.  64 KB; a kernel using it places it at LDS address 0
// (first in its dynamic LDS, with no static LDS), so a lookup address is
// (byte << 8) | ((lane % 32) << 3) with no base to add.
constexpr int kRepTabBytes = 256 * 256;

// The 16 levels, read from the kernel arguments into scalar registers at
// kernel entry.  The empty asm consumes them there, so their scalar loads go
// out with the first batch of argument loads; otherwise the compiler issues
// them just before the table is built, behind the kernel's first weight
// loads, and the table build then waits for those to drain.
struct Levels {
  float v[16];
};
__device__ __forceinline__ Levels load_levels(const Nf4Tables& tb) {
  Levels l;
#pragma unroll
  for (int j = 0; j < 16; ++j) l.v[j] = tb.q[j];
  asm volatile("" ::"s"(l.v[0]), "s"(l.v[1]), "s"(l.v[2]), "s"(l.v[3]), "s"(l.v[4]),
               "s"(l.v[5]), "s"(l.v[6]), "s"(l.v[7]), "s"(l.v[8]), "s"(l.v[9]), "s"(l.v[10]),
               "s"(l.v[11]), "s"(l.v[12]), "s"(l.v[13]), "s"(l.v[14]), "s"(l.v[15]));
  return l;
}

// Every thread of an NT-thread workgroup writes entry (tid % 256) into
// 32 * 256 / NT of its copies; the copy order is rotated by the entry, so
// the 32 lanes of a half-wave write distinct bank pairs.
template <int NT>
__device__ __forceinline__ void build_rep_pair_table(char* tab, const Levels& lv, int tid) {
  static_assert(NT % 256 == 0 && NT <= 8192, "whole copies per thread");
  constexpr int kCopies = 32 * 256 / NT;
  const int e = tid & 255, c0 = (tid >> 8) * kCopies;
  float lo = 0.f, hi = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    lo = ((e & 15) == j) ? lv.v[j] : lo;
    hi = ((e >> 4) == j) ? lv.v[j] : hi;
  }
#pragma unroll
  for (int c = 0; c < kCopies; ++c)
    reinterpret_cast<float2*>(tab)[32 * e + ((c0 + c + e) & 31)] = make_float2(lo, hi);
}

// Dequantization in registers, without a lookup table in memory.  For one
// block with constant c_hat, the 16 possible weights bf16_rne(fl32(q_j c_hat))
// are formed once (16 multiplies, 8 conversions) and split into byte planes:
// lo[a] holds the low bytes of weights 4a .. 4a+3, hi[a] their high bytes.
// A code then selects its bytes with v_perm_b32: one permute picks from 8
// entries by the code's low 3 bits, a second one chooses between the two
// halves of the table by bit 3.
struct Bf16Planes {
  uint32_t lo[4], hi[4];
};
__device__ __forceinline__ Bf16Planes block_planes(const Levels& lv, float chat) {
  uint32_t P[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) P[m] = pack_bf16x2(lv.v[2 * m] * chat, lv.v[2 * m + 1] * chat);
  Bf16Planes t;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    t.lo[a] = __builtin_amdgcn_perm(P[2 * a + 1], P[2 * a], 0x06040200u);
    t.hi[a] = __builtin_amdgcn_perm(P[2 * a + 1], P[2 * a], 0x07050301u);
  }
  return t;
}

// The four bytes of plane pl (lo or hi) for the four codes whose low 3 bits
// are the bytes of sel, bit 3 given as 4 in the bytes of half (+ 0x03020100).
__device__ __forceinline__ uint32_t plane_pick(const uint32_t* pl, uint32_t sel, uint32_t half) {
  return __builtin_amdgcn_perm(__builtin_amdgcn_perm(pl[3], pl[2], sel),
                               __builtin_amdgcn_perm(pl[1], pl[0], sel), half);
}

// The 8 codes of w (4 bytes, elements in order, even element in the low
// nibble) -> 8 consecutive bf16 weights (4 dwords).
__device__ __forceinline__ u32x4 dequant8_planes(uint32_t w, const Bf16Planes& t) {
  const uint32_t se = w & 0x07070707u;                            // even elements
  const uint32_t so = (w >> 4) & 0x07070707u;                     // odd elements
  const uint32_t me = ((w >> 1) & 0x04040404u) | 0x03020100u;
  const uint32_t mo = ((w >> 5) & 0x04040404u) | 0x03020100u;
  const uint32_t le = plane_pick(t.lo, se, me), he = plane_pick(t.hi, se, me);
  const uint32_t lo = plane_pick(t.lo, so, mo), ho = plane_pick(t.hi, so, mo);
  // bf16 pairs (elements 0, 2), (4, 6) and (1, 3), (5, 7) ...
  const uint32_t e01 = __builtin_amdgcn_perm(he, le, 0x05010400u);
  const uint32_t e23 = __builtin_amdgcn_perm(he, le, 0x07030602u);
  const uint32_t o01 = __builtin_amdgcn_perm(ho, lo, 0x05010400u);
  const uint32_t o23 = __builtin_amdgcn_perm(ho, lo, 0x07030602u);
  // ... interleaved into element order
  return u32x4{__builtin_amdgcn_perm(o01, e01, 0x05040100u),
               __builtin_amdgcn_perm(o01, e01, 0x07060302u),
               __builtin_amdgcn_perm(o23, e23, 0x05040100u),
               __builtin_amdgcn_perm(o23, e23, 0x07060302u)};
}

typedef __attribute__((address_space(3))) const f32x2 LdsF32x2;

// The level pair of byte B of w from the replicated table.  ta holds the
// lane's copy offset in byte 0; the address is (byte << 8) | copy offset,
// built by one v_perm_b32 (byte 0 from ta, byte 1 = byte B of w, bytes 2
// and 3 zero), which the scheduler can move like any other VALU op.
template <int B>
__device__ __forceinline__ f32x2 rep_lookup(uint32_t ta, uint32_t w) {
  const uint32_t a = __builtin_amdgcn_perm(w, ta, 0x0C0C0000u | ((4u + B) << 8));
  return *reinterpret_cast<LdsF32x2*>(static_cast<uintptr_t>(a));
}

__device__ __forceinline__ uint32_t rep_lane_base(int lane) {
  return static_cast<uint32_t>(lane & 31) << 3;
}

// v moved across lanes by a DPP control word (all rows and banks enabled).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Raw buffer access: a descriptor over [p, p + nbytes) in scalar registers
// and 32-bit byte offsets; reads outside the range return zero.
typedef __amdgpu_buffer_rsrc_t BufRes;
constexpr int kBufDword3 = 0x00020000;   // raw, untyped buffer (gfx9 family)

__device__ __forceinline__ BufRes make_bufres(const void* p, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0,
                                           static_cast<int>(nbytes), kBufDword3);
}
__device__ __forceinline__ u32x4 buf_load16(BufRes r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load_u8(BufRes r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}
__device__ __forceinline__ float buf_load_f32(BufRes r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// Block constant: c_hat = fl32(e * d) with double quantization (8-bit e per
// block, one fp32 d per 256 blocks), else the block's stored fp32 absmax.
__device__ __forceinline__ float block_scale(const uint8_t* absmax_q,
                                             const float* absmax_scale,
                                             int64_t block, bool dq) {
  return dq ? static_cast<float>(absmax_q[block]) * absmax_scale[block >> 8]
            : absmax_scale[block];
}

// Weight forms the tiled GEMMs read: 4-bit codes with double-quantized block
// constants, 4-bit codes with fp32 block constants, or a bf16 weight.
enum WeightForm : int { kFormDq = 0, kFormNoDq = 1, kFormDense = 2 };

// D += A . B for one 16x16x32 bf16 MFMA.  Lane l supplies row (l % 16) of A
// and column (l % 16) of B, each with the 8 reduction elements 8*(l/16)..+7;
// lane l receives D rows 4*(l/16)..+3 of column l % 16.
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// v_perm_b32 selector patterns for building bf16 pairs from two dwords.
// perm(hi_src, lo_src, sel): bytes 0-3 index lo_src, 4-7 index hi_src.
constexpr uint32_t kSelLoHalves = 0x05040100u;   // lo16(lo_src) | lo16(hi_src)<<16
constexpr uint32_t kSelHiHalves = 0x07060302u;   // hi16(lo_src) | hi16(hi_src)<<16

// Transpose an 8x8 tile of 16-bit elements held as 8 rows of 4 dwords.
// in[i] = row i (elements (i,0..7)); out[j] = column j (elements (0..7,j)).
__device__ __forceinline__ void transpose8x8_b16(const u32x4* in, u32x4* out) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int p = j >> 1;
    const uint32_t sel = (j & 1) ? kSelHiHalves : kSelLoHalves;
    uint32_t d[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      d[q] = __builtin_amdgcn_perm(in[2 * q + 1][p], in[2 * q][p], sel);
    }
    out[j] = u32x4{d[0], d[1], d[2], d[3]};
  }
}

}  // namespace qnf4
