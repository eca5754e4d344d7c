// fa_common.hpp -- device helpers shared by the forward and backward kernels.
//
// gfx950 (CDNA4) facts these helpers rely on:
//  * A wavefront has 64 lanes.
//  * v_mfma_f32_32x32x16_{f16,bf16}: D(32x32,f32) = A(32x16) * B(16x32) + C.
//    A lane l supplies 8 consecutive K-slots of row (l % 32) of A, and the
//    same 8 K-slots of column (l % 32) of B; lanes 0-31 and 32-63 cover the
//    two halves of K.  Because A and B use the same slot order, any
//    consistent assignment of real indices to (lane half, element) pairs
//    gives the right contraction.
//  * The 16 accumulator registers of lane l hold column n = l % 32 and rows
//    m = 8*(r/4) + 4*(l/32) + (r%4), r = 0..15.
//  * LDS has 64 banks of 4 bytes; ds_read_b128 is served 16 lanes (256
//    bytes) at a time and ds_read_b64_tr_b16 32 lanes at a time.  Tiles are
//    stored as 16-byte chunks with an XOR swizzle inside every 256-byte line
//    (swz() for tiles read only by rows, dual_chunk() for tiles also read
//    transposed), so that the lanes served together hit distinct banks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct Fp16 {
  static constexpr int id = 0;
};
struct Bf16 {
  static constexpr int id = 1;
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <class T>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c);

template <>
__device__ __forceinline__ f32x16 mfma32<Fp16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x16 mfma32<Bf16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Two floats -> one dword of two 16-bit values (lo = a), round to nearest even.
template <class T>
__device__ __forceinline__ uint32_t pack2(float a, float b);

template <>
__device__ __forceinline__ uint32_t pack2<Fp16>(float a, float b) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 v = {(_Float16)a, (_Float16)b};  // one v_cvt_pk_f16_f32
  return __builtin_bit_cast(uint32_t, v);
}

template <>
__device__ __forceinline__ uint32_t pack2<Bf16>(float a, float b) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const b2 v = {(__bf16)a, (__bf16)b};  // one v_cvt_pk_bf16_f32
  return __builtin_bit_cast(uint32_t, v);
}

// acc + lo + hi of a packed pair of 16-bit values, in FP32.
template <class T>
__device__ __forceinline__ float add_pair(uint32_t w, float acc);

// fp16: two v_fma_mix_f32 (each half widened exactly, times 1.0, added with
// one FP32 rounding).  These run on the vector ALU beside an MFMA; a v_dot2
// would wait for the matrix core (measured on gfx950: a dependent v_dot2c per
// 32x32x16 MFMA stretches it from 33 to 48 cycles).
template <>
__device__ __forceinline__ float add_pair<Fp16>(uint32_t w, float acc) {
  asm("v_fma_mix_f32 %0, %1, 1.0, %0 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mix_f32 %0, %1, 1.0, %0 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "+v"(acc)
      : "v"(w));
  return acc;
}

template <>
__device__ __forceinline__ float add_pair<Bf16>(uint32_t w, float acc) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, w), b2{(__bf16)1.0f, (__bf16)1.0f}, acc, false);
}

// Eight floats (elements lo..lo+7 of an accumulator) -> one MFMA operand.
template <class T>
__device__ __forceinline__ u32x4 pack8(const f32x16& s, int lo) {
  u32x4 r;
  r[0] = pack2<T>(s[lo + 0], s[lo + 1]);
  r[1] = pack2<T>(s[lo + 2], s[lo + 3]);
  r[2] = pack2<T>(s[lo + 4], s[lo + 5]);
  r[3] = pack2<T>(s[lo + 6], s[lo + 7]);
  return r;
}

// 16-byte-chunk swizzle: within each 256-byte line (16 chunks) the chunk
// position is XORed with the line index.
__device__ __forceinline__ int swz(int chunk) { return chunk ^ ((chunk >> 4) & 15); }

// Chunk swizzle for a tile (RC 16-byte chunks per row) that is read both by
// rows (ds_read_b128, served 16 lanes at a time: 16 different rows, same
// logical chunk) and transposed (ds_read_b64_tr_b16, served 32 lanes at a
// time: 4 consecutive aligned rows x 4 adjacent chunks).  With 64 banks of 4
// bytes a 256-byte line holds 16 chunk positions.  RC = 16 (one row per
// line): the XOR value 4*(r%4) + (r/4)%4 takes all 16 values over 16
// consecutive rows, and over 4 aligned rows its bits 2-3 differ, so the
// 4 x 4 chunks of a transposed read land on 16 distinct positions.  RC = 8
// (two rows per line, odd rows in the upper half): 4*((r/2)%2) + (r/4)%4
// takes 8 distinct values on the even and on the odd rows of 16 consecutive
// rows, and differs in bit 2 between the two even (or odd) rows of 4
// aligned rows.  Both depend only on the low four bits of the row.
template <int RC>
__device__ __forceinline__ int dual_xor(int r) {
  return RC == 16 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}
template <int RC>
__device__ __forceinline__ int dual_chunk(int r, int c) {
  return r * RC + (c ^ dual_xor<RC>(r));
}

// Swap bits 2 and 3 of a row index inside a 32-row MFMA block.  Reading
// operand rows in this order makes accumulator register r of lane-half g
// hold row 16*(r/8) + 8*g + (r%8) -- eight consecutive rows per half -- so a
// probability tile can be fed straight back as the K-operand of the next
// product with 16-byte LDS reads on the other operand.
__device__ __forceinline__ int perm23(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// Row (within its 32-row block) held by accumulator register r of lane-half g
// when operand rows were read in perm23 order.
__device__ __forceinline__ int acc_row(int r, int g) { return ((r >> 3) << 4) + (g << 3) + (r & 7); }

// Value of x in the lane 32 positions away, combined with x by max / add.
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Direct HBM -> LDS copies and transposing LDS reads (gfx950).
// ---------------------------------------------------------------------------
// buffer_load_dwordx4 ... lds: every lane fetches 16 bytes at its own byte
// offset into a buffer resource; lane l's bytes land at lds_wave_base + 16*l,
// and lds_wave_base must be the same for the whole wave.  Completion is
// tracked by vmcnt.  A raw buffer resource (stride 0) of `bytes` bytes makes
// every load at or past byte `bytes` return zero without touching memory,
// which is how partial tiles are read.  The descriptor lives in scalar
// registers when `base` and `bytes` are wave-uniform.  Word 3 (0x00020000)
// is the gfx9 family's data-format field for untyped 32-bit loads.
//
// A buffer resource lives in scalar registers, so `base` and `bytes` must be
// the same in every lane (every caller passes one tile of its workgroup).
// They are read from the first lane: where the compiler cannot prove them
// uniform it would otherwise wrap each load in a loop over the distinct
// values of the lanes (measured in the backward's dK/dV pass: sixteen such
// loops per two query tiles).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  void* ub = (void*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// Direct copy of one 64-row tile of a row-major [rows, D] tensor by NT
// threads: copy i of this lane reads the 16-byte chunk at element offset
// src0 + i*NT*8 of the tile and lands at dst + i*NT (dst already includes
// the wave's 64-chunk offset).  Only `valid` rows (1 .. 64) of the tile lie
// inside the tensor; chunks of later rows read as zero, and callers mask
// those rows out of the result.
template <int D, int LPT, int NT>
__device__ __forceinline__ void copy_tile_rows(const uint16_t* tile, int src0, u32x4* dst, int valid) {
  const __amdgpu_buffer_rsrc_t r = buffer_rsrc(tile, valid * D * 2);
#pragma unroll
  for (int i = 0; i < LPT; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(dst + i * NT), 16,
                                             src0 * 2, i * NT * 16, 0, 0);
}

// The non-empty key tiles of a key-padding mask, as a workgroup walks them:
// positions 0 .. end-1 of the batch element's compacted tile list.  A window
// of 64 consecutive positions is held one per lane (tile index and the two
// halves of its visibility word) and read with v_readlane, so a lookup costs
// no memory access; positions must be looked up in increasing order, and the
// window is refilled (one vector load per lane) once every 64 positions.
struct TileWindow {
  const int* list;
  const uint64_t* words;
  int end;
  int base;
  uint32_t t, lo, hi;

  // Positions start .. end-1 will be looked up.
  __device__ __forceinline__ void init(const int* list_b, const uint64_t* words_b, int n, int lane, int start = 0) {
    list = list_b;
    words = words_b;
    end = n;
    fill(start, lane);
  }
  __device__ __forceinline__ void fill(int b0, int lane) {
    base = b0;
    t = lo = hi = 0;
    if (b0 + lane < end) {
      const int tile = list[b0 + lane];
      const uint64_t w = words[tile];
      t = (uint32_t)tile;
      lo = (uint32_t)w;
      hi = (uint32_t)(w >> 32);
    }
  }
  // Tile at position i (i < end) and its word; call tile(i) before word(i).
  __device__ __forceinline__ int tile(int i, int lane) {
    if (i - base >= 64) fill(i, lane);
    return __builtin_amdgcn_readlane((int)t, i - base);
  }
  __device__ __forceinline__ void word(int i, uint32_t& wlo, uint32_t& whi) const {
    wlo = (uint32_t)__builtin_amdgcn_readlane((int)lo, i - base);
    whi = (uint32_t)__builtin_amdgcn_readlane((int)hi, i - base);
  }
};

// True when key kb*32 + acc_row(r, g) of a 64-key tile is hidden by the
// tile's visibility word (wlo: keys 0-31, whi: keys 32-63).
__device__ __forceinline__ bool key_hidden(uint32_t wlo, uint32_t whi, int kb, int r, int g) {
  const uint32_t wk = (kb ? whi : wlo) >> (8 * g);
  return ((wk >> (16 * (r >> 3) + (r & 7))) & 1u) == 0;
}

// ---------------------------------------------------------------------------
// Dropout: Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011).  Per round the two 64 x 64 -> 128
// bit products M0*c0 and M1*c2 are formed and c = (hi1 ^ c1 ^ k0, lo1,
// hi0 ^ c3 ^ k1, lo0); the key is then bumped by the Weyl constants.
// Query i, key j of head bh uses counter (j / 16, i, bh, offset) and key
// (seed, 0); the 256 output bits are 16 values of 16 bits, key 16t + e
// taking bits 16*(e % 4) .. +15 of word e / 4, and the key is kept iff its
// value >= thr = floor(p * 65536).
// ---------------------------------------------------------------------------
constexpr uint64_t kPhiloxM0 = 0xD2E7470EE14C6C93ull;
constexpr uint64_t kPhiloxM1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhiloxW0 = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kPhiloxW1 = 0xBB67AE8584CAA73Bull;

// The 128-bit product a*m as (hi, lo) from four 32x32->64 multiply-adds
// (v_mad_u64_u32): with a = a1:a0 and m = m1:m0 in 32-bit halves,
// t = a0*m1 + hi(a0*m0) and u = a1*m0 + lo(t) cannot overflow 64 bits, the
// low word is lo(a0*m0) | lo(u) << 32 and the high word a1*m1 + hi(t) + hi(u).
__device__ __forceinline__ void mulhilo64(uint64_t a, uint64_t m, uint64_t& hi, uint64_t& lo) {
  const uint32_t a0 = (uint32_t)a, a1 = (uint32_t)(a >> 32);
  const uint32_t m0 = (uint32_t)m, m1 = (uint32_t)(m >> 32);
  const uint64_t p00 = (uint64_t)a0 * m0;
  const uint64_t t = (uint64_t)a0 * m1 + (p00 >> 32);
  const uint64_t u = (uint64_t)a1 * m0 + (uint32_t)t;
  lo = (uint32_t)p00 | (u << 32);
  hi = (uint64_t)a1 * m1 + ((t >> 32) + (u >> 32));
}

__device__ __forceinline__ void philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3, uint64_t k0,
                                              uint64_t k1, uint64_t (&out)[4]) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint64_t hi0, lo0, hi1, lo1;
    mulhilo64(c0, kPhiloxM0, hi0, lo0);
    mulhilo64(c2, kPhiloxM1, hi1, lo1);
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

// 16-bit value e (0..7) of a group of 8 held in two 64-bit words.
__device__ __forceinline__ uint32_t half8_value(uint64_t w0, uint64_t w1, int e) {
  return (uint32_t)(((e < 4 ? w0 : w1) >> (16 * (e & 3))) & 0xFFFFu);
}

// The value of x held by the lane 32 positions away (lane-half g = lane / 32).
__device__ __forceinline__ uint32_t xhalf_partner(uint32_t x, int g) {
  auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return g ? r[0] : r[1];
}

// Keep bits of the 16 keys a lane of an S^T accumulator holds for one
// 32-key block (query per lane, register r holding key acc_row(r, g)):
// the block's keys are Philox groups t0 = key0/16 and t0+1; lane-half g
// computes group t0+g, keeps the 8 values of its own half and swaps the
// other 8 with its partner, which needs them.  Bit r of the result is the
// keep decision of register r.
__device__ __forceinline__ uint32_t dropout_bits_st(int key0, int query, uint64_t bh, uint64_t seed,
                                                    uint64_t offset, uint32_t thr, int g) {
  uint64_t w[4];
  philox4x64_10((uint64_t)(key0 / 16 + g), (uint64_t)(uint32_t)query, bh, offset, seed, 0, w);
  // own half g: words 2g, 2g+1; the partner needs half 1-g of this group.
  const uint64_t own0 = g ? w[2] : w[0], own1 = g ? w[3] : w[1];
  const uint64_t snd0 = g ? w[0] : w[2], snd1 = g ? w[1] : w[3];
  const uint64_t rcv0 = ((uint64_t)xhalf_partner((uint32_t)(snd0 >> 32), g) << 32) |
                        xhalf_partner((uint32_t)snd0, g);
  const uint64_t rcv1 = ((uint64_t)xhalf_partner((uint32_t)(snd1 >> 32), g) << 32) |
                        xhalf_partner((uint32_t)snd1, g);
  // registers 0-7: group t0, values 8g .. 8g+7; registers 8-15: group t0+1, same values
  const uint64_t a0 = g ? rcv0 : own0, a1 = g ? rcv1 : own1;  // group t0, half g
  const uint64_t b0 = g ? own0 : rcv0, b1 = g ? own1 : rcv1;  // group t0+1, half g
  uint32_t bits = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    bits |= (half8_value(a0, a1, e) >= thr ? 1u : 0u) << e;
    bits |= (half8_value(b0, b1, e) >= thr ? 1u : 0u) << (8 + e);
  }
  return bits;
}

// Keep bits of 16 consecutive keys 16t .. 16t+15 for one query (bit e = key
// 16t + e).
__device__ __forceinline__ uint32_t dropout_bits16(int t, int query, uint64_t bh, uint64_t seed, uint64_t offset,
                                                   uint32_t thr) {
  uint64_t w[4];
  philox4x64_10((uint64_t)t, (uint64_t)(uint32_t)query, bh, offset, seed, 0, w);
  uint32_t bits = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e)
    bits |= ((uint32_t)((w[e >> 2] >> (16 * (e & 3))) & 0xFFFFu) >= thr ? 1u : 0u) << e;
  return bits;
}

// Wait until this wave's outstanding global loads (including LDS-bound ones)
// have completed.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ds_read_b64_tr_b16: inside each group of 16 lanes, lane j points at four
// consecutive 16-bit values R_j[0..3]; lane i receives R_{4k + i/4}[i % 4]
// for k = 0..3.  Pointing lane j at row (k0 + j/4), columns c0 + 4*(j%4)
// .. +3 of a row-major tile hands lane i the column c0 + i of rows k0..k0+3:
// a transposed MFMA operand read straight from a row-major tile.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const void* lds_addr) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)lds_addr);
  return __builtin_bit_cast(u32x2, v);
}

// ---------------------------------------------------------------------------
// MFMAs with explicit register classes (inline assembly).  The compiler
// assigns MFMA accumulators to one register class per kernel; kernels that
// need more than 256 live registers per wave place operands by hand: scores
// in VGPRs, Q fragments and O accumulators in AGPRs.  Inline assembly is
// opaque to the compiler's hazard checks, so the wait states gfx950 requires
// are placed by hand: 12 between an MFMA that writes a register and a vector
// instruction that reads it (scores_ready and o_ready give 16), and 2 between
// a vector write and an MFMA reading that register as an operand (FRESH).
// The register allocator may itself add such a write (a copy back from a
// register parked in the other class) right before an MFMA; the generated
// code of every kernel that uses these helpers is scanned for both hazards
// by the test suite.
// ---------------------------------------------------------------------------
// S (VGPR) = A (VGPR) * B (AGPR), accumulator started at zero.  FRESH:
// two wait states go first, for an operand that a vector instruction may
// have written just before (including copies the register allocator adds).
template <class T, bool FRESH = false>
__device__ __forceinline__ void mfma_s_first(f32x16& d, const u32x4& a, const u32x4& b) {
  if constexpr (T::id == Fp16::id) {
    if constexpr (FRESH)
      asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
    else
      asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
  } else {
    if constexpr (FRESH)
      asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
    else
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
  }
}
// S (VGPR) += A (VGPR) * B (AGPR).
template <class T, bool FRESH = false>
__device__ __forceinline__ void mfma_s_acc(f32x16& d, const u32x4& a, const u32x4& b) {
  if constexpr (T::id == Fp16::id) {
    if constexpr (FRESH)
      asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
    else
      asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
  } else {
    if constexpr (FRESH)
      asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
    else
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
  }
}
// O (AGPR) += A (VGPR) * B (VGPR); FRESH: B was just written by vector
// instructions, so two wait states go first.
template <class T, bool FRESH>
__device__ __forceinline__ void mfma_o(f32x16& d, const u32x4& a, const u32x4& b) {
  if constexpr (T::id == Fp16::id) {
    if constexpr (FRESH)
      asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
    else
      asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
  } else {
    if constexpr (FRESH)
      asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
    else
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
  }
}
// 16 wait states after MFMAs that wrote the four score accumulators of a
// tile, before any vector instruction reads them (ties them so that no read
// is scheduled above).
__device__ __forceinline__ void scores_ready(f32x16 (&s)[2][2]) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(s[0][0]), "+v"(s[0][1]), "+v"(s[1][0]), "+v"(s[1][1]));
}
__device__ __forceinline__ void scores_ready(f32x16 (&s)[1][2]) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(s[0][0]), "+v"(s[0][1]));
}
// Workgroup barrier without the memory fence __syncthreads adds (which
// waits for every load in flight, the tile copies included).  Callers wait
// for exactly the copies the barrier must cover; the memory clobber keeps
// the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// 16 wait states after the last MFMA into O, before vector reads of O
// (one or two query blocks, head size 128 or 64).
__device__ __forceinline__ void o_ready(f32x16 (&o)[2][4]) {
  asm volatile("s_nop 7\n\ts_nop 7"
               : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[0][2]), "+a"(o[0][3]), "+a"(o[1][0]), "+a"(o[1][1]),
                 "+a"(o[1][2]), "+a"(o[1][3]));
}
__device__ __forceinline__ void o_ready(f32x16 (&o)[2][2]) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[1][0]), "+a"(o[1][1]));
}
__device__ __forceinline__ void o_ready(f32x16 (&o)[1][4]) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[0][2]), "+a"(o[0][3]));
}
__device__ __forceinline__ void o_ready(f32x16 (&o)[1][2]) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+a"(o[0][0]), "+a"(o[0][1]));
}

// Wave-uniform votes (every lane of the wave is active where these are used).
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }
__device__ __forceinline__ bool wave_all(bool p) { return __builtin_amdgcn_ballot_w64(!p) == 0; }

}  // namespace fa
