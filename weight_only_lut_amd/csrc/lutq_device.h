// Device-side building blocks shared by the lutq kernels (gfx950 only).
//
// Terms used throughout:
//  tile   : 16 consecutive weight rows (output features n).
//  chunk  : 128 consecutive codes along K.
//  block  : one (tile, chunk) pair = 64 lane slots x (4*BITS) bytes, the unit
//           that one wavefront loads with one coalesced load per lane.
//  slot L : L = 16*q + r holds row 16*t + r, codes k = 128*c + 32*j + 8*q + e
//           (j = 0..3 "k-step", e = 0..7).
//  pair table: 256 entries of two fp16 values (T[c_even], T[c_odd]) indexed
//           by a byte assembled from two codes, stored 64 times in LDS so
//           that lane L always reads copy L: entry (idx, copy) lives at byte
//           address (idx << 8) | (copy << 2), which spreads the 64 lanes of a
//           lookup over 64 distinct banks whatever the codes are (FLUTE
//           abstract: a vectorized, duplicated table against shared-memory
//           bandwidth limits).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace lutq {

constexpr int kTileRows = 16;
constexpr int kChunk = 128;
constexpr int kWave = 64;
constexpr int kPairEntries = 256;
constexpr int kCopies = 64;
constexpr int kTableWords = kPairEntries * kCopies;  // 16384 dwords = 64 KiB
// Word 3 of a raw (unstructured, stride 0) buffer resource on gfx9-family
// GPUs: 32-bit data format, no swizzle; offsets are bytes, range-checked
// against the record count.
constexpr int kBufferRsrcWord3 = 0x00020000;
// Buffer offsets past the record count of every resource the kernels build
// (each spans at most 64 MiB): kOutOfRange marks a pipeline step past the
// wave's last chunk, kRowOutOfRange a batch row past M. Either may be added
// to the other and to an in-resource offset without wrapping 32 bits.
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr uint32_t kRowOutOfRange = 0x40000000u;

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Bytes of one lane slot and number of dwords it spans.
template <int BITS> struct Slot {
  static constexpr int kBytes = 4 * BITS;
  static constexpr int kDwords = BITS;
};

// Codes of one lane slot in registers.
template <int BITS> struct SlotRegs { uint32_t d[BITS]; };

// A raw buffer resource over `bytes` bytes at `base`. Loads through it at
// an offset at or past `bytes` return zeros without a memory access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes,
                                           kBufferRsrcWord3);
}

// Cache policy of the code stream: nontemporal (read once).
constexpr int kNontemporal = 2;

// One lane slot of codes at byte offset `off` of the resource.
template <int BITS>
__device__ __forceinline__ SlotRegs<BITS> load_slot(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  SlotRegs<BITS> r;
  if constexpr (BITS == 4) {
    const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kNontemporal));
    r.d[0] = v.x; r.d[1] = v.y; r.d[2] = v.z; r.d[3] = v.w;
  } else if constexpr (BITS == 3) {
    const u32x3 v = __builtin_bit_cast(u32x3, __builtin_amdgcn_raw_buffer_load_b96(rs, off, 0, kNontemporal));
    r.d[0] = v.x; r.d[1] = v.y; r.d[2] = v.z;
  } else {
    const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, kNontemporal));
    r.d[0] = v.x; r.d[1] = v.y;
  }
  return r;
}

// The four pair-index bytes of k-step j (one byte per pair e/2 = 0..3).
// Only the bits a table index uses are meaningful; the pair table repeats its
// entries over the unused high bits, so no masking is needed here.
template <int BITS>
__device__ __forceinline__ uint32_t step_indices(const SlotRegs<BITS>& s, int j) {
  if constexpr (BITS == 4) {
    return s.d[j];
  } else if constexpr (BITS == 2) {
    const uint32_t w = s.d[j >> 1];
    return (j & 1) ? (w >> 4) : w;
  } else {
    // low 2-bit planes as nibbles (as BITS == 2), high bits from word 2
    const uint32_t lo = s.d[j >> 1];
    const uint32_t l = (j & 1) ? (lo >> 4) : lo;
    const uint32_t h = s.d[2];
    uint32_t hs;
    switch (j) {
      case 0: hs = h; break;
      case 1: hs = h >> 2; break;
      case 2: hs = h << 4; break;
      default: hs = h << 2; break;
    }
    // bits 0-3 of each byte from the low planes, bits 4-7 from the high plane
    return (l & 0x0F0F0F0Fu) | (hs & 0xF0F0F0F0u);  // one v_bfi_b32
  }
}

// LDS byte address of pair-table entry (byte `i` of `idx4`, copy = lane):
// v_perm puts the index byte in bits 8-15 and the lane byte (lane*4) in bits
// 0-7 -- one VALU op per lookup.
__device__ __forceinline__ uint32_t pair_addr(uint32_t idx4, uint32_t lane_byte, int i) {
  const uint32_t sel = 0x0C0C0000u | ((4u + (uint32_t)i) << 8);
  return __builtin_amdgcn_perm(idx4, lane_byte, sel);
}

__device__ __forceinline__ uint32_t lds_load(const uint32_t* table, uint32_t byte_addr) {
  return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(table) + byte_addr);
}

// Keeps the compiler from moving this wave's memory operations across the
// call, for data that lanes exchange through LDS. It emits no instruction:
// LDS executes one wave's operations in issue order.
__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Decode the two codes of a pair index for table building.
template <int BITS>
__device__ __forceinline__ void pair_codes(uint32_t idx, uint32_t& c0, uint32_t& c1) {
  if constexpr (BITS == 4) {
    c0 = idx & 15u; c1 = (idx >> 4) & 15u;
  } else if constexpr (BITS == 2) {
    c0 = idx & 3u; c1 = (idx >> 2) & 3u;
  } else {
    c0 = (idx & 3u) | (((idx >> 4) & 1u) << 2);
    c1 = ((idx >> 2) & 3u) | (((idx >> 5) & 1u) << 2);
  }
}

// T[lane mod 2^BITS] (fp16 bits in the low half) for every lane. The table
// is read with uniform loads (the compiler issues them as scalar loads) and
// spread to lanes with selects; `lut` must be 4-byte aligned.
template <int BITS>
__device__ __forceinline__ uint32_t lut_to_lanes(const uint16_t* lut, int lane) {
  constexpr int kWords = (1 << BITS) / 2;
  const uint32_t* w = reinterpret_cast<const uint32_t*>(lut);
  uint32_t words[kWords];
#pragma unroll
  for (int i = 0; i < kWords; ++i) words[i] = __builtin_amdgcn_readfirstlane(w[i]);
  const int e = lane & ((1 << BITS) - 1);
  uint32_t v = words[0];
#pragma unroll
  for (int i = 1; i < kWords; ++i) v = (e >> 1) == i ? words[i] : v;
  return (e & 1) ? (v >> 16) : (v & 0xFFFFu);
}

// Per-group data types: up to kMaxTypes tables share the LDS pair table,
// kCopies / kMaxTypes copies each. Entry (idx, type, copy) lives at byte
// (idx << 8) | (type << 6) | (copy << 2): the same single v_perm builds the
// address, from a lane byte (type << 6) | ((lane mod 16) << 2).
constexpr int kMaxTypes = 4;
constexpr int kTypedCopies = kCopies / kMaxTypes;

// Table (lane >> BITS) entry (lane mod 2^BITS) for lanes 0 .. 4 * 2^BITS - 1
// (repeating beyond), from `ntypes` tables stored one after another; a table
// past ntypes repeats table 0. One per-lane load per workgroup.
template <int BITS>
__device__ __forceinline__ uint32_t typed_lut_lane(const uint16_t* luts, int ntypes, int lane) {
  constexpr int L = 1 << BITS;
  const int e = lane & (kMaxTypes * L - 1);
  const int t = e >> BITS;
  return luts[(t < ntypes ? t : 0) * L + (e & (L - 1))];
}

// Binary-coded weights: the entry of pair index idx holds, for each plane p
// (p < BITS), the fp16 pair (bit_p(c0), bit_p(c1)) of 0.0 / 1.0 as dword p;
// entries are 8 bytes (2 planes) or 16 (3 or 4), and the 256-byte row of
// idx holds 256 / that many copies (lane l reads copy l mod copies).
constexpr int kCopyBytes = 256;
template <int BITS> constexpr int kBcqEntryBytes = BITS == 2 ? 8 : 16;

template <int BITS>
__device__ __forceinline__ u32x4 lds_load_bcq(const uint32_t* table, uint32_t byte_addr) {
  const char* b = reinterpret_cast<const char*>(table) + byte_addr;
  if constexpr (BITS == 2) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(b);
    return u32x4{v.x, v.y, 0u, 0u};
  } else {
    // 3 planes read 16 bytes too: a 12-byte LDS read measured slower
    // (12.3 -> 14.6 us on a 14336 x 4096 matrix at batch 1)
    return *reinterpret_cast<const u32x4*>(b);
  }
}

// Binary-coded weights on the MFMA path: the planes' fp16 (bit, bit) pairs
// of k-step j decoded in registers instead of looked up. For each plane, one
// or two bit operations place every pair's two bits as the two 4-bit halves
// of a byte, as FP4 (E2M1) codes that are 0 or one power of two (a bit in
// the mantissa or exponent field, never the sign); gfx950's scaled FP4 to
// fp16 conversion turns byte i into the fp16 pair of pair i, with the scale
// that makes the power of two 1.0 -- so pw[i][p] is exactly the entry the
// table of build_bcq_table holds for pair i, plane p. The bit positions are
// those step_indices gives: BITS = 4, codes c0 | c1 << 4; BITS = 2 and 3,
// the two low bits of c0 and c1 in bits 0-3 and (BITS = 3) the high bits
// of c0 and c1 in bits 4 and 5.
template <int BITS>
__device__ __forceinline__ void bcq_planes_decode(uint32_t idx4, u32x4 (&pw)[4]) {
  uint32_t d[4] = {0u, 0u, 0u, 0u};
  float sc[4] = {1.f, 1.f, 1.f, 1.f};
  if constexpr (BITS == 4) {
    d[0] = idx4 & 0x11111111u; sc[0] = 2.f;        // mantissa bit: 0.5
    d[1] = idx4 & 0x22222222u;                     // low exponent bit: 1.0
    d[2] = idx4 & 0x44444444u; sc[2] = 0.5f;       // high exponent bit: 2.0
    d[3] = (idx4 >> 1) & 0x44444444u; sc[3] = 0.5f;  // bit 3 (the sign) moved to 2.0
  } else {
    const uint32_t w2 = idx4 << 2;  // c1's low bits into the upper half
    d[0] = (idx4 & 0x01010101u) | (w2 & 0x10101010u); sc[0] = 2.f;
    d[1] = (idx4 & 0x02020202u) | (w2 & 0x20202020u);
    if constexpr (BITS == 3) d[2] = ((idx4 >> 3) & 0x02020202u) | (idx4 & 0x20202020u);
  }
#pragma unroll
  for (int pl = 0; pl < BITS; ++pl) {
    pw[0][pl] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d[pl], sc[pl], 0));
    pw[1][pl] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d[pl], sc[pl], 1));
    pw[2][pl] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d[pl], sc[pl], 2));
    pw[3][pl] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d[pl], sc[pl], 3));
  }
}

template <int BITS, int THREADS>
__device__ __forceinline__ void build_bcq_table(uint32_t* table, int tid) {
  static_assert(THREADS % kPairEntries == 0, "whole threads per entry");
  constexpr int kPerEntry = THREADS / kPairEntries;
  constexpr int kStores = kCopyBytes / 16;                 // 16-byte stores per entry row
  constexpr int C = kStores / kPerEntry;                    // stores per thread
  static_assert(C >= 1 && (C & (C - 1)) == 0, "power-of-two stores per thread");
  const uint32_t idx = (uint32_t)tid / kPerEntry;
  const uint32_t part = (uint32_t)tid % kPerEntry;
  uint32_t c0, c1;
  pair_codes<BITS>(idx, c0, c1);
  uint32_t d[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int pl = 0; pl < BITS; ++pl)
    d[pl] = (((c0 >> pl) & 1u) ? 0x3C00u : 0u) | (((c1 >> pl) & 1u) ? 0x3C000000u : 0u);
  const u32x4 q = BITS == 2 ? u32x4{d[0], d[1], d[0], d[1]} : u32x4{d[0], d[1], d[2], d[3]};
  u32x4* dst = reinterpret_cast<u32x4*>(table) + idx * kStores + part * C;
  // rotated by the thread, as in build_pair_table
#pragma unroll
  for (int k = 0; k < C; ++k) dst[(k + (uint32_t)tid) & (C - 1)] = q;
}

// Fill the duplicated pair table. `lut_lane` holds T[lane] in lanes
// 0..2^BITS-1 of every wave; entries are gathered with cross-lane reads.
// THREADS / 256 threads share an entry: each computes the entry's value once
// and writes its share of the 64 copies as 16-byte stores. Store k of a
// thread goes to chunk (k + thread) mod C of its share. Measured on gfx950
// (SQ_LDS_BANK_CONFLICT), 16-byte stores are served eight lanes at a time
// over 32 four-byte banks: rotating by the entry instead put the two threads
// of an entry (8 waves) on the same banks, 64 conflict cycles per wave; by
// the thread, eight consecutive lanes always cover the 32 banks. The caller
// issues a barrier before the first lookup.
template <int BITS, int THREADS, bool TYPED = false>
__device__ __forceinline__ void build_pair_table(uint32_t* table, uint32_t lut_lane, int tid) {
  static_assert(THREADS % kPairEntries == 0, "whole threads per entry");
  constexpr int kPerEntry = THREADS / kPairEntries;   // threads per entry
  constexpr int kCopiesPer = kCopies / kPerEntry;      // copies each thread writes
  constexpr int C = kCopiesPer / 4;                    // 16-byte stores per thread
  static_assert(kCopiesPer % 4 == 0 && (C & (C - 1)) == 0, "power-of-two 16-byte stores");
  const uint32_t idx = (uint32_t)tid / kPerEntry;
  const uint32_t part = (uint32_t)tid % kPerEntry;
  uint32_t c0, c1;
  pair_codes<BITS>(idx, c0, c1);
  u32x4* dst = reinterpret_cast<u32x4*>(table + idx * kCopies + part * kCopiesPer);
  if constexpr (!TYPED) {
    const uint32_t v0 = (uint32_t)__shfl((int)lut_lane, (int)c0) & 0xFFFFu;
    const uint32_t v1 = (uint32_t)__shfl((int)lut_lane, (int)c1) & 0xFFFFu;
    const uint32_t v = v0 | (v1 << 16);
    const u32x4 q = {v, v, v, v};
#pragma unroll
    for (int k = 0; k < C; ++k) dst[(k + (uint32_t)tid) & (C - 1)] = q;
  } else {
    // the pair of every type (lut_lane holds table t's entries at lanes t 2^BITS + c)
    uint32_t v[kMaxTypes];
#pragma unroll
    for (int t = 0; t < kMaxTypes; ++t) {
      const uint32_t v0 = (uint32_t)__shfl((int)lut_lane, (int)((t << BITS) | c0)) & 0xFFFFu;
      const uint32_t v1 = (uint32_t)__shfl((int)lut_lane, (int)((t << BITS) | c1)) & 0xFFFFu;
      v[t] = v0 | (v1 << 16);
    }
#pragma unroll
    for (int k = 0; k < C; ++k) {
      const int slot4 = (k + tid) & (C - 1);                      // 16-byte store in the share
      const int type = (int)(part * kCopiesPer + 4 * slot4) / kTypedCopies;
      uint32_t w = v[0];
#pragma unroll
      for (int t = 1; t < kMaxTypes; ++t) w = type == t ? v[t] : w;
      dst[slot4] = u32x4{w, w, w, w};
    }
  }
}

// acc += dot(x from lane 4j+i of this lane's 16-lane row, p_i), i = 0..3, in
// that order: four v_dot2c_f32_f16 whose DPP row_newbcast reads the
// activation pair straight from the broadcasting lane, so no separate
// broadcast move is issued. `j` must fold to a constant, and the four k-steps
// j = 0..3 of one accumulator must be issued as one chain, in order: between
// them the accumulator is read only by the next DPP dot.
// The compiler inserts no wait states around inline assembly, so the chain
// carries its own:
//  - s_nop 1 before step 0: the "manually inserted wait states" table of the
//    CDNA3 and CDNA4 instruction set references requires 2 between a VALU
//    write of a VGPR and a DPP read of it (x is written by VALU in the bf16
//    path, and the accumulator is zeroed just before);
//  - s_nop 3 after step 3: that table has no entry for a plain VALU read of a
//    DPP dot's result, but on gfx950 (built with AMD clang 22.0.0git, ROCm
//    7.2.0) such a read within 2 wait states saw the value from before the
//    dot; 3 sufficed, 4 are given;
//  - none in between: DPP dots chained on one accumulator read it correctly
//    back to back (as the four dots of one step already do).
// The GEMV parity tests (every shape and variant, bit-exact one-hot cases
// included) fail if any of these is too small.
#define LUTQ_DOT2_BCAST4(PRE, POST, A, B, C, D)                                      \
  asm(PRE                                                                           \
      "v_dot2c_f32_f16_dpp %0, %1, %2 row_newbcast:" #A " row_mask:0xf bank_mask:0xf\n\t" \
      "v_dot2c_f32_f16_dpp %0, %1, %3 row_newbcast:" #B " row_mask:0xf bank_mask:0xf\n\t" \
      "v_dot2c_f32_f16_dpp %0, %1, %4 row_newbcast:" #C " row_mask:0xf bank_mask:0xf\n\t" \
      "v_dot2c_f32_f16_dpp %0, %1, %5 row_newbcast:" #D " row_mask:0xf bank_mask:0xf\n\t" \
      POST                                                                           \
      : "+v"(acc)                                                                    \
      : "v"(x), "v"(p0), "v"(p1), "v"(p2), "v"(p3))
__device__ __forceinline__ float dot2_bcast4(float acc, uint32_t x, uint32_t p0, uint32_t p1,
                                             uint32_t p2, uint32_t p3, int j) {
  switch (j) {
    case 0: LUTQ_DOT2_BCAST4("s_nop 1\n\t", "", 0, 1, 2, 3); break;
    case 1: LUTQ_DOT2_BCAST4("", "", 4, 5, 6, 7); break;
    case 2: LUTQ_DOT2_BCAST4("", "", 8, 9, 10, 11); break;
    default: LUTQ_DOT2_BCAST4("", "s_nop 3", 12, 13, 14, 15); break;
  }
  return acc;
}
#undef LUTQ_DOT2_BCAST4

// Calls f(std::integral_constant<int, I>{}) for I = 0 .. N-1 (unrolled).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ f16x2 as_f16x2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (f16)f);  // round to nearest even
}

// Sum of the two fp16 values of a packed pair, in fp32 (one dot with 1, 1).
__device__ __forceinline__ float pair_sum(uint32_t pr) {
  const f16x2 one = {(f16)1.0f, (f16)1.0f};
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pr), one, 0.f, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Maximum over the 64 lanes of the wave.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  auto dm = [](uint32_t a, auto ctrl) {
    constexpr int C = decltype(ctrl)::value;
    const uint32_t b = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, C, 0xF, 0xF, false);
    return a > b ? a : b;
  };
  v = dm(v, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
  v = dm(v, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
  v = dm(v, std::integral_constant<int, 0x141>{});  // row_half_mirror
  v = dm(v, std::integral_constant<int, 0x140>{});  // row_mirror
  const uint32_t a = (uint32_t)__shfl_xor((int)v, 16);
  v = v > a ? v : a;
  const uint32_t b = (uint32_t)__shfl_xor((int)v, 32);
  return v > b ? v : b;
}

// Sum over the 16 lanes of a row as a butterfly (partners under xor 1, 2,
// then the mirrored half and quarter rows): every addition is a + b in one
// lane and b + a in its partner, so all 16 lanes end with the same bits.
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0x141>(v);  // row_half_mirror: quads 0 <-> 1 of each half row
  v += dpp_f32<0x140>(v);  // row_mirror: halves of the row
  return v;
}

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// bf16 activations are converted per (batch row, 128-weight chunk): scaled
// by a power of two that puts the chunk's largest magnitude in [2^14, 2^15),
// every value within 2^31 of it is an exact fp16 value, so the fp16 dot and
// MFMA arithmetic runs unchanged and the chunk's partial sums are scaled
// back by the inverse power of two (exact). `amax` holds the largest bf16
// magnitude (bits & 0x7FFF) of the chunk; the shift is 141 - exponent field.
__device__ __forceinline__ int bf16_chunk_shift(uint32_t amax) { return 141 - (int)(amax >> 7); }
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t v, int shift) {
  const float lo = __builtin_ldexpf(__builtin_bit_cast(float, v << 16), shift);
  const float hi = __builtin_ldexpf(__builtin_bit_cast(float, v & 0xFFFF0000u), shift);
  // exact values: the rounding mode of the pack does not matter
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}
__device__ __forceinline__ uint32_t bf16x2_absmax(uint32_t v) {
  const uint32_t a = v & 0x7FFFu, b = (v >> 16) & 0x7FFFu;
  return a > b ? a : b;
}
// Running magnitude maximum of bf16 pairs, per half (v_pk_max_u16), and its
// final value: on sign-cleared bf16 bits the integer order is the order of
// magnitudes.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u16x2 bf16x2_absmax_acc(u16x2 acc, uint32_t v) {
  return __builtin_elementwise_max(acc, __builtin_bit_cast(u16x2, v & 0x7FFF7FFFu));
}
__device__ __forceinline__ uint32_t u16x2_max(u16x2 v) {
  return v[0] > v[1] ? (uint32_t)v[0] : (uint32_t)v[1];
}
// Maximum over the lanes l, l ^ 16, l ^ 32 and l ^ 48, with the gfx950 lane
// swaps (VALU, no LDS): each swap exchanges half of one copy with half of
// the other, so the larger of the pair is the maximum with the partner
// lane, whichever way round the halves moved. (A float sum written the same
// way compiled here to x + x, dropping the swapped copy; this integer form
// reads both registers, and the bf16 parity tests fail if it does not.)
__device__ __forceinline__ uint32_t max_over_quarters(uint32_t a) {
  const auto h = __builtin_amdgcn_permlane32_swap(a, a, false, false);
  const uint32_t b = h[0] > h[1] ? h[0] : h[1];
  const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  return r[0] > r[1] ? r[0] : r[1];
}

// The sum over the lanes r, r + 16, r + 32, r + 48 (r < 16), in lane r:
// (x_r + x_r+16) + (x_r+32 + x_r+48), the order of a shuffle butterfly over
// lane distance 16 then 32. v_permlane16_swap exchanges the odd 16-lane rows
// of its first operand with the even rows of its second, v_permlane32_swap
// the upper half of the first with the lower half of the second; pairing x
// with zero leaves each lane r of row 0 (and of row 2) with x_r and its
// partner. Only lanes 0..15 hold the sum. (VALU; no LDS round trips.)
// (Written in assembly: with the builtins, AMD clang 22.0.0git of ROCm 7.2.0
// added the first swapped register to itself instead of to the second. The
// s_nop gives the 2 wait states that the CDNA4 instruction set reference's
// wait-state table asks for between a VALU write of a VGPR and a
// cross-lane operation reading it; the compiler adds none around inline
// assembly. The GEMV parity tests fail if either is wrong.)
__device__ __forceinline__ float sum_over_quarters_r(float x) {
  uint32_t a0 = __builtin_bit_cast(uint32_t, x), a1 = 0u;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a0), "+v"(a1));
  uint32_t c0 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, a0) + __builtin_bit_cast(float, a1));
  uint32_t c1 = 0u;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(c0), "+v"(c1));
  return __builtin_bit_cast(float, c0) + __builtin_bit_cast(float, c1);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(f16, h);
}

}  // namespace lutq
