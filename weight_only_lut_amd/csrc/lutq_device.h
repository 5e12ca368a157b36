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

template <int BITS>
__device__ __forceinline__ SlotRegs<BITS> load_slot(const uint8_t* p) {
  SlotRegs<BITS> r;
  if constexpr (BITS == 4) {
    u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    r.d[0] = v.x; r.d[1] = v.y; r.d[2] = v.z; r.d[3] = v.w;
  } else if constexpr (BITS == 3) {
    u32x3 v = __builtin_nontemporal_load(reinterpret_cast<const u32x3*>(p));
    r.d[0] = v.x; r.d[1] = v.y; r.d[2] = v.z;
  } else {
    u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
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

// Fill the duplicated pair table. `lut_lane` holds T[lane] in lanes
// 0..2^BITS-1 of every wave; entries are gathered with cross-lane reads.
// THREADS / 256 threads share an entry: each computes the entry's value once
// and writes its share of the 64 copies as 16-byte stores. Store k of a
// thread goes to chunk (k + entry) mod C of its share, so the 64 lanes of a
// store instruction cover all 64 banks evenly (4 dwords per bank, the
// minimum for 16-byte stores) instead of piling onto two bank groups. The
// caller issues a barrier before the first lookup.
template <int BITS, int THREADS>
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
  const uint32_t v0 = (uint32_t)__shfl((int)lut_lane, (int)c0) & 0xFFFFu;
  const uint32_t v1 = (uint32_t)__shfl((int)lut_lane, (int)c1) & 0xFFFFu;
  const uint32_t v = v0 | (v1 << 16);
  const u32x4 q = {v, v, v, v};
  u32x4* dst = reinterpret_cast<u32x4*>(table + idx * kCopies + part * kCopiesPer);
#pragma unroll
  for (int k = 0; k < C; ++k) dst[(k + idx) & (C - 1)] = q;
}

// DPP row_newbcast:n -- every lane of each 16-lane row reads lane n of that
// row. `n` must fold to a constant after unrolling.
__device__ __forceinline__ uint32_t row_newbcast(uint32_t v, int n) {
  switch (n) {
    case 0: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x150, 0xF, 0xF, false);
    case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x151, 0xF, 0xF, false);
    case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x152, 0xF, 0xF, false);
    case 3: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x153, 0xF, 0xF, false);
    case 4: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x154, 0xF, 0xF, false);
    case 5: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x155, 0xF, 0xF, false);
    case 6: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x156, 0xF, 0xF, false);
    case 7: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x157, 0xF, 0xF, false);
    case 8: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x158, 0xF, 0xF, false);
    case 9: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x159, 0xF, 0xF, false);
    case 10: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x15a, 0xF, 0xF, false);
    case 11: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x15b, 0xF, 0xF, false);
    case 12: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x15c, 0xF, 0xF, false);
    case 13: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x15d, 0xF, 0xF, false);
    case 14: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x15e, 0xF, 0xF, false);
    case 15: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x15f, 0xF, 0xF, false);
    default: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x15f, 0xF, 0xF, false);
  }
}

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

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(f16, h);
}

}  // namespace lutq
