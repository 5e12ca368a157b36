// Round-to-nearest quantization onto a lookup table (gfx950): fp32 weights
// -> one code per byte plus fp16 scales, the input of the repack; and the
// weight error sum (w - s * T[c])^2 that drives the logarithmic-base search.
//
// "PTQ-damage" abstract: round-to-nearest at group-128 granularity. FLUTE
// abstract: the grid is an arbitrary table, uniform or not. LogbQuant
// abstract: tensor-wise scales, logarithmic tables with an adjustable base.
//
// Layout: a group of 128 weights spans 8 lanes (16 weights per lane, four
// 16-byte loads), a wave takes 1024 weights per step and loads the next step
// while it codes this one. The group's extrema come from a lane reduction
// (DPP), its scale from fp64 arithmetic rounded once to fp16, and each code
// from comparisons of the fp32 weight against per-group fp32 thresholds that
// decide exactly what the fp64 quotient w / s decides against the table's
// midpoints (derivation at thr32 below): three thresholds in registers pick a
// quarter of the sorted table, one 16-byte LDS read brings that quarter's
// three thresholds and four codes. Tensor-wise scales take three launches:
// per-workgroup extrema, one reduction to the scale, then the codes.
#include <climits>

#include "lutq_quant.h"

namespace lutq {

// fp64 -> fp16 bits, round to nearest even, directly (no pass through fp32,
// which would round twice). Inputs here are finite and >= 0 or signed small
// values; infinities and NaN map to the fp16 infinity / a quiet NaN.
__host__ __device__ uint16_t f64_to_f16_rne(double d) {
  uint64_t b;
  __builtin_memcpy(&b, &d, 8);
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  const int ex = (int)((b >> 52) & 0x7FF);
  const uint64_t man = b & ((1ull << 52) - 1);
  if (ex == 0x7FF) return sign | 0x7C00u | (man ? 0x200u : 0u);
  const int e = ex - 1023;  // unbiased exponent (zero and fp64 subnormals land below)
  if (e > 15) return sign | 0x7C00u;
  const uint64_t sig = (ex ? (1ull << 52) : 0ull) | man;  // 53-bit significand
  int shift;        // bits dropped from sig
  uint32_t hexp;    // fp16 exponent field before rounding
  if (e >= -14) {   // normal fp16: keep 10 fraction bits
    shift = 42;
    hexp = (uint32_t)(e + 15);
  } else {          // subnormal fp16: units of 2^-24
    shift = 28 - e; // value / 2^-24 = sig * 2^(e - 52 + 24)
    hexp = 0;
    if (shift > 63) return sign;  // below half of the smallest subnormal
  }
  uint64_t m = sig >> shift;
  const uint64_t rem = sig & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (m & 1))) ++m;
  if (hexp == 0) return sign | (uint16_t)m;  // a carry into bit 10 is the smallest normal
  uint32_t mm = (uint32_t)(m & 0x3FF);       // drop the implicit bit
  if (m >> 11) {                             // rounding carried out of the significand
    mm = 0;
    ++hexp;
  }
  if (hexp >= 31) return sign | 0x7C00u;
  return sign | (uint16_t)((hexp << 10) | mm);
}

namespace {

struct QuantParams {
  const void* w;           // weights, fp32 or (kWeightF16 / kWeightBf16) 16-bit
  const uint16_t* lut;
  uint8_t* codes;          // null: do not write codes
  uint16_t* scales;        // null: do not write scales
  double* err_partial;     // per workgroup; null: no error
  float* extrema;          // tensor-wise: per-workgroup [max, min]
  uint16_t* tscale;        // tensor-wise: the scale (fp16 bits)
  double* acc_partial;     // table tuning: per workgroup [2][L] sums (w s, s^2) per code
  long long n;             // weights
  int N, K, group, rule;
  long long nrows;         // groups (grouped) or 128-weight pieces (tensor-wise)
};

constexpr int kQuantThreads = 256;
constexpr int kQuantWaves = kQuantThreads / kWave;
constexpr int kLaneElems = 16;                // weights per lane per step: four 16-byte loads
constexpr int kStep = kWave * kLaneElems;     // weights per wave per step (held groups)
constexpr int kPiece = 128;                   // a 128-weight piece spans 8 lanes
constexpr int kMaxAreas = kStep / kPiece;     // groups per wave per step, at most

__device__ __forceinline__ double h2d(uint16_t h) { return (double)__builtin_bit_cast(_Float16, h); }

// Weights: fp32, or fp16 / bf16 widened to fp32 (exactly) on load.
constexpr int kWeightF32 = 0, kWeightF16 = 1, kWeightBf16 = 2;

template <int WT>
__device__ __forceinline__ f32x4 widen4(u32x2 v) {
  f32x4 r;
  if constexpr (WT == kWeightF16) {
    r[0] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v.x & 0xFFFFu));
    r[1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v.x >> 16));
    r[2] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v.y & 0xFFFFu));
    r[3] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v.y >> 16));
  } else {
    r[0] = __builtin_bit_cast(float, v.x << 16);
    r[1] = __builtin_bit_cast(float, v.x & 0xFFFF0000u);
    r[2] = __builtin_bit_cast(float, v.y << 16);
    r[3] = __builtin_bit_cast(float, v.y & 0xFFFF0000u);
  }
  return r;
}

// Four weights at element offset e of a buffer resource.
template <int WT>
__device__ __forceinline__ f32x4 load_weights4(__amdgpu_buffer_rsrc_t rs, uint32_t e) {
  if constexpr (WT == kWeightF32) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, 4u * e, 0, kNontemporal));
  } else {
    return widen4<WT>(
        __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, 2u * e, 0, kNontemporal)));
  }
}

// Four weights (vector i) of a plain pointer.
template <int WT>
struct Weights4 {
  const void* base;
  __device__ __forceinline__ f32x4 at(long long i) const {
    if constexpr (WT == kWeightF32)
      return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(base) + i);
    else
      return widen4<WT>(__builtin_nontemporal_load(reinterpret_cast<const u32x2*>(base) + i));
  }
};

// The table as one lane needs it. With the L entries sorted ascending,
// midpoint m lies between sorted entries m and m + 1; lane j (mod 8) of a
// group owns midpoints j and j + 8 when the group's thresholds are built.
template <int L>
struct Table {
  double mid_a, mid_b;      // midpoints j and j + 8 (0 where they do not exist)
  bool up_a, up_b;          // an exact tie there goes to the upper entry (its code is the lower)
  uint32_t ord_lo, ord_hi;  // code of sorted entry q in bits 4(q mod 8) of ord_lo (q < 8) / ord_hi
  double tmax, tmin, amax;
};

// Sorts the table in LDS (rank by value, ties by index: entries are
// distinct) and fills the lane's view; `tval` (LDS, L entries) receives the
// entries in code order. Contains a workgroup barrier.
template <int L>
__device__ void load_table(const uint16_t* lut, Table<L>& t, double* tval) {
  __shared__ double sv[L];
  __shared__ uint32_t so[L];
  const int tid = threadIdx.x;
  if (tid < L) {
    const double v = h2d(lut[tid]);
    int rank = 0;
    for (int i = 0; i < L; ++i) {
      const double u = h2d(lut[i]);
      rank += (u < v) || (u == v && i < tid);
    }
    sv[rank] = v;
    so[rank] = (uint32_t)tid;
    tval[tid] = v;
  }
  __syncthreads();
  const int j = tid & 7;
  t.mid_a = t.mid_b = 0.0;
  t.up_a = t.up_b = false;
  if (j < L - 1) {
    t.mid_a = (sv[j] + sv[j + 1]) * 0.5;  // exact: fp16 values
    t.up_a = so[j + 1] < so[j];
  }
  if (j + 8 < L - 1) {
    t.mid_b = (sv[j + 8] + sv[j + 9]) * 0.5;
    t.up_b = so[j + 9] < so[j + 8];
  }
  t.ord_lo = t.ord_hi = 0;
#pragma unroll
  for (int q = 0; q < L; ++q) {
    if (q < 8) t.ord_lo |= so[q] << (4 * q);
    else t.ord_hi |= so[q] << (4 * (q - 8));
  }
  t.tmin = sv[0];
  t.tmax = sv[L - 1];
  t.amax = fmax(-sv[0], sv[L - 1]);
}

// fp64 -> fp16 bits, round to nearest even, for 0 <= d <= 65504: round to
// odd into fp32 (truncate, then set the last bit if anything was dropped),
// then round to nearest even into fp16. fp32 keeps 13 more significand bits
// than fp16, so the two roundings give the one correct rounding (Boldo and
// Melquiond, "Emulation of FMA and correctly rounded sums: proved algorithms
// using rounding to odd").
__device__ __forceinline__ uint16_t f16_bits(double d) {
  float f = (float)d;
  const double b = (double)f;
  if (b != d) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if (b > d) --u;
    f = __builtin_bit_cast(float, u | 1u);
  }
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// fp16 scale bits from the extrema of a group (or of the tensor).
__device__ __forceinline__ uint16_t scale_bits(float mx, float mn, int rule, double tmax,
                                               double tmin, double amax) {
  double s = rule == kRuleAbsmax ? fmax((double)mx, -(double)mn) / amax
                                 : fmax((double)mx / tmax, (double)mn / tmin);
  s = fmin(s, 65504.0);  // s >= 0 under both rules
  const uint16_t h = f16_bits(s);
  return (h & 0x7FFF) == 0 ? (uint16_t)0x3C00 : h;  // zero -> 1
}

// Why fp32 thresholds decide exactly what the fp64 quotient decides. Let w be
// an fp32 weight, s > 0 an fp16 scale and m a midpoint of two fp16 entries
// (at most 40 significant bits). t = m * s has at most 51 bits, so it is
// exact in fp64. If w / s != m, then |w / s - m| = |w - t| / s, where w - t
// is a nonzero multiple of w's last bit or of t's; either way it exceeds half
// an fp64 ulp of m, so rounding the quotient cannot reach m and
//   fl(w / s) > m  <=>  w > t,   fl(w / s) == m  <=>  w == t.
// For every fp32 w:  w > t  <=> w > (largest fp32 <= t),
//                    w >= t <=> w > (largest fp32 <  t).
// `up` picks the second form (an exact tie goes to the upper entry).
__device__ __forceinline__ float prev_f32(float f) {  // next fp32 toward -infinity (f finite)
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) == 0) return __builtin_bit_cast(float, 0x80000001u);
  return __builtin_bit_cast(float, (int32_t)u > 0 ? u - 1 : u + 1);
}
__device__ __forceinline__ float thr32(double t, bool up) {
  const float f = (float)t;  // |t| < 2^33: finite
  const double b = (double)f;
  return (up ? b >= t : b > t) ? prev_f32(f) : f;
}

// Integer keys with the order of the floats (finite values): max / min on
// them fuse with DPP moves into one instruction.
__device__ __forceinline__ int fkey(float f) {
  const int u = __builtin_bit_cast(int, f);
  return u ^ ((u >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float funkey(int k) {
  return __builtin_bit_cast(float, k ^ ((k >> 31) & 0x7FFFFFFF));
}
template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i in each half row
constexpr int kDppMirror = 0x140;      // lane i <-> 15 - i in each row

// Max and min over the G consecutive lanes of a group (G = 8 .. 64).
template <int G, bool MAX>
__device__ __forceinline__ int group_reduce(int k) {
  auto op = [](int a, int b) { return MAX ? max(a, b) : min(a, b); };
  k = op(k, dpp<kDppXor1>(k));
  k = op(k, dpp<kDppXor2>(k));
  k = op(k, dpp<kDppHalfMirror>(k));       // quads of a half row
  if constexpr (G >= 16) k = op(k, dpp<kDppMirror>(k));   // halves of a row
  if constexpr (G >= 32) k = op(k, __shfl_xor(k, 16));
  if constexpr (G >= 64) k = op(k, __shfl_xor(k, 32));
  return k;
}

// The search structure of one group, in LDS (five 16-byte rows):
//   row q < 4: thresholds 4q, 4q + 1, 4q + 2 and, in .w, the codes of sorted
//              positions 4q .. 4q + 3 (one byte each);
//   row 4    : thresholds 3, 7, 11.
// A weight's sorted position is 4q + c: q from thresholds 3 / 7 / 11 (held
// in registers), c from the three thresholds of row q; the code is byte c of
// row q's .w. Threshold m sits in slot thr_slot(m) of the 20 floats.
__device__ __forceinline__ int thr_slot(int m) { return (m & 3) == 3 ? 16 + (m >> 2) : m; }

// Codes of sorted positions 4q .. 4q + 3 as four bytes.
template <int L>
__device__ __forceinline__ uint32_t row_codes(const Table<L>& t, int q) {
  const uint32_t nib = (q < 2 ? t.ord_lo : t.ord_hi) >> (16 * (q & 1));
  return (nib & 0xF) | ((nib >> 4 & 0xF) << 8) | ((nib >> 8 & 0xF) << 16) | ((nib >> 12 & 0xF) << 24);
}

// Registers a lane keeps per group for the first level of the search.
struct Level1 { float a, b, c; f32x4 row0; };

template <int L>
__device__ __forceinline__ uint32_t code_of(float w, const Level1& l1, const f32x4* area) {
  f32x4 r;
  if constexpr (L == 16) {
    const bool b3 = w > l1.b;                       // threshold 7
    const bool b2 = w > (b3 ? l1.c : l1.a);         // threshold 11 or 3
    r = area[(b3 ? 2 : 0) + (int)b2];
  } else if constexpr (L == 8) {
    r = area[(int)(w > l1.a)];                      // threshold 3
  } else {
    r = l1.row0;
  }
  const uint32_t c = (uint32_t)(w > r[0]) + (uint32_t)(w > r[1]) + (uint32_t)(w > r[2]);
  // through a scalar: a bit cast of a vector element reads the vector's first one
  const float codes = r[3];
  return __builtin_amdgcn_ubfe(__builtin_bit_cast(uint32_t, codes), c * 8, 8);
}

// Fixed-order workgroup sum of one double per lane -> err_partial[block].
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ void block_error(double e, double* out) {
  __shared__ double we[kQuantWaves];
  e = wave_sum(e);
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & 63) == 0) we[wave] = e;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < kQuantWaves; ++i) t += we[i];
    out[blockIdx.x] = t;
  }
}

// A raw buffer resource over elements [e0, n) of `base` (`esize` bytes each):
// offsets past the end read zeros and drop stores.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tail_rsrc(const void* base, long long e0,
                                                            long long n, int esize) {
  const long long rem = n - e0;
  if (rem <= 0) return make_rsrc(base, 0);
  const long long bytes = rem * esize;
  return make_rsrc(static_cast<const char*>(base) + e0 * esize,
                   (uint32_t)(bytes < (1ll << 30) ? bytes : (1ll << 30)));
}

// Ordering of a wave's own LDS traffic: LDS executes one wave's operations
// in order, so only the compiler has to be kept from moving them.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Round-to-nearest onto the table.
// Held groups (GL > 0): a group of 16 GL weights spans GL consecutive lanes,
// 16 weights per lane (float4 i of lane j at 4 j + 4 GL i), and stays in
// registers between its extrema and its codes; a wave takes 1024 weights per
// step (64 / GL groups) and loads the next step while coding this one.
// Tensor-wise: the same with GL = 8 over 128-weight pieces and one scale.
// GL == 0: groups of any multiple of 128 over 8 lanes, read twice (extrema,
// then codes), 8 groups per step.
// ACC (table tuning): the scales are given (p.scales, or the tensor scale),
// and every weight adds w s and s^2 to its code's sums: each thread keeps its
// own sums in LDS, [part][code][thread] (lanes never share a bank), summed
// in a fixed order at the end into the workgroup's partials.
template <int L, int GL, bool ERR, bool TENSOR, int WT, bool ACC = false>
__global__ __launch_bounds__(kQuantThreads) void quant_kernel(const QuantParams p) {
  constexpr int ES = WT == kWeightF32 ? 4 : 2;  // bytes per weight
  static_assert(!ACC || ERR, "table tuning reports the error too");
  __shared__ double tval[L];
  __shared__ double tacc[ACC ? 2 : 1][ACC ? L : 1][ACC ? kQuantThreads : 1];
  if constexpr (ACC) {
#pragma unroll
    for (int c = 0; c < L; ++c) tacc[0][c][threadIdx.x] = tacc[1][c][threadIdx.x] = 0.0;
  }
  __shared__ f32x4 areas[kQuantWaves][kMaxAreas][5];
  Table<L> t;
  load_table<L>(p.lut, t, tval);
  constexpr int G = GL > 0 ? GL : 8;        // lanes per group
  constexpr int kGroups = kWave / G;        // groups per step
  const int lane = threadIdx.x & (kWave - 1);
  // wave-uniform in a scalar register, so that the buffer resources built
  // from it are too (a per-lane resource costs a loop over distinct values)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int r = lane / G;                   // group within the step
  const int j = lane % G;
  f32x4* area = areas[wave][TENSOR ? 0 : r];
  const long long gsize = TENSOR ? kPiece : p.group;          // weights per group
  const long long per_step = gsize * kGroups;
  const long long nunits = (p.nrows + kGroups - 1) / kGroups;
  const long long nwaves = (long long)gridDim.x * kQuantWaves;
  const long long wave0 = (long long)blockIdx.x * kQuantWaves + wave;

  // the codes column of every search row, once
  if (lane < kMaxAreas * 4) {
    f32x4* a = areas[wave][lane >> 2];
    a[lane & 3][3] = __builtin_bit_cast(float, row_codes<L>(t, lane & 3));
  }

  Level1 l1;
  double s = 1.0;
  // This group's thresholds for scale s16 into its area, then level 1 back.
  auto build = [&](uint16_t s16) __attribute__((always_inline)) {
    s = h2d(s16);
    wave_lds_fence();  // the previous group's reads come first
    if (j < 8) {
      if (j < L - 1) reinterpret_cast<float*>(area)[thr_slot(j)] = thr32(t.mid_a * s, t.up_a);
      if (j + 8 < L - 1)
        reinterpret_cast<float*>(area)[thr_slot(j + 8)] = thr32(t.mid_b * s, t.up_b);
    }
    wave_lds_fence();
    if constexpr (L == 4) {
      l1.row0 = area[0];
    } else {
      const f32x4 r4 = area[4];
      l1.a = r4[0];
      l1.b = r4[1];
      l1.c = r4[2];
    }
  };
  if constexpr (TENSOR) build(*p.tscale);
  else wave_lds_fence();
  double err = 0.0;

  // Scale of a group from this lane's extrema keys; store it, build the search.
  auto prepare = [&](int kmx, int kmn, long long gi) __attribute__((always_inline)) {
    const float mx = funkey(group_reduce<G, true>(kmx));
    const float mn = funkey(group_reduce<G, false>(kmn));
    const uint16_t s16 = scale_bits(mx, mn, p.rule, t.tmax, t.tmin, t.amax);
    if (p.scales && j == 0 && gi < p.nrows) p.scales[gi] = s16;
    build(s16);
  };
  // Table tuning: the group's given scale.
  auto prepare_given = [&](long long gi) __attribute__((always_inline)) {
    build(gi < p.nrows ? p.scales[gi] : (uint16_t)0x3C00);
  };
  auto extrema = [&](f32x4 v, int& kmx, int& kmn) __attribute__((always_inline)) {
    kmx = max(kmx, fkey(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]))));
    kmn = min(kmn, fkey(fminf(fminf(v[0], v[1]), fminf(v[2], v[3]))));
  };
  // Codes of four weights -> one dword of bytes; error of the active ones.
  auto code4 = [&](f32x4 v, bool active) __attribute__((always_inline)) {
    uint32_t packed = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t code = code_of<L>(v[c], l1, area);
      packed |= code << (8 * c);
      if constexpr (ERR) {
        const double d = (double)v[c] - tval[code] * s;
        err += active ? d * d : 0.0;
      }
      if constexpr (ACC) {
        if (active) {
          // LDS fp64 adds without a returned value (ds_add_f64): one LDS
          // operation each instead of a read and a write. The slots are this
          // thread's own and updated in program order, so the sums are those
          // of plain adds (no operand comes near the fp64 denormal range).
          __hip_atomic_fetch_add(&tacc[0][code][threadIdx.x], (double)v[c] * s, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WORKGROUP);
          __hip_atomic_fetch_add(&tacc[1][code][threadIdx.x], s * s, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
    }
    return packed;
  };
  // four weights at element offset `e` of the resource, as fp32 (exact)
  auto load = [&](__amdgpu_buffer_rsrc_t rs, uint32_t e) __attribute__((always_inline)) {
    return load_weights4<WT>(rs, e);
  };
  auto store = [&](__amdgpu_buffer_rsrc_t rc, uint32_t off, uint32_t v) __attribute__((always_inline)) {
    __builtin_amdgcn_raw_buffer_store_b32(v, rc, off, 0, 0);
  };

  if constexpr (GL > 0 || TENSOR) {
    const uint32_t lane_off = (uint32_t)(r * gsize + 4 * j);  // weights, from the step's start
    f32x4 bufA[4], bufB[4];
    auto fetch = [&](f32x4 (&b)[4], long long unit) __attribute__((always_inline)) {
      const auto rs = tail_rsrc(p.w, unit * per_step, p.n, ES);
#pragma unroll
      for (int i = 0; i < 4; ++i) b[i] = load(rs, lane_off + 4 * G * i);
    };
    auto step = [&](const f32x4 (&b)[4], long long unit) __attribute__((always_inline)) {
      const long long gi = unit * kGroups + r;
      if constexpr (!TENSOR && ACC) {
        prepare_given(gi);
      } else if constexpr (!TENSOR) {
        int kmx = INT_MIN, kmn = INT_MAX;
#pragma unroll
        for (int i = 0; i < 4; ++i) extrema(b[i], kmx, kmn);
        prepare(kmx, kmn, gi);
      }
      const bool active = gi < p.nrows;
      const auto rc = tail_rsrc(p.codes, unit * per_step, p.codes ? p.n : 0, 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t packed = code4(b[i], active);
        if (p.codes) store(rc, lane_off + 4 * G * i, packed);
      }
    };
    long long unit = wave0;
    if (unit < nunits) {
      fetch(bufA, unit);
      for (;;) {
        fetch(bufB, unit + nwaves);  // past the end: zeros, no memory access
        step(bufA, unit);
        unit += nwaves;
        if (unit >= nunits) break;
        fetch(bufA, unit + nwaves);
        step(bufB, unit);
        unit += nwaves;
        if (unit >= nunits) break;
      }
    }
  } else {
    const int pieces = (int)(gsize / kPiece);
    const uint32_t lane_off = (uint32_t)(r * gsize + 4 * j);
    for (long long unit = wave0; unit < nunits; unit += nwaves) {
      const long long gi = unit * kGroups + r;
      const auto rs = tail_rsrc(p.w, unit * per_step, p.n, ES);
      if constexpr (ACC) {
        prepare_given(gi);
      } else {
        int kmx = INT_MIN, kmn = INT_MAX;
        for (int q = 0; q < pieces; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) extrema(load(rs, lane_off + q * kPiece + 32 * i), kmx, kmn);
        prepare(kmx, kmn, gi);
      }
      const bool active = gi < p.nrows;
      const auto rc = tail_rsrc(p.codes, unit * per_step, p.codes ? p.n : 0, 1);
      for (int q = 0; q < pieces; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t off = lane_off + q * kPiece + 32 * i;
          const uint32_t packed = code4(load(rs, off), active);
          if (p.codes) store(rc, off, packed);
        }
    }
  }
  if constexpr (ERR) block_error(err, p.err_partial);  // contains a barrier
  if constexpr (ACC) {
    if (threadIdx.x < 2 * L) {
      const int part = threadIdx.x / L, code = threadIdx.x % L;
      double sum = 0.0;
      for (int i = 0; i < kQuantThreads; ++i) sum += tacc[part][code][i];
      p.acc_partial[((size_t)blockIdx.x * 2 + part) * L + code] = sum;
    }
  }
}

// Table tuning: the new table from all workgroups' sums, each used entry the
// fp16 value of sum(w s) / sum(s^2); an unused entry keeps its value. If that
// would repeat an fp16 value, the table stays and *stop is set. One
// workgroup of kTuneThreads: thread t adds sum t % 2L of the workgroups
// t / 2L, t / 2L + S, ... (S = kTuneThreads / 2L slots; neighbouring threads
// read neighbouring doubles), then the S slot sums are added in slot order,
// so the result does not depend on timing.
constexpr int kTuneThreads = 1024;
template <int L>
__global__ __launch_bounds__(kTuneThreads) void tune_update_kernel(const double* part, int nblocks,
                                                                   uint16_t* lut, int* stop) {
  constexpr int kSums = 2 * L, kSlots = kTuneThreads / kSums;
  __shared__ double red[kSlots][kSums];
  __shared__ uint16_t nt[L];
  __shared__ int sstop;
  const int t = threadIdx.x, sum = t % kSums, slot = t / kSums;
  double acc = 0.0;
#pragma unroll 8
  for (int b = slot; b < nblocks; b += kSlots) acc += part[(size_t)b * kSums + sum];
  red[slot][sum] = acc;
  __syncthreads();
  if (t < L) {
    double num = 0.0, den = 0.0;
    for (int j = 0; j < kSlots; ++j) {
      num += red[j][t];
      den += red[j][L + t];
    }
    nt[t] = den > 0.0 ? f64_to_f16_rne(num / den) : lut[t];
  }
  __syncthreads();
  if (t == 0) {
    bool dup = false;
    for (int a = 0; a < L; ++a)
      for (int b = a + 1; b < L; ++b) dup |= h2d(nt[a]) == h2d(nt[b]);
    sstop = dup ? 1 : 0;
    *stop = sstop;
  }
  __syncthreads();
  if (t < L && !sstop) lut[t] = nt[t];
}

// Tensor-wise, pass 1: per-workgroup max and min.
template <int WT>
__global__ __launch_bounds__(kQuantThreads) void tensor_extrema_kernel(const QuantParams p) {
  __shared__ float part[2][kQuantWaves];
  const long long nvec = p.n / 4;  // n is a multiple of 128
  float mx = -__builtin_huge_valf(), mn = __builtin_huge_valf();
  const Weights4<WT> src{p.w};
  const long long stride = (long long)gridDim.x * kQuantThreads;
  long long i = (long long)blockIdx.x * kQuantThreads + threadIdx.x;
  for (; i + 3 * stride < nvec; i += 4 * stride) {  // four loads in flight
    f32x4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = src.at(i + k * stride);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      mx = fmaxf(mx, fmaxf(fmaxf(v[k][0], v[k][1]), fmaxf(v[k][2], v[k][3])));
      mn = fminf(mn, fminf(fminf(v[k][0], v[k][1]), fminf(v[k][2], v[k][3])));
    }
  }
  for (; i < nvec; i += stride) {
    const f32x4 v = src.at(i);
    mx = fmaxf(mx, fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
    mn = fminf(mn, fminf(fminf(v[0], v[1]), fminf(v[2], v[3])));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, o));
    mn = fminf(mn, __shfl_xor(mn, o));
  }
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & 63) == 0) {
    part[0][wave] = mx;
    part[1][wave] = mn;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < kQuantWaves; ++k) {
      mx = fmaxf(mx, part[0][k]);
      mn = fminf(mn, part[1][k]);
    }
    p.extrema[2 * blockIdx.x + 0] = mx;
    p.extrema[2 * blockIdx.x + 1] = mn;
  }
}

// Tensor-wise, pass 2 (one workgroup): the scale from all partial extrema.
template <int L>
__global__ __launch_bounds__(kQuantThreads) void tensor_scale_kernel(const QuantParams p, int nparts) {
  __shared__ float part[2][kQuantWaves];
  float mx = -__builtin_huge_valf(), mn = __builtin_huge_valf();
  // (unrolled so that the loads are in flight together; max and min do not
  // depend on the order)
#pragma unroll 8
  for (int i = threadIdx.x; i < nparts; i += kQuantThreads) {
    mx = fmaxf(mx, p.extrema[2 * i + 0]);
    mn = fminf(mn, p.extrema[2 * i + 1]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, o));
    mn = fminf(mn, __shfl_xor(mn, o));
  }
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & 63) == 0) {
    part[0][wave] = mx;
    part[1][wave] = mn;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 0; k < kQuantWaves; ++k) {
      mx = fmaxf(mx, part[0][k]);
      mn = fminf(mn, part[1][k]);
    }
    double tmin = h2d(p.lut[0]), tmax = tmin;
    for (int k = 1; k < L; ++k) {
      tmin = fmin(tmin, h2d(p.lut[k]));
      tmax = fmax(tmax, h2d(p.lut[k]));
    }
    const uint16_t s16 = scale_bits(mx, mn, p.rule, tmax, tmin, fmax(-tmin, tmax));
    *p.tscale = s16;
    if (p.scales) p.scales[0] = s16;
  }
}

// Fixed-order sum of the per-workgroup errors (one workgroup).
__global__ __launch_bounds__(kQuantThreads) void error_sum_kernel(const double* part, int nparts,
                                                                   double* out) {
  __shared__ double s[kQuantThreads];
  // thread i adds parts i, i + 256, ... in that order, eight loads in flight
  // at a time (past the end a load repeats part 0 and is not added)
  double t = 0.0;
  for (int i0 = threadIdx.x; i0 < nparts; i0 += 8 * kQuantThreads) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * kQuantThreads;
      v[u] = part[i < nparts ? i : 0];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) t = i0 + u * kQuantThreads < nparts ? t + v[u] : t;
  }
  s[threadIdx.x] = t;
  __syncthreads();
  if (threadIdx.x == 0) {
    double total = 0.0;
    for (int i = 0; i < kQuantThreads; ++i) total += s[i];
    *out = total;
  }
}

template <int L, int GL, bool TENSOR, int WT>
void launch_codes(const QuantParams& p, int nblocks, bool err, hipStream_t s) {
  if (err)
    quant_kernel<L, GL, true, TENSOR, WT><<<nblocks, kQuantThreads, 0, s>>>(p);
  else
    quant_kernel<L, GL, false, TENSOR, WT><<<nblocks, kQuantThreads, 0, s>>>(p);
}

// Workgroups for `units` wave steps: one step per wave, at most kQuantMaxBlocks.
int blocks_for(long long units) {
  const long long want = (units + kQuantWaves - 1) / kQuantWaves;
  return (int)(want < kQuantMaxBlocks ? want : kQuantMaxBlocks);
}

template <int L, int WT>
hipError_t launch_l(const QuantScratch& sc, const QuantParams& p0, bool err, hipStream_t s) {
  QuantParams p = p0;
  p.err_partial = sc.err_partial;
  int nblocks;
  if (p.group != 0) {
    p.nrows = p.n / p.group;
    const int gl = p.group / kLaneElems;  // lanes per held group
    const int per_step = gl == 8 || gl == 16 || gl == 32 || gl == 64 ? kWave / gl : 8;
    nblocks = blocks_for((p.nrows + per_step - 1) / per_step);
    switch (gl) {
      case 8: launch_codes<L, 8, false, WT>(p, nblocks, err, s); break;
      case 16: launch_codes<L, 16, false, WT>(p, nblocks, err, s); break;
      case 32: launch_codes<L, 32, false, WT>(p, nblocks, err, s); break;
      case 64: launch_codes<L, 64, false, WT>(p, nblocks, err, s); break;
      default: launch_codes<L, 0, false, WT>(p, nblocks, err, s); break;
    }
  } else {
    p.extrema = sc.extrema;
    p.tscale = sc.tscale;
    p.nrows = p.n / kPiece;
    const long long want = (p.n / 4 + kQuantThreads - 1) / kQuantThreads;
    const int nx = (int)(want < kQuantMaxBlocks ? want : kQuantMaxBlocks);
    tensor_extrema_kernel<WT><<<nx, kQuantThreads, 0, s>>>(p);
    tensor_scale_kernel<L><<<1, kQuantThreads, 0, s>>>(p, nx);
    nblocks = blocks_for((p.nrows + kMaxAreas - 1) / kMaxAreas);
    launch_codes<L, 8, true, WT>(p, nblocks, err, s);
  }
  if (err) error_sum_kernel<<<1, kQuantThreads, 0, s>>>(sc.err_partial, nblocks, sc.err_total);
  return hipGetLastError();
}

template <int WT>
hipError_t launch_w(const QuantScratch& sc, const QuantParams& p, int bits, bool error,
                    hipStream_t s) {
  switch (bits) {
    case 2: return launch_l<4, WT>(sc, p, error, s);
    case 3: return launch_l<8, WT>(sc, p, error, s);
    default: return launch_l<16, WT>(sc, p, error, s);
  }
}

// One tuning pass: codes under the given scales, the error and the per-code
// sums (grouped: p.scales; tensor-wise: the scale already in sc.tscale).
template <int L, int WT>
hipError_t launch_tune_l(const QuantScratch& sc, const QuantParams& p0, hipStream_t s, int* nb) {
  QuantParams p = p0;
  p.err_partial = sc.err_partial;
  p.acc_partial = sc.acc_partial;
  int nblocks;
  if (p.group != 0) {
    p.nrows = p.n / p.group;
    const int gl = p.group / kLaneElems;
    const int per_step = gl == 8 || gl == 16 || gl == 32 || gl == 64 ? kWave / gl : 8;
    nblocks = blocks_for((p.nrows + per_step - 1) / per_step);
    switch (gl) {
      case 8: quant_kernel<L, 8, true, false, WT, true><<<nblocks, kQuantThreads, 0, s>>>(p); break;
      case 16: quant_kernel<L, 16, true, false, WT, true><<<nblocks, kQuantThreads, 0, s>>>(p); break;
      case 32: quant_kernel<L, 32, true, false, WT, true><<<nblocks, kQuantThreads, 0, s>>>(p); break;
      case 64: quant_kernel<L, 64, true, false, WT, true><<<nblocks, kQuantThreads, 0, s>>>(p); break;
      default: quant_kernel<L, 0, true, false, WT, true><<<nblocks, kQuantThreads, 0, s>>>(p); break;
    }
  } else {
    p.tscale = sc.tscale;
    p.nrows = p.n / kPiece;
    nblocks = blocks_for((p.nrows + kMaxAreas - 1) / kMaxAreas);
    quant_kernel<L, 8, true, true, WT, true><<<nblocks, kQuantThreads, 0, s>>>(p);
  }
  error_sum_kernel<<<1, kQuantThreads, 0, s>>>(sc.err_partial, nblocks, sc.err_total);
  *nb = nblocks;
  return hipGetLastError();
}

template <int WT>
hipError_t launch_tune_w(const QuantScratch& sc, const QuantParams& p, int bits, hipStream_t s,
                         int* nb) {
  switch (bits) {
    case 2: return launch_tune_l<4, WT>(sc, p, s, nb);
    case 3: return launch_tune_l<8, WT>(sc, p, s, nb);
    default: return launch_tune_l<16, WT>(sc, p, s, nb);
  }
}

}  // namespace

hipError_t launch_tune_pass(const QuantScratch& sc, const void* w, int wdtype, const uint16_t* lut,
                            int bits, int N, int K, int group, const uint16_t* scales,
                            bool update, hipStream_t s) {
  QuantParams p;
  __builtin_memset(&p, 0, sizeof p);
  p.w = w;
  p.lut = lut;
  p.scales = const_cast<uint16_t*>(scales);
  p.n = (long long)N * K;
  p.N = N;
  p.K = K;
  p.group = group;
  int nb = 0;
  hipError_t e;
  switch (wdtype) {
    case kWeightF16: e = launch_tune_w<kWeightF16>(sc, p, bits, s, &nb); break;
    case kWeightBf16: e = launch_tune_w<kWeightBf16>(sc, p, bits, s, &nb); break;
    default: e = launch_tune_w<kWeightF32>(sc, p, bits, s, &nb); break;
  }
  if (e != hipSuccess || !update) return e;
  switch (bits) {
    case 2: tune_update_kernel<4><<<1, kTuneThreads, 0, s>>>(sc.acc_partial, nb, const_cast<uint16_t*>(lut), sc.stop); break;
    case 3: tune_update_kernel<8><<<1, kTuneThreads, 0, s>>>(sc.acc_partial, nb, const_cast<uint16_t*>(lut), sc.stop); break;
    default: tune_update_kernel<16><<<1, kTuneThreads, 0, s>>>(sc.acc_partial, nb, const_cast<uint16_t*>(lut), sc.stop); break;
  }
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantScratch& sc, const void* w, int wdtype, const uint16_t* lut,
                           int bits, int N, int K, int group, int rule, uint8_t* codes,
                           uint16_t* scales, bool error, hipStream_t s) {
  QuantParams p;
  __builtin_memset(&p, 0, sizeof p);
  p.w = w;
  p.lut = lut;
  p.codes = codes;
  p.scales = scales;
  p.n = (long long)N * K;
  p.N = N;
  p.K = K;
  p.group = group;
  p.rule = rule;
  switch (wdtype) {
    case kWeightF16: return launch_w<kWeightF16>(sc, p, bits, error, s);
    case kWeightBf16: return launch_w<kWeightBf16>(sc, p, bits, error, s);
    default: return launch_w<kWeightF32>(sc, p, bits, error, s);
  }
}

}  // namespace lutq
