// Round-to-nearest quantization onto a lookup table (gfx950): fp32 weights
// -> one code per byte plus fp16 scales, the input of the repack; and the
// weight error sum (w - s * T[c])^2 that drives the logarithmic-base search.
//
// "PTQ-damage" abstract: round-to-nearest at group-128 granularity. FLUTE
// abstract: the grid is an arbitrary table, uniform or not. LogbQuant
// abstract: tensor-wise scales, logarithmic tables with an adjustable base.
//
// One wave per group (grouped scales): lanes hold consecutive element pairs,
// the group's max / min / |max| come from a wave reduction, the scale from
// fp64 arithmetic rounded once to fp16, and every code from the fp64
// quotient w / s compared exactly against the table's midpoints. Tensor-wise
// scales take three launches: per-workgroup extrema, one reduction to the
// scale, then the codes.
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
  const float* w;
  const uint16_t* lut;
  uint8_t* codes;          // null: do not write codes
  uint16_t* scales;        // null: do not write scales
  double* err_partial;     // per workgroup; null: no error
  float* extrema;          // tensor-wise: per-workgroup [max, min, |max|]
  uint16_t* tscale;        // tensor-wise: the scale (fp16 bits)
  long long n;             // elements (tensor-wise kernels)
  int N, K, group, rule;
  long long ngroups;       // groups of `group` elements (grouped kernel)
};

constexpr int kQuantThreads = 256;
constexpr int kQuantWaves = kQuantThreads / kWave;

__device__ inline double h2d(uint16_t h) { return (double)__builtin_bit_cast(_Float16, h); }

// The table, sorted: midpoints between neighbours, the code of each sorted
// entry and the lower code of each neighbour pair (for exact ties).
template <int L>
struct Grid {
  double mid[L - 1];
  uint32_t ord[L];
  uint32_t tie[L - 1];
  double tmax, tmin, amax;
};

template <int L>
__device__ void load_grid(const uint16_t* lut, Grid<L>& g) {
  __shared__ double sv[L];
  __shared__ uint32_t so[L];
  const int tid = threadIdx.x;
  if (tid < L) {
    const double v = h2d(lut[tid]);
    int rank = 0;
    for (int j = 0; j < L; ++j) {
      const double u = h2d(lut[j]);
      rank += (u < v) || (u == v && j < tid);
    }
    sv[rank] = v;
    so[rank] = (uint32_t)tid;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < L; ++j) g.ord[j] = so[j];
#pragma unroll
  for (int j = 0; j + 1 < L; ++j) {
    g.mid[j] = (sv[j] + sv[j + 1]) * 0.5;  // exact: fp16 values
    g.tie[j] = min(so[j], so[j + 1]);
  }
  g.tmin = sv[0];
  g.tmax = sv[L - 1];
  g.amax = fmax(-sv[0], sv[L - 1]);
}

// Code of the entry nearest to r; an exact tie to the lower code.
template <int L>
__device__ inline uint32_t nearest_code(double r, const Grid<L>& g) {
  uint32_t c = g.ord[0];
#pragma unroll
  for (int j = 0; j + 1 < L; ++j) c = r > g.mid[j] ? g.ord[j + 1] : (r == g.mid[j] ? g.tie[j] : c);
  return c;
}

// fp16 scale bits from the extrema of a group (or of the tensor).
template <int L>
__device__ inline uint16_t scale_bits(float mx, float mn, float am, int rule, const Grid<L>& g) {
  double s = rule == kRuleAbsmax ? (double)am / g.amax
                                      : fmax((double)mx / g.tmax, (double)mn / g.tmin);
  s = fmin(s, 65504.0);
  uint16_t h = f64_to_f16_rne(s);
  if ((h & 0x7FFF) == 0) h = 0x3C00;  // zero -> 1
  return h;
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ inline float wave_min(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o));
  return v;
}
__device__ inline double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Fixed-order workgroup sum of one double per wave -> err_partial[block].
__device__ inline void block_error(double e, double* out) {
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

// Codes (and error) for the pair of weights (w0, w1) under scale s16.
template <int L, bool ERR>
__device__ inline uint32_t code_pair(float w0, float w1, uint16_t s16, const Grid<L>& g,
                                     const uint16_t* lut, double& err) {
  const double s = h2d(s16);
  const uint32_t c0 = nearest_code<L>((double)w0 / s, g);
  const uint32_t c1 = nearest_code<L>((double)w1 / s, g);
  if constexpr (ERR) {
    const double d0 = (double)w0 - h2d(lut[c0]) * s;
    const double d1 = (double)w1 - h2d(lut[c1]) * s;
    err += d0 * d0 + d1 * d1;
  }
  return c0 | (c1 << 8);
}

// Grouped scales: one wave per group, groups dealt round-robin to waves.
template <int L, bool ERR>
__global__ __launch_bounds__(kQuantThreads) void quant_group_kernel(const QuantParams p) {
  Grid<L> g;
  load_grid<L>(p.lut, g);
  const int lane = threadIdx.x & 63;
  const long long nwaves = (long long)gridDim.x * kQuantWaves;
  const int gpr = p.K / p.group;
  const int pieces = p.group / kChunk;  // 128 elements per piece, 2 per lane
  double err = 0.0;
  for (long long gi = (long long)blockIdx.x * kQuantWaves + threadIdx.x / kWave; gi < p.ngroups;
       gi += nwaves) {
    const long long row = gi / gpr;
    const long long e0 = row * p.K + (gi - row * gpr) * (long long)p.group;
    const float2* src = reinterpret_cast<const float2*>(p.w + e0) + lane;
    float mx = -__builtin_huge_valf(), mn = __builtin_huge_valf(), am = 0.f;
    for (int i = 0; i < pieces; ++i) {
      const float2 v = src[i * kWave];
      mx = fmaxf(mx, fmaxf(v.x, v.y));
      mn = fminf(mn, fminf(v.x, v.y));
      am = fmaxf(am, fmaxf(fabsf(v.x), fabsf(v.y)));
    }
    mx = wave_max(mx);
    mn = wave_min(mn);
    am = wave_max(am);
    const uint16_t s16 = scale_bits<L>(mx, mn, am, p.rule, g);
    if (p.scales && lane == 0) p.scales[gi] = s16;
    for (int i = 0; i < pieces; ++i) {
      const float2 v = src[i * kWave];
      const uint32_t cc = code_pair<L, ERR>(v.x, v.y, s16, g, p.lut, err);
      if (p.codes)
        *reinterpret_cast<uint16_t*>(p.codes + e0 + 2 * (i * kWave + lane)) = (uint16_t)cc;
    }
  }
  if constexpr (ERR) block_error(err, p.err_partial);
}

// Tensor-wise, pass 1: per-workgroup max, min, |max| over pairs of weights.
__global__ __launch_bounds__(kQuantThreads) void tensor_extrema_kernel(const QuantParams p) {
  __shared__ float part[3][kQuantWaves];
  const long long npairs = p.n / 2;
  float mx = -__builtin_huge_valf(), mn = __builtin_huge_valf(), am = 0.f;
  const float2* src = reinterpret_cast<const float2*>(p.w);
  for (long long i = (long long)blockIdx.x * kQuantThreads + threadIdx.x; i < npairs;
       i += (long long)gridDim.x * kQuantThreads) {
    const float2 v = src[i];
    mx = fmaxf(mx, fmaxf(v.x, v.y));
    mn = fminf(mn, fminf(v.x, v.y));
    am = fmaxf(am, fmaxf(fabsf(v.x), fabsf(v.y)));
  }
  mx = wave_max(mx);
  mn = wave_min(mn);
  am = wave_max(am);
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & 63) == 0) {
    part[0][wave] = mx;
    part[1][wave] = mn;
    part[2][wave] = am;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < kQuantWaves; ++i) {
      mx = fmaxf(mx, part[0][i]);
      mn = fminf(mn, part[1][i]);
      am = fmaxf(am, part[2][i]);
    }
    p.extrema[3 * blockIdx.x + 0] = mx;
    p.extrema[3 * blockIdx.x + 1] = mn;
    p.extrema[3 * blockIdx.x + 2] = am;
  }
}

// Tensor-wise, pass 2 (one workgroup): the scale from all partial extrema.
template <int L>
__global__ __launch_bounds__(kQuantThreads) void tensor_scale_kernel(const QuantParams p, int nparts) {
  Grid<L> g;
  load_grid<L>(p.lut, g);
  float mx = -__builtin_huge_valf(), mn = __builtin_huge_valf(), am = 0.f;
  for (int i = threadIdx.x; i < nparts; i += kQuantThreads) {
    mx = fmaxf(mx, p.extrema[3 * i + 0]);
    mn = fminf(mn, p.extrema[3 * i + 1]);
    am = fmaxf(am, p.extrema[3 * i + 2]);
  }
  __shared__ float part[3][kQuantWaves];
  mx = wave_max(mx);
  mn = wave_min(mn);
  am = wave_max(am);
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & 63) == 0) {
    part[0][wave] = mx;
    part[1][wave] = mn;
    part[2][wave] = am;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 0; i < kQuantWaves; ++i) {
      mx = fmaxf(mx, part[0][i]);
      mn = fminf(mn, part[1][i]);
      am = fmaxf(am, part[2][i]);
    }
    const uint16_t s16 = scale_bits<L>(mx, mn, am, p.rule, g);
    *p.tscale = s16;
    if (p.scales) p.scales[0] = s16;
  }
}

// Tensor-wise, pass 3: codes (and error) under the one scale.
template <int L, bool ERR>
__global__ __launch_bounds__(kQuantThreads) void tensor_codes_kernel(const QuantParams p) {
  Grid<L> g;
  load_grid<L>(p.lut, g);
  const uint16_t s16 = *p.tscale;
  const long long npairs = p.n / 2;
  const float2* src = reinterpret_cast<const float2*>(p.w);
  double err = 0.0;
  for (long long i = (long long)blockIdx.x * kQuantThreads + threadIdx.x; i < npairs;
       i += (long long)gridDim.x * kQuantThreads) {
    const float2 v = src[i];
    const uint32_t cc = code_pair<L, ERR>(v.x, v.y, s16, g, p.lut, err);
    if (p.codes) *reinterpret_cast<uint16_t*>(p.codes + 2 * i) = (uint16_t)cc;
  }
  if constexpr (ERR) block_error(err, p.err_partial);
}

// Fixed-order sum of the per-workgroup errors (one workgroup).
__global__ __launch_bounds__(kQuantThreads) void error_sum_kernel(const double* part, int nparts,
                                                                   double* out) {
  __shared__ double s[kQuantThreads];
  double t = 0.0;
  for (int i = threadIdx.x; i < nparts; i += kQuantThreads) t += part[i];
  s[threadIdx.x] = t;
  __syncthreads();
  if (threadIdx.x == 0) {
    double total = 0.0;
    for (int i = 0; i < kQuantThreads; ++i) total += s[i];
    *out = total;
  }
}

template <int L>
hipError_t launch_l(const QuantScratch& sc, const QuantParams& p0, bool err, hipStream_t s) {
  QuantParams p = p0;
  p.err_partial = sc.err_partial;
  int nblocks;
  if (p.group != 0) {
    const long long want = (p.ngroups + kQuantWaves - 1) / kQuantWaves;
    nblocks = (int)(want < kQuantMaxBlocks ? want : kQuantMaxBlocks);
    if (err)
      quant_group_kernel<L, true><<<nblocks, kQuantThreads, 0, s>>>(p);
    else
      quant_group_kernel<L, false><<<nblocks, kQuantThreads, 0, s>>>(p);
  } else {
    p.extrema = sc.extrema;
    p.tscale = sc.tscale;
    const long long want = (p.n / 2 + kQuantThreads - 1) / kQuantThreads;
    nblocks = (int)(want < kQuantMaxBlocks ? want : kQuantMaxBlocks);
    tensor_extrema_kernel<<<nblocks, kQuantThreads, 0, s>>>(p);
    tensor_scale_kernel<L><<<1, kQuantThreads, 0, s>>>(p, nblocks);
    if (err)
      tensor_codes_kernel<L, true><<<nblocks, kQuantThreads, 0, s>>>(p);
    else
      tensor_codes_kernel<L, false><<<nblocks, kQuantThreads, 0, s>>>(p);
  }
  if (err) error_sum_kernel<<<1, kQuantThreads, 0, s>>>(sc.err_partial, nblocks, sc.err_total);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const QuantScratch& sc, const float* w, const uint16_t* lut, int bits,
                           int N, int K, int group, int rule, uint8_t* codes, uint16_t* scales,
                           bool error, hipStream_t s) {
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
  p.ngroups = group ? p.n / group : 0;
  switch (bits) {
    case 2: return launch_l<4>(sc, p, error, s);
    case 3: return launch_l<8>(sc, p, error, s);
    default: return launch_l<16>(sc, p, error, s);
  }
}

}  // namespace lutq
