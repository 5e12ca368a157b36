// The fused LUT-dequantize + matmul kernels (gfx950).
//
// y[m, n] = sum_g s[n, g] * sum_{k in g} x[m, k] * T[c[n, k]]
//
// FLUTE abstract: only the packed codes travel from HBM to registers; the
// table sits in on-chip memory, vectorized (two fp16 entries per lookup) and
// duplicated against bank conflicts. BitMoD abstract: the scale multiplies
// the per-group partial sum, so table values enter the products unscaled and
// exact, and each group costs one fp32 multiply-add.
//
// Workgroup: 8 waves; the block covers 4 tiles (64 rows) and a range of
// 128-code chunks, dealt to the waves round-robin. Each wave streams the four
// 1 KiB (at 4 bits) blocks of a chunk with one coalesced load per lane,
// prefetching PF chunks ahead; codes, scales and activations of a chunk are
// loaded together so the in-order load counter never waits on a prefetch.
//
// Two compute policies share that skeleton:
//  GEMV (batch 1..8): lane L = 16q + r owns row r of a tile and k-quarter q.
//    Each lookup yields (T[c0], T[c1]); v_dot2_f32_f16 multiplies it by the
//    matching activation pair, which one VGPR per batch row holds for all
//    four quarters and a DPP row_newbcast hands to the 16 lanes of the
//    quarter. The four quarters are summed across lanes at the end.
//  MFMA (batch up to 32): the decoded pairs of k-step j are exactly the B
//    operand of v_mfma_f32_16x16x32_f16 (lane: row r, k = 32j + 8q .. +7);
//    the A operand is the matching 16x32 activation tile straight from
//    global memory (L2-resident).
// Waves are combined in LDS in a fixed order; splits along K across
// workgroups are combined by the last-arriving workgroup, again in a fixed
// order, so results are deterministic.
#include "lutq_internal.h"

namespace lutq {

template <int BITS, bool MFMA, int MROWS, bool GROUPED>
__global__ __launch_bounds__(kThreads) void matmul_kernel(const MatmulParams p) {
  constexpr int TPW = kTilesPerWg;
  constexpr int ROWS = TPW * kTileRows;
  constexpr int PF = 2;
  constexpr int MT = MFMA ? MROWS / 16 : 1;
  constexpr int SLOT = 4 * BITS;
  constexpr int BLOCK = kWave * SLOT;
  static_assert(kWaves * ROWS * MROWS <= kTableWords, "reduction buffer exceeds LDS table");

  __shared__ __attribute__((aligned(16))) uint32_t table[kTableWords];
  __shared__ int arrive_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, q = lane >> 4;
  const uint32_t lane_byte = (uint32_t)lane << 2;

  const int rb = blockIdx.x / p.ksplit;
  const int ks = blockIdx.x - rb * p.ksplit;
  const int c_begin = ks * p.cps;
  const int c_end = min(p.nchunks, c_begin + p.cps);
  const int span = max(0, c_end - c_begin);
  const int nmine = span > wave ? (span - wave + kWaves - 1) / kWaves : 0;
  const int tile0 = rb * TPW;
  const int ntl = min(TPW, p.ntiles - tile0);
  const int cpg = GROUPED ? p.group / kChunk : 1;       // chunks per group
  const int gpr = GROUPED ? p.K / p.group : 0;          // groups per row

  const uint8_t* tbase[TPW];
  size_t srow[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    tbase[t] = p.packed + (size_t)(tile0 + t) * p.nchunks * BLOCK + lane * SLOT;
    srow[t] = (size_t)min(p.N - 1, (tile0 + t) * kTileRows + r) * gpr;
  }

  // activation offsets of this lane within a chunk
  // GEMV: lane 16q + 4j + i holds the pair x[128c + 32j + 8q + 2i .. +1]
  const int gx_off = 32 * (r >> 2) + 8 * q + 2 * (r & 3);
  // MFMA: lane (row r, quarter q) holds x[row][128c + 32j + 8q .. +7]
  const int ax_off = 8 * q;

  SlotRegs<BITS> cbuf[PF][TPW];
  uint16_t sbuf[PF][TPW];
  uint32_t xbuf[PF][MFMA ? 1 : MROWS];
  u32x4 abuf[PF][MT][MFMA ? 4 : 1];

  auto issue = [&](auto S, int c) {
    constexpr int s = decltype(S)::value;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      if (t < ntl) {
        cbuf[s][t] = load_slot<BITS>(tbase[t] + (size_t)c * BLOCK);
        if constexpr (GROUPED) sbuf[s][t] = p.scales[srow[t] + c / cpg];
      }
    }
    if constexpr (!MFMA) {
#pragma unroll
      for (int m = 0; m < MROWS; ++m)
        xbuf[s][m] = (m < p.M)
            ? *reinterpret_cast<const uint32_t*>(p.x + (size_t)m * p.K + (size_t)c * kChunk + gx_off)
            : 0u;
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row = mt * 16 + r;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x4 v = {0u, 0u, 0u, 0u};
          if (row < p.M)
            v = *reinterpret_cast<const u32x4*>(p.x + (size_t)row * p.K + (size_t)c * kChunk +
                                                 32 * j + ax_off);
          abuf[s][mt][j] = v;
        }
      }
    }
  };

  float gacc[TPW][MFMA ? 1 : MROWS];
  f32x4 macc[TPW][MT];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
#pragma unroll
    for (int m = 0; m < (MFMA ? 1 : MROWS); ++m) gacc[t][m] = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) macc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto compute = [&](auto S, int c) {
    constexpr int s = decltype(S)::value;
    (void)c;
    if constexpr (!MFMA) {
      // k-step outer, tile inner: each activation broadcast serves all tiles
      float cs[TPW][MROWS];
#pragma unroll
      for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int m = 0; m < MROWS; ++m) cs[t][m] = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t idx4[TPW];
#pragma unroll
        for (int t = 0; t < TPW; ++t) idx4[t] = t < ntl ? step_indices<BITS>(cbuf[s][t], j) : 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // row_newbcast:(4j+i): every lane of a 16-lane row reads lane 4j+i of that row
          uint32_t xv[MROWS];
#pragma unroll
          for (int m = 0; m < MROWS; ++m) xv[m] = row_newbcast(xbuf[s][m], 4 * j + i);
#pragma unroll
          for (int t = 0; t < TPW; ++t) {
            if (t >= ntl) continue;
            const uint32_t pr = lds_load(table, pair_addr(idx4[t], lane_byte, i));
#pragma unroll
            for (int m = 0; m < MROWS; ++m)
              cs[t][m] = __builtin_amdgcn_fdot2(as_f16x2(xv[m]), as_f16x2(pr), cs[t][m], false);
          }
        }
      }
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        if (t >= ntl) continue;
        if constexpr (GROUPED) {
          const float sc = f16_bits_to_f32(sbuf[s][t]);
#pragma unroll
          for (int m = 0; m < MROWS; ++m) gacc[t][m] = __builtin_fmaf(sc, cs[t][m], gacc[t][m]);
        } else {
#pragma unroll
          for (int m = 0; m < MROWS; ++m) gacc[t][m] += cs[t][m];
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        if (t >= ntl) continue;
        f32x4 cg[MT];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t idx4 = step_indices<BITS>(cbuf[s][t], j);
          u32x4 bq;
          bq.x = lds_load(table, pair_addr(idx4, lane_byte, 0));
          bq.y = lds_load(table, pair_addr(idx4, lane_byte, 1));
          bq.z = lds_load(table, pair_addr(idx4, lane_byte, 2));
          bq.w = lds_load(table, pair_addr(idx4, lane_byte, 3));
          const f16x8 b = __builtin_bit_cast(f16x8, bq);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const f16x8 a = __builtin_bit_cast(f16x8, abuf[s][mt][j]);
            if constexpr (GROUPED) {
              cg[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                  a, b, j == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : cg[mt], 0, 0, 0);
            } else {
              macc[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, macc[t][mt], 0, 0, 0);
            }
          }
        }
        if constexpr (GROUPED) {
          const float sc = f16_bits_to_f32(sbuf[s][t]);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) macc[t][mt][e] = __builtin_fmaf(sc, cg[mt][e], macc[t][mt][e]);
        }
      }
    }
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  static_assert(PF == 2, "pipeline written for two stages");

  const int cw = c_begin + wave;  // this wave's chunks: cw, cw + 8, cw + 16, ...
  if (nmine > 0) issue(S0{}, cw);
  if (nmine > 1) issue(S1{}, cw + kWaves);

  build_pair_table<BITS>(table, p.lut, tid, kThreads);
  __syncthreads();

  for (int i0 = 0; i0 < nmine; i0 += PF) {
    compute(S0{}, cw + i0 * kWaves);
    if (i0 + 2 < nmine) issue(S0{}, cw + (i0 + 2) * kWaves);
    if (i0 + 1 < nmine) {
      compute(S1{}, cw + (i0 + 1) * kWaves);
      if (i0 + 3 < nmine) issue(S1{}, cw + (i0 + 3) * kWaves);
    }
  }

  // ---- combine the waves (fixed order) ------------------------------------
  __syncthreads();  // every wave is done with the table; reuse it
  float* red = reinterpret_cast<float*>(table);  // [kWaves][ROWS][MROWS]
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    if constexpr (!MFMA) {
#pragma unroll
      for (int m = 0; m < MROWS; ++m) {
        float v = gacc[t][m];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (q == 0) red[(wave * ROWS + t * kTileRows + r) * MROWS + m] = v;
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          red[(wave * ROWS + t * kTileRows + r) * MROWS + mt * 16 + 4 * q + e] = macc[t][mt][e];
    }
  }
  __syncthreads();

  const float tscale = GROUPED ? 1.f : f16_bits_to_f32(p.scales[0]);
  const int items = ROWS * p.M;
  for (int it = tid; it < items; it += kThreads) {
    const int m = it / ROWS, row = it - m * ROWS;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += red[(w * ROWS + row) * MROWS + m];
    v *= tscale;
    const int n = tile0 * kTileRows + row;
    if (p.ksplit == 1) {
      if (n < p.N) p.y[(size_t)m * p.N + n] = f32_to_f16_bits(v);
    } else {
      float* dst = p.partial + (((size_t)rb * p.ksplit + ks) * MROWS + m) * ROWS + row;
      __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (p.ksplit == 1) return;

  // ---- split-K: the last workgroup of this row block sums the splits ------
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t old =
        __hip_atomic_fetch_add(p.counters + rb, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    arrive_last = (old == (uint32_t)(p.ksplit - 1));
  }
  __syncthreads();
  if (!arrive_last) return;
  __threadfence();
  for (int it = tid; it < items; it += kThreads) {
    const int m = it / ROWS, row = it - m * ROWS;
    const int n = tile0 * kTileRows + row;
    float v = 0.f;
    for (int k2 = 0; k2 < p.ksplit; ++k2)
      v += __hip_atomic_load(p.partial + (((size_t)rb * p.ksplit + k2) * MROWS + m) * ROWS + row,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (n < p.N) p.y[(size_t)m * p.N + n] = f32_to_f16_bits(v);
  }
  if (tid == 0) __hip_atomic_store(p.counters + rb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int BITS, bool MFMA, int MROWS>
static hipError_t launch_t(const MatmulParams& p, hipStream_t s) {
  const int nrb = row_blocks(p.ntiles);
  const dim3 grid((unsigned)nrb * (unsigned)p.ksplit);
  if (p.group != 0)
    matmul_kernel<BITS, MFMA, MROWS, true><<<grid, kThreads, 0, s>>>(p);
  else
    matmul_kernel<BITS, MFMA, MROWS, false><<<grid, kThreads, 0, s>>>(p);
  return hipGetLastError();
}

template <int BITS>
static hipError_t launch_bits(const MatmulParams& p, int path, hipStream_t s) {
  if (path == kPathMfma) {
    if (p.M <= 16) return launch_t<BITS, true, 16>(p, s);
    return launch_t<BITS, true, 32>(p, s);
  }
  if (p.M <= 1) return launch_t<BITS, false, 1>(p, s);
  if (p.M <= 2) return launch_t<BITS, false, 2>(p, s);
  if (p.M <= 4) return launch_t<BITS, false, 4>(p, s);
  return launch_t<BITS, false, 8>(p, s);
}

hipError_t launch_matmul(const MatmulParams& p, int bits, int path, hipStream_t s) {
  switch (bits) {
    case 2: return launch_bits<2>(p, path, s);
    case 3: return launch_bits<3>(p, path, s);
    default: return launch_bits<4>(p, path, s);
  }
}

}  // namespace lutq
