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
// Workgroup: 4 or 8 waves; the block covers TPW tiles of 16 rows (1 to 8)
// and a range of 128-code chunks, dealt to the waves round-robin. Each wave
// streams the TPW 1 KiB (at 4 bits) blocks of a chunk, one coalesced load per
// lane and tile, keeping several chunks in flight; codes, scales and
// activations of a chunk are loaded together so the in-order load counter
// never waits on a prefetch.
//
// Two compute policies share that skeleton:
//  GEMV (batch 1..8): lane L = 16q + r owns row r of a tile and k-quarter q.
//    Each lookup yields (T[c0], T[c1]); v_dot2_f32_f16 multiplies it by the
//    matching activation pair, which one VGPR per batch row holds for all
//    four quarters and a DPP row_newbcast hands to the 16 lanes of the
//    quarter. The four quarters are summed across lanes at the end.
//  MFMA (batch up to 32): the decoded pairs of k-step j are exactly the B
//    operand of v_mfma_f32_16x16x32_f16 (lane: row r, k = 32j + 8q .. +7);
//    the A operand is the matching 16x32 activation tile, loaded from
//    global memory (L2-resident) in fragment order, or (8-wave shapes from
//    9 batch rows) loaded row-contiguous and rearranged through LDS.
// Binary-coded weights (AlphaTuning abstract: binary planes and separate
// scaling factors) run the same skeleton with one partial sum per plane: the
// GEMV reads each pair's plane bits from an LDS table, the MFMA path decodes
// them in registers (bcq_planes_decode) and needs no table.
// Waves are combined in LDS in a fixed order; splits along K across
// workgroups are combined by the last-arriving workgroup, again in a fixed
// order, so results are deterministic.
#include "lutq_internal.h"


namespace lutq {

// BITS: code width; MFMA: compute policy; MROWS: batch rows per launch;
// GROUPED: per-group (else per-tensor) scales; PF: register slots of the load
// pipeline (PF - 1 chunks in flight while one is computed);
// TPW: 16-row tiles per wave (and per workgroup); WAVES: waves per workgroup,
// which split the K range; OCC: waves per SIMD the register budget targets;
// XS: MFMA activations staged through LDS (see below).
template <int BITS, bool MFMA, int MROWS, bool GROUPED, bool ZP, bool TYPED, bool BCQ, bool BF16, int PF,
          int TPW, int WAVES, int OCC, bool XS>
__global__ __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(OCC)))
void matmul_kernel(const MatmulParams pk) {
  // A fused launch covers several matrices: this workgroup's row block picks
  // its matrix (a wave-uniform scan of at most kMaxSegments entries) and
  // works on it exactly as a launch of that matrix alone would.
  MatmulParams p = pk;
  int rb_base = 0;
  if (pk.nseg > 1) {
    const int rbg = blockIdx.x / pk.ksplit;
    int si = 0;
#pragma unroll
    for (int i = 1; i < kMaxSegments; ++i)
      if (i < pk.nseg && rbg >= pk.seg[i].rb_begin) si = i;
    p.packed = pk.seg[si].packed;
    p.lut = pk.seg[si].lut;
    p.scales = pk.seg[si].scales;
    p.zeros = pk.seg[si].zeros;
    p.y = pk.seg[si].y;
    p.N = pk.seg[si].N;
    p.ntiles = pk.seg[si].ntiles;
    rb_base = pk.seg[si].rb_begin;
  }
  constexpr int kThreads = WAVES * kWave;
  constexpr int kWaves = WAVES;
  // Binary-coded weights: BITS planes, one alpha stream per plane in place
  // of the scales, and plane sums (zero points' activation sums included).
  static_assert(!BCQ || (GROUPED && !ZP && !TYPED), "binary coding has its own parameters");
  static_assert(!BF16 || (!ZP && !TYPED && !BCQ), "bf16 activations: plain tables only");
  constexpr int QS = BCQ ? BITS : 1;      // scale-like streams (alpha planes)
  constexpr bool XSUM = ZP || BCQ;        // needs the groups' activation sums
  constexpr int ROWS = TPW * kTileRows;
  constexpr int MT = MFMA ? MROWS / 16 : 1;
  // Staged (XS): activations are loaded row-contiguous and turned into
  // fragments through a per-wave LDS area (see compute), XL loads of 4 rows
  // per chunk. The launch picks it for 8-wave shapes only: at one wave per
  // SIMD the LDS round trip sits in the wave's critical path and costs more
  // than the scattered loads it replaces (measured).
  static_assert(!XS || MFMA, "staging feeds MFMA fragments");
  constexpr int XL = MROWS / 4;
  constexpr int kXRowBytes = 2 * kChunk;                 // one row of a chunk
  constexpr int kXStageWords = MROWS * kXRowBytes / 4;   // per wave (4 or 8 KiB)
  constexpr int SLOT = 4 * BITS;
  constexpr int BLOCK = kWave * SLOT;
  static_assert(PF >= 2, "at least one chunk in flight while another is computed");
  // Cross-wave reduction buffer (reuses the LDS of the table and the
  // activation staging areas): [wave][m][row] with a row pitch of ROWS + 4,
  // so that the MFMA accumulator stores (lanes r, q -> rows r, batch rows
  // 4q + e) and the row-contiguous final reads both spread over distinct
  // banks.
  constexpr int RP = ROWS + 4;
  static_assert(ROWS % 16 == 0, "pitch rule assumes whole tiles");
  constexpr int kRedWords = kWaves * MROWS * RP;
  // Binary-coded weights on the MFMA path decode their planes in registers
  // and need no table.
  constexpr int kTabWords = (BCQ && MFMA) ? 0 : kTableWords;
  constexpr int kMainWords = kTabWords + (XS ? kWaves * kXStageWords : 0);
  constexpr int kLdsWords = kRedWords > kMainWords ? kRedWords : kMainWords;
  static_assert(kThreads >= kPairEntries, "table build needs one thread per entry");

  __shared__ __attribute__((aligned(16))) uint32_t table[kLdsWords];
  uint32_t* const xstage = table + kTabWords;  // staged: per-wave areas
  __shared__ int arrive_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, q = lane >> 4;
  // LDS lane byte: this lane's copy of every table entry (BCQ entries are
  // 8 or 16 bytes, kBcqEntryBytes<BITS>, with 256 / that many copies)
  const uint32_t lane_byte =
      BCQ ? ((uint32_t)lane & (kCopyBytes / kBcqEntryBytes<BITS> - 1)) * kBcqEntryBytes<BITS>
          : (uint32_t)lane << 2;

  // The table values, one per lane (lanes >= 2^BITS repeat the table).
  // Read with wave-uniform (scalar) loads: they do not queue behind the
  // vector loads of the code stream, so the LDS table is ready early.
  uint32_t lut_lane = 0;
  if constexpr (TYPED) lut_lane = typed_lut_lane<BITS>(p.lut, p.ntypes, lane);
  else if constexpr (!BCQ) lut_lane = lut_to_lanes<BITS>(p.lut, lane);

  const int rb = blockIdx.x / p.ksplit;            // row block of the launch (split-K slots)
  const int ks = blockIdx.x - rb * p.ksplit;
  const int rbm = rb - rb_base;                     // row block within its matrix
  const int c_begin = ks * p.cps;
  const int c_end = min(p.nchunks, c_begin + p.cps);
  const int span = max(0, c_end - c_begin);
  // this wave's chunks: cw, cw + WAVES, cw + 2 WAVES, ... (nmine of them)
  const int cw = c_begin + wave;
  const int nmine = span > wave ? (span - wave + kWaves - 1) / kWaves : 0;
  // Scales come in batches of SB steps (see below); the pipeline loop is
  // unrolled over U steps, a multiple of both PF and SB, so register slots
  // and batch positions are compile-time constants.
  constexpr int SB = 4;
  constexpr int U = !GROUPED || PF % SB == 0 ? PF : (SB % PF == 0 ? SB : PF * SB);
  static_assert(U == PF || U == 2 * PF, "the loop tail below covers one slot round");
  const int nsteps = (nmine + PF - 1) / PF * PF;
  const int tile0 = rbm * TPW;
  const int cpg = GROUPED ? p.group / kChunk : 1;       // chunks per group
  const int gpr = GROUPED ? p.K / p.group : 0;          // groups per row

  // Every pipeline step issues the same loads, so the in-order load counter
  // is waited on exactly. The loads go through raw buffer resources that
  // cover exactly this workgroup's data; steps past the wave's last chunk
  // use an out-of-range offset, and tiles and rows past the end of the
  // matrix or batch fall outside the resource, so they read zeros without
  // a memory access. Their results are never stored.
  const int tiles_here = min(TPW, p.ntiles - tile0);
  const uint32_t tile_bytes = (uint32_t)p.nchunks * BLOCK;
  const __amdgpu_buffer_rsrc_t crsrc =
      make_rsrc(p.packed + (size_t)tile0 * tile_bytes, (uint32_t)tiles_here * tile_bytes);
  const uint32_t lane_off = (uint32_t)lane * SLOT;
  uint32_t coff[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) coff[t] = (uint32_t)t * tile_bytes + lane_off;

  // Scales of this block's rows, [rows][groups]. One 2-byte load per tile
  // fetches a batch of SB = 4 steps: lane (q, r) takes row 16t + r at the
  // group of step 4b + q. Each step then hands its lane row to all four lane
  // rows with ds_bpermute, so a step costs no scale load of its own (a
  // per-step load touches 16 cache lines, one per row, for 32 bytes).
  const int row0 = tile0 * kTileRows;
  const uint32_t rows_here = (uint32_t)min(ROWS, p.N - row0);
  // (binary coding: plane p's alphas [N][groups] follow plane p - 1's)
  __amdgpu_buffer_rsrc_t srsrc[QS];
#pragma unroll
  for (int pl = 0; pl < QS; ++pl)
    srsrc[pl] = make_rsrc(p.scales + ((size_t)pl * p.N + row0) * gpr,
                          GROUPED ? rows_here * (uint32_t)gpr * 2u : 0u);
  uint32_t soff[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) soff[t] = 2u * (uint32_t)(t * kTileRows + r) * (uint32_t)gpr;
  // Zero points (same layout and batching as the scales). A matrix without
  // them gets an empty resource: every load reads z = 0, and s * (acc - 0)
  // is the plain rescale.
  const __amdgpu_buffer_rsrc_t zrsrc = make_rsrc(
      ZP ? p.zeros + (size_t)row0 * gpr : nullptr,
      ZP && p.zeros ? rows_here * (uint32_t)gpr * 2u : 0u);
  // Data type ids, one byte per group, batched like the scales.
  const __amdgpu_buffer_rsrc_t trsrc = make_rsrc(
      TYPED ? p.types + (size_t)row0 * gpr : nullptr, TYPED ? rows_here * (uint32_t)gpr : 0u);

  // activations of this launch's M rows
  const __amdgpu_buffer_rsrc_t xrsrc =
      make_rsrc(p.x, 2u * (uint32_t)p.M * (uint32_t)p.K);
  // GEMV: lane 16q + 4j + i holds the pair x[m][128c + 32j + 8q + 2i .. +1]
  uint32_t xoff[MFMA ? 1 : MROWS];
  if constexpr (!MFMA) {
    const uint32_t gx_boff = 2u * (32 * (r >> 2) + 8 * q + 2 * (r & 3));
#pragma unroll
    for (int m = 0; m < MROWS; ++m)
      xoff[m] = m < p.M ? 2u * (uint32_t)m * (uint32_t)p.K + gx_boff : kRowOutOfRange;
  }
  // MFMA: lane (row r, quarter q) holds x[row][128c + 32j + 8q .. +7]
  uint32_t aboff[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    aboff[mt] = mt * 16 + r < p.M ? 2u * ((uint32_t)(mt * 16 + r) * (uint32_t)p.K + 8 * q)
                                  : kRowOutOfRange;
  // Staged: load i brings rows 4i .. 4i + 3 of the chunk, lane 16v + u the
  // 16-byte piece u (k = 8u .. 8u + 7) of row 4i + v, so each row is one
  // contiguous 256-byte run (the fragment order above puts 16 rows in 16
  // consecutive lanes: 64 separate accesses per load)
  uint32_t xloff[XS ? XL : 1];
  if constexpr (XS) {
#pragma unroll
    for (int i = 0; i < XL; ++i) {
      const int row = 4 * i + (lane >> 4);
      xloff[i] = row < p.M ? 2u * (uint32_t)row * (uint32_t)p.K + 16u * (uint32_t)(lane & 15)
                           : kRowOutOfRange;
    }
  }

  SlotRegs<BITS> cbuf[PF][TPW];
  uint32_t scur[QS][TPW], snext[QS][TPW];  // scale (alpha) batches: in use, in flight
  uint32_t zcur[ZP ? TPW : 1], znext[ZP ? TPW : 1];  // zero-point batches
  uint32_t tcur[TYPED ? TPW : 1], tnext[TYPED ? TPW : 1];  // type-id batches
  uint32_t xbuf[PF][MFMA ? 1 : MROWS];
  u32x4 abuf[PF][MT][MFMA ? 4 : 1];
  u32x4 xl[XS ? PF : 1][XS ? XL : 1];  // staged: the row-contiguous pieces

  // chunk of pipeline step i, or -1 past the wave's last chunk
  auto chunk = [&](int i) { return i < nmine ? cw + i * kWaves : -1; };

  auto issue = [&](auto S, int c) __attribute__((always_inline)) {
    constexpr int s = decltype(S)::value;
    const bool live = c >= 0;  // wave-uniform
    // Activations first, then the codes tile by tile: the load counter
    // drains in issue order, so tile t can be computed as soon as its own
    // codes have landed, while the later tiles' codes are still in flight.
    const uint32_t xb = live ? (uint32_t)c * (2 * kChunk) : kOutOfRange;
    if constexpr (!MFMA) {
#pragma unroll
      for (int m = 0; m < MROWS; ++m)
        xbuf[s][m] = __builtin_amdgcn_raw_buffer_load_b32(xrsrc, xoff[m] + xb, 0, 0);
    } else if constexpr (XS) {
#pragma unroll
      for (int i = 0; i < XL; ++i)
        xl[s][i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrsrc, xloff[i] + xb, 0, 0));
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          abuf[s][mt][j] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrsrc, aboff[mt] + xb + 64 * j, 0, 0));
    }
    const uint32_t cb = live ? (uint32_t)c * BLOCK : kOutOfRange;
#pragma unroll
    for (int t = 0; t < TPW; ++t) cbuf[s][t] = load_slot<BITS>(crsrc, coff[t] + cb);
  };

  // the scale batch of steps i0 .. i0 + SB - 1 into snext
  auto issue_scales = [&](int i0) __attribute__((always_inline)) {
    const int c = chunk(i0 + q);  // per lane
    uint32_t sb = kOutOfRange;
    if (c >= 0) sb = 2u * (cpg == 1 ? (uint32_t)c : (uint32_t)c / (uint32_t)cpg);
#pragma unroll
    for (int pl = 0; pl < QS; ++pl)
#pragma unroll
      for (int t = 0; t < TPW; ++t)
        snext[pl][t] = __builtin_amdgcn_raw_buffer_load_b16(srsrc[pl], soff[t] + sb, 0, 0);
    if constexpr (ZP) {
#pragma unroll
      for (int t = 0; t < TPW; ++t)
        znext[t] = __builtin_amdgcn_raw_buffer_load_b16(zrsrc, soff[t] + sb, 0, 0);
    }
    if constexpr (TYPED) {
      const uint32_t tb = sb == kOutOfRange ? kOutOfRange : sb >> 1;  // one byte per group
#pragma unroll
      for (int t = 0; t < TPW; ++t)
        tnext[t] = __builtin_amdgcn_raw_buffer_load_b8(trsrc, (soff[t] >> 1) + tb, 0, 0);
    }
  };
  // the scale of this lane's row at step position u (0 .. SB-1) of the batch
  auto step_scale = [&](int t, int u, int pl = 0) __attribute__((always_inline)) {
    const int v = __builtin_amdgcn_ds_bpermute((16 * u + r) * 4, (int)scur[pl][t]);
    return f16_bits_to_f32((uint16_t)v);
  };
  // the LDS lane byte of tile t at step position u: this lane's copy, and
  // with data types the type of its row's group
  auto step_lane_byte = [&](int t, int u) __attribute__((always_inline)) {
    if constexpr (!TYPED) {
      return lane_byte;
    } else {
      const uint32_t v = (uint32_t)__builtin_amdgcn_ds_bpermute((16 * u + r) * 4, (int)tcur[t]);
      return ((v & (kMaxTypes - 1)) << 6) | ((uint32_t)r << 2);
    }
  };
  auto step_zero = [&](int t, int u) __attribute__((always_inline)) {
    const int v = __builtin_amdgcn_ds_bpermute((16 * u + r) * 4, (int)zcur[ZP ? t : 0]);
    return f16_bits_to_f32((uint16_t)v);
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

  // One chunk (128 codes) of every tile.
  auto compute = [&](auto S, auto B) __attribute__((always_inline)) {
    constexpr int s = decltype(S)::value;
    constexpr int u = decltype(B)::value;  // position in the scale batch
    if constexpr (!MFMA) {
      // bf16 activations: this chunk of each batch row (one pair per lane)
      // to fp16 under the chunk's power-of-two shift; fm undoes it
      float fm[BF16 ? MROWS : 1];
      if constexpr (BF16) {
#pragma unroll
        for (int m = 0; m < MROWS; ++m) {
          const int sh = bf16_chunk_shift(wave_max_u32(bf16x2_absmax(xbuf[s][m])));
          xbuf[s][m] = bf16x2_to_f16x2(xbuf[s][m], sh);
          fm[m] = __builtin_ldexpf(1.f, -sh);
        }
      }
      // k-step outer, tile inner: each activation broadcast serves all tiles
      // (binary coding: one partial sum per plane)
      float cs[QS][TPW][MROWS];
#pragma unroll
      for (int pl = 0; pl < QS; ++pl)
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
          for (int m = 0; m < MROWS; ++m) cs[pl][t][m] = 0.f;
      uint32_t lbt[TPW];
#pragma unroll
      for (int t = 0; t < TPW; ++t) lbt[t] = step_lane_byte(t, u);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t idx4[TPW];
#pragma unroll
        for (int t = 0; t < TPW; ++t) idx4[t] = step_indices<BITS>(cbuf[s][t], j);
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          if constexpr (!BCQ) {
            uint32_t pr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) pr[i] = lds_load(table, pair_addr(idx4[t], lbt[t], i));
            // pair i of k-step j meets the activations of lane 4j+i of the row
#pragma unroll
            for (int m = 0; m < MROWS; ++m)
              cs[0][t][m] = dot2_bcast4(cs[0][t][m], xbuf[s][m], pr[0], pr[1], pr[2], pr[3], j);
          } else {
            // one entry per pair holds every plane's (bit, bit) pair
            u32x4 pw[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) pw[i] = lds_load_bcq<BITS>(table, pair_addr(idx4[t], lbt[t], i));
#pragma unroll
            for (int pl = 0; pl < QS; ++pl)
#pragma unroll
              for (int m = 0; m < MROWS; ++m)
                cs[pl][t][m] = dot2_bcast4(cs[pl][t][m], xbuf[s][m], pw[0][pl], pw[1][pl], pw[2][pl],
                                           pw[3][pl], j);
          }
        }
      }
      // Zero points: lane row q multiplied the activations of the 16 lanes of
      // its row (k = 32j + 8q + e), so its share of the group's activation
      // sum is the sum over that row (a butterfly: every lane gets the same
      // value), computed once for all tiles.
      float xq[XSUM ? MROWS : 1];
      if constexpr (XSUM) {
#pragma unroll
        for (int m = 0; m < MROWS; ++m) xq[m] = row_sum16(pair_sum(xbuf[s][m]));
      }
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        if constexpr (BCQ) {
          // sum_k x (2 bit_p - 1) = 2 S_p - X per plane, times its alpha
#pragma unroll
          for (int pl = 0; pl < QS; ++pl) {
            const float a = step_scale(t, u, pl);
#pragma unroll
            for (int m = 0; m < MROWS; ++m)
              gacc[t][m] = __builtin_fmaf(a, __builtin_fmaf(2.f, cs[pl][t][m], -xq[m]), gacc[t][m]);
          }
        } else if constexpr (GROUPED) {
          const float sc = step_scale(t, u);
          if constexpr (ZP) {
            const float z = step_zero(t, u);
#pragma unroll
            for (int m = 0; m < MROWS; ++m)
              gacc[t][m] = __builtin_fmaf(sc, __builtin_fmaf(-z, xq[m], cs[0][t][m]), gacc[t][m]);
          } else {
#pragma unroll
            for (int m = 0; m < MROWS; ++m)
              gacc[t][m] = __builtin_fmaf(BF16 ? sc * fm[BF16 ? m : 0] : sc, cs[0][t][m], gacc[t][m]);
          }
        } else if constexpr (BF16) {
#pragma unroll
          for (int m = 0; m < MROWS; ++m) gacc[t][m] = __builtin_fmaf(fm[m], cs[0][t][m], gacc[t][m]);
        } else {
#pragma unroll
          for (int m = 0; m < MROWS; ++m) gacc[t][m] += cs[0][t][m];
        }
      }
    } else {
      // The decoded pairs of k-step j are the B operand. The lookups of tile
      // t + 1 are issued before the MFMAs of tile t, so the LDS latency hides
      // behind them even with a single wave per SIMD.
      u32x4 bq[2][4];
      auto lookup = [&](int t, u32x4(&dst)[4]) __attribute__((always_inline)) {
        const uint32_t lb = step_lane_byte(t, u);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t idx4 = step_indices<BITS>(cbuf[s][t], j);
          dst[j].x = lds_load(table, pair_addr(idx4, lb, 0));
          dst[j].y = lds_load(table, pair_addr(idx4, lb, 1));
          dst[j].z = lds_load(table, pair_addr(idx4, lb, 2));
          dst[j].w = lds_load(table, pair_addr(idx4, lb, 3));
        }
      };
      if constexpr (XS) {
        // The chunk's MROWS x 128 activations into this wave's LDS area, then
        // back out as fragments (lane r, q of fragment mt, j: row 16 mt + r,
        // piece 4j + q). Row `row` stores piece u at position u ^ (row & 15):
        // the 16 lanes writing a row cover every bank once, and the 16 lanes
        // reading one piece of rows 16 mt + 0..15 hit distinct banks.
        char* xw = reinterpret_cast<char*>(xstage + wave * kXStageWords);
        wave_lds_order();  // the previous chunk's fragment reads come first
#pragma unroll
        for (int i = 0; i < XL; ++i) {
          const int row = 4 * i + (lane >> 4);
          *reinterpret_cast<u32x4*>(xw + row * kXRowBytes + 16 * ((lane & 15) ^ (row & 15))) =
              xl[s][i];
        }
        wave_lds_order();
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            abuf[s][mt][j] = *reinterpret_cast<const u32x4*>(
                xw + (16 * mt + r) * kXRowBytes + 16 * ((4 * j + q) ^ r));
      }
      // bf16 activations: each batch row's chunk (32 values per lane, its
      // four quarters in lanes r, r + 16, r + 32, r + 48) to fp16 under the
      // chunk's shift; fe[mt][e] undoes it for accumulator row 4q + e
      f32x4 fe[BF16 ? MT : 1];
      if constexpr (BF16) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          u16x2 m2 = {0, 0};
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int w = 0; w < 4; ++w) m2 = bf16x2_absmax_acc(m2, abuf[s][mt][j][w]);
          const int sh = bf16_chunk_shift(max_over_quarters(u16x2_max(m2)));
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int w = 0; w < 4; ++w) abuf[s][mt][j][w] = bf16x2_to_f16x2(abuf[s][mt][j][w], sh);
          const float f = __builtin_ldexpf(1.f, -sh);   // of batch row mt 16 + r
#pragma unroll
          for (int e = 0; e < 4; ++e)
            fe[mt][e] = __builtin_bit_cast(
                float, __builtin_amdgcn_ds_bpermute((4 * q + e) * 4, __builtin_bit_cast(int, f)));
        }
      }
      if constexpr (!BCQ) lookup(0, bq[0]);
      // Zero points: the group's activation sums, in the accumulator layout
      // (a B operand of ones gives C[m][n] = sum_k x[m][k] in every column),
      // once for all tiles.
      f32x4 xs[XSUM ? MT : 1];
      if constexpr (XSUM) {
        const f16x8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          xs[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < 4; ++j)
            xs[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                __builtin_bit_cast(f16x8, abuf[s][mt][j]), ones, xs[mt], 0, 0, 0);
        }
      }
      if constexpr (BCQ) {
        // Binary coding: every plane's (bit, bit) pairs of k-step j, decoded
        // in registers (bcq_planes_decode); plane p's four pairs are its B
        // operand.
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          f32x4 cg[QS][MT];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            u32x4 pw[4];
            bcq_planes_decode<BITS>(step_indices<BITS>(cbuf[s][t], j), pw);
#pragma unroll
            for (int pl = 0; pl < QS; ++pl) {
              const f16x8 b = __builtin_bit_cast(f16x8, u32x4{pw[0][pl], pw[1][pl], pw[2][pl], pw[3][pl]});
#pragma unroll
              for (int mt = 0; mt < MT; ++mt)
                cg[pl][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    __builtin_bit_cast(f16x8, abuf[s][mt][j]), b,
                    j == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : cg[pl][mt], 0, 0, 0);
            }
          }
#pragma unroll
          for (int pl = 0; pl < QS; ++pl) {
            const float a = step_scale(t, u, pl);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                macc[t][mt][e] = __builtin_fmaf(a, __builtin_fmaf(2.f, cg[pl][mt][e], -xs[mt][e]),
                                                macc[t][mt][e]);
          }
        }
        return;
      }
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        if (t + 1 < TPW) lookup(t + 1, bq[(t + 1) & 1]);
        // keep the scheduler from sinking those lookups below the MFMAs
        __builtin_amdgcn_sched_barrier(0);
        f32x4 cg[MT];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f16x8 b = __builtin_bit_cast(f16x8, bq[t & 1][j]);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const f16x8 a = __builtin_bit_cast(f16x8, abuf[s][mt][j]);
            if constexpr (GROUPED || BF16) {
              // the chunk's partial sum starts from zero and is rescaled below
              cg[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                  a, b, j == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : cg[mt], 0, 0, 0);
            } else {
              macc[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, macc[t][mt], 0, 0, 0);
            }
          }
        }
        if constexpr (BF16) {
          const float sc = GROUPED ? step_scale(t, u) : 1.f;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              macc[t][mt][e] = __builtin_fmaf(sc * fe[mt][e], cg[mt][e], macc[t][mt][e]);
        } else if constexpr (GROUPED) {
          const float sc = step_scale(t, u);
          if constexpr (ZP) {
            const float z = step_zero(t, u);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                macc[t][mt][e] = __builtin_fmaf(sc, __builtin_fmaf(-z, xs[mt][e], cg[mt][e]),
                                                macc[t][mt][e]);
          } else {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
              for (int e = 0; e < 4; ++e) macc[t][mt][e] = __builtin_fmaf(sc, cg[mt][e], macc[t][mt][e]);
          }
        }
      }
    }
  };

  // Software pipeline: PF register slots; the load of step i + PF - 1 is
  // issued before step i is computed, so PF - 1 chunks are in flight during
  // every compute step, and the scale batch of steps i + SB .. i + 2SB - 1 is
  // issued when step i opens a batch. Within the loop every step issues the
  // same loads (those past the wave's last chunk read nothing); the loop
  // ends with the wave's last chunk.
  // The first chunk's loads go out before the first scale batch: the load
  // counter drains in issue order, so the first step's wait for its codes
  // does not include the scales, which it needs only at its end (measured
  // 7.8 -> 7.6 us on 14336 x 4096 at batch 1, 4.65 -> 4.39 us on 4096 x
  // 4096; issuing the scales after every prologue chunk instead lost 0.3 us
  // on 4096 x 14336).
  issue(std::integral_constant<int, 0>{}, chunk(0));
  if constexpr (GROUPED) issue_scales(0);
  static_for<PF - 2>([&](auto S) {
    constexpr int i = decltype(S)::value + 1;
    issue(std::integral_constant<int, i>{}, chunk(i));
  });

  if constexpr (BCQ) {
    if constexpr (!MFMA) build_bcq_table<BITS, kThreads>(table, tid);
  } else {
    build_pair_table<BITS, kThreads, TYPED>(table, lut_lane, tid);
  }
  __syncthreads();

  // One step at position u of a U-step group starting at i0. Steps past the
  // wave's last chunk (at most PF - 1) issue loads that read nothing and
  // skip the compute; keeping the issue unconditional keeps the in-order
  // load counter the same on every path, so its waits stay exact.
  // (always inlined: an outlined copy would move the register arrays it
  // captures into scratch memory)
  auto step = [&](auto S, int i0) __attribute__((always_inline)) {
    constexpr int u = decltype(S)::value;
    const int i = i0 + u;
    if constexpr (GROUPED && u % SB == 0) {
#pragma unroll
      for (int pl = 0; pl < QS; ++pl)
#pragma unroll
        for (int t = 0; t < TPW; ++t) scur[pl][t] = snext[pl][t];
      if constexpr (ZP) {
#pragma unroll
        for (int t = 0; t < TPW; ++t) zcur[t] = znext[t];
      }
      if constexpr (TYPED) {
#pragma unroll
        for (int t = 0; t < TPW; ++t) tcur[t] = tnext[t];
      }
      issue_scales(i + SB);
    }
    issue(std::integral_constant<int, (u + PF - 1) % PF>{}, chunk(i + PF - 1));
    if (i < nmine)
      compute(std::integral_constant<int, u % PF>{}, std::integral_constant<int, u % SB>{});
  };
  int i0 = 0;
  for (; i0 + U <= nsteps; i0 += U) static_for<U>([&](auto S) { step(S, i0); });
  if constexpr (U > PF) {
    if (i0 < nsteps) static_for<PF>([&](auto S) { step(S, i0); });
  }

  // ---- combine the waves (fixed order) ------------------------------------
  __syncthreads();  // every wave is done with the table and staging areas; reuse them
  float* red = reinterpret_cast<float*>(table);  // [kWaves][MROWS][RP]
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    if constexpr (!MFMA) {
#pragma unroll
      for (int m = 0; m < MROWS; ++m) {
        const float v = sum_over_quarters_r(gacc[t][m]);
        if (q == 0) red[(wave * MROWS + m) * RP + t * kTileRows + r] = v;
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          red[(wave * MROWS + mt * 16 + 4 * q + e) * RP + t * kTileRows + r] = macc[t][mt][e];
    }
  }
  __syncthreads();

  const float tscale = GROUPED ? 1.f : f16_bits_to_f32(p.scales[0]);
  const int items = ROWS * p.M;
  for (int it = tid; it < items; it += kThreads) {
    const int m = it / ROWS, row = it - m * ROWS;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += red[(w * MROWS + m) * RP + row];
    v *= tscale;
    const int n = tile0 * kTileRows + row;
    if (p.ksplit == 1) {
      if (n < p.N) p.y[(size_t)m * p.N + n] = BF16 ? f32_to_bf16_bits(v) : f32_to_f16_bits(v);
    } else {
      float* dst = p.partial + (((size_t)rb * p.ksplit + ks) * MROWS + m) * ROWS + row;
      __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (p.ksplit == 1) return;

  // ---- split-K: the last workgroup of this row block sums the splits ------
  // Ordering without agent-scope fences. An agent-scope release fence on
  // gfx950 writes back the whole L2 of the XCD (buffer_wbl2), which costs
  // ~100 us over a few hundred workgroups, so the hand-off is built from
  // these rules of the AMDGPU memory model for this target instead:
  //  1. every partial is stored with an agent-scope atomic store, which the
  //     hardware writes through to the device-coherent level (not left dirty
  //     in this XCD's L2), and the last workgroup reads them with
  //     agent-scope atomic loads, which read that level (no stale L2 copy);
  //  2. a store's vmcnt slot is released only when the store is
  //     acknowledged, i.e. visible at that level: the wait below (inline
  //     assembly with a memory clobber, so the compiler cannot sink the
  //     stores below it) makes all of this thread's partials visible
  //     before the barrier;
  //  3. the arrival counter is bumped (agent-scope atomic, performed at the
  //     same level) by one thread after the barrier, i.e. after every
  //     thread's wait; the workgroup that sees the last count reads the
  //     partials only after a second barrier, which the compiler does not
  //     move memory operations across.
  // So a partial is visible before its workgroup's arrival is counted, and
  // read only after every arrival was counted.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const uint32_t old =
        __hip_atomic_fetch_add(p.counters + rb, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    arrive_last = (old == (uint32_t)(p.ksplit - 1));
  }
  __syncthreads();
  if (!arrive_last) return;
  for (int it = tid; it < items; it += kThreads) {
    const int m = it / ROWS, row = it - m * ROWS;
    const int n = tile0 * kTileRows + row;
    // The splits' partials in split order, eight loads in flight at a time
    // (a load-then-add loop waits out one device round trip per split).
    // Past the last split the load repeats a valid address and its value is
    // not added, so every load is unconditional and the sum is the plain
    // in-order one.
    const float* part = p.partial + ((size_t)rb * p.ksplit * MROWS + m) * ROWS + row;
    const size_t kstride = (size_t)MROWS * ROWS;
    float v = 0.f;
    for (int k0 = 0; k0 < p.ksplit; k0 += 8) {
      float t[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        t[u] = __hip_atomic_load(part + (size_t)min(k0 + u, p.ksplit - 1) * kstride,
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int u = 0; u < 8; ++u) v = k0 + u < p.ksplit ? v + t[u] : v;
    }
    if (n < p.N) p.y[(size_t)m * p.N + n] = BF16 ? f32_to_bf16_bits(v) : f32_to_f16_bits(v);
  }
  if (tid == 0) __hip_atomic_store(p.counters + rb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Kernel shapes. GEMV: 8 waves, each covering 1 or 2 tiles. MFMA: 8 or 7
// tiles per wave with 4 waves (wide matrices: each activation fragment feeds
// 8 or 7 tiles), 4 tiles with 4 waves (8 at 32 batch rows), 2 tiles with 8
// waves (narrow matrices, which need many workgroups to fill the device), or
// 1 tile with 8 waves (at most one tile per CU on a short K).
constexpr int kPf = 2;

// Host-side shape rules: compiled once (in the width-4 object).
#if LUTQ_MATMUL_BITS == 4
bool tiles_supported(int path, int tiles) {
  if (path == kPathMfma) return tiles == 1 || tiles == 2 || tiles == 4 || tiles == 7 || tiles == 8;
  return tiles == 1 || tiles == 2;
}

// Measured on MI355X over the Llama-3-8B and Llama-70B projection shapes: the
// widest shape that still gives most CUs a workgroup wins, except that 8
// tiles only pay at 32 batch rows. MFMA workgroups are bound by their own
// lookups, so the busiest CU sets the time: 7 tiles when that puts exactly
// one workgroup on every CU (28672 rows: 8 tiles leave 32 of 256 CUs idle,
// 4 tiles put two workgroups on 192 of them; 31.6 -> 27.4 us at 32 batch
// rows, 26.6 -> 21.6 us at 16). At most one tile per CU on a short K (fewer
// than 64 chunks): one tile per workgroup, which spreads the rows over the
// most CUs without the round trips of a K split (4096 x 4096: 6.97 -> 6.38
// us at 16 batch rows; 1024 x 4096: 6.87 -> 5.78 us). A long K keeps two
// tiles and splits K instead (4096 x 14336 at 16 rows: 12.41 us against
// 13.37 with one tile).
int pick_tiles(int path, int mrows, int ntiles, int nchunks, int cus) {
  if (path != kPathMfma) return ntiles >= 2 * cus ? 2 : 1;
  if (ntiles > 6 * cus && ntiles <= 7 * cus) return 7;
  if (mrows > 16 && ntiles >= 6 * cus) return 8;
  if (ntiles >= 2 * cus) return 4;
  if (ntiles <= cus && nchunks < 64) return 1;
  return 2;
}
#endif

template <int BITS, bool MFMA, int MROWS, int TPW, int WAVES, int OCC, bool XS = false>
static hipError_t launch_t(const MatmulParams& p, hipStream_t s) {
  const int nrb = p.nseg > 1 ? p.nrb : (p.ntiles + TPW - 1) / TPW;
  const dim3 grid((unsigned)nrb * (unsigned)p.ksplit);
  // Grouped scales at 32 batch rows x 7 or 8 tiles need more than the 256
  // registers of two waves per SIMD; these shapes run on at most one
  // workgroup per CU, so one wave per SIMD costs nothing.
  constexpr int OCC_G = (MFMA && MROWS == 32 && TPW >= 7) ? 1 : OCC;
  // Chunks in flight per wave: 4 for one-tile GEMV at one batch row (narrow
  // matrices, where each wave has few chunks and little else to overlap the
  // loads with; measured 4.5 -> 4.0 us on a 1024 x 4096 projection, 10.0 ->
  // 8.3 us on 4096 x 14336), else 2 (wider shapes lose occupancy with 4).
  constexpr int PFK = (!MFMA && MROWS == 1 && TPW == 1) ? 4 : kPf;
  const dim3 block(WAVES * kWave);
  // flags: GROUPED, ZP, TYPED, BCQ, BF16
#define LUTQ_LAUNCH(G, Z, T, Q, H, OCCV, XSV)                                              \
  matmul_kernel<BITS, MFMA, MROWS, G, Z, T, Q, H, PFK, TPW, WAVES, OCCV, XSV><<<grid, block, 0, s>>>(p)
  if (p.bcq) {
    // binary-coded weights: staged at 32 batch rows only (at 16, staging the
    // 2-tile shape measured 16.0 -> 17.3 us on 14336 x 4096, q = 3). Four
    // planes at 32 rows x 4 tiles take the 4-wave shape (launch_mfma), so
    // the 8-wave one, which would spill, is not built for them.
    if constexpr (BITS == 4 && MFMA && MROWS == 32 && TPW == 4 && WAVES == 8)
      return hipErrorInvalidValue;
    else
      LUTQ_LAUNCH(true, false, false, true, false, OCC_G, XS && MROWS == 32);
  } else if (p.bf16) {
    // bf16 activations, plain tables
    if (p.group == 0)
      LUTQ_LAUNCH(false, false, false, false, true, OCC, XS);
    else
      LUTQ_LAUNCH(true, false, false, false, true, OCC_G, XS);
  } else if (p.group == 0) {
    LUTQ_LAUNCH(false, false, false, false, false, OCC, XS);
  } else if (p.types && p.zp) {
    LUTQ_LAUNCH(true, true, true, false, false, OCC_G, XS);
  } else if (p.types) {
    LUTQ_LAUNCH(true, false, true, false, false, OCC_G, XS);
  } else if (p.zp) {
    LUTQ_LAUNCH(true, true, false, false, false, OCC_G, XS);
  } else {
    LUTQ_LAUNCH(true, false, false, false, false, OCC_G, XS);
  }
#undef LUTQ_LAUNCH
  return hipGetLastError();
}

// The 8-wave shapes stage their activations (XS) at 32 batch rows, and at 16
// when the slice holds more than 8 rows: the direct loads of missing rows
// cost nothing, so at up to 8 rows the staging round trip does not pay
// (measured: 5.9 -> 6.5 us at 5 rows, 12.8 -> 11.5 us at 12 on narrow
// matrices).
template <int BITS, int MROWS>
static hipError_t launch_mfma(const MatmulParams& p, int tiles, hipStream_t s) {
  switch (tiles) {
    case 8: return launch_t<BITS, true, MROWS, 8, 4, 2>(p, s);
    case 7: return launch_t<BITS, true, MROWS, 7, 4, 2>(p, s);
    case 4:
      if constexpr (MROWS == 32) {
        // four binary planes' operands at 32 rows need more than the 256
        // registers of two waves per SIMD: one wave per SIMD, unstaged
        if (BITS == 4 && p.bcq) return launch_t<BITS, true, MROWS, 4, 4, 1>(p, s);
        return launch_t<BITS, true, MROWS, 4, 8, 2, true>(p, s);
      } else {
        return launch_t<BITS, true, MROWS, 4, 4, 2>(p, s);
      }
    case 1:
      // one tile per workgroup: matrices of at most one tile per CU get a
      // workgroup on every CU without splitting K
      if constexpr (MROWS == 32) {
        return launch_t<BITS, true, MROWS, 1, 8, 2, true>(p, s);
      } else {
        if (p.M > 8) return launch_t<BITS, true, MROWS, 1, 8, 2, true>(p, s);
        return launch_t<BITS, true, MROWS, 1, 8, 2>(p, s);
      }
    default:
      if constexpr (MROWS == 32) {
        return launch_t<BITS, true, MROWS, 2, 8, 2, true>(p, s);
      } else {
        if (p.M > 8) return launch_t<BITS, true, MROWS, 2, 8, 2, true>(p, s);
        return launch_t<BITS, true, MROWS, 2, 8, 2>(p, s);
      }
  }
}

// GEMV with 4 or 8 batch rows needs more registers than the occupancy target
// of the 1-2 row kernels allows.
template <int BITS, int MROWS>
static hipError_t launch_gemv(const MatmulParams& p, int tiles, hipStream_t s) {
  constexpr int OCC = MROWS <= 2 ? 4 : 2;
  switch (tiles) {
    case 1: return launch_t<BITS, false, MROWS, 1, 8, OCC>(p, s);
    default: return launch_t<BITS, false, MROWS, 2, 8, OCC>(p, s);
  }
}

template <int BITS>
hipError_t launch_matmul_bits(const MatmulParams& p, int path, int tiles, hipStream_t s) {
  if (path == kPathMfma) {
    if (p.M <= 16) return launch_mfma<BITS, 16>(p, tiles, s);
    return launch_mfma<BITS, 32>(p, tiles, s);
  }
  if (p.M <= 1) return launch_gemv<BITS, 1>(p, tiles, s);
  if (p.M <= 2) return launch_gemv<BITS, 2>(p, tiles, s);
  if (p.M <= 4) return launch_gemv<BITS, 4>(p, tiles, s);
  return launch_gemv<BITS, 8>(p, tiles, s);
}

// This file is compiled once per code width (the build passes
// -DLUTQ_MATMUL_BITS=2, 3 and 4), so the widths' kernels compile in parallel.
#ifndef LUTQ_MATMUL_BITS
#error "compile with -DLUTQ_MATMUL_BITS=2, 3 or 4"
#endif
template hipError_t launch_matmul_bits<LUTQ_MATMUL_BITS>(const MatmulParams&, int, int, hipStream_t);

}  // namespace lutq
