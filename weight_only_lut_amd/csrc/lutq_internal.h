// Internal interface between the C-ABI host code and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "lutq_device.h"

namespace lutq {

// One matrix of a fused launch: its own codes, table, scales and output;
// its row blocks are [rb_begin, rb_begin + ceil(ntiles / tiles)) of the grid.
struct MatmulSegment {
  const uint8_t* packed;
  const uint16_t* lut;
  const uint16_t* scales;
  const uint16_t* zeros;  // per-group zero points like the scales, or null (z = 0)
  uint16_t* y;            // fp16 [M, N] (this launch's slice of rows)
  int N, ntiles, rb_begin, pad;
};
constexpr int kMaxSegments = 4;

struct MatmulParams {
  const uint16_t* x;      // fp16 [M, K] (this launch's slice of rows)
  const uint8_t* packed;  // wave-block layout
  const uint16_t* lut;    // fp16 [2^bits]
  const uint16_t* scales; // fp16 [N, K/group] or [1]
  const uint16_t* zeros;  // fp16 [N, K/group] zero points, or null (grouped only)
  uint16_t* y;            // fp16 [M, N] (this launch's slice of rows)
  float* partial;         // split-K partial sums, or null when ksplit == 1
  uint32_t* counters;     // split-K arrival counters (zero between launches)
  int M;                  // rows of x in this launch (<= the kernel's row capacity)
  int N, K, group;        // group == 0: one scale per tensor
  int nchunks, ntiles;
  int ksplit;             // workgroups per row block along K
  int cps;                // chunks per split
  bool zp;                // zero points in this launch (any matrix); grouped only
  bool bcq;               // binary-coded weights: scales = alphas [BITS][N][K/group], no table
  bool bf16;              // x and y are bf16 (plain tables only)
  const uint8_t* types;   // per-group data type ids [N, K/group], or null (one table)
  int ntypes;             // tables at lut ([ntypes][2^bits]) when types is set
  // Fused launch (nseg > 1): matrices sharing x, K, bits and group; the
  // fields packed .. y, N and ntiles above are then taken from seg[].
  int nseg;
  int nrb;                // row blocks of the whole launch (all segments)
  MatmulSegment seg[kMaxSegments];
};

enum Path { kPathGemv = 1, kPathMfma = 2 };

// Split-K arrival counters at the start of a scratch buffer: one 32-bit
// counter per row block of a launch (up to 16384), zero between launches.
constexpr size_t kSplitCounterBytes = 64 * 1024;

// The fixed scratch of lutq_matmul_noalloc (counters, then partial sums), per
// device; static_scratch returns the current device's copy, looked up (and
// its counters cleared on stream s) on the first call for that device.
constexpr size_t kStaticScratchBytes = 8u << 20;
hipError_t static_scratch(void** out, hipStream_t s);

// Rows of x one launch of each path handles.
constexpr int kGemvMaxRows = 8;
constexpr int kMfmaMaxRows = 32;

// Shapes of the matmul workgroup compiled for each path, as the number of
// 16-row output tiles each wave covers (every wave of a workgroup covers the
// same tiles and takes its own K chunks). Wider shapes share each activation
// fragment across more tiles; narrower ones give small matrices more
// workgroups.
bool tiles_supported(int path, int tiles);
// The shape the automatic plan picks for a launch of `mrows` batch rows over
// `ntiles` tiles and `nchunks` K chunks on a device with `cus` compute units.
int pick_tiles(int path, int mrows, int ntiles, int nchunks, int cus);

hipError_t launch_repack(const uint8_t* codes, uint8_t* dst, int N, int K, int bits,
                         hipStream_t s);
hipError_t launch_unpack(const uint8_t* src, uint8_t* codes, int N, int K, int bits,
                         hipStream_t s);
hipError_t launch_fill_u16(uint16_t* p, long long n, uint16_t v, hipStream_t s);

// One launch over rows [0, p.M) of x; p.M <= kGemvMaxRows (GEMV) or
// kMfmaMaxRows (MFMA); `tiles` passes tiles_supported(path, tiles).
// launch_matmul_bits<B> is defined in lutq_matmul.hip, which is compiled
// once per code width B.
template <int BITS>
hipError_t launch_matmul_bits(const MatmulParams& p, int path, int tiles, hipStream_t s);
extern template hipError_t launch_matmul_bits<2>(const MatmulParams&, int, int, hipStream_t);
extern template hipError_t launch_matmul_bits<3>(const MatmulParams&, int, int, hipStream_t);
extern template hipError_t launch_matmul_bits<4>(const MatmulParams&, int, int, hipStream_t);
inline hipError_t launch_matmul(const MatmulParams& p, int bits, int path, int tiles,
                                hipStream_t s) {
  switch (bits) {
    case 2: return launch_matmul_bits<2>(p, path, tiles, s);
    case 3: return launch_matmul_bits<3>(p, path, tiles, s);
    default: return launch_matmul_bits<4>(p, path, tiles, s);
  }
}

}  // namespace lutq
