// Internal interface of the quantizer (round-to-nearest onto a table): the
// device scratch it needs, carved from the library's per-stream buffer, and
// its launcher. Kept apart from the matmul's internal header so that the
// matmul kernel's sources do not change when the quantizer does.
#pragma once

#include "lutq_internal.h"

namespace lutq {

// At most kQuantMaxBlocks workgroups per pass.
constexpr int kQuantMaxBlocks = 2048;
enum QuantRule { kRuleAbsmax = 0, kRuleRange = 1 };  // the LUTQ_RULE_* values
struct QuantScratch {
  double* err_partial;  // [kQuantMaxBlocks]
  double* err_total;    // [1]
  float* extrema;       // [3 * kQuantMaxBlocks]
  uint16_t* tscale;     // [1]
  double* acc_partial;  // table tuning: [kQuantMaxBlocks][2][16]
  int* stop;            // table tuning: the last update would have repeated a value
};
constexpr size_t kQuantScratchBytes = kQuantMaxBlocks * sizeof(double) + 64 +
                                      3 * kQuantMaxBlocks * sizeof(float) + 64 +
                                      kQuantMaxBlocks * 2 * 16 * sizeof(double) + 64;

// codes / scales may be null (not written); error: also fill err_total.
// wdtype: the LUTQ_WEIGHT_* value of the weights at w.
hipError_t launch_quantize(const QuantScratch& sc, const void* w, int wdtype, const uint16_t* lut,
                           int bits, int N, int K, int group, int rule, uint8_t* codes,
                           uint16_t* scales, bool error, hipStream_t s);

// One table-tuning step on the device table `lut` (updated in place):
// codes under the given scales (grouped: `scales`; tensor-wise: the scale
// left in sc.tscale by a launch_quantize of the same weights), the weight
// error into sc.err_total, then (if `update`) the new table or *sc.stop = 1.
hipError_t launch_tune_pass(const QuantScratch& sc, const void* w, int wdtype, const uint16_t* lut,
                            int bits, int N, int K, int group, const uint16_t* scales,
                            bool update, hipStream_t s);

// fp64 -> fp16 bits, round to nearest even (host and device).
__host__ __device__ uint16_t f64_to_f16_rne(double d);

}  // namespace lutq
