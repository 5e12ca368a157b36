// Peak microbenchmarks of the machine the product runs on: the floors that
// the matmul kernels are measured against.
//
// Each entry point enqueues one launch of a small kernel; the caller times
// it (the benchmark replays many launches in a HIP graph, exactly as it
// times the matmul). The kernels do nothing useful: every result goes to a
// caller-owned sink so that the compiler keeps the work.
#include "../../include/lutq.h"
#include "../../include/lutq_peaks.h"
#include "lutq_internal.h"

namespace lutq {
namespace {

// Launch floor: a kernel with no work.
__global__ void peak_empty_kernel() {}

// Streaming read: the shape that read fastest on MI355X among those tried
// (full occupancy, one 16-byte nontemporal load per lane and sweep, waves
// sweeping the buffer in address order). With STORE, every wave ends with
// one 16-byte store per lane of its first four lanes, as a kernel that
// writes a small result does.
template <bool STORE>
__global__ __launch_bounds__(256) void peak_stream_kernel(const u32x4* __restrict__ p, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  const size_t nthreads = (size_t)gridDim.x * blockDim.x;
  const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (size_t i = tid; i < n16; i += nthreads) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if constexpr (STORE) {
    if ((threadIdx.x & 63) < 4) sink[(tid >> 6) * 4 + (threadIdx.x & 63)] = acc;
  } else {
    if (acc == 0x9E3779B9u) sink[0] = acc;  // practically never; keeps the loads
  }
}

// fp16 MFMA issue rate: every wave runs `iters` rounds of eight independent
// accumulations (independent, so the matrix pipe is never waiting on a
// result), on operands held in registers.
template <int KIND>
__global__ void peak_mfma_kernel(float* __restrict__ sink, int iters) {
  const int lane = threadIdx.x & 63;
  const f16x8 a = {(f16)(lane & 7), (f16)1, (f16)0.5f, (f16)(-1), (f16)2, (f16)0.25f, (f16)3, (f16)(-0.5f)};
  const f16x8 b = {(f16)0.125f, (f16)(lane >> 3), (f16)(-2), (f16)1, (f16)0.5f, (f16)1, (f16)(-1), (f16)4};
  float s = 0.f;
  if constexpr (KIND == LUTQ_PEAK_MFMA_16X16X32) {
    f32x4 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, (float)i};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[i], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  } else {
    typedef float f32x16 __attribute__((ext_vector_type(16)));
    f32x16 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][e] = (float)(i + e);
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[i], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[i][e];
  }
  if (lane == 0) sink[blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)] = s;
}

// Random 32-bit LDS reads in the access pattern of the duplicated pair
// table: 256 entries of 64 copies (64 KiB), entry (idx, copy) at byte
// (idx << 8) | (copy << 2), lane L always reading its own copy (so the 64
// lanes of an instruction hit 64 distinct banks). Each lane holds 16 random
// entries, one address register each, and reads all 16 every round (LDS has
// no cache, so repeating them costs what new ones would). An empty asm
// statement marks the address registers as changed every round, so the
// compiler reissues each read as its own ds_read_b32 (different base
// registers cannot merge into a two-address read); the values are summed
// three at a time.
__global__ void peak_lds_kernel(uint32_t* __restrict__ sink, int iters) {
  __shared__ uint32_t table[16384];
  for (int i = threadIdx.x; i < 16384; i += blockDim.x) table[i] = (uint32_t)i * 2654435761u;
  __syncthreads();
  const uint32_t lane = threadIdx.x & 63u;
  uint32_t h = (uint32_t)(blockIdx.x * blockDim.x + threadIdx.x) * 0x9E3779B9u + 1u;
  uint32_t addr[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    h ^= h << 13;
    h ^= h >> 17;
    h ^= h << 5;
    addr[k] = ((h & 255u) << 8) | (lane << 2);  // byte address of (entry, own copy)
  }
  uint32_t acc = 0;
  for (int it = 0; it < iters; ++it) {
    uint32_t v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) asm volatile("" : "+v"(addr[k]));  // no instruction
#pragma unroll
    for (int k = 0; k < 16; ++k)
      v[k] = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(table) + addr[k]);
#pragma unroll
    for (int k = 0; k < 16; k += 2) acc = acc + v[k] + v[k + 1];
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;  // practically never; keeps the reads
}

constexpr int kStreamGrid = 2048;  // 8 workgroups of 4 waves per CU on 256 CUs

int check_launch() { return hipGetLastError() == hipSuccess ? LUTQ_OK : LUTQ_EHIP; }

}  // namespace
}  // namespace lutq

extern "C" {

int lutq_peak_empty(void* stream) {
  lutq::peak_empty_kernel<<<1, 64, 0, (hipStream_t)stream>>>();
  return lutq::check_launch();
}

size_t lutq_peak_stream_sink_bytes(void) { return (size_t)lutq::kStreamGrid * 4 * 4 * sizeof(uint32_t); }

int lutq_peak_stream(const void* buf, size_t bytes, int store, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16) return LUTQ_EINVAL;
  if ((uintptr_t)buf % 16 || (uintptr_t)sink % 16) return LUTQ_EALIGN;
  const auto* p = reinterpret_cast<const lutq::u32x4*>(buf);
  if (store)
    lutq::peak_stream_kernel<true><<<lutq::kStreamGrid, 256, 0, (hipStream_t)stream>>>(p, bytes / 16, sink);
  else
    lutq::peak_stream_kernel<false><<<lutq::kStreamGrid, 256, 0, (hipStream_t)stream>>>(p, bytes / 16, sink);
  return lutq::check_launch();
}

int lutq_peak_mfma(int kind, int waves_per_simd, int iters, float* sink, void* stream) {
  if (!sink || iters < 1 || waves_per_simd < 1 || waves_per_simd > 4) return LUTQ_EINVAL;
  if (kind != LUTQ_PEAK_MFMA_16X16X32 && kind != LUTQ_PEAK_MFMA_32X32X16) return LUTQ_EINVAL;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return LUTQ_EHIP;
  const dim3 grid((unsigned)cus), block((unsigned)(4 * waves_per_simd * 64));
  if (kind == LUTQ_PEAK_MFMA_16X16X32)
    lutq::peak_mfma_kernel<LUTQ_PEAK_MFMA_16X16X32><<<grid, block, 0, (hipStream_t)stream>>>(sink, iters);
  else
    lutq::peak_mfma_kernel<LUTQ_PEAK_MFMA_32X32X16><<<grid, block, 0, (hipStream_t)stream>>>(sink, iters);
  return lutq::check_launch();
}

int lutq_peak_lds(int waves_per_cu, int iters, uint32_t* sink, void* stream) {
  if (!sink || iters < 1 || waves_per_cu < 1 || waves_per_cu > 16) return LUTQ_EINVAL;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return LUTQ_EHIP;
  lutq::peak_lds_kernel<<<(unsigned)cus, (unsigned)(waves_per_cu * 64), 0, (hipStream_t)stream>>>(sink, iters);
  return lutq::check_launch();
}

}  // extern "C"
