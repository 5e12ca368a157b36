// Offline restructuring of the code matrix into the wave-block layout, its
// inverse (a test hook), and a small fill kernel.
//
// FLUTE abstract: the quantized weight matrix is restructured offline so that
// unpacking in the matmul needs few bit operations. Here one thread produces
// one lane slot (32 codes of one row, read as four 8-byte pieces), so the
// write of a 64-lane block is one contiguous store of 256*BITS bytes, and the
// matmul reads the same block back with one coalesced load per lane. The byte layout is specified in
// include/lutq.h.
#include "lutq_internal.h"

namespace lutq {

// code (j, e) of a slot -> its value in the row: k = 128*c + 32*j + 8*q + e
template <int BITS>
__global__ __launch_bounds__(256) void repack_kernel(const uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ dst, int N, int K,
                                                     int nchunks, long long nslots) {
  for (long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x; gid < nslots;
       gid += (long long)gridDim.x * blockDim.x) {
  const int L = (int)(gid & 63);
  const long long blk = gid >> 6;
  const int c = (int)(blk % nchunks);
  const long long t = blk / nchunks;
  const long long n = t * kTileRows + (L & 15);
  const int q = L >> 4;
  const uint32_t mask = (1u << BITS) - 1u;

  // the 8 codes of k-step j are adjacent in the row: one 8-byte load each,
  // so a wave's loads for one j cover 32 contiguous bytes of each of its 16 rows
  uint64_t v[4] = {0, 0, 0, 0};
  if (n < N) {
    const uint8_t* src = codes + n * K + (long long)c * kChunk + 8 * q;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = *reinterpret_cast<const uint64_t*>(src + 32 * j);
  }
  uint32_t cd[4][8];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) cd[j][e] = (uint32_t)(v[j] >> (8 * e)) & mask;

  uint32_t out[4] = {0, 0, 0, 0};
  if constexpr (BITS == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        out[j] |= (cd[j][2 * i] | (cd[j][2 * i + 1] << 4)) << (8 * i);
  } else {
    // 2-bit part: dword j/2, byte i, nibble j%2
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t nib = (cd[j][2 * i] & 3u) | ((cd[j][2 * i + 1] & 3u) << 2);
        out[j >> 1] |= nib << (8 * i + 4 * (j & 1));
      }
    if constexpr (BITS == 3) {
      const int hoff[4] = {4, 6, 0, 2};
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t hb = (cd[j][2 * i] >> 2) | ((cd[j][2 * i + 1] >> 2) << 1);
          out[2] |= hb << (8 * i + hoff[j]);
        }
    }
  }
  uint8_t* o = dst + gid * (4 * BITS);
  if constexpr (BITS == 4) {
    *reinterpret_cast<u32x4*>(o) = u32x4{out[0], out[1], out[2], out[3]};
  } else if constexpr (BITS == 3) {
    *reinterpret_cast<u32x2*>(o) = u32x2{out[0], out[1]};  // 12-byte slots: 8-byte aligned
    *reinterpret_cast<uint32_t*>(o + 8) = out[2];
  } else {
    *reinterpret_cast<u32x2*>(o) = u32x2{out[0], out[1]};
  }
  }
}

template <int BITS>
__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t* __restrict__ src,
                                                     uint8_t* __restrict__ codes, int N, int K,
                                                     int nchunks, long long nslots) {
  for (long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x; gid < nslots;
       gid += (long long)gridDim.x * blockDim.x) {
  const int L = (int)(gid & 63);
  const long long blk = gid >> 6;
  const int c = (int)(blk % nchunks);
  const long long t = blk / nchunks;
  const long long n = t * kTileRows + (L & 15);
  const int q = L >> 4;
  if (n >= N) continue;
  const uint32_t* in = reinterpret_cast<const uint32_t*>(src + gid * (4 * BITS));
  uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < BITS; ++i) w[i] = in[i];
  const int hoff[4] = {4, 6, 0, 2};
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = e >> 1, odd = e & 1;
      uint32_t v;
      if constexpr (BITS == 4) {
        v = (w[j] >> (8 * i + 4 * odd)) & 15u;
      } else {
        const uint32_t nib = (w[j >> 1] >> (8 * i + 4 * (j & 1))) & 15u;
        v = odd ? (nib >> 2) : (nib & 3u);
        if constexpr (BITS == 3) {
          const uint32_t hb = (w[2] >> (8 * i + hoff[j])) & 3u;
          v |= ((odd ? (hb >> 1) : hb) & 1u) << 2;
        }
      }
      codes[n * K + (long long)c * kChunk + 32 * j + 8 * q + e] = (uint8_t)v;
    }
  }
}

__global__ void fill_u16_kernel(uint16_t* __restrict__ p, long long n, uint16_t v) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x)
    p[i] = v;
}

hipError_t launch_repack(const uint8_t* codes, uint8_t* dst, int N, int K, int bits,
                         hipStream_t s) {
  const int nchunks = K / kChunk;
  const long long ntiles = (N + kTileRows - 1) / kTileRows;
  const long long nslots = ntiles * nchunks * kWave;
  const unsigned grid = (unsigned)std::min<long long>((nslots + 255) / 256, 1 << 20);
  switch (bits) {
    case 2: repack_kernel<2><<<grid, 256, 0, s>>>(codes, dst, N, K, nchunks, nslots); break;
    case 3: repack_kernel<3><<<grid, 256, 0, s>>>(codes, dst, N, K, nchunks, nslots); break;
    default: repack_kernel<4><<<grid, 256, 0, s>>>(codes, dst, N, K, nchunks, nslots); break;
  }
  return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t* src, uint8_t* codes, int N, int K, int bits,
                         hipStream_t s) {
  const int nchunks = K / kChunk;
  const long long ntiles = (N + kTileRows - 1) / kTileRows;
  const long long nslots = ntiles * nchunks * kWave;
  const unsigned grid = (unsigned)std::min<long long>((nslots + 255) / 256, 1 << 20);
  switch (bits) {
    case 2: unpack_kernel<2><<<grid, 256, 0, s>>>(src, codes, N, K, nchunks, nslots); break;
    case 3: unpack_kernel<3><<<grid, 256, 0, s>>>(src, codes, N, K, nchunks, nslots); break;
    default: unpack_kernel<4><<<grid, 256, 0, s>>>(src, codes, N, K, nchunks, nslots); break;
  }
  return hipGetLastError();
}

hipError_t launch_fill_u16(uint16_t* p, long long n, uint16_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<long long>((n + 255) / 256, 1 << 20);
  fill_u16_kernel<<<grid, 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

}  // namespace lutq
