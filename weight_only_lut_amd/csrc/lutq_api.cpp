// C-ABI host side of lutq: argument validation, planning, split-K scratch and
// kernel launches. Every public function validates before touching the GPU,
// so argument errors are reported without any HIP call.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/lutq.h"
#include "lutq_quant.h"

namespace {

thread_local int g_last_hip = 0;

int hip_fail(hipError_t e) {
  g_last_hip = (int)e;
  return LUTQ_EHIP;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_bits_group(int K, int bits, int group) {
  if (bits < 2 || bits > 4) return LUTQ_EBITS;
  if (group < 0) return LUTQ_EGROUP;
  if (K % lutq::kChunk) return LUTQ_EGROUP;
  if (group != 0 && (group % lutq::kChunk || K % group)) return LUTQ_EGROUP;
  return LUTQ_OK;
}

int check_sizes(int N, int K) {
  if (N < 0 || K < 0) return LUTQ_EINVAL;
  if (N > LUTQ_MAX_N || K > LUTQ_MAX_K) return LUTQ_EUNSUPPORTED;
  if ((long long)N * K > LUTQ_MAX_NK) return LUTQ_EUNSUPPORTED;
  return LUTQ_OK;
}

int check_desc(const lutq_packed_t* p) {
  if (!p) return LUTQ_EINVAL;
  if (p->magic != LUTQ_MAGIC || p->version != LUTQ_LAYOUT_VERSION) return LUTQ_EMISMATCH;
  int rc = check_sizes(p->N, p->K);
  if (rc) return rc;
  rc = check_bits_group(p->K, p->bits, p->group);
  if (rc) return rc;
  if (p->nbytes != lutq_packed_bytes(p->N, p->K, p->bits, p->group)) return LUTQ_EMISMATCH;
  if (p->nbytes && !p->data) return LUTQ_EINVAL;
  if (!aligned(p->data, 16)) return LUTQ_EALIGN;
  return LUTQ_OK;
}

// Split-K scratch: one buffer per (device, stream), allocated on first need
// and grown when a call needs more. An outgrown buffer is retired, not freed:
// work still queued on the stream, or a HIP graph captured earlier, may hold
// its address, so retired buffers are freed only by lutq_shutdown. Nothing is
// allocated while the stream is being captured (LUTQ_ECAPTURE): a call that
// needs new scratch must run once eagerly on that stream first. The counters
// are zeroed at allocation by the library's fill kernel on the caller's
// stream (ordered before the launches that use them), and every launch
// leaves them at zero.
struct Scratch {
  void* base = nullptr;
  size_t bytes = 0;
};
std::mutex g_mu;
std::map<std::pair<int, void*>, Scratch> g_scratch;
std::vector<std::pair<int, void*>> g_retired;  // (device, base), freed by lutq_shutdown
constexpr size_t kCounterBytes = lutq::kSplitCounterBytes;
constexpr size_t kMinScratchBytes = 8u << 20;

int get_scratch(void* stream, size_t partial_bytes, float** partial, uint32_t** counters) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  std::lock_guard<std::mutex> lk(g_mu);
  Scratch& s = g_scratch[{dev, stream}];
  const size_t need = kCounterBytes + partial_bytes;
  if (s.bytes < need) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing((hipStream_t)stream, &st);
    if (e != hipSuccess) return hip_fail(e);
    if (st != hipStreamCaptureStatusNone) return LUTQ_ECAPTURE;
    size_t bytes = need > 2 * s.bytes ? need : 2 * s.bytes;
    if (bytes < kMinScratchBytes) bytes = kMinScratchBytes;
    void* base = nullptr;
    e = hipMalloc(&base, bytes);
    if (e != hipSuccess) return hip_fail(e);
    e = lutq::launch_fill_u16(reinterpret_cast<uint16_t*>(base), (long long)(kCounterBytes / 2), 0,
                              (hipStream_t)stream);
    if (e != hipSuccess) {
      (void)hipFree(base);  // nothing was enqueued
      return hip_fail(e);
    }
    if (s.base) g_retired.emplace_back(dev, s.base);
    s.base = base;
    s.bytes = bytes;
  }
  *counters = reinterpret_cast<uint32_t*>(s.base);
  *partial = reinterpret_cast<float*>(reinterpret_cast<char*>(s.base) + kCounterBytes);
  return LUTQ_OK;
}

// Compute units of the current device, cached per device ordinal.
int cu_count() {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    v = 256;
  cache[dev] = v;
  return v;
}

int rows_per_launch(int path) {
  return path == LUTQ_PATH_MFMA ? lutq::kMfmaMaxRows : lutq::kGemvMaxRows;
}

int kernel_path(int path) { return path == LUTQ_PATH_MFMA ? lutq::kPathMfma : lutq::kPathGemv; }

// K lengths (in 128-code chunks) for the split-K plan.
constexpr int kSplitMinChunks = 64;  // K >= 8192
constexpr int kSplitChunks = 32;     // chunks per split, at least

// Checks the caller's options (NULL = all automatic) and copies them to *o.
int read_options(const lutq_options_t* opts, lutq_options_t* o) {
  std::memset(o, 0, sizeof *o);
  if (!opts) return LUTQ_OK;
  for (int i = 0; i < 4; ++i)
    if (opts->reserved[i]) return LUTQ_EINVAL;
  if (opts->dtype != LUTQ_DTYPE_F16 && opts->dtype != LUTQ_DTYPE_BF16) return LUTQ_EINVAL;
  if (opts->path < LUTQ_PATH_AUTO || opts->path > LUTQ_PATH_MFMA || opts->ksplit < 0 ||
      opts->tiles < 0)
    return LUTQ_EINVAL;
  if (opts->tiles &&
      (opts->path == LUTQ_PATH_AUTO || !lutq::tiles_supported(kernel_path(opts->path), opts->tiles)))
    return LUTQ_EINVAL;
  *o = *opts;
  return LUTQ_OK;
}

// Fills the automatic fields of *o (checked by read_options) for an
// M x N x K product (M, N, K > 0).
void plan(int M, int N, int K, int cus, lutq_options_t* o) {
  const int nchunks = K / lutq::kChunk;
  const int ntiles = (N + lutq::kTileRows - 1) / lutq::kTileRows;
  if (o->path == LUTQ_PATH_AUTO) {
    // Batch rows up to which GEMV beats MFMA (measured on MI355X over the
    // Llama projection shapes): on wide matrices MFMA wins from 2 rows; on
    // narrow ones, which run GEMV at one tile per wave, GEMV keeps up to 4
    // rows, or 2 when K is long enough for the MFMA path to split it.
    const int gemv_max = ntiles >= 2 * cus ? 1 : (nchunks >= kSplitMinChunks ? 2 : 4);
    o->path = M <= gemv_max ? LUTQ_PATH_GEMV : LUTQ_PATH_MFMA;
  }
  const int kpath = kernel_path(o->path);
  if (o->tiles == 0) {
    const int rl = rows_per_launch(o->path);
    o->tiles = lutq::pick_tiles(kpath, M < rl ? M : rl, ntiles, nchunks, cus);
  }
  const int nrb = (ntiles + o->tiles - 1) / o->tiles;
  if (o->ksplit == 0) {
    // A split along K puts two memory round trips (the partial stores, then
    // the last workgroup's reads) on the critical path: a few microseconds.
    // MFMA workgroups at more than 8 batch rows (or on a long K) carry
    // enough compute that splitting pays as soon as the row blocks cover at
    // most half the CUs. One-tile MFMA workgroups (a short K) are lighter:
    // split only above 16 batch rows on at most a quarter of the CUs, until
    // half of them are covered (1024 x 4096 at 32 rows: 7.78 us unsplit,
    // 7.22 in 2, 7.41 in 4). GEMV workgroups are light: split only a long K
    // (each split keeping at least kSplitChunks chunks) on fewer row blocks
    // than CUs.
    int k = 1;
    if (o->path == LUTQ_PATH_MFMA && o->tiles == 1) {
      if (M > 16 && 4 * nrb <= cus) k = cus / (2 * nrb);
    } else if (o->path == LUTQ_PATH_MFMA) {
      if (2 * nrb <= cus && (M > 8 || nchunks >= kSplitMinChunks)) k = cus / nrb;
    } else if (nrb < cus && nchunks >= kSplitMinChunks) {
      k = cus / nrb;
      if (k > nchunks / kSplitChunks) k = nchunks / kSplitChunks;
      if (k < 1) k = 1;
    }
    o->ksplit = k;
  }
  if (o->ksplit > nchunks) o->ksplit = nchunks > 0 ? nchunks : 1;
}

// The product for `count` matrices sharing x and K (descriptors already
// checked, each matching K; bits and group equal across them). One launch
// per batch slice covers every matrix with N > 0.
int run_matmul(const uint16_t* x, const lutq_matmul_item_t* items, int count, int M, int K,
               const lutq_options_t* opts, void* stream, const uint8_t* types = nullptr,
               int ntypes = 0, bool bcq = false, bool noalloc = false) {
  lutq_options_t o;
  int rc = read_options(opts, &o);
  if (rc) return rc;
  const bool bf16 = o.dtype == LUTQ_DTYPE_BF16;
  if (bf16 && (bcq || types)) return LUTQ_EUNSUPPORTED;
  int live[LUTQ_MAX_FUSED];
  int nlive = 0, ntiles_all = 0;
  for (int i = 0; i < count; ++i) {
    const int N = items[i].packed->N;
    if (N == 0) continue;
    live[nlive++] = i;
    ntiles_all += (N + lutq::kTileRows - 1) / lutq::kTileRows;
  }
  if (M == 0 || nlive == 0) return LUTQ_OK;
  bool zp = false;
  for (int j = 0; j < nlive; ++j) {
    const lutq_matmul_item_t& it = items[live[j]];
    if (!it.y) return LUTQ_EINVAL;
    if (!aligned(it.y, 2)) return LUTQ_EALIGN;
    if (it.zeros) {
      if (bf16) return LUTQ_EUNSUPPORTED;
      if (it.packed->group == 0) return LUTQ_EGROUP;  // zero points are per group
      if (!aligned(it.zeros, 2)) return LUTQ_EALIGN;
      zp = true;
    }
    if (K == 0) continue;
    if ((!bcq && !it.lut) || !it.scales) return LUTQ_EINVAL;
    if ((!bcq && !aligned(it.lut, 4)) || !aligned(it.scales, 2)) return LUTQ_EALIGN;
  }
  hipStream_t s = (hipStream_t)stream;
  if (K == 0) {  // the empty sum; x, the tables and the scales are not read
    for (int j = 0; j < nlive; ++j) {
      const lutq_matmul_item_t& it = items[live[j]];
      hipError_t e = lutq::launch_fill_u16(it.y, (long long)M * it.packed->N, 0, s);
      if (e != hipSuccess) return hip_fail(e);
    }
    return LUTQ_OK;
  }
  if (!x) return LUTQ_EINVAL;
  if (!aligned(x, 16)) return LUTQ_EALIGN;

  plan(M, ntiles_all * lutq::kTileRows, K, cu_count(), &o);
  const int path = kernel_path(o.path);
  const int ksplit = o.ksplit;
  const int rl = rows_per_launch(o.path);

  lutq::MatmulParams p;
  std::memset(&p, 0, sizeof p);
  const lutq_packed_t* d0 = items[live[0]].packed;
  p.K = K;
  p.group = d0->group;
  p.nchunks = K / lutq::kChunk;
  p.ksplit = ksplit;
  p.cps = (p.nchunks + ksplit - 1) / ksplit;
  int nrb = 0;
  for (int j = 0; j < nlive; ++j) {
    const lutq_matmul_item_t& it = items[live[j]];
    lutq::MatmulSegment& g = p.seg[j];
    g.packed = (const uint8_t*)it.packed->data;
    g.lut = it.lut;
    g.scales = it.scales;
    g.zeros = it.zeros;
    g.y = it.y;
    g.N = it.packed->N;
    g.ntiles = (g.N + lutq::kTileRows - 1) / lutq::kTileRows;
    g.rb_begin = nrb;
    nrb += (g.ntiles + o.tiles - 1) / o.tiles;
  }
  // the first matrix also in the plain fields (the single-matrix launch)
  p.packed = p.seg[0].packed;
  p.lut = p.seg[0].lut;
  p.scales = p.seg[0].scales;
  p.zeros = p.seg[0].zeros;
  p.zp = zp;
  p.types = types;
  p.ntypes = ntypes;
  p.bcq = bcq;
  p.bf16 = bf16;
  p.N = p.seg[0].N;
  p.ntiles = p.seg[0].ntiles;
  p.nseg = nlive;
  p.nrb = nrb;
  if (ksplit > 1) {
    if ((size_t)nrb * sizeof(uint32_t) > kCounterBytes) return LUTQ_EUNSUPPORTED;
    const size_t rows = (size_t)o.tiles * lutq::kTileRows;
    const size_t pbytes = (size_t)nrb * (size_t)ksplit * rl * rows * sizeof(float);
    if (noalloc) {
      // the fixed array of lutq_static.hip: counters, then partial sums
      if (pbytes > lutq::kStaticScratchBytes - kCounterBytes) return LUTQ_EUNSUPPORTED;
      void* base = nullptr;
      hipError_t e = lutq::static_scratch(&base, (hipStream_t)stream);
      if (e != hipSuccess) return hip_fail(e);
      p.counters = reinterpret_cast<uint32_t*>(base);
      p.partial = reinterpret_cast<float*>(reinterpret_cast<char*>(base) + kCounterBytes);
    } else {
      rc = get_scratch(stream, pbytes, &p.partial, &p.counters);
      if (rc) return rc;
    }
  }
  const int bits = d0->bits;
  for (int m0 = 0; m0 < M; m0 += rl) {
    p.M = (M - m0) < rl ? (M - m0) : rl;
    p.x = x + (size_t)m0 * K;
    for (int j = 0; j < nlive; ++j) p.seg[j].y = items[live[j]].y + (size_t)m0 * p.seg[j].N;
    p.y = p.seg[0].y;
    hipError_t e = lutq::launch_matmul(p, bits, path, o.tiles, s);
    if (e != hipSuccess) return hip_fail(e);
  }
  return LUTQ_OK;
}

}  // namespace

extern "C" {

size_t lutq_packed_bytes(int N, int K, int bits, int group) {
  if (check_sizes(N, K) || check_bits_group(K, bits, group)) return 0;
  if (N == 0 || K == 0) return 0;
  const size_t ntiles = (size_t)(N + lutq::kTileRows - 1) / lutq::kTileRows;
  return ntiles * lutq::kTileRows * (size_t)K * (size_t)bits / 8;
}

int lutq_repack(const uint8_t* codes, int N, int K, int bits, int group, void* dst,
                size_t dst_bytes, lutq_packed_t* out, void* stream) {
  if (!out) return LUTQ_EINVAL;
  int rc = check_sizes(N, K);
  if (rc) return rc;
  rc = check_bits_group(K, bits, group);
  if (rc) return rc;
  const size_t need = lutq_packed_bytes(N, K, bits, group);
  if (need) {
    if (!codes || !dst) return LUTQ_EINVAL;
    if (!aligned(dst, 16) || !aligned(codes, 8)) return LUTQ_EALIGN;
    if (dst_bytes < need) return LUTQ_ESIZE;
    const char* a = (const char*)codes;
    const char* b = (const char*)dst;
    if (a < b + need && b < a + (size_t)N * K) return LUTQ_EINVAL;  // overlap
    hipError_t e = lutq::launch_repack(codes, (uint8_t*)dst, N, K, bits, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  lutq_packed_t d;
  std::memset(&d, 0, sizeof d);
  d.magic = LUTQ_MAGIC;
  d.version = LUTQ_LAYOUT_VERSION;
  d.N = N;
  d.K = K;
  d.bits = bits;
  d.group = group;
  d.nbytes = need;
  d.data = need ? dst : nullptr;
  *out = d;
  return LUTQ_OK;
}

int lutq_unpack(const lutq_packed_t* packed, uint8_t* codes_out, void* stream) {
  int rc = check_desc(packed);
  if (rc) return rc;
  if (packed->nbytes == 0) return LUTQ_OK;
  if (!codes_out) return LUTQ_EINVAL;
  hipError_t e = lutq::launch_unpack((const uint8_t*)packed->data, codes_out, packed->N, packed->K,
                                     packed->bits, (hipStream_t)stream);
  return e == hipSuccess ? LUTQ_OK : hip_fail(e);
}

int lutq_plan(int M, int N, int K, int bits, const lutq_options_t* req, lutq_options_t* out) {
  if (!out || M < 0) return LUTQ_EINVAL;
  int rc = check_sizes(N, K);
  if (rc) return rc;
  if (bits < 2 || bits > 4) return LUTQ_EBITS;
  if (K % lutq::kChunk) return LUTQ_EGROUP;
  lutq_options_t o;
  rc = read_options(req, &o);
  if (rc) return rc;
  plan(M > 0 ? M : 1, N > 0 ? N : 1, K > 0 ? K : lutq::kChunk, cu_count(), &o);
  *out = o;
  return LUTQ_OK;
}

int lutq_matmul_ex(const uint16_t* x, const lutq_packed_t* packed, const uint16_t* lut,
                   const uint16_t* scales, uint16_t* y, int M, int N, int K,
                   const lutq_options_t* opts, void* stream) {
  int rc = check_desc(packed);
  if (rc) return rc;
  if (M < 0 || N < 0 || K < 0) return LUTQ_EINVAL;
  if (N != packed->N || K != packed->K) return LUTQ_EMISMATCH;
  const lutq_matmul_item_t item = {packed, lut, scales, nullptr, y};
  return run_matmul(x, &item, 1, M, K, opts, stream);
}

int lutq_matmul_noalloc(const uint16_t* x, const lutq_packed_t* packed, const uint16_t* lut,
                        const uint16_t* scales, uint16_t* y, int M, int N, int K,
                        const lutq_options_t* opts, void* stream) {
  int rc = check_desc(packed);
  if (rc) return rc;
  if (M < 0 || N < 0 || K < 0) return LUTQ_EINVAL;
  if (N != packed->N || K != packed->K) return LUTQ_EMISMATCH;
  const lutq_matmul_item_t item = {packed, lut, scales, nullptr, y};
  return run_matmul(x, &item, 1, M, K, opts, stream, nullptr, 0, false, true);
}

int lutq_matmul_typed(const uint16_t* x, const lutq_packed_t* packed, const uint16_t* luts,
                      int ntypes, const uint8_t* types, const uint16_t* scales,
                      const uint16_t* zeros, uint16_t* y, int M, int N, int K,
                      const lutq_options_t* opts, void* stream) {
  int rc = check_desc(packed);
  if (rc) return rc;
  if (M < 0 || N < 0 || K < 0) return LUTQ_EINVAL;
  if (N != packed->N || K != packed->K) return LUTQ_EMISMATCH;
  if (packed->group == 0) return LUTQ_EGROUP;  // a data type per group
  if (ntypes < 1 || ntypes > LUTQ_MAX_TYPES) return LUTQ_EINVAL;
  if ((size_t)N * K > 0 && !types) return LUTQ_EINVAL;
  const lutq_matmul_item_t item = {packed, luts, scales, zeros, y};
  return run_matmul(x, &item, 1, M, K, opts, stream, types, ntypes);
}

int lutq_matmul_bcq(const uint16_t* x, const lutq_packed_t* packed, const uint16_t* alphas,
                    uint16_t* y, int M, int N, int K, const lutq_options_t* opts, void* stream) {
  int rc = check_desc(packed);
  if (rc) return rc;
  if (M < 0 || N < 0 || K < 0) return LUTQ_EINVAL;
  if (N != packed->N || K != packed->K) return LUTQ_EMISMATCH;
  if (packed->group == 0) return LUTQ_EGROUP;  // an alpha per plane, row and group
  const lutq_matmul_item_t item = {packed, nullptr, alphas, nullptr, y};
  return run_matmul(x, &item, 1, M, K, opts, stream, nullptr, 0, true);
}

int lutq_matmul_zp(const uint16_t* x, const lutq_packed_t* packed, const uint16_t* lut,
                   const uint16_t* scales, const uint16_t* zeros, uint16_t* y, int M, int N, int K,
                   const lutq_options_t* opts, void* stream) {
  int rc = check_desc(packed);
  if (rc) return rc;
  if (M < 0 || N < 0 || K < 0) return LUTQ_EINVAL;
  if (N != packed->N || K != packed->K) return LUTQ_EMISMATCH;
  if (packed->group == 0) return LUTQ_EGROUP;
  if (!zeros && (size_t)N * K > 0) return LUTQ_EINVAL;
  const lutq_matmul_item_t item = {packed, lut, scales, zeros, y};
  return run_matmul(x, &item, 1, M, K, opts, stream);
}

int lutq_matmul_multi(const uint16_t* x, const lutq_matmul_item_t* items, int count, int M, int K,
                      const lutq_options_t* opts, void* stream) {
  if (!items || count < 1 || count > LUTQ_MAX_FUSED) return LUTQ_EINVAL;
  if (M < 0 || K < 0) return LUTQ_EINVAL;
  for (int i = 0; i < count; ++i) {
    const int rc = check_desc(items[i].packed);
    if (rc) return rc;
    const lutq_packed_t* d = items[i].packed;
    const lutq_packed_t* d0 = items[0].packed;
    if (d->K != K || d->bits != d0->bits || d->group != d0->group) return LUTQ_EMISMATCH;
  }
  return run_matmul(x, items, count, M, K, opts, stream);
}

int lutq_matmul(const uint16_t* x, const lutq_packed_t* packed, const uint16_t* lut,
                const uint16_t* scales, uint16_t* y, int M, int N, int K, void* stream) {
  return lutq_matmul_ex(x, packed, lut, scales, y, M, N, K, nullptr, stream);
}

}  // extern "C"

namespace {

static_assert(LUTQ_MAX_FUSED == lutq::kMaxSegments, "one kernel segment per fused matrix");
static_assert(LUTQ_NOALLOC_SCRATCH_BYTES == lutq::kStaticScratchBytes, "the fixed scratch array");
static_assert(LUTQ_MAX_TYPES == lutq::kMaxTypes, "tables the pair table holds");
static_assert(LUTQ_RULE_ABSMAX == lutq::kRuleAbsmax && LUTQ_RULE_RANGE == lutq::kRuleRange,
              "rule values");

// Arguments shared by the quantizer entry points; N, K > 0 after this.
int check_quant(const void* w, int wdtype, const uint16_t* lut, int bits, int N, int K, int group,
                int rule) {
  int rc = check_sizes(N, K);
  if (rc) return rc;
  rc = check_bits_group(K, bits, group);
  if (rc) return rc;
  if (rule != LUTQ_RULE_ABSMAX && rule != LUTQ_RULE_RANGE) return LUTQ_EINVAL;
  if (wdtype != LUTQ_WEIGHT_F32 && wdtype != LUTQ_WEIGHT_F16 && wdtype != LUTQ_WEIGHT_BF16)
    return LUTQ_EINVAL;
  if (N == 0 || K == 0) return LUTQ_OK;
  if (!w || !lut) return LUTQ_EINVAL;
  // four weights per load: 16 bytes of fp32, 8 of fp16 / bf16
  if (!aligned(w, wdtype == LUTQ_WEIGHT_F32 ? 16 : 8) || !aligned(lut, 2)) return LUTQ_EALIGN;
  return LUTQ_OK;
}

// The quantizer's scratch, carved out of the per-stream buffer; `extra` bytes
// after it (16-byte aligned) for the caller.
int quant_scratch(void* stream, size_t extra, lutq::QuantScratch* sc, void** extra_out) {
  float* base = nullptr;
  uint32_t* counters = nullptr;
  int rc = get_scratch(stream, lutq::kQuantScratchBytes + 64 + extra, &base, &counters);
  if (rc) return rc;
  char* b = reinterpret_cast<char*>(base);
  sc->err_partial = reinterpret_cast<double*>(b);
  b += lutq::kQuantMaxBlocks * sizeof(double);
  sc->err_total = reinterpret_cast<double*>(b);
  b += 64;
  sc->extrema = reinterpret_cast<float*>(b);
  b += 3 * lutq::kQuantMaxBlocks * sizeof(float);
  sc->tscale = reinterpret_cast<uint16_t*>(b);
  b += 64;
  sc->acc_partial = reinterpret_cast<double*>(b);
  b += lutq::kQuantMaxBlocks * 2 * 16 * sizeof(double);
  sc->stop = reinterpret_cast<int*>(b);
  b += 64;
  if (extra_out) *extra_out = b;
  return LUTQ_OK;
}

// Runs the error pass and copies the total to the host (waits for the stream).
int quant_error_to_host(const lutq::QuantScratch& sc, const void* w, int wdtype,
                        const uint16_t* lut, int bits, int N, int K, int group, int rule,
                        double* err, hipStream_t s) {
  hipError_t e = lutq::launch_quantize(sc, w, wdtype, lut, bits, N, K, group, rule, nullptr,
                                       nullptr, true, s);
  if (e != hipSuccess) return hip_fail(e);
  e = hipMemcpyAsync(err, sc.err_total, sizeof(double), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail(e);
  e = hipStreamSynchronize(s);
  return e == hipSuccess ? LUTQ_OK : hip_fail(e);
}

static_assert(LUTQ_WEIGHT_F32 == 0 && LUTQ_WEIGHT_F16 == 1 && LUTQ_WEIGHT_BF16 == 2,
              "the quantizer kernels' weight type values");

}  // namespace

extern "C" {

int lutq_quantize_ex(const void* w, int wdtype, const uint16_t* lut, int bits, int N, int K,
                     int group, int rule, uint8_t* codes, uint16_t* scales, void* stream) {
  int rc = check_quant(w, wdtype, lut, bits, N, K, group, rule);
  if (rc) return rc;
  if (N == 0 || K == 0) return LUTQ_OK;
  if (!codes || !scales) return LUTQ_EINVAL;
  if (!aligned(codes, 4) || !aligned(scales, 2)) return LUTQ_EALIGN;
  lutq::QuantScratch sc;
  std::memset(&sc, 0, sizeof sc);
  if (group == 0) {  // tensor-wise: the extrema and the scale pass through scratch
    rc = quant_scratch(stream, 0, &sc, nullptr);
    if (rc) return rc;
  }
  hipError_t e = lutq::launch_quantize(sc, w, wdtype, lut, bits, N, K, group, rule, codes, scales,
                                       false, (hipStream_t)stream);
  return e == hipSuccess ? LUTQ_OK : hip_fail(e);
}

int lutq_quantize(const float* w, const uint16_t* lut, int bits, int N, int K, int group,
                  int rule, uint8_t* codes, uint16_t* scales, void* stream) {
  return lutq_quantize_ex(w, LUTQ_WEIGHT_F32, lut, bits, N, K, group, rule, codes, scales, stream);
}

int lutq_quant_error_ex(const void* w, int wdtype, const uint16_t* lut, int bits, int N, int K,
                        int group, int rule, double* err, void* stream) {
  if (!err) return LUTQ_EINVAL;
  int rc = check_quant(w, wdtype, lut, bits, N, K, group, rule);
  if (rc) return rc;
  if (N == 0 || K == 0) {
    *err = 0.0;
    return LUTQ_OK;
  }
  lutq::QuantScratch sc;
  rc = quant_scratch(stream, 0, &sc, nullptr);
  if (rc) return rc;
  return quant_error_to_host(sc, w, wdtype, lut, bits, N, K, group, rule, err,
                             (hipStream_t)stream);
}

int lutq_quant_error(const float* w, const uint16_t* lut, int bits, int N, int K, int group,
                     int rule, double* err, void* stream) {
  return lutq_quant_error_ex(w, LUTQ_WEIGHT_F32, lut, bits, N, K, group, rule, err, stream);
}

int lutq_log_base_search_ex(const void* w, int wdtype, int bits, int N, int K, int group,
                            const double* bases, int nbases, int* best, double* errors,
                            void* stream) {
  if (!best || !bases || nbases < 1) return LUTQ_EINVAL;
  uint16_t dummy = 0;
  int rc = check_quant(w, wdtype, &dummy, bits, N, K, group, LUTQ_RULE_ABSMAX);
  if (rc) return rc;
  const int L = 1 << bits, half = L / 2;
  for (int i = 0; i < nbases; ++i) {
    if (!(bases[i] > 1.0) || !std::isfinite(bases[i])) return LUTQ_EINVAL;
    // the table must not repeat an fp16 value (it does once base^-k underflows)
    uint16_t prev = lutq::f64_to_f16_rne(1.0);
    for (int k = 1; k < half; ++k) {
      const uint16_t h = lutq::f64_to_f16_rne(std::pow(bases[i], -(double)k));
      if (h == prev) return LUTQ_EINVAL;
      prev = h;
    }
  }
  if (N == 0 || K == 0) {
    *best = 0;
    if (errors)
      for (int i = 0; i < nbases; ++i) errors[i] = 0.0;
    return LUTQ_OK;
  }
  lutq::QuantScratch sc;
  void* tbl = nullptr;
  rc = quant_scratch(stream, 64, &sc, &tbl);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  double best_err = 0.0;
  for (int i = 0; i < nbases; ++i) {
    // code = sign bit on top of the exponent bits: (-1)^sign * base^-k
    uint16_t host_tbl[16];
    for (int c = 0; c < L; ++c) {
      const int k = c % half;
      const double v = std::pow(bases[i], -(double)k);
      host_tbl[c] = lutq::f64_to_f16_rne(c >= half ? -v : v);
    }
    hipError_t e = hipMemcpyAsync(tbl, host_tbl, L * sizeof(uint16_t), hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e);
    double err = 0.0;
    rc = quant_error_to_host(sc, w, wdtype, (const uint16_t*)tbl, bits, N, K, group,
                             LUTQ_RULE_ABSMAX, &err, s);
    if (rc) return rc;
    if (errors) errors[i] = err;
    if (i == 0 || err < best_err) {
      best_err = err;
      *best = i;
    }
  }
  return LUTQ_OK;
}

int lutq_tune_table(const void* w, int wdtype, uint16_t* lut, int bits, int N, int K, int group,
                    int rule, int iters, uint16_t* scales, double* errors, int* updates,
                    void* stream) {
  if (!updates || iters < 0) return LUTQ_EINVAL;
  int rc = check_quant(w, wdtype, lut, bits, N, K, group, rule);
  if (rc) return rc;
  *updates = 0;
  if (N == 0 || K == 0) {
    if (errors)
      for (int i = 0; i <= iters; ++i) errors[i] = 0.0;
    return LUTQ_OK;
  }
  if (scales && !aligned(scales, 2)) return LUTQ_EALIGN;
  // the fixed scales: the caller's buffer, or scratch after the quantizer's
  const size_t nsc = group ? (size_t)N * (K / group) : 1;
  lutq::QuantScratch sc;
  void* extra = nullptr;
  rc = quant_scratch(stream, scales ? 0 : nsc * sizeof(uint16_t) + 64, &sc, &extra);
  if (rc) return rc;
  uint16_t* sbuf = scales ? scales : reinterpret_cast<uint16_t*>(extra);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = lutq::launch_quantize(sc, w, wdtype, lut, bits, N, K, group, rule, nullptr, sbuf,
                                       false, s);
  if (e != hipSuccess) return hip_fail(e);
  for (int k = 0; k <= iters; ++k) {
    e = lutq::launch_tune_pass(sc, w, wdtype, lut, bits, N, K, group, sbuf, k < iters, s);
    if (e != hipSuccess) return hip_fail(e);
    double err = 0.0;
    int stop = 0;
    e = hipMemcpyAsync(&err, sc.err_total, sizeof err, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipMemcpyAsync(&stop, sc.stop, sizeof stop, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e);
    if (errors) errors[k] = err;
    if (k == iters || stop) break;
    ++*updates;
  }
  return LUTQ_OK;
}

int lutq_log_base_search(const float* w, int bits, int N, int K, int group, const double* bases,
                         int nbases, int* best, double* errors, void* stream) {
  return lutq_log_base_search_ex(w, LUTQ_WEIGHT_F32, bits, N, K, group, bases, nbases, best,
                                 errors, stream);
}

const char* lutq_strerror(int status) {
  switch (status) {
    case LUTQ_OK: return "success";
    case LUTQ_EINVAL: return "invalid argument (null pointer, negative size or bad option)";
    case LUTQ_EBITS: return "bits must be 2, 3 or 4";
    case LUTQ_EGROUP: return "group must be 0 or a multiple of 128 dividing K, and K a multiple of 128";
    case LUTQ_EALIGN: return "misaligned pointer (x and packed data need 16 bytes, lut 4, others 2)";
    case LUTQ_EMISMATCH: return "shape or layout does not match the packed descriptor";
    case LUTQ_ESIZE: return "destination buffer too small";
    case LUTQ_EHIP: return "HIP runtime error";
    case LUTQ_EUNSUPPORTED: return "size beyond the supported limits";
    case LUTQ_ECAPTURE:
      return "the call needs new scratch memory while its stream is being captured into a graph "
             "(run it once eagerly on that stream first)";
    default: return "unknown lutq status";
  }
}

int lutq_last_hip_error(void) { return g_last_hip; }

void lutq_shutdown(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  int cur = 0;
  (void)hipGetDevice(&cur);
  auto release = [](int dev, void* base) {
    (void)hipSetDevice(dev);
    (void)hipFree(base);
  };
  for (auto& kv : g_scratch)
    if (kv.second.base) release(kv.first.first, kv.second.base);
  for (auto& r : g_retired) release(r.first, r.second);
  (void)hipSetDevice(cur);
  g_scratch.clear();
  g_retired.clear();
}

}  // extern "C"
