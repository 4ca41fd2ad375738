// C-ABI layer of libtq.so: argument validation, codebook handles, device
// tables and kernel launches.  Declarations and contracts: include/tq.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "tq.h"
#include "tq_internal.h"
#include "tq_kernels.h"

// Scratch of tq_decode_attention_static, for callers that cannot allocate:
// one copy of this array per GPU, loaded with the code object and held until
// the process ends.  On the host `scratch` names a stand-in, not the device
// copy: host code only ever uses the address hipGetSymbolAddress returns for
// the current device (scratch_address below).
constexpr size_t kStaticScratchBytes = size_t{16} << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

thread_local std::string g_last_error;

tq_status fail(tq_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

tq_status ok() {
  return TQ_OK;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Switches to `device` for the lifetime of the guard, restoring the caller's.
struct DeviceGuard {
  int prev = -1;
  bool changed = false;
  hipError_t err = hipSuccess;
  explicit DeviceGuard(int device) {
    err = hipGetDevice(&prev);
    if (err != hipSuccess) return;
    if (prev != device) {
      err = hipSetDevice(device);
      changed = (err == hipSuccess);
    }
  }
  ~DeviceGuard() {
    if (changed) (void)hipSetDevice(prev);
  }
};

int cu_count(int device) {
  static std::mutex mu;
  static std::vector<int> cache;
  std::lock_guard<std::mutex> lock(mu);
  if (device >= static_cast<int>(cache.size())) cache.resize(device + 1, 0);
  if (cache[device] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || v <= 0) v = 256;
    cache[device] = v;
  }
  return cache[device];
}

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

// IEEE binary16 bits of a float, round to nearest even (normal and subnormal
// results; the tables only hold finite values well inside the range).
uint16_t f16_bits_rne(float v) {
  uint32_t u;
  std::memcpy(&u, &v, 4);
  const uint32_t sign = (u >> 16) & 0x8000u;
  const uint32_t au = u & 0x7fffffffu;
  if (au >= 0x47800000u) return static_cast<uint16_t>(sign | 0x7c00u);   // overflow -> inf
  if (au < 0x38800000u) {                                                  // subnormal or zero
    float a;
    std::memcpy(&a, &au, 4);
    const float scaled = a * 16777216.0f;   // a / 2^-24
    const uint32_t q = static_cast<uint32_t>(std::nearbyint(scaled));
    return static_cast<uint16_t>(sign | q);
  }
  const uint32_t mant = au & 0x7fffffu;
  const int32_t exp = static_cast<int32_t>(au >> 23) - 127 + 15;
  uint32_t h = (static_cast<uint32_t>(exp) << 10) | (mant >> 13);
  const uint32_t rem = mant & 0x1fffu;
  if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) ++h;   // carries into the exponent correctly
  return static_cast<uint16_t>(sign | h);
}

float f16_bits_to_float(uint16_t b) {
  const uint32_t sign = (b & 0x8000u) << 16, e = (b >> 10) & 0x1fu, m = b & 0x3ffu;
  float r;
  if (e == 0) {
    r = std::ldexp(static_cast<float>(m), -24);
    uint32_t u;
    std::memcpy(&u, &r, 4);
    u |= sign;
    std::memcpy(&r, &u, 4);
    return r;
  }
  const uint32_t u = sign | ((e + 112u) << 23) | (m << 13);
  std::memcpy(&r, &u, 4);
  return r;
}

std::mutex g_scratch_mu;
std::vector<void *> g_scratch_addr;   // per device ordinal; null until resolved

// Device address of `scratch` on `device`, resolved once per device with that
// device current (codebook set-up does it; the entry point's first call on a
// device otherwise).  Allocates nothing on the GPU.
tq_status scratch_address(int device, void **out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (device < 0) return fail(TQ_ERR_INVALID_ARG, "scratch needs a GPU device");
  if (device < static_cast<int>(g_scratch_addr.size()) && g_scratch_addr[device] != nullptr) {
    *out = g_scratch_addr[device];
    return ok();
  }
  DeviceGuard guard(device);
  if (guard.err != hipSuccess) return fail(TQ_ERR_DEVICE, "hipSetDevice(%d): %s", device, hipGetErrorString(guard.err));
  void *p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || p == nullptr)
    return fail(TQ_ERR_DEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", device, hipGetErrorString(e));
  if (device >= static_cast<int>(g_scratch_addr.size())) g_scratch_addr.resize(device + 1, nullptr);
  g_scratch_addr[device] = p;
  *out = p;
  return ok();
}

tq_status upload_tables(tq_codebook *cb) {
  const tq::HostTables &h = cb->host;
  const int d = h.d, m = h.m;
  // Device tables are only built for the GPU path's shape.
  size_t off = 0;
  cb->off_centroids = off;
  off = align256(off + tq::kMaxLevels * sizeof(float));
  cb->off_thresholds = off;
  off = align256(off + tq::kMaxLevels * sizeof(float));
  cb->off_rot_frag = off;
  off = align256(off + tq::kFragBytes);
  cb->off_qjl_frag = off;
  off = align256(off + (m > 0 ? tq::kFragBytes : 0));
  cb->off_dec_rot_frag = off;
  off = align256(off + tq::kFragBytes);
  cb->off_dec_qjl_frag = off;
  off = align256(off + (m > 0 ? tq::kFragBytes : 0));
  cb->off_rot_f32 = off;
  off = align256(off + static_cast<size_t>(d) * d * sizeof(float));
  cb->off_rot_t_f32 = off;
  off = align256(off + static_cast<size_t>(d) * d * sizeof(float));
  cb->off_qjl_rot_t_f32 = off;
  off = align256(off + static_cast<size_t>(m) * d * sizeof(float));
  cb->off_key_lut = off;
  off = align256(off + tq::kKeyLutBytes);
  cb->off_pair_lut = off;
  off = align256(off + tq::kPairLutBytes);
  cb->off_qcells = off;
  off = align256(off + tq::kQuantCellEntries * 4 * sizeof(float));
  cb->off_mkey_lut = off;
  off = align256(off + tq::kMKeyLutBytes);
  cb->off_mval_lut = off;
  off = align256(off + tq::kMValLutBytes);
  cb->off_sign_lut = off;
  off = align256(off + tq::kSignLutBytes);
  const bool split = h.n_wide > 0;
  if (split) {
    cb->off_qcells_w = off;
    off = align256(off + tq::kQuantCellEntries * 4 * sizeof(float));
    cb->off_mkey_lut_w = off;
    off = align256(off + tq::kMKeyLutBytes);
    cb->off_mval_lut_w = off;
    off = align256(off + tq::kMValLutBytes);
  }
  cb->dev_bytes = off;

  std::vector<unsigned char> img(off, 0);
  std::memcpy(img.data() + cb->off_centroids, h.centroids.data(), h.centroids.size() * sizeof(float));
  std::memcpy(img.data() + cb->off_thresholds, h.thresholds.data(), h.thresholds.size() * sizeof(float));
  // split widths: Pi's output rows and S's input columns follow the encode's
  // split coordinate order (the wide coordinates in blocks 0..3); the QJL
  // fragments hold -S (the encode takes each sign bit from -p)
  tq::pack_encode_fragments(h.rotation.data(), img.data() + cb->off_rot_frag, split, false, false);
  if (m > 0) tq::pack_encode_fragments(h.qjl.data(), img.data() + cb->off_qjl_frag, false, split, true);
  std::memcpy(img.data() + cb->off_rot_f32, h.rotation.data(), h.rotation.size() * sizeof(float));
  float *rt = reinterpret_cast<float *>(img.data() + cb->off_rot_t_f32);
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) rt[i * d + j] = h.rotation[static_cast<size_t>(j) * d + i];
  // the matrix-core decode's query operands: Pi (its rows in the encode's
  // coordinate order) and S Pi, in fp16 hi/lo
  if (!tq::pack_decode_fragments(h.rotation64.data(), img.data() + cb->off_dec_rot_frag, split))
    return fail(TQ_ERR_UNSUPPORTED, "rotation entry out of the decode operands' fp16 range");
  if (m > 0) {
    // S Pi in double, rounded once per use: the decode projects the raw query
    // with it (s = S Pi q) instead of projecting Pi q with S.
    std::vector<double> sp(static_cast<size_t>(m) * d);
    for (int r = 0; r < m; ++r)
      for (int i = 0; i < d; ++i) {
        double v = 0.0;
        for (int j = 0; j < d; ++j)
          v += h.qjl64[static_cast<size_t>(r) * d + j] * h.rotation64[static_cast<size_t>(j) * d + i];
        sp[static_cast<size_t>(r) * d + i] = v;
      }
    float *st = reinterpret_cast<float *>(img.data() + cb->off_qjl_rot_t_f32);
    for (int i = 0; i < d; ++i)
      for (int r = 0; r < m; ++r) st[i * m + r] = static_cast<float>(sp[static_cast<size_t>(r) * d + i]);
    if (!tq::pack_decode_fragments(sp.data(), img.data() + cb->off_dec_qjl_frag, false))
      return fail(TQ_ERR_UNSUPPORTED, "S Pi entry out of the decode operands' fp16 range");
  }
  auto pair = [](uint16_t x, uint16_t y) { return static_cast<uint32_t>(x) | (static_cast<uint32_t>(y) << 16); };
  // Matrix-core decode operand tables of one codebook (layouts in
  // tq_kernels.h): centroid c as (hi, lo) with lo = c - hi, two per 32-bit word.
  auto operand_tables = [&](const std::vector<float> &cent, int b, size_t off_k, size_t off_v) {
    const int levels = 1 << b, mask = levels - 1;
    std::vector<uint16_t> hi(levels), lo(levels), khi(levels), klo(levels);
    for (int k = 0; k < levels; ++k) {
      hi[k] = tq::bf16_bits_rne(cent[k]);
      lo[k] = tq::bf16_bits_rne(cent[k] - tq::bf16_bits_to_float(hi[k]));
      // keys: fp16 (hi, lo) of 256 c (the score products run in fp16)
      const float x = 256.0f * cent[k];
      khi[k] = f16_bits_rne(x);
      klo[k] = f16_bits_rne(x - f16_bits_to_float(khi[k]));
    }
    uint32_t *mk = reinterpret_cast<uint32_t *>(img.data() + off_k);
    uint32_t *mv = reinterpret_cast<uint32_t *>(img.data() + off_v);
    for (int e = 0; e < (1 << (2 * b)); ++e) {
      const int c0 = e & mask, c1 = (e >> b) & mask;
      mk[2 * e] = pair(khi[c0], klo[c0]);
      mk[2 * e + 1] = pair(khi[c1], klo[c1]);
      mv[2 * e] = pair(hi[c0], lo[c0]);   // values: bf16 (hi, lo) of c
      mv[2 * e + 1] = pair(hi[c1], lo[c1]);
    }
  };
  operand_tables(h.centroids, h.bits, cb->off_mkey_lut, cb->off_mval_lut);
  if (split) operand_tables(h.wide_centroids, h.bits + 1, cb->off_mkey_lut_w, cb->off_mval_lut_w);
  {
    uint32_t *sg = reinterpret_cast<uint32_t *>(img.data() + cb->off_sign_lut);
    const uint16_t plus = 0x3C00, minus = 0xBC00;   // fp16 +1, -1
    for (int e = 0; e < 256; ++e)
      for (int p = 0; p < 4; ++p)
        sg[e * 4 + p] = pair(((e >> (2 * p)) & 1) ? plus : minus, ((e >> (2 * p + 1)) & 1) ? plus : minus);
  }
  {
    const int b = h.bits, mask = (1 << b) - 1;
    const int entries = 1 << tq::key_lut_bits(b), coords = tq::key_lut_coords(b);
    float *kl = reinterpret_cast<float *>(img.data() + cb->off_key_lut);
    for (int e = 0; e < entries; ++e)
      for (int c = 0; c < coords; ++c) kl[e * coords + c] = h.centroids[(e >> (c * b)) & mask];
    float *pl = reinterpret_cast<float *>(img.data() + cb->off_pair_lut);
    for (int e = 0; e < (1 << (2 * b)); ++e) {
      pl[2 * e] = h.centroids[e & mask];
      pl[2 * e + 1] = h.centroids[(e >> b) & mask];
    }
  }
  if (!tq::build_quant_cells(h.thresholds.data(), h.centroids.data(), h.levels,
                             reinterpret_cast<float *>(img.data() + cb->off_qcells), &cb->qscale, &cb->qbias))
    return fail(TQ_ERR_UNSUPPORTED, "codebook thresholds do not fit the quantizer cell grid");
  if (split) {
    float qs = 0.f, qb = 0.f;
    if (!tq::build_quant_cells(h.wide_thresholds.data(), h.wide_centroids.data(), 2 * h.levels,
                               reinterpret_cast<float *>(img.data() + cb->off_qcells_w), &qs, &qb) ||
        qs != cb->qscale || qb != cb->qbias)
      return fail(TQ_ERR_UNSUPPORTED, "wide codebook thresholds do not fit the quantizer cell grid");
  }
  DeviceGuard guard(cb->device);
  if (guard.err != hipSuccess) return fail(TQ_ERR_DEVICE, "hipSetDevice(%d): %s", cb->device, hipGetErrorString(guard.err));
  hipError_t e = hipMalloc(&cb->dev_buf, off);
  if (e != hipSuccess) {
    cb->dev_buf = nullptr;
    return fail(TQ_ERR_ALLOC, "hipMalloc(%zu): %s", off, hipGetErrorString(e));
  }
  e = hipMemcpy(cb->dev_buf, img.data(), off, hipMemcpyHostToDevice);
  if (e != hipSuccess) return fail(TQ_ERR_DEVICE, "hipMemcpy: %s", hipGetErrorString(e));
  return ok();
}

template <typename T>
const T *dev_ptr(const tq_codebook *cb, size_t off) {
  return reinterpret_cast<const T *>(static_cast<const unsigned char *>(cb->dev_buf) + off);
}

tq_status build_codebook(int32_t head_dim, int32_t mse_bits, int32_t wide_coords, int32_t qjl_dim, uint64_t rot_seed,
                         uint64_t qjl_seed, int32_t device, tq_codebook **out) {
  if (out == nullptr) return fail(TQ_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (device < -1) return fail(TQ_ERR_INVALID_ARG, "device must be >= -1");
  if (device >= 0) {
    if (head_dim != tq::kHeadDim)
      return fail(TQ_ERR_UNSUPPORTED, "the GPU path supports head_dim 128 only (got %d)", head_dim);
    if (qjl_dim != 0 && qjl_dim != tq::kQjlDim)
      return fail(TQ_ERR_UNSUPPORTED, "the GPU path supports qjl_dim 0 or 128 only (got %d)", qjl_dim);
    if (wide_coords != 0 && wide_coords != tq::kSplitWide)
      return fail(TQ_ERR_UNSUPPORTED, "the GPU path supports wide_coords 0 or %d only (got %d)", tq::kSplitWide,
                  wide_coords);
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || device >= count)
      return fail(TQ_ERR_INVALID_ARG, "device %d not present (%d devices)", device, count);
  }
  tq_codebook *cb = new (std::nothrow) tq_codebook();
  if (cb == nullptr) return fail(TQ_ERR_ALLOC, "host allocation failed");
  std::string err;
  if (!tq::build_host_tables(head_dim, mse_bits, wide_coords, qjl_dim, rot_seed, qjl_seed, &cb->host, &err)) {
    delete cb;
    return fail(TQ_ERR_INVALID_ARG, "%s", err.c_str());
  }
  cb->rot_seed = rot_seed;
  cb->qjl_seed = qjl_seed;
  cb->device = device;
  if (device >= 0) {
    tq_status s = upload_tables(cb);
    void *scr = nullptr;
    if (s == TQ_OK) s = scratch_address(device, &scr);   // set-up of the allocation-free decode
    if (s != TQ_OK) {
      tq_codebook_free(cb);
      return s;
    }
  }
  *out = cb;
  return ok();
}

}  // namespace

extern "C" {

tq_status tq_codebook_build(int32_t head_dim, int32_t mse_bits, int32_t qjl_dim, uint64_t rot_seed,
                            uint64_t qjl_seed, int32_t device, tq_codebook **out) {
  return build_codebook(head_dim, mse_bits, 0, qjl_dim, rot_seed, qjl_seed, device, out);
}

tq_status tq_codebook_build_split(int32_t head_dim, int32_t mse_bits, int32_t wide_coords, int32_t qjl_dim,
                                  uint64_t rot_seed, uint64_t qjl_seed, int32_t device, tq_codebook **out) {
  return build_codebook(head_dim, mse_bits, wide_coords, qjl_dim, rot_seed, qjl_seed, device, out);
}

tq_status tq_codebook_split_info(const tq_codebook *cb, int32_t *wide_coords, int32_t *wide_bits) {
  if (cb == nullptr) return fail(TQ_ERR_INVALID_ARG, "codebook is NULL");
  if (wide_coords) *wide_coords = cb->host.n_wide;
  if (wide_bits) *wide_bits = cb->host.n_wide > 0 ? cb->host.bits + 1 : 0;
  return ok();
}

tq_status tq_codebook_export_wide(const tq_codebook *cb, float *centroids, float *thresholds) {
  if (cb == nullptr) return fail(TQ_ERR_INVALID_ARG, "codebook is NULL");
  const tq::HostTables &h = cb->host;
  if (h.n_wide == 0) return fail(TQ_ERR_INVALID_ARG, "the codebook has no wide coordinates");
  if (centroids) std::memcpy(centroids, h.wide_centroids.data(), h.wide_centroids.size() * sizeof(float));
  if (thresholds) std::memcpy(thresholds, h.wide_thresholds.data(), h.wide_thresholds.size() * sizeof(float));
  return ok();
}

tq_status tq_codebook_free(tq_codebook *cb) {
  if (cb == nullptr) return ok();
  tq_status s = TQ_OK;
  if (cb->dev_buf != nullptr) {
    DeviceGuard guard(cb->device);
    if (hipFree(cb->dev_buf) != hipSuccess) s = fail(TQ_ERR_DEVICE, "hipFree failed");
  }
  delete cb;
  return s;
}

tq_status tq_codebook_info(const tq_codebook *cb, int32_t *head_dim, int32_t *mse_bits, int32_t *qjl_dim,
                           int32_t *device) {
  if (cb == nullptr) return fail(TQ_ERR_INVALID_ARG, "codebook is NULL");
  if (head_dim) *head_dim = cb->host.d;
  if (mse_bits) *mse_bits = cb->host.bits;
  if (qjl_dim) *qjl_dim = cb->host.m;
  if (device) *device = cb->device;
  return ok();
}

tq_status tq_codebook_export(const tq_codebook *cb, float *centroids, float *thresholds, float *rotation,
                             float *qjl) {
  if (cb == nullptr) return fail(TQ_ERR_INVALID_ARG, "codebook is NULL");
  const tq::HostTables &h = cb->host;
  if (qjl != nullptr && h.m == 0) return fail(TQ_ERR_INVALID_ARG, "qjl requested but qjl_dim is 0");
  if (centroids) std::memcpy(centroids, h.centroids.data(), h.centroids.size() * sizeof(float));
  if (thresholds) std::memcpy(thresholds, h.thresholds.data(), h.thresholds.size() * sizeof(float));
  if (rotation) std::memcpy(rotation, h.rotation.data(), h.rotation.size() * sizeof(float));
  if (qjl) std::memcpy(qjl, h.qjl.data(), h.qjl.size() * sizeof(float));
  return ok();
}

tq_status tq_codebook_export_f64(const tq_codebook *cb, double *centroids, double *thresholds, double *rotation,
                                 double *qjl) {
  if (cb == nullptr) return fail(TQ_ERR_INVALID_ARG, "codebook is NULL");
  const tq::HostTables &h = cb->host;
  if (qjl != nullptr && h.m == 0) return fail(TQ_ERR_INVALID_ARG, "qjl requested but qjl_dim is 0");
  if (centroids) std::memcpy(centroids, h.centroids64.data(), h.centroids64.size() * sizeof(double));
  if (thresholds) std::memcpy(thresholds, h.thresholds64.data(), h.thresholds64.size() * sizeof(double));
  if (rotation) std::memcpy(rotation, h.rotation64.data(), h.rotation64.size() * sizeof(double));
  if (qjl) std::memcpy(qjl, h.qjl64.data(), h.qjl64.size() * sizeof(double));
  return ok();
}

tq_status tq_record_words(const tq_codebook *cb, int32_t *code_words, int32_t *sign_words) {
  if (cb == nullptr) return fail(TQ_ERR_INVALID_ARG, "codebook is NULL");
  const int bitsum = cb->host.d * cb->host.bits + cb->host.n_wide;
  if (code_words) *code_words = (bitsum + 31) / 32;
  if (sign_words) *sign_words = cb->host.m / 32;
  return ok();
}

}  // extern "C"

namespace {

// Validation and launch arguments of an encode (no launch).
tq_status prepare_encode(const tq_codebook *cb, const void *x, tq_dtype x_dtype, int64_t n, int64_t x_row_stride,
                         const int64_t *dst_row, int64_t cache_rows, uint32_t *codes, uint32_t *signs, float *norms,
                         float *res_norms, float *dbg_rot, float *dbg_proj, tq::EncodeArgs *out) {
  if (cb == nullptr) return fail(TQ_ERR_INVALID_ARG, "codebook is NULL");
  if (cb->device < 0) return fail(TQ_ERR_INVALID_ARG, "host-only codebook cannot encode");
  const int d = cb->host.d, m = cb->host.m;
  if (x_dtype != TQ_F32 && x_dtype != TQ_BF16) return fail(TQ_ERR_INVALID_ARG, "x_dtype must be TQ_F32 or TQ_BF16");
  if (n < 0) return fail(TQ_ERR_INVALID_ARG, "n < 0");
  if (n == 0) return ok();   // nothing to launch
  if (x == nullptr || codes == nullptr || norms == nullptr) return fail(TQ_ERR_INVALID_ARG, "x, codes and norms are required");
  if (x_row_stride < d) return fail(TQ_ERR_INVALID_ARG, "x_row_stride (%lld) < head_dim", static_cast<long long>(x_row_stride));
  const size_t esize = (x_dtype == TQ_F32) ? 4 : 2;
  if (!aligned(x, 16) || (static_cast<size_t>(x_row_stride) * esize) % 16 != 0)
    return fail(TQ_ERR_INVALID_ARG, "x and its row stride must be 16-byte aligned");
  if ((m > 0) != (signs != nullptr) || (m > 0) != (res_norms != nullptr))
    return fail(TQ_ERR_INVALID_ARG, "signs and res_norms must be given iff qjl_dim > 0");
  if (dbg_proj != nullptr && m == 0) return fail(TQ_ERR_INVALID_ARG, "dbg_proj needs qjl_dim > 0");
  if (cache_rows < 0 || (dst_row == nullptr && cache_rows < n))
    return fail(TQ_ERR_INVALID_ARG, "cache_rows (%lld) too small for n (%lld)", static_cast<long long>(cache_rows),
                static_cast<long long>(n));
  if (!aligned(codes, 4) || !aligned(norms, 4) || (signs && !aligned(signs, 4)) || (res_norms && !aligned(res_norms, 4)) ||
      (dbg_rot && !aligned(dbg_rot, 16)) || (dbg_proj && !aligned(dbg_proj, 16)) || (dst_row && !aligned(dst_row, 8)))
    return fail(TQ_ERR_INVALID_ARG, "misaligned output pointer");
  tq::EncodeArgs a{};
  a.x = x;
  a.x_stride = x_row_stride;
  a.n = n;
  a.dst_row = dst_row;
  a.cache_rows = cache_rows;
  a.codes = codes;
  a.signs = signs;
  a.norms = norms;
  a.res_norms = res_norms;
  a.dbg_rot = dbg_rot;
  a.dbg_proj = dbg_proj;
  a.frag_rot = dev_ptr<uint4>(cb, cb->off_rot_frag);
  a.frag_qjl = (m > 0) ? dev_ptr<uint4>(cb, cb->off_qjl_frag) : nullptr;
  a.qlut = dev_ptr<float4>(cb, cb->off_qcells);
  a.qlut_wide = cb->host.n_wide > 0 ? dev_ptr<float4>(cb, cb->off_qcells_w) : nullptr;
  a.qscale = cb->qscale;
  a.qbias = cb->qbias;
  *out = a;
  return ok();
}

tq_status run_encode(const tq_codebook *cb, const tq::EncodeArgs &a, bool x_f32, void *stream) {
  DeviceGuard guard(cb->device);
  if (guard.err != hipSuccess) return fail(TQ_ERR_DEVICE, "hipSetDevice: %s", hipGetErrorString(guard.err));
  hipError_t e = tq::launch_encode(a, cb->host.bits, cb->host.m > 0, x_f32, cb->host.n_wide > 0,
                                   cu_count(cb->device), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(TQ_ERR_DEVICE, "encode launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

tq_status tq_encode_kv(const tq_codebook *cb, const void *x, tq_dtype x_dtype, int64_t n, int64_t x_row_stride,
                       const int64_t *dst_row, int64_t cache_rows, uint32_t *codes, uint32_t *signs, float *norms,
                       float *res_norms, float *dbg_rot, float *dbg_proj, void *stream) {
  tq::EncodeArgs a{};
  tq_status st = prepare_encode(cb, x, x_dtype, n, x_row_stride, dst_row, cache_rows, codes, signs, norms, res_norms,
                                dbg_rot, dbg_proj, &a);
  if (st != TQ_OK || n == 0) return st;
  return run_encode(cb, a, x_dtype == TQ_F32, stream);
}

tq_status tq_decode_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int64_t t_cap,
                                    size_t *bytes) {
  if (bytes == nullptr) return fail(TQ_ERR_INVALID_ARG, "bytes is NULL");
  if (batch < 1 || n_q_heads < 1 || n_kv_heads < 1 || t_cap < 1 || n_q_heads % n_kv_heads != 0)
    return fail(TQ_ERR_INVALID_ARG, "bad sizes (batch %d, heads %d/%d, t_cap %lld)", batch, n_q_heads, n_kv_heads,
                static_cast<long long>(t_cap));

  *bytes = tq::plan_decode(batch, n_q_heads, n_kv_heads, t_cap).total_bytes;
  return ok();
}

}  // extern "C"

namespace {

// Validation and launch arguments of the key side of a decode (the query, the
// key cache, seq_len, the workspace and the scores output); no launch.
tq_status prepare_keys(const tq_codebook *kcb, const void *q, tq_dtype q_dtype, const tq_cache *k,
                       const int32_t *seq_len, int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t n_new,
                       float softmax_scale, float *scores, void *workspace, size_t workspace_bytes,
                       tq::DecodeArgs *out_args) {
  if (kcb == nullptr) return fail(TQ_ERR_INVALID_ARG, "codebook is NULL");
  if (kcb->device < 0) return fail(TQ_ERR_INVALID_ARG, "the codebook must live on a GPU device");
  if (q == nullptr || k == nullptr || seq_len == nullptr || workspace == nullptr)
    return fail(TQ_ERR_INVALID_ARG, "NULL argument");
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return fail(TQ_ERR_INVALID_ARG, "bad q_dtype");
  if (batch < 1 || n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads != 0)
    return fail(TQ_ERR_INVALID_ARG, "bad sizes (batch %d, heads %d/%d)", batch, n_q_heads, n_kv_heads);
  const int g = n_q_heads / n_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return fail(TQ_ERR_UNSUPPORTED, "q heads per kv head must be 1, 2, 4 or 8 (got %d)", g);
  // grid limits: y = n_kv_heads * n_new, z = batch; the combine launches batch * n_q_heads * n_new groups
  if (n_new < 1 || batch > 65535 || static_cast<int64_t>(n_new) * n_kv_heads > 65535 ||
      static_cast<int64_t>(batch) * n_q_heads * n_new > (int64_t{1} << 24))
    return fail(TQ_ERR_INVALID_ARG, "bad sizes (batch %d, n_new %d, heads %d/%d): need batch <= 65535, "
                "n_new * n_kv_heads <= 65535, batch * n_q_heads * n_new <= 2^24", batch, n_new, n_q_heads, n_kv_heads);
  if (k->t_cap < 1) return fail(TQ_ERR_INVALID_ARG, "t_cap must be >= 1");
  if (k->t_cap > (int64_t{1} << 30)) return fail(TQ_ERR_UNSUPPORTED, "t_cap above 2^30");

  const int m = kcb->host.m;
  if (k->codes == nullptr || k->norms == nullptr) return fail(TQ_ERR_INVALID_ARG, "cache codes/norms are required");
  if ((m > 0) != (k->signs != nullptr) || (m > 0) != (k->res_norms != nullptr))
    return fail(TQ_ERR_INVALID_ARG, "key signs/res_norms must be given iff the key codebook has qjl_dim > 0");
  if (!aligned(k->codes, 16) || (k->signs && !aligned(k->signs, 16)) || !aligned(k->norms, 4) ||
      (k->res_norms && !aligned(k->res_norms, 4)) || !aligned(q, 4) || !aligned(workspace, 256) ||
      !aligned(seq_len, 4) || (scores && !aligned(scores, 4)))
    return fail(TQ_ERR_INVALID_ARG, "misaligned pointer");
  const tq::DecodePlan plan = tq::plan_chunk(batch, n_q_heads, n_kv_heads, n_new, k->t_cap);
  if (workspace_bytes < plan.total_bytes)
    return fail(TQ_ERR_INVALID_ARG, "workspace too small (%zu < %zu)", workspace_bytes, plan.total_bytes);
  tq::DecodeArgs a{};
  a.q = q;
  a.q_bf16 = (q_dtype == TQ_BF16);
  a.k_codes = k->codes;
  a.k_signs = k->signs;
  a.k_norms = k->norms;
  a.k_res = k->res_norms;
  a.t_cap = k->t_cap;
  a.seq_len = seq_len;
  a.batch = batch;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.n_new = n_new;
  a.k_bits = kcb->host.bits;
  a.qjl_m = m;
  a.scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt(static_cast<float>(kcb->host.d));
  a.qjl_coef = m > 0 ? static_cast<float>(std::sqrt(3.14159265358979323846 / 2.0) / m) : 0.f;
  a.scores = scores;
  a.rot_k_t = dev_ptr<float>(kcb, kcb->off_rot_t_f32);
  a.qjl_rot_t = m > 0 ? dev_ptr<float>(kcb, kcb->off_qjl_rot_t_f32) : nullptr;
  a.k_frag_rot = dev_ptr<uint4>(kcb, kcb->off_rot_frag);
  a.k_frag_qjl = m > 0 ? dev_ptr<uint4>(kcb, kcb->off_qjl_frag) : nullptr;
  a.k_dfrag_rot = dev_ptr<uint4>(kcb, kcb->off_dec_rot_frag);
  a.k_dfrag_qjl = m > 0 ? dev_ptr<uint4>(kcb, kcb->off_dec_qjl_frag) : nullptr;
  a.k_lut = dev_ptr<float>(kcb, kcb->off_key_lut);
  a.k_pair = dev_ptr<float>(kcb, kcb->off_pair_lut);
  a.mk_lut = dev_ptr<void>(kcb, kcb->off_mkey_lut);
  a.sg_lut = dev_ptr<void>(kcb, kcb->off_sign_lut);
  a.k_split = kcb->host.n_wide > 0;
  a.mk_lut_w = a.k_split ? dev_ptr<void>(kcb, kcb->off_mkey_lut_w) : nullptr;
  a.norm_vec4 = (k->t_cap % 4 == 0) && aligned(k->norms, 16) && (k->res_norms == nullptr || aligned(k->res_norms, 16));
  if (a.k_split && !(n_new == 1 && a.norm_vec4 && a.t_cap <= tq::kMDecodeMaxTcap))
    return fail(TQ_ERR_UNSUPPORTED, "split-width keys are read by the single-query matrix-core decode only: "
                "n_new 1, t_cap a multiple of 4, 16-byte aligned norm arrays");
  unsigned char *ws = static_cast<unsigned char *>(workspace);
  a.ws_qslot = reinterpret_cast<float *>(ws + plan.off_qslot);
  a.ws_part_o = reinterpret_cast<float *>(ws + plan.off_part_o);
  a.ws_part_ml = reinterpret_cast<float *>(ws + plan.off_part_ml);
  a.chunk = plan.chunk;
  a.n_chunks = plan.n_chunks;
  *out_args = a;
  return ok();
}

// Validation and launch arguments of a decode (no launch): the key side, then
// the value cache, its codebook and the output.
tq_status prepare_decode(const tq_codebook *kcb, const tq_codebook *vcb, const void *q, tq_dtype q_dtype,
                         const tq_cache *k, const tq_cache *v, const int32_t *seq_len, int32_t batch,
                         int32_t n_q_heads, int32_t n_kv_heads, int32_t n_new, float softmax_scale, void *out,
                         tq_dtype out_dtype, float *dbg_scores, void *workspace, size_t workspace_bytes,
                         tq::DecodeArgs *out_args) {
  if (kcb == nullptr || vcb == nullptr) return fail(TQ_ERR_INVALID_ARG, "codebook is NULL");
  if (kcb->device < 0 || vcb->device != kcb->device)
    return fail(TQ_ERR_INVALID_ARG, "codebooks must live on the same GPU device");
  if (kcb->host.d != vcb->host.d) return fail(TQ_ERR_INVALID_ARG, "key and value head_dim differ");
  if (vcb->host.m != 0) return fail(TQ_ERR_INVALID_ARG, "the value codebook must have qjl_dim 0");
  if (v == nullptr || out == nullptr) return fail(TQ_ERR_INVALID_ARG, "NULL argument");
  if (out_dtype != TQ_F32 && out_dtype != TQ_BF16) return fail(TQ_ERR_INVALID_ARG, "bad out_dtype");
  tq::DecodeArgs a{};
  const tq_status st = prepare_keys(kcb, q, q_dtype, k, seq_len, batch, n_q_heads, n_kv_heads, n_new, softmax_scale,
                                    dbg_scores, workspace, workspace_bytes, &a);
  if (st != TQ_OK) return st;
  if (v->t_cap != k->t_cap) return fail(TQ_ERR_INVALID_ARG, "key/value t_cap must match");
  if (v->codes == nullptr || v->norms == nullptr) return fail(TQ_ERR_INVALID_ARG, "cache codes/norms are required");
  if (!aligned(v->codes, 16) || !aligned(v->norms, 4) || !aligned(out, 4))
    return fail(TQ_ERR_INVALID_ARG, "misaligned pointer");
  a.v_codes = v->codes;
  a.v_norms = v->norms;
  a.v_bits = vcb->host.bits;
  a.out = out;
  a.out_bf16 = (out_dtype == TQ_BF16);
  a.rot_v = dev_ptr<float>(vcb, vcb->off_rot_f32);
  a.v_lut = dev_ptr<float>(vcb, vcb->off_pair_lut);
  a.mv_lut = dev_ptr<void>(vcb, vcb->off_mval_lut);
  a.v_split = vcb->host.n_wide > 0;
  a.mv_lut_w = a.v_split ? dev_ptr<void>(vcb, vcb->off_mval_lut_w) : nullptr;
  a.norm_vec4 = a.norm_vec4 && aligned(v->norms, 16);
  if (a.k_split != a.v_split)
    return fail(TQ_ERR_UNSUPPORTED, "split widths need both codebooks split (keys %d, values %d wide coordinates)",
                kcb->host.n_wide, vcb->host.n_wide);
  if (a.v_split && !tq::mdecode_can_run(a))
    return fail(TQ_ERR_UNSUPPORTED, "split-width values are read by the single-query matrix-core decode only: "
                "t_cap a multiple of 4, 16-byte aligned norm arrays");
  *out_args = a;
  return ok();
}

tq_status run_decode(const tq_codebook *kcb, const tq::DecodeArgs &a, void *stream) {
  DeviceGuard guard(kcb->device);
  if (guard.err != hipSuccess) return fail(TQ_ERR_DEVICE, "hipSetDevice: %s", hipGetErrorString(guard.err));
  hipError_t e = tq::launch_decode(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(TQ_ERR_DEVICE, "decode launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

tq_status tq_decode_attention(const tq_codebook *kcb, const tq_codebook *vcb, const void *q, tq_dtype q_dtype,
                              const tq_cache *k, const tq_cache *v, const int32_t *seq_len, int32_t batch,
                              int32_t n_q_heads, int32_t n_kv_heads, float softmax_scale, void *out,
                              tq_dtype out_dtype, float *dbg_scores, void *workspace, size_t workspace_bytes,
                              void *stream) {
  tq::DecodeArgs a{};
  const tq_status st = prepare_decode(kcb, vcb, q, q_dtype, k, v, seq_len, batch, n_q_heads, n_kv_heads, 1,
                                      softmax_scale, out, out_dtype, dbg_scores, workspace, workspace_bytes, &a);
  if (st != TQ_OK) return st;
  return run_decode(kcb, a, stream);
}

tq_status tq_decode_attention_static(const tq_codebook *kcb, const tq_codebook *vcb, const void *q,
                                     tq_dtype q_dtype, const tq_cache *k, const tq_cache *v, const int32_t *seq_len,
                                     int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, float softmax_scale,
                                     void *out, tq_dtype out_dtype, float *dbg_scores, void *stream) {
  if (kcb == nullptr) return fail(TQ_ERR_INVALID_ARG, "codebook is NULL");
  if (kcb->device < 0) return fail(TQ_ERR_INVALID_ARG, "the codebook must live on a GPU device");
  if (k == nullptr) return fail(TQ_ERR_INVALID_ARG, "NULL argument");
  if (batch < 1 || n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads != 0 || k->t_cap < 1)
    return fail(TQ_ERR_INVALID_ARG, "bad sizes (batch %d, heads %d/%d)", batch, n_q_heads, n_kv_heads);
  const size_t need = tq::plan_decode(batch, n_q_heads, n_kv_heads, k->t_cap).total_bytes;
  if (need > kStaticScratchBytes)
    return fail(TQ_ERR_INVALID_ARG, "these sizes need %zu bytes of scratch; the static scratch holds %zu", need,
                kStaticScratchBytes);
  void *scr = nullptr;
  tq_status st = scratch_address(kcb->device, &scr);
  if (st != TQ_OK) return st;
  tq::DecodeArgs a{};
  st = prepare_decode(kcb, vcb, q, q_dtype, k, v, seq_len, batch, n_q_heads, n_kv_heads, 1, softmax_scale, out,
                      out_dtype, dbg_scores, scr, kStaticScratchBytes, &a);
  if (st != TQ_OK) return st;
  return run_decode(kcb, a, stream);
}

tq_status tq_chunk_attention(const tq_codebook *kcb, const tq_codebook *vcb, const void *q, tq_dtype q_dtype,
                             const tq_cache *k, const tq_cache *v, const int32_t *seq_len, int32_t batch,
                             int32_t n_q_heads, int32_t n_kv_heads, int32_t n_new, float softmax_scale, void *out,
                             tq_dtype out_dtype, void *workspace, size_t workspace_bytes, void *stream) {
  tq::DecodeArgs a{};
  const tq_status st = prepare_decode(kcb, vcb, q, q_dtype, k, v, seq_len, batch, n_q_heads, n_kv_heads, n_new,
                                      softmax_scale, out, out_dtype, nullptr, workspace, workspace_bytes, &a);
  if (st != TQ_OK) return st;
  if (!tq::chunk_uses_mfma(n_q_heads / n_kv_heads, n_new)) return run_decode(kcb, a, stream);
  DeviceGuard guard(kcb->device);
  if (guard.err != hipSuccess) return fail(TQ_ERR_DEVICE, "hipSetDevice: %s", hipGetErrorString(guard.err));
  const hipError_t e = tq::launch_chunk_mfma(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(TQ_ERR_DEVICE, "chunk attention launch: %s", hipGetErrorString(e));
  return ok();
}

tq_status tq_chunk_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t n_new, int64_t t_cap,
                                   size_t *bytes) {
  if (bytes == nullptr) return fail(TQ_ERR_INVALID_ARG, "bytes is NULL");
  if (batch < 1 || n_q_heads < 1 || n_kv_heads < 1 || t_cap < 1 || n_new < 1 || n_q_heads % n_kv_heads != 0)
    return fail(TQ_ERR_INVALID_ARG, "bad sizes (batch %d, heads %d/%d, n_new %d, t_cap %lld)", batch, n_q_heads,
                n_kv_heads, n_new, static_cast<long long>(t_cap));
  *bytes = tq::plan_chunk(batch, n_q_heads, n_kv_heads, n_new, t_cap).total_bytes;
  return ok();
}

tq_status tq_append_decode(const tq_codebook *kcb, const tq_codebook *vcb, const void *k_new, const void *v_new,
                           tq_dtype kv_dtype, const void *q, tq_dtype q_dtype, const tq_cache *k, const tq_cache *v,
                           int32_t *seq_len, int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                           float softmax_scale, void *out, tq_dtype out_dtype, void *workspace,
                           size_t workspace_bytes, void *stream) {
  tq::DecodeArgs da{};
  tq_status st = prepare_decode(kcb, vcb, q, q_dtype, k, v, seq_len, batch, n_q_heads, n_kv_heads, 1, softmax_scale,
                                out, out_dtype, nullptr, workspace, workspace_bytes, &da);
  if (st != TQ_OK) return st;
  if (k_new == nullptr || v_new == nullptr) return fail(TQ_ERR_INVALID_ARG, "k_new and v_new are required");
  const int64_t n = static_cast<int64_t>(batch) * n_kv_heads;
  const int64_t rows = n * k->t_cap;
  const int d = kcb->host.d;
  tq::EncodeArgs ka{}, va{};
  st = prepare_encode(kcb, k_new, kv_dtype, n, d, nullptr, rows, const_cast<uint32_t *>(k->codes),
                      const_cast<uint32_t *>(k->signs), const_cast<float *>(k->norms), const_cast<float *>(k->res_norms),
                      nullptr, nullptr, &ka);
  if (st != TQ_OK) return st;
  st = prepare_encode(vcb, v_new, kv_dtype, n, d, nullptr, rows, const_cast<uint32_t *>(v->codes), nullptr,
                      const_cast<float *>(v->norms), nullptr, nullptr, nullptr, &va);
  if (st != TQ_OK) return st;
  for (tq::EncodeArgs *ea : {&ka, &va}) {
    ea->append_len = seq_len;
    ea->append_heads = n_kv_heads;
    ea->t_cap = k->t_cap;
  }
  da.seq_add = 1;
  da.seq_inc = seq_len;
  if (kv_dtype == TQ_BF16 && kcb->host.n_wide == 0 && vcb->host.n_wide == 0) {
    // keys and values side by side in one launch
    DeviceGuard guard(kcb->device);
    if (guard.err != hipSuccess) return fail(TQ_ERR_DEVICE, "hipSetDevice: %s", hipGetErrorString(guard.err));
    const hipError_t e = tq::launch_encode_pair(ka, kcb->host.bits, kcb->host.m > 0, va, vcb->host.bits,
                                                cu_count(kcb->device), static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(TQ_ERR_DEVICE, "append encode launch: %s", hipGetErrorString(e));
  } else {
    if ((st = run_encode(kcb, ka, kv_dtype == TQ_F32, stream)) != TQ_OK) return st;
    if ((st = run_encode(vcb, va, kv_dtype == TQ_F32, stream)) != TQ_OK) return st;
  }
  return run_decode(kcb, da, stream);
}

tq_status tq_attention_logits(const tq_codebook *kcb, const void *q, tq_dtype q_dtype, const tq_cache *k,
                              const int32_t *seq_len, int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                              float softmax_scale, float *logits, void *workspace, size_t workspace_bytes,
                              void *stream) {
  if (logits == nullptr) return fail(TQ_ERR_INVALID_ARG, "logits is NULL");
  tq::DecodeArgs a{};
  const tq_status st = prepare_keys(kcb, q, q_dtype, k, seq_len, batch, n_q_heads, n_kv_heads, 1, softmax_scale,
                                    logits, workspace, workspace_bytes, &a);
  if (st != TQ_OK) return st;
  DeviceGuard guard(kcb->device);
  if (guard.err != hipSuccess) return fail(TQ_ERR_DEVICE, "hipSetDevice: %s", hipGetErrorString(guard.err));
  const hipError_t e = tq::launch_logits(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(TQ_ERR_DEVICE, "logits launch: %s", hipGetErrorString(e));
  return ok();
}

const char *tq_status_string(tq_status s) {
  switch (s) {
    case TQ_OK: return "TQ_OK";
    case TQ_ERR_INVALID_ARG: return "TQ_ERR_INVALID_ARG";
    case TQ_ERR_UNSUPPORTED: return "TQ_ERR_UNSUPPORTED";
    case TQ_ERR_ALLOC: return "TQ_ERR_ALLOC";
    case TQ_ERR_DEVICE: return "TQ_ERR_DEVICE";
  }
  return "TQ_UNKNOWN_STATUS";
}

const char *tq_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
