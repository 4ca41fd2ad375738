// Encode kernel: norm, rotation, threshold quantization, residual, 1-bit QJL
// sketch and bit packing of KV vectors, fused in one pass (gfx950).
//
// [admirer.cn memory-wall article, section 2, stage one]: rotate, store the
// length, quantize each rotated coordinate by threshold lookup into the
// precomputed Lloyd-Max codebook.  [Same section, stage two] and
// [intelliparadigm "3-bit" article, §2.1.2]: keys also store sign(S r) of the
// residual r, binarized as `projected > 0`.
//
// Design (one wave = 16*NT vectors per tile, 8 waves per work-group):
//  * Both products are dense 128x128 contractions, so they run on MFMA
//    (v_mfma_f32_16x16x32_bf16, fp32 accumulate).  To keep fp32-level
//    accuracy the fp32 matrices are split into bf16 hi + lo parts: bf16 inputs
//    are exact in bf16, so y = (Pi_hi + Pi_lo) x takes two passes; the residual
//    is fp32, so p = S_hi r_hi + S_lo r_hi + S_hi r_lo takes three.
//  * The matrices' rows and columns are permuted when packed (host side) so
//    that, in the MFMA register layout, lane (j, kk) -- j = lane % 16 the
//    vector, kk = lane / 16 -- loads input coordinates 32kk..32kk+31 as its B
//    operand and receives output coordinates 32kk..32kk+31 in its
//    accumulators.  Every later step (quantize, residual, second GEMM's B
//    operand, sign word, code words) then stays inside the lane: no shuffles
//    except the two xor-reductions for the norms.
//  * Quantization is exact threshold counting through a fine cell table: the
//    cell of y gives the number of thresholds surely below y and the one
//    threshold (if any) that can still lie between, plus the two centroids
//    the residual needs; one comparison finishes the count.
//  * Pi and S fragments (32 KiB per bf16 split) are staged once per
//    work-group in LDS; work-groups are persistent and grid-stride over
//    tiles; two waves per SIMD overlap one wave's loads with the other's math.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>

#include "tq_internal.h"
#include "tq_kernels.h"

namespace tq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kNT = 2;    // 16-vector MFMA column blocks per wave tile
// Waves per work-group (keys: one work-group per CU, 128 KiB of LDS for the
// Pi and S fragments; values: two per CU, 64 KiB).  Twelve-wave key groups
// (three waves per SIMD) were measured slower: their register budget of 168
// forces spills.
template <bool QJL> struct EncGeom {
  static constexpr int kWaves = 8;
  static constexpr int kThreads = 64 * kWaves;
};
constexpr int kFragU4 = static_cast<int>(kFragBytesPerSplit / 16);  // uint4 per split

__device__ __forceinline__ bf16x8 u4_as_bf16(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ bf16x2 u32_as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// (w << 1) | (the sign bit of np): with np = -p (the QJL fragments hold -S),
// that bit is [p > 0] for every p but NaN (and -0, which an accumulator started
// at +0 cannot produce), in one funnel shift.
__device__ __forceinline__ uint32_t shift_in_sign(uint32_t w, float np) {
  return __builtin_amdgcn_alignbit(w, __float_as_uint(np), 31);
}

// y - c rounded on its own, never fused with the product that formed y: the
// residual is the same in every instantiation (with and without the debug
// outputs, which keep y), so the sign bits are too.
__device__ __forceinline__ float sub_unfused(float y, float c) {
#pragma clang fp contract(off)
  return y - c;
}

// Round 8 floats to bf16 (RNE) and return hi and lo = bf16(v - hi).
// The rounded pairs are unpacked back to fp32 with a shift and a mask (the
// generic conversion would round each element a second time).
__device__ __forceinline__ void split_bf16(const f32x8 &v, bf16x8 &hi, bf16x8 &lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t hp = __builtin_convertvector((f32x2){v[2 * p], v[2 * p + 1]}, bf16x2_t);
    h[p] = __builtin_bit_cast(uint32_t, hp);
    const float b0 = __uint_as_float(h[p] << 16), b1 = __uint_as_float(h[p] & 0xffff0000u);
    const bf16x2_t lp = __builtin_convertvector((f32x2){v[2 * p] - b0, v[2 * p + 1] - b1}, bf16x2_t);
    l[p] = __builtin_bit_cast(uint32_t, lp);
  }
  hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
}


// out = the A low bits of (a1:a0) followed by the bits of (b1:b0), as four
// words (A a multiple of 16 in 16..64).
template <int A>
__device__ __forceinline__ void concat_bits(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, uint32_t (&out)[4]) {
  static_assert(A % 16 == 0 && A >= 16 && A <= 64, "A in 16..64, a multiple of 16");
  const uint64_t a = (static_cast<uint64_t>(a1) << 32) | a0, b = (static_cast<uint64_t>(b1) << 32) | b0;
  const uint64_t lo = (A == 64) ? a : (a & ((uint64_t{1} << A) - 1)) | (b << A);
  const uint64_t hi = (A == 64) ? b : (b >> (64 - A));
  out[0] = static_cast<uint32_t>(lo);
  out[1] = static_cast<uint32_t>(lo >> 32);
  out[2] = static_cast<uint32_t>(hi);
  out[3] = static_cast<uint32_t>(hi >> 32);
}

// One lane's 32 input coordinates of one vector.
template <bool XF32> struct XRegs;
template <> struct XRegs<false> { uint4 w[4]; };
template <> struct XRegs<true> { float4 w[8]; };

// Columns past the last vector (n >= 1 whenever a tile exists) read the last
// vector again: every load stays in bounds with no predication, and nothing
// computed for those columns is stored.  MFMA columns, the norm's lane
// exchange (lanes of one vector) and the emit never mix columns.
template <bool XF32, int NT>
__device__ __forceinline__ void load_x(const EncodeArgs &a, int64_t tile, int j, int kk, XRegs<XF32> (&x)[NT]) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int64_t vec = tile * (16 * NT) + nt * 16 + j;
    const int64_t row = vec < a.n ? vec : a.n - 1;
    if constexpr (!XF32) {
      const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.x) + row * a.x_stride + 32 * kk);
#pragma unroll
      for (int s = 0; s < 4; ++s) x[nt].w[s] = src[s];
    } else {
      const float4 *src = reinterpret_cast<const float4 *>(static_cast<const float *>(a.x) + row * a.x_stride + 32 * kk);
#pragma unroll
      for (int s = 0; s < 8; ++s) x[nt].w[s] = src[s];
    }
  }
}

// Cache row of input vector `vec` (-1: not written).
__device__ __forceinline__ int64_t dest_row(const EncodeArgs &a, int64_t vec, bool valid) {
  if (!valid) return -1;
  if (a.dst_row != nullptr) return a.dst_row[vec];
  if (a.append_len != nullptr) {
    const int32_t t = a.append_len[vec / a.append_heads];
    return (t >= 0 && t < a.t_cap) ? vec * a.t_cap + t : -1;
  }
  return vec;
}

// The encode of work-group `block` of `nblocks` over the rows of `a`;
// s_frag holds (QJL ? 4 : 2) fragment splits, s_qlut the cell table.
template <int BITS, bool QJL, bool XF32, bool DBG, bool SPLIT>
__device__ __forceinline__ void encode_body(const EncodeArgs &a, uint4 *s_frag, float4 *s_qlut, int block,
                                            int nblocks) {
  constexpr int NT = kNT;
  constexpr int kWaves = EncGeom<QJL>::kWaves;
  constexpr int kThreads = EncGeom<QJL>::kThreads;
#define TQ_ENC_BLOCK block
#define TQ_ENC_NBLOCKS nblocks
#include "tq_encode_body.inc"
#undef TQ_ENC_BLOCK
#undef TQ_ENC_NBLOCKS
}

template <int BITS, bool QJL, bool XF32, bool DBG, bool SPLIT>
__global__ __launch_bounds__(EncGeom<QJL>::kThreads) void encode_kernel(EncodeArgs a) {
  constexpr int NT = kNT;
  constexpr int kWaves = EncGeom<QJL>::kWaves;
  constexpr int kThreads = EncGeom<QJL>::kThreads;
  __shared__ uint4 s_frag[(QJL ? 4 : 2) * kFragU4];
  __shared__ float4 s_qlut[(SPLIT ? 2 : 1) * kQuantCellEntries];

#define TQ_ENC_BLOCK blockIdx.x
#define TQ_ENC_NBLOCKS gridDim.x
#include "tq_encode_body.inc"
#undef TQ_ENC_BLOCK
#undef TQ_ENC_NBLOCKS
}

// A decode-loop step's keys and values in one launch: work-groups
// 0 .. k_blocks - 1 encode the key rows (ka), the rest the value rows (va),
// sharing one LDS block sized for the keys' four fragment splits.  bf16 input.
template <int KBITS, bool KQJL, int VBITS>
__global__ __launch_bounds__(EncGeom<true>::kThreads) void encode_pair_kernel(EncodeArgs ka, EncodeArgs va,
                                                                              int k_blocks) {
  static_assert(EncGeom<true>::kThreads == EncGeom<false>::kThreads, "one work-group size for both");
  __shared__ uint4 s_frag[4 * kFragU4];
  __shared__ float4 s_qlut[kQuantCellEntries];
  if (static_cast<int>(blockIdx.x) < k_blocks) {
    encode_body<KBITS, KQJL, false, false, false>(ka, s_frag, s_qlut, blockIdx.x, k_blocks);
  } else {
    encode_body<VBITS, false, false, false, false>(va, s_frag, s_qlut, blockIdx.x - k_blocks, gridDim.x - k_blocks);
  }
}

// Work-groups of an encode of a.n rows.
int encode_grid(const EncodeArgs &a, bool qjl, int num_cus) {
  const int64_t tiles = (a.n + 16 * kNT - 1) / (16 * kNT);
  constexpr int kWaves = EncGeom<true>::kWaves;
  const int64_t wgs = (tiles + kWaves - 1) / kWaves;
  // Keys need the Pi and S fragments (128 KiB of LDS): one work-group per CU;
  // values need only Pi's (64 KiB) and fewer registers: two per CU.
  const int per_cu = qjl ? 1 : 2;
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(wgs, static_cast<int64_t>(num_cus) * per_cu)));
}

template <int KBITS, bool KQJL>
hipError_t launch_pair_k(const EncodeArgs &ka, const EncodeArgs &va, int vbits, int kb, int vb, hipStream_t stream) {
  const dim3 grid(kb + vb), block(EncGeom<true>::kThreads);
  switch (vbits) {
    case 1: hipLaunchKernelGGL((encode_pair_kernel<KBITS, KQJL, 1>), grid, block, 0, stream, ka, va, kb); break;
    case 2: hipLaunchKernelGGL((encode_pair_kernel<KBITS, KQJL, 2>), grid, block, 0, stream, ka, va, kb); break;
    case 3: hipLaunchKernelGGL((encode_pair_kernel<KBITS, KQJL, 3>), grid, block, 0, stream, ka, va, kb); break;
    case 4: hipLaunchKernelGGL((encode_pair_kernel<KBITS, KQJL, 4>), grid, block, 0, stream, ka, va, kb); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int BITS, bool QJL, bool XF32, bool SPLIT>
hipError_t launch_t(const EncodeArgs &a, int num_cus, hipStream_t stream) {
  const int grid = encode_grid(a, QJL, num_cus);
  if (a.dbg_rot != nullptr || a.dbg_proj != nullptr)
    hipLaunchKernelGGL((encode_kernel<BITS, QJL, XF32, true, SPLIT>), dim3(grid), dim3(EncGeom<QJL>::kThreads), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((encode_kernel<BITS, QJL, XF32, false, SPLIT>), dim3(grid), dim3(EncGeom<QJL>::kThreads), 0,
                       stream, a);
  return hipGetLastError();
}

template <int BITS, bool SPLIT>
hipError_t launch_bits(const EncodeArgs &a, bool qjl, bool x_f32, int num_cus, hipStream_t stream) {
  if (qjl)
    return x_f32 ? launch_t<BITS, true, true, SPLIT>(a, num_cus, stream)
                 : launch_t<BITS, true, false, SPLIT>(a, num_cus, stream);
  return x_f32 ? launch_t<BITS, false, true, SPLIT>(a, num_cus, stream)
               : launch_t<BITS, false, false, SPLIT>(a, num_cus, stream);
}

}  // namespace

void pack_encode_fragments(const float *mat, void *dst, bool split_rows, bool split_cols, bool negate) {
  // Element (t, s, lane, e) of a split is A[row][col] of the 16x16x32 MFMA tile
  // t, k-step s: lane % 16 picks output row enc_coord(i / 4, t, i % 4) with
  // i = lane % 16 (the coordinate that lane group i / 4 receives), element e
  // with lane / 16 picks input column enc_coord(lane / 16, 2s + e / 4, e % 4)
  // (the coordinate that lane group holds as element e of its k-step s).
  uint16_t *out = static_cast<uint16_t *>(dst);
  for (int split = 0; split < 2; ++split)
    for (int t = 0; t < 8; ++t)
      for (int s = 0; s < 4; ++s)
        for (int lane = 0; lane < 64; ++lane)
          for (int e = 0; e < 8; ++e) {
            const int i = lane & 15, kq = lane >> 4;
            const int row = enc_coord(split_rows, i >> 2, t, i & 3);
            const int col = enc_coord(split_cols, kq, 2 * s + (e >> 2), e & 3);
            const float v = negate ? -mat[row * kHeadDim + col] : mat[row * kHeadDim + col];
            const uint16_t hi = bf16_bits_rne(v);
            const uint16_t val = split == 0 ? hi : bf16_bits_rne(v - bf16_bits_to_float(hi));
            out[((((split * 8 + t) * 4 + s) * 64 + lane) * 8) + e] = val;
          }
}

bool build_quant_cells(const float *thresholds, const float *centroids, int levels, float *cells,
                       float *qscale, float *qbias) {
  // Cells of width w = 2/K over [-1, 1] (K = 256); the kernel computes
  // cell = byte(y * K/2 + K/2 - 1/2) with v_cvt_pk_u8_f32 (round to nearest
  // even, saturated to 0 .. 255, NaN -> 0): floor(y * K/2 + K/2) except where
  // y lies exactly on a cell edge, which may give the cell below.  A rotated
  // unit vector has |y| <= 1 up to rounding; larger or smaller values (a norm
  // lost to underflow) land in the end cells, which count every threshold or
  // none.  For each cell: the count of thresholds below (lo - eps), the single
  // threshold in [lo - eps, hi + eps] (NaN if none) and the centroids on
  // either side of it.  eps covers the rounding of the cell computation and
  // the edge case above; more than one candidate fails the build.
  const double w = 2.0 / kQuantCells, eps = 0.05 * w;
  const int nt = levels - 1;
  for (int i = 0; i < nt; ++i)
    if (!(std::fabs(thresholds[i]) < 1.0 - 2 * w)) return false;
  for (int k = 0; k < kQuantCellEntries; ++k) {
    const double lo = -1.0 + k * w, hi = lo + w;
    int below = 0, cand = -1, ncand = 0;
    for (int i = 0; i < nt; ++i) {
      if (thresholds[i] < lo - eps) {
        ++below;
      } else if (thresholds[i] <= hi + eps) {
        ++ncand;
        cand = i;
      }
    }
    if (ncand > 1 || (ncand == 1 && cand != below)) return false;
    uint32_t cbits = static_cast<uint32_t>(below);
    std::memcpy(&cells[4 * k], &cbits, 4);
    cells[4 * k + 1] = ncand ? thresholds[cand] : std::nanf("");
    cells[4 * k + 2] = centroids[below];
    cells[4 * k + 3] = centroids[std::min(below + 1, levels - 1)];
  }
  *qscale = static_cast<float>(kQuantCells / 2.0);
  *qbias = static_cast<float>(kQuantCells / 2.0 - 0.5);
  return true;
}

hipError_t launch_encode_pair(const EncodeArgs &ka, int kbits, bool kqjl, const EncodeArgs &va, int vbits,
                              int num_cus, hipStream_t stream) {
  if (ka.dbg_rot != nullptr || ka.dbg_proj != nullptr || va.dbg_rot != nullptr) return hipErrorInvalidValue;
  const int kb = encode_grid(ka, kqjl, num_cus), vb = encode_grid(va, false, num_cus);
  switch (kbits * 2 + (kqjl ? 1 : 0)) {
    case 2: return launch_pair_k<1, false>(ka, va, vbits, kb, vb, stream);
    case 3: return launch_pair_k<1, true>(ka, va, vbits, kb, vb, stream);
    case 4: return launch_pair_k<2, false>(ka, va, vbits, kb, vb, stream);
    case 5: return launch_pair_k<2, true>(ka, va, vbits, kb, vb, stream);
    case 6: return launch_pair_k<3, false>(ka, va, vbits, kb, vb, stream);
    case 7: return launch_pair_k<3, true>(ka, va, vbits, kb, vb, stream);
    case 8: return launch_pair_k<4, false>(ka, va, vbits, kb, vb, stream);
    case 9: return launch_pair_k<4, true>(ka, va, vbits, kb, vb, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_encode(const EncodeArgs &a, int bits, bool qjl, bool x_f32, bool split, int num_cus,
                         hipStream_t stream) {
  if (split) {
    // b' + 1 <= 4 bits on the wide coordinates
    if (a.qlut_wide == nullptr) return hipErrorInvalidValue;
    switch (bits) {
      case 1: return launch_bits<1, true>(a, qjl, x_f32, num_cus, stream);
      case 2: return launch_bits<2, true>(a, qjl, x_f32, num_cus, stream);
      case 3: return launch_bits<3, true>(a, qjl, x_f32, num_cus, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (bits) {
    case 1: return launch_bits<1, false>(a, qjl, x_f32, num_cus, stream);
    case 2: return launch_bits<2, false>(a, qjl, x_f32, num_cus, stream);
    case 3: return launch_bits<3, false>(a, qjl, x_f32, num_cus, stream);
    case 4: return launch_bits<4, false>(a, qjl, x_f32, num_cus, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tq
