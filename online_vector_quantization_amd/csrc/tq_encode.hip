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
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kFragU4 = static_cast<int>(kFragBytesPerSplit / 16);  // uint4 per split

__device__ __forceinline__ bf16x8 u4_as_bf16(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Round 8 floats to bf16 (RNE) and return hi and lo = bf16(v - hi).
__device__ __forceinline__ void split_bf16(const f32x8 &v, bf16x8 &hi, bf16x8 &lo) {
  hi = __builtin_convertvector(v, bf16x8);
  const f32x8 back = __builtin_convertvector(hi, f32x8);
  lo = __builtin_convertvector(v - back, bf16x8);
}

__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// One lane's 32 input coordinates of one vector.
template <bool XF32> struct XRegs;
template <> struct XRegs<false> { uint4 w[4]; };
template <> struct XRegs<true> { float4 w[8]; };

template <bool XF32, int NT>
__device__ __forceinline__ void load_x(const EncodeArgs &a, int64_t tile, int j, int kk, XRegs<XF32> (&x)[NT]) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int64_t vec = tile * (16 * NT) + nt * 16 + j;
    const bool valid = vec < a.n;
    if constexpr (!XF32) {
      const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.x) + vec * a.x_stride + 32 * kk);
#pragma unroll
      for (int s = 0; s < 4; ++s) x[nt].w[s] = valid ? src[s] : make_uint4(0, 0, 0, 0);
    } else {
      const float4 *src = reinterpret_cast<const float4 *>(static_cast<const float *>(a.x) + vec * a.x_stride + 32 * kk);
#pragma unroll
      for (int s = 0; s < 8; ++s) x[nt].w[s] = valid ? src[s] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
}

template <int BITS, bool QJL, bool XF32, int NT>
__global__ __launch_bounds__(kThreads) void encode_kernel(EncodeArgs a) {
  __shared__ uint4 s_frag[(QJL ? 4 : 2) * kFragU4];
  __shared__ float4 s_qlut[kQuantCells];

  const int tid = threadIdx.x;
  for (int i = tid; i < 2 * kFragU4; i += kThreads) s_frag[i] = a.frag_rot[i];
  if constexpr (QJL) {
    for (int i = tid; i < 2 * kFragU4; i += kThreads) s_frag[2 * kFragU4 + i] = a.frag_qjl[i];
  }
  for (int i = tid; i < kQuantCells; i += kThreads) s_qlut[i] = a.qlut[i];
  __syncthreads();

  const uint4 *rot_hi = s_frag;
  const uint4 *rot_lo = s_frag + kFragU4;
  const uint4 *qjl_hi = s_frag + 2 * kFragU4;
  const uint4 *qjl_lo = s_frag + 3 * kFragU4;

  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int j = lane & 15;
  const int kk = lane >> 4;
  const int64_t n = a.n;
  const int64_t tiles = (n + 16 * NT - 1) / (16 * NT);
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kWaves;
  const float qscale = a.qscale, qbias = a.qbias;

  for (int64_t tile = static_cast<int64_t>(blockIdx.x) * kWaves + wave; tile < tiles; tile += stride) {
    XRegs<XF32> cur[NT];
    load_x<XF32, NT>(a, tile, j, kk, cur);

    int64_t vec[NT];
    bool valid[NT];
    bf16x8 bx[NT][4];
    bf16x8 bxlo[NT][4];
    float nu[NT], inv[NT];

    // ---- B operands and norms
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      vec[nt] = tile * (16 * NT) + nt * 16 + j;
      valid[nt] = vec[nt] < n;
      float ss = 0.f;
      if constexpr (!XF32) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint4 w = cur[nt].w[s];
          bx[nt][s] = u4_as_bf16(w);
          const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const float v0 = bf16lo_to_f32(ws[h]);
            const float v1 = bf16hi_to_f32(ws[h]);
            ss = fmaf(v0, v0, ss);
            ss = fmaf(v1, v1, ss);
          }
        }
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float4 p0 = cur[nt].w[2 * s], p1 = cur[nt].w[2 * s + 1];
          const f32x8 v = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
          split_bf16(v, bx[nt][s], bxlo[nt][s]);
        }
      }
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      nu[nt] = sqrtf(ss);
      inv[nt] = (nu[nt] == 0.f) ? 0.f : 1.f / nu[nt];
    }

    // ---- y = Pi x (M = output coordinate, N = vector, K = input coordinate);
    // consecutive MFMAs always target different accumulators.
    f32x4 acc[NT][8];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[nt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // keep the scheduler from hoisting every fragment load of the tile
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const bf16x8 ah = u4_as_bf16(rot_hi[(t * 4 + s) * 64 + lane]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt][t] = mfma(ah, bx[nt][s], acc[nt][t]);
        if constexpr (XF32) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[nt][t] = mfma(ah, bxlo[nt][s], acc[nt][t]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const bf16x8 al = u4_as_bf16(rot_lo[(t * 4 + s) * 64 + lane]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt][t] = mfma(al, bx[nt][s], acc[nt][t]);
      }
    }

    __builtin_amdgcn_sched_barrier(0);
    // ---- quantize, residual, pack (lane holds y[32kk + 4t + e] of vector vec[nt])
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      uint32_t words[BITS];
#pragma unroll
      for (int w = 0; w < BITS; ++w) words[w] = 0u;
      float rr = 0.f;
      const bool dbg = a.dbg_rot != nullptr && valid[nt];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        float yv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float y = acc[nt][t][e] * inv[nt];
          yv[e] = y;
          // cell of y: thresholds below the cell are counted in q.x; q.y is the
          // only threshold that may lie in the cell (NaN when none); q.z / q.w
          // are the centroids below / above it.
          const int cell = min(max(static_cast<int>(fmaf(y, qscale, qbias)), 0), kQuantCells - 1);
          const float4 q = s_qlut[cell];
          const bool up = y >= q.y;
          const uint32_t idx = __float_as_uint(q.x) + (up ? 1u : 0u);
          const int pos = (4 * t + e) * BITS;
          words[pos / 32] |= idx << (pos % 32);
          if ((pos % 32) + BITS > 32) words[pos / 32 + 1] |= idx >> (32 - (pos % 32));
          if constexpr (QJL) {
            const float r = y - (up ? q.w : q.z);
            rr = fmaf(r, r, rr);
            acc[nt][t][e] = r;   // keep the residual in place of y
          }
        }
        if (dbg)
          *reinterpret_cast<float4 *>(a.dbg_rot + vec[nt] * kHeadDim + 32 * kk + 4 * t) =
              make_float4(yv[0], yv[1], yv[2], yv[3]);
      }
      int64_t row = vec[nt];
      if (a.dst_row != nullptr) row = valid[nt] ? a.dst_row[vec[nt]] : -1;
      const bool ok = valid[nt] && row >= 0 && row < a.cache_rows;
      if (ok) {
        uint32_t *cp = a.codes + row * (4 * BITS) + kk * BITS;
        if constexpr (BITS == 4) {
          *reinterpret_cast<uint4 *>(cp) = make_uint4(words[0], words[1], words[2], words[3]);
        } else if constexpr (BITS == 2) {
          *reinterpret_cast<uint2 *>(cp) = make_uint2(words[0], words[1]);
        } else {
#pragma unroll
          for (int w = 0; w < BITS; ++w) cp[w] = words[w];
        }
      }
      if constexpr (QJL) {
        rr += __shfl_xor(rr, 16);
        rr += __shfl_xor(rr, 32);
        if (ok && kk == 0) a.res_norms[row] = sqrtf(rr);
      }
      if (ok && kk == 0) a.norms[row] = nu[nt];
    }

    if constexpr (QJL) {
      // ---- p = S r (M = projection index, N = vector, K = rotated coordinate)
      f32x4 accp[NT][8];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int t = 0; t < 8; ++t) accp[nt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 rh[NT], rl[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const f32x8 v = {acc[nt][2 * s][0],     acc[nt][2 * s][1],     acc[nt][2 * s][2],
                           acc[nt][2 * s][3],     acc[nt][2 * s + 1][0], acc[nt][2 * s + 1][1],
                           acc[nt][2 * s + 1][2], acc[nt][2 * s + 1][3]};
          split_bf16(v, rh[nt], rl[nt]);
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const bf16x8 ah = u4_as_bf16(qjl_hi[(t * 4 + s) * 64 + lane]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) accp[nt][t] = mfma(ah, rh[nt], accp[nt][t]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) accp[nt][t] = mfma(ah, rl[nt], accp[nt][t]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const bf16x8 al = u4_as_bf16(qjl_lo[(t * 4 + s) * 64 + lane]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) accp[nt][t] = mfma(al, rh[nt], accp[nt][t]);
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        // sign word: bit (4t + e) = [p > 0]; built most significant bit first
        uint32_t sw = 0u;
#pragma unroll
        for (int t = 7; t >= 0; --t)
#pragma unroll
          for (int e = 3; e >= 0; --e) sw = (sw << 1) | (accp[nt][t][e] > 0.f ? 1u : 0u);
        if (a.dbg_proj != nullptr && valid[nt]) {
#pragma unroll
          for (int t = 0; t < 8; ++t)
            *reinterpret_cast<float4 *>(a.dbg_proj + vec[nt] * kQjlDim + 32 * kk + 4 * t) =
                make_float4(accp[nt][t][0], accp[nt][t][1], accp[nt][t][2], accp[nt][t][3]);
        }
        int64_t row = vec[nt];
        if (a.dst_row != nullptr) row = valid[nt] ? a.dst_row[vec[nt]] : -1;
        if (valid[nt] && row >= 0 && row < a.cache_rows) a.signs[row * (kQjlDim / 32) + kk] = sw;
      }
    }
  }
}

template <int BITS, bool QJL, bool XF32>
hipError_t launch_t(const EncodeArgs &a, int num_cus, hipStream_t stream) {
  constexpr int NT = 2;
  const int64_t tiles = (a.n + 16 * NT - 1) / (16 * NT);
  const int64_t wgs = (tiles + kWaves - 1) / kWaves;
  const int grid = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(wgs, num_cus)));
  hipLaunchKernelGGL((encode_kernel<BITS, QJL, XF32, NT>), dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_bits(const EncodeArgs &a, bool qjl, bool x_f32, int num_cus, hipStream_t stream) {
  if (qjl) return x_f32 ? launch_t<BITS, true, true>(a, num_cus, stream) : launch_t<BITS, true, false>(a, num_cus, stream);
  return x_f32 ? launch_t<BITS, false, true>(a, num_cus, stream) : launch_t<BITS, false, false>(a, num_cus, stream);
}

}  // namespace

void pack_encode_fragments(const float *mat, void *dst) {
  // Element (t, s, lane, e) of a split is A[row][col] of the 16x16x32 MFMA tile
  // t, k-step s: lane % 16 picks output row 32*((lane%16)/4) + 4t + (lane%4),
  // element e with lane / 16 picks input column 32*(lane/16) + 8s + e.
  uint16_t *out = static_cast<uint16_t *>(dst);
  for (int split = 0; split < 2; ++split)
    for (int t = 0; t < 8; ++t)
      for (int s = 0; s < 4; ++s)
        for (int lane = 0; lane < 64; ++lane)
          for (int e = 0; e < 8; ++e) {
            const int i = lane & 15, kq = lane >> 4;
            const int row = 32 * (i >> 2) + 4 * t + (i & 3);
            const int col = 32 * kq + 8 * s + e;
            const float v = mat[row * kHeadDim + col];
            const uint16_t hi = bf16_bits_rne(v);
            const uint16_t val = split == 0 ? hi : bf16_bits_rne(v - bf16_bits_to_float(hi));
            out[((((split * 8 + t) * 4 + s) * 64 + lane) * 8) + e] = val;
          }
}

bool build_quant_cells(const float *thresholds, const float *centroids, int levels, float *cells,
                       float *qscale, float *qbias) {
  // Cells of width w over [-Y, Y) with Y = 0.5; the kernel computes
  // cell = clamp(int(y * K/(2Y) + K/2), 0, K-1).  For each cell: the count of
  // thresholds below (lo - eps), the single threshold in [lo - eps, hi + eps]
  // (NaN if none) and the centroids on either side of it.  eps covers the
  // rounding of the cell computation; more than one candidate fails the build.
  const double Y = 0.5, w = 2.0 * Y / kQuantCells, eps = 0.05 * w;
  const int nt = levels - 1;
  for (int i = 0; i < nt; ++i)
    if (!(std::fabs(thresholds[i]) < Y - 2 * w)) return false;
  for (int k = 0; k < kQuantCells; ++k) {
    const double lo = -Y + k * w, hi = lo + w;
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
  *qscale = static_cast<float>(kQuantCells / (2.0 * Y));
  *qbias = static_cast<float>(kQuantCells / 2.0);
  return true;
}

hipError_t launch_encode(const EncodeArgs &a, int bits, bool qjl, bool x_f32, int num_cus,
                         hipStream_t stream) {
  switch (bits) {
    case 1: return launch_bits<1>(a, qjl, x_f32, num_cus, stream);
    case 2: return launch_bits<2>(a, qjl, x_f32, num_cus, stream);
    case 3: return launch_bits<3>(a, qjl, x_f32, num_cus, stream);
    case 4: return launch_bits<4>(a, qjl, x_f32, num_cus, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tq
