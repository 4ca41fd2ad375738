// Encode kernel: norm, rotation, threshold quantization, residual, 1-bit QJL
// sketch and bit packing of KV vectors, fused in one pass (gfx950).
//
// [admirer.cn memory-wall article, section 2, stage one]: rotate, store the
// length, quantize each rotated coordinate by threshold lookup into the
// precomputed Lloyd-Max codebook.  [Same section, stage two] and
// [intelliparadigm "3-bit" article, §2.1.2]: keys also store sign(S r) of the
// residual r, binarized as `projected > 0`.
//
// Design (one wave = 16*NT vectors per tile):
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
//  * Pi and S fragments (32 KiB per bf16 split) are staged once per
//    work-group in LDS; work-groups are persistent and grid-stride over tiles.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>

#include "tq_internal.h"
#include "tq_kernels.h"

namespace tq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
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

template <int BITS, bool QJL, bool XF32, int NT>
__global__ __launch_bounds__(kThreads) void encode_kernel(EncodeArgs a) {
  constexpr int L = 1 << BITS;
  __shared__ uint4 s_frag[(QJL ? 4 : 2) * kFragU4];
  __shared__ float s_cent[kMaxLevels];

  const int tid = threadIdx.x;
  for (int i = tid; i < 2 * kFragU4; i += kThreads) s_frag[i] = a.frag_rot[i];
  if constexpr (QJL) {
    for (int i = tid; i < 2 * kFragU4; i += kThreads) s_frag[2 * kFragU4 + i] = a.frag_qjl[i];
  }
  if (tid < kMaxLevels) s_cent[tid] = a.centroids[tid];
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

  for (int64_t tile = static_cast<int64_t>(blockIdx.x) * kWaves + wave; tile < tiles;
       tile += static_cast<int64_t>(gridDim.x) * kWaves) {
    int64_t vec[NT];
    bool valid[NT];
    bf16x8 bx[NT][4];
    bf16x8 bxlo[NT][4];
    float nu[NT], inv[NT];

    // ---- load 32 consecutive coordinates of one vector per lane; norms
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      vec[nt] = tile * (16 * NT) + nt * 16 + j;
      valid[nt] = vec[nt] < n;
      float ss = 0.f;
      if constexpr (!XF32) {
        const uint4 *src = reinterpret_cast<const uint4 *>(
            static_cast<const uint16_t *>(a.x) + vec[nt] * a.x_stride + 32 * kk);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          uint4 w = valid[nt] ? src[s] : make_uint4(0, 0, 0, 0);
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
        const float4 *src = reinterpret_cast<const float4 *>(
            static_cast<const float *>(a.x) + vec[nt] * a.x_stride + 32 * kk);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          float4 p0 = valid[nt] ? src[2 * s] : make_float4(0.f, 0.f, 0.f, 0.f);
          float4 p1 = valid[nt] ? src[2 * s + 1] : make_float4(0.f, 0.f, 0.f, 0.f);
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

    // ---- y = Pi x (M = output coordinate, N = vector, K = input coordinate)
    f32x4 acc[NT][8];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[nt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const bf16x8 ah = u4_as_bf16(rot_hi[(t * 4 + s) * 64 + lane]);
        const bf16x8 al = u4_as_bf16(rot_lo[(t * 4 + s) * 64 + lane]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          acc[nt][t] = mfma(ah, bx[nt][s], acc[nt][t]);
          acc[nt][t] = mfma(al, bx[nt][s], acc[nt][t]);
          if constexpr (XF32) acc[nt][t] = mfma(ah, bxlo[nt][s], acc[nt][t]);
        }
      }
    }

#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      // lane holds y[32kk + 4t + e] of vector vec[nt] in acc[nt][t][e]
      uint32_t words[BITS];
#pragma unroll
      for (int w = 0; w < BITS; ++w) words[w] = 0u;
      float rr = 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float y = acc[nt][t][e] * inv[nt];
          uint32_t idx = 0;
#pragma unroll
          for (int i = 0; i < L - 1; ++i) idx += (y >= a.thresholds[i]) ? 1u : 0u;
          const int pos = (4 * t + e) * BITS;
          words[pos / 32] |= idx << (pos % 32);
          if ((pos % 32) + BITS > 32) words[pos / 32 + 1] |= idx >> (32 - (pos % 32));
          if constexpr (QJL) {
            const float r = y - s_cent[idx];
            rr = fmaf(r, r, rr);
            acc[nt][t][e] = r;   // keep the residual in place of y
          } else {
            acc[nt][t][e] = y;
          }
          if (a.dbg_rot != nullptr && valid[nt]) a.dbg_rot[vec[nt] * kHeadDim + 32 * kk + 4 * t + e] = y;
        }
      }
      int64_t row = vec[nt];
      if (a.dst_row != nullptr) row = valid[nt] ? a.dst_row[vec[nt]] : -1;
      const bool ok = valid[nt] && row >= 0 && row < a.cache_rows;
      if (ok) {
        uint32_t *cp = a.codes + row * (4 * BITS) + kk * BITS;
#pragma unroll
        for (int w = 0; w < BITS; ++w) cp[w] = words[w];
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
      bf16x8 rh[NT][4], rl[NT][4];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const f32x8 v = {acc[nt][2 * s][0],     acc[nt][2 * s][1],     acc[nt][2 * s][2],
                           acc[nt][2 * s][3],     acc[nt][2 * s + 1][0], acc[nt][2 * s + 1][1],
                           acc[nt][2 * s + 1][2], acc[nt][2 * s + 1][3]};
          split_bf16(v, rh[nt][s], rl[nt][s]);
        }
      f32x4 accp[NT][8];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int t = 0; t < 8; ++t) accp[nt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const bf16x8 ah = u4_as_bf16(qjl_hi[(t * 4 + s) * 64 + lane]);
          const bf16x8 al = u4_as_bf16(qjl_lo[(t * 4 + s) * 64 + lane]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            accp[nt][t] = mfma(ah, rh[nt][s], accp[nt][t]);
            accp[nt][t] = mfma(al, rh[nt][s], accp[nt][t]);
            accp[nt][t] = mfma(ah, rl[nt][s], accp[nt][t]);
          }
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        uint32_t sw = 0u;
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p = accp[nt][t][e];
            sw |= (p > 0.f ? 1u : 0u) << (4 * t + e);
            if (a.dbg_proj != nullptr && valid[nt])
              a.dbg_proj[vec[nt] * kQjlDim + 32 * kk + 4 * t + e] = p;
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
  const int per_cu = QJL ? 1 : 2;
  const int grid = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(wgs, static_cast<int64_t>(num_cus) * per_cu)));
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
