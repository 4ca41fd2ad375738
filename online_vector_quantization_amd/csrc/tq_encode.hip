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

// (w << 1) | [p > 0] as one compare and one add with carry.
__device__ __forceinline__ uint32_t shift_in_positive(uint32_t w, float p) {
  uint32_t r;
  asm volatile("v_cmp_lt_f32 vcc, 0, %1\n\tv_addc_co_u32 %0, vcc, %2, %2, vcc" : "=v"(r) : "v"(p), "v"(w) : "vcc");
  return r;
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

template <int BITS, bool QJL, bool XF32, bool DBG>
__global__ __launch_bounds__(EncGeom<QJL>::kThreads) void encode_kernel(EncodeArgs a) {
  constexpr int NT = kNT;
  constexpr int kWaves = EncGeom<QJL>::kWaves;
  constexpr int kThreads = EncGeom<QJL>::kThreads;
  __shared__ uint4 s_frag[(QJL ? 4 : 2) * kFragU4];
  __shared__ float4 s_qlut[kQuantCellEntries];

  const int tid = threadIdx.x;
  for (int i = tid; i < 2 * kFragU4; i += kThreads) s_frag[i] = a.frag_rot[i];
  if constexpr (QJL) {
    for (int i = tid; i < 2 * kFragU4; i += kThreads) s_frag[2 * kFragU4 + i] = a.frag_qjl[i];
  }
  for (int i = tid; i < kQuantCellEntries; i += kThreads) s_qlut[i] = a.qlut[i];
  __syncthreads();


  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int j = lane & 15;
  // Per-lane fragment indices for the Pi and S halves of LDS, opaque to the
  // compiler: every fragment read is then one base register plus an
  // immediate offset (S's half lies beyond the 64 KiB immediate range of
  // the s_frag base, which otherwise costs a register per fragment).
  uint32_t rot_l = lane, qjl_l = lane + 2 * kFragU4;
  asm volatile("" : "+v"(rot_l), "+v"(qjl_l));
  const int kk = lane >> 4;
  const int64_t n = a.n;
  const int64_t tiles = (n + 16 * NT - 1) / (16 * NT);
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kWaves;
  const float qscale = a.qscale, qbias = a.qbias;

  for (int64_t tile = static_cast<int64_t>(blockIdx.x) * kWaves + wave; tile < tiles; tile += stride) {
    XRegs<XF32> cur[NT];
    load_x<XF32, NT>(a, tile, j, kk, cur);

    bf16x8 bx[NT][4];
    bf16x8 bxlo[XF32 ? NT : 1][4];
    float nu[NT], inv[NT];

    // ---- B operands and norms
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float ss = 0.f;
      if constexpr (!XF32) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint4 w = cur[nt].w[s];
          bx[nt][s] = u4_as_bf16(w);
          // x_i^2 summed two at a time (bf16 products are exact in fp32)
          ss = __builtin_amdgcn_fdot2_f32_bf16(u32_as_bf16x2(w.x), u32_as_bf16x2(w.x), ss, false);
          ss = __builtin_amdgcn_fdot2_f32_bf16(u32_as_bf16x2(w.y), u32_as_bf16x2(w.y), ss, false);
          ss = __builtin_amdgcn_fdot2_f32_bf16(u32_as_bf16x2(w.z), u32_as_bf16x2(w.z), ss, false);
          ss = __builtin_amdgcn_fdot2_f32_bf16(u32_as_bf16x2(w.w), u32_as_bf16x2(w.w), ss, false);
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

    int64_t vec[NT];
    bool valid[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      vec[nt] = tile * (16 * NT) + nt * 16 + j;
      valid[nt] = vec[nt] < n;
    }

    // Output block t of y = Pi x (M = output coordinate, N = vector, K = input
    // coordinate) gives the lane y[32 kk + 4 t + e] of vector vec[nt].
    auto rotate_block = [&](int t, f32x4 (&acc)[NT]) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 ah = u4_as_bf16(s_frag[rot_l + (t * 4 + s) * 64]);
        const bf16x8 al = u4_as_bf16(s_frag[rot_l + kFragU4 + (t * 4 + s) * 64]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma(ah, bx[nt][s], acc[nt]);
        if constexpr (XF32) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma(ah, bxlo[nt][s], acc[nt]);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma(al, bx[nt][s], acc[nt]);
      }
    };

    uint32_t words[NT][BITS];
    float rr[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      rr[nt] = 0.f;
#pragma unroll
      for (int w = 0; w < BITS; ++w) words[nt][w] = 0u;
    }
    // Quantize, residual and pack of block t; the residual goes to rv.
    auto quantize_block = [&](int t, f32x4 (&acc)[NT], float (&rv)[NT][4]) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float y = acc[nt][e] * inv[nt];
          // cell of y: q.x counts the thresholds below the cell; q.y is the only
          // threshold that may lie in the cell (NaN when none); q.z / q.w are the
          // centroids below / above it.
          // |y| <= 1 up to rounding gives cells 0 .. kQuantCells; the clamp only
          // matters for inputs whose norm is lost to underflow
          const uint32_t cell = min(__float2uint_rz(fmaf(y, qscale, qbias)), static_cast<uint32_t>(kQuantCellEntries - 1));
          const float4 q = s_qlut[cell];
          const bool up = y >= q.y;
          const uint32_t idx = __float_as_uint(q.x) + (up ? 1u : 0u);
          const int pos = (4 * t + e) * BITS;
          words[nt][pos / 32] |= idx << (pos % 32);
          if ((pos % 32) + BITS > 32) words[nt][pos / 32 + 1] |= idx >> (32 - (pos % 32));
          if constexpr (QJL) {
            const float r = y - (up ? q.w : q.z);
            rr[nt] = fmaf(r, r, rr[nt]);
            rv[nt][e] = r;
          }
          if constexpr (DBG) acc[nt][e] = y;
        }
        if constexpr (DBG) {
          if (a.dbg_rot != nullptr && valid[nt])
            *reinterpret_cast<float4 *>(a.dbg_rot + vec[nt] * kHeadDim + 32 * kk + 4 * t) =
                make_float4(acc[nt][0], acc[nt][1], acc[nt][2], acc[nt][3]);
        }
        // materialize the packed words now: otherwise the compiler sinks the
        // packing into the final (conditional) store and keeps every
        // coordinate's operands live until then
#pragma unroll
        for (int w = 0; w < BITS; ++w) asm volatile("" : "+v"(words[nt][w]));
        if constexpr (QJL) asm volatile("" : "+v"(rr[nt]));
      }
    };

    // QJL k-step s takes rotated coordinates 32 kk + 8 s .. + 7 of the lane,
    // i.e. blocks 2 s and 2 s + 1: their residuals, split into bf16 hi and lo.
    f32x4 pacc[QJL ? 8 : 1][NT];
    if constexpr (QJL) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) pacc[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    auto qjl_step = [&](int s, const bf16x8 (&rh)[NT], const bf16x8 (&rl)[NT]) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const bf16x8 sh = u4_as_bf16(s_frag[qjl_l + (t * 4 + s) * 64]);
        const bf16x8 sl = u4_as_bf16(s_frag[qjl_l + kFragU4 + (t * 4 + s) * 64]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) pacc[t][nt] = mfma(sh, rh[nt], pacc[t][nt]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) pacc[t][nt] = mfma(sh, rl[nt], pacc[t][nt]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) pacc[t][nt] = mfma(sl, rh[nt], pacc[t][nt]);
      }
    };

    // ---- software pipeline over the 8 output blocks: step t quantizes block t
    // (vector work) while the MFMAs of block t + 1 and, on even steps, of the
    // QJL k-step whose residual pair was completed on the step before
    // (independent of it) execute.
    f32x4 racc[2][NT];
    bf16x8 rh[QJL ? NT : 1], rl[QJL ? NT : 1];
    float rpend[QJL ? NT : 1][4];
    rotate_block(0, racc[0]);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      __builtin_amdgcn_sched_barrier(0);
      if (t < 7) rotate_block(t + 1, racc[(t + 1) & 1]);
      if constexpr (QJL) {
        if (t >= 2 && (t & 1) == 0) qjl_step(t / 2 - 1, rh, rl);
      }
      float rv[NT][4];
      quantize_block(t, racc[t & 1], rv);
      if constexpr (QJL) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if ((t & 1) == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) rpend[nt][e] = rv[nt][e];
          } else {
            const f32x8 v = {rpend[nt][0], rpend[nt][1], rpend[nt][2], rpend[nt][3], rv[nt][0], rv[nt][1], rv[nt][2], rv[nt][3]};
            split_bf16(v, rh[nt], rl[nt]);
          }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (QJL) qjl_step(3, rh, rl);

    // ---- emit codes, norms, residual norms
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int64_t row = dest_row(a, vec[nt], valid[nt]);
      const bool ok = valid[nt] && row >= 0 && row < a.cache_rows;
      if constexpr (QJL) {
        rr[nt] += __shfl_xor(rr[nt], 16);
        rr[nt] += __shfl_xor(rr[nt], 32);
      }
      if (ok) {
        uint32_t *cp = a.codes + row * (4 * BITS) + kk * BITS;
        if constexpr (BITS == 4) {
          *reinterpret_cast<uint4 *>(cp) = make_uint4(words[nt][0], words[nt][1], words[nt][2], words[nt][3]);
        } else if constexpr (BITS == 2) {
          *reinterpret_cast<uint2 *>(cp) = make_uint2(words[nt][0], words[nt][1]);
        } else {
#pragma unroll
          for (int w = 0; w < BITS; ++w) cp[w] = words[nt][w];
        }
        if (kk == 0) {
          a.norms[row] = nu[nt];
          if constexpr (QJL) a.res_norms[row] = sqrtf(rr[nt]);
        }
      }
      if constexpr (QJL) {
        // sign word bit (4 t + e) = [p > 0], built most significant bit first
        uint32_t sw = 0u;
#pragma unroll
        for (int t = 7; t >= 0; --t)
#pragma unroll
          for (int e = 3; e >= 0; --e) sw = shift_in_positive(sw, pacc[t][nt][e]);
        if constexpr (DBG) {
          if (a.dbg_proj != nullptr && valid[nt]) {
#pragma unroll
            for (int t = 0; t < 8; ++t)
              *reinterpret_cast<float4 *>(a.dbg_proj + vec[nt] * kQjlDim + 32 * kk + 4 * t) =
                  make_float4(pacc[t][nt][0], pacc[t][nt][1], pacc[t][nt][2], pacc[t][nt][3]);
          }
        }
        if (ok) a.signs[row * (kQjlDim / 32) + kk] = sw;
      }
    }
  }
}

template <int BITS, bool QJL, bool XF32>
hipError_t launch_t(const EncodeArgs &a, int num_cus, hipStream_t stream) {
  const int64_t tiles = (a.n + 16 * kNT - 1) / (16 * kNT);
  constexpr int kWaves = EncGeom<QJL>::kWaves;
  const int64_t wgs = (tiles + kWaves - 1) / kWaves;
  // Keys need the Pi and S fragments (128 KiB of LDS): one work-group per CU;
  // values need only Pi's (64 KiB) and fewer registers: two per CU.
  const int per_cu = QJL ? 1 : 2;
  const int grid = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(wgs, static_cast<int64_t>(num_cus) * per_cu)));
  if (a.dbg_rot != nullptr || a.dbg_proj != nullptr)
    hipLaunchKernelGGL((encode_kernel<BITS, QJL, XF32, true>), dim3(grid), dim3(EncGeom<QJL>::kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((encode_kernel<BITS, QJL, XF32, false>), dim3(grid), dim3(EncGeom<QJL>::kThreads), 0, stream, a);
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
  // Cells of width w = 2/K over [-1, 1]; the kernel computes
  // cell = min(uint(y * K/2 + K/2), entries - 1) (truncating, negative -> 0,
  // NaN -> 0).  A rotated unit vector has |y| <= 1 up to rounding, so cells
  // 0 .. K (K: y at or just above 1) are what occur; the guard entries past K
  // repeat the last cell.  For each cell: the count of thresholds below (lo - eps), the
  // single threshold in [lo - eps, hi + eps] (NaN if none) and the centroids
  // on either side of it.  eps covers the rounding of the cell computation;
  // more than one candidate fails the build.
  const double w = 2.0 / kQuantCells, eps = 0.05 * w;
  const int nt = levels - 1;
  for (int i = 0; i < nt; ++i)
    if (!(std::fabs(thresholds[i]) < 1.0 - 2 * w)) return false;
  for (int k = 0; k < kQuantCellEntries; ++k) {
    const double lo = -1.0 + std::min(k, kQuantCells) * w, hi = lo + w;
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
