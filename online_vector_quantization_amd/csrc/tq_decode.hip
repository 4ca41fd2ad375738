// Decode-attention kernels over the compressed KV cache (gfx950, no MFMA).
//
// [cc-newplayer explainer, technical breakdown item 4]: Q is not compressed;
// attention runs over the compressed K and V with dequantization.
// [Same page, item 2]: rotation preserves inner products, so the query is
// rotated once (q~ = Pi q) instead of un-rotating every key, and the values
// are summed in the rotated domain and rotated back once at the end.
// [admirer.cn memory-wall article, section 2, stage two] and
// [intelliparadigm "3-bit" article, §2.1.2 and §2.2]: the 1-bit QJL sketch
// corrects the key inner product without bias:
//     <q~, r> ~ sqrt(pi/2)/m * gamma * <S q~, 2z - 1>.
// [same memory-wall article, section 1]: decode is memory-bound, so the kernel
// streams the packed codes once and keeps everything else on chip.
//
// Three launches on the caller's stream:
//  1. qprep:   per (b, q head): q~ = Pi_k q and s = S q~ into the workspace.
//  2. partial: per (b, kv head, token chunk): scores of the chunk's tokens for
//              the g q heads of that kv head, chunk-local softmax statistics
//              (max, sum) and the rotated-domain value sum.
//  3. combine: per (b, q head): log-sum-exp merge of the chunks, o = Pi_v^T o~,
//              write fp32 or bf16.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "tq_kernels.h"

namespace tq {
namespace {

constexpr int D = kHeadDim;
constexpr int kTile = 256;          // tokens scored per pass (one per thread)
constexpr int kPartThreads = 256;
constexpr int kMaxG = 16;

__device__ __forceinline__ float load_q(const void *q, int q_bf16, int64_t idx) {
  if (q_bf16) {
    const uint16_t b = static_cast<const uint16_t *>(q)[idx];
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
  }
  return static_cast<const float *>(q)[idx];
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// ---------------------------------------------------------------- 1. qprep
__global__ __launch_bounds__(D) void qprep_kernel(DecodeArgs a) {
  __shared__ float s_q[D];
  __shared__ float s_qr[D];
  const int bh = blockIdx.x;
  const int i = threadIdx.x;
  const int m = a.qjl_m;
  s_q[i] = load_q(a.q, a.q_bf16, static_cast<int64_t>(bh) * D + i);
  __syncthreads();
  // q~_i = sum_j Pi[i][j] q_j, reading Pi^T row-major so threads stay coalesced.
  float acc = 0.f;
  for (int jj = 0; jj < D; ++jj) acc = fmaf(a.rot_k_t[jj * D + i], s_q[jj], acc);
  s_qr[i] = acc;
  float *dst = a.ws_qprep + static_cast<int64_t>(bh) * (D + m);
  dst[i] = acc;
  __syncthreads();
  for (int r = i; r < m; r += D) {
    float sacc = 0.f;
    for (int jj = 0; jj < D; ++jj) sacc = fmaf(a.qjl_t[jj * m + r], s_qr[jj], sacc);
    dst[D + r] = sacc;
  }
}

// ---------------------------------------------------------------- 2. partial
template <int KB, int VB, bool QJL, int G>
__global__ __launch_bounds__(kPartThreads) void partial_kernel(DecodeArgs a) {
  constexpr int KW = D * KB / 32;   // key code words per token
  constexpr int VW = D * VB / 32;   // value code words per token
  constexpr int M = QJL ? kQjlDim : 0;
  __shared__ float s_q[G][D];
  __shared__ float s_s[G][QJL ? kQjlDim : 1];
  __shared__ float s_p[G][kTile];
  __shared__ float s_ck[kMaxLevels], s_cv[kMaxLevels];
  __shared__ float s_run_m[G], s_run_l[G], s_alpha[G];
  __shared__ float s_red[2][G][D];

  const int chunk_id = blockIdx.x;
  const int hk = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int hq0 = hk * G;

  int T = a.seq_len[b];
  T = T < 0 ? 0 : (T > a.t_cap ? static_cast<int>(a.t_cap) : T);
  const int t_begin = chunk_id * a.chunk;
  const int t_end = min(T, t_begin + a.chunk);

  for (int i = tid; i < G * D; i += kPartThreads) {
    const int h = i / D, jj = i % D;
    s_q[h][jj] = a.ws_qprep[static_cast<int64_t>(b * a.n_q_heads + hq0 + h) * (D + M) + jj];
  }
  if constexpr (QJL) {
    for (int i = tid; i < G * M; i += kPartThreads) {
      const int h = i / M, r = i % M;
      s_s[h][r] = a.ws_qprep[static_cast<int64_t>(b * a.n_q_heads + hq0 + h) * (D + M) + D + r];
    }
  }
  if (tid < kMaxLevels) {
    s_ck[tid] = a.k_centroids[tid];
    s_cv[tid] = a.v_centroids[tid];
  }
  if (tid < G) {
    s_run_m[tid] = -INFINITY;
    s_run_l[tid] = 0.f;
  }
  __syncthreads();

  const int64_t row0 = (static_cast<int64_t>(b) * a.n_kv_heads + hk) * a.t_cap;
  const int jv = tid & (D - 1);      // value coordinate owned in the V phase
  const int half = tid >> 7;         // which parity of tokens
  float acc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) acc[h] = 0.f;

  for (int tb = t_begin; tb < t_end; tb += kTile) {
    const int n_tok = min(kTile, t_end - tb);
    // ---- scores: one token per thread
    {
      const int t = tb + tid;
      float l[G];
      if (tid < n_tok) {
        const int64_t row = row0 + t;
        const uint32_t *kc = a.k_codes + row * KW;
        float dot[G];
#pragma unroll
        for (int h = 0; h < G; ++h) dot[h] = 0.f;
#pragma unroll
        for (int w = 0; w < KW; ++w) {
          const uint32_t word = kc[w];
          const uint32_t next = (w + 1 < KW) ? kc[w + 1] : 0u;
          // coordinates whose first bit lies in this word
          const int c_first = (w * 32 + KB - 1) / KB;
          const int c_last = min(D - 1, (w * 32 + 31) / KB);
          for (int c = c_first; c <= c_last; ++c) {
            const int bit = c * KB - w * 32;
            uint32_t code = word >> bit;
            if (bit + KB > 32) code |= next << (32 - bit);
            code &= (1u << KB) - 1u;
            const float cv = s_ck[code];
#pragma unroll
            for (int h = 0; h < G; ++h) dot[h] = fmaf(s_q[h][c], cv, dot[h]);
          }
        }
        const float nu = a.k_norms[row];
        if constexpr (QJL) {
          const uint32_t *ks = a.k_signs + row * (M / 32);
          float sd[G];
#pragma unroll
          for (int h = 0; h < G; ++h) sd[h] = 0.f;
          for (int w = 0; w < M / 32; ++w) {
            const uint32_t word = ks[w];
            for (int i = 0; i < 32; ++i) {
              const float sg = ((word >> i) & 1u) ? 1.f : -1.f;
#pragma unroll
              for (int h = 0; h < G; ++h) sd[h] = fmaf(s_s[h][w * 32 + i], sg, sd[h]);
            }
          }
          const float gq = a.qjl_coef * a.k_res[row];
#pragma unroll
          for (int h = 0; h < G; ++h) dot[h] = fmaf(gq, sd[h], dot[h]);
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          l[h] = a.scale * nu * dot[h];
          if (a.dbg_scores != nullptr)
            a.dbg_scores[(static_cast<int64_t>(b) * a.n_q_heads + hq0 + h) * a.t_cap + t] = l[h];
        }
      } else {
#pragma unroll
        for (int h = 0; h < G; ++h) l[h] = -INFINITY;
      }
#pragma unroll
      for (int h = 0; h < G; ++h) s_p[h][tid] = l[h];
    }
    __syncthreads();
    // ---- tile max and running rescale (wave w handles heads w, w+4, ...)
    {
      const int lane = tid & 63, wave = tid >> 6;
      for (int h = wave; h < G; h += kPartThreads / 64) {
        float mx = fmaxf(fmaxf(s_p[h][lane], s_p[h][lane + 64]), fmaxf(s_p[h][lane + 128], s_p[h][lane + 192]));
        for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        const float m_old = s_run_m[h];
        const float m_new = fmaxf(m_old, mx);
        float sum = 0.f;
        for (int k = lane; k < kTile; k += 64) {
          const float p = (k < n_tok) ? __expf(s_p[h][k] - m_new) : 0.f;
          s_p[h][k] = p;
          sum += p;
        }
        for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
        if (lane == 0) {
          const float alpha = (m_old == -INFINITY) ? 0.f : __expf(m_old - m_new);
          s_alpha[h] = alpha;
          s_run_l[h] = s_run_l[h] * alpha + sum;
          s_run_m[h] = m_new;
        }
      }
    }
    __syncthreads();
    // ---- rotated-domain value sum: thread owns coordinate jv, tokens of parity `half`
    {
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] *= s_alpha[h];
      const int wsel = (jv * VB) / 32;
      const int bit = (jv * VB) % 32;
      for (int k = half; k < n_tok; k += 2) {
        const int64_t row = row0 + tb + k;
        const uint32_t *vc = a.v_codes + row * VW;
        uint32_t code = vc[wsel] >> bit;
        if (bit + VB > 32) code |= vc[wsel + 1] << (32 - bit);
        code &= (1u << VB) - 1u;
        const float val = s_cv[code] * a.v_norms[row];
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h] = fmaf(s_p[h][k], val, acc[h]);
      }
    }
    __syncthreads();
  }

  // ---- merge the two token parities and write the chunk's partials
#pragma unroll
  for (int h = 0; h < G; ++h) s_red[half][h][jv] = acc[h];
  __syncthreads();
  for (int i = tid; i < G * D; i += kPartThreads) {
    const int h = i / D, jj = i % D;
    const int64_t bh = static_cast<int64_t>(b) * a.n_q_heads + hq0 + h;
    a.ws_part_o[(bh * a.n_chunks + chunk_id) * D + jj] = s_red[0][h][jj] + s_red[1][h][jj];
  }
  if (tid < G) {
    const int64_t bh = static_cast<int64_t>(b) * a.n_q_heads + hq0 + tid;
    a.ws_part_ml[(bh * a.n_chunks + chunk_id) * 2 + 0] = s_run_m[tid];
    a.ws_part_ml[(bh * a.n_chunks + chunk_id) * 2 + 1] = s_run_l[tid];
  }
}

// ---------------------------------------------------------------- 3. combine
__global__ __launch_bounds__(D) void combine_kernel(DecodeArgs a) {
  __shared__ float s_o[D];
  __shared__ float s_w[1024];
  __shared__ float s_scal[2];
  const int bh = blockIdx.x;
  const int i = threadIdx.x;
  const int nc = a.n_chunks;
  const float *ml = a.ws_part_ml + static_cast<int64_t>(bh) * nc * 2;
  if (i == 0) {
    float mx = -INFINITY;
    for (int c = 0; c < nc; ++c)
      if (ml[2 * c + 1] > 0.f) mx = fmaxf(mx, ml[2 * c]);
    float tot = 0.f;
    for (int c = 0; c < nc; ++c) {
      const float w = (ml[2 * c + 1] > 0.f) ? __expf(ml[2 * c] - mx) : 0.f;
      if (c < 1024) s_w[c] = w;
      tot += w * ml[2 * c + 1];
    }
    s_scal[0] = tot;
  }
  __syncthreads();
  const float tot = s_scal[0];
  float o = 0.f;
  const float *po = a.ws_part_o + static_cast<int64_t>(bh) * nc * D;
  for (int c = 0; c < nc; ++c) {
    const float w = s_w[c];
    if (w != 0.f) o = fmaf(w, po[c * D + i], o);
  }
  s_o[i] = (tot > 0.f) ? o / tot : 0.f;
  __syncthreads();
  // o = Pi_v^T o~ : out_i = sum_j Pi_v[j][i] o~_j
  float r = 0.f;
  for (int jj = 0; jj < D; ++jj) r = fmaf(a.rot_v[jj * D + i], s_o[jj], r);
  if (a.out_bf16) {
    static_cast<uint16_t *>(a.out)[static_cast<int64_t>(bh) * D + i] = f32_to_bf16_rne(r);
  } else {
    static_cast<float *>(a.out)[static_cast<int64_t>(bh) * D + i] = r;
  }
}

template <int KB, int VB, bool QJL>
hipError_t launch_partial_g(const DecodeArgs &a, int g, dim3 grid, hipStream_t stream) {
  switch (g) {
#define TQ_G(GG) \
  case GG: hipLaunchKernelGGL((partial_kernel<KB, VB, QJL, GG>), grid, dim3(kPartThreads), 0, stream, a); break;
    TQ_G(1) TQ_G(2) TQ_G(4) TQ_G(8) TQ_G(16)
#undef TQ_G
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KB, int VB>
hipError_t launch_partial_q(const DecodeArgs &a, int g, dim3 grid, hipStream_t stream) {
  return a.qjl_m > 0 ? launch_partial_g<KB, VB, true>(a, g, grid, stream)
                     : launch_partial_g<KB, VB, false>(a, g, grid, stream);
}

template <int KB>
hipError_t launch_partial_v(const DecodeArgs &a, int g, dim3 grid, hipStream_t stream) {
  switch (a.v_bits) {
    case 1: return launch_partial_q<KB, 1>(a, g, grid, stream);
    case 2: return launch_partial_q<KB, 2>(a, g, grid, stream);
    case 3: return launch_partial_q<KB, 3>(a, g, grid, stream);
    case 4: return launch_partial_q<KB, 4>(a, g, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

DecodePlan plan_decode(int batch, int n_q_heads, int n_kv_heads, int64_t t_cap) {
  // Aim at ~1024 work-groups over (b, kv head, chunk); chunks are multiples of
  // the 256-token tile.
  DecodePlan p{};
  const int64_t rows = static_cast<int64_t>(batch) * n_kv_heads;
  const int64_t max_chunks = std::max<int64_t>(1, (t_cap + kTile - 1) / kTile);
  int64_t want = std::max<int64_t>(1, (1024 + rows - 1) / std::max<int64_t>(1, rows));
  want = std::min(want, max_chunks);
  int64_t chunk = (t_cap + want - 1) / want;
  chunk = std::max<int64_t>(kTile, ((chunk + kTile - 1) / kTile) * kTile);
  p.chunk = static_cast<int>(chunk);
  p.n_chunks = static_cast<int>(std::max<int64_t>(1, (t_cap + chunk - 1) / chunk));
  const int64_t bh = static_cast<int64_t>(batch) * n_q_heads;
  auto align = [](size_t v) { return (v + 255) & ~static_cast<size_t>(255); };
  p.off_qprep = 0;
  p.off_part_o = align(p.off_qprep + static_cast<size_t>(bh) * (D + kQjlDim) * sizeof(float));
  p.off_part_ml = align(p.off_part_o + static_cast<size_t>(bh) * p.n_chunks * D * sizeof(float));
  p.total_bytes = align(p.off_part_ml + static_cast<size_t>(bh) * p.n_chunks * 2 * sizeof(float));
  return p;
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
  const int g = a.n_q_heads / a.n_kv_heads;
  if (a.n_chunks > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(qprep_kernel, dim3(a.batch * a.n_q_heads), dim3(D), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(a.n_chunks, a.n_kv_heads, a.batch);
  switch (a.k_bits) {
    case 1: e = launch_partial_v<1>(a, g, grid, stream); break;
    case 2: e = launch_partial_v<2>(a, g, grid, stream); break;
    case 3: e = launch_partial_v<3>(a, g, grid, stream); break;
    case 4: e = launch_partial_v<4>(a, g, grid, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(combine_kernel, dim3(a.batch * a.n_q_heads), dim3(D), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tq
