// Decode attention over the compressed KV cache (gfx950, no MFMA): a main
// kernel over (batch, kv head, token chunk) and a small combine kernel.
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
// Work-group = (batch b, kv head, chunk of tokens), 8 waves:
//  0. prologue: q~ = Pi_k q and s = S q~ for the g q heads of this kv head
//     (parallel partial dot products reduced in LDS); q~, s go to a per-group
//     workspace slot so that the main loop can read them as scalar (uniform)
//     operands; a nibble table of signed partial sums of s, a key
//     dequantization table and a value pair table are built in LDS.
//  1. each wave, per 64-token tile:
//     * scores, one token per lane: key codes dequantized through the LDS
//       table (one lookup per code byte) times q~ from scalar registers; the
//       sign term is a sum of nibble-table lookups;
//     * online softmax (running max and sum per head);
//     * value sum, two rotated coordinates per lane: the tile's value records
//       are staged in LDS, each token's weight is broadcast with readlane and a
//       pair table dequantizes two codes at once.
//  2. the waves merge; the chunk's (max, sum, rotated output) go to the
//     workspace.
// A second, small launch merges the chunks of each (b, q head) (log-sum-exp),
// applies Pi_v^T and writes the output.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "tq_kernels.h"

namespace tq {
namespace {

constexpr int D = kHeadDim;
// Waves per work-group (8: each wave usually gets several 64-token tiles,
// which amortizes the per-wave prologue and merge).
template <int G> struct Geom {
  static constexpr int kWaves = 8;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kParts = kThreads / 128;    // prologue split of the d-long dot products
};
constexpr int kSignLut = 32 * 16;       // floats per q head: 32 nibble positions x 16
constexpr int kRecStride = 20;          // staged value record: up to 16 words, a zero pad word, 16-B rows
constexpr int kQSlot = D + kQjlDim;     // floats per q head in a workspace slot

typedef const float __attribute__((address_space(4))) *uniform_fptr;

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

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Key dequantization table per lookup:
//   KB=1: a nibble (4 codes) -> float4, 16 entries
//   KB=2: a byte (4 codes)   -> float4, 256 entries
//   KB=3: 6 bits (2 codes)   -> float2, 64 entries
//   KB=4: a byte (2 codes)   -> float2, 256 entries
template <int KB> struct KeyLut {
  static constexpr int kBitsPerLookup = key_lut_bits(KB);
  static constexpr int kCoords = key_lut_coords(KB);
  static constexpr int kEntries = 1 << kBitsPerLookup;
  static constexpr int kLookups = D / kCoords;
};

// One lane's token record of a 64-token tile.  The key part of the next tile
// is loaded one tile ahead; the value part at the top of its own tile, so its
// latency hides behind the key work.
template <int KW> struct KeyRegs {
  uint4 kc[KW / 4];   // key code words
  uint4 sg;           // key sign words
  float nu, gamma;
};
struct ValRegs {
  uint4 vc[4];        // value code words (first VW/4 used)
  float nu_v;
};

template <int KW, bool QJL>
__device__ __forceinline__ KeyRegs<KW> load_keys(const DecodeArgs &a, int64_t row) {
  KeyRegs<KW> r;
  const uint4 *kc = reinterpret_cast<const uint4 *>(a.k_codes + row * KW);
#pragma unroll
  for (int w = 0; w < KW / 4; ++w) r.kc[w] = kc[w];
  r.sg = make_uint4(0, 0, 0, 0);
  r.gamma = 0.f;
  if constexpr (QJL) {
    r.sg = *reinterpret_cast<const uint4 *>(a.k_signs + row * (kQjlDim / 32));
    r.gamma = a.k_res[row];
  }
  r.nu = a.k_norms[row];
  return r;
}

__device__ __forceinline__ ValRegs load_values(const DecodeArgs &a, int64_t row, int VW) {
  ValRegs r;
  const uint4 *vc = reinterpret_cast<const uint4 *>(a.v_codes + row * VW);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint4 t = make_uint4(0, 0, 0, 0);
    if (w < VW / 4) t = vc[w];
    r.vc[w] = t;
  }
  r.nu_v = a.v_norms[row];
  return r;
}

template <int G> struct Lds {
  using GM = Geom<G>;
  struct Pro {      // prologue
    float q[G][D];
    float part[GM::kParts][G][D];
    float qr[G][D];
    float s[G][D];
  };
  union Shared {
    Pro pro;
    uint32_t vrec[GM::kWaves][64 * kRecStride];
    float merge[GM::kWaves][G][D];
  };
};

template <int KB, bool QJL, int G>
__global__ __launch_bounds__(Geom<G>::kThreads) void decode_kernel(DecodeArgs a) {
  using KL = KeyLut<KB>;
  constexpr int kWaves = Geom<G>::kWaves;
  constexpr int kThreads = Geom<G>::kThreads;
  constexpr int kParts = Geom<G>::kParts;
  constexpr int kJ = D / kParts;    // prologue: coordinates per partial dot product
  constexpr int kPass = 64 * kWaves;
  constexpr int KW = D * KB / 32;   // key code words per token
  __shared__ float s_kdeq[KL::kEntries * KL::kCoords];
  __shared__ float2 s_vdeq[256];
  __shared__ float s_slut[QJL ? G : 1][kSignLut];
  __shared__ typename Lds<G>::Shared sh;
  __shared__ float s_ml[kWaves][G][2];

  const int chunk_id = blockIdx.x;
  const int hk = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hq0 = hk * G;
  const int VB = a.v_bits;
  const int VW = 4 * VB;
  const int row_id = b * a.n_kv_heads + hk;             // (b, kv head)
  const int group_id = row_id * a.n_chunks + chunk_id;  // this work-group

  int T = a.seq_len[b];
  T = T < 0 ? 0 : (T > a.t_cap ? static_cast<int>(a.t_cap) : T);
  const int t_begin = chunk_id * a.chunk;
  const int t_end = min(T, t_begin + a.chunk);
  const int64_t row0 = static_cast<int64_t>(row_id) * a.t_cap;
  auto row_of = [&](int tb) -> int64_t { return row0 + ((tb + lane < t_end) ? tb + lane : tb); };
  // First tile's records are requested before the prologue so that their
  // latency overlaps it.
  const int tb0 = t_begin + wave * 64;
  KeyRegs<KW> cur{};
  ValRegs vcur{};
  if (tb0 < t_end) {
    cur = load_keys<KW, QJL>(a, row_of(tb0));
    vcur = load_values(a, row_of(tb0), VW);
  }

  // ------------------------------------------------------------ 0. prologue
  for (int e = tid; e < G * D; e += kThreads)
    sh.pro.q[e / D][e % D] = load_q(a.q, a.q_bf16, static_cast<int64_t>(b * a.n_q_heads + hq0) * D + e);
  {
    // dequantization tables, precomputed per codebook
    const uint4 *kl = reinterpret_cast<const uint4 *>(a.k_lut);
    uint4 *kd = reinterpret_cast<uint4 *>(s_kdeq);
    for (int e = tid; e < KL::kEntries * KL::kCoords / 4; e += kThreads) kd[e] = kl[e];
    const uint4 *vl = reinterpret_cast<const uint4 *>(a.v_lut);
    uint4 *vd = reinterpret_cast<uint4 *>(s_vdeq);
    for (int e = tid; e < (1 << (2 * VB)) / 2; e += kThreads) vd[e] = vl[e];
  }
  __syncthreads();
  float *slot = a.ws_qslot + static_cast<int64_t>(group_id) * G * kQSlot;
  {
    // q~_i = sum_j Pi[i][j] q_j: thread (i, part) sums j in [kJ part, kJ part + kJ)
    const int i = tid & (D - 1), part = tid >> 7;
    float acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = 0.f;
    float pv[kJ];
#pragma unroll
    for (int jj = 0; jj < kJ; ++jj) pv[jj] = a.rot_k_t[(kJ * part + jj) * D + i];
#pragma unroll
    for (int jj = 0; jj < kJ; ++jj)
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] = fmaf(pv[jj], sh.pro.q[h][kJ * part + jj], acc[h]);
#pragma unroll
    for (int h = 0; h < G; ++h) sh.pro.part[part][h][i] = acc[h];
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += kThreads) {
    const int h = e / D, i = e % D;
    float v = 0.f;
#pragma unroll
    for (int pp = 0; pp < kParts; ++pp) v += sh.pro.part[pp][h][i];
    sh.pro.qr[h][i] = v;
    slot[h * kQSlot + i] = v;
  }
  if constexpr (QJL) {
    __syncthreads();
    const int r = tid & (D - 1), part = tid >> 7;
    float acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = 0.f;
    float sv[kJ];
#pragma unroll
    for (int jj = 0; jj < kJ; ++jj) sv[jj] = a.qjl_t[(kJ * part + jj) * kQjlDim + r];
#pragma unroll
    for (int jj = 0; jj < kJ; ++jj)
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] = fmaf(sv[jj], sh.pro.qr[h][kJ * part + jj], acc[h]);
#pragma unroll
    for (int h = 0; h < G; ++h) sh.pro.part[part][h][r] = acc[h];
    __syncthreads();
    for (int e = tid; e < G * kQjlDim; e += kThreads) {
      const int h = e / kQjlDim, i = e % kQjlDim;
      float v = 0.f;
#pragma unroll
      for (int pp = 0; pp < kParts; ++pp) v += sh.pro.part[pp][h][i];
      sh.pro.s[h][i] = v;
      slot[h * kQSlot + D + i] = v;
    }
    __syncthreads();
    // lut[h][pos][nib] = sum_{k<4} s_h[4 pos + k] * (bit k of nib ? +1 : -1)
    for (int e = tid; e < G * kSignLut; e += kThreads) {
      const int h = e / kSignLut, pos = (e % kSignLut) >> 4, nib = e & 15;
      float v = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) v += ((nib >> k) & 1) ? sh.pro.s[h][4 * pos + k] : -sh.pro.s[h][4 * pos + k];
      s_slut[h][e % kSignLut] = v;
    }
  }
  // The slot is re-read below through the scalar cache, which reads the L2 of
  // this work-group's own XCD (and was invalidated at kernel start): waiting
  // for this wave's stores to complete is enough; no device-wide write-back.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // ------------------------------------------------------------ 1. main loop
  const uniform_fptr qs = (uniform_fptr)slot;

  const int vstart = 2 * lane * VB;     // this lane owns rotated coordinates 2 lane, 2 lane + 1
  const int vword = vstart >> 5;
  const int vshift = vstart & 31;
  const uint32_t vmask2 = (1u << (2 * VB)) - 1u;
  uint32_t *rec = sh.vrec[wave];

  float m_run[G], l_run[G], acc0[G], acc1[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
    acc0[h] = 0.f;
    acc1[h] = 0.f;
  }

  for (int tb = tb0; tb < t_end; tb += kPass) {
    const int t = tb + lane;
    const bool valid = t < t_end;
    if (tb != tb0) vcur = load_values(a, row_of(tb), VW);
    KeyRegs<KW> nxt{};
    if (tb + kPass < t_end) nxt = load_keys<KW, QJL>(a, row_of(tb + kPass));
    float l[G];
    {
      uint32_t kw[KW];
#pragma unroll
      for (int w = 0; w < KW / 4; ++w) {
        kw[4 * w] = cur.kc[w].x;
        kw[4 * w + 1] = cur.kc[w].y;
        kw[4 * w + 2] = cur.kc[w].z;
        kw[4 * w + 3] = cur.kc[w].w;
      }
      const uint4 sv4 = cur.sg;
      const float gamma = cur.gamma;
      const float nu = cur.nu;
      float dot[G], snap[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        dot[h] = 0.f;
        snap[h] = 0.f;
      }
      // q~ comes from scalar loads of the slot; the pointer is re-laundered
      // every few coordinates (depending on the products two groups back) so
      // that only two groups of scalar values are live: one in use, one in flight.
      uniform_fptr qv = qs;
      constexpr int kRelaunder = (32 / G > KL::kCoords) ? 32 / G : KL::kCoords;
#pragma unroll
      for (int g = 0; g < KL::kLookups; ++g) {
        const int c0 = g * KL::kCoords;
        if ((c0 % kRelaunder) == 0) {
#pragma unroll
          for (int h = 0; h < G; ++h) asm volatile("" : "+s"(qv) : "v"(snap[h]));
#pragma unroll
          for (int h = 0; h < G; ++h) snap[h] = dot[h];
        }
        const int bit = g * KL::kBitsPerLookup;
        const int w = bit >> 5, sh_ = bit & 31;
        uint32_t idx;
        if (sh_ + KL::kBitsPerLookup <= 32) {
          idx = (kw[w] >> sh_) & (KL::kEntries - 1);
        } else {
          idx = __builtin_amdgcn_alignbit(kw[w + 1], kw[w], sh_) & (KL::kEntries - 1);
        }
        if constexpr (KL::kCoords == 4) {
          const float4 v = reinterpret_cast<const float4 *>(s_kdeq)[idx];
#pragma unroll
          for (int h = 0; h < G; ++h) {
            dot[h] = fmaf(qv[h * kQSlot + c0 + 0], v.x, dot[h]);
            dot[h] = fmaf(qv[h * kQSlot + c0 + 1], v.y, dot[h]);
            dot[h] = fmaf(qv[h * kQSlot + c0 + 2], v.z, dot[h]);
            dot[h] = fmaf(qv[h * kQSlot + c0 + 3], v.w, dot[h]);
          }
        } else {
          const float2 v = reinterpret_cast<const float2 *>(s_kdeq)[idx];
#pragma unroll
          for (int h = 0; h < G; ++h) {
            dot[h] = fmaf(qv[h * kQSlot + c0 + 0], v.x, dot[h]);
            dot[h] = fmaf(qv[h * kQSlot + c0 + 1], v.y, dot[h]);
          }
        }
      }
      if constexpr (QJL) {
        const uint32_t sw[4] = {sv4.x, sv4.y, sv4.z, sv4.w};
        float sd[G];
#pragma unroll
        for (int h = 0; h < G; ++h) sd[h] = 0.f;
        uint32_t lut_off = 0;   // always 0; opaque so that only 8 positions of loads are in flight
#pragma unroll
        for (int p = 0; p < 32; ++p) {
          if ((p & 7) == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) asm volatile("" : "+v"(lut_off) : "v"(sd[h]));
          }
          const uint32_t nib = ((sw[p >> 3] >> (4 * (p & 7))) & 15u) + lut_off;
#pragma unroll
          for (int h = 0; h < G; ++h) sd[h] += s_slut[h][p * 16 + nib];
        }
        const float gq = a.qjl_coef * gamma;
#pragma unroll
        for (int h = 0; h < G; ++h) dot[h] = fmaf(gq, sd[h], dot[h]);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        l[h] = valid ? a.scale * nu * dot[h] : -INFINITY;
        if (a.dbg_scores != nullptr && valid)
          a.dbg_scores[(static_cast<int64_t>(b) * a.n_q_heads + hq0 + h) * a.t_cap + t] = l[h];
      }
    }
    // ---- stage this lane's value record
    {
      uint4 *dst = reinterpret_cast<uint4 *>(rec + lane * kRecStride);
#pragma unroll
      for (int w = 0; w < 4; ++w)
        if (w < VW / 4) dst[w] = vcur.vc[w];
      rec[lane * kRecStride + VW] = 0u;
    }
    const float nu_v = vcur.nu_v;
    // ---- online softmax over this wave's tile
    float w_tok[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mx = wave_max(l[h]);
      const float m_new = fmaxf(m_run[h], mx);
      const float alpha = (m_run[h] == -INFINITY) ? 0.f : __expf(m_run[h] - m_new);
      const float p = valid ? __expf(l[h] - m_new) : 0.f;
      l_run[h] = l_run[h] * alpha + wave_sum(p);
      m_run[h] = m_new;
      acc0[h] *= alpha;
      acc1[h] *= alpha;
      w_tok[h] = p * nu_v;   // zero for lanes past the end of the chunk
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---- value sum over all 64 staged tokens (weights of missing tokens are 0)
    for (int kb = 0; kb < 64; kb += 8) {
      float2 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t w0 = rec[(kb + u) * kRecStride + vword];
        const uint32_t w1 = rec[(kb + u) * kRecStride + vword + 1];
        const uint32_t win = __builtin_amdgcn_alignbit(w1, w0, vshift) & vmask2;
        v[u] = s_vdeq[win];
      }
      // all the group's weights first, so that the scalar results are ready
      // (no hazard stalls) by the time the products read them
      float wk[8][G];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int h = 0; h < G; ++h) wk[u][h] = readlane_f(w_tok[h], kb + u);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          acc0[h] = fmaf(wk[u][h], v[u].x, acc0[h]);
          acc1[h] = fmaf(wk[u][h], v[u].y, acc1[h]);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    cur = nxt;
  }

  // ------------------------------------------------------------ 2. merge waves
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s_ml[wave][h][0] = m_run[h];
      s_ml[wave][h][1] = l_run[h];
    }
  }
  __syncthreads();   // every wave is done with its staged records
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, s_ml[w][h][0]);
    const float f = (m_run[h] == -INFINITY) ? 0.f : __expf(m_run[h] - mx);
    sh.merge[wave][h][2 * lane] = acc0[h] * f;
    sh.merge[wave][h][2 * lane + 1] = acc1[h] * f;
  }
  __syncthreads();
  float *part_o = a.ws_part_o + static_cast<int64_t>(group_id) * G * D;
  for (int e = tid; e < G * D; e += kThreads) {
    const int h = e / D, j = e % D;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += sh.merge[w][h][j];
    part_o[e] = s;
  }
  if (tid < G) {
    const int h = tid;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, s_ml[w][h][0]);
    float lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (s_ml[w][h][0] != -INFINITY) lsum += s_ml[w][h][1] * __expf(s_ml[w][h][0] - mx);
    a.ws_part_ml[(static_cast<int64_t>(group_id) * G + h) * 2 + 0] = mx;
    a.ws_part_ml[(static_cast<int64_t>(group_id) * G + h) * 2 + 1] = lsum;
  }

}

// Merge of the chunks of one (b, q head): log-sum-exp weights, rotated sum,
// then o = Pi_v^T o~.  A separate launch: the kernel boundary makes every
// chunk's partials visible across XCDs without an in-kernel device fence.
constexpr int kCombThreads = 512;

__global__ __launch_bounds__(kCombThreads) void combine_kernel(DecodeArgs a) {
  __shared__ float s_w[kMaxDecodeChunks];
  __shared__ float s_l[kMaxDecodeChunks];
  __shared__ float s_o[4][D];
  __shared__ float s_r[4][D];
  __shared__ float s_scal[2];
  const int bhq = blockIdx.x;                  // b * Hq + q head
  const int b = bhq / a.n_q_heads;
  const int hq = bhq % a.n_q_heads;
  const int g = a.n_q_heads / a.n_kv_heads;
  const int hk = hq / g, h = hq % g;
  const int row_id = b * a.n_kv_heads + hk;
  const int tid = threadIdx.x;
  const int nc = a.n_chunks;
  const int64_t grp0 = static_cast<int64_t>(row_id) * nc;
  for (int c = tid; c < nc; c += kCombThreads) {
    const float m = a.ws_part_ml[((grp0 + c) * g + h) * 2];
    const float l = a.ws_part_ml[((grp0 + c) * g + h) * 2 + 1];
    s_w[c] = (l > 0.f) ? m : -INFINITY;
    s_l[c] = l;
  }
  // Prefetch Pi_v for the final product while the weights are computed:
  // thread (i, quarter) covers j in [32 quarter, 32 quarter + 32).
  const int i = tid & (D - 1), quarter = tid >> 7;
  float pv[32];
#pragma unroll
  for (int jj = 0; jj < 32; ++jj) pv[jj] = a.rot_v[(32 * quarter + jj) * D + i];
  __syncthreads();
  if (tid < 64) {
    float mx = -INFINITY;
    for (int c = tid; c < nc; c += 64) mx = fmaxf(mx, s_w[c]);
    mx = wave_max(mx);
    float tot = 0.f;
    for (int c = tid; c < nc; c += 64) {
      const float w = (s_w[c] == -INFINITY) ? 0.f : __expf(s_w[c] - mx);
      s_w[c] = w;
      tot += w * s_l[c];
    }
    tot = wave_sum(tot);
    if (tid == 0) s_scal[0] = (tot > 0.f) ? 1.f / tot : 0.f;
  }
  __syncthreads();
  const float inv = s_scal[0];
  {
    // rotated output: thread (j, quarter) sums chunks c = quarter, quarter + 4, ...
    float o = 0.f;
#pragma unroll 8
    for (int c = quarter; c < nc; c += 4) o = fmaf(s_w[c], a.ws_part_o[((grp0 + c) * g + h) * D + i], o);
    s_o[quarter][i] = o;
  }
  __syncthreads();
  {
    float r = 0.f;
#pragma unroll
    for (int jj = 0; jj < 32; ++jj) {
      const int j = 32 * quarter + jj;
      r = fmaf(pv[jj], (s_o[0][j] + s_o[1][j] + s_o[2][j] + s_o[3][j]) * inv, r);
    }
    s_r[quarter][i] = r;
  }
  __syncthreads();
  if (tid < D) {
    const float r = s_r[0][tid] + s_r[1][tid] + s_r[2][tid] + s_r[3][tid];
    const int64_t o_idx = static_cast<int64_t>(bhq) * D + tid;
    if (a.out_bf16) {
      static_cast<uint16_t *>(a.out)[o_idx] = f32_to_bf16_rne(r);
    } else {
      static_cast<float *>(a.out)[o_idx] = r;
    }
  }
}

template <int KB, bool QJL>
hipError_t launch_g(const DecodeArgs &a, int g, dim3 grid, hipStream_t stream) {
  switch (g) {
#define TQ_G(GG) \
  case GG: hipLaunchKernelGGL((decode_kernel<KB, QJL, GG>), grid, dim3(Geom<GG>::kThreads), 0, stream, a); break;
    TQ_G(1) TQ_G(2) TQ_G(4) TQ_G(8)
#undef TQ_G
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KB>
hipError_t launch_q(const DecodeArgs &a, int g, dim3 grid, hipStream_t stream) {
  return a.qjl_m > 0 ? launch_g<KB, true>(a, g, grid, stream) : launch_g<KB, false>(a, g, grid, stream);
}

}  // namespace

DecodePlan plan_decode(int batch, int n_q_heads, int n_kv_heads, int64_t t_cap) {
  // Aim at ~256 work-groups (one per CU) of 8 waves over (b, kv head, chunk);
  // a chunk is a multiple of the 512-token work-group pass and there are at
  // most kMaxDecodeChunks.
  DecodePlan p{};
  const int64_t rows = static_cast<int64_t>(batch) * n_kv_heads;
  const int64_t g = n_q_heads / std::max(1, n_kv_heads);
  const int64_t kPass = 512;
  const int64_t target = 256;
  const int64_t passes = std::max<int64_t>(1, (t_cap + kPass - 1) / kPass);
  int64_t want = std::max<int64_t>(1, (target + rows - 1) / std::max<int64_t>(1, rows));
  want = std::min<int64_t>(std::min<int64_t>(want, passes), kMaxDecodeChunks);
  const int64_t passes_per_chunk = (passes + want - 1) / want;
  p.chunk = static_cast<int>(passes_per_chunk * kPass);
  p.n_chunks = static_cast<int>((t_cap + p.chunk - 1) / p.chunk);
  const int64_t groups = rows * p.n_chunks;
  auto align = [](size_t v) { return (v + 255) & ~static_cast<size_t>(255); };
  p.off_qslot = 0;
  p.off_part_o = align(p.off_qslot + static_cast<size_t>(groups) * g * kQSlot * sizeof(float));
  p.off_part_ml = align(p.off_part_o + static_cast<size_t>(groups) * g * D * sizeof(float));
  p.total_bytes = align(p.off_part_ml + static_cast<size_t>(groups) * g * 2 * sizeof(float));
  return p;
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
  const int g = a.n_q_heads / a.n_kv_heads;
  if (a.n_chunks > kMaxDecodeChunks) return hipErrorInvalidValue;
  const dim3 grid(a.n_chunks, a.n_kv_heads, a.batch);
  hipError_t e;
  switch (a.k_bits) {
    case 1: e = launch_q<1>(a, g, grid, stream); break;
    case 2: e = launch_q<2>(a, g, grid, stream); break;
    case 3: e = launch_q<3>(a, g, grid, stream); break;
    case 4: e = launch_q<4>(a, g, grid, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(combine_kernel, dim3(a.batch * a.n_q_heads), dim3(kCombThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tq
