// Multi-query (prefill-chunk) attention over the compressed KV cache on the
// matrix cores (gfx950, v_mfma_f32_32x32x16_bf16).
//
// [admirer.cn memory-wall article, section 1]: every new token attends over
// the keys and values of all tokens up to itself; [same article, section 2]
// and [cc-newplayer explainer, technical breakdown item 4]: attention runs on
// the compressed cache with dequantization.  With n_new new queries per
// (b, q head) the scores and the value sum are dense contractions over a
// (query rows x tokens) tile, so each dequantized key and value tile serves
// every query row of its kv head.  The arithmetic is the decode's:
//     l = scale * nu_t * ( <q~, c_k[code_t]> + sqrt(pi/2)/m * gamma_t <s, 2 z_t - 1> ),
//     o~ = sum_t softmax(l)_t nu^v_t c_v[code^v_t],   o = Pi_v^T o~,
// with q~ = Pi_k q and s = S Pi_k q ([explainer item 2]: the query is rotated
// once instead of every key; [intelliparadigm "3-bit" article, §2.1.2]: the
// QJL residual estimate).  fp32 accuracy from bf16 operands: every fp32
// operand is split as hi + lo (bf16 each) and a product takes the three
// passes hi*hi + hi*lo + lo*hi; the +-1 signs are exact in bf16 (two passes).
//
// Launches: the tile kernel and a merge kernel (log-sum-exp merge of the
// token chunks, Pi_v^T, output).
//
// Tile kernel: work-group = (64 query rows of one kv head, chunk of tokens),
// 8 waves (two per SIMD).  Its prologue forms q~ and s of its rows on the
// matrix cores from the codebook's bf16 hi/lo fragments of Pi_k and S.  Row m of kv head hk is query j = m / g of q head
// hk g + m % g, at position seq_len - n_new + j; it sees tokens below
// clamp(seq_len - n_new + j + 1, 0, t_cap).  The tokens are split among the
// waves (split-K): wave (row half, quarter) takes 32 of every 128 tokens for
// its 32 rows and keeps its own softmax state and output, so a step needs no
// barrier and no score or weight tile in LDS.  Per 32-token step it
//   1. forms the transposed scores (tokens x rows) from key codes dequantized
//      straight into MFMA operands, scales them, masks causally;
//   2. runs the online softmax of each row (one lane pair per row) and turns
//      the weights P = p nu^v into bf16 hi/lo operands in registers;
//   3. accumulates O^T += V^T P^T, dequantizing its own value records.
// At the end the four quarters of each row half merge through LDS, and the
// chunk's (max, sum, rotated output) per row go to the workspace in the
// decode's partial layout.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "tq_kernels.h"

namespace tq {
namespace {

constexpr int D = kHeadDim;
constexpr int kRows = 64;               // query rows per work-group: two halves of 32
constexpr int kStep = 32;               // tokens per wave step
constexpr int kQuart = 4;               // waves per row half, each a quarter of every kTile tokens
constexpr int kTile = kStep * kQuart;   // 128: token chunks are whole multiples of this
constexpr int kWaves = 2 * kQuart;
constexpr int kThreads = 64 * kWaves;
constexpr int kSStride = D + 8;         // bf16 per row of the LDS copy of s (16 B pad)
constexpr int kSlot = 64 * 65;          // floats per wave in the final merge: 64 registers x 64 lanes, rows of 65
// A row's running max (log2 units) is raised only when a score exceeds it by
// more than this (weights stay <= 2^12), so most steps rescale nothing.
constexpr float kLazy2 = 12.f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f32x4 mfma16h(const f16x8 &a, const f16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// fp16 hi parts of (a, b) packed (a in the low half), or with lo set their
// lo parts fp16(a - hi)
__device__ __forceinline__ uint32_t split_f16(float a, float b, bool lo) {
  const f16x2 h = __builtin_convertvector((f32x2){a, b}, f16x2);
  const f16x2 l = __builtin_convertvector((f32x2){a - static_cast<float>(h[0]), b - static_cast<float>(h[1])}, f16x2);
  return __builtin_bit_cast(uint32_t, lo ? l : h);
}

// (a, b) rounded to bf16 (nearest even): a in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// hi = bf16(x), lo = bf16(x - hi), for a pair of values.
__device__ __forceinline__ void split_pair(float a, float b, uint32_t &hi, uint32_t &lo) {
  hi = pack_bf16(a, b);
  lo = pack_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
  return __builtin_bit_cast(bf16x8, make_uint4(w0, w1, w2, w3));
}

// v combined with the value of lane l ^ 32 (one v_permlane32_swap): every lane
// gets op(v[l mod 32], v[l mod 32 + 32]) bit for bit
__device__ __forceinline__ float max_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Split-K tile kernel.  Wave (row half mh, quarter kq) owns rows
// m0 + 32 mh .. + 31 and tokens t_begin + 32 kq + 128 i .. + 31 of its chunk;
// it keeps its own running max, sum and output for its rows, and the four
// quarters of a row half merge once, at the end.
//
// Per 32-token step the wave forms the transposed scores S^T (tokens x rows)
// with v_mfma_f32_32x32x16_bf16: A = the key codes dequantized per token
// (lane = token, coordinates 64 hi + 8 ks .. + 7 at k-step ks, one
// pair-table lookup per two codes), B = q~ of the rows (lane = row, the same
// coordinates, in registers), three passes hi*hi + hi*lo + lo*hi; the QJL
// term takes A = the signs (+-1, exact), B = s from LDS, two passes.  In this
// layout a lane holds 16 tokens of one row, so the row's softmax needs one
// exchange with the lane 32 away, and its weights P are already the B operand
// of the value product O^T += V^T P^T (coordinates x rows), whose A operand,
// lane = coordinate group, dequantizes the tokens that P's k index runs over.
// Nothing passes through LDS per step but the wave's own value records and
// per-token factors, read back by its own lanes (LDS accesses of one wave
// complete in order, so no barrier is needed).
template <int KB, int VB, bool QJL>
__global__ __launch_bounds__(kThreads) void chunk_kernel(DecodeArgs a) {
  constexpr int KH = 2 * KB;              // key code words per half record (64 coordinates)
  constexpr int KW = 2 * KH;
  constexpr int VW = 4 * VB;              // value code words per token
  constexpr int kKP = 1 << (2 * KB), kVP = 1 << (2 * VB);
  constexpr uint32_t kKMask = kKP - 1, kVMask = (1u << VB) - 1;
  constexpr int kVst = kStep * VW + 4;    // a wave's value records (+ the word past the last one)
  // The hi and lo halves of a pair-table entry sit in two arrays whose
  // distance the pad keeps out of reach of a merged two-address LDS read, so
  // each half loads straight into its MFMA operand register.
  struct Smem {
    uint32_t kh[kKP + 1];
    uint32_t pad0[300];
    uint32_t kl[kKP + 1];
    uint32_t vh[kVP + 1];
    uint32_t pad1[300];
    uint32_t vl[kVP + 1];
    alignas(16) uint4 sgn[QJL ? 256 : 1];   // sign byte -> eight bf16 +-1 (set bit: +1)
    alignas(16) float ml[kWaves][32][2];    // per wave and row: running max (log2 units), sum
    alignas(16) union {
      struct {
        uint16_t sh[QJL ? kRows * kSStride : 8];   // s as bf16 hi, [row][coordinate]
        uint16_t sl[QJL ? kRows * kSStride : 8];   // and lo
        uint16_t qh[kRows * kSStride];             // prologue: q~ as bf16 hi, [row][coordinate]
        uint16_t ql[kRows * kSStride];             // and lo
        uint16_t xh[kRows * kSStride];             // prologue: the scaled queries as fp16 hi, [row][coordinate]
        uint16_t xl[kRows * kSStride];             // and lo
        int xexp[kRows];                           // prologue: each row's power-of-two query scale
        uint32_t vst[kWaves][kVst];                // each wave's value records of its step
        float fac[kWaves][3][kStep];               // per token: scale log2(e) nu, coef gamma, nu^v
      } loop;
      float slot[kWaves][kSlot];   // each wave's output scaled to the row half's max: [register][lane], rows of 65
    } u;
  };
  __shared__ Smem sm;

  const int g = a.n_q_heads / a.n_kv_heads;
  const int rows_total = g * a.n_new;
  const int n_mb = (rows_total + kRows - 1) / kRows;
  const int chunk_id = blockIdx.x;
  const int hk = blockIdx.y / n_mb;
  const int m0 = (blockIdx.y % n_mb) * kRows;
  const int b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int mh = wave & 1, kq = wave >> 1;
  const int row_id = b * a.n_kv_heads + hk;
  const int64_t row0 = static_cast<int64_t>(row_id) * a.t_cap;
  const int t_cap = static_cast<int>(a.t_cap);

  // tokens row m sees: [0, win(m)); rows grow with j, so the block's last row sees most
  const int sl = a.seq_len[b];
  auto win = [&](int m) {
    const int w = sl - a.n_new + m / g + 1;
    return w < 0 ? 0 : (w > t_cap ? t_cap : w);
  };
  const int t_begin = chunk_id * a.chunk;
  const int t_end = min(win(min(m0 + kRows, rows_total) - 1), t_begin + a.chunk);

  // ---- prologue: pair and sign tables, s in LDS, q~ in registers
  for (int e = tid; e < kKP; e += kThreads) {
    uint32_t h2, l2;
    split_pair(a.k_pair[2 * e], a.k_pair[2 * e + 1], h2, l2);
    sm.kh[e] = h2;
    sm.kl[e] = l2;
  }
  for (int e = tid; e < kVP; e += kThreads) {
    uint32_t h2, l2;
    split_pair(a.v_lut[2 * e], a.v_lut[2 * e + 1], h2, l2);
    sm.vh[e] = h2;
    sm.vl[e] = l2;
  }
  if constexpr (QJL) {
    for (int e = tid; e < 256; e += kThreads) {
      uint32_t z[4];
#pragma unroll
      for (int p = 0; p < 4; ++p)
        z[p] = 0xBF80BF80u ^ (((e >> (2 * p)) & 1u) << 15) ^ (((e >> (2 * p + 1)) & 1u) << 31);
      sm.sgn[e] = make_uint4(z[0], z[1], z[2], z[3]);
    }
  }
  // The block's queries into LDS as fp16 hi/lo of 2^x q, x per row bringing
  // the row's largest |q| into [64, 128) (thread: row tid / 8, coordinates
  // 16 (tid % 8) .. + 15, the row's eight threads adjacent lanes; rows past
  // the last read as zero; a bf16 query has no lo part).
  const bool q_bf16 = a.q_bf16 != 0;
  {
    const int r = tid >> 3, c0 = 16 * (tid & 7);
    const int m = m0 + r;
    float qv[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) qv[k] = 0.f;
    if (m < rows_total) {
      const int64_t qi = (static_cast<int64_t>(b * a.n_q_heads + hk * g + m % g) * a.n_new + m / g) * D + c0;
      // 4-byte reads: the query need only be 4-byte aligned
      if (q_bf16) {
        const uint32_t *src = reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(a.q) + qi);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const uint32_t w = src[k];
          qv[2 * k] = __uint_as_float(w << 16);
          qv[2 * k + 1] = __uint_as_float(w & 0xffff0000u);
        }
      } else {
        const float *src = static_cast<const float *>(a.q) + qi;
#pragma unroll
        for (int k = 0; k < 16; ++k) qv[k] = src[k];
      }
    }
    float mx = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) mx = fmaxf(mx, fabsf(qv[k]));
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    int ex = 0;
    (void)frexpf(mx, &ex);
    const int xe = (mx > 0.f && mx < INFINITY) ? 7 - ex : 0;
    uint32_t h[8], l[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float y0 = ldexpf(qv[2 * k], xe), y1 = ldexpf(qv[2 * k + 1], xe);
      h[k] = split_f16(y0, y1, false);
      l[k] = split_f16(y0, y1, true);
    }
    uint4 *dh = reinterpret_cast<uint4 *>(&sm.u.loop.xh[r * kSStride + c0]);
    uint4 *dl = reinterpret_cast<uint4 *>(&sm.u.loop.xl[r * kSStride + c0]);
    dh[0] = make_uint4(h[0], h[1], h[2], h[3]);
    dh[1] = make_uint4(h[4], h[5], h[6], h[7]);
    dl[0] = make_uint4(l[0], l[1], l[2], l[3]);
    dl[1] = make_uint4(l[4], l[5], l[6], l[7]);
    if ((tid & 7) == 0) sm.u.loop.xexp[r] = xe;
  }
  // q~ = Pi_k q and s = S Pi_k q of the block's rows on the matrix cores
  // (v_mfma_f32_16x16x32_f16), from the codebook's fp16 hi/lo fragments of
  // 2^kDecFragExp Pi_k and 2^kDecFragExp S Pi_k (the encode's layout): wave t
  // takes output tile t of both, whose lane (n, kq) receives coordinates
  // 32 kq + 4 t .. + 3 of row n of an N-block, and reads each fragment once.
  // B operand: lane (n, kq), element e of k-step ks = query coordinate
  // 32 kq + 8 ks + e of row n.  The passes hi*hi + lo*hi (+ hi*lo for fp32
  // queries) keep 22 significant bits of either operand; q~ and s are then
  // split into the bf16 hi/lo operands of the scores.
  const int n16 = lane & 15, kq4 = lane >> 4;
  f16x8 ph[4], pl[4], fsh[QJL ? 4 : 1], fsl[QJL ? 4 : 1];
  {
    const uint4 *fr = a.k_dfrag_rot;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      ph[ks] = __builtin_bit_cast(f16x8, fr[((0 * 8 + wave) * 4 + ks) * 64 + lane]);
      pl[ks] = __builtin_bit_cast(f16x8, fr[((1 * 8 + wave) * 4 + ks) * 64 + lane]);
    }
    if constexpr (QJL) {
      const uint4 *fq = a.k_dfrag_qjl;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        fsh[ks] = __builtin_bit_cast(f16x8, fq[((0 * 8 + wave) * 4 + ks) * 64 + lane]);
        fsl[ks] = __builtin_bit_cast(f16x8, fq[((1 * 8 + wave) * 4 + ks) * 64 + lane]);
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int nb = 0; nb < kRows / 16; ++nb) {
    f32x4 aq = {0.f, 0.f, 0.f, 0.f}, as = aq;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int xo = (16 * nb + n16) * kSStride + 32 * kq4 + 8 * ks;
      const f16x8 bh = *reinterpret_cast<const f16x8 *>(&sm.u.loop.xh[xo]);
      aq = mfma16h(ph[ks], bh, aq);
      aq = mfma16h(pl[ks], bh, aq);
      if constexpr (QJL) {
        as = mfma16h(fsh[ks], bh, as);
        as = mfma16h(fsl[ks], bh, as);
      }
      if (!q_bf16) {
        const f16x8 bl = *reinterpret_cast<const f16x8 *>(&sm.u.loop.xl[xo]);
        aq = mfma16h(ph[ks], bl, aq);
        if constexpr (QJL) as = mfma16h(fsh[ks], bl, as);
      }
    }
    // undo the operands' scales 2^kDecFragExp and 2^x of the row
    const float un = ldexpf(1.f, -(kDecFragExp + sm.u.loop.xexp[16 * nb + n16]));
    const int qo = (16 * nb + n16) * kSStride + 32 * kq4 + 4 * wave;
    uint32_t h0, l0, h1, l1;
    split_pair(aq[0] * un, aq[1] * un, h0, l0);
    split_pair(aq[2] * un, aq[3] * un, h1, l1);
    *reinterpret_cast<uint2 *>(&sm.u.loop.qh[qo]) = make_uint2(h0, h1);
    *reinterpret_cast<uint2 *>(&sm.u.loop.ql[qo]) = make_uint2(l0, l1);
    if constexpr (QJL) {
      split_pair(as[0] * un, as[1] * un, h0, l0);
      split_pair(as[2] * un, as[3] * un, h1, l1);
      *reinterpret_cast<uint2 *>(&sm.u.loop.sh[qo]) = make_uint2(h0, h1);
      *reinterpret_cast<uint2 *>(&sm.u.loop.sl[qo]) = make_uint2(l0, l1);
    }
  }
  __syncthreads();
  // B operands of the scores: row m0 + 32 mh + l32, coordinates 64 hi + 8 ks .. + 7 of q~
  const int mrow = m0 + 32 * mh + l32;
  const bool row_live = mrow < rows_total;
  bf16x8 qb_h[8], qb_l[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const int qo = (32 * mh + l32) * kSStride + 64 * hi + 8 * ks;
    qb_h[ks] = *reinterpret_cast<const bf16x8 *>(&sm.u.loop.qh[qo]);
    qb_l[ks] = *reinterpret_cast<const bf16x8 *>(&sm.u.loop.ql[qo]);
  }
  __syncthreads();

  const bool wave_live = m0 + 32 * mh < rows_total;
  const int w_first = wave_live ? win(m0 + 32 * mh) : 0;   // the smallest window of the wave's rows
  const int w_row = row_live ? win(mrow) : 0;
  // value operand: A-row l32 of block cb is coordinate 4 l32 + cb, whose
  // four codes are 4 VB bits at this offset of a token's record
  const int vwo = (4 * VB * l32) >> 5, vsh = (4 * VB * l32) & 31;
  uint32_t *const vst = sm.u.loop.vst[wave];
  float (&fac)[3][kStep] = sm.u.loop.fac[wave];

  float m_run = -INFINITY, l_lane = 0.f;
  f32x16 o[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[cb][r] = 0.f;

  // One step's records in registers, loaded one step ahead.  Lane (token
  // l32, half hi): that token's key codes and signs of coordinates 64 hi ..
  // + 63 and its factors (tokens past t_end read the last valid one, masked
  // below); the value records of the step's 32 tokens, one contiguous block,
  // lane L its words 2 VB L .. + 2 VB - 1 (words of missing tokens read as 0).
  struct Rec {
    uint32_t kc[KH];
    uint32_t sg[2];
    float nu, gq, nv;
    uint32_t vw[2 * VB];
  };
  const float nu_scale = a.scale * kLog2e;
  auto load_step = [&](int t0) {
    Rec r;
    const int tok = min(t0 + l32, t_end - 1);
    const int64_t row = row0 + tok;
    const uint32_t *kp = a.k_codes + row * KW + KH * hi;
    if constexpr (KH % 4 == 0) {
#pragma unroll
      for (int w = 0; w < KH / 4; ++w) {
        const uint4 x = reinterpret_cast<const uint4 *>(kp)[w];
        r.kc[4 * w] = x.x;
        r.kc[4 * w + 1] = x.y;
        r.kc[4 * w + 2] = x.z;
        r.kc[4 * w + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int w = 0; w < KH / 2; ++w) {
        const uint2 x = reinterpret_cast<const uint2 *>(kp)[w];
        r.kc[2 * w] = x.x;
        r.kc[2 * w + 1] = x.y;
      }
    }
    r.sg[0] = r.sg[1] = 0u;
    r.gq = 0.f;
    if constexpr (QJL) {
      const uint2 x = reinterpret_cast<const uint2 *>(a.k_signs + row * (kQjlDim / 32))[hi];
      r.sg[0] = x.x;
      r.sg[1] = x.y;
      r.gq = a.qjl_coef * a.k_res[row];
    }
    r.nu = nu_scale * a.k_norms[row];
    r.nv = a.v_norms[row];
    const int nvalid = min(kStep, t_end - t0) * VW;
    const uint32_t *vp = a.v_codes + (row0 + t0) * VW;
#pragma unroll
    for (int u = 0; u < VB; ++u) {
      const int w = 2 * VB * lane + 2 * u;
      const uint2 x = w < nvalid ? *reinterpret_cast<const uint2 *>(vp + w) : make_uint2(0u, 0u);
      r.vw[2 * u] = x.x;
      r.vw[2 * u + 1] = x.y;
    }
    return r;
  };

  int t0 = t_begin + kStep * kq;
  Rec cur{};
  if (wave_live && t0 < t_end) cur = load_step(t0);
  for (; wave_live && t0 < t_end; t0 += kTile) {
    // stage the step's value records and factors (this wave's reads of the
    // previous step's were issued before these writes)
#pragma unroll
    for (int u = 0; u < VB; ++u)
      *reinterpret_cast<uint2 *>(vst + 2 * VB * lane + 2 * u) = make_uint2(cur.vw[2 * u], cur.vw[2 * u + 1]);
    if (hi == 0) {
      fac[0][l32] = cur.nu;
      fac[1][l32] = cur.gq;
      fac[2][l32] = cur.nv;
    }
    Rec nxt = cur;
    if (t0 + kTile < t_end) nxt = load_step(t0 + kTile);

    // ---- scores S^T: C row = token 8 (r / 4) + 4 hi + r % 4 of the step, column = row l32
    f32x16 sacc, tacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sacc[r] = 0.f;
      tacc[r] = 0.f;
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      // codes of coordinates 64 hi + 8 ks .. + 7: 8 KB bits of the half record
      constexpr int kBits = 8 * KB;
      const int bit = kBits * ks, w = bit >> 5, shf = bit & 31;
      uint32_t bits;
      if (shf + kBits > 32)
        bits = __builtin_amdgcn_alignbit(cur.kc[w + 1], cur.kc[w], shf);
      else
        bits = cur.kc[w] >> shf;
      uint32_t h[4], l[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t idx = (bits >> (2 * KB * p)) & kKMask;
        h[p] = sm.kh[idx];
        l[p] = sm.kl[idx];
      }
      const bf16x8 ka_h = as_bf16x8(h[0], h[1], h[2], h[3]);
      const bf16x8 ka_l = as_bf16x8(l[0], l[1], l[2], l[3]);
      sacc = mfma(ka_h, qb_h[ks], sacc);
      sacc = mfma(ka_h, qb_l[ks], sacc);
      sacc = mfma(ka_l, qb_h[ks], sacc);
      if constexpr (QJL) {
        const uint32_t byte = (cur.sg[ks >> 2] >> (8 * (ks & 3))) & 0xffu;
        const bf16x8 z = __builtin_bit_cast(bf16x8, sm.sgn[byte]);
        const int srow = (32 * mh + l32) * kSStride + 64 * hi + 8 * ks;
        tacc = mfma(z, *reinterpret_cast<const bf16x8 *>(&sm.u.loop.sh[srow]), tacc);
        tacc = mfma(z, *reinterpret_cast<const bf16x8 *>(&sm.u.loop.sl[srow]), tacc);
      }
    }
    // logits in log2 units
    float lg[16];
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      const float4 nu4 = *reinterpret_cast<const float4 *>(&fac[0][8 * R + 4 * hi]);
      const float nuv[4] = {nu4.x, nu4.y, nu4.z, nu4.w};
      float gqv[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (QJL) {
        const float4 g4 = *reinterpret_cast<const float4 *>(&fac[1][8 * R + 4 * hi]);
        gqv[0] = g4.x;
        gqv[1] = g4.y;
        gqv[2] = g4.z;
        gqv[3] = g4.w;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = 4 * R + u;
        const float dot = QJL ? fmaf(gqv[u], tacc[r], sacc[r]) : sacc[r];
        lg[r] = nuv[u] * dot;
      }
    }
    if (t0 + kStep > w_first) {   // some token of the step is past some row's window
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (t0 + 8 * (r >> 2) + 4 * hi + (r & 3) >= w_row) lg[r] = -INFINITY;
    }

    // ---- online softmax of row mrow: lanes l32 and l32 + 32 hold its 32 tokens
    float mx = lg[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, lg[r]);
    mx = max_halves(mx);
    if (__any(mx > m_run + kLazy2)) {
      const bool grow = mx > m_run + kLazy2;
      const float m_new = grow ? mx : m_run;
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_lane *= alpha;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[cb][r] *= alpha;
      m_run = m_new;
    }
    const float mref = (m_run == -INFINITY) ? 0.f : m_run;
    // P = p nu^v as bf16 hi/lo B operands: k-step s takes registers 8 s .. 8 s + 7
    uint32_t ph[8], pl[8];
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      const float4 v4 = *reinterpret_cast<const float4 *>(&fac[2][8 * R + 4 * hi]);
      const float nvv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
      for (int u = 0; u < 4; u += 2) {
        const int r = 4 * R + u;
        const float p0 = __builtin_amdgcn_exp2f(lg[r] - mref);
        const float p1 = __builtin_amdgcn_exp2f(lg[r + 1] - mref);
        l_lane += p0 + p1;
        split_pair(p0 * nvv[u], p1 * nvv[u + 1], ph[r >> 1], pl[r >> 1]);
      }
    }

    // ---- O^T += V^T P^T: A-row l32 of block cb = coordinate 4 l32 + cb; k
    // index 8 hi + e of k-step s = token 16 s + 8 (e / 4) + 4 hi + e % 4
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      uint32_t gw[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tok = 16 * s + 8 * (e >> 2) + 4 * hi + (e & 3);
        const uint32_t *rp = vst + tok * VW + vwo;
        if constexpr (VB == 3)
          gw[e] = __builtin_amdgcn_alignbit(rp[1], rp[0], vsh);
        else
          gw[e] = rp[0] >> vsh;
      }
      const bf16x8 pb_h = as_bf16x8(ph[4 * s], ph[4 * s + 1], ph[4 * s + 2], ph[4 * s + 3]);
      const bf16x8 pb_l = as_bf16x8(pl[4 * s], pl[4 * s + 1], pl[4 * s + 2], pl[4 * s + 3]);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        uint32_t h[4], l[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t idx = ((gw[2 * u] >> (VB * cb)) & kVMask) | (((gw[2 * u + 1] >> (VB * cb)) & kVMask) << VB);
          h[u] = sm.vh[idx];
          l[u] = sm.vl[idx];
        }
        const bf16x8 va_h = as_bf16x8(h[0], h[1], h[2], h[3]);
        const bf16x8 va_l = as_bf16x8(l[0], l[1], l[2], l[3]);
        o[cb] = mfma(va_h, pb_h, o[cb]);
        o[cb] = mfma(va_h, pb_l, o[cb]);
        o[cb] = mfma(va_l, pb_h, o[cb]);
      }
    }
    cur = nxt;
  }

  // ---- merge of the four quarters of each row half, then the chunk's partials
  // in the decode's layout: group (query row of (b, kv head, j), chunk), then head h
  {
    const float l_row = sum_halves(l_lane);
    if (hi == 0) {
      sm.ml[wave][l32][0] = m_run;
      sm.ml[wave][l32][1] = l_row;
    }
  }
  __syncthreads();   // every wave is past its loop: the slots may overwrite the loop's LDS
  {
    float M = -INFINITY;
#pragma unroll
    for (int q = 0; q < kQuart; ++q) M = fmaxf(M, sm.ml[2 * q + mh][l32][0]);
    const float sc = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
    float *slot = sm.u.slot[wave];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) slot[(r + 16 * cb) * 65 + lane] = o[cb][r] * sc;
  }
  __syncthreads();
  {
    // thread: row R of the block, coordinates 16 (tid % 8) .. + 15
    const int R = tid >> 3, c0 = 16 * (tid & 7);
    const int rmh = R >> 5, rj = R & 31;
    const int m = m0 + R;
    if (m < rows_total) {
      float M = -INFINITY;
#pragma unroll
      for (int q = 0; q < kQuart; ++q) M = fmaxf(M, sm.ml[2 * q + rmh][rj][0]);
      float out[16];
#pragma unroll
      for (int c16 = 0; c16 < 16; ++c16) {
        // coordinate c: block cb = c % 4, A-row i = c / 4 = 8 (r / 4) + 4 hh + r % 4
        const int c = c0 + c16, i = c >> 2, cb = c & 3;
        const int r = 4 * (i >> 3) + (i & 3), ln = rj + 32 * ((i >> 2) & 1);
        float v = 0.f;
#pragma unroll
        for (int q = 0; q < kQuart; ++q) v += sm.u.slot[2 * q + rmh][(r + 16 * cb) * 65 + ln];
        out[c16] = v;
      }
      const int nc = a.n_chunks;
      const int64_t grp = (static_cast<int64_t>(row_id) * a.n_new + m / g) * nc + chunk_id;
      float4 *dst = reinterpret_cast<float4 *>(a.ws_part_o + (grp * g + m % g) * D + c0);
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) dst[k4] = make_float4(out[4 * k4], out[4 * k4 + 1], out[4 * k4 + 2], out[4 * k4 + 3]);
      if ((tid & 7) == 0) {
        float L = 0.f;
#pragma unroll
        for (int q = 0; q < kQuart; ++q) {
          const float mq = sm.ml[2 * q + rmh][rj][0];
          if (mq != -INFINITY) L += sm.ml[2 * q + rmh][rj][1] * __builtin_amdgcn_exp2f(mq - M);
        }
        a.ws_part_ml[(grp * g + m % g) * 2] = (M == -INFINITY) ? -INFINITY : M * kLn2;
        a.ws_part_ml[(grp * g + m % g) * 2 + 1] = L;
      }
    }
  }
}

template <int KB, int VB>
hipError_t launch_tiles_v(const DecodeArgs &a, dim3 grid, hipStream_t stream) {
  if (a.qjl_m > 0) {
    hipLaunchKernelGGL((chunk_kernel<KB, VB, true>), grid, dim3(kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL((chunk_kernel<KB, VB, false>), grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

template <int KB>
hipError_t launch_tiles(const DecodeArgs &a, dim3 grid, hipStream_t stream) {
  switch (a.v_bits) {
    case 1: return launch_tiles_v<KB, 1>(a, grid, stream);
    case 2: return launch_tiles_v<KB, 2>(a, grid, stream);
    case 3: return launch_tiles_v<KB, 3>(a, grid, stream);
    case 4: return launch_tiles_v<KB, 4>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

DecodePlan plan_chunk_mfma(int batch, int n_q_heads, int n_kv_heads, int n_new, int64_t t_cap) {
  // ~256 work-groups over (b, kv head, 64-row block, token chunk); a chunk is
  // whole tiles, at most kMaxDecodeChunks per row.
  DecodePlan p{};
  const int64_t g = n_q_heads / std::max(1, n_kv_heads);
  const int64_t n_mb = (g * n_new + kRows - 1) / kRows;
  const int64_t wg_rows = static_cast<int64_t>(batch) * n_kv_heads * n_mb;
  const int64_t tiles = std::max<int64_t>(1, (t_cap + kTile - 1) / kTile);
  int64_t want = std::max<int64_t>(1, (256 + wg_rows - 1) / wg_rows);
  want = std::min<int64_t>(std::min<int64_t>(want, tiles), kMaxDecodeChunks);
  p.chunk = static_cast<int>((tiles + want - 1) / want * kTile);
  p.n_chunks = static_cast<int>((t_cap + p.chunk - 1) / p.chunk);
  const int64_t qrows = static_cast<int64_t>(batch) * n_kv_heads * n_new;   // (b, kv head, j)
  const int64_t groups = qrows * p.n_chunks;
  auto align = [](size_t v) { return (v + 255) & ~static_cast<size_t>(255); };
  p.off_qslot = 0;
  p.off_part_o = 0;
  p.off_part_ml = align(p.off_part_o + static_cast<size_t>(groups) * g * D * sizeof(float));
  p.total_bytes = align(p.off_part_ml + static_cast<size_t>(groups) * g * 2 * sizeof(float));
  return p;
}

hipError_t launch_chunk_mfma(const DecodeArgs &a, hipStream_t stream) {
  const int g = a.n_q_heads / a.n_kv_heads;
  const int n_mb = (g * a.n_new + kRows - 1) / kRows;
  if (a.n_chunks > kMaxDecodeChunks || a.v_bits < 1 || a.v_bits > 4 || a.n_new < 1 || g < 1 || g > 8 || a.k_split ||
      static_cast<int64_t>(a.n_kv_heads) * n_mb > 65535 || a.k_dfrag_rot == nullptr ||
      (a.qjl_m > 0 && a.k_dfrag_qjl == nullptr))
    return hipErrorInvalidValue;
  hipError_t e = hipSuccess;
  const dim3 grid(a.n_chunks, a.n_kv_heads * n_mb, a.batch);
  switch (a.k_bits) {
    case 1: e = launch_tiles<1>(a, grid, stream); break;
    case 2: e = launch_tiles<2>(a, grid, stream); break;
    case 3: e = launch_tiles<3>(a, grid, stream); break;
    case 4: e = launch_tiles<4>(a, grid, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  return launch_combine(a, stream);
}

}  // namespace tq
