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
// Launches: a query-prep kernel (q~ and s of every query row, fp32), the
// tile kernel, and the decode's combine kernel (log-sum-exp merge of the
// token chunks, Pi_v^T, output).
//
// Tile kernel: work-group = (64 query rows of one kv head, chunk of tokens),
// 8 waves (two per SIMD).  Row m of kv head hk is query j = m / g of q head
// hk g + m % g, at position seq_len - n_new + j; it sees tokens below
// clamp(seq_len - n_new + j + 1, 0, t_cap).  Per 128-token tile:
//   1. the tile's key and value records are staged in LDS (and the next
//      tile's are requested);
//   2. the values are dequantized into a transposed (coordinate x token)
//      bf16 hi/lo tile;
//   3. wave (row half, token quarter) computes its 32 x 32 score block from
//      key codes dequantized straight into MFMA operands, scales and masks
//      it, and stores it in LDS;
//   4. eight threads per row run the online softmax over the 128 tokens and
//      store P = p nu^v as bf16 hi/lo;
//   5. wave (row half, coordinate quarter) rescales (when a running max
//      moved) and accumulates its 32 x 32 output block: P x V.
// The chunk's (max, sum, rotated output) per row go to the workspace in the
// decode's partial layout.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "tq_kernels.h"

namespace tq {
namespace {

constexpr int D = kHeadDim;
constexpr int kRows = 64;               // query rows per work-group
constexpr int kTile = 128;              // tokens per tile
constexpr int kThreads = 512;           // 8 waves
constexpr int kSmT = kThreads / kRows;  // softmax threads per row (16 tokens each)
constexpr int kVtStride = kTile + 8;    // bf16 per coordinate row of the value tile (16 B pad)
constexpr int kPStride = kTile + 8;     // bf16 per row of P
constexpr int kScStride = kTile + 4;    // floats per row of the score tile
constexpr int kQpStride = 2 * D;        // floats per query row in the prep buffer: q~ then s
constexpr int kSStride = D + 8;         // bf16 per row of the LDS copy of s (16 B pad)
// A row's running max is raised only when a score exceeds it by more than
// this (weights stay <= e^8), so most tiles rescale nothing.
constexpr float kLazy = 8.f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
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

__device__ __forceinline__ float load_query(const void *q, int q_bf16, int64_t idx) {
  if (q_bf16) return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t *>(q)[idx]) << 16);
  return static_cast<const float *>(q)[idx];
}

// q~ = Pi_k q and s = (S Pi_k) q of the g query rows of one (b, kv head, j)
// per work-group, written to rows ((b Hkv + hk) n_new + j) g + h of the prep
// buffer.  Thread (column c, part pp): c < d is column c of Pi_k^T, d + i
// column i of (S Pi_k)^T; part pp holds entries 32 pp .. 32 pp + 31 of it
// (all reads issued before the first product) and forms their partial dot
// products with all g queries, which the four parts then sum in LDS.  Each
// matrix is read once per g rows, and each thread's chain is 32 long.
constexpr int kQpParts = 4;
constexpr int kQpThreads = 2 * D * kQpParts;
constexpr int kQpSpan = D / kQpParts;   // matrix entries per thread

template <bool QJL, int G>
__global__ __launch_bounds__(kQpThreads) void qprep_kernel(DecodeArgs a) {
  __shared__ float sq[G][D];
  __shared__ float part[kQpParts][G][2 * D];
  const int qrow = blockIdx.x;   // (b Hkv + hk) n_new + j
  const int j = qrow % a.n_new;
  const int bhk = qrow / a.n_new;
  const int b = bhk / a.n_kv_heads, hk = bhk % a.n_kv_heads;
  const int tid = threadIdx.x;
  const int col = tid & (2 * D - 1), pp = tid / (2 * D);
  const int i = col & (D - 1);
  const bool active = col < D || QJL;   // uniform per wave (D is a multiple of 64)
  const float *mat = col < D ? a.rot_k_t : a.qjl_rot_t;
  float cv[kQpSpan];
  if (active) {
#pragma unroll
    for (int jj = 0; jj < kQpSpan; ++jj) cv[jj] = mat[(kQpSpan * pp + jj) * D + i];
  }
  for (int e = tid; e < G * D; e += kQpThreads)
    sq[e / D][e % D] =
        load_query(a.q, a.q_bf16, (static_cast<int64_t>(b * a.n_q_heads + hk * G + e / D) * a.n_new + j) * D + e % D);
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float acc = 0.f;
    if (active) {
#pragma unroll
      for (int jj = 0; jj < kQpSpan; ++jj) acc = fmaf(cv[jj], sq[h][kQpSpan * pp + jj], acc);
    }
    part[pp][h][col] = acc;
  }
  __syncthreads();
  for (int e = tid; e < G * 2 * D; e += kQpThreads) {
    const int h = e / (2 * D), c = e % (2 * D);
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < kQpParts; ++q) v += part[q][h][c];
    a.ws_qprep[(static_cast<int64_t>(qrow) * G + h) * kQpStride + c] = v;
  }
}

template <int KB, bool QJL>
__global__ __launch_bounds__(kThreads) void chunk_kernel(DecodeArgs a) {
  constexpr int KW = D * KB / 32;       // key code words per token
  constexpr int kKMask = (1 << (2 * KB)) - 1;
  __shared__ uint2 s_kpair[1 << (2 * KB)];     // two key codes -> (hi pair, lo pair)
  __shared__ uint2 s_vpair[256];               // two value codes -> (hi pair, lo pair)
  __shared__ uint32_t s_kc[kTile * KW];
  __shared__ uint32_t s_sg[QJL ? kTile * 4 : 1];
  __shared__ float s_knu[kTile], s_gam[kTile], s_vnu[kTile];
  __shared__ uint32_t s_vc[kTile * 16];
  __shared__ __align__(16) uint16_t s_vth[D * kVtStride];
  __shared__ __align__(16) uint16_t s_vtl[D * kVtStride];
  // the score tile and P share one region: the softmax reads every score
  // into registers, waits, then writes P
  __shared__ __align__(16) union {
    float sc[kRows * kScStride];
    struct {
      uint16_t h[kRows * kPStride];
      uint16_t l[kRows * kPStride];
    } p;
  } s_tile;
  float *const s_sc = s_tile.sc;
  uint16_t *const s_ph = s_tile.p.h;
  uint16_t *const s_pl = s_tile.p.l;
  __shared__ float s_alpha[kRows];
  // the QJL query operand s as bf16 hi/lo, [row][coordinate]: read per k-step
  // (in registers it would not fit beside q~ at two waves per SIMD)
  __shared__ __align__(16) uint16_t s_sh[QJL ? kRows * kSStride : 8];
  __shared__ __align__(16) uint16_t s_sl[QJL ? kRows * kSStride : 8];
  __shared__ int s_rescale;   // some row of the tile raised its running max

  const int g = a.n_q_heads / a.n_kv_heads;
  const int rows_total = g * a.n_new;
  const int n_mb = (rows_total + kRows - 1) / kRows;
  const int chunk_id = blockIdx.x;
  const int hk = blockIdx.y / n_mb;
  const int m0 = (blockIdx.y % n_mb) * kRows;
  const int b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int mblk = wave & 1;             // row half (scores and P x V)
  const int nb = wave >> 1;              // token quarter (scores)
  const int cb = wave >> 1;              // 32-coordinate block (P x V)
  const int VB = a.v_bits, VW = 4 * VB;
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

  // ---- prologue: pair tables, query operands, state
  {
    for (int e = tid; e <= kKMask; e += kThreads) {
      uint32_t h2, l2;
      split_pair(a.k_pair[2 * e], a.k_pair[2 * e + 1], h2, l2);
      s_kpair[e] = make_uint2(h2, l2);
    }
    for (int e = tid; e < (1 << (2 * VB)); e += kThreads) {
      uint32_t h2, l2;
      split_pair(a.v_lut[2 * e], a.v_lut[2 * e + 1], h2, l2);
      s_vpair[e] = make_uint2(h2, l2);
    }
  }
  // A operands of the scores: row 32 mblk + l32 of the block, coordinates
  // 16 ks + 8 hi .. + 7 of q~ (and of s)
  bf16x8 qa_h[8], qa_l[8];
  if constexpr (QJL) {
    // thread: row tid / 8, coordinates 16 (tid % 8) .. + 15 of s
    const int r = tid >> 3, c0 = 16 * (tid & 7);
    const bool live = m0 + r < rows_total;
    const float *sp = a.ws_qprep + (static_cast<int64_t>(row_id) * rows_total + (live ? m0 + r : 0)) * kQpStride + D + c0;
    uint32_t h[8], l[8];
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      const float4 v = live ? reinterpret_cast<const float4 *>(sp)[k4] : make_float4(0.f, 0.f, 0.f, 0.f);
      split_pair(v.x, v.y, h[2 * k4], l[2 * k4]);
      split_pair(v.z, v.w, h[2 * k4 + 1], l[2 * k4 + 1]);
    }
    uint4 *dh = reinterpret_cast<uint4 *>(&s_sh[r * kSStride + c0]);
    uint4 *dl = reinterpret_cast<uint4 *>(&s_sl[r * kSStride + c0]);
    dh[0] = make_uint4(h[0], h[1], h[2], h[3]);
    dh[1] = make_uint4(h[4], h[5], h[6], h[7]);
    dl[0] = make_uint4(l[0], l[1], l[2], l[3]);
    dl[1] = make_uint4(l[4], l[5], l[6], l[7]);
  }
  {
    const int mq = m0 + 32 * mblk + l32;
    const bool live = mq < rows_total;
    const float *qp = a.ws_qprep + (static_cast<int64_t>(row_id) * rows_total + (live ? mq : 0)) * kQpStride;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
      if (live) {
        x0 = *reinterpret_cast<const float4 *>(qp + 16 * ks + 8 * hi);
        x1 = *reinterpret_cast<const float4 *>(qp + 16 * ks + 8 * hi + 4);
      }
      uint32_t h[4], l[4];
      split_pair(x0.x, x0.y, h[0], l[0]);
      split_pair(x0.z, x0.w, h[1], l[1]);
      split_pair(x1.x, x1.y, h[2], l[2]);
      split_pair(x1.z, x1.w, h[3], l[3]);
      qa_h[ks] = as_bf16x8(h[0], h[1], h[2], h[3]);
      qa_l[ks] = as_bf16x8(l[0], l[1], l[2], l[3]);
    }
  }
  // softmax role: row sm of the block, tokens 16 sq .. 16 sq + 15 of a tile
  const int sm = tid / kSmT, sq = tid % kSmT;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o;
#pragma unroll
  for (int r = 0; r < 16; ++r) o[r] = 0.f;

  // A tile's records, one thread's share (tokens past the tile's end read as
  // zero codes): at most one uint4 of key codes and one of value codes (a
  // tile holds 32 KW and 32 VW of them), and for threads < 128 the token's
  // sign words and norms.  Loaded one tile ahead.
  struct Rec {
    uint4 kc, vc, sg;
    float knu, vnu, gam;
  };
  auto load_tile = [&](int t0) {
    Rec r;
    const int nt = min(kTile, t_end - t0);
    r.kc = make_uint4(0u, 0u, 0u, 0u);
    r.vc = r.kc;
    r.sg = r.kc;
    r.knu = r.vnu = r.gam = 0.f;
    if (tid < kTile * KW / 4 && tid / (KW / 4) < nt)
      r.kc = reinterpret_cast<const uint4 *>(a.k_codes + (row0 + t0) * KW)[tid];
    if (tid < kTile * VW / 4 && tid / VB < nt) r.vc = reinterpret_cast<const uint4 *>(a.v_codes + (row0 + t0) * VW)[tid];
    if (tid < nt) {
      r.knu = a.k_norms[row0 + t0 + tid];
      r.vnu = a.v_norms[row0 + t0 + tid];
      if constexpr (QJL) {
        r.gam = a.k_res[row0 + t0 + tid];
        r.sg = reinterpret_cast<const uint4 *>(a.k_signs)[row0 + t0 + tid];
      }
    }
    return r;
  };
  Rec nxt{};
  if (t_begin < t_end) nxt = load_tile(t_begin);

  for (int t0 = t_begin; t0 < t_end; t0 += kTile) {
    // ---- 1. stage the records; the previous tile's readers of these
    // buffers finished before its softmax barrier
    if (tid < kTile * KW / 4) reinterpret_cast<uint4 *>(s_kc)[tid] = nxt.kc;
    if (tid < kTile * VW / 4) reinterpret_cast<uint4 *>(s_vc)[tid] = nxt.vc;
    if (tid < kTile) {
      s_knu[tid] = nxt.knu;
      s_vnu[tid] = nxt.vnu;
      if constexpr (QJL) {
        s_gam[tid] = nxt.gam;
        reinterpret_cast<uint4 *>(s_sg)[tid] = nxt.sg;
      }
    }
    __syncthreads();
    if (tid == 0) s_rescale = 0;   // every reader of the previous tile's flag is past this barrier
    if (t0 + kTile < t_end) nxt = load_tile(t0 + kTile);

    // ---- 2. values -> transposed bf16 hi/lo tile [coordinate][token]
    {
      const int tok = tid & (kTile - 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int grp = tid / kTile + 4 * i;   // coordinates 8 grp .. 8 grp + 7
        const int bit = 8 * grp * VB;
        const int w = bit >> 5, sh = bit & 31;
        const uint32_t w0 = s_vc[tok * VW + w];
        const uint32_t w1 = (sh + 8 * VB > 32) ? s_vc[tok * VW + w + 1] : 0u;
        const uint32_t bits = __builtin_amdgcn_alignbit(w1, w0, sh);
        const uint32_t pmask = (1u << (2 * VB)) - 1u;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint2 e = s_vpair[(bits >> (2 * VB * p)) & pmask];
          const int c = 8 * grp + 2 * p;
          s_vth[c * kVtStride + tok] = static_cast<uint16_t>(e.x);
          s_vth[(c + 1) * kVtStride + tok] = static_cast<uint16_t>(e.x >> 16);
          s_vtl[c * kVtStride + tok] = static_cast<uint16_t>(e.y);
          s_vtl[(c + 1) * kVtStride + tok] = static_cast<uint16_t>(e.y >> 16);
        }
      }
    }

    // ---- 3. scores of rows 32 mblk .., tokens 32 nb + l32
    {
      const int tk = 32 * nb + l32;
      f32x16 sacc, tacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sacc[r] = 0.f;
        tacc[r] = 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        // codes of coordinates 16 ks + 8 hi .. + 7: 8 KB bits
        const int bit = (16 * ks + 8 * hi) * KB;
        const int w = bit >> 5, sh = bit & 31;
        const uint32_t w0 = s_kc[tk * KW + w];
        const uint32_t w1 = (sh + 8 * KB > 32) ? s_kc[tk * KW + w + 1] : 0u;
        const uint32_t bits = __builtin_amdgcn_alignbit(w1, w0, sh);
        uint32_t bh[4], bl[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint2 e = s_kpair[(bits >> (2 * KB * p)) & kKMask];
          bh[p] = e.x;
          bl[p] = e.y;
        }
        const bf16x8 kb_h = as_bf16x8(bh[0], bh[1], bh[2], bh[3]);
        const bf16x8 kb_l = as_bf16x8(bl[0], bl[1], bl[2], bl[3]);
        sacc = mfma(qa_h[ks], kb_h, sacc);
        sacc = mfma(qa_h[ks], kb_l, sacc);
        sacc = mfma(qa_l[ks], kb_h, sacc);
        if constexpr (QJL) {
          // signs 16 ks + 8 hi .. + 7 as bf16 +-1 (set bit: +1)
          const uint32_t b8 = (s_sg[tk * 4 + (ks >> 1)] >> (16 * (ks & 1) + 8 * hi)) & 0xffu;
          uint32_t z[4];
#pragma unroll
          for (int p = 0; p < 4; ++p)
            z[p] = 0xBF80BF80u ^ (((b8 >> (2 * p)) & 1u) << 15) ^ (((b8 >> (2 * p + 1)) & 1u) << 31);
          const bf16x8 zb = as_bf16x8(z[0], z[1], z[2], z[3]);
          const int srow = (32 * mblk + l32) * kSStride + 16 * ks + 8 * hi;
          tacc = mfma(*reinterpret_cast<const bf16x8 *>(&s_sh[srow]), zb, tacc);
          tacc = mfma(*reinterpret_cast<const bf16x8 *>(&s_sl[srow]), zb, tacc);
        }
      }
      const float nu = s_knu[tk];
      const float gq = QJL ? a.qjl_coef * s_gam[tk] : 0.f;
      const int t = t0 + tk;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int mr = 32 * mblk + 8 * (r >> 2) + 4 * hi + (r & 3);
        const int m = m0 + mr;
        const bool live = m < rows_total && t < t_end && t < win(m);
        const float dot = QJL ? fmaf(gq, tacc[r], sacc[r]) : sacc[r];
        s_sc[mr * kScStride + tk] = live ? a.scale * nu * dot : -INFINITY;
      }
    }
    __syncthreads();

    // ---- 4. online softmax, kSmT (8) threads per row
    {
      float lv[16];
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const float4 v = *reinterpret_cast<const float4 *>(&s_sc[sm * kScStride + 16 * sq + 4 * k4]);
        lv[4 * k4] = v.x;
        lv[4 * k4 + 1] = v.y;
        lv[4 * k4 + 2] = v.z;
        lv[4 * k4 + 3] = v.w;
      }
      float mx = lv[0];
#pragma unroll
      for (int k = 1; k < 16; ++k) mx = fmaxf(mx, lv[k]);
      mx = fmaxf(mx, __shfl_xor(mx, 1));
      mx = fmaxf(mx, __shfl_xor(mx, 2));
      mx = fmaxf(mx, __shfl_xor(mx, 4));
      // lazy max: raised only past m_run + kLazy (alpha = 1 otherwise)
      const bool grow = mx > m_run + kLazy;
      const float m_new = grow ? mx : m_run;
      const float alpha = grow ? __expf(m_run - m_new) : 1.f;   // exp(-inf) = 0 for a first max
      if (grow) s_rescale = 1;
      float ls = 0.f;
      uint32_t ph[8], pl[8];
#pragma unroll
      for (int k = 0; k < 16; k += 2) {
        const float p0 = (lv[k] == -INFINITY) ? 0.f : __expf(lv[k] - m_new);
        const float p1 = (lv[k + 1] == -INFINITY) ? 0.f : __expf(lv[k + 1] - m_new);
        ls += p0 + p1;
        split_pair(p0 * s_vnu[16 * sq + k], p1 * s_vnu[16 * sq + k + 1], ph[k / 2], pl[k / 2]);
      }
      ls += __shfl_xor(ls, 1);
      ls += __shfl_xor(ls, 2);
      ls += __shfl_xor(ls, 4);
      l_run = l_run * alpha + ls;
      m_run = m_new;
      __syncthreads();   // every score is read: P may overwrite them
      uint4 *dh = reinterpret_cast<uint4 *>(&s_ph[sm * kPStride + 16 * sq]);
      uint4 *dl = reinterpret_cast<uint4 *>(&s_pl[sm * kPStride + 16 * sq]);
      dh[0] = make_uint4(ph[0], ph[1], ph[2], ph[3]);
      dh[1] = make_uint4(ph[4], ph[5], ph[6], ph[7]);
      dl[0] = make_uint4(pl[0], pl[1], pl[2], pl[3]);
      dl[1] = make_uint4(pl[4], pl[5], pl[6], pl[7]);
      if (sq == 0) s_alpha[sm] = alpha;
    }
    __syncthreads();
    const bool rescale = s_rescale != 0;

    // ---- 5. o = alpha o + P x V for rows 32 mblk .., coordinates 32 cb ..
    {
      if (rescale) {
#pragma unroll
        for (int r = 0; r < 16; ++r) o[r] *= s_alpha[32 * mblk + 8 * (r >> 2) + 4 * hi + (r & 3)];
      }
#pragma unroll
      for (int ks = 0; ks < kTile / 16; ++ks) {
        const int prow = (32 * mblk + l32) * kPStride + 16 * ks + 8 * hi;
        const bf16x8 pa_h = *reinterpret_cast<const bf16x8 *>(&s_ph[prow]);
        const bf16x8 pa_l = *reinterpret_cast<const bf16x8 *>(&s_pl[prow]);
        const int vrow = (32 * cb + l32) * kVtStride + 16 * ks + 8 * hi;
        const bf16x8 vb_h = *reinterpret_cast<const bf16x8 *>(&s_vth[vrow]);
        const bf16x8 vb_l = *reinterpret_cast<const bf16x8 *>(&s_vtl[vrow]);
        o = mfma(pa_h, vb_h, o);
        o = mfma(pa_h, vb_l, o);
        o = mfma(pa_l, vb_h, o);
      }
    }
  }

  // ---- the chunk's partials, in the decode's layout: group (query row of
  // (b, kv head, j), chunk), then head h
  const int nc = a.n_chunks;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = m0 + 32 * mblk + 8 * (r >> 2) + 4 * hi + (r & 3);
    if (m < rows_total) {
      const int64_t grp = (static_cast<int64_t>(row_id) * a.n_new + m / g) * nc + chunk_id;
      a.ws_part_o[(grp * g + m % g) * D + 32 * cb + l32] = o[r];
    }
  }
  if (sq == 0 && m0 + sm < rows_total) {
    const int m = m0 + sm;
    const int64_t grp = (static_cast<int64_t>(row_id) * a.n_new + m / g) * nc + chunk_id;
    a.ws_part_ml[(grp * g + m % g) * 2] = m_run;
    a.ws_part_ml[(grp * g + m % g) * 2 + 1] = l_run;
  }
}

template <int KB>
hipError_t launch_tiles(const DecodeArgs &a, dim3 grid, hipStream_t stream) {
  if (a.qjl_m > 0) {
    hipLaunchKernelGGL((chunk_kernel<KB, true>), grid, dim3(kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL((chunk_kernel<KB, false>), grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
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
  p.off_qprep = align(p.off_part_ml + static_cast<size_t>(groups) * g * 2 * sizeof(float));
  p.total_bytes = align(p.off_qprep + static_cast<size_t>(qrows) * g * kQpStride * sizeof(float));
  return p;
}

hipError_t launch_chunk_mfma(const DecodeArgs &a, hipStream_t stream) {
  const int g = a.n_q_heads / a.n_kv_heads;
  const int n_mb = (g * a.n_new + kRows - 1) / kRows;
  if (a.n_chunks > kMaxDecodeChunks || a.v_bits < 1 || a.v_bits > 4 || a.n_new < 1 ||
      static_cast<int64_t>(a.n_kv_heads) * n_mb > 65535 || a.ws_qprep == nullptr)
    return hipErrorInvalidValue;
  const int n_qrows = a.batch * a.n_kv_heads * a.n_new;   // (b, kv head, j)
  const bool qjl = a.qjl_m > 0;
  switch (g) {
#define TQ_QP(GG)                                                                                   \
  case GG:                                                                                          \
    if (qjl)                                                                                        \
      hipLaunchKernelGGL((qprep_kernel<true, GG>), dim3(n_qrows), dim3(kQpThreads), 0, stream, a);  \
    else                                                                                            \
      hipLaunchKernelGGL((qprep_kernel<false, GG>), dim3(n_qrows), dim3(kQpThreads), 0, stream, a); \
    break;
    TQ_QP(1) TQ_QP(2) TQ_QP(4) TQ_QP(8)
#undef TQ_QP
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
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
