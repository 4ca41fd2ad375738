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
// Work-group = (batch b, kv head [x query of a chunk], chunk of tokens), 8 waves:
//  0. prologue: q~ = Pi_k q and s = S q~ = (S Pi_k) q for the g q heads of
//     this kv head (parallel partial dot products reduced in LDS, all their
//     global reads issued at once); q~ goes to a per-group workspace slot so
//     that the main loop can read it as scalar (uniform) operands; a nibble
//     table of signed partial sums of s, a key dequantization table and a
//     value pair table are built in LDS.
//  1. each wave, per 64-token tile:
//     * scores, one token per lane: for 1- and 2-bit codes and g >= 2 a sum
//       of table lookups, one per code nibble, each giving that nibble's
//       partial dot product for all g heads; for 3-bit codes and g = 2, 4 one
//       lookup per pair of codes; otherwise key codes dequantized through an
//       LDS table times q~ from scalar registers; the sign term is
//       a sum of table lookups, each giving 4 signs' partial sum for all g
//       heads at once;
//     * online softmax with a lazily raised running max;
//     * value sum: the tile's weights and value records are staged in LDS
//       (records read as one coalesced block); lane (token group, coordinate
//       group) accumulates 8 rotated coordinates x g heads over 16 tokens,
//       a pair table dequantizing two codes per lookup.
//  2. the waves merge; the chunk's (max, sum) and its partial output, rotated
//     back by Pi_v^T (linear, so it commutes with the merge), go to the
//     workspace.
// A second, small launch merges the chunks of each (b, q head) (log-sum-exp)
// and writes the output; when every row is one chunk (and no sequence length
// is to be advanced) the main kernel writes the output itself.
//
// The same kernel serves two more calls: with SC (scores only) it ends after
// the key phase of each tile and writes every l_t (no values, no merge, no
// second launch); with n_new > 1 queries per (b, q head) the grid's y
// dimension also runs over the query j, whose causal window
// seq_len - n_new + j + 1 is uniform across the work-group.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "tq_kernels.h"

namespace tq {
namespace {

constexpr int D = kHeadDim;
// Waves per work-group.  8 for every g: 12 (g = 2, 4) and 16 (g = 1) fit the
// registers too, but measured no faster (the 8B-layer decode took 7% longer).
constexpr int decode_waves(int) { return 8; }

template <int G> struct Geom {
  static constexpr int kWaves = decode_waves(G);
  static constexpr int kThreads = 64 * kWaves;
  // prologue split of the d-long dot products over 128 kParts threads (the
  // others skip that step); a power of two so that it divides d
  static constexpr int kParts = kThreads >= 1024 ? 8 : 4;
};
constexpr int kSignLut = 32 * 16;       // sign-table entries per q head: 32 nibble positions x 16

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
  uint4 v[4];         // the tile's value code words, read flat: uint4 number lane + 64 k
  float nu_v;         // this lane's token's value norm
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

// The value records of tokens [tb, tb + n_valid) are consecutive cache rows,
// so the tile is one contiguous block of 64 * VW words: lane L reads its
// 16-byte pieces L, L + 64, ... (fully coalesced); pieces of missing tokens
// read as zero.  The norm is read per token (one per lane).
__device__ __forceinline__ ValRegs load_values(const DecodeArgs &a, int64_t row_tb, int n_valid, int64_t row_lane,
                                               int VW, int lane) {
  ValRegs r;
  const uint4 *base = reinterpret_cast<const uint4 *>(a.v_codes + row_tb * VW);
  const int lim = n_valid * VW;    // words of valid records
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int f = lane + 64 * k;
    uint4 t = make_uint4(0, 0, 0, 0);
    if (4 * k < VW && 4 * f < lim) t = base[f];
    r.v[k] = t;
  }
  r.nu_v = a.v_norms[row_lane];
  return r;
}

template <int G> struct Lds {
  using GM = Geom<G>;
  struct Pro {      // prologue
    float q[G][D];
    float part[GM::kParts][G][D];
    float part_s[GM::kParts][G][D];
    float s[G][D];
    float qr[G][D];
  };
  struct Loop {     // main loop, one region per wave
    uint32_t vrec[GM::kWaves][64 * 16 + 4];   // a tile's value code words, records back to back (+ pad)
    float wts[GM::kWaves][64 * G];            // per token, the g heads' weights p * nu_v
  };
  struct Epi {      // after the loop
    float merge[GM::kWaves][G][D];   // per-wave rotated sums; then the 4 partial products of Pi_v^T
    float ot[G][D];                  // the work-group's rotated sum
  };
  union Shared {
    Pro pro;
    Loop loop;
    Epi epi;
  };
};

// g consecutive floats from LDS (one 4-, 8- or 16-byte read per 4 heads)
template <int G>
__device__ __forceinline__ void lds_load_g(const float *p, float (&v)[G]) {
  if constexpr (G == 1) {
    v[0] = p[0];
  } else if constexpr (G == 2) {
    const float2 t = *reinterpret_cast<const float2 *>(p);
    v[0] = t.x;
    v[1] = t.y;
  } else {
#pragma unroll
    for (int q4 = 0; q4 < G / 4; ++q4) {
      const float4 t = reinterpret_cast<const float4 *>(p)[q4];
      v[4 * q4] = t.x;
      v[4 * q4 + 1] = t.y;
      v[4 * q4 + 2] = t.z;
      v[4 * q4 + 3] = t.w;
    }
  }
}

template <int G>
__device__ __forceinline__ void lds_store_g(float *p, const float (&v)[G]) {
  if constexpr (G == 1) {
    p[0] = v[0];
  } else if constexpr (G == 2) {
    *reinterpret_cast<float2 *>(p) = make_float2(v[0], v[1]);
  } else {
#pragma unroll
    for (int q4 = 0; q4 < G / 4; ++q4)
      reinterpret_cast<float4 *>(p)[q4] = make_float4(v[4 * q4], v[4 * q4 + 1], v[4 * q4 + 2], v[4 * q4 + 3]);
  }
}

// Query-specific lookup tables (sign table, and the key tables below) hold,
// per nibble position p and nibble value n, one float per head.  Layout: for
// g <= 4 entry (p, n) is g consecutive floats, float offset (16 p + n) g + h;
// for g = 8 the heads are split into two quads, [p][quad][n][4], offset
// ((2 p + h / 4) 16 + n) 4 + h % 4, so that the 64 lanes reading one position
// (each its own n) touch every LDS bank at most once per 16-byte read.

// Ordering without instructions: x is made to depend on the g values d, so
// whatever uses x waits for them.  One asm statement per call: the compiler
// separates consecutive inline-asm statements with s_nop.
template <int G, typename T>
__device__ __forceinline__ void depend_v(T &x, const float (&d)[G]) {
  if constexpr (G == 1) {
    asm volatile("" : "+v"(x) : "v"(d[0]));
  } else if constexpr (G == 2) {
    asm volatile("" : "+v"(x) : "v"(d[0]), "v"(d[1]));
  } else if constexpr (G == 4) {
    asm volatile("" : "+v"(x) : "v"(d[0]), "v"(d[1]), "v"(d[2]), "v"(d[3]));
  } else {
    asm volatile("" : "+v"(x) : "v"(d[0]), "v"(d[1]), "v"(d[2]), "v"(d[3]), "v"(d[4]), "v"(d[5]), "v"(d[6]), "v"(d[7]));
  }
}
// four values at once (g = 8 table reads, four positions in flight)
__device__ __forceinline__ void depend4_v(uint32_t *o, const float (&d)[8]) {
  asm volatile("" : "+v"(o[0]), "+v"(o[1]), "+v"(o[2]), "+v"(o[3])
               : "v"(d[0]), "v"(d[1]), "v"(d[2]), "v"(d[3]), "v"(d[4]), "v"(d[5]), "v"(d[6]), "v"(d[7]));
}
template <int G, typename T>
__device__ __forceinline__ void depend_s(T &x, const float (&d)[G]) {
  if constexpr (G == 1) {
    asm volatile("" : "+s"(x) : "v"(d[0]));
  } else if constexpr (G == 2) {
    asm volatile("" : "+s"(x) : "v"(d[0]), "v"(d[1]));
  } else if constexpr (G == 4) {
    asm volatile("" : "+s"(x) : "v"(d[0]), "v"(d[1]), "v"(d[2]), "v"(d[3]));
  } else {
    asm volatile("" : "+s"(x) : "v"(d[0]), "v"(d[1]), "v"(d[2]), "v"(d[3]), "v"(d[4]), "v"(d[5]), "v"(d[6]), "v"(d[7]));
  }
}

// Nibble n's entry starts n * 4 g bytes into its position for g <= 4, and
// n * 16 bytes into each 4-head group for g = 8: the scaled index fits in a
// byte.  Two masks spread the 8 nibbles of a code word, already scaled, into
// the bytes of two registers (even nibbles, odd nibbles), and one byte
// extract per lookup remains.  o[k] = byte offset of nibble k's entry.
template <int G>
__device__ __forceinline__ void nibble_offsets(uint32_t w, uint32_t (&o)[8]) {
  constexpr int S = G == 1 ? 2 : (G == 2 ? 3 : 4);   // log2 of the entry (group) size in bytes
  constexpr uint32_t M = 0x0F0F0F0Fu << S;
  const uint32_t ev = (w << S) & M;
  const uint32_t od = (S == 4) ? (w & M) : ((w >> (4 - S)) & M);
  o[0] = ev & 0xFFu;
  o[2] = __builtin_amdgcn_ubfe(ev, 8, 8);
  o[4] = __builtin_amdgcn_ubfe(ev, 16, 8);
  o[6] = ev >> 24;
  o[1] = od & 0xFFu;
  o[3] = __builtin_amdgcn_ubfe(od, 8, 8);
  o[5] = __builtin_amdgcn_ubfe(od, 16, 8);
  o[7] = od >> 24;
}

// tab_load with the entry's byte offset (nibble_offsets) within position p.
template <int G>
__device__ __forceinline__ void tab_load_off(const float *tab, int p, uint32_t off, float (&v)[G]) {
  if constexpr (G <= 4) {
    lds_load_g<G>(reinterpret_cast<const float *>(reinterpret_cast<const char *>(tab + p * 16 * G) + off), v);
  } else {
#pragma unroll
    for (int q4 = 0; q4 < G / 4; ++q4) {
      const float4 t = *reinterpret_cast<const float4 *>(reinterpret_cast<const char *>(tab + (p * (G / 4) + q4) * 64) + off);
      v[4 * q4] = t.x;
      v[4 * q4 + 1] = t.y;
      v[4 * q4 + 2] = t.z;
      v[4 * q4 + 3] = t.w;
    }
  }
}

// Float offset e of a table entry -> (p, n, h), the inverse of the layout above.
template <int G>
__device__ __forceinline__ void tab_entry(int e, int &p, int &n, int &h) {
  p = e / (16 * G);
  const int r = e % (16 * G);
  if constexpr (G <= 4) {
    n = r / G;
    h = r % G;
  } else {
    n = (r % 64) / 4;
    h = (r / 64) * 4 + (r & 3);
  }
}

// Key scores by table (for 1- and 2-bit key codes and g >= 2): a nibble of
// codes covers 4 / b' coordinates, and the table entry (p, n, h) is the
// partial dot product of q~_h with the centroids that nibble n encodes at
// position p.  One lookup then replaces 4 / b' multiply-adds per head.
template <int KB, int G> struct KeyTab {
  static constexpr bool kOn = (KB == 1 || KB == 2) && G >= 2;
  static constexpr int kCpn = kOn ? 4 / KB : 1;         // coordinates per nibble
  static constexpr int kPos = D / kCpn;                  // nibble positions
  static constexpr int kFloats = kOn ? kPos * 16 * G : 1;
};

// Key scores by table for 3-bit codes and g = 2, 4: the entry (p, e, h), float
// offset (64 p + e) g + h, is the partial dot product of q~_h with the two
// centroids that the 6-bit index e (codes 2p, 2p + 1) encodes.  One lookup
// and g adds replace 2 g multiply-adds.  64 KiB at g = 4; g = 8 would need
// 128 KiB and keeps the multiply-adds.
template <int KB, int G> struct KeyPairTab {
  static constexpr bool kOn = KB == 3 && G >= 2 && G <= 4;
  static constexpr int kPos = D / 2;                     // code pairs
  static constexpr int kFloats = kOn ? kPos * 64 * G : 1;
};

// Softmax weights are exp(l - m) against a running max m that is only raised
// when a score exceeds it by more than kLazy (then the sums and accumulators
// are rescaled); otherwise every weight is at most e^kLazy.  The result is the
// same softmax, with far fewer wave reductions and rescales.
constexpr float kLazy = 8.f;

// SC (scores only): the prologue and key phase alone; every l_t of the chunk
// goes to a.scores and the kernel ends after its last tile.
template <int KB, bool QJL, int G, bool SC>
__global__ __launch_bounds__(Geom<G>::kThreads) void decode_kernel(DecodeArgs a) {
  using KL = KeyLut<KB>;
  constexpr int kWaves = Geom<G>::kWaves;
  constexpr int kThreads = Geom<G>::kThreads;
  constexpr int kParts = Geom<G>::kParts;
  constexpr int kJ = D / kParts;    // prologue: coordinates per partial dot product
  constexpr int kPass = 64 * kWaves;
  constexpr int KW = D * KB / 32;   // key code words per token
  using KT = KeyTab<KB, G>;
  using KP = KeyPairTab<KB, G>;
  constexpr int kFlight = G >= 8 ? 4 : 8;   // table positions read ahead (32 floats for g = 4, 8)
  // One block, tables first: every table lookup's address is then an index
  // plus a constant below 64 KiB, which the LDS instruction's offset field
  // holds (no add per lookup).
  struct Smem {
    alignas(16) float2 vdeq[SC ? 1 : 256];              // value pair table
    alignas(16) float kdeq[KL::kEntries * KL::kCoords];  // key dequantization table
    // QJL sign table, entry (pos, nib, h) = sum_{k<4} s_h[4 pos + k] * (bit k of nib ? +1 : -1)
    alignas(16) float slut[QJL ? kSignLut * G : 1];
    alignas(16) float ktab[KT::kFloats > KP::kFloats ? KT::kFloats : KP::kFloats];   // key-code tables (KeyTab, KeyPairTab)
    alignas(16) typename Lds<G>::Shared sh;
    alignas(16) float ml[kWaves][G][2];
  };
  __shared__ Smem smem;
  float2 *const s_vdeq = smem.vdeq;
  float *const s_kdeq = smem.kdeq;
  float *const s_slut = smem.slut;
  float *const s_ktab = smem.ktab;
  typename Lds<G>::Shared &sh = smem.sh;
  float (&s_ml)[kWaves][G][2] = smem.ml;

  const int chunk_id = blockIdx.x;
  const int hk = blockIdx.y / a.n_new;        // kv head
  const int jq = blockIdx.y - hk * a.n_new;   // query of the chunk: position seq_len - n_new + jq
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hq0 = hk * G;
  const int VB = a.v_bits;
  const int VW = 4 * VB;
  const int row_id = b * a.n_kv_heads + hk;             // (b, kv head): the cache row
  const int qrow = row_id * a.n_new + jq;               // (b, kv head, query)
  const int group_id = qrow * a.n_chunks + chunk_id;    // this work-group

  // causal window: the query at position p sees cached tokens 0 .. p
  int T = a.seq_len[b] + a.seq_add - (a.n_new - 1 - jq);
  T = T < 0 ? 0 : (T > a.t_cap ? static_cast<int>(a.t_cap) : T);
  const int t_begin = chunk_id * a.chunk;
  const int t_end = min(T, t_begin + a.chunk);
  const int64_t row0 = static_cast<int64_t>(row_id) * a.t_cap;
  auto row_of = [&](int tb) -> int64_t { return row0 + ((tb + lane < t_end) ? tb + lane : tb); };
  const int tb0 = t_begin + wave * 64;

  // ------------------------------------------------------------ 0. prologue
  // Every global read of the prologue is issued up front: this thread's slices
  // of Pi_k^T and (S Pi_k)^T, the query and the codebook tables.  Thread
  // (i, part) then forms the partial dot products over j in [kJ part, kJ part + kJ)
  // of q~_i = sum_j Pi[i][j] q_j and s_i = sum_j (S Pi)[i][j] q_j.
  const int pi_ = tid & (D - 1), part = tid >> 7;
  const bool in_pro = part < kParts;   // wave-uniform
  float pv[kJ], sv[QJL ? kJ : 1];
  if (in_pro) {
#pragma unroll
    for (int jj = 0; jj < kJ; ++jj) pv[jj] = a.rot_k_t[(kJ * part + jj) * D + pi_];
    if constexpr (QJL) {
#pragma unroll
      for (int jj = 0; jj < kJ; ++jj) sv[jj] = a.qjl_rot_t[(kJ * part + jj) * kQjlDim + pi_];
    }
  }
  for (int e = tid; e < G * D; e += kThreads)
    sh.pro.q[e / D][e % D] =
        load_q(a.q, a.q_bf16, (static_cast<int64_t>(b * a.n_q_heads + hq0 + e / D) * a.n_new + jq) * D + e % D);
  {
    // dequantization tables, precomputed per codebook
    const uint4 *kl = reinterpret_cast<const uint4 *>(a.k_lut);
    uint4 *kd = reinterpret_cast<uint4 *>(s_kdeq);
    for (int e = tid; e < KL::kEntries * KL::kCoords / 4; e += kThreads) kd[e] = kl[e];
    if constexpr (!SC) {
      const uint4 *vl = reinterpret_cast<const uint4 *>(a.v_lut);
      uint4 *vd = reinterpret_cast<uint4 *>(s_vdeq);
      for (int e = tid; e < (1 << (2 * VB)) / 2; e += kThreads) vd[e] = vl[e];
    }
  }
  __syncthreads();
  // The first tile's records are requested now: after the prologue's own reads
  // (the wait for those must not include HBM latency, since memory reads
  // retire in order) and early enough to overlap the rest of the prologue.
  KeyRegs<KW> cur{};
  ValRegs vcur{};
  if (tb0 < t_end) {
    cur = load_keys<KW, QJL>(a, row_of(tb0));
    if constexpr (!SC) vcur = load_values(a, row0 + tb0, t_end - tb0, row_of(tb0), VW, lane);
  }
  if (in_pro) {
    float aq[G], as[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      aq[h] = 0.f;
      as[h] = 0.f;
    }
#pragma unroll
    for (int jj = 0; jj < kJ; ++jj)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float qj = sh.pro.q[h][kJ * part + jj];
        aq[h] = fmaf(pv[jj], qj, aq[h]);
        if constexpr (QJL) as[h] = fmaf(sv[jj], qj, as[h]);
      }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sh.pro.part[part][h][pi_] = aq[h];
      if constexpr (QJL) sh.pro.part_s[part][h][pi_] = as[h];
    }
  }
  __syncthreads();
  // q~ goes to this work-group's slot, coordinate-major ([i][h]) so that the
  // main loop reads a few coordinates of all g heads with one scalar load.
  float *slot = a.ws_qslot + static_cast<int64_t>(group_id) * G * D;
  for (int e = tid; e < G * D; e += kThreads) {
    const int h = e / D, i = e % D;
    float v = 0.f, w = 0.f;
#pragma unroll
    for (int pp = 0; pp < kParts; ++pp) {
      v += sh.pro.part[pp][h][i];
      if constexpr (QJL) w += sh.pro.part_s[pp][h][i];
    }
    if constexpr (!KT::kOn && !KP::kOn) slot[i * G + h] = v;
    sh.pro.qr[h][i] = v;
    if constexpr (QJL) sh.pro.s[h][i] = w;
  }
  __syncthreads();
  if constexpr (QJL) {
    for (int e = tid; e < G * kSignLut; e += kThreads) {
      int pos, nib, h;
      tab_entry<G>(e, pos, nib, h);
      float v = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) v += ((nib >> k) & 1) ? sh.pro.s[h][4 * pos + k] : -sh.pro.s[h][4 * pos + k];
      s_slut[e] = v;
    }
  }
  if constexpr (KT::kOn) {
    // centroid of code value c is coordinate 0 of dequantization entry c
    for (int e = tid; e < KT::kFloats; e += kThreads) {
      int pos, nib, h;
      tab_entry<G>(e, pos, nib, h);
      float v = 0.f;
#pragma unroll
      for (int k = 0; k < KT::kCpn; ++k)
        v = fmaf(sh.pro.qr[h][KT::kCpn * pos + k], s_kdeq[((nib >> (KB * k)) & ((1 << KB) - 1)) * KL::kCoords], v);
      s_ktab[e] = v;
    }
  }
  if constexpr (KP::kOn) {
    // dequantization entry e holds (centroid of code e & 7, centroid of code e >> 3)
    for (int e = tid; e < KP::kFloats; e += kThreads) {
      const int pos = e / (64 * G), r = e % (64 * G);
      const int n = r / G, h = r % G;
      s_ktab[e] = fmaf(sh.pro.qr[h][2 * pos], s_kdeq[2 * n], sh.pro.qr[h][2 * pos + 1] * s_kdeq[2 * n + 1]);
    }
  }
  // The slot is re-read below through the scalar cache, which reads the L2 of
  // this work-group's own XCD (and was invalidated at kernel start): waiting
  // for this wave's stores to complete is enough; no device-wide write-back.
  // This holds only while (1) no other work-group of the launch writes this
  // slot (launch_main checks that the grid gives every work-group its own
  // 64-byte aligned slot), (2) no scalar load of the slot happens before these
  // stores (the main loop's first use of qs goes through depend_s on values
  // computed after this point, which keeps the compiler from hoisting it).
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // ------------------------------------------------------------ 1. main loop
  const uniform_fptr qs = (uniform_fptr)slot;

  // value sum layout: lane = (token group tg, coordinate group cg); the lane
  // owns rotated coordinates 8 cg .. 8 cg + 7 and tokens 4 i + tg of a tile
  const int cg = lane & 15, tg = lane >> 4;
  const int vbit = 8 * VB * cg;
  const int vword = vbit >> 5;
  const int vshift = vbit & 31;
  const uint32_t vmask8 = ((1u << (2 * VB)) - 1u) << 3;
  uint32_t *rec = sh.loop.vrec[wave];
  float *wts = sh.loop.wts[wave];

  float m_run[G], l_lane[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_lane[h] = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[h][k] = 0.f;
  }

  for (int tb = tb0; tb < t_end; tb += kPass) {
    const int t = tb + lane;
    const bool valid = t < t_end;
    if constexpr (!SC)
      if (tb != tb0) vcur = load_values(a, row0 + tb, t_end - tb, row_of(tb), VW, lane);
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
      if constexpr (KT::kOn && G <= 4) {
        // one code word (8 positions) at a time: its word is made to depend
        // on the sums so far, so only one word's reads are in flight
#pragma unroll
        for (int wi = 0; wi < KT::kPos / 8; ++wi) {
          uint32_t w = kw[wi];
          depend_v<G>(w, dot);
          uint32_t o[8];
          nibble_offsets<G>(w, o);
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            float v[G];
            tab_load_off<G>(s_ktab, 8 * wi + k, o[k], v);
#pragma unroll
            for (int h = 0; h < G; ++h) dot[h] += v[h];
          }
        }
      } else if constexpr (KT::kOn) {
        // g = 8: kFlight positions' reads in flight, their offsets made to
        // depend on the sums so far
#pragma unroll
        for (int wi = 0; wi < KT::kPos / 8; ++wi) {
          uint32_t o[8];
          nibble_offsets<G>(kw[wi], o);
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            if constexpr (G == 8) {
              static_assert(kFlight == 4, "g = 8 keeps four positions in flight");
              if ((k % 4) == 0) depend4_v(&o[k], dot);
            }
            float v[G];
            tab_load_off<G>(s_ktab, 8 * wi + k, o[k], v);
#pragma unroll
            for (int h = 0; h < G; ++h) dot[h] += v[h];
          }
        }
      }
      if constexpr (KP::kOn) {
        // one lookup per code pair; every 8th pair's index is made to depend
        // on the sums so far, so only 8 lookups are in flight
#pragma unroll
        for (int p = 0; p < KP::kPos; ++p) {
          const int bit = 6 * p, w = bit >> 5, s_ = bit & 31;
          uint32_t e = (s_ + 6 <= 32) ? ((kw[w] >> s_) & 63u) : (__builtin_amdgcn_alignbit(kw[w + 1], kw[w], s_) & 63u);
          if ((p % 8) == 0) depend_v<G>(e, dot);
          float v[G];
          lds_load_g<G>(s_ktab + (p * 64 + e) * G, v);
#pragma unroll
          for (int h = 0; h < G; ++h) dot[h] += v[h];
        }
      }
      uniform_fptr qv = qs;
      constexpr int kRelaunder = (32 / G > KL::kCoords) ? 32 / G : KL::kCoords;
#pragma unroll
      for (int g = 0; g < ((KT::kOn || KP::kOn) ? 0 : KL::kLookups); ++g) {
        const int c0 = g * KL::kCoords;
        if ((c0 % kRelaunder) == 0) {
          depend_s<G>(qv, snap);
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
            dot[h] = fmaf(qv[(c0 + 0) * G + h], v.x, dot[h]);
            dot[h] = fmaf(qv[(c0 + 1) * G + h], v.y, dot[h]);
            dot[h] = fmaf(qv[(c0 + 2) * G + h], v.z, dot[h]);
            dot[h] = fmaf(qv[(c0 + 3) * G + h], v.w, dot[h]);
          }
        } else {
          const float2 v = reinterpret_cast<const float2 *>(s_kdeq)[idx];
#pragma unroll
          for (int h = 0; h < G; ++h) {
            dot[h] = fmaf(qv[(c0 + 0) * G + h], v.x, dot[h]);
            dot[h] = fmaf(qv[(c0 + 1) * G + h], v.y, dot[h]);
          }
        }
      }
      if constexpr (QJL) {
        // sign term: one table read per 4 signs gives all g heads' partial sums
        const uint32_t sw[4] = {sv4.x, sv4.y, sv4.z, sv4.w};
        float sd[G];
#pragma unroll
        for (int h = 0; h < G; ++h) sd[h] = 0.f;
#pragma unroll
        for (int wi = 0; wi < 4; ++wi) {
          uint32_t w = sw[wi];
          if constexpr (G <= 4) depend_v<G>(w, sd);
          uint32_t o[8];
          nibble_offsets<G>(w, o);
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            if constexpr (G == 8) {
              if ((k % 4) == 0) depend4_v(&o[k], sd);
            }
            float v[G];
            tab_load_off<G>(s_slut, 8 * wi + k, o[k], v);
#pragma unroll
            for (int h = 0; h < G; ++h) sd[h] += v[h];
          }
        }
        const float gq = a.qjl_coef * gamma;
#pragma unroll
        for (int h = 0; h < G; ++h) dot[h] = fmaf(gq, sd[h], dot[h]);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        l[h] = valid ? a.scale * nu * dot[h] : -INFINITY;
        if ((SC || a.scores != nullptr) && valid)
          a.scores[((static_cast<int64_t>(b) * a.n_q_heads + hq0 + h) * a.n_new + jq) * a.t_cap + t] = l[h];
      }
    }
    if constexpr (SC) {
      cur = nxt;
      continue;
    }
    // ---- online softmax (lazy running max)
    bool grow = false;
#pragma unroll
    for (int h = 0; h < G; ++h) grow = grow || (l[h] > m_run[h] + kLazy);
    if (__any(grow)) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float m_new = fmaxf(m_run[h], wave_max(l[h]));
        const float alpha = (m_run[h] == -INFINITY) ? 0.f : __expf(m_run[h] - m_new);
        m_run[h] = m_new;
        l_lane[h] *= alpha;
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[h][k] *= alpha;
      }
    }
    float w_tok[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float p = valid ? __expf(l[h] - m_run[h]) : 0.f;
      l_lane[h] += p;
      w_tok[h] = p * vcur.nu_v;   // zero for lanes past the end of the chunk
    }
    // ---- stage the weights and the value records of this tile
    lds_store_g<G>(wts + lane * G, w_tok);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (4 * k < VW) reinterpret_cast<uint4 *>(rec)[lane + 64 * k] = vcur.v[k];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---- value sum: 16 tokens per lane, 8 coordinates x g heads each
#pragma unroll 4
    for (int i = 0; i < 16; ++i) {
      const int tok = 4 * i + tg;
      float wv[G];
      lds_load_g<G>(wts + tok * G, wv);
      const uint32_t w0 = rec[tok * VW + vword];
      const uint32_t w1 = rec[tok * VW + vword + 1];
      // byte offset of pair k in the table (8 bytes per entry) with one shift
      // and one mask: pairs 0, 1 from the slice times 8 (they lie below bit
      // 16, so nothing is shifted out), pairs 2, 3 from the slice shifted 3
      // less to the right
      const uint32_t slice = __builtin_amdgcn_alignbit(w1, w0, vshift);
      const uint32_t slice8 = slice << 3;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t off = (k < 2 ? (slice8 >> (2 * VB * k)) : (slice >> (2 * VB * k - 3))) & vmask8;
        const float2 c = *reinterpret_cast<const float2 *>(reinterpret_cast<const char *>(s_vdeq) + off);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          acc[h][2 * k] = fmaf(wv[h], c.x, acc[h][2 * k]);
          acc[h][2 * k + 1] = fmaf(wv[h], c.y, acc[h][2 * k + 1]);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    cur = nxt;
  }

  if constexpr (SC) return;   // uniform: no barrier follows for any thread

  // ------------------------------------------------------------ 2. merge waves
  // The chunk's partial output leaves the work-group rotated back, o = Pi_v^T o~
  // (linear, so the merge of the chunks commutes with it): thread (i4, q4)
  // applies rows 32 q4 .. 32 q4 + 31 of column i4 of Pi_v, requested now so
  // that the wave merge hides their latency.
  static_assert(kThreads == 4 * D, "the inverse rotation maps 512 threads to (coordinate, quarter)");
  const int i4 = tid & (D - 1), q4 = tid >> 7;
  float pvr[32];
#pragma unroll
  for (int jj = 0; jj < 32; ++jj) pvr[jj] = a.rot_v[(32 * q4 + jj) * D + i4];
  float l_wave[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l_wave[h] = wave_sum(l_lane[h]);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      acc[h][k] += __shfl_xor(acc[h][k], 16);
      acc[h][k] += __shfl_xor(acc[h][k], 32);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s_ml[wave][h][0] = m_run[h];
      s_ml[wave][h][1] = l_wave[h];
    }
  }
  __syncthreads();   // every wave is done with its staged records
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, s_ml[w][h][0]);
    const float f = (m_run[h] == -INFINITY) ? 0.f : __expf(m_run[h] - mx);
    if (tg == 0) {
#pragma unroll
      for (int k = 0; k < 8; ++k) sh.epi.merge[wave][h][8 * cg + k] = acc[h][k] * f;
    }
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += kThreads) {
    const int h = e / D, j = e % D;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += sh.epi.merge[w][h][j];
    sh.epi.ot[h][j] = s;
  }
  __syncthreads();
  {
    float r[G];
#pragma unroll
    for (int h = 0; h < G; ++h) r[h] = 0.f;
#pragma unroll
    for (int jj = 0; jj < 32; ++jj)
#pragma unroll
      for (int h = 0; h < G; ++h) r[h] = fmaf(pvr[jj], sh.epi.ot[h][32 * q4 + jj], r[h]);
    // the quarters' products go where the per-wave sums were (read before the barrier above)
    float *red = &sh.epi.merge[0][0][0];   // [4][G][D]
#pragma unroll
    for (int h = 0; h < G; ++h) red[(q4 * G + h) * D + i4] = r[h];
  }
  __syncthreads();
  if (a.n_chunks == 1 && a.seq_inc == nullptr) {
    // The row is this one chunk: normalize and write the output here (the
    // merge launch is skipped); (1 / l) o is what it would compute for one chunk.
    const float *red = &sh.epi.merge[0][0][0];
    for (int e = tid; e < G * D; e += kThreads) {
      const int h = e / D, i = e % D;
      float mx = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, s_ml[w][h][0]);
      float lsum = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w)
        if (s_ml[w][h][0] != -INFINITY) lsum += s_ml[w][h][1] * __expf(s_ml[w][h][0] - mx);
      const float inv = (lsum > 0.f) ? 1.f / lsum : 0.f;
      const float o = fmaf(inv, red[e] + red[G * D + e] + red[2 * G * D + e] + red[3 * G * D + e], 0.f);
      const int64_t o_idx = ((static_cast<int64_t>(b) * a.n_q_heads + hq0 + h) * a.n_new + jq) * D + i;
      if (a.out_bf16) {
        static_cast<uint16_t *>(a.out)[o_idx] = f32_to_bf16_rne(o);
      } else {
        static_cast<float *>(a.out)[o_idx] = o;
      }
    }
    return;
  }
  float *part_o = a.ws_part_o + static_cast<int64_t>(group_id) * G * D;
  {
    const float *red = &sh.epi.merge[0][0][0];
    for (int e = tid; e < G * D; e += kThreads)
      part_o[e] = red[e] + red[G * D + e] + red[2 * G * D + e] + red[3 * G * D + e];
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

// Merge of the chunks for the matrix-core chunk kernel, whose partial outputs
// stay rotated: log-sum-exp weights, rotated sums, then o = Pi_v^T o~.  A
// work-group merges the g rows of one (b, kv head, query), so it reads Pi_v
// once for all of them; a launch of its own, whose boundary makes every
// chunk's partials visible across XCDs without an in-kernel device fence.
// Every global read (this thread's slice of Pi_v and its rows' partial
// outputs) is issued before the chunk weights are formed.
constexpr int kCombThreads = 512;
constexpr int kCombRegs = 32;   // partial outputs per row held in registers; more chunks are read in a loop

__global__ __launch_bounds__(kCombThreads) void combine_kernel(DecodeArgs a) {
  __shared__ float s_w[8][kMaxDecodeChunks];   // row h: chunk weights divided by the total
  __shared__ float s_o[8][D];                  // row h: merged rotated sum
  __shared__ float s_r[4][8][D];               // quarter products of Pi_v^T
  const int qrow = blockIdx.x;                 // (b * Hkv + kv head) * n_new + query
  const int jq = qrow % a.n_new;
  const int bhk = qrow / a.n_new;
  const int b = bhk / a.n_kv_heads, hk = bhk % a.n_kv_heads;
  const int g = a.n_q_heads / a.n_kv_heads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nc = a.n_chunks;
  const int64_t grp0 = static_cast<int64_t>(qrow) * nc;
  const int64_t cstride = static_cast<int64_t>(g) * D;
  // thread (i, quarter): rows quarter and quarter + 4 at coordinate i, then
  // Pi_v rows 32 quarter .. 32 quarter + 31 of column i for every row
  const int i = tid & (D - 1), quarter = tid >> 7;
  const int h0 = quarter, h1 = quarter + 4;
  const bool has0 = h0 < g, has1 = h1 < g;
  float pv[32];
#pragma unroll
  for (int jj = 0; jj < 32; ++jj) pv[jj] = a.rot_v[(32 * quarter + jj) * D + i];
  const float *pb0 = a.ws_part_o + (grp0 * g + h0) * D + i;
  const float *pb1 = a.ws_part_o + (grp0 * g + h1) * D + i;
  float po0[kCombRegs], po1[kCombRegs];
#pragma unroll
  for (int c = 0; c < kCombRegs; ++c) {
    po0[c] = (has0 && c < nc) ? pb0[c * cstride] : 0.f;
    po1[c] = (has1 && c < nc) ? pb1[c * cstride] : 0.f;
  }
  // wave h < g: the chunk weights of row h (lane c: chunks c and c + 64)
  if (wave < g) {
    const int h = wave;
    float m0 = -INFINITY, l0 = 0.f, m1 = -INFINITY, l1 = 0.f;
    if (lane < nc) {
      m0 = a.ws_part_ml[((grp0 + lane) * g + h) * 2];
      l0 = a.ws_part_ml[((grp0 + lane) * g + h) * 2 + 1];
    }
    if (lane + 64 < nc) {
      m1 = a.ws_part_ml[((grp0 + lane + 64) * g + h) * 2];
      l1 = a.ws_part_ml[((grp0 + lane + 64) * g + h) * 2 + 1];
    }
    static_assert(kMaxDecodeChunks <= 128, "two chunk weights per lane");
    if (!(l0 > 0.f)) m0 = -INFINITY;
    if (!(l1 > 0.f)) m1 = -INFINITY;
    const float mx = wave_max(fmaxf(m0, m1));
    const float w0 = (m0 == -INFINITY) ? 0.f : __expf(m0 - mx);
    const float w1 = (m1 == -INFINITY) ? 0.f : __expf(m1 - mx);
    const float tot = wave_sum(w0 * l0 + w1 * l1);
    const float inv = (tot > 0.f) ? 1.f / tot : 0.f;
    s_w[h][lane] = w0 * inv;
    s_w[h][lane + 64] = w1 * inv;
  }
  __syncthreads();
  if (has0) {
    float o = 0.f;
#pragma unroll
    for (int c = 0; c < kCombRegs; ++c) o = fmaf(s_w[h0][c], po0[c], o);
    for (int c = kCombRegs; c < nc; ++c) o = fmaf(s_w[h0][c], pb0[c * cstride], o);
    s_o[h0][i] = o;
  }
  if (has1) {
    float o = 0.f;
#pragma unroll
    for (int c = 0; c < kCombRegs; ++c) o = fmaf(s_w[h1][c], po1[c], o);
    for (int c = kCombRegs; c < nc; ++c) o = fmaf(s_w[h1][c], pb1[c * cstride], o);
    s_o[h1][i] = o;
  }
  __syncthreads();
  for (int h = 0; h < g; ++h) {
    float r = 0.f;
#pragma unroll
    for (int j4 = 0; j4 < 8; ++j4) {
      const float4 v = *reinterpret_cast<const float4 *>(&s_o[h][32 * quarter + 4 * j4]);
      r = fmaf(pv[4 * j4], v.x, r);
      r = fmaf(pv[4 * j4 + 1], v.y, r);
      r = fmaf(pv[4 * j4 + 2], v.z, r);
      r = fmaf(pv[4 * j4 + 3], v.w, r);
    }
    s_r[quarter][h][i] = r;
  }
  __syncthreads();
  for (int e = tid; e < g * D; e += kCombThreads) {
    const int h = e / D, c = e % D;
    const float r = s_r[0][h][c] + s_r[1][h][c] + s_r[2][h][c] + s_r[3][h][c];
    const int64_t o_idx = ((static_cast<int64_t>(b) * a.n_q_heads + hk * g + h) * a.n_new + jq) * D + c;
    if (a.out_bf16) {
      static_cast<uint16_t *>(a.out)[o_idx] = f32_to_bf16_rne(r);
    } else {
      static_cast<float *>(a.out)[o_idx] = r;
    }
  }
  // Append steps: the sequence has one more cached token (the main kernel,
  // the only reader of seq_len, has completed).
  if (a.seq_inc != nullptr && hk == 0 && jq == 0 && tid == 0) {
    const int32_t s = a.seq_inc[b];
    if (s >= 0 && s < a.t_cap) a.seq_inc[b] = s + 1;
  }
}

// Merge of the chunks of one (b, q head) for the decode kernel, whose partial
// outputs are already rotated back: o = sum_c w_c o_c / sum_c w_c l_c with
// w_c = exp(m_c - max m).  Two waves, thread i = output coordinate i; each
// wave forms the chunk weights itself, so no work-group barrier is needed.
// Every global read is issued before the weights are formed.
constexpr int kOutThreads = 128;
constexpr int kOutRegs = 32;   // partial outputs held in registers; more chunks are read in a loop

__global__ __launch_bounds__(kOutThreads) void combine_out_kernel(DecodeArgs a) {
  __shared__ float s_w[kOutThreads / 64][kMaxDecodeChunks];
  const int bhq = blockIdx.x;                  // (b * Hq + q head) * n_new + query
  const int jq = bhq % a.n_new;
  const int b = bhq / a.n_new / a.n_q_heads;
  const int hq = bhq / a.n_new % a.n_q_heads;
  const int g = a.n_q_heads / a.n_kv_heads;
  const int hk = hq / g, h = hq % g;
  const int qrow = (b * a.n_kv_heads + hk) * a.n_new + jq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nc = a.n_chunks;
  const int64_t grp0 = static_cast<int64_t>(qrow) * nc;
  const float *po = a.ws_part_o + (grp0 * g + h) * D + tid;   // chunk c at + c * g * D
  const int64_t cstride = static_cast<int64_t>(g) * D;
  float pr[kOutRegs];
#pragma unroll
  for (int c = 0; c < kOutRegs; ++c) pr[c] = (c < nc) ? po[c * cstride] : 0.f;
  float m0 = -INFINITY, l0 = 0.f, m1 = -INFINITY, l1 = 0.f;
  if (lane < nc) {
    m0 = a.ws_part_ml[((grp0 + lane) * g + h) * 2];
    l0 = a.ws_part_ml[((grp0 + lane) * g + h) * 2 + 1];
  }
  if (lane + 64 < nc) {
    m1 = a.ws_part_ml[((grp0 + lane + 64) * g + h) * 2];
    l1 = a.ws_part_ml[((grp0 + lane + 64) * g + h) * 2 + 1];
  }
  static_assert(kMaxDecodeChunks <= 128, "two chunk weights per lane");
  if (!(l0 > 0.f)) m0 = -INFINITY;
  if (!(l1 > 0.f)) m1 = -INFINITY;
  const float mx = wave_max(fmaxf(m0, m1));
  const float w0 = (m0 == -INFINITY) ? 0.f : __expf(m0 - mx);
  const float w1 = (m1 == -INFINITY) ? 0.f : __expf(m1 - mx);
  const float tot = wave_sum(w0 * l0 + w1 * l1);
  const float inv = (tot > 0.f) ? 1.f / tot : 0.f;
  s_w[wave][lane] = w0 * inv;
  s_w[wave][lane + 64] = w1 * inv;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float o = 0.f;
#pragma unroll
  for (int c = 0; c < kOutRegs; ++c) o = fmaf(s_w[wave][c], pr[c], o);
  for (int c = kOutRegs; c < nc; ++c) o = fmaf(s_w[wave][c], po[c * cstride], o);
  const int64_t o_idx = static_cast<int64_t>(bhq) * D + tid;
  if (a.out_bf16) {
    static_cast<uint16_t *>(a.out)[o_idx] = f32_to_bf16_rne(o);
  } else {
    static_cast<float *>(a.out)[o_idx] = o;
  }
  // Append steps: the sequence has one more cached token (the main kernel,
  // the only reader of seq_len, has completed).
  if (a.seq_inc != nullptr && hq == 0 && jq == 0 && tid == 0) {
    const int32_t sl = a.seq_inc[b];
    if (sl >= 0 && sl < a.t_cap) a.seq_inc[b] = sl + 1;
  }
}

template <int KB, bool QJL, bool SC>
hipError_t launch_g(const DecodeArgs &a, int g, dim3 grid, hipStream_t stream) {
  switch (g) {
#define TQ_G(GG) \
  case GG: hipLaunchKernelGGL((decode_kernel<KB, QJL, GG, SC>), grid, dim3(Geom<GG>::kThreads), 0, stream, a); break;
    TQ_G(1) TQ_G(2) TQ_G(4) TQ_G(8)
#undef TQ_G
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KB, bool SC>
hipError_t launch_q(const DecodeArgs &a, int g, dim3 grid, hipStream_t stream) {
  return a.qjl_m > 0 ? launch_g<KB, true, SC>(a, g, grid, stream) : launch_g<KB, false, SC>(a, g, grid, stream);
}

// Work-group (chunk, kv head x query, batch) of the grid below owns q~ slot
// group_id = ((b Hkv + hk) n_new + j) n_chunks + chunk: one slot each, g * d
// floats at g * d * 4 bytes apart from a 64-byte aligned base, so no two
// work-groups of a launch share a cache line of the slots (the main loop
// re-reads its own slot through the scalar cache, which is coherent only with
// this work-group's own completed stores).
bool qslots_disjoint(const DecodeArgs &a, int g) {
  static_assert((kHeadDim * sizeof(float)) % 64 == 0, "a slot spans whole 64-byte lines");
  if (reinterpret_cast<uintptr_t>(a.ws_qslot) % 64 != 0) return false;
  const int64_t groups = static_cast<int64_t>(a.batch) * a.n_kv_heads * a.n_new * a.n_chunks;
  const uintptr_t end = reinterpret_cast<uintptr_t>(a.ws_qslot) + static_cast<uintptr_t>(groups) * g * kHeadDim * 4;
  // the slots end before the partial outputs begin (the plan's layout)
  return a.ws_part_o == nullptr || end <= reinterpret_cast<uintptr_t>(a.ws_part_o);
}

template <bool SC>
hipError_t launch_main(const DecodeArgs &a, hipStream_t stream) {
  const int g = a.n_q_heads / a.n_kv_heads;
  if (a.n_chunks > kMaxDecodeChunks || a.n_new < 1 || a.n_kv_heads * a.n_new > 65535) return hipErrorInvalidValue;
  if (!qslots_disjoint(a, g)) return hipErrorInvalidValue;
  const dim3 grid(a.n_chunks, a.n_kv_heads * a.n_new, a.batch);
  switch (a.k_bits) {
    case 1: return launch_q<1, SC>(a, g, grid, stream);
    case 2: return launch_q<2, SC>(a, g, grid, stream);
    case 3: return launch_q<3, SC>(a, g, grid, stream);
    case 4: return launch_q<4, SC>(a, g, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

DecodePlan plan_decode(int batch, int n_q_heads, int n_kv_heads, int64_t t_cap) {
  // Aim at ~256 work-groups (one per CU) over (b, kv head, chunk), at most
  // kMaxDecodeChunks per row.  A chunk is a multiple of 256 tokens: 4k
  // 64-token tiles, dealt to the waves in turn, give each of the 4 SIMDs k.
  DecodePlan p{};
  const int64_t rows = static_cast<int64_t>(batch) * n_kv_heads;
  const int64_t g = n_q_heads / std::max(1, n_kv_heads);
  const int64_t kStep = 256;
  const int64_t target = 256;
  const int64_t passes = std::max<int64_t>(1, (t_cap + kStep - 1) / kStep);
  int64_t want = std::max<int64_t>(1, (target + rows - 1) / std::max<int64_t>(1, rows));
  want = std::min<int64_t>(std::min<int64_t>(want, passes), kMaxDecodeChunks);
  const int64_t passes_per_chunk = (passes + want - 1) / want;
  p.chunk = static_cast<int>(passes_per_chunk * kStep);
  p.n_chunks = static_cast<int>((t_cap + p.chunk - 1) / p.chunk);
  const int64_t groups = rows * p.n_chunks;
  auto align = [](size_t v) { return (v + 255) & ~static_cast<size_t>(255); };
  p.off_qslot = 0;
  p.off_part_o = align(p.off_qslot + static_cast<size_t>(groups) * g * D * sizeof(float));
  p.off_part_ml = align(p.off_part_o + static_cast<size_t>(groups) * g * D * sizeof(float));
  p.total_bytes = align(p.off_part_ml + static_cast<size_t>(groups) * g * 2 * sizeof(float));
  return p;
}

DecodePlan plan_chunk(int batch, int n_q_heads, int n_kv_heads, int n_new, int64_t t_cap) {
  const int g = n_q_heads / std::max(1, n_kv_heads);
  return chunk_uses_mfma(g, n_new) ? plan_chunk_mfma(batch, n_q_heads, n_kv_heads, n_new, t_cap)
                                   : plan_decode(batch * n_new, n_q_heads, n_kv_heads, t_cap);
}

hipError_t launch_combine(const DecodeArgs &a, hipStream_t stream) {
  if (a.n_chunks > kMaxDecodeChunks) return hipErrorInvalidValue;
  if (a.n_q_heads / a.n_kv_heads > 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(combine_kernel, dim3(a.batch * a.n_kv_heads * a.n_new), dim3(kCombThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
  if (a.n_chunks > kMaxDecodeChunks) return hipErrorInvalidValue;
  // single queries where the matrix cores are faster (mdecode_applies): the
  // matrix-core decode; other single queries, and chunks of queries below the
  // matrix-core chunk kernel's size: this file's per-head kernel
  const hipError_t e = mdecode_applies(a) ? launch_mdecode_main(a, false, stream) : launch_main<false>(a, stream);
  if (e != hipSuccess || (a.n_chunks == 1 && a.seq_inc == nullptr)) return e;   // one chunk per row: no merge
  hipLaunchKernelGGL(combine_out_kernel, dim3(a.batch * a.n_q_heads * a.n_new), dim3(kOutThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_logits(const DecodeArgs &a, hipStream_t stream) {
  if (a.scores == nullptr) return hipErrorInvalidValue;
  // the key phase of the kernel launch_decode picks for the same arguments,
  // so the logits equal the decode's own bit for bit
  return mdecode_applies(a) ? launch_mdecode_main(a, true, stream) : launch_main<true>(a, stream);
}

}  // namespace tq
