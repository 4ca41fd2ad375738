// Decode attention over the compressed KV cache on the matrix cores (gfx950,
// v_mfma_f32_16x16x32_bf16): the g query heads of one KV head share every
// dequantized key and value, so the per-token work is a dense (g heads x
// tokens) contraction for the scores and a dense (g heads x tokens) x
// (tokens x d) one for the value sum.  Dequantizing once per token row and
// letting the matrix cores multiply removes the g-fold vector-ALU work of a
// per-head decode.
//
// The arithmetic is the method's ([cc-newplayer explainer, technical
// breakdown items 2 and 4]: the query is rotated once and stays uncompressed,
// attention runs on the compressed K and V with dequantization;
// [admirer.cn memory-wall article, section 2, stage two] and
// [intelliparadigm "3-bit" article, §2.1.2]: the 1-bit QJL estimate of the
// residual's inner product):
//     l_t = scale * nu_t * ( <q~, c_k[code_t]> + sqrt(pi/2)/m * gamma_t * <s, 2 z_t - 1> ),
//     o~  = sum_t softmax(l)_t nu^v_t c_v[code^v_t],   o = Pi_v^T o~,
// with q~ = Pi_k q and s = S Pi_k q.
//
// fp32-level accuracy from 16-bit operands: every fp32 operand is split as
// hi + lo.  The 16 columns of each product carry the g <= 8 heads twice:
// column h holds the query's hi part and column 8 + h its lo part (for the
// value sum: the weights' hi and lo parts), and the dequantized operand is
// applied as its hi part and then its lo part.  The two columns of a head add
// up to the full product (the +-1 signs are exact and need no lo part).  The
// score products take fp16 parts (22 significant bits; per-head power-of-two
// scales keep them in range), because a score can be a small difference of
// large terms; the value sum, whose result only needs absolute accuracy,
// takes bf16 parts.
//
// Work-group = (batch b, kv head, chunk of tokens), 8 waves.  Prologue: the
// lookup tables in LDS (key code pairs, or code quads for 1- and 2-bit codes,
// -> (hi, lo) centroid operands; sign bytes -> eight +-1; pairs of tokens'
// value codes -> (hi, lo) centroid operands), then q~ and s of the g heads on
// the matrix cores from fp16 hi/lo fragments of Pi_k and S Pi_k (22-bit
// operands, fp32-level results), and the query operands split into
// registers.  Main loop: each wave owns every eighth 32-token tile of the
// chunk, with its own running max, sum and output accumulators; tile i's
// value phase and tile i + 1's score phase run in one block while later
// tiles' records load, and the two waves of a SIMD take turns at a raised
// priority.  Per tile and 16-token half: 8 MFMAs give the key term, 4 the
// sign term; the score's two columns are added across lanes, the online
// softmax (running max raised lazily) forms p nu^v, split hi/lo into the
// value product's B operand; 8 MFMAs accumulate the value sum.  Epilogue:
// the waves merge, Pi_v^T rotates the chunk's sum back, and the work-group
// writes the output (one chunk per row) or its partial for the merge launch.
//
// Register layout of v_mfma_f32_16x16x32_bf16 (lane l, n = l % 16,
// kq = l / 16): A operand A[n][8 kq .. 8 kq + 7]; B operand B[8 kq ..][n];
// result C[4 kq + e][n], e = 0..3.  Here:
//   scores  C[token][column] = K^(tokens x coords) Q(coords x columns): lane
//           (n, kq) dequantizes token n's coordinates 32 kq + 4 s .. + 3 at
//           k-step s, each as its (hi, lo) pair (its KB code words in one
//           load), and receives tokens 4 kq + e of every column n;
//   values  C[coord][column] = V^T(coords x tokens) P(tokens x columns): row n
//           of block cb is coordinate 8 n + cb, so lane (n, kq) dequantizes
//           coordinates 8 n .. 8 n + 7 (one 8 b'-bit field per token) of the
//           tokens whose scores it received: the softmax output feeds the B
//           operand without a transposition.
//
// Split widths (SPL: both codebooks put rotated coordinates 0..63 on the
// (b' + 1)-bit codebook, 64..127 on the b'-bit one, records holding the wide
// codes first) [cc-newplayer explainer, technical breakdown item 1;
// intelliparadigm "3-bit" article, §2.1]: the coordinate orders change so that
// every lane sees both widths at compile-time positions.  Key k-steps 0..3
// carry wide coordinates 16 kq + 4 s + i and k-steps 4..7 narrow ones
// 64 + 16 kq + 4 (s - 4) + i; value blocks 0..3 are wide coordinates
// 4 n + cb and blocks 4..7 narrow ones 64 + 4 n + cb - 4.  Each width has its
// own key and value tables.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "tq_kernels.h"

namespace tq {
namespace {

constexpr int D = kHeadDim;
#ifndef TQ_MDEC_WAVES
#define TQ_MDEC_WAVES 8
#endif
constexpr int kWaves = TQ_MDEC_WAVES;     // 8 or more (the prologue and epilogue use the first 512 threads)
constexpr int kThreads = 64 * kWaves;
static_assert(kWaves >= 8, "the prologue and the inverse rotation map 512 threads");
constexpr int kTile = 32;                 // tokens per wave tile (two 16-token halves)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// A head's running max (log2 units) is raised only when a score exceeds it by
// more than this, so the weights stay below 2^12 and most tiles rescale nothing.
constexpr float kLazy2 = 12.f;
// The key operand table holds fp16 hi/lo parts of 256 c (exact power-of-two
// scale), which keeps every centroid's lo part in fp16's normal range.
constexpr float kKeyScale = 256.f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
  return __builtin_bit_cast(bf16x8, make_uint4(w0, w1, w2, w3));
}

// (a, b) rounded to bf16 (nearest even), a in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma_f16(const f16x8 &a, const f16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f16x8 as_f16x8(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
  return __builtin_bit_cast(f16x8, make_uint4(w0, w1, w2, w3));
}

// The fp16 hi parts of (a, b) packed (a in the low half), or with lo set
// their lo parts fp16(a - hi).  Both halves are exact in fp32, so hi + lo
// carries 22 significant bits.
__device__ __forceinline__ uint32_t split_f16(float a, float b, bool lo) {
  const f16x2 h = __builtin_convertvector((f32x2){a, b}, f16x2);
  const f16x2 l = __builtin_convertvector((f32x2){a - static_cast<float>(h[0]), b - static_cast<float>(h[1])}, f16x2);
  return __builtin_bit_cast(uint32_t, lo ? l : h);
}

// The value of lane l ^ 8 (the other column of the same head): a rotation by
// 8 within each row of 16 lanes.
__device__ __forceinline__ float swap8(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t swap8u(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x128, 0xF, 0xF, false));
}

__device__ __forceinline__ float load_query(const void *q, int q_bf16, int64_t idx) {
  if (q_bf16) return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t *>(q)[idx]) << 16);
  return static_cast<const float *>(q)[idx];
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Striped LDS tables: entry e of copy j sits at byte e * kRow + j * kEntryBytes,
// and lane (n, kq) reads copy n % kCopies.  The lanes that the LDS serves
// together then read distinct banks whatever entries they pick.
template <int ENTRY_BYTES, int COPIES> struct Striped {
  static constexpr int kEntryBytes = ENTRY_BYTES;
  static constexpr int kCopies = COPIES;
  static constexpr int kRow = ENTRY_BYTES * COPIES;
  static constexpr int kShift = __builtin_ctz(kRow);
};
constexpr int kPairCopies = 16;   // 8-byte entries: 16 lanes x 2 banks per pass
constexpr int kSignCopies = 8;    // 16-byte entries: 8 lanes x 4 banks per pass
using PairTab = Striped<8, kPairCopies>;
using SignTab = Striped<16, kSignCopies>;

// Split widths: record words a lane reads for its 16 wide / 16 narrow key
// codes (16 w bits from a 16-bit boundary: two words once they may cross one)
// and for its 4 wide / 4 narrow value codes (4 w bits: two words for w = 3).
constexpr int split_key_words(int w) { return w > 2 ? 2 : 1; }
constexpr int split_val_words(int w) { return w == 3 ? 2 : 1; }
// Words of a lane's key codes per token (kKeyWords) and of its value fields
// per token (kValWords); split widths: the wide codes' words, then the narrow ones'.
template <int KB, bool SPL>
constexpr int kKeyWords = SPL ? split_key_words(KB + 1) + split_key_words(KB) : KB;
template <int VB, bool SPL>
constexpr int kValWords = SPL ? split_val_words(VB + 1) + split_val_words(VB) : (VB == 3 ? 2 : 1);

// (hi:lo) = the NW words at w, shifted right by sh bits (sh < 32).
template <int NW>
__device__ __forceinline__ void funnel(const uint32_t *w, int sh, uint32_t &lo, uint32_t &hi) {
  if constexpr (NW == 1) {
    lo = w[0] >> sh;
    hi = 0u;
  } else {
    lo = __builtin_amdgcn_alignbit(w[1], w[0], sh);
    hi = w[1] >> sh;
  }
}

// One wave's share of a 32-token tile: its records, loaded one tile ahead.
template <int KB, int VB, bool QJL, bool SC, bool SPL> struct Tile {
  uint32_t kc[2][kKeyWords<KB, SPL>];   // key code words of token n of each half
  uint32_t sg[2];              // sign word kq of token n of each half
  float knu[4], gam[4];        // tokens 4 kq + e of the lane's own half (columns 0..7: the first)
  uint32_t vf[SC ? 1 : 8][kValWords<VB, SPL>];   // value words holding the lane's coordinates of tokens T(i)
  float vnu[SC ? 1 : 4];       // value norms of the lane's own half's tokens
};

// Split widths: first record word and bit shift of a lane's key codes (wide:
// coordinates 16 kq .., narrow: 64 + 16 kq ..) and of its value fields (wide:
// coordinates 4 n .. 4 n + 3, narrow: 64 + 4 n ..) in a record of
// split_code_words(b') words.
template <int B> struct SplitRec {
  static constexpr int W = B + 1, N = B, CW = split_code_words(B);
  static constexpr int key_wide_bit(int kq) { return 16 * kq * W; }
  static constexpr int key_narrow_bit(int kq) { return 64 * W + 16 * kq * N; }
  static constexpr int val_wide_bit(int n) { return 4 * n * W; }
  static constexpr int val_narrow_bit(int n) { return 64 * W + 4 * n * N; }
};

// Token T(i) of the lane's value fields: 4 kq + (i & 3) of half i >> 2.
// One code path for every tile (the compiler's wait counts then stay exact
// across iterations): token indices are clamped to the row's last cached
// token (tiles past seq_len are masked when used), byte offsets are 32-bit
// on a uniform row base, and the norms come four at a time (the row length
// is a multiple of 4 and the norm arrays 16-byte aligned on this path).
// PART selects what is loaded: the key side (bit 0: codes, signs, norms,
// residual norms) and / or the value side (bit 1: value fields and norms).
template <int PART, int KB, int VB, bool QJL, bool SC, bool SPL>
__device__ __forceinline__ void load_tile(const DecodeArgs &a, int64_t row0, int tb, int n, int kq, bool lo_col,
                                          Tile<KB, VB, QJL, SC, SPL> &r) {
  // words per record
  constexpr int KW = SPL ? split_code_words(KB) : 4 * KB;
  constexpr int VW = SPL ? split_code_words(VB) : 4 * VB;
  const int last = static_cast<int>(a.t_cap) - 1;
  const unsigned char *kbase = reinterpret_cast<const unsigned char *>(a.k_codes + row0 * KW);
  // four consecutive tokens 4 kq .. 4 kq + 3 of the lane's own half (aligned
  // to 4; a group past the row's end repeats its last group, masked later)
  const uint32_t t4 = static_cast<uint32_t>(min(tb + 16 * (lo_col ? 1 : 0) + 4 * kq, last - 3)) * 4u;
#pragma unroll
  for (int hf = 0; hf < 2 && (PART & 1); ++hf) {
    const uint32_t tk = static_cast<uint32_t>(min(tb + 16 * hf + n, last));
    if constexpr (SPL) {
      // the lane's 16 W wide bits lie within words w0, w0 + 1 (the second
      // only read when they can reach it), its 16 N narrow bits likewise;
      // every word read lies inside the record
      using R = SplitRec<KB>;
      constexpr int NWW = split_key_words(R::W), NWN = split_key_words(R::N);
      const uint32_t kw = static_cast<uint32_t>(R::key_wide_bit(kq) >> 5);
      const uint32_t kn = static_cast<uint32_t>(R::key_narrow_bit(kq) >> 5);
      const unsigned char *rec = kbase + tk * (KW * 4u);
#pragma unroll
      for (int w = 0; w < NWW; ++w) r.kc[hf][w] = *reinterpret_cast<const uint32_t *>(rec + 4 * (kw + w));
#pragma unroll
      for (int w = 0; w < NWN; ++w) r.kc[hf][NWW + w] = *reinterpret_cast<const uint32_t *>(rec + 4 * (kn + w));
    } else {
      const uint32_t ko = (tk * (4 * KB) + kq * KB) * 4u;
#pragma unroll
      for (int w = 0; w < KB; ++w) r.kc[hf][w] = *reinterpret_cast<const uint32_t *>(kbase + 4 * w + ko);
    }
    if constexpr (QJL)
      r.sg[hf] = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const unsigned char *>(a.k_signs + row0 * 4) +
                                                     (tk * 4u + kq) * 4u);
  }
  if constexpr ((PART & 1) != 0) {
    const float4 nv = *reinterpret_cast<const float4 *>(reinterpret_cast<const unsigned char *>(a.k_norms + row0) + t4);
    r.knu[0] = nv.x; r.knu[1] = nv.y; r.knu[2] = nv.z; r.knu[3] = nv.w;
    if constexpr (QJL) {
      const float4 gv = *reinterpret_cast<const float4 *>(reinterpret_cast<const unsigned char *>(a.k_res + row0) + t4);
      r.gam[0] = gv.x; r.gam[1] = gv.y; r.gam[2] = gv.z; r.gam[3] = gv.w;
    }
  }
  if constexpr (!SC && (PART & 2) != 0) {
    const unsigned char *vbase = reinterpret_cast<const unsigned char *>(a.v_codes + row0 * VW);
    // first tokens of the lane's two groups of four (4 kq .. + 3 of each
    // half); t_cap is a multiple of 4, so a group lies wholly inside the row
    // or wholly past it (then it repeats the row's last group, masked later)
    const int tg0 = min(tb + 4 * kq, last - 3), tg1 = min(tb + 16 + 4 * kq, last - 3);
    if constexpr (SPL) {
      // wide field: 4 W bits from word vw, narrow: 4 N bits from word vn; a
      // 3-bit field may straddle into the next word (read when inside the record)
      using R = SplitRec<VB>;
      constexpr int NWW = split_val_words(R::W), NWN = split_val_words(R::N);
      const int vw = R::val_wide_bit(n) >> 5, vn = R::val_narrow_bit(n) >> 5;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t tv = static_cast<uint32_t>((i < 4 ? tg0 : tg1) + (i & 3));
        const unsigned char *rec = vbase + tv * (VW * 4u);
        r.vf[i][0] = *reinterpret_cast<const uint32_t *>(rec + 4 * vw);
        if constexpr (NWW == 2) r.vf[i][1] = *reinterpret_cast<const uint32_t *>(rec + 4 * vw + 4);
        r.vf[i][NWW] = *reinterpret_cast<const uint32_t *>(rec + 4 * vn);
        if constexpr (NWN == 2) r.vf[i][NWW + 1] = (vn + 1 < VW) ? *reinterpret_cast<const uint32_t *>(rec + 4 * vn + 4) : 0u;
      }
    } else {
      const int w0 = (8 * n * VB) >> 5;   // first word of the lane's value field
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t tv = static_cast<uint32_t>((i < 4 ? tg0 : tg1) + (i & 3));
        const uint32_t vo = (tv * VW + w0) * 4u;
        r.vf[i][0] = *reinterpret_cast<const uint32_t *>(vbase + vo);
        if constexpr (VB == 3) r.vf[i][1] = (w0 + 1 < VW) ? *reinterpret_cast<const uint32_t *>(vbase + vo + 4) : 0u;
      }
    }
    const float4 vv = *reinterpret_cast<const float4 *>(reinterpret_cast<const unsigned char *>(a.v_norms + row0) + t4);
    r.vnu[0] = vv.x; r.vnu[1] = vv.y; r.vnu[2] = vv.z; r.vnu[3] = vv.w;
  }
}

// The 8 b'-bit field of coordinates 8 n .. 8 n + 7 of one token.
template <int VB>
__device__ __forceinline__ uint32_t value_field(const uint32_t (&w)[VB == 3 ? 2 : 1], int n) {
  const int sh = (8 * n * VB) & 31;
  if constexpr (VB == 4) return w[0];
  if constexpr (VB == 3) return __builtin_amdgcn_alignbit(w[1], w[0], sh) & 0xFFFFFFu;
  if constexpr (VB == 2) return (w[0] >> sh) & 0xFFFFu;
  return (w[0] >> sh) & 0xFFu;
}

// Even-indexed codes of an 8-code field (VB bits each), kept in place.
template <int VB> struct EvenMask;
template <> struct EvenMask<1> { static constexpr uint32_t v = 0x55u; };
template <> struct EvenMask<2> { static constexpr uint32_t v = 0x3333u; };
template <> struct EvenMask<3> { static constexpr uint32_t v = 0x1C71C7u; };
template <> struct EvenMask<4> { static constexpr uint32_t v = 0x0F0F0F0Fu; };

// Bits [bit, bit + WIDTH) of the 64-bit value (hi:lo); bit and WIDTH known at
// compile time after unrolling.
template <int WIDTH>
__device__ __forceinline__ uint32_t bits_at(uint32_t lo, uint32_t hi, int bit) {
  constexpr uint32_t kMask = (1u << WIDTH) - 1u;
  if (bit >= 32) return (hi >> (bit - 32)) & kMask;
  if (bit + WIDTH <= 32) return (lo >> bit) & kMask;
  return __builtin_amdgcn_alignbit(hi, lo, bit) & kMask;
}

template <int KB, int VB, bool QJL, bool SC, bool SPL>
__global__ __launch_bounds__(kThreads) void mdecode_kernel(DecodeArgs a) {
  // 1- and 2-bit key codes (uniform widths, with the value sum): one 16-byte
  // lookup per k-step, a table of code quads (four coordinates' (hi, lo)
  // operands); otherwise two lookups per k-step into the table of code pairs
  // (the scores-only kernel keeps the smaller table: two work-groups per CU)
  constexpr bool kQuad = KB <= 2 && !SPL && !SC;
  constexpr int kKeyEntries = kQuad ? 1 : 1 << (2 * KB);
  constexpr int kQuadEntries = kQuad ? 1 << (4 * KB) : 1;
  constexpr int kValEntries = SC ? 1 : 1 << (2 * VB);
  // split widths: the wide codebooks' tables (b' + 1 bits)
  constexpr int kKeyEntriesW = SPL ? 1 << (2 * KB + 2) : 1;
  constexpr int kValEntriesW = (SPL && !SC) ? 1 << (2 * VB + 2) : 1;
  struct Smem {
    alignas(16) unsigned char ktab[kKeyEntries * PairTab::kRow];
    alignas(16) unsigned char qtab[kQuadEntries * SignTab::kRow];
    alignas(16) unsigned char vtab[kValEntries * PairTab::kRow];
    alignas(16) unsigned char ktab_w[kKeyEntriesW * PairTab::kRow];
    alignas(16) unsigned char vtab_w[kValEntriesW * PairTab::kRow];
    alignas(16) unsigned char stab[QJL ? 256 * SignTab::kRow : 16];
    union {
      struct {
        // fp16 hi / lo of the g scaled queries, [head][coordinate]: the B
        // operands of the prologue's products (rows of D + 8: the 8 heads'
        // 16-byte reads of one k-step spread over the banks), and each head's
        // power of two
        alignas(16) uint16_t xh[8][D + 8];
        alignas(16) uint16_t xl[8][D + 8];
        int xexp[8];
        float qt[8][D];                // q~ (scaled), [head][coordinate]
        float st[8][D];                // s (scaled)
        int fexp[8][2];                // per head: the fp16 operands' power-of-two scales
      } pro;
      struct {
        // each wave's rotated sum, weighted by its max: coordinate c of head h
        // at [c / 32][h][c % 32] (rows of 33 words: the 32 lanes that store
        // one register, (h, c / 32) = (lane % 8, lane / 16), hit 32 banks)
        float o[kWaves][4][8][33];
      } epi;
      struct {
        float ot[8][D];          // the work-group's rotated sum
        float red[4][8][D];      // quarter products of Pi_v^T
      } inv;
    } u;
    float ml[kWaves][8][2];
  };
  __shared__ Smem sm;

  const int chunk_id = blockIdx.x;
  const int hk = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, kq = lane >> 4;
  const bool lo_col = n >= 8;
  const int hcol = n & 7;                  // the head of this lane's column
  const int G = a.n_q_heads / a.n_kv_heads;
  const bool live_col = hcol < G;
  const int row_id = b * a.n_kv_heads + hk;
  const int group_id = row_id * a.n_chunks + chunk_id;
  const int64_t row0 = static_cast<int64_t>(row_id) * a.t_cap;
  int T = a.seq_len[b] + a.seq_add;
  T = T < 0 ? 0 : (T > a.t_cap ? static_cast<int>(a.t_cap) : T);
  const int t_begin = chunk_id * a.chunk;
  const int t_end = min(T, t_begin + a.chunk);

  Tile<KB, VB, QJL, SC, SPL> ta{};
  const int t0 = t_begin + wave * kTile;

  // ------------------------------------------------------------ prologue
  // Striped copies of the codebooks' tables (key code pairs -> fp16 (hi, lo)
  // of 256 c per code, pairs of tokens' value codes -> bf16 (hi, lo) of c per
  // token, sign bytes -> eight fp16 +-1).  The tables sit in L2; they are
  // filled before the wave's first tile is requested, since a wait for one
  // load also waits for every load issued before it.
  {
    auto fill_pairs = [&](unsigned char *dst, const void *src, int entries) {
      const uint2 *t = reinterpret_cast<const uint2 *>(src);
      for (int i = tid; i < entries * PairTab::kCopies; i += kThreads)
        *reinterpret_cast<uint2 *>(dst + (i / PairTab::kCopies) * PairTab::kRow + (i % PairTab::kCopies) * 8) =
            t[i / PairTab::kCopies];
    };
    if constexpr (kQuad) {
      // quad q = codes (q & m, q >> 2 KB): the pair entries of its two halves
      const uint2 *t = reinterpret_cast<const uint2 *>(a.mk_lut);
      constexpr int kPairMask = (1 << (2 * KB)) - 1;
      for (int i = tid; i < kQuadEntries * SignTab::kCopies; i += kThreads) {
        const int q = i / SignTab::kCopies;
        const uint2 lo = t[q & kPairMask], hi = t[q >> (2 * KB)];
        *reinterpret_cast<uint4 *>(sm.qtab + q * SignTab::kRow + (i % SignTab::kCopies) * 16) =
            make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
    } else {
      fill_pairs(sm.ktab, a.mk_lut, kKeyEntries);
    }
    if constexpr (SPL) fill_pairs(sm.ktab_w, a.mk_lut_w, kKeyEntriesW);
    if constexpr (!SC) {
      fill_pairs(sm.vtab, a.mv_lut, kValEntries);
      if constexpr (SPL) fill_pairs(sm.vtab_w, a.mv_lut_w, kValEntriesW);
    }
    if constexpr (QJL) {
      const uint4 *st = reinterpret_cast<const uint4 *>(a.sg_lut);
      for (int i = tid; i < 256 * SignTab::kCopies; i += kThreads)
        *reinterpret_cast<uint4 *>(sm.stab + (i / SignTab::kCopies) * SignTab::kRow + (i % SignTab::kCopies) * 16) =
            st[i / SignTab::kCopies];
    }
  }
  // q~ = Pi_k q and s = S Pi_k q of the g heads on the matrix cores
  // (v_mfma_f32_16x16x32_f16), from the codebook's fp16 hi/lo fragments of
  // 2^kDecFragExp Pi_k and 2^kDecFragExp S Pi_k in the encode's layout: wave
  // t takes output block t of both, whose lane (n, kq) receives coordinate
  // enc_coord(kq, t, e) of q~ (32 kq + 4 t + e of s) for head n (B columns
  // 8..15 are zero).  B element e of k-step ks is query coordinate 32 kq +
  // 8 ks + e, as fp16 hi/lo of 2^xe q with a per-head power of two xe that
  // brings the largest |q| into [64, 128) (a bf16 query has no lo part).  The
  // passes hi*hi + lo*hi (+ hi*lo for fp32 queries) keep 22 significant bits
  // of either operand.  The fragments and the queries are requested first,
  // then the wave's first tile, whose HBM latency the products hide.
  {
    const bool in_mm = wave < 8;   // wave-uniform: wave h < 8 also reads head h's query
    f16x8 ph[4], pl[4], fsh[QJL ? 4 : 1], fsl[QJL ? 4 : 1];
    float q0 = 0.f, q1 = 0.f;
    if (in_mm) {
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
      if (wave < G) {   // lane l: coordinates 2 l, 2 l + 1
        const int64_t qi = (static_cast<int64_t>(b) * a.n_q_heads + hk * G + wave) * D + 2 * lane;
        q0 = load_query(a.q, a.q_bf16, qi);
        q1 = load_query(a.q, a.q_bf16, qi + 1);
      }
    }
    if (t0 < t_end) load_tile<3, KB, VB, QJL, SC, SPL>(a, row0, t0, n, kq, lo_col, ta);
    if (in_mm) {
      float mx = fmaxf(fabsf(q0), fabsf(q1));
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      int ex = 0;
      (void)frexpf(mx, &ex);
      const int xe = (mx > 0.f && mx < INFINITY) ? 7 - ex : 0;
      const float y0 = ldexpf(q0, xe), y1 = ldexpf(q1, xe);
      *reinterpret_cast<uint32_t *>(&sm.u.pro.xh[wave][2 * lane]) = split_f16(y0, y1, false);
      *reinterpret_cast<uint32_t *>(&sm.u.pro.xl[wave][2 * lane]) = split_f16(y0, y1, true);
      if (lane == 0) sm.u.pro.xexp[wave] = xe;
    }
    if constexpr (!QJL) {
      for (int e = tid; e < 8 * D; e += kThreads) sm.u.pro.st[e / D][e % D] = 0.f;
    }
    __syncthreads();
    // scaled by scale * log2 e (the sign term also by sqrt(pi/2)/m); heads past g are zero
    const float qsc = a.scale * kLog2e, ssc = a.scale * kLog2e * a.qjl_coef;
    if (in_mm) {
      const bool q_f32 = a.q_bf16 == 0;
      const f16x8 zero8 = as_f16x8(0u, 0u, 0u, 0u);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acs = acc;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int xo = 32 * kq + 8 * ks;
        const f16x8 bh = lo_col ? zero8 : *reinterpret_cast<const f16x8 *>(&sm.u.pro.xh[hcol][xo]);
        acc = mfma_f16(ph[ks], bh, acc);
        acc = mfma_f16(pl[ks], bh, acc);
        if constexpr (QJL) {
          acs = mfma_f16(fsh[ks], bh, acs);
          acs = mfma_f16(fsl[ks], bh, acs);
        }
        if (q_f32) {
          const f16x8 bl = lo_col ? zero8 : *reinterpret_cast<const f16x8 *>(&sm.u.pro.xl[hcol][xo]);
          acc = mfma_f16(ph[ks], bl, acc);
          if constexpr (QJL) acs = mfma_f16(fsh[ks], bl, acs);
        }
      }
      if (!lo_col) {
        const bool live = hcol < G;
        const float un = ldexpf(1.f, -(kDecFragExp + sm.u.pro.xexp[hcol]));   // the operands' scales
        const float kq_ = un * qsc, ks_ = un * ssc;
        const int c = enc_coord(SPL, kq, wave, 0);   // q~ coordinates c .. c + 3
        *reinterpret_cast<float4 *>(&sm.u.pro.qt[hcol][c]) =
            live ? make_float4(acc[0] * kq_, acc[1] * kq_, acc[2] * kq_, acc[3] * kq_) : make_float4(0.f, 0.f, 0.f, 0.f);
        if constexpr (QJL) {
          *reinterpret_cast<float4 *>(&sm.u.pro.st[hcol][32 * kq + 4 * wave]) =
              live ? make_float4(acs[0] * ks_, acs[1] * ks_, acs[2] * ks_, acs[3] * ks_) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
    }
    __syncthreads();
    // per head, a power of two that brings the largest |q~| (and |s|) into
    // [64, 128): the fp16 operands then keep full precision and cannot overflow
    if (wave < 8) {
      const int h = wave;   // one wave per head slot
      float mq = fmaxf(fabsf(sm.u.pro.qt[h][lane]), fabsf(sm.u.pro.qt[h][lane + 64]));
      float ms = fmaxf(fabsf(sm.u.pro.st[h][lane]), fabsf(sm.u.pro.st[h][lane + 64]));
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        mq = fmaxf(mq, __shfl_xor(mq, off));
        ms = fmaxf(ms, __shfl_xor(ms, off));
      }
      if (lane == 0) {
        int eq = 0, es = 0;
        (void)frexpf(mq, &eq);
        (void)frexpf(ms, &es);
        sm.u.pro.fexp[h][0] = (mq > 0.f && mq < INFINITY) ? 7 - eq : 0;
        sm.u.pro.fexp[h][1] = (ms > 0.f && ms < INFINITY) ? 7 - es : 0;
      }
    }
  }
  __syncthreads();
  // The scores' B operands, column n: the query part of head n % 8 times
  // 2^fexp (fp16 hi part in columns 0..7, lo part in 8..15, zero for columns
  // past g).  Key product, k-step s: K-element pair i carries coordinate
  // 32 kq + 4 s + i (split widths: 64 (s / 4) + 16 kq + 4 (s % 4) + i) twice
  // (the key operand holds its (hi, lo) parts); sign product, k-step s:
  // QJL coordinates 32 kq + 8 s .. + 7 once.  The products
  // come out scaled by 2^fexp_q * kKeyScale (key term) and 2^fexp_s (sign
  // term): undone per lane below.
  f16x8 qop[8], sop[QJL ? 4 : 1];
  const int eq = sm.u.pro.fexp[hcol][0], es = sm.u.pro.fexp[hcol][1];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    uint32_t wq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = SPL ? 64 * (s >> 2) + 16 * kq + 4 * (s & 3) + i : 32 * kq + 4 * s + i;
      const float x = ldexpf(sm.u.pro.qt[hcol][c], eq);
      wq[i] = split_f16(x, x, lo_col);
    }
    qop[s] = as_f16x8(wq[0], wq[1], wq[2], wq[3]);
  }
  if constexpr (QJL) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t ws[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int c = 32 * kq + 8 * s + 2 * p;
        ws[p] = split_f16(ldexpf(sm.u.pro.st[hcol][c], es), ldexpf(sm.u.pro.st[hcol][c + 1], es), lo_col);
      }
      sop[s] = as_f16x8(ws[0], ws[1], ws[2], ws[3]);
    }
  }
  // l2 = nu * (key term + gamma * sign term) with the operand scales undone:
  // key products carry 2^eq * kKeyScale, sign products 2^es
  const float inv_k = ldexpf(1.f / kKeyScale, -eq);
  const float rat_s = ldexpf(kKeyScale, eq - es);   // sign term in key-product units

  // ------------------------------------------------------------ main loop
  float m_run = -INFINITY;   // this head's running max (log2 units), equal in all its lanes
  float l_lane = 0.f;        // sum of this lane's weights
  f32x4 oacc[8];
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) oacc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint32_t lane_p = 8u * (n % PairTab::kCopies);   // this lane's copy in the pair tables
  const uint32_t lane_s = 16u * (n % SignTab::kCopies);  // and in the sign table
  // split widths: bit offsets of the lane's key codes and value fields within
  // the first word load_tile reads for them
  const int sh_kw = SPL ? SplitRec<KB>::key_wide_bit(kq) & 31 : 0;
  const int sh_kn = SPL ? SplitRec<KB>::key_narrow_bit(kq) & 31 : 0;
  const int sh_vw = (SPL && !SC) ? SplitRec<VB>::val_wide_bit(n) & 31 : 0;
  const int sh_vn = (SPL && !SC) ? SplitRec<VB>::val_narrow_bit(n) & 31 : 0;

  // One tile: scores (key and sign products), online softmax, value product.
  // Scores of one tile: l2[e] = the score (log2 units) of token 4 kq + e of
  // the lane's own half, -inf past the row's end; written out when asked.
  auto score_tile = [&](const Tile<KB, VB, QJL, SC, SPL> &cur, int tb, float (&l2)[4]) {
    const bool full = tb + kTile <= t_end;
    // ---- scores C[token 4 kq + e][column n] of both halves.  K-element
    // pair i of k-step s is (hi, lo) of coordinate 32 kq + 4 s + i (keys), or
    // signs 32 kq + 8 s + 2 i, + 1 (sign term).
    f32x4 sacc[2], tacc[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      sacc[hf] = f32x4{0.f, 0.f, 0.f, 0.f};
      tacc[hf] = sacc[hf];
      // split widths: the lane's 16 wide codes (bits of kw1:kw0) and 16
      // narrow codes (kn1:kn0), shifted to bit 0
      uint32_t kw0 = 0, kw1 = 0, kn0 = 0, kn1 = 0;
      if constexpr (SPL) {
        constexpr int NWW = split_key_words(KB + 1);
        funnel<NWW>(&cur.kc[hf][0], sh_kw, kw0, kw1);
        funnel<split_key_words(KB)>(&cur.kc[hf][NWW], sh_kn, kn0, kn1);
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        if constexpr (kQuad) {
          // quad s: bits [4 KB s, 4 KB s + 4 KB) of the lane's codes (within one word)
          constexpr int kBits = 4 * KB;
          const int bit = kBits * s, w = bit >> 5, sh = bit & 31;
          const uint32_t idx = (cur.kc[hf][w] >> sh) & ((1u << kBits) - 1u);
          const uint4 e = *reinterpret_cast<const uint4 *>(sm.qtab + (idx << SignTab::kShift) + lane_s);
          sacc[hf] = mfma_f16(as_f16x8(e.x, e.y, e.z, e.w), qop[s], sacc[hf]);
          continue;
        }
        uint32_t ka[2];
        const bool wide = SPL && s < 4;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          uint32_t idx;
          if constexpr (SPL) {
            // pair q of the step's width: bits [2 w q, 2 w q + 2 w)
            const int q = 2 * (s & 3) + p;
            idx = wide ? bits_at<2 * KB + 2>(kw0, kw1, (2 * KB + 2) * q) : bits_at<2 * KB>(kn0, kn1, 2 * KB * q);
          } else {
            // pair q = 2 s + p: bits [2 KB q, 2 KB q + 2 KB) of the lane's codes
            constexpr int kMask = (1 << (2 * KB)) - 1;
            const int bit = 2 * KB * (2 * s + p), w = bit >> 5, sh = bit & 31;
            if (sh + 2 * KB <= 32) {
              idx = (cur.kc[hf][w] >> sh) & kMask;
            } else {
              idx = __builtin_amdgcn_alignbit(cur.kc[hf][w + 1], cur.kc[hf][w], sh) & kMask;
            }
          }
          ka[p] = (idx << PairTab::kShift) + lane_p;
        }
        const unsigned char *kt = wide ? sm.ktab_w : sm.ktab;
        const uint2 e0 = *reinterpret_cast<const uint2 *>(kt + ka[0]);
        const uint2 e1 = *reinterpret_cast<const uint2 *>(kt + ka[1]);
        sacc[hf] = mfma_f16(as_f16x8(e0.x, e0.y, e1.x, e1.y), qop[s], sacc[hf]);
      }
      if constexpr (QJL) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint32_t by = (cur.sg[hf] >> (8 * s)) & 255u;
          const uint4 z = *reinterpret_cast<const uint4 *>(sm.stab + (by << SignTab::kShift) + lane_s);
          tacc[hf] = mfma_f16(as_f16x8(z.x, z.y, z.z, z.w), sop[s], tacc[hf]);
        }
      }
    }
    // ---- the head's full score: its two columns summed across lanes n and
    // n ^ 8; lanes of columns 0..7 keep the first half's tokens, 8..15 the second's
    const int tk0 = tb + 16 * (lo_col ? 1 : 0) + 4 * kq;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float y = (lo_col ? sacc[1][e] : sacc[0][e]) + swap8(lo_col ? sacc[0][e] : sacc[1][e]);
      if constexpr (QJL) {
        const float yt = (lo_col ? tacc[1][e] : tacc[0][e]) + swap8(lo_col ? tacc[0][e] : tacc[1][e]);
        y = fmaf(cur.gam[e] * rat_s, yt, y);
      }
      l2[e] = (full || tk0 + e < t_end) ? (cur.knu[e] * inv_k) * y : -INFINITY;
    }
    if (SC || a.scores != nullptr) {
      if (live_col) {
        float *sp = a.scores + (static_cast<int64_t>(b) * a.n_q_heads + hk * G + hcol) * a.t_cap;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (full || tk0 + e < t_end) sp[tk0 + e] = l2[e] * kLn2;
      }
    }
  };

  // Online softmax of one tile's scores and its value products.
  auto value_tile = [&](const Tile<KB, VB, QJL, SC, SPL> &cur, const float (&l2)[4], int tb) {
    const bool full = tb + kTile <= t_end;
    const int tk0 = tb + 16 * (lo_col ? 1 : 0) + 4 * kq;
    if constexpr (!SC) {
      // ---- online softmax, running max raised lazily (wave-uniform decision)
      const float tmax = fmaxf(fmaxf(l2[0], l2[1]), fmaxf(l2[2], l2[3]));
      if (__any(tmax > m_run + kLazy2)) {
        float hm = fmaxf(tmax, swap8(tmax));
        hm = fmaxf(hm, __shfl_xor(hm, 16));
        hm = fmaxf(hm, __shfl_xor(hm, 32));
        const float m_new = fmaxf(m_run, hm);
        const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_lane *= alpha;
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) oacc[cb] *= alpha;
      }
      float w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool valid = full || tk0 + e < t_end;
        const float p = valid ? __builtin_amdgcn_exp2f(l2[e] - m_run) : 0.f;
        l_lane += p;
        w[e] = valid ? p * cur.vnu[e] : 0.f;
      }
      // B operands of the value products, one per half: K-element pair i =
      // token 4 kq + i of that half, the weight's hi part (columns 0..7) or lo
      // part (8..15) twice.  A lane holds its own half's weights; the other
      // half's part comes from lane n ^ 8.
      const uint32_t h01 = pack_bf16(w[0], w[1]), h23 = pack_bf16(w[2], w[3]);
      const uint32_t l01 = pack_bf16(w[0] - __uint_as_float(h01 << 16), w[1] - __uint_as_float(h01 & 0xffff0000u));
      const uint32_t l23 = pack_bf16(w[2] - __uint_as_float(h23 << 16), w[3] - __uint_as_float(h23 & 0xffff0000u));
      const uint32_t own01 = lo_col ? l01 : h01, own23 = lo_col ? l23 : h23;
      const uint32_t r01 = swap8u(lo_col ? h01 : l01), r23 = swap8u(lo_col ? h23 : l23);
      bf16x8 pb[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const bool mine = (hf == 1) == lo_col;
        const uint32_t p01 = mine ? own01 : r01, p23 = mine ? own23 : r23;
        pb[hf] = as_bf16x8(__builtin_amdgcn_perm(p01, p01, 0x01000100u), __builtin_amdgcn_perm(p01, p01, 0x03020302u),
                           __builtin_amdgcn_perm(p23, p23, 0x01000100u), __builtin_amdgcn_perm(p23, p23, 0x03020302u));
      }
      // ---- value sum: block cb, row n = coordinate 8 n + cb (split widths:
      // 4 n + cb wide, 64 + 4 n + cb - 4 narrow); K-element pair i = (hi, lo)
      // of token 4 kq + i of the half
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        if constexpr (SPL) {
          // per width: the 4 codes of the lane's coordinates of tokens
          // (2 pp, 2 pp + 1), paired per coordinate as in the uniform case
          constexpr int W = VB + 1, N = VB, NWW = split_val_words(W), NWN = split_val_words(N);
          constexpr uint32_t MW = EvenMask<W>::v & ((1u << (4 * W)) - 1u);
          constexpr uint32_t MN = EvenMask<N>::v & ((1u << (4 * N)) - 1u);
          uint32_t EW[2], OW[2], EN[2], ON[2];
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            const uint32_t *v0 = cur.vf[4 * hf + 2 * pp];
            const uint32_t *v1 = cur.vf[4 * hf + 2 * pp + 1];
            uint32_t w0, w1, n0, n1, hi;
            funnel<NWW>(v0, sh_vw, w0, hi);
            funnel<NWW>(v1, sh_vw, w1, hi);
            funnel<NWN>(v0 + NWW, sh_vn, n0, hi);
            funnel<NWN>(v1 + NWW, sh_vn, n1, hi);
            w0 &= (1u << (4 * W)) - 1u;
            w1 &= (1u << (4 * W)) - 1u;
            n0 &= (1u << (4 * N)) - 1u;
            n1 &= (1u << (4 * N)) - 1u;
            EW[pp] = (w0 & MW) | ((w1 & MW) << W);
            OW[pp] = ((w0 >> W) & MW) | (w1 & (MW << W));
            EN[pp] = (n0 & MN) | ((n1 & MN) << N);
            ON[pp] = ((n0 >> N) & MN) | (n1 & (MN << N));
          }
#pragma unroll
          for (int cb = 0; cb < 8; ++cb) {
            const bool wide = cb < 4;
            const int c = cb & 3;
            const int width = wide ? W : N;
            const uint32_t mask = (1u << (2 * width)) - 1u;
            const int sh = 2 * width * (c >> 1);
            const uint32_t s0 = wide ? ((c & 1) ? OW[0] : EW[0]) : ((c & 1) ? ON[0] : EN[0]);
            const uint32_t s1 = wide ? ((c & 1) ? OW[1] : EW[1]) : ((c & 1) ? ON[1] : EN[1]);
            const uint32_t i0 = (s0 >> sh) & mask, i1 = (s1 >> sh) & mask;
            const unsigned char *vt = wide ? sm.vtab_w : sm.vtab;
            const uint2 e0 = *reinterpret_cast<const uint2 *>(vt + (i0 << PairTab::kShift) + lane_p);
            const uint2 e1 = *reinterpret_cast<const uint2 *>(vt + (i1 << PairTab::kShift) + lane_p);
            oacc[cb] = mfma(as_bf16x8(e0.x, e0.y, e1.x, e1.y), pb[hf], oacc[cb]);
          }
        } else {
          uint32_t E[2], O[2];
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            // tokens (2 pp, 2 pp + 1) of the half: the pair index of every
            // coordinate, even coordinates in E, odd ones in O
            constexpr uint32_t M = EvenMask<VB>::v;
            const uint32_t f0 = value_field<VB>(cur.vf[4 * hf + 2 * pp], n);
            const uint32_t f1 = value_field<VB>(cur.vf[4 * hf + 2 * pp + 1], n);
            E[pp] = (f0 & M) | ((f1 & M) << VB);
            O[pp] = ((f0 >> VB) & M) | (f1 & (M << VB));
          }
#pragma unroll
          for (int cb = 0; cb < 8; ++cb) {
            constexpr uint32_t kMask = (1u << (2 * VB)) - 1u;
            const int sh = 2 * VB * (cb >> 1);
            const uint32_t i0 = (((cb & 1) ? O[0] : E[0]) >> sh) & kMask;
            const uint32_t i1 = (((cb & 1) ? O[1] : E[1]) >> sh) & kMask;
            const uint2 e0 = *reinterpret_cast<const uint2 *>(sm.vtab + (i0 << PairTab::kShift) + lane_p);
            const uint2 e1 = *reinterpret_cast<const uint2 *>(sm.vtab + (i1 << PairTab::kShift) + lane_p);
            oacc[cb] = mfma(as_bf16x8(e0.x, e0.y, e1.x, e1.y), pb[hf], oacc[cb]);
          }
        }
      }
    }
  };

  constexpr int kStride = kWaves * kTile;
  Tile<KB, VB, QJL, SC, SPL> tn{};
  if constexpr (SC) {
    // scores only: two key buffers in turn, one scored while the next loads
    for (int tt = t0; tt < t_end; tt += 2 * kStride) {
      float l2[4];
      if (tt + kStride < t_end) load_tile<1, KB, VB, QJL, SC, SPL>(a, row0, tt + kStride, n, kq, lo_col, tn);
      score_tile(ta, tt, l2);
      if (tt + kStride >= t_end) break;
      if (tt + 2 * kStride < t_end) load_tile<1, KB, VB, QJL, SC, SPL>(a, row0, tt + 2 * kStride, n, kq, lo_col, ta);
      score_tile(tn, tt + kStride, l2);
    }
  } else if (t0 < t_end) {
    // Software pipeline over the wave's tiles: the value phase of tile i and
    // the score phase of tile i + 1 are independent and form one basic block
    // (after the softmax's rescale branch), so the lookups and products of one
    // run under the other's.  Buffer ta / tn alternate: while one holds tile
    // i's values and the other tile i + 1's keys, tile i + 1's values and tile
    // i + 2's keys load into the free halves.  Loads past the row's end read
    // its last token (in bounds); their scores are masked to -inf, and the
    // last step scores one such tile that nothing uses.
    //
    // Waves w and w + 4 share a SIMD, whose scheduler issues the older wave
    // first: left alone, one of them finishes its tiles long before the other,
    // which then runs its last tiles with no partner to overlap.  Each wave
    // therefore raises its priority on every other tile, the two in opposite
    // phase, so that they take turns.  (Tiles stay statically assigned, so the
    // result does not depend on the timing.)
    load_tile<1, KB, VB, QJL, SC, SPL>(a, row0, t0 + kStride, n, kq, lo_col, tn);
    float la[4], lb[4];
    score_tile(ta, t0, la);
    int turn = wave >> 2;
    for (int tt = t0;;) {
      if (++turn & 1) __builtin_amdgcn_s_setprio(1); else __builtin_amdgcn_s_setprio(0);
      load_tile<2, KB, VB, QJL, SC, SPL>(a, row0, tt + kStride, n, kq, lo_col, tn);
      load_tile<1, KB, VB, QJL, SC, SPL>(a, row0, tt + 2 * kStride, n, kq, lo_col, ta);
      value_tile(ta, la, tt);
      score_tile(tn, tt + kStride, lb);
      tt += kStride;
      if (tt >= t_end) break;
      if (++turn & 1) __builtin_amdgcn_s_setprio(1); else __builtin_amdgcn_s_setprio(0);
      load_tile<2, KB, VB, QJL, SC, SPL>(a, row0, tt + kStride, n, kq, lo_col, ta);
      load_tile<1, KB, VB, QJL, SC, SPL>(a, row0, tt + 2 * kStride, n, kq, lo_col, tn);
      value_tile(tn, lb, tt);
      score_tile(ta, tt + kStride, la);
      tt += kStride;
      if (tt >= t_end) break;
    }
  }

  if constexpr (SC) return;   // uniform: no barrier follows for any thread
  __builtin_amdgcn_s_setprio(0);

  // ------------------------------------------------------------ merge waves
  // Pi_v^T of the chunk's sum: thread (i4, q4) applies rows 32 q4 .. + 31 of
  // column i4 of Pi_v; requested now so that the merge hides their latency.
  const int i4 = tid & (D - 1), q4 = tid >> 7;
  const bool in_inv = q4 < 4;   // wave-uniform: the first 512 threads
  float pvr[32];
  if (in_inv) {
#pragma unroll
    for (int jj = 0; jj < 32; ++jj) pvr[jj] = a.rot_v[(32 * q4 + jj) * D + i4];
  }
  // the head's sum over its 8 lanes (columns n, n ^ 8 and the four kq)
  float lh = l_lane + swap8(l_lane);
  lh += __shfl_xor(lh, 16);
  lh += __shfl_xor(lh, 32);
  if (lane < 8) {
    sm.ml[wave][lane][0] = m_run;
    sm.ml[wave][lane][1] = lh;
  }
  __syncthreads();
  {
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, sm.ml[w][hcol][0]);
    const float fw = (m_run == -INFINITY) ? 0.f : exp2f(m_run - mx);
    // rows 4 kq + e of block cb are coordinates 8 (4 kq + e) + cb (split
    // widths: 64 (cb / 4) + 4 (4 kq + e) + cb % 4)
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = (oacc[cb][e] + swap8(oacc[cb][e])) * fw;
        const int c = SPL ? 64 * (cb >> 2) + 16 * kq + 4 * e + (cb & 3) : 32 * kq + 8 * e + cb;
        if (!lo_col) sm.u.epi.o[wave][c >> 5][hcol][c & 31] = v;
      }
  }
  __syncthreads();
  {
    constexpr int kPer = (8 * D + kThreads - 1) / kThreads;
    float s[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int e = tid + k * kThreads;   // (head, coordinate)
      float v = 0.f;
      if (e < 8 * D) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) v += sm.u.epi.o[w][(e % D) >> 5][e / D][e & 31];
      }
      s[k] = v;
    }
    __syncthreads();   // every wave's sums are read: the region is reused
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int e = tid + k * kThreads;
      if (e < 8 * D) sm.u.inv.ot[e / D][e % D] = s[k];
    }
  }
  __syncthreads();
  if (in_inv) {
    // heads outermost: one uniform branch per head, its 32 LDS reads issued
    // together (a head test inside the coordinate loop became one branch and
    // one LDS round trip per product)
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      if (h < G) {
        float r = 0.f;
#pragma unroll
        for (int jj = 0; jj < 32; ++jj) r = fmaf(pvr[jj], sm.u.inv.ot[h][32 * q4 + jj], r);
        sm.u.inv.red[q4][h][i4] = r;
      }
    }
  }
  __syncthreads();
  // the chunk's (max, sum) per head, max in natural-log units (the merge's)
  auto chunk_ml = [&](int h, float &mx, float &lsum) {
    mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, sm.ml[w][h][0]);
    lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (sm.ml[w][h][0] != -INFINITY) lsum += sm.ml[w][h][1] * exp2f(sm.ml[w][h][0] - mx);
  };
  if (a.n_chunks == 1 && a.seq_inc == nullptr) {
    for (int e = tid; e < G * D; e += kThreads) {
      const int h = e / D, i = e % D;
      float mx, lsum;
      chunk_ml(h, mx, lsum);
      const float inv = (lsum > 0.f) ? 1.f / lsum : 0.f;
      const float o = fmaf(inv, sm.u.inv.red[0][h][i] + sm.u.inv.red[1][h][i] + sm.u.inv.red[2][h][i] +
                                    sm.u.inv.red[3][h][i], 0.f);
      const int64_t o_idx = (static_cast<int64_t>(b) * a.n_q_heads + hk * G + h) * D + i;
      if (a.out_bf16) {
        static_cast<uint16_t *>(a.out)[o_idx] = f32_to_bf16_rne(o);
      } else {
        static_cast<float *>(a.out)[o_idx] = o;
      }
    }
    return;
  }
  float *part_o = a.ws_part_o + static_cast<int64_t>(group_id) * G * D;
  for (int e = tid; e < G * D; e += kThreads) {
    const int h = e / D, i = e % D;
    part_o[e] = sm.u.inv.red[0][h][i] + sm.u.inv.red[1][h][i] + sm.u.inv.red[2][h][i] + sm.u.inv.red[3][h][i];
  }
  if (tid < G) {
    float mx, lsum;
    chunk_ml(tid, mx, lsum);
    a.ws_part_ml[(static_cast<int64_t>(group_id) * G + tid) * 2 + 0] = mx * kLn2;
    a.ws_part_ml[(static_cast<int64_t>(group_id) * G + tid) * 2 + 1] = lsum;
  }
}

template <int KB, bool QJL, bool SC, bool SPL>
hipError_t launch_v(const DecodeArgs &a, dim3 grid, hipStream_t stream) {
  if constexpr (SC) {
    // scores only: no value table (the VB argument is unused)
    hipLaunchKernelGGL((mdecode_kernel<KB, 4, QJL, true, SPL>), grid, dim3(kThreads), 0, stream, a);
  } else {
    switch (a.v_bits) {
#define TQ_V(VV) \
  case VV: hipLaunchKernelGGL((mdecode_kernel<KB, VV, QJL, false, SPL>), grid, dim3(kThreads), 0, stream, a); break;
      TQ_V(1) TQ_V(2) TQ_V(3)
#undef TQ_V
      case 4:
        if constexpr (SPL) return hipErrorInvalidValue;   // split widths: b' + 1 <= 4
        else hipLaunchKernelGGL((mdecode_kernel<KB, 4, QJL, false, false>), grid, dim3(kThreads), 0, stream, a);
        break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

template <int KB, bool SC, bool SPL>
hipError_t launch_k(const DecodeArgs &a, dim3 grid, hipStream_t stream) {
  return a.qjl_m > 0 ? launch_v<KB, true, SC, SPL>(a, grid, stream) : launch_v<KB, false, SC, SPL>(a, grid, stream);
}

}  // namespace

hipError_t launch_mdecode_main(const DecodeArgs &a, bool scores_only, hipStream_t stream) {
  const int g = a.n_q_heads / a.n_kv_heads;
  if (!mdecode_can_run(a) || a.n_chunks > kMaxDecodeChunks || g < 1 || g > 8 || a.n_kv_heads > 65535 ||
      a.mk_lut == nullptr || a.k_dfrag_rot == nullptr || (a.qjl_m > 0 && (a.k_dfrag_qjl == nullptr || a.sg_lut == nullptr)) ||
      (!scores_only && a.mv_lut == nullptr) || (a.k_split && a.mk_lut_w == nullptr) ||
      (!scores_only && (a.v_split != a.k_split || (a.v_split && a.mv_lut_w == nullptr))))
    return hipErrorInvalidValue;
  const dim3 grid(a.n_chunks, a.n_kv_heads, a.batch);
  if (a.k_split) {
    // split widths (both codebooks): b' + 1 <= 4
    switch (a.k_bits) {
      case 1: return scores_only ? launch_k<1, true, true>(a, grid, stream) : launch_k<1, false, true>(a, grid, stream);
      case 2: return scores_only ? launch_k<2, true, true>(a, grid, stream) : launch_k<2, false, true>(a, grid, stream);
      case 3: return scores_only ? launch_k<3, true, true>(a, grid, stream) : launch_k<3, false, true>(a, grid, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (a.k_bits) {
    case 1: return scores_only ? launch_k<1, true, false>(a, grid, stream) : launch_k<1, false, false>(a, grid, stream);
    case 2: return scores_only ? launch_k<2, true, false>(a, grid, stream) : launch_k<2, false, false>(a, grid, stream);
    case 3: return scores_only ? launch_k<3, true, false>(a, grid, stream) : launch_k<3, false, false>(a, grid, stream);
    case 4: return scores_only ? launch_k<4, true, false>(a, grid, stream) : launch_k<4, false, false>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

bool pack_decode_fragments(const double *mat, void *dst, bool split_rows) {
  // Element (t, s, lane, e) as in pack_encode_fragments: lane % 16 picks output
  // row enc_coord(i / 4, t, i % 4), element e with lane / 16 picks input
  // column 32 (lane / 16) + 8 s + e.
  const double sc = static_cast<double>(1 << kDecFragExp);
  uint16_t *out = static_cast<uint16_t *>(dst);
  for (int i = 0; i < kHeadDim * kHeadDim; ++i)
    if (!(std::fabs(mat[i]) < 128.0)) return false;
  for (int t = 0; t < 8; ++t)
    for (int s = 0; s < 4; ++s)
      for (int lane = 0; lane < 64; ++lane)
        for (int e = 0; e < 8; ++e) {
          const int i = lane & 15, kq = lane >> 4;
          const int row = enc_coord(split_rows, i >> 2, t, i & 3);
          const int col = 32 * kq + 8 * s + e;
          const double v = sc * mat[row * kHeadDim + col];
          const _Float16 hi = static_cast<_Float16>(static_cast<float>(v));
          const _Float16 lo = static_cast<_Float16>(static_cast<float>(v - static_cast<double>(hi)));
          const size_t at = (((static_cast<size_t>(t) * 4 + s) * 64 + lane) * 8) + e;
          out[at] = __builtin_bit_cast(uint16_t, hi);
          out[kFragBytesPerSplit / 2 + at] = __builtin_bit_cast(uint16_t, lo);
        }
  return true;
}

}  // namespace tq
