// Kernel argument blocks and launchers of libtq.so (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace tq {

constexpr int kHeadDim = 128;    // the GPU path's d
constexpr int kQjlDim = 128;     // the GPU path's m for keys
constexpr int kMaxLevels = 16;   // 2^4
// Split widths on the GPU path: rotated coordinates 0..63 take the
// (b' + 1)-bit codebook, 64..127 the b'-bit one; a record holds the 64 wide
// codes (at running offsets) and then the 64 narrow ones.
constexpr int kSplitWide = 64;
constexpr int split_code_words(int b) { return 2 * (2 * b + 1); }

// Rotated coordinate that encode lane group kq (lane / 16) receives as element
// e of output block t: 32 kq + 4 t + e, or with split widths 64 (t / 4) +
// 16 kq + 4 (t % 4) + e, which puts the wide coordinates in blocks 0..3 and
// the narrow ones in 4..7 of every lane.
__host__ __device__ constexpr int enc_coord(bool split, int kq, int t, int e) {
  return split ? 64 * (t >> 2) + 16 * kq + 4 * (t & 3) + e : 32 * kq + 4 * t + e;
}

// Encode operands are bf16 fragments laid out so that each lane of a wave
// reads its 16-byte A operand of v_mfma_f32_16x16x32_bf16 with one LDS load:
// [split hi/lo][m-tile 0..7][k-step 0..3][lane 0..63] x 8 bf16.
constexpr size_t kFragBytesPerSplit = 8 * 4 * 64 * 16;   // 32 KiB
constexpr size_t kFragBytes = 2 * kFragBytesPerSplit;     // hi + lo

// Quantizer cell table: kQuantCells cells over [-1, 1], one float4 entry each
// (see build_quant_cells); the kernel's cell index is one saturating byte
// conversion, so 256 cells.
constexpr int kQuantCells = 256;
constexpr int kQuantCellEntries = kQuantCells;

struct EncodeArgs {
  const void *x;
  int64_t x_stride;        // elements between rows
  int64_t n;
  const int64_t *dst_row;  // may be null
  int64_t cache_rows;
  // Append mode (dst_row null, append_len set): vector i goes to row
  // i * t_cap + append_len[i / append_heads], skipped when that position is
  // outside [0, t_cap).
  const int32_t *append_len;
  int append_heads;
  int64_t t_cap;
  uint32_t *codes;
  uint32_t *signs;
  float *norms;
  float *res_norms;
  float *dbg_rot;
  float *dbg_proj;
  const uint4 *frag_rot;   // kFragBytes
  const uint4 *frag_qjl;   // kFragBytes (keys with QJL): fragments of -S
  const float4 *qlut;      // kQuantCellEntries quantizer cells
  const float4 *qlut_wide; // split widths: the wide codebook's cells (else null)
  float qscale, qbias;     // cell = byte(y * qscale + qbias): round to nearest even, saturated to 0 .. 255, NaN -> 0
};

// Fills `dst` (kFragBytes) with the hi/lo bf16 fragments of the 128 x 128
// row-major matrix `mat` (rows = outputs, columns = inputs).  split_rows puts
// the output rows in the split coordinate order of enc_coord (the rotation's
// outputs are the rotated coordinates); split_cols does so for the input
// columns (S's inputs are the rotated residual's coordinates).  negate packs
// -mat (the QJL matrix: the encode then reads -p, whose sign bit is the sketch).
void pack_encode_fragments(const float *mat, void *dst, bool split_rows, bool split_cols, bool negate);

// The matrix-core decode's query products take fp16 operands: the fragments
// hold fp16 hi and lo of 2^kDecFragExp * mat (128 x 128, row-major, entries
// of magnitude below 2^7 so that the scaled hi part stays finite), with lo
// the rounding of the remainder (22 significant bits in all), in the layout of
// pack_encode_fragments.  split_rows as there; the inputs are the query's
// coordinates in natural order.
constexpr int kDecFragExp = 8;
// False if an entry is too large for the scaled fp16 parts.
bool pack_decode_fragments(const double *mat, void *dst, bool split_rows);

// Builds the quantizer cell table (4 floats per cell); false if the
// thresholds do not fit the cell grid (then the GPU path is unsupported).
bool build_quant_cells(const float *thresholds, const float *centroids, int levels, float *cells,
                       float *qscale, float *qbias);

// Enqueues the encode kernel; returns the launch error (hipSuccess on success).
hipError_t launch_encode(const EncodeArgs &a, int bits, bool qjl, bool x_f32, bool split, int num_cus,
                         hipStream_t stream);
// Keys (ka) and values (va, no QJL) of bf16 rows in one launch, no debug outputs.
hipError_t launch_encode_pair(const EncodeArgs &ka, int kbits, bool kqjl, const EncodeArgs &va, int vbits,
                              int num_cus, hipStream_t stream);

constexpr int kMaxDecodeChunks = 128;   // chunks per (batch, kv head)

// Decode dequantization tables (built once per codebook on the host).
// Key table: one lookup turns kCoords codes into floats:
//   b'=1: 4 bits (4 codes), 16 entries;  b'=2: 8 bits (4 codes), 256 entries;
//   b'=3: 6 bits (2 codes), 64 entries;  b'=4: 8 bits (2 codes), 256 entries.
// Entry e, coordinate c holds centroid[(e >> (c * b')) & (2^b' - 1)].
constexpr int key_lut_bits(int b) { return b == 1 ? 4 : (b == 3 ? 6 : 8); }
constexpr int key_lut_coords(int b) { return key_lut_bits(b) / b; }
constexpr size_t kKeyLutBytes = 256 * 4 * sizeof(float);     // largest key table
// Value pair table: 2^(2b) entries of (centroid[e & m], centroid[(e >> b) & m]).
constexpr size_t kPairLutBytes = 256 * 2 * sizeof(float);

// Operand tables of the matrix-core decode (built once per codebook on the
// host).  Every centroid c is carried as one 32-bit word: its hi part in the
// low half, lo = c - hi in the high half.  Key table: index (code a) | (code
// b) << b', two words: the fp16 parts of 256 c_a, then of 256 c_b.  Value
// table: index (code of token t) | (code of token t') << b', two words: the
// bf16 parts of c_t, then of c_t'.  Sign table: a byte of sign bits -> eight
// fp16 +-1 (set bit +1) in four words.
constexpr size_t kMKeyLutBytes = 256 * 2 * sizeof(uint32_t);   // largest (b' = 4)
constexpr size_t kMValLutBytes = 256 * 2 * sizeof(uint32_t);
constexpr size_t kSignLutBytes = 256 * 4 * sizeof(uint32_t);

struct DecodePlan {
  int chunk;               // tokens per work-group chunk
  int n_chunks;
  size_t off_qslot;        // bytes into the workspace: float[groups][d][g], q~ per work-group (coordinate-major)
  size_t off_part_o;       // float[groups][g][d]: rotated partial outputs
  size_t off_part_ml;      // float[groups][g][2]: running max and sum
  size_t total_bytes;
};

DecodePlan plan_decode(int batch, int n_q_heads, int n_kv_heads, int64_t t_cap);

// Chunk attention: the matrix-core kernel serves n_new * g >= kChunkMfmaRows
// query rows per kv head; fewer go through the decode kernel (one work-group
// per (kv head, query)).
constexpr int kChunkMfmaRows = 16;
inline bool chunk_uses_mfma(int g, int n_new) { return g * n_new >= kChunkMfmaRows; }
DecodePlan plan_chunk_mfma(int batch, int n_q_heads, int n_kv_heads, int n_new, int64_t t_cap);
// The plan tq_chunk_attention runs with (either kind).
DecodePlan plan_chunk(int batch, int n_q_heads, int n_kv_heads, int n_new, int64_t t_cap);

struct DecodeArgs {
  const void *q;
  int q_bf16;
  const uint32_t *k_codes;
  const uint32_t *k_signs;
  const float *k_norms;
  const float *k_res;
  const uint32_t *v_codes;
  const float *v_norms;
  int64_t t_cap;
  const int32_t *seq_len;
  int seq_add;             // tokens attended: clamp(seq_len[b] + seq_add, 0, t_cap)
  int32_t *seq_inc;        // if set: seq_len[b] += 1 after the step when 0 <= seq_len[b] < t_cap
  int batch, n_q_heads, n_kv_heads;
  int n_new;               // queries per (b, q head); query j sits at position seq_len[b] - n_new + j
  int k_bits, v_bits, qjl_m;
  float scale;
  float qjl_coef;          // sqrt(pi/2)/m
  void *out;
  int out_bf16;
  float *scores;           // float[B][Hq][t_cap] scaled logits of t < T; optional for attention, the output of the logits-only kernel
  const float *rot_k_t;    // Pi_k^T row-major (d x d): entry [i][j] = Pi_k[j][i]
  const float *qjl_rot_t;  // (S Pi_k)^T row-major (d x m): s = S Pi_k q in one product
  const uint4 *k_frag_rot; // chunk attention: bf16 hi/lo operand fragments of Pi_k (the encode's layout)
  const uint4 *k_frag_qjl; // and of -S (keys with QJL)
  const uint4 *k_dfrag_rot; // matrix-core decode: fp16 hi/lo fragments of 2^kDecFragExp Pi_k
  const uint4 *k_dfrag_qjl; // and of 2^kDecFragExp S Pi_k (keys with QJL)
  const float *rot_v;      // Pi_v row-major (d x d)
  const float *k_lut;      // key dequantization table (kKeyLutBytes)
  const float *v_lut;      // value pair table (kPairLutBytes)
  const float *k_pair;     // key pair table (kPairLutBytes layout, key codebook)
  const void *mk_lut;          // key operand table of the key codebook
  const void *mv_lut;          // value operand table of the value codebook
  const void *sg_lut;          // sign table
  int k_split, v_split;        // split widths (kSplitWide wide coordinates) of the key / value codebook
  const void *mk_lut_w;        // split keys: the wide codebook's key operand table
  const void *mv_lut_w;        // split values: the wide codebook's value operand table
  int norm_vec4;               // t_cap % 4 == 0 and the norm arrays 16-byte aligned (four norms per load)
  float *ws_qslot;
  float *ws_part_o;        // [B*Hkv][n_chunks][g][d]: rotated back (decode kernel) or rotated (chunk kernel)
  float *ws_part_ml;       // [B*Hkv][n_chunks][g][2]
  int chunk, n_chunks;
};

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
// The matrix-core decode's main launch (n_new = 1): the output for one-chunk
// rows, else the chunks' partials for the merge launch; scores only with
// scores_only (every l_t to a.scores, nothing else).
hipError_t launch_mdecode_main(const DecodeArgs &a, bool scores_only, hipStream_t stream);
// Rows up to this many tokens take the matrix-core decode (its per-lane cache
// offsets are 32-bit byte offsets within a row: 72 bytes per token at most).
constexpr int64_t kMDecodeMaxTcap = (int64_t{1} << 31) / 72;
// Whether the matrix-core decode can read these arguments: single queries
// over rows of a multiple of 4 tokens (up to kMDecodeMaxTcap) with 16-byte
// aligned norm arrays.
inline bool mdecode_can_run(const DecodeArgs &a) {
  return a.n_new == 1 && a.t_cap <= kMDecodeMaxTcap && a.norm_vec4 != 0;
}
// Which decode serves a call (decode, logits and the decode-loop step alike):
// the matrix-core decode where it is measured faster -- g = 8, and g = 4 with
// 3- or 4-bit key codes -- and for split widths, which only it reads; the
// per-head vector decode otherwise (at g = 4 with 1- or 2-bit key codes its
// nibble tables cost less than the matrix-core tile: 8B layer 27.8 against
// 33.3 us, batched b = 2 57.7 against 67.8 us).
inline bool mdecode_applies(const DecodeArgs &a) {
  const int g = a.n_q_heads / a.n_kv_heads;
  return mdecode_can_run(a) && (a.k_split || a.v_split || g == 8 || (g == 4 && a.k_bits >= 3));
}
// Scores only: the decode's key phase, writing every l_t to a.scores (no value
// phase, no combine; the value fields are not read).
hipError_t launch_logits(const DecodeArgs &a, hipStream_t stream);
// The merge of the chunk kernel's rotated partials (log-sum-exp, Pi_v^T, output).
hipError_t launch_combine(const DecodeArgs &a, hipStream_t stream);
// Chunk attention on the matrix cores: the tiles (whose prologue forms q~ and s), the merge.
hipError_t launch_chunk_mfma(const DecodeArgs &a, hipStream_t stream);

}  // namespace tq
