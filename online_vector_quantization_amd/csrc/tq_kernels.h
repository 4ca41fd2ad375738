// Kernel argument blocks and launchers of libtq.so (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace tq {

constexpr int kHeadDim = 128;    // the GPU path's d
constexpr int kQjlDim = 128;     // the GPU path's m for keys
constexpr int kMaxLevels = 16;   // 2^4

// Encode operands are bf16 fragments laid out so that each lane of a wave
// reads its 16-byte A operand of v_mfma_f32_16x16x32_bf16 with one LDS load:
// [split hi/lo][m-tile 0..7][k-step 0..3][lane 0..63] x 8 bf16.
constexpr size_t kFragBytesPerSplit = 8 * 4 * 64 * 16;   // 32 KiB
constexpr size_t kFragBytes = 2 * kFragBytesPerSplit;     // hi + lo

struct EncodeArgs {
  const void *x;
  int64_t x_stride;        // elements between rows
  int64_t n;
  const int64_t *dst_row;  // may be null
  int64_t cache_rows;
  uint32_t *codes;
  uint32_t *signs;
  float *norms;
  float *res_norms;
  float *dbg_rot;
  float *dbg_proj;
  const uint4 *frag_rot;   // kFragBytes
  const uint4 *frag_qjl;   // kFragBytes (keys with QJL)
  float centroids[kMaxLevels];
  float thresholds[kMaxLevels];
};

// Fills `dst` (kFragBytes) with the hi/lo bf16 fragments of the 128 x 128
// row-major matrix `mat` (rows = outputs, columns = inputs).
void pack_encode_fragments(const float *mat, void *dst);

// Enqueues the encode kernel; returns the launch error (hipSuccess on success).
hipError_t launch_encode(const EncodeArgs &a, int bits, bool qjl, bool x_f32, int num_cus,
                         hipStream_t stream);

struct DecodePlan {
  int chunk;               // tokens per work-group chunk
  int n_chunks;
  size_t off_qprep;        // bytes into the workspace
  size_t off_part_o;
  size_t off_part_ml;
  size_t total_bytes;
};

DecodePlan plan_decode(int batch, int n_q_heads, int n_kv_heads, int64_t t_cap);

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
  int batch, n_q_heads, n_kv_heads;
  int k_bits, v_bits, qjl_m;
  float scale;
  float qjl_coef;          // sqrt(pi/2)/m
  void *out;
  int out_bf16;
  float *dbg_scores;
  const float *rot_k_t;    // Pi_k^T row-major (d x d): entry [i][j] = Pi_k[j][i]
  const float *qjl_t;      // S^T row-major (d x m)
  const float *rot_v;      // Pi_v row-major (d x d)
  float k_centroids[kMaxLevels];
  float v_centroids[kMaxLevels];
  float *ws_qprep;         // [B*Hq][d + m]
  float *ws_part_o;        // [B*Hq][n_chunks][d]
  float *ws_part_ml;       // [B*Hq][n_chunks][2]
  int chunk, n_chunks;
};

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);

}  // namespace tq
