// Internal declarations shared by the host setup, the C-ABI layer and the
// kernel launchers of libtq.so.  Not installed; the public ABI is include/tq.h.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "tq.h"

namespace tq {

// Host-side tables of one codebook handle (all row-major).
struct HostTables {
  int d = 0, bits = 0, m = 0, levels = 0;
  std::vector<double> centroids64, thresholds64, rotation64, qjl64;
  std::vector<float> centroids, thresholds, rotation, qjl;
  // Split widths: rotated coordinates 0 .. n_wide - 1 take the (bits + 1)-bit
  // codebook below (empty when n_wide == 0), the others the bits-bit one above.
  int n_wide = 0;
  std::vector<double> wide_centroids64, wide_thresholds64;
  std::vector<float> wide_centroids, wide_thresholds;
};

// Builds every host table; returns false (with `err` set) on bad input.
bool build_host_tables(int d, int bits, int n_wide, int m, uint64_t rot_seed, uint64_t qjl_seed,
                       HostTables *out, std::string *err);

// Pieces exposed for the CPU tests of the library's own setup code.
double sphere_coord_cdf(double t, int d);
void lloyd_max_sphere(int d, int bits, std::vector<double> *centroids,
                      std::vector<double> *thresholds, int *iterations);
void seeded_normals(uint64_t seed, size_t count, double *out);
void haar_orthogonal(int d, uint64_t seed, double *pi_rowmajor);

// bf16 round-to-nearest-even of a float, as raw bits.
uint16_t bf16_bits_rne(float v);
float bf16_bits_to_float(uint16_t b);

}  // namespace tq

// Device-side part of a codebook handle (owned by the C-ABI layer).
struct tq_codebook {
  tq::HostTables host;
  uint64_t rot_seed = 0, qjl_seed = 0;
  int device = -1;
  void *dev_buf = nullptr;        // one hipMalloc holding every device table
  size_t dev_bytes = 0;
  // Offsets (bytes) into dev_buf.
  size_t off_centroids = 0;       // float[L]
  size_t off_thresholds = 0;      // float[L-1] (padded)
  size_t off_rot_frag = 0;        // encode A-operand fragments of Pi: hi then lo
  size_t off_qjl_frag = 0;        // encode A-operand fragments of S: hi then lo
  size_t off_dec_rot_frag = 0;    // decode fp16 fragments of 2^kDecFragExp Pi: hi then lo
  size_t off_dec_qjl_frag = 0;    // decode fp16 fragments of 2^kDecFragExp S Pi: hi then lo
  size_t off_rot_f32 = 0;         // float[d*d] row-major Pi
  size_t off_rot_t_f32 = 0;       // float[d*d] row-major Pi^T
  size_t off_qjl_rot_t_f32 = 0;   // float[d*m] row-major (S Pi)^T
  size_t off_key_lut = 0;         // decode key dequantization table
  size_t off_pair_lut = 0;        // decode value pair table
  size_t off_qcells = 0;          // encode quantizer cell table
  size_t off_mkey_lut = 0;        // matrix-core decode: key operand table
  size_t off_mval_lut = 0;        // matrix-core decode: value operand table
  size_t off_sign_lut = 0;        // matrix-core decode: sign table
  // Split widths: the wide codebook's encode cell table and matrix-core
  // decode operand tables (0 when the codebook has no wide coordinates).
  size_t off_qcells_w = 0;
  size_t off_mkey_lut_w = 0;
  size_t off_mval_lut_w = 0;
  float qscale = 0.f, qbias = 0.f;
};
