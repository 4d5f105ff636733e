// Launch descriptors shared by the host side of the C ABI (dpg_api.hip) and
// the kernels (dpg_kernels.hip). Layer tables travel as kernel arguments, up
// to kMaxLayers layers per launch; larger calls are split into several
// launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dpg {

constexpr int kThreads = 256;  // every kernel: 4 wavefronts of 64 lanes
constexpr int kMaxLayers = 32;

// Tile sizes (rows x cols x k) of the matrix-core kernels.
constexpr int kProjBM = 128, kProjBN = 64, kProjBK = 32;     // Xt = P A^T
constexpr int kSampBM = 128, kSampBN = 128, kSampBK = 32;    // Xt_i dY_i
constexpr int kBackBM = 128, kBackBN = 128, kBackBK = 32;    // P^T U

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
inline int64_t ceil_div(int64_t x, int64_t m) { return (x + m - 1) / m; }

// ---- P generation (row-major [r][ld] for the projection, or transposed
//      [d_in][ld] for the back-projection)
struct GenPLayer {
  void* out;
  int32_t d_in;
  int32_t ld;
  uint32_t layer_id;
  int32_t n_ctr;      // ceil(r * d_in / 4) counters
  int32_t block0;     // first block of this layer
  int32_t pad;
};
struct GenPArgs {
  GenPLayer L[kMaxLayers];
  int32_t n_layers;
  int32_t r;
  float scale;        // 1 / sqrt(r)
  uint32_t k0, k1, step_word;
};

// ---- Xt = P A^T, written per sample as Xt[b][j][t] (row stride ldt)
struct ProjLayer {
  const void* A;      // [B*T][d_in]
  const void* P;      // [r][ldp]
  void* Xt;           // [B][r][ldt]
  int32_t d_in;
  int32_t ldp;
  int32_t m_tiles;    // over r
  int32_t n_tiles;    // over B*T
  int32_t block0;
  int32_t pad;
};
struct ProjArgs {
  ProjLayer L[kMaxLayers];
  int32_t n_layers;
  int32_t n_blocks;   // logical blocks (grid is rounded up to a multiple of 8)
  int32_t B, T, r, ldt;
};

// ---- per-sample products Xt_i dY_i: squared-norm partials, or the scaled
//      sum over a group of samples
struct SampLayer {
  const void* dY;     // [B*T][d_out]
  const void* Xt;     // [B][r][ldt]
  float* part;        // sum mode: [groups][r][d_out]
  int32_t d_out;
  int32_t m_tiles;    // over r
  int32_t n_tiles;    // over d_out
  int32_t slot0;      // norm mode: first partial slot of this layer
  int32_t block0;
  int32_t pad;
};
struct SampArgs {
  SampLayer L[kMaxLayers];
  int32_t n_layers;
  int32_t n_blocks;
  int32_t B, T, r, ldt;
  int32_t groups;       // sum mode: sample groups
  int32_t per_group;    // sum mode: samples per group
  int32_t n_slots;      // norm mode: partial slots per sample
  float* norm_part;     // norm mode: [B][n_slots]
  const float* scales;  // sum mode: [B]
};

// ---- n_i, s_i from the partials
struct ScaleArgs {
  const float* norm_part;  // [B][n_slots]
  int32_t n_slots;
  float clip_C;
  float* scales;           // [B]
  float* norms_out;        // [B] or null
};

// ---- G_priv = (sum_g part_g + sigma C Z) / B
struct FinLayer {
  const float* part;  // [groups][r*d_out]
  float* out;         // [r*d_out]
  int32_t n_elem;     // r * d_out
  uint32_t layer_id;
  int32_t block0;
  int32_t pad;
};
struct FinArgs {
  FinLayer L[kMaxLayers];
  int32_t n_layers;
  int32_t groups;
  float noise_scale;  // sigma * C (0: no noise term)
  float inv_B;
  uint32_t k0, k1, step_word;
};

// ---- Adam in the projected space; writes U transposed, Ut[n][j]
struct AdamLayer {
  const float* g;
  float* m;
  float* v;
  void* Ut;           // [d_out][ldr]
  int32_t d_out;
  int32_t n_elem;     // r * d_out
  int32_t block0;
  int32_t pad;
};
struct AdamArgs {
  AdamLayer L[kMaxLayers];
  int32_t n_layers;
  int32_t r, ldr;
  float beta1, beta2, one_m_beta1, one_m_beta2, bc1, bc2, eps;
};

// ---- W -= lr Pt Ut^T
struct BackLayer {
  const void* Pt;     // [d_in][ldr]
  const void* Ut;     // [d_out][ldr]
  float* W;           // [d_in][d_out]
  int32_t d_in, d_out;
  int32_t m_tiles, n_tiles;
  int32_t block0;
  int32_t pad;
};
struct BackArgs {
  BackLayer L[kMaxLayers];
  int32_t n_layers;
  int32_t n_blocks;
  int32_t r, ldr;
  float lr;
};

// Launchers (dpg_kernels.hip). Each returns the hipError_t of its launch.
hipError_t launch_gen_p(const GenPArgs& a, int n_blocks, bool bf16_out,
                        bool transposed, hipStream_t s);
hipError_t launch_proj(const ProjArgs& a, bool bf16_in, bool vec, hipStream_t s);
hipError_t launch_samp_norm(const SampArgs& a, bool bf16_in, bool pair,
                            hipStream_t s);
hipError_t launch_samp_sum(const SampArgs& a, bool bf16_in, bool pair,
                           hipStream_t s);
hipError_t launch_scale(const ScaleArgs& a, int B, hipStream_t s);
hipError_t launch_fin(const FinArgs& a, int n_blocks, hipStream_t s);
hipError_t launch_adam(const AdamArgs& a, int n_blocks, bool bf16_out,
                       hipStream_t s);
hipError_t launch_back(const BackArgs& a, bool bf16_in, hipStream_t s);
hipError_t launch_philox_normals(uint32_t k0, uint32_t k1, uint32_t layer_id,
                                 uint32_t step_word, uint32_t tag,
                                 uint32_t start, uint32_t n, float* z_out,
                                 uint32_t* words_out, hipStream_t s);

}  // namespace dpg
