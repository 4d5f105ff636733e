// Launch descriptors shared by the host side of the C ABI (dpg_api.hip) and
// the kernels (dpg_kernels.hip). Layer tables travel as kernel arguments, up
// to kMaxLayers layers per launch; larger calls are split into several
// launches. Beside its layer table, each argument block carries the layers'
// first blocks as one contiguous array (first_block), which the launch
// functions fill from the table: a block finds its layer from that array
// with a few wide scalar loads, all in flight together.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dpg {

constexpr int kThreads = 256;  // every kernel: 4 wavefronts of 64 lanes
constexpr int kScaleThreads = 1024;  // (but the per-sample norm kernel: 16)
constexpr int kMaxLayers = 48;
static_assert(kMaxLayers >= 16, "the layer lookup scans 16 entries first");

// Matrix-core tiles: 128 x 128 outputs per block; the K step is 128 for
// bf16 operands and 32 for fp32 operands.
constexpr int kTileM = 128, kTileN = 128;
constexpr int kBackN = 64;  // back-projection: 128 x 64 output tiles
// Partial sums (sum-pass groups, projection splits) are read this many
// partials at a time, all loads in flight together.
constexpr int kSumBatch = 8;
// Large projections (bf16, r and B*T whole multiples of 256, d_in of 64):
// 256 x 256 output tiles, K steps of 64, operands copied to LDS by direct
// loads (two stages of P, three of A), 16 waves per block.
constexpr int kBigM = 256, kBigN = 256, kBigK = 64;
constexpr int kSampBigK = 64;  // K step (over t) of the large norm and sum kernel
// Large back-projection: 256 (d_in) x 128 (d_out) tiles, K steps of 32 over r,
// 4-wave blocks, two per CU.
constexpr int kBackBigN = 128, kBackBigK = 32;
// The sum pass folds the per-sample norm and clip factor into its prologue
// when a group holds at most this many samples and each sample at most this
// many norm partials.
constexpr int kFuseMaxGroup = 64, kFuseMaxSlots = 1024;
// At most this many samples per sum group (their clip factors sit in LDS).
constexpr int kSumMaxGroup = 1024;
constexpr int kStepBf16 = 128, kStepF32 = 32;

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
inline int64_t ceil_div(int64_t x, int64_t m) { return (x + m - 1) / m; }

// ---- P generation: P[j][k] = z / sqrt(r), row-major with row stride ld
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
  int32_t first_block[kMaxLayers];  // L[i].block0; INT32_MAX past n_layers
  int32_t n_layers;
  int32_t r;
  float scale;        // 1 / sqrt(r)
  uint32_t k0, k1, step_word;
  uint32_t tag;       // stream tag: 0 for P, 3 for norm-estimate probes
};

// ---- Xt = P A^T over a K range; written per sample as Xt[b][j][t] (row
//      stride ldt) when the layer is not split, else as an fp32 partial
//      part[split][j][n] (n = b*T + t) summed afterwards by the xsum kernel
struct ProjLayer {
  const void* A;      // [B*T][d_in]
  const void* P;      // [r][ldp]
  void* Xt;           // [B][r][ldt]
  float* part;        // [splits][r][B*T] when splits > 1
  int32_t d_in;
  int32_t ldp;
  int32_t m_tiles;    // over r
  int32_t n_tiles;    // over B*T
  int32_t splits;     // K ranges
  int32_t steps_per_split;
  int32_t block0;
  int32_t pad;
};
struct ProjArgs {
  ProjLayer L[kMaxLayers];
  int32_t first_block[kMaxLayers];  // L[i].block0; INT32_MAX past n_layers
  int32_t n_layers;
  int32_t n_blocks;   // logical blocks (grid is rounded up to a multiple of 8)
  int32_t B, T, r, ldt;
  int32_t off32;      // activation tiles addressable with 32-bit byte offsets
  int32_t full;       // every tile and step is full, with off32 and 16-byte rows
  int32_t groups2;    // 8-wave blocks: two wave groups split each block's steps
  int32_t big;        // proj_big_kernel: kBigM x kBigN tiles, steps of kBigK
};

struct XsumLayer {
  const float* part;  // [splits][r][B*T]
  void* Xt;           // [B][r][ldt]
  int32_t splits;
  int32_t block0;
};
struct XsumArgs {
  XsumLayer L[kMaxLayers];
  int32_t first_block[kMaxLayers];  // L[i].block0; INT32_MAX past n_layers
  int32_t n_layers;
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
  int32_t n_chunks;   // norm mode with res_tiles: runs of column tiles per sample
  float* ghat;        // norm mode, or null: each sample's product tile is also
                      // stored here, [B][r][d_out] fp32 (streaming form)
};
struct SampArgs {
  SampLayer L[kMaxLayers];
  int32_t first_block[kMaxLayers];  // L[i].block0; INT32_MAX past n_layers
  int32_t n_layers;
  int32_t n_blocks;
  int32_t B, T, r, ldt;
  int32_t per_block;    // samples per block (norm: a run, sum: a group)
  int32_t res_tiles;    // norm mode, T within one step: a block keeps one
                        // sample's Xt tile in LDS and sweeps this many
                        // column tiles of its dY (0: runs of samples)
  int32_t n_slots;      // norm mode: partial slots per sample
  int32_t off32;        // one sample's dY addressable with 32-bit byte offsets
  int32_t full;         // every tile and step full (r, d_out whole tiles, T
                        // whole steps), with off32 and paired dY columns
  float* norm_part;     // norm mode: [B][n_slots] (sum mode reads it when fused)
  const float* scales;  // sum mode: [B] (unused when fused)
  int32_t fuse_scale;   // sum mode: compute s_i from norm_part in the prologue
  float clip_C;         // sum mode, fused
  float* norms_out;     // sum mode, fused: [B] or null (written by layer 0's
                        // first tile of each group)
  int32_t big;          // samp_big_kernel: kBigM x kBigN tiles, steps of
                        // kSampBigK, 16 partial slots per (sample, tile)
};

// ---- n_i, s_i from the partials
struct ScaleArgs {
  const float* norm_part;  // [B][n_slots]
  int32_t n_slots;
  float clip_C;
  float* scales;           // [B]
  float* norms_out;        // [B] or null
};

// ---- streaming form: norm_sq[i] += sum_k part[i][k] (one layer's partials)
struct NormAccArgs {
  const float* norm_part;  // [B][n_slots]
  int32_t n_slots;
  int32_t B;
  float* norm_sq;          // [B], read-modify-write
};
// ---- streaming form: n_i = sqrt(norm_sq[i]), s_i = min(1, C / n_i)
struct ClipArgs {
  const float* norm_sq;    // [B]
  int32_t B;
  float clip_C;
  float* scales;           // [B]
  float* norms_out;        // [B] or null
};

// ---- G_priv = (sum_g w_g part_g + sigma C Z) / B  (w_g = 1 without weights)
struct FinLayer {
  const float* part;  // [groups][r*d_out]
  float* out;         // [r*d_out]
  float* m;           // with Adam: [r*d_out] first moment, in place
  float* v;           // with Adam: [r*d_out] second moment, in place
  void* U;            // with Adam: [r*d_out] direction, operand type
  int32_t n_elem;     // r * d_out
  uint32_t layer_id;
  int32_t block0;
  int32_t pad;
};
struct FinArgs {
  FinLayer L[kMaxLayers];
  int32_t first_block[kMaxLayers];  // L[i].block0; INT32_MAX past n_layers
  const float* weights;  // [groups] or null (streaming form: the clip factors)
  int32_t n_layers;
  int32_t groups;
  float noise_scale;  // sigma * C (0: no noise term)
  float inv_B;
  uint32_t k0, k1, step_word;
  // with Adam (the one-call step): constants as in PrepArgs
  float beta1, beta2, one_m_beta1, one_m_beta2, bc1, bc2, eps;
};

// ---- update call, first launch: Adam on [r][d_out] (U written row-major in
//      the operand type) and P regenerated row-major [r][d_in]
struct AdamLayer {
  const float* g;
  float* m;
  float* v;
  void* U;            // [r][d_out]
  int32_t n_elem;     // r * d_out
  int32_t block0;
};
struct PrepArgs {
  AdamLayer A[kMaxLayers];
  GenPLayer P[kMaxLayers];
  int32_t first_a[kMaxLayers];  // A[i].block0; INT32_MAX past n_layers
  int32_t first_p[kMaxLayers];  // P[i].block0; INT32_MAX past n_layers
  int32_t n_layers;
  int32_t adam_blocks;  // blocks [0, adam_blocks) run Adam, the rest gen P
  int32_t r;
  float beta1, beta2, one_m_beta1, one_m_beta2, bc1, bc2, eps;
  float p_scale;
  uint32_t k0, k1, step_word;
};

// ---- W -= lr P^T U, reading P [r][d_in] and U [r][d_out] directly
struct BackLayer {
  const void* P;      // [r][ldp]
  const void* U;      // [r][d_out]
  float* W;           // [d_in][d_out]
  int32_t d_in, d_out;
  int32_t ldp;        // row stride of P (>= d_in)
  int32_t pad;
  int32_t m_tiles, n_tiles;
  int32_t block0;
  int32_t n_chunks;   // with res_tiles: runs of column tiles per row tile
};
struct BackArgs {
  BackLayer L[kMaxLayers];
  int32_t first_block[kMaxLayers];  // L[i].block0; INT32_MAX past n_layers
  int32_t n_layers;
  int32_t n_blocks;
  int32_t r;
  float lr;
  int32_t off32;      // P and U addressable with 32-bit byte offsets
  int32_t full;       // every tile and step full (d_in, d_out whole tiles, r
                      // whole steps), with off32 and paired columns
  int32_t res_tiles;  // r within one step: a block keeps its P tile in LDS
                      // and sweeps this many column tiles (0: one tile); with
                      // big, the run of column tiles of a block
  int32_t big;        // back_big_kernel: kBigM x kBackBigN tiles, steps of kBackBigK
};

// Records `msg` as the calling thread's last error (dpg_last_error) and
// returns `code` (dpg_api.hip; for the library's other host sources).
int record_error(int code, const char* msg);

// Launchers (dpg_kernels.hip). Each returns the hipError_t of its launch.
// first[i] = L[i].block0 for the n layers of a table, INT32_MAX after them
template <class Layer>
inline void index_layers(int32_t (&first)[kMaxLayers], const Layer (&L)[kMaxLayers], int n) {
  for (int i = 0; i < kMaxLayers; ++i) first[i] = i < n ? L[i].block0 : INT32_MAX;
}

hipError_t launch_gen_p(GenPArgs a, int n_blocks, bool bf16_out,
                        hipStream_t s);
hipError_t launch_proj(ProjArgs a, bool bf16_in, bool vec, hipStream_t s);
hipError_t launch_xsum(XsumArgs a, int n_blocks, bool bf16_out,
                       hipStream_t s);
hipError_t launch_samp_norm(SampArgs a, bool bf16_in, bool pair,
                            hipStream_t s);
hipError_t launch_samp_sum(SampArgs a, bool bf16_in, bool pair,
                           hipStream_t s);
hipError_t launch_scale(const ScaleArgs& a, int B, hipStream_t s);
hipError_t launch_fin(FinArgs a, int n_blocks, hipStream_t s);
// fin followed, per element, by the Adam update (m, v in place, U written
// in bf16 when bf16_out, else fp32)
hipError_t launch_fin_adam(FinArgs a, int n_blocks, bool bf16_out, hipStream_t s);
hipError_t launch_norm_acc(const NormAccArgs& a, hipStream_t s);
hipError_t launch_clip(const ClipArgs& a, hipStream_t s);
hipError_t launch_prep(PrepArgs a, int n_blocks, bool bf16_out,
                       hipStream_t s);
hipError_t launch_back(BackArgs a, bool bf16_in, bool pair, hipStream_t s);
hipError_t launch_philox_normals(uint32_t k0, uint32_t k1, uint32_t layer_id,
                                 uint32_t step_word, uint32_t tag,
                                 uint32_t start, uint32_t n, float* z_out,
                                 uint32_t* words_out, hipStream_t s);

}  // namespace dpg
