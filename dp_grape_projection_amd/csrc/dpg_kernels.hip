// HIP kernels of the DP-GRAPE private update step for gfx950.
//
// Method: "Memory-Efficient Differentially Private Training with Gradient
// Random Projection" (gist.science technical summary, Methodology): project
// every per-sample linear-layer gradient with a seeded Gaussian P (design
// choices 1, 2), clip by the global per-sample norm, sum and noise, Adam in
// the projected space (design choice 3), back-project into W.
//
// Per-sample projected gradients are never stored. The projection call runs
//   gen_p   P_l[r][d_in] from the seed (transient, bf16 or fp32)
//   proj    Xt_l[b][j][t] = sum_k P_l[j][k] A_l[b][t][k]   (one GEMM over B*T)
//   norm    for every (sample, tile): ||Xt_il dY_il||_F^2 partials
//   scale   n_i = sqrt(sum of partials over all layers), s_i = min(1, C/n_i)
//   sum     sum_i s_i Xt_il dY_il over groups of samples (second pass)
//   fin     G_priv = (sum over groups + sigma C Z) / B
// and the update call runs
//   adam    m, v in place; U = mhat / (sqrt(vhat) + eps), written as Ut[n][j]
//   gen_p   P_l again, transposed to Pt[k][j]
//   back    W -= lr Pt Ut^T
#include "dpg_device.hpp"
#include "dpg_internal.hpp"

namespace dpg {

template <class L>
__device__ __forceinline__ int find_layer(const L* layers, int n, int b) {
  int l = 0;
  for (int i = 1; i < n; ++i)
    if (b >= layers[i].block0) l = i;
  return l;
}

// Sum over the 256 threads of a block, in a fixed order (deterministic).
__device__ __forceinline__ float block_sum(float x, float* red4) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red4[wave] = x;
  __syncthreads();
  float t = 0.0f;
  if (threadIdx.x == 0) t = ((red4[0] + red4[1]) + red4[2]) + red4[3];
  return t;  // valid in thread 0 only
}

// ------------------------------------------------------------------ gen_p --

template <typename T, bool TRANSPOSED>
__global__ __launch_bounds__(kThreads) void gen_p_kernel(const GenPArgs a) {
  const int b = blockIdx.x;
  const GenPLayer& L = a.L[find_layer(a.L, a.n_layers, b)];
  const int c = (b - L.block0) * kThreads + static_cast<int>(threadIdx.x);
  if (c >= L.n_ctr) return;
  const StreamKey key{a.k0, a.k1, a.step_word, 0u};
  float z[4];
  normals_at(key, L.layer_id, static_cast<uint32_t>(c), z);
  const uint64_t total = static_cast<uint64_t>(a.r) * L.d_in;
  uint64_t e = 4ull * static_cast<uint64_t>(c);
  uint32_t j = static_cast<uint32_t>(e / L.d_in);
  uint32_t k = static_cast<uint32_t>(e - static_cast<uint64_t>(j) * L.d_in);
  T* out = static_cast<T*>(L.out);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (e + q < total) {
      const T val = from_float<T>(z[q] * a.scale);
      if (TRANSPOSED)
        out[static_cast<int64_t>(k) * L.ld + j] = val;
      else
        out[static_cast<int64_t>(j) * L.ld + k] = val;
    }
    if (++k == static_cast<uint32_t>(L.d_in)) {
      k = 0;
      ++j;
    }
  }
}

// ------------------------------------------------------------------- proj --

template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void proj_kernel(const ProjArgs a) {
  constexpr int BM = kProjBM, BN = kProjBN, BK = kProjBK;
  typedef TileShape<T, BM, BN, BK> Sh;
  __shared__ __attribute__((aligned(16))) T smem[(BM + BN) * Sh::S];
  const int lb = xcd_logical_block();
  if (lb >= a.n_blocks) return;
  const ProjLayer& L = a.L[find_layer(a.L, a.n_layers, lb)];
  const int tile = lb - L.block0;
  const int mt = tile % L.m_tiles, nt = tile / L.m_tiles;
  const int j0 = mt * BM, n0 = nt * BN;
  const int BT = a.B * a.T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  RowsLoader<T, BM, BK, true> la{static_cast<const T*>(L.P) +
                                     static_cast<int64_t>(j0) * L.ldp,
                                 L.ldp, a.r - j0, L.d_in};
  RowsLoader<T, BN, BK, VEC> lx{static_cast<const T*>(L.A) +
                                    static_cast<int64_t>(n0) * L.d_in,
                                L.d_in, BT - n0, L.d_in};
  Acc<Sh::MB, Sh::NB> acc;
  acc.zero();
  k_loop<T, BM, BN, BK>(la, lx, smem, smem + BM * Sh::S, acc, 0, L.d_in, tid);

  T* Xt = static_cast<T*>(L.Xt);
#pragma unroll
  for (int nb = 0; nb < Sh::NB; ++nb) {
    const int n = n0 + acc_col<Sh::WTN>(wn, nb, lane);
    if (n >= BT) continue;
    const int bi = n / a.T, t = n - bi * a.T;
    T* dst = Xt + static_cast<int64_t>(bi) * a.r * a.ldt + t;
#pragma unroll
    for (int mb = 0; mb < Sh::MB; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = j0 + acc_row<Sh::WTM>(wm, mb, i, lane);
        if (j < a.r)
          dst[static_cast<int64_t>(j) * a.ldt] = from_float<T>(acc.v[mb][nb][i]);
      }
  }
}

// ---------------------------------------------------------- norm and sum --

template <typename T, bool PAIR, bool SUM>
__global__ __launch_bounds__(kThreads) void samp_kernel(const SampArgs a) {
  constexpr int BM = kSampBM, BN = kSampBN, BK = kSampBK;
  typedef TileShape<T, BM, BN, BK> Sh;
  __shared__ __attribute__((aligned(16))) T smem[(BM + BN) * Sh::S];
  __shared__ float red4[4];
  const int lb = xcd_logical_block();
  if (lb >= a.n_blocks) return;
  const SampLayer& L = a.L[find_layer(a.L, a.n_layers, lb)];
  const int tile = lb - L.block0;
  const int mt = tile % L.m_tiles;
  const int rest = tile / L.m_tiles;
  const int nt = rest % L.n_tiles;
  const int g = rest / L.n_tiles;  // sample (norm) or sample group (sum)
  const int j0 = mt * BM, n0 = nt * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  int i_begin = g, i_end = g + 1;
  if (SUM) {
    i_begin = g * a.per_group;
    i_end = min(a.B, i_begin + a.per_group);
  }

  Acc<Sh::MB, Sh::NB> acc, tot;
  if (SUM) tot.zero();
  const T* Xt = static_cast<const T*>(L.Xt);
  const T* dY = static_cast<const T*>(L.dY);
  for (int i = i_begin; i < i_end; ++i) {
    RowsLoader<T, BM, BK, true> la{
        Xt + (static_cast<int64_t>(i) * a.r + j0) * a.ldt, a.ldt, a.r - j0, a.T};
    ColsLoader<T, BN, BK, PAIR> lc{
        dY + static_cast<int64_t>(i) * a.T * L.d_out + n0, L.d_out,
        L.d_out - n0, a.T};
    acc.zero();
    k_loop<T, BM, BN, BK>(la, lc, smem, smem + BM * Sh::S, acc, 0, a.T, tid);
    if (SUM) {
      const float s = a.scales[i];
#pragma unroll
      for (int mb = 0; mb < Sh::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < Sh::NB; ++nb)
#pragma unroll
          for (int q = 0; q < 16; ++q)
            tot.v[mb][nb][q] = fmaf(s, acc.v[mb][nb][q], tot.v[mb][nb][q]);
    } else {
      // Out-of-range rows and columns were loaded as zeros, so they add 0.
      float sq = 0.0f;
#pragma unroll
      for (int mb = 0; mb < Sh::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < Sh::NB; ++nb)
#pragma unroll
          for (int q = 0; q < 16; ++q)
            sq = fmaf(acc.v[mb][nb][q], acc.v[mb][nb][q], sq);
      const float t = block_sum(sq, red4);
      if (tid == 0)
        a.norm_part[static_cast<int64_t>(i) * a.n_slots + L.slot0 +
                    nt * L.m_tiles + mt] = t;
    }
  }
  if (SUM) {
    float* part = L.part + static_cast<int64_t>(g) * a.r * L.d_out;
#pragma unroll
    for (int nb = 0; nb < Sh::NB; ++nb) {
      const int n = n0 + acc_col<Sh::WTN>(wn, nb, lane);
      if (n >= L.d_out) continue;
#pragma unroll
      for (int mb = 0; mb < Sh::MB; ++mb)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int j = j0 + acc_row<Sh::WTM>(wm, mb, q, lane);
          if (j < a.r) part[static_cast<int64_t>(j) * L.d_out + n] = tot.v[mb][nb][q];
        }
    }
  }
}

// ------------------------------------------------------------------ scale --

__global__ __launch_bounds__(kThreads) void scale_kernel(const ScaleArgs a) {
  __shared__ float red4[4];
  const int i = blockIdx.x;
  const float* p = a.norm_part + static_cast<int64_t>(i) * a.n_slots;
  float s = 0.0f;
  for (int k = threadIdx.x; k < a.n_slots; k += kThreads) s += p[k];
  const float tot = block_sum(s, red4);
  if (threadIdx.x == 0) {
    const float n = sqrtf(tot);
    a.scales[i] = (n > a.clip_C) ? a.clip_C / n : 1.0f;
    if (a.norms_out) a.norms_out[i] = n;
  }
}

// -------------------------------------------------------------------- fin --

__global__ __launch_bounds__(kThreads) void fin_kernel(const FinArgs a) {
  const int b = blockIdx.x;
  const FinLayer& L = a.L[find_layer(a.L, a.n_layers, b)];
  const int c = (b - L.block0) * kThreads + static_cast<int>(threadIdx.x);
  const int64_t e0 = 4ll * c;
  if (e0 >= L.n_elem) return;
  float z[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (a.noise_scale != 0.0f) {
    const StreamKey key{a.k0, a.k1, a.step_word, 1u};
    normals_at(key, L.layer_id, static_cast<uint32_t>(c), z);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t e = e0 + q;
    if (e < L.n_elem) {
      float s = 0.0f;
      for (int g = 0; g < a.groups; ++g) s += L.part[g * static_cast<int64_t>(L.n_elem) + e];
      L.out[e] = fmaf(a.noise_scale, z[q], s) * a.inv_B;
    }
  }
}

// ------------------------------------------------------------------- adam --

template <typename T>
__global__ __launch_bounds__(kThreads) void adam_kernel(const AdamArgs a) {
  const int b = blockIdx.x;
  const AdamLayer& L = a.L[find_layer(a.L, a.n_layers, b)];
  const int c = (b - L.block0) * kThreads + static_cast<int>(threadIdx.x);
  const int64_t e0 = 4ll * c;
  if (e0 >= L.n_elem) return;
  T* Ut = static_cast<T*>(L.Ut);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t e = e0 + q;
    if (e < L.n_elem) {
      const float g = L.g[e];
      const float m = fmaf(a.beta1, L.m[e], a.one_m_beta1 * g);
      const float v = fmaf(a.beta2, L.v[e], a.one_m_beta2 * (g * g));
      L.m[e] = m;
      L.v[e] = v;
      const float u = (m / a.bc1) / (sqrtf(v / a.bc2) + a.eps);
      const int64_t j = e / L.d_out, n = e - j * L.d_out;
      Ut[n * a.ldr + j] = from_float<T>(u);
    }
  }
}

// ------------------------------------------------------------------- back --

template <typename T>
__global__ __launch_bounds__(kThreads) void back_kernel(const BackArgs a) {
  constexpr int BM = kBackBM, BN = kBackBN, BK = kBackBK;
  typedef TileShape<T, BM, BN, BK> Sh;
  __shared__ __attribute__((aligned(16))) T smem[(BM + BN) * Sh::S];
  const int lb = xcd_logical_block();
  if (lb >= a.n_blocks) return;
  const BackLayer& L = a.L[find_layer(a.L, a.n_layers, lb)];
  const int tile = lb - L.block0;
  const int nt = tile % L.n_tiles, mt = tile / L.n_tiles;
  const int m0 = mt * BM, n0 = nt * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  RowsLoader<T, BM, BK, true> la{static_cast<const T*>(L.Pt) +
                                     static_cast<int64_t>(m0) * a.ldr,
                                 a.ldr, L.d_in - m0, a.r};
  RowsLoader<T, BN, BK, true> lu{static_cast<const T*>(L.Ut) +
                                     static_cast<int64_t>(n0) * a.ldr,
                                 a.ldr, L.d_out - n0, a.r};
  Acc<Sh::MB, Sh::NB> acc;
  acc.zero();
  k_loop<T, BM, BN, BK>(la, lu, smem, smem + BM * Sh::S, acc, 0, a.r, tid);

#pragma unroll
  for (int nb = 0; nb < Sh::NB; ++nb) {
    const int n = n0 + acc_col<Sh::WTN>(wn, nb, lane);
    if (n >= L.d_out) continue;
#pragma unroll
    for (int mb = 0; mb < Sh::MB; ++mb)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int m = m0 + acc_row<Sh::WTM>(wm, mb, q, lane);
        if (m < L.d_in) {
          float* w = L.W + static_cast<int64_t>(m) * L.d_out + n;
          *w = fmaf(-a.lr, acc.v[mb][nb][q], *w);
        }
      }
  }
}

// ---------------------------------------------------------- philox stream --

__global__ __launch_bounds__(kThreads) void philox_normals_kernel(
    uint32_t k0, uint32_t k1, uint32_t layer_id, uint32_t step_word,
    uint32_t tag, uint32_t start, uint32_t n, float* z_out,
    uint32_t* words_out) {
  const uint32_t c_lo = start >> 2;
  const uint32_t c_hi = (start + n - 1) >> 2;
  const uint32_t c = c_lo + blockIdx.x * kThreads + threadIdx.x;
  if (c > c_hi) return;
  uint32_t w[4];
  philox4x32_10(c, layer_id, step_word, tag, k0, k1, w);
  float z[4];
  box_muller4(w, z);
  if (words_out) {
#pragma unroll
    for (int q = 0; q < 4; ++q) words_out[4ull * (c - c_lo) + q] = w[q];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint64_t e = 4ull * c + q;
    if (e >= start && e < static_cast<uint64_t>(start) + n) z_out[e - start] = z[q];
  }
}

// -------------------------------------------------------------- launchers --

static inline unsigned grid8(int n_blocks) {
  return static_cast<unsigned>(round_up(n_blocks, 8));
}

hipError_t launch_gen_p(const GenPArgs& a, int n_blocks, bool bf16_out,
                        bool transposed, hipStream_t s) {
  const dim3 g(n_blocks), b(kThreads);
  if (bf16_out) {
    if (transposed) hipLaunchKernelGGL((gen_p_kernel<bf16, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((gen_p_kernel<bf16, false>), g, b, 0, s, a);
  } else {
    if (transposed) hipLaunchKernelGGL((gen_p_kernel<float, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((gen_p_kernel<float, false>), g, b, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_proj(const ProjArgs& a, bool bf16_in, bool vec, hipStream_t s) {
  const dim3 g(grid8(a.n_blocks)), b(kThreads);
  if (bf16_in) {
    if (vec) hipLaunchKernelGGL((proj_kernel<bf16, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((proj_kernel<bf16, false>), g, b, 0, s, a);
  } else {
    if (vec) hipLaunchKernelGGL((proj_kernel<float, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((proj_kernel<float, false>), g, b, 0, s, a);
  }
  return hipGetLastError();
}

template <bool SUM>
static hipError_t launch_samp(const SampArgs& a, bool bf16_in, bool pair,
                              hipStream_t s) {
  const dim3 g(grid8(a.n_blocks)), b(kThreads);
  if (bf16_in) {
    if (pair) hipLaunchKernelGGL((samp_kernel<bf16, true, SUM>), g, b, 0, s, a);
    else hipLaunchKernelGGL((samp_kernel<bf16, false, SUM>), g, b, 0, s, a);
  } else {
    hipLaunchKernelGGL((samp_kernel<float, true, SUM>), g, b, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_samp_norm(const SampArgs& a, bool bf16_in, bool pair,
                            hipStream_t s) {
  return launch_samp<false>(a, bf16_in, pair, s);
}

hipError_t launch_samp_sum(const SampArgs& a, bool bf16_in, bool pair,
                           hipStream_t s) {
  return launch_samp<true>(a, bf16_in, pair, s);
}

hipError_t launch_scale(const ScaleArgs& a, int B, hipStream_t s) {
  hipLaunchKernelGGL(scale_kernel, dim3(B), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fin(const FinArgs& a, int n_blocks, hipStream_t s) {
  hipLaunchKernelGGL(fin_kernel, dim3(n_blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_adam(const AdamArgs& a, int n_blocks, bool bf16_out,
                       hipStream_t s) {
  if (bf16_out)
    hipLaunchKernelGGL(adam_kernel<bf16>, dim3(n_blocks), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(adam_kernel<float>, dim3(n_blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_back(const BackArgs& a, bool bf16_in, hipStream_t s) {
  const dim3 g(grid8(a.n_blocks)), b(kThreads);
  if (bf16_in) hipLaunchKernelGGL(back_kernel<bf16>, g, b, 0, s, a);
  else hipLaunchKernelGGL(back_kernel<float>, g, b, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_philox_normals(uint32_t k0, uint32_t k1, uint32_t layer_id,
                                 uint32_t step_word, uint32_t tag,
                                 uint32_t start, uint32_t n, float* z_out,
                                 uint32_t* words_out, hipStream_t s) {
  const uint32_t n_ctr = ((start + n - 1) >> 2) - (start >> 2) + 1;
  const unsigned blocks = (n_ctr + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(philox_normals_kernel, dim3(blocks), dim3(kThreads), 0, s,
                     k0, k1, layer_id, step_word, tag, start, n, z_out, words_out);
  return hipGetLastError();
}

}  // namespace dpg
