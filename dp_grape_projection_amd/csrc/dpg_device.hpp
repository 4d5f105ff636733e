// Device building blocks for the DP-GRAPE kernels on gfx950 (CDNA4).
//
//  * Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
//    Easy as 1, 2, 3", SC'11) and Box-Muller normals: the generator that
//    regenerates the projection P and draws the noise Z from a seed, as the
//    method requires of P ("Memory-Efficient Differentially Private Training
//    with Gradient Random Projection", technical summary, Methodology, design
//    choice 1). Stream layout: key = seed, counter = (e >> 2, layer_id,
//    step word, tag); u(x) = (2 (x >> 9) + 1) 2^-24; element e takes entry
//    e & 3 of (R0 cos t0, R0 sin t0, R1 cos t1, R1 sin t1).
//  * A 256-thread (4 x wave64) LDS-staged tile engine around the
//    v_mfma_f32_32x32x16_bf16 (bf16 operands) and v_mfma_f32_32x32x2_f32
//    (fp32 operands) matrix-core instructions, fp32 accumulation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dpg_internal.hpp"

namespace dpg {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

// Buffer resource over the 4 GiB from `base`, which must be the same in every
// lane (it is read from the first one; so are the loader's k0 and ld). The callers keep every offset inside
// the tensor. Loads through it take one per-lane 32-bit offset plus a
// block-uniform one, so a tile's loads share one address register and need
// no 64-bit address arithmetic.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  void* u = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(u, static_cast<short>(0),
                                           static_cast<int>(0xFFFFFFFFu), 0x00020000);
}

// Cache-policy operand of the buffer load and store builtins for data read
// or written once (the nt bit on gfx950): such lines are the first the L2
// evicts, so a stream of them does not push out operands that are re-read.
constexpr int kNonTemporal = 2;

// ---------------------------------------------------------------- random --

// Ten Philox rounds: each round multiplies c0 and c2 by the two round
// constants (32x32 -> 64 bit), and the key is bumped by the Weyl constants
// between rounds.
__device__ __forceinline__ void philox4x32_10(uint32_t c0, uint32_t c1,
                                              uint32_t c2, uint32_t c3,
                                              uint32_t k0, uint32_t k1,
                                              uint32_t out[4]) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    // one 32x32 -> 64-bit multiply gives both halves
    const uint64_t p0 = static_cast<uint64_t>(c0) * 0xD2511F53u;
    const uint64_t p1 = static_cast<uint64_t>(c2) * 0xCD9E8D57u;
    c0 = static_cast<uint32_t>(p1 >> 32) ^ c1 ^ k0;
    c1 = static_cast<uint32_t>(p1);
    c2 = static_cast<uint32_t>(p0 >> 32) ^ c3 ^ k1;
    c3 = static_cast<uint32_t>(p0);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

// Uniform in (0, 1): (2 (x >> 9) + 1) * 2^-24. The odd integer is < 2^24, so
// the conversion and the scaling are exact in fp32.
__device__ __forceinline__ float uniform_open01(uint32_t x) {
  return static_cast<float>(((x >> 9) << 1) | 1u) * 5.9604644775390625e-08f;
}

// Box-Muller is evaluated in float64 and each normal is rounded to fp32 once,
// so a normal is within half an fp32 ulp (2.4e-7 for |z| < 8) plus about
// 1e-11 of its exact value. (fp32 arithmetic alone cannot hold 1e-6 in the
// tails: there an ulp of z is 4.8e-7.) On gfx950 float64 adds and
// multiply-adds issue at the rate of non-packed fp32 ones.

// 1 / d for d in [1.7, 2.5], and 1 / sqrt(x) for a normal x > 0: the fp32
// hardware approximation (relative error about 2^-23), then one Newton-
// Raphson step in float64, y <- y (2 - d y) and y <- y (3 - x y^2) / 2,
// which squares the relative error (below 1e-13).
__device__ __forceinline__ double recip_mid(double d) {
  const double y = static_cast<double>(__builtin_amdgcn_rcpf(static_cast<float>(d)));
  return fma(y, fma(-d, y, 1.0), y);
}
__device__ __forceinline__ double rsqrt_pos(double x) {
  const double y = static_cast<double>(__builtin_amdgcn_rsqf(static_cast<float>(x)));
  return fma(0.5 * y, fma(-x * y, y, 1.0), y);
}

// ln u for u in (0, 1) (a normal double): u = m 2^e with m in [1/sqrt 2,
// sqrt 2), and ln m = 2 atanh(s) with s = (m - 1) / (m + 1), |s| <= 0.1716,
// from the odd series atanh(s) = s (1 + s^2/3 + s^4/5 + ...) cut after the
// s^10/11 term (truncation below 5e-11 relative).
__device__ __forceinline__ double ln_unit(double u) {
  double m = __builtin_amdgcn_frexp_mant(u);  // [0.5, 1)
  int e = __builtin_amdgcn_frexp_exp(u);
  if (m < 0.70710678118654752) {
    m *= 2.0;
    e -= 1;
  }
  const double s = (m - 1.0) * recip_mid(m + 1.0);
  const double s2 = s * s;
  double p = 1.0 / 11.0;
  p = fma(p, s2, 1.0 / 9.0);
  p = fma(p, s2, 1.0 / 7.0);
  p = fma(p, s2, 1.0 / 5.0);
  p = fma(p, s2, 1.0 / 3.0);
  p = fma(p, s2, 1.0);
  return fma(static_cast<double>(e), 0.69314718055994531, 2.0 * s * p);
}

// cos and sin of the angle 2 pi t for t in (0, 1) given in turns. Quadrant
// reduction is exact: q = round(4 t), f = t - q / 4 in [-1/8, 1/8] (t has 24
// significant bits), x = 2 pi f in [-pi/4, pi/4]. Taylor polynomials: sin
// through x^11 (truncation below 7e-12), cos through x^12 (below 4e-13);
// then the quadrant rotates (cos x, sin x) by q quarter turns.
__device__ __forceinline__ void cossin_turns(double t, double& c, double& s) {
  const double q = __builtin_rint(4.0 * t);
  const double x = (t - 0.25 * q) * 6.2831853071795865;
  const double x2 = x * x;
  double ps = -1.0 / 39916800.0;                  // -1/11!
  ps = fma(ps, x2, 1.0 / 362880.0);
  ps = fma(ps, x2, -1.0 / 5040.0);
  ps = fma(ps, x2, 1.0 / 120.0);
  ps = fma(ps, x2, -1.0 / 6.0);
  const double sx = fma(ps * x2, x, x);
  double pc = 1.0 / 479001600.0;                  // 1/12!
  pc = fma(pc, x2, -1.0 / 3628800.0);
  pc = fma(pc, x2, 1.0 / 40320.0);
  pc = fma(pc, x2, -1.0 / 720.0);
  pc = fma(pc, x2, 1.0 / 24.0);
  pc = fma(pc, x2, -0.5);
  const double cx = fma(pc, x2, 1.0);
  switch (static_cast<int>(q) & 3) {
    case 0: c = cx; s = sx; break;
    case 1: c = -sx; s = cx; break;
    case 2: c = -cx; s = -sx; break;
    default: c = sx; s = -cx; break;
  }
}

// Box-Muller on the pairs (w0, w1) and (w2, w3): R = sqrt(-2 ln u(w0)),
// z0 = R cos(2 pi u(w1)), z1 = R sin(2 pi u(w1)), and likewise for (w2, w3).
// u >= 2^-24, so the logarithm never sees a denormal.
__device__ __forceinline__ void box_muller4(const uint32_t w[4], float z[4]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const double u = static_cast<double>(uniform_open01(w[2 * h]));
    const double t = static_cast<double>(uniform_open01(w[2 * h + 1]));
    const double x = -2.0 * ln_unit(u);  // in [1.1e-7, 33.3]
    const double R = x * rsqrt_pos(x);
    double c, s;
    cossin_turns(t, c, s);
    z[2 * h] = static_cast<float>(R * c);
    z[2 * h + 1] = static_cast<float>(R * s);
  }
}

struct StreamKey {
  uint32_t k0, k1;       // seed low / high word
  uint32_t step_word;    // proj_step (tag 0) or step (tag 1)
  uint32_t tag;          // 0 = projection P, 1 = noise Z
};

// The four normals of counter c of one layer's stream.
__device__ __forceinline__ void normals_at(const StreamKey& key,
                                           uint32_t layer_id, uint32_t c,
                                           float z[4]) {
  uint32_t w[4];
  philox4x32_10(c, layer_id, key.step_word, key.tag, key.k0, key.k1, w);
  box_muller4(w, z);
}

// ------------------------------------------------------------ data types --

template <typename T> struct Vec16;
template <> struct Vec16<bf16> { typedef bf16x8 type; static constexpr int N = 8; };
template <> struct Vec16<float> { typedef f32x4 type; static constexpr int N = 4; };

__device__ __forceinline__ float to_float(bf16 x) { return static_cast<float>(x); }
__device__ __forceinline__ float to_float(float x) { return x; }
template <typename T> __device__ __forceinline__ T from_float(float x);
template <> __device__ __forceinline__ bf16 from_float<bf16>(float x) {
  return static_cast<bf16>(x);  // round to nearest even
}
template <> __device__ __forceinline__ float from_float<float>(float x) { return x; }

template <typename T> __device__ __forceinline__ T zero_val() { return from_float<T>(0.0f); }

// ----------------------------------------------------------- tile engine --
//
// A block of 4 waves computes C[BM x BN] = sum_k Aop[m][k] * Bop[n][k] with
// both operands staged in LDS as K-contiguous rows (sA[m][k], sB[n][k]). The
// waves are laid out WGM x WGN over the tile; each owns a WTM x WTN wave tile
// of MB x NB blocks of 32 x 32 computed with the 32x32 matrix-core
// instructions (fp32 accumulation).
//
// Accumulator layout of one 32x32 block: lane l, register i = 0..15 holds row
// 8*(i/4) + 4*(l >> 5) + (i & 3) and column (l & 31) of the block.
//
// Columns are interleaved across the NB blocks of a wave tile: LDS row
// nb*32 + q of the wave tile holds operand column NB*q + nb. Block nb's
// column q is therefore tile column NB*q + nb, and every lane owns NB
// consecutive output columns of each of its rows, so epilogues read and write
// NB-wide vectors.

template <typename T, int BM_, int BN_, int BK_, int WGM_, int WGN_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_;
  static_assert(WGM * WGN == 4, "4 waves per block");
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;
  static constexpr int MB = WTM / 32, NB = WTN / 32;
  static_assert(MB >= 1 && NB >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "tile");
  static_assert(BK % 16 == 0, "BK must be a multiple of 16");
  static constexpr int S = BK + 16 / static_cast<int>(sizeof(T));  // LDS row stride
  static constexpr int kLdsElems = (BM + BN) * S;

  __device__ __forceinline__ static int wave_m(int wave) { return wave % WGM; }
  __device__ __forceinline__ static int wave_n(int wave) { return wave / WGM; }
  // LDS row that holds B-operand column c of the tile.
  __device__ __forceinline__ static int b_row(int c) {
    const int wn = c / WTN, cl = c - wn * WTN;
    return wn * WTN + (cl % NB) * 32 + cl / NB;
  }
  // Tile row of accumulator register i of block mb.
  __device__ __forceinline__ static int acc_row(int wm, int mb, int i, int lane) {
    return wm * WTM + mb * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
  }
  // Tile column of block nb in this lane.
  __device__ __forceinline__ static int acc_col(int wn, int nb, int lane) {
    return wn * WTN + NB * (lane & 31) + nb;
  }
};

struct IdentityRows {
  __device__ __forceinline__ static int map(int c) { return c; }
};
template <class Tl>
struct BOperandRows {
  __device__ __forceinline__ static int map(int c) { return Tl::b_row(c); }
};

template <int MB, int NB>
struct Acc {
  f32x16 v[MB][NB];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int a = 0; a < MB; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) v[a][b][i] = 0.0f;
  }
  __device__ __forceinline__ void scale(float s) {
#pragma unroll
    for (int a = 0; a < MB; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) v[a][b][i] *= s;
  }
  __device__ __forceinline__ float sum_sq() const {
    float s = 0.0f;
#pragma unroll
    for (int a = 0; a < MB; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) s = fmaf(v[a][b][i], v[a][b][i], s);
    return s;
  }
};

// One BK-deep step of matrix-core work from LDS.
template <typename T, class Tl> struct Mma;

template <class Tl>
struct Mma<bf16, Tl> {
  __device__ __forceinline__ static void run(const bf16* sA, const bf16* sB,
                                             Acc<Tl::MB, Tl::NB>& acc, int wm,
                                             int wn, int lane) {
    const int r = lane & 31, kq = (lane >> 5) * 8;
#pragma unroll
    for (int kk = 0; kk < Tl::BK; kk += 16) {
      bf16x8 a[Tl::MB], b[Tl::NB];
#pragma unroll
      for (int mb = 0; mb < Tl::MB; ++mb)
        a[mb] = *reinterpret_cast<const bf16x8*>(
            sA + (wm * Tl::WTM + mb * 32 + r) * Tl::S + kk + kq);
#pragma unroll
      for (int nb = 0; nb < Tl::NB; ++nb)
        b[nb] = *reinterpret_cast<const bf16x8*>(
            sB + (wn * Tl::WTN + nb * 32 + r) * Tl::S + kk + kq);
#pragma unroll
      for (int mb = 0; mb < Tl::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < Tl::NB; ++nb)
          acc.v[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              a[mb], b[nb], acc.v[mb][nb], 0, 0, 0);
    }
  }
};

template <class Tl>
struct Mma<float, Tl> {
  __device__ __forceinline__ static void run(const float* sA, const float* sB,
                                             Acc<Tl::MB, Tl::NB>& acc, int wm,
                                             int wn, int lane) {
    const int r = lane & 31, kq = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < Tl::BK; kk += 2) {
      float a[Tl::MB], b[Tl::NB];
#pragma unroll
      for (int mb = 0; mb < Tl::MB; ++mb)
        a[mb] = sA[(wm * Tl::WTM + mb * 32 + r) * Tl::S + kk + kq];
#pragma unroll
      for (int nb = 0; nb < Tl::NB; ++nb)
        b[nb] = sB[(wn * Tl::WTN + nb * 32 + r) * Tl::S + kk + kq];
#pragma unroll
      for (int mb = 0; mb < Tl::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < Tl::NB; ++nb)
          acc.v[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(
              a[mb], b[nb], acc.v[mb][nb], 0, 0, 0);
    }
  }
};

// Loads ROWS x BK of a K-contiguous source (row stride ld elements; rows
// >= nrows and columns >= K read as zero) into registers, then stores source
// row c into LDS row Map::map(c). VEC: 16-byte loads (needs ld % (16 /
// sizeof(T)) == 0 and a 16-byte aligned base); otherwise element loads.
template <typename T, int ROWS, int BK, bool VEC, class Map>
struct RowsLoader {
  typedef typename Vec16<T>::type V;
  static constexpr int VN = Vec16<T>::N;
  static constexpr int CPR = BK / VN;                // chunks per row
  static constexpr int PER = ROWS * CPR / kThreads;  // chunks per thread
  static_assert(PER >= 1 && (ROWS * CPR) % kThreads == 0, "bad tiling");
  static constexpr int S = BK + VN;

  int64_t ld;
  int nrows;
  int K;
  V reg[PER];

  // off32: every byte offset of the tile from `base` fits in 32 bits (lets
  // a full tile use block-uniform base + 32-bit lane offset addressing).
  // FULL: the caller guarantees a full tile with off32 (the edge code is not
  // compiled, which also keeps the loads free of data-dependent branches).
  template <bool FULL = false>
  __device__ __forceinline__ void load(const T* base, int k0, int tid,
                                       bool off32) {
    static_assert(!FULL || VEC, "full tiles use 16-byte loads");
    if (FULL || (VEC && off32 && nrows >= ROWS && k0 + BK <= K)) {
      const char* bb = reinterpret_cast<const char*>(base);
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int ci = tid + p * kThreads;
        const uint32_t off = (static_cast<uint32_t>(ci / CPR) * static_cast<uint32_t>(ld) +
                              static_cast<uint32_t>(k0 + (ci % CPR) * VN)) * sizeof(T);
        reg[p] = *reinterpret_cast<const V*>(bb + off);
      }
      return;
    }
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int ci = tid + p * kThreads;
      const int row = ci / CPR;
      const int k = k0 + (ci % CPR) * VN;
      V v;
#pragma unroll
      for (int q = 0; q < VN; ++q) v[q] = zero_val<T>();
      if (row < nrows && k < K) {
        const T* src = base + static_cast<int64_t>(row) * ld + k;
        if constexpr (VEC) {
          v = *reinterpret_cast<const V*>(src);
          if (k + VN > K) {
#pragma unroll
            for (int q = 0; q < VN; ++q)
              if (k + q >= K) v[q] = zero_val<T>();
          }
        } else {
#pragma unroll
          for (int q = 0; q < VN; ++q)
            if (k + q < K) v[q] = src[q];
        }
      }
      reg[p] = v;
    }
  }

  __device__ __forceinline__ void store(T* sX, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int ci = tid + p * kThreads;
      const int row = Map::map(ci / CPR);
      const int kc = (ci % CPR) * VN;
      *reinterpret_cast<V*>(sX + row * S + kc) = reg[p];
    }
  }
};

// Loads BK x COLS of an N-contiguous source X[k][n] (row stride ld) and
// stores it transposed into LDS (column c -> LDS row Map::map(c), k
// contiguous), so that the contraction index ends up contiguous for the
// matrix cores. Rows >= K and columns >= ncols read as zero. Each thread
// gathers 8 consecutive k of one or two columns.
template <typename T, int COLS, int BK, bool PAIR, class Map>
struct ColsLoader;

// bf16, PAIR: 32-bit loads (2 columns) from 8 consecutive rows, split into
// two 8-element k-vectors (needs an even ld, an even column offset of the
// base and a 4-byte aligned base).
// BUF: full tiles are read with buffer loads (one lane offset, block-uniform
// row offsets). This is used where the 64-bit address arithmetic of the plain
// loads made the compiler wait for a step's first prefetched loads before it
// issued the rest.
template <int COLS, int BK, class Map, bool BUF = false>
struct ColsLoaderPair {
  static constexpr int S = BK + 8;
  static constexpr int ITEMS = (COLS / 2) * (BK / 8);
  static constexpr int PER = ITEMS / kThreads;
  static_assert(PER >= 1 && ITEMS % kThreads == 0, "bad tiling");
  int64_t ld;
  int ncols;
  int K;
  uint32_t w[PER][8];

  template <bool FULL = false>
  __device__ __forceinline__ void load(const bf16* base, int k0, int tid,
                                       bool off32) {
    if constexpr (FULL && BUF) {
      // item p: columns 2 (tid % (COLS / 2)) + 0..1, rows k0 + 8 (tid /
      // (COLS / 2) + p kThreads / (COLS / 2)) + j; all but the lane part is
      // block-uniform
      static_assert(kThreads % (COLS / 2) == 0, "a thread keeps its column pair");
      const __amdgpu_buffer_rsrc_t rs = tile_rsrc(base);
      const uint32_t stride = static_cast<uint32_t>(ld) * 2u;
      const uint32_t lo = static_cast<uint32_t>(tid / (COLS / 2)) * 8u * stride +
                          static_cast<uint32_t>(tid % (COLS / 2)) * 4u;
#pragma unroll
      for (int p = 0; p < PER; ++p) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t so = __builtin_amdgcn_readfirstlane(
              (static_cast<uint32_t>(k0) +
               static_cast<uint32_t>(p * (kThreads / (COLS / 2)) * 8 + j)) * stride);
          w[p][j] = __builtin_amdgcn_raw_buffer_load_b32(rs, lo, so, 0);
        }
      }
      return;
    }
    if (FULL || (off32 && ncols >= COLS && k0 + BK <= K)) {
      const char* bb = reinterpret_cast<const char*>(base);
      const uint32_t stride = static_cast<uint32_t>(ld) * 2u;
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int it = tid + p * kThreads;
        const uint32_t c = (it % (COLS / 2)) * 2;
        const uint32_t k = k0 + (it / (COLS / 2)) * 8;
        const uint32_t off = k * stride + c * 2u;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          w[p][j] = *reinterpret_cast<const uint32_t*>(bb + off + j * stride);
      }
      return;
    }
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int it = tid + p * kThreads;
      const int c = (it % (COLS / 2)) * 2;
      const int k = k0 + (it / (COLS / 2)) * 8;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t x = 0;
        if (k + j < K) {
          const bf16* src = base + static_cast<int64_t>(k + j) * ld + c;
          if (c + 1 < ncols) {
            x = *reinterpret_cast<const uint32_t*>(src);
          } else if (c < ncols) {
            x = static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(src));
          }
        }
        w[p][j] = x;
      }
    }
  }

  __device__ __forceinline__ void store(bf16* sX, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int it = tid + p * kThreads;
      const int c = (it % (COLS / 2)) * 2;
      const int kc = (it / (COLS / 2)) * 8;
      u32x4 lo, hi;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t a = w[p][2 * j], b = w[p][2 * j + 1];
        lo[j] = (a & 0xFFFFu) | (b << 16);
        hi[j] = (a >> 16) | (b & 0xFFFF0000u);
      }
      *reinterpret_cast<u32x4*>(sX + Map::map(c) * S + kc) = lo;
      *reinterpret_cast<u32x4*>(sX + Map::map(c + 1) * S + kc) = hi;
    }
  }
};

template <int COLS, int BK, class Map>
struct ColsLoader<bf16, COLS, BK, true, Map> : ColsLoaderPair<COLS, BK, Map, false> {};

// bf16, element loads (odd row stride or unaligned base).
template <int COLS, int BK, class Map>
struct ColsLoader<bf16, COLS, BK, false, Map> {
  static constexpr int S = BK + 8;
  static constexpr int ITEMS = COLS * (BK / 8);
  static constexpr int PER = ITEMS / kThreads;
  static_assert(PER >= 1 && ITEMS % kThreads == 0, "bad tiling");
  int64_t ld;
  int ncols;
  int K;
  uint32_t h[PER][4];  // 8 bf16 packed in pairs

  template <bool FULL = false>
  __device__ __forceinline__ void load(const bf16* base, int k0, int tid, bool) {
    static_assert(!FULL, "element loads have no full-tile form");
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int it = tid + p * kThreads;
      const int c = it % COLS;
      const int k = k0 + (it / COLS) * 8;
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        uint32_t lo = 0, hi = 0;
        if (c < ncols) {
          if (k + j < K)
            lo = *reinterpret_cast<const uint16_t*>(
                base + static_cast<int64_t>(k + j) * ld + c);
          if (k + j + 1 < K)
            hi = *reinterpret_cast<const uint16_t*>(
                base + static_cast<int64_t>(k + j + 1) * ld + c);
        }
        h[p][j / 2] = lo | (hi << 16);
      }
    }
  }

  __device__ __forceinline__ void store(bf16* sX, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int it = tid + p * kThreads;
      const int c = it % COLS;
      const int kc = (it / COLS) * 8;
      u32x4 v;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = h[p][j];
      *reinterpret_cast<u32x4*>(sX + Map::map(c) * S + kc) = v;
    }
  }
};

// fp32: a thread loads one column from 4 consecutive rows (4-byte loads,
// consecutive lanes on consecutive columns) and stores one 16-byte k-vector.
template <int COLS, int BK, bool PAIR, class Map>
struct ColsLoader<float, COLS, BK, PAIR, Map> {
  static constexpr int S = BK + 4;
  static constexpr int ITEMS = COLS * (BK / 4);
  static constexpr int PER = ITEMS / kThreads;
  static_assert(PER >= 1 && ITEMS % kThreads == 0, "bad tiling");
  int64_t ld;
  int ncols;
  int K;
  f32x4 reg[PER];

  template <bool FULL = false>  // one form for every tile
  __device__ __forceinline__ void load(const float* base, int k0, int tid, bool) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int it = tid + p * kThreads;
      const int c = it % COLS;
      const int k = k0 + (it / COLS) * 4;
      f32x4 v;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v[j] = (k + j < K && c < ncols)
                   ? base[static_cast<int64_t>(k + j) * ld + c]
                   : 0.0f;
      reg[p] = v;
    }
  }

  __device__ __forceinline__ void store(float* sX, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int it = tid + p * kThreads;
      const int c = it % COLS;
      const int kc = (it / COLS) * 4;
      *reinterpret_cast<f32x4*>(sX + Map::map(c) * S + kc) = reg[p];
    }
  }
};

// Runs n_steps BK-deep steps. load_step(s) issues the global loads of step s
// into the loaders' registers; the loads of step s + 1 are in flight while
// step s runs on the matrix cores. prologue() runs once, after the loads of
// step 0 are issued and before the first barrier (its LDS writes are visible
// to pre_step). pre_step(s) runs before step s is accumulated and returns
// whether to accumulate it (the same value in every thread of the block);
// after_step(s) runs once step s has been accumulated.
template <typename T, class Tl, class LA, class LB, class LoadStep, class Prologue,
          class PreStep, class AfterStep>
__device__ __forceinline__ void run_steps(LA& la, LB& lb, T* smem,
                                          Acc<Tl::MB, Tl::NB>& acc, int n_steps,
                                          int tid, LoadStep load_step,
                                          Prologue prologue, PreStep pre_step,
                                          AfterStep after_step) {
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = Tl::wave_m(wave), wn = Tl::wave_n(wave);
  T* sA = smem;
  T* sB = smem + Tl::BM * Tl::S;
  if (n_steps <= 0) return;
  load_step(0);
  prologue();
  for (int s = 0; s < n_steps; ++s) {
    __syncthreads();  // the previous step finished reading LDS
    la.store(sA, tid);
    lb.store(sB, tid);
    __syncthreads();
    if (s + 1 < n_steps) load_step(s + 1);
    if (pre_step(s)) Mma<T, Tl>::run(sA, sB, acc, wm, wn, lane);
    after_step(s);
  }
}

template <typename T, class Tl, class LA, class LB, class LoadStep, class AfterStep>
__device__ __forceinline__ void run_steps(LA& la, LB& lb, T* smem,
                                          Acc<Tl::MB, Tl::NB>& acc, int n_steps,
                                          int tid, LoadStep load_step,
                                          AfterStep after_step) {
  run_steps<T, Tl>(la, lb, smem, acc, n_steps, tid, load_step, [] {},
                   [](int) { return true; }, after_step);
}

// Blocks are dispatched round-robin over the 8 XCDs (each with its own L2).
// This maps the hardware block id to a logical id so that consecutive
// logical blocks run on the same XCD; gridDim.x must be a multiple of 8.
__device__ __forceinline__ int xcd_logical_block() {
  const int per = gridDim.x >> 3;
  return (blockIdx.x & 7) * per + (blockIdx.x >> 3);
}

}  // namespace dpg
