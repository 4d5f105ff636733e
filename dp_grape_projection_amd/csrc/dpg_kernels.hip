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
//   proj    Xt_l[b][j][t] = sum_k P_l[j][k] A_l[b][t][k] (one GEMM over all
//           B*T rows, split over d_in when that balances the chip)
//   xsum    sums the split partials of Xt (only for split layers)
//   norm    for every (sample, tile): ||Xt_il dY_il||_F^2 partials
//   scale   n_i = sqrt(sum of partials over all layers), s_i = min(1, C/n_i)
//   sum     sum_i s_i Xt_il dY_il over groups of samples (second pass)
//   fin     G_priv = (sum over groups + sigma C Z) / B
// and the update call runs
//   prep    Adam on [r][d_out] (m, v in place; U row-major) and P regenerated
//   back    W -= lr P^T U
#include <type_traits>

#include "dpg_device.hpp"
#include "dpg_internal.hpp"

namespace dpg {

template <typename T> struct StepK { static constexpr int v = sizeof(T) == 2 ? kStepBf16 : kStepF32; };
template <typename T> using MainTile = Tile<T, kTileM, kTileN, StepK<T>::v, 4, 1>;

template <typename T> struct Vec4;
template <> struct Vec4<bf16> { typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 type; };
template <> struct Vec4<float> { typedef f32x4 type; };

// The layer of block b among n: the last one whose first block is <= b
// (first blocks are non-decreasing, the unused entries INT32_MAX). The array
// is read with wide scalar loads in flight together (its first 16 entries
// always, the rest only for launches of more than 16 layers); the selects
// stay on the scalar unit.
__device__ __forceinline__ int find_layer(const int32_t (&first)[kMaxLayers], int n, int b) {
  int l = 0;
#pragma unroll
  for (int i = 1; i < 16; ++i) l = b >= first[i] ? i : l;
  if (n > 16) {
#pragma unroll
    for (int i = 16; i < kMaxLayers; ++i) l = b >= first[i] ? i : l;
  }
  return l;
}

// Sum over the 64 lanes of a wave (butterfly, deterministic).
// Caller pointers are only element aligned; vector accesses to them are
// taken when the pointer allows them (the test is uniform per layer).
__device__ __forceinline__ bool is_aligned(const void* p, unsigned bytes) {
  return (reinterpret_cast<uintptr_t>(p) & (bytes - 1)) == 0;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
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

// Four values of T at dst (dst 4-element aligned).
template <typename T>
__device__ __forceinline__ void store4(T* dst, float a, float b, float c, float d) {
  typename Vec4<T>::type v;
  v[0] = from_float<T>(a);
  v[1] = from_float<T>(b);
  v[2] = from_float<T>(c);
  v[3] = from_float<T>(d);
  *reinterpret_cast<typename Vec4<T>::type*>(dst) = v;
}

// ------------------------------------------------------------------ gen_p --

// One thread per Philox counter c of one layer: elements e = 4c .. 4c+3 of
// P (row-major, row stride ld).
template <typename T>
__device__ __forceinline__ void gen_p_thread(const GenPLayer& L, int c, int r,
                                             float scale, const StreamKey& key) {
  if (c >= L.n_ctr) return;
  float z[4];
  normals_at(key, L.layer_id, static_cast<uint32_t>(c), z);
  const uint64_t total = static_cast<uint64_t>(r) * L.d_in;
  const uint64_t e = 4ull * static_cast<uint64_t>(c);
  uint32_t j = static_cast<uint32_t>(e / L.d_in);
  uint32_t k = static_cast<uint32_t>(e - static_cast<uint64_t>(j) * L.d_in);
  T* out = static_cast<T*>(L.out);
  if ((L.d_in & 3) == 0 && (L.ld & 3) == 0) {
    // the four elements lie in one row, 4-aligned
    store4<T>(out + static_cast<int64_t>(j) * L.ld + k, z[0] * scale,
              z[1] * scale, z[2] * scale, z[3] * scale);
    return;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (e + q < total)
      out[static_cast<int64_t>(j) * L.ld + k] = from_float<T>(z[q] * scale);
    if (++k == static_cast<uint32_t>(L.d_in)) {
      k = 0;
      ++j;
    }
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void gen_p_kernel(const GenPArgs a) {
  const int b = blockIdx.x;
  const GenPLayer& L = a.L[find_layer(a.first_block, a.n_layers, b)];
  const StreamKey key{a.k0, a.k1, a.step_word, a.tag};
  gen_p_thread<T>(L, (b - L.block0) * kThreads + static_cast<int>(threadIdx.x),
                  a.r, a.scale, key);
}

// ------------------------------------------------------------------- proj --

// FULL: every tile of the launch is full (see ProjArgs::full); the loads are
// compiled without their edge code.
// NG = 2: the block has two groups of 4 waves that take alternate K steps of
// the block's range (each with its own LDS tiles), and the second group's
// accumulator is added into the first's through LDS at the end. This gives
// 8 waves per block without more split partials.
template <typename T, bool VEC, bool FULL, int NG>
__global__ __launch_bounds__(kThreads * NG, 3 - NG) void proj_kernel(const ProjArgs a) {
  typedef MainTile<T> Tl;
  __shared__ __attribute__((aligned(16))) T smem_all[NG * Tl::kLdsElems];
  const int grp = NG == 1 ? 0 : static_cast<int>(threadIdx.x) / kThreads;
  T* smem = smem_all + grp * Tl::kLdsElems;
  const int lb = xcd_logical_block();
  if (lb >= a.n_blocks) return;
  const ProjLayer& L = a.L[find_layer(a.first_block, a.n_layers, lb)];
  const int local = lb - L.block0;
  const int mt = local % L.m_tiles;
  const int rest = local / L.m_tiles;
  const int nt = rest % L.n_tiles;
  const int split = rest / L.n_tiles;
  const int j0 = mt * Tl::BM, n0 = nt * Tl::BN;
  const int BT = a.B * a.T;
  const int tid = static_cast<int>(threadIdx.x) % kThreads, lane = tid & 63, wave = tid >> 6;
  const int n_steps_all = (L.d_in + Tl::BK - 1) / Tl::BK;
  const int s_begin = split * L.steps_per_split;
  const int s_end = min(n_steps_all, s_begin + L.steps_per_split);
  // this group's steps: s_begin + grp, + NG, ...; both groups run the same
  // number of iterations (the barriers are shared), the second one's last
  // one empty when the range is odd (it loads the last real step again)
  const int n_iter = (s_end - s_begin + NG - 1) / NG;

  RowsLoader<T, Tl::BM, Tl::BK, true, IdentityRows> la{L.ldp, a.r - j0, L.d_in, {}};
  RowsLoader<T, Tl::BN, Tl::BK, VEC, BOperandRows<Tl>> lx{L.d_in, BT - n0, L.d_in, {}};
  const T* Pb = static_cast<const T*>(L.P) + static_cast<int64_t>(j0) * L.ldp;
  const T* Ab = static_cast<const T*>(L.A) + static_cast<int64_t>(n0) * L.d_in;
  Acc<Tl::MB, Tl::NB> acc;
  acc.zero();
  run_steps<T, Tl>(
      la, lx, smem, acc, n_iter, tid,
      [&](int q) {
        const int k0 = min(s_begin + q * NG + grp, s_end - 1) * Tl::BK;
        la.template load<FULL>(Pb, k0, tid, a.off32);
        lx.template load<FULL>(Ab, k0, tid, a.off32);
      },
      [] {}, [&](int q) { return s_begin + q * NG + grp < s_end; }, [](int) {});
  if constexpr (NG == 2) {
    // second group's accumulator into the first's, element by element
    // (thread tid of both groups holds the same elements)
    float* red = reinterpret_cast<float*>(smem_all);
    constexpr int kAcc = Tl::MB * Tl::NB * 16;
    static_assert(kAcc * kThreads * sizeof(float) <= NG * Tl::kLdsElems * sizeof(T),
                  "LDS holds one group's accumulator");
    __syncthreads();  // every wave finished its last step's LDS reads
    if (grp == 1) {
#pragma unroll
      for (int nb = 0; nb < Tl::NB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) red[(nb * 16 + i) * kThreads + tid] = acc.v[0][nb][i];
    }
    __syncthreads();
    if (grp == 1) return;
#pragma unroll
    for (int nb = 0; nb < Tl::NB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc.v[0][nb][i] += red[(nb * 16 + i) * kThreads + tid];
  }

  // Each lane owns 4 consecutive columns n (= rows of A) of 16 rows j.
  const int wm = Tl::wave_m(wave);
  const int nq = n0 + Tl::acc_col(0, 0, lane);  // first of the 4 columns
  if (L.splits == 1) {
    T* Xt = static_cast<T*>(L.Xt);
    if ((a.T & 3) == 0) {
      if (nq >= BT) return;
      const int bi = nq / a.T, t = nq - bi * a.T;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = j0 + Tl::acc_row(wm, 0, i, lane);
        if (j < a.r)
          store4<T>(Xt + (static_cast<int64_t>(bi) * a.r + j) * a.ldt + t,
                    acc.v[0][0][i], acc.v[0][1][i], acc.v[0][2][i], acc.v[0][3][i]);
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int n = nq + nb;
        if (n >= BT) continue;
        const int bi = n / a.T, t = n - bi * a.T;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = j0 + Tl::acc_row(wm, 0, i, lane);
          if (j < a.r)
            Xt[(static_cast<int64_t>(bi) * a.r + j) * a.ldt + t] =
                from_float<T>(acc.v[0][nb][i]);
        }
      }
    }
  } else {
    float* part = L.part + static_cast<int64_t>(split) * a.r * BT;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = j0 + Tl::acc_row(wm, 0, i, lane);
      if (j >= a.r) continue;
      float* dst = part + static_cast<int64_t>(j) * BT + nq;
      if ((BT & 3) == 0) {
        if (nq < BT)
          *reinterpret_cast<f32x4*>(dst) = f32x4{acc.v[0][0][i], acc.v[0][1][i],
                                                 acc.v[0][2][i], acc.v[0][3][i]};
      } else {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          if (nq + nb < BT) dst[nb] = acc.v[0][nb][i];
      }
    }
  }
}

// buf[j] = the 16 bytes at src + j * stride for j < n (1 <= n <= kSumBatch),
// every load issued before any is used: the switch enters a straight run of
// loads, so no wait falls between them, and no load is repeated.
__device__ __forceinline__ void load_batch(f32x4 (&buf)[kSumBatch], const float* src,
                                           int64_t stride, int n) {
  static_assert(kSumBatch == 8, "one case per batch size");
  switch (n) {
    default:
      buf[7] = *reinterpret_cast<const f32x4*>(src + 7 * stride);
      [[fallthrough]];
    case 7:
      buf[6] = *reinterpret_cast<const f32x4*>(src + 6 * stride);
      [[fallthrough]];
    case 6:
      buf[5] = *reinterpret_cast<const f32x4*>(src + 5 * stride);
      [[fallthrough]];
    case 5:
      buf[4] = *reinterpret_cast<const f32x4*>(src + 4 * stride);
      [[fallthrough]];
    case 4:
      buf[3] = *reinterpret_cast<const f32x4*>(src + 3 * stride);
      [[fallthrough]];
    case 3:
      buf[2] = *reinterpret_cast<const f32x4*>(src + 2 * stride);
      [[fallthrough]];
    case 2:
      buf[1] = *reinterpret_cast<const f32x4*>(src + stride);
      [[fallthrough]];
    case 1:
      buf[0] = *reinterpret_cast<const f32x4*>(src);
  }
}

// Large projections (bf16): a block computes a 256 (rows j of P) x 256
// (rows n of A) tile of X^T over its K range in steps of 64. Each step's two
// operand tiles (256 rows x 128 bytes each) are copied into LDS by direct
// global-to-LDS loads, one step ahead of the matrix cores (two stages). A
// row's eight 16-byte chunks are stored XOR-swizzled by a function of the row
// so that the rows an MFMA operand read touches spread over the banks: a
// 16-byte LDS read serves 16 lanes (256 bytes) at a time, and rows of 128
// bytes put even rows in one half of the 64 banks and odd rows in the other,
// so chunk c of row R goes to slot c ^ (R / 2 mod 8), which gives the 16
// consecutive rows of a lane group 16 different bank ranges. 16 waves, 4
// (j) x 4 (n), four on each SIMD; each computes 64 x 64 with 32x32x16
// MFMAs. (8 waves of 128 x 64 read a third fewer fragments a step, but two
// waves on a SIMD hide less LDS and barrier latency: at dec24 the 16-wave
// form is 5 % faster, at long1 3 % slower.)
typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void gbl_void_t;

// vmcnt(n) (n < 64) with the other counters left alone.
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {  // the encoding must be an immediate
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 12: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;  // (stricter: wait for all)
  }
}
// lgkmcnt(0) with the other counters left alone.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One direct global-to-LDS copy of 16 bytes per lane through a buffer
// resource: lane offset `voff` (kept in a register across a loop) plus the
// block-uniform `soff`; the 1 KiB a wave copies lands at `lds` (uniform).
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                            uint32_t soff, char* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)lds, 16, voff,
                                           __builtin_amdgcn_readfirstlane(soff), 0, 0);
}

// 16-byte LDS read of a matrix-core fragment through a restrict-qualified
// pointer: the alias-scope information lets the compiler keep the read clear
// of the direct global-to-LDS copies in flight (without it, it may wait for
// all of them first; the kernels order copies and reads themselves).
__device__ __forceinline__ bf16x8 lds_read_b128(const char* __restrict__ p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ float lds_read_f32(const float* __restrict__ p) { return *p; }

// BK: K step (elements). Two stages of P and three of A; rows of a stage
// are BK * 2 bytes in CH chunks of 16 bytes; chunk c of row R sits in slot
// c ^ (R / 2 mod CH).
//
// Matrix-core schedule: a wave's fragments are double-buffered over the K
// sub-steps of 16 and across steps. In each sub-step the wave issues one
// MFMA (its operand wait then covers only the reads issued during the
// previous sub-step), then the next sub-step's fragment reads, then the other
// three MFMAs, so LDS latency hides behind matrix-core work. In the last
// sub-step of step s, after two MFMAs, every wave has read all of step s:
// it waits for its copies of step s + 1, meets the others at the barrier,
// refills P's stage of step s with step s + 2 and A's with step s + 3, and
// reads the first fragments of step s + 1 while the remaining two MFMAs
// run.
template <int BK>
__global__ __launch_bounds__(4 * kThreads, 1) void proj_big_kernel(const ProjArgs a) {
  constexpr int kRowBytes = BK * 2;
  constexpr int CH = kRowBytes / 16;                 // chunks per row
  constexpr int kRowsPerCopy = 1024 / kRowBytes;      // rows per 1 KiB copy
  constexpr int kCopiesPerTile = kBigM / kRowsPerCopy;
  constexpr int kCopiesPerWave = 2 * kCopiesPerTile / 16;  // per step
  constexpr int kTileBytes = kBigM * kRowBytes;
  constexpr int KK = BK / 16;                         // sub-steps per step
  static_assert(kBigM == kBigN && BK % 16 == 0 && (CH & (CH - 1)) == 0 && KK >= 2, "tile shape");
  static_assert(kCopiesPerWave * 16 == 2 * kCopiesPerTile, "copies per wave");
  // Three stages of the A tile (the operand streamed from HBM, whose copies
  // run two steps ahead of their use) and two of P (L2-resident): 160 KiB.
  constexpr int NA = 3;
  constexpr int kCopiesA = kCopiesPerWave / 2;       // per wave and step, of each operand
  __shared__ __attribute__((aligned(1024))) char smem[(2 + NA) * kTileBytes];
  const int lb = xcd_logical_block();
  if (lb >= a.n_blocks) return;
  const ProjLayer& L = a.L[find_layer(a.first_block, a.n_layers, lb)];
  const int local = lb - L.block0;
  const int mt = local % L.m_tiles;
  const int rest = local / L.m_tiles;
  const int nt = rest % L.n_tiles;
  const int split = rest / L.n_tiles;
  const int j0 = mt * kBigM, n0 = nt * kBigN;
  const int BT = a.B * a.T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 3, wn = wave >> 2;
  const int n_steps_all = L.d_in / BK;
  const int s_begin = split * L.steps_per_split;
  const int s_end = min(n_steps_all, s_begin + L.steps_per_split);
  const int n_steps = s_end - s_begin;
  const int64_t p_row = static_cast<int64_t>(L.ldp) * 2, a_row = static_cast<int64_t>(L.d_in) * 2;
  // 16 consecutive rows (the rows a 16-lane group reads) cover both halves
  // of the 64 banks with 8 different slots each
  auto slot = [](int R, int c) { return c ^ ((R >> 1) & (CH - 1)); };

  // Copies K step `step` into stage `stage`: copy q of wave w fills row
  // block g = q * 16 + w (P blocks first, then A blocks); lane l writes slot
  // l % CH of row l / CH of the block, loading the chunk that the swizzle
  // puts there (it is an involution). A block's index has the parity of w,
  // so each lane's offset within its block is the same for every copy of a
  // wave and stays in a register: copies go through buffer resources on P
  // and A (the plan keeps both within 32-bit offsets), the block and step in
  // the uniform offset.
  static_assert(CH == 8 && kRowsPerCopy == 8 && kCopiesPerTile % 2 == 0, "copy layout");
  const __amdgpu_buffer_rsrc_t rsP = tile_rsrc(L.P), rsA = tile_rsrc(L.A);
  const uint32_t p_rb = static_cast<uint32_t>(p_row), a_rb = static_cast<uint32_t>(a_row);
  const uint32_t chunk = static_cast<uint32_t>(((lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7)) << 4);
  const uint32_t voffP = static_cast<uint32_t>(lane >> 3) * p_rb + chunk;
  const uint32_t voffA = static_cast<uint32_t>(lane >> 3) * a_rb + chunk;
  // P stage q at q * kTileBytes (q < 2), A stage q at (2 + q) * kTileBytes
  auto issue_p = [&](int step, int stage) {
    char* sb = smem + stage * kTileBytes;
    const uint32_t kb = static_cast<uint32_t>(s_begin + step) * kRowBytes;
#pragma unroll
    for (int q = 0; q < kCopiesA; ++q) {
      const int gi = q * 16 + wave;
      const uint32_t row0 = static_cast<uint32_t>(j0 + gi * kRowsPerCopy);
      copy_to_lds(rsP, voffP, row0 * p_rb + kb, sb + gi * 1024);
    }
  };
  auto issue_a = [&](int step, int stage) {
    char* sb = smem + (2 + stage) * kTileBytes;
    const uint32_t kb = static_cast<uint32_t>(s_begin + step) * kRowBytes;
#pragma unroll
    for (int q = 0; q < kCopiesA; ++q) {
      const int gi = q * 16 + wave;
      const uint32_t row0 = static_cast<uint32_t>(n0 + gi * kRowsPerCopy);
      copy_to_lds(rsA, voffA, row0 * a_rb + kb, sb + gi * 1024);
    }
  };

  Acc<2, 2> acc;
  acc.zero();
  const int r32 = lane & 31, kh = lane >> 5;
  // fragments of sub-step kk of the step in stage `stage`: this lane's
  // 16-byte chunk is k = 16 kk + 8 kh
  auto read_frags = [&](int step, int kk, bf16x8* af, bf16x8* bfr) {
    const char* sP = smem + (step & 1) * kTileBytes;
    const char* sA = smem + (2 + step % NA) * kTileBytes;
    const int c = 2 * kk + kh;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int j = 64 * wm + 32 * mb + r32;
      af[mb] = lds_read_b128(sP + j * kRowBytes + slot(j, c) * 16);
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int n = 64 * wn + 32 * nb + r32;
      bfr[nb] = lds_read_b128(sA + n * kRowBytes + slot(n, c) * 16);
    }
  };
  // MFMAs q0 .. q1 - 1 of a sub-step's eight (q = 2 mb + nb)
  auto mma = [&](const bf16x8* af, const bf16x8* bfr, int q0, int q1) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (q >= q0 && q < q1)
        acc.v[q >> 1][q & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            af[q >> 1], bfr[q & 1], acc.v[q >> 1][q & 1], 0, 0, 0);
  };

  // Copies in issue order: P and A of step 0; P of step 1, A of steps 1 ..
  // NA - 1; then at the barrier ending step s, P of step s + 2 and A of
  // step s + NA. So before that barrier, step s + 1's copies are complete
  // once at most the A copies of step s + 2 (NA = 3) are still in flight:
  // loads return in order.
  bf16x8 fa[2][2], fb[2][2];
  int a_stage = 0;  // the A stage of step s: s mod NA
  if (n_steps > 0) {
    issue_p(0, 0);
    issue_a(0, 0);
    wait_vm(0);
    lds_barrier();
    if (n_steps > 1) {
      issue_p(1, 1);
      issue_a(1, 1);
    }
    if (n_steps > 2) issue_a(2, 2);
    read_frags(0, 0, fa[0], fb[0]);
  }
  for (int s = 0; s < n_steps; ++s) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int cur = kk & 1, nxt = cur ^ 1;
      const int first = kk + 1 < KK ? 1 : 2;
      __builtin_amdgcn_sched_barrier(0);
      mma(fa[cur], fb[cur], 0, first);
      __builtin_amdgcn_sched_barrier(0);
      if (kk + 1 < KK) {
        read_frags(s, kk + 1, fa[nxt], fb[nxt]);
      } else if (s + 1 < n_steps) {
        wait_lgkm0();  // this wave's reads of step s's stages are complete
        // its copies of step s + 1 landed
        if (s + 2 < n_steps) wait_vm(kCopiesA);
        else wait_vm(0);
        lds_barrier();
        if (s + 2 < n_steps) issue_p(s + 2, s & 1);
        if (s + NA < n_steps) issue_a(s + NA, a_stage);
        read_frags(s + 1, 0, fa[nxt], fb[nxt]);
      }
      __builtin_amdgcn_sched_barrier(0);
      mma(fa[cur], fb[cur], first, 4);
      __builtin_amdgcn_sched_barrier(0);
    }
    a_stage = a_stage + 1 == NA ? 0 : a_stage + 1;
  }

  // lane: column n0 + 64 wn + 32 nb + r32; registers i: rows
  // 8 (i / 4) + 4 kh + i % 4 of each 32-row block. Stores go through buffer
  // resources: one per-lane offset and uniform row offsets (the plan keeps
  // Xt and a split partial within 32-bit byte offsets).
  if (L.splits == 1) {
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(L.Xt);
    const uint32_t row2 = static_cast<uint32_t>(a.ldt) * 2u;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int n = n0 + 64 * wn + 32 * nb + r32;
      const int bi = n / a.T, t = n - bi * a.T;
      const uint32_t lo = (static_cast<uint32_t>(bi * a.r + j0 + 64 * wm + 4 * kh)) * row2 +
                          static_cast<uint32_t>(t) * 2u;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const bf16 v = from_float<bf16>(acc.v[mb][nb][i]);
          __builtin_amdgcn_raw_buffer_store_b16(
              __builtin_bit_cast(unsigned short, v), rs, lo,
              __builtin_amdgcn_readfirstlane(
                  static_cast<uint32_t>(32 * mb + 8 * (i >> 2) + (i & 3)) * row2),
              0);
        }
    }
  } else {
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(
        L.part + (static_cast<int64_t>(split) * a.r + j0 + 64 * wm) * BT);
    const uint32_t row4 = static_cast<uint32_t>(BT) * 4u;
    const uint32_t lo = static_cast<uint32_t>(4 * kh) * row4 +
                        static_cast<uint32_t>(n0 + 64 * wn + r32) * 4u;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float v = acc.v[mb][nb][i];
          __builtin_amdgcn_raw_buffer_store_b32(
              __builtin_bit_cast(uint32_t, v), rs, lo + 128u * nb,
              __builtin_amdgcn_readfirstlane(
                  static_cast<uint32_t>(32 * mb + 8 * (i >> 2) + (i & 3)) * row4),
              0);
        }
  }
}

// Xt[b][j][t] = sum over splits of part[s][j][b*T + t]; one thread per 4
// consecutive n of one row j.
template <typename T>
__global__ __launch_bounds__(kThreads) void xsum_kernel(const XsumArgs a) {
  const int b = blockIdx.x;
  const XsumLayer& L = a.L[find_layer(a.first_block, a.n_layers, b)];
  const int BT = a.B * a.T;
  const int per_row = (BT + 3) / 4;
  const int64_t idx = static_cast<int64_t>(b - L.block0) * kThreads + threadIdx.x;
  if (idx >= static_cast<int64_t>(per_row) * a.r) return;
  const int j = static_cast<int>(idx / per_row);
  const int n = static_cast<int>(idx - static_cast<int64_t>(j) * per_row) * 4;
  const int64_t plane = static_cast<int64_t>(a.r) * BT;
  const float* src = L.part + static_cast<int64_t>(j) * BT + n;
  T* Xt = static_cast<T*>(L.Xt);
  if ((a.T & 3) == 0) {
    // up to kSumBatch splits in flight together, added in split order
    const int last = L.splits - 1;
    f32x4 buf[kSumBatch];
    f32x4 s;
    for (int s0 = 0; s0 <= last; s0 += kSumBatch) {
      load_batch(buf, src + s0 * plane, plane, last + 1 - s0);
#pragma unroll
      for (int j = 0; j < kSumBatch; ++j) {
        const int sp = s0 + j;
        if (sp > last) break;
        if (sp == 0) {
          s = buf[0];
        } else {
          s[0] += buf[j][0];
          s[1] += buf[j][1];
          s[2] += buf[j][2];
          s[3] += buf[j][3];
        }
      }
    }
    const int bi = n / a.T, t = n - bi * a.T;
    store4<T>(Xt + (static_cast<int64_t>(bi) * a.r + j) * a.ldt + t, s[0], s[1],
              s[2], s[3]);
  } else {
    for (int q = 0; q < 4; ++q) {
      if (n + q >= BT) break;
      float s = src[q];
      for (int sp = 1; sp < L.splits; ++sp) s += src[q + sp * plane];
      const int bi = (n + q) / a.T, t = (n + q) - bi * a.T;
      Xt[(static_cast<int64_t>(bi) * a.r + j) * a.ldt + t] = from_float<T>(s);
    }
  }
}

// Stores a tile accumulator with waves 4 x 1 (each lane NB = 4 or 2
// consecutive columns of 16 rows) into dst = [r][d_out], rows j0 ..,
// columns n0 ..; rows >= r and columns >= d_out are skipped.
template <class Tl>
__device__ __forceinline__ void store_tile(float* dst, const Acc<Tl::MB, Tl::NB>& acc,
                                           int r, int d_out, int j0, int n0,
                                           int wave, int lane) {
  constexpr int NB = Tl::NB;
  static_assert(Tl::MB == 1 && (NB == 4 || NB == 2) && Tl::WGN == 1, "4 x 1 waves");
  const int wm = Tl::wave_m(wave);
  const int nq = n0 + Tl::acc_col(0, 0, lane);  // this lane's NB columns
  const bool vec = (d_out % NB) == 0 && nq + NB - 1 < d_out && is_aligned(dst, NB * 4);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int j = j0 + Tl::acc_row(wm, 0, i, lane);
    if (j >= r || nq >= d_out) continue;
    float* p = dst + static_cast<int64_t>(j) * d_out + nq;
    if (vec) {
      if constexpr (NB == 4)
        *reinterpret_cast<f32x4*>(p) =
            f32x4{acc.v[0][0][i], acc.v[0][1][i], acc.v[0][2][i], acc.v[0][3][i]};
      else
        *reinterpret_cast<f32x2*>(p) = f32x2{acc.v[0][0][i], acc.v[0][1][i]};
    } else {
#pragma unroll
      for (int q = 0; q < NB; ++q)
        if (nq + q < d_out) p[q] = acc.v[0][q][i];
    }
  }
}

// ---------------------------------------------------------- norm and sum --

// Norm mode: squared-norm partials of Xt_i dY_i per (sample, tile, wave).
// Sum mode: sum_i s_i Xt_i dY_i over a group of samples, into one fp32
// partial per (group, tile). The sum keeps a single accumulator R expressed
// in units of the current sample's clip factor: before sample i it is
// rescaled by c / s_i (c = the factor of the previous sample), the sample's
// product is added by the matrix cores, and the final R is multiplied by the
// last factor. A sample with s_i = 0 (its norm overflowed) is skipped.
template <typename T, int BN, bool PAIR, bool SUM, bool FULL>
__global__ __launch_bounds__(kThreads, 2) void samp_kernel(const SampArgs a) {
  typedef Tile<T, kTileM, BN, StepK<T>::v, 4, 1> Tl;
  __shared__ __attribute__((aligned(16))) T smem[Tl::kLdsElems];
  __shared__ float s_grp[SUM ? kSumMaxGroup : 1];  // the group's clip factors
  const int lb = xcd_logical_block();
  if (lb >= a.n_blocks) return;
  const int li = find_layer(a.first_block, a.n_layers, lb);
  const SampLayer& L = a.L[li];
  const int local = lb - L.block0;
  const int mt = local % L.m_tiles;
  const int rest = local / L.m_tiles;
  const int nt = rest % L.n_tiles;
  const int g = rest / L.n_tiles;  // run (norm) or group (sum) of samples
  const int j0 = mt * Tl::BM, n0 = nt * Tl::BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i_begin = g * a.per_block;
  const int i_end = min(a.B, i_begin + a.per_block);
  const int kc = (a.T + Tl::BK - 1) / Tl::BK;  // steps per sample

  RowsLoader<T, Tl::BM, Tl::BK, true, IdentityRows> la{a.ldt, a.r - j0, a.T, {}};
  // paired bf16 columns: the norm mode reads full tiles with buffer loads
  typename std::conditional<
      std::is_same<T, bf16>::value && PAIR,
      ColsLoaderPair<Tl::BN, Tl::BK, BOperandRows<Tl>, !SUM>,
      ColsLoader<T, Tl::BN, Tl::BK, PAIR, BOperandRows<Tl>>>::type lc{L.d_out, L.d_out - n0,
                                                                        a.T, {}};
  const T* Xt = static_cast<const T*>(L.Xt);
  const T* dY = static_cast<const T*>(L.dY);

  Acc<Tl::MB, Tl::NB> acc;
  acc.zero();
  float c = 0.0f;  // sum mode: factor R is expressed in (0 while R is empty)
  bool on = true;  // sum mode: the current sample is accumulated
  run_steps<T, Tl>(
      la, lc, smem, acc, (i_end - i_begin) * kc, tid,
      [&](int s) {
        const int i = i_begin + s / kc, k0 = (s % kc) * Tl::BK;
        la.template load<FULL>(Xt + (static_cast<int64_t>(i) * a.r + j0) * a.ldt, k0, tid, a.off32);
        lc.template load<FULL>(dY + static_cast<int64_t>(i) * a.T * L.d_out + n0, k0, tid, a.off32);
      },
      [&] {
        if (!SUM) return;
        if (!a.fuse_scale) {
          // the factors from the scale launch, so that every step reads them
          // from LDS (a load that may come from global memory would make the
          // step wait for the next step's prefetched tiles)
          for (int q = tid; q < i_end - i_begin; q += kThreads) s_grp[q] = a.scales[i_begin + q];
          return;
        }
        // Per-sample global norm and clip factor of this group: wave w takes
        // samples w, w + 4, ...; lane l adds slots l, l + 64, ... in order,
        // then the lanes are combined by a fixed butterfly. Every block of
        // the group computes the same values.
        const int jn = (a.n_slots + 63) >> 6;  // <= kFuseMaxSlots / 64
        for (int q = wave; q < i_end - i_begin; q += 4) {
          const float* p = a.norm_part + static_cast<int64_t>(i_begin + q) * a.n_slots;
          float v[kFuseMaxSlots / 64];
#pragma unroll
          for (int j = 0; j < kFuseMaxSlots / 64; ++j)
            if (j < jn) v[j] = p[min(lane + 64 * j, a.n_slots - 1)];
          float t = 0.0f;
#pragma unroll
          for (int j = 0; j < kFuseMaxSlots / 64; ++j)
            if (j < jn && lane + 64 * j < a.n_slots) t += v[j];
          const float n = sqrtf(wave_sum(t));
          if (lane == 0) {
            s_grp[q] = (n > a.clip_C) ? a.clip_C / n : 1.0f;
            if (a.norms_out && li == 0 && mt == 0 && nt == 0) a.norms_out[i_begin + q] = n;
          }
        }
      },
      [&](int s) -> bool {
        if (!SUM) return true;
        if (s % kc == 0) {
          const float si = s_grp[s / kc];
          on = si > 0.0f;
          if (on) {
            if (c != 0.0f && c != si) acc.scale(c / si);
            c = si;
          }
        }
        return on;
      },
      [&](int s) {
        if (SUM || s % kc != kc - 1) return;
        // Rows and columns outside the layer were loaded as zeros.
        const int i = i_begin + s / kc;
        const float t = wave_sum(acc.sum_sq());
        if (lane == 0)
          a.norm_part[static_cast<int64_t>(i) * a.n_slots +
                      4 * (L.slot0 + nt * L.m_tiles + mt) + wave] = t;
        if (L.ghat)
          store_tile<Tl>(L.ghat + static_cast<int64_t>(i) * a.r * L.d_out, acc, a.r,
                         L.d_out, j0, n0, wave, lane);
        acc.zero();
      });

  if (SUM) {
    acc.scale(c);
    store_tile<Tl>(L.part + static_cast<int64_t>(g) * a.r * L.d_out, acc, a.r, L.d_out,
                   j0, n0, wave, lane);
  }
}

// Norm mode for T within one step: the block loads one sample's Xt tile
// (rows j0 .. j0 + 127) into LDS once and sweeps a run of column tiles of
// that sample's dY, writing the same per-(sample, tile, wave) partials as
// samp_kernel. Xt is read once per run instead of once per column tile.
template <typename T, bool PAIR, bool FULL>
__global__ __launch_bounds__(kThreads, 2) void norm_res_kernel(const SampArgs a) {
  typedef MainTile<T> Tl;
  __shared__ __attribute__((aligned(16))) T smem[Tl::kLdsElems];
  const int lb = xcd_logical_block();
  if (lb >= a.n_blocks) return;
  const int li = find_layer(a.first_block, a.n_layers, lb);
  const SampLayer& L = a.L[li];
  const int local = lb - L.block0;
  const int mt = local % L.m_tiles;
  const int rest = local / L.m_tiles;
  const int c = rest % L.n_chunks;  // run of column tiles (runs of one sample
  const int i = rest / L.n_chunks;  // are neighbours: they share Xt in L2)
  const int nt0 = c * a.res_tiles, nt1 = min(L.n_tiles, nt0 + a.res_tiles);
  const int j0 = mt * Tl::BM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = Tl::wave_m(wave), wn = Tl::wave_n(wave);
  T* sA = smem;
  T* sB = smem + Tl::BM * Tl::S;

  RowsLoader<T, Tl::BM, Tl::BK, true, IdentityRows> la{a.ldt, a.r - j0, a.T, {}};
  ColsLoader<T, Tl::BN, Tl::BK, PAIR, BOperandRows<Tl>> lc{L.d_out, 0, a.T, {}};
  const T* Xt = static_cast<const T*>(L.Xt) + (static_cast<int64_t>(i) * a.r + j0) * a.ldt;
  const T* dY = static_cast<const T*>(L.dY) + static_cast<int64_t>(i) * a.T * L.d_out;
  la.template load<FULL>(Xt, 0, tid, a.off32);
  lc.ncols = L.d_out - nt0 * Tl::BN;
  lc.template load<FULL>(dY + nt0 * Tl::BN, 0, tid, a.off32);
  la.store(sA, tid);
  Acc<Tl::MB, Tl::NB> acc;
  acc.zero();
  for (int nt = nt0; nt < nt1; ++nt) {
    __syncthreads();  // the previous tile finished reading sB (and sA is written)
    lc.store(sB, tid);
    __syncthreads();
    if (nt + 1 < nt1) {
      lc.ncols = L.d_out - (nt + 1) * Tl::BN;
      lc.template load<FULL>(dY + (nt + 1) * Tl::BN, 0, tid, a.off32);
    }
    Mma<T, Tl>::run(sA, sB, acc, wm, wn, lane);
    // Rows and columns outside the layer were loaded as zeros.
    const float t = wave_sum(acc.sum_sq());
    if (lane == 0)
      a.norm_part[static_cast<int64_t>(i) * a.n_slots +
                  4 * (L.slot0 + nt * L.m_tiles + mt) + wave] = t;
    if (L.ghat)
      store_tile<Tl>(L.ghat + static_cast<int64_t>(i) * a.r * L.d_out, acc, a.r, L.d_out,
                     j0, nt * Tl::BN, wave, lane);
    acc.zero();
  }
}

// Norm and sum passes in 256 x 256 tiles (rows j of Xt over r, columns n of
// dY over d_out) for bf16 with r and d_out whole tiles and T a multiple of
// kSampBigK: one 16-wave block per CU, K steps over t, two stages of direct
// global-to-LDS copies, the step index running over (sample, t) so that the
// copies flow on across the samples of a block. Xt tiles (t contiguous) sit
// in LDS as the projection's P tiles do. dY tiles stay row-major [t][n], 512
// bytes a row, chunk c of row t in slot c ^ 4 (t % 4); the matrix cores' B
// operand is read from them with the transposing LDS read: in each group of
// 16 lanes, lane q gives four consecutive n of row t0 + q / 4, and lane j
// receives element j % 4 of what lanes j / 4, 4 + j / 4, 8 + j / 4 and
// 12 + j / 4 gave, i.e. four consecutive t of one column. Waves are 4 (j) x 4
// (n), each computing 64 x 64 (as in the projection). Norm mode writes one
// squared-norm partial per (sample, tile, wave), 16 per (sample, tile); sum
// mode keeps the running clipped sum of samp_kernel.
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Slot of 16-byte chunk c in row k of a k-major LDS tile with 512-byte rows.
__device__ __forceinline__ int kmajor_slot(int k, int c) { return c ^ (4 * (k & 3)); }

// Transposing LDS read of four 16-bit values. The restrict-qualified pointer
// gives the read alias-scope information; without it the compiler makes the
// read wait for every direct global-to-LDS copy in flight (the kernels order
// those copies against their reads with explicit waits and barriers).
__device__ __forceinline__ v4i16 lds_read_tr(const char* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
}

// Matrix-core operand of a 32x32x16 product from a k-major LDS tile (rows of
// ROW bytes, 256 or 512, kmajor_slot swizzle): lane l receives rows k0 + 8
// (l / 32) .. + 7 of column c0 + l % 32. In each group of 16 lanes, lane q
// addresses four consecutive columns of row k0 + 8 (l / 32) + 4 h + q / 4;
// the transposing read hands lane j element j % 4 of the values lanes j / 4,
// 4 + j / 4, ... addressed, which is four consecutive rows of one column.
// The 32 lanes of a half-wave read four rows of 64 bytes; the swizzle puts
// them in 16 different 16-byte bank groups for either row length.
template <int ROW = 512>
__device__ __forceinline__ bf16x8 frag_kmajor(const char* tile, int k0, int c0, int lane) {
  static_assert(ROW == 256 || ROW == 512, "rows of 16 or 32 chunks");
  const int q16 = lane & 15, nh = (lane >> 4) & 1, kh = lane >> 5;
  const int n = c0 + 16 * nh + 4 * (q16 & 3);
  v4i16 h[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = k0 + 8 * kh + 4 * i + (q16 >> 2);
    h[i] = lds_read_tr(tile + t * ROW + kmajor_slot(t, n >> 3) * 16 + (n & 7) * 2);
  }
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

template <bool SUM>
__global__ __launch_bounds__(4 * kThreads, 1) void samp_big_kernel(const SampArgs a) {
  constexpr int BK = kSampBigK;
  constexpr int kRowA = BK * 2, CHA = kRowA / 16;        // Xt tile rows
  constexpr int kRowB = kBigN * 2, CHB = kRowB / 16;     // dY tile rows
  constexpr int kTileBytes = kBigM * kRowA;
  constexpr int kBlocksA = kTileBytes / 1024;            // 1 KiB copies per tile
  constexpr int kCopies = 2 * kBlocksA / 16;             // per wave and step
  constexpr int kStageBytes = 2 * kTileBytes;
  static_assert(kTileBytes == BK * kRowB && kBigM == kBigN, "equal square tiles");
  static_assert(kCopies * 16 == 2 * kBlocksA && kCopies % 2 == 0, "copies per wave");
  static_assert(CHA == 8 && CHB == 32, "swizzles assume 128- and 512-byte rows");
  // the stages, then (sum mode) the group's clip factors: one LDS object
  // (with the factors in an array of their own the compiler made the main
  // loop's fragment reads wait for the copies in flight)
  __shared__ __attribute__((aligned(1024))) char smem[2 * kStageBytes + (SUM ? kSumMaxGroup * 4 : 0)];
  float* s_grp = reinterpret_cast<float*>(smem + 2 * kStageBytes);
  const int lb = xcd_logical_block();
  if (lb >= a.n_blocks) return;
  const int li = find_layer(a.first_block, a.n_layers, lb);
  const SampLayer& L = a.L[li];
  const int local = lb - L.block0;
  const int mt = local % L.m_tiles;
  const int rest = local / L.m_tiles;
  const int nt = rest % L.n_tiles;
  const int g = rest / L.n_tiles;  // run (norm) or group (sum) of samples
  const int j0 = mt * kBigM, n0 = nt * kBigN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 3, wn = wave >> 2;
  const int i_begin = g * a.per_block;
  const int i_end = min(a.B, i_begin + a.per_block);
  const int kc = a.T / BK;  // steps per sample
  const int n_steps = (i_end - i_begin) * kc;
  // 16 consecutive rows cover both halves of the 64 banks with 8 slots each
  auto slot_a = [](int R, int c) { return c ^ ((R >> 1) & (CHA - 1)); };

  // Copies step `step` into stage `stage`: copy q of wave w fills 1 KiB
  // block q * 16 + w (Xt blocks of 8 rows first, then dY blocks of 2 rows);
  // lane l writes the block's 16-byte slot l, loading the chunk that the
  // swizzle puts there (the swizzles are involutions). A block's index has
  // the parity of w, so each lane's offset within its block is fixed for a
  // wave and stays in a register; copies go through buffer resources on the
  // layer's Xt and dY (the plan keeps both within 32-bit offsets), the
  // sample, step and block in the uniform offset.
  const __amdgpu_buffer_rsrc_t rsX = tile_rsrc(L.Xt), rsY = tile_rsrc(L.dY);
  const uint32_t xr = static_cast<uint32_t>(a.ldt) * 2u, yr = static_cast<uint32_t>(L.d_out) * 2u;
  const uint32_t voffX = static_cast<uint32_t>(lane >> 3) * xr +
                         static_cast<uint32_t>(((lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7)) << 4);
  const uint32_t voffY = static_cast<uint32_t>(lane >> 5) * yr +
                         static_cast<uint32_t>(((lane & 31) ^ (4 * ((2 * (wave & 1) + (lane >> 5)) & 3))) << 4);
  auto issue = [&](int step, int stage) {
    char* sb = smem + stage * kStageBytes;
    const int i = i_begin + step / kc, k0 = (step % kc) * BK;
    const uint32_t bx = static_cast<uint32_t>(i * a.r + j0) * xr + static_cast<uint32_t>(k0) * 2u;
    const uint32_t by = static_cast<uint32_t>(i * a.T + k0) * yr + static_cast<uint32_t>(n0) * 2u;
#pragma unroll
    for (int q = 0; q < kCopies; ++q) {
      const int blk = q * 16 + wave;
      if (q < kCopies / 2)
        copy_to_lds(rsX, voffX, bx + static_cast<uint32_t>(blk * (1024 / kRowA)) * xr, sb + blk * 1024);
      else
        copy_to_lds(rsY, voffY, by + static_cast<uint32_t>((blk - kBlocksA) * (1024 / kRowB)) * yr,
                    sb + blk * 1024);
    }
  };

  if (SUM) {
    if (!a.fuse_scale) {
      for (int q = tid; q < i_end - i_begin; q += 4 * kThreads) s_grp[q] = a.scales[i_begin + q];
    } else {
      // per-sample global norm and clip factor of this group, summed in the
      // same order as samp_kernel (wave w takes samples w, w + 16, ...)
      const int jn = (a.n_slots + 63) >> 6;
      for (int q = wave; q < i_end - i_begin; q += 16) {
        const float* p = a.norm_part + static_cast<int64_t>(i_begin + q) * a.n_slots;
        float v[kFuseMaxSlots / 64];
#pragma unroll
        for (int j = 0; j < kFuseMaxSlots / 64; ++j)
          if (j < jn) v[j] = p[min(lane + 64 * j, a.n_slots - 1)];
        float t = 0.0f;
#pragma unroll
        for (int j = 0; j < kFuseMaxSlots / 64; ++j)
          if (j < jn && lane + 64 * j < a.n_slots) t += v[j];
        const float n = sqrtf(wave_sum(t));
        if (lane == 0) {
          s_grp[q] = (n > a.clip_C) ? a.clip_C / n : 1.0f;
          if (a.norms_out && li == 0 && mt == 0 && nt == 0) a.norms_out[i_begin + q] = n;
        }
      }
    }
    __syncthreads();
  }

  Acc<2, 2> acc;
  acc.zero();
  float c = 0.0f;  // sum mode: factor the accumulator is expressed in
  bool on = true;  // sum mode: the current sample is accumulated
  const int r32 = lane & 31, kh = lane >> 5;
  // fragments of sub-step kk of the step in stage `stage`: Xt rows (this
  // lane's chunk t = 16 kk + 8 kh ..) and, through the transposing read,
  // dY columns
  auto read_frags = [&](int stage, int kk, bf16x8* af, bf16x8* bfr) {
    const char* sX = smem + stage * kStageBytes;
    const char* sY = sX + kTileBytes;
    const int cx = 2 * kk + kh;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int j = 64 * wm + 32 * mb + r32;
      af[mb] = lds_read_b128(sX + j * kRowA + slot_a(j, cx) * 16);
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) bfr[nb] = frag_kmajor(sY, 16 * kk, 64 * wn + 32 * nb, lane);
  };
  auto mma = [&](const bf16x8* af, const bf16x8* bfr, int q0, int q1) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (q >= q0 && q < q1)
        acc.v[q >> 1][q & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            af[q >> 1], bfr[q & 1], acc.v[q >> 1][q & 1], 0, 0, 0);
  };
  // the schedule of proj_big_kernel: fragments double-buffered over the
  // sub-steps and across steps, the stage wait and barrier in the middle of
  // the last sub-step, the refill into the stage just read
  constexpr int KK = BK / 16;
  bf16x8 fa[2][2], fb[2][2];
  if (n_steps > 0) {
    issue(0, 0);
    wait_vm(0);
    lds_barrier();
    if (n_steps > 1) issue(1, 1);
    read_frags(0, 0, fa[0], fb[0]);
  }
  for (int s = 0; s < n_steps; ++s) {
    if (SUM && s % kc == 0) {
      const float si = lds_read_f32(s_grp + s / kc);
      on = si > 0.0f;
      if (on) {
        if (c != 0.0f && c != si) acc.scale(c / si);
        c = si;
      }
    }
    // the step's body with and without its matrix-core work (a sample whose
    // clip factor is 0 is read and waited for but not accumulated); two
    // instances, so that the hot one has no branches between its MFMAs
    auto body = [&](auto with_mma) {
      constexpr bool M = decltype(with_mma)::value;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int cur = kk & 1, nxt = cur ^ 1;
        const int first = kk + 1 < KK ? 1 : 2;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (M) mma(fa[cur], fb[cur], 0, first);
        __builtin_amdgcn_sched_barrier(0);
        if (kk + 1 < KK) {
          read_frags(s & 1, kk + 1, fa[nxt], fb[nxt]);
        } else if (s + 1 < n_steps) {
          wait_lgkm0();  // this wave's reads of stage s & 1 are complete
          wait_vm(0);    // its copies of step s + 1 landed
          lds_barrier();
          if (s + 2 < n_steps) issue(s + 2, s & 1);
          read_frags((s + 1) & 1, 0, fa[nxt], fb[nxt]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (M) mma(fa[cur], fb[cur], first, 4);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (on) body(std::true_type{});
    else body(std::false_type{});
    if (!SUM && s % kc == kc - 1) {
      const int i = i_begin + s / kc;
      const float t = wave_sum(acc.sum_sq());
      if (lane == 0)
        a.norm_part[static_cast<int64_t>(i) * a.n_slots +
                    16 * (L.slot0 + nt * L.m_tiles + mt) + wave] = t;
      if (L.ghat) {
        // the sample's product tile into ghat [B][r][d_out], through a buffer
        // resource on the wave's 64 rows (lane: column n0 + 64 wn + 32 nb +
        // r32; register q: row 32 mb + 8 (q / 4) + 4 kh + q % 4)
        const __amdgpu_buffer_rsrc_t rs = tile_rsrc(
            L.ghat + (static_cast<int64_t>(i) * a.r + j0 + 64 * wm) * L.d_out);
        const uint32_t row4 = static_cast<uint32_t>(L.d_out) * 4u;
        const uint32_t lo = static_cast<uint32_t>(4 * kh) * row4 +
                            static_cast<uint32_t>(n0 + 64 * wn + r32) * 4u;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
              // (the element is copied out first: a bit cast of a vector
              // element lvalue compiles to a cast of element 0)
              const float x = acc.v[mb][nb][q];
              __builtin_amdgcn_raw_buffer_store_b32(
                  __builtin_bit_cast(uint32_t, x), rs, lo + 128u * nb,
                  __builtin_amdgcn_readfirstlane(
                      static_cast<uint32_t>(32 * mb + 8 * (q >> 2) + (q & 3)) * row4),
                  0);
            }
      }
      acc.zero();
    }
  }

  if (SUM) {
    // the group's partial [r][d_out], through a buffer resource on the
    // wave's 64 rows (lane: column n0 + 64 wn + 32 nb + r32; register q:
    // row 32 mb + 8 (q / 4) + 4 kh + q % 4). One lane offset and uniform
    // row offsets: per-element 64-bit addresses here raised the register
    // pressure of the whole kernel enough that the main loop's fragment
    // reads waited for the step's copies.
    acc.scale(c);
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(
        L.part + (static_cast<int64_t>(g) * a.r + j0 + 64 * wm) * L.d_out);
    const uint32_t row4 = static_cast<uint32_t>(L.d_out) * 4u;
    const uint32_t lo = static_cast<uint32_t>(4 * kh) * row4 +
                        static_cast<uint32_t>(n0 + 64 * wn + r32) * 4u;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const float x = acc.v[mb][nb][q];
          __builtin_amdgcn_raw_buffer_store_b32(
              __builtin_bit_cast(uint32_t, x), rs, lo + 128u * nb,
              __builtin_amdgcn_readfirstlane(
                  static_cast<uint32_t>(32 * mb + 8 * (q >> 2) + (q & 3)) * row4),
              0);
        }
  }
}

// ------------------------------------------------------------------ scale --

__global__ __launch_bounds__(kScaleThreads) void scale_kernel(const ScaleArgs a) {
  // one block per sample; thread t adds the 16-byte groups t, t + 1024,
  // ... of the sample's slots (n_slots is a multiple of 4: every tiling
  // writes 4 or 16 partials per tile), then a fixed-order reduction
  __shared__ float red[kScaleThreads / 64];
  const int i = blockIdx.x, tid = threadIdx.x;
  const float* p = a.norm_part + static_cast<int64_t>(i) * a.n_slots;
  float s = 0.0f;
  const f32x4* p4 = reinterpret_cast<const f32x4*>(p);
  const int n4 = a.n_slots >> 2;
#pragma unroll 4
  for (int k = tid; k < n4; k += kScaleThreads) {
    const f32x4 v = p4[k];
    s += (v[0] + v[1]) + (v[2] + v[3]);
  }
  s = wave_sum(s);
  if ((tid & 63) == 0) red[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) {
    float tot = 0.0f;
#pragma unroll
    for (int w = 0; w < kScaleThreads / 64; ++w) tot += red[w];
    const float n = sqrtf(tot);
    a.scales[i] = (n > a.clip_C) ? a.clip_C / n : 1.0f;
    if (a.norms_out) a.norms_out[i] = n;
  }
}

// -------------------------------------------------------------------- fin --

// Adam direction of one element with the moments updated in place (H:
// PrepArgs or FinArgs, which carry the same constants).
template <class H>
__device__ __forceinline__ float adam_dir(const H& a, float g, float& m, float& v) {
  m = fmaf(a.beta1, m, a.one_m_beta1 * g);
  v = fmaf(a.beta2, v, a.one_m_beta2 * (g * g));
  return (m / a.bc1) / (sqrtf(v / a.bc2) + a.eps);
}

// G_priv = (sum_g w_g part_g + sigma C Z) / B for 4 elements per thread;
// with ADAM, each element then takes the Adam update (m, v in place, the
// direction written to U in the operand type T).
template <typename T, bool ADAM>
__global__ __launch_bounds__(kThreads) void fin_kernel(const FinArgs a) {
  const int b = blockIdx.x;
  const FinLayer& L = a.L[find_layer(a.first_block, a.n_layers, b)];
  const int c = (b - L.block0) * kThreads + static_cast<int>(threadIdx.x);
  const int64_t e0 = 4ll * c;
  if (e0 >= L.n_elem) return;
  float z[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  const bool vec = (L.n_elem & 3) == 0 && is_aligned(L.part, 16) && is_aligned(L.out, 16) &&
                   (!ADAM || (is_aligned(L.m, 16) && is_aligned(L.v, 16)));
  if (vec) {
    // The partials are loaded up to kSumBatch at a time, all in flight
    // together, with the moments and the noise computed while they arrive;
    // they are added in group order.
    const float* part = L.part + e0;
    const int64_t plane = L.n_elem;
    const int last = a.groups - 1;
    f32x4 buf[kSumBatch];
    load_batch(buf, part, plane, a.groups);
    f32x4 m, v;
    if (ADAM) {
      m = *reinterpret_cast<const f32x4*>(L.m + e0);
      v = *reinterpret_cast<const f32x4*>(L.v + e0);
    }
    if (a.noise_scale != 0.0f) {
      const StreamKey key{a.k0, a.k1, a.step_word, 1u};
      normals_at(key, L.layer_id, static_cast<uint32_t>(c), z);
    }
    // with weights, a sample whose factor is 0 (its norm overflowed) is
    // skipped rather than multiplied
    f32x4 s = buf[0];
    if (a.weights) {
      const float w = a.weights[0];
#pragma unroll
      for (int q = 0; q < 4; ++q) s[q] = w != 0.0f ? s[q] * w : 0.0f;
    }
    for (int g0 = 0; g0 < a.groups; g0 += kSumBatch) {
      if (g0 > 0) load_batch(buf, part + g0 * plane, plane, a.groups - g0);
#pragma unroll
      for (int j = 0; j < kSumBatch; ++j) {
        const int g = g0 + j;
        if (g == 0) continue;
        if (g > last) break;
        if (a.weights) {
          const float w = a.weights[g];
          if (w != 0.0f) {
#pragma unroll
            for (int q = 0; q < 4; ++q) s[q] = fmaf(w, buf[j][q], s[q]);
          }
        } else {
          s[0] += buf[j][0];
          s[1] += buf[j][1];
          s[2] += buf[j][2];
          s[3] += buf[j][3];
        }
      }
    }
    f32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = fmaf(a.noise_scale, z[q], s[q]) * a.inv_B;
    *reinterpret_cast<f32x4*>(L.out + e0) = o;
    if (ADAM) {
      float u[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float mq = m[q], vq = v[q];
        u[q] = adam_dir(a, o[q], mq, vq);
        m[q] = mq;
        v[q] = vq;
      }
      *reinterpret_cast<f32x4*>(L.m + e0) = m;
      *reinterpret_cast<f32x4*>(L.v + e0) = v;
      store4<T>(static_cast<T*>(L.U) + e0, u[0], u[1], u[2], u[3]);
    }
    return;
  }
  if (a.noise_scale != 0.0f) {
    const StreamKey key{a.k0, a.k1, a.step_word, 1u};
    normals_at(key, L.layer_id, static_cast<uint32_t>(c), z);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t e = e0 + q;
    if (e < L.n_elem) {
      float s = 0.0f;
      for (int g = 0; g < a.groups; ++g) {
        const float v = L.part[g * static_cast<int64_t>(L.n_elem) + e];
        if (!a.weights) s += v;
        else if (a.weights[g] != 0.0f) s = fmaf(a.weights[g], v, s);
      }
      const float o = fmaf(a.noise_scale, z[q], s) * a.inv_B;
      L.out[e] = o;
      if (ADAM) {
        float m = L.m[e], v = L.v[e];
        const float u = adam_dir(a, o, m, v);
        L.m[e] = m;
        L.v[e] = v;
        static_cast<T*>(L.U)[e] = from_float<T>(u);
      }
    }
  }
}

// ------------------------------------------------------------------- prep --


template <typename T>
__global__ __launch_bounds__(kThreads) void prep_kernel(const PrepArgs a) {
  const int b = blockIdx.x;
  if (b >= a.adam_blocks) {
    const int bp = b - a.adam_blocks;
    const GenPLayer& L = a.P[find_layer(a.first_p, a.n_layers, bp)];
    const StreamKey key{a.k0, a.k1, a.step_word, 0u};
    gen_p_thread<T>(L, (bp - L.block0) * kThreads + static_cast<int>(threadIdx.x),
                    a.r, a.p_scale, key);
    return;
  }
  const AdamLayer& L = a.A[find_layer(a.first_a, a.n_layers, b)];
  const int c = (b - L.block0) * kThreads + static_cast<int>(threadIdx.x);
  const int64_t e0 = 4ll * c;
  if (e0 >= L.n_elem) return;
  T* U = static_cast<T*>(L.U);
  if ((L.n_elem & 3) == 0 && is_aligned(L.g, 16) && is_aligned(L.m, 16) && is_aligned(L.v, 16)) {
    const f32x4 g = *reinterpret_cast<const f32x4*>(L.g + e0);
    f32x4 m = *reinterpret_cast<const f32x4*>(L.m + e0);
    f32x4 v = *reinterpret_cast<const f32x4*>(L.v + e0);
    float u[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float mq = m[q], vq = v[q];
      u[q] = adam_dir(a, g[q], mq, vq);
      m[q] = mq;
      v[q] = vq;
    }
    *reinterpret_cast<f32x4*>(L.m + e0) = m;
    *reinterpret_cast<f32x4*>(L.v + e0) = v;
    store4<T>(U + e0, u[0], u[1], u[2], u[3]);
    return;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t e = e0 + q;
    if (e < L.n_elem) {
      float m = L.m[e], v = L.v[e];
      const float u = adam_dir(a, L.g[e], m, v);
      L.m[e] = m;
      L.v[e] = v;
      U[e] = from_float<T>(u);
    }
  }
}

// ------------------------------------------------------------------- back --

template <typename T> using BackTile = Tile<T, kTileM, kBackN, StepK<T>::v, 4, 1>;

template <typename T, bool PAIR, bool FULL>
__global__ __launch_bounds__(kThreads, 2) void back_kernel(const BackArgs a) {
  typedef BackTile<T> Tl;
  static_assert(Tl::MB == 1 && Tl::NB == 2, "back tile");
  typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
  __shared__ __attribute__((aligned(16))) T smem[Tl::kLdsElems];
  const int lb = xcd_logical_block();
  if (lb >= a.n_blocks) return;
  const BackLayer& L = a.L[find_layer(a.first_block, a.n_layers, lb)];
  const int local = lb - L.block0;
  const int nt = local % L.n_tiles, mt = local / L.n_tiles;
  const int m0 = mt * Tl::BM, n0 = nt * Tl::BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = Tl::wave_m(wave);
  const int nq = n0 + Tl::acc_col(0, 0, lane);  // this lane's 2 columns
  const bool vec = (L.d_out & 1) == 0 && is_aligned(L.W, 8);

  // W rows of this lane (2 consecutive columns each), fetched before the
  // operands so that both are in flight together.
  // interior tile: every row and column in range (block-uniform)
  const bool full = FULL || (vec && m0 + Tl::BM <= L.d_in && n0 + Tl::BN <= L.d_out);
  f32x2 w[16];
  if (full) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = m0 + Tl::acc_row(wm, 0, i, lane);
      w[i] = *reinterpret_cast<const f32x2*>(L.W + static_cast<int64_t>(m) * L.d_out + nq);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = m0 + Tl::acc_row(wm, 0, i, lane);
      f32x2 x = {0.0f, 0.0f};
      if (m < L.d_in && nq < L.d_out) {
        const float* src = L.W + static_cast<int64_t>(m) * L.d_out + nq;
        if (vec) {
          x = *reinterpret_cast<const f32x2*>(src);
        } else {
          x[0] = src[0];
          if (nq + 1 < L.d_out) x[1] = src[1];
        }
      }
      w[i] = x;
    }
  }

  ColsLoader<T, Tl::BM, Tl::BK, PAIR, IdentityRows> lp{L.ldp, L.d_in - m0, a.r, {}};
  ColsLoader<T, Tl::BN, Tl::BK, PAIR, BOperandRows<Tl>> lu{L.d_out, L.d_out - n0, a.r, {}};
  const T* Pb = static_cast<const T*>(L.P) + m0;
  const T* Ub = static_cast<const T*>(L.U) + n0;
  Acc<Tl::MB, Tl::NB> acc;
  acc.zero();
  run_steps<T, Tl>(
      lp, lu, smem, acc, (a.r + Tl::BK - 1) / Tl::BK, tid,
      [&](int s) {
        lp.template load<FULL>(Pb, s * Tl::BK, tid, a.off32);
        lu.template load<FULL>(Ub, s * Tl::BK, tid, a.off32);
      },
      [](int) {});

  if (full) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = m0 + Tl::acc_row(wm, 0, i, lane);
      f32x2 x = w[i];
      x[0] = fmaf(-a.lr, acc.v[0][0][i], x[0]);
      x[1] = fmaf(-a.lr, acc.v[0][1][i], x[1]);
      *reinterpret_cast<f32x2*>(L.W + static_cast<int64_t>(m) * L.d_out + nq) = x;
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m = m0 + Tl::acc_row(wm, 0, i, lane);
    if (m >= L.d_in || nq >= L.d_out) continue;
    f32x2 x = w[i];
    x[0] = fmaf(-a.lr, acc.v[0][0][i], x[0]);
    x[1] = fmaf(-a.lr, acc.v[0][1][i], x[1]);
    float* dst = L.W + static_cast<int64_t>(m) * L.d_out + nq;
    if (vec) {
      *reinterpret_cast<f32x2*>(dst) = x;
    } else {
      dst[0] = x[0];
      if (nq + 1 < L.d_out) dst[1] = x[1];
    }
  }
}

// Back-projection for r within one step: the block keeps its P tile (128
// rows of d_in) in LDS and sweeps a run of 64-column tiles of W, loading the
// next tile's W (registers) and U (staged) while the current one runs on the
// matrix cores.
template <typename T, bool PAIR, bool FULL>
__global__ __launch_bounds__(kThreads, 2) void back_res_kernel(const BackArgs a) {
  typedef BackTile<T> Tl;
  static_assert(Tl::MB == 1 && Tl::NB == 2, "back tile");
  typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
  __shared__ __attribute__((aligned(16))) T smem[Tl::kLdsElems];
  const int lb = xcd_logical_block();
  if (lb >= a.n_blocks) return;
  const BackLayer& L = a.L[find_layer(a.first_block, a.n_layers, lb)];
  const int local = lb - L.block0;
  const int c = local % L.n_chunks, mt = local / L.n_chunks;
  const int nt0 = c * a.res_tiles, nt1 = min(L.n_tiles, nt0 + a.res_tiles);
  const int m0 = mt * Tl::BM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = Tl::wave_m(wave), wn = Tl::wave_n(wave);
  const int lq = Tl::acc_col(0, 0, lane);  // this lane's 2 columns in a tile
  const bool vec = (L.d_out & 1) == 0 && is_aligned(L.W, 8);
  T* sA = smem;
  T* sB = smem + Tl::BM * Tl::S;

  // W rows of this lane in column tile nt (2 consecutive columns each)
  auto load_w = [&](int nt, f32x2* w) {
    const int nq = nt * Tl::BN + lq;
    if (FULL || (vec && m0 + Tl::BM <= L.d_in && (nt + 1) * Tl::BN <= L.d_out)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = m0 + Tl::acc_row(wm, 0, i, lane);
        w[i] = *reinterpret_cast<const f32x2*>(L.W + static_cast<int64_t>(m) * L.d_out + nq);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = m0 + Tl::acc_row(wm, 0, i, lane);
      f32x2 x = {0.0f, 0.0f};
      if (m < L.d_in && nq < L.d_out) {
        const float* src = L.W + static_cast<int64_t>(m) * L.d_out + nq;
        if (vec) {
          x = *reinterpret_cast<const f32x2*>(src);
        } else {
          x[0] = src[0];
          if (nq + 1 < L.d_out) x[1] = src[1];
        }
      }
      w[i] = x;
    }
  };
  auto store_w = [&](int nt, const f32x2* w, const Acc<1, 2>& acc) {
    const int nq = nt * Tl::BN + lq;
    const bool full = FULL || (vec && m0 + Tl::BM <= L.d_in && (nt + 1) * Tl::BN <= L.d_out);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = m0 + Tl::acc_row(wm, 0, i, lane);
      f32x2 x = w[i];
      x[0] = fmaf(-a.lr, acc.v[0][0][i], x[0]);
      x[1] = fmaf(-a.lr, acc.v[0][1][i], x[1]);
      float* dst = L.W + static_cast<int64_t>(m) * L.d_out + nq;
      if (full) {
        *reinterpret_cast<f32x2*>(dst) = x;
      } else if (m < L.d_in && nq < L.d_out) {
        if (vec) {
          *reinterpret_cast<f32x2*>(dst) = x;
        } else {
          dst[0] = x[0];
          if (nq + 1 < L.d_out) dst[1] = x[1];
        }
      }
    }
  };

  ColsLoader<T, Tl::BM, Tl::BK, PAIR, IdentityRows> lp{L.ldp, L.d_in - m0, a.r, {}};
  ColsLoader<T, Tl::BN, Tl::BK, PAIR, BOperandRows<Tl>> lu{L.d_out, 0, a.r, {}};
  const T* U = static_cast<const T*>(L.U);
  f32x2 w[16], wnext[16];
  load_w(nt0, w);
  lp.template load<FULL>(static_cast<const T*>(L.P) + m0, 0, tid, a.off32);
  lu.ncols = L.d_out - nt0 * Tl::BN;
  lu.template load<FULL>(U + nt0 * Tl::BN, 0, tid, a.off32);
  lp.store(sA, tid);
  Acc<1, 2> acc;
  for (int nt = nt0; nt < nt1; ++nt) {
    __syncthreads();  // the previous tile finished reading sB (and sA is written)
    lu.store(sB, tid);
    __syncthreads();
    const bool more = nt + 1 < nt1;
    if (more) {
      load_w(nt + 1, wnext);
      lu.ncols = L.d_out - (nt + 1) * Tl::BN;
      lu.template load<FULL>(U + (nt + 1) * Tl::BN, 0, tid, a.off32);
    }
    acc.zero();
    Mma<T, Tl>::run(sA, sB, acc, wm, wn, lane);
    store_w(nt, w, acc);
    if (more) {
#pragma unroll
      for (int i = 0; i < 16; ++i) w[i] = wnext[i];
    }
  }
}

// W -= lr P^T U in 256 x 128 tiles (rows m of W over d_in, columns n over
// d_out) for bf16 with d_in a multiple of 256, d_out of 128 and r of 32.
// Blocks of 4 waves (2 (m) x 2 (n), each 128 x 64), two per CU, so that one
// block's read-modify-write of W (the HBM traffic that bounds this pass)
// runs while the other block's matrix cores work. A block sweeps a run of
// column tiles of one row tile, its K steps of 32 over r running on from
// tile to tile, with two stages of direct global-to-LDS copies (a stage is
// refilled as soon as every wave has read it). P [r][d_in] and U [r][d_out]
// are k-major and stay so in LDS (rows of 512 and 256 bytes); both
// matrix-core operands come from the transposing read. W goes through a
// buffer resource, one 32-row block at a time, the next block's loads in
// flight while the current one is stored.
__global__ __launch_bounds__(kThreads, 2) void back_big_kernel(const BackArgs a) {
  constexpr int BK = kBackBigK;
  constexpr int kRowP = kBigM * 2, kRowU = kBackBigN * 2;      // 512- and 256-byte rows
  constexpr int kTileP = BK * kRowP, kTileU = BK * kRowU;     // 16 and 8 KiB
  constexpr int kStage = kTileP + kTileU;
  constexpr int kCopiesP = kTileP / 1024 / 4, kCopiesU = kTileU / 1024 / 4;  // per wave and step
  static_assert(kCopiesP == 4 && kCopiesU == 2 && BK == 32, "copy layout");
  constexpr int NS = 3;  // stages: copies run up to two steps ahead
  __shared__ __attribute__((aligned(1024))) char smem[NS * kStage];
  const int lb = xcd_logical_block();
  if (lb >= a.n_blocks) return;
  const BackLayer& L = a.L[find_layer(a.first_block, a.n_layers, lb)];
  // Blocks of a layer: groups of (up to) 8 row tiles; in a group, each run
  // of column tiles for each of its rows, the rows varying fastest. The
  // blocks an XCD runs at once are consecutive, so they cover about 8 rows
  // by 8 runs: 8 slices of P, each read again for every tile of its runs,
  // and 8 slices of U, each read by 8 blocks at about the same time, stay
  // in that XCD's L2.
  const int local = lb - L.block0;
  const int grp = local / (8 * L.n_chunks), rem = local - grp * 8 * L.n_chunks;
  const int g = min(8, L.m_tiles - 8 * grp);
  const int ch = rem / g, mt = 8 * grp + (rem - ch * g);
  const int nt0 = ch * a.res_tiles, nt1 = min(L.n_tiles, nt0 + a.res_tiles);
  const int m0 = mt * kBigM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int r32 = lane & 31, kh = lane >> 5;
  const int kr = a.r / BK;  // steps per tile
  const int n_steps = (nt1 - nt0) * kr;
  const uint32_t p_rb = static_cast<uint32_t>(L.ldp) * 2u, u_rb = static_cast<uint32_t>(L.d_out) * 2u;

  // Copies step `step` into stage `stage`: copy q < 4 of wave w fills P
  // block q * 4 + w (k rows 2 b and 2 b + 1, 512 bytes each), copy q >= 4 U
  // block (q - 4) * 4 + w (k rows 4 b .. 4 b + 3, 256 bytes each); lane l
  // writes 16-byte slot l of the block, loading the chunk the swizzle puts
  // there (an involution). The lane offsets are fixed for a wave (a P block
  // has the parity of w; the U swizzle does not depend on the block), so
  // they stay in registers; buffer resources on P and U (the plan keeps
  // both within 32-bit offsets).
  const __amdgpu_buffer_rsrc_t rsP = tile_rsrc(L.P), rsU = tile_rsrc(L.U);
  const uint32_t voffP = static_cast<uint32_t>(lane >> 5) * p_rb +
                         static_cast<uint32_t>(((lane & 31) ^ (4 * ((2 * (wave & 1) + (lane >> 5)) & 3))) << 4);
  const uint32_t voffU = static_cast<uint32_t>(lane >> 4) * u_rb +
                         static_cast<uint32_t>(((lane & 15) ^ (4 * ((lane >> 4) & 3))) << 4);
  auto issue = [&](int step, int stage) {
    char* sb = smem + stage * kStage;
    const int nt = nt0 + step / kr;
    const uint32_t k0 = static_cast<uint32_t>((step % kr) * BK);
#pragma unroll
    for (int q = 0; q < kCopiesP; ++q) {
      const int blk = q * 4 + wave;
      copy_to_lds(rsP, voffP, (k0 + 2u * blk) * p_rb + static_cast<uint32_t>(m0) * 2u, sb + blk * 1024);
    }
#pragma unroll
    for (int q = 0; q < kCopiesU; ++q) {
      const int blk = q * 4 + wave;
      copy_to_lds(rsU, voffU, (k0 + 4u * blk) * u_rb + static_cast<uint32_t>(nt * kBackBigN) * 2u,
                  sb + kTileP + blk * 1024);
    }
  };

  // lane: columns 64 wn + 32 nb + r32 of the tile; registers i: rows
  // 8 (i / 4) + 4 kh + i % 4 of each 32-row block mb, of the wave's 128
  // rows: one lane offset, the rest uniform
  const __amdgpu_buffer_rsrc_t w_rs =
      tile_rsrc(L.W + static_cast<int64_t>(m0 + 128 * wm) * L.d_out);
  const uint32_t row4 = static_cast<uint32_t>(L.d_out) * 4u;
  const uint32_t w_lane = static_cast<uint32_t>(4 * kh) * row4 +
                          static_cast<uint32_t>(64 * wn + r32) * 4u;
  auto w_soff = [&](int nt, int mb, int i) {
    return __builtin_amdgcn_readfirstlane(
        static_cast<uint32_t>(32 * mb + 8 * (i >> 2) + (i & 3)) * row4 +
        static_cast<uint32_t>(nt) * (kBackBigN * 4u));
  };
  typedef float WBlock[2][16];
  auto load_w = [&](int nt, int mb, WBlock& w) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        w[nb][i] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(w_rs, w_lane + 128u * nb, w_soff(nt, mb, i), kNonTemporal));
  };
  Acc<4, 2> acc;
  auto store_w = [&](int nt, int mb, const WBlock& w) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float x = fmaf(-a.lr, acc.v[mb][nb][i], w[nb][i]);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), w_rs,
                                              w_lane + 128u * nb, w_soff(nt, mb, i), kNonTemporal);
      }
  };

  // vmcnt(n) for the counts below (6 copies a wave and step, 32 loads a
  // W block): vmcnt's low four bits sit in bits 3:0 of the operand, its
  // high two in bits 15:14; a count above 63 waits for 63
  auto wait_ops = [](int n) {
    switch (n) {
      case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
      case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
      case 12: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
      case 32: __builtin_amdgcn_s_waitcnt(0x8F70); break;
      case 38: __builtin_amdgcn_s_waitcnt(0x8F76); break;
      case 44: __builtin_amdgcn_s_waitcnt(0x8F7C); break;
      default:
        if (n > 63) __builtin_amdgcn_s_waitcnt(0xCF7F);
        else __builtin_amdgcn_s_waitcnt(0x0F70);  // (stricter: wait for all)
        break;
    }
  };
  constexpr int kCopies = kCopiesP + kCopiesU;
  acc.zero();
  if (n_steps > 0) {
    // steps 0 .. NS - 1 in flight; wait for step 0
#pragma unroll
    for (int q = 0; q < NS; ++q)
      if (q < n_steps) issue(q, q);
    wait_ops((min(NS, n_steps) - 1) * kCopies);
    lds_barrier();
  }
  WBlock w0, w1;
  int stage = 0;
  // A tile's W: rows 0-31 (block 0) are loaded at the start of its
  // second-last K step, rows 32-63 at the start of its last, the other two
  // blocks after its product is complete; each block is stored as soon as
  // its loads are in, the next block's loads in flight meanwhile.
  for (int s = 0; s < n_steps; ++s) {
    const int ks = s % kr;
    const bool last = ks == kr - 1;
    const int nt = nt0 + s / kr;
    if (ks == kr - 2 || (kr == 1 && last)) load_w(nt, 0, w0);
    if (kr >= 2 && last) load_w(nt, 1, w1);
    const char* sP = smem + stage * kStage;
    const char* sU = sP + kTileP;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[4], bfr[2];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) af[mb] = frag_kmajor<kRowP>(sP, 16 * kk, 128 * wm + 32 * mb, lane);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) bfr[nb] = frag_kmajor<kRowU>(sU, 16 * kk, 64 * wn + 32 * nb, lane);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc.v[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr[nb],
                                                                 acc.v[mb][nb], 0, 0, 0);
    }
    if (s + 1 < n_steps) {
      wait_lgkm0();  // this wave's reads of stage `stage` are complete
      // its copies of step s + 1 landed: loads return in order, so what
      // was issued after them may stay in flight: the copies of steps
      // s + 2 .. s + NS - 1 and the W loads of this step and the one before
      // (64 of them in a tile's last step, so a wait for 63 there: the
      // first 7 of block 0's loads, a step old, complete as well); unless
      // W stores are outstanding too (the previous step ended a tile):
      // stores may complete out of order, so then wait for all
      const int w_after = (kr >= 2 && last) ? 64 : (ks == kr - 2 || (kr == 1 && last)) ? 32 : 0;
      if (s % kr == 0 && s > 0) wait_vm(0);
      else wait_ops((min(s + NS - 1, n_steps - 1) - (s + 1)) * kCopies + w_after);
      lds_barrier();
      // every wave has read stage `stage`: it takes step s + NS
      if (s + NS < n_steps) issue(s + NS, stage);
    }
    stage = stage + 1 == NS ? 0 : stage + 1;
    if (last) {
      if (kr == 1) load_w(nt, 1, w1);
      store_w(nt, 0, w0);
      load_w(nt, 2, w0);
      store_w(nt, 1, w1);
      load_w(nt, 3, w1);
      store_w(nt, 2, w0);
      store_w(nt, 3, w1);
      acc.zero();
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


// ------------------------------------------------------ streaming form --

// norm_sq[i] += sum of one layer's partials of sample i: one wave per
// sample, lane l adds slots l, l + 64, ... in order, then a fixed butterfly.
__global__ __launch_bounds__(kThreads) void norm_acc_kernel(const NormAccArgs a) {
  const int i = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= a.B) return;
  const float* p = a.norm_part + static_cast<int64_t>(i) * a.n_slots;
  float t = 0.0f;
  for (int k = lane; k < a.n_slots; k += 64) t += p[k];
  t = wave_sum(t);
  if (lane == 0) a.norm_sq[i] += t;
}

// n_i = sqrt(norm_sq[i]), s_i = min(1, C / n_i).
__global__ __launch_bounds__(kThreads) void clip_kernel(const ClipArgs a) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= a.B) return;
  const float n = sqrtf(a.norm_sq[i]);
  a.scales[i] = (n > a.clip_C) ? a.clip_C / n : 1.0f;
  if (a.norms_out) a.norms_out[i] = n;
}

// -------------------------------------------------------------- launchers --

static inline unsigned grid8(int n_blocks) {
  return static_cast<unsigned>(round_up(n_blocks, 8));
}

hipError_t launch_gen_p(GenPArgs a, int n_blocks, bool bf16_out,
                        hipStream_t s) {
  index_layers(a.first_block, a.L, a.n_layers);
  const dim3 g(n_blocks), b(kThreads);
  if (bf16_out) hipLaunchKernelGGL(gen_p_kernel<bf16>, g, b, 0, s, a);
  else hipLaunchKernelGGL(gen_p_kernel<float>, g, b, 0, s, a);
  return hipGetLastError();
}

template <int NG>
static hipError_t launch_proj_ng(const ProjArgs& a, bool bf16_in, bool vec, hipStream_t s) {
  const dim3 g(grid8(a.n_blocks)), b(kThreads * NG);
  if (bf16_in) {
    if (a.full) hipLaunchKernelGGL((proj_kernel<bf16, true, true, NG>), g, b, 0, s, a);
    else if (vec) hipLaunchKernelGGL((proj_kernel<bf16, true, false, NG>), g, b, 0, s, a);
    else hipLaunchKernelGGL((proj_kernel<bf16, false, false, NG>), g, b, 0, s, a);
  } else {
    if (a.full) hipLaunchKernelGGL((proj_kernel<float, true, true, NG>), g, b, 0, s, a);
    else if (vec) hipLaunchKernelGGL((proj_kernel<float, true, false, NG>), g, b, 0, s, a);
    else hipLaunchKernelGGL((proj_kernel<float, false, false, NG>), g, b, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_proj(ProjArgs a, bool bf16_in, bool vec, hipStream_t s) {
  index_layers(a.first_block, a.L, a.n_layers);
  if (a.big) {
    hipLaunchKernelGGL((proj_big_kernel<kBigK>), dim3(grid8(a.n_blocks)),
                       dim3(4 * kThreads), 0, s, a);
    return hipGetLastError();
  }
  return a.groups2 ? launch_proj_ng<2>(a, bf16_in, vec, s)
                   : launch_proj_ng<1>(a, bf16_in, vec, s);
}

hipError_t launch_xsum(XsumArgs a, int n_blocks, bool bf16_out,
                       hipStream_t s) {
  index_layers(a.first_block, a.L, a.n_layers);
  if (bf16_out) hipLaunchKernelGGL(xsum_kernel<bf16>, dim3(n_blocks), dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(xsum_kernel<float>, dim3(n_blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

// FULL (all tiles full, paired columns): the loads are compiled without
// their edge code.
template <int BN, bool SUM>
static hipError_t launch_samp(const SampArgs& a, bool bf16_in, bool pair,
                              hipStream_t s) {
  const dim3 g(grid8(a.n_blocks)), b(kThreads);
  if (bf16_in) {
    if (a.full) hipLaunchKernelGGL((samp_kernel<bf16, BN, true, SUM, true>), g, b, 0, s, a);
    else if (pair) hipLaunchKernelGGL((samp_kernel<bf16, BN, true, SUM, false>), g, b, 0, s, a);
    else hipLaunchKernelGGL((samp_kernel<bf16, BN, false, SUM, false>), g, b, 0, s, a);
  } else {
    if (a.full) hipLaunchKernelGGL((samp_kernel<float, BN, true, SUM, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((samp_kernel<float, BN, true, SUM, false>), g, b, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_samp_norm(SampArgs a, bool bf16_in, bool pair,
                            hipStream_t s) {
  index_layers(a.first_block, a.L, a.n_layers);
  if (a.big) {
    hipLaunchKernelGGL(samp_big_kernel<false>, dim3(grid8(a.n_blocks)), dim3(4 * kThreads), 0, s, a);
    return hipGetLastError();
  }
  if (a.res_tiles == 0) return launch_samp<kTileN, false>(a, bf16_in, pair, s);
  const dim3 g(grid8(a.n_blocks)), b(kThreads);
  if (bf16_in) {
    if (a.full) hipLaunchKernelGGL((norm_res_kernel<bf16, true, true>), g, b, 0, s, a);
    else if (pair) hipLaunchKernelGGL((norm_res_kernel<bf16, true, false>), g, b, 0, s, a);
    else hipLaunchKernelGGL((norm_res_kernel<bf16, false, false>), g, b, 0, s, a);
  } else {
    if (a.full) hipLaunchKernelGGL((norm_res_kernel<float, true, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((norm_res_kernel<float, true, false>), g, b, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_samp_sum(SampArgs a, bool bf16_in, bool pair,
                           hipStream_t s) {
  index_layers(a.first_block, a.L, a.n_layers);
  if (a.big) {
    hipLaunchKernelGGL(samp_big_kernel<true>, dim3(grid8(a.n_blocks)), dim3(4 * kThreads), 0, s, a);
    return hipGetLastError();
  }
  return launch_samp<kTileN, true>(a, bf16_in, pair, s);
}

hipError_t launch_scale(const ScaleArgs& a, int B, hipStream_t s) {
  hipLaunchKernelGGL(scale_kernel, dim3(B), dim3(kScaleThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_norm_acc(const NormAccArgs& a, hipStream_t s) {
  const unsigned blocks = static_cast<unsigned>((a.B + kThreads / 64 - 1) / (kThreads / 64));
  hipLaunchKernelGGL(norm_acc_kernel, dim3(blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_clip(const ClipArgs& a, hipStream_t s) {
  const unsigned blocks = static_cast<unsigned>((a.B + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(clip_kernel, dim3(blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fin(FinArgs a, int n_blocks, hipStream_t s) {
  index_layers(a.first_block, a.L, a.n_layers);
  hipLaunchKernelGGL((fin_kernel<float, false>), dim3(n_blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fin_adam(FinArgs a, int n_blocks, bool bf16_out, hipStream_t s) {
  index_layers(a.first_block, a.L, a.n_layers);
  if (bf16_out)
    hipLaunchKernelGGL((fin_kernel<bf16, true>), dim3(n_blocks), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((fin_kernel<float, true>), dim3(n_blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prep(PrepArgs a, int n_blocks, bool bf16_out,
                       hipStream_t s) {
  index_layers(a.first_a, a.A, a.n_layers);
  index_layers(a.first_p, a.P, a.n_layers);
  if (bf16_out)
    hipLaunchKernelGGL(prep_kernel<bf16>, dim3(n_blocks), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(prep_kernel<float>, dim3(n_blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_back(BackArgs a, bool bf16_in, bool pair, hipStream_t s) {
  index_layers(a.first_block, a.L, a.n_layers);
  const dim3 g(grid8(a.n_blocks)), b(kThreads);
  if (a.big) {
    hipLaunchKernelGGL(back_big_kernel, g, dim3(kThreads), 0, s, a);
    return hipGetLastError();
  }
  if (a.res_tiles > 0) {
    if (!bf16_in) {
      if (a.full) hipLaunchKernelGGL((back_res_kernel<float, true, true>), g, b, 0, s, a);
      else hipLaunchKernelGGL((back_res_kernel<float, true, false>), g, b, 0, s, a);
    } else if (a.full) {
      hipLaunchKernelGGL((back_res_kernel<bf16, true, true>), g, b, 0, s, a);
    } else if (pair) {
      hipLaunchKernelGGL((back_res_kernel<bf16, true, false>), g, b, 0, s, a);
    } else {
      hipLaunchKernelGGL((back_res_kernel<bf16, false, false>), g, b, 0, s, a);
    }
  } else if (bf16_in) {
    if (a.full) hipLaunchKernelGGL((back_kernel<bf16, true, true>), g, b, 0, s, a);
    else if (pair) hipLaunchKernelGGL((back_kernel<bf16, true, false>), g, b, 0, s, a);
    else hipLaunchKernelGGL((back_kernel<bf16, false, false>), g, b, 0, s, a);
  } else {
    if (a.full) hipLaunchKernelGGL((back_kernel<float, true, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((back_kernel<float, true, false>), g, b, 0, s, a);
  }
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
