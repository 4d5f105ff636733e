// Host side of the C ABI declared in include/dpg.h: argument validation,
// workspace planning and launch sequencing on the caller's stream. Nothing
// is allocated here and no state survives a call (apart from the calling
// thread's last error message).
#include <algorithm>
#include <functional>
#include <queue>
#include <set>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "dpg.h"
#include "dpg_internal.hpp"

using namespace dpg;

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

bool debug_sync() {
  static const bool on = [] {
    const char* v = std::getenv("DPG_DEBUG_SYNC");
    return v && v[0] && v[0] != '0';
  }();
  return on;
}

// ---- kernel-timing diagnostics (off unless dpg_timing_enable(1))
enum Kind { K_GEN_P, K_PROJ, K_XSUM, K_NORM, K_SCALE, K_SUM, K_FIN, K_PREP,
            K_BACK, K_CLIP, K_COUNT };
static_assert(K_COUNT == DPG_N_KERNEL_KINDS, "kernel kinds");
const char* const kKindName[K_COUNT] = {"gen_p", "proj", "xsum", "norm", "scale",
                                        "sum", "fin", "prep", "back", "clip"};
struct TimedLaunch {
  int kind;
  hipEvent_t start, stop;
};
std::mutex g_timing_mu;
bool g_timing_on = false;
std::vector<TimedLaunch> g_pending;
double g_total_ms[K_COUNT] = {};
int64_t g_launches[K_COUNT] = {};

// Brackets one launch with events on its stream when timing is enabled.
struct LaunchTimer {
  int kind;
  hipStream_t s;
  hipEvent_t start = nullptr;
  LaunchTimer(int k, hipStream_t st) : kind(k), s(st) {
    std::lock_guard<std::mutex> g(g_timing_mu);
    if (!g_timing_on) return;
    if (hipEventCreate(&start) != hipSuccess) { start = nullptr; return; }
    if (hipEventRecord(start, s) != hipSuccess) {
      (void)hipEventDestroy(start);
      start = nullptr;
    }
  }
  // A launch whose events could not be made or recorded is left untimed.
  void done() {
    if (!start) return;
    hipEvent_t stop;
    if (hipEventCreate(&stop) != hipSuccess) {
      (void)hipEventDestroy(start);
      start = nullptr;
      return;
    }
    if (hipEventRecord(stop, s) != hipSuccess) {
      (void)hipEventDestroy(start);
      (void)hipEventDestroy(stop);
      start = nullptr;
      return;
    }
    std::lock_guard<std::mutex> g(g_timing_mu);
    g_pending.push_back({kind, start, stop});
    start = nullptr;
  }
};

// Checks a launch; with DPG_DEBUG_SYNC=1 also waits for it to finish.
int check(hipError_t e, const char* what, hipStream_t s) {
  if (e == hipSuccess && debug_sync()) e = hipStreamSynchronize(s);
  if (e != hipSuccess)
    return fail(DPG_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return DPG_OK;
}

// A timed launch: `fn` enqueues one kernel and returns its hipError_t.
template <class F>
int timed(int kind, hipStream_t s, F fn) {
  LaunchTimer t(kind, s);
  const hipError_t e = fn();
  t.done();
  return check(e, kKindName[kind], s);
}

constexpr size_t kAlign = 256;
constexpr uint64_t kMaxU32 = 0xFFFFFFFFull;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

size_t elem_size(int32_t dtype) { return dtype == DPG_BF16 ? 2 : 4; }

bool valid_dtype(int32_t dtype) { return dtype == DPG_FP32 || dtype == DPG_BF16; }

// Shape checks shared by every call. Limits keep every kernel index in range:
// r*d_in and r*d_out below 2^31 fit the int32 element counts of the Adam
// and final passes (and the 32-bit Philox element counter), and tile counts
// fit int32.
constexpr int64_t kMaxRD = (1ll << 31) - 8;
int check_layer_shape(int64_t d_in, int64_t d_out, int32_t r, int idx) {
  const std::string at = " (layer index " + std::to_string(idx) + ")";
  if (d_in < 1 || d_out < 1)
    return fail(DPG_ERR_INVALID_ARG, "d_in and d_out must be >= 1" + at);
  if (d_in > (1 << 30) || d_out > (1 << 30))
    return fail(DPG_ERR_INVALID_ARG, "d_in and d_out must be <= 2^30" + at);
  if (static_cast<int64_t>(r) * d_in > kMaxRD || static_cast<int64_t>(r) * d_out > kMaxRD)
    return fail(DPG_ERR_INVALID_ARG, "r*d_in and r*d_out must be < 2^31 - 8" + at);
  return DPG_OK;
}

template <class L>
int check_unique_ids(const L* layers, int32_t n) {
  std::vector<uint32_t> ids(n);
  for (int i = 0; i < n; ++i) ids[i] = layers[i].layer_id;
  std::sort(ids.begin(), ids.end());
  for (int i = 1; i < n; ++i)
    if (ids[i] == ids[i - 1])
      return fail(DPG_ERR_INVALID_ARG,
                  "duplicate layer_id " + std::to_string(ids[i]));
  return DPG_OK;
}

// ------------------------------------------------ projection call planning --

// Blocks resident at once that the split and grouping heuristics aim at: two
// per compute unit of an MI355X (256 CUs), the occupancy the tiled kernels
// run at (their register use allows two 256-thread blocks per CU).
int64_t target_blocks(int32_t) { return 512; }

int step_of(int32_t dtype) { return dtype == DPG_BF16 ? kStepBf16 : kStepF32; }

// Tiling of the two per-sample passes (squared-norm partials, clipped sum).
struct SampPlan {
  bool big = false;  // samp_big_kernel: kBigM x kBigN tiles, 16 waves
  std::vector<int32_t> m_tiles, n_tiles, slot0;  // per layer; slot0 in tiles
  int32_t n_slots = 0;         // partials per sample: one per (tile, wave)
  int32_t norm_per_block = 1;  // samples per norm block
  int32_t norm_res_tiles = 0;  // column tiles per norm block (T within one step)
  int32_t groups = 1, per_group = 1;  // sum pass
  bool fuse_scale = false;             // sum pass computes s_i itself
};

struct ProjPlan {
  int64_t ldt = 0;             // row stride of Xt (T rounded up to 8)
  std::vector<int64_t> ldp;    // row stride of P per layer
  std::vector<size_t> off_P, off_Xt, off_part, off_xpart;
  std::vector<int32_t> m_tiles_proj, n_tiles_proj, splits, steps_per_split;  // projection
  bool big = false;             // projection in proj_big_kernel tiles
  // per-sample passes: the regular tiling, and the large one where the
  // shapes allow it (taken when dY is 16-byte aligned; the workspace holds
  // either)
  SampPlan samp, samp_big;
  bool has_samp_big = false;
  // T long against r (8 r <= T): the norm pass also stores every sample's
  // product [r][d_out] (fp32, in the partial region), and the final pass
  // sums those with the clip factors as weights instead of a second pass
  // over dY; the stored products move at most half the bytes of dY
  bool hat_sum = false;
  size_t off_norm = 0, off_scales = 0, total = 0;
};

int validate_proj_shapes(const dpg_layer_grad* layers, int32_t n_layers,
                         int64_t B, int64_t T, int32_t r, int32_t dtype) {
  if (!layers) return fail(DPG_ERR_INVALID_ARG, "layers is NULL");
  if (n_layers < 1 || n_layers > (1 << 20))
    return fail(DPG_ERR_INVALID_ARG, "n_layers must be in [1, 2^20]");
  if (B < 1 || T < 1 || r < 1)
    return fail(DPG_ERR_INVALID_ARG, "B, T and r must be >= 1");
  if (B * T > (1ll << 30))
    return fail(DPG_ERR_INVALID_ARG, "B*T must be <= 2^30");
  if (!valid_dtype(dtype)) return fail(DPG_ERR_INVALID_ARG, "unknown dtype");
  for (int i = 0; i < n_layers; ++i) {
    const int st = check_layer_shape(layers[i].d_in, layers[i].d_out, r, i);
    if (st) return st;
    if (layers[i].reserved != 0)
      return fail(DPG_ERR_INVALID_ARG, "reserved field must be 0");
    if (B * T * std::max(layers[i].d_in, layers[i].d_out) > (1ll << 46) ||
        static_cast<int64_t>(r) * B * T > (1ll << 40))
      return fail(DPG_ERR_INVALID_ARG, "layer too large");
  }
  return check_unique_ids(layers, n_layers);
}

ProjPlan plan_proj(const dpg_layer_grad* layers, int32_t n_layers, int64_t B,
                   int64_t T, int32_t r, int32_t dtype) {
  ProjPlan p;
  const size_t es = elem_size(dtype);
  const int64_t BK = step_of(dtype);
  const int64_t BT = B * T;
  p.ldt = round_up(T, 8);
  const int32_t mt = static_cast<int32_t>(ceil_div(r, kTileM));
  // Projection: K steps per block chosen so that about half of `target`
  // blocks share the work; a layer whose d_in needs more steps is split over
  // d_in. Every split writes an fp32 partial of Xt that the xsum kernel reads
  // back, so splits are kept twice as long as one round of resident blocks
  // would need.
  int64_t units = 0;
  for (int l = 0; l < n_layers; ++l)
    units += mt * ceil_div(BT, kTileN) * ceil_div(layers[l].d_in, BK);
  const int64_t target = target_blocks(dtype);
  const int64_t steps_per_block = std::max<int64_t>(1, ceil_div(units, target / 2));
  // Large bf16 projections run in 256 x 256 tiles with K steps of 64, one
  // 16-wave block per CU. The K steps per block minimise an estimate of the
  // time in steps (per launch, below) plus the split partials.
  // (its epilogue stores use 32-bit offsets: all of Xt, and 256 rows of a
  // split partial)
  p.big = dtype == DPG_BF16 && r % kBigM == 0 && BT % kBigN == 0 && BT >= 2 * kBigN &&
          static_cast<uint64_t>(B) * r * p.ldt * 2 < (1ull << 32) &&
          static_cast<uint64_t>(BT) * 4 * kBigM < (1ull << 32);
  // (its copies go through buffer resources: each layer's A and P within
  // 32-bit offsets)
  for (int l = 0; l < n_layers; ++l)
    if (layers[l].d_in % kBigK != 0 ||
        static_cast<uint64_t>(BT) * layers[l].d_in * 2 >= (1ull << 32) ||
        static_cast<uint64_t>(r) * round_up(layers[l].d_in, 8) * 2 >= (1ull << 32))
      p.big = false;
  // A launch with fewer large tiles than CUs would split d_in and add the
  // partials back; the regular tiles, four times as many, fill the chip
  // without that once they number at least the CUs. This is the case of
  // per-layer calls (the streaming form) at r = 256 or 512 and B·T in the
  // thousands, unless the layers are long enough in d_in (more than 64
  // large K steps) for the split partials to be a small part of the work;
  // launches of several large layers keep the large tiles.
  {
    const int64_t per_launch = std::min<int64_t>(n_layers, kMaxLayers), cus = target / 2;
    int64_t max_steps = 0;
    for (int l = 0; l < n_layers; ++l) max_steps = std::max<int64_t>(max_steps, layers[l].d_in / kBigK);
    if (p.big && (r / kBigM) * (BT / kBigN) * per_launch < cus &&
        mt * ceil_div(BT, kTileN) * per_launch >= cus && max_steps <= 64)
      p.big = false;
  }
  int64_t big_sps = 0;
  if (p.big) {
    const int64_t tiles = (r / kBigM) * (BT / kBigN), cus = target / 2;
    int64_t max_steps = 1;
    for (int l = 0; l < n_layers; ++l)
      max_steps = std::max<int64_t>(max_steps, layers[l].d_in / kBigK);
    // Candidates: the K steps per block that split the longest layer into
    // 1, 2, ... (at most 1024) parts, and any layer into 1 to 4 parts.
    std::set<int64_t> cand;
    for (int64_t parts = 1; parts <= std::min<int64_t>(max_steps, 1024); ++parts)
      cand.insert(ceil_div(max_steps, parts));
    for (int l = 0; l < n_layers; ++l)
      for (int64_t parts = 1; parts <= 4; ++parts)
        cand.insert(ceil_div(layers[l].d_in / kBigK, parts));
    // Time of one launch in K steps. A launch of at most 4 rounds of
    // resident blocks is simulated as the hardware runs it: each XCD takes a
    // contiguous range of the logical blocks (xcd_logical_block) in order,
    // one block per CU as CUs free up, so blocks of unequal lengths can
    // leave a long tail; a longer launch is estimated as max(work / CUs,
    // longest block).
    auto launch_steps = [&](int l0, int l1, int64_t sps) {
      std::vector<int64_t> lens;
      int64_t work = 0, longest = 0;
      for (int l = l0; l < l1; ++l) {
        const int64_t steps = layers[l].d_in / kBigK, sp = ceil_div(steps, sps),
                      per = ceil_div(steps, sp);
        work += tiles * steps;
        longest = std::max(longest, per);
        if (static_cast<int64_t>(lens.size()) <= 4 * cus)
          for (int64_t k = 0; k < sp; ++k)
            lens.insert(lens.end(), tiles, std::min(per, steps - k * per));
      }
      const int64_t blocks = static_cast<int64_t>(lens.size());
      if (blocks > 4 * cus) return std::max(ceil_div(work, cus), longest);
      const int64_t per_xcd = ceil_div(blocks, 8), slots = cus / 8;
      int64_t span = 0;
      for (int64_t x = 0; x < 8; ++x) {
        // the CUs' finish times; the next block goes to the earliest
        std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>> busy(
            std::greater<int64_t>(), std::vector<int64_t>(slots, 0));
        int64_t end = 0;
        for (int64_t b = x * per_xcd; b < std::min(blocks, (x + 1) * per_xcd); ++b) {
          const int64_t t = busy.top() + lens[b];
          busy.pop();
          busy.push(t);
          end = std::max(end, t);
        }
        span = std::max(span, end);
      }
      return span;
    };
    double best = -1.0;
    for (auto it = cand.rbegin(); it != cand.rend(); ++it) {  // longest first
      const int64_t sps = *it;
      double part = 0.0;
      int64_t steps_total = 0;
      for (int l0 = 0; l0 < n_layers; l0 += kMaxLayers)
        steps_total += launch_steps(l0, std::min(n_layers, l0 + kMaxLayers), sps);
      for (int l = 0; l < n_layers; ++l) {
        const int64_t sp = ceil_div(layers[l].d_in / kBigK, sps);
        if (sp > 1) part += 2.0 * sp * r * BT * 4;
      }
      // the split partials (written, then read back by the xsum launch),
      // counted at a third of the bytes a K step moves per CU: measured,
      // a split of dec24's 8192-wide layers cost about three times what
      // their bytes at that rate predict
      const double t = static_cast<double>(steps_total) +
                       3.0 * part / (static_cast<double>(kBigM + kBigN) * kBigK * 2 * cus);
      if (best < 0.0 || t < best) {
        best = t;
        big_sps = sps;
      }
    }
  }
  size_t off = 0;
  for (int l = 0; l < n_layers; ++l) {
    const int64_t ldp = round_up(layers[l].d_in, 8);
    p.ldp.push_back(ldp);
    p.off_P.push_back(off);
    off = align_up(off + static_cast<size_t>(r) * ldp * es);
    p.off_Xt.push_back(off);
    off = align_up(off + static_cast<size_t>(B) * r * p.ldt * es);
    const int64_t nsteps = p.big ? layers[l].d_in / kBigK : ceil_div(layers[l].d_in, BK);
    int64_t splits = ceil_div(nsteps, p.big ? big_sps : steps_per_block);
    const int64_t sps = ceil_div(nsteps, splits);
    splits = ceil_div(nsteps, sps);
    p.m_tiles_proj.push_back(p.big ? static_cast<int32_t>(r / kBigM) : mt);
    p.n_tiles_proj.push_back(static_cast<int32_t>(p.big ? BT / kBigN : ceil_div(BT, kTileN)));
    p.splits.push_back(static_cast<int32_t>(splits));
    p.steps_per_split.push_back(static_cast<int32_t>(sps));
    p.off_xpart.push_back(off);
    if (splits > 1) off = align_up(off + static_cast<size_t>(splits) * r * BT * 4);
  }
  int64_t d_out_sum = 0;
  for (int l = 0; l < n_layers; ++l) d_out_sum += layers[l].d_out;

  // Regular per-sample passes: 128 x 128 tiles, 4 waves, two blocks per CU.
  SampPlan& q = p.samp;
  int64_t tiles_s = 0;
  for (int l = 0; l < n_layers; ++l) {
    const int32_t nt = static_cast<int32_t>(ceil_div(layers[l].d_out, kTileN));
    q.m_tiles.push_back(mt);
    q.n_tiles.push_back(nt);
    q.slot0.push_back(q.n_slots / 4);
    q.n_slots += 4 * mt * nt;  // one partial per wave
    tiles_s += static_cast<int64_t>(mt) * nt;
  }
  // Both per-sample passes give each block a run of samples of one tile. The
  // run length is chosen to minimise (rounds of resident blocks) x (samples
  // per block), so that the last round is not a small fraction of the chip.
  // Norm pass, T within one step: one sample per block, which keeps its Xt
  // tile in LDS over a run of column tiles (ties: the longer run).
  if (ceil_div(T, BK) == 1) {
    int64_t best = -1, max_nt = 1;
    for (int l = 0; l < n_layers; ++l)
      max_nt = std::max<int64_t>(max_nt, ceil_div(layers[l].d_out, kTileN));
    for (int64_t per = 1; per <= max_nt; ++per) {
      int64_t blocks = 0;
      for (int l = 0; l < n_layers; ++l)
        blocks += mt * B * ceil_div(ceil_div(layers[l].d_out, kTileN), per);
      const int64_t cost = ceil_div(blocks, target) * per;
      if (best < 0 || cost <= best) {
        best = cost;
        q.norm_res_tiles = static_cast<int32_t>(per);
      }
    }
  }
  // Norm pass otherwise: runs of up to 8 samples (ties: the longer run).
  {
    int64_t best = -1;
    for (int64_t pb = 1; pb <= std::min<int64_t>(8, B); ++pb) {
      const int64_t cost = ceil_div(tiles_s * ceil_div(B, pb), target) * pb;
      if (best < 0 || cost <= best) {
        best = cost;
        q.norm_per_block = static_cast<int32_t>(pb);
      }
    }
  }
  // Sum pass: sample groups, each adding one fp32 partial of G_priv that the
  // final pass reads back. The group size minimises the bytes the chip moves:
  // (rounds of resident blocks) x (blocks per round) x (operand bytes per
  // block), plus the partials written and read again (ties: fewer groups).
  {
    const double tile_bytes =
        static_cast<double>(ceil_div(T, BK)) * BK * (kTileM + kTileN) * es;
    double best = -1.0;
    for (int64_t per = std::min<int64_t>(B, kSumMaxGroup); per >= 1; --per) {
      const int64_t g = ceil_div(B, per);
      const double main = static_cast<double>(ceil_div(tiles_s * g, target)) * target *
                          per * tile_bytes;
      const double part = 2.0 * g * r * static_cast<double>(d_out_sum) * 4.0;
      if (best < 0.0 || main + part < best) {
        best = main + part;
        q.per_group = static_cast<int32_t>(per);
      }
    }
  }
  q.groups = static_cast<int32_t>(ceil_div(B, q.per_group));
  q.fuse_scale = q.per_group <= kFuseMaxGroup && q.n_slots <= kFuseMaxSlots;

  // Large per-sample passes (bf16; r, d_out whole 256 x 256 tiles; T whole
  // K steps): one 16-wave block per CU, launched kMaxLayers layers at a time.
  // The norm run and the sum group minimise the same estimates, summed over
  // the launches, with the rounds of resident blocks counted in K steps
  // (plus two per block for the pipeline's fill).
  p.has_samp_big = dtype == DPG_BF16 && r % kBigM == 0 && T % kSampBigK == 0;
  // (stored products: 32-bit offsets over 256 rows; copies through buffer
  // resources: each layer's dY and Xt within 32-bit offsets)
  if (static_cast<uint64_t>(B) * r * round_up(T, 8) * 2 >= (1ull << 32)) p.has_samp_big = false;
  for (int l = 0; l < n_layers; ++l)
    if (layers[l].d_out % kBigN != 0 ||
        static_cast<uint64_t>(layers[l].d_out) * 4 * kBigM >= (1ull << 32) ||
        static_cast<uint64_t>(B) * T * layers[l].d_out * 2 >= (1ull << 32))
      p.has_samp_big = false;
  if (p.has_samp_big) {
    SampPlan& b = p.samp_big;
    b.big = true;
    const int32_t mtb = r / kBigM;
    std::vector<int64_t> chunk_tiles;
    for (int l = 0; l < n_layers; ++l) {
      const int32_t nt = static_cast<int32_t>(layers[l].d_out / kBigN);
      b.m_tiles.push_back(mtb);
      b.n_tiles.push_back(nt);
      b.slot0.push_back(b.n_slots / 16);
      b.n_slots += 16 * mtb * nt;  // one partial per wave
      if (l % kMaxLayers == 0) chunk_tiles.push_back(0);
      chunk_tiles.back() += static_cast<int64_t>(mtb) * nt;
    }
    const int64_t cus = target / 2, kc = T / kSampBigK;
    auto step_rounds = [&](int64_t per) {
      const int64_t runs = ceil_div(B, per);
      int64_t t = 0;
      for (int64_t c : chunk_tiles) t += ceil_div(c * runs, cus) * (per * kc + 2);
      return t;
    };
    int64_t best = -1;
    for (int64_t pb = 1; pb <= std::min<int64_t>(B, kSumMaxGroup); ++pb) {
      const int64_t cost = step_rounds(pb);
      if (best < 0 || cost <= best) {
        best = cost;
        b.norm_per_block = static_cast<int32_t>(pb);
      }
    }
    const double step_bytes = static_cast<double>(kBigM + kBigN) * kSampBigK * es;
    double best_sum = -1.0;
    for (int64_t per = std::min<int64_t>(B, kSumMaxGroup); per >= 1; --per) {
      const int64_t g = ceil_div(B, per);
      const double cost = static_cast<double>(step_rounds(per)) * cus * step_bytes +
                          2.0 * g * r * static_cast<double>(d_out_sum) * 4.0;
      if (best_sum < 0.0 || cost < best_sum) {
        best_sum = cost;
        b.per_group = static_cast<int32_t>(per);
      }
    }
    b.groups = static_cast<int32_t>(ceil_div(B, b.per_group));
    b.fuse_scale = b.per_group <= kFuseMaxGroup && b.n_slots <= kFuseMaxSlots;
  }

  p.hat_sum = 8 * static_cast<int64_t>(r) <= T;
  const int32_t groups = std::max<int64_t>({static_cast<int64_t>(q.groups),
                                            p.has_samp_big ? p.samp_big.groups : 0,
                                            p.hat_sum ? B : 0});
  const int32_t n_slots = std::max(q.n_slots, p.has_samp_big ? p.samp_big.n_slots : 0);
  for (int l = 0; l < n_layers; ++l) {
    p.off_part.push_back(off);
    off = align_up(off + static_cast<size_t>(groups) * r * layers[l].d_out * 4);
  }
  p.off_norm = off;
  off = align_up(off + static_cast<size_t>(B) * n_slots * 4);
  p.off_scales = off;
  off = align_up(off + static_cast<size_t>(B) * 4);
  p.total = off;
  return p;
}

// ---------------------------------------------------- update call planning --

struct AdamPlan {
  std::vector<size_t> off_P, off_U;
  size_t total = 0;
};

int validate_adam_shapes(const dpg_layer_param* params, int32_t n_layers,
                         int32_t r, int32_t dtype) {
  if (!params) return fail(DPG_ERR_INVALID_ARG, "params is NULL");
  if (n_layers < 1 || n_layers > (1 << 20))
    return fail(DPG_ERR_INVALID_ARG, "n_layers must be in [1, 2^20]");
  if (r < 1) return fail(DPG_ERR_INVALID_ARG, "r must be >= 1");
  if (!valid_dtype(dtype)) return fail(DPG_ERR_INVALID_ARG, "unknown dtype");
  for (int i = 0; i < n_layers; ++i) {
    const int st = check_layer_shape(params[i].d_in, params[i].d_out, r, i);
    if (st) return st;
    if (params[i].reserved != 0)
      return fail(DPG_ERR_INVALID_ARG, "reserved field must be 0");
  }
  return check_unique_ids(params, n_layers);
}

AdamPlan plan_adam(const dpg_layer_param* params, int32_t n_layers, int32_t r,
                   int32_t dtype) {
  AdamPlan p;
  const size_t es = elem_size(dtype);
  size_t off = 0;
  for (int l = 0; l < n_layers; ++l) {
    p.off_P.push_back(off);
    off = align_up(off + static_cast<size_t>(params[l].d_in) * r * es);
    p.off_U.push_back(off);
    off = align_up(off + static_cast<size_t>(params[l].d_out) * r * es);
  }
  p.total = off;
  return p;
}

int check_workspace(void* ws, size_t have, size_t need) {
  if (need > 0 && !ws) return fail(DPG_ERR_WORKSPACE, "workspace is NULL");
  if (have < need)
    return fail(DPG_ERR_WORKSPACE, "workspace too small: need " +
                                       std::to_string(need) + " bytes, got " +
                                       std::to_string(have));
  if (reinterpret_cast<uintptr_t>(ws) % kAlign != 0)
    return fail(DPG_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return DPG_OK;
}

int check_seed_steps(uint64_t step, uint64_t proj_step) {
  if (step < 1 || step > kMaxU32)
    return fail(DPG_ERR_INVALID_ARG, "step must be in [1, 2^32)");
  if (proj_step > kMaxU32)
    return fail(DPG_ERR_INVALID_ARG, "proj_step must be < 2^32");
  return DPG_OK;
}

bool aligned(const void* p, size_t a) {
  return reinterpret_cast<uintptr_t>(p) % a == 0;
}

// Fills one P-generation descriptor; returns its number of blocks.
int fill_gen_p(GenPLayer& L, void* out, int64_t d_in, int64_t ld,
               uint32_t layer_id, int32_t r, int block0) {
  L.out = out;
  L.d_in = static_cast<int32_t>(d_in);
  L.ld = static_cast<int32_t>(ld);
  L.layer_id = layer_id;
  L.n_ctr = static_cast<int32_t>((static_cast<uint64_t>(r) * d_in + 3) / 4);
  L.block0 = block0;
  return static_cast<int>(ceil_div(L.n_ctr, kThreads));
}

// W -= lr P^T U for layers [l0, l1) of `params` (one launch): P_of(l) is
// layer l's P (row stride ldp_of(l)), U_of(l) its U [r][d_out], in the
// operand type.
template <class PF, class LF, class UF>
int enqueue_back(const dpg_layer_param* params, int l0, int l1, int32_t r,
                 int32_t dtype, double lr, PF P_of, LF ldp_of, UF U_of,
                 hipStream_t s) {
  const bool bf16 = dtype == DPG_BF16;
  BackArgs b;
  std::memset(&b, 0, sizeof(b));
  b.r = r;
  b.lr = static_cast<float>(lr);
  // r within one step: each block keeps its P tile and sweeps a run of
  // column tiles; the run minimises (rounds of resident blocks) x (tiles
  // per block), ties to the longer run
  if (ceil_div(r, step_of(dtype)) == 1) {
    int64_t best = -1, max_nt = 1;
    for (int l = l0; l < l1; ++l)
      max_nt = std::max<int64_t>(max_nt, ceil_div(params[l].d_out, kBackN));
    for (int64_t per = 1; per <= max_nt; ++per) {
      int64_t nb = 0;
      for (int l = l0; l < l1; ++l)
        nb += ceil_div(params[l].d_in, kTileM) * ceil_div(ceil_div(params[l].d_out, kBackN), per);
      const int64_t cost = ceil_div(nb, target_blocks(dtype)) * per;
      if (best < 0 || cost <= best) {
        best = cost;
        b.res_tiles = static_cast<int32_t>(per);
      }
    }
  }
  // Large bf16 back-projections (r over one step, a multiple of kBackBigK;
  // d_in whole 256-row tiles, d_out whole 128-column tiles; 16-byte aligned
  // rows): 4-wave blocks, two per CU, each sweeping a run of column tiles;
  // the run minimises (rounds of resident blocks) x (tiles per block) x (K
  // steps per tile plus about eight steps' worth of W traffic), ties to the
  // longer run, and is at most an eighth of every layer's column tiles, so
  // that each group of 8 row tiles has at least 8 runs: the blocks one XCD
  // runs at once then share 8 slices of P and 8 of U (the kernel's block
  // order), instead of each re-reading a P slice of its own from HBM.
  b.big = bf16 && r % kBackBigK == 0 && r > step_of(dtype);
  for (int l = l0; l < l1; ++l)
    if (params[l].d_in % kBigM != 0 || params[l].d_out % kBackBigN != 0 ||
        !aligned(params[l].W, 16) || !aligned(P_of(l), 16) || !aligned(U_of(l), 16) ||
        (ldp_of(l) * elem_size(dtype)) % 16 != 0 ||
        static_cast<uint64_t>(params[l].d_out) * 4 * kBigM >= (1ull << 32) ||  // W: 32-bit offsets
        static_cast<uint64_t>(r) * ldp_of(l) * 2 >= (1ull << 32) ||          // P, U: buffer copies
        static_cast<uint64_t>(r) * params[l].d_out * 2 >= (1ull << 32))
      b.big = 0;
  if (b.big) {
    int64_t best = -1, max_per = INT64_MAX;
    for (int l = l0; l < l1; ++l)
      max_per = std::min<int64_t>(max_per, std::max<int64_t>(1, params[l].d_out / kBackBigN / 8));
    const int64_t resident = target_blocks(dtype), kr = r / kBackBigK;
    for (int64_t per = 1; per <= max_per; ++per) {
      int64_t nb = 0;
      for (int l = l0; l < l1; ++l)
        nb += (params[l].d_in / kBigM) * ceil_div(params[l].d_out / kBackBigN, per);
      const int64_t cost = ceil_div(nb, resident) * per * (kr + 8);
      if (best < 0 || cost <= best) {
        best = cost;
        b.res_tiles = static_cast<int32_t>(per);
      }
    }
    int blocks = 0;
    for (int l = l0; l < l1; ++l) {
      BackLayer& L = b.L[l - l0];
      L.P = P_of(l);
      L.U = U_of(l);
      L.ldp = static_cast<int32_t>(ldp_of(l));
      L.W = params[l].W;
      L.d_in = static_cast<int32_t>(params[l].d_in);
      L.d_out = static_cast<int32_t>(params[l].d_out);
      L.m_tiles = static_cast<int32_t>(params[l].d_in / kBigM);
      L.n_tiles = static_cast<int32_t>(params[l].d_out / kBackBigN);
      L.n_chunks = static_cast<int32_t>(ceil_div(L.n_tiles, b.res_tiles));
      L.block0 = blocks;
      blocks += L.m_tiles * L.n_chunks;
    }
    b.n_layers = l1 - l0;
    b.n_blocks = blocks;
    return timed(K_BACK, s, [&] { return launch_back(b, bf16, true, s); });
  }
  int blocks = 0;
  bool pair = true;
  for (int l = l0; l < l1; ++l) {
    BackLayer& L = b.L[l - l0];
    L.P = P_of(l);
    L.U = U_of(l);
    L.ldp = static_cast<int32_t>(ldp_of(l));
    L.W = params[l].W;
    L.d_in = static_cast<int32_t>(params[l].d_in);
    L.d_out = static_cast<int32_t>(params[l].d_out);
    L.m_tiles = static_cast<int32_t>(ceil_div(params[l].d_in, kTileM));
    L.n_tiles = static_cast<int32_t>(ceil_div(params[l].d_out, kBackN));
    L.block0 = blocks;
    if (b.res_tiles > 0) {
      L.n_chunks = static_cast<int32_t>(ceil_div(L.n_tiles, b.res_tiles));
      blocks += L.m_tiles * L.n_chunks;
    } else {
      blocks += L.m_tiles * L.n_tiles;
    }
    // bf16: P and U are gathered two columns (4 bytes) at a time
    pair = pair && ldp_of(l) % 2 == 0 && params[l].d_out % 2 == 0;
  }
  b.n_layers = l1 - l0;
  b.n_blocks = blocks;
  b.off32 = 1;
  for (int l = l0; l < l1; ++l)
    if (static_cast<uint64_t>(r) * std::max<int64_t>(ldp_of(l), params[l].d_out) *
            elem_size(dtype) >= (1ull << 31))
      b.off32 = 0;
  // every tile and step full: d_in, d_out whole tiles, r whole steps, W
  // rows 8-byte aligned
  b.full = pair && b.off32 && r % step_of(dtype) == 0;
  for (int l = l0; l < l1; ++l)
    if (params[l].d_in % kTileM != 0 || params[l].d_out % kBackN != 0 || !aligned(params[l].W, 8))
      b.full = 0;
  return timed(K_BACK, s, [&] { return launch_back(b, bf16, pair, s); });
}

// Adam and back-projection settings of the one-call step.
struct StepUpdate {
  const dpg_layer_param* params;
  double lr, beta1, beta2, eps;
};

// Bytes of the one-call step's U buffers, appended after the projection
// workspace (offsets relative to its start).
size_t step_u_bytes(const dpg_layer_grad* layers, int32_t n_layers, int32_t r,
                    int32_t dtype, size_t base, std::vector<size_t>* off_U) {
  size_t off = base;
  for (int l = 0; l < n_layers; ++l) {
    if (off_U) off_U->push_back(off);
    off = align_up(off + static_cast<size_t>(r) * layers[l].d_out * elem_size(dtype));
  }
  return off - base;
}

int check_adam_hyper(double lr, double beta1, double beta2, double eps) {
  if (!(lr > 0.0) || std::isinf(lr))
    return fail(DPG_ERR_INVALID_ARG, "lr must be finite and > 0");
  if (!(beta1 >= 0.0 && beta1 < 1.0) || !(beta2 >= 0.0 && beta2 < 1.0))
    return fail(DPG_ERR_INVALID_ARG, "beta1 and beta2 must be in [0, 1)");
  if (!(eps > 0.0) || std::isinf(eps))
    return fail(DPG_ERR_INVALID_ARG, "eps must be finite and > 0");
  return DPG_OK;
}

int check_clip_sigma(double clip_C, double sigma) {
  if (!(clip_C > 0.0))
    return fail(DPG_ERR_INVALID_ARG, "clip_C must be > 0");
  if (!(sigma >= 0.0) || std::isinf(sigma))
    return fail(DPG_ERR_INVALID_ARG, "sigma must be finite and >= 0");
  if (std::isinf(clip_C) && sigma != 0.0)
    return fail(DPG_ERR_INVALID_ARG, "sigma must be 0 when clip_C is infinite");
  return DPG_OK;
}

// Probe stream tag of the randomized-clipping norm estimate (P uses 0, the
// noise 1).
constexpr uint32_t kTagProbe = 3;

// The projection call. With ghat == nullptr: the whole batch step (norms,
// clip, sum, noise into each layer's G_priv). With ghat: the streaming form
// for one layer (its product tiles into ghat, its squared norms added into
// norm_sq); clip_C, sigma, step and sample_norms are then unused.
// With upd (the one-call step): the final stage also runs Adam on G_priv,
// and the back-projection follows, reading the P this call generated; the
// U buffers live after the projection workspace.
// With rc_scales (the randomized-clipping norm estimate, on layers whose A
// and dY the caller has swapped, so that "P" holds the probes on the d_out
// side): P is drawn from the probe stream, the call stops after the norms,
// and the clip factors go to rc_scales; sigma and G_priv are unused.
int project_impl(const dpg_layer_grad* layers, int32_t n_layers, int64_t B,
                 int64_t T, int32_t r, int32_t dtype, double clip_C,
                 double sigma, uint64_t seed, uint64_t step,
                 uint64_t proj_step, float* sample_norms, void* workspace,
                 size_t workspace_bytes, void* stream, float* ghat,
                 float* norm_sq, const StepUpdate* upd = nullptr,
                 float* rc_scales = nullptr) {
  const bool layer_mode = ghat != nullptr;
  const bool rc = rc_scales != nullptr;
  int st = validate_proj_shapes(layers, n_layers, B, T, r, dtype);
  if (st) return st;
  for (int i = 0; i < n_layers; ++i)
    if (!layers[i].A || !layers[i].dY || (!layer_mode && !rc && !layers[i].G_priv))
      return fail(DPG_ERR_INVALID_ARG,
                  "NULL data pointer in layer index " + std::to_string(i));
  if (layer_mode && !norm_sq) return fail(DPG_ERR_INVALID_ARG, "norm_sq is NULL");
  if (!layer_mode && (st = check_clip_sigma(clip_C, rc ? 0.0 : sigma))) return st;
  if ((st = check_seed_steps(layer_mode ? 1 : step, proj_step))) return st;
  const ProjPlan p = plan_proj(layers, n_layers, B, T, r, dtype);
  std::vector<size_t> off_U;
  const size_t u_bytes = upd ? step_u_bytes(layers, n_layers, r, dtype, p.total, &off_U) : 0;
  if ((st = check_workspace(workspace, workspace_bytes, p.total + u_bytes))) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const bool bf16 = dtype == DPG_BF16;
  const int vec_elems = static_cast<int>(16 / elem_size(dtype));
  float* norm_part = reinterpret_cast<float*>(ws + p.off_norm);
  float* scales = reinterpret_cast<float*>(ws + p.off_scales);
  const uint32_t k0 = static_cast<uint32_t>(seed), k1 = static_cast<uint32_t>(seed >> 32);
  const int64_t BT = B * T;

  for (int l0 = 0; l0 < n_layers; l0 += kMaxLayers) {
    const int l1 = std::min(n_layers, l0 + kMaxLayers);
    // 1. P_l, row-major [r][ldp], regenerated from the seed
    {
      GenPArgs a;
      std::memset(&a, 0, sizeof(a));
      a.r = r;
      a.scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(r)));
      a.k0 = k0;
      a.k1 = k1;
      a.step_word = static_cast<uint32_t>(proj_step);
      a.tag = rc ? kTagProbe : 0u;
      int blocks = 0;
      for (int l = l0; l < l1; ++l)
        blocks += fill_gen_p(a.L[l - l0], ws + p.off_P[l], layers[l].d_in,
                             p.ldp[l], layers[l].layer_id, r, blocks);
      a.n_layers = l1 - l0;
      if ((st = timed(K_GEN_P, s, [&] { return launch_gen_p(a, blocks, bf16, s); })))
        return st;
    }
    // 2. Xt_l = P_l A_l^T, per sample [r][T] (or split partials)
    ProjArgs a;
    std::memset(&a, 0, sizeof(a));
    a.B = static_cast<int32_t>(B);
    a.T = static_cast<int32_t>(T);
    a.r = r;
    a.ldt = static_cast<int32_t>(p.ldt);
    XsumArgs x;
    std::memset(&x, 0, sizeof(x));
    x.B = a.B;
    x.T = a.T;
    x.r = r;
    x.ldt = a.ldt;
    int blocks = 0, xblocks = 0, nx = 0;
    bool vec = true;
    for (int l = l0; l < l1; ++l) {
      ProjLayer& L = a.L[l - l0];
      L.A = layers[l].A;
      L.P = ws + p.off_P[l];
      L.Xt = ws + p.off_Xt[l];
      L.part = reinterpret_cast<float*>(ws + p.off_xpart[l]);
      L.d_in = static_cast<int32_t>(layers[l].d_in);
      L.ldp = static_cast<int32_t>(p.ldp[l]);
      L.m_tiles = p.m_tiles_proj[l];
      L.n_tiles = p.n_tiles_proj[l];
      L.splits = p.splits[l];
      L.steps_per_split = p.steps_per_split[l];
      L.block0 = blocks;
      blocks += L.m_tiles * L.n_tiles * L.splits;
      vec = vec && layers[l].d_in % vec_elems == 0 && aligned(layers[l].A, 16);
      if (L.splits > 1) {
        XsumLayer& X = x.L[nx++];
        X.part = L.part;
        X.Xt = L.Xt;
        X.splits = L.splits;
        X.block0 = xblocks;
        xblocks += static_cast<int>(ceil_div(ceil_div(BT, 4) * r, kThreads));
      }
    }
    a.n_layers = l1 - l0;
    a.n_blocks = blocks;
    if (p.big) {
      // the direct copies need 16-byte aligned rows of A; otherwise the
      // regular kernel runs these layers unsplit (no partials are needed)
      a.big = 1;
      for (int l = l0; l < l1; ++l)
        if (!aligned(layers[l].A, 16)) a.big = 0;
      if (!a.big) {
        blocks = 0;
        nx = 0;
        xblocks = 0;
        const int64_t BK = step_of(dtype);
        for (int l = l0; l < l1; ++l) {
          ProjLayer& L = a.L[l - l0];
          L.m_tiles = static_cast<int32_t>(ceil_div(r, kTileM));
          L.n_tiles = static_cast<int32_t>(ceil_div(BT, kTileN));
          L.splits = 1;
          L.steps_per_split = static_cast<int32_t>(ceil_div(layers[l].d_in, BK));
          L.block0 = blocks;
          blocks += L.m_tiles * L.n_tiles;
        }
        a.n_blocks = blocks;
      }
    }
    // 32-bit tile offsets: 128 rows of A or of P (row stride ldp)
    a.off32 = 1;
    for (int l = l0; l < l1; ++l)
      if (static_cast<uint64_t>(kTileN) * p.ldp[l] * elem_size(dtype) >= (1ull << 31))
        a.off32 = 0;
    // every tile and step full: r and B*T whole tiles, d_in whole steps
    a.full = vec && a.off32 && r % kTileM == 0 && BT % kTileN == 0;
    for (int l = l0; l < l1; ++l)
      if (layers[l].d_in % step_of(dtype) != 0) a.full = 0;
    // two wave groups per block when every block has at least two K steps
    // to share (the plan gives about one block per CU)
    a.groups2 = 1;
    for (int l = l0; l < l1; ++l)
      if (p.steps_per_split[l] < 2) a.groups2 = 0;
    if ((st = timed(K_PROJ, s, [&] { return launch_proj(a, bf16, vec, s); }))) return st;
    if (nx > 0) {
      x.n_layers = nx;
      if ((st = timed(K_XSUM, s, [&] { return launch_xsum(x, xblocks, bf16, s); })))
        return st;
    }
  }

  // the large per-sample kernel copies dY rows with 16-byte transfers (in
  // the streaming form it also stores each sample's product tile)
  const bool hat_sum = p.hat_sum && !layer_mode && !rc;
  bool samp_big = p.has_samp_big;
  for (int l = 0; l < n_layers; ++l)
    if (!aligned(layers[l].dY, 16)) samp_big = false;
  const SampPlan& sp = samp_big ? p.samp_big : p.samp;
  auto fill_samp = [&](SampArgs& a, int l0, int l1, bool sum, bool* pair) {
    std::memset(&a, 0, sizeof(a));
    a.big = sp.big;
    a.B = static_cast<int32_t>(B);
    a.T = static_cast<int32_t>(T);
    a.r = r;
    a.ldt = static_cast<int32_t>(p.ldt);
    a.per_block = sum ? sp.per_group : sp.norm_per_block;
    a.res_tiles = sum ? 0 : sp.norm_res_tiles;
    a.n_slots = sp.n_slots;
    a.norm_part = norm_part;
    a.scales = scales;
    a.fuse_scale = sum && sp.fuse_scale;
    a.clip_C = static_cast<float>(clip_C);
    a.norms_out = (sum && sp.fuse_scale && l0 == 0) ? sample_norms : nullptr;
    const int64_t runs = ceil_div(B, a.per_block);
    int blocks = 0;
    *pair = true;
    for (int l = l0; l < l1; ++l) {
      SampLayer& L = a.L[l - l0];
      L.dY = layers[l].dY;
      L.Xt = ws + p.off_Xt[l];
      L.part = reinterpret_cast<float*>(ws + p.off_part[l]);
      L.d_out = static_cast<int32_t>(layers[l].d_out);
      L.m_tiles = sp.m_tiles[l];
      L.n_tiles = sp.n_tiles[l];
      L.slot0 = sp.slot0[l];
      L.block0 = blocks;
      if (a.res_tiles > 0) {
        L.n_chunks = static_cast<int32_t>(ceil_div(L.n_tiles, a.res_tiles));
        blocks += static_cast<int>(L.m_tiles * L.n_chunks * B);
      } else {
        blocks += static_cast<int>(L.m_tiles * L.n_tiles * runs);
      }
      // bf16: dY is gathered two columns (4 bytes) at a time
      *pair = *pair && layers[l].d_out % 2 == 0 && aligned(layers[l].dY, 4);
    }
    a.n_layers = l1 - l0;
    a.n_blocks = blocks;
    // 32-bit tile offsets: one sample of dY, and 128 rows of Xt
    a.off32 = static_cast<uint64_t>(kTileM) * p.ldt * elem_size(dtype) < (1ull << 31);
    for (int l = l0; l < l1; ++l)
      if (static_cast<uint64_t>(T) * layers[l].d_out * elem_size(dtype) >= (1ull << 31))
        a.off32 = 0;
    // every tile and step full: r and d_out whole tiles, T whole steps
    a.full = *pair && a.off32 && r % kTileM == 0 && T % step_of(dtype) == 0;
    for (int l = l0; l < l1; ++l)
      if (layers[l].d_out % kTileN != 0) a.full = 0;
  };
  // 3. squared-norm partials of every (sample, layer, tile), and with
  //    hat_sum every sample's product
  for (int l0 = 0; l0 < n_layers; l0 += kMaxLayers) {
    const int l1 = std::min(n_layers, l0 + kMaxLayers);
    SampArgs a;
    bool pair;
    fill_samp(a, l0, l1, false, &pair);
    if (layer_mode) a.L[0].ghat = ghat;
    if (hat_sum)
      for (int l = l0; l < l1; ++l) a.L[l - l0].ghat = reinterpret_cast<float*>(ws + p.off_part[l]);
    if ((st = timed(K_NORM, s, [&] { return launch_samp_norm(a, bf16, pair, s); })))
      return st;
  }
  if (layer_mode) {
    NormAccArgs a{norm_part, sp.n_slots, static_cast<int32_t>(B), norm_sq};
    return timed(K_CLIP, s, [&] { return launch_norm_acc(a, s); });
  }
  if (rc) {
    ScaleArgs a;
    a.norm_part = norm_part;
    a.n_slots = sp.n_slots;
    a.clip_C = static_cast<float>(clip_C);
    a.scales = rc_scales;
    a.norms_out = sample_norms;
    return timed(K_SCALE, s, [&] { return launch_scale(a, static_cast<int>(B), s); });
  }
  // 4. per-sample norm and clip factor (needs every layer's partials); the
  //    sum pass does it itself when the groups are small
  if (!sp.fuse_scale || hat_sum) {
    ScaleArgs a;
    a.norm_part = norm_part;
    a.n_slots = sp.n_slots;
    a.clip_C = static_cast<float>(clip_C);
    a.scales = scales;
    a.norms_out = sample_norms;
    if ((st = timed(K_SCALE, s, [&] { return launch_scale(a, static_cast<int>(B), s); })))
      return st;
  }
  // 5-6. clipped sum over samples (or, with hat_sum, over the stored
  //      products weighted by the clip factors in the final pass), then
  //      noise and 1/B
  const double noise = sigma == 0.0 ? 0.0 : sigma * clip_C;
  for (int l0 = 0; l0 < n_layers; l0 += kMaxLayers) {
    const int l1 = std::min(n_layers, l0 + kMaxLayers);
    SampArgs a;
    bool pair;
    if (!hat_sum) {
      fill_samp(a, l0, l1, true, &pair);
      if ((st = timed(K_SUM, s, [&] { return launch_samp_sum(a, bf16, pair, s); })))
        return st;
    }
    FinArgs f;
    std::memset(&f, 0, sizeof(f));
    f.groups = hat_sum ? static_cast<int32_t>(B) : sp.groups;
    f.weights = hat_sum ? scales : nullptr;
    f.noise_scale = static_cast<float>(noise);
    f.inv_B = static_cast<float>(1.0 / static_cast<double>(B));
    f.k0 = k0;
    f.k1 = k1;
    f.step_word = static_cast<uint32_t>(step);
    int blocks = 0;
    for (int l = l0; l < l1; ++l) {
      FinLayer& L = f.L[l - l0];
      L.part = reinterpret_cast<const float*>(ws + p.off_part[l]);
      L.out = layers[l].G_priv;
      L.n_elem = static_cast<int32_t>(static_cast<int64_t>(r) * layers[l].d_out);
      L.layer_id = layers[l].layer_id;
      L.block0 = blocks;
      blocks += static_cast<int>(ceil_div(ceil_div(L.n_elem, 4), kThreads));
    }
    f.n_layers = l1 - l0;
    if (!upd) {
      if ((st = timed(K_FIN, s, [&] { return launch_fin(f, blocks, s); }))) return st;
      continue;
    }
    // the one-call step: Adam on G_priv in the same pass, then W -= lr P^T U
    const double t = static_cast<double>(step);
    f.beta1 = static_cast<float>(upd->beta1);
    f.beta2 = static_cast<float>(upd->beta2);
    f.one_m_beta1 = static_cast<float>(1.0 - upd->beta1);
    f.one_m_beta2 = static_cast<float>(1.0 - upd->beta2);
    f.bc1 = static_cast<float>(1.0 - std::pow(upd->beta1, t));
    f.bc2 = static_cast<float>(1.0 - std::pow(upd->beta2, t));
    f.eps = static_cast<float>(upd->eps);
    for (int l = l0; l < l1; ++l) {
      FinLayer& L = f.L[l - l0];
      L.m = upd->params[l].m;
      L.v = upd->params[l].v;
      L.U = ws + off_U[l];
    }
    if ((st = timed(K_FIN, s, [&] { return launch_fin_adam(f, blocks, bf16, s); })))
      return st;
    if ((st = enqueue_back(upd->params, l0, l1, r, dtype, upd->lr,
                           [&](int l) { return ws + p.off_P[l]; },
                           [&](int l) { return p.ldp[l]; },
                           [&](int l) { return ws + off_U[l]; }, s)))
      return st;
  }
  return DPG_OK;
}

// Validates the one-call step's update arguments and runs it in `workspace`.
int private_step_impl(const dpg_layer_grad* layers, const dpg_layer_param* params,
                      int32_t n_layers, int64_t B, int64_t T, int32_t r, int32_t dtype,
                      double clip_C, double sigma, double lr, double beta1, double beta2,
                      double eps, uint64_t seed, uint64_t step, uint64_t proj_step,
                      float* sample_norms, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (!params) return fail(DPG_ERR_INVALID_ARG, "params is NULL");
  int st = validate_adam_shapes(params, n_layers, r, dtype);
  if (st) return st;
  if (!layers) return fail(DPG_ERR_INVALID_ARG, "layers is NULL");
  for (int i = 0; i < n_layers; ++i) {
    if (params[i].d_in != layers[i].d_in || params[i].d_out != layers[i].d_out ||
        params[i].layer_id != layers[i].layer_id)
      return fail(DPG_ERR_INVALID_ARG, "params and layers differ at layer index " +
                                           std::to_string(i));
    if (!params[i].W || !params[i].m || !params[i].v)
      return fail(DPG_ERR_INVALID_ARG,
                  "NULL data pointer in layer index " + std::to_string(i));
  }
  if ((st = check_adam_hyper(lr, beta1, beta2, eps))) return st;
  const StepUpdate upd{params, lr, beta1, beta2, eps};
  return project_impl(layers, n_layers, B, T, r, dtype, clip_C, sigma, seed, step,
                      proj_step, sample_norms, workspace, workspace_bytes, stream,
                      nullptr, nullptr, &upd);
}

}  // namespace

int dpg::record_error(int code, const char* msg) { return fail(code, msg); }

extern "C" {

int dpg_version(void) { return 10100; }

const char* dpg_status_string(int status) {
  switch (status) {
    case DPG_OK: return "DPG_OK";
    case DPG_ERR_INVALID_ARG: return "DPG_ERR_INVALID_ARG: invalid argument";
    case DPG_ERR_WORKSPACE: return "DPG_ERR_WORKSPACE: workspace missing, too small or misaligned";
    case DPG_ERR_UNSUPPORTED: return "DPG_ERR_UNSUPPORTED: unsupported configuration";
    case DPG_ERR_HIP: return "DPG_ERR_HIP: HIP runtime error";
    default: return "unknown dpg status";
  }
}

const char* dpg_last_error(void) { return g_last_error.c_str(); }

int dpg_project_workspace_size(const dpg_layer_grad* layers, int32_t n_layers,
                               int64_t B, int64_t T, int32_t r, int32_t dtype,
                               size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(DPG_ERR_INVALID_ARG, "bytes is NULL");
  const int st = validate_proj_shapes(layers, n_layers, B, T, r, dtype);
  if (st) return st;
  *bytes = plan_proj(layers, n_layers, B, T, r, dtype).total;
  return DPG_OK;
}

int dpg_adam_workspace_size(const dpg_layer_param* params, int32_t n_layers,
                            int32_t r, int32_t dtype, size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(DPG_ERR_INVALID_ARG, "bytes is NULL");
  const int st = validate_adam_shapes(params, n_layers, r, dtype);
  if (st) return st;
  *bytes = plan_adam(params, n_layers, r, dtype).total;
  return DPG_OK;
}

int dpg_project_clip_noise(const dpg_layer_grad* layers, int32_t n_layers,
                           int64_t B, int64_t T, int32_t r, int32_t dtype,
                           double clip_C, double sigma, uint64_t seed,
                           uint64_t step, uint64_t proj_step,
                           float* sample_norms, void* workspace,
                           size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  return project_impl(layers, n_layers, B, T, r, dtype, clip_C, sigma, seed, step,
                      proj_step, sample_norms, workspace, workspace_bytes, stream,
                      nullptr, nullptr);
}

int dpg_step_workspace_size(const dpg_layer_grad* layers, int32_t n_layers,
                            int64_t B, int64_t T, int32_t r, int32_t dtype,
                            size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(DPG_ERR_INVALID_ARG, "bytes is NULL");
  const int st = validate_proj_shapes(layers, n_layers, B, T, r, dtype);
  if (st) return st;
  const ProjPlan p = plan_proj(layers, n_layers, B, T, r, dtype);
  *bytes = p.total + step_u_bytes(layers, n_layers, r, dtype, p.total, nullptr);
  return DPG_OK;
}

int dpg_private_step(const dpg_layer_grad* layers, const dpg_layer_param* params,
                     int32_t n_layers, int64_t B, int64_t T, int32_t r,
                     int32_t dtype, double clip_C, double sigma, double lr,
                     double beta1, double beta2, double eps, uint64_t seed,
                     uint64_t step, uint64_t proj_step, float* sample_norms,
                     void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  return private_step_impl(layers, params, n_layers, B, T, r, dtype, clip_C, sigma, lr,
                           beta1, beta2, eps, seed, step, proj_step, sample_norms,
                           workspace, workspace_bytes, stream);
}

namespace {
// The estimate's layers with A and dY swapped: the projection kernels then
// form dY_i Q^T (the probes on the d_out side) and the norm pass
// ||(dY_i Q^T)^T A_i||^2 = ||A_i^T dY_i Q^T||^2.
int rc_swapped(const dpg_layer_grad* layers, int32_t n_layers, std::vector<dpg_layer_grad>* out) {
  if (!layers) return fail(DPG_ERR_INVALID_ARG, "layers is NULL");
  if (n_layers < 1 || n_layers > (1 << 20))
    return fail(DPG_ERR_INVALID_ARG, "n_layers must be in [1, 2^20]");
  out->assign(layers, layers + n_layers);
  for (auto& L : *out) {
    std::swap(L.d_in, L.d_out);
    std::swap(L.A, L.dY);
    L.G_priv = nullptr;
  }
  return DPG_OK;
}
}  // namespace

int dpg_rc_norms_workspace_size(const dpg_layer_grad* layers, int32_t n_layers, int64_t B,
                                int64_t T, int32_t k, int32_t dtype, size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(DPG_ERR_INVALID_ARG, "bytes is NULL");
  std::vector<dpg_layer_grad> sw;
  int st = rc_swapped(layers, n_layers, &sw);
  if (st) return st;
  if ((st = validate_proj_shapes(sw.data(), n_layers, B, T, k, dtype))) return st;
  *bytes = plan_proj(sw.data(), n_layers, B, T, k, dtype).total;
  return DPG_OK;
}

int dpg_rc_norms(const dpg_layer_grad* layers, int32_t n_layers, int64_t B, int64_t T,
                 int32_t k, int32_t dtype, double clip_C, uint64_t seed, uint64_t step,
                 float* norms, float* scales, void* workspace, size_t workspace_bytes,
                 void* stream) {
  g_last_error.clear();
  if (!norms || !scales) return fail(DPG_ERR_INVALID_ARG, "norms and scales must not be NULL");
  std::vector<dpg_layer_grad> sw;
  const int st = rc_swapped(layers, n_layers, &sw);
  if (st) return st;
  return project_impl(sw.data(), n_layers, B, T, k, dtype, clip_C, 0.0, seed, step, step, norms,
                      workspace, workspace_bytes, stream, nullptr, nullptr, nullptr, scales);
}

int dpg_project_layer_workspace_size(const dpg_layer_grad* layer, int64_t B,
                                     int64_t T, int32_t r, int32_t dtype,
                                     size_t* bytes) {
  return dpg_project_workspace_size(layer, 1, B, T, r, dtype, bytes);
}

int dpg_project_layer(const dpg_layer_grad* layer, int64_t B, int64_t T,
                      int32_t r, int32_t dtype, uint64_t seed,
                      uint64_t proj_step, float* G_hat, float* norm_sq,
                      void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!G_hat) return fail(DPG_ERR_INVALID_ARG, "G_hat is NULL");
  return project_impl(layer, 1, B, T, r, dtype, 1.0, 0.0, seed, 1, proj_step,
                      nullptr, workspace, workspace_bytes, stream, G_hat, norm_sq);
}

int dpg_clip_workspace_size(int64_t B, size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(DPG_ERR_INVALID_ARG, "bytes is NULL");
  if (B < 1 || B > (1ll << 30)) return fail(DPG_ERR_INVALID_ARG, "B must be in [1, 2^30]");
  *bytes = align_up(static_cast<size_t>(B) * 4);
  return DPG_OK;
}

int dpg_clip_sum_noise(const dpg_layer_hat* layers, int32_t n_layers,
                       int64_t B, int32_t r, double clip_C, double sigma,
                       uint64_t seed, uint64_t step, const float* norm_sq,
                       float* sample_norms, void* workspace,
                       size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!layers) return fail(DPG_ERR_INVALID_ARG, "layers is NULL");
  if (n_layers < 1 || n_layers > (1 << 20))
    return fail(DPG_ERR_INVALID_ARG, "n_layers must be in [1, 2^20]");
  if (B < 1 || B > (1ll << 30) || r < 1)
    return fail(DPG_ERR_INVALID_ARG, "B must be in [1, 2^30] and r >= 1");
  if (!norm_sq) return fail(DPG_ERR_INVALID_ARG, "norm_sq is NULL");
  int st;
  for (int i = 0; i < n_layers; ++i) {
    if ((st = check_layer_shape(1, layers[i].d_out, r, i))) return st;
    if (layers[i].reserved != 0)
      return fail(DPG_ERR_INVALID_ARG, "reserved field must be 0");
    if (!layers[i].G_hat || !layers[i].G_priv)
      return fail(DPG_ERR_INVALID_ARG,
                  "NULL data pointer in layer index " + std::to_string(i));
  }
  if ((st = check_unique_ids(layers, n_layers))) return st;
  if ((st = check_clip_sigma(clip_C, sigma))) return st;
  if ((st = check_seed_steps(step, 0))) return st;
  if ((st = check_workspace(workspace, workspace_bytes, align_up(static_cast<size_t>(B) * 4))))
    return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* scales = static_cast<float*>(workspace);
  ClipArgs c{norm_sq, static_cast<int32_t>(B), static_cast<float>(clip_C), scales,
             sample_norms};
  if ((st = timed(K_CLIP, s, [&] { return launch_clip(c, s); }))) return st;
  const double noise = sigma == 0.0 ? 0.0 : sigma * clip_C;
  for (int l0 = 0; l0 < n_layers; l0 += kMaxLayers) {
    const int l1 = std::min(n_layers, l0 + kMaxLayers);
    FinArgs f;
    std::memset(&f, 0, sizeof(f));
    f.weights = scales;
    f.groups = static_cast<int32_t>(B);
    f.noise_scale = static_cast<float>(noise);
    f.inv_B = static_cast<float>(1.0 / static_cast<double>(B));
    f.k0 = static_cast<uint32_t>(seed);
    f.k1 = static_cast<uint32_t>(seed >> 32);
    f.step_word = static_cast<uint32_t>(step);
    int blocks = 0;
    for (int l = l0; l < l1; ++l) {
      FinLayer& L = f.L[l - l0];
      L.part = layers[l].G_hat;
      L.out = layers[l].G_priv;
      L.n_elem = static_cast<int32_t>(static_cast<int64_t>(r) * layers[l].d_out);
      L.layer_id = layers[l].layer_id;
      L.block0 = blocks;
      blocks += static_cast<int>(ceil_div(ceil_div(L.n_elem, 4), kThreads));
    }
    f.n_layers = l1 - l0;
    if ((st = timed(K_FIN, s, [&] { return launch_fin(f, blocks, s); }))) return st;
  }
  return DPG_OK;
}

int dpg_adam_backproject(const dpg_layer_param* params, int32_t n_layers,
                         int32_t r, int32_t dtype, double lr, double beta1,
                         double beta2, double eps, uint64_t seed, uint64_t step,
                         uint64_t proj_step, void* workspace,
                         size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  int st = validate_adam_shapes(params, n_layers, r, dtype);
  if (st) return st;
  for (int i = 0; i < n_layers; ++i)
    if (!params[i].G_priv || !params[i].W || !params[i].m || !params[i].v)
      return fail(DPG_ERR_INVALID_ARG,
                  "NULL data pointer in layer index " + std::to_string(i));
  if ((st = check_adam_hyper(lr, beta1, beta2, eps))) return st;
  if ((st = check_seed_steps(step, proj_step))) return st;
  const AdamPlan p = plan_adam(params, n_layers, r, dtype);
  if ((st = check_workspace(workspace, workspace_bytes, p.total))) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const bool bf16 = dtype == DPG_BF16;
  const double t = static_cast<double>(step);
  for (int l0 = 0; l0 < n_layers; l0 += kMaxLayers) {
    const int l1 = std::min(n_layers, l0 + kMaxLayers);
    // 5. Adam on [r][d_out] (U row-major) and P_l regenerated [r][d_in]
    PrepArgs a;
    std::memset(&a, 0, sizeof(a));
    a.r = r;
    a.beta1 = static_cast<float>(beta1);
    a.beta2 = static_cast<float>(beta2);
    a.one_m_beta1 = static_cast<float>(1.0 - beta1);
    a.one_m_beta2 = static_cast<float>(1.0 - beta2);
    a.bc1 = static_cast<float>(1.0 - std::pow(beta1, t));
    a.bc2 = static_cast<float>(1.0 - std::pow(beta2, t));
    a.eps = static_cast<float>(eps);
    a.p_scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(r)));
    a.k0 = static_cast<uint32_t>(seed);
    a.k1 = static_cast<uint32_t>(seed >> 32);
    a.step_word = static_cast<uint32_t>(proj_step);
    int blocks = 0;
    for (int l = l0; l < l1; ++l) {
      AdamLayer& L = a.A[l - l0];
      L.g = params[l].G_priv;
      L.m = params[l].m;
      L.v = params[l].v;
      L.U = ws + p.off_U[l];
      L.n_elem = static_cast<int32_t>(static_cast<int64_t>(r) * params[l].d_out);
      L.block0 = blocks;
      blocks += static_cast<int>(ceil_div(ceil_div(L.n_elem, 4), kThreads));
    }
    a.adam_blocks = blocks;
    int pblocks = 0;
    for (int l = l0; l < l1; ++l)
      pblocks += fill_gen_p(a.P[l - l0], ws + p.off_P[l], params[l].d_in,
                            params[l].d_in, params[l].layer_id, r, pblocks);
    a.n_layers = l1 - l0;
    if ((st = timed(K_PREP, s, [&] { return launch_prep(a, blocks + pblocks, bf16, s); })))
      return st;
    // 6. W -= lr P^T U
    if ((st = enqueue_back(params, l0, l1, r, dtype, lr,
                           [&](int l) { return ws + p.off_P[l]; },
                           [&](int l) { return params[l].d_in; },
                           [&](int l) { return ws + p.off_U[l]; }, s)))
      return st;
  }
  return DPG_OK;
}

int dpg_timing_enable(int on) {
  std::lock_guard<std::mutex> g(g_timing_mu);
  g_timing_on = on != 0;
  return DPG_OK;
}

int dpg_timing_read(double* total_ms, int64_t* launches, int32_t n_kinds,
                    int reset) {
  g_last_error.clear();
  std::vector<TimedLaunch> pend;
  {
    std::lock_guard<std::mutex> g(g_timing_mu);
    pend.swap(g_pending);
  }
  hipError_t err = hipSuccess;
  double add[K_COUNT] = {};
  int64_t cnt[K_COUNT] = {};
  for (const TimedLaunch& t : pend) {
    float ms = 0.0f;
    hipError_t e = hipEventSynchronize(t.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.start, t.stop);
    if (e != hipSuccess && err == hipSuccess) err = e;
    if (e == hipSuccess) {
      add[t.kind] += ms;
      cnt[t.kind] += 1;
    }
    (void)hipEventDestroy(t.start);
    (void)hipEventDestroy(t.stop);
  }
  std::lock_guard<std::mutex> g(g_timing_mu);
  for (int k = 0; k < K_COUNT; ++k) {
    g_total_ms[k] += add[k];
    g_launches[k] += cnt[k];
  }
  for (int k = 0; k < K_COUNT && k < n_kinds; ++k) {
    if (total_ms) total_ms[k] = g_total_ms[k];
    if (launches) launches[k] = g_launches[k];
  }
  if (reset)
    for (int k = 0; k < K_COUNT; ++k) {
      g_total_ms[k] = 0.0;
      g_launches[k] = 0;
    }
  if (err != hipSuccess)
    return fail(DPG_ERR_HIP, std::string("timing events: ") + hipGetErrorString(err));
  return DPG_OK;
}

const char* dpg_kernel_name(int kind) {
  return (kind >= 0 && kind < K_COUNT) ? kKindName[kind] : "";
}

int dpg_philox_normals(uint64_t seed, uint32_t layer_id, uint32_t step_word,
                       uint32_t tag, uint64_t start, uint64_t n, float* z_out,
                       uint32_t* words_out, void* stream) {
  g_last_error.clear();
  if (n == 0) return DPG_OK;
  if (!z_out) return fail(DPG_ERR_INVALID_ARG, "z_out is NULL");
  if (start + n > kMaxU32 || start + n < start)
    return fail(DPG_ERR_INVALID_ARG, "start + n must be < 2^32");
  hipStream_t s = static_cast<hipStream_t>(stream);
  return check(launch_philox_normals(static_cast<uint32_t>(seed),
                                     static_cast<uint32_t>(seed >> 32), layer_id,
                                     step_word, tag, static_cast<uint32_t>(start),
                                     static_cast<uint32_t>(n), z_out, words_out, s),
               "philox_normals", s);
}

}  // extern "C"
