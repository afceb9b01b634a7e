// Host side of the verification library: handle, workspace, argument
// checks and stream-ordered launches of the kernels in sv_kernels.hpp.
#include "spec_verify.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <mutex>

#include "sv_drift.hpp"
#include "sv_trunc.hpp"
#include "sv_trunc32.hpp"

#ifndef SV_U_BF16
#define SV_U_BF16 4
#endif
#ifndef SV_U_F32
#define SV_U_F32 4
#endif
#ifndef SV_U_MAX
#define SV_U_MAX 4
#endif

namespace {

constexpr int kMaxSeg = 16;
constexpr long long kWalkGrid = 2048;   // walk-order reading: workgroups after position 0
static_assert(kMaxSeg <= sv::kTopmMaxSeg, "top-m lists are laid out for kTopmMaxSeg segments");
constexpr int kProfCalls = 4096;
constexpr double kLog2e = 1.4426950408889634073599246810018921;

// last error of spec_verify_noalloc on this thread (it has no handle to hold it)
thread_local char g_noalloc_err[256] = {0};

struct Launch {
  int vec;          // elements per chunk: 8 (bf16) / 4 (fp32) vector path, 1 scalar path
  int nseg;         // segments per row in the streaming pass
  int seg_chunks;   // chunks per segment
  int ntiles;       // draw tiles per row
};

}  // namespace

struct spec_verify_handle {
  int device = 0;
  int max_batch = 0, K = 0, V = 0, dtype = 0;
  double decay = 0.99;
  sv::RowPart* parts = nullptr;
  sv::DrawRow* draw = nullptr;
  sv::TileSums* tsum = nullptr;
  double* table = nullptr;            // bf16 exponential table of the current call
  int tiles_per_group = 16;           // draw tiles per workgroup (tuning)
  int fused_min_batch = 0;            // smallest batch for one workgroup per sequence, 0 = off
  int finish_seq = 1;                 // scan + draw + pick in one kernel after the streaming pass
  int claim_tiles = 1;                // finish_seq's wavefronts claim draw tiles from a counter
  double* ema = nullptr;
  int32_t* steps = nullptr;
  int32_t* streak = nullptr;          // tree-shape policy state, per slot
  sv::DevStats* stats = nullptr;
  int ntiles_max = 0;
  unsigned long long calls = 0;
  double* aux_p = nullptr;
  double* aux_q = nullptr;
  double* aux_z = nullptr;
  int32_t* aux_argmax = nullptr;
  hipEvent_t* prof_ev = nullptr;   // 3 events per recorded call
  bool prof_call_end = false;      // also record the end of each call
  sv::Rules rules{};   // stopping rules and tree-shape policy for later calls
  sv::Trunc trunc{nullptr, nullptr};       // top-k / top-p truncation for later calls
  int drift_m = 0;                         // draft residual side output: support width
  int32_t* drift_sup = nullptr;            //   [max_batch][K][m] support, null = off
  double* drift_res = nullptr;             //   [max_batch][K][m] residuals
  uint64_t* topm_lists = nullptr;          // streaming-pass top-m lists (allocated by set_residual)
  int topm_nseg = 0;                       // segments per row of this call's lists, 0 = none
  bool topm_merged = false;                // this call's finish also merged the lists
  double res_invT = 1.0;                   // this call's 1 / temperature
  int merge_in_finish = 1;     // lists merged inside the finish when they fit (0: own kernel)
  int walk = 0;                // stochastic calls read rows in walk order (spec_verify_set_walk_order)
  int32_t* walk_seq = nullptr;  // walk-order reading: sequences whose walk keeps position 0
  uint32_t* walk_cnt = nullptr; //   and their count
  int lds_cu = 160 * 1024;                 // LDS bytes per compute unit
  int prof_cap = 0, prof_n = 0;
  int target_wgs = 2048;   // streaming-pass workgroups to aim for (tuning)
  int target_wgs_max = 6144;  // the same for the argmax pass (greedy, margin)
  int n_cu = 256;          // compute units of the device
  int nseg_force = 0;      // fixed segment count (tuning), 0 = automatic
  int trunc32_buf = 1;     // fp32 truncation: walk the digits over an LDS copy of the few candidates (0 = digit reads only)
  int trunc32_list = 1;    // fp32 truncation: settle rows from one read's top-k list first (0 = off)
  int trunc32_one = 1;     // fp32 truncation: rows with top-p alone in one read after the list pass (0 = off)
  char err[256] = {0};
};

namespace {

int fail(spec_verify_handle* h, int code, const char* fmt, ...) {
  if (h != nullptr) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(h->err, sizeof(h->err), fmt, ap);
    va_end(ap);
  }
  return code;
}

int check_launch(spec_verify_handle* h, const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(h, SV_EHIP, "%s: %s", what, hipGetErrorString(e));
  return SV_OK;
}

inline int div_up(long long a, long long b) { return int((a + b - 1) / b); }

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  return (s != nullptr && *s) ? atoi(s) : dflt;
}

// argmax: the max pass, which does less arithmetic per byte and finishes its
// segments sooner; it is planned for more workgroups (about three rounds of
// the resident ones) so that the last round's tail stays short
Launch plan(const spec_verify_handle* h, int B, int rows, int vec, int U, bool argmax = false) {
  Launch L;
  L.vec = vec;
  const long long nchunks = h->V / vec;
  const long long min_seg = (long long)sv::kBlock * U;
  int max_nseg = int(nchunks / min_seg);
  if (max_nseg < 1) max_nseg = 1;
  if (max_nseg > kMaxSeg) max_nseg = kMaxSeg;
  // with per-sequence draft counts some (row, segment) workgroups exit at
  // once; four times as many, shorter ones keep the other rows evenly spread
  const long long base = argmax ? h->target_wgs_max : h->target_wgs;
  const long long target =
      h->rules.k != nullptr ? std::max(base, 4ll * h->target_wgs) : base;
  int nseg = h->nseg_force > 0 ? h->nseg_force : div_up(target, (long long)B * rows);
  if (nseg > max_nseg) nseg = max_nseg;
  if (nseg < 1) nseg = 1;
  L.seg_chunks = div_up(nchunks, nseg);
  L.nseg = div_up(nchunks, L.seg_chunks);
  if (L.nseg < 1) L.nseg = 1;
  L.ntiles = div_up(nchunks, sv::kTileChunks);
  return L;
}

// entries per sign of the bf16 exponential table that the scaled lookups use:
// exponent fields from 2^-25 up, as many as keep |x * c| < 1000
int tab_half(double c) {
  int n = sv::kTabMaxExp;
  while (n > 1 && std::ldexp(1.0, n - 25) * c > 1000.0) --n;
  return n * 128;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// static LDS bytes of a kernel (SIZE_MAX when the runtime cannot say)
template <class F>
size_t static_lds(F* kernel) {
  hipFuncAttributes fa;
  return hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(kernel)) == hipSuccess
             ? fa.sharedSizeBytes
             : SIZE_MAX / 4;
}

// Event k (0: before the streaming pass, 1: after it, 2: after the call) of
// the current recorded call.
void prof_mark(spec_verify_handle* h, int k, hipStream_t s) {
  if (h->prof_ev != nullptr && h->prof_n < h->prof_cap)
    (void)hipEventRecord(h->prof_ev[3 * h->prof_n + k], s);
}

// Stochastic mode, multi-kernel pipeline: streaming pass over every
// (row, segment), acceptance scan, draw tile sums, pick.
template <int DT, int VEC, int U>
int run_stochastic(spec_verify_handle* h, int B, const void* target, const void* draft,
                   const int32_t* tokens, const float* uniforms, float c, double c64,
                   int32_t* out_tokens, int32_t* out_len, uint32_t* hist, hipStream_t s) {
  const int K = h->K, V = h->V;
  const int rows = 2 * K + 1;
  bool topm = false;
  if constexpr ((DT == sv::DT_BF16 && VEC == 8) || (DT == sv::DT_F32 && VEC == 4))
    topm = h->drift_sup != nullptr && h->topm_lists != nullptr;
  // walk-order reading (not with the residual side output, which needs every
  // draft row): the streaming pass runs in stages of positions, each planned
  // as if every sequence were still being walked
  const bool walk = h->walk && !topm;
  sv::Rules rules = h->rules;
  rules.walk = walk ? 1 : 0;
  // (walk-order reading: position 0's two rows are planned for half the usual
  // workgroups, i.e. segments twice as long, which measured a little faster:
  // c3 87.0 against 91.9 us per call)
  const Launch L = plan(h, B, walk ? 4 : rows, VEC, U);
  const bool tab = (DT == sv::DT_BF16 && VEC == 8);
  const int n_half = tab_half(c64);
  const int groups = div_up(L.ntiles, h->tiles_per_group);
  const int grid_seq = div_up(B, sv::kWavesPerBlock);
  const sv::StageRows all_rows{0, K + 1, 0, K, 0, nullptr};
  prof_mark(h, 0, s);
  if constexpr ((DT == sv::DT_BF16 && VEC == 8) || (DT == sv::DT_F32 && VEC == 4)) {
    // the residual side output takes its draft-row candidates from this pass
    if (topm) {
      hipLaunchKernelGGL((sv::rowstats_sum<DT, VEC, U, true>), dim3(unsigned(B * rows * L.nseg)),
                         dim3(sv::kBlock), 0, s, target, draft, 0, K, V, L.nseg, L.seg_chunks, c,
                         h->rules.k, h->parts, hist, h->drift_m, h->topm_lists, tokens, all_rows,
                         uniforms);
      h->topm_nseg = L.nseg;
    }
  }
  if (walk) {
    // position 0's rows of every sequence; then the sequences whose walk
    // keeps position 0 are listed, and their rows of positions 1..K (target
    // rows 1..k_b, draft rows 1..k_b-1) are streamed by a fixed grid
    const sv::StageRows first{0, 1, 0, 1, 0, h->walk_cnt};
    hipLaunchKernelGGL((sv::rowstats_sum<DT, VEC, U>), dim3(unsigned(B * 2 * L.nseg)),
                       dim3(sv::kBlock), 0, s, target, draft, 0, K, V, L.nseg, L.seg_chunks, c,
                       h->rules.k, h->parts, hist, 0, nullptr, tokens, first, uniforms);
    hipLaunchKernelGGL(sv::walk_gate, dim3(unsigned(grid_seq)), dim3(sv::kBlock), 0, s, B, K, V,
                       L.nseg, h->parts, h->rules.k, tokens, uniforms, c, 1, h->walk_seq,
                       h->walk_cnt);
    const long long rest = (long long)B * (2 * K - 1) * L.nseg;
    hipLaunchKernelGGL((sv::rowstats_sum_list<DT, VEC, U>),
                       dim3(unsigned(std::min<long long>(rest, kWalkGrid))), dim3(sv::kBlock), 0,
                       s, target, draft, K, V, L.nseg, L.seg_chunks, c, h->rules.k, h->parts,
                       tokens, h->walk_seq, h->walk_cnt, 1);
  } else if (!topm) {
    hipLaunchKernelGGL((sv::rowstats_sum<DT, VEC, U>), dim3(unsigned(B * rows * L.nseg)),
                       dim3(sv::kBlock), 0, s, target, draft, 0, K, V, L.nseg, L.seg_chunks, c,
                       h->rules.k, h->parts, hist, 0, nullptr, tokens, all_rows, uniforms);
  }
  int rc = check_launch(h, "rowstats_sum");
  prof_mark(h, 1, s);
  if (rc) return rc;
  h->topm_merged = false;
  if (h->finish_seq && L.ntiles <= sv::kFMaxTiles && rows <= sv::kFMaxRows) {
    // with at least two sequences per compute unit, 512-thread workgroups
    // let two sequences share a unit, so one's scan and pick overlap the
    // other's loads (c5: 918 -> 899 us per call); below that, 1024 threads
    // keep every unit's waves on its one sequence
    const bool half = B >= 2 * h->n_cu;
    const int NT = half ? sv::kFinishBlockHalf : sv::kFinishBlock;
    auto kern = half ? sv::finish_seq<DT, VEC, sv::kFinishBlockHalf, false>
                     : sv::finish_seq<DT, VEC, sv::kFinishBlock, false>;
    // the lists' merge inside the finish, one wavefront per drafted position
    // after its draw tiles, when a position's lists hold at most 256 slots and
    // their keys fit in the LDS the finish leaves (one or two workgroups per
    // compute unit as above); else drift_merge after it
    sv::MergeJob mj;
    size_t dyn = 0;
    if (topm && h->merge_in_finish && K < NT / sv::kWave &&
        sv::merge_fits(L.nseg, h->drift_m, V)) {
      const size_t need = size_t(K) * sv::merge_lds_words() * 8;
      static const size_t lds_static[2] = {static_lds(sv::finish_seq<DT, VEC, sv::kFinishBlock,
                                                                    false>),
                                           static_lds(sv::finish_seq<DT, VEC,
                                                                    sv::kFinishBlockHalf, false>)};
      if ((lds_static[half ? 1 : 0] + need) * (half ? 2 : 1) <= size_t(h->lds_cu)) {
        mj.lists = h->topm_lists;
        mj.nseg = L.nseg;
        mj.m = h->drift_m;
        mj.invT = h->res_invT;
        mj.sup = h->drift_sup;
        mj.res = h->drift_res;
        dyn = need;
        h->topm_merged = true;
      }
    }
    hipLaunchKernelGGL(kern, dim3(B), dim3(NT), dyn, s, K, V, L.nseg, h->parts, target, draft,
                       tokens, uniforms, c, c64, n_half, rules, out_tokens, out_len, hist,
                       h->ema, h->steps, h->decay, h->stats, h->aux_p, h->aux_q, h->aux_z,
                       nullptr, mj, h->claim_tiles);
    return check_launch(h, "finish_seq");
  }
  hipLaunchKernelGGL((sv::scan_stochastic<DT>), dim3(grid_seq), dim3(sv::kBlock), 0, s, 0, B, K,
                     V, L.nseg, h->parts, target, draft, tokens, uniforms, c, rules, out_tokens,
                     out_len, hist, h->ema, h->steps, h->decay, h->stats, h->draw, h->aux_p, h->aux_q,
                     h->aux_z, tab ? h->table : nullptr, n_half, c64);
  if ((rc = check_launch(h, "scan_stochastic"))) return rc;
  hipLaunchKernelGGL((sv::draw<DT, VEC>), dim3(B * groups), dim3(sv::kBlock), 0, s, 0, B, K, V,
                     L.ntiles, h->tiles_per_group, groups, target, draft, h->draw, c64, n_half,
                     h->table, h->tsum);
  if ((rc = check_launch(h, "draw"))) return rc;
  hipLaunchKernelGGL((sv::draw_pick<DT, VEC>), dim3(grid_seq), dim3(sv::kBlock), 0, s, 0, B, K,
                     V, L.ntiles, target, draft, h->draw, uniforms, c64, h->tsum, out_tokens,
                     h->stats, h->aux_z);
  return check_launch(h, "draw_pick");
}

// Stochastic mode with top-k / top-p truncation (bf16 rows): the truncation
// passes instead of the streaming pass (the window pass over every needed
// row, then the full-histogram pass over the rows it handed over, if any),
// then the per-sequence finish with masked tables.
template <int VEC>
int run_trunc(spec_verify_handle* h, int B, const void* target, const void* draft,
              const int32_t* tokens, const float* uniforms, float c, double c64,
              int32_t* out_tokens, int32_t* out_len, uint32_t* hist, hipStream_t s) {
  const int K = h->K, V = h->V;
  const int rows = 2 * K + 1;
  const int ntiles = div_up(V / VEC, sv::kTileChunks);
  if (ntiles > sv::kFMaxTiles || rows > sv::kFMaxRows)
    return fail(h, SV_EUNSUPPORTED, "truncation needs V <= %d (bf16)",
                sv::kFMaxTiles * sv::kTileChunks * VEC);
  // walk-order reading (not with the residual side output, which reads every
  // draft row): both truncation passes over position 0's rows of every
  // sequence, the sequences whose walk keeps position 0 listed, then both
  // passes over their other rows
  const bool walk = h->walk && h->drift_sup == nullptr;
  sv::Rules rules = h->rules;
  rules.walk = walk ? 1 : 0;
  int rc;
  prof_mark(h, 0, s);
  if (walk) {
    const sv::RowSel first{0, 1, 0, 1, nullptr, nullptr};
    const sv::RowSel rest{1, K + 1, 1, K, h->walk_seq, h->walk_cnt};
    hipLaunchKernelGGL((sv::rowstats_trunc_win<VEC>), dim3(unsigned(B * 2)), dim3(sv::kTwBlock), 0,
                       s, target, draft, B, K, V, c, c64, h->trunc, h->rules.k, h->parts, hist,
                       first, h->walk_cnt);
    hipLaunchKernelGGL((sv::rowstats_trunc<VEC>), dim3(unsigned(std::min(B * 2, h->n_cu))),
                       dim3(sv::kTrBlock), 0, s, target, draft, B, K, V, c, c64, h->trunc,
                       h->rules.k, h->parts, first);
    hipLaunchKernelGGL(sv::walk_gate_trunc, dim3(unsigned(div_up(B, sv::kBlock))),
                       dim3(sv::kBlock), 0, s, B, K, V, h->parts, target, draft, h->rules.k,
                       tokens, uniforms, c64, h->walk_seq, h->walk_cnt);
    hipLaunchKernelGGL((sv::rowstats_trunc_win<VEC>),
                       dim3(unsigned(std::max(1, B * (2 * K - 1)))), dim3(sv::kTwBlock), 0, s,
                       target, draft, B, K, V, c, c64, h->trunc, h->rules.k, h->parts, nullptr,
                       rest, nullptr);
    hipLaunchKernelGGL((sv::rowstats_trunc<VEC>), dim3(unsigned(h->n_cu)), dim3(sv::kTrBlock), 0,
                       s, target, draft, B, K, V, c, c64, h->trunc, h->rules.k, h->parts, rest);
    rc = check_launch(h, "truncation passes (walk order)");
    prof_mark(h, 1, s);
    if (rc) return rc;
  } else {
    const sv::RowSel all{0, K + 1, 0, K, nullptr, nullptr};
    hipLaunchKernelGGL((sv::rowstats_trunc_win<VEC>), dim3(unsigned(B * rows)),
                       dim3(sv::kTwBlock), 0, s, target, draft, B, K, V, c, c64, h->trunc,
                       h->rules.k, h->parts, hist, all, nullptr);
    rc = check_launch(h, "rowstats_trunc_win");
    prof_mark(h, 1, s);
    if (rc) return rc;
    hipLaunchKernelGGL((sv::rowstats_trunc<VEC>), dim3(unsigned(std::min(B * rows, h->n_cu))),
                       dim3(sv::kTrBlock), 0, s, target, draft, B, K, V, c, c64, h->trunc,
                       h->rules.k, h->parts, all);
    if ((rc = check_launch(h, "rowstats_trunc"))) return rc;
  }
  hipLaunchKernelGGL((sv::finish_seq<sv::DT_BF16, VEC, sv::kFinishBlock, true>), dim3(B),
                     dim3(sv::kFinishBlock), 0, s, K, V, 1, h->parts, target, draft, tokens,
                     uniforms, c, c64, tab_half(c64), rules, out_tokens, out_len, hist, h->ema,
                     h->steps, h->decay, h->stats, h->aux_p, h->aux_q, h->aux_z, h->trunc.k,
                     sv::MergeJob{}, h->claim_tiles);
  return check_launch(h, "finish_seq (truncated)");
}

// Stochastic mode with top-k / top-p truncation (fp32 rows): the list pass
// (16-byte chunks) settles most rows in one read, the multi-read pass takes
// the rows it hands over (every needed row for other chunks), then the
// per-sequence finish, whose draw compares each value's order key with its
// row's threshold.
template <int VEC>
int run_trunc32(spec_verify_handle* h, int B, const void* target, const void* draft,
                const int32_t* tokens, const float* uniforms, float c, double c64,
                int32_t* out_tokens, int32_t* out_len, uint32_t* hist, hipStream_t s) {
  const int K = h->K, V = h->V;
  const int rows = 2 * K + 1;
  const int ntiles = div_up(V / VEC, sv::kTileChunks);
  if (ntiles > sv::kFMaxTiles || rows > sv::kFMaxRows)
    return fail(h, SV_EUNSUPPORTED, "truncation needs V <= %d (fp32)",
                sv::kFMaxTiles * sv::kTileChunks * VEC);
  int lg = 0;                        // ceil(log2 V): fixed-point masses keep 61 - lg bits
  while ((1ll << lg) < (long long)V) ++lg;
  const bool list = VEC == 4 && h->trunc32_list;
  // the truncation passes over the rows sel selects (grid: one workgroup per
  // candidate row); the first launch clears the histogram and `clear`
  auto passes = [&](const sv::RowSel& sel, int grid, uint32_t* hist_, uint32_t* clear) -> int {
    int rc_ = SV_OK;
    if constexpr (VEC == 4) {
      if (list) {
        hipLaunchKernelGGL((sv::rowstats_trunc32_list<VEC>), dim3(unsigned(grid)),
                           dim3(sv::kT1Block), 0, s, target, draft, K, V, c, c64, 61 - lg,
                           h->trunc, h->rules.k, h->parts, hist_, B, sel, clear);
        rc_ = check_launch(h, "rowstats_trunc32_list");
        // the rows the list pass handed over (top-p alone, top-k past its
        // lists or tied at the k-th value): one read each where the copy
        // suffices
        if (rc_ == SV_OK && h->trunc32_one) {
          hipLaunchKernelGGL((sv::rowstats_trunc32_topp<VEC>), dim3(unsigned(grid)),
                             dim3(sv::kTPBlock), 0, s, target, draft, K, V, c, c64, 61 - lg,
                             h->trunc, h->rules.k, h->parts, B, sel);
          rc_ = check_launch(h, "rowstats_trunc32_topp");
        }
      }
    }
    if (rc_) return rc_;
    hipLaunchKernelGGL((sv::rowstats_trunc32<VEC>), dim3(unsigned(grid)), dim3(sv::kT32Block), 0,
                       s, target, draft, K, V, c, c64, 61 - lg, h->trunc32_buf, list ? 1 : 0,
                       h->trunc, h->rules.k, h->parts, list ? nullptr : hist_, B, sel,
                       list ? nullptr : clear);
    return check_launch(h, "rowstats_trunc32");
  };
  // walk-order reading (not with the residual side output, which reads every
  // draft row): the passes over position 0's rows of every sequence, the
  // sequences whose walk keeps position 0 listed, then the passes over their
  // other rows (a grid for every possible row; the rest return at once)
  const bool walk = h->walk && h->drift_sup == nullptr;
  sv::Rules rules = h->rules;
  rules.walk = walk ? 1 : 0;
  int rc;
  prof_mark(h, 0, s);
  if (walk) {
    const sv::RowSel first{0, 1, 0, 1, nullptr, nullptr};
    const sv::RowSel rest{1, K + 1, 1, K, h->walk_seq, h->walk_cnt};
    rc = passes(first, B * 2, hist, h->walk_cnt);
    if (rc) return rc;
    hipLaunchKernelGGL(sv::walk_gate_trunc32, dim3(unsigned(div_up(B, sv::kBlock))),
                       dim3(sv::kBlock), 0, s, B, K, V, h->parts, target, draft, h->rules.k,
                       tokens, uniforms, c64, h->walk_seq, h->walk_cnt);
    if ((rc = check_launch(h, "walk_gate_trunc32"))) return rc;
    rc = passes(rest, std::max(1, B * (2 * K - 1)), nullptr, nullptr);
  } else {
    const sv::RowSel all{0, K + 1, 0, K, nullptr, nullptr};
    rc = passes(all, B * rows, hist, nullptr);
  }
  prof_mark(h, 1, s);                // the truncation passes
  if (rc) return rc;
  if (B >= 2 * h->n_cu)                // as in run_stochastic
    hipLaunchKernelGGL((sv::finish_seq<sv::DT_F32, VEC, sv::kFinishBlockHalf, true>), dim3(B),
                       dim3(sv::kFinishBlockHalf), 0, s, K, V, 1, h->parts, target, draft,
                       tokens, uniforms, c, c64, 0, rules, out_tokens, out_len, hist, h->ema,
                       h->steps, h->decay, h->stats, h->aux_p, h->aux_q, h->aux_z, nullptr,
                       sv::MergeJob{}, h->claim_tiles);
  else
    hipLaunchKernelGGL((sv::finish_seq<sv::DT_F32, VEC, sv::kFinishBlock, true>), dim3(B),
                       dim3(sv::kFinishBlock), 0, s, K, V, 1, h->parts, target, draft, tokens,
                       uniforms, c, c64, 0, rules, out_tokens, out_len, hist, h->ema, h->steps,
                       h->decay, h->stats, h->aux_p, h->aux_q, h->aux_z, nullptr,
                       sv::MergeJob{}, h->claim_tiles);
  return check_launch(h, "finish_seq (truncated)");
}

// Stochastic mode, one workgroup per sequence (large batches).
template <int DT, int VEC, int U>
int run_fused(spec_verify_handle* h, int B, const void* target, const void* draft,
              const int32_t* tokens, const float* uniforms, float c, double c64,
              int32_t* out_tokens, int32_t* out_len, uint32_t* hist, hipStream_t s) {
  const int K = h->K, V = h->V;
  prof_mark(h, 0, s);
  hipLaunchKernelGGL(sv::zero_hist, dim3(1), dim3(64), 0, s, hist, K + 1);
  int rc = check_launch(h, "zero_hist");
  if (rc) return rc;
  hipLaunchKernelGGL((sv::verify_fused<DT, VEC, U>), dim3(B), dim3(sv::kFBlock), 0, s, K, V,
                     target, draft, tokens, uniforms, c, c64, tab_half(c64), h->rules, out_tokens,
                     out_len, hist, h->ema, h->steps, h->decay, h->stats, h->aux_p, h->aux_q,
                     h->aux_z);
  rc = check_launch(h, "verify_fused");
  prof_mark(h, 1, s);
  return rc;
}

// whether the one-workgroup-per-sequence kernel serves this call
bool use_fused(const spec_verify_handle* h, int B, int vec) {
  if (h->fused_min_batch <= 0 || B < h->fused_min_batch || vec == 1 || h->walk) return false;
  const long long ntiles = ((long long)h->V / vec + sv::kTileChunks - 1) / sv::kTileChunks;
  return ntiles <= sv::kFMaxTiles && 2 * h->K + 1 <= sv::kFMaxRows;
}

template <int DT, int VEC, int U>
int run_argmax(spec_verify_handle* h, const Launch& L, int B, const void* target,
               const int32_t* tokens, bool margin, double invT, double tau,
               int32_t* out_tokens, int32_t* out_len, uint32_t* hist, hipStream_t s) {
  const int K = h->K, V = h->V;
  const int rows = K + 1;
  const int grid2 = div_up(B, sv::kWavesPerBlock);
  sv::Rules rules = h->rules;
  rules.walk = h->walk ? 1 : 0;
  prof_mark(h, 0, s);
  if (h->walk) {
    // walk-order reading: target row 0 of every sequence, then the rows
    // 1..k_b of the sequences whose walk keeps position 0 (as for stochastic
    // calls)
    hipLaunchKernelGGL((sv::rowstats_max<DT, VEC, U>), dim3(unsigned((long long)B * L.nseg)),
                       dim3(sv::kBlock), 0, s, target, K, V, L.nseg, L.seg_chunks, h->rules.k,
                       h->parts, hist, 0, 1, h->walk_cnt);
    if (margin)
      hipLaunchKernelGGL((sv::walk_gate_argmax<DT, true>), dim3(grid2), dim3(sv::kBlock), 0, s, B,
                         K, V, L.nseg, h->parts, target, h->rules.k, tokens, invT, tau, 1,
                         h->walk_seq, h->walk_cnt);
    else
      hipLaunchKernelGGL((sv::walk_gate_argmax<DT, false>), dim3(grid2), dim3(sv::kBlock), 0, s,
                         B, K, V, L.nseg, h->parts, target, h->rules.k, tokens, invT, tau, 1,
                         h->walk_seq, h->walk_cnt);
    const long long rest = (long long)B * K * L.nseg;
    hipLaunchKernelGGL((sv::rowstats_max_list<DT, VEC, U>),
                       dim3(unsigned(std::max(1ll, std::min<long long>(rest, kWalkGrid)))),
                       dim3(sv::kBlock), 0, s, target, K, V, L.nseg, L.seg_chunks, h->rules.k,
                       h->parts, h->walk_seq, h->walk_cnt, 1);
  } else {
    hipLaunchKernelGGL((sv::rowstats_max<DT, VEC, U>), dim3(unsigned((long long)B * rows * L.nseg)),
                       dim3(sv::kBlock), 0, s, target, K, V, L.nseg, L.seg_chunks, h->rules.k,
                       h->parts, hist, 0, rows, nullptr);
  }
  int rc = check_launch(h, "rowstats_max");
  prof_mark(h, 1, s);
  if (rc) return rc;
  if (margin)
    hipLaunchKernelGGL((sv::scan_argmax<DT, true>), dim3(grid2), dim3(sv::kBlock), 0, s, B, K, V,
                       L.nseg, h->parts, target, tokens, invT, tau, rules, out_tokens, out_len,
                       hist,
                       h->ema, h->steps, h->decay, h->stats, h->aux_p, h->aux_q, h->aux_z,
                       h->aux_argmax);
  else
    hipLaunchKernelGGL((sv::scan_argmax<DT, false>), dim3(grid2), dim3(sv::kBlock), 0, s, B, K,
                       V, L.nseg, h->parts, target, tokens, invT, tau, rules, out_tokens, out_len,
                       hist,
                       h->ema, h->steps, h->decay, h->stats, h->aux_p, h->aux_q, h->aux_z,
                       h->aux_argmax);
  return check_launch(h, "scan_argmax");
}

// The residual side output after a stochastic call: from the streaming pass's
// lists when this call's pass kept them, else reading the draft rows.
template <int DT, int VEC>
void launch_residual(spec_verify_handle* h, int B, bool vec, const void* target,
                     const void* draft, double invT, const int32_t* out_len, hipStream_t s) {
  const dim3 grid(unsigned(B * h->K));
  if (h->topm_merged) return;          // done inside the finish
  if (h->topm_nseg > 0)
    hipLaunchKernelGGL(sv::drift_merge<DT>, grid, dim3(sv::kWave),
                       size_t(h->topm_nseg) * sv::kWavesPerBlock * std::min(h->drift_m, h->V) * 8,
                       s, target, draft, h->K, h->V, invT, h->drift_m, h->topm_nseg,
                       h->topm_lists, h->rules.k, out_len, h->drift_sup, h->drift_res);
  else if (vec)
    hipLaunchKernelGGL((sv::drift_residual<DT, VEC>), grid, dim3(sv::kDriftBlock), 0, s, target,
                       draft, h->K, h->V, invT, h->drift_m, h->rules.k, out_len, h->drift_sup,
                       h->drift_res);
  else
    hipLaunchKernelGGL((sv::drift_residual<DT, 1>), grid, dim3(sv::kDriftBlock), 0, s, target,
                       draft, h->K, h->V, invT, h->drift_m, h->rules.k, out_len, h->drift_sup,
                       h->drift_res);
}

// whether a call reads 16-byte chunks (the 128-bit load path)
bool use_vec(const spec_verify_handle* h, const void* target, const void* draft, int mode) {
  const int full_vec = h->dtype == SV_DTYPE_BF16 ? 8 : 4;
  bool vec = (h->V % full_vec) == 0 && aligned(target, 16);
  if (mode == SV_MODE_STOCHASTIC) vec = vec && aligned(draft, 16);
  return vec;
}

int verify_call(spec_verify_handle* h, int B, const void* target, const void* draft,
                const int32_t* tokens, const float* uniforms, float temperature, int mode,
                float tau, int32_t* out_tokens, int32_t* out_len, uint32_t* out_hist,
                hipStream_t stream);

void free_all(spec_verify_handle* h) {
  void* ptrs[] = {h->parts, h->draw,  h->tsum,  h->table,      h->ema,     h->steps,
                  h->streak, h->stats, h->topm_lists, h->walk_seq, h->walk_cnt};
  for (void* p : ptrs)
    if (p != nullptr) (void)hipFree(p);
}

}  // namespace

extern "C" {

const char* spec_verify_version(void) { return "specverify 0.1 (gfx950)"; }

int spec_verify_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (buf == nullptr || sink == nullptr || bytes < 16 || bytes % 16 != 0 || !aligned(buf, 16))
    return SV_EINVAL;
  const long long chunks = (long long)(bytes / 16);
  const long long span = 16032;   // one 128256-token bf16 row
  hipLaunchKernelGGL(sv::read_probe, dim3(unsigned(div_up(chunks, span))), dim3(sv::kBlock), 0,
                     stream, static_cast<const sv::u32x4*>(buf), chunks, span, sink);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}

int spec_verify_init(spec_verify_handle** out, int max_batch, int K, int V, int logits_dtype,
                     double ema_decay) {
  if (out == nullptr) return SV_EINVAL;
  *out = nullptr;
  if (logits_dtype != SV_DTYPE_F32 && logits_dtype != SV_DTYPE_BF16) return SV_EUNSUPPORTED;
  if (max_batch < 1 || K < 1 || K > 63 || V < 1) return SV_EINVAL;
  if ((long long)V * (K + 1) >= (1ll << 31)) return SV_EINVAL;
  if (!(ema_decay >= 0.0 && ema_decay <= 1.0)) return SV_EINVAL;

  spec_verify_handle* h = new (std::nothrow) spec_verify_handle();
  if (h == nullptr) return SV_ENOMEM;
  h->max_batch = max_batch;
  h->K = K;
  h->V = V;
  h->dtype = logits_dtype;
  h->decay = ema_decay;
  h->target_wgs = env_int("SPEC_VERIFY_TARGET_WGS", 2048);
  h->target_wgs_max = env_int("SPEC_VERIFY_TARGET_WGS_MAX", 6144);
  h->nseg_force = env_int("SPEC_VERIFY_NSEG", 0);
  h->trunc32_buf = env_int("SPEC_VERIFY_TRUNC32_BUF", 1);
  h->trunc32_list = env_int("SPEC_VERIFY_TRUNC32_LIST", 1);
  h->trunc32_one = env_int("SPEC_VERIFY_TRUNC32_ONE", 1);
  h->tiles_per_group = env_int("SPEC_VERIFY_TILES_PER_GROUP", 16);
  if (h->tiles_per_group < 1) h->tiles_per_group = 1;
  h->fused_min_batch = env_int("SPEC_VERIFY_FUSED_MIN_B", 0);
  h->finish_seq = env_int("SPEC_VERIFY_FINISH_SEQ", 1);
  h->claim_tiles = env_int("SPEC_VERIFY_CLAIM_TILES", 1);
  h->merge_in_finish = env_int("SPEC_VERIFY_MERGE_IN_FINISH", 1);
  if (hipGetDevice(&h->device) != hipSuccess) {
    delete h;
    return SV_EHIP;
  }
  int n_cu = 0;
  if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, h->device) ==
          hipSuccess && n_cu > 0)
    h->n_cu = n_cu;
  int lds = 0;
  if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                            h->device) == hipSuccess && lds > 0)
    h->lds_cu = lds;
  h->ntiles_max = div_up(V, sv::kTileChunks);   // scalar path has the most tiles
  const size_t n_parts = (size_t)max_batch * (2 * K + 1) * kMaxSeg;
  const size_t n_tiles = (size_t)max_batch * h->ntiles_max;
  bool ok = hipMalloc(&h->parts, n_parts * sizeof(sv::RowPart)) == hipSuccess &&
            hipMalloc(&h->draw, (size_t)max_batch * sizeof(sv::DrawRow)) == hipSuccess &&
            hipMalloc(&h->tsum, n_tiles * sizeof(sv::TileSums)) == hipSuccess &&
            hipMalloc(&h->table, (size_t)sv::kTabMax * sizeof(double)) == hipSuccess &&
            hipMalloc(&h->ema, (size_t)max_batch * sizeof(double)) == hipSuccess &&
            hipMalloc(&h->steps, (size_t)max_batch * sizeof(int32_t)) == hipSuccess &&
            hipMalloc(&h->streak, (size_t)max_batch * sizeof(int32_t)) == hipSuccess &&
            hipMalloc(&h->stats, sizeof(sv::DevStats)) == hipSuccess &&
            hipMalloc(&h->walk_seq, (size_t)max_batch * sizeof(int32_t)) == hipSuccess &&
            hipMalloc(&h->walk_cnt, 64) == hipSuccess;
  if (!ok) {
    free_all(h);
    delete h;
    return SV_ENOMEM;
  }
  hipLaunchKernelGGL(sv::fill_f64_i32, dim3(div_up(max_batch, 256)), dim3(256), 0, nullptr,
                     h->ema, h->steps, max_batch, 0.0, 0);
  hipLaunchKernelGGL(sv::fill_i32, dim3(div_up(max_batch, 256)), dim3(256), 0, nullptr, h->streak,
                     max_batch, 0);
  h->rules.pol.streak = h->streak;
  hipLaunchKernelGGL(sv::fill_u64, dim3(1), dim3(64), 0, nullptr,
                     reinterpret_cast<unsigned long long*>(h->stats),
                     int(sizeof(sv::DevStats) / 8));
  if (hipGetLastError() != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    free_all(h);
    delete h;
    return SV_EHIP;
  }
  *out = h;
  return SV_OK;
}

int spec_verify_destroy(spec_verify_handle* h) {
  if (h == nullptr) return SV_OK;
  (void)spec_verify_profile(h, 0);
  (void)hipDeviceSynchronize();
  free_all(h);
  delete h;
  return SV_OK;
}

int spec_verify_set_aux(spec_verify_handle* h, double* p_d, double* q_d, double* z,
                        int32_t* argmax) {
  if (h == nullptr) return SV_EINVAL;
  h->aux_p = p_d;
  h->aux_q = q_d;
  h->aux_z = z;
  h->aux_argmax = argmax;
  return SV_OK;
}

int spec_verify_set_stops(spec_verify_handle* h, int eos_token, const int32_t* draft_len,
                          const int32_t* max_emit) {
  if (h == nullptr || eos_token < -1) return SV_EINVAL;
  h->rules.eos = eos_token;
  h->rules.k = draft_len;
  h->rules.m = max_emit;
  return SV_OK;
}

int spec_verify_set_truncation(spec_verify_handle* h, const int32_t* top_k, const float* top_p) {
  if (h == nullptr) return SV_EINVAL;
  if (top_k != nullptr && !aligned(top_k, 4)) return fail(h, SV_EINVAL, "misaligned top_k");
  if (top_p != nullptr && !aligned(top_p, 4)) return fail(h, SV_EINVAL, "misaligned top_p");
  h->trunc.k = top_k;
  h->trunc.p = top_p;
  return SV_OK;
}

int spec_verify_set_residual(spec_verify_handle* h, int m, int32_t* out_support,
                             double* out_residual) {
  if (h == nullptr) return SV_EINVAL;
  if (out_support == nullptr) {
    h->drift_sup = nullptr;
    h->drift_res = nullptr;
    h->drift_m = 0;
    return SV_OK;
  }
  if (m < 1 || m > sv::kDriftMaxM || out_residual == nullptr)
    return fail(h, SV_EINVAL, "residual side output needs 1 <= m <= %d and both arrays",
                sv::kDriftMaxM);
  if (!aligned(out_support, 4) || !aligned(out_residual, 8))
    return fail(h, SV_EINVAL, "misaligned residual arrays");
  if (h->topm_lists == nullptr) {
    // the streaming pass's top-m lists: every (draft row, segment, wavefront)
    const size_t bytes = (size_t)h->max_batch * h->K * kMaxSeg * sv::kTopmRowSlots * 8;
    int prev = 0;
    (void)hipGetDevice(&prev);
    if (hipSetDevice(h->device) != hipSuccess)
      return fail(h, SV_EHIP, "cannot select device %d", h->device);
    const hipError_t e = hipMalloc((void**)&h->topm_lists, bytes);
    (void)hipSetDevice(prev);
    if (e != hipSuccess) {
      h->topm_lists = nullptr;
      return fail(h, SV_ENOMEM, "top-m lists (%zu bytes): %s", bytes, hipGetErrorString(e));
    }
  }
  h->drift_m = m;
  h->drift_sup = out_support;
  h->drift_res = out_residual;
  return SV_OK;
}

int spec_verify_set_walk_order(spec_verify_handle* h, int on) {
  if (h == nullptr || (on != 0 && on != 1)) return SV_EINVAL;
  h->walk = on;
  return SV_OK;
}

int spec_verify(spec_verify_handle* h, int B, const void* target, const void* draft,
                const int32_t* tokens, const float* uniforms, float temperature, int mode,
                float tau, int32_t* out_tokens, int32_t* out_len, uint32_t* out_hist,
                hipStream_t stream) {
  if (h == nullptr) return SV_EINVAL;
  h->err[0] = 0;
  h->topm_nseg = 0;
  if (B < 1 || B > h->max_batch) return fail(h, SV_EINVAL, "B=%d outside [1, %d]", B, h->max_batch);
  return verify_call(h, B, target, draft, tokens, uniforms, temperature, mode, tau, out_tokens,
                     out_len, out_hist, stream);
}

}  // extern "C"

namespace {

// The checks and launches of one verification on a handle whose workspace is
// in place (the library's own, or the static scratch array).
int verify_call(spec_verify_handle* h, int B, const void* target, const void* draft,
                const int32_t* tokens, const float* uniforms, float temperature, int mode,
                float tau, int32_t* out_tokens, int32_t* out_len, uint32_t* out_hist,
                hipStream_t stream) {
  if (target == nullptr || tokens == nullptr || out_tokens == nullptr || out_len == nullptr ||
      out_hist == nullptr)
    return fail(h, SV_EINVAL, "required pointer is NULL");
  if (mode != SV_MODE_STOCHASTIC && mode != SV_MODE_GREEDY && mode != SV_MODE_MARGIN)
    return fail(h, SV_EINVAL, "unknown mode %d", mode);
  const size_t es = h->dtype == SV_DTYPE_BF16 ? 2 : 4;
  if (mode == SV_MODE_STOCHASTIC) {
    if (draft == nullptr || uniforms == nullptr)
      return fail(h, SV_EINVAL, "stochastic mode needs draft logits and uniforms");
    if (!(std::isfinite(temperature) && temperature > 0.0f))
      return fail(h, SV_EINVAL, "temperature must be finite and > 0");
    if (!aligned(draft, es) || !aligned(uniforms, 4))
      return fail(h, SV_EINVAL, "misaligned draft logits or uniforms");
  }
  if (mode == SV_MODE_MARGIN) {
    if (!(std::isfinite(temperature) && temperature > 0.0f))
      return fail(h, SV_EINVAL, "temperature must be finite and > 0");
    if (!std::isfinite(tau)) return fail(h, SV_EINVAL, "tau must be finite");
  }
  if (!aligned(target, es) || !aligned(tokens, 4) || !aligned(out_tokens, 4) ||
      !aligned(out_len, 4) || !aligned(out_hist, 4))
    return fail(h, SV_EINVAL, "misaligned pointer");

  const bool vec = use_vec(h, target, draft, mode);

  int rc = SV_OK;
  const double c64 = kLog2e / double(temperature);
  const float c = float(c64);
  h->topm_merged = false;
  h->res_invT = 1.0 / double(temperature);
  const bool trunc = h->trunc.k != nullptr || h->trunc.p != nullptr;
  if (mode == SV_MODE_STOCHASTIC && trunc && h->dtype == SV_DTYPE_F32) {
    if (vec)
      rc = run_trunc32<4>(h, B, target, draft, tokens, uniforms, c, c64, out_tokens, out_len,
                          out_hist, stream);
    else
      rc = run_trunc32<1>(h, B, target, draft, tokens, uniforms, c, c64, out_tokens, out_len,
                          out_hist, stream);
  } else if (mode == SV_MODE_STOCHASTIC && trunc) {
    if (vec)
      rc = run_trunc<8>(h, B, target, draft, tokens, uniforms, c, c64, out_tokens, out_len,
                        out_hist, stream);
    else
      rc = run_trunc<1>(h, B, target, draft, tokens, uniforms, c, c64, out_tokens, out_len,
                        out_hist, stream);
  } else if (mode == SV_MODE_STOCHASTIC) {
    if (h->dtype == SV_DTYPE_BF16 && vec && use_fused(h, B, 8))
      rc = run_fused<sv::DT_BF16, 8, 8>(h, B, target, draft, tokens, uniforms, c, c64, out_tokens,
                                        out_len, out_hist, stream);
    else if (h->dtype == SV_DTYPE_F32 && vec && use_fused(h, B, 4))
      rc = run_fused<sv::DT_F32, 4, 8>(h, B, target, draft, tokens, uniforms, c, c64, out_tokens,
                                       out_len, out_hist, stream);
    else if (h->dtype == SV_DTYPE_BF16) {
      if (vec)
        rc = run_stochastic<sv::DT_BF16, 8, SV_U_BF16>(h, B, target, draft, tokens, uniforms, c,
                                                       c64, out_tokens, out_len, out_hist, stream);
      else
        rc = run_stochastic<sv::DT_BF16, 1, 8>(h, B, target, draft, tokens, uniforms, c, c64,
                                                out_tokens, out_len, out_hist, stream);
    } else {
      if (vec)
        rc = run_stochastic<sv::DT_F32, 4, SV_U_F32>(h, B, target, draft, tokens, uniforms, c,
                                                     c64, out_tokens, out_len, out_hist, stream);
      else
        rc = run_stochastic<sv::DT_F32, 1, 8>(h, B, target, draft, tokens, uniforms, c, c64,
                                               out_tokens, out_len, out_hist, stream);
    }
  } else {
    const bool margin = mode == SV_MODE_MARGIN;
    const double invT = margin ? 1.0 / double(temperature) : 1.0;
    const int rows = h->K + 1;
    if (h->dtype == SV_DTYPE_BF16) {
      if (vec)
        rc = run_argmax<sv::DT_BF16, 8, SV_U_MAX>(h, plan(h, B, rows, 8, SV_U_MAX, true), B, target,
                                                  tokens, margin, invT, double(tau), out_tokens,
                                                  out_len, out_hist, stream);
      else
        rc = run_argmax<sv::DT_BF16, 1, 8>(h, plan(h, B, rows, 1, 8, true), B, target, tokens, margin,
                                           invT, double(tau), out_tokens, out_len, out_hist,
                                           stream);
    } else {
      if (vec)
        rc = run_argmax<sv::DT_F32, 4, SV_U_MAX>(h, plan(h, B, rows, 4, SV_U_MAX, true), B, target,
                                                 tokens, margin, invT, double(tau), out_tokens,
                                                 out_len, out_hist, stream);
      else
        rc = run_argmax<sv::DT_F32, 1, 8>(h, plan(h, B, rows, 1, 8, true), B, target, tokens, margin,
                                          invT, double(tau), out_tokens, out_len, out_hist,
                                          stream);
    }
  }
  if (rc == SV_OK && mode == SV_MODE_STOCHASTIC && h->drift_sup != nullptr) {
    const double invT = 1.0 / double(temperature);
    if (h->dtype == SV_DTYPE_BF16)
      launch_residual<sv::DT_BF16, 8>(h, B, vec, target, draft, invT, out_len, stream);
    else
      launch_residual<sv::DT_F32, 4>(h, B, vec, target, draft, invT, out_len, stream);
    rc = check_launch(h, "drift_residual");
  }
  if (rc == SV_OK) {
    ++h->calls;
    if (h->prof_ev != nullptr && h->prof_n < h->prof_cap) {
      if (h->prof_call_end) prof_mark(h, 2, stream);
      ++h->prof_n;
    }
  }
  return rc;
}

}  // namespace

extern "C" {

int spec_verify_profile(spec_verify_handle* h, int enable) {
  if (h == nullptr) return SV_EINVAL;
  if (h->prof_ev != nullptr) {
    (void)hipDeviceSynchronize();
    for (int i = 0; i < 3 * h->prof_cap; ++i) (void)hipEventDestroy(h->prof_ev[i]);
    delete[] h->prof_ev;
    h->prof_ev = nullptr;
    h->prof_cap = h->prof_n = 0;
  }
  if (!enable) return SV_OK;
  h->prof_ev = new (std::nothrow) hipEvent_t[3 * kProfCalls];
  if (h->prof_ev == nullptr) return SV_ENOMEM;
  // timing-only events: no system-scope fence when they complete, so that
  // recording them perturbs the calls they bracket as little as possible
  for (int i = 0; i < 3 * kProfCalls; ++i) {
    if (hipEventCreateWithFlags(&h->prof_ev[i], hipEventDisableSystemFence) != hipSuccess) {
      for (int k = 0; k < i; ++k) (void)hipEventDestroy(h->prof_ev[k]);
      delete[] h->prof_ev;
      h->prof_ev = nullptr;
      return fail(h, SV_EHIP, "hipEventCreate failed");
    }
  }
  h->prof_cap = kProfCalls;
  h->prof_n = 0;
  h->prof_call_end = (enable & 2) != 0;
  return SV_OK;
}

int spec_verify_profile_read(spec_verify_handle* h, double* stream_pass_ms, double* call_ms,
                             int* n_calls) {
  if (h == nullptr || h->prof_ev == nullptr) return SV_EINVAL;
  double a = 0.0, b = 0.0;
  for (int i = 0; i < h->prof_n; ++i) {
    float t1 = 0.f, t2 = 0.f;
    const int last = h->prof_call_end ? 2 : 1;
    if (hipEventSynchronize(h->prof_ev[3 * i + last]) != hipSuccess ||
        hipEventElapsedTime(&t1, h->prof_ev[3 * i], h->prof_ev[3 * i + 1]) != hipSuccess ||
        (h->prof_call_end &&
         hipEventElapsedTime(&t2, h->prof_ev[3 * i], h->prof_ev[3 * i + 2]) != hipSuccess))
      return fail(h, SV_EHIP, "event timing failed");
    a += t1;
    b += t2;
  }
  if (stream_pass_ms != nullptr) *stream_pass_ms = a;
  if (call_ms != nullptr) *call_ms = b;
  if (n_calls != nullptr) *n_calls = h->prof_n;
  h->prof_n = 0;
  return SV_OK;
}

int spec_verify_get_ema(spec_verify_handle* h, double* ema_dev, int32_t* steps_dev,
                        hipStream_t stream) {
  if (h == nullptr) return SV_EINVAL;
  if (ema_dev != nullptr &&
      hipMemcpyAsync(ema_dev, h->ema, (size_t)h->max_batch * sizeof(double),
                     hipMemcpyDeviceToDevice, stream) != hipSuccess)
    return fail(h, SV_EHIP, "get_ema copy failed");
  if (steps_dev != nullptr &&
      hipMemcpyAsync(steps_dev, h->steps, (size_t)h->max_batch * sizeof(int32_t),
                     hipMemcpyDeviceToDevice, stream) != hipSuccess)
    return fail(h, SV_EHIP, "get_ema copy failed");
  return SV_OK;
}

int spec_verify_set_ema(spec_verify_handle* h, const double* ema_dev, const int32_t* steps_dev,
                        hipStream_t stream) {
  if (h == nullptr || ema_dev == nullptr || steps_dev == nullptr) return SV_EINVAL;
  if (hipMemcpyAsync(h->ema, ema_dev, (size_t)h->max_batch * sizeof(double),
                     hipMemcpyDeviceToDevice, stream) != hipSuccess ||
      hipMemcpyAsync(h->steps, steps_dev, (size_t)h->max_batch * sizeof(int32_t),
                     hipMemcpyDeviceToDevice, stream) != hipSuccess)
    return fail(h, SV_EHIP, "set_ema copy failed");
  return SV_OK;
}

int spec_verify_reset_ema(spec_verify_handle* h, hipStream_t stream) {
  if (h == nullptr) return SV_EINVAL;
  hipLaunchKernelGGL(sv::fill_f64_i32, dim3(div_up(h->max_batch, 256)), dim3(256), 0, stream,
                     h->ema, h->steps, h->max_batch, 0.0, 0);
  hipLaunchKernelGGL(sv::fill_i32, dim3(div_up(h->max_batch, 256)), dim3(256), 0, stream,
                     h->streak, h->max_batch, 0);
  return check_launch(h, "reset_ema");
}

int spec_verify_set_policy(spec_verify_handle* h, const float* draft_conf, double d,
                           int32_t* out_shape, double* out_dcs) {
  if (h == nullptr) return SV_EINVAL;
  if (draft_conf == nullptr) {
    h->rules.pol.conf = nullptr;
    h->rules.pol.shape = nullptr;
    h->rules.pol.dcs = nullptr;
    return SV_OK;
  }
  if (out_shape == nullptr || !(std::isfinite(d) && d > 0.0))
    return fail(h, SV_EINVAL, "policy needs out_shape and a finite divisor d > 0");
  if (!aligned(draft_conf, 4) || !aligned(out_shape, 4) || !aligned(out_dcs, 8))
    return fail(h, SV_EINVAL, "misaligned policy array");
  h->rules.pol.conf = draft_conf;
  h->rules.pol.shape = out_shape;
  h->rules.pol.dcs = out_dcs;
  h->rules.pol.d = d;
  return SV_OK;
}

int spec_verify_get_stats(spec_verify_handle* h, spec_verify_stats* out, int reset,
                          hipStream_t stream) {
  if (h == nullptr || out == nullptr) return SV_EINVAL;
  sv::DevStats d;
  if (hipMemcpyAsync(&d, h->stats, sizeof(d), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return fail(h, SV_EHIP, "get_stats copy failed");
  out->sequences = d.sequences;
  out->invalid = d.invalid;
  out->zero_q_accepts = d.zero_q_accepts;
  out->z0_fallbacks = d.z0_fallbacks;
  out->calls = h->calls;
  if (reset) {
    hipLaunchKernelGGL(sv::fill_u64, dim3(1), dim3(64), 0, stream,
                       reinterpret_cast<unsigned long long*>(h->stats),
                       int(sizeof(sv::DevStats) / 8));
    h->calls = 0;
    return check_launch(h, "reset_stats");
  }
  return SV_OK;
}

const char* spec_verify_last_error(const spec_verify_handle* h) {
  if (h == nullptr) return g_noalloc_err[0] != 0 ? g_noalloc_err : "null handle";
  return h->err;
}

}  // extern "C"

// --------------------------------------------------------------------------
// Allocation-free entry point: one verification with no handle, its
// workspace in a fixed device array of this library (one copy per GPU).
// --------------------------------------------------------------------------

namespace {

constexpr size_t kScratchBytes = size_t(1) << 20;    // per GPU, held until the process ends
constexpr size_t kScratchAlign = 256;
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

struct ScratchDev {
  std::once_flag once;
  void* ptr = nullptr;            // device address of `scratch` on this GPU
  hipError_t err = hipSuccess;
  int n_cu = 256;
};
ScratchDev g_scratch[kMaxDevices];

// Once per device, with that device current: the device address of this
// GPU's copy of the array (the host-side name is only a stand-in for it).
void scratch_setup(ScratchDev& d, int dev) {
  void* p = nullptr;
  d.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  d.ptr = d.err == hipSuccess ? p : nullptr;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      n > 0)
    d.n_cu = n;
}

int noalloc_fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_noalloc_err, sizeof(g_noalloc_err), fmt, ap);
  va_end(ap);
  return code;
}

size_t align_up(size_t x) { return (x + kScratchAlign - 1) / kScratchAlign * kScratchAlign; }

}  // namespace

extern "C" {

int spec_verify_noalloc(int B, int K, int V, int logits_dtype, const void* target,
                        const void* draft, const int32_t* tokens, const float* uniforms,
                        float temperature, int mode, float tau, int32_t* out_tokens,
                        int32_t* out_len, uint32_t* out_hist, hipStream_t stream) {
  g_noalloc_err[0] = 0;
  if (logits_dtype != SV_DTYPE_F32 && logits_dtype != SV_DTYPE_BF16)
    return noalloc_fail(SV_EUNSUPPORTED, "unknown logit dtype %d", logits_dtype);
  if (B < 1 || K < 1 || K > 63 || V < 1 || (long long)V * (K + 1) >= (1ll << 31))
    return noalloc_fail(SV_EINVAL, "sizes B=%d K=%d V=%d outside the supported range", B, K, V);
  if (mode != SV_MODE_STOCHASTIC && mode != SV_MODE_GREEDY && mode != SV_MODE_MARGIN)
    return noalloc_fail(SV_EINVAL, "unknown mode %d", mode);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return noalloc_fail(SV_EHIP, "no usable current device");
  ScratchDev& sd = g_scratch[dev];
  std::call_once(sd.once, scratch_setup, std::ref(sd), dev);
  if (sd.ptr == nullptr)
    return noalloc_fail(SV_EHIP, "scratch address: %s", hipGetErrorString(sd.err));

  // a handle on the stack (host memory) whose workspace pointers lie in the
  // scratch array; the routes that need more workspace are refused
  spec_verify_handle h;
  h.device = dev;
  h.max_batch = B;
  h.K = K;
  h.V = V;
  h.dtype = logits_dtype;
  h.n_cu = sd.n_cu;
  const bool vec = use_vec(&h, target, draft, mode);
  const bool stoch = mode == SV_MODE_STOCHASTIC;
  const int rows = stoch ? 2 * K + 1 : K + 1;
  const int v = vec ? (logits_dtype == SV_DTYPE_BF16 ? 8 : 4) : 1;
  int U = 8;
  if (vec) U = !stoch ? SV_U_MAX : logits_dtype == SV_DTYPE_BF16 ? SV_U_BF16 : SV_U_F32;
  const Launch L = plan(&h, B, rows, v, U, !stoch);
  if (stoch && (L.ntiles > sv::kFMaxTiles || rows > sv::kFMaxRows))
    return noalloc_fail(SV_EUNSUPPORTED,
                        "stochastic calls without allocation need V <= %d for this layout",
                        sv::kFMaxTiles * sv::kTileChunks * v);
  const size_t off_ema = align_up(sizeof(sv::DevStats));
  const size_t off_steps = align_up(off_ema + (size_t)B * sizeof(double));
  const size_t off_parts = align_up(off_steps + (size_t)B * sizeof(int32_t));
  const size_t need = off_parts + (size_t)B * rows * L.nseg * sizeof(sv::RowPart);
  if (need > kScratchBytes)
    return noalloc_fail(SV_EINVAL,
                        "B=%d K=%d V=%d needs %zu bytes of scratch; the limit is %zu", B, K, V,
                        need, kScratchBytes);
  unsigned char* base = static_cast<unsigned char*>(sd.ptr);
  h.stats = reinterpret_cast<sv::DevStats*>(base);
  h.ema = reinterpret_cast<double*>(base + off_ema);
  h.steps = reinterpret_cast<int32_t*>(base + off_steps);
  h.parts = reinterpret_cast<sv::RowPart*>(base + off_parts);
  // counters and the per-call EMA start from zero (fill kernels: no memset
  // nodes when the call is captured into a graph)
  hipLaunchKernelGGL(sv::fill_u64, dim3(1), dim3(64), 0, stream,
                     reinterpret_cast<unsigned long long*>(h.stats),
                     int(sizeof(sv::DevStats) / 8));
  hipLaunchKernelGGL(sv::fill_f64_i32, dim3(div_up(B, 256)), dim3(256), 0, stream, h.ema,
                     h.steps, B, 0.0, 0);
  int rc = check_launch(&h, "scratch clear");
  if (rc == SV_OK)
    rc = verify_call(&h, B, target, draft, tokens, uniforms, temperature, mode, tau, out_tokens,
                     out_len, out_hist, stream);
  if (rc != SV_OK) {
    snprintf(g_noalloc_err, sizeof(g_noalloc_err), "%s", h.err);
    return rc;
  }
  return SV_OK;
}

}  // extern "C"
