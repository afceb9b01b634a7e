// Draft residual side output over bf16 logit rows (gfx950).
//
// At every drafted position the target's distribution is known as well as
// the draft's; restricted to a shared top-m support, the target
// log-probability minus the draft log-probability is the residual a draft
// recalibration memory learns from ([DRIFT] "The update rule and its
// objective"). The support is the draft's top m tokens (ties to the lower
// index), listed by descending draft logit, and both temperature softmaxes are
// renormalised on it:
//   r(v) = (x_t(v) - x_d(v)) / T - LSE_S(x_t / T) + LSE_S(x_d / T).
//
// The support comes from the top-m candidate lists of sv_topm.hpp, by one of
// two routes:
//   - inside the streaming pass (rowstats_sum with its top-m lists on), whose
//     draft-row workgroups keep a list per wavefront while they stream the
//     row and store each list's keys; drift_merge then takes, per drafted
//     position, the m largest keys of that row's lists;
//   - drift_residual, one 256-thread workgroup per drafted position that
//     reads the draft row once, for calls whose rows are read by another pass
//     (truncation, one kernel per sequence) or are not in 16-byte chunks.
// Logits are bf16 or fp32 (DT).
// Only valid sequences (the scan's accept length is read to tell) and drafted
// positions i < k_b get a support; both routes end in support_residual.
#pragma once

#include "sv_kernels.hpp"

namespace sv {

constexpr int kDriftMaxM = 64;
constexpr int kDriftBlock = 256;
constexpr int kDriftWaves = kDriftBlock / kWave;
constexpr int kDriftCap = 448;       // keys per wavefront list (drift_residual)
constexpr int kDriftUnroll = 4;      // chunks per thread per group (two groups in flight)
constexpr int kTopmMaxSeg = 16;      // streaming-pass segments per row, at most
constexpr int kTopmListSlots = kDriftMaxM;            // stored keys per wavefront list
constexpr int kTopmRowSlots = kWavesPerBlock * kTopmListSlots;   // per (row, segment)
constexpr int kMergeCap = kTopmMaxSeg * kTopmRowSlots;           // keys per drafted position

// no support here: -1 and NaN in the m slots (whole workgroup, uniform)
__device__ inline void no_support(int m, int32_t* out_support, double* out_res) {
  if (int(threadIdx.x) < m) {
    out_support[threadIdx.x] = -1;
    out_res[threadIdx.x] = __builtin_nan("");
  }
}

template <int DT, int VEC>
__global__ __launch_bounds__(kDriftBlock) void drift_residual(
    const void* __restrict__ target, const void* __restrict__ draft, int K, int V, double invT,
    int m, const int32_t* __restrict__ kdraft, const int32_t* __restrict__ accept_len,
    int32_t* __restrict__ out_support, double* __restrict__ out_res) {
  using C = Chunk<DT, VEC>;
  using raw_t = typename C::raw_t;
  constexpr bool kVector = VEC > 1;         // 16-byte chunks (8 bf16 or 4 fp32)
  __shared__ uint64_t s_keys[kDriftWaves][kDriftCap];
  __shared__ uint32_t s_bins[kDriftWaves][256];
  __shared__ u32x4 s_stage[kDriftWaves][kVector ? kTopmStage : 1];
  __shared__ uint32_t s_stage_at[kDriftWaves][kVector ? kTopmStage : 1];
  __shared__ uint32_t s_count[kDriftWaves];
  __shared__ unsigned long long s_thr;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int b = int(blockIdx.x) / K, i = int(blockIdx.x) % K;
  const long long o0 = ((long long)b * K + i) * m;
  const int kb = kdraft != nullptr ? kdraft[b] : K;
  if (accept_len[b] < 0 || i >= kb) return no_support(m, out_support + o0, out_res + o0);
  const void* drow = row_ptr<DT>(target, draft, b, K + 1 + i, K, V);
  const void* trow = row_ptr<DT>(target, draft, b, i, K, V);
  const uint32_t mm = uint32_t(min(m, V));
  if (tid == 0) s_thr = 0ull;
  __syncthreads();
  TopM<DT> tm;
  tm.init(s_keys[wid], s_bins[wid], &s_thr, kDriftCap, mm, s_stage[wid], s_stage_at[wid]);

  // ---- one read of the draft row; one group's loads are in flight while
  // the other is filtered (indexes past the row are clamped to its last
  // chunk and filter nothing) ----
  const long long nchunks = V / VEC;
  constexpr long long kPerIt = (long long)kDriftBlock * kDriftUnroll;
  const long long nit = (nchunks + kPerIt - 1) / kPerIt;
  auto load_group = [&](long long it, raw_t (&raw)[kDriftUnroll]) {
#pragma unroll
    for (int u = 0; u < kDriftUnroll; ++u) {
      const long long ci = (it * kDriftUnroll + u) * kDriftBlock + tid;
      raw[u] = C::load(drow, ci < nchunks ? ci : nchunks - 1);
    }
  };
  auto filter_group = [&](long long it, const raw_t (&raw)[kDriftUnroll]) {
    if constexpr (kVector) {
      const long long c0 = it * kDriftUnroll * kDriftBlock + tid;
      float cm[kDriftUnroll];
      uint32_t ok = 0;
#pragma unroll
      for (int u = 0; u < kDriftUnroll; ++u) {
        cm[u] = chunk_max<DT>(raw[u]);
        ok |= c0 + (long long)u * kDriftBlock < nchunks ? 1u << u : 0u;
      }
      if (it == 0) tm.template seed<kDriftUnroll>(cm, ok);   // start the threshold
#pragma unroll
      for (int u = 0; u < kDriftUnroll; ++u) {
        const long long cu = c0 + (long long)u * kDriftBlock;
        tm.stage_chunk(((ok >> u) & 1u) != 0u && cm[u] >= tm.thr_f, raw[u], uint32_t(cu));
      }
    } else {
#pragma unroll
      for (int u = 0; u < kDriftUnroll; ++u) {
        const long long ci = (it * kDriftUnroll + u) * kDriftBlock + tid;
        // one value per chunk: its bits in raw[u]
        const float x = __uint_as_float(DT == DT_BF16 ? raw[u] << 16 : raw[u]);
        const uint32_t pend = ci < nchunks && x >= tm.thr_f ? 1u : 0u;
        if (__ballot(pend != 0u) == 0ull) continue;   // uniform: the common case
        tm.offer(pend, [&](int) -> uint32_t { return raw[u]; }, ci);
      }
    }
  };
  {
    // two register sets in turn; loads are unconditional, so the compiler's
    // wait counts stay exact
    raw_t ga[kDriftUnroll], gb[kDriftUnroll];
    load_group(0, ga);
#pragma unroll 1
    for (long long it = 0; it < nit; it += 2) {
      load_group(it + 1, gb);
      filter_group(it, ga);
      load_group(it + 2, ga);
      filter_group(it + 1, gb);
    }
  }
  if constexpr (kVector) tm.flush();
  tm.compact();                                 // at most mm keys per wavefront
  if (lane == 0) s_count[wid] = tm.fill;
  __syncthreads();

  // ---- merge, keep the mm largest keys, residuals on wavefront 0 ----
  if (wid != 0) return;
  uint32_t n = tm.fill;
#pragma unroll
  for (int w = 1; w < kDriftWaves; ++w) {
    const uint32_t cw = s_count[w];
    for (uint32_t e = uint32_t(lane); e < cw; e += kWave) s_keys[0][n + e] = s_keys[w][e];
    n += cw;
  }
  wave_sync();
  tm.fill = n;
  tm.compact();                                 // exactly mm keys remain
  support_residual<DT>(s_keys[0], mm, drow, trow, invT, m, out_support + o0, out_res + o0);
}

// One wavefront: drafted position (b, i)'s support and residuals from the
// lists the streaming pass stored for its draft row (nseg segments x 4
// wavefronts, mm = min(m, V) slots each, empty slots 0): the m largest keys,
// ranked, then the two log-sum-exps. keys: LDS for nseg * 4 * mm keys;
// bins: 256 words of LDS; thr: one LDS word (all this wavefront's).
template <int DT>
__device__ __forceinline__ void merge_position(const void* __restrict__ target,
                                      const void* __restrict__ draft, int K, int V, double invT,
                                      int m, int nseg, const uint64_t* __restrict__ lists, int b,
                                      int i, uint64_t* keys, uint32_t* bins,
                                      unsigned long long* thr, int32_t* __restrict__ out_support,
                                      double* __restrict__ out_res) {
  const int lane = threadIdx.x & (kWave - 1);
  const long long o0 = ((long long)b * K + i) * m;
  const uint32_t mm = uint32_t(min(m, V));
  const uint64_t* L = lists + ((long long)b * K + i) * nseg * kTopmRowSlots;
  // slot e of the nseg * 4 lists of mm slots: list e / mm, slot e % mm; eight
  // loads per lane are issued before any is used
  const uint32_t n_slots = uint32_t(nseg * kWavesPerBlock) * mm;
  uint32_t fill = 0;
  for (uint32_t base = 0; base < n_slots; base += 8u * kWave) {
    uint64_t k[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t e = base + uint32_t(q * kWave + lane);
      k[q] = e < n_slots ? L[(e / mm) * kTopmListSlots + e % mm] : 0ull;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const bool put = k[q] != 0ull;                   // keys are never 0
      const uint64_t mask = __ballot(put);
      if (put) keys[fill + lanes_below(mask)] = k[q];
      fill += uint32_t(__popcll(mask));
    }
  }
  if (lane == 0) *thr = 0ull;
  wave_sync();
  TopM<DT> tm;
  tm.init(keys, bins, thr, n_slots, mm);
  tm.fill = fill;
  tm.compact();                                 // exactly mm keys remain
  support_residual<DT>(keys, mm, row_ptr<DT>(target, draft, b, K + 1 + i, K, V),
                       row_ptr<DT>(target, draft, b, i, K, V), invT, m, out_support + o0,
                       out_res + o0);
}

// The residual merge run inside the per-sequence finish: its wavefront 1 + i
// takes drafted position i (needs K < waves per workgroup) while wavefront 0
// runs the acceptance scan. lds: per position, nseg * 4 * min(m, V) keys,
// then 256 bin words (128 u64) and the threshold word, from lds.
struct MergeJob {
  const uint64_t* lists = nullptr;     // null: no merge in the finish
  int nseg = 0, m = 0;
  double invT = 1.0;
  int32_t* sup = nullptr;
  double* res = nullptr;
};

__host__ __device__ inline int merge_lds_words(int nseg, int m, int V) {
  return nseg * kWavesPerBlock * (m < V ? m : V) + 128 + 1;
}

// Position i of sequence b after the finish's partials are combined: the
// call's validity taken as the scan takes it (stopping rules, finite
// normalisers of rows 0..k_b and K+1..K+k_b, drafted tokens in [0, V)), then
// no support (invalid call, or i >= k_b) or merge_position.
template <int DT>
__device__ __forceinline__ void merge_in_finish(const MergeJob& mj, uint64_t* lds,
                                                const Rules& sp, int b, int i, int K, int V,
                                                const void* __restrict__ target,
                                                const void* __restrict__ draft, const double* fS,
                                                const int32_t* tok) {
  const int lane = threadIdx.x & (kWave - 1);
  int kb, me;
  bool lane_bad;
  stops_of(sp, b, K, kb, me, lane_bad);
  if (lane <= kb) lane_bad |= !finite_pos(fS[lane]);
  if (lane < kb) {
    lane_bad |= !finite_pos(fS[K + 1 + lane]);
    const int d = tok[lane];
    lane_bad |= !(d >= 0 && d < V);
  }
  const long long o0 = ((long long)b * K + i) * mj.m;
  if (__any(lane_bad) || i >= kb) {
    if (lane < mj.m) {
      mj.sup[o0 + lane] = -1;
      mj.res[o0 + lane] = __builtin_nan("");
    }
    return;
  }
  uint64_t* keys = lds + (long long)i * merge_lds_words(mj.nseg, mj.m, V);
  const int nk = mj.nseg * kWavesPerBlock * min(mj.m, V);
  merge_position<DT>(target, draft, K, V, mj.invT, mj.m, mj.nseg, mj.lists, b, i, keys,
                     reinterpret_cast<uint32_t*>(keys + nk),
                     reinterpret_cast<unsigned long long*>(keys + nk + 128), mj.sup, mj.res);
}

// Per drafted position: merge_position on one wavefront after the call's
// outcome (accept_len < 0, or a position past k_b: no support); dynamic LDS
// of nseg * 4 * min(m, V) keys.
template <int DT>
__global__ __launch_bounds__(kWave) void drift_merge(
    const void* __restrict__ target, const void* __restrict__ draft, int K, int V, double invT,
    int m, int nseg, const uint64_t* __restrict__ lists, const int32_t* __restrict__ kdraft,
    const int32_t* __restrict__ accept_len, int32_t* __restrict__ out_support,
    double* __restrict__ out_res) {
  extern __shared__ uint64_t s_keys[];
  __shared__ uint32_t s_bins[256];
  __shared__ unsigned long long s_thr;
  const int b = int(blockIdx.x) / K, i = int(blockIdx.x) % K;
  const long long o0 = ((long long)b * K + i) * m;
  const int kb = kdraft != nullptr ? kdraft[b] : K;
  if (accept_len[b] < 0 || i >= kb) return no_support(m, out_support + o0, out_res + o0);
  merge_position<DT>(target, draft, K, V, invT, m, nseg, lists, b, i, s_keys, s_bins, &s_thr,
                     out_support, out_res);
}

}  // namespace sv
