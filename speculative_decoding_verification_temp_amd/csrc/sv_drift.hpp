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
  __shared__ uint32_t s_wg[8];
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
  // with a whole first group, every wavefront's threshold starts from the
  // workgroup's 256 thread maxima of that group (their m-th largest is at
  // most the row's m-th largest value): far fewer candidates than from one
  // wavefront's chunk maxima
  const bool wg_seed = kVector && nchunks >= kPerIt;
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
      if (it == 0 && wg_seed) {        // uniform: every thread is here
        float gm = cm[0];
#pragma unroll
        for (int u = 1; u < kDriftUnroll; ++u) gm = fmaxf(gm, cm[u]);
        const uint32_t gbits = __float_as_uint(gm);
        uint32_t key = DT == DT_BF16 ? bf16_key(gbits >> 16) : order_key<DT_F32>(gbits);
        if (!(gm == gm)) key = 0u;    // (a NaN counts as nothing)
        const uint32_t t =
            wg_kth_top16<DT == DT_BF16 ? 16 : 32>(key, tm.want, &s_bins[0][0], s_wg);
        tm.thr = uint64_t(t) << 32;
        tm.thr_f = order_floor<DT>(t);
        if (tid == 0) atomicMax(&s_thr, (unsigned long long)tm.thr);
      } else if (it == 0) {
        tm.template seed<kDriftUnroll>(cm, ok);   // start the threshold
      }
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
// takes drafted position i (needs K < waves per workgroup) once its share of
// the draw's tiles is read, with at most 64 kMergeHeld keys per position
// (nseg * 4 * min(m, V) list slots), so that every key stays in a register
// of one lane: load the lists (merge_load), rank every key by counting the
// larger ones, gather the target logits at the m selected tokens only, and
// write the residuals (merge_in_finish).
constexpr int kMergeHeld = 4;
struct MergeJob {
  const uint64_t* lists = nullptr;     // null: no merge in the finish
  int nseg = 0, m = 0;
  double invT = 1.0;
  int32_t* sup = nullptr;
  double* res = nullptr;
};

// LDS words per merged position (one slot per list slot, rounded up to a
// whole number of wavefront rows)
__host__ __device__ inline int merge_lds_words() { return kWave * kMergeHeld; }
__host__ __device__ inline bool merge_fits(int nseg, int m, int V) {
  return nseg * kWavesPerBlock * (m < V ? m : V) <= kWave * kMergeHeld;
}

// A lane's list slots p * 64 + lane (key 0: empty).
struct MergeHeld {
  uint64_t key[kMergeHeld];
};

// Slot e of the nseg * 4 lists of mm slots (list e / mm, slot e % mm) into
// keys[e] (LDS, read by the whole wavefront next) and this lane's slots into
// h. The lists of positions this call's streaming pass skipped (past k_b, or
// an invalid k_b) hold earlier calls' keys, or nothing written yet; they are
// loaded all the same and never used.
template <int DT>
__device__ __forceinline__ void merge_load(const MergeJob& mj, uint64_t* keys, int b, int i,
                                           int K, int V, MergeHeld& h) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t mm = uint32_t(min(mj.m, V));
  const uint32_t n_slots = uint32_t(mj.nseg * kWavesPerBlock) * mm;
  const uint64_t* L = mj.lists + ((long long)b * K + i) * mj.nseg * kTopmRowSlots;
#pragma unroll
  for (int p = 0; p < kMergeHeld; ++p) {
    const uint32_t e = uint32_t(p * kWave + lane);
    h.key[p] = e < n_slots ? L[(e / mm) * kTopmListSlots + e % mm] : 0ull;
  }
#pragma unroll
  for (int p = 0; p < kMergeHeld; ++p) keys[p * kWave + lane] = h.key[p];
}

// ranks of the held keys among keys[0..n) (the number of larger keys; keys
// are distinct, 0 is never counted)
template <int Q>
__device__ __forceinline__ void merge_count(const uint64_t* keys, uint32_t n, const MergeHeld& h,
                                            uint32_t (&rank)[kMergeHeld]) {
#pragma unroll 8
  for (uint32_t e = 0; e < n; ++e) {
    const uint64_t k = keys[e];
#pragma unroll
    for (int p = 0; p < Q; ++p) rank[p] += k > h.key[p] ? 1u : 0u;
  }
}

// After merge_load and a wavefront sync, with the finish's partials
// combined: the call's validity taken as the scan takes it (stopping rules, finite normalisers of
// rows 0..k_b and K+1..K+k_b, drafted tokens in [0, V)); then no support
// (invalid call, or i >= k_b), or the min(m, V) largest held keys, each
// written at its rank with
//   (x_t(v)/T - LSE_S(x_t/T)) - (x_d(v)/T - LSE_S(x_d/T)),
// slots min(m, V)..m-1 -1 and NaN.
template <int DT>
__device__ __forceinline__ void merge_in_finish(const MergeJob& mj, const uint64_t* keys,
                                                const MergeHeld& h, const Rules& sp, int b,
                                                int i, int K, int V,
                                                const void* __restrict__ target,
                                                const double* fS, const int32_t* tok) {
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
  const uint32_t mm = uint32_t(min(mj.m, V));
  if (__any(lane_bad) || i >= kb) {
    if (lane < mj.m) {
      mj.sup[o0 + lane] = -1;
      mj.res[o0 + lane] = __builtin_nan("");
    }
    return;
  }
  const uint32_t n_slots = uint32_t(mj.nseg * kWavesPerBlock) * mm;
  uint32_t rank[kMergeHeld] = {};
  if (n_slots <= 2u * kWave) merge_count<2>(keys, n_slots, h, rank);
  else merge_count<kMergeHeld>(keys, n_slots, h, rank);
  // the target logit gathered at the selected tokens only (each read takes
  // a whole cache line); the draft logit is the value its key encodes (the
  // keys of -0 and +0 agree, and the residual does not tell them apart)
  const void* trow = row_ptr<DT>(target, nullptr, b, i, K, V);
  bool sel[kMergeHeld];
  float xt[kMergeHeld];
#pragma unroll
  for (int p = 0; p < kMergeHeld; ++p) {
    sel[p] = h.key[p] != 0ull && rank[p] < mm;
    xt[p] = sel[p] ? load_logit<DT>(trow, int(~uint32_t(h.key[p]))) : 0.0f;
  }
  double at[kMergeHeld], ad[kMergeHeld];
  double mt = -__builtin_inf(), md = -__builtin_inf();
#pragma unroll
  for (int p = 0; p < kMergeHeld; ++p) {
    const float xd = order_floor<DT>(uint32_t(h.key[p] >> 32));
    at[p] = sel[p] ? double(xt[p]) * mj.invT : -__builtin_inf();
    ad[p] = sel[p] ? double(xd) * mj.invT : -__builtin_inf();
    mt = fmax(mt, at[p]);
    md = fmax(md, ad[p]);
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    mt = fmax(mt, __shfl_xor(mt, o, kWave));
    md = fmax(md, __shfl_xor(md, o, kWave));
  }
  double et = 0.0, ed = 0.0;
#pragma unroll
  for (int p = 0; p < kMergeHeld; ++p) {
    et += sel[p] ? exp(at[p] - mt) : 0.0;
    ed += sel[p] ? exp(ad[p] - md) : 0.0;
  }
  const double lse_t = mt + log(wave_sum(et));
  const double lse_d = md + log(wave_sum(ed));
#pragma unroll
  for (int p = 0; p < kMergeHeld; ++p) {
    if (sel[p]) {
      mj.sup[o0 + rank[p]] = int32_t(~uint32_t(h.key[p]));
      mj.res[o0 + rank[p]] = (at[p] - lse_t) - (ad[p] - lse_d);
    }
  }
  if (uint32_t(lane) >= mm && lane < mj.m) {
    mj.sup[o0 + lane] = -1;
    mj.res[o0 + lane] = __builtin_nan("");
  }
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
