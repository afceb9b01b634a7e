// Streaming passes over the logit rows (gfx950).
//
//   rowstats_sum   every (row, segment) of the target and draft logits:
//                  running sum of softmax terms relative to an integer
//                  reference exponent (stochastic mode).
//   rowstats_max   every (row, segment) of the target logits: max,
//                  lowest-index argmax and a NaN flag (greedy and margin).
//
// Both keep their per-segment partials in a fixed order; reruns are bitwise
// identical.
#pragma once

#include "sv_device.hpp"
#include "sv_topm.hpp"

namespace sv {

// --------------------------------------------------------------------------
// Row addressing. Stochastic rows of sequence b: r = 0..K are target rows,
// r = K+1..2K are draft rows 0..K-1. Greedy/margin rows: r = 0..K target.
// --------------------------------------------------------------------------
template <int DT>
__device__ inline const void* row_ptr(const void* target, const void* draft, int b, int r,
                                      int K, int V) {
  constexpr int s = elem_bytes<DT>();
  if (r <= K)
    return static_cast<const char*>(target) + ((long long)b * (K + 1) + r) * (long long)V * s;
  return static_cast<const char*>(draft) + ((long long)b * K + (r - K - 1)) * (long long)V * s;
}

// --------------------------------------------------------------------------
// Streaming softmax normaliser. Each lane keeps a float64 sum S of
// 2^(x*c - R) with an integer reference R >= max(x)*c; when a new chunk group
// raises the maximum, S is rescaled by an exact power of two. Within a group
// the terms are added pairwise in fp32 and the group total is added to S in
// fp64.
// --------------------------------------------------------------------------
//
// With TOPM (16-byte chunks only), the workgroups of draft rows also keep a
// Where the sum from the top over bins[0..256) (thread t holds bin t) first
// reaches goal: the highest t whose sum over the bins >= t is >= goal, and in
// above the sum over the bins > t. Needs all kBlock threads; sw: 8 words of
// LDS. (The first sum, over all bins, must reach goal.)
__device__ inline void wg_suffix_cut(const uint32_t* bins, uint32_t goal, uint32_t* sw,
                                     uint32_t& cut, uint32_t& above) {
  static_assert(kBlock == 256 && kWavesPerBlock == 4, "one bin per thread");
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const uint32_t c = bins[tid];
  uint32_t v = c;                      // sum over this wavefront's lanes >= lane
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t u = __shfl_down(v, o, kWave);
    if (lane + o < kWave) v += u;
  }
  if (lane == 0) sw[wid] = v;
  __syncthreads();
  uint32_t add = 0u;
#pragma unroll
  for (int w = 0; w < kWavesPerBlock; ++w) add += w > wid ? sw[w] : 0u;
  const uint32_t suf = v + add;        // non-increasing in tid
  const uint32_t n = uint32_t(__popcll(__ballot(suf >= goal)));
  __syncthreads();                     // sw read before it is written again
  if (lane == 0) sw[wid] = n;
  __syncthreads();
  uint32_t t = 0u;
#pragma unroll
  for (int w = 0; w < kWavesPerBlock; ++w) t += sw[w];
  cut = t - 1u;
  if (uint32_t(tid) == cut) sw[4] = suf - c;
  __syncthreads();
  above = sw[4];
  __syncthreads();
}

// A lower bound of the m-th largest (1 <= m <= 256) of the kBits-bit keys
// held one per thread of the workgroup: that key's top 16 bits, lower bits 0,
// from two rounds of 256 bins (the top byte, then the next byte among the
// keys in the chosen top-byte bin). Needs all kBlock threads; bins: 512
// words of LDS, sw: 8.
template <int kBits>
__device__ inline uint32_t wg_kth_top16(uint32_t key, uint32_t m, uint32_t* bins, uint32_t* sw) {
  constexpr int s1 = kBits - 8, s2 = kBits - 16;
  const int tid = threadIdx.x;
  bins[tid] = 0u;
  bins[kBlock + tid] = 0u;
  __syncthreads();
  atomicAdd(&bins[key >> s1], 1u);
  __syncthreads();
  uint32_t b1, above1, b2, above2;
  wg_suffix_cut(bins, m, sw, b1, above1);
  if ((key >> s1) == b1) atomicAdd(&bins[kBlock + ((key >> s2) & 255u)], 1u);
  __syncthreads();
  wg_suffix_cut(bins + kBlock, m - above1, sw, b2, above2);
  return (b1 << s1) | (b2 << s2);
}

// The rows one launch of the stochastic streaming pass covers in every
// sequence: target rows t0..t1-1 and draft rows d0..d1-1 (all of them:
// 0..K+1, 0..K). gate > 0 (walk-order reading): a workgroup streams its row
// only when the walk reaches position gate, i.e. positions 0..gate-1, whose
// rows earlier launches streamed, are all kept (acceptance tested exactly as
// the scans test it, from the same partials). The library's walk-order
// reading streams position 0 this way and the rest through a list of the
// sequences whose walk goes on (walk_gate, rowstats_sum_list).
struct StageRows {
  int t0, t1, d0, d1, gate;
  uint32_t* clear;   // set to 0 by workgroup 0 (the next stage's list count), or null
};

// Rows of a pass that takes them one after another (the truncation passes):
// target rows t0..t1-1 and draft rows d0..d1-1 of every sequence, or of the
// listed sequences seqs[0 .. *count) when seqs is set. Candidate it in
// 0 .. total(B) - 1 is row at(it) of sequence it / per_seq().
struct RowSel {
  int t0, t1, d0, d1;
  const int32_t* seqs;
  const uint32_t* count;
  __device__ int per_seq() const { return (t1 - t0) + (d1 - d0); }
  __device__ long long total(int B) const {
    return (long long)(seqs != nullptr ? int(*count) : B) * per_seq();
  }
  __device__ void at(long long it, int K, int& b, int& r) const {
    const int nr = per_seq(), nt = t1 - t0;
    const long long s = it / nr;
    const int lr = int(it % nr);
    b = seqs != nullptr ? seqs[s] : int(s);
    r = lr < nt ? t0 + lr : K + 1 + d0 + (lr - nt);
  }
};

// Whether the walk of sequence b keeps every position below p (p <= K),
// given the partials of their rows (one wavefront; lane i tests position i;
// a position with an unusable token or row stops the walk).
__device__ inline bool walk_reaches(const RowPart* __restrict__ parts, int b, int K, int V,
                                    int nseg, int p, int kb, const int32_t* __restrict__ tokens,
                                    const float* __restrict__ uniforms, float c) {
  const int lane = threadIdx.x & (kWave - 1);
  const int rows = 2 * K + 1;
  bool stop = false;
  if (lane < p && lane < kb) {
    const RowPart* pt = parts + ((long long)b * rows + lane) * nseg;
    const RowPart* pd = parts + ((long long)b * rows + K + 1 + lane) * nseg;
    float Rt, Rd;
    double St, Sd;
    combine_sum_parts(pt, nseg, Rt, St);
    combine_sum_parts(pd, nseg, Rd, Sd);
    const int d = tokens[(long long)b * K + lane];
    stop = !(d >= 0 && d < V) || !finite_pos(St) || !finite_pos(Sd);
    if (!stop) {
      double P, Q;
      stop = !accept_position(pt->m, pd->m, Rt, St, Rd, Sd,
                              double(uniforms[(long long)b * (K + 1) + lane]), c, P, Q);
    }
  }
  return __ballot(stop) == 0ull;
}

// top-m candidate list per wavefront (sv_topm.hpp) for the draft residual
// side output and store it, as at most m keys followed by zeros, at
//   topm_lists[((b K + i) nseg + seg) 4 + wavefront][0..m)
// (64 slots per list). The list is fed from each full group of chunks the
// wavefront reads with all 64 lanes together; the few chunks a lane reads
// after its wavefront's lanes part (at most 2U - 1) are read again and fed
// at the end. The normaliser is computed exactly as without TOPM.
constexpr int kTopmCapFused = 448;   // keys per wavefront list in the streaming pass

// One (row, segment) of the stochastic streaming pass: the segment's softmax
// normaliser relative to an integer reference, the logit at the row's
// drafted token, and with TOPM the draft row's top-m candidate lists; the
// workgroup's partial goes to parts[(b (2K+1) + r) nseg + seg]. Called once
// per workgroup (rowstats_sum) or for each listed row segment in turn
// (rowstats_sum_list); every thread of the workgroup calls it.
template <int DT, int VEC, int U, bool TOPM>
__device__ __forceinline__ void stream_segment(
    const void* __restrict__ target, const void* __restrict__ draft, int b, int r, int seg,
    int K, int V, int nseg, int seg_chunks, float c, RowPart* __restrict__ parts, int topm_m,
    uint64_t* __restrict__ topm_lists, const int32_t* __restrict__ tokens) {
  using C = Chunk<DT, VEC>;
  const int tid = threadIdx.x;
  const int rows = 2 * K + 1;
  const long long wg = ((long long)b * rows + r) * nseg + seg;   // global (row, segment)
  const void* row = row_ptr<DT>(target, draft, b, r, K, V);
  const long long nchunks = V / VEC;
  const long long c0 = (long long)seg * seg_chunks;
  const long long c1 = min(c0 + (long long)seg_chunks, nchunks);
  // the logit at this row's drafted token (target row i < K and draft row i
  // hold position i's), loaded now and stored with the row's partial, so the
  // scan that follows need not gather it; NaN when there is none or it is
  // out of range (the scan checks the token itself)
  float x_drafted = __builtin_nanf("");
  if (tokens != nullptr && tid == 0 && r != K) {
    const int i = r < K ? r : r - K - 1;
    const int d = tokens[(long long)b * K + i];
    if (d >= 0 && d < V) x_drafted = load_logit<DT>(row, d);
  }

  [[maybe_unused]] TopM<DT> tm;
  [[maybe_unused]] const bool topm_row = TOPM && r > K;   // uniform
  [[maybe_unused]] long long topm_next = c0 + tid;        // first chunk not yet fed
  [[maybe_unused]] bool topm_seeded = false;              // uniform
  if constexpr (TOPM) {
    __shared__ uint64_t s_tk[kWavesPerBlock][kTopmCapFused];
    __shared__ uint32_t s_tb[kWavesPerBlock][256];
    __shared__ u32x4 s_ts[kWavesPerBlock][kTopmStage];
    __shared__ uint32_t s_ta[kWavesPerBlock][kTopmStage];
    __shared__ unsigned long long s_tt;
    if (tid == 0) s_tt = 0ull;
    __syncthreads();
    tm.init(s_tk[tid / kWave], s_tb[tid / kWave], &s_tt, kTopmCapFused,
            uint32_t(min(topm_m, V)), s_ts[tid / kWave], s_ta[tid / kWave]);
  }
  // With a whole group for every thread, the first group starts every
  // wavefront's threshold from the workgroup's 256 lane maxima (their m-th
  // largest is at most the row's m-th largest value): a quarter as many
  // candidates as one wavefront's chunk maxima give, and no compaction is
  // needed along the way.
  [[maybe_unused]] const bool wg_seed = topm_row && (c1 - c0) >= (long long)U * kBlock;
  [[maybe_unused]] __shared__ uint32_t s_wg[TOPM ? 8 : 1];

  float R = kRefInit;
  double S = 0.0;
  long long ci = c0 + tid;
  // full groups of U chunks per lane
  for (; ci + (long long)(U - 1) * kBlock < c1; ci += (long long)U * kBlock) {
    typename C::raw_t raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) raw[u] = C::load(row, ci + (long long)u * kBlock);
    float x[U][C::N];
#pragma unroll
    for (int u = 0; u < U; ++u) C::unpack(raw[u], x[u]);
    float gm = x[0][0];
    [[maybe_unused]] float cm[U];
    if constexpr (TOPM) {   // chunk maxima first (the same maximum)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        cm[u] = x[u][0];
#pragma unroll
        for (int k = 1; k < C::N; ++k) cm[u] = fmaxf(cm[u], x[u][k]);
        gm = fmaxf(gm, cm[u]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int k = 0; k < C::N; ++k) gm = fmaxf(gm, x[u][k]);
    }
    const float Rn = fmaxf(R, ceilf(gm * c));
    S = rescale(S, R, Rn);
    R = Rn;
    float t[U * C::N];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int k = 0; k < C::N; ++k) t[u * C::N + k] = term(x[u][k], c, R);
#pragma unroll
    for (int w = 1; w < U * C::N; w <<= 1)
#pragma unroll
      for (int k = 0; k + w < U * C::N; k += 2 * w) t[k] += t[k + w];
    S += (double)t[0];
    if constexpr (TOPM) {
      if (wg_seed && !topm_seeded) {   // every thread is in this first group
        const uint32_t gbits = __float_as_uint(gm);
        uint32_t key = DT == DT_BF16 ? bf16_key(gbits >> 16) : order_key<DT_F32>(gbits);
        if (!(gm == gm)) key = 0u;    // (a NaN counts as nothing)
        const uint32_t t = wg_kth_top16<DT == DT_BF16 ? 16 : 32>(
            key, tm.want, tm.bins - (tid / kWave) * 256, s_wg);
        tm.thr = uint64_t(t) << 32;
        tm.thr_f = order_floor<DT>(t);
        if (tid == 0) atomicMax(tm.shared, (unsigned long long)tm.thr);
        topm_seeded = true;
      }
      if (topm_row && __builtin_amdgcn_read_exec() == ~0ull) {   // all 64 lanes here
        if (!topm_seeded) {   // the first group's chunk maxima start the threshold
          tm.template seed<U>(cm, (1u << U) - 1u);
          topm_seeded = true;
        }
        if (__ballot(gm >= tm.thr_f) != 0ull) {
#pragma unroll
          for (int u = 0; u < U; ++u)
            tm.stage_chunk(cm[u] >= tm.thr_f, raw[u], uint32_t(ci + (long long)u * kBlock));
          // a tighter threshold early stages fewer chunks (measured a small
          // gain with the wavefront seed)
          if (!wg_seed && tm.fill > 2 * tm.want) tm.compact();
        }
        topm_next = ci + (long long)U * kBlock;
      }
    }
  }
  // remainder, one chunk at a time
  for (; ci < c1; ci += kBlock) {
    typename C::raw_t raw = C::load(row, ci);
    float x[C::N];
    C::unpack(raw, x);
    float gm = x[0];
#pragma unroll
    for (int k = 1; k < C::N; ++k) gm = fmaxf(gm, x[k]);
    const float Rn = fmaxf(R, ceilf(gm * c));
    S = rescale(S, R, Rn);
    R = Rn;
    float t[C::N];
#pragma unroll
    for (int k = 0; k < C::N; ++k) t[k] = term(x[k], c, R);
#pragma unroll
    for (int w = 1; w < C::N; w <<= 1)
#pragma unroll
      for (int k = 0; k + w < C::N; k += 2 * w) t[k] += t[k + w];
    S += (double)t[0];
  }

  if constexpr (TOPM) {
    if (topm_row) {   // the lanes are together again: feed the chunks read apart
      typename C::raw_t raw[2 * U - 1];
#pragma unroll
      for (int j = 0; j < 2 * U - 1; ++j) {
        const long long cc = topm_next + (long long)j * kBlock;
        raw[j] = C::load(row, cc < c1 ? cc : c0);
      }
#pragma unroll
      for (int j = 0; j < 2 * U - 1; ++j) {
        const long long cc = topm_next + (long long)j * kBlock;
        tm.stage_chunk(cc < c1 && chunk_max<DT>(raw[j]) >= tm.thr_f, raw[j], uint32_t(cc));
      }
      tm.flush();
      tm.compact();
      const int lane = tid & (kWave - 1);
      uint64_t* out = topm_lists +
                      ((((long long)b * K + (r - K - 1)) * nseg + seg) * kWavesPerBlock +
                       tid / kWave) * 64;
      for (uint32_t e = uint32_t(lane); e < tm.want; e += kWave)
        out[e] = e < tm.fill ? tm.keys[e] : 0ull;
    }
  }

  // workgroup combine: common reference, exact rescale, fixed-order sums
  __shared__ float sR[kWavesPerBlock];
  __shared__ double sS[kWavesPerBlock];
  const int lane = tid & (kWave - 1), wid = tid / kWave;
  float Rw = wave_max(R);
  double Sw = wave_sum(rescale(S, R, Rw));
  if (lane == 0) {
    sR[wid] = Rw;
    sS[wid] = Sw;
  }
  __syncthreads();
  if (tid == 0) {
    float Rb = sR[0];
#pragma unroll
    for (int w = 1; w < kWavesPerBlock; ++w) Rb = fmaxf(Rb, sR[w]);
    double Sb = 0.0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) Sb += rescale(sS[w], sR[w], Rb);
    RowPart p;
    p.S = Sb;
    p.R = Rb;
    p.m = x_drafted;
    p.idx = -1;
    p.flags = 0;
    parts[wg] = p;
  }
}

template <int DT, int VEC, int U, bool TOPM = false>
__global__ __launch_bounds__(kBlock, TOPM ? 4 : 1) void rowstats_sum(
    const void* __restrict__ target, const void* __restrict__ draft, int b0, int K, int V,
    int nseg, int seg_chunks, float c, const int32_t* __restrict__ kdraft,
    RowPart* __restrict__ parts, uint32_t* __restrict__ hist, int topm_m,
    uint64_t* __restrict__ topm_lists, const int32_t* __restrict__ tokens, StageRows sr,
    const float* __restrict__ uniforms) {
  static_assert(!TOPM || (DT == DT_BF16 && VEC == 8) || (DT == DT_F32 && VEC == 4),
                "top-m lists need 16-byte chunks");
  const int tid = threadIdx.x;
  const int nt = sr.t1 - sr.t0, nr = nt + (sr.d1 - sr.d0);   // rows per sequence here
  const long long lw = (long long)b0 * nr * nseg + blockIdx.x;
  const int seg = int(lw % nseg);
  const long long lrow = lw / nseg;
  const int b = int(lrow / nr), lr = int(lrow % nr);
  const int r = lr < nt ? sr.t0 + lr : K + 1 + sr.d0 + (lr - nt);
  if (blockIdx.x == 0 && hist != nullptr && tid <= K) hist[tid] = 0u;
  if (blockIdx.x == 0 && sr.clear != nullptr && tid == 0) *sr.clear = 0u;
  // with per-sequence draft counts k_b, target rows past k_b and draft rows
  // k_b.. are never read again: skip them (uniform over the workgroup)
  const int kb = kdraft != nullptr ? kdraft[b] : K;
  if (kdraft != nullptr && (r <= K ? r > kb : r - K - 1 >= kb)) return;
  // walk-order reading: rows of positions the walk does not reach are never
  // read (wavefront 0 decides for the workgroup)
  if (sr.gate > 0) {
    __shared__ int s_reach;
    if (tid < kWave) {
      const bool reach = walk_reaches(parts, b, K, V, nseg, sr.gate, kb, tokens, uniforms, c);
      if (tid == 0) s_reach = reach ? 1 : 0;
    }
    __syncthreads();
    if (!s_reach) return;
  }

  stream_segment<DT, VEC, U, TOPM>(target, draft, b, r, seg, K, V, nseg, seg_chunks, c, parts,
                                   topm_m, topm_lists, tokens);
}

// Walk-order reading, after the streaming pass over position 0: one
// wavefront per sequence tests positions below p0 from their partials (as
// walk_reaches does for a gated workgroup) and lists the sequences whose walk
// reaches p0 and that have rows there (k_b >= p0) in seqs[0 .. *count) (in
// no particular order; count starts at 0).
__global__ __launch_bounds__(kBlock) void walk_gate(
    int B, int K, int V, int nseg, const RowPart* __restrict__ parts,
    const int32_t* __restrict__ kdraft, const int32_t* __restrict__ tokens,
    const float* __restrict__ uniforms, float c, int p0, int32_t* __restrict__ seqs,
    uint32_t* __restrict__ count) {
  const int lane = threadIdx.x & (kWave - 1);
  const int b = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  if (b >= B) return;                              // (the whole wavefront)
  const int kb = kdraft != nullptr ? kdraft[b] : K;
  if (!(kb >= p0 && kb <= K)) return;              // nothing there to read
  if (walk_reaches(parts, b, K, V, nseg, p0, kb, tokens, uniforms, c) && lane == 0)
    seqs[atomicAdd(count, 1u)] = b;
}

// Walk-order reading: the row segments of positions p0..K (target rows
// p0..K, draft rows p0..K-1) of the listed sequences, spread over a fixed
// grid that loops over them, so that sequences whose walk ended cost no
// workgroup. Each segment's partial is the one rowstats_sum would write.
template <int DT, int VEC, int U>
__global__ __launch_bounds__(kBlock) void rowstats_sum_list(
    const void* __restrict__ target, const void* __restrict__ draft, int K, int V, int nseg,
    int seg_chunks, float c, const int32_t* __restrict__ kdraft, RowPart* __restrict__ parts,
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ seqs,
    const uint32_t* __restrict__ count, int p0) {
  const int nt = K + 1 - p0, nr = nt + (K - p0);
  const long long items = (long long)(*count) * nr * nseg;
  for (long long it = blockIdx.x; it < items; it += gridDim.x) {
    const int seg = int(it % nseg);
    const long long lrow = it / nseg;
    const int b = seqs[lrow / nr], lr = int(lrow % nr);
    const int r = lr < nt ? p0 + lr : K + 1 + p0 + (lr - nt);
    const int kb = kdraft != nullptr ? kdraft[b] : K;
    if (kdraft != nullptr && (r <= K ? r > kb : r - K - 1 >= kb)) continue;   // (uniform)
    stream_segment<DT, VEC, U, false>(target, draft, b, r, seg, K, V, nseg, seg_chunks, c,
                                      parts, 0, nullptr, tokens);
    __syncthreads();                 // the combine's LDS is reused by the next segment
  }
}

// --------------------------------------------------------------------------
// Streaming max / argmax / NaN flag over target rows (greedy, margin).
// A lane remembers the first chunk in which its running maximum was reached
// and finds the lowest matching element in it at the end.
// --------------------------------------------------------------------------
// One (target row, segment) of the argmax pass: the segment's maximum, its
// lowest index and a NaN flag, written to parts[(b (K+1) + r) nseg + seg].
// Called once per workgroup (rowstats_max) or for each listed row segment in
// turn (rowstats_max_list); every thread of the workgroup calls it.
template <int DT, int VEC, int U>
__device__ __forceinline__ void max_segment(const void* __restrict__ target, int b, int r,
                                            int seg, int K, int V, int nseg, int seg_chunks,
                                            RowPart* __restrict__ parts) {
  using C = Chunk<DT, VEC>;
  const int tid = threadIdx.x;
  const long long wg = ((long long)b * (K + 1) + r) * nseg + seg;
  const void* row = row_ptr<DT>(target, nullptr, b, r, K, V);
  const long long nchunks = V / VEC;
  const long long c0 = (long long)seg * seg_chunks;
  const long long c1 = min(c0 + (long long)seg_chunks, nchunks);

  float best = -__builtin_inff();
  long long best_c = -1;
  typename C::raw_t best_raw{};
  uint32_t nan = 0;
  long long ci = c0 + tid;
  for (; ci + (long long)(U - 1) * kBlock < c1; ci += (long long)U * kBlock) {
    typename C::raw_t raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) raw[u] = C::load(row, ci + (long long)u * kBlock);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float x[C::N];
      C::unpack(raw[u], x);
      float cm = x[0];
#pragma unroll
      for (int k = 1; k < C::N; ++k) cm = fmaxf(cm, x[k]);
      nan |= C::nan_bits(raw[u]);
      const bool up = cm > best;
      best = up ? cm : best;
      best_c = up ? ci + (long long)u * kBlock : best_c;
      best_raw = up ? raw[u] : best_raw;
    }
  }
  for (; ci < c1; ci += kBlock) {
    typename C::raw_t raw = C::load(row, ci);
    float x[C::N];
    C::unpack(raw, x);
    float cm = x[0];
#pragma unroll
    for (int k = 1; k < C::N; ++k) cm = fmaxf(cm, x[k]);
    nan |= C::nan_bits(raw);
    const bool up = cm > best;
    best = up ? cm : best;
    best_c = up ? ci : best_c;
    best_raw = up ? raw : best_raw;
  }
  int idx = -1;
  if (best_c >= 0) {
    float x[C::N];
    C::unpack(best_raw, x);
    int e = C::N - 1;
#pragma unroll
    for (int k = C::N - 1; k >= 0; --k) e = (x[k] == best) ? k : e;
    idx = int(best_c * VEC + e);
  }

  __shared__ float sm[kWavesPerBlock];
  __shared__ int si[kWavesPerBlock];
  __shared__ uint32_t sn[kWavesPerBlock];
  const int lane = tid & (kWave - 1), wid = tid / kWave;
  wave_argmax(best, idx);
  nan = wave_or(nan);
  if (lane == 0) {
    sm[wid] = best;
    si[wid] = idx;
    sn[wid] = nan;
  }
  __syncthreads();
  if (tid == 0) {
    float m = sm[0];
    int i = si[0];
    uint32_t f = sn[0];
#pragma unroll
    for (int w = 1; w < kWavesPerBlock; ++w) {
      argmax_combine(m, i, sm[w], si[w]);
      f |= sn[w];
    }
    RowPart p;
    p.S = 0.0;
    p.R = 0.0f;
    p.m = m;
    p.idx = i;
    p.flags = f ? 1 : 0;
    parts[wg] = p;
  }
}

// Every (target row, segment) of target rows r0 .. r0 + nr - 1 of every
// sequence (all of them: r0 = 0, nr = K + 1); workgroup 0 clears the
// histogram and, when set, the walk-order list count.
template <int DT, int VEC, int U>
__global__ __launch_bounds__(kBlock) void rowstats_max(const void* __restrict__ target, int K,
                                                       int V, int nseg, int seg_chunks,
                                                       const int32_t* __restrict__ kdraft,
                                                       RowPart* __restrict__ parts,
                                                       uint32_t* __restrict__ hist, int r0,
                                                       int nr, uint32_t* __restrict__ clear) {
  const int tid = threadIdx.x;
  const long long lw = blockIdx.x;
  const int seg = int(lw % nseg);
  const long long lrow = lw / nseg;
  const int b = int(lrow / nr), r = r0 + int(lrow % nr);
  if (lw == 0 && hist != nullptr && tid <= K) hist[tid] = 0u;
  if (lw == 0 && clear != nullptr && tid == 0) *clear = 0u;
  if (kdraft != nullptr && r > kdraft[b]) return;   // target row past k_b: not needed
  max_segment<DT, VEC, U>(target, b, r, seg, K, V, nseg, seg_chunks, parts);
}

// The greedy or margin test of one drafted position from its target row's
// combined maximum m and lowest argmax A ([SMB] "The Guarantee Behind
// Rejection Sampling": greedy keeps a draft that is the target's argmax;
// [MNW] the margin rule also keeps one whose probability ratio to the top-1
// token exceeds tau). Every place that takes this decision (the argmax scan
// and the walk-order gate) calls this one function. ratio: the margin ratio.
template <int DT, bool MARGIN>
__device__ inline bool argmax_kept(const void* __restrict__ target, int b, int i, int K, int V,
                                   int d, int A, float m, double invT, double tau,
                                   double& ratio) {
  if constexpr (MARGIN) {
    const float xd = load_logit<DT>(row_ptr<DT>(target, nullptr, b, i, K, V), d);
    ratio = exp((double(xd) - double(m)) * invT);
    return (d == A) || (ratio > tau);
  } else {
    return d == A;
  }
}

// The greedy or margin walk of sequence b keeps every position below p
// (one wavefront; lane i tests position i from its row's partials; an
// unusable row or token stops the walk).
template <int DT, bool MARGIN>
__device__ inline bool argmax_walk_reaches(const RowPart* __restrict__ parts,
                                           const void* __restrict__ target, int b, int K, int V,
                                           int nseg, int p, int kb,
                                           const int32_t* __restrict__ tokens, double invT,
                                           double tau) {
  const int lane = threadIdx.x & (kWave - 1);
  bool stop = false;
  if (lane < p && lane < kb) {
    float m;
    int A, nan;
    combine_max_parts(parts + ((long long)b * (K + 1) + lane) * nseg, nseg, m, A, nan);
    const int d = tokens[(long long)b * K + lane];
    stop = nan != 0 || !(m > -__builtin_inff() && m < __builtin_inff()) || A < 0 ||
           !(d >= 0 && d < V);
    if (!stop) {
      double ratio;
      stop = !argmax_kept<DT, MARGIN>(target, b, lane, K, V, d, A, m, invT, tau, ratio);
    }
  }
  return __ballot(stop) == 0ull;
}

// Walk-order reading of greedy and margin calls, after the argmax pass over
// target row 0: lists the sequences whose walk keeps position 0 and that
// have rows past it (k_b >= 1), as walk_gate does for stochastic calls.
template <int DT, bool MARGIN>
__global__ __launch_bounds__(kBlock) void walk_gate_argmax(
    int B, int K, int V, int nseg, const RowPart* __restrict__ parts,
    const void* __restrict__ target, const int32_t* __restrict__ kdraft,
    const int32_t* __restrict__ tokens, double invT, double tau, int p0,
    int32_t* __restrict__ seqs, uint32_t* __restrict__ count) {
  const int lane = threadIdx.x & (kWave - 1);
  const int b = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  if (b >= B) return;                              // (the whole wavefront)
  const int kb = kdraft != nullptr ? kdraft[b] : K;
  if (!(kb >= p0 && kb <= K)) return;
  if (argmax_walk_reaches<DT, MARGIN>(parts, target, b, K, V, nseg, p0, kb, tokens, invT, tau) &&
      lane == 0)
    seqs[atomicAdd(count, 1u)] = b;
}

// Walk-order reading: the (target row, segment)s of rows p0..K of the listed
// sequences over a fixed grid, as rowstats_sum_list does for stochastic calls.
template <int DT, int VEC, int U>
__global__ __launch_bounds__(kBlock) void rowstats_max_list(
    const void* __restrict__ target, int K, int V, int nseg, int seg_chunks,
    const int32_t* __restrict__ kdraft, RowPart* __restrict__ parts,
    const int32_t* __restrict__ seqs, const uint32_t* __restrict__ count, int p0) {
  const int nr = K + 1 - p0;
  const long long items = (long long)(*count) * nr * nseg;
  for (long long it = blockIdx.x; it < items; it += gridDim.x) {
    const int seg = int(it % nseg);
    const long long lrow = it / nseg;
    const int b = seqs[lrow / nr], r = p0 + int(lrow % nr);
    if (kdraft != nullptr && r > kdraft[b]) continue;   // (uniform)
    max_segment<DT, VEC, U>(target, b, r, seg, K, V, nseg, seg_chunks, parts);
    __syncthreads();                 // the combine's LDS is reused by the next segment
  }
}

}  // namespace sv
