// Top-k / top-p truncation passes over bf16 logit rows (gfx950).
//
// p and q are the distributions the samplers really use, after temperature
// and truncation, and the same truncation has to hold in the acceptance ratio,
// the residual and the bonus draw ([RNR] s.1 and s.2). The rules: top-k keeps
// the values at or above the k-th largest (counted with multiplicity, so ties
// at the cut stay); top-p then keeps, from the top, whole value levels up to
// and including the first level at which the kept mass reaches top_p of the
// top-k mass.
//
// Each needed row (target rows 0..k_b, draft rows 0..k_b-1) is read once and
// its values counted into an exact histogram by value. Every value of one
// level has the same softmax term, so the histogram gives all the truncation
// needs:
//   * the row maximum and the integer reference R = ceil(max * c);
//   * top-k: the threshold is the level at which the count of values at or
//     above it, from the top, first reaches k;
//   * level masses count * 2^(x c - R), the top-k normaliser S_k, and top-p:
//     the threshold is the level at which the mass at or above it, from the
//     top, first reaches top_p * S_k;
//   * the truncated normaliser: the mass at or above the final threshold.
// Output: one RowPart per row with S = truncated normaliser (relative to
// 2^R), R, idx = threshold key (bf16_key order). A row holding NaN or +inf,
// or without a finite maximum, or a sequence whose top_p is not > 0, gets
// S = NaN, which makes the sequence invalid in the scan.
//
// Two passes share the work. The window pass (rowstats_trunc_win, at the end
// of this file) takes every row whose values are all zeros, -inf or inside
// the finish's table window 2^-25 <= |x| < 2^7: 8192 bins with 32-bit
// counters in 32 KiB of LDS, so that several rows share a compute unit. It
// marks any other row, and the full pass (rowstats_trunc) then counts those
// rows over all 65536 16-bit keys: one 1024-thread workgroup per row, 16-bit
// counters two to a 32-bit word (128 KiB).
//
// In the full pass a counter wraps only when one value occurs more than
// 65535 times in the row. The first count adds without looking; the counts
// are then summed and compared with V. On a mismatch the row is counted
// again, in two passes with returning atomics: first only the even keys (low
// halves), where a wrap's carry into the still-empty high half is taken back
// at once, then only the odd keys (high halves), whose carries leave the
// word. Each wrap is recorded in a short list (65536 more for that key); as
// the halves are never counted at the same time, no count sees another
// half's carry. A row that still does not add up (more wraps than the list
// holds) is marked invalid.
#pragma once

#include "sv_fused.hpp"

namespace sv {

constexpr int kTrBlock = 1024;
constexpr int kTrWaves = kTrBlock / kWave;
constexpr int kHistWords = 32768;                    // 65536 16-bit counters
constexpr int kKeysPerThread = 65536 / kTrBlock;     // 64 consecutive keys per thread
constexpr int kMaxWraps = 32;

constexpr int kTruncRedo = 2;   // RowPart flag: the row needs the full-histogram pass

// Truncation settings of one call, per sequence (null: that rule is off).
struct Trunc {
  const int32_t* k;    // top_k; <= 0 or >= V: off
  const float* p;      // top_p; >= 1: off; not > 0: invalid sequence
};

typedef short s16x2 __attribute__((ext_vector_type(2)));

// bf16_key of both halves of a word of two bf16 values: x ^ 0x8000 for
// x >= 0, (x ^ 0xffff) + 1 for x < 0, with 16-bit lanes
__device__ __forceinline__ uint32_t bf16_keys2(uint32_t w) {
  const s16x2 sw = __builtin_bit_cast(s16x2, w);
  const u16x2 neg = __builtin_bit_cast(u16x2, (s16x2)(sw >> (s16x2){15, 15}));
  const uint32_t m = __builtin_bit_cast(uint32_t, neg) | 0x80008000u;
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, w ^ m) - neg);
}

// LDS word of histogram word w = key >> 1. Thread t of the scan owns words
// 32t .. 32t + 31 (keys 64t .. 64t + 63), read as eight 16-byte chunks; the
// chunks of each segment are permuted by the low 3 bits of t, so that when
// every thread reads chunk q of its own segment the wavefront's reads spread
// over all banks instead of landing on one.
__device__ __forceinline__ uint32_t hist_word(uint32_t w) { return w ^ ((w >> 3) & 0x1cu); }

// Counting modes: every key without looking, or (careful) only the even or
// only the odd keys, recording wraps.
enum { kCountFast = 0, kCountEven = 1, kCountOdd = 2 };

template <int MODE>
__device__ __forceinline__ void count_key(uint32_t* H, uint32_t key, uint32_t* nwrap,
                                          uint32_t* wraps) {
  const uint32_t w = hist_word(key >> 1), sh = (key & 1u) << 4;
  if constexpr (MODE == kCountFast) {
    atomicAdd(&H[w], 1u << sh);
  } else {
    if ((key & 1u) != (MODE == kCountOdd ? 1u : 0u)) return;
    const uint32_t old = atomicAdd(&H[w], 1u << sh);
    if (((old >> sh) & 0xffffu) == 0xffffu) {
      if (MODE == kCountEven) atomicSub(&H[w], 0x10000u);   // the carry into the high half
      const uint32_t slot = atomicAdd(nwrap, 1u);
      if (slot < uint32_t(kMaxWraps)) wraps[slot] = key;
    }
  }
}

template <int VEC, int MODE>
__device__ __forceinline__ void count_chunk(const typename Chunk<DT_BF16, VEC>::raw_t& raw,
                                            uint32_t* H, uint32_t* nwrap, uint32_t* wraps) {
  if constexpr (VEC == 8) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t k2 = bf16_keys2(raw[q]);
      count_key<MODE>(H, k2 & 0xffffu, nwrap, wraps);
      count_key<MODE>(H, k2 >> 16, nwrap, wraps);
    }
  } else {
    count_key<MODE>(H, bf16_key(raw), nwrap, wraps);
  }
}

// Count the row's values into the histogram (cleared first, except before
// the odd-key pass, which completes the even-key one).
template <int VEC, int MODE>
__device__ __forceinline__ void count_row(const void* row, int V, uint32_t* H, uint32_t* nwrap,
                                          uint32_t* wraps) {
  using C = Chunk<DT_BF16, VEC>;
  const int tid = threadIdx.x;
  if constexpr (MODE != kCountOdd) {
    for (int i = tid; i < kHistWords / 4; i += kTrBlock)
      reinterpret_cast<u32x4*>(H)[i] = (u32x4){0u, 0u, 0u, 0u};
    if (tid == 0) *nwrap = 0u;
    __syncthreads();
  }
  constexpr int U = 4;
  const long long nchunks = V / VEC;
  long long ci = tid;
  for (; ci + (long long)(U - 1) * kTrBlock < nchunks; ci += (long long)U * kTrBlock) {
    typename C::raw_t raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) raw[u] = C::load(row, ci + (long long)u * kTrBlock);
#pragma unroll
    for (int u = 0; u < U; ++u) count_chunk<VEC, MODE>(raw[u], H, nwrap, wraps);
  }
  for (; ci < nchunks; ci += kTrBlock) count_chunk<VEC, MODE>(C::load(row, ci), H, nwrap, wraps);
  __syncthreads();
}

// ---- workgroup reductions over the NW wavefronts (fixed order) ----
template <typename T_, int NW = kTrWaves>
__device__ inline T_ tr_sum(T_ v, T_* s) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  if (lane == 0) s[wid] = v;
  __syncthreads();
  T_ t = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) t += s[w];
  __syncthreads();
  return t;
}

template <int NW = kTrWaves>
__device__ inline int tr_max(int v, int* s) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
  if (lane == 0) s[wid] = v;
  __syncthreads();
  int t = s[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) t = max(t, s[w]);
  __syncthreads();
  return t;
}

// Sum of v over the threads with a larger index (= the higher keys), and the
// total over all threads.
template <typename T_, int NW = kTrWaves>
__device__ inline T_ tr_above(T_ v, T_* s, T_& total) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  T_ incl = v;      // sum over lanes lane..63 of this wavefront
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const T_ u = __shfl_down(incl, o, kWave);
    if (lane + o < kWave) incl += u;
  }
  T_ excl = __shfl_down(incl, 1, kWave);
  if (lane == kWave - 1) excl = 0;
  if (lane == 0) s[wid] = incl;
  __syncthreads();
  T_ hi = 0, tot = 0;
#pragma unroll
  for (int w = NW - 1; w >= 0; --w) {
    if (w > wid) hi += s[w];
    tot += s[w];
  }
  __syncthreads();
  total = tot;
  return hi + excl;
}

template <int VEC>
// One workgroup per compute unit takes the rows sel selects (candidates
// blockIdx.x, blockIdx.x + gridDim.x, ...): its threads first check up to
// 1024 of them at once and list the ones the window pass handed over, then
// the workgroup counts the listed rows one after another.
__global__ __launch_bounds__(kTrBlock) void rowstats_trunc(
    const void* __restrict__ target, const void* __restrict__ draft, int B, int K, int V,
    float c, double c64, Trunc tr, const int32_t* __restrict__ kdraft,
    RowPart* __restrict__ parts, RowSel sel) {
  __shared__ uint32_t H[kHistWords];
  __shared__ uint32_t s_wraps[kMaxWraps];
  __shared__ uint32_t s_nwrap;
  __shared__ uint32_t s_u[kTrWaves];
  __shared__ int s_i[kTrWaves];
  __shared__ double s_d[kTrWaves];
  __shared__ uint32_t s_key;
  __shared__ double s_S;
  __shared__ long long s_rows[kTrBlock];
  __shared__ int s_nrows;
  const int tid = threadIdx.x;
  const int rows = 2 * K + 1;
  const long long nrows = sel.total(B);
  for (long long g0 = blockIdx.x; g0 < nrows; g0 += (long long)gridDim.x * kTrBlock) {
  if (tid == 0) s_nrows = 0;
  __syncthreads();
  {
    const long long cand = g0 + (long long)tid * gridDim.x;
    if (cand < nrows) {
      int cb, cr;
      sel.at(cand, K, cb, cr);
      bool need = true;              // rows past the draft count are not needed
      if (kdraft != nullptr) {
        const int kb = kdraft[cb];
        need = !(cr <= K ? cr > kb : cr - K - 1 >= kb);
      }
      const long long grow = (long long)cb * rows + cr;
      if (need && parts[grow].flags == kTruncRedo) s_rows[atomicAdd(&s_nrows, 1)] = grow;
    }
  }
  __syncthreads();
  const int n_listed = s_nrows;
  for (int li = 0; li < n_listed; ++li) {
  const long long grow = s_rows[li];
  const int b = int(grow / rows), r = int(grow % rows);
  __syncthreads();                   // the previous row's scan is over
  const void* row = row_ptr<DT_BF16>(target, draft, b, r, K, V);
  const uint32_t k0 = uint32_t(tid) * kKeysPerThread;

  // The scan phase walks this thread's keys k0 .. k0 + 63 one 16-byte chunk
  // (8 keys) at a time: chunk q holds the counts of keys k0 + 8q + e, e < 8,
  // key k0 + 8q + 2i in the low and k0 + 8q + 2i + 1 in the high half of word
  // i. A key that wrapped in the careful count has 65536 more per recorded
  // wrap.
  uint32_t nwrap = 0;
  auto chunk = [&](int q) -> u32x4 {
    return reinterpret_cast<const u32x4*>(H)[tid * (kKeysPerThread / 8) + (q ^ (tid & 7))];
  };
  auto wrap_extra = [&](uint32_t key) -> uint32_t {
    uint32_t n = 0;
    const int nw = min(int(nwrap), kMaxWraps);
#pragma unroll 1
    for (int e = 0; e < nw; ++e) n += s_wraps[e] == key ? 65536u : 0u;
    return n;
  };
  auto thread_total = [&]() -> uint32_t {
    nwrap = s_nwrap;
    uint32_t t = 0;
#pragma unroll 2
    for (int q = 0; q < kKeysPerThread / 8; ++q) {
      const u32x4 v = chunk(q);
#pragma unroll
      for (int i = 0; i < 4; ++i) t += (v[i] & 0xffffu) + (v[i] >> 16);
    }
    if (nwrap != 0u)
#pragma unroll 1
      for (int e = 0; e < min(int(nwrap), kMaxWraps); ++e)
        t += (s_wraps[e] >> 6) == uint32_t(tid) ? 65536u : 0u;
    return t;
  };

  // ---- 1. count; totals, maximum, non-finite values ----
  count_row<VEC, kCountFast>(row, V, H, &s_nwrap, s_wraps);
  uint32_t n_t = thread_total();
  bool bad = false;
  if (tr_sum(n_t, s_u) != uint32_t(V)) {      // a counter wrapped: count again, carefully
    count_row<VEC, kCountEven>(row, V, H, &s_nwrap, s_wraps);
    count_row<VEC, kCountOdd>(row, V, H, &s_nwrap, s_wraps);
    n_t = thread_total();
    bad = tr_sum(n_t, s_u) != uint32_t(V) || nwrap > uint32_t(kMaxWraps);
  }
  // bit i of nz: key k0 + i occurs in the row
  uint64_t nz = 0;
#pragma unroll 1
  for (int q = 0; q < kKeysPerThread / 8; ++q) {
    const u32x4 v = chunk(q);
    uint32_t bits = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      bits |= ((v[i] & 0xffffu) ? 1u : 0u) << (2 * i) | ((v[i] >> 16) ? 2u : 0u) << (2 * i);
    nz |= uint64_t(bits) << (8 * q);
  }
  if (nwrap != 0u)
#pragma unroll 1
    for (int e = 0; e < min(int(nwrap), kMaxWraps); ++e)
      if ((s_wraps[e] >> 6) == uint32_t(tid)) nz |= 1ull << (s_wraps[e] & 63u);
  // finite keys of this thread (only the first and last few threads hold others)
  uint64_t fin = ~0ull, nonfin = 0;
  if (k0 <= kKeyNegInf || k0 + uint32_t(kKeysPerThread - 1) >= kKeyPosInf) {
    fin = 0;
#pragma unroll 1
    for (int i = 0; i < kKeysPerThread; ++i) {
      const uint32_t key = k0 + uint32_t(i);
      if (key_finite(key)) fin |= 1ull << i;
      if (key < kKeyNegInf || key >= kKeyPosInf) nonfin |= 1ull << i;
    }
  }
  const int top_t = (nz & fin) ? int(k0) + 63 - __builtin_clzll(nz & fin) : 0;
  const int top = tr_max(top_t, s_i);
  bad = bad || tr_max((nz & nonfin) ? 1 : 0, s_i) != 0 || top == 0;
  const float R = top > 0 ? ceilf(key_value(uint32_t(top)) * c) : 0.0f;
  // count of key k0 + i from LDS
  auto count_of = [&](int i) -> uint32_t {
    const uint32_t key = k0 + uint32_t(i);
    const uint32_t n = (H[hist_word(key >> 1)] >> ((key & 1u) << 4)) & 0xffffu;
    return nwrap != 0u ? n + wrap_extra(key) : n;
  };

  // ---- 2. top-k threshold from the counts ----
  const int kk = tr.k != nullptr ? tr.k[b] : 0;
  uint32_t tk = 0u;
  if (kk >= 1 && kk < V) {
    uint32_t n_all;
    const uint32_t above = tr_above(n_t, s_u, n_all);
    const int cut = tr_max(above + n_t >= uint32_t(kk) ? tid : -1, s_i);
    if (tid == cut) {
      uint32_t acc = above;
      for (uint64_t m = nz; m != 0;) {
        const int i = 63 - __builtin_clzll(m);
        m &= ~(1ull << i);
        acc += count_of(i);
        if (acc >= uint32_t(kk)) {
          s_key = k0 + uint32_t(i);
          break;
        }
      }
    }
    __syncthreads();
    tk = s_key;
    __syncthreads();
  }

  // ---- 3. level masses at or above the top-k threshold, S_k ----
  // The occurring finite keys at or above tk, largest first; the top-p walk
  // below repeats the same operations in the same order.
  const uint64_t ge = tk <= k0 ? ~0ull
                      : tk > k0 + uint32_t(kKeysPerThread - 1) ? 0ull : (~0ull << (tk - k0));
  const uint64_t live = nz & fin & ge;
  double M_t = 0.0;
  for (uint64_t m = live; m != 0;) {
    const int i = 63 - __builtin_clzll(m);
    m &= ~(1ull << i);
    M_t = __builtin_fma(double(count_of(i)), level_term(k0 + uint32_t(i), c64, R), M_t);
  }
  double S_k;
  const double above_m = tr_above(M_t, s_d, S_k);

  // ---- 4. top-p threshold from the masses ----
  const float pp = tr.p != nullptr ? tr.p[b] : 1.0f;
  bad = bad || !(pp > 0.0f);
  uint32_t thr = tk;
  double S_tr = S_k;
  if (pp < 1.0f && !bad) {
    const double goal = double(pp) * S_k;
    const int cut = tr_max(above_m + M_t >= goal ? tid : -1, s_i);
    if (cut >= 0) {
      if (tid == cut) {
        double part = 0.0;
        for (uint64_t m = live; m != 0;) {
          const int i = 63 - __builtin_clzll(m);
          m &= ~(1ull << i);
          part = __builtin_fma(double(count_of(i)), level_term(k0 + uint32_t(i), c64, R), part);
          if (above_m + part >= goal) {
            s_key = k0 + uint32_t(i);
            s_S = above_m + part;
            break;
          }
        }
      }
      __syncthreads();
      thr = s_key;
      S_tr = s_S;
    }
  }
  if (tid == 0) {
    RowPart p;
    p.S = bad ? __builtin_nan("") : S_tr;
    p.R = R;
    p.m = 0.0f;
    p.idx = int(thr);
    p.flags = 0;
    parts[grow] = p;
  }
  }
  __syncthreads();                   // the list is read before it is reset
  }
}

// ---------------------------------------------------------------------------
// Window pass (the common case): one 512-thread workgroup per needed row
// counts the row into 8192 bins with 32-bit counters (32 KiB of LDS, so that
// several rows share a compute unit and one row's scan overlaps another's
// reads). The bins ascend with the value: bin 0 holds -inf, bins 1 .. 3968
// the negative values with 2^-24 <= |x| < 2^7 (one bin per value), bin 3969
// the negative values with |x| < 2^-24, bin 3970 zero, bin 3971 the positive
// values below 2^-24, bins 3972 .. 7939 the positive window values; bin 8191
// counts every other value (|x| >= 2^7, +inf, NaN). The two bins of tiny
// values hold several values each: their masses are summed value by value
// in a second read of the row (only rows that have such values), and a row
// whose maximum or threshold falls in one of them is handed over. A row with
// a value in bin 8191 is handed over too: marked kTruncRedo and left to the
// full-histogram pass above.
// ---------------------------------------------------------------------------
constexpr int kTwBlock = 512;
constexpr int kTwWaves = kTwBlock / kWave;
using u16x2 = unsigned short __attribute__((ext_vector_type(2)));

constexpr int kWinBins = 8192;
constexpr int kBinsPerThread = kWinBins / kTwBlock;      // 16
constexpr int kWinELo = 127 - 24;                        // smallest window exponent field
constexpr int kWinHalf = 31 * 128;                       // 3968 window values per sign
constexpr int kWinZero = kWinHalf + 2;                   // 3970
constexpr int kTinyNeg = kWinZero - 1, kTinyPos = kWinZero + 1;
constexpr int kWinOther = kWinBins - 1;
constexpr uint32_t kTinyKey = 0xffffffffu;               // a cut inside a tiny-value bin

// key (bf16_key order) of bin i < kWinOther outside the tiny-value bins
__device__ inline uint32_t win_key(int i) {
  if (i == 0) return kKeyNegInf;
  if (i == kWinZero) return 0x8000u;
  const uint32_t mag = uint32_t(i > kWinZero ? i - kTinyPos - 1 : kTinyNeg - 1 - i) +
                       uint32_t(kWinELo << 7);
  return i > kWinZero ? 0x8000u + mag : 0x8000u - mag;
}

// bin of one bf16 value, without branches
__device__ __forceinline__ uint32_t win_bin(uint32_t bits) {
  const uint32_t mag = bits & 0x7fffu;
  const uint32_t off2 = mag - uint32_t((kWinELo << 7) - 2);          // window: 2 .. 3969
  const int neg = int(bits << 16) >> 31;                              // 0 or -1
  const uint32_t wb = uint32_t(kWinZero) + ((off2 ^ uint32_t(neg)) - uint32_t(neg));
  const uint32_t tiny = uint32_t(kWinZero) + ((1u ^ uint32_t(neg)) - uint32_t(neg));
  const uint32_t sp = mag == 0u ? uint32_t(kWinZero)
                      : mag < uint32_t(kWinELo << 7) ? tiny
                      : bits == 0xff80u ? 0u : uint32_t(kWinOther);
  return off2 - 2u < uint32_t(kWinHalf) ? wb : sp;
}

// One row (b, r) of the window pass, by the whole workgroup; its partial goes
// to parts[b (2K + 1) + r]. The workgroup's LDS is free again after a
// barrier.
template <int VEC>
__device__ __forceinline__ void trunc_win_row(const void* __restrict__ target,
                                              const void* __restrict__ draft, int b, int r,
                                              int K, int V, float c, double c64, const Trunc& tr,
                                              RowPart* __restrict__ parts) {
  using C = Chunk<DT_BF16, VEC>;
  __shared__ uint32_t H[kWinBins];
  __shared__ uint32_t s_u[kTwWaves];
  __shared__ int s_i[kTwWaves];
  __shared__ double s_d[kTwWaves];
  __shared__ uint32_t s_key;
  __shared__ double s_S;
  const int tid = threadIdx.x;
  const int rows = 2 * K + 1;
  const long long grow = (long long)b * rows + r;
  const void* row = row_ptr<DT_BF16>(target, draft, b, r, K, V);

  // ---- 1. count: groups of U chunks per thread, the next group's loads
  // issued before the current group is counted ----
  for (int i = tid; i < kWinBins / 4; i += kTwBlock)
    reinterpret_cast<u32x4*>(H)[i] = (u32x4){0u, 0u, 0u, 0u};
  __syncthreads();
  {
    constexpr int U = 4;
    using raw_t = typename C::raw_t;
    const long long nchunks = V / VEC;
    const long long span = (long long)U * kTwBlock;
    const long long first = nchunks - tid - (long long)(U - 1) * kTwBlock;
    const long long G = first > 0 ? (first + span - 1) / span : 0;   // whole groups
    auto load_group = [&](long long g, raw_t (&a)[U]) {
#pragma unroll
      for (int u = 0; u < U; ++u) a[u] = C::load(row, tid + g * span + (long long)u * kTwBlock);
    };
    // a chunk whose 8 values all lie in the window takes the short bin
    // formula; any other chunk classifies each value
    auto count_chunk = [&](const raw_t& raw) {
      if constexpr (VEC == 8) {
        // both values of a word at once in packed 16-bit lanes (low half
        // first): o = |x| pattern - (window base - 2), which wraps far above
        // the window for values below it
        u16x2 o[4], worst2 = {0, 0};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // bit-cast a scalar copy: the cast of a vector element reads element 0
          const uint32_t w = raw[q];
          const u16x2 v = __builtin_bit_cast(u16x2, w);
          o[q] = (v & (u16x2)(0x7fff)) - (u16x2)(uint16_t((kWinELo << 7) - 2));
          worst2 = __builtin_elementwise_max(worst2, o[q] - (u16x2)(2));
        }
        if (max(uint32_t(worst2.x), uint32_t(worst2.y)) < uint32_t(kWinHalf)) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t w = raw[q];
            const u16x2 v = __builtin_bit_cast(u16x2, w);
            const u16x2 neg = (u16x2)(0) - (v >> (u16x2)(15));   // 0xffff where negative
            const u16x2 bin = (u16x2)(uint16_t(kWinZero)) + ((o[q] ^ neg) - neg);
            atomicAdd(&H[bin.x], 1u);
            atomicAdd(&H[bin.y], 1u);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            atomicAdd(&H[win_bin((e & 1) ? raw[e >> 1] >> 16 : raw[e >> 1] & 0xffffu)], 1u);
        }
      } else {
        atomicAdd(&H[win_bin(raw)], 1u);
      }
      __builtin_amdgcn_sched_barrier(0);   // one chunk's bins at a time
    };
    if (G > 0) {
      raw_t a[U];
      load_group(0, a);
      for (long long g = 0; g + 1 < G; ++g) {
        raw_t n[U];
        load_group(g + 1, n);
#pragma unroll
        for (int u = 0; u < U; ++u) count_chunk(a[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) a[u] = n[u];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) count_chunk(a[u]);
    }
    for (long long ci = tid + G * span; ci < nchunks; ci += kTwBlock) count_chunk(C::load(row, ci));
  }
  __syncthreads();
  // rows this pass does not finish go to the full pass (uniform decisions)
  auto hand_over = [&]() {
    if (tid == 0) {
      RowPart p;
      p.S = __builtin_nan("");
      p.R = 0.0f;
      p.m = 0.0f;
      p.idx = 0;
      p.flags = kTruncRedo;
      parts[grow] = p;
    }
  };
  if (H[kWinOther] != 0u) {          // values outside the window
    hand_over();
    return;
  }
  const bool tiny_vals = H[kTinyNeg] + H[kTinyPos] != 0u;

  // ---- 2. this thread's levels: bins 16t + 15 down to 16t ----
  const int bin0 = tid * kBinsPerThread;
  uint32_t cnt[kBinsPerThread];
#pragma unroll
  for (int q = 0; q < kBinsPerThread / 4; ++q) {
    const u32x4 v = reinterpret_cast<const u32x4*>(H)[tid * (kBinsPerThread / 4) + q];
    cnt[4 * q] = v[0];
    cnt[4 * q + 1] = v[1];
    cnt[4 * q + 2] = v[2];
    cnt[4 * q + 3] = v[3];
  }
  uint32_t n_t = 0;
  int top_t = -1;                    // highest occupied bin above -inf
#pragma unroll
  for (int j = 0; j < kBinsPerThread; ++j) {
    n_t += cnt[j];
    if (cnt[j] != 0u && bin0 + j > 0) top_t = bin0 + j;
  }
  const int top_bin = tr_max<kTwWaves>(top_t, s_i);
  if (top_bin == kTinyNeg || top_bin == kTinyPos) {   // the maximum is a tiny value
    hand_over();
    return;
  }
  bool bad = top_bin < 0;            // no finite value
  const float R = bad ? 0.0f : ceilf(key_value(win_key(top_bin)) * c);

  // Masses of the tiny-value bins. Each such value's term is 2^(x c - R)
  // with |x c| < 2^-24 c: for c <= 4 (temperatures above about 0.36) it is
  // 2^-R to within 1.7e-7 relative, the level terms' own accuracy, and the
  // bin mass is its count times 2^-R; otherwise every value's term is summed
  // in a second read of the row.
  double tmass[2] = {0.0, 0.0};      // [negative, positive]
  if (tiny_vals && !bad && c64 <= 4.0) {
    const double z = level_term(0x8000u, c64, R);
    tmass[0] = double(H[kTinyNeg]) * z;
    tmass[1] = double(H[kTinyPos]) * z;
  } else if (tiny_vals && !bad) {
    const long long nchunks = V / VEC;
    double mn = 0.0, mp = 0.0;
    for (long long ci = tid; ci < nchunks; ci += kTwBlock) {
      const typename C::raw_t raw = C::load(row, ci);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        uint32_t bits;
        if constexpr (VEC == 8)
          bits = (e & 1) ? raw[e >> 1] >> 16 : raw[e >> 1] & 0xffffu;
        else
          bits = raw;
        const uint32_t mag = bits & 0x7fffu;
        if (mag != 0u && mag < uint32_t(kWinELo << 7)) {
          const double t = level_term(bf16_key(bits), c64, R);
          if (bits & 0x8000u)
            mn += t;
          else
            mp += t;
        }
      }
    }
    tmass[0] = tr_sum<double, kTwWaves>(mn, s_d);
    tmass[1] = tr_sum<double, kTwWaves>(mp, s_d);
  }
  // mass of bin i at the reference R; it and the sums below are never
  // fused, so the mass loop and the top-p walk give bitwise-equal partial
  // sums
  auto bin_mass = [&](int i, uint32_t n) -> double {
#pragma clang fp contract(off)
    if (i == kTinyNeg) return tmass[0];
    if (i == kTinyPos) return tmass[1];
    return double(n) * level_term(win_key(i), c64, R);
  };

  // ---- 3. top-k threshold bin from the counts (one thread holds the cut) ----
  const int kk = tr.k != nullptr ? tr.k[b] : 0;
  int tk = 0;                        // smallest kept bin
  if (kk >= 1 && kk < V) {
    uint32_t n_all;
    const uint32_t above = tr_above<uint32_t, kTwWaves>(n_t, s_u, n_all);
    if (above < uint32_t(kk) && above + n_t >= uint32_t(kk)) {
      uint32_t acc = above;
      int cut = bin0;
      bool found = false;
#pragma unroll
      for (int j = kBinsPerThread - 1; j >= 0; --j) {
        acc += cnt[j];
        if (!found && acc >= uint32_t(kk)) {
          cut = bin0 + j;
          found = true;
        }
      }
      s_key = uint32_t(cut);
    }
    __syncthreads();
    tk = int(s_key);
    __syncthreads();
    if (tk == kTinyNeg || tk == kTinyPos) {   // the k-th value is a tiny one
      hand_over();
      return;
    }
  }

  // ---- 4. level masses at or above the top-k threshold, S_k (the top-p
  // walk repeats these operations in the same order) ----
  double M_t = 0.0;
#pragma unroll
  for (int j = kBinsPerThread - 1; j >= 0; --j) {
    if (cnt[j] != 0u && bin0 + j > 0 && bin0 + j >= tk) {
#pragma clang fp contract(off)
      M_t = M_t + bin_mass(bin0 + j, cnt[j]);
    }
  }
  double S_k;
  const double above_m = tr_above<double, kTwWaves>(M_t, s_d, S_k);

  // ---- 5. top-p threshold bin from the masses ----
  const float pp = tr.p != nullptr ? tr.p[b] : 1.0f;
  bad = bad || !(pp > 0.0f);
  int thr = tk;
  double S_tr = S_k;
  if (pp < 1.0f && !bad) {
    const double goal = double(pp) * S_k;
    const int cut = tr_max<kTwWaves>(above_m + M_t >= goal ? tid : -1, s_i);
    if (cut >= 0) {
      if (tid == cut) {
        double part = 0.0;
        bool found = false;
        int last = bin0;
#pragma unroll
        for (int j = kBinsPerThread - 1; j >= 0; --j) {
          if (cnt[j] != 0u && bin0 + j > 0 && bin0 + j >= tk) {
            {
#pragma clang fp contract(off)
              part = part + bin_mass(bin0 + j, cnt[j]);
            }
            last = bin0 + j;
            if (!found && above_m + part >= goal) {
              s_key = uint32_t(bin0 + j);
              s_S = above_m + part;
              found = true;
            }
          }
        }
        if (!found) {                // equal partial sums make this unreachable
          s_key = uint32_t(last);
          s_S = above_m + part;
        }
      }
      __syncthreads();
      thr = int(s_key);
      S_tr = s_S;
      if (thr == kTinyNeg || thr == kTinyPos) {   // the top-p cut is inside a tiny bin
        hand_over();
        return;
      }
    }
  }
  if (tid == 0) {
    RowPart p;
    p.S = bad ? __builtin_nan("") : S_tr;
    p.R = R;
    p.m = 0.0f;
    p.idx = int(win_key(thr));
    p.flags = 0;
    parts[grow] = p;
  }
}

// The window pass, one workgroup per row that sel selects: every needed row
// of every sequence, or with walk-order reading position 0's rows of every
// sequence and then the other rows of the listed sequences (a grid sized for
// every sequence: the workgroups past the listed rows return at once).
// Workgroup 0 clears the histogram and, when set, the list count.
template <int VEC>
__global__ __launch_bounds__(kTwBlock) void rowstats_trunc_win(
    const void* __restrict__ target, const void* __restrict__ draft, int B, int K, int V,
    float c, double c64, Trunc tr, const int32_t* __restrict__ kdraft,
    RowPart* __restrict__ parts, uint32_t* __restrict__ hist, RowSel sel,
    uint32_t* __restrict__ clear) {
  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && hist != nullptr && tid <= K) hist[tid] = 0u;
  if (blockIdx.x == 0 && clear != nullptr && tid == 0) *clear = 0u;
  if ((long long)blockIdx.x >= sel.total(B)) return;
  int b, r;
  sel.at(blockIdx.x, K, b, r);
  if (kdraft != nullptr) {           // rows past the draft count are not needed
    const int kb = kdraft[b];
    if (r <= K ? r > kb : r - K - 1 >= kb) return;
  }
  trunc_win_row<VEC>(target, draft, b, r, K, V, c, c64, tr, parts);
}

// Walk-order reading of truncated bf16 calls, after both truncation passes
// over position 0's rows: lists the sequences whose walk keeps position 0
// and that have rows past it (k_b >= 1), one thread per sequence, with the
// scan's own truncated acceptance test (trunc_accept_bf16).
__global__ __launch_bounds__(kBlock) void walk_gate_trunc(
    int B, int K, int V, const RowPart* __restrict__ parts, const void* __restrict__ target,
    const void* __restrict__ draft, const int32_t* __restrict__ kdraft,
    const int32_t* __restrict__ tokens, const float* __restrict__ uniforms, double c64,
    int32_t* __restrict__ seqs, uint32_t* __restrict__ count) {
  const int b = int(blockIdx.x) * kBlock + int(threadIdx.x);
  if (b >= B) return;
  const int kb = kdraft != nullptr ? kdraft[b] : K;
  if (!(kb >= 1 && kb <= K)) return;
  const int rows = 2 * K + 1;
  const RowPart pt = parts[(long long)b * rows];
  const RowPart pd = parts[(long long)b * rows + K + 1];
  const int d = tokens[(long long)b * K];
  if (!(finite_pos(pt.S) && finite_pos(pd.S) && d >= 0 && d < V)) return;
  const float xt = load_logit<DT_BF16>(row_ptr<DT_BF16>(target, draft, b, 0, K, V), d);
  const float xd = load_logit<DT_BF16>(row_ptr<DT_BF16>(target, draft, b, K + 1, K, V), d);
  double P, Q;
  if (trunc_accept_bf16(xt, xd, pt.R, pt.S, uint32_t(pt.idx), pd.R, pd.S, uint32_t(pd.idx),
                        double(uniforms[(long long)b * (K + 1)]), c64, P, Q))
    seqs[atomicAdd(count, 1u)] = b;
}

}  // namespace sv
