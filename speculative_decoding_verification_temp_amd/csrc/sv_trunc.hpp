// Top-k / top-p truncation pass over bf16 logit rows (gfx950).
//
// p and q are the distributions the samplers really use, after temperature
// and truncation, and the same truncation has to hold in the acceptance ratio,
// the residual and the bonus draw ([RNR] s.1 and s.2). The rules: top-k keeps
// the values at or above the k-th largest (counted with multiplicity, so ties
// at the cut stay); top-p then keeps, from the top, whole value levels up to
// and including the first level at which the kept mass reaches top_p of the
// top-k mass.
//
// One 1024-thread workgroup per needed row (target rows 0..k_b, draft rows
// 0..k_b-1) reads the row once and counts its values into an exact histogram
// over the 65536 order-preserving 16-bit keys (bf16_key), held in LDS as
// 16-bit counters, two to a 32-bit word (128 KiB). Every value of one level
// has the same softmax term, so the histogram gives all the truncation needs:
//   * the row maximum and the integer reference R = ceil(max * c);
//   * top-k: the threshold is the level at which the count of values at or
//     above it, from the top, first reaches k;
//   * level masses count * 2^(x c - R), the top-k normaliser S_k, and top-p:
//     the threshold is the level at which the mass at or above it, from the
//     top, first reaches top_p * S_k;
//   * the truncated normaliser: the mass at or above the final threshold.
// Output: one RowPart per row with S = truncated normaliser (relative to
// 2^R), R, idx = threshold key. A row holding NaN or +inf, or without a
// finite maximum, or a sequence whose top_p is not > 0, gets S = NaN, which
// makes the sequence invalid in the scan.
//
// A 16-bit counter wraps only when one value occurs more than 65535 times in
// the row. The first count adds without looking; the counts are then summed
// and compared with V. On a mismatch the row is counted again, in two passes
// with returning atomics: first only the even keys (low halves), where a
// wrap's carry into the still-empty high half is taken back at once, then
// only the odd keys (high halves), whose carries leave the word. Each wrap is
// recorded in a short list (65536 more for that key); as the halves are never
// counted at the same time, no count sees another half's carry. A row that
// still does not add up (more wraps than the list holds) is marked invalid.
#pragma once

#include "sv_fused.hpp"

namespace sv {

constexpr int kTrBlock = 1024;
constexpr int kTrWaves = kTrBlock / kWave;
constexpr int kHistWords = 32768;                    // 65536 16-bit counters
constexpr int kKeysPerThread = 65536 / kTrBlock;     // 64 consecutive keys per thread
constexpr int kMaxWraps = 32;

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

// ---- workgroup reductions over the 16 wavefronts (fixed order) ----
template <typename T_>
__device__ inline T_ tr_sum(T_ v, T_* s) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  if (lane == 0) s[wid] = v;
  __syncthreads();
  T_ t = 0;
#pragma unroll
  for (int w = 0; w < kTrWaves; ++w) t += s[w];
  __syncthreads();
  return t;
}

__device__ inline int tr_max(int v, int* s) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
  if (lane == 0) s[wid] = v;
  __syncthreads();
  int t = s[0];
#pragma unroll
  for (int w = 1; w < kTrWaves; ++w) t = max(t, s[w]);
  __syncthreads();
  return t;
}

// Sum of v over the threads with a larger index (= the higher keys), and the
// total over all threads.
template <typename T_>
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
  for (int w = kTrWaves - 1; w >= 0; --w) {
    if (w > wid) hi += s[w];
    tot += s[w];
  }
  __syncthreads();
  total = tot;
  return hi + excl;
}

template <int VEC>
__global__ __launch_bounds__(kTrBlock) void rowstats_trunc(
    const void* __restrict__ target, const void* __restrict__ draft, int K, int V, float c,
    double c64, Trunc tr, const int32_t* __restrict__ kdraft, RowPart* __restrict__ parts,
    uint32_t* __restrict__ hist) {
  __shared__ uint32_t H[kHistWords];
  __shared__ uint32_t s_wraps[kMaxWraps];
  __shared__ uint32_t s_nwrap;
  __shared__ uint32_t s_u[kTrWaves];
  __shared__ int s_i[kTrWaves];
  __shared__ double s_d[kTrWaves];
  __shared__ uint32_t s_key;
  __shared__ double s_S;
  const int tid = threadIdx.x;
  const int rows = 2 * K + 1;
  const long long grow = blockIdx.x;
  const int b = int(grow / rows), r = int(grow % rows);
  if (blockIdx.x == 0 && hist != nullptr && tid <= K) hist[tid] = 0u;
  if (kdraft != nullptr) {           // rows past the draft count are not needed
    const int kb = kdraft[b];
    if (r <= K ? r > kb : r - K - 1 >= kb) return;
  }
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

}  // namespace sv
