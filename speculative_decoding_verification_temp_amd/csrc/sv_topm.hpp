// Order keys of logits and top-m selection over logit rows by
// wavefront-private candidate lists (gfx950).
//
// Token v of a row is ranked by the key
//   (order-preserving key of its logit << 32) | (2^32 - 1 - v),
// 48 bits for bf16 logits (16-bit order key), 64 for fp32 (32-bit),
// so a larger logit comes first, equal logits fall to the lower index, and no
// two tokens share a key: the row's top m tokens are its m largest keys. A
// wavefront appends the keys that reach its threshold to a list in LDS; when
// the list is nearly full it finds the m-th largest key in it (byte-wise
// radix select) and keeps only the keys at or above it, which becomes its
// threshold. The m-th largest key of any part of a row is at most the row's
// m-th largest, so no top-m token is ever dropped, and the wavefronts of a
// workgroup may share their thresholds through one LDS word. Filtering costs
// a float compare per value: a logit's order key reaches the threshold's
// upper 32 bits exactly when the logit, as a float, is at least the value
// those bits encode.
#pragma once

#include "sv_device.hpp"

namespace sv {

// Order-preserving 16-bit key of a bf16 value (bits = its 16-bit pattern):
// 0x8000 + |x| for x >= 0, 0x8000 - |x| for x < 0 (|x| as the 15-bit pattern),
// so larger values have larger keys and -0 shares the key of +0. Keys run
// from 1 (the largest negative NaN) to 0xffff; finite values lie in
// [0x81, 0xff7f], -inf is 0x80 and +inf 0xff80. A truncated row keeps the
// values whose key is at least its threshold key; threshold 0 keeps all.
__device__ inline uint32_t bf16_key(uint32_t bits) {
  const uint32_t mag = bits & 0x7fffu;
  return (bits & 0x8000u) ? 0x8000u - mag : 0x8000u + mag;
}
constexpr uint32_t kKeyNegInf = 0x80u, kKeyPosInf = 0xff80u;

// the bf16 value of a key
__device__ inline float key_value(uint32_t key) {
  const uint32_t bits = key >= 0x8000u ? key - 0x8000u : (0x8000u | (0x8000u - key));
  return __uint_as_float(bits << 16);
}

__device__ inline bool key_finite(uint32_t key) { return key > kKeyNegInf && key < kKeyPosInf; }

// the least float whose bf16 key reaches `key` (-inf for keys up to -inf's)
__device__ inline float key_floor(uint32_t key) {
  return key <= kKeyNegInf ? -__builtin_inff() : key_value(key);
}

// Order key of a logit of type DT from its bits, the bf16 construction on 32
// bits for fp32 (-0 and +0 alike); keys are never 0 for non-NaN values.
template <int DT>
__device__ inline uint32_t order_key(uint32_t bits) {
  if constexpr (DT == DT_BF16) {
    return bf16_key(bits);
  } else {
    const uint32_t mag = bits & 0x7fffffffu;
    return (bits & 0x80000000u) ? 0x80000000u - mag : 0x80000000u + mag;
  }
}

// the least float whose order key reaches `key` (-inf for keys up to -inf's)
template <int DT>
__device__ inline float order_floor(uint32_t key) {
  if constexpr (DT == DT_BF16) {
    return key_floor(key);
  } else {
    constexpr uint32_t kNegInfKey = 0x80000000u - 0x7f800000u;
    if (key <= kNegInfKey) return -__builtin_inff();
    const uint32_t bits = key >= 0x80000000u ? key - 0x80000000u : 0x80000000u | (0x80000000u - key);
    return __uint_as_float(bits);
  }
}

// the shift of the top byte of a token key
template <int DT>
constexpr int key_top_shift() {
  return DT == DT_BF16 ? 40 : 56;
}

// LDS written by some lanes of a wavefront, then read by others
__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// active lanes of `mask` below this lane
__device__ inline uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u));
}

// The want-th largest (1 <= want <= n) of the n distinct keys buf[0..n), all
// below 2^(top_shift + 8), by byte-wise radix select from the top byte down: each round
// counts the keys that match the bytes chosen so far into 256 bins private to
// the wavefront and walks the bins from the top; it stops as soon as a single
// key is left. Called by all 64 lanes of one wavefront.
__device__ inline uint64_t wave_kth_largest(const uint64_t* buf, int n, uint32_t want,
                                            uint32_t* bins, int top_shift) {
  const int lane = threadIdx.x & (kWave - 1);
  uint64_t prefix = 0, pmask = 0;
#pragma unroll 1
  for (int shift = top_shift; shift >= 0; shift -= 8) {
    for (int q = lane; q < 256; q += kWave) bins[q] = 0u;
    wave_sync();
    for (int e = lane; e < n; e += kWave) {
      const uint64_t v = buf[e];
      if ((v & pmask) == prefix) atomicAdd(&bins[uint32_t(v >> shift) & 255u], 1u);
    }
    wave_sync();
    // lane L walks bins 255 - 4L down to 252 - 4L; lanes in order cover 255..0
    uint32_t c[4], s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[j] = bins[255 - 4 * lane - j];
      s += c[j];
    }
    uint32_t incl = s;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const uint32_t u = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += u;
    }
    const uint32_t excl = incl - s;
    const bool mine = excl < want && incl >= want;   // exactly one lane
    uint32_t byte = 0, above = 0, at = 0;
    if (mine) {
      uint32_t acc = excl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (at == 0u && acc + c[j] >= want) {
          byte = uint32_t(255 - 4 * lane - j);
          above = acc;
          at = c[j];
        }
        acc += c[j];
      }
    }
    const int src = __ffsll((unsigned long long)__ballot(mine)) - 1;
    byte = __shfl(byte, src, kWave);
    above = __shfl(above, src, kWave);
    at = __shfl(at, src, kWave);
    want -= above;
    prefix |= uint64_t(byte) << shift;
    pmask |= uint64_t(255) << shift;
    wave_sync();                                     // bins are cleared next round
    if (at == 1u) {
      uint64_t r = 0;
      for (int e = lane; e < n; e += kWave) {
        const uint64_t v = buf[e];
        if ((v & pmask) == prefix) r = v;
      }
#pragma unroll
      for (int o = kWave / 2; o > 0; o >>= 1) {
        const uint64_t u = __shfl_xor(r, o, kWave);
        r = u > r ? u : r;
      }
      return r;
    }
  }
  return prefix;
}

// Values of a 16-byte chunk of logits: 8 bf16 (low half of each word first)
// or 4 fp32.
template <int DT> struct ChunkVals;
template <> struct ChunkVals<DT_BF16> {
  static constexpr int N = 8;
  // value e as a float (e known at compile time)
  __device__ static float value(const u32x4& r, int e) {
    return __uint_as_float((e & 1) ? r[e >> 1] & 0xffff0000u : r[e >> 1] << 16);
  }
  // bits of value e (e may differ between lanes)
  __device__ static uint32_t bits(const u32x4& r, int e) {
    const uint32_t w = (e & 4) ? ((e & 2) ? r[3] : r[2]) : ((e & 2) ? r[1] : r[0]);
    return (e & 1) ? w >> 16 : w & 0xffffu;
  }
};
template <> struct ChunkVals<DT_F32> {
  static constexpr int N = 4;
  __device__ static float value(const u32x4& r, int e) { return __uint_as_float(r[e]); }
  __device__ static uint32_t bits(const u32x4& r, int e) {
    return (e & 2) ? ((e & 1) ? r[3] : r[2]) : ((e & 1) ? r[1] : r[0]);
  }
};

// the values of a chunk at or above thr_f, as bits 0..N-1
template <int DT>
__device__ inline uint32_t chunk_pend(const u32x4& r, float thr_f) {
  uint32_t pend = 0;
#pragma unroll
  for (int e = 0; e < ChunkVals<DT>::N; ++e)
    pend |= ChunkVals<DT>::value(r, e) >= thr_f ? 1u << e : 0u;
  return pend;
}

// the largest value of a chunk (NaN values ignored)
template <int DT>
__device__ inline float chunk_max(const u32x4& r) {
  float mx = ChunkVals<DT>::value(r, 0);
#pragma unroll
  for (int e = 1; e < ChunkVals<DT>::N; ++e) mx = fmaxf(mx, ChunkVals<DT>::value(r, e));
  return mx;
}

constexpr int kTopmStage = 128;   // staged chunks per wavefront

// The candidate list of one wavefront over logits of type DT. Every member
// function is called by all 64 lanes of the wavefront together; fill, thr,
// thr_f and nstage are the same in every lane. Chunks whose largest value
// reaches the threshold are first staged in LDS (kTopmStage per wavefront)
// and filtered 64 at a time, one per lane, so that the insert rounds run
// with every lane busy whichever lanes found the candidates.
template <int DT>
struct TopM {
  uint64_t* keys;              // cap entries of LDS
  uint32_t* bins;              // 256 words of LDS
  unsigned long long* shared;  // the workgroup's threshold (LDS)
  uint32_t cap, want;          // list size (>= want + 64, and >= 64 N for seed<N>); m
  uint32_t fill;
  uint64_t thr;                // keys below it cannot be among the m largest
  float thr_f;                 // order_floor of thr's logit key
  u32x4* stage;                // kTopmStage staged chunks (LDS)
  uint32_t* stage_at;          // their chunk indexes in the row
  uint32_t nstage;

  __device__ void init(uint64_t* k, uint32_t* b, unsigned long long* s, uint32_t c, uint32_t w,
                       u32x4* st = nullptr, uint32_t* st_at = nullptr) {
    keys = k;
    bins = b;
    shared = s;
    cap = c;
    want = w;
    fill = 0;
    thr = 0;
    thr_f = -__builtin_inff();
    stage = st;
    stage_at = st_at;
    nstage = 0;
  }

  // keep the keys at or above max(the want-th largest key, the shared threshold)
  __device__ void compact() {
    const int lane = threadIdx.x & (kWave - 1);
    uint64_t t = thr;
    if (fill > want) {
      const uint64_t kth = wave_kth_largest(keys, int(fill), want, bins, key_top_shift<DT>());
      t = kth > t ? kth : t;
      if (lane == 0) atomicMax(shared, (unsigned long long)t);
    }
    const uint64_t sh = __hip_atomic_load(shared, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    t = sh > t ? sh : t;
    uint32_t out = 0;          // in place: a key moves only to a lower slot
    for (uint32_t base = 0; base < fill; base += kWave) {
      const uint32_t e = base + uint32_t(lane);
      const uint64_t v = e < fill ? keys[e] : 0ull;
      const bool keep = e < fill && v >= t;
      const uint64_t mask = __ballot(keep);
      if (keep) keys[out + lanes_below(mask)] = v;
      out += uint32_t(__popcll(mask));
    }
    wave_sync();
    fill = out;
    thr = t;
    thr_f = order_floor<DT>(uint32_t(t >> 32));
  }

  // Offer the values of one chunk whose bits in `pend` are set (value e has
  // index idx0 + e and logit bits bits_of(e)); one value per lane and round,
  // as many rounds as the busiest lane needs.
  template <class BitsOf>
  __device__ void offer(uint32_t pend, BitsOf bits_of, long long idx0) {
    while (__ballot(pend != 0u) != 0ull) {
      if (fill > cap - uint32_t(kWave)) compact();
      const bool act = pend != 0u;
      const int e = act ? __builtin_ctz(pend) : 0;
      pend &= pend - 1u;
      const uint64_t k =
          (uint64_t(order_key<DT>(bits_of(e))) << 32) | uint64_t(~uint32_t(idx0 + e));
      const bool put = act && k >= thr;
      const uint64_t mask = __ballot(put);
      if (put) keys[fill + lanes_below(mask)] = k;
      fill += uint32_t(__popcll(mask));
    }
  }

  // Start the threshold from values already at hand: the want-th largest of
  // v[q] over the lanes (slots q with bit q of `ok` set), each taken with the
  // lowest key its value can have, is at most the row's want-th largest
  // token key. Needs an empty list; chunk maxima are the usual v.
  template <int N>
  __device__ void seed(const float (&v)[N], uint32_t ok) {
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t n = 0;
#pragma unroll
    for (int q = 0; q < N; ++q) {
      const bool put = ((ok >> q) & 1u) != 0u && v[q] == v[q];
      const uint32_t bits =
          DT == DT_BF16 ? __float_as_uint(v[q]) >> 16 : __float_as_uint(v[q]);
      const uint64_t mask = __ballot(put);
      if (put) keys[n + lanes_below(mask)] = uint64_t(order_key<DT>(bits)) << 32;
      n += uint32_t(__popcll(mask));
    }
    wave_sync();
    if (n >= want) {
      const uint64_t t = wave_kth_largest(keys, int(n), want, bins, key_top_shift<DT>());
      if (t > thr) {
        thr = t;
        thr_f = order_floor<DT>(uint32_t(t >> 32));
        if (lane == 0) atomicMax(shared, (unsigned long long)t);
      }
    }
    wave_sync();
  }

  // Stage this lane's 16-byte chunk number `at` of the row (values of
  // indexes E at .. E at + E - 1) when `cand`; filter the staged chunks once
  // fewer than 64 slots are free.
  __device__ void stage_chunk(bool cand, const u32x4& ch, uint32_t at) {
    const uint64_t mask = __ballot(cand);
    if (mask == 0ull) return;
    if (cand) {
      const uint32_t slot = nstage + lanes_below(mask);
      stage[slot] = ch;
      stage_at[slot] = at;
    }
    nstage += uint32_t(__popcll(mask));
    if (nstage > uint32_t(kTopmStage - kWave)) flush();
  }

  // Filter every staged chunk against the current threshold, one per lane.
  __device__ void flush() {
    const int lane = threadIdx.x & (kWave - 1);
    wave_sync();
    for (uint32_t base = 0; base < nstage; base += kWave) {
      const uint32_t e = base + uint32_t(lane);
      const bool has = e < nstage;
      u32x4 ch = {0u, 0u, 0u, 0u};
      uint32_t at = 0;
      if (has) {
        ch = stage[e];
        at = stage_at[e];
      }
      const uint32_t pend = has ? chunk_pend<DT>(ch, thr_f) : 0u;
      offer(pend, [&](int q) { return ChunkVals<DT>::bits(ch, q); },
            (long long)at * ChunkVals<DT>::N);
    }
    nstage = 0;
    wave_sync();
  }
};

// The residual side output of one drafted position from its support: the
// `mm` keys keys[0..mm) (the draft row's top mm tokens, any order) are ranked
// by key, and at rank r the token and
//   (x_t(v)/T - LSE_S(x_t/T)) - (x_d(v)/T - LSE_S(x_d/T))
// are written; slots mm..m-1 get -1 and NaN. One whole wavefront; mm <= 64.
template <int DT>
__device__ inline void support_residual(const uint64_t* keys, uint32_t mm, const void* drow,
                                        const void* trow, double invT, int m,
                                        int32_t* __restrict__ out_support,
                                        double* __restrict__ out_res) {
  const int lane = threadIdx.x & (kWave - 1);
  const bool has = uint32_t(lane) < mm;
  const uint64_t key = has ? keys[lane] : 0ull;
  int rank = 0;
  for (int o = 0; o < int(mm); ++o) {
    const uint64_t ko = __shfl(key, o, kWave);
    rank += (has && ko > key) ? 1 : 0;
  }
  const int v = has ? int(~uint32_t(key)) : -1;
  const double ad = has ? double(load_logit<DT>(drow, v)) * invT : -__builtin_inf();
  const double at = has ? double(load_logit<DT>(trow, v)) * invT : -__builtin_inf();
  double mt = at, md = ad;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    mt = fmax(mt, __shfl_xor(mt, o, kWave));
    md = fmax(md, __shfl_xor(md, o, kWave));
  }
  const double lse_t = mt + log(wave_sum(has ? exp(at - mt) : 0.0));
  const double lse_d = md + log(wave_sum(has ? exp(ad - md) : 0.0));
  if (has) {
    out_support[rank] = v;
    out_res[rank] = (at - lse_t) - (ad - lse_d);
  } else if (lane < m) {
    out_support[lane] = -1;
    out_res[lane] = __builtin_nan("");
  }
}

}  // namespace sv
