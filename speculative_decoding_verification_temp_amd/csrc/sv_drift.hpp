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
// One 256-thread workgroup per (sequence, drafted position i < k_b) of a
// valid sequence (the scan's accept length is read to tell) reads the draft
// row once. Token v is ranked by the 48-bit key
//   (order-preserving bf16 key << 32) | (2^32 - 1 - v),
// so a larger logit comes first, equal logits fall to the lower index, and no
// two tokens share a key: the support is the m largest keys. Each wavefront
// appends the keys that reach its threshold to an LDS list; before the list
// could overflow it finds the m-th largest key in it (byte-wise radix select)
// and keeps only the keys at or above it, which becomes its new threshold.
// The m-th largest key of any part of the row is at most the row's m-th
// largest, so no support token is ever dropped, and the wavefronts may share
// their thresholds through one LDS word. The common case, a chunk with no key
// at the threshold, costs a float compare per value: a bf16 key reaches the
// threshold's upper 16 bits exactly when the value, widened to float, is at
// least the value those bits encode. At the end wavefront 0 merges the
// four lists, keeps the m largest keys, ranks them and forms the two float64
// log-sum-exps over them.
#pragma once

#include "sv_kernels.hpp"

namespace sv {

constexpr int kDriftMaxM = 64;
constexpr int kDriftBlock = 256;
constexpr int kDriftWaves = kDriftBlock / kWave;
constexpr int kDriftCap = 1024;      // keys per wavefront list
constexpr int kDriftUnroll = 4;      // chunks per thread per group (two groups in flight)

// LDS written by some lanes of a wavefront, then read by others
__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// the float a bf16 key stands for (-inf for keys at or below -inf's)
__device__ inline float key_float(uint32_t key) {
  const uint32_t bits = key >= 0x8000u ? key - 0x8000u : 0x8000u | min(0x8000u - key, 0x7f80u);
  return __uint_as_float(bits << 16);
}

// active lanes of `mask` below this lane
__device__ inline uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u));
}

// The want-th largest (1 <= want <= n) of the n distinct keys buf[0..n), all
// below 2^48, by byte-wise radix select from the top byte down: each round
// counts the keys that match the bytes chosen so far into 256 bins private to
// the wavefront and walks the bins from the top; it stops as soon as a single
// key is left. Called by all lanes of one wavefront.
__device__ inline uint64_t wave_kth_largest(const uint64_t* buf, int n, uint32_t want,
                                            uint32_t* bins) {
  const int lane = threadIdx.x & (kWave - 1);
  uint64_t prefix = 0, pmask = 0;
#pragma unroll 1
  for (int shift = 40; shift >= 0; shift -= 8) {
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

template <int VEC>
__global__ __launch_bounds__(kDriftBlock) void drift_residual(
    const void* __restrict__ target, const void* __restrict__ draft, int K, int V, double invT,
    int m, const int32_t* __restrict__ kdraft, const int32_t* __restrict__ accept_len,
    int32_t* __restrict__ out_support, double* __restrict__ out_res) {
  using C = Chunk<DT_BF16, VEC>;
  __shared__ uint64_t s_keys[kDriftWaves][kDriftCap];
  __shared__ uint32_t s_bins[kDriftWaves][256];
  __shared__ uint32_t s_count[kDriftWaves];
  __shared__ unsigned long long s_thr;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int b = int(blockIdx.x) / K, i = int(blockIdx.x) % K;
  const long long o0 = ((long long)b * K + i) * m;
  const int kb = kdraft != nullptr ? kdraft[b] : K;
  if (accept_len[b] < 0 || i >= kb) {          // no residual here (uniform)
    if (tid < m) {
      out_support[o0 + tid] = -1;
      out_res[o0 + tid] = __builtin_nan("");
    }
    return;
  }
  const void* drow = row_ptr<DT_BF16>(target, draft, b, K + 1 + i, K, V);
  const void* trow = row_ptr<DT_BF16>(target, draft, b, i, K, V);
  const uint32_t mm = uint32_t(min(m, V));
  if (tid == 0) s_thr = 0ull;
  __syncthreads();

  uint64_t* keys = s_keys[wid];
  uint32_t* bins = s_bins[wid];
  uint32_t fill = 0;           // wavefront-uniform
  uint64_t thr = 0;            // keys below it cannot be in the support
  float thr_f = key_float(0u); // the value of thr's bf16 key
  // keep the keys at or above max(the want-th largest key, the shared threshold)
  auto compact = [&](uint32_t want) {
    uint64_t t = thr;
    if (fill > want) {
      const uint64_t kth = wave_kth_largest(keys, int(fill), want, bins);
      t = kth > t ? kth : t;
      if (lane == 0) atomicMax(&s_thr, (unsigned long long)t);
    }
    const uint64_t shared =
        __hip_atomic_load(&s_thr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    t = shared > t ? shared : t;
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
    thr_f = key_float(uint32_t(t >> 32));
  };

  // ---- one read of the draft row; the next group's loads are in flight
  // while a group is filtered (indexes past the row are clamped to its last
  // chunk and ignored) ----
  const long long nchunks = V / VEC;
  constexpr long long kPerIt = (long long)kDriftBlock * kDriftUnroll;
  constexpr uint32_t kPerChunk = uint32_t(kWave * VEC);   // keys one chunk step can add
  const long long nit = (nchunks + kPerIt - 1) / kPerIt;
  using raw_t = typename C::raw_t;
  auto load_group = [&](long long it, raw_t (&raw)[kDriftUnroll]) {
#pragma unroll
    for (int u = 0; u < kDriftUnroll; ++u) {
      const long long ci = (it * kDriftUnroll + u) * kDriftBlock + tid;
      raw[u] = C::load(drow, ci < nchunks ? ci : nchunks - 1);
    }
  };
  // bits of value e of a chunk (e may differ between lanes)
  auto value_bits = [&](const raw_t& r, int e) -> uint32_t {
    if constexpr (VEC == 8) {
      const uint32_t w = (e & 4) ? ((e & 2) ? r[3] : r[2]) : ((e & 2) ? r[1] : r[0]);
      return (e & 1) ? w >> 16 : w & 0xffffu;
    } else {
      return r;
    }
  };
  auto filter_group = [&](long long it, const raw_t (&raw)[kDriftUnroll]) {
#pragma unroll
    for (int u = 0; u < kDriftUnroll; ++u) {
      const long long ci = (it * kDriftUnroll + u) * kDriftBlock + tid;
      // the values of this lane's chunk that may reach the threshold
      uint32_t pend = 0;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        uint32_t hi;                           // the value's bits in a float's upper half
        if constexpr (VEC == 8)
          hi = (e & 1) ? raw[u][e >> 1] & 0xffff0000u : raw[u][e >> 1] << 16;
        else
          hi = raw[u] << 16;
        pend |= __uint_as_float(hi) >= thr_f ? 1u << e : 0u;
      }
      if (ci >= nchunks) pend = 0u;
      if (__ballot(pend != 0u) == 0ull) continue;   // uniform: the common case
      if (fill > uint32_t(kDriftCap) - kPerChunk) compact(mm);
      // one value per lane and round, as many rounds as the busiest lane needs
      while (__ballot(pend != 0u) != 0ull) {
        const bool act = pend != 0u;
        const int e = act ? __builtin_ctz(pend) : 0;
        pend &= pend - 1u;
        const uint64_t k = (uint64_t(bf16_key(value_bits(raw[u], e))) << 32) |
                           uint64_t(~uint32_t(ci * VEC + e));
        const bool put = act && k >= thr;
        const uint64_t mask = __ballot(put);
        if (put) keys[fill + lanes_below(mask)] = k;
        fill += uint32_t(__popcll(mask));
      }
    }
  };
  {
    // two register sets in turn; loads are unconditional, so the compiler's
    // wait counts stay exact, and groups past the row filter nothing
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
  compact(mm);                                  // at most mm keys per wavefront
  if (lane == 0) s_count[wid] = fill;
  __syncthreads();

  // ---- merge, keep the mm largest keys, rank, residuals on wavefront 0 ----
  if (wid != 0) return;
  {
    uint32_t n = fill;
#pragma unroll
    for (int w = 1; w < kDriftWaves; ++w) {
      const uint32_t cw = s_count[w];
      for (uint32_t e = uint32_t(lane); e < cw; e += kWave) keys[n + e] = s_keys[w][e];
      n += cw;
    }
    wave_sync();
    fill = n;
  }
  compact(mm);                                  // exactly mm keys remain
  const bool has = uint32_t(lane) < mm;
  const uint64_t key = has ? keys[lane] : 0ull;
  int rank = 0;
  for (int o = 0; o < int(mm); ++o) {
    const uint64_t ko = __shfl(key, o, kWave);
    rank += (has && ko > key) ? 1 : 0;
  }
  const int v = has ? int(~uint32_t(key)) : -1;
  const double ad = has ? double(load_logit<DT_BF16>(drow, v)) * invT : -__builtin_inf();
  const double at = has ? double(load_logit<DT_BF16>(trow, v)) * invT : -__builtin_inf();
  double mt = at, md = ad;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    mt = fmax(mt, __shfl_xor(mt, o, kWave));
    md = fmax(md, __shfl_xor(md, o, kWave));
  }
  const double lse_t = mt + log(wave_sum(has ? exp(at - mt) : 0.0));
  const double lse_d = md + log(wave_sum(has ? exp(ad - md) : 0.0));
  if (has) {
    out_support[o0 + rank] = v;
    out_res[o0 + rank] = (at - lse_t) - (ad - lse_d);
  } else if (lane < m) {
    out_support[o0 + lane] = -1;
    out_res[o0 + lane] = __builtin_nan("");
  }
}

}  // namespace sv
