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
// One 1024-thread workgroup per (sequence, drafted position i < k_b) of a
// valid sequence (the scan's accept length is read to tell): the draft row is
// counted into the full pass's exact 65536-key histogram (with its careful
// recount when a 16-bit counter wraps), the m-th largest value follows from
// the counts, a second read of the row collects the tokens above it into one
// LDS list and the tokens tied with it into another (slots by atomics, the
// loads pipelined as in the count), the lowest-index ties are picked by
// ranking the tie list (with more ties than the list holds, a third read
// walks the row in index order), and wavefront 0 ranks the m tokens and forms
// the two float64 log-sum-exps over them.
#pragma once

#include "sv_trunc.hpp"

namespace sv {

constexpr int kDriftMaxM = 64;
constexpr int kTieCap = kTrBlock;   // ties at the threshold kept unordered

// inclusive prefix of v over the threads of the workgroup in index order, and
// the workgroup total
__device__ inline uint32_t tr_prefix(uint32_t v, uint32_t* s, uint32_t& total) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  uint32_t incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t u = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += u;
  }
  if (lane == kWave - 1) s[wid] = incl;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kTrWaves; ++w) {
    if (w < wid) before += s[w];
    tot += s[w];
  }
  __syncthreads();
  total = tot;
  return before + incl;
}

template <int VEC>
__global__ __launch_bounds__(kTrBlock) void drift_residual(
    const void* __restrict__ target, const void* __restrict__ draft, int K, int V, double invT,
    int m, const int32_t* __restrict__ kdraft, const int32_t* __restrict__ accept_len,
    int32_t* __restrict__ out_support, double* __restrict__ out_res) {
  using C = Chunk<DT_BF16, VEC>;
  __shared__ uint32_t H[kHistWords];
  __shared__ uint32_t s_wraps[kMaxWraps];
  __shared__ uint32_t s_nwrap;
  __shared__ uint32_t s_u[kTrWaves];
  __shared__ int s_i[kTrWaves];
  __shared__ uint32_t s_key, s_above, s_fill, s_ties, s_ntie;
  __shared__ int s_sel[kDriftMaxM];
  __shared__ int s_tie[kTieCap];
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
  const int mm = min(m, V);
  const uint32_t k0 = uint32_t(tid) * kKeysPerThread;

  // ---- 1. exact histogram of the draft row ----
  uint32_t nwrap = 0;
  auto count_of = [&](int ii) -> uint32_t {
    const uint32_t key = k0 + uint32_t(ii);
    uint32_t n = (H[hist_word(key >> 1)] >> ((key & 1u) << 4)) & 0xffffu;
    if (nwrap != 0u) {
      const int nw = min(int(nwrap), kMaxWraps);
#pragma unroll 1
      for (int e = 0; e < nw; ++e) n += s_wraps[e] == key ? 65536u : 0u;
    }
    return n;
  };
  auto thread_total = [&]() -> uint32_t {
    nwrap = s_nwrap;
    uint32_t t = 0;
#pragma unroll 2
    for (int q = 0; q < kKeysPerThread / 8; ++q) {
      const u32x4 v = reinterpret_cast<const u32x4*>(H)[tid * (kKeysPerThread / 8) + (q ^ (tid & 7))];
#pragma unroll
      for (int w = 0; w < 4; ++w) t += (v[w] & 0xffffu) + (v[w] >> 16);
    }
    if (nwrap != 0u)
#pragma unroll 1
      for (int e = 0; e < min(int(nwrap), kMaxWraps); ++e)
        t += (s_wraps[e] >> 6) == uint32_t(tid) ? 65536u : 0u;
    return t;
  };
  count_row<VEC, kCountFast>(drow, V, H, &s_nwrap, s_wraps);
  uint32_t n_t = thread_total();
  if (tr_sum(n_t, s_u) != uint32_t(V)) {
    count_row<VEC, kCountEven>(drow, V, H, &s_nwrap, s_wraps);
    count_row<VEC, kCountOdd>(drow, V, H, &s_nwrap, s_wraps);
    n_t = thread_total();
  }

  // ---- 2. the mm-th largest key and the count strictly above it ----
  {
    uint32_t n_all;
    const uint32_t above = tr_above(n_t, s_u, n_all);
    if (above < uint32_t(mm) && above + n_t >= uint32_t(mm)) {
      uint32_t acc = above;
#pragma unroll 1
      for (int ii = kKeysPerThread - 1; ii >= 0; --ii) {
        const uint32_t n = count_of(ii);
        if (acc + n >= uint32_t(mm)) {
          s_key = k0 + uint32_t(ii);
          s_above = acc;
          break;
        }
        acc += n;
      }
    }
    if (tid == 0) {
      s_fill = 0u;
      s_ties = 0u;
      s_ntie = 0u;
    }
    __syncthreads();
  }
  const uint32_t kth = s_key, n_above = s_above;
  const uint32_t need = uint32_t(mm) - n_above;   // ties at kth to take, lowest indices first

  // ---- 3. collect: every token above kth (fewer than mm), and the ties at
  // kth, in one pipelined read ----
  const long long nchunks = V / VEC;
  auto collect_chunk = [&](const typename C::raw_t& raw, long long ci) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      uint32_t bits;
      if constexpr (VEC == 8)
        bits = (e & 1) ? raw[e >> 1] >> 16 : raw[e >> 1] & 0xffffu;
      else
        bits = raw;
      const uint32_t key = bf16_key(bits);
      if (key > kth) {
        const uint32_t slot = atomicAdd(&s_fill, 1u);
        if (slot < uint32_t(kDriftMaxM)) s_sel[slot] = int(ci * VEC + e);
      } else if (key == kth) {
        const uint32_t slot = atomicAdd(&s_ntie, 1u);
        if (slot < uint32_t(kTieCap)) s_tie[slot] = int(ci * VEC + e);
      }
    }
  };
  {
    constexpr int U = 4;
    long long ci = tid;
    for (; ci + (long long)(U - 1) * kTrBlock < nchunks; ci += (long long)U * kTrBlock) {
      typename C::raw_t raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) raw[u] = C::load(drow, ci + (long long)u * kTrBlock);
#pragma unroll
      for (int u = 0; u < U; ++u) collect_chunk(raw[u], ci + (long long)u * kTrBlock);
    }
    for (; ci < nchunks; ci += kTrBlock) collect_chunk(C::load(drow, ci), ci);
  }
  __syncthreads();
  const uint32_t ntie = s_ntie;
  if (ntie <= uint32_t(kTieCap)) {
    // the `need` lowest indices among the ties: rank each by index
    if (tid < int(ntie)) {
      const int v = s_tie[tid];
      uint32_t rank = 0;
#pragma unroll 4
      for (uint32_t o = 0; o < ntie; ++o) rank += s_tie[o] < v ? 1u : 0u;
      if (rank < need) s_sel[n_above + rank] = v;
    }
  } else {
    // more ties than the list holds: walk the row in index order (blocks of
    // kTrBlock chunks, thread order = index order) and take the first `need`
    for (long long c0 = 0; c0 < nchunks && s_ties < need; c0 += kTrBlock) {
      const long long ci = c0 + tid;
      uint32_t bits[VEC];
      if (ci < nchunks) {
        const typename C::raw_t raw = C::load(drow, ci);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          if constexpr (VEC == 8)
            bits[e] = (e & 1) ? raw[e >> 1] >> 16 : raw[e >> 1] & 0xffffu;
          else
            bits[e] = raw;
        }
      }
      uint32_t ties = 0;
#pragma unroll
      for (int e = 0; e < VEC; ++e) ties += (ci < nchunks && bf16_key(bits[e]) == kth) ? 1u : 0u;
      uint32_t blk_ties;
      const uint32_t incl = tr_prefix(ties, s_u, blk_ties);
      const uint32_t base = s_ties;
      uint32_t t = base + incl - ties;             // ties before this thread's
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        if (ci < nchunks && bf16_key(bits[e]) == kth) {
          if (t < need) s_sel[n_above + t] = int(ci * VEC + e);
          ++t;
        }
      }
      __syncthreads();
      if (tid == 0) s_ties = base + blk_ties;
      __syncthreads();
    }
  }
  __syncthreads();

  // ---- 4. rank the mm tokens, residuals on wavefront 0 ----
  if (wid == 0) {
    int v = -1;
    float xd = 0.0f;
    if (lane < mm) {
      v = s_sel[lane];
      xd = load_logit<DT_BF16>(drow, v);
    }
    // rank: descending draft logit, then ascending index
    int rank = 0;
    for (int o = 0; o < mm; ++o) {
      const int vo = __shfl(v, o, kWave);
      const float xo = __shfl(xd, o, kWave);
      rank += (lane < mm && (xo > xd || (xo == xd && vo < v))) ? 1 : 0;
    }
    const double at = lane < mm ? double(load_logit<DT_BF16>(trow, v)) * invT : -__builtin_inf();
    const double ad = lane < mm ? double(xd) * invT : -__builtin_inf();
    double mt = at, md = ad;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
      mt = fmax(mt, __shfl_xor(mt, o, kWave));
      md = fmax(md, __shfl_xor(md, o, kWave));
    }
    const double lse_t = mt + log(wave_sum(lane < mm ? exp(at - mt) : 0.0));
    const double lse_d = md + log(wave_sum(lane < mm ? exp(ad - md) : 0.0));
    if (lane < mm) {
      out_support[o0 + rank] = v;
      out_res[o0 + rank] = (at - lse_t) - (ad - lse_d);
    } else if (lane < m) {
      out_support[o0 + lane] = -1;
      out_res[o0 + lane] = __builtin_nan("");
    }
  }
}

}  // namespace sv
