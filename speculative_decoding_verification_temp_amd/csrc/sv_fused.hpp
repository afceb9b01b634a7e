// Stochastic verification with one workgroup per sequence.
//
// One launch does the whole path for each sequence, with all communication
// inside the workgroup (LDS and barriers), none across workgroups:
//   1. stream the sequence's 2K+1 logit rows once (128-bit non-temporal
//      loads, a rolling prefetch buffer that runs across row boundaries) and
//      keep per-wavefront softmax partials of every row in LDS;
//   2. combine the partials in a fixed order and run the acceptance scan on
//      one wavefront (first rejection j, emitted tokens, histogram, EMA);
//   3. re-read row pair j (or target row K for the bonus) and form the draw's
//      float64 tile sums in LDS;
//   4. pick the token from the tile sums and the re-read crossing tile.
// A whole grid of sequences streams at full HBM bandwidth as long as every
// compute unit holds at least one sequence, so the host uses this kernel for
// large batches and the multi-kernel pipeline otherwise.
#pragma once

#include "sv_kernels.hpp"

namespace sv {

constexpr int kFBlock = 1024;
constexpr int kFGroup = 4;          // chunks per reference update in the streaming pass
constexpr int kFWaves = kFBlock / kWave;
constexpr int kFMaxRows = 127;      // 2K + 1 for K <= 63
constexpr int kFMaxTiles = 256;     // draw tiles per row held in LDS

template <int DT, int VEC, int U>
__global__ __launch_bounds__(kFBlock) void verify_fused(
    int K, int V, const void* __restrict__ target, const void* __restrict__ draft,
    const int32_t* __restrict__ tokens, const float* __restrict__ uniforms, float c, double c64,
    int n_half, int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_len,
    uint32_t* __restrict__ hist, double* __restrict__ ema, int32_t* __restrict__ steps,
    double decay, DevStats* __restrict__ st, double* aux_p, double* aux_q, double* aux_z) {
  using C = Chunk<DT, VEC>;
  constexpr bool kTab = (DT == DT_BF16 && VEC == 8);
  __shared__ double T[kTab ? kTabMax : 1];
  __shared__ float pR[kFMaxRows][kFWaves];
  __shared__ double pS[kFMaxRows][kFWaves];
  __shared__ float fR[kFMaxRows];
  __shared__ double fS[kFMaxRows];
  __shared__ TileSums tiles[kFMaxTiles];
  __shared__ DrawRow s_dr;
  __shared__ int s_bad_token;

  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int rows = 2 * K + 1;
  const long long nchunks = V / VEC;
  const int kmax = int((nchunks + kFBlock - 1) / kFBlock);   // chunk slots per thread per row
  const int total = rows * kmax;

  // drafted tokens outside [0, V) make the sequence invalid: skip the rows
  if (wid == 0) {
    const int d = lane < K ? tokens[(long long)b * K + lane] : 0;
    const bool bad = __any(lane < K && !(d >= 0 && d < V));
    if (lane == 0) s_bad_token = bad ? 1 : 0;
  }
  __syncthreads();
  if (s_bad_token) {
    if (wid == 0) {
      if (aux_p != nullptr && lane < K) aux_p[(long long)b * K + lane] = __builtin_nan("");
      if (aux_q != nullptr && lane < K) aux_q[(long long)b * K + lane] = __builtin_nan("");
      if (aux_z != nullptr && lane == 0) aux_z[b] = -1.0;
      emit_and_update(lane, b, K, 0, true, tokens, out_tokens, out_len, hist, ema, steps, decay,
                      st, -1, 0);
    }
    return;
  }

  // ---- 1. streaming pass ----
  // Thread tid owns chunks tid, tid + kFBlock, ... of every row, taken in
  // groups of kFGroup chunk slots (slots past the row end are empty, so a
  // group never spans two rows). Two groups are in flight at once, and even
  // and odd groups keep separate (R, S) accumulators so that consecutive
  // groups do not wait on each other; both merge exactly at the row end.
  auto row_base = [&](int r) -> const void* { return row_ptr<DT>(target, draft, b, r, K, V); };
  const int gpr = (kmax + kFGroup - 1) / kFGroup;            // groups per row
  const int ngroups = rows * gpr;
  typename C::raw_t buf[2][kFGroup];
  auto issue = [&](int g, typename C::raw_t (&dst)[kFGroup]) {
    const int r = g / gpr, k0 = (g - r * gpr) * kFGroup;
    const void* base = row_base(r);
#pragma unroll
    for (int q = 0; q < kFGroup; ++q) {
      const long long ci = tid + (long long)(k0 + q) * kFBlock;
      if (ci < nchunks) dst[q] = C::load(base, ci);
    }
  };
  if (ngroups > 0) issue(0, buf[0]);
  if (ngroups > 1) issue(1, buf[1]);
  if constexpr (kTab) {
    for (int i = tid; i < 2 * n_half; i += kFBlock) T[i] = exp_table_entry(i, n_half, c64);
  }

  float Ra[2] = {kRefInit, kRefInit};
  double Sa[2] = {0.0, 0.0};
  int cur = 0;
  auto flush = [&]() {
    const float Rl = fmaxf(Ra[0], Ra[1]);
    const double Sl = rescale(Sa[0], Ra[0], Rl) + rescale(Sa[1], Ra[1], Rl);
    const float Rw = wave_max(Rl);
    const double Sw = wave_sum(rescale(Sl, Rl, Rw));
    if (lane == 0) {
      pR[cur][wid] = Rw;
      pS[cur][wid] = Sw;
    }
    Ra[0] = Ra[1] = kRefInit;
    Sa[0] = Sa[1] = 0.0;
  };
  for (int g0 = 0; g0 < ngroups; g0 += 2) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int g = g0 + h2;
      if (g < ngroups) {
        const int r = g / gpr, k0 = (g - r * gpr) * kFGroup;
        if (r != cur) {            // previous row finished (uniform over the workgroup)
          flush();
          cur = r;
        }
        float x[kFGroup][C::N];
        bool valid[kFGroup];
        float gm = -__builtin_inff();
#pragma unroll
        for (int q = 0; q < kFGroup; ++q) {
          valid[q] = tid + (long long)(k0 + q) * kFBlock < nchunks;
          C::unpack(buf[h2][q], x[q]);
#pragma unroll
          for (int e = 0; e < C::N; ++e) {
            x[q][e] = valid[q] ? x[q][e] : -__builtin_inff();
            gm = fmaxf(gm, x[q][e]);
          }
        }
        const float Rn = fmaxf(Ra[h2], ceilf(gm * c));
        Sa[h2] = rescale(Sa[h2], Ra[h2], Rn);
        Ra[h2] = Rn;
        float t[kFGroup * C::N];
#pragma unroll
        for (int q = 0; q < kFGroup; ++q)
#pragma unroll
          for (int e = 0; e < C::N; ++e) t[q * C::N + e] = term(x[q][e], c, Rn);
#pragma unroll
        for (int w = 1; w < kFGroup * C::N; w <<= 1)
#pragma unroll
          for (int e = 0; e + w < kFGroup * C::N; e += 2 * w) t[e] += t[e + w];
        Sa[h2] += (double)t[0];
        if (g + 2 < ngroups) issue(g + 2, buf[h2]);
      }
    }
  }
  flush();
  __syncthreads();
  for (int r = tid; r < rows; r += kFBlock) {
    float Rr = pR[r][0];
#pragma unroll
    for (int w = 1; w < kFWaves; ++w) Rr = fmaxf(Rr, pR[r][w]);
    double Sr = 0.0;
#pragma unroll
    for (int w = 0; w < kFWaves; ++w) Sr += rescale(pS[r][w], pR[r][w], Rr);
    fR[r] = Rr;
    fS[r] = Sr;
  }
  __syncthreads();

  // ---- 2. acceptance scan on wavefront 0 ----
  if (wid == 0) {
    float Rt = 0.0f, Rd = 0.0f;
    double St = 1.0, Sd = 1.0;
    bool lane_bad = false;
    if (lane <= K) {
      Rt = fR[lane];
      St = fS[lane];
      lane_bad |= !finite_pos(St);
    }
    int d = 0;
    double P = 0.0, Q = 1.0;
    bool keep = true, zq = false;
    if (lane < K) {
      Rd = fR[K + 1 + lane];
      Sd = fS[K + 1 + lane];
      lane_bad |= !finite_pos(Sd);
      d = tokens[(long long)b * K + lane];
      if (!lane_bad) {
        const float xt = load_logit<DT>(row_base(lane), d);
        const float xd = load_logit<DT>(row_base(K + 1 + lane), d);
        P = double(term(xt, c, Rt)) / St;
        Q = double(term(xd, c, Rd)) / Sd;
        const double u = uniforms[(long long)b * (K + 1) + lane];
        keep = (P >= Q) || (u < P / Q);
        zq = keep && Q == 0.0;
      }
    }
    const bool bad = __any(lane_bad);
    const unsigned long long rej = __ballot(lane < K && !keep);
    const int j = rej ? __ffsll((long long)rej) - 1 : K;
    if (aux_p != nullptr && lane < K) aux_p[(long long)b * K + lane] = bad ? __builtin_nan("") : P;
    if (aux_q != nullptr && lane < K) aux_q[(long long)b * K + lane] = bad ? __builtin_nan("") : Q;
    const float Rtj = __shfl(Rt, j, kWave), Rdj = __shfl(Rd, j, kWave);
    const double Stj = __shfl(St, j, kWave), Sdj = __shfl(Sd, j, kWave);
    if (lane == 0) {
      DrawRow dr;
      dr.rho = Stj / Sdj;
      dr.R_t = Rtj;
      dr.R_d = Rdj;
      dr.j = bad ? -1 : j;
      dr.pad = 0;
      s_dr = dr;
      if (bad && aux_z != nullptr) aux_z[b] = -1.0;
    }
    const unsigned long long zqm = __ballot(zq && lane < j);
    if (lane == 0 && !bad && zqm)
      atomicAdd(&st->zero_q_accepts, (unsigned long long)__popcll(zqm));
    emit_and_update(lane, b, K, j, bad, tokens, out_tokens, out_len, hist, ema, steps, decay, st,
                    -1, d);
  }
  __syncthreads();
  const DrawRow dr = s_dr;
  if (dr.j < 0) return;

  // ---- 3. draw tile sums of row pair j (or target row K) ----
  DrawRows<DT, VEC> W;
  W.init(target, draft, dr, b, K, V, c64);
  const int ntiles = int((nchunks + kTileChunks - 1) / kTileChunks);
  for (int t = wid; t < ntiles; t += kFWaves) {
    typename C::raw_t rt[kTileChunksPerLane], rd[kTileChunksPerLane];
#pragma unroll
    for (int k = 0; k < kTileChunksPerLane; ++k) {
      const long long ci = (long long)t * kTileChunks + (long long)k * kWave + lane;
      if (ci < nchunks) W.load(ci, rt[k], rd[k]);
    }
    double E = 0.0, Ed = 0.0, A = 0.0, Bd = 0.0;
#pragma unroll
    for (int k = 0; k < kTileChunksPerLane; ++k) {
      const long long ci = (long long)t * kTileChunks + (long long)k * kWave + lane;
      if (ci < nchunks) {
        double et[C::N], ed[C::N];
        chunk_terms_tab<DT, VEC>(T, n_half, W, rt[k], rd[k], et, ed);
#pragma unroll
        for (int e = 0; e < C::N; ++e) {
          E += et[e];
          Ed += ed[e];
          const bool pos = et[e] > dr.rho * ed[e];
          A += pos ? et[e] : 0.0;
          Bd += pos ? ed[e] : 0.0;
        }
      }
    }
    E = wave_sum(E);
    if (W.residual) {
      Ed = wave_sum(Ed);
      A = wave_sum(A);
      Bd = wave_sum(Bd);
    }
    if (lane == 0) {
      TileSums s;
      s.E = E;
      s.Ed = Ed;
      s.A = A;
      s.Bd = Bd;
      tiles[t] = s;
    }
  }
  __syncthreads();

  // ---- 4. pick ----
  if (wid == 0)
    pick_token<DT, VEC>(b, K, V, ntiles, dr, W, tiles, uniforms, out_tokens, st, aux_z, lane);
}

__global__ void zero_hist(uint32_t* hist, int n) {
  if (int(threadIdx.x) < n) hist[threadIdx.x] = 0u;
}

}  // namespace sv
