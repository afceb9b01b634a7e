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
constexpr int kFinishBlock = 1024;   // threads per sequence after the multi-workgroup pass

// Shared state of the workgroup-wide pick.
struct PickShared {
  double base, tgt, rho, zres, St;
  double wsum[16];
  int tile, which, clamp, fallback, token;
  int whit[16], wlp[16];
};

// Phase 4 over a whole workgroup: wavefront 0 forms the exact normalisers,
// the tile weights and the crossing tile; then thread t of the first
// kTileChunks threads re-reads chunk t of that tile (in-tile index order),
// and a workgroup prefix scan over the chunk sums finds the token.
template <int DT, int VEC, int NT>
__device__ __forceinline__ void pick_token_block(int b, int K, int V, int ntiles, const DrawRow& dr,
                                 const DrawRows<DT, VEC>& W, const TileSums* ts,
                                 const float* __restrict__ uniforms,
                                 int32_t* __restrict__ out_tokens, DevStats* __restrict__ st,
                                 double* aux_z, PickShared& sh) {
  using C = Chunk<DT, VEC>;
  static_assert(NT >= kTileChunks && NT / kWave <= 16, "pick needs one thread per tile chunk");
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  if (wid == 0) {
    double St = 0.0, Sd = 0.0;
    for (int t = lane; t < ntiles; t += kWave) {
      St += ts[t].E;
      Sd += ts[t].Ed;
    }
    St = __shfl(wave_sum(St), 0, kWave);
    Sd = __shfl(wave_sum(Sd), 0, kWave);
    const double rho = W.residual ? St / Sd : 0.0;
    const double drho = dr.rho - rho;
    int which = W.residual ? 1 : 0;
    double total = tiles_total(ts, ntiles, lane, which, drho);
    const double zres = which ? total : -1.0;
    const bool fallback = W.residual && !(total > 0.0);
    if (fallback) {
      which = 0;
      total = tiles_total(ts, ntiles, lane, 0, drho);
    }
    const double tgt = double(uniforms[(long long)b * (K + 1) + K]) * total;
    int tile = -1, last_pos = -1;
    double base = 0.0, carry = 0.0;
    for (int t0 = 0; t0 < ntiles && tile < 0; t0 += kWave) {
      double v = 0.0;
      if (t0 + lane < ntiles) v = tile_weight(ts[t0 + lane], which, drho);
      const double incl = carry + wave_incl_scan(v, lane);
      const unsigned long long hit = __ballot(t0 + lane < ntiles && incl > tgt);
      const unsigned long long pos = __ballot(t0 + lane < ntiles && v > 0.0);
      if (pos) last_pos = t0 + 63 - __clzll((long long)pos);
      if (hit) {
        const int l = __ffsll((long long)hit) - 1;
        tile = t0 + l;
        base = __shfl(incl - v, l, kWave);
      }
      carry = __shfl(incl, kWave - 1, kWave);
    }
    const bool clamp = tile < 0;
    if (clamp) tile = last_pos;
    if (lane == 0) {
      sh.base = base;
      sh.tgt = tgt;
      sh.rho = rho;
      sh.zres = zres;
      sh.St = St;
      sh.tile = tile;
      sh.which = which;
      sh.clamp = clamp;
      sh.fallback = fallback;
    }
  }
  __syncthreads();
  const int tile = sh.tile, which = sh.which;
  const bool clamp = sh.clamp;
  const double rho = sh.rho, tgt = sh.tgt;
  const long long nchunks = V / VEC;
  const long long ci = (long long)tile * kTileChunks + tid;
  const bool valid = tid < kTileChunks && tile >= 0 && ci < nchunks;
  typename C::raw_t rt, rd;
  double cs = 0.0;
  int lp = -1;
  if (valid) {
    W.load(ci, rt, rd);
#pragma unroll
    for (int e = 0; e < C::N; ++e) {
      const double wv = W.weight(rt, rd, e, which, rho);
      cs += wv;
      lp = wv > 0.0 ? int(ci * VEC + e) : lp;
    }
  }
  // workgroup inclusive scan of the chunk sums (chunk order = thread order)
  const double wincl = wave_incl_scan(cs, lane);
  int wlp = lp;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) wlp = max(wlp, __shfl_xor(wlp, o, kWave));
  if (lane == kWave - 1) sh.wsum[wid] = wincl;
  if (lane == 0) sh.wlp[wid] = wlp;
  __syncthreads();
  double before = sh.base;
  for (int w = 0; w < wid; ++w) before += sh.wsum[w];
  const double incl = before + wincl;
  const unsigned long long hit = __ballot(valid && !clamp && incl > tgt);
  if (lane == 0) sh.whit[wid] = hit ? wid * kWave + __ffsll((long long)hit) - 1 : -1;
  __syncthreads();
  int first = -1, last_elem = -1;
  for (int w = 0; w < NT / kWave; ++w) {
    if (first < 0 && sh.whit[w] >= 0) first = sh.whit[w];
    last_elem = max(last_elem, sh.wlp[w]);
  }
  if (tid == 0) sh.token = -1;
  __syncthreads();
  if (first >= 0 && tid == first) {
    double run = incl - cs;
    int tok = -1;
#pragma unroll
    for (int e = 0; e < C::N; ++e) {
      run += W.weight(rt, rd, e, which, rho);
      if (tok < 0 && run > tgt) tok = int(ci * VEC + e);
    }
    sh.token = tok >= 0 ? tok : lp;       // the chunk holds positive weight
  }
  __syncthreads();
  if (tid == 0) {
    const int token = sh.token >= 0 ? sh.token : last_elem;
    out_tokens[(long long)b * (K + 1) + dr.j] = token;
    if (aux_z != nullptr) aux_z[b] = W.residual ? fmax(sh.zres, 0.0) / sh.St : -1.0;
    if (sh.fallback) atomicAdd(&st->z0_fallbacks, 1ull);
  }
}

// Phases 2-4 for one sequence, given its row statistics in LDS (fR, fS):
// the acceptance scan on wavefront 0, the draw's float64 tile sums of row
// pair j over all wavefronts of the workgroup, then the pick.
template <int DT, int VEC, int NT>
__device__ __forceinline__ void finish_sequence(
    int b, int K, int V, const void* __restrict__ target, const void* __restrict__ draft,
    const int32_t* __restrict__ tokens, const float* __restrict__ uniforms, float c, double c64,
    int n_half, const double* T, const float* fR, const double* fS, TileSums* tiles,
    DrawRow& s_dr, PickShared& psh, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ out_len,
    uint32_t* __restrict__ hist, double* __restrict__ ema, int32_t* __restrict__ steps,
    double decay, DevStats* __restrict__ st, double* aux_p, double* aux_q, double* aux_z) {
  using C = Chunk<DT, VEC>;
  constexpr int kW = NT / kWave;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const long long nchunks = V / VEC;
  auto row_base = [&](int r) -> const void* { return row_ptr<DT>(target, draft, b, r, K, V); };
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
      lane_bad |= !(d >= 0 && d < V);   // checked before the gather below
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
  // wavefront w takes tiles w, w + kW, ...; the next tile's chunks are loaded
  // while the current one is summed
  DrawRows<DT, VEC> W;
  W.init(target, draft, dr, b, K, V, c64);
  const int ntiles = int((nchunks + kTileChunks - 1) / kTileChunks);
  for (int t = wid; t < ntiles; t += kW) {
    double E = 0.0, Ed = 0.0, A = 0.0, Bd = 0.0;
#pragma unroll
    for (int k = 0; k < kTileChunksPerLane; ++k) {
      const long long ci = (long long)t * kTileChunks + (long long)k * kWave + lane;
      if (ci < nchunks) {
        typename C::raw_t a, d;
        W.load(ci, a, d);
        accum_chunk<DT, VEC>(T, n_half, W, a, d, dr.rho, E, Ed, A, Bd);
      }
    }
    E = wave_sum(E);
    if (W.residual) {
      Ed = wave_sum(Ed);
      A = wave_sum(A);
      Bd = wave_sum(Bd);
    }
    if (lane == 0) {
      TileSums ts;
      ts.E = E;
      ts.Ed = Ed;
      ts.A = A;
      ts.Bd = Bd;
      tiles[t] = ts;
    }
  }
  __syncthreads();

  // ---- 4. pick ----
  pick_token_block<DT, VEC, NT>(b, K, V, ntiles, dr, W, tiles, uniforms, out_tokens, st, aux_z,
                                psh);
}

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
  __shared__ PickShared psh;
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

  finish_sequence<DT, VEC, kFBlock>(b, K, V, target, draft, tokens, uniforms, c, c64, n_half, T,
                                    fR, fS, tiles, s_dr, psh, out_tokens, out_len, hist, ema,
                                    steps,
                                    decay, st, aux_p, aux_q, aux_z);
}

// After the multi-workgroup streaming pass: one workgroup per sequence
// combines the row partials (fixed order) and runs phases 2-4.
template <int DT, int VEC, int NT>
__global__ __launch_bounds__(NT) void finish_seq(
    int K, int V, int nseg, const RowPart* __restrict__ parts, const void* __restrict__ target,
    const void* __restrict__ draft, const int32_t* __restrict__ tokens,
    const float* __restrict__ uniforms, float c, double c64, int n_half,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_len, uint32_t* __restrict__ hist,
    double* __restrict__ ema, int32_t* __restrict__ steps, double decay,
    DevStats* __restrict__ st, double* aux_p, double* aux_q, double* aux_z) {
  constexpr bool kTab = (DT == DT_BF16 && VEC == 8);
  __shared__ double T[kTab ? kTabMax : 1];
  __shared__ float fR[kFMaxRows];
  __shared__ double fS[kFMaxRows];
  __shared__ TileSums tiles[kFMaxTiles];
  __shared__ DrawRow s_dr;
  __shared__ PickShared psh;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int rows = 2 * K + 1;
  if constexpr (kTab) {
    for (int i = tid; i < 2 * n_half; i += NT) T[i] = exp_table_entry(i, n_half, c64);
  }
  for (int r = tid; r < rows; r += NT) {
    float R;
    double S;
    combine_sum_parts(parts + ((long long)b * rows + r) * nseg, nseg, R, S);
    fR[r] = R;
    fS[r] = S;
  }
  __syncthreads();
  finish_sequence<DT, VEC, NT>(b, K, V, target, draft, tokens, uniforms, c, c64, n_half, T,
                                    fR, fS, tiles, s_dr, psh, out_tokens, out_len, hist, ema,
                                    steps,
                                    decay, st, aux_p, aux_q, aux_z);
}

__global__ void zero_hist(uint32_t* hist, int n) {
  if (int(threadIdx.x) < n) hist[threadIdx.x] = 0u;
}

}  // namespace sv
