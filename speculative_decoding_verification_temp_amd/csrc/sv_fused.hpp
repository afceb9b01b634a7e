// Stochastic verification with one 1024-thread workgroup per sequence after
// the streaming pass (finish_seq, the default for up to 256 draw tiles per
// row, i.e. V <= 524288), or for the whole path (verify_fused).
//
// Per sequence, with all communication inside the workgroup (LDS and
// barriers), none across workgroups:
//   1. (verify_fused only) stream the sequence's 2K+1 logit rows once and keep
//      per-wavefront softmax partials of every row in LDS; finish_seq instead
//      combines the streaming pass's per-segment partials;
//   2. combine the partials in a fixed order and run the acceptance scan on
//      one wavefront (first rejection j, stopping rules, emitted tokens,
//      histogram, EMA);
//   3. re-read row pair j (or target row k_b for the bonus) and form the
//      draw's float64 tile sums in LDS;
//   4. pick the token from the tile sums and the re-read crossing tile.
// verify_fused is off unless SPEC_VERIFY_FUSED_MIN_B is set: at 4 waves per
// SIMD its streaming part is slower than the separate streaming pass, and its
// finish gains no overlap.
#pragma once

#include "sv_drift.hpp"

namespace sv {

constexpr int kFBlock = 1024;
constexpr int kFGroup = 4;          // chunks per reference update in the streaming pass
constexpr int kFWaves = kFBlock / kWave;
constexpr int kFMaxRows = 127;      // 2K + 1 for K <= 63
constexpr int kFMaxTiles = 256;     // draw tiles per row held in LDS
constexpr int kFinishBlock = 1024;   // threads per sequence after the multi-workgroup pass
constexpr int kFinishBlockHalf = 512;   // the same with two sequences per compute unit

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

// Draw tile sums of bf16 rows straight from the table entries 2^(x * c),
// scaled by 2^-R once per tile instead of once per term. When both rows'
// references satisfy |R| <= kUnscaledMaxR, every term of the rows is a normal
// float64 number no larger than about 2^R (x * c <= R over a row), so
//   E  = 2^-Rt sum Tt,   Ed = 2^-Rd sum Td,
//   A  = 2^-Rt sum over {Tt > rho2 Td} of (Tt - rho2 Td),
//   Bd = 2^-Rd sum over the same set of Td,   rho2 = rho 2^(Rt - Rd),
// are the sums of the scaled terms, formed with one exact scaling per tile.
// A table lookup costs a few packed 16-bit operations per word of two values:
// offset = bits - base per half (the sign stays in bit 15 for in-window
// values), byte offset = (offset << 3) with the sign put back in bit 15.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
constexpr float kUnscaledMaxR = 500.0f;
constexpr uint32_t kTabOutBits = 0x70007000u;   // offset >= 4096 in either half

// Table byte offsets of the two bf16 values of word w: the low 16 bits of
// the result for the low value, the high 16 bits for the high one, each
// ((bits - base) << 3) with the value's sign in bit 15 (one bit insert). For a
// value inside the window bit 15 of the shifted offset is already 0; for any
// other value the offset is meaningless but still a 16-bit offset, i.e.
// inside the table. ORs the raw offsets into acc, whose kTabOutBits then flag
// such values. The empty asm keeps the packed offsets as one value, so that
// each half costs one extract.
__device__ __forceinline__ uint32_t tab_offsets2(uint32_t w, uint32_t& acc) {
  constexpr unsigned short kB = (unsigned short)(kTabELo << 7);
  const u16x2 o = __builtin_bit_cast(u16x2, w) - (u16x2){kB, kB};
  acc |= __builtin_bit_cast(uint32_t, o);
  const uint32_t sh = __builtin_bit_cast(uint32_t, (u16x2)(o << (u16x2){3, 3}));
  uint32_t p = (w & 0x80008000u) | sh;
  asm volatile("" : "+v"(p));
  return p;
}

__device__ __forceinline__ double tab_at(const double* T, uint32_t byte_off) {
  return *reinterpret_cast<const double*>(reinterpret_cast<const char*>(T) + byte_off);
}

// 2^(x * c) of one bf16 value: its table entry, or exp2_acc outside the
// window (0 there when the row's truncation drops the value; inside the
// window the table itself holds 0 for dropped values)
__device__ __forceinline__ double term_unscaled(const double* T, uint32_t bits, double c,
                                                uint32_t thr) {
  const uint32_t off = (bits & 0x7fffu) - uint32_t(kTabELo << 7);
  if (off < uint32_t(kTabStride)) return T[off + ((bits & 0x8000u) ? kTabStride : 0)];
  return bf16_key(bits) >= thr ? exp2_acc(double(__uint_as_float(bits << 16)) * c) : 0.0;
}

// fp32 rows: 2^y = 2^n * 2^(i/4096) * 2^r in float64, with 4096 n + i the
// nearest integer to 4096 y (read from the low bits of y + 1.5 * 2^40, whose
// unit in the last place is 2^-12; every step exact), |r| <= 2^-13, a
// 4096-entry LDS table T2[i] = 2^(i/4096) and the degree-2 Taylor polynomial
// of 2^r (truncation error below 1.1e-13 relative, far inside what the draw's
// comparisons resolve). y <= -1100 (including -inf) gives 0.
constexpr int kTab2 = 4096;
__device__ inline double exp2_frac_entry(int i) { return exp2_acc_hi(double(i) * (1.0 / 4096.0)); }
__device__ __forceinline__ double exp2_tab(double y, const double* T2) {
  constexpr double L = 0.6931471805599453094172321214581766;   // ln 2
  constexpr double a2 = L * L / 2;
  constexpr double kShift = 0x1.8p40;
  y = fmax(y, -1100.0);
  const double ys = y + kShift;
  const int k = int(uint32_t(__double_as_longlong(ys)));      // 4096 n + i (two's complement)
  const double r = y - (ys - kShift);
  const double p = __builtin_fma(__builtin_fma(a2, r, L), r, 1.0);
  return __builtin_ldexp(T2[k & (kTab2 - 1)] * p, k >> 12);
}

__device__ __forceinline__ void accum_pair_u(double et, double ed, double rho2, double& E,
                                             double& Ed, double& A, double& Bd) {
  E += et;
  Ed += ed;
  const double dv = __builtin_fma(-rho2, ed, et);
  const double s = dv > 0.0 ? 1.0 : 0.0;
  A = __builtin_fma(s, dv, A);
  Bd = __builtin_fma(s, ed, Bd);
}

// A unit is kUnitChunks chunks of 8 bf16 values per lane and row; a tile is
// kUnits units.
constexpr int kUnitChunks = 1;
constexpr int kUnits = kTileChunksPerLane / kUnitChunks;
struct UnitBuf {
  u32x4 a[kUnitChunks], d[kUnitChunks];
};

// word i of chunk k of a unit, by selects (no indexing of the register arrays)
__device__ __forceinline__ uint32_t word_at(const u32x4 (&a)[kUnitChunks], int k, int i) {
  static_assert(kUnitChunks <= 2, "select chain covers two chunks");
  u32x4 x = a[0];
  if constexpr (kUnitChunks == 2) x = k == 0 ? a[0] : a[1];
  return i == 0 ? x[0] : i == 1 ? x[1] : i == 2 ? x[2] : x[3];
}

// one lane's sums over one unit (chunks c0 + k * kWave; RAGGED: chunks at or
// past nchunks are skipped). Tt, Td: the target and draft rows' tables (one
// table unless the rows are truncated), thr_t, thr_d their threshold keys.
// MASK (truncated fp32 rows): a value whose order key is below its row's
// threshold contributes 0.
template <int DT, bool RESID, bool RAGGED, bool MASK = false>
__device__ __forceinline__ void unit_sums(const double* Tt, const double* Td, uint32_t thr_t,
                                          uint32_t thr_d, const UnitBuf& u, long long c0,
                                          long long nchunks, double rho2, double c, double& E,
                                          double& Ed, double& A, double& Bd) {
  E = Ed = A = Bd = 0.0;
  if constexpr (DT == DT_F32) {      // 4 fp32 values per chunk, terms from exp2_tab
    if constexpr (MASK) {
      // a unit in which no lane holds a kept value adds nothing: skip its
      // terms (most units, when the truncation keeps few values)
      bool kept = false;
#pragma unroll
      for (int k = 0; k < kUnitChunks; ++k) {
        if (RAGGED && c0 + (long long)k * kWave >= nchunks) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          kept |= order_key<DT_F32>(u.a[k][q]) >= thr_t;
          if constexpr (RESID) kept |= order_key<DT_F32>(u.d[k][q]) >= thr_d;
        }
      }
      if (!__any(kept)) return;
    }
#pragma unroll
    for (int k = 0; k < kUnitChunks; ++k) {
      if (RAGGED && c0 + (long long)k * kWave >= nchunks) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        double et = 0.0, ed = 0.0;
        if constexpr (MASK) {
          // a term is formed only in value slots where some lane keeps one
          // (few with top-p: its kept values lie scattered over the row)
          const bool kt = order_key<DT_F32>(u.a[k][q]) >= thr_t;
          if (__any(kt)) {
            et = exp2_tab(double(__uint_as_float(u.a[k][q])) * c, Tt);
            if (!kt) et = 0.0;
          }
          if constexpr (RESID) {
            const bool kd = order_key<DT_F32>(u.d[k][q]) >= thr_d;
            if (__any(kd)) {
              ed = exp2_tab(double(__uint_as_float(u.d[k][q])) * c, Tt);
              if (!kd) ed = 0.0;
            }
          }
        } else {
          et = exp2_tab(double(__uint_as_float(u.a[k][q])) * c, Tt);
          if constexpr (RESID) ed = exp2_tab(double(__uint_as_float(u.d[k][q])) * c, Tt);
        }
        if constexpr (RESID)
          accum_pair_u(et, ed, rho2, E, Ed, A, Bd);
        else
          E += et;
      }
    }
    return;
  }
  uint32_t acc = 0;
#pragma unroll
  for (int k = 0; k < kUnitChunks; ++k) {
    if (RAGGED && c0 + (long long)k * kWave >= nchunks) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t pt = tab_offsets2(u.a[k][q], acc);
      const double t0 = tab_at(Tt, pt & 0xffffu), t1 = tab_at(Tt, pt >> 16);
      if constexpr (RESID) {
        const uint32_t pd = tab_offsets2(u.d[k][q], acc);
        const double f0 = tab_at(Td, pd & 0xffffu), f1 = tab_at(Td, pd >> 16);
        accum_pair_u(t0, f0, rho2, E, Ed, A, Bd);
        accum_pair_u(t1, f1, rho2, E, Ed, A, Bd);
      } else {
        E += t0;
        E += t1;
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // one chunk's lookups in flight at a time
  }
  if (acc & kTabOutBits) {     // a value outside the window: this lane again, term by term
    E = Ed = A = Bd = 0.0;
#pragma unroll 1
    for (int v = 0; v < kUnitChunks * 8; ++v) {
      const int k = v >> 3, q = v & 7;
      if (RAGGED && c0 + (long long)k * kWave >= nchunks) break;
      const uint32_t wt = word_at(u.a, k, q >> 1);
      const double et = term_unscaled(Tt, (q & 1) ? wt >> 16 : wt & 0xffffu, c, thr_t);
      if constexpr (RESID) {
        const uint32_t wd = word_at(u.d, k, q >> 1);
        const double ed = term_unscaled(Td, (q & 1) ? wd >> 16 : wd & 0xffffu, c, thr_d);
        accum_pair_u(et, ed, rho2, E, Ed, A, Bd);
      } else {
        E += et;
      }
    }
  }
}

// Tile sums of the draw rows. A wavefront takes its tiles as a stream of
// units, with the units of one tile in flight: the loads of unit i + kUnits
// are issued right after unit i has been summed, so a wavefront keeps
// kUnits - 1 units of loads outstanding while it computes. Wavefront w takes
// tiles w, w + NW, w + 2 NW, ... or, with a claim counter in LDS (next, set
// to 0 before the phase), each time the lowest tile no wavefront has claimed
// yet: the wavefronts of a SIMD do not progress at one rate, and claiming
// lets the faster ones take more tiles (and a wavefront with other work
// joins when it is done). Either way a wavefront's tiles come in increasing
// order and every tile but the row's last is whole, so only the last tile a
// wavefront takes can be ragged. Chunks past the row end are clamped to the
// last chunk for loading and skipped in the sums.
template <int DT, int VEC, bool RESID, int NW, bool MASK = false>
__device__ __forceinline__ void tiles_unscaled(const double* Tt, const double* Td,
                                               const void* trow, const void* drow,
                                               const DrawRow& dr, double c, int ntiles,
                                               long long nchunks, TileSums* tiles, int wid,
                                               int lane, int* next = nullptr) {
  using C = Chunk<DT, VEC>;
  const double rho2 = RESID ? __builtin_ldexp(dr.rho, int(dr.R_t) - int(dr.R_d)) : 0.0;
  const int st = -int(dr.R_t), sd = -int(dr.R_d);
  auto unit_c0 = [&](int t, int u) -> long long {
    return (long long)t * kTileChunks + (long long)u * kUnitChunks * kWave + lane;
  };
  auto load_unit = [&](int t, int u, UnitBuf& b) {
    const long long c0 = unit_c0(t, u);
#pragma unroll
    for (int k = 0; k < kUnitChunks; ++k) {
      const long long ci = min(c0 + (long long)k * kWave, nchunks - 1);
      b.a[k] = C::load(trow, ci);
      if constexpr (RESID) b.d[k] = C::load(drow, ci);
    }
  };
  auto finish_tile = [&](int t, double E, double Ed, double A, double Bd) {
    E = wave_sum(E);
    if constexpr (RESID) {
      Ed = wave_sum(Ed);
      A = wave_sum(A);
      Bd = wave_sum(Bd);
    }
    if (lane == 0) {
      TileSums ts;
      ts.E = __builtin_ldexp(E, st);
      ts.Ed = RESID ? __builtin_ldexp(Ed, sd) : 0.0;
      ts.A = RESID ? __builtin_ldexp(A, st) : 0.0;
      ts.Bd = RESID ? __builtin_ldexp(Bd, sd) : 0.0;
      tiles[t] = ts;
    }
  };
  // this wavefront's tile after t (its first for t < 0)
  auto claim = [&](int t) -> int {
    if (next == nullptr) return t < 0 ? wid : t + NW;
    int v = 0;
    if (lane == 0) v = atomicAdd(next, 1);
    return __builtin_amdgcn_readfirstlane(v);
  };
  int t = claim(-1);
  if (t >= ntiles) return;
  UnitBuf b[kUnits];
#pragma unroll
  for (int u = 0; u < kUnits; ++u) load_unit(t, u, b[u]);
  // a tile with a successor is whole, and its loop body issues the
  // successor's loads unconditionally
  int tn = claim(t);
  while (tn < ntiles) {
    double E = 0.0, Ed = 0.0, A = 0.0, Bd = 0.0;
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      double e, ed, a, bd;
      unit_sums<DT, RESID, false, MASK>(Tt, Td, dr.thr_t, dr.thr_d, b[u], unit_c0(t, u),
                                        nchunks, rho2, c, e, ed, a, bd);
      load_unit(tn, u, b[u]);
      E += e;
      Ed += ed;
      A += a;
      Bd += bd;
    }
    finish_tile(t, E, Ed, A, Bd);
    t = tn;
    tn = claim(t);
  }
  double E = 0.0, Ed = 0.0, A = 0.0, Bd = 0.0;
  const bool whole = (long long)(t + 1) * kTileChunks <= nchunks;
#pragma unroll
  for (int u = 0; u < kUnits; ++u) {
    double e, ed, a, bd;
    if (whole)
      unit_sums<DT, RESID, false, MASK>(Tt, Td, dr.thr_t, dr.thr_d, b[u], unit_c0(t, u),
                                        nchunks, rho2, c, e, ed, a, bd);
    else
      unit_sums<DT, RESID, true, MASK>(Tt, Td, dr.thr_t, dr.thr_d, b[u], unit_c0(t, u),
                                       nchunks, rho2, c, e, ed, a, bd);
    E += e;
    Ed += ed;
    A += a;
    Bd += bd;
  }
  finish_tile(t, E, Ed, A, Bd);
}

// Tile sums of truncated fp32 draw rows. Such rows keep few of their values
// (the others' terms are 0), so a wavefront first gathers, per value slot of
// a unit, the pairs that either row keeps into its LDS buffer (a dropped
// value as -inf, whose term is 0): a float compare of each value against its
// row's threshold value, which is the key compare (order_floor gives the
// least float of the key, and compares keep subnormals), and the slot's
// ballot places the pair. The terms are then formed for the gathered pairs
// only, one per lane in gather order (so every sum is the same from run to
// run), when the buffer could not take another unit and at each tile's end.
// Loads run as in tiles_unscaled: the units of the next tile are issued as
// the units of this one are gathered (after the last tile, the last tile's
// again, so that the loads are unconditional).
constexpr int kSparseCap = 512;    // gathered pairs per wavefront

template <int VEC, bool RESID, int NW>
__device__ __forceinline__ void tiles_sparse32(const double* T2, const void* trow,
                                               const void* drow, const DrawRow& dr, double c,
                                               int ntiles, long long nchunks, TileSums* tiles,
                                               int wid, int lane, float2* buf) {
  using C = Chunk<DT_F32, VEC>;
  static_assert(VEC == 4 && kUnitChunks == 1, "units of one 16-byte chunk per lane and row");
  const double rho2 = RESID ? __builtin_ldexp(dr.rho, int(dr.R_t) - int(dr.R_d)) : 0.0;
  const int st = -int(dr.R_t), sd = -int(dr.R_d);
  const float ft = order_floor<DT_F32>(dr.thr_t);
  const float fd = RESID ? order_floor<DT_F32>(dr.thr_d) : __builtin_inff();
  constexpr float kNegInf = -__builtin_inff();
  const int my_tiles = wid < ntiles ? (ntiles - 1 - wid) / NW + 1 : 0;
  if (my_tiles == 0) return;
  auto unit_c0 = [&](int ti, int u) -> long long {
    return (long long)(wid + ti * NW) * kTileChunks + (long long)u * kWave + lane;
  };
  auto load_unit = [&](int ti, int u, UnitBuf& b) {
    const long long ci = min(unit_c0(ti, u), nchunks - 1);
    b.a[0] = C::load(trow, ci);
    if constexpr (RESID) b.d[0] = C::load(drow, ci);
  };
  uint32_t n = 0;                      // pairs in the buffer (the same in every lane)
  double E = 0.0, Ed = 0.0, A = 0.0, Bd = 0.0;
  auto drain = [&]() {
    wave_sync();
    for (uint32_t e = uint32_t(lane); e < n; e += kWave) {
      const float2 v = buf[e];
      const double et = exp2_tab(double(v.x) * c, T2);
      if constexpr (RESID)
        accum_pair_u(et, exp2_tab(double(v.y) * c, T2), rho2, E, Ed, A, Bd);
      else
        E += et;
    }
    n = 0;
    wave_sync();
  };
  UnitBuf b[kUnits];
#pragma unroll
  for (int u = 0; u < kUnits; ++u) load_unit(0, u, b[u]);
  for (int ti = 0; ti < my_tiles; ++ti) {
    const int tn = ti + 1 < my_tiles ? ti + 1 : ti;
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      if (n > uint32_t(kSparseCap - 4 * kWave)) drain();
      const bool in = unit_c0(ti, u) < nchunks;
      bool kt[4], kd[4], any = false;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        kt[q] = in && __uint_as_float(b[u].a[0][q]) >= ft;
        kd[q] = RESID && in && __uint_as_float(b[u].d[0][q]) >= fd;
        any |= kt[q] || kd[q];
      }
      if (__any(any)) {                // (a unit without a kept value is common with top-k)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bool take = kt[q] || kd[q];
          const unsigned long long m = __ballot(take);
          if (take)
            buf[n + lanes_below(m)] =
                make_float2(kt[q] ? __uint_as_float(b[u].a[0][q]) : kNegInf,
                            kd[q] ? __uint_as_float(b[u].d[0][q]) : kNegInf);
          n += uint32_t(__popcll(m));
        }
      }
      load_unit(tn, u, b[u]);
    }
    drain();
    double Et = wave_sum(E);
    double Edt = 0.0, At = 0.0, Bdt = 0.0;
    if constexpr (RESID) {
      Edt = wave_sum(Ed);
      At = wave_sum(A);
      Bdt = wave_sum(Bd);
    }
    if (lane == 0) {
      TileSums ts;
      ts.E = __builtin_ldexp(Et, st);
      ts.Ed = RESID ? __builtin_ldexp(Edt, sd) : 0.0;
      ts.A = RESID ? __builtin_ldexp(At, st) : 0.0;
      ts.Bd = RESID ? __builtin_ldexp(Bdt, sd) : 0.0;
      tiles[wid + ti * NW] = ts;
    }
    E = Ed = A = Bd = 0.0;
  }
}

// The same for truncated bf16 draw rows: a gathered pair is the two 16-bit
// values in one word (target low, draft high), and its terms come from the
// rows' masked tables (term_unscaled: 0 for a value its row drops), so a
// pair gathered for one row's sake adds nothing for the other. A value is
// gathered when, as a float, it is at least its row's threshold value (the
// key compare). 16 wavefronts x kSparseCap16 words of LDS beside the two
// tables.
constexpr int kSparseCap16 = 256;   // gathered pairs per wavefront

template <bool RESID, int NW>
__device__ __forceinline__ void tiles_sparse16(const double* Tt, const double* Td,
                                               const void* trow, const void* drow,
                                               const DrawRow& dr, double c, int ntiles,
                                               long long nchunks, TileSums* tiles, int wid,
                                               int lane, uint32_t* buf) {
  using C = Chunk<DT_BF16, 8>;
  static_assert(kUnitChunks == 1, "units of one 16-byte chunk per lane and row");
  const double rho2 = RESID ? __builtin_ldexp(dr.rho, int(dr.R_t) - int(dr.R_d)) : 0.0;
  const int st = -int(dr.R_t), sd = -int(dr.R_d);
  const float ft = key_floor(dr.thr_t);
  const float fd = RESID ? key_floor(dr.thr_d) : __builtin_inff();
  const int my_tiles = wid < ntiles ? (ntiles - 1 - wid) / NW + 1 : 0;
  if (my_tiles == 0) return;
  auto unit_c0 = [&](int ti, int u) -> long long {
    return (long long)(wid + ti * NW) * kTileChunks + (long long)u * kWave + lane;
  };
  auto load_unit = [&](int ti, int u, UnitBuf& b) {
    const long long ci = min(unit_c0(ti, u), nchunks - 1);
    b.a[0] = C::load(trow, ci);
    if constexpr (RESID) b.d[0] = C::load(drow, ci);
  };
  uint32_t n = 0;                      // pairs in the buffer (the same in every lane)
  double E = 0.0, Ed = 0.0, A = 0.0, Bd = 0.0;
  auto drain = [&]() {
    wave_sync();
    for (uint32_t e = uint32_t(lane); e < n; e += kWave) {
      const uint32_t w = buf[e];
      const double et = term_unscaled(Tt, w & 0xffffu, c, dr.thr_t);
      if constexpr (RESID)
        accum_pair_u(et, term_unscaled(Td, w >> 16, c, dr.thr_d), rho2, E, Ed, A, Bd);
      else
        E += et;
    }
    n = 0;
    wave_sync();
  };
  UnitBuf b[kUnits];
#pragma unroll
  for (int u = 0; u < kUnits; ++u) load_unit(0, u, b[u]);
  for (int ti = 0; ti < my_tiles; ++ti) {
    const int tn = ti + 1 < my_tiles ? ti + 1 : ti;
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      const bool in = unit_c0(ti, u) < nchunks;
      // value v of the chunk: word v / 2, low half for even v
      auto val = [](const u32x4& r, int v) {
        return __uint_as_float((v & 1) ? r[v >> 1] & 0xffff0000u : r[v >> 1] << 16);
      };
      bool kt[8], kd[8], any = false;
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        kt[v] = in && val(b[u].a[0], v) >= ft;
        kd[v] = RESID && in && val(b[u].d[0], v) >= fd;
        any |= kt[v] || kd[v];
      }
      if (__any(any)) {                // (a unit without a kept value is common with top-k)
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          if (n > uint32_t(kSparseCap16 - kWave)) drain();
          const bool take = kt[v] || kd[v];
          const unsigned long long m = __ballot(take);
          if (take) {
            const uint32_t wt = b[u].a[0][v >> 1], wd = RESID ? b[u].d[0][v >> 1] : 0u;
            const uint32_t lo = (v & 1) ? wt >> 16 : wt & 0xffffu;
            const uint32_t hi = (v & 1) ? wd >> 16 : wd & 0xffffu;
            buf[n + lanes_below(m)] = lo | (hi << 16);
          }
          n += uint32_t(__popcll(m));
        }
      }
      load_unit(tn, u, b[u]);
    }
    drain();
    double Et = wave_sum(E);
    double Edt = 0.0, At = 0.0, Bdt = 0.0;
    if constexpr (RESID) {
      Edt = wave_sum(Ed);
      At = wave_sum(A);
      Bdt = wave_sum(Bd);
    }
    if (lane == 0) {
      TileSums ts;
      ts.E = __builtin_ldexp(Et, st);
      ts.Ed = RESID ? __builtin_ldexp(Edt, sd) : 0.0;
      ts.A = RESID ? __builtin_ldexp(At, st) : 0.0;
      ts.Bd = RESID ? __builtin_ldexp(Bdt, sd) : 0.0;
      tiles[wid + ti * NW] = ts;
    }
    E = Ed = A = Bd = 0.0;
  }
}

// Phase 4 when the tile sums came from tiles_unscaled. Wavefronts 0-3 each
// find the crossing tile from the tile sums (the same arithmetic in each, so
// the same tile); thread t < kTileChunks then re-reads chunk t of that tile,
// forms its 8 exact weights from the table relative to 2^Rt,
//   residual: max(0, Tt - rho2 Td) with the exact rho2 = (St / Sd) 2^(Rt - Rd),
//   bonus or Z = 0 fallback: Tt,
// and a prefix over the chunk sums in token order finds the token, compared
// against u * total scaled by 2^Rt (exact).
template <int DT, int VEC, int NT>
__device__ __forceinline__ void pick_unscaled(int b, int K, int ntiles, long long nchunks,
                                              const DrawRow& dr, const void* trow,
                                              const void* drow, bool residual, const double* Tt,
                                              const double* Td, double c, const TileSums* ts,
                                              const float* __restrict__ uniforms,
                                              int32_t* __restrict__ out_tokens,
                                              DevStats* __restrict__ st, double* aux_z,
                                              PickShared& sh) {
  using C = Chunk<DT, VEC>;
  static_assert(NT >= kTileChunks, "pick needs one thread per tile chunk");
  constexpr int kPW = kTileChunks / kWave;      // wavefronts in the pick
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  int tile = -1, which = 0;
  bool clamp = false, fallback = false;
  double tgt = 0.0, base = 0.0, rho2 = 0.0, zres = -1.0, St = 0.0;
  double wv[C::N];
  double cs = 0.0;
  int lp = -1;
  long long ci = 0;
  bool valid = false;
  if (wid < kPW) {
    double Sd = 0.0;
    for (int t = lane; t < ntiles; t += kWave) {
      St += ts[t].E;
      Sd += ts[t].Ed;
    }
    St = __shfl(wave_sum(St), 0, kWave);
    Sd = __shfl(wave_sum(Sd), 0, kWave);
    const double rho = residual ? St / Sd : 0.0;
    const double drho = dr.rho - rho;
    which = residual ? 1 : 0;
    double total = tiles_total(ts, ntiles, lane, which, drho);
    zres = which ? total : -1.0;
    fallback = residual && !(total > 0.0);
    if (fallback) {
      which = 0;
      total = tiles_total(ts, ntiles, lane, 0, drho);
    }
    tgt = double(uniforms[(long long)b * (K + 1) + K]) * total;
    int last_pos = -1;
    double carry = 0.0;
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
    clamp = tile < 0;
    if (clamp) tile = last_pos;
    rho2 = which ? __builtin_ldexp(rho, int(dr.R_t) - int(dr.R_d)) : 0.0;
    // this thread's chunk of the crossing tile
    ci = (long long)tile * kTileChunks + tid;
    valid = tile >= 0 && ci < nchunks;
    const long long cl = valid ? ci : 0;
    const u32x4 wt = C::load(trow, cl);
    const u32x4 wd = which ? C::load(drow, cl) : wt;
#pragma unroll
    for (int e = 0; e < C::N; ++e) {
      double et, ed = 0.0;
      if constexpr (DT == DT_BF16) {
        et = term_unscaled(Tt, (e & 1) ? wt[e >> 1] >> 16 : wt[e >> 1] & 0xffffu, c, dr.thr_t);
        if (which)
          ed = term_unscaled(Td, (e & 1) ? wd[e >> 1] >> 16 : wd[e >> 1] & 0xffffu, c, dr.thr_d);
      } else {        // fp32: threshold 0 (untruncated rows) keeps every value
        et = order_key<DT_F32>(wt[e]) >= dr.thr_t ? exp2_tab(double(__uint_as_float(wt[e])) * c, Tt)
                                                  : 0.0;
        if (which)
          ed = order_key<DT_F32>(wd[e]) >= dr.thr_d
                   ? exp2_tab(double(__uint_as_float(wd[e])) * c, Tt)
                   : 0.0;
      }
      wv[e] = which ? fmax(__builtin_fma(-rho2, ed, et), 0.0) : et;
      if (!valid) wv[e] = 0.0;
      cs += wv[e];
      lp = wv[e] > 0.0 ? int(ci * VEC + e) : lp;
    }
    // compare in units of 2^-Rt
    tgt = __builtin_ldexp(tgt, int(dr.R_t));
    base = __builtin_ldexp(base, int(dr.R_t));
  }
  const double wincl = wave_incl_scan(cs, lane);
  int wlp = lp;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) wlp = max(wlp, __shfl_xor(wlp, o, kWave));
  if (wid < kPW && lane == kWave - 1) sh.wsum[wid] = wincl;
  if (wid < kPW && lane == 0) sh.wlp[wid] = wlp;
  __syncthreads();
  if (wid < kPW) {
    double before = base;
#pragma unroll
    for (int w = 0; w < kPW; ++w) before += w < wid ? sh.wsum[w] : 0.0;
    const double incl = before + wincl;
    const unsigned long long hit = __ballot(valid && !clamp && incl > tgt);
    int tok = -1;
    if (hit && lane == __ffsll((long long)hit) - 1) {
      double run = incl - cs;
#pragma unroll
      for (int e = 0; e < C::N; ++e) {
        run += wv[e];
        if (tok < 0 && run > tgt) tok = int(ci * VEC + e);
      }
      if (tok < 0) tok = lp;            // the chunk holds positive weight
    }
    tok = __shfl(tok, hit ? __ffsll((long long)hit) - 1 : 0, kWave);
    if (lane == 0) sh.whit[wid] = hit ? tok : -1;
  }
  __syncthreads();
  if (tid == 0) {
    int token = -1, last_elem = -1;
#pragma unroll
    for (int w = 0; w < kPW; ++w) {
      if (token < 0) token = sh.whit[w];
      last_elem = max(last_elem, sh.wlp[w]);
    }
    if (token < 0) token = last_elem;
    out_tokens[(long long)b * (K + 1) + dr.j] = token;
    if (aux_z != nullptr) aux_z[b] = residual ? fmax(zres, 0.0) / St : -1.0;
    if (fallback) atomicAdd(&st->z0_fallbacks, 1ull);
  }
}

// Phases 2-4 for one sequence, given its row statistics in LDS (fR, fS):
// the acceptance scan on wavefront 0, the draw's float64 tile sums of row
// pair j over all wavefronts of the workgroup, then the pick.
// TRUNC: fK holds each row's truncation threshold key and fS its truncated
// normaliser, a sum of level_term (bf16) or value_term (fp32) values; p(d)
// and q(d) are formed with the same terms and are 0 for dropped values. For
// bf16 rows, once j is known T is filled with two tables, the target row's
// and the draft row's, each 0 at the values its row drops; fp32 rows keep the
// one table and the draw compares each value's order key with its row's
// threshold (without TRUNC, T is one table built by the caller, or, with
// TABLE_IN_SCAN, by wavefronts 1.. while wavefront 0 runs the scan).
struct NoSideWork {
  __device__ void operator()() const {}
};

template <int DT, int VEC, int NT, bool TRUNC, bool TABLE_IN_SCAN, class SideWork = NoSideWork>
__device__ __forceinline__ void finish_sequence(
    int b, int K, int V, const void* __restrict__ target, const void* __restrict__ draft,
    const int32_t* __restrict__ tokens, const float* __restrict__ uniforms, float c, double c64,
    Rules sp, int n_half, double* T, const float* fR, const double* fS, const uint32_t* fK,
    TileSums* tiles,
    DrawRow& s_dr, PickShared& psh, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ out_len,
    uint32_t* __restrict__ hist, double* __restrict__ ema, int32_t* __restrict__ steps,
    double decay, DevStats* __restrict__ st, double* aux_p, double* aux_q, double* aux_z,
    float2* sparse = nullptr, const float* fX = nullptr, const int32_t* pre_tok = nullptr,
    const float* pre_u = nullptr, uint32_t* sparse16 = nullptr, int trunc_k = 0,
    SideWork side = SideWork{}, int* tile_ctr = nullptr) {
  using C = Chunk<DT, VEC>;
  constexpr int kW = NT / kWave;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const long long nchunks = V / VEC;
  auto row_base = [&](int r) -> const void* { return row_ptr<DT>(target, draft, b, r, K, V); };
  // ---- 2. acceptance scan on wavefront 0 ----
  // (its emission, histogram and EMA update follow the barrier, off the path
  // to the draw: the EMA update waits on a global load)
  int e_kb = 0, e_n = 0, e_cpos = -1, e_d = 0;
  bool e_bad = true;
  if (wid == 0) {
    int kb, m;
    bool lane_bad;
    stops_of(sp, b, K, kb, m, lane_bad);
    float Rt = 0.0f, Rd = 0.0f;
    double St = 1.0, Sd = 1.0;
    uint32_t kt = 0u, kd = 0u;
    if (lane <= kb) {
      Rt = fR[lane];
      St = fS[lane];
      if constexpr (TRUNC) kt = fK[lane];
      lane_bad |= !finite_pos(St);
    }
    int d = 0;
    double P = 0.0, Q = 1.0;
    bool keep = true, zq = false;
    if (lane < kb) {
      Rd = fR[K + 1 + lane];
      Sd = fS[K + 1 + lane];
      if constexpr (TRUNC) kd = fK[K + 1 + lane];
      lane_bad |= !finite_pos(Sd);
      d = pre_tok != nullptr ? pre_tok[lane] : tokens[(long long)b * K + lane];
      lane_bad |= !(d >= 0 && d < V);   // checked before the gather below
      if (!lane_bad) {
        // the logits at d: from the streaming pass's partials when it kept
        // them (fX), else gathered here
        const float xt = fX != nullptr ? fX[lane] : load_logit<DT>(row_base(lane), d);
        const float xd = fX != nullptr ? fX[K + 1 + lane] : load_logit<DT>(row_base(K + 1 + lane), d);
        const double u = pre_u != nullptr ? pre_u[lane] : uniforms[(long long)b * (K + 1) + lane];
        if constexpr (TRUNC && DT == DT_BF16) {
          // the same level terms as the truncated normalisers; 0 when dropped
          keep = trunc_accept_bf16(xt, xd, Rt, St, kt, Rd, Sd, kd, u, c64, P, Q);
        } else if constexpr (TRUNC) {
          // fp32: the terms the truncation pass summed (0 for -inf); 0 when dropped
          keep = trunc_accept_f32(xt, xd, Rt, St, kt, Rd, Sd, kd, u, c64, P, Q);
        } else {
          keep = accept_position(xt, xd, Rt, St, Rd, Sd, u, c, P, Q);
        }
        zq = keep && Q == 0.0;
      }
    }
    const bool bad = sequence_bad(lane, kb, sp.walk != 0, lane_bad, keep);
    const Walk w = walk_outcome(lane, kb, m, sp.eos, keep, d);
    const int j = w.j;
    // (walk-order reading: nothing past the first rejection was read)
    const bool no_pq = bad || lane >= kb || (sp.walk && lane > j);
    if (aux_p != nullptr && lane < K) aux_p[(long long)b * K + lane] = no_pq ? __builtin_nan("") : P;
    if (aux_q != nullptr && lane < K) aux_q[(long long)b * K + lane] = no_pq ? __builtin_nan("") : Q;
    const float Rtj = __shfl(Rt, j, kWave), Rdj = __shfl(Rd, j, kWave);
    const double Stj = __shfl(St, j, kWave), Sdj = __shfl(Sd, j, kWave);
    const uint32_t ktj = __shfl(kt, j, kWave), kdj = __shfl(kd, j, kWave);
    if (lane == 0) {
      DrawRow dr;
      dr.rho = Stj / Sdj;
      dr.R_t = Rtj;
      dr.R_d = Rdj;
      dr.j = (bad || w.cpos < 0) ? -1 : j;     // -1: invalid, or no correction emitted
      dr.kb = kb;
      dr.thr_t = ktj;
      dr.thr_d = kdj;
      s_dr = dr;
      if (tile_ctr != nullptr) *tile_ctr = 0;   // the draw's first unclaimed tile
      if (dr.j < 0 && aux_z != nullptr) aux_z[b] = -1.0;
    }
    const unsigned long long zqm = __ballot(zq && lane < j);
    if (lane == 0 && !bad && zqm)
      atomicAdd(&st->zero_q_accepts, (unsigned long long)__popcll(zqm));
    e_kb = kb;
    e_n = w.n;
    e_cpos = w.cpos;
    e_d = d;
    e_bad = bad;
  } else {
    if constexpr (TABLE_IN_SCAN && DT == DT_BF16 && VEC == 8) {
      for (int i = tid - kWave; i < kTabMax; i += NT - kWave) T[i] = exp_table_entry(i, c64);
    }
    if constexpr (TABLE_IN_SCAN && DT == DT_F32 && VEC == 4) {
      for (int i = tid - kWave; i < kTab2; i += NT - kWave) T[i] = exp2_frac_entry(i);
    }
  }
  __syncthreads();
  if (wid == 0)
    emit_and_update(lane, b, K, e_kb, e_n, e_cpos, -1, e_bad, out_tokens, out_len, hist, ema,
                    steps, decay, st, e_d, sp.pol);
  const DrawRow dr = s_dr;
  if (dr.j < 0) {
    side();
    return;
  }
  constexpr bool kTab = (DT == DT_BF16 && VEC == 8);
  if constexpr (TRUNC && kTab) {
    for (int i = tid; i < kTabMax; i += NT) {
      const double e = exp_table_entry(i, c64);
      const uint32_t kx = bf16_key(tab_bits(i));
      T[i] = kx >= dr.thr_t ? e : 0.0;
      T[kTabMax + i] = kx >= dr.thr_d ? e : 0.0;
    }
    __syncthreads();
  }
  const double* Tt = T;
  const double* Td = (TRUNC && kTab) ? T + kTabMax : T;

  // ---- 3. draw tile sums of row pair j (or target row K) ----
  DrawRows<DT, VEC> W;
  W.init(target, draft, dr, b, K, V, c64);
  const int ntiles = int((nchunks + kTileChunks - 1) / kTileChunks);
  // bf16 rows with moderate references: table terms without per-term scaling
  // (tiles_unscaled); otherwise every term scaled by 2^-R as it is formed
  bool unscaled = false;
  constexpr bool kFast = (DT == DT_BF16 && VEC == 8) || (DT == DT_F32 && VEC == 4);
  if constexpr (kFast)
    unscaled = fabsf(dr.R_t) <= kUnscaledMaxR && (!W.residual || fabsf(dr.R_d) <= kUnscaledMaxR);
  // with claimed tiles a wavefront with side work does it first and then
  // joins the draw; with fixed tiles the lower wavefronts, which finish their
  // tiles first, do it afterwards
  const bool side_first = tile_ctr != nullptr && unscaled;
  if (side_first) side();
  if (unscaled) {
    // truncated fp32 rows: gather the kept values first (a pair of rows
    // without truncation keeps every value: the dense loop)
    bool gathered = false;
    if constexpr (TRUNC && DT == DT_F32 && VEC == 4) {
      if (sparse != nullptr && (dr.thr_t != 0u || (W.residual && dr.thr_d != 0u))) {
        if (W.residual)
          tiles_sparse32<VEC, true, kW>(Tt, W.trow, W.drow, dr, c64, ntiles, nchunks, tiles, wid,
                                        lane, sparse + wid * kSparseCap);
        else
          tiles_sparse32<VEC, false, kW>(Tt, W.trow, W.drow, dr, c64, ntiles, nchunks, tiles,
                                         wid, lane, sparse + wid * kSparseCap);
        gathered = true;
      }
    }
    if constexpr (TRUNC && DT == DT_BF16 && VEC == 8) {
      // bf16 table lookups are cheap: gathering pays only when the rows keep
      // few values, as a small top-k bounds them (measured at c3: 4-5 us
      // faster with top-k 20 or 50, 3.6 us slower with top-p 0.95 alone,
      // which keeps about 13% of V over both rows)
      if (sparse16 != nullptr && (dr.thr_t != 0u || (W.residual && dr.thr_d != 0u)) &&
          trunc_k >= 1 && trunc_k <= V / 32) {
        if (W.residual)
          tiles_sparse16<true, kW>(Tt, Td, W.trow, W.drow, dr, c64, ntiles, nchunks, tiles, wid,
                                   lane, sparse16 + wid * kSparseCap16);
        else
          tiles_sparse16<false, kW>(Tt, Td, W.trow, W.drow, dr, c64, ntiles, nchunks, tiles, wid,
                                    lane, sparse16 + wid * kSparseCap16);
        gathered = true;
      }
    }
    if constexpr (kFast) {
      constexpr bool kMask = TRUNC && DT == DT_F32;
      if (gathered) {
      } else if (W.residual) {
        tiles_unscaled<DT, VEC, true, kW, kMask>(Tt, Td, W.trow, W.drow, dr, c64, ntiles,
                                                 nchunks, tiles, wid, lane, tile_ctr);
      } else {
        tiles_unscaled<DT, VEC, false, kW, kMask>(Tt, Td, W.trow, W.drow, dr, c64, ntiles,
                                                  nchunks, tiles, wid, lane, tile_ctr);
      }
    }
  } else {
    for (int t = wid; t < ntiles; t += kW) {
      double E = 0.0, Ed = 0.0, A = 0.0, Bd = 0.0;
#pragma unroll
      for (int k = 0; k < kTileChunksPerLane; ++k) {
        const long long ci = (long long)t * kTileChunks + (long long)k * kWave + lane;
        if (ci < nchunks) {
          typename C::raw_t a, d;
          W.load(ci, a, d);
          accum_chunk<DT, VEC>(Tt, Td, n_half, W, a, d, dr.rho, E, Ed, A, Bd);
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
  }
  if (!side_first) side();
  __syncthreads();

  // ---- 4. pick ----
  if constexpr (kFast) {
    if (unscaled) {
      pick_unscaled<DT, VEC, NT>(b, K, ntiles, nchunks, dr, W.trow, W.drow, W.residual, Tt, Td,
                                 c64, tiles,
                        uniforms, out_tokens, st, aux_z, psh);
      return;
    }
  }
  pick_token_block<DT, VEC, NT>(b, K, V, ntiles, dr, W, tiles, uniforms, out_tokens, st, aux_z,
                                psh);
}

template <int DT, int VEC, int U>
__global__ __launch_bounds__(kFBlock) void verify_fused(
    int K, int V, const void* __restrict__ target, const void* __restrict__ draft,
    const int32_t* __restrict__ tokens, const float* __restrict__ uniforms, float c, double c64,
    int n_half, Rules sp, int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_len,
    uint32_t* __restrict__ hist, double* __restrict__ ema, int32_t* __restrict__ steps,
    double decay, DevStats* __restrict__ st, double* aux_p, double* aux_q, double* aux_z) {
  using C = Chunk<DT, VEC>;
  constexpr bool kTab = (DT == DT_BF16 && VEC == 8);
  constexpr bool kTab2F = (DT == DT_F32 && VEC == 4);
  __shared__ double T[kTab ? kTabMax : kTab2F ? kTab2 : 1];
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

  // drafted tokens outside [0, V) at tested positions make the sequence
  // invalid: skip the rows (bad stopping rules are flagged by the scan)
  if (wid == 0) {
    int kb, m;
    bool sbad;
    stops_of(sp, b, K, kb, m, sbad);
    const int d = lane < kb ? tokens[(long long)b * K + lane] : 0;
    const bool bad = __any(lane < kb && !(d >= 0 && d < V));
    if (lane == 0) s_bad_token = bad ? 1 : 0;
  }
  __syncthreads();
  if (s_bad_token) {
    if (wid == 0) {
      if (aux_p != nullptr && lane < K) aux_p[(long long)b * K + lane] = __builtin_nan("");
      if (aux_q != nullptr && lane < K) aux_q[(long long)b * K + lane] = __builtin_nan("");
      if (aux_z != nullptr && lane == 0) aux_z[b] = -1.0;
      emit_and_update(lane, b, K, 0, 0, -1, -1, true, out_tokens, out_len, hist, ema, steps,
                      decay, st, 0, sp.pol);
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
    for (int i = tid; i < kTabMax; i += kFBlock) T[i] = exp_table_entry(i, c64);
  }
  if constexpr (kTab2F) {
    for (int i = tid; i < kTab2; i += kFBlock) T[i] = exp2_frac_entry(i);
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

  finish_sequence<DT, VEC, kFBlock, false, false>(b, K, V, target, draft, tokens, uniforms, c, c64, sp,
                                           n_half, T, fR, fS, nullptr, tiles, s_dr, psh,
                                           out_tokens, out_len, hist, ema,
                                    steps,
                                    decay, st, aux_p, aux_q, aux_z);
}

// After the multi-workgroup streaming pass: one workgroup per sequence
// combines the row partials (fixed order) and runs phases 2-4. TRUNC: after
// a truncation pass instead (sv_trunc.hpp for bf16 rows, sv_trunc32.hpp for
// fp32), with one partial per row whose idx holds the row's threshold key.
// (four wavefronts per SIMD: two 512-thread workgroups share a compute unit)
template <int DT, int VEC, int NT, bool TRUNC>
__global__ __launch_bounds__(NT, 4) void finish_seq(
    int K, int V, int nseg, const RowPart* __restrict__ parts, const void* __restrict__ target,
    const void* __restrict__ draft, const int32_t* __restrict__ tokens,
    const float* __restrict__ uniforms, float c, double c64, int n_half, Rules sp,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_len, uint32_t* __restrict__ hist,
    double* __restrict__ ema, int32_t* __restrict__ steps, double decay,
    DevStats* __restrict__ st, double* aux_p, double* aux_q, double* aux_z,
    const int32_t* __restrict__ trunc_k, MergeJob mj, int claim) {
  constexpr bool kTab = (DT == DT_BF16 && VEC == 8);
  constexpr bool kTab2F = (DT == DT_F32 && VEC == 4);
  __shared__ double T[kTab ? (TRUNC ? 2 * kTabMax : kTabMax) : kTab2F ? kTab2 : 1];
  __shared__ float fR[kFMaxRows];
  __shared__ double fS[kFMaxRows];
  __shared__ uint32_t fK[TRUNC ? kFMaxRows : 1];
  __shared__ TileSums tiles[kFMaxTiles];
  __shared__ DrawRow s_dr;
  __shared__ PickShared psh;
  __shared__ int s_claim;              // the draw's tile claim counter
  // truncated fp32 rows: the gathered value pairs, kSparseCap per wavefront
  __shared__ float2 sparse[TRUNC && kTab2F ? (NT / kWave) * kSparseCap : 1];
  __shared__ uint32_t sparse16[TRUNC && kTab ? (NT / kWave) * kSparseCap16 : 1];
  // after the streaming pass: each row's logit at its drafted token (RowPart
  // m), and the sequence's tokens and uniforms, loaded with the partials
  __shared__ float fX[TRUNC ? 1 : kFMaxRows];
  __shared__ int32_t s_tok[kWave];
  __shared__ float s_u[kWave];
  extern __shared__ uint64_t s_merge[];     // the residual merge's keys (dynamic)
  const int b = blockIdx.x, tid = threadIdx.x;
  const int rows = 2 * K + 1;
  // the residual merge of drafted position wid - 1 on wavefront wid: its
  // lists are loaded now, beside the partials, and merged after the scan
  const int wid = tid / kWave;
  const bool mwave = !TRUNC && mj.lists != nullptr && wid >= 1 && wid <= K;
  MergeHeld held;
  uint64_t* mkeys = mwave ? s_merge + (wid - 1) * merge_lds_words() : s_merge;
  if (mwave) merge_load<DT>(mj, mkeys, b, wid - 1, K, V, held);
  if (tid >= NT - kWave) {             // the last wavefront: tokens and uniforms
    const int l = tid - (NT - kWave);
    if (l < K) s_tok[l] = tokens[(long long)b * K + l];
    if (l <= K) s_u[l] = uniforms[(long long)b * (K + 1) + l];
  }
  for (int r = tid; r < rows; r += NT) {
    float R;
    double S;
    const RowPart* pr = parts + ((long long)b * rows + r) * nseg;
    combine_sum_parts(pr, nseg, R, S);
    fR[r] = R;
    fS[r] = S;
    if constexpr (TRUNC) fK[r] = uint32_t(pr->idx);
    else fX[r] = pr->m;
  }
  __syncthreads();
  // the merge itself: before the wavefront's share of the draw tiles when it
  // claims them (the others take more), after it with fixed tiles, or when
  // the call draws nothing
  auto merge = [&]() {
    if (mwave) {
      wave_sync();
      merge_in_finish<DT>(mj, mkeys, held, sp, b, wid - 1, K, V, target, fS, s_tok);
    }
  };
  // the fp32 table does not depend on the truncation: built during the scan
  finish_sequence<DT, VEC, NT, TRUNC, !TRUNC || DT == DT_F32>(b, K, V, target, draft, tokens, uniforms, c, c64, sp,
                                      n_half, T, fR, fS, fK, tiles, s_dr, psh, out_tokens,
                                      out_len, hist, ema, steps, decay, st, aux_p, aux_q, aux_z,
                                      TRUNC && kTab2F ? sparse : nullptr, TRUNC ? nullptr : fX,
                                      s_tok, s_u, TRUNC && kTab ? sparse16 : nullptr,
                                      trunc_k != nullptr ? trunc_k[b] : 0, merge,
                                      claim ? &s_claim : nullptr);
}

__global__ void zero_hist(uint32_t* hist, int n) {
  if (int(threadIdx.x) < n) hist[threadIdx.x] = 0u;
}

}  // namespace sv
