// Device helpers for the verification kernels: logit chunk loads and
// unpacking, exact power-of-two rescaling of running sums, and fixed-order
// wavefront / workgroup reductions (results never depend on timing).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kWave = 64;
constexpr int kBlock = 256;                 // threads per workgroup (4 wavefronts)
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kTileChunksPerLane = 4;       // draw tile: 4 chunks per lane of one wavefront
constexpr int kTileChunks = kWave * kTileChunksPerLane;
constexpr float kRefInit = -1.0e30f;        // reference exponent before any finite logit

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

enum { DT_F32 = 0, DT_BF16 = 1 };

// A chunk is the unit one lane loads at once: 16 bytes on the vector path
// (8 bf16 or 4 fp32 logits), one element on the scalar path.
template <int DT, int VEC> struct Chunk;

template <> struct Chunk<DT_BF16, 8> {
  static constexpr int N = 8;
  using raw_t = u32x4;
  __device__ static inline raw_t load(const void* row, long long c) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row) + c);
  }
  __device__ static inline void unpack(const raw_t& r, float (&x)[N]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = __uint_as_float(r[k] << 16);
      x[2 * k + 1] = __uint_as_float(r[k] & 0xffff0000u);
    }
  }
  // true iff any element is NaN (exponent all ones, mantissa non-zero)
  __device__ static inline uint32_t nan_bits(const raw_t& r) {
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t lo = r[k] & 0x7fffu, hi = (r[k] >> 16) & 0x7fffu;
      m |= (lo > 0x7f80u) | (hi > 0x7f80u);
    }
    return m;
  }
};

template <> struct Chunk<DT_F32, 4> {
  static constexpr int N = 4;
  using raw_t = u32x4;
  __device__ static inline raw_t load(const void* row, long long c) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row) + c);
  }
  __device__ static inline void unpack(const raw_t& r, float (&x)[N]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = __uint_as_float(r[k]);
  }
  __device__ static inline uint32_t nan_bits(const raw_t& r) {
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) m |= ((r[k] & 0x7fffffffu) > 0x7f800000u);
    return m;
  }
};

template <> struct Chunk<DT_BF16, 1> {
  static constexpr int N = 1;
  using raw_t = uint32_t;
  __device__ static inline raw_t load(const void* row, long long c) {
    return reinterpret_cast<const uint16_t*>(row)[c];
  }
  __device__ static inline void unpack(const raw_t& r, float (&x)[N]) {
    x[0] = __uint_as_float(r << 16);
  }
  __device__ static inline uint32_t nan_bits(const raw_t& r) { return (r & 0x7fffu) > 0x7f80u; }
};

template <> struct Chunk<DT_F32, 1> {
  static constexpr int N = 1;
  using raw_t = uint32_t;
  __device__ static inline raw_t load(const void* row, long long c) {
    return reinterpret_cast<const uint32_t*>(row)[c];
  }
  __device__ static inline void unpack(const raw_t& r, float (&x)[N]) { x[0] = __uint_as_float(r); }
  __device__ static inline uint32_t nan_bits(const raw_t& r) {
    return (r & 0x7fffffffu) > 0x7f800000u;
  }
};

template <int DT> __device__ inline float load_logit(const void* row, long long v) {
  if constexpr (DT == DT_BF16)
    return __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(row)[v]) << 16);
  else
    return reinterpret_cast<const float*>(row)[v];
}

template <int DT> constexpr int elem_bytes() { return DT == DT_BF16 ? 2 : 4; }

// One softmax term relative to an integer reference exponent R:
// 2^(x * c - R), where c = log2(e) / T. The same expression (one fma, one
// hardware exp2) is used wherever a term is formed, so a row and its gathered
// element, and two bitwise-equal rows, give bitwise-equal results.
__device__ inline float term(float x, float c, float R) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf(x, c, -R));
}

// 2^a in float64: a = n + f with n = rint(a), |f| <= 1/2, 2^f by its Taylor
// series (Horner), then an exact scaling by 2^n. Arguments below -1100
// (including -inf) give 0. Used where single-precision exponentials are not
// accurate enough: the per-token weights of the correction/bonus draw, whose
// prefix sums are compared with a uniform at the resolution of one token's
// share of a large vocabulary. DEG = 9 (about 1e-11 relative at |f| = 1/2,
// far less near f = 0) for per-token use; DEG = 12 (below 2e-16) for the
// tables built once per workgroup.
template <int DEG>
__device__ inline double exp2_taylor(double a) {
  constexpr double L = 0.6931471805599453094172321214581766;   // ln 2
  double cf[DEG + 1];
  cf[0] = 1.0;
#pragma unroll
  for (int k = 1; k <= DEG; ++k) cf[k] = cf[k - 1] * L / k;
  a = fmax(a, -1100.0);
  const double n = __builtin_rint(a);
  const double f = a - n;
  double p = cf[DEG];
#pragma unroll
  for (int k = DEG - 1; k >= 0; --k) p = __builtin_fma(p, f, cf[k]);
  return __builtin_ldexp(p, int(n));
}
__device__ inline double exp2_acc(double a) { return exp2_taylor<9>(a); }
__device__ inline double exp2_acc_hi(double a) { return exp2_taylor<12>(a); }

// Scale a float64 sum by 2^(from - to) exactly (from <= to, both integers or
// the initial reference). Saturating conversion keeps the empty state at 0.
__device__ inline double rescale(double s, float from, float to) {
  float d = fmaxf(from - to, -2000.0f);   // also maps NaN (inf - inf) to -2000
  return __builtin_ldexp(s, int(d));
}

// ---- wavefront reductions (fixed butterfly order) ----

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ inline double wave_sum(double v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ inline uint32_t wave_or(uint32_t v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v |= __shfl_xor(v, o, kWave);
  return v;
}

// (value, index) max; equal values keep the lower index. Index -1 = empty.
__device__ inline void argmax_combine(float& m, int& i, float m2, int i2) {
  bool take = (i2 >= 0) && (i < 0 || m2 > m || (m2 == m && i2 < i));
  m = take ? m2 : m;
  i = take ? i2 : i;
}

__device__ inline void wave_argmax(float& m, int& i) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    float m2 = __shfl_xor(m, o, kWave);
    int i2 = __shfl_xor(i, o, kWave);
    argmax_combine(m, i, m2, i2);
  }
}

// Inclusive prefix sum over the lanes of a wavefront (Hillis-Steele).
__device__ inline double wave_incl_scan(double v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    double u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  return v;
}

// Per-row partial produced by the streaming pass, one per (row, segment).
struct RowPart {
  double S;      // sum of 2^(x*c - R) over the segment (stochastic rows)
  float R;       // integer reference exponent of S
  float m;       // max raw logit (greedy/margin rows)
  int idx;       // lowest index attaining m (greedy/margin rows), -1 if none
  int flags;     // bit 0: NaN seen (greedy/margin rows)
};

// A row's normaliser from its segments' partials: common reference, exact
// rescale, fixed order.
__device__ inline void combine_sum_parts(const RowPart* p, int nseg, float& R, double& S) {
  R = p[0].R;
  for (int s = 1; s < nseg; ++s) R = fmaxf(R, p[s].R);
  S = 0.0;
  for (int s = 0; s < nseg; ++s) S += rescale(p[s].S, p[s].R, R);
}

__device__ inline bool finite_pos(double S) { return S > 0.0 && S < __builtin_inf(); }

// A row's maximum, lowest argmax and NaN flag from its segments' partials.
__device__ inline void combine_max_parts(const RowPart* p, int nseg, float& m, int& idx,
                                         int& nan) {
  m = p[0].m;
  idx = p[0].idx;
  nan = p[0].flags;
  for (int s = 1; s < nseg; ++s) {
    argmax_combine(m, idx, p[s].m, p[s].idx);
    nan |= p[s].flags;
  }
}

// The acceptance test of one drafted position ([SMB] "The Guarantee Behind
// Rejection Sampling"; [RNR] s.2): from the logits of its drafted token in
// the target and draft rows and the rows' normalisers, P = p(d), Q = q(d);
// the draft is kept iff P >= Q or u < P / Q. Every place that takes this
// decision (the scans and the walk-order gate of the streaming pass) calls
// this one function, so they agree bit for bit.
__device__ inline bool accept_position(float xt, float xd, float Rt, double St, float Rd,
                                       double Sd, double u, float c, double& P, double& Q) {
  P = double(term(xt, c, Rt)) / St;
  Q = double(term(xd, c, Rd)) / Sd;
  return (P >= Q) || (u < P / Q);
}

// Final statistics of the row a sequence draws from, left by the scan for the
// draw kernels.
struct DrawRow {
  double rho;    // S_t / S_d from the streaming pass: sign test of p - q
  float R_t, R_d;
  int j;         // rejection index (kb = bonus), -1 = nothing to draw
  int kb;        // drafts tested in this sequence
  uint32_t thr_t, thr_d;   // truncation: smallest kept value key of each row (0 = all)
};

// Per-tile sums left by the draw's first phase, all relative to the row
// references R_t, R_d, with rho the streaming pass's S_t / S_d: E = sum e_t(v),
// Ed = sum e_d(v), and over the tokens with e_t(v) > rho * e_d(v):
// A = sum (e_t(v) - rho * e_d(v)), Bd = sum e_d(v). For the exact ratio rho',
// the tile's residual weight is A + (rho - rho') * Bd.
struct TileSums {
  double E, Ed, A, Bd;
};

struct DevStats {
  unsigned long long sequences;
  unsigned long long invalid;
  unsigned long long zero_q_accepts;
  unsigned long long z0_fallbacks;
};

}  // namespace sv
