// Top-k / top-p truncation passes over fp32 logit rows (gfx950).
//
// Two passes: the list pass at the end of this file settles most rows with
// top-k in one read from the row's top k + 1 token keys; the multi-read pass
// described here takes every other row (and every row not in 16-byte chunks).
//
// The rules are those of the bf16 passes in sv_trunc.hpp ([RNR] s.1 and s.2):
// top-k keeps the values at or above the k-th largest, counted with
// multiplicity; top-p then keeps, from the top, whole value levels up to and
// including the first level at which the kept mass reaches top_p of the
// top-k mass. A bf16 row has at most 65536 distinct values, so one bin per
// value is possible there; an fp32 row may hold V distinct values. This pass
// narrows the 32-bit order key of sv_topm.hpp instead, one digit at a time
// (bits 31..20, then 19..10, then 9..0), with one read of the row per digit:
//   read A    the row maximum (and so R = ceil(max * c)), non-finite values,
//             and (top-k) counts by the first digit;
//   reads B-C (top-k) counts by the second digit inside the first digit's
//             cut bin, then by the third inside the second's, which gives the
//             k-th largest key exactly; the same reads sum the masses of the
//             values above the cut bins and inside them;
//   read D    (no top-k) masses by the first digit;
//   reads E-F (top-p) masses by the second and third digit inside the bins
//             where the mass from the top crosses top_p of the top-k mass,
//             skipped when the top-k reads already hold them.
// A bin of the third digit is one value level, so the last walk gives the
// exact threshold key. All reads use cached loads: a row read again is
// usually still in the last-level cache.
//
// Most rows need fewer reads: when the values that can matter number at most
// kT32Buf, one more read copies their keys into LDS and the same digit walks
// run over the copy instead of the row. With top-k they are the values from
// the first digit's cut bin upwards (two reads in all). With top-p alone,
// read A also counts the values by first digit and estimates the row's
// normaliser; a bound on each bin's mass then places the crossing, and the
// values from a bin at or below it upwards are copied (two reads), or, when
// they do not fit, the mass read finds the crossing bin and its values are
// copied (three reads). A row with neither rule (a sequence without
// truncation in a truncated batch) takes one read: read A also sums its
// terms over a running reference.
//
// Masses are softmax terms 2^(x c - R), each rounded once to unsigned 64-bit
// fixed point with FX = 61 - ceil(log2 V) fraction bits (a term is at most
// about 1, so no sum reaches 2^62), and summed with integer LDS atomics. The
// sums are exact: they do not depend on the order in which lanes add, a
// digit's bin sums add up to the coarser digit's bin, and so a finer walk
// always finds the cut the coarser walk located. The rounding costs at most
// V 2^-(FX+1) against a normaliser of at least 1/2, below 1e-8 relative.
//
// Output: one RowPart per needed row, as the bf16 passes write it: S = the
// truncated normaliser relative to 2^R, R, idx = the threshold key (0 keeps
// every value). A row holding NaN or +inf or no finite value, or a sequence
// whose top_p is not > 0, gets S = NaN (the scan then marks the sequence
// invalid). So does a row whose reads disagree (a walk that finds no cut,
// which only a row changed during the call can cause): no bin index is ever
// used unchecked. Rows past a sequence's draft count are not read.
#pragma once

#include "sv_trunc.hpp"

namespace sv {

constexpr int kT32Block = 512;
constexpr int kT32Waves = kT32Block / kWave;
constexpr int kT32Bins1 = 4096;     // first digit: key bits 31..20
constexpr int kT32Bins = 1024;      // second and third digits: bits 19..10 and 9..0
constexpr int kT32Buf = kT32Bins1;  // keys copied into LDS (in the first digit's count array)
constexpr uint32_t kKey32NegInf = 0x80000000u - 0x7f800000u;
constexpr uint32_t kKey32PosInf = 0x80000000u + 0x7f800000u;

typedef unsigned long long u64;

// A term 2^(x c - R) in fixed point with `scale` = 2^FX.
__device__ inline u64 fixed_term(float x, double c64, float R, double scale) {
  return u64(__builtin_rint(value_term(x, c64, R) * scale));
}

// What one read of the row gathers; every field is uniform over the workgroup.
struct T32Sel {
  bool count;                  // counts of the keys with (key & cmask) == cval,
  uint32_t cmask, cval;        //   by bin (key >> cshift) & (kT32Bins - 1)
  int cshift;
  bool m1;                     // first-digit masses of the keys >= m1_floor
  uint32_t m1_floor;
  bool m2;                     // second-digit masses of the keys in first-digit
  uint32_t m2_bin, m2_floor;   //   bin m2_bin that are >= m2_floor
  bool m3;                     // third-digit masses of the keys with key >> 10
  uint32_t m3_sel, m3_floor;   //   == m3_sel that are >= m3_floor
};

__device__ inline T32Sel t32_none() {
  T32Sel s;
  s.count = s.m1 = s.m2 = s.m3 = false;
  s.cmask = s.cval = 0u;
  s.cshift = 0;
  s.m1_floor = s.m2_bin = s.m2_floor = s.m3_sel = s.m3_floor = 0u;
  return s;
}

// the VEC-value chunk ci of an fp32 row with a cached load
template <int VEC>
__device__ inline void t32_load(const void* row, long long ci, uint32_t (&v)[VEC]) {
  if constexpr (VEC == 4) {
    const u32x4 r = reinterpret_cast<const u32x4*>(row)[ci];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = r[q];
  } else {
    v[0] = reinterpret_cast<const uint32_t*>(row)[ci];
  }
}

// One read of the row, f(bits) per value. Four chunks per thread are in
// flight (indexes past the row are clamped for the load and skipped).
template <int VEC, typename F>
__device__ inline void t32_stream(const void* row, long long nchunks, F&& f) {
  constexpr int U = 4;
  for (long long c0 = threadIdx.x; c0 < nchunks; c0 += (long long)U * kT32Block) {
    uint32_t v[U][VEC];
#pragma unroll
    for (int u = 0; u < U; ++u)
      t32_load<VEC>(row, min(c0 + (long long)u * kT32Block, nchunks - 1), v[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c0 + (long long)u * kT32Block >= nchunks) break;
#pragma unroll
      for (int q = 0; q < VEC; ++q) f(v[u][q]);
    }
  }
  __syncthreads();
}

template <int VEC>
__device__ inline void t32_read(const void* row, long long nchunks, const T32Sel& s, double c64,
                                float R, double scale, uint32_t* cnt, u64* m1, u64* m2, u64* m3) {
  t32_stream<VEC>(row, nchunks, [&](uint32_t bits) {
    const uint32_t key = order_key<DT_F32>(bits);
    if (s.count && (key & s.cmask) == s.cval)
      atomicAdd(&cnt[(key >> s.cshift) & uint32_t(kT32Bins - 1)], 1u);
    const bool in1 = s.m1 && key >= s.m1_floor;
    const bool in2 = s.m2 && (key >> 20) == s.m2_bin && key >= s.m2_floor;
    const bool in3 = s.m3 && (key >> 10) == s.m3_sel && key >= s.m3_floor;
    if (in1 || in2 || in3) {
      const u64 t = fixed_term(__uint_as_float(bits), c64, R, scale);
      if (in1) atomicAdd(&m1[key >> 20], t);
      if (in2) atomicAdd(&m2[(key >> 10) & uint32_t(kT32Bins - 1)], t);
      if (in3) atomicAdd(&m3[key & uint32_t(kT32Bins - 1)], t);
    }
  });
}

// The same gathering over n keys held in LDS (each passed on as the bits of
// its value; -0 comes back as +0, which has the same key).
__device__ inline void t32_read_buf(const uint32_t* buf, int n, const T32Sel& s, double c64,
                                    float R, double scale, u64* m1, u64* m2, u64* m3) {
  for (int i = threadIdx.x; i < n; i += kT32Block) {
    const uint32_t key = buf[i];
    const bool in1 = s.m1 && key >= s.m1_floor;
    const bool in2 = s.m2 && (key >> 20) == s.m2_bin && key >= s.m2_floor;
    const bool in3 = s.m3 && (key >> 10) == s.m3_sel && key >= s.m3_floor;
    if (in1 || in2 || in3) {
      const u64 t = fixed_term(order_floor<DT_F32>(key), c64, R, scale);
      if (in1) atomicAdd(&m1[key >> 20], t);
      if (in2) atomicAdd(&m2[(key >> 10) & uint32_t(kT32Bins - 1)], t);
      if (in3) atomicAdd(&m3[key & uint32_t(kT32Bins - 1)], t);
    }
  }
  __syncthreads();
}

__device__ inline uint32_t t32_max(uint32_t v, uint32_t* s) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = max(v, uint32_t(__shfl_xor(int(v), o, kWave)));
  if (lane == 0) s[wid] = v;
  __syncthreads();
  uint32_t t = s[0];
#pragma unroll
  for (int w = 1; w < kT32Waves; ++w) t = max(t, s[w]);
  __syncthreads();
  return t;
}

// Per-walk LDS: reduction slots and the cut thread's answer.
struct T32Walk {
  u64 red[kT32Waves];
  uint32_t red32[kT32Waves];
  double redd[kT32Waves];
  int ired[kT32Waves];
  u64 above;
  double above_d;
  int bin;
};

// The bin at which the sum from the top first reaches goal (> 0): the highest
// bin b whose inclusive sum from the top, over bins >= b, is >= goal. Returns
// b, or -1 when the total stays below goal, and in `above` the sum over the
// bins above b (the total when -1). Thread t holds bins NB/512 * t onwards.
// T: uint32_t (counts), u64 (fixed-point masses) or double (mass bounds).
template <typename T, int NB>
__device__ inline int t32_walk(const T* v, T goal, T& above, T32Walk& w) {
  constexpr int BPT = NB / kT32Block;
  const int tid = threadIdx.x;
  T own = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) own += v[tid * BPT + i];
  T total;
  T abv;
  if constexpr (__is_same(T, double))
    abv = tr_above<T, kT32Waves>(own, w.redd, total);
  else if constexpr (sizeof(T) == 8)
    abv = tr_above<T, kT32Waves>(own, w.red, total);
  else
    abv = tr_above<T, kT32Waves>(own, w.red32, total);
  const int cut = tr_max<kT32Waves>(abv + own >= goal ? tid : -1, w.ired);
  if (tid == cut) {
    T acc = abv;
    for (int i = BPT - 1; i >= 0; --i) {
      const T x = v[tid * BPT + i];
      if (acc + x >= goal) {
        w.bin = tid * BPT + i;
        if constexpr (__is_same(T, double))
          w.above_d = acc;
        else
          w.above = u64(acc);
        break;
      }
      acc += x;
    }
  }
  __syncthreads();
  const int bin = cut >= 0 ? w.bin : -1;
  if constexpr (__is_same(T, double))
    above = cut >= 0 ? w.above_d : total;
  else
    above = cut >= 0 ? T(w.above) : total;
  __syncthreads();
  return bin;
}

template <int NB>
__device__ inline u64 t32_sum(const u64* v, T32Walk& w) {
  constexpr int BPT = NB / kT32Block;
  u64 own = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) own += v[threadIdx.x * BPT + i];
  return tr_sum<u64, kT32Waves>(own, w.red);
}

template <typename T_, int NB>
__device__ inline void t32_clear(T_* a) {
  for (int i = threadIdx.x; i < NB; i += kT32Block) a[i] = T_(0);
}

// ---- the buffered routes: up to kT32Buf keys in LDS ----

// The k-th largest of n keys in LDS (1 <= k <= n), digit by digit with
// counts in the mass arrays; ok = false if a walk finds no cut (not expected).
__device__ inline uint32_t t32_buf_kth(const uint32_t* buf, int n, uint32_t k, u64* m1, u64* m2,
                                       u64* m3, T32Walk& w, bool& ok) {
  const int tid = threadIdx.x;
  t32_clear<u64, kT32Bins1>(m1);
  t32_clear<u64, kT32Bins>(m2);
  t32_clear<u64, kT32Bins>(m3);
  __syncthreads();
  for (int i = tid; i < n; i += kT32Block) atomicAdd(&m1[buf[i] >> 20], 1ull);
  __syncthreads();
  u64 rem = k, abv;
  const int q1 = t32_walk<u64, kT32Bins1>(m1, rem, abv, w);
  ok = q1 >= 0;
  if (!ok) return 0u;
  rem -= abv;
  for (int i = tid; i < n; i += kT32Block) {
    const uint32_t key = buf[i];
    if ((key >> 20) == uint32_t(q1)) atomicAdd(&m2[(key >> 10) & uint32_t(kT32Bins - 1)], 1ull);
  }
  __syncthreads();
  const int q2 = t32_walk<u64, kT32Bins>(m2, rem, abv, w);
  ok = q2 >= 0;
  if (!ok) return 0u;
  rem -= abv;
  const uint32_t sel = (uint32_t(q1) << 10) | uint32_t(q2);
  for (int i = tid; i < n; i += kT32Block) {
    const uint32_t key = buf[i];
    if ((key >> 10) == sel) atomicAdd(&m3[key & uint32_t(kT32Bins - 1)], 1ull);
  }
  __syncthreads();
  const int q3 = t32_walk<u64, kT32Bins>(m3, rem, abv, w);
  ok = q3 >= 0;
  return (sel << 10) | uint32_t(q3 >= 0 ? q3 : 0);
}

// The fixed-point mass of the keys >= floor among n keys in LDS.
__device__ inline u64 t32_buf_mass(const uint32_t* buf, int n, uint32_t floor, double c64, float R,
                                   double scale, T32Walk& w) {
  u64 own = 0;
  for (int i = threadIdx.x; i < n; i += kT32Block) {
    const uint32_t key = buf[i];
    if (key >= floor) own += fixed_term(order_floor<DT_F32>(key), c64, R, scale);
  }
  return tr_sum<u64, kT32Waves>(own, w.red);
}

// The top-p level among n keys in LDS that form a top part of the row (or
// the part of it below a mass already counted): the three digit walks over
// the masses of the keys >= floor. Returns false when their mass stays below
// goal; else thr = the level's key and mass = the mass at or above it.
__device__ inline bool t32_buf_level(const uint32_t* buf, int n, uint32_t floor, u64 goal,
                                     double c64, float R, double scale, u64* m1, u64* m2,
                                     u64* m3, T32Walk& w, uint32_t& thr, u64& mass) {
  t32_clear<u64, kT32Bins1>(m1);
  t32_clear<u64, kT32Bins>(m2);
  t32_clear<u64, kT32Bins>(m3);
  __syncthreads();
  T32Sel sb = t32_none();
  sb.m1 = true;
  sb.m1_floor = floor;
  t32_read_buf(buf, n, sb, c64, R, scale, m1, m2, m3);
  u64 a1, a2, a3;
  const int q1 = t32_walk<u64, kT32Bins1>(m1, goal, a1, w);
  if (q1 < 0) return false;
  sb = t32_none();
  sb.m2 = true;
  sb.m2_bin = uint32_t(q1);
  sb.m2_floor = floor;
  t32_read_buf(buf, n, sb, c64, R, scale, m1, m2, m3);
  const int q2 = t32_walk<u64, kT32Bins>(m2, goal - a1, a2, w);
  if (q2 < 0) return false;
  sb = t32_none();
  sb.m3 = true;
  sb.m3_sel = (uint32_t(q1) << 10) | uint32_t(q2);
  sb.m3_floor = floor;
  t32_read_buf(buf, n, sb, c64, R, scale, m1, m2, m3);
  const int q3 = t32_walk<u64, kT32Bins>(m3, goal - a1 - a2, a3, w);
  if (q3 < 0) return false;
  thr = (uint32_t(q1) << 20) | (uint32_t(q2) << 10) | uint32_t(q3);
  mass = a1 + a2 + a3 + m3[q3];
  return true;
}

// Copy the keys of the row with (key >> 20) in [lo, hi] into buf; returns
// how many there were (more than kT32Buf: only the first kT32Buf stored).
template <int VEC>
__device__ inline uint32_t t32_gather(const void* row, long long nchunks, uint32_t lo, uint32_t hi,
                                      uint32_t* buf, uint32_t* s_n) {
  if (threadIdx.x == 0) *s_n = 0u;
  __syncthreads();
  t32_stream<VEC>(row, nchunks, [&](uint32_t bits) {
    const uint32_t key = order_key<DT_F32>(bits);
    const uint32_t d = key >> 20;
    if (d >= lo && d <= hi) {
      const uint32_t pos = atomicAdd(s_n, 1u);
      if (pos < uint32_t(kT32Buf)) buf[pos] = key;
    }
  });
  const uint32_t n = *s_n;
  __syncthreads();
  return n;
}

// One workgroup per row that sel selects (workgroup i takes candidate i:
// every needed row, or with walk-order reading position 0's rows and then
// the listed sequences' other rows; workgroups past the candidates return at
// once). only_redo: skip the rows the list pass below has settled (flags !=
// kTruncRedo). The list and one-read passes below take their rows the same
// way.
template <int VEC>
__global__ __launch_bounds__(kT32Block) void rowstats_trunc32(
    const void* __restrict__ target, const void* __restrict__ draft, int K, int V, float c,
    double c64, int fx, int use_buf, int only_redo, Trunc tr, const int32_t* __restrict__ kdraft,
    RowPart* __restrict__ parts, uint32_t* __restrict__ hist, int B, RowSel sel,
    uint32_t* __restrict__ clear) {
  __shared__ uint32_t cnt[kT32Bins1];
  __shared__ u64 m1[kT32Bins1];
  __shared__ u64 m2[kT32Bins], m3[kT32Bins];
  __shared__ uint32_t s_u[kT32Waves];
  __shared__ uint32_t s_n;
  __shared__ float s_rf[kT32Waves];
  __shared__ double s_sd[kT32Waves];
  __shared__ T32Walk w;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  if (blockIdx.x == 0 && hist != nullptr && tid <= K) hist[tid] = 0u;
  if (blockIdx.x == 0 && clear != nullptr && tid == 0) *clear = 0u;
  const int rows = 2 * K + 1;
  if ((long long)blockIdx.x >= sel.total(B)) return;   // (walk-order list stage)
  int b, r;
  sel.at(blockIdx.x, K, b, r);
  const long long grow = (long long)b * rows + r;
  if (kdraft != nullptr) {           // rows past the draft count are not needed
    const int kb = kdraft[b];
    if (r <= K ? r > kb : r - K - 1 >= kb) return;
  }
  // after the list pass: only the rows it handed over
  if (only_redo && parts[grow].flags != kTruncRedo) return;
  const void* row = row_ptr<DT_F32>(target, draft, b, r, K, V);
  const long long nchunks = V / VEC;
  const double scale = __builtin_ldexp(1.0, fx);
  const int kk = tr.k != nullptr ? tr.k[b] : 0;
  const bool kon = kk >= 1 && kk < V;
  const float pp = tr.p != nullptr ? tr.p[b] : 1.0f;
  const bool pon = pp < 1.0f;
  auto put = [&](double S, float R, uint32_t thr) {
    if (tid == 0) {
      RowPart p;
      p.S = S;
      p.R = R;
      p.m = 0.0f;
      p.idx = int(thr);
      p.flags = 0;
      parts[grow] = p;
    }
  };

  // ---- read A: maximum, non-finite values, first-digit counts ----
  t32_clear<uint32_t, kT32Bins1>(cnt);
  t32_clear<u64, kT32Bins1>(m1);
  t32_clear<u64, kT32Bins>(m2);
  t32_clear<u64, kT32Bins>(m3);
  __syncthreads();
  uint32_t top = 0u, nonfin = 0u;
  const bool count1 = kon || (pon && use_buf);
  // top-p alone: the row's normaliser too, from float terms whose exponent
  // x c - R carries c as two floats (about 1e-7 relative), over a running
  // reference in registers; it places the top-p goal for the route below
  const bool est = pon && !kon && use_buf;
  // neither rule: the whole row's normaliser from this read, with the terms
  // p(d) and q(d) are formed with (value_term), over a running reference
  const bool plain = !pon && !kon;
  const float c_lo = float(c64 - double(c));
  float Ra = kRefInit;
  double Sa = 0.0;
  t32_stream<VEC>(row, nchunks, [&](uint32_t bits) {
    const uint32_t key = order_key<DT_F32>(bits);
    const bool fin = key > kKey32NegInf && key < kKey32PosInf;
    top = max(top, fin ? key : 0u);
    nonfin |= (key < kKey32NegInf || key >= kKey32PosInf) ? 1u : 0u;
    if (count1) atomicAdd(&cnt[key >> 20], 1u);
    if (est && fin) {                // (-inf adds 0; its product with c_lo may be NaN)
      const float x = __uint_as_float(bits);
      const float xc = x * c;
      if (xc > Ra) {                 // a new reference (rare after the first values)
        const float Rn = ceilf(xc);
        Sa = rescale(Sa, Ra, Rn);
        Ra = Rn;
      }
      Sa += double(__builtin_amdgcn_exp2f(__builtin_fmaf(x, c_lo, __builtin_fmaf(x, c, -Ra))));
    }
    if (plain && fin) {
      const float x = __uint_as_float(bits);
      const float xc = x * c;
      if (xc > Ra) {
        const float Rn = ceilf(xc);
        Sa = rescale(Sa, Ra, Rn);
        Ra = Rn;
      }
      Sa += value_term(x, c64, Ra);
    }
  });
  top = t32_max(top, s_u);
  const bool bad = t32_max(nonfin, s_u) != 0u || top == 0u || !(pp > 0.0f);
  if (bad) return put(__builtin_nan(""), 0.0f, 0u);
  const float R = ceilf(order_floor<DT_F32>(top) * c);
  if (plain) {
    const float Rw = wave_max(Ra);
    const double Sw = wave_sum(rescale(Sa, Ra, Rw));
    if (lane == 0) {
      s_rf[wid] = Rw;
      s_sd[wid] = Sw;
    }
    __syncthreads();
    double S_all = 0.0;
#pragma unroll
    for (int q = 0; q < kT32Waves; ++q) S_all += rescale(s_sd[q], s_rf[q], R);
    return put(S_all, R, 0u);
  }

  // ---- top-p alone: the candidates from the counts and a mass bound ----
  // Bin b of the first digit holds cnt[b] values of at most its largest
  // value v_b, so cnt[b] term(v_b) bounds its mass from above, and the
  // crossing lies at or below the highest bin whose bound from the top
  // reaches the goal. The values of that bin and of as many bins below it as
  // fit in LDS are copied by one more read (a top part of the row), and the
  // three digit walks run over them in LDS with exact masses; when their mass
  // reaches the goal the row is settled, else it takes the mass reads below.
  bool counts_ok = true;             // cnt holds the first-digit counts
  if (est) {
    const float Rw = wave_max(Ra);
    const double Sw = wave_sum(rescale(Sa, Ra, Rw));
    if (lane == 0) {
      s_rf[wid] = Rw;
      s_sd[wid] = Sw;
    }
    __syncthreads();
    double S_all = 0.0;
#pragma unroll
    for (int q = 0; q < kT32Waves; ++q) S_all += rescale(s_sd[q], s_rf[q], R);
    const u64 goal = max(u64(__builtin_ceil(double(pp) * S_all * scale)), 1ull);
    double* ubd = reinterpret_cast<double*>(m1);       // the bounds, in m1's space
    for (int i = tid; i < kT32Bins1; i += kT32Block) {
      const uint32_t n_i = cnt[i];
      double ub = 0.0;
      if (n_i != 0u) {
        const double t = value_term(order_floor<DT_F32>((uint32_t(i) << 20) | 0xfffffu), c64, R);
        ub = double(n_i) * (t * (1.0 + 1e-6) * scale + 1.0);
      }
      ubd[i] = ub;
    }
    __syncthreads();
    double abd;
    const int bu = t32_walk<double, kT32Bins1>(ubd, double(goal), abd, w);   // crossing <= bu
    uint32_t ca;
    const int bf = t32_walk<uint32_t, kT32Bins1>(cnt, uint32_t(kT32Buf) + 1u, ca, w);
    const int bl = bf + 1;           // bins bl.. hold at most kT32Buf values
    if (bu >= 0 && bl <= bu) {
      uint32_t own = 0u;
      for (int i = tid; i < kT32Bins1; i += kT32Block) own += i >= bl ? cnt[i] : 0u;
      const uint32_t n_hi = tr_sum<uint32_t, kT32Waves>(own, w.red32);
      const uint32_t n =
          t32_gather<VEC>(row, nchunks, uint32_t(bl), uint32_t(kT32Bins1 - 1), cnt, &s_n);
      counts_ok = false;
      uint32_t thr;
      u64 mass;
      if (n == n_hi &&
          t32_buf_level(cnt, int(n), 0u, goal, c64, R, scale, m1, m2, m3, w, thr, mass))
        return put(__builtin_ldexp(double(mass), -fx), R, thr);
    }
    // not settled: the mass reads below (m1 is cleared for them)
    t32_clear<u64, kT32Bins1>(m1);
    __syncthreads();
  }

  // ---- top-k: the k-th largest key, digit by digit ----
  uint32_t tk = 0u, b1 = 0u, b2 = 0u;
  if (kon) {
    uint32_t rem = uint32_t(kk), abv;
    const int c1 = t32_walk<uint32_t, kT32Bins1>(cnt, rem, abv, w);   // the total is V >= k
    if (c1 < 0) return put(__builtin_nan(""), 0.0f, 0u);
    b1 = uint32_t(c1);
    const uint32_t n_hi = abv + cnt[b1];   // values in bins b1 and above
    if (use_buf && n_hi <= uint32_t(kT32Buf)) {
      // ---- buffered: every value top-k can keep, sorted in LDS ----
      __syncthreads();                 // cnt[b1] read before cnt holds keys
      const uint32_t n = t32_gather<VEC>(row, nchunks, b1, uint32_t(kT32Bins1 - 1), cnt, &s_n);
      if (n != n_hi) return put(__builtin_nan(""), 0.0f, 0u);
      bool ok;
      tk = t32_buf_kth(cnt, int(n), uint32_t(kk), m1, m2, m3, w, ok);
      if (!ok) return put(__builtin_nan(""), 0.0f, 0u);
      const u64 Sb = t32_buf_mass(cnt, int(n), tk, c64, R, scale, w);
      if (!pon) return put(__builtin_ldexp(double(Sb), -fx), R, tk);
      u64 goal = u64(__builtin_ceil(double(pp) * double(Sb)));
      goal = min(max(goal, 1ull), Sb);
      uint32_t thr;
      u64 mass;
      if (!t32_buf_level(cnt, int(n), tk, goal, c64, R, scale, m1, m2, m3, w, thr, mass))
        return put(__builtin_nan(""), 0.0f, 0u);
      return put(__builtin_ldexp(double(mass), -fx), R, thr);
    }
    rem -= abv;
    t32_clear<uint32_t, kT32Bins>(cnt);
    __syncthreads();
    T32Sel s = t32_none();           // read B
    s.count = true;
    s.cmask = 0xfff00000u;
    s.cval = b1 << 20;
    s.cshift = 10;
    s.m1 = b1 + 1u < uint32_t(kT32Bins1);
    s.m1_floor = (b1 + 1u) << 20;
    s.m2 = true;
    s.m2_bin = b1;
    t32_read<VEC>(row, nchunks, s, c64, R, scale, cnt, m1, m2, m3);
    const int c2 = t32_walk<uint32_t, kT32Bins>(cnt, rem, abv, w);
    if (c2 < 0) return put(__builtin_nan(""), 0.0f, 0u);
    b2 = uint32_t(c2);
    rem -= abv;
    t32_clear<uint32_t, kT32Bins>(cnt);
    __syncthreads();
    s = t32_none();                  // read C
    s.count = true;
    s.cmask = 0xfffffc00u;
    s.cval = (b1 << 20) | (b2 << 10);
    s.cshift = 0;
    s.m3 = true;
    s.m3_sel = (b1 << 10) | b2;
    t32_read<VEC>(row, nchunks, s, c64, R, scale, cnt, m1, m2, m3);
    const int c3 = t32_walk<uint32_t, kT32Bins>(cnt, rem, abv, w);
    if (c3 < 0) return put(__builtin_nan(""), 0.0f, 0u);
    const uint32_t b3 = uint32_t(c3);
    tk = (b1 << 20) | (b2 << 10) | b3;
    // kept masses: drop what lies below the cut at each digit and fold each
    // cut bin into the coarser digit
    for (int i = tid; i < kT32Bins; i += kT32Block)
      if (uint32_t(i) < b3) m3[i] = 0ull;
    __syncthreads();
    const u64 mk2 = t32_sum<kT32Bins>(m3, w);
    for (int i = tid; i < kT32Bins; i += kT32Block)
      if (uint32_t(i) < b2) m2[i] = 0ull;
    if (tid == 0) m2[b2] = mk2;
    __syncthreads();
    const u64 mk1 = t32_sum<kT32Bins>(m2, w);
    if (tid == 0) m1[b1] = mk1;
    __syncthreads();
  } else {
    T32Sel s = t32_none();           // read D
    s.m1 = true;
    t32_read<VEC>(row, nchunks, s, c64, R, scale, cnt, m1, m2, m3);
  }
  const u64 S_k = t32_sum<kT32Bins1>(m1, w);
  if (!pon) return put(__builtin_ldexp(double(S_k), -fx), R, tk);

  // ---- top-p: the level where the mass from the top reaches top_p S_k ----
  u64 goal = u64(__builtin_ceil(double(pp) * double(S_k)));
  goal = min(max(goal, 1ull), S_k);
  u64 a1, a2, a3;
  const int q1 = t32_walk<u64, kT32Bins1>(m1, goal, a1, w);
  if (q1 < 0) return put(__builtin_nan(""), 0.0f, 0u);
  const uint32_t p1 = uint32_t(q1);
  goal -= a1;
  if (!kon && use_buf && counts_ok && cnt[p1] <= uint32_t(kT32Buf)) {
    // ---- buffered: the crossing bin's values, sorted in LDS ----
    const uint32_t n_p = cnt[p1];
    __syncthreads();                   // cnt[p1] read before cnt holds keys
    const uint32_t n = t32_gather<VEC>(row, nchunks, p1, p1, cnt, &s_n);
    if (n != n_p) return put(__builtin_nan(""), 0.0f, 0u);
    uint32_t thr;
    u64 mass;
    if (!t32_buf_level(cnt, int(n), 0u, goal, c64, R, scale, m1, m2, m3, w, thr, mass))
      return put(__builtin_nan(""), 0.0f, 0u);
    return put(__builtin_ldexp(double(a1 + mass), -fx), R, thr);
  }
  const bool same1 = kon && p1 == b1;      // m2 already holds p1's kept masses
  if (!same1) {
    t32_clear<u64, kT32Bins>(m2);
    __syncthreads();
    T32Sel s = t32_none();           // read E
    s.m2 = true;
    s.m2_bin = p1;
    s.m2_floor = tk;
    t32_read<VEC>(row, nchunks, s, c64, R, scale, cnt, m1, m2, m3);
  }
  const int q2 = t32_walk<u64, kT32Bins>(m2, goal, a2, w);
  if (q2 < 0) return put(__builtin_nan(""), 0.0f, 0u);
  const uint32_t p2 = uint32_t(q2);
  goal -= a2;
  if (!(same1 && p2 == b2)) {
    t32_clear<u64, kT32Bins>(m3);
    __syncthreads();
    T32Sel s = t32_none();           // read F
    s.m3 = true;
    s.m3_sel = (p1 << 10) | p2;
    s.m3_floor = tk;
    t32_read<VEC>(row, nchunks, s, c64, R, scale, cnt, m1, m2, m3);
  }
  const int q3 = t32_walk<u64, kT32Bins>(m3, goal, a3, w);
  if (q3 < 0) return put(__builtin_nan(""), 0.0f, 0u);
  const uint32_t p3 = uint32_t(q3);
  const u64 S_p = a1 + a2 + a3 + m3[p3];
  put(__builtin_ldexp(double(S_p), -fx), R, (p1 << 20) | (p2 << 10) | p3);
}

// ---------------------------------------------------------------------------
// Top-p alone in one read (16-byte chunks). With top-p alone the kept set is
// not bounded in advance, but at the shapes this library serves it is a few
// thousand tokens: a sample of the row (one slice of kTPBlock chunks in
// kT32SampleEvery, up to kT32SampleMax slices) counted by the first digit of
// the order key sets a cut, the lower edge of the bin in which the count from
// the top reaches about kT32SampleTarget values of the whole row, and the rest
// of the row then streams once (the sampled slices are not read again). The
// stream forms the row's largest value, the normaliser estimate (float terms
// whose exponent carries c as two floats, c_hi <= c and c_lo = c - c_hi > 0,
// summed in single precision over a lane's 16 values and in float64 across
// groups, over a running reference: about 2e-7 relative) and copies into LDS
// every value at or above the cut: a float compare against the least value of
// the cut's bin (exact for a normal cut value; a cut at zero or a subnormal
// value leaves the row to the multi-read pass), each copied value placed by
// its value slot's ballot, one counter update per wavefront and group. A NaN
// makes the sum NaN and +inf the maximum infinite (and the sum NaN): either
// hands the row over. When no value was lost and the copy's exact fixed-point
// masses reach top_p of the normaliser, the copy (a top part of the row) holds
// the crossing and three digit walks over its keys give the level; the first
// digit is counted relative to the cut (kTPBins1 bins). Otherwise the row
// stays marked kTruncRedo for the multi-read pass.
// 53 KB of LDS (the third digit's masses reuse the second's) and at most 80
// registers give three workgroups per compute unit.
// ---------------------------------------------------------------------------
constexpr int kTPBlock = 512;
constexpr int kTPWaves = kTPBlock / kWave;
constexpr int kTPBins1 = 512;                    // first digit, from the cut up
constexpr int kT32BufOne = 10112;                // values the copy holds
constexpr int kT32SampleEvery = 16;
constexpr int kT32SampleMax = 4;
constexpr int kT32SampleTarget = 6000;

struct TPWalk {
  u64 red[kTPWaves];
  uint32_t red32[kTPWaves];
  int ired[kTPWaves];
  u64 above;
  int bin;
};

// The bin (of NB, NB = kTPBlock or a multiple) at which the sum from the top
// first reaches goal, as t32_walk, over this kernel's workgroup.
template <typename T, int NB>
__device__ inline int tp_walk(const T* v, T goal, T& above, TPWalk& w) {
  constexpr int BPT = NB / kTPBlock;
  static_assert(BPT >= 1 && NB % kTPBlock == 0, "at least one bin per thread");
  const int tid = threadIdx.x;
  T own = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) own += v[tid * BPT + i];
  T total;
  T abv;
  if constexpr (sizeof(T) == 8)
    abv = tr_above<T, kTPWaves>(own, w.red, total);
  else
    abv = tr_above<T, kTPWaves>(own, w.red32, total);
  const int cut = tr_max<kTPWaves>(abv + own >= goal ? tid : -1, w.ired);
  if (tid == cut) {
    T acc = abv;
    for (int i = BPT - 1; i >= 0; --i) {
      const T x = v[tid * BPT + i];
      if (acc + x >= goal) {
        w.bin = tid * BPT + i;
        w.above = u64(acc);
        break;
      }
      acc += x;
    }
  }
  __syncthreads();
  const int bin = cut >= 0 ? w.bin : -1;
  above = cut >= 0 ? T(w.above) : total;
  __syncthreads();
  return bin;
}

template <int VEC>
__global__ __launch_bounds__(kTPBlock, 6) void rowstats_trunc32_topp(
    const void* __restrict__ target, const void* __restrict__ draft, int K, int V, float c,
    double c64, int fx, Trunc tr, const int32_t* __restrict__ kdraft,
    RowPart* __restrict__ parts, int B, RowSel sel) {
  static_assert(VEC == 4, "the one-read route reads 16-byte chunks");
  static_assert(kT32SampleMax == 4, "the sample is one group of four slices");
  __shared__ uint32_t buf[kT32BufOne];   // sample counts by first digit, then the copy
  __shared__ u64 m1[kTPBins1], m2[kT32Bins];    // the third digit reuses m2
  u64* const m3 = m2;
  __shared__ uint32_t s_u[kTPWaves];
  __shared__ uint32_t s_n;
  __shared__ float s_rf[kTPWaves];
  __shared__ double s_sd[kTPWaves];
  __shared__ TPWalk w;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int rows = 2 * K + 1;
  if ((long long)blockIdx.x >= sel.total(B)) return;   // (walk-order list stage)
  int b, r;
  sel.at(blockIdx.x, K, b, r);
  const long long grow = (long long)b * rows + r;
  if (kdraft != nullptr) {           // rows past the draft count are not needed
    const int kb = kdraft[b];
    if (r <= K ? r > kb : r - K - 1 >= kb) return;
  }
  const int kk = tr.k != nullptr ? tr.k[b] : 0;
  const float pp = tr.p != nullptr ? tr.p[b] : 1.0f;
  const bool kon = kk >= 1 && kk < V;
  const bool pon = pp < 1.0f && pp > 0.0f;
  // the rows the list pass handed over (kTruncRedo) that have a rule: top-p
  // alone, or top-k (with or without top-p) beyond the list's size or tied at
  // the k-th value; a row with neither rule or an invalid top_p is the
  // multi-read pass's
  if (!(kon || pon) || !(pp > 0.0f) || parts[grow].flags != kTruncRedo) return;
  // the row's base comes from the arguments and the workgroup index (the
  // same in every lane); chunks are indexed with 32-bit offsets (a row holds
  // fewer than 2^27 chunks)
  const u32x4* row4 = static_cast<const u32x4*>(row_ptr<DT_F32>(target, draft, b, r, K, V));
  const int nchunks = V / VEC;
  const double scale = __builtin_ldexp(1.0, fx);
  // c = c_hi + c_lo with c_hi rounded toward zero, so c_lo >= 0; c_lo is kept
  // at least 2^-126 so that -inf times it stays -inf (never NaN), which adds
  // at most x 2^-126 to a finite exponent x c: nothing at this precision
  float c_hi = float(c64);
  if (double(c_hi) > c64) c_hi = __uint_as_float(__float_as_uint(c_hi) - 1u);
  const float c_lo = fmaxf(float(c64 - double(c_hi)), 0x1p-126f);

  for (int i = tid; i < kT32Bins1; i += kTPBlock) buf[i] = 0u;
  if (tid == 0) s_n = 0u;
  __syncthreads();

  // A lane's group is 16 values (four chunks); values outside the row are
  // -inf, whose term is 0 and which no cut keeps.
  float fmax_l = -__builtin_inff();     // the lane's largest value (NaN passed over)
  float Ra = kRefInit;
  double Sa = 0.0;
  constexpr uint32_t kNegInfBits = 0xff800000u;
  auto sums = [&](const uint32_t (&v)[4][VEC]) {
    // the reference follows the group's largest value (terms <= 1)
    float fmx = __uint_as_float(v[0][0]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = (u == 0 ? 1 : 0); e < VEC; ++e) fmx = fmaxf(fmx, __uint_as_float(v[u][e]));
    fmax_l = fmaxf(fmax_l, fmx);
    const float mx = fmx * c_hi;
    if (mx > Ra) {
      const float Rn = ceilf(mx);
      Sa = rescale(Sa, Ra, Rn);
      Ra = Rn;
    }
    // terms 2^(x c - R) with x c carried as two floats; -inf adds 0, NaN
    // makes the sum NaN
    float g = 0.0f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float x = __uint_as_float(v[u][e]);
        g += __builtin_amdgcn_exp2f(__builtin_fmaf(x, c_lo, __builtin_fmaf(x, c_hi, -Ra)));
      }
    Sa += double(g);
  };
  // copy the values of a group at or above cut_f: each value slot's ballot
  // gives its values' places; one counter update per wavefront. A group that
  // would pass the end of the copy is not written (the count still grows, and
  // the row is handed over).
  auto copy = [&](const uint32_t (&v)[4][VEC], float cut_f) {
    unsigned long long mk[4][VEC];     // each slot's ballot, taken once
    uint32_t tot = 0u;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        mk[u][e] = __ballot(__uint_as_float(v[u][e]) >= cut_f);
        tot += uint32_t(__popcll(mk[u][e]));
      }
    if (tot == 0u) return;
    uint32_t base = 0u;
    if (lane == 0) base = atomicAdd(&s_n, tot);
    base = uint32_t(__builtin_amdgcn_readfirstlane(int(base)));
    if (base + tot > uint32_t(kT32BufOne)) return;
    uint32_t base4 = base * 4u;        // byte offsets: one shift-add per slot
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const unsigned long long m = mk[u][e];
        if (__uint_as_float(v[u][e]) >= cut_f) {
          const uint32_t at = __builtin_amdgcn_mbcnt_hi(
              uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
          *reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(buf) + (base4 + (at << 2))) =
              v[u][e];
        }
        base4 += uint32_t(__popcll(m)) * 4u;
      }
  };

  // The slices in order, the sampled ones skipped (non-sampled slice vs is
  // slice vs + 1 + min(3, vs / 15)), four to a group: whole groups of whole
  // slices first, then the remainder (at most three whole slices and the
  // partial last one) as one group.
  const int nsl = (nchunks + kTPBlock - 1) / kTPBlock;
  const int nfull = nchunks / kTPBlock;
  const int nsamp = min(kT32SampleMax, (nsl + kT32SampleEvery - 1) / kT32SampleEvery);
  const int nv = nsl - nsamp;
  auto slice_of = [](int vs) {
    return vs + 1 + min(kT32SampleMax - 1, vs / (kT32SampleEvery - 1));
  };
  auto whole = [&](int g) { return g + 3 < nv && slice_of(g + 3) < nfull; };
  // chunk indexes past the row are clamped to its last chunk (loaded, not used)
  auto load_group = [&](int g, uint32_t (&v)[4][VEC]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const u32x4 x = row4[min(slice_of(g + u) * kTPBlock + tid, nchunks - 1)];
#pragma unroll
      for (int e = 0; e < VEC; ++e) v[u][e] = x[e];
    }
  };

  // ---- the sample: slices 0, 16, 32, 48 of kTPBlock chunks ----
  uint32_t sk[kT32SampleMax][VEC];
  int n_sampled = 0;
#pragma unroll
  for (int q = 0; q < kT32SampleMax; ++q) {
    const int s0 = kTPBlock * kT32SampleEvery * q;
    n_sampled += max(0, min(kTPBlock, nchunks - s0));
    const u32x4 x = row4[min(s0 + tid, nchunks - 1)];
#pragma unroll
    for (int e = 0; e < VEC; ++e) sk[q][e] = x[e];
  }
#pragma unroll
  for (int q = 0; q < kT32SampleMax; ++q)
    if (kTPBlock * kT32SampleEvery * q + tid >= nchunks) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) sk[q][e] = kNegInfBits;
    }
  sums(sk);
#pragma unroll
  for (int q = 0; q < kT32SampleMax; ++q) {
    const bool in = kTPBlock * kT32SampleEvery * q + tid < nchunks;
#pragma unroll
    for (int e = 0; e < VEC; ++e)
      if (in) atomicAdd(&buf[order_key<DT_F32>(sk[q][e]) >> 20], 1u);
  }
  __syncthreads();
  // with top-k the copy should hold the top k values and a margin
  const long long target_n = kon ? max(kT32SampleTarget, kk + kk / 4 + 64) : kT32SampleTarget;
  const uint32_t want = uint32_t(min(target_n * n_sampled / nchunks + 1, (long long)V));
  uint32_t abv1;
  const int bx = tp_walk<uint32_t, kT32Bins1>(buf, want, abv1, w);
  // the copy starts at the bin in which the sample's count reaches want (at
  // bin 0 when it never does); never at -inf or below
  const uint32_t cut = bx >= 0 ? uint32_t(bx) : 0u;   // (tp_walk ends with a barrier)
  const uint32_t cut_key = max(cut << 20, kKey32NegInf + 1u);
  const float cut_f = order_floor<DT_F32>(cut_key);
  // a cut at zero or at a subnormal value: the float compare and the key
  // order could part there, so the multi-read pass takes the row
  if (!(fabsf(cut_f) >= 0x1p-126f)) return;
  copy(sk, cut_f);

  // ---- the rest of the row, once ----
  int vs = 0;
  // whole groups two at a time, the next group's loads issued before this
  // group's arithmetic (after the last whole group, this group's again: the
  // loads are unconditional, so every wait count stays exact)
  if (whole(0)) {
    uint32_t va[4][VEC], vb[4][VEC];
    load_group(0, va);
    for (;;) {
      const bool nb = whole(vs + 4);
      load_group(nb ? vs + 4 : vs, vb);
      sums(va);
      copy(va, cut_f);
      vs += 4;
      if (!nb) break;
      const bool na = whole(vs + 4);
      load_group(na ? vs + 4 : vs, va);
      sums(vb);
      copy(vb, cut_f);
      vs += 4;
      if (!na) break;
    }
  }
  if (vs < nv) {
    uint32_t v[4][VEC];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ci = vs + u < nv ? slice_of(vs + u) * kTPBlock + tid : nchunks;
      if (ci < nchunks) {
        const u32x4 x = row4[ci];
#pragma unroll
        for (int e = 0; e < VEC; ++e) v[u][e] = x[e];
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) v[u][e] = kNegInfBits;
      }
    }
    sums(v);
    copy(v, cut_f);
  }
  __syncthreads();

  // the row's largest value (as its order key) and the normaliser estimate
  const uint32_t top = t32_max(order_key<DT_F32>(__float_as_uint(fmax_l)), s_u);
  const float Rw = wave_max(Ra);
  const double Sw = wave_sum(rescale(Sa, Ra, Rw));
  if (lane == 0) {
    s_rf[wid] = Rw;
    s_sd[wid] = Sw;
  }
  __syncthreads();
  // +inf, no finite value, or a NaN anywhere (the sum): the multi-read pass
  // reports the row
  if (top >= kKey32PosInf || top <= kKey32NegInf) return;
  const float R = ceilf(order_floor<DT_F32>(top) * c);
  double S_all = 0.0;
#pragma unroll
  for (int q = 0; q < kTPWaves; ++q) S_all += rescale(s_sd[q], s_rf[q], R);
  if (!(S_all > 0.0 && S_all < __builtin_inf())) return;
  const int n = int(s_n);
  const uint32_t topb = top >> 20;
  if (n > kT32BufOne || topb < cut || topb - cut >= uint32_t(kTPBins1)) return;
  if (kon && n < kk) return;         // the copy must hold the top k values

  // ---- digit walks over the copy's keys ----
  for (int i = tid; i < n; i += kTPBlock) buf[i] = order_key<DT_F32>(buf[i]);
  // The key at which the sum from the top over the copy's keys >= floor first
  // reaches goal (counts: each key adds 1; masses: its fixed-point term),
  // digit by digit (the first digit relative to the cut); false when the sum
  // stays below goal. mass = the sum over the keys at or above the level.
  auto walk3 = [&](bool counts, uint32_t floor, u64 goal, uint32_t& thr, u64& mass) -> bool {
    auto add = [&](uint32_t key) -> u64 {
      return counts ? 1ull : fixed_term(order_floor<DT_F32>(key), c64, R, scale);
    };
    for (int i = tid; i < kTPBins1; i += kTPBlock) m1[i] = 0ull;
    for (int i = tid; i < kT32Bins; i += kTPBlock) m2[i] = 0ull;
    __syncthreads();
    for (int i = tid; i < n; i += kTPBlock) {
      const uint32_t key = buf[i];
      const uint32_t bin = (key >> 20) - cut;    // every copied key is >= cut_key
      if (key >= floor && bin < uint32_t(kTPBins1)) atomicAdd(&m1[bin], add(key));
    }
    __syncthreads();
    u64 a1, a2, a3;
    const int q1 = tp_walk<u64, kTPBins1>(m1, goal, a1, w);
    if (q1 < 0) return false;
    const uint32_t d1 = uint32_t(q1) + cut;
    for (int i = tid; i < n; i += kTPBlock) {
      const uint32_t key = buf[i];
      if ((key >> 20) == d1 && key >= floor)
        atomicAdd(&m2[(key >> 10) & uint32_t(kT32Bins - 1)], add(key));
    }
    __syncthreads();
    const int q2 = tp_walk<u64, kT32Bins>(m2, goal - a1, a2, w);
    if (q2 < 0) return false;
    const uint32_t sel = (d1 << 10) | uint32_t(q2);
    for (int i = tid; i < kT32Bins; i += kTPBlock) m3[i] = 0ull;   // (tp_walk ended with a barrier)
    __syncthreads();
    for (int i = tid; i < n; i += kTPBlock) {
      const uint32_t key = buf[i];
      if ((key >> 10) == sel && key >= floor) atomicAdd(&m3[key & uint32_t(kT32Bins - 1)], add(key));
    }
    __syncthreads();
    const int q3 = tp_walk<u64, kT32Bins>(m3, goal - a1 - a2, a3, w);
    if (q3 < 0) return false;
    thr = (sel << 10) | uint32_t(q3);
    mass = a1 + a2 + a3 + m3[q3];
    __syncthreads();                   // m3 read before the next walk clears it
    return true;
  };
  auto put = [&](u64 mass, uint32_t thr) {
    if (tid == 0) {
      RowPart p;
      p.S = __builtin_ldexp(double(mass), -fx);
      p.R = R;
      p.m = 0.0f;
      p.idx = int(thr);
      p.flags = 0;
      parts[grow] = p;
    }
  };
  uint32_t thr;
  u64 mass;
  if (!kon) {
    // top-p alone: the level where the mass from the top reaches top_p of
    // the normaliser estimate
    const u64 goal = max(u64(__builtin_ceil(double(pp) * S_all * scale)), 1ull);
    if (walk3(false, 0u, goal, thr, mass)) put(mass, thr);
    return;
  }
  // top-k: the k-th largest key (every value equal to it is kept), the exact
  // mass at or above it, then with top-p the level where the mass from the
  // top reaches top_p of that mass
  uint32_t tk;
  if (!walk3(true, 0u, u64(kk), tk, mass)) return;
  u64 own = 0;
  for (int i = tid; i < n; i += kTPBlock) {
    const uint32_t key = buf[i];
    if (key >= tk) own += fixed_term(order_floor<DT_F32>(key), c64, R, scale);
  }
  const u64 S_k = tr_sum<u64, kTPWaves>(own, w.red);
  if (!pon) return put(S_k, tk);
  u64 goal = u64(__builtin_ceil(double(pp) * double(S_k)));
  goal = min(max(goal, 1ull), S_k);
  if (walk3(false, tk, goal, thr, mass)) put(mass, thr);
}

// ---------------------------------------------------------------------------
// List pass (16-byte chunks): one read of the row settles most rows. A
// 256-thread workgroup keeps the row's top k + 1 token keys in the top-m
// candidate lists of sv_topm.hpp while it forms, in the same read, the row's
// maximum and checks for NaN and +inf. The merged list, sorted, gives the
// k-th largest value and, when the next token's value differs from it, every
// value top-k keeps; the top-k mass and the top-p level then follow from
// fixed-point prefix masses. A row the list cannot settle (k + 1 >
// kT1MaxWant, a tie across the top-k cut) is marked kTruncRedo for the pass
// above, and so is every row without top-k: with top-p alone the kept set is
// not bounded in advance (a thousand tokens and more at the c5 shape), and a
// row with neither rule needs its whole mass. Keeping the pass to top-k rows
// keeps it at 4 workgroups per compute unit (registers and LDS).
// ---------------------------------------------------------------------------
constexpr int kT1Block = 256;
constexpr int kT1Waves = kT1Block / kWave;
constexpr int kT1Cap = 448;                        // keys per wavefront list
constexpr uint32_t kT1MaxWant = kT1Cap - kWave;    // 384
constexpr int kT1Unroll = 4;                       // chunks per thread per group
constexpr int kT1Per = (kT1MaxWant + kWave - 1) / kWave;   // list entries per lane (6)

// inclusive prefix over the lanes of a wavefront (u64)
__device__ inline u64 wave_incl_scan_u64(u64 v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const u64 u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  return v;
}

template <int VEC>
__global__ __launch_bounds__(kT1Block) void rowstats_trunc32_list(
    const void* __restrict__ target, const void* __restrict__ draft, int K, int V, float c,
    double c64, int fx, Trunc tr, const int32_t* __restrict__ kdraft,
    RowPart* __restrict__ parts, uint32_t* __restrict__ hist, int B, RowSel sel,
    uint32_t* __restrict__ clear) {
  static_assert(VEC == 4, "the list pass reads 16-byte chunks");
  __shared__ uint64_t s_keys[kT1Waves * kT1Cap];    // the lists, then merged in place
  __shared__ uint32_t s_bins[kT1Waves][256];
  __shared__ u32x4 s_stage[kT1Waves][kTopmStage];
  __shared__ uint32_t s_stage_at[kT1Waves][kTopmStage];
  __shared__ u64 s_P[kT1MaxWant];
  __shared__ uint32_t s_count[kT1Waves], s_flag[kT1Waves];
  __shared__ float s_M[kT1Waves];
  __shared__ unsigned long long s_thr;
  __shared__ uint32_t s_n;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  if (blockIdx.x == 0 && hist != nullptr && tid <= K) hist[tid] = 0u;
  if (blockIdx.x == 0 && clear != nullptr && tid == 0) *clear = 0u;
  const int rows = 2 * K + 1;
  if ((long long)blockIdx.x >= sel.total(B)) return;   // (walk-order list stage)
  int b, r;
  sel.at(blockIdx.x, K, b, r);
  const long long grow = (long long)b * rows + r;
  if (kdraft != nullptr) {
    const int kb = kdraft[b];
    if (r <= K ? r > kb : r - K - 1 >= kb) return;
  }
  const int kk = tr.k != nullptr ? tr.k[b] : 0;
  const bool kon = kk >= 1 && kk < V;
  const float pp = tr.p != nullptr ? tr.p[b] : 1.0f;
  const bool pon = pp < 1.0f;
  auto put = [&](double S, float R, uint32_t thr, int flags) {
    if (tid == 0) {
      RowPart p;
      p.S = S;
      p.R = R;
      p.m = 0.0f;
      p.idx = int(thr);
      p.flags = flags;
      parts[grow] = p;
    }
  };
  if (!(pp > 0.0f)) return put(__builtin_nan(""), 0.0f, 0u, 0);
  if (!kon || uint32_t(kk) + 1u > kT1MaxWant) return put(0.0, 0.0f, 0u, kTruncRedo);
  const uint32_t want = uint32_t(kk) + 1u;
  const bool complete = want >= uint32_t(V);         // the list holds every token
  const void* row = row_ptr<DT_F32>(target, draft, b, r, K, V);
  if (tid == 0) s_thr = 0ull;
  __syncthreads();
  TopM<DT_F32> tm;
  tm.init(s_keys + wid * kT1Cap, s_bins[wid], &s_thr, kT1Cap, want, s_stage[wid],
          s_stage_at[wid]);

  // ---- the one read: candidate lists, running-reference normaliser, checks ----
  const long long nchunks = V / VEC;
  constexpr long long kPerIt = (long long)kT1Block * kT1Unroll;
  const long long nit = (nchunks + kPerIt - 1) / kPerIt;
  float gmax = -__builtin_inff();
  uint32_t nonfin = 0u;
  auto load_group = [&](long long it, u32x4 (&raw)[kT1Unroll]) {
#pragma unroll
    for (int u = 0; u < kT1Unroll; ++u) {
      const long long ci = (it * kT1Unroll + u) * kT1Block + tid;
      raw[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row) +
                                          (ci < nchunks ? ci : nchunks - 1));
    }
  };
  auto filter_group = [&](long long it, const u32x4 (&raw)[kT1Unroll]) {
    const long long c0 = it * kT1Unroll * kT1Block + tid;
    float cm[kT1Unroll];
    uint32_t ok = 0;
    float gm = -__builtin_inff();
#pragma unroll
    for (int u = 0; u < kT1Unroll; ++u) {
      const bool in = c0 + (long long)u * kT1Block < nchunks;
      ok |= in ? 1u << u : 0u;
      cm[u] = chunk_max<DT_F32>(raw[u]);
      gm = in ? fmaxf(gm, cm[u]) : gm;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t m = raw[u][q] & 0x7fffffffu;
        nonfin |= (in && (m > 0x7f800000u || raw[u][q] == 0x7f800000u)) ? 1u : 0u;
      }
    }
    gmax = fmaxf(gmax, gm);
    if (it == 0) tm.template seed<kT1Unroll>(cm, ok);
#pragma unroll
    for (int u = 0; u < kT1Unroll; ++u)
      tm.stage_chunk(((ok >> u) & 1u) != 0u && cm[u] >= tm.thr_f, raw[u],
                     uint32_t(c0 + (long long)u * kT1Block));
  };
  {
    u32x4 ga[kT1Unroll], gb[kT1Unroll];
    load_group(0, ga);
#pragma unroll 1
    for (long long it = 0; it < nit; it += 2) {
      load_group(it + 1, gb);
      filter_group(it, ga);
      load_group(it + 2, ga);
      if (it + 1 < nit) filter_group(it + 1, gb);
    }
  }
  tm.flush();
  tm.compact();                                 // at most want keys per wavefront
  {
    const uint32_t fw = wave_or(nonfin);
    const float Mw = wave_max(gmax);
    if (lane == 0) {
      s_M[wid] = Mw;
      s_flag[wid] = fw;
      s_count[wid] = tm.fill;
    }
  }
  __syncthreads();
  float M = s_M[0];
  uint32_t bad = s_flag[0];
#pragma unroll
  for (int w = 1; w < kT1Waves; ++w) {
    M = fmaxf(M, s_M[w]);
    bad |= s_flag[w];
  }
  if (bad != 0u || !(M > -__builtin_inff())) return put(__builtin_nan(""), 0.0f, 0u, 0);
  const float R = ceilf(M * c);

  // ---- merge the lists in place, keep the want largest keys, sort them ----
  // List w (at most want <= kT1MaxWant keys at w kT1Cap) moves down to the
  // end of the lists before it: the target lies below the source, and each
  // 64-key step reads its keys before any later step's writes reach them.
  if (wid == 0) {
    uint32_t n = s_count[0];
#pragma unroll
    for (int w = 1; w < kT1Waves; ++w) {
      const uint32_t cw = s_count[w];
      for (uint32_t e0 = 0; e0 < cw; e0 += kWave) {
        const uint32_t e = e0 + uint32_t(lane);
        const uint64_t k = e < cw ? s_keys[w * kT1Cap + e] : 0ull;
        wave_sync();
        if (e < cw) s_keys[n + e] = k;
        wave_sync();
      }
      n += cw;
    }
    TopM<DT_F32> mg;
    mg.init(s_keys, s_bins[0], &s_thr, kT1Waves * kT1Cap, want);
    mg.fill = n;
    mg.compact();
    if (lane == 0) s_n = mg.fill;
  }
  __syncthreads();
  const int n = int(s_n);
  {
    int n2 = 1;
    while (n2 < n) n2 <<= 1;
    for (int i = n + tid; i < n2; i += kT1Block) s_keys[i] = 0ull;
    __syncthreads();
    for (int k2 = 2; k2 <= n2; k2 <<= 1) {
      for (int j = k2 >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < n2; i += kT1Block) {
          const int l = i ^ j;
          if (l > i) {
            const uint64_t a = s_keys[i], bb = s_keys[l];
            if ((i & k2) == 0 ? a < bb : a > bb) {
              s_keys[i] = bb;
              s_keys[l] = a;
            }
          }
        }
        __syncthreads();
      }
    }
  }
  if (n < int(want) || n < 1) return put(0.0, 0.0f, 0u, kTruncRedo);   // (not expected)
  if (wid != 0) return;

  // ---- wavefront 0: the cut, the masses, the top-p level ----
  auto key32 = [&](int i) -> uint32_t { return uint32_t(s_keys[i] >> 32); };
  const double scale = __builtin_ldexp(1.0, fx);
  uint32_t tk = 0u;
  int n_k = n;                                   // list entries in the top-k set
  {
    tk = key32(kk - 1);
    if (!complete && key32(kk) == tk) {          // the tie may go on past the list
      if (lane == 0) {
        RowPart p;
        p.S = 0.0;
        p.R = 0.0f;
        p.m = 0.0f;
        p.idx = 0;
        p.flags = kTruncRedo;
        parts[grow] = p;
      }
      return;
    }
    n_k = kk;
    if (complete)
      while (n_k < n && key32(n_k) == tk) ++n_k;
  }
  // prefix masses over the list's first n_k entries: lane l holds kT1Per of them
  const int base = lane * kT1Per;
  u64 loc[kT1Per], own = 0;
#pragma unroll
  for (int e = 0; e < kT1Per; ++e) {
    const int i = base + e;
    if (i < n_k) own += fixed_term(order_floor<DT_F32>(key32(i)), c64, R, scale);
    loc[e] = own;
  }
  const u64 incl = wave_incl_scan_u64(own, lane);
  const u64 before = incl - own;
  const u64 total = __shfl(incl, kWave - 1, kWave);
#pragma unroll
  for (int e = 0; e < kT1Per; ++e)
    if (base + e < n_k) s_P[base + e] = before + loc[e];
  wave_sync();
  if (!pon) {
    if (lane == 0) {
      RowPart p;
      p.S = __builtin_ldexp(double(total), -fx);
      p.R = R;
      p.m = 0.0f;
      p.idx = int(tk);
      p.flags = 0;
      parts[grow] = p;
    }
    return;
  }
  // top-p inside the top-k set (rows with top-p alone took the pass above)
  u64 goal = u64(__builtin_ceil(double(pp) * double(total)));
  goal = min(max(goal, 1ull), total);
  int first = -1;
#pragma unroll
  for (int e = kT1Per - 1; e >= 0; --e)
    if (base + e < n_k && s_P[base + e] >= goal) first = base + e;
  const unsigned long long hit = __ballot(first >= 0);
  const int i0 = hit ? __shfl(first, __ffsll((long long)hit) - 1, kWave) : -1;
  int flags = 0;
  uint32_t thr = 0u;
  u64 S_p = 0;
  if (i0 < 0) {
    flags = kTruncRedo;                          // (not expected: P[n_k - 1] = total)
  } else {
    thr = key32(i0);
    int end = i0;                                // last entry of the level
    while (end + 1 < n_k && key32(end + 1) == thr) ++end;
    S_p = s_P[end];
  }
  if (lane == 0) {
    RowPart p;
    p.S = flags ? 0.0 : __builtin_ldexp(double(S_p), -fx);
    p.R = R;
    p.m = 0.0f;
    p.idx = int(thr);
    p.flags = flags;
    parts[grow] = p;
  }
}

// Walk-order reading of truncated fp32 calls, after the truncation passes over
// position 0's rows: lists the sequences whose walk keeps position 0 and that
// have rows past it (k_b >= 1), one thread per sequence, with the scan's own
// truncated fp32 acceptance test (trunc_accept_f32).
__global__ __launch_bounds__(kBlock) void walk_gate_trunc32(
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
  const float xt = load_logit<DT_F32>(row_ptr<DT_F32>(target, draft, b, 0, K, V), d);
  const float xd = load_logit<DT_F32>(row_ptr<DT_F32>(target, draft, b, K + 1, K, V), d);
  double P, Q;
  if (trunc_accept_f32(xt, xd, pt.R, pt.S, uint32_t(pt.idx), pd.R, pd.S, uint32_t(pd.idx),
                       double(uniforms[(long long)b * (K + 1)]), c64, P, Q))
    seqs[atomicAdd(count, 1u)] = b;
}

}  // namespace sv
