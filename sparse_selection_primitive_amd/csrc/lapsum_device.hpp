// Device building blocks of the gfx950 Fast LapSum kernels.
//
// Method: "Fast LapSum: Exact Differentiable Top-k at Million Scale",
//   section 2.1 (eq. (1): p_i = F((r_i - b)/t), F the unit Laplace CDF;
//   eq. (2): sum_i p_i = k fixes b), section 2.2 (full-sort solver: sort,
//   one stable prefix/suffix scan giving the threshold curve, index lookup of
//   the balancing interval, closed-form root; probabilistic bracketing).
//
// Numerics used by every solver in this library:
//   * Sums of shifted exponentials are carried as "anchored" pairs: a fp32
//     anchor key a and an fp64 sum s of exp(+-(x_i - a)/t) over a range whose
//     terms are all <= 1.  Re-anchoring multiplies by exp of a key difference,
//     computed from the two fp32 keys (never as a product of many step
//     multipliers), so every term keeps a relative error of a few 1e-7
//     whatever the number of elements in between.  s == 0 marks an empty
//     range (a non-empty range always contains its anchor's term, 1).
//   * The threshold curve is the budget at the sorted knots,
//       g_j = f(s_j) = (P_j - 1)/2 + #{i >= j} - S_j/2,
//     with P_j (resp. S_j) the anchored sum of everything at or below
//     (at or above) knot j.  The root inside the located interval solves
//       P/(2y) + c - Q y/2 = k,   y = exp((b - x)/t),
//     for an anchor knot x, P = sum_{below} e^{(s_i-x)/t},
//     Q = sum_{above} e^{-(s_i-x)/t} and c = #above: the positive root of
//     Q y^2 - 2(c-k) y - P = 0, taken in log form without cancellation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define LDEV __device__ __forceinline__

namespace lapsum {

constexpr double kLog2e = 1.4426950408889634074;
constexpr int kWave = 64;

// Budget and temperature of one row: from the optional per-row arrays,
// else the call's (host-checked) scalars.  Per-row values outside
// 0 < k < n, 0 < t < inf (NaN included) are replaced by k = n/2, t = 1, so
// every kernel runs its normal course; the row's outputs are then set to
// NaN and the row flagged invalid.  Returns whether the values were valid.
LDEV bool row_params(const double *krow, const double *trow, int64_t row, int64_t n, double &k, double &t) {
  if (krow) k = krow[row];
  if (trow) t = trow[row];
  const bool ok = k > 0.0 && k < (double)n && t > 0.0 && t < INFINITY;
  if (!ok) {
    k = 0.5 * (double)n;
    t = 1.0;
  }
  return ok;
}

// ------------------------------------------------------ LDS poisoning
// Debug build (compiled with LAPSUM_LDS_POISON): every byte of an LDS object
// is set to 0xFF at kernel entry (NaN as fp32 and fp64, all ones as an
// integer), so a read of LDS that no thread of the launch wrote first shows
// up as NaN or a wrong count in the outputs.  Every thread of the workgroup
// must call it.  In the product build it compiles to nothing.
template <class T>
LDEV void lds_poison(T &obj) {
#ifdef LAPSUM_LDS_POISON
  static_assert(sizeof(T) % 4 == 0, "LDS objects are poisoned a word at a time");
  uint32_t *q = reinterpret_cast<uint32_t *>(&obj);
  for (uint32_t i = threadIdx.x; i < (uint32_t)(sizeof(T) / 4); i += blockDim.x) q[i] = 0xFFFFFFFFu;
  __syncthreads();
#else
  (void)obj;
#endif
}

// ------------------------------------------------------------------ keys
// Order-preserving map of fp32 onto uint32: the unsigned order of keys is
// the numeric order of finite values (-0.0 sorts just below +0.0).
LDEV uint32_t key_of(float x) {
  uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
LDEV float value_of(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}
LDEV uint32_t to_bits(uint32_t v) { return v; }
LDEV uint32_t to_bits(float v) { return __float_as_uint(v); }
template <class T>
LDEV T from_bits(uint32_t v) {
  if constexpr (sizeof(T) == 4 && T(0.5) != T(0)) return __uint_as_float(v);
  else return v;
}

// exp(d/t) for d <= 0, with c = log2(e)/t: the product in fp64, the power of
// two by the hardware exp2 in fp32 (results below 2^-126 flush toward 0,
// which only drops terms far below the anchored sums' unit term).
LDEV float wexp(double d, double c) { return __builtin_amdgcn_exp2f((float)(d * c)); }
LDEV float wexpf(float d, float cf) { return __builtin_amdgcn_exp2f(d * cf); }

// ------------------------------------------------------- anchored sums
struct Pre {  // prefix-type: s = sum exp((x_i - a)/t) over a range ending at its anchor a
  float a;
  double s;
};
struct Suf {  // suffix-type: s = sum exp(-(x_i - a)/t) over a range starting at its anchor a
  float a;
  double s;
};

// left range followed by right range
LDEV Pre join(Pre l, Pre r, double c) {
  if (r.s == 0.0) return l;
  if (l.s == 0.0) return r;
  return Pre{r.a, l.s * (double)wexp((double)l.a - (double)r.a, c) + r.s};
}
LDEV Suf join(Suf l, Suf r, double c) {
  if (l.s == 0.0) return r;
  if (r.s == 0.0) return l;
  return Suf{l.a, l.s + r.s * (double)wexp((double)l.a - (double)r.a, c)};
}

// ---------------------------------------------------- closed-form root
// b = x + t ln y, y the positive root of Q y^2 - 2(c-k) y - P = 0, given
// ln P and ln Q (either may be -inf for an empty side).  Logs are used
// throughout so that sums shifted by e^{-delta/t} far below the fp32/fp64
// range (t far below the gaps between scores) still place b correctly.
// With a = ln|c-k| and h = ln sqrt(PQ), ln(|c-k| + sqrt((c-k)^2 + PQ)) is
// m + ln(u + sqrt(1 + r^2)), m = max(a, h), r = e^{min(a,h) - m} <= 1 and
// u = 1 when a >= h, else r: no digits are lost to a tiny or huge PQ.
//
// Accuracy: b only needs ln y to about 1e-7 absolute (an error d in ln y
// moves b by t*d and the budget by at most d relative), so the logs below
// take the binary exponent exactly in fp64 and only the log of a mantissa in
// [0.5, 1) or of a value in [1, 1 + sqrt 2] in fp32 (absolute error ~1e-7);
// every sum and difference stays in fp64.
constexpr double kLn2 = 0.69314718055994530942;
LDEV double log_pos(double v) {  // ln v, v > 0 finite
  int ex;
  const double mt = frexp(v, &ex);  // v = mt 2^ex, mt in [0.5, 1)
  return (double)ex * kLn2 + (double)__logf((float)mt);
}
LDEV double solve_root(double x, double lnP, double lnQ, double cnt, double k, double t) {
  const double e = cnt - k;
  const double h = 0.5 * (lnP + lnQ);
  const double a = e != 0.0 ? log_pos(fabs(e)) : -INFINITY;
  const double m = fmax(a, h);
  double L = -INFINITY;
  if (m != -INFINITY) {
    const float r = __expf((float)(fmin(a, h) - m));  // in [0, 1]
    L = m + (double)__logf((a >= h ? 1.0f : r) + sqrtf(1.0f + r * r));
  }
  const double lny = (e >= 0.0) ? (L - lnQ) : (lnP - L);
  return x + t * lny;
}
LDEV double safe_log(double v) { return v > 0.0 ? log_pos(v) : -INFINITY; }

// --------------------------------------------------------- wave shuffles
// DPP lane move inside rows of 16 lanes (every pattern used here reads a
// lane of the same row, so no lane is left without a source)
template <int CTRL>
LDEV uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
template <int PATTERN>
LDEV uint32_t swz(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, PATTERN);
}
// value held by lane (lane ^ MASK) of the same wave
template <int MASK>
LDEV uint32_t xor_lanes(uint32_t v) {
  if constexpr (MASK == 1) return dpp<0xB1>(v);        // quad_perm [1,0,3,2]
  else if constexpr (MASK == 2) return dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  else if constexpr (MASK == 3) return dpp<0x1B>(v);   // quad_perm [3,2,1,0]
  else if constexpr (MASK == 7) return dpp<0x141>(v);  // row_half_mirror
  else if constexpr (MASK == 8) return dpp<0x128>(v);  // row_ror:8 (within 16 lanes)
  else if constexpr (MASK == 15) return dpp<0x140>(v); // row_mirror
  else if constexpr (MASK < 32) return swz<(MASK << 10) | 0x1F>(v);  // bit-mask swizzle
  else return (uint32_t)__shfl_xor((int)v, MASK, kWave);
}

LDEV int lane_id() { return (int)__lane_id(); }

// Row of this workgroup in a launch whose rows are folded over grid.y and
// grid.z (rows_grid in lapsum_internal.hpp); may be past the last row.
LDEV int64_t grid_row() { return (int64_t)blockIdx.y + (int64_t)gridDim.y * (int64_t)blockIdx.z; }

// ------------------------------------------------- whole-wave helpers
// A 64-lane wave is four DPP rows of 16 lanes.  Butterflies and scans run
// inside the rows on DPP moves; the four row results are then read once each
// with v_readlane (uniform values) and combined on every lane, so no step
// of a wave-wide sum, extreme or scan goes through LDS.
LDEV uint32_t read_lane(uint32_t v, int l) { return (uint32_t)__builtin_amdgcn_readlane((int)v, l); }
LDEV float read_lane(float v, int l) { return __uint_as_float(read_lane(__float_as_uint(v), l)); }
LDEV int read_lane(int v, int l) { return (int)read_lane((uint32_t)v, l); }
LDEV unsigned long long read_lane(unsigned long long v, int l) {
  return ((unsigned long long)read_lane((uint32_t)(v >> 32), l) << 32) | read_lane((uint32_t)v, l);
}
LDEV double read_lane(double v, int l) {
  return __longlong_as_double((long long)read_lane((unsigned long long)__double_as_longlong(v), l));
}
template <int CTRL>
LDEV unsigned long long dpp64(unsigned long long v) {
  return ((unsigned long long)dpp<CTRL>((uint32_t)(v >> 32)) << 32) | dpp<CTRL>((uint32_t)v);
}
template <int CTRL>
LDEV double dpp64(double v) {
  return __longlong_as_double((long long)dpp64<CTRL>((unsigned long long)__double_as_longlong(v)));
}
// value of lane (lane ^ M) of the same row, M = 1, 2, 4, 8 (a butterfly
// pairing: any pairing of the halves serves a commutative reduction)
template <int M>
LDEV uint32_t row_pair(uint32_t v) {
  return xor_lanes<M == 4 ? 7 : (M == 8 ? 15 : M)>(v);
}
template <int M>
LDEV unsigned long long row_pair(unsigned long long v) {
  return ((unsigned long long)row_pair<M>((uint32_t)(v >> 32)) << 32) | row_pair<M>((uint32_t)v);
}
template <int M>
LDEV double row_pair(double v) {
  return __longlong_as_double((long long)row_pair<M>((unsigned long long)__double_as_longlong(v)));
}
template <int M>
LDEV int row_pair(int v) {
  return (int)row_pair<M>((uint32_t)v);
}
// reduction over the whole wave (op commutative and associative), on every lane
template <class T, class Op>
LDEV T wave_reduce(T v, Op op) {
  v = op(v, row_pair<1>(v));
  v = op(v, row_pair<2>(v));
  v = op(v, row_pair<4>(v));
  v = op(v, row_pair<8>(v));
  return op(op(read_lane(v, 0), read_lane(v, 16)), op(read_lane(v, 32), read_lane(v, 48)));
}

template <int CTRL>
LDEV Pre dpp_pre(Pre x) {
  return Pre{__uint_as_float(dpp<CTRL>(__float_as_uint(x.a))), dpp64<CTRL>(x.s)};
}
template <int CTRL>
LDEV Suf dpp_suf(Suf x) {
  return Suf{__uint_as_float(dpp<CTRL>(__float_as_uint(x.a))), dpp64<CTRL>(x.s)};
}
// inclusive scans inside each row: a lane whose source lies before (after)
// its row start (end) reads zeros, i.e. an empty range
template <int OFF>
LDEV void row_pre_steps(Pre &inc, double c) {
  if constexpr (OFF < 16) {
    inc = join(dpp_pre<0x110 + OFF>(inc), inc, c);  // row_shr:OFF
    row_pre_steps<2 * OFF>(inc, c);
  }
}
template <int OFF>
LDEV void row_suf_steps(Suf &inc, double c) {
  if constexpr (OFF < 16) {
    inc = join(inc, dpp_suf<0x100 + OFF>(inc), c);  // row_shl:OFF
    row_suf_steps<2 * OFF>(inc, c);
  }
}
// inclusive sum of v over the lanes up to this one (whole wave)
LDEV uint32_t wave_incl_scan(uint32_t v) {
  v += dpp<0x111>(v);  // row_shr:1 (a lane before its row's start reads 0)
  v += dpp<0x112>(v);
  v += dpp<0x114>(v);
  v += dpp<0x118>(v);
  const uint32_t r0 = read_lane(v, 15), r1 = read_lane(v, 31), r2 = read_lane(v, 47);
  const int row = lane_id() >> 4;
  return v + (row == 0 ? 0u : (row == 1 ? r0 : (row == 2 ? r0 + r1 : r0 + r1 + r2)));
}
// P-type scan over the wave: returns the inclusive value, *ex the exclusive
LDEV Pre wave_scan(Pre x, double c, Pre *ex) {
  const int row = lane_id() >> 4;
  Pre inc = x;
  row_pre_steps<1>(inc, c);
  const Pre t0{read_lane(inc.a, 15), read_lane(inc.s, 15)};
  const Pre t01 = join(t0, Pre{read_lane(inc.a, 31), read_lane(inc.s, 31)}, c);
  const Pre t012 = join(t01, Pre{read_lane(inc.a, 47), read_lane(inc.s, 47)}, c);
  const Pre before = row == 0 ? Pre{0.0f, 0.0} : (row == 1 ? t0 : (row == 2 ? t01 : t012));
  *ex = join(before, dpp_pre<0x111>(inc), c);
  return join(before, inc, c);
}
// S-type scan over the wave (from the last lane down)
LDEV Suf wave_scan(Suf x, double c, Suf *ex) {
  const int row = lane_id() >> 4;
  Suf inc = x;
  row_suf_steps<1>(inc, c);
  const Suf t3{read_lane(inc.a, 48), read_lane(inc.s, 48)};
  const Suf t23 = join(Suf{read_lane(inc.a, 32), read_lane(inc.s, 32)}, t3, c);
  const Suf t123 = join(Suf{read_lane(inc.a, 16), read_lane(inc.s, 16)}, t23, c);
  const Suf after = row == 3 ? Suf{0.0f, 0.0} : (row == 2 ? t3 : (row == 1 ? t23 : t123));
  *ex = join(dpp_suf<0x101>(inc), after, c);
  return join(inc, after, c);
}

// ------------------------------------------------------------- teams
// A team owns one segment of sorted keys in a blocked layout: team lane l
// holds elements [l*E, l*E + E).  A WaveTeam is LANES (<= 64) consecutive
// lanes of one wave; a BlockTeam is the whole workgroup.

template <int LANES>
struct WaveTeam {
  static constexpr int kLanes = LANES;
  int lane;
  LDEV WaveTeam() : lane(lane_id() & (LANES - 1)) {}

  // dst[e] = partner's src[REV ? E-1-e : e], partner = lane ^ MASK
  template <int MASK, bool REV, int E, class T>
  LDEV void exchange(const T (&src)[E], T (&dst)[E]) const {
#pragma unroll
    for (int e = 0; e < E; ++e) dst[e] = from_bits<T>(xor_lanes<MASK>(to_bits(src[REV ? E - 1 - e : e])));
  }
  // Team-local lane moves.  Teams inside one DPP row (LANES <= 16) use DPP:
  // row_shr / row_shl for shifts, quad_perm and mirrors for the butterfly
  // (any pairing of the halves serves a sum); wider teams use ds_bpermute.
  template <int OFF>
  LDEV static uint32_t up(uint32_t v) {
    if constexpr (LANES <= 16) return dpp<0x110 + OFF>(v);
    else return (uint32_t)__shfl_up((int)v, OFF, LANES);
  }
  template <int OFF>
  LDEV static uint32_t down(uint32_t v) {
    if constexpr (LANES <= 16) return dpp<0x100 + OFF>(v);
    else return (uint32_t)__shfl_down((int)v, OFF, LANES);
  }
  template <int M>
  LDEV static uint32_t pair(uint32_t v) {  // partner of the butterfly step M
    if constexpr (LANES <= 16) return xor_lanes<M == 4 ? 7 : (M == 8 ? 15 : M)>(v);
    else return (uint32_t)__shfl_xor((int)v, M, LANES);
  }
  template <int OFF, class F>
  LDEV static double move64(double v, F f) {
    const unsigned long long u = (unsigned long long)__double_as_longlong(v);
    const uint32_t lo = f((uint32_t)u), hi = f((uint32_t)(u >> 32));
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
  }
  template <int OFF>
  LDEV static double up64(double v) {
    return move64<OFF>(v, [](uint32_t x) { return up<OFF>(x); });
  }
  template <int OFF>
  LDEV static double down64(double v) {
    return move64<OFF>(v, [](uint32_t x) { return down<OFF>(x); });
  }
  // exclusive prefix and suffix sums of v over the team (plain fp64)
  template <int OFF>
  LDEV void sum_scan_steps(double &pre, double &suf) const {
    if constexpr (OFF < LANES) {
      const double yp = up64<OFF>(pre), ys = down64<OFF>(suf);
      if (lane >= OFF) pre += yp;
      if (lane + OFF < LANES) suf += ys;
      sum_scan_steps<2 * OFF>(pre, suf);
    }
  }
  // (the exclusive values are the neighbours' inclusive ones, not the
  // inclusive ones minus the lane's own: that difference would cancel when
  // the lane's own value dwarfs the rest)
  LDEV void excl_sums(double vp, double vs, double *pre, double *suf) const {
    double ip = vp, is = vs;
    sum_scan_steps<1>(ip, is);
    const double ep = up64<1>(ip), es = down64<1>(is);
    *pre = lane == 0 ? 0.0 : ep;
    *suf = lane == LANES - 1 ? 0.0 : es;
  }
  template <int M>
  LDEV static void sum_steps(int &v) {
    if constexpr (M < LANES) {
      v += (int)pair<M>((uint32_t)v);
      sum_steps<2 * M>(v);
    }
  }
  template <int M>
  LDEV static void sum_steps(double &v) {
    if constexpr (M < LANES) {
      v += move64<M>(v, [](uint32_t x) { return pair<M>(x); });
      sum_steps<2 * M>(v);
    }
  }
  LDEV int sum(int v) const {
    if constexpr (LANES == kWave) return wave_reduce(v, [](int x, int y) { return x + y; });
    sum_steps<1>(v);
    return v;
  }
  LDEV double sum(double v) const {
    if constexpr (LANES == kWave) return wave_reduce(v, [](double x, double y) { return x + y; });
    sum_steps<1>(v);
    return v;
  }
  template <int M>
  LDEV static void sum_steps(unsigned long long &v) {
    if constexpr (M < LANES) {
      const uint32_t lo = pair<M>((uint32_t)v), hi = pair<M>((uint32_t)(v >> 32));
      v += ((unsigned long long)hi << 32) | lo;
      sum_steps<2 * M>(v);
    }
  }
  LDEV unsigned long long sum(unsigned long long v) const {
    if constexpr (LANES == kWave)
      return wave_reduce(v, [](unsigned long long x, unsigned long long y) { return x + y; });
    sum_steps<1>(v);
    return v;
  }
  // largest / smallest value over the team, on every lane
  template <int M, bool MAX>
  LDEV static void ext_steps(uint32_t &v) {
    if constexpr (M < LANES) {
      const uint32_t y = pair<M>(v);
      v = MAX ? (y > v ? y : v) : (y < v ? y : v);
      ext_steps<2 * M, MAX>(v);
    }
  }
  LDEV uint32_t umax(uint32_t v) const {
    if constexpr (LANES == kWave) return wave_reduce(v, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
    ext_steps<1, true>(v);
    return v;
  }
  LDEV uint32_t umin(uint32_t v) const {
    if constexpr (LANES == kWave) return wave_reduce(v, [](uint32_t x, uint32_t y) { return x < y ? x : y; });
    ext_steps<1, false>(v);
    return v;
  }
  // value of team lane src; a whole wave requires src to be the same on every lane
  LDEV double bcast(double v, int src) const {
    if constexpr (LANES == kWave) return read_lane(v, __builtin_amdgcn_readfirstlane(src));
    return __shfl(v, src, LANES);
  }
  LDEV float bcast(float v, int src) const {
    if constexpr (LANES == kWave) return read_lane(v, __builtin_amdgcn_readfirstlane(src));
    return __shfl(v, src, LANES);
  }
  LDEV void sync() const {}

  template <int OFF>
  LDEV void int_steps(int &inc) const {
    if constexpr (OFF < LANES) {
      const int y = (int)up<OFF>((uint32_t)inc);
      if (lane >= OFF) inc += y;
      int_steps<2 * OFF>(inc);
    }
  }
  // exclusive prefix sum over the team; *total gets the team's sum
  LDEV int excl_scan(int v, int *total) const {
    int inc = v;
    int_steps<1>(inc);
    *total = __shfl(inc, LANES - 1, LANES);
    return inc - v;
  }

  template <int OFF>
  LDEV void pre_steps(Pre &inc, double c) const {
    if constexpr (OFF < LANES) {
      const Pre y{__uint_as_float(up<OFF>(__float_as_uint(inc.a))), move64<OFF>(inc.s, [](uint32_t x) { return up<OFF>(x); })};
      if (lane >= OFF) inc = join(y, inc, c);
      pre_steps<2 * OFF>(inc, c);
    }
  }
  template <int OFF>
  LDEV void suf_steps(Suf &inc, double c) const {
    if constexpr (OFF < LANES) {
      const Suf y{__uint_as_float(down<OFF>(__float_as_uint(inc.a))), move64<OFF>(inc.s, [](uint32_t x) { return down<OFF>(x); })};
      if (lane + OFF < LANES) inc = join(inc, y, c);
      suf_steps<2 * OFF>(inc, c);
    }
  }
  LDEV Pre excl_scan(Pre x, double c) const {
    if constexpr (LANES == kWave) {
      Pre ex;
      wave_scan(x, c, &ex);
      return ex;
    }
    Pre inc = x;
    pre_steps<1>(inc, c);
    Pre ex{__uint_as_float(up<1>(__float_as_uint(inc.a))), move64<1>(inc.s, [](uint32_t v) { return up<1>(v); })};
    if (lane == 0) ex.s = 0.0;
    return ex;
  }
  LDEV Suf excl_scan(Suf x, double c) const {
    if constexpr (LANES == kWave) {
      Suf ex;
      wave_scan(x, c, &ex);
      return ex;
    }
    Suf inc = x;
    suf_steps<1>(inc, c);
    Suf ex{__uint_as_float(down<1>(__float_as_uint(inc.a))), move64<1>(inc.s, [](uint32_t v) { return down<1>(v); })};
    if (lane == LANES - 1) ex.s = 0.0;
    return ex;
  }
};

// LDS scratch of a BlockTeam: exchange buffer for cross-wave stages plus
// small slots for scans, sums and broadcasts.
template <int LANES, int E>
struct BlockTeamLds {
  uint32_t xchg[E * LANES];
  float wa[LANES / kWave];
  double ws[LANES / kWave];
  int wi[LANES / kWave];
  double bd;
  float bf;
};

template <int LANES, int E>
struct BlockTeam {
  static constexpr int kLanes = LANES;
  static constexpr int kWaves = LANES / kWave;
  int lane;
  BlockTeamLds<LANES, E> *lds;
  LDEV explicit BlockTeam(BlockTeamLds<LANES, E> *l) : lane((int)threadIdx.x), lds(l) {}

  template <int MASK, bool REV, class T>
  LDEV void exchange(const T (&src)[E], T (&dst)[E]) const {
    if constexpr (MASK < kWave) {
#pragma unroll
      for (int e = 0; e < E; ++e) dst[e] = from_bits<T>(xor_lanes<MASK>(to_bits(src[REV ? E - 1 - e : e])));
    } else {
      __syncthreads();
#pragma unroll
      for (int e = 0; e < E; ++e) lds->xchg[e * LANES + lane] = to_bits(src[e]);
      __syncthreads();
#pragma unroll
      for (int e = 0; e < E; ++e) dst[e] = from_bits<T>(lds->xchg[(REV ? E - 1 - e : e) * LANES + (lane ^ MASK)]);
    }
  }
  LDEV int sum(int v) const {
    v = wave_reduce(v, [](int x, int y) { return x + y; });
    __syncthreads();
    if ((lane & (kWave - 1)) == 0) lds->wi[lane / kWave] = v;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t += lds->wi[w];
    return t;
  }
  LDEV double sum(double v) const {
    v = wave_reduce(v, [](double x, double y) { return x + y; });
    __syncthreads();
    if ((lane & (kWave - 1)) == 0) lds->ws[lane / kWave] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t += lds->ws[w];
    return t;
  }
  LDEV double bcast(double v, int src) const {
    __syncthreads();
    if (lane == src) lds->bd = v;
    __syncthreads();
    return lds->bd;
  }
  LDEV float bcast(float v, int src) const {
    __syncthreads();
    if (lane == src) lds->bf = v;
    __syncthreads();
    return lds->bf;
  }
  LDEV void sync() const { __syncthreads(); }

  // Scans: each wave scans its lanes (DPP + v_readlane), the wave totals go
  // through LDS, and every wave scans the kWaves totals inside one DPP row
  // to get what lies before (after) it.
  LDEV Pre excl_scan(Pre x, double c) const {
    static_assert(kWaves <= 16, "wave totals are scanned inside one DPP row");
    const int wl = lane & (kWave - 1), w = lane / kWave;
    Pre ex;
    const Pre inc = wave_scan(x, c, &ex);
    __syncthreads();
    if (wl == kWave - 1) {
      lds->wa[w] = inc.a;
      lds->ws[w] = inc.s;
    }
    __syncthreads();
    Pre tw = wl < kWaves ? Pre{lds->wa[wl], lds->ws[wl]} : Pre{0.0f, 0.0};
    row_pre_steps<1>(tw, c);
    const int src = __builtin_amdgcn_readfirstlane(w - 1);  // the same on every lane of the wave
    const Pre wp = w == 0 ? Pre{0.0f, 0.0} : Pre{read_lane(tw.a, src), read_lane(tw.s, src)};
    return join(wp, ex, c);
  }
  LDEV Suf excl_scan(Suf x, double c) const {
    static_assert(kWaves <= 16, "wave totals are scanned inside one DPP row");
    const int wl = lane & (kWave - 1), w = lane / kWave;
    Suf ex;
    const Suf inc = wave_scan(x, c, &ex);
    __syncthreads();
    if (wl == 0) {
      lds->wa[w] = inc.a;
      lds->ws[w] = inc.s;
    }
    __syncthreads();
    Suf tw = wl < kWaves ? Suf{lds->wa[wl], lds->ws[wl]} : Suf{0.0f, 0.0};
    row_suf_steps<1>(tw, c);
    const int src = __builtin_amdgcn_readfirstlane(w + 1);
    const Suf ws = w == kWaves - 1 ? Suf{0.0f, 0.0} : Suf{read_lane(tw.a, src), read_lane(tw.s, src)};
    return join(ex, ws, c);
  }
};

// ------------------------------------------------------- bitonic sort
// Ascending sort of E*LANES keys held blocked across a team.  Network: for
// each merge size 2^s, one stage pairing i with i ^ (2^s - 1) (the mirror
// of its block), then stages pairing i with i ^ d for d = 2^(s-2) .. 1; the
// lower index keeps the minimum.  Stages with d < E stay in registers;
// larger ones exchange with lane (lane ^ mask) of the team.  Keys are either
// order-preserving uint32 keys or finite fp32 values (padding +inf); for
// fp32 a cross-lane step is one median: med3(own, partner, -inf) is the
// minimum, med3(own, partner, +inf) the maximum.
template <int D, bool MIRROR, int E, class T, class Team>
LDEV void bitonic_stage(T (&key)[E], const Team &team) {
  if constexpr (D < E) {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      if ((i & D) == 0) {
        const int j = MIRROR ? (i ^ (2 * D - 1)) : (i ^ D);
        const T x = key[i], y = key[j];
        key[i] = min(x, y);
        key[j] = max(x, y);
      }
    }
  } else {
    constexpr int LM = D / E;
    constexpr int MASK = MIRROR ? (2 * LM - 1) : LM;
    T recv[E];
    team.template exchange<MASK, MIRROR>(key, recv);
    const bool lower = (team.lane & LM) == 0;
    if constexpr (sizeof(T) == 4 && T(0.5) != T(0)) {
      const float bound = lower ? -INFINITY : INFINITY;
#pragma unroll
      for (int e = 0; e < E; ++e) key[e] = __builtin_amdgcn_fmed3f(key[e], recv[e], bound);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) key[e] = lower ? min(key[e], recv[e]) : max(key[e], recv[e]);
    }
  }
}

template <int D, int E, class T, class Team>
LDEV void bitonic_cleaners(T (&key)[E], const Team &team) {
  if constexpr (D >= 1) {
    bitonic_stage<D, false>(key, team);
    bitonic_cleaners<D / 2>(key, team);
  }
}

template <int S, int LOGN, int E, class T, class Team>
LDEV void bitonic_merges(T (&key)[E], const Team &team) {
  if constexpr (S <= LOGN) {
    constexpr int HALF = 1 << (S - 1);
    bitonic_stage<HALF, true>(key, team);
    bitonic_cleaners<HALF / 2>(key, team);
    bitonic_merges<S + 1, LOGN>(key, team);
  }
}

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

template <int E, class T, class Team>
LDEV void bitonic_sort(T (&key)[E], const Team &team) {
  constexpr int NP = E * Team::kLanes;
  bitonic_merges<1, ilog2(NP)>(key, team);
}

// ----------------------------------------------------- segment solve
// Inputs describing one part of a sorted segment held by a team:
struct PartInfo {
  int nvalid;        // valid sorted keys in this part (a prefix of the team's blocked range)
  double above;      // #elements of the whole problem at or after this part's first element
  Pre seed_lo;       // everything before the part (left tail, earlier tiles)
  Suf seed_hi;       // everything after the part (later tiles, right tail)
  bool first;        // the part starts the segment: nothing but seed_lo lies below it
  bool last;         // the part ends the segment: nothing but seed_hi lies above it
};

// Threshold curve + locate + closed-form root over one team part
// (section 2.2, full-sort solver).  s[] are the part's sorted values,
// blocked (lane l holds indices l*E..l*E+E-1), nv of them valid in this
// lane.  Returns b on every team lane.
template <int E, class Team>
LDEV double segment_solve(const float (&s)[E], int nv, const PartInfo &part, double k, double t, double c,
                          float cf, const Team &team) {
  // step multipliers between consecutive knots of this lane
  float mul[E];
  mul[0] = 0.0f;
#pragma unroll
  for (int e = 1; e < E; ++e) mul[e] = (e < nv) ? wexpf(s[e - 1] - s[e], cf) : 0.0f;

  // lane aggregates
  double pl = 0.0, sl = 0.0;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (e < nv) pl = pl * (double)mul[e] + 1.0;
#pragma unroll
  for (int e = E - 1; e >= 0; --e)
    if (e < nv) sl = (e + 1 < E ? sl * (double)mul[e + 1] : 0.0) + 1.0;
  float last_s = s[0];
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (e < nv) last_s = s[e];
  const Pre mine_p{last_s, nv > 0 ? pl : 0.0};
  const Suf mine_s{s[0], nv > 0 ? sl : 0.0};

  const Pre pin = join(part.seed_lo, team.excl_scan(mine_p, c), c);
  const Suf sin = join(team.excl_scan(mine_s, c), part.seed_hi, c);

  // full P_j for this lane's knots
  double P[E];
  double acc = (pin.s == 0.0) ? 0.0 : pin.s * (double)wexp((double)pin.a - (double)s[0], c);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (e < nv) acc = (e == 0 ? acc : acc * (double)mul[e]) + 1.0;
    P[e] = acc;
  }
  const double s_after = (sin.s == 0.0) ? 0.0 : sin.s * (double)wexp((double)last_s - (double)sin.a, c);

  // threshold curve and the count of knots with g_j >= k
  const int base = team.lane * E;
  int cnt = 0;
  {
    double S = 0.0;
#pragma unroll
    for (int e = E - 1; e >= 0; --e) {
      if (e < nv) {
        S = (e == nv - 1) ? s_after + 1.0 : S * (double)mul[e + 1 < E ? e + 1 : 0] + 1.0;
        const double g = 0.5 * (P[e] - 1.0) + (part.above - (double)(base + e)) - 0.5 * S;
        cnt += (g >= k) ? 1 : 0;
      }
    }
  }
  const int Mp = team.sum(nv);
  const int jstar = team.sum(cnt) - 1;  // -1 .. Mp-1, part-local

  // the lane holding the first knot above b (or the last knot) solves
  const bool right_end = (jstar + 1 >= Mp);
  const int owner = Mp == 0 ? 0 : (right_end ? (Mp - 1) / E : (jstar + 1) / E);
  double b = 0.0;
  if (team.lane == owner) {
    // Anchor knot x and the two sums around it in the form ln(A) + B/t:
    // P-side (everything at or below x) and Q-side (everything above the
    // interval that holds b), plus the count above and the interval ends.
    const double it = 1.0 / t;
    double x, PA, PB = 0.0, QA, QB = 0.0, cabove, lo = -INFINITY, hi = INFINITY;
    if (Mp == 0) {
      // no knots in this part: the seeds alone bound b
      const bool has_lo = pin.s != 0.0;
      x = has_lo ? (double)pin.a : (double)sin.a;
      PA = has_lo ? pin.s : 0.0;
      QA = sin.s;
      QB = has_lo ? x - (double)sin.a : 0.0;
      cabove = part.above;
    } else if (!right_end) {
      const int e1 = jstar + 1 - base;  // first knot above b, in this lane
      double S1 = 1.0, S = 0.0, Pm = 0.0;
      float s1 = s[0], sm = s[0];
#pragma unroll
      for (int e = E - 1; e >= 0; --e) {
        if (e < nv) {
          S = (e == nv - 1) ? s_after + 1.0 : S * (double)mul[e + 1 < E ? e + 1 : 0] + 1.0;
          if (e == e1) {
            S1 = S;
            s1 = s[e];
          }
        }
        if (e == e1 - 1) {
          Pm = P[e];
          sm = s[e];
        }
      }
      const bool below_all = e1 == 0 && part.first && owner == 0;  // b below every knot
      if (e1 > 0) {
        x = sm;  // the knot just below, in this lane
        PA = Pm;
      } else if (!below_all) {
        x = pin.a;  // the knot just below: last of the previous lane or tile
        PA = pin.s;
      } else {
        x = s1;
        PA = pin.s;
        PB = (double)pin.a - x;
      }
      QA = S1;
      QB = below_all ? 0.0 : x - (double)s1;
      cabove = below_all ? part.above : part.above - (double)(jstar + 1);
      if (!below_all) lo = x;
      hi = s1;
    } else {
      const int e0 = Mp - 1 - base;
      x = s[0];
      PA = P[0];
#pragma unroll
      for (int e = 1; e < E; ++e)
        if (e == e0) {
          x = s[e];
          PA = P[e];
        }
      QA = sin.s;
      QB = x - (double)sin.a;
      cabove = part.above - (double)Mp;
      lo = x;
      hi = (part.last || sin.s == 0.0) ? INFINITY : (double)sin.a;
    }
    const double lP = PA > 0.0 ? log_pos(PA) + PB * it : -INFINITY;
    const double lQ = QA > 0.0 ? log_pos(QA) + QB * it : -INFINITY;
    b = solve_root(x, lP, lQ, cabove, k, t);
    b = fmin(fmax(b, lo), hi);
  }
  return team.bcast(b, owner);
}

// ----------------------------------------------------------- row state
// Per-row state of the bracketing and full-sort pipelines (workspace).
struct RowState {
  double a_lo, a_hi;        // bracket
  double tail_lo, tail_hi;  // S_L, S_R
  unsigned long long count_lo, count_hi;
  unsigned long long band;  // M: atomic append counter
  double b;                 // threshold from the band solve or the fallback
  uint32_t kmin, kmax;      // key range of the band
  int32_t flags;
  int32_t pad0;
  double k, t, c;           // full-sort path: the row's budget, temperature, log2(e)/t
  float cf;                 //   (its own with per-row values, else the call's)
  int32_t pad1;
  int64_t blo, bhi;         // bracketing with per-row budgets: the row's order-statistic indices
  int64_t set0;             // whole rows, second bucket level: start of the crowded bucket in the first
                            // level's keys (its size in band, its key extremes in kmin / kmax, everything
                            // below / above it in a_lo, tail_lo, count_lo / a_hi, tail_hi, count_hi)
};

// Row state flags (never reported): the row's crowded balancing bucket
// waits for the second bucket level; the row's bracket missed and its
// whole-row solve waits for the bucket launches after the band kernels.
constexpr int32_t kFlagNested = 1 << 16;
constexpr int32_t kFlagDeferred = 1 << 17;

// Per-call reset of one row's state (bracket open unless forced).
LDEV void reset_row_state(RowState *st, int64_t row, int32_t flags, int has_override, double o_lo, double o_hi) {
  RowState z;
  z.a_lo = has_override ? o_lo : -INFINITY;
  z.a_hi = has_override ? o_hi : INFINITY;
  z.tail_lo = 0.0;
  z.tail_hi = 0.0;
  z.count_lo = 0;
  z.count_hi = 0;
  z.band = 0;
  z.b = 0.0;
  z.kmin = 0xFFFFFFFFu;
  z.kmax = 0u;
  z.flags = flags;
  z.pad0 = 0;
  z.k = z.t = z.c = 0.0;
  z.cf = 0.0f;
  z.pad1 = 0;
  z.blo = 0;
  z.bhi = 0;
  z.set0 = 0;
  st[row] = z;
}

}  // namespace lapsum
