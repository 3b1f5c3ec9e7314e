// On-chip (register + LDS) kernels for rows of up to 8192 scores.
//
// Forward ("Fast LapSum: Exact Differentiable Top-k at Million Scale",
// section 2.2, full-sort solver; section 2.1, eq. (1) for the apply): one
// team of lanes owns one row.  The row is read once from HBM, sorted by a
// bitonic network in registers (cross-lane stages by DPP / swizzle within a
// wave, through LDS across waves), scanned into the threshold curve,
// located, solved in closed form, and p is written from the original
// values still held in registers.  The only HBM traffic is r in, p and b out.
//
// Backward (section 2.1, analytic VJP): one team per row reads g and p once,
// forms D = sum d and G = sum g d in fp64, and writes dr = d (g - G/D).
//
// Band solve (section 2.2, probabilistic bracketing, step 3): the same
// sort + curve + root on the compacted middle band, seeded with the tail
// sums of the streaming pass, followed by the certification of step 4.
#include "bucket_dev.hpp"
#include "filter_dev.hpp"
#include "widen_dev.hpp"

namespace lapsum {

LDEV bool aligned16(const void *q) { return ((uintptr_t)q & 15u) == 0; }
typedef float f4 __attribute__((ext_vector_type(4)));

// p = F((x - b)/t); z2 = (x - b) log2(e)/t formed from an fp64 difference.
LDEV float laplace_cdf_at(float x, double b, double c) {
  const float z2 = (float)(((double)x - b) * c);
  return z2 < 0.0f ? 0.5f * __builtin_amdgcn_exp2f(z2) : 1.0f - 0.5f * __builtin_amdgcn_exp2f(-z2);
}

// Where lane `lane` of a team of LANES keeps its E scores of the row.  On
// the vector path slot e = 4q + i is element q*4*LANES + 4*lane + i: each
// 16-byte load or store instruction of the team covers 64*LANES contiguous
// bytes.  Otherwise slot e is element lane*E + e.  (The sort does not care
// which scores a lane starts with; the apply writes each p where its score
// came from.)
template <int E, int LANES>
LDEV int slot_index(int lane, int e, bool vec) {
  return vec ? (e >> 2) * (4 * LANES) + 4 * lane + (e & 3) : lane * E + e;
}

template <int E, int LANES>
LDEV void load_row(const float *rr, int n, int lane, bool ok, bool vec, float (&v)[E]) {
  if (vec && (E % 4) == 0) {
#pragma unroll
    for (int q = 0; q < E; q += 4) {
      const int i = slot_index<E, LANES>(lane, q, true);
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (ok && i < n) {
        // rows are read once and written once: non-temporal, so nothing is
        // left dirty in L2 for the end-of-kernel write-back
        const f4 y = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(rr + i));
        x = make_float4(y.x, y.y, y.z, y.w);
      }
      v[q] = x.x;
      v[q + 1] = x.y;
      v[q + 2] = x.z;
      v[q + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = slot_index<E, LANES>(lane, e, false);
      v[e] = (ok && i < n) ? rr[i] : 0.0f;
    }
  }
}

template <int E, int LANES>
LDEV void store_row(float *pp, int n, int lane, bool ok, bool vec, const float (&v)[E]) {
  if (!ok) return;
  if (vec && (E % 4) == 0) {
#pragma unroll
    for (int q = 0; q < E; q += 4) {
      const int i = slot_index<E, LANES>(lane, q, true);
      if (i < n) {
        const f4 y = {v[q], v[q + 1], v[q + 2], v[q + 3]};
        __builtin_nontemporal_store(y, reinterpret_cast<f4 *>(pp + i));
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = slot_index<E, LANES>(lane, e, false);
      if (i < n) pp[i] = v[e];
    }
  }
}

// Root over the certified window's sorted candidates when they span few
// temperatures.  The candidates s_0 <= ... <= s_{M-1} (blocked: lane l holds
// s[l*E .. l*E+nv-1]) all lie at or above a0, everything below a0 is the
// tail S = sum e^{(r - a0)/t}, and nothing lies above the window.  With every
// sum anchored at a0 (u_i = e^{(s_i - a0)/t} >= 1 and v_i = 1/u_i, held in
// fp64, whose range covers them and their sums over at most 1024 knots when
// (s_{M-1} - a0) c <= kWindowSpan), the threshold curve at knot j is
//   g_j = (S + sum_{i<j} u_i) v_j / 2 + (M - j - 1/2) - u_j (sum_{i>j} v_i) / 2
// (the knot itself counts F(0) = 1/2): plain prefix and suffix sums over the
// team replace the re-anchored scans.  The last knot with g_j >= k is just
// below the root, and the closed form between it and the next knot gives b
// (section 2.2, full-sort solver: threshold curve, index lookup, closed-form
// root).  Returns b on every team lane.
constexpr float kWindowSpan = 1000.0f;  // largest (s_{M-1} - a0) log2(e)/t of the fast solve

template <int E, int LANES>
LDEV double window_root(const WaveTeam<LANES> &team, const float (&s)[E], int nv, int M, float a0, double S,
                        double k, double t) {
  // u = 2^z and v = 2^-z, z = (s - a0) log2(e)/t formed in fp64 and split
  // into its integer part (applied exactly by ldexp) and a fraction in
  // [0, 1) for exp2: u and v carry the exp2's relative error only, however
  // large z is
  double u[E], v[E];
  double lu = 0.0, lv = 0.0;
  const double c = kLog2e / t;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const double z = ((double)s[e] - (double)a0) * c;  // >= 0
    const double zi = floor(z);
    const float zf = (float)(z - zi);
    u[e] = e < nv ? __builtin_ldexp((double)__builtin_amdgcn_exp2f(zf), (int)zi) : 0.0;
    v[e] = e < nv ? __builtin_ldexp((double)__builtin_amdgcn_exp2f(-zf), -(int)zi) : 0.0;
    lu += u[e];
    lv += v[e];
  }
  // the u sums of the lanes before this one, the v sums of those after it
  double pu, sv;
  team.excl_sums(lu, lv, &pu, &sv);
  const int base = team.lane * E;
  // threshold curve at this lane's knots; the count of knots with g >= k
  double below[E], above[E];
  {
    double acc = S + pu;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      below[e] = acc;  // S + sum over knots before this one, at a0
      acc += u[e];
    }
    double acc2 = sv;
#pragma unroll
    for (int e = E - 1; e >= 0; --e) {
      above[e] = acc2;  // sum over knots after this one, at a0
      acc2 += v[e];
    }
  }
  int cnt = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (e < nv) {
      const double g = 0.5 * below[e] * v[e] + ((double)(M - base - e) - 0.5) - 0.5 * u[e] * above[e];
      cnt += g >= k ? 1 : 0;
    }
  }
  const int js = team.sum(cnt) - 1;  // -1 .. M-1: the last knot with g >= k
  const int owner = js < 0 ? 0 : js / E;
  // the first knot above the root, for the clamp (this lane's next knot is
  // its own or the first of the next lane)
  const float nxt_lane = __uint_as_float(WaveTeam<LANES>::template down<1>(__float_as_uint(s[0])));
  double b = 0.0;
  if (team.lane == owner) {
    double x, PA, QA, cab, hi;
    if (js < 0) {  // below every knot: everything at a0
      x = a0;
      PA = S;
      QA = sv + lv;  // lane 0: all of the knots
      cab = (double)M;
      hi = s[0];
    } else {
      const int e0 = js - base;
      x = s[0];
      PA = below[0] * v[0] + 1.0;
      QA = u[0] * above[0];
      hi = js + 1 < M ? nxt_lane : INFINITY;
#pragma unroll
      for (int e = 1; e < E; ++e) {
        if (e == e0) {
          x = s[e];
          PA = below[e] * v[e] + 1.0;
          QA = u[e] * above[e];
        }
        if (e == e0 + 1 && e < nv) hi = s[e];
      }
      cab = (double)(M - 1 - js);
    }
    const double lP = PA > 0.0 ? log_pos(PA) : -INFINITY;
    const double lQ = QA > 0.0 ? log_pos(QA) : -INFINITY;
    b = solve_root(x, lP, lQ, cab, k, t);
    b = fmin(fmax(b, x), hi);
  }
  return team.bcast(b, owner);
}

// Certified window for a small budget: with the K-th largest (K = ceil(k))
// of the lanes' second-largest scores as a (for K above half the lane
// count, the 2K-th largest of the lanes' two largest), at least 2K >= 2k
// scores are >= a, each with p >= 1/2 at b = a, so f(a) >= k and b >= a.  Only the
// scores >= a (the candidates, typically a few times k) are sorted and
// scanned; everything below a enters as one exact tail sum anchored at a,
// exactly as the bracketing band solve seeds its scan.  A budget near n uses
// the complement: b(-r, n - k) = -b(r, k).  Returns false (and the caller
// sorts the whole row) when k and n - k both exceed the lane count or the
// candidates overflow the 4*LANES buffer.  buf: this team's 4*LANES floats
// of LDS.
// MIRROR (the complement, k > LANES) is a template argument so the sign
// folds into the instructions' operand modifiers.
template <int E, int LANES, bool MIRROR>
LDEV bool window_solve(const WaveTeam<LANES> &team, const float (&v)[E], const bool (&valid)[E], int n, double k,
                       double t, double c, float cf, float *buf, double &b_out) {
  constexpr int CAP = 4 * LANES;
  const double kk = MIRROR ? (double)n - k : k;
  if (kk > (double)LANES) return false;
  constexpr float sg = MIRROR ? -1.0f : 1.0f;
  float m1 = -INFINITY, m2 = -INFINITY;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    // the two largest: m2 <= m1 stays true, so the new second is a median
    const float w = valid[e] ? sg * v[e] : -INFINITY;
    m2 = __builtin_amdgcn_fmed3f(m1, m2, w);
    m1 = fmaxf(m1, w);
  }
  const int K = (int)ceil(kk);
  float a;
  if (K > LANES / 2) {
    // a budget near the lane count: the 2K-th largest of the lanes' two
    // largest scores (at least 2K scores are >= it, and it is never below
    // the K-th largest second score), which keeps the window small
    float x2[2] = {m2, m1};
    bitonic_sort<2>(x2, team);
    a = team.bcast(x2[0], LANES - K);
  } else {
    float x[1] = {m2};
    bitonic_sort<1>(x, team);
    a = team.bcast(x[0], LANES - K);
  }
  if (!(a > -INFINITY)) return false;
  int mine = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) mine += (valid[e] && sg * v[e] >= a) ? 1 : 0;
  int C;
  int o = team.excl_scan(mine, &C);
  if (C > CAP) return false;
  // tail below a, anchored at a: this lane's E terms (each <= 1) in fp32,
  // the lane sums in fp64
  float Sl = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float w = sg * v[e];
    if (valid[e] && w >= a) buf[o++] = w;
    if (valid[e] && w < a) Sl += __builtin_amdgcn_exp2f((w - a) * cf);
  }
  const double S = team.sum((double)Sl);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  PartInfo part;
  part.above = (double)C;
  part.seed_lo = Pre{a, S};
  part.seed_hi = Suf{0.0f, 0.0};
  part.first = true;
  part.last = true;
  double bw;
  // the candidates sorted at two per lane when every team of the wave has
  // at most 2*LANES of them (the usual case), else at four per lane
  if (__ballot(C > 2 * LANES) == 0ull) {
    float s2[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) s2[q] = 2 * team.lane + q < C ? buf[2 * team.lane + q] : INFINITY;
    bitonic_sort<2>(s2, team);
    const int nv = min(max(C - 2 * team.lane, 0), 2);
#pragma unroll
    for (int q = 0; q < 2; ++q) s2[q] = q < nv ? s2[q] : 0.0f;
    // the window's span: its largest candidate is the team's last valid one
    const float top = team.bcast(nv == 2 ? s2[1] : s2[0], (C - 1) / 2);
    if ((top - a) * cf <= kWindowSpan) {
      bw = window_root<2>(team, s2, nv, C, a, S, kk, t);
    } else {
      part.nvalid = nv;
      bw = segment_solve<2>(s2, nv, part, kk, t, c, cf, team);
    }
  } else {
    float s4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) s4[q] = 4 * team.lane + q < C ? buf[4 * team.lane + q] : INFINITY;
    bitonic_sort<4>(s4, team);
    const int nv = min(max(C - 4 * team.lane, 0), 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) s4[q] = q < nv ? s4[q] : 0.0f;
    const float last = nv == 4 ? s4[3] : (nv == 3 ? s4[2] : (nv == 2 ? s4[1] : s4[0]));
    const float top = team.bcast(last, (C - 1) / 4);
    if ((top - a) * cf <= kWindowSpan) {
      bw = window_root<4>(team, s4, nv, C, a, S, kk, t);
    } else {
      part.nvalid = nv;
      bw = segment_solve<4>(s4, nv, part, kk, t, c, cf, team);
    }
  }
  b_out = MIRROR ? -bw : bw;
  return true;
}

// Whole forward of one row held by a team.  FULL: n == E * lanes, so every
// lane holds E valid scores and no validity test is needed.  good = false
// (per-row k or t out of range) writes NaN p and b and flags the row.
template <int E, bool FULL, class Team>
LDEV void onchip_row_forward(const Team &team, const float *rr, int n_arg, bool ok, double k, double t, float *pp,
                             double *bout, lapsum_row_stats *stats, float *wbuf = nullptr, bool good = true) {
  const int n = FULL ? E * Team::kLanes : n_arg;
  constexpr int LANES = Team::kLanes;
  const bool vec = (n & 3) == 0 && aligned16(rr) && aligned16(pp);
  const int base = team.lane * E;  // first sorted position held by this lane
  float v[E];
  load_row<E, LANES>(rr, n, team.lane, ok, vec, v);
  bool valid[E];
#pragma unroll
  for (int e = 0; e < E; ++e) valid[e] = FULL || (ok && slot_index<E, LANES>(team.lane, e, vec) < n);
  const double c = kLog2e / t;
  const float cf = (float)c;

  double b = 0.0;
  bool done = !ok;  // rows past the end compute nothing and store nothing
  if constexpr (Team::kLanes <= kWave) {
    if (wbuf != nullptr && !done)
      done = k > (double)LANES ? window_solve<E, LANES, true>(team, v, valid, n, k, t, c, cf, wbuf, b)
                               : window_solve<E, LANES, false>(team, v, valid, n, k, t, c, cf, wbuf, b);
  }
  if (!done) {
    // the scores themselves are sorted (finite, so fp32 order is numeric
    // order; equal values, -0 and +0 included, need no order among them)
    float s[E];
#pragma unroll
    for (int e = 0; e < E; ++e) s[e] = valid[e] ? v[e] : INFINITY;

    bitonic_sort<E>(s, team);

    const int nv = FULL ? E : (ok ? min(max(n - base, 0), E) : 0);
#pragma unroll
    for (int e = 0; e < E; ++e) s[e] = (e < nv) ? s[e] : 0.0f;

    PartInfo part;
    part.nvalid = nv;
    part.above = (double)n;
    part.seed_lo = Pre{0.0f, 0.0};
    part.seed_hi = Suf{0.0f, 0.0};
    part.first = true;
    part.last = true;
    b = segment_solve<E>(s, nv, part, k, t, c, cf, team);
  }

  // p = F((x - b)/t) in fp32 with b split into bh + bl: x - bh is exact or
  // rounds relative to itself, and (x - bh) cf - bl cf is one fused
  // multiply-add, so p carries a few 1e-8 absolute error at most
  const float bh = (float)b, bl = (float)(b - (double)bh);
  const float blcf = bl * cf;
  float out[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float z2 = __builtin_fmaf(v[e] - bh, cf, -blcf);
    const float h = __builtin_amdgcn_exp2f(-1.0f - fabsf(z2));  // e^{-|z|}/2
    out[e] = z2 < 0.0f ? h : 1.0f - h;
  }
  if (!good) {
#pragma unroll
    for (int e = 0; e < E; ++e) out[e] = __builtin_nanf("");
    b = __builtin_nan("");
  }
  store_row<E, LANES>(pp, n, team.lane, ok, vec, out);
  if (ok && team.lane == 0) {
    *bout = b;
    if (stats) {
      stats->a_lo = -INFINITY;
      stats->a_hi = INFINITY;
      stats->tail_lo = 0.0;
      stats->tail_hi = 0.0;
      stats->count_lo = 0;
      stats->count_hi = 0;
      stats->band = n;
      stats->flags = good ? 0 : LAPSUM_FLAG_INVALID;
      stats->reserved = 0;
    }
  }
}

// Teams inside one wave: NP = LANES * E <= 1024, 256 threads = 256/LANES rows.
// PR: per-row k and t (then each team reads its own; the scalar build keeps
// them uniform, in scalar registers).
template <int NP, int LANES, bool FULL, bool PR>
LDEV void onchip_forward_wave_body(const float *__restrict__ r, int64_t rows, int n, double k, double t,
                                   const RowParams &rp, float *__restrict__ p, double *__restrict__ b,
                                   lapsum_row_stats *stats, float *wbuf) {
  constexpr int E = NP / LANES;
  WaveTeam<LANES> team;
  const int64_t row = (int64_t)blockIdx.x * (256 / LANES) + threadIdx.x / LANES;
  const bool ok = row < rows;
  const int64_t rr = ok ? row : 0;
  bool good = true;
  if constexpr (PR) good = row_params(rp.k, rp.t, rr, n, k, t);
  onchip_row_forward<E, FULL>(team, r + rr * n, n, ok, k, t, p + rr * n, b + rr, stats ? stats + rr : nullptr,
                              wbuf + (threadIdx.x / LANES) * (4 * LANES), good);
}

// Rows of exactly NP scores: at most 128 VGPRs, so four waves fit on each
// SIMD and a batch of small rows runs in one round (the per-row build would
// otherwise just exceed it).
template <int NP, int LANES, bool PR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void onchip_forward_wave(
    const float *__restrict__ r, int64_t rows, int n, double k, double t, RowParams rp, float *__restrict__ p,
    double *__restrict__ b, lapsum_row_stats *stats) {
  __shared__ float wbuf[4 * 256];  // candidate buffers of the certified window, 4*LANES per team
  lds_poison(wbuf);
  onchip_forward_wave_body<NP, LANES, true, PR>(r, rows, n, k, t, rp, p, b, stats, wbuf);
}

// Ragged rows (n < NP): the validity tests need more registers, and two
// waves per SIMD without spills beat four with them.
template <int NP, int LANES, bool PR>
__global__ __launch_bounds__(256) void onchip_forward_wave_ragged(const float *__restrict__ r, int64_t rows, int n,
                                                                  double k, double t, RowParams rp,
                                                                  float *__restrict__ p, double *__restrict__ b,
                                                                  lapsum_row_stats *stats) {
  __shared__ float wbuf[4 * 256];
  lds_poison(wbuf);
  onchip_forward_wave_body<NP, LANES, false, PR>(r, rows, n, k, t, rp, p, b, stats, wbuf);
}

// One row per workgroup: NP = 16 * LANES, LANES threads.
template <int NP, bool PR>
__global__ __launch_bounds__(NP / 16) void onchip_forward_block(const float *__restrict__ r, int64_t rows, int n,
                                                                double k, double t, RowParams rp,
                                                                float *__restrict__ p, double *__restrict__ b,
                                                                lapsum_row_stats *stats) {
  constexpr int E = 16, LANES = NP / 16;
  __shared__ BlockTeamLds<LANES, E> lds;
  lds_poison(lds);
  BlockTeam<LANES, E> team(&lds);
  const int64_t row = grid_row();
  if (row >= rows) return;
  bool good = true;
  if constexpr (PR) good = row_params(rp.k, rp.t, row, n, k, t);
  onchip_row_forward<E, false>(team, r + row * n, n, true, k, t, p + row * n, b + row, stats ? stats + row : nullptr,
                               nullptr, good);
}

template <int NP, int LANES, bool PR>
static hipError_t launch_fwd_wave(const float *r, int64_t rows, int n, double k, double t, RowParams rp, float *p,
                                  double *b, lapsum_row_stats *stats, hipStream_t s) {
  constexpr int RPB = 256 / LANES;
  const int64_t grid = (rows + RPB - 1) / RPB;
  if (n == NP)
    hipLaunchKernelGGL((onchip_forward_wave<NP, LANES, PR>), dim3((unsigned)grid), dim3(256), 0, s, r, rows, n, k,
                       t, rp, p, b, stats);
  else
    hipLaunchKernelGGL((onchip_forward_wave_ragged<NP, LANES, PR>), dim3((unsigned)grid), dim3(256), 0, s, r, rows,
                       n, k, t, rp, p, b, stats);
  return hipGetLastError();
}

template <int NP, bool PR>
static hipError_t launch_fwd_block(const float *r, int64_t rows, int n, double k, double t, RowParams rp, float *p,
                                   double *b, lapsum_row_stats *stats, hipStream_t s) {
  hipLaunchKernelGGL((onchip_forward_block<NP, PR>), rows_grid(1u, rows), dim3(NP / 16), 0, s, r, rows, n, k, t, rp,
                     p, b, stats);
  return hipGetLastError();
}

template <bool PR>
static hipError_t onchip_forward_by_size(const float *r, int64_t rows, int n, double k, double t, RowParams rp,
                                         float *p, double *b, lapsum_row_stats *stats, hipStream_t s) {
  if (n <= 64) return launch_fwd_wave<64, 16, PR>(r, rows, n, k, t, rp, p, b, stats, s);
  if (n <= 128) return launch_fwd_wave<128, 16, PR>(r, rows, n, k, t, rp, p, b, stats, s);
  if (n <= 256) return launch_fwd_wave<256, 16, PR>(r, rows, n, k, t, rp, p, b, stats, s);
  if (n <= 512) return launch_fwd_wave<512, 32, PR>(r, rows, n, k, t, rp, p, b, stats, s);
  if (n <= 1024) return launch_fwd_wave<1024, 64, PR>(r, rows, n, k, t, rp, p, b, stats, s);
  if (n <= 2048) return launch_fwd_block<2048, PR>(r, rows, n, k, t, rp, p, b, stats, s);
  if (n <= 4096) return launch_fwd_block<4096, PR>(r, rows, n, k, t, rp, p, b, stats, s);
  return launch_fwd_block<8192, PR>(r, rows, n, k, t, rp, p, b, stats, s);
}

hipError_t launch_onchip_forward(const float *r, int64_t rows, int n, double k, double t, RowParams rp, float *p,
                                 double *b, lapsum_row_stats *stats, hipStream_t s) {
  return rp.any() ? onchip_forward_by_size<true>(r, rows, n, k, t, rp, p, b, stats, s)
                  : onchip_forward_by_size<false>(r, rows, n, k, t, rp, p, b, stats, s);
}

// ------------------------------------------------------------ backward
// One team per row, 256/LANES rows per workgroup and step; each workgroup
// strides over the row groups and loads the next group's g and p before it
// reduces and writes the current one, so reads and writes overlap.
template <int NP, int LANES>
LDEV void bwd_row(const WaveTeam<LANES> &team, const float (&gv)[NP / LANES], const float (&pv)[NP / LANES],
                  int64_t row, bool ok, int n, bool vec, float inv_t, float *__restrict__ dr, float *__restrict__ dk,
                  lapsum_row_stats *stats, bool good = true) {
  constexpr int E = NP / LANES;
  double D = 0.0, G = 0.0;
  float q[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    // min(p, 1 - p) is the Laplace density at the score (times t)
    q[e] = (ok && slot_index<E, LANES>(team.lane, e, vec) < n) ? fminf(pv[e], 1.0f - pv[e]) : 0.0f;
    D += (double)q[e];
    G += (double)gv[e] * (double)q[e];
  }
  D = team.sum(D);
  G = team.sum(G);
  const double dkd = D > 0.0 ? G / D : 0.0;
  float out[E];
#pragma unroll
  for (int e = 0; e < E; ++e)
    out[e] = !good ? __builtin_nanf("") : (D > 0.0 ? q[e] * inv_t * (float)((double)gv[e] - dkd) : 0.0f);
  store_row<E, LANES>(dr + row * n, n, team.lane, ok, vec, out);
  if (ok && team.lane == 0) {
    dk[row] = good ? (float)dkd : __builtin_nanf("");
    if (stats && !good) atomicOr(&stats[row].flags, LAPSUM_FLAG_INVALID);
    else if (stats && !(D > 0.0)) atomicOr(&stats[row].flags, LAPSUM_FLAG_DEGENERATE);
  }
}

template <int NP, int LANES, bool PR>
__global__ __launch_bounds__(256) void onchip_backward_wave(const float *__restrict__ g, const float *__restrict__ p,
                                                            int64_t rows, int n, double t, RowParams rp,
                                                            float *__restrict__ dr, float *__restrict__ dk,
                                                            lapsum_row_stats *stats) {
  constexpr int E = NP / LANES, RPW = 256 / LANES;
  WaveTeam<LANES> team;
  const bool vec = (n & 3) == 0 && aligned16(g) && aligned16(p) && aligned16(dr);
  const float inv_t = (float)(1.0 / t);
  const int64_t groups = (rows + RPW - 1) / RPW;
  const int sub = threadIdx.x / LANES;
  int64_t grp = blockIdx.x;
  float gv[E], pv[E];
  {
    const int64_t row = grp * RPW + sub;
    const bool ok = grp < groups && row < rows;
    const int64_t rr = ok ? row : 0;
    load_row<E, LANES>(g + rr * n, n, team.lane, ok, vec, gv);
    load_row<E, LANES>(p + rr * n, n, team.lane, ok, vec, pv);
  }
  for (; grp < groups; grp += gridDim.x) {
    const int64_t nrow = (grp + gridDim.x) * RPW + sub;
    const bool nok = grp + gridDim.x < groups && nrow < rows;
    const int64_t nr = nok ? nrow : 0;
    float gn[E], pn[E];
    load_row<E, LANES>(g + nr * n, n, team.lane, nok, vec, gn);
    load_row<E, LANES>(p + nr * n, n, team.lane, nok, vec, pn);
    const int64_t row = grp * RPW + sub;
    const bool ok = row < rows;
    if constexpr (PR) {
      double kr = 0.5 * (double)n, tr = t;
      const bool good = row_params(nullptr, rp.t, ok ? row : 0, n, kr, tr);
      bwd_row<NP, LANES>(team, gv, pv, ok ? row : 0, ok, n, vec, (float)(1.0 / tr), dr, dk, stats, good);
    } else {
      bwd_row<NP, LANES>(team, gv, pv, ok ? row : 0, ok, n, vec, inv_t, dr, dk, stats);
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      gv[e] = gn[e];
      pv[e] = pn[e];
    }
  }
}

bool onchip_backward_supported(int64_t n) { return n >= 1 && n <= 1024; }

constexpr int64_t kBwdMaxGroups = 4096;  // workgroups of the on-chip backward, at most

template <int NP, int LANES>
static hipError_t launch_bwd_wave(const float *g, const float *p, int64_t rows, int n, double t, RowParams rp,
                                  float *dr, float *dk, lapsum_row_stats *stats, hipStream_t s) {
  constexpr int RPB = 256 / LANES;
  const int64_t groups = (rows + RPB - 1) / RPB;
  const int64_t grid = groups < kBwdMaxGroups ? groups : kBwdMaxGroups;
  if (rp.t != nullptr)
    hipLaunchKernelGGL((onchip_backward_wave<NP, LANES, true>), dim3((unsigned)grid), dim3(256), 0, s, g, p, rows, n,
                       t, rp, dr, dk, stats);
  else
    hipLaunchKernelGGL((onchip_backward_wave<NP, LANES, false>), dim3((unsigned)grid), dim3(256), 0, s, g, p, rows,
                       n, t, rp, dr, dk, stats);
  return hipGetLastError();
}

hipError_t launch_onchip_backward(const float *g, const float *p, int64_t rows, int n, double t, RowParams rp,
                                  float *dr, float *dk, lapsum_row_stats *stats, hipStream_t s) {
  if (n <= 64) return launch_bwd_wave<64, 16>(g, p, rows, n, t, rp, dr, dk, stats, s);
  if (n <= 128) return launch_bwd_wave<128, 16>(g, p, rows, n, t, rp, dr, dk, stats, s);
  if (n <= 256) return launch_bwd_wave<256, 16>(g, p, rows, n, t, rp, dr, dk, stats, s);
  if (n <= 512) return launch_bwd_wave<512, 32>(g, p, rows, n, t, rp, dr, dk, stats, s);
  return launch_bwd_wave<1024, 64>(g, p, rows, n, t, rp, dr, dk, stats, s);
}

// ----------------------------------------------------------- band solve
// One workgroup of 512 threads per row; the band (at most NP keys) is
// gathered from the filter's per-workgroup slots, sorted, and solved with the
// tail sums as boundary seeds.  The result is certified: the root must lie
// inside [a_L, a_R).  A row whose bracket missed (or whose band overflowed)
// is then sorted and solved in full by the same workgroup, so no separate
// fallback launch is needed on this path.
constexpr int kBandNT = 512;

// Sort + solve + certify the band of one row with NP >= m keys (m = band
// size), E = NP / kBandNT keys per thread.
template <int NP, class Lds>
LDEV void band_onchip_row(const uint32_t *__restrict__ slots, const uint32_t *soffs, int gx, int64_t row, int m,
                          RowState &S, double k, double t, Lds &lds) {
  constexpr int E = NP / kBandNT;
  BlockTeam<kBandNT, E> team(reinterpret_cast<BlockTeamLds<kBandNT, E> *>(&lds));
  const int base = team.lane * E;
  // slot holding index `base`: the last b with soffs[b] <= base
  int lo = 0, hi = gx - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int)soffs[mid] <= base) lo = mid;
    else hi = mid - 1;
  }
  int b = lo;
  uint32_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    // every load issued unconditionally (slot 0's first key past the band's
    // end), so none waits for the one before
    const int j = base + e;
    const bool in = j < m;
    if (in)
      while ((int)soffs[b + 1] <= j) ++b;
    const int64_t at = in ? (row * gx + b) * kBandSlot + (j - (int)soffs[b]) : row * gx * kBandSlot;
    key[e] = slots[at];
  }
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (base + e >= m) key[e] = 0xFFFFFFFFu;
  bitonic_sort<E>(key, team);
  const int nv = min(max(m - base, 0), E);
  float s[E];
#pragma unroll
  for (int e = 0; e < E; ++e) s[e] = (e < nv) ? value_of(key[e]) : 0.0f;

  const double c = kLog2e / t;
  PartInfo part;
  part.nvalid = nv;
  part.above = (double)m + (double)S.count_hi;
  part.seed_lo = Pre{(float)S.a_lo, S.count_lo ? S.tail_lo : 0.0};
  part.seed_hi = Suf{(float)S.a_hi, S.count_hi ? S.tail_hi : 0.0};
  part.first = true;
  part.last = true;
  const double bb = segment_solve<E>(s, nv, part, k, t, c, (float)c, team);
  if (threadIdx.x == 0) {
    S.b = bb;
    const bool hit = (bb >= S.a_lo) && (bb < S.a_hi);
    S.flags |= hit ? LAPSUM_FLAG_HIT : LAPSUM_FLAG_FALLBACK;
  }
  __syncthreads();
}

// The band's actual size picks the sort (1024 .. NPMAX keys), so a band far
// below its capacity is not sorted at the capacity.
template <int NPMAX>
__global__ __launch_bounds__(kBandNT) void band_solve_onchip(const uint32_t *__restrict__ slots,
                                                             const FilterPartial *__restrict__ part, int gx,
                                                             int64_t rows, int64_t n, int64_t cap,
                                                             RowState *__restrict__ st, double k, double t,
                                                             SegArgs fb) {
  union BandLds {
    BlockTeamLds<kBandNT, NPMAX / kBandNT> band;
    SegLds<kBandNT> full;
  };
  __shared__ BandLds lds;
  __shared__ uint32_t soffs[kMaxFilterBlocks + 1];
  __shared__ int fall;
  lds_poison(lds);
  lds_poison(soffs);
  lds_poison(fall);
  const int64_t row = grid_row();
  if (row >= rows) return;
  RowState &S = st[row];
  // the streaming filter's partials of the row: totals and slot offsets
  const FilterTotals T = filter_totals<kBandNT>(part + row * gx, gx, n, cap, soffs);
  if (threadIdx.x == 0) store_filter_totals(S, T);
  __syncthreads();
  if (!T.overflow) {
    const int m = (int)S.band;
    if (m <= 1024 || NPMAX == 1024) band_onchip_row<1024>(slots, soffs, gx, row, m, S, k, t, lds);
    else if (m <= 2048 || NPMAX == 2048) band_onchip_row<(NPMAX < 2048 ? NPMAX : 2048)>(slots, soffs, gx, row, m, S, k, t, lds);
    else if (m <= 4096 || NPMAX == 4096) band_onchip_row<(NPMAX < 4096 ? NPMAX : 4096)>(slots, soffs, gx, row, m, S, k, t, lds);
    else band_onchip_row<NPMAX>(slots, soffs, gx, row, m, S, k, t, lds);
  }
  if (threadIdx.x == 0) fall = (S.flags & LAPSUM_FLAG_FALLBACK) != 0;
  __syncthreads();
  if (fall && !fb.defer) missed_row<kBandNT>(fb, (int)row, lds.full);
}

hipError_t launch_band_onchip(const uint32_t *slots, const void *partials, int gx, int64_t rows, int64_t n,
                              int64_t cap, RowState *st, double k, double t, const SegArgs &fb, hipStream_t s) {
  const FilterPartial *part = reinterpret_cast<const FilterPartial *>(partials);
  const dim3 grid = rows_grid(1u, rows);
  if (cap <= 1024)
    hipLaunchKernelGGL(band_solve_onchip<1024>, grid, dim3(kBandNT), 0, s, slots, part, gx, rows, n, cap, st, k, t,
                       fb);
  else if (cap <= 2048)
    hipLaunchKernelGGL(band_solve_onchip<2048>, grid, dim3(kBandNT), 0, s, slots, part, gx, rows, n, cap, st, k, t,
                       fb);
  else if (cap <= 4096)
    hipLaunchKernelGGL(band_solve_onchip<4096>, grid, dim3(kBandNT), 0, s, slots, part, gx, rows, n, cap, st, k, t,
                       fb);
  else
    hipLaunchKernelGGL(band_solve_onchip<8192>, grid, dim3(kBandNT), 0, s, slots, part, gx, rows, n, cap, st, k, t,
                       fb);
  return hipGetLastError();
}

}  // namespace lapsum
