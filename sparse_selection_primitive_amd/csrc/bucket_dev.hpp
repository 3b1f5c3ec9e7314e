// Bucketed selection of the balancing interval ("Fast LapSum: Exact
// Differentiable Top-k at Million Scale", section 2.2, full-sort solver:
// threshold curve, index lookup of the balancing interval, closed-form
// root), shared by the bucketed band solve (band.hip) and the one-workgroup
// fallback of a row whose bracket missed (onchip.hip, band.hip).
//
// The keys of a set are spread over buckets by their leading bits above the
// set's smallest key; every key of bucket j is below every key of bucket
// j + 1.  The anchored sums of a bucket need only its largest and smallest
// key (they are order-free fixed-point sums), so the threshold curve at the
// bucket ends, and with it the bucket that holds the root, is found without
// sorting; only that bucket is sorted, and the root is taken inside it.
#pragma once

#include <limits.h>

#include "segment_dev.hpp"

namespace lapsum {

// ------------------------------------------------ order-free bucket sums
// Each term e^{-|x - anchor|/t} of a bucket lies in [0, 1] and is added as a
// 64-bit fixed-point number with agg_frac_bits(count) fraction bits, so the
// sum stays below 2^62 and is exact integer arithmetic in any order: the
// aggregates (and everything computed from them) are bitwise reproducible.
// A term loses at most 2^-(fb+1) to the rounding; fb >= 30 for any bucket.
LDEV int agg_frac_bits(uint32_t cnt) { return 62 - (32 - __clz((int)cnt)); }
LDEV unsigned long long fixed_term(float v, int fb) { return __float2ull_rn(ldexpf(v, fb)); }
LDEV double fixed_value(unsigned long long v, int fb) { return ldexp((double)v, -fb); }

// ----------------------------------------------------------- bucket search
// The bucket that holds the root, and what lies around it.
struct BucketPick {
  int J;                  // -1: the set is empty
  int64_t cnt, start;     // keys of bucket J, keys below it (in the set)
  float lo_a, hi_a;       // everything below / above bucket J, seeds included:
  double lo_s, hi_s;      //   a P-type sum (lo) and an S-type sum (hi)
  int first, last;        // no key of the set lies below / above bucket J
};

// The first NSEARCH threads of a workgroup of NT threads hold PER
// consecutive buckets each (aggregates g: aP/sP anchored at the bucket's
// largest key, aS/sS at its smallest; counts cnt).  The set has `total`
// keys; seed_lo / seed_hi hold everything below / above it and cR counts
// the keys above it.  Scan of the bucket aggregates (inside each wave on
// DPP, the wave totals through LDS), threshold curve at the last key of
// every non-empty bucket, and the balancing bucket: the first whose last
// key has g < k, else the last non-empty one.  Every thread of the
// workgroup must call; all of them get the pick.
template <int NT, int NSEARCH, int PER>
LDEV BucketPick bucket_search(const TileAgg (&g)[PER], const uint32_t (&cnt)[PER], Pre seed_lo, Suf seed_hi,
                              double cR, int64_t total, double k, double c) {
  constexpr int NW = NSEARCH / kWave;
  static_assert(NW <= 16 && NSEARCH <= NT, "search waves are combined inside one DPP row");
  __shared__ float tw_a[2][NW];
  __shared__ double tw_s[2][NW];
  __shared__ uint32_t tw_c[NW];
  __shared__ int red[3][NW];
  __shared__ BucketPick pick;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const bool searcher = threadIdx.x < NSEARCH;
  const int j0 = threadIdx.x * PER;
  // this thread's buckets joined, then exclusive scans over the search
  // threads (counts, P-type and S-type sums)
  Pre tp{0.0f, 0.0}, xp{0.0f, 0.0};
  Suf ts{0.0f, 0.0}, xs{0.0f, 0.0};
  uint32_t ct = 0u, xc = 0u;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    tp = join(tp, Pre{g[u].aP, g[u].sP}, c);
    ct += cnt[u];
  }
#pragma unroll
  for (int u = PER - 1; u >= 0; --u) ts = join(Suf{g[u].aS, g[u].sS}, ts, c);
  if (searcher) {
    const Pre ip = wave_scan(tp, c, &xp);
    const Suf is = wave_scan(ts, c, &xs);
    const uint32_t ic = wave_incl_scan(ct);
    xc = ic - ct;
    if (lane == kWave - 1) {
      tw_a[0][w] = ip.a;
      tw_s[0][w] = ip.s;
      tw_c[w] = ic;
    }
    if (lane == 0) {
      tw_a[1][w] = is.a;
      tw_s[1][w] = is.s;
    }
  }
  __syncthreads();
  int first_lt = INT_MAX, first_ne = INT_MAX, last_ne = -1;
  Pre before[PER];
  Suf after[PER];
  uint32_t st0[PER];
  if (searcher) {
    Pre twp = lane < NW ? Pre{tw_a[0][lane], tw_s[0][lane]} : Pre{0.0f, 0.0};
    Suf tws = lane < NW ? Suf{tw_a[1][lane], tw_s[1][lane]} : Suf{0.0f, 0.0};
    row_pre_steps<1>(twp, c);
    row_suf_steps<1>(tws, c);
    const int wb = __builtin_amdgcn_readfirstlane(w - 1), wa = __builtin_amdgcn_readfirstlane(w + 1);
    const Pre wp = w == 0 ? Pre{0.0f, 0.0} : Pre{read_lane(twp.a, wb), read_lane(twp.s, wb)};
    const Suf ws = w == NW - 1 ? Suf{0.0f, 0.0} : Suf{read_lane(tws.a, wa), read_lane(tws.s, wa)};
    uint32_t cbase = xc;
    for (int i = 0; i < w; ++i) cbase += tw_c[i];
    // everything before / after each bucket of this thread
    before[0] = join(seed_lo, join(wp, xp, c), c);
    after[PER - 1] = join(join(xs, ws, c), seed_hi, c);
#pragma unroll
    for (int u = 1; u < PER; ++u) before[u] = join(before[u - 1], Pre{g[u - 1].aP, g[u - 1].sP}, c);
#pragma unroll
    for (int u = PER - 2; u >= 0; --u) after[u] = join(Suf{g[u + 1].aS, g[u + 1].sS}, after[u + 1], c);
    // threshold curve at the last key of every non-empty bucket
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      st0[u] = cbase;
      cbase += cnt[u];
      if (cnt[u] > 0u) {
        const int j = j0 + u;
        const Pre pl = join(before[u], Pre{g[u].aP, g[u].sP}, c);
        const Suf sa = after[u];
        const double s_last = 1.0 + (sa.s == 0.0 ? 0.0 : sa.s * (double)wexp((double)pl.a - (double)sa.a, c));
        const int64_t j_last = (int64_t)st0[u] + cnt[u] - 1;
        const double gv = 0.5 * (pl.s - 1.0) + ((double)(total - j_last) + cR) - 0.5 * s_last;
        if (gv < k) first_lt = min(first_lt, j);
        first_ne = min(first_ne, j);
        last_ne = max(last_ne, j);
      }
    }
    first_lt = wave_reduce(first_lt, [](int x, int y) { return min(x, y); });
    first_ne = wave_reduce(first_ne, [](int x, int y) { return min(x, y); });
    last_ne = wave_reduce(last_ne, [](int x, int y) { return max(x, y); });
    if (lane == 0) {
      red[0][w] = first_lt;
      red[1][w] = first_ne;
      red[2][w] = last_ne;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    first_lt = min(first_lt, red[0][i]);
    first_ne = min(first_ne, red[1][i]);
    last_ne = max(last_ne, red[2][i]);
  }
  const int J = first_lt != INT_MAX ? first_lt : last_ne;  // -1: empty set
  if (J < 0 && threadIdx.x == 0) {
    pick.J = -1;
    pick.cnt = 0;
    pick.start = 0;
    pick.lo_a = seed_lo.a;
    pick.lo_s = seed_lo.s;
    pick.hi_a = seed_hi.a;
    pick.hi_s = seed_hi.s;
    pick.first = 1;
    pick.last = 1;
  }
  if (J >= 0 && searcher && (int)threadIdx.x == J / PER) {
    const int u0 = J % PER;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      if (u == u0) {
        pick.J = J;
        pick.cnt = cnt[u];
        pick.start = st0[u];
        pick.lo_a = before[u].a;
        pick.lo_s = before[u].s;
        pick.hi_a = after[u].a;
        pick.hi_s = after[u].s;
        pick.first = J == first_ne;
        pick.last = J == last_ne;
      }
    }
  }
  __syncthreads();
  const BucketPick out = pick;
  __syncthreads();  // the next call may overwrite `pick`
  return out;
}

// --------------------------------------------------------- sorting a range
// The whole workgroup sorts the keys kb[0 .. cnt) in place: stable LSD
// radix passes (8-bit digits) over the keys relative to `kb0`, the lowest
// key the range may hold (they differ from it in their low `bits` bits);
// tb is scratch of the same size.
template <int NT>
LDEV void block_radix_sort(uint32_t *kb, uint32_t *tb, int64_t cnt, uint32_t kb0, int bits, RankLds<NT> &L) {
  constexpr int TT = NT * kKpt;
  __shared__ uint32_t h[256];
  for (int64_t i = threadIdx.x; i < cnt; i += NT) kb[i] -= kb0;
  __syncthreads();
  uint32_t *src = kb, *dst = tb;
  const int npass = (bits + 7) / 8;
  const int64_t ntiles = (cnt + TT - 1) / TT;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  for (int pass = 0; pass < npass; ++pass) {
    const int sh = 8 * pass;
    for (int i = threadIdx.x; i < 256; i += NT) h[i] = 0u;
    __syncthreads();
    for (int64_t i = threadIdx.x; i < cnt; i += NT) atomicAdd(&h[(src[i] >> sh) & 255u], 1u);
    __syncthreads();
    uint32_t run = wg_excl_scan<NT>(threadIdx.x < 256 ? h[threadIdx.x] : 0u, L.wsum);
    for (int64_t tile = 0; tile < ntiles; ++tile) {
      uint32_t key[kKpt];
      int dig[kKpt];
#pragma unroll
      for (int q = 0; q < kKpt; ++q) {
        const int64_t gi = tile * TT + w * (kWave * kKpt) + q * kWave + lane;
        const bool valid = gi < cnt;
        key[q] = valid ? src[gi] : 0u;
        dig[q] = valid ? (int)((key[q] >> sh) & 255u) : 256;
      }
      const int vc = (int)min((int64_t)TT, cnt - tile * TT);
      run += scatter_tile<NT>(key, dig, sh, vc, run, dst, L);
    }
    uint32_t *x = src;
    src = dst;
    dst = x;
  }
  for (int64_t i = threadIdx.x; i < cnt; i += NT) kb[i] = src[i] + kb0;
  __syncthreads();
}

// One wave sorts a range of cnt <= 64*E keys in registers (blocked, E per
// lane) and solves for the root inside it.
template <int E>
LDEV double wave_sort_solve(const uint32_t *kb, int cnt, PartInfo part, double k, double t, double c, float cf) {
  WaveTeam<kWave> team;
  const int base = team.lane * E;
  uint32_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) key[e] = (base + e < cnt) ? kb[base + e] : 0xFFFFFFFFu;
  bitonic_sort<E>(key, team);
  const int nv = min(max(cnt - base, 0), E);
  float s[E];
#pragma unroll
  for (int e = 0; e < E; ++e) s[e] = (e < nv) ? value_of(key[e]) : 0.0f;
  part.nvalid = nv;
  return segment_solve<E>(s, nv, part, k, t, c, cf, team);
}

// The whole workgroup sorts a range of cnt keys in place (kb; tb scratch of
// the same size; the keys differ from kb0 in their low `bits` bits) and
// solves for the root inside it, given everything around it.
template <int NT>
LDEV double sorted_range_solve(uint32_t *kb, uint32_t *tb, int64_t cnt, uint32_t kb0, int bits, Pre slo, Suf shi,
                               double cR, bool first, bool last, TileAgg *ta, Pre *tp, Suf *tsuf, double k,
                               double t, double c, float cf, SegLds<NT> &L) {
  constexpr int TT = NT * kKpt;
  block_radix_sort<NT>(kb, tb, cnt, kb0, bits, L.rk);
  BlockTeam<NT, 1> team(&L.tm);
  for (int64_t t0 = 0; t0 < cnt; t0 += TT) {
    float s[kKpt];
    const int nv = load_sorted_at<NT>(kb, t0, cnt, 0u, s);
    tile_aggregate<NT>(s, nv, c, cf, team, ta + t0 / TT);
  }
  __syncthreads();
  return locate_sorted<NT>(kb, cnt, 0u, slo, shi, cR, first, last, ta, tp, tsuf, k, t, c, cf, team);
}

// ----------------------------------------------------- one-workgroup fallback
constexpr int kFallbackSort = 1 << 16;  // largest balancing bucket sorted directly

template <class F>
LDEV void fallback_each_key(const SegArgs &a, int row, const uint32_t *src, int64_t len, int nt, F &&f) {
  if (src != nullptr) {
    for (int64_t i = threadIdx.x; i < len; i += nt) f(src[i]);
    return;
  }
  typedef float f4 __attribute__((ext_vector_type(4)));
  const float *rr = a.r + (int64_t)row * a.n;
  if ((a.n & 3) == 0 && ((uintptr_t)rr & 15u) == 0) {
    constexpr int U = 4;
    const int64_t n4 = a.n >> 2;
    for (int64_t i0 = threadIdx.x; i0 < n4; i0 += (int64_t)nt * U) {
      f4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = i0 + (int64_t)u * nt;
        v[u] = i < n4 ? __builtin_nontemporal_load(reinterpret_cast<const f4 *>(rr) + i) : f4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (i0 + (int64_t)u * nt < n4) {
          f(key_of(v[u].x));
          f(key_of(v[u].y));
          f(key_of(v[u].z));
          f(key_of(v[u].w));
        }
      }
    }
  } else {
    for (int64_t i = threadIdx.x; i < a.n; i += nt) f(key_of(rr[i]));
  }
}

// Exact root over one key set and everything around it, by nested bucket
// selection: per level the buckets of the current set (counts and key
// extremes in one pass, fixed-point sums in a second), the balancing bucket,
// and its keys gathered into a key buffer.  A bucket of at most
// kFallbackSort keys (or of one distinct key) is sorted and solved; a larger
// one becomes the next level's set, seeded with everything around it.  The
// set is the row's scores (src == NULL, len = n) or len keys in src; kmin /
// kmax bound its keys; slo / shi hold everything below / above it and cR
// counts the elements above it.  Gathers go to the row's key buffer
// `cur` (0: A, 1: B) first, then alternate.  Returns b on every thread.
// Bucket of a key in a set bucketed by its bits above kmin (clamped to the
// last bucket).
LDEV uint32_t bucket_of(uint32_t key, uint32_t kmin, int shift) {
  const uint32_t j = (key - kmin) >> shift;
  return j < (uint32_t)(kFallbackBuckets - 1) ? j : (uint32_t)(kFallbackBuckets - 1);
}

template <int NT>
LDEV double bucket_set_solve(const SegArgs &a, int row, const uint32_t *src, int64_t len, int cur, uint32_t kmin,
                             uint32_t kmax, Pre slo, Suf shi, double cR, SegLds<NT> &L) {
  constexpr int PER = kFallbackBuckets / NT;
  static_assert(PER * NT == kFallbackBuckets, "every bucket has a thread");
  BucketSelLds &B = L.bs;
  const int lane = threadIdx.x & (kWave - 1);
  const unsigned long long ltmask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t *buf[2] = {a.A + (int64_t)row * a.stride, a.B + (int64_t)row * a.stride};
  const double c = a.c;
  double b = 0.0;
  for (;;) {
    const uint32_t span = len > 1 && kmax > kmin ? kmax - kmin : 0u;
    const int sbits = span == 0u ? 0 : 32 - __clz((int)span);
    const int shift = max(sbits - kFallbackBucketBits, 0);
    // counts and key extremes of the buckets
    for (int j = threadIdx.x; j < kFallbackBuckets; j += NT) {
      B.cnt[j] = 0u;
      B.kmx[j] = 0u;
      B.kmn[j] = 0xFFFFFFFFu;
      B.sp[j] = 0ull;
      B.ss[j] = 0ull;
    }
    __syncthreads();
    fallback_each_key(a, row, src, len, NT, [&](uint32_t key) {
      const uint32_t j = bucket_of(key, kmin, shift);
      atomicAdd(&B.cnt[j], 1u);
      atomicMax(&B.kmx[j], key);
      atomicMin(&B.kmn[j], key);
    });
    __syncthreads();
    // fixed-point sums anchored at the bucket extremes
    fallback_each_key(a, row, src, len, NT, [&](uint32_t key) {
      const uint32_t j = bucket_of(key, kmin, shift);
      const int fb = agg_frac_bits(B.cnt[j]);
      const double x = (double)value_of(key);
      atomicAdd(&B.sp[j], fixed_term(wexp(x - (double)value_of(B.kmx[j]), c), fb));
      atomicAdd(&B.ss[j], fixed_term(wexp((double)value_of(B.kmn[j]) - x, c), fb));
    });
    __syncthreads();
    TileAgg g[PER];
    uint32_t cnt[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int j = threadIdx.x * PER + u;
      cnt[u] = B.cnt[j];
      const int fb = cnt[u] > 0u ? agg_frac_bits(cnt[u]) : 0;
      g[u] = cnt[u] > 0u ? TileAgg{value_of(B.kmx[j]), value_of(B.kmn[j]), fixed_value(B.sp[j], fb),
                                   fixed_value(B.ss[j], fb)}
                         : TileAgg{0.0f, 0.0f, 0.0, 0.0};
    }
    const BucketPick P = bucket_search<NT, NT, PER>(g, cnt, slo, shi, cR, len, a.k, c);
    const uint32_t jmin = P.J >= 0 ? B.kmn[P.J] : 0u, jmax = P.J >= 0 ? B.kmx[P.J] : 0u;
    const Pre plo{P.lo_a, P.lo_s};
    const Suf phi{P.hi_a, P.hi_s};
    const double cR_eff = (double)(len - P.start - P.cnt) + cR;
    if (P.J < 0) {
      // nothing left (an empty set): the seeds alone place the root
      BlockTeam<NT, 1> team(&L.tm);
      b = locate_sorted<NT>(buf[cur], 0, 0u, plo, phi, cR_eff, true, true, a.tagg, a.tpre, a.tsuf, a.k, a.t, c,
                            a.cf, team);
      break;
    }
    // the keys of the balancing bucket into buf[cur]
    if (threadIdx.x == 0) B.ctr = 0u;
    __syncthreads();
    const uint32_t J = (uint32_t)P.J;
    uint32_t *dst = buf[cur];
    fallback_each_key(a, row, src, len, NT, [&](uint32_t key) {
      const bool in = bucket_of(key, kmin, shift) == J;
      const unsigned long long m = __ballot(in);
      if (m != 0ull) {
        const int leader = __ffsll((long long)m) - 1;
        uint32_t base = 0u;
        if (lane == leader) base = atomicAdd(&B.ctr, (uint32_t)__popcll(m));
        base = (uint32_t)__shfl((int)base, leader, kWave);
        if (in) dst[base + (uint32_t)__popcll(m & ltmask)] = key;
      }
    });
    __syncthreads();
    const bool single = jmin == jmax;  // one distinct key: already in order
    if (P.cnt <= kFallbackSort || single || shift == 0) {
      const int64_t o = (int64_t)row * a.max_tiles;
      b = sorted_range_solve<NT>(dst, buf[cur ^ 1], P.cnt, jmin, single ? 0 : shift, plo, phi, cR_eff, P.first != 0,
                                 P.last != 0, a.tagg + o, a.tpre + o, a.tsuf + o, a.k, a.t, c, a.cf, L);
      break;
    }
    // a large bucket: the next level's set
    src = dst;
    len = P.cnt;
    cur ^= 1;
    kmin = jmin;
    kmax = jmax;
    slo = plo;
    shi = phi;
    cR = cR_eff;
  }
  return b;
}

// The deterministic fallback for one row, run by a whole workgroup of NT
// threads: the row's key range (one pass over the scores), then the nested
// bucket selection over all of them.  Each level narrows the key range by
// 2^11, so at most three levels follow the first.  The result is the exact
// root of the whole row, independent of the bracket.
template <int NT>
LDEV void fallback_row(const SegArgs &a, int row, SegLds<NT> &L) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  // key range of the row (per-wave extremes through the widening scratch)
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  fallback_each_key(a, row, nullptr, a.n, NT, [&](uint32_t key) {
    kmin = min(kmin, key);
    kmax = max(kmax, key);
  });
  kmin = wave_reduce(kmin, [](uint32_t x, uint32_t y) { return x < y ? x : y; });
  kmax = wave_reduce(kmax, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
  if (lane == 0) {
    L.wd.kext[0][w] = kmin;
    L.wd.kext[1][w] = kmax;
  }
  __syncthreads();
  for (int i = 0; i < NW; ++i) {
    kmin = min(kmin, L.wd.kext[0][i]);
    kmax = max(kmax, L.wd.kext[1][i]);
  }
  __syncthreads();
  const double b = bucket_set_solve<NT>(a, row, nullptr, a.n, 0, kmin, kmax, Pre{0.0f, 0.0}, Suf{0.0f, 0.0}, 0.0, L);
  if (threadIdx.x == 0) a.st[row].b = b;
  __syncthreads();
}

}  // namespace lapsum
