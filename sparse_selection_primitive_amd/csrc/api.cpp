// Host runtime of the C ABI declared in include/lapsum.h: argument checks,
// path choice, bracket indices, workspace layout and the launch sequence of
// each path on the caller's stream.  No device memory is allocated here and
// the stream is never synchronised.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "lapsum_device.hpp"
#include "lapsum_internal.hpp"

using namespace lapsum;

namespace {

constexpr size_t kAlign = 256;
constexpr int64_t kOnchipMaxN = LAPSUM_ONCHIP_MAX_N;
constexpr int64_t kBucketMaxAutoN = (int64_t)1 << 20;
constexpr int kDefaultWiden = 2;  // widened brackets tried after a miss, by default

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

struct Layout {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  }
};

// Offsets of the workspace regions of the large-row solver for `rows` rows
// of stride `stride` (a multiple of kTile).
struct SegRegions {
  size_t A, B, tagg, tpre, tsuf;
  int64_t stride;
  int max_tiles;
};

SegRegions seg_regions(Layout &L, int64_t rows, int64_t len) {
  SegRegions r;
  r.stride = round_up(len < 1 ? 1 : len, kTile);
  r.max_tiles = (int)(r.stride / kTile);
  const size_t keys = (size_t)rows * (size_t)r.stride * sizeof(uint32_t);
  r.A = L.take(keys);
  r.B = L.take(keys);
  r.tagg = L.take((size_t)rows * (size_t)r.max_tiles * tile_agg_bytes());
  r.tpre = L.take((size_t)rows * (size_t)r.max_tiles * pre_bytes());
  r.tsuf = L.take((size_t)rows * (size_t)r.max_tiles * suf_bytes());
  return r;
}

// Offsets of the workspace regions of the bucketed sort + solve: the band of
// the bracketing path (slots from gx filter workgroups), or whole rows of the
// full-sort path (full = true, n scores per row).
struct BandRegions {
  size_t keys, tmp, hist, hext, btot, bstart, bagg, bkey, bsum, tagg, tpre, tsuf, mm;
  int nblk, group, max_tiles;
  int64_t chunk;
};

BandRegions band_regions(Layout &L, int64_t rows, int64_t cap, int gx, bool full, int64_t n) {
  BandRegions r;
  r.group = 0;
  r.chunk = 0;
  r.mm = 0;
  r.nblk = full ? full_count_blocks(n, &r.chunk) : band_count_blocks(gx, &r.group);
  r.max_tiles = (int)(cap / kTile);
  const size_t keys = (size_t)rows * (size_t)cap * sizeof(uint32_t);
  const size_t nb = (size_t)rows * kBandBuckets;
  r.keys = L.take(keys);
  r.tmp = L.take(keys);
  r.hist = L.take(nb * (size_t)r.nblk * sizeof(uint32_t));
  r.hext = full ? L.take(2 * nb * (size_t)r.nblk * sizeof(uint32_t)) : 0;
  r.btot = L.take(nb * sizeof(uint32_t));
  r.bstart = L.take(nb * sizeof(uint32_t));
  r.bagg = full ? 0 : L.take(nb * tile_agg_bytes());
  r.bkey = full ? L.take(2 * nb * sizeof(uint32_t)) : 0;
  r.bsum = full ? L.take(2 * nb * sizeof(unsigned long long)) : 0;
  r.tagg = L.take((size_t)rows * (size_t)r.max_tiles * tile_agg_bytes());
  r.tpre = L.take((size_t)rows * (size_t)r.max_tiles * pre_bytes());
  r.tsuf = L.take((size_t)rows * (size_t)r.max_tiles * suf_bytes());
  if (full) r.mm = L.take((size_t)rows * (size_t)r.nblk * 2 * sizeof(uint32_t));
  return r;
}

// Offsets of the workspace regions of the whole-row radix sort and the
// solve over the sorted rows.
struct SortRegions {
  size_t A, B, cnt, dtot, ta, tp, ts;
  int64_t stride;
  int ntiles, nst;
};

SortRegions sort_regions(Layout &L, int64_t rows, int64_t n) {
  SortRegions r;
  r.stride = sort_stride(n);
  r.ntiles = sort_tiles(n);
  r.nst = solve_tiles(n);
  const size_t keys = (size_t)rows * (size_t)r.stride * sizeof(uint32_t);
  r.A = L.take(keys);
  r.B = L.take(keys);
  r.cnt = L.take((size_t)rows * 256 * (size_t)r.ntiles * sizeof(uint32_t));
  r.dtot = L.take((size_t)rows * 256 * sizeof(uint32_t));
  r.ta = L.take((size_t)rows * (size_t)r.nst * tile_agg_bytes());
  r.tp = L.take((size_t)rows * (size_t)r.nst * pre_bytes());
  r.ts = L.take((size_t)rows * (size_t)r.nst * suf_bytes());
  return r;
}

SortArgs sort_args(const SortRegions &R, char *ws, int64_t rows, int64_t n, const float *r, RowState *st, double k,
                   double t, RowParams rp) {
  SortArgs a;
  a.rows = rows;
  a.n = n;
  a.r = r;
  a.A = reinterpret_cast<uint32_t *>(ws + R.A);
  a.B = reinterpret_cast<uint32_t *>(ws + R.B);
  a.stride = R.stride;
  a.ntiles = R.ntiles;
  a.cnt = reinterpret_cast<uint32_t *>(ws + R.cnt);
  a.dtot = reinterpret_cast<uint32_t *>(ws + R.dtot);
  a.nst = R.nst;
  a.ta = reinterpret_cast<TileAgg *>(ws + R.ta);
  a.tp = reinterpret_cast<Pre *>(ws + R.tp);
  a.ts = reinterpret_cast<Suf *>(ws + R.ts);
  a.st = st;
  a.k = k;
  a.t = t;
  a.rp = rp;
  return a;
}

struct Plan {
  int path = 0;
  int sample_log2 = 0;
  int64_t m = 0, lo = 0, hi = 0;
  int nwiden = 0;  // widened brackets tried after a miss
  int64_t wlo[kMaxWiden] = {}, whi[kMaxWiden] = {};
  int64_t cap = 0;  // band capacity per row
  bool band_onchip = false;
  bool per_row = false;  // per-row k or t
  double delta = 0.0;    // bracketing: the miss bound of the first bracket
  // forward layout
  size_t fwd_bytes = 0;
  size_t st = 0, samples = 0, spart = 0, fpart = 0, slots = 0, offs = 0, tail = 0;
  int tailq = 0;  // depth of the per-group top lists (0: the general selection)
  int fgx = 0;
  BandRegions bnd{};
  SegRegions full_seg{};
  // bracketing with the spread fallback: the missed rows' own states and the
  // whole-row bucket regions their solve runs in
  bool spread = false;
  size_t st2 = 0;
  int64_t spread_cap = 0;
  BandRegions spread_bnd{};
  SortRegions srt{};
  size_t bis_state = 0, bis_part = 0;
  int bis_gx = 0;
  // backward layout
  size_t bwd_bytes = 0;
  size_t bpart = 0;
  int bgx = 0;
};

// Equal-tailed binomial order-statistic indices (host side of the
// localisation step), with a small cache per thread (the first bracket and
// its widened ones of the same call shape).
struct BracketCacheEntry {
  int64_t n = -1, m = -1, lo = 0, hi = 0;
  double k = -1.0, delta = -1.0;
};
constexpr int kBracketCache = 8;

lapsum_status bracket_indices(int64_t n, double k, int64_t m, double delta, int64_t *lo_out, int64_t *hi_out) {
  thread_local BracketCacheEntry cache[kBracketCache];
  thread_local int next = 0;
  for (const BracketCacheEntry &e : cache) {
    if (e.n == n && e.k == k && e.m == m && e.delta == delta) {
      *lo_out = e.lo;
      *hi_out = e.hi;
      return LAPSUM_OK;
    }
  }
  // N ~ Bin(m, q), q = 1 - k/n: log pmf by the ratio recurrence from j = 0
  const double lq = std::log1p(-k / (double)n);  // ln q
  const double l1q = std::log(k / (double)n);    // ln (1 - q)
  std::vector<double> lp((size_t)m + 1);
  lp[0] = (double)m * l1q;
  for (int64_t j = 0; j < m; ++j)
    lp[(size_t)j + 1] = lp[(size_t)j] + std::log((double)(m - j) / (double)(j + 1)) + lq - l1q;
  // normalise against the maximum to avoid underflow of the bulk, then sum tails
  double mx = lp[0];
  for (double v : lp) mx = v > mx ? v : mx;
  std::vector<double> pmf((size_t)m + 1);
  long double tot = 0.0L;
  for (int64_t j = 0; j <= m; ++j) {
    pmf[(size_t)j] = std::exp(lp[(size_t)j] - mx);
    tot += pmf[(size_t)j];
  }
  const double half = 0.5 * delta;
  // lo = max{l in [0, m] : P(N <= l-1) <= delta/2}
  int64_t lo = 0;
  long double acc = 0.0L;
  for (int64_t l = 1; l <= m; ++l) {
    acc += pmf[(size_t)(l - 1)];
    if ((double)(acc / tot) <= half)
      lo = l;
    else
      break;
  }
  // hi = min{h in [1, m+1] : P(N >= h) <= delta/2}
  int64_t hi = m + 1;
  acc = 0.0L;
  for (int64_t h = m; h >= 1; --h) {
    acc += pmf[(size_t)h];
    if ((double)(acc / tot) <= half)
      hi = h;
    else
      break;
  }
  BracketCacheEntry &e = cache[next];
  next = (next + 1) % kBracketCache;
  e.n = n;
  e.k = k;
  e.m = m;
  e.delta = delta;
  e.lo = lo;
  e.hi = hi;
  *lo_out = lo;
  *hi_out = hi;
  return LAPSUM_OK;
}

lapsum_status check_common(int64_t rows, int64_t n, double t) {
  if (rows < 1 || n < 1 || n > LAPSUM_MAX_N || rows > LAPSUM_MAX_ROWS) return LAPSUM_ERR_SHAPE;
  if ((double)rows * (double)n > 4.0e18) return LAPSUM_ERR_SHAPE;
  if (!std::isfinite(t) || !(t > 0.0)) return LAPSUM_ERR_T;
  return LAPSUM_OK;
}

// Workspace of the backward: depends on (rows, n) only.
void bwd_layout(int64_t rows, int64_t n, Plan &P) {
  Layout B;
  if (!onchip_backward_supported(n)) {
    P.bgx = bwd_grid_x(rows, n);
    P.bpart = B.take(bwd_partial_bytes(rows, P.bgx));
  }
  P.bwd_bytes = B.off;
}

lapsum_status make_plan(int64_t rows, int64_t n, double k, double t, const lapsum_options *opt, Plan &P) {
  lapsum_options o;
  lapsum_options_init(&o);
  if (opt) o = *opt;
  // per-row values replace the scalars, which are then neither used nor checked
  const bool per_row = o.k_rows != nullptr || o.t_rows != nullptr;
  lapsum_status st = check_common(rows, n, o.t_rows ? 1.0 : t);
  if (st != LAPSUM_OK) return st;
  if (!o.k_rows && (!std::isfinite(k) || !(k > 0.0) || !(k < (double)n))) return LAPSUM_ERR_K;
  if (o.path < LAPSUM_PATH_AUTO || o.path > LAPSUM_PATH_BISECT) return LAPSUM_ERR_OPTION;
  if (o.sample_log2 != 0 && (o.sample_log2 < 4 || o.sample_log2 > 20)) return LAPSUM_ERR_OPTION;
  if (!(o.delta == 0.0 || (o.delta > 0.0 && o.delta < 1.0))) return LAPSUM_ERR_OPTION;
  if (o.band_capacity < 0) return LAPSUM_ERR_OPTION;
  if (o.bracket_override && !(o.bracket_override[0] < o.bracket_override[1])) return LAPSUM_ERR_OPTION;
  if (o.widen_steps < -1 || o.widen_steps > kMaxWiden) return LAPSUM_ERR_OPTION;
  if (o.spread_fallback < 0 || o.spread_fallback > 1) return LAPSUM_ERR_OPTION;

  int path = o.path;
  if (path == LAPSUM_PATH_AUTO)
    path = n <= kOnchipMaxN ? LAPSUM_PATH_ONCHIP : (n <= kBucketMaxAutoN ? LAPSUM_PATH_BUCKET : LAPSUM_PATH_BRACKET);
  if (path == LAPSUM_PATH_ONCHIP && n > kOnchipMaxN) return LAPSUM_ERR_PATH;
  P.path = path;
  P.per_row = per_row;

  Layout F;
  if (path == LAPSUM_PATH_BUCKET) {
    P.st = F.take((size_t)rows * row_state_bytes());
    P.cap = round_up(n, kTile);
    P.bnd = band_regions(F, rows, P.cap, 0, true, n);
  } else if (path == LAPSUM_PATH_SORT) {
    P.st = F.take((size_t)rows * row_state_bytes());
    P.srt = sort_regions(F, rows, n);
  } else if (path == LAPSUM_PATH_BISECT) {
    P.st = F.take((size_t)rows * row_state_bytes());
    if (!bisect_onchip(n)) {
      P.bis_gx = bisect_grid_x(rows, n);
      P.bis_state = F.take(bisect_state_bytes(rows));
      P.bis_part = F.take(bisect_partial_bytes(rows, P.bis_gx));
    }
  } else if (path == LAPSUM_PATH_BRACKET) {
    int sl = o.sample_log2;
    if (sl == 0) {
      sl = 4;
      if (n >= 256) {
        sl = (int)std::floor(std::log2((double)n / 16.0));
        sl = sl < 4 ? 4 : (sl > 16 ? 16 : sl);
      }
    }
    P.sample_log2 = sl;
    P.m = (int64_t)1 << sl;
    const double delta = o.delta == 0.0 ? 1e-6 : o.delta;
    P.delta = delta;
    // with a budget per row the indices are the rows' own (set on the device);
    // the band is sized for the widest bracket, that of k = n/2
    bracket_indices(n, per_row && o.k_rows ? 0.5 * (double)n : k, P.m, delta, &P.lo, &P.hi);
    // widened brackets: step i takes the indices for delta * 1e-6^i, kept
    // only where they are wider than the bracket before them (none with
    // per-row budgets or the spread fallback: a missed row goes straight to
    // the exact whole-row solve)
    const int steps = (per_row || o.spread_fallback)
                          ? 0
                          : (o.widen_steps == 0 ? kDefaultWiden : (o.widen_steps < 0 ? 0 : o.widen_steps));
    int64_t plo = P.lo, phi = P.hi;
    double d = delta;
    for (int i = 0; i < steps; ++i) {
      d *= 1e-6;
      int64_t wl = 0, wh = 0;
      bracket_indices(n, k, P.m, d, &wl, &wh);
      if (wl < plo || wh > phi) {
        P.wlo[P.nwiden] = wl;
        P.whi[P.nwiden] = wh;
        ++P.nwiden;
        plo = wl;
        phi = wh;
      }
    }
    if (o.band_capacity > 0) {
      P.cap = o.band_capacity;
    } else {
      const int64_t lo_eff = P.lo, hi_eff = P.hi;  // lo = 0 / hi = m+1 mean open ends
      const double frac = (double)(hi_eff - lo_eff) / (double)P.m;
      double cap = 3.0 * frac * (double)n + 1024.0;
      if (cap > (double)n) cap = (double)n;
      P.cap = (int64_t)std::ceil(cap);
    }
    if (P.cap < 1) P.cap = 1;
    // per-row values: the bucketed band solve, which reads each row's own
    // k and t (the on-chip one takes the call's)
    P.band_onchip = P.cap <= kOnchipMaxN && !per_row;
    if (!P.band_onchip) P.cap = round_up(P.cap, kTile);
    P.st = F.take((size_t)rows * row_state_bytes());
    P.samples = F.take((size_t)rows * (size_t)P.m * sizeof(float));
    P.spart = F.take(sample_start_bytes(rows, P.m));
    P.tailq = per_row ? 0 : tail_depth(P.m, P.lo, P.hi);
    if (P.tailq > 0) P.tail = F.take(tail_bytes(rows, P.m, P.tailq));
    P.fgx = filter_grid_x(rows, n, P.cap);
    P.fpart = F.take(filter_partial_bytes(rows, P.fgx));
    P.slots = F.take(band_slot_bytes(rows, P.fgx));
    P.offs = F.take(band_offs_bytes(rows, P.fgx));
    if (!P.band_onchip) P.bnd = band_regions(F, rows, P.cap, P.fgx, false, n);
    if (o.spread_fallback) {
      // a missed row is solved by the whole-row bucket launches after the
      // band kernels; the one-workgroup fallback's buffers are not needed
      // (its argument block points at the bucket regions, never read)
      P.spread = true;
      P.st2 = F.take((size_t)rows * row_state_bytes());
      P.spread_cap = round_up(n, kTile);
      P.spread_bnd = band_regions(F, rows, P.spread_cap, 0, true, n);
      P.full_seg.A = P.spread_bnd.keys;
      P.full_seg.B = P.spread_bnd.tmp;
      P.full_seg.tagg = P.spread_bnd.tagg;
      P.full_seg.tpre = P.spread_bnd.tpre;
      P.full_seg.tsuf = P.spread_bnd.tsuf;
      P.full_seg.stride = P.spread_cap;
      P.full_seg.max_tiles = P.spread_bnd.max_tiles;
    } else {
      P.full_seg = seg_regions(F, rows, n);
    }
  }
  P.fwd_bytes = F.off;

  bwd_layout(rows, n, P);
  return LAPSUM_OK;
}

struct StageTimer {
  void *const *ev;
  hipStream_t s;
  void mark(int stage, int which) const {
    if (!ev) return;
    void *e = ev[2 * stage + which];
    if (e) (void)hipEventRecord((hipEvent_t)e, s);
  }
};

#define LAPSUM_TRY(expr)                       \
  do {                                         \
    hipError_t _e = (expr);                    \
    if (_e != hipSuccess) return LAPSUM_ERR_HIP; \
  } while (0)

SegArgs seg_args(const SegRegions &R, char *ws, int64_t rows, int64_t n, const float *r, RowState *st, double k,
                 double t) {
  SegArgs a{};
  a.rows = (int)rows;
  a.n = n;
  a.r = r;
  a.A = reinterpret_cast<uint32_t *>(ws + R.A);
  a.B = reinterpret_cast<uint32_t *>(ws + R.B);
  a.stride = R.stride;
  a.max_tiles = R.max_tiles;
  a.tagg = reinterpret_cast<TileAgg *>(ws + R.tagg);
  a.tpre = reinterpret_cast<Pre *>(ws + R.tpre);
  a.tsuf = reinterpret_cast<Suf *>(ws + R.tsuf);
  a.st = st;
  a.k = k;
  a.t = t;
  a.c = kLog2e / t;
  a.cf = (float)a.c;
  a.samples = nullptr;
  a.m = 0;
  a.nwiden = 0;
  for (int i = 0; i < kMaxWiden; ++i) a.wlo[i] = a.whi[i] = 0;
  return a;
}

// Band mode (slots non-null: the plan's band regions and capacity) or whole
// rows (r non-null: the given regions, cap = the padded row length).
BandArgs band_args(const Plan &P, const BandRegions &R, int64_t cap, char *ws, int64_t rows, RowState *st,
                   const uint32_t *slots, uint32_t *offs, double k, double t, const float *r, int64_t n,
                   RowParams rp) {
  BandArgs a{};
  a.rp = rp;
  a.nested = 0;  // the launcher decides
  a.src2 = nullptr;
  a.need = 0;
  a.st_out = nullptr;
  a.rows = (int)rows;
  a.gx = P.fgx;
  a.group = R.group;
  a.nblk = R.nblk;
  a.slots = slots;
  a.offs = offs;
  a.part = reinterpret_cast<const FilterPartial *>(ws + P.fpart);
  a.r = r;
  a.n = n;
  a.chunk = R.chunk;
  // about 32 keys per bucket: the whole row, or the band expected for this
  // capacity (a third of it)
  a.bbits = bucket_bits(r != nullptr ? n : cap / 3);
  a.mm = r != nullptr ? reinterpret_cast<uint32_t *>(ws + R.mm) : nullptr;
  a.st = st;
  a.keys = reinterpret_cast<uint32_t *>(ws + R.keys);
  a.tmp = reinterpret_cast<uint32_t *>(ws + R.tmp);
  a.hist = reinterpret_cast<uint32_t *>(ws + R.hist);
  a.btot = reinterpret_cast<uint32_t *>(ws + R.btot);
  a.bstart = reinterpret_cast<uint32_t *>(ws + R.bstart);
  a.hext = r != nullptr ? reinterpret_cast<uint32_t *>(ws + R.hext) : nullptr;
  a.bagg = r == nullptr ? reinterpret_cast<TileAgg *>(ws + R.bagg) : nullptr;
  a.bkey = r != nullptr ? reinterpret_cast<uint32_t *>(ws + R.bkey) : nullptr;
  a.bsum = r != nullptr ? reinterpret_cast<unsigned long long *>(ws + R.bsum) : nullptr;
  a.tagg = reinterpret_cast<TileAgg *>(ws + R.tagg);
  a.tpre = reinterpret_cast<Pre *>(ws + R.tpre);
  a.tsuf = reinterpret_cast<Suf *>(ws + R.tsuf);
  a.cap = cap;
  a.max_tiles = R.max_tiles;
  a.k = k;
  a.t = t;
  a.c = kLog2e / t;
  a.cf = (float)a.c;
  return a;
}

}  // namespace

extern "C" {

void lapsum_options_init(lapsum_options *opt) {
  if (!opt) return;
  std::memset(opt, 0, sizeof(*opt));
  opt->path = LAPSUM_PATH_AUTO;
}

const char *lapsum_status_string(lapsum_status st) {
  switch (st) {
    case LAPSUM_OK: return "ok";
    case LAPSUM_ERR_NULL: return "a required pointer is NULL";
    case LAPSUM_ERR_SHAPE: return "invalid shape (rows, n)";
    case LAPSUM_ERR_K: return "k must be finite with 0 < k < n";
    case LAPSUM_ERR_T: return "t must be finite and > 0";
    case LAPSUM_ERR_WORKSPACE: return "workspace too small or not 256-byte aligned";
    case LAPSUM_ERR_PATH: return "the requested path cannot run this shape";
    case LAPSUM_ERR_OPTION: return "an option is out of range";
    case LAPSUM_ERR_HIP: return "HIP launch or runtime error";
    case LAPSUM_ERR_SCRATCH: return "the call needs more scratch than the fixed no-alloc buffer holds";
  }
  return "unknown status";
}

lapsum_status lapsum_bracket_indices(int64_t n, double k, int64_t m, double delta, int64_t *lo, int64_t *hi) {
  if (!lo || !hi) return LAPSUM_ERR_NULL;
  if (n < 1 || n > LAPSUM_MAX_N || m < 1 || m > ((int64_t)1 << 24)) return LAPSUM_ERR_SHAPE;
  if (!std::isfinite(k) || !(k > 0.0) || !(k < (double)n)) return LAPSUM_ERR_K;
  if (!(delta > 0.0 && delta < 1.0)) return LAPSUM_ERR_OPTION;
  return bracket_indices(n, k, m, delta, lo, hi);
}

lapsum_status lapsum_plan(int64_t rows, int64_t n, double k, double t, const lapsum_options *opt,
                          lapsum_plan_info *out) {
  if (!out) return LAPSUM_ERR_NULL;
  Plan P;
  const lapsum_status st = make_plan(rows, n, k, t, opt, P);
  if (st != LAPSUM_OK) return st;
  std::memset(out, 0, sizeof(*out));
  out->path = P.path;
  out->sample_log2 = P.sample_log2;
  out->m = P.m;
  out->lo = P.per_row && P.path == LAPSUM_PATH_BRACKET ? -1 : P.lo;
  out->hi = P.per_row && P.path == LAPSUM_PATH_BRACKET ? -1 : P.hi;
  out->band_capacity = P.cap;
  out->band_onchip = P.band_onchip ? 1 : 0;
  out->filter_groups = P.fgx;
  out->forward_bytes = P.fwd_bytes;
  out->backward_bytes = P.bwd_bytes;
  return LAPSUM_OK;
}

size_t lapsum_workspace_bytes(int64_t rows, int64_t n, double k, double t, const lapsum_options *opt) {
  Plan P;
  if (make_plan(rows, n, k, t, opt, P) != LAPSUM_OK) return 0;
  return P.fwd_bytes > P.bwd_bytes ? P.fwd_bytes : P.bwd_bytes;
}

lapsum_status lapsum_forward(const float *r, int64_t rows, int64_t n, double k, double t, float *p, double *b,
                             void *workspace, size_t workspace_bytes, const lapsum_options *opt, void *stream) {
  Plan P;
  const lapsum_status st0 = make_plan(rows, n, k, t, opt, P);
  if (st0 != LAPSUM_OK) return st0;
  if (!r || !p || !b) return LAPSUM_ERR_NULL;
  if (P.fwd_bytes > 0) {
    if (!workspace) return LAPSUM_ERR_NULL;
    if (workspace_bytes < P.fwd_bytes || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
      return LAPSUM_ERR_WORKSPACE;
  }
  lapsum_options o;
  lapsum_options_init(&o);
  if (opt) o = *opt;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const StageTimer tm{o.stage_events, s};
  char *ws = reinterpret_cast<char *>(workspace);
  const RowParams rp{o.k_rows, o.t_rows};
  // Launch errors are read back with hipGetLastError(); drop any non-sticky
  // error an earlier, unrelated runtime call left pending on this thread.
  (void)hipGetLastError();

  if (P.path == LAPSUM_PATH_ONCHIP) {
    tm.mark(LAPSUM_STAGE_ONCHIP_FWD, 0);
    LAPSUM_TRY(launch_onchip_forward(r, rows, (int)n, k, t, rp, p, b, o.stats, s));
    tm.mark(LAPSUM_STAGE_ONCHIP_FWD, 1);
    return LAPSUM_OK;
  }

  RowState *rs = reinterpret_cast<RowState *>(ws + P.st);
  if (P.path == LAPSUM_PATH_BUCKET) {
    tm.mark(LAPSUM_STAGE_INIT, 0);
    LAPSUM_TRY(launch_init_rows(rs, rows, 0, nullptr, n, k, t, rp, s));
    tm.mark(LAPSUM_STAGE_INIT, 1);
    tm.mark(LAPSUM_STAGE_BUCKET, 0);
    const SegArgs none{};  // full rows have no bracket, so no fallback
    LAPSUM_TRY(launch_band_buckets(band_args(P, P.bnd, P.cap, ws, rows, rs, nullptr, nullptr, k, t, r, n, rp), none,
                                   s));
    tm.mark(LAPSUM_STAGE_BUCKET, 1);
  } else if (P.path == LAPSUM_PATH_SORT) {
    tm.mark(LAPSUM_STAGE_INIT, 0);
    LAPSUM_TRY(launch_init_rows(rs, rows, 0, nullptr, n, k, t, rp, s));
    tm.mark(LAPSUM_STAGE_INIT, 1);
    const SortArgs sa = sort_args(P.srt, ws, rows, n, r, rs, k, t, rp);
    tm.mark(LAPSUM_STAGE_SORT, 0);
    LAPSUM_TRY(launch_row_sort(sa, s));
    tm.mark(LAPSUM_STAGE_SORT, 1);
    tm.mark(LAPSUM_STAGE_SOLVE, 0);
    LAPSUM_TRY(launch_row_sort_solve(sa, s));
    tm.mark(LAPSUM_STAGE_SOLVE, 1);
  } else if (P.path == LAPSUM_PATH_BISECT) {
    tm.mark(LAPSUM_STAGE_INIT, 0);
    LAPSUM_TRY(launch_init_rows(rs, rows, 0, nullptr, n, k, t, rp, s));
    tm.mark(LAPSUM_STAGE_INIT, 1);
    tm.mark(LAPSUM_STAGE_BISECT, 0);
    if (bisect_onchip(n)) {
      // the on-chip bisection writes p and b itself
      LAPSUM_TRY(launch_bisect_onchip(r, rows, n, k, t, rp, p, b, s));
      tm.mark(LAPSUM_STAGE_BISECT, 1);
      if (o.stats) LAPSUM_TRY(launch_copy_stats(rs, rows, o.stats, s));
      return LAPSUM_OK;
    }
    LAPSUM_TRY(launch_bisect_stream(r, rows, n, k, t, rp, ws + P.bis_state, ws + P.bis_part, P.bis_gx, rs, s));
    tm.mark(LAPSUM_STAGE_BISECT, 1);
  } else {
    const double *ovr = o.bracket_override;
    if (ovr) {
      tm.mark(LAPSUM_STAGE_INIT, 0);
      LAPSUM_TRY(launch_init_rows(rs, rows, LAPSUM_FLAG_BRACKET, ovr, n, k, t, rp, s));
      tm.mark(LAPSUM_STAGE_INIT, 1);
    } else {
      // the sample kernel also resets the rows' state
      float *samples = reinterpret_cast<float *>(ws + P.samples);
      uint16_t *spart = reinterpret_cast<uint16_t *>(ws + P.spart);
      tm.mark(LAPSUM_STAGE_SAMPLE, 0);
      uint32_t *tail = P.tailq > 0 ? reinterpret_cast<uint32_t *>(ws + P.tail) : nullptr;
      LAPSUM_TRY(launch_sample(r, rows, n, t, P.m, o.seed, samples, spart, rs, LAPSUM_FLAG_BRACKET, tail, P.tailq,
                               o.t_rows, s));
      tm.mark(LAPSUM_STAGE_SAMPLE, 1);
      tm.mark(LAPSUM_STAGE_SELECT, 0);
      if (P.per_row) {
        // each row's own indices (and k, t) into its state; the selection reads them
        LAPSUM_TRY(launch_bracket_rows(o.k_rows, o.t_rows, k, t, rows, n, P.m, P.delta, rs, s));
        LAPSUM_TRY(launch_select(samples, spart, rows, P.m, -1, -1, rs, s));
      } else if (tail != nullptr) {
        LAPSUM_TRY(launch_select_tail(tail, rows, P.m, P.tailq, P.lo, P.hi, rs, s));
      } else {
        LAPSUM_TRY(launch_select(samples, spart, rows, P.m, P.lo, P.hi, rs, s));
      }
      tm.mark(LAPSUM_STAGE_SELECT, 1);
    }
    uint32_t *slots = reinterpret_cast<uint32_t *>(ws + P.slots);
    uint32_t *offs = reinterpret_cast<uint32_t *>(ws + P.offs);
    tm.mark(LAPSUM_STAGE_FILTER, 0);
    LAPSUM_TRY(launch_filter(r, rows, n, t, rs, slots, ws + P.fpart, P.fgx, P.per_row, s));
    tm.mark(LAPSUM_STAGE_FILTER, 1);
    tm.mark(LAPSUM_STAGE_BAND, 0);
    SegArgs fb = seg_args(P.full_seg, ws, rows, n, r, rs, k, t);
    fb.per_row = P.per_row ? 1 : 0;
    fb.defer = P.spread ? 1 : 0;
    if (!ovr) {  // a bracket given by the caller has no sample to widen from
      fb.samples = reinterpret_cast<const float *>(ws + P.samples);
      fb.m = P.m;
      fb.nwiden = P.nwiden;
      for (int i = 0; i < P.nwiden; ++i) {
        fb.wlo[i] = P.wlo[i];
        fb.whi[i] = P.whi[i];
      }
    }
    // the band kernels also run the fallback for rows whose bracket missed
    if (P.band_onchip)
      LAPSUM_TRY(launch_band_onchip(slots, ws + P.fpart, P.fgx, rows, n, P.cap, rs, k, t, fb, s));
    else
      LAPSUM_TRY(launch_band_buckets(band_args(P, P.bnd, P.cap, ws, rows, rs, slots, offs, k, t, nullptr, n, rp), fb,
                                     s));
    if (P.spread) {
      // the rows whose bracket missed (flagged in their own states): the
      // whole-row bucket solve on every workgroup, b written back to rs
      RowState *rs2 = reinterpret_cast<RowState *>(ws + P.st2);
      BandArgs wa = band_args(P, P.spread_bnd, P.spread_cap, ws, rows, rs2, nullptr, nullptr, k, t, r, n, rp);
      wa.need = kFlagDeferred;
      wa.st_out = rs;
      LAPSUM_TRY(launch_band_buckets(wa, SegArgs{}, s));
    }
    tm.mark(LAPSUM_STAGE_BAND, 1);
  }
  tm.mark(LAPSUM_STAGE_APPLY, 0);
  LAPSUM_TRY(launch_apply(r, rows, n, rs, t, rp, p, b, s));
  tm.mark(LAPSUM_STAGE_APPLY, 1);
  if (o.stats) LAPSUM_TRY(launch_copy_stats(rs, rows, o.stats, s));
  return LAPSUM_OK;
}

size_t lapsum_midpoint_workspace_bytes(int64_t rows, int64_t n) {
  if (check_common(rows, n, 1.0) != LAPSUM_OK) return 0;
  Layout L;
  sort_regions(L, rows, n);
  L.take(midpoint_partial_bytes(rows, midpoint_grid_x(rows, n)));
  return L.off;
}

lapsum_status lapsum_midpoint_mass(const float *r, int64_t rows, int64_t n, int64_t k, double t, double *b_mid,
                                   double *mass, void *workspace, size_t workspace_bytes, void *stream) {
  const lapsum_status st0 = check_common(rows, n, t);
  if (st0 != LAPSUM_OK) return st0;
  if (n < 2 || k < 1 || k > n - 1) return LAPSUM_ERR_K;
  if (!r || !b_mid || !mass || !workspace) return LAPSUM_ERR_NULL;
  Layout L;
  const SortRegions R = sort_regions(L, rows, n);
  const int gx = midpoint_grid_x(rows, n);
  const size_t part = L.take(midpoint_partial_bytes(rows, gx));
  if (workspace_bytes < L.off || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
    return LAPSUM_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char *ws = reinterpret_cast<char *>(workspace);
  (void)hipGetLastError();  // see lapsum_forward
  const SortArgs sa = sort_args(R, ws, rows, n, r, nullptr, (double)k, t, RowParams{nullptr, nullptr});
  LAPSUM_TRY(launch_row_sort(sa, s));
  LAPSUM_TRY(launch_midpoint(sa, k, b_mid, mass, ws + part, gx, s));
  return LAPSUM_OK;
}

}  // extern "C"

namespace {

// The backward's argument checks and launch sequence on a given scratch
// (a caller workspace, or the fixed no-alloc buffer when `fixed`).
lapsum_status backward_impl(const float *g, const float *p, const double *b, int64_t rows, int64_t n, double t,
                            float *dr, float *dk, void *workspace, size_t workspace_bytes, bool fixed,
                            const lapsum_options *opt, void *stream) {
  lapsum_options o;
  lapsum_options_init(&o);
  if (opt) o = *opt;
  lapsum_status st0 = check_common(rows, n, o.t_rows ? 1.0 : t);
  if (st0 != LAPSUM_OK) return st0;
  if (!g || !p || !b || !dr || !dk) return LAPSUM_ERR_NULL;
  const RowParams rp{nullptr, o.t_rows};
  Plan P;
  bwd_layout(rows, n, P);
  if (fixed) {
    if (P.bwd_bytes > LAPSUM_NOALLOC_SCRATCH_BYTES) return LAPSUM_ERR_SCRATCH;
  } else if (P.bwd_bytes > 0) {
    if (!workspace) return LAPSUM_ERR_NULL;
    if (workspace_bytes < P.bwd_bytes || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
      return LAPSUM_ERR_WORKSPACE;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const StageTimer tm{o.stage_events, s};
  (void)hipGetLastError();  // see lapsum_forward
  if (onchip_backward_supported(n)) {
    tm.mark(LAPSUM_STAGE_ONCHIP_BWD, 0);
    LAPSUM_TRY(launch_onchip_backward(g, p, rows, (int)n, t, rp, dr, dk, o.stats, s));
    tm.mark(LAPSUM_STAGE_ONCHIP_BWD, 1);
    return LAPSUM_OK;
  }
  if (fixed) LAPSUM_TRY(noalloc_scratch(&workspace));
  char *ws = reinterpret_cast<char *>(workspace);
  tm.mark(LAPSUM_STAGE_BWD_REDUCE, 0);
  LAPSUM_TRY(launch_bwd_reduce(g, p, rows, n, ws + P.bpart, P.bgx, s));
  tm.mark(LAPSUM_STAGE_BWD_REDUCE, 1);
  tm.mark(LAPSUM_STAGE_BWD_APPLY, 0);
  LAPSUM_TRY(launch_bwd_apply(g, p, rows, n, ws + P.bpart, P.bgx, t, rp, dr, dk, o.stats, s));
  tm.mark(LAPSUM_STAGE_BWD_APPLY, 1);
  return LAPSUM_OK;
}

}  // namespace

extern "C" {

lapsum_status lapsum_backward(const float *g, const float *p, const double *b, int64_t rows, int64_t n, double t,
                              float *dr, float *dk, void *workspace, size_t workspace_bytes,
                              const lapsum_options *opt, void *stream) {
  return backward_impl(g, p, b, rows, n, t, dr, dk, workspace, workspace_bytes, false, opt, stream);
}

lapsum_status lapsum_backward_noalloc(const float *g, const float *p, const double *b, int64_t rows, int64_t n,
                                      double t, float *dr, float *dk, const lapsum_options *opt, void *stream) {
  return backward_impl(g, p, b, rows, n, t, dr, dk, nullptr, 0, true, opt, stream);
}

}  // extern "C"
