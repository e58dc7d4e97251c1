// Sampled target row: temperature, top-k / top-p / min-p filtering and one
// inverse-CDF draw, computed by one workgroup in a single HBM pass.
//
// What is computed (xLLM docs, "Adaptive speculative inference", DSpark
// section "Launch example": a positive temperature samples the target with
// the ordinary sampler's top-k, top-p and min-p filters, and every verify row
// is sampled). With x the row, m its max and w_t = exp((x_t - m) / T):
//   rank order  = tokens by (x desc, index asc)
//   top-k       : first top_k tokens (off when top_k <= 0 or >= V)
//   top-p       : shortest prefix of those whose weight reaches top_p of
//                 their total, the crossing token kept (off when top_p >= 1)
//   min-p       : keep (x - m) / T >= ln(min_p) (off when min_p <= 0)
//   draw        : first token in rank order whose cumulative weight exceeds
//                 u times the survivors' total, u from Philox (device.hpp).
// Every decision is "the token at some rank", so it is enough to know the
// rank order and the cumulative weights near the few ranks that matter.
//
// How: the row is streamed once from HBM (row_stream.hpp) for its maximum
// and exponent sum, and every 16-byte vector leaves a 16-bit code of its
// maximum (rounded up to bfloat16, so an upper bound) in LDS. With the row
// maximum known, the capture threshold tau is exact: the maximum minus a
// window of 10 T (or the min-p cut), or, for a top-k row, the k-th largest
// vector maximum (a lower bound of the k-th largest element). A second pass
// over the codes picks the vectors that may hold an element >= tau, reads
// them again (from the device's last-level cache when the batch is small,
// mostly past the XCD's L2 otherwise: scattered 16-byte reads that cost one
// round trip of latency and whole lines of traffic) and keeps those
// elements in one candidate buffer. A 1024-bin histogram of (count, float64
// weight) over the candidates then locates each cut; only the bin a cut
// falls in is gathered and sorted. When the candidates cannot decide
// (survivor set or draw beyond them, too many candidates, huge tie groups),
// an exact radix-select over the whole row decides instead, reading the row
// again.
#pragma once

#include "kernels.hpp"
#include "row_stream.hpp"
#include "verify_common.hpp"

namespace vsv {

constexpr int kVM = 20480;      // vector-maximum codes per row (an entry covers S vectors when more)
constexpr int kCand = 4096;     // candidate slots per row
constexpr int kCapVec = 3072;   // most vectors a window capture reads again (about 1.2 elements each)
constexpr int kTopBins = 1024;  // top-k threshold: codes within this many of the maximum's
constexpr int kNB = 1024;       // histogram bins over the candidates
constexpr int kGather = 256;    // most elements one bin may hold
constexpr int kGatherFull = 512;  // the same for the whole-row locator
constexpr float kZcap = 10.0f;  // capture window below the row maximum, in units of T

struct Cand {
  float x;
  int idx;
};

// Order-preserving signed key of a float (-0 mapped to +0).
__device__ __forceinline__ int ord_key(float x) {
  const int b = __float_as_int(x == 0.0f ? 0.0f : x);
  return b >= 0 ? b : (b ^ 0x7FFFFFFF);
}
__device__ __forceinline__ float key_float(int k) { return __int_as_float(k >= 0 ? k : (k ^ 0x7FFFFFFF)); }
// Unsigned version (radix digits).
__device__ __forceinline__ uint32_t ord_ukey(float x) { return static_cast<uint32_t>(ord_key(x)) ^ 0x80000000u; }

template <int NT> struct SampledLds {
  static constexpr int NW = NT / kWave;
  static_assert(NT >= kGatherFull && kGatherFull >= kGather && NT <= 1024 && kNB % NT == 0 && kTopBins % NT == 0,
                "one gathered element per thread");
  union {
    struct {
      alignas(16) uint16_t l1[kVM];  // pass 1: entry codes; pass 2: indices of the picked entries
      uint16_t l2[kVM / 8];          // block codes (top-k rows)
    } vm;
    struct {
      int cnt[kNB + 1];
      double mass[kNB + 1];
      union {
        double wbin[kNB];     // bfloat16 rows: weight of each bin's value
        double gpm[kGatherFull];  // float32 rows: weight prefix of the gathered bin
      };
      Cand g[kGatherFull];
      Cand gs[kGatherFull];
    } post;
    struct {
      int cnt[256];
      double mass[256];
    } radix;
  } u;
  union {
    Cand cand[kCand];           // every element >= tau of the row
    int hist[NW][kTopBins];     // top-k threshold, before the capture
  } c;
  int ncand;
  int ovf;
  int gn;
  int bi[4];
  double bd[4];
  int red_i[NW];
  double red_d[2 * NW];
  RowScratch<NT> rs;
  LeanScratch<NT> ls;
  int row_next;  // the workgroup's next row (row queue)
  int ticket;    // its ticket (position in the queue)
  int last;      // this workgroup finished the call's last row
  uint16_t late[kLateRows];  // ordered queue: rows of the tickets past the grid
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float uni(float v) { return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v))); }
__device__ __forceinline__ void wave_lds_sync() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

__device__ __forceinline__ int mbcnt(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

// Lower *dst to v from the lowest lane of the wave that has a value. The
// callers' values grow with the thread index, so that lane holds the
// wave's least: one LDS atomic per wave, where one per lane would queue up
// to a workgroup's worth of same-address atomics (all threads past a cut
// qualify). Every lane of the wave must call it.
__device__ __forceinline__ void wave_first_min(int* dst, int v, bool has) {
  const uint64_t bal = __builtin_amdgcn_ballot_w64(has);
  if (has && lane_id() == __builtin_ctzll(bal)) atomicMin(dst, v);
}

// Row statistics of one decoded vector: running max and exponent sum (a
// sampled row needs no argmax position).
template <int N>
__device__ __forceinline__ void take_floats(RowPartial& p, const float* f, float vmax, float c) {
  p.best = fmaxf(p.best, vmax);
  partial_rebase(p, vmax, c);
  const float nmc = -p.mc;
  float e[N];
#pragma unroll
  for (int k = 0; k < N; ++k) e[k] = fast_exp2(fmaf(f[k], c, nmc));
  p.s += static_cast<double>(tree_sum<N>(e));
}

// The same for one vector of a group whose exponentials are summed in float
// before they reach the float64 sum: `gs` is the group's running float sum,
// rescaled with p.s when the exponent reference moves (both by an exact
// power of two). The caller adds gs to p.s once per group and keeps the
// group's maximum.
template <int N>
__device__ __forceinline__ void take_floats_group(RowPartial& p, const float* f, float vmax, float c, float& gs) {
  const float y = vmax * c;
  if (y > p.mc && y < FLT_MAX) {
    const float nm = ceilf(y);
    const bool had = p.mc > -FLT_MAX;
    const int d = static_cast<int>(fmaxf(p.mc - nm, -2000.f));
    p.s = had ? ldexp(p.s, d) : 0.0;
    gs = had ? ldexpf(gs, d) : 0.f;
    p.mc = nm;
  }
  const float nmc = -p.mc;
  float e[N];
#pragma unroll
  for (int k = 0; k < N; ++k) e[k] = fast_exp2(fmaf(f[k], c, nmc));
  gs += tree_sum<N>(e);
}

// ---------------------------------------------------------------- deciding

struct Pick {
  int idx;      // token (resolved lazily by the candidate locator: see token())
  int rank;     // 0-based position in the rank order
  double cum;   // cumulative weight through this token
  bool ok;      // false: the answer is not within reach of this locator
  int bin;      // candidate locator: the bin holding the token ...
  int off;      // ... and its position inside the bin's (x desc, idx asc) order
};

// Float64 weight exp((x - m) / T) of a logit, as the oracle defines it.
__device__ __forceinline__ double weight(float x, float m, double T) {
  return exp((static_cast<double>(x) - static_cast<double>(m)) / T);
}

// The stream weighs an element with exp2((x - m) c), c = log2(e) / T rounded
// to float; w = weight(x, m, T). The gap w - exp2((x - m) c) is
// -w (delta + delta^2 / 2 + ...) with delta = (x - m) dc and
// dc = c ln 2 - 1 / T (c_gap below). The float rounding of c bounds
// |delta| by 6e-8 |x - m| / T, so the first omitted term, w delta^3 / 6, is
// under float64 rounding of the total for every weight that is not itself
// negligible (|x - m| / T up to thousands).
__device__ __forceinline__ double c_gap(double c, double T) { return c * 0.69314718055994530942 - 1.0 / T; }
__device__ __forceinline__ double stream_gap(float x, float m, double w, double dc) {
  const double delta = (static_cast<double>(x) - static_cast<double>(m)) * dc;
  return -w * (delta + 0.5 * delta * delta);
}

// Block-wide inclusive scans (every thread one value; NT <= 1024).
template <int NT, typename T>
__device__ __forceinline__ T block_scan_incl(T v, T* scr, T& total) {
  const int lane = lane_id(), w = wave_id();
  v = wave_scan_incl(v);
  lds_barrier();
  if (lane == kWave - 1) scr[w] = v;
  lds_barrier();
  T before = 0, sum = 0;
#pragma unroll
  for (int k = 0; k < NT / kWave; ++k) {
    const T x = scr[k];
    before += (k < w) ? x : T(0);
    sum += x;
  }
  total = sum;
  return before + v;
}

// Block-wide inclusive scans of an int and one or two doubles at once: the
// same wave scans and the same sums over the waves as block_scan_incl, so
// the same results, behind one pair of barriers instead of one per value.
// si holds NT / kWave ints, sd twice that many doubles.
template <int NT, bool kTwo>
__device__ __forceinline__ void block_scan_incl_n(int& a, double& b, double& c, int* si, double* sd, int& ta, double& tb,
                                                  double& tc) {
  constexpr int NW = NT / kWave;
  const int lane = lane_id(), w = wave_id();
  a = wave_scan_incl(a);
  b = wave_scan_incl(b);
  if (kTwo) c = wave_scan_incl(c);
  lds_barrier();
  if (lane == kWave - 1) {
    si[w] = a;
    sd[w] = b;
    if (kTwo) sd[NW + w] = c;
  }
  lds_barrier();
  int ba = 0, sa = 0;
  double bb = 0, sb = 0, bc = 0, sc = 0;
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    const int xa = si[k];
    const double xb = sd[k];
    ba += (k < w) ? xa : 0;
    sa += xa;
    bb += (k < w) ? xb : 0.0;
    sb += xb;
    if (kTwo) {
      const double xc = sd[NW + k];
      bc += (k < w) ? xc : 0.0;
      sc += xc;
    }
  }
  ta = sa;
  tb = sb;
  tc = sc;
  a = ba + a;
  b = bb + b;
  if (kTwo) c = bc + c;
}
template <int NT>
__device__ __forceinline__ void block_scan_incl2(int& a, double& b, int* si, double* sd, int& ta, double& tb) {
  double c = 0.0, tc = 0.0;
  block_scan_incl_n<NT, false>(a, b, c, si, sd, ta, tb, tc);
}

// Order-preserving 16-bit code of a bfloat16 value (-0 mapped to +0), and back.
__device__ __forceinline__ int bf16_code(float x) {
  const uint32_t h = __float_as_uint(x == 0.0f ? 0.0f : x) >> 16;
  return (h & 0x8000u) ? static_cast<int>(~h & 0xFFFFu) : static_cast<int>(h | 0x8000u);
}
__device__ __forceinline__ float bf16_of_code(int o) {
  const uint32_t h = (o & 0x8000) ? static_cast<uint32_t>(o & 0x7FFF) : (~static_cast<uint32_t>(o) & 0xFFFFu);
  return __uint_as_float(h << 16);
}

// Locator over the captured candidates (every element >= tau of the row).
// The candidates are binned in rank order. bfloat16 rows bin by the value's
// code, so a bin holds one value and a cut inside it is plain arithmetic;
// float32 rows bin by value range and sort the bin a cut falls in.
template <typename E, int NT>
struct CandLocator {
  static constexpr bool kCode = sizeof(E) == 2;
  static constexpr int NW = NT / kWave;
  SampledLds<NT>& L;
  float m;
  double T;
  float tau;
  double scale;
  int mcode;        // bf16 code of the row maximum
  int nc;           // candidates in the bins
  double wtotal;    // weight of the whole row
  double c;         // the stream's float exponent scale log2(e) / T
  bool bad;         // a gather overflowed

  __device__ CandLocator(SampledLds<NT>& l, float m_, double T_, float tau_, double wt, double c_)
      : L(l), m(m_), T(T_), tau(tau_), scale(0), mcode(0), nc(0), wtotal(wt), c(c_), bad(false) {}

  __device__ int bin_of(float x) const {
    if (kCode) return mcode - bf16_code(x);
    const double d = static_cast<double>(m - x) * scale;
    return d < 0 ? 0 : (d >= kNB ? kNB - 1 : static_cast<int>(d));
  }
  __device__ bool in_bins(float x) const { return x >= tau && (!kCode || mcode - bf16_code(x) < kNB); }
  __device__ float bin_value(int b) const { return bf16_of_code(mcode - b); }

  // Build the bin counts and the exclusive prefixes of counts and weights.
  __device__ void build() {
    if (kCode) {
      mcode = bf16_code(m);
    } else {
      const float span = m - tau;
      scale = (span > 0.f && span < INFINITY) ? static_cast<double>(kNB) / static_cast<double>(span) : 0.0;
    }
    for (int b = threadIdx.x; b <= kNB; b += NT) {
      L.u.post.cnt[b] = 0;
      L.u.post.mass[b] = 0.0;
    }
    lds_barrier();
    // the stream summed every element with the rounded scale c; the
    // candidates' share is replaced by their exact weights
    double corr = 0.0;
    const double dc = c_gap(c, T);
    const int n = L.ncand;
    for (int j = threadIdx.x; j < n; j += NT) {
      const float x = L.c.cand[j].x;
      if (!in_bins(x)) continue;
      const int b = bin_of(x);
      atomicAdd(&L.u.post.cnt[b], 1);
      if (!kCode) {
        const double we = weight(x, m, T);
        atomicAdd(&L.u.post.mass[b], we);
        corr += stream_gap(x, m, we, dc);
      }
    }
    lds_barrier();
    constexpr int PER = kNB / NT;
    int lc[PER];
    double lm[PER];
    int sc = 0;
    double sm = 0.0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int b = threadIdx.x * PER + k;
      lc[k] = L.u.post.cnt[b];
      if (kCode) {
        // one value per bin: weight = count * exp((v - m) / T)
        double wb = 0.0;
        if (lc[k]) {
          const float v = bin_value(b);
          wb = weight(v, m, T);
          corr += lc[k] * stream_gap(v, m, wb, dc);
          lm[k] = lc[k] * wb;
          L.u.post.mass[b] = wb;   // per-element weight of the bin's value
        } else {
          lm[k] = 0.0;
        }
      } else {
        lm[k] = L.u.post.mass[b];
      }
      sc += lc[k];
      sm += lm[k];
    }
    int tc, ic = sc;
    double tm, tcorr, im = sm;
    block_scan_incl_n<NT, true>(ic, im, corr, L.red_i, L.red_d, tc, tm, tcorr);
    wtotal += tcorr;
    int ec = ic - sc;
    double em = im - sm;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int b = threadIdx.x * PER + k;
      if (kCode) L.u.post.wbin[b] = L.u.post.mass[b];
      L.u.post.cnt[b] = ec;
      L.u.post.mass[b] = em;
      ec += lc[k];
      em += lm[k];
    }
    if (threadIdx.x == 0) {
      L.u.post.cnt[kNB] = tc;
      L.u.post.mass[kNB] = tm;
    }
    lds_barrier();
    nc = tc;
  }

  __device__ double total_mass() const { return wtotal; }

  // At least the weight of any element the bins do not hold: those below
  // tau and, for bfloat16 rows (bins by code, kNB codes down from the
  // maximum's), the candidates at kNB or more codes below the maximum's,
  // which are no larger than the value of code mcode - kNB. A window that
  // reaches zero or below spans far more than kNB codes.
  __device__ double beyond_weight() const {
    float v = tau;
    if (kCode && mcode >= kNB) v = fmaxf(v, bf16_of_code(mcode - kNB));
    return weight(v, m, T);
  }

  // First bin b whose inclusive prefix satisfies pred; kNB if none.
  template <typename Pred>
  __device__ int first_bin(Pred pred) {
    if (threadIdx.x == 0) L.bi[0] = kNB;
    lds_barrier();
    constexpr int PER = kNB / NT;
    // bins threadIdx.x * PER .. : a wave covers a contiguous bin range, so the
    // first qualifying lane of the first qualifying wave holds the answer
    int mine = kNB;
#pragma unroll
    for (int k = PER - 1; k >= 0; --k) {
      const int b = threadIdx.x * PER + k;
      if (L.u.post.cnt[b + 1] > L.u.post.cnt[b] && pred(b)) mine = b;
    }
    const uint64_t bal = __ballot(mine < kNB);
    if (bal && lane_id() == __builtin_ctzll(bal)) atomicMin(&L.bi[0], mine);
    lds_barrier();
    const int b = L.bi[0];
    lds_barrier();
    return b;
  }

  // Gather bin b's elements sorted by (x desc, idx asc) into gs; float32 also
  // prefixes their weights into gpm. Returns the count (or -1 if too many).
  __device__ int gather(int b) {
    if (threadIdx.x == 0) L.gn = 0;
    lds_barrier();
    const int n = L.ncand;
    for (int j = threadIdx.x; j < n; j += NT) {
      const Cand e = L.c.cand[j];
      if (!in_bins(e.x) || bin_of(e.x) != b) continue;
      const int pos = atomicAdd(&L.gn, 1);
      if (pos < kGather) L.u.post.g[pos] = e;
    }
    lds_barrier();
    const int cb = L.gn;
    lds_barrier();
    if (cb > kGather) return -1;
    for (int q = threadIdx.x; q < cb; q += NT) {
      const Cand e = L.u.post.g[q];
      int r = 0;
      for (int o = 0; o < cb; ++o) {
        const Cand d = L.u.post.g[o];
        r += (d.x > e.x || (d.x == e.x && d.idx < e.idx)) ? 1 : 0;
      }
      L.u.post.gs[r] = e;
    }
    lds_barrier();
    if (!kCode) {
      double wv = 0.0;
      if (static_cast<int>(threadIdx.x) < cb) wv = weight(L.u.post.gs[threadIdx.x].x, m, T);
      double tot;
      const double incl = block_scan_incl<NT, double>(wv, L.red_d, tot);
      if (static_cast<int>(threadIdx.x) < cb) L.u.post.gpm[threadIdx.x] = incl;
      lds_barrier();
    }
    return cb;
  }

  // Cumulative weight through position j of bin b (after gather for float32).
  __device__ double cum_at(int b, int j) const {
    return kCode ? L.u.post.mass[b] + static_cast<double>(j + 1) * L.u.post.wbin[b]
                 : L.u.post.mass[b] + L.u.post.gpm[j];
  }

  // Token at 0-based rank k - 1.
  __device__ Pick by_count(int k) {
    Pick p{0, k - 1, 0.0, false, 0, 0};
    const int r = k - 1;
    if (r < 0 || r >= nc) return p;
    const int b = first_bin([&](int bb) { return L.u.post.cnt[bb + 1] > r; });
    if (b >= kNB) return p;
    const int j = r - L.u.post.cnt[b];
    if (!kCode) {
      const int cb = gather(b);
      if (cb < 0 || j >= cb) {
        bad = bad || cb < 0;
        return p;
      }
      p.idx = L.u.post.gs[j].idx;
    }
    p.bin = b;
    p.off = j;
    p.cum = cum_at(b, j);
    p.ok = true;
    lds_barrier();
    return p;
  }

  // First rank whose cumulative weight reaches (>=, or > when strict) target.
  __device__ Pick by_mass(double target, bool strict) {
    Pick p{0, 0, 0.0, false, 0, 0};
    const int b = first_bin([&](int bb) {
      const double hi = L.u.post.mass[bb + 1];
      return strict ? (hi > target) : (hi >= target);
    });
    if (b >= kNB) return p;
    const int cb = kCode ? (L.u.post.cnt[b + 1] - L.u.post.cnt[b]) : gather(b);
    if (cb <= 0) {
      bad = bad || cb < 0;
      return p;
    }
    const double base = L.u.post.mass[b];
    int j = cb - 1;
    if (kCode) {
      const double wb = L.u.post.wbin[b];
      if (wb > 0.0) {
        const double q = (target - base) / wb;
        j = strict ? static_cast<int>(floor(q)) : static_cast<int>(ceil(q)) - 1;
        j = j < 0 ? 0 : (j > cb - 1 ? cb - 1 : j);
        // settle rounding against the exact comparison used for the prefix
        while (j > 0 && (strict ? cum_at(b, j - 1) > target : cum_at(b, j - 1) >= target)) --j;
        while (j < cb - 1 && !(strict ? cum_at(b, j) > target : cum_at(b, j) >= target)) ++j;
      }
    } else {
      for (int q = 0; q < cb; ++q) {
        const double cq = base + L.u.post.gpm[q];
        if (strict ? (cq > target) : (cq >= target)) {
          j = q;
          break;
        }
      }
      p.idx = L.u.post.gs[j].idx;
    }
    p.bin = b;
    p.off = j;
    p.rank = L.u.post.cnt[b] + j;
    p.cum = cum_at(b, j);
    p.ok = true;
    lds_barrier();
    return p;
  }

  // Candidates with (x - m) / T >= lnmp; exact unless every candidate passes.
  __device__ int count_minp(double lnmp, bool& exact) {
    int cnt = 0;
    const int n = L.ncand;
    for (int j = threadIdx.x; j < n; j += NT) {
      const float x = L.c.cand[j].x;
      if (in_bins(x) && (static_cast<double>(x) - static_cast<double>(m)) / T >= lnmp) ++cnt;
    }
    cnt = block_reduce<NT>(cnt, SumOp(), L.red_i);
    exact = cnt < nc;
    return cnt;
  }

  // The token of a pick (bf16: the off-th smallest index of the bin's value).
  __device__ int token(const Pick& p) {
    if (!kCode) return p.idx;
    const int cb = gather(p.bin);
    if (cb < 0 || p.off >= cb) {
      bad = true;
      return 0;
    }
    const int t = L.u.post.gs[p.off].idx;
    lds_barrier();
    return t;
  }
};

// Every element of a row, in 16-byte loads (its 16-byte-aligned body) and
// single loads (the elements before and after it): f(x, index) runs once
// per element, on some thread, in no particular order. Loads go out
// kRowEachB at a time per thread (the whole-row passes below are paced by
// their arithmetic, not by their loads).
constexpr int kRowEachB = 2;
template <typename E, int NT, typename F>
__device__ __forceinline__ void row_each(const E* __restrict__ row, int V, F f) {
  constexpr int N = Elem<E>::kVec;
  const uintptr_t addr = reinterpret_cast<uintptr_t>(row);
  int head = static_cast<int>(((16u - (addr & 15u)) & 15u) / sizeof(E));
  if (head > V) head = V;
  const int nvec = (V - head) / N;
  const int body_end = head + nvec * N;
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<E*>(row + head), 0, nvec * 16, 0x00020000);
  for (int v0 = threadIdx.x; v0 < nvec; v0 += NT * kRowEachB) {
    u32x4 w[kRowEachB];
#pragma unroll
    for (int b = 0; b < kRowEachB; ++b) {
      const int q = v0 + b * NT;
      w[b] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, q < nvec ? static_cast<uint32_t>(q) * 16u : 0xFFFFFFF0u, 0, 0);
    }
#pragma unroll
    for (int b = 0; b < kRowEachB; ++b) {
      const int q = v0 + b * NT;
      if (q < nvec) {
        float x[N];
        Elem<E>::decode(w[b], x);
#pragma unroll
        for (int k = 0; k < N; ++k) f(x[k], head + q * N + k);
      }
    }
  }
  const int t = static_cast<int>(threadIdx.x);
  if (t < head) f(Elem<E>::at(row, t), t);
  if (body_end + t < V) f(Elem<E>::at(row, body_end + t), body_end + t);
}

// Float64 2^a by Tang's table-driven method (ACM TOMS 15(2), 1989):
// a = n + j / 64 + r with integer n, 0 <= j < 64 and 0 <= r < 1/64, so
// 2^a = 2^n * 2^(j/64) * 2^r, with 2^(j/64) from a 64-entry table and 2^r
// from the Taylor series of e^(r ln 2) to degree 6 (the first omitted term
// is under 4e-18 relative). Arguments below -1100 give 0.
struct Exp2Table {
  static constexpr double kL = 0.69314718055994530942;   // ln 2
  static constexpr double k1 = kL, k2 = k1 * kL / 2, k3 = k2 * kL / 3, k4 = k3 * kL / 4, k5 = k4 * kL / 5,
                          k6 = k5 * kL / 6;
  double* t;
  // every thread calls it; the caller's barrier publishes the table
  __device__ void fill() const {
    if (threadIdx.x < 64) t[threadIdx.x] = exp2(static_cast<double>(threadIdx.x) / 64.0);
  }
  __device__ double operator()(double a) const {
    a = a > -1100.0 ? a : -1100.0;
    const double s = floor(a * 64.0);
    const int n = static_cast<int>(s);
    const double r = a - s * (1.0 / 64.0);
    const double p = 1.0 + r * (k1 + r * (k2 + r * (k3 + r * (k4 + r * (k5 + r * k6)))));
    return ldexp(t[n & 63] * p, n >> 6);
  }
};

// Exact locator over the whole row: a search of the rank order (value
// desc, index asc) by count or by float64 mass, on the elements'
// order-preserving keys. A level bins a key range (lo, hi] by (hi - k) >> s
// into kNB bins, the last one taking everything further below. Level 0
// starts at the row maximum's key with s = 16 (one bfloat16 value per bin)
// and its counts and weights serve every query of the row. A query finds
// the bin that holds its answer: a bin of at most kGatherFull elements is
// gathered and ranked in LDS, a bin of one value resolves its ties in index
// order, and any other bin is binned again, 2^10 times finer (the last bin:
// the next kNB - 1 steps below). Each level reads the row once; most
// elements of a row land in the last bin, so each lane sums that bin's
// share itself and adds it once. Bins weigh their elements with the
// table-driven float64 exponential below (a few units in the last place of
// exp((x - m) / T)); ranked bins and ties use exp itself.
template <typename E, int NT>
struct FullLocator {
  static constexpr int NW = NT / kWave;
  static constexpr int kS0 = 16;
  // finer levels' counts and weights live in the candidate area
  static constexpr size_t kFineMass = ((kNB + 1) * sizeof(int) + 7) / 8 * 8;
  static constexpr size_t kTable = kFineMass + (kNB + 1) * sizeof(double);
  static_assert(sizeof(Cand) * kCand >= kTable + 64 * sizeof(double),
                "finer levels and the table fit the candidate area");
  SampledLds<NT>& L;
  const E* __restrict__ row;
  int V;
  float m;
  double T;
  double wtot;
  uint32_t kmax;
  uint32_t kmin0;   // lowest key of the row
  bool built;

  struct Level {
    uint32_t hi, lo;  // keys in (lo, hi]; no lower bound unless has_lo
    bool has_lo;
    int s;
    int base_c;       // elements ranked above the range
    double base_m;    // and their weight
  };

  __device__ __forceinline__ FullLocator(SampledLds<NT>& l, const E* r, int V_, float m_, double T_)
      : L(l), row(r), V(V_), m(m_), T(T_), wtot(0.0), kmax(ord_ukey(m_)), kmin0(0u), built(false) {}

  __device__ __forceinline__ float at(int e) const { return Elem<E>::at(row, e); }
  __device__ __forceinline__ int* cnt(bool fine) { return fine ? reinterpret_cast<int*>(&L.c) : L.u.post.cnt; }
  __device__ __forceinline__ double* mass(bool fine) {
    return fine ? reinterpret_cast<double*>(reinterpret_cast<char*>(&L.c) + kFineMass) : L.u.post.mass;
  }
  __device__ __forceinline__ static bool in_range(const Level& lv, uint32_t k) {
    return k <= lv.hi && (!lv.has_lo || k > lv.lo);
  }

  // Counts and weights of the level's bins, as exclusive prefixes (totals
  // at index kNB); returns the range's lowest key.
  __device__ __forceinline__ uint32_t histogram(const Level& lv, bool fine) {
    int* c = cnt(fine);
    double* ms = mass(fine);
    for (int b = threadIdx.x; b <= kNB; b += NT) {
      c[b] = 0;
      ms[b] = 0.0;
    }
    if (threadIdx.x == 0) L.bi[2] = -1;   // as unsigned: the largest key
    lds_barrier();
    const Exp2Table ex{reinterpret_cast<double*>(reinterpret_cast<char*>(&L.c) + kTable)};
    ex.fill();
    lds_barrier();
    int oc = 0;
    double om = 0.0;
    uint32_t lowest = 0xFFFFFFFFu;
    const double c2 = 1.4426950408889634074 / T;
    row_each<E, NT>(row, V, [&](float x, int) {
      const uint32_t k = ord_ukey(x);
      if (!in_range(lv, k)) return;
      lowest = k < lowest ? k : lowest;
      const uint32_t d = (lv.hi - k) >> lv.s;
      const double w = ex((static_cast<double>(x) - static_cast<double>(m)) * c2);
      if (d < static_cast<uint32_t>(kNB - 1)) {
        atomicAdd(&c[d], 1);
        atomicAdd(&ms[d], w);
      } else {
        ++oc;
        om += w;
      }
    });
    oc = wave_all(oc, SumOp());
    om = wave_sum_f64(om);
    lowest = wave_all(lowest, MinOp());
    if (lane_id() == 0) {
      if (oc) {
        atomicAdd(&c[kNB - 1], oc);
        atomicAdd(&ms[kNB - 1], om);
      }
      atomicMin(reinterpret_cast<unsigned int*>(&L.bi[2]), lowest);
    }
    lds_barrier();
    const uint32_t kmin = static_cast<uint32_t>(L.bi[2]);
    constexpr int PER = kNB / NT;
    int lc[PER];
    double lm[PER];
    int sc = 0;
    double sm = 0.0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int b = threadIdx.x * PER + k;
      lc[k] = c[b];
      lm[k] = ms[b];
      sc += lc[k];
      sm += lm[k];
    }
    int tc, ic = sc;
    double tm, im = sm;
    block_scan_incl2<NT>(ic, im, L.red_i, L.red_d, tc, tm);
    int ec = ic - sc;
    double em = im - sm;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int b = threadIdx.x * PER + k;
      c[b] = ec;
      ms[b] = em;
      ec += lc[k];
      em += lm[k];
    }
    if (threadIdx.x == 0) {
      c[kNB] = tc;
      ms[kNB] = tm;
    }
    lds_barrier();
    return kmin;
  }

  __device__ __forceinline__ void build() {
    if (built) return;
    kmin0 = histogram(Level{kmax, 0u, false, kS0, 0, 0.0}, false);
    wtot = L.u.post.mass[kNB];
    built = true;
  }

  __device__ __forceinline__ double total_mass() {
    build();
    return wtot;
  }

  // The whole row is held: nothing lies beyond it.
  __device__ __forceinline__ double beyond_weight() const { return 0.0; }

  // Does rank position r, with cumulative weight cw through it, reach the
  // query?
  __device__ __forceinline__ static bool reached(bool by_weight, double target, int rank, bool strict, int r,
                                                 double cw) {
    return by_weight ? (strict ? cw > target : cw >= target) : r >= rank;
  }

  // First non-empty bin of the level whose inclusive prefix reaches the
  // query; kNB if none.
  __device__ __forceinline__ int first_bin(const Level& lv, bool fine, bool by_weight, double target, int rank,
                                           bool strict) {
    const int* c = cnt(fine);
    const double* ms = mass(fine);
    if (threadIdx.x == 0) L.bi[0] = kNB;
    lds_barrier();
    constexpr int PER = kNB / NT;
    int mine = kNB;
#pragma unroll
    for (int k = PER - 1; k >= 0; --k) {
      const int b = threadIdx.x * PER + k;
      if (c[b + 1] > c[b] &&
          reached(by_weight, target, rank, strict, lv.base_c + c[b + 1] - 1, lv.base_m + ms[b + 1]))
        mine = b;
    }
    const uint64_t bal = __ballot(mine < kNB);
    if (bal && lane_id() == __builtin_ctzll(bal)) atomicMin(&L.bi[0], mine);
    lds_barrier();
    const int b = L.bi[0];
    lds_barrier();
    return b;
  }

  // The bin's elements ranked in LDS (nb <= kGatherFull): the answer's position
  // among them, with their exact weights.
  __device__ __forceinline__ Pick gather_pick(const Level& bl, int nb, bool by_weight, double target, int rank,
                                              bool strict) {
    if (threadIdx.x == 0) L.gn = 0;
    lds_barrier();
    row_each<E, NT>(row, V, [&](float x, int e) {
      if (!in_range(bl, ord_ukey(x))) return;
      const int pos = atomicAdd(&L.gn, 1);
      if (pos < kGatherFull) L.u.post.g[pos] = Cand{x, e};
    });
    lds_barrier();
    const int cb = min(L.gn, kGatherFull);
    lds_barrier();
    for (int q = threadIdx.x; q < cb; q += NT) {
      const Cand e = L.u.post.g[q];
      int r = 0;
      for (int o = 0; o < cb; ++o) {
        const Cand d = L.u.post.g[o];
        r += (d.x > e.x || (d.x == e.x && d.idx < e.idx)) ? 1 : 0;
      }
      L.u.post.gs[r] = e;
    }
    lds_barrier();
    double wv = 0.0;
    if (static_cast<int>(threadIdx.x) < cb) wv = weight(L.u.post.gs[threadIdx.x].x, m, T);
    double tot;
    const double incl = block_scan_incl<NT, double>(wv, L.red_d, tot);
    // the first position that reaches the query (the last one if none does)
    if (threadIdx.x == 0) L.bi[1] = cb - 1;
    lds_barrier();
    const int j = static_cast<int>(threadIdx.x);
    wave_first_min(&L.bi[1], j, j < cb && reached(by_weight, target, rank, strict, bl.base_c + j, bl.base_m + incl));
    if (j < cb) L.u.post.gpm[j] = incl;
    lds_barrier();
    const int jj = max(L.bi[1], 0);
    Pick p{0, bl.base_c + jj, 0.0, cb > 0 && cb == nb, 0, 0};
    if (cb > 0) {
      p.idx = L.u.post.gs[jj].idx;
      p.cum = bl.base_m + L.u.post.gpm[jj];
    }
    lds_barrier();
    return p;
  }

  // A bin whose nb elements all hold one value: the answer's position
  // among the ties, then that tie in index order (each wave counts the
  // ties of its contiguous share of the row; the share holding the answer
  // is read again).
  __device__ __forceinline__ Pick tie_pick(const Level& bl, int nb, bool by_weight, double target, int rank,
                                           bool strict) {
    const int w = wave_id(), lane = lane_id();
    const int seg = (V + NW - 1) / NW;
    const int e0 = min(V, w * seg), e1 = min(V, e0 + seg);
    int mine = 0;
    float val = 0.f;
    bool have = false;
    for (int base = e0; base < e1; base += kWave) {
      const int e = base + lane;
      const float x = e < e1 ? at(e) : 0.f;
      const bool hit = e < e1 && in_range(bl, ord_ukey(x));
      const uint64_t bal = __ballot(hit);
      if (bal && !have) {
        val = __shfl(x, __builtin_ctzll(bal));
        have = true;
      }
      mine += __popcll(bal);
    }
    if (lane == 0) {
      L.red_i[w] = mine;
      if (have) L.bd[1] = static_cast<double>(val);   // any tie's value
    }
    lds_barrier();
    const double tw = weight(static_cast<float>(L.bd[1]), m, T);
    int j;
    if (by_weight) {
      j = 0;
      if (tw > 0.0) {
        const double q = (target - bl.base_m) / tw;
        j = strict ? static_cast<int>(floor(q)) : static_cast<int>(ceil(q)) - 1;
        j = j < 0 ? 0 : (j >= nb ? nb - 1 : j);
        // settle rounding against the exact comparison
        while (j > 0 && reached(true, target, 0, strict, 0, bl.base_m + j * tw)) --j;
        while (j < nb - 1 && !reached(true, target, 0, strict, 0, bl.base_m + (j + 1) * tw)) ++j;
      }
    } else {
      j = rank - bl.base_c;
    }
    j = j < 0 ? 0 : (j >= nb ? nb - 1 : j);
    // the share holding tie j, and the tie's place in it
    int before = 0, ws = -1;
    for (int k = 0; k < NW; ++k) {
      const int ck = L.red_i[k];
      if (ws < 0 && j < before + ck) ws = k;
      if (ws < 0) before += ck;
    }
    if (threadIdx.x == 0) L.bi[3] = 0;
    lds_barrier();
    if (w == ws) {
      int need = j - before;
      for (int base = e0; base < e1; base += kWave) {
        const int e = base + lane;
        const bool hit = e < e1 && in_range(bl, ord_ukey(at(e)));
        const uint64_t bal = __ballot(hit);
        const int n = __popcll(bal);
        if (need < n) {
          // the (need + 1)-th set bit of bal
          uint64_t bb = bal;
          for (int k = 0; k < need; ++k) bb &= bb - 1;
          if (lane == 0) L.bi[3] = base + __builtin_ctzll(bb);
          break;
        }
        need -= n;
      }
    }
    lds_barrier();
    Pick p{L.bi[3], bl.base_c + j, bl.base_m + static_cast<double>(j + 1) * tw, ws >= 0, 0, 0};
    lds_barrier();
    return p;
  }

  // The rank reached by the query: by weight, the first rank whose
  // cumulative weight passes `target` (strictly if `strict`); else rank
  // `rank`. A weight query beyond the row answers with the row's last rank.
  __device__ __forceinline__ Pick locate(bool by_weight, double target, int rank, bool strict) {
    build();
    Level lv{kmax, 0u, false, kS0, 0, 0.0};
    bool fine = false;
    uint32_t kmin = kmin0;   // the level's lowest key
    for (int depth = 0; depth < 12; ++depth) {
      int b = first_bin(lv, fine, by_weight, target, rank, strict);
      if (b >= kNB) {
        if (!by_weight || depth > 0) break;
        by_weight = false;   // past the total: the row's last rank
        rank = V - 1;
        b = first_bin(lv, fine, false, 0.0, rank, false);
        if (b >= kNB) break;
      }
      const int* c = cnt(fine);
      const double* ms = mass(fine);
      const int nb = c[b + 1] - c[b];
      Level bl;
      bl.hi = lv.hi - (static_cast<uint32_t>(b) << lv.s);
      if (b < kNB - 1) {
        const int64_t lo = static_cast<int64_t>(lv.hi) - (static_cast<int64_t>(b + 1) << lv.s);
        bl.has_lo = lo >= 0;
        bl.lo = bl.has_lo ? static_cast<uint32_t>(lo) : 0u;
      } else {
        bl.lo = lv.lo;
        bl.has_lo = lv.has_lo;
      }
      bl.base_c = lv.base_c + c[b];
      bl.base_m = lv.base_m + ms[b];
      // one value per bin: a key step (s = 0), or a bfloat16 row's level-0
      // step (2^16 keys from a bfloat16 key hold one bfloat16 key)
      const bool one_value = b < kNB - 1 && (lv.s == 0 || (sizeof(E) == 2 && lv.s == kS0));
      lds_barrier();
      if (nb <= kGatherFull) return gather_pick(bl, nb, by_weight, target, rank, strict);
      if (one_value) return tie_pick(bl, nb, by_weight, target, rank, strict);
      if (b < kNB - 1) {
        bl.s = lv.s >= 10 ? lv.s - 10 : 0;
      } else {
        // the rest of the range, down to its lowest key: steps that cover
        // it in kNB bins
        bl.has_lo = kmin > 0u;
        bl.lo = bl.has_lo ? kmin - 1u : 0u;
        const uint32_t span = bl.hi - kmin;
        int sw = 0;
        while (sw < 31 && (span >> sw) >= static_cast<uint32_t>(kNB)) ++sw;
        bl.s = sw;
      }
      lv = bl;
      fine = true;
      kmin = histogram(lv, true);
    }
    return Pick{0, 0, 0.0, false, 0, 0};
  }

  __device__ __forceinline__ Pick by_count(int k) {
    if (k < 1 || k > V) return Pick{0, k - 1, 0.0, false, 0, 0};
    return locate(false, 0.0, k - 1, false);
  }

  __device__ __forceinline__ Pick by_mass(double target, bool strict) { return locate(true, target, 0, strict); }

  __device__ __forceinline__ int token(const Pick& p) const { return p.idx; }

  __device__ __forceinline__ int count_minp(double lnmp, bool& exact) {
    int c = 0;
    for (int e = threadIdx.x; e < V; e += NT)
      c += ((static_cast<double>(at(e)) - static_cast<double>(m)) / T >= lnmp) ? 1 : 0;
    exact = true;
    return block_reduce<NT>(c, SumOp(), L.red_i);
  }
};

// The filtered draw, given a locator. Returns false if the locator cannot
// decide.
template <class Loc>
__device__ __forceinline__ bool decide(Loc& loc, int V, int top_k, double top_p, double min_p, double u, int& token) {
  const bool tk = top_k > 0 && top_k < V;
  const bool tp = top_p < 1.0;
  const bool mp = min_p > 0.0;
  int L1;
  double W1;
  if (tk) {
    const Pick p = loc.by_count(top_k);
    if (!p.ok) return false;
    L1 = top_k;
    W1 = p.cum;
  } else {
    L1 = V;
    W1 = loc.total_mass();
  }
  int Ls = L1;
  double Ws = W1;
  if (tp) {
    const Pick p = loc.by_mass(top_p * W1, false);
    if (!p.ok) {
      // The cut lies beyond what the locator holds (a candidate locator's
      // prefix of the rank order): every element it holds survives, and
      // the survivors weigh top_p * W1 plus less than the weight of one
      // element below it. A draw that reaches the same held element for
      // every such weight is decided; any other is left to the caller.
      if (tk || mp) return false;
      const double lo = top_p * W1, hi = lo + loc.beyond_weight();
      const Pick a = loc.by_mass(u * lo, true);
      if (!a.ok) return false;
      const Pick b = loc.by_mass(u * hi, true);
      if (!b.ok || b.rank != a.rank) return false;
      token = loc.token(a);
      return true;
    }
    Ls = p.rank + 1;
    Ws = p.cum;
  }
  if (mp) {
    bool exact = false;
    const int lm = loc.count_minp(log(min_p), exact);
    if (!exact && Ls > lm) return false;
    if (exact && lm < Ls) {
      Ls = lm > 0 ? lm : 1;
      const Pick p = loc.by_count(Ls);
      if (!p.ok) return false;
      Ws = p.cum;
    }
  }
  Pick s = loc.by_mass(u * Ws, true);
  if (!s.ok) return false;
  if (s.rank >= Ls) {
    s = loc.by_count(Ls);
    if (!s.ok) return false;
  }
  token = loc.token(s);
  return true;
}

}  // namespace vsv

namespace vsv {

// ---------------------------------------------------------------- capture

// Order-preserving 16-bit code of x rounded up to bfloat16: an upper bound
// of x in code order (exact for bfloat16 values; -0 counts as +0).
__device__ __forceinline__ int up_code(float x) {
  const uint32_t u = __float_as_uint(x == 0.0f ? 0.0f : x);
  uint32_t h = u >> 16;
  // a positive value with bits below bfloat16 rounds its magnitude up; a
  // negative one truncates toward zero, which is up as well
  if ((u & 0xFFFFu) && !(u & 0x80000000u)) h += 1;
  return (h & 0x8000u) ? static_cast<int>(~h & 0xFFFFu) : static_cast<int>(h | 0x8000u);
}

// Entries of the vector-maximum codes: entry (r, t) = l1[r * NT + t] covers
// the vectors of thread t's slot steps r * S .. r * S + S - 1 (vector
// k * NT + t for step k). S = 1 while a row has at most kVM vectors. Block
// (b, t) = l2[b * NT + t] is the largest code of entries (8b .. 8b + 7, t).
struct VmPlan {
  int S;       // slot steps per entry
  int rows;    // entry rows written (entries = rows * NT)
  int blocks;  // blocks of eight entry rows (blocks * NT of them)
};

// The code of a vector maximum: for bfloat16 rows the maximum is a bfloat16
// value, so its code is exact and needs no rounding (-0 is first made +0);
// float32 maxima are rounded up (up_code).
template <typename E>
__device__ __forceinline__ int vmax_code(float v) {
  if constexpr (sizeof(E) == 2) {
    const uint32_t b = __float_as_uint(v + 0.0f);
    const uint32_t flip = (static_cast<uint32_t>(static_cast<int32_t>(b) >> 31) & 0x7FFFu) | 0x8000u;
    return static_cast<int>((b >> 16) ^ flip);
  } else {
    return up_code(v);
  }
}

template <bool B> struct BoolC { static constexpr bool value = B; };

// Pass 1: stream one sampled row for the statistics of stream_row, and leave
// the code of every vector's maximum in L.u.vm. bf16 rows load with the
// caches' normal policy, so that pass 2's reads of a few vectors find them
// there; fp32 rows stream past the caches like greedy rows (timed on the
// large mixed bf16 batch, streaming loads made the launch 285 -> 306 us; on
// the ragged fp32 batch they took it from 92.8 to 90.4 us).
template <typename E, int NT, int U>
__device__ __forceinline__ VmPlan stream_sampled(const E* __restrict__ row, int V, float c, RowPartial& p,
                                                 SampledLds<NT>& L) {
  constexpr int N = Elem<E>::kVec;
  constexpr int kRowsVM = kVM / NT;
  const int tid = threadIdx.x;
  const uintptr_t addr = reinterpret_cast<uintptr_t>(row);
  int head = static_cast<int>(((16u - (addr & 15u)) & 15u) / sizeof(E));
  if (head > V) head = V;
  const int nvec = (V - head) / N;
  const int body_end = head + nvec * N;
  // Body vectors through a buffer resource: the lane's byte offset is fixed
  // and a step's is uniform (a scalar offset), so loads cost no vector
  // address arithmetic; vectors past the body read as zero.
  const __amdgpu_buffer_rsrc_t rsrc = vec_rsrc(row + head, nvec);
  const int lane_off = tid * 16;
  auto load = [&](int first) {   // vector first + tid
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, lane_off, first * 16,
                                                                           sizeof(E) == 4 ? kLoadStream : kLoadNormal));
  };
  // Rolling slots: slot u holds vector g*G + u*NT + tid of group g; it is
  // decoded, then reloaded at once with the same vector of group g+1, so
  // U-1 vectors per lane are always in flight and the loop carries no
  // register copies (a copy at the latch would wait for every load).
  constexpr int G = U * NT;
  const int nfull = nvec / G;
  const int steps = nvec > 0 ? (nvec > nfull * G ? nfull + 1 : nfull) * U : 0;
  VmPlan plan{max(1, (steps + kRowsVM - 1) / kRowsVM), 0, 0};

  const bool has_head = tid < head;
  const float xh = has_head ? Elem<E>::at(row, tid) : -INFINITY;
  u32x4 slot[U];
  if (nvec > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) slot[u] = load(u * NT);
  }
  if (has_head) take_scalar<false>(p, xh, tid, c, INFINITY, 0);

  int bmax = 0;   // the largest code of the current block
  auto push = [&](int code) {
    L.u.vm.l1[plan.rows * NT + tid] = static_cast<uint16_t>(code);
    bmax = max(bmax, code);
    if ((++plan.rows & 7) == 0) {
      L.u.vm.l2[plan.blocks * NT + tid] = static_cast<uint16_t>(bmax);
      ++plan.blocks;
      bmax = 0;
    }
  };
  // kOne: one entry per vector (S = 1), its code straight from the vector's
  // maximum; otherwise the running maximum of S slot steps (uniform
  // countdown) makes one entry
  auto body = [&](auto one) {
    constexpr bool kOne = decltype(one)::value;
    float run = -INFINITY;
    int left = plan.S;
    auto note = [&](float vmax) {
      if constexpr (kOne) {
        push(vmax_code<E>(vmax));
      } else {
        run = fmaxf(run, vmax);
        if (--left == 0) {
          push(up_code(run));
          run = -INFINITY;
          left = plan.S;
        }
      }
    };
    for (int g = 0; g < nfull; ++g) {
      if constexpr (sizeof(E) == 2) {
        // a bfloat16 group's U vectors: maxima by IEEE maximum (a NaN
        // propagates and is remembered), exponentials summed in float, one
        // float64 add (float32 rows, with deeper slots, keep the per-vector
        // form: the group form spills there)
        float gmax = -INFINITY, gs = 0.f;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float f[N];
          const float vmax = vec_max<E, true>(slot[u], f);
          slot[u] = load((g + 1) * G + u * NT);
          take_floats_group<N>(p, f, vmax, c, gs);
          note(vmax);
          gmax = __builtin_elementwise_maximum(gmax, vmax);
        }
        p.s += static_cast<double>(gs);
        p.best = __builtin_elementwise_maximum(p.best, gmax);
        p.bad |= (gmax != gmax) ? 1 : 0;
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float f[N];
          const float vmax = vec_max<E>(slot[u], f);
          slot[u] = load((g + 1) * G + u * NT);
          take_floats<N>(p, f, vmax, c);
          note(vmax);
        }
      }
    }
    if (nvec > nfull * G) {
      // the slots hold group nfull, the partial last one
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int q = nfull * G + tid + u * NT;
        float f[N];
        float vmax = -INFINITY;
        if (q < nvec) {
          vmax = vec_max<E>(slot[u], f);
          take_floats<N>(p, f, vmax, c);
        }
        note(vmax);
      }
    }
    if constexpr (!kOne) {
      if (left != plan.S) push(up_code(run));
    }
  };
  if (nvec > 0) {
    if (plan.S == 1)
      body(BoolC<true>{});
    else
      body(BoolC<false>{});
    if (plan.rows & 7) {
      L.u.vm.l2[plan.blocks * NT + tid] = static_cast<uint16_t>(bmax);
      ++plan.blocks;
    }
  }
  const int tail = V - body_end;
  if (tid < tail) take_scalar<false>(p, Elem<E>::at(row, body_end + tid), body_end + tid, c, INFINITY, 0);
  return plan;
}

// Counts of vector-maximum codes >= each of the codes ct[0 .. C-1], over the
// row's entries (every thread reads eight codes at a time).
template <int NT, int C>
__device__ __forceinline__ void count_codes(SampledLds<NT>& L, const VmPlan& plan, const int* ct, int* out) {
  constexpr int NW = NT / kWave;
  const int ne = plan.rows * NT;   // a multiple of 8: NT is
  int n[C];
#pragma unroll
  for (int i = 0; i < C; ++i) n[i] = 0;
  for (int g = threadIdx.x; g * 8 < ne; g += NT) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(&L.u.vm.l1[g * 8]);
    const uint32_t h[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int code = static_cast<int>((h[q / 2] >> (16 * (q & 1))) & 0xFFFFu);
#pragma unroll
      for (int i = 0; i < C; ++i) n[i] += code >= ct[i] ? 1 : 0;
    }
  }
#pragma unroll
  for (int i = 0; i < C; ++i) n[i] = wave_all(n[i], SumOp());
  lds_barrier();
  if (lane_id() == 0) {
#pragma unroll
    for (int i = 0; i < C; ++i) L.c.hist[0][wave_id() * C + i] = n[i];
  }
  lds_barrier();
#pragma unroll
  for (int i = 0; i < C; ++i) {
    int t = 0;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) t += L.c.hist[0][ww * C + i];
    out[i] = t;
  }
  lds_barrier();
}

// The k-th largest block code (l2) within kTopBins codes of mc, or -1 when
// fewer than k lie there. k blocks hold an entry code at least that large,
// so it bounds the k-th largest entry code from below.
template <int NT>
__device__ int kth_block_code(SampledLds<NT>& L, const VmPlan& plan, int k, int mc) {
  constexpr int PER = kTopBins / NT;
  const int tid = threadIdx.x;
  int* h = L.c.hist[0];
#pragma unroll
  for (int q = 0; q < PER; ++q) h[tid * PER + q] = 0;
  if (tid == 0) L.bi[0] = kTopBins;
  lds_barrier();
  for (int g = tid; g < plan.blocks * NT; g += NT) {
    const int d = mc - static_cast<int>(L.u.vm.l2[g]);
    if (d >= 0 && d < kTopBins) atomicAdd(&h[d], 1);
  }
  lds_barrier();
  int cnt[PER];
  int sc = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    cnt[q] = h[tid * PER + q];
    sc += cnt[q];
  }
  int tot;
  const int incl = block_scan_incl<NT, int>(sc, L.red_i, tot);
  int run = incl - sc, found = kTopBins;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    run += cnt[q];
    if (run >= k && found == kTopBins) found = tid * PER + q;
  }
  // Every thread past the k-th code lowers the result itself. One atomic per
  // wave (wave_first_min) finishes top-k rows' selection sooner, but on the
  // ragged fp32 batch (586 rows for 512 workgroups) the greedy rows handed
  // out last then stream beside that faster selection several us slower and
  // end the launch: 87.2 instead of 79.4 us per launch back to back (a
  // 64-request batch gains 1.7 us).
  if (found < kTopBins) atomicMin(&L.bi[0], found);
  lds_barrier();
  const int b = L.bi[0];
  lds_barrier();
  return b < kTopBins ? mc - b : -1;
}

// The k-th largest vector-maximum code among those within `span` of the
// row maximum's, as a value: a lower bound of the row's k-th largest element
// (k vectors have a maximum at least that large; float32 codes are rounded
// up, so the bound steps down one code). `have` codes lie in range (at
// least k). Few of them (at most kGather): they are gathered and ranked;
// otherwise a histogram over the range finds the code.
template <typename E, int NT>
__device__ float kth_code_value(SampledLds<NT>& L, const VmPlan& plan, int k, int mc, int span, int have) {
  constexpr int NW = NT / kWave;
  constexpr int PER = kTopBins / NT;
  const int tid = threadIdx.x, w = wave_id(), lane = lane_id();
  const int ne = plan.rows * NT;
  const int lo = mc - span + 1;
  int code = 0;
  if (have <= kGather) {
    // gather the codes >= lo (indices irrelevant) and rank them
    if (tid == 0) L.gn = 0;
    lds_barrier();
    for (int g = tid; g * 8 < ne; g += NT) {
      const u32x4 cw = *reinterpret_cast<const u32x4*>(&L.u.vm.l1[g * 8]);
      const uint32_t hw[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int c = static_cast<int>((hw[q / 2] >> (16 * (q & 1))) & 0xFFFFu);
        if (c >= lo) {
          const int pos = atomicAdd(&L.gn, 1);
          if (pos < kGather) L.c.hist[0][pos] = c;
        }
      }
    }
    lds_barrier();
    const int n = min(L.gn, kGather);
    if (tid == 0) L.bi[0] = -1;
    lds_barrier();
    if (tid < n) {
      // the code with exactly k - 1 codes above it, or the last of a tie
      // group that straddles rank k - 1
      const int mine = L.c.hist[0][tid];
      int above = 0, equal_before = 0;
      for (int o = 0; o < n; ++o) {
        const int c = L.c.hist[0][o];
        above += c > mine ? 1 : 0;
        equal_before += (c == mine && o < tid) ? 1 : 0;
      }
      if (above + equal_before == k - 1) L.bi[0] = mine;
    }
    lds_barrier();
    code = L.bi[0];
    lds_barrier();
    if (code < 0) return -INFINITY;
  } else {
    int* h = L.c.hist[w];
    for (int b = lane; b < kTopBins; b += kWave) h[b] = 0;
    wave_lds_sync();
    for (int g = tid; g * 8 < ne; g += NT) {
      const u32x4 cw = *reinterpret_cast<const u32x4*>(&L.u.vm.l1[g * 8]);
      const uint32_t hw[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int d = mc - static_cast<int>((hw[q / 2] >> (16 * (q & 1))) & 0xFFFFu);
        if (d >= 0 && d < span) atomicAdd(&h[d], 1);
      }
    }
    lds_barrier();
    int cnt[PER];
    int sc = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      int v = 0;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) v += L.c.hist[ww][tid * PER + q];
      cnt[q] = v;
      sc += v;
    }
    if (tid == 0) L.bi[0] = kTopBins;
    int tot;
    const int incl = block_scan_incl<NT, int>(sc, L.red_i, tot);
    int run = incl - sc, found = kTopBins;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      run += cnt[q];
      if (run >= k && found == kTopBins) found = tid * PER + q;
    }
    wave_first_min(&L.bi[0], found, found < kTopBins);
    lds_barrier();
    const int b = L.bi[0];
    lds_barrier();
    if (b >= kTopBins) return -INFINITY;
    code = mc - b;
  }
  return bf16_of_code(code - (sizeof(E) == 2 ? 0 : 1));
}

// A capture threshold for a top-p cut, from the vector-maximum codes alone:
// a value tau such that the vectors whose maximum reaches tau weigh, by
// their maxima alone, at least `target` (relative to the row maximum's
// weight). Each such vector holds at least its maximum, so the elements
// >= tau weigh at least as much. bfloat16 codes are exact: tau is the
// value of the lowest code needed. float32 codes are rounded up, so an
// entry of code k has its maximum above the value of code k - 1: that
// value weighs the entry and serves as tau (the capture then also takes
// the entries of code k - 1). Weights use the stream's float scale c.
// Returns -INFINITY when the codes within kSpan of the maximum's fall
// short; `count` receives the entries the capture at tau reads.
template <typename E, int NT>
__device__ float mass_code_threshold(SampledLds<NT>& L, const VmPlan& plan, float m, float c, double target,
                                     int& count) {
  constexpr int NW = NT / kWave;
  constexpr int PER = kTopBins / NT;
  constexpr int kDown = sizeof(E) == 2 ? 0 : 1;
  const int tid = threadIdx.x, w = wave_id(), lane = lane_id();
  const int ne = plan.rows * NT;
  const int mc = up_code(m);
  // codes within kSpan of the maximum's (two binades): few entries reach
  // them, so their LDS counts stay cheap; rows whose top-p mass lies further
  // down take the window's threshold (kSpan = 1024 made the large mixed
  // batch 3.4 us slower)
  constexpr int kSpan = 256;
  int* h = L.c.hist[w];
  for (int b = lane; b < kSpan; b += kWave) h[b] = 0;
  wave_lds_sync();
  for (int g = tid; g * 8 < ne; g += NT) {
    const u32x4 cw = *reinterpret_cast<const u32x4*>(&L.u.vm.l1[g * 8]);
    const uint32_t hw[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int d = mc - static_cast<int>((hw[q / 2] >> (16 * (q & 1))) & 0xFFFFu);
      if (d >= 0 && d < kSpan) atomicAdd(&h[d], 1);
    }
  }
  lds_barrier();
  int cnt[PER];
  double wb[PER];
  int sc = 0;
  double sw = 0.0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int b = tid * PER + q;
    int v = 0;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) v += b < kSpan ? L.c.hist[ww][b] : 0;
    cnt[q] = v;
    wb[q] = v ? v * exp2(static_cast<double>(bf16_of_code(mc - b - kDown) - m) * static_cast<double>(c)) : 0.0;
    sc += v;
    sw += wb[q];
  }
  if (tid == 0) L.bi[0] = kTopBins;
  int tc, ic = sc;
  double tw, iw = sw;
  block_scan_incl2<NT>(ic, iw, L.red_i, L.red_d, tc, tw);
  int rc = ic - sc;
  double rw = iw - sw;
  int found = kTopBins;
  int incl[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    rc += cnt[q];
    rw += wb[q];
    incl[q] = rc;
    if (rw >= target && found == kTopBins) found = tid * PER + q;
  }
  wave_first_min(&L.bi[0], found, found < kTopBins);
  lds_barrier();
  const int b = L.bi[0];
  // entries the capture reads: codes down to bin b + kDown (below the
  // histogram: unknown, reported as more than any cap)
  const int last = b + kDown;
  if (last >= kTopBins) {
    if (tid == 0) L.bi[1] = INT32_MAX;
  } else {
#pragma unroll
    for (int q = 0; q < PER; ++q)
      if (tid * PER + q == last) L.bi[1] = incl[q];
  }
  lds_barrier();
  count = b < kTopBins ? L.bi[1] : 0;
  lds_barrier();
  return b < kTopBins ? bf16_of_code(mc - b - kDown) : -INFINITY;
}

// The capture threshold: at least `floor_tau`, and high enough that at most
// `cap` vectors (top-k rows: exactly the k-th largest) qualify. Counting
// passes decide whether the floor suffices and, if not, which range of
// codes holds the cut.
template <typename E, int NT>
__device__ float capture_threshold(SampledLds<NT>& L, const VmPlan& plan, float m, float floor_tau, int k, bool topk) {
  const int mc = up_code(m);
  const int spans[3] = {16, 128, kTopBins};
  if (topk && k <= plan.blocks * NT) {
    // the k-th largest block code: a lower bound of the k-th largest entry
    // code, close to it when the top entries lie in distinct blocks
    const int cb = kth_block_code<NT>(L, plan, k, mc);
    if (cb >= 0) return bf16_of_code(cb - (sizeof(E) == 2 ? 0 : 1));
  }
  if (!topk) {
    // the window fits as it is (the usual case): one count decides
    const int c0 = up_code(floor_tau);
    int n0;
    count_codes<NT, 1>(L, plan, &c0, &n0);
    if (n0 <= k) return floor_tau;
  }
  const int ct[3] = {mc - spans[0] + 1, mc - spans[1] + 1, mc - spans[2] + 1};
  int n[3];
  count_codes<NT, 3>(L, plan, ct, n);
  // the narrowest range holding k codes
  int span = -1, have = 0;
  for (int i = 0; i < 3 && span < 0; ++i)
    if (n[i] >= k) {
      span = spans[i];
      have = n[i];
    }
  if (span < 0) return topk ? -INFINITY : floor_tau;
  const float t = kth_code_value<E, NT>(L, plan, k, mc, span, have);
  return fmaxf(t, floor_tau);
}

// Pass 2: every element >= tau of the row into L.c.cand (L.ncand of them).
// Each wave picks the entries of its share whose code reaches tau's (their
// indices overwrite the front of the share), reads their vectors again in
// batches (every load in a batch issued before any is used) and appends the
// elements >= tau, reserving room with one LDS atomic per step. Returns
// false if the row has more than kCand such elements.
template <typename E, int NT>
__device__ bool capture_row(const E* __restrict__ row, int V, float tau, const VmPlan& plan, SampledLds<NT>& L) {
  constexpr int N = Elem<E>::kVec;
  constexpr int NW = NT / kWave;
  // entries per lane per batch: a bf16 row's picks (about 125 per wave on
  // the large mixed batch) fill two slots per lane, and empty slots still
  // cost their decode (2 took that batch from 260.4 to 257.7 us); fp32
  // entries cover two vectors each and keep 8 (2 made the ragged fp32
  // batch 4.5 us slower)
  constexpr int kB = sizeof(E) == 2 ? 2 : 8;
  const int w = wave_id(), lane = lane_id();
  const uintptr_t addr = reinterpret_cast<uintptr_t>(row);
  int head = static_cast<int>(((16u - (addr & 15u)) & 15u) / sizeof(E));
  if (head > V) head = V;
  const int nvec = (V - head) / N;
  const int body_end = head + nvec * N;
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<E*>(row + head), 0, nvec * 16, 0x00020000);
  if (threadIdx.x == 0) {
    L.ncand = 0;
    L.ovf = 0;
  }
  lds_barrier();
  const int ct = up_code(tau);

  // A: pick the share's entries whose code reaches tau's, eight codes per
  // lane per step (a share is a multiple of 8 entries); their indices
  // overwrite the front of the share (a step writes below what it read)
  const int ne = plan.rows * NT;
  const int per = ((ne + NW - 1) / NW + 7) / 8 * 8;
  const int s0 = w * per, s1 = min(ne, s0 + per);
  int np = 0;
  for (int base = s0; base < s1; base += kWave * 8) {
    const int e8 = base + lane * 8;
    u32x4 cw = {0u, 0u, 0u, 0u};
    if (e8 < s1) cw = *reinterpret_cast<const u32x4*>(&L.u.vm.l1[e8]);
    const uint32_t hw[4] = {cw.x, cw.y, cw.z, cw.w};
    bool any = false;
#pragma unroll
    for (int q = 0; q < 8; ++q) any |= static_cast<int>((hw[q / 2] >> (16 * (q & 1))) & 0xFFFFu) >= ct;
    if (__ballot(any) == 0) continue;   // nothing picked: nothing written
    wave_lds_sync();  // this step's reads come before its writes
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int code = static_cast<int>((hw[q / 2] >> (16 * (q & 1))) & 0xFFFFu);
      const bool pick = e8 < s1 && code >= ct;   // s1 is a multiple of 8
      const uint64_t bal = __ballot(pick);
      if (pick) L.u.vm.l1[s0 + np + mbcnt(bal)] = static_cast<uint16_t>(e8 + q);
      np += __popcll(bal);
    }
    wave_lds_sync();
  }

  // B: their vectors, kB entries per lane at a time; a lane past the list
  // (or a vector past the row) loads through an out-of-range offset, which
  // returns zero without touching memory, and its elements are ignored. A
  // lane counts its elements >= tau, a wave scan places them, and one LDS
  // atomic per batch reserves the wave's room.
  for (int j0 = 0; j0 < np; j0 += kWave * kB) {
    for (int sstep = 0; sstep < plan.S; ++sstep) {
      u32x4 v[kB];
      int vi[kB];
#pragma unroll
      for (int b = 0; b < kB; ++b) {
        const int j = j0 + b * kWave + lane;
        int q = -1;
        if (j < np) {
          const int e = L.u.vm.l1[s0 + j];
          q = ((e / NT) * plan.S + sstep) * NT + (e % NT);
          if (q >= nvec) q = -1;
        }
        vi[b] = q;
        const uint32_t off = q >= 0 ? static_cast<uint32_t>(q) * 16u : 0xFFFFFFF0u;
        v[b] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0);
      }
      int mine = 0;
#pragma unroll
      for (int b = 0; b < kB; ++b) {
        float f[N];
        Elem<E>::decode(v[b], f);
#pragma unroll
        for (int k = 0; k < N; ++k) mine += (vi[b] >= 0 && f[k] >= tau) ? 1 : 0;
      }
      // the write pass decodes again rather than keeping every element live
#pragma unroll
      for (int b = 0; b < kB; ++b) asm volatile("" : "+v"(v[b]));
      const int incl = wave_scan_incl(mine);
      const int total = read_lane(incl, kWave - 1);
      if (total == 0) continue;
      int base = 0;
      if (lane == 0) base = atomicAdd(&L.ncand, total);
      base = __builtin_amdgcn_readfirstlane(base);
      int pos = base + incl - mine;
#pragma unroll
      for (int b = 0; b < kB; ++b) {
        if (vi[b] < 0) continue;
        float f[N];
        Elem<E>::decode(v[b], f);
#pragma unroll
        for (int k = 0; k < N; ++k) {
          if (f[k] >= tau) {
            if (pos < kCand) L.c.cand[pos] = Cand{f[k], head + vi[b] * N + k};
            ++pos;
          }
        }
      }
    }
  }

  // C: elements outside the 16-byte body (wave 0: lanes 0 .. 7 the head,
  // lanes 8 .. 15 the tail)
  if (w == 0) {
    const int te = body_end + (lane - 8);
    const bool hv = lane < head;
    const bool tv = lane >= 8 && lane < 16 && te < V;
    const int e = hv ? lane : te;
    const float x = (hv || tv) ? Elem<E>::at(row, e) : -INFINITY;
    const bool take = (hv || tv) && x >= tau;
    const uint64_t bal = __ballot(take);
    if (bal) {
      int base = 0;
      if (lane == 0) base = atomicAdd(&L.ncand, __popcll(bal));
      base = __builtin_amdgcn_readfirstlane(base);
      const int pos = base + mbcnt(bal);
      if (take && pos < kCand) L.c.cand[pos] = Cand{x, e};
    }
  }
  lds_barrier();
  const bool ok = L.ncand <= kCand;
  lds_barrier();
  return ok;
}

// The filtered draw decided over the whole row (FullLocator). Out of line,
// so that its registers do not count against the common path, with the
// locator inlined into it: every call level adds stack that the launch
// must reserve for every wave (with about 380 bytes per lane the ragged
// fp32 batch ran 1.3 us slower even with no row taking this path; with
// about 220, 0.9 us).
template <typename E, int NT>
__device__ __noinline__ int full_decide(const E* __restrict__ row, int V, float m, double Td, int top_k, double top_p,
                                        double min_p, double u, SampledLds<NT>& L) {
  FullLocator<E, NT> fl(L, row, V, m, Td);
  int t = 0;
  decide(fl, V, top_k, top_p, min_p, u, t);
  return t;
}

// Outcome of one sampled row.
struct SampledOut {
  int token;
  double lse;
  int bits;
  int slow;   // 1 if the exact whole-row path decided
};

// One workgroup samples row `row` of request `req` (local row j) with the
// request's parameters q (temperature q.T > 0). `after_stream(true)` runs
// once the row has been read (true: a long tail of work follows).
template <typename E, int NT, int U, typename Hook>
__device__ __forceinline__ SampledOut sampled_row(const VerifyArgs& a, const E* __restrict__ row, int req, int j,
                                                  const ReqParams& q, SampledLds<NT>& L, Hook after_stream) {
  SampledOut out{0, 0.0, 0, 0};
  const float T = q.T;
  int top_k = q.top_k;
  float top_p = q.top_p;
  float min_p = q.min_p;
  if (!(top_p > 0.f && top_p <= 1.f) || !(min_p >= 0.f && min_p <= 1.f) || !(T < INFINITY)) {
    out.bits |= VSV_FLAG_PARAMS;
    if (!(top_p > 0.f && top_p <= 1.f)) top_p = 1.f;
    if (!(min_p >= 0.f && min_p <= 1.f)) min_p = 0.f;
  }
  const double Td = static_cast<double>(T);
  const float c = 1.4426950408889634f / T;

  RowPartial p;
  partial_init(p);
  const VmPlan plan = stream_sampled<E, NT, U>(row, a.V, c, p, L);
  after_stream(true);   // selection and draw follow
  // with more rows than workgroups, other rows' streams go first (sampled.hip)
  if (a.R > static_cast<int>(gridDim.x)) __builtin_amdgcn_s_setprio(kSelectPrio);
  const NoKeep nokeep;
  const RowStats res = finish_row_lean<E, NT, U, false>(p, L.ls, nokeep, row, a.V);
  // the sum holds the maximum's own term (at least 1/2), so float log2
  // keeps the log-sum-exp within a few units of float rounding
  out.lse = 0.69314718f * (res.mref + __log2f(static_cast<float>(res.sum)));
  if (!(res.max < INFINITY) || !(res.max > -INFINITY) || !isfinite(out.lse)) out.bits |= VSV_FLAG_LOGITS;
  const float m = res.max;

  // Capture threshold: T * kZcap below the maximum (weights under e^-kZcap
  // of the max's), or exactly the min-p cut when min-p alone filters, but
  // no lower than the kCapVec-th largest vector maximum, so the candidates
  // fit. A top-k cut is a count, which an outlying maximum can push below
  // any window, so a top-k row captures down to its k-th largest vector
  // maximum instead. Whether the candidates suffice is decided from exact
  // mass accounting afterwards.
  // whole-row weight relative to the maximum, with the stream's exponents
  // (x * c with c = log2(e) / T rounded to float); CandLocator::build swaps
  // the candidates' share for their exact float64 weights
  const double wtot = res.sum * exp2(static_cast<double>(res.mref) -
                                     static_cast<double>(m) * static_cast<double>(c));
  const bool tk = top_k > 0 && top_k < a.V;
  float tau = -INFINITY;
  if (!out.bits) {
    if (tk) {
      tau = capture_threshold<E, NT>(L, plan, m, -INFINITY, top_k, true);
    } else {
      float dcap = T * kZcap;
      if (min_p > 0.f && top_p >= 1.f) {
        const float dm = static_cast<float>(-Td * log(static_cast<double>(min_p))) * 1.0001f + 1e-6f;
        dcap = fminf(dcap, dm);
      }
      const float floor_tau = (dcap < INFINITY) ? m - dcap : -INFINITY;
      // top-p rows: capture only down to where the vectors' maxima alone
      // already hold the top-p mass (with a margin for the streamed total's
      // rounding), when that takes at most kCapVec entries; the window's
      // threshold otherwise. On the large mixed bf16 batch (top-p 0.95 at
      // T = 0.7) this took the launch from 283.0 to 271.8 us.
      int nmass = 0;
      const float tmass = top_p < 1.f ? mass_code_threshold<E, NT>(L, plan, m, c, top_p * wtot * 1.001, nmass)
                                      : -INFINITY;
      if (tmass > -INFINITY && nmass <= kCapVec)
        tau = fmaxf(tmass, floor_tau);
      else
        tau = capture_threshold<E, NT>(L, plan, m, floor_tau, kCapVec, false);
    }
  }
  const double u = row_uniform(a.seed, a.offset, req, j);
  int token = 0;
  bool done = false;
  if (!out.bits && tau > -INFINITY && capture_row<E, NT>(row, a.V, tau, plan, L)) {
    CandLocator<E, NT> loc(L, m, Td, tau, wtot, static_cast<double>(c));
    loc.build();
    int t = 0;
    done = decide(loc, a.V, top_k, static_cast<double>(top_p), static_cast<double>(min_p), u, t) && !loc.bad;
    if (done) token = t;
  }
  if (!done && !(out.bits & VSV_FLAG_LOGITS)) {
    lds_barrier();
    token = full_decide<E, NT>(row, a.V, m, Td, top_k, static_cast<double>(top_p), static_cast<double>(min_p), u, L);
    out.slow = 1;
  }
  lds_barrier();
  out.token = token;
  return out;
}

}  // namespace vsv
