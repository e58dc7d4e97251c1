// Verification with probabilistic drafts (gfx950): the rejection sampler of
// speculative decoding over a packed batch.
//
// What is computed, per request i with drafts d_0 .. d_{K-1}: p_j is the
// target's law at row j (the sampled path's filtered, renormalised softmax
// of x_j / T_i, or the point mass at the arg-max when T_i = 0) and q_j the
// draft's (the softmax of the draft row over the request's draft
// temperature, or the point mass at that row's arg-max when it is 0). Draft
// j passes when u_acc * q_j(d_j) < p_j(d_j), i.e. with probability
// min(1, p / q). The first rejected row emits the inverse-CDF draw of
// max(0, p_j - q_j) in the target's rank order (value descending, index
// ascending; first cumulative weight strictly above u times the total), and
// a request whose drafts all pass emits the bonus row's draw from p_K. The
// pages name this case and leave it unsupported (xLLM docs, "Adaptive
// speculative inference", DSpark section "Launch example"): their point-mass
// drafts, which the sampled path verifies, are its special case.
//
// How: exact first. One workgroup per row streams the target row for its
// maximum and arg-max. A sampled row then gathers a head of its rank order
// (whole bands of z = (x - m) / T, up to 4096 entries) into LDS and sorts
// it; when that head decides the top-k / top-p cut, the survivor set, the
// own draw and the residual draw of max(0, p - q) are block scans over the
// sorted list. Otherwise the sampled path's exact whole-row radix locator
// settles them (several passes over the row, which stays in the caches).
// The draft row is read once for its maximum and exponent sum. Each row
// stores a tagged word; the workgroup that finishes last runs the
// per-request scan.
#include "probabilistic.hpp"
#include "sampled_row.hpp"
#include "verify_common.hpp"

namespace vsv {

namespace {

constexpr int kBands = 64;  // bands of z = (x - m) / T, a quarter wide, for the top-p head

// Visits every element e = threadIdx.x + k NT of a row as f(e, value),
// with the loads of kBatch steps issued before any is used. These loops run
// over rows already in the caches; with one load per iteration each thread
// would wait out every load's latency in turn.
template <typename E, int NT, typename F>
__device__ __forceinline__ void for_each_elem(const E* __restrict__ row, int V, F f) {
  constexpr int kBatch = 8;
  for (int base = threadIdx.x; base < V; base += NT * kBatch) {
    float xs[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int e = base + b * NT;
      xs[b] = e < V ? Elem<E>::at(row, e) : 0.f;
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int e = base + b * NT;
      if (e < V) f(e, xs[b]);
    }
  }
}

// Uniforms of (request, local row): word 0 of the row's Philox block draws
// the token (the sampled path's u), word 1 tests acceptance.
__device__ __forceinline__ void prob_uniforms(uint64_t seed, uint64_t offset, int request, int row, double& u,
                                              double& u_acc) {
  const Philox4 o = philox4x32_10(
      Philox4{static_cast<uint32_t>(row), static_cast<uint32_t>(request), static_cast<uint32_t>(offset),
              static_cast<uint32_t>(offset >> 32)},
      static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
  u = static_cast<double>(o.x >> 8) * (1.0 / 16777216.0);
  u_acc = static_cast<double>(o.y >> 8) * (1.0 / 16777216.0);
}

// The survivor set, a prefix of the rank order: its size, its total weight
// and its last token (key and index).
struct Support {
  int n;
  double w;
  uint32_t key;
  int idx;
};

// The filters in the sampled path's order: top-k count, top-p mass over the
// top-k survivors (the crossing token kept), min-p cut.
template <typename E, int NT>
__device__ Support support(FullLocator<E, NT>& loc, int V, int top_k, double top_p, double min_p) {
  // `last` is the survivor set's last token whenever a filter has cut it
  int n = V;
  double w;
  Pick last{};
  bool have = false;
  if (top_k > 0 && top_k < V) {
    n = top_k;
    last = loc.by_count(top_k);
    w = last.cum;
    have = true;
  } else {
    w = loc.total_mass();
  }
  if (top_p < 1.0) {
    last = loc.by_mass(top_p * w, false);
    n = last.rank + 1;
    w = last.cum;
    have = true;
  }
  if (min_p > 0.0) {
    bool exact = false;
    const int lm = loc.count_minp(log(min_p), exact);
    if (lm < n) {
      n = lm > 0 ? lm : 1;
      last = loc.by_count(n);
      w = last.cum;
      have = true;
    }
  }
  if (!have) last = loc.by_count(n);
  return Support{n, w, ord_ukey(loc.at(last.idx)), last.idx};
}

__device__ __forceinline__ bool in_support(uint32_t k, int e, const Support& s) {
  return k > s.key || (k == s.key && e <= s.idx);
}

// The draft's law: softmax of the draft row over Td, or the point mass at
// its lowest arg-max when Td = 0.
struct DraftLaw {
  float my;
  double Td;
  double Z;
  int h;
  __device__ double q(float y, int e) const {
    if (Td > 0.0) return exp((static_cast<double>(y) - static_cast<double>(my)) / Td) / Z;
    return e == h ? 1.0 : 0.0;
  }
};

// One pass over the draft row: each thread keeps a running maximum and the
// float64 sum of exp((y - max) / Td) rescaled when its maximum grows (for
// Td = 0, the lowest index of its maximum). Returns false when the row has
// a NaN or no finite maximum.
template <typename E, int NT>
__device__ bool draft_law(const E* __restrict__ y, int V, double Td, SampledLds<NT>& L, DraftLaw& q) {
  float mx = -INFINITY;
  double sum = 0.0;
  int h = INT32_MAX, nan = 0;
  for_each_elem<E, NT>(y, V, [&](int e, float v) {
    if (v != v) {
      nan = 1;
    } else if (v > mx) {
      if (Td > 0.0) sum = sum * exp((static_cast<double>(mx) - static_cast<double>(v)) / Td) + 1.0;
      mx = v;
      h = e;
    } else if (Td > 0.0 && mx > -INFINITY) {
      sum += exp((static_cast<double>(v) - static_cast<double>(mx)) / Td);
    }
  });
  nan = block_reduce<NT>(nan, MaxOp(), L.red_i);
  const double md = block_reduce<NT>(static_cast<double>(mx), MaxOp(), L.red_d);
  q.my = static_cast<float>(md);
  q.Td = Td;
  q.Z = 1.0;
  q.h = 0;
  if (nan || !(md > -INFINITY) || !(md < INFINITY)) return false;
  if (Td > 0.0) {
    const double part = mx > -INFINITY ? sum * exp((static_cast<double>(mx) - md) / Td) : 0.0;
    q.Z = block_reduce<NT>(part, SumOp(), L.red_d);
  } else {
    // each thread's first index of its maximum is its lowest (indices grow)
    q.h = block_reduce<NT>(mx == q.my ? h : INT32_MAX, MinOp(), L.red_i);
  }
  return true;
}

// The residual draw: the first token in rank order whose cumulative
// max(0, p - q) exceeds u times the residual's total, or -1 if the residual
// has no mass.
template <typename E, int NT>
__device__ int residual_draw(const E* __restrict__ x, const E* __restrict__ y, int V, float m, double T,
                             const Support& s, const DraftLaw& q, double u, SampledLds<NT>& L) {
  // the draft row is read only at survivors
  auto mass = [&](int e, float xv, uint32_t& k) -> double {
    k = ord_ukey(xv);
    if (!in_support(k, e, s)) return 0.0;
    const double r = weight(xv, m, T) / s.w - q.q(Elem<E>::at(y, e), e);
    return r > 0.0 ? r : 0.0;
  };
  // radix descent over the keys (8-bit digits, most significant first),
  // counting only tokens of positive residual mass
  uint32_t prefix = 0;
  for (int d = 0; d < 4; ++d) {
    const int shift = 24 - 8 * d;
    for (int b = threadIdx.x; b < 256; b += NT) {
      L.u.radix.cnt[b] = 0;
      L.u.radix.mass[b] = 0.0;
    }
    lds_barrier();
    for_each_elem<E, NT>(x, V, [&](int e, float xv) {
      if (d > 0 && (ord_ukey(xv) >> (shift + 8)) != prefix) return;
      uint32_t k;
      const double r = mass(e, xv, k);
      if (!(r > 0.0)) return;
      const int dig = static_cast<int>((k >> shift) & 255u);
      atomicAdd(&L.u.radix.cnt[dig], 1);
      atomicAdd(&L.u.radix.mass[dig], r);
    });
    lds_barrier();
    if (threadIdx.x == 0) {
      if (d == 0) {
        double t = 0.0;
        for (int b = 255; b >= 0; --b) t += L.u.radix.mass[b];
        L.bd[2] = u * t;  // the target
        L.bd[0] = 0.0;    // mass above the located prefix
      }
      const double target = L.bd[2];
      double w = L.bd[0], wl = 0.0;
      int dsel = -1, dl = -1;
      for (int dig = 255; dig >= 0; --dig) {
        if (L.u.radix.cnt[dig] == 0) continue;
        const double nw = w + L.u.radix.mass[dig];
        dl = dig;
        wl = w;
        if (nw > target) {
          dsel = dig;
          break;
        }
        w = nw;
      }
      // a target at the total (rounding) takes the last token with mass
      if (dsel < 0) {
        dsel = dl;
        w = wl;
      }
      L.bi[0] = dsel;
      L.bd[0] = w;
    }
    lds_barrier();
    const int dsel = L.bi[0];
    if (dsel < 0) return -1;  // uniform: no mass at all
    prefix = (prefix << 8) | static_cast<uint32_t>(dsel);
  }
  const uint32_t key = prefix;
  const double target = L.bd[2];
  double acc = L.bd[0];
  lds_barrier();
  // the located key's tokens in index order
  int mylast = -1;
  for (int base = 0; base < V; base += NT * 8) {
    const int lo = base + static_cast<int>(threadIdx.x) * 8;
    float xs[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) xs[b] = lo + b < V ? Elem<E>::at(x, lo + b) : 0.f;
    double c = 0.0;
    for (int b = 0; b < 8 && lo + b < V; ++b) {
      if (ord_ukey(xs[b]) != key) continue;
      uint32_t k;
      const double r = mass(lo + b, xs[b], k);
      if (r > 0.0) {
        c += r;
        mylast = lo + b;
      }
    }
    double tot;
    const double incl = block_scan_incl<NT, double>(c, L.red_d, tot);
    if (threadIdx.x == 0) L.bi[3] = INT32_MAX;
    lds_barrier();
    if (c > 0.0 && acc + (incl - c) <= target && acc + incl > target) {
      double run = acc + (incl - c);
      int pick = -1;
      for (int b = 0; b < 8 && lo + b < V; ++b) {
        if (ord_ukey(xs[b]) != key) continue;
        uint32_t k;
        const double r = mass(lo + b, xs[b], k);
        if (r > 0.0) {
          pick = lo + b;
          run += r;
          if (run > target) break;
        }
      }
      atomicMin(&L.bi[3], pick);
    }
    lds_barrier();
    const int found = L.bi[3];
    lds_barrier();
    if (found != INT32_MAX) return found;
    acc += tot;
  }
  return block_reduce<NT>(mylast, MaxOp(), L.red_i);
}

// When the survivors fit in the candidate buffer (the usual case: top-p
// keeps a small head of the order) they are gathered into LDS and sorted
// into rank order (bitonic; key descending, index ascending). The own draw
// and the residual draw are then scans over that list. Returns n, the
// entries c[0 .. n) of L.c.cand.
template <typename E, int NT, typename Pred>
__device__ int gather_sorted(const E* __restrict__ x, int V, int count, Pred keep, SampledLds<NT>& L) {
  int P = 1;
  while (P < count) P <<= 1;
  Cand* c = L.c.cand;
  if (threadIdx.x == 0) L.ncand = 0;
  for (int k = threadIdx.x; k < P; k += NT) c[k] = Cand{-INFINITY, INT32_MAX};
  lds_barrier();
  for_each_elem<E, NT>(x, V, [&](int e, float xv) {
    if (!keep(e, xv)) return;
    const int slot = atomicAdd(&L.ncand, 1);
    if (slot < P) c[slot] = Cand{xv, e};
  });
  lds_barrier();
  // rank order; the padding (index INT32_MAX, lowest key) sorts last
  auto before = [](const Cand& a, const Cand& b) {
    const uint32_t ka = a.idx == INT32_MAX ? 0u : ord_ukey(a.x) + 1u;
    const uint32_t kb = b.idx == INT32_MAX ? 0u : ord_ukey(b.x) + 1u;
    return ka > kb || (ka == kb && a.idx < b.idx);
  };
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < P / 2; t += NT) {
        const int lo = 2 * t - (t & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const Cand a = c[lo], b = c[hi];
        if (before(b, a) == up) {
          c[lo] = b;
          c[hi] = a;
        }
      }
      lds_barrier();
    }
  }
  return min(L.ncand, P);
}

// Position of the first of n listed entries whose cumulative mass exceeds u
// times the list's total (the last entry with mass if rounding leaves the
// target at the total), or -1 if the list has no mass. A block scan over
// contiguous runs of the list finds the run; its thread walks it.
template <int NT, typename Mass>
__device__ int scan_pick(int n, Mass mass, double u, SampledLds<NT>& L, bool strict = true, double of = -1.0,
                         bool last_if_none = true) {
  const int per = (n + NT - 1) / NT;
  const int k0 = min(n, static_cast<int>(threadIdx.x) * per), k1 = min(n, k0 + per);
  double seg = 0.0;
  int mylast = -1;
  for (int k = k0; k < k1; ++k) {
    const double r = mass(k);
    seg += r;
    if (r > 0.0) mylast = k;
  }
  double total;
  const double incl = block_scan_incl<NT, double>(seg, L.red_d, total);
  if (!(total > 0.0)) return -1;  // uniform
  const double target = u * (of < 0.0 ? total : of);
  auto past = [&](double c) { return strict ? c > target : c >= target; };
  if (threadIdx.x == 0) L.bi[3] = INT32_MAX;
  lds_barrier();
  if (seg > 0.0 && !past(incl - seg) && past(incl)) {
    double run = incl - seg;
    int pick = -1;
    for (int k = k0; k < k1; ++k) {
      const double r = mass(k);
      if (r > 0.0) {
        pick = k;
        run += r;
        if (past(run)) break;
      }
    }
    atomicMin(&L.bi[3], pick);
  }
  lds_barrier();
  int k = L.bi[3];
  if (k == INT32_MAX) k = last_if_none ? block_reduce<NT>(mylast, MaxOp(), L.red_i) : -1;
  lds_barrier();
  return k;
}

}  // namespace

template <typename E, int NT, int U>
__global__ __launch_bounds__(NT) void verify_probabilistic_kernel(VerifyArgs a, ProbArgs pa) {
  __shared__ SampledLds<NT> L;
  static_assert(sizeof(TailScratch) <= sizeof(L.c), "tail staging aliases the candidate buffer");
  const uint32_t tag = call_tag(a);
  const int r = static_cast<int>(blockIdx.x);
  const E* __restrict__ row = static_cast<const E*>(a.logits) + static_cast<int64_t>(r) * a.ld;
  const RowMeta m = load_meta(a, r, a.owner[r]);
  const int req = m.req < 0 ? 0 : m.req;
  const float T = a.temperature[req];
  const float Tq = pa.draft_temperature[req];
  int top_k = a.top_k[req];
  float top_p = a.top_p[req];
  float min_p = a.min_p[req];
  int bits = 0;
  if (m.req >= 0) {
    if (!(T >= 0.f && T < INFINITY) || !(Tq >= 0.f && Tq < INFINITY)) bits |= VSV_FLAG_PARAMS;
    if (!(top_p > 0.f && top_p <= 1.f)) {
      bits |= VSV_FLAG_PARAMS;
      top_p = 1.f;
    }
    if (!(min_p >= 0.f && min_p <= 1.f)) {
      bits |= VSV_FLAG_PARAMS;
      min_p = 0.f;
    }
  }

  // the target row's maximum and lowest arg-max
  RowPartial p;
  partial_init(p);
  GroupKeep<U> keep{};
  constexpr float kLog2e = 1.4426950408889634f;
  stream_row<E, NT, U, false>(row, a.V, kLog2e, INFINITY, 0, p, keep);
  const RowResult res = finish_row<E, NT, U, false, true>(p, L.rs, keep, row, a.V);
  int token = res.argmax == INT32_MAX ? 0 : res.argmax;
  if (!(res.max < INFINITY) || res.argmax == INT32_MAX || !isfinite(res.lse)) bits |= VSV_FLAG_LOGITS;

  bool accept = false;
  const bool live = m.req >= 0 && !(bits & VSV_FLAG_LOGITS);
  if (live && T > 0.f && T < INFINITY) {
    const double Td = static_cast<double>(T);
    lds_barrier();
    FullLocator<E, NT> fl(L, row, a.V, res.max, Td);
    const Cand* c = L.c.cand;
    Support s{0, 0.0, 0u, 0};
    bool listed = false;
    const bool tk = top_k > 0 && top_k < a.V;
    if (tk ? top_k <= kCand : top_p < 1.f) {
      // the survivors from a sorted head of the order: one pass counts the
      // elements in bands of z = (x - m) / T (and, without top-k, takes the
      // total weight); the widest head of whole bands that fits the list is
      // gathered and sorted. Bands are monotone in x, so the head is a
      // prefix of the rank order. It decides when it holds the top-k, or
      // top_p of the total.
      const float mx = res.max;
      auto band = [&](float xv) {
        const double z = (static_cast<double>(xv) - static_cast<double>(mx)) / Td;
        return z > -16.0 ? min(static_cast<int>(-z * 4.0), kBands - 1) : kBands - 1;
      };
      for (int b = threadIdx.x; b < kBands; b += NT) L.u.radix.cnt[b] = 0;
      lds_barrier();
      double sw = 0.0;
      for_each_elem<E, NT>(row, a.V, [&](int, float xv) {
        if (!tk) sw += weight(xv, mx, Td);
        atomicAdd(&L.u.radix.cnt[band(xv)], 1);
      });
      const double W = block_reduce<NT>(sw, SumOp(), L.red_d);
      if (threadIdx.x == 0) {
        int cum = 0, top = -1;
        for (int b = 0; b < kBands && cum + L.u.radix.cnt[b] <= kCand; ++b) {
          cum += L.u.radix.cnt[b];
          top = b;
        }
        L.bi[0] = top;
        L.bi[1] = cum;
      }
      lds_barrier();
      const int top = L.bi[0], cnt = L.bi[1];
      lds_barrier();
      if (top >= 0 && cnt >= (tk ? top_k : 1)) {
        const int nl = gather_sorted<E, NT>(row, a.V, cnt, [&](int, float xv) { return band(xv) <= top; }, L);
        auto wt = [&](int k) { return weight(c[k].x, mx, Td); };
        int n = -1;
        if (tk) {
          n = top_k;
          if (top_p < 1.f) {
            double s1 = 0.0;
            for (int q = threadIdx.x; q < top_k; q += NT) s1 += wt(q);
            const double W1 = block_reduce<NT>(s1, SumOp(), L.red_d);
            n = scan_pick<NT>(top_k, wt, static_cast<double>(top_p), L, false, W1, true) + 1;
          }
        } else {
          n = scan_pick<NT>(nl, wt, static_cast<double>(top_p), L, false, W, false) + 1;
        }
        if (n > 0) {
          if (min_p > 0.f) {
            bool exact = false;
            const int lm = fl.count_minp(log(static_cast<double>(min_p)), exact);
            if (lm < n) n = lm > 0 ? lm : 1;
          }
          double sn = 0.0;
          for (int q = threadIdx.x; q < n; q += NT) sn += wt(q);
          const double w = block_reduce<NT>(sn, SumOp(), L.red_d);
          s = Support{n, w, ord_ukey(c[n - 1].x), c[n - 1].idx};
          listed = true;
        }
      }
    }
    if (!listed) {
      s = support(fl, a.V, top_k, static_cast<double>(top_p), static_cast<double>(min_p));
      listed = s.n <= kCand;
      if (listed) gather_sorted<E, NT>(row, a.V, s.n, [&](int e, float xv) { return in_support(ord_ukey(xv), e, s); }, L);
    }
    const int n = s.n;
    double u, ua;
    prob_uniforms(a.seed, a.offset, m.req, m.j, u, ua);
    if (listed) {
      const int k = scan_pick<NT>(n, [&](int k) { return weight(c[k].x, res.max, Td); }, u, L);
      token = c[k < 0 ? 0 : k].idx;
    } else {
      Pick own = fl.by_mass(u * s.w, true);
      if (own.rank >= s.n) own = fl.by_count(s.n);
      token = own.idx;
    }
    if (m.j < m.K) {
      const E* __restrict__ y = static_cast<const E*>(pa.draft_logits) + static_cast<int64_t>(r - m.req) * pa.dld;
      const double Tdq = (Tq >= 0.f && Tq < INFINITY) ? static_cast<double>(Tq) : 0.0;
      DraftLaw q;
      if (!draft_law<E, NT>(y, a.V, Tdq, L, q)) {
        bits |= VSV_FLAG_LOGITS;
      } else {
        const int d = m.draft;
        if (d >= 0 && d < a.V) {
          const float xd = Elem<E>::at(row, d);
          const double pd = in_support(ord_ukey(xd), d, s) ? weight(xd, res.max, Td) / s.w : 0.0;
          accept = ua * q.q(Elem<E>::at(y, d), d) < pd;
        }
        int t = -1;
        if (listed) {
          const int k = scan_pick<NT>(n, [&](int k) {
            const double r = weight(c[k].x, res.max, Td) / s.w - q.q(Elem<E>::at(y, c[k].idx), c[k].idx);
            return r > 0.0 ? r : 0.0;
          }, u, L);
          if (k >= 0) t = c[k].idx;
        } else {
          t = residual_draw<E, NT>(row, y, a.V, res.max, Td, s, q, u, L);
        }
        if (t >= 0) token = t;
      }
    }
  } else if (live) {
    // a greedy target is the point mass at its arg-max: a draft passes
    // exactly when it is the arg-max, and the residual is the arg-max too
    accept = m.j < m.K && m.draft == token;
  }
  if (threadIdx.x == 0) {
    const uint32_t word = row_word(a, m, token, accept, bits);
    if (bits) set_flag(a, bits);
    if (a.row_token) a.row_token[r] = token;
    store_agent64(a.ws_row + r, tagged(tag, word));
    const uint32_t done = __hip_atomic_fetch_add(a.ws_queue + kQueueDone, 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    L.last = done + 1 == gridDim.x;
  }
  lds_barrier();
  if (L.last) {
    if (threadIdx.x == 0) store_agent(a.ws_queue + kQueueDone, 0u);
    words_tail<NT>(a, tag, *reinterpret_cast<TailScratch*>(&L.c));
  }
}

template <typename E>
static hipError_t launch_probabilistic_t(const VerifyArgs& a, const ProbArgs& p, hipStream_t s) {
  verify_probabilistic_kernel<E, kVerifyThreads, SampledDepth<E>::kGreedy>
      <<<dim3(a.R), dim3(kVerifyThreads), 0, s>>>(a, p);
  return hipGetLastError();
}

hipError_t launch_verify_probabilistic(const VerifyArgs& a, const ProbArgs& p, hipStream_t s) {
  return a.dtype == VSV_BF16 ? launch_probabilistic_t<uint16_t>(a, p, s) : launch_probabilistic_t<float>(a, p, s);
}

}  // namespace vsv
