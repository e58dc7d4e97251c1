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
// How: rows come from the persistent row queue (row_queue.hpp), two
// workgroups per CU. A sampled row takes the sampled path's first pass (its
// maximum, streamed total weight and vector-maximum codes), captures every
// element at or above the sampled path's capture threshold into LDS and
// ranks them (a counting sort over bfloat16 codes, a bitonic sort for
// float32); the streamed total is corrected with the captured elements'
// exact float64 weights. When that head decides the top-k / top-p / min-p
// cut, the survivor set, the own draw and the residual draw of max(0, p - q)
// are block scans over LDS arrays of weights and residual masses.
// Otherwise the sampled path's exact whole-row locator settles them, out of
// line. A draft row is read once, in float32, for its maximum and exponent
// sum. Each row stores a tagged word; the workgroup that finishes last runs
// the per-request scan.
#include "probabilistic.hpp"
#include "row_queue.hpp"
#include "sampled_row.hpp"
#include "verify_common.hpp"

namespace vsv {

namespace {

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

// Exact locator over the whole row for the probabilistic path: radix select
// on the order-preserving key (four 8-bit digits, most significant first),
// then the tie of the located value in index order. It reads the row several
// times and weighs every element in float64 on each pass, so it is slower
// than the sampled path's histogram search, but its few registers keep the
// probabilistic kernel, which calls it out of line with much of its row
// state live, from spilling around the call: with the histogram search
// there, the mixed batch ran at 0.85 ms instead of 0.64.
template <typename E, int NT>
struct RadixLocator {
  SampledLds<NT>& L;
  const E* __restrict__ row;
  int V;
  float m;
  double T;
  double wtot;

  __device__ RadixLocator(SampledLds<NT>& l, const E* r, int V_, float m_, double T_)
      : L(l), row(r), V(V_), m(m_), T(T_), wtot(0.0) {}

  __device__ float at(int e) const { return Elem<E>::at(row, e); }

  __device__ double total_mass() {
    double s = 0.0;
    for (int e = threadIdx.x; e < V; e += NT) s += weight(at(e), m, T);
    wtot = block_reduce<NT>(s, SumOp(), L.red_d);
    return wtot;
  }

  // The located value's key and the count / weight strictly above it.
  __device__ void radix(bool by_weight, double target, int rank, bool strict, uint32_t& key, int& above_c,
                        double& above_m, int& tie_c, double& tie_w) {
    // by_weight: locate the first rank whose cumulative weight reaches
    // target; otherwise locate rank `rank`. Weights are accumulated either way.
    uint32_t prefix = 0;
    above_c = 0;
    above_m = 0.0;
    for (int d = 0; d < 4; ++d) {
      const int shift = 24 - 8 * d;
      for (int b = threadIdx.x; b < 256; b += NT) {
        L.u.radix.cnt[b] = 0;
        L.u.radix.mass[b] = 0.0;
      }
      lds_barrier();
      for (int e = threadIdx.x; e < V; e += NT) {
        const float x = at(e);
        const uint32_t k = ord_ukey(x);
        if (d > 0 && (k >> (shift + 8)) != prefix) continue;
        const int dig = (k >> shift) & 255;
        atomicAdd(&L.u.radix.cnt[dig], 1);
        atomicAdd(&L.u.radix.mass[dig], weight(x, m, T));
      }
      lds_barrier();
      if (threadIdx.x == 0) {
        int dsel = 0, c = above_c;
        double w = above_m;
        for (int dig = 255; dig >= 0; --dig) {
          const int nc2 = c + L.u.radix.cnt[dig];
          const double nw = w + L.u.radix.mass[dig];
          const bool hit = by_weight ? (strict ? nw > target : nw >= target) : (rank < nc2);
          if (hit && L.u.radix.cnt[dig] > 0) {
            dsel = dig;
            break;
          }
          c = nc2;
          w = nw;
          dsel = dig;
        }
        L.bi[0] = dsel;
        L.bi[1] = c;
        L.bd[0] = w;
        L.bi[2] = L.u.radix.cnt[dsel];
      }
      lds_barrier();
      prefix = (prefix << 8) | static_cast<uint32_t>(L.bi[0]);
      above_c = L.bi[1];
      above_m = L.bd[0];
      tie_c = L.bi[2];
      lds_barrier();
    }
    key = prefix;
    const int kk = static_cast<int>(prefix ^ 0x80000000u);
    tie_w = weight(key_float(kk), m, T);
  }

  // Index of the (n+1)-th element (0-based n) whose key equals `key`,
  // scanning the row in index order in chunks of 8 per thread.
  __device__ int nth_tie(uint32_t key, int n) {
    int need = n;
    for (int base = 0; base < V; base += NT * 8) {
      const int lo = base + static_cast<int>(threadIdx.x) * 8;
      int c = 0;
      for (int e = lo; e < lo + 8 && e < V; ++e) c += (ord_ukey(at(e)) == key) ? 1 : 0;
      int tot;
      const int incl = block_scan_incl<NT, int>(c, L.red_i, tot);
      const int excl = incl - c;
      if (threadIdx.x == 0) L.bi[3] = -1;
      lds_barrier();
      if (need >= excl && need < incl) {
        int k = need - excl;
        for (int e = lo; e < lo + 8 && e < V; ++e) {
          if (ord_ukey(at(e)) == key) {
            if (k == 0) {
              L.bi[3] = e;
              break;
            }
            --k;
          }
        }
      }
      lds_barrier();
      const int found = L.bi[3];
      lds_barrier();
      if (found >= 0) return found;
      need -= tot;
    }
    return 0;
  }

  __device__ Pick by_count(int k) {
    Pick p{0, k - 1, 0.0, false, 0, 0};
    if (k < 1 || k > V) return p;
    uint32_t key;
    int ac, tc;
    double am, tw;
    radix(false, 0.0, k - 1, false, key, ac, am, tc, tw);
    const int j = k - 1 - ac;
    p.idx = nth_tie(key, j);
    p.cum = am + static_cast<double>(j + 1) * tw;
    p.ok = true;
    return p;
  }

  __device__ Pick by_mass(double target, bool strict) {
    Pick p{0, 0, 0.0, false, 0, 0};
    uint32_t key;
    int ac, tc;
    double am, tw;
    radix(true, target, 0, strict, key, ac, am, tc, tw);
    int j = 0;
    if (tw > 0.0) {
      const double q = (target - am) / tw;
      j = strict ? static_cast<int>(floor(q)) : static_cast<int>(ceil(q)) - 1;
      // settle rounding against the exact comparison
      while (j > 0 && (strict ? am + j * tw > target : am + j * tw >= target)) --j;
      while (j < tc - 1 && !(strict ? am + (j + 1) * tw > target : am + (j + 1) * tw >= target)) ++j;
    }
    j = j < 0 ? 0 : (j >= tc ? tc - 1 : j);
    p.idx = nth_tie(key, j);
    p.rank = ac + j;
    p.cum = am + static_cast<double>(j + 1) * tw;
    p.ok = true;
    return p;
  }

  __device__ int token(const Pick& p) const { return p.idx; }

  __device__ int count_minp(double lnmp, bool& exact) {
    int c = 0;
    for (int e = threadIdx.x; e < V; e += NT)
      c += ((static_cast<double>(at(e)) - static_cast<double>(m)) / T >= lnmp) ? 1 : 0;
    exact = true;
    return block_reduce<NT>(c, SumOp(), L.red_i);
  }
};

// The filters in the sampled path's order: top-k count, top-p mass over the
// top-k survivors (the crossing token kept), min-p cut.
template <typename E, int NT>
__device__ __forceinline__ Support support(RadixLocator<E, NT>& loc, int V, int top_k, double top_p, double min_p) {
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

// The draft row's law in one streaming pass, float32 exponentials: for
// Td > 0 each thread keeps a running maximum, an integer exponent reference
// and the float64 sum of float32 group sums of exp2(y * c - mc), with
// c = log2(e) / Td split into a float and its float remainder (so the
// rounding of c adds no error proportional to |y|; what is left is the
// float rounding of each exponent, random across elements); Z is that sum
// rebased to the row maximum. For Td = 0 the row's lowest arg-max. Returns
// false when the row has a NaN or no finite maximum.
template <typename E, int NT, int U>
__device__ bool draft_law_stream(const E* __restrict__ y, int V, double Td, SampledLds<NT>& L, DraftLaw& q) {
  constexpr int N = Elem<E>::kVec;
  q.Td = Td;
  q.Z = 1.0;
  q.h = 0;
  if (!(Td > 0.0)) {
    RowPartial p;
    partial_init(p);
    QueueKeep<E, U> keep{};
    stream_row<E, NT, U, false, QueueKeep<E, U>, NoHook, true>(y, V, 1.4426950408889634f, INFINITY, 0, p, keep);
    const RowStats st = finish_row_lean<E, NT, U, false>(p, L.ls, keep, y, V);
    q.my = st.max;
    q.h = st.argmax;
    return !(st.sum != st.sum) && st.max > -INFINITY && st.max < INFINITY && st.argmax != INT32_MAX;
  }
  const double cd = 1.4426950408889634074 / Td;
  const float chi = static_cast<float>(cd);
  const float clo = static_cast<float>(cd - static_cast<double>(chi));
  float mx = -INFINITY, mc = -FLT_MAX;
  double sum = 0.0;
  int nan = 0;
  auto rebase = [&](float vmax) {
    const float yy = vmax * chi;
    if (yy > mc && yy < FLT_MAX) {
      const float nm = ceilf(yy);
      sum = (mc > -FLT_MAX) ? ldexp(sum, static_cast<int>(fmaxf(mc - nm, -2000.f))) : 0.0;
      mc = nm;
    }
  };
  // -inf (a zero-probability logit, or a masked lane) is clamped to the
  // lowest float first: with a negative remainder clo, -inf * clo would
  // meet -inf * chi as inf - inf; the clamped term is exactly 0
  auto term = [&](float v) {
    const float w = fmaxf(v, -FLT_MAX);
    return fast_exp2(fmaf(w, clo, fmaf(w, chi, -mc)));
  };
  const uintptr_t addr = reinterpret_cast<uintptr_t>(y);
  int head = static_cast<int>(((16u - (addr & 15u)) & 15u) / sizeof(E));
  if (head > V) head = V;
  const int nvec = (V - head) / N;
  // Groups of U vectors per thread (vector g * G + u * NT + tid of group g),
  // two groups in turn: one group's loads are in flight while the other is
  // reduced. Loads go through a buffer resource over the body (vectors past
  // it read as zero and are masked) with the streaming policy.
  constexpr int G = U * NT;
  const __amdgpu_buffer_rsrc_t rsrc = vec_rsrc(y + head, nvec);
  const int lane_off = static_cast<int>(threadIdx.x) * 16;
  const int ngroups = (nvec + G - 1) / G;
  auto load_group = [&](u32x4* w, int g) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      w[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, lane_off, (g * G + u * NT) * 16,
                                                                             kLoadStream));
  };
  auto reduce_group = [&](const u32x4* w, int base) {
    float f[U][N];
    float gmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      Elem<E>::decode(w[u], f[u]);
      const bool in = base + u * NT < nvec;
#pragma unroll
      for (int k = 0; k < N; ++k) {
        if (!in) f[u][k] = -INFINITY;
        nan |= f[u][k] != f[u][k] ? 1 : 0;
        gmax = fmaxf(gmax, f[u][k]);
      }
    }
    mx = fmaxf(mx, gmax);
    rebase(gmax);
    float e[U * N];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int k = 0; k < N; ++k) e[u * N + k] = term(f[u][k]);
    sum += static_cast<double>(tree_sum<U * N>(e));
  };
  u32x4 A[U], B[U];
  if (ngroups > 0) load_group(A, 0);
  if (ngroups > 1) load_group(B, 1);
  for (int g = 0; g < ngroups; g += 2) {
    const int ba = g * G + static_cast<int>(threadIdx.x);
    if (ba < nvec) reduce_group(A, ba);
    if (g + 2 < ngroups) load_group(A, g + 2);
    if (g + 1 < ngroups) {
      const int bb = ba + G;
      if (bb < nvec) reduce_group(B, bb);
      if (g + 3 < ngroups) load_group(B, g + 3);
    }
  }
  const int body_end = head + nvec * N;
  auto scalar = [&](float v) {
    nan |= v != v ? 1 : 0;
    mx = fmaxf(mx, v);
    rebase(v);
    sum += static_cast<double>(term(v));
  };
  if (static_cast<int>(threadIdx.x) < head) scalar(Elem<E>::at(y, threadIdx.x));
  if (static_cast<int>(threadIdx.x) < V - body_end) scalar(Elem<E>::at(y, body_end + threadIdx.x));
  nan = block_reduce<NT>(nan, MaxOp(), L.red_i);
  const float my = block_reduce<NT>(mx, MaxOp(), reinterpret_cast<float*>(L.red_d));
  const float mg = block_reduce<NT>(mc, MaxOp(), reinterpret_cast<float*>(L.red_d));
  q.my = my;
  if (nan || !(my > -INFINITY) || !(my < INFINITY)) return false;
  const double part = (mc > -FLT_MAX) ? ldexp(sum, static_cast<int>(fmaxf(mc - mg, -2000.f))) : 0.0;
  const double tot = block_reduce<NT>(part, SumOp(), L.red_d);
  q.Z = tot * exp2(static_cast<double>(mg) - static_cast<double>(my) * cd);
  return q.Z > 0.0 && q.Z < INFINITY;
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

// Sort c[0 .. P) (P a power of two) into rank order: key descending, index
// ascending; padding (index INT32_MAX) sorts last. Bitonic, in LDS.
template <int NT>
__device__ void sort_rank(Cand* c, int P) {
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
}

// Rank order of the nc candidates c[0 .. nc) (every element >= tau, all at
// most the maximum mx). bfloat16 rows: a counting sort over the values'
// codes below the maximum's (a code is one value), then each entry takes
// its place inside its code by counting the entries of that code with a
// lower index. float32 rows, or codes spanning kCodeBins or more: the
// bitonic sort. Scratch: the LDS union u (a Cand buffer and two code
// arrays), free once the capture is done.
constexpr int kCodeBins = 1024;
template <typename E, int NT>
__device__ void rank_candidates(SampledLds<NT>& L, int nc, float mx) {
  Cand* c = L.c.cand;
  static_assert(sizeof(L.u) >= kCand * sizeof(Cand) + 2 * (kCodeBins + 1) * sizeof(int), "sort scratch");
  Cand* tmp = reinterpret_cast<Cand*>(&L.u);
  int* start = reinterpret_cast<int*>(tmp + kCand);
  int* cur = start + kCodeBins + 1;
  bool counting = sizeof(E) == 2;
  const int mcode = bf16_code(mx);
  if (counting) {
    int span = 0;
    for (int k = threadIdx.x; k < nc; k += NT) span = max(span, mcode - bf16_code(c[k].x));
    span = block_reduce<NT>(span, MaxOp(), L.red_i);
    counting = span < kCodeBins;
  }
  if (!counting) {
    int P = 1;
    while (P < nc) P <<= 1;
    for (int k = nc + static_cast<int>(threadIdx.x); k < P; k += NT) c[k] = Cand{-INFINITY, INT32_MAX};
    lds_barrier();
    sort_rank<NT>(c, P);
    return;
  }
  for (int b = threadIdx.x; b <= kCodeBins; b += NT) start[b] = 0;
  lds_barrier();
  for (int k = threadIdx.x; k < nc; k += NT) atomicAdd(&start[mcode - bf16_code(c[k].x)], 1);
  lds_barrier();
  // exclusive scan of the counts, code below the maximum ascending (value
  // descending); every thread owns kCodeBins / NT consecutive codes
  constexpr int PER = kCodeBins / NT;
  static_assert(kCodeBins % NT == 0, "codes per thread");
  int own[PER];
  int sum = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    own[q] = start[threadIdx.x * PER + q];
    sum += own[q];
  }
  int total = 0;
  int before = block_scan_incl<NT, int>(sum, L.red_i, total) - sum;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int b = threadIdx.x * PER + q;
    start[b] = before;
    cur[b] = before;
    before += own[q];
  }
  if (threadIdx.x == 0) start[kCodeBins] = total;
  lds_barrier();
  for (int k = threadIdx.x; k < nc; k += NT) {
    const Cand e = c[k];
    tmp[atomicAdd(&cur[mcode - bf16_code(e.x)], 1)] = e;
  }
  lds_barrier();
  // equal codes are equal values: their order is the index order
  for (int q = threadIdx.x; q < nc; q += NT) {
    const Cand e = tmp[q];
    const int b = mcode - bf16_code(e.x);
    const int s0 = start[b], s1 = start[b + 1];
    int below = 0;
    for (int t = s0; t < s1; ++t) below += tmp[t].idx < e.idx ? 1 : 0;
    c[s0 + below] = e;
  }
  lds_barrier();
}

// When the survivors fit in the candidate buffer (the usual case: top-p
// keeps a small head of the order) they are gathered into LDS and sorted
// into rank order (bitonic; key descending, index ascending). The own draw
// and the residual draw are then scans over that list. Returns n, the
// entries c[0 .. n) of L.c.cand.
template <typename E, int NT, typename Pred>
__device__ __forceinline__ int gather_sorted(const E* __restrict__ x, int V, int count, Pred keep, SampledLds<NT>& L) {
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
  sort_rank<NT>(c, P);
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

// Survivor set of a sampled row whose cut the captured head did not decide,
// by the sampled path's whole-row locator (several passes over the row,
// which stays in the caches); the survivors are listed in rank order with
// their weights when they fit the candidate buffer, else the own draw is
// located directly. Out of line: the common path keeps its registers.
template <typename E, int NT>
__device__ __noinline__ void slow_support(const E* __restrict__ row, int V, float mx, double Td, int top_k,
                                          double top_p, double min_p, double u, SampledLds<NT>& L, Support& s,
                                          bool& listed, int& own) {
  RadixLocator<E, NT> fl(L, row, V, mx, Td);
  s = support(fl, V, top_k, top_p, min_p);
  listed = s.n <= kCand;
  own = 0;
  if (listed) {
    const Support sv = s;
    gather_sorted<E, NT>(row, V, sv.n, [&](int e, float xv) { return in_support(ord_ukey(xv), e, sv); }, L);
    // the locator is done with the union u: the list's weights go there
    double* wl = reinterpret_cast<double*>(&L.u);
    const Cand* c = L.c.cand;
    for (int k = threadIdx.x; k < sv.n; k += NT) wl[k] = weight(c[k].x, mx, Td);
    lds_barrier();
  } else {
    Pick p = fl.by_mass(u * s.w, true);
    if (p.rank >= s.n) p = fl.by_count(s.n);
    own = p.idx;
  }
}

// One row of the batch: its token, acceptance and word. `after_stream` is
// called once the target row has been streamed, with true when the row's
// remaining work is long (a sampled target).
template <typename E, int NT, int U, typename Hook>
__device__ __forceinline__ void prob_kernel_row(const VerifyArgs& a, const ProbArgs& pa, uint32_t tag, int r,
                                                SampledLds<NT>& L, Hook after_stream) {
  const E* __restrict__ row = static_cast<const E*>(a.logits) + static_cast<int64_t>(r) * a.ld;
  const int own = a.owner[r];
  const ReqParams q = load_params(a, own);
  const float Tq = pa.draft_temperature[(own >= 0 && own < a.B) ? own : 0];
  const RowMeta m = load_meta(a, r, own);
  const float T = q.T;
  int top_k = q.top_k;
  float top_p = q.top_p;
  float min_p = q.min_p;
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

  int token = 0;
  bool accept = false;
  const bool sampled = m.req >= 0 && T > 0.f && T < INFINITY;
  float fast_tau = -INFINITY;
  double fast_wtot = 0.0, fast_c = 0.0;
  VmPlan fast_plan{};
  float mx = 0.f;
  if (!sampled) {
    // the target row's maximum and lowest arg-max
    RowPartial p;
    partial_init(p);
    QueueKeep<E, U> keep{};
    constexpr float kLog2e = 1.4426950408889634f;
    stream_row<E, NT, U, false, QueueKeep<E, U>, NoHook, true>(row, a.V, kLog2e, INFINITY, 0, p, keep);
    after_stream(false);
    const RowStats st = finish_row_lean<E, NT, U, false>(p, L.ls, keep, row, a.V);
    token = st.argmax == INT32_MAX ? 0 : st.argmax;
    if (!(st.max < INFINITY) || st.argmax == INT32_MAX || st.sum != st.sum) bits |= VSV_FLAG_LOGITS;
  } else {
    // the sampled path's first pass: maximum, streamed total weight at
    // scale c = log2(e) / T, and the vector-maximum codes for the capture
    const float c = 1.4426950408889634f / T;
    RowPartial p;
    partial_init(p);
    const VmPlan plan = stream_sampled<E, NT, SampledDepth<E>::kPass1>(row, a.V, c, p, L);
    after_stream(true);
    const NoKeep nk;
    const RowStats st = finish_row_lean<E, NT, U, false>(p, L.ls, nk, row, a.V);
    mx = st.max;
    if (!(mx < INFINITY) || !(mx > -INFINITY) || !(st.sum > 0.0) || !(st.sum < INFINITY)) bits |= VSV_FLAG_LOGITS;
    if (!(bits & VSV_FLAG_LOGITS)) {
      // capture threshold as the sampled path takes it
      const bool tk0 = top_k > 0 && top_k < a.V;
      float tau = -INFINITY;
      if (tk0) {
        tau = capture_threshold<E, NT>(L, plan, mx, -INFINITY, top_k, true);
      } else {
        float dcap = T * kZcap;
        if (min_p > 0.f && top_p >= 1.f) {
          const float dm = static_cast<float>(-static_cast<double>(T) * log(static_cast<double>(min_p))) * 1.0001f +
                           1e-6f;
          dcap = fminf(dcap, dm);
        }
        tau = capture_threshold<E, NT>(L, plan, mx, (dcap < INFINITY) ? mx - dcap : -INFINITY, kCapVec, false);
      }
      fast_tau = tau;
      fast_wtot = st.sum * exp2(static_cast<double>(st.mref) - static_cast<double>(mx) * static_cast<double>(c));
      fast_c = static_cast<double>(c);
      fast_plan = plan;
    }
  }

  const bool live = m.req >= 0 && !(bits & VSV_FLAG_LOGITS);
  if (live && sampled) {
    const double Td = static_cast<double>(T);
    const Cand* c = L.c.cand;
    Support s{0, 0.0, 0u, 0};
    bool listed = false;
    const bool tk = top_k > 0 && top_k < a.V;
    // Fast path: every element >= tau captured into the candidate list
    // (a complete head of the rank order), sorted into rank order; the
    // streamed total with the candidates' share replaced by their exact
    // weights. The survivor set is then a prefix of the list whenever its
    // cut lies inside the list.
    if (fast_tau > -INFINITY && capture_row<E, NT>(row, a.V, fast_tau, fast_plan, L)) {
      const int nc = min(L.ncand, kCand);
      double corr = 0.0;
      const double dc = c_gap(fast_c, Td);
      for (int k = threadIdx.x; k < nc; k += NT) corr += stream_gap(c[k].x, mx, weight(c[k].x, mx, Td), dc);
      const double W = fast_wtot + block_reduce<NT>(corr, SumOp(), L.red_d);
      rank_candidates<E, NT>(L, nc, mx);
      // the candidates' weights, once, in LDS (the union u is free again)
      double* wl = reinterpret_cast<double*>(&L.u);
      for (int k = threadIdx.x; k < nc; k += NT) wl[k] = weight(c[k].x, mx, Td);
      lds_barrier();
      auto wt = [&](int k) { return wl[k]; };
      int n = 0;
      if (tk) {
        if (top_k <= nc) {
          n = top_k;
          if (top_p < 1.f) {
            double s1 = 0.0;
            for (int q = threadIdx.x; q < top_k; q += NT) s1 += wt(q);
            const double W1 = block_reduce<NT>(s1, SumOp(), L.red_d);
            n = scan_pick<NT>(top_k, wt, static_cast<double>(top_p), L, false, W1, true) + 1;
          }
        }
      } else if (top_p < 1.f) {
        n = scan_pick<NT>(nc, wt, static_cast<double>(top_p), L, false, W, false) + 1;
      } else if (min_p > 0.f) {
        n = nc;   // min-p alone: its cut must lie inside the list (checked below)
      }
      if (n > 0 && min_p > 0.f) {
        // min-p keeps the prefix with (x - m) / T >= ln(min_p)
        const double lm = log(static_cast<double>(min_p));
        int cnt = 0;
        for (int q = threadIdx.x; q < n; q += NT)
          cnt += ((static_cast<double>(c[q].x) - static_cast<double>(mx)) / Td >= lm) ? 1 : 0;
        const int keep_n = block_reduce<NT>(cnt, SumOp(), L.red_i);
        if (!tk && top_p >= 1.f && keep_n == nc) n = 0;   // the cut may lie below the list
        else n = keep_n > 0 ? keep_n : 1;
      }
      if (n > 0) {
        double sn = 0.0;
        for (int q = threadIdx.x; q < n; q += NT) sn += wt(q);
        const double w = block_reduce<NT>(sn, SumOp(), L.red_d);
        s = Support{n, w, ord_ukey(c[n - 1].x), c[n - 1].idx};
        listed = true;
      }
    }
    lds_barrier();
    double u, ua;
    prob_uniforms(a.seed, a.offset, m.req, m.j, u, ua);
    if (!listed) {
      if (threadIdx.x == 0 && a.slow_rows) atomicAdd(a.slow_rows, 1);
      slow_support<E, NT>(row, a.V, mx, Td, top_k, static_cast<double>(top_p), static_cast<double>(min_p), u, L, s,
                          listed, token);
    }
    const int n = s.n;
    double* wl = reinterpret_cast<double*>(&L.u);   // listed: the n weights in rank order
    if (listed) {
      const int k = scan_pick<NT>(n, [&](int k) { return wl[k]; }, u, L);
      token = c[k < 0 ? 0 : k].idx;
    }
    if (m.j < m.K) {
      const E* __restrict__ y = static_cast<const E*>(pa.draft_logits) + static_cast<int64_t>(r - m.req) * pa.dld;
      const double Tdq = (Tq >= 0.f && Tq < INFINITY) ? static_cast<double>(Tq) : 0.0;
      DraftLaw q;
      if (!draft_law_stream<E, NT, U>(y, a.V, Tdq, L, q)) {
        bits |= VSV_FLAG_LOGITS;
      } else {
        const int d = m.draft;
        if (d >= 0 && d < a.V) {
          const float xd = Elem<E>::at(row, d);
          const double pd = in_support(ord_ukey(xd), d, s) ? weight(xd, mx, Td) / s.w : 0.0;
          accept = ua * q.q(Elem<E>::at(y, d), d) < pd;
        }
        int t = -1;
        if (listed) {
          // residual masses over the list, in place of the weights; the
          // draft row's values are gathered kResBatch at a time per thread
          constexpr int kResBatch = 4;
          for (int base = 0; base < n; base += NT * kResBatch) {
            float yv[kResBatch];
#pragma unroll
            for (int b = 0; b < kResBatch; ++b) {
              const int k = base + b * NT + static_cast<int>(threadIdx.x);
              yv[b] = k < n ? Elem<E>::at(y, c[k].idx) : 0.f;
            }
#pragma unroll
            for (int b = 0; b < kResBatch; ++b) {
              const int k = base + b * NT + static_cast<int>(threadIdx.x);
              if (k < n) {
                const double r = wl[k] / s.w - q.q(yv[b], c[k].idx);
                wl[k] = r > 0.0 ? r : 0.0;
              }
            }
          }
          lds_barrier();
          const int k = scan_pick<NT>(n, [&](int k) { return wl[k]; }, u, L);
          if (k >= 0) t = c[k].idx;
        } else {
          t = residual_draw<E, NT>(row, y, a.V, mx, Td, s, q, u, L);
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
    if (r != a.withheld_row) store_agent64(a.ws_row + r, tagged(tag, word));
  }
}

// Rows come from the persistent row queue (row_queue.hpp), in row order.
template <typename E, int NT, int U>
// two workgroups per CU (4 waves per SIMD): at most 128 VGPRs
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) void verify_probabilistic_kernel(
    VerifyArgs a, ProbArgs pa) {
  __shared__ SampledLds<NT> L;
  const uint32_t tag = call_tag(a);
  row_queue_loop<NT, false>(a, tag, L, [&](int r, auto hook) { prob_kernel_row<E, NT, U>(a, pa, tag, r, L, hook); });
}

template <typename E>
static hipError_t launch_probabilistic_t(VerifyArgs a, const ProbArgs& p, hipStream_t s) {
  static int cached[64];
  int dev = 0, grid = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
    if (cached[dev] <= 0)
      cached[dev] = resident_groups(verify_probabilistic_kernel<E, kVerifyThreads, SampledDepth<E>::kGreedy>,
                                    kVerifyThreads, a.cus);
    grid = cached[dev];
  }
  if (grid <= 0) grid = 256;
  if (grid > a.R) grid = a.R;
  a.ordered = 0;
  verify_probabilistic_kernel<E, kVerifyThreads, SampledDepth<E>::kGreedy>
      <<<dim3(grid), dim3(kVerifyThreads), 0, s>>>(a, p);
  return hipGetLastError();
}

hipError_t launch_verify_probabilistic(const VerifyArgs& a, const ProbArgs& p, hipStream_t s) {
  return a.dtype == VSV_BF16 ? launch_probabilistic_t<uint16_t>(a, p, s) : launch_probabilistic_t<float>(a, p, s);
}

}  // namespace vsv
