// One-pass streaming statistics of a vocab-wide logits row, computed by one
// workgroup: maximum, lowest arg-max, log-sum-exp of x * c and (for relaxed
// acceptance) the rank of one token.
//
// Each thread walks 16-byte vectors tid, tid + NT, ... (a wave reads 1 KiB
// contiguous per load instruction), so its own elements arrive in increasing
// index order. Per group of U vectors it takes the group max (v_max3 chains)
// and, when that max beats its running best, keeps the group's raw vectors in
// registers, so the arg-max lane is found at the end without reading the row
// again. Every element's exp2(x*c - mc) is summed in float32 within its group
// (a short tree) and the group sums accumulate in float64; mc is a per-thread
// exponent reference held at an integer (log2 units) just above the thread's
// running max, so every rescale is an exact power of two and the largest
// terms carry the smallest rounding.
#pragma once

#include "device.hpp"

namespace vsv {

struct RowPartial {
  float best;   // largest value seen (-inf if none)
  int bpos;     // where it was first seen: see bvec
  int bvec;     // 0: bpos is its element index; 1: bpos is the element index
                // of the 16-byte vector holding it; 2: bpos is the vector
                // index of the first vector of the thread's group holding it
                // (whose data the stream kept, see GroupKeep)
  float mc;     // exponent reference (log2 domain, integer-valued once set)
  double s;     // sum of exp2(x*c - mc)
  int rank;     // elements ordered before token d (relaxed acceptance)
  int bad;      // a NaN was seen where the IEEE maximum (kMax3) would hide it
};

struct RowResult {
  float max;     // row maximum
  int argmax;    // lowest index attaining it (INT32_MAX if no finite value)
  double lse;    // log(sum exp(x * c * ln2)) in natural units
  int rank;      // number of elements ordered before d
  double sum;    // sum of exp2(x * c - mref)
  float mref;    // exponent reference of `sum`
};

// What finish_row combines across threads: the best value and its lowest
// index, the exponent reference and the sum relative to it, the rank count.
struct RowRed {
  double s;
  float best;
  int idx;
  float mc;
  int rank;
};

// LDS for finish_row: one partial per wave.
template <int NT> struct RowScratch {
  RowRed r[NT / kWave];
};

// Registers holding the raw vectors of the thread's best group (arg-max
// rows), or nothing.
struct NoKeep {
  static constexpr bool kOn = false;
  static constexpr bool kReload = false;
};
template <int U> struct GroupKeep {
  static constexpr bool kOn = true;
  static constexpr bool kReload = false;
  u32x4 w[U];
};
// The stream keeps no vectors: the few lanes whose best group holds the
// block maximum read that group again at the end (one load round trip)
// instead of every lane copying a group into registers whenever its best
// improves.
struct ReloadKeep {
  static constexpr bool kOn = false;
  static constexpr bool kReload = true;
};
// Greedy rows inside the persistent sampled and probabilistic kernels:
// bfloat16 rows, whose stream is bound by its vector instructions, drop the
// per-group copies and read the best group again; float32 rows keep it
// (their stream is not, and the extra round trip would lengthen the rows
// that end a launch).
template <typename E, int U> struct QueueKeepT { using type = GroupKeep<U>; };
template <int U> struct QueueKeepT<uint16_t, U> { using type = ReloadKeep; };
template <typename E, int U> using QueueKeep = typename QueueKeepT<E, U>::type;

__device__ __forceinline__ void partial_init(RowPartial& p) {
  p.best = -INFINITY;
  p.bpos = INT32_MAX;
  p.bvec = 0;
  p.mc = -FLT_MAX;
  p.s = 0.0;
  p.rank = 0;
  p.bad = 0;
}

// Raise the reference to ceil(vmax * c) if vmax * c exceeds it; the sum is
// rescaled by an exact power of two. Non-finite maxima leave it alone (such
// rows are flagged).
__device__ __forceinline__ void partial_rebase(RowPartial& p, float vmax, float c) {
  const float y = vmax * c;
  if (y > p.mc && y < FLT_MAX) {
    const float nm = ceilf(y);
    p.s = (p.mc > -FLT_MAX) ? ldexp(p.s, static_cast<int>(fmaxf(p.mc - nm, -2000.f))) : 0.0;
    p.mc = nm;
  }
}

// Largest power of two not above n (n >= 1).
constexpr int pow2_floor(int n) { return n < 2 ? 1 : 2 * pow2_floor(n / 2); }

// Pairwise sum of n floats: a power of two folds its upper half onto its
// lower half until one value is left; any other n sums its largest
// power-of-two prefix and the rest separately.
template <int n>
__device__ __forceinline__ float tree_sum(float* e) {
  static_assert(n >= 1, "at least one term");
  constexpr int p = pow2_floor(n);
  if constexpr (p != n) {
    return tree_sum<p>(e) + tree_sum<n - p>(e + p);
  } else {
#pragma unroll
    for (int w = n / 2; w >= 1; w /= 2)
#pragma unroll
      for (int k = 0; k < w; ++k) e[k] = e[k] + e[k + w];
    return e[0];
  }
}

// One element outside the row's 16-byte body. A head element (before the
// body, kHead) has a lower index than every body element, so it also takes
// the thread's best when it only ties it: it may be reduced after the body
// and still keep the lowest index of the maximum.
template <bool kRank, bool kHead = false>
__device__ __forceinline__ void take_scalar(RowPartial& p, float x, int e, float c, float xd, int d) {
  if (kHead ? (x >= p.best) : (x > p.best)) {
    p.best = x;
    p.bpos = e;
    p.bvec = 0;
  }
  partial_rebase(p, x, c);
  p.s += static_cast<double>(fast_exp2(fmaf(x, c, -p.mc)));
  p.bad |= (x != x) ? 1 : 0;
  if (kRank) p.rank += (x > xd || (x == xd && e < d)) ? 1 : 0;
}

// Decode one 16-byte vector into f and return its maximum. kMax3 takes the
// IEEE maximum (NaN propagates, -0 < +0), which gfx950 folds three operands
// at a time into v_maximum3_f32 with no NaN-quieting step per operand; only
// callers whose rows are flagged anyway when they hold a NaN, and who
// compare the result with ==, use it.
template <typename E, bool kMax3 = false>
__device__ __forceinline__ float vec_max(const u32x4& w, float* f) {
  constexpr int N = Elem<E>::kVec;
  Elem<E>::decode(w, f);
  float vmax = f[0];
#pragma unroll
  for (int k = 1; k < N; ++k) vmax = kMax3 ? __builtin_elementwise_maximum(vmax, f[k]) : fmaxf(vmax, f[k]);
  return vmax;
}

// A single vector (the sampled stream's last group).
template <typename E, bool kRank>
__device__ __forceinline__ void take_vector(RowPartial& p, const u32x4& w, int e0, float c, float xd, int d) {
  constexpr int N = Elem<E>::kVec;
  float f[N];
  const float vmax = vec_max<E>(w, f);
  const bool gt = vmax > p.best;
  p.best = gt ? vmax : p.best;
  p.bpos = gt ? e0 : p.bpos;
  p.bvec = gt ? 1 : p.bvec;
  partial_rebase(p, vmax, c);
  const float nmc = -p.mc;
  float e[N];
#pragma unroll
  for (int k = 0; k < N; ++k) e[k] = fast_exp2(fmaf(f[k], c, nmc));
  p.s += static_cast<double>(tree_sum<N>(e));
  if (kRank) {
    if (vmax >= xd) {
#pragma unroll
      for (int k = 0; k < N; ++k) p.rank += (f[k] > xd || (f[k] == xd && e0 + k < d)) ? 1 : 0;
    }
  }
}

struct NoCapture {
  __device__ __forceinline__ void operator()(int, float) const {}
};

// A group of U vectors of one thread: one best/rescale update for the group.
// `cap(u, vmax)` sees each vector's max before the exponentials are summed.
// kPartial: the group is a row's partial last one, and its vectors at or
// beyond nvec (loaded duplicates or zeros) count as -inf; other groups carry
// no masking code at all.
template <typename E, int U, int NT, bool kRank, bool kPartial = false, typename Keep = NoKeep,
          typename Cap = NoCapture, bool kMax3 = false>
__device__ __forceinline__ void take_group(RowPartial& p, const u32x4* w, int v, int head, float c, float xd, int d,
                                           Keep& keep, int nvec = 0, Cap cap = Cap()) {
  constexpr int N = Elem<E>::kVec;
  float f[U][N];
  float vmx[U];
  float gmax = -INFINITY;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    vmx[u] = vec_max<E, kMax3>(w[u], f[u]);
    if (kPartial && v + u * NT >= nvec) {
      vmx[u] = -INFINITY;
#pragma unroll
      for (int k = 0; k < N; ++k) f[u][k] = -INFINITY;
    }
    gmax = kMax3 ? __builtin_elementwise_maximum(gmax, vmx[u]) : fmaxf(gmax, vmx[u]);
  }
  // the IEEE maximum carries a NaN into the group max, which then neither
  // becomes the best nor sets the exponent reference: remember it instead
  if constexpr (kMax3) p.bad |= (gmax != gmax) ? 1 : 0;
#pragma unroll
  for (int u = 0; u < U; ++u) cap(u, vmx[u]);
  const bool gt = gmax > p.best;
  p.best = gt ? gmax : p.best;
  p.bpos = gt ? v : p.bpos;      // group: first vector index
  p.bvec = gt ? 2 : p.bvec;
  if constexpr (Keep::kOn) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      keep.w[u].x = gt ? w[u].x : keep.w[u].x;
      keep.w[u].y = gt ? w[u].y : keep.w[u].y;
      keep.w[u].z = gt ? w[u].z : keep.w[u].z;
      keep.w[u].w = gt ? w[u].w : keep.w[u].w;
    }
  }
  partial_rebase(p, gmax, c);
  const float nmc = -p.mc;
  float e[U * N];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int k = 0; k < N; ++k) e[u * N + k] = fast_exp2(fmaf(f[u][k], c, nmc));
  p.s += static_cast<double>(tree_sum<U * N>(e));
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (kRank) {
      const int e0 = head + (v + u * NT) * N;
      if (vmx[u] >= xd && (!kPartial || v + u * NT < nvec)) {
#pragma unroll
        for (int k = 0; k < N; ++k) p.rank += (f[u][k] > xd || (f[u][k] == xd && e0 + k < d)) ? 1 : 0;
      }
    }
  }
}

struct NoHook {
  __device__ __forceinline__ void operator()() const {}
};

// Issue the loads of group h: vectors h*U*NT + tid + u*NT, u < U. Addresses
// are clamped to the row's last vector instead of predicated, so no load sits
// behind a branch; the compiler can then count the loads in flight and wait
// for exactly the group it reduces next (a predicated load makes it wait for
// every load, including the prefetch just issued). Clamped duplicates are
// never reduced. Requires nvec >= 1.
template <int NT, int U>
__device__ __forceinline__ void load_group(u32x4* dst, const u32x4* __restrict__ vp, int h, int nvec) {
  const int base = h * (U * NT) + static_cast<int>(threadIdx.x);
#pragma unroll
  for (int u = 0; u < U; ++u) dst[u] = load_stream(vp + min(base + u * NT, nvec - 1));
}

// Cache policy of a buffer load: 0 normal, 2 nontemporal.
constexpr int kLoadNormal = 0;
constexpr int kLoadStream = 2;

// The same group through a buffer resource over the row's nvec body
// vectors: the lane's byte offset is fixed and the group's is uniform (a
// scalar offset), so a load costs no vector address arithmetic. Vectors
// past the body read as zero without touching memory; the partial group is
// reduced with those vectors masked.
template <int NT, int U, int kAux>
__device__ __forceinline__ void load_group_rsrc(u32x4* dst, __amdgpu_buffer_rsrc_t rsrc, int h) {
  const int lane_off = static_cast<int>(threadIdx.x) * 16;
#pragma unroll
  for (int u = 0; u < U; ++u)
    dst[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rsrc, lane_off, (h * (U * NT) + u * NT) * 16, kAux));
}

// Buffer resource over n 16-byte vectors at p (nothing when n is 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t vec_rsrc(const void* p, int n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, n * 16, 0x00020000);
}


// Stream row[0 .. V) into this thread's partial. c = log2(e) / T. `hook` runs
// once, right after the first group's loads are issued, so loads it issues
// overlap the stream instead of trailing it. `keep` receives the thread's
// best group (GroupKeep) or is ignored (NoKeep).
template <typename E, int NT, int U, bool kRank, typename Keep = NoKeep, typename Hook = NoHook, bool kMax3 = false>
__device__ __forceinline__ void stream_row(const E* __restrict__ row, int V, float c, float xd, int d,
                                           RowPartial& p, Keep& keep, Hook hook = Hook()) {
  constexpr int N = Elem<E>::kVec;
  const int tid = threadIdx.x;
  const uintptr_t addr = reinterpret_cast<uintptr_t>(row);
  int head = static_cast<int>(((16u - (addr & 15u)) & 15u) / sizeof(E));
  if (head > V) head = V;
  const int nvec = (V - head) / N;
  const int body_end = head + nvec * N;
  const __amdgpu_buffer_rsrc_t rsrc = vec_rsrc(row + head, nvec);

  // Full groups of U vectors per thread, two buffers in turn: while one
  // group is reduced the next one's loads are in flight. The group after the
  // last full one is the partial group (possibly empty), reduced with its
  // missing vectors masked.
  constexpr int G = U * NT;
  const int nfull = nvec / G;
  if (nvec > 0) {
    u32x4 a[U], b[U];
    load_group_rsrc<NT, U, kLoadStream>(a, rsrc, 0);
    hook();
    int g = 0;
    for (; g + 2 <= nfull; g += 2) {
      load_group_rsrc<NT, U, kLoadStream>(b, rsrc, g + 1);
      take_group<E, U, NT, kRank, false, Keep, NoCapture, kMax3>(p, a, g * G + tid, head, c, xd, d, keep);
      load_group_rsrc<NT, U, kLoadStream>(a, rsrc, g + 2);
      take_group<E, U, NT, kRank, false, Keep, NoCapture, kMax3>(p, b, (g + 1) * G + tid, head, c, xd, d, keep);
    }
    if (g < nfull) {
      load_group_rsrc<NT, U, kLoadStream>(b, rsrc, g + 1);
      take_group<E, U, NT, kRank, false, Keep, NoCapture, kMax3>(p, a, g * G + tid, head, c, xd, d, keep);
      take_group<E, U, NT, kRank, true, Keep, NoCapture, kMax3>(p, b, nfull * G + tid, head, c, xd, d, keep, nvec);
    } else {
      take_group<E, U, NT, kRank, true, Keep, NoCapture, kMax3>(p, a, nfull * G + tid, head, c, xd, d, keep, nvec);
    }
  } else {
    hook();
  }

  if (tid < head) take_scalar<kRank, true>(p, Elem<E>::at(row, tid), tid, c, xd, d);
  const int tail = V - body_end;
  if (tid < tail) take_scalar<kRank>(p, Elem<E>::at(row, body_end + tid), body_end + tid, c, xd, d);
}

// Power-of-two rescale of a partial sum from reference mc to m >= mc (a
// thread that saw nothing holds mc = -FLT_MAX and contributes 0).
__device__ __forceinline__ double rebase_sum(double s, float mc, float m) {
  return (mc > -FLT_MAX) ? ldexp(s, static_cast<int>(fmaxf(mc - m, -2000.f))) : 0.0;
}

__device__ __forceinline__ RowRed combine(const RowRed& a, const RowRed& b) {
  RowRed r;
  r.best = fmaxf(a.best, b.best);
  r.idx = (a.best > b.best) ? a.idx : (b.best > a.best) ? b.idx : min(a.idx, b.idx);
  r.mc = fmaxf(a.mc, b.mc);
  r.s = rebase_sum(a.s, a.mc, r.mc) + rebase_sum(b.s, b.mc, r.mc);
  r.rank = a.rank + b.rank;
  return r;
}

// This thread's lowest index of its best value: the scalar position, or the
// first match in the kept group (vectors bpos + u * STRIDE, u < U, of the
// row's 16-byte-aligned body, which starts `head` elements in and holds
// `nvec` vectors). INT32_MAX if the thread saw no finite value.
template <typename E, int STRIDE, int U, typename Keep>
__device__ __forceinline__ int lane_argmax(const RowPartial& p, const Keep& keep, int head, int nvec) {
  static_assert(Keep::kOn, "the arg-max lane is found in the kept group");
  constexpr int N = Elem<E>::kVec;
  int idx = INT32_MAX;
  if (p.best > -INFINITY) {
    if (p.bvec == 2) {
#pragma unroll
      for (int u = U - 1; u >= 0; --u) {
        const int q = p.bpos + u * STRIDE;
        float f[N];
        Elem<E>::decode(keep.w[u], f);
#pragma unroll
        for (int k = N - 1; k >= 0; --k) idx = (q < nvec && f[k] == p.best) ? head + q * N + k : idx;
      }
    } else {
      idx = p.bpos;
    }
  }
  return idx;
}

// The partial of a whole wave (every lane receives it; every lane must be
// active): the largest value,
// the lowest index holding it, every sum rebased to the largest exponent
// reference and added, the rank counts added.
template <bool kRank = true>
__device__ __forceinline__ RowRed wave_red(const RowRed& r) {
  RowRed o;
  o.best = wave_all(r.best, MaxOp());
  o.idx = wave_all(r.best == o.best ? r.idx : INT32_MAX, MinOp());
  o.mc = wave_all(r.mc, MaxOp());
  o.s = wave_sum_f64(rebase_sum(r.s, r.mc, o.mc));
  o.rank = kRank ? wave_all(r.rank, SumOp()) : 0;
  return o;
}

// Combine the block's partials in one round (wave shuffles, one LDS slot per
// wave, one barrier). Every thread receives the result. With kArgmax, each
// thread first finds the lowest index of its best value in the group `keep`
// holds (or takes the scalar position); `row` and V locate that group.
template <typename E, int NT, int U, bool kRank, bool kArgmax, typename Keep>
__device__ __forceinline__ RowResult finish_row(const RowPartial& p, RowScratch<NT>& s, const Keep& keep,
                                                const E* __restrict__ row, int V) {
  constexpr int N = Elem<E>::kVec;
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;

  int idx = INT32_MAX;
  if constexpr (kArgmax) {
    const uintptr_t addr = reinterpret_cast<uintptr_t>(row);
    int head = static_cast<int>(((16u - (addr & 15u)) & 15u) / sizeof(E));
    if (head > V) head = V;
    idx = lane_argmax<E, NT, U>(p, keep, head, (V - head) / N);
  }
  RowRed r = wave_red<kRank>(RowRed{p.s, p.best, idx, p.mc, kRank ? p.rank : 0});
  if (lane == 0) s.r[w] = r;
  lds_barrier();
  r = s.r[0];
#pragma unroll
  for (int k = 1; k < NW; ++k) r = combine(r, s.r[k]);

  RowResult out;
  out.max = r.best;
  out.argmax = r.idx;
  out.rank = r.rank;
  out.sum = r.s;
  out.mref = r.mc;
  out.lse = 0.69314718055994530942 * (static_cast<double>(r.mc) + log2(r.s));
  return out;
}

// LDS for finish_row_lean: two rounds of one value per wave.
template <int NT> struct LeanScratch {
  float mx[NT / kWave];
  float mc[NT / kWave];
  float s[NT / kWave];
  int idx[NT / kWave];
  int rank[NT / kWave];
};

// What a workgroup's stream of (part of) a row leaves: its maximum, the
// lowest index holding it, the exponent reference and the sum of
// exp2(x * c - mref), the rank count.
struct RowStats {
  float max;
  int argmax;
  float mref;
  double sum;
  int rank;
};

// Block combination of the threads' partials in two rounds, with the least
// work per wave (every wave of a launch reaches it at about the same time,
// so its instructions add to the launch): round 1 takes the block maximum
// and exponent reference (every thread's reference is already an integer in
// log2 units, so sums rebase exactly); round 2 adds the rebased sums (float
// per wave: the terms are positive, so the wave sum's relative error stays
// below 64 float roundings; float64 across waves), and takes the lowest
// index of the maximum, which only lanes holding the block maximum search
// for in their kept group (NoKeep: no index). Every thread receives the
// result.
template <typename E, int NT, int U, bool kRank, typename Keep>
__device__ __forceinline__ RowStats finish_row_lean(const RowPartial& p, LeanScratch<NT>& sc, const Keep& keep,
                                                    const E* __restrict__ row, int V) {
  constexpr int N = Elem<E>::kVec;
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const float mw = wave_all(p.best, MaxOp());
  const float cw = wave_all(p.mc, MaxOp());
  if (lane == 0) {
    sc.mx[w] = mw;
    sc.mc[w] = cw;
  }
  lds_barrier();
  float m = sc.mx[0], mg = sc.mc[0];
#pragma unroll
  for (int k = 1; k < NW; ++k) {
    m = fmaxf(m, sc.mx[k]);
    mg = fmaxf(mg, sc.mc[k]);
  }
  int idx = INT32_MAX;
  if constexpr (Keep::kOn || Keep::kReload) {
    if (p.best == m) {
      const uintptr_t addr = reinterpret_cast<uintptr_t>(row);
      int head = static_cast<int>(((16u - (addr & 15u)) & 15u) / sizeof(E));
      if (head > V) head = V;
      const int nvec = (V - head) / N;
      if constexpr (Keep::kReload) {
        GroupKeep<U> again;
        if (p.bvec == 2) {
          const __amdgpu_buffer_rsrc_t rsrc = vec_rsrc(row + head, nvec);
#pragma unroll
          for (int u = 0; u < U; ++u)
            again.w[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       rsrc, (p.bpos + u * NT) * 16, 0, kLoadNormal));
        }
        idx = lane_argmax<E, NT, U>(p, again, head, nvec);
      } else {
        idx = lane_argmax<E, NT, U>(p, keep, head, nvec);
      }
    }
  }
  float sl = (p.mc > -FLT_MAX) ? static_cast<float>(ldexp(p.s, static_cast<int>(fmaxf(p.mc - mg, -2000.f)))) : 0.f;
  if (p.bad) sl = __builtin_nanf("");   // the row is flagged through its sum
  const float sw = wave_all(sl, SumOp());
  const int iw = wave_all(idx, MinOp());
  const int rw = kRank ? wave_all(p.rank, SumOp()) : 0;
  if (lane == 0) {
    sc.s[w] = sw;
    sc.idx[w] = iw;
    sc.rank[w] = rw;
  }
  lds_barrier();
  RowStats out{m, INT32_MAX, mg, 0.0, 0};
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    out.sum += static_cast<double>(sc.s[k]);
    out.argmax = min(out.argmax, sc.idx[k]);
    out.rank += sc.rank[k];
  }
  return out;
}

}  // namespace vsv
