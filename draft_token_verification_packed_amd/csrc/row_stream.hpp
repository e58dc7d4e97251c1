// One-pass streaming statistics of a vocab-wide logits row, computed by one
// workgroup: maximum, lowest arg-max, log-sum-exp of x * c and (for relaxed
// acceptance) the rank of one token.
//
// Each thread walks 16-byte vectors tid, tid + NT, ... (a wave reads 1 KiB
// contiguous per load instruction), so its own elements arrive in increasing
// index order. Per group of U vectors it takes the group max (v_max3 chains)
// and remembers the first group whose max beats its running best; only the
// thread holding the row maximum re-reads that group at the end to find the
// exact lane. Every element's exp2(x*c - mc) is summed in float32 within its
// group (a short tree) and the group sums accumulate in float64; mc is a
// per-thread exponent reference held at an integer (log2 units) just above
// the thread's running max, so every rescale is an exact power of two and
// the largest terms carry the smallest rounding.
#pragma once

#include "device.hpp"

namespace vsv {

struct RowPartial {
  float best;   // largest value seen (-inf if none)
  int bpos;     // where it was first seen: see bvec
  int bvec;     // 0: bpos is its element index; 1: bpos is the element index
                // of the 16-byte vector holding it; 2: bpos is the vector
                // index of the first vector of the thread's group holding it
  float mc;     // exponent reference (log2 domain, integer-valued once set)
  double s;     // sum of exp2(x*c - mc)
  int rank;     // elements ordered before token d (relaxed acceptance)
};

struct RowResult {
  float max;     // row maximum
  int argmax;    // lowest index attaining it (INT32_MAX if no finite value)
  double lse;    // log(sum exp(x * c * ln2)) in natural units
  int rank;      // number of elements ordered before d
  double sum;    // sum of exp2(x * c - mref)
  float mref;    // exponent reference of `sum`
};

// LDS for finish_row: one slot per wave per reduced quantity.
template <int NT> struct RowScratch {
  float f[NT / kWave][2];
  int i[NT / kWave][2];
  double d[NT / kWave];
};

__device__ __forceinline__ void partial_init(RowPartial& p) {
  p.best = -INFINITY;
  p.bpos = INT32_MAX;
  p.bvec = 0;
  p.mc = -FLT_MAX;
  p.s = 0.0;
  p.rank = 0;
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

// Pairwise sum of n (a power of two) floats.
template <int n>
__device__ __forceinline__ float tree_sum(float* e) {
#pragma unroll
  for (int w = n / 2; w >= 1; w /= 2)
#pragma unroll
    for (int k = 0; k < w; ++k) e[k] = e[k] + e[k + w];
  return e[0];
}

template <bool kRank>
__device__ __forceinline__ void take_scalar(RowPartial& p, float x, int e, float c, float xd, int d) {
  if (x > p.best) {
    p.best = x;
    p.bpos = e;
    p.bvec = 0;
  }
  partial_rebase(p, x, c);
  p.s += static_cast<double>(fast_exp2(fmaf(x, c, -p.mc)));
  if (kRank) p.rank += (x > xd || (x == xd && e < d)) ? 1 : 0;
}

// Decode one 16-byte vector into f and return its maximum.
template <typename E>
__device__ __forceinline__ float vec_max(const u32x4& w, float* f) {
  constexpr int N = Elem<E>::kVec;
  Elem<E>::decode(w, f);
  float vmax = f[0];
#pragma unroll
  for (int k = 1; k < N; ++k) vmax = fmaxf(vmax, f[k]);
  return vmax;
}

// A single vector (the predicated last group).
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
template <typename E, int U, int NT, bool kRank, typename Cap = NoCapture>
__device__ __forceinline__ void take_group(RowPartial& p, const u32x4* w, int v, int head, float c, float xd, int d,
                                           Cap cap = Cap()) {
  constexpr int N = Elem<E>::kVec;
  float f[U][N];
  float vmx[U];
  float gmax = -INFINITY;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    vmx[u] = vec_max<E>(w[u], f[u]);
    gmax = fmaxf(gmax, vmx[u]);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) cap(u, vmx[u]);
  const bool gt = gmax > p.best;
  p.best = gt ? gmax : p.best;
  p.bpos = gt ? v : p.bpos;      // group: first vector index
  p.bvec = gt ? 2 : p.bvec;
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
      if (vmx[u] >= xd) {
#pragma unroll
        for (int k = 0; k < N; ++k) p.rank += (f[u][k] > xd || (f[u][k] == xd && e0 + k < d)) ? 1 : 0;
      }
    }
  }
}

struct NoHook {
  __device__ __forceinline__ void operator()() const {}
};

// Stream row[0 .. V) into this thread's partial. c = log2(e) / T. `hook` runs
// once, right after the first group's loads are issued, so loads it issues
// overlap the stream instead of trailing it.
template <typename E, int NT, int U, bool kRank, typename Hook = NoHook>
__device__ __forceinline__ void stream_row(const E* __restrict__ row, int V, float c, float xd, int d,
                                           RowPartial& p, Hook hook = Hook()) {
  constexpr int N = Elem<E>::kVec;
  const int tid = threadIdx.x;
  const uintptr_t addr = reinterpret_cast<uintptr_t>(row);
  int head = static_cast<int>(((16u - (addr & 15u)) & 15u) / sizeof(E));
  if (head > V) head = V;
  const int nvec = (V - head) / N;
  const int body_end = head + nvec * N;

  const u32x4* __restrict__ vp = reinterpret_cast<const u32x4*>(row + head);
  // Groups of U vectors per thread, software-pipelined: the loads of group
  // g + 1 are in flight while group g is reduced. Only the last group can be
  // partial; its loads and updates are predicated on the vector index.
  constexpr int G = U * NT;
  const int ngroups = (nvec + G - 1) / G;
  int v = tid;
  u32x4 cur[U];
  if (ngroups > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (ngroups > 1 || v + u * NT < nvec) cur[u] = load_stream(vp + v + u * NT);
  }
  hook();
  if (tid < head) take_scalar<kRank>(p, Elem<E>::at(row, tid), tid, c, xd, d);
  if (ngroups > 0) {
    for (int g = 1; g < ngroups; ++g) {
      u32x4 nxt[U];
      const int vn = v + G;
      const bool full = g + 1 < ngroups;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (full || vn + u * NT < nvec) nxt[u] = load_stream(vp + vn + u * NT);
      take_group<E, U, NT, kRank>(p, cur, v, head, c, xd, d);
#pragma unroll
      for (int u = 0; u < U; ++u) cur[u] = nxt[u];
      v = vn;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (v + u * NT < nvec) take_vector<E, kRank>(p, cur[u], head + (v + u * NT) * N, c, xd, d);
  }

  const int tail = V - body_end;
  if (tid < tail) take_scalar<kRank>(p, Elem<E>::at(row, body_end + tid), body_end + tid, c, xd, d);
}

// Combine the block's partials in two rounds (max and exponent reference;
// then arg-max index, sum and rank). Every thread receives the result. `row`
// is the streamed row: the thread holding the maximum re-reads its group.
template <typename E, int NT, int U, bool kRank, bool kArgmax = true>
__device__ __forceinline__ RowResult finish_row(RowPartial& p, RowScratch<NT>& s, const E* __restrict__ row) {
  constexpr int N = Elem<E>::kVec;
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;

  const float m1 = wave_reduce(p.best, MaxOp());
  const float m2 = wave_reduce(p.mc, MaxOp());
  if (lane == 0) {
    s.f[w][0] = m1;
    s.f[w][1] = m2;
  }
  __syncthreads();
  float mx = s.f[0][0], mref = s.f[0][1];
#pragma unroll
  for (int k = 1; k < NW; ++k) {
    mx = fmaxf(mx, s.f[k][0]);
    mref = fmaxf(mref, s.f[k][1]);
  }

  int idx = INT32_MAX;
  if (kArgmax && p.best == mx && mx > -INFINITY) {
    if (p.bvec == 2) {
      const uintptr_t addr = reinterpret_cast<uintptr_t>(row);
      const int head = static_cast<int>(((16u - (addr & 15u)) & 15u) / sizeof(E));
      const u32x4* vp = reinterpret_cast<const u32x4*>(row + head);
#pragma unroll
      for (int u = U - 1; u >= 0; --u) {
        float f[N];
        Elem<E>::decode(vp[p.bpos + u * NT], f);
#pragma unroll
        for (int k = N - 1; k >= 0; --k) idx = (f[k] == p.best) ? head + (p.bpos + u * NT) * N + k : idx;
      }
    } else if (p.bvec) {
      float f[N];
      Elem<E>::decode(*reinterpret_cast<const u32x4*>(row + p.bpos), f);
#pragma unroll
      for (int k = N - 1; k >= 0; --k) idx = (f[k] == p.best) ? p.bpos + k : idx;
    } else {
      idx = p.bpos;
    }
  }
  // both references are integers (or -FLT_MAX for a thread that saw nothing)
  const double term = (p.mc > -FLT_MAX) ? ldexp(p.s, static_cast<int>(fmaxf(p.mc - mref, -2000.f))) : 0.0;
  idx = wave_reduce(idx, MinOp());
  const double sw = wave_reduce(term, SumOp());
  const int rk = kRank ? wave_reduce(p.rank, SumOp()) : 0;
  if (lane == 0) {
    s.i[w][0] = idx;
    s.i[w][1] = rk;
    s.d[w] = sw;
  }
  __syncthreads();
  RowResult r;
  r.max = mx;
  r.argmax = s.i[0][0];
  r.rank = s.i[0][1];
  double sum = s.d[0];
#pragma unroll
  for (int k = 1; k < NW; ++k) {
    r.argmax = min(r.argmax, s.i[k][0]);
    r.rank += s.i[k][1];
    sum += s.d[k];
  }
  r.lse = 0.69314718055994530942 * (static_cast<double>(mref) + log2(sum));
  r.sum = sum;
  r.mref = mref;
  return r;
}

}  // namespace vsv
