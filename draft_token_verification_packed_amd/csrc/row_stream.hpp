// One-pass streaming statistics of a vocab-wide logits row, computed by one
// workgroup: maximum, lowest arg-max, log-sum-exp of x * scale and (for
// relaxed acceptance) the rank of one token.
//
// Each thread walks 16-byte vectors tid, tid + NT, ... (a wave reads 1 KiB
// contiguous per load instruction), so its own elements arrive in increasing
// index order. Per vector it takes the vector max (v_max3 chain), keeps the
// first vector whose max beats its running best (the exact lane is resolved
// once at the end by re-reading that vector), and adds exp2(x*c - mc) to two
// partial sums. mc is a per-thread exponent reference that is only moved
// when a value would exceed it by 2^24, so the rescale branch is rare.
#pragma once

#include "device.hpp"

namespace vsv {

struct RowPartial {
  float best;   // largest value seen (-inf if none)
  int bpos;     // element index of that value, or start of its vector
  int bvec;     // 1: bpos is a vector start still to be resolved
  float mc;     // exponent reference (log2 domain)
  float s0, s1; // sum of exp2(x*c - mc)
  int rank;     // elements ordered before token d (relaxed acceptance)
};

struct RowResult {
  float max;     // row maximum
  int argmax;    // lowest index attaining it (INT32_MAX if no finite value)
  double lse;    // log(sum exp(x / T)) in natural units
  int rank;      // number of elements ordered before d
};

__device__ __forceinline__ void partial_init(RowPartial& p) {
  p.best = -INFINITY;
  p.bpos = INT32_MAX;
  p.bvec = 0;
  p.mc = -FLT_MAX;
  p.s0 = 0.f;
  p.s1 = 0.f;
  p.rank = 0;
}

__device__ __forceinline__ void partial_rescale(RowPartial& p, float vmax, float c) {
  const float nm = vmax * c;
  const float sc = fast_exp2(p.mc - nm);
  p.s0 *= sc;
  p.s1 *= sc;
  p.mc = nm;
}

template <bool kRank>
__device__ __forceinline__ void take_scalar(RowPartial& p, float x, int e, float c, float xd, int d) {
  if (x > p.best) {
    p.best = x;
    p.bpos = e;
    p.bvec = 0;
  }
  if (fmaf(x, c, -p.mc) > 24.0f) partial_rescale(p, x, c);
  p.s0 += fast_exp2(fmaf(x, c, -p.mc));
  if (kRank) p.rank += (x > xd || (x == xd && e < d)) ? 1 : 0;
}

template <typename E, bool kRank>
__device__ __forceinline__ void take_vector(RowPartial& p, const u32x4& w, int e0, float c, float xd, int d) {
  constexpr int N = Elem<E>::kVec;
  float f[N];
  Elem<E>::decode(w, f);
  float vmax = f[0];
#pragma unroll
  for (int k = 1; k < N; ++k) vmax = fmaxf(vmax, f[k]);
  const bool gt = vmax > p.best;
  p.best = gt ? vmax : p.best;
  p.bpos = gt ? e0 : p.bpos;
  p.bvec = gt ? 1 : p.bvec;
  if (fmaf(vmax, c, -p.mc) > 24.0f) partial_rescale(p, vmax, c);
  const float nmc = -p.mc;
#pragma unroll
  for (int k = 0; k < N; k += 2) {
    p.s0 += fast_exp2(fmaf(f[k], c, nmc));
    p.s1 += fast_exp2(fmaf(f[k + 1], c, nmc));
  }
  if (kRank) {
    if (vmax >= xd) {
#pragma unroll
      for (int k = 0; k < N; ++k) p.rank += (f[k] > xd || (f[k] == xd && e0 + k < d)) ? 1 : 0;
    }
  }
}

// Stream row[0 .. V) into this thread's partial. c = log2(e) / T.
template <typename E, int NT, int U, bool kRank>
__device__ __forceinline__ void stream_row(const E* __restrict__ row, int V, float c, float xd, int d,
                                           RowPartial& p) {
  constexpr int N = Elem<E>::kVec;
  const int tid = threadIdx.x;
  const uintptr_t addr = reinterpret_cast<uintptr_t>(row);
  int head = static_cast<int>(((16u - (addr & 15u)) & 15u) / sizeof(E));
  if (head > V) head = V;
  const int nvec = (V - head) / N;
  const int body_end = head + nvec * N;

  if (tid < head) take_scalar<kRank>(p, Elem<E>::at(row, tid), tid, c, xd, d);

  const u32x4* __restrict__ vp = reinterpret_cast<const u32x4*>(row + head);
  int v = tid;
  for (; v + (U - 1) * NT < nvec; v += U * NT) {
    u32x4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = load_stream(vp + v + u * NT);
#pragma unroll
    for (int u = 0; u < U; ++u) take_vector<E, kRank>(p, w[u], head + (v + u * NT) * N, c, xd, d);
  }
  for (; v < nvec; v += NT) take_vector<E, kRank>(p, load_stream(vp + v), head + v * N, c, xd, d);

  const int tail = V - body_end;
  if (tid < tail) take_scalar<kRank>(p, Elem<E>::at(row, body_end + tid), body_end + tid, c, xd, d);
}

// Combine the block's partials. Every thread receives the result.
// `scr_f`, `scr_i` and `scr_d` each hold NT / 64 entries.
template <typename E, int NT>
__device__ __forceinline__ RowResult finish_row(const E* __restrict__ row, RowPartial& p, float* scr_f,
                                                int* scr_i, double* scr_d) {
  constexpr int N = Elem<E>::kVec;
  int idx = INT32_MAX;
  if (p.best > -INFINITY) {
    if (p.bvec) {
      float f[N];
      Elem<E>::decode(*reinterpret_cast<const u32x4*>(row + p.bpos), f);
#pragma unroll
      for (int k = N - 1; k >= 0; --k) idx = (f[k] == p.best) ? p.bpos + k : idx;
    } else {
      idx = p.bpos;
    }
  }
  RowResult r;
  r.max = block_reduce<NT>(p.best, MaxOp(), scr_f);
  r.argmax = block_reduce<NT>(p.best == r.max ? idx : INT32_MAX, MinOp(), scr_i);
  const float mref = block_reduce<NT>(p.mc, MaxOp(), scr_f);
  const double term = static_cast<double>(p.s0 + p.s1) *
                      exp2(static_cast<double>(p.mc) - static_cast<double>(mref));
  const double s = block_reduce<NT>(term, SumOp(), scr_d);
  r.lse = 0.69314718055994530942 * (static_cast<double>(mref) + log2(s));
  r.rank = block_reduce<NT>(p.rank, SumOp(), scr_i);
  return r;
}

}  // namespace vsv
