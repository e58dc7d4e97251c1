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
// How: while streaming the row once (row_stream.hpp), each wave keeps the
// candidate tokens above a wave-uniform threshold in LDS. A 16-byte vector
// whose max clears the threshold is parked in the wave's ring with one
// ballot; full rings are drained in bulk into the wave's candidate buffer,
// and a full buffer is compacted with a 64-bin histogram that raises the
// threshold. Each wave's buffer therefore holds every element of the wave's
// share of the row above its final threshold, and the union holds every
// element above the largest of them. Afterwards a 1024-bin histogram of
// (count, float64 weight) over the union locates each cut; only the bin a
// cut falls in is gathered and sorted. When the candidates cannot decide
// (survivor set or draw beyond them, huge tie groups), an exact radix-select
// over the whole row decides instead, reading the row again.
#pragma once

#include "kernels.hpp"
#include "row_stream.hpp"

namespace vsv {

constexpr int kEW = 768;        // candidate slots per wave
constexpr int kRing = 128;      // parked vectors per wave
constexpr int kNB = 1024;       // histogram bins over the candidates
constexpr int kGather = 256;    // most elements one bin may hold
constexpr float kZcap = 10.0f;  // capture window below the running max, in units of T

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
  static_assert(NT >= kGather && NT <= 1024 && kNB % NT == 0, "one gathered element per thread");
  static_assert(sizeof(double) * kNB >= sizeof(double) * kGather, "weight views share storage");
  Cand elem[NW][kEW];
  union {
    struct {
      u32x4 v[NW][kRing];
      int e0[NW][kRing];
    } ring;
    struct {
      int cnt[kNB + 1];
      double mass[kNB + 1];
      union {
        double wbin[kNB];     // bfloat16 rows: weight of each bin's value
        double gpm[kGather];  // float32 rows: weight prefix of the gathered bin
      };
      Cand g[kGather];
      Cand gs[kGather];
    } post;
    struct {
      int cnt[256];
      double mass[256];
    } radix;
  } u;
  int whist[NW][64];
  float wtau[NW];
  int wn[NW];
  int wovf[NW];
  int mkey;
  int gn;
  int bi[4];
  double bd[4];
  int red_i[NW];
  double red_d[2 * NW];
  RowScratch<NT> rs;
  int row_next;  // the workgroup's next row (row queue)
  int last;      // this workgroup finished the call's last row
};

// Per-wave capture state; every lane holds the same values.
struct WaveCap {
  int ring_n;    // parked vectors
  int elem_n;    // candidates in the buffer
  float tau_w;   // threshold raised by compaction
  float tau;     // effective threshold, max(tau_w, running max - window)
  float dcap;    // capture window (x units)
  int ovf;       // the buffer could not hold the wave's candidates
  int kmin;      // compaction never keeps fewer candidates than this
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

// Keep only the wave's candidates at or above its current threshold
// (entries parked before the threshold last rose may lie below it).
template <int NT>
__device__ __forceinline__ void wave_filter(SampledLds<NT>& L, WaveCap& s) {
  const int lane = lane_id();
  Cand* buf = L.elem[wave_id()];
  int n = 0;
  for (int base = 0; base < s.elem_n; base += kWave) {
    const int q = base + lane;
    Cand e{-INFINITY, 0};
    if (q < s.elem_n) e = buf[q];
    const bool keep = q < s.elem_n && e.x >= s.tau;
    const uint64_t bal = __ballot(keep);
    wave_lds_sync();
    if (keep) buf[n + mbcnt(bal)] = e;   // n + rank <= q: reads of this chunk are done
    n += __popcll(bal);
    wave_lds_sync();
  }
  s.elem_n = n;
}

// Make room in the wave's buffer: drop entries below the threshold, and if
// more than `target` remain, raise the threshold (64 value bins between it
// and the wave's largest candidate) so that about `target` are kept.
// Returns false if nothing can be dropped.
template <int NT>
__device__ bool wave_compact(SampledLds<NT>& L, WaveCap& s, int target) {
  const int w = wave_id(), lane = lane_id();
  Cand* buf = L.elem[w];
  const int before = s.elem_n;
  wave_filter<NT>(L, s);
  if (s.elem_n <= target) return s.elem_n < before;
  // histogram range: the buffer's own values (the threshold may be far below)
  float hi = -INFINITY, lo = INFINITY;
  for (int q = lane; q < s.elem_n; q += kWave) {
    hi = fmaxf(hi, buf[q].x);
    lo = fminf(lo, buf[q].x);
  }
  hi = uni(wave_reduce(hi, MaxOp()));
  lo = uni(wave_reduce(lo, MinOp()));
  if (!(hi > lo) || !(hi - lo < INFINITY)) return s.elem_n < before;
  const float inv = 64.0f / (hi - lo);
  L.whist[w][lane] = 0;
  wave_lds_sync();
  for (int q = lane; q < s.elem_n; q += kWave) {
    int b = static_cast<int>((hi - buf[q].x) * inv);
    b = b < 0 ? 0 : (b > 63 ? 63 : b);
    atomicAdd(&L.whist[w][b], 1);
  }
  wave_lds_sync();
  const int c1 = L.whist[w][lane];
  const int incl = wave_inclusive_scan(c1);
  const uint64_t reach = __ballot(incl >= target);
  const int b = reach ? __builtin_ctzll(reach) : 63;
  // entries of bins 0 .. b-1 stay; refine bin b with 64 sub-bins so that the
  // kept count lands near the target instead of jumping a whole bin
  const int before_b = read_lane(incl - c1, b);
  const float bhi = hi - static_cast<float>(b) / inv;
  const float sinv = inv * 64.0f;
  L.whist[w][lane] = 0;
  wave_lds_sync();
  for (int q = lane; q < s.elem_n; q += kWave) {
    const float x = buf[q].x;
    const int bb = static_cast<int>((hi - x) * inv);
    if ((bb < 0 ? 0 : (bb > 63 ? 63 : bb)) != b) continue;
    int sb = static_cast<int>((bhi - x) * sinv);
    sb = sb < 0 ? 0 : (sb > 63 ? 63 : sb);
    atomicAdd(&L.whist[w][sb], 1);
  }
  wave_lds_sync();
  const int incl2 = before_b + wave_inclusive_scan(L.whist[w][lane]);
  const uint64_t reach2 = __ballot(incl2 >= target);
  int sbk = reach2 ? __builtin_ctzll(reach2) : 63;
  if (b == 63 && sbk == 63) sbk = 62;  // something must go
  // keep values >= lower edge of sub-bin sbk of bin b
  const float nt = bhi - static_cast<float>(sbk + 1) / sinv;
  if (nt > s.tau) {
    s.tau_w = fmaxf(s.tau_w, nt);
    s.tau = nt;
    wave_filter<NT>(L, s);
  }
  return s.elem_n < before;
}

// Move the parked vectors' elements at or above the threshold into the
// buffer. Lane l reads 32-bit word l % 4 of parked vector l / 4 (one or two
// elements), so a step covers 16 vectors with one compare, ballot and write
// per element; the words of four steps (64 vectors) are read together, so a
// batch costs a single LDS round trip. When a batch does not fit, the buffer
// is compacted first (which raises the threshold) and the batch re-tested.
template <typename E, int NT>
__device__ __forceinline__ void wave_drain(SampledLds<NT>& L, WaveCap& s) {
  constexpr int EPW = 4 / sizeof(E);   // elements per 32-bit word
  constexpr int kStep = kWave / 4;     // vectors per step
  constexpr int kBatch = 4;            // steps per batch
  constexpr int M = kBatch * EPW;      // elements per lane per batch
  const int w = wave_id(), lane = lane_id();
  if (s.ring_n == 0) return;
  wave_lds_sync();
  const int q = lane & 3, jl = lane >> 2;
  const uint32_t* ring = reinterpret_cast<const uint32_t*>(&L.u.ring.v[w][0]);
  for (int j0 = 0; j0 < s.ring_n; j0 += kStep * kBatch) {
    float x[M];
    int e[M];
    bool have[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int jj = j0 + b * kStep + jl;
      have[b] = jj < s.ring_n;
      const int j = min(jj, kRing - 1);
      const uint32_t word = ring[j * 4 + q];
      const int e0 = L.u.ring.e0[w][j] + q * EPW;
#pragma unroll
      for (int h = 0; h < EPW; ++h) {
        x[b * EPW + h] = EPW == 1 ? __uint_as_float(word)
                                  : __uint_as_float(h == 0 ? (word << 16) : (word & 0xFFFF0000u));
        e[b * EPW + h] = e0 + h;
      }
    }
    // steps past the ring's fill level hold nothing: skip them (uniform)
    const int steps = min(kBatch, (s.ring_n - j0 + kStep - 1) / kStep);
    auto count = [&]() {
      int n = 0;
#pragma unroll
      for (int i = 0; i < M; ++i)
        if (i / EPW < steps) n += __popcll(__ballot(have[i / EPW] && x[i] >= s.tau));
      return n;
    };
    if (s.elem_n + count() > kEW) {
      // A top-k row keeps only its top_k + 32: the k-th largest of the
      // elements seen so far can only rise, so it is a safe threshold, and
      // a high one parks far fewer vectors later. Other rows keep half.
      if (!wave_compact<NT>(L, s, s.kmin > 0 ? s.kmin : kEW / 2) || s.elem_n + count() > kEW) {
        s.ovf = 1;
        s.tau = INFINITY;  // stop capturing: this row goes to the exact path
        break;
      }
    }
#pragma unroll
    for (int i = 0; i < M; ++i) {
      if (i / EPW >= steps) break;
      const bool take = have[i / EPW] && x[i] >= s.tau;
      const uint64_t bal = __ballot(take);
      if (take) L.elem[w][s.elem_n + mbcnt(bal)] = Cand{x[i], e[i]};
      s.elem_n += __popcll(bal);
    }
  }
  s.ring_n = 0;
  wave_lds_sync();
}

// Park without draining; returns true when the ring needs a drain before
// the next park.
template <int NT>
__device__ __forceinline__ bool wave_park_only(SampledLds<NT>& L, WaveCap& s, const u32x4& v, int e0, float vmax,
                                               bool valid) {
  const bool take = valid && vmax >= s.tau;
  const uint64_t bal = __ballot(take);
  if (bal == 0) return false;
  const int w = wave_id();
  if (take) {
    const int pos = s.ring_n + mbcnt(bal);
    L.u.ring.v[w][pos] = v;
    L.u.ring.e0[w][pos] = e0;
  }
  s.ring_n += __popcll(bal);
  return s.ring_n > kRing - kWave;
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

// Append single elements (row head / tail) directly to the buffer.
template <int NT>
__device__ __forceinline__ void wave_take_scalar(SampledLds<NT>& L, WaveCap& s, float x, int e, bool valid) {
  const bool take = valid && x >= s.tau;
  const uint64_t bal = __ballot(take);
  if (bal == 0) return;
  const int n = __popcll(bal);
  if (s.elem_n + n > kEW && !wave_compact<NT>(L, s, s.kmin > 0 ? s.kmin : kEW / 2)) {
    s.ovf = 1;
    s.tau = INFINITY;
    return;
  }
  const bool take2 = valid && x >= s.tau;
  const uint64_t bal2 = __ballot(take2);
  if (s.elem_n + __popcll(bal2) > kEW) {
    s.ovf = 1;
    s.tau = INFINITY;
    return;
  }
  if (take2) L.elem[wave_id()][s.elem_n + mbcnt(bal2)] = Cand{x, e};
  s.elem_n += __popcll(bal2);
  wave_lds_sync();
}

// Starting threshold from the whole block's first group: every wave
// publishes its max before any reads it back.
template <int NT>
__device__ __forceinline__ void block_start_max(SampledLds<NT>& L, WaveCap& s, float lane_best) {
  const float wm = wave_reduce(lane_best, MaxOp());
  if (lane_id() == 0 && wm > -INFINITY) atomicMax(&L.mkey, ord_key(wm));
  lds_barrier();
  const float m = key_float(uni(L.mkey));
  const float t = m - s.dcap;
  if (t > s.tau) s.tau = t;
}

// Share the wave's running max and pull in the block's.
template <int NT>
__device__ __forceinline__ void wave_sync_max(SampledLds<NT>& L, WaveCap& s, float lane_best) {
  const float wm = wave_reduce(lane_best, MaxOp());
  if (lane_id() == 0 && wm > -INFINITY) atomicMax(&L.mkey, ord_key(wm));
  wave_lds_sync();
  const float m = key_float(uni(L.mkey));
  const float t = m - s.dcap;
  if (t > s.tau && !s.ovf) s.tau = t;
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
    for (int w = 0; w < NW; ++w) {
      const int n = L.wn[w];
      for (int j = threadIdx.x; j < n; j += NT) {
        const float x = L.elem[w][j].x;
        if (!in_bins(x)) continue;
        const int b = bin_of(x);
        atomicAdd(&L.u.post.cnt[b], 1);
        if (!kCode) {
          const double we = weight(x, m, T);
          atomicAdd(&L.u.post.mass[b], we);
          corr += we - exp2((static_cast<double>(x) - static_cast<double>(m)) * c);
        }
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
          corr += lc[k] * (wb - exp2((static_cast<double>(v) - static_cast<double>(m)) * c));
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
    int tc;
    double tm, tcorr;
    const int ic = block_scan_incl<NT, int>(sc, L.red_i, tc);
    const double im = block_scan_incl<NT, double>(sm, L.red_d, tm);
    block_scan_incl<NT, double>(corr, L.red_d + NW, tcorr);
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
    for (int w = 0; w < NW; ++w) {
      const int n = L.wn[w];
      for (int j = threadIdx.x; j < n; j += NT) {
        const Cand e = L.elem[w][j];
        if (!in_bins(e.x) || bin_of(e.x) != b) continue;
        const int pos = atomicAdd(&L.gn, 1);
        if (pos < kGather) L.u.post.g[pos] = e;
      }
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
    for (int w = 0; w < NW; ++w) {
      const int n = L.wn[w];
      for (int j = threadIdx.x; j < n; j += NT) {
        const float x = L.elem[w][j].x;
        if (in_bins(x) && (static_cast<double>(x) - static_cast<double>(m)) / T >= lnmp) ++cnt;
      }
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

// Exact locator over the whole row: radix select on the order-preserving
// key (four 8-bit digits, most significant first), then the tie of the
// located value in index order. Reads the row several times; used only when
// the candidates cannot decide.
template <typename E, int NT>
struct FullLocator {
  SampledLds<NT>& L;
  const E* __restrict__ row;
  int V;
  float m;
  double T;
  double wtot;

  __device__ FullLocator(SampledLds<NT>& l, const E* r, int V_, float m_, double T_)
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

// The filtered draw, given a locator. Returns false if the locator cannot
// decide.
template <class Loc>
__device__ bool decide(Loc& loc, int V, int top_k, double top_p, double min_p, double u, int& token) {
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
    if (!p.ok) return false;
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

// Stream one sampled row: the statistics of stream_row plus candidate capture.
template <typename E, int NT, int U>
__device__ __forceinline__ void stream_sampled(const E* __restrict__ row, int V, float c, RowPartial& p,
                                               SampledLds<NT>& L, WaveCap& s) {
  constexpr int N = Elem<E>::kVec;
  const int tid = threadIdx.x;
  const uintptr_t addr = reinterpret_cast<uintptr_t>(row);
  int head = static_cast<int>(((16u - (addr & 15u)) & 15u) / sizeof(E));
  if (head > V) head = V;
  const int nvec = (V - head) / N;
  const int body_end = head + nvec * N;
  const u32x4* __restrict__ vp = reinterpret_cast<const u32x4*>(row + head);
  // Rolling slots: slot u holds vector g*G + u*NT + tid of group g; it is
  // decoded and parked, then reloaded at once with the same vector of group
  // g+1, so U-1 vectors per lane are always in flight and the loop carries
  // no register copies (a copy at the latch would wait for every load).
  // Loads are unconditional (clamped as in load_group, row_stream.hpp).
  constexpr int G = U * NT;
  const int nfull = nvec / G;

  // head elements first: a load issued after the slots' would make the
  // first wait cover them too
  const bool has_head = tid < head;
  const float xh = has_head ? Elem<E>::at(row, tid) : -INFINITY;
  u32x4 slot[U];
  if (nvec > 0) load_group<NT, U>(slot, vp, 0, nvec);

  // Starting threshold: the block's max over its first group (and head).
  {
    float m0 = xh;
    if (nvec > 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (tid + u * NT < nvec) {
          float f[N];
          m0 = fmaxf(m0, vec_max<E>(slot[u], f));
        }
      }
    }
    block_start_max<NT>(L, s, m0);
  }
  if (has_head) take_scalar<false>(p, xh, tid, c, INFINITY, 0);
  wave_take_scalar<NT>(L, s, xh, tid, has_head);

  if (nvec > 0) {
    for (int g = 0; g < nfull; ++g) {
      const int v = g * G + tid;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float f[N];
        const float vmax = vec_max<E>(slot[u], f);
        const int e0 = head + (v + u * NT) * N;
        const bool full = wave_park_only<NT>(L, s, slot[u], e0, vmax, true);
        slot[u] = load_stream(vp + min(v + G + u * NT, nvec - 1));
        take_floats<N>(p, f, vmax, c);
        if (full) wave_drain<E, NT>(L, s);
      }
      wave_sync_max<NT>(L, s, p.best);
    }
    // the slots now hold group nfull, the partial last one
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = nfull * G + tid + u * NT;
      const bool valid = q < nvec;
      float f[N];
      float vmax = -INFINITY;
      if (valid) {
        vmax = vec_max<E>(slot[u], f);
        take_floats<N>(p, f, vmax, c);
      }
      if (wave_park_only<NT>(L, s, slot[u], head + q * N, vmax, valid)) wave_drain<E, NT>(L, s);
    }
  }

  const int tail = V - body_end;
  const bool has_tail = tid < tail;
  const float xt = has_tail ? Elem<E>::at(row, body_end + tid) : -INFINITY;
  if (has_tail) take_scalar<false>(p, xt, body_end + tid, c, INFINITY, 0);
  wave_take_scalar<NT>(L, s, xt, body_end + tid, has_tail);
  wave_drain<E, NT>(L, s);
}

// Outcome of one sampled row.
struct SampledOut {
  int token;
  double lse;
  int bits;
  int slow;   // 1 if the exact whole-row path decided
};

// One workgroup samples row `row` of request `req` (local row j) at
// temperature T > 0. `after_stream` runs once the row has been read.
template <typename E, int NT, int U, typename Hook>
__device__ __forceinline__ SampledOut sampled_row(const VerifyArgs& a, const E* __restrict__ row, int req, int j, float T,
                                  SampledLds<NT>& L, Hook after_stream) {
  SampledOut out{0, 0.0, 0, 0};
  int top_k = a.top_k[req];
  float top_p = a.top_p[req];
  float min_p = a.min_p[req];
  if (!(top_p > 0.f && top_p <= 1.f) || !(min_p >= 0.f && min_p <= 1.f) || !(T < INFINITY)) {
    out.bits |= VSV_FLAG_PARAMS;
    if (!(top_p > 0.f && top_p <= 1.f)) top_p = 1.f;
    if (!(min_p >= 0.f && min_p <= 1.f)) min_p = 0.f;
  }
  const double Td = static_cast<double>(T);
  const float c = 1.4426950408889634f / T;

  // Capture window below the running max: T * kZcap (weights under e^-kZcap
  // of the max's), or exactly the min-p cut when min-p alone filters. A
  // top-k cut is a count, which an outlying max can push below any window,
  // so top-k rows use no window: compaction alone raises their threshold and
  // always keeps top_k + 32 candidates per wave (the union then holds the
  // whole top-k set whenever top_k + 32 fits a wave's buffer).
  const bool tk = top_k > 0 && top_k < a.V;
  float dcap = tk ? FLT_MAX : T * kZcap;
  if (min_p > 0.f && top_p >= 1.f && !tk) {
    const float dm = static_cast<float>(-Td * log(static_cast<double>(min_p))) * 1.0001f + 1e-6f;
    dcap = fminf(dcap, dm);
  }
  if (!(dcap < INFINITY)) dcap = FLT_MAX;
  const int kmin = tk ? min(top_k + 32, kEW - 2 * kWave) : 0;

  const int w = wave_id();
  if (threadIdx.x == 0) L.mkey = INT32_MIN;
  lds_barrier();
  WaveCap s{0, 0, -INFINITY, -INFINITY, dcap, 0, kmin};

  RowPartial p;
  partial_init(p);
  stream_sampled<E, NT, U>(row, a.V, c, p, L, s);
  after_stream();
  if (lane_id() == 0) {
    L.wtau[w] = s.ovf ? INFINITY : s.tau;
    L.wn[w] = s.elem_n;
    L.wovf[w] = s.ovf;
  }
  const NoKeep nokeep;
  const RowResult res = finish_row<E, NT, U, false, false>(p, L.rs, nokeep, row, a.V);
  out.lse = res.lse;
  if (!(res.max < INFINITY) || !(res.max > -INFINITY) || !isfinite(res.lse)) out.bits |= VSV_FLAG_LOGITS;

  constexpr int NW = NT / kWave;
  float tau = -INFINITY;
  int ovf = 0;
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    tau = fmaxf(tau, L.wtau[k]);
    ovf |= L.wovf[k];
  }
  const float m = res.max;
  const double u = row_uniform(a.seed, a.offset, req, j);
  // whole-row weight relative to the maximum, with the stream's exponents
  // (x * c with c = log2(e) / T rounded to float); CandLocator::build swaps
  // the candidates' share for their exact float64 weights
  const double wtot = res.sum * exp2(static_cast<double>(res.mref) -
                                     static_cast<double>(m) * static_cast<double>(c));
  int token = 0;
  bool done = false;
  if (!ovf && !out.bits) {
    CandLocator<E, NT> loc(L, m, Td, tau, wtot, static_cast<double>(c));
    loc.build();
    int t = 0;
    done = decide(loc, a.V, top_k, static_cast<double>(top_p), static_cast<double>(min_p), u, t) && !loc.bad;
    if (done) token = t;
  }
  if (!done && !(out.bits & VSV_FLAG_LOGITS)) {
    lds_barrier();
    FullLocator<E, NT> fl(L, row, a.V, m, Td);
    int t = 0;
    decide(fl, a.V, top_k, static_cast<double>(top_p), static_cast<double>(min_p), u, t);
    token = t;
    out.slow = 1;
  }
  lds_barrier();
  out.token = token;
  return out;
}

}  // namespace vsv
