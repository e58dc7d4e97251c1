// Adaptive target-verify allocation (xLLM docs, "Adaptive speculative
// inference": the enable_adaptive_target_verify switch and the section
// "Adaptive target verification from MTP logits").
//
// Every request proposed K drafts, each with a draft confidence score (the
// selected token's draft probability). The host fixes a padded budget of G
// target rows ahead of the round; the scores of the current round stay on
// the device and decide how many leading drafts k_i of each request the
// target verifies, after which the verify rows are packed.
//
// A draft is accepted only if every earlier draft of its request is, so its
// predicted acceptance is the running product of its request's scores
// (float32, left to right, scores clamped to [0, 1] with NaN as 0). The
// G - B rows beyond the B bonus rows go to the positions with the largest
// products, ties broken by request and then position, ascending; products
// never grow along a request, so each request receives a prefix.
//
// One workgroup does the whole batch (B * K <= kMaxAllocPositions,
// B <= kMaxAllocRequests):
//  1. products into LDS as their float32 bit patterns (non-negative, so the
//     integer order is the value order; -0 is stored as +0);
//  2. the M-th largest pattern (M = G - B) by a three-pass radix select
//     (11 + 11 + 10 bits) over a 2048-bin LDS histogram;
//  3. per request: positions above the threshold, plus the tied positions
//     that the request-ordered scan of tie counts leaves within M;
//  4. offsets by a block scan of (k_i + 1), kept in LDS; then one thread per
//     packed row finds its request by binary search over them and writes
//     the row's owner, source row and draft token.
#include "allocate.hpp"
#include "device.hpp"

namespace vsv {

namespace {

constexpr int kAllocThreads = 1024;   // fewer threads were slower: 512, 256, 128
                                      // took 12.6, 19.9, 37.0 us at B=512, K=7
constexpr int kAllocBins = 2048;
constexpr int kBinsPerThread = kAllocBins / kAllocThreads;
static_assert(kAllocBins % kAllocThreads == 0, "whole bins per thread");
constexpr int kAllocWaves = kAllocThreads / kWave;
static_assert(kMaxAllocPositions < (1 << 15), "two counts share one 32-bit scan");

struct AllocScratch {
  uint32_t key[kMaxAllocPositions];    // products as bit patterns
  int off[kMaxAllocRequests + 1];      // row offsets
  uint32_t hist[kAllocBins];
  int scan[kAllocWaves];
  int digit, above;
};

// Multiply the running product by the clamped score c; returns its pattern.
__device__ __forceinline__ uint32_t clamp_bits(float c, float& run) {
  const float s = (c >= 0.f) ? fminf(c, 1.f) : 0.f;   // NaN and negatives give 0
  run = run * s;
  return __float_as_uint(run) & 0x7FFFFFFFu;
}

// k_i for the requests [i0, i1) of this thread, given the threshold pattern
// tau, the positions still to take among ties (`need`) and the number of tied
// positions of earlier requests (`ties_before`).
template <typename F>
__device__ __forceinline__ void walk_requests(const AllocScratch& s, int K, int i0, int i1, uint32_t tau,
                                              int need, int ties_before, F&& emit) {
  int e = ties_before;
  for (int i = i0; i < i1; ++i) {
    int gt = 0, eq = 0;
    for (int j = 0; j < K; ++j) {
      const uint32_t k = s.key[i * K + j];
      gt += k > tau;
      eq += k == tau;
    }
    const int take = min(eq, max(0, need - e));
    e += eq;
    emit(i, gt + take);
  }
}

__global__ __launch_bounds__(kAllocThreads) void allocate_kernel(AllocArgs a) {
  __shared__ AllocScratch s;
  const int t = threadIdx.x;
  const int B = a.B, K = a.K, N = a.B * a.K, M = a.G - a.B;

  // 1. running products of the clamped scores. The scores come in with one
  //    coalesced load per position and the products are formed in LDS, so
  //    the whole step costs one global round trip.
  for (int q = t; q < N; q += kAllocThreads) s.key[q] = __float_as_uint(a.conf[q]);
  lds_barrier();
  for (int i = t; i < B; i += kAllocThreads) {
    float run = 1.f;
    for (int j = 0; j < K; ++j) s.key[i * K + j] = clamp_bits(__uint_as_float(s.key[i * K + j]), run);
  }
  lds_barrier();
  if (a.prefix)
    for (int q = t; q < N; q += kAllocThreads) a.prefix[q] = __uint_as_float(s.key[q]);

  // 2. tau = the M-th largest pattern (M >= 1); with M = 0 no position is
  //    taken, which a threshold above every pattern expresses.
  uint32_t tau = 0xFFFFFFFFu;
  if (M > 0) {
    uint32_t prefix = 0;
    int remaining = M;
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const int width = pass == 2 ? 10 : 11;
      const uint32_t hi_mask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + width));
      const uint32_t dmask = (1u << width) - 1u;
      for (int b = t; b < kAllocBins; b += kAllocThreads) s.hist[b] = 0;
      lds_barrier();
      for (int q = t; q < N; q += kAllocThreads) {
        const uint32_t k = s.key[q];
        if ((k & hi_mask) == prefix) atomicAdd(&s.hist[(k >> shift) & dmask], 1u);
      }
      lds_barrier();
      // bins in descending digit order, kBinsPerThread consecutive ones per
      // thread; the bin holding the remaining-th largest pattern is the one
      // whose count of patterns above it is < remaining <= that count plus
      // its own
      const int dtop = kAllocBins - 1 - kBinsPerThread * t;
      int h[kBinsPerThread];
      int mine = 0;
#pragma unroll
      for (int b = 0; b < kBinsPerThread; ++b) {
        h[b] = static_cast<int>(s.hist[dtop - b]);
        mine += h[b];
      }
      int total;
      int above = block_exclusive_scan<kAllocThreads>(mine, s.scan, total);
#pragma unroll
      for (int b = 0; b < kBinsPerThread; ++b) {
        if (above < remaining && remaining <= above + h[b]) {
          s.digit = dtop - b;
          s.above = above;
        }
        above += h[b];
      }
      lds_barrier();
      prefix |= static_cast<uint32_t>(s.digit) << shift;
      remaining -= s.above;
    }
    tau = prefix;
  }

  // 3. verify lengths: this thread's contiguous requests [i0, i1)
  const int per = (B + kAllocThreads - 1) / kAllocThreads;
  const int i0 = min(B, t * per), i1 = min(B, i0 + per);
  int gt_sum = 0, eq_sum = 0;
  for (int i = i0; i < i1; ++i)
    for (int j = 0; j < K; ++j) {
      const uint32_t k = s.key[i * K + j];
      gt_sum += k > tau;
      eq_sum += k == tau;
    }
  // one scan of both counts, packed as gt * 2^16 + eq (each at most
  // kMaxAllocPositions < 2^16, so neither half carries into the other)
  int both_total;
  const int both_before = block_exclusive_scan<kAllocThreads>((gt_sum << 16) | eq_sum, s.scan, both_total);
  const int ties_before = both_before & 0xFFFF;
  const int need = M - (both_total >> 16);   // tied positions to take, in request order
  int rows = 0;
  walk_requests(s, K, i0, i1, tau, need, ties_before, [&](int, int k) { rows += k + 1; });
  int rows_total;
  int off = block_exclusive_scan<kAllocThreads>(rows, s.scan, rows_total);
  walk_requests(s, K, i0, i1, tau, need, ties_before, [&](int i, int k) {
    a.verify_len[i] = k;
    a.row_offsets[i] = off;
    s.off[i] = off;
    off += k + 1;
  });
  if (t == 0) {
    a.row_offsets[B] = a.G;
    s.off[B] = a.G;
  }
  lds_barrier();

  // 4. pack: packed row r belongs to the request i with off[i] <= r < off[i+1]
  for (int r = t; r < a.G; r += kAllocThreads) {
    int lo = 0, hi = B - 1;   // largest i with off[i] <= r
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s.off[mid] <= r) lo = mid; else hi = mid - 1;
    }
    const int i = lo, j = r - s.off[lo];
    a.row_owner[r] = i;
    if (a.row_source) a.row_source[r] = i * (K + 1) + j;
    // (j < K and r - i < G - B follow from the offsets; checked anyway so
    // that no write can leave the buffers)
    if (a.packed_drafts && r < s.off[i + 1] - 1 && j < K && r - i < a.G - B)
      a.packed_drafts[r - i] = a.drafts[i * K + j];
  }
}

}  // namespace

hipError_t launch_allocate(const AllocArgs& a, hipStream_t s) {
  allocate_kernel<<<dim3(1), dim3(kAllocThreads), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace vsv
