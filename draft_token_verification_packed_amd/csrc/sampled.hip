// Sampled verification kernel (gfx950): rows of requests with temperature
// > 0 draw their token (sampled_row.hpp), rows of greedy requests take the
// arg-max, and the per-request scan (verify_common.hpp) ends the launch.
#include "verify_common.hpp"
#include "sampled_row.hpp"

namespace vsv {

// ---------------------------------------------------------------- sampled

// Rows of requests with temperature > 0 draw their token (sampled_row.hpp);
// rows of greedy requests take the arg-max exactly as verify_greedy does.
// Acceptance is strict: the draft must equal the row's token.
//
// A sampled row costs several times a greedy one, and the hardware's
// in-order workgroup dispatch leaves CUs idle behind such uneven rows. So
// the grid is persistent (as many workgroups as fit on the device at once)
// and each workgroup takes rows from a queue in the workspace. It asks for
// its next row once the current row has been read from memory, so the
// request's latency hides behind the row's last steps while the rows still
// go to the workgroups that free up first. The workgroup that finishes last
// resets the queue and runs the per-request scan.
template <typename E, int NT, int U, typename Hook>
__device__ __forceinline__ void sampled_kernel_row(const VerifyArgs& a, uint32_t tag, int r, SampledLds<NT>& L,
                                                   Hook after_stream) {
  const E* __restrict__ row = static_cast<const E*>(a.logits) + static_cast<int64_t>(r) * a.ld;
  const RowMeta m = load_meta(a, r, a.owner[r]);
  const float T = a.temperature[m.req < 0 ? 0 : m.req];
  int token = 0, bits = 0, slow = 0;
  double lse = 0.0;
  if (m.req >= 0 && T > 0.f) {
    const SampledOut o = sampled_row<E, NT, SampledDepth<E>::kPass1>(a, row, m.req, m.j, T, L, after_stream);
    token = o.token;
    lse = o.lse;
    bits = o.bits;
    slow = o.slow;
  } else {
    RowPartial p;
    partial_init(p);
    GroupKeep<U> keep{};
    constexpr float kLog2e = 1.4426950408889634f;
    stream_row<E, NT, U, false, GroupKeep<U>, NoHook, true>(row, a.V, kLog2e, INFINITY, 0, p, keep);
    after_stream();
    const RowStats res = finish_row_lean<E, NT, U, false>(p, L.ls, keep, row, a.V);
    token = res.argmax;
    // float log2 of a sum holding the maximum's own term (at least 1/2)
    lse = 0.69314718f * (res.mref + __log2f(static_cast<float>(res.sum)));
    if (!(res.max < INFINITY) || token == INT32_MAX || !isfinite(lse)) bits |= VSV_FLAG_LOGITS;
    if (token == INT32_MAX) token = 0;
    if (m.req >= 0 && !(T >= 0.f)) bits |= VSV_FLAG_PARAMS;
  }
  if (threadIdx.x == 0) {
    const uint32_t word = row_word(a, m, token, m.draft == token, bits);
    if (bits) set_flag(a, bits);
    if (slow && a.slow_rows) atomicAdd(a.slow_rows, 1);
    if (a.row_token) a.row_token[r] = token;
    if (a.row_lse) a.row_lse[r] = static_cast<float>(lse);
    if (r != a.withheld_row) store_agent64(a.ws_row + r, tagged(tag, word));
  }
}

// The order in which the queue hands out rows. A sampled row costs several
// times a greedy one, and when a batch has few rows per workgroup slot the
// rows handed out last decide when the launch ends. So the sampled
// requests' rows go first and the greedy rows last (longest first), each
// group in request order. One workgroup writes the order into the
// workspace before the verification launch. A layout it cannot trust
// (offsets not 0 = off[0] < off[1] < ... < off[B] = R) keeps the plain row
// order; the verification launch flags such a layout as before.
template <int NT>
__global__ __launch_bounds__(NT) void sampled_order_kernel(VerifyArgs a) {
  __shared__ int scan[NT / kWave];
  const int t = threadIdx.x;
  const int per = (a.B + NT - 1) / NT;
  const int i0 = min(a.B, t * per), i1 = min(a.B, i0 + per);
  int ns = 0, ng = 0, bad = 0;
  for (int i = i0; i < i1; ++i) {
    const int r0 = a.offsets[i], r1 = a.offsets[i + 1];
    bad |= !(r0 >= 0 && r1 > r0 && r1 <= a.R) || (i == 0 && r0 != 0) || (i == a.B - 1 && r1 != a.R);
    const int n = bad ? 0 : r1 - r0;
    if (a.temperature[i] > 0.f) ns += n; else ng += n;
  }
  int ns_total, ng_total;
  const int s_before = block_exclusive_scan<NT>(ns, scan, ns_total);
  const int g_before = block_exclusive_scan<NT>(ng, scan, ng_total);
  if (__syncthreads_or(bad) || ns_total + ng_total != a.R) {
    for (int q = t; q < a.R; q += NT) a.ws_perm[q] = q;
    return;
  }
  int ps = s_before, pg = ns_total + g_before;
  for (int i = i0; i < i1; ++i) {
    const int r0 = a.offsets[i], r1 = a.offsets[i + 1];
    int& pos = a.temperature[i] > 0.f ? ps : pg;
    for (int r = r0; r < r1; ++r) a.ws_perm[pos++] = r;
  }
}

__device__ __forceinline__ uint32_t queue_take(const VerifyArgs& a) {
  return __hip_atomic_fetch_add(a.ws_queue + kQueueNext, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename E, int NT, int U>
// two workgroups per CU (4 waves per SIMD): at most 128 VGPRs
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) void verify_sampled_kernel(VerifyArgs a) {
  __shared__ SampledLds<NT> L;
  static_assert(sizeof(TailScratch) <= sizeof(L.c), "tail staging aliases the candidate buffer");
  const uint32_t tag = call_tag(a);
  // Tickets: a workgroup's first ticket is its own index when the rows come
  // in ws_perm order (the grid has at most R workgroups), else it comes
  // from the queue like every later one.
  const uint32_t R = static_cast<uint32_t>(a.R);
  const uint32_t P = a.ordered ? gridDim.x : 0u;
  auto row_of = [&](uint32_t q) -> int {
    return q < R ? (a.ordered ? a.ws_perm[q] : static_cast<int>(q)) : a.R;
  };
  if (threadIdx.x == 0) L.row_next = row_of(a.ordered ? blockIdx.x : queue_take(a));
  lds_barrier();
  int r = L.row_next;
  while (r < a.R) {
    // the next row's ticket is in flight during the row's last steps; the
    // row's barriers separate this read of row_next from the write below
    uint32_t next = 0;
    sampled_kernel_row<E, NT, U>(a, tag, r, L, [&]() {
      if (threadIdx.x == 0) next = queue_take(a);
    });
    if (threadIdx.x == 0) L.row_next = row_of(next + P);
    lds_barrier();
    r = L.row_next;
  }
  // Every ticket of this workgroup has been taken and its rows published
  // (release); the last workgroup to get here sees all rows (acquire).
  if (threadIdx.x == 0) {
    const uint32_t done = __hip_atomic_fetch_add(a.ws_queue + kQueueDone, 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    L.last = done + 1 == gridDim.x;
  }
  lds_barrier();
  if (L.last) {
    if (threadIdx.x == 0) {
      store_agent(a.ws_queue + kQueueNext, 0u);
      store_agent(a.ws_queue + kQueueDone, 0u);
    }
    words_tail<NT>(a, tag, *reinterpret_cast<TailScratch*>(&L.c));
  }
}

// Workgroups of the sampled kernel that fit on the current device at once
// (cached per device), or 0 if unknown.
template <typename E>
static int sampled_resident(int cus) {
  static int cached[64];
  int dev = 0;
  if (cus <= 0 || hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, verify_sampled_kernel<E, kVerifyThreads, SampledDepth<E>::kGreedy>,
                                                   kVerifyThreads, 0) != hipSuccess ||
      per_cu <= 0)
    return 0;
  const int n = per_cu * cus;
  if (dev < 64) cached[dev] = n;
  return n;
}

template <typename E>
static hipError_t launch_sampled_t(const VerifyArgs& a, hipStream_t s) {
  int grid = sampled_resident<E>(a.groups);
  if (grid <= 0) grid = 256;
  if (grid > a.R) grid = a.R;
  // Longest rows first only where the batch has at most two rows per
  // workgroup slot: with more, the rows handed out last are a small part of
  // the launch, and the order's lookup would add a load to every row.
  VerifyArgs b = a;
  b.ordered = (a.ws_perm && a.R <= 2 * grid) ? 1 : 0;
  if (b.ordered) {
    sampled_order_kernel<kOrderThreads><<<dim3(1), dim3(kOrderThreads), 0, s>>>(b);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  verify_sampled_kernel<E, kVerifyThreads, SampledDepth<E>::kGreedy><<<dim3(grid), dim3(kVerifyThreads), 0, s>>>(b);
  return hipGetLastError();
}

hipError_t launch_verify_sampled(const VerifyArgs& a, hipStream_t s) {
  return a.dtype == VSV_BF16 ? launch_sampled_t<uint16_t>(a, s) : launch_sampled_t<float>(a, s);
}

}  // namespace vsv
