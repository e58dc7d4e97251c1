// Sampled verification kernel (gfx950): rows of requests with temperature
// > 0 draw their token (sampled_row.hpp), rows of greedy requests take the
// arg-max, and the per-request scan (verify_common.hpp) ends the launch.
#include "verify_common.hpp"
#include "row_queue.hpp"
#include "sampled_row.hpp"

namespace vsv {

// ---------------------------------------------------------------- sampled

// Rows of requests with temperature > 0 draw their token (sampled_row.hpp);
// rows of greedy requests take the arg-max exactly as verify_greedy does.
// Acceptance is strict: the draft must equal the row's token. Rows come
// from the persistent row queue (row_queue.hpp).
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
    QueueKeep<E, U> keep{};
    constexpr float kLog2e = 1.4426950408889634f;
    stream_row<E, NT, U, false, QueueKeep<E, U>, NoHook, true>(row, a.V, kLog2e, INFINITY, 0, p, keep);
    after_stream(false);
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

template <typename E, int NT, int U>
// two workgroups per CU (4 waves per SIMD): at most 128 VGPRs
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) void verify_sampled_kernel(VerifyArgs a) {
  __shared__ SampledLds<NT> L;
  const uint32_t tag = call_tag(a);
  row_queue_loop<NT>(a, tag, L, [&](int r, auto hook) { sampled_kernel_row<E, NT, U>(a, tag, r, L, hook); });
}

// Workgroups of the sampled kernel that fit on the current device at once
// (cached per device), or 0 if unknown.
template <typename E>
static int sampled_resident(int cus) {
  static int cached[64];
  int dev = 0;
  if (cus <= 0 || hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  const int n = resident_groups(verify_sampled_kernel<E, kVerifyThreads, SampledDepth<E>::kGreedy>, kVerifyThreads, cus);
  if (dev < 64 && n > 0) cached[dev] = n;
  return n;
}

template <typename E>
static hipError_t launch_sampled_t(const VerifyArgs& a, hipStream_t s) {
  int grid = sampled_resident<E>(a.cus);
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
