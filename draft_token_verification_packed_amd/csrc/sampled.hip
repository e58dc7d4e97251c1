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
// A compile-time int as a value (template arguments of generic lambdas).
template <int V_> struct IntC { static constexpr int value = V_; };

template <typename E, int NT, int U, typename Hook>
__device__ __forceinline__ void sampled_kernel_row(const VerifyArgs& a, uint32_t tag, int r, SampledLds<NT>& L,
                                                   Hook after_stream) {
  const E* __restrict__ row = static_cast<const E*>(a.logits) + static_cast<int64_t>(r) * a.ld;
  // Streams run at a higher wave priority than a sampled row's selection
  // and draw, which lower it once the row is read when the batch has more
  // rows than workgroups: a CU's issue slots go first to the waves that keep
  // loads in flight, and the selection fills the rest. On the ragged fp32
  // batch this took the launch from 90.4 to 85.4 us (its late greedy rows
  // stream beside selecting workgroups), on the large mixed bf16 batch from
  // 284.3 to 282.5. With one row per workgroup every selection is on the
  // launch's critical path, and lowering it cost 1.5 us (mixed, 512 rows).
  __builtin_amdgcn_s_setprio(kStreamPrio);
  const int own = a.owner[r];
  // The request's parameters go out with the row's metadata: all of them
  // for fp32 rows, the temperature alone for bf16 rows, whose filter
  // parameters are loaded once the row is known to be sampled (timed on the
  // ragged fp32 and large mixed bf16 batches, each choice was the faster
  // for its element type).
  constexpr bool kAll = sizeof(E) == 4;
  ReqParams q{};
  if constexpr (kAll) q = load_params(a, own);
  else q.T = a.temperature[(own >= 0 && own < a.B) ? own : 0];
  const RowMeta m = load_meta(a, r, own);
  const float T = q.T;
  int token = 0, bits = 0, slow = 0;
  double lse = 0.0;
  if (m.req >= 0 && T > 0.f) {
    if constexpr (!kAll) {
      q.top_k = a.top_k[m.req];
      q.top_p = a.top_p[m.req];
      q.min_p = a.min_p[m.req];
    }
    const SampledOut o = sampled_row<E, NT, SampledDepth<E>::kPass1>(a, row, m.req, m.j, q, L, after_stream);
    token = o.token;
    lse = o.lse;
    bits = o.bits;
    slow = o.slow;
  } else {
    auto greedy = [&](auto uc) {
      constexpr int UG = decltype(uc)::value;
      RowPartial p;
      partial_init(p);
      QueueKeep<E, UG> keep{};
      constexpr float kLog2e = 1.4426950408889634f;
      stream_row<E, NT, UG, false, QueueKeep<E, UG>, NoHook, true>(row, a.V, kLog2e, INFINITY, 0, p, keep);
      after_stream(false);
      return finish_row_lean<E, NT, UG, false>(p, L.ls, keep, row, a.V);
    };
    // fp32 greedy rows stream in groups of U when the batch has more rows
    // than workgroups (the rows that start late then stream beside selecting
    // workgroups and need their loads in flight), in groups of two when every
    // row starts at once (the sampled rows' streams, which end the launch,
    // then keep a larger share of the memory system: ragged fp32 batches of
    // 64 and 100 requests went from 64.3 to 58.6 us and from 78.4 to 76.1)
    RowStats res;
    if (sizeof(E) == 4 && U != 2 && a.R <= static_cast<int>(gridDim.x)) res = greedy(IntC<2>{});
    else res = greedy(IntC<U>{});
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

template <typename E, int NT, int U>
// two workgroups per CU (4 waves per SIMD): at most 128 VGPRs
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) void verify_sampled_kernel(VerifyArgs a) {
  __shared__ SampledLds<NT> L;
  const uint32_t tag = call_tag(a);
  row_queue_loop<NT, true>(a, tag, L, [&](int r, auto hook) { sampled_kernel_row<E, NT, U>(a, tag, r, L, hook); });
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
  // A sampled row costs several times a greedy one. Where the batch has more
  // rows than CUs but at most two rows per workgroup, the sampled requests'
  // rows go first (row_queue.hpp): CUs then pair a sampled row with a greedy
  // one, and the rows handed out last are greedy. With more rows, those
  // handed out last are a small part of the launch; with at most one row
  // per CU, no CU holds two rows.
  VerifyArgs b = a;
  b.ordered = (a.R > a.cus && a.R <= 2 * grid && a.R - grid <= kLateRows && a.R <= 0x7FFF) ? 1 : 0;
  verify_sampled_kernel<E, kVerifyThreads, SampledDepth<E>::kGreedy><<<dim3(grid), dim3(kVerifyThreads), 0, s>>>(b);
  return hipGetLastError();
}

hipError_t launch_verify_sampled(const VerifyArgs& a, hipStream_t s) {
  return a.dtype == VSV_BF16 ? launch_sampled_t<uint16_t>(a, s) : launch_sampled_t<float>(a, s);
}

}  // namespace vsv
