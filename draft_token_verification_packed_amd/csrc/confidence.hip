// Draft confidence: c_q = exp(y[s_q] - logsumexp(y)) over raw draft logits
// (xLLM docs, "Adaptive speculative inference", section "Adaptive target
// verification from MTP logits": the selected token's draft probability is
// the predicted acceptance score). One workgroup streams one draft row once.
#include "kernels.hpp"
#include "row_stream.hpp"

namespace vsv {

template <typename E, int NT, int U>
__global__ __launch_bounds__(NT) void confidence_kernel(ConfidenceArgs a) {
  __shared__ RowScratch<NT> scr;
  const int q = blockIdx.x;
  const E* __restrict__ row = static_cast<const E*>(a.logits) + static_cast<int64_t>(q) * a.ld;
  int sel = -1;
  float ysel = 0.f;
  if (a.selected) {
    sel = a.selected[q];
    if (sel >= 0 && sel < a.V) ysel = Elem<E>::at(row, sel);
  }
  RowPartial p;
  partial_init(p);
  NoKeep nokeep;
  constexpr float kLog2e = 1.4426950408889634f;
  stream_row<E, NT, U, false>(row, a.V, kLog2e, INFINITY, 0, p, nokeep);
  const RowResult res = finish_row<E, NT, U, false, false>(p, scr, nokeep, row, a.V);
  if (threadIdx.x == 0) {
    int bits = 0;
    if (!(res.max < INFINITY) || !(res.max > -INFINITY) || !isfinite(res.lse)) bits |= VSV_FLAG_LOGITS;
    double c;
    if (!a.selected) {
      c = exp(static_cast<double>(res.max) - res.lse);
    } else if (sel >= 0 && sel < a.V) {
      c = exp(static_cast<double>(ysel) - res.lse);
    } else {
      c = 0.0;
      bits |= VSV_FLAG_TOKEN;
    }
    a.confidence[q] = static_cast<float>(c);
    if (a.lse) a.lse[q] = static_cast<float>(res.lse);
    if (bits && a.error_flag) atomicOr(a.error_flag, bits);
  }
}

template <typename E>
static hipError_t launch_t(const ConfidenceArgs& a, hipStream_t s) {
  confidence_kernel<E, kConfThreads, kUnroll><<<dim3(a.D), dim3(kConfThreads), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_confidence(const ConfidenceArgs& a, hipStream_t s) {
  return a.dtype == VSV_BF16 ? launch_t<uint16_t>(a, s) : launch_t<float>(a, s);
}

}  // namespace vsv
