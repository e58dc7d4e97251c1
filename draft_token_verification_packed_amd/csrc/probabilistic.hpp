// Verification with probabilistic drafts: launch interface.
#pragma once
#include "kernels.hpp"

namespace vsv {

// The draft model's rows and temperatures. Draft row q (same element type
// and vocabulary as the target rows) is the distribution draft token q was
// drawn from; request i's draft j sits at q = off[i] - i + j, the layout of
// the draft tokens.
struct ProbArgs {
  const void* draft_logits;        // [R - B, dld]
  int64_t dld;
  const float* draft_temperature;  // [B]; 0 = the draft row's arg-max was proposed
};

hipError_t launch_verify_probabilistic(const VerifyArgs& a, const ProbArgs& p, hipStream_t s);

}  // namespace vsv
