// Internal interface between the C ABI (abi.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vspec_verify.h"

namespace vsv {

// Threads per row workgroup and 16-byte loads in flight per thread.
#ifndef VSV_VERIFY_THREADS
#define VSV_VERIFY_THREADS 512
#endif
#ifndef VSV_UNROLL
#define VSV_UNROLL 2
#endif
constexpr int kVerifyThreads = VSV_VERIFY_THREADS;
constexpr int kUnroll = VSV_UNROLL;

// Everything a verify launch needs, passed by value as the kernel argument.
struct VerifyArgs {
  const void* logits;
  int64_t ld;
  int32_t V, B, R, dtype;
  const int32_t* offsets;
  const int32_t* owner;
  const int32_t* drafts;
  int32_t relaxed_k;
  // sampled only
  const float* temperature;
  const int32_t* top_k;
  const float* top_p;
  const float* min_p;
  uint64_t seed, offset;
  // outputs
  int32_t* accepted_len;
  int32_t* next_token;
  int32_t* out_offsets;
  int32_t* out_tokens;
  int32_t* row_token;
  float* row_lse;
  int32_t* error_flag;
  int32_t* slow_rows;
  // workspace
  int32_t* ws_ticket;   // finished-row counter
  uint32_t* ws_row;     // [R] emitted token of the row | 0x80000000 if its draft was accepted
};

struct ConfidenceArgs {
  const void* logits;
  int64_t ld;
  int32_t V, D, dtype;
  const int32_t* selected;
  float* confidence;
  float* lse;
  int32_t* error_flag;
};

// Workspace layout (bytes, 256-aligned pieces).
constexpr size_t kWsAlign = 256;
inline size_t ws_align(size_t b) { return (b + kWsAlign - 1) / kWsAlign * kWsAlign; }
inline size_t ws_bytes(int32_t B, int32_t R, int32_t /*sampled*/) {
  (void)B;
  return kWsAlign + ws_align(static_cast<size_t>(R) * 4);
}

hipError_t launch_verify_greedy(const VerifyArgs& a, hipStream_t s);
hipError_t launch_verify_sampled(const VerifyArgs& a, hipStream_t s);
hipError_t launch_confidence(const ConfidenceArgs& a, hipStream_t s);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

}  // namespace vsv
