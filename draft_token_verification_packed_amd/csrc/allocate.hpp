// Internal interface between the C ABI (abi.cpp) and the adaptive
// verify-allocation kernel (allocate.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vsv {

// One workgroup holds a batch's products and offsets in LDS.
constexpr int kMaxAllocPositions = 16384;   // B * K
constexpr int kMaxAllocRequests = 8192;     // B

struct AllocArgs {
  const float* conf;       // [B * K] draft confidence, request-major
  const int32_t* drafts;   // [B * K] or NULL
  int32_t B, K, G;         // requests, drafts per request, row budget
  int32_t* verify_len;     // [B]
  int32_t* row_offsets;    // [B + 1]
  int32_t* row_owner;      // [G]
  int32_t* row_source;     // [G] or NULL
  int32_t* packed_drafts;  // [G - B] or NULL
  float* prefix;           // [B * K] or NULL
};

hipError_t launch_allocate(const AllocArgs& a, hipStream_t s);

}  // namespace vsv
