// C ABI entry points: host-side validation, workspace carving and launch.
// Nothing here synchronises, allocates or reads device memory.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "allocate.hpp"
#include "kernels.hpp"
#include "probabilistic.hpp"

using vsv::VerifyArgs;

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elem_size(int32_t dtype) { return dtype == VSV_BF16 ? 2 : 4; }

bool dtype_ok(int32_t dtype) { return dtype == VSV_F32 || dtype == VSV_BF16; }

// Row whose result word the next launches leave unpublished (-1: none); set
// only by vsv_test_withhold_row_word.
std::atomic<int32_t> g_withheld_row{-1};

// CUs of the current device (cached per device); 0 if the count is unknown.
int device_cus() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 0;
  if (dev < 64) cached[dev] = cus;
  return cus;
}

// Common checks of a batch and its outputs; fills the shared launch args.
vsv_status prepare(const vsv_batch* b, const vsv_outputs* o, void* ws, size_t ws_bytes, int32_t sampled,
                   VerifyArgs* a, bool* empty) {
  *empty = false;
  if (!b || !o) return VSV_EINVAL;
  if (b->num_requests < 0 || b->num_rows < b->num_requests) return VSV_EINVAL;
  if (b->num_requests == 0) {
    if (b->num_rows != 0) return VSV_EINVAL;
    *empty = true;
    return VSV_OK;
  }
  if (!dtype_ok(b->dtype) || b->vocab < 1 || b->vocab > vsv::kMaxVocab || b->ld < b->vocab) return VSV_EINVAL;
  // a row is addressed through a buffer resource with a 32-bit byte size
  if (static_cast<int64_t>(b->vocab) * elem_size(b->dtype) > vsv::kMaxRowBytes) return VSV_EINVAL;
  if (!b->logits || !aligned(b->logits, elem_size(b->dtype))) return VSV_EINVAL;
  if (!b->row_offsets || !b->row_owner) return VSV_EINVAL;
  if (b->num_rows > b->num_requests && !b->draft_tokens) return VSV_EINVAL;
  if (!o->accepted_len || !o->next_token || !o->out_offsets || !o->out_tokens) return VSV_EINVAL;
  // the last row must be addressable with 64-bit element offsets
  if (b->ld > (INT64_MAX / 4) / (b->num_rows > 0 ? b->num_rows : 1)) return VSV_EINVAL;
  if (!ws || !aligned(ws, vsv::kWsAlign)) return VSV_EWORKSPACE;
  if (ws_bytes < vsv::ws_bytes(b->num_requests, b->num_rows, sampled)) return VSV_EWORKSPACE;

  VerifyArgs& v = *a;
  v = VerifyArgs{};
  v.logits = b->logits;
  v.ld = b->ld;
  v.V = b->vocab;
  v.B = b->num_requests;
  v.R = b->num_rows;
  v.dtype = b->dtype;
  v.offsets = b->row_offsets;
  v.owner = b->row_owner;
  v.drafts = b->draft_tokens;
  v.relaxed_k = 1;
  v.accepted_len = o->accepted_len;
  v.next_token = o->next_token;
  v.out_offsets = o->out_offsets;
  v.out_tokens = o->out_tokens;
  v.row_token = o->row_token;
  v.row_lse = o->row_lse;
  v.error_flag = o->error_flag;
  v.slow_rows = o->slow_rows;
  v.withheld_row = g_withheld_row.load(std::memory_order_relaxed);
  char* w = static_cast<char*>(ws);
  v.ws_epoch = reinterpret_cast<uint32_t*>(w);
  v.ws_queue = reinterpret_cast<uint32_t*>(w + 64);
  v.ws_row = reinterpret_cast<uint64_t*>(w + vsv::kWsAlign);
  v.ws_part = reinterpret_cast<uint64_t*>(w + vsv::kWsAlign + vsv::ws_row_bytes(b->num_rows));
  v.cus = device_cus();
  return VSV_OK;
}

}  // namespace

extern "C" {

size_t vsv_workspace_bytes(int32_t num_requests, int32_t num_rows, int32_t sampled) {
  if (num_requests < 0 || num_rows < 0) return 0;
  return vsv::ws_bytes(num_requests, num_rows, sampled);
}

vsv_status vsv_workspace_init(void* workspace, size_t bytes, hipStream_t stream) {
  if (!workspace || !aligned(workspace, 4) || bytes % 4) return VSV_EINVAL;
  return vsv::launch_zero(workspace, bytes, stream) == hipSuccess ? VSV_OK : VSV_EHIP;
}

vsv_status vsv_verify_greedy(const vsv_batch* batch, int32_t relaxed_topk, const vsv_outputs* out,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  VerifyArgs a;
  bool empty = false;
  const vsv_status st = prepare(batch, out, workspace, workspace_bytes, 0, &a, &empty);
  if (st != VSV_OK || empty) return st;
  if (relaxed_topk < 1 || relaxed_topk > batch->vocab) return VSV_EINVAL;
  a.relaxed_k = relaxed_topk;
  return vsv::launch_verify_greedy(a, stream) == hipSuccess ? VSV_OK : VSV_EHIP;
}

vsv_status vsv_verify_greedy_relaxed(const vsv_batch* batch, const vsv_relax* relax, const vsv_outputs* out,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!relax) return VSV_EINVAL;
  VerifyArgs a;
  bool empty = false;
  const vsv_status st = prepare(batch, out, workspace, workspace_bytes, 0, &a, &empty);
  if (st != VSV_OK || empty) return st;
  if (relax->topk < 1 || relax->topk > batch->vocab) return VSV_EINVAL;
  if (!(relax->margin >= 0.f) || !(relax->margin < INFINITY)) return VSV_EINVAL;
  if (relax->from_position < 0 || relax->after_tokens < 0) return VSV_EINVAL;
  if (relax->num_protected < 0 || relax->num_protected > VSV_MAX_PROTECTED) return VSV_EINVAL;
  if (relax->num_protected > 0 && !relax->protected_ids) return VSV_EINVAL;
  a.relaxed_k = relax->topk;
  a.margin = relax->margin;
  a.from_pos = relax->from_position;
  a.after_tok = relax->after_tokens;
  a.generated = relax->generated;
  a.prot = relax->num_protected > 0 ? relax->protected_ids : nullptr;
  a.nprot = relax->num_protected;
  // top-K alone needs none of the extra decision inputs
  a.relax_var = (relax->margin > 0.f || relax->from_position > 0 || relax->after_tokens > 0 ||
                 relax->num_protected > 0) ? 1 : 0;
  return vsv::launch_verify_greedy(a, stream) == hipSuccess ? VSV_OK : VSV_EHIP;
}

vsv_status vsv_verify_sampled(const vsv_batch* batch, const float* temperature, const int32_t* top_k,
                              const float* top_p, const float* min_p, uint64_t seed, uint64_t offset,
                              const vsv_outputs* out, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  VerifyArgs a;
  bool empty = false;
  const vsv_status st = prepare(batch, out, workspace, workspace_bytes, 1, &a, &empty);
  if (st != VSV_OK || empty) return st;
  if (!temperature || !top_k || !top_p || !min_p) return VSV_EINVAL;
  a.temperature = temperature;
  a.top_k = top_k;
  a.top_p = top_p;
  a.min_p = min_p;
  a.seed = seed;
  a.offset = offset;
  return vsv::launch_verify_sampled(a, stream) == hipSuccess ? VSV_OK : VSV_EHIP;
}

vsv_status vsv_verify_probabilistic(const vsv_batch* batch, const void* draft_logits, int64_t draft_ld,
                                    const float* temperature, const int32_t* top_k, const float* top_p,
                                    const float* min_p, const float* draft_temperature, uint64_t seed,
                                    uint64_t offset, const vsv_outputs* out, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  VerifyArgs a;
  bool empty = false;
  const vsv_status st = prepare(batch, out, workspace, workspace_bytes, 0, &a, &empty);
  if (st != VSV_OK || empty) return st;
  if (!temperature || !top_k || !top_p || !min_p || !draft_temperature) return VSV_EINVAL;
  const int32_t D = batch->num_rows - batch->num_requests;
  if (D > 0) {
    if (!draft_logits || !aligned(draft_logits, elem_size(batch->dtype))) return VSV_EINVAL;
    if (draft_ld < batch->vocab || draft_ld > (INT64_MAX / 4) / D) return VSV_EINVAL;
  }
  a.temperature = temperature;
  a.top_k = top_k;
  a.top_p = top_p;
  a.min_p = min_p;
  a.seed = seed;
  a.offset = offset;
  const vsv::ProbArgs p{draft_logits, draft_ld, draft_temperature};
  return vsv::launch_verify_probabilistic(a, p, stream) == hipSuccess ? VSV_OK : VSV_EHIP;
}

vsv_status vsv_draft_confidence(const void* draft_logits, int32_t dtype, int32_t vocab, int64_t ld,
                                int32_t num_draft_rows, const int32_t* selected, float* confidence,
                                float* lse, int32_t* error_flag, hipStream_t stream) {
  if (num_draft_rows < 0) return VSV_EINVAL;
  if (num_draft_rows == 0) return VSV_OK;
  if (!dtype_ok(dtype) || vocab < 1 || ld < vocab) return VSV_EINVAL;
  if (!draft_logits || !aligned(draft_logits, elem_size(dtype)) || !confidence) return VSV_EINVAL;
  if (ld > (INT64_MAX / 4) / num_draft_rows) return VSV_EINVAL;
  vsv::ConfidenceArgs a{draft_logits, ld, vocab, num_draft_rows, dtype, selected, confidence, lse, error_flag};
  return vsv::launch_confidence(a, stream) == hipSuccess ? VSV_OK : VSV_EHIP;
}

vsv_status vsv_allocate_verify(const float* confidence, const int32_t* draft_tokens, int32_t num_requests,
                               int32_t num_drafts, int32_t row_budget, int32_t* verify_len, int32_t* row_offsets,
                               int32_t* row_owner, int32_t* row_source, int32_t* packed_drafts, float* prefix,
                               hipStream_t stream) {
  const int32_t B = num_requests, K = num_drafts, G = row_budget;
  if (B < 0 || K < 0 || G < B) return VSV_EINVAL;
  if (static_cast<int64_t>(G) > static_cast<int64_t>(B) * (K + 1)) return VSV_EINVAL;
  if (B == 0) return VSV_OK;
  if (B > vsv::kMaxAllocRequests || static_cast<int64_t>(B) * K > vsv::kMaxAllocPositions) return VSV_EINVAL;
  if (K > 0 && !confidence) return VSV_EINVAL;
  if (!verify_len || !row_offsets || !row_owner) return VSV_EINVAL;
  if ((draft_tokens == nullptr) != (packed_drafts == nullptr)) return VSV_EINVAL;
  vsv::AllocArgs a{confidence, draft_tokens, B, K, G, verify_len, row_offsets, row_owner, row_source,
                   G > B ? packed_drafts : nullptr, prefix};
  return vsv::launch_allocate(a, stream) == hipSuccess ? VSV_OK : VSV_EHIP;
}

const char* vsv_status_string(vsv_status status) {
  switch (status) {
    case VSV_OK: return "ok";
    case VSV_EINVAL: return "invalid argument";
    case VSV_EUNSUPPORTED: return "unsupported option";
    case VSV_EWORKSPACE: return "workspace missing, misaligned or too small";
    case VSV_EHIP: return "HIP launch failed";
    case VSV_ELIMIT: return "batch larger than the static scratch serves";
  }
  return "unknown status";
}

vsv_status vsv_test_withhold_row_word(int32_t row) {
  if (row < -1) return VSV_EINVAL;
  g_withheld_row.store(row, std::memory_order_relaxed);
  return VSV_OK;
}

int32_t vsv_version(void) { return 103; }

}  // extern "C"
