// Internal interface between the C ABI (abi.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vspec_verify.h"

namespace vsv {

// Threads per row workgroup, and 16-byte vectors per thread per group (the
// loads of one group are in flight while the previous group is reduced). The
// sampled stream carries the candidate capture and keeps smaller groups, so
// its registers stay within two workgroups per CU.
#ifndef VSV_VERIFY_THREADS
#define VSV_VERIFY_THREADS 512
#endif
#ifndef VSV_ROW_THREADS
#define VSV_ROW_THREADS 256
#endif
#ifndef VSV_CONF_THREADS
#define VSV_CONF_THREADS 512
#endif
#ifndef VSV_UNROLL
#define VSV_UNROLL 2
#endif
#ifndef VSV_UNROLL_ROWS
#define VSV_UNROLL_ROWS 2
#endif
constexpr int kVerifyThreads = VSV_VERIFY_THREADS;
constexpr int kRowThreads = VSV_ROW_THREADS;
constexpr int kConfThreads = VSV_CONF_THREADS;     // draft-confidence rows
constexpr int kUnroll = VSV_UNROLL;
constexpr int kUnrollRows = VSV_UNROLL_ROWS;

// Load depth of a sampled launch, by element type. Pass 1 of a sampled row
// keeps kPass1 rolling 16-byte vectors per lane (kPass1 - 1 loads in flight);
// greedy rows stream in groups of kGreedy vectors, two groups in turn. Each
// workgroup takes rows one after another, so a launch is paced by its rows'
// latencies and by how long its workgroups spend selecting instead of
// streaming. Swept over pass-1 depths 2 to 8 and greedy groups 2 to 5 (fp32
// and bf16 separately) on the ragged fp32 batch (B=128, 586 rows), the
// large mixed bf16 batch (B=512, 4096 rows) and 64-request versions of both:
// fp32 5 / 3 took the ragged batch from 83.8 to 79.4 us (8 / 4 before; 6 / 5
// and 5 / 2 made it 98 and 89 us); bf16 3 / 3 took the mixed batch from
// 262.4 to 260.4 us (4 / 3 reached 258.3 there but cost the 64-request
// mixed batch 2-4 us; 2 / 3 made it 266 us).
template <typename E> struct SampledDepth;
template <> struct SampledDepth<float> {
  static constexpr int kPass1 = 5, kGreedy = 3;
};
template <> struct SampledDepth<uint16_t> {
  static constexpr int kPass1 = 3, kGreedy = 3;
};
// Wave priorities inside the queue kernels: row streams run at kStreamPrio,
// a sampled row's selection and draw at kSelectPrio.
constexpr int kStreamPrio = 1;
constexpr int kSelectPrio = 0;
// Sampled launches hand out the sampled requests' rows first where a batch
// has more rows than CUs but at most two per workgroup; each workgroup keeps
// the rows of the tickets past the grid in LDS (16-bit row numbers), at
// most kLateRows of them.
constexpr int kLateRows = 1024;

// Everything a verify launch needs, passed by value as the kernel argument.
struct VerifyArgs {
  const void* logits;
  int64_t ld;
  int32_t V, B, R, dtype;
  const int32_t* offsets;
  const int32_t* owner;
  const int32_t* drafts;
  int32_t relaxed_k;
  // relaxed acceptance beyond top-K (greedy only): margin, gates, protected
  // ids; relax_var is set when any of them is in force
  int32_t relax_var;
  float margin;
  int32_t from_pos, after_tok;
  const int32_t* generated;
  const int32_t* prot;
  int32_t nprot;
  int32_t cus;          // CUs of the device (0 if unknown)
  int32_t parts;        // greedy: workgroups per row (set at launch)
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
  // row whose result word the row-per-workgroup kernels leave unpublished
  // (a host-set test hook for the scan's bounded wait); -1: none
  int32_t withheld_row;
  // workspace (zero before its first use). Words handed between workgroups
  // carry the call's tag in their high half, so a call finds only its own
  // and nothing has to be cleared afterwards:
  //  ws_epoch [1] calls completed on this workspace; the call's tag is
  //           derived from it and the last workgroup advances it
  //  ws_queue [kQueueWords] sampled verification's row queue: the next row
  //           to hand out and the workgroups done; the last workgroup of a
  //           call resets both to 0
  //  ws_row   [R] 64-bit words; a row handled by one workgroup stores the
  //           token it emits | kAcceptBit if its draft was accepted
  //  ws_part  [part_slot_count(R)][kPartWords] 64-bit words; with P parts
  //           per row, slot r * (P - 1) + p holds the statistics part p of
  //           row r gathered (p < P - 1)
  uint32_t* ws_epoch;
  uint32_t* ws_queue;
  uint64_t* ws_row;
  uint64_t* ws_part;
  // sampled: the queue hands out the sampled requests' rows first (each
  // workgroup derives the order at its start, row_queue.hpp)
  int32_t ordered;
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

// Greedy verification runs one workgroup per row part. Rows of more than
// about 1.5 kPartBytes are cut into parts of about kPartBytes, so no
// workgroup streams a whole fp32 row alone; a batch too small to give every
// CU a few workgroups cuts its rows further, into enough parts for about
// kPartsPerCU / 2 workgroups per CU (parts of at least kMinPartBytes). Timed
// on EAGLE-shaped bf16 batches (V=152064) on MI355X (256 CUs): 20 rows take
// 8.6 us in 16 parts each against 14.6 in two, 160 rows 15.4 us in four
// parts against 19.8 for one workgroup per CU streaming an equal share of
// the batch, and from about 320 rows on two parts per row is the rule's own
// choice.
// Parts per row: one per about kPartBytes of logits, at most kMaxRowParts.
#ifndef VSV_PART_BYTES
#define VSV_PART_BYTES 152064
#endif
#ifndef VSV_FORCE_PARTS
#define VSV_FORCE_PARTS 0
#endif
constexpr int64_t kPartBytes = VSV_PART_BYTES;
// Small batches: parts per row aim at kPartsPerCU / 2 workgroups per CU in
// all, with parts of at least kMinPartBytes.
#ifndef VSV_PARTS_PER_CU
#define VSV_PARTS_PER_CU 5
#endif
constexpr int kPartsPerCU = VSV_PARTS_PER_CU;
constexpr int64_t kMinPartBytes = 16384;
constexpr int kMaxRowParts = 16;
// Partial slots (kPartWords words each: max, its index, exponent reference,
// the float64 sum as two halves, rank count) the workspace holds for the
// parts of a batch of R rows: max(R + kSpareSlots, kPartSlots), so a batch
// of any size can cut its rows in two.
constexpr int kPartSlots = 8192;
constexpr int kSpareSlots = 1024;
constexpr int kPartWords = 6;
constexpr size_t part_slot_count(int32_t R) {
  return static_cast<size_t>(R > 0 ? R : 0) + kSpareSlots > static_cast<size_t>(kPartSlots)
             ? static_cast<size_t>(R > 0 ? R : 0) + kSpareSlots
             : static_cast<size_t>(kPartSlots);
}

// Workspace layout (bytes, 256-aligned pieces). The first piece holds the
// call counter (offset 0) and the row queue's two words (offsets 64 and 128,
// apart so that they sit in different cache lines).
constexpr size_t kWsAlign = 256;
constexpr int kQueueNext = 0;
constexpr int kQueueDone = 16;
constexpr int kQueueWords = 17;
constexpr size_t ws_align(size_t b) { return (b + kWsAlign - 1) / kWsAlign * kWsAlign; }
constexpr size_t ws_row_bytes(int32_t R) { return ws_align(static_cast<size_t>(R > 0 ? R : 1) * 8); }
// The partials area: one slot for each part but a row's last.
constexpr size_t ws_part_bytes(int32_t R) { return ws_align(part_slot_count(R) * kPartWords * 8); }
// Greedy and sampled calls need the same workspace.
constexpr size_t ws_bytes(int32_t B, int32_t R, int32_t sampled) {
  (void)B;
  (void)sampled;
  return kWsAlign + ws_row_bytes(R) + ws_part_bytes(R);
}
// Tokens travel in the low 30 bits of a row word.
constexpr int32_t kMaxVocab = 0x3FFFFFFF;
// Bytes of one row of logits: rows are read through buffer resources whose
// size is a signed 32-bit count.
constexpr int64_t kMaxRowBytes = 0x7FFFFFF0;

hipError_t launch_verify_greedy(const VerifyArgs& a, hipStream_t s);
hipError_t launch_verify_sampled(const VerifyArgs& a, hipStream_t s);
hipError_t launch_confidence(const ConfidenceArgs& a, hipStream_t s);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

}  // namespace vsv
