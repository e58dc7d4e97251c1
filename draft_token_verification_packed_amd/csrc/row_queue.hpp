// Persistent row queue shared by the sampled and probabilistic verification
// kernels (gfx950).
//
// Their rows cost very different amounts (a sampled row several times a
// greedy one), and the hardware's in-order workgroup dispatch would leave
// CUs idle behind the uneven rows. So the grid is persistent (as many
// workgroups as fit on the device at once) and each workgroup takes rows
// from a queue in the workspace. It asks for its next row once the current
// row has been read from memory (the row function calls the hook it is
// given at that point), so the request's latency hides behind the row's
// last steps while rows still go to the workgroups that free up first. The
// workgroup that finishes last resets the queue and runs the per-request
// scan.
#pragma once

#include "verify_common.hpp"

namespace vsv {

__device__ __forceinline__ uint32_t queue_take(const VerifyArgs& a) {
  return __hip_atomic_fetch_add(a.ws_queue + kQueueNext, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Runs row(r, hook) for every row this workgroup is handed, then the end of
// the call. The row function calls hook(long_tail) once its row has been
// streamed; long_tail says that the row's work after the stream is long (a
// sampled row's selection and draw). The next ticket is taken then, unless
// the row's tail is long and the queue is near its end: a workgroup that
// commits to a row while it still has tens of microseconds of work would
// leave that row waiting while other workgroups run out of rows. Such a
// ticket is taken when the row is done. Lds provides `row_next`, `ticket`,
// `last` and a candidate area `c` that the per-request scan may use as
// staging once every row is done.
template <int NT, typename Lds, typename RowFn>
__device__ __forceinline__ void row_queue_loop(const VerifyArgs& a, uint32_t tag, Lds& L, RowFn row) {
  static_assert(sizeof(TailScratch) <= sizeof(L.c), "tail staging aliases the candidate area");
  // Tickets: a workgroup's first ticket is its own index when the rows come
  // in ws_perm order (the grid has at most R workgroups), else it comes
  // from the queue like every later one.
  const uint32_t R = static_cast<uint32_t>(a.R);
  const uint32_t P = a.ordered ? gridDim.x : 0u;
  auto row_of = [&](uint32_t q) -> int {
    return q < R ? (a.ordered ? a.ws_perm[q] : static_cast<int>(q)) : a.R;
  };
  if (threadIdx.x == 0) {
    const uint32_t q = a.ordered ? blockIdx.x : queue_take(a);
    L.ticket = static_cast<int>(q < R ? q : R);
    L.row_next = row_of(q);
  }
  lds_barrier();
  // the row is the same for every lane: read it as a scalar, so that what is
  // derived from it (row pointers, buffer resources) stays in scalar
  // registers
  int r = __builtin_amdgcn_readfirstlane(L.row_next);
  uint32_t q = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(L.ticket));
  while (r < a.R) {
    // the next ticket is in flight during the row's last steps; the row's
    // barriers separate these reads of row_next and ticket from the writes
    // below
    uint32_t next = 0;
    bool taken = false;
    // uniform: more than two rows per workgroup are still to be handed out
    const bool plenty = q + 2 * gridDim.x < R;
    row(r, [&](bool long_tail) {
      if (!taken && (plenty || !long_tail)) {
        if (threadIdx.x == 0) next = queue_take(a);
        taken = true;
      }
    });
    if (threadIdx.x == 0) {
      if (!taken) next = queue_take(a);
      const uint32_t nq = next + P;
      L.ticket = static_cast<int>(nq < R ? nq : R);
      L.row_next = row_of(nq);
    }
    lds_barrier();
    r = __builtin_amdgcn_readfirstlane(L.row_next);
    q = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(L.ticket));
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

// Workgroups of `kernel` (NT threads, static LDS only) that fit on the
// current device at once, given its CU count; 0 if unknown.
template <typename K>
inline int resident_groups(K kernel, int NT, int cus) {
  int per_cu = 0;
  if (cus <= 0 || hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, NT, 0) != hipSuccess || per_cu <= 0)
    return 0;
  return per_cu * cus;
}

}  // namespace vsv
