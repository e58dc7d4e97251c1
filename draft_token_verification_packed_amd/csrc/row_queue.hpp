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

// Ordered queue (a.ordered): the sampled requests' rows come first and the
// greedy requests' rows last, each group in request order. The first
// tickets go to the workgroups in index order, which the hardware spreads
// over the CUs one workgroup per CU before it places a second, so each CU
// gets a sampled row and a greedy one where the batch allows; and the rows
// handed out last, when the batch has more rows than workgroups, are cheap
// ones. Every workgroup derives the order itself at its start, from the row
// offsets and temperatures (one round of loads and one block scan of the
// two row counts, packed into 16-bit halves: R <= 0x7FFF): the row of its
// own first ticket (its index) goes to L.row_next and the rows of the
// tickets past the grid to L.late. A layout it cannot trust (offsets not
// 0 = off[0] < ... < off[B] = R) keeps the plain row order; the rows then
// flag it as before.
template <int NT, typename Lds>
__device__ __forceinline__ void ordered_start(const VerifyArgs& a, Lds& L) {
  int* scan = reinterpret_cast<int*>(&L.c);   // free until the first row
  const int t = threadIdx.x;
  const int G = static_cast<int>(gridDim.x);
  const int per = (a.B + NT - 1) / NT;
  const int i0 = min(a.B, t * per), i1 = min(a.B, i0 + per);
  int ns = 0, ng = 0, bad = 0;
  for (int i = i0; i < i1; ++i) {
    const int r0 = a.offsets[i], r1 = a.offsets[i + 1];
    bad |= !(r0 >= 0 && r1 > r0 && r1 <= a.R) || (i == 0 && r0 != 0) || (i == a.B - 1 && r1 != a.R);
    if (a.temperature[i] > 0.f) ns += r1 - r0; else ng += r1 - r0;
  }
  // every request valid: the offsets rise from 0 to R, so the counts add up
  // to R <= 0x7FFF and the packed halves neither carry nor reach the sign
  bool plain = __syncthreads_or(bad) != 0;
  int s_before = 0, g_before = 0, ns_total = 0;
  if (!plain) {
    int total;
    const int before = block_exclusive_scan<NT>((ns << 16) | ng, scan, total);
    s_before = before >> 16;
    g_before = before & 0xFFFF;
    ns_total = total >> 16;
    plain = ns_total + (total & 0xFFFF) != a.R;
  }
  if (plain) {
    for (int q = G + t; q < a.R; q += NT) L.late[q - G] = static_cast<uint16_t>(q);
    if (t == 0) L.row_next = static_cast<int>(blockIdx.x);
  } else {
    int ps = s_before, pg = ns_total + g_before;
    for (int i = i0; i < i1; ++i) {
      const int r0 = a.offsets[i], r1 = a.offsets[i + 1];
      int& pos = a.temperature[i] > 0.f ? ps : pg;
      for (int r = r0; r < r1; ++r, ++pos) {
        if (pos == static_cast<int>(blockIdx.x)) L.row_next = r;
        if (pos >= G) L.late[pos - G] = static_cast<uint16_t>(r);
      }
    }
  }
  if (t == 0) L.ticket = static_cast<int>(blockIdx.x);
}

// Runs row(r, hook) for every row this workgroup is handed, then the end of
// the call. The row function calls hook(long_tail) once its row has been
// streamed; long_tail says that the row's work after the stream is long (a
// sampled row's selection and draw). The next ticket is taken then, unless
// the row's tail is long and the queue is near its end: a workgroup that
// commits to a row while it still has tens of microseconds of work would
// leave that row waiting while other workgroups run out of rows. Such a
// ticket is taken when the row is done. Lds provides `row_next`, `ticket`,
// `last`, `late` and a candidate area `c` that the per-request scan may use
// as staging once every row is done. kMayOrder: the launch may use the
// ordered queue (a.ordered); without it a.ordered is ignored.
template <int NT, bool kMayOrder, typename Lds, typename RowFn>
__device__ __forceinline__ void row_queue_loop(const VerifyArgs& a, uint32_t tag, Lds& L, RowFn row) {
  static_assert(sizeof(TailScratch) <= sizeof(L.c), "tail staging aliases the candidate area");
  // Tickets: in the ordered queue a workgroup's first ticket is its own
  // index and later ones come from the queue, offset by the grid; otherwise
  // every ticket comes from the queue.
  const uint32_t R = static_cast<uint32_t>(a.R);
  const bool ordered = kMayOrder && a.ordered;
  const uint32_t P = ordered ? gridDim.x : 0u;
  auto row_of = [&](uint32_t q) -> int {
    return q < R ? (ordered ? static_cast<int>(L.late[q - P]) : static_cast<int>(q)) : a.R;
  };
  if (ordered) {
    ordered_start<NT>(a, L);
  } else if (threadIdx.x == 0) {
    const uint32_t q = queue_take(a);
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
