// Greedy verification kernels (gfx950).
//
// Persistent: one workgroup per CU streams an equal share of the batch's
// chunks (kernels.hpp) and stores one partial per row it touched (max and
// its lowest index, exponent reference and sum of exponentials, rank count;
// the workgroup holding a row's first chunk adds the row's draft
// information). The last workgroup merges each row, decides its token and
// acceptance, and runs the per-request scan (verify_common.hpp). No atomics
// on global memory.
//
// Batches with more rows than CUs: one workgroup per row decides the row and
// stores its word (emitted token, accept bit); the workgroup of the last row
// runs the same per-request scan.
#include "verify_common.hpp"

namespace vsv {

// ---------------------------------------------------------------- greedy

// Fields of a partial (one tagged 64-bit word each).
enum : int { kPBest = 0, kPIdx, kPMc, kPSum, kPRank, kPInfo };
// Row information, stored with the partial of the workgroup holding the
// row's first chunk: the draft token in the low 30 bits (kNoDraft if the row
// has none or it is out of range), whether the row is a verify row, whether
// its owner entry is inconsistent.
constexpr uint32_t kInfoVerify = 1u << 30;
constexpr uint32_t kInfoBadLayout = 1u << 31;

__device__ __forceinline__ uint32_t row_info(const VerifyArgs& a, const RowMeta& m, int& bits) {
  if (m.req < 0) {
    bits |= VSV_FLAG_LAYOUT;
    return kInfoBadLayout | kNoDraft;
  }
  if (m.j >= m.K) return kNoDraft;
  if (m.draft < 0 || m.draft >= a.V) {
    bits |= VSV_FLAG_TOKEN;
    return kInfoVerify | kNoDraft;
  }
  return kInfoVerify | static_cast<uint32_t>(m.draft);
}

// The row's word from its merged statistics and its information.
template <bool kRelaxed>
__device__ __forceinline__ uint32_t greedy_word(const VerifyArgs& a, const RowRed& red, uint32_t info, int token) {
  const uint32_t d = info & kTokenMask;
  if ((info & kInfoVerify) && !(info & kInfoBadLayout) && d != kNoDraft) {
    const bool ok = kRelaxed ? (red.rank < a.relaxed_k) : (static_cast<int>(d) == token);
    if (ok) return d | kAcceptBit;
  }
  return static_cast<uint32_t>(token);
}

// Geometry of the persistent decomposition: R rows of cpr chunks each,
// Q = R * cpr chunks, workgroup p owning chunks [Q p / P, Q (p + 1) / P).
struct ChunkPlan {
  int64_t Q;
  int P, cpr;
  __device__ int64_t lo(int p) const { return Q * p / P; }
};

// Partials are stored field-major (field f of every slot, then field f + 1),
// so the lanes of a tail wave, which merge consecutive rows, read
// consecutive words: a wave's load touches a few cache lines, not one line
// per lane.
__device__ __forceinline__ uint64_t* slot_word(const VerifyArgs& a, int64_t slot, int f) {
  return a.ws_part + static_cast<size_t>(f) * (static_cast<size_t>(a.R) + kMaxGroups) + static_cast<size_t>(slot);
}

// Store field f of a partial (lanes 0 .. kPartWords - 1 of a wave together
// store the whole slot).
__device__ __forceinline__ void put_partial_field(const VerifyArgs& a, int64_t slot, int f, const RowRed& r,
                                                  uint32_t info, uint32_t tag) {
  uint32_t v = info;
  if (f == kPBest) v = __float_as_uint(r.best);
  if (f == kPIdx) v = static_cast<uint32_t>(r.idx);
  if (f == kPMc) v = __float_as_uint(r.mc);
  if (f == kPSum) v = __float_as_uint(static_cast<float>(r.s));
  if (f == kPRank) v = static_cast<uint32_t>(r.rank);
  store_agent64(slot_word(a, slot, f), tagged(tag, v));
}

template <bool kRelaxed>
__device__ __forceinline__ RowRed slot_red(const uint32_t* v) {
  return RowRed{static_cast<double>(__uint_as_float(v[kPSum])), __uint_as_float(v[kPBest]), static_cast<int>(v[kPIdx]),
                __uint_as_float(v[kPMc]), kRelaxed ? static_cast<int>(v[kPRank]) : 0};
}

// The workgroup whose range holds chunk g, from the table lo[0 .. P] of
// range starts: a double-precision estimate, then exact steps.
__device__ __forceinline__ int owner_in(const int64_t* lo, const ChunkPlan& plan, int64_t g) {
  int p = static_cast<int>(static_cast<double>(g) * plan.P / static_cast<double>(plan.Q));
  p = p < 0 ? 0 : (p >= plan.P ? plan.P - 1 : p);
  while (p > 0 && lo[p] > g) --p;
  while (p < plan.P - 1 && lo[p + 1] <= g) ++p;
  return p;
}

// Row r merged over the workgroups whose ranges hold its chunks (slots
// r + p; with fewer chunks than workgroups some ranges between them are
// empty and store nothing). Slots are taken two at a time: both are loaded
// together and, while either is still in flight, reloaded together, so a
// wait costs one round trip however many of its words are missing.
template <bool kRelaxed>
__device__ __forceinline__ RowRed merge_slots(const VerifyArgs& a, const ChunkPlan& plan, const int64_t* lo, int r,
                                              uint32_t tag, uint32_t& info, int& budget, int& stalled) {
  const int64_t g0 = static_cast<int64_t>(r) * plan.cpr;
  const int p1 = owner_in(lo, plan, g0 + plan.cpr - 1);
  int q = owner_in(lo, plan, g0);
  RowRed acc{0.0, -INFINITY, INT32_MAX, -FLT_MAX, 0};
  bool first = true;
  while (q <= p1) {
    int q2 = q + 1;
    while (q2 <= p1 && lo[q2] == lo[q2 + 1]) ++q2;
    const bool two = q2 <= p1;
    uint64_t w[2][kPartWords];
    auto load_all = [&]() {
#pragma unroll
      for (int f = 0; f < kPartWords; ++f) w[0][f] = load_agent64(slot_word(a, r + q, f));
      if (two) {
#pragma unroll
        for (int f = 0; f < kPartWords; ++f) w[1][f] = load_agent64(slot_word(a, r + q2, f));
      }
    };
    auto complete = [&]() {
      bool ok = true;
#pragma unroll
      for (int f = 0; f < kPartWords; ++f) {
        ok = ok && static_cast<uint32_t>(w[0][f] >> 32) == tag;
        ok = ok && (!two || static_cast<uint32_t>(w[1][f] >> 32) == tag);
      }
      return ok;
    };
    load_all();
    while (!complete() && budget > 0) {
      --budget;
      __builtin_amdgcn_s_sleep(2);
      load_all();
    }
    stalled |= complete() ? 0 : 1;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (k == 1 && !two) break;
      uint32_t v[kPartWords];
#pragma unroll
      for (int f = 0; f < kPartWords; ++f) v[f] = static_cast<uint32_t>(w[k][f]);
      acc = combine(acc, slot_red<kRelaxed>(v));
      if (first) info = v[kPInfo];
      first = false;
    }
    // next pair
    q = two ? q2 + 1 : p1 + 1;
    while (q <= p1 && lo[q] == lo[q + 1]) ++q;
  }
  return acc;
}

// Run by the last persistent workgroup after its own range: merge every
// row, decide its token and acceptance, write the row outputs, then the
// per-request scan.
template <int NT, bool kRelaxed>
__device__ __forceinline__ void greedy_tail(const VerifyArgs& a, const ChunkPlan& plan, uint32_t tag, TailScratch& t,
                                            int64_t* lo) {
  const int tid = threadIdx.x;
  for (int q = tid; q <= plan.P; q += NT) lo[q] = plan.lo(q);
  lds_barrier();
  int stalled = 0, bits = 0, budget = kPollBudget;
  for (int r = tid; r < a.R; r += NT) {
    uint32_t info = kNoDraft;
    const RowRed red = merge_slots<kRelaxed>(a, plan, lo, r, tag, info, budget, stalled);
    int token = red.idx;
    // the sum holds the maximum's own term (at least 1/2), so float log2
    // keeps the log-sum-exp within a few units of float rounding
    const float lse = 0.69314718f * (red.mc + __log2f(static_cast<float>(red.s)));
    if (!(red.best < INFINITY) || token == INT32_MAX || !isfinite(lse)) {
      bits |= VSV_FLAG_LOGITS;
      if (token == INT32_MAX) token = 0;
    }
    const uint32_t word = greedy_word<kRelaxed>(a, red, info, token);
    if (a.row_token) a.row_token[r] = token;
    if (a.row_lse) a.row_lse[r] = lse;
    if (r < kTailStage) t.words[r] = word;
    else store_agent64(a.ws_row + r, word);
  }
  if (bits) set_flag(a, bits);
  if (stalled) set_flag(a, VSV_FLAG_STALLED);
  if (a.R > kTailStage) {
    // words of later rows went to the workspace: a full barrier after their
    // stores have completed, so no read of them moves above it
    wait_memory();
    __syncthreads();
  } else {
    lds_barrier();
  }
  // a batch whose words all sit in LDS scans without any global load, so no
  // wait in the scan can stall behind the row outputs just stored
  if (a.R <= kTailStage)
    scan_requests<NT>(a, t, [&](int row) -> uint32_t { return t.words[row]; });
  else
    scan_requests<NT>(a, t, [&](int row) -> uint32_t {
      return row < kTailStage ? t.words[row] : static_cast<uint32_t>(load_agent64(a.ws_row + row));
    });
  end_call(a, tag);
}

// A row's geometry: its 16-byte-aligned body starts `head` elements in (at
// byte `boff`) and is `nvec` vectors long; one buffer resource covers the
// whole row [0, V) (or nothing at all).
template <typename E>
struct RowGeo {
  const E* row;
  int head, nvec;
  uint32_t boff;
  __amdgpu_buffer_rsrc_t rsrc;
};

template <typename E>
__device__ __forceinline__ RowGeo<E> row_geo(const VerifyArgs& a, int r, bool valid) {
  constexpr int N = Elem<E>::kVec;
  RowGeo<E> g;
  g.row = static_cast<const E*>(a.logits) + static_cast<int64_t>(r) * a.ld;
  const uintptr_t addr = reinterpret_cast<uintptr_t>(g.row);
  g.head = static_cast<int>(((16u - (addr & 15u)) & 15u) / sizeof(E));
  if (g.head > a.V) g.head = a.V;
  g.nvec = (a.V - g.head) / N;
  g.boff = static_cast<uint32_t>(g.head * sizeof(E));
  g.rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<E*>(g.row), 0,
                                             valid ? static_cast<int>(a.V * sizeof(E)) : 0, 0x00020000);
  return g;
}

// Buffer offset no row reaches: a load through it returns zero without
// touching memory.
constexpr uint32_t kNoOffset = 0xFFFFFFF0u;

// Loads of chunk k: vectors k * CH + u * 64 + lane of the row's body, and the
// lane's edge element (lanes 0 .. 7: the head elements before the body, with
// the row's first chunk; lanes 8 .. 15: the tail elements after it, with the
// last chunk). Every load is issued unconditionally through the row's
// resource (what lies outside the row reads as zero and is masked where it
// is reduced), so no load sits behind a branch and the waits before a chunk
// is reduced count only the loads issued after it.
template <typename E, int U>
__device__ __forceinline__ void load_chunk(u32x4* dst, uint32_t& edge, const RowGeo<E>& g, int k, int cpr, int V,
                                           int lane) {
  constexpr int CH = kWave * U;
  constexpr int N = Elem<E>::kVec;
#pragma unroll
  for (int u = 0; u < U; ++u)
    dst[u] = __builtin_amdgcn_raw_buffer_load_b128(g.rsrc, g.boff + static_cast<uint32_t>((k * CH + u * kWave + lane) * 16),
                                                   0, 2 /* nt */);
  const int te = g.head + g.nvec * N + (lane - 8);
  uint32_t off = kNoOffset;
  off = (k == 0 && lane < g.head) ? static_cast<uint32_t>(lane * sizeof(E)) : off;
  off = (k == cpr - 1 && lane >= 8 && lane < 16 && te < V) ? static_cast<uint32_t>(te * sizeof(E)) : off;
  if constexpr (sizeof(E) == 2)
    edge = __builtin_amdgcn_raw_buffer_load_b16(g.rsrc, off, 0, 0);
  else
    edge = __builtin_amdgcn_raw_buffer_load_b32(g.rsrc, off, 0, 0);
}

template <typename E>
__device__ __forceinline__ float edge_value(uint32_t e) {
  return sizeof(E) == 2 ? __uint_as_float(e << 16) : __uint_as_float(e);
}

// Persistent greedy verification: one workgroup per CU, an equal contiguous
// range of chunks each, chunks handed to waves through an LDS counter. A wave
// keeps the partial of the row it is in and parks it in LDS when it moves on;
// the workgroup then stores one partial per row it touched (slot r + p).
template <typename E, int NT, int U, bool kRelaxed>
__global__ __launch_bounds__(NT) void verify_greedy_kernel(VerifyArgs a) {
  constexpr int NW = NT / kWave;
  constexpr int CH = kWave * U;
  static_assert(NW >= kPartWords, "one lane per partial field");
  __shared__ RowRed slots[kMaxLocalRows][NW];
  __shared__ float s_xd[kMaxLocalRows];
  __shared__ int s_d[kMaxLocalRows];
  __shared__ uint32_t s_info[kMaxLocalRows];
  __shared__ int s_next;
  __shared__ TailScratch tail;
  __shared__ int64_t s_lo[kMaxGroups + 1];

  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int p = blockIdx.x;
  const uint32_t tag = call_tag(a);
  // request ranges for the scan (used by the last workgroup only): loaded
  // now and staged in LDS right after streaming, where the wait is free
  const ReqRange first = load_range(a, tid);
  const ChunkPlan plan{static_cast<int64_t>(a.R) * a.cpr, static_cast<int>(gridDim.x), a.cpr};
  const int64_t lo = plan.lo(p), hi = plan.lo(p + 1);
  const int row_lo = static_cast<int>(lo / a.cpr);
  const int t_lo = static_cast<int>(lo - static_cast<int64_t>(row_lo) * a.cpr);  // first chunk's index in its row
  const int nch = static_cast<int>(hi - lo);
  const int nloc = nch > 0 ? static_cast<int>((hi - 1) / a.cpr) - row_lo + 1 : 0;

  for (int k = tid; k < nloc * NW; k += NT) slots[k / NW][k % NW] = RowRed{0.0, -INFINITY, INT32_MAX, -FLT_MAX, 0};
  if (tid == 0) s_next = 0;
  // Row information. Relaxed rows need the draft's own logit before their
  // chunks are reduced, so wave 0 gathers it first; otherwise the last wave
  // gathers the information of the rows whose first chunk is here while the
  // other waves stream (it joins them afterwards).
  auto gather_info = [&]() {
    if (lane < nloc) {
      const int r = row_lo + lane;
      const bool first = static_cast<int64_t>(r) * a.cpr >= lo;
      if (kRelaxed || first) {
        const RowMeta m = load_meta(a, r, a.owner[r]);
        int bits = 0;
        const uint32_t info = row_info(a, m, bits);
        if (first) {
          s_info[lane] = info;
          if (bits) set_flag(a, bits);
        }
        if (kRelaxed) {
          const E* row = static_cast<const E*>(a.logits) + static_cast<int64_t>(r) * a.ld;
          const bool dv = m.draft >= 0 && m.draft < a.V;
          s_d[lane] = dv ? m.draft : -1;
          s_xd[lane] = dv ? Elem<E>::at(row, m.draft) : INFINITY;
        }
      }
    }
  };
  if (kRelaxed && w == 0) gather_info();
  lds_barrier();
  if (!kRelaxed && w == NW - 1) gather_info();

  auto grab = [&]() -> int {
    int c = 0;
    if (lane == 0) c = atomicAdd(&s_next, 1);
    return __builtin_amdgcn_readfirstlane(c);
  };

  RowPartial pt;
  partial_init(pt);
  GroupKeep<U> keep{};
  int row = -1, row_head = 0, row_nvec = 0;
  float xd = INFINITY;
  int d = 0;
  constexpr float kLog2e = 1.4426950408889634f;
  auto flush = [&]() {
    if (row < 0) return;
    const int idx = lane_argmax<E, kWave, U>(pt, keep, row_head, row_nvec);
    const RowRed r = wave_red<kRelaxed>(RowRed{pt.s, pt.best, idx, pt.mc, kRelaxed ? pt.rank : 0});
    if (lane == 0) slots[row - row_lo][w] = r;
  };

  // A chunk handed to this wave: its number in the workgroup's range, its
  // row and index in the row, and that row's geometry. A wave's chunks come
  // in increasing order, so each position is the previous one moved forward
  // by the difference of the numbers. All of it is the same for every lane
  // and stays on the scalar unit.
  struct Slot {
    int c, r, k;
    RowGeo<E> g;
  };
  auto first_slot = [&](int c) {
    Slot sl;
    sl.c = c;
    const int t = t_lo + c;
    sl.r = row_lo + t / a.cpr;
    sl.k = t - (sl.r - row_lo) * a.cpr;
    sl.g = row_geo<E>(a, sl.r, c < nch);
    return sl;
  };
  auto after = [&](const Slot& prev, int c) {
    Slot sl;
    sl.c = c;
    const bool valid = c < nch;
    sl.r = prev.r;
    sl.k = prev.k + (valid ? c - prev.c : 0);
    while (sl.k >= a.cpr) {
      sl.k -= a.cpr;
      ++sl.r;
    }
    sl.g = (sl.r == prev.r && valid) ? prev.g : row_geo<E>(a, sl.r, valid);
    return sl;
  };
  auto process = [&](const Slot& sl, u32x4* w, uint32_t edge) {
    if (sl.r != row) {
      flush();
      partial_init(pt);
      row = sl.r;
      row_head = sl.g.head;
      row_nvec = sl.g.nvec;
      if (kRelaxed) {
        xd = s_xd[row - row_lo];
        d = s_d[row - row_lo];
      }
    }
    const int v0 = sl.k * CH + lane;
    const bool live = sl.c < nch;   // past the range: reduces nothing
    // the row's last chunk: its vectors past the body count as -inf (they
    // are masked after decoding; the load registers are never overwritten,
    // which would make the compiler wait for every load in flight)
    if (live && (sl.k + 1) * CH <= sl.g.nvec)
      take_group<E, U, kWave, kRelaxed>(pt, w, v0, sl.g.head, kLog2e, xd, d, keep);
    else
      take_group<E, U, kWave, kRelaxed, true>(pt, w, v0, sl.g.head, kLog2e, xd, d, keep, live ? sl.g.nvec : 0);
    if (!live) return;
    // elements outside the row's 16-byte body (misaligned rows or a vocab
    // that is not a multiple of the vector), loaded with the chunk
    if (sl.k == 0 && lane < sl.g.head) take_scalar<kRelaxed, true>(pt, edge_value<E>(edge), lane, kLog2e, xd, d);
    if (sl.k == a.cpr - 1) {
      const int e = sl.g.head + sl.g.nvec * Elem<E>::kVec + (lane - 8);
      if (lane >= 8 && lane < 16 && e < a.V) take_scalar<kRelaxed>(pt, edge_value<E>(edge), e, kLog2e, xd, d);
    }
  };

  // Two buffers in turn, no copies: while one chunk is reduced the other's
  // loads are in flight, and the next chunk number is fetched before the
  // reduction so its LDS round trip is hidden. Both halves run every
  // iteration (the loop's only exit is at its top), so every path into a
  // reduction has the same loads in flight and the compiler's waits count
  // exactly the other buffer's loads.
  Slot sa = first_slot(grab());
  u32x4 A[U], B[U];
  uint32_t ea, eb;
  load_chunk<E, U>(A, ea, sa.g, sa.k, a.cpr, a.V, lane);
  Slot sb = after(sa, grab());
  load_chunk<E, U>(B, eb, sb.g, sb.k, a.cpr, a.V, lane);
  while (sa.c < nch) {
    const int ca = grab();
    process(sa, A, ea);
    sa = after(sb, ca);
    load_chunk<E, U>(A, ea, sa.g, sa.k, a.cpr, a.V, lane);
    const int cb = grab();
    process(sb, B, eb);
    sb = after(sa, cb);
    load_chunk<E, U>(B, eb, sb.g, sb.k, a.cpr, a.V, lane);
  }
  flush();
  tail.first[tid] = first;
  lds_barrier();

  // one partial per row touched (slot r + p), a wave per row: its lanes
  // combine the waves' slots; the row information goes with the first
  for (int k = w; k < nloc; k += NW) {
    RowRed r = lane < NW ? slots[k][lane] : RowRed{0.0, -INFINITY, INT32_MAX, -FLT_MAX, 0};
    r = wave_red<kRelaxed>(r);
    const int rr = row_lo + k;
    const bool first = static_cast<int64_t>(rr) * a.cpr >= lo;
    if (lane < kPartWords) put_partial_field(a, static_cast<int64_t>(rr) + p, lane, r, first ? s_info[k] : kNoDraft, tag);
  }
  if (p == plan.P - 1) greedy_tail<NT, kRelaxed>(a, plan, tag, tail, s_lo);
}

// One workgroup per row part (a.parts = P parts per row, 1 <= P <=
// kMaxRowParts), for batches with more rows than CUs. The parts of a row
// are consecutive workgroups, each streaming an equal share of the row's
// 16-byte body (the first also takes the elements before it, the last those
// after it). Each part combines its threads (finish_row_lean). Parts
// 0 .. P - 2 store their statistics as tagged words and exit; the last
// part, dispatched after them (so its wait always ends), gathers them
// across one wave, merges them with its own, decides the row and hands its
// word to the scan run by the launch's last workgroup.
template <typename E, int NT, int U, bool kRelaxed>
__global__ __launch_bounds__(NT) void verify_greedy_rows_kernel(VerifyArgs a) {
  __shared__ LeanScratch<NT> scr;
  __shared__ TailScratch tail;
  __shared__ int s_prot[VSV_MAX_PROTECTED];
  static_assert(VSV_MAX_PROTECTED % NT == 0 || NT % VSV_MAX_PROTECTED == 0, "protected ids per thread");
  constexpr int kProtPer = VSV_MAX_PROTECTED >= NT ? VSV_MAX_PROTECTED / NT : 1;
  const int P = a.parts;
  const int r = static_cast<int>(blockIdx.x) / P;
  const int part = static_cast<int>(blockIdx.x) - r * P;
  const uint32_t tag = call_tag(a);
  const E* __restrict__ row = static_cast<const E*>(a.logits) + static_cast<int64_t>(r) * a.ld;
  // the part's elements [e0, e1): equal shares of the row's 16-byte body
  int e0, e1;
  part_range<E>(row, a.V, P, part, e0, e1);
  const bool last = part == P - 1;
  const int owner = a.owner[r];
  RowMeta m{-1, 0, 0, -1};
  float xd = INFINITY;
  if (kRelaxed) {
    m = load_meta(a, r, owner);
    if (m.draft >= 0 && m.draft < a.V) xd = Elem<E>::at(row, m.draft);
  }
  RowPartial p;
  partial_init(p);
  GroupKeep<U> keep{};
  constexpr float kLog2e = 1.4426950408889634f;
  // The last part gathers what the row's decision needs while the first
  // loads are in flight (values only, used after the stream): the row's
  // metadata and, for the relaxed variants, the draft's logit, the
  // request's generated-token count and its share of the protected ids.
  float xm = xd;
  int gen = 0;
  int prot_reg[kProtPer];
#pragma unroll
  for (int k = 0; k < kProtPer; ++k) prot_reg[k] = -1;
  auto hook = [&]() {
    if (last) {
      if (!kRelaxed) m = load_meta(a, r, owner);
      if (a.relax_var) {
        if (!kRelaxed && m.draft >= 0 && m.draft < a.V) xm = Elem<E>::at(row, m.draft);
        if (a.generated && m.req >= 0) gen = a.generated[m.req];
#pragma unroll
        for (int k = 0; k < kProtPer; ++k) {
          const int q = static_cast<int>(threadIdx.x) + k * NT;
          if (q < a.nprot) prot_reg[k] = a.prot[q];
        }
      }
    }
  };
  // element indices inside the part are relative to e0, so the draft's is too
  stream_row<E, NT, U, kRelaxed, GroupKeep<U>, decltype(hook), true>(row + e0, e1 - e0, kLog2e, xd,
                                                                      kRelaxed ? m.draft - e0 : 0, p, keep, hook);
  if (last && a.relax_var) {
#pragma unroll
    for (int k = 0; k < kProtPer; ++k) {
      const int q = static_cast<int>(threadIdx.x) + k * NT;
      if (q < VSV_MAX_PROTECTED) s_prot[q] = prot_reg[k];   // ordered by the epilogue's barriers
    }
  }
  const RowStats st = finish_row_lean<E, NT, U, kRelaxed>(p, scr, keep, row + e0, e1 - e0);
  const int idx = st.argmax == INT32_MAX ? INT32_MAX : e0 + st.argmax;
  uint64_t* slots = part_slots(a, r, P);
  if (!last) {
    put_part_stats(slots, part, st, idx, tag);
  } else if (threadIdx.x < kWave) {
    // wave 0: lane q < P - 1 gathers part q's words, lane P - 1 holds this
    // part's result, and one wave reduction merges them (largest max,
    // lowest index among equal maxima, sums rebased to the largest
    // reference, ranks added)
    const int lane = threadIdx.x;
    RowRed mine{0.0, -INFINITY, INT32_MAX, -FLT_MAX, 0};
    int stalled = 0;
    if (lane < P - 1) {
      mine = get_part_stats(slots, lane, tag, stalled);
    } else if (lane == P - 1) {
      mine = RowRed{st.sum, st.max, idx, st.mref, st.rank};
    }
    const RowRed red = wave_red<kRelaxed>(mine);
    stalled = wave_all(stalled, MaxOp());
    // relaxed variants: is the draft or the greedy token protected? (every
    // lane checks its share of the ids)
    bool prot = false;
    if (a.relax_var && a.nprot > 0) {
      bool hit = false;
      for (int k = lane; k < a.nprot; k += kWave) hit |= s_prot[k] == m.draft || s_prot[k] == red.idx;
      prot = __builtin_amdgcn_ballot_w64(hit) != 0;
    }
    if (lane == 0) {
      // the sum holds the maximum's own term (at least 1/2), so float log2
      // keeps the log-sum-exp within a few units of float rounding
      const float lse = 0.69314718f * (red.mc + __log2f(static_cast<float>(red.s)));
      int token = red.idx;
      int bits = stalled ? VSV_FLAG_STALLED : 0;
      if (!(red.best < INFINITY) || token == INT32_MAX || !isfinite(lse)) {
        bits |= VSV_FLAG_LOGITS;
        if (token == INT32_MAX) token = 0;
      }
      const bool ok = a.relax_var ? relaxed_ok(a, m, token, red.best, xm, red.rank, prot, gen)
                                  : (kRelaxed ? (red.rank < a.relaxed_k) : (m.draft == token));
      const uint32_t word = row_word(a, m, token, ok, bits);
      if (bits) set_flag(a, bits);
      if (a.row_token) a.row_token[r] = token;
      if (a.row_lse) a.row_lse[r] = lse;
      if (r != a.withheld_row) store_agent64(a.ws_row + r, tagged(tag, word));
    }
  }
  if (blockIdx.x == gridDim.x - 1) words_tail<NT>(a, tag, tail);
}

// Parts per row for the row kernel: about one part per kPartBytes of the
// row, at most kMaxRowParts, and no more partial slots than the workspace
// holds (R * (P - 1) <= max(R + kMaxGroups, kPartSlots)); rows too short
// for two such parts are halved where halves give the CUs a more even count
// of parts.
inline int row_parts(const VerifyArgs& a, int64_t row_bytes) {
#if VSV_FORCE_PARTS > 0
  int P = VSV_FORCE_PARTS;
#else
  int P = static_cast<int>((row_bytes + kPartBytes / 2) / kPartBytes);
#endif
  P = P < 1 ? 1 : (P > kMaxRowParts ? kMaxRowParts : P);
  const int64_t R = a.R > 0 ? a.R : 1;
  const int64_t slots = R + kMaxGroups > kPartSlots ? R + kMaxGroups : kPartSlots;
  const int64_t cap = 1 + slots / R;
  if (P > cap) P = static_cast<int>(cap);
  if (P == 1 && a.groups > 0 && 2 * R <= slots) {
    // ceil(R S / CUs) / (R S / CUs) closer to 1 with S = 2 than with S = 1
    const int64_t c = a.groups, r1 = R, r2 = 2 * R;
    const int64_t w1 = (r1 + c - 1) / c, w2 = (r2 + c - 1) / c;
    if (w2 * r1 < w1 * r2) P = 2;   // w2 / r2 < w1 / r1, exactly
  }
  return P;
}

template <typename E, bool kRelaxed>
static hipError_t launch_greedy_t(VerifyArgs a, hipStream_t s) {
  constexpr int N = Elem<E>::kVec;
  constexpr int CH = kWave * kUnroll;
  // the relaxed variants decide rows in the row kernel's merging lane only
  if (!a.relax_var && greedy_persistent(a.R, a.groups)) {
    const int nvmax = a.V / N;
    a.cpr = nvmax > 0 ? (nvmax + CH - 1) / CH : 1;
    verify_greedy_kernel<E, kGreedyThreads, kUnroll, kRelaxed><<<dim3(a.groups), dim3(kGreedyThreads), 0, s>>>(a);
  } else {
    a.parts = row_parts(a, static_cast<int64_t>(a.V) * static_cast<int64_t>(sizeof(E)));
    const int64_t grid = static_cast<int64_t>(a.R) * a.parts;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    verify_greedy_rows_kernel<E, kRowThreads, kUnrollRows, kRelaxed>
        <<<dim3(static_cast<unsigned>(grid)), dim3(kRowThreads), 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_verify_greedy(const VerifyArgs& a, hipStream_t s) {
  if (a.dtype == VSV_BF16)
    return a.relaxed_k > 1 ? launch_greedy_t<uint16_t, true>(a, s) : launch_greedy_t<uint16_t, false>(a, s);
  return a.relaxed_k > 1 ? launch_greedy_t<float, true>(a, s) : launch_greedy_t<float, false>(a, s);
}

// ---------------------------------------------------------------- workspace

__global__ void zero_words_kernel(uint32_t* p, size_t n) {
  for (size_t k = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; k < n;
       k += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[k] = 0u;
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  zero_words_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s>>>(static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

}  // namespace vsv
