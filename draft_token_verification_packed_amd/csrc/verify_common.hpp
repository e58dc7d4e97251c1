// Pieces shared by the verification kernels (gfx950): call tags, row
// metadata, row words and the per-request scan that ends every launch.
//
// One launch verifies a whole ragged batch; packing boundaries stay on the
// device and nothing waits on the host (xLLM docs, "Adaptive speculative
// inference", DSpark section "Launch example").
//
// The per-request scan: prefix-accept count per request, exclusive scan of
// emitted lengths over the batch, scatter of emitted tokens. Words handed
// between workgroups carry the call's tag, so nothing has to be cleared
// after a call.
#pragma once

#include "kernels.hpp"
#include "row_stream.hpp"

namespace vsv {

constexpr uint32_t kAcceptBit = 0x80000000u;
constexpr uint32_t kTokenMask = 0x3FFFFFFFu;
constexpr uint32_t kNoDraft = kTokenMask;     // never a valid token (vocab < 2^30)
// Polls one thread of a tail may spend waiting, over all the words it reads
// (each poll waits for a load from the device-coherent level, about a
// microsecond): past it the tail stops waiting, uses what it has and flags
// the launch, so the grid always drains within a fraction of a second.
constexpr int kPollBudget = 1 << 18;

// ---------------------------------------------------------------- call tags

// The tag of this call: derived from the workspace's call counter, never 0
// and different from the previous 2^31 - 1 calls' tags.
__device__ __forceinline__ uint32_t call_tag(const VerifyArgs& a) {
  return ((load_agent(a.ws_epoch) + 1u) & 0x7FFFFFFFu) | 0x80000000u;
}
__device__ __forceinline__ uint64_t tagged(uint32_t tag, uint32_t v) {
  return (static_cast<uint64_t>(tag) << 32) | v;
}
// Wait (within the thread's poll budget) for the word at `w` to carry `tag`.
__device__ __forceinline__ uint32_t poll_tagged(const uint64_t* w, uint32_t tag, int& budget, int& stalled) {
  uint64_t x = load_agent64(w);
  while (static_cast<uint32_t>(x >> 32) != tag && budget > 0) {
    --budget;
    __builtin_amdgcn_s_sleep(2);
    x = load_agent64(w);
  }
  stalled |= (static_cast<uint32_t>(x >> 32) == tag) ? 0 : 1;
  return static_cast<uint32_t>(x);
}
// The last workgroup ends the call: the next call uses the next tag.
__device__ __forceinline__ void end_call(const VerifyArgs& a, uint32_t tag) {
  if (threadIdx.x == 0) store_agent(a.ws_epoch, tag & 0x7FFFFFFFu);
}

// ---------------------------------------------------------------- row parts

// A row streamed in P parts by P workgroups: its 16-byte body cut into
// equal shares (the first part also takes the elements before the body, the
// last those after it). Part p holds elements [e0, e1).
template <typename E>
__device__ __forceinline__ void part_range(const E* row, int V, int P, int part, int& e0, int& e1) {
  constexpr int N = Elem<E>::kVec;
  e0 = 0;
  e1 = V;
  if (P > 1) {
    const uintptr_t addr = reinterpret_cast<uintptr_t>(row);
    int head = static_cast<int>(((16u - (addr & 15u)) & 15u) / sizeof(E));
    if (head > V) head = V;
    const int64_t nv = (V - head) / N;
    e0 = part == 0 ? 0 : head + static_cast<int>(nv * part / P) * N;
    e1 = part == P - 1 ? V : head + static_cast<int>(nv * (part + 1) / P) * N;
  }
}

// Words of a part's statistics (row-major in the workspace's partials area,
// parts 0 .. P - 2 of row r at slots r * (P - 1) + p, kPartStatWords words
// per slot): max, its lowest index, exponent reference, the float64 sum as
// two halves, rank count.
constexpr int kPartStatWords = kPartWords;
__device__ __forceinline__ uint64_t* part_slots(const VerifyArgs& a, int r, int P) {
  return a.ws_part + static_cast<size_t>(r) * (P - 1) * kPartStatWords;
}
// Store part `part`'s statistics (threads 0 .. kPartStatWords - 1, one
// tagged word each); idx is the row-relative index of the part's maximum.
__device__ __forceinline__ void put_part_stats(uint64_t* slots, int part, const RowStats& st, int idx, uint32_t tag) {
  if (threadIdx.x < kPartStatWords) {
    const uint64_t sb = __builtin_bit_cast(uint64_t, st.sum);
    const uint32_t v[kPartStatWords] = {__float_as_uint(st.max), static_cast<uint32_t>(idx),
                                        __float_as_uint(st.mref), static_cast<uint32_t>(sb),
                                        static_cast<uint32_t>(sb >> 32), static_cast<uint32_t>(st.rank)};
    uint32_t mine = v[0];
#pragma unroll
    for (int f = 1; f < kPartStatWords; ++f) mine = threadIdx.x == f ? v[f] : mine;
    store_agent64(slots + static_cast<size_t>(part) * kPartStatWords + threadIdx.x, tagged(tag, mine));
  }
}
// Lane q < P - 1 of the merging wave: part q's statistics, polled until
// they carry the call's tag (within the poll budget; `stalled` records a
// give-up).
__device__ __forceinline__ RowRed get_part_stats(const uint64_t* slots, int q, uint32_t tag, int& stalled) {
  const uint64_t* hw = slots + static_cast<size_t>(q) * kPartStatWords;
  uint64_t w[kPartStatWords];
  auto load_all = [&]() {
#pragma unroll
    for (int f = 0; f < kPartStatWords; ++f) w[f] = load_agent64(hw + f);
  };
  auto complete = [&]() {
    bool ok = true;
#pragma unroll
    for (int f = 0; f < kPartStatWords; ++f) ok = ok && static_cast<uint32_t>(w[f] >> 32) == tag;
    return ok;
  };
  int budget = kPollBudget;
  load_all();
  while (!complete() && budget > 0) {
    --budget;
    __builtin_amdgcn_s_sleep(2);
    load_all();
  }
  stalled = complete() ? 0 : 1;
  const uint64_t sb = (static_cast<uint64_t>(static_cast<uint32_t>(w[4])) << 32) | static_cast<uint32_t>(w[3]);
  return RowRed{__builtin_bit_cast(double, sb), __uint_as_float(static_cast<uint32_t>(w[0])),
                static_cast<int>(static_cast<uint32_t>(w[1])), __uint_as_float(static_cast<uint32_t>(w[2])),
                static_cast<int>(static_cast<uint32_t>(w[5]))};
}

// ---------------------------------------------------------------- rows

// Per-row metadata: request, local row, draft token.
struct RowMeta {
  int req;    // owning request (-1 if the owner map is inconsistent)
  int j;      // local row within the request
  int K;      // draft rows of the request
  int draft;  // draft token for verify rows, -1 otherwise
};

// Metadata of row r whose owner entry has already been read as `i`.
__device__ __forceinline__ RowMeta load_meta(const VerifyArgs& a, int r, int i) {
  RowMeta m{-1, 0, 0, -1};
  if (i < 0 || i >= a.B) return m;
  const int r0 = a.offsets[i];
  const int r1 = a.offsets[i + 1];
  const int q = r - i;
  const int dq = (q >= 0 && q < a.R - a.B) ? a.drafts[q] : -1;
  if (r < r0 || r >= r1) return m;
  m.req = i;
  m.j = r - r0;
  m.K = r1 - r0 - 1;
  m.draft = (m.j < m.K) ? dq : -1;
  return m;
}

// A row's request parameters, loaded at the owner entry's request (request
// 0 if the entry is out of range) together with the row's metadata: both
// depend only on the owner entry, so the loads go out in one round trip.
// They are the request's own wherever the metadata confirms the owner
// (m.req >= 0, and then m.req == owner).
struct ReqParams {
  float T;
  int top_k;
  float top_p, min_p;
};
__device__ __forceinline__ ReqParams load_params(const VerifyArgs& a, int owner) {
  const int i = (owner >= 0 && owner < a.B) ? owner : 0;
  return ReqParams{a.temperature[i], a.top_k[i], a.top_p[i], a.min_p[i]};
}

__device__ __forceinline__ void set_flag(const VerifyArgs& a, int bits) {
  if (a.error_flag) atomicOr(a.error_flag, bits);
}

// The word a row hands to the scan: the draft (accepted) or its own target
// token. Flags layout and token-range problems in `bits`.
__device__ __forceinline__ uint32_t row_word(const VerifyArgs& a, const RowMeta& m, int token, bool accept_ok,
                                             int& bits) {
  if (m.req < 0) {
    bits |= VSV_FLAG_LAYOUT;
    return static_cast<uint32_t>(token);
  }
  if (m.j < m.K) {
    if (m.draft < 0 || m.draft >= a.V) {
      bits |= VSV_FLAG_TOKEN;
    } else if (accept_ok) {
      return static_cast<uint32_t>(m.draft) | kAcceptBit;
    }
  }
  return static_cast<uint32_t>(token);
}

// Relaxed greedy acceptance of row (request m.req, draft position m.j):
// the greedy token always passes; another draft passes only past the
// position and generated-token gates, when neither it nor the greedy token
// is protected, and when top-K (rank below relaxed_k) or the margin
// (max - x[d] < margin, in double) holds. Out-of-range drafts are rejected
// by row_word.
__device__ __forceinline__ bool relaxed_ok(const VerifyArgs& a, const RowMeta& m, int token, float best, float xd,
                                           int rank, bool prot, int gen) {
  if (m.draft == token) return true;
  if (m.j < a.from_pos || static_cast<int64_t>(gen) + m.j < static_cast<int64_t>(a.after_tok)) return false;
  if (prot) return false;
  if (a.relaxed_k > 1 && rank < a.relaxed_k) return true;
  return a.margin > 0.f && static_cast<double>(best) - static_cast<double>(xd) < static_cast<double>(a.margin);
}

// ---------------------------------------------------------------- scan

// Rows whose words the scan stages in LDS.
constexpr int kTailStage = 4096;

// Row offsets of request i and the next one.
struct ReqRange {
  int r0, r1;
};

// LDS of the per-request scan: the words of the first STAGE rows, the
// block scan's per-wave sums, and the ranges of the first NT requests
// (staged early).
template <int NT, int STAGE>
struct TailScratchT {
  static constexpr int kStage = STAGE;
  uint32_t words[STAGE];
  int scan[16];
  ReqRange first[NT];
};
using TailScratch = TailScratchT<1024, kTailStage>;

// The tails load the ranges of the first NT requests early and stage them
// in LDS, so the scan never waits on a global load: on this architecture
// such a wait would also wait for every store issued before it.
__device__ __forceinline__ ReqRange load_range(const VerifyArgs& a, int i) {
  return i < a.B ? ReqRange{a.offsets[i], a.offsets[i + 1]} : ReqRange{0, 0};
}

// Per-request scan over the row words (token | kAcceptBit if the row's draft
// was accepted): prefix-accept count, exclusive scan of (a_i + 1), scatter of
// the emitted tokens. `word(r)` returns row r's word; `first` holds the range
// of request tid.
template <int NT, typename Scratch, typename Word>
__device__ __forceinline__ void scan_requests(const VerifyArgs& a, Scratch& t, Word word) {
  const int tid = threadIdx.x;
  int carry = 0;
  // Requests go to the threads from the top down (request base + k to thread
  // NT - 1 - k): the rows were handled from thread 0 up, so with R + B <= NT
  // the scanning waves have no loads or stores of their own in flight, and
  // none of their waits stalls behind the row outputs just stored. Emitted
  // positions then come from a suffix scan over the threads.
  auto block = [&](int base, const ReqRange& rg) {
    const int i = base + (NT - 1 - tid);
    int acc = 0, r0 = 0, len = 0;
    uint32_t nxt = 0;
    bool ok = false;
    if (i < a.B) {
      r0 = rg.r0;
      const int r1 = rg.r1;
      ok = r0 >= 0 && r1 > r0 && r1 <= a.R && (i != 0 || r0 == 0) && (i != a.B - 1 || r1 == a.R);
      if (ok) {
        const int K = r1 - r0 - 1;
        while (acc < K && (word(r0 + acc) & kAcceptBit)) ++acc;
        nxt = word(r0 + acc);
      } else {
        set_flag(a, VSV_FLAG_LAYOUT);
      }
      len = acc + 1;
    }
    int total = 0;
    const int before = block_exclusive_scan<NT>(len, t.scan, total);
    // lengths of this block's requests below i: threads above this one
    const int pos = carry + total - before - len;
    if (i < a.B) {
      const int nt = static_cast<int>(nxt & kTokenMask);
      a.accepted_len[i] = acc;
      a.next_token[i] = nt;
      a.out_offsets[i] = pos;
      if (ok)
        for (int q = 0; q < acc && pos + q < a.R; ++q) a.out_tokens[pos + q] = static_cast<int>(word(r0 + q) & kTokenMask);
      if (pos + acc < a.R) a.out_tokens[pos + acc] = nt;
    }
    carry += total;
  };
  // the first NT requests use the ranges staged in LDS; the block is peeled
  // so that no load of a later block shares its path
  block(0, t.first[NT - 1 - tid]);
  for (int base = NT; base < a.B; base += NT) block(base, load_range(a, base + (NT - 1 - tid)));
  if (tid == 0) a.out_offsets[a.B] = carry;
}

// Run by the workgroup that ends the launch when rows are handled by one
// workgroup each: gather every row's word (the first kTailStage in LDS,
// later ones where they are read) and run the per-request scan.
// Gather the words of rows [0, n) into LDS: each thread loads its words
// kGatherBatch at a time, all loads of a batch in flight together, and polls
// again only the words not yet tagged for this call, so a thread waits one
// round trip per batch instead of one per word.
constexpr int kGatherBatch = 8;
template <int NT>
__device__ __forceinline__ void gather_words(const VerifyArgs& a, uint32_t tag, uint32_t* words, int n, int& budget,
                                             int& stalled) {
  const int tid = threadIdx.x;
  for (int k0 = tid; k0 < n; k0 += NT * kGatherBatch) {
    uint64_t w[kGatherBatch];
#pragma unroll
    for (int b = 0; b < kGatherBatch; ++b) {
      const int k = k0 + b * NT;
      w[b] = load_agent64(a.ws_row + (k < n ? k : 0));
    }
#pragma unroll
    for (int b = 0; b < kGatherBatch; ++b) {
      const int k = k0 + b * NT;
      if (k < n) {
        uint32_t v = static_cast<uint32_t>(w[b]);
        if (static_cast<uint32_t>(w[b] >> 32) != tag) v = poll_tagged(a.ws_row + k, tag, budget, stalled);
        words[k] = v;
      }
    }
  }
}

template <int NT, typename Scratch>
__device__ __forceinline__ void words_tail(const VerifyArgs& a, uint32_t tag, Scratch& t) {
  constexpr int kStage = Scratch::kStage;
  const int tid = threadIdx.x;
  t.first[tid] = load_range(a, tid);
  int stalled = 0, budget = kPollBudget;
  const int staged = min(a.R, kStage);
  gather_words<NT>(a, tag, t.words, staged, budget, stalled);
  lds_barrier();
  if (a.R <= kStage)
    scan_requests<NT>(a, t, [&](int row) -> uint32_t { return t.words[row]; });
  else
    scan_requests<NT>(a, t, [&](int row) -> uint32_t {
      return row < staged ? t.words[row] : poll_tagged(a.ws_row + row, tag, budget, stalled);
    });
  if (stalled) set_flag(a, VSV_FLAG_STALLED);
  end_call(a, tag);
}

}  // namespace vsv
