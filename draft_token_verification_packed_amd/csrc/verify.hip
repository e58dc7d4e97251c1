// Greedy verification kernel (gfx950): one workgroup per row part. Each
// part streams its share of the row and stores its statistics; the row's
// last part merges them, decides the row's token and acceptance and stores
// the row's word (emitted token, accept bit); the launch's last workgroup
// runs the per-request scan (verify_common.hpp). No atomics on global
// memory.
#include "verify_common.hpp"

namespace vsv {

// ---------------------------------------------------------------- greedy

// One workgroup per row part (a.parts = P parts per row, 1 <= P <=
// kMaxRowParts). The parts of a row are consecutive workgroups, each
// streaming an equal share of the row's 16-byte body (the first also takes
// the elements before it, the last those after it). Each part combines its
// threads (finish_row_lean). Parts
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

// Parts per row: about one part per kPartBytes of the row or, for batches
// too small to give every CU a few workgroups, enough parts for about
// kPartsPerCU * CUs / 2 workgroups in all (parts of at least kMinPartBytes);
// at most kMaxRowParts, and no more partial slots than the workspace holds
// (R * (P - 1) <= part_slot_count(R)). Rows too short for two parts are
// halved where halves give the CUs a more even count of parts.
inline int row_parts(const VerifyArgs& a, int64_t row_bytes) {
#if VSV_FORCE_PARTS > 0
  int P = VSV_FORCE_PARTS;
#else
  int P = static_cast<int>((row_bytes + kPartBytes / 2) / kPartBytes);
#endif
  P = P < 1 ? 1 : (P > kMaxRowParts ? kMaxRowParts : P);
#if VSV_FORCE_PARTS == 0
  if (a.cus > 0 && a.R > 0) {
    int64_t want = static_cast<int64_t>(a.cus) * kPartsPerCU / 2 / a.R;
    const int64_t most = row_bytes / kMinPartBytes;
    if (want > most) want = most;
    if (want > kMaxRowParts) want = kMaxRowParts;
    if (want > P) P = static_cast<int>(want);
  }
#endif
  const int64_t R = a.R > 0 ? a.R : 1;
  const int64_t slots = static_cast<int64_t>(part_slot_count(a.R));
  const int64_t cap = 1 + slots / R;
  if (P > cap) P = static_cast<int>(cap);
  if (P == 1 && a.cus > 0 && 2 * R <= slots) {
    // ceil(R S / CUs) / (R S / CUs) closer to 1 with S = 2 than with S = 1
    const int64_t c = a.cus, r1 = R, r2 = 2 * R;
    const int64_t w1 = (r1 + c - 1) / c, w2 = (r2 + c - 1) / c;
    if (w2 * r1 < w1 * r2) P = 2;   // w2 / r2 < w1 / r1, exactly
  }
  return P;
}

template <typename E, bool kRelaxed>
static hipError_t launch_greedy_t(VerifyArgs a, hipStream_t s) {
  a.parts = row_parts(a, static_cast<int64_t>(a.V) * static_cast<int64_t>(sizeof(E)));
  const int64_t grid = static_cast<int64_t>(a.R) * a.parts;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  verify_greedy_rows_kernel<E, kRowThreads, kUnrollRows, kRelaxed>
      <<<dim3(static_cast<unsigned>(grid)), dim3(kRowThreads), 0, s>>>(a);
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
