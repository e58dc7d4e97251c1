// Packed draft-token verification kernels (gfx950).
//
// One launch verifies a whole ragged batch. Workgroup r streams target row r
// once from HBM and decides the row's target token and whether the row's
// draft token is accepted. It publishes one word per row (the token the row
// would emit, with the top bit set when its draft was accepted) and takes a
// ticket; the workgroup that draws the last ticket runs the per-request
// prefix-accept scan, the exclusive scan of emitted lengths over the batch
// and the scatter of emitted tokens. No second launch and no host round trip
// are needed: packing boundaries stay on the device (xLLM docs, "Adaptive
// speculative inference", DSpark section "Launch example").
#include "kernels.hpp"
#include "row_stream.hpp"
#include "sampled_row.hpp"

namespace vsv {

constexpr uint32_t kAcceptBit = 0x80000000u;

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

__device__ __forceinline__ void set_flag(const VerifyArgs& a, int bits) {
  if (a.error_flag) atomicOr(a.error_flag, bits);
}

// Rows whose words the tail stages in LDS with one round of loads.
constexpr int kTailStage = 4096;

struct TailScratch {
  uint32_t words[kTailStage];
  int scan[16];
};

// The last workgroup to finish: prefix-accept scan per request, exclusive
// scan of (a_i + 1) over the batch, scatter of the emitted tokens. The words
// of the first kTailStage rows are staged in LDS in the same round of loads
// as the row offsets (row 0 of request 0 is row 0), so a batch of up to that
// many rows costs one round trip; later rows are read directly.
template <int NT>
__device__ void batch_tail(const VerifyArgs& a, TailScratch& t) {
  const int tid = threadIdx.x;
  const int staged = min(a.R, kTailStage);
  for (int k = tid; k < staged; k += NT) t.words[k] = load_agent(a.ws_row + k);
  __syncthreads();
  auto word = [&](int row) -> uint32_t { return row < staged ? t.words[row] : load_agent(a.ws_row + row); };
  int carry = 0;
  for (int base = 0; base < a.B; base += NT) {
    const int i = base + tid;
    int acc = 0, r0 = 0, len = 0;
    uint32_t nxt = 0;
    bool ok = false;
    if (i < a.B) {
      r0 = a.offsets[i];
      const int r1 = a.offsets[i + 1];
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
    const int pos = carry + block_exclusive_scan<NT>(len, t.scan, total);
    if (i < a.B) {
      const int nt = static_cast<int>(nxt & ~kAcceptBit);
      a.accepted_len[i] = acc;
      a.next_token[i] = nt;
      a.out_offsets[i] = pos;
      if (ok)
        for (int q = 0; q < acc && pos + q < a.R; ++q) a.out_tokens[pos + q] = static_cast<int>(word(r0 + q) & ~kAcceptBit);
      if (pos + acc < a.R) a.out_tokens[pos + acc] = nt;
    }
    carry += total;
  }
  if (tid == 0) {
    a.out_offsets[a.B] = carry;
    store_int_agent(a.ws_ticket, 0);  // leave the workspace zeroed for the next call
  }
}

// Publish this row's word and, if this is the last row, run the tail.
template <int NT>
__device__ __forceinline__ void publish_and_maybe_tail(const VerifyArgs& a, int r, uint32_t word, TailScratch& tail) {
  __shared__ int s_last;
  if (threadIdx.x == 0) {
    store_agent(a.ws_row + r, word);
    wait_memory();
    s_last = (ticket_agent(a.ws_ticket) == a.R - 1);
  }
  __syncthreads();
  if (s_last) batch_tail<NT>(a, tail);
}

// The word a row publishes: the draft (accepted) or its own target token.
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

template <typename E, int NT, int U, bool kRelaxed>
__global__ __launch_bounds__(NT) void verify_greedy_kernel(VerifyArgs a) {
  __shared__ RowScratch<NT> scr;
  __shared__ TailScratch tail;
  const int r = blockIdx.x;
  const E* __restrict__ row = static_cast<const E*>(a.logits) + static_cast<int64_t>(r) * a.ld;
  const int owner = a.owner[r];

  RowMeta m{-1, 0, 0, -1};
  float xd = INFINITY;
  if (kRelaxed) {
    // the rank test needs the draft's own logit before streaming
    m = load_meta(a, r, owner);
    if (m.draft >= 0 && m.draft < a.V) xd = Elem<E>::at(row, m.draft);
  }
  RowPartial p;
  partial_init(p);
  constexpr float kLog2e = 1.4426950408889634f;
  stream_row<E, NT, U, kRelaxed>(row, a.V, kLog2e, xd, kRelaxed ? m.draft : 0, p, [&]() {
    if (!kRelaxed) m = load_meta(a, r, owner);
  });
  const RowResult res = finish_row<E, NT, U, kRelaxed>(p, scr, row);

  uint32_t word = 0;
  if (threadIdx.x == 0) {
    int token = res.argmax;
    int bits = 0;
    if (!(res.max < INFINITY) || token == INT32_MAX || !isfinite(res.lse)) {
      bits |= VSV_FLAG_LOGITS;
      if (token == INT32_MAX) token = 0;
    }
    const bool ok = kRelaxed ? (res.rank < a.relaxed_k) : (m.draft == token);
    word = row_word(a, m, token, ok, bits);
    if (bits) set_flag(a, bits);
    if (a.row_token) a.row_token[r] = token;
    if (a.row_lse) a.row_lse[r] = static_cast<float>(res.lse);
  }
  publish_and_maybe_tail<NT>(a, r, word, tail);
}

template <typename E>
static hipError_t launch_greedy_t(const VerifyArgs& a, hipStream_t s) {
  const dim3 grid(a.R), block(kVerifyThreads);
  if (a.relaxed_k > 1)
    verify_greedy_kernel<E, kVerifyThreads, kUnroll, true><<<grid, block, 0, s>>>(a);
  else
    verify_greedy_kernel<E, kVerifyThreads, kUnroll, false><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_verify_greedy(const VerifyArgs& a, hipStream_t s) {
  return a.dtype == VSV_BF16 ? launch_greedy_t<uint16_t>(a, s) : launch_greedy_t<float>(a, s);
}

// ---------------------------------------------------------------- sampled

// Rows of requests with temperature > 0 draw their token (sampled_row.hpp);
// rows of greedy requests take the arg-max exactly as verify_greedy does.
// Acceptance is strict: the draft must equal the row's token.
template <typename E, int NT, int U>
__global__ __launch_bounds__(NT) void verify_sampled_kernel(VerifyArgs a) {
  __shared__ SampledLds<NT> L;
  static_assert(sizeof(TailScratch) <= sizeof(L.elem), "tail staging aliases the candidate buffers");
  const int r = blockIdx.x;
  const E* __restrict__ row = static_cast<const E*>(a.logits) + static_cast<int64_t>(r) * a.ld;
  const RowMeta m = load_meta(a, r, a.owner[r]);
  const float T = a.temperature[m.req < 0 ? 0 : m.req];
  int token = 0, bits = 0, slow = 0;
  double lse = 0.0;
  if (m.req >= 0 && T > 0.f) {
    const SampledOut o = sampled_row<E, NT, U>(a, row, m.req, m.j, T, L, NoHook());
    token = o.token;
    lse = o.lse;
    bits = o.bits;
    slow = o.slow;
  } else {
    RowPartial p;
    partial_init(p);
    constexpr float kLog2e = 1.4426950408889634f;
    stream_row<E, NT, U, false>(row, a.V, kLog2e, INFINITY, 0, p);
    const RowResult res = finish_row<E, NT, U, false>(p, L.rs, row);
    token = res.argmax;
    lse = res.lse;
    if (!(res.max < INFINITY) || token == INT32_MAX || !isfinite(res.lse)) bits |= VSV_FLAG_LOGITS;
    if (token == INT32_MAX) token = 0;
    if (m.req >= 0 && !(T >= 0.f)) bits |= VSV_FLAG_PARAMS;
  }
  uint32_t word = 0;
  if (threadIdx.x == 0) {
    word = row_word(a, m, token, m.draft == token, bits);
    if (bits) set_flag(a, bits);
    if (slow && a.slow_rows) atomicAdd(a.slow_rows, 1);
    if (a.row_token) a.row_token[r] = token;
    if (a.row_lse) a.row_lse[r] = static_cast<float>(lse);
  }
  publish_and_maybe_tail<NT>(a, r, word, *reinterpret_cast<TailScratch*>(&L.elem[0][0]));
}

template <typename E>
static hipError_t launch_sampled_t(const VerifyArgs& a, hipStream_t s) {
  verify_sampled_kernel<E, kVerifyThreads, kUnroll><<<dim3(a.R), dim3(kVerifyThreads), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_verify_sampled(const VerifyArgs& a, hipStream_t s) {
  return a.dtype == VSV_BF16 ? launch_sampled_t<uint16_t>(a, s) : launch_sampled_t<float>(a, s);
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
