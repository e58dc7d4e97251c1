// Packed draft-token verification kernels (gfx950).
//
// One launch verifies a whole ragged batch. Workgroup r streams target row r
// once from HBM and decides the row's target token and whether the row's
// draft token is accepted. The workgroup that finishes last (device-scope
// ticket) then runs the per-request prefix-accept scan, the exclusive scan of
// emitted lengths over the batch and the scatter of emitted tokens, so no
// second launch and no host round trip is needed (the pages' verifier keeps
// packing boundaries on the device: xLLM docs, "Adaptive speculative
// inference", DSpark section "Launch example").
#include "kernels.hpp"
#include "row_stream.hpp"
#if VSV_HAVE_SAMPLED
#include "sampled_row.hpp"
#endif

namespace vsv {

// Per-row metadata: request, local row, draft token.
struct RowMeta {
  int req;    // owning request (-1 if the owner map is inconsistent)
  int j;      // local row within the request
  int K;      // draft rows of the request
  int draft;  // draft token for verify rows, -1 otherwise
};

__device__ __forceinline__ RowMeta load_meta(const VerifyArgs& a, int r) {
  RowMeta m{-1, 0, 0, -1};
  const int i = a.owner[r];
  if (i < 0 || i >= a.B) return m;
  const int r0 = a.offsets[i];
  const int r1 = a.offsets[i + 1];
  if (r < r0 || r >= r1) return m;
  m.req = i;
  m.j = r - r0;
  m.K = r1 - r0 - 1;
  if (m.j < m.K) {
    const int q = r - i;
    m.draft = (q >= 0 && q < a.R - a.B) ? a.drafts[q] : -1;
  }
  return m;
}

__device__ __forceinline__ void set_flag(const VerifyArgs& a, int bits) {
  if (a.error_flag) atomicOr(a.error_flag, bits);
}

// The last workgroup to finish: prefix-accept scan per request, exclusive
// scan of (a_i + 1) over the batch, scatter of the emitted tokens.
template <int NT>
__device__ void batch_tail(const VerifyArgs& a, int* scr) {
  const int tid = threadIdx.x;
  int carry = 0;
  for (int base = 0; base < a.B; base += NT) {
    const int i = base + tid;
    int acc = 0, nxt = 0, r0 = 0, len = 0;
    bool ok = false;
    if (i < a.B) {
      r0 = a.offsets[i];
      const int r1 = a.offsets[i + 1];
      ok = r0 >= 0 && r1 > r0 && r1 <= a.R && (i != 0 || r0 == 0) && (i != a.B - 1 || r1 == a.R);
      if (ok) {
        const int K = r1 - r0 - 1;
        while (acc < K && a.ws_row_acc[r0 + acc]) ++acc;
        nxt = a.ws_row_token[r0 + acc];
      } else {
        set_flag(a, VSV_FLAG_LAYOUT);
      }
      len = acc + 1;
    }
    int total = 0;
    const int pos = carry + block_exclusive_scan<NT>(len, scr, total);
    if (i < a.B) {
      a.accepted_len[i] = acc;
      a.next_token[i] = nxt;
      a.out_offsets[i] = pos;
      if (ok && r0 >= i) {
        // r0 - i + q indexes the request's drafts; the bound also holds for
        // offsets that are consistent locally but not across the batch
        const int nd = a.R - a.B;
        for (int q = 0; q < acc && pos + q < a.R && r0 - i + q < nd; ++q)
          a.out_tokens[pos + q] = a.drafts[r0 - i + q];
      }
      if (pos + acc < a.R) a.out_tokens[pos + acc] = nxt;
    }
    carry += total;
  }
  if (tid == 0) {
    a.out_offsets[a.B] = carry;
    *a.ws_ticket = 0;  // leave the workspace zeroed for the next call
  }
}

// Publish this row's decision and, if this is the last row, run the tail.
template <int NT>
__device__ __forceinline__ void finish_and_maybe_tail(const VerifyArgs& a, int r, int token, int accept,
                                                      int* scr) {
  __shared__ int s_last;
  if (threadIdx.x == 0) {
    a.ws_row_token[r] = token;
    a.ws_row_acc[r] = accept;
    __threadfence();
    const int t = atomicAdd(a.ws_ticket, 1);
    s_last = (t == a.R - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  batch_tail<NT>(a, scr);
}

template <typename E, int NT, int U, bool kRelaxed>
__global__ __launch_bounds__(NT) void verify_greedy_kernel(VerifyArgs a) {
  __shared__ float scr_f[NT / kWave];
  __shared__ int scr_i[NT / kWave];
  __shared__ double scr_d[NT / kWave];
  const int r = blockIdx.x;
  const E* __restrict__ row = static_cast<const E*>(a.logits) + static_cast<int64_t>(r) * a.ld;

  RowMeta m;
  float xd = INFINITY;
  if (kRelaxed) {
    // the rank test needs the draft's own logit before streaming
    m = load_meta(a, r);
    if (m.draft >= 0 && m.draft < a.V) xd = Elem<E>::at(row, m.draft);
  }
  RowPartial p;
  partial_init(p);
  constexpr float kLog2e = 1.4426950408889634f;
  stream_row<E, NT, U, kRelaxed>(row, a.V, kLog2e, xd, kRelaxed ? m.draft : 0, p);
  if (!kRelaxed) m = load_meta(a, r);
  const RowResult res = finish_row<E, NT>(row, p, scr_f, scr_i, scr_d);

  int token = res.argmax;
  int accept = 0;
  if (threadIdx.x == 0) {
    int bits = 0;
    if (!(res.max < INFINITY) || token == INT32_MAX || !isfinite(res.lse)) {
      bits |= VSV_FLAG_LOGITS;
      if (token == INT32_MAX) token = 0;
    }
    if (m.req < 0) bits |= VSV_FLAG_LAYOUT;
    if (m.req >= 0 && m.j < m.K) {
      if (m.draft < 0 || m.draft >= a.V) {
        bits |= VSV_FLAG_TOKEN;
      } else {
        accept = kRelaxed ? (res.rank < a.relaxed_k) : (m.draft == token);
      }
    }
    if (bits) set_flag(a, bits);
    if (a.row_token) a.row_token[r] = token;
    if (a.row_lse) a.row_lse[r] = static_cast<float>(res.lse);
  }
  finish_and_maybe_tail<NT>(a, r, token, accept, scr_i);
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
#if VSV_HAVE_SAMPLED

template <typename E, int NT, int U>
__global__ __launch_bounds__(NT) void verify_sampled_kernel(VerifyArgs a) {
  __shared__ float scr_f[NT / kWave];
  __shared__ int scr_i[NT / kWave];
  __shared__ double scr_d[NT / kWave];
  const int r = blockIdx.x;
  const E* __restrict__ row = static_cast<const E*>(a.logits) + static_cast<int64_t>(r) * a.ld;
  const RowMeta m = load_meta(a, r);
  int token = 0, accept = 0;
  const int req = m.req < 0 ? 0 : m.req;
  const float T = a.temperature[req];
  if (m.req >= 0 && T > 0.f) {
    token = sampled_row<E, NT, U>(a, row, m.req, m.j, T, scr_f, scr_i, scr_d);
  } else {
    RowPartial p;
    partial_init(p);
    constexpr float kLog2e = 1.4426950408889634f;
    stream_row<E, NT, U, false>(row, a.V, kLog2e, INFINITY, 0, p);
    const RowResult res = finish_row<E, NT>(row, p, scr_f, scr_i, scr_d);
    token = res.argmax;
    if (threadIdx.x == 0) {
      int bits = 0;
      if (!(res.max < INFINITY) || token == INT32_MAX || !isfinite(res.lse)) {
        bits |= VSV_FLAG_LOGITS;
        if (token == INT32_MAX) token = 0;
      }
      if (!(T >= 0.f)) bits |= VSV_FLAG_PARAMS;
      if (bits) set_flag(a, bits);
      if (a.row_token) a.row_token[r] = token;
      if (a.row_lse) a.row_lse[r] = static_cast<float>(res.lse);
    }
  }
  if (threadIdx.x == 0) {
    if (m.req < 0) set_flag(a, VSV_FLAG_LAYOUT);
    if (m.req >= 0 && m.j < m.K) {
      if (m.draft < 0 || m.draft >= a.V)
        set_flag(a, VSV_FLAG_TOKEN);
      else
        accept = (m.draft == token);
    }
  }
  finish_and_maybe_tail<NT>(a, r, token, accept, scr_i);
}

template <typename E>
static hipError_t launch_sampled_t(const VerifyArgs& a, hipStream_t s) {
  verify_sampled_kernel<E, kVerifyThreads, kUnroll><<<dim3(a.R), dim3(kVerifyThreads), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_verify_sampled(const VerifyArgs& a, hipStream_t s) {
  return a.dtype == VSV_BF16 ? launch_sampled_t<uint16_t>(a, s) : launch_sampled_t<float>(a, s);
}
#else
hipError_t launch_verify_sampled(const VerifyArgs&, hipStream_t) { return hipErrorNotSupported; }
#endif

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
