// Device helpers shared by the verification kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <float.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

namespace vsv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- elements
// A row is streamed in 16-byte vectors: 4 float32 or 8 bfloat16 logits.

template <typename E> struct Elem;

template <> struct Elem<float> {
  static constexpr int kVec = 4;
  __device__ static __forceinline__ u32x4 neg_inf() { return u32x4{0xFF800000u, 0xFF800000u, 0xFF800000u, 0xFF800000u}; }
  __device__ static __forceinline__ float at(const float* p, int64_t i) { return p[i]; }
  __device__ static __forceinline__ void decode(const u32x4& w, float* f) {
    f[0] = __uint_as_float(w.x);
    f[1] = __uint_as_float(w.y);
    f[2] = __uint_as_float(w.z);
    f[3] = __uint_as_float(w.w);
  }
};

// bfloat16 is the top half of a float32: the low element of a 32-bit word
// is widened by a shift, the high one by masking.
template <> struct Elem<uint16_t> {
  static constexpr int kVec = 8;
  __device__ static __forceinline__ u32x4 neg_inf() { return u32x4{0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u}; }
  __device__ static __forceinline__ float at(const uint16_t* p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
  }
  __device__ static __forceinline__ void decode(const u32x4& w, float* f) {
    f[0] = __uint_as_float(w.x << 16);
    f[1] = __uint_as_float(w.x & 0xFFFF0000u);
    f[2] = __uint_as_float(w.y << 16);
    f[3] = __uint_as_float(w.y & 0xFFFF0000u);
    f[4] = __uint_as_float(w.z << 16);
    f[5] = __uint_as_float(w.z & 0xFFFF0000u);
    f[6] = __uint_as_float(w.w << 16);
    f[7] = __uint_as_float(w.w & 0xFFFF0000u);
  }
};

// Streaming load: the logits are read exactly once, so keep them out of
// the caches' way (nt bit).
__device__ __forceinline__ u32x4 load_stream(const u32x4* p) {
  return __builtin_nontemporal_load(p);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- cross-workgroup data
// Data one workgroup hands to another inside a launch moves only through
// agent-scope relaxed atomic loads and stores: on gfx950 these are sc1
// accesses, coherent across the XCDs' separate L2 caches, so no device-wide
// fence (an L2 write-back plus invalidate per workgroup) is needed.

__device__ __forceinline__ void store_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_agent(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory access this wave issued has completed (on gfx950
// stores are counted in vmcnt, so this includes their acknowledgement).
__device__ __forceinline__ void wait_memory() { __builtin_amdgcn_s_waitcnt(0); }
__device__ __forceinline__ void store_agent64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_agent64(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- barriers

// Workgroup barrier for LDS traffic. The kernels exchange data between waves
// only through LDS (global words between workgroups carry tags and are
// polled), so a barrier needs to order LDS operations alone. A full
// __syncthreads also waits for every global store and load the wave has in
// flight (on this architecture one counter covers both), which puts a
// memory round trip on the critical path wherever results were just stored.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------- reductions

struct MaxOp {
  template <typename T> __device__ __forceinline__ T operator()(T a, T b) const { return a > b ? a : b; }
};
struct MinOp {
  template <typename T> __device__ __forceinline__ T operator()(T a, T b) const { return a < b ? a : b; }
};
struct SumOp {
  template <typename T> __device__ __forceinline__ T operator()(T a, T b) const { return a + b; }
};

// Wave-wide exchanges without LDS. A DPP move reads another lane's register
// in the same instruction; lanes whose source lies outside the pattern (or
// whose row is masked off) read 0. 64-bit values move as two halves.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ int dpp_move(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, false);
}
template <int CTRL, int ROWS = 0xF, typename T>
__device__ __forceinline__ T dpp_val(T x) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, dpp_move<CTRL, ROWS>(__builtin_bit_cast(int, x)));
  } else {
    const int2 h = __builtin_bit_cast(int2, x);
    int2 o;
    o.x = dpp_move<CTRL, ROWS>(h.x);
    o.y = dpp_move<CTRL, ROWS>(h.y);
    return __builtin_bit_cast(T, o);
  }
}
template <typename T>
__device__ __forceinline__ T read_lane(T x, int lane) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
  } else {
    const int2 h = __builtin_bit_cast(int2, x);
    int2 o;
    o.x = __builtin_amdgcn_readlane(h.x, lane);
    o.y = __builtin_amdgcn_readlane(h.y, lane);
    return __builtin_bit_cast(T, o);
  }
}

// Reduction over the wave: row rotations by 8, 4, 2 and 1 lanes give every
// lane the value of its row of 16, and four lane reads combine the rows as
// (row0 op row1) op (row2 op row3). The result is uniform (every lane holds
// it). Every lane of the wave must be active.
template <typename T, typename Op>
__device__ __forceinline__ T wave_all(T v, Op op) {
  v = op(v, dpp_val<0x128>(v));
  v = op(v, dpp_val<0x124>(v));
  v = op(v, dpp_val<0x122>(v));
  v = op(v, dpp_val<0x121>(v));
  return op(op(read_lane(v, 0), read_lane(v, 16)), op(read_lane(v, 32), read_lane(v, 48)));
}
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  return wave_all(v, op);
}
__device__ __forceinline__ double wave_sum_f64(double v) { return wave_all(v, SumOp()); }

// Every thread receives the reduction of `v` over the block. `scratch` holds
// NT / 64 values; the leading barrier makes back-to-back calls safe.
template <int NT, typename T, typename Op>
__device__ __forceinline__ T block_reduce(T v, Op op, T* scratch) {
  v = wave_reduce(v, op);
  lds_barrier();
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[threadIdx.x / kWave] = v;
  lds_barrier();
  T r = scratch[0];
#pragma unroll
  for (int w = 1; w < NT / kWave; ++w) r = op(r, scratch[w]);
  return r;
}

// Inclusive prefix sum over the wave: right shifts by 1, 2, 4 and 8 lanes
// scan each row of 16, then row broadcasts carry the last lane of row 0
// into row 1 and of row 2 into row 3 (broadcast 15), and the last lane of
// row 1 into rows 2 and 3 (broadcast 31). Every lane must be active.
template <typename T>
__device__ __forceinline__ T wave_scan_incl(T v) {
  v += dpp_val<0x111>(v);
  v += dpp_val<0x112>(v);
  v += dpp_val<0x114>(v);
  v += dpp_val<0x118>(v);
  v += dpp_val<0x142, 0xA>(v);
  v += dpp_val<0x143, 0xC>(v);
  return v;
}

__device__ __forceinline__ int wave_inclusive_scan(int v) { return wave_scan_incl(v); }

// Exclusive prefix sum over the block; `total` receives the block sum.
// `scratch` holds NT / 64 ints.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int& total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int incl = wave_inclusive_scan(v);
  lds_barrier();
  if (lane == kWave - 1) scratch[w] = incl;
  lds_barrier();
  int before = 0, sum = 0;
#pragma unroll
  for (int k = 0; k < NT / kWave; ++k) {
    const int s = scratch[k];
    before += (k < w) ? s : 0;
    sum += s;
  }
  total = sum;
  return before + incl - v;
}

// ---------------------------------------------------------------- Philox
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two
// 32x32->64 multiplies whose halves are XOR-mixed with the other counter
// words and the key; the key is bumped by two Weyl constants between rounds.

struct Philox4 { uint32_t x, y, z, w; };

__device__ __forceinline__ Philox4 philox4x32_10(Philox4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = 0xD2511F53u * c.x;
    const uint32_t hi0 = __umulhi(0xD2511F53u, c.x);
    const uint32_t lo1 = 0xCD9E8D57u * c.z;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c.z);
    c = Philox4{hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0};
  }
  return c;
}

// Uniform on the 2^-24 grid in [0, 1) for (request, local row).
__device__ __forceinline__ double row_uniform(uint64_t seed, uint64_t offset, int request, int row) {
  const Philox4 o = philox4x32_10(
      Philox4{static_cast<uint32_t>(row), static_cast<uint32_t>(request),
              static_cast<uint32_t>(offset), static_cast<uint32_t>(offset >> 32)},
      static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
  return static_cast<double>(o.x >> 8) * (1.0 / 16777216.0);
}

}  // namespace vsv
