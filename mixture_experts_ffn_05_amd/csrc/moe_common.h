// Shared device and host helpers for libmoe's gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "libmoe.h"

namespace moe {

// Raw 16-bit storage of a bfloat16 value.
typedef uint16_t bf16_t;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;

__device__ __forceinline__ float bf16_to_f32(uint32_t v) { return __uint_as_float(v << 16); }

// float32 -> bfloat16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float load_as_f32(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_as_f32(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

__device__ __forceinline__ void store_from_f32(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_from_f32(bf16_t* p, int64_t i, float v) {
  p[i] = (bf16_t)f32_to_bf16_rne(v);
}

// silu(g) * u with silu(g) = g / (1 + exp(-g)), in fp32.
__device__ __forceinline__ float swiglu(float g, float u) { return g / (1.0f + expf(-g)) * u; }

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + expf(-z)); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Bits of lanes below the calling lane.
__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ int wave_inclusive_scan(int v) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int o = __shfl_up(v, d, kWave);
    if (lane_id() >= d) v += o;
  }
  return v;
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = max(v, __shfl_xor(v, d, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;
}

// NV independent fixed-order sums, v[j] = sum over z = 0 .. n-1 of
// p[j][z * stride] (0 where valid[j] is false).  Each batch of B slices issues
// the loads of every sum before adding them, so the NV sums cost about the load
// latency of one; each sum still adds its slices in the order z = 0, 1, ...
template <int NV, int B>
__device__ __forceinline__ void sum_slices_n(const float* const (&p)[NV], const bool (&valid)[NV], int64_t stride,
                                             int n, float (&v)[NV]) {
#pragma unroll
  for (int j = 0; j < NV; ++j) v[j] = 0.f;
  for (int z = 0; z < n; z += B) {
    float a[NV][B];
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
      for (int u = 0; u < B; ++u) a[j][u] = (valid[j] && z + u < n) ? p[j][(int64_t)(z + u) * stride] : 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
      for (int u = 0; u < B; ++u)
        if (z + u < n) v[j] += a[j][u];
  }
}

// Fixed-order sum over z of p[z * stride], z = 0 .. n-1, eight loads in flight.
__device__ __forceinline__ float sum_slices(const float* __restrict__ p, int64_t stride, int n) {
  float v = 0.f;
  int z = 0;
  for (; z + 8 <= n; z += 8) {
    float a[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) a[u] = p[(int64_t)(z + u) * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) v += a[u];
  }
  for (; z < n; ++z) v += p[(int64_t)z * stride];
  return v;
}

// ---- LDS rings fed by direct loads (global_load_lds: HBM -> LDS, no register round trip) ----

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define MOE_LDS(T, ptr) ((__attribute__((address_space(3))) T*)(ptr))
#define MOE_GLOBAL(T, ptr) ((const __attribute__((address_space(1))) T*)(ptr))

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for an LDS ring.  __syncthreads() (and a fence on LDS
// alone) makes the compiler wait for every outstanding direct load first --
// they count as vector-memory operations -- which would drain the ring.  The
// ring's loads are waited for explicitly with wait_vmcnt before this barrier;
// the "memory" clobber keeps the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The 8 consecutive-k bf16 values of an MFMA B fragment from two
// ds_read_b64_tr_b16 reads (k 0-3 and k 4-7).
__device__ __forceinline__ u32x4 pack_tr_pair(i16x4 lo, i16x4 hi) {
  return u32x4{(uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16),
               (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16),
               (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16),
               (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16)};
}

}  // namespace moe

// Host-side launchers implemented in the kernel translation units.  Each
// returns hipSuccess or the launch error; arguments were validated by the API.
namespace moe_launch {

size_t route_workspace_bytes(int dt, int T, int H, int E);
bool router_small(int dt, int T, int E);
hipError_t route_partials_small(const void* x, const void* w_router, int T, int H, int E, void* workspace,
                                int* nsplit, hipStream_t s);
bool route_scatter_fusable(int T, int top_k, int E);
hipError_t route_scatter_fused(int dt, const float* partial, int nsplit, const float* bias, float* logits, int T,
                               int H, int E, int top_k, int32_t* ids, float* weights, const void* x,
                               int32_t* scatter_index, int32_t* row_token, int32_t* offsets, int32_t* status_words,
                               void* x_scattered, hipStream_t s);
hipError_t route(int dt, const void* x, const void* w_router, const float* bias, int T, int H, int E,
                 int top_k, int32_t* ids, float* weights, float* logits, void* workspace, hipStream_t s);

size_t scatter_workspace_bytes(int T, int top_k, int E);
hipError_t build_scatter(int dt, const void* x, const int32_t* ids, int T, int H, int E, int top_k,
                         int32_t* scatter_index, int32_t* row_token, int32_t* offsets,
                         int32_t* status_words, void* x_scattered, void* workspace, hipStream_t s);

// Grouped GEMMs.  `offsets` may be null: one group of `rows` rows.
// `role` (0 routed experts, 1 shared expert) only selects a separately named
// kernel instantiation so that profiles tell the two apart.
// bt: weight layout, 0 = [K, N] per group (N contiguous), 1 = [N, K] (K contiguous).
// a_rows (optional): routed row r of the product is row a_rows[r] of `a`, which has a_src_rows rows
// (gather-on-load: `a` is then the layer input x and a_rows the scatter's row_token).
hipError_t grouped_swiglu_fc1(int dt, int bt, const void* a, const int32_t* offsets, int groups, int rows,
                              const void* w1, int64_t w1_group_stride, int K, int I, void* act,
                              int role, int cu_count, hipStream_t s, const int32_t* a_rows = nullptr,
                              int a_src_rows = 0);
hipError_t grouped_fc2(int dt, int bt, const void* act, const int32_t* offsets, int groups, int rows,
                       const void* w2, int64_t w2_group_stride, int K, int N, float* out,
                       const float* row_scale, int accumulate, int plain_store, int role, int cu_count,
                       hipStream_t s);

// MXFP8 weights (e4m3 codes [N, K] per group, e8m0 scales per 8 along the
// intermediate axis: [2I / 8, K] for fc1, [N, K / 8] for fc2); K a multiple of 128.
hipError_t grouped_swiglu_fc1_mx8(const void* a, const int32_t* offsets, int groups, int rows, const void* w1q,
                                  const void* w1s, int K, int I, void* act, int role, int cu_count, hipStream_t s);
hipError_t grouped_fc2_mx8(const void* act, const int32_t* offsets, int groups, int rows, const void* w2q,
                           const void* w2s, int K, int N, float* out, const float* row_scale, int accumulate,
                           int plain_store, int role, int cu_count, hipStream_t s);

hipError_t fused_fc1_mx8(const void* xs, const int32_t* offsets, int E, int R, const void* w1q, const void* w1s,
                         int H, int I, void* act, const void* x, int T, const void* ws1q, const void* ws1s, int I_s,
                         void* act_s, int cu_count, hipStream_t s);
hipError_t fused_fc2_mx8(const void* act, const int32_t* offsets, int E, int R, const void* w2q, const void* w2s,
                         int I, int H, float* y_rows, const void* act_s, int T, const void* ws2q, const void* ws2s,
                         int I_s, const float* gate, int accumulate, float* y, int cu_count, hipStream_t s);

// Routed groups and the shared expert in one launch (bf16, reduction sizes
// multiples of 64, and a shared expert that is light next to the routed
// weights; fused_supported() decides from the shapes).
bool fused_supported(int dt, int H, int I, int I_s, int E, int R, int T);
// moe_tile_config of the routed experts' launch of fc1 (call 0) or fc2 (call 1); I_s > 0: the *_and_shared call.
int tile_config(int dt, int call, int R, int H, int E, int I, int T, int I_s, int cu_count);
hipError_t fused_fc1(int bt, const void* xs, const int32_t* offsets, int E, int R, const void* w1, int H, int I,
                     void* act, const void* x, int T, const void* ws1, int I_s, void* act_s, int cu_count,
                     hipStream_t s, const int32_t* a_rows = nullptr);
hipError_t fused_fc2(int bt, const void* act, const int32_t* offsets, int E, int R, const void* w2, int I, int H,
                     float* y_rows, const void* act_s, int T, const void* ws2, int I_s, const float* gate,
                     int accumulate, float* y, int cu_count, hipStream_t s);

// weights may be null: every slot then counts with weight 1 (the backward's gather of input gradients).
hipError_t gather_combine(const float* y_rows, const int32_t* scatter_index, const float* weights,
                          int T, int H, int top_k, int accumulate, float* y, hipStream_t s);

// Backward of the routed experts (routes fixed).  wt_nk: 0 = weights stored
// [K, N] per group as in the forward (x @ W), 1 = [N, K].
hipError_t grouped_swiglu_fc1_save(int dt, int bt, const void* a, const int32_t* offsets, int groups, int rows,
                                   const void* w1, int64_t w1_group_stride, int K, int I, void* act, void* h_pre,
                                   int cu_count, hipStream_t s);
hipError_t scatter_grad(int dt, const float* dy, const float* y_rows, const float* weights,
                        const int32_t* scatter_index, int T, int H, int top_k, int R, void* d_rows, float* d_weights,
                        hipStream_t s);
hipError_t grouped_fc2_dgrad_swiglu(int dt, int wt_nk, const void* d_rows, const int32_t* offsets, int groups,
                                    int rows, const void* w2, int I, int H, const void* h_pre, void* d_h,
                                    int cu_count, hipStream_t s);
hipError_t grouped_fc1_dgrad(int dt, int wt_nk, const void* d_h, const int32_t* offsets, int groups, int rows,
                             const void* w1, int H, int I, float* d_xs, int cu_count, hipStream_t s);
// out[g] = P[rows of g]^T Q[rows of g]: P [rows, M], Q [rows, N], out [groups, M, N] (element type of dt).
// role (1: fc1's weight gradient, 2: fc2's) only selects a separately named kernel for profiles.
hipError_t grouped_wgrad(int dt, const void* P, const void* Q, const int32_t* offsets, int groups, int rows, int M,
                         int N, void* out, int role, int cu_count, hipStream_t s);
hipError_t shared_gate(int dt, const void* x, const void* w_gate, int T, int H, float* gate,
                       hipStream_t s);

}  // namespace moe_launch
