// Router GEMM and top-k softmax.
//
// PLENA_Compiler PR #69, section "Group E": the router GEMM (x @ W_r) is a
// stage of its own.  PLENA_Simulator PR #97, section "C_SET_TOPK_REG":
// topk_softmax is generic in the expert count and in k.
//
// Kernels:
//   route_logits_bf16  x[T,H] @ W_r[H,E] on MFMA (16x16x32 bf16, fp32 accumulate),
//                      64 tokens x 64 experts per workgroup, optional fp32 bias.
//   route_logits_f32   the same product for float32 inputs, one thread per logit.
//   topk_softmax       one wave64 per token: k rounds of a wave arg-max under the
//                      key (logit descending, index ascending, NaN lowest), then
//                      a softmax over the k selected logits.
#include "moe_common.h"

#include <math.h>

namespace moe {
namespace {

constexpr int kRtBM = 64;   // tokens per workgroup
constexpr int kRtBN = 64;   // experts per workgroup
constexpr int kRtBK = 64;   // reduction slice per step
constexpr int kRtLds = 72;  // padded LDS row (bf16 elements)

__global__ __launch_bounds__(256) void route_logits_bf16(const bf16_t* __restrict__ x,
                                                         const bf16_t* __restrict__ w,
                                                         const float* __restrict__ bias, int T, int H,
                                                         int E, float* __restrict__ logits) {
  __shared__ __attribute__((aligned(16))) bf16_t sX[kRtBM * kRtLds];  // [token][k]
  __shared__ __attribute__((aligned(16))) bf16_t sW[kRtBN * kRtLds];  // [expert][k]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * kRtBM, e0 = blockIdx.y * kRtBN;
  f32x4 acc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < H; k0 += kRtBK) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int v = tid + 256 * i, r = v >> 3, ko = v & 7, gk = k0 + ko * 8;
      u32x4 val = u32x4{0u, 0u, 0u, 0u};
      if (t0 + r < T && gk < H) val = *(const u32x4*)(x + (int64_t)(t0 + r) * H + gk);
      *(u32x4*)(sX + r * kRtLds + ko * 8) = val;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int v = tid + 256 * i, kk = v >> 6, e = v & 63;
      bf16_t val = 0;
      if (k0 + kk < H && e0 + e < E) val = w[(int64_t)(k0 + kk) * E + e0 + e];
      sW[e * kRtLds + kk] = val;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4 a = *(const u32x4*)(sX + (wave * 16 + (lane & 15)) * kRtLds + ks * 32 + (lane >> 4) * 8);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const u32x4 b = *(const u32x4*)(sW + (nb * 16 + (lane & 15)) * kRtLds + ks * 32 + (lane >> 4) * 8);
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                          __builtin_bit_cast(bf16x8, b), acc[nb], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // 16x16 accumulator layout: row = 4*(lane/16) + r, column = lane%16.
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = t0 + wave * 16 + 4 * (lane >> 4) + r;
      const int col = e0 + nb * 16 + (lane & 15);
      if (row < T && col < E) {
        const float v = acc[nb][r];
        logits[(int64_t)row * E + col] = bias ? v + bias[col] : v;
      }
    }
  }
}

__global__ __launch_bounds__(256) void route_logits_f32(const float* __restrict__ x,
                                                        const float* __restrict__ w,
                                                        const float* __restrict__ bias, int T, int H,
                                                        int E, float* __restrict__ logits) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)T * E) return;
  const int t = (int)(i / E), e = (int)(i % E);
  float acc = 0.f;
  for (int h = 0; h < H; ++h) acc = fmaf(x[(int64_t)t * H + h], w[(int64_t)h * E + e], acc);
  logits[i] = bias ? acc + bias[e] : acc;
}

// True if candidate (v, e) ranks before (bv, be): larger value, then lower index.
__device__ __forceinline__ bool ranks_before(float v, int e, float bv, int be) {
  return v > bv || (v == bv && e < be);
}

__global__ __launch_bounds__(256) void topk_softmax(const float* __restrict__ logits, int T, int E, int k,
                                                    int32_t* __restrict__ ids, float* __restrict__ weights) {
  constexpr int kPer = kMaxExperts / kWave;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (int64_t)t * E;
  float key[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int e = lane + kWave * q;
    const float v = e < E ? row[e] : -INFINITY;
    key[q] = (v != v) ? -INFINITY : v;
  }
  uint32_t taken = 0;
  float my_sel = 0.f;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int e = lane + kWave * q;
      if (e < E && !((taken >> q) & 1u) && ranks_before(key[q], e, bv, be)) {
        bv = key[q];
        be = e;
      }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      const float ov = __shfl_xor(bv, d, kWave);
      const int oe = __shfl_xor(be, d, kWave);
      if (ranks_before(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == 0) ids[(int64_t)t * k + j] = be;
    if (lane == j) my_sel = row[be];
  }
  const float m = __shfl(my_sel, 0, kWave);
  const float ex = lane < k ? expf(my_sel - m) : 0.f;
  const float s = wave_sum(ex);
  if (lane < k) weights[(int64_t)t * k + lane] = ex / s;
}

}  // namespace
}  // namespace moe

namespace moe_launch {

hipError_t route(int dt, const void* x, const void* w_router, const float* bias, int T, int H, int E,
                 int top_k, int32_t* ids, float* weights, float* logits, hipStream_t s) {
  using namespace moe;
  if (dt == 1) {
    dim3 grid((T + kRtBM - 1) / kRtBM, (E + kRtBN - 1) / kRtBN);
    hipLaunchKernelGGL(route_logits_bf16, grid, dim3(256), 0, s, (const bf16_t*)x,
                       (const bf16_t*)w_router, bias, T, H, E, logits);
  } else {
    const int64_t n = (int64_t)T * E;
    hipLaunchKernelGGL(route_logits_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (const float*)x, (const float*)w_router, bias, T, H, E, logits);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(topk_softmax, dim3((T + 3) / 4), dim3(256), 0, s, (const float*)logits, T, E, top_k,
                     ids, weights);
  return hipGetLastError();
}

}  // namespace moe_launch
