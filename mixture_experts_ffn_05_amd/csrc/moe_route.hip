// Router GEMM and top-k softmax.
//
// PLENA_Compiler PR #69, section "Group E": the router GEMM (x @ W_r) is a
// stage of its own.  PLENA_Simulator PR #97, section "C_SET_TOPK_REG":
// topk_softmax is generic in the expert count and in k.
//
// Kernels:
//   router_transpose_bf16  W_r [H,E] -> [E_pad,H] in the caller's workspace, so that
//                          both operands of the router product are K-contiguous.
//   router_logits_mfma     x[T,H] @ W_r on MFMA (16x16x32 bf16, fp32 accumulate),
//                          16 tokens x 64 experts per workgroup, split-K over its
//                          4 waves with a fixed-order reduction, optional fp32 bias.
//   route_logits_f32       the same product for float32 inputs, one thread per logit.
//   topk_softmax       one wave64 per token: k rounds of a wave arg-max under the
//                      key (logit descending, index ascending, NaN lowest), then
//                      a softmax over the k selected logits.
#include "moe_common.h"

#include <math.h>

namespace moe {
namespace {

constexpr int kRtTok = 16;   // tokens per workgroup
constexpr int kRtExp = 64;   // experts per workgroup (4 MFMA column blocks of 16)

int padded_experts(int E) { return (E + 15) / 16 * 16; }

// W_r [H, E] (E contiguous) -> wt [E_pad, H] (H contiguous), zero rows for e >= E.
__global__ __launch_bounds__(256) void router_transpose_bf16(const bf16_t* __restrict__ w, int H, int E, int E_pad,
                                                             bf16_t* __restrict__ wt) {
  __shared__ bf16_t tile[64][65];
  const int h0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int hh = i >> 6, ee = i & 63;
    const int h = h0 + hh, e = e0 + ee;
    tile[hh][ee] = (h < H && e < E) ? w[(int64_t)h * E + e] : (bf16_t)0;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int ee = i >> 6, hh = i & 63;
    const int h = h0 + hh, e = e0 + ee;
    if (h < H && e < E_pad) wt[(int64_t)e * H + h] = tile[hh][ee];
  }
}

// logits[t, e] for 16 tokens x 64 experts per workgroup.  Both MFMA operands are
// K-contiguous (x rows and the transposed router rows), so each lane loads its
// 16x16x32 fragments straight from global memory; the 4 waves split H into
// quarters and their partial sums are added in a fixed order through LDS.
__global__ __launch_bounds__(256) void router_logits_mfma(const bf16_t* __restrict__ x,
                                                          const bf16_t* __restrict__ wt,
                                                          const float* __restrict__ bias, int T, int H, int E,
                                                          int E_pad, float* __restrict__ logits) {
  __shared__ float red[4][kRtTok][kRtExp + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * kRtTok, e0 = blockIdx.y * kRtExp;
  const int nblk = min(4, (E_pad - e0) / 16);
  const int kq = ((H + 127) / 128) * 32;   // per-wave share of H, a multiple of 32
  const int kbeg = wave * kq, kend = min(H, kbeg + kq);
  const int row = t0 + (lane & 15);
  const int koff = (lane >> 4) * 8;
  const bool row_ok = row < T;
  const bf16_t* xr = x + (int64_t)(row_ok ? row : 0) * H;
  f32x4 acc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k = kbeg; k < kend; k += 32) {
    const int kk = k + koff;
    const bool k_ok = kk < kend;
    const u32x4 a = (row_ok && k_ok) ? *(const u32x4*)(xr + kk) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      if (nb < nblk) {
        const int e = e0 + nb * 16 + (lane & 15);
        const u32x4 b = k_ok ? *(const u32x4*)(wt + (int64_t)e * H + kk) : u32x4{0u, 0u, 0u, 0u};
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                          __builtin_bit_cast(bf16x8, b), acc[nb], 0, 0, 0);
      }
    }
  }
  // 16x16 accumulator layout: row = 4*(lane/16) + r, column = lane%16.
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][4 * (lane >> 4) + r][nb * 16 + (lane & 15)] = acc[nb][r];
  __syncthreads();
  for (int i = tid; i < kRtTok * kRtExp; i += 256) {
    const int tt = i / kRtExp, ee = i % kRtExp;
    const int t = t0 + tt, e = e0 + ee;
    if (t < T && e < E) {
      const float v = ((red[0][tt][ee] + red[1][tt][ee]) + red[2][tt][ee]) + red[3][tt][ee];
      logits[(int64_t)t * E + e] = bias ? v + bias[e] : v;
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

size_t route_workspace_bytes(int dt, int H, int E) {
  if (dt != 1) return 0;
  return (size_t)moe::padded_experts(E) * H * sizeof(moe::bf16_t);
}

hipError_t route(int dt, const void* x, const void* w_router, const float* bias, int T, int H, int E,
                 int top_k, int32_t* ids, float* weights, float* logits, void* workspace, hipStream_t s) {
  using namespace moe;
  if (dt == 1) {
    const int E_pad = padded_experts(E);
    bf16_t* wt = (bf16_t*)workspace;
    hipLaunchKernelGGL(router_transpose_bf16, dim3((H + 63) / 64, (E_pad + 63) / 64), dim3(256), 0, s,
                       (const bf16_t*)w_router, H, E, E_pad, wt);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    dim3 grid((T + kRtTok - 1) / kRtTok, (E_pad + kRtExp - 1) / kRtExp);
    hipLaunchKernelGGL(router_logits_mfma, grid, dim3(256), 0, s, (const bf16_t*)x, (const bf16_t*)wt, bias, T, H,
                       E, E_pad, logits);
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
