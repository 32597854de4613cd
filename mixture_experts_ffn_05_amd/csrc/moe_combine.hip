// Weighted gather of routed outputs back to token order, and the shared-expert gate.
//
// VeOmni docs "Fused MoE Kernel Notes", section "Scatter/gather layout":
// moe_gather sums the routed expert outputs back to [tokens, hidden].  The
// hf-adapters PR #2 commit on the loop-on-topk decode combine replaces an
// index_add (a read-modify-write that breaks when indices repeat, and the k
// rows of one token all target that token) with a per-token reduction over
// the k slots.  gather_combine is that pull-form reduction: one workgroup per
// token reads its k rows with 16-byte loads and writes each output element
// once, so duplicate routes carry no write hazard and no atomics are needed.
//
// PLENA_Compiler PR #69, section "Group C -- shared experts": Qwen2-MoE's
// shared expert is scaled by sigmoid(x @ w_gate), one scalar per token.
// shared_gate computes that scalar: one wave64 per token, fp32 dot product.
#include "moe_common.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void gather_combine_k(const f32x4* __restrict__ y_rows,
                                                        const int32_t* __restrict__ scatter_index,
                                                        const float* __restrict__ weights, int T, int H, int k,
                                                        int accumulate, f32x4* __restrict__ y) {
  __shared__ int32_t s_idx[kMaxTopK];
  __shared__ float s_w[kMaxTopK];
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    s_idx[threadIdx.x] = scatter_index[(int64_t)t * k + threadIdx.x];
    s_w[threadIdx.x] = weights ? weights[(int64_t)t * k + threadIdx.x] : 1.0f;
  }
  __syncthreads();
  const int hv = H / 4;
  // Two 16-byte columns per thread at a time (c and c + 256), and for each the
  // slots in batches of 8: all loads of a batch, for both columns, are issued
  // before its adds, which still run in slot order.  Each routed row is read
  // once (non-temporal loads).
  for (int c0 = threadIdx.x; c0 < hv; c0 += 512) {
    const int c1 = c0 + 256;
    const bool has1 = c1 < hv;
    f32x4 sum0 = accumulate ? y[(int64_t)t * hv + c0] : f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 sum1 = accumulate && has1 ? y[(int64_t)t * hv + c1] : f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < k; j0 += 8) {
      f32x4 v0[8], v1[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u;
        const int r = j < k ? s_idx[j] : -1;
        const f32x4* row = y_rows + (int64_t)r * hv;
        v0[u] = r >= 0 ? __builtin_nontemporal_load(row + c0) : f32x4{0.f, 0.f, 0.f, 0.f};
        v1[u] = r >= 0 && has1 ? __builtin_nontemporal_load(row + c1) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u;
        if (j < k && s_idx[j] >= 0) {
          sum0 += s_w[j] * v0[u];
          sum1 += s_w[j] * v1[u];
        }
      }
    }
    y[(int64_t)t * hv + c0] = sum0;
    if (has1) y[(int64_t)t * hv + c1] = sum1;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void shared_gate_k(const T* __restrict__ x, const T* __restrict__ w_gate, int Tn,
                                                     int H, float* __restrict__ gate) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  float s = 0.f;
  for (int h = lane; h < H; h += kWave) s = fmaf(load_as_f32(x, (int64_t)t * H + h), load_as_f32(w_gate, h), s);
  s = wave_sum(s);
  if (lane == 0) gate[t] = sigmoidf_(s);
}

}  // namespace
}  // namespace moe

namespace moe_launch {

hipError_t gather_combine(const float* y_rows, const int32_t* scatter_index, const float* weights, int T, int H,
                          int top_k, int accumulate, float* y, hipStream_t s) {
  using namespace moe;
  hipLaunchKernelGGL(gather_combine_k, dim3(T), dim3(256), 0, s, (const f32x4*)y_rows, scatter_index, weights, T, H,
                     top_k, accumulate, (f32x4*)y);
  return hipGetLastError();
}

hipError_t shared_gate(int dt, const void* x, const void* w_gate, int T, int H, float* gate, hipStream_t s) {
  using namespace moe;
  const dim3 grid((T + 3) / 4);
  if (dt == 1)
    hipLaunchKernelGGL(shared_gate_k<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)x, (const bf16_t*)w_gate, T, H,
                       gate);
  else
    hipLaunchKernelGGL(shared_gate_k<float>, grid, dim3(256), 0, s, (const float*)x, (const float*)w_gate, T, H, gate);
  return hipGetLastError();
}

}  // namespace moe_launch
