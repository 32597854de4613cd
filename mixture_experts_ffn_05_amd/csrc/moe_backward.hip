// Backward of the routed combine: the output gradient scattered into the
// expert-grouped rows, and the route weights' gradient.
//
// VeOmni docs "Fused MoE Kernel Notes", section "Backward grouped-GEMM launch
// bound": the fc2 output gradient is moe_scatter of the layer's output
// gradient through scatter_index.  The forward combine weights row
// r = scatter_index[t, j] by w[t, j], so that row's gradient is w[t, j] * dy[t],
// and the gradient of w[t, j] is the dot product dy[t] . y_rows[r].  One
// workgroup per token reads dy[t] once per slot (it stays in L1/L2) and its k
// rows with 16-byte loads; the dot product is reduced in a fixed order (lanes,
// then waves in index order), so results do not depend on timing.
#include "moe_common.h"

namespace moe {
namespace {

__device__ __forceinline__ void store4(float* p, f32x4 v) { *(f32x4*)p = v; }
__device__ __forceinline__ void store4(bf16_t* p, f32x4 v) {
  *(u32x2*)p = u32x2{f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16),
                     f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16)};
}

template <typename T>
__global__ __launch_bounds__(256) void scatter_grad_k(const f32x4* __restrict__ dy, const f32x4* __restrict__ y_rows,
                                                      const float* __restrict__ weights,
                                                      const int32_t* __restrict__ scatter_index, int H, int k, int R,
                                                      T* __restrict__ d_rows, float* __restrict__ d_weights) {
  __shared__ int32_t s_idx[kMaxTopK];
  __shared__ float s_w[kMaxTopK];
  __shared__ float s_part[kMaxTopK][4];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < k) {
    const int r = scatter_index[(int64_t)t * k + tid];
    s_idx[tid] = (r >= 0 && r < R) ? r : -1;
    s_w[tid] = weights[(int64_t)t * k + tid];
  }
  __syncthreads();
  const int hv = H / 4;
  const f32x4* dyt = dy + (int64_t)t * hv;
  for (int j = 0; j < k; ++j) {
    const int r = s_idx[j];
    if (r < 0) continue;  // uniform across the workgroup
    const float w = s_w[j];
    const f32x4* yr = y_rows + (int64_t)r * hv;
    T* dr = d_rows + (int64_t)r * H;
    float part = 0.f;
    for (int c = tid; c < hv; c += 256) {
      const f32x4 g = dyt[c];
      const f32x4 y = yr[c];
      part += g[0] * y[0] + g[1] * y[1] + g[2] * y[2] + g[3] * y[3];
      store4(dr + 4 * c, f32x4{w * g[0], w * g[1], w * g[2], w * g[3]});
    }
    part = wave_sum(part);
    if (lane == 0) s_part[j][wave] = part;
  }
  __syncthreads();
  if (tid < k) {
    const int j = tid;
    d_weights[(int64_t)t * k + j] = s_idx[j] < 0 ? 0.f : ((s_part[j][0] + s_part[j][1]) + s_part[j][2]) + s_part[j][3];
  }
}

}  // namespace
}  // namespace moe

namespace moe_launch {

hipError_t scatter_grad(int dt, const float* dy, const float* y_rows, const float* weights,
                        const int32_t* scatter_index, int T, int H, int top_k, int R, void* d_rows, float* d_weights,
                        hipStream_t s) {
  using namespace moe;
  if (dt == 1)
    hipLaunchKernelGGL(scatter_grad_k<bf16_t>, dim3(T), dim3(256), 0, s, (const f32x4*)dy, (const f32x4*)y_rows,
                       weights, scatter_index, H, top_k, R, (bf16_t*)d_rows, d_weights);
  else
    hipLaunchKernelGGL(scatter_grad_k<float>, dim3(T), dim3(256), 0, s, (const f32x4*)dy, (const f32x4*)y_rows,
                       weights, scatter_index, H, top_k, R, (float*)d_rows, d_weights);
  return hipGetLastError();
}

}  // namespace moe_launch
