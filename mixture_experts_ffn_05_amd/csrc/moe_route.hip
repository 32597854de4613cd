// Router GEMM and top-k softmax.
//
// PLENA_Compiler PR #69, section "Group E": the router GEMM (x @ W_r) is a
// stage of its own.  PLENA_Simulator PR #97, section "C_SET_TOPK_REG":
// topk_softmax is generic in the expert count and in k.
//
// Kernels:
//   router_logits_valu     up to 16 tokens (bf16, E a multiple of 8): x @ W_r on the
//                          vector ALUs straight from W_r's [H,E] layout, H split
//                          across workgroups; partial sums land in the workspace.
//   router_transpose_bf16  W_r [H,E] -> [E_pad,H] in the caller's workspace, so that
//                          both operands of the router product are K-contiguous.
//   router_logits_mfma     x[T,H] @ W_r on MFMA (16x16x32 bf16, fp32 accumulate),
//                          16 (or 64 for T >= 256) tokens x 64 experts per workgroup, H split across
//                          workgroups (grid.z) and across each workgroup's 4 waves;
//                          partial sums land in the workspace.
//   route_logits_f32       the same product for float32 inputs, one thread per logit.
//   topk_softmax           one wave64 per token: adds the partial sums in a fixed
//                          order (+ bias) into the logits, then topk_wave: k rounds
//                          of a wave arg-max under the key (logit descending, index
//                          ascending, NaN lowest) and a softmax over the k selected
//                          logits.
#include "moe_common.h"
#include "moe_topk.h"

#include <math.h>

#include <type_traits>

namespace moe {
namespace {

constexpr int kRtTok = 16;   // tokens per MFMA row block
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

// Partial logits over one slice of H for 16*MB tokens x 64 experts per
// workgroup.  Both MFMA operands are K-contiguous (x rows and the transposed
// router rows), so each lane loads its 16x16x32 fragments straight from global
// memory, four k-substeps (128 k) at a time so that many loads are in flight;
// each router fragment feeds the MB 16-token row blocks (MB = 4 for many tokens
// cuts the router-row traffic per MFMA by 2.5x; the product is bound by those
// loads).  The 4 waves split the workgroup's slice; their sums are added in a
// fixed order through LDS.  grid.z splits H into `ksplit` slices;
// partial[z][t][e] is summed over z in a fixed order by topk_softmax, so the
// result does not depend on scheduling.
template <int MB>
__global__ __launch_bounds__(256) void router_logits_mfma(const bf16_t* __restrict__ x,
                                                          const bf16_t* __restrict__ wt, int T, int H, int E_pad,
                                                          int kslice, float* __restrict__ partial) {
  constexpr int kTok = 16 * MB;
  __shared__ float red[4][kTok][kRtExp + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * kTok, e0 = blockIdx.y * kRtExp;
  const int nblk = min(4, (E_pad - e0) / 16);
  const int zbeg = blockIdx.z * kslice, zend = min(H, zbeg + kslice);
  const int kq = ((kslice + 127) / 128) * 32;   // per-wave share of the slice, a multiple of 32
  const int kbeg = zbeg + wave * kq, kend = min(zend, kbeg + kq);
  const int koff = (lane >> 4) * 8;
  const bf16_t* xr[MB];
  bool row_ok[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int row = t0 + 16 * mb + (lane & 15);
    row_ok[mb] = row < T;
    xr[mb] = x + (int64_t)(row_ok[mb] ? row : 0) * H;
  }
  f32x4 acc[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Steps of 64 k.  Full steps load unconditionally (a row past T reads row 0
  // and a column block past E_pad reads the last router row; neither result
  // is stored), so the only wait before a step's MFMAs is for that step's own
  // loads; the last, partial step masks k past the slice end with zeros.  The
  // MFMAs run in k order in every form below.
  struct Step {
    u32x4 a[MB][2], b[2][4];
  };
  auto load = [&](Step& st, int k, auto masked) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kk = k + 32 * u + koff;
      const bool k_ok = kk < kend;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        if constexpr (decltype(masked)::value)
          st.a[mb][u] = (row_ok[mb] && k_ok) ? *(const u32x4*)(xr[mb] + kk) : u32x4{0u, 0u, 0u, 0u};
        else
          st.a[mb][u] = *(const u32x4*)(xr[mb] + kk);
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int e = e0 + nb * 16 + (lane & 15);
        if constexpr (decltype(masked)::value)
          st.b[u][nb] = (k_ok && nb < nblk) ? *(const u32x4*)(wt + (int64_t)e * H + kk) : u32x4{0u, 0u, 0u, 0u};
        else
          st.b[u][nb] = *(const u32x4*)(wt + (int64_t)min(e, E_pad - 1) * H + kk);
      }
    }
  };
  auto mfmas = [&](const Step& st) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, st.a[mb][u]),
                                                                __builtin_bit_cast(bf16x8, st.b[u][nb]), acc[mb][nb],
                                                                0, 0, 0);
  };
  const int nfull = kend > kbeg ? (kend - kbeg) / 64 : 0;
  Step s0;
  if constexpr (MB == 1) {
    // One row block: two register sets in turn, so one step's loads are in flight while the
    // other set's MFMAs run.  The loop's loads are unconditional (the last one or two steps
    // are peeled off), so the waits before each MFMA group cover only the older set; the
    // scheduling barriers keep each phase where it is written.  With four row blocks a second
    // set would halve the waves each SIMD holds, and those waves hide the load latency better.
    Step s1;
    if (nfull > 0) {
      load(s0, kbeg, std::false_type{});
      int i = 0;
      for (; i + 3 <= nfull; i += 2) {
        load(s1, kbeg + 64 * (i + 1), std::false_type{});
        __builtin_amdgcn_sched_barrier(0);
        mfmas(s0);
        __builtin_amdgcn_sched_barrier(0);
        load(s0, kbeg + 64 * (i + 2), std::false_type{});
        __builtin_amdgcn_sched_barrier(0);
        mfmas(s1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (i + 2 == nfull) {
        load(s1, kbeg + 64 * (i + 1), std::false_type{});
        __builtin_amdgcn_sched_barrier(0);
        mfmas(s0);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(s1);
      } else {
        mfmas(s0);
      }
    }
  } else {
    for (int i = 0; i < nfull; ++i) {
      load(s0, kbeg + 64 * i, std::false_type{});
      __builtin_amdgcn_sched_barrier(0);   // all of the step's loads in flight before the first wait
      mfmas(s0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const int ktail = kbeg + 64 * nfull;
  if (ktail < kend) {
    load(s0, ktail, std::true_type{});
    mfmas(s0);
  }
  // 16x16 accumulator layout: row = 4*(lane/16) + r, column = lane%16.
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][16 * mb + 4 * (lane >> 4) + r][nb * 16 + (lane & 15)] = acc[mb][nb][r];
  __syncthreads();
  float* out = partial + (int64_t)blockIdx.z * T * E_pad;
  for (int i = tid; i < kTok * kRtExp; i += 256) {
    const int tt = i / kRtExp, ee = i % kRtExp;
    const int t = t0 + tt, e = e0 + ee;
    if (t < T && e < E_pad)
      out[(int64_t)t * E_pad + e] = ((red[0][tt][ee] + red[1][tt][ee]) + red[2][tt][ee]) + red[3][tt][ee];
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
// Small token counts: partial logits over one slice of H for up to kVTok
// tokens and every expert, reading W_r in its [H, E] layout (E a multiple of
// 8), so no transposed copy is made.  Thread (hl, o) owns experts [8o, 8o+8)
// (one 16-byte load per row) and rows hl, hl + nh, ... of the slice; the
// tokens' x values of the slice are staged in LDS as [row][token] floats.  The
// nh row lanes' sums are added in a fixed order through LDS.
constexpr int kVTok = 4;
constexpr int kVMaxSlice = 1024;

__global__ __launch_bounds__(256) void router_logits_valu(const bf16_t* __restrict__ x, const bf16_t* __restrict__ w,
                                                          int T, int H, int E, int kslice,
                                                          float* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) float xs[kVMaxSlice * kVTok];
  extern __shared__ float red[];  // [nh][kVTok][E]
  const int tid = threadIdx.x;
  const int O = E / 8, nh = 256 / O;
  const int t0 = blockIdx.x * kVTok, nt = min(kVTok, T - t0);
  const int h0 = blockIdx.y * kslice, hn = min(kslice, H - h0);
  for (int i = tid; i < hn * kVTok; i += 256) {
    const int hh = i / kVTok, tt = i % kVTok;
    xs[i] = tt < nt ? bf16_to_f32(x[(int64_t)(t0 + tt) * H + h0 + hh]) : 0.f;
  }
  __syncthreads();
  const int o = tid % O, hl = tid / O;
  if (hl < nh) {
    float acc[kVTok][8];
#pragma unroll
    for (int t = 0; t < kVTok; ++t)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[t][j] = 0.f;
    const bf16_t* wp = w + (int64_t)h0 * E + 8 * o;
#pragma unroll 8
    for (int hh = hl; hh < hn; hh += nh) {
      const u32x4 wv = *(const u32x4*)(wp + (int64_t)hh * E);
      const f32x4 xv = *(const f32x4*)(xs + hh * kVTok);
      float wf[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wf[2 * j] = __uint_as_float(wv[j] << 16);
        wf[2 * j + 1] = __uint_as_float(wv[j] & 0xffff0000u);
      }
#pragma unroll
      for (int t = 0; t < kVTok; ++t)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[t][j] = fmaf(xv[t], wf[j], acc[t][j]);
    }
#pragma unroll
    for (int t = 0; t < kVTok; ++t)
#pragma unroll
      for (int j = 0; j < 8; ++j) red[(hl * kVTok + t) * E + 8 * o + j] = acc[t][j];
  }
  __syncthreads();
  float* out = partial + (int64_t)blockIdx.y * T * E;
  for (int i = tid; i < nt * E; i += 256) {
    const int tt = i / E, e = i % E;
    float v = 0.f;
    for (int q = 0; q < nh; ++q) v += red[(q * kVTok + tt) * E + e];
    out[(int64_t)(t0 + tt) * E + e] = v;
  }
}

// One wave64 per token.  With `partial` set, the logits are first assembled
// as the fixed-order sum of `nsplit` partial products (+ bias) and written to
// `logits`; otherwise `logits` already holds them.
// Q logits per lane (E <= 64 Q).  The partial sums of all Q logits of a lane
// are added together, a batch of slices at a time, so that the lane waits for
// about nsplit / B load latencies rather than Q times as many.
template <int Q>
__global__ __launch_bounds__(256) void topk_softmax(const float* __restrict__ partial, int nsplit, int stride_e,
                                                    const float* __restrict__ bias, float* __restrict__ logits,
                                                    int T, int E, int k, int32_t* __restrict__ ids,
                                                    float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float* row = logits + (int64_t)t * E;
  float raw[Q];
  bool ok[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) ok[q] = lane + kWave * q < E;
  if (partial) {
    const float* ptr[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) ptr[q] = partial + (int64_t)t * stride_e + lane + kWave * q;
    sum_slices_n<Q, (Q >= 8 ? 2 : 16 / Q)>(ptr, ok, (int64_t)T * stride_e, nsplit, raw);
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int e = lane + kWave * q;
      if (ok[q]) {
        if (bias) raw[q] += bias[e];
        row[e] = raw[q];
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < Q; ++q) raw[q] = ok[q] ? row[lane + kWave * q] : 0.f;
  }
#pragma unroll
  for (int q = 0; q < Q; ++q)
    if (!ok[q]) raw[q] = -INFINITY;
  int id;
  float wgt;
  topk_wave(raw, E, k, id, wgt);
  if (lane < k) {
    ids[(int64_t)t * k + lane] = id;
    weights[(int64_t)t * k + lane] = wgt;
  }
}

}  // namespace
}  // namespace moe

namespace moe_launch {

// Small-T router (bf16, E a multiple of 8, at most 16 tokens): at most 32
// slices of H per token group (more only when H exceeds 32768); 32 rather than
// 8 measured 10% faster routing at one token.
bool router_small(int dt, int T, int E) { return dt == 1 && E % 8 == 0 && T <= 16; }

struct Split {
  int nz, kslice;
};

Split router_valu_split(int T, int H) {
  using namespace moe;
  const int chunks = (T + kVTok - 1) / kVTok;
  int nz = (512 + chunks - 1) / chunks;
  if (nz > 32) nz = 32;  // short W_r streams per workgroup; the top-k pass adds the slices eight at a time
  const int min_nz = (H + kVMaxSlice - 1) / kVMaxSlice;
  if (nz < min_nz) nz = min_nz;
  int kslice = ((H + nz - 1) / nz + 7) / 8 * 8;
  if (kslice > kVMaxSlice) kslice = kVMaxSlice;
  return Split{(H + kslice - 1) / kslice, kslice};
}

// Tokens per workgroup of the MFMA router: 64 (four 16-token row blocks per
// router fragment) once there are enough tokens to fill the grid, else 16.
int router_mfma_tokens(int T) { return T >= 256 ? 4 * moe::kRtTok : moe::kRtTok; }

// MFMA router: slices of H (multiples of 128) so that the grid covers about
// 512 workgroups.
Split router_mfma_split(int T, int H, int E) {
  using namespace moe;
  const int tok = router_mfma_tokens(T);
  const int tiles = ((T + tok - 1) / tok) * ((padded_experts(E) + kRtExp - 1) / kRtExp);
  int ks = (512 + tiles - 1) / tiles;
  const int max_ks = (H + 127) / 128;
  if (ks > max_ks) ks = max_ks;
  if (ks < 1) ks = 1;
  const int kslice = ((H + ks - 1) / ks + 127) / 128 * 128;
  return Split{(H + kslice - 1) / kslice, kslice};
}

size_t wt_bytes(int H, int E) {
  return ((size_t)moe::padded_experts(E) * H * sizeof(moe::bf16_t) + 255) & ~(size_t)255;
}

size_t route_workspace_bytes(int dt, int T, int H, int E) {
  if (dt != 1) return 0;
  if (router_small(dt, T, E)) return (size_t)router_valu_split(T, H).nz * T * E * sizeof(float);
  return wt_bytes(H, E) + (size_t)router_mfma_split(T, H, E).nz * T * moe::padded_experts(E) * sizeof(float);
}

hipError_t route_partials_small(const void* x, const void* w_router, int T, int H, int E, void* workspace,
                                int* nsplit, hipStream_t s) {
  using namespace moe;
  const Split sp = router_valu_split(T, H);
  const size_t lds = (size_t)(256 / (E / 8)) * kVTok * E * sizeof(float);
  hipLaunchKernelGGL(router_logits_valu, dim3((T + kVTok - 1) / kVTok, sp.nz), dim3(256), lds, s,
                     (const bf16_t*)x, (const bf16_t*)w_router, T, H, E, sp.kslice, (float*)workspace);
  *nsplit = sp.nz;
  return hipGetLastError();
}

// topk_softmax with the logits-per-lane specialization for E.
hipError_t launch_topk(const float* partial, int nsplit, int stride_e, const float* bias, float* logits, int T, int E,
                       int k, int32_t* ids, float* weights, hipStream_t s) {
  using namespace moe;
  const dim3 grid((T + 3) / 4), block(256);
  switch (topk_per_lane(E)) {
    case 1: hipLaunchKernelGGL(topk_softmax<1>, grid, block, 0, s, partial, nsplit, stride_e, bias, logits, T, E, k, ids, weights); break;
    case 2: hipLaunchKernelGGL(topk_softmax<2>, grid, block, 0, s, partial, nsplit, stride_e, bias, logits, T, E, k, ids, weights); break;
    case 4: hipLaunchKernelGGL(topk_softmax<4>, grid, block, 0, s, partial, nsplit, stride_e, bias, logits, T, E, k, ids, weights); break;
    case 8: hipLaunchKernelGGL(topk_softmax<8>, grid, block, 0, s, partial, nsplit, stride_e, bias, logits, T, E, k, ids, weights); break;
    default: hipLaunchKernelGGL(topk_softmax<kTopkPer>, grid, block, 0, s, partial, nsplit, stride_e, bias, logits, T, E, k, ids, weights); break;
  }
  return hipGetLastError();
}

hipError_t route(int dt, const void* x, const void* w_router, const float* bias, int T, int H, int E,
                 int top_k, int32_t* ids, float* weights, float* logits, void* workspace, hipStream_t s) {
  using namespace moe;
  hipError_t err;
  if (router_small(dt, T, E)) {
    int nz = 0;
    if ((err = route_partials_small(x, w_router, T, H, E, workspace, &nz, s)) != hipSuccess) return err;
    return launch_topk((const float*)workspace, nz, E, bias, logits, T, E, top_k, ids, weights, s);
  }
  if (dt == 1) {
    const int E_pad = padded_experts(E);
    const Split sp = router_mfma_split(T, H, E);
    bf16_t* wt = (bf16_t*)workspace;
    float* partial = (float*)((char*)workspace + wt_bytes(H, E));
    hipLaunchKernelGGL(router_transpose_bf16, dim3((H + 63) / 64, (E_pad + 63) / 64), dim3(256), 0, s,
                       (const bf16_t*)w_router, H, E, E_pad, wt);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const int tok = router_mfma_tokens(T);
    dim3 grid((T + tok - 1) / tok, (E_pad + kRtExp - 1) / kRtExp, sp.nz);
    if (tok == 4 * kRtTok)
      hipLaunchKernelGGL(router_logits_mfma<4>, grid, dim3(256), 0, s, (const bf16_t*)x, (const bf16_t*)wt, T, H,
                         E_pad, sp.kslice, partial);
    else
      hipLaunchKernelGGL(router_logits_mfma<1>, grid, dim3(256), 0, s, (const bf16_t*)x, (const bf16_t*)wt, T, H,
                         E_pad, sp.kslice, partial);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    return launch_topk((const float*)partial, sp.nz, E_pad, bias, logits, T, E, top_k, ids, weights, s);
  }
  const int64_t n = (int64_t)T * E;
  hipLaunchKernelGGL(route_logits_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     (const float*)x, (const float*)w_router, bias, T, H, E, logits);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  return launch_topk(nullptr, 0, E, nullptr, logits, T, E, top_k, ids, weights, s);
}

}  // namespace moe_launch
