// Grouped GEMMs of the expert FFNs: fc1 (gate/up) with the SwiGLU epilogue,
// and fc2 (down) with an fp32 store or a scaled accumulate.
//
// VeOmni docs "Fused MoE Kernel Notes", section "Backward grouped-GEMM launch
// bound": a same-N/K grouped GEMM must cover the largest expert group, and the
// token count is not a safe bound (section "Duplicate top-k routes").  Here the
// tile walk is built on the device from the realized expert_offsets: group g
// contributes ceil(c_g / 128) row tiles, so a group of any size up to R rows is
// covered and an empty group reads no weights.  The host only sizes a
// persistent grid from the worst case floor(R/128) + min(E, R) row tiles.
//
// bf16 path (gfx950 MFMA v_mfma_f32_32x32x16_bf16, fp32 accumulate):
//   * workgroup tile 128 rows x 128 staged weight columns, reduction slice 64;
//     4 waves in a 2x2 arrangement, each owning 64 rows x 64 columns
//     (2x2 blocks of 32x32).  fc1 stages the gate columns [n0, n0+64) and the
//     matching up columns [I+n0, I+n0+64) side by side, so each lane holds the
//     gate and up accumulators of the same output element and applies
//     silu(g)*u before rounding to bf16.
//   * activations are K-contiguous and are copied to LDS as 16-byte rows;
//     weights are N-contiguous ([K, N] per expert), so each thread loads a
//     4 (k) x 8 (n) block, transposes it in registers and writes column-major
//     k-quads to LDS with an XOR swizzle on the quad index, which keeps the
//     16-byte MFMA operand reads conflict-free.
//   * persistent grid: each workgroup walks tile ids slot, slot+grid, ...;
//     ids are ordered expert-major, then column tile, then row tile, so
//     consecutive ids share one weight slab; the slot is remapped so that
//     consecutive ids land on the same XCD (workgroups are dealt to the 8
//     XCDs round-robin) and share its L2.
// f32 path: one thread per output element (used by the float32 workload).
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kBM = 128;
constexpr int kBNB = 128;  // staged weight columns per tile
constexpr int kBK = 64;
constexpr int kLds = 72;   // padded LDS row in bf16 elements (144 bytes)
constexpr int kThreads = 256;
constexpr int kXcds = 8;

enum Epilogue { kSwiGLU = 0, kStoreF32 = 1, kScaleAdd = 2 };

template <typename T>
struct GemmParams {
  const T* a;               // [rows, K]
  const int32_t* offsets;   // [groups+1], or null for one group of `rows` rows
  int groups;
  int rows;
  int K;
  int N;                    // output columns
  const T* b;               // group g: b + g*b_stride, row-major [K, ldb]
  int64_t b_stride;
  int ldb;
  int up_off;               // SwiGLU: column offset of the up half inside b
  void* out;                // SwiGLU: T [rows, N]; otherwise float [rows, N]
  const float* row_scale;   // kScaleAdd: per-row factor, or null for 1
  int accumulate;           // kScaleAdd: add into out instead of overwriting
  int n_tiles;              // output column tiles per group
};

__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                  0, 0, 0);
}

template <int EPI>
__device__ __forceinline__ int wave_col_base(int nb, int wn) {
  return EPI == kSwiGLU ? (64 * nb + 32 * wn) : (64 * wn + 32 * nb);
}

template <int EPI>
__device__ __forceinline__ void run_tile_bf16(const GemmParams<bf16_t>& p, int g, int row0, int row_end, int n0,
                                              bf16_t* __restrict__ sA, bf16_t* __restrict__ sB) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const bf16_t* __restrict__ bg = p.b + (int64_t)g * p.b_stride;

  // This thread's weight octet: columns [c, c+8) of the staged tile.
  const int co = tid & 15, kq = tid >> 4;
  int bcol;
  bool bcol_ok;
  if (EPI == kSwiGLU) {
    const int c = co * 8;
    const int nc = n0 + (c & 63);
    bcol = (c < 64 ? 0 : p.up_off) + nc;
    bcol_ok = nc < p.N;
  } else {
    bcol = n0 + co * 8;
    bcol_ok = bcol < p.N;
  }
  const int swz = 2 * (co & 7);

  f32x16 acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;

  u32x4 ra[4], rb[4];
  const int nk = (p.K + kBK - 1) / kBK;

  auto load = [&](int kt) {
    const int k0 = kt * kBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = tid + kThreads * i, r = v >> 3, ko = v & 7;
      const int row = row0 + r, k = k0 + ko * 8;
      ra[i] = (row < row_end && k < p.K) ? *(const u32x4*)(p.a + (int64_t)row * p.K + k) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = k0 + kq * 4 + i;
      rb[i] = (bcol_ok && k < p.K) ? *(const u32x4*)(bg + (int64_t)k * p.ldb + bcol) : u32x4{0u, 0u, 0u, 0u};
    }
  };

  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = tid + kThreads * i, r = v >> 3, ko = v & 7;
      *(u32x4*)(sA + r * kLds + ko * 8) = ra[i];
    }
#pragma unroll
    for (int cl = 0; cl < 8; ++cl) {
      const int d = cl >> 1, sh = (cl & 1) * 16;
      const uint32_t v0 = (rb[0][d] >> sh) & 0xffffu, v1 = (rb[1][d] >> sh) & 0xffffu;
      const uint32_t v2 = (rb[2][d] >> sh) & 0xffffu, v3 = (rb[3][d] >> sh) & 0xffffu;
      *(u32x2*)(sB + (co * 8 + cl) * kLds + 4 * (kq ^ swz)) = u32x2{v0 | (v1 << 16), v2 | (v3 << 16)};
    }
  };

  auto compute = [&]() {
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      u32x4 af[2], bf[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        af[mb] = *(const u32x4*)(sA + (wm * 64 + mb * 32 + (lane & 31)) * kLds + ks * 16 + (lane >> 5) * 8);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int col = wave_col_base<EPI>(nb, wn) + (lane & 31);
        const int oct = (ks * 2 + (lane >> 5)) ^ ((col >> 3) & 7);
        bf[nb] = *(const u32x4*)(sB + col * kLds + oct * 8);
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma32(af[mb], bf[nb], acc[mb][nb]);
    }
  };

  load(0);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
    store();
    __syncthreads();
    if (kt + 1 < nk) load(kt + 1);
    compute();
  }

  // 32x32 accumulator layout: column = lane%32, row = 8*(i/4) + 4*(lane/32) + i%4.
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = row0 + wm * 64 + mb * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      if (row >= row_end) continue;
      if (EPI == kSwiGLU) {
        const int col = n0 + 32 * wn + (lane & 31);
        if (col < p.N)
          ((bf16_t*)p.out)[(int64_t)row * p.N + col] = (bf16_t)f32_to_bf16_rne(swiglu(acc[mb][0][i], acc[mb][1][i]));
      } else {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int col = n0 + 64 * wn + 32 * nb + (lane & 31);
          if (col >= p.N) continue;
          float* o = (float*)p.out + (int64_t)row * p.N + col;
          const float v = acc[mb][nb][i];
          if (EPI == kStoreF32) {
            *o = v;
          } else {
            const float sc = p.row_scale ? p.row_scale[row] : 1.0f;
            *o = (p.accumulate ? *o : 0.0f) + sc * v;
          }
        }
      }
    }
  }
}

template <int EPI>
__global__ __launch_bounds__(kThreads, 2) void grouped_gemm_bf16(GemmParams<bf16_t> p) {
  __shared__ __attribute__((aligned(16))) bf16_t sA[kBM * kLds];
  __shared__ __attribute__((aligned(16))) bf16_t sB[kBNB * kLds];
  __shared__ int32_t sOff[kMaxExperts + 1];
  __shared__ int32_t sPre[kMaxExperts + 1];
  __shared__ int32_t sWave[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = p.groups;
  // Group bounds, clamped to [0, rows] so that no tile can leave the buffers.
  for (int i = tid; i <= G; i += kThreads) {
    int v = p.offsets ? p.offsets[i] : (i == 0 ? 0 : p.rows);
    sOff[i] = min(max(v, 0), p.rows);
  }
  __syncthreads();
  // Exclusive prefix of row tiles per group (4 consecutive groups per thread).
  int loc[4], s = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int g = tid * 4 + q;
    const int c = g < G ? max(sOff[g + 1] - sOff[g], 0) : 0;
    loc[q] = s;
    s += (c + kBM - 1) / kBM;
  }
  const int incl = wave_inclusive_scan(s);
  if (lane == 63) sWave[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < wave; ++i) base += sWave[i];
  const int excl = base + incl - s;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int g = tid * 4 + q;
    if (g < G) sPre[g] = excl + loc[q];
  }
  if (tid == 0) sPre[G] = sWave[0] + sWave[1] + sWave[2] + sWave[3];
  __syncthreads();

  const int64_t nt = p.n_tiles;
  const int64_t total = (int64_t)sPre[G] * nt;
  const int nslot = gridDim.x;
  const int slot = (blockIdx.x % kXcds) * (nslot / kXcds) + blockIdx.x / kXcds;
  for (int64_t id = slot; id < total; id += nslot) {
    int lo = 0, hi = G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int64_t)sPre[mid] * nt <= id) lo = mid; else hi = mid - 1;
    }
    const int g = lo;
    const int64_t local = id - (int64_t)sPre[g] * nt;
    const int mt = sPre[g + 1] - sPre[g];
    const int ntile = (int)(local / mt), mtile = (int)(local % mt);
    const int row0 = sOff[g] + mtile * kBM;
    const int n0 = ntile * (EPI == kSwiGLU ? 64 : 128);
    run_tile_bf16<EPI>(p, g, row0, sOff[g + 1], n0, sA, sB);
  }
}

// float32 path: one thread per output element.
template <int EPI>
__global__ __launch_bounds__(256) void grouped_gemm_f32(GemmParams<float> p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)p.rows * p.N) return;
  const int row = (int)(i / p.N), col = (int)(i % p.N);
  const int G = p.groups;
  int g = 0;
  if (p.offsets) {
    const int end_all = min(max(p.offsets[G], 0), p.rows);
    if (row >= end_all) return;
    int lo = 0, hi = G - 1;  // largest g with offsets[g] <= row
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.offsets[mid] <= row) lo = mid; else hi = mid - 1;
    }
    g = lo;
  }
  const float* bg = p.b + (int64_t)g * p.b_stride;
  const float* ar = p.a + (int64_t)row * p.K;
  if (EPI == kSwiGLU) {
    float gs = 0.f, us = 0.f;
    for (int k = 0; k < p.K; ++k) {
      const float av = ar[k];
      gs = fmaf(av, bg[(int64_t)k * p.ldb + col], gs);
      us = fmaf(av, bg[(int64_t)k * p.ldb + p.up_off + col], us);
    }
    ((float*)p.out)[(int64_t)row * p.N + col] = swiglu(gs, us);
  } else {
    float v = 0.f;
    for (int k = 0; k < p.K; ++k) v = fmaf(ar[k], bg[(int64_t)k * p.ldb + col], v);
    float* o = (float*)p.out + (int64_t)row * p.N + col;
    if (EPI == kStoreF32) {
      *o = v;
    } else {
      const float sc = p.row_scale ? p.row_scale[row] : 1.0f;
      *o = (p.accumulate ? *o : 0.0f) + sc * v;
    }
  }
}

int persistent_grid(int64_t upper_tiles, int cu_count) {
  int64_t g = upper_tiles < (int64_t)2 * cu_count ? upper_tiles : (int64_t)2 * cu_count;
  if (g < 1) g = 1;
  g = (g + kXcds - 1) / kXcds * kXcds;
  return (int)g;
}

int64_t upper_row_tiles(int rows, int groups) {
  return (int64_t)rows / kBM + (groups < rows ? groups : rows);
}

}  // namespace
}  // namespace moe

namespace moe_launch {

hipError_t grouped_swiglu_fc1(int dt, const void* a, const int32_t* offsets, int groups, int rows, const void* w1,
                              int64_t w1_group_stride, int K, int I, void* act, int cu_count, hipStream_t s) {
  using namespace moe;
  if (dt == 1) {
    GemmParams<bf16_t> p{(const bf16_t*)a, offsets, groups, rows, K, I, (const bf16_t*)w1, w1_group_stride,
                         2 * I, I, act, nullptr, 0, (I + 63) / 64};
    const int grid = persistent_grid(upper_row_tiles(rows, groups) * p.n_tiles, cu_count);
    hipLaunchKernelGGL(grouped_gemm_bf16<kSwiGLU>, dim3(grid), dim3(kThreads), 0, s, p);
  } else {
    GemmParams<float> p{(const float*)a, offsets, groups, rows, K, I, (const float*)w1, w1_group_stride,
                        2 * I, I, act, nullptr, 0, 0};
    const int64_t n = (int64_t)rows * I;
    hipLaunchKernelGGL(grouped_gemm_f32<kSwiGLU>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t grouped_fc2(int dt, const void* act, const int32_t* offsets, int groups, int rows, const void* w2,
                       int64_t w2_group_stride, int K, int N, float* out, const float* row_scale, int accumulate,
                       int plain_store, int cu_count, hipStream_t s) {
  using namespace moe;
  if (dt == 1) {
    GemmParams<bf16_t> p{(const bf16_t*)act, offsets, groups, rows, K, N, (const bf16_t*)w2, w2_group_stride,
                         N, 0, out, row_scale, accumulate, (N + 127) / 128};
    const int grid = persistent_grid(upper_row_tiles(rows, groups) * p.n_tiles, cu_count);
    if (plain_store)
      hipLaunchKernelGGL(grouped_gemm_bf16<kStoreF32>, dim3(grid), dim3(kThreads), 0, s, p);
    else
      hipLaunchKernelGGL(grouped_gemm_bf16<kScaleAdd>, dim3(grid), dim3(kThreads), 0, s, p);
  } else {
    GemmParams<float> p{(const float*)act, offsets, groups, rows, K, N, (const float*)w2, w2_group_stride,
                        N, 0, out, row_scale, accumulate, 0};
    const int64_t n = (int64_t)rows * N;
    const dim3 grid((unsigned)((n + 255) / 256));
    if (plain_store)
      hipLaunchKernelGGL(grouped_gemm_f32<kStoreF32>, grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL(grouped_gemm_f32<kScaleAdd>, grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace moe_launch
