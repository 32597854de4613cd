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
//   router_pad_bf16        odd E only: W_r [H,E] -> [H,E+1] with a zero column in the
//                          caller's workspace (the ring kernel loads W_r 4 bytes a lane).
//   router_logits_ring     x[T,H] @ W_r on MFMA (16x16x32 bf16, fp32 accumulate) from
//                          W_r's own [H,E] layout: 64 tokens x 64 experts per
//                          workgroup (128 x 256 for many tokens and experts), both
//                          operands streamed through an LDS ring by direct loads,
//                          H split across workgroups; partial sums land in the
//                          workspace.
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

constexpr int kRtBK = 64;     // k per ring step

int padded_experts(int E) { return (E + 15) / 16 * 16; }
// The ring kernel reads W_r with 4-byte loads, so an odd E first gets a zero column.
int ring_experts(int E) { return (E + 1) & ~1; }

// W_r [H, E] -> [H, E + 1] with a zero last column (odd E only).
__global__ __launch_bounds__(256) void router_pad_bf16(const bf16_t* __restrict__ w, int H, int E,
                                                       bf16_t* __restrict__ wp) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int Ep = E + 1;
  if (i >= (int64_t)H * Ep) return;
  const int64_t h = i / Ep;
  const int e = (int)(i - h * Ep);
  wp[i] = e < E ? w[h * E + e] : (bf16_t)0;
}

// Swizzle of a W_r row of BN experts in LDS: the 32-byte slot (16 experts) s of
// row r sits at slot s ^ rt_wslot<BN>(r).  A transposing B-fragment read covers
// 4 rows x 16 experts per 16 lanes, and a half-wave the rows {0-3, 8-11} (+4,
// +16, +32) of one slot; the swizzle sends those 8 rows to 8 different 32-byte
// windows of the 256-byte bank space.  128-byte rows (BN = 64) alternate
// between two halves of it, so bits 1 and 3 of the row pick the slot; 512-byte
// rows (BN = 256) all start at offset 0, so bits 0, 1 and 3 do.
template <int BN>
__device__ __forceinline__ int rt_wslot(int r) {
  static_assert(BN == 64 || BN == 256, "W_r tile widths of 64 or 256 experts");
  if constexpr (BN == 64) return ((r >> 1) & 1) | ((r >> 2) & 2);
  else return (r & 3) | ((r >> 1) & 4);
}

// Partial router logits over one slice of H for a tile of BM tokens x BN
// experts, from x [T, H] and W_r in its own [H, E] layout (E even).
//
// The slice streams through an LDS ring of S steps of 64 k, filled with direct
// loads (HBM -> LDS, no register round trip), so S - 1 steps' loads are in
// flight while one step is multiplied:
//  * x rows as 128-byte LDS rows, the 16-byte chunk c of row m at chunk
//    c ^ ((m >> 1) & 7): an A-fragment read (one chunk of 16 consecutive rows)
//    is then conflict-free;
//  * W_r rows (E-contiguous) as LDS rows of BN experts, swizzled by rt_wslot,
//    loaded 4 bytes a lane (E need only be even).  A B fragment (8 consecutive
//    k of one expert) is assembled from two ds_read_b64_tr_b16 reads: within
//    each 16-lane group, lane c receives element c % 4 of the 8-byte rows read
//    by lanes c/4, c/4 + 4, c/4 + 8 and c/4 + 12, so lanes that read a 4 (k) x
//    16 (expert) block get 4 consecutive k of their own expert.
// WM x WN waves each own (BM/WM) x (BN/WN) outputs as 16x16 blocks
// (v_mfma_f32_16x16x32_bf16, fp32 accumulate in k order).  Rows past T and
// experts past E are fetched from clamped addresses and feed only outputs
// that are never stored or read; k past H (the last slice of an H that is not
// a multiple of 64) is zeroed in LDS.  partial[z][t][e] is summed over z in a
// fixed order by topk_softmax, so the logits do not depend on scheduling.
//
// The grid is 1-D.  Workgroups are dealt to the 8 XCDs in turn, so the id is
// remapped: the expert tiles of one (token tile, slice) pair are consecutive
// workgroups of one XCD and share the x tile through its L2.  Ids past the last
// pair (the grid is padded to a multiple of 8 pairs) exit at once.
template <int BM, int BN, int WM, int WN, int S>
__global__ __launch_bounds__(WM * WN * 64) void router_logits_ring(const bf16_t* __restrict__ x,
                                                                   const bf16_t* __restrict__ w, int T, int H, int E,
                                                                   int E_pad, int kslice, int n_t, int n_e, int nz,
                                                                   float* __restrict__ partial) {
  constexpr int BK = kRtBK, NW = WM * WN, NT = NW * 64;
  constexpr int kWRow = BN * 2;                // bytes of one W_r row in LDS
  constexpr int kXStage = BM * BK * 2, kWStage = BK * kWRow, kStage = kXStage + kWStage;
  constexpr int kXLoads = kXStage / 1024 / NW;  // 16-byte loads (1 KiB per wave) per wave and step
  constexpr int kWLoads = kWStage / 256 / NW;   // 4-byte loads (256 B per wave) per wave and step
  constexpr int kLoads = kXLoads + kWLoads;
  constexpr int MB = BM / WM / 16, NB = BN / WN / 16;  // 16x16 blocks per wave
  static_assert(kXLoads >= 1 && kXStage % (1024 * NW) == 0 && kWStage % (256 * NW) == 0, "loads per wave");
  static_assert(S >= 2 && (S - 2) * kLoads < 64 && S * kStage <= 160 * 1024, "ring shape");
  __shared__ __attribute__((aligned(1024))) unsigned char ring[S * kStage];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = (int)(blockIdx.x >> 3);
  const int pair = (slot / n_e) * 8 + (int)(blockIdx.x & 7);
  if (pair >= n_t * nz) return;  // whole workgroup, before any barrier
  const int zb = pair / n_t;
  const int t0 = (pair - zb * n_t) * BM, e0 = (slot % n_e) * BN;
  const int kbeg = zb * kslice, kend = min(H, kbeg + kslice);
  const int nsteps = (kend - kbeg + BK - 1) / BK;

  // Per-lane sources of the direct loads (fixed over the slice but for k).
  int64_t xsrc[kXLoads];
  int xk[kXLoads];
#pragma unroll
  for (int j = 0; j < kXLoads; ++j) {
    const int m = (wave * kXLoads + j) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((m >> 1) & 7);
    xsrc[j] = (int64_t)min(t0 + m, T - 1) * H;
    xk[j] = 8 * c;
  }
  int wrow[kWLoads];
  int wcol[kWLoads];
#pragma unroll
  for (int j = 0; j < kWLoads; ++j) {
    const int b = (wave * kWLoads + j) * 256 + 4 * lane;  // byte inside the stage's W_r tile
    const int r = b / kWRow, d = (b % kWRow) / 4;        // row, 4-byte word in the row
    wrow[j] = r;
    wcol[j] = min(e0 + 16 * ((d >> 3) ^ rt_wslot<BN>(r)) + 2 * (d & 7), E - 2);
  }
  auto issue = [&](int step) {
    unsigned char* st = ring + (step % S) * kStage;
    const int k0 = kbeg + step * BK;
#pragma unroll
    for (int j = 0; j < kXLoads; ++j)
      __builtin_amdgcn_global_load_lds(MOE_GLOBAL(void, x + xsrc[j] + min(k0 + xk[j], H - 8)),
                                       MOE_LDS(void, st + (wave * kXLoads + j) * 1024), 16, 0, 0);
#pragma unroll
    for (int j = 0; j < kWLoads; ++j)
      __builtin_amdgcn_global_load_lds(MOE_GLOBAL(void, w + (int64_t)min(k0 + wrow[j], H - 1) * E + wcol[j]),
                                       MOE_LDS(void, st + kXStage + (wave * kWLoads + j) * 256), 4, 0, 0);
  };

  const int wm = wave / WN, wn = wave % WN;
  const int g = lane >> 4, s16 = lane & 15;
  f32x4 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int s = 0; s < S - 1 && s < nsteps; ++s) issue(s);
  for (int kt = 0; kt < nsteps; ++kt) {
    if (nsteps - 1 - kt >= S - 2) wait_vmcnt<(S - 2) * kLoads>(); else wait_vmcnt<0>();
    lds_barrier();
    unsigned char* st = ring + (kt % S) * kStage;
    const int kvalid = kend - (kbeg + kt * BK);
    if (kvalid < BK) {  // the last step of a ragged H: zero k >= H in both operands
      for (int i = tid; i < BM * 8; i += NT) {
        const int m = i >> 3, c = i & 7;
        if (8 * c >= kvalid) *(u32x4*)(st + m * 128 + 16 * (c ^ ((m >> 1) & 7))) = u32x4{0u, 0u, 0u, 0u};
      }
      for (int i = tid; i < (BK - kvalid) * (kWRow / 16); i += NT)
        *(u32x4*)(st + kXStage + (kvalid + i / (kWRow / 16)) * kWRow + 16 * (i % (kWRow / 16))) =
            u32x4{0u, 0u, 0u, 0u};
      lds_barrier();
    }
    if (kt + S - 1 < nsteps) issue(kt + S - 1);  // refills the stage every wave finished with in step kt - 1
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      u32x4 a[MB], b[NB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int m = wm * (BM / WM) + 16 * mb + s16;
        const int c = 4 * u + g;
        a[mb] = *(const u32x4*)(st + m * 128 + 16 * (c ^ ((m >> 1) & 7)));
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int r = 32 * u + 8 * g + (s16 >> 2);
        const int sl = wn * NB + nb;
        const unsigned char* p_lo = st + kXStage + r * kWRow + 32 * (sl ^ rt_wslot<BN>(r)) + 8 * (s16 & 3);
        const unsigned char* p_hi =
            st + kXStage + (r + 4) * kWRow + 32 * (sl ^ rt_wslot<BN>(r + 4)) + 8 * (s16 & 3);
        b[nb] = pack_tr_pair(__builtin_amdgcn_ds_read_tr16_b64_v4i16(MOE_LDS(i16x4, p_lo)),
                             __builtin_amdgcn_ds_read_tr16_b64_v4i16(MOE_LDS(i16x4, p_hi)));
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[mb]),
                                                                __builtin_bit_cast(bf16x8, b[nb]), acc[mb][nb], 0,
                                                                0, 0);
    }
  }
  // 16x16 accumulator layout: row = 4*(lane/16) + r, column = lane%16.
  float* out = partial + (int64_t)zb * T * E_pad;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int e = e0 + wn * (BN / WN) + 16 * nb + s16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + wm * (BM / WM) + 16 * mb + 4 * g + r;
        if (t < T && e < E_pad) out[(int64_t)t * E_pad + e] = acc[mb][nb][r];
      }
    }
}

// The two ring configurations: 64 tokens x 64 experts, 4 waves, 4 stages (two
// workgroups per CU), and for many tokens and more than 64 experts 128 tokens x
// 256 experts, 8 waves, 3 stages (one workgroup per CU): every expert of a
// token tile in one workgroup, so each x tile is staged once rather than once
// per 64 experts, which keeps more of x's HBM reads in flight.
struct RingSmall { static constexpr int BM = 64, BN = 64, WM = 2, WN = 2, S = 4, kWgsPerCu = 2; };
struct RingWide { static constexpr int BM = 128, BN = 256, WM = 2, WN = 4, S = 3, kWgsPerCu = 1; };

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

// Ring configuration for (T, E): the wide tile once there are more than 64 experts and at least 1024
// tokens, so that eight 128-token tiles or more keep the chip busy; f receives the configuration.
template <class F>
auto with_ring(int T, int E, F&& f) {
  if (moe::ring_experts(E) > 64 && T >= 1024) return f(moe::RingWide{});
  return f(moe::RingSmall{});
}

// Ring router: slices of H (multiples of 64, at least two steps each) so that the grid covers about one
// round of the workgroups the ring's LDS lets each CU hold, with at most 32 slices.
Split router_ring_split(int T, int H, int E) {
  using namespace moe;
  return with_ring(T, E, [&](auto cfg) {
    using C = decltype(cfg);
    const int tiles = ((T + C::BM - 1) / C::BM) * ((ring_experts(E) + C::BN - 1) / C::BN);
    const int target = 256 * C::kWgsPerCu;
    int nz = (target + tiles - 1) / tiles;
    int max_nz = H / (2 * kRtBK);
    if (max_nz > 32) max_nz = 32;
    if (nz > max_nz) nz = max_nz;
    if (nz < 1) nz = 1;
    const int kslice = ((H + nz - 1) / nz + kRtBK - 1) / kRtBK * kRtBK;
    return Split{(H + kslice - 1) / kslice, kslice};
  });
}

// Bytes of the zero-padded router copy an odd E needs (none for an even E).
size_t pad_bytes(int H, int E) {
  if (moe::ring_experts(E) == E) return 0;
  return ((size_t)H * moe::ring_experts(E) * sizeof(moe::bf16_t) + 255) & ~(size_t)255;
}

size_t route_workspace_bytes(int dt, int T, int H, int E) {
  if (dt != 1) return 0;
  if (router_small(dt, T, E)) return (size_t)router_valu_split(T, H).nz * T * E * sizeof(float);
  return pad_bytes(H, E) + (size_t)router_ring_split(T, H, E).nz * T * moe::padded_experts(E) * sizeof(float);
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
    const int E_pad = padded_experts(E), Er = ring_experts(E);
    const bf16_t* wr = (const bf16_t*)w_router;
    if (Er != E) {
      hipLaunchKernelGGL(router_pad_bf16, dim3((unsigned)(((int64_t)H * Er + 255) / 256)), dim3(256), 0, s,
                         (const bf16_t*)w_router, H, E, (bf16_t*)workspace);
      if ((err = hipGetLastError()) != hipSuccess) return err;
      wr = (const bf16_t*)workspace;
    }
    float* partial = (float*)((char*)workspace + pad_bytes(H, E));
    const Split sp = router_ring_split(T, H, E);
    with_ring(T, E, [&](auto cfg) {
      using C = decltype(cfg);
      const int n_t = (T + C::BM - 1) / C::BM, n_e = (Er + C::BN - 1) / C::BN;
      const dim3 grid((unsigned)((n_t * sp.nz + 7) / 8 * 8 * n_e));
      hipLaunchKernelGGL((router_logits_ring<C::BM, C::BN, C::WM, C::WN, C::S>), grid, dim3(C::WM * C::WN * 64), 0,
                         s, (const bf16_t*)x, wr, T, H, Er, E_pad, sp.kslice, n_t, n_e, sp.nz, partial);
      return 0;
    });
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
