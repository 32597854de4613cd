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
// bf16 pipelined path (reduction size a multiple of 64; every configuration):
//   * workgroup tile BM x BN staged weight columns, reduction slice BK, WM x WN
//     wave positions (times KW split-K waves), each owning (BM/WM) x (BN/WN)
//     as 32x32 MFMA blocks (v_mfma_f32_32x32x16_bf16, fp32 accumulate); the
//     shapes are listed with PipeCfg below (32 to 256 rows, 128 or 256
//     columns, 4 or 8 waves).
//   * operands travel HBM -> LDS with global_load_lds_dwordx4 (no register
//     round trip) through a STAGES-deep ring of LDS buffers, so several
//     reduction slices are in flight while the MFMAs consume an older one.
//     Each lane's 16 bytes land at LDS base + 16*lane, so the XOR swizzles
//     below are applied by choosing which 16-byte chunk each lane fetches.
//   * where a SIMD runs at most two waves, each wave alternates between two
//     fragment sets: the next substep's LDS reads are interleaved with the
//     current substep's MFMAs, across slice boundaries too (run_tile_pipe_v1).
//   * activations ([rows, K], K-contiguous) sit in LDS as 128-byte rows with
//     the 16-byte chunk index XORed by (row >> 1) & 7; an MFMA A fragment is
//     one conflict-free ds_read_b128.  With a_rows set (gather-on-load), row r
//     is fetched from row a_rows[r] of the layer input instead of from a
//     scattered copy; the offsets are fixed per tile, so this costs one index
//     load per lane and tile.
//   * weights ([K, N] per expert, N-contiguous) sit in LDS in that natural
//     layout (chunk index XORed by 4*(k & 3)); the B fragment (8 consecutive
//     k of one column) is assembled from two ds_read_b64_tr_b16 transpose
//     reads: within each 16-lane group, lane c receives element c%4 of the
//     8-byte rows read by lanes c/4, c/4+4, c/4+8 and c/4+12, so lanes that
//     read a 4 (k) x 16 (n) block get 4 consecutive k of their own column.
//   * rows past a group's end and columns past N are fetched from clamped
//     addresses; they only feed output rows/columns that are never stored.
//
// bf16 generic path (any multiple-of-8 sizes; register-staged):
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

#include <type_traits>

namespace moe {
namespace {

constexpr int kBM = 128;
constexpr int kBNB = 128;  // staged weight columns per tile
constexpr int kBK = 64;
constexpr int kLds = 72;   // padded LDS row in bf16 elements (144 bytes)
constexpr int kThreads = 256;
constexpr int kXcds = 8;

// kSwiGLUSave: the SwiGLU epilogue that also stores the fc1 pre-activation
// (training forward); kSwiGLUBwd: the gradient of SwiGLU applied to the
// accumulated gradient of its output (backward through fc2).
enum Epilogue { kSwiGLU = 0, kStoreF32 = 1, kScaleAdd = 2, kSwiGLUSave = 3, kSwiGLUBwd = 4 };

// Epilogues whose staged weight columns are gate/up pairs of the same outputs.
constexpr bool paired(int epi) { return epi == kSwiGLU || epi == kSwiGLUSave; }

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
  int bt;                   // 0: b rows are k ([K, ldb], N contiguous); 1: b rows are n ([N, ldb = K], K contiguous)
  const uint8_t* sc;        // MXFP8: e8m0 scales of group 0 (b then holds e4m3 codes, [N, K] bytes)
  int64_t sc_stride;        // MXFP8: bytes between the scales of consecutive groups
  const void* aux;          // kSwiGLUBwd: fc1 pre-activation T [rows, 2N] (gate columns, then up columns)
  void* out2;               // kSwiGLUSave: fc1 pre-activation out, T [rows, 2N]
  const int32_t* a_rows;    // optional: row r of A is row a_rows[r] of `a` ([a_src_rows, K]), else row r
  int a_src_rows;           // rows of `a` when a_rows is set (indices are clamped to [0, a_src_rows))
};

// Source row of A for row r (gather-on-load when a_rows is set).
template <typename T>
__device__ __forceinline__ int64_t a_src_row(const GemmParams<T>& p, int r) {
  return p.a_rows ? (int64_t)min(max(p.a_rows[r], 0), p.a_src_rows - 1) : (int64_t)r;
}

// SwiGLU output at (row, col) from the gate and up accumulators; with
// kSwiGLUSave the two pre-activations are stored as well.
template <int EPI, typename T>
__device__ __forceinline__ void epi_swiglu(const GemmParams<T>& p, int64_t row, int col, float g, float u) {
  store_from_f32((T*)p.out, row * p.N + col, swiglu(g, u));
  if (EPI == kSwiGLUSave) {
    T* h = (T*)p.out2 + row * 2 * p.N;
    store_from_f32(h, col, g);
    store_from_f32(h, p.N + col, u);
  }
}

// Backward through SwiGLU at (row, col): `da` is the gradient of silu(g) * u.
// dg = da * u * s * (1 + g * (1 - s)) with s = sigmoid(g), du = da * g * s;
// they land in columns col and N + col of the output row, like g and u.
template <typename T>
__device__ __forceinline__ void epi_swiglu_bwd(const GemmParams<T>& p, int64_t row, int col, float da) {
  const T* h = (const T*)p.aux + row * 2 * p.N;
  const float g = load_as_f32(h, col), u = load_as_f32(h, p.N + col);
  const float s = sigmoidf_(g);
  T* d = (T*)p.out + row * 2 * p.N;
  store_from_f32(d, col, da * u * s * (1.0f + g * (1.0f - s)));
  store_from_f32(d, p.N + col, da * g * s);
}

__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                  0, 0, 0);
}

template <int EPI>
__device__ __forceinline__ int wave_col_base(int nb, int wn) {
  return paired(EPI) ? (64 * nb + 32 * wn) : (64 * wn + 32 * nb);
}

template <int EPI>
__device__ __forceinline__ void run_tile_bf16(const GemmParams<bf16_t>& p, int g, int row0, int row_end, int n0,
                                              bf16_t* __restrict__ sA, bf16_t* __restrict__ sB) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const bf16_t* __restrict__ bg = p.b + (int64_t)g * p.b_stride;

  // [K, N] weights: this thread's weight octet is columns [c, c+8) of the staged tile.
  const int co = tid & 15, kq = tid >> 4;
  int bcol;
  bool bcol_ok;
  if (paired(EPI)) {
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
      ra[i] = (row < row_end && k < p.K) ? *(const u32x4*)(p.a + a_src_row(p, row) * p.K + k) : u32x4{0u, 0u, 0u, 0u};
    }
    if (p.bt) {  // [N, K] weights: 8 consecutive k of one staged column, like the activations
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int v = tid + kThreads * i, c = v >> 3, ko = v & 7;
        const int k = k0 + ko * 8;
        int nrow;
        bool ok;
        if (paired(EPI)) {
          const int nc = n0 + (c & 63);
          nrow = (c < 64 ? 0 : p.up_off) + nc;
          ok = nc < p.N;
        } else {
          nrow = n0 + c;
          ok = nrow < p.N;
        }
        rb[i] = (ok && k < p.K) ? *(const u32x4*)(bg + (int64_t)nrow * p.ldb + k) : u32x4{0u, 0u, 0u, 0u};
      }
      return;
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
    if (p.bt) {  // k-octet ko of column c lands at octet ko ^ ((c >> 3) & 7) of the column's LDS row
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int v = tid + kThreads * i, c = v >> 3, ko = v & 7;
        *(u32x4*)(sB + c * kLds + 8 * (ko ^ ((c >> 3) & 7))) = rb[i];
      }
      return;
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
      if (paired(EPI)) {
        const int col = n0 + 32 * wn + (lane & 31);
        if (col < p.N) epi_swiglu<EPI>(p, row, col, acc[mb][0][i], acc[mb][1][i]);
      } else {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int col = n0 + 64 * wn + 32 * nb + (lane & 31);
          if (col >= p.N) continue;
          if (EPI == kSwiGLUBwd) {
            epi_swiglu_bwd(p, row, col, acc[mb][nb][i]);
            continue;
          }
          float* o = (float*)p.out + (int64_t)row * p.N + col;
          const float v = acc[mb][nb][i];
          if (EPI == kStoreF32) {
            __builtin_nontemporal_store(v, o);  // read once, by the next call
          } else {
            const float sc = p.row_scale ? p.row_scale[row] : 1.0f;
            *o = (p.accumulate ? *o : 0.0f) + sc * v;
          }
        }
      }
    }
  }
}

// Group bounds (clamped to [0, rows], so that no tile can leave the buffers)
// and the exclusive prefix of row tiles per group, built in LDS by the whole
// workgroup of NT threads.  Returns the number of row tiles.  With sAct set,
// also the exclusive prefix of groups that fill exactly one row tile
// (sAct[G] = their number).
template <int BM, int NT, typename T>
__device__ __forceinline__ int build_tile_prefix(const GemmParams<T>& p, int32_t* sOff, int32_t* sPre,
                                                 int32_t* sWave, int32_t* sAct = nullptr) {
  constexpr int kPer = (kMaxExperts + NT - 1) / NT;  // consecutive groups per thread
  constexpr int kWaves = NT / kWave;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = p.groups;
  for (int i = tid; i <= G; i += NT) {
    const int v = p.offsets ? p.offsets[i] : (i == 0 ? 0 : p.rows);
    sOff[i] = min(max(v, 0), p.rows);
  }
  __syncthreads();
  int loc[kPer], s = 0;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int g = tid * kPer + q;
    const int c = g < G ? max(sOff[g + 1] - sOff[g], 0) : 0;
    loc[q] = s;
    s += (c + BM - 1) / BM;
  }
  const int incl = wave_inclusive_scan(s);
  if (lane == 63) sWave[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < wave; ++i) base += sWave[i];
  const int excl = base + incl - s;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int g = tid * kPer + q;
    if (g < G) sPre[g] = excl + loc[q];
  }
  if (tid == 0) {
    int total = 0;
    for (int i = 0; i < kWaves; ++i) total += sWave[i];
    sPre[G] = total;
  }
  __syncthreads();
  if (sAct) {  // the same scan over "group has exactly one row tile"
    int la[kPer], a = 0;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int g = tid * kPer + q;
      la[q] = a;
      a += (g < G && sPre[g + 1] - sPre[g] == 1) ? 1 : 0;
    }
    const int ia = wave_inclusive_scan(a);
    if (lane == 63) sWave[wave] = ia;
    __syncthreads();
    int ab = 0;
    for (int i = 0; i < wave; ++i) ab += sWave[i];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int g = tid * kPer + q;
      if (g < G) sAct[g] = ab + ia - a + la[q];
    }
    if (tid == 0) {
      int total = 0;
      for (int i = 0; i < kWaves; ++i) total += sWave[i];
      sAct[G] = total;
    }
    __syncthreads();
  }
  return sPre[G];
}

struct TileCoord {
  int g, row0, row_end, ntile;
  bool single;   // the group fits in one row tile (its weights are read once)
};

// Tile ids run expert-major, then column tile, then row tile.
template <int BM>
__device__ __forceinline__ TileCoord decode_tile(int64_t id, int G, int64_t nt, const int32_t* sOff,
                                                 const int32_t* sPre) {
  int lo = 0, hi = G - 1;  // largest g with sPre[g]*nt <= id: a non-empty group
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)sPre[mid] * nt <= id) lo = mid; else hi = mid - 1;
  }
  const int64_t local = id - (int64_t)sPre[lo] * nt;
  const int mt = sPre[lo + 1] - sPre[lo];
  TileCoord c;
  c.g = lo;
  c.ntile = (int)(local / mt);
  c.row0 = sOff[lo] + (int)(local % mt) * BM;
  c.row_end = sOff[lo + 1];
  c.single = sOff[lo + 1] - sOff[lo] <= BM;
  return c;
}

// The weight-streaming tile's order.  A group that fits in one row tile
// streams each weight slab from HBM once (HBM-bound); a group of m > 1 row
// tiles reads each slab once and re-reads it from L2 m - 1 times (MFMA-bound).
// In expert-major order a few large groups (skewed routing) would run all
// together, with HBM idle, and the single-tile groups after them with the
// MFMAs idle.  Here the tiles of single-tile groups (expert-major, then
// column) and those of multi-tile groups (expert, column, row) are cut into
// chunks of one XCD's share of the grid, and the two kinds of chunk are
// spread evenly: chunk j is a multi-tile chunk when
// floor((j+1)*CB/CC) > floor(j*CB/CC), for CB such chunks out of CC.  The row
// tiles of one slab stay adjacent inside a chunk, so they run at the same
// time on one XCD and share the slab in its L2.  The last chunk of each kind
// is padded; its padding ids decode to no tile.
struct SpreadWalk {
  int64_t nt;     // column tiles
  int64_t ns;     // tiles of single-tile groups
  int64_t nb;     // tiles of multi-tile groups
  int64_t chunk;  // ids per chunk
  int64_t cb;     // chunks of multi-tile groups
  int64_t cc;     // chunks in all
  __device__ int64_t ids() const { return cc * chunk; }
};

__device__ __forceinline__ SpreadWalk make_spread_walk(int G, int64_t nt, int64_t total, const int32_t* sAct) {
  SpreadWalk w;
  w.nt = nt;
  w.ns = (int64_t)sAct[G] * nt;
  w.nb = total - w.ns;
  w.chunk = max((int)gridDim.x / kXcds, 1);
  w.cb = (w.nb + w.chunk - 1) / w.chunk;
  w.cc = w.cb + (w.ns + w.chunk - 1) / w.chunk;
  return w;
}

// Tile of walk id `id` (0 <= id < w.ids()); false for a padding id.
template <int BM>
__device__ __forceinline__ bool decode_tile_spread(int64_t id, int G, const SpreadWalk& w, const int32_t* sOff,
                                                   const int32_t* sPre, const int32_t* sAct, TileCoord& c) {
  const int64_t j = id / w.chunk, r = id - j * w.chunk;
  const int64_t cb_before = j * w.cb / w.cc;  // multi-tile chunks before chunk j
  const int64_t nt = w.nt;
  int lo = 0, hi = G - 1;
  if ((j + 1) * w.cb / w.cc != cb_before) {
    const int64_t b = cb_before * w.chunk + r;
    if (b >= w.nb) return false;
    // largest g with (sPre[g] - sAct[g]) * nt <= b: a multi-tile group
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int64_t)(sPre[mid] - sAct[mid]) * nt <= b) lo = mid; else hi = mid - 1;
    }
    const int64_t local = b - (int64_t)(sPre[lo] - sAct[lo]) * nt;
    const int mt = sPre[lo + 1] - sPre[lo];
    c.ntile = (int)(local / mt);
    c.row0 = sOff[lo] + (int)(local % mt) * BM;
  } else {
    const int64_t a = (j - cb_before) * w.chunk + r;
    if (a >= w.ns) return false;
    // largest g with sAct[g] <= a / nt: the single-tile group of that rank
    const int rank = (int)(a / nt);
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sAct[mid] <= rank) lo = mid; else hi = mid - 1;
    }
    c.ntile = (int)(a % nt);
    c.row0 = sOff[lo];
  }
  c.g = lo;
  c.row_end = sOff[lo + 1];
  c.single = sOff[lo + 1] - sOff[lo] <= BM;
  return true;
}

// Consecutive slots run on one XCD (workgroups are dealt to the 8 XCDs round-robin).
__device__ __forceinline__ int xcd_slot() {
  const int nslot = gridDim.x;
  return (blockIdx.x % kXcds) * (nslot / kXcds) + blockIdx.x / kXcds;
}

template <int EPI, int ROLE>
__global__ __launch_bounds__(kThreads, 2) void grouped_gemm_bf16_generic(GemmParams<bf16_t> p) {
  __shared__ __attribute__((aligned(16))) bf16_t sA[kBM * kLds];
  __shared__ __attribute__((aligned(16))) bf16_t sB[kBNB * kLds];
  __shared__ int32_t sOff[kMaxExperts + 1];
  __shared__ int32_t sPre[kMaxExperts + 1];
  __shared__ int32_t sWave[4];
  const int mtiles = build_tile_prefix<kBM, kThreads>(p, sOff, sPre, sWave);
  const int64_t nt = p.n_tiles;
  const int64_t total = (int64_t)mtiles * nt;
  for (int64_t id = xcd_slot(); id < total; id += gridDim.x) {
    const TileCoord c = decode_tile<kBM>(id, p.groups, nt, sOff, sPre);
    run_tile_bf16<EPI>(p, c.g, c.row0, c.row_end, c.ntile * (paired(EPI) ? 64 : 128), sA, sB);
  }
}

// ------------------------------------------------------------------------------------------
// Pipelined bf16 path
// ------------------------------------------------------------------------------------------
// Cache policy of the direct loads of expert weights for a group that fits in
// one row tile: non-temporal (the nt bit of the instruction's cache-policy
// field).  Each of those weight bytes is read once per call, so keeping it out
// of the cache lines the activations and the other in-flight slices live in
// pays: measured on MI355X, the DeepSeek-V3-shaped routed fc1 (groups of ~100
// rows) went from 2.99 to 2.86 ms; the DeepSeek-V2-Lite-shaped decode (T = 64)
// fc1 from 0.182 to 0.127 ms and fc2 from 0.110 to 0.069 ms.  A group spanning
// several row tiles re-reads its weights once per row tile, and those re-reads
// hit in L2 only under the default policy (Qwen2-shaped fc1, ~273-row groups
// in 128-row tiles: 0.30 ms default, 0.40 ms non-temporal), so the policy is
// chosen per tile.  Activation loads keep the default policy (non-temporal
// activations measured 13% slower: every column tile re-reads them).
constexpr int kWeightLoadPolicy = 2;

// Shape of one pipelined configuration: workgroup tile BM x BN (staged weight
// columns), reduction slice BK, STAGES-deep LDS ring; WM x WN x KW waves.
// Each (WM, WN) position owns (BM/WM) x (BN/WN) as 32x32 MFMA blocks; with
// KW > 1, KW waves share one position and split every slice's 16-deep MFMA
// substeps between them, and their accumulators are added in a fixed order
// through LDS before the epilogue (more waves and more bytes in flight per
// tile when a tile holds few rows).
template <int BM_, int BN_, int BK_, int STAGES_, int WM_ = 2, int WN_ = 2, int KW_ = 1>
struct PipeCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_, WM = WM_, WN = WN_, KW = KW_;
  static constexpr int kPos = WM * WN;                  // wave positions in the tile
  static constexpr int kWaves = kPos * KW;
  static constexpr int NT = kWaves * kWave;
  static constexpr int kARow = BK * 2;                  // bytes of one activation row in LDS
  static constexpr int kAChunks = BK / 8;               // 16-byte chunks per activation row
  static constexpr int kAStage = BM * kARow;
  static constexpr int kBStage = BK * BN * 2;
  static constexpr int kStage = kAStage + kBStage;
  static constexpr int kALoads = kAStage / 1024 / kWaves;  // 1 KiB direct loads per wave per slice
  static constexpr int kBLoads = kBStage / 1024 / kWaves;
  static constexpr int kLoads = kALoads + kBLoads;
  static constexpr int kARowsPerLoad = 1024 / kARow;
  static constexpr int kBChunks = BN / 8;               // 16-byte chunks per weight row
  static constexpr int kBRowsPerLoad = 64 / kBChunks;
  static constexpr int kMB = BM / WM / 32;              // 32-row blocks per wave
  static constexpr int kNB = BN / WN / 32;              // 32-column blocks per wave
  static constexpr int kKS = BK / 16;                   // MFMA k-substeps per slice
  static constexpr int kKSW = kKS / KW;                 // substeps per wave
  static constexpr int kLds = STAGES * kStage;
  static constexpr int kRed = (KW - 1) * kPos * kMB * kNB * 16 * kWave * 4;  // split-K partials
  // Workgroups per CU that fit the 160 KiB of LDS (ring + ~9 KiB of tile tables).
  static constexpr int kFit = (160 * 1024) / (kLds + 9 * 1024);
  static constexpr int kWgsPerCu = kFit < 1 ? 1 : (kFit > 4 ? 4 : kFit);
  static_assert(kAStage % (1024 * kWaves) == 0 && kBStage % (1024 * kWaves) == 0,
                "slices must split into 1 KiB loads per wave");
  static_assert(kMB >= 1 && kNB >= 2 && kNB % 2 == 0, "wave tile must hold whole 32x32 blocks");
  static_assert(kBChunks == 8 || kBChunks >= 16, "the weight swizzle needs 8 or at least 16 chunks per row");
  static_assert(kKS % KW == 0, "substeps must split evenly between the split-K waves");
  static_assert(kRed <= kLds, "split-K partials must fit in the ring");
};

// LDS swizzles of the ring (gfx950 LDS: 64 banks of 4 bytes; a 16-byte read
// serves 16 lanes per cycle, an 8-byte read 32 lanes).
//  * an A fragment read touches one 16-byte chunk of 16 consecutive
//    activation rows per cycle.  A 256-byte bank window holds W = 256/rowbytes
//    rows; XORing the chunk index with (row / W) mod chunks puts the 16 rows
//    into 16 distinct bank groups.
//  * a transpose read of 32 lanes touches 4 consecutive k rows x 32 columns
//    (4 chunks per row).  With 256-byte rows (16+ chunks) all 4 rows sit on
//    one bank window and XORing the chunk index with 4 * (k & 3) sends them to
//    disjoint 64-byte quarters; with 128-byte rows (8 chunks) rows k and k+2
//    collide, and XORing with 4 * ((k >> 1) & 1) separates them.
template <class C>
__device__ __forceinline__ int a_swizzle(int row) { return (row / (256 / C::kARow)) % C::kAChunks; }
template <class C>
__device__ __forceinline__ int b_swizzle(int k) { return C::kBChunks >= 16 ? 4 * (k & 3) : 4 * ((k >> 1) & 1); }

template <int EPI, class C>
__device__ __forceinline__ int pipe_col_base(int nb, int wn) {
  // SwiGLU: blocks [0, kNB/2) are gate columns, [kNB/2, kNB) the matching up columns.
  return paired(EPI)
             ? ((nb < C::kNB / 2 ? 0 : C::BN / 2) + wn * (C::BN / 2 / C::WN) + 32 * (nb % (C::kNB / 2)))
             : (wn * (C::BN / C::WN) + 32 * nb);
}

// threadIdx.x passed through an empty asm statement.  A persistent kernel
// runs many tiles; values derived from the thread index (load and LDS
// offsets) are then recomputed at the start of each tile instead of being
// hoisted out of the tile loop, where they would stay live, and spill, across
// the code of the other tile configuration in a fused launch.
__device__ __forceinline__ int tile_thread() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// First tile row of 32-row block mb of the waves in wave row wm.  With
// several wave rows the blocks are dealt out alternately (block b belongs to
// wave row b mod WM), so that in a partial row tile every wave row holds about
// the same number of live blocks.
template <class C>
__device__ __forceinline__ int block_row(int wm, int mb) {
  return (mb * C::WM + wm) * 32;
}

// Direct loads of one reduction slice (activations, then weights) into a ring
// stage; wnt: the weights are read once (non-temporal policy).
template <class C>
__device__ __forceinline__ void pipe_issue(unsigned char* __restrict__ st, const bf16_t* a_k, const bf16_t* b_k,
                                           const int64_t* a_off, const int* b_off, bool wnt, int tid) {
  const int wave = tid >> 6;
#pragma unroll
  for (int i = 0; i < C::kALoads; ++i)
    if (C::STAGES != 2 || a_off[i] >= 0)
      __builtin_amdgcn_global_load_lds(MOE_GLOBAL(void, a_k + a_off[i]),
                                       MOE_LDS(void, st + (wave * C::kALoads + i) * 1024), 16, 0, 0);
  if (wnt) {
#pragma unroll
    for (int i = 0; i < C::kBLoads; ++i)
      __builtin_amdgcn_global_load_lds(MOE_GLOBAL(void, b_k + b_off[i]),
                                       MOE_LDS(void, st + C::kAStage + (wave * C::kBLoads + i) * 1024), 16, 0,
                                       kWeightLoadPolicy);
  } else {
#pragma unroll
    for (int i = 0; i < C::kBLoads; ++i)
      __builtin_amdgcn_global_load_lds(MOE_GLOBAL(void, b_k + b_off[i]),
                                       MOE_LDS(void, st + C::kAStage + (wave * C::kBLoads + i) * 1024), 16, 0, 0);
  }
}

// One pipeline step: start the loads of a future slice into `wst`, then run
// the MFMAs of the slice held in `rst`.  The two stages never coincide; the
// __restrict__ qualifiers tell the compiler so, which lets it skip waiting
// for the in-flight direct loads before the LDS reads below.
template <int EPI, class C, bool BT>
__device__ __forceinline__ void pipe_step(unsigned char* __restrict__ wst, const unsigned char* __restrict__ rst,
                                          bool issue, const bf16_t* a_k, const bf16_t* b_k, const int64_t* a_off,
                                          const int* b_off, f32x16 (&acc)[C::kMB][C::kNB], int wn, int wm, int kw,
                                          bool wnt, int tid) {
  const int lane = tid & 63;
  if (issue) pipe_issue<C>(wst, a_k, b_k, a_off, b_off, wnt, tid);
  const unsigned char* As = rst;
  const unsigned char* Bs = rst + C::kAStage;
  const int grp = lane >> 4, s16 = lane & 15;
  const int b_row_in = 8 * (grp >> 1) + (s16 >> 2);  // k row inside a 16-k substep; row & 3 == s16 >> 2
  const int b_chunk_lo = (s16 & 3) >> 1;
  const int b_byte = (s16 & 1) * 8;

  auto load_frags = [&](int ks, u32x4 (&af)[C::kMB], u32x4 (&bfr)[C::kNB]) {
#pragma unroll
    for (int mb = 0; mb < C::kMB; ++mb) {
      const int m = block_row<C>(wm, mb) + (lane & 31);
      const int chunk = (2 * ks + (lane >> 5)) ^ a_swizzle<C>(m);
      af[mb] = *(const u32x4*)(As + m * C::kARow + chunk * 16);
    }
#pragma unroll
    for (int nb = 0; nb < C::kNB; ++nb) {
      if constexpr (BT) {  // [n][k] tile: one 16-byte read of 8 consecutive k, as for the activations
        const int n = pipe_col_base<EPI, C>(nb, wn) + (lane & 31);
        const int chunk = (2 * ks + (lane >> 5)) ^ a_swizzle<C>(n);
        bfr[nb] = *(const u32x4*)(Bs + n * C::kARow + chunk * 16);
        continue;
      }
      const int c0 = pipe_col_base<EPI, C>(nb, wn) + 16 * (grp & 1);
      const int row = 16 * ks + b_row_in;
      const int chunk = (c0 / 8 + b_chunk_lo) ^ b_swizzle<C>(s16 >> 2);
      const unsigned char* ptr = Bs + row * (2 * C::BN) + chunk * 16 + b_byte;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(MOE_LDS(i16x4, ptr));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(MOE_LDS(i16x4, ptr + 4 * (2 * C::BN)));
      bfr[nb] = pack_tr_pair(lo, hi);
    }
  };
  // This wave's substeps are kw, kw+KW, ...; the fragments of the next one
  // are read while the MFMAs of the current one run.
  u32x4 af[2][C::kMB], bfr[2][C::kNB];
  load_frags(kw, af[0], bfr[0]);
#pragma unroll
  for (int j = 0; j < C::kKSW; ++j) {
    if (j + 1 < C::kKSW) load_frags(kw + (j + 1) * C::KW, af[(j + 1) & 1], bfr[(j + 1) & 1]);
#pragma unroll
    for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < C::kNB; ++nb) acc[mb][nb] = mfma32(af[j & 1][mb], bfr[j & 1][nb], acc[mb][nb]);
  }
}

// Split-K reduction (KW > 1) and epilogue of one tile whose accumulators the
// waves hold; the ring must be idle (every wave past its last LDS read).
template <int EPI, class C>
__device__ __forceinline__ void finish_tile(const GemmParams<bf16_t>& p, f32x16 (&acc)[C::kMB][C::kNB], int row0,
                                            int row_end, int n0, unsigned char* __restrict__ smem, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  const int kw = wave / C::kPos, wpos = wave % C::kPos;
  const int wm = wpos / C::WN, wn = wpos % C::WN;
  if constexpr (C::KW > 1) {
    // Split-K partials through the (now idle) ring: waves kw >= 1 store theirs,
    // wave kw == 0 of each position adds them in the order kw = 1, 2, ... and
    // runs the epilogue.
    float* red = (float*)smem;
    auto slot = [&](int q, int mb, int nb, int i) {
      return ((((q - 1) * C::kPos + wpos) * C::kMB + mb) * C::kNB + nb) * 16 * kWave + i * kWave + lane;
    };
    if (kw > 0) {
#pragma unroll
      for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
        for (int nb = 0; nb < C::kNB; ++nb)
#pragma unroll
          for (int i = 0; i < 16; ++i) red[slot(kw, mb, nb, i)] = acc[mb][nb][i];
    }
    lds_barrier();
    if (kw == 0) {
      for (int q = 1; q < C::KW; ++q)
#pragma unroll
        for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
          for (int nb = 0; nb < C::kNB; ++nb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mb][nb][i] += red[slot(q, mb, nb, i)];
    }
    lds_barrier();  // partials consumed before the next tile refills the ring
    if (kw > 0) return;
  }

  // 32x32 accumulator layout: column = lane%32, row = 8*(i/4) + 4*(lane/32) + i%4.
#pragma unroll
  for (int mb = 0; mb < C::kMB; ++mb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = row0 + block_row<C>(wm, mb) + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      if (row >= row_end) continue;
      if (paired(EPI)) {
#pragma unroll
        for (int j = 0; j < C::kNB / 2; ++j) {
          const int col = n0 + wn * (C::BN / 2 / C::WN) + 32 * j + (lane & 31);
          if (col < p.N) epi_swiglu<EPI>(p, row, col, acc[mb][j][i], acc[mb][j + C::kNB / 2][i]);
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < C::kNB; ++nb) {
          const int col = n0 + wn * (C::BN / C::WN) + 32 * nb + (lane & 31);
          if (col >= p.N) continue;
          if (EPI == kSwiGLUBwd) {
            epi_swiglu_bwd(p, row, col, acc[mb][nb][i]);
            continue;
          }
          float* o = (float*)p.out + (int64_t)row * p.N + col;
          const float v = acc[mb][nb][i];
          if (EPI == kStoreF32) {
            __builtin_nontemporal_store(v, o);  // read once, by the next call
          } else {
            const float sc = p.row_scale ? p.row_scale[row] : 1.0f;
            *o = (p.accumulate ? *o : 0.0f) + sc * v;
          }
        }
      }
    }
  }
}

template <int EPI, class C, bool BT>
__device__ __forceinline__ void run_tile_pipe_v0(const GemmParams<bf16_t>& p, int g, int row0, int row_end, int n0,
                                              unsigned char* __restrict__ smem, bool wnt) {
  const int tid = tile_thread(), lane = tid & 63, wave = tid >> 6;
  const int kw = wave / C::kPos, wpos = wave % C::kPos;
  const int wm = wpos / C::WN, wn = wpos % C::WN;
  const bf16_t* __restrict__ bg = p.b + (int64_t)g * p.b_stride;
  const int K = p.K, ldb = p.ldb;

  // Per-lane source offsets (elements) of this wave's direct loads, slice 0.
  // Rows past the group end only feed output rows that are never stored: with
  // a 2-stage ring (whose waits drain every load) they are not fetched at all
  // (offset -1) and their LDS rows keep stale data; deeper rings, whose waits
  // count loads per slice, fetch the group's last row instead.
  int64_t a_off[C::kALoads];
#pragma unroll
  for (int i = 0; i < C::kALoads; ++i) {
    const int r = (wave * C::kALoads + i) * C::kARowsPerLoad + lane / C::kAChunks;
    const int chunk = (lane % C::kAChunks) ^ a_swizzle<C>(r);
    const int row = min(row0 + r, row_end - 1);
    a_off[i] = (C::STAGES == 2 && row0 + r >= row_end) ? -1 : a_src_row(p, row) * K + chunk * 8;
  }
  int b_off[C::kBLoads];
#pragma unroll
  for (int i = 0; i < C::kBLoads; ++i) {
    if constexpr (BT) {
      // [N, K] weights stage like the activations: LDS row r is staged column r.
      const int r = (wave * C::kBLoads + i) * C::kARowsPerLoad + lane / C::kAChunks;
      const int chunk = (lane % C::kAChunks) ^ a_swizzle<C>(r);
      int nrow;
      if (paired(EPI)) {
        const int half = C::BN / 2;
        const int nc = n0 + r % half;
        nrow = (nc < p.N ? nc : 0) + (r < half ? 0 : p.up_off);
      } else {
        const int nc = n0 + r;
        nrow = nc < p.N ? nc : 0;
      }
      b_off[i] = nrow * ldb + chunk * 8;
      continue;
    }
    const int kr = (wave * C::kBLoads + i) * C::kBRowsPerLoad + lane / C::kBChunks;
    const int chunk = (lane % C::kBChunks) ^ b_swizzle<C>(kr);
    int col;
    if (paired(EPI)) {
      const int half = C::kBChunks / 2;
      const int nc = n0 + 8 * (chunk % half);
      col = (nc < p.N ? nc : 0) + (chunk < half ? 0 : p.up_off);
    } else {
      const int nc = n0 + 8 * chunk;
      col = nc < p.N ? nc : 0;
    }
    b_off[i] = kr * ldb + col;
  }
  const int64_t b_step = BT ? (int64_t)C::BK : (int64_t)C::BK * ldb;  // elements per reduction slice
  const int nk = K / C::BK;

  f32x16 acc[C::kMB][C::kNB];
#pragma unroll
  for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < C::kNB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;

  const bf16_t* a_base = p.a;
#pragma unroll
  for (int s = 0; s < C::STAGES - 1; ++s)
    if (s < nk)
      pipe_issue<C>(smem + s * C::kStage, a_base + s * C::BK, bg + s * b_step, a_off, b_off, wnt, tid);

  for (int kt = 0; kt < nk; ++kt) {
    if (nk - 1 - kt >= C::STAGES - 2) wait_vmcnt<(C::STAGES - 2) * C::kLoads>(); else wait_vmcnt<0>();
    lds_barrier();
    const int kn = kt + C::STAGES - 1;
    pipe_step<EPI, C, BT>(smem + (kn % C::STAGES) * C::kStage, smem + (kt % C::STAGES) * C::kStage, kn < nk,
                          a_base + kn * C::BK, bg + kn * b_step, a_off, b_off, acc, wn, wm, kw, wnt, tid);
  }
  lds_barrier();  // every wave is done with the ring before the next tile refills it
  finish_tile<EPI, C>(p, acc, row0, row_end, n0, smem, tid);
}


// MFMA fragments of one 16-deep substep of a wave: its activation blocks and
// its weight blocks.
template <class C>
struct PipeFrags {
  u32x4 a[C::kMB];
  u32x4 b[C::kNB];
};

// Reads the fragments of substep `ks` of the slice held in ring stage `rst`.
template <int EPI, class C, bool BT>
__device__ __forceinline__ void pipe_read(const unsigned char* __restrict__ rst, int ks, int wm, int wn,
                                          PipeFrags<C>& f, int tid) {
  const int lane = tid & 63;
  const unsigned char* As = rst;
  const unsigned char* Bs = rst + C::kAStage;
  const int grp = lane >> 4, s16 = lane & 15;
#pragma unroll
  for (int mb = 0; mb < C::kMB; ++mb) {
    const int m = block_row<C>(wm, mb) + (lane & 31);
    const int chunk = (2 * ks + (lane >> 5)) ^ a_swizzle<C>(m);
    f.a[mb] = *(const u32x4*)(As + m * C::kARow + chunk * 16);
  }
#pragma unroll
  for (int nb = 0; nb < C::kNB; ++nb) {
    if constexpr (BT) {  // [n][k] tile: one 16-byte read of 8 consecutive k, as for the activations
      const int n = pipe_col_base<EPI, C>(nb, wn) + (lane & 31);
      const int chunk = (2 * ks + (lane >> 5)) ^ a_swizzle<C>(n);
      f.b[nb] = *(const u32x4*)(Bs + n * C::kARow + chunk * 16);
    } else {
      const int b_row_in = 8 * (grp >> 1) + (s16 >> 2);  // k row inside a 16-k substep; row & 3 == s16 >> 2
      const int c0 = pipe_col_base<EPI, C>(nb, wn) + 16 * (grp & 1);
      const int row = 16 * ks + b_row_in;
      const int chunk = (c0 / 8 + ((s16 & 3) >> 1)) ^ b_swizzle<C>(s16 >> 2);
      const unsigned char* ptr = Bs + row * (2 * C::BN) + chunk * 16 + (s16 & 1) * 8;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(MOE_LDS(i16x4, ptr));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(MOE_LDS(i16x4, ptr + 4 * (2 * C::BN)));
      f.b[nb] = pack_tr_pair(lo, hi);
    }
  }
}

template <class C>
__device__ __forceinline__ void pipe_mfmas(const PipeFrags<C>& f, f32x16 (&acc)[C::kMB][C::kNB]) {
#pragma unroll
  for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < C::kNB; ++nb) acc[mb][nb] = mfma32(f.a[mb], f.b[nb], acc[mb][nb]);
}

// Scheduling pattern of one substep: each MFMA is followed by up to PER LDS
// reads of the next substep's fragments (R reads in all), so that the reads
// run under the MFMAs and the last MFMAs leave the reads time to land.
template <int I, int M, int R, int PER>
__device__ __forceinline__ void sched_mfma_reads() {
  if constexpr (I < M) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    constexpr int r = R < PER ? R : PER;
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);  // r LDS reads
    sched_mfma_reads<I + 1, M, R - r, PER>();
  }
}

template <class C, bool BT>
__device__ __forceinline__ void sched_substep() {
  constexpr int M = C::kMB * C::kNB;
  constexpr int R = C::kMB + C::kNB * (BT ? 1 : 2);
  constexpr int slots = M > 2 ? M - 2 : 1;
  sched_mfma_reads<0, M, R, (R + slots - 1) / slots>();
}

// Main loop with the fragments of the next substep read while the MFMAs of
// the current one run, across slice boundaries too: a slice's last substep
// first waits for the next slice (its own loads, then the workgroup barrier,
// after which no wave reads the current stage any more), refills the current
// stage with the slice STAGES ahead, and reads the next slice's first
// fragments; only then do its MFMAs run.  A wave's substeps alternate between
// two fragment sets, so the number of substeps per slice must be even.
template <int EPI, class C, bool BT>
__device__ __forceinline__ void run_tile_pipe_v1(const GemmParams<bf16_t>& p, int g, int row0, int row_end, int n0,
                                                 unsigned char* __restrict__ smem, bool wnt) {
  static_assert(C::kKSW % 2 == 0, "substeps per slice alternate between two fragment sets");
  const int tid = tile_thread(), lane = tid & 63, wave = tid >> 6;
  const int kw = wave / C::kPos, wpos = wave % C::kPos;
  const int wm = wpos / C::WN, wn = wpos % C::WN;
  const bf16_t* __restrict__ bg = p.b + (int64_t)g * p.b_stride;
  const int K = p.K, ldb = p.ldb;

  int64_t a_off[C::kALoads];
#pragma unroll
  for (int i = 0; i < C::kALoads; ++i) {
    const int r = (wave * C::kALoads + i) * C::kARowsPerLoad + lane / C::kAChunks;
    const int chunk = (lane % C::kAChunks) ^ a_swizzle<C>(r);
    const int row = min(row0 + r, row_end - 1);
    a_off[i] = (C::STAGES == 2 && row0 + r >= row_end) ? -1 : a_src_row(p, row) * K + chunk * 8;
  }
  int b_off[C::kBLoads];
#pragma unroll
  for (int i = 0; i < C::kBLoads; ++i) {
    if constexpr (BT) {
      const int r = (wave * C::kBLoads + i) * C::kARowsPerLoad + lane / C::kAChunks;
      const int chunk = (lane % C::kAChunks) ^ a_swizzle<C>(r);
      int nrow;
      if (paired(EPI)) {
        const int half = C::BN / 2;
        const int nc = n0 + r % half;
        nrow = (nc < p.N ? nc : 0) + (r < half ? 0 : p.up_off);
      } else {
        const int nc = n0 + r;
        nrow = nc < p.N ? nc : 0;
      }
      b_off[i] = nrow * ldb + chunk * 8;
    } else {
      const int kr = (wave * C::kBLoads + i) * C::kBRowsPerLoad + lane / C::kBChunks;
      const int chunk = (lane % C::kBChunks) ^ b_swizzle<C>(kr);
      int col;
      if (paired(EPI)) {
        const int half = C::kBChunks / 2;
        const int nc = n0 + 8 * (chunk % half);
        col = (nc < p.N ? nc : 0) + (chunk < half ? 0 : p.up_off);
      } else {
        const int nc = n0 + 8 * chunk;
        col = nc < p.N ? nc : 0;
      }
      b_off[i] = kr * ldb + col;
    }
  }
  const int64_t b_step = BT ? (int64_t)C::BK : (int64_t)C::BK * ldb;
  const int nk = K / C::BK;

  f32x16 acc[C::kMB][C::kNB];
#pragma unroll
  for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < C::kNB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;

  const bf16_t* a_base = p.a;
#pragma unroll
  for (int s = 0; s < C::STAGES - 1; ++s)
    if (s < nk) pipe_issue<C>(smem + s * C::kStage, a_base + s * C::BK, bg + s * b_step, a_off, b_off, wnt, tid);
  // slice 0 has landed in every wave (newer slices may still be in flight)
  if (nk - 1 >= C::STAGES - 2) wait_vmcnt<(C::STAGES - 2) * C::kLoads>(); else wait_vmcnt<0>();
  lds_barrier();
  // the last stage is free: slice STAGES-1 goes there (later slices are issued
  // at the slice boundaries below, STAGES slices ahead)
  if (C::STAGES - 1 < nk)
    pipe_issue<C>(smem + (C::STAGES - 1) * C::kStage, a_base + (C::STAGES - 1) * C::BK,
                  bg + (C::STAGES - 1) * b_step, a_off, b_off, wnt, tid);

  PipeFrags<C> f0, f1;
  pipe_read<EPI, C, BT>(smem, kw, wm, wn, f0, tid);
  // One slice; the last one (LAST) has no boundary.  The last slice is peeled
  // off the loop so that no branch separates a boundary's reads from the
  // MFMAs that hide them.
  auto slice = [&](int kt, auto last) {
    const unsigned char* rst = smem + (kt % C::STAGES) * C::kStage;
#pragma unroll
    for (int j = 0; j < C::kKSW; ++j) {
      PipeFrags<C>& cur = (j & 1) ? f1 : f0;
      PipeFrags<C>& nxt = (j & 1) ? f0 : f1;
      if (j + 1 < C::kKSW) {
        pipe_read<EPI, C, BT>(rst, kw + (j + 1) * C::KW, wm, wn, nxt, tid);
      } else if constexpr (!decltype(last)::value) {
        // the previous substep's MFMAs all issue before this wave waits at the barrier
        __builtin_amdgcn_sched_barrier(0);
        if (nk - 2 - kt >= C::STAGES - 2) wait_vmcnt<(C::STAGES - 2) * C::kLoads>(); else wait_vmcnt<0>();
        lds_barrier();
        const int kn = kt + C::STAGES;
        if (kn < nk)
          pipe_issue<C>(smem + (kt % C::STAGES) * C::kStage, a_base + kn * C::BK, bg + kn * b_step, a_off, b_off,
                        wnt, tid);
        pipe_read<EPI, C, BT>(smem + ((kt + 1) % C::STAGES) * C::kStage, kw, wm, wn, nxt, tid);
      }
      pipe_mfmas<C>(cur, acc);
      sched_substep<C, BT>();
    }
  };
  for (int kt = 0; kt + 1 < nk; ++kt) slice(kt, std::false_type{});
  slice(nk - 1, std::true_type{});
  lds_barrier();  // every wave is done with the ring before the next tile refills it
  finish_tile<EPI, C>(p, acc, row0, row_end, n0, smem, tid);
}

// The loop with two fragment sets holds about 24-48 more VGPRs per lane; it is
// used where each SIMD runs at most two waves of the kernel (256 VGPRs each).
// With four waves per SIMD the extra registers would cost a workgroup per CU
// (128x256x32 with 8 waves: 117 -> 140 VGPRs, 12-24% slower measured).
template <class C>
constexpr bool pipe_loop_v1() {
  return C::kKSW % 2 == 0 && C::kWgsPerCu * C::kWaves <= 8;
}

// Configuration C with a wave's MFMA rows cut to its first MB 32-row blocks.
// The ring (loads, stages, barriers) is C's; only the fragment reads, MFMAs,
// accumulators and epilogue rows of the wave shrink.
template <class C, int MB>
struct RowBlocks : C {
  static constexpr int kMB = MB;
};

// Runs the tile with the wave's MFMA rows cut to nmb 32-row blocks (1 <= nmb
// <= kMB): one loop instance per block count, chosen by a wave-uniform branch.
// Every instance issues the same loads and barriers, so the waves of one
// workgroup may take different instances.
template <int EPI, class C, bool BT, int MB>
__device__ __forceinline__ void run_tile_rows(const GemmParams<bf16_t>& p, int g, int row0, int row_end, int n0,
                                              unsigned char* __restrict__ smem, bool wnt, int nmb) {
  if constexpr (MB > 1) {
    if (nmb < MB) {
      run_tile_rows<EPI, C, BT, MB - 1>(p, g, row0, row_end, n0, smem, wnt, nmb);
      return;
    }
  }
  using R = std::conditional_t<MB == C::kMB, C, RowBlocks<C, MB>>;
  if constexpr (pipe_loop_v1<C>())
    run_tile_pipe_v1<EPI, R, BT>(p, g, row0, row_end, n0, smem, wnt);
  else
    run_tile_pipe_v0<EPI, R, BT>(p, g, row0, row_end, n0, smem, wnt);
}

// A partial row tile: each wave runs only its 32-row blocks that hold rows of
// the group (at least one, so that every wave keeps the same control flow);
// blocks wholly past the group end are neither read from LDS nor multiplied.
// The tile's live blocks are dealt to the wave rows as block_row deals them.
template <int EPI, class C, bool BT>
__device__ __forceinline__ void run_tile_pipe(const GemmParams<bf16_t>& p, int g, int row0, int row_end, int n0,
                                              unsigned char* __restrict__ smem, bool wnt) {
  const int wm = ((int)(threadIdx.x >> 6) % C::kPos) / C::WN;
  const int blocks = (row_end - row0 + 31) / 32;  // live blocks of the tile
  const int nmb = __builtin_amdgcn_readfirstlane(min(max((blocks - wm + C::WM - 1) / C::WM, 1), C::kMB));
  run_tile_rows<EPI, C, BT, C::kMB>(p, g, row0, row_end, n0, smem, wnt, nmb);
}

// The weight-streaming configuration walks its tiles in decode_tile_spread's order.
template <class C>
constexpr bool spread_walk() { return C::BN == 512; }

template <int EPI, class C, int ROLE, bool BT>
__global__ __launch_bounds__(C::NT, C::kWgsPerCu) void grouped_gemm_bf16_pipe(GemmParams<bf16_t> p) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  __shared__ int32_t sOff[kMaxExperts + 1];
  __shared__ int32_t sPre[kMaxExperts + 1];
  __shared__ int32_t sAct[spread_walk<C>() ? kMaxExperts + 1 : 1];
  __shared__ int32_t sWave[C::kWaves];
  const int mtiles = build_tile_prefix<C::BM, C::NT>(p, sOff, sPre, sWave, spread_walk<C>() ? sAct : nullptr);
  const int64_t nt = p.n_tiles;
  const int64_t total = (int64_t)mtiles * nt;
  SpreadWalk sw{};
  if constexpr (spread_walk<C>()) sw = make_spread_walk(p.groups, nt, total, sAct);
  const int64_t ids = spread_walk<C>() ? sw.ids() : total;
  const int out_cols = paired(EPI) ? C::BN / 2 : C::BN;
  for (int64_t id = xcd_slot(); id < ids; id += gridDim.x) {
    TileCoord c;
    if constexpr (spread_walk<C>()) {
      if (!decode_tile_spread<C::BM>(id, p.groups, sw, sOff, sPre, sAct, c)) continue;
    } else {
      c = decode_tile<C::BM>(id, p.groups, nt, sOff, sPre);
    }
    run_tile_pipe<EPI, C, BT>(p, c.g, c.row0, c.row_end, c.ntile * out_cols, smem, c.single);
  }
}

// Routed expert groups and the shared expert in one persistent launch.  The
// routed tiles stream expert weights that are read once (HBM-bound when
// groups are small); the shared-expert tiles reuse one weight over all T rows
// (MFMA-bound).  Tile ids of the two problems are interleaved evenly in units
// of U ids (unit j is shared when floor((j+1)*Us/Utotal) > floor(j*Us/Utotal)),
// so every CU works on both kinds at once and each hides the other's stalls.
// U is one tile, or with the weight-streaming walk one XCD's share of the grid:
// consecutive shared tiles are the row tiles of one weight slab, which then
// run together on one XCD and share the slab in its L2.  A unit past the end
// of its problem's tiles is padding and decodes to no tile.
// The two problems may use different tile configurations CR and CS (same
// thread count; the LDS ring is sized for the larger of the two), so the
// shared expert can take the dense tile while the routed groups take the
// weight-streaming one.
template <class CR, class CS>
constexpr int fused_lds() {
  return CR::kLds > CS::kLds ? CR::kLds : CS::kLds;
}
template <class CR, class CS>
constexpr int fused_wgs() {
  return CR::kWgsPerCu < CS::kWgsPerCu ? CR::kWgsPerCu : CS::kWgsPerCu;
}

template <int EPI_R, int EPI_S, class CR, class CS, bool BT>
__global__ __launch_bounds__(CR::NT, (fused_wgs<CR, CS>())) void grouped_gemm_bf16_fused(GemmParams<bf16_t> pr,
                                                                                          GemmParams<bf16_t> ps) {
  static_assert(CR::NT == CS::NT, "both configurations run in the same workgroups");
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  __shared__ int32_t sOff[kMaxExperts + 1];
  __shared__ int32_t sPre[kMaxExperts + 1];
  __shared__ int32_t sAct[spread_walk<CR>() ? kMaxExperts + 1 : 1];
  __shared__ int32_t sWave[CR::kWaves];
  const int mtiles = build_tile_prefix<CR::BM, CR::NT>(pr, sOff, sPre, sWave, spread_walk<CR>() ? sAct : nullptr);
  const int64_t ntr = pr.n_tiles;
  SpreadWalk sw{};
  if constexpr (spread_walk<CR>()) sw = make_spread_walk(pr.groups, ntr, (int64_t)mtiles * ntr, sAct);
  const int64_t tiles_r = spread_walk<CR>() ? sw.ids() : (int64_t)mtiles * ntr;  // routed ids, padding included
  const int64_t mts = (ps.rows + CS::BM - 1) / CS::BM;
  const int64_t tiles_s = mts * ps.n_tiles;
  const int64_t unit = spread_walk<CR>() ? sw.chunk : 1;
  const int64_t units_s = (tiles_s + unit - 1) / unit;
  const int64_t units = units_s + (tiles_r + unit - 1) / unit;
  const int out_r = paired(EPI_R) ? CR::BN / 2 : CR::BN;
  const int out_s = paired(EPI_S) ? CS::BN / 2 : CS::BN;
  for (int64_t id = xcd_slot(); id < units * unit; id += gridDim.x) {
    const int64_t j = id / unit, r = id - j * unit;
    const int64_t s_before = j * units_s / units;  // shared units before unit j
    if ((j + 1) * units_s / units != s_before) {
      const int64_t st = s_before * unit + r;
      if (st >= tiles_s) continue;
      const int ntile = (int)(st / mts), mtile = (int)(st % mts);
      run_tile_pipe<EPI_S, CS, BT>(ps, 0, mtile * CS::BM, ps.rows, ntile * out_s, smem, ps.rows <= CS::BM);
    } else {
      const int64_t rt = (j - s_before) * unit + r;
      if (rt >= tiles_r) continue;
      TileCoord c;
      if constexpr (spread_walk<CR>()) {
        if (!decode_tile_spread<CR::BM>(rt, pr.groups, sw, sOff, sPre, sAct, c)) continue;
      } else {
        c = decode_tile<CR::BM>(rt, pr.groups, ntr, sOff, sPre);
      }
      run_tile_pipe<EPI_R, CR, BT>(pr, c.g, c.row0, c.row_end, c.ntile * out_r, smem, c.single);
    }
  }
}

// ------------------------------------------------------------------------------------------
// MXFP8 weights: e4m3 codes with one e8m0 scale per 8 elements along the intermediate axis
// ------------------------------------------------------------------------------------------
// PLENA_Compiler PR #69, section "Group C -- shared experts" (fusion-identity
// paragraph).  Codes are stored [N, K] per group (K contiguous, one byte each).
// Their scales run along N for fc1 (kScaleN: scale [n / 8][k]) and along K for
// fc2 (kScaleK: scale [n][k / 8]).  Each ring stage holds the activation tile
// (bf16, as in the pipelined path), the code tile ([BN][BK] bytes) and the
// scale tile, all by direct loads (the scale tile with 4-byte loads, so every
// wave issues the same number of loads).  A weight fragment is one 8-byte LDS
// read of codes plus their scales, converted to bf16 by
// v_cvt_scalef32_pk_bf16_fp8 right before the bf16 MFMA.  An e4m3 value times
// a power of two has at most four significant bits, so the conversion is exact
// whenever the result is a normal bf16 (e8m0 exponents 10..246).
enum ScaleAxis { kScaleN = 0, kScaleK = 1 };

template <int BM_, int BN_, int BK_, int STAGES_, int WM_, int WN_, int KW_>
struct MxCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_, WM = WM_, WN = WN_, KW = KW_;
  static constexpr int kPos = WM * WN;
  static constexpr int kWaves = kPos * KW;
  static constexpr int NT = kWaves * kWave;
  static constexpr int kARow = BK * 2;                  // activation row bytes (bf16)
  static constexpr int kAChunks = BK / 8;
  static constexpr int kAStage = BM * kARow;
  static constexpr int kBRow = BK;                      // code row bytes
  static constexpr int kBChunks = BK / 16;
  static constexpr int kBStage = BN * BK;
  static constexpr int kSStage = BN * BK / 8;
  static constexpr int kStage = kAStage + kBStage + kSStage;
  static constexpr int kALoads = kAStage / 1024 / kWaves;
  static constexpr int kBLoads = kBStage / 1024 / kWaves;
  static constexpr int kSLoads = kSStage / 256 / kWaves;  // 4 bytes per lane
  static constexpr int kLoads = kALoads + kBLoads + kSLoads;
  static constexpr int kARowsPerLoad = 1024 / kARow;
  static constexpr int kBRowsPerLoad = 1024 / kBRow;
  static constexpr int kMB = BM / WM / 32;
  static constexpr int kNB = BN / WN / 32;
  static constexpr int kKS = BK / 16;
  static constexpr int kKSW = kKS / KW;
  static constexpr int kLds = STAGES * kStage;
  static constexpr int kRed = (KW - 1) * kPos * kMB * kNB * 16 * kWave * 4;
  static constexpr int kFit = (160 * 1024) / (kLds + 9 * 1024);
  static constexpr int kWgsPerCu = kFit < 1 ? 1 : (kFit > 4 ? 4 : kFit);
  static_assert(kAStage % (1024 * kWaves) == 0 && kBStage % (1024 * kWaves) == 0 &&
                    kSStage % (256 * kWaves) == 0,
                "slices must split evenly into direct loads per wave");
  static_assert(kMB >= 1 && kNB >= 2 && kNB % 2 == 0, "wave tile must hold whole 32x32 blocks");
  static_assert(kKS % KW == 0 && kRed <= kLds, "split-K layout");
  static_assert(BK == 128, "the scale tiles below assume 128-deep slices");
};

// Decode shapes: 32-row tiles, 128 staged columns, 128-deep slices, 2-stage
// ring, 4 waves (2 column positions x 2 split-K waves), two workgroups per CU
// (the best of three decode configurations measured).  Prefill shapes: 128 x
// 256 tiles with 8 waves, which convert each weight fragment once per 128 rows.
typedef MxCfg<32, 128, 128, 2, 1, 2, 2> MxCfgDecode;
typedef MxCfg<128, 256, 128, 2, 2, 4, 1> MxCfgPrefill;

template <int ROWBYTES>
__device__ __forceinline__ int row_swizzle(int row) {
  return (row / (256 / ROWBYTES)) % (ROWBYTES / 16);
}

// 2^(s - 127) for e8m0 byte s in 1..254 (the kernels require exponents 10..246
// anyway; 0 and the NaN code 255 are not decoded).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) { return __uint_as_float(s << 23); }

// Two e4m3 codes (bytes 0-1, or with HI bytes 2-3, of `codes`) times `scale`, as bf16x2.
template <bool HI>
__device__ __forceinline__ uint32_t cvt_bf16x2(uint32_t codes, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, scale, HI));
}

// 8 consecutive-k codes of one column, one scale for all of them (kScaleK).
__device__ __forceinline__ u32x4 mx_frag_one_scale(u32x2 c, float f) {
  return u32x4{cvt_bf16x2<false>(c[0], f), cvt_bf16x2<true>(c[0], f), cvt_bf16x2<false>(c[1], f),
               cvt_bf16x2<true>(c[1], f)};
}

// 8 consecutive-k codes of one column with a scale each (kScaleN): each
// conversion scales a pair by one factor, so the pair's two halves come from
// two conversions.
template <bool HI>
__device__ __forceinline__ uint32_t mx_pair_two_scales(uint32_t word, uint32_t sbytes) {
  const uint32_t lo_val = cvt_bf16x2<HI>(word, e8m0_to_f32(sbytes & 0xffu));
  const uint32_t hi_val = cvt_bf16x2<HI>(word, e8m0_to_f32((sbytes >> 8) & 0xffu));
  return (lo_val & 0xffffu) | (hi_val & 0xffff0000u);
}

__device__ __forceinline__ u32x4 mx_frag_eight_scales(u32x2 c, u32x2 sw) {
  return u32x4{mx_pair_two_scales<false>(c[0], sw[0]), mx_pair_two_scales<true>(c[0], sw[0] >> 16),
               mx_pair_two_scales<false>(c[1], sw[1]), mx_pair_two_scales<true>(c[1], sw[1] >> 16)};
}

// Raw fragments of one MX substep: the activation blocks, and per weight
// block 8 codes plus their scale bytes (8 for kScaleN, 1 for kScaleK).
template <class C>
struct MxFrags {
  u32x4 a[C::kMB];
  u32x2 codes[C::kNB];
  u32x2 scales[C::kNB];
};

template <int EPI, class C, int SAX>
__device__ __forceinline__ void mx_read(const unsigned char* __restrict__ As, const unsigned char* __restrict__ Bs,
                                        const unsigned char* __restrict__ Ss, int ks, int wm, int wn,
                                        MxFrags<C>& f) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int mb = 0; mb < C::kMB; ++mb) {
    const int m = block_row<C>(wm, mb) + (lane & 31);
    const int chunk = (2 * ks + (lane >> 5)) ^ row_swizzle<C::kARow>(m);
    f.a[mb] = *(const u32x4*)(As + m * C::kARow + chunk * 16);
  }
#pragma unroll
  for (int nb = 0; nb < C::kNB; ++nb) {
    const int n = pipe_col_base<EPI, C>(nb, wn) + (lane & 31);
    const int kg = lane >> 5;  // k = 16 ks + 8 kg .. + 7
    const int chunk = ks ^ row_swizzle<C::kBRow>(n);
    f.codes[nb] = *(const u32x2*)(Bs + n * C::kBRow + chunk * 16 + 8 * kg);
    if (SAX == kScaleK)
      f.scales[nb] = u32x2{(uint32_t)Ss[n * (C::BK / 8) + 2 * ks + kg], 0u};
    else
      f.scales[nb] = *(const u32x2*)(Ss + (n / 8) * C::BK + 16 * ks + 8 * kg);
  }
}

// One MX pipeline step: start the direct loads of a future slice into `wst`,
// then run this wave's substeps of the slice held in `rst`, reading the
// fragments of the next substep while the current one is converted and
// multiplied.  The __restrict__ stage pointers let the compiler skip waiting
// for the in-flight direct loads before the LDS reads.
// Direct loads of one slice (activations, codes, scales) into a ring stage;
// wnt: the weights are read once (non-temporal policy, as in the bf16 path).
template <class C, int POL>
__device__ __forceinline__ void mx_issue_pol(unsigned char* __restrict__ st, const bf16_t* a_k,
                                             const unsigned char* b_k, const unsigned char* s_k, const int64_t* a_off,
                                             const int* b_off, const int* s_off) {
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < C::kALoads; ++i)
    if (C::STAGES != 2 || a_off[i] >= 0)
      __builtin_amdgcn_global_load_lds(MOE_GLOBAL(void, a_k + a_off[i]),
                                       MOE_LDS(void, st + (wave * C::kALoads + i) * 1024), 16, 0, 0);
#pragma unroll
  for (int i = 0; i < C::kBLoads; ++i)
    __builtin_amdgcn_global_load_lds(MOE_GLOBAL(void, b_k + b_off[i]),
                                     MOE_LDS(void, st + C::kAStage + (wave * C::kBLoads + i) * 1024), 16, 0, POL);
#pragma unroll
  for (int i = 0; i < C::kSLoads; ++i)
    __builtin_amdgcn_global_load_lds(MOE_GLOBAL(void, s_k + s_off[i]),
                                     MOE_LDS(void, st + C::kAStage + C::kBStage + (wave * C::kSLoads + i) * 256), 4,
                                     0, POL);
}

template <class C>
__device__ __forceinline__ void mx_issue(unsigned char* __restrict__ st, const bf16_t* a_k, const unsigned char* b_k,
                                         const unsigned char* s_k, const int64_t* a_off, const int* b_off,
                                         const int* s_off, bool wnt) {
  if (wnt)
    mx_issue_pol<C, kWeightLoadPolicy>(st, a_k, b_k, s_k, a_off, b_off, s_off);
  else
    mx_issue_pol<C, 0>(st, a_k, b_k, s_k, a_off, b_off, s_off);
}

template <int EPI, class C, int SAX>
__device__ __forceinline__ void mx_step(unsigned char* __restrict__ wst, const unsigned char* __restrict__ rst,
                                        bool issue, const bf16_t* a_k, const unsigned char* b_k,
                                        const unsigned char* s_k, const int64_t* a_off, const int* b_off,
                                        const int* s_off, f32x16 (&acc)[C::kMB][C::kNB], int wn, int wm, int kw,
                                        bool wnt) {
  if (issue) mx_issue<C>(wst, a_k, b_k, s_k, a_off, b_off, s_off, wnt);
  const unsigned char* As = rst;
  const unsigned char* Bs = rst + C::kAStage;
  const unsigned char* Ss = rst + C::kAStage + C::kBStage;
  MxFrags<C> fr[2];
  mx_read<EPI, C, SAX>(As, Bs, Ss, kw, wm, wn, fr[0]);
#pragma unroll
  for (int j = 0; j < C::kKSW; ++j) {
    if (j + 1 < C::kKSW) mx_read<EPI, C, SAX>(As, Bs, Ss, kw + (j + 1) * C::KW, wm, wn, fr[(j + 1) & 1]);
    const MxFrags<C>& f = fr[j & 1];
    u32x4 bfr[C::kNB];
#pragma unroll
    for (int nb = 0; nb < C::kNB; ++nb)
      bfr[nb] = SAX == kScaleK ? mx_frag_one_scale(f.codes[nb], e8m0_to_f32(f.scales[nb][0]))
                               : mx_frag_eight_scales(f.codes[nb], f.scales[nb]);
#pragma unroll
    for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < C::kNB; ++nb) acc[mb][nb] = mfma32(f.a[mb], bfr[nb], acc[mb][nb]);
  }
}

template <int EPI, class C, int SAX>
__device__ __forceinline__ void run_tile_mx(const GemmParams<bf16_t>& p, int g, int row0, int row_end, int n0,
                                            unsigned char* __restrict__ smem, bool wnt) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kw = wave / C::kPos, wpos = wave % C::kPos;
  const int wm = wpos / C::WN, wn = wpos % C::WN;
  const int K = p.K;
  const unsigned char* __restrict__ bq = (const unsigned char*)p.b + (int64_t)g * p.b_stride;
  const unsigned char* __restrict__ bs = p.sc + (int64_t)g * p.sc_stride;

  // Weight row (an n in [0, rows of the group's weight)) of staged column r;
  // columns past N read row 0 and only feed outputs that are never stored.
  auto wrow = [&](int r) -> int {
    if (paired(EPI)) {
      const int half = C::BN / 2;
      const int nc = n0 + r % half;
      return (nc < p.N ? nc : 0) + (r < half ? 0 : p.up_off);
    }
    const int nc = n0 + r;
    return nc < p.N ? nc : 0;
  };

  // Rows past the group end: not fetched in 2-stage rings, as in run_tile_pipe.
  int64_t a_off[C::kALoads];
#pragma unroll
  for (int i = 0; i < C::kALoads; ++i) {
    const int r = (wave * C::kALoads + i) * C::kARowsPerLoad + lane / C::kAChunks;
    const int chunk = (lane % C::kAChunks) ^ row_swizzle<C::kARow>(r);
    const int row = min(row0 + r, row_end - 1);
    a_off[i] = (C::STAGES == 2 && row0 + r >= row_end) ? -1 : a_src_row(p, row) * K + chunk * 8;
  }
  int b_off[C::kBLoads];
#pragma unroll
  for (int i = 0; i < C::kBLoads; ++i) {
    const int r = (wave * C::kBLoads + i) * C::kBRowsPerLoad + lane / C::kBChunks;
    const int chunk = (lane % C::kBChunks) ^ row_swizzle<C::kBRow>(r);
    b_off[i] = wrow(r) * K + chunk * 16;
  }
  int s_off[C::kSLoads];
#pragma unroll
  for (int i = 0; i < C::kSLoads; ++i) {
    const int j = wave * C::kSLoads + i;  // 256-byte piece of the scale tile
    if (SAX == kScaleN) {
      // [BN / 8][BK] bytes: piece j holds scale rows 2j and 2j + 1
      const int srow = 2 * j + lane / 32, col = 4 * (lane % 32);
      s_off[i] = (wrow(8 * srow) / 8) * K + col;
    } else {
      // [BN][BK / 8] bytes: piece j holds staged columns 16j .. 16j + 15
      const int r = 16 * j + lane / 4, col = 4 * (lane % 4);
      s_off[i] = wrow(r) * (K / 8) + col;
    }
  }
  constexpr int kSStep = SAX == kScaleN ? C::BK : C::BK / 8;  // scale bytes per slice along k
  const int nk = K / C::BK;

  f32x16 acc[C::kMB][C::kNB];
#pragma unroll
  for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < C::kNB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;

  // Prologue: the first STAGES - 1 slices (the second stage pointer of each
  // call is unused because nothing is computed yet).
#pragma unroll
  for (int s = 0; s < C::STAGES - 1; ++s)
    if (s < nk)
      mx_issue<C>(smem + s * C::kStage, p.a + (int64_t)s * C::BK, bq + (int64_t)s * C::BK,
                  bs + (int64_t)s * kSStep, a_off, b_off, s_off, wnt);

  for (int kt = 0; kt < nk; ++kt) {
    if (nk - 1 - kt >= C::STAGES - 2) wait_vmcnt<(C::STAGES - 2) * C::kLoads>(); else wait_vmcnt<0>();
    lds_barrier();
    const int kn = kt + C::STAGES - 1;
    mx_step<EPI, C, SAX>(smem + (kn % C::STAGES) * C::kStage, smem + (kt % C::STAGES) * C::kStage, kn < nk,
                         p.a + (int64_t)kn * C::BK, bq + (int64_t)kn * C::BK, bs + (int64_t)kn * kSStep, a_off,
                         b_off, s_off, acc, wn, wm, kw, wnt);
  }
  lds_barrier();  // every wave is done with the ring before the next tile refills it
  finish_tile<EPI, C>(p, acc, row0, row_end, n0, smem, tid);
}

template <int EPI, class C, int SAX, int ROLE>
__global__ __launch_bounds__(C::NT, C::kWgsPerCu) void grouped_gemm_mx8(GemmParams<bf16_t> p) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  __shared__ int32_t sOff[kMaxExperts + 1];
  __shared__ int32_t sPre[kMaxExperts + 1];
  __shared__ int32_t sWave[C::kWaves];
  const int mtiles = build_tile_prefix<C::BM, C::NT>(p, sOff, sPre, sWave);
  const int64_t nt = p.n_tiles;
  const int64_t total = (int64_t)mtiles * nt;
  const int out_cols = paired(EPI) ? C::BN / 2 : C::BN;
  for (int64_t id = xcd_slot(); id < total; id += gridDim.x) {
    const TileCoord c = decode_tile<C::BM>(id, p.groups, nt, sOff, sPre);
    run_tile_mx<EPI, C, SAX>(p, c.g, c.row0, c.row_end, c.ntile * out_cols, smem, c.single);
  }
}

// MXFP8 routed groups and the MXFP8 shared expert in one persistent launch
// (tiles interleaved as in grouped_gemm_bf16_fused).
template <int EPI_R, int EPI_S, class C, int SAX>
__global__ __launch_bounds__(C::NT, C::kWgsPerCu) void grouped_gemm_mx8_fused(GemmParams<bf16_t> pr,
                                                                               GemmParams<bf16_t> ps) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  __shared__ int32_t sOff[kMaxExperts + 1];
  __shared__ int32_t sPre[kMaxExperts + 1];
  __shared__ int32_t sWave[C::kWaves];
  const int mtiles = build_tile_prefix<C::BM, C::NT>(pr, sOff, sPre, sWave);
  const int64_t ntr = pr.n_tiles;
  const int64_t tiles_r = (int64_t)mtiles * ntr;
  const int64_t mts = (ps.rows + C::BM - 1) / C::BM;
  const int64_t tiles_s = mts * ps.n_tiles;
  const int64_t total = tiles_r + tiles_s;
  const int out_r = paired(EPI_R) ? C::BN / 2 : C::BN;
  const int out_s = paired(EPI_S) ? C::BN / 2 : C::BN;
  for (int64_t id = xcd_slot(); id < total; id += gridDim.x) {
    const int64_t s_before = id * tiles_s / total;
    if ((id + 1) * tiles_s / total != s_before) {
      const int ntile = (int)(s_before / mts), mtile = (int)(s_before % mts);
      run_tile_mx<EPI_S, C, SAX>(ps, 0, mtile * C::BM, ps.rows, ntile * out_s, smem, ps.rows <= C::BM);
    } else {
      const TileCoord c = decode_tile<C::BM>(id - s_before, pr.groups, ntr, sOff, sPre);
      run_tile_mx<EPI_R, C, SAX>(pr, c.g, c.row0, c.row_end, c.ntile * out_r, smem, c.single);
    }
  }
}

// ------------------------------------------------------------------------------------------
// Weight gradients: out[g] = P[rows of g]^T Q[rows of g] (same-M/N grouped GEMM)
// ------------------------------------------------------------------------------------------
// VeOmni docs "Fused MoE Kernel Notes", section "Backward grouped-GEMM launch
// bound": the weight gradients are a grouped GEMM whose groups share the output
// shape [M, N] and differ in reduction length -- the group's row count, which
// comes from the realized expert_offsets like every other bound here.
//
// P [rows, M] and Q [rows, N] are row-major, so both operands sit in LDS like
// the [K, N] weight tile of the forward path: a group row (the reduction index
// k) per LDS row, M or N across it, 16-byte chunks XOR-swizzled by the row.
// Both MFMA fragments come from two ds_read_b64_tr_b16 transpose reads each:
// an A fragment (8 consecutive k of one output row) and a B fragment (8
// consecutive k of one output column) have the same register layout.  A
// group's last slice is partial unless its row count is a multiple of BK: its
// rows past the group end are fetched from the group's last row and then
// overwritten with zeros in LDS, so no other group's rows contribute.  A group
// with no rows stores a zero tile.
template <int BM_, int BN_, int BK_, int STAGES_, int WM_, int WN_>
struct WgCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_, WM = WM_, WN = WN_;
  static constexpr int kWaves = WM * WN;
  static constexpr int NT = kWaves * kWave;
  static constexpr int kPChunks = BM / 8, kQChunks = BN / 8;   // 16-byte chunks per LDS row
  static constexpr int kPRow = BM * 2, kQRow = BN * 2;           // LDS row bytes
  static constexpr int kPStage = BK * kPRow, kQStage = BK * kQRow;
  static constexpr int kStage = kPStage + kQStage;
  static constexpr int kPLoads = kPStage / 1024 / kWaves, kQLoads = kQStage / 1024 / kWaves;
  static constexpr int kLoads = kPLoads + kQLoads;
  static constexpr int kPRowsPerLoad = 64 / kPChunks, kQRowsPerLoad = 64 / kQChunks;
  static constexpr int kMB = BM / WM / 32, kNB = BN / WN / 32;
  static constexpr int kKS = BK / 16;
  static constexpr int kLds = STAGES * kStage;
  static constexpr int kFit = (160 * 1024) / (kLds + 1024);
  static constexpr int kWgsPerCu = kFit < 1 ? 1 : (kFit > 4 ? 4 : kFit);
  static_assert(kPChunks >= 8 && kQChunks >= 8 && kPChunks <= 64 && kQChunks <= 64, "tile widths 64..512");
  static_assert(kPStage % (1024 * kWaves) == 0 && kQStage % (1024 * kWaves) == 0,
                "slices must split into 1 KiB loads per wave");
  static_assert(kMB >= 1 && kNB >= 1, "wave tile must hold whole 32x32 blocks");
};

// 128x128 tiles, 32-deep slices, a 32 KiB two-stage ring: four workgroups per
// CU.  Measured on MI355X against 64-deep slices, 3- to 6-stage rings,
// 128x256 / 256x128 / 64x256 tiles, 8-byte stores of a swapped product,
// non-temporal stores and an M-fastest tile order: all within a few percent or
// slower.
typedef WgCfg<128, 128, 32, 2, 2, 2> WgCfgUsed;

struct WgParams {
  const bf16_t* p;          // [rows, M]
  const bf16_t* q;          // [rows, N]
  const int32_t* offsets;   // [groups + 1]
  int groups, rows, M, N;
  bf16_t* out;              // [groups, M, N]
  int m_tiles, n_tiles;
};

// Swizzle of a k-major tile with CHUNKS 16-byte chunks per row (see a_swizzle/b_swizzle).
template <int CHUNKS>
__device__ __forceinline__ int kn_swizzle(int k) { return CHUNKS >= 16 ? 4 * (k & 3) : 4 * ((k >> 1) & 1); }

// MFMA fragment of the 32 columns [c_blk, c_blk + 32) of a k-major LDS tile,
// k rows [16 ks, 16 ks + 16): lane L gets column c_blk + L % 32, k = 8 (L / 32) .. + 7.
template <int CHUNKS>
__device__ __forceinline__ u32x4 kn_frag(const unsigned char* __restrict__ tile, int c_blk, int ks) {
  const int lane = threadIdx.x & 63, grp = lane >> 4, s16 = lane & 15;
  const int row = 16 * ks + 8 * (grp >> 1) + (s16 >> 2);
  const int c0 = c_blk + 16 * (grp & 1);
  const int chunk = (c0 / 8 + ((s16 & 3) >> 1)) ^ kn_swizzle<CHUNKS>(s16 >> 2);
  const unsigned char* ptr = tile + row * (16 * CHUNKS) + chunk * 16 + (s16 & 1) * 8;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(MOE_LDS(i16x4, ptr));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(MOE_LDS(i16x4, ptr + 4 * 16 * CHUNKS));
  return pack_tr_pair(lo, hi);
}

template <class C>
__device__ __forceinline__ void wg_compute(const unsigned char* __restrict__ st, f32x16 (&acc)[C::kMB][C::kNB],
                                           int wm, int wn) {
  const unsigned char* Ps = st;
  const unsigned char* Qs = st + C::kPStage;
  u32x4 af[2][C::kMB], bf[2][C::kNB];
  auto read = [&](int ks, u32x4 (&a)[C::kMB], u32x4 (&b)[C::kNB]) {
#pragma unroll
    for (int mb = 0; mb < C::kMB; ++mb) a[mb] = kn_frag<C::kPChunks>(Ps, wm * (C::BM / C::WM) + 32 * mb, ks);
#pragma unroll
    for (int nb = 0; nb < C::kNB; ++nb) b[nb] = kn_frag<C::kQChunks>(Qs, wn * (C::BN / C::WN) + 32 * nb, ks);
  };
  read(0, af[0], bf[0]);
#pragma unroll
  for (int ks = 0; ks < C::kKS; ++ks) {
    if (ks + 1 < C::kKS) read(ks + 1, af[(ks + 1) & 1], bf[(ks + 1) & 1]);
    // The product is taken swapped (the Q fragment as the MFMA's A operand),
    // so that a lane holds four consecutive output columns of one output row
    // for the LDS-staged epilogue.
#pragma unroll
    for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < C::kNB; ++nb)
        acc[mb][nb] = mfma32(bf[ks & 1][nb], af[ks & 1][mb], acc[mb][nb]);
  }
}

constexpr int kBandM = 8, kBandN = 16;   // tiles per group run in 8 x 16 blocks (L2 reuse)

// Position of a workgroup in its stream of slices: tile id (>= total when the
// stream is exhausted), the tile's group, row range and output corner, and the
// slice kt of nk.
struct WgCursor {
  int64_t id;
  int g, lo, hi, m0, n0, kt, nk;
};

template <class C>
__device__ __forceinline__ void wg_locate(const WgParams& p, int64_t per_group, WgCursor& c) {
  c.g = (int)(c.id / per_group);
  const int rem = (int)(c.id % per_group);
  c.lo = min(max(p.offsets[c.g], 0), p.rows);
  c.hi = max(min(max(p.offsets[c.g + 1], 0), p.rows), c.lo);
  // Blocks of up to kBandM x kBandN tiles (a band of M tiles, then blocks of N
  // tiles along it; N fastest inside a block): the 128 consecutive ids an XCD
  // runs at once read kBandM + kBandN operand tiles, which stay in its L2.
  const int band = rem / (kBandM * p.n_tiles);
  const int r1 = rem % (kBandM * p.n_tiles);
  const int sm = min(kBandM, p.m_tiles - band * kBandM);
  const int blk = r1 / (sm * kBandN);
  const int r2 = r1 % (sm * kBandN);
  const int sn = min(kBandN, p.n_tiles - blk * kBandN);
  c.m0 = (band * kBandM + r2 / sn) * C::BM;
  c.n0 = (blk * kBandN + r2 % sn) * C::BN;
  c.kt = 0;
  c.nk = (c.hi - c.lo + C::BK - 1) / C::BK;
}

// Zero tile of a group without rows (16-byte stores; N is a multiple of 8).
template <class C>
__device__ __forceinline__ void wg_store_zero(const WgParams& p, const WgCursor& c) {
  constexpr int kChunks = C::BN / 8;
  bf16_t* out = p.out + (int64_t)c.g * p.M * p.N;
  for (int v = threadIdx.x; v < C::BM * kChunks; v += C::NT) {
    const int m = c.m0 + v / kChunks, n = c.n0 + 8 * (v % kChunks);
    if (m < p.M && n < p.N) *(u32x4*)(out + (int64_t)m * p.N + n) = u32x4{0u, 0u, 0u, 0u};
  }
}

// Moves c to the first tile at or after c.id whose group has rows; with ZERO,
// stores the zero tiles of the empty groups it passes.
template <class C, bool ZERO>
__device__ __forceinline__ void wg_seek(const WgParams& p, int64_t per_group, int64_t total, WgCursor& c) {
  while (c.id < total) {
    wg_locate<C>(p, per_group, c);
    if (c.nk > 0) return;
    if (ZERO) wg_store_zero<C>(p, c);
    c.id += gridDim.x;
  }
}

// Direct loads of slice c.kt of tile c into ring stage `st`: rows
// lo + kt*BK .. + BK - 1, clamped to the group's last row; columns past M or N
// read column 0 (they only feed outputs that are never stored).
template <class C>
__device__ __forceinline__ void wg_issue(unsigned char* __restrict__ st, const WgParams& p, const WgCursor& c) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row0 = c.lo + c.kt * C::BK, last = c.hi - 1;
#pragma unroll
  for (int i = 0; i < C::kPLoads; ++i) {
    const int kr = (wave * C::kPLoads + i) * C::kPRowsPerLoad + lane / C::kPChunks;
    const int col = c.m0 + 8 * ((lane % C::kPChunks) ^ kn_swizzle<C::kPChunks>(kr));
    const int row = min(row0 + kr, last);
    __builtin_amdgcn_global_load_lds(MOE_GLOBAL(void, p.p + (int64_t)row * p.M + (col < p.M ? col : 0)),
                                     MOE_LDS(void, st + (wave * C::kPLoads + i) * 1024), 16, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < C::kQLoads; ++i) {
    const int kr = (wave * C::kQLoads + i) * C::kQRowsPerLoad + lane / C::kQChunks;
    const int col = c.n0 + 8 * ((lane % C::kQChunks) ^ kn_swizzle<C::kQChunks>(kr));
    const int row = min(row0 + kr, last);
    __builtin_amdgcn_global_load_lds(MOE_GLOBAL(void, p.q + (int64_t)row * p.N + (col < p.N ? col : 0)),
                                     MOE_LDS(void, st + C::kPStage + (wave * C::kQLoads + i) * 1024), 16, 0, 0);
  }
}

template <class C>
__device__ __forceinline__ void wg_store_tile_staged(const WgParams& p, const WgCursor& c,
                                                     f32x16 (&acc)[C::kMB][C::kNB], int wm, int wn,
                                                     unsigned char* __restrict__ stage) {
  static_assert(C::BM / C::WM == 64 && C::BN / C::WN == 64, "staged epilogue: 64x64 per wave");
  static_assert(C::NT / kWave * 4096 <= C::kStage, "staged epilogue: 4 KiB per wave in one stage");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  unsigned char* buf = stage + wave * 4096;
  bf16_t* out = p.out + (int64_t)c.g * p.M * p.N;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int r = lane & 31;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x16& a = acc[mb][nb];
        const u32x2 v{f32_to_bf16_rne(a[4 * q]) | (f32_to_bf16_rne(a[4 * q + 1]) << 16),
                      f32_to_bf16_rne(a[4 * q + 2]) | (f32_to_bf16_rne(a[4 * q + 3]) << 16)};
        const int chunk = (4 * nb + q) ^ ((r >> 1) & 7);
        *(u32x2*)(buf + r * 128 + chunk * 16 + 8 * (lane >> 5)) = v;
      }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 8 * j + (lane >> 3), ch = lane & 7;
      const u32x4 v = *(const u32x4*)(buf + row * 128 + ((ch ^ ((row >> 1) & 7)) * 16));
      const int m = c.m0 + wm * 64 + 32 * mb + row, n = c.n0 + wn * 64 + 8 * ch;
      if (m < p.M && n < p.N) *(u32x4*)(out + (int64_t)m * p.N + n) = v;
    }
  }
#pragma unroll
  for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < C::kNB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;
}

// A workgroup's tiles (ids slot, slot + grid, ... group-major, then in the
// blocks described at wg_locate, so consecutive ids share a group's rows and
// an XCD's L2, and neighbouring output tiles of one row band are written together)
// form one stream of reduction slices.  The LDS ring keeps STAGES - 1 slices
// in flight across tile boundaries, so the next tile's loads overlap the
// current tile's last MFMAs and its stores; groups are short (a few hundred
// rows), so a ring restarted per tile would expose the load latency on every
// tile.  Tiles of groups without rows take no slices: the issue cursor stores
// their zero tiles as it passes them.
// ROLE (1: fc1's weights, 2: fc2's) only names the two launches apart in profiles.
template <class C, int ROLE>
__global__ __launch_bounds__(C::NT, C::kWgsPerCu) void grouped_wgrad_bf16(WgParams p) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int tid = threadIdx.x, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int64_t per_group = (int64_t)p.m_tiles * p.n_tiles;
  const int64_t total = per_group * p.groups;

  WgCursor ic;
  ic.id = xcd_slot();
  wg_seek<C, true>(p, per_group, total, ic);
  WgCursor cc = ic;
  int outstanding = 0;  // slices issued and not yet consumed
  auto issue_next = [&](int stage) {
    wg_issue<C>(smem + stage * C::kStage, p, ic);
    ++outstanding;
    if (++ic.kt == ic.nk) {
      ic.id += gridDim.x;
      wg_seek<C, true>(p, per_group, total, ic);
    }
  };
#pragma unroll
  for (int s = 0; s < C::STAGES - 1; ++s)
    if (ic.id < total) issue_next(s);

  f32x16 acc[C::kMB][C::kNB];
#pragma unroll
  for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < C::kNB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;

  int stage = 0;
  while (cc.id < total) {
    // The slice in `stage` has landed once at most `outstanding - 1` newer slices' loads are pending.
    if (outstanding - 1 >= C::STAGES - 2) wait_vmcnt<(C::STAGES - 2) * C::kLoads>(); else wait_vmcnt<0>();
    lds_barrier();
    unsigned char* st = smem + stage * C::kStage;
    const int valid = (cc.hi - cc.lo) - cc.kt * C::BK;
    if (valid < C::BK) {
      // A group's partial last slice: zero its rows past the group end.
      for (int b = valid * C::kPRow + tid * 16; b < C::kPStage; b += C::NT * 16)
        *(u32x4*)(st + b) = u32x4{0u, 0u, 0u, 0u};
      for (int b = valid * C::kQRow + tid * 16; b < C::kQStage; b += C::NT * 16)
        *(u32x4*)(st + C::kPStage + b) = u32x4{0u, 0u, 0u, 0u};
      lds_barrier();
    }
    // The stage consumed in the previous iteration is free (every wave passed the barrier).
    if (ic.id < total) issue_next((stage + C::STAGES - 1) % C::STAGES);
    wg_compute<C>(st, acc, wm, wn);
    --outstanding;
    if (++cc.kt == cc.nk) {
      lds_barrier();  // every wave is done reading `st`; the next iteration's barrier frees it again
      wg_store_tile_staged<C>(p, cc, acc, wm, wn, st);
      cc.id += gridDim.x;
      wg_seek<C, false>(p, per_group, total, cc);
    }
    stage = (stage + 1) % C::STAGES;
  }
}

// float32 weight gradients: one thread per output element, rows of its group in order.
__global__ __launch_bounds__(256) void grouped_wgrad_f32(const float* __restrict__ P, const float* __restrict__ Q,
                                                        const int32_t* __restrict__ offsets, int groups, int rows,
                                                        int M, int N, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)groups * M * N) return;
  const int g = (int)(i / ((int64_t)M * N));
  const int64_t mn = i % ((int64_t)M * N);
  const int m = (int)(mn / N), n = (int)(mn % N);
  const int lo = min(max(offsets[g], 0), rows);
  const int hi = max(min(max(offsets[g + 1], 0), rows), lo);
  float v = 0.f;
  for (int r = lo; r < hi; ++r) v = fmaf(P[(int64_t)r * M + m], Q[(int64_t)r * N + n], v);
  out[i] = v;
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
  const float* ar = p.a + a_src_row(p, row) * p.K;
  // element (k, n) of the group's weight
  auto w = [&](int k, int n) { return p.bt ? bg[(int64_t)n * p.ldb + k] : bg[(int64_t)k * p.ldb + n]; };
  if (paired(EPI)) {
    float gs = 0.f, us = 0.f;
    for (int k = 0; k < p.K; ++k) {
      const float av = ar[k];
      gs = fmaf(av, w(k, col), gs);
      us = fmaf(av, w(k, p.up_off + col), us);
    }
    epi_swiglu<EPI>(p, row, col, gs, us);
  } else {
    float v = 0.f;
    for (int k = 0; k < p.K; ++k) v = fmaf(ar[k], w(k, col), v);
    if (EPI == kSwiGLUBwd) {
      epi_swiglu_bwd(p, row, col, v);
      return;
    }
    float* o = (float*)p.out + (int64_t)row * p.N + col;
    if (EPI == kStoreF32) {
      *o = v;
    } else {
      const float sc = p.row_scale ? p.row_scale[row] : 1.0f;
      *o = (p.accumulate ? *o : 0.0f) + sc * v;
    }
  }
}

int persistent_grid(int64_t upper_tiles, int slots) {
  int64_t g = upper_tiles < (int64_t)slots ? upper_tiles : (int64_t)slots;
  if (g < 1) g = 1;
  g = (g + kXcds - 1) / kXcds * kXcds;
  return (int)g;
}

int64_t upper_row_tiles(int rows, int groups) {
  return (int64_t)rows / kBM + (groups < rows ? groups : rows);
}

// Launch one pipelined instantiation (persistent grid, dynamic LDS ring).
template <int EPI, class C, int ROLE, bool BT>
hipError_t launch_pipe(GemmParams<bf16_t> p, int cu_count, hipStream_t s) {
  if (p.K % C::BK != 0) return launch_pipe<EPI, PipeCfg<128, 128, 64, 2>, ROLE, BT>(p, cu_count, s);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&grouped_gemm_bf16_pipe<EPI, C, ROLE, BT>),
      hipFuncAttributeMaxDynamicSharedMemorySize, C::kLds);
  if (attr != hipSuccess) return attr;
  const int out_cols = paired(EPI) ? C::BN / 2 : C::BN;
  p.n_tiles = (p.N + out_cols - 1) / out_cols;
  const int64_t ub_m = (int64_t)p.rows / C::BM + (p.groups < p.rows ? p.groups : p.rows);
  const int grid = persistent_grid(ub_m * p.n_tiles, cu_count * C::kWgsPerCu);
  hipLaunchKernelGGL((grouped_gemm_bf16_pipe<EPI, C, ROLE, BT>), dim3(grid), dim3(C::NT), C::kLds, s, p);
  return hipGetLastError();
}

template <int EPI, int SAX, int ROLE, class C>
hipError_t launch_mx8_cfg(GemmParams<bf16_t> p, int cu_count, hipStream_t s) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&grouped_gemm_mx8<EPI, C, SAX, ROLE>), hipFuncAttributeMaxDynamicSharedMemorySize,
      C::kLds);
  if (attr != hipSuccess) return attr;
  const int out_cols = paired(EPI) ? C::BN / 2 : C::BN;
  p.n_tiles = (p.N + out_cols - 1) / out_cols;
  const int64_t ub_m = (int64_t)p.rows / C::BM + (p.groups < p.rows ? p.groups : p.rows);
  const int grid = persistent_grid(ub_m * p.n_tiles, cu_count * C::kWgsPerCu);
  hipLaunchKernelGGL((grouped_gemm_mx8<EPI, C, SAX, ROLE>), dim3(grid), dim3(C::NT), C::kLds, s, p);
  return hipGetLastError();
}

// Groups of at most 32 rows on average (decode) take the 32-row tile; larger
// ones a 128-row tile, which converts each weight fragment once per 128 rows.
inline bool mx_decode_shape(const GemmParams<bf16_t>& p) {
  const int64_t active = p.groups < p.rows ? p.groups : p.rows;
  return (int64_t)p.rows / (active > 0 ? active : 1) <= 32;
}

template <int EPI, int SAX, int ROLE>
hipError_t launch_mx8(GemmParams<bf16_t> p, int cu_count, hipStream_t s) {
  if (!mx_decode_shape(p)) return launch_mx8_cfg<EPI, SAX, ROLE, MxCfgPrefill>(p, cu_count, s);
  return launch_mx8_cfg<EPI, SAX, ROLE, MxCfgDecode>(p, cu_count, s);
}

template <int EPI_R, int EPI_S, int SAX, class C>
hipError_t launch_mx8_fused_cfg(GemmParams<bf16_t> pr, GemmParams<bf16_t> ps, int cu_count, hipStream_t s) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&grouped_gemm_mx8_fused<EPI_R, EPI_S, C, SAX>),
      hipFuncAttributeMaxDynamicSharedMemorySize, C::kLds);
  if (attr != hipSuccess) return attr;
  const int out_r = paired(EPI_R) ? C::BN / 2 : C::BN;
  const int out_s = paired(EPI_S) ? C::BN / 2 : C::BN;
  pr.n_tiles = (pr.N + out_r - 1) / out_r;
  ps.n_tiles = (ps.N + out_s - 1) / out_s;
  const int64_t ub_r = ((int64_t)pr.rows / C::BM + (pr.groups < pr.rows ? pr.groups : pr.rows)) * pr.n_tiles;
  const int64_t tiles_s = (int64_t)((ps.rows + C::BM - 1) / C::BM) * ps.n_tiles;
  const int grid = persistent_grid(ub_r + tiles_s, cu_count * C::kWgsPerCu);
  hipLaunchKernelGGL((grouped_gemm_mx8_fused<EPI_R, EPI_S, C, SAX>), dim3(grid), dim3(C::NT), C::kLds, s, pr, ps);
  return hipGetLastError();
}

template <int EPI_R, int EPI_S, int SAX>
hipError_t launch_mx8_fused(GemmParams<bf16_t> pr, GemmParams<bf16_t> ps, int cu_count, hipStream_t s) {
  if (!(mx_decode_shape(pr) && ps.rows <= 64))
    return launch_mx8_fused_cfg<EPI_R, EPI_S, SAX, MxCfgPrefill>(pr, ps, cu_count, s);
  return launch_mx8_fused_cfg<EPI_R, EPI_S, SAX, MxCfgDecode>(pr, ps, cu_count, s);
}

// The pipelined configurations (BM, BN, BK, STAGES, WM, WN, KW) the selection
// below can return.
typedef PipeCfg<128, 128, 64, 2> CfgSmall;          // 4 waves; narrow dense outputs, backward dgrad
typedef PipeCfg<256, 256, 64, 2, 2, 4> CfgDense;    // 8 waves (2 x 4, 128 x 64 each), one workgroup per CU
typedef PipeCfg<128, 256, 32, 2, 2, 4> CfgMid;      // 8 waves, 48 KiB ring: two workgroups per CU
typedef PipeCfg<128, 512, 32, 3, 1, 8> CfgWide;     // 8 waves (1 x 8, 128 x 64 each), 120 KiB 3-stage ring
typedef PipeCfg<32, 128, 64, 4, 1, 2, 2> CfgDecode; // 4 waves (2 column positions x 2 split-K waves)
typedef PipeCfg<32, 64, 64, 4, 1, 1, 2> CfgDecodeNarrow;  // 2 waves (split-K), two workgroups per CU

// Calls f(Cfg{}) for a pipelined configuration.
template <class F>
hipError_t with_cfg(int v, F&& f) {
  switch (v) {
    case MOE_TILE_256x256: return f(CfgDense{});
    case MOE_TILE_128x256: return f(CfgMid{});
    case MOE_TILE_128x512: return f(CfgWide{});
    case MOE_TILE_32x128: return f(CfgDecode{});
    case MOE_TILE_32x64: return f(CfgDecodeNarrow{});
    default: return f(CfgSmall{});
  }
}

// Configuration for a problem, from the host-known sizes only (measured on
// MI355X across the Scout-, Qwen2-, DeepSeek-V2-Lite- and DeepSeek-V3-shaped
// layers):
//  * groups that average 512 rows or more (the shared expert, dense prefill)
//    take the 256x256 tile with 8 waves, which halves the L2->LDS traffic per
//    MFMA and keeps two waves per SIMD.
//    That tile gives way to the 128x128 one when its tiles would fill the
//    CUs' workgroup slots much less evenly (a narrow output with few row
//    tiles: 128 tiles of 256x256 leave half the CUs idle, where 512 tiles of
//    128x128 fill both slots of every CU; 158 us against 118 us for the
//    Qwen2-shaped shared fc2);
//  * groups of at most 32 rows (decode) take a 32-row tile whose waves split
//    the reduction, so that many more tiles, each with several weight slices
//    in flight, stream the expert weights;
//  * everything else (skewed routing, many mid-sized groups) takes 128-row
//    tiles, which waste fewer MFMA rows on partial tiles: a 128x256 tile with
//    8 waves and 32-deep slices (half the activation or weight re-reads of a
//    128-column tile; its 48 KiB ring leaves room for two workgroups per CU,
//    5-9% faster than 64-deep slices at one per CU for fc1, 4-11% faster than
//    the 128x128 tile for fc2).  Deeper rings (3-8 slices in flight at one
//    workgroup per CU) measured 3-15% slower on every prefill shape.
int64_t rows_per_active_group(const GemmParams<bf16_t>& p) {
  const int64_t active = p.groups < p.rows ? p.groups : p.rows;  // at most one group per row
  return (int64_t)p.rows / (active > 0 ? active : 1);
}

// Share of the workgroup slots (slots = CUs x workgroups per CU) that the
// tiles of a configuration keep busy over all its waves of tiles, for groups
// of equal size.
template <int EPI, class C>
double slot_fill(const GemmParams<bf16_t>& p, int cu_count) {
  const int64_t groups = p.groups > 0 ? p.groups : 1;
  const int64_t per_group = (p.rows + groups - 1) / groups;
  const int out_cols = paired(EPI) ? C::BN / 2 : C::BN;
  const int64_t tiles = groups * ((per_group + C::BM - 1) / C::BM) * ((p.N + out_cols - 1) / out_cols);
  const int64_t slots = (int64_t)cu_count * C::kWgsPerCu;
  const int64_t waves = (tiles + slots - 1) / slots;
  return waves > 0 ? (double)tiles / (double)(waves * slots) : 1.0;
}

constexpr int64_t kDecodeRows = 32;
// Groups of at most this many rows on average stream their weights (fewer rows
// than the ~312 FLOP per weight byte at which 2.5 PFLOP/s meets 8 TB/s) and take
// the wide tile: measured on MI355X it wins at 128 rows per group (the Scout-
// and DeepSeek-V3-shaped layers: routed fc1 0.69 -> 0.59 ms and 3.37 -> 2.85 ms)
// and loses to the mid-size tile at 273 (Qwen2-shaped: 0.29 vs 0.42 ms).
constexpr int64_t kWideRows = 192;

// Decode sizes whose 32 x 128 tiles (routed, plus the shared expert's in a
// fused launch) would leave CUs idle take the 32 x 64 tile, which doubles the
// tiles streaming the weights: measured on MI355X, the DeepSeek-V2-Lite-shaped
// fc2 at one token (112 tiles of 32 x 128 for 256 CUs) 26.1 -> 20.5 us.  Not
// for fc1: its paired gate/up columns would be fetched in 64-byte pieces
// (24.9 -> 35 us measured), and not once the 32 x 128 tiles fill the CUs
// (T = 64: 3-5% slower).
bool decode_narrow(bool paired_epi, const GemmParams<bf16_t>& p, int shared_rows, int shared_n, int cu_count) {
  if (paired_epi) return false;
  const int64_t active = p.groups < p.rows ? p.groups : p.rows;
  int64_t tiles = active * ((p.N + 127) / 128);
  if (shared_rows > 0) tiles += (int64_t)((shared_rows + 31) / 32) * ((shared_n + 127) / 128);
  return tiles < cu_count;
}

template <int EPI, int ROLE>
int pick_pipe_variant(const GemmParams<bf16_t>& p, int cu_count) {
  if (rows_per_active_group(p) <= kDecodeRows && p.K % 128 == 0)
    return decode_narrow(paired(EPI), p, 0, 0, cu_count) ? MOE_TILE_32x64 : MOE_TILE_32x128;
  const int64_t rows_per_group = (int64_t)p.rows / (p.groups > 0 ? p.groups : 1);
  if (rows_per_group >= 512)
    return slot_fill<EPI, CfgDense>(p, cu_count) + 0.25 < slot_fill<EPI, CfgSmall>(p, cu_count) ? MOE_TILE_128x128
                                                                                               : MOE_TILE_256x256;
  if (ROLE == 2) return MOE_TILE_128x128;
  return rows_per_active_group(p) <= kWideRows ? MOE_TILE_128x512 : MOE_TILE_128x256;
}

template <int EPI_R, int EPI_S, class CR, class CS, bool BT>
hipError_t launch_fused(GemmParams<bf16_t> pr, GemmParams<bf16_t> ps, int cu_count, hipStream_t s) {
  if (pr.K % CR::BK != 0 || ps.K % CS::BK != 0)
    return launch_fused<EPI_R, EPI_S, CfgSmall, CfgSmall, BT>(pr, ps, cu_count, s);
  constexpr int lds = fused_lds<CR, CS>();
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&grouped_gemm_bf16_fused<EPI_R, EPI_S, CR, CS, BT>),
      hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  const int out_r = paired(EPI_R) ? CR::BN / 2 : CR::BN;
  const int out_s = paired(EPI_S) ? CS::BN / 2 : CS::BN;
  pr.n_tiles = (pr.N + out_r - 1) / out_r;
  ps.n_tiles = (ps.N + out_s - 1) / out_s;
  const int64_t ub_r = ((int64_t)pr.rows / CR::BM + (pr.groups < pr.rows ? pr.groups : pr.rows)) * pr.n_tiles;
  const int64_t tiles_s = (int64_t)((ps.rows + CS::BM - 1) / CS::BM) * ps.n_tiles;
  const int grid = persistent_grid(ub_r + tiles_s, cu_count * fused_wgs<CR, CS>());
  hipLaunchKernelGGL((grouped_gemm_bf16_fused<EPI_R, EPI_S, CR, CS, BT>), dim3(grid), dim3(CR::NT), lds, s, pr, ps);
  return hipGetLastError();
}

constexpr int kFusedDenseSharedRows = 512;

int pick_fused_variant(const GemmParams<bf16_t>& pr, const GemmParams<bf16_t>& ps, bool paired_epi, int cu_count) {
  const int64_t per_group = (int64_t)pr.rows / (pr.groups > 0 ? pr.groups : 1);
  if (per_group >= 512 && ps.rows >= 512) return MOE_TILE_256x256;
  if (rows_per_active_group(pr) <= kDecodeRows && ps.rows <= 2 * kDecodeRows && pr.K % 128 == 0 && ps.K % 128 == 0)
    return decode_narrow(paired_epi, pr, ps.rows, ps.N, cu_count) ? MOE_TILE_32x64 : MOE_TILE_32x128;
  return rows_per_active_group(pr) <= kWideRows ? MOE_TILE_128x512 : MOE_TILE_128x256;
}

template <int EPI_R, int EPI_S>
hipError_t launch_fused_bf16(const GemmParams<bf16_t>& pr, const GemmParams<bf16_t>& ps, int cu_count,
                             hipStream_t s) {
  const int v = pick_fused_variant(pr, ps, paired(EPI_R), cu_count);
  // The weight-streaming routed tile runs the shared expert's fc2 with the
  // dense tile when the shared expert has rows enough to fill it.  Its fc1
  // (SwiGLU) keeps the weight-streaming tile for both: measured on MI355X,
  // Scout-shaped fc1 0.886 -> 0.853 ms and DeepSeek-V3-shaped 3.00 -> 2.99 ms
  // against the dense shared tile (fc2 within 1% either way).  Each wave
  // holds a 128 x 64 tile in both configurations.
  if (v == MOE_TILE_128x512 && ps.rows >= kFusedDenseSharedRows && !paired(EPI_R)) {
    if (pr.bt) return launch_fused<EPI_R, EPI_S, CfgWide, CfgDense, true>(pr, ps, cu_count, s);
    return launch_fused<EPI_R, EPI_S, CfgWide, CfgDense, false>(pr, ps, cu_count, s);
  }
  if (pr.bt)
    return with_cfg(v, [&](auto c) {
      return launch_fused<EPI_R, EPI_S, decltype(c), decltype(c), true>(pr, ps, cu_count, s);
    });
  return with_cfg(v, [&](auto c) {
    return launch_fused<EPI_R, EPI_S, decltype(c), decltype(c), false>(pr, ps, cu_count, s);
  });
}

template <int EPI, int ROLE>
hipError_t launch_bf16(GemmParams<bf16_t> p, int cu_count, hipStream_t s) {
  if (p.K % 64 == 0) {
    if (p.bt)
      return with_cfg(pick_pipe_variant<EPI, ROLE>(p, cu_count),
                      [&](auto c) { return launch_pipe<EPI, decltype(c), ROLE, true>(p, cu_count, s); });
    return with_cfg(pick_pipe_variant<EPI, ROLE>(p, cu_count),
                    [&](auto c) { return launch_pipe<EPI, decltype(c), ROLE, false>(p, cu_count, s); });
  }
  p.n_tiles = paired(EPI) ? (p.N + 63) / 64 : (p.N + 127) / 128;
  const int grid = persistent_grid(upper_row_tiles(p.rows, p.groups) * p.n_tiles, 2 * cu_count);
  hipLaunchKernelGGL((grouped_gemm_bf16_generic<EPI, ROLE>), dim3(grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace
}  // namespace moe

namespace moe_launch {

// Weights of one group: bt == 0: [K, 2I] (fc1) / [K, N] (fc2), N contiguous;
// bt == 1: [2I, K] / [N, K], K contiguous.  fc1's up half starts at column
// (bt == 0) or row (bt == 1) I.
hipError_t grouped_swiglu_fc1(int dt, int bt, const void* a, const int32_t* offsets, int groups, int rows,
                              const void* w1, int64_t w1_group_stride, int K, int I, void* act, int role,
                              int cu_count, hipStream_t s, const int32_t* a_rows, int a_src_rows) {
  using namespace moe;
  const int ldb = bt ? K : 2 * I;
  if (dt == 1) {
    GemmParams<bf16_t> p{(const bf16_t*)a, offsets, groups, rows, K, I, (const bf16_t*)w1, w1_group_stride,
                         ldb, I, act, nullptr, 0, 0, bt};
    p.a_rows = a_rows;
    p.a_src_rows = a_src_rows;
    return role ? launch_bf16<kSwiGLU, 1>(p, cu_count, s) : launch_bf16<kSwiGLU, 0>(p, cu_count, s);
  }
  GemmParams<float> p{(const float*)a, offsets, groups, rows, K, I, (const float*)w1, w1_group_stride,
                      ldb, I, act, nullptr, 0, 0, bt};
  p.a_rows = a_rows;
  p.a_src_rows = a_src_rows;
  const int64_t n = (int64_t)rows * I;
  hipLaunchKernelGGL(grouped_gemm_f32<kSwiGLU>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t grouped_fc2(int dt, int bt, const void* act, const int32_t* offsets, int groups, int rows,
                       const void* w2, int64_t w2_group_stride, int K, int N, float* out, const float* row_scale,
                       int accumulate, int plain_store, int role, int cu_count, hipStream_t s) {
  using namespace moe;
  const int ldb = bt ? K : N;
  if (dt == 1) {
    GemmParams<bf16_t> p{(const bf16_t*)act, offsets, groups, rows, K, N, (const bf16_t*)w2, w2_group_stride,
                         ldb, 0, out, row_scale, accumulate, 0, bt};
    if (plain_store) return role ? launch_bf16<kStoreF32, 1>(p, cu_count, s) : launch_bf16<kStoreF32, 0>(p, cu_count, s);
    return role ? launch_bf16<kScaleAdd, 1>(p, cu_count, s) : launch_bf16<kScaleAdd, 0>(p, cu_count, s);
  }
  GemmParams<float> p{(const float*)act, offsets, groups, rows, K, N, (const float*)w2, w2_group_stride,
                      ldb, 0, out, row_scale, accumulate, 0, bt};
  const int64_t n = (int64_t)rows * N;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (plain_store)
    hipLaunchKernelGGL(grouped_gemm_f32<kStoreF32>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(grouped_gemm_f32<kScaleAdd>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

// One launch for both problems pays off when the shared expert's MFMA work is
// small next to the routed weight stream (decode, many large experts), or when
// the routed groups stream their weights through the wide tile while the
// shared expert takes the dense one: its tiles then fill the gaps of the
// weight-bound routed tiles.  With mid-size or dense routed groups a large
// shared expert runs faster in a launch of its own (measured on MI355X:
// Qwen2-shaped fc2 0.30 ms in two launches against 0.36 ms in one).
bool fused_supported(int dt, int H, int I, int I_s, int E, int R, int T) {
  using namespace moe;
  if (!(dt == 1 && H % 64 == 0 && I % 64 == 0 && I_s % 64 == 0)) return false;
  // Weight-streaming routed groups (the wide tile) leave the MFMAs idle most of
  // the time; the shared expert's dense tiles fill them in the same launch
  // (Scout-shaped layer: fc1 0.93 -> 0.91 ms, fc2 0.57 -> 0.52 ms).
  const int64_t active = E < R ? E : R;
  if ((int64_t)R / (active > 0 ? active : 1) <= kWideRows && R / (active > 0 ? active : 1) > kDecodeRows) return true;
  const double routed_bytes = (double)active * 3.0 * H * I * 2.0;
  const double shared_flops = 6.0 * T * H * I_s;
  return shared_flops < 50.0 * routed_bytes;
}

int tile_config(int dt, int call, int R, int H, int E, int I, int T, int I_s, int cu_count) {
  using namespace moe;
  if (dt != 1) return MOE_TILE_F32;
  GemmParams<bf16_t> p{};
  p.rows = R;
  p.groups = E;
  p.K = call == 0 ? H : I;
  p.N = call == 0 ? I : H;
  if (I_s > 0 && fused_supported(dt, H, I, I_s, E, R, T)) {
    GemmParams<bf16_t> ps{};
    ps.rows = T;
    ps.groups = 1;
    ps.K = call == 0 ? H : I_s;
    ps.N = call == 0 ? I_s : H;
    return pick_fused_variant(p, ps, call == 0, cu_count);
  }
  if (p.K % 64 != 0) return MOE_TILE_GENERIC;
  return call == 0 ? pick_pipe_variant<kSwiGLU, 0>(p, cu_count) : pick_pipe_variant<kStoreF32, 0>(p, cu_count);
}

hipError_t fused_fc1(int bt, const void* xs, const int32_t* offsets, int E, int R, const void* w1, int H, int I,
                     void* act, const void* x, int T, const void* ws1, int I_s, void* act_s, int cu_count,
                     hipStream_t s, const int32_t* a_rows) {
  using namespace moe;
  GemmParams<bf16_t> pr{(const bf16_t*)xs, offsets, E, R, H, I, (const bf16_t*)w1, (int64_t)H * 2 * I,
                        bt ? H : 2 * I, I, act, nullptr, 0, 0, bt};
  pr.a_rows = a_rows;  // with a_rows set, xs is x and routed row r is x[a_rows[r]]
  pr.a_src_rows = T;
  GemmParams<bf16_t> ps{(const bf16_t*)x, nullptr, 1, T, H, I_s, (const bf16_t*)ws1, 0,
                        bt ? H : 2 * I_s, I_s, act_s, nullptr, 0, 0, bt};
  return launch_fused_bf16<kSwiGLU, kSwiGLU>(pr, ps, cu_count, s);
}

hipError_t fused_fc2(int bt, const void* act, const int32_t* offsets, int E, int R, const void* w2, int I, int H,
                     float* y_rows, const void* act_s, int T, const void* ws2, int I_s, const float* gate,
                     int accumulate, float* y, int cu_count, hipStream_t s) {
  using namespace moe;
  GemmParams<bf16_t> pr{(const bf16_t*)act, offsets, E, R, I, H, (const bf16_t*)w2, (int64_t)I * H,
                        bt ? I : H, 0, y_rows, nullptr, 0, 0, bt};
  GemmParams<bf16_t> ps{(const bf16_t*)act_s, nullptr, 1, T, I_s, H, (const bf16_t*)ws2, 0,
                        bt ? I_s : H, 0, y, gate, accumulate, 0, bt};
  return launch_fused_bf16<kStoreF32, kScaleAdd>(pr, ps, cu_count, s);
}

// MXFP8 weights (codes [N, K] bytes per group, scales as described above),
// bf16 activations; K must be a multiple of 128.
hipError_t grouped_swiglu_fc1_mx8(const void* a, const int32_t* offsets, int groups, int rows, const void* w1q,
                                  const void* w1s, int K, int I, void* act, int role, int cu_count, hipStream_t s) {
  using namespace moe;
  GemmParams<bf16_t> p{(const bf16_t*)a, offsets, groups, rows, K, I, (const bf16_t*)w1q, (int64_t)2 * I * K,
                       K, I, act, nullptr, 0, 0, 1, (const uint8_t*)w1s, (int64_t)2 * I / 8 * K};
  return role ? launch_mx8<kSwiGLU, kScaleN, 1>(p, cu_count, s) : launch_mx8<kSwiGLU, kScaleN, 0>(p, cu_count, s);
}

hipError_t grouped_fc2_mx8(const void* act, const int32_t* offsets, int groups, int rows, const void* w2q,
                           const void* w2s, int K, int N, float* out, const float* row_scale, int accumulate,
                           int plain_store, int role, int cu_count, hipStream_t s) {
  using namespace moe;
  GemmParams<bf16_t> p{(const bf16_t*)act, offsets, groups, rows, K, N, (const bf16_t*)w2q, (int64_t)N * K,
                       K, 0, out, row_scale, accumulate, 0, 1, (const uint8_t*)w2s, (int64_t)N * (K / 8)};
  if (plain_store)
    return role ? launch_mx8<kStoreF32, kScaleK, 1>(p, cu_count, s) : launch_mx8<kStoreF32, kScaleK, 0>(p, cu_count, s);
  return role ? launch_mx8<kScaleAdd, kScaleK, 1>(p, cu_count, s) : launch_mx8<kScaleAdd, kScaleK, 0>(p, cu_count, s);
}

hipError_t fused_fc1_mx8(const void* xs, const int32_t* offsets, int E, int R, const void* w1q, const void* w1s,
                         int H, int I, void* act, const void* x, int T, const void* ws1q, const void* ws1s, int I_s,
                         void* act_s, int cu_count, hipStream_t s) {
  using namespace moe;
  GemmParams<bf16_t> pr{(const bf16_t*)xs, offsets, E, R, H, I, (const bf16_t*)w1q, (int64_t)2 * I * H,
                        H, I, act, nullptr, 0, 0, 1, (const uint8_t*)w1s, (int64_t)2 * I / 8 * H};
  GemmParams<bf16_t> ps{(const bf16_t*)x, nullptr, 1, T, H, I_s, (const bf16_t*)ws1q, 0,
                        H, I_s, act_s, nullptr, 0, 0, 1, (const uint8_t*)ws1s, 0};
  return launch_mx8_fused<kSwiGLU, kSwiGLU, kScaleN>(pr, ps, cu_count, s);
}

hipError_t fused_fc2_mx8(const void* act, const int32_t* offsets, int E, int R, const void* w2q, const void* w2s,
                         int I, int H, float* y_rows, const void* act_s, int T, const void* ws2q, const void* ws2s,
                         int I_s, const float* gate, int accumulate, float* y, int cu_count, hipStream_t s) {
  using namespace moe;
  GemmParams<bf16_t> pr{(const bf16_t*)act, offsets, E, R, I, H, (const bf16_t*)w2q, (int64_t)H * I,
                        I, 0, y_rows, nullptr, 0, 0, 1, (const uint8_t*)w2s, (int64_t)H * (I / 8)};
  GemmParams<bf16_t> ps{(const bf16_t*)act_s, nullptr, 1, T, I_s, H, (const bf16_t*)ws2q, 0,
                        I_s, 0, y, gate, accumulate, 0, 1, (const uint8_t*)ws2s, 0};
  return launch_mx8_fused<kStoreF32, kScaleAdd, kScaleK>(pr, ps, cu_count, s);
}

// Training forward of fc1: the SwiGLU output plus the pre-activation
// h_pre [rows, 2I] (gate columns, then up columns) in the element type.
hipError_t grouped_swiglu_fc1_save(int dt, int bt, const void* a, const int32_t* offsets, int groups, int rows,
                                   const void* w1, int64_t w1_group_stride, int K, int I, void* act, void* h_pre,
                                   int cu_count, hipStream_t s) {
  using namespace moe;
  const int ldb = bt ? K : 2 * I;
  if (dt == 1) {
    GemmParams<bf16_t> p{(const bf16_t*)a, offsets, groups, rows, K, I, (const bf16_t*)w1, w1_group_stride,
                         ldb, I, act, nullptr, 0, 0, bt};
    p.out2 = h_pre;
    return launch_bf16<kSwiGLUSave, 0>(p, cu_count, s);
  }
  GemmParams<float> p{(const float*)a, offsets, groups, rows, K, I, (const float*)w1, w1_group_stride,
                      ldb, I, act, nullptr, 0, 0, bt};
  p.out2 = h_pre;
  const int64_t n = (int64_t)rows * I;
  hipLaunchKernelGGL(grouped_gemm_f32<kSwiGLUSave>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

// Input gradient through fc2 and SwiGLU: d_h = SwiGLU'(h_pre) * (d_rows W2^T),
// d_rows [rows, H], W2 per group [I, H] (wt_nk == 0) or [H, I] (wt_nk == 1).
hipError_t grouped_fc2_dgrad_swiglu(int dt, int wt_nk, const void* d_rows, const int32_t* offsets, int groups,
                                    int rows, const void* w2, int I, int H, const void* h_pre, void* d_h,
                                    int cu_count, hipStream_t s) {
  using namespace moe;
  // As a GEMM with reduction H and I output columns, W2 [I, H] is the [N, K]
  // layout and W2 [H, I] the [K, N] layout.
  const int bt = wt_nk ? 0 : 1;
  const int ldb = bt ? H : I;
  if (dt == 1) {
    GemmParams<bf16_t> p{(const bf16_t*)d_rows, offsets, groups, rows, H, I, (const bf16_t*)w2, (int64_t)I * H,
                         ldb, 0, d_h, nullptr, 0, 0, bt};
    p.aux = h_pre;
    return launch_bf16<kSwiGLUBwd, 2>(p, cu_count, s);
  }
  GemmParams<float> p{(const float*)d_rows, offsets, groups, rows, H, I, (const float*)w2, (int64_t)I * H,
                      ldb, 0, d_h, nullptr, 0, 0, bt};
  p.aux = h_pre;
  const int64_t n = (int64_t)rows * I;
  hipLaunchKernelGGL(grouped_gemm_f32<kSwiGLUBwd>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

// Input gradient through fc1: d_xs [rows, H] (float32) = d_h W1^T, d_h
// [rows, 2I], W1 per group [H, 2I] (wt_nk == 0) or [2I, H] (wt_nk == 1).
hipError_t grouped_fc1_dgrad(int dt, int wt_nk, const void* d_h, const int32_t* offsets, int groups, int rows,
                             const void* w1, int H, int I, float* d_xs, int cu_count, hipStream_t s) {
  using namespace moe;
  const int bt = wt_nk ? 0 : 1;
  const int ldb = bt ? 2 * I : H;
  if (dt == 1) {
    GemmParams<bf16_t> p{(const bf16_t*)d_h, offsets, groups, rows, 2 * I, H, (const bf16_t*)w1,
                         (int64_t)2 * I * H, ldb, 0, d_xs, nullptr, 0, 0, bt};
    return launch_bf16<kStoreF32, 2>(p, cu_count, s);
  }
  GemmParams<float> p{(const float*)d_h, offsets, groups, rows, 2 * I, H, (const float*)w1, (int64_t)2 * I * H,
                      ldb, 0, d_xs, nullptr, 0, 0, bt};
  const int64_t n = (int64_t)rows * H;
  hipLaunchKernelGGL(grouped_gemm_f32<kStoreF32>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t grouped_wgrad(int dt, const void* P, const void* Q, const int32_t* offsets, int groups, int rows, int M,
                         int N, void* out, int role, int cu_count, hipStream_t s) {
  using namespace moe;
  if (dt == 1) {
    typedef WgCfgUsed C;
    auto kern = role == 1 ? &grouped_wgrad_bf16<C, 1> : &grouped_wgrad_bf16<C, 2>;
    static const hipError_t attr1 = hipFuncSetAttribute(reinterpret_cast<const void*>(&grouped_wgrad_bf16<C, 1>),
                                                        hipFuncAttributeMaxDynamicSharedMemorySize, C::kLds);
    static const hipError_t attr2 = hipFuncSetAttribute(reinterpret_cast<const void*>(&grouped_wgrad_bf16<C, 2>),
                                                        hipFuncAttributeMaxDynamicSharedMemorySize, C::kLds);
    if (attr1 != hipSuccess) return attr1;
    if (attr2 != hipSuccess) return attr2;
    WgParams p{(const bf16_t*)P, (const bf16_t*)Q, offsets, groups, rows, M, N, (bf16_t*)out,
               (M + C::BM - 1) / C::BM, (N + C::BN - 1) / C::BN};
    const int64_t tiles = (int64_t)p.m_tiles * p.n_tiles * groups;
    const int grid = persistent_grid(tiles, cu_count * C::kWgsPerCu);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(C::NT), C::kLds, s, p);
    return hipGetLastError();
  }
  const int64_t n = (int64_t)groups * M * N;
  hipLaunchKernelGGL(grouped_wgrad_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (const float*)P,
                     (const float*)Q, offsets, groups, rows, M, N, (float*)out);
  return hipGetLastError();
}

}  // namespace moe_launch
