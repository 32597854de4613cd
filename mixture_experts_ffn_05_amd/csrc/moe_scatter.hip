// Expert-grouped row layout (scatter build).
//
// VeOmni docs "Fused MoE Kernel Notes", section "Scatter/gather layout": the
// routed pairs of [T, H] tokens expand to [T*k, H] rows grouped by expert, and
// scatter_index maps each (token, slot) pair to its row.  Section "Duplicate
// top-k routes": one token may send several slots to one expert, so a group can
// hold more than T rows -- nothing below assumes a bound of T.
//
// The layout is a stable counting sort of the pairs p = t*k + j by expert id.
// It is deterministic: the only atomics are integer count increments, whose
// result does not depend on their order, and every row comes from a fixed scan.
//   scatter_count  each wave64 takes a chunk of 1024 consecutive pairs and counts
//                  them per expert with LDS atomic adds.
//   scatter_scan   one workgroup: per expert, an exclusive scan of the chunk
//                  counts (chunk bases); across experts, an exclusive scan of the
//                  totals (expert_offsets), the largest group and the number of
//                  out-of-range ids.
//   scatter_rank   one workgroup per chunk, one quarter of it per wave; a pair's
//                  row is offsets[e] plus its chunk's base, the counts of the
//                  earlier quarters and the number of earlier pairs of the
//                  quarter with the same expert, kept as a running per-expert
//                  cursor in LDS.  Lanes holding the same expert are found with
//                  ceil(log2 E) ballots, for all rounds of the quarter at once so
//                  that they overlap.
//   scatter_copy   x_scattered[r] = x[row_token[r]], 16-byte vector copies (skipped when
//                  x_scattered is NULL: the fc1 call then gathers the rows on load).
// Up to 4 chunks (decode, and prefill up to 4096 pairs) take scatter_small,
// which runs count, scan and rank in one workgroup of 4 waves (the pairs split
// evenly between them), and for at most 256 rows of at most 256 KiB in all
// also the row copy.
#include "moe_common.h"
#include "moe_topk.h"

#include <type_traits>

namespace moe {
namespace {

constexpr int kChunk = 1024;              // pairs per wave
constexpr int kIters = kChunk / kWave;    // ballot rounds per chunk
constexpr int kWavesPerBlock = 4;

// Lanes (bitmask) whose expert id equals the calling lane's, for each of N
// rounds of pairs p0 + it * 64 + lane; 0 for lanes whose pair is at or past end, or whose
// id is outside [0, E).  All lanes of the wave must call it.  The bit loop is
// outermost, so the ballots of the N rounds do not depend on each other and
// overlap instead of forming one long chain per round.
template <int N>
__device__ __forceinline__ void round_masks(const int (&ev)[N], int64_t p0, int end, int E, int nbits, int lane,
                                            uint64_t (&m)[N]) {
  const int64_t live = end - p0;  // rounds from live / 64 on hold no pair and are skipped
  bool in_range[N];
#pragma unroll
  for (int it = 0; it < N; ++it) {
    in_range[it] = it * kWave + lane < live && ev[it] >= 0 && ev[it] < E;
    m[it] = it * kWave < live ? __ballot(in_range[it]) : 0ull;
  }
  for (int b = 0; b < nbits; ++b) {
#pragma unroll
    for (int it = 0; it < N; ++it) {
      if (it * kWave < live) {  // wave-uniform
        const bool bit = (ev[it] >> b) & 1;
        const uint64_t on = __ballot(in_range[it] && bit);
        m[it] &= bit ? on : ~on;
      }
    }
  }
#pragma unroll
  for (int it = 0; it < N; ++it)
    if (!in_range[it]) m[it] = 0ull;
}

// The expert ids of N rounds of pairs p0 + it * 64 + lane below end (-1 from
// end on), all loads issued before any is used.
template <int N>
__device__ __forceinline__ void load_rounds(const int32_t* ids, int end, int64_t p0, int lane, int (&ev)[N]) {
#pragma unroll
  for (int it = 0; it < N; ++it) {
    const int64_t p = p0 + it * kWave + lane;
    ev[it] = p < end ? ids[p] : -1;
  }
}

// Rows of N rounds of pairs p0 + it * 64 + lane below end: a pair's row is the running
// cursor of its expert plus the number of lower lanes with the same expert; the
// highest such lane advances the cursor.
template <int N>
__device__ __forceinline__ void rank_rounds(const int (&ev)[N], int64_t p0, int end, int E, int k, int nbits, int lane,
                                            int32_t* cursor, int32_t* __restrict__ scatter_index,
                                            int32_t* __restrict__ row_token, int32_t* lds_row_token = nullptr) {
  uint64_t m[N];
  round_masks<N>(ev, p0, end, E, nbits, lane, m);
  const uint64_t above = lane == 63 ? 0ull : (~0ull << (lane + 1));
  const uint64_t below = lanemask_lt();
#pragma unroll
  for (int it = 0; it < N; ++it) {
    if (p0 + it * kWave >= end) break;  // the remaining rounds are past end
    const int64_t p = p0 + it * kWave + lane;
    const int e = ev[it];
    const bool in_range = m[it] != 0ull;  // a lane in range always finds itself
    int r = -1;
    if (in_range) {
      const int b = cursor[e];
      r = b + __popcll(m[it] & below);
      if ((m[it] & above) == 0ull) cursor[e] = b + __popcll(m[it]);
    }
    if (p < end) scatter_index[p] = r;
    if (in_range) {
      row_token[r] = (int)(p / k);
      if (lds_row_token) lds_row_token[r] = (int)(p / k);
    }
  }
}

// Compact forms for the one-workgroup path.  It runs once per call, with cold
// instruction caches, so its loops are not unrolled: one iteration per 64-pair
// round, the id reloaded each round (ids may be in global memory or LDS).
//
// Lanes (bitmask) whose expert id equals the calling lane's; 0 for a lane with
// in_range false.  All lanes of the wave must call it.
__device__ __forceinline__ uint64_t same_expert_lanes(int e, bool in_range, int nbits) {
  uint64_t m = __ballot(in_range);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t on = __ballot(in_range && bit);
    m &= bit ? on : ~on;
  }
  return in_range ? m : 0ull;
}

// Per-expert counts of the pairs [p0, end) into h (LDS atomic adds); returns how
// many of them have an id outside [0, E).
__device__ __forceinline__ int count_segment(const int32_t* ids, int64_t p0, int end, int E, int lane, int32_t* h) {
  int nbad = 0;
#pragma unroll 1
  for (int64_t q = p0; q < end; q += kWave) {
    const int64_t p = q + lane;
    const bool live = p < end;
    const int e = live ? ids[p] : -1;
    const bool in_range = live && e >= 0 && e < E;
    nbad += __popcll(__ballot(live && !in_range));
    if (in_range) atomicAdd(h + e, 1);
  }
  return nbad;
}

// Rows of the pairs [p0, end), in pair order from the per-expert cursors.
__device__ __forceinline__ void rank_segment(const int32_t* ids, int64_t p0, int end, int E, int k, int nbits,
                                             int lane, int32_t* cursor, int32_t* __restrict__ scatter_index,
                                             int32_t* __restrict__ row_token, int32_t* lds_row_token) {
  const uint64_t above = lane == 63 ? 0ull : (~0ull << (lane + 1));
  const uint64_t below = lanemask_lt();
#pragma unroll 1
  for (int64_t q = p0; q < end; q += kWave) {
    const int64_t p = q + lane;
    const bool live = p < end;
    const int e = live ? ids[p] : -1;
    const bool in_range = live && e >= 0 && e < E;
    const uint64_t m = same_expert_lanes(e, in_range, nbits);
    int r = -1;
    if (in_range) {
      const int b = cursor[e];
      r = b + __popcll(m & below);
      if ((m & above) == 0ull) cursor[e] = b + __popcll(m);
    }
    if (live) scatter_index[p] = r;
    if (in_range) {
      row_token[r] = (int)(p / k);
      if (lds_row_token) lds_row_token[r] = (int)(p / k);
    }
  }
}

// Per-expert counts of N rounds of pairs p0 + it * 64 + lane below end into the
// LDS histogram h; returns the number of those pairs whose id is outside [0, E).
template <int N>
__device__ __forceinline__ int count_rounds(const int (&ev)[N], int64_t p0, int end, int E, int lane, int32_t* h) {
  int nbad = 0;
#pragma unroll
  for (int it = 0; it < N; ++it) {
    if (p0 + it * kWave < end) {  // wave-uniform: rounds past end hold no pair
      const bool live = p0 + it * kWave + lane < end;
      const int e = ev[it];
      const bool in_range = live && e >= 0 && e < E;
      nbad += __popcll(__ballot(live && !in_range));
      if (in_range) atomicAdd(h + e, 1);
    }
  }
  return nbad;
}

__global__ __launch_bounds__(256) void scatter_count(const int32_t* __restrict__ ids, int R, int E, int nchunks, int32_t* __restrict__ cnt,
                                                     int32_t* __restrict__ bad) {
  extern __shared__ int32_t hist[];  // [4][E]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < kWavesPerBlock * E; i += 256) hist[i] = 0;
  __syncthreads();
  const int c = blockIdx.x * kWavesPerBlock + w;
  int nbad = 0;
  if (c < nchunks) {
    int ev[kIters];
    load_rounds<kIters>(ids, R, (int64_t)c * kChunk, lane, ev);
    nbad = count_rounds<kIters>(ev, (int64_t)c * kChunk, R, E, lane, hist + w * E);
  }
  __syncthreads();
  if (c < nchunks) {
    for (int e = lane; e < E; e += kWave) cnt[(int64_t)c * E + e] = hist[w * E + e];
    if (lane == 0) bad[c] = nbad;
  }
}

__global__ __launch_bounds__(1024) void scatter_scan(int32_t* __restrict__ cnt, const int32_t* __restrict__ bad,
                                                     int nchunks, int E, int R, int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ status, int32_t* __restrict__ row_token) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t wmax[16];
  __shared__ int32_t wbad[16];
  __shared__ int32_t s_total;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int total_e = 0;
  if (tid < E) {  // chunk bases of expert tid (each thread owns one column), 16 chunks' loads in flight at once
    constexpr int kBatch = 16;
    int run = 0;
    for (int c0 = 0; c0 < nchunks; c0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) v[u] = c0 + u < nchunks ? cnt[(int64_t)(c0 + u) * E + tid] : 0;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (c0 + u < nchunks) cnt[(int64_t)(c0 + u) * E + tid] = run;
        run += v[u];
      }
    }
    total_e = run;
  }
  int my_bad = 0;  // out-of-range ids, summed over the chunks by the whole workgroup
  for (int c = tid; c < nchunks; c += 1024) my_bad += bad[c];
  const int incl = wave_inclusive_scan(total_e);
  const int mx = wave_max(total_e);
  const int bad_w = wave_inclusive_scan(my_bad);
  if (lane == 63) {
    wsum[w] = incl;
    wbad[w] = bad_w;
  }
  if (lane == 0) wmax[w] = mx;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < w; ++i) base += wsum[i];
  if (tid < E) offsets[tid] = base + incl - total_e;
  if (tid == 0) {
    int total = 0, maxg = 0, nbad = 0;
    for (int i = 0; i < 16; ++i) {
      total += wsum[i];
      maxg = max(maxg, wmax[i]);
      nbad += wbad[i];
    }
    offsets[E] = total;
    status[0] = maxg;
    status[1] = nbad;
    s_total = total;
  }
  __syncthreads();
  for (int r = s_total + tid; r < R; r += 1024) row_token[r] = -1;
}

// Workgroup c ranks chunk c; wave w takes its quarter, pairs c * 1024 + 256 w
// onward.  The waves recount their quarters per expert (LDS atomics), and wave
// w's cursor for expert e starts at the chunk's base plus the counts of waves
// 0 .. w-1, so every pair gets the row a single pass over the chunk would give.
__global__ __launch_bounds__(256) void scatter_rank(const int32_t* __restrict__ ids, int R, int E, int k, int nbits,
                                                    int nchunks, const int32_t* __restrict__ chunk_base,
                                                    const int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ scatter_index,
                                                    int32_t* __restrict__ row_token) {
  constexpr int kQ = kIters / kWavesPerBlock;  // rounds per wave
  extern __shared__ int32_t cursor_all[];  // [4][E]: quarter counts, then cursors
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = blockIdx.x;
  for (int i = tid; i < kWavesPerBlock * E; i += 256) cursor_all[i] = 0;
  __syncthreads();
  const int64_t p0 = (int64_t)c * kChunk + (int64_t)w * kQ * kWave;
  int ev[kQ];
  load_rounds<kQ>(ids, R, p0, lane, ev);
  count_rounds<kQ>(ev, p0, R, E, lane, cursor_all + w * E);
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    int run = chunk_base[(int64_t)c * E + e] + offsets[e];
#pragma unroll
    for (int q = 0; q < kWavesPerBlock; ++q) {
      const int v = cursor_all[q * E + e];
      cursor_all[q * E + e] = run;
      run += v;
    }
  }
  __syncthreads();
  rank_rounds<kQ>(ev, p0, R, E, k, nbits, lane, cursor_all + w * E, scatter_index, row_token);
}

// The whole scatter build in one workgroup of NW waves: count, scan and rank in
// one launch.  The pairs are split into nseg contiguous segments of whole
// 64-pair rounds (at most 16 rounds each), one per wave, counted and then
// ranked with the compact loops above; segment w's cursor for expert e starts at
// offsets[e] plus the counts of segments 0 .. w-1, so the rows are those of one
// pass in pair order.  hist holds nseg x E counts, then cursors.  With fold set
// (at most kFoldRows rows), the same workgroup also copies the rows, reading
// row_token from LDS.
constexpr int kSmallWaves = 16;
constexpr int kFoldRows = 256;
constexpr int64_t kFoldBytes = 256 * 1024;
constexpr int kSmallHist = 8192;  // LDS counters of the one-workgroup path (32 KiB)

// Segments of the one-workgroup path for R pairs: one per wave, as many as kSmallHist holds, and no more
// than there are 64-pair rounds (each segment adds a step to the per-expert scan).
int block_segments(int NW, int E, int R) {
  int n = NW < kSmallHist / E ? NW : kSmallHist / E;
  const int rounds = (R + kWave - 1) / kWave;
  if (n > rounds) n = rounds;
  return n < 1 ? 1 : n;
}

struct BlockLds {
  int32_t* hist;        // [nseg][E]
  int32_t* wsum;        // [NW]
  int32_t* wmax;        // [NW]
  int32_t* wbad;        // [NW]
  int32_t* row_token;   // [kFoldRows]
};

// The scatter build of R <= nseg * 1024 pairs; ids may point to global memory or to LDS.
template <int NW>
__device__ __forceinline__ void scatter_block(const int32_t* ids, int R, int E, int k, int nbits, int nseg,
                                              int32_t* __restrict__ scatter_index, int32_t* __restrict__ row_token,
                                              int32_t* __restrict__ offsets, int32_t* __restrict__ status,
                                              int fold, const u32x4* __restrict__ x, int row_vecs,
                                              u32x4* __restrict__ xs, const BlockLds& L) {
  constexpr int NT = NW * kWave;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < nseg * E; i += NT) L.hist[i] = 0;
  __syncthreads();
  const int seg = ((R + nseg - 1) / nseg + kWave - 1) / kWave * kWave;  // pairs per segment, whole rounds
  const int64_t p0 = (int64_t)w * seg;
  const int pend = (int)min((int64_t)R, p0 + seg);
  const bool has = w < nseg && p0 < R;
  int nbad = 0;
  if (has) nbad = count_segment(ids, p0, pend, E, lane, L.hist + w * E);
  if (lane == 0) L.wbad[w] = nbad;
  __syncthreads();
  // Per expert: segment bases, then the exclusive scan of the totals.  Thread
  // tid owns experts tid, tid + NT, ...; the scan runs over the experts in
  // index order, one block of NT experts after the other.
  int carry = 0, maxg = 0;
  for (int e0 = 0; e0 < E; e0 += NT) {
    const int e = e0 + tid;
    int total_e = 0;
    if (e < E) {
      int run = 0;
      for (int c = 0; c < nseg; ++c) {
        const int v = L.hist[c * E + e];
        L.hist[c * E + e] = run;
        run += v;
      }
      total_e = run;
    }
    const int incl = wave_inclusive_scan(total_e);
    const int mx = wave_max(total_e);
    if (lane == 63) L.wsum[w] = incl;
    if (lane == 0) L.wmax[w] = mx;
    __syncthreads();
    int base = carry;
    for (int i = 0; i < w; ++i) base += L.wsum[i];
    if (e < E) {
      const int excl = base + incl - total_e;
      offsets[e] = excl;
      for (int c = 0; c < nseg; ++c) L.hist[c * E + e] += excl;
    }
    for (int i = 0; i < NW; ++i) {
      carry += L.wsum[i];
      maxg = max(maxg, L.wmax[i]);
    }
    __syncthreads();  // wsum / wmax are rewritten by the next block of experts
  }
  if (tid == 0) {
    int bad = 0;
    for (int i = 0; i < NW; ++i) bad += L.wbad[i];
    offsets[E] = carry;
    status[0] = maxg;
    status[1] = bad;
  }
  const int total = carry;
  for (int r = total + tid; r < R; r += NT) row_token[r] = -1;
  if (has)
    rank_segment(ids, p0, pend, E, k, nbits, lane, L.hist + w * E, scatter_index, row_token,
                 fold ? L.row_token : nullptr);
  if (fold) {
    __syncthreads();
    const int n = total * row_vecs;
    for (int i = tid; i < n; i += NT) {
      const int r = i / row_vecs, v = i - r * row_vecs;
      xs[(int64_t)r * row_vecs + v] = x[(int64_t)L.row_token[r] * row_vecs + v];
    }
  }
}

#define MOE_BLOCK_LDS(NW)                                                                        \
  extern __shared__ int32_t hist[];                                                              \
  __shared__ int32_t wsum[NW], wmax[NW], wbad[NW];                                               \
  __shared__ int32_t s_row_token[kFoldRows];                                                     \
  const BlockLds lds{hist, wsum, wmax, wbad, s_row_token};

template <int NW>
__global__ __launch_bounds__(NW * 64) void scatter_small(const int32_t* __restrict__ ids, int R, int E, int k,
                                                         int nbits, int nseg, int32_t* __restrict__ scatter_index,
                                                         int32_t* __restrict__ row_token,
                                                         int32_t* __restrict__ offsets, int32_t* __restrict__ status,
                                                         int fold, const u32x4* __restrict__ x, int row_vecs,
                                                         u32x4* __restrict__ xs) {
  MOE_BLOCK_LDS(NW)
  scatter_block<NW>(ids, R, E, k, nbits, nseg, scatter_index, row_token, offsets, status, fold, x, row_vecs, xs, lds);
}

// Routing and scatter of at most kRsTokens tokens (and kRsLogits logits) in
// one workgroup: the workgroup first assembles every logit (fixed-order sum of
// the partial logits + bias) into the logits output and LDS; each wave then
// runs topk_wave for its tokens from the LDS copy, the selections go to global
// memory and to LDS, and the workgroup builds the scatter from the LDS copy.
constexpr int kRsTokens = 16;
constexpr int kRsLogits = 4096;

template <int NW, int Q>
__global__ __launch_bounds__(NW * 64) void route_scatter_small(
    const float* __restrict__ partial, int nsplit, const float* __restrict__ bias, float* __restrict__ logits,
    int T, int E, int k, int32_t* __restrict__ topk_ids, float* __restrict__ topk_weights, int nbits, int nseg,
    int32_t* __restrict__ scatter_index, int32_t* __restrict__ row_token, int32_t* __restrict__ offsets,
    int32_t* __restrict__ status, int fold, const u32x4* __restrict__ x, int row_vecs, u32x4* __restrict__ xs) {
  MOE_BLOCK_LDS(NW)
  __shared__ int32_t s_ids[kRsTokens * kMaxTopK];
  __shared__ float s_logits[kRsLogits];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // Logits: each the fixed-order sum of its slices (+ bias).  With at most one
  // logit per thread, all of its slice loads go out together (32 at a time);
  // otherwise four logits per thread at a time, 8 slices each.
  constexpr int kNT = NW * kWave;
  if (T * E <= kNT) {
    if (tid < T * E) {
      const float* ptr[1] = {partial + tid};
      const bool ok[1] = {true};
      float v[1];
      sum_slices_n<1, 32>(ptr, ok, (int64_t)T * E, nsplit, v);
      if (bias) v[0] += bias[tid % E];
      logits[tid] = v[0];
      s_logits[tid] = v[0];
    }
  }
  for (int i0 = tid; T * E > kNT && i0 < T * E; i0 += 4 * kNT) {
    const float* ptr[4];
    bool ok[4];
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ok[j] = i0 + j * kNT < T * E;
      ptr[j] = partial + i0 + j * kNT;
    }
    sum_slices_n<4, 8>(ptr, ok, (int64_t)T * E, nsplit, v);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = i0 + j * kNT;
      if (!ok[j]) continue;
      if (bias) v[j] += bias[i % E];
      logits[i] = v[j];
      s_logits[i] = v[j];
    }
  }
  __syncthreads();
  for (int t = w; t < T; t += NW) {
    float raw[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int e = lane + kWave * q;
      raw[q] = e < E ? s_logits[t * E + e] : -INFINITY;
    }
    int id;
    float wgt;
    topk_wave(raw, E, k, id, wgt);
    if (lane < k) {
      topk_ids[(int64_t)t * k + lane] = id;
      topk_weights[(int64_t)t * k + lane] = wgt;
      s_ids[t * k + lane] = id;
    }
  }
  __syncthreads();
  scatter_block<NW>(s_ids, T * k, E, k, nbits, nseg, scatter_index, row_token, offsets, status, fold, x, row_vecs,
                    xs, lds);
}

constexpr int kCopyRows = 8;

__global__ __launch_bounds__(256) void scatter_copy(const u32x4* __restrict__ x, const int32_t* __restrict__ row_token,
                                                    const int32_t* __restrict__ offsets, int E, int R, int row_vecs,
                                                    u32x4* __restrict__ xs) {
  const int nvalid = offsets[E];
  const int r0 = blockIdx.x * kCopyRows;
  for (int rr = 0; rr < kCopyRows; ++rr) {
    const int r = r0 + rr;
    if (r >= nvalid || r >= R) break;
    const int t = row_token[r];
    const u32x4* src = x + (int64_t)t * row_vecs;
    u32x4* dst = xs + (int64_t)r * row_vecs;
    for (int v = threadIdx.x; v < row_vecs; v += 256) dst[v] = src[v];
  }
}

int num_chunks(int R) { return (R + kChunk - 1) / kChunk; }

}  // namespace
}  // namespace moe

namespace moe_launch {

size_t scatter_workspace_bytes(int T, int top_k, int E) {
  const int64_t R = (int64_t)T * top_k;
  const int64_t nchunks = (R + moe::kChunk - 1) / moe::kChunk;
  return (size_t)(nchunks * (E + 1) * 4 + 256);
}

hipError_t build_scatter(int dt, const void* x, const int32_t* ids, int T, int H, int E, int top_k,
                         int32_t* scatter_index, int32_t* row_token, int32_t* offsets, int32_t* status_words,
                         void* x_scattered, void* workspace, hipStream_t s) {
  using namespace moe;
  const int R = T * top_k;
  const int nchunks = num_chunks(R);
  const int nblk = (nchunks + kWavesPerBlock - 1) / kWavesPerBlock;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  hipError_t err;
  const int elem = dt == 1 ? 2 : 4;
  const int row_vecs = (int)((int64_t)H * elem / 16);
  const int nseg = block_segments(4, E, R);
  if ((int64_t)nseg * kChunk >= R) {
    const int fold = x_scattered && R <= kFoldRows && (int64_t)R * row_vecs * 16 <= kFoldBytes;
    const size_t lds = (size_t)nseg * E * sizeof(int32_t);
    hipLaunchKernelGGL(scatter_small<4>, dim3(1), dim3(256), lds, s, ids, R, E, top_k, nbits, nseg,
                       scatter_index, row_token, offsets, status_words, fold, (const u32x4*)x, row_vecs,
                       (u32x4*)x_scattered);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (fold) return hipSuccess;
  } else {
    int32_t* cnt = (int32_t*)workspace;
    int32_t* bad = cnt + (int64_t)nchunks * E;
    const size_t lds = (size_t)kWavesPerBlock * E * sizeof(int32_t);
    hipLaunchKernelGGL(scatter_count, dim3(nblk), dim3(256), lds, s, ids, R, E, nchunks, cnt, bad);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(scatter_scan, dim3(1), dim3(1024), 0, s, cnt, (const int32_t*)bad, nchunks, E, R, offsets,
                       status_words, row_token);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(scatter_rank, dim3(nchunks), dim3(256), lds, s, ids, R, E, top_k, nbits, nchunks,
                       (const int32_t*)cnt, (const int32_t*)offsets, scatter_index, row_token);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (!x_scattered) return hipSuccess;  // rows gathered on load by the fc1 call instead
  hipLaunchKernelGGL(scatter_copy, dim3((R + kCopyRows - 1) / kCopyRows), dim3(256), 0, s, (const u32x4*)x,
                     (const int32_t*)row_token, (const int32_t*)offsets, E, R, row_vecs, (u32x4*)x_scattered);
  return hipGetLastError();
}

bool route_scatter_fusable(int T, int top_k, int E) {
  using namespace moe;
  const int R = T * top_k;
  // the launch takes 4 waves up to 4 tokens, else 16, and R <= 16 * 32 pairs always fit its segments
  return T <= kRsTokens && T * E <= kRsLogits && top_k <= kMaxTopK &&
         (int64_t)block_segments(T <= 4 ? 4 : kSmallWaves, E, R) * kChunk >= R;
}

hipError_t route_scatter_fused(int dt, const float* partial, int nsplit, const float* bias, float* logits, int T,
                               int H, int E, int top_k, int32_t* ids, float* weights, const void* x,
                               int32_t* scatter_index, int32_t* row_token, int32_t* offsets, int32_t* status_words,
                               void* x_scattered, hipStream_t s) {
  using namespace moe;
  const int R = T * top_k;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const int elem = dt == 1 ? 2 : 4;
  const int row_vecs = (int)((int64_t)H * elem / 16);
  const int fold = x_scattered && R <= kFoldRows && (int64_t)R * row_vecs * 16 <= kFoldBytes;
  auto launch = [&](auto nw, auto q) {
    constexpr int NW = decltype(nw)::value, Q = decltype(q)::value;
    const int nseg = block_segments(NW, E, R);
    const size_t lds = (size_t)nseg * E * sizeof(int32_t);
    hipLaunchKernelGGL((route_scatter_small<NW, Q>), dim3(1), dim3(NW * 64), lds, s, partial, nsplit, bias, logits,
                       T, E, top_k, ids, weights, nbits, nseg, scatter_index, row_token, offsets, status_words,
                       fold, (const u32x4*)x, row_vecs, (u32x4*)x_scattered);
  };
  auto with_q = [&](auto nw) {
    switch (topk_per_lane(E)) {
      case 1: launch(nw, std::integral_constant<int, 1>{}); break;
      case 2: launch(nw, std::integral_constant<int, 2>{}); break;
      case 4: launch(nw, std::integral_constant<int, 4>{}); break;
      case 8: launch(nw, std::integral_constant<int, 8>{}); break;
      default: launch(nw, std::integral_constant<int, kTopkPer>{}); break;
    }
  };
  if (T <= 4)  // one token per wave
    with_q(std::integral_constant<int, 4>{});
  else
    with_q(std::integral_constant<int, kSmallWaves>{});
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || fold || !x_scattered) return err;  // rows copied, or not wanted
  hipLaunchKernelGGL(scatter_copy, dim3((R + kCopyRows - 1) / kCopyRows), dim3(256), 0, s, (const u32x4*)x,
                     (const int32_t*)row_token, (const int32_t*)offsets, E, R, row_vecs, (u32x4*)x_scattered);
  return hipGetLastError();
}

}  // namespace moe_launch
