// Dispatch: group the T*k (token, slot) entries by expert in token order,
// with per-expert capacity (page "MoE: how sparse activation saves compute",
// sections 3.5, 3.6 and 3.8).
//
// Three launches, no host synchronisation, integer-only and deterministic:
//   1. count: each block histograms one chunk of entries in LDS;
//   2. scan:  one block turns the per-chunk histograms into per-chunk
//             exclusive bases (chunk order = token order), L_i, offsets and
//             kept offsets;
//   3. rank:  one wave per chunk walks its entries 64 at a time; lanes that
//             name the same expert find each other with ballots over the
//             expert id bits, so each entry's rank is
//             base[chunk][e] + (earlier lanes with e) -- a stable,
//             token-order rank without atomics deciding any order.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kChunk = 1024;  // entries per chunk
constexpr int kMaxN = 1024;

// Blocks past the last chunk (when stats != nullptr): block (band, slice)
// sums rows [64 slice, 64 slice + 64) of the router's partial rows [rows][N]
// for a band of EW experts -- 256 / EW rows at a time, EW lanes a row
// (reads coalesced along the experts), then a fixed tree -- and leaves the
// sums in the slice's first row.  The scan launch adds the slices in order.
constexpr int kStatsSlice = 64;

__device__ void stats_slice(float *__restrict__ part_p, int32_t *__restrict__ part_cnt, int rows,
                            int N, int EW, int band, int slice) {
  __shared__ float sp[256];
  __shared__ int sc[256];
  const int rr = threadIdx.x / EW, e = threadIdx.x % EW;
  const int rpp = 256 / EW;
  const int n = band * EW + e;
  const int r0 = slice * kStatsSlice;
  const int r1 = r0 + kStatsSlice < rows ? r0 + kStatsSlice : rows;
  float p = 0.f;
  int c = 0;
  if (n < N)
    for (int wv = r0 + rr; wv < r1; wv += rpp) {
      p += part_p[(int64_t)wv * N + n];
      c += part_cnt[(int64_t)wv * N + n];
    }
  sp[threadIdx.x] = p;
  sc[threadIdx.x] = c;
  __syncthreads();
  for (int s = rpp / 2; s > 0; s >>= 1) {
    if (rr < s) {
      sp[threadIdx.x] += sp[threadIdx.x + s * EW];
      sc[threadIdx.x] += sc[threadIdx.x + s * EW];
    }
    __syncthreads();
  }
  // Only this block reads these columns of this slice, and it has finished.
  if (rr == 0 && n < N) {
    part_p[(int64_t)r0 * N + n] = sp[e];
    part_cnt[(int64_t)r0 * N + n] = sc[e];
  }
}

int stats_band_width(int N) {
  int ew = 8;  // a power of two, 8 .. 64
  while (ew < 64 && ew < N) ew *= 2;
  return ew;
}

__global__ __launch_bounds__(256) void dispatch_count_kernel(
    const int32_t *__restrict__ idx, int64_t E, int N, int32_t *__restrict__ blk_counts, int nblk,
    float *__restrict__ part_p, int32_t *__restrict__ part_cnt, int rows, int EW) {
  if ((int)blockIdx.x >= nblk) {
    const int sb = (int)blockIdx.x - nblk;
    const int slices = (rows + kStatsSlice - 1) / kStatsSlice;
    stats_slice(part_p, part_cnt, rows, N, EW, sb / slices, sb % slices);
    return;
  }
  __shared__ int32_t hist[kMaxN];
  for (int n = threadIdx.x; n < N; n += blockDim.x) hist[n] = 0;
  __syncthreads();
  const int64_t lo = (int64_t)blockIdx.x * kChunk;
  const int64_t hi = lo + kChunk < E ? lo + kChunk : E;
  for (int64_t j = lo + threadIdx.x; j < hi; j += blockDim.x) {
    const int e = idx[j];
    if (e >= 0 && e < N) atomicAdd(&hist[e], 1);  // integer: order-free
  }
  __syncthreads();
  for (int n = threadIdx.x; n < N; n += blockDim.x)
    blk_counts[(int64_t)blockIdx.x * N + n] = hist[n];
}

// Inclusive block scan of one value per thread (blockDim.x == 1024).
// First level of a halving tree over n values: the largest power of two
// below n (0 for n = 1), so that its levels pair exactly the nonzero ones.
__device__ __forceinline__ int tree_top(int n) {
  int s = 1;
  while (s < n) s <<= 1;
  return s >> 1;
}

// Inclusive scan of v over threads 0 .. n - 1 (the values of threads n and
// above are not used and need not be zero): log2(n) steps instead of
// log2(blockDim), each with its two barriers.
__device__ int block_incl_scan(int v, int *tmp, int n) {
  tmp[threadIdx.x] = v;
  __syncthreads();
  for (int o = 1; o < n; o <<= 1) {
    const int add = (int)threadIdx.x >= o ? tmp[threadIdx.x - o] : 0;
    __syncthreads();
    tmp[threadIdx.x] += add;
    __syncthreads();
  }
  const int r = tmp[threadIdx.x];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(1024) void dispatch_scan_kernel(
    int32_t *__restrict__ blk_counts, int nblk, int N, int capacity, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ kept_offsets,
    const float *__restrict__ part_p, const int32_t *__restrict__ part_cnt, int rows, int64_t T,
    float alpha, float *__restrict__ stats) {
  __shared__ int tmp[1024];
  __shared__ float red[1024];
  const int n = threadIdx.x;  // N <= 1024: one expert per thread
  if (stats != nullptr) {
    // f_n = (arg-max count) / T and P_n = (sum of p) / T from the count
    // launch's slice sums, in slice order; N sum_n f_n P_n by a fixed tree.
    float fp = 0.f;
    if (n < N) {
      float p = 0.f;
      int64_t c = 0;
      for (int r = 0; r < rows; r += kStatsSlice) {
        p += part_p[(int64_t)r * N + n];
        c += part_cnt[(int64_t)r * N + n];
      }
      const float f = (float)((double)c / (double)T);
      const float P = p / (float)T;
      stats[n] = f;
      stats[N + n] = P;
      fp = f * P;
    }
    red[n] = fp;
    __syncthreads();
    // Levels at or past N would add the zeros of threads N and above.
    for (int s = tree_top(N); s > 0; s >>= 1) {
      if (n < s) red[n] += red[n + s];
      __syncthreads();
    }
    if (n == 0) {
      const float v = (float)N * red[0];
      stats[2 * N] = v;
      stats[2 * N + 1] = alpha * v;
    }
  }
  int total = 0;
  if (n < N) {
    // 16 chunks' counts are loaded before any of their bases is stored, so
    // the loads are in flight together (a store to the same array would
    // otherwise hold back the next load).
    constexpr int kB = 16;
    for (int b0 = 0; b0 < nblk; b0 += kB) {
      int c[kB];
#pragma unroll
      for (int j = 0; j < kB; ++j)
        c[j] = b0 + j < nblk ? blk_counts[(int64_t)(b0 + j) * N + n] : 0;
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        if (b0 + j < nblk) blk_counts[(int64_t)(b0 + j) * N + n] = total;  // the chunk's base
        total += c[j];
      }
    }
    counts[n] = total;
  }
  const int kept = (n < N) ? ((capacity >= 0 && total > capacity) ? capacity : total) : 0;
  const int inc_all = block_incl_scan(n < N ? total : 0, tmp, N);
  const int inc_kept = block_incl_scan(kept, tmp, N);
  if (n < N) {
    offsets[n + 1] = inc_all;
    kept_offsets[n + 1] = inc_kept;
  }
  if (n == 0) {
    offsets[0] = 0;
    kept_offsets[0] = 0;
  }
}

__global__ __launch_bounds__(64) void dispatch_rank_kernel(
    const int32_t *__restrict__ idx, int64_t E, int N, int nbits, int capacity,
    const int32_t *__restrict__ blk_counts, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ kept_offsets, int32_t *__restrict__ perm,
    int32_t *__restrict__ row_of, uint8_t *__restrict__ drop) {
  __shared__ int32_t base[kMaxN];
  const int lane = threadIdx.x;
  for (int n = lane; n < N; n += 64) base[n] = blk_counts[(int64_t)blockIdx.x * N + n];
  __syncthreads();
  const int64_t lo = (int64_t)blockIdx.x * kChunk;
  const int64_t hi = lo + kChunk < E ? lo + kChunk : E;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t j0 = lo; j0 < hi; j0 += 64) {
    const int64_t j = j0 + lane;
    int e = (j < hi) ? idx[j] : -1;
    const bool ok = e >= 0 && e < N;
    if (!ok) e = -1;
    uint64_t same = __ballot(ok);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = ok && ((e >> b) & 1);
      const uint64_t ones = __ballot(bit);
      same &= bit ? ones : ~ones;
    }
    int r = 0;
    if (ok) r = base[e] + __popcll(same & below);
    __syncthreads();  // every lane has read base[] before it moves on
    if (ok && (63 - __clzll(same)) == lane) base[e] += __popcll(same);
    __syncthreads();
    if (j < hi) {
      if (ok) {
        perm[offsets[e] + r] = (int32_t)j;
        const bool kept = capacity < 0 || r < capacity;
        row_of[j] = kept ? kept_offsets[e] + r : -1;
        drop[j] = kept ? 0 : 1;
      } else {
        row_of[j] = -1;
        drop[j] = 1;
      }
    }
  }
}

// Small inputs (at most 1024 entries): the balance statistics and the whole
// dispatch in one 1024-thread block.  Wave w takes entries 64w .. 64w+63;
// lanes naming the same expert find each other with ballots over the expert
// id bits (rank within the wave), each group's highest lane records the
// group size in hist[w][e], and an entry's rank is its rank within the wave
// plus hist[w'][e] over the earlier waves w' -- the same stable token-order
// rank as the chunked kernels, with no atomics deciding any order.
constexpr int kTailWaves = 16;
constexpr int kTailMaxN = 1024;

__global__ __launch_bounds__(1024) void small_tail_kernel(
    const float *__restrict__ part_p, const int32_t *__restrict__ part_cnt, int waves, int64_t T,
    float alpha, float *__restrict__ stats, const int32_t *__restrict__ idx, int E, int N,
    int nbits, int capacity, int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ kept_offsets, int32_t *__restrict__ perm, int32_t *__restrict__ row_of,
    uint8_t *__restrict__ drop) {
  __shared__ int32_t hist[kTailWaves][kTailMaxN];
  __shared__ int32_t base_all[kTailMaxN], base_kept[kTailMaxN];
  __shared__ int tmp[1024];
  __shared__ float red[1024];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // The dispatch's expert id, requested before the statistics so that its
  // latency overlaps theirs.
  int e = (perm != nullptr && tid < E) ? idx[tid] : -1;
  if (stats != nullptr) {
    // f_n = (argmax count) / T, P_n = (sum of p) / T, partial rows summed in
    // row order; N * sum_n f_n P_n by a fixed tree.  The rows come through
    // LDS 1024 values at a time, every thread loading one (one round trip
    // per 1024 values instead of one per 8 rows).
    float fp = 0.f;
    float p = 0.f;
    int64_t c = 0;
    const int64_t nval = (int64_t)waves * N;
    for (int64_t v0 = 0; v0 < nval; v0 += 1024) {
      const int64_t v = v0 + tid;
      red[tid] = v < nval ? part_p[v] : 0.f;
      tmp[tid] = v < nval ? part_cnt[v] : 0;
      __syncthreads();
      if (tid < N) {
        // this chunk's rows of column tid, in row order
        const int64_t r0 = (v0 + N - 1 - tid) / N;  // first row r with r N + tid >= v0
        for (int64_t r = r0; r * N + tid < v0 + 1024 && r < waves; ++r) {
          p += red[r * N + tid - v0];
          c += tmp[r * N + tid - v0];
        }
      }
      __syncthreads();
    }
    if (tid < N) {
      const float f = (float)((double)c / (double)T);
      const float P = p / (float)T;
      stats[tid] = f;
      stats[N + tid] = P;
      fp = f * P;
    }
    red[tid] = fp;
    __syncthreads();
    // Levels at or past N would add the zeros of threads N and above.
    for (int s = tree_top(N); s > 0; s >>= 1) {
      if (tid < s) red[tid] += red[tid + s];
      __syncthreads();
    }
    if (tid == 0) {
      const float v = (float)N * red[0];
      stats[2 * N] = v;
      stats[2 * N + 1] = alpha * v;
    }
  }
  if (perm == nullptr) return;

  for (int i = tid; i < kTailWaves * N; i += 1024) hist[i / N][i % N] = 0;
  __syncthreads();
  const bool ok = e >= 0 && e < N;
  if (!ok) e = -1;
  uint64_t same = __ballot(ok);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = ok && ((e >> b) & 1);
    const uint64_t ones = __ballot(bit);
    same &= bit ? ones : ~ones;
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int r_wave = ok ? __popcll(same & below) : 0;
  if (ok && (63 - __clzll(same)) == lane) hist[wave][e] = __popcll(same);
  __syncthreads();

  // Per-expert totals, offsets and kept offsets (thread n = expert n).
  int total = 0;
  if (tid < N)
    for (int w = 0; w < kTailWaves; ++w) total += hist[w][tid];
  const int kept = (tid < N) ? ((capacity >= 0 && total > capacity) ? capacity : total) : 0;
  const int inc_all = block_incl_scan(tid < N ? total : 0, tmp, N);
  const int inc_kept = block_incl_scan(kept, tmp, N);
  if (tid < N) {
    base_all[tid] = inc_all - total;
    base_kept[tid] = inc_kept - kept;
    counts[tid] = total;
    offsets[tid + 1] = inc_all;
    kept_offsets[tid + 1] = inc_kept;
  }
  if (tid == 0) {
    offsets[0] = 0;
    kept_offsets[0] = 0;
  }
  __syncthreads();

  if (tid < E) {
    if (ok) {
      int r = r_wave;
      for (int w = 0; w < wave; ++w) r += hist[w][e];
      perm[base_all[e] + r] = tid;
      const bool keep = capacity < 0 || r < capacity;
      row_of[tid] = keep ? base_kept[e] + r : -1;
      drop[tid] = keep ? 0 : 1;
    } else {
      row_of[tid] = -1;
      drop[tid] = 1;
    }
  }
}

}  // namespace

int dispatch_blocks(int64_t entries) { return (int)((entries + kChunk - 1) / kChunk); }

hipError_t launch_dispatch(const int32_t *idx, int64_t T, int k, int N, int capacity,
                           int32_t *counts, int32_t *offsets, int32_t *kept_offsets,
                           int32_t *perm, int32_t *row_of, uint8_t *drop,
                           int32_t *blk_counts, float *part_p, int32_t *part_cnt,
                           int rows, float alpha, float *stats, hipStream_t st) {
  const int64_t E = T * k;
  const int nblk = dispatch_blocks(E);
  int nbits = 0;
  while ((1 << nbits) < N) ++nbits;
  const int ew = stats_band_width(N);
  const int sblocks =
      stats != nullptr ? ((N + ew - 1) / ew) * ((rows + kStatsSlice - 1) / kStatsSlice) : 0;
  hipLaunchKernelGGL(dispatch_count_kernel, dim3(nblk + sblocks), dim3(256), 0, st, idx, E, N,
                     blk_counts, nblk, part_p, part_cnt, rows, ew);
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(1024), 0, st, blk_counts, nblk, N,
                     capacity, counts, offsets, kept_offsets, part_p, part_cnt, rows, T, alpha,
                     stats);
  hipLaunchKernelGGL(dispatch_rank_kernel, dim3(nblk), dim3(64), 0, st, idx, E, N, nbits,
                     capacity, blk_counts, offsets, kept_offsets, perm, row_of, drop);
  return hipGetLastError();
}

bool small_tail_fits(int64_t entries, int N) {
  return entries <= kTailWaves * 64 && N <= kTailMaxN;
}

hipError_t launch_small_tail(const float *part_p, const int32_t *part_cnt, int waves, int64_t T,
                             float alpha, float *stats, const int32_t *idx, int k, int N,
                             int capacity, int32_t *counts, int32_t *offsets,
                             int32_t *kept_offsets, int32_t *perm, int32_t *row_of,
                             uint8_t *drop, hipStream_t st) {
  int nbits = 0;
  while ((1 << nbits) < N) ++nbits;
  hipLaunchKernelGGL(small_tail_kernel, dim3(1), dim3(1024), 0, st, part_p, part_cnt, waves, T,
                     alpha, stats, idx, (int)(T * k), N, nbits, capacity, counts, offsets,
                     kept_offsets, perm, row_of, drop);
  return hipGetLastError();
}

}  // namespace moe
