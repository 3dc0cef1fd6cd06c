// Mesh utilities: replay order by step count and the largest step count.
//
// Lane ordering.  Trajectories of one ensemble need different numbers of
// accepted steps (the GRADSOLVE review, Strengths, quotes a max/mean of
// 1.33-1.34 from the paper's Table 5).  A wavefront replays for as many steps
// as its longest lane needs, so slots are reordered by decreasing n_steps:
// neighbouring lanes then carry nearly equal work.  The sort is a stable LSD
// radix sort over 8-bit digits of key = max_steps - n_steps (deterministic:
// no atomics) of (key, trajectory) pairs; the sorted trajectories are the
// replay order.  The mesh itself is not moved: with the tiled step log a lane
// reads whole 128-byte chunks of its trajectory wherever they lie.
#include "dadj_internal.hpp"

namespace dadj {
namespace {

constexpr int SORT_THREADS = 256;
constexpr int SORT_ITEMS = 4;                 // per thread
constexpr int SORT_TILE = SORT_THREADS * SORT_ITEMS;
constexpr int RADIX = 256;

__device__ __forceinline__ unsigned digit_of(unsigned key, int shift) {
  return (key >> shift) & (RADIX - 1);
}

// keys from n_steps; values = source slot
__global__ __launch_bounds__(SORT_THREADS) void k_init_keys(int64_t n, int32_t max_steps,
                                                            const int32_t *__restrict__ nsteps,
                                                            unsigned *__restrict__ keys,
                                                            int32_t *__restrict__ vals) {
  const int64_t j = (int64_t)blockIdx.x * SORT_THREADS + threadIdx.x;
  if (j >= n) return;
  int s = nsteps[j];
  s = s < 0 ? 0 : (s > max_steps ? max_steps : s);
  keys[j] = (unsigned)(max_steps - s);
  vals[j] = (int32_t)j;
}

// counts[d * ntiles + tile] = number of keys of the tile with digit d
__global__ __launch_bounds__(SORT_THREADS) void k_hist(int64_t n, int shift,
                                                       const unsigned *__restrict__ keys,
                                                       unsigned *__restrict__ counts,
                                                       int64_t ntiles) {
  __shared__ unsigned h[RADIX];
  h[threadIdx.x] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * SORT_TILE;
  for (int r = 0; r < SORT_ITEMS; ++r) {
    const int64_t e = base + r * SORT_THREADS + threadIdx.x;
    if (e < n) atomicAdd(&h[digit_of(keys[e], shift)], 1u);
  }
  __syncthreads();
  counts[(int64_t)threadIdx.x * ntiles + blockIdx.x] = h[threadIdx.x];
}

// exclusive scan of counts[0..m) in place, one workgroup
__global__ __launch_bounds__(SORT_THREADS) void k_scan(unsigned *__restrict__ counts, int64_t m) {
  __shared__ unsigned part[SORT_THREADS];
  __shared__ unsigned carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int64_t base = 0; base < m; base += SORT_THREADS) {
    const int64_t e = base + threadIdx.x;
    const unsigned v = e < m ? counts[e] : 0u;
    part[threadIdx.x] = v;
    __syncthreads();
    for (int off = 1; off < SORT_THREADS; off <<= 1) {
      const unsigned add = threadIdx.x >= (unsigned)off ? part[threadIdx.x - off] : 0u;
      __syncthreads();
      part[threadIdx.x] += add;
      __syncthreads();
    }
    if (e < m) counts[e] = carry + part[threadIdx.x] - v;
    __syncthreads();
    if (threadIdx.x == SORT_THREADS - 1) carry += part[SORT_THREADS - 1];
    __syncthreads();
  }
}

// Multi-workgroup exclusive scan of counts[0..m): each workgroup scans a
// segment of SCAN_SEG values in place and writes the segment total; the
// totals are scanned (k_scan) and added back (k_scan_add).
constexpr int SCAN_SEG = SORT_THREADS * 4;

__global__ __launch_bounds__(SORT_THREADS) void k_scan_seg(unsigned *__restrict__ counts,
                                                           int64_t m,
                                                           unsigned *__restrict__ seg_total) {
  __shared__ unsigned part[SORT_THREADS];
  const int64_t base = (int64_t)blockIdx.x * SCAN_SEG + (int64_t)threadIdx.x * 4;
  unsigned v[4], t = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[q] = (base + q < m) ? counts[base + q] : 0u;
    t += v[q];
  }
  part[threadIdx.x] = t;
  __syncthreads();
  for (int off = 1; off < SORT_THREADS; off <<= 1) {
    const unsigned add = threadIdx.x >= (unsigned)off ? part[threadIdx.x - off] : 0u;
    __syncthreads();
    part[threadIdx.x] += add;
    __syncthreads();
  }
  unsigned run = part[threadIdx.x] - t;  // exclusive prefix of this thread's items
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (base + q < m) counts[base + q] = run;
    run += v[q];
  }
  if (threadIdx.x == SORT_THREADS - 1) seg_total[blockIdx.x] = part[SORT_THREADS - 1];
}

__global__ __launch_bounds__(SORT_THREADS) void k_scan_add(unsigned *__restrict__ counts,
                                                           int64_t m,
                                                           const unsigned *__restrict__ seg_off) {
  const unsigned add = seg_off[blockIdx.x];
  const int64_t base = (int64_t)blockIdx.x * SCAN_SEG;
  for (int q = threadIdx.x; q < SCAN_SEG; q += SORT_THREADS)
    if (base + q < m) counts[base + q] += add;
}

// stable scatter of one tile: rank among equal digits of earlier elements
__global__ __launch_bounds__(SORT_THREADS) void k_scatter(int64_t n, int shift, int64_t ntiles,
                                                          const unsigned *__restrict__ counts,
                                                          const unsigned *__restrict__ kin,
                                                          const int32_t *__restrict__ vin,
                                                          unsigned *__restrict__ kout,
                                                          int32_t *__restrict__ vout) {
  constexpr int NW = SORT_THREADS / 64;
  __shared__ unsigned run[RADIX];          // running count per digit within the tile
  __shared__ unsigned wcnt[NW][RADIX];     // per-wave counts of the current round
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  run[threadIdx.x] = 0;
  const int64_t base = (int64_t)blockIdx.x * SORT_TILE;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r = 0; r < SORT_ITEMS; ++r) {
    for (int q = 0; q < NW; ++q) wcnt[q][threadIdx.x] = 0;
    __syncthreads();
    const int64_t e = base + r * SORT_THREADS + threadIdx.x;
    const bool valid = e < n;
    const unsigned key = valid ? kin[e] : 0u;
    const unsigned d = digit_of(key, shift);
    // lanes of this wave holding the same digit
    uint64_t same = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (d >> b) & 1u;
      const uint64_t m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    const unsigned rank_w = (unsigned)__popcll(same & lt);
    if (valid && rank_w == 0) wcnt[w][d] = (unsigned)__popcll(same);
    __syncthreads();
    if (valid) {
      unsigned pre = run[d];
      for (int q = 0; q < w; ++q) pre += wcnt[q][d];
      const unsigned pos = counts[(int64_t)d * ntiles + blockIdx.x] + pre + rank_w;
      kout[pos] = key;
      vout[pos] = vin[e];
    }
    __syncthreads();
    unsigned tot = 0;
    for (int q = 0; q < NW; ++q) tot += wcnt[q][threadIdx.x];
    run[threadIdx.x] += tot;
    __syncthreads();
  }
}

// Replay table: lane j (trajectory perm[j]) reads its trajectory's 128-byte
// chunks of the tiled log whole (one line each) and writes them as B
// consecutive rows, each store a contiguous row segment across the
// wavefront; zeros after n_steps.  The chunk rows are split into ranges of
// `tpy` over the second grid dimension, so that a small ensemble still puts
// many wavefronts in flight.
typedef double dvec2 __attribute__((ext_vector_type(2)));
typedef float fvec4 __attribute__((ext_vector_type(4)));
constexpr int QUADS = CHUNK_BYTES / 16;  // 16-byte pieces per chunk

__device__ __forceinline__ void load_chunk(const double *src, double (&v)[CHUNK_BYTES / 8]) {
  const dvec2 *s = (const dvec2 *)src;
#pragma unroll
  for (int q = 0; q < QUADS; ++q) {
    const dvec2 x = s[q];
    v[2 * q] = x.x;
    v[2 * q + 1] = x.y;
  }
}
__device__ __forceinline__ void load_chunk(const float *src, float (&v)[CHUNK_BYTES / 4]) {
  const fvec4 *s = (const fvec4 *)src;
#pragma unroll
  for (int q = 0; q < QUADS; ++q) {
    const fvec4 x = s[q];
    v[4 * q] = x.x;
    v[4 * q + 1] = x.y;
    v[4 * q + 2] = x.z;
    v[4 * q + 3] = x.w;
  }
}

template <class T>
__global__ __launch_bounds__(SORT_THREADS) void k_replay_table(
    int64_t n, int32_t max_steps, const T *__restrict__ h, const int32_t *__restrict__ nsteps,
    const int32_t *__restrict__ perm, T *__restrict__ out, int32_t rows, int32_t tpy) {
  constexpr int B = CHUNK_BYTES / (int)sizeof(T);
  const int64_t j = (int64_t)blockIdx.x * SORT_THREADS + threadIdx.x;
  if (j >= n) return;
  const int64_t tr = perm ? perm[j] : j;
  int N = nsteps[tr];
  N = N < 0 ? 0 : (N > max_steps ? max_steps : N);
  const int tmax = (rows + B - 1) / B;
  const int t0 = (int)blockIdx.y * tpy;
  const int t1 = t0 + tpy < tmax ? t0 + tpy : tmax;
  for (int t = t0; t < t1; ++t) {
    T c[B];
    if (t * B < N) {
      load_chunk(h + ((int64_t)t * n + tr) * B, c);
    } else {
#pragma unroll
      for (int b = 0; b < B; ++b) c[b] = T(0);
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int k = t * B + b;
      if (k < rows) out[(int64_t)k * n + j] = k < N ? c[b] : T(0);
    }
  }
}

// Largest value of ns[0..n): MAX_BLOCKS workgroups each reduce a strided
// share into out[1 + block], then one workgroup reduces those into out[0].
constexpr int MAX_BLOCKS = 256;

__global__ __launch_bounds__(1024) void k_max_steps(int64_t n, const int32_t *__restrict__ ns,
                                                    int32_t *__restrict__ out) {
  __shared__ int part[1024];
  int m = 0;
  for (int64_t j = (int64_t)blockIdx.x * 1024 + threadIdx.x; j < n;
       j += (int64_t)gridDim.x * 1024)
    m = ns[j] > m ? ns[j] : m;
  part[threadIdx.x] = m;
  __syncthreads();
  for (int off = 512; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off && part[threadIdx.x + off] > part[threadIdx.x])
      part[threadIdx.x] = part[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[1 + blockIdx.x] = part[0];
}

__global__ __launch_bounds__(MAX_BLOCKS) void k_max_final(int nb, int32_t *__restrict__ out) {
  __shared__ int part[MAX_BLOCKS];
  part[threadIdx.x] = (int)threadIdx.x < nb ? out[1 + threadIdx.x] : 0;
  __syncthreads();
  for (int off = MAX_BLOCKS / 2; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off && part[threadIdx.x + off] > part[threadIdx.x])
      part[threadIdx.x] = part[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = part[0];
}

// Zero chunks t >= ceil(N_i / B) of every trajectory i (the padding of a
// record taken with deferred padding).  Thread i walks its chunk rows; a
// wavefront writes 64 adjacent chunks per row, as QUADS 16-byte stores per
// lane.
template <class T>
__global__ __launch_bounds__(SORT_THREADS) void k_mesh_pad(int64_t n, int32_t n_chunks,
                                                           int32_t max_steps,
                                                           const int32_t *__restrict__ nsteps,
                                                           T *__restrict__ h) {
  constexpr int B = CHUNK_BYTES / (int)sizeof(T);
  const int64_t i = (int64_t)blockIdx.x * SORT_THREADS + threadIdx.x;
  if (i >= n) return;
  int N = nsteps[i];
  N = N < 0 ? 0 : (N > max_steps ? max_steps : N);
  for (int t = (N + B - 1) / B; t < n_chunks; ++t) {
    dvec2 *dst = (dvec2 *)(h + ((int64_t)t * n + i) * B);
#pragma unroll
    for (int q = 0; q < QUADS; ++q) dst[q] = dvec2{0.0, 0.0};
  }
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

int key_bits(int32_t max_steps) {
  int b = 1;
  while (b < 31 && (1u << b) <= (unsigned)max_steps) ++b;
  return b;
}

}  // namespace

size_t sort_workspace_bytes(int64_t n) {
  const int64_t ntiles = (n + SORT_TILE - 1) / SORT_TILE;
  const int64_t m = ntiles * RADIX;
  const int64_t nseg = (m + SCAN_SEG - 1) / SCAN_SEG;
  return 3 * align_up((size_t)n * 4) + align_up((size_t)m * 4) + align_up((size_t)nseg * 4);
}

// Radix passes ping-pong between (kA, vA) and (kB, vB); the values of the
// last pass land in `perm`, which serves as one of the two value buffers.
hipError_t launch_mesh_sort(const ProbArgs &pr, int64_t n, const int32_t *nsteps, int32_t *perm,
                            void *ws, size_t ws_bytes, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (ws_bytes < sort_workspace_bytes(n)) return hipErrorInvalidValue;
  const int64_t ntiles = (n + SORT_TILE - 1) / SORT_TILE;
  const int bits = key_bits(pr.max_steps);
  const int passes = (bits + 7) / 8;
  char *q = (char *)ws;
  unsigned *kA = (unsigned *)q; q += align_up((size_t)n * 4);
  unsigned *kB = (unsigned *)q; q += align_up((size_t)n * 4);
  int32_t *vX = (int32_t *)q; q += align_up((size_t)n * 4);
  unsigned *counts = (unsigned *)q; q += align_up((size_t)ntiles * RADIX * 4);
  unsigned *seg_total = (unsigned *)q;
  const int64_t m = ntiles * RADIX;
  const unsigned nseg = (unsigned)((m + SCAN_SEG - 1) / SCAN_SEG);
  // choose the initial value buffer so that the last pass writes `perm`
  int32_t *vA = (passes % 2 == 0) ? perm : vX;
  int32_t *vB = (passes % 2 == 0) ? vX : perm;
  const unsigned g1 = (unsigned)((n + SORT_THREADS - 1) / SORT_THREADS);
  hipLaunchKernelGGL(k_init_keys, g1, SORT_THREADS, 0, s, n, pr.max_steps, nsteps, kA, vA);
  for (int shift = 0; shift < bits; shift += 8) {
    hipLaunchKernelGGL(k_hist, (unsigned)ntiles, SORT_THREADS, 0, s, n, shift, kA, counts, ntiles);
    hipLaunchKernelGGL(k_scan_seg, nseg, SORT_THREADS, 0, s, counts, m, seg_total);
    hipLaunchKernelGGL(k_scan, 1, SORT_THREADS, 0, s, seg_total, (int64_t)nseg);
    hipLaunchKernelGGL(k_scan_add, nseg, SORT_THREADS, 0, s, counts, m, seg_total);
    hipLaunchKernelGGL(k_scatter, (unsigned)ntiles, SORT_THREADS, 0, s, n, shift, ntiles, counts,
                       kA, vA, kB, vB);
    unsigned *tk = kA; kA = kB; kB = tk;
    int32_t *tv = vA; vA = vB; vB = tv;
  }
  return hipGetLastError();
}

// Wavefronts the replay table aims for.  Split over trajectories alone, a
// 65536-trajectory ensemble launches 1024 wavefronts (one per SIMD) and
// streams at 2.5 TB/s; split also over row ranges to about 65536 wavefronts
// it reaches 4.5 TB/s (4096: 4.0, 32768: 4.4, 131072: 4.5), and the
// 2^20-trajectory table goes from 3.5 to 3.6 TB/s.
constexpr int64_t TABLE_WAVES = 65536;

hipError_t launch_replay_table(const ProbArgs &pr, int64_t n, const void *h,
                               const int32_t *nsteps, const int32_t *perm, void *h_rows,
                               int32_t rows, hipStream_t s) {
  if (n == 0 || rows <= 0) return hipSuccess;
  const unsigned g1 = (unsigned)((n + SORT_THREADS - 1) / SORT_THREADS);
  const int B = chunk_steps(pr.dtype);
  const int64_t tmax = (rows + B - 1) / B;
  const int64_t waves = (n + 63) / 64;
  int64_t ny = (TABLE_WAVES + waves - 1) / waves;
  ny = ny < 1 ? 1 : (ny > tmax ? tmax : ny);
  ny = ny > 65535 ? 65535 : ny;
  const int64_t tpy = (tmax + ny - 1) / ny;
  ny = (tmax + tpy - 1) / tpy;
  const dim3 grid(g1, (unsigned)ny);
  if (pr.dtype == DA_F64)
    hipLaunchKernelGGL(k_replay_table<double>, grid, SORT_THREADS, 0, s, n, pr.max_steps,
                       (const double *)h, nsteps, perm, (double *)h_rows, rows, (int32_t)tpy);
  else
    hipLaunchKernelGGL(k_replay_table<float>, grid, SORT_THREADS, 0, s, n, pr.max_steps,
                       (const float *)h, nsteps, perm, (float *)h_rows, rows, (int32_t)tpy);
  return hipGetLastError();
}

hipError_t launch_mesh_pad(const ProbArgs &pr, int64_t n, const int32_t *nsteps, void *h,
                           hipStream_t s) {
  const unsigned g = (unsigned)((n + SORT_THREADS - 1) / SORT_THREADS);
  if (pr.dtype == DA_F64)
    hipLaunchKernelGGL(k_mesh_pad<double>, g, SORT_THREADS, 0, s, n, pr.n_chunks, pr.max_steps,
                       nsteps, (double *)h);
  else
    hipLaunchKernelGGL(k_mesh_pad<float>, g, SORT_THREADS, 0, s, n, pr.n_chunks, pr.max_steps,
                       nsteps, (float *)h);
  return hipGetLastError();
}

size_t max_steps_scratch_ints() { return 1 + MAX_BLOCKS; }

hipError_t launch_max_steps(int64_t n, const int32_t *nsteps, int32_t *dev_out, hipStream_t s) {
  int64_t nb = (n + 1023) / 1024;
  nb = nb < 1 ? 1 : (nb > MAX_BLOCKS ? MAX_BLOCKS : nb);
  hipLaunchKernelGGL(k_max_steps, (unsigned)nb, 1024, 0, s, n, nsteps, dev_out);
  hipLaunchKernelGGL(k_max_final, 1, MAX_BLOCKS, 0, s, (int)nb, dev_out);
  return hipGetLastError();
}

}  // namespace dadj
