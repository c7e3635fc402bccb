// k2_sort.hip -- stable sort of queries and keys by Sort-LSH bucket.
//
// The sparse branch groups similar tokens by sorting them on their hash code
// ("Two Efficient Attentions, One Denominator Problem", section "Two efficient
// branches can still be mis-scaled": the sparse branch keeps only selected
// high-similarity pairs).  For every (b, h) and separately for q and k, the
// permutation perm[rank] = original index orders tokens by (code, index): a
// stable counting sort in three passes over tiles of 2048 codes:
//   1. per-tile bucket histogram (LDS integer atomics), stored bucket-major;
//   2. exclusive scan of the [bucket][tile] counts of each segment: the first
//      sorted rank of every (bucket, tile);
//   3. per tile, each wave ranks its 8 rounds of 64 codes in order: equal codes
//      inside a round are found with one ballot per code bit, earlier waves and
//      rounds are counted in LDS, so every element gets a unique, stable rank.
// Integer-only, hence bit-exact and deterministic.
#include "elsaa_internal.hpp"

namespace elsaa {
namespace {

constexpr int kWaves = 4;
constexpr int kRounds = kSortTile / (kWaves * 64);  // 8

__global__ __launch_bounds__(256) void elsaa_k2_sort_hist(const uint16_t *__restrict__ codes,
                                                          int N, int nb, int T,
                                                          uint32_t *__restrict__ hist) {
  extern __shared__ uint32_t h[];
  const int tile = blockIdx.x;
  const long long s = blockIdx.y;
  for (int b = threadIdx.x; b < nb; b += 256) h[b] = 0;
  __syncthreads();
  const uint16_t *c = codes + s * N;
  const int base = tile * kSortTile;
  for (int e = threadIdx.x; e < kSortTile; e += 256) {
    const int i = base + e;
    if (i < N) atomicAdd(&h[c[i]], 1u);
  }
  __syncthreads();
  uint32_t *out = hist + s * static_cast<long long>(nb) * T;
  for (int b = threadIdx.x; b < nb; b += 256) out[static_cast<long long>(b) * T + tile] = h[b];
}

// In-place exclusive scan of M counts per segment; one 1024-thread block each.
__global__ __launch_bounds__(1024) void elsaa_k2_sort_scan(uint32_t *__restrict__ hist,
                                                           long long M) {
  __shared__ uint32_t part[1024];
  uint32_t *p = hist + static_cast<long long>(blockIdx.x) * M;
  const int tid = threadIdx.x;
  const long long per = (M + 1023) / 1024;
  const long long lo = tid * per;
  const long long hi = lo + per < M ? lo + per : M;
  uint32_t sum = 0;
  for (long long i = lo; i < hi; ++i) sum += p[i];
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // Hillis-Steele inclusive scan
    const uint32_t add = tid >= off ? part[tid - off] : 0u;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  uint32_t run = part[tid] - sum;  // exclusive prefix of this thread's run
  for (long long i = lo; i < hi; ++i) {
    const uint32_t c = p[i];
    p[i] = run;
    run += c;
  }
}

__global__ __launch_bounds__(256) void elsaa_k2_sort_scatter(const uint16_t *__restrict__ codes,
                                                             int N, int ns, int nb, int T,
                                                             const uint32_t *__restrict__ offs,
                                                             int32_t *__restrict__ perm) {
  extern __shared__ uint32_t cnt[];  // [kWaves][nb]
  const int tile = blockIdx.x;
  const long long s = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint16_t *c = codes + s * N;
  const uint32_t *o = offs + s * static_cast<long long>(nb) * T;
  int32_t *pm = perm + s * N;
  const int wbase = tile * kSortTile + wave * (kSortTile / kWaves);
  uint32_t *wc = cnt + wave * nb;

  for (int b = tid; b < kWaves * nb; b += 256) cnt[b] = 0;
  __syncthreads();
  for (int r = 0; r < kRounds; ++r) {
    const int i = wbase + r * 64 + lane;
    if (i < N) atomicAdd(&wc[c[i]], 1u);
  }
  __syncthreads();
  for (int b = tid; b < nb; b += 256) {  // counts of earlier waves in this tile
    uint32_t run = 0;
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t t = cnt[w * nb + b];
      cnt[w * nb + b] = run;
      run += t;
    }
  }
  __syncthreads();

  const unsigned long long lt = (1ull << lane) - 1ull;
  for (int r = 0; r < kRounds; ++r) {
    const int i = wbase + r * 64 + lane;
    const bool valid = i < N;
    const uint32_t code = valid ? c[i] : 0u;
    unsigned long long mask = __ballot(valid);
    for (int bit = 0; bit < ns; ++bit) {
      const bool set = (code >> bit) & 1u;
      const unsigned long long bb = __ballot(set);
      mask &= set ? bb : ~bb;
    }
    const int rank = __popcll(mask & lt);
    const int leader = __ffsll(static_cast<long long>(mask)) - 1;
    uint32_t before = 0;
    if (valid && lane == leader) {
      before = wc[code];
      wc[code] = before + static_cast<uint32_t>(__popcll(mask));
    }
    before = __shfl(before, leader < 0 ? 0 : leader);
    if (valid) {
      const uint32_t dest = o[static_cast<long long>(code) * T + tile] + before + rank;
      pm[dest] = i;
    }
    // the leader's counter update must land before the next round reads it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

}  // namespace

hipError_t launch_sort(const Geometry &g, const Buffers &buf, hipStream_t stream) {
  const int S = 2 * g.BH;
  const int T = g.sort_tiles;
  hipLaunchKernelGGL(elsaa_k2_sort_hist, dim3(T, S), dim3(256), g.nb_sort * 4, stream, buf.scode,
                     g.N, g.nb_sort, T, buf.hist);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(elsaa_k2_sort_scan, dim3(S), dim3(1024), 0, stream, buf.hist,
                     static_cast<long long>(g.nb_sort) * T);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(elsaa_k2_sort_scatter, dim3(T, S), dim3(256), kWaves * g.nb_sort * 4, stream,
                     buf.scode, g.N, g.ns, g.nb_sort, T, buf.hist, buf.perm);
  return hipGetLastError();
}

}  // namespace elsaa
