// k2_sort.hip -- stable sort of queries and keys by Sort-LSH bucket.
//
// The sparse branch groups similar tokens by sorting them on their hash code
// ("Two Efficient Attentions, One Denominator Problem", section "Two efficient
// branches can still be mis-scaled": the sparse branch keeps only selected
// high-similarity pairs).  For every (b, h) and separately for q and k, the
// permutation perm[rank] = original index orders tokens by (code, index): a
// stable counting sort.  Equal codes inside a round of 64 are found with one
// ballot per code bit and placed in lane order after those of earlier rounds
// and waves, so every element gets a unique, stable rank.
//
// A segment whose waves each hold at most 32 rounds of codes (N <= 32768 with
// 16 waves, LDS permitting) is sorted by one workgroup, in LDS: each wave
// loads its contiguous run of codes into registers at once, per-wave
// histograms, a bucket-major scan (first sorted position of every (bucket,
// wave)), the ranking pass, and the permutation written out in order.  Longer
// segments take three passes over tiles of 2048 codes:
//   1. per-tile bucket histogram (LDS integer atomics), stored bucket-major;
//   2. exclusive scan of the [bucket][tile] counts of each segment: the first
//      sorted rank of every (bucket, tile);
//   3. per tile, each wave ranks its 8 rounds of 64 codes in order.
// Integer-only, hence bit-exact and deterministic.
#include "elsaa_internal.hpp"

namespace elsaa {
namespace {

constexpr int kWaves = 4;
constexpr int kRounds = kSortTile / (kWaves * 64);  // 8

// Lanes of the wave that are valid and hold this lane's code (ns bits): one
// ballot per code bit, each folded in as same &= ~(ballot ^ my_bit_as_mask),
// one three-input bit operation per half (truth table 0x90: a & ~(b ^ c)).
__device__ __forceinline__ unsigned long long same_code_lanes(uint32_t code, bool valid, int ns) {
  const unsigned long long v = __ballot(valid);
  uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
  for (int bit = 0; bit < ns; ++bit) {
    const uint32_t m = static_cast<uint32_t>(__builtin_amdgcn_sbfe(static_cast<int>(code), bit, 1));  // 0 or ~0
    const unsigned long long bb = __ballot(m != 0u);
    lo = __builtin_amdgcn_bitop3_b32(lo, static_cast<uint32_t>(bb), m, 0x90);
    hi = __builtin_amdgcn_bitop3_b32(hi, static_cast<uint32_t>(bb >> 32), m, 0x90);
  }
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}

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
    const unsigned long long mask = same_code_lanes(code, valid, ns);
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

// One workgroup per segment (see the file comment).  Each wave holds the
// codes of its run (at most kSegRounds rounds of 64) in registers, loaded at
// once.  LDS: [W][nb] counters, W scan words, and the segment's permutation as
// 16-bit indices.
constexpr int kSegRounds = 32;
__global__ __launch_bounds__(1024) void elsaa_k2_sort_segment(const uint16_t *__restrict__ codes, int N,
                                                              int ns, int32_t *__restrict__ perm) {
  extern __shared__ uint32_t lds[];
  const int nb = 1 << ns;
  const int W = static_cast<int>(blockDim.x >> 6);
  uint32_t *cnt = lds;                                        // [W][nb]
  uint32_t *part = lds + W * nb;                              // [W]
  uint16_t *lperm = reinterpret_cast<uint16_t *>(part + W);   // [N]
  const long long s = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint16_t *c = codes + s * N;
  const int chunk = ((N + W - 1) / W + 63) / 64 * 64;  // at most kSegRounds * 64
  const int j_begin = wave * chunk < N ? wave * chunk : N;
  const int j_end = j_begin + chunk < N ? j_begin + chunk : N;
  const int rounds = (j_end - j_begin + 63) / 64;

  // code of element j_begin + 64 q + lane; 0xffffffff past the run
  uint32_t code[kSegRounds];
#pragma unroll
  for (int q = 0; q < kSegRounds; ++q) {
    const int j = j_begin + q * 64 + lane;
    code[q] = 0xffffffffu;
    if (q < rounds && j < j_end) code[q] = c[j];
  }
  for (int i = tid; i < W * nb; i += W * 64) cnt[i] = 0u;
  __syncthreads();
  uint32_t *wc = cnt + wave * nb;
#pragma unroll
  for (int q = 0; q < kSegRounds; ++q)
    if (q < rounds && code[q] != 0xffffffffu) atomicAdd(&wc[code[q]], 1u);
  __syncthreads();
  {  // bucket-major exclusive scan of the [bucket][wave] counts
    const int nthreads = W * 64;
    const int per = (nb + nthreads - 1) / nthreads;
    const int b_lo = tid * per < nb ? tid * per : nb;
    const int b_hi = b_lo + per < nb ? b_lo + per : nb;
    uint32_t sum = 0;
    for (int b = b_lo; b < b_hi; ++b)
      for (int w = 0; w < W; ++w) sum += cnt[w * nb + b];
    uint32_t run = block_exclusive_scan(sum, part, lane, wave);
    for (int b = b_lo; b < b_hi; ++b)
      for (int w = 0; w < W; ++w) {
        const uint32_t t = cnt[w * nb + b];
        cnt[w * nb + b] = run;
        run += t;
      }
  }
  __syncthreads();

  const unsigned long long lt = (1ull << lane) - 1ull;
#pragma unroll
  for (int q = 0; q < kSegRounds; ++q) {
    if (q < rounds) {
      const bool valid = code[q] != 0xffffffffu;
      const uint32_t cv = valid ? code[q] : 0u;
      const unsigned long long same = same_code_lanes(cv, valid, ns);
      // every lane of a group of equal codes reads the group's counter (one
      // address, a broadcast) and writes back the same advanced value, so no
      // leader lane and no shuffle is needed
      const uint32_t before = wc[cv];
      if (valid) {
        wc[cv] = before + static_cast<uint32_t>(__popcll(same));
        lperm[before + static_cast<uint32_t>(__popcll(same & lt))] = static_cast<uint16_t>(j_begin + q * 64 + lane);
      }
      // No wait between rounds: a wave's LDS accesses are carried out in
      // issue order, so the next round's read of a counter sees this round's
      // update, and the compiler keeps the (possibly aliasing) read after the
      // write.
    }
  }
  __syncthreads();
  int32_t *pm = perm + s * N;
  for (int i = tid; i < N; i += W * 64) pm[i] = lperm[i];
}

// Waves of the one-workgroup sort, or 0 when the segment does not fit (LDS,
// or more than kSegRounds rounds a wave).
int segment_sort_waves(const Geometry &g, size_t *lds) {
  if (g.N > 65536) return 0;
  constexpr size_t kLdsMax = 160 * 1024;
  for (int w = 16; w >= 1; w /= 2) {
    const size_t bytes = (static_cast<size_t>(w) * g.nb_sort + w) * 4 + static_cast<size_t>(g.N) * 2;
    if (bytes <= kLdsMax) {
      *lds = bytes;
      const int chunk = ((g.N + w - 1) / w + 63) / 64 * 64;
      return chunk <= kSegRounds * 64 ? w : 0;
    }
  }
  return 0;
}

}  // namespace

hipError_t launch_sort(const Geometry &g, const Buffers &buf, hipStream_t stream) {
  const int S = 2 * g.BH;
  size_t seg_lds = 0;
  const int seg_waves = segment_sort_waves(g, &seg_lds);
  if (seg_waves > 0) {
    hipLaunchKernelGGL(elsaa_k2_sort_segment, dim3(S), dim3(seg_waves * 64), seg_lds, stream, buf.scode, g.N,
                       g.ns, buf.perm);
    return hipGetLastError();
  }
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
