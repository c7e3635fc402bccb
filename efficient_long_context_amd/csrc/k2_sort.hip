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
//   3. per tile, each wave ranks its 8 rounds of 64 codes in order into the
//      tile's sorted order in LDS, and the tile writes it out in that order.
// Integer-only, hence bit-exact and deterministic.
#include "elsaa_internal.hpp"

namespace elsaa {
namespace {

constexpr int kWaves = 4;
constexpr int kRounds = kSortTile / (kWaves * 64);  // 8 rounds of 64 codes a wave

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

// Tiles of kW waves x kRounds rounds of 64 codes: 4 waves (2048 codes) for
// the Sort-LSH sort; the RACE build's tiled rank takes 16 (8192 codes) when
// 16 waves' counters fit 64 KB of LDS.
template <typename CT, int kW>
__global__ __launch_bounds__(kW * 64) void elsaa_k2_sort_hist(const CT *__restrict__ codes, int N, int nb,
                                                              int T, uint32_t *__restrict__ hist) {
  constexpr int kTile = kW * kRounds * 64;
  extern __shared__ uint32_t h[];
  const int tile = blockIdx.x;
  const long long s = blockIdx.y;
  for (int b = threadIdx.x; b < nb; b += kW * 64) h[b] = 0;
  __syncthreads();
  const CT *c = codes + s * N;
  const int base = tile * kTile;
  for (int e = threadIdx.x; e < kTile; e += kW * 64) {
    const int i = base + e;
    if (i < N) atomicAdd(&h[c[i]], 1u);
  }
  __syncthreads();
  uint32_t *out = hist + s * static_cast<long long>(nb) * T;
  for (int b = threadIdx.x; b < nb; b += kW * 64) out[static_cast<long long>(b) * T + tile] = h[b];
}

// In-place exclusive scan of the M = nb * T counts of each segment, one
// 1024-thread block per segment, in chunks of 1024 * kScanPer counts: each
// thread owns kScanPer consecutive counts of a chunk, requested at once as
// 16-byte pieces (so the chunk's loads are all in flight together), then a
// block scan of the per-thread sums and a running carry across chunks.
constexpr int kScanPer = 64;
__global__ __launch_bounds__(1024) void elsaa_k2_sort_scan(uint32_t *__restrict__ hist, long long M) {
  __shared__ uint32_t part[16];
  uint32_t *p = hist + static_cast<long long>(blockIdx.x) * M;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t carry = 0;
  for (long long c0 = 0; c0 < M; c0 += 1024ll * kScanPer) {
    const long long lo = c0 + static_cast<long long>(tid) * kScanPer;
    uint32_t v[kScanPer];
    // 16-byte pieces when M is a multiple of 4 (every segment's counts then
    // start 16-byte aligned); otherwise, and past the end, element by element
    if (lo + kScanPer <= M && (M & 3) == 0) {
#pragma unroll
      for (int e = 0; e < kScanPer; e += 4) {
        const u32x4 x = *reinterpret_cast<const u32x4 *>(p + lo + e);
        v[e] = x[0]; v[e + 1] = x[1]; v[e + 2] = x[2]; v[e + 3] = x[3];
      }
    } else {
#pragma unroll
      for (int e = 0; e < kScanPer; ++e) v[e] = lo + e < M ? p[lo + e] : 0u;
    }
    uint32_t sum = 0;
#pragma unroll
    for (int e = 0; e < kScanPer; ++e) sum += v[e];
    uint32_t run = block_exclusive_scan(sum, part, lane, wave);
    if (tid == 1023) part[0] = run + sum;  // the chunk's total (after the scan's reads of part)
    run += carry;
#pragma unroll
    for (int e = 0; e < kScanPer; ++e) {
      const uint32_t c = v[e];
      v[e] = run;
      run += c;
    }
    if (lo + kScanPer <= M && (M & 3) == 0) {
#pragma unroll
      for (int e = 0; e < kScanPer; e += 4)
        *reinterpret_cast<u32x4 *>(p + lo + e) = u32x4{v[e], v[e + 1], v[e + 2], v[e + 3]};
    } else {
#pragma unroll
      for (int e = 0; e < kScanPer; ++e)
        if (lo + e < M) p[lo + e] = v[e];
    }
    __syncthreads();
    carry += part[0];
    __syncthreads();  // part is reused by the next chunk's scan
  }
}

// Per tile: each wave ranks its 8 rounds of 64 codes in order into the
// tile's own sorted order (the tile's codes by bucket, stable), staged in
// LDS with each slot's position in the segment's order, then the tile writes
// its slots in order: consecutive lanes write consecutive positions of a
// bucket's run, instead of 64 scattered positions per store.  Every lane of a
// group of equal codes reads the group's counter (one address, a broadcast)
// and writes back the same advanced value, adding its rank inside the group;
// a wave's LDS accesses are carried out in issue order, so the next round's
// read sees the update without a wait.
template <int kW>
constexpr size_t scatter_lds_bytes(int nb) {
  return (static_cast<size_t>(kW) * nb + 16 + nb + 2 * kW * kRounds * 64) * 4;
}

// kBallot: stable ranks from the ballots (the Sort-LSH sort, whose
// permutation is part of the method); otherwise each element takes the next
// slot of its (wave, bucket) counter from an LDS atomic that returns the old
// value, one instruction a round instead of one ballot per code bit: a fixed
// order run to run (the RACE build needs only a deterministic order of each
// bucket's keys).
template <typename CT, typename PT, int kW, bool kBallot>
__global__ __launch_bounds__(kW * 64) void elsaa_k2_sort_scatter(const CT *__restrict__ codes, int N, int ns,
                                                                 int nb, int T,
                                                                 const uint32_t *__restrict__ offs,
                                                                 PT *__restrict__ perm) {
  constexpr int kTile = kW * kRounds * 64;
  extern __shared__ uint32_t lds[];
  uint32_t *cnt = lds;                  // [kW][nb] running tile-local sorted slots
  uint32_t *part = cnt + kW * nb;       // [16] scan scratch
  uint32_t *delta = part + 16;          // [nb] segment position minus tile slot, per bucket
  uint32_t *spos = delta + nb;          // [kTile] segment position of each slot
  uint32_t *sidx = spos + kTile;        // [kTile] element of each slot
  const int tile = blockIdx.x;
  const long long s = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const CT *c = codes + s * N;
  const uint32_t *o = offs + s * static_cast<long long>(nb) * T;
  PT *pm = perm + s * N;
  const int wbase = tile * kTile + wave * (kRounds * 64);
  uint32_t *wc = cnt + wave * nb;

  uint32_t code[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int i = wbase + r * 64 + lane;
    code[r] = i < N ? static_cast<uint32_t>(c[i]) : 0xffffffffu;
  }
  for (int b = tid; b < kW * nb; b += kW * 64) cnt[b] = 0;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kRounds; ++r)
    if (code[r] != 0xffffffffu) atomicAdd(&wc[code[r]], 1u);
  __syncthreads();
  {  // tile-local bucket-major exclusive scan of the [bucket][wave] counts
    constexpr int kThreads = kW * 64;
    const int per = (nb + kThreads - 1) / kThreads;
    const int b_lo = tid * per < nb ? tid * per : nb;
    const int b_hi = b_lo + per < nb ? b_lo + per : nb;
    uint32_t sum = 0;
    for (int b = b_lo; b < b_hi; ++b)
      for (int w = 0; w < kW; ++w) sum += cnt[w * nb + b];
    uint32_t run = block_exclusive_scan(sum, part, lane, wave);
    for (int b = b_lo; b < b_hi; ++b) {
      delta[b] = o[static_cast<long long>(b) * T + tile] - run;  // modulo 2^32
      for (int w = 0; w < kW; ++w) {
        const uint32_t t = cnt[w * nb + b];
        cnt[w * nb + b] = run;
        run += t;
      }
    }
  }
  __syncthreads();

  const unsigned long long lt = (1ull << lane) - 1ull;
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const bool valid = code[r] != 0xffffffffu;
    const uint32_t cv = valid ? code[r] : 0u;
    uint32_t slot;
    if constexpr (kBallot) {
      const unsigned long long same = same_code_lanes(cv, valid, ns);
      const uint32_t before = wc[cv];
      if (valid) wc[cv] = before + static_cast<uint32_t>(__popcll(same));
      slot = before + static_cast<uint32_t>(__popcll(same & lt));
    } else {
      slot = valid ? atomicAdd(&wc[cv], 1u) : 0u;
    }
    if (valid) {
      sidx[slot] = static_cast<uint32_t>(wbase + r * 64 + lane);
      spos[slot] = slot + delta[cv];
    }
  }
  __syncthreads();
  const int valid_slots = N - tile * kTile < kTile ? N - tile * kTile : kTile;
  for (int i = tid; i < valid_slots; i += kW * 64) pm[spos[i]] = static_cast<PT>(sidx[i]);
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

bool sort_is_tiled(const Geometry &g) {
  size_t lds = 0;
  return segment_sort_waves(g, &lds) == 0;
}

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
  hipLaunchKernelGGL((elsaa_k2_sort_hist<uint16_t, kWaves>), dim3(T, S), dim3(kWaves * 64), g.nb_sort * 4, stream,
                     buf.scode, g.N, g.nb_sort, T, buf.hist);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(elsaa_k2_sort_scan, dim3(S), dim3(1024), 0, stream, buf.hist,
                     static_cast<long long>(g.nb_sort) * T);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((elsaa_k2_sort_scatter<uint16_t, int32_t, kWaves, true>), dim3(T, S), dim3(kWaves * 64),
                     scatter_lds_bytes<kWaves>(g.nb_sort), stream, buf.scode, g.N, g.ns, g.nb_sort, T, buf.hist,
                     buf.perm);
  return hipGetLastError();
}

namespace {
// Waves per tile of the tiled rank: 16 when their counters fit 64 KB of LDS.
int tiled_waves(int bits) { return (1 << bits) <= 1024 ? 16 : kWaves; }

template <typename CT, typename PT, int kW>
hipError_t tiled_sort_t(const void *codes, int N, int bits, long long S, uint32_t *hist, void *perm,
                        hipStream_t stream) {
  const int nb = 1 << bits;
  const int T = tiled_sort_tiles(N, bits);
  hipLaunchKernelGGL((elsaa_k2_sort_hist<CT, kW>), dim3(T, static_cast<unsigned>(S)), dim3(kW * 64), nb * 4,
                     stream, static_cast<const CT *>(codes), N, nb, T, hist);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(elsaa_k2_sort_scan, dim3(static_cast<unsigned>(S)), dim3(1024), 0, stream, hist,
                     static_cast<long long>(nb) * T);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((elsaa_k2_sort_scatter<CT, PT, kW, false>), dim3(T, static_cast<unsigned>(S)), dim3(kW * 64),
                     scatter_lds_bytes<kW>(nb), stream, static_cast<const CT *>(codes), N, bits, nb, T, hist,
                     static_cast<PT *>(perm));
  return hipGetLastError();
}

template <typename CT, typename PT>
hipError_t tiled_sort_w(const void *codes, int N, int bits, long long S, uint32_t *hist, void *perm,
                        hipStream_t stream) {
  return tiled_waves(bits) == 16 ? tiled_sort_t<CT, PT, 16>(codes, N, bits, S, hist, perm, stream)
                                 : tiled_sort_t<CT, PT, kWaves>(codes, N, bits, S, hist, perm, stream);
}
}  // namespace

int tiled_sort_tiles(int N, int bits) {
  const int tile = tiled_waves(bits) * kRounds * 64;
  return (N + tile - 1) / tile;
}

hipError_t launch_tiled_sort(const void *codes, int code_bytes, int N, int bits, long long S, uint32_t *hist,
                             void *perm, int index_bytes, hipStream_t stream) {
  if (code_bytes == 1)
    return index_bytes == 2 ? tiled_sort_w<uint8_t, uint16_t>(codes, N, bits, S, hist, perm, stream)
                            : tiled_sort_w<uint8_t, int32_t>(codes, N, bits, S, hist, perm, stream);
  return index_bytes == 2 ? tiled_sort_w<uint16_t, uint16_t>(codes, N, bits, S, hist, perm, stream)
                          : tiled_sort_w<uint16_t, int32_t>(codes, N, bits, S, hist, perm, stream);
}

}  // namespace elsaa
