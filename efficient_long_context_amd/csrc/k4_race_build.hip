// k4_race_build.hip -- RACE tables: per-bucket value sums and key counts.
//
// The low-rank branch compresses the keys into hash-bucket summaries ("Two
// Efficient Attentions, One Denominator Problem", section "Two efficient
// branches can still be mis-scaled"): for every table l and bucket b,
//   count[l][b] = #{keys j : code_l(k_j) = b},   sum[l][b][:] = sum of v_j over them.
//
// Built as a segmented reduction over codes sorted per table, in two kernels:
//   rank    one workgroup per (b, h, table): a counting sort of the table's N
//           key codes, giving every bucket's keys as one contiguous run of the
//           table's permutation, the run starts and the counts;
//   gather  one wave per (b, h, table, part of the positions): the wave sums
//           the value rows of whole buckets, in run order, in registers and
//           writes each bucket row once.
// No floating-point atomics (LDS float atomics are slow on gfx950 and would make
// the summation order vary): every bucket is summed by one wave in run order,
// so the tables are deterministic.  Heavy buckets (repeated tokens) are just
// long runs.
#include "elsaa_internal.hpp"

namespace elsaa {
namespace {


// ------------------------------------------------------------ shared parts --
// A lane's 16-byte piece of a value row: kLanesPerRow lanes share a row, so
// one load instruction fetches kRowsPerLoad rows (8 for bfloat16 rows of 64
// columns), and a lane accumulates kCols columns of its row group.
template <typename VT, int D> struct Piece {
  static constexpr int kCols = 16 / static_cast<int>(sizeof(VT));
  static constexpr int kLanesPerRow = D / kCols;
  static constexpr int kRowsPerLoad = 64 / kLanesPerRow;
  static constexpr int kRowBytes = D * static_cast<int>(sizeof(VT));
  static __device__ __forceinline__ void add(u32x4 r, float *a, const Bf16Adder &ad) {
    if constexpr (sizeof(VT) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[2 * e] = ad.lo(a[2 * e], r[e]);
        a[2 * e + 1] = ad.hi(a[2 * e + 1], r[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] += __uint_as_float(r[e]);
    }
  }
};

// Lanes l and l ^ m (m a multiple of kLPR below 64) hold partial sums of the
// same kCols columns.  Sums them, leaving each lane kCols / (64 / kLPR) of the
// column totals: one exchange per lane bit halves what a lane holds (bit 4 and
// bit 5 with the gfx950 permlane swaps, whose two outputs are the lane's own
// and its partner's value of the pair's even or odd member; bit 3 with a DPP
// row rotation by 8).  The lane keeps column transposed_column(m) in out[m].
template <int kCols, int kLPR>
__device__ __forceinline__ void lane_group_transpose_sum(const float (&in)[kCols],
                                                         float (&out)[kCols * kLPR / 64], int lane) {
  static_assert(kLPR == 8 || kLPR == 16 || kLPR == 32, "lane group width");
  float v[kCols];
#pragma unroll
  for (int k = 0; k < kCols; ++k) v[k] = in[k];
  int n = kCols;
  if constexpr (kLPR <= 16) {  // lane bit 4: keep index 2j + bit4
#pragma unroll
    for (int j = 0; j < kCols / 2; ++j) {
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[2 * j]), __float_as_uint(v[2 * j + 1]),
                                                      false, false);
      v[j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    n /= 2;
  }
  {  // lane bit 5: keep index 2j + bit5
#pragma unroll
    for (int j = 0; j < kCols / 2; ++j) {
      if (2 * j + 1 < n) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[2 * j]),
                                                        __float_as_uint(v[2 * j + 1]), false, false);
        v[j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
      }
    }
    n /= 2;
  }
  if constexpr (kLPR <= 8) {  // lane bit 3: keep index 2j + bit3
    const bool odd = (lane >> 3) & 1;
#pragma unroll
    for (int j = 0; j < kCols / 2; ++j) {
      if (2 * j + 1 < n) {
        const float keep = odd ? v[2 * j + 1] : v[2 * j];
        const float send = odd ? v[2 * j] : v[2 * j + 1];
        v[j] = keep + __uint_as_float(__builtin_amdgcn_mov_dpp(__float_as_uint(send), 0x128, 0xf, 0xf, false));
      }
    }
    n /= 2;
  }
#pragma unroll
  for (int m = 0; m < kCols * kLPR / 64; ++m) out[m] = v[m];
}

// Column (of the lane's kCols) whose total lane_group_transpose_sum leaves in
// out[m]: the kept indices compose bit4, then bit5, then bit3 of the lane.
template <int kCols, int kLPR>
__device__ __forceinline__ int transposed_column(int m, int lane) {
  int k = m;
  if constexpr (kLPR <= 8) k = 2 * k + ((lane >> 3) & 1);
  k = 2 * k + ((lane >> 5) & 1);
  if constexpr (kLPR <= 16) k = 2 * k + ((lane >> 4) & 1);
  return k;
}

// ----------------------------------------------------------- rank + gather --
//   rank    one workgroup per (b, h, table): a counting sort of the table's N
//           key codes (read contiguously: key codes are stored table-major)
//           with per-wave LDS histograms, a bucket-major scan, then each key
//           taking the next slot of its (wave, bucket) counter from an LDS
//           atomic that returns the old value.  The sorted key indices are
//           staged in LDS (N <= 65536) and written in order; the run start of
//           every bucket and the bucket counts go out too.
//   gather  one wave per (b, h, table, part of the positions): the wave owns
//           the buckets whose run starts in its part, stages their key
//           indices in LDS and sums the value rows bucket by bucket: 16-byte
//           lane pieces (8 rows of 64 bfloat16 columns per load), two batches
//           of 4 loads in flight and none past the part's end (every load
//           instruction costs the texture addresser the same ~20 cycles,
//           whether its lanes are in range or not, and that unit bounds this
//           kernel), a scalar test per load for the common case of a load
//           inside one bucket, and at a bucket end a transposing lane
//           reduction whose column sums are stored as the table row.
//           Waves of one (b, h) are consecutive and so share an XCD's L2,
//           which then holds the value rows its tables gather.
//   The sorted key indices are 16-bit (PT = uint16_t) whenever N <= 65536,
//   halving the permutation's write here and its read in the gather.
// Gather part p (positions from lo_p = N p / parts) owns the buckets whose
// run starts in [lo_p, lo_{p+1}); its first one is the first bucket starting
// at or after lo_p: bucket b + 1, at position `end`, for every lo_p in
// (start, end] of a nonempty bucket b.  Entry 0 (bucket 0, position 0) and
// entry `parts` (2^P, N) are written separately.
__device__ __forceinline__ void part_entries(int b, uint32_t start, uint32_t end, int N, int parts,
                                             int32_t *__restrict__ rp2) {
  if (end <= start) return;
  long long pp = static_cast<long long>(start) * parts / N;
  while (pp < parts && static_cast<long long>(N) * pp / parts <= static_cast<long long>(start)) ++pp;
  for (; pp < parts && static_cast<long long>(N) * pp / parts <= static_cast<long long>(end); ++pp) {
    rp2[2 * pp] = b + 1;
    rp2[2 * pp + 1] = static_cast<int32_t>(end);
  }
}

template <typename CT>
__global__ __launch_bounds__(1024) void elsaa_k4_race_rank(
    const CT *__restrict__ kcodes, int N, int L, int BH, int P, long long rows, int parts,
    uint16_t *__restrict__ rperm, int32_t *__restrict__ rstart, int32_t *__restrict__ rpart,
    float *__restrict__ tcnt, uint32_t *__restrict__ hash_flagged) {
  extern __shared__ uint32_t lds[];
  if (blockIdx.x == 0 && threadIdx.x == 0) *hash_flagged = 0u;  // the fix-up has run
  const int nb = 1 << P;
  const int W = static_cast<int>(blockDim.x >> 6);
  uint32_t *cnt = lds;           // [W][nb] counts, then running offsets
  uint32_t *part = lds + W * nb;  // [W] scan
  // [N] (N <= 65536), 16-byte aligned for the vector copy-out
  uint16_t *lperm = reinterpret_cast<uint16_t *>(lds + (W * nb + W + 3) / 4 * 4);
  const long long unit = blockIdx.x;  // (b, h) * L + table
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long long bh = unit / L;
  const int l = static_cast<int>(unit % L);
  const CT *c = kcodes + static_cast<long long>(l) * rows + bh * N;  // code of key j at c[j]
  const int chunk = ((N + W - 1) / W + 63) / 64 * 64;
  const int j_begin = wave * chunk < N ? wave * chunk : N;
  const int j_end = j_begin + chunk < N ? j_begin + chunk : N;

  // The wave's codes in 16-byte pieces (kVec codes each): piece p of a batch
  // starting at jb is codes jb + (64 p + lane) kVec .. +kVec-1, so each piece
  // load of the wave reads one contiguous kilobyte.  N is a multiple of 64
  // (the chunk is), so every piece lies wholly inside or outside the run and
  // is 16-byte aligned.  The first batch stays in registers for the ranking
  // pass (all of the run when it fits).
  constexpr int kVec = 16 / static_cast<int>(sizeof(CT));
  constexpr int kPieces = 4;
  constexpr int kBatch = 64 * kPieces * kVec;
  auto load_batch = [&](int jb, u32x4 (&pc)[kPieces]) {
#pragma unroll
    for (int p = 0; p < kPieces; ++p) {
      const int j = jb + (p * 64 + lane) * kVec;
      pc[p] = (u32x4){0u, 0u, 0u, 0u};
      if (j < j_end) pc[p] = *reinterpret_cast<const u32x4 *>(c + j);
    }
  };
  auto code_of = [](const u32x4 &pc, int e) -> uint32_t {
    constexpr int kBits = 8 * static_cast<int>(sizeof(CT));
    const uint32_t word = pc[e * kBits / 32];
    return (word >> ((e * kBits) % 32)) & ((1u << kBits) - 1u);
  };
  // calls f(code, j) for every code of the batch at jb inside the run
  auto for_batch = [&](int jb, const u32x4 (&pc)[kPieces], auto &&f) {
#pragma unroll
    for (int p = 0; p < kPieces; ++p) {
      const int j = jb + (p * 64 + lane) * kVec;
      if (j < j_end) {
#pragma unroll
        for (int e = 0; e < kVec; ++e) f(code_of(pc[p], e), j + e);
      }
    }
  };

  for (int i = tid; i < W * nb; i += W * 64) cnt[i] = 0u;
  u32x4 first[kPieces];
  if (j_begin < j_end) load_batch(j_begin, first);
  __syncthreads();
  uint32_t *wc = cnt + wave * nb;
  auto count = [&](uint32_t code, int) { atomicAdd(&wc[code], 1u); };
  if (j_begin < j_end) for_batch(j_begin, first, count);
  for (int jb = j_begin + kBatch; jb < j_end; jb += kBatch) {
    u32x4 pc[kPieces];
    load_batch(jb, pc);
    for_batch(jb, pc, count);
  }
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
    int32_t *rs = rstart + unit * (nb + 1);
    int32_t *rp2 = rpart + unit * (parts + 1) * 2;
    for (int b = b_lo; b < b_hi; ++b) {
      rs[b] = static_cast<int32_t>(run);
      const uint32_t r0 = run;
      for (int w = 0; w < W; ++w) {
        const uint32_t t = cnt[w * nb + b];
        cnt[w * nb + b] = run;
        run += t;
      }
      tcnt[unit * nb + b] = static_cast<float>(run - r0);
      part_entries(b, r0, run, N, parts, rp2);
    }
    if (tid == 0) {
      rs[nb] = N;
      rp2[0] = 0;  // part 0 starts at bucket 0, position 0
      rp2[1] = 0;
      rp2[2 * parts] = nb;  // end of the last part
      rp2[2 * parts + 1] = N;
    }
  }
  __syncthreads();
  // sorted key indices: staged in LDS and written out in order (coalesced)
  uint16_t *rp = rperm + (static_cast<long long>(l) * BH + bh) * N;
  auto place = [&](uint32_t code, int j) {
    const uint32_t pos = atomicAdd(&wc[code], 1u);
    lperm[pos] = static_cast<uint16_t>(j);
  };
  if (j_begin < j_end) for_batch(j_begin, first, place);
  for (int jb = j_begin + kBatch; jb < j_end; jb += kBatch) {
    u32x4 pc[kPieces];
    load_batch(jb, pc);
    for_batch(jb, pc, place);
  }
  __syncthreads();
  // 8 indices a 16-byte piece (N is a multiple of 64)
  for (int i = tid; i < N / 8; i += W * 64)
    reinterpret_cast<u32x4 *>(rp)[i] = reinterpret_cast<const u32x4 *>(lperm)[i];
}

// Run table of the tiled rank (segments too long for one workgroup's LDS):
// the tiled sort has left the scanned [bucket][tile] counts of segment
// (table l, (b, h)), whose tile-0 word of bucket b is that bucket's run start.
// One workgroup per (b, h, table) writes the run starts, the counts and the
// gather's part table.
__global__ __launch_bounds__(256) void elsaa_k4_race_runs(const uint32_t *__restrict__ offs, int N, int L, int BH,
                                                          int P, int T, int parts, int32_t *__restrict__ rstart,
                                                          int32_t *__restrict__ rpart, float *__restrict__ tcnt,
                                                          uint32_t *__restrict__ hash_flagged) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *hash_flagged = 0u;  // the fix-up has run
  const int nb = 1 << P;
  const long long unit = blockIdx.x;  // (b, h) * L + table
  const long long bh = unit / L;
  const int l = static_cast<int>(unit % L);
  const uint32_t *o = offs + (static_cast<long long>(l) * BH + bh) * nb * T;
  int32_t *rs = rstart + unit * (nb + 1);
  int32_t *rp2 = rpart + unit * (parts + 1) * 2;
  for (int b = threadIdx.x; b < nb; b += 256) {
    const uint32_t start = o[static_cast<long long>(b) * T];
    const uint32_t end = b + 1 < nb ? o[static_cast<long long>(b + 1) * T] : static_cast<uint32_t>(N);
    rs[b] = static_cast<int32_t>(start);
    tcnt[unit * nb + b] = static_cast<float>(end - start);
    part_entries(b, start, end, N, parts, rp2);
  }
  if (threadIdx.x == 0) {
    rs[nb] = N;
    rp2[0] = 0;
    rp2[1] = 0;
    rp2[2 * parts] = nb;
    rp2[2 * parts + 1] = N;
  }
}

constexpr int kGatherWaves = 4;       // waves per gather workgroup
constexpr int kGatherStage = 512;     // key indices a wave stages in LDS at once
constexpr int kGatherSlack = 128;     // staged entries read past the end by the last batch

// A wave sums D columns of rows of DS columns: with DS = 2 D the (b, h)'s
// work is done in two column halves, each half's passes (all tables) reading
// half of every row, so the rows the half's in-flight waves touch are half
// as many bytes (at d = 128, 4 MB per 8 MB token block: one XCD's L2).
template <typename VT, int D, typename PT, typename TS, int DS>
__global__ __launch_bounds__(kGatherWaves * 64) void elsaa_k4_race_gather(
    const VT *__restrict__ v, const PT *__restrict__ rperm, const int32_t *__restrict__ rstart,
    const int32_t *__restrict__ rpart, int N, int L, int BH, int P, int parts, long long waves_total,
    int xcd_local, TS *__restrict__ tsum) {
  using PC = Piece<VT, D>;
  constexpr int kCols = PC::kCols, kLPR = PC::kLanesPerRow;
  constexpr int kRPI = PC::kRowsPerLoad;
  constexpr int kI = 4;              // load instructions per batch
  constexpr int kBP = kI * kRPI;     // positions per batch
  // the stage holds key indices as stored (PT), from a 16-byte boundary of
  // the permutation at or below the stage's first position
  constexpr int kE = 16 / static_cast<int>(sizeof(PT));  // key indices per 16-byte piece
  constexpr int kStageCap = kGatherStage + kE + kGatherSlack;
  constexpr int kStageLoads = ((kGatherStage + 2 * kE - 2) / kE + 1 + 63) / 64;
  static_assert(kBP + kE <= kGatherSlack, "a stage's last batch reads inside the stage");
  __shared__ __align__(16) PT stage_all[kGatherWaves][kStageCap];
  const int nb = 1 << P;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  // xcd_local: consecutive workgroups (one (b, h) after another) on one XCD,
  // whose L2 then holds that (b, h)'s value rows; otherwise workgroups in
  // dispatch order, so every XCD works on the same (b, h) at once and its
  // value rows (too many for one L2) stay in the last-level cache
  const long long wg = xcd_local ? xcd_logical_block(blockIdx.x, gridDim.x) : static_cast<long long>(blockIdx.x);
  const long long u = wg * kGatherWaves + wave;
  if (u >= waves_total) return;  // whole wave; the kernel has no barriers
  PT *stage = stage_all[wave];
  static_assert(DS == D || DS == 2 * D, "whole rows or column halves");
  const int prt = static_cast<int>(u % parts);
  // work order (b, h), column half, table, part
  const long long rest = u / parts;
  const int half = DS == D ? 0 : static_cast<int>((rest / L) % 2);
  const long long bh = DS == D ? rest / L : rest / (2ll * L);
  const long long unit = bh * L + rest % L;  // (b, h) * L + table
  const int32_t *rs = rstart + unit * (nb + 1);
  const PT *rp = rperm + (static_cast<long long>(unit % L) * BH + bh) * N;
  TS *ts = tsum + unit * nb * static_cast<long long>(DS) + half * D;

  // owned buckets [b0, b1) and their positions [p_lo, p_hi), from the part
  // table the rank kernel wrote (the buckets whose run starts in this part's
  // positions; the last part also owns the empty buckets that start at N)
  const int2 *pt = reinterpret_cast<const int2 *>(rpart) + unit * (parts + 1) + prt;
  const int2 here = pt[0], next = pt[1];
  const int b0 = __builtin_amdgcn_readfirstlane(here.x);
  const int p_lo = __builtin_amdgcn_readfirstlane(here.y);
  const int b1 = __builtin_amdgcn_readfirstlane(next.x);
  const int p_hi = __builtin_amdgcn_readfirstlane(next.y);
  if (b0 >= b1) return;

  const int cc = lane % kLPR;       // column piece
  const int my_off = lane / kLPR;   // this lane's row within a load
  const Bf16Adder adder;
  int b = b0;
  // run end of bucket bk: a wave-uniform (scalar) load, waited on the scalar
  // counter, so a bucket end does not wait for the value rows in flight
  auto end_of = [&](int bk) -> int { return __builtin_amdgcn_readfirstlane(rs[bk + 1]); };
  int bend = end_of(b0);
  float a[kCols];
#pragma unroll
  for (int k = 0; k < kCols; ++k) a[k] = 0.0f;
  // bucket b is complete: transposing lane reduction, then the lane's column
  // sums go straight to the table row
  auto flush = [&]() {
    float r[kCols / kRPI];
    lane_group_transpose_sum<kCols, kLPR>(a, r, lane);
#pragma unroll
    for (int m = 0; m < kCols / kRPI; ++m)
      ts[b * static_cast<long long>(DS) + cc * kCols + transposed_column<kCols, kLPR>(m, lane)] =
          Elem<TS>::store_val(r[m]);
#pragma unroll
    for (int k = 0; k < kCols; ++k) a[k] = 0.0f;
  };
  if (p_lo == p_hi) {  // only empty buckets
    for (; b < b1; ++b) flush();
    return;
  }
  const __amdgpu_buffer_rsrc_t vrs =
      make_rsrc(v + bh * N * static_cast<long long>(DS) + half * D,
                static_cast<uint32_t>(N) * (PC::kRowBytes * (DS / D)) - half * PC::kRowBytes);
  const uint32_t cbyte = static_cast<uint32_t>(cc) * 16u;
  for (int s0 = p_lo; s0 < p_hi; s0 += kGatherStage) {
    const int s1 = s0 + kGatherStage < p_hi ? s0 + kGatherStage : p_hi;
    // stage the key indices of positions [s0a, s1) in 16-byte pieces, every
    // load issued before the first store (entries past s1 are stale and never
    // used; N is a multiple of kE, so no piece crosses the end of the
    // permutation)
    const int s0a = s0 - s0 % kE;
    {
      u32x4 pcs[kStageLoads];
#pragma unroll
      for (int t = 0; t < kStageLoads; ++t) {
        const int pos = s0a + (t * 64 + lane) * kE;
        pcs[t] = (u32x4){0u, 0u, 0u, 0u};
        if (pos < s1) pcs[t] = *reinterpret_cast<const u32x4 *>(rp + pos);
      }
#pragma unroll
      for (int t = 0; t < kStageLoads; ++t) {
        const int pos = s0a + (t * 64 + lane) * kE;
        if (pos < s1) *reinterpret_cast<u32x4 *>(stage + (pos - s0a)) = pcs[t];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    // positions at or past s1 (in the stage's last batch) load from an offset
    // past the buffer's end, which reads zero and fetches nothing
    auto load_batch = [&](int pbase, u32x4 (&r)[kI]) {
      uint32_t off[kI];
      const PT *lp = stage + (pbase - s0a) + my_off;
#pragma unroll
      for (int i = 0; i < kI; ++i)
        off[i] = static_cast<uint32_t>(lp[i * kRPI]) * (PC::kRowBytes * (DS / D)) + cbyte;
#pragma unroll
      for (int i = 0; i < kI; ++i) off[i] = pbase + i * kRPI + my_off < s1 ? off[i] : 0x80000000u;
#pragma unroll
      for (int i = 0; i < kI; ++i)
        r[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, off[i], 0, 0));
    };
    auto consume = [&](int pbase, const u32x4 (&r)[kI]) {
#pragma unroll
      for (int i = 0; i < kI; ++i) {
        const int p = pbase + i * kRPI;
        const int pe = p + kRPI < s1 ? p + kRPI : s1;
        const int my = p + my_off;
        const int stop0 = pe < bend ? pe : bend;
        if (my < stop0) PC::add(r[i], a, adder);
        if (pe >= bend && p < s1) {
          int cur = stop0;
          do {
            if (cur == bend) {
              flush();
              ++b;
              bend = b < b1 ? end_of(b) : 0x7fffffff;
            }
            const int stop = pe < bend ? pe : bend;
            if (my >= cur && my < stop) PC::add(r[i], a, adder);
            cur = stop;
          } while (cur < pe || cur == bend);
        }
      }
    };
    // two batches in flight and none loaded past the stage's end: the loop
    // runs while batches k, k + 1 and k + 2 all exist, and the last one or
    // two batches are consumed after it (straight-line code, so every wait
    // covers exactly the batch it precedes)
    const int nbat = (s1 - s0 + kBP - 1) / kBP;
    u32x4 ra[kI], rb[kI];
    load_batch(s0, ra);
    int k = 0;
    for (; k + 2 < nbat; k += 2) {
      load_batch(s0 + (k + 1) * kBP, rb);
      consume(s0 + k * kBP, ra);
      load_batch(s0 + (k + 2) * kBP, ra);
      consume(s0 + (k + 1) * kBP, rb);
    }
    if (nbat - k == 2) {
      load_batch(s0 + (k + 1) * kBP, rb);
      consume(s0 + k * kBP, ra);
      consume(s0 + (k + 1) * kBP, rb);
    } else {
      consume(s0 + k * kBP, ra);
    }
    // the stage may be overwritten only after every lane has read it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  }
}

// Token-blocked build: the tables of (b, h) are the sums over its blocks,
// taken in block order, of the blocks' binary32 partial tables.  Threads
// below n4 sum four columns of one table row each; the next nc threads one
// count each.
template <typename VT>
__global__ __launch_bounds__(256) void elsaa_k4_race_blocks_sum(const float *__restrict__ psum,
                                                               const float *__restrict__ pcnt, int blocks,
                                                               long long row_elems, long long cnt_elems,
                                                               long long n4, long long nc, VT *__restrict__ tsum,
                                                               float *__restrict__ tcnt) {
  const long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n4) {
    // row_elems = L 2^P D values per (b, h), a multiple of 4
    const long long e = i * 4;
    const long long bh = e / row_elems;
    const float *p = psum + bh * blocks * row_elems + (e - bh * row_elems);
    float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int t = 0; t < blocks; ++t) {
      float x[4];
      Elem<float>::load4(p + t * row_elems, x);
#pragma unroll
      for (int m = 0; m < 4; ++m) a[m] += x[m];
    }
    Elem<VT>::store4(tsum + e, a);
  } else if (i < n4 + nc) {
    const long long e = i - n4;
    const long long bh = e / cnt_elems;
    const float *p = pcnt + bh * blocks * cnt_elems + (e - bh * cnt_elems);
    float a = 0.0f;
    for (int t = 0; t < blocks; ++t) a += p[t * cnt_elems];
    tcnt[e] = a;
  }
}

}  // namespace


namespace {

// One workgroup per (b, h, table) ranks the table's codes in LDS when its
// counters and the segment's 16-bit permutation fit with two workgroups per
// CU, else with one (then with as many waves as fit, up to 16); returns its
// waves, or 0 for the tiled rank.
int staged_rank_waves(const Geometry &g) {
  if (g.N > 65536) return 0;
  const int nb = g.nb_race;
  int waves = 16384 / nb;  // LDS counters: waves * nb * 4 bytes <= 64 KB
  waves = waves < 1 ? 1 : (waves > 16 ? 16 : waves);
  constexpr size_t kRankLdsTwoPerCu = 78 * 1024, kRankLdsOnePerCu = 150 * 1024;
  auto rank_lds = [&](int w) {  // + 16: the staged indices start 16-byte aligned
    return (static_cast<size_t>(w) * nb + w) * 4 + static_cast<size_t>(g.N) * 2 + 16;
  };
  int w2 = waves;
  while (w2 > 4 && rank_lds(w2) > kRankLdsTwoPerCu) w2 /= 2;
  if (rank_lds(w2) <= kRankLdsTwoPerCu) return w2;
  int w1 = 16;
  while (w1 > 4 && rank_lds(w1) > kRankLdsOnePerCu) w1 /= 2;
  return rank_lds(w1) > kRankLdsOnePerCu ? 0 : w1;
}

template <typename PT>
hipError_t launch_race_build_pt(const Geometry &g, const RaceBuildIO &io, hipStream_t stream) {
  const int nb = g.nb_race;
  PT *rperm = reinterpret_cast<PT *>(io.rperm);
  const long long units = static_cast<long long>(g.BH) * g.L;
  const int waves = staged_rank_waves(g);
  if (waves > 0) {
    const size_t rlds = (static_cast<size_t>(waves) * nb + waves) * 4 + static_cast<size_t>(g.N) * 2 + 16;
    uint16_t *rp16 = reinterpret_cast<uint16_t *>(io.rperm);
    if (g.rcb == 1)
      hipLaunchKernelGGL((elsaa_k4_race_rank<uint8_t>), dim3(static_cast<unsigned>(units)), dim3(waves * 64), rlds,
                         stream, static_cast<const uint8_t *>(io.codes), g.N, g.L, g.BH, g.P, g.rows,
                         race_parts(g.N), rp16, io.rstart, io.rpart, io.tcnt, io.flag);
    else
      hipLaunchKernelGGL((elsaa_k4_race_rank<uint16_t>), dim3(static_cast<unsigned>(units)), dim3(waves * 64), rlds,
                         stream, static_cast<const uint16_t *>(io.codes), g.N, g.L, g.BH, g.P, g.rows,
                         race_parts(g.N), rp16, io.rstart, io.rpart, io.tcnt, io.flag);
  } else {
    // tiled counting sort of the L * BH segments (table-major, as the codes
    // are), then the run table from its scanned counts
    hipError_t e = launch_tiled_sort(io.codes, g.rcb, g.N, g.P, units, io.hist, io.rperm,
                                     static_cast<int>(sizeof(PT)), stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(elsaa_k4_race_runs, dim3(static_cast<unsigned>(units)), dim3(256), 0, stream, io.hist,
                       g.N, g.L, g.BH, g.P, tiled_sort_tiles(g.N, g.P), race_parts(g.N), io.rstart, io.rpart,
                       io.tcnt, io.flag);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int parts = race_parts(g.N);
  const long long waves_total = units * parts;
  const long long wgs = (waves_total + kGatherWaves - 1) / kGatherWaves;
  const dim3 grid(static_cast<unsigned>((wgs + kXcdCount - 1) / kXcdCount * kXcdCount));
  auto gather = [&](auto vt, auto dc) {
    using VT = decltype(vt);
    constexpr int D = decltype(dc)::value;
    // one (b, h)'s value rows fit within twice an XCD's 4 MB L2: keep its
    // gathers on one XCD (gathers of 128-byte rows ran at the addresser's
    // rate up to 8 MB of rows per XCD); beyond that spread each (b, h) over
    // all XCDs, so its rows stay in the last-level cache
    const int xcd_local = static_cast<long long>(g.N) * D * sizeof(VT) <= (8ll << 20) ? 1 : 0;
    if constexpr (sizeof(VT) == 2) {
      if (io.blocks > 1) {  // binary32 partial tables
        if constexpr (D == 128) {  // in column halves
          const long long wt = 2 * waves_total;
          const long long wg2 = (wt + kGatherWaves - 1) / kGatherWaves;
          const dim3 grid2(static_cast<unsigned>((wg2 + kXcdCount - 1) / kXcdCount * kXcdCount));
          hipLaunchKernelGGL((elsaa_k4_race_gather<VT, 64, PT, float, 128>), grid2, dim3(kGatherWaves * 64), 0,
                             stream, static_cast<const VT *>(io.values), rperm, io.rstart, io.rpart, g.N, g.L,
                             g.BH, g.P, parts, wt, xcd_local, static_cast<float *>(io.tsum));
        } else {
          hipLaunchKernelGGL((elsaa_k4_race_gather<VT, D, PT, float, D>), grid, dim3(kGatherWaves * 64), 0,
                             stream, static_cast<const VT *>(io.values), rperm, io.rstart, io.rpart, g.N, g.L,
                             g.BH, g.P, parts, waves_total, xcd_local, static_cast<float *>(io.tsum));
        }
        return;
      }
    }
    hipLaunchKernelGGL((elsaa_k4_race_gather<VT, D, PT, VT, D>), grid, dim3(kGatherWaves * 64), 0, stream,
                       static_cast<const VT *>(io.values), rperm, io.rstart, io.rpart, g.N, g.L, g.BH, g.P,
                       parts, waves_total, xcd_local, static_cast<VT *>(io.tsum));
  };
  using D64 = std::integral_constant<int, 64>;
  using D128 = std::integral_constant<int, 128>;
  if (g.bf16 && !io.values_f32) {
    if (g.D == 64) gather(uint16_t{}, D64{});
    else gather(uint16_t{}, D128{});
  } else {
    if (g.D == 64) gather(float{}, D64{});
    else gather(float{}, D128{});
  }
  return hipGetLastError();
}

}  // namespace

size_t race_hist_bytes(const Geometry &g) {
  if (staged_rank_waves(g) > 0) return 0;
  return static_cast<size_t>(g.L) * g.BH * g.nb_race * tiled_sort_tiles(g.N, g.P) * 4;
}

int race_blocks(const Geometry &g) {
  constexpr long long kBlockBytes = 8ll << 20;
  const long long es = g.bf16 ? 2 : 4;
  const long long head = static_cast<long long>(g.N) * g.D * es;
  if (head <= kBlockBytes) return 1;
  int blocks = 2;
  while (static_cast<long long>(g.N) / blocks * g.D * es > kBlockBytes) blocks *= 2;
  // whole 64-key groups per block (the rank's 16-byte index pieces), and
  // partial tables no larger than twice the rows they sum
  const long long nblk = g.N / blocks;
  if (g.N % (64ll * blocks) != 0) return 1;
  if (static_cast<long long>(g.L) * g.nb_race * 4 > 2 * nblk * es) return 1;
  return blocks;
}

Geometry race_block_geometry(const Geometry &g) {
  const int blocks = race_blocks(g);
  Geometry gb = g;
  gb.BH = g.BH * blocks;
  gb.N = g.N / blocks;
  return gb;
}

hipError_t launch_race_build_io(const Geometry &g, const RaceBuildIO &io, hipStream_t stream) {
  if (io.blocks > 1) {
    // rank and gather over (b, h, block) heads into the partial tables, then
    // their sums in block order
    Geometry gb = g;
    gb.BH = g.BH * io.blocks;
    gb.N = g.N / io.blocks;
    RaceBuildIO ib = io;
    ib.tsum = io.psum;
    ib.tcnt = io.pcnt;
    hipError_t e = gb.N <= 65536 ? launch_race_build_pt<uint16_t>(gb, ib, stream)
                                 : launch_race_build_pt<int32_t>(gb, ib, stream);
    if (e != hipSuccess) return e;
    const long long row_elems = static_cast<long long>(g.L) * g.nb_race * g.D;
    const long long cnt_elems = static_cast<long long>(g.L) * g.nb_race;
    const long long n4 = g.BH * row_elems / 4, nc = g.BH * cnt_elems;
    const dim3 grid(static_cast<unsigned>((n4 + nc + 255) / 256));
    if (g.bf16 && !io.values_f32)
      hipLaunchKernelGGL((elsaa_k4_race_blocks_sum<uint16_t>), grid, dim3(256), 0, stream, io.psum, io.pcnt,
                         io.blocks, row_elems, cnt_elems, n4, nc, static_cast<uint16_t *>(io.tsum), io.tcnt);
    else
      hipLaunchKernelGGL((elsaa_k4_race_blocks_sum<float>), grid, dim3(256), 0, stream, io.psum, io.pcnt,
                         io.blocks, row_elems, cnt_elems, n4, nc, static_cast<float *>(io.tsum), io.tcnt);
    return hipGetLastError();
  }
  // 16-bit key indices whenever they fit
  return g.N <= 65536 ? launch_race_build_pt<uint16_t>(g, io, stream)
                      : launch_race_build_pt<int32_t>(g, io, stream);
}

hipError_t launch_race_build(const Geometry &g, const void *v, const Buffers &buf,
                             hipStream_t stream) {
  RaceBuildIO io;
  io.codes = static_cast<const char *>(buf.rcode) + static_cast<size_t>(g.rows) * g.L * g.rcb;
  io.values = v;
  io.values_f32 = false;
  io.rperm = buf.rperm;
  io.hist = buf.hist;  // shared with the sort, which runs after this stage
  io.rstart = buf.rstart;
  io.rpart = buf.rpart;
  io.tsum = buf.tsum;
  io.tcnt = buf.tcnt;
  io.flag = flagged_any(buf.flags, g.rows);  // the fix-up has run: cleared for the next call
  io.blocks = race_blocks(g);
  io.psum = buf.psum;
  io.pcnt = buf.pcnt;
  return launch_race_build_io(g, io, stream);
}

}  // namespace elsaa
