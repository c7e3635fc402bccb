// k4_race_build.hip -- RACE tables: per-bucket value sums and key counts.
//
// The low-rank branch compresses the keys into hash-bucket summaries ("Two
// Efficient Attentions, One Denominator Problem", section "Two efficient
// branches can still be mis-scaled"): for every table l and bucket b,
//   count[l][b] = #{keys j : code_l(k_j) = b},   sum[l][b][:] = sum of v_j over them.
//
// Built as a segmented reduction over sorted codes, in two kernels:
//   sort    one workgroup per (b, h, table): a stable counting sort of the N
//           key codes (integer LDS histograms per wave, a scan, and ranks from
//           one ballot per code bit), giving the keys of every bucket as one
//           contiguous run of the table's permutation, plus the run starts;
//   reduce  one wave per (b, h, table, 64 value columns, part of the buckets):
//           lanes are the 64 columns; the wave walks its buckets' runs in order,
//           loading 16 key rows ahead, sums each run in registers and writes the
//           bucket row and its count once.
// No floating-point atomics (LDS float atomics are slow on gfx950 and would make
// the summation order vary): every bucket is summed by one wave in ascending
// key order, so the tables are deterministic.  Heavy buckets (repeated tokens)
// are just long runs.
#include "elsaa_internal.hpp"

namespace elsaa {
namespace {


// --------------------------------------------------------------------- fused --
// One workgroup per (b, h, table) when the whole table fits in LDS: the table
// accumulates in LDS while the keys are taken in tiles of up to S keys.  Per
// tile: a stable counting sort of the tile's codes into an LDS permutation
// (per-wave integer histograms, a bucket-major scan, ballot ranks), then every
// wave sums a balanced share of the sorted positions, bucket by bucket, in
// registers (16-byte lane pieces, several rows per load instruction, one batch
// in flight while the previous one is added) and adds each finished bucket's
// row into the LDS table, which only that wave touches in this tile.  The permutation never
// leaves the chip; value rows are read once per table.
constexpr int kFusedWaves = 16;

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

// Exclusive prefix sum of one value per thread over a workgroup of
// kFusedWaves waves; `tmp` holds kFusedWaves words of LDS.  Two barriers.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t x, uint32_t *tmp, int lane,
                                                         int wave) {
  uint32_t inc = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(inc, off);
    if (lane >= off) inc += y;
  }
  if (lane == 63) tmp[wave] = inc;
  __syncthreads();
  uint32_t before = 0;
  for (int w = 0; w < wave; ++w) before += tmp[w];
  __syncthreads();  // tmp may be reused after this
  return before + inc - x;
}

template <typename CT, typename VT, int D>
__global__ __launch_bounds__(kFusedWaves * 64) void elsaa_k4_race_fused(
    const CT *__restrict__ kcodes, const VT *__restrict__ v, int N, int L, int P, int S, int G,
    long long units, VT *__restrict__ tsum, float *__restrict__ tcnt) {
  using PC = Piece<VT, D>;
  constexpr int W = kFusedWaves, kCols = PC::kCols, kLPR = PC::kLanesPerRow;
  constexpr int kRPI = PC::kRowsPerLoad;
  constexpr int kI = 8;              // load instructions per batch
  constexpr int kBP = kI * kRPI;     // positions per batch
  extern __shared__ uint32_t lds[];
  const int nb = 1 << P;
  float *acc = reinterpret_cast<float *>(lds);  // [nb][D]
  uint32_t *cnt = lds + nb * D;                 // [W][nb] counts, then running offsets
  uint32_t *bst = cnt + W * nb;                 // [nb + 1] tile-local run starts
  uint32_t *tot = bst + nb + 1;                 // [nb] keys per bucket over all tiles
  uint32_t *part = tot + nb;                    // [W * 64] scan
  uint16_t *lperm = reinterpret_cast<uint16_t *>(part + W * 64);  // [S + slack] tile-local key index

  // unit = ((b, h) * L + table) * G + bucket group; the G workgroups of a
  // table each count, rank and sum only the keys of their buckets [gb0, gb1)
  const long long unit = xcd_logical_block(blockIdx.x, gridDim.x);
  if (unit >= units) return;  // whole workgroup
  const long long tu = unit / G;
  const int grp = static_cast<int>(unit % G);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps wave ranges scalar
  const long long bh = tu / L;
  const int l = static_cast<int>(tu % L);
  const int gb0 = static_cast<int>(static_cast<long long>(nb) * grp / G);
  const int gb1 = static_cast<int>(static_cast<long long>(nb) * (grp + 1) / G);
  const long long rows = units / G / L * N;  // keys of all (b, h)
  const CT *c = kcodes + static_cast<long long>(l) * rows + bh * N;  // code of key j at c[j]
  const VT *vb = v + bh * N * static_cast<long long>(D);

  for (int i = tid; i < nb * D; i += W * 64) acc[i] = 0.0f;
  for (int i = tid; i < nb; i += W * 64) tot[i] = 0u;

  for (int t0 = 0; t0 < N; t0 += S) {
    const int M = N - t0 < S ? N - t0 : S;
    const int chunk = ((M + W - 1) / W + 63) / 64 * 64;
    const int j_begin = t0 + (wave * chunk < M ? wave * chunk : M);
    const int j_end = t0 + ((wave + 1) * chunk < M ? (wave + 1) * chunk : M);
    for (int i = tid; i < W * nb; i += W * 64) cnt[i] = 0u;
    __syncthreads();

    uint32_t *wc = cnt + wave * nb;
    // eight rounds of codes per call; loads are clamped, not skipped, so they
    // all issue before the first wait
    auto load_codes = [&](int j0, uint32_t (&code)[8]) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = j0 + q * 64 + lane;
        const uint32_t cv = static_cast<uint32_t>(c[j < j_end ? j : j_end - 1]);
        code[q] = j < j_end ? cv : 0xffffffffu;
      }
    };
    // only the keys of the group's buckets [gb0, gb1) are counted and ranked
    auto mine = [&](uint32_t code) {
      return code != 0xffffffffu && code >= static_cast<uint32_t>(gb0) && code < static_cast<uint32_t>(gb1);
    };
    for (int j0 = j_begin; j0 < j_end; j0 += 512) {
      uint32_t code[8];
      load_codes(j0, code);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (mine(code[q])) atomicAdd(&wc[code[q]], 1u);
    }
    __syncthreads();

    // bucket-major exclusive scan of the [bucket][wave] counts
    {
      const int nthreads = W * 64;
      const int per = (nb + nthreads - 1) / nthreads;
      const int b_lo = tid * per < nb ? tid * per : nb;
      const int b_hi = b_lo + per < nb ? b_lo + per : nb;
      uint32_t sum = 0;
      for (int b = b_lo; b < b_hi; ++b)
        for (int w = 0; w < W; ++w) sum += cnt[w * nb + b];
      uint32_t run = block_exclusive_scan(sum, part, lane, wave);
      for (int b = b_lo; b < b_hi; ++b) {
        bst[b] = run;
        const uint32_t r0 = run;
        for (int w = 0; w < W; ++w) {
          const uint32_t t = cnt[w * nb + b];
          cnt[w * nb + b] = run;
          run += t;
        }
        tot[b] += run - r0;
      }
      // end of the last run: the number of the group's keys in this tile
      if (b_lo < nb && b_hi == nb) bst[nb] = run;
    }
    __syncthreads();

    // Positions: each key takes the next slot of its (wave, bucket) counter
    // with an LDS atomic that returns the old value.  Keys of one bucket keep
    // the order of the waves, and of the rounds inside a wave; inside one
    // round the hardware's lane order decides.  The order only fixes how a
    // bucket's rows are summed.
    for (int j8 = j_begin; j8 < j_end; j8 += 512) {
      uint32_t codes8[8];
      load_codes(j8, codes8);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = j8 + q * 64 + lane;
        if (mine(codes8[q])) lperm[atomicAdd(&wc[codes8[q]], 1u)] = static_cast<uint16_t>(j - t0);
      }
    }
    __syncthreads();

    // The group's positions [PL, PH) split evenly over the waves: a wave owns
    // the group's buckets whose run starts in [lo, hi); the last wave also
    // owns the empty buckets that start at PH
    const int PL = static_cast<int>(bst[gb0]), PH = static_cast<int>(bst[gb1]);
    const long long Mg = PH - PL;
    const int lo = PL + static_cast<int>(Mg * wave / W);
    const int hi = wave == W - 1 ? PH + 1 : PL + static_cast<int>(Mg * (wave + 1) / W);
    int b0 = gb1, b1 = gb1;
    for (int bb = gb0; bb < gb1; bb += 64) {
      const int b = bb + lane;
      const int st = b < gb1 ? static_cast<int>(bst[b]) : PH + 1;
      const unsigned long long ge_lo = __ballot(b < gb1 && st >= lo);
      const unsigned long long ge_hi = __ballot(b < gb1 && st >= hi);
      if (b0 == gb1 && ge_lo) b0 = bb + __builtin_ctzll(ge_lo);
      if (b1 == gb1 && ge_hi) b1 = bb + __builtin_ctzll(ge_hi);
    }
    const int p_lo = static_cast<int>(bst[b0]), p_hi = static_cast<int>(bst[b1]);

    if (p_lo < p_hi) {
      const int cc = lane % kLPR;  // column piece
      const int my_off = lane / kLPR;  // this lane's row within a load: position p + my_off
      const Bf16Adder adder;
      int b = b0;
      int bend = __builtin_amdgcn_readfirstlane(static_cast<int>(bst[b0 + 1]));
      float a[kCols];
#pragma unroll
      for (int k = 0; k < kCols; ++k) a[k] = 0.0f;
      // Bucket b is complete: sum the partials of the lanes holding the same
      // columns (a transposing reduction: every exchange halves the values a
      // lane holds) and add the lane's kCols / kRPI column sums into the LDS
      // table.
      auto flush = [&]() {
        float r[kCols / kRPI];
        lane_group_transpose_sum<kCols, kLPR>(a, r, lane);
#pragma unroll
        for (int m = 0; m < kCols / kRPI; ++m)
          acc[b * D + cc * kCols + transposed_column<kCols, kLPR>(m, lane)] += r[m];
#pragma unroll
        for (int k = 0; k < kCols; ++k) a[k] = 0.0f;
      };
      // value rows of this tile through a buffer resource: 32-bit offsets
      const __amdgpu_buffer_rsrc_t vrs =
          make_rsrc(vb + static_cast<long long>(t0) * D, static_cast<uint32_t>(M) * PC::kRowBytes);
      const uint32_t cbyte = static_cast<uint32_t>(cc) * 16u;
      auto load_batch = [&](int pbase, u32x4 (&r)[kI]) {
        // positions past p_hi (up to 3 batches) read the next wave's entries or
        // the slack at the end of lperm; their rows are loaded (out-of-range
        // offsets read zero) and never added
        uint32_t jl[kI];
        const uint16_t *lp = lperm + pbase + my_off;
#pragma unroll
        for (int i = 0; i < kI; ++i) jl[i] = lp[i * kRPI];
#pragma unroll
        for (int i = 0; i < kI; ++i)
          r[i] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, jl[i] * PC::kRowBytes + cbyte, 0, 0));
      };
      // rows of positions [pbase, pbase + kBP).  Bucket ends never pass p_hi,
      // so one scalar test per load (its rows end before bucket b does) picks
      // the plain add; a load that reaches a bucket end takes the per-lane
      // path, which also flushes the bucket
      auto consume = [&](int pbase, const u32x4 (&r)[kI]) {
#pragma unroll
        for (int i = 0; i < kI; ++i) {
          const int p = pbase + i * kRPI;
          const int pe = p + kRPI < p_hi ? p + kRPI : p_hi;
          const int my = p + my_off;
          // rows before the end of bucket b (all of them, mostly)
          const int stop0 = pe < bend ? pe : bend;
          if (my < stop0) PC::add(r[i], a, adder);
          if (pe >= bend && p < p_hi) {  // the load reaches the end of bucket b
            int cur = stop0;
            do {
              if (cur == bend) {
                flush();
                ++b;
                // past the wave's last bucket (then cur == p_hi): no end to meet
                bend = b < b1 ? __builtin_amdgcn_readfirstlane(static_cast<int>(bst[b + 1])) : 0x7fffffff;
              }
              const int stop = pe < bend ? pe : bend;
              if (my >= cur && my < stop) PC::add(r[i], a, adder);
              cur = stop;
            } while (cur < pe || cur == bend);
          }
        }
      };
      u32x4 ra[kI], rb[kI];
      load_batch(p_lo, ra);
      for (int pc = p_lo; pc < p_hi; pc += 2 * kBP) {
        load_batch(pc + kBP, rb);
        consume(pc, ra);
        load_batch(pc + 2 * kBP, ra);
        consume(pc + kBP, rb);
      }
    }
    __syncthreads();
  }

  // the table leaves in the value dtype (sums were kept in binary32)
  VT *ts = tsum + tu * nb * static_cast<long long>(D);
  for (int i = gb0 * D + 4 * tid; i < gb1 * D; i += 4 * W * 64) Elem<VT>::store4(ts + i, acc + i);
  for (int i = gb0 + tid; i < gb1; i += W * 64) tcnt[tu * nb + i] = static_cast<float>(tot[i]);
}

// ----------------------------------------------------------- rank + gather --
// Two kernels, for any table size.
//   rank    one workgroup per (b, h, table): a counting sort of the table's N
//           key codes (per-wave LDS histograms, a bucket-major scan, then each
//           key takes the next slot of its (wave, bucket) counter from an LDS
//           atomic that returns the old value), writing the sorted key
//           indices, the run start of every bucket and the bucket counts;
//   gather  one wave per (b, h, table, part of the positions): the wave owns
//           the buckets whose run starts in its part, stages their key
//           indices in LDS and sums the value rows bucket by bucket as the
//           fused kernel does, writing each finished bucket row once.  Waves
//           of one (b, h) are consecutive and so share an XCD's L2, which then
//           holds the value rows all its tables gather.
template <typename CT>
__global__ __launch_bounds__(1024) void elsaa_k4_race_rank(
    const CT *__restrict__ kcodes, int N, int L, int P, long long rows, int staged,
    int32_t *__restrict__ rperm, int32_t *__restrict__ rstart, float *__restrict__ tcnt) {
  extern __shared__ uint32_t lds[];
  const int nb = 1 << P;
  const int W = static_cast<int>(blockDim.x >> 6);
  uint32_t *cnt = lds;           // [W][nb] counts, then running offsets
  uint32_t *part = lds + W * nb;  // [W] scan
  uint16_t *lperm = reinterpret_cast<uint16_t *>(part + W);  // [N] when staged (N <= 65536)
  const long long unit = blockIdx.x;  // (b, h) * L + table
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long long bh = unit / L;
  const int l = static_cast<int>(unit % L);
  const CT *c = kcodes + static_cast<long long>(l) * rows + bh * N;  // code of key j at c[j]
  const int chunk = ((N + W - 1) / W + 63) / 64 * 64;
  const int j_begin = wave * chunk < N ? wave * chunk : N;
  const int j_end = j_begin + chunk < N ? j_begin + chunk : N;

  for (int i = tid; i < W * nb; i += W * 64) cnt[i] = 0u;
  __syncthreads();
  uint32_t *wc = cnt + wave * nb;
  auto load_codes = [&](int j0, uint32_t (&code)[8]) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int j = j0 + q * 64 + lane;
      const uint32_t cv = static_cast<uint32_t>(c[j < j_end ? j : j_end - 1]);
      code[q] = j < j_end ? cv : 0xffffffffu;
    }
  };
  for (int j0 = j_begin; j0 < j_end; j0 += 512) {
    uint32_t code[8];
    load_codes(j0, code);
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (code[q] != 0xffffffffu) atomicAdd(&wc[code[q]], 1u);
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
    for (int b = b_lo; b < b_hi; ++b) {
      rs[b] = static_cast<int32_t>(run);
      const uint32_t r0 = run;
      for (int w = 0; w < W; ++w) {
        const uint32_t t = cnt[w * nb + b];
        cnt[w * nb + b] = run;
        run += t;
      }
      tcnt[unit * nb + b] = static_cast<float>(run - r0);
    }
    if (tid == 0) rs[nb] = N;
  }
  __syncthreads();
  // sorted key indices: staged in LDS and written out in order (coalesced),
  // or scattered straight to memory when N does not fit
  int32_t *rp = rperm + unit * N;
  for (int j8 = j_begin; j8 < j_end; j8 += 512) {
    uint32_t codes8[8];
    load_codes(j8, codes8);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int j = j8 + q * 64 + lane;
      if (codes8[q] != 0xffffffffu) {
        const uint32_t pos = atomicAdd(&wc[codes8[q]], 1u);
        if (staged) lperm[pos] = static_cast<uint16_t>(j);
        else rp[pos] = j;
      }
    }
  }
  if (staged) {
    __syncthreads();
    for (int i = tid; i < N; i += W * 64) rp[i] = lperm[i];
  }
}

constexpr int kGatherWaves = 4;       // waves per gather workgroup
constexpr int kGatherStage = 1024;    // key indices a wave stages in LDS at once
constexpr int kGatherSlack = 256;     // staged entries read past the end by the look-ahead

template <typename VT, int D>
__global__ __launch_bounds__(kGatherWaves * 64) void elsaa_k4_race_gather(
    const VT *__restrict__ v, const int32_t *__restrict__ rperm, const int32_t *__restrict__ rstart,
    int N, int L, int P, int parts, long long waves_total, VT *__restrict__ tsum) {
  using PC = Piece<VT, D>;
  constexpr int kCols = PC::kCols, kLPR = PC::kLanesPerRow;
  constexpr int kRPI = PC::kRowsPerLoad;
  constexpr int kI = 8;              // load instructions per batch
  constexpr int kBP = kI * kRPI;     // positions per batch
  __shared__ uint32_t stage_all[kGatherWaves][kGatherStage + kGatherSlack];
  const int nb = 1 << P;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const long long u = xcd_logical_block(blockIdx.x, gridDim.x) * kGatherWaves + wave;
  if (u >= waves_total) return;  // whole wave; the kernel has no barriers
  uint32_t *stage = stage_all[wave];
  const int prt = static_cast<int>(u % parts);
  const long long unit = u / parts;  // (b, h) * L + table
  const long long bh = unit / L;
  const int32_t *rs = rstart + unit * (nb + 1);
  const int32_t *rp = rperm + unit * N;
  VT *ts = tsum + unit * nb * static_cast<long long>(D);

  // owned buckets: those whose run starts in [lo, hi); the last part also owns
  // the empty buckets that start at N
  const int lo = static_cast<int>(static_cast<long long>(N) * prt / parts);
  const int hi = prt == parts - 1 ? N + 1 : static_cast<int>(static_cast<long long>(N) * (prt + 1) / parts);
  int b0 = nb, b1 = nb;
  for (int bb = 0; bb < nb; bb += 64) {
    const int b = bb + lane;
    const int st = b < nb ? rs[b] : N + 1;
    const unsigned long long ge_lo = __ballot(b < nb && st >= lo);
    const unsigned long long ge_hi = __ballot(b < nb && st >= hi);
    if (b0 == nb && ge_lo) b0 = bb + __builtin_ctzll(ge_lo);
    if (b1 == nb && ge_hi) b1 = bb + __builtin_ctzll(ge_hi);
    if (b1 != nb) break;
  }
  b0 = __builtin_amdgcn_readfirstlane(b0);
  b1 = __builtin_amdgcn_readfirstlane(b1);
  if (b0 >= b1) return;
  const int p_lo = __builtin_amdgcn_readfirstlane(rs[b0]);
  const int p_hi = __builtin_amdgcn_readfirstlane(rs[b1]);

  const int cc = lane % kLPR;       // column piece
  const int my_off = lane / kLPR;   // this lane's row within a load
  const Bf16Adder adder;
  int b = b0;
  int bend = __builtin_amdgcn_readfirstlane(rs[b0 + 1]);
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
      ts[b * static_cast<long long>(D) + cc * kCols + transposed_column<kCols, kLPR>(m, lane)] =
          Elem<VT>::store_val(r[m]);
#pragma unroll
    for (int k = 0; k < kCols; ++k) a[k] = 0.0f;
  };
  if (p_lo == p_hi) {  // only empty buckets
    for (; b < b1; ++b) flush();
    return;
  }
  const __amdgpu_buffer_rsrc_t vrs =
      make_rsrc(v + bh * N * static_cast<long long>(D), static_cast<uint32_t>(N) * PC::kRowBytes);
  const uint32_t cbyte = static_cast<uint32_t>(cc) * 16u;
  for (int s0 = p_lo; s0 < p_hi; s0 += kGatherStage) {
    const int s1 = s0 + kGatherStage < p_hi ? s0 + kGatherStage : p_hi;
    // stage the key indices of positions [s0, s1) (entries past s1 are stale:
    // the look-ahead may load their rows, which are never added)
    for (int i = lane; i < s1 - s0; i += 64) stage[i] = static_cast<uint32_t>(rp[s0 + i]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    auto load_batch = [&](int pbase, u32x4 (&r)[kI]) {
      uint32_t jl[kI];
      const uint32_t *lp = stage + (pbase - s0) + my_off;
#pragma unroll
      for (int i = 0; i < kI; ++i) jl[i] = lp[i * kRPI];
#pragma unroll
      for (int i = 0; i < kI; ++i)
        r[i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, jl[i] * PC::kRowBytes + cbyte, 0, 0));
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
              bend = b < b1 ? __builtin_amdgcn_readfirstlane(rs[b + 1]) : 0x7fffffff;
            }
            const int stop = pe < bend ? pe : bend;
            if (my >= cur && my < stop) PC::add(r[i], a, adder);
            cur = stop;
          } while (cur < pe || cur == bend);
        }
      }
    };
    u32x4 ra[kI], rb[kI];
    load_batch(s0, ra);
    for (int pc = s0; pc < s1; pc += 2 * kBP) {
      load_batch(pc + kBP, rb);
      consume(pc, ra);
      load_batch(pc + 2 * kBP, ra);
      consume(pc + kBP, rb);
    }
    // the stage may be overwritten only after every lane has read it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  }
}

#ifndef ELSAA_RACE_GROUPS
#define ELSAA_RACE_GROUPS 0  // 0: chosen per shape
#endif

double idle_fraction(long long units, int cus) {
  if (cus <= 0) return 0.0;
  const long long rounds = (units + cus - 1) / cus;
  return 1.0 - static_cast<double>(units) / static_cast<double>(rounds * cus);
}

// Bucket groups per table on the single-kernel path: each group is a
// workgroup that sorts the table's keys and sums its share of the buckets.
// Groups repeat the sort, so they are used only to give small problems (fewer
// tables than compute units) enough workgroups: up to 4 per table.
int race_groups(const Geometry &g) {
  if (ELSAA_RACE_GROUPS > 0) return ELSAA_RACE_GROUPS;
  const long long tables = static_cast<long long>(g.BH) * g.L;
  int G = 1;
  while (G < 4 && G < g.nb_race && tables * G < g.cus) G *= 2;
  return G;
}

// LDS bytes of the fused kernel for tile size S (0 if the table does not fit).
constexpr int kLpermSlack = 256;  // entries past S read by the gather's look-ahead

size_t fused_lds_bytes(int nb, int D, int S) {
  return (static_cast<size_t>(nb) * D + static_cast<size_t>(kFusedWaves) * nb + 2 * nb + 1 +
          kFusedWaves * 64) * 4 + (static_cast<size_t>(S) + kLpermSlack) * 2;
}

template <typename CT, typename VT>
void launch_fused(const Geometry &g, const void *rk, const void *v, int S, size_t lds,
                  const Buffers &buf, hipStream_t stream) {
  const int G = race_groups(g);
  const long long units = static_cast<long long>(g.BH) * g.L * G;
  const dim3 grid(static_cast<unsigned>((units + kXcdCount - 1) / kXcdCount * kXcdCount));
  const dim3 block(kFusedWaves * 64);
  if (g.D == 64)
    hipLaunchKernelGGL((elsaa_k4_race_fused<CT, VT, 64>), grid, block, lds, stream,
                       static_cast<const CT *>(rk), static_cast<const VT *>(v), g.N, g.L, g.P, S, G,
                       units, static_cast<VT *>(buf.tsum), buf.tcnt);
  else
    hipLaunchKernelGGL((elsaa_k4_race_fused<CT, VT, 128>), grid, block, lds, stream,
                       static_cast<const CT *>(rk), static_cast<const VT *>(v), g.N, g.L, g.P, S, G,
                       units, static_cast<VT *>(buf.tsum), buf.tcnt);
}

}  // namespace

#ifndef ELSAA_FUSED_TILE_MAX
#define ELSAA_FUSED_TILE_MAX 32768
#endif

int race_fused_tile(const Geometry &g) {
  const size_t fixed = fused_lds_bytes(g.nb_race, g.D, 0);
  if (fixed + 2 * 1024 > kFusedLdsMax) return 0;
  // Tiles bound the value rows the concurrent workgroups of one XCD gather
  // from (S rows of each (b, h)), so they stay in its L2; tile-local key
  // indices are 16-bit.
  int smax = static_cast<int>((kFusedLdsMax - fixed) / 2 / 1024 * 1024);
  smax = smax < ELSAA_FUSED_TILE_MAX ? smax : ELSAA_FUSED_TILE_MAX;
  const int n64 = (g.N + 63) / 64 * 64;
  return n64 < smax ? n64 : smax;
}

#ifndef ELSAA_RACE_SPLIT
#define ELSAA_RACE_SPLIT 1  // 1: rank + gather kernels; 0: single kernel where the table fits in LDS
#endif
#ifndef ELSAA_GATHER_POS
#define ELSAA_GATHER_POS 512  // positions per gather wave (before rounding to whole buckets)
#endif

bool race_split(const Geometry &g) { return ELSAA_RACE_SPLIT || race_fused_tile(g) == 0; }

double race_build_idle_fraction(const Geometry &g) {
  // the gather kernel of the two-kernel build fills the device
  if (race_split(g)) return 0.0;
  return idle_fraction(static_cast<long long>(g.BH) * g.L * race_groups(g), g.cus);
}

hipError_t launch_race_build(const Geometry &g, const void *v, const Buffers &buf,
                             hipStream_t stream) {
  const int nb = g.nb_race;
  const void *rk = static_cast<const char *>(buf.rcode) + static_cast<size_t>(g.rows) * g.L * g.rcb;
  if (!race_split(g)) {
    const int S = race_fused_tile(g);
    const size_t lds = fused_lds_bytes(nb, g.D, S);
    if (g.rcb == 1) {
      if (g.bf16) launch_fused<uint8_t, uint16_t>(g, rk, v, S, lds, buf, stream);
      else launch_fused<uint8_t, float>(g, rk, v, S, lds, buf, stream);
    } else {
      if (g.bf16) launch_fused<uint16_t, uint16_t>(g, rk, v, S, lds, buf, stream);
      else launch_fused<uint16_t, float>(g, rk, v, S, lds, buf, stream);
    }
    return hipGetLastError();
  }
  const long long units = static_cast<long long>(g.BH) * g.L;
  int waves = 16384 / nb;  // LDS counters: waves * nb * 4 bytes <= 64 KB
  waves = waves < 1 ? 1 : (waves > 16 ? 16 : waves);
  // stage the sorted indices in LDS when N fits, keeping two workgroups per CU
  constexpr size_t kRankLdsTwoPerCu = 78 * 1024;
  auto rank_lds = [&](int w, bool st) {
    return (static_cast<size_t>(w) * nb + w) * 4 + (st ? static_cast<size_t>(g.N) * 2 : 0);
  };
  bool staged = g.N <= 65536;
  while (staged && waves > 4 && rank_lds(waves, true) > kRankLdsTwoPerCu) waves /= 2;
  if (rank_lds(waves, staged) > kRankLdsTwoPerCu) staged = false;
  const size_t rlds = rank_lds(waves, staged);
  if (g.rcb == 1)
    hipLaunchKernelGGL(elsaa_k4_race_rank<uint8_t>, dim3(static_cast<unsigned>(units)), dim3(waves * 64), rlds,
                       stream, static_cast<const uint8_t *>(rk), g.N, g.L, g.P, g.rows, staged ? 1 : 0, buf.rperm,
                       buf.rstart, buf.tcnt);
  else
    hipLaunchKernelGGL(elsaa_k4_race_rank<uint16_t>, dim3(static_cast<unsigned>(units)), dim3(waves * 64), rlds,
                       stream, static_cast<const uint16_t *>(rk), g.N, g.L, g.P, g.rows, staged ? 1 : 0, buf.rperm,
                       buf.rstart, buf.tcnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int parts = (g.N + ELSAA_GATHER_POS - 1) / ELSAA_GATHER_POS;
  const long long waves_total = units * parts;
  const long long wgs = (waves_total + kGatherWaves - 1) / kGatherWaves;
  const dim3 grid(static_cast<unsigned>((wgs + kXcdCount - 1) / kXcdCount * kXcdCount));
  if (g.bf16) {
    if (g.D == 64)
      hipLaunchKernelGGL((elsaa_k4_race_gather<uint16_t, 64>), grid, dim3(kGatherWaves * 64), 0, stream,
                         static_cast<const uint16_t *>(v), buf.rperm, buf.rstart, g.N, g.L, g.P, parts,
                         waves_total, static_cast<uint16_t *>(buf.tsum));
    else
      hipLaunchKernelGGL((elsaa_k4_race_gather<uint16_t, 128>), grid, dim3(kGatherWaves * 64), 0, stream,
                         static_cast<const uint16_t *>(v), buf.rperm, buf.rstart, g.N, g.L, g.P, parts,
                         waves_total, static_cast<uint16_t *>(buf.tsum));
  } else {
    if (g.D == 64)
      hipLaunchKernelGGL((elsaa_k4_race_gather<float, 64>), grid, dim3(kGatherWaves * 64), 0, stream,
                         static_cast<const float *>(v), buf.rperm, buf.rstart, g.N, g.L, g.P, parts, waves_total,
                         static_cast<float *>(buf.tsum));
    else
      hipLaunchKernelGGL((elsaa_k4_race_gather<float, 128>), grid, dim3(kGatherWaves * 64), 0, stream,
                         static_cast<const float *>(v), buf.rperm, buf.rstart, g.N, g.L, g.P, parts, waves_total,
                         static_cast<float *>(buf.tsum));
  }
  return hipGetLastError();
}

}  // namespace elsaa
