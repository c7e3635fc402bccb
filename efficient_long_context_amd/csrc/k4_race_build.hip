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
//           of 8 loads in flight, a scalar test per load for the common case
//           of a load inside one bucket, and at a bucket end a transposing
//           lane reduction whose column sums are stored as the table row.
//           Waves of one (b, h) are consecutive and so share an XCD's L2,
//           which then holds the value rows its tables gather.
//   The sorted key indices are 16-bit (PT = uint16_t) whenever N <= 65536,
//   halving the permutation's write here and its read in the gather.
template <typename CT, typename PT>
__global__ __launch_bounds__(1024) void elsaa_k4_race_rank(
    const CT *__restrict__ kcodes, int N, int L, int P, long long rows, int staged, int parts,
    PT *__restrict__ rperm, int32_t *__restrict__ rstart, int32_t *__restrict__ rpart,
    float *__restrict__ tcnt, uint32_t *__restrict__ hash_flagged) {
  extern __shared__ uint32_t lds[];
  if (blockIdx.x == 0 && threadIdx.x == 0) *hash_flagged = 0u;  // the fix-up has run
  const int nb = 1 << P;
  const int W = static_cast<int>(blockDim.x >> 6);
  uint32_t *cnt = lds;           // [W][nb] counts, then running offsets
  uint32_t *part = lds + W * nb;  // [W] scan
  // [N] when staged (N <= 65536), 16-byte aligned for the vector copy-out
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
    // gather part p (positions from lo_p = N p / parts) owns the buckets whose
    // run starts in [lo_p, lo_{p+1}); its first one is the first bucket starting
    // at or after lo_p: bucket b + 1 when lo_p lies in (start_b, end_b]
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
      if (run > r0) {
        long long pp = static_cast<long long>(r0) * parts / N;
        while (pp < parts && static_cast<long long>(N) * pp / parts <= static_cast<long long>(r0)) ++pp;
        for (; pp < parts && static_cast<long long>(N) * pp / parts <= static_cast<long long>(run); ++pp) {
          rp2[2 * pp] = b + 1;
          rp2[2 * pp + 1] = static_cast<int32_t>(run);
        }
      }
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
  // sorted key indices: staged in LDS and written out in order (coalesced),
  // or scattered straight to memory when N does not fit
  PT *rp = rperm + unit * N;
  auto place = [&](uint32_t code, int j) {
    const uint32_t pos = atomicAdd(&wc[code], 1u);
    if (staged) lperm[pos] = static_cast<uint16_t>(j);
    else rp[pos] = static_cast<PT>(j);
  };
  if (j_begin < j_end) for_batch(j_begin, first, place);
  for (int jb = j_begin + kBatch; jb < j_end; jb += kBatch) {
    u32x4 pc[kPieces];
    load_batch(jb, pc);
    for_batch(jb, pc, place);
  }
  if (staged) {
    __syncthreads();
    if constexpr (sizeof(PT) == 2) {  // 8 indices a 16-byte piece (N is a multiple of 64)
      for (int i = tid; i < N / 8; i += W * 64)
        reinterpret_cast<u32x4 *>(rp)[i] = reinterpret_cast<const u32x4 *>(lperm)[i];
    } else {
      for (int i = tid; i < N; i += W * 64) rp[i] = static_cast<PT>(lperm[i]);
    }
  }
}

constexpr int kGatherWaves = 4;       // waves per gather workgroup
constexpr int kGatherStage = 1024;    // key indices a wave stages in LDS at once
constexpr int kGatherSlack = 256;     // staged entries read past the end by the look-ahead

template <typename VT, int D, typename PT>
__global__ __launch_bounds__(kGatherWaves * 64) void elsaa_k4_race_gather(
    const VT *__restrict__ v, const PT *__restrict__ rperm, const int32_t *__restrict__ rstart,
    const int32_t *__restrict__ rpart, int N, int L, int P, int parts, long long waves_total,
    VT *__restrict__ tsum) {
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
  const PT *rp = rperm + unit * N;
  VT *ts = tsum + unit * nb * static_cast<long long>(D);

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

}  // namespace


namespace {

template <typename PT>
hipError_t launch_race_build_pt(const Geometry &g, const void *v, const Buffers &buf, hipStream_t stream) {
  const int nb = g.nb_race;
  const void *rk = static_cast<const char *>(buf.rcode) + static_cast<size_t>(g.rows) * g.L * g.rcb;
  PT *rperm = reinterpret_cast<PT *>(buf.rperm);
  const long long units = static_cast<long long>(g.BH) * g.L;
  int waves = 16384 / nb;  // LDS counters: waves * nb * 4 bytes <= 64 KB
  waves = waves < 1 ? 1 : (waves > 16 ? 16 : waves);
  // stage the sorted indices in LDS when N fits, keeping two workgroups per CU
  constexpr size_t kRankLdsTwoPerCu = 78 * 1024;
  auto rank_lds = [&](int w, bool st) {  // + 16: the staged indices start 16-byte aligned
    return (static_cast<size_t>(w) * nb + w) * 4 + (st ? static_cast<size_t>(g.N) * 2 + 16 : 0);
  };
  bool staged = g.N <= 65536;
  while (staged && waves > 4 && rank_lds(waves, true) > kRankLdsTwoPerCu) waves /= 2;
  if (rank_lds(waves, staged) > kRankLdsTwoPerCu) staged = false;
  const size_t rlds = rank_lds(waves, staged);
  if (g.rcb == 1)
    hipLaunchKernelGGL((elsaa_k4_race_rank<uint8_t, PT>), dim3(static_cast<unsigned>(units)), dim3(waves * 64),
                       rlds, stream, static_cast<const uint8_t *>(rk), g.N, g.L, g.P, g.rows, staged ? 1 : 0,
                       race_parts(g.N), rperm, buf.rstart, buf.rpart, buf.tcnt, flagged_any(buf.flags, g.rows));
  else
    hipLaunchKernelGGL((elsaa_k4_race_rank<uint16_t, PT>), dim3(static_cast<unsigned>(units)), dim3(waves * 64),
                       rlds, stream, static_cast<const uint16_t *>(rk), g.N, g.L, g.P, g.rows, staged ? 1 : 0,
                       race_parts(g.N), rperm, buf.rstart, buf.rpart, buf.tcnt, flagged_any(buf.flags, g.rows));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int parts = race_parts(g.N);
  const long long waves_total = units * parts;
  const long long wgs = (waves_total + kGatherWaves - 1) / kGatherWaves;
  const dim3 grid(static_cast<unsigned>((wgs + kXcdCount - 1) / kXcdCount * kXcdCount));
  auto gather = [&](auto vt, auto dc) {
    using VT = decltype(vt);
    constexpr int D = decltype(dc)::value;
    hipLaunchKernelGGL((elsaa_k4_race_gather<VT, D, PT>), grid, dim3(kGatherWaves * 64), 0, stream,
                       static_cast<const VT *>(v), rperm, buf.rstart, buf.rpart, g.N, g.L, g.P, parts,
                       waves_total, static_cast<VT *>(buf.tsum));
  };
  using D64 = std::integral_constant<int, 64>;
  using D128 = std::integral_constant<int, 128>;
  if (g.bf16) {
    if (g.D == 64) gather(uint16_t{}, D64{});
    else gather(uint16_t{}, D128{});
  } else {
    if (g.D == 64) gather(float{}, D64{});
    else gather(float{}, D128{});
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_race_build(const Geometry &g, const void *v, const Buffers &buf,
                             hipStream_t stream) {
  // 16-bit key indices whenever they fit (the workspace holds 32-bit ones)
  return g.N <= 65536 ? launch_race_build_pt<uint16_t>(g, v, buf, stream)
                      : launch_race_build_pt<int32_t>(g, v, buf, stream);
}

}  // namespace elsaa
