// k4_race_build.hip -- RACE tables: per-bucket value sums and key counts.
//
// The low-rank branch compresses the keys into hash-bucket summaries ("Two
// Efficient Attentions, One Denominator Problem", section "Two efficient
// branches can still be mis-scaled"): for every table l and bucket b,
//   count[l][b] = #{keys j : code_l(k_j) = b},   sum[l][b][:] = sum of v_j over them.
//
// Work unit = (b, h, table l, column slice of 64 value columns, range of RB <= 32
// consecutive buckets).  One wave owns one unit and keeps its RB bucket rows in
// registers: lane c holds column c of every bucket of the range, indexed by a
// wave-uniform bucket (lowered to M0-relative register moves).
// The wave scans every key of (b, h) in index order, 64 codes per ballot, and
// adds the value row of each key whose bucket falls in its range, eight keys
// per straight-line round (a round that runs out of keys adds a zero row).  No
// accumulator is shared, adds happen in key order, and no atomics are used
// (LDS float atomics are slow on gfx950 and would make the order, hence the
// rounding, vary), so the result is deterministic; repeated keys cost the same
// as distinct ones.  Bucket counts come from a separate integer histogram.
//
// A workgroup of 8 waves shares one column slice: tiles of 64 key rows (and
// their code block) are loaded into a ring of four register sets, converted to
// fp32 once and staged in LDS for all 8 waves.  Barriers order LDS only, so the
// prefetches stay in flight across them.  Workgroups of one (b, h) are mapped
// to one XCD (dispatch is round-robin over the 8 XCDs) so its value rows are
// fetched into one L2.
#include "elsaa_internal.hpp"

namespace elsaa {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kTK = 64;       // keys per staged tile
constexpr int kMaxRB = 32;    // buckets per wave
constexpr int kRound = 8;     // keys added per straight-line round

// One thread's share of a tile: 8 consecutive values of one key row and 16
// bytes of the tile's code block (the codes of 64 consecutive keys are one
// contiguous block of 64 * L codes).  Loads are unconditional (addresses
// clamped in bounds), so the compiler never waits for a prefetch before the
// tile is staged.
typedef float f32x32 __attribute__((ext_vector_type(32)));

template <typename VT>
struct TileRegs {
  VT x[8];
  uint4 c;
};

template <typename VT, typename CT>
__global__ __launch_bounds__(kThreads) void elsaa_k4_race_build(
    const VT *__restrict__ v, const CT *__restrict__ kcodes, int N, int D, int L, int nb, int RB,
    int nr, int wg_per_cs, int wg_per_bh, int wg_real, float *__restrict__ tsum) {
  extern __shared__ __align__(16) float lds[];
  const int code_words = (kTK * L * static_cast<int>(sizeof(CT)) + 15) / 16;  // 16-byte words per tile
  float *tile = lds;                                         // [kTK + 1][64] fp32; row kTK is zero
  CT *tcode = reinterpret_cast<CT *>(lds + (kTK + 1) * 64);  // [kTK][L], in kThreads x 16 bytes
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // XCD-aware order: consecutive logical workgroups share an XCD.
  const int logical = static_cast<int>(xcd_logical_block(blockIdx.x, gridDim.x));
  if (logical >= wg_real) return;  // whole workgroup exits together
  const long long bh = logical / wg_per_bh;
  const int wg = logical % wg_per_bh;
  const int cs = wg / wg_per_cs;
  const int u = (wg % wg_per_cs) * kWaves + wave;
  const bool active = u < L * nr;
  const int l = active ? u / nr : 0;
  const int r = active ? u % nr : 0;
  const int base = r * RB;

  // one register vector (a wave-uniform element index compiles to M0-relative
  // moves); larger or split vectors make the compiler copy or select whole
  // vectors per add, so a wave owns at most 32 buckets
  f32x32 acc = {};
  if (tid < 64) tile[kTK * 64 + tid] = 0.0f;

  const long long seg = bh * N;
  const int tk = tid >> 3, tc = (tid & 7) * 8;  // tile loader: key tk, columns tc .. tc+7
  const VT *vsrc = v + seg * D + cs * 64 + tc;
  const uint4 *csrc = reinterpret_cast<const uint4 *>(kcodes + seg * L);  // 16-byte aligned: 64 L | N L
  const int n_tiles = N / kTK;  // N is a multiple of 64 (the chunk is)
  const bool code_loader = tid < code_words;

  auto load = [&](TileRegs<VT> &p, int t) {
    const int tt = t < n_tiles ? t : n_tiles - 1;  // past the end: reload the last tile
    const VT *src = vsrc + static_cast<long long>(tt * kTK + tk) * D;
    if constexpr (sizeof(VT) == 2) {
      *reinterpret_cast<u16x8 *>(p.x) = *reinterpret_cast<const u16x8 *>(src);
    } else {
      *reinterpret_cast<f32x4 *>(p.x) = *reinterpret_cast<const f32x4 *>(src);
      *reinterpret_cast<f32x4 *>(p.x + 4) = *reinterpret_cast<const f32x4 *>(src + 4);
    }
    p.c = csrc[static_cast<long long>(tt) * code_words + (code_loader ? tid : 0)];  // all threads load
  };

  auto step = [&](TileRegs<VT> &p, int t) {
    lds_barrier();  // previous tile fully consumed
    f32x4 lo, hi;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo[e] = Elem<VT>::load(p.x + e);
      hi[e] = Elem<VT>::load(p.x + 4 + e);
    }
    *reinterpret_cast<f32x4 *>(tile + tk * 64 + tc) = lo;
    *reinterpret_cast<f32x4 *>(tile + tk * 64 + tc + 4) = hi;
    reinterpret_cast<uint4 *>(tcode)[tid] = p.c;  // unconditional: words past the block are unused
    lds_barrier();
    load(p, t + 4);  // refill this ring slot four tiles ahead
    if (!active || t >= n_tiles) return;  // steps past the end only keep the ring uniform
    const int rel = static_cast<int>(tcode[lane * L + l]) - base;
    unsigned long long mask = __ballot(static_cast<unsigned>(rel) < static_cast<unsigned>(RB));
    while (mask) {
      int idx[kRound], rbs[kRound];
#pragma unroll
      for (int q = 0; q < kRound; ++q) {
        const bool any = mask != 0;
        const int i = any ? __builtin_ctzll(mask) : 0;
        mask &= mask - 1;
        idx[q] = any ? i : kTK;  // the zero row
        rbs[q] = any ? __builtin_amdgcn_readlane(rel, i) : 0;
      }
      float val[kRound];
#pragma unroll
      for (int q = 0; q < kRound; ++q) val[q] = tile[idx[q] * 64 + lane];
#pragma unroll
      for (int q = 0; q < kRound; ++q) acc[rbs[q]] += val[q];
    }
  };

  TileRegs<VT> p0, p1, p2, p3;
  load(p0, 0);
  load(p1, 1);
  load(p2, 2);
  load(p3, 3);
  // uniform trip count and an unconditional body: every wave reaches every
  // barrier, and the compiler can wait for one ring slot at a time
  for (int t = 0; t < n_tiles; t += 4) {
    step(p0, t);
    step(p1, t + 1);
    step(p2, t + 2);
    step(p3, t + 3);
  }

  if (!active) return;
  float *out = tsum + (bh * L + l) * static_cast<long long>(nb) * D + cs * 64 + lane;
#pragma unroll
  for (int rb = 0; rb < kMaxRB; ++rb)
    if (rb < RB) out[static_cast<long long>(base + rb) * D] = acc[rb];
}

// Bucket counts: one workgroup per (b, h, table), an LDS histogram of the N
// codes with integer atomics (exact in any order).
template <typename CT>
__global__ __launch_bounds__(256) void elsaa_k4_race_counts(const CT *__restrict__ kcodes, int N,
                                                            int L, int nb, float *__restrict__ tcnt) {
  extern __shared__ uint32_t hist[];
  const long long bh = blockIdx.y;
  const int l = blockIdx.x;
  for (int b = threadIdx.x; b < nb; b += 256) hist[b] = 0;
  __syncthreads();
  const CT *c = kcodes + bh * N * static_cast<long long>(L) + l;
  for (int j = threadIdx.x; j < N; j += 256) atomicAdd(&hist[c[static_cast<long long>(j) * L]], 1u);
  __syncthreads();
  float *out = tcnt + (bh * L + l) * static_cast<long long>(nb);
  for (int b = threadIdx.x; b < nb; b += 256) out[b] = static_cast<float>(hist[b]);
}

}  // namespace

hipError_t launch_race_build(const Geometry &g, const void *v, const Buffers &buf,
                             hipStream_t stream) {
  const int RB = g.nb_race < kMaxRB ? g.nb_race : kMaxRB;
  const int nr = g.nb_race / RB;
  const int ncs = g.D / 64;
  const int wg_per_cs = (g.L * nr + kWaves - 1) / kWaves;
  const int wg_per_bh = wg_per_cs * ncs;
  const long long wg_real = static_cast<long long>(wg_per_bh) * g.BH;
  const long long grid = (wg_real + kXcdCount - 1) / kXcdCount * kXcdCount;
  const size_t lds = static_cast<size_t>(kTK + 1) * 64 * 4 + static_cast<size_t>(kThreads) * 16;
  const void *rk = static_cast<const char *>(buf.rcode) + static_cast<size_t>(g.rows) * g.L * g.rcb;
  const dim3 cgrid(g.L, g.BH);
  const size_t clds = static_cast<size_t>(g.nb_race) * 4;
  if (g.rcb == 1)
    hipLaunchKernelGGL(elsaa_k4_race_counts<uint8_t>, cgrid, dim3(256), clds, stream,
                       static_cast<const uint8_t *>(rk), g.N, g.L, g.nb_race, buf.tcnt);
  else
    hipLaunchKernelGGL(elsaa_k4_race_counts<uint16_t>, cgrid, dim3(256), clds, stream,
                       static_cast<const uint16_t *>(rk), g.N, g.L, g.nb_race, buf.tcnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
#define ELSAA_K4_LAUNCH(VT, CT)                                                                   \
  hipLaunchKernelGGL((elsaa_k4_race_build<VT, CT>), dim3(grid), dim3(kThreads), lds, stream,     \
                     static_cast<const VT *>(v), static_cast<const CT *>(rk), g.N, g.D, g.L,      \
                     g.nb_race, RB, nr, wg_per_cs, wg_per_bh, static_cast<int>(wg_real), buf.tsum)
  if (g.bf16) {
    if (g.rcb == 1) ELSAA_K4_LAUNCH(uint16_t, uint8_t);
    else ELSAA_K4_LAUNCH(uint16_t, uint16_t);
  } else {
    if (g.rcb == 1) ELSAA_K4_LAUNCH(float, uint8_t);
    else ELSAA_K4_LAUNCH(float, uint16_t);
  }
#undef ELSAA_K4_LAUNCH
  return hipGetLastError();
}

}  // namespace elsaa
