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

constexpr int kSortWavesMax = 16;
constexpr int kReduceBatch = 16;  // key rows in flight per wave

// ---------------------------------------------------------------------- sort --
template <typename CT>
__global__ __launch_bounds__(kSortWavesMax * 64) void elsaa_k4_race_sort(
    const CT *__restrict__ kcodes, int N, int L, int P, int chunk, int32_t *__restrict__ perm,
    int32_t *__restrict__ bstart) {
  extern __shared__ uint32_t cnt[];  // [waves][nb]: counts, then running offsets
  __shared__ uint32_t part[kSortWavesMax * 64];
  const int nb = 1 << P;
  const int nthreads = blockDim.x, waves = nthreads >> 6;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l = blockIdx.x;
  const long long bh = blockIdx.y;
  const long long seg = bh * N;
  const long long unit = bh * L + l;
  const CT *c = kcodes + seg * L + l;  // code of key j at c[j * L]
  const int j_begin = wave * chunk;
  const int j_end = j_begin + chunk < N ? j_begin + chunk : N;

  for (int i = tid; i < waves * nb; i += nthreads) cnt[i] = 0;
  __syncthreads();
  uint32_t *wc = cnt + wave * nb;
  // codes are read 8 rounds at a time so the loads overlap (one latency per 512 keys)
  auto load_codes = [&](int j0, uint32_t (&code)[8]) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int j = j0 + q * 64 + lane;
      code[q] = j < j_end ? static_cast<uint32_t>(c[static_cast<long long>(j) * L]) : 0xffffffffu;
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

  // bucket-major exclusive scan of the [bucket][wave] counts
  const int per = (nb + nthreads - 1) / nthreads;
  const int b_lo = tid * per < nb ? tid * per : nb;
  const int b_hi = b_lo + per < nb ? b_lo + per : nb;
  uint32_t sum = 0;
  for (int b = b_lo; b < b_hi; ++b)
    for (int w = 0; w < waves; ++w) sum += cnt[w * nb + b];
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < nthreads; off <<= 1) {  // inclusive Hillis-Steele scan
    const uint32_t add = tid >= off ? part[tid - off] : 0u;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  uint32_t run = part[tid] - sum;
  int32_t *bs = bstart + unit * (nb + 1);
  for (int b = b_lo; b < b_hi; ++b) {
    bs[b] = static_cast<int32_t>(run);
    for (int w = 0; w < waves; ++w) {
      const uint32_t t = cnt[w * nb + b];
      cnt[w * nb + b] = run;
      run += t;
    }
  }
  if (tid == 0) bs[nb] = N;
  __syncthreads();

  // stable ranks: each wave walks its chunk in order, 64 keys per round
  int32_t *pm = perm + unit * N;
  const unsigned long long lt = (1ull << lane) - 1ull;
  for (int j8 = j_begin; j8 < j_end; j8 += 512) {
  uint32_t codes8[8];
  load_codes(j8, codes8);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int j0 = j8 + q * 64;
    const int j = j0 + lane;
    const bool valid = j < j_end;
    const uint32_t code = valid ? codes8[q] : 0u;
    unsigned long long mask = __ballot(valid);
    for (int bit = 0; bit < P; ++bit) {
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
    if (valid) pm[before + rank] = j;
    // the leader's counter update must land before the next round reads it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  }
  }
}

// -------------------------------------------------------------------- reduce --
template <typename VT>
__global__ __launch_bounds__(256) void elsaa_k4_race_reduce(
    const VT *__restrict__ v, const int32_t *__restrict__ perm, const int32_t *__restrict__ bstart,
    int N, int D, int L, int P, int ncs, int parts, long long units, float *__restrict__ tsum,
    float *__restrict__ tcnt) {
  const int lane = threadIdx.x & 63;
  // consecutive units (same (b, h), same value rows) run on one XCD's L2
  const long long u = xcd_logical_block(blockIdx.x, gridDim.x) * 4 + (threadIdx.x >> 6);
  if (u >= units) return;  // whole wave
  const int nb = 1 << P;
  const int part = static_cast<int>(u % parts);
  const int cs = static_cast<int>((u / parts) % ncs);
  const long long tu = u / (static_cast<long long>(parts) * ncs);  // (b, h) * L + table
  const long long bh = tu / L;
  const int32_t *bs = bstart + tu * (nb + 1);
  const int32_t *pm = perm + tu * N;
  const VT *vcol = v + bh * N * static_cast<long long>(D) + cs * 64 + lane;

  // buckets owned: those whose run starts in [lo, hi); the last part also owns
  // the empty buckets that start at N
  const int lo = static_cast<int>(static_cast<long long>(N) * part / parts);
  const int hi = part == parts - 1 ? N + 1 : static_cast<int>(static_cast<long long>(N) * (part + 1) / parts);
  int b0 = nb, b1 = nb;
  for (int bb = 0; bb < nb; bb += 64) {
    const int b = bb + lane;
    const int s = b < nb ? bs[b] : N + 1;
    const unsigned long long ge_lo = __ballot(b < nb && s >= lo);
    const unsigned long long ge_hi = __ballot(b < nb && s >= hi);
    if (b0 == nb && ge_lo) b0 = bb + __builtin_ctzll(ge_lo);
    if (b1 == nb && ge_hi) b1 = bb + __builtin_ctzll(ge_hi);
  }

  for (int b = b0; b < b1; ++b) {
    const int p0 = bs[b], p1 = bs[b + 1];
    float acc = 0.0f;
    for (int p = p0; p < p1; p += kReduceBatch) {
      const int n = p1 - p < kReduceBatch ? p1 - p : kReduceBatch;
      // lanes 0..15 fetch the batch's key indices (clamped inside the run)
      const int jl = pm[p + (lane < n ? lane : n - 1)];
      float val[kReduceBatch];
#pragma unroll
      for (int q = 0; q < kReduceBatch; ++q) {
        const int j = __builtin_amdgcn_readlane(jl, q < n ? q : n - 1);
        val[q] = Elem<VT>::load(vcol + static_cast<long long>(j) * D);
      }
#pragma unroll
      for (int q = 0; q < kReduceBatch; ++q)
        if (q < n) acc += val[q];  // ascending key order within the bucket
    }
    tsum[(tu * nb + b) * static_cast<long long>(D) + cs * 64 + lane] = acc;
    if (cs == 0 && lane == 0) tcnt[tu * nb + b] = static_cast<float>(p1 - p0);
  }
}

}  // namespace

hipError_t launch_race_build(const Geometry &g, const void *v, const Buffers &buf,
                             hipStream_t stream) {
  const int nb = g.nb_race;
  int waves = 16384 / nb;  // LDS counts: waves * nb * 4 bytes <= 64 KB
  waves = waves < 1 ? 1 : (waves > kSortWavesMax ? kSortWavesMax : waves);
  const int chunk = ((g.N + waves - 1) / waves + 63) / 64 * 64;
  const void *rk = static_cast<const char *>(buf.rcode) + static_cast<size_t>(g.rows) * g.L * g.rcb;
  const dim3 sgrid(g.L, g.BH);
  const size_t slds = static_cast<size_t>(waves) * nb * 4;
  if (g.rcb == 1)
    hipLaunchKernelGGL(elsaa_k4_race_sort<uint8_t>, sgrid, dim3(waves * 64), slds, stream,
                       static_cast<const uint8_t *>(rk), g.N, g.L, g.P, chunk, buf.rperm, buf.rstart);
  else
    hipLaunchKernelGGL(elsaa_k4_race_sort<uint16_t>, sgrid, dim3(waves * 64), slds, stream,
                       static_cast<const uint16_t *>(rk), g.N, g.L, g.P, chunk, buf.rperm, buf.rstart);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int ncs = g.D / 64;
  const long long tables = static_cast<long long>(g.BH) * g.L * ncs;
  long long parts = (8192 + tables - 1) / tables;  // aim for ~8K waves
  parts = parts < 1 ? 1 : (parts > nb ? nb : parts);
  const long long units = tables * parts;
  const dim3 rgrid(static_cast<unsigned>(((units + 3) / 4 + kXcdCount - 1) / kXcdCount * kXcdCount));
  if (g.bf16)
    hipLaunchKernelGGL(elsaa_k4_race_reduce<uint16_t>, rgrid, dim3(256), 0, stream,
                       static_cast<const uint16_t *>(v), buf.rperm, buf.rstart, g.N, g.D, g.L, g.P,
                       ncs, static_cast<int>(parts), units, buf.tsum, buf.tcnt);
  else
    hipLaunchKernelGGL(elsaa_k4_race_reduce<float>, rgrid, dim3(256), 0, stream,
                       static_cast<const float *>(v), buf.rperm, buf.rstart, g.N, g.D, g.L, g.P, ncs,
                       static_cast<int>(parts), units, buf.tsum, buf.tcnt);
  return hipGetLastError();
}

}  // namespace elsaa
