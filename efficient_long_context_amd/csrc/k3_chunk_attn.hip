// k3_chunk_attn.hip -- exact softmax attention inside Sort-LSH chunks.
//
// The sparse branch evaluates its selected query-key pairs exactly ("Two
// Efficient Attentions, One Denominator Problem", section "Two efficient
// branches can still be mis-scaled").  Selection: queries and keys are in
// bucket-sorted order; the chunk c of w sorted queries attends the sorted keys
// [max(0, (c-1) w), (c+1) w) -- its own chunk and the previous one.  Scores are
// <q, k> / sqrt(d), non-causal, unmasked.  Outputs, at the query's original
// position: o_s = softmax-weighted sum of values, and lse = log sum exp(score),
// the log of the sparse branch's softmax mass Z_s used by the fusion.
//
// bf16 kernel (d = 64 or 128): one workgroup per QT sorted queries (QT = 128
// with 8 waves when w is a multiple of 128, else 64 with 4 waves; a tile never
// straddles chunks).  Each wave owns 16 queries, whose Q^T fragments stay in
// registers.  Key blocks of 64 gathered rows are staged in LDS -- K row-major
// (padded rows), V transposed so the PV operand reads contiguous keys -- and
// the next block's rows are loaded into registers while the current one is
// used.  S^T = K Q^T and O^T = V^T P^T run on 16x16x32 bf16 MFMA with fp32
// accumulation; the softmax is online in the exp2 domain (v_exp_f32 directly:
// every argument is <= 0), P is rounded to bf16 for the PV product and the row
// sum is taken from the fp32 P.  Workgroups of neighbouring tiles (which share
// key blocks) are mapped to the same XCD.
#include "elsaa_internal.hpp"

namespace elsaa {
namespace {

constexpr int kKBlock = 64;



template <int D, int QT, int NB>
__global__ __launch_bounds__(QT * 4) void elsaa_k3_chunk_attn_bf16(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ perm_q, const int32_t *__restrict__ perm_k, int N, int w,
    int tiles_per_seg, int n_tiles, float scale_log2, uint16_t *__restrict__ o_s,
    float *__restrict__ lse) {
  constexpr int kThreads = QT * 4;      // 16 queries per wave
  constexpr int kKeys = NB * kKBlock;   // keys staged at once
  constexpr int kKRow = D + 8;          // padded K row in LDS (bf16 elements)
  constexpr int kVRow = kKeys + 4;      // padded V^T row in LDS: 2-word bank shift per row
  constexpr int kKChunks = kKeys * (D / 8);          // 16-byte pieces of the staged K rows
  constexpr int kVPairs = (kKeys / 2) * (D / 8);     // (key pair, 8-column) pieces of V
  constexpr int kKPer = (kKChunks + kThreads - 1) / kThreads;
  constexpr int kVPer = (kVPairs + kThreads - 1) / kThreads;
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t *Ks = smem;                  // [kKeys][kKRow]
  uint16_t *Vt = smem + kKeys * kKRow;  // [D][kVRow]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const long long tile = xcd_logical_block(blockIdx.x, gridDim.x);
  if (tile >= n_tiles) return;  // padding workgroup (whole group exits)
  const long long bh = tile / tiles_per_seg;
  const int r0 = static_cast<int>(tile % tiles_per_seg) * QT;
  const int c = r0 / w;
  const int lo = c > 0 ? (c - 1) * w : 0;
  const int hi = (c + 1) * w;
  const long long seg = bh * N;
  const int32_t *pk = perm_k + seg;

  // Q^T operand: lane holds query r16 of this wave, d-slice g*8 .. +7 of each 32.
  const int qidx = perm_q[seg + r0 + wave * 16 + r16];
  const uint16_t *qrow = q + (seg + qidx) * D;
  bf16x8 bq[D / 32];
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk)
    bq[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8 *>(qrow + kk * 32 + g * 8));

  f32x4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
  // m: the reference point of the exponentials, score * log2(e) / sqrt(d)
  // units; it trails the running maximum by less than kLazy, so every
  // exp2(s - m) stays below 2^kLazy and o and l are rescaled only when the
  // maximum grows past it (the final o / l does not depend on m).
  constexpr float kLazy = 8.0f;
  float m = -INFINITY;
  // running sum of the bfloat16 weights P (the ones fed to the PV product):
  // a 16x16x32 product of an all-ones A with P, every lane of query r16
  // holds the column sum
  f32x4 l_acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const bf16x8 ones = __builtin_bit_cast(bf16x8, (u16x8)0x3f80);

  // Stages of up to NB key blocks: all of a stage's rows are requested at
  // once (K piece i -> row i / (D/8), chunk i % (D/8); V piece i -> key pair
  // i % (kKeys/2), chunk i / (kKeys/2)), staged in LDS (V transposed) behind
  // one barrier, then the stage's blocks are processed without further syncs.
  // With a window of 2w <= kKeys keys the whole window is one stage.
  for (int s0 = lo; s0 < hi; s0 += kKeys) {
    const int nkeys = hi - s0 < kKeys ? hi - s0 : kKeys;  // a multiple of 64
    int kj[kKPer], v0[kVPer], v1[kVPer];
#pragma unroll
    for (int p = 0; p < kKPer; ++p) {
      int j = (tid + p * kThreads) / (D / 8);
      j = j < nkeys ? j : nkeys - 1;  // clamped: rows past the stage are reloads, not used
      kj[p] = pk[s0 + j];
    }
#pragma unroll
    for (int p = 0; p < kVPer; ++p) {
      int jp = (tid + p * kThreads) % (kKeys / 2);
      jp = 2 * jp + 1 < nkeys ? jp : nkeys / 2 - 1;
      v0[p] = pk[s0 + 2 * jp];
      v1[p] = pk[s0 + 2 * jp + 1];
    }
    u16x8 kreg[kKPer], vreg0[kVPer], vreg1[kVPer];
#pragma unroll
    for (int p = 0; p < kKPer; ++p) {
      const int i = tid + p * kThreads;
      kreg[p] = *reinterpret_cast<const u16x8 *>(k + (seg + kj[p]) * D + (i % (D / 8)) * 8);
    }
#pragma unroll
    for (int p = 0; p < kVPer; ++p) {
      const int ch = ((tid + p * kThreads) / (kKeys / 2)) % (D / 8);
      vreg0[p] = *reinterpret_cast<const u16x8 *>(v + (seg + v0[p]) * D + ch * 8);
      vreg1[p] = *reinterpret_cast<const u16x8 *>(v + (seg + v1[p]) * D + ch * 8);
    }
    if (s0 != lo) __syncthreads();  // previous stage fully consumed
#pragma unroll
    for (int p = 0; p < kKPer; ++p) {
      const int i = tid + p * kThreads;
      if (i < kKChunks) {
        const int j = i / (D / 8), ch = i % (D / 8);
        *reinterpret_cast<u16x8 *>(Ks + j * kKRow + ch * 8) = kreg[p];
      }
    }
#pragma unroll
    for (int p = 0; p < kVPer; ++p) {
      const int i = tid + p * kThreads;
      if (i < kVPairs) {
        const int jp = i % (kKeys / 2), ch = i / (kKeys / 2);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t word = static_cast<uint32_t>(vreg0[p][e]) | (static_cast<uint32_t>(vreg1[p][e]) << 16);
          *reinterpret_cast<uint32_t *>(Vt + (ch * 8 + e) * kVRow + 2 * jp) = word;
        }
      }
    }
    __syncthreads();

    for (int blk = 0; blk < nkeys / kKBlock; ++blk) {
      const uint16_t *Kb = Ks + blk * kKBlock * kKRow;
      // S^T tiles: lane holds keys kt*16 + g*4 + i for query r16
      f32x4 s[kKBlock / 16];
#pragma unroll
      for (int kt = 0; kt < kKBlock / 16; ++kt) {
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
          const bf16x8 a = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u16x8 *>(Kb + (kt * 16 + r16) * kKRow + kk * 32 + g * 8));
          acc = mfma16x16x32(a, bq[kk], acc);
        }
        s[kt] = acc;
      }
      float bmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < kKBlock / 16; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) bmax = fmaxf(bmax, s[kt][i]);
      {  // max over the 4 lane groups (lanes r16, r16 + 16, r16 + 32, r16 + 48)
        const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(bmax), __float_as_uint(bmax), false, false);
        bmax = fmaxf(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
        const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(bmax), __float_as_uint(bmax), false, false);
        bmax = fmaxf(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
      }
      const float m_blk = bmax * scale_log2;
      if (__ballot(m_blk > m + kLazy)) {  // some query of the wave moves its reference point
        const float m_new = fmaxf(m, m_blk);
        const float corr = __builtin_amdgcn_exp2f(m - m_new);  // 0 on the first block (m = -inf)
        m = m_new;
        l_acc *= corr;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[dt] *= corr;
      }

      // P = exp2(s * scale - m); PV over two 32-key steps
#pragma unroll
      for (int m2 = 0; m2 < kKBlock / 32; ++m2) {
        uint32_t pw[4];
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * m2][i], scale_log2, -m));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * m2][i + 1], scale_log2, -m));
          const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * m2 + 1][i], scale_log2, -m));
          const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * m2 + 1][i + 1], scale_log2, -m));
          pw[i / 2] = pack_bf16x2(p0, p1);
          pw[2 + i / 2] = pack_bf16x2(p2, p3);
        }
        const bf16x8 bp = __builtin_bit_cast(bf16x8, (uint4){pw[0], pw[1], pw[2], pw[3]});
        l_acc = mfma16x16x32(ones, bp, l_acc);
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const uint16_t *vr = Vt + (dt * 16 + r16) * kVRow + blk * kKBlock + m2 * 32 + g * 4;
          const uint2 lo4 = *reinterpret_cast<const uint2 *>(vr);
          const uint2 hi4 = *reinterpret_cast<const uint2 *>(vr + 16);
          const bf16x8 av = __builtin_bit_cast(bf16x8, (uint4){lo4.x, lo4.y, hi4.x, hi4.y});
          o[dt] = mfma16x16x32(av, bp, o[dt]);
        }
      }
    }
  }

  const float l_tot = l_acc[0];
  const float inv = 1.0f / l_tot;
  uint16_t *orow = o_s + (seg + qidx) * D;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const uint2 outv = {pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv),
                        pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv)};
    *reinterpret_cast<uint2 *>(orow + dt * 16 + g * 4) = outv;
  }
  if (g == 0) lse[seg + qidx] = (m + log2f(l_tot)) * 0.69314718055994530942f;
}

// fp32 inputs: one thread per sorted query, binary32 arithmetic throughout.
template <int D>
__global__ __launch_bounds__(128) void elsaa_k3_chunk_attn_f32(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const int32_t *__restrict__ perm_q, const int32_t *__restrict__ perm_k, int N, int w,
    float scale_log2, float *__restrict__ o_s, float *__restrict__ lse) {
  const int rank = blockIdx.x * 128 + threadIdx.x;
  if (rank >= N) return;
  const long long seg = static_cast<long long>(blockIdx.y) * N;
  const int c = rank / w;
  const int lo = c > 0 ? (c - 1) * w : 0;
  const int hi = (c + 1) * w;
  const int qidx = perm_q[seg + rank];
  const float *qr = q + (seg + qidx) * D;
  float acc[D];
  for (int e = 0; e < D; ++e) acc[e] = 0.0f;
  float m = -INFINITY, l = 0.0f;
  for (int t = lo; t < hi; ++t) {
    const int kidx = perm_k[seg + t];
    const float *kr = k + (seg + kidx) * D;
    float dot = 0.0f;
    for (int e = 0; e < D; ++e) dot = __builtin_fmaf(qr[e], kr[e], dot);
    const float s2 = dot * scale_log2;
    const float m_new = fmaxf(m, s2);
    const float corr = exp2f(m - m_new);
    const float p = exp2f(s2 - m_new);
    m = m_new;
    l = l * corr + p;
    const float *vr = v + (seg + kidx) * D;
    for (int e = 0; e < D; ++e) acc[e] = acc[e] * corr + p * vr[e];
  }
  const float inv = 1.0f / l;
  float *orow = o_s + (seg + qidx) * D;
  for (int e = 0; e < D; ++e) orow[e] = acc[e] * inv;
  lse[seg + qidx] = (m + log2f(l)) * 0.69314718055994530942f;
}

// LDS bytes of the bf16 kernel staging NB key blocks.
constexpr size_t attn_lds_bytes(int D, int NB) {
  return (static_cast<size_t>(NB) * kKBlock * (D + 8) + static_cast<size_t>(D) * (NB * kKBlock + 4)) * 2;
}

template <int D, int QT, int NB>
hipError_t launch_bf16(const Geometry &g, const void *q, const void *k, const void *v,
                       const Buffers &buf, float scale_log2, hipStream_t stream) {
  const int tiles_per_seg = g.N / QT;
  const long long n_tiles = static_cast<long long>(tiles_per_seg) * g.BH;
  const long long grid = (n_tiles + kXcdCount - 1) / kXcdCount * kXcdCount;
  hipLaunchKernelGGL((elsaa_k3_chunk_attn_bf16<D, QT, NB>), dim3(static_cast<unsigned>(grid)),
                     dim3(QT * 4), attn_lds_bytes(D, NB), stream, static_cast<const uint16_t *>(q),
                     static_cast<const uint16_t *>(k), static_cast<const uint16_t *>(v), buf.perm,
                     buf.perm + g.rows, g.N, g.w, tiles_per_seg, static_cast<int>(n_tiles),
                     scale_log2, static_cast<uint16_t *>(buf.o_s), buf.lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_attention(const Geometry &g, const void *q, const void *k, const void *v,
                                  const Buffers &buf, hipStream_t stream) {
  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(g.D));
  const int32_t *pq = buf.perm;
  const int32_t *pk = buf.perm + g.rows;
  if (g.bf16) {
    // 128-query tiles when w allows; key stages of 4 blocks (d = 64: the whole
    // 256-key window of w = 128) or 2, keeping LDS <= 72 KB (two workgroups
    // per CU)
    const bool wide = g.w % 128 == 0;
    if (g.D == 64)
      return wide ? launch_bf16<64, 128, 4>(g, q, k, v, buf, scale_log2, stream)
                  : launch_bf16<64, 64, 2>(g, q, k, v, buf, scale_log2, stream);
    return wide ? launch_bf16<128, 128, 2>(g, q, k, v, buf, scale_log2, stream)
                : launch_bf16<128, 64, 2>(g, q, k, v, buf, scale_log2, stream);
  }
  const dim3 grid((g.N + 127) / 128, g.BH);
  if (g.D == 64)
    hipLaunchKernelGGL(elsaa_k3_chunk_attn_f32<64>, grid, dim3(128), 0, stream,
                       static_cast<const float *>(q), static_cast<const float *>(k),
                       static_cast<const float *>(v), pq, pk, g.N, g.w, scale_log2,
                       static_cast<float *>(buf.o_s), buf.lse);
  else
    hipLaunchKernelGGL(elsaa_k3_chunk_attn_f32<128>, grid, dim3(128), 0, stream,
                       static_cast<const float *>(q), static_cast<const float *>(k),
                       static_cast<const float *>(v), pq, pk, g.N, g.w, scale_log2,
                       static_cast<float *>(buf.o_s), buf.lse);
  return hipGetLastError();
}

}  // namespace elsaa
