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
// bf16 kernel (d = 64 or 128): one workgroup of 4 waves per 64 sorted queries
// (w is a multiple of 64, so a tile never straddles chunks).  Each wave owns 16
// queries.  Key blocks of 64 gathered rows are staged in LDS: K row-major
// (padded rows), V transposed (so the PV operand reads contiguous keys).
// S^T = K Q^T and O^T = V^T P^T run on 16x16x32 bf16 MFMA with fp32
// accumulation; the softmax is online (running max in the exp2 domain), with
// P rounded to bf16 for the PV product and the row sum taken from the fp32 P.
#include "elsaa_internal.hpp"

namespace elsaa {
namespace {

constexpr int kQTile = 64;
constexpr int kKBlock = 64;

template <int D>
__global__ __launch_bounds__(256) void elsaa_k3_chunk_attn_bf16(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ perm_q, const int32_t *__restrict__ perm_k, int N, int w,
    float scale_log2, uint16_t *__restrict__ o_s, float *__restrict__ lse) {
  constexpr int kKRow = D + 8;        // padded K row in LDS (bf16 elements)
  constexpr int kVRow = kKBlock + 8;  // padded V^T row in LDS
  __shared__ __align__(16) uint16_t Ks[kKBlock * kKRow];
  __shared__ __align__(16) uint16_t Vt[D * kVRow];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const long long bh = blockIdx.y;
  const int r0 = blockIdx.x * kQTile;
  const int c = r0 / w;
  const int lo = c > 0 ? (c - 1) * w : 0;
  const int hi = (c + 1) * w;
  const long long seg = bh * N;

  // Q^T operand: lane holds query (r16) of this wave, d-slice g*8 .. +7 of each 32.
  const int qidx = perm_q[seg + r0 + wave * 16 + r16];
  const uint16_t *qrow = q + (seg + qidx) * D;
  bf16x8 bq[D / 32];
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk)
    bq[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8 *>(qrow + kk * 32 + g * 8));

  f32x4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
  float m = -INFINITY;  // running max of score * log2(e) / sqrt(d)
  float l_part = 0.0f;  // this lane's share of the running sum

  for (int kb = lo; kb < hi; kb += kKBlock) {
    __syncthreads();  // previous block fully consumed
    // K block: 64 rows x D/8 chunks of 16 bytes
    for (int idx = tid; idx < kKBlock * (D / 8); idx += 256) {
      const int j = idx / (D / 8), ch = idx % (D / 8);
      const int kidx = perm_k[seg + kb + j];
      *reinterpret_cast<u16x8 *>(Ks + j * kKRow + ch * 8) =
          *reinterpret_cast<const u16x8 *>(k + (seg + kidx) * D + ch * 8);
    }
    // V block transposed: thread takes keys 2*jp, 2*jp+1 and an 8-wide d chunk
    for (int idx = tid; idx < (kKBlock / 2) * (D / 8); idx += 256) {
      const int jp = idx % (kKBlock / 2), ch = idx / (kKBlock / 2);
      const int k0 = perm_k[seg + kb + 2 * jp], k1 = perm_k[seg + kb + 2 * jp + 1];
      const u16x8 v0 = *reinterpret_cast<const u16x8 *>(v + (seg + k0) * D + ch * 8);
      const u16x8 v1 = *reinterpret_cast<const u16x8 *>(v + (seg + k1) * D + ch * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t word = static_cast<uint32_t>(v0[e]) | (static_cast<uint32_t>(v1[e]) << 16);
        *reinterpret_cast<uint32_t *>(Vt + (ch * 8 + e) * kVRow + 2 * jp) = word;
      }
    }
    __syncthreads();

    // S^T tiles: lane holds keys kt*16 + g*4 + i for query r16
    f32x4 s[kKBlock / 16];
#pragma unroll
    for (int kt = 0; kt < kKBlock / 16; ++kt) {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u16x8 *>(Ks + (kt * 16 + r16) * kKRow + kk * 32 + g * 8));
        acc = mfma16x16x32(a, bq[kk], acc);
      }
      s[kt] = acc;
    }
    float bmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < kKBlock / 16; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) bmax = fmaxf(bmax, s[kt][i]);
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
    const float m_new = fmaxf(m, bmax * scale_log2);
    const float corr = exp2f(m - m_new);  // 0 on the first block (m = -inf)
    m = m_new;
    l_part *= corr;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] *= corr;

    // P = exp2(s * scale - m); PV over two 32-key steps
#pragma unroll
    for (int m2 = 0; m2 < kKBlock / 32; ++m2) {
      u16x8 pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p0 = exp2f(__builtin_fmaf(s[2 * m2][i], scale_log2, -m));
        const float p1 = exp2f(__builtin_fmaf(s[2 * m2 + 1][i], scale_log2, -m));
        l_part += p0 + p1;
        pb[i] = f32_to_bf16_bits(p0);
        pb[4 + i] = f32_to_bf16_bits(p1);
      }
      const bf16x8 bp = __builtin_bit_cast(bf16x8, pb);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const uint16_t *vr = Vt + (dt * 16 + r16) * kVRow + m2 * 32 + g * 4;
        const u16x4 lo4 = *reinterpret_cast<const u16x4 *>(vr);
        const u16x4 hi4 = *reinterpret_cast<const u16x4 *>(vr + 16);
        const u16x8 av = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        o[dt] = mfma16x16x32(__builtin_bit_cast(bf16x8, av), bp, o[dt]);
      }
    }
  }

  float l_tot = l_part + __shfl_xor(l_part, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const float inv = 1.0f / l_tot;
  uint16_t *orow = o_s + (seg + qidx) * D;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    u16x4 outv;
#pragma unroll
    for (int i = 0; i < 4; ++i) outv[i] = f32_to_bf16_bits(o[dt][i] * inv);
    *reinterpret_cast<u16x4 *>(orow + dt * 16 + g * 4) = outv;
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

}  // namespace

hipError_t launch_chunk_attention(const Geometry &g, const void *q, const void *k, const void *v,
                                  const Buffers &buf, hipStream_t stream) {
  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(g.D));
  const int32_t *pq = buf.perm;
  const int32_t *pk = buf.perm + g.rows;
  if (g.bf16) {
    const dim3 grid(g.N / kQTile, g.BH);
    if (g.D == 64)
      hipLaunchKernelGGL(elsaa_k3_chunk_attn_bf16<64>, grid, dim3(256), 0, stream,
                         static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                         static_cast<const uint16_t *>(v), pq, pk, g.N, g.w, scale_log2,
                         static_cast<uint16_t *>(buf.o_s), buf.lse);
    else
      hipLaunchKernelGGL(elsaa_k3_chunk_attn_bf16<128>, grid, dim3(256), 0, stream,
                         static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                         static_cast<const uint16_t *>(v), pq, pk, g.N, g.w, scale_log2,
                         static_cast<uint16_t *>(buf.o_s), buf.lse);
  } else {
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
  }
  return hipGetLastError();
}

}  // namespace elsaa
