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
// accumulation; the softmax is online in the exp2 domain (v_exp_f32 directly)
// with a lazily moved reference point, so an exponent argument can reach +8
// (see attend_stage); P is rounded to bf16 for the PV product and the row sum
// is the sum of those bf16 weights (an MFMA of an all-ones operand with P).
// Workgroups of neighbouring tiles (which share key blocks) are mapped to the
// same XCD.  At d = 128 with w a multiple of 256, a workgroup takes 256
// queries (eight waves of 32) and every wave also stages key blocks.  With one sort bucket (sort_bits = 0) the sorted order is the
// original one: the kIdent instances index tokens directly and read no
// permutation.
#include <type_traits>

#include "elsaa_internal.hpp"

namespace elsaa {
namespace {

constexpr int kKBlock = 64;

// Original index of sorted rank r of the segment starting at row `seg`: the
// permutation's entry, or r itself when the order is the identity.
template <bool kIdent>
__device__ __forceinline__ int sorted_index(const int32_t *__restrict__ perm, long long seg, int r) {
  if constexpr (kIdent) {
    return r;
  } else {
    return perm[seg + r];
  }
}



// One stage of staged keys (nkeys, a multiple of 64, of at most kKeys) for
// QG groups of 16 queries of a wave: S^T = K Q^T on MFMA (each K fragment read
// from LDS serves every group), the online softmax in the exp2 domain with a
// lazily moved reference point m, P rounded to bfloat16, O^T += V^T P^T (each
// V fragment serves every group) and the running row sum of P (an all-ones A
// times P).  m trails the running maximum by less than kLazy, so every
// exp2(s - m) stays below 2^kLazy and o and l are rescaled only when the
// maximum grows past it (the final o / l does not depend on m).
template <int D, int kKeys, int QG>
__device__ __forceinline__ void attend_stage(const uint16_t *Ks, const uint16_t *Vt, int nkeys,
                                             const bf16x8 (&bq)[QG][D / 32], f32x4 (&o)[QG][D / 16],
                                             f32x4 (&l_acc)[QG], float (&m)[QG], float scale_log2,
                                             const bf16x8 &ones, int g, int r16) {
  constexpr int kKRow = D + 8;
  constexpr int kVRow = kKeys + 4;
  constexpr float kLazy = 8.0f;
  for (int blk = 0; blk < nkeys / kKBlock; ++blk) {
    const uint16_t *Kb = Ks + blk * kKBlock * kKRow;
    // S^T tiles: lane holds keys kt*16 + g*4 + i for query r16 of each group
    f32x4 s[QG][kKBlock / 16];
#pragma unroll
    for (int kt = 0; kt < kKBlock / 16; ++kt) {
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) s[qg][kt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u16x8 *>(Kb + (kt * 16 + r16) * kKRow + kk * 32 + g * 8));
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) s[qg][kt] = mfma16x16x32(a, bq[qg][kk], s[qg][kt]);
      }
    }
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
      float bmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < kKBlock / 16; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) bmax = fmaxf(bmax, s[qg][kt][i]);
      // max over the 4 lane groups (lanes r16, r16 + 16, r16 + 32, r16 + 48)
      const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(bmax), __float_as_uint(bmax), false, false);
      bmax = fmaxf(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
      const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(bmax), __float_as_uint(bmax), false, false);
      bmax = fmaxf(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
      const float m_blk = bmax * scale_log2;
      if (__ballot(m_blk > m[qg] + kLazy)) {  // some query of the group moves its reference point
        const float m_new = fmaxf(m[qg], m_blk);
        const float corr = __builtin_amdgcn_exp2f(m[qg] - m_new);  // 0 on the first block (m = -inf)
        m[qg] = m_new;
        l_acc[qg] *= corr;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[qg][dt] *= corr;
      }
    }

    // P = exp2(s * scale - m); PV over two 32-key steps
#pragma unroll
    for (int m2 = 0; m2 < kKBlock / 32; ++m2) {
      bf16x8 bp[QG];
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) {
        uint32_t pw[4];
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qg][2 * m2][i], scale_log2, -m[qg]));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qg][2 * m2][i + 1], scale_log2, -m[qg]));
          const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qg][2 * m2 + 1][i], scale_log2, -m[qg]));
          const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qg][2 * m2 + 1][i + 1], scale_log2, -m[qg]));
          pw[i / 2] = pack_bf16x2(p0, p1);
          pw[2 + i / 2] = pack_bf16x2(p2, p3);
        }
        bp[qg] = __builtin_bit_cast(bf16x8, (uint4){pw[0], pw[1], pw[2], pw[3]});
        l_acc[qg] = mfma16x16x32(ones, bp[qg], l_acc[qg]);
      }
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const uint16_t *vr = Vt + (dt * 16 + r16) * kVRow + blk * kKBlock + m2 * 32 + g * 4;
        const uint2 lo4 = *reinterpret_cast<const uint2 *>(vr);
        const uint2 hi4 = *reinterpret_cast<const uint2 *>(vr + 16);
        const bf16x8 av = __builtin_bit_cast(bf16x8, (uint4){lo4.x, lo4.y, hi4.x, hi4.y});
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) o[qg][dt] = mfma16x16x32(av, bp[qg], o[qg][dt]);
      }
    }
  }
}

// NBLK key blocks of 64 (K row-major with rows of D + 8, V transposed with
// rows of kVRow) for the 16 queries of a wave, fully unrolled and software
// pipelined: block b + 1's S^T products are issued before block b's softmax,
// so the matrix cores work while the vector ALUs exponentiate.  Same
// arithmetic as attend_stage.
template <int D, int kVRow, int NBLK>
__device__ __forceinline__ void attend_blocks(const uint16_t *const (&Kb)[NBLK], const uint16_t *const (&Vb)[NBLK],
                                              const bf16x8 (&bq)[D / 32], f32x4 (&o)[D / 16], f32x4 &l_acc,
                                              float &m, float scale_log2, const bf16x8 &ones, int g, int r16) {
  constexpr int kKRow = D + 8;
  constexpr float kLazy = 8.0f;
  auto scores = [&](const uint16_t *K, f32x4 (&s)[kKBlock / 16]) {
#pragma unroll
    for (int kt = 0; kt < kKBlock / 16; ++kt) {
      s[kt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u16x8 *>(K + (kt * 16 + r16) * kKRow + kk * 32 + g * 8));
        s[kt] = mfma16x16x32(a, bq[kk], s[kt]);
      }
    }
  };
  f32x4 s[2][kKBlock / 16];
  scores(Kb[0], s[0]);
#pragma unroll
  for (int b = 0; b < NBLK; ++b) {
    f32x4 (&sc)[kKBlock / 16] = s[b & 1];
    if (b + 1 < NBLK) scores(Kb[b + 1], s[(b + 1) & 1]);
    float bmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < kKBlock / 16; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) bmax = fmaxf(bmax, sc[kt][i]);
    const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(bmax), __float_as_uint(bmax), false, false);
    bmax = fmaxf(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
    const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(bmax), __float_as_uint(bmax), false, false);
    bmax = fmaxf(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
    const float m_blk = bmax * scale_log2;
    if (__ballot(m_blk > m + kLazy)) {
      const float m_new = fmaxf(m, m_blk);
      const float corr = __builtin_amdgcn_exp2f(m - m_new);
      m = m_new;
      l_acc *= corr;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) o[dt] *= corr;
    }
#pragma unroll
    for (int m2 = 0; m2 < kKBlock / 32; ++m2) {
      uint32_t pw[4];
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[2 * m2][i], scale_log2, -m));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[2 * m2][i + 1], scale_log2, -m));
        const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[2 * m2 + 1][i], scale_log2, -m));
        const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[2 * m2 + 1][i + 1], scale_log2, -m));
        pw[i / 2] = pack_bf16x2(p0, p1);
        pw[2 + i / 2] = pack_bf16x2(p2, p3);
      }
      const bf16x8 bp = __builtin_bit_cast(bf16x8, (uint4){pw[0], pw[1], pw[2], pw[3]});
      l_acc = mfma16x16x32(ones, bp, l_acc);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const uint16_t *vr = Vb[b] + (dt * 16 + r16) * kVRow + m2 * 32 + g * 4;
        const uint2 lo4 = *reinterpret_cast<const uint2 *>(vr);
        const uint2 hi4 = *reinterpret_cast<const uint2 *>(vr + 16);
        const bf16x8 av = __builtin_bit_cast(bf16x8, (uint4){lo4.x, lo4.y, hi4.x, hi4.y});
        o[dt] = mfma16x16x32(av, bp, o[dt]);
      }
    }
  }
}

template <int D, int QT, int NB, bool kIdent>
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

  // Q^T operand: lane holds query r16 of this wave, d-slice g*8 .. +7 of each 32.
  const int qidx = sorted_index<kIdent>(perm_q, seg, r0 + wave * 16 + r16);
  const uint16_t *qrow = q + (seg + qidx) * D;
  bf16x8 bq[1][D / 32];
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk)
    bq[0][kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8 *>(qrow + kk * 32 + g * 8));

  f32x4 o[1][D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[0][dt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
  // m: the reference point of the exponentials, in score * log2(e) / sqrt(d)
  // units; l_acc: the running sum of the bfloat16 weights P (those fed to
  // the PV product) as a 16x16x32 product of an all-ones A with P: every
  // lane of query r16 holds the column sum
  float m[1] = {-INFINITY};
  f32x4 l_acc[1] = {{0.0f, 0.0f, 0.0f, 0.0f}};
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
      kj[p] = sorted_index<kIdent>(perm_k, seg, s0 + j);
    }
#pragma unroll
    for (int p = 0; p < kVPer; ++p) {
      int jp = (tid + p * kThreads) % (kKeys / 2);
      jp = 2 * jp + 1 < nkeys ? jp : nkeys / 2 - 1;
      v0[p] = sorted_index<kIdent>(perm_k, seg, s0 + 2 * jp);
      v1[p] = sorted_index<kIdent>(perm_k, seg, s0 + 2 * jp + 1);
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

    attend_stage<D, kKeys, 1>(Ks, Vt, nkeys, bq, o, l_acc, m, scale_log2, ones, g, r16);
  }

  const float l_tot = l_acc[0][0];
  const float inv = 1.0f / l_tot;
  uint16_t *orow = o_s + (seg + qidx) * D;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const uint2 outv = {pack_bf16x2(o[0][dt][0] * inv, o[0][dt][1] * inv),
                        pack_bf16x2(o[0][dt][2] * inv, o[0][dt][3] * inv)};
    *reinterpret_cast<uint2 *>(orow + dt * 16 + g * 4) = outv;
  }
  if (g == 0) lse[seg + qidx] = (m[0] + log2f(l_tot)) * 0.69314718055994530942f;
}

// Pipelined bf16 kernel for 128-query tiles (w a multiple of 128): one
// persistent workgroup per compute unit walks a contiguous run of tiles
// (neighbouring tiles share key rows, which then come from the XCD's L2).  A
// job is one stage of up to NB key blocks of one tile.  Waves 0-3 (consumers,
// 32 queries each as two groups of 16 that share every K and V fragment read
// from LDS) compute job n from one LDS buffer while waves 4-7 (producers)
// write job n+1's K rows and transposed V rows, loaded into registers during
// job n-1, into the other buffer, then request job n+2's rows and job n+3's
// key indices.  One barrier per job separates the two; it orders LDS only, so
// loads stay in flight across it.  Consumers also load the next tile's query
// rows one tile ahead.
template <int D, int NB, bool kIdent>
__global__ __launch_bounds__(512) void elsaa_k3_chunk_attn_pc(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ perm_q, const int32_t *__restrict__ perm_k, int N, int w,
    int tiles_per_seg, long long n_tiles, long long tiles_per_wg, float scale_log2,
    uint16_t *__restrict__ o_s, float *__restrict__ lse) {
  constexpr int QT = 128;
  constexpr int QG = 2;  // query groups of 16 per consumer wave
  constexpr int kConsumerWaves = QT / (16 * QG);
  constexpr int kPThreads = 256;                   // producer threads
  constexpr int kKeys = NB * kKBlock;
  constexpr int kKRow = D + 8;
  constexpr int kVRow = kKeys + 4;
  constexpr int kBufElems = kKeys * kKRow + D * kVRow;
  constexpr int kKChunks = kKeys * (D / 8);        // 16-byte pieces of K rows
  constexpr int kVPairs = (kKeys / 2) * (D / 8);   // (key pair, 8-column) pieces of V
  static_assert(kKChunks % kPThreads == 0 && kVPairs % kPThreads == 0, "producer share");
  constexpr int kKPer = kKChunks / kPThreads;
  constexpr int kVPer = kVPairs / kPThreads;
  extern __shared__ __align__(16) uint16_t smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long long t_begin = xcd_logical_block(blockIdx.x, gridDim.x) * tiles_per_wg;
  const long long t_end = t_begin + tiles_per_wg < n_tiles ? t_begin + tiles_per_wg : n_tiles;
  if (t_begin >= t_end) return;  // whole workgroup

  // Jobs: (tile, first key of the stage); a tile's window is [lo, hi).  The
  // sequence is the same in every wave; a job at tile t_end means "none".
  struct Job { long long tile; int s0, lo, hi; };
  auto first_job = [&](long long t) {
    const int c = static_cast<int>(t % tiles_per_seg) * QT / w;
    Job j{t, 0, c > 0 ? (c - 1) * w : 0, (c + 1) * w};
    j.s0 = j.lo;
    return j;
  };
  auto next_job = [&](const Job &j) {
    if (j.s0 + kKeys < j.hi) return Job{j.tile, j.s0 + kKeys, j.lo, j.hi};
    return first_job(j.tile + 1);
  };

  if (wave >= kConsumerWaves) {
    // ------------------------------------------------------------ producer
    const int ptid = tid - kConsumerWaves * 64;
    int kj[kKPer], v0[kVPer], v1[kVPer];  // key indices of the next job to load
    u16x8 kreg[kKPer], vreg0[kVPer], vreg1[kVPer];
    auto load_idx = [&](const Job &j) {
      const long long pseg = (j.tile / tiles_per_seg) * N;
      const int nkeys = j.hi - j.s0 < kKeys ? j.hi - j.s0 : kKeys;
#pragma unroll
      for (int p = 0; p < kKPer; ++p) {
        int r = (ptid + p * kPThreads) / (D / 8);
        r = r < nkeys ? r : nkeys - 1;  // rows past the stage are reloads, never used
        kj[p] = sorted_index<kIdent>(perm_k, pseg, j.s0 + r);
      }
#pragma unroll
      for (int p = 0; p < kVPer; ++p) {
        int jp = (ptid + p * kPThreads) % (kKeys / 2);
        jp = 2 * jp + 1 < nkeys ? jp : nkeys / 2 - 1;
        v0[p] = sorted_index<kIdent>(perm_k, pseg, j.s0 + 2 * jp);
        v1[p] = sorted_index<kIdent>(perm_k, pseg, j.s0 + 2 * jp + 1);
      }
    };
    auto load_rows = [&](const Job &j) {
      const long long seg = (j.tile / tiles_per_seg) * N;
#pragma unroll
      for (int p = 0; p < kKPer; ++p)
        kreg[p] = *reinterpret_cast<const u16x8 *>(k + (seg + kj[p]) * D + ((ptid + p * kPThreads) % (D / 8)) * 8);
#pragma unroll
      for (int p = 0; p < kVPer; ++p) {
        const int ch = (ptid + p * kPThreads) / (kKeys / 2);
        vreg0[p] = *reinterpret_cast<const u16x8 *>(v + (seg + v0[p]) * D + ch * 8);
        vreg1[p] = *reinterpret_cast<const u16x8 *>(v + (seg + v1[p]) * D + ch * 8);
      }
    };
    auto store_rows = [&](uint16_t *buf) {
      uint16_t *Ks = buf, *Vt = buf + kKeys * kKRow;
#pragma unroll
      for (int p = 0; p < kKPer; ++p) {
        const int i = ptid + p * kPThreads;
        *reinterpret_cast<u16x8 *>(Ks + (i / (D / 8)) * kKRow + (i % (D / 8)) * 8) = kreg[p];
      }
#pragma unroll
      for (int p = 0; p < kVPer; ++p) {
        const int i = ptid + p * kPThreads;
        const int jp = i % (kKeys / 2), ch = i / (kKeys / 2);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t word = static_cast<uint32_t>(vreg0[p][e]) | (static_cast<uint32_t>(vreg1[p][e]) << 16);
          *reinterpret_cast<uint32_t *>(Vt + (ch * 8 + e) * kVRow + 2 * jp) = word;
        }
      }
    };
    Job cur = first_job(t_begin);  // job 0
    load_idx(cur);
    load_rows(cur);
    Job nxt = next_job(cur);  // job 1
    if (nxt.tile < t_end) load_idx(nxt);
    store_rows(smem);  // job 0 -> buffer 0
    if (nxt.tile < t_end) {
      load_rows(nxt);
      const Job n2 = next_job(nxt);
      if (n2.tile < t_end) load_idx(n2);
    }
    lds_barrier();  // job 0 ready
    for (int n = 1; nxt.tile < t_end; ++n) {  // nxt = job n, its rows in flight
      store_rows(smem + (n & 1) * kBufElems);  // buffer n&1 was read during job n-2
      const Job n1 = next_job(nxt);
      if (n1.tile < t_end) {
        load_rows(n1);  // indices loaded one job ago
        const Job n2 = next_job(n1);
        if (n2.tile < t_end) load_idx(n2);
      }
      lds_barrier();  // job n ready; consumers done with job n-1
      nxt = n1;
    }
    return;
  }

  // -------------------------------------------------------------- consumer
  const int g = lane >> 4, r16 = lane & 15;
  // query rows: group qg's query of this lane, d-slice g*8 .. +7 of each 32
  auto q_index = [&](long long t, int qg) -> int {
    const long long tt = t < t_end ? t : t_end - 1;
    return sorted_index<kIdent>(perm_q, (tt / tiles_per_seg) * N,
                                static_cast<int>(tt % tiles_per_seg) * QT + (wave * QG + qg) * 16 + r16);
  };
  auto load_q = [&](long long t, int qi, bf16x8 (&dst)[D / 32]) {
    const long long tt = t < t_end ? t : t_end - 1;
    const uint16_t *qrow = q + ((tt / tiles_per_seg) * N + qi) * D;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      dst[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8 *>(qrow + kk * 32 + g * 8));
  };
  bf16x8 bq[QG][D / 32], bq_next[QG][D / 32];
  int qidx[QG], qidx_n1[QG], qidx_n2[QG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    qidx[qg] = q_index(t_begin, qg);
    qidx_n1[qg] = q_index(t_begin + 1, qg);
    qidx_n2[qg] = 0;
  }
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) load_q(t_begin, qidx[qg], bq[qg]);

  f32x4 o[QG][D / 16], l_acc[QG];
  float m[QG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[qg][dt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    l_acc[qg] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    m[qg] = -INFINITY;
  }
  const bf16x8 ones = __builtin_bit_cast(bf16x8, (u16x8)0x3f80);

  Job cur = first_job(t_begin);
  for (int n = 0; cur.tile < t_end; ++n) {
    lds_barrier();  // job n staged in buffer n&1
    if (cur.s0 == cur.lo) {  // first job of a tile: the next tile's query rows, the one after's indices
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) load_q(cur.tile + 1, qidx_n1[qg], bq_next[qg]);
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) qidx_n2[qg] = q_index(cur.tile + 2, qg);
    }
    const uint16_t *buf = smem + (n & 1) * kBufElems;
    const int nkeys = cur.hi - cur.s0 < kKeys ? cur.hi - cur.s0 : kKeys;
    attend_stage<D, kKeys, QG>(buf, buf + kKeys * kKRow, nkeys, bq, o, l_acc, m, scale_log2, ones, g, r16);
    const Job nx = next_job(cur);
    if (nx.tile != cur.tile) {  // tile complete: normalise, write, reset
      const long long seg = (cur.tile / tiles_per_seg) * N;
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) {
        const float l_tot = l_acc[qg][0];
        const float inv = 1.0f / l_tot;
        uint16_t *orow = o_s + (seg + qidx[qg]) * D;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const uint2 outv = {pack_bf16x2(o[qg][dt][0] * inv, o[qg][dt][1] * inv),
                              pack_bf16x2(o[qg][dt][2] * inv, o[qg][dt][3] * inv)};
          *reinterpret_cast<uint2 *>(orow + dt * 16 + g * 4) = outv;
          o[qg][dt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
        }
        if (g == 0) lse[seg + qidx[qg]] = (m[qg] + log2f(l_tot)) * 0.69314718055994530942f;
        l_acc[qg] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
        m[qg] = -INFINITY;
        qidx[qg] = qidx_n1[qg];
        qidx_n1[qg] = qidx_n2[qg];
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) bq[qg][kk] = bq_next[qg][kk];
      }
    }
    cur = nx;
  }
}

// Sliding-window kernel for d = 64 and w = 128 (a 128-query tile is one
// chunk, whose window is the previous chunk and its own).  Consecutive tiles
// of a persistent workgroup share a chunk, so each tile gathers only its own
// chunk's 128 K and V rows: chunks live in a ring of three LDS slots (tile m
// reads slots m % 3 and (m + 1) % 3, and its own chunk is written to slot
// (m + 1) % 3 while tile m - 1 is computed).  Waves 8-11 produce: they store
// a tile's K and V rows, requested three tiles earlier into one of three
// register sets, then request the rows of the tile three ahead into that set
// (gathered rows come from HBM, and a tile of compute does not cover their
// latency) and write the original indices of its queries to one of four LDS
// index slots.  Waves 0-7 compute 16 queries each; they load their query rows
// for the next tile while computing the current one.  One LDS-only barrier
// per tile.
//
// Fused epilogue (kFuseL = L in {8, 16}): instead of writing o_s and its LSE,
// each computing wave finishes its 16 queries with the RACE gather, the gates
// and the fusion of the forward pass (the same arithmetic as the separate
// fusion kernel): it requests the queries' L table codes with their query
// rows, then gathers the L bucket rows (bfloat16, two 16-byte pieces a lane)
// and counts, the gate inputs, and writes y.  The transposed V rows are
// staged in a permuted row order so that a lane's O^T results are the 16
// consecutive columns g*16 .. g*16+15 of its query: table rows, gate inputs
// and y are then read and written as whole 16-byte pieces.  The sparse
// output never goes to memory (except as an optional aux output).
struct FuseArgs {
  const uint8_t *qcodes;   // [BH*N][L] query RACE codes (P <= 8)
  const uint16_t *tsum;    // [BH][L][2^P][64] bucket sums, bfloat16
  const float *tcnt;       // [BH][L][2^P] bucket counts
  const uint16_t *x_gate;  // [B][N][64]
  const float *gate_w;     // [2][H][64]
  const float *gate_b;     // [2][H]
  int H, P;
  float lambda;
  uint16_t *out;           // [BH][N][64]
  // optional aux outputs (NULL: not written)
  uint16_t *o_s;
  float *lse, *z_lr, *alpha, *g_s, *g_lr, *o_lr;
};

// The fused epilogue of one computing wave's 16 queries (d = 64): lane
// (g, r16) holds columns g*16 + dt*4 + i of query r16's unnormalised sparse
// output in o[dt][i] (1/l_tot = inv), its LSE, and the query's L codes in cw.
//   Z_lr = (1/L) sum_l count_l[c_l],  num = (1/L) sum_l sum_l[c_l][:],
//   o_lr = num / Z_lr (0 where Z_lr = 0),  g = sigmoid(<x_gate, W> + b),
//   alpha = 1 / (1 + exp(log(lambda Z_lr) - lse)) (1 where lambda Z_lr = 0),
//   y = g_s alpha o_s + g_lr o_lr
// ("ELSAA: Efficient Low-Rank and Sparse Attention Approximation for Training
// Transformers", first paragraph; "Two Efficient Attentions, One Denominator
// Problem", section "Two efficient branches can still be mis-scaled").  The
// table rows are requested four tables at a time, two sets in flight.  The
// next tile's query rows (qnext) are waited for before the stores: the vector
// memory counter retires in issue order.
template <int L>
__device__ __forceinline__ void fused_epilogue(const FuseArgs &fz, const f32x4 (&o)[4], float inv, float lse_v,
                                               const uint32_t (&cw)[L / 4], long long bh, int qidx, int N,
                                               int g, const float *gw_lds, const u16x8 (&qnext)[2]) {
  constexpr int D = 64;
  // o_s rounded to bfloat16 (as the separate fusion reads it), packed: the
  // registers of the fp32 values are free for the table rows
  uint32_t os[8];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    os[2 * dt] = pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv);
    os[2 * dt + 1] = pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv);
  }
  constexpr int kBatches = L / 4;
  static_assert(kBatches == 2 || kBatches == 4, "8 or 16 tables");
  const int nb = 1 << fz.P;
  const int h = static_cast<int>(bh % fz.H);
  const long long b = bh / fz.H;
  const __amdgpu_buffer_rsrc_t ts_rs =
      make_rsrc(fz.tsum + bh * L * nb * D, static_cast<uint32_t>(L * nb * D * 2));
  const __amdgpu_buffer_rsrc_t tc_rs = make_rsrc(fz.tcnt + bh * L * nb, static_cast<uint32_t>(L * nb * 4));
  const __amdgpu_buffer_rsrc_t xg_rs = make_rsrc(fz.x_gate + b * N * 64, static_cast<uint32_t>(N) * 128u);
  const uint32_t lane_off = static_cast<uint32_t>(g) * 32u;  // columns g*16 .. +15, bfloat16
  auto code_of = [&](int l) -> uint32_t { return (cw[l >> 2] >> (8 * (l & 3))) & 0xffu; };
  auto issue = [&](int batch, u32x4 (&dst)[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int l = batch * 4 + j;
      const uint32_t off = code_of(l) * static_cast<uint32_t>(D * 2) + lane_off;
      const int soff = l * nb * D * 2;
      dst[2 * j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ts_rs, off, soff, 0));
      dst[2 * j + 1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ts_rs, off + 16, soff, 0));
    }
  };
  // gate inputs of the query (columns g*16 .. +15) and the counts of tables
  // g, g + 4, ... (lane group g's byte of every code word)
  u32x4 xg0, xg1;
  float cnt[kBatches];
  auto issue_gate_and_counts = [&]() {
    const uint32_t xo = static_cast<uint32_t>(qidx) * 128u + lane_off;
    xg0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xg_rs, xo, 0, 0));
    xg1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xg_rs, xo + 16, 0, 0));
#pragma unroll
    for (int r = 0; r < kBatches; ++r) {
      const uint32_t c = (cw[r] >> (8 * g)) & 0xffu;  // code of table 4 r + g
      cnt[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          tc_rs, (static_cast<uint32_t>((4 * r + g) * nb) + c) * 4u, 0, 0));
    }
  };
  const Bf16Adder adder;
  float num[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) num[j] = 0.0f;
  auto accumulate = [&](const u32x4 (&src)[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w = src[2 * j + half][e];
          num[8 * half + 2 * e] = adder.lo(num[8 * half + 2 * e], w);
          num[8 * half + 2 * e + 1] = adder.hi(num[8 * half + 2 * e + 1], w);
        }
  };
  // two batches (8 tables) in flight; the gate inputs and counts follow the
  // first two (three batches in flight spill at 16 tables, and measured slower)
  u32x4 ta[8], tb[8];
  issue(0, ta);
  issue(1, tb);
  issue_gate_and_counts();
#pragma unroll
  for (int bt = 0; bt < kBatches; bt += 2) {
    accumulate(ta);
    if (bt + 2 < kBatches) issue(bt + 2, ta);
    accumulate(tb);
    if (bt + 3 < kBatches) issue(bt + 3, tb);
  }
  // gate logits: this lane's 16 products, then the query's four lanes
  float a0 = 0.0f, a1 = 0.0f, z = 0.0f;
  const float *w0 = gw_lds + h * 64 + g * 16;
  const float *w1 = gw_lds + (fz.H + h) * 64 + g * 16;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t word = e < 4 ? xg0[e] : xg1[e - 4];
    const float x0 = __uint_as_float(word << 16), x1 = __uint_as_float(word & 0xffff0000u);
    a0 = __builtin_fmaf(x0, w0[2 * e], a0);
    a0 = __builtin_fmaf(x1, w0[2 * e + 1], a0);
    a1 = __builtin_fmaf(x0, w1[2 * e], a1);
    a1 = __builtin_fmaf(x1, w1[2 * e + 1], a1);
  }
#pragma unroll
  for (int r = 0; r < kBatches; ++r) z += cnt[r];
  a0 = sum_over_lane_groups<16>(a0);
  a1 = sum_over_lane_groups<16>(a1);
  z = sum_over_lane_groups<16>(z);
  const float g_s = __builtin_amdgcn_rcpf(1.0f + __expf(-(a0 + fz.gate_b[h])));
  const float g_lr = __builtin_amdgcn_rcpf(1.0f + __expf(-(a1 + fz.gate_b[fz.H + h])));
  const float z_lr = z * (1.0f / static_cast<float>(L));
  const float rz = z > 0.0f ? __builtin_amdgcn_rcpf(z) : 0.0f;  // (num / L) / (z / L); 0 where z = 0
  const float mass_lr = fz.lambda * z_lr;
  const float alpha = mass_lr > 0.0f ? __builtin_amdgcn_rcpf(1.0f + __expf(__logf(mass_lr) - lse_v)) : 1.0f;
  const float cs = g_s * alpha, cl = g_lr * rz;
  float y[16];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    y[2 * j] = __builtin_fmaf(cs, __uint_as_float(os[j] << 16), cl * num[2 * j]);
    y[2 * j + 1] = __builtin_fmaf(cs, __uint_as_float(os[j] & 0xffff0000u), cl * num[2 * j + 1]);
  }
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) asm volatile("" : "+v"(y[0]) : "v"(qnext[kk]) : "memory");
  const long long row = bh * N + qidx;
  uint16_t *yrow = fz.out + row * D + g * 16;
  *reinterpret_cast<u32x4 *>(yrow) = u32x4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                                           pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
  *reinterpret_cast<u32x4 *>(yrow + 8) = u32x4{pack_bf16x2(y[8], y[9]), pack_bf16x2(y[10], y[11]),
                                               pack_bf16x2(y[12], y[13]), pack_bf16x2(y[14], y[15])};
  if (fz.o_s) {
    uint16_t *orow = fz.o_s + row * D + g * 16;
    *reinterpret_cast<u32x4 *>(orow) = u32x4{os[0], os[1], os[2], os[3]};
    *reinterpret_cast<u32x4 *>(orow + 8) = u32x4{os[4], os[5], os[6], os[7]};
  }
  if (fz.o_lr) {
    float *lrow = fz.o_lr + row * D + g * 16;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<f32x4 *>(lrow + 4 * j) =
          f32x4{num[4 * j] * rz, num[4 * j + 1] * rz, num[4 * j + 2] * rz, num[4 * j + 3] * rz};
  }
  if (g == 0) {
    if (fz.lse) fz.lse[row] = lse_v;
    if (fz.z_lr) fz.z_lr[row] = z_lr;
    if (fz.alpha) fz.alpha[row] = alpha;
    if (fz.g_s) fz.g_s[row] = g_s;
    if (fz.g_lr) fz.g_lr[row] = g_lr;
  }
}

template <bool kIdent, int kFuseL>
__global__ __launch_bounds__(768) void elsaa_k3_chunk_attn_slide(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ perm_q, const int32_t *__restrict__ perm_k, int N,
    int tiles_per_seg, long long n_tiles, long long tiles_per_wg, float scale_log2,
    uint16_t *__restrict__ o_s, float *__restrict__ lse, FuseArgs fz) {
  constexpr int D = 64, W = 128;
  constexpr int kConsumerWaves = 8;
  constexpr int kPThreads = 256;
  constexpr int kKRow = D + 8;
  constexpr int kVRow = W + 4;
  constexpr int kSlotElems = W * kKRow + D * kVRow;  // one chunk: K rows, V^T
  constexpr int kKChunks = W * (D / 8);
  constexpr int kVPairs = (W / 2) * (D / 8);
  constexpr int kKPer = kKChunks / kPThreads;  // 4
  constexpr int kVPer = kVPairs / kPThreads;   // 2
  extern __shared__ __align__(16) uint16_t smem[];
  int32_t *qidx_lds = reinterpret_cast<int32_t *>(smem + 3 * kSlotElems);  // [4][W], tile m in m % 4
  float *gw_lds = reinterpret_cast<float *>(qidx_lds + 4 * W);  // fused: gate weights [2][H][64]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long long t_begin = xcd_logical_block(blockIdx.x, gridDim.x) * tiles_per_wg;
  const long long t_end = t_begin + tiles_per_wg < n_tiles ? t_begin + tiles_per_wg : n_tiles;
  if (t_begin >= t_end) return;  // whole workgroup
  if constexpr (kFuseL > 0) {  // visible to the computing waves after the first barrier
    for (int i = tid; i < 2 * fz.H * 64; i += 768) gw_lds[i] = fz.gate_w[i];
  }
  // V^T row of column c: the O^T tile dt holds columns g*16 + dt*4 + i in its
  // rows 4 g + i, so that lane group g's results are columns g*16 .. +15
  auto vt_row = [](int c) { return ((c >> 2) & 3) * 16 + (c >> 4) * 4 + (c & 3); };
  auto chunk_of = [&](long long t) { return static_cast<int>(t % tiles_per_seg); };
  auto seg_of = [&](long long t) { return (t / tiles_per_seg) * N; };
  // piece of a row at a 32-bit byte offset from its segment's first row (the
  // host keeps a segment's rows below 2^31 bytes): a uniform base plus one
  // offset register per load
  auto piece = [](const uint16_t *base, int row, int ch) {
    const uint32_t off = static_cast<uint32_t>(row) * (D * 2) + static_cast<uint32_t>(ch) * 16;
    return *reinterpret_cast<const u16x8 *>(reinterpret_cast<const char *>(base) + off);
  };

  if (wave >= kConsumerWaves) {
    // ------------------------------------------------------------ producer
    const int ptid = tid - kConsumerWaves * 64;
    // Thread ptid's K pieces are rows ptid / 8 + 32 p, chunk ptid % 8; its V
    // pieces are chunks ptid / 64 + 4 p of the key pair ptid % 64 (one pair
    // for every p); thread ptid < 128 also fetches the tile's query ptid.
    struct Idx {  // key indices of a chunk, query index of a tile
      int kj[kKPer], v0, v1, qj;
    };
    struct Rows {  // this thread's pieces of a chunk's K and V rows
      u16x8 k[kKPer], v0[kVPer], v1[kVPer];
    };
    // key indices of chunk c and query indices of tile t (whose chunk is c)
    auto load_idx = [&](Idx &ix, long long t, int c, bool with_q) {
      const long long seg = seg_of(t);
#pragma unroll
      for (int p = 0; p < kKPer; ++p) ix.kj[p] = sorted_index<kIdent>(perm_k, seg, c * W + (ptid + p * kPThreads) / (D / 8));
      static_assert(kPThreads % (W / 2) == 0, "every V piece of a thread is one key pair");
      ix.v0 = sorted_index<kIdent>(perm_k, seg, c * W + 2 * (ptid % (W / 2)));
      ix.v1 = sorted_index<kIdent>(perm_k, seg, c * W + 2 * (ptid % (W / 2)) + 1);
      // threads from W on: a repeat, not stored
      if (with_q) ix.qj = sorted_index<kIdent>(perm_q, seg, c * W + ptid % W);
    };
    auto load_rows = [&](Rows &r, const Idx &ix, long long t) {
      const long long seg = seg_of(t);
      const uint16_t *ks = k + seg * D, *vs = v + seg * D;
#pragma unroll
      for (int p = 0; p < kKPer; ++p) r.k[p] = piece(ks, ix.kj[p], (ptid + p * kPThreads) % (D / 8));
#pragma unroll
      for (int p = 0; p < kVPer; ++p) {
        const int ch = (ptid + p * kPThreads) / (W / 2);
        r.v0[p] = piece(vs, ix.v0, ch);
        r.v1[p] = piece(vs, ix.v1, ch);
      }
    };
    auto store_rows = [&](const Rows &r, int slot) {
      uint16_t *Ks = smem + slot * kSlotElems, *Vt = Ks + W * kKRow;
#pragma unroll
      for (int p = 0; p < kKPer; ++p) {
        const int i = ptid + p * kPThreads;
        *reinterpret_cast<u16x8 *>(Ks + (i / (D / 8)) * kKRow + (i % (D / 8)) * 8) = r.k[p];
      }
#pragma unroll
      for (int p = 0; p < kVPer; ++p) {
        const int i = ptid + p * kPThreads;
        const int jp = i % (W / 2), ch = i / (W / 2);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t word = static_cast<uint32_t>(r.v0[p][e]) | (static_cast<uint32_t>(r.v1[p][e]) << 16);
          *reinterpret_cast<uint32_t *>(Vt + vt_row(ch * 8 + e) * kVRow + 2 * jp) = word;
        }
      }
    };
    // original indices of tile t's queries to index slot (t - t_begin) % 4
    auto store_qidx = [&](const Idx &ix, long long t) {
      if (ptid < W) qidx_lds[static_cast<int>((t - t_begin) & 3) * W + ptid] = ix.qj;
    };
    Idx i0, i1, i2;
    Rows r0, r1, r2;
    // Every step issues the same loads (past the last tile they repeat it and
    // are not stored), so the count of loads in flight at each wait is the
    // same on every path and each wait covers only the set it stores.
    auto clamp_t = [&](long long t) { return t < t_end ? t : t_end - 1; };
    auto indices = [&](Idx &ix, long long t) { load_idx(ix, clamp_t(t), chunk_of(clamp_t(t)), true); };
    auto rows = [&](Rows &r, const Idx &ix, long long t) {
      load_rows(r, ix, clamp_t(t));
      store_qidx(ix, t);
    };
    // prologue: the first tile's previous chunk goes to slot 0; then tiles 0,
    // 1 and 2 are requested, and tile 3's indices, in the order of the steps
    // (tile j + 1's indices, then tile j's rows)
    const int c_begin = chunk_of(t_begin);
    if (c_begin > 0) {
      load_idx(i0, t_begin, c_begin - 1, false);
      load_rows(r0, i0, t_begin);
      store_rows(r0, 0);
    }
    indices(i0, t_begin);
    indices(i1, t_begin + 1);
    rows(r0, i0, t_begin);
    indices(i2, t_begin + 2);
    rows(r1, i1, t_begin + 1);
    indices(i0, t_begin + 3);
    rows(r2, i2, t_begin + 2);
    // tile m = t - t_begin: its chunk to slot (m + 1) % 3 (tile m - 1 is being
    // computed from the other two); then tile m + 4's indices into the set
    // tile m + 1 used, and tile m + 3's rows (indices loaded one step ago)
    // into the set just stored.  Tile m + 3's index slot held tile m - 1's,
    // which the computing waves read before barrier m - 1.
    auto step = [&](Rows &r, const Idx &use, Idx &next, long long t) {
      const int m = static_cast<int>(t - t_begin);
      store_rows(r, (m + 1) % 3);
      indices(next, t + 4);
      rows(r, use, t + 3);
      lds_barrier();  // tile m ready; tile m - 1 computed
    };
    long long t = t_begin;
    for (; t + 2 < t_end; t += 3) {
      step(r0, i0, i1, t);
      step(r1, i1, i2, t + 1);
      step(r2, i2, i0, t + 2);
    }
    if (t < t_end) step(r0, i0, i1, t);
    if (t + 1 < t_end) step(r1, i1, i2, t + 1);
    return;
  }

  // -------------------------------------------------------------- consumer
  const int g = lane >> 4, r16 = lane & 15;
  const bf16x8 ones = __builtin_bit_cast(bf16x8, (u16x8)0x3f80);
  const int qrow = wave * 16 + r16;  // this lane's query of every tile
  // Q^T operand: lane holds its query's d-slice g*8 .. +7 of each 32
  auto load_q = [&](u16x8 (&dst)[D / 32], long long t, int qi) {
    const uint16_t *qs = q + seg_of(t) * D;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) dst[kk] = piece(qs, qi, kk * 4 + g);
  };
  // The query rows of tile t + 1 are loaded during tile t and waited for
  // before tile t's output stores (the vector memory counter retires in issue
  // order: a wait after the stores would wait for them too).  Every load is
  // unconditional (the last tile loads its own rows again), so no branch
  // merges a pending and a completed load.
  u16x8 qnext[D / 32];
  int qidx_next = 0;
  if (t_begin < t_end) {
    lds_barrier();  // tile 0's chunks staged
    qidx_next = qidx_lds[qrow];
    load_q(qnext, t_begin, qidx_next);
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) asm volatile("" ::"v"(qnext[kk]) : "memory");
  }
  for (long long t = t_begin; t < t_end; ++t) {
    const int m_idx = static_cast<int>(t - t_begin);
    const int c = chunk_of(t);
    if (m_idx > 0) lds_barrier();  // tile m_idx's chunks staged
    bf16x8 bq[D / 32];
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) bq[kk] = __builtin_bit_cast(bf16x8, qnext[kk]);
    const int qidx = qidx_next;
    const long long bh = t / tiles_per_seg;
    // fused: the query's L table codes, in flight during the attention (a
    // query's codes are contiguous: kFuseL bytes)
    uint32_t cw[kFuseL > 0 ? kFuseL / 4 : 1];
    if constexpr (kFuseL > 0) {
      const __amdgpu_buffer_rsrc_t qc_rs =
          make_rsrc(fz.qcodes + bh * N * kFuseL, static_cast<uint32_t>(N) * kFuseL);
      const uint32_t off = static_cast<uint32_t>(qidx) * kFuseL;
      if constexpr (kFuseL == 16) {
        const u32x4 w4 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(qc_rs, off, 0, 0));
#pragma unroll
        for (int e = 0; e < 4; ++e) cw[e] = w4[e];
      } else {
        static_assert(kFuseL == 8, "8 or 16 tables");
        const auto w2 = __builtin_amdgcn_raw_buffer_load_b64(qc_rs, off, 0, 0);
        cw[0] = w2[0];
        cw[1] = w2[1];
      }
    }
    {  // the next tile's query rows, in flight during this tile
      const bool more = t + 1 < t_end;
      qidx_next = more ? qidx_lds[((m_idx + 1) & 3) * W + qrow] : qidx;
      load_q(qnext, more ? t + 1 : t, qidx_next);
    }
    f32x4 o[D / 16], l_acc = {0.0f, 0.0f, 0.0f, 0.0f};
    float m = -INFINITY;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    const uint16_t *own = smem + ((m_idx + 1) % 3) * kSlotElems;
    if (c > 0) {
      const uint16_t *prev = smem + (m_idx % 3) * kSlotElems;
      const uint16_t *const kb[4] = {prev, prev + 64 * kKRow, own, own + 64 * kKRow};
      const uint16_t *const vb[4] = {prev + W * kKRow, prev + W * kKRow + 64, own + W * kKRow, own + W * kKRow + 64};
      attend_blocks<D, kVRow, 4>(kb, vb, bq, o, l_acc, m, scale_log2, ones, g, r16);
    } else {
      const uint16_t *const kb[2] = {own, own + 64 * kKRow};
      const uint16_t *const vb[2] = {own + W * kKRow, own + W * kKRow + 64};
      attend_blocks<D, kVRow, 2>(kb, vb, bq, o, l_acc, m, scale_log2, ones, g, r16);
    }
    const long long seg = seg_of(t);
    const float l_tot = l_acc[0];
    float inv = 1.0f / l_tot;
    const float lse_v = (m + log2f(l_tot)) * 0.69314718055994530942f;
    // lane group g holds columns g*16 + dt*4 + i of its query in o[dt][i]
    if constexpr (kFuseL == 0) {
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) asm volatile("" : "+v"(inv) : "v"(qnext[kk]) : "memory");
      uint16_t *orow = o_s + (seg + qidx) * D + g * 16;
      *reinterpret_cast<u32x4 *>(orow) =
          u32x4{pack_bf16x2(o[0][0] * inv, o[0][1] * inv), pack_bf16x2(o[0][2] * inv, o[0][3] * inv),
                pack_bf16x2(o[1][0] * inv, o[1][1] * inv), pack_bf16x2(o[1][2] * inv, o[1][3] * inv)};
      *reinterpret_cast<u32x4 *>(orow + 8) =
          u32x4{pack_bf16x2(o[2][0] * inv, o[2][1] * inv), pack_bf16x2(o[2][2] * inv, o[2][3] * inv),
                pack_bf16x2(o[3][0] * inv, o[3][1] * inv), pack_bf16x2(o[3][2] * inv, o[3][3] * inv)};
      if (g == 0) lse[seg + qidx] = lse_v;
    } else {
      fused_epilogue<kFuseL>(fz, o, inv, lse_v, cw, bh, qidx, N, g, gw_lds, qnext);
    }
  }
}

// d = 128, w a multiple of 256: one workgroup per 256 sorted queries (a
// whole chunk when w = 256), eight waves of 32 queries (two groups of 16 that
// share every K and V fragment read from LDS, so each fragment serves 32
// queries: at d = 128 the LDS reads of 16-query fragments would outweigh the
// matrix work).  No producer waves: all eight waves stage each block of 64
// window keys (K row-major, V transposed) into one of two LDS buffers, the
// next block's rows in flight in registers while the current block is
// computed, with one LDS-only barrier per block.  Key indices are requested a
// block before their rows, so neither a permutation load nor a row load is
// waited for in the block that issues it, and rows come through buffer loads
// with 32-bit offsets from the segment's base (N * d * 2 < 2^32 bytes).
// Neighbouring tiles share a chunk of keys and run on one XCD.
template <bool kIdent>
__global__ __launch_bounds__(512) void elsaa_k3_chunk_attn_c256(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ perm_q, const int32_t *__restrict__ perm_k, int N, int w, int tiles_per_seg,
    long long n_tiles, float scale_log2, uint16_t *__restrict__ o_s, float *__restrict__ lse) {
  constexpr int D = 128, QT = 256, QG = 2;
  constexpr int kKRow = D + 8, kVRow = kKBlock + 4;
  constexpr int kBufElems = kKBlock * kKRow + D * kVRow;
  constexpr int kKPer = kKBlock * (D / 8) / 512;        // 2 K pieces per thread
  constexpr int kVPer = (kKBlock / 2) * (D / 8) / 512;  // 1 V (pair, chunk) per thread
  extern __shared__ __align__(16) uint16_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const long long tile = xcd_logical_block(blockIdx.x, gridDim.x);
  if (tile >= n_tiles) return;  // padding workgroup (whole group exits)
  const long long seg = (tile / tiles_per_seg) * N;
  const int r0 = static_cast<int>(tile % tiles_per_seg) * QT;
  const int c = r0 / w;
  const int lo = c > 0 ? (c - 1) * w : 0, hi = (c + 1) * w;
  // the segment's K and V rows and key permutation as buffers: 32-bit
  // offsets, no 64-bit address arithmetic per gathered row
  const __amdgpu_buffer_rsrc_t k_rs = make_rsrc(k + seg * D, static_cast<uint32_t>(N) * (D * 2));
  const __amdgpu_buffer_rsrc_t v_rs = make_rsrc(v + seg * D, static_cast<uint32_t>(N) * (D * 2));
  const __amdgpu_buffer_rsrc_t pk_rs = make_rsrc(perm_k + seg, static_cast<uint32_t>(N) * 4u);
  auto key_index = [&](int r) -> int {
    if constexpr (kIdent) {
      return r;
    } else {
      return __builtin_amdgcn_raw_buffer_load_b32(pk_rs, static_cast<uint32_t>(r) * 4u, 0, 0);
    }
  };
  // staging: thread tid holds K pieces (row (tid + 512 p) / 16, chunk
  // (tid + 512 p) % 16) and the V pair tid % 32, chunk tid / 32
  int kj[kKPer], vj0[kVPer], vj1[kVPer];
  u16x8 kr[kKPer], vr0[kVPer], vr1[kVPer];
  auto load_idx = [&](int s0) {
#pragma unroll
    for (int p = 0; p < kKPer; ++p) kj[p] = key_index(s0 + (tid + 512 * p) / (D / 8));
#pragma unroll
    for (int p = 0; p < kVPer; ++p) {
      const int jp = (tid + 512 * p) % (kKBlock / 2);
      vj0[p] = key_index(s0 + 2 * jp);
      vj1[p] = key_index(s0 + 2 * jp + 1);
    }
  };
  auto row = [&](__amdgpu_buffer_rsrc_t rs, int j, int piece) -> u16x8 {
    return __builtin_bit_cast(u16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                         rs, static_cast<uint32_t>(j) * (D * 2) + piece * 16, 0, 0));
  };
  auto load_rows = [&]() {
#pragma unroll
    for (int p = 0; p < kKPer; ++p) kr[p] = row(k_rs, kj[p], (tid + 512 * p) % (D / 8));
#pragma unroll
    for (int p = 0; p < kVPer; ++p) {
      const int ch = (tid + 512 * p) / (kKBlock / 2);
      vr0[p] = row(v_rs, vj0[p], ch);
      vr1[p] = row(v_rs, vj1[p], ch);
    }
  };
  auto store_rows = [&](uint16_t *buf) {
    uint16_t *Ks = buf, *Vt = buf + kKBlock * kKRow;
#pragma unroll
    for (int p = 0; p < kKPer; ++p) {
      const int i = tid + 512 * p;
      *reinterpret_cast<u16x8 *>(Ks + (i / (D / 8)) * kKRow + (i % (D / 8)) * 8) = kr[p];
    }
#pragma unroll
    for (int p = 0; p < kVPer; ++p) {
      const int i = tid + 512 * p;
      const int jp = i % (kKBlock / 2), ch = i / (kKBlock / 2);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<uint32_t *>(Vt + (ch * 8 + e) * kVRow + 2 * jp) =
            static_cast<uint32_t>(vr0[p][e]) | (static_cast<uint32_t>(vr1[p][e]) << 16);
    }
  };
  // the wave's 32 queries: Q^T operands, lane holds d-slice g*8 .. +7 of each 32
  int qidx[QG];
  bf16x8 bq[QG][D / 32];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    qidx[qg] = sorted_index<kIdent>(perm_q, seg, r0 + wave * 32 + qg * 16 + r16);
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      bq[qg][kk] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u16x8 *>(q + (seg + qidx[qg]) * D + kk * 32 + g * 8));
  }
  f32x4 o[QG][D / 16], l_acc[QG];
  float m[QG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[qg][dt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    l_acc[qg] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    m[qg] = -INFINITY;
  }
  const bf16x8 ones = __builtin_bit_cast(bf16x8, (u16x8)0x3f80);

  // rows are requested one block ahead, their indices two blocks ahead (the
  // last request repeats the last block's indices and goes unused)
  load_idx(lo);
  load_rows();
  load_idx(lo + kKBlock);
  for (int s0 = lo, b = 0; s0 < hi; s0 += kKBlock, ++b) {
    uint16_t *buf = smem + (b & 1) * kBufElems;
    store_rows(buf);  // waits for this block's rows
    if (s0 + kKBlock < hi) load_rows();  // the next block's rows, in flight during this block
    load_idx(s0 + 2 * kKBlock < hi ? s0 + 2 * kKBlock : hi - kKBlock);
    lds_barrier();  // block b staged; every wave is past block b - 1
    attend_stage<D, kKBlock, QG>(buf, buf + kKBlock * kKRow, kKBlock, bq, o, l_acc, m, scale_log2, ones, g, r16);
  }
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    const float l_tot = l_acc[qg][0];
    const float inv = 1.0f / l_tot;
    uint16_t *orow = o_s + (seg + qidx[qg]) * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      *reinterpret_cast<uint2 *>(orow + dt * 16 + g * 4) =
          make_uint2(pack_bf16x2(o[qg][dt][0] * inv, o[qg][dt][1] * inv),
                     pack_bf16x2(o[qg][dt][2] * inv, o[qg][dt][3] * inv));
    if (g == 0) lse[seg + qidx[qg]] = (m[qg] + log2f(l_tot)) * 0.69314718055994530942f;
  }
}

// LDS bytes of the sliding-window kernel: three chunk slots, four
// query-index slots and, fused, the gate weights of every head.
constexpr size_t attn_slide_lds_bytes(int fused_heads) {
  return 3 * (static_cast<size_t>(128) * (64 + 8) + static_cast<size_t>(64) * (128 + 4)) * 2 + 4 * 128 * 4 +
         static_cast<size_t>(fused_heads) * 2 * 64 * 4;
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
  const int qidx = perm_q ? perm_q[seg + rank] : rank;  // no permutation: the identity
  const float *qr = q + (seg + qidx) * D;
  float acc[D];
  for (int e = 0; e < D; ++e) acc[e] = 0.0f;
  float m = -INFINITY, l = 0.0f;
  for (int t = lo; t < hi; ++t) {
    const int kidx = perm_k ? perm_k[seg + t] : t;
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

template <int D, int QT, int NB, bool kIdent>
hipError_t launch_bf16(const Geometry &g, const void *q, const void *k, const void *v,
                       const int32_t *pq, const int32_t *pk, void *o_s, float *lse, float scale_log2,
                       hipStream_t stream) {
  const int tiles_per_seg = g.N / QT;
  const long long n_tiles = static_cast<long long>(tiles_per_seg) * g.BH;
  const long long grid = (n_tiles + kXcdCount - 1) / kXcdCount * kXcdCount;
  hipLaunchKernelGGL((elsaa_k3_chunk_attn_bf16<D, QT, NB, kIdent>), dim3(static_cast<unsigned>(grid)),
                     dim3(QT * 4), attn_lds_bytes(D, NB), stream, static_cast<const uint16_t *>(q),
                     static_cast<const uint16_t *>(k), static_cast<const uint16_t *>(v), pq, pk, g.N, g.w,
                     tiles_per_seg, static_cast<int>(n_tiles), scale_log2, static_cast<uint16_t *>(o_s), lse);
  return hipGetLastError();
}

// LDS bytes of the pipelined kernel: two stage buffers.
constexpr size_t attn_pc_lds_bytes(int D, int NB) { return 2 * attn_lds_bytes(D, NB); }

template <int D, int NB, bool kIdent>
hipError_t launch_bf16_pc(const Geometry &g, const void *q, const void *k, const void *v,
                          const int32_t *pq, const int32_t *pk, void *o_s, float *lse, float scale_log2,
                          hipStream_t stream) {
  const int tiles_per_seg = g.N / 128;
  const long long n_tiles = static_cast<long long>(tiles_per_seg) * g.BH;
  // one workgroup per compute unit (two stage buffers fill its LDS), a
  // multiple of the XCD count, each taking a contiguous run of tiles
  long long wgs = (g.cus + kXcdCount - 1) / kXcdCount * kXcdCount;
  if (wgs > n_tiles) wgs = (n_tiles + kXcdCount - 1) / kXcdCount * kXcdCount;
  const long long tiles_per_wg = (n_tiles + wgs - 1) / wgs;
  hipLaunchKernelGGL((elsaa_k3_chunk_attn_pc<D, NB, kIdent>), dim3(static_cast<unsigned>(wgs)), dim3(512),
                     attn_pc_lds_bytes(D, NB), stream, static_cast<const uint16_t *>(q),
                     static_cast<const uint16_t *>(k), static_cast<const uint16_t *>(v), pq, pk, g.N, g.w,
                     tiles_per_seg, n_tiles, tiles_per_wg, scale_log2, static_cast<uint16_t *>(o_s), lse);
  return hipGetLastError();
}

template <bool kIdent, int kFuseL>
hipError_t launch_bf16_slide(const Geometry &g, const void *q, const void *k, const void *v,
                             const int32_t *pq, const int32_t *pk, void *o_s, float *lse, float scale_log2,
                             const FuseArgs &fz, hipStream_t stream) {
  const int tiles_per_seg = g.N / 128;
  const long long n_tiles = static_cast<long long>(tiles_per_seg) * g.BH;
  long long wgs = (g.cus + kXcdCount - 1) / kXcdCount * kXcdCount;
  if (wgs > n_tiles) wgs = (n_tiles + kXcdCount - 1) / kXcdCount * kXcdCount;
  const long long tiles_per_wg = (n_tiles + wgs - 1) / wgs;
  hipLaunchKernelGGL((elsaa_k3_chunk_attn_slide<kIdent, kFuseL>), dim3(static_cast<unsigned>(wgs)), dim3(768),
                     attn_slide_lds_bytes(kFuseL > 0 ? g.H : 0), stream, static_cast<const uint16_t *>(q),
                     static_cast<const uint16_t *>(k), static_cast<const uint16_t *>(v), pq, pk, g.N,
                     tiles_per_seg, n_tiles, tiles_per_wg, scale_log2, static_cast<uint16_t *>(o_s), lse, fz);
  return hipGetLastError();
}

template <bool kIdent>
hipError_t launch_bf16_c256(const Geometry &g, const void *q, const void *k, const void *v, const int32_t *pq,
                            const int32_t *pk, void *o_s, float *lse, float scale_log2, hipStream_t stream) {
  const int tiles_per_seg = g.N / 256;
  const long long n_tiles = static_cast<long long>(tiles_per_seg) * g.BH;
  const long long grid = (n_tiles + kXcdCount - 1) / kXcdCount * kXcdCount;
  constexpr size_t kLds = 2 * (static_cast<size_t>(kKBlock) * (128 + 8) + static_cast<size_t>(128) * (kKBlock + 4)) * 2;
  hipLaunchKernelGGL((elsaa_k3_chunk_attn_c256<kIdent>), dim3(static_cast<unsigned>(grid)), dim3(512), kLds, stream,
                     static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                     static_cast<const uint16_t *>(v), pq, pk, g.N, g.w, tiles_per_seg, n_tiles, scale_log2,
                     static_cast<uint16_t *>(o_s), lse);
  return hipGetLastError();
}

template <bool kIdent>
hipError_t launch_bf16_any(const Geometry &g, const void *q, const void *k, const void *v, const int32_t *pq,
                           const int32_t *pk, void *o_s, float *lse, float scale_log2, hipStream_t stream) {
  if (g.D == 128 && g.w % 256 == 0 && g.N < (1 << 24))  // 32-bit buffer offsets
    return launch_bf16_c256<kIdent>(g, q, k, v, pq, pk, o_s, lse, scale_log2, stream);
  // 128-query tiles when w allows; key stages of 4 blocks (d = 64: the whole
  // 256-key window of w = 128) or 2, keeping LDS <= 72 KB (two workgroups
  // per CU)
  const bool wide = g.w % 128 == 0;
  if (g.D == 64 && g.w == 128)
    return launch_bf16_slide<kIdent, 0>(g, q, k, v, pq, pk, o_s, lse, scale_log2, FuseArgs{}, stream);
  if (g.D == 64)
    return wide ? launch_bf16_pc<64, 4, kIdent>(g, q, k, v, pq, pk, o_s, lse, scale_log2, stream)
                : launch_bf16<64, 64, 2, kIdent>(g, q, k, v, pq, pk, o_s, lse, scale_log2, stream);
  return wide ? launch_bf16_pc<128, 2, kIdent>(g, q, k, v, pq, pk, o_s, lse, scale_log2, stream)
              : launch_bf16<128, 64, 2, kIdent>(g, q, k, v, pq, pk, o_s, lse, scale_log2, stream);
}

}  // namespace

hipError_t launch_chunk_attention(const Geometry &g, const void *q, const void *k, const void *v,
                                  const Buffers &buf, void *o_s, hipStream_t stream) {
  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(g.D));
  // one sort bucket: no permutation is read (the identity order)
  const int32_t *pq = g.identity ? nullptr : buf.perm;
  const int32_t *pk = g.identity ? nullptr : buf.perm + g.rows;
  if (g.bf16)
    return g.identity ? launch_bf16_any<true>(g, q, k, v, pq, pk, o_s, buf.lse, scale_log2, stream)
                      : launch_bf16_any<false>(g, q, k, v, pq, pk, o_s, buf.lse, scale_log2, stream);
  const dim3 grid((g.N + 127) / 128, g.BH);
  if (g.D == 64)
    hipLaunchKernelGGL(elsaa_k3_chunk_attn_f32<64>, grid, dim3(128), 0, stream,
                       static_cast<const float *>(q), static_cast<const float *>(k),
                       static_cast<const float *>(v), pq, pk, g.N, g.w, scale_log2,
                       static_cast<float *>(o_s), buf.lse);
  else
    hipLaunchKernelGGL(elsaa_k3_chunk_attn_f32<128>, grid, dim3(128), 0, stream,
                       static_cast<const float *>(q), static_cast<const float *>(k),
                       static_cast<const float *>(v), pq, pk, g.N, g.w, scale_log2,
                       static_cast<float *>(o_s), buf.lse);
  return hipGetLastError();
}

bool attention_fusable(const Geometry &g) {
  // the sliding-window kernel's shape (bfloat16, d = 64, w = 128), 8 or 16
  // tables of byte codes, gate inputs of width 64, both branches, and the
  // gate weights of every head in LDS
  return g.bf16 && g.D == 64 && g.w == 128 && (g.L == 8 || g.L == 16) && g.P <= 8 && g.DG == 64 &&
         g.run_sparse && g.run_race && g.H <= 64;
}

hipError_t launch_attention_fused(const Geometry &g, const void *q, const void *k, const void *v,
                                  const void *x_gate, const float *gate_w, const float *gate_b,
                                  const Buffers &buf, const elsaa_aux_t *aux, void *out, hipStream_t stream) {
  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(g.D));
  const int32_t *pq = g.identity ? nullptr : buf.perm;
  const int32_t *pk = g.identity ? nullptr : buf.perm + g.rows;
  FuseArgs fz{};
  fz.qcodes = static_cast<const uint8_t *>(buf.rcode);
  fz.tsum = static_cast<const uint16_t *>(buf.tsum);
  fz.tcnt = buf.tcnt;
  fz.x_gate = static_cast<const uint16_t *>(x_gate);
  fz.gate_w = gate_w;
  fz.gate_b = gate_b;
  fz.H = g.H;
  fz.P = g.P;
  fz.lambda = g.lambda;
  fz.out = static_cast<uint16_t *>(out);
  if (aux) {
    fz.o_s = static_cast<uint16_t *>(aux->o_sparse);
    fz.lse = aux->lse_s;
    fz.z_lr = aux->z_lr;
    fz.alpha = aux->alpha;
    fz.g_s = aux->g_s;
    fz.g_lr = aux->g_lr;
    fz.o_lr = aux->o_lowrank;
  }
  auto go = [&](auto ident, auto fl) {
    return launch_bf16_slide<decltype(ident)::value, decltype(fl)::value>(g, q, k, v, pq, pk, nullptr, nullptr,
                                                                          scale_log2, fz, stream);
  };
  using T = std::true_type;
  using F = std::false_type;
  using L8 = std::integral_constant<int, 8>;
  using L16 = std::integral_constant<int, 16>;
  if (g.identity) return g.L == 16 ? go(T{}, L16{}) : go(T{}, L8{});
  return g.L == 16 ? go(F{}, L16{}) : go(F{}, L8{});
}

}  // namespace elsaa
