// k6_backward.hip -- the backward pass: gradients of the forward output with
// respect to q, k, v, x_gate, W_g, b_g and lambda, for training ("ELSAA:
// Efficient Low-Rank and Sparse Attention Approximation for Training
// Transformers", first paragraph: a training framework with a learnable
// lambda; "ELSAA combines sparsity and low-rank methods to reduce transformer
// attention complexity": it acts on the attention computation at run time).
// Hash codes, permutations and bucket counts are piecewise constant in the
// inputs and carry no gradient.  With dy = dL/dy, per query i (original index):
//   y = c_s o_s + c_lr o_lr, (c_s, c_lr) = (g_s alpha, g_lr), or (g_s, g_lr)
//     with alpha fixed to one, (0, 1) RACE only, (1, 0) sparse only;
//   alpha = Z_s / (Z_s + lambda Z_lr):  d alpha / d lse = alpha (1 - alpha),
//     d alpha / d lambda = -alpha^2 Z_lr / Z_s;
//   sparse branch (flash-style, P recomputed from the stored LSE):
//     do = c_s dy,  delta_i = do_i . o_s,i - dL/dlse_i,
//     ds_ij = p_ij (do_i . v_j - delta_i),  dq_i = sum_j ds_ij k_j / sqrt d,
//     dk_j = sum_i ds_ij q_i / sqrt d,  dv_j = sum_i p_ij do_i;
//   low-rank branch: o_lr = num / Z_lr with Z_lr constant, so bucket b of
//     table l receives dT_l[b] = sum over its queries of c_lr dy_i / (L Z_lr,i),
//     and dv_j gains sum_l dT_l[c_l(k_j)];
//   gates: da = dg g (1 - g), dW = sum da x_gate, db = sum da, dx_gate = sum_h da W.
// Kernels (all deterministic: no atomics, fixed summation orders):
//   prep     per query: z, o_lr and the gates as the forward's fusion saved
//            them (ELSAA_OPT_SAVE_FOR_BACKWARD) or recomputed like it, alpha, and
//            writes do and the RACE row c_lr dy / z (both in dtype), delta,
//            da_s, da_lr and the query's share of dL/dlambda;
//   dq, dkv  the sparse branch: bfloat16 tiles of 64 sorted queries (keys) on
//            MFMA (S^T = K Q^T, dP^T = V dO^T, dQ^T = K^T dS^T; and S = Q K^T,
//            dP = dO V^T, dV^T = dO^T P, dK^T = Q^T dS), key (query) blocks of
//            64 staged in LDS with their transposes; binary32 inputs: 16 lanes
//            per row;
//   RACE     the query codes transposed table-major, then the forward's RACE
//            build (a per-table counting sort and segmented sums) over the
//            query rows gives dT; a per-key gather adds it to dv;
//   gates    dx_gate per token; dW_g, db_g and dlambda as per-block partial
//            sums reduced in a fixed order.
#include <type_traits>

#include "elsaa_internal.hpp"

namespace elsaa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// Sum over the 16 lanes of a row group (lane bits 0-3).
__device__ __forceinline__ float sum16(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 8);
  return x;
}

template <typename VT, int C>
__device__ __forceinline__ void load_cols(const VT *p, float (&out)[C]) {
#pragma unroll
  for (int c = 0; c < C; c += 4) Elem<VT>::load4(p + c, out + c);
}

template <typename VT, int C>
__device__ __forceinline__ void store_cols(VT *p, const float (&val)[C]) {
#pragma unroll
  for (int c = 0; c < C; c += 4) Elem<VT>::store4(p + c, val + c);
}

template <bool kIdent>
__device__ __forceinline__ int sorted_at(const int32_t *__restrict__ perm, long long seg, int r) {
  if constexpr (kIdent) {
    return r;
  } else {
    return perm[seg + r];
  }
}

// ------------------------------------------------------------------ prep --
struct PrepArgs {
  const void *dy;         // [BH][N][D] dtype
  const void *o_s;        // [BH][N][D] dtype (the sparse output; NULL for RACE only)
  const float *lse;       // [BH][N]
  const void *qcodes;     // [BH*N][L] query RACE codes
  const void *tsum;       // [BH][L][2^P][D] dtype
  const float *tcnt;      // [BH][L][2^P]
  const void *x_gate;     // [B][N][DG] dtype
  const float *gate_w;    // [2][H][DG]
  const float *gate_b;    // [2][H]
  // saved by the forward (ELSAA_OPT_SAVE_FOR_BACKWARD; else NULL)
  const void *sv_olr;     // [BH][N][D] dtype
  const float *sv_z, *sv_gs, *sv_glr;  // [BH][N]
  int H, N, L, P, DG, rcb, variant;
  float lambda;
  void *do_s;             // out [BH][N][D] dtype
  float *delta;           // out [BH][N]
  void *dcon;             // out [BH][N][D] dtype: c_lr dy / z (0 where z = 0)
  float *da_s, *da_lr;    // out [BH][N]
  float *dlam;            // out [BH][N]: the query's share of dL/dlambda
};

template <typename VT, int D>
__global__ __launch_bounds__(256) void elsaa_k6_bwd_prep(PrepArgs a, long long rows) {
  constexpr int C = D / 16;
  const int sub = threadIdx.x & 15;
  const long long r = (static_cast<long long>(blockIdx.x) * 256 + threadIdx.x) >> 4;
  if (r >= rows) return;  // whole row groups (rows is a multiple of 16)
  const long long bh = r / a.N;
  const int h = static_cast<int>(bh % a.H);
  const long long b = bh / a.H;
  const int i = static_cast<int>(r - bh * a.N);
  const bool sparse = a.variant != ELSAA_VARIANT_RACE_ONLY;
  const bool race = a.variant != ELSAA_VARIANT_SPARSE_ONLY;
  const bool gated = a.variant == ELSAA_VARIANT_FULL || a.variant == ELSAA_VARIANT_NO_ALPHA;
  const int nb = 1 << a.P;

  float dy[C];
  load_cols<VT, C>(static_cast<const VT *>(a.dy) + r * D + sub * C, dy);
  float os[C];
#pragma unroll
  for (int c = 0; c < C; ++c) os[c] = 0.0f;
  float lse_i = 0.0f;
  if (sparse) {
    load_cols<VT, C>(static_cast<const VT *>(a.o_s) + r * D + sub * C, os);
    lse_i = a.lse[r];
  }
  // low-rank output, as the fusion computes it: o_lr = sum of rows / sum of counts
  float z = 0.0f, olr[C];
#pragma unroll
  for (int c = 0; c < C; ++c) olr[c] = 0.0f;
  if (race && a.sv_olr) {
    load_cols<VT, C>(static_cast<const VT *>(a.sv_olr) + r * D + sub * C, olr);
    z = a.sv_z[r];
  } else if (race) {
    for (int l = 0; l < a.L; ++l) {
      const uint32_t code = a.rcb == 1 ? static_cast<const uint8_t *>(a.qcodes)[r * a.L + l]
                                       : static_cast<const uint16_t *>(a.qcodes)[r * a.L + l];
      const long long t = (bh * a.L + l) * nb + code;
      z += a.tcnt[t];
      float row[C];
      load_cols<VT, C>(static_cast<const VT *>(a.tsum) + t * D + sub * C, row);
#pragma unroll
      for (int c = 0; c < C; ++c) olr[c] += row[c];
    }
    const float rz = z > 0.0f ? 1.0f / z : 0.0f;
#pragma unroll
    for (int c = 0; c < C; ++c) olr[c] *= rz;
  }
  float g_s = 1.0f, g_lr = 1.0f, alpha = 1.0f;
  if (gated && a.sv_gs) {
    g_s = a.sv_gs[r];
    g_lr = a.sv_glr[r];
  } else if (gated) {
    float a0 = 0.0f, a1 = 0.0f;
    const VT *x = static_cast<const VT *>(a.x_gate) + (b * a.N + i) * a.DG;
    const float *w0 = a.gate_w + static_cast<long long>(h) * a.DG;
    const float *w1 = a.gate_w + static_cast<long long>(a.H + h) * a.DG;
    for (int e = sub; e < a.DG; e += 16) {
      const float xe = Elem<VT>::load(x + e);
      a0 = __builtin_fmaf(xe, w0[e], a0);
      a1 = __builtin_fmaf(xe, w1[e], a1);
    }
    a0 = sum16(a0);
    a1 = sum16(a1);
    g_s = 1.0f / (1.0f + __expf(-(a0 + a.gate_b[h])));
    g_lr = 1.0f / (1.0f + __expf(-(a1 + a.gate_b[a.H + h])));
  }
  if (gated) {
    const float mass = a.lambda * z / static_cast<float>(a.L);
    if (a.variant == ELSAA_VARIANT_FULL && mass > 0.0f) alpha = 1.0f / (1.0f + __expf(__logf(mass) - lse_i));
  }
  float dy_os = 0.0f, dy_olr = 0.0f;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    dy_os = __builtin_fmaf(dy[c], os[c], dy_os);
    dy_olr = __builtin_fmaf(dy[c], olr[c], dy_olr);
  }
  dy_os = sum16(dy_os);
  dy_olr = sum16(dy_olr);
  float c_s = 1.0f, c_lr = 1.0f, dlse = 0.0f, da_s = 0.0f, da_lr = 0.0f, dlam = 0.0f;
  if (a.variant == ELSAA_VARIANT_FULL) {
    c_s = g_s * alpha;
    c_lr = g_lr;
    const float dalpha = g_s * dy_os;
    dlse = dalpha * alpha * (1.0f - alpha);
    if (z > 0.0f) dlam = -dalpha * alpha * alpha * __expf(__logf(z / static_cast<float>(a.L)) - lse_i);
    da_s = alpha * dy_os * g_s * (1.0f - g_s);
    da_lr = dy_olr * g_lr * (1.0f - g_lr);
  } else if (a.variant == ELSAA_VARIANT_NO_ALPHA) {
    c_s = g_s;
    c_lr = g_lr;
    da_s = dy_os * g_s * (1.0f - g_s);
    da_lr = dy_olr * g_lr * (1.0f - g_lr);
  } else if (a.variant == ELSAA_VARIANT_RACE_ONLY) {
    c_s = 0.0f;
  } else {
    c_lr = 0.0f;
  }
  if (sparse) {
    float dov[C];
#pragma unroll
    for (int c = 0; c < C; ++c) dov[c] = c_s * dy[c];
    store_cols<VT, C>(static_cast<VT *>(a.do_s) + r * D + sub * C, dov);
    if (sub == 0) a.delta[r] = c_s * dy_os - dlse;
  }
  if (race) {
    const float sc = (c_lr != 0.0f && z > 0.0f) ? c_lr / z : 0.0f;
    float dc[C];
#pragma unroll
    for (int c = 0; c < C; ++c) dc[c] = sc * dy[c];
    store_cols<VT, C>(static_cast<VT *>(a.dcon) + r * D + sub * C, dc);
  }
  if (sub == 0) {
    a.da_s[r] = da_s;
    a.da_lr[r] = da_lr;
    a.dlam[r] = dlam;
  }
}

// -------------------------------------------------- sparse branch, bf16 --
// Staging of 64 rows (sorted ranks [s0, s0 + 64) of the segment, through perm)
// of two tensors x and y: row-major ([64][D + 8]) and, when kXT / kYT, also
// transposed ([D][64 + 4], row pairs packed in 32-bit words).  Each of the 256
// threads owns kPer (row pair, 8-column chunk) items.  The indices of a block
// are requested two blocks ahead and its rows one block ahead (into
// registers), so the loads overlap the previous block's products.
template <int D, bool kIdent, bool kXT, bool kYT, int kT = 256>
struct Stager {
  static constexpr int kRow = D + 8, kTRow = 64 + 4;
  static constexpr int kItems = 32 * (D / 8);              // (row pair, 8-column chunk) items
  static constexpr int kPer = (kItems + kT - 1) / kT;      // items a thread stages
  static constexpr bool kAll = kItems % kT == 0;           // every thread has kPer items
  int j0[kPer], j1[kPer];
  u16x8 x0[kPer], x1[kPer], y0[kPer], y1[kPer];
  __device__ __forceinline__ void load_idx(const int32_t *__restrict__ perm, long long seg, int s0, int tid) {
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int it = (tid + kT * p) % kItems;  // threads past the items repeat one (never stored)
      const int jp = it % 32;
      j0[p] = sorted_at<kIdent>(perm, seg, s0 + 2 * jp);
      j1[p] = sorted_at<kIdent>(perm, seg, s0 + 2 * jp + 1);
    }
  }
  __device__ __forceinline__ void load_rows(const uint16_t *__restrict__ x, const uint16_t *__restrict__ y,
                                            long long seg, int tid) {
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int ch = ((tid + kT * p) % kItems) / 32;
      x0[p] = *reinterpret_cast<const u16x8 *>(x + (seg + j0[p]) * D + ch * 8);
      x1[p] = *reinterpret_cast<const u16x8 *>(x + (seg + j1[p]) * D + ch * 8);
      y0[p] = *reinterpret_cast<const u16x8 *>(y + (seg + j0[p]) * D + ch * 8);
      y1[p] = *reinterpret_cast<const u16x8 *>(y + (seg + j1[p]) * D + ch * 8);
    }
  }
  __device__ __forceinline__ void store(uint16_t *xs, uint16_t *ys, uint16_t *xt, uint16_t *yt, int tid) const {
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      if (!kAll && tid + kT * p >= kItems) continue;
      const int jp = (tid + kT * p) % 32, ch = (tid + kT * p) / 32;
      *reinterpret_cast<u16x8 *>(xs + (2 * jp) * kRow + ch * 8) = x0[p];
      *reinterpret_cast<u16x8 *>(xs + (2 * jp + 1) * kRow + ch * 8) = x1[p];
      *reinterpret_cast<u16x8 *>(ys + (2 * jp) * kRow + ch * 8) = y0[p];
      *reinterpret_cast<u16x8 *>(ys + (2 * jp + 1) * kRow + ch * 8) = y1[p];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if constexpr (kXT)
          *reinterpret_cast<uint32_t *>(xt + (ch * 8 + e) * kTRow + 2 * jp) =
              static_cast<uint32_t>(x0[p][e]) | (static_cast<uint32_t>(x1[p][e]) << 16);
        if constexpr (kYT)
          *reinterpret_cast<uint32_t *>(yt + (ch * 8 + e) * kTRow + 2 * jp) =
              static_cast<uint32_t>(y0[p][e]) | (static_cast<uint32_t>(y1[p][e]) << 16);
      }
    }
  }
};

// 16-row tile products of a 64-row block held in LDS (rows row-major, kRow
// elements) with the wave's 16 columns (b[kk], the d-slice g*8 .. +7 of each
// 32): out[t] holds rows t*16 + g*4 + i of the lane's column.
template <int D>
__device__ __forceinline__ void block_times_cols(const uint16_t *rows, const bf16x8 (&b)[D / 32], f32x4 (&out)[4],
                                                 int g, int r16) {
  constexpr int kRow = D + 8;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    out[t] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8 *>(rows + (t * 16 + r16) * kRow +
                                                                                   kk * 32 + g * 8));
      out[t] = mfma16x16x32(a, b[kk], out[t]);
    }
  }
}

// acc[dt] += X^T W over the 64 rows of a block: X^T held transposed in LDS
// ([D][64 + 4]) and W the block's 64 x 16 weights of the lane's column in the
// layout of block_times_cols (w[t][i] is row t*16 + g*4 + i), packed to bf16
// per 32-row step in the order the transposed reads use.
template <int D>
__device__ __forceinline__ void transposed_times_weights(const uint16_t *xt, const f32x4 (&w)[4],
                                                         f32x4 (&acc)[D / 16], int g, int r16) {
  constexpr int kTRow = 64 + 4;
#pragma unroll
  for (int m2 = 0; m2 < 2; ++m2) {
    const bf16x8 bw = __builtin_bit_cast(
        bf16x8, (uint4){pack_bf16x2(w[2 * m2][0], w[2 * m2][1]), pack_bf16x2(w[2 * m2][2], w[2 * m2][3]),
                        pack_bf16x2(w[2 * m2 + 1][0], w[2 * m2 + 1][1]),
                        pack_bf16x2(w[2 * m2 + 1][2], w[2 * m2 + 1][3])});
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const uint16_t *xr = xt + (dt * 16 + r16) * kTRow + m2 * 32 + g * 4;
      const uint2 lo4 = *reinterpret_cast<const uint2 *>(xr);
      const uint2 hi4 = *reinterpret_cast<const uint2 *>(xr + 16);
      const bf16x8 a = __builtin_bit_cast(bf16x8, (uint4){lo4.x, lo4.y, hi4.x, hi4.y});
      acc[dt] = mfma16x16x32(a, bw, acc[dt]);
    }
  }
}

// dq: one workgroup per QT sorted queries (QT / 16 waves of 16; QT divides
// w), over the keys of their window in blocks of 64.
template <int D, bool kIdent, int QT>
__global__ __launch_bounds__(QT * 4) void elsaa_k6_bwd_dq_bf16(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ perm_q, const int32_t *__restrict__ perm_k, const uint16_t *__restrict__ do_s,
    const float *__restrict__ lse, const float *__restrict__ delta, int N, int w, int tiles_per_seg,
    float scale_log2, float scale, uint16_t *__restrict__ dq) {
  constexpr int kRow = D + 8, kTRow = 64 + 4;
  __shared__ __align__(16) uint16_t Ks[64 * kRow];
  __shared__ __align__(16) uint16_t Vs[64 * kRow];
  __shared__ __align__(16) uint16_t Kt[D * kTRow];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const long long tile = blockIdx.x;
  const long long seg = (tile / tiles_per_seg) * N;
  const int r0 = static_cast<int>(tile % tiles_per_seg) * QT;
  const int c = r0 / w;
  const int lo = c > 0 ? (c - 1) * w : 0, hi = (c + 1) * w;
  const int qidx = sorted_at<kIdent>(perm_q, seg, r0 + wave * 16 + r16);
  bf16x8 bq[D / 32], bdo[D / 32];
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    bq[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8 *>(q + (seg + qidx) * D + kk * 32 + g * 8));
    bdo[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8 *>(do_s + (seg + qidx) * D + kk * 32 + g * 8));
  }
  const float lse2 = lse[seg + qidx] * kLog2e, dlt = delta[seg + qidx];
  f32x4 acc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) acc[dt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
  using St = Stager<D, kIdent, true, false, QT * 4>;
  St st;
  st.load_idx(perm_k, seg, lo, tid);
  st.load_rows(k, v, seg, tid);
  int nxt[St::kPer][2];  // indices of the block after next
  for (int s0 = lo; s0 < hi; s0 += 64) {
    if (s0 != lo) __syncthreads();  // the previous block is consumed
    st.store(Ks, Vs, Kt, nullptr, tid);
    // the next block's indices were requested during the previous block
    if (s0 + 64 < hi) {
      if (s0 != lo) {
#pragma unroll
        for (int p = 0; p < st.kPer; ++p) {
          st.j0[p] = nxt[p][0];
          st.j1[p] = nxt[p][1];
        }
      } else {
        st.load_idx(perm_k, seg, s0 + 64, tid);
      }
      st.load_rows(k, v, seg, tid);
      if (s0 + 128 < hi) {
        St ix;
        ix.load_idx(perm_k, seg, s0 + 128, tid);
#pragma unroll
        for (int p = 0; p < st.kPer; ++p) {
          nxt[p][0] = ix.j0[p];
          nxt[p][1] = ix.j1[p];
        }
      }
    }
    __syncthreads();
    f32x4 s[4], dp[4];
    block_times_cols<D>(Ks, bq, s, g, r16);   // S^T: keys x the wave's queries
    block_times_cols<D>(Vs, bdo, dp, g, r16); // dP^T
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][i], scale_log2, -lse2));
        s[t][i] = p * (dp[t][i] - dlt);  // dS^T
      }
    transposed_times_weights<D>(Kt, s, acc, g, r16);  // dQ^T += K^T dS^T
  }
  uint16_t *row = dq + (seg + qidx) * D;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
    *reinterpret_cast<uint2 *>(row + dt * 16 + g * 4) =
        make_uint2(pack_bf16x2(acc[dt][0] * scale, acc[dt][1] * scale),
                   pack_bf16x2(acc[dt][2] * scale, acc[dt][3] * scale));
}

// dk, dv: one workgroup per QT sorted keys (QT / 16 waves of 16; QT divides w)
// of chunk c, over the sorted queries that attend them, [c w, min((c + 2) w,
// N)), in blocks of 64.
template <int D, bool kIdent, int QT>
__global__ __launch_bounds__(QT * 4) void elsaa_k6_bwd_dkv_bf16(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ perm_q, const int32_t *__restrict__ perm_k, const uint16_t *__restrict__ do_s,
    const float *__restrict__ lse, const float *__restrict__ delta, int N, int w, int tiles_per_seg,
    float scale_log2, float scale, uint16_t *__restrict__ dk, float *__restrict__ dv_acc) {
  constexpr int kRow = D + 8, kTRow = 64 + 4;
  extern __shared__ __align__(16) uint16_t lds[];
  uint16_t *Qs = lds, *Os = Qs + 64 * kRow, *Qt = Os + 64 * kRow, *Ot = Qt + D * kTRow;
  float *lse_s = reinterpret_cast<float *>(Ot + D * kTRow);  // [64], times log2(e)
  float *dlt_s = lse_s + 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const long long tile = blockIdx.x;
  const long long seg = (tile / tiles_per_seg) * N;
  const int t0 = static_cast<int>(tile % tiles_per_seg) * QT;
  const int c = t0 / w;
  const int lo = c * w, hi = (c + 2) * w < N ? (c + 2) * w : N;
  const int kidx = sorted_at<kIdent>(perm_k, seg, t0 + wave * 16 + r16);
  bf16x8 bk[D / 32], bv[D / 32];
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    bk[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8 *>(k + (seg + kidx) * D + kk * 32 + g * 8));
    bv[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8 *>(v + (seg + kidx) * D + kk * 32 + g * 8));
  }
  f32x4 dkt[D / 16], dvt[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    dkt[dt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    dvt[dt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
  }
  using St = Stager<D, kIdent, true, true, QT * 4>;
  St st;
  st.load_idx(perm_q, seg, lo, tid);
  st.load_rows(q, do_s, seg, tid);
  // the LSE and delta of the block's queries, one thread per query
  int qi_next = tid < 64 ? sorted_at<kIdent>(perm_q, seg, lo + tid) : 0;
  float lse_next = tid < 64 ? lse[seg + qi_next] * kLog2e : 0.0f;
  float dlt_next = tid < 64 ? delta[seg + qi_next] : 0.0f;
  int nxt[St::kPer][2];
  for (int s0 = lo; s0 < hi; s0 += 64) {
    if (s0 != lo) __syncthreads();
    st.store(Qs, Os, Qt, Ot, tid);
    if (tid < 64) {
      lse_s[tid] = lse_next;
      dlt_s[tid] = dlt_next;
    }
    if (s0 + 64 < hi) {
      if (s0 != lo) {
#pragma unroll
        for (int p = 0; p < St::kPer; ++p) {
          st.j0[p] = nxt[p][0];
          st.j1[p] = nxt[p][1];
        }
      } else {
        st.load_idx(perm_q, seg, s0 + 64, tid);
      }
      st.load_rows(q, do_s, seg, tid);
      if (tid < 64) {
        qi_next = sorted_at<kIdent>(perm_q, seg, s0 + 64 + tid);
        lse_next = lse[seg + qi_next] * kLog2e;
        dlt_next = delta[seg + qi_next];
      }
      if (s0 + 128 < hi) {
        St ix;
        ix.load_idx(perm_q, seg, s0 + 128, tid);
#pragma unroll
        for (int p = 0; p < St::kPer; ++p) {
          nxt[p][0] = ix.j0[p];
          nxt[p][1] = ix.j1[p];
        }
      }
    }
    __syncthreads();
    f32x4 s[4], dp[4];
    block_times_cols<D>(Qs, bk, s, g, r16);   // S: queries x the wave's keys
    block_times_cols<D>(Os, bv, dp, g, r16);  // dP
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const f32x4 l4 = *reinterpret_cast<const f32x4 *>(lse_s + t * 16 + g * 4);
      const f32x4 d4 = *reinterpret_cast<const f32x4 *>(dlt_s + t * 16 + g * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][i], scale_log2, -l4[i]));
        s[t][i] = p;                     // P
        dp[t][i] = p * (dp[t][i] - d4[i]);  // dS
      }
    }
    transposed_times_weights<D>(Ot, s, dvt, g, r16);   // dV^T += dO^T P
    transposed_times_weights<D>(Qt, dp, dkt, g, r16);  // dK^T += Q^T dS
  }
  uint16_t *krow = dk + (seg + kidx) * D;
  float *vrow = dv_acc + (seg + kidx) * D;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    *reinterpret_cast<uint2 *>(krow + dt * 16 + g * 4) =
        make_uint2(pack_bf16x2(dkt[dt][0] * scale, dkt[dt][1] * scale),
                   pack_bf16x2(dkt[dt][2] * scale, dkt[dt][3] * scale));
    *reinterpret_cast<f32x4 *>(vrow + dt * 16 + g * 4) = dvt[dt];
  }
}

// ------------------------------------------------- sparse branch, fp32 --
// 16 lanes per row (D/16 columns each), binary32 throughout.
template <int D>
__global__ __launch_bounds__(256) void elsaa_k6_bwd_dq_f32(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const int32_t *__restrict__ perm_q, const int32_t *__restrict__ perm_k, const float *__restrict__ do_s,
    const float *__restrict__ lse, const float *__restrict__ delta, int N, int w, long long rows, float scale,
    float *__restrict__ dq) {
  constexpr int C = D / 16;
  const int sub = threadIdx.x & 15;
  const long long rr = (static_cast<long long>(blockIdx.x) * 256 + threadIdx.x) >> 4;  // sorted row
  if (rr >= rows) return;
  const long long seg = rr / N * N;
  const int rank = static_cast<int>(rr - seg);
  const int c = rank / w;
  const int lo = c > 0 ? (c - 1) * w : 0, hi = (c + 1) * w;
  const int qi = perm_q ? perm_q[rr] : rank;
  float qv[C], dov[C], acc[C];
  load_cols<float, C>(q + (seg + qi) * D + sub * C, qv);
  load_cols<float, C>(do_s + (seg + qi) * D + sub * C, dov);
#pragma unroll
  for (int e = 0; e < C; ++e) acc[e] = 0.0f;
  const float l = lse[seg + qi], dl = delta[seg + qi];
  for (int t = lo; t < hi; ++t) {
    const int j = perm_k ? perm_k[seg + t] : t;
    float kv[C], vv[C];
    load_cols<float, C>(k + (seg + j) * D + sub * C, kv);
    load_cols<float, C>(v + (seg + j) * D + sub * C, vv);
    float sd = 0.0f, dp = 0.0f;
#pragma unroll
    for (int e = 0; e < C; ++e) {
      sd = __builtin_fmaf(qv[e], kv[e], sd);
      dp = __builtin_fmaf(dov[e], vv[e], dp);
    }
    sd = sum16(sd);
    dp = sum16(dp);
    const float ds = expf(sd * scale - l) * (dp - dl);
#pragma unroll
    for (int e = 0; e < C; ++e) acc[e] = __builtin_fmaf(ds, kv[e], acc[e]);
  }
#pragma unroll
  for (int e = 0; e < C; ++e) acc[e] *= scale;
  store_cols<float, C>(dq + (seg + qi) * D + sub * C, acc);
}

template <int D>
__global__ __launch_bounds__(256) void elsaa_k6_bwd_dkv_f32(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const int32_t *__restrict__ perm_q, const int32_t *__restrict__ perm_k, const float *__restrict__ do_s,
    const float *__restrict__ lse, const float *__restrict__ delta, int N, int w, long long rows, float scale,
    float *__restrict__ dk, float *__restrict__ dv_acc) {
  constexpr int C = D / 16;
  const int sub = threadIdx.x & 15;
  const long long rr = (static_cast<long long>(blockIdx.x) * 256 + threadIdx.x) >> 4;  // sorted key row
  if (rr >= rows) return;
  const long long seg = rr / N * N;
  const int rank = static_cast<int>(rr - seg);
  const int c = rank / w;
  const int lo = c * w, hi = (c + 2) * w < N ? (c + 2) * w : N;
  const int kj = perm_k ? perm_k[rr] : rank;
  float kv[C], vv[C], dka[C], dva[C];
  load_cols<float, C>(k + (seg + kj) * D + sub * C, kv);
  load_cols<float, C>(v + (seg + kj) * D + sub * C, vv);
#pragma unroll
  for (int e = 0; e < C; ++e) dka[e] = dva[e] = 0.0f;
  for (int t = lo; t < hi; ++t) {
    const int i = perm_q ? perm_q[seg + t] : t;
    float qv[C], dov[C];
    load_cols<float, C>(q + (seg + i) * D + sub * C, qv);
    load_cols<float, C>(do_s + (seg + i) * D + sub * C, dov);
    float sd = 0.0f, dp = 0.0f;
#pragma unroll
    for (int e = 0; e < C; ++e) {
      sd = __builtin_fmaf(qv[e], kv[e], sd);
      dp = __builtin_fmaf(dov[e], vv[e], dp);
    }
    sd = sum16(sd);
    dp = sum16(dp);
    const float p = expf(sd * scale - lse[seg + i]);
    const float ds = p * (dp - delta[seg + i]);
#pragma unroll
    for (int e = 0; e < C; ++e) {
      dka[e] = __builtin_fmaf(ds, qv[e], dka[e]);
      dva[e] = __builtin_fmaf(p, dov[e], dva[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < C; ++e) dka[e] *= scale;
  store_cols<float, C>(dk + (seg + kj) * D + sub * C, dka);
  store_cols<float, C>(dv_acc + (seg + kj) * D + sub * C, dva);
}

// --------------------------------------------------------- RACE branch --
// Query codes [rows][L] -> table-major [L][rows] (the RACE build's layout).
template <typename CT>
__global__ void elsaa_k6_bwd_codes_t(const CT *__restrict__ src, CT *__restrict__ dst, long long rows, int L) {
  const long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;  // destination element
  if (i < rows * L) dst[i] = src[(i % rows) * L + i / rows];
}

// dv_j = (sparse part) + sum_l dT_l[c_l(k_j)]: 16 lanes per key, original order.
template <typename VT, int D, typename CT>
__global__ __launch_bounds__(256) void elsaa_k6_bwd_dv(const float *__restrict__ dv_acc, const CT *__restrict__ kcodes,
                                                       const VT *__restrict__ dT, long long rows, int N, int L,
                                                       int P, VT *__restrict__ dv) {
  constexpr int C = D / 16;
  const int sub = threadIdx.x & 15;
  const long long r = (static_cast<long long>(blockIdx.x) * 256 + threadIdx.x) >> 4;
  if (r >= rows) return;
  const long long bh = r / N;
  float acc[C];
#pragma unroll
  for (int e = 0; e < C; ++e) acc[e] = 0.0f;
  if (dv_acc) load_cols<float, C>(dv_acc + r * D + sub * C, acc);
  if (dT) {
    for (int l = 0; l < L; ++l) {
      const long long t = (bh * L + l) * (1ll << P) + kcodes[static_cast<long long>(l) * rows + r];
      float row[C];
      load_cols<VT, C>(dT + t * D + sub * C, row);
#pragma unroll
      for (int e = 0; e < C; ++e) acc[e] += row[e];
    }
  }
  store_cols<VT, C>(dv + r * D + sub * C, acc);
}

// The same sum, gathered the way the forward's fusion gathers table rows: a
// workgroup of four waves takes 64 consecutive keys of one (b, h), stages
// their L codes per table in LDS (one 64-byte load per table), and each wave
// step covers 64 / (lanes per row) keys with 16-byte lane pieces, its LC row
// loads (LC = 8 or 16) issued together: one load instruction per table for
// 8 keys of bfloat16 d = 64, where 16 lanes per key took four.
template <typename VT, int D, typename CT, int LC>
__global__ __launch_bounds__(256) void elsaa_k6_bwd_dv_wide(const float *__restrict__ dv_acc,
                                                            const CT *__restrict__ kcodes, const VT *__restrict__ dT,
                                                            long long rows, int N, int P, VT *__restrict__ dv) {
  constexpr int kCols = 16 / static_cast<int>(sizeof(VT));  // columns per lane
  constexpr int kLPR = D / kCols;                           // lanes per key
  constexpr int kKPS = 64 / kLPR;                           // keys per wave step
  __shared__ CT codes[LC][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long long r0 = static_cast<long long>(blockIdx.x) * 64;  // N is a multiple of 64
  const long long bh = r0 / N;
  for (int i = tid; i < LC * 64; i += 256) codes[i >> 6][i & 63] = kcodes[static_cast<long long>(i >> 6) * rows + r0 + (i & 63)];
  __syncthreads();
  const int cc = lane % kLPR;
  const long long nb = 1ll << P;
  const VT *tb = dT ? dT + bh * LC * nb * D + cc * kCols : nullptr;
#pragma unroll
  for (int st = 0; st < 16 / kKPS; ++st) {
    const int kk = wave * 16 + st * kKPS + lane / kLPR;  // key within the block
    const long long r = r0 + kk;
    float acc[kCols];
#pragma unroll
    for (int e = 0; e < kCols; ++e) acc[e] = 0.0f;
    if (dv_acc) {
#pragma unroll
      for (int e = 0; e < kCols; e += 4) {
        const f32x4 x = *reinterpret_cast<const f32x4 *>(dv_acc + r * D + cc * kCols + e);
        acc[e] = x[0]; acc[e + 1] = x[1]; acc[e + 2] = x[2]; acc[e + 3] = x[3];
      }
    }
    if (tb) {
      u32x4 t[LC];
#pragma unroll
      for (int l = 0; l < LC; ++l)
        t[l] = *reinterpret_cast<const u32x4 *>(tb + (l * nb + static_cast<long long>(codes[l][kk])) * D);
#pragma unroll
      for (int l = 0; l < LC; ++l) {
        if constexpr (sizeof(VT) == 2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[2 * e] += __uint_as_float(t[l][e] << 16);
            acc[2 * e + 1] += __uint_as_float(t[l][e] & 0xffff0000u);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] += __uint_as_float(t[l][e]);
        }
      }
    }
    if constexpr (sizeof(VT) == 2) {
      *reinterpret_cast<u32x4 *>(dv + r * D + cc * kCols) =
          u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                pack_bf16x2(acc[6], acc[7])};
    } else {
      *reinterpret_cast<f32x4 *>(dv + r * D + cc * kCols) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    }
  }
}

// -------------------------------------------------------------- gates --
// dx_gate[b][i][e] = sum_h da_s[b][h][i] W_g[0][h][e] + da_lr[b][h][i] W_g[1][h][e]
template <typename VT>
__global__ __launch_bounds__(256) void elsaa_k6_bwd_dxgate(const float *__restrict__ da_s, const float *__restrict__ da_lr,
                                                           const float *__restrict__ gate_w, int B, int H, int N,
                                                           int DG, VT *__restrict__ dx) {
  const long long idx = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<long long>(B) * N * DG) return;
  const int e = static_cast<int>(idx % DG);
  const long long t = idx / DG;  // b * N + i
  const long long b = t / N;
  const int i = static_cast<int>(t - b * N);
  float acc = 0.0f;
  // four heads a round, their loads issued together
  int h = 0;
  for (; h + 4 <= H; h += 4) {
    float a[4], c[4], w[4], v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const long long r = (b * H + h + u) * N + i;
      a[u] = da_s[r];
      c[u] = da_lr[r];
      w[u] = gate_w[static_cast<long long>(h + u) * DG + e];
      v[u] = gate_w[static_cast<long long>(H + h + u) * DG + e];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc = __builtin_fmaf(a[u], w[u], acc);
      acc = __builtin_fmaf(c[u], v[u], acc);
    }
  }
  for (; h < H; ++h) {
    const long long r = (b * H + h) * N + i;
    acc = __builtin_fmaf(da_s[r], gate_w[static_cast<long long>(h) * DG + e], acc);
    acc = __builtin_fmaf(da_lr[r], gate_w[static_cast<long long>(H + h) * DG + e], acc);
  }
  dx[idx] = Elem<VT>::store_val(acc);
}

// Partial sums over a block of tokens of head h: dW_g[0][h][:], dW_g[1][h][:],
// db_g[0][h], db_g[1][h] and dL/dlambda, into part[h][blk][2 DG + 3].  Wave w
// takes tokens t_lo + w, + 4, ... (its da values are wave-uniform loads), lanes
// the gate columns; the four waves' sums are added in LDS in wave order.
template <typename VT, int kPer>  // kPer >= DG / 64: gate columns per lane
__global__ __launch_bounds__(256) void elsaa_k6_bwd_gate_part(const float *__restrict__ da_s,
                                                              const float *__restrict__ da_lr,
                                                              const float *__restrict__ dlam, const VT *__restrict__ x,
                                                              int B, int H, int N, int DG, float *__restrict__ part) {
  __shared__ float red[4][2 * 512 + 3];
  const int h = blockIdx.x, blk = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long long tokens = static_cast<long long>(B) * N;
  const long long per = (tokens + kGateBlocks - 1) / kGateBlocks;
  const long long t_lo = blk * per, t_hi = t_lo + per < tokens ? t_lo + per : tokens;
  float w0[kPer], w1[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) w0[j] = w1[j] = 0.0f;
  float b0 = 0.0f, b1 = 0.0f, lam = 0.0f;
  // kU tokens a round, every load of the round issued before the first use
  // (one token at a time left each wave a chain of dependent loads)
  constexpr int kU = 8;
  for (long long t0 = t_lo + wave; t0 < t_hi; t0 += 4 * kU) {
    float s0[kU], s1[kU], sl[kU], xe[kU][kPer];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const long long t = t0 + 4 * u;
      const bool ok = t < t_hi;
      const long long tc = ok ? t : t_lo;
      const long long b = tc / N;
      const long long r = (b * H + h) * N + (tc - b * N);
      // loads at clamped addresses and selects (no branch around a load,
      // which would wait for it at the branch's end)
      const float a0 = da_s[r], a1 = da_lr[r], al = dlam[r];
      s0[u] = ok ? a0 : 0.0f;
      s1[u] = ok ? a1 : 0.0f;
      sl[u] = ok ? al : 0.0f;
      const VT *xr = x + tc * DG;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int e = lane + 64 * j;
        const float xv = Elem<VT>::load(xr + (e < DG ? e : DG - 1));
        xe[u][j] = e < DG ? xv : 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      b0 += s0[u];
      b1 += s1[u];
      lam += sl[u];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        w0[j] = __builtin_fmaf(s0[u], xe[u][j], w0[j]);
        w1[j] = __builtin_fmaf(s1[u], xe[u][j], w1[j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = lane + 64 * j;
    if (e < DG) {
      red[wave][e] = w0[j];
      red[wave][DG + e] = w1[j];
    }
  }
  if (lane == 0) {
    red[wave][2 * DG] = b0;
    red[wave][2 * DG + 1] = b1;
    red[wave][2 * DG + 2] = lam;
  }
  __syncthreads();
  float *out = part + (static_cast<long long>(h) * kGateBlocks + blk) * (2 * DG + 3);
  for (int e = threadIdx.x; e < 2 * DG + 3; e += 256) out[e] = ((red[0][e] + red[1][e]) + red[2][e]) + red[3][e];
}

// The same partial sums with every head in one workgroup (d_gate <= 64,
// H <= kMaxH): a token's gate-input row is read by four waves instead of once
// per head.  Block blk stages the da_s, da_lr and dL/dlambda shares of its
// tokens for every head in LDS (coalesced rows of each head); then its 16
// waves split into four head groups of four: wave (group, quarter) takes the
// group's heads and tokens t_lo + quarter, + 4, ... in order, lanes the gate
// columns.  The quarters' sums of each head are added in LDS in quarter
// order into part[h][blk][2 DG + 3], the layout gate_reduce reads.  The
// same kernel writes dx_gate from the staged shares.
constexpr int kMaxH = 16;
constexpr int kHeadGroups = 4;
template <typename VT>
__global__ __launch_bounds__(1024) void elsaa_k6_bwd_gate_part_heads(const float *__restrict__ da_s,
                                                                     const float *__restrict__ da_lr,
                                                                     const float *__restrict__ dlam,
                                                                     const VT *__restrict__ x, const float *__restrict__ gate_w,
                                                                     int B, int H, int N, int DG,
                                                                     float *__restrict__ part, VT *__restrict__ dx) {
  constexpr int kHpg = kMaxH / kHeadGroups;  // heads a group holds at most
  extern __shared__ float st[];  // [3][H][per] staged shares, then [4][H][2 DG + 3] quarter sums
  const int blk = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wave / 4, tq = wave % 4;
  const int hpg = (H + kHeadGroups - 1) / kHeadGroups;
  const long long tokens = static_cast<long long>(B) * N;
  const int per = static_cast<int>((tokens + kGateBlocks - 1) / kGateBlocks);
  const long long t_lo = static_cast<long long>(blk) * per;
  const int n = static_cast<int>(t_lo + per < tokens ? per : (tokens > t_lo ? tokens - t_lo : 0));
  // staging: row (a, h) holds array a's shares of head h for tokens t_lo ..
  // t_lo + n - 1; kR rows a round, every load of the round issued before its
  // stores (one row at a time left each thread a chain of dependent loads)
  constexpr int kR = 12;
  for (int r0 = 0; r0 < 3 * H; r0 += kR) {
    for (int j = tid; j < n; j += 1024) {
      const long long t = t_lo + j;
      const long long b = t / N;
      const long long i = t - b * N;
      float v[kR];
#pragma unroll
      for (int u = 0; u < kR; ++u) {
        const int row = r0 + u < 3 * H ? r0 + u : 3 * H - 1;
        const int a = row / H, h = row - a * H;
        const float *src = a == 0 ? da_s : (a == 1 ? da_lr : dlam);
        v[u] = src[(b * H + h) * N + i];
      }
#pragma unroll
      for (int u = 0; u < kR; ++u)
        if (r0 + u < 3 * H) st[(r0 + u) * per + j] = v[u];
    }
  }
  __syncthreads();
  const int e = lane < DG ? lane : DG - 1;  // clamped column (lanes past d_gate add zeros)
  {  // dx_gate of the block's tokens: wave w takes tokens w, w + 16, ...; the
     // heads in order, as the per-token kernel adds them
    float g0[kMaxH], g1[kMaxH];
#pragma unroll
    for (int h = 0; h < kMaxH; ++h) {
      g0[h] = h < H ? gate_w[static_cast<long long>(h) * DG + e] : 0.0f;
      g1[h] = h < H ? gate_w[static_cast<long long>(H + h) * DG + e] : 0.0f;
    }
    for (int j = wave; j < n; j += 16) {
      float acc = 0.0f;
#pragma unroll
      for (int h = 0; h < kMaxH; ++h) {
        if (h < H) {
          acc = __builtin_fmaf(st[h * per + j], g0[h], acc);
          acc = __builtin_fmaf(st[(H + h) * per + j], g1[h], acc);
        }
      }
      if (lane < DG) dx[(t_lo + j) * DG + lane] = Elem<VT>::store_val(acc);
    }
  }
  float w0[kHpg], w1[kHpg], b0[kHpg], b1[kHpg], lm[kHpg];
#pragma unroll
  for (int k = 0; k < kHpg; ++k) w0[k] = w1[k] = b0[k] = b1[k] = lm[k] = 0.0f;
  constexpr int kU = 8;                     // tokens a round, their rows requested together
  for (int j0 = tq; j0 < n; j0 += 4 * kU) {
    float xe[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int j = j0 + 4 * u < n ? j0 + 4 * u : n - 1;
      const float xv = Elem<VT>::load(x + (t_lo + j) * DG + e);
      xe[u] = lane < DG ? xv : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int j = j0 + 4 * u;
      if (j < n) {
#pragma unroll
        for (int k = 0; k < kHpg; ++k) {
          const int h = hg * hpg + k;
          if (k < hpg && h < H) {
            const float s0 = st[h * per + j], s1 = st[(H + h) * per + j];
            w0[k] = __builtin_fmaf(s0, xe[u], w0[k]);
            w1[k] = __builtin_fmaf(s1, xe[u], w1[k]);
            b0[k] += s0;
            b1[k] += s1;
            lm[k] += st[(2 * H + h) * per + j];
          }
        }
      }
    }
  }
  __syncthreads();  // the staged shares are consumed: the LDS holds the quarter sums next
  const int stride = 2 * DG + 3;
  float *red = st + static_cast<long long>(tq) * H * stride;
#pragma unroll
  for (int k = 0; k < kHpg; ++k) {
    const int h = hg * hpg + k;
    if (k < hpg && h < H) {
      if (lane < DG) {
        red[h * stride + lane] = w0[k];
        red[h * stride + DG + lane] = w1[k];
      }
      if (lane == 0) {
        red[h * stride + 2 * DG] = b0[k];
        red[h * stride + 2 * DG + 1] = b1[k];
        red[h * stride + 2 * DG + 2] = lm[k];
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < H * stride; i += 1024) {
    const int h = i / stride, c = i - h * stride;
    const long long hs = static_cast<long long>(H) * stride;
    part[(static_cast<long long>(h) * kGateBlocks + blk) * stride + c] =
        ((st[i] + st[hs + i]) + st[2 * hs + i]) + st[3 * hs + i];
  }
}

// Block h < H: dW_g and db_g of head h; block H: dL/dlambda.  Partials are
// added in block order (eight independent running sums, then combined).
__global__ __launch_bounds__(256) void elsaa_k6_bwd_gate_reduce(const float *__restrict__ part, int H, int DG,
                                                                int with_lambda, float *__restrict__ dgate_w,
                                                                float *__restrict__ dgate_b, float *__restrict__ dlambda) {
  const int h = blockIdx.x;
  const int stride = 2 * DG + 3;
  // sum over kGateBlocks entries stride apart: eight running sums (entry
  // blk goes to sum blk % 8), 32 entries requested at a time
  auto sum_blocks = [&](const float *p) {
    static_assert(kGateBlocks % 32 == 0, "whole rounds of 32 partial sums");
    float acc[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = 0.0f;
    for (int blk = 0; blk < kGateBlocks; blk += 32) {
      float v[32];
#pragma unroll
      for (int u = 0; u < 32; ++u) v[u] = p[static_cast<long long>(blk + u) * stride];
#pragma unroll
      for (int u = 0; u < 32; ++u) acc[u % 8] += v[u];
    }
    return ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  };
  if (h < H) {
    const float *p = part + static_cast<long long>(h) * kGateBlocks * stride;
    for (int e = threadIdx.x; e < 2 * DG + 2; e += 256) {
      const float s = sum_blocks(p + e);
      if (e < DG) dgate_w[static_cast<long long>(h) * DG + e] = s;
      else if (e < 2 * DG) dgate_w[static_cast<long long>(H + h) * DG + (e - DG)] = s;
      else if (e == 2 * DG) dgate_b[h] = s;
      else dgate_b[H + h] = s;
    }
  } else {
    // thread t adds the dL/dlambda shares of heads t, t + 256, ... (in that
    // order), then thread 0 adds the threads' sums in thread order: head
    // order whenever H <= 256
    __shared__ float lam_t[256];
    float own = 0.0f;
    for (int hh = threadIdx.x; hh < H; hh += 256)
      own += sum_blocks(part + static_cast<long long>(hh) * kGateBlocks * stride + 2 * DG + 2);
    lam_t[threadIdx.x] = own;
    __syncthreads();
    if (threadIdx.x == 0) {
      float s = 0.0f;
      for (int t = 0; t < (H < 256 ? H : 256); ++t) s += lam_t[t];
      *dlambda = with_lambda ? s : 0.0f;
    }
  }
}

__global__ void elsaa_k6_bwd_zero_f32(float *__restrict__ p, long long n) {
  const long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

unsigned blocks_for(long long threads) { return static_cast<unsigned>((threads + 255) / 256); }

template <int D, bool kIdent>
void launch_sparse_bf16(const Geometry &g, const void *q, const void *k, const void *v, const int32_t *pq,
                        const int32_t *pk, const BackwardBuffers &bb, const float *lse, void *dq, void *dk,
                        hipStream_t stream) {
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  const float scale_log2 = scale * kLog2e;
  constexpr size_t kLds = (2 * 64 * (D + 8) + 2 * D * (64 + 4)) * 2 + 2 * 64 * 4;
  auto tiles = [&](int qt) { return static_cast<unsigned>(static_cast<long long>(g.N / qt) * g.BH); };
  auto dq_launch = [&](auto qt) {
    constexpr int QT = decltype(qt)::value;
    hipLaunchKernelGGL((elsaa_k6_bwd_dq_bf16<D, kIdent, QT>), dim3(tiles(QT)), dim3(QT * 4), 0, stream,
                       static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                       static_cast<const uint16_t *>(v), pq, pk, static_cast<const uint16_t *>(bb.do_s), lse,
                       bb.delta, g.N, g.w, g.N / QT, scale_log2, scale, static_cast<uint16_t *>(dq));
  };
  // dq: 128-query tiles when w allows at d = 64 (each staged key block serves
  // twice the queries: 232 -> 210 us at text32k); dk, dv: 64-key tiles (128
  // took 398 against 340 us: 157 VGPRs leave one 8-wave workgroup per CU)
  if (D == 64 && g.w % 128 == 0) dq_launch(std::integral_constant<int, 128>{});
  else dq_launch(std::integral_constant<int, 64>{});
  hipLaunchKernelGGL((elsaa_k6_bwd_dkv_bf16<D, kIdent, 64>), dim3(tiles(64)), dim3(256), kLds, stream,
                     static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                     static_cast<const uint16_t *>(v), pq, pk, static_cast<const uint16_t *>(bb.do_s), lse,
                     bb.delta, g.N, g.w, g.N / 64, scale_log2, scale, static_cast<uint16_t *>(dk), bb.dv_acc);
}

template <int D>
void launch_sparse_f32(const Geometry &g, const void *q, const void *k, const void *v, const int32_t *pq,
                       const int32_t *pk, const BackwardBuffers &bb, const float *lse, void *dq, void *dk,
                       hipStream_t stream) {
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  const unsigned grid = blocks_for(g.rows * 16);
  hipLaunchKernelGGL(elsaa_k6_bwd_dq_f32<D>, dim3(grid), dim3(256), 0, stream, static_cast<const float *>(q),
                     static_cast<const float *>(k), static_cast<const float *>(v), pq, pk,
                     static_cast<const float *>(bb.do_s), lse, bb.delta, g.N, g.w, g.rows, scale,
                     static_cast<float *>(dq));
  hipLaunchKernelGGL(elsaa_k6_bwd_dkv_f32<D>, dim3(grid), dim3(256), 0, stream, static_cast<const float *>(q),
                     static_cast<const float *>(k), static_cast<const float *>(v), pq, pk,
                     static_cast<const float *>(bb.do_s), lse, bb.delta, g.N, g.w, g.rows, scale,
                     static_cast<float *>(dk), bb.dv_acc);
}

template <typename VT, int D>
hipError_t launch_backward_t(const Geometry &g, const BackwardInputs &in, const Buffers &fb,
                             const BackwardBuffers &bb, const BackwardOutputs &out, hipStream_t stream) {
  const bool sparse = g.run_sparse, race = g.run_race;
  const bool gated = g.variant == ELSAA_VARIANT_FULL || g.variant == ELSAA_VARIANT_NO_ALPHA;
  const size_t rows = static_cast<size_t>(g.rows);
  hipError_t e = hipSuccess;
  auto check = [&]() {
    if (e == hipSuccess) e = hipGetLastError();
    return e == hipSuccess;
  };
  // 1. per query: the fusion's derivatives
  PrepArgs pa{};
  pa.dy = in.dy;
  pa.o_s = race ? fb.o_s : in.y;  // sparse only: o_s is the forward output itself
  pa.lse = fb.lse;
  pa.qcodes = fb.rcode;
  pa.tsum = fb.tsum;
  pa.tcnt = fb.tcnt;
  pa.x_gate = in.x_gate;
  pa.gate_w = in.gate_w;
  pa.gate_b = in.gate_b;
  pa.sv_olr = fb.sv_olr;
  pa.sv_z = fb.sv_z;
  pa.sv_gs = fb.sv_gs;
  pa.sv_glr = fb.sv_glr;
  pa.H = g.H; pa.N = g.N; pa.L = g.L; pa.P = g.P; pa.DG = g.DG; pa.rcb = g.rcb; pa.variant = g.variant;
  pa.lambda = in.lambda;
  pa.do_s = bb.do_s; pa.delta = bb.delta; pa.dcon = bb.dcon;
  pa.da_s = bb.da_s; pa.da_lr = bb.da_lr; pa.dlam = bb.dlam;
  hipLaunchKernelGGL((elsaa_k6_bwd_prep<VT, D>), dim3(blocks_for(g.rows * 16)), dim3(256), 0, stream, pa, g.rows);
  if (!check()) return e;
  // 2. sparse branch: dq, dk and the sparse part of dv
  const int32_t *pq = g.identity ? nullptr : fb.perm;
  const int32_t *pk = g.identity ? nullptr : fb.perm + g.rows;
  if (sparse) {
    if constexpr (sizeof(VT) == 2) {
      if (g.identity) launch_sparse_bf16<D, true>(g, in.q, in.k, in.v, pq, pk, bb, fb.lse, out.dq, out.dk, stream);
      else launch_sparse_bf16<D, false>(g, in.q, in.k, in.v, pq, pk, bb, fb.lse, out.dq, out.dk, stream);
    } else {
      launch_sparse_f32<D>(g, in.q, in.k, in.v, pq, pk, bb, fb.lse, out.dq, out.dk, stream);
    }
    if (!check()) return e;
  } else {
    for (void *p : {out.dq, out.dk}) {
      e = launch_fill_zero(p, rows * D * sizeof(VT), stream);
      if (e != hipSuccess) return e;
    }
  }
  // 3. RACE branch: dT by the forward's RACE build over the query rows, then dv
  if (race) {
    if (g.rcb == 1)
      hipLaunchKernelGGL(elsaa_k6_bwd_codes_t<uint8_t>, dim3(blocks_for(g.rows * g.L)), dim3(256), 0, stream,
                         static_cast<const uint8_t *>(fb.rcode), static_cast<uint8_t *>(bb.qcode_t), g.rows, g.L);
    else
      hipLaunchKernelGGL(elsaa_k6_bwd_codes_t<uint16_t>, dim3(blocks_for(g.rows * g.L)), dim3(256), 0, stream,
                         static_cast<const uint16_t *>(fb.rcode), static_cast<uint16_t *>(bb.qcode_t), g.rows, g.L);
    if (!check()) return e;
    RaceBuildIO io;
    io.codes = bb.qcode_t;
    io.values = bb.dcon;
    io.values_f32 = false;  // rows and sums in dtype, accumulated in binary32
    io.rperm = bb.qrperm;
    io.hist = bb.qhist;
    io.rstart = bb.qrstart;
    io.rpart = bb.qrpart;
    io.tsum = bb.dT;
    io.tcnt = bb.qtcnt;
    io.flag = bb.flag;
    e = launch_race_build_io(g, io, stream);
    if (e != hipSuccess) return e;
  }
  {
    const float *dva = sparse ? bb.dv_acc : nullptr;
    const VT *dT = race ? static_cast<const VT *>(bb.dT) : nullptr;
    const void *kc = static_cast<const char *>(fb.rcode) + rows * g.L * g.rcb;  // key codes, table-major
    const unsigned kblocks = static_cast<unsigned>(g.rows / 64);
    auto wide = [&](auto ct, auto lc) {
      using CT = decltype(ct);
      constexpr int LC = decltype(lc)::value;
      hipLaunchKernelGGL((elsaa_k6_bwd_dv_wide<VT, D, CT, LC>), dim3(kblocks), dim3(256), 0, stream, dva,
                         static_cast<const CT *>(kc), dT, g.rows, g.N, g.P, static_cast<VT *>(out.dv));
    };
    using L8 = std::integral_constant<int, 8>;
    using L16 = std::integral_constant<int, 16>;
    if (g.L == 16 || g.L == 8) {
      if (g.rcb == 1) {
        if (g.L == 16) wide(uint8_t{}, L16{});
        else wide(uint8_t{}, L8{});
      } else {
        if (g.L == 16) wide(uint16_t{}, L16{});
        else wide(uint16_t{}, L8{});
      }
    } else if (g.rcb == 1) {
      hipLaunchKernelGGL((elsaa_k6_bwd_dv<VT, D, uint8_t>), dim3(blocks_for(g.rows * 16)), dim3(256), 0, stream, dva,
                         static_cast<const uint8_t *>(kc), dT, g.rows, g.N, g.L, g.P, static_cast<VT *>(out.dv));
    } else {
      hipLaunchKernelGGL((elsaa_k6_bwd_dv<VT, D, uint16_t>), dim3(blocks_for(g.rows * 16)), dim3(256), 0, stream,
                         dva, static_cast<const uint16_t *>(kc), dT, g.rows, g.N, g.L, g.P,
                         static_cast<VT *>(out.dv));
    }
    if (!check()) return e;
  }
  // 4. gates and lambda
  const long long nx = static_cast<long long>(g.B) * g.N * g.DG;
  if (gated) {
    const long long per = (static_cast<long long>(g.B) * g.N + kGateBlocks - 1) / kGateBlocks;
    const size_t heads_lds = static_cast<size_t>(
        4 * (3 * g.H * per > 4ll * g.H * (2 * g.DG + 3) ? 3 * g.H * per : 4ll * g.H * (2 * g.DG + 3)));
    if (g.DG <= 64 && g.H <= kMaxH && heads_lds <= 64 * 1024) {
      hipLaunchKernelGGL(elsaa_k6_bwd_gate_part_heads<VT>, dim3(kGateBlocks), dim3(1024), heads_lds, stream, bb.da_s,
                         bb.da_lr, bb.dlam, static_cast<const VT *>(in.x_gate), in.gate_w, g.B, g.H, g.N, g.DG,
                         bb.gate_part, static_cast<VT *>(out.dx_gate));
    } else {
      hipLaunchKernelGGL(elsaa_k6_bwd_dxgate<VT>, dim3(blocks_for(nx)), dim3(256), 0, stream, bb.da_s, bb.da_lr,
                         in.gate_w, g.B, g.H, g.N, g.DG, static_cast<VT *>(out.dx_gate));
      if (!check()) return e;
      auto gate_part = [&](auto kp) {
        constexpr int kPer = decltype(kp)::value;
        hipLaunchKernelGGL((elsaa_k6_bwd_gate_part<VT, kPer>), dim3(g.H, kGateBlocks), dim3(256), 0, stream,
                           bb.da_s, bb.da_lr, bb.dlam, static_cast<const VT *>(in.x_gate), g.B, g.H, g.N, g.DG,
                           bb.gate_part);
      };
      if (g.DG <= 64) gate_part(std::integral_constant<int, 1>{});
      else if (g.DG <= 128) gate_part(std::integral_constant<int, 2>{});
      else if (g.DG <= 256) gate_part(std::integral_constant<int, 4>{});
      else gate_part(std::integral_constant<int, 8>{});
    }
    if (!check()) return e;
    hipLaunchKernelGGL(elsaa_k6_bwd_gate_reduce, dim3(g.H + 1), dim3(256), 0, stream, bb.gate_part, g.H, g.DG,
                       g.variant == ELSAA_VARIANT_FULL ? 1 : 0, out.dgate_w, out.dgate_b, out.dlambda);
    check();
  } else {
    e = launch_fill_zero(out.dx_gate, static_cast<size_t>(nx) * sizeof(VT), stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(elsaa_k6_bwd_zero_f32, dim3(blocks_for(2ll * g.H * g.DG)), dim3(256), 0, stream,
                       out.dgate_w, 2ll * g.H * g.DG);
    hipLaunchKernelGGL(elsaa_k6_bwd_zero_f32, dim3(1), dim3(256), 0, stream, out.dgate_b, 2ll * g.H);
    hipLaunchKernelGGL(elsaa_k6_bwd_zero_f32, dim3(1), dim3(256), 0, stream, out.dlambda, 1ll);
    check();
  }
  return e;
}

}  // namespace

hipError_t launch_backward(const Geometry &g, const BackwardInputs &in, const Buffers &fb,
                           const BackwardBuffers &bb, const BackwardOutputs &out, hipStream_t stream) {
  if (g.bf16)
    return g.D == 64 ? launch_backward_t<uint16_t, 64>(g, in, fb, bb, out, stream)
                     : launch_backward_t<uint16_t, 128>(g, in, fb, bb, out, stream);
  return g.D == 64 ? launch_backward_t<float, 64>(g, in, fb, bb, out, stream)
                   : launch_backward_t<float, 128>(g, in, fb, bb, out, stream);
}

}  // namespace elsaa
