// k5_fuse.hip -- RACE gather, token-wise gates and the denominator-aware fusion.
//
// Per query i of head h in batch b (original token order):
//   Z_lr  = (1/L) sum_l count_l[code_l(q_i)]        collision-count mass
//   num   = (1/L) sum_l sum_l[code_l(q_i)][:]       low-rank numerator
//   o_lr  = num / Z_lr  (0 where Z_lr = 0)
//   g_s   = sigmoid(<x_gate[b,i,:], W[0,h,:]> + c[0,h]),  g_lr likewise with [1]
//   alpha = Z_s / (Z_s + lambda Z_lr) = 1 / (1 + exp(log(lambda Z_lr) - lse_i)),
//           1 where lambda Z_lr = 0
//   y     = g_s alpha o_s + g_lr o_lr
// ("ELSAA: Efficient Low-Rank and Sparse Attention Approximation for Training
// Transformers", first paragraph: the sparse branch is scaled by its estimated
// attention mass relative to the low-rank branch, then gated; "Two Efficient
// Attentions, One Denominator Problem", sections "Two efficient branches can
// still be mis-scaled" and "The ablation isolates the actual contribution":
// the multiplier acts on the sparse branch only, the gates are independent.)
//
// The RACE-only variant (race_only != 0) outputs y = o_lr: the sparse output,
// its LSE and the gates are neither read nor computed.
//
// Three layouts.  L in {8, 16} (the wide path): 16-byte lane pieces, so a load
// instruction gathers 8 table rows of bfloat16 d = 64; a workgroup serves a
// run of queries of one (b, h) with that (b, h)'s bucket counts staged in LDS
// and the gate weight rows in registers; a query's L codes arrive in one
// vector load, the next step's while the current step is gathered.  Any
// other L: d/4 lanes per query, one code and one row load per table.  In both
// the gate dot products are split over the query's lanes and reduced with xor
// shuffles, and consecutive workgroups run on one XCD, so its L2 holds the
// tables of the few (b, h) it serves.  For bfloat16 d = 64 with 16 tables of
// at most 256 buckets (the LDS path) a workgroup copies its (b, h)'s tables
// into LDS one at a time and reads the query rows there.
#include <type_traits>

#include "elsaa_internal.hpp"

namespace elsaa {
namespace {

// Waves the fuse is spread over (each streams a contiguous run of queries).
#ifndef ELSAA_FUSE_WAVES
#define ELSAA_FUSE_WAVES 65536
#endif
constexpr long long kFuseWaves = ELSAA_FUSE_WAVES;

struct AuxOut {
  float *z_lr, *alpha, *g_s, *g_lr, *o_lr;
  // saved for the backward pass (NULL: not saved): o_lr in the value dtype,
  // and per query the raw count sum z (= L Z_lr), g_s and g_lr
  void *sv_olr;
  float *sv_z, *sv_gs, *sv_glr;
};

// ------------------------------------------------------------- any-L path --
// Any number of tables: d/4 lanes per query, 4 value columns each, one code
// load and one row load per table (clamped loads past L are not added).
template <int D, typename VT, typename CT>
__global__ __launch_bounds__(256) void elsaa_k5_fuse(
    const VT *__restrict__ o_s, const float *__restrict__ lse, const CT *__restrict__ qcodes,
    const VT *__restrict__ tsum, const float *__restrict__ tcnt, const VT *__restrict__ x_gate,
    const float *__restrict__ gate_w, const float *__restrict__ gate_b, int H, int N, int L,
    int P, int DG, float lambda, int race_only, long long total, long long qpw, VT *__restrict__ out,
    AuxOut aux) {
  constexpr int kLPQ = D / 4;      // lanes per query, 4 value columns each
  constexpr int kQPS = 64 / kLPQ;  // queries per wave step
  const int lane = threadIdx.x & 63;
  const int sub = lane % kLPQ;
  const long long wv = xcd_logical_block(blockIdx.x, gridDim.x) * 4 +
                       __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const long long q_begin = wv * qpw;
  const long long q_end = q_begin + qpw < total ? q_begin + qpw : total;
  if (q_begin >= q_end) return;  // whole wave
  const int nb = 1 << P;

  // (b, h, i) of the step's first query, advanced once per step: N is a
  // multiple of 64 (a multiple of the chunk) and runs start at multiples of
  // kQPS, so the queries of a step share (b, h) and no division is needed
  long long bh = q_begin / N;
  int i0 = static_cast<int>(q_begin - bh * N);
  int h = static_cast<int>(bh % H);
  long long b = bh / H;

  for (long long q0 = q_begin; q0 < q_end; q0 += kQPS) {
    const long long qi = q0 + lane / kLPQ;
    const bool valid = qi < q_end;  // always true for these sizes; kept as a guard
    const int i = i0 + lane / kLPQ;
    const VT *ts = tsum + bh * L * nb * static_cast<long long>(D) + sub * 4;
    const float *tc = tcnt + bh * L * nb;

    float osv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float lse_i = 0.0f;
    if (!race_only) {
      Elem<VT>::load4(o_s + qi * D + sub * 4, osv);
      lse_i = lse[qi];
    }
    const VT *xg = x_gate + (b * N + i) * DG;
    const float *w0 = gate_w + static_cast<long long>(h) * DG;
    const float *w1 = gate_w + static_cast<long long>(H + h) * DG;

    f32x4 num = {0.0f, 0.0f, 0.0f, 0.0f};
    float z = 0.0f;
    const CT *qc = qcodes + qi * L;
    for (int l0 = 0; l0 < L; l0 += 8) {
      float t[8][4];
      float cnt[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int l = l0 + e < L ? l0 + e : L - 1;  // clamped: extra rows are loaded, not added
        const long long row = static_cast<long long>(l) * nb + qc[l];
        Elem<VT>::load4(ts + row * D, t[e]);
        cnt[e] = tc[row];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (l0 + e < L) {
#pragma unroll
          for (int k = 0; k < 4; ++k) num[k] += t[e][k];
          if (sub == 0) z += cnt[e];
        }
    }

    float a0 = 0.0f, a1 = 0.0f;
    for (int e = sub; e < DG && !race_only; e += kLPQ) {
      const float x = Elem<VT>::load(xg + e);
      a0 = __builtin_fmaf(x, w0[e], a0);
      a1 = __builtin_fmaf(x, w1[e], a1);
    }
#pragma unroll
    for (int off = kLPQ / 2; off > 0; off >>= 1) {
      a0 += __shfl_xor(a0, off);
      a1 += __shfl_xor(a1, off);
      z += __shfl_xor(z, off);
    }
    const float g_s = __builtin_amdgcn_rcpf(1.0f + __expf(-(a0 + gate_b[h])));
    const float g_lr = __builtin_amdgcn_rcpf(1.0f + __expf(-(a1 + gate_b[H + h])));

    const float z_lr = z / static_cast<float>(L);
    f32x4 o_lr = {0.0f, 0.0f, 0.0f, 0.0f};
    if (z > 0.0f) o_lr = num * __builtin_amdgcn_rcpf(z);  // (num / L) / (z / L)

    const float mass_lr = lambda * z_lr;
    const float alpha = mass_lr > 0.0f ? __builtin_amdgcn_rcpf(1.0f + __expf(__logf(mass_lr) - lse_i)) : 1.0f;

    const float ws = race_only ? 0.0f : g_s * alpha;
    const float wl = race_only ? 1.0f : g_lr;
    if (valid) {
      float yv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) yv[e] = __builtin_fmaf(ws, osv[e], wl * o_lr[e]);
      Elem<VT>::store4(out + qi * D + sub * 4, yv);
      if (aux.o_lr) *reinterpret_cast<f32x4 *>(aux.o_lr + qi * D + sub * 4) = o_lr;
      if (aux.sv_olr) {
        const float lr4[4] = {o_lr[0], o_lr[1], o_lr[2], o_lr[3]};
        Elem<VT>::store4(static_cast<VT *>(aux.sv_olr) + qi * D + sub * 4, lr4);
      }
      if (sub == 0 && aux.sv_z) {
        aux.sv_z[qi] = z;
        aux.sv_gs[qi] = g_s;
        aux.sv_glr[qi] = g_lr;
      }
      if (sub == 0) {
        if (aux.z_lr) aux.z_lr[qi] = z_lr;
        if (!race_only) {
          if (aux.alpha) aux.alpha[qi] = alpha;
          if (aux.g_s) aux.g_s[qi] = g_s;
          if (aux.g_lr) aux.g_lr[qi] = g_lr;
        }
      }
    }
    i0 += kQPS;
    if (i0 == N) {
      i0 = 0;
      ++bh;
      if (++h == H) {
        h = 0;
        ++b;
      }
    }
  }
}

// ---------------------------------------------------------------- wide path --
// L in {8, 16}: 16-byte lane pieces (8 lanes per query for bfloat16 rows of 64
// columns), so one load instruction gathers 8 table rows.  A workgroup serves
// a run of R queries of one (b, h) (see launch_wide for R): the bucket counts
// of that (b, h) are staged in LDS once (L 2^P <= 16384 words) and read
// there, the two gate weight rows are loaded once, and the four waves take
// the run's steps in turn.
template <typename VT, int GE> struct GateIn;  // GE consecutive gate inputs of one lane
// unpack: the lane's GE gate inputs from their raw words (loaded as 16, 8 or
// 4 bytes into the leading words of a u32x4)
template <> struct GateIn<uint16_t, 8> {
  static __device__ __forceinline__ void unpack(const u32x4 &w, float *x) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(w[e] << 16);
      x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  }
};
template <> struct GateIn<uint16_t, 4> {
  static __device__ __forceinline__ void unpack(const u32x4 &w, float *x) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      x[2 * e] = __uint_as_float(w[e] << 16);
      x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  }
};
template <> struct GateIn<float, 4> {
  static __device__ __forceinline__ void unpack(const u32x4 &w, float *x) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(w[e]);
  }
};
template <> struct GateIn<float, 2> {
  static __device__ __forceinline__ void unpack(const u32x4 &w, float *x) {
    x[0] = __uint_as_float(w[0]);
    x[1] = __uint_as_float(w[1]);
  }
};

// One query's lane piece (kCols value columns) once its gate dot products
// a0, a1 and its count sum z are reduced over the query's lanes and its L
// table sums num are complete: the gates, Z_lr, alpha, o_lr and y.  Shared by
// the wide and LDS paths (the same arithmetic, so the same results).
// Reciprocals use v_rcp_f32 (1 ulp).
template <int kCols> struct Piece16 {
  float g_s, g_lr, z_lr, alpha;
  float o_lr[kCols], y[kCols];
};
template <int kCols>
__device__ __forceinline__ Piece16<kCols> fuse_piece(float a0, float a1, float z, const float *num, const float *osv,
                                                     float lse_i, float gb0, float gb1, float lambda, float inv_l,
                                                     int race_only) {
  Piece16<kCols> f;
  f.g_s = __builtin_amdgcn_rcpf(1.0f + __expf(-(a0 + gb0)));
  f.g_lr = __builtin_amdgcn_rcpf(1.0f + __expf(-(a1 + gb1)));
  f.z_lr = z * inv_l;
  const float rz = z > 0.0f ? __builtin_amdgcn_rcpf(z) : 0.0f;  // (num / L) / (z / L); 0 where z = 0
  const float mass_lr = lambda * f.z_lr;
  f.alpha = mass_lr > 0.0f ? __builtin_amdgcn_rcpf(1.0f + __expf(__logf(mass_lr) - lse_i)) : 1.0f;
  const float ws = race_only ? 0.0f : f.g_s * f.alpha;
  const float wl = race_only ? 1.0f : f.g_lr;
#pragma unroll
  for (int k = 0; k < kCols; ++k) {
    f.o_lr[k] = num[k] * rz;
    f.y[k] = __builtin_fmaf(ws, osv[k], wl * f.o_lr[k]);
  }
  return f;
}

// The requested per-stage outputs and the values saved for the backward of
// one query's lane piece (columns sub * kCols ..; per-query values from the
// query's first lane).
template <int kCols, typename VT>
__device__ __forceinline__ void store_piece_aux(const AuxOut &aux, long long qi, int D, int sub, float z,
                                                const Piece16<kCols> &f, int race_only) {
  if (aux.o_lr) {
#pragma unroll
    for (int k = 0; k < kCols; k += 4)
      *reinterpret_cast<f32x4 *>(aux.o_lr + qi * D + sub * kCols + k) =
          f32x4{f.o_lr[k], f.o_lr[k + 1], f.o_lr[k + 2], f.o_lr[k + 3]};
  }
  if (aux.sv_olr) {
#pragma unroll
    for (int k = 0; k < kCols; k += 4)
      Elem<VT>::store4(static_cast<VT *>(aux.sv_olr) + qi * D + sub * kCols + k, f.o_lr + k);
  }
  if (sub == 0 && aux.sv_z) {
    aux.sv_z[qi] = z;
    aux.sv_gs[qi] = f.g_s;
    aux.sv_glr[qi] = f.g_lr;
  }
  if (sub == 0) {
    if (aux.z_lr) aux.z_lr[qi] = f.z_lr;
    if (!race_only) {
      if (aux.alpha) aux.alpha[qi] = f.alpha;
      if (aux.g_s) aux.g_s[qi] = f.g_s;
      if (aux.g_lr) aux.g_lr[qi] = f.g_lr;
    }
  }
}

// With DS = 2 D (rows of 128 bfloat16 columns) a workgroup serves its run
// twice, once per column half: the table rows its waves gather at a time are
// then half of every row (2 MB of a (b, h)'s 16 tables of 2^10 buckets), and
// the workgroups of an XCD, which start together, keep to one half at a time.
template <int D, typename VT, typename CT, int LC, int DS = D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void elsaa_k5_fuse_wide(
    const VT *__restrict__ o_s, const float *__restrict__ lse, const CT *__restrict__ qcodes,
    const VT *__restrict__ tsum, const float *__restrict__ tcnt, const VT *__restrict__ x_gate,
    const float *__restrict__ gate_w, const float *__restrict__ gate_b, int H, int N, int P,
    int DG, float lambda, int race_only, int R, int runs, long long units, VT *__restrict__ out, AuxOut aux) {
  constexpr int kES = static_cast<int>(sizeof(VT));
  constexpr int kCols = 16 / kES;         // value columns per lane
  constexpr int kLPQ = D / kCols;         // lanes per query
  constexpr int kQPS = 64 / kLPQ;         // queries per wave step
  constexpr int kRowBytes = D * kES;      // bytes of a lane group's piece of a row
  constexpr int kRowStride = DS * kES;    // bytes of a whole row
  static_assert(DS == D || DS == 2 * D, "whole rows or column halves");
  constexpr int cb = static_cast<int>(sizeof(CT));
  constexpr int kCW = LC * cb / 4;        // 32-bit words of one query's codes
  constexpr int kGE = 64 / kLPQ;          // gate inputs per lane when d_gate = 64
  constexpr int kCntPer = (LC + kLPQ - 1) / kLPQ;  // counts summed by one lane
  extern __shared__ float cnt_lds[];      // [L][2^P] counts of this (b, h)

  const long long unit = xcd_logical_block(blockIdx.x, gridDim.x);
  if (unit >= units) return;  // whole workgroup
  const long long bh = unit / runs;
  const int i_run = static_cast<int>(unit % runs) * R;
  const int run_len = N - i_run < R ? N - i_run : R;  // the (b, h)'s last run may be shorter
  const int h = static_cast<int>(bh % H);
  const long long b = bh / H;
  const int nb = 1 << P;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sub = lane % kLPQ;

  // bucket counts of this (b, h) into LDS
  {
    const f32x4 *src = reinterpret_cast<const f32x4 *>(tcnt + bh * LC * nb);
    for (int i = tid; i < LC * nb / 4; i += 256) reinterpret_cast<f32x4 *>(cnt_lds)[i] = src[i];
  }
  // gate weights of head h (this lane's kGE columns)
  const bool gate_fast = DG == 64;
  __shared__ float gw_lds[2][64];  // gate weights of head h when d_gate = 64
  if (gate_fast && tid < 128)
    gw_lds[tid >> 6][tid & 63] = gate_w[static_cast<long long>((tid >> 6) * H + h) * DG + (tid & 63)];
  const float gb0 = gate_b[h], gb1 = gate_b[H + h];
  const uint32_t vbase = static_cast<uint32_t>(sub) * 16u;
  const Bf16Adder adder;
  __syncthreads();

  // the four waves take the run's steps in turn (a run is a multiple of 64
  // queries, so of 4 kQPS)
  const int my_steps = run_len / (4 * kQPS);
  auto i_of = [&](int st) { return i_run + (wave + 4 * st) * kQPS; };
  // the streamed tensors of this (b, h) through buffer resources: a scalar
  // base and 32-bit lane offsets keep the per-lane addresses in one register
  const __amdgpu_buffer_rsrc_t qc_rs =
      make_rsrc(qcodes + bh * N * LC, static_cast<uint32_t>(N) * LC * cb);
  const __amdgpu_buffer_rsrc_t lse_rs = make_rsrc(lse + bh * N, static_cast<uint32_t>(N) * 4u);
  const __amdgpu_buffer_rsrc_t xg_rs =
      make_rsrc(x_gate + b * N * DG, static_cast<uint32_t>(N) * DG * kES);
  for (int half = 0; half < DS / D; ++half) {
    // this half's columns of the tables, the sparse output and the output
    const int col0 = half * D;
    const uint32_t cut = static_cast<uint32_t>(col0 * kES);
    const __amdgpu_buffer_rsrc_t ts_rs = make_rsrc(tsum + bh * LC * nb * static_cast<long long>(DS) + col0,
                                                   static_cast<uint32_t>(LC * nb * kRowStride) - cut);
    const __amdgpu_buffer_rsrc_t os_rs =
        make_rsrc(o_s + bh * N * static_cast<long long>(DS) + col0, static_cast<uint32_t>(N) * kRowStride - cut);
    const __amdgpu_buffer_rsrc_t out_rs =
        make_rsrc(out + bh * N * static_cast<long long>(DS) + col0, static_cast<uint32_t>(N) * kRowStride - cut);
    auto load_codes = [&](int i0, uint32_t (&w)[kCW]) {
      const uint32_t off = static_cast<uint32_t>(i0 + lane / kLPQ) * (LC * cb);
      if constexpr (kCW % 4 == 0) {
#pragma unroll
        for (int k = 0; k < kCW / 4; ++k) {
          const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(qc_rs, off, 16 * k, 0));
#pragma unroll
          for (int e = 0; e < 4; ++e) w[4 * k + e] = v[e];
        }
      } else {
        static_assert(kCW == 2, "8 code bytes per query");
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(qc_rs, off, 0, 0);
        w[0] = v[0];
        w[1] = v[1];
      }
    };
    uint32_t cw[kCW];
    load_codes(i_of(0), cw);
    // the streamed inputs of a step (sparse output, its LSE, gate inputs) are
    // requested one step ahead, so their HBM latency overlaps the table gathers
    auto load_stream = [&](int i0, u32x4 &os_raw, float &lse_v, u32x4 &xg_raw) {
      if (race_only) return;  // y = o_lr: no sparse output, LSE or gate inputs
      const uint32_t ii = static_cast<uint32_t>(i0 + lane / kLPQ);
      os_raw = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(os_rs, ii * kRowStride + vbase, 0, 0));
      lse_v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(lse_rs, ii * 4u, 0, 0));
      if (gate_fast) {
        const uint32_t xo = (ii * static_cast<uint32_t>(DG) + static_cast<uint32_t>(sub * kGE)) * kES;
        if constexpr (kGE * kES == 16) {
          xg_raw = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xg_rs, xo, 0, 0));
        } else if constexpr (kGE * kES == 8) {
          const auto t2 = __builtin_amdgcn_raw_buffer_load_b64(xg_rs, xo, 0, 0);
          xg_raw = u32x4{t2[0], t2[1], 0u, 0u};
        } else {
          xg_raw = u32x4{__builtin_amdgcn_raw_buffer_load_b32(xg_rs, xo, 0, 0), 0u, 0u, 0u};
        }
      }
    };
    u32x4 os_next = {0u, 0u, 0u, 0u}, xg_next = {0u, 0u, 0u, 0u};
    float lse_next = 0.0f;
    load_stream(i_of(0), os_next, lse_next, xg_next);

    for (int st = 0; st < my_steps; ++st) {
      const int i = i_of(st) + lane / kLPQ;
      const int i_next = st + 1 < my_steps ? i_of(st + 1) : i_of(st);
      const long long qi = bh * N + i;
      const u32x4 os_raw = os_next, xg_raw = xg_next;
      const float lse_i = lse_next;

      // table rows of the L buckets (offsets relative to table l, whose base
      // goes in the scalar offset)
      u32x4 t[LC];
#pragma unroll
      for (int l = 0; l < LC; ++l) {
        const uint32_t word = cw[l * cb / 4];
        const int byte = l * cb % 4;
        uint32_t off;
        if constexpr (kRowStride == 256) {
          const uint32_t sel = cb == 1 ? (0x0c0c0000u | ((4u + byte) << 8))
                                       : (0x0c000000u | ((5u + byte) << 16) | ((4u + byte) << 8));
          off = __builtin_amdgcn_perm(word, vbase, sel);
        } else {
          const uint32_t c = (word >> (byte * 8)) & (cb == 1 ? 0xffu : 0xffffu);
          off = c * static_cast<uint32_t>(kRowStride) + vbase;
        }
        t[l] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ts_rs, off, l * nb * kRowStride, 0));
      }
      // the next step's streamed inputs
      load_stream(i_next, os_next, lse_next, xg_next);
      // sparse output and gate inputs of this step
      float osv[kCols];
      if constexpr (kES == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          osv[2 * e] = __uint_as_float(os_raw[e] << 16);
          osv[2 * e + 1] = __uint_as_float(os_raw[e] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) osv[e] = __uint_as_float(os_raw[e]);
      }
      const VT *xg = x_gate + (b * N + i) * DG;
      float xv[kGE];
      if (gate_fast) GateIn<VT, kGE>::unpack(xg_raw, xv);

      // counts from LDS: lane sub adds tables sub, sub + kLPQ, ...
      float z = 0.0f;
#pragma unroll
      for (int r = 0; r < kCntPer; ++r) {
        const int l = sub + r * kLPQ;
        if (l < LC) {
          const int widx = l * cb / 4;
          uint32_t wsel = cw[0];
#pragma unroll
          for (int k = 1; k < kCW; ++k) wsel = widx == k ? cw[k] : wsel;
          const uint32_t c = (wsel >> ((l * cb % 4) * 8)) & (cb == 1 ? 0xffu : 0xffffu);
          z += cnt_lds[l * nb + c];
        }
      }
      // next step's codes, in flight while this step finishes
      load_codes(i_next, cw);

      float num[kCols];
#pragma unroll
      for (int k = 0; k < kCols; ++k) num[k] = 0.0f;
#pragma unroll
      for (int l = 0; l < LC; ++l) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (kES == 2) {
            num[2 * e] = adder.lo(num[2 * e], t[l][e]);
            num[2 * e + 1] = adder.hi(num[2 * e + 1], t[l][e]);
          } else {
            num[e] += __uint_as_float(t[l][e]);
          }
        }
      }

      float a0 = 0.0f, a1 = 0.0f;
      if (race_only) {
      } else if (gate_fast) {
#pragma unroll
        for (int e = 0; e < kGE; ++e) {
          a0 = __builtin_fmaf(xv[e], gw_lds[0][sub * kGE + e], a0);
          a1 = __builtin_fmaf(xv[e], gw_lds[1][sub * kGE + e], a1);
        }
      } else {
        for (int e = sub; e < DG; e += kLPQ) {
          const float x = Elem<VT>::load(xg + e);
          a0 = __builtin_fmaf(x, gate_w[static_cast<long long>(h) * DG + e], a0);
          a1 = __builtin_fmaf(x, gate_w[static_cast<long long>(H + h) * DG + e], a1);
        }
      }
#pragma unroll
      for (int off = kLPQ / 2; off > 0; off >>= 1) {
        a0 += __shfl_xor(a0, off);
        a1 += __shfl_xor(a1, off);
        z += __shfl_xor(z, off);
      }
      const Piece16<kCols> f =
          fuse_piece<kCols>(a0, a1, z, num, osv, lse_i, gb0, gb1, lambda, 1.0f / static_cast<float>(LC), race_only);
      float yv[kCols];
#pragma unroll
      for (int k = 0; k < kCols; ++k) yv[k] = f.y[k];
      // The next step's streamed inputs and codes are waited for here, before
      // this step's store: the vector memory counter retires in issue order,
      // so a wait for them after the store would also wait for the store.
      asm volatile("" : "+v"(yv[0]) : "v"(os_next), "v"(xg_next), "v"(lse_next) : "memory");
#pragma unroll
      for (int k = 0; k < kCW; ++k) asm volatile("" : "+v"(yv[0]) : "v"(cw[k]) : "memory");
      const uint32_t yo = static_cast<uint32_t>(i) * kRowStride + vbase;
      if constexpr (kES == 2) {
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3]), pack_bf16x2(yv[4], yv[5]),
                  pack_bf16x2(yv[6], yv[7])},
            out_rs, yo, 0, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{__float_as_uint(yv[0]), __float_as_uint(yv[1]), __float_as_uint(yv[2]), __float_as_uint(yv[3])},
            out_rs, yo, 0, 0);
      }
      store_piece_aux<kCols, VT>(aux, qi, DS, sub + half * kLPQ, z, f, race_only);
    }
  }  // column halves
}

template <int D, typename VT, typename CT, int LC>
void launch_wide(const Geometry &g, const void *x_gate, const float *gate_w, const float *gate_b,
                 const Buffers &buf, const AuxOut &aux, void *out, hipStream_t stream) {
  constexpr int kQPS = 64 / (D / (16 / static_cast<int>(sizeof(VT))));
  static_assert(64 % (4 * kQPS) == 0, "runs of 64 queries hold whole steps of every wave");
  // Runs of R queries (a multiple of 64) of one (b, h).  While four
  // workgroups fit a CU (128 VGPRs a lane, the staged counts small), runs of
  // 512: many short workgroups overlap each other's start and end (runs sized
  // to fill exactly one round measured 128 µs against 122 at text32k).  When
  // the staged counts allow fewer (2^10 buckets: 64 KB), one round of
  // workgroups, each staging its counts once (683 µs against 722 at
  // needle256k); a (b, h)'s last run may then be shorter.
  const size_t lds = static_cast<size_t>(LC) * g.nb_race * 4;
  int per_cu = static_cast<int>((160 * 1024) / (lds + 1024));
  per_cu = per_cu < 1 ? 1 : (per_cu > 4 ? 4 : per_cu);
  long long R = 512, runs;
  if (per_cu == 4) {
    while (R > 64 && (g.N % R != 0)) R /= 2;
    runs = g.N / R;
  } else {
    const long long slots = static_cast<long long>(g.cus) * per_cu;
    runs = slots / g.BH;  // runs per (b, h)
    if (runs < 1) runs = 1;
    R = (g.N + runs - 1) / runs;
    R = (R + 63) / 64 * 64;
    runs = (g.N + R - 1) / R;
  }
  const long long units = static_cast<long long>(g.BH) * runs;
  const long long grid = (units + kXcdCount - 1) / kXcdCount * kXcdCount;
  // rows of 128 bfloat16 columns: in column halves
  constexpr bool kHalves = D == 128 && sizeof(VT) == 2;
  hipLaunchKernelGGL((elsaa_k5_fuse_wide<kHalves ? 64 : D, VT, CT, LC, D>), dim3(static_cast<unsigned>(grid)),
                     dim3(256), lds, stream, static_cast<const VT *>(buf.o_s), buf.lse,
                     static_cast<const CT *>(buf.rcode), static_cast<const VT *>(buf.tsum), buf.tcnt,
                     static_cast<const VT *>(x_gate), gate_w, gate_b, g.H, g.N, g.P, g.DG, g.lambda,
                     g.run_sparse ? 0 : 1, static_cast<int>(R), static_cast<int>(runs), units,
                     static_cast<VT *>(out), aux);
}

template <int D, typename VT, typename CT>
void launch_any(const Geometry &g, const void *x_gate, const float *gate_w, const float *gate_b,
                const Buffers &buf, const AuxOut &aux, void *out, hipStream_t stream) {
  constexpr int kQPS = 64 / (D / 4);
  const long long total = g.rows;
  long long qpw = (total + kFuseWaves - 1) / kFuseWaves;  // each wave streams a run of queries
  qpw = (qpw + kQPS - 1) / kQPS * kQPS;
  const long long waves = (total + qpw - 1) / qpw;
  const long long blocks = ((waves + 3) / 4 + kXcdCount - 1) / kXcdCount * kXcdCount;
  hipLaunchKernelGGL((elsaa_k5_fuse<D, VT, CT>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     stream, static_cast<const VT *>(buf.o_s), buf.lse,
                     static_cast<const CT *>(buf.rcode), static_cast<const VT *>(buf.tsum), buf.tcnt,
                     static_cast<const VT *>(x_gate), gate_w, gate_b, g.H, g.N, g.L, g.P, g.DG,
                     g.lambda, g.run_sparse ? 0 : 1, total, qpw, static_cast<VT *>(out), aux);
}

// ----------------------------------------------------------------- LDS path --
// bfloat16, d = 64, d_gate = 64, 2^P <= 256 and an even L: a workgroup of
// eight waves serves a tile of 512 queries of one (b, h), and that (b, h)'s
// tables pass through LDS one at a time (2^P rows of 128 B: 32 KB at P = 8)
// with their counts, so a query's L table rows are LDS reads instead of
// texture gathers from L2 (in the wide path those are 16 of the 21 vector
// memory instructions of a step at L = 16, and the texture path bounds it).
// Two LDS buffers: table l + 1 is copied from L2 straight into LDS (no
// registers) while table l is read.  The tile's codes are staged once; each
// wave keeps the sums of its 64 queries in registers over the passes, adding
// the tables in order 0, 1, ..., L - 1 as the wide path does (the same fp32
// sums); the sparse output, LSE and gate inputs are then streamed
// kLdsFuseAhead steps ahead of the epilogue.  About 75 KB of LDS: two
// workgroups share a CU.
constexpr int kLdsFuseWaves = 8;
constexpr int kLdsFuseSteps = 8;                                 // 8-query steps per wave
constexpr int kLdsFuseTile = kLdsFuseWaves * kLdsFuseSteps * 8;  // queries per workgroup
constexpr int kLdsFuseAhead = 2;                                 // steps of streamed inputs in flight

// s_waitcnt vmcnt(0) with the other counters left free (gfx9 encoding)
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int LC>
__global__ __launch_bounds__(kLdsFuseWaves * 64) __attribute__((amdgpu_waves_per_eu(4))) void elsaa_k5_fuse_lds(
    const uint16_t *__restrict__ o_s, const float *__restrict__ lse, const uint8_t *__restrict__ qcodes,
    const uint16_t *__restrict__ tsum, const float *__restrict__ tcnt, const uint16_t *__restrict__ x_gate,
    const float *__restrict__ gate_w, const float *__restrict__ gate_b, int H, int N, int P, float lambda,
    int race_only, int tiles, long long units, uint16_t *__restrict__ out, AuxOut aux) {
  constexpr int D = 64, kRowBytes = 128, kCols = 8;
  constexpr int kS = kLdsFuseSteps, kT = kLdsFuseWaves * 64, kA = kLdsFuseAhead;
  static_assert(LC % 2 == 0 && kS % kA == 0, "whole buffer pairs and prefetch slots");
  // two buffers of 2^P rows x 8 pieces and their counts, as separate arrays:
  // a copy in flight into one then provably does not alias reads of the
  // other, and the compiler's wait before those reads is not needed
  __shared__ __align__(16) u32x4 tab0[256 * 8], tab1[256 * 8];
  __shared__ __align__(16) float cnt0[256], cnt1[256];
  __shared__ __align__(16) u32x4 code_lds[kLdsFuseTile * LC / 16];
  __shared__ float gw_lds[2][64];

  const long long unit = xcd_logical_block(blockIdx.x, gridDim.x);
  if (unit >= units) return;  // whole workgroup
  const long long bh = unit / tiles;
  const int i_tile = static_cast<int>(unit % tiles) * kLdsFuseTile;
  const int run_len = N - i_tile < kLdsFuseTile ? N - i_tile : kLdsFuseTile;  // a multiple of 64
  const int h = static_cast<int>(bh % H);
  const long long b = bh / H;
  const int nb = 1 << P;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sub = lane & 7, qs = lane >> 3;
  const bool active = wave * 64 < run_len;  // wave-uniform

  const u32x4 *tsrc = reinterpret_cast<const u32x4 *>(tsum + bh * LC * nb * static_cast<long long>(D));
  const float *csrc = tcnt + bh * LC * nb;
  // table l and its counts into LDS buffer `buf`: wave-instructions of 64
  // lanes x 16 bytes (1 KB of consecutive rows; lane j's piece lands j * 16
  // bytes past the instruction's LDS base), counts 64 lanes x 4 bytes
  auto stage = [&](int l, u32x4 *tab, float *cnt) {
    const u32x4 *src = tsrc + static_cast<long long>(l) * nb * 8;
    const int np = nb * 8;
    for (int c = wave; c * 64 < np; c += kLdsFuseWaves) {
      const int piece = c * 64 + lane;
      if (piece < np) __builtin_amdgcn_global_load_lds(src + piece, tab + c * 64, 16, 0, 0);
    }
    const float *cs = csrc + static_cast<long long>(l) * nb;
    for (int c = wave; c * 64 < nb; c += kLdsFuseWaves) {
      const int k = c * 64 + lane;
      if (k < nb) __builtin_amdgcn_global_load_lds(cs + k, cnt + c * 64, 4, 0, 0);
    }
  };

  // the tile's codes (L bytes a query; the tile starts on a 16-byte
  // boundary since N and the tile are multiples of 64 queries)
  {
    const u32x4 *src = reinterpret_cast<const u32x4 *>(qcodes + (bh * N + i_tile) * LC);
    const int n = run_len * LC / 16;
    for (int k = tid; k < n; k += kT) code_lds[k] = src[k];
  }
  if (tid < 128) gw_lds[tid >> 6][tid & 63] = gate_w[static_cast<long long>((tid >> 6) * H + h) * 64 + (tid & 63)];
  const float gb0 = gate_b[h], gb1 = gate_b[H + h];
  stage(0, tab0, cnt0);

  wait_vm_all();
  __syncthreads();  // codes, gate weights, table 0

  stage(1, tab1, cnt1);

  float num[kS][kCols], z[kS];
#pragma unroll
  for (int s = 0; s < kS; ++s) {
    z[s] = 0.0f;
#pragma unroll
    for (int k = 0; k < kCols; ++k) num[s][k] = 0.0f;
  }
  const Bf16Adder adder;

  // table l from (tab, cnt); then, once every wave is past it, table l + 2
  // into the same buffer
  auto pass = [&](int l, const u32x4 *tab, const float *cnt, u32x4 *tab_w, float *cnt_w) {
    if (active) {
#pragma unroll
      for (int s = 0; s < kS; ++s) {
        const uint32_t c = reinterpret_cast<const uint8_t *>(code_lds)[(wave * 64 + s * 8 + qs) * LC + l];
        const u32x4 r = tab[c * 8 + sub];
        const float cn = cnt[c];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          num[s][2 * e] = adder.lo(num[s][2 * e], r[e]);
          num[s][2 * e + 1] = adder.hi(num[s][2 * e + 1], r[e]);
        }
        z[s] += sub == 0 ? cn : 0.0f;  // one lane of the query counts
        if (s % 4 == 3) __builtin_amdgcn_sched_barrier(0);
      }
    }
    wait_vm_all();    // this thread's copies of table l + 1 have landed
    __syncthreads();  // every wave has read this buffer and copied table l + 1
    if (l + 2 < LC) stage(l + 2, tab_w, cnt_w);
  };
#pragma unroll 1
  for (int l = 0; l < LC; l += 2) {
    pass(l, tab0, cnt0, tab0, cnt0);
    pass(l + 1, tab1, cnt1, tab1, cnt1);
  }
  if (!active) return;  // no barrier follows

  const __amdgpu_buffer_rsrc_t os_rs =
      make_rsrc(o_s + bh * N * static_cast<long long>(D), static_cast<uint32_t>(N) * kRowBytes);
  const __amdgpu_buffer_rsrc_t lse_rs = make_rsrc(lse + bh * N, static_cast<uint32_t>(N) * 4u);
  const __amdgpu_buffer_rsrc_t xg_rs = make_rsrc(x_gate + b * N * 64, static_cast<uint32_t>(N) * kRowBytes);
  const __amdgpu_buffer_rsrc_t out_rs =
      make_rsrc(out + bh * N * static_cast<long long>(D), static_cast<uint32_t>(N) * kRowBytes);
  const uint32_t vbase = static_cast<uint32_t>(sub) * 16u;
  auto q_of = [&](int s) { return i_tile + wave * 64 + s * 8 + qs; };
  u32x4 os_in[kA], xg_in[kA];
  float lse_in[kA];
  auto load_stream = [&](int s, int slot) {
    const uint32_t ii = static_cast<uint32_t>(q_of(s));
    os_in[slot] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(os_rs, ii * kRowBytes + vbase, 0, 0));
    lse_in[slot] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(lse_rs, ii * 4u, 0, 0));
    xg_in[slot] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xg_rs, ii * kRowBytes + vbase, 0, 0));
  };
#pragma unroll
  for (int a = 0; a < kA; ++a) {
    if (race_only) {  // y = o_lr: no sparse output, LSE or gate inputs
      os_in[a] = xg_in[a] = u32x4{0u, 0u, 0u, 0u};
      lse_in[a] = 0.0f;
    } else {
      load_stream(a, a);
    }
  }
#pragma unroll
  for (int s = 0; s < kS; ++s) {
    const int slot = s % kA;
    const u32x4 os_raw = os_in[slot], xg_raw = xg_in[slot];
    const float lse_i = lse_in[slot];
    // the inputs kA steps ahead go out before this step's store, so waiting
    // for them never waits for a store
    if (s + kA < kS && !race_only) load_stream(s + kA, slot);
    const int i = q_of(s);
    const long long qi = bh * N + i;
    float osv[kCols], xv[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      osv[2 * e] = __uint_as_float(os_raw[e] << 16);
      osv[2 * e + 1] = __uint_as_float(os_raw[e] & 0xffff0000u);
    }
    GateIn<uint16_t, 8>::unpack(xg_raw, xv);
    float a0 = 0.0f, a1 = 0.0f, zz = z[s];
    if (!race_only) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a0 = __builtin_fmaf(xv[e], gw_lds[0][sub * 8 + e], a0);
        a1 = __builtin_fmaf(xv[e], gw_lds[1][sub * 8 + e], a1);
      }
    }
#pragma unroll
    for (int off = 4; off > 0; off >>= 1) {
      a0 += __shfl_xor(a0, off);
      a1 += __shfl_xor(a1, off);
      zz += __shfl_xor(zz, off);
    }
    const Piece16<kCols> f = fuse_piece<kCols>(a0, a1, zz, num[s], osv, lse_i, gb0, gb1, lambda,
                                               1.0f / static_cast<float>(LC), race_only);
    __builtin_amdgcn_raw_buffer_store_b128(
        u32x4{pack_bf16x2(f.y[0], f.y[1]), pack_bf16x2(f.y[2], f.y[3]), pack_bf16x2(f.y[4], f.y[5]),
              pack_bf16x2(f.y[6], f.y[7])},
        out_rs, static_cast<uint32_t>(i) * kRowBytes + vbase, 0, 0);
    store_piece_aux<kCols, uint16_t>(aux, qi, D, sub, zz, f, race_only);
    __builtin_amdgcn_sched_barrier(0);  // one step at a time (the sums hold the registers)
  }
}

template <int LC>
void launch_lds(const Geometry &g, const void *x_gate, const float *gate_w, const float *gate_b,
                const Buffers &buf, const AuxOut &aux, void *out, hipStream_t stream) {
  const long long tiles = (g.N + kLdsFuseTile - 1) / kLdsFuseTile;
  const long long units = static_cast<long long>(g.BH) * tiles;
  const long long grid = (units + kXcdCount - 1) / kXcdCount * kXcdCount;
  hipLaunchKernelGGL((elsaa_k5_fuse_lds<LC>), dim3(static_cast<unsigned>(grid)), dim3(kLdsFuseWaves * 64), 0,
                     stream, static_cast<const uint16_t *>(buf.o_s), buf.lse,
                     static_cast<const uint8_t *>(buf.rcode), static_cast<const uint16_t *>(buf.tsum), buf.tcnt,
                     static_cast<const uint16_t *>(x_gate), gate_w, gate_b, g.H, g.N, g.P, g.lambda,
                     g.run_sparse ? 0 : 1, static_cast<int>(tiles), units, static_cast<uint16_t *>(out), aux);
}

// the LDS path applies: bfloat16 d = 64 rows, one code byte (2^P <= 256 rows
// a table), d_gate = 64, and 16 tables.  With 8 tables its table passes save
// less than the epilogue loses by streaming its inputs only after them: the
// step was slower (vision16k 0.436 against 0.431 ms median) and the wide path
// is kept; at 16 tables the step gains (text32k 0.428 against 0.432 ms).
bool fuse_lds_applies(const Geometry &g) {
  return g.bf16 && g.D == 64 && g.rcb == 1 && g.nb_race <= 256 && g.DG == 64 && g.L == 16;
}

template <int D, typename VT>
hipError_t launch_d(const Geometry &g, const void *x_gate, const float *gate_w, const float *gate_b,
                    const Buffers &buf, const AuxOut &aux, void *out, hipStream_t stream) {
  if constexpr (D == 64 && std::is_same_v<VT, uint16_t>) {
    if (fuse_lds_applies(g)) {
      launch_lds<16>(g, x_gate, gate_w, gate_b, buf, aux, out, stream);
      return hipGetLastError();
    }
  }
  if (g.rcb == 1) {
    if (g.L == 16) launch_wide<D, VT, uint8_t, 16>(g, x_gate, gate_w, gate_b, buf, aux, out, stream);
    else if (g.L == 8) launch_wide<D, VT, uint8_t, 8>(g, x_gate, gate_w, gate_b, buf, aux, out, stream);
    else launch_any<D, VT, uint8_t>(g, x_gate, gate_w, gate_b, buf, aux, out, stream);
  } else {
    if (g.L == 16) launch_wide<D, VT, uint16_t, 16>(g, x_gate, gate_w, gate_b, buf, aux, out, stream);
    else if (g.L == 8) launch_wide<D, VT, uint16_t, 8>(g, x_gate, gate_w, gate_b, buf, aux, out, stream);
    else launch_any<D, VT, uint16_t>(g, x_gate, gate_w, gate_b, buf, aux, out, stream);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fuse(const Geometry &g, const void *x_gate, const float *gate_w,
                       const float *gate_b, const Buffers &buf, const elsaa_aux_t *aux,
                       void *out, hipStream_t stream) {
  AuxOut a = {nullptr, nullptr, nullptr, nullptr, nullptr, buf.sv_olr, buf.sv_z, buf.sv_gs, buf.sv_glr};
  if (aux) {
    a.z_lr = aux->z_lr;
    a.alpha = aux->alpha;
    a.g_s = aux->g_s;
    a.g_lr = aux->g_lr;
    a.o_lr = aux->o_lowrank;
  }
  if (g.bf16)
    return g.D == 64 ? launch_d<64, uint16_t>(g, x_gate, gate_w, gate_b, buf, a, out, stream)
                     : launch_d<128, uint16_t>(g, x_gate, gate_w, gate_b, buf, a, out, stream);
  return g.D == 64 ? launch_d<64, float>(g, x_gate, gate_w, gate_b, buf, a, out, stream)
                   : launch_d<128, float>(g, x_gate, gate_w, gate_b, buf, a, out, stream);
}

}  // namespace elsaa
