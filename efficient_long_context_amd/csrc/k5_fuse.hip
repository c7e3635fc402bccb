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
// Layout: d/4 lanes per query, 4 value columns per lane (16-byte table reads),
// the gate dot products split over the same lanes and reduced with xor
// shuffles inside the query's lane group.  Each wave streams a contiguous run
// of queries, loading the next step's RACE codes while the current step's
// table rows are gathered; consecutive waves run on one XCD, so its L2 holds
// the tables of the few (b, h) it serves.
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
};

// LC = number of RACE tables when it is 8 or 16 (codes of a query arrive in
// one 16- or 32-byte load and every lane holds all of them); LC = 0 takes any
// L with one code load per table.
template <int D, typename VT, typename CT, int LC>
__global__ __launch_bounds__(256) void elsaa_k5_fuse(
    const VT *__restrict__ o_s, const float *__restrict__ lse, const CT *__restrict__ qcodes,
    const VT *__restrict__ tsum, const float *__restrict__ tcnt, const VT *__restrict__ x_gate,
    const float *__restrict__ gate_w, const float *__restrict__ gate_b, int H, int N, int L_rt,
    int P, int DG, float lambda, long long total, long long qpw, VT *__restrict__ out, AuxOut aux) {
  constexpr int kLPQ = D / 4;      // lanes per query, 4 value columns each
  constexpr int kQPS = 64 / kLPQ;  // queries per wave step
  constexpr int kCodeWords = LC * static_cast<int>(sizeof(CT)) / 4;  // 32-bit words of codes
  const int L = LC ? LC : L_rt;
  const int lane = threadIdx.x & 63;
  const int sub = lane % kLPQ;
  // readfirstlane: the wave index is uniform, so everything derived from it
  // (query run, (b, h), table bases) stays in scalar registers
  const long long wv = xcd_logical_block(blockIdx.x, gridDim.x) * 4 +
                       __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const long long q_begin = wv * qpw;
  const long long q_end = q_begin + qpw < total ? q_begin + qpw : total;
  if (q_begin >= q_end) return;  // whole wave
  const int nb = 1 << P;

  // all LC codes of the lane's query as kCodeWords 32-bit words (8, 16 or 32
  // bytes; clamped queries are computed, not stored)
  constexpr int kCW = kCodeWords > 0 ? kCodeWords : 1;
  uint32_t cw[kCW];
  auto load_codes = [&](long long q0, uint32_t (&w)[kCW]) {
    if constexpr (LC > 0) {
      long long q = q0 + lane / kLPQ;
      q = q < q_end ? q : q_end - 1;
      const CT *src = qcodes + q * LC;
      if constexpr (kCodeWords % 4 == 0) {
#pragma unroll
        for (int k = 0; k < kCodeWords / 4; ++k) {
          const u32x4 v = reinterpret_cast<const u32x4 *>(src)[k];
#pragma unroll
          for (int e = 0; e < 4; ++e) w[4 * k + e] = v[e];
        }
      } else {
        static_assert(kCodeWords == 2, "8 code bytes per query");
        const uint2 v = *reinterpret_cast<const uint2 *>(src);
        w[0] = v.x;
        w[1] = v.y;
      }
    }
  };
  auto code_of = [&](int l) -> int {  // l known at compile time after unrolling
    constexpr int cb = static_cast<int>(sizeof(CT));
    const uint32_t word = cw[l * cb / 4];
    return static_cast<int>((word >> ((l * cb % 4) * 8)) & (cb == 1 ? 0xffu : 0xffffu));
  };
  load_codes(q_begin, cw);

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
    // tables of this (b, h) through buffer resources: 32-bit per-lane offsets
    constexpr int kES = static_cast<int>(sizeof(VT));  // table element bytes
    const __amdgpu_buffer_rsrc_t ts_rs =
        make_rsrc(tsum + bh * L * nb * static_cast<long long>(D), static_cast<uint32_t>(L * nb * D * kES));
    const __amdgpu_buffer_rsrc_t tc_rs = make_rsrc(tcnt + bh * L * nb, static_cast<uint32_t>(L * nb * 4));
    const VT *ts = tsum + bh * L * nb * static_cast<long long>(D) + sub * 4;
    const float *tc = tcnt + bh * L * nb;

    // the sparse output, its LSE and the gate inputs load while the tables are gathered
    float osv[4];
    Elem<VT>::load4(o_s + qi * D + sub * 4, osv);
    const float lse_i = lse[qi];
    const VT *xg = x_gate + (b * N + i) * DG;
    const float *w0 = gate_w + static_cast<long long>(h) * DG;
    const float *w1 = gate_w + static_cast<long long>(H + h) * DG;
    const bool gate_fast = DG == 4 * kLPQ;
    float xv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    f32x4 wa = {0.0f, 0.0f, 0.0f, 0.0f}, wb = {0.0f, 0.0f, 0.0f, 0.0f};
    if (gate_fast) {
      Elem<VT>::load4(xg + sub * 4, xv);
      wa = *reinterpret_cast<const f32x4 *>(w0 + sub * 4);
      wb = *reinterpret_cast<const f32x4 *>(w1 + sub * 4);
    }

    f32x4 num = {0.0f, 0.0f, 0.0f, 0.0f};
    float z = 0.0f;
    if constexpr (LC > 0) {
      // lane sub < LC adds the count of table sub; the group sums them below
      constexpr int cb = static_cast<int>(sizeof(CT));
      if (sub < LC) {
        const int widx = sub * cb / 4;
        uint32_t wsel = cw[0];
#pragma unroll
        for (int k = 1; k < kCW; ++k) wsel = widx == k ? cw[k] : wsel;
        const uint32_t c = (wsel >> ((sub * cb % 4) * 8)) & (cb == 1 ? 0xffu : 0xffffu);
        z = __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(tc_rs, (static_cast<uint32_t>(sub * nb) + c) * 4u, 0, 0));
      }
      // byte offset of the lane's 4-column piece of row code_l of table l,
      // relative to the table: code * d * es + 4 es sub.  For 256-byte rows
      // (binary32, d = 64) one byte permute places the code above the lane
      // offset.
      const uint32_t vbase = static_cast<uint32_t>(sub) * 4u * kES;
      auto row_off = [&](int l) -> uint32_t {
        const uint32_t word = cw[l * cb / 4];
        const int byte = l * cb % 4;
        if constexpr (D * kES == 256) {
          const uint32_t sel = cb == 1 ? (0x0c0c0000u | ((4u + byte) << 8))
                                       : (0x0c000000u | ((5u + byte) << 16) | ((4u + byte) << 8));
          return __builtin_amdgcn_perm(word, vbase, sel);
        } else {
          const uint32_t c = (word >> (byte * 8)) & (cb == 1 ? 0xffu : 0xffffu);
          return c * static_cast<uint32_t>(D * kES) + vbase;
        }
      };
      using Piece = typename std::conditional<kES == 2, uint2, f32x4>::type;
      Piece t[LC];
#pragma unroll
      for (int l = 0; l < LC; ++l) {
        if constexpr (kES == 2)
          t[l] = __builtin_bit_cast(
              uint2, __builtin_amdgcn_raw_buffer_load_b64(ts_rs, row_off(l), l * nb * (D * kES), 0));
        else
          t[l] = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(ts_rs, row_off(l), l * nb * (D * kES), 0));
      }
      long long qn = q0 + kQPS < q_end ? q0 + kQPS : q0;
      load_codes(qn, cw);  // next step's codes, in flight while this step finishes
#pragma unroll
      for (int l = 0; l < LC; ++l) {
        if constexpr (kES == 2) {
          num[0] += __uint_as_float(t[l].x << 16);
          num[1] += __uint_as_float(t[l].x & 0xffff0000u);
          num[2] += __uint_as_float(t[l].y << 16);
          num[3] += __uint_as_float(t[l].y & 0xffff0000u);
        } else {
          num += t[l];
        }
      }
    } else {
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
    }

    // gates: with d_gate = 4 x (lanes per query) each lane takes 4 consecutive
    // inputs in one load; any other width takes the strided loop
    float a0 = 0.0f, a1 = 0.0f;
    if (gate_fast) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a0 = __builtin_fmaf(xv[e], wa[e], a0);
        a1 = __builtin_fmaf(xv[e], wb[e], a1);
      }
    } else {
      for (int e = sub; e < DG; e += kLPQ) {
        const float x = Elem<VT>::load(xg + e);
        a0 = __builtin_fmaf(x, w0[e], a0);
        a1 = __builtin_fmaf(x, w1[e], a1);
      }
    }
#pragma unroll
    for (int off = kLPQ / 2; off > 0; off >>= 1) {
      a0 += __shfl_xor(a0, off);
      a1 += __shfl_xor(a1, off);
      z += __shfl_xor(z, off);
    }
    // reciprocals with v_rcp_f32 (1 ulp)
    const float g_s = __builtin_amdgcn_rcpf(1.0f + __expf(-(a0 + gate_b[h])));
    const float g_lr = __builtin_amdgcn_rcpf(1.0f + __expf(-(a1 + gate_b[H + h])));

    const float z_lr = z * (1.0f / static_cast<float>(L));
    f32x4 o_lr = {0.0f, 0.0f, 0.0f, 0.0f};
    if (z > 0.0f) o_lr = num * __builtin_amdgcn_rcpf(z);  // (num / L) / (z / L)

    const float mass_lr = lambda * z_lr;
    const float alpha = mass_lr > 0.0f ? __builtin_amdgcn_rcpf(1.0f + __expf(__logf(mass_lr) - lse_i)) : 1.0f;

    const float ws = g_s * alpha;
    if (valid) {
      float yv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) yv[e] = __builtin_fmaf(ws, osv[e], g_lr * o_lr[e]);
      Elem<VT>::store4(out + qi * D + sub * 4, yv);
      if (aux.o_lr) *reinterpret_cast<f32x4 *>(aux.o_lr + qi * D + sub * 4) = o_lr;
      if (sub == 0) {
        if (aux.z_lr) aux.z_lr[qi] = z_lr;
        if (aux.alpha) aux.alpha[qi] = alpha;
        if (aux.g_s) aux.g_s[qi] = g_s;
        if (aux.g_lr) aux.g_lr[qi] = g_lr;
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

template <int D, typename VT, typename CT, int LC>
void launch_l(const Geometry &g, const void *x_gate, const float *gate_w, const float *gate_b,
              const Buffers &buf, const AuxOut &aux, void *out, hipStream_t stream) {
  constexpr int kQPS = 64 / (D / 4);
  const long long total = g.rows;
  long long qpw = (total + kFuseWaves - 1) / kFuseWaves;  // each wave streams a run of queries
  qpw = (qpw + kQPS - 1) / kQPS * kQPS;
  const long long waves = (total + qpw - 1) / qpw;
  const long long blocks = ((waves + 3) / 4 + kXcdCount - 1) / kXcdCount * kXcdCount;
  hipLaunchKernelGGL((elsaa_k5_fuse<D, VT, CT, LC>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     stream, static_cast<const VT *>(buf.o_s), buf.lse,
                     static_cast<const CT *>(buf.rcode), static_cast<const VT *>(buf.tsum), buf.tcnt,
                     static_cast<const VT *>(x_gate), gate_w, gate_b, g.H, g.N, g.L, g.P, g.DG,
                     g.lambda, total, qpw, static_cast<VT *>(out), aux);
}

template <int D, typename VT>
hipError_t launch_d(const Geometry &g, const void *x_gate, const float *gate_w, const float *gate_b,
                    const Buffers &buf, const AuxOut &aux, void *out, hipStream_t stream) {
  if (g.rcb == 1) {
    if (g.L == 16) launch_l<D, VT, uint8_t, 16>(g, x_gate, gate_w, gate_b, buf, aux, out, stream);
    else if (g.L == 8) launch_l<D, VT, uint8_t, 8>(g, x_gate, gate_w, gate_b, buf, aux, out, stream);
    else launch_l<D, VT, uint8_t, 0>(g, x_gate, gate_w, gate_b, buf, aux, out, stream);
  } else {
    if (g.L == 16) launch_l<D, VT, uint16_t, 16>(g, x_gate, gate_w, gate_b, buf, aux, out, stream);
    else if (g.L == 8) launch_l<D, VT, uint16_t, 8>(g, x_gate, gate_w, gate_b, buf, aux, out, stream);
    else launch_l<D, VT, uint16_t, 0>(g, x_gate, gate_w, gate_b, buf, aux, out, stream);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fuse(const Geometry &g, const void *x_gate, const float *gate_w,
                       const float *gate_b, const Buffers &buf, const elsaa_aux_t *aux,
                       void *out, hipStream_t stream) {
  AuxOut a = {nullptr, nullptr, nullptr, nullptr, nullptr};
  if (aux) a = {aux->z_lr, aux->alpha, aux->g_s, aux->g_lr, aux->o_lowrank};
  if (g.bf16)
    return g.D == 64 ? launch_d<64, uint16_t>(g, x_gate, gate_w, gate_b, buf, a, out, stream)
                     : launch_d<128, uint16_t>(g, x_gate, gate_w, gate_b, buf, a, out, stream);
  return g.D == 64 ? launch_d<64, float>(g, x_gate, gate_w, gate_b, buf, a, out, stream)
                   : launch_d<128, float>(g, x_gate, gate_w, gate_b, buf, a, out, stream);
}

}  // namespace elsaa
