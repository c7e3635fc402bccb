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
// shuffles inside the query's lane group.
#include <type_traits>

#include "elsaa_internal.hpp"

namespace elsaa {
namespace {

struct AuxOut {
  float *z_lr, *alpha, *g_s, *g_lr, *o_lr;
};

template <int D, typename VT, typename CT>
__global__ __launch_bounds__(256) void elsaa_k5_fuse(
    const VT *__restrict__ o_s, const float *__restrict__ lse, const CT *__restrict__ qcodes,
    const float *__restrict__ tsum, const float *__restrict__ tcnt, const VT *__restrict__ x_gate,
    const float *__restrict__ gate_w, const float *__restrict__ gate_b, int H, int N, int L,
    int P, int DG, float lambda, long long total, VT *__restrict__ out, AuxOut aux) {
  constexpr int kLanesPerQuery = D / 4;
  constexpr int kQueriesPerBlock = 256 / kLanesPerQuery;
  const int sub = threadIdx.x % kLanesPerQuery;
  const long long gq = static_cast<long long>(blockIdx.x) * kQueriesPerBlock + threadIdx.x / kLanesPerQuery;
  const bool valid = gq < total;
  const long long qi = valid ? gq : 0;
  const long long bh = qi / N;
  const int i = static_cast<int>(qi % N);
  const int h = static_cast<int>(bh % H);
  const long long b = bh / H;
  const int nb = 1 << P;

  // Every independent load is issued before the first use: RACE rows (in
  // groups of 16 tables), the sparse output, its LSE and the gate inputs.
  // Summing as loads arrive would serialise their memory latencies.
  const CT *qc = qcodes + qi * L;
  const float *ts = tsum + bh * L * nb * static_cast<long long>(D) + sub * 4;
  const float *tc = tcnt + bh * L * nb;
  const VT *os = o_s + qi * D + sub * 4;
  float osv[4];
  Elem<VT>::load4(os, osv);
  const float lse_i = lse[qi];

  float z = 0.0f;
  f32x4 num = {0.0f, 0.0f, 0.0f, 0.0f};
  auto gather = [&](auto group, int l0) {
    constexpr int G = decltype(group)::value;
    long long row[G];
#pragma unroll
    for (int e = 0; e < G; ++e) {
      const int l = l0 + e < L ? l0 + e : L - 1;  // clamped: extra rows are loaded, not added
      row[e] = static_cast<long long>(l) * nb + qc[l];
    }
    f32x4 t[G];
    float c[G];
#pragma unroll
    for (int e = 0; e < G; ++e) {
      t[e] = *reinterpret_cast<const f32x4 *>(ts + row[e] * D);
      c[e] = tc[row[e]];
    }
#pragma unroll
    for (int e = 0; e < G; ++e) {
      if (l0 + e < L) {
        num += t[e];
        z += c[e];
      }
    }
  };
  // no loop for L <= 16: keeps the compiler from draining loads at a loop header
  if (L <= 4) gather(std::integral_constant<int, 4>(), 0);
  else if (L <= 8) gather(std::integral_constant<int, 8>(), 0);
  else if (L <= 16) gather(std::integral_constant<int, 16>(), 0);
  else for (int l0 = 0; l0 < L; l0 += 16) gather(std::integral_constant<int, 16>(), l0);

  // gates: with d_gate = 4 x (lanes per query) each lane takes 4 consecutive
  // inputs in one load; any other width takes the strided loop
  const VT *xg = x_gate + (b * N + i) * DG;
  const float *w0 = gate_w + static_cast<long long>(h) * DG;
  const float *w1 = gate_w + static_cast<long long>(H + h) * DG;
  float a0 = 0.0f, a1 = 0.0f;
  if (DG == 4 * kLanesPerQuery) {
    float xv[4];
    Elem<VT>::load4(xg + sub * 4, xv);
    const f32x4 wa = *reinterpret_cast<const f32x4 *>(w0 + sub * 4);
    const f32x4 wb = *reinterpret_cast<const f32x4 *>(w1 + sub * 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a0 = __builtin_fmaf(xv[e], wa[e], a0);
      a1 = __builtin_fmaf(xv[e], wb[e], a1);
    }
  } else {
    for (int e = sub; e < DG; e += kLanesPerQuery) {
      const float xv = Elem<VT>::load(xg + e);
      a0 = __builtin_fmaf(xv, w0[e], a0);
      a1 = __builtin_fmaf(xv, w1[e], a1);
    }
  }
#pragma unroll
  for (int off = kLanesPerQuery / 2; off > 0; off >>= 1) {
    a0 += __shfl_xor(a0, off);
    a1 += __shfl_xor(a1, off);
  }
  const float g_s = 1.0f / (1.0f + __expf(-(a0 + gate_b[h])));
  const float g_lr = 1.0f / (1.0f + __expf(-(a1 + gate_b[H + h])));

  const float z_lr = z / static_cast<float>(L);
  f32x4 o_lr = {0.0f, 0.0f, 0.0f, 0.0f};
  if (z > 0.0f) o_lr = num * (1.0f / z);  // (num / L) / (z / L)

  const float mass_lr = lambda * z_lr;
  const float alpha = mass_lr > 0.0f ? 1.0f / (1.0f + __expf(__logf(mass_lr) - lse_i)) : 1.0f;

  VT *dst = out + qi * D + sub * 4;
  const float ws = g_s * alpha;
  if (valid) {
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e] = Elem<VT>::store_val(__builtin_fmaf(ws, osv[e], g_lr * o_lr[e]));
    if (aux.o_lr) *reinterpret_cast<f32x4 *>(aux.o_lr + qi * D + sub * 4) = o_lr;
    if (sub == 0) {
      if (aux.z_lr) aux.z_lr[qi] = z_lr;
      if (aux.alpha) aux.alpha[qi] = alpha;
      if (aux.g_s) aux.g_s[qi] = g_s;
      if (aux.g_lr) aux.g_lr[qi] = g_lr;
    }
  }
}

template <int D, typename VT>
hipError_t launch_d(const Geometry &g, const void *x_gate, const float *gate_w, const float *gate_b,
                    const Buffers &buf, const AuxOut &aux, void *out, hipStream_t stream) {
  constexpr int kQueriesPerBlock = 256 / (D / 4);
  const long long total = g.rows;
  const dim3 grid(static_cast<unsigned>((total + kQueriesPerBlock - 1) / kQueriesPerBlock));
  const VT *os = static_cast<const VT *>(buf.o_s);
  const VT *xg = static_cast<const VT *>(x_gate);
  VT *o = static_cast<VT *>(out);
  if (g.rcb == 1)
    hipLaunchKernelGGL((elsaa_k5_fuse<D, VT, uint8_t>), grid, dim3(256), 0, stream, os, buf.lse,
                       static_cast<const uint8_t *>(buf.rcode), buf.tsum, buf.tcnt, xg, gate_w,
                       gate_b, g.H, g.N, g.L, g.P, g.DG, g.lambda, total, o, aux);
  else
    hipLaunchKernelGGL((elsaa_k5_fuse<D, VT, uint16_t>), grid, dim3(256), 0, stream, os, buf.lse,
                       static_cast<const uint16_t *>(buf.rcode), buf.tsum, buf.tcnt, xg, gate_w,
                       gate_b, g.H, g.N, g.L, g.P, g.DG, g.lambda, total, o, aux);
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
