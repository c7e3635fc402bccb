// k4_race_build.hip -- RACE tables: per-bucket value sums and key counts.
//
// The low-rank branch compresses the keys into hash-bucket summaries ("Two
// Efficient Attentions, One Denominator Problem", section "Two efficient
// branches can still be mis-scaled"): for every table l and bucket b,
//   count[l][b] = #{keys j : code_l(k_j) = b},   sum[l][b][:] = sum of v_j over them.
//
// All L tables of one (b, h), restricted to a slice of dc value columns, live in
// LDS (dc is the widest power of two that keeps the slice within 64 KB); one
// workgroup per (b, h, column slice) streams every key once.  Lanes are keys
// (64 per step).  Wave w owns tables l = w, w+4, ...: no two waves ever touch
// the same accumulator, and each wave adds its keys in a fixed order with LDS
// fp32 atomic adds (same-address lanes of one instruction are serialised by
// the LDS in lane order).  Counts are integer atomics, exact in any order.
#include "elsaa_internal.hpp"

namespace elsaa {
namespace {

template <int DC, typename VT, typename CT>
__global__ __launch_bounds__(256) void elsaa_k4_race_build(
    const VT *__restrict__ v, const CT *__restrict__ kcodes, int N, int D, int L, int P,
    float *__restrict__ tsum, float *__restrict__ tcnt) {
  extern __shared__ __align__(16) float tab[];  // [L][nb][DC] then counts [L][nb] (slice 0)
  const int nb = 1 << P;
  const int slice = blockIdx.x;
  const long long bh = blockIdx.y;
  const int c0 = slice * DC;
  const bool do_counts = slice == 0;
  uint32_t *cnt = reinterpret_cast<uint32_t *>(tab + static_cast<size_t>(L) * nb * DC);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tab_words = L * nb * DC + (do_counts ? L * nb : 0);
  for (int i = tid; i < tab_words; i += 256) tab[i] = 0.0f;
  __syncthreads();

  const long long seg = bh * N;
  for (int j0 = 0; j0 < N; j0 += 64) {
    const int j = j0 + lane;
    if (j < N) {
      float val[DC];
      const VT *vr = v + (seg + j) * D + c0;
#pragma unroll
      for (int cc = 0; cc < DC; ++cc) val[cc] = Elem<VT>::load(vr + cc);
      const CT *kc = kcodes + (seg + j) * L;
      for (int l = wave; l < L; l += 4) {
        const int b = kc[l];
        float *dst = tab + (static_cast<size_t>(l) * nb + b) * DC;
#pragma unroll
        for (int cc = 0; cc < DC; ++cc) atomicAdd(dst + cc, val[cc]);
        if (do_counts) atomicAdd(cnt + l * nb + b, 1u);
      }
    }
  }
  __syncthreads();
  float *out = tsum + bh * L * nb * static_cast<long long>(D);
  for (int i = tid; i < L * nb * DC; i += 256) {
    const int cc = i % DC;
    const int lb = i / DC;  // l * nb + b
    out[static_cast<long long>(lb) * D + c0 + cc] = tab[i];
  }
  if (do_counts) {
    float *oc = tcnt + bh * L * nb;
    for (int i = tid; i < L * nb; i += 256) oc[i] = static_cast<float>(cnt[i]);
  }
}

template <int DC, typename VT>
hipError_t launch_dc(const Geometry &g, const void *v, const Buffers &buf, hipStream_t stream) {
  const dim3 grid(g.D / DC, g.BH);
  const size_t lds = (static_cast<size_t>(g.L) * g.nb_race * DC + static_cast<size_t>(g.L) * g.nb_race) * 4;
  const VT *vp = static_cast<const VT *>(v);
  const int32_t *dummy = nullptr;
  (void)dummy;
  if (g.rcb == 1)
    hipLaunchKernelGGL((elsaa_k4_race_build<DC, VT, uint8_t>), grid, dim3(256), lds, stream, vp,
                       static_cast<const uint8_t *>(buf.rcode) + g.rows * g.L, g.N, g.D, g.L, g.P,
                       buf.tsum, buf.tcnt);
  else
    hipLaunchKernelGGL((elsaa_k4_race_build<DC, VT, uint16_t>), grid, dim3(256), lds, stream, vp,
                       static_cast<const uint16_t *>(buf.rcode) + g.rows * g.L, g.N, g.D, g.L, g.P,
                       buf.tsum, buf.tcnt);
  return hipGetLastError();
}

template <typename VT>
hipError_t launch_vt(const Geometry &g, const void *v, const Buffers &buf, hipStream_t stream) {
  switch (g.dc) {
    case 1: return launch_dc<1, VT>(g, v, buf, stream);
    case 2: return launch_dc<2, VT>(g, v, buf, stream);
    case 4: return launch_dc<4, VT>(g, v, buf, stream);
    case 8: return launch_dc<8, VT>(g, v, buf, stream);
    case 16: return launch_dc<16, VT>(g, v, buf, stream);
    case 32: return launch_dc<32, VT>(g, v, buf, stream);
    case 64: return launch_dc<64, VT>(g, v, buf, stream);
    default: return launch_dc<128, VT>(g, v, buf, stream);
  }
}

}  // namespace

hipError_t launch_race_build(const Geometry &g, const void *v, const Buffers &buf,
                             hipStream_t stream) {
  return g.bf16 ? launch_vt<uint16_t>(g, v, buf, stream) : launch_vt<float>(g, v, buf, stream);
}

}  // namespace elsaa
