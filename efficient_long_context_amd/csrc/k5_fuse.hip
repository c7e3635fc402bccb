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
// Two layouts.  L in {8, 16} (the wide path): 16-byte lane pieces, so a load
// instruction gathers 8 table rows of bfloat16 d = 64; a workgroup serves a
// run of queries of one (b, h) with that (b, h)'s bucket counts staged in LDS
// and the gate weight rows in registers; a query's L codes arrive in one
// vector load, the next step's while the current step is gathered.  Any
// other L: d/4 lanes per query, one code and one row load per table.  In both
// the gate dot products are split over the query's lanes and reduced with xor
// shuffles, and consecutive workgroups run on one XCD, so its L2 holds the
// tables of the few (b, h) it serves.
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

// ------------------------------------------------------------- any-L path --
// Any number of tables: d/4 lanes per query, 4 value columns each, one code
// load and one row load per table (clamped loads past L are not added).
template <int D, typename VT, typename CT>
__global__ __launch_bounds__(256) void elsaa_k5_fuse(
    const VT *__restrict__ o_s, const float *__restrict__ lse, const CT *__restrict__ qcodes,
    const VT *__restrict__ tsum, const float *__restrict__ tcnt, const VT *__restrict__ x_gate,
    const float *__restrict__ gate_w, const float *__restrict__ gate_b, int H, int N, int L,
    int P, int DG, float lambda, long long total, long long qpw, VT *__restrict__ out, AuxOut aux) {
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

    float osv[4];
    Elem<VT>::load4(o_s + qi * D + sub * 4, osv);
    const float lse_i = lse[qi];
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
    for (int e = sub; e < DG; e += kLPQ) {
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

// ---------------------------------------------------------------- wide path --
// L in {8, 16}: 16-byte lane pieces (8 lanes per query for bfloat16 rows of 64
// columns), so one load instruction gathers 8 table rows.  A workgroup serves
// a run of R queries of one (b, h): the bucket counts of that (b, h) are staged
// in LDS once (L 2^P <= 16384 words) and read there, the two gate weight rows
// are loaded once, and each wave streams R/4 queries.
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

template <int D, typename VT, typename CT, int LC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void elsaa_k5_fuse_wide(
    const VT *__restrict__ o_s, const float *__restrict__ lse, const CT *__restrict__ qcodes,
    const VT *__restrict__ tsum, const float *__restrict__ tcnt, const VT *__restrict__ x_gate,
    const float *__restrict__ gate_w, const float *__restrict__ gate_b, int H, int N, int P,
    int DG, float lambda, int R, long long units, VT *__restrict__ out, AuxOut aux) {
  constexpr int kES = static_cast<int>(sizeof(VT));
  constexpr int kCols = 16 / kES;         // value columns per lane
  constexpr int kLPQ = D / kCols;         // lanes per query
  constexpr int kQPS = 64 / kLPQ;         // queries per wave step
  constexpr int kRowBytes = D * kES;
  constexpr int cb = static_cast<int>(sizeof(CT));
  constexpr int kCW = LC * cb / 4;        // 32-bit words of one query's codes
  constexpr int kGE = 64 / kLPQ;          // gate inputs per lane when d_gate = 64
  constexpr int kCntPer = (LC + kLPQ - 1) / kLPQ;  // counts summed by one lane
  extern __shared__ float cnt_lds[];      // [L][2^P] counts of this (b, h)

  const long long unit = xcd_logical_block(blockIdx.x, gridDim.x);
  if (unit >= units) return;  // whole workgroup
  const int runs = N / R;
  const long long bh = unit / runs;
  const int i_run = static_cast<int>(unit % runs) * R;
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
  const __amdgpu_buffer_rsrc_t ts_rs =
      make_rsrc(tsum + bh * LC * nb * static_cast<long long>(D), static_cast<uint32_t>(LC * nb * kRowBytes));
  const uint32_t vbase = static_cast<uint32_t>(sub) * 16u;
  const Bf16Adder adder;
  __syncthreads();

  const int per_wave = R / 4;
  const int i_begin = i_run + wave * per_wave;
  // the streamed tensors of this (b, h) through buffer resources: a scalar
  // base and 32-bit lane offsets keep the per-lane addresses in one register
  const __amdgpu_buffer_rsrc_t qc_rs =
      make_rsrc(qcodes + bh * N * LC, static_cast<uint32_t>(N) * LC * cb);
  const __amdgpu_buffer_rsrc_t os_rs =
      make_rsrc(o_s + bh * N * static_cast<long long>(D), static_cast<uint32_t>(N) * kRowBytes);
  const __amdgpu_buffer_rsrc_t lse_rs = make_rsrc(lse + bh * N, static_cast<uint32_t>(N) * 4u);
  const __amdgpu_buffer_rsrc_t xg_rs =
      make_rsrc(x_gate + b * N * DG, static_cast<uint32_t>(N) * DG * kES);
  const __amdgpu_buffer_rsrc_t out_rs =
      make_rsrc(out + bh * N * static_cast<long long>(D), static_cast<uint32_t>(N) * kRowBytes);
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
  load_codes(i_begin, cw);
  // the streamed inputs of a step (sparse output, its LSE, gate inputs) are
  // requested one step ahead, so their HBM latency overlaps the table gathers
  auto load_stream = [&](int i0, u32x4 &os_raw, float &lse_v, u32x4 &xg_raw) {
    const uint32_t ii = static_cast<uint32_t>(i0 + lane / kLPQ);
    os_raw = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(os_rs, ii * kRowBytes + vbase, 0, 0));
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
  load_stream(i_begin, os_next, lse_next, xg_next);

  for (int step = 0; step < per_wave; step += kQPS) {
    const int i = i_begin + step + lane / kLPQ;
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
      if constexpr (kRowBytes == 256) {
        const uint32_t sel = cb == 1 ? (0x0c0c0000u | ((4u + byte) << 8))
                                     : (0x0c000000u | ((5u + byte) << 16) | ((4u + byte) << 8));
        off = __builtin_amdgcn_perm(word, vbase, sel);
      } else {
        const uint32_t c = (word >> (byte * 8)) & (cb == 1 ? 0xffu : 0xffffu);
        off = c * static_cast<uint32_t>(kRowBytes) + vbase;
      }
      t[l] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ts_rs, off, l * nb * kRowBytes, 0));
    }
    // the next step's streamed inputs
    load_stream(step + kQPS < per_wave ? i_begin + step + kQPS : i_begin + step, os_next, lse_next, xg_next);
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
    load_codes(step + kQPS < per_wave ? i_begin + step + kQPS : i_begin + step, cw);

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
    if (gate_fast) {
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
    // reciprocals with v_rcp_f32 (1 ulp)
    const float g_s = __builtin_amdgcn_rcpf(1.0f + __expf(-(a0 + gb0)));
    const float g_lr = __builtin_amdgcn_rcpf(1.0f + __expf(-(a1 + gb1)));
    const float z_lr = z * (1.0f / static_cast<float>(LC));
    const float rz = z > 0.0f ? __builtin_amdgcn_rcpf(z) : 0.0f;  // (num / L) / (z / L); 0 where z = 0
    const float mass_lr = lambda * z_lr;
    const float alpha = mass_lr > 0.0f ? __builtin_amdgcn_rcpf(1.0f + __expf(__logf(mass_lr) - lse_i)) : 1.0f;
    const float ws = g_s * alpha;

    float o_lr[kCols], yv[kCols];
#pragma unroll
    for (int k = 0; k < kCols; ++k) {
      o_lr[k] = num[k] * rz;
      yv[k] = __builtin_fmaf(ws, osv[k], g_lr * o_lr[k]);
    }
    // The next step's streamed inputs and codes are waited for here, before
    // this step's store: the vector memory counter retires in issue order,
    // so a wait for them after the store would also wait for the store.
    asm volatile("" : "+v"(yv[0]) : "v"(os_next), "v"(xg_next), "v"(lse_next) : "memory");
#pragma unroll
    for (int k = 0; k < kCW; ++k) asm volatile("" : "+v"(yv[0]) : "v"(cw[k]) : "memory");
    const uint32_t yo = static_cast<uint32_t>(i) * kRowBytes + vbase;
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
    if (aux.o_lr) {
#pragma unroll
      for (int k = 0; k < kCols; k += 4)
        *reinterpret_cast<f32x4 *>(aux.o_lr + qi * D + sub * kCols + k) =
            f32x4{o_lr[k], o_lr[k + 1], o_lr[k + 2], o_lr[k + 3]};
    }
    if (sub == 0) {
      if (aux.z_lr) aux.z_lr[qi] = z_lr;
      if (aux.alpha) aux.alpha[qi] = alpha;
      if (aux.g_s) aux.g_s[qi] = g_s;
      if (aux.g_lr) aux.g_lr[qi] = g_lr;
    }
  }
}

template <int D, typename VT, typename CT, int LC>
void launch_wide(const Geometry &g, const void *x_gate, const float *gate_w, const float *gate_b,
                 const Buffers &buf, const AuxOut &aux, void *out, hipStream_t stream) {
  constexpr int kQPS = 64 / (D / (16 / static_cast<int>(sizeof(VT))));
  // queries per workgroup: the largest of 512, 256, 128, 64 that divides N and
  // gives every wave whole steps (N is a multiple of 64)
  int R = 512;
  while (R > 64 && (g.N % R != 0)) R /= 2;
  while (R / 4 < kQPS) R *= 2;  // not reached for d <= 128
  const long long units = static_cast<long long>(g.BH) * (g.N / R);
  const long long grid = (units + kXcdCount - 1) / kXcdCount * kXcdCount;
  const size_t lds = static_cast<size_t>(LC) * g.nb_race * 4;
  hipLaunchKernelGGL((elsaa_k5_fuse_wide<D, VT, CT, LC>), dim3(static_cast<unsigned>(grid)), dim3(256), lds,
                     stream, static_cast<const VT *>(buf.o_s), buf.lse,
                     static_cast<const CT *>(buf.rcode), static_cast<const VT *>(buf.tsum), buf.tcnt,
                     static_cast<const VT *>(x_gate), gate_w, gate_b, g.H, g.N, g.P, g.DG, g.lambda, R,
                     units, static_cast<VT *>(out), aux);
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
                     g.lambda, total, qpw, static_cast<VT *>(out), aux);
}

template <int D, typename VT>
hipError_t launch_d(const Geometry &g, const void *x_gate, const float *gate_w, const float *gate_b,
                    const Buffers &buf, const AuxOut &aux, void *out, hipStream_t stream) {
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
  AuxOut a = {nullptr, nullptr, nullptr, nullptr, nullptr};
  if (aux) a = {aux->z_lr, aux->alpha, aux->g_s, aux->g_lr, aux->o_lowrank};
  if (g.bf16)
    return g.D == 64 ? launch_d<64, uint16_t>(g, x_gate, gate_w, gate_b, buf, a, out, stream)
                     : launch_d<128, uint16_t>(g, x_gate, gate_w, gate_b, buf, a, out, stream);
  return g.D == 64 ? launch_d<64, float>(g, x_gate, gate_w, gate_b, buf, a, out, stream)
                   : launch_d<128, float>(g, x_gate, gate_w, gate_b, buf, a, out, stream);
}

}  // namespace elsaa
