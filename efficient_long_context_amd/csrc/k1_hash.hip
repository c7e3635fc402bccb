// k1_hash.hip -- Sort-LSH and RACE sign-random-projection codes for every query
// and key ("Two Efficient Attentions, One Denominator Problem", section "Two
// efficient branches can still be mis-scaled": the sparse branch selects pairs
// by hashing, the RACE branch summarises keys by hash bucket).
//
// One thin GEMM per 16-row tile:  P^T[plane][row] = <plane, x_row>  for all
// R = sort_bits + L*P hyperplanes, on bf16 MFMA (16x16x32, fp32 accumulate).
// Code bit t is [exact <x, plane_t> > 0].  MFMA accumulation order and rounding
// are unspecified, so a bit is taken from the fp32 result only when
//     |p32| > tau = (d + 2) 2^-22 |x| |r| + d 2^-124,
// twice the worst-case error of any fp32 summation order of d exact bf16
// products (allowing truncation and flushed subnormals); otherwise the sign is
// recomputed exactly: binary64 dot product with its own error bound, and, if
// that is still undecided, a fixed-point (Kulisch) accumulation of the exact
// products.  Rows or planes with an element outside [2^-60, 2^60] (nonzero)
// always take the exact path, so the bound never meets overflow or underflow.
#include "elsaa_internal.hpp"

namespace elsaa {
namespace {

constexpr int kRowsPerTile = 16;
constexpr int kTilesPerWg = 32;  // 512 rows per workgroup

__device__ __forceinline__ bool in_safe_range(float a) {
  a = fabsf(a);
  return (a == 0.0f) || (a >= 0x1p-60f && a <= 0x1p60f);
}

// Sign of the exact sum of the d products x_e * r_e (each exact in binary64),
// via a fixed-point accumulator of 32-bit digits held in 64-bit limbs (no carry
// can overflow a limb within d <= 128 additions).  Products of binary32 or
// bfloat16 values lie in [2^-298, 2^256]; the least significant bit of a
// binary64 significand can then sit down to 2^-350.  Bit positions
// [-352, 288) are covered.
template <typename T>
__device__ __noinline__ int kulisch_dot_sign(const T *x, const T *r, int d) {
  constexpr int kLimbs = 20;  // 640 bits
  constexpr int kEmin = -352;
  long long acc[kLimbs];
  for (int j = 0; j < kLimbs; ++j) acc[j] = 0;
  for (int e = 0; e < d; ++e) {
    const double p = static_cast<double>(Elem<T>::load(x + e)) *
                     static_cast<double>(Elem<T>::load(r + e));
    if (p == 0.0) continue;
    const unsigned long long bits = static_cast<unsigned long long>(__double_as_longlong(p));
    int ex = static_cast<int>((bits >> 52) & 0x7ff);
    unsigned long long m = bits & ((1ull << 52) - 1);
    if (ex == 0) ex = 1; else m |= (1ull << 52);
    int pos = ex - 1075 - kEmin;  // p = +-m * 2^(ex - 1075)
    if (pos < 0) pos = 0;          // unreachable for binary32/bfloat16 inputs
    int limb = pos >> 5;
    if (limb > kLimbs - 3) limb = kLimbs - 3;  // unreachable; keeps indexing in bounds
    const int sh = pos & 31;
    const unsigned long long lo = (m << sh) & 0xffffffffull;
    const unsigned long long mid = (sh == 0 ? (m >> 32) : (m >> (32 - sh))) & 0xffffffffull;
    const unsigned long long hi = (sh == 0 ? 0ull : (m >> (64 - sh))) & 0xffffffffull;
    if (bits >> 63) {
      acc[limb] -= static_cast<long long>(lo);
      acc[limb + 1] -= static_cast<long long>(mid);
      acc[limb + 2] -= static_cast<long long>(hi);
    } else {
      acc[limb] += static_cast<long long>(lo);
      acc[limb + 1] += static_cast<long long>(mid);
      acc[limb + 2] += static_cast<long long>(hi);
    }
  }
  for (int j = 0; j < kLimbs - 1; ++j) {
    const long long c = acc[j] >> 32;  // floor division by 2^32
    acc[j] -= c * 4294967296ll;
    acc[j + 1] += c;
  }
  if (acc[kLimbs - 1] != 0) return acc[kLimbs - 1] > 0 ? 1 : -1;
  for (int j = kLimbs - 2; j >= 0; --j)
    if (acc[j] != 0) return 1;
  return 0;
}

// Exact sign of <x, r> for two rows of d stored values (binary32 or bfloat16):
// a binary64 sum of the exact products with its rounding-error bound decides
// almost every case; the rest goes to the fixed-point accumulator.
template <typename T>
__device__ __noinline__ int exact_dot_sign(const T *x, const T *r, int d) {
  double s = 0.0, sabs = 0.0;
  for (int e = 0; e < d; ++e) {
    const double p = static_cast<double>(Elem<T>::load(x + e)) *
                     static_cast<double>(Elem<T>::load(r + e));  // exact
    s += p;
    sabs += fabs(p);
  }
  const double bound = static_cast<double>(d + 1) * 0x1p-52 * sabs;
  if (s > bound) return 1;
  if (s < -bound) return -1;
  return kulisch_dot_sign<T>(x, r, d);
}

// Write one row's codes: the sort code (bits [0, ns)) and L race codes (bits
// ns + l*P + t).  `get` returns the 32-bit word w of the row's plane-bit mask.
template <typename GetWord>
__device__ __forceinline__ uint32_t bit_field(GetWord get, int pos, int n) {
  if (n == 0) return 0u;
  const int wd = pos >> 5, sh = pos & 31;
  unsigned long long x = static_cast<unsigned long long>(get(wd)) |
                         (static_cast<unsigned long long>(get(wd + 1)) << 32);
  return static_cast<uint32_t>((x >> sh) & ((1ull << n) - 1ull));
}

// ---------------------------------------------------------------- bf16 path --
template <int D>
__global__ __launch_bounds__(256) void elsaa_k1_hash_bf16(
    const uint16_t *__restrict__ xq, const uint16_t *__restrict__ xk,
    const uint16_t *__restrict__ planes, int R, int ns, int L, int P, long long rows,
    uint16_t *__restrict__ scode, void *__restrict__ rcode, int rcb) {
  constexpr int kLdsRow = D + 8;  // padded plane row (bf16 elements)
  extern __shared__ __align__(16) unsigned char smem[];
  const int R_pad = (R + 15) & ~15;
  const int n_words = (R_pad + 31) >> 5;
  uint16_t *sp = reinterpret_cast<uint16_t *>(smem);
  float *spn = reinterpret_cast<float *>(smem + static_cast<size_t>(R_pad) * kLdsRow * 2);
  int *ssafe = reinterpret_cast<int *>(spn + R_pad);
  uint32_t *smask = reinterpret_cast<uint32_t *>(ssafe + R_pad);  // [4 waves][16 rows][8 words]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tensor = blockIdx.y;
  const uint16_t *x = tensor ? xk : xq;

  // Stage the hyperplanes (zero rows beyond R) and their norms.
  for (int idx = tid; idx < R_pad * (D / 8); idx += 256) {
    const int t = idx / (D / 8), ch = idx % (D / 8);
    u16x8 val = (u16x8)0;
    if (t < R) val = *reinterpret_cast<const u16x8 *>(planes + static_cast<size_t>(t) * D + ch * 8);
    *reinterpret_cast<u16x8 *>(sp + t * kLdsRow + ch * 8) = val;
  }
  __syncthreads();
  for (int t = tid; t < R_pad; t += 256) {
    float ss = 0.0f;
    int safe = 1;
    for (int e = 0; e < D; ++e) {
      const float f = bf16_bits_to_f32(sp[t * kLdsRow + e]);
      ss += f * f;
      safe &= in_safe_range(f) ? 1 : 0;
    }
    spn[t] = sqrtf(ss);
    ssafe[t] = safe;
  }
  __syncthreads();

  const int g = lane >> 4, r16 = lane & 15;
  const long long n_tiles = (rows + kRowsPerTile - 1) / kRowsPerTile;
  uint32_t *wmask = smask + wave * 16 * 8;
  const float c_rel = static_cast<float>(D + 2) * 0x1p-22f;
  const float c_abs = static_cast<float>(D) * 0x1p-124f;

  for (int it = wave; it < kTilesPerWg; it += 4) {
    const long long tile = static_cast<long long>(blockIdx.x) * kTilesPerWg + it;
    if (tile >= n_tiles) break;
    const long long row = tile * kRowsPerTile + r16;
    const bool valid = row < rows;
    const uint16_t *xr = x + (valid ? row : 0) * D;

    bf16x8 b[D / 32];
    float ss = 0.0f;
    int safe = 1;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      u16x8 raw = (u16x8)0;
      if (valid) raw = *reinterpret_cast<const u16x8 *>(xr + kk * 32 + g * 8);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float f = bf16_bits_to_f32(raw[i]);
        ss += f * f;
        safe &= in_safe_range(f) ? 1 : 0;
      }
      b[kk] = __builtin_bit_cast(bf16x8, raw);
    }
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    safe &= __shfl_xor(safe, 16);
    safe &= __shfl_xor(safe, 32);
    const float xnorm = sqrtf(ss);

    uint32_t cur = 0;
    for (int pt = 0; pt < R_pad / 16; ++pt) {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u16x8 *>(sp + (pt * 16 + r16) * kLdsRow + kk * 32 + g * 8));
        acc = mfma16x16x32(a, b[kk], acc);
      }
      // lane holds <plane pt*16 + g*4 + i, row r16>
      uint32_t bits = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = pt * 16 + g * 4 + i;
        if (t < R && valid) {
          const float p = acc[i];
          const float tau = c_rel * xnorm * spn[t] + c_abs;
          int bit;
          if (safe && ssafe[t] && fabsf(p) > tau) {
            bit = p > 0.0f;
          } else {
            bit = exact_dot_sign<uint16_t>(xr, sp + t * kLdsRow, D) > 0;
          }
          bits |= static_cast<uint32_t>(bit) << ((pt & 1) * 16 + g * 4 + i);
        }
      }
      bits |= __shfl_xor(bits, 16);
      bits |= __shfl_xor(bits, 32);
      cur = (pt & 1) ? (cur | bits) : bits;
      if ((pt & 1) || pt == R_pad / 16 - 1) {
        if (lane < 16) wmask[lane * 8 + (pt >> 1)] = cur;
      }
    }
    // wave-local LDS: make the mask words visible to the lanes that extract codes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // Extract and store codes: lane (row r16, group g) writes table groups g, g+4, ...
    const long long orow = tile * kRowsPerTile + r16;
    if (orow < rows) {
      auto get = [&](int wd) -> uint32_t { return wd < n_words ? wmask[r16 * 8 + wd] : 0u; };
      const long long out_row = static_cast<long long>(tensor) * rows + orow;
      if (g == 0) scode[out_row] = static_cast<uint16_t>(bit_field(get, 0, ns));
      if (rcb == 1) {
        uint8_t *rc = reinterpret_cast<uint8_t *>(rcode) + out_row * L;
        if ((L & 3) == 0) {
          for (int j = g; j < L / 4; j += 4) {
            uint32_t word = 0;
            for (int e = 0; e < 4; ++e)
              word |= bit_field(get, ns + (4 * j + e) * P, P) << (8 * e);
            reinterpret_cast<uint32_t *>(rc)[j] = word;
          }
        } else {
          for (int l = g; l < L; l += 4) rc[l] = static_cast<uint8_t>(bit_field(get, ns + l * P, P));
        }
      } else {
        uint16_t *rc = reinterpret_cast<uint16_t *>(rcode) + out_row * L;
        if ((L & 1) == 0) {
          for (int j = g; j < L / 2; j += 4) {
            const uint32_t word = bit_field(get, ns + (2 * j) * P, P) |
                                  (bit_field(get, ns + (2 * j + 1) * P, P) << 16);
            reinterpret_cast<uint32_t *>(rc)[j] = word;
          }
        } else {
          for (int l = g; l < L; l += 4) rc[l] = static_cast<uint16_t>(bit_field(get, ns + l * P, P));
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// ----------------------------------------------------------------- fp32 path --
// One thread per row; binary32 FMA dot products (error <= gamma_d sum|x_i r_i|,
// covered by the same tau), exact fallback as above.
__global__ __launch_bounds__(256) void elsaa_k1_hash_f32(
    const float *__restrict__ xq, const float *__restrict__ xk, const float *__restrict__ planes,
    int D, int R, int ns, int L, int P, long long rows, uint16_t *__restrict__ scode,
    void *__restrict__ rcode, int rcb) {
  const long long row = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (row >= rows) return;
  const int tensor = blockIdx.y;
  const float *xr = (tensor ? xk : xq) + row * D;
  float ss = 0.0f;
  int safe = 1;
  for (int e = 0; e < D; ++e) {
    ss += xr[e] * xr[e];
    safe &= in_safe_range(xr[e]) ? 1 : 0;
  }
  const float xnorm = sqrtf(ss);
  const float c_rel = static_cast<float>(D + 2) * 0x1p-22f;
  const float c_abs = static_cast<float>(D) * 0x1p-124f;
  const long long out_row = static_cast<long long>(tensor) * rows + row;
  uint32_t code = 0;
  for (int t = 0; t < R; ++t) {
    const float *pr = planes + static_cast<size_t>(t) * D;
    float p = 0.0f, rs = 0.0f;
    int psafe = 1;
    for (int e = 0; e < D; ++e) {
      p = __builtin_fmaf(xr[e], pr[e], p);
      rs += pr[e] * pr[e];
      psafe &= in_safe_range(pr[e]) ? 1 : 0;
    }
    const float tau = c_rel * xnorm * sqrtf(rs) + c_abs;
    int bit;
    if (safe && psafe && fabsf(p) > tau) bit = p > 0.0f;
    else bit = exact_dot_sign<float>(xr, pr, D) > 0;
    // plane t feeds the sort code (t < ns) or bit (t - ns) % P of table (t - ns) / P
    const int local = t < ns ? t : (t - ns) % P;
    code |= static_cast<uint32_t>(bit) << local;
    const bool last = t < ns ? (t == ns - 1) : (local == P - 1);
    if (last) {
      if (t < ns) {
        scode[out_row] = static_cast<uint16_t>(code);
      } else {
        const int l = (t - ns) / P;
        if (rcb == 1) reinterpret_cast<uint8_t *>(rcode)[out_row * L + l] = static_cast<uint8_t>(code);
        else reinterpret_cast<uint16_t *>(rcode)[out_row * L + l] = static_cast<uint16_t>(code);
      }
      code = 0;
    }
  }
  if (ns == 0) scode[out_row] = 0;
  if (P == 0) {
    for (int l = 0; l < L; ++l) {
      if (rcb == 1) reinterpret_cast<uint8_t *>(rcode)[out_row * L + l] = 0;
      else reinterpret_cast<uint16_t *>(rcode)[out_row * L + l] = 0;
    }
  }
}

}  // namespace

hipError_t launch_hash(const Geometry &g, const void *q, const void *k, const void *planes,
                       const Buffers &buf, hipStream_t stream) {
  if (g.bf16) {
    const int R_pad = (g.R + 15) & ~15;
    const long long n_tiles = (g.rows + kRowsPerTile - 1) / kRowsPerTile;
    const dim3 grid(static_cast<unsigned>((n_tiles + kTilesPerWg - 1) / kTilesPerWg), 2);
    const size_t lds = static_cast<size_t>(R_pad) * (g.D + 8) * 2 + static_cast<size_t>(R_pad) * 8 +
                       4 * 16 * 8 * 4;
    if (g.D == 64)
      hipLaunchKernelGGL(elsaa_k1_hash_bf16<64>, grid, dim3(256), lds, stream,
                         static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                         static_cast<const uint16_t *>(planes), g.R, g.ns, g.L, g.P, g.rows,
                         buf.scode, buf.rcode, g.rcb);
    else
      hipLaunchKernelGGL(elsaa_k1_hash_bf16<128>, grid, dim3(256), lds, stream,
                         static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                         static_cast<const uint16_t *>(planes), g.R, g.ns, g.L, g.P, g.rows,
                         buf.scode, buf.rcode, g.rcb);
  } else {
    const dim3 grid(static_cast<unsigned>((g.rows + 255) / 256), 2);
    hipLaunchKernelGGL(elsaa_k1_hash_f32, grid, dim3(256), 0, stream,
                       static_cast<const float *>(q), static_cast<const float *>(k),
                       static_cast<const float *>(planes), g.D, g.R, g.ns, g.L, g.P, g.rows,
                       buf.scode, buf.rcode, g.rcb);
  }
  return hipGetLastError();
}

}  // namespace elsaa
