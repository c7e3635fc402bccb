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

// Sum over the 64 lanes of a wave of a binary64 value, every lane receiving
// the total, without a round trip through LDS: two quad permutes (lane bits 0
// and 1), the half-row and row mirrors (bits 2 and 3), then the permlane swaps
// across lane bits 4 and 5.  A pairwise tree of depth 6; each step adds a
// value and its partner's, in an order the two lanes share.
template <int kCtrl>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_mov_dpp(static_cast<int>(static_cast<uint32_t>(u)), kCtrl, 0xf, 0xf, false));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_mov_dpp(static_cast<int>(static_cast<uint32_t>(u >> 32)), kCtrl, 0xf, 0xf, false));
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}
template <bool kBit5>
__device__ __forceinline__ double swap_add_f64(double x) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  const uint32_t lo = static_cast<uint32_t>(u), hi = static_cast<uint32_t>(u >> 32);
  const auto rl = kBit5 ? __builtin_amdgcn_permlane32_swap(lo, lo, false, false)
                        : __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  const auto rh = kBit5 ? __builtin_amdgcn_permlane32_swap(hi, hi, false, false)
                        : __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  const double a = __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(rh[0]) << 32) | rl[0]));
  const double b = __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(rh[1]) << 32) | rl[1]));
  return a + b;  // (lower row's value) + (upper row's value) in both lanes
}
__device__ __forceinline__ double wave_sum_f64(double x) {
  x += dpp_f64<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp_f64<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  x += dpp_f64<0x141>(x);  // row_half_mirror: the other quad of the 8
  x += dpp_f64<0x140>(x);  // row_mirror: the other 8 of the row of 16
  x = swap_add_f64<false>(x);
  return swap_add_f64<true>(x);
}

// Exact sign of <x, r> for two rows of d bfloat16 values, one wave, lanes over
// the elements.  A bfloat16 value is M 2^E with an integer M < 2^8 (E = e - 134
// for a normal exponent field e, M = 128 + fraction; E = -133 and M = fraction
// for subnormals), so every product is an integer below 2^16 times 2^(Ex + Er).
// When the nonzero products' exponents span at most 39 they are shifted to the
// smallest one and added as 64-bit integers (d 2^16 2^39 < 2^63: exact, and
// integer addition is associative, so any reduction order gives the same
// value).  Returns -1, 0, 1, or 2 when the span is wider (caller falls back).
__device__ __forceinline__ void bf16_split(uint16_t b, int &m, int &e) {
  const int ef = (b >> 7) & 0xff, frac = b & 0x7f;
  m = ef ? (frac | 0x80) : frac;
  e = ef ? ef - 134 : -133;
}

template <int D>
__device__ int wave_exact_sign_bf16(const uint16_t *x, const uint16_t *r, int lane) {
  constexpr int kPer = D / 64;
  constexpr int kNone = 1 << 20;
  int pm[kPer], pe[kPer];
  bool neg[kPer];
  int emin = kNone, emax = -kNone;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const uint16_t bx = x[lane + 64 * j], br = r[lane + 64 * j];
    int mx, ex, mr, er;
    bf16_split(bx, mx, ex);
    bf16_split(br, mr, er);
    pm[j] = mx * mr;
    pe[j] = ex + er;
    neg[j] = ((bx ^ br) & 0x8000) != 0;
    if (pm[j] != 0) {
      emin = pe[j] < emin ? pe[j] : emin;
      emax = pe[j] > emax ? pe[j] : emax;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const int a = __shfl_xor(emin, off), b = __shfl_xor(emax, off);
    emin = a < emin ? a : emin;
    emax = b > emax ? b : emax;
  }
  if (emin == kNone) return 0;  // every product is zero
  if (emax - emin > 39) return 2;
  long long acc = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const long long t = static_cast<long long>(pm[j]) << (pm[j] ? pe[j] - emin : 0);
    acc += neg[j] ? -t : t;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  return acc > 0 ? 1 : (acc < 0 ? -1 : 0);
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
// A workgroup of 4 waves hashes 64 rows per step (16 per wave).  The rows of
// the next step are loaded into registers while the current step is hashed and
// staged in LDS at the top of the next step.  NPT = R_pad / 16 plane tiles is a
// compile-time count.
//
// Certification, per row: the row passes the range check when its largest
// |element| lies in [2^-40, 2^40] (then |x|^2 is a normal binary32 and dropping
// squares of elements below 2^-63 changes |x| by a relative 2^-40 at most).
// tau_row = |x| * max_t(c |r_t|) + d 2^-124 bounds the error of every plane's
// projection of that row (c = (d + 2) 2^-22, twice the worst-case relative
// error of d fp32 additions; d 2^-124 covers flushed subnormal products and
// partial sums).  Projections within tau of zero are re-decided in binary64 by
// the whole wave; planes outside the range, rows that fail the check, and
// projections binary64 cannot decide send the row to the exact fix-up kernel.
//
// Bits.  A lane's MFMA result holds four planes of one row.  Rather than
// testing each projection, its sign bit is shifted into a per-lane word (one
// v_alignbit per projection) and the smallest |projection| of the lane is
// kept (v_min3); only a wave with some projection at or below tau redoes the
// projections and re-decides those one by one.  The planes are staged in LDS
// in the order that makes the shifted-in bits land on their final positions:
// lane group g of tile pair (2w, 2w+1) owns byte g of mask word w (see
// tile_plane); a last unpaired tile gives each group a nibble.  Padding rows
// of the last tile repeat plane 0, so every projection is real and no
// per-lane padding test is needed (bits of planes >= R are never read).
//
// Plane held by row m of plane tile pt, for npt tiles in all.
__host__ __device__ constexpr int tile_plane(int pt, int m, int npt) {
  return 32 * (pt >> 1) + ((pt | 1) < npt ? 8 * (m >> 2) + 7 - 4 * (pt & 1) : 4 * (m >> 2) + 3) - (m & 3);
}

template <int D, int NPT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5))) void elsaa_k1_hash_bf16(
    const uint16_t *__restrict__ xq, const uint16_t *__restrict__ xk,
    const uint16_t *__restrict__ planes, int R, int ns, int L, int P, long long rows,
    uint16_t *__restrict__ scode, void *__restrict__ rcode, int rcb, uint8_t *__restrict__ flags,
    long long rows_per_wg) {
  constexpr int kLdsRow = D + 8;  // padded row (bf16 elements)
  constexpr int kRPad = NPT * 16;
  constexpr int kWords = (kRPad + 31) / 32;
  constexpr int kStepRows = 64;
  __shared__ __align__(16) uint16_t sp[kRPad * kLdsRow];
  __shared__ float s_red[2];  // max_t c|r_t| and "all planes in range"
  // per wave, for 8-bit codes: keys -- the codes of its 16 rows, table-major
  // [table][16 rows] (L <= 64), stored as one 16-byte piece per table;
  // queries -- the plane masks of its 16 rows, row-major with kQRowB bytes a
  // row (an odd number of words, so the 16 rows fall in distinct banks)
  constexpr int kQRowB = 4 * ((kWords + 1) | 1);
  static_assert(16 * kQRowB <= 64 * 16, "query mask rows fit the wave's buffer");
  // The same buffer holds the row of the projection the wave's exact path is
  // deciding (d bf16), which ends before the codes are written.
  static_assert(D * 2 <= 64 * 16, "one row fits the wave's buffer");
  __shared__ __align__(16) uint8_t kcl[4][64 * 16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tensor = blockIdx.y;
  const uint16_t *x = tensor ? xk : xq;

  // Stage the hyperplanes in tile order (rows past R repeat plane 0).
  for (int idx = tid; idx < kRPad * (D / 8); idx += 256) {
    const int pr = idx / (D / 8), ch = idx % (D / 8);
    const int t = tile_plane(pr >> 4, pr & 15, NPT);
    const u16x8 val = *reinterpret_cast<const u16x8 *>(planes + static_cast<size_t>(t < R ? t : 0) * D + ch * 8);
    *reinterpret_cast<u16x8 *>(sp + pr * kLdsRow + ch * 8) = val;
  }
  __syncthreads();
  if (wave == 0) {  // plane norms: wave 0, lane t handles staged rows t, t+64, ...
    float rmax = 0.0f;
    int ok = 1;
    for (int t = lane; t < kRPad; t += 64) {
      float ss = 0.0f, amax = 0.0f;
      for (int e = 0; e < D; ++e) {
        const float f = bf16_bits_to_f32(sp[t * kLdsRow + e]);
        ss = __builtin_fmaf(f, f, ss);
        amax = fmaxf(amax, fabsf(f));
      }
      ok &= (amax >= 0x1p-40f && amax <= 0x1p40f) ? 1 : 0;
      rmax = fmaxf(rmax, sqrtf(ss));
    }
    for (int off = 32; off > 0; off >>= 1) {
      rmax = fmaxf(rmax, __shfl_xor(rmax, off));
      ok &= __shfl_xor(ok, off);
    }
    if (lane == 0) {
      s_red[0] = static_cast<float>(D + 2) * 0x1p-22f * rmax;
      s_red[1] = ok ? 1.0f : 0.0f;
    }
  }
  __syncthreads();
  const float c_plane = s_red[0];
  const bool planes_ok = s_red[1] != 0.0f;
  const float c_abs = static_cast<float>(D) * 0x1p-124f;

  const int g = lane >> 4, r16 = lane & 15;
  const long long row_begin = static_cast<long long>(blockIdx.x) * rows_per_wg;
  const long long row_end = row_begin + rows_per_wg < rows ? row_begin + rows_per_wg : rows;

  // Each wave hashes rows r0 + 16 w .. +15 of every 64-row step of the
  // workgroup's range, on its own (no workgroup barrier in the loop): a
  // lane's 16-byte piece of its row (d-slice kk*32 + g*8 .. +7) is exactly
  // its part of the MFMA operand, so rows go from memory straight to
  // registers, the next step's in flight while this one is hashed.
  auto load_rows = [&](long long r0, u32x4 (&dst)[D / 32]) {
    const long long row = r0 + wave * 16 + r16;
    // clamped to the range's last row (just read, so a cache hit); results of
    // clamped rows are discarded
    const long long rr = row < row_end ? row : row_end - 1;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) dst[kk] = *reinterpret_cast<const u32x4 *>(x + rr * D + kk * 32 + g * 8);
  };
  // 8-bit codes on byte boundaries go through the wave's LDS buffer
  const bool byte_codes = P == 8 && ns % 8 == 0 && L % 4 == 0 && L <= 64;
  uint8_t *kw = kcl[wave];
  u32x4 nxt[D / 32];
  load_rows(row_begin, nxt);
  for (long long r0 = row_begin; r0 < row_end; r0 += kStepRows) {
    u32x4 cur[D / 32];
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) cur[kk] = nxt[kk];
    // in flight while this step is hashed (unconditional: the last step loads
    // clamped rows it never uses, and no branch splits the wait for them)
    load_rows(r0 + kStepRows, nxt);

    const int lrow = wave * 16 + r16;
    const long long row = r0 + lrow;
    const bool valid = row < row_end;

    // |x|^2 of the row (lane group g holds a quarter of it): bfloat16 squares
    // are exact in binary32, summed by v_dot2_f32_bf16
    float ss = 0.0f;
    bf16x8 b[D / 32];
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      const u32x4 raw = cur[kk];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t wv = raw[i];  // (bit_cast of raw[i] itself reads element 0 with this clang)
        const bf16x2 h = __builtin_bit_cast(bf16x2, wv);
        ss = __builtin_amdgcn_fdot2_f32_bf16(h, h, ss, false);
      }
      b[kk] = __builtin_bit_cast(bf16x8, raw);
    }
    ss = sum_over_lane_groups<16>(ss);
    // Range check: |x|^2 in [2^-72, 2^80] puts every element at or below 2^40
    // and the largest at or above 2^-40 (d <= 128); NaN and Inf fail it.
    const bool row_ok = planes_ok && ss >= 0x1p-72f && ss <= 0x1p80f;
    // tau = +inf sends every projection of this row to the exact path
    const float tau = row_ok ? __builtin_fmaf(sqrtf(ss), c_plane, c_abs) : INFINITY;

    auto project = [&](int pt) {
      f32x4 a4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u16x8 *>(sp + (pt * 16 + r16) * kLdsRow + kk * 32 + g * 8));
        a4 = mfma16x16x32(a, b[kk], a4);
      }
      return a4;  // lane holds the projections of row r16 on staged rows pt*16 + g*4 + i
    };
    // bit position of projection (pt, i) in its lane's word, in shifted-in order
    auto bit_pos = [](int pt, int i) {
      return ((pt | 1) < NPT ? 7 - 4 * (pt & 1) : 3) - i;
    };
    uint32_t words[kWords];
#pragma unroll
    for (int w = 0; w < kWords; ++w) words[w] = 0u;
    // bit pt: some certified-range row of the wave has a projection on plane
    // tile pt within tau of zero (wave-uniform; one compare per tile)
    uint32_t tile_mask = 0u;
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt) {
      const f32x4 a4 = project(pt);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        words[pt >> 1] = __builtin_amdgcn_alignbit(words[pt >> 1], __float_as_uint(a4[i]), 31);
      const float tmin = fminf(fminf(fabsf(a4[0]), fabsf(a4[1])), fminf(fabsf(a4[2]), fabsf(a4[3])));
      tile_mask |= (__ballot(valid && row_ok && !(tmin > tau)) != 0ull ? 1u : 0u) << pt;
    }
    // sign bit 1 = negative: the code bit is its complement wherever |p| > tau
#pragma unroll
    for (int w = 0; w < kWords; ++w) words[w] = ~words[w];
    bool undecided = valid && !row_ok;
    // Each uncertified projection is re-decided by the whole wave, lanes over
    // the d products (exact in binary64), summed by a cross-lane tree of depth
    // log2(64) (+1 for d = 128 with two products per lane); the sign is taken
    // when |sum| exceeds (depth + 1) 2^-52 sum |p_i|, else from the exact
    // integer sum; only a product exponent span too wide for it flags the row.
    // About 1e-4 of the projections of unit-scale rows are uncertified, which
    // is one wave step in four at 16 x 136 projections a step, and mostly one
    // plane tile of the step: only the marked tiles are projected again.
    if (tile_mask != 0u) {
      unsigned long long unsure = 0ull;  // bit 4 pt + i: projection not certified
      // recomputed, not kept: the plane reads below must not be merged with the
      // first pass's, which would hold all its projections live
      asm volatile("" ::: "memory");
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) {
        if ((tile_mask >> pt) & 1u) {
          const f32x4 a4 = project(pt);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            unsure |= static_cast<unsigned long long>(!(fabsf(a4[i]) > tau)) << (pt * 4 + i);
        }
      }
      // rows outside the certified range go to the exact fix-up kernel whole
      if (!valid || !row_ok) unsure = 0ull;
      uint16_t *xs = reinterpret_cast<uint16_t *>(kw);  // the source lane's row, staged below
      for (unsigned long long pending = __ballot(unsure != 0ull); pending;
           pending = __ballot(unsure != 0ull)) {
        const int src = __builtin_ctzll(pending);  // wave-uniform
        const unsigned long long sb =
            static_cast<unsigned long long>(static_cast<uint32_t>(__builtin_amdgcn_readlane(
                static_cast<int>(unsure), src))) |
            (static_cast<unsigned long long>(static_cast<uint32_t>(
                 __builtin_amdgcn_readlane(static_cast<int>(unsure >> 32), src)))
             << 32);
        const int bpos = __builtin_ctzll(sb);
        // the source lane's row to LDS from the operand registers of its four
        // lanes (lanes of the previous projection have read theirs: LDS
        // accesses of a wave complete in order)
        if (r16 == (src & 15)) {
#pragma unroll
          for (int kk = 0; kk < D / 32; ++kk) *reinterpret_cast<u32x4 *>(xs + kk * 32 + g * 8) = cur[kk];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
        const uint16_t *ps = sp + ((bpos >> 2) * 16 + (src >> 4) * 4 + (bpos & 3)) * kLdsRow;
        double sum = 0.0, sabs = 0.0;
#pragma unroll
        for (int e = lane; e < D; e += 64) {
          const double prod = static_cast<double>(bf16_bits_to_f32(xs[e])) *
                              static_cast<double>(bf16_bits_to_f32(ps[e]));  // exact
          sum += prod;
          sabs += fabs(prod);
        }
        sum = wave_sum_f64(sum);
        sabs = wave_sum_f64(sabs);
        constexpr int kDepth = 6 + D / 64;
        const double bound = static_cast<double>(kDepth + 1) * 0x1p-52 * sabs;
        // within the bound (exact ties included): the integer sum decides
        int sgn = sum > bound ? 1 : (sum < -bound ? -1 : 2);
        if (__builtin_amdgcn_readlane(sgn, src) == 2) sgn = wave_exact_sign_bf16<D>(xs, ps, lane);
        if (lane == src) {
          unsure &= unsure - 1ull;
          if (sgn != 2) {
            const int pt = bpos >> 2;
            const uint32_t m = 1u << bit_pos(pt, bpos & 3);
#pragma unroll
            for (int q = 0; q < kWords; ++q)
              if ((pt >> 1) == q) words[q] = sgn > 0 ? (words[q] | m) : (words[q] & ~m);
          } else {
            undecided = true;
          }
        }
      }
    }
    const unsigned long long undecided_mask = __ballot(undecided);
    // The next step's rows are waited for here, after the last change to the
    // mask words and before this step's code stores: the memory counter
    // retires in issue order, so a wait placed after the stores would also
    // wait for their completion.
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) asm volatile("" : "+v"(words[0]) : "v"(nxt[kk]) : "memory");
    if (undecided_mask != 0ull && lane == 0) *flagged_any(flags, rows) = 1u;
    const long long out_row = static_cast<long long>(tensor) * rows + row;
    if (byte_codes) {
      // 8-bit codes starting on a byte boundary (ns is 0 or 8).  Group g holds
      // byte g of every plane-mask word w (mask byte 4 w + g) in the low 8 bits
      // of words[w]; an unpaired last tile gives nibble g of the word's low
      // half instead, and pairs of groups are merged into bytes 4 w + g / 2.
      // Each lane writes its bytes to the wave's LDS buffer: the row-major mask
      // of its row (queries) or its codes in table-major order (keys).
      uint32_t byte0 = 0u;  // mask byte 0 (the sort code), valid in group 0
#pragma unroll
      for (int w = 0; w < kWords; ++w) {
        uint32_t byte;
        int bidx;  // mask byte this lane writes, -1 for none
        if (2 * w + 1 < NPT) {
          byte = words[w] & 0xffu;
          bidx = 4 * w + g;
        } else {
          const uint32_t v = (words[w] & 0xfu) << (4 * (g & 1));
          const auto sw = __builtin_amdgcn_permlane16_swap(v, v, false, false);  // groups g and g ^ 1
          byte = sw[0] | sw[1];
          bidx = (g & 1) ? -1 : 4 * w + (g >> 1);
        }
        if (w == 0) byte0 = byte;
        const int l = bidx - ns / 8;  // table of a key code byte
        const bool put = tensor == 0 ? bidx >= 0 : (bidx >= 0 && l >= 0 && l < L);
        const int at = tensor == 0 ? r16 * kQRowB + bidx : l * 16 + r16;
        if (put) kw[at] = static_cast<uint8_t>(byte);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
      if (valid && g == 0) {
        if (ns > 0) scode[out_row] = static_cast<uint16_t>(byte0 & ((1u << ns) - 1u));
        // a projection binary64 could not decide: the exact pass redoes the row
        flags[out_row] = ((undecided_mask >> r16) & 0x0001000100010001ull) ? 1 : 0;
      }
      if (tensor == 0) {
        // row-major codes: code word j is mask bytes ns/8 + 4j .. +3, a byte
        // funnel of two aligned words of the row; the wave's 16 rows are
        // consecutive, so its stores cover one contiguous block
        if (valid) {
          const uint8_t *rowb = kw + r16 * kQRowB;
          uint32_t *rc = reinterpret_cast<uint32_t *>(reinterpret_cast<uint8_t *>(rcode) + out_row * L);
          for (int j = g; j < L / 4; j += 4) {
            const int bp = ns / 8 + 4 * j;
            const uint32_t lo = *reinterpret_cast<const uint32_t *>(rowb + (bp & ~3));
            const uint32_t hi = *reinterpret_cast<const uint32_t *>(rowb + (bp & ~3) + 4);
            rc[j] = __builtin_amdgcn_alignbyte(hi, lo, bp & 3);
          }
        }
      } else {  // table-major codes: lane t stores table t's 16 rows of this wave
        const long long rs = r0 + wave * 16;
        for (int t = lane; t < L; t += 64) {
          uint8_t *dst = reinterpret_cast<uint8_t *>(rcode) + rows * L + static_cast<long long>(t) * rows + rs;
          const uint8_t *src = kw + t * 16;
          if (rows % 16 == 0 && rs + 16 <= row_end) {
            *reinterpret_cast<u32x4 *>(dst) = *reinterpret_cast<const u32x4 *>(src);
          } else {
            for (int e = 0; e < 16 && rs + e < row_end; ++e) dst[e] = src[e];
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");  // read before the next step writes
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
      continue;
    }
    // Other code widths: OR the four groups' bytes (nibbles for an unpaired
    // last tile) so every lane of a row holds the row's full plane mask, then
    // cut each code out of it.
#pragma unroll
    for (int w = 0; w < kWords; ++w) {
      const int nbits = 2 * w + 1 < NPT ? 8 : 4;
      uint32_t v = (words[w] & ((1u << nbits) - 1u)) << (g * nbits);
      const auto r16s = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      v = r16s[0] | r16s[1];
      const auto r32s = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      words[w] = r32s[0] | r32s[1];
    }
    auto get = [&](int wd) -> uint32_t {
      uint32_t r = 0u;
#pragma unroll
      for (int w = 0; w < kWords; ++w) r = wd == w ? words[w] : r;
      return r;
    };
    if (valid) {
      if (g == 0) {
        if (ns > 0) scode[out_row] = static_cast<uint16_t>(words[0] & ((1u << ns) - 1u));  // ns <= 12
        flags[out_row] = ((undecided_mask >> r16) & 0x0001000100010001ull) ? 1 : 0;
      }
      for (int l = g; l < L; l += 4) {
        const uint32_t code = bit_field(get, ns + l * P, P);
        const long long ci = race_code_index(tensor, row, l, rows, L);
        if (rcb == 1) reinterpret_cast<uint8_t *>(rcode)[ci] = static_cast<uint8_t>(code);
        else reinterpret_cast<uint16_t *>(rcode)[ci] = static_cast<uint16_t>(code);
      }
    }
  }
}

// ------------------------------------------------------------ exact fix-up --
// Rows flagged by the bf16 pass get every code bit recomputed exactly: one wave
// per row, lanes over hyperplanes.  Each lane forms the binary64 dot product of
// the exact products with its rounding bound (d + 1) 2^-52 sum |p_i|, which
// decides the sign unless the sum is within that bound of zero; only then is
// the fixed-point accumulation used.  Bits are gathered with ballots.
// Grid-stride over all rows: every wave reaches the end.
template <int D>
__global__ __launch_bounds__(256) void elsaa_k1_hash_fixup(
    const uint16_t *__restrict__ xq, const uint16_t *__restrict__ xk,
    const uint16_t *__restrict__ planes, int R, int ns, int L, int P, long long rows,
    const uint8_t *__restrict__ flags, uint16_t *__restrict__ scode, void *__restrict__ rcode,
    int rcb) {
  if (*flagged_any(const_cast<uint8_t *>(flags), rows) == 0u) return;  // no row flagged
  const int lane = threadIdx.x & 63;
  const long long waves = static_cast<long long>(gridDim.x) * 4;
  const long long total = 2 * rows;
  for (long long r0 = (static_cast<long long>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * 1024; r0 < total;
       r0 += waves * 1024) {
    // 1024 rows' flags per wave load (16 per lane); flagged rows are then
    // handled one at a time
    const long long f0 = r0 + lane * 16;
    uint32_t fm = 0u;  // bit e: row f0 + e is flagged
    if (f0 + 16 <= total) {
      const u32x4 w = *reinterpret_cast<const u32x4 *>(flags + f0);
#pragma unroll
      for (int e = 0; e < 16; ++e) fm |= ((w[e >> 2] >> (8 * (e & 3))) & 0xffu) ? (1u << e) : 0u;
    } else {
      for (int e = 0; f0 + e < total; ++e) fm |= flags[f0 + e] ? (1u << e) : 0u;
    }
    for (unsigned long long lanes = __ballot(fm != 0u); lanes; lanes = __ballot(fm != 0u)) {
      const int src = __builtin_ctzll(lanes);
      const uint32_t sm = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(fm), src));
      const long long r = r0 + src * 16 + __builtin_ctz(sm);
      if (lane == src) fm &= fm - 1u;
      const uint16_t *xr = (r < rows ? xq + r * D : xk + (r - rows) * D);
      u16x8 xv[D / 8];
#pragma unroll
      for (int c = 0; c < D / 8; ++c) xv[c] = *reinterpret_cast<const u16x8 *>(xr + c * 8);
      unsigned long long m[4];  // plane-bit masks, planes 64 q .. 64 q + 63
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int t = qd * 64 + lane;
        bool bit = false;
        if (qd * 64 < R) {  // wave-uniform
          const int tt = t < R ? t : R - 1;
          const uint16_t *pr = planes + static_cast<long long>(tt) * D;
          u16x8 pv[D / 8];
#pragma unroll
          for (int c = 0; c < D / 8; ++c) pv[c] = *reinterpret_cast<const u16x8 *>(pr + c * 8);
          double sum = 0.0, sabs = 0.0;
#pragma unroll
          for (int c = 0; c < D / 8; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const double prod = static_cast<double>(bf16_bits_to_f32(xv[c][e])) *
                                  static_cast<double>(bf16_bits_to_f32(pv[c][e]));  // exact
              sum += prod;
              sabs += fabs(prod);
            }
          const double bound = static_cast<double>(D + 1) * 0x1p-52 * sabs;
          int sgn = sum > bound ? 1 : (sum < -bound ? -1 : (sabs == 0.0 ? 0 : 2));
          if (sgn == 2) sgn = kulisch_dot_sign<uint16_t>(xr, pr, D);
          bit = t < R && sgn > 0;
        }
        m[qd] = __ballot(bit);
      }
      auto get = [&](int wd) -> uint32_t {
        if (wd >= 8) return 0u;
        const unsigned long long mm = m[wd >> 1];
        return (wd & 1) ? static_cast<uint32_t>(mm >> 32) : static_cast<uint32_t>(mm);
      };
      if (lane == 0 && ns > 0) scode[r] = static_cast<uint16_t>(bit_field(get, 0, ns));
      for (int l = lane; l < L; l += 64) {
        const uint32_t c = bit_field(get, ns + l * P, P);
        const long long ci = race_code_index(r >= rows ? 1 : 0, r >= rows ? r - rows : r, l, rows, L);
        if (rcb == 1) reinterpret_cast<uint8_t *>(rcode)[ci] = static_cast<uint8_t>(c);
        else reinterpret_cast<uint16_t *>(rcode)[ci] = static_cast<uint16_t>(c);
      }
    }
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
        const long long ci = race_code_index(tensor, row, (t - ns) / P, rows, L);
        if (rcb == 1) reinterpret_cast<uint8_t *>(rcode)[ci] = static_cast<uint8_t>(code);
        else reinterpret_cast<uint16_t *>(rcode)[ci] = static_cast<uint16_t>(code);
      }
      code = 0;
    }
  }
  if (P == 0) {
    for (int l = 0; l < L; ++l) {
      const long long ci = race_code_index(tensor, row, l, rows, L);
      if (rcb == 1) reinterpret_cast<uint8_t *>(rcode)[ci] = 0;
      else reinterpret_cast<uint16_t *>(rcode)[ci] = 0;
    }
  }
}

}  // namespace

template <int D, int NPT>
void launch_bf16(const Geometry &g, const void *q, const void *k, const void *planes,
                 const Buffers &buf, hipStream_t stream) {
  // One round of workgroups, equal shares of 64-row steps: as many
  // workgroups as the device holds at once (two tensors, grid.y), so no
  // partial second round leaves compute units idle.
  static const int per_cu = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, elsaa_k1_hash_bf16<D, NPT>, 256, 0) != hipSuccess ||
        n < 1)
      n = 1;
    return n;
  }();
  const long long steps = (g.rows + 63) / 64;
  long long wgs = static_cast<long long>(g.cus) * per_cu / 2;
  wgs = wgs < 1 ? 1 : (wgs < steps ? wgs : steps);
  const long long steps_per_wg = (steps + wgs - 1) / wgs;
  wgs = (steps + steps_per_wg - 1) / steps_per_wg;
  const dim3 grid(static_cast<unsigned>(wgs), 2);
  hipLaunchKernelGGL((elsaa_k1_hash_bf16<D, NPT>), grid, dim3(256), 0, stream,
                     static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                     static_cast<const uint16_t *>(planes), g.R, g.ns, g.L, g.P, g.rows, buf.scode,
                     buf.rcode, g.rcb, buf.flags, steps_per_wg * 64);
}

template <int D, int NPT = 1>
void dispatch_npt(int npt, const Geometry &g, const void *q, const void *k, const void *planes,
                  const Buffers &buf, hipStream_t stream) {
  if constexpr (NPT < 16) {
    if (npt > NPT) return dispatch_npt<D, NPT + 1>(npt, g, q, k, planes, buf, stream);
  }
  launch_bf16<D, NPT>(g, q, k, planes, buf, stream);
}

hipError_t launch_hash(const Geometry &g, const void *q, const void *k, const void *planes,
                       const Buffers &buf, hipStream_t stream) {
  // No planes (sort_bits = race_bits = 0): every RACE code is zero, and with
  // one sort bucket nothing reads sort codes.  The planes pointer may be NULL.
  if (g.R == 0) return launch_fill_zero(buf.rcode, 2 * static_cast<size_t>(g.rows) * g.L * g.rcb, stream);
  if (g.bf16) {
    const int npt = g.R > 0 ? (g.R + 15) / 16 : 1;  // R <= 256: at most 16 plane tiles
    if (g.D == 64) dispatch_npt<64>(npt, g, q, k, planes, buf, stream);
    else dispatch_npt<128>(npt, g, q, k, planes, buf, stream);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long fix_blocks = (2 * g.rows + 4095) / 4096;  // 4 waves x 1024 rows
    const dim3 fgrid(static_cast<unsigned>(fix_blocks < 1024 ? fix_blocks : 1024));
    if (g.D == 64)
      hipLaunchKernelGGL(elsaa_k1_hash_fixup<64>, fgrid, dim3(256), 0, stream,
                         static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                         static_cast<const uint16_t *>(planes), g.R, g.ns, g.L, g.P, g.rows,
                         buf.flags, buf.scode, buf.rcode, g.rcb);
    else
      hipLaunchKernelGGL(elsaa_k1_hash_fixup<128>, fgrid, dim3(256), 0, stream,
                         static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                         static_cast<const uint16_t *>(planes), g.R, g.ns, g.L, g.P, g.rows,
                         buf.flags, buf.scode, buf.rcode, g.rcb);
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
