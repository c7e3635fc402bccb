// elsaa_internal.hpp -- shared definitions of the ELSAA gfx950 kernels and the
// host library that launches them.  Not part of the public ABI (include/elsaa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "elsaa.h"

namespace elsaa {

// ----------------------------------------------------------------------------
// Problem geometry derived from elsaa_params_t (host side).
// ----------------------------------------------------------------------------
struct Geometry {
  int B, H, N, D, DG;
  int ns;        // Sort-LSH bits
  int w;         // chunk
  int L, P;      // RACE tables, bits
  int BH;
  long long rows;  // BH * N (rows of q, and of k)
  int R;         // hyperplane rows = ns + L * P
  int nb_sort;   // 2^ns
  int nb_race;   // 2^P
  int rcb;       // bytes per RACE code: 1 if P <= 8 else 2
  int sort_tiles;  // ceil(N / kSortTile)
  bool bf16;
  float lambda;
  int cus;       // compute units of the device (set at launch; 256 otherwise)
  int variant;   // elsaa_variant_t
  bool run_sparse;  // the Sort-LSH branch runs (not RACE_ONLY)
  bool run_race;    // the RACE branch runs (not SPARSE_ONLY)
  bool identity;    // sort_bits == 0: the stable order is the original one, no sort
  bool fused;       // the fusion runs in the chunk attention's epilogue (no o_s, LSE buffers)
  bool save;        // the fusion keeps o_lr, z and the gates for the backward pass
};

// Device buffers carved out of the caller's workspace.
struct Buffers {
  uint16_t *scode;  // [2][BH][N]     q codes then k codes
  void *rcode;      // q codes [BH*N][L], then k codes [L][BH*N]; uint8 or uint16
  int32_t *perm;    // [2][BH][N]
  uint8_t *flags;   // [2][BH][N]     rows whose codes need the exact pass,
                    // then one word: nonzero when any row may be flagged
  uint32_t *hist;   // [2][BH][nb_sort][sort_tiles] -> exclusive offsets; then
                    // the RACE build's tiled rank counts (race_hist_bytes)
  int32_t *rperm;   // [L][BH][N]     keys of each table sorted by bucket
  int32_t *rstart;  // [BH][L][nb_race + 1] run start of each bucket in rperm
  int32_t *rpart;   // [BH][L][parts + 1][2] per gather part: first owned bucket, its run start
  void *tsum;       // [BH][L][nb_race][D] bucket sums, stored in dtype
  float *tcnt;      // [BH][L][nb_race]
  float *psum;      // [BH][race_blocks][L][nb_race][D] partial tables (race_blocks > 1, else NULL)
  float *pcnt;      // [BH][race_blocks][L][nb_race] partial counts
  void *o_s;        // [BH][N][D] in dtype
  float *lse;       // [BH][N]
  // kept for the backward pass (ELSAA_OPT_SAVE_FOR_BACKWARD; else NULL):
  void *sv_olr;     // [BH][N][D] o_lr in dtype
  float *sv_z, *sv_gs, *sv_glr;  // [BH][N] raw count sum z = L Z_lr, g_s, g_lr
};

// The word after the exact-pass flags (2 rows bytes): the hash sets it when it flags
// a row, the fix-up kernel skips its scan while it is zero, and the RACE rank
// kernel (which runs after the fix-up) clears it for the next call.  Stale
// contents only cost a scan that finds nothing.
__host__ __device__ __forceinline__ uint32_t *flagged_any(uint8_t *flags, long long rows) {
  return reinterpret_cast<uint32_t *>(flags + 2 * rows);
}

// Element index of the RACE code of (row, table l) in Buffers::rcode: query
// codes are row-major [rows][L] (the fusion reads a query's L codes
// together), key codes table-major [L][rows] after them (the RACE build reads
// one table's codes of consecutive keys).
__host__ __device__ __forceinline__ long long race_code_index(int tensor, long long row, int l, long long rows,
                                                              int L) {
  return tensor == 0 ? row * L + l : rows * L + static_cast<long long>(l) * rows + row;
}

// Positions of one table's sorted keys per RACE gather wave ("part"), before
// rounding to whole buckets.
constexpr int kGatherPos = 256;
__host__ __device__ __forceinline__ int race_parts(int N) { return (N + kGatherPos - 1) / kGatherPos; }

constexpr int kSortTile = 2048;         // elements per sort tile (4 waves x 8 rounds x 64)

// Launchers (each enqueues on `stream`, returns hipError_t of the launch).
// Zero bytes [p, p + n) (p 16-byte aligned) with a fill kernel: no
// hipMemsetAsync, so a caller may capture the forward pass into a graph.
hipError_t launch_fill_zero(void *p, size_t n, hipStream_t stream);
hipError_t launch_hash(const Geometry &g, const void *q, const void *k, const void *planes,
                       const Buffers &buf, hipStream_t stream);
hipError_t launch_sort(const Geometry &g, const Buffers &buf, hipStream_t stream);
// The sort takes the tiled path, which uses Buffers::hist (shared with the
// RACE build's tiled rank); otherwise one workgroup per segment, no scratch.
bool sort_is_tiled(const Geometry &g);
// o_s goes to `o_s` (buf.o_s, or the output itself for SPARSE_ONLY).
hipError_t launch_chunk_attention(const Geometry &g, const void *q, const void *k,
                                  const void *v, const Buffers &buf, void *o_s, hipStream_t stream);
hipError_t launch_race_build(const Geometry &g, const void *v, const Buffers &buf,
                             hipStream_t stream);
// The RACE build over any codes and rows: per table, the counts of codes[l][row]
// and the per-bucket sums of the rows (the forward sums values by key code;
// the backward sums query gradients by query code).
struct RaceBuildIO {
  const void *codes;  // [L][BH*N] codes, uint8 if P <= 8 else uint16
  const void *values; // [BH][N][D] rows
  bool values_f32;    // rows and sums are binary32 (else the problem's dtype)
  void *rperm;        // [L][BH][N] sorted indices (uint16 when N <= 65536, else int32)
  uint32_t *hist;     // race_hist_bytes(g): tile counts of the tiled rank (unused when staged)
  int32_t *rstart;    // [BH][L][2^P + 1]
  int32_t *rpart;     // [BH][L][parts + 1][2]
  void *tsum;         // [BH][L][2^P][D] sums
  float *tcnt;        // [BH][L][2^P] counts
  uint32_t *flag;     // a word the rank kernel clears
  // token blocks (race_blocks): with blocks > 1 the tables are first built
  // per (b, h, block of N / blocks consecutive keys) into binary32 partial
  // tables, then summed over the blocks in block order into tsum and tcnt
  int blocks = 1;
  float *psum = nullptr;  // [BH][blocks][L][2^P][D]
  float *pcnt = nullptr;  // [BH][blocks][L][2^P]
};
// Token blocks of the forward's RACE build: 1, or, when a (b, h)'s value rows
// exceed 8 MB, the power of two that cuts them into blocks of at most 8 MB
// (which one XCD's L2 and its share of the last-level cache serve to all L
// tables' passes); 1 again when the blocks would not hold whole 64-key groups
// or their partial tables would exceed twice the rows they sum.
int race_blocks(const Geometry &g);
// The geometry the RACE build's rank and gather run on: (b, h, block) as
// B * H * blocks heads of N / blocks keys.
Geometry race_block_geometry(const Geometry &g);
hipError_t launch_race_build_io(const Geometry &g, const RaceBuildIO &io, hipStream_t stream);
// Scratch of the RACE build's tiled rank (0 when one workgroup per table
// ranks in LDS): [L][BH][2^P][tiles] counts.
size_t race_hist_bytes(const Geometry &g);
// Tiled counting sort (k2_sort.hip) of S segments of N codes (code_bytes 1 or
// 2, `bits` bits), segment s at codes + s N, into perm + s N (index_bytes 2
// or 4): buckets in ascending order, each bucket's elements in an order that
// is the same on every run (tiles in order; inside a tile, the LDS unit's
// order of same-address atomics).  hist holds S 2^bits tiled_sort_tiles(N,
// bits) words; it is left with the scanned counts: word (s, b, 0) of
// [S][2^bits][tiles] is the first sorted position of bucket b.
int tiled_sort_tiles(int N, int bits);
hipError_t launch_tiled_sort(const void *codes, int code_bytes, int N, int bits, long long S,
                             uint32_t *hist, void *perm, int index_bytes, hipStream_t stream);

// Backward pass (k6_backward.hip).  The forward's workspace (Buffers) still
// holds that call's codes, permutations, tables, o_s and LSE.
struct BackwardInputs {
  const void *q, *k, *v, *x_gate, *y, *dy;
  const float *gate_w, *gate_b;
  float lambda;  // the caller's lambda (the variant decides whether alpha uses it)
};
struct BackwardBuffers {
  void *do_s;        // [BH][N][D] dtype
  float *delta;      // [BH][N]
  void *dcon;        // [BH][N][D] dtype
  float *da_s, *da_lr, *dlam;  // [BH][N]
  float *dv_acc;     // [BH][N][D] binary32, the sparse part of dv
  void *qcode_t;     // [L][BH*N] query codes, table-major
  void *qrperm;      // [L][BH][N]
  uint32_t *qhist;   // race_hist_bytes(g)
  int32_t *qrstart;  // [BH][L][2^P + 1]
  int32_t *qrpart;   // [BH][L][parts + 1][2]
  void *dT;          // [BH][L][2^P][D] dtype
  float *qtcnt;      // [BH][L][2^P]
  float *gate_part;  // [H][64][2 d_gate + 3]
  uint32_t *flag;
};
// Token blocks of the backward's gate-gradient partial sums (reduced in order).
constexpr int kGateBlocks = 256;
struct BackwardOutputs {
  void *dq, *dk, *dv, *dx_gate;
  float *dgate_w, *dgate_b, *dlambda;
};
hipError_t launch_backward(const Geometry &g, const BackwardInputs &in, const Buffers &fb,
                           const BackwardBuffers &bb, const BackwardOutputs &out, hipStream_t stream);
// Chunk attention with the RACE gather, gates and fusion in its epilogue, for
// the shapes attention_fusable() accepts: writes y to `out` (and the aux
// outputs of both stages that are requested), never o_s or its LSE.
bool attention_fusable(const Geometry &g);
hipError_t launch_attention_fused(const Geometry &g, const void *q, const void *k, const void *v,
                                  const void *x_gate, const float *gate_w, const float *gate_b,
                                  const Buffers &buf, const elsaa_aux_t *aux, void *out, hipStream_t stream);
hipError_t launch_fuse(const Geometry &g, const void *x_gate, const float *gate_w,
                       const float *gate_b, const Buffers &buf, const elsaa_aux_t *aux,
                       void *out, hipStream_t stream);

// ----------------------------------------------------------------------------
// Device helpers.
// ----------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two binary32 values to packed bfloat16, round to nearest even (one
// v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 h = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even binary32 -> bfloat16 bits (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Adds a bfloat16 half of a packed word to a binary32 accumulator in one
// instruction: v_dot2_f32_bf16 with weights (1, 0) or (0, 1), i.e. acc + x * 1
// + y * 0, instead of unpacking (shift or mask) and adding.  The weight words
// are made by s_mov_b32 inside asm: left to the compiler, 0x00003f80 can be
// re-encoded as the inline constant 1.0, which the instruction reads as the
// other half.
struct Bf16Adder {
  uint32_t wlo, whi;
  __device__ __forceinline__ Bf16Adder() {
    asm("s_mov_b32 %0, 0x3f80" : "=s"(wlo));
    asm("s_mov_b32 %0, 0x3f800000" : "=s"(whi));
  }
  __device__ __forceinline__ float lo(float acc, uint32_t w) const {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, wlo),
                                           acc, false);
  }
  __device__ __forceinline__ float hi(float acc, uint32_t w) const {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, whi),
                                           acc, false);
  }
};

// Raw buffer resource over `bytes` bytes at `base` (a wave-uniform address):
// loads through it take a 32-bit per-lane offset plus a scalar offset, and
// offsets at or past `bytes` read zero.  Word 3 is the gfx9 raw-buffer format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float *p) { return *p; }
  // four consecutive values; p must be 16-byte aligned
  static __device__ __forceinline__ void load4(const float *p, float *out) {
    const float4 x = *reinterpret_cast<const float4 *>(p);
    out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
  }
  static __device__ __forceinline__ float store_val(float f) { return f; }
  // four consecutive values in one store; p must be 16-byte aligned
  static __device__ __forceinline__ void store4(float *p, const float *v) {
    *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t *p) { return bf16_bits_to_f32(*p); }
  // four consecutive values; p must be 8-byte aligned
  static __device__ __forceinline__ void load4(const uint16_t *p, float *out) {
    const uint2 x = *reinterpret_cast<const uint2 *>(p);
    out[0] = __uint_as_float(x.x << 16); out[1] = __uint_as_float(x.x & 0xffff0000u);
    out[2] = __uint_as_float(x.y << 16); out[3] = __uint_as_float(x.y & 0xffff0000u);
  }
  static __device__ __forceinline__ uint16_t store_val(float f) { return f32_to_bf16_bits(f); }
  // four consecutive values in one store; p must be 8-byte aligned
  static __device__ __forceinline__ void store4(uint16_t *p, const float *v) {
    *reinterpret_cast<uint2 *>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  }
};

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2).
// Maps the hardware workgroup index of a 1-D grid of `grid` workgroups (a
// multiple of 8) to a logical index such that consecutive logical workgroups
// run on the same XCD and share its L2.
constexpr int kXcdCount = 8;
__device__ __forceinline__ long long xcd_logical_block(long long hw_block, long long grid) {
  return (hw_block % kXcdCount) * (grid / kXcdCount) + hw_block / kXcdCount;
}

// Exclusive prefix sum of one value per thread over the workgroup; `tmp`
// holds one word of LDS per wave.  Two barriers.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t x, uint32_t *tmp, int lane,
                                                         int wave) {
  uint32_t inc = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(inc, off);
    if (lane >= off) inc += y;
  }
  if (lane == 63) tmp[wave] = inc;
  __syncthreads();
  uint32_t before = 0;
  for (int w = 0; w < wave; ++w) before += tmp[w];
  __syncthreads();  // tmp may be reused after this
  return before + inc - x;
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also waits
// for every outstanding global load of the wave (its release fence covers all
// address spaces), which would drain register prefetches issued ahead of it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Sum of x over the lanes l ^ m for every m that is a multiple of kGroup
// below 64 (kGroup in {8, 16, 32}): lane-group reductions without LDS.
// xor 8 inside a 16-lane row is a DPP rotation by 8; xor 16 and xor 32 are
// the gfx950 permlane swaps, whose two results always add to the pair sum.
template <int kGroup>
__device__ __forceinline__ float sum_over_lane_groups(float x) {
  static_assert(kGroup == 8 || kGroup == 16 || kGroup == 32, "group width");
  if constexpr (kGroup <= 8)
    x += __uint_as_float(__builtin_amdgcn_mov_dpp(__float_as_uint(x), 0x128, 0xf, 0xf, false));
  if constexpr (kGroup <= 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace elsaa
