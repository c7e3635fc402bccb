/*
 * elsaa.h -- C ABI of the ELSAA attention forward pass on AMD Instinct MI355X
 * (gfx950).
 *
 * ELSAA ("ELSAA: Efficient Low-Rank and Sparse Attention Approximation for
 * Training Transformers", arxivlens summary, first paragraph; and "Two
 * Efficient Attentions, One Denominator Problem", section "Two efficient
 * branches can still be mis-scaled") combines, over already-formed dense
 * Q/K/V:
 *   - an exact sparse branch (here Sort-LSH: sign-random-projection hash of
 *     every query and key, stable sort by bucket, exact softmax attention of
 *     each chunk of w sorted queries over its own and the previous chunk of w
 *     sorted keys), which also yields the per-query log of its softmax mass
 *     Z_s;
 *   - a low-rank branch (RACE: keys scatter their values and a count into L
 *     hash tables of 2^P buckets; each query gathers the buckets it hashes to,
 *     giving a numerator and a collision-count mass Z_lr);
 *   - a denominator-aware fusion: alpha_i = Z_s,i / (Z_s,i + lambda Z_lr,i)
 *     scales the sparse output only, then independent token-wise sigmoid gates
 *     weight the two branches:  y_i = g_s,i alpha_i o_s,i + g_lr,i o_lr,i.
 *
 * Conventions
 *   - Every data pointer is a DEVICE pointer owned by the caller; the library
 *     allocates no memory.  Its only state is the compute-unit count of each
 *     device, queried on first use.
 *   - All tensors are dense, row-major, contiguous.  Tensor pointers (inputs,
 *     outputs and aux outputs) are 16-byte aligned, gate parameters 4-byte
 *     aligned, and the workspace 256-byte aligned (hipMalloc and PyTorch
 *     allocations are); a misaligned pointer is rejected (ELSAA_ERR_INVALID_ARG,
 *     or ELSAA_ERR_WORKSPACE for the workspace).
 *   - Work is enqueued on params->stream (a hipStream_t; NULL = the default
 *     stream) and is asynchronous: the caller synchronises before reading.
 *   - Every argument is validated on the host before the first launch; on an
 *     error the call returns a negative status and launches nothing.
 *   - elsaa_last_error() returns a message for the last failing call on the
 *     calling thread.
 *   - Calls that share a workspace must not overlap; calls with distinct
 *     workspaces may run concurrently on different streams.
 *   - NaN or Inf inputs propagate into the outputs; they are not trapped.
 *   - With the environment variable ELSAA_DEBUG set to a nonzero integer when
 *     the library is first called, elsaa_forward synchronises the stream after
 *     every stage and reports the first stage whose kernels failed
 *     (ELSAA_ERR_DEVICE, the stage named in elsaa_last_error()).  For
 *     debugging only: the calls then block, and must not be captured into a
 *     HIP graph.
 */
#ifndef ELSAA_H
#define ELSAA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ELSAA_ABI_VERSION 2

typedef enum {
  ELSAA_DTYPE_F32 = 0,  /* IEEE binary32                                     */
  ELSAA_DTYPE_BF16 = 1  /* bfloat16 (8-bit exponent, 7 stored fraction bits) */
} elsaa_dtype_t;

/* Which output the call produces.  The full operator and its three
 * single-mechanism relatives that the pages compare it with ("Two Efficient
 * Attentions, One Denominator Problem", sections "The ablation isolates the
 * actual contribution", "Workload structure matters more than a single
 * leaderboard" and "Length extrapolation is the strongest robustness
 * signal"): the ablation with the sparse multiplier fixed to one, a model
 * with the RACE branch alone and one with the sparse (Sort-LSH) branch alone.
 * A branch-only variant runs only the stages its branch needs. */
typedef enum {
  ELSAA_VARIANT_FULL = 0,        /* y = g_s alpha o_s + g_lr o_lr                   */
  ELSAA_VARIANT_NO_ALPHA = 1,    /* y = g_s o_s + g_lr o_lr (alpha fixed to 1)      */
  ELSAA_VARIANT_RACE_ONLY = 2,   /* y = o_lr: hash (RACE planes), RACE build and
                                    gather only; no sort, no chunk attention       */
  ELSAA_VARIANT_SPARSE_ONLY = 3  /* y = o_s: hash (sort planes), sort and chunk
                                    attention only; no RACE stages, no gates      */
} elsaa_variant_t;

enum {
  ELSAA_OK = 0,
  ELSAA_ERR_INVALID_ARG = -1, /* null pointer, bad size, bad lambda ...         */
  ELSAA_ERR_UNSUPPORTED = -2, /* valid for the method, outside what the kernels
                                 implement (see elsaa_params_t limits)          */
  ELSAA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required    */
  ELSAA_ERR_DEVICE = -4       /* a HIP launch or copy reported an error        */
};

/* Optional per-stage outputs, for tests and diagnostics.  Every member may be
 * NULL (not written).  Each non-NULL member is a device buffer of the stated
 * shape; writing them costs extra HBM traffic.  A branch-only variant leaves
 * the members of the stages it skips unwritten (RACE_ONLY: sort codes,
 * permutations, o_sparse, lse_s, alpha, g_s, g_lr; SPARSE_ONLY: RACE codes,
 * tables, z_lr, alpha, g_s, g_lr, o_lowrank).  With sort_bits = 0 the
 * permutations are the identity and the sort codes zero. */
typedef struct {
  uint16_t *sort_code_q;  /* [B][H][N]    Sort-LSH code of each query           */
  uint16_t *sort_code_k;  /* [B][H][N]    Sort-LSH code of each key             */
  void *race_code_q;      /* [B][H][N][L] RACE codes, uint8 if P <= 8 else uint16 */
  void *race_code_k;      /* [B][H][N][L]                                       */
  int32_t *perm_q;        /* [B][H][N]    sorted rank -> original query index   */
  int32_t *perm_k;        /* [B][H][N]    sorted rank -> original key index     */
  float *race_sum;        /* [B][H][L][2^P][d] per-bucket sums of values, as
                             stored: accumulated in binary32, then rounded once
                             to dtype (bfloat16 runs keep bfloat16 tables)       */
  float *race_cnt;        /* [B][H][L][2^P]    per-bucket key counts            */
  void *o_sparse;         /* [B][H][N][d] sparse-branch output, in dtype        */
  float *lse_s;           /* [B][H][N]    log Z_s (natural log)                 */
  float *z_lr;            /* [B][H][N]    low-rank mass Z_lr                    */
  float *alpha;           /* [B][H][N]    sparse multiplier                     */
  float *g_s;             /* [B][H][N]    sparse gate                           */
  float *g_lr;            /* [B][H][N]    low-rank gate                         */
  float *o_lowrank;       /* [B][H][N][d] low-rank branch output o_lr (fp32)    */
} elsaa_aux_t;

/* Problem description.  Limits of this implementation (outside them the call
 * returns ELSAA_ERR_UNSUPPORTED):
 *   d in {64, 128};  1 <= d_gate <= 512;
 *   0 <= sort_bits <= 12 (the sort keeps 2^sort_bits counters per wave in
 *   LDS);  0 <= race_bits <= 12;  1 <= race_tables <= 64;
 *   sort_bits + race_tables * race_bits <= 256 hyperplanes;
 *   race_tables * 2^race_bits <= 16384;
 *   chunk is a multiple of 64 (the attention kernels step over keys in
 *   blocks of 64) and divides N;  1 <= N <= 2^24;  B * H <= 32767;
 *   every per-(b, h) extent in bytes -- N * d * elem (q, k, v, out), N *
 *   d_gate * elem (x_gate of one b) -- is below 2^31 (the kernels address a
 *   head's rows with 32-bit offsets); for bfloat16 and d = 128 this is
 *   N < 2^23, for binary32 and d = 128 N < 2^22. */
typedef struct {
  int32_t B, H, N, d, d_gate;
  int32_t sort_bits;   /* n_s: bits of the Sort-LSH code (0 = one bucket)        */
  int32_t chunk;       /* w: chunk length in sorted order                        */
  int32_t race_tables; /* L: number of RACE hash tables                          */
  int32_t race_bits;   /* P: bits per RACE code (0 = one bucket per table)       */
  float lambda;        /* >= 0 and finite; 0 fixes the sparse multiplier to one */
  elsaa_dtype_t dtype; /* of q, k, v, x_gate, hyperplanes and out                */
  elsaa_variant_t variant; /* ELSAA_VARIANT_FULL for the operator itself         */
  const float *gate_w; /* device [2][H][d_gate]: [0] sparse gate, [1] low-rank   */
  const float *gate_b; /* device [2][H]                                           */
  void *workspace;     /* device scratch, >= elsaa_workspace_bytes(params) bytes */
  size_t workspace_bytes;
  void *stream;        /* hipStream_t; NULL = default stream                      */
  elsaa_aux_t *aux;    /* host pointer to optional outputs; NULL = none           */
  void *const *stage_events; /* host array of 10 hipEvent_t, or NULL.  Events
                        2i and 2i+1 are recorded just before and just after
                        stage i (0 hash, 1 sort, 2 RACE build, 3 chunk
                        attention, 4 gather/gates/fusion) on params->stream,
                        so elapsed(2i, 2i+1) times stage i.  The caller
                        creates and owns the events.                             */
  uint32_t options;    /* bit set of ELSAA_OPT_* (0 = defaults)                   */
} elsaa_params_t;

/* elsaa_params_t.options bits. */
enum {
  /* Run the RACE gather, gates and fusion in the epilogue of the chunk
   * attention, so the sparse output and its LSE never go to memory (the
   * workspace holds neither).  Applies to bfloat16, d = 64, chunk = 128, 8 or
   * 16 tables of P <= 8 bits, d_gate = 64, H <= 64 and ELSAA_VARIANT_FULL or
   * NO_ALPHA; elsewhere it is ignored.  Off by default: on MI355X its per-tile
   * table gathers run after the tile's attention instead of beside it, and the
   * two separate kernels are faster (see the design notes). */
  ELSAA_OPT_FUSED_EPILOGUE = 1u << 0,
  /* Training: the fusion also keeps, in the workspace, what the backward pass
   * would otherwise recompute with a second gather of the L table rows per
   * query: o_lr (in dtype) and per query the count sum, g_s and g_lr.  The
   * workspace grows by B H N (d elem + 12) bytes (elsaa_workspace_bytes
   * includes it); the forward writes that much more.  Takes precedence over
   * ELSAA_OPT_FUSED_EPILOGUE, which the backward cannot use. */
  ELSAA_OPT_SAVE_FOR_BACKWARD = 1u << 1
};

/* Host-only check of every field of *p except the device pointers' targets.
 * Returns ELSAA_OK or a negative status; never touches the device. */
int elsaa_validate(const elsaa_params_t *p);

/* Host-only: workspace bytes elsaa_forward needs for *p (0 if *p is invalid;
 * elsaa_validate says why).  Independent of p->workspace. */
size_t elsaa_workspace_bytes(const elsaa_params_t *p);

/* The forward pass.
 *   q, k, v     [B][H][N][d]      dtype
 *   x_gate      [B][N][d_gate]    dtype; one gate input per token, shared by heads
 *               (not read by the branch-only variants)
 *   hyperplanes [sort_bits + L*P][d] dtype; rows 0..sort_bits-1 are the Sort-LSH
 *               planes (row t gives code bit t, least significant first), then
 *               table l's P planes at rows sort_bits + l*P + t.  Shared by all
 *               (b, h); used for queries and keys alike.  May be NULL when
 *               sort_bits + L*P = 0.
 *   out         [B][H][N][d]      dtype, in original token order.
 * Hash bit semantics: bit = 1 iff the exact dot product of the stored vector
 * with the plane is > 0 (exact zero gives 0), independent of summation order.
 * Softmax scale 1/sqrt(d).  Chunk c (sorted ranks [c w, (c+1) w)) attends
 * sorted key ranks [max(0, (c-1) w), (c+1) w).  With sort_bits = 0 every
 * token shares one bucket, the stable order is the original one and the
 * sparse branch is local-window attention over consecutive tokens (the
 * local selection named beside LSH in the arxivlens summary's first
 * paragraph); the sort stage is then skipped and the kernels index tokens
 * directly.  Z_lr and the low-rank numerator
 * are means over the L tables; o_lr = 0 and alpha = 1 where Z_lr = 0.
 * Returns ELSAA_OK once every kernel is enqueued. */
int elsaa_forward(const void *q, const void *k, const void *v, const void *x_gate,
                  const void *hyperplanes, const elsaa_params_t *params, void *out);

/* Bytes of the fixed device scratch elsaa_forward_noalloc uses (64 MiB). */
#define ELSAA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * forward pass as elsaa_forward, with the same arguments, outputs and errors,
 * except that params->workspace and params->workspace_bytes are ignored.  Its
 * scratch is a fixed array of ELSAA_NOALLOC_SCRATCH_BYTES in device memory,
 * one per device, which the library holds from its load until the process
 * ends; the call itself allocates nothing.  A problem whose
 * elsaa_workspace_bytes() exceeds ELSAA_NOALLOC_SCRATCH_BYTES is rejected with
 * ELSAA_ERR_WORKSPACE before any device call.  Every call on a device shares
 * that device's array and no kernel relies on its previous contents: calls on
 * one device that overlap in time (concurrent streams, or host threads) race
 * on it and must be serialised by the caller. */
int elsaa_forward_noalloc(const void *q, const void *k, const void *v, const void *x_gate,
                          const void *hyperplanes, const elsaa_params_t *params, void *out);

/* Host-only: scratch bytes elsaa_backward needs for *p, beyond the forward's
 * workspace (0 if *p is invalid or outside the backward's limits;
 * elsaa_validate and elsaa_last_error say why). */
size_t elsaa_backward_workspace_bytes(const elsaa_params_t *p);

/* The backward pass, for training ("ELSAA: Efficient Low-Rank and Sparse
 * Attention Approximation for Training Transformers", first paragraph: a
 * training framework with a learnable lambda): given dy = dL/dy for the output
 * y of the elsaa_forward call made with the same inputs and *params, writes
 *   dq, dk, dv  [B][H][N][d]     dtype   dL/dq, dL/dk, dL/dv
 *   dx_gate     [B][N][d_gate]   dtype   dL/dx_gate
 *   dgate_w     [2][H][d_gate]   binary32, dgate_b [2][H] binary32, and
 *   *dlambda    one binary32 (dL/dlambda; 0 unless the variant is FULL).
 * Hash codes, permutations and bucket counts are constants (piecewise constant
 * in the inputs); the sparse branch recomputes its probabilities from the
 * stored LSE.  params->workspace must still hold that forward call's results
 * (nothing may run on it in between) and the forward must not have used
 * ELSAA_OPT_FUSED_EPILOGUE (which keeps o_s and the LSE out of memory):
 * otherwise ELSAA_ERR_UNSUPPORTED.  y is the forward's output (read only by
 * ELSAA_VARIANT_SPARSE_ONLY, whose o_s it is).  bwd_workspace is caller-owned
 * device scratch of at least elsaa_backward_workspace_bytes(params) bytes,
 * 256-byte aligned.  Every gradient is written (zeros where a variant has none); the
 * summation orders are fixed, so results repeat bit for bit.  Asynchronous on
 * params->stream like the forward; validation as in elsaa_forward. */
int elsaa_backward(const void *q, const void *k, const void *v, const void *x_gate, const void *y,
                   const void *dy, const elsaa_params_t *params, void *bwd_workspace,
                   size_t bwd_workspace_bytes, void *dq, void *dk, void *dv, void *dx_gate,
                   float *dgate_w, float *dgate_b, float *dlambda);

/* Static name of a status code ("ELSAA_OK", ...). */
const char *elsaa_status_str(int status);

/* Message describing the last failing call on this thread ("" if none). */
const char *elsaa_last_error(void);

/* ELSAA_ABI_VERSION of the loaded library. */
int elsaa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ELSAA_H */
