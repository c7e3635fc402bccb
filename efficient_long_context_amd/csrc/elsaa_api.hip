// elsaa_api.hip -- host side of the C ABI declared in include/elsaa.h:
// validation, workspace layout and the launch sequence of the forward pass.
//
// Launch order (no host synchronisation), all on the caller's stream:
//   hash (q and k)  ->  RACE build (rank, gather)  ->  sort (hist, scan,
//   scatter; q and k)  ->  chunk attention  ->  RACE gather + gates + fusion
//   ->  optional aux copies.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "elsaa_internal.hpp"

// Scratch of elsaa_forward_noalloc: a fixed array in device memory, one copy
// per device (allocated when the code object is loaded on it, held until the
// process ends), shared by every call on that device.  Host code never uses
// the array's name as an address (on the host it is only a stand-in): the
// device address of each device's copy comes from hipGetSymbolAddress, taken
// once per device with that device current (device_scratch below).
static __device__ __align__(256) char scratch[ELSAA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Compute units of each device, queried once (the persistent kernels size
// their grids by it).
constexpr int kMaxDevices = 64;
std::mutex g_cus_mu;
int g_cus[kMaxDevices] = {0};

hipError_t device_cus(int device, int *cus) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_cus_mu);
  if (g_cus[device] == 0) {
    const hipError_t e = hipDeviceGetAttribute(&g_cus[device], hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess) return e;
  }
  *cus = g_cus[device];
  return hipSuccess;
}

// A second stream per device, for the sort to overlap the RACE build (they
// depend only on the hash; the sort keeps one workgroup per segment busy,
// 2 B H of them, far fewer than the compute units).  Created once per device
// at default priority; the fork and join events are reused, each call
// recording and waiting on them under the device's mutex (a wait binds to the
// event's latest record when it is enqueued).
struct SideStream {
  std::mutex mu;
  bool ready = false;
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
SideStream g_side[kMaxDevices];
std::mutex g_side_mu;

hipError_t side_stream(int device, SideStream **out) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_side_mu);
  SideStream &ss = g_side[device];
  if (!ss.ready) {
    hipError_t e = hipStreamCreateWithFlags(&ss.stream, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ss.join, hipEventDisableTiming);
    if (e != hipSuccess) return e;
    ss.ready = true;
  }
  *out = &ss;
  return hipSuccess;
}

// The integer a C caller stored in an enum field.  A value outside the enum's
// range is valid C but undefined to load as the C++ enum type, so the bits
// are copied out instead.
template <typename E>
int enum_bits(const E &e) {
  static_assert(sizeof(E) == sizeof(int), "enum fields are int-sized");
  int v;
  memcpy(&v, &e, sizeof(v));
  return v;
}

// Fills the geometry; returns ELSAA_OK or an error status with a message.
int make_geometry(const elsaa_params_t *p, elsaa::Geometry *g) {
  if (!p) return fail(ELSAA_ERR_INVALID_ARG, "params is NULL");
  if (p->B < 1 || p->H < 1 || p->N < 1)
    return fail(ELSAA_ERR_INVALID_ARG, "B, H, N must be >= 1 (got %d, %d, %d)", p->B, p->H, p->N);
  if (p->d < 1 || p->d_gate < 1)
    return fail(ELSAA_ERR_INVALID_ARG, "d and d_gate must be >= 1 (got %d, %d)", p->d, p->d_gate);
  if (p->chunk < 1 || p->N % p->chunk != 0)
    return fail(ELSAA_ERR_INVALID_ARG, "chunk must be >= 1 and divide N (chunk %d, N %d)", p->chunk, p->N);
  if (p->sort_bits < 0 || p->race_bits < 0 || p->race_tables < 1)
    return fail(ELSAA_ERR_INVALID_ARG, "sort_bits >= 0, race_bits >= 0, race_tables >= 1 required");
  if (!(p->lambda >= 0.0f) || !isfinite(p->lambda))
    return fail(ELSAA_ERR_INVALID_ARG, "lambda must be finite and >= 0");
  const int dtype = enum_bits(p->dtype), variant = enum_bits(p->variant);
  if (dtype != ELSAA_DTYPE_F32 && dtype != ELSAA_DTYPE_BF16)
    return fail(ELSAA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (variant < ELSAA_VARIANT_FULL || variant > ELSAA_VARIANT_SPARSE_ONLY)
    return fail(ELSAA_ERR_INVALID_ARG, "unknown variant %d", variant);
  if (!p->gate_w || !p->gate_b) return fail(ELSAA_ERR_INVALID_ARG, "gate_w / gate_b is NULL");
  // limits of this implementation
  if (p->d != 64 && p->d != 128) return fail(ELSAA_ERR_UNSUPPORTED, "d must be 64 or 128 (got %d)", p->d);
  if (p->d_gate > 512) return fail(ELSAA_ERR_UNSUPPORTED, "d_gate must be <= 512 (got %d)", p->d_gate);
  if (p->sort_bits > 12) return fail(ELSAA_ERR_UNSUPPORTED, "sort_bits must be <= 12 (got %d)", p->sort_bits);
  if (p->race_bits > 12) return fail(ELSAA_ERR_UNSUPPORTED, "race_bits must be <= 12 (got %d)", p->race_bits);
  if (p->race_tables > 64) return fail(ELSAA_ERR_UNSUPPORTED, "race_tables must be <= 64 (got %d)", p->race_tables);
  const long long R = static_cast<long long>(p->sort_bits) + static_cast<long long>(p->race_tables) * p->race_bits;
  if (R > 256) return fail(ELSAA_ERR_UNSUPPORTED, "sort_bits + race_tables * race_bits must be <= 256 (got %lld)", R);
  if ((static_cast<long long>(p->race_tables) << p->race_bits) > 16384)
    return fail(ELSAA_ERR_UNSUPPORTED, "race_tables * 2^race_bits must be <= 16384");
  if (p->chunk % 64 != 0) return fail(ELSAA_ERR_UNSUPPORTED, "chunk must be a multiple of 64 (got %d)", p->chunk);
  if (p->N > (1 << 24)) return fail(ELSAA_ERR_UNSUPPORTED, "N must be <= 2^24 (got %d)", p->N);
  const long long BH = static_cast<long long>(p->B) * p->H;
  if (BH > 32767) return fail(ELSAA_ERR_UNSUPPORTED, "B * H must be <= 32767 (got %lld)", BH);
  // The kernels address one head's rows (and one batch's gate inputs) through
  // 32-bit byte offsets and buffer resources with 32-bit sizes.
  const long long es = dtype == ELSAA_DTYPE_BF16 ? 2 : 4;
  const long long head_bytes = static_cast<long long>(p->N) * p->d * es;
  const long long gate_bytes = static_cast<long long>(p->N) * p->d_gate * es;
  if (head_bytes >= (1ll << 31) || gate_bytes >= (1ll << 31))
    return fail(ELSAA_ERR_UNSUPPORTED,
                "per-(b, h) tensors must be below 2^31 bytes (N * d * elem = %lld, N * d_gate * elem = %lld)",
                head_bytes, gate_bytes);

  g->B = p->B; g->H = p->H; g->N = p->N; g->D = p->d; g->DG = p->d_gate;
  g->ns = p->sort_bits; g->w = p->chunk; g->L = p->race_tables; g->P = p->race_bits;
  g->BH = static_cast<int>(BH);
  g->rows = BH * p->N;
  g->R = static_cast<int>(R);
  g->nb_sort = 1 << p->sort_bits;
  g->nb_race = 1 << p->race_bits;
  g->rcb = p->race_bits <= 8 ? 1 : 2;
  g->sort_tiles = (p->N + elsaa::kSortTile - 1) / elsaa::kSortTile;
  g->bf16 = dtype == ELSAA_DTYPE_BF16;
  g->lambda = variant == ELSAA_VARIANT_NO_ALPHA ? 0.0f : p->lambda;
  g->cus = 256;
  g->variant = variant;
  g->run_sparse = variant != ELSAA_VARIANT_RACE_ONLY;
  g->run_race = variant != ELSAA_VARIANT_SPARSE_ONLY;
  g->identity = p->sort_bits == 0;
  if (p->options & ~static_cast<uint32_t>(ELSAA_OPT_FUSED_EPILOGUE | ELSAA_OPT_SAVE_FOR_BACKWARD))
    return fail(ELSAA_ERR_INVALID_ARG, "unknown option bits 0x%x", p->options);
  g->fused = false;
  g->save = (p->options & ELSAA_OPT_SAVE_FOR_BACKWARD) != 0 && g->run_race;
  g->fused = (p->options & ELSAA_OPT_FUSED_EPILOGUE) != 0 && !g->save && elsaa::attention_fusable(*g);
  return ELSAA_OK;
}

// Workspace layout; with base == nullptr only the size is computed.
size_t carve(const elsaa::Geometry &g, char *base, elsaa::Buffers *b) {
  size_t off = 0;
  auto take = [&](size_t bytes) -> char * {
    char *ptr = base ? base + off : nullptr;
    off += align256(bytes);
    return ptr;
  };
  const size_t rows = static_cast<size_t>(g.rows);
  const size_t es = g.bf16 ? 2 : 4;
  elsaa::Buffers t;
  t.scode = reinterpret_cast<uint16_t *>(take(2 * rows * 2));
  t.rcode = take(2 * rows * g.L * g.rcb);
  t.perm = reinterpret_cast<int32_t *>(take(2 * rows * 4));
  t.flags = reinterpret_cast<uint8_t *>(take(2 * rows + 4));  // + one word: any row flagged
  // the sort's tile counts, and before them (the RACE build runs first) the
  // tiled RACE rank's
  // (the RACE build ranks and gathers over (b, h, token block) heads)
  const elsaa::Geometry gr = elsaa::race_block_geometry(g);
  const size_t rblocks = static_cast<size_t>(elsaa::race_blocks(g));
  const size_t sort_hist = 2 * static_cast<size_t>(g.BH) * g.nb_sort * g.sort_tiles * 4;
  const size_t race_hist = elsaa::race_hist_bytes(gr);
  t.hist = reinterpret_cast<uint32_t *>(take(sort_hist > race_hist ? sort_hist : race_hist));
  // per-table key permutation and run starts of the RACE build
  t.rperm = reinterpret_cast<int32_t *>(take(static_cast<size_t>(g.BH) * g.L * g.N * 4));
  t.rstart = reinterpret_cast<int32_t *>(take(static_cast<size_t>(gr.BH) * g.L * (g.nb_race + 1) * 4));
  t.rpart = reinterpret_cast<int32_t *>(take(static_cast<size_t>(gr.BH) * g.L * (elsaa::race_parts(gr.N) + 1) * 8));
  t.tsum = take(static_cast<size_t>(g.BH) * g.L * g.nb_race * g.D * es);
  t.tcnt = reinterpret_cast<float *>(take(static_cast<size_t>(g.BH) * g.L * g.nb_race * 4));
  t.psum = rblocks > 1 ? reinterpret_cast<float *>(take(g.BH * rblocks * g.L * g.nb_race * g.D * 4)) : nullptr;
  t.pcnt = rblocks > 1 ? reinterpret_cast<float *>(take(g.BH * rblocks * g.L * g.nb_race * 4)) : nullptr;
  // the sparse output and its LSE round-trip through memory unless the fusion
  // runs in the attention's epilogue
  t.o_s = g.fused ? nullptr : take(rows * g.D * es);
  t.lse = g.fused ? nullptr : reinterpret_cast<float *>(take(rows * 4));
  t.sv_olr = g.save ? take(rows * g.D * es) : nullptr;
  t.sv_z = g.save ? reinterpret_cast<float *>(take(rows * 4)) : nullptr;
  t.sv_gs = g.save ? reinterpret_cast<float *>(take(rows * 4)) : nullptr;
  t.sv_glr = g.save ? reinterpret_cast<float *>(take(rows * 4)) : nullptr;
  if (b) *b = t;
  return off;
}

// Backward scratch layout; with base == nullptr only the size is computed.
size_t carve_bwd(const elsaa::Geometry &g, char *base, elsaa::BackwardBuffers *b) {
  size_t off = 0;
  auto take = [&](size_t bytes) -> char * {
    char *ptr = base ? base + off : nullptr;
    off += align256(bytes);
    return ptr;
  };
  const size_t rows = static_cast<size_t>(g.rows);
  const size_t es = g.bf16 ? 2 : 4;
  const size_t tab = static_cast<size_t>(g.BH) * g.L * g.nb_race;
  elsaa::BackwardBuffers t;
  t.do_s = take(rows * g.D * es);
  t.delta = reinterpret_cast<float *>(take(rows * 4));
  t.dcon = take(rows * g.D * es);
  t.da_s = reinterpret_cast<float *>(take(rows * 4));
  t.da_lr = reinterpret_cast<float *>(take(rows * 4));
  t.dlam = reinterpret_cast<float *>(take(rows * 4));
  t.dv_acc = reinterpret_cast<float *>(take(rows * g.D * 4));
  t.qcode_t = take(rows * g.L * g.rcb);
  t.qrperm = take(static_cast<size_t>(g.BH) * g.L * g.N * 4);
  t.qhist = reinterpret_cast<uint32_t *>(take(elsaa::race_hist_bytes(g)));
  t.qrstart = reinterpret_cast<int32_t *>(take(static_cast<size_t>(g.BH) * g.L * (g.nb_race + 1) * 4));
  t.qrpart = reinterpret_cast<int32_t *>(take(static_cast<size_t>(g.BH) * g.L * (elsaa::race_parts(g.N) + 1) * 8));
  t.dT = take(tab * g.D * es);
  t.qtcnt = reinterpret_cast<float *>(take(tab * 4));
  t.gate_part = reinterpret_cast<float *>(take(static_cast<size_t>(g.H) * elsaa::kGateBlocks * (2 * g.DG + 3) * 4));
  t.flag = reinterpret_cast<uint32_t *>(take(4));
  if (b) *b = t;
  return off;
}

// Limits the backward adds to the forward's.
int backward_geometry(const elsaa_params_t *p, elsaa::Geometry *g) {
  const int st = make_geometry(p, g);
  if (st != ELSAA_OK) return st;
  if (g->fused)
    return fail(ELSAA_ERR_UNSUPPORTED,
                "the backward needs the forward's o_s and LSE: run the forward without ELSAA_OPT_FUSED_EPILOGUE");
  return ELSAA_OK;
}

__global__ void fill_zero_bytes(uint8_t *__restrict__ p, long long n) {
  const long long i = (static_cast<long long>(blockIdx.x) * 256 + threadIdx.x) * 16;
  if (i + 16 <= n) {
    *reinterpret_cast<elsaa::u32x4 *>(p + i) = (elsaa::u32x4){0u, 0u, 0u, 0u};
  } else {
    for (long long j = i; j < n; ++j) p[j] = 0;
  }
}

// perm[s][r] = r: the stable order of one bucket (sort_bits = 0).
__global__ void identity_perm(int32_t *__restrict__ perm, long long n, int N) {
  const long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) perm[i] = static_cast<int32_t>(i % N);
}

__global__ void widen_bf16(const uint16_t *__restrict__ src, float *__restrict__ dst, long long n) {
  const long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) dst[i] = elsaa::bf16_bits_to_f32(src[i]);
}

// Key RACE codes are kept table-major [L][rows]; the aux layout is [rows][L].
template <typename CT>
__global__ void codes_to_row_major(const CT *__restrict__ src, CT *__restrict__ dst, long long rows, int L) {
  const long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;  // destination element
  if (i < rows * L) dst[i] = src[(i % L) * rows + i / L];
}

hipError_t copy_aux(const elsaa::Geometry &g, const elsaa::Buffers &buf, const elsaa_aux_t *aux,
                    const void *out, hipStream_t s) {
  const size_t rows = static_cast<size_t>(g.rows);
  const size_t es = g.bf16 ? 2 : 4;
  const bool sp = g.run_sparse, rc = g.run_race;
  const bool sorted = sp && !g.identity;  // a sort ran: codes and permutations are in the workspace
  struct Item { void *dst; const void *src; size_t bytes; };
  const Item items[] = {
      {sorted ? aux->sort_code_q : nullptr, buf.scode, rows * 2},
      {sorted ? aux->sort_code_k : nullptr, buf.scode + rows, rows * 2},
      {rc ? aux->race_code_q : nullptr, buf.rcode, rows * g.L * g.rcb},
      {sorted ? aux->perm_q : nullptr, buf.perm, rows * 4},
      {sorted ? aux->perm_k : nullptr, buf.perm + rows, rows * 4},
      {rc ? aux->race_sum : nullptr, g.bf16 ? nullptr : buf.tsum,
       static_cast<size_t>(g.BH) * g.L * g.nb_race * g.D * 4},
      {rc ? aux->race_cnt : nullptr, buf.tcnt, static_cast<size_t>(g.BH) * g.L * g.nb_race * 4},
      // SPARSE_ONLY writes o_s as the output itself; the fused attention
      // writes these two aux outputs itself
      {sp && !g.fused ? aux->o_sparse : nullptr, rc ? buf.o_s : out, rows * g.D * es},
      {sp && !g.fused ? aux->lse_s : nullptr, buf.lse, rows * 4},
  };
  for (const Item &it : items) {
    if (!it.dst || !it.src) continue;
    const hipError_t e = hipMemcpyAsync(it.dst, it.src, it.bytes, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return e;
  }
  if (sp && g.identity) {  // one bucket: zero codes, identity permutations
    const long long n = g.rows;
    const dim3 grid(static_cast<unsigned>((n + 255) / 256));
    for (uint16_t *c : {aux->sort_code_q, aux->sort_code_k}) {
      if (!c) continue;
      const hipError_t e = elsaa::launch_fill_zero(c, rows * 2, s);
      if (e != hipSuccess) return e;
    }
    for (int32_t *pm : {aux->perm_q, aux->perm_k}) {
      if (!pm) continue;
      hipLaunchKernelGGL(identity_perm, grid, dim3(256), 0, s, pm, n, g.N);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (rc && aux->race_code_k) {
    const long long n = g.rows * g.L;
    const void *src = static_cast<const char *>(buf.rcode) + rows * g.L * g.rcb;
    if (g.rcb == 1)
      hipLaunchKernelGGL(codes_to_row_major<uint8_t>, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                         static_cast<const uint8_t *>(src), static_cast<uint8_t *>(aux->race_code_k), g.rows, g.L);
    else
      hipLaunchKernelGGL(codes_to_row_major<uint16_t>, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                         s, static_cast<const uint16_t *>(src), static_cast<uint16_t *>(aux->race_code_k), g.rows,
                         g.L);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (rc && g.bf16 && aux->race_sum) {  // bfloat16 tables widen to the binary32 aux layout
    const long long n = static_cast<long long>(g.BH) * g.L * g.nb_race * g.D;
    hipLaunchKernelGGL(widen_bf16, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                       static_cast<const uint16_t *>(buf.tsum), aux->race_sum, n);
    return hipGetLastError();
  }
  return hipSuccess;
}

// ELSAA_DEBUG (read once): synchronise and check after every stage.
bool debug_mode() {
  static const bool on = [] {
    const char *v = getenv("ELSAA_DEBUG");
    return v != nullptr && atoi(v) != 0;
  }();
  return on;
}

bool misaligned(const void *ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) != 0; }

int check_pointers(const elsaa::Geometry &g, const void *q, const void *k, const void *v, const void *x_gate,
                   const void *hyperplanes, const elsaa_params_t *params, const void *out);
int enqueue_forward(elsaa::Geometry &g, const void *q, const void *k, const void *v, const void *x_gate,
                    const void *hyperplanes, const elsaa_params_t *params, void *out, char *ws, SideStream *side);

constexpr size_t kNoAllocScratchBytes = ELSAA_NOALLOC_SCRATCH_BYTES;
std::mutex g_scratch_mu;
char *g_scratch[kMaxDevices] = {nullptr};

hipError_t device_scratch(int device, char **ptr) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[device]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[device] = static_cast<char *>(p);
  }
  *ptr = g_scratch[device];
  return hipSuccess;
}

}  // namespace

namespace elsaa {

hipError_t launch_fill_zero(void *p, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const long long pieces = static_cast<long long>((n + 15) / 16);
  hipLaunchKernelGGL(fill_zero_bytes, dim3(static_cast<unsigned>((pieces + 255) / 256)), dim3(256), 0, stream,
                     static_cast<uint8_t *>(p), static_cast<long long>(n));
  return hipGetLastError();
}

}  // namespace elsaa

extern "C" {

int elsaa_abi_version(void) { return ELSAA_ABI_VERSION; }

const char *elsaa_status_str(int status) {
  switch (status) {
    case ELSAA_OK: return "ELSAA_OK";
    case ELSAA_ERR_INVALID_ARG: return "ELSAA_ERR_INVALID_ARG";
    case ELSAA_ERR_UNSUPPORTED: return "ELSAA_ERR_UNSUPPORTED";
    case ELSAA_ERR_WORKSPACE: return "ELSAA_ERR_WORKSPACE";
    case ELSAA_ERR_DEVICE: return "ELSAA_ERR_DEVICE";
    default: return "ELSAA_ERR_UNKNOWN";
  }
}

const char *elsaa_last_error(void) { return g_last_error; }

int elsaa_validate(const elsaa_params_t *p) {
  elsaa::Geometry g;
  return make_geometry(p, &g);
}

size_t elsaa_workspace_bytes(const elsaa_params_t *p) {
  elsaa::Geometry g;
  if (make_geometry(p, &g) != ELSAA_OK) return 0;
  return carve(g, nullptr, nullptr);
}

int elsaa_forward(const void *q, const void *k, const void *v, const void *x_gate,
                  const void *hyperplanes, const elsaa_params_t *params, void *out) {
  elsaa::Geometry g;
  int st = make_geometry(params, &g);
  if (st == ELSAA_OK) st = check_pointers(g, q, k, v, x_gate, hyperplanes, params, out);
  if (st != ELSAA_OK) return st;
  const size_t need = carve(g, nullptr, nullptr);
  if (!params->workspace || params->workspace_bytes < need)
    return fail(ELSAA_ERR_WORKSPACE, "workspace of %zu bytes required (given %zu%s)", need,
                params->workspace_bytes, params->workspace ? "" : ", NULL");
  if (misaligned(params->workspace, 256))
    return fail(ELSAA_ERR_WORKSPACE, "the workspace must be 256-byte aligned");
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e == hipSuccess) e = device_cus(device, &g.cus);
  if (e != hipSuccess) return fail(ELSAA_ERR_DEVICE, "HIP error: %s", hipGetErrorString(e));
  // the sort overlaps the RACE build on the device's second stream when both
  // run and the sort needs no scratch the RACE build also uses (the tile
  // counts, shared by the tiled sort and the tiled RACE rank)
  SideStream *side = nullptr;
  const bool shared_hist =
      elsaa::sort_is_tiled(g) && elsaa::race_hist_bytes(elsaa::race_block_geometry(g)) > 0;
  if (g.run_sparse && g.run_race && !g.identity && !g.fused && !shared_hist && !debug_mode()) {
    e = side_stream(device, &side);
    if (e != hipSuccess) return fail(ELSAA_ERR_DEVICE, "HIP error: %s", hipGetErrorString(e));
  }
  return enqueue_forward(g, q, k, v, x_gate, hyperplanes, params, out, static_cast<char *>(params->workspace),
                         side);
}

size_t elsaa_backward_workspace_bytes(const elsaa_params_t *p) {
  elsaa::Geometry g;
  if (backward_geometry(p, &g) != ELSAA_OK) return 0;
  return carve_bwd(g, nullptr, nullptr);
}

int elsaa_backward(const void *q, const void *k, const void *v, const void *x_gate, const void *y,
                   const void *dy, const elsaa_params_t *params, void *bwd_workspace,
                   size_t bwd_workspace_bytes, void *dq, void *dk, void *dv, void *dx_gate,
                   float *dgate_w, float *dgate_b, float *dlambda) {
  elsaa::Geometry g;
  int st = backward_geometry(params, &g);
  if (st != ELSAA_OK) return st;
  if (!q || !k || !v || !x_gate || !dy || !dq || !dk || !dv || !dx_gate || !dgate_w || !dgate_b || !dlambda ||
      (!y && g.variant == ELSAA_VARIANT_SPARSE_ONLY))
    return fail(ELSAA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  for (const void *ptr : {q, k, v, x_gate, y, dy, static_cast<const void *>(dq), static_cast<const void *>(dk),
                          static_cast<const void *>(dv), static_cast<const void *>(dx_gate)})
    if (misaligned(ptr, 16)) return fail(ELSAA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (misaligned(params->gate_w, 4) || misaligned(params->gate_b, 4) || misaligned(dgate_w, 4) ||
      misaligned(dgate_b, 4) || misaligned(dlambda, 4))
    return fail(ELSAA_ERR_INVALID_ARG, "gate parameters and their gradients must be 4-byte aligned");
  const size_t need_fwd = carve(g, nullptr, nullptr);
  if (!params->workspace || params->workspace_bytes < need_fwd || misaligned(params->workspace, 256))
    return fail(ELSAA_ERR_WORKSPACE, "params->workspace must be the forward call's workspace (%zu bytes, 256-byte "
                "aligned)", need_fwd);
  const size_t need = carve_bwd(g, nullptr, nullptr);
  if (!bwd_workspace || bwd_workspace_bytes < need)
    return fail(ELSAA_ERR_WORKSPACE, "backward workspace of %zu bytes required (given %zu%s)", need,
                bwd_workspace_bytes, bwd_workspace ? "" : ", NULL");
  if (misaligned(bwd_workspace, 256)) return fail(ELSAA_ERR_WORKSPACE, "the backward workspace must be 256-byte aligned");
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e == hipSuccess) e = device_cus(device, &g.cus);
  if (e != hipSuccess) return fail(ELSAA_ERR_DEVICE, "HIP error: %s", hipGetErrorString(e));
  elsaa::Buffers fb;
  carve(g, static_cast<char *>(params->workspace), &fb);
  elsaa::BackwardBuffers bb;
  carve_bwd(g, static_cast<char *>(bwd_workspace), &bb);
  elsaa::BackwardInputs in{q, k, v, x_gate, y, dy, params->gate_w, params->gate_b, params->lambda};
  elsaa::BackwardOutputs out{dq, dk, dv, dx_gate, dgate_w, dgate_b, dlambda};
  hipStream_t s = static_cast<hipStream_t>(params->stream);
  e = elsaa::launch_backward(g, in, fb, bb, out, s);
  if (e == hipSuccess && debug_mode()) e = hipStreamSynchronize(s);
  if (e == hipSuccess && debug_mode()) e = hipGetLastError();
  if (e != hipSuccess) return fail(ELSAA_ERR_DEVICE, "HIP error in the backward pass: %s", hipGetErrorString(e));
  g_last_error[0] = '\0';
  return ELSAA_OK;
}

int elsaa_forward_noalloc(const void *q, const void *k, const void *v, const void *x_gate,
                          const void *hyperplanes, const elsaa_params_t *params, void *out) {
  elsaa::Geometry g;
  int st = make_geometry(params, &g);
  if (st == ELSAA_OK) st = check_pointers(g, q, k, v, x_gate, hyperplanes, params, out);
  if (st != ELSAA_OK) return st;
  const size_t need = carve(g, nullptr, nullptr);
  if (need > kNoAllocScratchBytes)
    return fail(ELSAA_ERR_WORKSPACE,
                "elsaa_forward_noalloc: the problem needs %zu bytes of scratch, above the fixed %zu "
                "(ELSAA_NOALLOC_SCRATCH_BYTES); use elsaa_forward with a workspace",
                need, kNoAllocScratchBytes);
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e == hipSuccess) e = device_cus(device, &g.cus);
  char *scratch_ptr = nullptr;
  if (e == hipSuccess) e = device_scratch(device, &scratch_ptr);
  if (e != hipSuccess) return fail(ELSAA_ERR_DEVICE, "HIP error: %s", hipGetErrorString(e));
  return enqueue_forward(g, q, k, v, x_gate, hyperplanes, params, out, scratch_ptr, nullptr);
}

}  // extern "C"

namespace {

int check_pointers(const elsaa::Geometry &g, const void *q, const void *k, const void *v, const void *x_gate,
                   const void *hyperplanes, const elsaa_params_t *params, const void *out) {
  if (!q || !k || !v || !x_gate || !out || (!hyperplanes && g.R > 0))
    return fail(ELSAA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(x_gate, 16) ||
      misaligned(hyperplanes, 16) || misaligned(out, 16))
    return fail(ELSAA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (misaligned(params->gate_w, 4) || misaligned(params->gate_b, 4))
    return fail(ELSAA_ERR_INVALID_ARG, "gate parameters must be 4-byte aligned");
  if (const elsaa_aux_t *a = params->aux) {
    const void *ptrs[] = {a->sort_code_q, a->sort_code_k, a->race_code_q, a->race_code_k, a->perm_q, a->perm_k,
                          a->race_sum, a->race_cnt, a->o_sparse, a->lse_s, a->z_lr, a->alpha, a->g_s, a->g_lr,
                          a->o_lowrank};
    for (const void *ptr : ptrs)
      if (misaligned(ptr, 16)) return fail(ELSAA_ERR_INVALID_ARG, "aux output pointers must be 16-byte aligned");
  }
  return ELSAA_OK;
}

// Enqueues every stage on params->stream with the scratch buffers carved out
// of `ws` (at least carve(g) bytes, 256-byte aligned).  With `side`, the sort
// runs on that stream between a fork after the hash and a join before the
// chunk attention, overlapping the RACE build.
int enqueue_forward(elsaa::Geometry &g, const void *q, const void *k, const void *v, const void *x_gate,
                    const void *hyperplanes, const elsaa_params_t *params, void *out, char *ws, SideStream *side) {
  elsaa::Buffers buf;
  carve(g, ws, &buf);
  hipStream_t s = static_cast<hipStream_t>(params->stream);
  hipError_t e = hipSuccess;

  // stage_events[2i] / [2i+1] bracket stage i (hash, sort, RACE build, chunk
  // attention, fusion); a stage a variant skips is an empty interval
  void *const *ev = params->stage_events;
  auto mark_on = [&](int i, hipStream_t st) -> hipError_t {
    return ev ? hipEventRecord(static_cast<hipEvent_t>(ev[i]), st) : hipSuccess;
  };
  auto mark = [&](int i) -> hipError_t { return mark_on(i, s); };
  std::unique_lock<std::mutex> side_lock;
  if (side) side_lock = std::unique_lock<std::mutex>(side->mu);
  const bool dbg = debug_mode();
  const char *stage = "";
  auto run = [&](const char *name, auto &&launch) {
    if (e != hipSuccess) return;
    stage = name;
    e = launch();
    if (e == hipSuccess && dbg) e = hipStreamSynchronize(s);
    if (e == hipSuccess && dbg) e = hipGetLastError();
  };
  // Planes of the stages that run: RACE_ONLY skips the sort planes, and
  // SPARSE_ONLY hashes only them (no RACE codes are made).
  elsaa::Geometry gh = g;
  const void *planes = hyperplanes;
  if (!g.run_sparse) {
    gh.ns = 0;
    gh.R = g.L * g.P;
    if (planes) planes = static_cast<const char *>(planes) + static_cast<size_t>(g.ns) * g.D * (g.bf16 ? 2 : 4);
  } else if (!g.run_race) {
    gh.L = 1;
    gh.P = 0;
    gh.rcb = 1;
    gh.R = g.ns;
  }
  const bool need_hash = g.run_race || !g.identity;
  e = mark(0);
  if (need_hash) run("hash", [&] { return elsaa::launch_hash(gh, q, k, planes, buf, s); });
  if (e == hipSuccess) e = mark(1);
  if (side) {  // fork: the sort on the side stream, after the hash
    if (e == hipSuccess) e = hipEventRecord(side->fork, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(side->stream, side->fork, 0);
    if (e == hipSuccess) e = mark_on(2, side->stream);
    run("sort", [&] { return elsaa::launch_sort(g, buf, side->stream); });
    if (e == hipSuccess) e = mark_on(3, side->stream);
    if (e == hipSuccess) e = hipEventRecord(side->join, side->stream);
  }
  if (e == hipSuccess) e = mark(4);
  if (g.run_race) run("RACE build", [&] { return elsaa::launch_race_build(g, v, buf, s); });
  if (e == hipSuccess) e = mark(5);
  if (side) {  // join
    if (e == hipSuccess) e = hipStreamWaitEvent(s, side->join, 0);
  } else {
    if (e == hipSuccess) e = mark(2);
    if (g.run_sparse && !g.identity) run("sort", [&] { return elsaa::launch_sort(g, buf, s); });
    if (e == hipSuccess) e = mark(3);
  }
  if (side_lock.owns_lock()) side_lock.unlock();
  if (e == hipSuccess) e = mark(6);
  if (g.fused)
    run("chunk attention + fusion", [&] {
      return elsaa::launch_attention_fused(g, q, k, v, x_gate, params->gate_w, params->gate_b, buf, params->aux,
                                           out, s);
    });
  else if (g.run_sparse)
    run("chunk attention",
        [&] { return elsaa::launch_chunk_attention(g, q, k, v, buf, g.run_race ? buf.o_s : out, s); });
  if (e == hipSuccess) e = mark(7);
  if (e == hipSuccess) e = mark(8);
  if (g.run_race && !g.fused)
    run("fusion",
        [&] { return elsaa::launch_fuse(g, x_gate, params->gate_w, params->gate_b, buf, params->aux, out, s); });
  if (e == hipSuccess) e = mark(9);
  if (params->aux) run("aux outputs", [&] { return copy_aux(g, buf, params->aux, out, s); });
  if (e != hipSuccess) return fail(ELSAA_ERR_DEVICE, "HIP error in stage '%s': %s", stage, hipGetErrorString(e));
  g_last_error[0] = '\0';
  return ELSAA_OK;
}

}  // namespace
