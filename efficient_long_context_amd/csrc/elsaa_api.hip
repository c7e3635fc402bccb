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
#include <string.h>

#include <mutex>

#include "elsaa_internal.hpp"

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
  if (p->dtype != ELSAA_DTYPE_F32 && p->dtype != ELSAA_DTYPE_BF16)
    return fail(ELSAA_ERR_INVALID_ARG, "unknown dtype %d", static_cast<int>(p->dtype));
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

  g->B = p->B; g->H = p->H; g->N = p->N; g->D = p->d; g->DG = p->d_gate;
  g->ns = p->sort_bits; g->w = p->chunk; g->L = p->race_tables; g->P = p->race_bits;
  g->BH = static_cast<int>(BH);
  g->rows = BH * p->N;
  g->R = static_cast<int>(R);
  g->nb_sort = 1 << p->sort_bits;
  g->nb_race = 1 << p->race_bits;
  g->rcb = p->race_bits <= 8 ? 1 : 2;
  g->sort_tiles = (p->N + elsaa::kSortTile - 1) / elsaa::kSortTile;
  g->bf16 = p->dtype == ELSAA_DTYPE_BF16;
  g->lambda = p->lambda;
  g->cus = 256;
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
  t.hist = reinterpret_cast<uint32_t *>(take(2 * static_cast<size_t>(g.BH) * g.nb_sort * g.sort_tiles * 4));
  // per-table key permutation and run starts of the RACE build
  t.rperm = reinterpret_cast<int32_t *>(take(static_cast<size_t>(g.BH) * g.L * g.N * 4));
  t.rstart = reinterpret_cast<int32_t *>(take(static_cast<size_t>(g.BH) * g.L * (g.nb_race + 1) * 4));
  t.rpart = reinterpret_cast<int32_t *>(take(static_cast<size_t>(g.BH) * g.L * (elsaa::race_parts(g.N) + 1) * 8));
  t.tsum = take(static_cast<size_t>(g.BH) * g.L * g.nb_race * g.D * es);
  t.tcnt = reinterpret_cast<float *>(take(static_cast<size_t>(g.BH) * g.L * g.nb_race * 4));
  t.o_s = take(rows * g.D * es);
  t.lse = reinterpret_cast<float *>(take(rows * 4));
  if (b) *b = t;
  return off;
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
                    hipStream_t s) {
  const size_t rows = static_cast<size_t>(g.rows);
  const size_t es = g.bf16 ? 2 : 4;
  struct Item { void *dst; const void *src; size_t bytes; };
  const Item items[] = {
      {aux->sort_code_q, buf.scode, rows * 2},
      {aux->sort_code_k, buf.scode + rows, rows * 2},
      {aux->race_code_q, buf.rcode, rows * g.L * g.rcb},
      {aux->perm_q, buf.perm, rows * 4},
      {aux->perm_k, buf.perm + rows, rows * 4},
      {aux->race_sum, g.bf16 ? nullptr : buf.tsum, static_cast<size_t>(g.BH) * g.L * g.nb_race * g.D * 4},
      {aux->race_cnt, buf.tcnt, static_cast<size_t>(g.BH) * g.L * g.nb_race * 4},
      {aux->o_sparse, buf.o_s, rows * g.D * es},
      {aux->lse_s, buf.lse, rows * 4},
  };
  for (const Item &it : items) {
    if (!it.dst || !it.src) continue;
    const hipError_t e = hipMemcpyAsync(it.dst, it.src, it.bytes, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return e;
  }
  if (aux->race_code_k) {
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
  if (g.bf16 && aux->race_sum) {  // bfloat16 tables widen to the binary32 aux layout
    const long long n = static_cast<long long>(g.BH) * g.L * g.nb_race * g.D;
    hipLaunchKernelGGL(widen_bf16, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                       static_cast<const uint16_t *>(buf.tsum), aux->race_sum, n);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

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
  const int st = make_geometry(params, &g);
  if (st != ELSAA_OK) return st;
  if (!q || !k || !v || !x_gate || !out || (!hyperplanes && g.R > 0))
    return fail(ELSAA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  auto misaligned = [](const void *ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) != 0; };
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
  const size_t need = carve(g, nullptr, nullptr);
  if (!params->workspace || params->workspace_bytes < need)
    return fail(ELSAA_ERR_WORKSPACE, "workspace of %zu bytes required (given %zu%s)", need,
                params->workspace_bytes, params->workspace ? "" : ", NULL");
  if (misaligned(params->workspace, 256))
    return fail(ELSAA_ERR_WORKSPACE, "the workspace must be 256-byte aligned");
  elsaa::Buffers buf;
  carve(g, static_cast<char *>(params->workspace), &buf);
  hipStream_t s = static_cast<hipStream_t>(params->stream);

  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e == hipSuccess) e = device_cus(device, &g.cus);
  if (e != hipSuccess) return fail(ELSAA_ERR_DEVICE, "HIP error: %s", hipGetErrorString(e));

  // stage_events[2i] / [2i+1] bracket stage i (hash, sort, RACE build, chunk
  // attention, fusion)
  void *const *ev = params->stage_events;
  auto mark = [&](int i) -> hipError_t {
    return ev ? hipEventRecord(static_cast<hipEvent_t>(ev[i]), s) : hipSuccess;
  };
  e = mark(0);
  if (e == hipSuccess) e = elsaa::launch_hash(g, q, k, hyperplanes, buf, s);
  if (e == hipSuccess) e = mark(1);
  if (e == hipSuccess) e = mark(4);
  if (e == hipSuccess) e = elsaa::launch_race_build(g, v, buf, s);
  if (e == hipSuccess) e = mark(5);
  if (e == hipSuccess) e = mark(2);
  if (e == hipSuccess) e = elsaa::launch_sort(g, buf, s);
  if (e == hipSuccess) e = mark(3);
  if (e == hipSuccess) e = mark(6);
  if (e == hipSuccess) e = elsaa::launch_chunk_attention(g, q, k, v, buf, s);
  if (e == hipSuccess) e = mark(7);
  if (e == hipSuccess) e = mark(8);
  if (e == hipSuccess) e = elsaa::launch_fuse(g, x_gate, params->gate_w, params->gate_b, buf, params->aux, out, s);
  if (e == hipSuccess) e = mark(9);
  if (e == hipSuccess && params->aux) e = copy_aux(g, buf, params->aux, s);
  if (e != hipSuccess) return fail(ELSAA_ERR_DEVICE, "HIP error: %s", hipGetErrorString(e));
  g_last_error[0] = '\0';
  return ELSAA_OK;
}

}  // extern "C"
