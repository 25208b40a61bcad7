// C ABI of libswimba.so: argument validation, chunk planning and dispatch.
// No allocation, no synchronisation; every error is reported before launch.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>

#include "swimba.h"
#include "swimba_internal.hpp"

namespace swimba {

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];  // 0 = not yet queried

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

bool dtype_ok(swimba_dtype d) { return d == SWIMBA_F32 || d == SWIMBA_BF16; }

// Sizes and options only (enough for the workspace query).  `design`:
// 0 mixed, 1 separate (per expert), 2 separate per routing slot, 3 separate
// per expert with every expert advancing at every token.
int validate_scan(const swimba_scan_args* a, int design) {
  if (a == nullptr || design < 0 || design > 3) return SWIMBA_EINVAL;
  const bool separate = design == 1 || design == 3;
  if (a->B < 0 || a->L < 0 || a->D < 1 || a->N < 1 || a->E < 1 || a->k < 1 || a->k > a->E ||
      a->chunk < 0)
    return SWIMBA_EINVAL;
  if (!dtype_ok(a->in_dtype) || !dtype_ok(a->y_dtype)) return SWIMBA_EINVAL;
  if (a->carry != SWIMBA_CARRY_AUTO && a->carry != SWIMBA_CARRY_REWALK &&
      a->carry != SWIMBA_CARRY_FIXUP)
    return SWIMBA_EINVAL;
  if (a->a_form != SWIMBA_A_DIAGONAL && a->a_form != SWIMBA_A_SCALAR) return SWIMBA_EINVAL;
  if (a->disc != SWIMBA_DISC_EULER && a->disc != SWIMBA_DISC_ZOH) return SWIMBA_EINVAL;
  if (a->N != SWIMBA_STATE_N) return SWIMBA_EUNSUPPORTED;
  if (a->E > SWIMBA_MAX_EXPERTS) return SWIMBA_EUNSUPPORTED;
  // the per-slot scan stages up to 16 expert tables in LDS; beyond, it reads
  // the rows from memory with k <= 2
  if (design == 2 && a->E > 16 && a->k > 2) return SWIMBA_EUNSUPPORTED;
  // the mixed scan with more than 16 experts reads expert rows through 32-bit
  // buffer offsets
  if (design == 0 && a->E > 16 && (size_t)a->E * a->D * SWIMBA_STATE_N * 4 > 0x7fffffffu)
    return SWIMBA_EUNSUPPORTED;
  // per-slot scan: k x 16 states per lane in registers
  if (design == 2 && a->k > 4) return SWIMBA_EUNSUPPORTED;
  return SWIMBA_OK;
}

// Pointers the launch will dereference (the backward reads no y).
int validate_scan_pointers(const swimba_scan_args* a, bool need_y = true) {
  if (a->A == nullptr || a->dt_bias == nullptr || a->Dskip == nullptr) return SWIMBA_EINVAL;
  if (a->B > 0 && a->L > 0) {
    if (a->x == nullptr || a->dt_raw == nullptr || a->Bm == nullptr || a->Cm == nullptr ||
        a->idx == nullptr || a->gate == nullptr || (need_y && a->y == nullptr))
      return SWIMBA_EINVAL;
    // B_t and C_t rows are staged as 16-byte vectors
    if ((reinterpret_cast<uintptr_t>(a->Bm) & 15) || (reinterpret_cast<uintptr_t>(a->Cm) & 15))
      return SWIMBA_EINVAL;
  }
  return SWIMBA_OK;
}

}  // namespace

int stream_device(hipStream_t s) {
  int dev = -1;
  if (s != nullptr && hipStreamGetDevice(s, &dev) == hipSuccess) return dev;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  return dev;
}

int device_cus(int dev) {
  if (dev < 0 && hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev < 0 || dev >= kMaxDevices) return 256;
  int v = g_cus[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0)
      v = 256;
    g_cus[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

namespace {

// Tokens per chunk when the caller leaves the choice to the library, for a
// lane-per-channel scan over B * ntiles independent recurrences of length L.
// `small_ok`: the kernel may run the small-problem layout (two 4-wave
// workgroups per CU); *small tells whether it was chosen.
int auto_chunk(long long B, long long L, int ntiles, int E, bool separate, bool small_ok,
               bool* small, int dev) {
  const long long cus = device_cus(dev);
  const long long base = B * ntiles;
  long long want, min_chunk = 128;
  *small = false;
  if (separate) {
    // A workgroup per (sequence, tile, chunk) with one wave per expert (16
    // waves beyond 16 experts).  A CU holds about 20 such waves (five per
    // SIMD at the passes' register use) and the LDS of two workgroups, or of
    // ten with at most 4 experts (16-token rounds).  One chunk when the
    // (sequence, tile) workgroups fill those slots; else as many chunks as
    // fill them once.  The fix-up stops once every carried state has
    // decayed, which takes a number of selections per expert rather than of
    // tokens, so long chunks keep it a small part of the work.
    const long long per_cu = E <= 4 ? (20 / E < 10 ? 20 / E : 10) : (E > 10 ? 1 : 2);
    const long long slots = cus * per_cu;
    want = base >= slots ? 1 : slots / base;
    min_chunk = 256;
  } else if (base * (L / 256) >= 16 * cus) {
    // about four resident waves per SIMD (16 per CU) from the independent
    // (b, tile) recurrences, in chunks no shorter than a few fix-up horizons
    want = (16 * cus + base - 1) / base;
  } else {
    // Too few recurrences for that: two 4-wave workgroups per CU (two
    // waves per SIMD, every SIMD busy), i.e. the largest multiple of 4
    // chunks per tile whose workgroups all fit at once.
    *small = small_ok;
    want = 2 * 4 * cus / base;
    if (*small && want >= 4) want = want / 4 * 4;
    min_chunk = 64;
  }
  const long long maxc = (L + min_chunk - 1) / min_chunk;
  if (want > maxc) want = maxc;
  if (want < 1) want = 1;
  long long chunk = (L + want - 1) / want;
  if (separate) chunk = (chunk + 63) / 64 * 64;  // whole staging rounds
  return (int)chunk;
}

// Chunk count and the P / H (/ flags) workspace of a chunked scan whose
// chunk pass writes `rows` state rows per (sequence, chunk, channel).
void plan_layout(const ScanPlan& in, int B, int L, int D, int chunk, size_t rows, bool flags,
                 bool tflags, ScanPlan* p) {
  *p = in;
  if (chunk > L) chunk = L;
  p->chunk = chunk;
  p->nchunks = (int)(((long long)L + chunk - 1) / chunk);
  if (p->nchunks > 1) {
    const size_t arr = (size_t)B * p->nchunks * rows * D * sizeof(float);
    p->off_P = 0;
    p->off_H = align256(arr);
    p->off_flags = p->off_H + align256(arr);
    p->off_tflags = p->off_flags +
                    (flags ? align256((size_t)B * p->nchunks * p->ntiles * sizeof(int32_t)) : 0);
    p->bytes = p->off_tflags + (tflags ? align256((size_t)p->ntiles * sizeof(int32_t)) : 0);
  }
}

}  // namespace

int plan_scan(const swimba_scan_args* a, int design, ScanPlan* p, int dev) {
  int rc = validate_scan(a, design);
  if (rc != SWIMBA_OK) return rc;
  const bool separate = design == 1 || design == 3, slots = design == 2;
  ScanPlan q;
  q.ntiles = (a->D + 63) / 64;
  q.waves = (!separate && !slots && a->E > 8) ? 8 : 4;
  if (a->L == 0 || a->B == 0) {
    *p = q;
    return SWIMBA_OK;
  }
  bool small = false;  // mixed scan with too little work for four waves per SIMD
  const int chunk =
      a->chunk > 0 ? a->chunk
                   : auto_chunk(a->B, a->L, q.ntiles, a->E, separate,
                                slots || a->E <= 8 || a->E > 16, &small, dev);
  const size_t rows = separate ? (size_t)a->E * SWIMBA_STATE_N
                               : (slots ? (size_t)a->k * SWIMBA_STATE_N : SWIMBA_STATE_N);
  plan_layout(q, a->B, a->L, a->D, chunk, rows, true, !separate && a->E > 16, p);
  // chunks of one tile share the workgroup's expert table: 8 waves when there
  // are enough chunks to fill them (and the problem is not the small case)
  if (!separate && !slots && p->nchunks >= 8 && !small) p->waves = 8;
  return SWIMBA_OK;
}

int plan_backward(const swimba_scan_grad_args* g, BwdPlan* p, int dev) {
  if (g == nullptr) return SWIMBA_EINVAL;
  const swimba_scan_args* a = &g->fwd;
  ScanPlan sp;
  int rc = plan_scan(a, 0, &sp, dev);
  if (rc != SWIMBA_OK) return rc;
  if (!dtype_ok(g->dy_dtype)) return SWIMBA_EINVAL;
  if (a->a_form != SWIMBA_A_DIAGONAL || a->disc != SWIMBA_DISC_EULER) return SWIMBA_EUNSUPPORTED;
  // the backward's passes stage the E expert tables in LDS
  if (a->E > 16) return SWIMBA_EUNSUPPORTED;
  *p = BwdPlan();
  // four chunks (waves) per chunk-pass workgroup: at the small layers that
  // gives whole rounds of workgroups per CU (eight left half of the CUs with
  // one workgroup and half with two)
  p->waves = 4;
  if (backward_lds_bytes(a->E, a->k, p->waves) > 160 * 1024 ||
      backward_grad_lds_bytes(a->E, a->k) > 160 * 1024)
    return SWIMBA_EUNSUPPORTED;
  p->ntiles = sp.ntiles;
  if (a->B == 0 || a->L == 0) return SWIMBA_OK;
  // Own chunking (the forward is recomputed here): about four waves per SIMD
  // in the chunk pass (a wave per chunk), chunks of whole 8-token blocks and
  // at least 64 tokens; a caller's chunk size is kept.
  if (a->chunk > 0) {
    p->chunk = sp.chunk;
  } else {
    const long long cus = device_cus(dev);
    const long long base = (long long)a->B * sp.ntiles;
    long long want = (16 * cus + base - 1) / base;
    const long long maxc = (a->L + 63) / 64;
    if (want > maxc) want = maxc;
    if (want < 1) want = 1;
    const long long ch = (a->L + want - 1) / want;
    p->chunk = (int)((ch + 7) / 8 * 8);
  }
  p->nchunks = (int)(((long long)a->L + p->chunk - 1) / p->chunk);
  p->ncg = (p->nchunks + p->waves - 1) / p->waves;
  const size_t B = (size_t)a->B, L = (size_t)a->L, D = (size_t)a->D, E = (size_t)a->E;
  const size_t arr = B * p->nchunks * SWIMBA_STATE_N * D * sizeof(float);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align256(bytes);
    return at;
  };
  p->off_P = take(arr);
  p->off_H = take(arr);
  p->off_adj = take(arr);
  // checkpoints before every block of 8 tokens but a chunk's first: the
  // chunk pass's local state and its decay product since the chunk's start
  p->nbk = (p->chunk + 7) / 8 - 1;
  const size_t ck = B * p->nchunks * (size_t)p->nbk * SWIMBA_STATE_N * D * sizeof(float);
  p->off_ckH = take(ck);
  p->off_ckG = take(ck);
  p->off_red = take((size_t)p->ntiles * B * L * backward_red_width(a->k) * sizeof(float));
  p->off_pA = take(B * p->nchunks * E * D * SWIMBA_STATE_N * sizeof(float));
  p->off_pBD = take(B * p->nchunks * E * 2 * D * sizeof(float));
  p->bytes = o;
  return SWIMBA_OK;
}

int plan_streams(const swimba_stream_args* a, ScanPlan* p, int dev) {
  if (a == nullptr) return SWIMBA_EINVAL;
  if (a->B < 0 || a->L < 0 || a->D < 1 || a->N < 1 || a->k < 1 || a->chunk < 0)
    return SWIMBA_EINVAL;
  if (!dtype_ok(a->in_dtype) || !dtype_ok(a->y_dtype)) return SWIMBA_EINVAL;
  if (a->carry != SWIMBA_CARRY_AUTO && a->carry != SWIMBA_CARRY_REWALK &&
      a->carry != SWIMBA_CARRY_FIXUP)
    return SWIMBA_EINVAL;
  if (a->N != SWIMBA_STATE_N || a->k > 4) return SWIMBA_EUNSUPPORTED;
  ScanPlan q;
  q.ntiles = (a->D + 63) / 64;
  if (a->L == 0 || a->B == 0) {
    *p = q;
    return SWIMBA_OK;
  }
  // no expert table in LDS: every problem may take the small-problem layout
  bool small = false;
  const int chunk =
      a->chunk > 0 ? a->chunk : auto_chunk(a->B, a->L, q.ntiles, 1, false, true, &small, dev);
  plan_layout(q, a->B, a->L, a->D, chunk, SWIMBA_STATE_N, false, false, p);
  return SWIMBA_OK;
}

namespace {

__global__ void fill_initial_state(const float* h0, float* h, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) h[i] = h0 ? h0[i] : 0.f;
}

int empty_sequence(const swimba_scan_args* a, int design, hipStream_t s) {
  if (a->h_final == nullptr || a->B == 0) return SWIMBA_OK;
  // trajectories per (sequence, channel)
  const size_t per = (design == 1 || design == 3) ? a->E : (design == 2 ? a->k : 1);
  const size_t n = (size_t)a->B * per * a->D * SWIMBA_STATE_N;
  hipLaunchKernelGGL(fill_initial_state, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     a->h0, a->h_final, n);
  return hipGetLastError() == hipSuccess ? SWIMBA_OK : SWIMBA_EHIP;
}

int run_scan(const swimba_scan_args* a, void* ws, size_t ws_bytes, hipStream_t s, int design) {
  ScanPlan p;
  int rc = plan_scan(a, design, &p, stream_device(s));
  if (rc != SWIMBA_OK) return rc;
  rc = validate_scan_pointers(a);
  if (rc != SWIMBA_OK) return rc;
  if (p.bytes > 0) {
    if (ws == nullptr || ws_bytes < p.bytes || (reinterpret_cast<uintptr_t>(ws) & 255) != 0)
      return SWIMBA_EWORKSPACE;
  }
  if (a->B == 0 || a->L == 0) {
    if (a->phase_events)
      for (int i = 0; i < 6; ++i) (void)hipEventRecord(a->phase_events[i], s);
    return empty_sequence(a, design, s);
  }
  if (design == 1 || design == 3) return launch_scan_separate(a, p, ws, s, design == 3);
  if (design == 2) return launch_scan_slots(a, p, ws, s);
  return launch_scan(a, p, ws, s);
}

int run_streams(const swimba_stream_args* a, void* ws, size_t ws_bytes, hipStream_t s) {
  ScanPlan p;
  int rc = plan_streams(a, &p, stream_device(s));
  if (rc != SWIMBA_OK) return rc;
  if (a->A == nullptr || a->dt_bias == nullptr) return SWIMBA_EINVAL;
  // each lane reads its A row as 16-byte vectors
  if (reinterpret_cast<uintptr_t>(a->A) & 15) return SWIMBA_EINVAL;
  if (a->B > 0 && a->L > 0) {
    if (a->X == nullptr || a->dt_raw == nullptr || a->Bs == nullptr || a->Cs == nullptr ||
        a->gate == nullptr || a->y == nullptr)
      return SWIMBA_EINVAL;
    // B and C streams are staged as pairs of elements
    const uintptr_t pair = a->in_dtype == SWIMBA_BF16 ? 3 : 7;
    if ((reinterpret_cast<uintptr_t>(a->Bs) & pair) || (reinterpret_cast<uintptr_t>(a->Cs) & pair))
      return SWIMBA_EINVAL;
  }
  if (p.bytes > 0) {
    if (ws == nullptr || ws_bytes < p.bytes || (reinterpret_cast<uintptr_t>(ws) & 255) != 0)
      return SWIMBA_EWORKSPACE;
  }
  if (a->B == 0 || a->L == 0) {
    if (a->phase_events)
      for (int i = 0; i < 6; ++i) (void)hipEventRecord(a->phase_events[i], s);
    if (a->h_final == nullptr || a->B == 0) return SWIMBA_OK;
    const size_t n = (size_t)a->B * a->D * SWIMBA_STATE_N;
    hipLaunchKernelGGL(fill_initial_state, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       a->h0, a->h_final, n);
    return hipGetLastError() == hipSuccess ? SWIMBA_OK : SWIMBA_EHIP;
  }
  const bool in_bf = a->in_dtype == SWIMBA_BF16, out_bf = a->y_dtype == SWIMBA_BF16;
  if (in_bf && out_bf) return launch_streams_bb(a, p, ws, s);
  if (in_bf) return launch_streams_bf(a, p, ws, s);
  if (out_bf) return launch_streams_fb(a, p, ws, s);
  return launch_streams_ff(a, p, ws, s);
}

int run_backward(const swimba_scan_grad_args* g, void* ws, size_t ws_bytes, hipStream_t s) {
  BwdPlan p;
  int rc = plan_backward(g, &p, stream_device(s));
  if (rc != SWIMBA_OK) return rc;
  const swimba_scan_args* a = &g->fwd;
  if (a->A == nullptr || a->dt_bias == nullptr || a->Dskip == nullptr || g->dA == nullptr ||
      g->ddt_bias == nullptr || g->dDskip == nullptr)
    return SWIMBA_EINVAL;
  const bool work = a->B > 0 && a->L > 0;
  if (work) {
    rc = validate_scan_pointers(a, false);
    if (rc != SWIMBA_OK) return rc;
    if (g->dy == nullptr || g->dx == nullptr || g->ddt_raw == nullptr || g->dBm == nullptr ||
        g->dCm == nullptr || g->dgate == nullptr)
      return SWIMBA_EINVAL;
    if (ws == nullptr || ws_bytes < p.bytes || (reinterpret_cast<uintptr_t>(ws) & 255) != 0)
      return SWIMBA_EWORKSPACE;
  }
  if (!work) {
    // no tokens: the parameter gradients are zero and dh0 = dh_final
    const size_t na = (size_t)a->E * a->D * SWIMBA_STATE_N, nb = (size_t)a->E * a->D;
    hipLaunchKernelGGL(fill_initial_state, dim3((unsigned)((na + 255) / 256)), dim3(256), 0, s,
                       nullptr, g->dA, na);
    hipLaunchKernelGGL(fill_initial_state, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s,
                       nullptr, g->ddt_bias, nb);
    hipLaunchKernelGGL(fill_initial_state, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s,
                       nullptr, g->dDskip, nb);
    if (g->dh0 != nullptr && a->B > 0) {
      const size_t nh = (size_t)a->B * a->D * SWIMBA_STATE_N;
      hipLaunchKernelGGL(fill_initial_state, dim3((unsigned)((nh + 255) / 256)), dim3(256), 0,
                         s, g->dh_final, g->dh0, nh);
    }
    return hipGetLastError() == hipSuccess ? SWIMBA_OK : SWIMBA_EHIP;
  }
  const bool in_bf = a->in_dtype == SWIMBA_BF16, dy_bf = g->dy_dtype == SWIMBA_BF16;
  if (in_bf && dy_bf) return launch_backward_bb(g, p, ws, s);
  if (in_bf) return launch_backward_bf(g, p, ws, s);
  if (dy_bf) return launch_backward_fb(g, p, ws, s);
  return launch_backward_ff(g, p, ws, s);
}

// Chunk workspace of swimba_scan_noalloc: a fixed array in device memory,
// one copy per device, allocated with the code object and held until the
// process ends.  Host code never passes `scratch` itself to a kernel (its
// name is a host-side stand-in there): the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
constexpr size_t kScratchBytes = SWIMBA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::atomic<void*> g_scratch[kMaxDevices];  // nullptr = not yet looked up
std::mutex g_scratch_mu;

// Device address of `scratch` on device `dev`, or nullptr if HIP fails.
void* scratch_ptr(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  void* q = nullptr;
  const hipError_t e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
  if (cur != dev) (void)hipSetDevice(cur);
  if (e != hipSuccess || q == nullptr) return nullptr;
  g_scratch[dev].store(q, std::memory_order_release);
  return q;
}

int run_scan_noalloc(const swimba_scan_args* a, hipStream_t s) {
  const int dev = stream_device(s);
  ScanPlan p;
  const int rc = plan_scan(a, 0, &p, dev);
  if (rc != SWIMBA_OK) return rc;
  if (p.bytes > kScratchBytes) return SWIMBA_ESCRATCH;
  void* ws = nullptr;
  if (p.bytes > 0) {
    // the launch below needs valid arguments; look the buffer up only then
    const int prc = validate_scan_pointers(a);
    if (prc != SWIMBA_OK) return prc;
    ws = scratch_ptr(dev);
    if (ws == nullptr) return SWIMBA_EHIP;
  }
  return run_scan(a, ws, p.bytes > 0 ? kScratchBytes : 0, s, 0);
}

}  // namespace
}  // namespace swimba

using namespace swimba;

extern "C" {

int swimba_route(const void* x, swimba_dtype x_dtype, const float* Wr, int64_t T, int D, int E,
                 int k, int32_t* idx, float* gate, hipStream_t stream) {
  if (T < 0 || D < 1 || E < 1 || k < 1 || k > E || !dtype_ok(x_dtype)) return SWIMBA_EINVAL;
  if (E > SWIMBA_MAX_EXPERTS) return SWIMBA_EUNSUPPORTED;
  if (T == 0) return SWIMBA_OK;
  if (x == nullptr || Wr == nullptr || idx == nullptr || gate == nullptr) return SWIMBA_EINVAL;
  return launch_route(x, x_dtype, Wr, T, D, E, k, idx, gate, stream);
}

size_t swimba_scan_workspace_size(const swimba_scan_args* a, int design) {
  ScanPlan p;
  if (plan_scan(a, design, &p, -1) != SWIMBA_OK) return 0;
  return p.bytes;
}

int swimba_scan_plan(const swimba_scan_args* a, int design, int* chunk, int* nchunks) {
  ScanPlan p;
  const int rc = plan_scan(a, design, &p, -1);
  if (rc != SWIMBA_OK) return rc;
  if (chunk) *chunk = p.chunk;
  if (nchunks) *nchunks = p.nchunks;
  return SWIMBA_OK;
}

int swimba_scan(const swimba_scan_args* a, void* ws, size_t ws_bytes, hipStream_t stream) {
  return run_scan(a, ws, ws_bytes, stream, 0);
}

int swimba_scan_noalloc(const swimba_scan_args* a, hipStream_t stream) {
  return run_scan_noalloc(a, stream);
}

int swimba_scan_separate(const swimba_scan_args* a, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  return run_scan(a, ws, ws_bytes, stream, 1);
}

int swimba_scan_slots(const swimba_scan_args* a, void* ws, size_t ws_bytes, hipStream_t stream) {
  return run_scan(a, ws, ws_bytes, stream, 2);
}

int swimba_scan_all_experts(const swimba_scan_args* a, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  return run_scan(a, ws, ws_bytes, stream, 3);
}

size_t swimba_scan_backward_workspace_size(const swimba_scan_grad_args* g) {
  BwdPlan p;
  if (plan_backward(g, &p, -1) != SWIMBA_OK) return 0;
  return p.bytes;
}

int swimba_scan_backward(const swimba_scan_grad_args* g, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  return run_backward(g, ws, ws_bytes, stream);
}

size_t swimba_scan_streams_workspace_size(const swimba_stream_args* a) {
  ScanPlan p;
  if (plan_streams(a, &p, -1) != SWIMBA_OK) return 0;
  return p.bytes;
}

int swimba_scan_streams_plan(const swimba_stream_args* a, int* chunk, int* nchunks) {
  ScanPlan p;
  const int rc = plan_streams(a, &p, -1);
  if (rc != SWIMBA_OK) return rc;
  if (chunk) *chunk = p.chunk;
  if (nchunks) *nchunks = p.nchunks;
  return SWIMBA_OK;
}

int swimba_scan_streams(const swimba_stream_args* a, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  return run_streams(a, ws, ws_bytes, stream);
}

int swimba_step(const swimba_step_args* a, hipStream_t stream) {
  if (a == nullptr) return SWIMBA_EINVAL;
  if (a->B < 0 || a->D < 1 || a->N < 1 || a->E < 1 || a->k < 1 || a->k > a->E)
    return SWIMBA_EINVAL;
  if (!dtype_ok(a->in_dtype) || !dtype_ok(a->y_dtype)) return SWIMBA_EINVAL;
  if (a->a_form != SWIMBA_A_DIAGONAL && a->a_form != SWIMBA_A_SCALAR) return SWIMBA_EINVAL;
  if (a->disc != SWIMBA_DISC_EULER && a->disc != SWIMBA_DISC_ZOH) return SWIMBA_EINVAL;
  if (a->N != SWIMBA_STATE_N || a->E > SWIMBA_MAX_EXPERTS) return SWIMBA_EUNSUPPORTED;
  if (a->B == 0) return SWIMBA_OK;
  if (a->x == nullptr || a->dt_raw == nullptr || a->Bm == nullptr || a->Cm == nullptr ||
      a->A == nullptr || a->dt_bias == nullptr || a->Dskip == nullptr || a->state == nullptr ||
      a->y == nullptr)
    return SWIMBA_EINVAL;
  if (a->idx == nullptr && a->Wr == nullptr) return SWIMBA_EINVAL;
  if (a->idx != nullptr && a->gate == nullptr) return SWIMBA_EINVAL;
  // state (and a diagonal A) are read as 16-byte vectors
  if ((reinterpret_cast<uintptr_t>(a->state) & 15) ||
      (a->a_form == SWIMBA_A_DIAGONAL && (reinterpret_cast<uintptr_t>(a->A) & 15)))
    return SWIMBA_EINVAL;
  return launch_step(a, stream);
}

const char* swimba_status_string(int status) {
  switch (status) {
    case SWIMBA_OK:
      return "ok";
    case SWIMBA_EINVAL:
      return "invalid argument";
    case SWIMBA_EUNSUPPORTED:
      return "unsupported configuration";
    case SWIMBA_EWORKSPACE:
      return "workspace too small or not 256-byte aligned";
    case SWIMBA_EHIP:
      return "HIP launch failed";
    case SWIMBA_ESCRATCH:
      return "problem needs more workspace than the library's fixed scratch buffer holds";
    default:
      return "unknown status";
  }
}

}  // extern "C"
