// Dispatch of the mixed scan over (input dtype, output dtype) and the chunk
// carry pass shared with the separate design.  Kernels: scan_mixed.hpp.
#include "scan_mixed.hpp"

namespace swimba {
namespace mixed {

// Pass 2: carried-in state of every chunk, sequential over chunks.  One thread
// per (b, n, d); loads of the next chunks are issued ahead of the dependent
// chain.  There are few threads (16 D per sequence), so workgroups are one
// wave each and spread over every compute unit.
constexpr int kCarryThreads = 64;
__global__ __launch_bounds__(kCarryThreads) void mix_carry_kernel(int B, int C, int D, int E,
                                                        const float* __restrict__ P,
                                                        float* __restrict__ H,
                                                        float* __restrict__ h_final,
                                                        int separate) {
  // separate: the "n" axis spans E * 16 (one state per expert); rows of P/H are
  // [B][C][rows][D] with rows = 16 or E * 16
  const int rows = separate ? E * kN : kN;
  const size_t total = (size_t)B * rows * D;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int d = (int)(i % D);
  const int r = (int)((i / D) % rows);
  const int b = (int)(i / ((size_t)D * rows));
  const size_t stride = (size_t)rows * D;
  const size_t base = (size_t)b * C * stride + (size_t)r * D + d;
  float h = H[base];  // chunk 0 started from h0: its end state is exact
  // chunks 1 .. C-1 in batches of 16; each batch's loads are issued a batch
  // ahead, before the current batch's stores, so the chain waits for memory
  // once per batch.  Loads past chunk C-1 read chunk C-1 again (unused).
  constexpr int U8 = 16;
  float he[U8], pc[U8];
  auto load_batch = [&](int c0, float* hb, float* pb) {
#pragma unroll
    for (int u = 0; u < U8; ++u) {
      const size_t o = base + (size_t)min(c0 + u, C - 1) * stride;
      hb[u] = H[o];
      pb[u] = P[o];
    }
  };
  load_batch(1, he, pc);
  for (int c0 = 1; c0 < C; c0 += U8) {
    float hn[U8], pn[U8];
    load_batch(c0 + U8, hn, pn);
#pragma unroll
    for (int u = 0; u < U8; ++u) {
      if (c0 + u < C) {
        H[base + (size_t)(c0 + u) * stride] = h;
        h = fmaf(pc[u], h, he[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < U8; ++u) {
      he[u] = hn[u];
      pc[u] = pn[u];
    }
  }
  if (h_final != nullptr) {
    if (separate) {
      const int e = r / kN, n = r % kN;
      h_final[(((size_t)b * E + e) * D + d) * kN + n] = h;
    } else {
      h_final[((size_t)b * D + d) * kN + r] = h;
    }
  }
}

// Contraction check of the expert tables for the scans that read expert rows
// from memory: flags[tile] = 1 if any A[e, d, :] of the tile's 64 channels is
// not strictly negative (or NaN).  One workgroup of 1024 threads per tile;
// each thread issues all its loads (at most 16: E <= 64 experts x 64
// channels x 16 states = 16384 floats as 16-byte vectors, or 4096 scalars)
// before testing any, from clamped (valid) indices.  VEC: A is 16-byte
// aligned (diagonal A only).
constexpr int kFlagThreads = 1024;
template <bool VEC>
__global__ __launch_bounds__(kFlagThreads) void a_flags_kernel(const float* __restrict__ A, int E,
                                                                int D, int scalar_a,
                                                                int32_t* __restrict__ flags) {
  const int tile = blockIdx.x, d0 = tile * 64;
  const int nd = min(64, D - d0);
  const int tid = threadIdx.x;
  int bad = 0;
  if (VEC && !scalar_a) {
    // expert e's rows of the tile: nd * 16 contiguous floats = nd * 4 vectors
    const int r4 = nd * 4, total = E * r4;
    float4 v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int i = min(tid + j * kFlagThreads, total - 1);
      const int e = i / r4, r = i % r4;
      v[j] = reinterpret_cast<const float4*>(A + ((size_t)e * D + d0) * kN)[r];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j)
      bad |= !(v[j].x < 0.f) | !(v[j].y < 0.f) | !(v[j].z < 0.f) | !(v[j].w < 0.f);
  } else {
    // one float per (expert, channel) (scalar A) or per (expert, channel,
    // state): E * nd * per values, read 16 per thread per round
    const int per = scalar_a ? 1 : kN;
    const int total = E * nd * per;
    for (int base = 0; base < total; base += 16 * kFlagThreads) {
      float v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int i = min(base + tid + j * kFlagThreads, total - 1);
        const int e = i / (nd * per), r = i % (nd * per);
        v[j] = A[((size_t)e * D + d0) * per + r];
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) bad |= !(v[j] < 0.f);
    }
  }
  bad = __syncthreads_or(bad);
  if (tid == 0) flags[tile] = bad ? 1 : 0;
}

}  // namespace mixed

int launch_a_flags(const float* A, int E, int D, bool scalar_a, int32_t* flags, hipStream_t st) {
  const int ntiles = (D + 63) / 64;
  const bool vec = !scalar_a && (reinterpret_cast<uintptr_t>(A) & 15) == 0 && E <= 64;
  if (vec)
    hipLaunchKernelGGL(mixed::a_flags_kernel<true>, dim3((unsigned)ntiles),
                       dim3(mixed::kFlagThreads), 0, st, A, E, D, 0, flags);
  else
    hipLaunchKernelGGL(mixed::a_flags_kernel<false>, dim3((unsigned)ntiles),
                       dim3(mixed::kFlagThreads), 0, st, A, E, D, scalar_a ? 1 : 0, flags);
  return hipGetLastError() == hipSuccess ? SWIMBA_OK : SWIMBA_EHIP;
}

int launch_scan_ff(const swimba_scan_args*, const ScanPlan&, void*, hipStream_t);
int launch_scan_fb(const swimba_scan_args*, const ScanPlan&, void*, hipStream_t);
int launch_scan_bf(const swimba_scan_args*, const ScanPlan&, void*, hipStream_t);
int launch_scan_bb(const swimba_scan_args*, const ScanPlan&, void*, hipStream_t);

int launch_scan(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  const bool in_bf = a->in_dtype == SWIMBA_BF16, out_bf = a->y_dtype == SWIMBA_BF16;
  if (in_bf && out_bf) return launch_scan_bb(a, pl, ws, st);
  if (in_bf) return launch_scan_bf(a, pl, ws, st);
  if (out_bf) return launch_scan_fb(a, pl, ws, st);
  return launch_scan_ff(a, pl, ws, st);
}

// Shared with the separate design (same chunk-carry arithmetic per state row).
int launch_carry(int B, int C, int D, int E, const float* P, float* H, float* h_final,
                 int separate, hipStream_t st, const hipEvent_t* ev) {
  const size_t rows = separate ? (size_t)E * kN : kN;
  const size_t total = (size_t)B * rows * D;
  constexpr unsigned nt = mixed::kCarryThreads;
  return launch_timed(mixed::mix_carry_kernel, dim3((unsigned)((total + nt - 1) / nt)), dim3(nt),
                      0, st, ev, B, C, D, E, P, H, h_final, separate);
}

}  // namespace swimba
