// Backward pass of the mixed scan: the passes that do not depend on the
// dtypes (reverse carry, reductions), the argument plan and the dispatch.
// Kernels of the dtype-dependent passes: scan_backward.hpp.
#include "scan_backward.hpp"

namespace swimba {
namespace bwd {

// ---------------------------------------------------------------- pass 3
// Incoming adjoint of every chunk, backward over chunks; one thread per
// (b, n, d).
__global__ __launch_bounds__(256) void bwd_reverse_carry_kernel(int B, int C, int D,
                                                                const float* __restrict__ P,
                                                                float* __restrict__ K,
                                                                const float* __restrict__ dhf,
                                                                float* __restrict__ dh0) {
  const size_t total = (size_t)B * kN * D;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int d = (int)(i % D);
  const int n = (int)((i / D) % kN);
  const int b = (int)(i / ((size_t)D * kN));
  const size_t stride = (size_t)kN * D;
  const size_t base = (size_t)b * C * stride + (size_t)n * D + d;
  float kap = dhf != nullptr ? dhf[((size_t)b * D + d) * kN + n] : 0.f;
  // chunks C-1 .. 0 in batches of 8, each batch's loads issued a batch ahead
  // of the current batch's stores (loads before chunk 0 read chunk 0, unused)
  constexpr int U8 = 8;
  float sd[U8], pc[U8];
  auto load_batch = [&](int c0, float* sb, float* pb) {
#pragma unroll
    for (int u = 0; u < U8; ++u) {
      const size_t o = base + (size_t)max(c0 - u, 0) * stride;
      sb[u] = K[o];
      pb[u] = P[o];
    }
  };
  load_batch(C - 1, sd, pc);
  for (int c0 = C - 1; c0 >= 0; c0 -= U8) {
    float sn[U8], pn[U8];
    load_batch(c0 - U8, sn, pn);
#pragma unroll
    for (int u = 0; u < U8; ++u) {
      if (c0 - u >= 0) {
        K[base + (size_t)(c0 - u) * stride] = kap;
        kap = fmaf(pc[u], kap, sd[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < U8; ++u) {
      sd[u] = sn[u];
      pc[u] = pn[u];
    }
  }
  if (dh0 != nullptr) dh0[((size_t)b * D + d) * kN + n] = kap;
}

int reverse_carry(const BwdParams& p, hipStream_t st) {
  const size_t total = (size_t)p.B * kN * p.D;
  hipLaunchKernelGGL(bwd_reverse_carry_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256),
                     0, st, p.B, p.nchunks, p.D, p.P, p.adj, p.dhf, p.dh0);
  return hipGetLastError() == hipSuccess ? SWIMBA_OK : SWIMBA_EHIP;
}

// ---------------------------------------------------------------- pass 5
// sum_w src[w * stride] for w = 0 .. n-1, added in that order; the loads are
// issued eight at a time so that one memory round trip serves eight terms.
__device__ __forceinline__ float ordered_sum(const float* __restrict__ src, size_t stride, int n) {
  float s = 0.f;
  int w = 0;
  for (; w + 8 <= n; w += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[(size_t)(w + u) * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; w < n; ++w) s += src[(size_t)w * stride];
  return s;
}

// dB, dC and dgate: the per-tile channel sums ([tile][token][R]: dB, dC,
// then the gate terms) added in tile order.
__global__ __launch_bounds__(256) void bwd_reduce_tokens_kernel(const float* __restrict__ red,
                                                                int ntiles, size_t tokens, int k,
                                                                int R, float* __restrict__ dB,
                                                                float* __restrict__ dC,
                                                                float* __restrict__ dgate) {
  const int W = 2 * kN + k;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= tokens * W) return;
  const size_t bt = i / W;
  const int col = (int)(i % W);
  const float s = ordered_sum(red + bt * R + col, tokens * R, ntiles);
  if (col < kN)
    dB[bt * kN + col] = s;
  else if (col < 2 * kN)
    dC[bt * kN + col - kN] = s;
  else
    dgate[bt * k + col - 2 * kN] = s;
}

// dA, dbias and dDskip: the per-(sequence, chunk) partials added in order.
__global__ __launch_bounds__(256) void bwd_reduce_params_kernel(const float* __restrict__ pA,
                                                                const float* __restrict__ pBD,
                                                                int slots, int E, int D,
                                                                float* __restrict__ dA,
                                                                float* __restrict__ dbias,
                                                                float* __restrict__ dDsk) {
  const size_t na = (size_t)E * D * kN, nb = (size_t)E * D;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < na) {
    dA[i] = ordered_sum(pA + i, na, slots);
  } else if (i < na + 2 * nb) {
    const size_t j = i - na;                  // [which][e][d]
    const int which = (int)(j / nb);
    const size_t ed = j % nb;
    const int e = (int)(ed / D), dd = (int)(ed % D);
    // pBD is [slot][E][2][D]: consecutive slots lie E * 2 * D floats apart
    (which == 0 ? dbias : dDsk)[ed] = ordered_sum(pBD + ((size_t)e * 2 + which) * D + dd,
                                                  (size_t)E * 2 * D, slots);
  }
}

int reduce_outputs(const BwdParams& p, float* dB, float* dC, float* dgate, float* dA,
                   float* dbias, float* dDsk, hipStream_t st) {
  const size_t tokens = (size_t)p.B * p.L;
  const size_t n1 = tokens * (2 * kN + p.k);
  hipLaunchKernelGGL(bwd_reduce_tokens_kernel, dim3((unsigned)((n1 + 255) / 256)), dim3(256), 0,
                     st, p.red, p.ntiles, tokens, p.k, backward_red_width(p.k), dB, dC, dgate);
  if (hipGetLastError() != hipSuccess) return SWIMBA_EHIP;
  const size_t n2 = (size_t)p.E * p.D * (kN + 2);
  hipLaunchKernelGGL(bwd_reduce_params_kernel, dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0,
                     st, p.pA, p.pBD, p.B * p.nchunks, p.E, p.D, dA, dbias, dDsk);
  return hipGetLastError() == hipSuccess ? SWIMBA_OK : SWIMBA_EHIP;
}

}  // namespace bwd
}  // namespace swimba
