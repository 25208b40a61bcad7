// Backward pass of the parameter-space-mixed scan for gfx950: the gradients
// of every input of swimba_scan given dL/dy (and dL/dh_final).
//
// Pages: "Swimba: Switch Mamba Model Scales State Space Models" (French
// summary, "Résultats Expérimentaux": the Swimba layers are trained, which
// needs these gradients) and "Mamba y las SSMs: el retorno del estado
// persistente" ("Mamba": the selective recurrence being differentiated).
//
// With lam_t = dL/dh_t, the adjoint runs backward in time,
//   lam_t = C_t dy_t + a_{t+1} lam_{t+1},
// and every gradient at token t is a product of lam_t, the state h_{t-1} and
// the token's own quantities.  The passes, all exact up to fp32 rounding:
//  1. chunk pass (forward in time, every chunk from zero state, chunk 0 from
//     h0): end state and decay P = prod a of each chunk as in the forward
//     scan, and the chunk's adjoint seed S_c = sum_t (prod_{s<=tau<=t} a_tau)
//     C_t dy_t -- the adjoint that the chunk alone sends to the token before
//     it, accumulated forward with a running product of the decays;
//  2. forward carry (shared kernel): carried-in state of every chunk;
//  3. reverse carry: incoming adjoint of every chunk, kappa_{c-1} =
//     P(c) kappa_c + S_c from kappa_last = dL/dh_final; dh0 = kappa_{-1};
//  4. gradient pass, one wave per chunk: walk the chunk forward from its
//     carried-in state writing every state h_t to the workspace, then walk it
//     backward from its incoming adjoint, reading h_{t-1}, and form the
//     gradients.  Per-channel gradients (dx, ddt_raw) are stored directly;
//     sums over channels (dB, dC, dgate) are reduced across the wave with a
//     lane butterfly and stored per 64-channel tile; per-expert parameter
//     gradients (dA, dbias, dDskip) are added into the workgroup's LDS
//     accumulators and stored per workgroup;
//  5. reductions over tiles and over workgroups, in a fixed order.
// The LDS accumulators take adds from the four waves of a workgroup in no
// fixed order, so dA, dbias and dDskip may differ between runs in the last
// bits; every other output is deterministic.
#pragma once
#include "scan_common.hpp"
#include "swimba_device.hpp"
#include "swimba_internal.hpp"

namespace swimba {
namespace bwd {

using stage::kTB;
using stage::Ring;
using stage::ring_bytes;
using stage::rsrc_t;
using stage::wave_sync;

constexpr int kRed = 2 * kN;  // dB and dC values per token in the tile sums

struct BwdParams {
  int B, L, D, E, k;
  int chunk, nchunks, ntiles, ncg;
  const void* x;
  const void* dt;
  const void* Bm;
  const void* Cm;
  const int32_t* idx;
  const float* gate;
  const float* A;
  const float* bias;
  const float* Dsk;
  const float* h0;
  const void* dy;
  const float* dhf;
  float* dx;      // [B][L][D]
  float* ddt;     // [B][L][D]
  float* dh0;     // [B][D][16] or null
  float* P;       // [B][C][16][D] chunk decays
  float* H;       // [B][C][16][D] chunk end states, then carried-in states
  float* adj;     // [B][C][16][D] adjoint seeds, then incoming adjoints
  float* hs;      // [B][L][D][16] states of the gradient pass
  float* red;     // [ntiles][B*L][kRed + k] per-tile channel sums
  float* pA;      // [B*ncg][E][D][16] per-workgroup dA
  float* pBD;     // [B*ncg][E][2][D] per-workgroup dbias, dDskip
};

// LDS of a workgroup: the tile's expert table, the per-wave rings and either
// the chunk pass's decay sums or the gradient pass's accumulators.
struct Smem {
  float4* A;      // [E][4][64]
  float2* BD;     // [E][64]
  float* U;       // chunk pass: [waves][E][64]
  float* accA;    // gradient pass: [E][16][64]
  float* accB;    // gradient pass: [E][2][64] (dbias, dDskip)
  Ring ring;
};

__host__ __device__ inline size_t table_bytes(int E) { return (size_t)E * (4 * 64 * 16 + 64 * 8); }
__host__ __device__ inline size_t extra_bytes(int E, bool grad, int waves) {
  return grad ? (size_t)E * (16 * 64 * 4 + 2 * 64 * 4) : (size_t)waves * E * 64 * 4;
}
__host__ inline size_t smem_bytes(int E, int k, bool grad, int waves) {
  return table_bytes(E) + extra_bytes(E, grad, waves) + ring_bytes(k) * waves;
}

__device__ __forceinline__ Smem smem_layout(int E, int k, bool grad, int waves, int wave) {
  extern __shared__ float4 smem_bwd[];
  char* p = reinterpret_cast<char*>(smem_bwd);
  Smem s;
  s.A = reinterpret_cast<float4*>(p);
  p += (size_t)E * 4 * 64 * 16;
  s.BD = reinterpret_cast<float2*>(p);
  p += (size_t)E * 64 * 8;
  s.U = reinterpret_cast<float*>(p);
  s.accA = reinterpret_cast<float*>(p);
  s.accB = reinterpret_cast<float*>(p + (size_t)E * 16 * 64 * 4);
  p += extra_bytes(E, grad, waves);
  p += ring_bytes(k) * wave;
  s.ring.bc = reinterpret_cast<float*>(p);
  s.ring.e = reinterpret_cast<int32_t*>(p + 2 * kTB * 32 * 4);
  s.ring.g = reinterpret_cast<float*>(p + 2 * kTB * 32 * 4 + 2 * kTB * k * 4);
  return s;
}

// Per-lane streamed rows of one block of kTB tokens: x, dt_raw and dy.
template <typename TIn, typename TDy>
struct BlockRows {
  TIn x[kTB], r[kTB];
  TDy g[kTB];
};

template <typename TIn, typename TDy>
__device__ __forceinline__ void load_rows(const BwdParams& p, size_t tok, int valid,
                                          uint32_t off_in, uint32_t off_dy, bool want_dy,
                                          BlockRows<TIn, TDy>& o) {
  const rsrc_t rx = stage::rows_rsrc<TIn>(p.x, tok, valid, p.D);
  const rsrc_t rr = stage::rows_rsrc<TIn>(p.dt, tok, valid, p.D);
  const rsrc_t rg = stage::rows_rsrc<TDy>(p.dy, tok, valid, p.D);
  const uint32_t row_in = (uint32_t)p.D * (uint32_t)sizeof(TIn);
  const uint32_t row_dy = (uint32_t)p.D * (uint32_t)sizeof(TDy);
#pragma unroll
  for (int i = 0; i < kTB; ++i) {
    // the scalar offset is not range-checked: rows past the end re-read the last
    const uint32_t ii = (uint32_t)min(i, valid - 1);
    o.x[i] = stage::buf_load<TIn>(rx, off_in, ii * row_in);
    o.r[i] = stage::buf_load<TIn>(rr, off_in, ii * row_in);
    if (want_dy) o.g[i] = stage::buf_load<TDy>(rg, off_dy, ii * row_dy);
  }
}

// Mixed parameters of one token for one lane: Delta, delta, beta, and the
// mixed transition Abar[n] (natural units).
template <int K>
struct Mix {
  float dlt, z, delta;
};

template <int K>
__device__ __forceinline__ Mix<K> mix_scalars(const Smem& s, const int* e, const float* gw, int k,
                                              int lane, float rv) {
  float beta = 0.f, delta = 0.f;
  const int kk = K > 0 ? K : k;
#pragma unroll
  for (int j = 0; j < (K > 0 ? K : 16); ++j) {
    if (K == 0 && j >= kk) break;
    const float2 bd = s.BD[e[j] * 64 + lane];
    beta = fmaf(gw[j], bd.x, beta);
    delta = fmaf(gw[j], bd.y, delta);
  }
  Mix<K> m;
  m.z = rv + beta;
  m.dlt = softplus_f32(m.z);
  m.delta = delta;
  return m;
}

template <int K>
__device__ __forceinline__ void mix_abar(const Smem& s, const int* e, const float* gw, int k,
                                         int lane, float* ab) {
#pragma unroll
  for (int n = 0; n < kN; ++n) ab[n] = 0.f;
  const int kk = K > 0 ? K : k;
#pragma unroll
  for (int j = 0; j < (K > 0 ? K : 16); ++j) {
    if (K == 0 && j >= kk) break;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 a = s.A[(e[j] * 4 + q) * 64 + lane];
      ab[4 * q + 0] = fmaf(gw[j], a.x, ab[4 * q + 0]);
      ab[4 * q + 1] = fmaf(gw[j], a.y, ab[4 * q + 1]);
      ab[4 * q + 2] = fmaf(gw[j], a.z, ab[4 * q + 2]);
      ab[4 * q + 3] = fmaf(gw[j], a.w, ab[4 * q + 3]);
    }
  }
}

__device__ __forceinline__ void read_routing(const Ring& ring, int slot, int i, int k, int* e,
                                             float* g, int kmax) {
  for (int j = 0; j < kmax; ++j) {
    if (j < k) {
      e[j] = ring.e[(slot * kTB + i) * k + j];
      g[j] = ring.g[(slot * kTB + i) * k + j];
    }
  }
}

// Wave sums of NV (a power of two, <= 64) values per lane, as a
// transpose-reduce: each exchange sends half of the remaining values to the
// partner lane and adds the half it receives, so the set halves per level.
// Afterwards v[0] of lane l holds the 64-lane sum of one value; for NV = 32
// that is value l >> 1.
template <int NV>
__device__ __forceinline__ void wave_transpose_sum(float* v, int lane) {
  int mask = 32;
#pragma unroll
  for (int cnt = NV; cnt > 1; cnt >>= 1, mask >>= 1) {
    const int half = cnt / 2;
    const bool upper = (lane & mask) != 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const float send = upper ? v[i] : v[half + i];
      const float keep = upper ? v[half + i] : v[i];
      v[i] = keep + __shfl_xor(send, mask, 64);
    }
  }
  for (; mask >= 1; mask >>= 1) v[0] += __shfl_xor(v[0], mask, 64);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Grid of the chunk and gradient passes: (sequence, chunk group, tile), tile
// fastest; wave w of a WAVES-wave workgroup takes chunk cg * WAVES + w.
struct Task {
  int b, cg, tile, c;
};
template <int WAVES>
__device__ __forceinline__ Task task(const BwdParams& p) {
  int bid = blockIdx.x;
  Task t;
  t.tile = bid % p.ntiles;
  bid /= p.ntiles;
  t.cg = bid % p.ncg;
  t.b = bid / p.ncg;
  t.c = t.cg * WAVES + uniform((int)(threadIdx.x >> 6));
  return t;
}

// ---------------------------------------------------------------- pass 1
template <typename TIn, typename TDy, int WAVES, int K>
__global__ __launch_bounds__(WAVES * 64) void bwd_chunk_kernel(BwdParams p) {
  const int lane = threadIdx.x & 63, wave = uniform((int)(threadIdx.x >> 6));
  const int k = K > 0 ? K : p.k;
  const Smem s = smem_layout(p.E, k, false, WAVES, wave);
  const Task tk = task<WAVES>(p);
  const int d0 = tk.tile * 64, d = d0 + lane;
  const bool active = d < p.D;
  int bad = stage::load_table(p, s.A, s.BD, d0, false);
  float* U = s.U + wave * p.E * 64;
  for (int e = 0; e < p.E; ++e) U[e * 64 + lane] = 0.f;
  bad = __syncthreads_or(bad);
  (void)bad;
  if (tk.c >= p.nchunks) return;  // no barrier below
  const int t0 = tk.c * p.chunk, t1 = min(p.L, t0 + p.chunk);
  const size_t row = (size_t)tk.b * p.L;
  const size_t total = (size_t)p.B * p.L;
  constexpr int KW = (kTB * (K > 0 ? K : 16) + 63) / 64;

  float h[kN], G[kN], S[kN];
#pragma unroll
  for (int n = 0; n < kN; ++n) {
    h[n] = (tk.c == 0 && p.h0 != nullptr && active) ? p.h0[((size_t)tk.b * p.D + d) * kN + n]
                                                    : 0.f;
    G[n] = 1.f;
    S[n] = 0.f;
  }
  const uint32_t off_in = active ? (uint32_t)d * (uint32_t)sizeof(TIn) : stage::kOffNone;
  const uint32_t off_dy = active ? (uint32_t)d * (uint32_t)sizeof(TDy) : stage::kOffNone;
  stage::Stager<TIn, KW> st;
  st.init(lane);
  auto valid_at = [&](int t) { return (int)min((size_t)kTB, total - (row + t)); };
  BlockRows<TIn, TDy> cur, nxt;
  int gate_bad = 0;
  st.issue(p, row + t0, valid_at(t0), k);
  load_rows<TIn, TDy>(p, row + t0, valid_at(t0), off_in, off_dy, true, cur);
  st.commit(s.ring, 0, min(kTB, t1 - t0), k, p.E, lane, gate_bad);
  int slot = 0;
  for (int tb = t0; tb < t1; tb += kTB, slot ^= 1) {
    const int n = min(kTB, t1 - tb), tn = tb + kTB;
    const bool more = tn < t1;
    if (more) {
      st.issue(p, row + tn, valid_at(tn), k);
      load_rows<TIn, TDy>(p, row + tn, valid_at(tn), off_in, off_dy, true, nxt);
    }
    wave_sync();
#pragma unroll
    for (int i = 0; i < kTB; ++i) {
      if (i >= n) break;
      int e[K > 0 ? K : 16];
      float gw[K > 0 ? K : 16];
      read_routing(s.ring, slot, i, k, e, gw, K > 0 ? K : 16);
      const float xv = active ? to_f32(cur.x[i]) : 0.f, rv = active ? to_f32(cur.r[i]) : 0.f;
      const float gy = active ? to_f32(cur.g[i]) : 0.f;
      const Mix<K> mx = mix_scalars<K>(s, e, gw, k, lane, rv);
      float ab[kN];
      mix_abar<K>(s, e, gw, k, lane, ab);
      const float dl2 = mx.dlt * kLog2e;
#pragma unroll
      for (int j = 0; j < (K > 0 ? K : 16); ++j) {
        if (j >= k) break;
        U[e[j] * 64 + lane] += dl2 * gw[j];
      }
      const float4* bc = reinterpret_cast<const float4*>(s.ring.bc + (slot * kTB + i) * 32);
      const float dx = mx.dlt * xv;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 b4 = bc[q], c4 = bc[4 + q];
        const float bv[4] = {b4.x, b4.y, b4.z, b4.w}, cv[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int nn = 4 * q + r;
          const float a = hw_exp2(dl2 * ab[nn]);
          h[nn] = fmaf(a, h[nn], dx * bv[r]);
          G[nn] *= a;
          S[nn] = fmaf(G[nn], cv[r] * gy, S[nn]);
        }
      }
    }
    if (more) {
      st.commit(s.ring, slot ^ 1, min(kTB, t1 - tn), k, p.E, lane, gate_bad);
      cur = nxt;
    }
  }
  if (!active) return;
  // chunk decay exp2(sum_e U_e A[e, d, n])
  float m[kN];
#pragma unroll
  for (int nn = 0; nn < kN; ++nn) m[nn] = 0.f;
  for (int e = 0; e < p.E; ++e) {
    const float u = U[e * 64 + lane];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 a = s.A[(e * 4 + q) * 64 + lane];
      m[4 * q + 0] = fmaf(u, a.x, m[4 * q + 0]);
      m[4 * q + 1] = fmaf(u, a.y, m[4 * q + 1]);
      m[4 * q + 2] = fmaf(u, a.z, m[4 * q + 2]);
      m[4 * q + 3] = fmaf(u, a.w, m[4 * q + 3]);
    }
  }
  const size_t base = (((size_t)tk.b * p.nchunks + tk.c) * kN) * p.D + d;
#pragma unroll
  for (int nn = 0; nn < kN; ++nn) {
    p.P[base + (size_t)nn * p.D] = hw_exp2(m[nn]);
    p.H[base + (size_t)nn * p.D] = h[nn];
    p.adj[base + (size_t)nn * p.D] = S[nn];
  }
}

// ---------------------------------------------------------------- pass 4
template <typename TIn, typename TDy, int WAVES, int K>
__global__ __launch_bounds__(WAVES * 64) void bwd_grad_kernel(BwdParams p) {
  const int lane = threadIdx.x & 63, wave = uniform((int)(threadIdx.x >> 6));
  const int k = K > 0 ? K : p.k;
  constexpr int KM = K > 0 ? K : 16;
  const Smem s = smem_layout(p.E, k, true, WAVES, wave);
  const Task tk = task<WAVES>(p);
  const int d0 = tk.tile * 64, d = d0 + lane;
  const bool active = d < p.D;
  stage::load_table(p, s.A, s.BD, d0, false);
  for (int i = threadIdx.x; i < p.E * (16 + 2) * 64; i += blockDim.x) s.accA[i] = 0.f;
  __syncthreads();

  if (tk.c < p.nchunks) {
    const int t0 = tk.c * p.chunk, t1 = min(p.L, t0 + p.chunk);
    const size_t row = (size_t)tk.b * p.L;
    const size_t total = (size_t)p.B * p.L;
    constexpr int KW = (kTB * KM + 63) / 64;
    const uint32_t off_in = active ? (uint32_t)d * (uint32_t)sizeof(TIn) : stage::kOffNone;
    const uint32_t off_dy = active ? (uint32_t)d * (uint32_t)sizeof(TDy) : stage::kOffNone;
    const int dd = active ? d : 0;
    auto valid_at = [&](int t) { return (int)min((size_t)kTB, total - (row + t)); };
    stage::Stager<TIn, KW> st;
    st.init(lane);
    int gate_bad = 0;
    const size_t cbase = (((size_t)tk.b * p.nchunks + tk.c) * kN) * p.D + dd;
    auto load_hin = [&](float* h) {
#pragma unroll
      for (int n = 0; n < kN; ++n) {
        float v = 0.f;
        if (active) {
          if (tk.c > 0)
            v = p.H[cbase + (size_t)n * p.D];
          else if (p.h0 != nullptr)
            v = p.h0[((size_t)tk.b * p.D + d) * kN + n];
        }
        h[n] = v;
      }
    };
    float4* hs4 = reinterpret_cast<float4*>(p.hs);

    // ---- forward: every state of the chunk, from its carried-in state
    float h[kN];
    load_hin(h);
    {
      BlockRows<TIn, TDy> cur, nxt;
      st.issue(p, row + t0, valid_at(t0), k);
      load_rows<TIn, TDy>(p, row + t0, valid_at(t0), off_in, off_dy, true, cur);
      st.commit(s.ring, 0, min(kTB, t1 - t0), k, p.E, lane, gate_bad);
      int slot = 0;
      for (int tb = t0; tb < t1; tb += kTB, slot ^= 1) {
        const int n = min(kTB, t1 - tb), tn = tb + kTB;
        const bool more = tn < t1;
        if (more) {
          st.issue(p, row + tn, valid_at(tn), k);
          load_rows<TIn, TDy>(p, row + tn, valid_at(tn), off_in, off_dy, true, nxt);
        }
        wave_sync();
#pragma unroll
        for (int i = 0; i < kTB; ++i) {
          if (i >= n) break;
          int e[KM];
          float gw[KM];
          read_routing(s.ring, slot, i, k, e, gw, KM);
          const float xv = active ? to_f32(cur.x[i]) : 0.f, rv = active ? to_f32(cur.r[i]) : 0.f;
          const Mix<K> mx = mix_scalars<K>(s, e, gw, k, lane, rv);
          float ab[kN];
          mix_abar<K>(s, e, gw, k, lane, ab);
          const float dl2 = mx.dlt * kLog2e, dx = mx.dlt * xv;
          const float4* bc = reinterpret_cast<const float4*>(s.ring.bc + (slot * kTB + i) * 32);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 b4 = bc[q];
            const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int nn = 4 * q + r;
              h[nn] = fmaf(hw_exp2(dl2 * ab[nn]), h[nn], dx * bv[r]);
            }
          }
          if (active) {
            float4* dst = hs4 + ((row + tb + i) * (size_t)p.D + d) * 4;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              dst[q] = make_float4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
          }
          // dC partials dy h_t, summed over the tile's channels
          const float gy = active ? to_f32(cur.g[i]) : 0.f;
          float v[kN];
#pragma unroll
          for (int nn = 0; nn < kN; ++nn) v[nn] = gy * h[nn];
          wave_transpose_sum<kN>(v, lane);
          if ((lane & 3) == 0) p.red[((size_t)tk.tile * total + row + tb + i) * (kRed + k) + kN +
                                     (lane >> 2)] = v[0];
        }
        if (more) {
          st.commit(s.ring, slot ^ 1, min(kTB, t1 - tn), k, p.E, lane, gate_bad);
          cur = nxt;
        }
      }
    }

    // ---- backward: blocks from the last, tokens from the last
    float mu[kN];
#pragma unroll
    for (int n = 0; n < kN; ++n) mu[n] = active ? p.adj[cbase + (size_t)n * p.D] : 0.f;
    const int nblk = (t1 - t0 + kTB - 1) / kTB;
    const int kr = kRed + k;
    float* red = p.red + (size_t)tk.tile * total * kr;
    BlockRows<TIn, TDy> cur;
    {
      const int tb = t0 + (nblk - 1) * kTB;
      st.issue(p, row + tb, valid_at(tb), k);
      load_rows<TIn, TDy>(p, row + tb, valid_at(tb), off_in, off_dy, true, cur);
      st.commit(s.ring, 0, min(kTB, t1 - tb), k, p.E, lane, gate_bad);
    }
    int slot = 0;
    for (int blk = nblk - 1; blk >= 0; --blk, slot ^= 1) {
      const int tb = t0 + blk * kTB;
      const int n = min(kTB, t1 - tb);
      const bool more = blk > 0;
      if (more) st.issue(p, row + tb - kTB, kTB, k);
      wave_sync();
#pragma unroll
      for (int ii = 0; ii < kTB; ++ii) {
        const int i = kTB - 1 - ii;
        if (i < n) {
        const int t = tb + i;
        const size_t bt = row + t;
        int e[KM];
        float gw[KM];
        read_routing(s.ring, slot, i, k, e, gw, KM);
        const float xv = active ? to_f32(cur.x[i]) : 0.f, rv = active ? to_f32(cur.r[i]) : 0.f;
        const float gy = active ? to_f32(cur.g[i]) : 0.f;
        // h_{t-1}
        float hp[kN];
        if (active && t > t0) {
          const float4* sp = hs4 + ((bt - 1) * (size_t)p.D + d) * 4;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 v = sp[q];
            hp[4 * q] = v.x;
            hp[4 * q + 1] = v.y;
            hp[4 * q + 2] = v.z;
            hp[4 * q + 3] = v.w;
          }
        } else {
          load_hin(hp);  // zeros on inactive lanes
        }
        float* rr = red + bt * kr;
        const Mix<K> mx = mix_scalars<K>(s, e, gw, k, lane, rv);
        const float dl2 = mx.dlt * kLog2e;
        const float dxs = mx.dlt * xv;
        const float4* bc = reinterpret_cast<const float4*>(s.ring.bc + (slot * kTB + i) * 32);
        float ab[kN], w[kN], vb[kN];
        mix_abar<K>(s, e, gw, k, lane, ab);
        float slb = 0.f, swa = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 b4 = bc[q], c4 = bc[4 + q];
          const float bv[4] = {b4.x, b4.y, b4.z, b4.w}, cv[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int nn = 4 * q + r;
            const float a = hw_exp2(dl2 * ab[nn]);
            const float lam = fmaf(cv[r], gy, mu[nn]);
            vb[nn] = lam * dxs;
            slb = fmaf(lam, bv[r], slb);
            w[nn] = lam * a * hp[nn];
            swa = fmaf(w[nn], ab[nn], swa);
            mu[nn] = a * lam;
          }
        }
        const float ddelta_dt = fmaf(xv, slb, swa);              // dL/dDelta
        const float sig = hw_exp2((mx.z - mx.dlt) * kLog2e);     // sigmoid(z)
        const float dz = ddelta_dt * sig;
        const float gyx = gy * xv;
        if (active) {
          p.dx[bt * p.D + d] = fmaf(mx.delta, gy, mx.dlt * slb);
          p.ddt[bt * p.D + d] = dz;
        }
        // per expert: dA += g Delta w, dbias, dDskip, and the gates' partials
        float dgp[KM];
#pragma unroll
        for (int j = 0; j < KM; ++j) {
          if (j >= k) break;
          const int ej = e[j];
          const float gd = gw[j] * mx.dlt;
          float sa = 0.f;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 a4 = s.A[(ej * 4 + q) * 64 + lane];
            const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int nn = 4 * q + r;
              sa = fmaf(av[r], w[nn], sa);
              __hip_atomic_fetch_add(&s.accA[(ej * kN + nn) * 64 + lane], gd * w[nn],
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
          }
          const float2 bd = s.BD[ej * 64 + lane];
          __hip_atomic_fetch_add(&s.accB[(ej * 2) * 64 + lane], gw[j] * dz, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WORKGROUP);
          __hip_atomic_fetch_add(&s.accB[(ej * 2 + 1) * 64 + lane], gw[j] * gyx,
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          dgp[j] = fmaf(bd.x, dz, fmaf(bd.y, gyx, mx.dlt * sa));
        }
        // dB partials over the tile's channels (inactive lanes hold zeros)
        wave_transpose_sum<kN>(vb, lane);
        if ((lane & 3) == 0) rr[lane >> 2] = vb[0];
        // the gates' sums over the tile's channels
#pragma unroll
        for (int j = 0; j < KM; ++j) {
          if (j >= k) break;
          const float sj = wave_sum(dgp[j]);
          if (lane == j) rr[kRed + j] = sj;
        }
        }
      }
      if (more) {
        st.commit(s.ring, slot ^ 1, kTB, k, p.E, lane, gate_bad);
        load_rows<TIn, TDy>(p, row + tb - kTB, kTB, off_in, off_dy, true, cur);
      }
    }
  }
  __syncthreads();
  // the workgroup's parameter-gradient partials
  const size_t slotwg = (size_t)tk.b * p.ncg + tk.cg;
  for (int i = threadIdx.x; i < p.E * kN * 64; i += blockDim.x) {
    const int e = i / (kN * 64), nn = (i / 64) % kN, l = i % 64;
    if (d0 + l < p.D)
      p.pA[((slotwg * p.E + e) * p.D + d0 + l) * kN + nn] = s.accA[(e * kN + nn) * 64 + l];
  }
  for (int i = threadIdx.x; i < p.E * 2 * 64; i += blockDim.x) {
    const int e = i / 128, w2 = (i / 64) % 2, l = i % 64;
    if (d0 + l < p.D) p.pBD[((slotwg * p.E + e) * 2 + w2) * p.D + d0 + l] = s.accB[i];
  }
}

// Passes 3 and 5 (scan_backward.hip): the reverse carry, and the reductions
// over tiles and workgroups into dB, dC, dgate, dA, dbias and dDskip.
int reverse_carry(const BwdParams& p, hipStream_t st);
int reduce_outputs(const BwdParams& p, float* dB, float* dC, float* dgate, float* dA,
                   float* dbias, float* dDsk, hipStream_t st);

template <typename TIn, typename TDy, int WAVES, int K>
int launch_bwd_t(const swimba_scan_grad_args* g, const BwdPlan& pl, void* ws, hipStream_t st) {
  const swimba_scan_args* a = &g->fwd;
  BwdParams p;
  p.B = a->B;
  p.L = a->L;
  p.D = a->D;
  p.E = a->E;
  p.k = a->k;
  p.chunk = pl.chunk;
  p.nchunks = pl.nchunks;
  p.ntiles = pl.ntiles;
  p.ncg = pl.ncg;
  p.x = a->x;
  p.dt = a->dt_raw;
  p.Bm = a->Bm;
  p.Cm = a->Cm;
  p.idx = a->idx;
  p.gate = a->gate;
  p.A = a->A;
  p.bias = a->dt_bias;
  p.Dsk = a->Dskip;
  p.h0 = a->h0;
  p.dy = g->dy;
  p.dhf = g->dh_final;
  p.dx = g->dx;
  p.ddt = g->ddt_raw;
  p.dh0 = g->dh0;
  char* w = static_cast<char*>(ws);
  p.P = reinterpret_cast<float*>(w + pl.off_P);
  p.H = reinterpret_cast<float*>(w + pl.off_H);
  p.adj = reinterpret_cast<float*>(w + pl.off_adj);
  p.hs = reinterpret_cast<float*>(w + pl.off_hs);
  p.red = reinterpret_cast<float*>(w + pl.off_red);
  p.pA = reinterpret_cast<float*>(w + pl.off_pA);
  p.pBD = reinterpret_cast<float*>(w + pl.off_pBD);

  const dim3 grid((unsigned)((size_t)p.B * p.ncg * p.ntiles)), block(WAVES * 64);
  const size_t smem1 = smem_bytes(p.E, p.k, false, WAVES);
  const size_t smem4 = smem_bytes(p.E, p.k, true, WAVES);
  allow_dynamic_lds(bwd_chunk_kernel<TIn, TDy, WAVES, K>, smem1);
  hipLaunchKernelGGL((bwd_chunk_kernel<TIn, TDy, WAVES, K>), grid, block, smem1, st, p);
  if (hipGetLastError() != hipSuccess) return SWIMBA_EHIP;
  int rc = launch_carry(p.B, p.nchunks, p.D, p.E, p.P, p.H, nullptr, 0, st, nullptr);
  if (rc != SWIMBA_OK) return rc;
  rc = reverse_carry(p, st);
  if (rc != SWIMBA_OK) return rc;
  allow_dynamic_lds(bwd_grad_kernel<TIn, TDy, WAVES, K>, smem4);
  hipLaunchKernelGGL((bwd_grad_kernel<TIn, TDy, WAVES, K>), grid, block, smem4, st, p);
  if (hipGetLastError() != hipSuccess) return SWIMBA_EHIP;
  return reduce_outputs(p, g->dBm, g->dCm, g->dgate, g->dA, g->ddt_bias, g->dDskip, st);
}

template <typename TIn, typename TDy, int WAVES>
int launch_bwd_w(const swimba_scan_grad_args* g, const BwdPlan& pl, void* ws, hipStream_t st) {
  switch (g->fwd.k) {
    case 1:
      return launch_bwd_t<TIn, TDy, WAVES, 1>(g, pl, ws, st);
    case 2:
      return launch_bwd_t<TIn, TDy, WAVES, 2>(g, pl, ws, st);
    default:
      return launch_bwd_t<TIn, TDy, WAVES, 0>(g, pl, ws, st);
  }
}

// Eight chunks (waves) share a workgroup's expert table and accumulators when
// the LDS allows it, four otherwise (E > 8).
template <typename TIn, typename TDy>
int launch_bwd_k(const swimba_scan_grad_args* g, const BwdPlan& pl, void* ws, hipStream_t st) {
  if (pl.waves == 8) return launch_bwd_w<TIn, TDy, 8>(g, pl, ws, st);
  return launch_bwd_w<TIn, TDy, 4>(g, pl, ws, st);
}

}  // namespace bwd
}  // namespace swimba
