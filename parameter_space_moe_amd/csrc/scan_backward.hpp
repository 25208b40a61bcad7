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
//  4. state pass (a lane per channel, a wave per chunk): walk each chunk
//     forward from its carried-in state, store every state h_t to the
//     workspace, and sum dy_t h_t over the tile's channels (dC);
//  5. gradient pass (four lanes per channel, four states each; a workgroup
//     per (sequence, chunk, 64-channel tile)): walk the chunk backward from
//     its incoming adjoint, reading h_{t-1}, and form the gradients.
//     dx and ddt_raw are stored per channel; sums over channels (dB, dgate)
//     are reduced across the wave and stored per wave; the per-expert
//     parameter gradients (dA, dbias, dDskip) accumulate in registers over
//     all experts with each token's dense gate vector (zero for unselected
//     experts), branch-free, and are stored per (sequence, chunk);
//  6. reductions over tiles, waves and chunks, in a fixed order.
// Every output is deterministic.
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
  float* redC;    // [ntiles][B*L][16] per-tile sums of dy h_t
  float* redB;    // [ntiles*4][B*L][16 + k] per-wave sums of the dB terms and the gate terms
  float* pA;      // [B*C][E][D][16] per-(sequence, chunk) dA
  float* pBD;     // [B*C][E][2][D] per-(sequence, chunk) dbias, dDskip
};

// LDS of a chunk-pass or state-pass workgroup: the tile's expert table and
// the per-wave rings.
struct Smem {
  float4* A;      // [E][4][64]
  float2* BD;     // [E][64]
  Ring ring;
};

__host__ __device__ inline size_t table_bytes(int E) { return (size_t)E * (4 * 64 * 16 + 64 * 8); }
__host__ inline size_t smem_bytes(int E, int k, int waves) {
  return table_bytes(E) + ring_bytes(k) * waves;
}

__device__ __forceinline__ Smem smem_layout(int E, int k, int waves, int wave) {
  extern __shared__ float4 smem_bwd[];
  char* p = reinterpret_cast<char*>(smem_bwd);
  Smem s;
  s.A = reinterpret_cast<float4*>(p);
  p += (size_t)E * 4 * 64 * 16;
  s.BD = reinterpret_cast<float2*>(p);
  p += (size_t)E * 64 * 8;
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

// The same rows for a wave whose four lanes of a quad share one channel: lane
// q of the quad holds tokens q and q + 4 of the block, and the quad exchanges
// them through DPP broadcasts when they are used, so each lane keeps a quarter
// of the block in registers.
template <typename TIn, typename TDy>
struct QuadRows {
  static constexpr int kH = kTB / 4;
  TIn x[kH], r[kH];
  TDy g[kH];
};

template <typename TIn, typename TDy>
__device__ __forceinline__ void load_quad_rows(const BwdParams& p, size_t tok, int valid,
                                               bool active, int d, int q,
                                               QuadRows<TIn, TDy>& o) {
  const rsrc_t rx = stage::rows_rsrc<TIn>(p.x, tok, valid, p.D);
  const rsrc_t rr = stage::rows_rsrc<TIn>(p.dt, tok, valid, p.D);
  const rsrc_t rg = stage::rows_rsrc<TDy>(p.dy, tok, valid, p.D);
#pragma unroll
  for (int h = 0; h < QuadRows<TIn, TDy>::kH; ++h) {
    // rows past the block's valid ones are out of the buffer's range: 0
    const uint32_t ii = (uint32_t)(q + 4 * h);
    const uint32_t vin = active ? ((uint32_t)d + ii * (uint32_t)p.D) * (uint32_t)sizeof(TIn)
                                : stage::kOffNone;
    const uint32_t vdy = active ? ((uint32_t)d + ii * (uint32_t)p.D) * (uint32_t)sizeof(TDy)
                                : stage::kOffNone;
    o.x[h] = stage::buf_load<TIn>(rx, vin, 0);
    o.r[h] = stage::buf_load<TIn>(rr, vin, 0);
    o.g[h] = stage::buf_load<TDy>(rg, vdy, 0);
  }
}

// Token i of a QuadRows block, broadcast from the quad lane that holds it
// (quad_perm [s,s,s,s]; i is a constant once the token loop is unrolled).
// The half is chosen by a select, not an index: an index into the array
// before unrolling keeps the rows in scratch memory.
template <typename T>
__device__ __forceinline__ float quad_token(const T* v, int i) {
  static_assert(kTB == 8, "two tokens per quad lane");
  const float f = to_f32(i < 4 ? v[0] : v[1]);
  switch (i & 3) {
    case 0: return dpp_mov<0x00>(f);
    case 1: return dpp_mov<0x55>(f);
    case 2: return dpp_mov<0xAA>(f);
    default: return dpp_mov<0xFF>(f);
  }
}

// Mixed scalars of one token for one lane: Delta, its argument z, and delta
// (the mixed transition exponents come from mix_abar).
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

// ab[n] = sum_j w_j A[e_j, d, n] for one lane's channel d; the callers pass
// w_j = Delta log2(e) g_j, so ab is the exponent of the token's decays.
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
      if (mask == 32) {
        v[i] = xchg_add<32>(v[i], v[half + i]);
      } else if (mask == 16) {
        v[i] = xchg_add<16>(v[i], v[half + i]);
      } else {
        // take both values first: otherwise the compiler turns the two
        // selects into a lane-dependent index into v, i.e. a compare-and-
        // select chain over the whole array
        float lo = v[i], hi = v[half + i];
        asm("" : "+v"(lo), "+v"(hi));
        const float send = upper ? lo : hi;
        const float keep = upper ? hi : lo;
        v[i] = keep + xor_lane_any(send, mask, lane);
      }
    }
  }
  for (; mask >= 1; mask >>= 1) v[0] += xor_lane_any(v[0], mask, lane);
}

__device__ __forceinline__ float wave_sum(float v) { return wave_sum64(v); }

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
  const Smem s = smem_layout(p.E, k, WAVES, wave);
  const Task tk = task<WAVES>(p);
  const int d0 = tk.tile * 64, d = d0 + lane;
  const bool active = d < p.D;
  int bad = stage::load_table(p, s.A, s.BD, d0, false);
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
      // mixed exponents m[n] = sum_j (Delta log2(e) g_j) A[e_j, d, n]
      const float dl2 = mx.dlt * kLog2e;
      float u[K > 0 ? K : 16];
#pragma unroll
      for (int j = 0; j < (K > 0 ? K : 16); ++j) u[j] = dl2 * gw[j];
      float mexp[kN];
      mix_abar<K>(s, e, u, k, lane, mexp);
      const float4* bc = reinterpret_cast<const float4*>(s.ring.bc + (slot * kTB + i) * 32);
      const float dx = mx.dlt * xv;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 b4 = bc[q], c4 = bc[4 + q];
        const float bv[4] = {b4.x, b4.y, b4.z, b4.w}, cv[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int nn = 4 * q + r;
          const float a = hw_exp2(mexp[nn]);
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
  // the chunk decay P = prod_t a_t is the running product G
  const size_t base = (((size_t)tk.b * p.nchunks + tk.c) * kN) * p.D + d;
#pragma unroll
  for (int nn = 0; nn < kN; ++nn) {
    p.P[base + (size_t)nn * p.D] = G[nn];
    p.H[base + (size_t)nn * p.D] = h[nn];
    p.adj[base + (size_t)nn * p.D] = S[nn];
  }
}

// ---------------------------------------------------------------- pass 4
template <typename TIn, typename TDy, int WAVES, int K>
__global__ __launch_bounds__(WAVES * 64) void bwd_state_kernel(BwdParams p) {
  const int lane = threadIdx.x & 63, wave = uniform((int)(threadIdx.x >> 6));
  const int k = K > 0 ? K : p.k;
  constexpr int KM = K > 0 ? K : 16;
  const Smem s = smem_layout(p.E, k, WAVES, wave);
  const Task tk = task<WAVES>(p);
  const int d0 = tk.tile * 64, d = d0 + lane;
  const bool active = d < p.D;
  stage::load_table(p, s.A, s.BD, d0, false);
  __syncthreads();
  if (tk.c >= p.nchunks) return;  // no barrier below
  const int t0 = tk.c * p.chunk, t1 = min(p.L, t0 + p.chunk);
  const size_t row = (size_t)tk.b * p.L;
  const size_t total = (size_t)p.B * p.L;
  constexpr int KW = (kTB * KM + 63) / 64;
  const uint32_t off_in = active ? (uint32_t)d * (uint32_t)sizeof(TIn) : stage::kOffNone;
  const uint32_t off_dy = active ? (uint32_t)d * (uint32_t)sizeof(TDy) : stage::kOffNone;
  auto valid_at = [&](int t) { return (int)min((size_t)kTB, total - (row + t)); };
  stage::Stager<TIn, KW> st;
  st.init(lane);
  int gate_bad = 0;
  float h[kN];
  const size_t cbase = (((size_t)tk.b * p.nchunks + tk.c) * kN) * p.D + (active ? d : 0);
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
  float4* hs4 = reinterpret_cast<float4*>(p.hs);
  float* redC = p.redC + (size_t)tk.tile * total * kN;
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
      // mixed exponents m[n] = sum_j (Delta log2(e) g_j) A[e_j, d, n]
      const float dl2 = mx.dlt * kLog2e, dx = mx.dlt * xv;
      float u[KM];
#pragma unroll
      for (int j = 0; j < KM; ++j) u[j] = dl2 * gw[j];
      float mexp[kN];
      mix_abar<K>(s, e, u, k, lane, mexp);
      const float4* bc = reinterpret_cast<const float4*>(s.ring.bc + (slot * kTB + i) * 32);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 b4 = bc[q];
        const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int nn = 4 * q + r;
          h[nn] = fmaf(hw_exp2(mexp[nn]), h[nn], dx * bv[r]);
        }
      }
      const size_t bt = row + tb + i;
      // stored as [token][4][D] float4 (plane q: states 4q..4q+3), so that
      // each store of the wave covers 1 KiB of consecutive channels
      if (active) {
        float4* dst = hs4 + bt * 4 * (size_t)p.D + d;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          dst[(size_t)q * p.D] = make_float4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
      }
      // dC terms dy h_t, summed over the tile's channels
      const float gy = active ? to_f32(cur.g[i]) : 0.f;
      float v[kN];
#pragma unroll
      for (int nn = 0; nn < kN; ++nn) v[nn] = gy * h[nn];
      wave_transpose_sum<kN>(v, lane);
      if ((lane & 3) == 0) redC[bt * kN + (lane >> 2)] = v[0];
    }
    if (more) {
      st.commit(s.ring, slot ^ 1, min(kTB, t1 - tn), k, p.E, lane, gate_bad);
      cur = nxt;
    }
  }
}

// ---------------------------------------------------------------- pass 5
// LDS of the gradient pass: the tile's A as [E][64 channels][16] floats, the
// (dt_bias, Dskip) table [E][64], and per wave its ring plus the dense gate
// vectors of the ring's tokens ([2][kTB][EMAX]).
template <int EMAX>
__host__ __device__ inline size_t rev_smem_bytes(int E, int k) {
  return (size_t)E * 64 * 16 * 4 + (size_t)E * 64 * 8 +
         4 * (ring_bytes(k) + (size_t)2 * kTB * EMAX * 4);
}

template <typename TIn, typename TDy, int K, int EMAX>
__global__ __launch_bounds__(256) void bwd_grad_kernel(BwdParams p) {
  extern __shared__ float4 smem_rev[];
  const int lane = threadIdx.x & 63, wave = uniform((int)(threadIdx.x >> 6));
  const int k = K > 0 ? K : p.k;
  constexpr int KM = K > 0 ? K : 16;
  float* sA = reinterpret_cast<float*>(smem_rev);                    // [E][64][16]
  float2* sBD = reinterpret_cast<float2*>(sA + (size_t)p.E * 64 * 16);  // [E][64]
  char* wp = reinterpret_cast<char*>(sBD + (size_t)p.E * 64) +
             (ring_bytes(k) + (size_t)2 * kTB * EMAX * 4) * wave;
  float* ringG = reinterpret_cast<float*>(wp);  // [2][kTB][EMAX]
  char* rp = wp + (size_t)2 * kTB * EMAX * 4;
  Ring ring;
  ring.bc = reinterpret_cast<float*>(rp);
  ring.e = reinterpret_cast<int32_t*>(rp + 2 * kTB * 32 * 4);
  ring.g = reinterpret_cast<float*>(rp + 2 * kTB * 32 * 4 + 2 * kTB * k * 4);

  int bid = blockIdx.x;
  const int tile = bid % p.ntiles;
  bid /= p.ntiles;
  const int c = bid % p.nchunks;
  const int b = bid / p.nchunks;
  const int q = lane & 3, cl = wave * 16 + (lane >> 2);  // channel within the tile
  const int d0 = tile * 64, d = d0 + cl;
  const bool active = d < p.D;
  // the tile's tables (zeros past D)
  for (int i = threadIdx.x; i < p.E * 64 * 4; i += blockDim.x) {
    const int e = i / 256, dl = (i / 4) % 64, qq = i % 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (d0 + dl < p.D) v = *reinterpret_cast<const float4*>(p.A + ((size_t)e * p.D + d0 + dl) * kN + 4 * qq);
    reinterpret_cast<float4*>(sA)[i] = v;
  }
  for (int i = threadIdx.x; i < p.E * 64; i += blockDim.x) {
    const int e = i / 64, dl = i % 64;
    float2 v = make_float2(0.f, 0.f);
    if (d0 + dl < p.D) v = make_float2(p.bias[(size_t)e * p.D + d0 + dl], p.Dsk[(size_t)e * p.D + d0 + dl]);
    sBD[i] = v;
  }
  __syncthreads();

  const int t0 = c * p.chunk, t1 = min(p.L, t0 + p.chunk);
  const size_t row = (size_t)b * p.L;
  const size_t total = (size_t)p.B * p.L;
  constexpr int KW = (kTB * KM + 63) / 64;
  auto valid_at = [&](int t) { return (int)min((size_t)kTB, total - (row + t)); };
  stage::Stager<TIn, KW> st;
  st.init(lane);
  int gate_bad = 0;
  const size_t cbase = (((size_t)b * p.nchunks + c) * kN) * p.D + (active ? d : 0);
  float mu[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) mu[r] = active ? p.adj[cbase + (size_t)(4 * q + r) * p.D] : 0.f;
  // dA of every expert for this lane's four states; dbias and dDskip are the
  // same on the four lanes of a channel, so lane q keeps them for the experts
  // e = q, q + 4, ... only
  float accA[EMAX][4], accB[EMAX / 4][2];
#pragma unroll
  for (int e = 0; e < EMAX; ++e)
#pragma unroll
    for (int r = 0; r < 4; ++r) accA[e][r] = 0.f;
#pragma unroll
  for (int e4 = 0; e4 < EMAX / 4; ++e4) accB[e4][0] = accB[e4][1] = 0.f;
  // dense gate vectors of a committed ring slot: G[t][e] = sum of the gates
  // of the slots of token t that chose expert e
  auto dense_gates = [&](int sl) {
    wave_sync();
    for (int l = lane; l < kTB * EMAX; l += 64) {
      const int tt = l / EMAX, ee = l % EMAX;
      float gsum = 0.f;
      for (int j = 0; j < k; ++j)
        if (ring.e[(sl * kTB + tt) * k + j] == ee) gsum += ring.g[(sl * kTB + tt) * k + j];
      ringG[(sl * kTB + tt) * EMAX + ee] = gsum;
    }
  };
  const float4* hs4 = reinterpret_cast<const float4*>(p.hs);
  const int kr = kN + k;
  float* redB = p.redB + ((size_t)tile * 4 + wave) * total * kr;
  const int nblk = (t1 - t0 + kTB - 1) / kTB;
  QuadRows<TIn, TDy> cur, nxt;
  {
    const int tb = t0 + (nblk - 1) * kTB;
    st.issue(p, row + tb, valid_at(tb), k);
    load_quad_rows<TIn, TDy>(p, row + tb, valid_at(tb), active, d, q, cur);
    st.commit(ring, 0, min(kTB, t1 - tb), k, p.E, lane, gate_bad);
    dense_gates(0);
  }
  int slot = 0;
  for (int blk = nblk - 1; blk >= 0; --blk, slot ^= 1) {
    const int tb = t0 + blk * kTB;
    const int n = min(kTB, t1 - tb);
    const bool more = blk > 0;
    if (more) {
      st.issue(p, row + tb - kTB, kTB, k);
      load_quad_rows<TIn, TDy>(p, row + tb - kTB, kTB, active, d, q, nxt);
    }
    // this block's previous states h_{t-1}, all issued before the first is
    // used, without branches: the stored state of token t - 1 (the ragged
    // tail and channels past D read valid rows whose values go unused; the
    // latter have a zero adjoint); the chunk's first token then takes the
    // carried-in state
    float4 hpb[kTB];
    const int dq = active ? d : 0;
#pragma unroll
    for (int i = 0; i < kTB; ++i) {
      const int tp = max(min(tb + i, t1 - 1) - 1, 0);
      hpb[i] = hs4[((row + tp) * 4 + q) * (size_t)p.D + dq];
    }
    if (tb == t0) {  // the chunk's first block (wave-uniform)
      float4 hin = make_float4(0.f, 0.f, 0.f, 0.f);
      if (active && c > 0)
        hin = make_float4(p.H[cbase + (size_t)(4 * q) * p.D], p.H[cbase + (size_t)(4 * q + 1) * p.D],
                          p.H[cbase + (size_t)(4 * q + 2) * p.D],
                          p.H[cbase + (size_t)(4 * q + 3) * p.D]);
      else if (active && p.h0 != nullptr)
        hin = *reinterpret_cast<const float4*>(p.h0 + ((size_t)b * p.D + d) * kN + 4 * q);
      hpb[0] = hin;
    }
    wave_sync();
#pragma unroll
    for (int ii = 0; ii < kTB; ++ii) {
      const int i = kTB - 1 - ii;
      if (i < n) {
        const int t = tb + i;
        const size_t bt = row + t;
        int e[KM];
        float gw[KM];
        read_routing(ring, slot, i, k, e, gw, KM);
        // (inactive channels load zeros)
        const float xv = quad_token(cur.x, i), rv = quad_token(cur.r, i);
        const float gy = quad_token(cur.g, i);
        const float hp[4] = {hpb[i].x, hpb[i].y, hpb[i].z, hpb[i].w};
        // mixed per-channel parameters (the four lanes of a channel agree)
        float beta = 0.f, delta = 0.f;
#pragma unroll
        for (int j = 0; j < KM; ++j) {
          if (j < k) {
            const float2 bd = sBD[e[j] * 64 + cl];
            beta = fmaf(gw[j], bd.x, beta);
            delta = fmaf(gw[j], bd.y, delta);
          }
        }
        const float z = rv + beta;
        const float dlt = softplus_f32(z);
        const float dl2 = dlt * kLog2e, dxs = dlt * xv;
        const float4 b4 = reinterpret_cast<const float4*>(ring.bc + (slot * kTB + i) * 32)[q];
        const float4 c4 = reinterpret_cast<const float4*>(ring.bc + (slot * kTB + i) * 32)[4 + q];
        const float bv[4] = {b4.x, b4.y, b4.z, b4.w}, cv[4] = {c4.x, c4.y, c4.z, c4.w};
        float aj[KM][4];
#pragma unroll
        for (int j = 0; j < KM; ++j) {
          if (j < k) {
            const float4 a4 = reinterpret_cast<const float4*>(sA)[(e[j] * 64 + cl) * 4 + q];
            aj[j][0] = a4.x;
            aj[j][1] = a4.y;
            aj[j][2] = a4.z;
            aj[j][3] = a4.w;
          }
        }
        float w[4], vb[4], sa[KM];
#pragma unroll
        for (int j = 0; j < KM; ++j) sa[j] = 0.f;
        float slb = 0.f, swa = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float abn = 0.f;
#pragma unroll
          for (int j = 0; j < KM; ++j)
            if (j < k) abn = fmaf(gw[j], aj[j][r], abn);
          const float a = hw_exp2(dl2 * abn);
          const float lam = fmaf(cv[r], gy, mu[r]);
          vb[r] = lam * dxs;
          slb = fmaf(lam, bv[r], slb);
          w[r] = lam * a * hp[r];
          swa = fmaf(w[r], abn, swa);
#pragma unroll
          for (int j = 0; j < KM; ++j)
            if (j < k) sa[j] = fmaf(aj[j][r], w[r], sa[j]);
          mu[r] = a * lam;
        }
        // sums over the channel's four lanes
        slb += xor_lane<1>(slb, lane);
        slb += xor_lane<2>(slb, lane);
        swa += xor_lane<1>(swa, lane);
        swa += xor_lane<2>(swa, lane);
        const float dz = fmaf(xv, slb, swa) * hw_exp2((z - dlt) * kLog2e);  // dDelta sigmoid(z)
        const float gyx = gy * xv;
        if (active && q == 0) {
          p.dx[bt * p.D + d] = fmaf(delta, gy, dlt * slb);
          p.ddt[bt * p.D + d] = dz;
        }
        float* rr = redB + bt * kr;
        // per-expert parameter gradients, all experts, with the dense gates
        {
          const float4* G4 = reinterpret_cast<const float4*>(ringG + (slot * kTB + i) * EMAX);
#pragma unroll
          for (int e4 = 0; e4 < EMAX / 4; ++e4) {
            const float4 gv4 = G4[e4];
            const float gv[4] = {gv4.x, gv4.y, gv4.z, gv4.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int ee = 4 * e4 + u;
              const float gd = gv[u] * dlt;
#pragma unroll
              for (int r = 0; r < 4; ++r) accA[ee][r] = fmaf(gd, w[r], accA[ee][r]);
            }
            // this lane's expert of the group: e = 4 e4 + q
            const float gq = q == 0 ? gv[0] : (q == 1 ? gv[1] : (q == 2 ? gv[2] : gv[3]));
            accB[e4][0] = fmaf(gq, dz, accB[e4][0]);
            accB[e4][1] = fmaf(gq, gyx, accB[e4][1]);
          }
        }
#pragma unroll
        for (int j = 0; j < KM; ++j) {
          if (j < k) {
            const float2 bd = sBD[e[j] * 64 + cl];
            const float part = fmaf(dlt, sa[j], q == 0 ? fmaf(bd.x, dz, bd.y * gyx) : 0.f);
            const float sj = wave_sum(part);
            if (lane == j) rr[kN + j] = sj;
          }
        }
        // dB terms summed over the wave's 16 channels: lanes of equal q hold
        // the same states; after two halving exchanges (masks 32, 16) and two
        // sums (8, 4) lane l holds state 4q + 2 bit5 + bit4
        {
          int mask = 32;
#pragma unroll
          for (int cnt = 4; cnt > 1; cnt >>= 1, mask >>= 1) {
            const int half = cnt / 2;
            const bool upper = (lane & mask) != 0;
#pragma unroll
            for (int r = 0; r < half; ++r) {
              // masks 32 and 16 only: the lane swap exchanges
              (void)upper;
              vb[r] = mask == 32 ? xchg_add<32>(vb[r], vb[half + r])
                                 : xchg_add<16>(vb[r], vb[half + r]);
            }
          }
          vb[0] += xor_lane<8>(vb[0], lane);
          vb[0] += xor_lane<4>(vb[0], lane);
          if ((lane & 12) == 0) rr[4 * q + 2 * ((lane >> 5) & 1) + ((lane >> 4) & 1)] = vb[0];
        }
      }
    }
    if (more) {
      st.commit(ring, slot ^ 1, kTB, k, p.E, lane, gate_bad);
      dense_gates(slot ^ 1);
      cur = nxt;
    }
  }
  // per-(sequence, chunk) parameter-gradient partials (lane q stores the dbias
  // and dDskip sums of the experts it kept)
  if (active) {
    const size_t slotbc = (size_t)b * p.nchunks + c;
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      if (e < p.E) {
        reinterpret_cast<float4*>(p.pA)[((slotbc * p.E + e) * p.D + d) * 4 + q] =
            make_float4(accA[e][0], accA[e][1], accA[e][2], accA[e][3]);
      }
    }
#pragma unroll
    for (int e4 = 0; e4 < EMAX / 4; ++e4) {
      const int e = 4 * e4 + q;
      if (e < p.E) {
        p.pBD[((slotbc * p.E + e) * 2) * p.D + d] = accB[e4][0];
        p.pBD[((slotbc * p.E + e) * 2 + 1) * p.D + d] = accB[e4][1];
      }
    }
  }
}

// Passes 3 and 6 (scan_backward.hip): the reverse carry, and the reductions
// over tiles, waves and chunks into dB, dC, dgate, dA, dbias and dDskip.
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
  p.redC = reinterpret_cast<float*>(w + pl.off_redC);
  p.redB = reinterpret_cast<float*>(w + pl.off_redB);
  p.pA = reinterpret_cast<float*>(w + pl.off_pA);
  p.pBD = reinterpret_cast<float*>(w + pl.off_pBD);

  const dim3 grid((unsigned)((size_t)p.B * p.ncg * p.ntiles)), block(WAVES * 64);
  const size_t smem1 = smem_bytes(p.E, p.k, WAVES);
  allow_dynamic_lds(bwd_chunk_kernel<TIn, TDy, WAVES, K>, smem1);
  hipLaunchKernelGGL((bwd_chunk_kernel<TIn, TDy, WAVES, K>), grid, block, smem1, st, p);
  if (hipGetLastError() != hipSuccess) return SWIMBA_EHIP;
  int rc = launch_carry(p.B, p.nchunks, p.D, p.E, p.P, p.H, nullptr, 0, st, nullptr);
  if (rc != SWIMBA_OK) return rc;
  rc = reverse_carry(p, st);
  if (rc != SWIMBA_OK) return rc;
  // the state pass uses the chunk pass's layout (its decay sums unused)
  allow_dynamic_lds(bwd_state_kernel<TIn, TDy, WAVES, K>, smem1);
  hipLaunchKernelGGL((bwd_state_kernel<TIn, TDy, WAVES, K>), grid, block, smem1, st, p);
  if (hipGetLastError() != hipSuccess) return SWIMBA_EHIP;
  const dim3 grid5((unsigned)((size_t)p.B * p.nchunks * p.ntiles));
  if (p.E <= 4) {
    const size_t smem5 = rev_smem_bytes<4>(p.E, p.k);
    allow_dynamic_lds(bwd_grad_kernel<TIn, TDy, K, 4>, smem5);
    hipLaunchKernelGGL((bwd_grad_kernel<TIn, TDy, K, 4>), grid5, dim3(256), smem5, st, p);
  } else if (p.E <= 8) {
    const size_t smem5 = rev_smem_bytes<8>(p.E, p.k);
    allow_dynamic_lds(bwd_grad_kernel<TIn, TDy, K, 8>, smem5);
    hipLaunchKernelGGL((bwd_grad_kernel<TIn, TDy, K, 8>), grid5, dim3(256), smem5, st, p);
  } else {
    const size_t smem5 = rev_smem_bytes<16>(p.E, p.k);
    allow_dynamic_lds(bwd_grad_kernel<TIn, TDy, K, 16>, smem5);
    hipLaunchKernelGGL((bwd_grad_kernel<TIn, TDy, K, 16>), grid5, dim3(256), smem5, st, p);
  }
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

// Eight chunks (waves) share a workgroup's expert table in the chunk and
// state passes when the LDS allows it, four otherwise.
template <typename TIn, typename TDy>
int launch_bwd_k(const swimba_scan_grad_args* g, const BwdPlan& pl, void* ws, hipStream_t st) {
  if (pl.waves == 8) return launch_bwd_w<TIn, TDy, 8>(g, pl, ws, st);
  return launch_bwd_w<TIn, TDy, 4>(g, pl, ws, st);
}

}  // namespace bwd
}  // namespace swimba
