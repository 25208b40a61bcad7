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
//     it, accumulated forward with a running product of the decays.  Before
//     every block of 8 tokens but the first it also keeps a checkpoint: the
//     local state and the running decay product;
//  2. forward carry (shared kernel): carried-in state of every chunk;
//  3. reverse carry: incoming adjoint of every chunk, kappa_{c-1} =
//     P(c) kappa_c + S_c from kappa_last = dL/dh_final; dh0 = kappa_{-1};
//  4. gradient pass (four lanes per channel, four states each; a workgroup
//     per (sequence, chunk, 64-channel tile)): walk the chunk's blocks
//     backward; rebuild each block's states forward from its checkpoint
//     (local state + decay product x carried-in state), then run the adjoint
//     backward over the block from the chunk's incoming adjoint and form the
//     gradients.  dx and ddt_raw are stored per channel; the per-expert
//     parameter gradients (dA, dbias, dDskip) accumulate in LDS for the
//     selected experts of each token and are stored per (sequence, chunk);
//     sums over channels (dB, dC, dgate) are reduced across each wave's
//     channels with lane exchanges, across the waves in LDS, and stored per
//     tile;
//  5. reductions over tiles and chunks, in a fixed order.
// No state is stored per token: the workspace holds per-chunk records, the
// block checkpoints (8 bytes per token and channel) and the partial sums.
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
  int nbk;        // block checkpoints per chunk
  float* P;       // [B][C][16][D] chunk decays
  float* H;       // [B][C][16][D] chunk end states, then carried-in states
  float* adj;     // [B][C][16][D] adjoint seeds, then incoming adjoints
  float* ckH;     // [B][C][nbk][4][D] float4: local state before blocks 1..
  float* ckG;     // [B][C][nbk][4][D] float4: decay product since the chunk's start
  float* red;     // [ntiles][B*L][R] per-tile sums of the dB, dC and gate terms
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
      // checkpoint before the next block: local state and decay product
      if (active) {
        const size_t sk = ((size_t)tk.b * p.nchunks + tk.c) * p.nbk + (tb - t0) / kTB;
        float4* ch4 = reinterpret_cast<float4*>(p.ckH) + sk * 4 * (size_t)p.D + d;
        float4* cg4 = reinterpret_cast<float4*>(p.ckG) + sk * 4 * (size_t)p.D + d;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          ch4[(size_t)q * p.D] = make_float4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
          cg4[(size_t)q * p.D] = make_float4(G[4 * q], G[4 * q + 1], G[4 * q + 2], G[4 * q + 3]);
        }
      }
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
// LDS of the gradient pass: the tile's A as [E][64 channels][16] floats and
// its gradient accumulator of the same shape, the (dt_bias, Dskip) table
// [E][64] and its accumulator, one staging ring shared by the four waves, and
// the waves' per-token channel sums of one block ([4][kTB][2 kN + 4k]: dB,
// dC, then per gate slot the partial sums of the four lanes q).  Every
// per-token access is unconditional: lanes without an accumulator entry of
// their own (q = 2, 3 for dbias/dDskip) add into a private sink.
struct GradLds {
  float4* A;     // [E][64][4]: lane (channel, q) reads states 4q..4q+3
  float4* accA;  // [E][64][4]
  float2* BD;    // [E][64]
  float* accX;   // [E][64][2]: dbias (lane q = 0), dDskip (lane q = 1)
  float* sink;   // [128]: where lanes q = 2, 3 write their (unused) accX terms
  Ring ring;
  float* red;    // [4][kTB][2 kN + 4k]
};

__device__ __forceinline__ GradLds grad_layout(int E, int k) {
  extern __shared__ float4 smem_grad[];
  GradLds g;
  g.A = smem_grad;
  g.accA = g.A + (size_t)E * 256;
  g.BD = reinterpret_cast<float2*>(g.accA + (size_t)E * 256);
  g.accX = reinterpret_cast<float*>(g.BD + (size_t)E * 64);
  g.sink = g.accX + (size_t)E * 128;
  char* rp = reinterpret_cast<char*>(g.sink + 128);
  g.ring.bc = reinterpret_cast<float*>(rp);
  g.ring.e = reinterpret_cast<int32_t*>(rp + 2 * kTB * 32 * 4);
  g.ring.g = reinterpret_cast<float*>(rp + 2 * kTB * 32 * 4 + 2 * kTB * k * 4);
  g.red = reinterpret_cast<float*>(rp + ring_bytes(k));
  return g;
}

// Entry i >> 2 of v on the quad lane i & 3, broadcast to the quad (i is a
// constant once the token loop is unrolled).
__device__ __forceinline__ float quad_pick(const float* v, int i) {
  const float f = i < 4 ? v[0] : v[1];
  switch (i & 3) {
    case 0: return dpp_mov<0x00>(f);
    case 1: return dpp_mov<0x55>(f);
    case 2: return dpp_mov<0xAA>(f);
    default: return dpp_mov<0xFF>(f);
  }
}

// Sums of four per-lane values v[0..3] over the wave's 16 channels (the lanes
// of equal q).  Returns, on lane (q, bit 4, bit 5), the sum of value
// 2 bit5 + bit4; lanes whose channel bits 2 and 3 are clear hold distinct
// results.
__device__ __forceinline__ float channel_sum4(const float* v) {
  const float u0 = xchg_add<32>(v[0], v[2]);  // bit 5 clear: v0, set: v2
  const float u1 = xchg_add<32>(v[1], v[3]);  // bit 5 clear: v1, set: v3
  float w = xchg_add<16>(u0, u1);             // bit 4 clear: u0, set: u1
  w += dpp_mov<0x124>(w);                     // row_ror:4
  w += dpp_mov<0x128>(w);                     // row_ror:8
  return w;
}

// Sums of the per-lane gate terms of slots j < k over all 64 lanes, written
// as slot j's four partials dst[4 j .. 4 j + 3] (the total, then zeros).
template <int K>
__device__ __forceinline__ void gate_sums(const float* part, int k, int lane, float* dst) {
#pragma unroll
  for (int j = 0; j < (K > 0 ? K : 16); ++j) {
    if (j < k) {
      const float v = wave_sum64(part[j]);
      if (lane < 4) dst[4 * j + lane] = lane == 0 ? v : 0.f;
    }
  }
}

// For two gate slots: the dB terms v[0..3] of channel_sum4 and the gate
// terms p0, p1 in one exchange tree.  Lane (q, bit 4, bit 5) gets dB value
// 2 bit5 + bit4 in *sb and, on every lane, the partial sum of slot bit5 over
// the lanes of its q in *sp.
__device__ __forceinline__ void channel_sum4_gates2(const float* v, float p0, float p1,
                                                   float* sb, float* sp) {
  const float u0 = xchg_add<32>(v[0], v[2]);
  const float u1 = xchg_add<32>(v[1], v[3]);
  const float u2 = xchg_add<32>(p0, p1);     // bit 5 clear: slot 0, set: slot 1
  float w = xchg_add<16>(u0, u1);
  float g = xchg_add<16>(u2, u2);
  w += dpp_mov<0x124>(w);                    // row_ror:4
  g += dpp_mov<0x128>(g);                    // row_ror:8 (= lane ^ 8)
  w += dpp_mov<0x128>(w);
  g += dpp_mov<0x1B>(dpp_mov<0x141>(g));     // lane ^ 4: half-row mirror, quad reverse
  *sb = w;
  *sp = g;
}

template <typename TIn, typename TDy, int K>
__global__ __launch_bounds__(256) void bwd_grad_kernel(BwdParams p) {
  const int lane = threadIdx.x & 63, wave = uniform((int)(threadIdx.x >> 6));
  const int k = K > 0 ? K : p.k;
  constexpr int KM = K > 0 ? K : 16;
  const int E = p.E;
  const GradLds s = grad_layout(E, k);
  const int R = 2 * kN + 4 * k;               // per-wave sums in LDS
  const int RO = 2 * kN + ((k + 1) & ~1);     // per-tile sums in memory

  int bid = blockIdx.x;
  const int tile = bid % p.ntiles;
  bid /= p.ntiles;
  const int c = bid % p.nchunks;
  const int b = bid / p.nchunks;
  const int q = lane & 3, cl = wave * 16 + (lane >> 2);  // channel within the tile
  const int d0 = tile * 64, d = d0 + cl;
  const bool active = d < p.D;
  // the tile's tables (zeros past D) and zeroed accumulators
  for (int i = threadIdx.x; i < E * 256; i += blockDim.x) {
    const int e = i >> 8, dl = (i >> 2) & 63, qq = i & 3;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (d0 + dl < p.D)
      v = *reinterpret_cast<const float4*>(p.A + ((size_t)e * p.D + d0 + dl) * kN + 4 * qq);
    s.A[i] = v;
    s.accA[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int i = threadIdx.x; i < E * 64; i += blockDim.x) {
    const int e = i >> 6, dl = i & 63;
    float2 v = make_float2(0.f, 0.f);
    if (d0 + dl < p.D)
      v = make_float2(p.bias[(size_t)e * p.D + d0 + dl], p.Dsk[(size_t)e * p.D + d0 + dl]);
    s.BD[i] = v;
    reinterpret_cast<float2*>(s.accX)[i] = make_float2(0.f, 0.f);
  }

  const int t0 = c * p.chunk, t1 = min(p.L, t0 + p.chunk);
  const size_t row = (size_t)b * p.L;
  const size_t total = (size_t)p.B * p.L;
  constexpr int KW = (kTB * KM + 63) / 64;
  auto valid_at = [&](int t) { return (int)min((size_t)kTB, total - (row + t)); };
  stage::Stager<TIn, KW> st;  // wave 0 stages the shared ring
  st.init(lane);
  int gate_bad = 0;
  const size_t cbase = (((size_t)b * p.nchunks + c) * kN) * p.D + (active ? d : 0);
  // the chunk's carried-in state and incoming adjoint (zeros past D)
  float hin[4], mu[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float v = 0.f;
    if (active) {
      if (c > 0)
        v = p.H[cbase + (size_t)(4 * q + r) * p.D];
      else if (p.h0 != nullptr)
        v = p.h0[((size_t)b * p.D + d) * kN + 4 * q + r];
    }
    hin[r] = v;
    mu[r] = active ? p.adj[cbase + (size_t)(4 * q + r) * p.D] : 0.f;
  }
  // checkpoint before block blk >= 1 (chunk 0 started from h0 itself, so its
  // local states are the states)
  const float4* ckH4 = reinterpret_cast<const float4*>(p.ckH);
  const float4* ckG4 = reinterpret_cast<const float4*>(p.ckG);
  auto load_ck = [&](int blk, float4& h4, float4& g4) {
    h4 = g4 = make_float4(0.f, 0.f, 0.f, 0.f);
    if (blk > 0 && active) {
      const size_t sk = ((size_t)b * p.nchunks + c) * p.nbk + blk - 1;
      h4 = ckH4[(sk * 4 + q) * (size_t)p.D + d];
      g4 = ckG4[(sk * 4 + q) * (size_t)p.D + d];
    }
  };
  const int nblk = (t1 - t0 + kTB - 1) / kTB;
  QuadRows<TIn, TDy> cur, nxt;
  float4 ckh, ckg, ckh_n, ckg_n;
  {
    const int tb = t0 + (nblk - 1) * kTB;
    if (wave == 0) st.issue(p, row + tb, valid_at(tb), k);
    load_quad_rows<TIn, TDy>(p, row + tb, valid_at(tb), active, d, q, cur);
    load_ck(nblk - 1, ckh, ckg);
    if (wave == 0) st.commit(s.ring, 0, min(kTB, t1 - tb), k, E, lane, gate_bad);
  }
  __syncthreads();  // tables, accumulators and the first ring slot

  float* red = s.red + wave * kTB * R;
  float* sink = s.sink + (threadIdx.x >> 2) * 2 + (q & 1);
  const float q0 = q == 0 ? 1.f : 0.f;
  float* out = p.red + (size_t)tile * total * RO;
  int slot = 0;
  for (int blk = nblk - 1; blk >= 0; --blk, slot ^= 1) {
    const int tb = t0 + blk * kTB;
    const int n = min(kTB, t1 - tb);
    const bool more = blk > 0;
    if (more) {
      if (wave == 0) st.issue(p, row + tb - kTB, kTB, k);
      load_quad_rows<TIn, TDy>(p, row + tb - kTB, kTB, active, d, q, nxt);
      load_ck(blk - 1, ckh_n, ckg_n);
    }
    const int32_t* re = s.ring.e + slot * kTB * k;
    const float* rg = s.ring.g + slot * kTB * k;
    const float4* bc4 = reinterpret_cast<const float4*>(s.ring.bc + slot * kTB * 32);

    // per-channel scalars of this lane's two tokens, q and q + 4: Delta, the
    // slope sigmoid(z) of softplus, and the mixed skip weight
    float dltq[2], sigq[2], delq[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int i = q + 4 * hh;
      float beta = 0.f, delta = 0.f;
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        if (j < k) {
          const float2 bd = s.BD[re[i * k + j] * 64 + cl];
          const float gj = rg[i * k + j];
          beta = fmaf(gj, bd.x, beta);
          delta = fmaf(gj, bd.y, delta);
        }
      }
      const float z = to_f32(cur.r[hh]) + beta;
      dltq[hh] = softplus_f32(z);
      sigq[hh] = hw_exp2((z - dltq[hh]) * kLog2e);
      delq[hh] = delta;
    }

    // the block's states, forward from the checkpoint; dC terms dy_t h_t
    float h[4];
    {
      const float hs[4] = {ckh.x, ckh.y, ckh.z, ckh.w}, gs[4] = {ckg.x, ckg.y, ckg.z, ckg.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) h[r] = blk == 0 ? hin[r] : (c > 0 ? fmaf(gs[r], hin[r], hs[r]) : hs[r]);
    }
    float ac[kTB][4], ahc[kTB][4];
    float dltc[kTB], xc[kTB], gyc[kTB];  // per token, the same on the quad
#pragma unroll
    for (int i = 0; i < kTB; ++i) {
      if (i < n) {
        const float dlt = quad_pick(dltq, i);
        const float xv = quad_token(cur.x, i), gy = quad_token(cur.g, i);
        dltc[i] = dlt;
        xc[i] = xv;
        gyc[i] = gy;
        const float dl2 = dlt * kLog2e, dxs = dlt * xv;
        const float4 b4 = bc4[i * 8 + q];
        const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
        float abn[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < KM; ++j) {
          if (j < k) {
            const float gj = rg[i * k + j];
            const float4 a4 = s.A[re[i * k + j] * 256 + cl * 4 + q];
            abn[0] = fmaf(gj, a4.x, abn[0]);
            abn[1] = fmaf(gj, a4.y, abn[1]);
            abn[2] = fmaf(gj, a4.z, abn[2]);
            abn[3] = fmaf(gj, a4.w, abn[3]);
          }
        }
        float hc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a = hw_exp2(dl2 * abn[r]);
          ac[i][r] = a;
          ahc[i][r] = a * h[r];
          h[r] = fmaf(a, h[r], dxs * bv[r]);
          hc[r] = gy * h[r];
        }
        const float sc = channel_sum4(hc);
        if ((lane & 12) == 0) red[i * R + kN + 4 * q + 2 * (lane >> 5) + ((lane >> 4) & 1)] = sc;
      }
    }

    // the adjoint backward over the block
    float dxr[2] = {0.f, 0.f}, dzr[2] = {0.f, 0.f};
#pragma unroll
    for (int ii = 0; ii < kTB; ++ii) {
      const int i = kTB - 1 - ii;
      if (i < n) {
        const float dlt = dltc[i], sig = quad_pick(sigq, i);
        const float delta = quad_pick(delq, i);
        const float xv = xc[i], gy = gyc[i];
        const float dxs = dlt * xv;
        const float4 b4 = bc4[i * 8 + q], c4 = bc4[i * 8 + 4 + q];
        const float bv[4] = {b4.x, b4.y, b4.z, b4.w}, cv[4] = {c4.x, c4.y, c4.z, c4.w};
        // the selected experts' rows and accumulator entries, read first; with
        // one or two slots the entries are read before any is written back
        // (two slots of one expert add both terms into both copies, below)
        constexpr bool kEarly = K == 1 || K == 2;
        int ej[KM];
        float gj[KM], xa[KM];
        float4 aj[KM], acc[KM];
        float2 bdj[KM];
        float* px[KM];
#pragma unroll
        for (int j = 0; j < KM; ++j) {
          if (j < k) {
            ej[j] = re[i * k + j] * 64 + cl;
            gj[j] = rg[i * k + j];
            aj[j] = s.A[ej[j] * 4 + q];
            bdj[j] = s.BD[ej[j]];
            px[j] = q < 2 ? s.accX + ej[j] * 2 + q : sink;
            if constexpr (kEarly) {
              acc[j] = s.accA[ej[j] * 4 + q];
              xa[j] = *px[j];
            }
          }
        }
        float vb[4], w[4];
        float slb = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float lam = fmaf(cv[r], gy, mu[r]);
          vb[r] = lam * dxs;
          slb = fmaf(lam, bv[r], slb);
          w[r] = lam * ahc[i][r];
          mu[r] = ac[i][r] * lam;
        }
        float sa[KM];
        float swa = 0.f;
#pragma unroll
        for (int j = 0; j < KM; ++j) {
          if (j < k) {
            sa[j] = fmaf(aj[j].x, w[0], fmaf(aj[j].y, w[1], fmaf(aj[j].z, w[2], aj[j].w * w[3])));
            swa = fmaf(gj[j], sa[j], swa);
          }
        }
        // sums over the channel's four lanes
        slb += xor_lane<1>(slb, lane);
        slb += xor_lane<2>(slb, lane);
        swa += xor_lane<1>(swa, lane);
        swa += xor_lane<2>(swa, lane);
        const float dz = fmaf(xv, slb, swa) * sig;  // dL/dz = dL/dDelta sigmoid(z)
        const float dxv = fmaf(delta, gy, dlt * slb);
        const float gyx = gy * xv;
        if (q == (i & 3)) {
          dxr[i >> 2] = dxv;
          dzr[i >> 2] = dz;
        }
        // the selected experts' parameter gradients and the gate terms (the
        // dt_bias and Dskip terms of the gate are counted on lane q = 0 only)
        const float xsel = q == 0 ? dz : gyx;
        const float dzq = q0 * dz, gyxq = q0 * gyx;
        float ca[KM], cx[KM], part[KM];
#pragma unroll
        for (int j = 0; j < KM; ++j) {
          if (j < k) {
            ca[j] = gj[j] * dlt;
            cx[j] = gj[j];
            part[j] = fmaf(dlt, sa[j], fmaf(bdj[j].x, dzq, bdj[j].y * gyxq));
          }
        }
        if constexpr (K == 2) {
          // one expert in both slots (never from a top-k router): both copies
          // take both terms (the test is wave-uniform: a scalar branch)
          if (uniform(re[i * k]) == uniform(re[i * k + 1])) {
            ca[0] = ca[1] = ca[0] + ca[1];
            cx[0] = cx[1] = cx[0] + cx[1];
          }
        }
#pragma unroll
        for (int j = 0; j < KM; ++j) {
          if (j < k) {
            if constexpr (!kEarly) {
              acc[j] = s.accA[ej[j] * 4 + q];
              xa[j] = *px[j];
            }
            acc[j].x = fmaf(ca[j], w[0], acc[j].x);
            acc[j].y = fmaf(ca[j], w[1], acc[j].y);
            acc[j].z = fmaf(ca[j], w[2], acc[j].z);
            acc[j].w = fmaf(ca[j], w[3], acc[j].w);
            xa[j] = fmaf(cx[j], xsel, xa[j]);
            if constexpr (!kEarly) {
              s.accA[ej[j] * 4 + q] = acc[j];
              *px[j] = xa[j];
            }
          }
        }
        if constexpr (kEarly) {
#pragma unroll
          for (int j = 0; j < K; ++j) {
            s.accA[ej[j] * 4 + q] = acc[j];
            *px[j] = xa[j];
          }
        }
        const int bcol = 4 * q + 2 * (lane >> 5) + ((lane >> 4) & 1);
        if constexpr (K == 2) {
          float sb, sp;
          channel_sum4_gates2(vb, part[0], part[1], &sb, &sp);
          if ((lane & 12) == 0) red[i * R + bcol] = sb;
          if ((lane & 28) == 0) red[i * R + 2 * kN + 4 * (lane >> 5) + q] = sp;
        } else {
          const float sb = channel_sum4(vb);
          if ((lane & 12) == 0) red[i * R + bcol] = sb;
          gate_sums<K>(part, k, lane, red + i * R + 2 * kN);
        }
      }
    }
    // this lane's tokens' dx and ddt_raw
    if (active) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int i = q + 4 * hh;
        if (i < n) {
          const size_t o = (row + tb + i) * (size_t)p.D + d;
          p.dx[o] = dxr[hh];
          p.ddt[o] = dzr[hh];
        }
      }
    }
    if (more && wave == 0) st.commit(s.ring, slot ^ 1, kTB, k, E, lane, gate_bad);
    __syncthreads();  // the block's wave sums are in LDS; the next ring slot is staged
    // (sums over the four waves; a gate slot also adds its four partials)
    for (int v = threadIdx.x; v < n * RO; v += blockDim.x) {
      const int i = v / RO, col = v - i * RO;
      float sum;
      if (col < 2 * kN) {
        const float* rv = s.red + i * R + col;
        sum = ((rv[0] + rv[kTB * R]) + rv[2 * kTB * R]) + rv[3 * kTB * R];
      } else {
        const int j = min(col - 2 * kN, k - 1);
        const float* rv = s.red + i * R + 2 * kN + 4 * j;
        sum = 0.f;
        for (int ww = 0; ww < 4; ++ww)
          sum += ((rv[ww * kTB * R] + rv[ww * kTB * R + 1]) + rv[ww * kTB * R + 2]) +
                 rv[ww * kTB * R + 3];
      }
      out[(row + tb + i) * RO + col] = sum;
    }
    __syncthreads();  // the sums are read: the next block may overwrite them
    if (more) {
      cur = nxt;
      ckh = ckh_n;
      ckg = ckg_n;
    }
  }
  // per-(sequence, chunk) parameter-gradient partials: each lane stores the
  // accumulator entries it owns
  if (active) {
    const size_t slotbc = (size_t)b * p.nchunks + c;
    for (int e = 0; e < E; ++e) {
      reinterpret_cast<float4*>(p.pA)[((slotbc * E + e) * p.D + d) * 4 + q] =
          s.accA[(e * 64 + cl) * 4 + q];
      if (q < 2) p.pBD[((slotbc * E + e) * 2 + q) * p.D + d] = s.accX[(e * 64 + cl) * 2 + q];
    }
  }
}

// Passes 3 and 5 (scan_backward.hip): the reverse carry, and the reductions
// over tiles and chunks into dB, dC, dgate, dA, dbias and dDskip.
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
  p.nbk = pl.nbk;
  p.P = reinterpret_cast<float*>(w + pl.off_P);
  p.H = reinterpret_cast<float*>(w + pl.off_H);
  p.adj = reinterpret_cast<float*>(w + pl.off_adj);
  p.ckH = reinterpret_cast<float*>(w + pl.off_ckH);
  p.ckG = reinterpret_cast<float*>(w + pl.off_ckG);
  p.red = reinterpret_cast<float*>(w + pl.off_red);
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
  const dim3 grid4((unsigned)((size_t)p.B * p.nchunks * p.ntiles));
  const size_t smem4 = backward_grad_lds_bytes(p.E, p.k);
  allow_dynamic_lds(bwd_grad_kernel<TIn, TDy, K>, smem4);
  hipLaunchKernelGGL((bwd_grad_kernel<TIn, TDy, K>), grid4, dim3(256), smem4, st, p);
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

// Four chunks (waves) share a workgroup's expert table in the chunk pass.
template <typename TIn, typename TDy>
int launch_bwd_k(const swimba_scan_grad_args* g, const BwdPlan& pl, void* ws, hipStream_t st) {
  (void)pl.waves;
  return launch_bwd_w<TIn, TDy, 4>(g, pl, ws, st);
}

}  // namespace bwd
}  // namespace swimba
