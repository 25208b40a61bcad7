// Parameter-space-mixed selective scan (Swimba) for gfx950.
//
// Pages: "Swimba: Switch Mamba Model Scales State Space Models" (Dutch summary,
// "Kernmechanisme van Swimba": the selected experts' parameters are mixed with
// the router weights and one recurrence runs; Theorem 1: the result is a single
// selective SSM; Theorem 3: contractive transitions keep it stable) and
// "Mamba y las SSMs: el retorno del estado persistente" ("Mamba": transition
// exp(Delta A), selective B_t and C_t; Figure 2: the state stays on chip while
// inputs and outputs stream from HBM).
//
// Layout of the work.  A lane owns one channel d of one sequence b and keeps its
// 16 fp32 states in VGPRs for a whole chunk of tokens.  The 64 lanes of a wave
// are 64 consecutive channels of the same token, so everything per token
// (routing, gates, B_t, C_t) is wave-uniform: a per-wave LDS ring stages it one
// block of 8 tokens ahead, while x, dt_raw and y stream as coalesced 64-lane
// rows.  The expert parameters of the wave's 64 channels are staged once in LDS
// as one block of 16-byte rows per expert -- A x log2(e) in four rows of four
// states, then (dt_bias, Dskip) -- so each selected expert costs one address
// and five conflict-free reads per token.  The waves of a workgroup are
// consecutive chunks of the same channel tile and share that table.
//
// More than 16 experts do not fit that table (5 KiB per expert and tile):
// then each selected expert's rows are read from memory per token (A is
// L2-resident), with buffer loads at the expert's offset, and the chunk
// decays are summed in registers.
//
// The walk runs pairs of 8-token blocks with the two ring slots and two x /
// dt_raw buffers fixed in the code (no register copies between blocks); a
// ragged tail block or a ragged tile takes a guarded path after the full
// blocks.
//
// Long sequences are cut into chunks so that enough waves run at once.  Chunks
// are joined in three passes, all exact up to fp32 rounding:
//   1. chunk pass: every chunk from a zero state (chunk 0 from h0); it writes
//      provisional y, its end state, and its total decay
//      P[n] = prod_t exp(Delta_t Abar_t[n]) = exp2(sum_e U_e A[e, d, n] log2 e),
//      where U_e = sum over the chunk's tokens and slots that selected e of
//      Delta_t g_j; the U_e are added up per wave in LDS;
//   2. carry pass: h_in(c+1) = P(c) * h_in(c) + h_end(c) over the chunks;
//   3. fix-up pass: chunk c >= 1 re-runs from h_in(c), tracking the carried part
//      g = (prod of decays) * h_in.  With A < 0 and gates >= 0 every decay is in
//      (0, 1], so once |g| is below 2^-24 of the state on every lane the rest of
//      the chunk equals the provisional y to fp32 resolution and the pass stops.
//      When the contraction does not hold (flagged by the chunk pass) or the
//      caller asks for it, the whole chunk is recomputed.
#pragma once
#include <type_traits>

#include "scan_common.hpp"
#include "swimba_device.hpp"
#include "swimba_internal.hpp"

namespace swimba {
namespace mixed {

using stage::kTB;
using stage::Ring;
using stage::ring_bytes;
using stage::wave_sync;

constexpr float kFixupTol = 5.9604645e-08f;  // 2^-24
constexpr float kTiny = 1e-30f;
// 16-byte rows of 64 lanes per expert in the LDS table: diagonal A as four
// rows of (A x log2 e) for states 4q..4q+3, then (dt_bias, Dskip, 0, 0);
// scalar A: one row (A x log2 e, dt_bias, Dskip, 0).
constexpr int kRowsDiag = 5;

struct MixParams {
  int B, L, D, E, k;
  int chunk, nchunks, ntiles;
  int carry;  // SWIMBA_CARRY_REWALK or SWIMBA_CARRY_FIXUP
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
  void* y;
  float* h_final;
  float* P;           // [B][C][16][D] chunk decays
  float* H;           // [B][C][16][D] chunk end states, then carried-in states
  int32_t* flags;     // [B][C][ntiles] 1 = contraction not guaranteed
  const int32_t* tflags;  // [ntiles] 1 = some A of the tile is not negative (rows
                          // read from memory; the table path checks while staging)
};

// Expert rows read from memory per token (more experts than the LDS table
// holds): buffers over A, dt_bias and Dskip, and the lane's offsets into a
// row (past every buffer for lanes beyond D: those loads return 0).
struct Rows {
  stage::rsrc_t a, bias, dsk;
  uint32_t voa, vob;
};

// Table modes of the mixed passes (TM): 0 = expert rows read from memory
// per token (more than 32 experts, or more than 16 with a scalar A); 1 =
// every expert's rows in an LDS table (E <= 16); 2 = only the A rows in the
// table (17 <= E <= 32, diagonal A: 4 KB per expert), dt_bias and Dskip read
// from memory per token.
__host__ __device__ constexpr int table_mode(int emax, bool scalar_a) {
  return emax <= 16 ? 1 : ((emax <= 32 && !scalar_a) ? 2 : 0);
}
// LDS a workgroup of table mode 2 may use (the CU's 160 KiB)
constexpr size_t kTabModeLds = (size_t)160 << 10;
__host__ __device__ inline int table_rows(bool scalar_a, int tm = 1) {
  return scalar_a ? 1 : (tm == 2 ? 4 : kRowsDiag);
}
__host__ __device__ inline size_t table_bytes(int E, bool scalar_a, int tm = 1) {
  return (size_t)E * table_rows(scalar_a, tm) * 64 * 16;
}
// A wave's ring: the shared staging layout plus, per (token, slot), the byte
// offset of the selected expert's U column.
__host__ __device__ inline size_t ring_bytes_u(int k) {
  return ring_bytes(k) + (size_t)2 * kTB * k * 4;
}
// byte stride of one expert's rows in the table
__host__ __device__ inline int expert_stride(bool scalar_a, int tm = 1) {
  return table_rows(scalar_a, tm) * 64 * 16;
}

// LDS: the workgroup's expert table, then per wave a staging ring (dynamic
// LDS); in the chunk pass also the wave's sums U_e as [EMAX][64] floats, in a
// separate static LDS array so that the compiler knows the sums' stores do
// not touch the table and may issue the next token's table reads before them.
struct Smem {
  const float4* T;  // [E][rows][64]
  float* U;         // [EMAX][64], chunk pass only
  Ring ring;        // this wave's ring
};

__device__ __forceinline__ Smem smem_layout(int E, int k, int wave, bool scalar_a, int tm = 1) {
  extern __shared__ float4 smem_raw[];
  Smem s;
  char* p = reinterpret_cast<char*>(smem_raw);
  s.T = reinterpret_cast<const float4*>(p);
  p += table_bytes(E, scalar_a, tm);
  p += ring_bytes_u(k) * wave;
  s.ring.bc = reinterpret_cast<float*>(p);
  s.ring.e = reinterpret_cast<int32_t*>(p + 2 * kTB * 32 * 4);
  s.ring.g = reinterpret_cast<float*>(p + 2 * kTB * 32 * 4 + 2 * kTB * k * 4);
  s.ring.uo = reinterpret_cast<int32_t*>(p + ring_bytes(k));
  s.U = nullptr;
  return s;
}

// dynamic LDS of the chunk and fix-up passes
__host__ inline size_t smem_bytes(int E, int k, int waves, bool scalar_a, int tm = 1) {
  return table_bytes(E, scalar_a, tm) + ring_bytes_u(k) * waves;
}

// Stage the tile's expert parameters (A scaled by log2 e); returns 1 if any A
// in the tile is not strictly negative (including NaN).  Lanes past D get
// zeros.
__device__ __forceinline__ int load_table(const MixParams& p, float4* T, int d0, bool scalar_a,
                                          int tm = 1) {
  int bad = 0;
  const int nthr = blockDim.x;
  if (scalar_a) {
    for (int i = threadIdx.x; i < p.E * 64; i += nthr) {
      const int e = i >> 6, d = d0 + (i & 63);
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (d < p.D) {
        const size_t o = (size_t)e * p.D + d;
        const float a = p.A[o];
        bad |= !(a < 0.f);
        v = make_float4(a * kLog2e, p.bias[o], p.Dsk[o], 0.f);
      }
      T[i] = v;
    }
    return bad;
  }
  // consecutive threads read consecutive 16-byte pieces of A[e, d0:d0+64, :]
  for (int i = threadIdx.x; i < p.E * 256; i += nthr) {
    const int e = i >> 8, dl = (i >> 2) & 63, q = i & 3;
    const int d = d0 + dl;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (d < p.D) {
      const float* a = p.A + ((size_t)e * p.D + d) * kN + q * 4;
      const float a0 = a[0], a1 = a[1], a2 = a[2], a3 = a[3];
      bad |= !(a0 < 0.f) | !(a1 < 0.f) | !(a2 < 0.f) | !(a3 < 0.f);
      v = make_float4(a0 * kLog2e, a1 * kLog2e, a2 * kLog2e, a3 * kLog2e);
    }
    T[(e * (tm == 2 ? 4 : kRowsDiag) + q) * 64 + dl] = v;
  }
  if (tm == 2) return bad;  // A rows only
  for (int i = threadIdx.x; i < p.E * 64; i += nthr) {
    const int e = i >> 6, dl = i & 63, d = d0 + dl;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (d < p.D) {
      const size_t o = (size_t)e * p.D + d;
      v = make_float4(p.bias[o], p.Dsk[o], 0.f, 0.f);
    }
    T[(e * kRowsDiag + 4) * 64 + dl] = v;
  }
  return bad;
}

// Lane's first table row of the expert whose rows start `eoff` bytes into
// the table (the ring holds that offset): one add; the expert's other rows
// are constant offsets from it.
__device__ __forceinline__ const float4* expert_rows(const Smem& s, int eoff, int lane) {
  return reinterpret_cast<const float4*>(reinterpret_cast<const char*>(s.T + lane) + eoff);
}

// This lane's entry of the wave's sum U_e, whose column starts `uoff` bytes
// into U.
__device__ __forceinline__ float* usum_at(float* U, int uoff, int lane) {
  return reinterpret_cast<float*>(reinterpret_cast<char*>(U + lane) + uoff);
}

// State update and readout of one token for one lane, given the per-state
// exponents m[n] = Delta Abar[n] log2(e) (SA: one exponent m[0]) and the
// Euler input dx = Delta x; bc points at the token's B_t (4 rows) and C_t
// (4 rows) in the ring.
template <bool TRACK, bool SA, bool ZOH>
__device__ __forceinline__ float update_readout(const float4* bc, const float* m, float dx,
                                                float* h, float* g) {
  const float a0 = SA ? hw_exp2(m[0]) : 0.f;
  const float dx0 = (SA && ZOH) ? dx * zoh_phi(a0, m[0]) : dx;
  float yv = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 b4 = bc[q], c4 = bc[4 + q];
    const float bv[4] = {b4.x, b4.y, b4.z, b4.w}, cv[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = 4 * q + r;
      const float a = SA ? a0 : hw_exp2(m[n]);
      const float inj = (ZOH && !SA) ? (dx * bv[r]) * zoh_phi(a, m[n]) : dx0 * bv[r];
      h[n] = fmaf(a, h[n], inj);
      yv = fmaf(cv[r], h[n], yv);
      if (TRACK && !SA) g[n] *= a;
    }
  }
  if (TRACK && SA) g[0] *= a0;
  return yv;
}

// One token of the mixed recurrence for one lane with k == K known at compile
// time.  Routing (experts e[j], gates gw[j]) is wave-uniform; each selected
// expert's table block is read with one address and all of the token's table
// reads are issued together.  ACC_U: add Delta g_j to the wave's sums U_e.
// PBD (rows from memory): the experts' (dt_bias, Dskip) were loaded ahead
// into pbd.
template <int K, bool TRACK, bool ACC_U, bool SA, bool ZOH, int TM, bool PBD = false>
__device__ __forceinline__ float mix_token_k(const Smem& s, const Rows& R, float* ms,
                                             const int* e, const int* uo, const float* gw,
                                             const float4* bc, int lane, float xv, float rv,
                                             float* h, float* g, const float2* pbd = nullptr) {
  float4 bd[K];
  float4 ar[SA ? 1 : K][4];
  float uold[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    if constexpr (TM >= 1) {
      if (ACC_U && TM == 1) uold[j] = *usum_at(s.U, uo[j], lane);
      const float4* te = expert_rows(s, e[j], lane);
      if constexpr (SA) {
        bd[j] = te[0];  // (A log2 e, dt_bias, Dskip, 0)
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) ar[j][q] = te[q * 64];
        if (TM == 1) bd[j] = te[4 * 64];  // (dt_bias, Dskip, 0, 0)
      }
    }
  }
  if constexpr (TM != 1) {
    // rows from memory: e[j] and uo[j] are the byte offsets of the expert's
    // A block (TM 0) and of its dt_bias / Dskip entries (wave-uniform)
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const uint32_t soa = (uint32_t)uniform(e[j]), sob = (uint32_t)uniform(uo[j]);
      const float bj = PBD ? pbd[j].x : stage::buf_load<float>(R.bias, R.vob, sob);
      const float dj = PBD ? pbd[j].y : stage::buf_load<float>(R.dsk, R.vob, sob);
      if constexpr (TM == 2) {
        bd[j] = make_float4(bj, dj, 0.f, 0.f);
      } else if constexpr (SA) {
        bd[j] = make_float4(stage::buf_load<float>(R.a, R.vob, sob), bj, dj, 0.f);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const stage::v4u v =
              __builtin_amdgcn_raw_buffer_load_b128(R.a, (int)(R.voa + q * 16), (int)soa, 0);
          ar[j][q] = make_float4(__uint_as_float(v.x), __uint_as_float(v.y),
                                 __uint_as_float(v.z), __uint_as_float(v.w));
        }
        bd[j] = make_float4(bj, dj, 0.f, 0.f);
      }
    }
  }
  // mixed dt_bias and Dskip
  float beta = 0.f, delta = 0.f;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    beta = fmaf(gw[j], SA ? bd[j].y : bd[j].x, beta);
    delta = fmaf(gw[j], SA ? bd[j].z : bd[j].y, delta);
  }
  const float dlt = softplus_f32(rv + beta);
  // rows from memory hold A itself: log2 e goes into u
  const float dls = TM >= 1 ? dlt : dlt * kLog2e;
  float u[K];
#pragma unroll
  for (int j = 0; j < K; ++j) u[j] = dls * gw[j];
  // mixed exponents m[n] = sum_j u_j A[e_j, d, n] log2 e
  float m[SA ? 1 : kN];
  if constexpr (SA) {
    m[0] = u[0] * bd[0].x;
#pragma unroll
    for (int j = 1; j < K; ++j) m[0] = fmaf(u[j], bd[j].x, m[0]);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 a = ar[0][q];
      m[4 * q + 0] = u[0] * a.x;
      m[4 * q + 1] = u[0] * a.y;
      m[4 * q + 2] = u[0] * a.z;
      m[4 * q + 3] = u[0] * a.w;
    }
#pragma unroll
    for (int j = 1; j < K; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 a = ar[j][q];
        m[4 * q + 0] = fmaf(u[j], a.x, m[4 * q + 0]);
        m[4 * q + 1] = fmaf(u[j], a.y, m[4 * q + 1]);
        m[4 * q + 2] = fmaf(u[j], a.z, m[4 * q + 2]);
        m[4 * q + 3] = fmaf(u[j], a.w, m[4 * q + 3]);
      }
  }
  if (ACC_U && TM != 1)
#pragma unroll
    for (int n = 0; n < (SA ? 1 : kN); ++n) ms[n] += m[n];
  const float yv = update_readout<TRACK, SA, ZOH>(bc, m, dlt * xv, h, g);
  if (ACC_U && TM == 1) {
    // U_e += u_j; a slot that repeats an earlier slot's expert adds onto
    // that slot's new value (both were read before either store)
    float unew[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      float base = uold[j];
#pragma unroll
      for (int i = 0; i < j; ++i) base = uo[i] == uo[j] ? unew[i] : base;
      unew[j] = base + u[j];
    }
#pragma unroll
    for (int j = 0; j < K; ++j) *usum_at(s.U, uo[j], lane) = unew[j];
  }
  return fmaf(delta, xv, yv);
}

// The same for k known only at run time (k > 2).
template <bool TRACK, bool ACC_U, bool SA, bool ZOH, int TM>
__device__ __forceinline__ float mix_token_any(const Smem& s, const Rows& R, float* ms, int k,
                                               const int* e, const int* uo, const float* gw,
                                               const float4* bc, int lane, float xv, float rv,
                                               float* h, float* g) {
  float beta = 0.f, delta = 0.f;
  for (int j = 0; j < k; ++j) {
    float bj, dj;
    if constexpr (TM == 1) {
      const float4 bd = expert_rows(s, e[j], lane)[SA ? 0 : 4 * 64];
      bj = SA ? bd.y : bd.x;
      dj = SA ? bd.z : bd.y;
    } else {
      const uint32_t sob = (uint32_t)uniform(uo[j]);
      bj = stage::buf_load<float>(R.bias, R.vob, sob);
      dj = stage::buf_load<float>(R.dsk, R.vob, sob);
    }
    beta = fmaf(gw[j], bj, beta);
    delta = fmaf(gw[j], dj, delta);
  }
  const float dlt = softplus_f32(rv + beta);
  const float dls = TM >= 1 ? dlt : dlt * kLog2e;
  float m[SA ? 1 : kN];
#pragma unroll
  for (int n = 0; n < (SA ? 1 : kN); ++n) m[n] = 0.f;
  for (int j = 0; j < k; ++j) {
    const float u = dls * gw[j];
    if (ACC_U && TM == 1) {
      float* up = usum_at(s.U, uo[j], lane);
      *up = *up + u;
    }
    if constexpr (TM >= 1) {
      const float4* te = expert_rows(s, e[j], lane);
      if constexpr (SA) {
        m[0] = fmaf(u, te[0].x, m[0]);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 a = te[q * 64];
          m[4 * q + 0] = fmaf(u, a.x, m[4 * q + 0]);
          m[4 * q + 1] = fmaf(u, a.y, m[4 * q + 1]);
          m[4 * q + 2] = fmaf(u, a.z, m[4 * q + 2]);
          m[4 * q + 3] = fmaf(u, a.w, m[4 * q + 3]);
        }
      }
    } else {
      const uint32_t soa = (uint32_t)uniform(e[j]), sob = (uint32_t)uniform(uo[j]);
      if constexpr (SA) {
        m[0] = fmaf(u, stage::buf_load<float>(R.a, R.vob, sob), m[0]);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const stage::v4u v =
              __builtin_amdgcn_raw_buffer_load_b128(R.a, (int)(R.voa + q * 16), (int)soa, 0);
          m[4 * q + 0] = fmaf(u, __uint_as_float(v.x), m[4 * q + 0]);
          m[4 * q + 1] = fmaf(u, __uint_as_float(v.y), m[4 * q + 1]);
          m[4 * q + 2] = fmaf(u, __uint_as_float(v.z), m[4 * q + 2]);
          m[4 * q + 3] = fmaf(u, __uint_as_float(v.w), m[4 * q + 3]);
        }
      }
    }
  }
  if (ACC_U && TM != 1)
#pragma unroll
    for (int n = 0; n < (SA ? 1 : kN); ++n) ms[n] += m[n];
  const float yv = update_readout<TRACK, SA, ZOH>(bc, m, dlt * xv, h, g);
  return fmaf(delta, xv, yv);
}

// One token from ring slot `slot`, position i (routing read from the ring).
template <int K, bool TRACK, bool ACC_U, bool SA, bool ZOH, int TM>
__device__ __forceinline__ float ring_token(const MixParams& p, const Smem& s, const Rows& R,
                                            float* ms, int slot, int i, int lane, float xv,
                                            float rv, float* h, float* g) {
  const float4* bc = reinterpret_cast<const float4*>(s.ring.bc + (slot * kTB + i) * 32);
  if constexpr (K > 0) {
    int ev[K], uv[K];
    float gv[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      ev[j] = s.ring.e[(slot * kTB + i) * K + j];
      gv[j] = s.ring.g[(slot * kTB + i) * K + j];
      uv[j] = (ACC_U || TM != 1) ? s.ring.uo[(slot * kTB + i) * K + j] : 0;
    }
    return mix_token_k<K, TRACK, ACC_U, SA, ZOH, TM>(s, R, ms, ev, uv, gv, bc, lane, xv, rv, h,
                                                      g);
  } else {
    const int k = p.k;
    int eb[16], ub[16];
    float gb[16];
    for (int j = 0; j < k; ++j) {
      eb[j] = s.ring.e[(slot * kTB + i) * k + j];
      gb[j] = s.ring.g[(slot * kTB + i) * k + j];
      ub[j] = (ACC_U || TM != 1) ? s.ring.uo[(slot * kTB + i) * k + j] : 0;
    }
    return mix_token_any<TRACK, ACC_U, SA, ZOH, TM>(s, R, ms, k, eb, ub, gb, bc, lane, xv, rv, h,
                                                     g);
  }
}

// True (on every lane) once the carried part g has decayed below fp32
// resolution of the state on every lane of the wave.
template <bool SA>
__device__ __forceinline__ bool carried_part_gone(const float* h, const float* g) {
  float mh = 0.f;
#pragma unroll
  for (int q = 0; q < kN; ++q) mh = fmaxf(mh, fabsf(h[q]));
  const float thr = fmaxf(kFixupTol * mh, kTiny);
  bool conv = true;
  if constexpr (SA) {
    conv = fabsf(g[0]) * g[1] <= thr;  // g[1] = max_n |h_in[n]|; NaN: not converged
  } else {
#pragma unroll
    for (int q = 0; q < kN; ++q) conv &= fabsf(g[q]) <= thr;  // NaN: not converged
  }
  return __all(conv);
}

// Store y of two consecutive tokens (rows i, i + 1 of the block's buffer):
// one conversion for both in bf16.
template <typename TOut>
__device__ __forceinline__ void store_y2(stage::rsrc_t ry, uint32_t yoff, uint32_t yrow, int i,
                                         float y0, float y1) {
  if constexpr (std::is_same<TOut, bf16_t>::value) {
    typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
    typedef float f2_t __attribute__((ext_vector_type(2)));
    const f2_t f = {y0, y1};
    const uint32_t pk = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf2_t));
    stage::buf_store(ry, yoff, (uint32_t)i * yrow, (bf16_t)(pk & 0xffffu));
    stage::buf_store(ry, yoff, (uint32_t)(i + 1) * yrow, (bf16_t)(pk >> 16));
  } else {
    stage::buf_store(ry, yoff, (uint32_t)i * yrow, y0);
    stage::buf_store(ry, yoff, (uint32_t)(i + 1) * yrow, y1);
  }
}

// Walk tokens [t0, t1) of sequence b for one lane, staging each block of kTB
// tokens' uniform data and x/dt_raw one block ahead.  With TRACK and
// `truncate`, stops once the carried part g has decayed on every lane.
// x, dt_raw and y go through per-block buffer resources (scalar token offsets,
// a fixed per-lane channel offset); the prefetch of the next block is issued
// before the current one computes and is waited on only when it is used.
template <typename TIn, typename TOut, int K, bool TRACK, bool ACC_U, bool SA, bool ZOH,
          int TM>
__device__ __forceinline__ void walk(const MixParams& p, const Smem& s, float* ms, int b, int t0,
                                     int t1, int d, bool active, bool full_tile, int lane,
                                     bool truncate, float* h, float* g, int& gate_bad) {
  constexpr int KW = (kTB * (K > 0 ? K : 16) + 63) / 64;
  const int k = K > 0 ? K : p.k;
  const int D = p.D;
  const size_t row = (size_t)b * p.L;
  const size_t total = (size_t)p.B * p.L;
  // lanes past D (ragged tile) read 0 and store nothing
  const uint32_t xoff = active ? (uint32_t)d * (uint32_t)sizeof(TIn) : stage::kOffNone;
  const uint32_t yoff = (uint32_t)d * (uint32_t)sizeof(TOut);
  const uint32_t xrow = (uint32_t)D * (uint32_t)sizeof(TIn);
  const uint32_t yrow = (uint32_t)D * (uint32_t)sizeof(TOut);
  TIn xa[kTB], ra[kTB], xb[kTB], rb[kTB];
  stage::Stager<TIn, KW> st;
  st.init(lane);
  Rows R;
  if constexpr (TM != 1) {
    const uint32_t nab = (uint32_t)p.E * (uint32_t)D * (SA ? 4u : (uint32_t)kN * 4u);
    const uint32_t nbb = (uint32_t)p.E * (uint32_t)D * 4u;
    R.a = stage::make_rsrc(p.A, nab);
    R.bias = stage::make_rsrc(p.bias, nbb);
    R.dsk = stage::make_rsrc(p.Dsk, nbb);
    R.voa = active ? (uint32_t)d * (uint32_t)kN * 4u : stage::kOffNone;
    R.vob = active ? (uint32_t)d * 4u : stage::kOffNone;
  }
  auto valid_at = [&](int t) { return (int)min((size_t)kTB, total - (row + t)); };
  auto load_xr = [&](int t, TIn* xs, TIn* rs) {
    const int v = valid_at(t);
    const stage::rsrc_t rx = stage::rows_rsrc<TIn>(p.x, row + t, v, D);
    const stage::rsrc_t rr = stage::rows_rsrc<TIn>(p.dt, row + t, v, D);
    // the scalar offset is not range-checked by the hardware: rows past the
    // tensor's end re-read its last row
#pragma unroll
    for (int i = 0; i < kTB; ++i) {
      const uint32_t so = (uint32_t)min(i, v - 1) * xrow;
      xs[i] = stage::buf_load<TIn>(rx, xoff, so);
      rs[i] = stage::buf_load<TIn>(rr, xoff, so);
    }
  };

  st.issue(p, row + t0, valid_at(t0), k);
  load_xr(t0, xa, ra);
  // ring offsets: table rows and sum columns, or (rows from memory) the
  // expert's A block and its dt_bias / Dskip row
  const int escale = TM >= 1 ? expert_stride(SA, TM) : D * (SA ? 4 : kN * 4);
  const int uscale = TM == 1 ? 64 * 4 : D * 4;
  st.commit(s.ring, 0, min(kTB, t1 - t0), k, p.E, lane, gate_bad, escale, uscale);

  int tb = t0;
  // One whole block at tb from ring slot SL and buffers xc/rc (compile-time
  // slot and buffers); prefetches the next block into xn/rn and the other
  // slot.  Returns false when the walk stops here (carried part decayed).
  auto fast_block = [&](auto SLOT, TIn* xc, TIn* rc, TIn* xn, TIn* rn) -> bool {
    constexpr int sl = decltype(SLOT)::value;
    const int tn = tb + kTB;
    const bool more = tn < t1;
    // the prefetch always runs (the last block re-reads itself): a
    // conditional load would make the compiler keep and copy the old buffers
    const int tl = more ? tn : tb;
    st.issue(p, row + tl, valid_at(tl), k);
    load_xr(tl, xn, rn);
    wave_sync();
    const stage::rsrc_t ry = stage::rows_rsrc<TOut>(p.y, row + tb, kTB, D);
#pragma unroll
    for (int i = 0; i < kTB; i += 2) {
      const float y0 = ring_token<K, TRACK, ACC_U, SA, ZOH, TM>(
          p, s, R, ms, sl, i, lane, to_f32(xc[i]), to_f32(rc[i]), h, g);
      const float y1 = ring_token<K, TRACK, ACC_U, SA, ZOH, TM>(
          p, s, R, ms, sl, i + 1, lane, to_f32(xc[i + 1]), to_f32(rc[i + 1]), h, g);
      store_y2<TOut>(ry, yoff, yrow, i, y0, y1);
    }
    if (TRACK && truncate && carried_part_gone<SA>(h, g)) return false;
    if (more)
      st.commit(s.ring, sl ^ 1, min(kTB, t1 - tn), k, p.E, lane, gate_bad, escale, uscale);
    tb = tn;
    return true;
  };

  int slot = 0;  // ring slot and buffer of the block at tb
  if (full_tile && K > 0 && TM == 1) {
    // whole blocks in pairs: slot 0 with xa/ra, then slot 1 with xb/rb
    const std::integral_constant<int, 0> s0;
    const std::integral_constant<int, 1> s1;
    while (tb + kTB <= t1) {
      if (!fast_block(s0, xa, ra, xb, rb)) return;
      if (tb + kTB > t1) {
        slot = 1;
        break;
      }
      if (!fast_block(s1, xb, rb, xa, ra)) return;
    }
    if (tb >= t1) return;
    if (slot == 1) {
#pragma unroll
      for (int i = 0; i < kTB; ++i) {
        xa[i] = xb[i];
        ra[i] = rb[i];
      }
    }
  }
  // Guarded blocks: the ragged tail of a full tile, or every block of a
  // ragged tile, of a runtime k or with expert rows read from memory (the
  // block at tb is in slot `slot`, xa/ra).
  for (; tb < t1; slot ^= 1) {
    const int n = min(kTB, t1 - tb);
    const int tn = tb + kTB;
    const bool more = tn < t1;
    if (more) {
      st.issue(p, row + tn, valid_at(tn), k);
      load_xr(tn, xb, rb);
    }
    wave_sync();
    // stores past the block's n tokens fall outside this buffer and are dropped
    const stage::rsrc_t ry = stage::rows_rsrc<TOut>(p.y, row + tb, n, D);
    if constexpr (TM != 1 && K > 0) {
      // dt_bias and Dskip (memory) of token i + 1's experts load while token
      // i computes: Delta, and so every state update, waits on them (the last
      // token reloads its own, unused)
      auto ring_bd = [&](int i, float2* bdv) {
#pragma unroll
        for (int j = 0; j < K; ++j) {
          const uint32_t sob = (uint32_t)uniform(s.ring.uo[(slot * kTB + i) * K + j]);
          bdv[j] = make_float2(stage::buf_load<float>(R.bias, R.vob, sob),
                               stage::buf_load<float>(R.dsk, R.vob, sob));
        }
      };
      float2 cur[K], nxt[K];
      ring_bd(0, cur);
#pragma unroll
      for (int i = 0; i < kTB; ++i) {
        if (i < n) {
          ring_bd(min(i + 1, n - 1), nxt);
          const float xv = active ? to_f32(xa[i]) : 0.f, rv = active ? to_f32(ra[i]) : 0.f;
          const float4* bc = reinterpret_cast<const float4*>(s.ring.bc + (slot * kTB + i) * 32);
          int ev[K], uv[K];
          float gv[K];
#pragma unroll
          for (int j = 0; j < K; ++j) {
            ev[j] = s.ring.e[(slot * kTB + i) * K + j];
            uv[j] = s.ring.uo[(slot * kTB + i) * K + j];
            gv[j] = s.ring.g[(slot * kTB + i) * K + j];
          }
          const float yv = mix_token_k<K, TRACK, ACC_U, SA, ZOH, TM, true>(
              s, R, ms, ev, uv, gv, bc, lane, xv, rv, h, g, cur);
          if (active) stage::buf_store(ry, yoff, (uint32_t)i * yrow, from_f32<TOut>(yv));
#pragma unroll
          for (int j = 0; j < K; ++j) cur[j] = nxt[j];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < kTB; ++i) {
        if (i < n) {
          const float xv = active ? to_f32(xa[i]) : 0.f, rv = active ? to_f32(ra[i]) : 0.f;
          const float yv = ring_token<K, TRACK, ACC_U, SA, ZOH, TM>(p, s, R, ms, slot, i, lane,
                                                                    xv, rv, h, g);
          if (active) stage::buf_store(ry, yoff, (uint32_t)i * yrow, from_f32<TOut>(yv));
        }
      }
    }
    if (TRACK && truncate && carried_part_gone<SA>(h, g)) return;
    if (more) {
      st.commit(s.ring, slot ^ 1, min(kTB, t1 - tn), k, p.E, lane, gate_bad, escale, uscale);
#pragma unroll
      for (int i = 0; i < kTB; ++i) {
        xa[i] = xb[i];
        ra[i] = rb[i];
      }
    }
    tb = tn;
  }
}

// Pass 1 (or the only pass when CHUNKED is false).  EMAX >= E: columns of
// each wave's sums U_e.
// EMAX > 16: the selected experts' rows come from memory (no table; the
// chunk decays are summed in registers).
template <typename TIn, typename TOut, int WAVES, int K, bool CHUNKED, bool SA, bool ZOH,
          int EMAX>
__global__ __launch_bounds__(WAVES * 64) void mix_chunk_kernel(MixParams p) {
  constexpr int TM = table_mode(EMAX, SA);
  constexpr bool TAB = TM >= 1;  // a table in LDS
  __shared__ float usum[CHUNKED && TM == 1 ? WAVES * EMAX * 64 : 1];
  const int wave = uniform((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  Smem s = smem_layout(TAB ? p.E : 0, K > 0 ? K : p.k, wave, SA, TM);
  if (CHUNKED && TM == 1) s.U = usum + wave * EMAX * 64;
  const int ncg = (p.nchunks + WAVES - 1) / WAVES;
  int bid = blockIdx.x;
  const int tile = bid % p.ntiles;
  bid /= p.ntiles;
  const int cg = bid % ncg;
  const int b = bid / ncg;
  const int d0 = tile * 64, d = d0 + lane;
  const bool active = d < p.D;

  int bad = 0;
  if constexpr (TAB) {
    bad = load_table(p, const_cast<float4*>(s.T), d0, SA, TM);
    if (CHUNKED && TM == 1)
      for (int e = 0; e < p.E; ++e) s.U[e * 64 + lane] = 0.f;
    bad = __syncthreads_or(bad);
  } else if (CHUNKED) {
    bad = p.tflags[tile];
  }

  const int c = cg * WAVES + wave;
  if (c >= p.nchunks) return;  // no barrier below
  const int t0 = c * p.chunk;
  const int t1 = min(p.L, t0 + p.chunk);

  float h[kN];
#pragma unroll
  for (int n = 0; n < kN; ++n)
    h[n] = (c == 0 && p.h0 != nullptr && active) ? p.h0[((size_t)b * p.D + d) * kN + n] : 0.f;

  // every chunk writes y (provisional for chunks >= 1, recomputed by the
  // fix-up pass where the carried-in state still matters)
  int gate_bad = 0;
  float lg[SA ? 1 : kN];  // the chunk's exponent sums (table mode 1: from U)
#pragma unroll
  for (int n = 0; n < (SA ? 1 : kN); ++n) lg[n] = 0.f;
  walk<TIn, TOut, K, false, CHUNKED, SA, ZOH, TM>(p, s, lg, b, t0, t1, d, active,
                                                   d0 + 64 <= p.D, lane, false, h, nullptr,
                                                   gate_bad);

  if (CHUNKED) {
    // total decay of the chunk: P[n] = exp2(sum_e U_e A[e, d, n] log2 e) (table
    // path; rows from memory: the summed exponents); with SA one decay per
    // channel, written to every state row for the carry pass
    for (int e = 0; e < (TM == 1 ? p.E : 0); ++e) {
      const float u = s.U[e * 64 + lane];
      const float4* te = s.T + e * (SA ? 64 : kRowsDiag * 64) + lane;
      if constexpr (SA) {
        lg[0] = fmaf(u, te[0].x, lg[0]);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 a = te[q * 64];
          lg[4 * q + 0] = fmaf(u, a.x, lg[4 * q + 0]);
          lg[4 * q + 1] = fmaf(u, a.y, lg[4 * q + 1]);
          lg[4 * q + 2] = fmaf(u, a.z, lg[4 * q + 2]);
          lg[4 * q + 3] = fmaf(u, a.w, lg[4 * q + 3]);
        }
      }
    }
    if (active) {
      const size_t base = (((size_t)b * p.nchunks + c) * kN) * p.D + d;
#pragma unroll
      for (int n = 0; n < kN; ++n) {
        p.P[base + (size_t)n * p.D] = hw_exp2(lg[SA ? 0 : n]);
        p.H[base + (size_t)n * p.D] = h[n];
      }
    }
    gate_bad = __any(gate_bad);
    if (lane == 0) p.flags[((size_t)b * p.nchunks + c) * p.ntiles + tile] = (bad | gate_bad) ? 1 : 0;
  } else if (p.h_final != nullptr && active) {
#pragma unroll
    for (int n = 0; n < kN; ++n) p.h_final[((size_t)b * p.D + d) * kN + n] = h[n];
  }
}

// Pass 3: chunks 1.. re-run from their carried-in state until the carried part
// has decayed away (or to the chunk's end).
template <typename TIn, typename TOut, int WAVES, int K, bool SA, bool ZOH, int EMAX>
__global__ __launch_bounds__(WAVES * 64) void mix_fixup_kernel(MixParams p) {
  constexpr int TM = table_mode(EMAX, SA);
  constexpr bool TAB = TM >= 1;  // a table in LDS
  const int wave = uniform((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const Smem s = smem_layout(TAB ? p.E : 0, K > 0 ? K : p.k, wave, SA, TM);
  const int nfix = p.nchunks - 1;
  const int ncg = (nfix + WAVES - 1) / WAVES;
  int bid = blockIdx.x;
  const int tile = bid % p.ntiles;
  bid /= p.ntiles;
  const int cg = bid % ncg;
  const int b = bid / ncg;
  const int d0 = tile * 64, d = d0 + lane;
  const bool active = d < p.D;
  if constexpr (TAB) {
    load_table(p, const_cast<float4*>(s.T), d0, SA, TM);
    __syncthreads();
  }

  const int c = 1 + cg * WAVES + wave;
  if (c >= p.nchunks) return;
  const int t0 = c * p.chunk;
  const int t1 = min(p.L, t0 + p.chunk);
  const size_t base = (((size_t)b * p.nchunks + c) * kN) * p.D + (active ? d : 0);
  float h[kN], g[kN];
#pragma unroll
  for (int n = 0; n < kN; ++n) {
    h[n] = active ? p.H[base + (size_t)n * p.D] : 0.f;
    g[n] = h[n];
  }
  if (SA) {
    // the carried part is G * h_in: track G and max |h_in|
    float mh = 0.f;
#pragma unroll
    for (int n = 0; n < kN; ++n) mh = fmaxf(mh, fabsf(h[n]));
    g[0] = 1.f;
    g[1] = mh;
  }
  const bool truncate = p.carry == SWIMBA_CARRY_FIXUP &&
                        p.flags[((size_t)b * p.nchunks + c) * p.ntiles + tile] == 0;
  int gate_bad = 0;
  walk<TIn, TOut, K, true, false, SA, ZOH, TM>(p, s, nullptr, b, t0, t1, d, active,
                                                d0 + 64 <= p.D, lane, truncate, h, g, gate_bad);
}

template <typename TIn, typename TOut, int WAVES, int K, bool SA, bool ZOH, int EMAX>
int launch_mixed_t(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  MixParams p;
  p.B = a->B;
  p.L = a->L;
  p.D = a->D;
  p.E = a->E;
  p.k = a->k;
  p.chunk = pl.chunk;
  p.nchunks = pl.nchunks;
  p.ntiles = pl.ntiles;
  p.carry = a->carry == SWIMBA_CARRY_REWALK ? SWIMBA_CARRY_REWALK : SWIMBA_CARRY_FIXUP;
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
  p.y = a->y;
  p.h_final = a->h_final;
  char* w = static_cast<char*>(ws);
  p.P = pl.nchunks > 1 ? reinterpret_cast<float*>(w + pl.off_P) : nullptr;
  p.H = pl.nchunks > 1 ? reinterpret_cast<float*>(w + pl.off_H) : nullptr;
  p.flags = pl.nchunks > 1 ? reinterpret_cast<int32_t*>(w + pl.off_flags) : nullptr;

  constexpr int TM = table_mode(EMAX, SA);
  constexpr bool TAB = TM >= 1;
  const size_t smem1 = smem_bytes(TAB ? p.E : 0, p.k, WAVES, SA, TM);
  const size_t smem3 = smem1;
  p.tflags = nullptr;
  if (!TAB && pl.nchunks > 1) {
    // contraction check of every tile's A (the table path checks while staging)
    int32_t* tf = reinterpret_cast<int32_t*>(w + pl.off_tflags);
    p.tflags = tf;
    const int rc = launch_a_flags(p.A, p.E, p.D, SA, tf, st);
    if (rc != SWIMBA_OK) return rc;
  }
  const hipEvent_t* ev = a->phase_events;  // (start, end) x (chunk, carry, fix-up)
  if (pl.nchunks <= 1) {
    p.nchunks = 1;
    dim3 grid((unsigned)((size_t)p.B * p.ntiles));
    allow_dynamic_lds(mix_chunk_kernel<TIn, TOut, WAVES, K, false, SA, ZOH, EMAX>, smem3);
    const int rc = launch_timed(mix_chunk_kernel<TIn, TOut, WAVES, K, false, SA, ZOH, EMAX>, grid,
                                dim3(WAVES * 64), smem3, st, ev, p);
    if (rc != SWIMBA_OK) return rc;
    record_skipped(ev ? ev + 2 : nullptr, st);
    record_skipped(ev ? ev + 4 : nullptr, st);
    return SWIMBA_OK;
  }
  const int ncg = (p.nchunks + WAVES - 1) / WAVES;
  dim3 grid1((unsigned)((size_t)p.B * ncg * p.ntiles));
  allow_dynamic_lds(mix_chunk_kernel<TIn, TOut, WAVES, K, true, SA, ZOH, EMAX>, smem1);
  int rc = launch_timed(mix_chunk_kernel<TIn, TOut, WAVES, K, true, SA, ZOH, EMAX>, grid1,
                        dim3(WAVES * 64), smem1, st, ev, p);
  if (rc != SWIMBA_OK) return rc;
  rc = launch_carry(p.B, p.nchunks, p.D, p.E, p.P, p.H, p.h_final, 0, st, ev ? ev + 2 : nullptr);
  if (rc != SWIMBA_OK) return rc;
  const int ncg3 = (p.nchunks - 1 + WAVES - 1) / WAVES;
  dim3 grid3((unsigned)((size_t)p.B * ncg3 * p.ntiles));
  allow_dynamic_lds(mix_fixup_kernel<TIn, TOut, WAVES, K, SA, ZOH, EMAX>, smem3);
  return launch_timed(mix_fixup_kernel<TIn, TOut, WAVES, K, SA, ZOH, EMAX>, grid3, dim3(WAVES * 64),
                      smem3, st, ev ? ev + 4 : nullptr, p);
}

template <typename TIn, typename TOut, int WAVES, bool SA, bool ZOH, int EMAX>
int launch_mixed_e(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  switch (a->k) {
    case 1:
      return launch_mixed_t<TIn, TOut, WAVES, 1, SA, ZOH, EMAX>(a, pl, ws, st);
    case 2:
      return launch_mixed_t<TIn, TOut, WAVES, 2, SA, ZOH, EMAX>(a, pl, ws, st);
    default:
      return launch_mixed_t<TIn, TOut, WAVES, 0, SA, ZOH, EMAX>(a, pl, ws, st);
  }
}

template <typename TIn, typename TOut, int WAVES, bool SA, bool ZOH>
int launch_mixed_k(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  if (a->E <= 8) return launch_mixed_e<TIn, TOut, WAVES, SA, ZOH, 8>(a, pl, ws, st);
  if (a->E <= 16) return launch_mixed_e<TIn, TOut, WAVES, SA, ZOH, 16>(a, pl, ws, st);
  // 17..32 experts with a diagonal A: the A rows in LDS (table mode 2), with
  // eight waves (two per SIMD) whose rings fit beside the table
  if constexpr (WAVES == 8 && !SA) {
    if (a->E <= 32 && smem_bytes(a->E, a->k, 8, false, 2) <= kTabModeLds)
      return launch_mixed_e<TIn, TOut, WAVES, SA, ZOH, 32>(a, pl, ws, st);
  }
  return launch_mixed_e<TIn, TOut, WAVES, SA, ZOH, 64>(a, pl, ws, st);
}

template <typename TIn, typename TOut, int WAVES, bool SA>
int launch_mixed_z(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  if (a->disc == SWIMBA_DISC_ZOH) return launch_mixed_k<TIn, TOut, WAVES, SA, true>(a, pl, ws, st);
  return launch_mixed_k<TIn, TOut, WAVES, SA, false>(a, pl, ws, st);
}

template <typename TIn, typename TOut>
int launch_mixed_w(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  if (a->a_form == SWIMBA_A_SCALAR) {
    if (pl.waves == 8) return launch_mixed_z<TIn, TOut, 8, true>(a, pl, ws, st);
    return launch_mixed_z<TIn, TOut, 4, true>(a, pl, ws, st);
  }
  if (pl.waves == 8) return launch_mixed_z<TIn, TOut, 8, false>(a, pl, ws, st);
  return launch_mixed_z<TIn, TOut, 4, false>(a, pl, ws, st);
}

}  // namespace mixed
}  // namespace swimba
