// Stream-mixed Swimba scan for gfx950: the transition A is shared by the
// experts, and the experts' injections B X and readout vectors C are mixed by
// the router weights.
//
// Pages: "Swimba: Switch Mamba Model Scales State Space Models" (Dutch summary,
// "Kernmechanisme van Swimba": each expert emits B_t, C_t and X_t streams, A is
// shared, h_t = A h_{t-1} + sum_e pi_{t,e} B^(e)_t X^(e)_t and
// y_t = (sum_e pi_{t,e} C^(e)_t)^T h_t; French summary, "Architecture de
// Swimba": one recurrence over the mixed streams) and "Mamba y las SSMs: el
// retorno del estado persistente" ("Mamba": the selective transition
// exp(Delta A)).  The step size is not an expert stream, so Delta =
// softplus(dt_raw + dt_bias) is shared; the transition is exp(Delta A[d, n])
// and the mixed injection enters as Delta * sum_j g_j B_j[n] X_j[d].
//
// Layout of the work follows the parameter-mixed scan: a lane owns channel d
// of one sequence and keeps its 16 states in VGPRs for a chunk of tokens; the
// 64 lanes of a wave are consecutive channels of one token.  With A shared,
// the lane's transition row A[d, :] lives in VGPRs for the whole walk and
// nothing per channel is read from LDS.  What is wave-uniform per token, the
// gate-weighted B streams g_j B_j[:] and the mixed readout c = sum_j g_j C_j[:],
// is formed once per token while staging and read back from a per-wave LDS
// ring as broadcast 16-byte rows.  X (k slots), dt_raw and y stream as
// coalesced 64-lane rows through per-block buffer resources.
//
// Chunks are joined as in the parameter-mixed scan: a chunk pass from zero
// state (chunk 0 from h0) that also writes each chunk's end state and decay
// P[n] = exp2(A[d, n] log2(e) * sum_t Delta_t), the shared carry pass, and a
// fix-up pass that re-walks chunks >= 1 from their carried-in state until the
// carried part has decayed below fp32 resolution.  The decays do not depend
// on the gates, so A < 0 alone makes every decay lie in (0, 1].
#pragma once
#include <type_traits>

#include "scan_common.hpp"
#include "swimba_device.hpp"
#include "swimba_internal.hpp"

namespace swimba {
namespace streams {

using stage::kTB;
using stage::rsrc_t;
using stage::wave_sync;

constexpr float kFixupTol = 5.9604645e-08f;  // 2^-24
constexpr float kTiny = 1e-30f;
constexpr int kMaxSlots = 4;

struct StreamParams {
  int B, L, D, k;
  int chunk, nchunks, ntiles;
  int carry;  // SWIMBA_CARRY_REWALK or SWIMBA_CARRY_FIXUP
  const void* X;    // [B][L][k][D]
  const void* dt;   // [B][L][D]
  const void* Bs;   // [B][L][k][16]
  const void* Cs;   // [B][L][k][16]
  const float* gate;  // [B][L][k]
  const float* A;     // [D][16]
  const float* bias;  // [D]
  const float* h0;
  void* y;
  float* h_final;
  float* P;  // [B][C][16][D] chunk decays
  float* H;  // [B][C][16][D] chunk end states, then carried-in states
};

// Per-wave ring: two blocks of kTB tokens, each token a row of (K + 1) x 16
// floats: g_j B_j[0..15] for every slot j, then c[0..15].
__host__ __device__ constexpr int ring_floats(int K) { return 2 * kTB * (K + 1) * kN; }

// Staging loads of one block.  Lane l stages token l / 8 and the state pair
// 2 (l % 8), 2 (l % 8) + 1 of every slot's B and C; it forms g_j B_j and the
// mixed readout for that pair and writes them to the ring.
template <typename TIn, int K>
struct StreamStager {
  using raw_t = std::conditional_t<sizeof(TIn) == 2, uint32_t, stage::v2u>;
  uint32_t pair_off, gate_off;
  raw_t pb[K], pc[K];
  uint32_t g[K];

  __device__ __forceinline__ void init(int lane) {
    const int tok = lane >> 3, pr = lane & 7;
    pair_off = (uint32_t)((tok * K * kN + 2 * pr) * (int)sizeof(TIn));
    gate_off = (uint32_t)(tok * K * 4);
  }

  __device__ __forceinline__ static raw_t load_pair(rsrc_t r, uint32_t off) {
    if constexpr (sizeof(TIn) == 2)
      return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
    else
      return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
  }

  __device__ __forceinline__ static float2 unpack(raw_t v) {
    if constexpr (sizeof(TIn) == 2)
      return make_float2(__uint_as_float(v << 16), __uint_as_float(v & 0xffff0000u));
    else
      return make_float2(__uint_as_float(v.x), __uint_as_float(v.y));
  }

  // Tokens [tok, tok + kTB) (global token index); `valid` of them exist in
  // the tensors, the rest read as 0.
  __device__ __forceinline__ void issue(const StreamParams& p, size_t tok, int valid) {
    const rsrc_t rb = stage::rows_rsrc<TIn>(p.Bs, tok, valid, K * kN);
    const rsrc_t rc = stage::rows_rsrc<TIn>(p.Cs, tok, valid, K * kN);
    const rsrc_t rg = stage::rows_rsrc<float>(p.gate, tok, valid, K);
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const uint32_t o = pair_off + (uint32_t)(j * kN * (int)sizeof(TIn));
      pb[j] = load_pair(rb, o);
      pc[j] = load_pair(rc, o);
      g[j] = __builtin_amdgcn_raw_buffer_load_b32(rg, (int)(gate_off + 4u * j), 0, 0);
    }
  }

  __device__ __forceinline__ void commit(float* ring, int slot, int lane) const {
    const int tok = lane >> 3, pr = lane & 7;
    float* dst = ring + (slot * kTB + tok) * (K + 1) * kN + 2 * pr;
    float cx = 0.f, cy = 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const float gj = __uint_as_float(g[j]);
      const float2 b = unpack(pb[j]), c = unpack(pc[j]);
      *reinterpret_cast<float2*>(dst + j * kN) = make_float2(gj * b.x, gj * b.y);
      cx = fmaf(gj, c.x, cx);
      cy = fmaf(gj, c.y, cy);
    }
    *reinterpret_cast<float2*>(dst + K * kN) = make_float2(cx, cy);
  }
};

// One token for one lane: Delta, the transition of each state, the mixed
// injection and the mixed readout (after the update).  `row` is the token's
// ring row; al = A[d, :] log2(e).
template <int K, bool TRACK, bool ACC_S>
__device__ __forceinline__ float stream_token(const float* row, const float* xv, float rv,
                                              float bias, const float* al, float* h, float* g,
                                              float& S) {
  const float dlt = softplus_f32(rv + bias);
  if (ACC_S) S += dlt;
  float dx[K];
#pragma unroll
  for (int j = 0; j < K; ++j) dx[j] = dlt * xv[j];
  const float4* r = reinterpret_cast<const float4*>(row);
  float yv = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float4 gb[K];
#pragma unroll
    for (int j = 0; j < K; ++j) gb[j] = r[j * 4 + q];
    const float4 c4 = r[K * 4 + q];
    const float cv[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int n = 4 * q + rr;
      const float a = hw_exp2(dlt * al[n]);
      auto comp = [&](const float4& v) { return rr == 0 ? v.x : rr == 1 ? v.y : rr == 2 ? v.z : v.w; };
      float inj = comp(gb[0]) * dx[0];
#pragma unroll
      for (int j = 1; j < K; ++j) inj = fmaf(comp(gb[j]), dx[j], inj);
      h[n] = fmaf(a, h[n], inj);
      yv = fmaf(cv[rr], h[n], yv);
      if (TRACK) g[n] *= a;
    }
  }
  return yv;
}

// Walk tokens [t0, t1) of sequence b for one lane (see the mixed scan's walk:
// the next block's loads are issued before the current block computes).
template <typename TIn, typename TOut, int K, bool TRACK, bool ACC_S>
__device__ __forceinline__ void walk(const StreamParams& p, float* ring, int b, int t0, int t1,
                                     int d, bool active, bool full_tile, int lane, bool truncate,
                                     const float* al, float bias, float* h, float* g, float& S) {
  const int D = p.D;
  const size_t row = (size_t)b * p.L;
  const size_t total = (size_t)p.B * p.L;
  // lanes past D (ragged tile) read 0 and store nothing
  const uint32_t xoff = active ? (uint32_t)d * (uint32_t)sizeof(TIn) : stage::kOffNone;
  const uint32_t yoff = (uint32_t)d * (uint32_t)sizeof(TOut);
  const uint32_t drow = (uint32_t)D * (uint32_t)sizeof(TIn);
  const uint32_t xrow = (uint32_t)K * drow;
  const uint32_t yrow = (uint32_t)D * (uint32_t)sizeof(TOut);
  TIn xc[kTB][K], rc[kTB], xn[kTB][K], rn[kTB];
  StreamStager<TIn, K> st;
  st.init(lane);
  auto valid_at = [&](int t) { return (int)min((size_t)kTB, total - (row + t)); };
  auto load_xr = [&](int t, TIn (*xs)[K], TIn* rs) {
    const int v = valid_at(t);
    const rsrc_t rx = stage::rows_rsrc<TIn>(p.X, row + t, v, K * D);
    const rsrc_t rr = stage::rows_rsrc<TIn>(p.dt, row + t, v, D);
    // the scalar offset is not range-checked by the hardware: rows past the
    // tensor's end re-read its last row
#pragma unroll
    for (int i = 0; i < kTB; ++i) {
      const uint32_t ii = (uint32_t)min(i, v - 1);
#pragma unroll
      for (int j = 0; j < K; ++j) xs[i][j] = stage::buf_load<TIn>(rx, xoff, ii * xrow + j * drow);
      rs[i] = stage::buf_load<TIn>(rr, xoff, ii * drow);
    }
  };

  st.issue(p, row + t0, valid_at(t0));
  load_xr(t0, xc, rc);
  st.commit(ring, 0, lane);

  int slot = 0;
  for (int tb = t0; tb < t1; tb += kTB, slot ^= 1) {
    const int n = min(kTB, t1 - tb);
    const int tn = tb + kTB;
    const bool more = tn < t1;
    if (more) {
      st.issue(p, row + tn, valid_at(tn));
      load_xr(tn, xn, rn);
    }
    wave_sync();
    // stores past the block's n tokens fall outside this buffer and are dropped
    const rsrc_t ry = stage::rows_rsrc<TOut>(p.y, row + tb, n, D);
    const float* rows = ring + slot * kTB * (K + 1) * kN;
    if (n == kTB && full_tile) {
#pragma unroll
      for (int i = 0; i < kTB; ++i) {
        float xv[K];
#pragma unroll
        for (int j = 0; j < K; ++j) xv[j] = to_f32(xc[i][j]);
        const float yv = stream_token<K, TRACK, ACC_S>(rows + i * (K + 1) * kN, xv,
                                                       to_f32(rc[i]), bias, al, h, g, S);
        stage::buf_store(ry, yoff, (uint32_t)i * yrow, from_f32<TOut>(yv));
      }
    } else {
#pragma unroll
      for (int i = 0; i < kTB; ++i) {
        if (i < n) {
          float xv[K];
#pragma unroll
          for (int j = 0; j < K; ++j) xv[j] = active ? to_f32(xc[i][j]) : 0.f;
          const float rv = active ? to_f32(rc[i]) : 0.f;
          const float yv = stream_token<K, TRACK, ACC_S>(rows + i * (K + 1) * kN, xv, rv, bias,
                                                         al, h, g, S);
          if (active) stage::buf_store(ry, yoff, (uint32_t)i * yrow, from_f32<TOut>(yv));
        }
      }
    }
    if (TRACK && truncate) {
      float mh = 0.f;
#pragma unroll
      for (int q = 0; q < kN; ++q) mh = fmaxf(mh, fabsf(h[q]));
      const float thr = fmaxf(kFixupTol * mh, kTiny);
      bool conv = true;
#pragma unroll
      for (int q = 0; q < kN; ++q) conv &= fabsf(g[q]) <= thr;  // NaN: not converged
      if (__all(conv)) break;
    }
    if (more) {
      st.commit(ring, slot ^ 1, lane);
#pragma unroll
      for (int i = 0; i < kTB; ++i) {
#pragma unroll
        for (int j = 0; j < K; ++j) xc[i][j] = xn[i][j];
        rc[i] = rn[i];
      }
    }
  }
}

// The lane's shared-transition row (times log2 e) and step-size bias; returns
// whether any of its A entries fails A < 0 (NaN included).  Lanes past D
// read channel D - 1.
__device__ __forceinline__ bool lane_params(const StreamParams& p, int d, float* al,
                                            float& bias) {
  const int dc = d < p.D ? d : p.D - 1;
  const float4* a4 = reinterpret_cast<const float4*>(p.A + (size_t)dc * kN);
  bool bad = false;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 v = a4[q];
    const float w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      bad |= !(w[r] < 0.f);
      al[4 * q + r] = w[r] * kLog2e;
    }
  }
  bias = p.bias[dc];
  return bad;
}

// Grid: (sequence, chunk group, tile), tile fastest; the WAVES waves of a
// workgroup take consecutive chunks of one tile.  Waves share nothing, so a
// wave without a chunk returns at once.
struct WaveTask {
  int b, tile, c;
};
template <int WAVES>
__device__ __forceinline__ WaveTask wave_task(const StreamParams& p, int nwalk, int first) {
  const int wave = uniform((int)(threadIdx.x >> 6));
  const int ncg = (nwalk + WAVES - 1) / WAVES;
  int bid = blockIdx.x;
  WaveTask w;
  w.tile = bid % p.ntiles;
  bid /= p.ntiles;
  w.c = first + (bid % ncg) * WAVES + wave;
  w.b = bid / ncg;
  return w;
}

// Pass 1 (or the only pass when CHUNKED is false).
template <typename TIn, typename TOut, int WAVES, int K, bool CHUNKED>
__global__ __launch_bounds__(WAVES * 64) void stream_chunk_kernel(StreamParams p) {
  extern __shared__ float4 smem_streams[];
  const int lane = threadIdx.x & 63;
  const WaveTask w = wave_task<WAVES>(p, p.nchunks, 0);
  if (w.c >= p.nchunks) return;
  float* ring = reinterpret_cast<float*>(smem_streams) +
                uniform((int)(threadIdx.x >> 6)) * ring_floats(K);
  const int d0 = w.tile * 64, d = d0 + lane;
  const bool active = d < p.D;
  const int t0 = w.c * p.chunk;
  const int t1 = min(p.L, t0 + p.chunk);

  float al[kN], bias;
  lane_params(p, d, al, bias);
  float h[kN];
#pragma unroll
  for (int n = 0; n < kN; ++n)
    h[n] = (w.c == 0 && p.h0 != nullptr && active) ? p.h0[((size_t)w.b * p.D + d) * kN + n] : 0.f;

  float S = 0.f;
  walk<TIn, TOut, K, false, CHUNKED>(p, ring, w.b, t0, t1, d, active, d0 + 64 <= p.D, lane, false,
                                     al, bias, h, nullptr, S);
  if (!active) return;
  if (CHUNKED) {
    const size_t base = (((size_t)w.b * p.nchunks + w.c) * kN) * p.D + d;
#pragma unroll
    for (int n = 0; n < kN; ++n) {
      p.P[base + (size_t)n * p.D] = hw_exp2(S * al[n]);
      p.H[base + (size_t)n * p.D] = h[n];
    }
  } else if (p.h_final != nullptr) {
#pragma unroll
    for (int n = 0; n < kN; ++n) p.h_final[((size_t)w.b * p.D + d) * kN + n] = h[n];
  }
}

// Pass 3: chunks 1.. re-run from their carried-in state until the carried part
// has decayed away (or to the chunk's end).
template <typename TIn, typename TOut, int WAVES, int K>
__global__ __launch_bounds__(WAVES * 64) void stream_fixup_kernel(StreamParams p) {
  extern __shared__ float4 smem_streams[];
  const int lane = threadIdx.x & 63;
  const WaveTask w = wave_task<WAVES>(p, p.nchunks - 1, 1);
  if (w.c >= p.nchunks) return;
  float* ring = reinterpret_cast<float*>(smem_streams) +
                uniform((int)(threadIdx.x >> 6)) * ring_floats(K);
  const int d0 = w.tile * 64, d = d0 + lane;
  const bool active = d < p.D;
  const int t0 = w.c * p.chunk;
  const int t1 = min(p.L, t0 + p.chunk);

  float al[kN], bias;
  const bool bad = lane_params(p, d, al, bias) && active;
  const size_t base = (((size_t)w.b * p.nchunks + w.c) * kN) * p.D + (active ? d : 0);
  float h[kN], g[kN];
#pragma unroll
  for (int n = 0; n < kN; ++n) {
    h[n] = active ? p.H[base + (size_t)n * p.D] : 0.f;
    g[n] = h[n];
  }
  const bool truncate = p.carry == SWIMBA_CARRY_FIXUP && !__any(bad);
  float S = 0.f;
  walk<TIn, TOut, K, true, false>(p, ring, w.b, t0, t1, d, active, d0 + 64 <= p.D, lane, truncate,
                                  al, bias, h, g, S);
}

template <typename TIn, typename TOut, int K>
int launch_streams_t(const swimba_stream_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  constexpr int WAVES = 4;
  StreamParams p;
  p.B = a->B;
  p.L = a->L;
  p.D = a->D;
  p.k = a->k;
  p.chunk = pl.chunk;
  p.nchunks = pl.nchunks;
  p.ntiles = pl.ntiles;
  p.carry = a->carry == SWIMBA_CARRY_REWALK ? SWIMBA_CARRY_REWALK : SWIMBA_CARRY_FIXUP;
  p.X = a->X;
  p.dt = a->dt_raw;
  p.Bs = a->Bs;
  p.Cs = a->Cs;
  p.gate = a->gate;
  p.A = a->A;
  p.bias = a->dt_bias;
  p.h0 = a->h0;
  p.y = a->y;
  p.h_final = a->h_final;
  char* w = static_cast<char*>(ws);
  p.P = pl.nchunks > 1 ? reinterpret_cast<float*>(w + pl.off_P) : nullptr;
  p.H = pl.nchunks > 1 ? reinterpret_cast<float*>(w + pl.off_H) : nullptr;

  const size_t smem = (size_t)WAVES * ring_floats(K) * sizeof(float);
  const hipEvent_t* ev = a->phase_events;  // (start, end) x (chunk, carry, fix-up)
  const dim3 block(WAVES * 64);
  if (pl.nchunks <= 1) {
    p.nchunks = 1;
    const dim3 grid((unsigned)((size_t)p.B * p.ntiles));
    const int rc = launch_timed(stream_chunk_kernel<TIn, TOut, WAVES, K, false>, grid, block,
                                smem, st, ev, p);
    if (rc != SWIMBA_OK) return rc;
    record_skipped(ev ? ev + 2 : nullptr, st);
    record_skipped(ev ? ev + 4 : nullptr, st);
    return SWIMBA_OK;
  }
  const int ncg = (p.nchunks + WAVES - 1) / WAVES;
  const dim3 grid1((unsigned)((size_t)p.B * ncg * p.ntiles));
  int rc = launch_timed(stream_chunk_kernel<TIn, TOut, WAVES, K, true>, grid1, block, smem, st,
                        ev, p);
  if (rc != SWIMBA_OK) return rc;
  rc = launch_carry(p.B, p.nchunks, p.D, 1, p.P, p.H, p.h_final, 0, st, ev ? ev + 2 : nullptr);
  if (rc != SWIMBA_OK) return rc;
  const int ncg3 = (p.nchunks - 1 + WAVES - 1) / WAVES;
  const dim3 grid3((unsigned)((size_t)p.B * ncg3 * p.ntiles));
  return launch_timed(stream_fixup_kernel<TIn, TOut, WAVES, K>, grid3, block, smem, st,
                      ev ? ev + 4 : nullptr, p);
}

template <typename TIn, typename TOut>
int launch_streams_k(const swimba_stream_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  switch (a->k) {
    case 1:
      return launch_streams_t<TIn, TOut, 1>(a, pl, ws, st);
    case 2:
      return launch_streams_t<TIn, TOut, 2>(a, pl, ws, st);
    case 3:
      return launch_streams_t<TIn, TOut, 3>(a, pl, ws, st);
    case 4:
      return launch_streams_t<TIn, TOut, 4>(a, pl, ws, st);
    default:
      return SWIMBA_EUNSUPPORTED;
  }
}

}  // namespace streams
}  // namespace swimba
