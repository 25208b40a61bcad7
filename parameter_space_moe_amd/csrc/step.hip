// One decoding step of the mixed Swimba scan on a persistent fp32 state, for
// gfx950.  Pages: "Mamba y las SSMs: el retorno del estado persistente"
// (Figure 2: the state persists across tokens and is updated once per token)
// and "Swimba: Switch Mamba Model Scales State Space Models" (Dutch summary,
// "Kernmechanisme van Swimba": route, mix the selected experts' parameters,
// one recurrence).
//
// The step moves 2 x 64 bytes of state per channel and does little arithmetic,
// so it is laid out for HBM streaming: four lanes share a channel and each owns
// four consecutive states (one float4), so a wave reads and writes 1 KiB of
// contiguous state per instruction.  The quad adds its partial readouts with
// two lane exchanges.  A workgroup of 16 waves handles one batch row (or one
// slice of a row when there are fewer rows than compute units).  When the
// routing is not given, the workgroup first computes the router for its row:
// 2*D bytes of x and the D x E router table, read once per row from L2, which
// costs less than a second launch and an HBM round trip of the routing.
#include "swimba_device.hpp"
#include "swimba_internal.hpp"

namespace swimba {
namespace {

// One workgroup of 16 waves per batch row (or per slice of a row when the
// batch is small): the row's router is computed once per workgroup, so Wr is
// read once per row per step.
constexpr int kStepThreads = 1024;
constexpr int kStepWaves = kStepThreads / 64;
constexpr int kStepChan = kStepThreads / 4;  // channels per workgroup iteration

struct StepParams {
  int B, D, E, k, slices;
  int scalar_a;  // A is [E][D]: one transition per expert and channel
  int zoh;       // zero-order-hold input term
  const void* x;
  const void* dt;
  const void* Bm;
  const void* Cm;
  const float* Wr;
  const int32_t* idx;
  const float* gate;
  int32_t* idx_out;
  float* gate_out;
  const float* A;
  const float* bias;
  const float* Dsk;
  float* state;
  void* y;
};

// Channels a thread handles per batch: all their loads are issued before any
// of them is used, so each thread keeps 4 x 16 bytes of state in flight.
constexpr int kBatch = 4;
// Channels a thread reads per round of the fused router (loads first): five
// per thread cover rows of up to 5120 channels in one round of loads.
constexpr int kRU = 5;

// A thread's loads of one batch: its quad of states of each of the kBatch
// channels, and x and dt_raw of the one channel whose scalar work it does
// (lane q of a quad: the batch's q-th channel).
template <typename TIn>
struct BatchLoads {
  float4 h[kBatch];
  TIn x, r;
};

// K > 0: k == K known at compile time (the parameter loads of a whole batch
// are issued together); K == 0: runtime k.  SA: A is [E][D] (K > 0 only; the
// runtime-k path reads p.scalar_a).  FUSED: the routing is computed here
// (p.Wr), else read from p.idx / p.gate.
template <typename TIn, typename TOut, int K, bool SA, bool FUSED>
__global__ __launch_bounds__(kStepThreads) void step_kernel(StepParams p) {
  __shared__ float s_part[kStepWaves][64];
  __shared__ int s_idx[64];
  __shared__ float s_gate[64];
  const int b = blockIdx.x / p.slices;
  const int slice = blockIdx.x % p.slices;
  const int tid = threadIdx.x, wave = uniform((int)(threadIdx.x >> 6)), lane = tid & 63;
  const TIn* X = reinterpret_cast<const TIn*>(p.x) + (size_t)b * p.D;
  const TIn* R = reinterpret_cast<const TIn*>(p.dt) + (size_t)b * p.D;
  const int per = (p.D + p.slices - 1) / p.slices;
  const int dbeg = slice * per, dend = min(p.D, dbeg + per);
  float4* St = reinterpret_cast<float4*>(p.state) + (size_t)b * p.D * 4;
  const int q = tid & 3;
  const int cl = tid >> 2;

  // state, x and dt_raw of this thread's first batch do not depend on the
  // routing: they start right after the router's first loads (loads retire
  // in issue order, so the router would otherwise wait for them)
  const int dsafe = dbeg < p.D ? dbeg : 0;  // a valid channel for idle loads
  auto issue = [&](int dc, BatchLoads<TIn>& L) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int d = dc + u * kStepChan + cl;
      const int dd = d < dend ? d : dsafe;
      // 32-bit offsets from the row's base (no 64-bit address arithmetic)
      L.h[u] = at32(St, (uint32_t)dd * 4 + q);
    }
    const int d = dc + q * kStepChan + cl;
    const int dd = d < dend ? d : dsafe;
    L.x = at32(X, (uint32_t)dd);
    L.r = at32(R, (uint32_t)dd);
  };
  BatchLoads<TIn> cur;

  if constexpr (!FUSED) {
    issue(dbeg, cur);
    if (tid < p.k) {
      int e = p.idx[(size_t)b * p.k + tid];
      s_idx[tid] = e < 0 ? 0 : (e >= p.E ? p.E - 1 : e);
      s_gate[tid] = p.gate[(size_t)b * p.k + tid];
    }
  } else {
    // router for row b (E <= 64): each thread sums a strided subset of the
    // channels (five at a time, loads first), then the wave adds with lane
    // exchanges and the waves add through LDS in a fixed order.  Rows of Wr
    // are read as 16-byte vectors when E is a multiple of 4 (one cache-line
    // visit per row instead of one per expert).
    const bool vec = (p.E & 3) == 0 && (reinterpret_cast<uintptr_t>(p.Wr) & 15) == 0;
    // Every workgroup reads all of Wr at the same time; starting each row at
    // a different channel spreads the reads over the L2 channels instead of
    // sending all compute units to the same lines at once.  The rotation
    // depends on the row only: the slices of a row add the same products in
    // the same order, so they compute bit-identical logits and agree on the
    // routing even at a near-tie.
    const int rot = (int)(((long long)b * 1031) % p.D);
    constexpr int kRound = kRU * kStepThreads;  // channels per round of loads
    // loads of one round: x at kRU channels and their Wr entries of experts
    // eb .. eb + 7, from clamped (valid) addresses, masked after
    auto round_loads = [&](int eb, int d0, float* xv, float (*wv)[8]) {
      const bool two = eb + 4 < p.E;  // the block's second group of 4 exists
#pragma unroll
      for (int u = 0; u < kRU; ++u) {
        const int d = d0 + u * kStepThreads;
        const bool ok = d < p.D;
        const int dr = d + rot;
        const int dd = ok ? (dr >= p.D ? dr - p.D : dr) : 0;
        const float xr = to_f32(X[dd]);
        xv[u] = ok ? xr : 0.f;
        if (vec) {
          const float4* w4 = reinterpret_cast<const float4*>(p.Wr + (size_t)dd * p.E + eb);
          const float4 lo = load_nt(w4), hi = load_nt(w4 + (two ? 1 : 0));
          wv[u][0] = lo.x;
          wv[u][1] = lo.y;
          wv[u][2] = lo.z;
          wv[u][3] = lo.w;
          wv[u][4] = hi.x;
          wv[u][5] = hi.y;
          wv[u][6] = hi.z;
          wv[u][7] = hi.w;
        } else {
          const float* w = p.Wr + (size_t)dd * p.E;
#pragma unroll
          for (int i = 0; i < 8; ++i) wv[u][i] = load_nt(w + min(eb + i, p.E - 1));
        }
      }
    };
    auto round_fma = [&](const float* xv, const float (*wv)[8], float* part) {
#pragma unroll
      for (int u = 0; u < kRU; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) part[i] = fmaf(xv[u], wv[u][i], part[i]);
    };
    // the first round's loads, then the state loads of the first batch, in
    // straight-line code: waiting for the router's data does not wait for
    // the state
    float xv0[kRU], wv0[kRU][8];
    round_loads(0, tid, xv0, wv0);
    issue(dbeg, cur);
    for (int eb = 0; eb < p.E; eb += 8) {
      float part[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) part[i] = 0.f;
      if (eb == 0) round_fma(xv0, wv0, part);
      for (int d0 = tid + (eb == 0 ? kRound : 0); d0 < p.D; d0 += kRound) {
        float xv[kRU], wv[kRU][8];
        round_loads(eb, d0, xv, wv);
        round_fma(xv, wv, part);
      }
      // the eight wave sums as one exchange tree: lane l ends with the sum
      // of partial l >> 3 (bits 5, 4, 3 select the partial, the rest is summed)
      float u4[4], u2[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) u4[i] = xchg_add<32>(part[i], part[i + 4]);
#pragma unroll
      for (int i = 0; i < 2; ++i) u2[i] = xchg_add<16>(u4[i], u4[i + 2]);
      const bool hi8 = (lane & 8) != 0;
      float v = (hi8 ? u2[1] : u2[0]) + xor_lane<8>(hi8 ? u2[0] : u2[1], lane);
      v += xor_lane<4>(v, lane);
      v += xor_lane<2>(v, lane);
      v += xor_lane<1>(v, lane);
      if ((lane & 7) == 0 && eb + (lane >> 3) < p.E) s_part[wave][eb + (lane >> 3)] = v;
    }
    __syncthreads();
    if (wave == 0) {
      // lane e holds logit e (waves added in order); top-k by a tournament
      // over the lanes: (logit desc, expert asc); softmax over the selected
      float v = 0.f;
      if (lane < p.E) {
#pragma unroll
        for (int w = 0; w < kStepWaves; ++w) v += s_part[w][lane];
      }
      bool free_e = lane < p.E;
      float m = 0.f, z = 0.f, my_l = 0.f;
      for (int j = 0; j < p.k; ++j) {
        float bv = v;
        int be = lane;
        bool bc = free_e;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          float ov;
          int oe, oci;
          if (off >= 16) {
            // lane swaps (bit moves, exact for the integer fields too)
            ov = off == 32 ? partner<32>(bv, lane) : partner<16>(bv, lane);
            oe = __float_as_int(off == 32 ? partner<32>(__int_as_float(be), lane)
                                          : partner<16>(__int_as_float(be), lane));
            oci = __float_as_int(off == 32 ? partner<32>(__int_as_float((int)bc), lane)
                                           : partner<16>(__int_as_float((int)bc), lane));
          } else {
            ov = xor_lane_any(bv, off, lane);
            oe = xor_lane_any(be, off, lane);
            oci = xor_lane_any((int)bc, off, lane);
          }
          const bool oc = oci != 0;
          bool take;
          if (!bc)
            take = oc;
          else if (!oc)
            take = false;
          else if (oe < be)
            take = !(bv > ov);
          else
            take = ov > bv;
          if (take) {
            bv = ov;
            be = oe;
            bc = true;
          }
        }
        if (lane == be) free_e = false;
        if (j == 0) m = bv;
        if (lane == j) {
          my_l = bv;
          s_idx[j] = be;
        }
        z += hw_exp2((bv - m) * kLog2e);
      }
      if (lane < p.k) s_gate[lane] = hw_exp2((my_l - m) * kLog2e) / z;
    }
  }
  __syncthreads();
  if (slice == 0 && tid < p.k) {
    if (p.idx_out) p.idx_out[(size_t)b * p.k + tid] = s_idx[tid];
    if (p.gate_out) p.gate_out[(size_t)b * p.k + tid] = s_gate[tid];
  }

  // state update: thread = (channel within the iteration, quad of states).
  // The per-channel scalars (Delta, the input and skip terms) are computed
  // once per channel: lane q of a quad for the batch's q-th channel, then
  // broadcast to the quad; lane q also stores that channel's y.
  const TIn* Bp = reinterpret_cast<const TIn*>(p.Bm) + (size_t)b * kN + 4 * q;
  const TIn* Cp = reinterpret_cast<const TIn*>(p.Cm) + (size_t)b * kN + 4 * q;
  float Bv[4], Cv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    Bv[i] = to_f32(Bp[i]);
    Cv[i] = to_f32(Cp[i]);
  }
  TOut* Y = reinterpret_cast<TOut*>(p.y) + (size_t)b * p.D;
  constexpr int KM = K > 0 ? K : 64;
  const int k = K > 0 ? K : p.k;
  int ev[K > 0 ? K : 1];
  float gv[K > 0 ? K : 1];
  const float* bzr[K > 0 ? K : 1];
  const float* dkr[K > 0 ? K : 1];
  const float* asr[K > 0 ? K : 1];
  const float4* avr[K > 0 ? K : 1];
  if constexpr (K > 0) {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      ev[j] = uniform(s_idx[j]);
      gv[j] = uniform(s_gate[j]);
      // the selected experts' rows (wave-uniform bases)
      bzr[j] = p.bias + (size_t)ev[j] * p.D;
      dkr[j] = p.Dsk + (size_t)ev[j] * p.D;
      asr[j] = p.A + (size_t)ev[j] * p.D;
      avr[j] = reinterpret_cast<const float4*>(p.A + (size_t)ev[j] * p.D * kN);
    }
  }
  const bool scalar_a = K > 0 ? SA : p.scalar_a != 0;
  (void)KM;
  for (int dc = dbeg; dc < dend; dc += kBatch * kStepChan) {
    const int dq = dc + q * kStepChan + cl;  // this lane's scalar channel
    const int ddq = dq < dend ? dq : dsafe;
    // the selected experts' parameters (L2): issued together and before the
    // next batch's state loads, so that waiting for them leaves the state
    // loads in flight
    float4 av[kBatch][K > 0 ? K : 1];
    float bz[K > 0 ? K : 1], dk[K > 0 ? K : 1];
    if constexpr (K > 0) {
#pragma unroll
      for (int j = 0; j < K; ++j) {
        bz[j] = at32(bzr[j], (uint32_t)ddq);
        dk[j] = at32(dkr[j], (uint32_t)ddq);
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int d = dc + u * kStepChan + cl;
        const int dd = d < dend ? d : dsafe;
#pragma unroll
        for (int j = 0; j < K; ++j)
          av[u][j] = SA ? make_float4(at32(asr[j], (uint32_t)dd), 0.f, 0.f, 0.f)
                        : at32(avr[j], (uint32_t)dd * 4 + q);
      }
    }
    // the next batch (past the end: a valid, unused reload), issued on
    // every iteration so every path has the same loads in flight
    BatchLoads<TIn> nxt;
    issue(dc + kBatch * kStepChan, nxt);
    // scalars of this lane's channel
    float beta = 0.f, delta = 0.f;
    if constexpr (K > 0) {
#pragma unroll
      for (int j = 0; j < K; ++j) {
        beta = fmaf(gv[j], bz[j], beta);
        delta = fmaf(gv[j], dk[j], delta);
      }
    } else {
      for (int j = 0; j < k; ++j) {
        const int e = s_idx[j];
        const float gj = s_gate[j];
        beta = fmaf(gj, p.bias[(size_t)e * p.D + ddq], beta);
        delta = fmaf(gj, p.Dsk[(size_t)e * p.D + ddq], delta);
      }
    }
    const float xq = to_f32(cur.x);
    const float dltq = softplus_f32(to_f32(cur.r) + beta);
    const float dl2q = dltq * kLog2e, dxq = dltq * xq, skq = delta * xq;
    float yq = 0.f;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int d = dc + u * kStepChan + cl;
      const bool active = d < dend;
      // channel u's scalars from quad lane u
      float dl2, dx, sk;
      if (u == 0) {
        dl2 = dpp_mov<0x00>(dl2q), dx = dpp_mov<0x00>(dxq), sk = dpp_mov<0x00>(skq);
      } else if (u == 1) {
        dl2 = dpp_mov<0x55>(dl2q), dx = dpp_mov<0x55>(dxq), sk = dpp_mov<0x55>(skq);
      } else if (u == 2) {
        dl2 = dpp_mov<0xAA>(dl2q), dx = dpp_mov<0xAA>(dxq), sk = dpp_mov<0xAA>(skq);
      } else {
        dl2 = dpp_mov<0xFF>(dl2q), dx = dpp_mov<0xFF>(dxq), sk = dpp_mov<0xFF>(skq);
      }
      float m[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (K > 0) {
#pragma unroll
        for (int j = 0; j < K; ++j) {
          m[0] = fmaf(gv[j], av[u][j].x, m[0]);
          m[1] = fmaf(gv[j], av[u][j].y, m[1]);
          m[2] = fmaf(gv[j], av[u][j].z, m[2]);
          m[3] = fmaf(gv[j], av[u][j].w, m[3]);
        }
      } else {
        const int dd = active ? d : dsafe;
        for (int j = 0; j < k; ++j) {
          const int e = s_idx[j];
          const float gj = s_gate[j];
          const float4 a =
              scalar_a ? make_float4(p.A[(size_t)e * p.D + dd], 0.f, 0.f, 0.f)
                       : *reinterpret_cast<const float4*>(p.A + ((size_t)e * p.D + dd) * kN +
                                                          4 * q);
          m[0] = fmaf(gj, a.x, m[0]);
          m[1] = fmaf(gj, a.y, m[1]);
          m[2] = fmaf(gj, a.z, m[2]);
          m[3] = fmaf(gj, a.w, m[3]);
        }
      }
      if (scalar_a) m[1] = m[2] = m[3] = m[0];
      float hv[4] = {cur.h[u].x, cur.h[u].y, cur.h[u].z, cur.h[u].w};
      float yv = 0.f;
      // the input term is chosen once per channel, not per state
      if (p.zoh) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = hw_exp2(dl2 * m[i]);
          hv[i] = fmaf(a, hv[i], (dx * Bv[i]) * zoh_phi(a, dl2 * m[i]));
          yv = fmaf(Cv[i], hv[i], yv);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          hv[i] = fmaf(hw_exp2(dl2 * m[i]), hv[i], dx * Bv[i]);
          yv = fmaf(Cv[i], hv[i], yv);
        }
      }
      // quad sum of the readout (lanes 4c..4c+3 hold one channel)
      yv += xor_lane<1>(yv, lane);
      yv += xor_lane<2>(yv, lane);
      if (q == u) yq = yv + sk;
      if (active) at32(St, (uint32_t)d * 4 + q) = make_float4(hv[0], hv[1], hv[2], hv[3]);
    }
    if (dq < dend) at32(Y, (uint32_t)dq) = from_f32<TOut>(yq);
    cur = nxt;
  }
}

template <typename TIn, typename TOut, bool FUSED>
int launch_step_k(int k, bool scalar_a, dim3 grid, dim3 block, const StepParams& p,
                  hipStream_t s) {
  if (k == 1 && scalar_a)
    hipLaunchKernelGGL((step_kernel<TIn, TOut, 1, true, FUSED>), grid, block, 0, s, p);
  else if (k == 1)
    hipLaunchKernelGGL((step_kernel<TIn, TOut, 1, false, FUSED>), grid, block, 0, s, p);
  else if (k == 2 && scalar_a)
    hipLaunchKernelGGL((step_kernel<TIn, TOut, 2, true, FUSED>), grid, block, 0, s, p);
  else if (k == 2)
    hipLaunchKernelGGL((step_kernel<TIn, TOut, 2, false, FUSED>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((step_kernel<TIn, TOut, 0, false, FUSED>), grid, block, 0, s, p);
  return hipGetLastError() == hipSuccess ? SWIMBA_OK : SWIMBA_EHIP;
}

template <typename TIn, typename TOut>
int launch_step_t(const swimba_step_args* a, hipStream_t s) {
  StepParams p;
  p.B = a->B;
  p.D = a->D;
  p.E = a->E;
  p.k = a->k;
  // one workgroup per row; small batches split rows so every CU has work
  const int cus = device_cus(stream_device(s));
  int slices = (cus + a->B - 1) / (a->B > 0 ? a->B : 1);
  const int maxs = (a->D + kStepChan - 1) / kStepChan;
  slices = slices < 1 ? 1 : (slices > maxs ? maxs : slices);
  p.slices = slices;
  p.x = a->x;
  p.dt = a->dt_raw;
  p.Bm = a->Bm;
  p.Cm = a->Cm;
  p.Wr = a->Wr;
  p.idx = a->idx;
  p.gate = a->gate;
  p.idx_out = a->idx_out;
  p.gate_out = a->gate_out;
  p.A = a->A;
  p.scalar_a = a->a_form == SWIMBA_A_SCALAR;
  p.zoh = a->disc == SWIMBA_DISC_ZOH;
  p.bias = a->dt_bias;
  p.Dsk = a->Dskip;
  p.state = a->state;
  p.y = a->y;
  const dim3 grid((unsigned)((size_t)a->B * slices)), block(kStepThreads);
  if (a->idx != nullptr) return launch_step_k<TIn, TOut, false>(a->k, p.scalar_a, grid, block, p, s);
  return launch_step_k<TIn, TOut, true>(a->k, p.scalar_a, grid, block, p, s);
}

}  // namespace

int launch_step(const swimba_step_args* a, hipStream_t s) {
  if (a->B == 0) return SWIMBA_OK;
  const bool in_bf = a->in_dtype == SWIMBA_BF16, out_bf = a->y_dtype == SWIMBA_BF16;
  if (in_bf && out_bf) return launch_step_t<bf16_t, bf16_t>(a, s);
  if (in_bf) return launch_step_t<bf16_t, float>(a, s);
  if (out_bf) return launch_step_t<float, bf16_t>(a, s);
  return launch_step_t<float, float>(a, s);
}

}  // namespace swimba
