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

template <typename TIn>
struct ChanLoads {
  float4 h;
  TIn x, r;
};

// K > 0: k == K known at compile time (the parameter loads of a whole batch
// are issued together); K == 0: runtime k.  SA: A is [E][D] (K > 0 only; the
// runtime-k path reads p.scalar_a).
template <typename TIn, typename TOut, int K, bool SA>
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
  // routing: start them before the router
  auto issue = [&](int dc, ChanLoads<TIn>* L) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int d = dc + u * kStepChan + cl;
      const int dd = d < dend ? d : dbeg;
      // 32-bit offsets from the row's base (no 64-bit address arithmetic)
      L[u].h = at32(St, (uint32_t)dd * 4 + q);
      L[u].x = at32(X, (uint32_t)dd);
      L[u].r = at32(R, (uint32_t)dd);
    }
  };
  ChanLoads<TIn> cur[kBatch];
  if (dbeg < dend) issue(dbeg, cur);

  if (p.idx != nullptr) {
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
    for (int eb = 0; eb < p.E; eb += 8) {
      const bool two = eb + 4 < p.E;  // the block's second group of 4 exists
      float part[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) part[i] = 0.f;
      for (int d0 = tid; d0 < p.D; d0 += kRU * kStepThreads) {
        float xv[kRU], wv[kRU][8];
        // unconditional loads from clamped (valid) addresses, masked after:
        // a load under a branch would be waited on inside that branch
        if (vec) {
#pragma unroll
          for (int u = 0; u < kRU; ++u) {
            const int d = d0 + u * kStepThreads;
            const bool ok = d < p.D;
            const int dr = d + rot;
            const int dd = ok ? (dr >= p.D ? dr - p.D : dr) : 0;
            const float xr = to_f32(X[dd]);
            xv[u] = ok ? xr : 0.f;
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
          }
        } else {
#pragma unroll
          for (int u = 0; u < kRU; ++u) {
            const int d = d0 + u * kStepThreads;
            const bool ok = d < p.D;
            const int dr = d + rot;
            const int dd = ok ? (dr >= p.D ? dr - p.D : dr) : 0;
            const float xr = to_f32(X[dd]);
            xv[u] = ok ? xr : 0.f;
            const float* w = p.Wr + (size_t)dd * p.E;
#pragma unroll
            for (int i = 0; i < 8; ++i) wv[u][i] = load_nt(w + min(eb + i, p.E - 1));
          }
        }
#pragma unroll
        for (int u = 0; u < kRU; ++u)
#pragma unroll
          for (int i = 0; i < 8; ++i) part[i] = fmaf(xv[u], wv[u][i], part[i]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float v = part[i];
        v = wave_sum64(v);
        if (lane == 0 && eb + i < p.E) s_part[wave][eb + i] = v;
      }
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

  // state update: thread = (channel within the iteration, quad of states)
  const TIn* Bp = reinterpret_cast<const TIn*>(p.Bm) + (size_t)b * kN + 4 * q;
  const TIn* Cp = reinterpret_cast<const TIn*>(p.Cm) + (size_t)b * kN + 4 * q;
  float Bv[4], Cv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    Bv[i] = to_f32(Bp[i]);
    Cv[i] = to_f32(Cp[i]);
  }
  TOut* Y = reinterpret_cast<TOut*>(p.y) + (size_t)b * p.D;
  if constexpr (K > 0) {
    int ev[K];
    float gv[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      ev[j] = uniform(s_idx[j]);
      gv[j] = uniform(s_gate[j]);
    }
    // the selected experts' rows (wave-uniform bases)
    const float* bzr[K];
    const float* dkr[K];
    const float* asr[K];
    const float4* avr[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      bzr[j] = p.bias + (size_t)ev[j] * p.D;
      dkr[j] = p.Dsk + (size_t)ev[j] * p.D;
      asr[j] = p.A + (size_t)ev[j] * p.D;
      avr[j] = reinterpret_cast<const float4*>(p.A + (size_t)ev[j] * p.D * kN);
    }
    for (int dc = dbeg; dc < dend; dc += kBatch * kStepChan) {
      // the selected experts' parameters of this batch's channels (L2): all
      // issued together and before the next batch's state loads, so that
      // waiting for them leaves the state loads in flight
      float4 av[kBatch][K];
      float bz[kBatch][K], dk[kBatch][K];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int d = dc + u * kStepChan + cl;
        const int dd = d < dend ? d : dbeg;
#pragma unroll
        for (int j = 0; j < K; ++j) {
          bz[u][j] = at32(bzr[j], (uint32_t)dd);
          dk[u][j] = at32(dkr[j], (uint32_t)dd);
          av[u][j] = SA ? make_float4(at32(asr[j], (uint32_t)dd), 0.f, 0.f, 0.f)
                        : at32(avr[j], (uint32_t)dd * 4 + q);
        }
      }
      // the next batch (past the end: a valid, unused reload of the first
      // channels), issued on every iteration so every path has the same
      // loads in flight
      ChanLoads<TIn> nxt[kBatch];
      issue(dc + kBatch * kStepChan, nxt);
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int d = dc + u * kStepChan + cl;
        const bool active = d < dend;
        const float xv = to_f32(cur[u].x), rv = to_f32(cur[u].r);
        float beta = 0.f, delta = 0.f;
        float m[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < K; ++j) {
          beta = fmaf(gv[j], bz[u][j], beta);
          delta = fmaf(gv[j], dk[u][j], delta);
          m[0] = fmaf(gv[j], av[u][j].x, m[0]);
          m[1] = fmaf(gv[j], av[u][j].y, m[1]);
          m[2] = fmaf(gv[j], av[u][j].z, m[2]);
          m[3] = fmaf(gv[j], av[u][j].w, m[3]);
        }
        if (SA) m[1] = m[2] = m[3] = m[0];
        const float dlt = softplus_f32(rv + beta);
        const float dl2 = dlt * kLog2e, dx = dlt * xv;
        float hv[4] = {cur[u].h.x, cur[u].h.y, cur[u].h.z, cur[u].h.w};
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
        if (active) {
          at32(St, (uint32_t)d * 4 + q) = make_float4(hv[0], hv[1], hv[2], hv[3]);
          if (q == 0) at32(Y, (uint32_t)d) = from_f32<TOut>(fmaf(delta, xv, yv));
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) cur[u] = nxt[u];
    }
    return;
  }
  for (int dc = dbeg; dc < dend; dc += kBatch * kStepChan) {
    ChanLoads<TIn> nxt[kBatch];
    const int dn = dc + kBatch * kStepChan;
    if (dn < dend) issue(dn, nxt);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int d = dc + u * kStepChan + cl;
      const bool active = d < dend;
      const int dd = active ? d : dbeg;
      const float xv = to_f32(cur[u].x), rv = to_f32(cur[u].r);
      float beta = 0.f, delta = 0.f;
      float m[4] = {0.f, 0.f, 0.f, 0.f};
      for (int j = 0; j < p.k; ++j) {
        const int e = s_idx[j];
        const float gj = s_gate[j];
        beta = fmaf(gj, p.bias[(size_t)e * p.D + dd], beta);
        delta = fmaf(gj, p.Dsk[(size_t)e * p.D + dd], delta);
        const float4 a =
            p.scalar_a
                ? make_float4(p.A[(size_t)e * p.D + dd], 0.f, 0.f, 0.f)
                : *reinterpret_cast<const float4*>(p.A + ((size_t)e * p.D + dd) * kN + 4 * q);
        m[0] = fmaf(gj, a.x, m[0]);
        m[1] = fmaf(gj, a.y, m[1]);
        m[2] = fmaf(gj, a.z, m[2]);
        m[3] = fmaf(gj, a.w, m[3]);
      }
      if (p.scalar_a) m[1] = m[2] = m[3] = m[0];
      const float dlt = softplus_f32(rv + beta);
      const float dl2 = dlt * kLog2e, dx = dlt * xv;
      float hv[4] = {cur[u].h.x, cur[u].h.y, cur[u].h.z, cur[u].h.w};
      float yv = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = hw_exp2(dl2 * m[i]);
        const float inj = p.zoh ? (dx * Bv[i]) * zoh_phi(a, dl2 * m[i]) : dx * Bv[i];
        hv[i] = fmaf(a, hv[i], inj);
        yv = fmaf(Cv[i], hv[i], yv);
      }
      // quad sum of the readout (lanes 4c..4c+3 hold one channel)
      yv += xor_lane<1>(yv, lane);
      yv += xor_lane<2>(yv, lane);
      if (active) {
        St[(size_t)d * 4 + q] = make_float4(hv[0], hv[1], hv[2], hv[3]);
        if (q == 0) Y[d] = from_f32<TOut>(fmaf(delta, xv, yv));
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) cur[u] = nxt[u];
  }
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
  if (a->k == 1 && p.scalar_a)
    hipLaunchKernelGGL((step_kernel<TIn, TOut, 1, true>), grid, block, 0, s, p);
  else if (a->k == 1)
    hipLaunchKernelGGL((step_kernel<TIn, TOut, 1, false>), grid, block, 0, s, p);
  else if (a->k == 2 && p.scalar_a)
    hipLaunchKernelGGL((step_kernel<TIn, TOut, 2, true>), grid, block, 0, s, p);
  else if (a->k == 2)
    hipLaunchKernelGGL((step_kernel<TIn, TOut, 2, false>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((step_kernel<TIn, TOut, 0, false>), grid, block, 0, s, p);
  return hipGetLastError() == hipSuccess ? SWIMBA_OK : SWIMBA_EHIP;
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
