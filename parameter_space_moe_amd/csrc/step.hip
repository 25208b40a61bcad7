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
// two lane exchanges.  A workgroup handles one slice of one batch row; when the
// routing is not given, every workgroup first computes the router for its row
// (the row is 2*D bytes, read from L2), which costs far less than a second
// launch.
#include "swimba_device.hpp"
#include "swimba_internal.hpp"

namespace swimba {
namespace {

constexpr int kStepThreads = 256;
constexpr int kStepChan = kStepThreads / 4;  // channels per workgroup iteration

struct StepParams {
  int B, D, E, k, slices;
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

template <typename TIn, typename TOut>
__global__ __launch_bounds__(kStepThreads) void step_kernel(StepParams p) {
  __shared__ float s_part[kStepThreads / 64][64];
  __shared__ int s_idx[64];
  __shared__ float s_gate[64];
  const int b = blockIdx.x / p.slices;
  const int slice = blockIdx.x % p.slices;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const TIn* X = reinterpret_cast<const TIn*>(p.x) + (size_t)b * p.D;
  const TIn* R = reinterpret_cast<const TIn*>(p.dt) + (size_t)b * p.D;

  if (p.idx != nullptr) {
    if (tid < p.k) {
      int e = p.idx[(size_t)b * p.k + tid];
      s_idx[tid] = e < 0 ? 0 : (e >= p.E ? p.E - 1 : e);
      s_gate[tid] = p.gate[(size_t)b * p.k + tid];
    }
  } else {
    // router for row b (E <= 64): each thread sums a strided subset of the
    // channels, then the wave adds with lane exchanges and the four waves add
    // through LDS in a fixed order.
    for (int eb = 0; eb < p.E; eb += 8) {
      float part[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) part[i] = 0.f;
      for (int d = tid; d < p.D; d += kStepThreads) {
        const float xv = to_f32(X[d]);
        const float* w = p.Wr + (size_t)d * p.E + eb;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (eb + i < p.E) part[i] = fmaf(xv, w[i], part[i]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float v = part[i];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
        if (lane == 0 && eb + i < p.E) s_part[wave][eb + i] = v;
      }
    }
    __syncthreads();
    if (tid < p.E) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kStepThreads / 64; ++w) v += s_part[w][tid];
      s_part[0][tid] = v;  // column tid is read and written by thread tid only
    }
    __syncthreads();
    if (tid == 0) {
      // top-k by (logit desc, expert asc); softmax over the selected logits
      uint64_t taken = 0;
      float m = 0.f, z = 0.f;
      for (int j = 0; j < p.k; ++j) {
        int best = -1;
        float bv = 0.f;
        for (int e = 0; e < p.E; ++e) {
          if ((taken >> e) & 1ull) continue;
          const float v = s_part[0][e];
          if (best < 0 || v > bv) {
            best = e;
            bv = v;
          }
        }
        taken |= 1ull << best;
        if (j == 0) m = bv;
        s_idx[j] = best;
        s_gate[j] = bv;
      }
      for (int j = 0; j < p.k; ++j) z += hw_exp2((s_gate[j] - m) * kLog2e);
      for (int j = 0; j < p.k; ++j) s_gate[j] = hw_exp2((s_gate[j] - m) * kLog2e) / z;
    }
  }
  __syncthreads();
  if (slice == 0 && tid < p.k) {
    if (p.idx_out) p.idx_out[(size_t)b * p.k + tid] = s_idx[tid];
    if (p.gate_out) p.gate_out[(size_t)b * p.k + tid] = s_gate[tid];
  }

  // state update: thread = (channel within the iteration, quad of states)
  const int q = tid & 3;
  const int cl = tid >> 2;
  const TIn* Bp = reinterpret_cast<const TIn*>(p.Bm) + (size_t)b * kN + 4 * q;
  const TIn* Cp = reinterpret_cast<const TIn*>(p.Cm) + (size_t)b * kN + 4 * q;
  float Bv[4], Cv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    Bv[i] = to_f32(Bp[i]);
    Cv[i] = to_f32(Cp[i]);
  }
  const int per = (p.D + p.slices - 1) / p.slices;
  const int dbeg = slice * per, dend = min(p.D, dbeg + per);
  TOut* Y = reinterpret_cast<TOut*>(p.y) + (size_t)b * p.D;
  float4* St = reinterpret_cast<float4*>(p.state) + (size_t)b * p.D * 4;
  for (int dc = dbeg; dc < dend; dc += kStepChan) {
    const int d = dc + cl;
    const bool active = d < dend;
    const int dd = active ? d : dbeg;
    float4 h = St[(size_t)dd * 4 + q];
    const float xv = to_f32(X[dd]), rv = to_f32(R[dd]);
    float beta = 0.f, delta = 0.f;
    float m[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < p.k; ++j) {
      const int e = s_idx[j];
      const float gj = s_gate[j];
      beta = fmaf(gj, p.bias[(size_t)e * p.D + dd], beta);
      delta = fmaf(gj, p.Dsk[(size_t)e * p.D + dd], delta);
      const float4 a = *reinterpret_cast<const float4*>(p.A + ((size_t)e * p.D + dd) * kN + 4 * q);
      m[0] = fmaf(gj, a.x, m[0]);
      m[1] = fmaf(gj, a.y, m[1]);
      m[2] = fmaf(gj, a.z, m[2]);
      m[3] = fmaf(gj, a.w, m[3]);
    }
    const float dlt = softplus_f32(rv + beta);
    const float dl2 = dlt * kLog2e, dx = dlt * xv;
    float hv[4] = {h.x, h.y, h.z, h.w};
    float yv = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = hw_exp2(dl2 * m[i]);
      hv[i] = fmaf(a, hv[i], dx * Bv[i]);
      yv = fmaf(Cv[i], hv[i], yv);
    }
    // quad sum of the readout (lanes 4c..4c+3 hold one channel)
    yv += __shfl_xor(yv, 1, 64);
    yv += __shfl_xor(yv, 2, 64);
    if (active) {
      St[(size_t)d * 4 + q] = make_float4(hv[0], hv[1], hv[2], hv[3]);
      if (q == 0) Y[d] = from_f32<TOut>(fmaf(delta, xv, yv));
    }
  }
}

template <typename TIn, typename TOut>
int launch_step_t(const swimba_step_args* a, hipStream_t s) {
  StepParams p;
  p.B = a->B;
  p.D = a->D;
  p.E = a->E;
  p.k = a->k;
  // enough workgroups to fill the chip: ~4 per CU
  const int cus = device_cus();
  int slices = (4 * cus + a->B - 1) / (a->B > 0 ? a->B : 1);
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
  p.bias = a->dt_bias;
  p.Dsk = a->Dskip;
  p.state = a->state;
  p.y = a->y;
  hipLaunchKernelGGL((step_kernel<TIn, TOut>), dim3((unsigned)((size_t)a->B * slices)),
                     dim3(kStepThreads), 0, s, p);
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
