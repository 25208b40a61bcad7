// Host-side launch interfaces between the C ABI (swimba_api.cpp) and the
// kernels.  Nothing here is exported.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "swimba.h"

namespace swimba {

// Chunk plan of one scan call.
struct ScanPlan {
  int ntiles = 0;       // 64-channel tiles: ceil(D / 64)
  int chunk = 0;        // tokens per chunk
  int nchunks = 0;      // ceil(L / chunk); <= 1 means a single pass
  int waves = 4;        // waves per workgroup (chunks sharing one table)
  size_t off_P = 0, off_H = 0, off_flags = 0, bytes = 0;  // workspace layout
  size_t off_tflags = 0;  // per-tile A checks (mixed scan with more than 16 experts)
};

// Plan of a backward call: the forward's chunking plus the workspace of the
// backward passes (all offsets 256-byte aligned).
struct BwdPlan {
  int ntiles = 0, chunk = 0, nchunks = 0, ncg = 0, waves = 4;
  int nbk = 0;  // block checkpoints per chunk: one before each block but the first
  size_t off_P = 0, off_H = 0, off_adj = 0, off_ckH = 0, off_ckG = 0, off_red = 0;
  size_t off_pA = 0, off_pBD = 0;
  size_t bytes = 0;
};

// Fills `p` for these arguments; returns a status.  Pure host arithmetic, with
// the compute-unit count of device `dev` (-1: the current device); a call
// plans for the device of its stream.
// design: 0 mixed, 1 separate per expert, 2 separate per routing slot, 3 separate
// per expert with every expert advancing at every token.
int plan_scan(const swimba_scan_args* a, int design, ScanPlan* p, int dev);
int plan_backward(const swimba_scan_grad_args* g, BwdPlan* p, int dev);
// Per-token channel sums of the backward's gradient pass: dB (16), dC (16)
// and the k gate terms, padded to an even count.
inline int backward_red_width(int k) { return 2 * SWIMBA_STATE_N + ((k + 1) & ~1); }
// LDS of the backward's gradient pass (four waves): the tile's expert tables
// (A, then dt_bias and Dskip), their gradient accumulators of the same
// shapes, a 512-byte sink, one staging ring shared by the waves, and the waves'
// per-token sums of one block.
inline size_t backward_grad_lds_bytes(int E, int k) {
  return (size_t)E * 64 * (2 * 16 * 4 + 2 * 8) + 128 * 4 +
         ((size_t)2 * 8 * 32 * 4 + (size_t)2 * 2 * 8 * k * 4) +
         (size_t)4 * 8 * (2 * SWIMBA_STATE_N + 4 * k) * 4;
}
// LDS of the backward's chunk pass: expert table and one staging ring per
// wave.
inline size_t backward_lds_bytes(int E, int k, int waves) {
  return (size_t)E * (4 * 64 * 16 + 64 * 8) +
         (size_t)waves * ((size_t)2 * 8 * 32 * 4 + (size_t)2 * 2 * 8 * k * 4);
}
int plan_streams(const swimba_stream_args* a, ScanPlan* p, int dev);

// Kernel launchers (validated arguments only).
int launch_route(const void* x, swimba_dtype xd, const float* Wr, int64_t T, int D, int E,
                 int k, int32_t* idx, float* gate, hipStream_t s);
int launch_scan(const swimba_scan_args* a, const ScanPlan& p, void* ws, hipStream_t s);
// all: every expert advances at every token (else only when selected)
int launch_scan_separate(const swimba_scan_args* a, const ScanPlan& p, void* ws, hipStream_t s,
                         bool all);
int launch_scan_slots(const swimba_scan_args* a, const ScanPlan& p, void* ws, hipStream_t s);
int launch_step(const swimba_step_args* a, hipStream_t s);
// Backward of the mixed scan, one launcher per (input, dL/dy) dtype pair.
int launch_backward_ff(const swimba_scan_grad_args* g, const BwdPlan& p, void* ws, hipStream_t s);
int launch_backward_fb(const swimba_scan_grad_args* g, const BwdPlan& p, void* ws, hipStream_t s);
int launch_backward_bf(const swimba_scan_grad_args* g, const BwdPlan& p, void* ws, hipStream_t s);
int launch_backward_bb(const swimba_scan_grad_args* g, const BwdPlan& p, void* ws, hipStream_t s);
// Stream-mixed scan, one launcher per (input, output) dtype pair.
int launch_streams_ff(const swimba_stream_args* a, const ScanPlan& p, void* ws, hipStream_t s);
int launch_streams_fb(const swimba_stream_args* a, const ScanPlan& p, void* ws, hipStream_t s);
int launch_streams_bf(const swimba_stream_args* a, const ScanPlan& p, void* ws, hipStream_t s);
int launch_streams_bb(const swimba_stream_args* a, const ScanPlan& p, void* ws, hipStream_t s);
// Pass 2 of the chunked scans: carried-in state per chunk (rows = 16, or 16 per
// trajectory: E * 16 per expert, k * 16 per routing slot, with E passed as the
// trajectory count).
int launch_carry(int B, int C, int D, int E, const float* P, float* H, float* h_final,
                 int separate, hipStream_t st, const hipEvent_t* ev);
// flags[tile] = 1 if any A of the tile's 64 channels is not negative.
int launch_a_flags(const float* A, int E, int D, bool scalar_a, int32_t* flags, hipStream_t st);

// Compute units of device `dev` (-1: the current device), cached per device.
int device_cus(int dev);
// The device a stream belongs to (the null stream: the current device); -1
// when HIP cannot tell.
int stream_device(hipStream_t s);

// Kernels that stage more than 64 KiB of dynamic LDS must say so before launch
// (gfx950 has 160 KiB per CU).
template <typename Kernel>
inline void allow_dynamic_lds(Kernel kernel, size_t bytes) {
  if (bytes > 65536)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

// Launch on `st`; when `ev` is given, ev[0] and ev[1] are stamped by the
// dispatch itself at the kernel's start and end (no extra stream packets).
template <typename... KArgs, typename... Args>
inline int launch_timed(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t smem,
                        hipStream_t st, const hipEvent_t* ev, Args... args) {
  if (ev)
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)smem, st, ev[0], ev[1], 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, smem, st, args...);
  return hipGetLastError() == hipSuccess ? SWIMBA_OK : SWIMBA_EHIP;
}

// Both events of a pass that does not run, recorded at this point of the stream.
inline void record_skipped(const hipEvent_t* ev, hipStream_t st) {
  if (ev) {
    (void)hipEventRecord(ev[0], st);
    (void)hipEventRecord(ev[1], st);
  }
}

}  // namespace swimba
