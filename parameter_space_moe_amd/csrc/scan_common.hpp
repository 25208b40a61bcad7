// Shared staging pieces of the chunked scans (mixed and separate designs):
// the per-wave LDS ring of wave-uniform per-token data, its vector-load
// staging one block ahead, and the expert table of a 64-channel tile.
//
// Parameter structs used with these templates provide: int L, E; const void
// *Bm, *Cm; const int32_t* idx; const float* gate, *A, *bias, *Dsk; int D.
#pragma once
#include "swimba_device.hpp"
#include "swimba_internal.hpp"

namespace swimba {
namespace stage {

constexpr int kTB = 8;  // tokens per staging block

// Per-wave LDS ring holding the wave-uniform data of two blocks of kTB tokens:
// B_t and C_t as fp32 (32 floats per token), the selected experts and gates.
struct Ring {
  float* bc;    // [2][kTB][32]
  int32_t* e;   // [2][kTB][k]
  float* g;     // [2][kTB][k]
  int32_t* uo = nullptr;  // [2][kTB][k] or null: a second scaled copy of e (commit)
};

__host__ __device__ constexpr size_t ring_bytes(int k) {
  return (size_t)2 * kTB * 32 * 4 + (size_t)2 * 2 * kTB * k * 4;
}

// Stage the tile's expert parameters; returns 1 if any A in the tile is not
// strictly negative (including NaN).  scalar_a: A is [E][D] (one transition
// per expert and channel) and the table [E][64] floats.
template <typename P>
__device__ __forceinline__ int load_table(const P& p, float4* sA, float2* sBD, int d0,
                                          bool scalar_a) {
  int bad = 0;
  const int nthr = blockDim.x;
  if (scalar_a) {
    float* sAs = reinterpret_cast<float*>(sA);
    for (int i = threadIdx.x; i < p.E * 64; i += nthr) {
      const int e = i >> 6, d = d0 + (i & 63);
      float v = 0.f;
      if (d < p.D) {
        v = p.A[(size_t)e * p.D + d];
        bad |= !(v < 0.f);
      }
      sAs[i] = v;
    }
  }
  for (int i = threadIdx.x; i < (scalar_a ? 0 : p.E * 256); i += nthr) {
    int e = i >> 8, r = i & 255, dl = r >> 2, q = r & 3;
    int d = d0 + dl;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (d < p.D) {
      const float* a = p.A + ((size_t)e * p.D + d) * kN + q * 4;
      v = make_float4(a[0], a[1], a[2], a[3]);
      bad |= !(v.x < 0.f) | !(v.y < 0.f) | !(v.z < 0.f) | !(v.w < 0.f);
    }
    sA[(e * 4 + q) * 64 + dl] = v;
  }
  for (int i = threadIdx.x; i < p.E * 64; i += nthr) {
    int e = i >> 6, dl = i & 63, d = d0 + dl;
    float2 v = make_float2(0.f, 0.f);
    if (d < p.D) v = make_float2(p.bias[(size_t)e * p.D + d], p.Dsk[(size_t)e * p.D + d]);
    sBD[i] = v;
  }
  return bad;
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// Buffer-resource addressing.  Every streamed tensor is read and written as a
// raw buffer whose base is the current block's first token: the per-lane part
// of each address is a loop-invariant VGPR offset, the per-token part a scalar
// offset, so the walk spends no vector instructions on addresses.  A buffer's
// size is the valid part of the block: loads whose per-lane offset falls past
// it return 0 and such stores are dropped.  The scalar offset is not part of
// that check, so callers keep scalar offsets inside the valid rows.
using rsrc_t = __amdgpu_buffer_rsrc_t;

// A per-lane offset past every buffer's size: loads with it return 0.  Lanes
// of a ragged tile (channel >= D) use it, because their channel offset alone
// can pass the range check while the unchecked scalar offset moves the
// address past the tensor's last row.
constexpr uint32_t kOffNone = 0x80000000u;
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // third dword of a raw (untyped, unswizzled) buffer on gfx9-family parts
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

template <typename T>
__device__ __forceinline__ T buf_load(rsrc_t r, uint32_t voff, uint32_t soff);
template <>
__device__ __forceinline__ bf16_t buf_load<bf16_t>(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
}
template <>
__device__ __forceinline__ float buf_load<float>(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0));
}

__device__ __forceinline__ void buf_store(rsrc_t r, uint32_t voff, uint32_t soff, bf16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ void buf_store(rsrc_t r, uint32_t voff, uint32_t soff, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)voff, (int)soff, 0);
}

// Buffer over tokens [tok, tok + n) of a [tokens, width] tensor of T.
template <typename T>
__device__ __forceinline__ rsrc_t rows_rsrc(const void* base, size_t tok, int n, int width) {
  return make_rsrc(reinterpret_cast<const T*>(base) + tok * (size_t)width,
                   (uint32_t)n * (uint32_t)width * (uint32_t)sizeof(T));
}

// Per-lane state of the staging loads of one block: the lane's 16-byte piece
// of B_t and of C_t, and up to KW routing words of idx and of gate.  The lane
// offsets are fixed for the whole walk.
template <typename TIn, int KW>
struct Stager {
  static constexpr int kPieces = kTB * kN * (int)sizeof(TIn) / 16;  // per vector per block
  uint32_t piece_off;
  uint32_t word_off[KW];
  v4u pb, pc;
  int32_t wi[KW], wg[KW];

  __device__ __forceinline__ void init(int lane) {
    piece_off = (uint32_t)(lane % kPieces) * 16u;
#pragma unroll
    for (int i = 0; i < KW; ++i) word_off[i] = (uint32_t)(lane + 64 * i) * 4u;
  }

  // Loads of tokens [tok, tok + kTB) (global token index); `valid` is how
  // many of them exist in the tensors (later ones read as 0).
  template <typename P>
  __device__ __forceinline__ void issue(const P& p, size_t tok, int valid, int k) {
    const rsrc_t rb = rows_rsrc<TIn>(p.Bm, tok, valid, kN);
    const rsrc_t rc = rows_rsrc<TIn>(p.Cm, tok, valid, kN);
    pb = __builtin_amdgcn_raw_buffer_load_b128(rb, (int)piece_off, 0, 0);
    pc = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)piece_off, 0, 0);
    const rsrc_t ri = rows_rsrc<int32_t>(p.idx, tok, valid, k);
    const rsrc_t rg = rows_rsrc<int32_t>(p.gate, tok, valid, k);
#pragma unroll
    for (int i = 0; i < KW; ++i) {
      wi[i] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(ri, (int)word_off[i], 0, 0);
      wg[i] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rg, (int)word_off[i], 0, 0);
    }
  }

  // Convert and write to ring slot `slot`; n = tokens of the block that are
  // used (their gates are checked for the contraction condition, g >= 0).
  // The expert ids are clamped to [0, E) and written times e_scale; with
  // ring.uo set, also times u_scale there (callers that address per-expert
  // LDS rows store byte offsets instead of ids).
  __device__ __forceinline__ void commit(const Ring& ring, int slot, int n, int k, int E,
                                         int lane, int& gate_bad, int e_scale = 1,
                                         int u_scale = 0) const {
    if (lane < kPieces) {
      constexpr int kVals = 16 / (int)sizeof(TIn);  // values per piece
      const int tok = lane * kVals / kN, col = lane * kVals % kN;
      float* dst = ring.bc + (slot * kTB + tok) * 32 + col;
      if (sizeof(TIn) == 2) {
        const uint32_t b4[4] = {pb.x, pb.y, pb.z, pb.w}, c4[4] = {pc.x, pc.y, pc.z, pc.w};
        float4* db = reinterpret_cast<float4*>(dst);
        float4* dc = reinterpret_cast<float4*>(dst + kN);
        db[0] = make_float4(__uint_as_float(b4[0] << 16), __uint_as_float(b4[0] & 0xffff0000u),
                            __uint_as_float(b4[1] << 16), __uint_as_float(b4[1] & 0xffff0000u));
        db[1] = make_float4(__uint_as_float(b4[2] << 16), __uint_as_float(b4[2] & 0xffff0000u),
                            __uint_as_float(b4[3] << 16), __uint_as_float(b4[3] & 0xffff0000u));
        dc[0] = make_float4(__uint_as_float(c4[0] << 16), __uint_as_float(c4[0] & 0xffff0000u),
                            __uint_as_float(c4[1] << 16), __uint_as_float(c4[1] & 0xffff0000u));
        dc[1] = make_float4(__uint_as_float(c4[2] << 16), __uint_as_float(c4[2] & 0xffff0000u),
                            __uint_as_float(c4[3] << 16), __uint_as_float(c4[3] & 0xffff0000u));
      } else {
        *reinterpret_cast<float4*>(dst) = make_float4(
            __uint_as_float(pb.x), __uint_as_float(pb.y), __uint_as_float(pb.z), __uint_as_float(pb.w));
        *reinterpret_cast<float4*>(dst + kN) = make_float4(
            __uint_as_float(pc.x), __uint_as_float(pc.y), __uint_as_float(pc.z), __uint_as_float(pc.w));
      }
    }
    const int nw = kTB * k;
#pragma unroll
    for (int i = 0; i < KW; ++i) {
      const int w = lane + 64 * i;
      if (w < nw) {
        int e = wi[i];
        e = e < 0 ? 0 : (e >= E ? E - 1 : e);
        ring.e[slot * nw + w] = e * e_scale;
        if (ring.uo != nullptr) ring.uo[slot * nw + w] = e * u_scale;
        const float gv = __int_as_float(wg[i]);
        if (w / k < n) gate_bad |= !(gv >= 0.f);
        ring.g[slot * nw + w] = gv;
      }
    }
  }
};

}  // namespace stage
}  // namespace swimba
