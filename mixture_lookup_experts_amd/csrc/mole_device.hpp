// Device-side helpers shared by the libmole kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mole_tables.hpp"

namespace mole {

constexpr int kWave = 64;  // CDNA wavefront width

// ---- bf16 <-> fp32 -----------------------------------------------------------
// bf16 is the upper half of an fp32 bit pattern.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// ---- element access for the two storage types ---------------------------------
// A "chunk" is 16 bytes of a row: 8 bf16 or 4 fp32 values.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kVec = 4;
  __device__ __forceinline__ static float load1(const float* p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static void unpack(const uint4& q, float* out) {
    out[0] = __uint_as_float(q.x); out[1] = __uint_as_float(q.y);
    out[2] = __uint_as_float(q.z); out[3] = __uint_as_float(q.w);
  }
};
template <> struct Elem<uint16_t> {  // bf16 bit patterns
  static constexpr int kVec = 8;
  __device__ __forceinline__ static float load1(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  __device__ __forceinline__ static void unpack(const uint4& q, float* out) {
    out[0] = bf16_lo(q.x); out[1] = bf16_hi(q.x); out[2] = bf16_lo(q.y); out[3] = bf16_hi(q.y);
    out[4] = bf16_lo(q.z); out[5] = bf16_hi(q.z); out[6] = bf16_lo(q.w); out[7] = bf16_hi(q.w);
  }
};

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Raw buffer resources: a buffer offset at or past a resource's byte count
// reads 0 and drops stores, so kOob (past every record) masks a load or a
// store without a branch.
constexpr uint32_t kOob = 0x80000000u;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

// 16-byte streaming store (non-temporal: the output is not re-read here).
typedef float f32x4_vec_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void stg16_nt(float* p, float a, float b, float c, float d) {
  const f32x4_vec_t v = {a, b, c, d};
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4_vec_t*>(p));
}

// GELU for the bf16 path: u * Phi(u), with Phi from the odd polynomial of
// mole_tables.hpp (kPhiPolyCoef, Horner in fp32, u clamped to the fitted
// interval, the result clamped to [0, 1]).  It costs ~14 full-rate VALU slots and no transcendental,
// which matters because a GEMM epilogue runs it once per hidden unit and row.
__device__ __forceinline__ float phi_poly(float u) {
  const float s = __builtin_amdgcn_fmed3f(u, -kPhiPolyRange, kPhiPolyRange) * (1.0f / kPhiPolyRange);
  const float s2 = s * s;
  float p = kPhiPolyCoef[kPhiPolyTerms - 1];
#pragma unroll
  for (int k = kPhiPolyTerms - 2; k >= 0; --k) p = fmaf(p, s2, kPhiPolyCoef[k]);
  return __builtin_amdgcn_fmed3f(fmaf(s, p, 0.5f), 0.0f, 1.0f);
}

// d GELU / du = Phi(u) + u phi(u), phi(u) = exp(-u^2/2) / sqrt(2 pi).
__device__ __forceinline__ float gelu_grad_poly(float u) {
  return fmaf(u * 0.3989422804014327f, __expf(-0.5f * u * u), phi_poly(u));
}

__device__ __forceinline__ float gelu_poly(float u) { return u * phi_poly(u); }

// ---- cross-lane reductions ----------------------------------------------------
// Reduce-scatter of NP per-lane partial sums over the W lanes (W a power of
// two, W <= 64) of a lane group: at the step with xor-mask m the lane keeps
// one half of its vector (the upper half when bit m of its lane id is set)
// and adds the partner's copy of that half.  After min(log2 NP, log2 W)
// steps each lane holds CNT = NP / min(NP, W) sums, for experts
// offset(lane) + i, i < CNT; the remaining masks (if W > NP) finish the sum.
template <int NP, int W, int M = 1, int CNT = NP>
struct ReduceScatter {
  __device__ __forceinline__ static void run(float* v, int lane) {
    if constexpr (M < W) {
      if constexpr (CNT > 1) {
        constexpr int H = CNT / 2;
        const bool hi = (lane & M) != 0;
#pragma unroll
        for (int i = 0; i < H; ++i) {
          const float keep = hi ? v[i + H] : v[i];
          const float send = hi ? v[i] : v[i + H];
          v[i] = keep + __shfl_xor(send, M, kWave);
        }
        ReduceScatter<NP, W, M * 2, H>::run(v, lane);
      } else {
        v[0] += __shfl_xor(v[0], M, kWave);
        ReduceScatter<NP, W, M * 2, 1>::run(v, lane);
      }
    }
  }
  // Number of values left per lane and the expert index of value 0.
  static constexpr int kLeft = NP / (NP < W ? NP : W);
  __device__ __forceinline__ static int offset(int lane) {
    int off = 0;
#pragma unroll
    for (int b = 0, span = NP / 2; span >= kLeft && (1 << b) < W && span > 0; ++b, span /= 2)
      if (lane & (1 << b)) off += span;
    return off;
  }
};

}  // namespace mole
