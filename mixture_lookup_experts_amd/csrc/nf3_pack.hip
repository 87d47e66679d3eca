// NF3 encoder: blocks of 64 consecutive elements of a table row, fp16
// absmax scale, 3-bit codes by threshold count, LSB-first bit stream.
// (MoLE article, results section: the lookup table keeps the model's
// quality when compressed to 3 bits, e.g. NF3.)
//
// Eight lanes own one 64-element block (8 elements = 16 bytes of bf16
// each), so a wavefront encodes 8 consecutive blocks from 1 KB of
// contiguous input with coalesced 16-byte loads.  Each lane forms the 24
// code bits of its 8 elements; lanes 0..5 of the group then assemble the
// block's six output dwords from two neighbours' bits with lane shuffles.
#include "mole_device.hpp"
#include "mole_kernels.hpp"

namespace mole {

// Thresholds: kNf3MidBits (mole_tables.hpp).

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* x);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* x) {
  Elem<uint16_t>::unpack(ldg16(p), x);
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* x) {
  Elem<float>::unpack(ldg16(p), x);
  Elem<float>::unpack(ldg16(p + 4), x + 4);
}

constexpr int kUnroll = 4;  // groups of 8 blocks per wave trip

template <typename T>
__global__ __launch_bounds__(256) void pack_nf3_kernel(const T* __restrict__ lut,
                                                       uint8_t* __restrict__ codes,
                                                       uint16_t* __restrict__ scales,
                                                       int64_t nblocks) {
  const int lane = threadIdx.x & 63;
  const int sub = lane & 7;
  float mid[7];
#pragma unroll
  for (int j = 0; j < 7; ++j) mid[j] = __uint_as_float(kNf3MidBits[j]);

  // Each wave takes kUnroll groups of 8 consecutive blocks per trip and
  // issues all their loads before encoding any: one memory round trip
  // per trip instead of per group.
  const int64_t waves_total = (int64_t)gridDim.x * (blockDim.x / 64);
  const int64_t wave_id = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  for (int64_t base = wave_id * 8 * kUnroll; base < nblocks; base += waves_total * 8 * kUnroll) {
    // Loads are unconditional, from the block index clamped into range (a
    // group past the end re-reads the last block and stores nothing): a
    // load under a branch would make the compiler wait for it there.
    float xs[kUnroll][8];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t bu = base + u * 8 + (lane >> 3);  // this group's block
      const int64_t b = bu < nblocks ? bu : nblocks - 1;
      load8<T>(lut + b * 64 + sub * 8, xs[u]);  // rows are contiguous: block b starts at 64 b
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t bu = base + u * 8 + (lane >> 3);
      const bool valid = bu < nblocks;
      const int64_t b = valid ? bu : nblocks - 1;
      const float* x = xs[u];
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(x[i]));
      a = fmaxf(a, __shfl_xor(a, 1, 64));
      a = fmaxf(a, __shfl_xor(a, 2, 64));
      a = fmaxf(a, __shfl_xor(a, 4, 64));
      a = fminf(a, 65504.f);
      const _Float16 s16 = (_Float16)a;  // v_cvt_f16_f32: round to nearest even
      const float sc = (float)s16;
      float thr[7];
#pragma unroll
      for (int j = 0; j < 7; ++j) thr[j] = __fmul_rn(mid[j], sc);
      uint32_t bits = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // The code is the number of thresholds below x; the thresholds are
        // non-decreasing (ascending midpoints times one non-negative scale,
        // each product rounded), so a branch-free binary search -- 3
        // compares and 4 selects -- counts the same as 7 compares (a NaN x
        // fails every compare either way).
        const float v = x[i];
        const bool b2 = v > thr[3];
        const bool b1 = v > (b2 ? thr[5] : thr[1]);
        const bool b0 = v > (b2 ? (b1 ? thr[6] : thr[4]) : (b1 ? thr[2] : thr[0]));
        uint32_t c = (b2 ? 4u : 0u) | (b1 ? 2u : 0u) | (b0 ? 1u : 0u);
        if (sc == 0.f) c = 3u;
        bits |= c << (3 * i);
      }
      // Output dword k of the block = stream bits [32k, 32k+32), taken from
      // the 24-bit pieces of lanes j0 = 32k/24 and j0+1.
      const int k = sub < 6 ? sub : 5;
      const int j0 = (32 * k) / 24, off = 32 * k - 24 * j0;
      const int gbase = lane & ~7;
      const uint32_t a0 = (uint32_t)__shfl((int)bits, gbase + j0, 64);
      const uint32_t a1 = (uint32_t)__shfl((int)bits, gbase + j0 + 1, 64);
      const uint32_t dw = (a0 >> off) | (a1 << (24 - off));
      if (valid && sub < 6)
        *reinterpret_cast<uint32_t*>(codes + b * 24 + 4 * sub) = dw;  // 24 code bytes per block
      if (valid && sub == 0) scales[b] = __builtin_bit_cast(uint16_t, s16);
    }
  }
}

hipError_t launch_pack_nf3(const void* lut, uint8_t* codes, uint16_t* scales, int64_t rows,
                           int64_t D, int dtype, hipStream_t s) {
  const int64_t nblocks = rows * (D / 64);
  if (nblocks == 0) return hipSuccess;
  const int64_t need = (nblocks + 32 * kUnroll - 1) / (32 * kUnroll);  // 32*kUnroll blocks per workgroup trip
  const unsigned grid = (unsigned)(need < 8192 ? need : 8192);
  if (dtype == kF32)
    hipLaunchKernelGGL((pack_nf3_kernel<float>), dim3(grid), dim3(256), 0, s, (const float*)lut,
                       codes, scales, nblocks);
  else
    hipLaunchKernelGGL((pack_nf3_kernel<uint16_t>), dim3(grid), dim3(256), 0, s,
                       (const uint16_t*)lut, codes, scales, nblocks);
  return hipGetLastError();
}

}  // namespace mole
