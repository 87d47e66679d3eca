// Encoders for the other table formats (MoLE article, results section: the
// lookup table keeps the model's quality at 3 bits, so it still carries
// redundancy; these are the 4- and 8-bit points next to NF3).
//
// NF4: the NormalFloat construction at 4 bits, blocks of 64 consecutive
// elements of a row with an fp16 absmax scale, code = number of the 15
// thresholds (fp32 midpoint x fp32 scale, one rounding) strictly below the
// value, the zero level (code 7) for an all-zero block, two codes per byte
// with the even element in the low nibble.  Eight lanes own a block, so a
// lane's 8 codes are exactly one output dword.
//
// int8: one fp32 scale per (v, e) row, s = absmax / 127 (IEEE division),
// code = rint(x / s) (IEEE division, ties to even) clamped to [-127, 127],
// all zero for an all-zero row.  One wavefront per row: an absmax pass and
// a coding pass over 8 elements per lane.
#include "mole_device.hpp"
#include "mole_kernels.hpp"

namespace mole {

// Thresholds: kNf4MidBits (mole_tables.hpp).

namespace {

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

}  // namespace

template <typename T>
__global__ __launch_bounds__(256) void pack_nf4_kernel(const T* __restrict__ lut, uint8_t* __restrict__ codes,
                                                       uint16_t* __restrict__ scales, int64_t nblocks) {
  const int lane = threadIdx.x & 63;
  const int sub = lane & 7;
  float mid[15];
#pragma unroll
  for (int j = 0; j < 15; ++j) mid[j] = __uint_as_float(kNf4MidBits[j]);
  const int64_t waves_total = (int64_t)gridDim.x * (blockDim.x / 64);
  const int64_t wave_id = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  for (int64_t base = wave_id * 8 * kUnroll; base < nblocks; base += waves_total * 8 * kUnroll) {
    // All loads of the trip first, from clamped block indices (a group past
    // the end re-reads the last block and stores nothing).
    float xs[kUnroll][8];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t bu = base + u * 8 + (lane >> 3);
      const int64_t b = bu < nblocks ? bu : nblocks - 1;
      load8<T>(lut + b * 64 + sub * 8, xs[u]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t bu = base + u * 8 + (lane >> 3);
      const bool valid = bu < nblocks;
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
      float thr[15];
#pragma unroll
      for (int j = 0; j < 15; ++j) thr[j] = __fmul_rn(mid[j], sc);
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // The code is the number of thresholds below x.  The thresholds are
        // non-decreasing (ascending midpoints times one non-negative
        // scale, each product rounded), so a branch-free binary search
        // over the 15 of them -- 4 compares and 11 selects -- counts the
        // same as 15 compares (a NaN x fails every compare either way).
        const float v = x[i];
        const bool b3 = v > thr[7];
        const bool b2 = v > (b3 ? thr[11] : thr[3]);
        const bool b1 = v > (b3 ? (b2 ? thr[13] : thr[9]) : (b2 ? thr[5] : thr[1]));
        const bool b0 = v > (b3 ? (b2 ? (b1 ? thr[14] : thr[12]) : (b1 ? thr[10] : thr[8]))
                                : (b2 ? (b1 ? thr[6] : thr[4]) : (b1 ? thr[2] : thr[0])));
        uint32_t c = (b3 ? 8u : 0u) | (b2 ? 4u : 0u) | (b1 ? 2u : 0u) | (b0 ? 1u : 0u);
        if (sc == 0.f) c = 7u;
        word |= c << (4 * i);
      }
      if (valid) {
        *reinterpret_cast<uint32_t*>(codes + bu * 32 + 4 * sub) = word;  // 32 code bytes per block
        if (sub == 0) scales[bu] = __builtin_bit_cast(uint16_t, s16);
      }
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void pack_int8_kernel(const T* __restrict__ lut, int8_t* __restrict__ codes,
                                                        float* __restrict__ scales, int64_t rows, int D) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;  // whole wavefront
  const T* row = lut + r * D;
  float a = 0.f;
  for (int i = lane * 8; i < D; i += 512) {
    float x[8];
    load8<T>(row + i, x);
#pragma unroll
    for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(x[k]));
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) a = fmaxf(a, __shfl_xor(a, m, 64));
  const float s = __fdiv_rn(a, 127.0f);
  for (int i = lane * 8; i < D; i += 512) {
    float x[8];
    load8<T>(row + i, x);
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float q = 0.f;
      if (s != 0.f) q = fminf(fmaxf(__builtin_rintf(__fdiv_rn(x[k], s)), -127.f), 127.f);
      w[k >> 2] |= ((uint32_t)(int)q & 0xFFu) << (8 * (k & 3));
    }
    *reinterpret_cast<uint2*>(codes + r * D + i) = make_uint2(w[0], w[1]);
  }
  if (lane == 0) scales[r] = s;
}

hipError_t launch_pack_nf4(const void* lut, uint8_t* codes, uint16_t* scales, int64_t rows, int64_t D, int dtype,
                           hipStream_t s) {
  const int64_t nblocks = rows * (D / 64);
  if (nblocks == 0) return hipSuccess;
  const int64_t need = (nblocks + 32 * kUnroll - 1) / (32 * kUnroll);
  const unsigned grid = (unsigned)(need < 8192 ? need : 8192);
  if (dtype == kF32)
    hipLaunchKernelGGL((pack_nf4_kernel<float>), dim3(grid), dim3(256), 0, s, (const float*)lut, codes, scales,
                       nblocks);
  else
    hipLaunchKernelGGL((pack_nf4_kernel<uint16_t>), dim3(grid), dim3(256), 0, s, (const uint16_t*)lut, codes,
                       scales, nblocks);
  return hipGetLastError();
}

hipError_t launch_pack_int8(const void* lut, int8_t* codes, float* scales, int64_t rows, int64_t D, int dtype,
                            hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const unsigned grid = (unsigned)((rows + 3) / 4);
  if (dtype == kF32)
    hipLaunchKernelGGL((pack_int8_kernel<float>), dim3(grid), dim3(256), 0, s, (const float*)lut, codes, scales,
                       rows, (int)D);
  else
    hipLaunchKernelGGL((pack_int8_kernel<uint16_t>), dim3(grid), dim3(256), 0, s, (const uint16_t*)lut, codes,
                       scales, rows, (int)D);
  return hipGetLastError();
}

}  // namespace mole
