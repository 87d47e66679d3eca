// Internal launcher declarations of libmole (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mole {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;

// combine_dense.hip, combine_nf3.hip
hipError_t launch_lookup_combine(const int64_t* ids, const void* h, const void* w_r, const void* lut,
                                 float* y, int64_t T, int64_t D, int64_t N, int dtype, bool vector_ok,
                                 hipStream_t s);
hipError_t launch_lookup_combine_nf3(const int64_t* ids, const void* h, const void* w_r,
                                     const uint8_t* codes, const uint16_t* scales, float* y,
                                     int64_t T, int64_t D, int64_t N, int dtype_h, hipStream_t s);
void nf3_levels_host(float* out);

// nf3_pack.hip
hipError_t launch_pack_nf3(const void* lut, uint8_t* codes, uint16_t* scales, int64_t rows,
                           int64_t D, int dtype, hipStream_t s);

// build_lut.hip
constexpr int kBuildTileM = 256;  // vocabulary rows per GEMM tile
size_t build_lut_min_workspace(int64_t D, int64_t F, int64_t N);
size_t build_lut_rec_workspace(int64_t V, int64_t D, int64_t F, int64_t N);
hipError_t launch_build_lut_bf16(const uint16_t* emb, const uint16_t* w_up, const uint16_t* w_down,
                                 uint16_t* lut, int64_t V, int64_t D, int64_t F, int64_t N,
                                 void* ws, size_t ws_bytes, hipStream_t s);
hipError_t launch_build_lut_f32(const float* emb, const float* w_up, const float* w_down, float* lut,
                                int64_t V, int64_t D, int64_t F, int64_t N, hipStream_t s);
constexpr int64_t kBuildF32MaxLds = 16384;  // D + F floats staged in LDS by the fp32 build

}  // namespace mole
