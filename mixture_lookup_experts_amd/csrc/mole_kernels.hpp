// Internal launcher declarations of libmole (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mole {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;

// combine_dense.hip, combine_nf3.hip
// gates_buf: scratch for the staged router's gates (row stride D; y if null).
// addp != null (bf16 only): y is read and the result added to it together with
// the nadd arrays addp + k * add_stride (the MoLE block's final pass).
hipError_t launch_lookup_combine(const int64_t* ids, const void* h, const void* w_r, const void* lut,
                                 float* y, int64_t T, int64_t D, int64_t N, int dtype, bool vector_ok,
                                 hipStream_t s, float* gates_buf = nullptr, const float* addp = nullptr,
                                 int nadd = 0, int64_t add_stride = 0);
hipError_t launch_lookup_combine_nf3(const int64_t* ids, const void* h, const void* w_r,
                                     const uint8_t* codes, const uint16_t* scales, float* y,
                                     int64_t T, int64_t D, int64_t N, int dtype_h, hipStream_t s);
enum { kFmtNf3 = 3, kFmtNf4 = 4, kFmtI8 = 8 };  // quantised table formats (bits per element)
// codes: NF3 [V][N][3D/8], NF4 [V][N][D/2], int8 [V][N][D]; scales: fp16
// [V][N][D/64] for NF3/NF4, fp32 [V][N] for int8.
hipError_t launch_lookup_combine_q(int fmt, const int64_t* ids, const void* h, const void* w_r,
                                   const uint8_t* codes, const void* scales, float* y, int64_t T, int64_t D,
                                   int64_t N, int dtype_h, hipStream_t s);
// quant_pack.hip
hipError_t launch_pack_nf4(const void* lut, uint8_t* codes, uint16_t* scales, int64_t rows, int64_t D, int dtype,
                           hipStream_t s);
hipError_t launch_pack_int8(const void* lut, int8_t* codes, float* scales, int64_t rows, int64_t D, int dtype,
                            hipStream_t s);

// nf3_pack.hip
hipError_t launch_pack_nf3(const void* lut, uint8_t* codes, uint16_t* scales, int64_t rows,
                           int64_t D, int dtype, hipStream_t s);

// check_ids.hip: *count += number of ids outside [0, V)
hipError_t launch_check_ids(const int64_t* ids, int64_t T, int64_t V, int* count, hipStream_t s);

// combine_grouped.hip: the combine over a batch grouped by id on the device;
// ws holds the grouped positions (grouped_workspace_bytes(T) bytes).
size_t grouped_workspace_bytes(int64_t T);
hipError_t launch_lookup_combine_grouped(const int64_t* ids, const uint16_t* h, const uint16_t* w_r,
                                         const uint16_t* lut, float* y, int64_t T, int D, int N, void* ws,
                                         hipStream_t s);
// The grouping-and-routing launch alone: positions in id order (pos_tok[p]
// = the token at position p, pos_row[p] = its id) and each token's gates
// (gates[t][NP], NP = N rounded up to a power of two, at most 16), all in ws.
hipError_t launch_group_route(const int64_t* ids, const uint16_t* h, const uint16_t* w_r, int64_t T, int D, int N,
                              void* ws, hipStream_t s, const int** pos_tok, const int** pos_row,
                              const float** gates);
// combine_nf3.hip: the NF3 combine over the grouped positions of
// launch_group_route (bf16 h, N <= 16, D % 64 == 0).
hipError_t launch_lookup_combine_nf3_grouped(const int* pos_tok, const int* pos_row, const float* gates,
                                             const uint8_t* codes, const uint16_t* scales, float* y, int64_t T,
                                             int64_t D, int64_t N, hipStream_t s);
// The same with the workspace in the library's static device array (T up to
// kGroupedNoAllocMaxT; no allocation).
constexpr int64_t kGroupedNoAllocMaxT = 65536;
hipError_t launch_lookup_combine_grouped_noalloc(const int64_t* ids, const uint16_t* h, const uint16_t* w_r,
                                                 const uint16_t* lut, float* y, int64_t T, int D, int N,
                                                 hipStream_t s);

// build_lut.hip
constexpr int kBuildTileM = 256;  // vocabulary rows per GEMM tile
size_t build_lut_min_workspace(int64_t D, int64_t F, int64_t N);
size_t build_lut_rec_workspace(int64_t V, int64_t D, int64_t F, int64_t N);
hipError_t launch_build_lut_bf16(const uint16_t* emb, const uint16_t* w_up, const uint16_t* w_down,
                                 uint16_t* lut, int64_t V, int64_t D, int64_t F, int64_t N,
                                 void* ws, size_t ws_bytes, hipStream_t s, uint16_t* pre = nullptr);
hipError_t launch_build_lut_f32(const float* emb, const float* w_up, const float* w_down, float* lut,
                                int64_t V, int64_t D, int64_t F, int64_t N, hipStream_t s);
constexpr int64_t kBuildF32MaxLds = 16384;  // D + F floats staged in LDS by the fp32 build
hipError_t launch_gemm_gelu_bf16(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, uint16_t* C,
                                 int64_t ldc, int M, int N, int K, hipStream_t s);

// GEMM operand storage (bit 0 for A, bit 1 for B): K-contiguous, A[m][k] at
// A[m*lda + k] (the default), or MN-major, A[m][k] at A[k*lda + m] (a
// transposed matrix read in place).
// Bits 2 and 3 select panel-major storage for A and for C: element (m, k)
// at base + (k / 256) * pstride + m * 256 + k % 256, so a 256-column panel
// of a tile's rows is one contiguous run (the build's hidden activations).
enum { kOpsKK = 0, kOpsAmn = 1, kOpsBmn = 2, kOpsMnMn = 3, kOpsApanel = 4, kOpsCpanel = 8 };
hipError_t launch_gemm_gelu_grad_bf16(const uint16_t* A, int64_t lda, int64_t sAz, const uint16_t* B, int64_t ldb,
                                      int64_t sBz, uint16_t* C, int64_t ldc, int64_t sCz, const uint16_t* aux, int M,
                                      int N, int K, int batch, hipStream_t s);
hipError_t launch_gemm_f32_bf16(const uint16_t* A, int64_t lda, int64_t sAz, const uint16_t* B, int64_t ldb,
                                int64_t sBz, float* C, int64_t ldc, int64_t sCz, int M, int N, int K, int batch,
                                hipStream_t s, int ops = kOpsKK);

// train.hip: training-mode forward and backward
struct TrainPlan {
  int dx_splits;         // K splits of the embedding-row gradient product
  // forward state (kept by the caller between the two calls)
  size_t x_off, g_off, u_off, o_off, fwd_total;
  // backward scratch (a second workspace); pwr_off also holds the row
  // gradients' partial sums (used after the router-weight sums are done)
  size_t gate_off, dz_off, do_off, du_off, pdx_off, pwr_off, bwd_total;
  int wr_chunks;         // token chunks of the router-weight gradient
  int seg;               // token-list positions per row-gradient chunk
  int64_t nseg;          // row-gradient chunks, ceil(T / seg)
};
TrainPlan train_plan(int64_t T, int64_t U, int64_t D, int64_t F, int64_t N);
hipError_t launch_train_forward(const int64_t* uniq, const int64_t* remap, const uint16_t* emb, const uint16_t* w_up,
                                const uint16_t* w_down, const uint16_t* h, const uint16_t* w_r, float* y, void* fwd,
                                int64_t T, int64_t U, int64_t D, int64_t F, int64_t N, hipStream_t s);
hipError_t launch_train_backward(const int64_t* uniq, const int64_t* remap, const int64_t* row_ptr, const int64_t* tok,
                                 const uint16_t* emb, const uint16_t* w_up, const uint16_t* w_down, const uint16_t* h,
                                 const uint16_t* w_r, const float* dy, const void* fwd, void* bwd, float* d_w_up,
                                 float* d_w_down, float* d_w_r, float* d_h, float* d_x, int64_t T, int64_t U,
                                 int64_t D, int64_t F, int64_t N, hipStream_t s);

// layer.hip: the MoLE block at inference (shared expert + routed lookup + residual)
struct LayerPlan {
  bool gemv;            // decode batch: both projections as weight-streaming products
  bool big_up;          // up-projection on the 256x256 build GEMM
  bool big_down;        // down-projection on the 256x256 build GEMM (fp32 partials per K split)
  int rm_up, rm_down;   // 32-row MFMA tiles per wave in the mid-size GEMM (tile height 32 * rm)
  int s_up, s_down;     // K splits of the two projections (1 = none)
  int64_t ks_up, ks_down;  // K range per split (multiple of 64)
  size_t yr_off, g_off, p_off, total;  // workspace: router gates fp32 [T][D] | G bf16 [T][F] | partials fp32
};
LayerPlan layer_plan(int64_t T, int64_t D, int64_t F);
hipError_t launch_layer_forward(const int64_t* ids, const uint16_t* h, const uint16_t* w_r, const uint16_t* lut,
                                const uint16_t* w_s_up, const uint16_t* w_s_down, float* x, int64_t T, int64_t D,
                                int64_t N, int64_t F, void* ws, hipStream_t s);

}  // namespace mole
