// Training mode of the routed experts (MoLE article, training section:
// every routed expert reads the token's shallow embedding, all experts are
// active with dense softmax gates, the router reads the contextual hidden
// state; inference section: the lookup table is this forward pass evaluated
// on every vocabulary row -- here it is evaluated on the batch's rows only).
//
// Forward, for the U distinct ids of a batch (uniq) and the token -> row map
// (remap):
//   X = Emb[uniq]                                    (gather)
//   G = GELU(X . W_up^T), O[:, e, :] = G_e . W_down[e]^T   (the build's two GEMMs)
//   y = sum_e softmax(W_r h)[e] O[remap, e, :]       (the lookup-combine)
// X, G and O stay in the caller's forward workspace for the backward pass.
//
// Backward for an upstream gradient dy [T][D] (fp32):
//   per token:   g = softmax(W_r h), dg_e = dy . O[remap, e], dz = g (dg - g.dg),
//                d_h = sum_e dz_e W_r[e]                     (gate_backward_kernel)
//   router:      d_W_r = dz^T . h                            (two reduction passes)
//   per row u:   dO[u][e] = sum_{t : remap t = u} g_te dy_t  (tokens grouped by row)
//   experts:     dU_e = (dO_e . W_down[e]) * GELU'(X . W_up^T)   (one GEMM epilogue)
//                d_W_down[e] = dO_e^T . G_e,  d_W_up[e] = dU_e^T . X,
//                d_X = dU . W_up  (= the gradient of the rows Emb[uniq])
// The five products run on the 256x256 MFMA GEMM (C = A . B^T with both
// operands K-contiguous, fp32 output); products whose contraction runs over
// rows (U) or over the weights' output dimension take LDS-tiled transposed
// copies of their operands.  dO, dU and the recomputed pre-activations are
// rounded to bf16 for the matrix cores; all sums are fp32.  The per-row
// gradient sums walk a host-built list of each row's tokens, so no atomics
// and the result does not depend on scheduling.
#include <algorithm>

#include "mole_device.hpp"
#include "mole_kernels.hpp"

namespace mole {

namespace {

constexpr int kTile = 64;      // transpose tile edge
constexpr int kWrChunk = 16;   // tokens per partial sum of the router-weight gradient

inline size_t round256(size_t x) { return (x + 255u) & ~(size_t)255u; }

// X[u][:] = emb[uniq[u]][:]
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t* __restrict__ emb,
                                                          const int64_t* __restrict__ uniq,
                                                          uint16_t* __restrict__ X, int D) {
  const int64_t u = blockIdx.x;
  const uint16_t* src = emb + uniq[u] * D;
  uint16_t* dst = X + u * D;
  for (int c = threadIdx.x; c < D / 8; c += 256)
    reinterpret_cast<uint4*>(dst)[c] = reinterpret_cast<const uint4*>(src)[c];
}

// out[b][c][r] = in[b][r][c] for r < R (zero for R <= r < Rpad), c < C; bf16.
// Needs C, Rpad, ld_in, ld_out, bs_in, bs_out multiples of 8 (16-byte rows of
// 8 elements both ways).  A 64 x 64 tile goes through LDS: 16-byte loads
// along c, 16-byte stores along r, each assembled from 8 LDS reads.
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ in, int64_t ld_in,
                                                        int64_t bs_in, uint16_t* __restrict__ out, int64_t ld_out,
                                                        int64_t bs_out, int R, int C, int Rpad) {
  __shared__ uint16_t tile[kTile][kTile + 8];  // row pitch 144 bytes
  const int r0 = blockIdx.x * kTile, c0 = blockIdx.y * kTile;
  const int64_t b = blockIdx.z;
  const uint16_t* src = in + b * bs_in;
  uint16_t* dst = out + b * bs_out;
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int q = tid + 256 * k;            // 512 16-byte pieces: row q / 8, column group q % 8
    const int i = q >> 3, cg = (q & 7) * 8;
    const int r = r0 + i, c = c0 + cg;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r < R && c < C) v = *reinterpret_cast<const uint4*>(src + (int64_t)r * ld_in + c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      tile[i][cg + 2 * j] = (uint16_t)(w[j] & 0xFFFFu);
      tile[i][cg + 2 * j + 1] = (uint16_t)(w[j] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int q = tid + 256 * k;            // output row c0 + q / 8, rows r0 + (q % 8) * 8 .. + 7
    const int i = q >> 3, rg = (q & 7) * 8;
    const int c = c0 + i, r = r0 + rg;
    if (c < C && r < Rpad) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = (uint32_t)tile[rg + 2 * j][i] | ((uint32_t)tile[rg + 2 * j + 1][i] << 16);
      *reinterpret_cast<uint4*>(dst + (int64_t)c * ld_out + r) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// Per token t (one workgroup): router logits and dg_e = dy_t . O[remap_t][e]
// as block sums, softmax and dz in LDS, then d_h[t] = sum_e dz_e W_r[e].
template <int NP>
__global__ __launch_bounds__(256) void gate_backward_kernel(const uint16_t* __restrict__ h,
                                                            const uint16_t* __restrict__ w_r,
                                                            const uint16_t* __restrict__ O,
                                                            const int64_t* __restrict__ remap,
                                                            const float* __restrict__ dy, float* __restrict__ g_out,
                                                            float* __restrict__ dz_out, float* __restrict__ d_h, int D,
                                                            int N) {
  __shared__ float red[4][2 * NP];
  __shared__ float dzs[NP];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint16_t* orow = O + remap[t] * (int64_t)N * D;
  float z[NP], dg[NP];
#pragma unroll
  for (int e = 0; e < NP; ++e) z[e] = dg[e] = 0.f;
  for (int d = tid; d < D; d += 256) {
    const float hv = bf16_to_f32(h[t * D + d]);
    const float yv = dy[t * D + d];
#pragma unroll
    for (int e = 0; e < NP; ++e) {
      if (e < N) {
        z[e] = fmaf(hv, bf16_to_f32(w_r[(int64_t)e * D + d]), z[e]);
        dg[e] = fmaf(yv, bf16_to_f32(orow[(int64_t)e * D + d]), dg[e]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < NP; ++e) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      z[e] += __shfl_xor(z[e], m, 64);
      dg[e] += __shfl_xor(dg[e], m, 64);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int e = 0; e < NP; ++e) {
      red[wave][e] = z[e];
      red[wave][NP + e] = dg[e];
    }
  }
  __syncthreads();
  if (tid == 0) {
    // (loops over the compile-time bound NP keep the arrays in registers)
    float zz[NP], gg[NP], dd[NP];
    float zmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < NP; ++e) {
      zz[e] = red[0][e] + red[1][e] + red[2][e] + red[3][e];
      dd[e] = red[0][NP + e] + red[1][NP + e] + red[2][NP + e] + red[3][NP + e];
      if (e < N) zmax = fmaxf(zmax, zz[e]);
    }
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < NP; ++e) {
      gg[e] = e < N ? expf(zz[e] - zmax) : 0.f;
      sum += gg[e];
    }
    float gdg = 0.f;
#pragma unroll
    for (int e = 0; e < NP; ++e) {
      gg[e] /= sum;
      gdg = fmaf(gg[e], dd[e], gdg);
    }
#pragma unroll
    for (int e = 0; e < NP; ++e) {
      if (e < N) {
        const float dzv = gg[e] * (dd[e] - gdg);
        g_out[t * N + e] = gg[e];
        dz_out[t * N + e] = dzv;
        dzs[e] = dzv;
      }
    }
  }
  __syncthreads();
  for (int d = tid; d < D; d += 256) {
    float acc = 0.f;
    for (int e = 0; e < N; ++e) acc = fmaf(dzs[e], bf16_to_f32(w_r[(int64_t)e * D + d]), acc);
    d_h[t * D + d] = acc;
  }
}

// Partial router-weight gradient over one chunk of tokens:
// P[chunk][e][d] = sum_{t in chunk} dz[t][e] h[t][d].
template <int NP>
__global__ __launch_bounds__(256) void wr_partial_kernel(const float* __restrict__ dz, const uint16_t* __restrict__ h,
                                                         float* __restrict__ P, int64_t T, int D, int N) {
  const int d = blockIdx.x * 256 + threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.y * kWrChunk;
  if (d >= D) return;
  float acc[NP];
#pragma unroll
  for (int e = 0; e < NP; ++e) acc[e] = 0.f;
  const int64_t t1 = T - t0 < kWrChunk ? T : t0 + kWrChunk;
  for (int64_t t = t0; t < t1; ++t) {
    const float hv = bf16_to_f32(h[t * D + d]);
#pragma unroll
    for (int e = 0; e < NP; ++e)
      if (e < N) acc[e] = fmaf(dz[t * N + e], hv, acc[e]);
  }
  float* out = P + (int64_t)blockIdx.y * N * D;
#pragma unroll
  for (int e = 0; e < NP; ++e)
    if (e < N) out[(int64_t)e * D + d] = acc[e];
}

// dO[u][e][d] = bf16( sum over the tokens t of row u of g[t][e] * dy[t][d] ).
// A workgroup owns 64 columns of one row; its four waves take every fourth
// token of the row (Zipf batches give a few rows hundreds of tokens) and
// meet in LDS.
template <int NP>
__global__ __launch_bounds__(256) void row_grad_kernel(const float* __restrict__ g, const float* __restrict__ dy,
                                                       const int64_t* __restrict__ row_ptr,
                                                       const int64_t* __restrict__ tok, uint16_t* __restrict__ dO,
                                                       int D, int N) {
  __shared__ float part[3][NP][64];
  const int64_t u = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int d = blockIdx.y * 64 + lane;
  const bool ok = d < D;
  float acc[NP];
#pragma unroll
  for (int e = 0; e < NP; ++e) acc[e] = 0.f;
  // Four tokens per wave and trip, their loads issued together (a hot row's
  // walk is a chain of dependent loads otherwise).
  const int64_t k0 = row_ptr[u], k1 = row_ptr[u + 1];
  for (int64_t k = k0 + wave; k < k1; k += 16) {
    int64_t t4[4];
    float y4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t kq = k + 4 * q;
      t4[q] = tok[kq < k1 ? kq : k1 - 1];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) y4[q] = (ok && k + 4 * q < k1) ? dy[t4[q] * D + d] : 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < NP; ++e)
        if (e < N) acc[e] = fmaf(g[t4[q] * N + e], y4[q], acc[e]);
  }
  if (wave > 0) {
#pragma unroll
    for (int e = 0; e < NP; ++e) part[wave - 1][e][lane] = acc[e];
  }
  __syncthreads();
  if (wave == 0 && ok) {
    uint16_t* out = dO + u * (int64_t)N * D + d;
#pragma unroll
    for (int e = 0; e < NP; ++e)
      if (e < N) out[(int64_t)e * D] = (uint16_t)f32_to_bf16_rne(acc[e] + part[0][e][lane] + part[1][e][lane] +
                                                                 part[2][e][lane]);
  }
}

// out[i] = sum_s P[s][i].
__global__ __launch_bounds__(256) void sum_partials_kernel(const float* __restrict__ P, int S, int64_t count,
                                                           float* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256) {
    float a[4] = {0.f, 0.f, 0.f, 0.f};  // four independent chains of loads
    int sp = 0;
    for (; sp + 4 <= S; sp += 4)
#pragma unroll
      for (int q = 0; q < 4; ++q) a[q] += P[(int64_t)(sp + q) * count + i];
    for (; sp < S; ++sp) a[0] += P[(int64_t)sp * count + i];
    out[i] = (a[0] + a[1]) + (a[2] + a[3]);
  }
}

unsigned grid_for(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(b, 8192));
}

hipError_t transpose(const uint16_t* in, int64_t ld_in, int64_t bs_in, uint16_t* out, int64_t ld_out, int64_t bs_out,
                     int64_t R, int64_t C, int64_t Rpad, int64_t batch, hipStream_t s) {
  const dim3 grid((unsigned)((Rpad + kTile - 1) / kTile), (unsigned)((C + kTile - 1) / kTile), (unsigned)batch);
  hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, s, in, ld_in, bs_in, out, ld_out, bs_out, (int)R, (int)C,
                     (int)Rpad);
  return hipGetLastError();
}

int next_pow2_int(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// The three per-expert-accumulator kernels, instantiated for the expert
// counts padded to a power of two (N <= 64).
#define MOLE_NP_SWITCH(KERNEL, GRID, STREAM, ...)                                                     \
  switch (NP) {                                                                                     \
    case 1: hipLaunchKernelGGL(KERNEL<1>, GRID, dim3(256), 0, STREAM, __VA_ARGS__); break;          \
    case 2: hipLaunchKernelGGL(KERNEL<2>, GRID, dim3(256), 0, STREAM, __VA_ARGS__); break;          \
    case 4: hipLaunchKernelGGL(KERNEL<4>, GRID, dim3(256), 0, STREAM, __VA_ARGS__); break;          \
    case 8: hipLaunchKernelGGL(KERNEL<8>, GRID, dim3(256), 0, STREAM, __VA_ARGS__); break;          \
    case 16: hipLaunchKernelGGL(KERNEL<16>, GRID, dim3(256), 0, STREAM, __VA_ARGS__); break;        \
    case 32: hipLaunchKernelGGL(KERNEL<32>, GRID, dim3(256), 0, STREAM, __VA_ARGS__); break;        \
    default: hipLaunchKernelGGL(KERNEL<64>, GRID, dim3(256), 0, STREAM, __VA_ARGS__); break;        \
  }

}  // namespace

TrainPlan train_plan(int64_t T, int64_t U, int64_t D, int64_t F, int64_t N) {
  TrainPlan p{};
  const int64_t NF = N * F;
  p.up = std::max<int64_t>(8, (U + 7) / 8 * 8);
  // K splits of d_X = dU . W_up (K = N*F): enough 256x256 tiles to fill the
  // chip, each split a multiple of 8 of K.
  const int64_t tiles = ((U + 255) / 256) * ((D + 255) / 256);
  p.dx_splits = 1;
  while (p.dx_splits < 16 && tiles * p.dx_splits < 256 && NF % (16 * p.dx_splits) == 0) p.dx_splits *= 2;
  p.wr_chunks = (int)((T + kWrChunk - 1) / kWrChunk);
  size_t o = 0;
  p.x_off = o; o += round256((size_t)U * D * 2);
  p.g_off = o; o += round256((size_t)U * NF * 2);
  p.o_off = o; o += round256((size_t)U * N * D * 2);
  p.fwd_total = o;
  o = 0;
  p.gate_off = o; o += round256((size_t)T * N * 4);
  p.dz_off = o; o += round256((size_t)T * N * 4);
  p.do_off = o; o += round256((size_t)U * N * D * 2);
  p.dot_off = o; o += round256((size_t)N * D * p.up * 2);
  p.u_off = o; o += round256((size_t)U * NF * 2);
  p.du_off = o; o += round256((size_t)U * NF * 2);
  p.dut_off = o; o += round256((size_t)NF * p.up * 2);
  p.gt_off = o; o += round256((size_t)NF * p.up * 2);
  p.xt_off = o; o += round256((size_t)D * p.up * 2);
  p.wdt_off = o; o += round256((size_t)NF * D * 2);
  p.wut_off = o; o += round256((size_t)D * NF * 2);
  p.pdx_off = o; o += round256((size_t)p.dx_splits * U * D * 4);
  p.pwr_off = o; o += round256((size_t)p.wr_chunks * N * D * 4);
  p.bwd_total = o;
  return p;
}

hipError_t launch_train_forward(const int64_t* uniq, const int64_t* remap, const uint16_t* emb, const uint16_t* w_up,
                                const uint16_t* w_down, const uint16_t* h, const uint16_t* w_r, float* y, void* fwd,
                                int64_t T, int64_t U, int64_t D, int64_t F, int64_t N, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const TrainPlan p = train_plan(T, U, D, F, N);
  char* base = static_cast<char*>(fwd);
  uint16_t* X = reinterpret_cast<uint16_t*>(base + p.x_off);
  uint16_t* G = reinterpret_cast<uint16_t*>(base + p.g_off);
  uint16_t* O = reinterpret_cast<uint16_t*>(base + p.o_off);
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)U), dim3(256), 0, s, emb, uniq, X, (int)D);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // The build restricted to the batch's rows: G for all U rows in one block.
  err = launch_build_lut_bf16(X, w_up, w_down, O, U, D, F, N, G, (size_t)U * N * F * 2, s);
  if (err != hipSuccess) return err;
  return launch_lookup_combine(remap, h, w_r, O, y, T, D, N, kBF16, true, s);
}

hipError_t launch_train_backward(const int64_t* uniq, const int64_t* remap, const int64_t* row_ptr, const int64_t* tok,
                                 const uint16_t* emb, const uint16_t* w_up, const uint16_t* w_down, const uint16_t* h,
                                 const uint16_t* w_r, const float* dy, const void* fwd, void* bwd, float* d_w_up,
                                 float* d_w_down, float* d_w_r, float* d_h, float* d_x, int64_t T, int64_t U,
                                 int64_t D, int64_t F, int64_t N, hipStream_t s) {
  (void)uniq;
  (void)emb;
  if (T == 0) return hipSuccess;
  const TrainPlan p = train_plan(T, U, D, F, N);
  const int64_t NF = N * F, Up = p.up;
  const char* fb = static_cast<const char*>(fwd);
  const uint16_t* X = reinterpret_cast<const uint16_t*>(fb + p.x_off);
  const uint16_t* G = reinterpret_cast<const uint16_t*>(fb + p.g_off);
  const uint16_t* O = reinterpret_cast<const uint16_t*>(fb + p.o_off);
  char* bb = static_cast<char*>(bwd);
  float* gate = reinterpret_cast<float*>(bb + p.gate_off);
  float* dz = reinterpret_cast<float*>(bb + p.dz_off);
  uint16_t* dO = reinterpret_cast<uint16_t*>(bb + p.do_off);
  uint16_t* dOT = reinterpret_cast<uint16_t*>(bb + p.dot_off);
  uint16_t* Upre = reinterpret_cast<uint16_t*>(bb + p.u_off);
  uint16_t* dU = reinterpret_cast<uint16_t*>(bb + p.du_off);
  uint16_t* dUT = reinterpret_cast<uint16_t*>(bb + p.dut_off);
  uint16_t* GT = reinterpret_cast<uint16_t*>(bb + p.gt_off);
  uint16_t* XT = reinterpret_cast<uint16_t*>(bb + p.xt_off);
  uint16_t* WdT = reinterpret_cast<uint16_t*>(bb + p.wdt_off);
  uint16_t* WuT = reinterpret_cast<uint16_t*>(bb + p.wut_off);
  float* Pdx = reinterpret_cast<float*>(bb + p.pdx_off);
  float* Pwr = reinterpret_cast<float*>(bb + p.pwr_off);
  const int NP = next_pow2_int((int)N);
  hipError_t err;
#define MOLE_TRY(x) do { err = (x); if (err != hipSuccess) return err; } while (0)

  // Gates: g, dz, d_h.
  MOLE_NP_SWITCH(gate_backward_kernel, dim3((unsigned)T), s, h, w_r, O, remap, dy, gate, dz, d_h, (int)D, (int)N);
  MOLE_TRY(hipGetLastError());
  // Router weights: chunked partial sums over tokens, then their sum.
  MOLE_NP_SWITCH(wr_partial_kernel, dim3((unsigned)((D + 255) / 256), (unsigned)p.wr_chunks), s, (const float*)dz,
                 h, Pwr, T, (int)D, (int)N);
  MOLE_TRY(hipGetLastError());
  hipLaunchKernelGGL(sum_partials_kernel, dim3(grid_for(N * D)), dim3(256), 0, s, (const float*)Pwr, p.wr_chunks,
                     N * D, d_w_r);
  MOLE_TRY(hipGetLastError());
  // Gradient of the batch's table rows, dO[u][e] = sum_t g_te dy_t.
  MOLE_NP_SWITCH(row_grad_kernel, dim3((unsigned)U, (unsigned)((D + 63) / 64)), s, (const float*)gate, dy, row_ptr,
                 tok, dO, (int)D, (int)N);
  MOLE_TRY(hipGetLastError());
  // Transposed operands: dO_e^T [D][Up], G_e^T [F][Up], X^T [D][Up],
  // W_down[e]^T [F][D], W_up^T [D][N*F].
  MOLE_TRY(transpose(dO, N * D, D, dOT, Up, D * Up, U, D, Up, N, s));
  MOLE_TRY(transpose(G, NF, F, GT, Up, F * Up, U, F, Up, N, s));
  MOLE_TRY(transpose(X, D, 0, XT, Up, 0, U, D, Up, 1, s));
  MOLE_TRY(transpose(w_down, F, D * F, WdT, D, F * D, D, F, D, N, s));
  MOLE_TRY(transpose(w_up, D, 0, WuT, NF, 0, NF, D, NF, 1, s));
  // Pre-activations again (not kept by the forward pass), then
  // dU = (dO_e . W_down[e]) * GELU'(u) in one GEMM epilogue.
  MOLE_TRY(launch_gemm_store_bf16(X, D, w_up, D, Upre, NF, (int)U, (int)NF, (int)D, s));
  MOLE_TRY(launch_gemm_gelu_grad_bf16(dO, N * D, D, WdT, D, F * D, dU, NF, F, Upre, (int)U, (int)F, (int)D, (int)N,
                                      s));
  MOLE_TRY(transpose(dU, NF, F, dUT, Up, F * Up, U, F, Up, N, s));
  // Weight gradients: d_W_down[e] = dO_e^T . G_e, d_W_up[e] = dU_e^T . X.
  MOLE_TRY(launch_gemm_f32_bf16(dOT, Up, D * Up, GT, Up, F * Up, d_w_down, F, D * F, (int)D, (int)F, (int)Up, (int)N,
                                s));
  MOLE_TRY(launch_gemm_f32_bf16(dUT, Up, F * Up, XT, Up, 0, d_w_up, D, F * D, (int)F, (int)D, (int)Up, (int)N, s));
  // Embedding rows: d_X = dU . W_up over K = N*F, in equal K splits.
  const int64_t ks = NF / p.dx_splits;
  MOLE_TRY(launch_gemm_f32_bf16(dU, NF, ks, WuT, NF, ks, Pdx, D, U * D, (int)U, (int)D, (int)ks, p.dx_splits, s));
  hipLaunchKernelGGL(sum_partials_kernel, dim3(grid_for(U * D)), dim3(256), 0, s, (const float*)Pdx, p.dx_splits,
                     U * D, d_x);
  return hipGetLastError();
#undef MOLE_TRY
}
#undef MOLE_NP_SWITCH

}  // namespace mole
