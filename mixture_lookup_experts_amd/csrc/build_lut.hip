// LUT reparameterisation: LUT[v][e][:] = W_down[e] . GELU(W_up[e] . Emb[v])
// for every vocabulary row v and expert e.  (MoLE article, inference
// section: the embedding weight matrix itself is the batch of expert
// inputs, which yields the complete token-id -> expert-output table.)
//
// bf16 path, per block of vocabulary rows [v0, v0 + Vc):
//   GEMM-1  G[Vc][N*F] = GELU(Emb[v0:] . W_up^T)       (all experts at once:
//           W_up [N][F][D] is one [N*F][D] operand); G rounded to bf16 into
//           the caller's workspace;
//   GEMM-2  LUT[v0:, e, :] = G[:, e*F:(e+1)*F] . W_down[e]^T   for each e
//           (grid z = expert), written with row stride N*D.
// Both are "NT" products C = A . B^T with A and B stored K-contiguous, so
// the MFMA operands come straight from K-contiguous rows.  Kernel: 256x256
// output tile per 256-thread workgroup, 4 waves in a 2x2 arrangement, each
// owning a 128x128 sub-tile of v_mfma_f32_32x32x16_bf16 accumulators; the
// K loop streams 64-wide slices of A and B through a double-buffered LDS
// ring (row = 128 bytes, 16-byte segments XOR-swizzled by row so both the
// staging writes and the fragment reads are bank-conflict free), with the
// next slice's global loads in flight during the current slice's MFMAs.
//
// fp32 path (small tables): one workgroup per (v, e) row: stage Emb[v] in
// LDS, each thread forms hidden units u[f] with fp32 FMAs and exact-form
// GELU (erff), then each thread forms output elements from the staged G.
#include "mole_device.hpp"
#include "mole_kernels.hpp"

namespace mole {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// GELU(u) = u * Phi(u) = u/2 * (1 + erf(u / sqrt 2)).
__device__ __forceinline__ float gelu_erf(float u) { return 0.5f * u * (1.0f + erff(u * 0.70710678118654752f)); }

enum { kEpiStore = 0, kEpiGelu = 1 };

constexpr int kBK = 64;  // K slice per LDS stage (64 bf16 = 128 bytes per row)

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void gemm_nt_bf16_kernel(
    const uint16_t* __restrict__ A, int64_t lda, int64_t sAz,
    const uint16_t* __restrict__ B, int64_t ldb, int64_t sBz,
    uint16_t* __restrict__ C, int64_t ldc, int64_t sCz, int M, int N, int K) {
  constexpr int WM = BM / 2, WN = BN / 2;     // wave sub-tile
  constexpr int TM = WM / 32, TN = WN / 32;   // MFMA tiles per wave
  constexpr int SA = BM * 8 / 256, SB = BN * 8 / 256;  // 16-byte segments per thread
  __shared__ uint4 smem[2][(BM + BN) * 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int z = blockIdx.z;
  A += z * sAz;
  B += z * sBz;
  C += z * sCz;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int seg = tid & 7;  // staging segment (constant per thread)

  uint4 ra[SA], rb[SB];
  auto gload = [&](int k0) {
    const int kk = k0 + seg * 8;
#pragma unroll
    for (int i = 0; i < SA; ++i) {
      const int row = (tid + i * 256) >> 3;
      const int gm = m0 + row;
      ra[i] = (gm < M && kk < K) ? ldg16(A + (int64_t)gm * lda + kk) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const int row = (tid + i * 256) >> 3;
      const int gn = n0 + row;
      rb[i] = (gn < N && kk < K) ? ldg16(B + (int64_t)gn * ldb + kk) : make_uint4(0, 0, 0, 0);
    }
  };
  auto swrite = [&](int st) {
#pragma unroll
    for (int i = 0; i < SA; ++i) {
      const int row = (tid + i * 256) >> 3;
      smem[st][row * 8 + (seg ^ (row & 7))] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const int row = (tid + i * 256) >> 3;
      smem[st][(BM + row) * 8 + (seg ^ (row & 7))] = rb[i];
    }
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (K + kBK - 1) / kBK;
  gload(0);
  swrite(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * kBK);
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int sg = 2 * ks + (lane >> 5);   // 16-byte segment holding this lane's 8 k values
      uint4 a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * WM + i * 32 + (lane & 31);
        a[i] = smem[st][r * 8 + (sg ^ (r & 7))];
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wn * WN + j * 32 + (lane & 31);
        b[j] = smem[st][(BM + r) * 8 + (sg ^ (r & 7))];
      }
      // Operands swapped (B tile as the matrix-core "A"): lane l then holds
      // C[m = l%32][n = 8*(r/4) + 4*(l/32) + r%4] in accumulator r, i.e.
      // four consecutive n per group of four registers.
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, b[j]),
                                                               __builtin_bit_cast(bf16x8_t, a[i]),
                                                               acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) swrite(st ^ 1);
    __syncthreads();
  }

  // Epilogue: (GELU), round to bf16, 8-byte stores of 4 consecutive columns.
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = m0 + wm * WM + i * 32 + (lane & 31);
    if (m >= M) continue;
    uint16_t* crow = C + (int64_t)m * ldc;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * WN + j * 32 + 8 * g + 4 * (lane >> 5);
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[q] = acc[i][j][4 * g + q];
          if constexpr (EPI == kEpiGelu) v[q] = gelu_erf(v[q]);
        }
        if (n + 3 < N) {
          *reinterpret_cast<uint2*>(crow + n) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (n + q < N) crow[n + q] = (uint16_t)f32_to_bf16_rne(v[q]);
        }
      }
    }
  }
}

constexpr int kBM = kBuildTileM, kBN = 256;

size_t build_lut_min_workspace(int64_t D, int64_t F, int64_t N) {
  (void)D;
  return (size_t)kBM * (size_t)(N * F) * 2u;
}

size_t build_lut_rec_workspace(int64_t V, int64_t D, int64_t F, int64_t N) {
  (void)D;
  const size_t row_bytes = (size_t)(N * F) * 2u;
  const size_t target = (size_t)256 << 20;  // about the size of the last-level (MALL) cache
  int64_t rows = (int64_t)(target / row_bytes) / kBM * kBM;
  if (rows < kBM) rows = kBM;
  const int64_t vpad = (V + kBM - 1) / kBM * kBM;
  if (rows > vpad) rows = vpad;
  return (size_t)rows * row_bytes;
}

hipError_t launch_build_lut_bf16(const uint16_t* emb, const uint16_t* w_up, const uint16_t* w_down,
                                 uint16_t* lut, int64_t V, int64_t D, int64_t F, int64_t N,
                                 void* ws, size_t ws_bytes, hipStream_t s) {
  const int64_t NF = N * F;
  const int64_t row_bytes = NF * 2;
  // Vocabulary rows per block: all of V when the workspace holds them,
  // otherwise a whole number of row tiles.
  int64_t vc = (int64_t)(ws_bytes / (size_t)row_bytes);
  if (vc >= V) vc = V;
  else vc = vc / kBM * kBM;
  uint16_t* G = static_cast<uint16_t*>(ws);
  for (int64_t v0 = 0; v0 < V; v0 += vc) {
    const int64_t mc = (V - v0 < vc) ? (V - v0) : vc;
    dim3 g1((unsigned)((NF + kBN - 1) / kBN), (unsigned)((mc + kBM - 1) / kBM), 1);
    hipLaunchKernelGGL((gemm_nt_bf16_kernel<kBM, kBN, kEpiGelu>), g1, dim3(256), 0, s,
                       emb + v0 * D, D, (int64_t)0, w_up, D, (int64_t)0, G, NF, (int64_t)0,
                       (int)mc, (int)NF, (int)D);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    dim3 g2((unsigned)((D + kBN - 1) / kBN), (unsigned)((mc + kBM - 1) / kBM), (unsigned)N);
    hipLaunchKernelGGL((gemm_nt_bf16_kernel<kBM, kBN, kEpiStore>), g2, dim3(256), 0, s,
                       (const uint16_t*)G, NF, F, w_down, F, D * F, lut + v0 * N * D, N * D, D,
                       (int)mc, (int)D, (int)F);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// fp32 path
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void build_lut_f32_kernel(const float* __restrict__ emb,
                                                            const float* __restrict__ w_up,
                                                            const float* __restrict__ w_down,
                                                            float* __restrict__ lut, int D, int F,
                                                            int N) {
  extern __shared__ float sh[];
  float* x = sh;       // [D]
  float* g = sh + D;   // [F]
  const int64_t v = blockIdx.x;
  const int e = blockIdx.y;
  for (int d = threadIdx.x; d < D; d += blockDim.x) x[d] = emb[v * D + d];
  __syncthreads();
  for (int f = threadIdx.x; f < F; f += blockDim.x) {
    const float* w = w_up + ((int64_t)e * F + f) * D;
    float u = 0.f;
    for (int d = 0; d < D; ++d) u = fmaf(x[d], w[d], u);
    g[f] = gelu_erf(u);
  }
  __syncthreads();
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    const float* w = w_down + ((int64_t)e * D + d) * F;
    float acc = 0.f;
    for (int f = 0; f < F; ++f) acc = fmaf(g[f], w[f], acc);
    lut[(v * N + e) * D + d] = acc;
  }
}

hipError_t launch_build_lut_f32(const float* emb, const float* w_up, const float* w_down, float* lut,
                                int64_t V, int64_t D, int64_t F, int64_t N, hipStream_t s) {
  const size_t lds = (size_t)(D + F) * sizeof(float);
  for (int64_t v0 = 0; v0 < V; v0 += 65535) {
    const int64_t vc = (V - v0 < 65535) ? (V - v0) : 65535;
    hipLaunchKernelGGL(build_lut_f32_kernel, dim3((unsigned)vc, (unsigned)N), dim3(256), lds, s,
                       emb + v0 * D, w_up, w_down, lut + v0 * N * D, (int)D, (int)F, (int)N);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace mole
