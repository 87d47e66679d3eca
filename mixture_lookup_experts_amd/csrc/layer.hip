// The MoLE block at inference: residual stream x plus the shared expert's
// FFN plus the router-weighted table rows,
//
//   x[t][:] += W_s_down . GELU(W_s_up . h[t]) + sum_e g[t][e] * LUT[id_t][e][:]
//
// (MoLE article, training section: shared experts and the router keep
// reading the previous layer's output; complexity analysis: at inference
// only the shared experts are still computed, the routed ones are lookups.)
//
// Launch sequence on one stream, all scratch in the caller's workspace:
//   1. up-projection G = GELU(h . W_s_up^T), rounded to bf16 ([T][F]):
//      long batches use the 256x256 build GEMM, shorter ones the mid-size
//      GEMM below, split over K into fp32 partials plus a GELU reduction
//      when the batch alone cannot fill the chip; decode batches (T <= 8)
//      stream the weights through gemv_kernel, one wavefront per weight row;
//   2. down-projection of G into fp32 partial sums P[s][T][D], one per K
//      split (long batches: the 256x256 build GEMM over equal K splits;
//      decode batches: gemv_kernel, one partial);
//   3. the routed lookup-combine as the block's final pass, reading x and
//      adding the partial sums and the gate-weighted table rows:
//      x += sum_s P[s] + sum_e g_e LUT[id, e]  (the shared expert's output
//      never makes a separate trip through memory as a finished tensor).
//
// Mid-size GEMM (C = A . B^T, A [M][lda] bf16 = activations, B [N][ldb]
// bf16 = a weight matrix stored output-major): a 256-thread workgroup owns
// a (32*RM) x 128 output tile; each wave owns 32 output columns and all
// 32*RM rows, as RM v_mfma_f32_32x32x16_bf16 tiles.  Per 64-wide K slice
// the A panel is staged once in LDS (shared by the four waves; rows of 128
// bytes, 16-byte segment s of row r stored at s ^ ((r/2) & 7)) and each
// wave streams its own 32 weight rows straight into registers, 64
// contiguous bytes per lane.  Inside a slice the K order is permuted the
// same way for both operands (lane half h, K step i covers k = 32h + 8i ..
// 32h + 8i + 7), which leaves every dot product unchanged and lets a lane
// fetch its 64 weight bytes in one run.  Double-buffered LDS, one barrier
// per slice.  Operands are read through buffer resources, so rows past the
// edge and K past the split's end read zeros.
#include <algorithm>

#include "mole_device.hpp"
#include "mole_kernels.hpp"

namespace mole {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kMidBN = 128;             // output columns per mid-size tile (4 waves x 32)
constexpr int kTargetBlocks = 512;      // two workgroups per compute unit
constexpr int kMaxSplits = 16;          // K splits per projection
constexpr int64_t kGemvMaxT = 8;        // decode batches up to this many tokens stream the weights

enum { kMidGelu = 0, kMidPartial = 1 };

struct MidArgs {
  const uint16_t* A; int64_t lda;  // [M][lda]
  const uint16_t* B; int64_t ldb;  // [N][ldb]
  void* C; int64_t ldc;            // GELU: bf16 [M][ldc]; partial: fp32 [splits][M][ldc]
  int64_t sCz;                     // partial: elements between splits
  int M, N, K, Ks, tiles_n;
};

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// NSL == 0: the K loop above (double-buffered, one slice ahead).  NSL > 0
// (short splits of at most NSL slices): every load of the split is issued
// at once -- all A slices, then all weight slices, in straight-line code so
// each wait covers only the loads it needs -- the A slices go to NSL LDS
// buffers behind one barrier, and the MFMAs follow slice by slice as the
// weights arrive.  One memory latency per split instead of one per slice.
template <int RM, int EPI, int NSL>
__global__ __launch_bounds__(256) void gemm_mid_kernel(MidArgs p) {
  constexpr int BM = 32 * RM;
  __shared__ uint4 lds[NSL > 2 ? NSL : 2][BM * 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int tm = blockIdx.x / p.tiles_n, tn = blockIdx.x % p.tiles_n;
  const int m0 = tm * BM, n0 = tn * kMidBN;
  const int kb = blockIdx.y * p.Ks;
  const int ke = p.K - kb < p.Ks ? p.K : kb + p.Ks;
  const int rows_a = p.M - m0 < BM ? p.M - m0 : BM;
  const int rows_b = p.N - n0 < kMidBN ? p.N - n0 : kMidBN;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.A + (int64_t)m0 * p.lda), (short)0, (int)(rows_a * p.lda * 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.B + (int64_t)n0 * p.ldb), (short)0, (int)(rows_b * p.ldb * 2), kRsrcWord3);

  // A staging: thread t moves segment t % 8 of rows t / 8 + 32 i, i < RM.
  const int aseg = tid & 7, arow0 = tid >> 3;
  uint32_t aoff[RM];
  int alds[RM];
#pragma unroll
  for (int i = 0; i < RM; ++i) {
    const int row = arow0 + 32 * i;
    aoff[i] = row < rows_a ? (uint32_t)(row * p.lda * 2 + aseg * 16) : kOob;
    alds[i] = row * 8 + (aseg ^ ((row >> 1) & 7));
  }
  // Weight rows: lane l of wave w reads row 32 w + l % 32, K values 32 h .. 32 h + 31 of the slice.
  const int brow = 32 * wave + l32;
  const uint32_t boff = brow < rows_b ? (uint32_t)(brow * p.ldb * 2 + half * 64) : kOob;

  f32x16_t acc[RM];
#pragma unroll
  for (int r = 0; r < RM; ++r)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[r][q] = 0.f;
  // MFMAs of one slice: A fragments from LDS buffer `buf`, weights from b[].
  auto mfma_slice = [&](int buf, const uint4* b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sg = 4 * half + i;
#pragma unroll
      for (int r = 0; r < RM; ++r) {
        const int row = 32 * r + l32;
        const uint4 a = lds[buf][row * 8 + (sg ^ ((row >> 1) & 7))];
        // Operands swapped (weights as the matrix-core "A"): lane l then holds
        // C[m = l % 32][n = 8 (q / 4) + 4 (l / 32) + q % 4] in accumulator q.
        acc[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, b[i]),
                                                         __builtin_bit_cast(bf16x8_t, a), acc[r], 0, 0, 0);
      }
    }
  };
  auto a_off = [&](int i, int k0) { return k0 + aseg * 8 < ke ? aoff[i] + (uint32_t)k0 * 2u : kOob; };
  auto b_off = [&](int c, int k0) { return k0 + 32 * half + 8 * c < ke ? boff + (uint32_t)(k0 + 8 * c) * 2u : kOob; };

  if constexpr (NSL > 0) {
    uint4 ast[NSL][RM], bst[NSL][4];
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
      for (int i = 0; i < RM; ++i) ast[sl][i] = buf_load16(ra, a_off(i, kb + 64 * sl));
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
      for (int c = 0; c < 4; ++c) bst[sl][c] = buf_load16(rb, b_off(c, kb + 64 * sl));
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
      for (int i = 0; i < RM; ++i) lds[sl][alds[i]] = ast[sl][i];
    __syncthreads();
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) mfma_slice(sl, bst[sl]);
  } else {
  uint4 astg[RM], bcur[4], bnxt[4];
  auto load_slice = [&](int k0, uint4* bdst) {
#pragma unroll
    for (int i = 0; i < RM; ++i) astg[i] = buf_load16(ra, a_off(i, k0));
#pragma unroll
    for (int c = 0; c < 4; ++c) bdst[c] = buf_load16(rb, b_off(c, k0));
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < RM; ++i) lds[buf][alds[i]] = astg[i];
  };

  const int ns = ke > kb ? (ke - kb + 63) / 64 : 0;
  if (ns > 0) {
    load_slice(kb, bcur);
    store_a(0);
  }
  __syncthreads();
  for (int s = 0; s < ns; ++s) {
    const int buf = s & 1;
    if (s + 1 < ns) load_slice(kb + (s + 1) * 64, bnxt);
    mfma_slice(buf, bcur);
    if (s + 1 < ns) store_a(buf ^ 1);
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 4; ++c) bcur[c] = bnxt[c];
  }
  }

  // Epilogue: lane l, accumulator group g (4 registers) = 4 consecutive columns.
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    const int m = m0 + 32 * r + l32;
    if (m >= p.M) continue;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int n = n0 + 32 * wave + 8 * g + 4 * half;
      if (n >= p.N) continue;
      const float v0 = acc[r][4 * g], v1 = acc[r][4 * g + 1], v2 = acc[r][4 * g + 2], v3 = acc[r][4 * g + 3];
      const int64_t o = (int64_t)m * p.ldc + n;
      if constexpr (EPI == kMidGelu) {
        uint2 w;
        w.x = pack_bf16x2(gelu_poly(v0), gelu_poly(v1));
        w.y = pack_bf16x2(gelu_poly(v2), gelu_poly(v3));
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.C) + o) = w;
      } else {
        float* dst = static_cast<float*>(p.C) + (int64_t)blockIdx.y * p.sCz + o;
        *reinterpret_cast<float4*>(dst) = make_float4(v0, v1, v2, v3);
      }
    }
  }
}

// sum_s P[s][i] for four consecutive i; all S loads are issued before the
// first add, so a short pass waits for memory once, not S times.
__device__ __forceinline__ float4 sum_splits(const float* __restrict__ P, int S, int64_t count, int64_t i) {
  float4 v[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s)
    if (s < S) v[s] = reinterpret_cast<const float4*>(P + (int64_t)s * count)[i];
  float4 a = v[0];
#pragma unroll
  for (int s = 1; s < kMaxSplits; ++s)
    if (s < S) {
      a.x += v[s].x; a.y += v[s].y; a.z += v[s].z; a.w += v[s].w;
    }
  return a;
}

// G[i] = bf16(GELU(sum_s P[s][i])).
__global__ __launch_bounds__(256) void gelu_reduce_kernel(const float* __restrict__ P, int S, int64_t count,
                                                          uint16_t* __restrict__ G) {
  const int64_t n4 = count / 4;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const float4 a = sum_splits(P, S, count, i);
    uint2 w;
    w.x = pack_bf16x2(gelu_poly(a.x), gelu_poly(a.y));
    w.y = pack_bf16x2(gelu_poly(a.z), gelu_poly(a.w));
    reinterpret_cast<uint2*>(G)[i] = w;
  }
}

// Decode-sized products: out[t][r] = epi( sum_k X[t][k] W[r][k] ) for
// T <= TT tokens (X bf16 [T][ldx], W bf16 [R][ldw] output-major).  `wpr`
// wavefronts (1, 2 or 4) of a workgroup share an output row: lanes stride
// over K in 16-byte chunks, four chunks' loads in flight at a time, every
// token's dot product in fp32, then a wavefront sum, and the row's wpr
// sums are added in wave order through LDS.  One row per wavefront keeps
// the most loads in flight across the chip (measured: four rows per
// wavefront, sharing the token chunks, was slower).  EPI kMidGelu:
// bf16(GELU) to C [T][ldc]; kMidPartial: fp32 to C [T][ldc].  Needs
// K % 8 == 0.
template <int TT, int EPI>
__global__ __launch_bounds__(256) void gemv_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                   const uint16_t* __restrict__ W, int64_t ldw, void* C,
                                                   int64_t ldc, int T, int R, int K, int wpr) {
  __shared__ float part[4][TT];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = wave / wpr, share = wave - slot * wpr;
  const int rr = blockIdx.x * (4 / wpr) + slot;
  const bool valid = rr < R;
  const int r = valid ? rr : R - 1;  // a slot past the end reads the last row and stores nothing
  const uint16_t* wrow = W + (int64_t)r * ldw;
  const int nchunk = K / 8, step = 64 * wpr;
  float acc[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) acc[t] = 0.f;
  for (int c0 = share * 64 + lane; c0 < nchunk; c0 += 4 * step) {
    // four chunks per trip, loads first (clamped in bounds, masked where used)
    uint4 wv[4], xv[4][TT];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + step * u < nchunk ? c0 + step * u : c0;
      wv[u] = ldg16(wrow + c * 8);
#pragma unroll
      for (int t = 0; t < TT; ++t) xv[u][t] = ldg16(X + (int64_t)(t < T ? t : 0) * ldx + c * 8);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (c0 + step * u < nchunk) {
        float wf[8];
        Elem<uint16_t>::unpack(wv[u], wf);
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          float xf[8];
          Elem<uint16_t>::unpack(xv[u][t], xf);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[t] = fmaf(xf[i], wf[i], acc[t]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc[t] += __shfl_xor(acc[t], m, 64);
  if (lane == 0) {
#pragma unroll
    for (int t = 0; t < TT; ++t) part[wave][t] = acc[t];
  }
  __syncthreads();
  if (share == 0 && lane < TT && valid) {
    const int t = lane;
    if (t < T) {
      float v = part[wave][t];
      for (int w = 1; w < wpr; ++w) v += part[wave + w][t];
      if constexpr (EPI == kMidGelu)
        static_cast<uint16_t*>(C)[t * ldc + r] = (uint16_t)f32_to_bf16_rne(gelu_poly(v));
      else
        static_cast<float*>(C)[t * ldc + r] = v;
    }
  }
}

// Wavefronts per row: enough that a lane has at most four chunks of the row
// (one trip of loads), up to four.
template <int EPI>
hipError_t launch_gemv(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw, void* C, int64_t ldc, int T,
                       int R, int K, hipStream_t s) {
  int wpr = 1;
  while (wpr < 4 && K / 8 > 256 * wpr) wpr *= 2;
  const int rows_per_block = 4 / wpr;
  const dim3 grid((unsigned)((R + rows_per_block - 1) / rows_per_block));
  if (T <= 1)
    hipLaunchKernelGGL((gemv_kernel<1, EPI>), grid, dim3(256), 0, s, X, ldx, W, ldw, C, ldc, T, R, K, wpr);
  else if (T <= 2)
    hipLaunchKernelGGL((gemv_kernel<2, EPI>), grid, dim3(256), 0, s, X, ldx, W, ldw, C, ldc, T, R, K, wpr);
  else if (T <= 4)
    hipLaunchKernelGGL((gemv_kernel<4, EPI>), grid, dim3(256), 0, s, X, ldx, W, ldw, C, ldc, T, R, K, wpr);
  else
    hipLaunchKernelGGL((gemv_kernel<8, EPI>), grid, dim3(256), 0, s, X, ldx, W, ldw, C, ldc, T, R, K, wpr);
  return hipGetLastError();
}

template <int RM, int EPI, int NSL>
hipError_t launch_mid_rm(const MidArgs& p, int tiles_m, int splits, hipStream_t s) {
  hipLaunchKernelGGL((gemm_mid_kernel<RM, EPI, NSL>), dim3((unsigned)(tiles_m * p.tiles_n), (unsigned)splits),
                     dim3(256), 0, s, p);
  return hipGetLastError();
}

// Short splits take the all-loads-at-once form for tile heights of 32 and
// 64 rows when at most one of its slices would be padding (4 slices for
// splits of 3-4, 8 for 7-8; measured: padding slices cost more than the
// loop saves); taller tiles and other splits loop.
template <int EPI>
hipError_t launch_mid(int rm, const MidArgs& p, int splits, hipStream_t s) {
  const int tiles_m = (p.M + 32 * rm - 1) / (32 * rm);
  const int ns = (p.Ks + 63) / 64;
  switch (rm) {
    case 1:
      if (ns >= 3 && ns <= 4) return launch_mid_rm<1, EPI, 4>(p, tiles_m, splits, s);
      if (ns >= 7 && ns <= 8) return launch_mid_rm<1, EPI, 8>(p, tiles_m, splits, s);
      return launch_mid_rm<1, EPI, 0>(p, tiles_m, splits, s);
    case 2:
      if (ns >= 3 && ns <= 4) return launch_mid_rm<2, EPI, 4>(p, tiles_m, splits, s);
      if (ns >= 7 && ns <= 8) return launch_mid_rm<2, EPI, 8>(p, tiles_m, splits, s);
      return launch_mid_rm<2, EPI, 0>(p, tiles_m, splits, s);
    default: return launch_mid_rm<4, EPI, 0>(p, tiles_m, splits, s);
  }
}

// Mid-size tile height for a projection with `out` output columns: the
// tallest tile (most reuse of each weight row) that still gives 128 tiles,
// else the shortest.
int pick_rm(int64_t T, int64_t out) {
  const int64_t tn = (out + kMidBN - 1) / kMidBN;
  for (int rm : {4, 2}) {
    if (T <= 32 * (rm / 2)) continue;  // a taller tile than the batch wastes its rows
    if (((T + 32 * rm - 1) / (32 * rm)) * tn >= 128) return rm;
  }
  return 1;
}

// K splits for a projection with `tiles` output tiles: enough workgroups to
// fill the chip, at least 128 of K per split, and partial sums of at most
// four times the weight matrix's bytes (sp * T * out * 4 <= 4 * K * out * 2).
int pick_splits(int64_t tiles, int64_t T, int64_t K) {
  int64_t sp = (kTargetBlocks + tiles - 1) / tiles;
  if (T <= 64 * 2) sp = std::max<int64_t>(sp, (K + 511) / 512);  // short splits load all at once
  sp = std::min<int64_t>(sp, std::max<int64_t>(1, K / 128));
  sp = std::min<int64_t>(sp, std::max<int64_t>(1, 2 * K / T));
  return (int)std::max<int64_t>(1, std::min<int64_t>(sp, kMaxSplits));
}

inline size_t round256(size_t x) { return (x + 255u) & ~(size_t)255u; }

// Workgroups for a grid-stride pass over n4 groups of four elements.
unsigned grid_1d(int64_t n4) {
  const int64_t b = (n4 + 255) / 256;
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(b, 4096));
}

}  // namespace

LayerPlan layer_plan(int64_t T, int64_t D, int64_t F) {
  LayerPlan pl{};
  if (T <= kGemvMaxT) {
    // decode batch: both projections stream their weights (gemv_kernel),
    // the down-projection as one partial
    pl.gemv = true;
    pl.s_up = pl.s_down = 1;
    pl.ks_up = D;
    pl.ks_down = F;
    pl.rm_up = pl.rm_down = 1;
    pl.yr_off = 0;
    pl.g_off = round256((size_t)T * (size_t)D * 4u);
    pl.p_off = pl.g_off + round256((size_t)T * (size_t)F * 2u);
    pl.total = pl.p_off + round256((size_t)T * (size_t)D * 4u);
    return pl;
  }
  // The 256x256 GEMM needs a full chip's worth of tiles (counting K splits)
  // to beat the mid-size one.
  pl.big_up = ((T + 255) / 256) * ((F + 255) / 256) >= 256;
  pl.rm_up = pick_rm(T, F);
  pl.s_up = pl.big_up ? 1 : pick_splits(((T + 32 * pl.rm_up - 1) / (32 * pl.rm_up)) * ((F + kMidBN - 1) / kMidBN), T, D);
  pl.ks_up = ((D + pl.s_up - 1) / pl.s_up + 63) / 64 * 64;
  pl.s_up = (int)((D + pl.ks_up - 1) / pl.ks_up);
  // Down-projection on the 256x256 GEMM: equal K splits (F / s, a multiple of
  // 64) until the tiles fill the chip.
  pl.big_down = false;
  const int64_t tiles_big = ((T + 255) / 256) * ((D + 255) / 256);
  if (T >= 2048 && D <= ((int64_t)1 << 20)) {
    for (int sp = 1; sp <= 8; sp *= 2) {
      if (F % (64 * sp) != 0) break;
      pl.big_down = true;
      pl.s_down = sp;
      pl.ks_down = F / sp;
      if (tiles_big * sp >= 256) break;
    }
  }
  pl.rm_down = pick_rm(T, D);
  if (!pl.big_down) {
    pl.s_down = pick_splits(((T + 32 * pl.rm_down - 1) / (32 * pl.rm_down)) * ((D + kMidBN - 1) / kMidBN), T, F);
    pl.ks_down = ((F + pl.s_down - 1) / pl.s_down + 63) / 64 * 64;
    pl.s_down = (int)((F + pl.ks_down - 1) / pl.ks_down);
  }
  const size_t yr = (size_t)T * (size_t)D * 4u;
  const size_t g = (size_t)T * (size_t)F * 2u;
  const size_t p_up = pl.s_up > 1 ? (size_t)pl.s_up * (size_t)T * (size_t)F * 4u : 0;
  const size_t p_down = (size_t)pl.s_down * (size_t)T * (size_t)D * 4u;
  pl.yr_off = 0;
  pl.g_off = round256(yr);
  pl.p_off = pl.g_off + round256(g);
  pl.total = pl.p_off + round256(std::max(p_up, p_down));
  return pl;
}

hipError_t launch_layer_forward(const int64_t* ids, const uint16_t* h, const uint16_t* w_r, const uint16_t* lut,
                                const uint16_t* w_s_up, const uint16_t* w_s_down, float* x, int64_t T, int64_t D,
                                int64_t N, int64_t F, void* ws, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const LayerPlan pl = layer_plan(T, D, F);
  char* base = static_cast<char*>(ws);
  float* yr = reinterpret_cast<float*>(base + pl.yr_off);
  uint16_t* G = reinterpret_cast<uint16_t*>(base + pl.g_off);
  float* P = reinterpret_cast<float*>(base + pl.p_off);

  hipError_t err;
  // 1. Shared expert, up-projection with GELU.
  if (pl.gemv) {
    err = launch_gemv<kMidGelu>(h, D, w_s_up, D, G, F, (int)T, (int)F, (int)D, s);
  } else if (pl.big_up) {
    err = launch_gemm_gelu_bf16(h, D, w_s_up, D, G, F, (int)T, (int)F, (int)D, s);
  } else {
    MidArgs a{h, D, w_s_up, D, nullptr, F, T * F, (int)T, (int)F, (int)D, (int)pl.ks_up,
              (int)((F + kMidBN - 1) / kMidBN)};
    if (pl.s_up == 1) {
      a.C = G;
      err = launch_mid<kMidGelu>(pl.rm_up, a, 1, s);
    } else {
      a.C = P;
      err = launch_mid<kMidPartial>(pl.rm_up, a, pl.s_up, s);
      if (err == hipSuccess) {
        hipLaunchKernelGGL(gelu_reduce_kernel, dim3(grid_1d(T * F / 4)), dim3(256), 0, s, P, pl.s_up, T * F, G);
        err = hipGetLastError();
      }
    }
  }
  if (err != hipSuccess) return err;

  // 2. Shared expert, down-projection: fp32 partial sums per K split.
  if (pl.gemv) {
    err = launch_gemv<kMidPartial>(G, F, w_s_down, F, P, D, (int)T, (int)D, (int)F, s);
  } else if (pl.big_down) {
    err = launch_gemm_f32_bf16(G, F, pl.ks_down, w_s_down, F, pl.ks_down, P, D, T * D, (int)T, (int)D,
                               (int)pl.ks_down, pl.s_down, s);
  } else {
    MidArgs b{G, F, w_s_down, F, P, D, T * D, (int)T, (int)D, (int)F, (int)pl.ks_down,
              (int)((D + kMidBN - 1) / kMidBN)};
    err = launch_mid<kMidPartial>(pl.rm_down, b, pl.s_down, s);
  }
  if (err != hipSuccess) return err;

  // 3. Routed lookup-combine, adding the shared expert's partial sums and the
  //    table rows to the residual stream (staged router gates go to yr).
  return launch_lookup_combine(ids, h, w_r, lut, x, T, D, N, kBF16, true, s, yr, P, pl.s_down, T * D);
}

}  // namespace mole
