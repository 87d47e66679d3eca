// Training mode of the routed experts (MoLE article, training section:
// every routed expert reads the token's shallow embedding, all experts are
// active with dense softmax gates, the router reads the contextual hidden
// state; inference section: the lookup table is this forward pass evaluated
// on every vocabulary row -- here it is evaluated on the batch's rows only).
//
// Forward, for the U distinct ids of a batch (uniq) and the token -> row map
// (remap):
//   X = Emb[uniq]                                    (gather)
//   Upre = X . W_up^T, G = GELU(Upre), O[:, e, :] = G_e . W_down[e]^T
//                                                    (the build's two GEMMs)
//   y = sum_e softmax(W_r h)[e] O[remap, e, :]       (the lookup-combine)
// X, Upre, G and O stay in the caller's forward workspace for the backward
// pass.
//
// Backward for an upstream gradient dy [T][D] (fp32):
//   per token:   g = softmax(W_r h), dg_e = dy . O[remap, e], dz = g (dg - g.dg),
//                d_h = sum_e dz_e W_r[e]                     (gate_backward_kernel)
//   router:      d_W_r = dz^T . h                            (two reduction passes)
//   per row u:   dO[u][e] = sum_{t : remap t = u} g_te dy_t  (tokens grouped by row)
//   experts:     dU_e = (dO_e . W_down[e]) * GELU'(X . W_up^T)   (one GEMM epilogue)
//                d_W_down[e] = dO_e^T . G_e,  d_W_up[e] = dU_e^T . X,
//                d_X = dU . W_up  (= the gradient of the rows Emb[uniq])
// The four products run on the 256x256 MFMA GEMM (C = A . B^T, fp32 or
// fused-epilogue output); operands whose contraction index is not the
// contiguous one (the rows U, or the weights' output dimension) are read in
// place as MN-major operands and transposed in registers on their way to
// LDS.  dO, dU and the pre-activations are rounded to bf16 for the matrix
// cores; all sums are fp32.  The per-row gradient sums walk a host-built
// list of the tokens grouped by row in fixed chunks and add the pieces of
// rows that cross chunks in chunk order, so no atomics and the result does
// not depend on scheduling.
#include <algorithm>

#include "mole_device.hpp"
#include "mole_kernels.hpp"

namespace mole {

namespace {

constexpr int kWrChunk = 16;   // tokens per partial sum of the router-weight gradient
constexpr int kMaxSeg = 64;    // most token-list positions per row-gradient chunk

// Columns per lane of the row-gradient walk: NP * CPL accumulators <= 64.
template <int NP>
struct RowGradCols {
  static constexpr int kCpl = NP >= 64 ? 1 : (NP >= 32 ? 2 : 4);
};

template <int CPL>
__device__ __forceinline__ void load_cols(const float* p, float* v) {
  if constexpr (CPL == 4) {
    const float4 q = *reinterpret_cast<const float4*>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  } else if constexpr (CPL == 2) {
    const float2 q = *reinterpret_cast<const float2*>(p);
    v[0] = q.x; v[1] = q.y;
  } else {
    v[0] = *p;
  }
}

template <int CPL>
__device__ __forceinline__ void load_bf16_cols(const uint16_t* p, float* v) {
  if constexpr (CPL == 4) {
    const uint2 q = *reinterpret_cast<const uint2*>(p);
    v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
  } else if constexpr (CPL == 2) {
    const uint32_t q = *reinterpret_cast<const uint32_t*>(p);
    v[0] = bf16_lo(q); v[1] = bf16_hi(q);
  } else {
    v[0] = bf16_to_f32(*p);
  }
}

template <int CPL>
__device__ __forceinline__ void store_bf16_cols(uint16_t* p, const float* v) {
  if constexpr (CPL == 4)
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  else if constexpr (CPL == 2)
    *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(v[0], v[1]);
  else
    *p = (uint16_t)f32_to_bf16_rne(v[0]);
}

template <int CPL>
__device__ __forceinline__ void store_f32_cols(float* p, const float* v) {
  if constexpr (CPL == 4)
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  else if constexpr (CPL == 2)
    *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
  else
    *p = v[0];
}

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

// Per token t (wpt = 1, 2 or 4 wavefronts of a workgroup, each over its
// share of the columns, 8 consecutive columns per lane and trip): router
// logits z_e = h_t . W_r[e] and dg_e = dy_t . O[remap_t][e] as lane sums, a
// reduce-scatter across each wavefront, the token's 2N totals summed from
// LDS in wave order by every lane, softmax and dz, then
// d_h[t] = sum_e dz_e W_r[e] over each wave's columns.
template <int NP, int WPT>
__global__ __launch_bounds__(256) void gate_backward_kernel(const uint16_t* __restrict__ h,
                                                            const uint16_t* __restrict__ w_r,
                                                            const uint16_t* __restrict__ O,
                                                            const int64_t* __restrict__ remap,
                                                            const float* __restrict__ dy, float* __restrict__ g_out,
                                                            float* __restrict__ dz_out, float* __restrict__ d_h,
                                                            int64_t T, int D, int N) {
  constexpr int wpt = WPT;
  using RS = ReduceScatter<2 * NP, kWave>;
  __shared__ float tot[4][2 * NP];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = wave / wpt, part = wave - slot * wpt;  // token slot of the workgroup, column share
  const int64_t tw = (int64_t)blockIdx.x * (4 / wpt) + slot;
  const bool valid = tw < T;
  const int64_t t = valid ? tw : T - 1;  // a slot past the end recomputes the last token and stores nothing
  const int span = (D / 8 + wpt - 1) / wpt * 8;
  const int c_lo = part * span, c_hi = min(D, c_lo + span);
  const uint16_t* orow = O + remap[t] * (int64_t)N * D;
  float v[2 * NP];  // z_e, then dg_e
#pragma unroll
  for (int e = 0; e < 2 * NP; ++e) v[e] = 0.f;
  for (int c = c_lo + lane * 8; c < c_hi; c += 512) {
    float hv[8], yv[8];
    Elem<uint16_t>::unpack(ldg16(h + t * D + c), hv);
    Elem<float>::unpack(ldg16(dy + t * D + c), yv);
    Elem<float>::unpack(ldg16(dy + t * D + c + 4), yv + 4);
#pragma unroll
    for (int e = 0; e < NP; ++e) {
      if (e < N) {
        float wv[8], ov[8];
        Elem<uint16_t>::unpack(ldg16(w_r + (int64_t)e * D + c), wv);
        Elem<uint16_t>::unpack(ldg16(orow + (int64_t)e * D + c), ov);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          v[e] = fmaf(hv[i], wv[i], v[e]);
          v[NP + e] = fmaf(yv[i], ov[i], v[NP + e]);
        }
      }
    }
  }
  RS::run(v, lane);
  {
    const int off = RS::offset(lane);
#pragma unroll
    for (int i = 0; i < RS::kLeft; ++i) tot[wave][off + i] = v[i];  // lanes with one offset hold one total
  }
  __syncthreads();
  float zz[NP], dd[NP];
  float zmax = -INFINITY;
#pragma unroll
  for (int e = 0; e < NP; ++e) {
    zz[e] = tot[slot * wpt][e];
    dd[e] = tot[slot * wpt][NP + e];
#pragma unroll
    for (int w = 1; w < wpt; ++w) {
      zz[e] += tot[slot * wpt + w][e];
      dd[e] += tot[slot * wpt + w][NP + e];
    }
    if (e < N) zmax = fmaxf(zmax, zz[e]);
  }
  // (every lane computes the same softmax; loops over the compile-time
  // bound NP keep the arrays in registers)
  float sum = 0.f;
#pragma unroll
  for (int e = 0; e < NP; ++e) {
    zz[e] = e < N ? expf(zz[e] - zmax) : 0.f;
    sum += zz[e];
  }
  float gdg = 0.f;
#pragma unroll
  for (int e = 0; e < NP; ++e) {
    zz[e] /= sum;
    gdg = fmaf(zz[e], dd[e], gdg);
  }
  float my_g = 0.f, my_dz = 0.f;
#pragma unroll
  for (int e = 0; e < NP; ++e) {
    dd[e] = zz[e] * (dd[e] - gdg);  // dz_e
    if (lane == e) {
      my_g = zz[e];
      my_dz = dd[e];
    }
  }
  if (valid && part == 0 && lane < N) {
    g_out[t * N + lane] = my_g;
    dz_out[t * N + lane] = my_dz;
  }
  for (int c = c_lo + lane * 8; c < c_hi; c += 512) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
    for (int e = 0; e < NP; ++e) {
      if (e < N) {
        float wv[8];
        Elem<uint16_t>::unpack(ldg16(w_r + (int64_t)e * D + c), wv);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(dd[e], wv[i], acc[i]);
      }
    }
    if (valid) {
      float4* o = reinterpret_cast<float4*>(d_h + t * D + c);
      o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

template <int NP> constexpr auto gate_backward_kernel_w1 = gate_backward_kernel<NP, 1>;
template <int NP> constexpr auto gate_backward_kernel_w2 = gate_backward_kernel<NP, 2>;
template <int NP> constexpr auto gate_backward_kernel_w4 = gate_backward_kernel<NP, 4>;

// Partial router-weight gradient over one chunk of tokens:
// P[chunk][e][d] = sum_{t in chunk} dz[t][e] h[t][d].  A workgroup owns
// 64*CPL columns; its four wavefronts take every fourth token of the chunk
// and their sums are added in wave order through LDS.
template <int NP>
__global__ __launch_bounds__(256) void wr_partial_kernel(const float* __restrict__ dz, const uint16_t* __restrict__ h,
                                                         float* __restrict__ P, int64_t T, int D, int N) {
  constexpr int CPL = RowGradCols<NP>::kCpl;
  __shared__ float part[3][NP * CPL][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c0 = (blockIdx.x * 64 + lane) * CPL;
  const bool ok = c0 < D;
  const int cc = ok ? c0 : 0;  // in-bounds column for the loads of an idle lane
  const int64_t t0 = (int64_t)blockIdx.y * kWrChunk;
  const int64_t t1 = T - t0 < kWrChunk ? T : t0 + kWrChunk;
  float acc[NP][CPL];
#pragma unroll
  for (int e = 0; e < NP; ++e)
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[e][c] = 0.f;
  for (int64_t t = t0 + wave; t < t1; t += 16) {
    float hv[4][CPL];
#pragma unroll
    for (int q = 0; q < 4; ++q) load_bf16_cols<CPL>(h + (t + 4 * q < t1 ? t + 4 * q : t1 - 1) * D + cc, hv[q]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (t + 4 * q < t1) {
#pragma unroll
        for (int e = 0; e < NP; ++e) {
          if (e < N) {
            const float ze = dz[(t + 4 * q) * N + e];
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[e][c] = fmaf(ze, hv[q][c], acc[e][c]);
          }
        }
      }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int e = 0; e < NP; ++e)
#pragma unroll
      for (int c = 0; c < CPL; ++c) part[wave - 1][e * CPL + c][lane] = acc[e][c];
  }
  __syncthreads();
  if (wave == 0 && ok) {
    float* out = P + (int64_t)blockIdx.y * N * D + c0;
#pragma unroll
    for (int e = 0; e < NP; ++e) {
      if (e < N) {
        float v[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c)
          v[c] = acc[e][c] + part[0][e * CPL + c][lane] + part[1][e * CPL + c][lane] + part[2][e * CPL + c][lane];
        store_f32_cols<CPL>(out + (int64_t)e * D, v);
      }
    }
  }
}

// Row gradients dO[u][e][d] = bf16( sum over the tokens t of row u of
// g[t][e] dy[t][d] ), by fixed chunks of `seg` positions of the token list
// grouped by row (tok, row_ptr), so that a row with hundreds of tokens (the
// head of a Zipf batch) is spread over many workgroups.  A row that lies
// inside one chunk is summed and written there.  A row cut by a chunk
// boundary leaves an fp32 partial sum per chunk it touches, in slot 0 of
// that chunk when the row holds the chunk's first position and in slot 1
// otherwise (it then starts inside the chunk and runs past its end);
// row_grad_fix_kernel adds those in chunk order.  Each wave owns 64*CPL
// columns and walks the chunk's positions in order.
template <int NP>
__global__ __launch_bounds__(256) void row_grad_kernel(const float* __restrict__ g, const float* __restrict__ dy,
                                                       const int64_t* __restrict__ remap,
                                                       const int64_t* __restrict__ row_ptr,
                                                       const int64_t* __restrict__ tok, uint16_t* __restrict__ dO,
                                                       float* __restrict__ part, int64_t T, int seg, int D, int N) {
  constexpr int CPL = RowGradCols<NP>::kCpl;
  __shared__ float gs[kMaxSeg][NP];
  __shared__ int64_t ts[kMaxSeg], rs[kMaxSeg + 1], k0s[kMaxSeg], k1s[kMaxSeg];
  const int64_t p0 = (int64_t)blockIdx.x * seg;
  const int len = (int)(T - p0 < seg ? T - p0 : seg);
  const int tid = threadIdx.x;
  if (tid < len) {
    const int64_t t = tok[p0 + tid];
    const int64_t r = remap[t];
    ts[tid] = t;
    rs[tid] = r;
    k0s[tid] = row_ptr[r];
    k1s[tid] = row_ptr[r + 1];
  }
  if (tid == 0) rs[len] = -1;  // sentinel: the last position ends its row's run
  __syncthreads();
  for (int i = tid; i < len * NP; i += 256) {
    const int q = i / NP, e = i % NP;
    gs[q][e] = e < N ? g[ts[q] * N + e] : 0.f;
  }
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6;
  const int c0 = ((blockIdx.y * 4 + wave) * 64 + lane) * CPL;
  if (c0 >= D) return;  // (no barrier follows)
  const int64_t pend = p0 + len;
  float acc[NP][CPL];
#pragma unroll
  for (int e = 0; e < NP; ++e)
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[e][c] = 0.f;
  // Positions in batches of four, double-buffered: the next batch's dy rows
  // are loaded (clamped to the chunk, so always in bounds) while this one
  // is summed.
  float ya[4][CPL], yb[4][CPL];
  auto load4 = [&](int pb, float (*y)[CPL]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int pq = pb + q < len ? pb + q : len - 1;
      load_cols<CPL>(dy + ts[pq] * D + c0, y[q]);
    }
  };
  auto walk4 = [&](int pb, float (*y)[CPL]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int pq = pb + q;
      if (pq < len) {
#pragma unroll
        for (int e = 0; e < NP; ++e) {
          const float ge = gs[pq][e];
#pragma unroll
          for (int c = 0; c < CPL; ++c) acc[e][c] = fmaf(ge, y[q][c], acc[e][c]);
        }
        const int64_t r = rs[pq];
        if (rs[pq + 1] != r) {  // end of this row's run in the chunk
          const int64_t k0 = k0s[pq], k1 = k1s[pq];
          if (k0 >= p0 && k1 <= pend) {
            uint16_t* out = dO + r * (int64_t)N * D + c0;
#pragma unroll
            for (int e = 0; e < NP; ++e)
              if (e < N) store_bf16_cols<CPL>(out + (int64_t)e * D, acc[e]);
          } else {
            const int slot = k0 <= p0 ? 0 : 1;
            float* out = part + ((int64_t)blockIdx.x * 2 + slot) * N * D + c0;
#pragma unroll
            for (int e = 0; e < NP; ++e)
              if (e < N) store_f32_cols<CPL>(out + (int64_t)e * D, acc[e]);
          }
#pragma unroll
          for (int e = 0; e < NP; ++e)
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[e][c] = 0.f;
        }
      }
    }
  };
  load4(0, ya);
  for (int pb = 0; pb < len; pb += 8) {
    load4(pb + 4, yb);
    walk4(pb, ya);
    load4(pb + 8, ya);
    walk4(pb + 4, yb);
  }
}

// Rows cut by chunk boundaries: the chunk in which such a row starts (it
// holds that chunk's last position and runs past it) sums the row's partials
// over every chunk it touches, in chunk order, and writes the bf16 row.
__global__ __launch_bounds__(256) void row_grad_fix_kernel(const float* __restrict__ part,
                                                           const int64_t* __restrict__ remap,
                                                           const int64_t* __restrict__ row_ptr,
                                                           const int64_t* __restrict__ tok, uint16_t* __restrict__ dO,
                                                           int64_t T, int seg, int64_t ND) {
  const int64_t j = blockIdx.x;
  const int64_t p0 = j * seg, pend = T - p0 < seg ? T : p0 + seg;
  const int64_t r = remap[tok[pend - 1]];
  const int64_t k0 = row_ptr[r], k1 = row_ptr[r + 1];
  if (!(k0 >= p0 && k1 > pend)) return;
  const int64_t jl = (k1 - 1) / seg;
  for (int64_t i = ((int64_t)blockIdx.y * 256 + threadIdx.x) * 4; i < ND; i += (int64_t)gridDim.y * 1024) {
    // chunks j, j+1, ... in four interleaved chains (a head row touches
    // dozens of chunks), added in chain order at the end
    float4 a[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) a[q] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int64_t jj = j; jj <= jl; jj += 4) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (jj + q <= jl) {
          const int slot = k0 <= (jj + q) * seg ? 0 : 1;
          const float4 x = *reinterpret_cast<const float4*>(part + ((jj + q) * 2 + slot) * ND + i);
          a[q].x += x.x;
          a[q].y += x.y;
          a[q].z += x.z;
          a[q].w += x.w;
        }
      }
    }
    const float s0 = (a[0].x + a[1].x) + (a[2].x + a[3].x), s1 = (a[0].y + a[1].y) + (a[2].y + a[3].y);
    const float s2 = (a[0].z + a[1].z) + (a[2].z + a[3].z), s3 = (a[0].w + a[1].w) + (a[2].w + a[3].w);
    *reinterpret_cast<uint2*>(dO + r * ND + i) = make_uint2(pack_bf16x2(s0, s1), pack_bf16x2(s2, s3));
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

// out[i] = sum_s P[s][i] for many partials (S > 16): a workgroup of 16
// wavefronts owns 256 outputs (a float4 per lane); wavefront r sums the
// partials s = r, r + 16, ... and the 16 sums are added in r order in LDS.
// Needs count % 4 == 0.
__global__ __launch_bounds__(1024) void sum_partials_wide_kernel(const float* __restrict__ P, int S, int64_t count,
                                                                 float* __restrict__ out) {
  __shared__ float4 red[16][64];
  const int lane = threadIdx.x & 63, r = threadIdx.x >> 6;
  const int64_t i = ((int64_t)blockIdx.x * 64 + lane) * 4;
  const bool ok = i < count;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;  // two chains
  int sp = r;
  for (; sp + 16 < S; sp += 32) {
    if (ok) {
      const float4 x = *reinterpret_cast<const float4*>(P + (int64_t)sp * count + i);
      const float4 y = *reinterpret_cast<const float4*>(P + (int64_t)(sp + 16) * count + i);
      a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
      b.x += y.x; b.y += y.y; b.z += y.z; b.w += y.w;
    }
  }
  if (sp < S && ok) {
    const float4 x = *reinterpret_cast<const float4*>(P + (int64_t)sp * count + i);
    a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
  }
  red[r][lane] = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
  __syncthreads();
  if (r == 0 && ok) {
    float4 t = red[0][lane];
    for (int k = 1; k < 16; ++k) {
      const float4 x = red[k][lane];
      t.x += x.x; t.y += x.y; t.z += x.z; t.w += x.w;
    }
    *reinterpret_cast<float4*>(out + i) = t;
  }
}

unsigned grid_for(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(b, 8192));
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
  // K splits of d_X = dU . W_up (K = N*F): enough 256x256 tiles to fill the
  // chip, each split a multiple of 8 of K.
  const int64_t tiles = ((U + 255) / 256) * ((D + 255) / 256);
  p.dx_splits = 1;
  while (p.dx_splits < 16 && tiles * p.dx_splits < 256 && NF % (16 * p.dx_splits) == 0) p.dx_splits *= 2;
  p.wr_chunks = (int)((T + kWrChunk - 1) / kWrChunk);
  // Row-gradient chunks: about 256 of them (a power-of-two size in [4, 64]).
  p.seg = 4;
  while (p.seg < kMaxSeg && (int64_t)p.seg * 256 < T) p.seg *= 2;
  p.nseg = (T + p.seg - 1) / p.seg;
  size_t o = 0;
  p.x_off = o; o += round256((size_t)U * D * 2);
  p.g_off = o; o += round256((size_t)U * NF * 2);
  p.u_off = o; o += round256((size_t)U * NF * 2);
  p.o_off = o; o += round256((size_t)U * N * D * 2);
  p.fwd_total = o;
  o = 0;
  p.gate_off = o; o += round256((size_t)T * N * 4);
  p.dz_off = o; o += round256((size_t)T * N * 4);
  p.do_off = o; o += round256((size_t)U * N * D * 2);
  p.du_off = o; o += round256((size_t)U * NF * 2);
  p.pdx_off = o; o += round256((size_t)p.dx_splits * U * D * 4);
  p.pwr_off = o; o += round256((size_t)std::max<int64_t>(p.wr_chunks, 2 * p.nseg) * N * D * 4);
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
  uint16_t* Upre = reinterpret_cast<uint16_t*>(base + p.u_off);
  uint16_t* O = reinterpret_cast<uint16_t*>(base + p.o_off);
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)U), dim3(256), 0, s, emb, uniq, X, (int)D);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // The build restricted to the batch's rows: G for all U rows in one block,
  // with the pre-activations kept for the backward pass.
  err = launch_build_lut_bf16(X, w_up, w_down, O, U, D, F, N, G, (size_t)U * N * F * 2, s, Upre);
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
  const int64_t NF = N * F;
  const char* fb = static_cast<const char*>(fwd);
  const uint16_t* X = reinterpret_cast<const uint16_t*>(fb + p.x_off);
  const uint16_t* G = reinterpret_cast<const uint16_t*>(fb + p.g_off);
  const uint16_t* Upre = reinterpret_cast<const uint16_t*>(fb + p.u_off);
  const uint16_t* O = reinterpret_cast<const uint16_t*>(fb + p.o_off);
  char* bb = static_cast<char*>(bwd);
  float* gate = reinterpret_cast<float*>(bb + p.gate_off);
  float* dz = reinterpret_cast<float*>(bb + p.dz_off);
  uint16_t* dO = reinterpret_cast<uint16_t*>(bb + p.do_off);
  uint16_t* dU = reinterpret_cast<uint16_t*>(bb + p.du_off);
  float* Pdx = reinterpret_cast<float*>(bb + p.pdx_off);
  float* Pwr = reinterpret_cast<float*>(bb + p.pwr_off);
  const int NP = next_pow2_int((int)N);
  hipError_t err;
#define MOLE_TRY(x) do { err = (x); if (err != hipSuccess) return err; } while (0)

  // Gates: g, dz, d_h.
  // Waves per token: up to 4 while the batch has fewer than 4096 tokens
  // and each wave keeps at least 256 columns.
  int wpt = 1;
  while (wpt < 4 && T * wpt < 4096 && D / (2 * wpt) >= 256) wpt *= 2;
  {
    const dim3 grid((unsigned)((T + 4 / wpt - 1) / (4 / wpt)));
    if (wpt == 4) {
      MOLE_NP_SWITCH(gate_backward_kernel_w4, grid, s, h, w_r, O, remap, dy, gate, dz, d_h, T, (int)D, (int)N);
    } else if (wpt == 2) {
      MOLE_NP_SWITCH(gate_backward_kernel_w2, grid, s, h, w_r, O, remap, dy, gate, dz, d_h, T, (int)D, (int)N);
    } else {
      MOLE_NP_SWITCH(gate_backward_kernel_w1, grid, s, h, w_r, O, remap, dy, gate, dz, d_h, T, (int)D, (int)N);
    }
  }
  MOLE_TRY(hipGetLastError());
  // Router weights: chunked partial sums over tokens, then their sum.
  {
    const int cpl = NP >= 64 ? 1 : (NP >= 32 ? 2 : 4);
    MOLE_NP_SWITCH(wr_partial_kernel, dim3((unsigned)((D + 64 * cpl - 1) / (64 * cpl)), (unsigned)p.wr_chunks), s,
                   (const float*)dz, h, Pwr, T, (int)D, (int)N);
  }
  MOLE_TRY(hipGetLastError());
  if (p.wr_chunks > 16)
    hipLaunchKernelGGL(sum_partials_wide_kernel, dim3((unsigned)((N * D + 255) / 256)), dim3(1024), 0, s,
                       (const float*)Pwr, p.wr_chunks, N * D, d_w_r);
  else
    hipLaunchKernelGGL(sum_partials_kernel, dim3(grid_for(N * D)), dim3(256), 0, s, (const float*)Pwr, p.wr_chunks,
                       N * D, d_w_r);
  MOLE_TRY(hipGetLastError());
  // Gradient of the batch's table rows, dO[u][e] = sum_t g_te dy_t, by
  // chunks of the token list (partials of cut rows in the router-weight
  // partials' region, which is free again), then the cut rows.
  {
    const int cpl = NP >= 64 ? 1 : (NP >= 32 ? 2 : 4);
    const dim3 grid((unsigned)p.nseg, (unsigned)((D + 256 * cpl - 1) / (256 * cpl)));
    MOLE_NP_SWITCH(row_grad_kernel, grid, s, (const float*)gate, dy, remap, row_ptr, tok, dO, Pwr, T, p.seg, (int)D,
                   (int)N);
    MOLE_TRY(hipGetLastError());
    const int64_t gy = std::min<int64_t>((N * D + 1023) / 1024, 32);
    hipLaunchKernelGGL(row_grad_fix_kernel, dim3((unsigned)p.nseg, (unsigned)gy), dim3(256), 0, s,
                       (const float*)Pwr, remap, row_ptr, tok, dO, T, p.seg, N * D);
    MOLE_TRY(hipGetLastError());
  }
  // dU = (dO_e . W_down[e]) * GELU'(u) in one GEMM epilogue (u kept by the
  // forward pass); W_down[e] is [D][F], read MN-major.
  MOLE_TRY(launch_gemm_gelu_grad_bf16(dO, N * D, D, w_down, F, D * F, dU, NF, F, Upre, (int)U, (int)F, (int)D,
                                      (int)N, s));
  // Weight gradients, contracted over the U rows with both operands read
  // MN-major: d_W_down[e] = dO_e^T . G_e, d_W_up[e] = dU_e^T . X.
  MOLE_TRY(launch_gemm_f32_bf16(dO, N * D, D, G, NF, F, d_w_down, F, D * F, (int)D, (int)F, (int)U, (int)N, s,
                                kOpsMnMn));
  MOLE_TRY(launch_gemm_f32_bf16(dU, NF, F, X, D, 0, d_w_up, D, F * D, (int)F, (int)D, (int)U, (int)N, s, kOpsMnMn));
  // Embedding rows: d_X = dU . W_up over K = N*F in equal K splits, W_up
  // ([N*F][D]) read MN-major.
  const int64_t ks = NF / p.dx_splits;
  MOLE_TRY(launch_gemm_f32_bf16(dU, NF, ks, w_up, D, ks * D, Pdx, D, U * D, (int)U, (int)D, (int)ks, p.dx_splits, s,
                                kOpsBmn));
  hipLaunchKernelGGL(sum_partials_kernel, dim3(grid_for(U * D)), dim3(256), 0, s, (const float*)Pdx, p.dx_splits,
                     U * D, d_x);
  return hipGetLastError();
#undef MOLE_TRY
}
#undef MOLE_NP_SWITCH

}  // namespace mole
