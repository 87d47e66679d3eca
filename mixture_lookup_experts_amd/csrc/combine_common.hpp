// Shared pieces of the lookup-combine kernels (dense and NF3 tables): the
// two routers, the group softmax and the host-side launch-shape choices.
#pragma once

#include "mole_device.hpp"
#include "mole_kernels.hpp"

namespace mole {

// ---------------------------------------------------------------------------
// Router: per-lane partial logits over the lane's 16-byte chunks of D.
// ---------------------------------------------------------------------------
template <typename T, int NP, bool VECTOR>
__device__ __forceinline__ void router_partials(const T* __restrict__ h_row, const T* __restrict__ w_r,
                                                int D, int N, int lig, int G, bool valid,
                                                float* part) {
#pragma unroll
  for (int e = 0; e < NP; ++e) part[e] = 0.f;
  if (!valid) return;
  if constexpr (VECTOR) {
    constexpr int V = Elem<T>::kVec;
    const int C = D / V;
    for (int r = lig; r < C; r += G) {
      float hv[V];
      Elem<T>::unpack(ldg16(h_row + (int64_t)r * V), hv);
#pragma unroll
      for (int e = 0; e < NP; ++e) {
        if (e < N) {
          float wv[V];
          Elem<T>::unpack(ldg16(w_r + (int64_t)e * D + (int64_t)r * V), wv);
#pragma unroll
          for (int j = 0; j < V; ++j) part[e] = fmaf(hv[j], wv[j], part[e]);
        }
      }
    }
  } else {
    for (int d = lig; d < D; d += G) {
      const float hv = Elem<T>::load1(h_row, d);
#pragma unroll
      for (int e = 0; e < NP; ++e)
        if (e < N) part[e] = fmaf(hv, Elem<T>::load1(w_r, (int64_t)e * D + d), part[e]);
    }
  }
}


typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMaxTokPerBlock = 16;  // one 16-row MFMA tile of tokens
constexpr int64_t kSimdsPerChip = 1024;  // MI355X: 256 compute units x 4 SIMDs

// Router on the matrix cores for the block's `tpb` (<= 16) tokens starting
// at t0: logits[t][e] = sum_d h[t0+t][d] * w_r[e][d] (bf16 products, fp32
// accumulation), then gates = softmax over e < N into gsh[t][NP].  Lane l
// of a wave supplies token row l%16 (A) and expert column l%16 (B) with the
// 8 consecutive d values of k-group l/16; the waves take every nw-th 32-wide
// K step, in batches of UB steps whose loads are all issued before the
// MFMAs that consume them (one memory round trip per batch).
//
// Two phases, because vector-memory counters retire in issue order: the
// kernel calls load_first() before issuing its table loads, so the router
// waits only for its own operands (not for the table rows queued behind
// them), and finish() after; the table loads stay in flight through the
// router's arithmetic and barriers.  finish() contains barriers: every
// thread of the block must call it.
template <int NP, int UBX = 0>
struct MfmaRouter {
  static constexpr int NT = (NP + 15) / 16, NPAD = NT * 16;
  // K steps per wave and batch of loads (UBX overrides: wide blocks have
  // fewer steps per wave)
  static constexpr int UB = UBX > 0 ? UBX : (NT == 1 ? 8 : (NT == 2 ? 4 : 2));
  uint4 a[UB], b[UB][NT];
  f32x4_t acc[NT];
  // Operands through buffer resources: h over the rows of the block's
  // tokens inside the batch, W_r over its N rows.  A lane's h offset is
  // kOob for a token row outside the tile or the batch (and for a K step
  // past the row), so its operand reads as zero without a select; W_r
  // columns of experts >= N read the clamped row N - 1, whose logits the
  // softmax ignores.
  __amdgpu_buffer_rsrc_t rh, rw;
  uint32_t hoff, woff[NT];
  int D, ksteps, nw, wave, kg;

  // Every load is issued unconditionally: loads under a divergent branch
  // would leave the compiler unsure how many loads are outstanding at the
  // join, and a select right after a load would make it wait there --
  // either way it would wait for the table rows issued after the router's
  // operands.
  __device__ __forceinline__ void load(int base) {
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int ks = base + u * nw;
      const uint32_t kb = (uint32_t)(ks * 32 + kg * 8) * 2u;  // byte offset in a row
      const bool kok = ks < ksteps && ks * 32 + kg * 8 < D;
      a[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rh, (int)(kok ? hoff + kb : kOob), 0, 0));
      // (past the row, A is zero: any finite W_r value will do, and the
      // offset stays inside the resource or reads zero)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        b[u][nt] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(woff[nt] + (kok ? kb : 0u)), 0, 0));
    }
  }
  __device__ __forceinline__ void mma(int) {
#pragma unroll
    for (int u = 0; u < UB; ++u)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[u]),
                                                          __builtin_bit_cast(bf16x8_t, b[u][nt]), acc[nt], 0, 0, 0);
  }
  // nwaves = the block's wavefronts (passed in: reading the block size
  // costs a dependent load of the dispatch packet).
  __device__ __forceinline__ void load_first(const uint16_t* __restrict__ h, const uint16_t* __restrict__ w,
                                             int64_t t0, int64_t T_, int tpb, int D_, int N_, int nwaves) {
    const int lane = threadIdx.x & 63, row = lane & 15;
    wave = threadIdx.x >> 6;
    nw = nwaves;
    kg = lane >> 4;
    D = D_;
    ksteps = (D + 31) / 32;
    const int64_t left = T_ - t0;
    const int rows = (int)(left < tpb ? left : tpb);  // token rows of the tile inside the batch (>= 1)
    rh = __builtin_amdgcn_make_buffer_rsrc((void*)(h + t0 * D), (short)0, rows * D * 2, kRsrcWord3);
    rw = __builtin_amdgcn_make_buffer_rsrc((void*)w, (short)0, N_ * D * 2, kRsrcWord3);
    hoff = row < rows ? (uint32_t)(row * D) * 2u : kOob;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int e = nt * 16 + row;
      woff[nt] = (uint32_t)((e < N_ ? e : N_ - 1) * D) * 2u;
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    load(wave);
  }
  // The matrix work alone (consumes the operand registers of load_first).
  __device__ __forceinline__ void compute() {
    mma(wave);
    for (int base = wave + UB * nw; base < ksteps; base += UB * nw) {
      load(base);
      mma(base);
    }
  }
  // The same when one batch covers the row (ceil(D / 32) <= UB * nwaves,
  // checked by the caller's host code): no second batch of loads, so no
  // second set of operand registers.
  __device__ __forceinline__ void compute_one_batch() { mma(wave); }

  __device__ __forceinline__ void finish(int tpb, int N, float* red /* [nw][16][NPAD] */, float* gsh /* [16][NP] */) {
    compute();
    if constexpr (NP <= 16) {
      if (nw * kWave >= 16 * NP) {
        reduce_wide(tpb, N, red, gsh);
        return;
      }
    }
    // lane l holds logits of tokens 4*(l/16) + r, expert nt*16 + l%16
    const int row = threadIdx.x & 15;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[(wave * 16 + 4 * kg + r) * NPAD + nt * 16 + row] = acc[nt][r];
    __syncthreads();
    if ((int)threadIdx.x < tpb) {
      const int tk = threadIdx.x;
      float z[NP];
      float zmax = -INFINITY;
#pragma unroll
      for (int e = 0; e < NP; ++e) {
        float s = 0.f;
        for (int w = 0; w < nw; ++w) s += red[(w * 16 + tk) * NPAD + e];
        z[e] = s;
        if (e < N) zmax = fmaxf(zmax, s);
      }
      float sum = 0.f;
#pragma unroll
      for (int e = 0; e < NP; ++e) {
        z[e] = (e < N) ? expf(z[e] - zmax) : 0.f;
        sum += z[e];
      }
      const float inv = 1.f / sum;
#pragma unroll
      for (int e = 0; e < NP; ++e) gsh[tk * NP + e] = z[e] * inv;
    }
    __syncthreads();
  }
  // Softmax with one thread per (token, expert): thread i < 16 NP sums the
  // partial logits of token i / NP, expert i % NP over the waves, and each
  // token's NP threads (consecutive lanes of one wavefront) form its softmax
  // with shuffles.  Needs NP <= 16 and at least 16 NP threads in the block.
  __device__ __forceinline__ void reduce_wide(int tpb, int N, float* red, float* gsh) {
    static_assert(NP <= 16, "one 16-column tile");
    const int row = threadIdx.x & 15;
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(wave * 16 + 4 * kg + r) * NPAD + row] = acc[0][r];
    __syncthreads();
    const int i = threadIdx.x;
    if (i < 16 * NP) {
      const int tk = i / NP, e = i % NP;
      float z = 0.f;
      for (int w = 0; w < nw; ++w) z += red[(w * 16 + tk) * NPAD + e];
      float m = e < N ? z : -INFINITY;
#pragma unroll
      for (int o = 1; o < NP; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
      const float p = e < N ? expf(z - m) : 0.f;
      float sum = p;
#pragma unroll
      for (int o = 1; o < NP; o <<= 1) sum += __shfl_xor(sum, o, kWave);
      if (tk < tpb) gsh[tk * NP + e] = p * (1.f / sum);
    }
    __syncthreads();
  }
};

// Reduce the partial logits of a token group and turn them into softmax
// gates held (identically) by every lane of the group.  Must be reached by
// every thread of the block (it contains a barrier).
template <int NP, int G>
__device__ __forceinline__ void group_gates(float* part, float* gate, int N, int lig,
                                            float* red /* [WG][NP] of this group */) {
  constexpr int W = G < kWave ? G : kWave;
  constexpr int WG = G > kWave ? G / kWave : 1;
  using RS = ReduceScatter<NP, W>;
  const int lane_w = lig % W, wig = lig / W;
  RS::run(part, lane_w);
  constexpr int kWriters = NP < W ? NP : W;
  if (lane_w < kWriters) {
    const int off = RS::offset(lane_w);
#pragma unroll
    for (int i = 0; i < RS::kLeft; ++i) red[wig * NP + off + i] = part[i];
  }
  __syncthreads();
  float zmax = -INFINITY;
#pragma unroll
  for (int e = 0; e < NP; ++e) {
    float z = 0.f;
#pragma unroll
    for (int w = 0; w < WG; ++w) z += red[w * NP + e];
    gate[e] = z;
    if (e < N) zmax = fmaxf(zmax, z);
  }
  float sum = 0.f;
#pragma unroll
  for (int e = 0; e < NP; ++e) {
    const float p = (e < N) ? expf(gate[e] - zmax) : 0.f;
    gate[e] = p;
    sum += p;
  }
  const float inv = 1.f / sum;
#pragma unroll
  for (int e = 0; e < NP; ++e) gate[e] *= inv;
}

// Router on the vector units for one token per lane group (used where a
// block holds a single token, so a 16-row MFMA tile would be 1/16 full and
// would need a second round of loads at large D): lane l of the group owns
// chunk l (and l + G, ...) of h and of every expert row of W_r, forms the
// per-expert partial dot products, and the group reduces them
// (group_gates).  Two phases as in MfmaRouter, so its operand loads go out
// before the table loads: load_first() loads the lane's first chunk from
// clamped (in-bounds) addresses, finish() consumes it, walks any further
// chunks and forms the gates.  finish() contains a barrier: every thread of
// the block must call it.
template <typename T, int NP>
struct LaneRouter {
  static constexpr int V = Elem<T>::kVec;
  uint4 hv, wv[NP];
  __device__ __forceinline__ void load_first(const T* __restrict__ h_row, const T* __restrict__ w_r, int D,
                                             int N, int lig) {
    const int C = D / V;
    const int c = lig < C ? lig : C - 1;
    hv = ldg16(h_row + (int64_t)c * V);
#pragma unroll
    for (int e = 0; e < NP; ++e) wv[e] = ldg16(w_r + (int64_t)(e < N ? e : N - 1) * D + (int64_t)c * V);
  }
  template <int G>
  __device__ __forceinline__ void finish(const T* __restrict__ h_row, const T* __restrict__ w_r, int D, int N,
                                         int lig, bool valid, float* gate, float* red /* [WG][NP] */) {
    float part[NP];
    partials<G>(h_row, w_r, D, N, lig, valid, part);
    group_gates<NP, G>(part, gate, N, lig, red);
  }
  // The lane's partial logits (consumes the registers of load_first, so a
  // caller can issue more loads between this and group_gates).
  template <int G>
  __device__ __forceinline__ void partials(const T* __restrict__ h_row, const T* __restrict__ w_r, int D, int N,
                                           int lig, bool valid, float* part) {
    // The first chunk is consumed unconditionally and masked by a multiply
    // (a select or a branch would let the compiler sink the loads into the
    // branch below).  Masked lanes read finite in-bounds data of their own
    // token (or of token 0 for a token past the batch, whose gates are
    // unused), so the multiply by zero is exact.
    const int C = D / V;
    const bool ok = valid && lig < C;
    const float okf = ok ? 1.f : 0.f;
    {
      float hf[V];
      Elem<T>::unpack(hv, hf);
#pragma unroll
      for (int e = 0; e < NP; ++e) {
        float wf[V];
        Elem<T>::unpack(wv[e], wf);
        float d = 0.f;
#pragma unroll
        for (int j = 0; j < V; ++j) d = fmaf(hf[j], wf[j], d);
        part[e] = d * (e < N ? okf : 0.f);
      }
    }
    if (ok) {
      float hf[V];
      for (int r = lig + G; r < C; r += G) {  // rows wider than G chunks
        Elem<T>::unpack(ldg16(h_row + (int64_t)r * V), hf);
#pragma unroll
        for (int e = 0; e < NP; ++e) {
          if (e < N) {
            float wf[V];
            Elem<T>::unpack(ldg16(w_r + (int64_t)e * D + (int64_t)r * V), wf);
#pragma unroll
            for (int j = 0; j < V; ++j) part[e] = fmaf(hf[j], wf[j], part[e]);
          }
        }
      }
    }
  }
};

// Router placement of a combine launch: fused on the matrix cores, fused
// on the vector units, or staged -- gates computed by router_gates_kernel
// beforehand and left in the first N floats of each token's output row.
enum { kRouterMfma = 0, kRouterLane = 1, kRouterStaged = 2 };

// Gates for the staged-router mode: 16 tokens per block on the matrix cores
// (a full MFMA tile, so W_r is read once per 16 tokens), written to the
// first N floats of each token's output row, which the combine kernel reads
// before it overwrites the row.
template <int NP>
__global__ __launch_bounds__(256) void router_gates_kernel(const uint16_t* __restrict__ h,
                                                           const uint16_t* __restrict__ w_r, float* __restrict__ y,
                                                           int64_t T_, int D, int N) {
  constexpr int NPAD = ((NP + 15) / 16) * 16;
  __shared__ float red[4 * 16 * NPAD];
  __shared__ float gsh[kMaxTokPerBlock * NP];
  const int64_t t0 = (int64_t)blockIdx.x * kMaxTokPerBlock;
  MfmaRouter<NP> rt;
  rt.load_first(h, w_r, t0, T_, kMaxTokPerBlock, D, N, 4);
  rt.finish(kMaxTokPerBlock, N, red, gsh);
  for (int i = threadIdx.x; i < kMaxTokPerBlock * N; i += blockDim.x) {
    const int tk = i / N, e = i - tk * N;
    if (t0 + tk < T_) y[(t0 + tk) * D + e] = gsh[tk * NP + e];
  }
}

// Batches of at least this many tokens, at widths where a block holds
// several tokens (below 128 lanes per token; wider tokens use the dense
// kernel's four-token wide blocks instead), route in a separate launch (see
// router_gates_kernel): the fused MFMA router of a 256-thread block re-reads
// W_r for every 2-4 tokens and holds its operands in registers through the
// gather, which at these sizes cost more than the second launch (measured
// on the 410M-class table before the wide blocks: T=4096 26.6 -> 21.0 us
// with Zipf ids, neutral at T=1024).
constexpr int64_t kStagedRouterMinT = 2048;

// ---------------------------------------------------------------------------
// Host-side dispatch
// ---------------------------------------------------------------------------
static inline int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Lanes per token: the smallest power of two in [lo, hi] covering the C
// chunks of a row (so each lane streams one chunk per expert row when it can).
static inline int pick_group(int C, int lo, int hi) {
  int G = lo;
  while (G < C && G < hi) G <<= 1;
  return G;
}

// Tokens per block: up to 16 (one MFMA tile of router rows) and at most 256
// threads, halved while the grid would have fewer than two blocks per
// compute unit -- small decode batches then spread over the whole chip --
// but never below one full wavefront per block.
static inline int pick_tokens_per_block(int64_t T, int G) {
  int tpb = 256 / G < 16 ? 256 / G : 16;
  const int min_tpb = G >= 64 ? 1 : 64 / G;
  while (tpb > min_tpb && (T + tpb - 1) / tpb < 512) tpb >>= 1;
  return tpb;
}

}  // namespace mole
