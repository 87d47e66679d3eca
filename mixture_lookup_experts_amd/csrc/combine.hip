// Lookup-combine kernels: router softmax + gather of each token's N x D
// table slab + gate-weighted sum, for a bf16/fp32 table and for the 3-bit
// NF3 table.  (MoLE article, inference section: retrieve each token's
// expert outputs by token id; training section: the router reads the
// contextual hidden state and all routed experts are active.)
//
// Work decomposition (one launch, no inter-block communication):
//   * a "group" of G lanes (G a power of two) owns one token; a block holds
//     up to 16 tokens, fewer when the batch is small so that the grid still
//     covers the 256 compute units;
//   * router, bf16: the block's logits [tokens x experts] come from
//     v_mfma_f32_16x16x32_bf16 tiles (tokens x 16 experts, K = 32 per
//     instruction), the waves splitting D, so W_r is read once per block;
//     partial tiles meet in LDS and one thread per token does the
//     max-subtracted softmax;
//   * router, fp32 or unaligned: lanes split D into chunks, form per-expert
//     partial dot products, reduce them across the group with a wavefront
//     reduce-scatter (xor shuffles) plus one LDS exchange;
//   * gather/combine: lane `l` of the group streams chunks l, l+G, ... of
//     every expert row of the token's contiguous slab LUT[id] with 16-byte
//     loads and accumulates in fp32.  The router's operands are loaded
//     first and the first batch of slab loads right after, so the router
//     waits only for its own operands and the slab arrives during the
//     router's arithmetic.
#include "mole_device.hpp"
#include "mole_kernels.hpp"

namespace mole {

// NF3 reconstruction levels: the NormalFloat construction at 3 bits (levels
// Phi^-1 of evenly spaced probabilities, 4 positive, 3 negative, an exact
// zero, normalised to [-1, 1]), rounded to fp32.  Bit patterns:
__constant__ uint32_t kNf3LevelBits[8] = {0xbf800000u, 0xbf08f740u, 0xbe7cdb98u, 0x00000000u,
                                          0x3e3bbcd2u, 0x3ec394b6u, 0x3f1f7bfeu, 0x3f800000u};

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
template <int NP>
struct MfmaRouter {
  static constexpr int NT = (NP + 15) / 16, NPAD = NT * 16;
  static constexpr int UB = NT == 1 ? 8 : (NT == 2 ? 4 : 2);
  uint4 a[UB], b[UB][NT];
  f32x4_t acc[NT];
  const uint16_t* hrow;
  const uint16_t* w_r;
  int D, N, ksteps, nw, wave, row, kg;
  bool tok_ok;

  // Every load is issued unconditionally from an in-bounds (clamped)
  // address and masked to zero only where it is consumed (mma, which
  // recomputes the masks): loads under a divergent branch would leave the
  // compiler unsure how many loads are outstanding at the join, and a select
  // right after a load would make it wait there -- either way it would wait
  // for the table rows issued after the router's operands.
  __device__ __forceinline__ bool k_ok(int base, int u) const {
    const int ks = base + u * nw;
    return ks < ksteps && ks * 32 + kg * 8 < D;
  }
  __device__ __forceinline__ void load(int base) {
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int kc = k_ok(base, u) ? (base + u * nw) * 32 + kg * 8 : 0;
      a[u] = ldg16(hrow + kc);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int e = nt * 16 + row;
        b[u][nt] = ldg16(w_r + (int64_t)(e < N ? e : N - 1) * D + kc);
      }
    }
  }
  __device__ __forceinline__ void mma(int base) {
    const uint4 zero = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const bool kok = k_ok(base, u);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8_t, (tok_ok && kok) ? a[u] : zero),
            __builtin_bit_cast(bf16x8_t, (nt * 16 + row < N && kok) ? b[u][nt] : zero), acc[nt], 0, 0, 0);
    }
  }
  __device__ __forceinline__ void load_first(const uint16_t* __restrict__ h, const uint16_t* __restrict__ w,
                                             int64_t t0, int64_t T_, int tpb, int D_, int N_) {
    lane_setup(h, w, t0, T_, tpb, D_, N_);
    load(wave);
  }
  __device__ __forceinline__ void lane_setup(const uint16_t* __restrict__ h, const uint16_t* __restrict__ w,
                                             int64_t t0, int64_t T_, int tpb, int D_, int N_) {
    const int lane = threadIdx.x & 63;
    wave = threadIdx.x >> 6;
    nw = blockDim.x >> 6;
    row = lane & 15;
    kg = lane >> 4;
    D = D_;
    N = N_;
    w_r = w;
    const int64_t tok = t0 + row;
    tok_ok = row < tpb && tok < T_;
    hrow = h + (tok_ok ? tok : 0) * (int64_t)D;
    ksteps = (D + 31) / 32;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  __device__ __forceinline__ void finish(int tpb, float* red /* [4][16][NPAD] */, float* gsh /* [16][NP] */) {
    mma(wave);
    for (int base = wave + UB * nw; base < ksteps; base += UB * nw) {
      load(base);
      mma(base);
    }
    // lane l holds logits of tokens 4*(l/16) + r, expert nt*16 + l%16
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

// ---------------------------------------------------------------------------
// bf16 / fp32 table
// ---------------------------------------------------------------------------
template <typename T, int NP, int G, bool VECTOR>
__global__ __launch_bounds__(256) void lookup_combine_kernel(
    const int64_t* __restrict__ ids, const T* __restrict__ h, const T* __restrict__ w_r,
    const T* __restrict__ lut, float* __restrict__ y, int64_t T_, int D, int N) {
  constexpr int WG = G > kWave ? G / kWave : 1;
  constexpr int MAXTPB = 256 / G < kMaxTokPerBlock ? 256 / G : kMaxTokPerBlock;
  constexpr int CH = VECTOR ? Elem<T>::kVec : 1;  // elements per chunk
  constexpr int EC = NP < 16 ? NP : 16;           // experts per batch of slab loads
  constexpr bool kMfmaRouter = VECTOR && sizeof(T) == 2;
  constexpr int NPAD = ((NP + 15) / 16) * 16;
  __shared__ float red[kMfmaRouter ? 4 * 16 * NPAD : MAXTPB * WG * NP];
  __shared__ float gsh[kMfmaRouter ? kMaxTokPerBlock * NP : 1];

  const int tid = threadIdx.x;
  const int tpb = blockDim.x / G;
  const int grp = tid / G, lig = tid % G;
  const int64_t t0 = (int64_t)blockIdx.x * tpb;
  const int64_t t = t0 + grp;
  const bool valid = t < T_;
  const int64_t tt = valid ? t : 0;
  const int C = D / CH;
  const int64_t id_ld = ids[tt];  // unconditional (tt is clamped): see MfmaRouter::load
  __builtin_amdgcn_sched_barrier(0);  // the id load goes out first: the table address waits on it alone
  const int64_t id = valid ? id_ld : 0;
  const T* slab = lut + id * (int64_t)N * D;

  // Router operands first, then the first batch of slab loads (chunk lig,
  // experts 0..EC-1); the router's arithmetic runs while the slab arrives.
  MfmaRouter<NP> rt;
  if constexpr (kMfmaRouter)
    rt.load_first(reinterpret_cast<const uint16_t*>(h), reinterpret_cast<const uint16_t*>(w_r), t0, T_, tpb, D,
                  N);
  __builtin_amdgcn_sched_barrier(0);
  // (Unconditional loads from clamped chunk and expert indices; lanes past
  // the row and experts past N read data they then ignore.)
  uint4 sv[EC];
  float sf[EC];
  {
    const int c0 = lig < C ? lig : C - 1;
#pragma unroll
    for (int e = 0; e < EC; ++e) {
      const int ec = e < N ? e : N - 1;
      if constexpr (VECTOR) sv[e] = ldg16(slab + (int64_t)ec * D + (int64_t)c0 * CH);
      else sf[e] = Elem<T>::load1(slab, (int64_t)ec * D + c0);
    }
  }

  __builtin_amdgcn_sched_barrier(0);

  float gate[NP];
  if constexpr (kMfmaRouter) {
    rt.finish(tpb, red, gsh);
#pragma unroll
    for (int e = 0; e < NP; ++e) gate[e] = gsh[grp * NP + e];
  } else {
    float part[NP];
    router_partials<T, NP, VECTOR>(h + tt * D, w_r, D, N, lig, G, valid, part);
    group_gates<NP, G>(part, gate, N, lig, red + grp * WG * NP);
  }
  if (!valid) return;

  for (int k = 0; k * G + lig < C; ++k) {
    const int c = k * G + lig;
    float acc[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) acc[j] = 0.f;
#pragma unroll
    for (int e0 = 0; e0 < NP; e0 += EC) {
      if (k != 0 || e0 != 0) {
#pragma unroll
        for (int e = 0; e < EC; ++e) {
          if (e0 + e < N) {
            if constexpr (VECTOR) sv[e] = ldg16(slab + (int64_t)(e0 + e) * D + (int64_t)c * CH);
            else sf[e] = Elem<T>::load1(slab, (int64_t)(e0 + e) * D + c);
          }
        }
      }
#pragma unroll
      for (int e = 0; e < EC; ++e) {
        if (e0 + e < N) {
          const float g = gate[e0 + e];
          if constexpr (VECTOR) {
            float v[CH];
            Elem<T>::unpack(sv[e], v);
#pragma unroll
            for (int j = 0; j < CH; ++j) acc[j] = fmaf(g, v[j], acc[j]);
          } else {
            acc[0] = fmaf(g, sf[e], acc[0]);
          }
        }
      }
    }
    float* yo = y + tt * D + (int64_t)c * CH;
    if constexpr (VECTOR) {
#pragma unroll
      for (int j = 0; j < CH; j += 4)
        stg16_nt(yo + j, acc[j], acc[j + 1], acc[j + 2], acc[j + 3]);
    } else {
      __builtin_nontemporal_store(acc[0], yo);
    }
  }
}

// ---------------------------------------------------------------------------
// NF3 table: 32 codes (12 bytes) per chunk, one fp16 scale per 64 elements.
// A token is owned by G = CP*S lanes: lane (s, c) = s*CP + c decodes chunk c
// (and c + CP, ... when a row has more than CP chunks) for the experts
// e = s, s + S, s + 2S, ...; the S partial sums of a chunk then meet in a
// reduce-scatter over the lanes c, c + CP, ..., so each lane stores 32/S of
// the chunk's outputs.  Splitting the experts across lanes keeps a full
// wavefront busy per token at the 160M/410M widths (24-32 chunks per row)
// and lets every lane issue all of its code loads in one batch.
// ---------------------------------------------------------------------------

// Halving reduce-scatter of the 32 per-lane sums over the S expert splits:
// at step b (xor mask CP << b) a lane keeps the half its split bit b
// selects and adds the partner's copy of it.  Afterwards the lane holds the
// 32/S sums of elements off(s) .. off(s) + 32/S - 1 of its chunk.
template <int CP, int S, int B = 0, int CNT = 32>
struct SplitReduce {
  __device__ __forceinline__ static void run(float* acc, int sp) {
    if constexpr ((1 << B) < S) {
      constexpr int H = CNT / 2;
      const bool hi = ((sp >> B) & 1) != 0;
#pragma unroll
      for (int i = 0; i < H; ++i) {
        const float keep = hi ? acc[i + H] : acc[i];
        const float send = hi ? acc[i] : acc[i + H];
        acc[i] = keep + __shfl_xor(send, CP << B, kWave);
      }
      SplitReduce<CP, S, B + 1, H>::run(acc, sp);
    }
  }
  __device__ __forceinline__ static int offset(int sp) {
    int off = 0;
#pragma unroll
    for (int b = 0; (1 << b) < S; ++b)
      if ((sp >> b) & 1) off += 16 >> b;
    return off;
  }
};

template <typename TH, int NP, int CP, int S>
__global__ __launch_bounds__(256) void lookup_combine_nf3_kernel(
    const int64_t* __restrict__ ids, const TH* __restrict__ h, const TH* __restrict__ w_r,
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    float* __restrict__ y, int64_t T_, int D, int N) {
  constexpr int G = CP * S;                        // lanes per token (<= 64)
  static_assert(G <= kWave, "a token's lanes must share one wavefront");
  constexpr int MAXTPB = 256 / G < kMaxTokPerBlock ? 256 / G : kMaxTokPerBlock;
  constexpr int EPL = (NP + S - 1) / S;            // experts per lane
  constexpr int EC = EPL < 8 ? EPL : 8;            // experts per batch of code loads
  constexpr int OUT = 32 / S;                      // outputs stored per lane and chunk
  constexpr bool kMfmaRouter = sizeof(TH) == 2;
  constexpr int NPAD = ((NP + 15) / 16) * 16;
  __shared__ float red[kMfmaRouter ? 4 * 16 * NPAD : MAXTPB * NP];
  __shared__ float gsh[kMaxTokPerBlock * NP];
  __shared__ float lv[8];

  const int tid = threadIdx.x;
  if (tid < 8) lv[tid] = __uint_as_float(kNf3LevelBits[tid]);
  const int tpb = blockDim.x / G;
  const int grp = tid / G, lig = tid % G;
  const int sp = lig / CP, ch = lig % CP;          // expert split, chunk
  const int64_t t0 = (int64_t)blockIdx.x * tpb;
  const int64_t t = t0 + grp;
  const bool valid = t < T_;
  const int64_t tt = valid ? t : 0;
  const int C = D / 32;                            // 32-element chunks per row
  const int64_t row_bytes = 3 * (int64_t)D / 8, nblk = D / 64;
  const int64_t id = valid ? ids[tt] : 0;
  const uint8_t* crow0 = codes + id * (int64_t)N * row_bytes;
  const uint16_t* srow0 = scales + id * (int64_t)N * nblk;

  uint3 cw[EC];
  uint32_t sc[EC];
  auto load_batch = [&](int c, int j0) {
#pragma unroll
    for (int j = 0; j < EC; ++j) {
      const int e = (j0 + j) * S + sp;
      if (e < N) {
        cw[j] = *reinterpret_cast<const uint3*>(crow0 + (int64_t)e * row_bytes + (int64_t)c * 12);
        sc[j] = srow0[(int64_t)e * nblk + (c >> 1)];
      }
    }
  };
  // First batch of code loads, then the router's operands.  (The reverse
  // order, as in the dense kernel, needs branch-free code loads, which cost
  // this kernel about 25 registers and one wave per SIMD of occupancy, more
  // than the overlap gains: a token's codes are only N*(3D/8 + D/32) bytes.)
  if (valid && ch < C) load_batch(ch, 0);
  MfmaRouter<NP> rt;
  if constexpr (kMfmaRouter)
    rt.load_first(reinterpret_cast<const uint16_t*>(h), reinterpret_cast<const uint16_t*>(w_r), t0, T_, tpb, D,
                  N);

  // Gates of the block's tokens into gsh[token][expert].
  if constexpr (kMfmaRouter) {
    rt.finish(tpb, red, gsh);
  } else {
    float part[NP];
    router_partials<TH, NP, true>(h + tt * D, w_r, D, N, lig, G, valid, part);
    float gate[NP];
    group_gates<NP, G>(part, gate, N, lig, red + grp * NP);
    if (lig == 0) {
#pragma unroll
      for (int e = 0; e < NP; ++e) gsh[grp * NP + e] = gate[e];
    }
    __syncthreads();
  }
  if (!valid) return;

  for (int k = 0; k * CP + ch < C; ++k) {
    const int c = k * CP + ch;
    float acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j0 = 0; j0 < EPL; j0 += EC) {
      if (k != 0 || j0 != 0) load_batch(c, j0);
#pragma unroll
      for (int j = 0; j < EC; ++j) {
        const int e = (j0 + j) * S + sp;
        if (e < N) {
          const float sv = (float)__builtin_bit_cast(_Float16, (uint16_t)sc[j]);
          const float ws = gsh[grp * NP + e] * sv;
          const uint32_t w[3] = {cw[j].x, cw[j].y, cw[j].z};
#pragma unroll
          for (int i = 0; i < 32; ++i) {
            const int pos = 3 * i, wd = pos >> 5, off = pos & 31;
            uint32_t code;
            if (off <= 29) code = (w[wd] >> off) & 7u;
            else code = __builtin_amdgcn_alignbit(w[wd + 1], w[wd], off) & 7u;
            acc[i] = fmaf(ws, lv[code], acc[i]);
          }
        }
      }
    }
    SplitReduce<CP, S>::run(acc, sp);
    float* yo = y + tt * D + (int64_t)c * 32 + SplitReduce<CP, S>::offset(sp);
    if constexpr (OUT >= 4) {
#pragma unroll
      for (int j = 0; j < OUT; j += 4) stg16_nt(yo + j, acc[j], acc[j + 1], acc[j + 2], acc[j + 3]);
    } else {
#pragma unroll
      for (int j = 0; j < OUT; ++j) __builtin_nontemporal_store(acc[j], yo + j);
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side dispatch
// ---------------------------------------------------------------------------
static int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Lanes per token: the smallest power of two in [lo, hi] covering the C
// chunks of a row (so each lane streams one chunk per expert row when it can).
static int pick_group(int C, int lo, int hi) {
  int G = lo;
  while (G < C && G < hi) G <<= 1;
  return G;
}

// Tokens per block: up to 16 (one MFMA tile of router rows) and at most 256
// threads, halved while the grid would have fewer than two blocks per
// compute unit -- small decode batches then spread over the whole chip --
// but never below one full wavefront per block.
static int pick_tokens_per_block(int64_t T, int G) {
  int tpb = 256 / G < 16 ? 256 / G : 16;
  const int min_tpb = G >= 64 ? 1 : 64 / G;
  while (tpb > min_tpb && (T + tpb - 1) / tpb < 512) tpb >>= 1;
  return tpb;
}

template <typename E, int NP, int G, bool VEC>
static hipError_t launch_dense(const int64_t* ids, const void* h, const void* w_r, const void* lut,
                               float* y, int64_t T, int D, int N, hipStream_t s) {
  const int tpb = pick_tokens_per_block(T, G);
  const int64_t blocks = (T + tpb - 1) / tpb;
  hipLaunchKernelGGL((lookup_combine_kernel<E, NP, G, VEC>), dim3((unsigned)blocks), dim3(G * tpb), 0, s,
                     ids, (const E*)h, (const E*)w_r, (const E*)lut, y, T, D, N);
  return hipGetLastError();
}

template <typename E, int NP, bool VEC>
static hipError_t dispatch_dense_g(int G, const int64_t* ids, const void* h, const void* w_r,
                                   const void* lut, float* y, int64_t T, int D, int N, hipStream_t s) {
  switch (G) {
    case 16: return launch_dense<E, NP, 16, VEC>(ids, h, w_r, lut, y, T, D, N, s);
    case 32: return launch_dense<E, NP, 32, VEC>(ids, h, w_r, lut, y, T, D, N, s);
    case 64: return launch_dense<E, NP, 64, VEC>(ids, h, w_r, lut, y, T, D, N, s);
    case 128: return launch_dense<E, NP, 128, VEC>(ids, h, w_r, lut, y, T, D, N, s);
    default: return launch_dense<E, NP, 256, VEC>(ids, h, w_r, lut, y, T, D, N, s);
  }
}

template <typename E, bool VEC>
static hipError_t dispatch_dense_np(int NP, int G, const int64_t* ids, const void* h, const void* w_r,
                                    const void* lut, float* y, int64_t T, int D, int N, hipStream_t s) {
  switch (NP) {
    case 1: return dispatch_dense_g<E, 1, VEC>(G, ids, h, w_r, lut, y, T, D, N, s);
    case 2: return dispatch_dense_g<E, 2, VEC>(G, ids, h, w_r, lut, y, T, D, N, s);
    case 4: return dispatch_dense_g<E, 4, VEC>(G, ids, h, w_r, lut, y, T, D, N, s);
    case 8: return dispatch_dense_g<E, 8, VEC>(G, ids, h, w_r, lut, y, T, D, N, s);
    case 16: return dispatch_dense_g<E, 16, VEC>(G, ids, h, w_r, lut, y, T, D, N, s);
    case 32: return dispatch_dense_g<E, 32, VEC>(G, ids, h, w_r, lut, y, T, D, N, s);
    default: return dispatch_dense_g<E, 64, VEC>(G, ids, h, w_r, lut, y, T, D, N, s);
  }
}

hipError_t launch_lookup_combine(const int64_t* ids, const void* h, const void* w_r, const void* lut,
                                 float* y, int64_t T, int64_t D, int64_t N, int dtype, bool vector_ok,
                                 hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int NP = next_pow2((int)N);
  const int elem_bytes = dtype == kF32 ? 4 : 2;
  const int vec = 16 / elem_bytes;
  const bool vector = vector_ok && (D % vec == 0);
  const int C = vector ? (int)(D / vec) : (int)D;
  const int G = pick_group(C, 16, 256);
  if (dtype == kF32)
    return vector ? dispatch_dense_np<float, true>(NP, G, ids, h, w_r, lut, y, T, (int)D, (int)N, s)
                  : dispatch_dense_np<float, false>(NP, G, ids, h, w_r, lut, y, T, (int)D, (int)N, s);
  return vector ? dispatch_dense_np<uint16_t, true>(NP, G, ids, h, w_r, lut, y, T, (int)D, (int)N, s)
                : dispatch_dense_np<uint16_t, false>(NP, G, ids, h, w_r, lut, y, T, (int)D, (int)N, s);
}

template <typename TH, int NP, int CP>
static hipError_t launch_nf3(const int64_t* ids, const void* h, const void* w_r, const uint8_t* codes,
                             const uint16_t* scales, float* y, int64_t T, int D, int N, hipStream_t s) {
  constexpr int S = 64 / CP < NP ? 64 / CP : NP;  // expert splits per token
  constexpr int G = CP * S;
  const int tpb = pick_tokens_per_block(T, G);
  const int64_t blocks = (T + tpb - 1) / tpb;
  hipLaunchKernelGGL((lookup_combine_nf3_kernel<TH, NP, CP, S>), dim3((unsigned)blocks), dim3(G * tpb), 0,
                     s, ids, (const TH*)h, (const TH*)w_r, codes, scales, y, T, D, N);
  return hipGetLastError();
}

template <typename TH, int NP>
static hipError_t dispatch_nf3_cp(int CP, const int64_t* ids, const void* h, const void* w_r,
                                  const uint8_t* codes, const uint16_t* scales, float* y, int64_t T,
                                  int D, int N, hipStream_t s) {
  switch (CP) {
    case 8: return launch_nf3<TH, NP, 8>(ids, h, w_r, codes, scales, y, T, D, N, s);
    case 16: return launch_nf3<TH, NP, 16>(ids, h, w_r, codes, scales, y, T, D, N, s);
    case 32: return launch_nf3<TH, NP, 32>(ids, h, w_r, codes, scales, y, T, D, N, s);
    default: return launch_nf3<TH, NP, 64>(ids, h, w_r, codes, scales, y, T, D, N, s);
  }
}

template <typename TH>
static hipError_t dispatch_nf3_np(int NP, int CP, const int64_t* ids, const void* h, const void* w_r,
                                  const uint8_t* codes, const uint16_t* scales, float* y, int64_t T,
                                  int D, int N, hipStream_t s) {
  switch (NP) {
    case 1: return dispatch_nf3_cp<TH, 1>(CP, ids, h, w_r, codes, scales, y, T, D, N, s);
    case 2: return dispatch_nf3_cp<TH, 2>(CP, ids, h, w_r, codes, scales, y, T, D, N, s);
    case 4: return dispatch_nf3_cp<TH, 4>(CP, ids, h, w_r, codes, scales, y, T, D, N, s);
    case 8: return dispatch_nf3_cp<TH, 8>(CP, ids, h, w_r, codes, scales, y, T, D, N, s);
    case 16: return dispatch_nf3_cp<TH, 16>(CP, ids, h, w_r, codes, scales, y, T, D, N, s);
    case 32: return dispatch_nf3_cp<TH, 32>(CP, ids, h, w_r, codes, scales, y, T, D, N, s);
    default: return dispatch_nf3_cp<TH, 64>(CP, ids, h, w_r, codes, scales, y, T, D, N, s);
  }
}

hipError_t launch_lookup_combine_nf3(const int64_t* ids, const void* h, const void* w_r,
                                     const uint8_t* codes, const uint16_t* scales, float* y,
                                     int64_t T, int64_t D, int64_t N, int dtype_h, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int NP = next_pow2((int)N);
  const int CP = pick_group((int)(D / 32), 8, 64);  // lanes per expert split: chunks of a row
  if (dtype_h == kF32)
    return dispatch_nf3_np<float>(NP, CP, ids, h, w_r, codes, scales, y, T, (int)D, (int)N, s);
  return dispatch_nf3_np<uint16_t>(NP, CP, ids, h, w_r, codes, scales, y, T, (int)D, (int)N, s);
}

void nf3_levels_host(float* out) {
  static const uint32_t bits[8] = {0xbf800000u, 0xbf08f740u, 0xbe7cdb98u, 0x00000000u,
                                   0x3e3bbcd2u, 0x3ec394b6u, 0x3f1f7bfeu, 0x3f800000u};
  for (int i = 0; i < 8; ++i) {
    union { uint32_t u; float f; } cv;
    cv.u = bits[i];
    out[i] = cv.f;
  }
}

}  // namespace mole
