// Lookup-combine over a bf16/fp32 table: router softmax + gather of each
// token's N x D table slab + gate-weighted sum.  (MoLE article, inference
// section: retrieve each token's expert outputs by token id; training
// section: the router reads the contextual hidden state and all routed
// experts are active.)
//
// Work decomposition (one launch, no inter-block communication):
//   * a "group" of G lanes (G a power of two) owns one token; a block holds
//     one token (small bf16 batches), four (bf16 batches from 1024 tokens
//     at 128-256 lanes per token, blocks of 4 G threads), or up to 16,
//     fewer when the batch is small so that the grid still covers the 256
//     compute units;
//   * router, bf16 with several tokens per block: the block's logits
//     [tokens x experts] come from v_mfma_f32_16x16x32_bf16 tiles (tokens x
//     16 experts, K = 32 per instruction), the waves splitting D, so W_r is
//     read once per block; partial tiles meet in LDS and the softmax runs
//     on one lane per (token, expert) (MfmaRouter);
//   * router, one token per block, fp32 or unaligned: lanes split D into
//     chunks, form per-expert partial dot products, reduce them across the
//     group with a wavefront reduce-scatter (xor shuffles) plus one LDS
//     exchange;
//   * gather/combine: lane `l` of the group streams chunks l, l+G, ... of
//     every expert row of the token's contiguous slab LUT[id] with 16-byte
//     loads and accumulates in fp32.  The router's operands are loaded
//     first and the first batch of slab loads right after, so the router
//     waits only for its own operands and the slab arrives during the
//     router's arithmetic.
#include "combine_common.hpp"

namespace mole {

// ---------------------------------------------------------------------------
// bf16 / fp32 table
// ---------------------------------------------------------------------------
// ADD (the MoLE block's last pass): y[t][d] += sum_s addp[s * add_stride + t * D + d]
// + the routed combine, i.e. y is the residual stream, read and written.
// Staged gates are read from `gates` (row stride D), which may be y itself:
// neither pointer is restrict-qualified, so the gate loads stay ahead of the
// barrier that precedes the first store.
template <typename T, int NP, int G, bool VECTOR, int MODE, bool ADD = false, int BT = 256>
__global__ __launch_bounds__(BT) void lookup_combine_kernel(
    const int64_t* __restrict__ ids, const T* __restrict__ h, const T* __restrict__ w_r,
    const T* __restrict__ lut, float* y, int64_t T_, int D, int N, int tpb,
    const float* gates, const float* __restrict__ addp, int nadd, int64_t add_stride) {
  constexpr int WG = G > kWave ? G / kWave : 1;
  constexpr int MAXTPB = BT / G < kMaxTokPerBlock ? BT / G : kMaxTokPerBlock;
  // BT > 256: wide blocks (MFMA router only): one router tile for the
  // block's BT / G tokens, each wavefront taking at most 4 of its K steps
  // (the host launches them only where ceil(D / 32) <= 4 BT / 64).
  constexpr bool kWide = BT > 256;
  static_assert(!kWide || (MODE == kRouterMfma && NP <= 16 && BT <= 1024), "wide blocks: MFMA router");
  constexpr int CH = VECTOR ? Elem<T>::kVec : 1;  // elements per chunk
  // Experts per batch of slab loads.  With the vector-unit router at 16
  // experts the slab goes out in two halves: the first before the router's
  // arithmetic, the second once the router's operand registers are free --
  // all 16 rows at once with the router's operands held 146 registers, three
  // wavefronts per SIMD instead of four.
  constexpr bool kLaneSplit = VECTOR && sizeof(T) == 2 && (MODE == kRouterLane || BT > 256) && NP == 16;
  constexpr int EC = kLaneSplit ? 8 : (NP < 16 ? NP : 16);
  // Router: on the matrix cores (bf16, several tokens per block), or on
  // the vector units with its loads first (one token per block, or fp32),
  // or element-wise (unaligned rows, or more than 16 experts in fp32).
  constexpr bool kStaged = MODE == kRouterStaged;
  constexpr bool kMfmaRouter = VECTOR && sizeof(T) == 2 && MODE == kRouterMfma;
  constexpr bool kLaneRouter = VECTOR && !kMfmaRouter && !kStaged && NP <= 16;
  constexpr int NPAD = ((NP + 15) / 16) * 16;
  __shared__ float red[kMfmaRouter ? (BT / kWave) * 16 * NPAD : MAXTPB * WG * NP];
  __shared__ float gsh[kMfmaRouter ? kMaxTokPerBlock * NP : 1];
  // bf16 tokens of at least a wavefront (G >= 64): when a token's chunks
  // fill its lanes exactly (C == G, one round), each wavefront's sums go
  // through its slice of LDS and come back as 16-byte pieces, so that one
  // store instruction writes 1 KB of the row (whole 128-byte lines) instead
  // of half-lines in two instructions (410M-class table, T = 4096 distinct
  // ids: 28.1 -> 27.2 us; 20 % of written bytes were partial lines).
  constexpr bool kStageOut = VECTOR && !ADD && sizeof(T) == 2 && G >= kWave;
  __shared__ float ys[kStageOut ? (BT / kWave) * kWave * CH : 1];

  // tpb (tokens per block, = blockDim.x / G) comes as an argument: reading
  // the block size costs a dependent load of the dispatch packet.
  const int tid = threadIdx.x;
  const int grp = tid / G, lig = tid % G;
  const int64_t t0 = (int64_t)blockIdx.x * tpb;
  const int64_t t = t0 + grp;
  const bool valid = t < T_;
  const int64_t tt = valid ? t : 0;
  const int C = D / CH;
  const int64_t id_ld = ids[tt];  // unconditional (tt is clamped): see MfmaRouter::load
  __builtin_amdgcn_sched_barrier(0);  // the id load goes out first

  // Router operands next, then the first batch of slab loads (chunk lig,
  // experts 0..EC-1); the router's arithmetic runs while the slab arrives.
  MfmaRouter<NP, kWide ? 4 : 0> rt;
  LaneRouter<T, kLaneRouter ? NP : 1> lr;
  if constexpr (kMfmaRouter)
    rt.load_first(reinterpret_cast<const uint16_t*>(h), reinterpret_cast<const uint16_t*>(w_r), t0, T_, tpb, D,
                  N, (G * tpb) / kWave);
  if constexpr (kLaneRouter) lr.load_first(h + tt * D, w_r, D, N, lig);
  // Staged gates: this token's N gates from the start of its own output row
  // (every lane of the group reads the same 16-byte words).
  constexpr int NG = kStaged ? (NP + 3) / 4 : 1;
  uint4 gq[NG];
  if constexpr (kStaged) {
#pragma unroll
    for (int q = 0; q < NG; ++q) gq[q] = ldg16(gates + tt * D + 4 * q);
  }
  __builtin_amdgcn_sched_barrier(0);
  const int64_t id = valid ? id_ld : 0;  // (the first wait on the id load is here)
  const T* slab = lut + id * (int64_t)N * D;
  // (Unconditional loads from clamped chunk and expert indices; lanes past
  // the row and experts past N read data they then ignore.)
  uint4 sv[EC];
  uint4 sv2[kLaneSplit ? EC : 1];
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
  if constexpr (kStaged) {
#pragma unroll
    for (int q = 0; q < NG; ++q) {
      const float g4[4] = {__uint_as_float(gq[q].x), __uint_as_float(gq[q].y), __uint_as_float(gq[q].z),
                           __uint_as_float(gq[q].w)};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * q + i < NP) gate[4 * q + i] = 4 * q + i < N ? g4[i] : 0.f;
    }
    // Every wave holds its tokens' gates before any wave overwrites the rows.
    __syncthreads();
  } else if constexpr (kMfmaRouter) {
    if constexpr (kWide) {
      rt.compute_one_batch();
      if constexpr (kLaneSplit) {
        // second half of the first chunk's expert rows, once the router's
        // operand registers are free (clamped as above)
        const int c0 = lig < C ? lig : C - 1;
#pragma unroll
        for (int e = 0; e < EC; ++e) {
          const int ec = EC + e < N ? EC + e : N - 1;
          sv2[e] = ldg16(slab + (int64_t)ec * D + (int64_t)c0 * CH);
        }
      }
      rt.reduce_wide(tpb, N, red, gsh);
    } else {
      rt.finish(tpb, N, red, gsh);
    }
#pragma unroll
    for (int e = 0; e < NP; ++e) gate[e] = gsh[grp * NP + e];
    if constexpr (G >= kWave) {
      // a wavefront serves one token: its gates are wave-uniform
#pragma unroll
      for (int e = 0; e < NP; ++e) gate[e] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(gate[e])));
    }
  } else if constexpr (kLaneRouter) {
    float part[NP];
    lr.template partials<G>(h + tt * D, w_r, D, N, lig, valid, part);
    if constexpr (kLaneSplit) {
      // second half of the first chunk's expert rows (clamped as above)
      const int c0 = lig < C ? lig : C - 1;
#pragma unroll
      for (int e = 0; e < EC; ++e) {
        const int ec = EC + e < N ? EC + e : N - 1;
        sv2[e] = ldg16(slab + (int64_t)ec * D + (int64_t)c0 * CH);
      }
    }
    group_gates<NP, G>(part, gate, N, lig, red + grp * WG * NP);
    if (tpb == 1) {
      // one token per block: the gates are block-uniform, keep them in scalar registers
#pragma unroll
      for (int e = 0; e < NP; ++e) gate[e] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(gate[e])));
    }
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
      if (kLaneSplit && k == 0 && e0 == EC) {
#pragma unroll
        for (int e = 0; e < EC; ++e) sv[e] = sv2[e];  // loaded during the router
      } else if (k != 0 || e0 != 0) {
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
    if constexpr (ADD) {
      static_assert(VECTOR, "the block's final pass reads 16-byte chunks");
      const int64_t o = tt * D + (int64_t)c * CH;
      // Partial sums four splits at a time: the four loads of a batch go out
      // together (indices clamped to the last split, the extra copies
      // weighted by zero), so a pass over S splits waits ceil(S / 4) times.
      float4 a[CH / 4];
#pragma unroll
      for (int j = 0; j < CH; j += 4) a[j / 4] = *reinterpret_cast<const float4*>(yo + j);
      for (int s0 = 0; s0 < nadd; s0 += 4) {
        float4 b[4][CH / 4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int sp = s0 + q < nadd ? s0 + q : nadd - 1;
#pragma unroll
          for (int j = 0; j < CH; j += 4) b[q][j / 4] = *reinterpret_cast<const float4*>(addp + sp * add_stride + o + j);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float wq = s0 + q < nadd ? 1.f : 0.f;
#pragma unroll
          for (int j = 0; j < CH / 4; ++j) {
            a[j].x = fmaf(wq, b[q][j].x, a[j].x);
            a[j].y = fmaf(wq, b[q][j].y, a[j].y);
            a[j].z = fmaf(wq, b[q][j].z, a[j].z);
            a[j].w = fmaf(wq, b[q][j].w, a[j].w);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < CH; j += 4)
        stg16_nt(yo + j, a[j / 4].x + acc[j], a[j / 4].y + acc[j + 1], a[j / 4].z + acc[j + 2],
                 a[j / 4].w + acc[j + 3]);
    } else if constexpr (VECTOR) {
      bool staged = false;
      if constexpr (kStageOut) {
        if (C == G) {  // uniform: every lane of the wavefront has chunk k * G + lig in this one round
          staged = true;
          const int wv = tid >> 6, lane = tid & 63;
          float* yw = ys + wv * (kWave * CH);
#pragma unroll
          for (int j = 0; j < CH; j += 4)
            *reinterpret_cast<float4*>(yw + lane * CH + j) = make_float4(acc[j], acc[j + 1], acc[j + 2], acc[j + 3]);
          __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
          float* yrow = y + tt * D + (int64_t)(c - lane) * CH;  // the wavefront's first chunk
#pragma unroll
          for (int q = 0; q < CH / 4; ++q) {
            const float4 v = *reinterpret_cast<const float4*>(yw + 4 * lane + 256 * q);
            stg16_nt(yrow + 4 * lane + 256 * q, v.x, v.y, v.z, v.w);
          }
        }
      }
      if (!staged) {
#pragma unroll
        for (int j = 0; j < CH; j += 4)
          stg16_nt(yo + j, acc[j], acc[j + 1], acc[j + 2], acc[j + 3]);
      }
    } else {
      __builtin_nontemporal_store(acc[0], yo);
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side dispatch
// ---------------------------------------------------------------------------

struct CombineExtra {
  float* gates_buf;    // where the staged router writes gates (row stride D); the combine's y if null
  const float* addp;   // ADD pass: partial sums added to y (null: plain combine)
  int nadd;
  int64_t add_stride;
};

template <typename E, int NP, int G, bool VEC, bool ADD>
static hipError_t launch_dense_add(const int64_t* ids, const void* h, const void* w_r, const void* lut, float* y,
                                   int64_t T, int D, int N, const CombineExtra& ex, hipStream_t s) {
  // Up to T = 1024 (bf16, NP <= 16, a token fills at least a wavefront): one
  // token per workgroup with the vector-unit router rather than the matrix-
  // core router over two; measured on the 410M-class table at T = 1024:
  // 10.95 -> 8.1 us with Zipf ids, 12.0 -> 10.0 us with distinct ids (no
  // change at T = 256, where a workgroup already holds one token).
  //
  // From T = 1024 on at widths of 128-256 lanes per token (D from 520 to
  // 2048 bf16): four tokens per workgroup of 4 G threads, routed together
  // on the matrix cores (each wavefront takes at most 4 of the K steps:
  // ceil(D / 32) <= 8 G / 32 = 4 * (4 G / 64)), so W_r is read once per
  // four tokens and the router's dot products leave the vector units.
  // Measured with distinct ids: 1B-class T = 1024 17.97 -> 15.11 us, T =
  // 4096 60.3 -> 58.0 us; 410M-class T = 1024 9.80 -> 8.27 us, T = 4096
  // 32.7 -> 28.7 us (the staged router's two launches).  Not for the
  // block's ADD pass, whose partial-sum loads do not fit the registers of
  // 16 wavefronts per compute unit, and not for rows wider than G chunks
  // (D > 2048: G stops at 256), whose K steps would not fit the one batch.
  if constexpr (!ADD && VEC && sizeof(E) == 2 && NP <= 16 && G >= 128) {
    if (T >= 1024 && D <= 8 * G) {
      constexpr int kTok = 4, BT = kTok * G;
      hipLaunchKernelGGL((lookup_combine_kernel<E, NP, G, VEC, kRouterMfma, ADD, BT>),
                         dim3((unsigned)((T + kTok - 1) / kTok)), dim3(BT), 0, s, ids, (const E*)h,
                         (const E*)w_r, (const E*)lut, y, T, D, N, kTok, (const float*)nullptr, ex.addp, ex.nadd,
                         ex.add_stride);
      return hipGetLastError();
    }
  }
  const bool one_token = VEC && sizeof(E) == 2 && NP <= 16 && G >= 64 && T <= 1024;
  const int tpb = one_token ? 1 : pick_tokens_per_block(T, G);
  const int64_t blocks = (T + tpb - 1) / tpb;
  float* gbuf = ex.gates_buf ? ex.gates_buf : y;
  if constexpr (VEC && sizeof(E) == 2) {
    // (The combine reads each token's gates as ceil(NP / 4) 16-byte words
    // from the head of its row: NP <= D keeps them inside the row.)
    if (T >= kStagedRouterMinT && tpb >= 2 && NP <= D) {
      const int64_t rblocks = (T + kMaxTokPerBlock - 1) / kMaxTokPerBlock;
      hipLaunchKernelGGL((router_gates_kernel<NP>), dim3((unsigned)rblocks), dim3(256), 0, s, (const uint16_t*)h,
                         (const uint16_t*)w_r, gbuf, T, D, N);
      hipLaunchKernelGGL((lookup_combine_kernel<E, NP, G, VEC, kRouterStaged, ADD>), dim3((unsigned)blocks),
                         dim3(G * tpb), 0, s, ids, (const E*)h, (const E*)w_r, (const E*)lut, y, T, D, N, tpb,
                         gbuf, ex.addp, ex.nadd, ex.add_stride);
      return hipGetLastError();
    }
  }
  // One token per block: the vector-unit router (see LaneRouter).
  if constexpr (VEC && sizeof(E) == 2 && NP <= 16 && G >= 64) {
    if (tpb == 1) {
      hipLaunchKernelGGL((lookup_combine_kernel<E, NP, G, VEC, kRouterLane, ADD>), dim3((unsigned)blocks), dim3(G),
                         0, s, ids, (const E*)h, (const E*)w_r, (const E*)lut, y, T, D, N, 1, gbuf, ex.addp,
                         ex.nadd, ex.add_stride);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((lookup_combine_kernel<E, NP, G, VEC, kRouterMfma, ADD>), dim3((unsigned)blocks),
                     dim3(G * tpb), 0, s, ids, (const E*)h, (const E*)w_r, (const E*)lut, y, T, D, N, tpb, gbuf,
                     ex.addp, ex.nadd, ex.add_stride);
  return hipGetLastError();
}

template <typename E, int NP, int G, bool VEC>
static hipError_t launch_dense(const int64_t* ids, const void* h, const void* w_r, const void* lut, float* y,
                               int64_t T, int D, int N, const CombineExtra& ex, hipStream_t s) {
  if constexpr (VEC && sizeof(E) == 2) {
    if (ex.addp) return launch_dense_add<E, NP, G, VEC, true>(ids, h, w_r, lut, y, T, D, N, ex, s);
  }
  return launch_dense_add<E, NP, G, VEC, false>(ids, h, w_r, lut, y, T, D, N, ex, s);
}

template <typename E, int NP, bool VEC>
static hipError_t dispatch_dense_g(int G, const int64_t* ids, const void* h, const void* w_r,
                                   const void* lut, float* y, int64_t T, int D, int N, const CombineExtra& ex,
                                   hipStream_t s) {
  switch (G) {
    case 16: return launch_dense<E, NP, 16, VEC>(ids, h, w_r, lut, y, T, D, N, ex, s);
    case 32: return launch_dense<E, NP, 32, VEC>(ids, h, w_r, lut, y, T, D, N, ex, s);
    case 64: return launch_dense<E, NP, 64, VEC>(ids, h, w_r, lut, y, T, D, N, ex, s);
    case 128: return launch_dense<E, NP, 128, VEC>(ids, h, w_r, lut, y, T, D, N, ex, s);
    default: return launch_dense<E, NP, 256, VEC>(ids, h, w_r, lut, y, T, D, N, ex, s);
  }
}

template <typename E, bool VEC>
static hipError_t dispatch_dense_np(int NP, int G, const int64_t* ids, const void* h, const void* w_r,
                                    const void* lut, float* y, int64_t T, int D, int N, const CombineExtra& ex,
                                    hipStream_t s) {
  switch (NP) {
    case 1: return dispatch_dense_g<E, 1, VEC>(G, ids, h, w_r, lut, y, T, D, N, ex, s);
    case 2: return dispatch_dense_g<E, 2, VEC>(G, ids, h, w_r, lut, y, T, D, N, ex, s);
    case 4: return dispatch_dense_g<E, 4, VEC>(G, ids, h, w_r, lut, y, T, D, N, ex, s);
    case 8: return dispatch_dense_g<E, 8, VEC>(G, ids, h, w_r, lut, y, T, D, N, ex, s);
    case 16: return dispatch_dense_g<E, 16, VEC>(G, ids, h, w_r, lut, y, T, D, N, ex, s);
    case 32: return dispatch_dense_g<E, 32, VEC>(G, ids, h, w_r, lut, y, T, D, N, ex, s);
    default: return dispatch_dense_g<E, 64, VEC>(G, ids, h, w_r, lut, y, T, D, N, ex, s);
  }
}

hipError_t launch_lookup_combine(const int64_t* ids, const void* h, const void* w_r, const void* lut,
                                 float* y, int64_t T, int64_t D, int64_t N, int dtype, bool vector_ok,
                                 hipStream_t s, float* gates_buf, const float* addp, int nadd,
                                 int64_t add_stride) {
  if (T == 0) return hipSuccess;
  const int NP = next_pow2((int)N);
  const int elem_bytes = dtype == kF32 ? 4 : 2;
  const int vec = 16 / elem_bytes;
  const bool vector = vector_ok && (D % vec == 0);
  if (addp && (dtype == kF32 || !vector)) return hipErrorInvalidValue;  // the block's pass is bf16, 16-byte chunks
  const int C = vector ? (int)(D / vec) : (int)D;
  const int G = pick_group(C, 16, 256);
  const CombineExtra ex{gates_buf, addp, nadd, add_stride};
  if (dtype == kF32)
    return vector ? dispatch_dense_np<float, true>(NP, G, ids, h, w_r, lut, y, T, (int)D, (int)N, ex, s)
                  : dispatch_dense_np<float, false>(NP, G, ids, h, w_r, lut, y, T, (int)D, (int)N, ex, s);
  return vector ? dispatch_dense_np<uint16_t, true>(NP, G, ids, h, w_r, lut, y, T, (int)D, (int)N, ex, s)
                : dispatch_dense_np<uint16_t, false>(NP, G, ids, h, w_r, lut, y, T, (int)D, (int)N, ex, s);
}

}  // namespace mole
