// Lookup-combine over a quantised table: router softmax + decode of each
// token's N x D codes + gate-weighted sum.  Formats: NF3 (3 bits per
// element, one fp16 absmax scale per 64 elements), NF4 (4 bits, same
// scales) and int8 (one fp32 scale per table row).  (MoLE article, results
// section: the table keeps the model's quality when compressed to 3 bits,
// e.g. NF3, so it still carries redundancy; inference section: each token's
// expert outputs are fetched by token id.)  The routers and the
// launch-shape helpers are shared with the dense-table kernel.
#include "combine_common.hpp"

namespace mole {

// Level tables: kNf3LevelBits / kNf4LevelBits (mole_tables.hpp).

// Per-format constants: bytes of codes per 32-element chunk, levels in the
// decode table (0: the code is the value), experts per batch of code loads.
template <int FMT> struct QFmt;
template <> struct QFmt<kFmtNf3> {
  static constexpr int kChunkBytes = 12, kLevels = 8, kBatch = 8;
  static constexpr int64_t row_bytes(int64_t D) { return 3 * D / 8; }
};
template <> struct QFmt<kFmtNf4> {
  static constexpr int kChunkBytes = 16, kLevels = 16, kBatch = 4;
  static constexpr int64_t row_bytes(int64_t D) { return D / 2; }
};
template <> struct QFmt<kFmtI8> {
  static constexpr int kChunkBytes = 32, kLevels = 0, kBatch = 4;
  static constexpr int64_t row_bytes(int64_t D) { return D; }
};

// ---------------------------------------------------------------------------
// A chunk is 32 elements of a row: 12 bytes of NF3 codes, 16 of NF4 or 32
// of int8; NF3 and NF4 chunks take one fp16 scale per 64 elements, int8 one
// fp32 scale per row.
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

// W > 1 (small batches, one token per block): the block's W wavefronts
// share one token.  Wavefront w takes the experts ((j W + w) S + s), the W
// of them route the token together (one lane group of 64 W lanes), and the
// per-wavefront partial sums of a chunk meet in LDS; each wavefront then
// stores a 1/W share of the chunk's outputs.  This spreads a decode-sized
// batch over W times as many wavefronts.
template <typename TH, int NP, int CP, int S, int MODE, int FMT = kFmtNf3, int W = 1, int BT = 256>
__global__ __launch_bounds__(BT) void lookup_combine_nf3_kernel(
    const int64_t* __restrict__ ids, const TH* __restrict__ h, const TH* __restrict__ w_r,
    const uint8_t* __restrict__ codes, const void* __restrict__ scales_v,
    float* __restrict__ y, int64_t T_, int D, int N, int tpb) {
  using Q = QFmt<FMT>;
  constexpr int G = CP * S;                        // lanes per token (<= 64)
  static_assert(G <= kWave, "a token's lanes must share one wavefront");
  constexpr int MAXTPB = BT / G < kMaxTokPerBlock ? BT / G : kMaxTokPerBlock;
  static_assert(W == 1 || (G == kWave && MODE == kRouterLane), "W > 1: one token per block, full wavefronts");
  constexpr int EPL = (NP + S * W - 1) / (S * W);  // experts per lane
  constexpr int EC = EPL < Q::kBatch ? EPL : Q::kBatch;  // experts per batch of code loads
  constexpr int CW = Q::kChunkBytes / 4;           // code dwords per chunk
  constexpr int OUT = 32 / S;                      // sums per lane and chunk after the split reduce
  static_assert(OUT % W == 0, "each wavefront stores a whole share of a lane's sums");
  constexpr int OW = OUT / W;                      // outputs stored per lane and chunk
  // Router: on the matrix cores (bf16 h, several tokens per block), else on
  // the vector units (one token per block, or fp32 h; element-wise beyond
  // 16 experts).
  static_assert(MODE != kRouterStaged, "the NF3 kernel routes in the same launch");
  constexpr bool kMfmaRouter = sizeof(TH) == 2 && MODE == kRouterMfma;
  constexpr bool kLaneRouter = !kMfmaRouter && NP <= 16;
  constexpr int NPAD = ((NP + 15) / 16) * 16;
  __shared__ float red[kMfmaRouter ? (BT / kWave) * 16 * NPAD : MAXTPB * NP];
  __shared__ float gsh[kMaxTokPerBlock * NP];
  // Decode table indexed by two consecutive codes at once (6 bits for NF3,
  // one byte for NF4): entry p holds the levels of codes p % L and p / L.
  // One LDS read and one bit-field extraction then serve two elements.
  __shared__ float2 lv2[Q::kLevels > 0 ? Q::kLevels * Q::kLevels : 1];
  // W > 1: the wavefronts' partial sums, [wavefront][sum][lane] (lane-minor:
  // conflict-free writes and reads).
  __shared__ float xw[W > 1 ? W * OUT * kWave : 1];
  // One token per wavefront: each round's outputs (CP chunks of 32) go
  // through this wavefront's slice of LDS, so that every 16-byte store
  // instruction writes 1 KB of the token's row (whole 128-byte lines).
  // Stored straight from the lanes, each line was written in four pieces
  // by four instructions and left L2 in parts: 25.4 MB written for the
  // 16.8 MB of y (410M-class table, T = 4096).
  constexpr bool kStageOut = W == 1 && G == kWave && OW >= 4;
  // (one wavefront per block in the vector-router launches, up to four in the others)
  __shared__ float ys[kStageOut ? (MODE == kRouterLane ? 1 : BT / kWave) * CP * 32 : 1];

  const int tid = threadIdx.x;
  if constexpr (FMT == kFmtNf3) {
    for (int i = tid; i < 64; i += blockDim.x)
      lv2[i] = make_float2(__uint_as_float(kNf3LevelBits[i & 7]), __uint_as_float(kNf3LevelBits[i >> 3]));
  } else if constexpr (FMT == kFmtNf4) {
    for (int i = tid; i < 256; i += blockDim.x)
      lv2[i] = make_float2(__uint_as_float(kNf4LevelBits[i & 15]), __uint_as_float(kNf4LevelBits[i >> 4]));
  }
  const int grp = tid / G, lig = tid % G;  // tpb = blockDim.x / G, passed in
  const int sp = lig / CP, ch = lig % CP;          // expert split, chunk
  const int wsp = W > 1 ? grp : 0;                 // W > 1: this wavefront's share of the experts
  const int64_t t0 = (int64_t)blockIdx.x * tpb;
  const int64_t t = W > 1 ? t0 : t0 + grp;
  const bool valid = t < T_;
  const int64_t tt = valid ? t : 0;
  const int C = D / 32;                            // 32-element chunks per row
  const int64_t row_bytes = Q::row_bytes(D), nblk = D / 64;
  const int64_t id = valid ? ids[tt] : 0;
  const uint8_t* crow0 = codes + id * (int64_t)N * row_bytes;
  const uint16_t* srow0 = static_cast<const uint16_t*>(scales_v) + id * (int64_t)N * nblk;  // NF3, NF4
  const float* srowf = static_cast<const float*>(scales_v) + id * (int64_t)N;               // int8

  uint32_t cw[EC][CW];
  uint32_t sc[EC];
  auto load_batch = [&](int c, int j0) {
#pragma unroll
    for (int j = 0; j < EC; ++j) {
      const int e = ((j0 + j) * W + wsp) * S + sp;
      if (e < N) {
        const uint8_t* src = crow0 + (int64_t)e * row_bytes + (int64_t)c * Q::kChunkBytes;
        if constexpr (FMT == kFmtNf3) {
          const uint3 v = *reinterpret_cast<const uint3*>(src);
          cw[j][0] = v.x; cw[j][1] = v.y; cw[j][2] = v.z;
        } else {
#pragma unroll
          for (int q = 0; q < CW / 4; ++q) {
            const uint4 v = *reinterpret_cast<const uint4*>(src + 16 * q);
            cw[j][4 * q] = v.x; cw[j][4 * q + 1] = v.y; cw[j][4 * q + 2] = v.z; cw[j][4 * q + 3] = v.w;
          }
        }
        if constexpr (FMT == kFmtI8) sc[j] = __float_as_uint(srowf[e]);
        else sc[j] = srow0[(int64_t)e * nblk + (c >> 1)];
      }
    }
  };
  // One token per wavefront (matrix-core router): the router's operands
  // first, then the first batch of code loads, branch-free through buffer
  // resources over the token's rows (wave-uniform base; expert and chunk
  // clamped), so the router's matrix work waits only for its own operands.
  // Measured on the 410M-class NF3 table at T = 4096: 18.1 -> 16.3 us.
  constexpr bool kReorder = kMfmaRouter && G == kWave && W == 1;
  MfmaRouter<NP, (NP <= 16 && BT > 256) ? 2048 / BT : 0> rt;
  LaneRouter<TH, kLaneRouter ? NP : 1> lr;
  if constexpr (kReorder) {
    rt.load_first(reinterpret_cast<const uint16_t*>(h), reinterpret_cast<const uint16_t*>(w_r), t0, T_, tpb, D,
                  N, (G * tpb) / kWave);
    const int64_t idu = ((int64_t)__builtin_amdgcn_readfirstlane((int)(id >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((int)id);
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(codes + idu * (int64_t)N * row_bytes), (short)0, (int)(N * row_bytes), kRsrcWord3);
    const int64_t srec = FMT == kFmtI8 ? 4 * (int64_t)N : 2 * (int64_t)N * nblk;  // scale bytes per table row
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(static_cast<const uint8_t*>(scales_v) + idu * srec), (short)0, (int)srec, kRsrcWord3);
    const int cc = ch < C ? ch : C - 1;
#pragma unroll
    for (int j = 0; j < EC; ++j) {
      const int e = (j * W + wsp) * S + sp, ec = e < N ? e : N - 1;
      const int co = ec * (int)row_bytes + cc * Q::kChunkBytes;
      if constexpr (FMT == kFmtNf3) {
        typedef uint32_t v3u __attribute__((ext_vector_type(3)));
        const v3u v = __builtin_amdgcn_raw_buffer_load_b96(rc, co, 0, 0);
        cw[j][0] = v.x; cw[j][1] = v.y; cw[j][2] = v.z;
      } else {
#pragma unroll
        for (int q = 0; q < CW / 4; ++q) {
          const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rc, co + 16 * q, 0, 0));
          cw[j][4 * q] = v.x; cw[j][4 * q + 1] = v.y; cw[j][4 * q + 2] = v.z; cw[j][4 * q + 3] = v.w;
        }
      }
      if constexpr (FMT == kFmtI8) sc[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * ec, 0, 0);
      else sc[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, 2 * (ec * (int)nblk + (cc >> 1)), 0, 0);
    }
  } else {
    // First batch of code loads, then the router's operands.  (The reverse
    // order needs branch-free code loads; with several tokens per wavefront
    // they cost this kernel about 25 registers and one wave per SIMD of
    // occupancy, more than the overlap gains.)
    if (valid && ch < C) load_batch(ch, 0);
    if constexpr (kMfmaRouter)
      rt.load_first(reinterpret_cast<const uint16_t*>(h), reinterpret_cast<const uint16_t*>(w_r), t0, T_, tpb, D,
                    N, (G * tpb) / kWave);
    if constexpr (kLaneRouter) lr.load_first(h + tt * D, w_r, D, N, W > 1 ? tid : lig);
  }

  // Gates of the block's tokens into gsh[token][expert].
  if constexpr (kMfmaRouter) {
    rt.finish(tpb, N, red, gsh);
  } else if constexpr (kLaneRouter) {
    float gate[NP];
    if constexpr (W > 1)
      lr.template finish<G * W>(h + tt * D, w_r, D, N, tid, valid, gate, red);
    else
      lr.template finish<G>(h + tt * D, w_r, D, N, lig, valid, gate, red + grp * NP);
    if (lig == 0) {
#pragma unroll
      for (int e = 0; e < NP; ++e) gsh[grp * NP + e] = gate[e];
    }
    __syncthreads();
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

  // Every lane walks the same number of chunk rounds (W > 1 has barriers
  // inside); a lane whose chunk is past the row does no work in a round.
  const int rounds = (C + CP - 1) / CP;
  for (int k = 0; k < rounds; ++k) {
    const int c = k * CP + ch;
    const bool act = c < C;
    float acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j0 = 0; j0 < EPL; j0 += EC) {
      if (act && (k != 0 || j0 != 0)) load_batch(c, j0);
#pragma unroll
      for (int j = 0; j < EC; ++j) {
        const int e = ((j0 + j) * W + wsp) * S + sp;
        if (act && e < N) {
          const float sv = FMT == kFmtI8 ? __uint_as_float(sc[j])
                                         : (float)__builtin_bit_cast(_Float16, (uint16_t)sc[j]);
          const float ws = gsh[grp * NP + e] * sv;
          const uint32_t* w = cw[j];
          if constexpr (FMT == kFmtNf3) {
            // code pair q = bits 6q .. 6q + 5 of the chunk's 96 bits
#pragma unroll
            for (int q = 0; q < 16; ++q) {
              const int pos = 6 * q, wd = pos >> 5, off = pos & 31;
              uint32_t pr;
              if (off <= 26) pr = (w[wd] >> off) & 63u;
              else pr = __builtin_amdgcn_alignbit(w[wd + 1], w[wd], off) & 63u;
              const float2 l = lv2[pr];
              acc[2 * q] = fmaf(ws, l.x, acc[2 * q]);
              acc[2 * q + 1] = fmaf(ws, l.y, acc[2 * q + 1]);
            }
          } else if constexpr (FMT == kFmtNf4) {
#pragma unroll
            for (int q = 0; q < 16; ++q) {
              const float2 l = lv2[(w[q >> 2] >> (8 * (q & 3))) & 255u];
              acc[2 * q] = fmaf(ws, l.x, acc[2 * q]);
              acc[2 * q + 1] = fmaf(ws, l.y, acc[2 * q + 1]);
            }
          } else {
#pragma unroll
            for (int i = 0; i < 32; ++i) {
              const int q = (int)(w[i >> 2] << (24 - 8 * (i & 3))) >> 24;  // signed byte i
              acc[i] = fmaf(ws, (float)q, acc[i]);
            }
          }
        }
      }
    }
    SplitReduce<CP, S>::run(acc, sp);
    if constexpr (W > 1) {
      // the W wavefronts' sums of this chunk meet in LDS (added in wavefront order)
#pragma unroll
      for (int j = 0; j < OUT; ++j) xw[(wsp * OUT + j) * kWave + lig] = acc[j];
      __syncthreads();
#pragma unroll
      for (int q = 0; q < OW; ++q) {
        float a = 0.f;
#pragma unroll
        for (int u = 0; u < W; ++u) a += xw[(u * OUT + wsp * OW + q) * kWave + lig];
        acc[q] = a;
      }
      __syncthreads();  // xw is rewritten in the next round
    }
    if constexpr (kStageOut) {
      // (lanes past the row write their unused sums too: those LDS words
      // are never stored)
      float* yw = ys + grp * (CP * 32);
#pragma unroll
      for (int j = 0; j < OW; j += 4)
        *reinterpret_cast<float4*>(yw + ch * 32 + SplitReduce<CP, S>::offset(sp) + j) =
            make_float4(acc[j], acc[j + 1], acc[j + 2], acc[j + 3]);
      // the wavefront's LDS accesses complete in order; the fence keeps the
      // compiler from moving the reads above the writes
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      const int lane = lig;
#pragma unroll
      for (int q = 0; q < CP * 32 / 256; ++q) {
        const int e = k * CP * 32 + 4 * lane + 256 * q;  // element of the token's row
        const float4 v = *reinterpret_cast<const float4*>(yw + 4 * lane + 256 * q);
        if (e < D) stg16_nt(y + tt * D + e, v.x, v.y, v.z, v.w);
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // the slice is rewritten next round
    } else if (act) {
      float* yo = y + tt * D + (int64_t)c * 32 + SplitReduce<CP, S>::offset(sp) + wsp * OW;
      if constexpr (OW >= 4) {
#pragma unroll
        for (int j = 0; j < OW; j += 4) stg16_nt(yo + j, acc[j], acc[j + 1], acc[j + 2], acc[j + 3]);
      } else {
#pragma unroll
        for (int j = 0; j < OW; ++j) __builtin_nontemporal_store(acc[j], yo + j);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// NF3 combine over a batch in grouped order (equal ids adjacent; see
// combine_grouped.hip): position p holds token pos_tok[p], table row
// pos_row[p], and the token's gates come precomputed in gates[token][NP].
// One token per wavefront, four per workgroup, the per-token kernel's lane
// layout, decode and staged stores.  Tokens that share an id run on
// neighbouring workgroups of one pass, so their rows are fetched from memory
// about once and then served from cache: this pays where every byte read is
// expensive, as for a table read in place over PCIe.
// ---------------------------------------------------------------------------
template <int NP, int CP, int S>
__global__ __launch_bounds__(256) void lookup_combine_nf3_grouped_kernel(
    const int* __restrict__ pos_tok, const int* __restrict__ pos_row, const float* __restrict__ gates,
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales, float* __restrict__ y, int64_t T_,
    int D, int N) {
  using Q = QFmt<kFmtNf3>;
  static_assert(CP * S == kWave, "one token per wavefront");
  constexpr int EPL = (NP + S - 1) / S;  // experts per lane
  constexpr int EC = EPL < Q::kBatch ? EPL : Q::kBatch;
  constexpr int OUT = 32 / S;
  static_assert(OUT >= 4, "whole 16-byte pieces per lane");
  __shared__ float2 lv2[64];
  __shared__ float ys[4 * CP * 32];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int i = tid; i < 64; i += 256)
    lv2[i] = make_float2(__uint_as_float(kNf3LevelBits[i & 7]), __uint_as_float(kNf3LevelBits[i >> 3]));
  __syncthreads();
  const int64_t p = (int64_t)blockIdx.x * 4 + wave;
  if (p >= T_) return;  // (wave-uniform; no barrier follows)
  const int64_t tok = __builtin_amdgcn_readfirstlane(pos_tok[p]);
  const int64_t id = __builtin_amdgcn_readfirstlane(pos_row[p]);
  const int sp = lane / CP, ch = lane % CP;
  const int C = D / 32, nblk = D / 64;
  const int64_t row_bytes = Q::row_bytes(D);
  const uint8_t* crow = codes + id * (int64_t)N * row_bytes;
  const uint16_t* srow = scales + id * (int64_t)N * nblk;
  float g[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = j * S + sp;
    g[j] = e < N ? gates[tok * NP + e] : 0.f;
  }
  const int rounds = (C + CP - 1) / CP;
  for (int k = 0; k < rounds; ++k) {
    const int c = k * CP + ch;
    const bool act = c < C;
    float acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j0 = 0; j0 < EPL; j0 += EC) {
      uint32_t cw[EC][3], sc[EC];
#pragma unroll
      for (int j = 0; j < EC; ++j) {
        const int e = (j0 + j) * S + sp;
        if (act && e < N) {
          const uint3 v = *reinterpret_cast<const uint3*>(crow + (int64_t)e * row_bytes + (int64_t)c * 12);
          cw[j][0] = v.x; cw[j][1] = v.y; cw[j][2] = v.z;
          sc[j] = srow[(int64_t)e * nblk + (c >> 1)];
        }
      }
#pragma unroll
      for (int j = 0; j < EC; ++j) {
        const int e = (j0 + j) * S + sp;
        if (act && e < N) {
          const float ws = g[j0 + j] * (float)__builtin_bit_cast(_Float16, (uint16_t)sc[j]);
          const uint32_t* w = cw[j];
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int pos = 6 * q, wd = pos >> 5, off = pos & 31;
            uint32_t pr;
            if (off <= 26) pr = (w[wd] >> off) & 63u;
            else pr = __builtin_amdgcn_alignbit(w[wd + 1], w[wd], off) & 63u;
            const float2 l = lv2[pr];
            acc[2 * q] = fmaf(ws, l.x, acc[2 * q]);
            acc[2 * q + 1] = fmaf(ws, l.y, acc[2 * q + 1]);
          }
        }
      }
    }
    SplitReduce<CP, S>::run(acc, sp);
    float* yw = ys + wave * (CP * 32);
#pragma unroll
    for (int j = 0; j < OUT; j += 4)
      *reinterpret_cast<float4*>(yw + ch * 32 + SplitReduce<CP, S>::offset(sp) + j) =
          make_float4(acc[j], acc[j + 1], acc[j + 2], acc[j + 3]);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
    for (int q = 0; q < CP * 32 / 256; ++q) {
      const int e = k * CP * 32 + 4 * lane + 256 * q;  // element of the token's row
      const float4 v = *reinterpret_cast<const float4*>(yw + 4 * lane + 256 * q);
      if (e < D) stg16_nt(y + tok * D + e, v.x, v.y, v.z, v.w);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // the slice is rewritten next round
  }
}

template <int NP, int CP>
static hipError_t launch_nf3_grouped(const int* pos_tok, const int* pos_row, const float* gates, const uint8_t* codes,
                                     const uint16_t* scales, float* y, int64_t T, int D, int N, hipStream_t s) {
  constexpr int S = 64 / CP;
  const int64_t blocks = (T + 3) / 4;
  hipLaunchKernelGGL((lookup_combine_nf3_grouped_kernel<NP, CP, S>), dim3((unsigned)blocks), dim3(256), 0, s, pos_tok,
                     pos_row, gates, codes, scales, y, T, D, N);
  return hipGetLastError();
}

template <int NP>
static hipError_t dispatch_nf3_grouped_cp(int CP, const int* pos_tok, const int* pos_row, const float* gates,
                                          const uint8_t* codes, const uint16_t* scales, float* y, int64_t T, int D,
                                          int N, hipStream_t s) {
  // (64 / CP expert splits per token: at most NP, so that every split has an expert)
  if constexpr (NP >= 8)
    if (CP == 8) return launch_nf3_grouped<NP, 8>(pos_tok, pos_row, gates, codes, scales, y, T, D, N, s);
  if constexpr (NP >= 4)
    if (CP == 16) return launch_nf3_grouped<NP, 16>(pos_tok, pos_row, gates, codes, scales, y, T, D, N, s);
  if constexpr (NP >= 2)
    if (CP == 32) return launch_nf3_grouped<NP, 32>(pos_tok, pos_row, gates, codes, scales, y, T, D, N, s);
  if (CP == 64) return launch_nf3_grouped<NP, 64>(pos_tok, pos_row, gates, codes, scales, y, T, D, N, s);
  return hipErrorInvalidValue;
}

hipError_t launch_lookup_combine_nf3_grouped(const int* pos_tok, const int* pos_row, const float* gates,
                                             const uint8_t* codes, const uint16_t* scales, float* y, int64_t T,
                                             int64_t D, int64_t N, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int NP = next_pow2((int)N);
  // lanes per expert split: the chunks of a row, at least 64 / NP so that a
  // token fills its wavefront with every split holding an expert
  int CP = pick_group((int)(D / 32), 8, 64);
  while (CP * NP < 64) CP *= 2;
  switch (NP) {
    case 1: return dispatch_nf3_grouped_cp<1>(CP, pos_tok, pos_row, gates, codes, scales, y, T, (int)D, (int)N, s);
    case 2: return dispatch_nf3_grouped_cp<2>(CP, pos_tok, pos_row, gates, codes, scales, y, T, (int)D, (int)N, s);
    case 4: return dispatch_nf3_grouped_cp<4>(CP, pos_tok, pos_row, gates, codes, scales, y, T, (int)D, (int)N, s);
    case 8: return dispatch_nf3_grouped_cp<8>(CP, pos_tok, pos_row, gates, codes, scales, y, T, (int)D, (int)N, s);
    case 16: return dispatch_nf3_grouped_cp<16>(CP, pos_tok, pos_row, gates, codes, scales, y, T, (int)D, (int)N, s);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------
// Host-side dispatch
// ---------------------------------------------------------------------------
// Tokens (wavefronts) per workgroup of the wide launch: 8 where that needs
// no more token slots per compute unit than 4 -- ceil(workgroups / 256 CUs)
// rounds of 8 against rounds of 4 -- else 4.  With 8, each workgroup
// streams W_r's K share once for twice as many tokens (at T = 4096, 16 MB
// of W_r through L2 instead of 32 MB); with 4, a batch that does not fill
// whole rounds of 8-token workgroups leaves fewer CUs idle.  Measured on
// the 410M-class NF3 table, 4 -> 8 tokens: T = 2048 distinct 10.1 -> 9.4
// us, Zipf 10.1 -> 9.0 us; T = 4096 distinct 15.0 -> 14.2 us, Zipf 14.6 ->
// 13.1 us; T = 16384 distinct 48.3 -> 44.0 us; but T = 1024 distinct 7.9 ->
// 8.5 us (128 workgroups for 256 CUs) and T = 3072 distinct 12.5 -> 13.0 us
// (384 workgroups: two rounds where 4 tokens take three of half the size).
static inline int quant_wide_tokens(int64_t T) {
  const int64_t r8 = ((T + 7) / 8 + 255) / 256, r4 = ((T + 3) / 4 + 255) / 256;
  return 8 * r8 <= 4 * r4 ? 8 : 4;
}

template <typename TH, int NP, int CP, int FMT>
static hipError_t launch_nf3(const int64_t* ids, const void* h, const void* w_r, const uint8_t* codes,
                             const void* scales, float* y, int64_t T, int D, int N, hipStream_t s) {
  constexpr int S = 64 / CP < NP ? 64 / CP : NP;  // expert splits per token
  constexpr int G = CP * S;
  // Below T = 1024 (bf16 h, NP <= 16, full-wavefront tokens): one token per
  // workgroup with the vector-unit router, spread over W wavefronts below.
  // From T = 1024 on, four tokens per workgroup (one per wavefront; or
  // eight, see quant_wide_tokens) with the
  // matrix-core router, whose operands go out before the code loads; on the
  // 410M-class table with distinct ids, against the one-token shapes: T =
  // 1024 NF3 9.26 -> 8.51 us, NF4 9.83 -> 9.01 us, int8 10.2 -> 8.3 us;
  // T = 4096 int8 26.4 -> 23.3 us.
  const bool full_wave = G == kWave && sizeof(TH) == 2 && NP <= 16;
  const bool one_token = full_wave && T < 1024;
  const int tpb = one_token ? 1 : (full_wave ? quant_wide_tokens(T) : pick_tokens_per_block(T, G));
  const int64_t blocks = (T + tpb - 1) / tpb;
  // (No staged-router launch here: the extra launch measured slower --
  // 410M-class NF3 table, T=4096: 20.1 -> 22.6 us.)
  // One token per block: the vector-unit router (see LaneRouter).
  if constexpr (sizeof(TH) == 2 && NP <= 16) {
    if (tpb == 1) {
      // Wavefronts per token: doubled (up to 4) while the batch would still
      // have at most two wavefronts per SIMD and every wavefront keeps at
      // least one expert per split.
      int W = 1;
      if constexpr (G == kWave)
        while (W < 4 && 2 * W * S <= NP && T * 2 * W <= 2 * kSimdsPerChip) W *= 2;
#define MOLE_NF3_W(WV)                                                                                     \
  hipLaunchKernelGGL((lookup_combine_nf3_kernel<TH, NP, CP, S, kRouterLane, FMT, WV>), dim3((unsigned)blocks), \
                     dim3(G * WV), 0, s, ids, (const TH*)h, (const TH*)w_r, codes, scales, y, T, D, N, 1)
      if constexpr (G == kWave) {
        if (W == 4) { MOLE_NF3_W(4); return hipGetLastError(); }
        if (W == 2) { MOLE_NF3_W(2); return hipGetLastError(); }
      }
      MOLE_NF3_W(1);
#undef MOLE_NF3_W
      return hipGetLastError();
    }
  }
  if constexpr (G == kWave && sizeof(TH) == 2 && NP <= 16) {
    if (full_wave && tpb == 8) {
      hipLaunchKernelGGL((lookup_combine_nf3_kernel<TH, NP, CP, S, kRouterMfma, FMT, 1, 8 * kWave>),
                         dim3((unsigned)blocks), dim3(G * tpb), 0, s, ids, (const TH*)h, (const TH*)w_r, codes,
                         scales, y, T, D, N, tpb);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((lookup_combine_nf3_kernel<TH, NP, CP, S, kRouterMfma, FMT>), dim3((unsigned)blocks),
                     dim3(G * tpb), 0, s, ids, (const TH*)h, (const TH*)w_r, codes, scales, y, T, D, N, tpb);
  return hipGetLastError();
}

template <typename TH, int NP, int FMT>
static hipError_t dispatch_nf3_cp(int CP, const int64_t* ids, const void* h, const void* w_r,
                                  const uint8_t* codes, const void* scales, float* y, int64_t T,
                                  int D, int N, hipStream_t s) {
  switch (CP) {
    case 8: return launch_nf3<TH, NP, 8, FMT>(ids, h, w_r, codes, scales, y, T, D, N, s);
    case 16: return launch_nf3<TH, NP, 16, FMT>(ids, h, w_r, codes, scales, y, T, D, N, s);
    case 32: return launch_nf3<TH, NP, 32, FMT>(ids, h, w_r, codes, scales, y, T, D, N, s);
    default: return launch_nf3<TH, NP, 64, FMT>(ids, h, w_r, codes, scales, y, T, D, N, s);
  }
}

template <typename TH, int FMT>
static hipError_t dispatch_nf3_np(int NP, int CP, const int64_t* ids, const void* h, const void* w_r,
                                  const uint8_t* codes, const void* scales, float* y, int64_t T,
                                  int D, int N, hipStream_t s) {
  switch (NP) {
    case 1: return dispatch_nf3_cp<TH, 1, FMT>(CP, ids, h, w_r, codes, scales, y, T, D, N, s);
    case 2: return dispatch_nf3_cp<TH, 2, FMT>(CP, ids, h, w_r, codes, scales, y, T, D, N, s);
    case 4: return dispatch_nf3_cp<TH, 4, FMT>(CP, ids, h, w_r, codes, scales, y, T, D, N, s);
    case 8: return dispatch_nf3_cp<TH, 8, FMT>(CP, ids, h, w_r, codes, scales, y, T, D, N, s);
    case 16: return dispatch_nf3_cp<TH, 16, FMT>(CP, ids, h, w_r, codes, scales, y, T, D, N, s);
    case 32: return dispatch_nf3_cp<TH, 32, FMT>(CP, ids, h, w_r, codes, scales, y, T, D, N, s);
    default: return dispatch_nf3_cp<TH, 64, FMT>(CP, ids, h, w_r, codes, scales, y, T, D, N, s);
  }
}

template <int FMT>
static hipError_t launch_q(const int64_t* ids, const void* h, const void* w_r, const uint8_t* codes,
                           const void* scales, float* y, int64_t T, int64_t D, int64_t N, int dtype_h,
                           hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int NP = next_pow2((int)N);
  const int CP = pick_group((int)(D / 32), 8, 64);  // lanes per expert split: chunks of a row
  if (dtype_h == kF32)
    return dispatch_nf3_np<float, FMT>(NP, CP, ids, h, w_r, codes, scales, y, T, (int)D, (int)N, s);
  return dispatch_nf3_np<uint16_t, FMT>(NP, CP, ids, h, w_r, codes, scales, y, T, (int)D, (int)N, s);
}

hipError_t launch_lookup_combine_nf3(const int64_t* ids, const void* h, const void* w_r,
                                     const uint8_t* codes, const uint16_t* scales, float* y,
                                     int64_t T, int64_t D, int64_t N, int dtype_h, hipStream_t s) {
  return launch_q<kFmtNf3>(ids, h, w_r, codes, scales, y, T, D, N, dtype_h, s);
}

hipError_t launch_lookup_combine_q(int fmt, const int64_t* ids, const void* h, const void* w_r,
                                   const uint8_t* codes, const void* scales, float* y, int64_t T, int64_t D,
                                   int64_t N, int dtype_h, hipStream_t s) {
  switch (fmt) {
    case kFmtNf3: return launch_q<kFmtNf3>(ids, h, w_r, codes, scales, y, T, D, N, dtype_h, s);
    case kFmtNf4: return launch_q<kFmtNf4>(ids, h, w_r, codes, scales, y, T, D, N, dtype_h, s);
    case kFmtI8: return launch_q<kFmtI8>(ids, h, w_r, codes, scales, y, T, D, N, dtype_h, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mole
