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
// output tile per workgroup of 4 waves in a 2x2 arrangement, each owning a
// 128x128 sub-tile of v_mfma_f32_32x32x16_bf16 accumulators, or (the build's
// GEMMs) of 8 waves in a 2x4 arrangement with 128x64 sub-tiles.  The
// K loop streams 64-wide slices of A and B through a double-buffered LDS
// ring (row = 128 bytes; 16-byte segment s of row r stored at s ^ ((r/2) & 7):
// the LDS serves 256 bytes (64 banks) per cycle, so the 16 lanes of one
// ds_read_b128 pass -- 16 consecutive rows -- and the 16 lanes of a staging
// write -- 2 rows x 8 segments -- each hit 16 distinct 16-byte bank groups).
// Each thread stages 16 (8) segments per slice in registers; the software
// pipeline writes one staged segment to LDS and at once re-issues its load
// for the slice after next, spread over the MFMAs of a K step, so every
// global load has a full slice of MFMA work to arrive, and the fragments of
// K step s+1 are read from LDS while the MFMAs of step s run.  The order of
// MFMA, LDS and global instructions is pinned with scheduling fences (left
// to itself the compiler sank the loads to the end of the loop, exposing
// their latency every slice).  Operands are read through buffer resources,
// so rows past the matrix edge read zeros and the K loop has no branches.
// Tiles are ordered per GEMM (see tile_of_block).  The GEMM-1 epilogue
// evaluates GELU with a polynomial normal CDF (see gelu_poly); output tiles
// whose rows lie far apart in memory (the LUT, row stride N*D) are staged in
// LDS and written as whole row segments (see EpiMode).
//
// fp32 path (small tables): one workgroup per (v, e) row: stage Emb[v] in
// LDS, each thread forms hidden units u[f] with fp32 FMAs and exact-form
// GELU (erff), then each thread forms output elements from the staged G.
#include <algorithm>

#include "mole_device.hpp"
#include "mole_kernels.hpp"

namespace mole {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// GELU(u) = u * Phi(u) = u/2 * (1 + erf(u / sqrt 2)), with the C library's
// erff (fp32 path).
__device__ __forceinline__ float gelu_erf(float u) { return 0.5f * u * (1.0f + erff(u * 0.70710678118654752f)); }

// Epilogue modes.  Direct: each lane stores 4 consecutive bf16 (8 bytes) of
// one row; the 32 rows of a store instruction are merged into full cache
// lines in L2 when rows are close together.  Staged: the tile goes through
// LDS and each wave writes two whole 512-byte row segments per instruction;
// measured faster once output rows are >= 16 KB apart (the LUT of the larger
// configurations), slower for narrow rows (two extra barriers).
// F32: the fp32 accumulators themselves, 16 bytes per lane (split-K partial
// sums of the MoLE block's down-projection, gradients).  GeluGrad: bf16 of
// acc * GELU'(u) with u read from `aux` at the same position (the backward
// pass of the experts' hidden activation).
// F32Staged: the fp32 tile goes through LDS in four passes of 64 rows, and
// every store writes a quarter of a 1 KB row segment (rows far apart).
// GeluPre: GELU(acc) to C and acc itself (bf16) to `pre`, laid out like C
// (the training forward keeps the pre-activations for the backward pass).
enum {
  kEpiStore = 0, kEpiGelu = 1, kEpiStoreStaged = 2, kEpiF32 = 3, kEpiGeluGrad = 4, kEpiF32Staged = 5,
  kEpiGeluPre = 6
};
constexpr int64_t kStagedMinRowBytes = 16384;

constexpr int kBK = 64;     // K slice per LDS stage (64 bf16 = 128 bytes per row)
constexpr int kPanel = 256; // columns per panel of a panel-major operand (the build's hidden activations)
constexpr int kXcds = 8;    // MI355X: 8 accelerator complex dies, each with its own L2
constexpr int kGroupM = 8;  // row tiles per raster band

struct GemmArgs {
  const uint16_t* A; int64_t lda, sAz;
  const uint16_t* B; int64_t ldb, sBz;
  uint16_t* C; int64_t ldc, sCz;
  int M, N, K;
  int tiles_m, tiles_n, batch;
  int xcd_order;  // 1: XCD-banded tile order, 0: row-major tile order
  const uint16_t* aux;  // GELU-gradient epilogue: bf16 pre-activations, laid out like C
  uint16_t* pre;        // GeluPre epilogue: bf16 pre-activations out, laid out like C
  int64_t a_pstride, c_pstride;  // panel-major A / C: elements from one 256-column panel to the next
};

// Map the hardware workgroup id to an output tile.
//  * xcd_order = 0: row-major over tiles (n fastest).  Concurrent workgroups
//    then cover one or two full rows of tiles: they share the A row panel
//    and write one contiguous stripe of C.  Used for the wide GEMM-1, whose
//    C (the hidden activations, up to several GB) must be written in long
//    runs -- a scattered order made the memory system write every output
//    line several times over.
//  * xcd_order = 1: workgroups go to the XCDs round-robin (id % 8), so
//    consecutive ids land on different L2 caches; renumbering gives each XCD
//    a contiguous run of logical tiles, walked in bands of kGroupM row tiles
//    column by column, so the tiles an XCD runs together share A row panels
//    and B column panels in its L2.  Used for GEMM-2 (narrow N = D).
__device__ __forceinline__ void tile_of_block(const GemmArgs& p, int& z, int& tm, int& tn) {
  const int b = blockIdx.x;
  if (!p.xcd_order) {
    tn = b % p.tiles_n;
    tm = (b / p.tiles_n) % p.tiles_m;
    z = b / (p.tiles_n * p.tiles_m);
    return;
  }
  const int total = p.tiles_m * p.tiles_n * p.batch;
  const int per = total / kXcds, rem = total % kXcds;
  const int xcd = b % kXcds, loc = b / kXcds;
  const int logical = xcd < rem ? xcd * (per + 1) + loc : rem * (per + 1) + (xcd - rem) * per + loc;
  const int per_z = p.tiles_m * p.tiles_n;
  z = logical / per_z;
  const int r = logical - z * per_z;
  const int band = r / (kGroupM * p.tiles_n);
  const int first_m = band * kGroupM;
  const int gm = p.tiles_m - first_m < kGroupM ? p.tiles_m - first_m : kGroupM;
  const int rin = r - band * kGroupM * p.tiles_n;
  tm = first_m + rin % gm;
  tn = rin / gm;
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

__device__ __forceinline__ uint32_t dword_of(const uint4& q, int i) {
  return i == 0 ? q.x : (i == 1 ? q.y : (i == 2 ? q.z : q.w));
}

// C[m][n] = epi( sum_k A[m][k] * B[n][k] ), bf16 in, fp32 accumulation;
// batch index z offsets A, B, C by sAz, sBz, sCz.  Requires N % 8 == 0
// (16-byte output chunks) and, with a K-contiguous operand, K % 8 == 0
// (16-byte K segments); an MN-major operand needs its M (or N) extent, ld
// and batch offset to be multiples of 8 and 63 * ld + 256 < 2^30.
template <int BM, int BN, int EPI, int OPS = kOpsKK, int NW = 4>
__global__ __launch_bounds__(NW * 64) void gemm_nt_bf16_kernel(GemmArgs p) {
  constexpr int NT = NW * 64;                 // threads
  constexpr int WGN = NW / 2;                 // waves along N (two along M)
  constexpr int WM = BM / 2, WN = BN / WGN;   // wave sub-tile
  constexpr int TM = WM / 32, TN = WN / 32;   // MFMA tiles per wave
  constexpr int SA = BM * 8 / NT, SB = BN * 8 / NT;  // 16-byte segments per thread
  constexpr int NS = SA + SB;                 // staging slots per thread
  constexpr int SPK = NS / 4;                 // slots written and re-loaded per K step
  constexpr int KS = kBK / 16;                // MFMA K steps per LDS stage
  // Four waves: 4x4 MFMA tiles per wave and 16 slots; eight waves (two per
  // SIMD): 4x2 tiles and 8 slots.  Either way one slot is handled after
  // every fourth MFMA of a K step, SPK per step.
  static_assert(KS == 4 && TM == 4 && TM * TN == 4 * SPK && (NW == 4 || NW == 8),
                "the software pipeline below is written for 4 K steps and one slot per 4 MFMAs");
  static_assert(NW == 4 || ((OPS & (kOpsAmn | kOpsBmn)) == 0 && EPI != kEpiF32Staged),
                "eight waves: K-contiguous operands and the direct or bf16-staged epilogues only");
  constexpr int kRing = (BM + BN) * 8;        // uint4 per LDS stage
  constexpr int kCPitch = BN / 8 + 1;         // staged output row pitch in uint4 (16-byte pad)
  constexpr int kLds = (EPI == kEpiStoreStaged && BM * kCPitch > 2 * kRing) ? BM * kCPitch : 2 * kRing;
  __shared__ uint4 lds[kLds];
  auto smem = reinterpret_cast<uint4(*)[kRing]>(lds);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  int z, tm, tn;
  tile_of_block(p, z, tm, tn);
  const int M = p.M, N = p.N, K = p.K;
  const int m0 = tm * BM, n0 = tn * BN;
  const int rows_a = M - m0 < BM ? M - m0 : BM;
  const int rows_b = N - n0 < BN ? N - n0 : BN;
  // Buffer resources over this tile's A and B row panels: a load past the
  // panel (a row beyond M or N) returns zeros without a branch.
  // Panel-major A: element (m, k) at A + (k / 256) * a_pstride + m * 256 + k % 256; the resource spans
  // the tile's rows in every panel the K range touches.
  constexpr bool kApanel = (OPS & kOpsApanel) != 0, kCpanel = (OPS & kOpsCpanel) != 0;
  const __amdgpu_buffer_rsrc_t ra_rs =
      kApanel ? __builtin_amdgcn_make_buffer_rsrc(
                    (void*)(p.A + z * p.sAz + (int64_t)m0 * kPanel), (short)0,
                    (int)(((K - 1) / kPanel) * p.a_pstride * 2 + (int64_t)rows_a * kPanel * 2), kRsrcWord3)
              : __builtin_amdgcn_make_buffer_rsrc((void*)(p.A + z * p.sAz + (int64_t)m0 * p.lda), (short)0,
                                                  (int)(rows_a * p.lda * 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rb_rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.B + z * p.sBz + (int64_t)n0 * p.ldb), (short)0, (int)(rows_b * p.ldb * 2), kRsrcWord3);

  // Staging slot s (0..15) of thread t, K-contiguous operand: 16-byte
  // segment (t & 7) of A row t/8 + 32 s (s < 8) or of B row t/8 + 32 (s - 8).
  // MN-major operand: slots in groups of four, group g (slots 4g .. 4g+3 of
  // the operand) holds k rows 4 kq .. 4 kq + 3 of the slice, kq = (t & 7) +
  // 8 (g % 2), at MN columns 8 (t/8) .. 8 (t/8) + 7; the group is transposed
  // in registers just before it goes to LDS, so both storages leave the same
  // LDS layout: row = M (or N) index, 64 k per row in 16-byte segments.
  const int seg = tid & 7;
  const int srow = tid >> 3;
  const int pseg = seg ^ ((srow >> 1) & 7);  // XOR swizzle ((row >> 1) & 7 is the same for all slots)
  auto is_mn = [](int s) { return s < SA ? (OPS & kOpsAmn) != 0 : (OPS & kOpsBmn) != 0; };
  uint32_t off[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const bool is_a = s < SA;
    const int idx = is_a ? s : s - SA;
    const int lim = is_a ? rows_a : rows_b;
    const int64_t ld = is_a ? p.lda : p.ldb;
    if (is_mn(s)) {
      const int kr = 4 * (seg + 8 * ((idx >> 2) & 1)) + (idx & 3);  // k row within the slice
      off[s] = (uint32_t)((kr * ld + srow * 8) * 2);
    } else {
      const int row = srow + (NT / 8) * idx;
      const int64_t pitch = (is_a && kApanel) ? kPanel : ld;
      off[s] = row < lim ? (uint32_t)(row * pitch * 2 + seg * 16) : kOob;
    }
  }
  // MN-major operand: a buffer resource over the slice's k rows, clipped to
  // the K rows left and, in the last row, to the tile's MN extent (reads
  // past it return zeros; in earlier rows they only feed output rows or
  // columns that are never stored).
  // (Branch-free: a slice past K gets zero records; its base is never read.)
  const uint16_t* mn_base_a = p.A + z * p.sAz + m0;
  const uint16_t* mn_base_b = p.B + z * p.sBz + n0;
  const int ld_a = (int)p.lda, ld_b = (int)p.ldb;
  // The values are uniform; readfirstlane keeps them in scalar registers
  // (otherwise the compiler wraps each load in a loop over distinct
  // descriptors).
  auto mn_rsrc = [&](bool is_a, int slice) {
    const int k0 = slice * kBK;
    const int ld = is_a ? ld_a : ld_b;
    const int kr = max(0, min(kBK, K - k0));  // k rows of the slice that exist
    const int nrec = __builtin_amdgcn_readfirstlane(max(0, (kr - 1) * ld + (is_a ? rows_a : rows_b)) * 2);
    const uint64_t addr = reinterpret_cast<uint64_t>((is_a ? mn_base_a : mn_base_b) + (int64_t)k0 * ld);
    const uint64_t base = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(addr >> 32)) << 32) |
                          (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)addr);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(base), (short)0, nrec, kRsrcWord3);
  };
  uint4 rs[NS];
  // Load slot s of K slice `slice` (past K: zeros).
  auto lslot = [&](int s, int slice) {
    if (is_mn(s)) {
      rs[s] = buf_load16(mn_rsrc(s < SA, slice), off[s]);
    } else {
      const int k0 = slice * kBK;
      const uint32_t kofs = (s < SA && kApanel)
                                ? (uint32_t)((k0 / kPanel) * p.a_pstride * 2 + (k0 % kPanel) * 2)
                                : (uint32_t)k0 * 2u;
      // (a row past the tile has off = kOob; kOob + kofs stays below 2^32 and past every record)
      const uint32_t o = (k0 + seg * 8 < K) ? off[s] + kofs : kOob;
      rs[s] = buf_load16(s < SA ? ra_rs : rb_rs, o);
    }
  };
  // MN-major group at slots s0 .. s0+3 (4 k rows of 8 MN values each) ->
  // 8 MN rows of 4 k values: slot s0 + q then holds MN rows 2q and 2q + 1.
  auto transpose_group = [&](int s0) {
    if (!is_mn(s0)) return;
    uint4 t[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t w[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = 2 * q + h;  // MN index within the block
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const uint32_t lo = dword_of(rs[s0 + 2 * pr], c >> 1), hi = dword_of(rs[s0 + 2 * pr + 1], c >> 1);
          // one byte permute: half (c & 1) of lo below the same half of hi
          w[2 * h + pr] = __builtin_amdgcn_perm(hi, lo, (c & 1) ? 0x07060302u : 0x05040100u);
        }
      }
      t[q] = make_uint4(w[0], w[1], w[2], w[3]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) rs[s0 + q] = t[q];
  };
  // Write slot s into LDS stage st.
  auto wslot = [&](int s, int st) {
    const bool is_a = s < SA;
    const int idx = is_a ? s : s - SA;
    if (is_mn(s)) {
      const int kq = seg + 8 * ((idx >> 2) & 1);
      uint2* sm2 = reinterpret_cast<uint2*>(smem[st]);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = srow * 8 + 2 * (idx & 3) + h;  // MN index within the tile
        const int at = ((is_a ? 0 : BM) + row) * 8 + ((kq >> 1) ^ ((row >> 1) & 7));
        sm2[at * 2 + (kq & 1)] = h ? make_uint2(rs[s].z, rs[s].w) : make_uint2(rs[s].x, rs[s].y);
      }
    } else {
      const int row = (is_a ? 0 : BM) + srow + (NT / 8) * idx;
      smem[st][row * 8 + pseg] = rs[s];
    }
  };
  // Fragments of one 16-wide K step: lane l reads row l%32 of each 32-row
  // MFMA tile, 8 consecutive k at 8*(l/32) (swizzled segment).
  auto fload = [&](int st, int ks, uint4* a, uint4* b) {
    const int sg = 2 * ks + (lane >> 5);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = wm * WM + i * 32 + (lane & 31);
      a[i] = smem[st][r * 8 + (sg ^ ((r >> 1) & 7))];
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int r = wn * WN + j * 32 + (lane & 31);
      b[j] = smem[st][(BM + r) * 8 + (sg ^ ((r >> 1) & 7))];
    }
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // The 16 MFMAs of one K step.  Operands swapped (B tile as the
  // matrix-core "A"): lane l then holds C[m = l%32][n = 8*(r/4) + 4*(l/32) +
  // r%4] in accumulator r, i.e. four consecutive n per group of four
  // registers.  After MFMAs 1, 5, 9 and 13, staging slot s0 + q goes to LDS
  // stage wst and is re-loaded from K slice `slice`.
  auto mfma_step = [&](const uint4* a, const uint4* b, int s0, int wst, int slice) {
#pragma unroll
    for (int x = 0; x < TM * TN; ++x) {
      const int i = x / TN, j = x % TN;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, b[j]),
                                                           __builtin_bit_cast(bf16x8_t, a[i]), acc[i][j], 0, 0, 0);
      if (x == 1) transpose_group(s0);
      if (x % 4 == 1) {
        wslot(s0 + x / 4, wst);
        lslot(s0 + x / 4, slice);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Pipeline invariant at the top of iteration kt (cur = kt & 1): LDS stage
  // cur holds slice kt; LDS stage cur^1 holds slots 0-3 of slice kt+1; the
  // registers of slots 4-15 hold (or are loading) slice kt+1 and those of
  // slots 0-3 slice kt+2; fa[0]/fb[0] hold K step 0 of slice kt.  Slots
  // 4-15 of slice kt+1 are written during K steps 0-2 (stage cur^1 was last
  // read before the previous barrier); after the barrier, K step 3 writes
  // slots 0-3 of slice kt+2 into stage cur, which every wave has finished
  // reading.
  const int nk = (K + kBK - 1) / kBK;
#pragma unroll
  for (int s = 0; s < NS; ++s) lslot(s, 0);
#pragma unroll
  for (int s0 = 0; s0 < NS; s0 += 4) transpose_group(s0);
#pragma unroll
  for (int s = 0; s < NS; ++s) wslot(s, 0);
#pragma unroll
  for (int s = 0; s < NS; ++s) lslot(s, 1);
  transpose_group(0);
#pragma unroll
  for (int s = 0; s < SPK; ++s) {
    wslot(s, 1);
    lslot(s, 2);
  }
  __syncthreads();
  uint4 fa[2][TM], fb[2][TN];
  fload(0, 0, fa[0], fb[0]);
  __builtin_amdgcn_sched_barrier(0);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    fload(cur, 1, fa[1], fb[1]);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(fa[0], fb[0], SPK, cur ^ 1, kt + 2);
    fload(cur, 2, fa[0], fb[0]);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(fa[1], fb[1], 2 * SPK, cur ^ 1, kt + 2);
    fload(cur, 3, fa[1], fb[1]);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(fa[0], fb[0], 3 * SPK, cur ^ 1, kt + 2);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    fload(cur ^ 1, 0, fa[0], fb[0]);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(fa[1], fb[1], 0, cur, kt + 3);
  }

  const int rows_c = M - m0 < BM ? M - m0 : BM;
  // Panel-major C (the tile is one 256-column panel): the tile's rows are a
  // contiguous run of 512-byte rows at C + (n0 / 256) * c_pstride + m0 * 256.
  static_assert(!kCpanel || (BN == kPanel && (EPI == kEpiGelu || EPI == kEpiStore)),
                "panel-major C: one panel per tile, direct bf16 epilogue");
  const int64_t ldc_t = kCpanel ? kPanel : p.ldc;  // row pitch of the tile's C rows
  const int ncol0 = kCpanel ? n0 : 0;              // column of the tile's C base
  const __amdgpu_buffer_rsrc_t rc_rs = __builtin_amdgcn_make_buffer_rsrc(
      kCpanel ? (void*)(p.C + z * p.sCz + (int64_t)(n0 / kPanel) * p.c_pstride + (int64_t)m0 * kPanel)
              : (void*)(p.C + z * p.sCz + (int64_t)m0 * p.ldc),
      (short)0, (int)(rows_c * ldc_t * 2), kRsrcWord3);
  // GELU-gradient epilogue: the u values of one row block of accumulators
  // (4 consecutive columns per group, 8 bytes) are loaded while the
  // previous block is stored; loading them between stores instead made
  // every wait for u also wait for the earlier stores (one counter).
  uint2 ub[2][EPI == kEpiGeluGrad ? TN : 1][4];
  __amdgpu_buffer_rsrc_t ru_rs = rc_rs;
  if constexpr (EPI == kEpiGeluGrad)
    ru_rs = __builtin_amdgcn_make_buffer_rsrc((void*)(p.aux + z * p.sCz + (int64_t)m0 * p.ldc), (short)0,
                                              (int)(rows_c * p.ldc * 2), kRsrcWord3);
  auto aux_load = [&](int i, uint2 (*dst)[4]) {
    const int mr = wm * WM + i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * WN + j * 32 + 8 * g + 4 * (lane >> 5);
        const uint32_t o = (mr < rows_c && n < N) ? (uint32_t)(mr * p.ldc * 2 + n * 2) : kOob;
        dst[j][g] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(ru_rs, (int)o, 0, 0));
      }
  };
  // (GELU or its gradient,) round to bf16, pack 4 consecutive columns into 8 bytes.
  auto packed = [&](int i, int j, int g, bool raw = false) {
    float v[4];
    if constexpr (EPI == kEpiGeluGrad) {
      // u at the same (row, column) as this accumulator group
      const uint2 uw = ub[i & 1][j][g];
      const float uv[4] = {bf16_lo(uw.x), bf16_hi(uw.x), bf16_lo(uw.y), bf16_hi(uw.y)};
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = acc[i][j][4 * g + q] * gelu_grad_poly(uv[q]);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[q] = acc[i][j][4 * g + q];
        if constexpr (EPI == kEpiGelu || EPI == kEpiGeluPre)
          if (!raw) v[q] = gelu_poly(v[q]);
      }
    }
    const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)v[0]) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[1]) << 16);
    const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)v[2]) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[3]) << 16);
    return make_uint2(lo, hi);
  };
  if constexpr (EPI == kEpiF32Staged) {
    static_assert(BM == 256 && BN == 256, "four 64-row passes of a 256-column tile");
    float* cf = reinterpret_cast<float*>(p.C) + z * p.sCz + (int64_t)m0 * p.ldc;
    const __amdgpu_buffer_rsrc_t rf_rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)cf, (short)0, (int)(rows_c * p.ldc * 4), kRsrcWord3);
    constexpr int kPitch = BN + 4;  // floats per staged row (16-byte pad: conflict-free float4 writes)
    float* cs = reinterpret_cast<float*>(lds);
    __syncthreads();  // every wave is done with the operand ring
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      // rows [64 pass, 64 pass + 64) belong to the waves with wm = pass / 2, MFMA rows i = 2 (pass % 2) + 0, 1
      if (wm == pass / 2) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
          const int i = 2 * (pass % 2) + ii;
          const int lr = ii * 32 + (lane & 31);  // row within the pass
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int nc = wn * WN + j * 32 + 8 * g + 4 * (lane >> 5);
              *reinterpret_cast<float4*>(cs + lr * kPitch + nc) =
                  make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
            }
        }
      }
      __syncthreads();
      const int c4 = tid & 63;  // 16-byte column group of the row
#pragma unroll 4
      for (int k = 0; k < 16; ++k) {
        const int lr = (tid >> 6) + 4 * k;
        const int row = 64 * pass + lr, n = n0 + 4 * c4;
        const float4 v = *reinterpret_cast<const float4*>(cs + lr * kPitch + 4 * c4);
        const uint32_t o = (row < rows_c && n < N) ? (uint32_t)((row * p.ldc + n) * 4) : kOob;
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v), rf_rs, (int)o, 0, 0);
      }
      __syncthreads();
    }
  } else if constexpr (EPI == kEpiF32) {
    // fp32 tile rows (buffer resource over rows_c rows of ldc floats).
    float* cf = reinterpret_cast<float*>(p.C) + z * p.sCz + (int64_t)m0 * p.ldc;
    const __amdgpu_buffer_rsrc_t rf_rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)cf, (short)0, (int)(rows_c * p.ldc * 4), kRsrcWord3);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int mr = wm * WM + i * 32 + (lane & 31);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * WN + j * 32 + 8 * g + 4 * (lane >> 5);
          const uint32_t o = (mr < rows_c && n < N) ? (uint32_t)((mr * p.ldc + n) * 4) : kOob;
          const uint4 v = make_uint4(__float_as_uint(acc[i][j][4 * g]), __float_as_uint(acc[i][j][4 * g + 1]),
                                     __float_as_uint(acc[i][j][4 * g + 2]), __float_as_uint(acc[i][j][4 * g + 3]));
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v),
                                                 rf_rs, (int)o, 0, 0);
        }
      }
    }
  } else if constexpr (EPI != kEpiStoreStaged) {
    // Direct: 8-byte stores through a buffer resource over this tile's rows
    // (rows past M and column groups past N take an out-of-range offset and
    // are dropped).
    __amdgpu_buffer_rsrc_t rp_rs = rc_rs;
    if constexpr (EPI == kEpiGeluPre)
      rp_rs = __builtin_amdgcn_make_buffer_rsrc((void*)(p.pre + z * p.sCz + (int64_t)m0 * p.ldc), (short)0,
                                                (int)(rows_c * p.ldc * 2), kRsrcWord3);
    if constexpr (EPI == kEpiGeluGrad) aux_load(0, ub[0]);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if constexpr (EPI == kEpiGeluGrad) {
        if (i + 1 < TM) aux_load(i + 1, ub[(i + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
      const int mr = wm * WM + i * 32 + (lane & 31);  // row within the tile
#pragma unroll
      for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * WN + j * 32 + 8 * g + 4 * (lane >> 5);
          const uint32_t o = (mr < rows_c && n < N) ? (uint32_t)(mr * ldc_t * 2 + (n - ncol0) * 2) : kOob;
          __builtin_amdgcn_raw_buffer_store_b64(
              __builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned int, packed(i, j, g)), rc_rs, (int)o,
              0, 0);
          if constexpr (EPI == kEpiGeluPre)
            __builtin_amdgcn_raw_buffer_store_b64(
                __builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned int, packed(i, j, g, true)), rp_rs,
                (int)o, 0, 0);
        }
      }
    }
  } else {
    // Staged: the tile goes to LDS (row pitch BN*2 + 16 bytes), then each
    // wave writes two whole tile rows per 16-byte store instruction.
    __syncthreads();  // every wave is done with the operand ring
    uint32_t* cs = reinterpret_cast<uint32_t*>(lds);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int mr = wm * WM + i * 32 + (lane & 31);
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int nc = wn * WN + j * 32 + 8 * g + 4 * (lane >> 5);
          *reinterpret_cast<uint2*>(cs + mr * (kCPitch * 4) + nc / 2) = packed(i, j, g);
        }
    }
    __syncthreads();
    constexpr int kChunks = BN / 8;  // 16-byte chunks per tile row
    constexpr int kRowsPerPass = NT / kChunks;
    const int ch = tid % kChunks;
    const int n = n0 + ch * 8;
#pragma unroll 4
    for (int r0 = 0; r0 < BM; r0 += kRowsPerPass) {
      const int row = r0 + tid / kChunks;
      const uint4 d = lds[row * kCPitch + ch];
      const uint32_t o = (row < rows_c && n < N) ? (uint32_t)(row * p.ldc * 2 + n * 2) : kOob;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, d),
                                             rc_rs, (int)o, 0, 0);
    }
  }
}

template <int BM, int BN, int EPI, int OPS = kOpsKK, int NW = 4>
static hipError_t launch_gemm(const uint16_t* A, int64_t lda, int64_t sAz, const uint16_t* B, int64_t ldb,
                              int64_t sBz, uint16_t* C, int64_t ldc, int64_t sCz, int M, int N, int K,
                              int batch, int xcd_order, hipStream_t s, const uint16_t* aux = nullptr,
                              uint16_t* pre = nullptr, int64_t a_pstride = 0, int64_t c_pstride = 0) {
  GemmArgs p{A, lda, sAz, B, ldb, sBz, C, ldc, sCz, M, N, K, (M + BM - 1) / BM, (N + BN - 1) / BN, batch,
             xcd_order, aux, pre, a_pstride, c_pstride};
  const int64_t total = (int64_t)p.tiles_m * p.tiles_n * batch;
  hipLaunchKernelGGL((gemm_nt_bf16_kernel<BM, BN, EPI, OPS, NW>), dim3((unsigned)total), dim3(NW * 64), 0, s, p);
  return hipGetLastError();
}

constexpr int kBM = kBuildTileM, kBN = 256;

size_t build_lut_min_workspace(int64_t D, int64_t F, int64_t N) {
  (void)D;
  return (size_t)kBM * (size_t)(N * F) * 2u;
}

size_t build_lut_rec_workspace(int64_t V, int64_t D, int64_t F, int64_t N) {
  (void)D;
  const size_t row_bytes = (size_t)(N * F) * 2u;
  // About 1 GB of hidden activations per block: each block re-reads both
  // weight tensors, so larger blocks cut that traffic (1B-class layer, one
  // build: 1024-row blocks 48.5 ms, 4096 rows 47.7 ms; 160M-class: 2.33 ->
  // 2.16 ms), while blocks of a few GB gain nothing more.
  const size_t target = (size_t)1 << 30;
  int64_t rows = (int64_t)(target / row_bytes) / kBM * kBM;
  if (rows < kBM) rows = kBM;
  const int64_t vpad = (V + kBM - 1) / kBM * kBM;
  if (rows > vpad) rows = vpad;
  return (size_t)rows * row_bytes;
}

// Tile order of GEMM-1 when its output is panel-major: the panels make every
// output tile one contiguous 128 KB run whatever the order, so the order can
// serve operand reuse (XCD bands: each XCD's concurrent tiles share W_up
// column panels in its L2).
constexpr int kGemm1PanelOrder = 1;

// Waves per workgroup of the build's two GEMMs: eight, two per SIMD, so that
// one wave's matrix instructions issue while the other waits at the slice
// barrier or for its LDS fragments (the 256x256 tile, the LDS ring and the
// order of every accumulation are those of the four-wave form, so the
// tables are bit-identical).  Measured on 1B-class builds: 47.7 -> 46.1 ms
// and 50.2 -> 49.0 ms (two boxes; GEMM-2 1769 -> 1713 us and GEMM-1 2152 ->
// 2133 us per 4096-row block); 160M-class 2.20 -> 2.03 ms.
constexpr int kBuildWaves1 = 8, kBuildWaves2 = 8;

hipError_t launch_build_lut_bf16(const uint16_t* emb, const uint16_t* w_up, const uint16_t* w_down,
                                 uint16_t* lut, int64_t V, int64_t D, int64_t F, int64_t N,
                                 void* ws, size_t ws_bytes, hipStream_t s, uint16_t* pre) {
  const int64_t NF = N * F;
  const int64_t row_bytes = NF * 2;
  // Hidden activations G of a block of vc vocabulary rows.  Panel-major
  // (256-column panels, [N*F/256][vc][256]) when F is a whole number of
  // panels: GEMM-1 then writes each output tile as one contiguous run and
  // GEMM-2 reads expert e's K range from panels e*F/256 .. (e+1)*F/256 - 1.
  // Row-major [vc][N*F] otherwise (and for the training forward, which keeps
  // G and the pre-activations for its backward pass).
  const bool panel = pre == nullptr && F % kPanel == 0;
  // Vocabulary rows per block: all of V when the workspace holds them,
  // otherwise a whole number of row tiles; panel-major blocks keep an
  // expert's K range under 2^31 bytes (32-bit buffer offsets).
  int64_t vc = (int64_t)(ws_bytes / (size_t)row_bytes);
  if (panel) vc = std::min<int64_t>(vc, ((int64_t)1 << 30) / F / kBM * kBM);
  if (vc >= V) vc = V;
  else vc = vc / kBM * kBM;
  uint16_t* G = static_cast<uint16_t*>(ws);
  const int64_t pstride = vc * kPanel;  // elements from one panel of G to the next
  for (int64_t v0 = 0; v0 < V; v0 += vc) {
    const int64_t mc = (V - v0 < vc) ? (V - v0) : vc;
    hipError_t err;
    if (pre)
      err = launch_gemm<kBM, kBN, kEpiGeluPre>(emb + v0 * D, D, 0, w_up, D, 0, G, NF, 0, (int)mc, (int)NF, (int)D, 1,
                                               /*xcd_order=*/0, s, nullptr, pre + v0 * NF);
    else if (panel)
      err = launch_gemm<kBM, kBN, kEpiGelu, kOpsCpanel, kBuildWaves1>(emb + v0 * D, D, 0, w_up, D, 0, G, kPanel, 0, (int)mc,
                                                        (int)NF, (int)D, 1, kGemm1PanelOrder, s, nullptr, nullptr,
                                                        0, pstride);
    else
      err = launch_gemm<kBM, kBN, kEpiGelu>(emb + v0 * D, D, 0, w_up, D, 0, G, NF, 0, (int)mc, (int)NF, (int)D, 1,
                                            /*xcd_order=*/0, s);
    if (err != hipSuccess) return err;
    const bool staged = N * D * 2 >= kStagedMinRowBytes;
    if (panel && staged)
      err = launch_gemm<kBM, kBN, kEpiStoreStaged, kOpsApanel, kBuildWaves2>(G, kPanel, (F / kPanel) * pstride, w_down, F, D * F,
                                                               lut + v0 * N * D, N * D, D, (int)mc, (int)D, (int)F,
                                                               (int)N, /*xcd_order=*/1, s, nullptr, nullptr, pstride);
    else if (panel)
      err = launch_gemm<kBM, kBN, kEpiStore, kOpsApanel, kBuildWaves2>(G, kPanel, (F / kPanel) * pstride, w_down, F, D * F,
                                                         lut + v0 * N * D, N * D, D, (int)mc, (int)D, (int)F, (int)N,
                                                         /*xcd_order=*/1, s, nullptr, nullptr, pstride);
    else if (staged)
      err = launch_gemm<kBM, kBN, kEpiStoreStaged>(G, NF, F, w_down, F, D * F, lut + v0 * N * D, N * D, D,
                                                   (int)mc, (int)D, (int)F, (int)N, /*xcd_order=*/1, s);
    else
      err = launch_gemm<kBM, kBN, kEpiStore>(G, NF, F, w_down, F, D * F, lut + v0 * N * D, N * D, D,
                                             (int)mc, (int)D, (int)F, (int)N, /*xcd_order=*/1, s);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

// GELU(A . B^T) rounded to bf16, one 256x256 tile per workgroup (the
// shared-expert up-projection of the MoLE block uses it for long batches).
hipError_t launch_gemm_gelu_bf16(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, uint16_t* C,
                                 int64_t ldc, int M, int N, int K, hipStream_t s) {
  return launch_gemm<kBM, kBN, kEpiGelu, kOpsKK, kBuildWaves1>(A, lda, 0, B, ldb, 0, C, ldc, 0, M, N, K, 1,
                                                              /*xcd_order=*/0, s);
}

// Whether an MN-major operand fits the kernel's 32-bit slice offsets and
// 16-byte loads (see the kernel's requirements).
static bool mn_operand_ok(int64_t ld, int64_t sz, int64_t extent) {
  return ld % 8 == 0 && sz % 8 == 0 && extent % 8 == 0 && 63 * ld + 256 < ((int64_t)1 << 30);
}

static bool ops_ok(int ops, int64_t lda, int64_t sAz, int M, int64_t ldb, int64_t sBz, int N, int K) {
  if ((ops & kOpsAmn) && !mn_operand_ok(lda, sAz, M)) return false;
  if ((ops & kOpsBmn) && !mn_operand_ok(ldb, sBz, N)) return false;
  if (ops != kOpsMnMn && K % 8 != 0) return false;  // a K-contiguous operand reads 16-byte K segments
  return N % 8 == 0;
}

// bf16 C = (A . B^T) * GELU'(aux) per batch index z, aux laid out like C
// (the gradient through the experts' hidden activation); B MN-major.
hipError_t launch_gemm_gelu_grad_bf16(const uint16_t* A, int64_t lda, int64_t sAz, const uint16_t* B, int64_t ldb,
                                      int64_t sBz, uint16_t* C, int64_t ldc, int64_t sCz, const uint16_t* aux, int M,
                                      int N, int K, int batch, hipStream_t s) {
  if (!ops_ok(kOpsBmn, lda, sAz, M, ldb, sBz, N, K)) return hipErrorInvalidValue;
  // Row-major tile order: measured 5-10 % faster than the XCD-banded order
  // on the 1B-class shape (U = 465, F = 8192, D = 2048), even on 410M-class.
  return launch_gemm<kBM, kBN, kEpiGeluGrad, kOpsBmn>(A, lda, sAz, B, ldb, sBz, C, ldc, sCz, M, N, K, batch,
                                                      /*xcd_order=*/0, s, aux);
}

template <int OPS>
static hipError_t launch_f32(const uint16_t* A, int64_t lda, int64_t sAz, const uint16_t* B, int64_t ldb, int64_t sBz,
                             float* C, int64_t ldc, int64_t sCz, int M, int N, int K, int batch, hipStream_t s) {
  // Rows 16 KB or more apart: stage through LDS and write whole row segments.
  if (ldc * 4 >= kStagedMinRowBytes)
    return launch_gemm<kBM, kBN, kEpiF32Staged, OPS>(A, lda, sAz, B, ldb, sBz, reinterpret_cast<uint16_t*>(C), ldc,
                                                     sCz, M, N, K, batch, /*xcd_order=*/1, s);
  return launch_gemm<kBM, kBN, kEpiF32, OPS>(A, lda, sAz, B, ldb, sBz, reinterpret_cast<uint16_t*>(C), ldc, sCz, M,
                                             N, K, batch, /*xcd_order=*/1, s);
}

// fp32 C = A . B^T per batch index z (split-K partial sums of the MoLE
// block's down-projection: z selects a K range through sAz and sBz; the
// training gradients, with MN-major operands).  C rows of ldc floats; needs
// 256 * ldc * 4 < 2^31.
hipError_t launch_gemm_f32_bf16(const uint16_t* A, int64_t lda, int64_t sAz, const uint16_t* B, int64_t ldb,
                                int64_t sBz, float* C, int64_t ldc, int64_t sCz, int M, int N, int K, int batch,
                                hipStream_t s, int ops) {
  if (!ops_ok(ops, lda, sAz, M, ldb, sBz, N, K)) return hipErrorInvalidValue;
  switch (ops) {
    case kOpsKK: return launch_f32<kOpsKK>(A, lda, sAz, B, ldb, sBz, C, ldc, sCz, M, N, K, batch, s);
    case kOpsBmn: return launch_f32<kOpsBmn>(A, lda, sAz, B, ldb, sBz, C, ldc, sCz, M, N, K, batch, s);
    case kOpsMnMn: return launch_f32<kOpsMnMn>(A, lda, sAz, B, ldb, sBz, C, ldc, sCz, M, N, K, batch, s);
    default: return hipErrorInvalidValue;
  }
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
