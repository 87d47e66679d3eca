// Lookup-combine over a batch grouped by distinct id (MoLE article,
// inference section: each token's expert outputs are fetched by token id;
// a prefill batch repeats ids -- Zipf-distributed text puts a few hundred
// tokens on the commonest ids -- and every token of one id reads the same
// N x D table slab).
//
// The host index (the tokens grouped by distinct id, tok, and the table
// row of each grouped position, rows) lets each slab be read once per run
// of equal ids instead of once per token:
//   * router_gates_kernel routes every token (16 per block, on the matrix
//     cores) and leaves its N gates at the head of its output row;
//   * a workgroup owns `seg` consecutive positions of the grouped token
//     list; it stages their gates in LDS (before any row is overwritten --
//     every token's row belongs to exactly one workgroup), then walks the
//     runs of equal ids: the run's slab is loaded once (8 columns per lane,
//     16-byte loads, N registers of 16 bytes) while the previous run is
//     combined, and every token of the run is written from registers.
// A row cut by a chunk boundary is loaded once per chunk it touches.
#include "combine_common.hpp"

namespace mole {

namespace {

constexpr int kGroupedThreads = 128;  // 8 columns per lane: 1024 columns per workgroup
constexpr int kMaxSegG = 64;

template <int NP>
__global__ __launch_bounds__(kGroupedThreads) void lookup_combine_grouped_kernel(
    const int64_t* __restrict__ rows, const int64_t* __restrict__ tok, const uint16_t* __restrict__ lut, float* y,
    int64_t T, int D, int N, int seg) {
  __shared__ float gs[kMaxSegG][NP];
  __shared__ int64_t ts[kMaxSegG], rowv[kMaxSegG];
  __shared__ int runs[kMaxSegG + 1];
  __shared__ int nruns_s;
  const int64_t p0 = (int64_t)blockIdx.x * seg;
  const int len = (int)(T - p0 < seg ? T - p0 : seg);
  const int tid = threadIdx.x;
  if (tid < len) {
    ts[tid] = tok[p0 + tid];
    rowv[tid] = rows[p0 + tid];
  }
  __syncthreads();
  if (tid == 0) {
    int n = 0;
    for (int q = 0; q < len; ++q)
      if (q == 0 || rowv[q] != rowv[q - 1]) runs[n++] = q;
    runs[n] = len;
    nruns_s = n;
  }
  // The first run's slab is requested before the gates are staged.
  const int c0 = (blockIdx.y * kGroupedThreads + tid) * 8;
  const int cc = c0 < D ? c0 : 0;  // an idle lane loads from column 0 and stores nothing
  uint4 sa[NP], sb[NP];
  {
    const uint16_t* base = lut + rowv[0] * (int64_t)N * D + cc;
#pragma unroll
    for (int e = 0; e < NP; ++e) sa[e] = ldg16(base + (int64_t)(e < N ? e : 0) * D);
  }
  for (int i = tid; i < len * NP; i += kGroupedThreads) {
    const int q = i / NP, e = i - (i / NP) * NP;
    gs[q][e] = e < N ? y[ts[q] * D + e] : 0.f;  // the router's gates at the head of the row
  }
  __syncthreads();
  const int nruns = nruns_s;
  if (c0 >= D) return;  // (no barrier follows)
  // Slab of run r (clamped to the last run, so the loads are unconditional).
  auto load_slab = [&](int r, uint4* S) {
    const int rr = r < nruns ? r : nruns - 1;
    const uint16_t* base = lut + rowv[runs[rr]] * (int64_t)N * D + c0;
#pragma unroll
    for (int e = 0; e < NP; ++e) S[e] = ldg16(base + (int64_t)(e < N ? e : 0) * D);
  };
  auto combine_run = [&](int r, const uint4* S) {
    for (int q = runs[r]; q < runs[r + 1]; ++q) {
      float acc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
      for (int e = 0; e < NP; ++e) {
        if (e < N) {
          float v[8];
          Elem<uint16_t>::unpack(S[e], v);
          const float g = gs[q][e];
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(g, v[i], acc[i]);
        }
      }
      float* yo = y + ts[q] * D + c0;
      stg16_nt(yo, acc[0], acc[1], acc[2], acc[3]);
      stg16_nt(yo + 4, acc[4], acc[5], acc[6], acc[7]);
    }
  };
  for (int r = 0; r < nruns; r += 2) {
    load_slab(r + 1, sb);
    combine_run(r, sa);
    load_slab(r + 2, sa);
    if (r + 1 < nruns) combine_run(r + 1, sb);
  }
}

// Chunk size: about 1024 chunks, a power of two in [4, 64].
int grouped_chunk(int64_t T) {
  int seg = 4;
  while (seg < kMaxSegG && (int64_t)seg * 1024 < T) seg *= 2;
  return seg;
}

}  // namespace

hipError_t launch_lookup_combine_grouped(const int64_t* rows, const int64_t* tok, const uint16_t* h,
                                         const uint16_t* w_r, const uint16_t* lut, float* y, int64_t T, int D, int N,
                                         hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int NP = N <= 1 ? 1 : (N <= 2 ? 2 : (N <= 4 ? 4 : (N <= 8 ? 8 : 16)));
  const unsigned rblocks = (unsigned)((T + kMaxTokPerBlock - 1) / kMaxTokPerBlock);
  const int seg = grouped_chunk(T);
  const dim3 grid((unsigned)((T + seg - 1) / seg), (unsigned)((D + 8 * kGroupedThreads - 1) / (8 * kGroupedThreads)));
#define MOLE_GROUPED(NPV)                                                                                      \
  hipLaunchKernelGGL((router_gates_kernel<NPV>), dim3(rblocks), dim3(256), 0, s, h, w_r, y, T, D, N);        \
  hipLaunchKernelGGL((lookup_combine_grouped_kernel<NPV>), grid, dim3(kGroupedThreads), 0, s, rows, tok, lut, y, \
                     T, D, N, seg)
  switch (NP) {
    case 1: MOLE_GROUPED(1); break;
    case 2: MOLE_GROUPED(2); break;
    case 4: MOLE_GROUPED(4); break;
    case 8: MOLE_GROUPED(8); break;
    default: MOLE_GROUPED(16); break;
  }
#undef MOLE_GROUPED
  return hipGetLastError();
}

}  // namespace mole
