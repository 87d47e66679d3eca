// Lookup-combine with the batch grouped by token id on the device (MoLE
// article, inference section: each token's expert outputs are fetched by
// token id; results section: the table keeps redundancy, and a prefill batch
// of natural text repeats ids -- under Zipf(1.1) a third of a 4096-token
// batch is distinct ids -- while every token of one id reads the same N x D
// slab).
//
// Two launches on the caller's stream, scratch in the caller's workspace:
//   1. group_route_kernel, two kinds of workgroups in one grid:
//      - grouping: one workgroup per chunk of kGroupChunk tokens puts the
//        chunk's tokens in an order where equal ids are adjacent.  An LDS
//        hash table (open addressing, twice as many slots as tokens) gives
//        each distinct id a slot and each token its rank among the slot's
//        tokens; an exclusive scan over the slot counts turns (slot, rank)
//        into the token's position.  Written: pos_tok[p] (the token at
//        position p) and pos_row[p] (its id).
//      - routing: one workgroup per 16 tokens computes their gates on the
//        matrix cores (one 16-row tile, the 16 wavefronts splitting D) and
//        writes them to gates[t][NP] (fp32).
//   2. lookup_combine_grouped_kernel: one workgroup per grouped position,
//      active where a run of equal ids starts (runs cut every 16
//      positions): it reads the run's slab once and writes each token of
//      the run.  Gates come from the workspace.
// The order of tokens inside a run depends on the order of the LDS atomics;
// each token's output does not (its sum runs over its own gates and slab in
// a fixed order).
#include <mutex>

#include "combine_common.hpp"

namespace mole {

namespace {

constexpr int kGroupChunk = 4096;               // tokens grouped together (one workgroup)
constexpr int kGroupSlots = 2 * kGroupChunk;    // LDS hash slots: a power of two, at least 2x the tokens
constexpr int kGroupThreads = 1024;
constexpr int kGroupPerThread = kGroupSlots / kGroupThreads;  // slots scanned per thread
constexpr int kTokPerThread = kGroupChunk / kGroupThreads;
constexpr int kGroupedSeg = 16;                 // longest run chunk one combine workgroup writes

__device__ __forceinline__ uint32_t slot_hash(uint32_t key) {
  // multiplicative hashing (Knuth), top bits select the slot
  return (key * 2654435761u) >> (32 - 13);
}
static_assert(kGroupSlots == 1 << 13, "slot_hash returns 13 bits");

// Gates of 16 tokens [t0, t0 + 16) on the matrix cores, all 16 wavefronts
// of the workgroup splitting D (one round of loads up to D = 2048 at 16
// experts), written to gates[t][NP].
template <int NP>
__device__ __forceinline__ void route_tile(const uint16_t* __restrict__ h, const uint16_t* __restrict__ w_r,
                                           float* __restrict__ gates, int64_t t0, int64_t T, int D, int N,
                                           float* red, float* gsh) {
  MfmaRouter<NP> rt;
  rt.load_first(h, w_r, t0, T, kMaxTokPerBlock, D, N, kGroupThreads / kWave);
  rt.finish(kMaxTokPerBlock, N, red, gsh);
  const int tid = threadIdx.x;
  if (tid < kMaxTokPerBlock * NP && t0 + tid / NP < T) gates[t0 * NP + tid] = gsh[tid];
}

template <int NP>
__global__ __launch_bounds__(kGroupThreads) void group_route_kernel(const int64_t* __restrict__ ids,
                                                                    const uint16_t* __restrict__ h,
                                                                    const uint16_t* __restrict__ w_r, int64_t T,
                                                                    int D, int N, int nchunks,
                                                                    int* __restrict__ pos_tok,
                                                                    int* __restrict__ pos_row,
                                                                    float* __restrict__ gates) {
  constexpr int NPAD = ((NP + 15) / 16) * 16;
  __shared__ int keys[kGroupSlots];
  __shared__ int cnt[kGroupSlots];
  __shared__ int wsum[kGroupThreads / kWave];
  static_assert(kGroupThreads / kWave * 16 * NPAD <= kGroupSlots && kMaxTokPerBlock * NP <= kGroupSlots,
                "the router's partial tiles and gates fit the hash arrays");
  if ((int)blockIdx.x >= nchunks) {
    // routing workgroup: its LDS is the hash arrays' space
    route_tile<NP>(h, w_r, gates, (int64_t)(blockIdx.x - nchunks) * kMaxTokPerBlock, T, D, N,
                   reinterpret_cast<float*>(keys), reinterpret_cast<float*>(cnt));
    return;
  }
  const int tid = threadIdx.x;
  const int64_t base = (int64_t)blockIdx.x * kGroupChunk;
  const int len = (int)(T - base < kGroupChunk ? T - base : kGroupChunk);
#pragma unroll
  for (int i = 0; i < kGroupPerThread; ++i) {
    keys[tid + i * kGroupThreads] = -1;
    cnt[tid + i * kGroupThreads] = 0;
  }
  int key[kTokPerThread];
#pragma unroll
  for (int i = 0; i < kTokPerThread; ++i) {
    const int q = tid + i * kGroupThreads;
    key[i] = (int)ids[base + (q < len ? q : 0)];
  }
  __syncthreads();
  // Insert: linear probing from the hashed slot.  At most kGroupChunk
  // distinct keys in kGroupSlots slots, so every probe finds its key or an
  // empty slot.  (An id of -1, invalid anyway, matches the empty marker and
  // is grouped like any other.)
  int slot[kTokPerThread], rank[kTokPerThread];
#pragma unroll
  for (int i = 0; i < kTokPerThread; ++i) {
    const int q = tid + i * kGroupThreads;
    slot[i] = 0;
    rank[i] = 0;
    if (q < len) {
      uint32_t sl = slot_hash((uint32_t)key[i]);
      for (int probe = 0; probe < kGroupSlots; ++probe) {
        const int old = atomicCAS(&keys[sl], -1, key[i]);
        if (old == -1 || old == key[i]) break;
        sl = (sl + 1) & (kGroupSlots - 1);
      }
      slot[i] = (int)sl;
      rank[i] = atomicAdd(&cnt[sl], 1);
    }
  }
  __syncthreads();
  // Exclusive scan of the slot counts: each thread owns kGroupPerThread
  // consecutive slots; wavefront scans of the thread totals, then of the
  // wavefront totals.
  int c[kGroupPerThread], run = 0;
#pragma unroll
  for (int i = 0; i < kGroupPerThread; ++i) {
    c[i] = cnt[tid * kGroupPerThread + i];
    run += c[i];
  }
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  int incl = run;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += o;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int wbase = 0;
  for (int w = 0; w < wave; ++w) wbase += wsum[w];
  int off = wbase + incl - run;
#pragma unroll
  for (int i = 0; i < kGroupPerThread; ++i) {
    cnt[tid * kGroupPerThread + i] = off;
    off += c[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kTokPerThread; ++i) {
    const int q = tid + i * kGroupThreads;
    if (q < len) {
      const int p = cnt[slot[i]] + rank[i];
      pos_tok[base + p] = (int)(base + q);
      pos_row[base + p] = key[i];
    }
  }
}

// One workgroup per grouped position p, active only where a run chunk
// starts: at p = 0, where the id changes, or at a multiple of kGroupedSeg
// inside a run (long runs are cut so that no workgroup writes more than
// kGroupedSeg rows).  An active workgroup reads its id's slab once -- lane l
// holds the 16-byte chunk l (and l + LANES, ...) of every expert row -- and
// writes the gate-weighted sum for each token of the run chunk.  The other
// workgroups exit at once.  Gates come from the workspace.
template <int NP, int LANES>
__global__ __launch_bounds__(LANES) void lookup_combine_grouped_kernel(
    const int* __restrict__ pos_tok, const int* __restrict__ pos_row, const float* __restrict__ gates,
    const uint16_t* __restrict__ lut, float* __restrict__ y, int64_t T, int D, int N) {
  static_assert(NP <= 16, "a lane holds one chunk of every expert row");
  __shared__ float gsh[kGroupedSeg * NP];
  __shared__ int ts[kGroupedSeg];
  const int lane = threadIdx.x;
  const int64_t p = blockIdx.x;
  const int row = pos_row[p];
  if (p != 0 && (p % kGroupedSeg) != 0 && pos_row[p - 1] == row) return;  // not a run-chunk start (uniform)
  const int C = D / 8;
  const uint16_t* slab = lut + (int64_t)row * N * D;
  // the slab's first chunk per lane goes out first
  uint4 sv[NP];
  {
    const int cc = lane < C ? lane : C - 1;
#pragma unroll
    for (int e = 0; e < NP; ++e) sv[e] = ldg16(slab + (int64_t)(e < N ? e : N - 1) * D + (int64_t)cc * 8);
  }
  // run chunk length: positions p .. p + len - 1 share the row (at most to the next multiple of kGroupedSeg)
  const int64_t lim = ((p / kGroupedSeg) + 1) * kGroupedSeg < T ? ((p / kGroupedSeg) + 1) * kGroupedSeg : T;
  int len = 1;
  while (p + len < lim && pos_row[p + len] == row) ++len;
  if (lane < len) ts[lane] = pos_tok[p + lane];
  __syncthreads();
  for (int i = lane; i < len * NP; i += LANES) gsh[i] = gates[(int64_t)ts[i / NP] * NP + i % NP];
  __syncthreads();
  for (int c = lane; c < C; c += LANES) {
    if (c != lane) {
#pragma unroll
      for (int e = 0; e < NP; ++e) sv[e] = ldg16(slab + (int64_t)(e < N ? e : N - 1) * D + (int64_t)c * 8);
    }
    for (int q = 0; q < len; ++q) {
      float acc[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = 0.f;
#pragma unroll
      for (int e = 0; e < NP; ++e) {
        if (e < N) {
          float v[8];
          Elem<uint16_t>::unpack(sv[e], v);
          const float g = gsh[q * NP + e];
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[j] = fmaf(g, v[j], acc[j]);
        }
      }
      float* yo = y + (int64_t)ts[q] * D + (int64_t)c * 8;
      stg16_nt(yo, acc[0], acc[1], acc[2], acc[3]);
      stg16_nt(yo + 4, acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

struct GroupedWs {
  size_t tok_off, row_off, gate_off, total;
};

constexpr size_t round256(size_t x) { return (x + 255u) & ~(size_t)255u; }

constexpr GroupedWs grouped_ws(int64_t T) {
  GroupedWs w{};
  w.tok_off = 0;
  w.row_off = round256((size_t)T * 4u);
  w.gate_off = w.row_off + round256((size_t)T * 4u);
  w.total = w.gate_off + round256((size_t)T * 16u * 4u);  // gates for up to 16 experts
  return w;
}
constexpr size_t grouped_ws_total_max() { return grouped_ws(kGroupedNoAllocMaxT).total; }

template <int NP>
hipError_t group_route_np(const int64_t* ids, const uint16_t* h, const uint16_t* w_r, int64_t T, int D, int N,
                          void* ws, hipStream_t s, int** pos_tok, int** pos_row, float** gates) {
  const GroupedWs lay = grouped_ws(T);
  char* base = static_cast<char*>(ws);
  *pos_tok = reinterpret_cast<int*>(base + lay.tok_off);
  *pos_row = reinterpret_cast<int*>(base + lay.row_off);
  *gates = reinterpret_cast<float*>(base + lay.gate_off);
  const int nchunks = (int)((T + kGroupChunk - 1) / kGroupChunk);
  const int64_t rtiles = (T + kMaxTokPerBlock - 1) / kMaxTokPerBlock;
  hipLaunchKernelGGL((group_route_kernel<NP>), dim3((unsigned)(nchunks + rtiles)), dim3(kGroupThreads), 0, s, ids,
                     h, w_r, T, D, N, nchunks, *pos_tok, *pos_row, *gates);
  return hipGetLastError();
}

template <int NP>
hipError_t launch_grouped_np(const int64_t* ids, const uint16_t* h, const uint16_t* w_r, const uint16_t* lut,
                             float* y, int64_t T, int D, int N, void* ws, hipStream_t s) {
  int *pos_tok, *pos_row;
  float* gates;
  hipError_t err = group_route_np<NP>(ids, h, w_r, T, D, N, ws, s, &pos_tok, &pos_row, &gates);
  if (err != hipSuccess) return err;
  // lanes per workgroup: the 16-byte chunks of a row, 64 to 256
  const int C = D / 8;
  if (C <= 64)
    hipLaunchKernelGGL((lookup_combine_grouped_kernel<NP, 64>), dim3((unsigned)T), dim3(64), 0, s, pos_tok, pos_row,
                       gates, lut, y, T, D, N);
  else if (C <= 128)
    hipLaunchKernelGGL((lookup_combine_grouped_kernel<NP, 128>), dim3((unsigned)T), dim3(128), 0, s, pos_tok,
                       pos_row, gates, lut, y, T, D, N);
  else
    hipLaunchKernelGGL((lookup_combine_grouped_kernel<NP, 256>), dim3((unsigned)T), dim3(256), 0, s, pos_tok,
                       pos_row, gates, lut, y, T, D, N);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Allocation-free variant: the workspace of up to kGroupedNoAllocMaxT tokens
// in a static device array (each GPU the library runs on holds its own copy
// until the process ends).  Host code never passes the array's name to a
// kernel (in host code it is only a stand-in for the symbol): the device
// address comes from hipGetSymbolAddress, looked up once per device with
// that device current, and kept.  Every call on one GPU shares the array, so
// calls that overlap on one GPU race; nothing in it needs clearing (each call
// writes every position and gate it reads).
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[grouped_ws_total_max()];  // 4.5 MiB
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device that runs `s` (the current
// device for the null stream).
hipError_t scratch_address(hipStream_t s, void** out) {
  int cur = 0;
  hipError_t err = hipGetDevice(&cur);
  if (err != hipSuccess) return err;
  int dev = cur;
  if (s != nullptr) {
    err = hipStreamGetDevice(s, &dev);
    if (err != hipSuccess) return err;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && (err = hipSetDevice(dev)) != hipSuccess) return err;
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (err == hipSuccess) err = e2;
    }
    if (err != hipSuccess) return err;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

size_t grouped_workspace_bytes(int64_t T) { return grouped_ws(T).total; }

hipError_t launch_lookup_combine_grouped_noalloc(const int64_t* ids, const uint16_t* h, const uint16_t* w_r,
                                                 const uint16_t* lut, float* y, int64_t T, int D, int N,
                                                 hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (T > kGroupedNoAllocMaxT) return hipErrorInvalidValue;
  void* ws = nullptr;
  const hipError_t err = scratch_address(s, &ws);
  if (err != hipSuccess) return err;
  return launch_lookup_combine_grouped(ids, h, w_r, lut, y, T, D, N, ws, s);
}

hipError_t launch_group_route(const int64_t* ids, const uint16_t* h, const uint16_t* w_r, int64_t T, int D, int N,
                              void* ws, hipStream_t s, const int** pos_tok, const int** pos_row,
                              const float** gates) {
  int *pt, *pr;
  float* g;
  const int NP = N <= 1 ? 1 : (N <= 2 ? 2 : (N <= 4 ? 4 : (N <= 8 ? 8 : 16)));
  hipError_t err;
  switch (NP) {
    case 1: err = group_route_np<1>(ids, h, w_r, T, D, N, ws, s, &pt, &pr, &g); break;
    case 2: err = group_route_np<2>(ids, h, w_r, T, D, N, ws, s, &pt, &pr, &g); break;
    case 4: err = group_route_np<4>(ids, h, w_r, T, D, N, ws, s, &pt, &pr, &g); break;
    case 8: err = group_route_np<8>(ids, h, w_r, T, D, N, ws, s, &pt, &pr, &g); break;
    default: err = group_route_np<16>(ids, h, w_r, T, D, N, ws, s, &pt, &pr, &g); break;
  }
  *pos_tok = pt;
  *pos_row = pr;
  *gates = g;
  return err;
}

hipError_t launch_lookup_combine_grouped(const int64_t* ids, const uint16_t* h, const uint16_t* w_r,
                                         const uint16_t* lut, float* y, int64_t T, int D, int N, void* ws,
                                         hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int NP = N <= 1 ? 1 : (N <= 2 ? 2 : (N <= 4 ? 4 : (N <= 8 ? 8 : 16)));
  switch (NP) {
    case 1: return launch_grouped_np<1>(ids, h, w_r, lut, y, T, D, N, ws, s);
    case 2: return launch_grouped_np<2>(ids, h, w_r, lut, y, T, D, N, ws, s);
    case 4: return launch_grouped_np<4>(ids, h, w_r, lut, y, T, D, N, ws, s);
    case 8: return launch_grouped_np<8>(ids, h, w_r, lut, y, T, D, N, ws, s);
    default: return launch_grouped_np<16>(ids, h, w_r, lut, y, T, D, N, ws, s);
  }
}

}  // namespace mole
