/*
 * mole.h -- C ABI of libmole.so, the MI355X (gfx950) hot path of
 * Mixture-of-Lookup-Experts (MoLE) inference.
 *
 * MoLE's routed experts read the token embedding instead of the previous
 * layer's output, so before inference every expert can be run once over the
 * whole vocabulary and replaced by a table indexed by token id; at inference
 * each token fetches its N expert outputs by id and mixes them with the
 * router's gates.  (MoLE article, "ICML 2025 Spotlight | MoLE" page:
 * sections "思考" (motivation), "训练阶段" (training), "推理阶段"
 * (inference) and "实验结果" (results, 3-bit table).)
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Pointers are device pointers (hipMalloc / torch CUDA tensors) unless
 *    the argument name ends in _host.  The caller owns every buffer; the
 *    library allocates no device memory.
 *  - Tensors are dense row-major with the shapes given below.  Element
 *    types: dtype MOLE_F32 = IEEE binary32, MOLE_BF16 = bfloat16.  The
 *    combine output y is always fp32.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default
 *    stream) and the call returns without waiting, except where a function
 *    says otherwise.  Inputs must stay valid until the work has run.
 *  - Every function returns MOLE_OK (0) or a negative status; argument
 *    errors are detected on the host before anything is enqueued.  After
 *    MOLE_ERR_HIP, mole_last_hip_error() gives the hipError_t (per thread).
 *  - Device pointers must be 16-byte aligned (MOLE_ERR_ALIGN otherwise).
 *  - Token ids must lie in [0, V); the GPU entry points do not check ids
 *    stored in device memory (an out-of-range id reads outside the table);
 *    mole_check_ids counts such ids on the device, for callers that want
 *    the check.
 *  - Entry points may be called from several threads; calls that write the
 *    same buffers must be ordered by the caller.  Device-side entry points
 *    keep no state between calls.  The staged host-side paths (host-resident
 *    and file-backed tables copied through a staging area) keep two pieces
 *    of process-wide state, created on first use: a pool of up to 64 gather
 *    threads, and one HIP event per distinct pinned staging area (the event
 *    that orders reuse of that area).  mole_release_host_state() frees both.
 *    The read-in-place (_mapped) entry points keep none.
 */
#ifndef MOLE_H
#define MOLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOLE_OK 0
#define MOLE_ERR_NULL (-1)        /* a required pointer is NULL */
#define MOLE_ERR_DIM (-2)         /* a size is negative, zero where it must not be, or inconsistent */
#define MOLE_ERR_DTYPE (-3)       /* unknown dtype code */
#define MOLE_ERR_ALIGN (-4)       /* a device pointer is not 16-byte aligned */
#define MOLE_ERR_WORKSPACE (-5)   /* workspace smaller than the minimum */
#define MOLE_ERR_UNSUPPORTED (-6) /* a valid but unsupported shape (e.g. N > 64) */
#define MOLE_ERR_HIP (-7)         /* a HIP runtime call or kernel launch failed */
#define MOLE_ERR_ID (-8)          /* a host-side token id is outside [0, V) */
#define MOLE_ERR_IO (-9)          /* a table file could not be read or written */
#define MOLE_ERR_FORMAT (-10)     /* not a MoLE NF3 table file of this version */
#define MOLE_ERR_HOST (-11)       /* a host-side allocation or thread creation failed */
#define MOLE_ERR_MEMORY (-12)     /* a host table is not page-locked memory the device can read */

#define MOLE_F32 0
#define MOLE_BF16 1

/* Static text for a status code. */
const char* mole_status_string(int status);

/* The hipError_t of the last failing HIP call on this thread (0 if none). */
int mole_last_hip_error(void);

/* ABI version of this header (increments on any signature change). */
int mole_abi_version(void);

/*
 * Free the process-wide host state of the host-resident and file-backed
 * paths: end the gather threads and destroy the staging-area events.  Call
 * it only when no other thread is inside a libmole call and the streams
 * have passed every host-resident call's copy (the events of the staging
 * areas are destroyed).  Later calls recreate the state on first use.
 * Returns MOLE_ERR_HIP if destroying an event fails (the rest is still
 * released).
 */
int mole_release_host_state(void);

/*
 * Copy the 8 NF3 reconstruction levels used by the library's kernels (fp32,
 * ascending, code c -> levels[c]) to host memory.  Host-only; no GPU call.
 */
int mole_nf3_levels(float* levels_host);

/*
 * Copy the 7 NF3 decision thresholds of mole_pack_nf3 at unit scale (fp32,
 * ascending: the nearest-even fp32 rounding of the exact midpoint of levels
 * j and j+1) to host memory.  Host-only.  The kernels read the same array.
 */
int mole_nf3_midpoints(float* mid_host);

/*
 * The normal-CDF polynomial behind GELU(u) = u * Phi(u) in the bf16 kernels
 * (the experts' activation; MoLE page, inference section: every expert runs
 * over the embedding matrix).  On [-range, range], with s = u / range:
 *     Phi(u) = 1/2 + s * (c[0] + c[1] s^2 + ... + c[9] s^18)   (fp32 Horner)
 * clamped to [0, 1]; outside the interval u is clamped to +-range first
 * (1 - Phi(4) = 3.2e-5 is the error there).  Copies the 10
 * fp32 coefficients to coef_host (n >= 10, else MOLE_ERR_DIM) and the
 * interval's half-width to *range.  Host-only; the kernels read the same
 * array.
 */
int mole_gelu_phi_coefficients(float* coef_host, int n, float* range);

/* ------------------------------------------------------------------------
 * LUT reparameterisation (inference section: the embedding weight matrix is
 * fed to every routed expert, giving the complete token-id -> expert-output
 * table):
 *
 *   LUT[v][e][:] = W_down[e] . GELU(W_up[e] . Emb[v])     for all v < V, e < N
 *
 * with GELU(u) = u * Phi(u) (erf form) and no biases.
 *   emb    [V][D]      w_up [N][F][D]     w_down [N][D][F]     lut [V][N][D]
 * (w_up and w_down are stored output-major, like a linear layer's weight.)
 * dtype MOLE_F32: everything fp32, fp32 arithmetic.
 * dtype MOLE_BF16: bf16 inputs and output; bf16 matrix-core products with
 *   fp32 accumulation; the hidden activation GELU(.) is rounded to bf16
 *   between the two products; LUT rounded to bf16 (nearest even).
 * Needs D % 8 == 0 and F % 8 == 0 for MOLE_BF16, and N*F and N*D at most
 * 2^22 (the row strides of the hidden activations and of the table: each
 * 256-row panel is addressed with 32-bit offsets); MOLE_ERR_UNSUPPORTED
 * otherwise.  (The largest configurations here use N*F = 131072.)
 *
 * workspace: device scratch for the bf16 hidden activations of a block of
 * vocabulary rows (ignored for MOLE_F32, may be NULL there).  Any size at
 * or above the minimum works; larger blocks mean fewer launches.
 * mole_build_lut_workspace_size() returns the minimum in *min_bytes and a
 * recommended size in *rec_bytes (either pointer may be NULL): blocks of
 * about 1 GB of hidden activations (every block re-reads the expert
 * weights, so larger blocks move less; beyond about 1 GB the build time no
 * longer changes).
 * ------------------------------------------------------------------------ */
int mole_build_lut_workspace_size(int64_t V, int64_t D, int64_t F, int64_t N, int dtype,
                                  size_t* min_bytes, size_t* rec_bytes);

int mole_build_lut(const void* emb, const void* w_up, const void* w_down, void* lut,
                   int64_t V, int64_t D, int64_t F, int64_t N, int dtype,
                   void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Lookup-combine (inference section: each token's expert outputs are
 * fetched by token id; training section: the router reads the contextual
 * hidden state and every routed expert is active):
 *
 *   g[t][:] = softmax_e( sum_d h[t][d] * w_r[e][d] )       (all N experts)
 *   y[t][d] = sum_e g[t][e] * LUT[ids[t]][e][d]
 *
 *   ids [T] int64      h [T][D]      w_r [N][D]      lut [V][N][D]
 *   y   [T][D] fp32 (written, never read)
 * h, w_r and lut share `dtype`.  Router dot products, softmax and the
 * combine accumulate in fp32.  T == 0 is a no-op.  1 <= N <= 64 and
 * D <= 2^20 (MOLE_ERR_UNSUPPORTED above: the kernels keep a token's N gates
 * in registers, and the routers address the rows of h and w_r with 32-bit
 * offsets); the same limits hold for every combine below.
 * ------------------------------------------------------------------------ */
int mole_lookup_combine(const int64_t* ids, const void* h, const void* w_r, const void* lut,
                        float* y, int64_t T, int64_t V, int64_t D, int64_t N, int dtype,
                        void* stream);

/* ------------------------------------------------------------------------
 * NF3 table compression (results section: the table still works at 3 bits,
 * e.g. NF3).  Per row r = v*N + e and block b of 64 consecutive elements:
 *   a = max |x| (fp32);  s = fp16(min(a, 65504)) rounded to nearest even;
 *   scales[r][b] = s (fp16 bits);
 *   code = #{ j : x > fp32(mid[j] * s) } for the 7 midpoints of the levels
 *          (strict: an exact tie takes the lower code); code 3 if s == 0;
 *   code i of row r sits at bits [3i, 3i+3) of the row's little-endian bit
 *   stream, LSB first (3D/8 bytes per row).
 * Levels: the NormalFloat construction at 3 bits (see mole_nf3_levels).
 *   lut [V][N][D] (dtype)   codes [V][N][3D/8] u8   scales [V][N][D/64] u16
 * Needs D % 64 == 0.  Codes and scales are bit-exact functions of the table.
 * ------------------------------------------------------------------------ */
int mole_pack_nf3(const void* lut, uint8_t* codes, uint16_t* scales,
                  int64_t V, int64_t N, int64_t D, int dtype, void* stream);

/*
 *   y[t][d] = sum_e g[t][e] * levels[code(ids[t], e, d)] * s(ids[t], e, d/64)
 * with g as in mole_lookup_combine; codes/scales laid out as produced by
 * mole_pack_nf3 for a table of V rows.  dtype_h is the dtype of h and w_r.
 * Needs D % 64 == 0.
 */
int mole_lookup_combine_nf3(const int64_t* ids, const void* h, const void* w_r,
                            const uint8_t* codes, const uint16_t* scales, float* y,
                            int64_t T, int64_t V, int64_t D, int64_t N, int dtype_h,
                            void* stream);

/* ------------------------------------------------------------------------
 * The MoLE block at inference (training section: shared experts and the
 * router keep reading the previous layer's output; complexity analysis: at
 * inference the shared experts are the only experts still computed, the
 * routed ones having become table lookups):
 *
 *   x[t][:] += W_s_down . GELU(W_s_up . h[t]) + y[t][:]
 *
 * where y is mole_lookup_combine(ids, h, w_r, lut) and the shared expert
 * has the routed experts' form (D -> F -> D, GELU(u) = u * Phi(u), no
 * biases).  x is the residual stream, read and written in place; pass a
 * zero-filled x to get the two expert terms alone.
 *   ids [T] int64   h [T][D]   w_r [N][D]   lut [V][N][D]
 *   w_s_up [F][D]   w_s_down [D][F]   (output-major, like the routed experts)
 *   x [T][D] fp32 (read and written)
 * dtype must be MOLE_BF16 (MOLE_ERR_UNSUPPORTED for MOLE_F32): bf16 inputs,
 * fp32 accumulation, the hidden activation rounded to bf16 between the two
 * products as in mole_build_lut, everything after the products in fp32.
 * Needs D % 8 == 0, F % 8 == 0 (MOLE_ERR_DIM), D <= 2^20 (as for the
 * combines) and F <= 2^22 (MOLE_ERR_UNSUPPORTED); 1 <= N <= 64.  T == 0 is
 * a no-op.
 *
 * workspace: device scratch (16-byte aligned) of at least the size that
 * mole_layer_workspace_size(T, D, F) returns (0 for T == 0): router gates,
 * the hidden activations and the down-projection's per-split fp32 partial
 * sums, which the final lookup-combine pass adds to x with the table rows.
 * Contents on return are unspecified.  Enqueued on `stream`, asynchronous,
 * no memset (capturable in a HIP graph).
 * ------------------------------------------------------------------------ */
int mole_layer_workspace_size(int64_t T, int64_t D, int64_t F, size_t* bytes);

int mole_layer_forward(const int64_t* ids, const void* h, const void* w_r, const void* lut,
                       const void* w_s_up, const void* w_s_down, float* x, int64_t T, int64_t V,
                       int64_t D, int64_t N, int64_t F, int dtype, void* workspace,
                       size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Other table formats (results section: the table keeps the model's quality
 * at 3 bits, so it still carries redundancy; these are the 4- and 8-bit
 * points next to NF3, with the same combine contract as
 * mole_lookup_combine_nf3).  Both need D % 64 == 0 (MOLE_ERR_DIM).
 *
 * NF4: the NormalFloat construction at 4 bits (16 levels, zero at code 7;
 * mole_nf4_levels copies them to host memory), blocks of 64 elements with
 * the fp16 absmax scale exactly as for NF3, code = number of the 15
 * thresholds fp32(mid[j] * s) strictly below x (code 7 when s == 0), two
 * codes per byte, element 2i in the low nibble of byte i (D/2 bytes a row).
 *   lut [V][N][D] (dtype)   codes [V][N][D/2] u8   scales [V][N][D/64] fp16 bits
 *
 * int8: one fp32 scale per (v, e) row: a = max |x| over the row,
 * s = a / 127 (IEEE division); code = rint(x / s) (IEEE division, ties to
 * even) clamped to [-127, 127], 0 when s == 0; x is reconstructed as code * s.
 *   lut [V][N][D] (dtype)   codes [V][N][D] int8   scales [V][N] fp32
 * Codes and scales of both formats are bit-exact functions of the table.
 * The combines compute y[t][d] = sum_e g[t][e] * xhat(ids[t], e, d) with g as
 * in mole_lookup_combine; dtype_h is the dtype of h and w_r.
 * ------------------------------------------------------------------------ */
int mole_nf4_levels(float* levels_host);

/* The 15 NF4 decision thresholds at unit scale (as mole_nf3_midpoints). */
int mole_nf4_midpoints(float* mid_host);

int mole_pack_nf4(const void* lut, uint8_t* codes, uint16_t* scales,
                  int64_t V, int64_t N, int64_t D, int dtype, void* stream);

int mole_lookup_combine_nf4(const int64_t* ids, const void* h, const void* w_r,
                            const uint8_t* codes, const uint16_t* scales, float* y,
                            int64_t T, int64_t V, int64_t D, int64_t N, int dtype_h,
                            void* stream);

int mole_pack_int8(const void* lut, int8_t* codes, float* scales,
                   int64_t V, int64_t N, int64_t D, int dtype, void* stream);

int mole_lookup_combine_int8(const int64_t* ids, const void* h, const void* w_r,
                             const int8_t* codes, const float* scales, float* y,
                             int64_t T, int64_t V, int64_t D, int64_t N, int dtype_h,
                             void* stream);

/* ------------------------------------------------------------------------
 * Training mode of the routed experts (training section: every routed
 * expert reads the token's shallow embedding Emb[id], all experts are
 * active with dense softmax gates, the router reads the contextual hidden
 * state h; the inference table is this forward pass on every vocabulary
 * row -- here it is evaluated on the batch's distinct rows only):
 *
 *   y[t][:] = sum_e softmax(W_r . h[t])[e] * W_down[e] . GELU(W_up[e] . Emb[ids[t]])
 *
 * and its gradients for an upstream dy [T][D] (fp32): d_w_up [N][F][D],
 * d_w_down [N][D][F], d_w_r [N][D], d_h [T][D] and d_x [U][D], the
 * gradient of the embedding rows Emb[uniq[u]] (a row used by several tokens
 * receives their sum; scatter-add it into the embedding gradient).
 *
 * mole_train_index: host-only.  Deduplicates ids_host[0..T) in first-
 * occurrence order: uniq_host[0..U) = the distinct ids, remap_host[t] = the
 * row of ids_host[t] among them, and the tokens of each row, grouped:
 * tok_host[row_ptr_host[u] .. row_ptr_host[u+1]) in increasing t
 * (row_ptr_host has U+1 entries; size it T+1).  *n_unique = U.
 * MOLE_ERR_ID for an id outside [0, V).  Copy uniq, remap, row_ptr and tok
 * to the device for the two calls below.
 *
 * mole_train_workspace_size: the forward workspace (kept by the caller from
 * the forward to the backward call: the gathered rows, the hidden pre- and
 * post-activations and the batch's table rows) and the backward scratch,
 * for T tokens and U distinct ids.
 *
 * mole_train_forward / mole_train_backward: bf16 only (MOLE_ERR_UNSUPPORTED
 * for MOLE_F32), D % 8 == 0 and F % 8 == 0 (MOLE_ERR_DIM), N*D, N*F and T
 * at most 2^20 and 1 <= N <= 64 (MOLE_ERR_UNSUPPORTED).  bf16 products with
 * fp32 accumulation; as in mole_build_lut the hidden activation is rounded
 * to bf16, the forward workspace keeps the bf16 pre-activations, and the
 * backward pass rounds the row gradients and the hidden gradients to bf16
 * for the matrix cores; all sums and every output are fp32.  Weight gradients are
 * overwritten, not accumulated.  Deterministic (no atomics).
 *   uniq [U] int64, remap [T] int64, row_ptr [U+1] int64, tok [T] int64 (device)
 *   emb [V][D], w_up [N][F][D], w_down [N][D][F], h [T][D], w_r [N][D] (bf16)
 *   y [T][D] fp32 (written)
 * ------------------------------------------------------------------------ */
int mole_train_index(const int64_t* ids_host, int64_t T, int64_t V, int64_t* uniq_host,
                     int64_t* remap_host, int64_t* row_ptr_host, int64_t* tok_host,
                     int64_t* n_unique);

int mole_train_workspace_size(int64_t T, int64_t U, int64_t D, int64_t F, int64_t N,
                              size_t* fwd_bytes, size_t* bwd_bytes);

int mole_train_forward(const int64_t* uniq, const int64_t* remap, const void* emb,
                       const void* w_up, const void* w_down, const void* h, const void* w_r,
                       float* y, int64_t T, int64_t U, int64_t V, int64_t D, int64_t F, int64_t N,
                       int dtype, void* fwd_ws, size_t fwd_bytes, void* stream);

int mole_train_backward(const int64_t* remap, const int64_t* row_ptr, const int64_t* tok,
                        const void* w_up, const void* w_down, const void* h, const void* w_r,
                        const float* dy, const void* fwd_ws, size_t fwd_bytes, void* bwd_ws,
                        size_t bwd_bytes, float* d_w_up, float* d_w_down, float* d_w_r,
                        float* d_h, float* d_x, int64_t T, int64_t U, int64_t V, int64_t D,
                        int64_t F, int64_t N, int dtype, void* stream);

/* ------------------------------------------------------------------------
 * Host-resident NF3 table (inference section: after reparameterisation the
 * table lives in lower-tier storage such as CPU memory, each token's
 * entries are looked up there and only the retrieved vectors are loaded
 * into GPU memory).
 *
 * mole_gather_nf3_host: host-only.  Deduplicates ids_host[0..T) (first
 * occurrence order), copies the U distinct rows' codes and scales into
 * codes_stage_host [U][N][3D/8] / scales_stage_host [U][N][D/64] and writes
 * remap_host[t] = index of ids_host[t] among the distinct ids, so that
 * row remap_host[t] of the staged table is row ids_host[t] of the full one.
 * *n_unique receives U.  nthreads <= 0 picks the hardware concurrency.
 * Returns MOLE_ERR_ID if an id is outside [0, V).
 *
 * mole_nf3_host_staging_size: *bytes = size of the staging area that
 * mole_lookup_combine_nf3_host needs for a batch of up to T tokens, both in
 * pinned host memory and on the device.  Layout for a batch with U distinct
 * ids, each section starting on a 16-byte boundary:
 *     remap  int64 [T]          (row of the staged table for each token)
 *     codes  uint8 [U][N][3D/8]
 *     scales fp16  [U][N][D/64]
 * Host-only; returns MOLE_ERR_DIM unless T >= 0, N > 0, D > 0, D % 64 == 0.
 *
 * mole_lookup_combine_nf3_host: gather on the calling thread as above into
 * stage_host (pinned, hipHostMalloc'ed; stage_bytes >= the staging size
 * for T), then enqueue on `stream` one host->device copy of the used part
 * of the staging area into stage_dev (device, 16-byte aligned, same size)
 * and the NF3 combine over the staged rows.  Because stage_host is rewritten
 * on the host, this function first waits (on the host) until the previous
 * call's copy out of the same stage_host has finished -- not for the rest of
 * the stream -- so the gather overlaps earlier GPU work; the rest is
 * asynchronous.  Calls that share a staging area must be issued on one
 * stream (stage_dev is then reused in stream order).  Not capturable in a
 * HIP graph (the gather runs on the host at call time).  The caller keeps
 * stage_host and stage_dev alive until the stream has passed the call.
 * *n_unique (may be NULL) receives U.  Returns MOLE_ERR_WORKSPACE if
 * stage_bytes is too small.
 * ------------------------------------------------------------------------ */
int mole_gather_nf3_host(const int64_t* ids_host, int64_t T, const uint8_t* codes_host,
                         const uint16_t* scales_host, int64_t V, int64_t N, int64_t D,
                         uint8_t* codes_stage_host, uint16_t* scales_stage_host,
                         int64_t* remap_host, int64_t* n_unique, int nthreads);

int mole_nf3_host_staging_size(int64_t T, int64_t N, int64_t D, size_t* bytes);

int mole_lookup_combine_nf3_host(const int64_t* ids_host, const void* h, const void* w_r,
                                 const uint8_t* codes_host, const uint16_t* scales_host,
                                 void* stage_host, void* stage_dev, size_t stage_bytes, float* y,
                                 int64_t T, int64_t V, int64_t D, int64_t N, int dtype_h,
                                 int nthreads, int64_t* n_unique, void* stream);

/* ------------------------------------------------------------------------
 * Host-resident NF3 table read in place (inference section: the table in
 * lower-tier storage, only the retrieved vectors crossing into the GPU).
 *
 * mole_lookup_combine_nf3_mapped: the NF3 combine of mole_lookup_combine_nf3
 * with the table left in page-locked host memory: the kernel reads each
 * token's N rows of codes and scales over PCIe as it combines them, so a
 * call is one launch -- no host-side dedupe or gather, no staging area, no
 * wait on the host.  ids (int64 [T]), h, w_r and y are device memory as for
 * mole_lookup_combine_nf3; codes_host [V][N][3D/8] and scales_host
 * [V][N][D/64] must each lie inside one page-locked host allocation made
 * through HIP (hipHostMalloc, or a pinned tensor of the framework) and must
 * not be written while a call that reads them is in flight.  Both ranges
 * are checked with the runtime's pointer attributes before anything is
 * enqueued: pageable or unknown memory, or a range that runs past the end
 * of the allocation holding its first byte, returns MOLE_ERR_MEMORY (a
 * kernel reading it would fault); a V whose table byte count overflows
 * int64 returns MOLE_ERR_DIM.  Every token reads its own rows, so repeated
 * ids cross PCIe again unless the GPU's caches still hold them; for large
 * batches with repeated ids mole_lookup_combine_nf3_host (one copy of the
 * distinct rows) moves fewer bytes.  Asynchronous on `stream`; capturable
 * in a HIP graph (the checks run at call time, the launch is the device
 * combine's).
 * ------------------------------------------------------------------------ */
int mole_lookup_combine_nf3_mapped(const int64_t* ids, const void* h, const void* w_r,
                                   const uint8_t* codes_host, const uint16_t* scales_host, float* y,
                                   int64_t T, int64_t V, int64_t D, int64_t N, int dtype_h, void* stream);

/* mole_lookup_combine_mapped: the same for the uncompressed table: the
 * combine of mole_lookup_combine with lut_host [V][N][D] (dtype, as h and
 * w_r) left in page-locked host memory allocated through HIP.  Each token
 * reads its N x D slab over PCIe (2 N D bytes in bf16: 64 KB per token at
 * N = 16, D = 2048).  Same checks, errors and graph behaviour as
 * mole_lookup_combine_nf3_mapped. */
int mole_lookup_combine_mapped(const int64_t* ids, const void* h, const void* w_r, const void* lut_host,
                               float* y, int64_t T, int64_t V, int64_t D, int64_t N, int dtype,
                               void* stream);

/* ------------------------------------------------------------------------
 * Host-resident NF3 tables of a stack of L layers, prefetched at the start
 * of a decode step (inference section: the table lives in lower-tier
 * storage and only the retrieved vectors are loaded into GPU memory; a
 * token's id is known before the first layer runs, so every layer's rows
 * can be fetched in one transfer ahead of the layers that use them).
 *
 * mole_nf3_host_stack_staging_size: *bytes = staging size (pinned host and
 * device alike) for up to T tokens and L layers.  Layout for a batch with U
 * distinct ids, each section on a 16-byte boundary:
 *     remap  int64 [T]
 *     then for each layer l:  codes_l uint8 [U][N][3D/8],  scales_l fp16 [U][N][D/64]
 *
 * mole_prefetch_nf3_host_stack: dedupe ids_host once, gather the U distinct
 * rows of every layer's host table (codes_host[l] [V][N][3D/8],
 * scales_host[l] [V][N][D/64], l < L; pinned or pageable) into stage_host
 * (pinned, 16-byte aligned) and enqueue on `stream` the host->device copy
 * of the used part into stage_dev -- in up to four pieces of consecutive
 * layers, each enqueued as soon as its rows are gathered, so the bus moves
 * one piece while the next is gathered.  codes_off[l] / scales_off[l] (host
 * arrays of L entries) receive the byte offsets of layer l's sections, so
 * layer l's combine, issued on the same stream after this call, is
 *     mole_lookup_combine_nf3(stage_dev, h_l, w_r_l,
 *         stage_dev + codes_off[l], stage_dev + scales_off[l], y_l,
 *         T, U, D, N, dtype_h, stream)
 * (the remap section at the start of stage_dev serves as the ids, and U,
 * the number of staged rows, as the vocabulary size).  Waiting and reuse rules as
 * for mole_lookup_combine_nf3_host (the previous copy out of the same
 * stage_host is waited for on the host; not capturable in a HIP graph).
 * *n_unique receives U.  Errors: MOLE_ERR_ID for an id outside [0, V),
 * MOLE_ERR_WORKSPACE if stage_bytes is below the staging size for T, L.
 * ------------------------------------------------------------------------ */
int mole_nf3_host_stack_staging_size(int64_t T, int64_t L, int64_t N, int64_t D, size_t* bytes);

int mole_prefetch_nf3_host_stack(const int64_t* ids_host, int64_t T,
                                 const uint8_t* const* codes_host, const uint16_t* const* scales_host,
                                 int64_t L, int64_t V, int64_t N, int64_t D, void* stage_host,
                                 void* stage_dev, size_t stage_bytes, size_t* codes_off,
                                 size_t* scales_off, int nthreads, int64_t* n_unique, void* stream);

/* ------------------------------------------------------------------------
 * mole_check_ids: optional device-side check of token ids (inference
 * section: a token's rows are found by direct addressing on its id, and the
 * combines do not check ids held in device memory).  Adds to *count (one
 * int32 in device memory, 4-byte aligned; the caller zeroes it) the number
 * of ids[0..T) outside [0, V).  One launch on `stream`, asynchronous; run it
 * before a combine and read *count when convenient (e.g. in debug builds).
 * T == 0 is a no-op.
 * ------------------------------------------------------------------------ */
int mole_check_ids(const int64_t* ids, int64_t T, int64_t V, int32_t* count, void* stream);

/* ------------------------------------------------------------------------
 * mole_lookup_combine_grouped: the combine of mole_lookup_combine with the
 * batch grouped by token id on the device (inference section: each token's
 * expert outputs are fetched by its id; results section: the table keeps
 * redundancy -- a prefill batch of natural text repeats ids, and every
 * token of one id reads the same N x D slab).  Two launches on `stream`:
 * the first groups each chunk of 4096 tokens so that equal ids are
 * adjacent (an LDS hash table and a scan) and, in other workgroups of the
 * same grid, routes the tokens (bf16 matrix cores, fp32 softmax, as
 * mole_lookup_combine), both into the workspace; the second reads each run
 * of equal ids' slab once per 16 grouped positions instead of once per
 * token.
 *   ids [T] int64 (device, 8-byte aligned)   h [T][D]   w_r [N][D]
 *   lut [V][N][D] (bf16)   y [T][D] fp32 (written)
 * y equals mole_lookup_combine's up to fp32 summation order (each token's
 * sum runs over its own gates and slab in expert order).  bf16 only, N <= 16,
 * D % 8 == 0 and V < 2^31 (MOLE_ERR_UNSUPPORTED otherwise).  Device ids are
 * not range-checked (see mole_check_ids).  T == 0 is a no-op.
 *
 * workspace: device scratch, 16-byte aligned, of at least the size that
 * mole_lookup_combine_grouped_workspace_size(T) returns (72 bytes per
 * token, each section rounded up to 256 bytes; 0 for T == 0): the grouped
 * positions and every token's gates.  Contents on return are unspecified.  No memset and no host synchronisation (capturable in a HIP
 * graph).
 * ------------------------------------------------------------------------ */
int mole_lookup_combine_grouped_workspace_size(int64_t T, size_t* bytes);

int mole_lookup_combine_grouped(const int64_t* ids, const void* h, const void* w_r, const void* lut, float* y,
                                int64_t T, int64_t V, int64_t D, int64_t N, int dtype, void* workspace,
                                size_t workspace_bytes, void* stream);

/* mole_lookup_combine_grouped_mapped: mole_lookup_combine_grouped with the
 * table lut_host [V][N][D] (bf16) left in page-locked host memory allocated
 * through HIP, read in place as in mole_lookup_combine_mapped (same checks
 * and MOLE_ERR_MEMORY).  Each run of equal ids reads its slab over PCIe
 * once, so a batch with repeated ids moves about its distinct rows instead
 * of one slab per token; ids, h, w_r, y and the workspace are device memory
 * as for mole_lookup_combine_grouped. */
int mole_lookup_combine_grouped_mapped(const int64_t* ids, const void* h, const void* w_r, const void* lut_host,
                                       float* y, int64_t T, int64_t V, int64_t D, int64_t N, int dtype,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* mole_lookup_combine_nf3_grouped: the NF3 combine of mole_lookup_combine_nf3
 * over the batch grouped by id on the device (the grouping and routing
 * launch of mole_lookup_combine_grouped, then the NF3 decode with each
 * position's token, row and gates from the workspace): tokens that share an
 * id run on neighbouring workgroups, so their rows are read from memory
 * about once.  bf16 h and w_r, N <= 16, D % 64 == 0 (MOLE_ERR_UNSUPPORTED /
 * MOLE_ERR_DIM otherwise); the workspace is device memory of at least
 * mole_lookup_combine_grouped_workspace_size(T) bytes, 16-byte aligned, and
 * needs no clearing.
 * mole_lookup_combine_nf3_grouped_mapped: the same with codes_host and
 * scales_host in page-locked host memory, read in place as in
 * mole_lookup_combine_nf3_mapped (same checks and MOLE_ERR_MEMORY).  For a
 * batch with repeated ids this moves about its distinct rows over PCIe. */
int mole_lookup_combine_nf3_grouped(const int64_t* ids, const void* h, const void* w_r, const uint8_t* codes,
                                    const uint16_t* scales, float* y, int64_t T, int64_t V, int64_t D, int64_t N,
                                    int dtype_h, void* workspace, size_t workspace_bytes, void* stream);

int mole_lookup_combine_nf3_grouped_mapped(const int64_t* ids, const void* h, const void* w_r,
                                           const uint8_t* codes_host, const uint16_t* scales_host, float* y,
                                           int64_t T, int64_t V, int64_t D, int64_t N, int dtype_h,
                                           void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * mole_lookup_combine_grouped_noalloc: mole_lookup_combine_grouped for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same arguments and
 * result, minus the workspace: the library keeps it in a static device array
 * of 4.5 MiB (each GPU it runs on holds one until the process ends), which
 * serves batches of up to MOLE_GROUPED_NOALLOC_MAX_T tokens
 * (MOLE_ERR_UNSUPPORTED above).  Allocates nothing.  Runs on the device of
 * `stream` (the current device for the null stream).  Every call on one GPU
 * shares that array: calls that overlap on one GPU (different streams, or
 * threads) race and must be ordered by the caller, e.g. on one stream.
 * ------------------------------------------------------------------------ */
#define MOLE_GROUPED_NOALLOC_MAX_T 65536

int mole_lookup_combine_grouped_noalloc(const int64_t* ids, const void* h, const void* w_r, const void* lut,
                                        float* y, int64_t T, int64_t V, int64_t D, int64_t N, int dtype,
                                        void* stream);

/* ------------------------------------------------------------------------
 * Disk tier: the NF3 table in a file (inference section: the table is kept
 * in lower-tier storage and only the retrieved outputs are loaded into GPU
 * memory; the offloading discussion names CPU memory and disk as such
 * tiers).  The file holds one record per vocabulary row, so a token's row
 * is one contiguous read:
 *
 *   bytes [0, 64): header, little-endian
 *       char    magic[8]      "MOLENF3" and a zero byte
 *       uint32  version       1
 *       uint32  header_bytes  64
 *       int64   V, N, D
 *       int64   record_bytes  N*3D/8 + N*(D/64)*2
 *       int64   data_offset   64
 *       int64   reserved      0
 *   record v at data_offset + v*record_bytes: the row's NF3 codes
 *       [N][3D/8] (as mole_pack_nf3 writes codes[v]), then its fp16 scales
 *       [N][D/64] (scales[v]).
 *
 * mole_nf3_file_write: host-only.  Creates (or truncates) `path` and writes
 * the header and the V records from a packed table in host memory
 * (codes_host [V][N][3D/8], scales_host [V][N][D/64]).  MOLE_ERR_IO if the
 * file cannot be created or written.
 *
 * mole_nf3_file_shape: host-only.  Reads the header of the open file `fd`
 * into *V, *N, *D.  MOLE_ERR_IO if it cannot be read, MOLE_ERR_FORMAT if it
 * is not a version-1 table file.
 *
 * mole_gather_nf3_file: host-only.  As mole_gather_nf3_host, with the rows
 * read from the open table file `fd` (one positioned read per distinct id,
 * straight into the two staging sections; the caller's file offset is not
 * used or moved).  MOLE_ERR_DIM if the header's V, N, D differ from the
 * arguments; MOLE_ERR_IO on a failed or short read.
 *
 * mole_lookup_combine_nf3_file: as mole_lookup_combine_nf3_host, with the
 * distinct rows read from the table file `fd` into the pinned staging area
 * (same staging contract, mole_nf3_host_staging_size).  The reads happen on
 * the calling thread before the copy is enqueued; y is written on `stream`.
 * ------------------------------------------------------------------------ */
int mole_nf3_file_write(const char* path, const uint8_t* codes_host, const uint16_t* scales_host,
                        int64_t V, int64_t N, int64_t D);

int mole_nf3_file_shape(int fd, int64_t* V, int64_t* N, int64_t* D);

int mole_gather_nf3_file(int fd, const int64_t* ids_host, int64_t T, int64_t V, int64_t N,
                         int64_t D, uint8_t* codes_stage_host, uint16_t* scales_stage_host,
                         int64_t* remap_host, int64_t* n_unique, int nthreads);

int mole_lookup_combine_nf3_file(int fd, const int64_t* ids_host, const void* h, const void* w_r,
                                 void* stage_host, void* stage_dev, size_t stage_bytes, float* y,
                                 int64_t T, int64_t V, int64_t D, int64_t N, int dtype_h,
                                 int nthreads, int64_t* n_unique, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOLE_H */
