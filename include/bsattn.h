/*
 * bsattn.h -- C ABI of the block-sparse flash-attention forward library for
 * AMD Instinct MI355X (gfx950), libbsattn.so.
 *
 * The operation.  For every batch b, head h and query row r:
 *   out[b,h,r,:] = sum_j softmax_j(scale * q[b,h,r,:] . k[b,h,j,:]) * v[b,h,j,:]
 *   lse[b,h,r]   = log sum_j exp(scale * q[b,h,r,:] . k[b,h,j,:])      (natural log)
 * where j runs only over keys whose key block is active for the query block of r:
 * block_mask[b,h,r/block_q,j/block_k] != 0.  All other scores count as -inf.  A
 * row with no active key block gets out = 0 and lse = -inf.
 * Source: "Writing Pallas Kernels for JAX" (rajatpandit.com), section "Writing the
 * Kernel Logic: Load, Compute, Store" (scaled scores, mask to -inf, softmax, times
 * V); "Pallas-Triton kernels and kernel auto-tuning" (robertdyro.com), section
 * "Flash Attention" (the tiled method computes the operator exactly, never
 * building the score matrix).
 *
 * Conventions shared by every entry point.
 *  - Every array argument is a DEVICE pointer owned by the caller.  Nothing is
 *    allocated on the call path of bsattn_compact_mask, bsattn_plan, bsattn_fwd,
 *    bsattn_fwd_config, bsattn_fwd_planned or bsattn_fwd_compacted; the caller
 *    passes a workspace.
 *  - Layouts: q, k, v, out are [B][H][S][D], contiguous, D fastest, all of one
 *    element type (fp32 or bf16 as IEEE bits); lse is float [B][H][S];
 *    block_mask is uint8 [B][H][S/block_q][S/block_k], any nonzero byte = active.
 *  - stream is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    asynchronously; results are valid once the stream has synchronised.
 *  - Every argument check runs on the host before any device work.  A failed
 *    check returns a nonzero bsattn_status and touches nothing.  A failed HIP
 *    call returns BSATTN_ERR_HIP and bsattn_last_hip_error() gives its code.
 *    No exception crosses this boundary and nothing aborts.
 *  - Calls on different streams may run concurrently if they use different
 *    workspaces and outputs.
 */
#ifndef BSATTN_H
#define BSATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { BSATTN_F32 = 0, BSATTN_BF16 = 1 } bsattn_dtype;

typedef enum {
    BSATTN_OK = 0,
    BSATTN_ERR_NULL = 1,        /* a required pointer is NULL */
    BSATTN_ERR_SHAPE = 2,       /* a size <= 0, S not divisible by a block size,
                                   an index would overflow int32, B*H*S*D >= 2^40,
                                   or S*D*4 >= 2^31 (one head is read through a
                                   buffer with a 32-bit byte range) */
    BSATTN_ERR_UNSUPPORTED = 3, /* D, dtype, block size or tile config not built */
    BSATTN_ERR_ALIGN = 4,       /* q/k/v/out not 16-byte or lse not 4-byte aligned */
    BSATTN_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required */
    BSATTN_ERR_SCALE = 6,       /* scale is NaN or infinite */
    BSATTN_ERR_ALIAS = 7,       /* out or lse overlaps q, k or v (or each other), or
                                   a forward workspace overlaps any of them or the
                                   mask arrays its plan reads */
    BSATTN_ERR_HIP = 8,         /* a HIP runtime call failed */
    BSATTN_ERR_IO = 9           /* a tuning-cache file could not be read or written */
} bsattn_status;

/* Kernel tiling of the attention kernel (the autotuner's search space).
 *   tile_q  query rows per workgroup: 64 or 128, must divide block_q; or 256
 *           with block_q 128: a workgroup takes two adjacent mask rows of a head
 *           (query blocks 2j and 2j+1), loads each K/V tile of the union of
 *           their block lists once for both, and each row computes only its own
 *           blocks (at most 2048 key blocks per row);
 *   tile_k  keys per inner step: 32, 64 or 128, must divide block_k;
 *   waves   wavefronts per workgroup (64 lanes each); a wave owns 32 or 64
 *           query rows, so waves is tile_q / 32 or tile_q / 64, or 8 with
 *           tile_q 128 for the two-group schedule (two 4-wave groups on the
 *           same rows, each taking every other key tile, merged at the end);
 *   stages  K/V tiles resident in LDS: 1 (load, barrier, compute), 2 or 3
 *           (later tiles are written while the current one is consumed).
 * bsattn_list_configs gives the combinations that are built.
 * A zero field means "choose automatically".  The kernel tiling never changes
 * the result beyond fp32 rounding order: block_q and block_k (the mask
 * granularity) do. */
typedef struct {
    int tile_q;
    int tile_k;
    int waves;
    int stages;
} bsattn_tile_config;

/* One timed variant, in the column layout of the tuning table in
 * "Pallas-Triton kernels and kernel auto-tuning", section "Auto-tuning". */
typedef struct {
    int id;
    bsattn_tile_config cfg;
    double t_mean_s;
    double t_std_s;
    double t_min_s;
} bsattn_tune_result;

/* Library version, (major << 16) | (minor << 8) | patch. */
int bsattn_version(void);

/* Static text for a status code (never NULL). */
const char* bsattn_status_string(int status);

/* The hipError_t of the last failed HIP call in this thread (0 if none). */
int bsattn_last_hip_error(void);

/* Workspace bytes needed by bsattn_compact_mask for a mask of B*H*n_q rows of
 * n_k blocks.  Returns BSATTN_ERR_SHAPE / BSATTN_ERR_NULL on bad arguments. */
int bsattn_compact_workspace_size(int B, int H, int n_q, int n_k, size_t* bytes);

/* Mask compaction (the first step of the forward): the per-query-block lists of
 * active key blocks, in CSR form.  For each mask row in (b, h, qi) row-major
 * order the active kj are listed in ascending order:
 *   row_ptr[0] = 0, row_ptr[i+1] = row_ptr[i] + (active blocks of row i),
 *   col_idx[row_ptr[i] .. row_ptr[i+1]) = those kj.
 * row_ptr has B*H*n_q + 1 entries; col_idx must have room for B*H*n_q*n_k
 * entries (only the first row_ptr[B*H*n_q] are written).  The result is unique
 * and bit-exact.  The mask pages describe the block-skipping idea only loosely
 * ("Writing Pallas Kernels for JAX", section "Writing the Kernel Logic": the mask
 * tile is read once per chunk); the list form is this library's. */
int bsattn_compact_mask(const uint8_t* block_mask, int B, int H, int n_q, int n_k,
                        int32_t* row_ptr, int32_t* col_idx, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Workspace bytes needed by bsattn_fwd, bsattn_fwd_config, bsattn_plan and
 * bsattn_fwd_planned (the same figure for all four). */
int bsattn_workspace_size(int B, int H, int S, int block_q, int block_k, size_t* bytes);

/* The forward pass: mask compaction, then the fused attention kernel (S = scale
 * Q K^T per active tile pair, an online softmax with running row max and row sum,
 * O += P V), writing out (same element type as q) and lse.
 *   D        64 or 128;   block_q, block_k   64 or 128;   S % block_q == 0 and
 *            S % block_k == 0;   scale  any finite fp32 (negative and 0 allowed);
 *   dtype    BSATTN_BF16 (fp32 accumulation, bf16 out) or BSATTN_F32.
 * The tile config comes from the environment (BSATTN_CONFIG="tq,tk,waves,stages"),
 * else from the autotuner's cache for this shape, else a built-in default: for bf16
 * with block_q 128 and at most 2048 key blocks per row the row-pair config
 * (256, 128, 8, 2) for D 128 and (256, 64, 8, 2) for D 64 (the other key-tile
 * depth if block_k rules the first out), otherwise the first legal entry of
 * bsattn_list_configs. */
int bsattn_fwd(const void* q, const void* k, const void* v, const uint8_t* block_mask,
               void* out, float* lse, int B, int H, int S, int D, int block_q, int block_k,
               float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream);

/* As bsattn_fwd with an explicit tile config (cfg == NULL or all-zero = auto).
 * It is exactly bsattn_plan followed by bsattn_fwd_planned on one workspace. */
int bsattn_fwd_config(const void* q, const void* k, const void* v, const uint8_t* block_mask,
                      void* out, float* lse, int B, int H, int S, int D, int block_q,
                      int block_k, float scale, int dtype, void* workspace,
                      size_t workspace_bytes, const bsattn_tile_config* cfg, void* stream);

/* The plan: the mask-dependent first step of bsattn_fwd, on its own.  Writes
 * into workspace, for every mask row in (b, h, qi) row-major order, the number of
 * active key blocks and their kj in ascending order (a list padded to n_k
 * entries), then the order in which the attention kernel dispatches its
 * workgroups: rows cut into 8 contiguous chunks (one per XCD of the chip), each
 * chunk head by head in (b, h) order and each head's rows longest first (or,
 * when a chunk spans more than 4096 head x count bins, longest first overall).  With R = B*H*(S/block_q), n_k = S/block_k and
 * A(x) = x rounded up to a multiple of 256, the plan is three int32 arrays:
 *   counts[R]              at byte 0;
 *   lists[R][n_k]          at byte A(4R), row i's kj in lists[i][0 .. counts[i]);
 *   order[8 * ceil(R/8)]   at byte A(4R) + A(4 R n_k): chunk x is
 *                          order[x*ceil(R/8) ..], its rows in the order above,
 *                          then -1 past the last row;
 *   porder[8 * ceil(P/8)]  at byte A(4R) + A(4 R n_k) + A(4 * 8 ceil(R/8)): the
 *                          same for the P = B*H*ceil(S/block_q / 2) pairs of
 *                          query blocks (2j, 2j+1) of a head, pair index
 *                          (b*H + h)*ceil(S/block_q / 2) + j, keyed by the
 *                          longer list of the two (used by tile_q 256).
 * The plan depends only on block_mask and (B, H, S,
 * block_q, block_k), never on q/k/v, D, dtype, scale or the tile config, so one
 * plan serves every call that shares the mask (the block mask is fixed ahead of
 * the kernel: "Writing Pallas Kernels for JAX", section "Writing the Kernel
 * Logic").  workspace_bytes >= bsattn_workspace_size(B, H, S, block_q, block_k);
 * the workspace is owned by the caller and must stay alive and unmodified until
 * the last bsattn_fwd_planned that reads it has completed on its stream. */
int bsattn_plan(const uint8_t* block_mask, int B, int H, int S, int block_q, int block_k,
                void* workspace, size_t workspace_bytes, void* stream);

/* The attention kernel alone, on a plan written by bsattn_plan for the same
 * mask and shape (B, H, S, block_q, block_k); any tile config may run on any
 * plan.  workspace is only read.  A workspace that holds no such plan gives
 * undefined values in out and lse but no access outside q, k, v, out, lse and
 * the workspace's first bsattn_workspace_size bytes (counts and entries are
 * clamped to the shape).  Arguments and checks otherwise as bsattn_fwd_config,
 * plus BSATTN_ERR_ALIAS when the plan region overlaps q, k, v, out or lse. */
int bsattn_fwd_planned(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                       int H, int S, int D, int block_q, int block_k, float scale, int dtype,
                       const void* workspace, size_t workspace_bytes,
                       const bsattn_tile_config* cfg, void* stream);

/* bsattn_fwd_config for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the plan goes to a fixed device array inside the library instead of a caller
 * workspace, of bsattn_noalloc_max_bytes() = 16 MiB per GPU, held until the
 * process ends.  This call allocates nothing and calls no allocating routine.
 * Arguments, layouts and checks as bsattn_fwd_config (cfg may be NULL); a shape
 * whose plan (bsattn_workspace_size) exceeds the array returns
 * BSATTN_ERR_WORKSPACE before any device work.  The array of the calling
 * thread's current device is used, which must be the device of stream.  Every
 * call on one GPU shares that GPU's array, and each call's plan launch rewrites
 * all of it that its attention launch reads, so nothing needs clearing between
 * calls; but calls that overlap on one GPU (other streams, other host threads)
 * race on the array and must be serialised by the caller. */
int bsattn_fwd_noalloc(const void* q, const void* k, const void* v, const uint8_t* block_mask,
                       void* out, float* lse, int B, int H, int S, int D, int block_q, int block_k,
                       float scale, int dtype, const bsattn_tile_config* cfg, void* stream);

/* Size in bytes of the fixed device array bsattn_fwd_noalloc plans into. */
size_t bsattn_noalloc_max_bytes(void);

/* The attention kernel alone, on lists already built by bsattn_compact_mask
 * (row_ptr, col_idx as that call wrote them, for the same mask).  This is the
 * attention step of bsattn_fwd reading CSR lists instead of a plan, for callers
 * that keep the mask in CSR form; workgroups go in mask-row order (no
 * longest-first dispatch).  row_ptr holds B*H*(S/block_q) + 1 entries and
 * col_idx col_idx_len entries (both on the device).  Malformed lists give
 * undefined values in out and lse but never an access outside them: each row's
 * span [row_ptr[r], row_ptr[r+1]) is clamped into [0, col_idx_len), its count to
 * at most S/block_k, and each entry into [0, S/block_k).  col_idx_len = 0 with a
 * non-NULL col_idx is allowed (every row is then empty).  cfg as in
 * bsattn_fwd_config. */
int bsattn_fwd_compacted(const void* q, const void* k, const void* v, const int32_t* row_ptr,
                         const int32_t* col_idx, size_t col_idx_len, void* out, float* lse, int B,
                         int H, int S, int D, int block_q, int block_k, float scale, int dtype,
                         const bsattn_tile_config* cfg, void* stream);

/* Number of tile configs built for (dtype, D, block_q, block_k), and the configs
 * themselves (up to cap are written to cfgs; cfgs may be NULL to count). */
int bsattn_list_configs(int dtype, int D, int block_q, int block_k, bsattn_tile_config* cfgs,
                        int cap, int* n);

/* ---- Element-level masks -------------------------------------------------------
 * The mask of "Writing Pallas Kernels for JAX" (section "Writing the Kernel Logic:
 * Load, Compute, Store") is an element tile per (query block, key block): a score
 * is kept where the tile is set and is -inf elsewhere.  Here it is given as
 *   block_states   uint8 [B][H][S/block_q][S/block_k]: 0 = empty block (every
 *                  element masked, never visited), 1 = full block (every element
 *                  kept), any other value = partial block;
 *   partial_index  int32 [B][H][S/block_q][S/block_k]: for a partial block, the
 *                  tile that holds its bits (read only where the state is > 1;
 *                  an index outside [0, n_tiles) is clamped into it);
 *   partial_bits   uint32 [n_tiles][block_q][block_k / 32]: element (i, j) of a
 *                  partial block is kept iff bit j % 32 of word j / 32 of row i of
 *                  its tile is set.  Tiles may be shared (e.g. one lower-triangular
 *                  tile for every diagonal block of an exact token-causal mask).
 * A query row with no kept element gets out = 0 and lse = -inf.  dtype bf16 or
 * fp32 as for bsattn_fwd (fp32 runs the fp32 kernel's configs); 1 <= n_tiles <= 32767 and
 * S / block_k <= 65536, else BSATTN_ERR_SHAPE.  The workspace is the same size
 * as for bsattn_fwd (bsattn_workspace_size) and has the plan layout of
 * bsattn_plan, except that a list entry of a partial block is kj | (tile + 1) << 16.
 * Tile configs: bsattn_list_configs_elem (row-pair configs, tile_q 256, need
 * block_q 128 and at most 2048 key blocks per row, as for block masks); with no
 * config the row-pair (256, 64, 8, 2) where it is legal, else the first legal
 * entry of that list. */

/* Plan for an element-level mask: bsattn_plan's lists and dispatch orders over
 * the non-empty blocks, each entry carrying its tile.  Arguments and ownership as
 * bsattn_plan; BSATTN_ERR_NULL for a NULL block_states, partial_index or workspace,
 * BSATTN_ERR_ALIGN if workspace or partial_index is not 4-byte aligned. */
int bsattn_plan_elem(const uint8_t* block_states, const int32_t* partial_index, int n_tiles, int B,
                     int H, int S, int block_q, int block_k, void* workspace,
                     size_t workspace_bytes, void* stream);

/* The attention kernel alone on a plan from bsattn_plan_elem (same mask, shape
 * and n_tiles); partial_bits as above, only read, 4-byte aligned, not
 * overlapping out, lse or the workspace (BSATTN_ERR_ALIAS).  Other arguments and
 * checks as bsattn_fwd_planned; cfg selects among bsattn_list_configs_elem. */
int bsattn_fwd_planned_elem(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                            int H, int S, int D, int block_q, int block_k, float scale, int dtype,
                            const uint32_t* partial_bits, int n_tiles, const void* workspace,
                            size_t workspace_bytes, const bsattn_tile_config* cfg, void* stream);

/* The forward pass with an element-level mask: exactly bsattn_plan_elem followed
 * by bsattn_fwd_planned_elem on one workspace. */
int bsattn_fwd_elem(const void* q, const void* k, const void* v, const uint8_t* block_states,
                    const int32_t* partial_index, const uint32_t* partial_bits, int n_tiles, void* out,
                    float* lse, int B, int H, int S, int D, int block_q, int block_k, float scale,
                    int dtype, void* workspace, size_t workspace_bytes,
                    const bsattn_tile_config* cfg, void* stream);

/* Tile configs built for element-level masks (as bsattn_list_configs; zero for
 * BSATTN_F32). */
int bsattn_list_configs_elem(int dtype, int D, int block_q, int block_k, bsattn_tile_config* cfgs,
                             int cap, int* n);

/* ---- fp8 forward ------------------------------------------------------------------
 * The forward above with q, k, v in fp8 e4m3 (OCP form, one byte per element, the
 * layout of torch.float8_e4m3fn), out in bf16 and lse in fp32 ("JAX Pallas and
 * Blackwell", section "What the Tutorial Covers": fp32 accumulators, fp8 only at
 * the boundary, in a kernel measured against the fp8 peak).  Both products run on the fp8 matrix cores with fp32
 * accumulation; scores, row maxima, exponentials, row sums and lse are fp32; the
 * softmax weights are rounded to e4m3 (relative error <= 2^-4, values below 2^-9
 * of the row's reference maximum flushed towards 0) before they multiply V.
 *   q, k, v  e4m3 [B][H][S][D] (device); out bf16 [B][H][S][D]; lse float
 *            [B][H][S]; block_mask as the forward.
 * D 64 or 128, block_q and block_k 64 or 128 (BSATTN_ERR_UNSUPPORTED); q, k, v,
 * out and the workspace 16-byte aligned, lse 4-byte aligned (BSATTN_ERR_ALIGN);
 * out or lse overlapping q, k, v or each other, or the workspace overlapping any
 * of them, gives BSATTN_ERR_ALIAS; other checks as bsattn_fwd.  The workspace
 * (bsattn_fp8_workspace_size bytes) holds the plan of bsattn_plan followed by a
 * copy of V rearranged per 64-key tile (B*H*S*D bytes, rewritten by every call).
 * bsattn_fwd_fp8_planned runs on a plan that bsattn_plan wrote into the first
 * part of that workspace.  Asynchronous on stream; nothing is allocated. */
int bsattn_fp8_workspace_size(int B, int H, int S, int D, int block_q, int block_k, size_t* bytes);
int bsattn_fwd_fp8(const void* q, const void* k, const void* v, const uint8_t* block_mask, void* out,
                   float* lse, int B, int H, int S, int D, int block_q, int block_k, float scale,
                   void* workspace, size_t workspace_bytes, void* stream);
int bsattn_fwd_fp8_planned(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                           int H, int S, int D, int block_q, int block_k, float scale, void* workspace,
                           size_t workspace_bytes, void* stream);

/* The fp8 forward with an element-level mask: block_states, partial_index,
 * partial_bits and n_tiles as for bsattn_fwd_elem ("Writing Pallas Kernels for
 * JAX", section "Writing the Kernel Logic": the mask tile is element-level, dropped
 * scores are -inf), q, k, v, out, lse, the workspace (bsattn_fp8_workspace_size
 * bytes) and the precision as for bsattn_fwd_fp8.  A query row with no kept element
 * gets out = 0 and lse = -inf.  Checks: those of bsattn_fwd_fp8 and of
 * bsattn_fwd_elem (n_tiles in 1 .. 32767 and S / block_k <= 65536, else
 * BSATTN_ERR_SHAPE; partial_bits and partial_index 4-byte aligned; partial_bits
 * overlapping out, lse or the workspace gives BSATTN_ERR_ALIAS), all before any
 * device work.  bsattn_fwd_fp8_planned_elem runs on a plan that bsattn_plan_elem
 * wrote into the first part of that workspace (same mask, shape and n_tiles). */
int bsattn_fwd_fp8_elem(const void* q, const void* k, const void* v, const uint8_t* block_states,
                        const int32_t* partial_index, const uint32_t* partial_bits, int n_tiles, void* out,
                        float* lse, int B, int H, int S, int D, int block_q, int block_k, float scale,
                        void* workspace, size_t workspace_bytes, void* stream);
int bsattn_fwd_fp8_planned_elem(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                                int H, int S, int D, int block_q, int block_k, float scale,
                                const uint32_t* partial_bits, int n_tiles, void* workspace,
                                size_t workspace_bytes, void* stream);

/* ---- Ragged dot -------------------------------------------------------------------
 * "Pallas-Triton kernels and kernel auto-tuning", section "Ragged Dot (Group Matrix
 * Multiplication)": rhs is a stack of G expert matrices; the rows of lhs go to the
 * experts in order, group g taking the next group_sizes[g] rows, and output row i
 * is lhs row i times its group's matrix:
 *   lhs          bf16 [M][K] row-major (device);
 *   rhs          bf16 [G][K][N] row-major (device);
 *   group_sizes  int32 [G] (device); a negative size counts as 0, and rows past M
 *                are dropped (groups are clamped to [0, M));
 *   out          [M][N], bf16 (out_dtype BSATTN_BF16, round to nearest even) or fp32
 *                (BSATTN_F32); rows past the sum of the sizes are written as 0.
 * fp32 accumulation.  K % 64 == 0, N % 128 == 0, K*N*2 < 2^31 (one expert is read
 * through a buffer with a 32-bit range), else BSATTN_ERR_SHAPE; dtype must be
 * BSATTN_BF16 (else BSATTN_ERR_UNSUPPORTED).  lhs, rhs, out and workspace 16-byte
 * aligned, group_sizes 4-byte aligned (BSATTN_ERR_ALIGN); out or the workspace
 * overlapping an input or each other gives BSATTN_ERR_ALIAS.  The workspace
 * (bsattn_ragged_dot_workspace_size bytes, owned by the caller) holds the work
 * plan: one item per (256-row tile, group) pair that share rows.  Asynchronous on
 * stream; nothing is allocated. */
int bsattn_ragged_dot_workspace_size(int M, int G, size_t* bytes);
int bsattn_ragged_dot(const void* lhs, const void* rhs, const int32_t* group_sizes, void* out, int M,
                      int K, int N, int G, int dtype, int out_dtype, void* workspace,
                      size_t workspace_bytes, void* stream);

/* The two steps of bsattn_ragged_dot on their own.  bsattn_ragged_plan reads
 * group_sizes and writes the work plan into workspace (items of int32 {row tile,
 * group or -1 for rows of no group, first row, end row}, then their count);
 * bsattn_ragged_dot_planned runs the product (and the zero rows) on a plan made
 * for the same M and G and only reads the workspace.  A workspace holding no such
 * plan gives undefined values in out (item fields are not re-checked). */
int bsattn_ragged_plan(const int32_t* group_sizes, int M, int G, void* workspace,
                       size_t workspace_bytes, void* stream);
int bsattn_ragged_dot_planned(const void* lhs, const void* rhs, void* out, int M, int K, int N, int G,
                              int dtype, int out_dtype, const void* workspace, size_t workspace_bytes,
                              void* stream);

/* ---- Backward ---------------------------------------------------------------------
 * Gradients of the forward above ("Writing Pallas Kernels for JAX", section "The
 * Empathy of the Void": a hand-written kernel gets no automatic gradient, its
 * author writes one).  For the upstream gradient dout = dL/dout, with
 * P[r][j] = exp(scale * q_r . k_j - lse_r) on the active keys of row r (0 elsewhere):
 *   dv_j = sum_r P[r][j] dout_r,            dP[r][j] = dout_r . v_j,
 *   delta_r = dout_r . out_r,               dS[r][j] = P[r][j] (dP[r][j] - delta_r),
 *   dq_r = scale sum_j dS[r][j] k_j,        dk_j = scale sum_r dS[r][j] q_r.
 * Arguments:
 *   q, k, v, out, dout  bf16 [B][H][S][D] (device; out and lse as written by the
 *                       forward of the same q, k, v, mask and scale);
 *   lse                 float [B][H][S] (device; -inf marks a row that saw no key);
 *   block_mask          uint8 [B][H][S/block_q][S/block_k] (device), as the forward;
 *   dq, dk, dv          [B][H][S][D] (device), bf16 (grad_dtype BSATTN_BF16, round to
 *                       nearest even) or fp32 (BSATTN_F32); every element is written
 *                       (rows and keys that no active block touches get 0).
 * dtype must be BSATTN_BF16, D 64 or 128, block_q and block_k 64 or 128
 * (BSATTN_ERR_UNSUPPORTED); shapes as the forward (BSATTN_ERR_SHAPE).  q, k, v, out,
 * dout, dq, dk, dv and the workspace 16-byte aligned, lse 4-byte aligned
 * (BSATTN_ERR_ALIGN); scale finite (BSATTN_ERR_SCALE); dq, dk, dv or the
 * workspace overlapping any other array argument or each other gives
 * BSATTN_ERR_ALIAS.  fp32 accumulation; the results do not depend on the launch
 * order (no atomics).  The workspace (bsattn_bwd_workspace_size bytes, owned by
 * the caller) holds the plan -- the forward plan of bsattn_plan (row lists, for
 * dq), then per key block (b, h, kj) its count and ascending list of query blocks
 * padded to n_q (int32, for dk and dv), and the dk/dv work items: a key block
 * seen by many query blocks is cut into pieces whose fp32 partial sums are added
 * in piece order -- and a scratch part: 8 bytes per row (lse * log2 e,
 * dout . out) and the partial sums (max(16, B*H*(S/block_k)/4) slots of
 * 2 * block_k * 128 floats).  Asynchronous on stream; nothing is allocated. */
int bsattn_bwd_workspace_size(int B, int H, int S, int block_q, int block_k, size_t* bytes);
int bsattn_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
               const void* dout, const uint8_t* block_mask, int B, int H, int S, int D, int block_q,
               int block_k, float scale, int dtype, void* dq, void* dk, void* dv, int grad_dtype,
               void* workspace, size_t workspace_bytes, void* stream);

/* The two steps of bsattn_bwd on their own.  bsattn_bwd_plan reads the mask and
 * writes the plan part of the workspace (it depends on the mask and shape only,
 * so one plan serves every backward call with that mask);
 * bsattn_bwd_planned runs the gradient kernels on it.  parts selects them (a
 * nonzero OR of the flags below, else BSATTN_ERR_UNSUPPORTED; BSATTN_BWD_ALL
 * is what bsattn_bwd runs): PREP writes the per-row scratch from out, lse and
 * dout; DQ writes dq; DKDV writes dk and dv.  DQ and DKDV read the scratch, so a
 * call without PREP relies on an earlier call with PREP on the same workspace,
 * out, lse and dout (a caller with no gradient for q runs PREP | DKDV).  Arrays
 * a call does not write are left untouched.  The lists' entries are clamped
 * into range, so a workspace holding no such plan gives wrong values but no
 * access out of bounds. */
enum { BSATTN_BWD_PREP = 4, BSATTN_BWD_DQ = 1, BSATTN_BWD_DKDV = 2, BSATTN_BWD_ALL = 7 };
int bsattn_bwd_plan(const uint8_t* block_mask, int B, int H, int S, int block_q, int block_k,
                    void* workspace, size_t workspace_bytes, void* stream);
int bsattn_bwd_planned(const void* q, const void* k, const void* v, const void* out, const float* lse,
                       const void* dout, int B, int H, int S, int D, int block_q, int block_k,
                       float scale, int dtype, void* dq, void* dk, void* dv, int grad_dtype, int parts,
                       void* workspace, size_t workspace_bytes, void* stream);

/* The backward of the element-level-mask forward (bsattn_fwd_elem): the gradients
 * above with P[r][j] = 0 for every (query, key) pair the element mask drops
 * ("Writing Pallas Kernels for JAX", section "Writing the Kernel Logic": a score
 * counts only where the mask tile is set; section "The Empathy of the Void": the
 * kernel's author writes its gradient).  block_states, partial_index,
 * partial_bits and n_tiles as in bsattn_fwd_elem (device; a tile index outside
 * [0, n_tiles) is clamped); out and lse are that forward's (a row that keeps
 * nothing has lse = -inf and gets dq = 0).  Other arguments, the workspace
 * (bsattn_bwd_workspace_size bytes: the plan is built from the nonzero block
 * states) and the error behaviour as bsattn_bwd; in addition NULL mask arrays give
 * BSATTN_ERR_NULL, n_tiles outside [1, 32767] BSATTN_ERR_SHAPE, partial_index or
 * partial_bits not 4-byte aligned BSATTN_ERR_ALIGN, and dq, dk, dv or the
 * workspace overlapping the mask arrays BSATTN_ERR_ALIAS.  Asynchronous on
 * stream; nothing is allocated. */
int bsattn_bwd_elem(const void* q, const void* k, const void* v, const void* out, const float* lse,
                    const void* dout, const uint8_t* block_states, const int32_t* partial_index,
                    const uint32_t* partial_bits, int n_tiles, int B, int H, int S, int D, int block_q,
                    int block_k, float scale, int dtype, void* dq, void* dk, void* dv, int grad_dtype,
                    void* workspace, size_t workspace_bytes, void* stream);

/* The gradient kernels of bsattn_bwd_elem alone, on a plan that bsattn_bwd_plan
 * made from the same block_states (as bsattn_bwd_planned for the block mask;
 * parts as there).  Argument checks as bsattn_bwd_elem and bsattn_bwd_planned. */
int bsattn_bwd_planned_elem(const void* q, const void* k, const void* v, const void* out, const float* lse,
                            const void* dout, const uint8_t* block_states, const int32_t* partial_index,
                            const uint32_t* partial_bits, int n_tiles, int B, int H, int S, int D,
                            int block_q, int block_k, float scale, int dtype, void* dq, void* dk, void* dv,
                            int grad_dtype, int parts, void* workspace, size_t workspace_bytes, void* stream);

/* Autotuner ("Pallas-Triton kernels and kernel auto-tuning", section
 * "Auto-tuning": parameterise tile sizes, warps and pipeline depth, time every
 * point, keep the fastest).  Times bsattn_fwd_config for every built config of
 * this shape on the caller's buffers (warmup runs, then iters timed runs each,
 * with HIP events on stream), writes the fastest to *best and records it in the
 * in-process cache under the key (dtype, D, block_q, block_k, S, B*H, mask
 * bucket), where the mask bucket is round(2 log2(active blocks / mask rows))
 * (-1 for an empty mask), counted on a host copy of block_mask; if cache_path is
 * not NULL it also merges the entry into that JSON file (BSATTN_ERR_IO if the file
 * cannot be written).  results (may be NULL) receives up to cap rows sorted by
 * t_mean; *n_results gets the number of configs timed.  out and lse are
 * overwritten.  This call synchronises the stream and may take seconds. */
int bsattn_autotune(const void* q, const void* k, const void* v, const uint8_t* block_mask,
                    void* out, float* lse, int B, int H, int S, int D, int block_q, int block_k,
                    float scale, int dtype, void* workspace, size_t workspace_bytes, int warmup,
                    int iters, bsattn_tile_config* best, bsattn_tune_result* results, int cap,
                    int* n_results, const char* cache_path, void* stream);

/* The tuned config for a mask of nnz active blocks on this shape (the entry of
 * its mask bucket), or with nnz < 0 the shape's entry of the densest mask bucket
 * tuned or loaded, which is also what bsattn_fwd and an all-zero cfg use (they do
 * not read the mask on the host).  Returns
 * BSATTN_OK and writes *cfg, BSATTN_ERR_UNSUPPORTED if no such entry exists,
 * BSATTN_ERR_NULL / BSATTN_ERR_SHAPE for a NULL cfg or a bad shape.  Host only. */
int bsattn_tune_lookup(int dtype, int D, int B, int H, int S, int block_q, int block_k, long long nnz,
                       bsattn_tile_config* cfg);

/* Load tuned configs from a JSON file written by bsattn_autotune into the
 * in-process cache (an entry of the same key is replaced).  Returns BSATTN_OK,
 * BSATTN_ERR_NULL for a NULL path, or BSATTN_ERR_IO if the file cannot be read. */
int bsattn_load_tune_cache(const char* cache_path);

/* Clear the in-process tuning cache. */
void bsattn_clear_tune_cache(void);

#ifdef __cplusplus
}
#endif

#endif /* BSATTN_H */
