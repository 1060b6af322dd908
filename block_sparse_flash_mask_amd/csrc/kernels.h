// kernels.h -- host-side launchers of the gfx950 kernels (internal to libbsattn.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace bsattn {

// Mask compaction (compact.hip).
hipError_t launch_compact_rows(const uint8_t* mask, int64_t R, int n_k, int32_t* counts,
                               int32_t* lists, hipStream_t stream);
// Element-level masks: row lists as launch_compact_rows from block states
// (0 empty, else active), each entry kj | (tile + 1) << 16 for a partial block
// (state > 1, tile = pidx clamped into [0, n_tiles)) or kj for a full one.
hipError_t launch_compact_rows_elem(const uint8_t* states, const int32_t* pidx, int n_tiles, int64_t R,
                                    int n_k, int32_t* counts, int32_t* lists, hipStream_t stream);
hipError_t launch_compact_scan(const int32_t* counts, int64_t R, int32_t* row_ptr,
                               hipStream_t stream);
// Dispatch orders per XCD chunk (head by head, longest first within a head):
// of the R mask rows in chunks of `chunk` (order: 8 * chunk entries), and of the
// B*H*ceil(n_q/2) pairs of adjacent rows (rows 2j, 2j+1 of a head, keyed by the
// longer of the two) in chunks of `pchunk` (porder: 8 * pchunk entries).
hipError_t launch_compact_order(const int32_t* counts, int64_t R, int n_q, int n_k, int64_t chunk,
                                int32_t* order, int64_t pchunk, int32_t* porder,
                                hipStream_t stream);
// The plan of a forward pass (row counts and lists as launch_compact_rows, both
// dispatch orders as launch_compact_order): one launch for masks of at most
// 4 MiB with rows of at most 128 blocks, else those two launches.
hipError_t launch_plan(const uint8_t* mask, int64_t R, int n_q, int n_k, int32_t* counts,
                       int32_t* lists, int64_t chunk, int32_t* order, int64_t pchunk,
                       int32_t* porder, hipStream_t stream);
hipError_t launch_compact_pack(const int32_t* counts, const int32_t* lists, int64_t R, int n_k,
                               const int32_t* row_ptr, int32_t* col_idx, hipStream_t stream);

// Ragged dot (ragged_dot.hip): the work-item bound of a plan (one item per
// (256-row tile, group) pair that share rows, plus the zero-fill items of the rows
// past the last group), the plan's bytes (items, then their count), the plan
// launch and the product launch on a plan.
inline int64_t ragged_max_items(int64_t M, int64_t G) { return (M + 255) / 256 + G + 1; }
inline size_t ragged_ws_bytes(int64_t M, int64_t G) { return (size_t)ragged_max_items(M, G) * 16 + 16; }
hipError_t launch_ragged_plan(const int32_t* group_sizes, int M, int G, void* workspace, hipStream_t stream);
// n_cu: compute units of the device (the 256 x 256 kernel takes whole rounds of them,
// the partial last round runs as quarter tiles); 0 runs everything in one launch.
hipError_t launch_ragged_planned(const void* lhs, const void* rhs, void* out, int M, int K, int N, int G,
                                 int out_f32, const void* workspace, int n_cu, hipStream_t stream);

// Backward (attn_bwd.hip): per-row (lse * log2 e, dout . out) into ld (float2
// [rows]), the column form of the mask (per key block: count, query-block list
// padded to n_q), and the dk/dv and dq kernels (bf16 inputs, D 64 or 128, block
// sizes 64 or 128; gradients bf16 or fp32).
hipError_t launch_bwd_prep(const void* out, const void* dout, const float* lse, void* ld, int64_t rows, int D,
                           hipStream_t stream);
hipError_t launch_bwd_cols(const uint8_t* mask, int64_t C, int n_q, int n_k, int32_t* counts, int32_t* lists,
                           hipStream_t stream);
// The dk/dv work items (BwdArgs) from the column counts: at most C + max_slots
// items (int4) and max_slots / 2 splits (int4); n_out = {items, splits}.
hipError_t launch_bwd_split(const int32_t* counts, int64_t C, int n_q, int max_slots, void* items, void* splits,
                            int32_t* n_out, hipStream_t stream);
hipError_t launch_bwd_main(const BwdArgs& a, int D, int out_f32, bool do_dq, bool do_dkdv, hipStream_t stream);

// Row-pair variants (tile_q = 2 * block_q = 256) build the union of two block
// lists in LDS, so they take masks of at most this many key blocks per row.
constexpr int kPairMaxBlocks = 2048;

// One compiled attention variant.
struct Variant {
    int dtype;   // 0 = fp32, 1 = bf16
    int D;
    int tile_q;
    int tile_k;
    int waves;
    int stages;
    hipError_t (*launch)(const FwdArgs& a, unsigned grid, hipStream_t stream);
};

// The two-group bf16 kernel (attn_bf16_pp.hip): 8 waves, 128 query rows, 32-key tiles.
template <int D>
hipError_t launch_bf16_pp(const FwdArgs& a, unsigned grid, hipStream_t stream);

// Tables of the built variants (attn_bf16.hip, attn_f32.hip).
const Variant* bf16_variants(int* n);
// The bf16 variants built for element-level masks (plain schedule, row pairs included).
const Variant* bf16_elem_variants(int* n);
const Variant* f32_variants(int* n);
// The fp32 variants with element-level masks.
const Variant* f32_elem_variants(int* n);
// fp8 forward (attn_fp8.hip): dtype 2, tile_k 64, one config per (D, tile_q); and
// the pre-pass that rearranges V per 64-key tile for its P V product (tiles =
// B*H*S/64).
const Variant* fp8_variants(int* n);
// The same fp8 configs with element-level masks.
const Variant* fp8_elem_variants(int* n);
hipError_t launch_fp8_vt(const void* v, void* vt, int64_t tiles, int D, hipStream_t stream);

}  // namespace bsattn
