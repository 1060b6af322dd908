// common.h -- device types and small helpers shared by the gfx950 kernels of
// libbsattn.so.  CDNA4 only: wave64, MFMA, 160 KiB LDS per workgroup.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Everything a forward launch needs; passed by value as the kernel argument.
struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    // Per-row key-block lists.  CSR form (ell_stride == 0): the list of mask row
    // r is list[row_ptr[r] .. row_ptr[r+1]).  Padded form (ell_stride > 0): it is
    // list[r*ell_stride .. r*ell_stride + counts[r]).
    const int32_t* row_ptr;
    const int32_t* counts;
    const int32_t* list;
    int ell_stride;
    int64_t list_len;  // CSR form: entries in list (each row's span is clamped into it)
    void* out;
    float* lse;
    int H, S, n_q, n_k;
    int block_q, block_k;
    // Dispatch.  Mask rows are cut into 8 chunks of `chunk` rows, one per XCD
    // (blockIdx b runs on XCD b % 8).  Block b takes position j = b / 8 of its
    // XCD's queue: row slot (b % 8) * chunk + j / sub_per_row, sub-tile
    // j % sub_per_row, so the sub-tiles of one row run side by side.  A slot is a
    // mask row itself, or order[slot] when order is not NULL; a row outside
    // [0, nrows) does nothing.
    const int32_t* order;
    int nrows;         // mask rows: B * H * n_q
    int chunk;         // row slots per XCD
    int sub_per_row;   // block_q / tile_q: workgroups per mask row (a power of 2)
    int sub_log2;      // log2(sub_per_row)
    int steps_log2;    // log2(block_k / tile_k): kernel steps per key block
    // Element-level masks: bit tiles [n_tiles][block_q][block_k / 32]; the list
    // entries then carry (tile + 1) << 16 for a partial block (0: full).
    const uint32_t* pbits;
    int n_tiles;
    float c;           // |scale| * log2(e)
    uint32_t qsign;    // 0x80008000 flips the sign of two packed bf16 (scale < 0)
    uint32_t qsign32;  // 0x80000000 flips an fp32 sign (scale < 0)
};

// Everything a backward launch needs (both main kernels take the same struct).
struct BwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* dout;
    const float2* ld;  // per row: (lse * log2 e, or +inf for lse = -inf; dout . out)
    // dq: the forward plan -- per mask row the count and the key-block list padded
    // to n_k, and the dispatch order of the rows in chunks of chunk_q per XCD.
    const int32_t* row_counts;
    const int32_t* row_lists;
    const int32_t* row_order;
    int n_rows, chunk_q;
    // dk, dv: per key block (column, (b*H + h)*n_k + kj) the query-block list
    // padded to n_q, and the work items over them: {column, first list entry,
    // entries, partial slot or -1}.  A column with more entries than the plan's
    // piece length is cut into pieces whose fp32 partial dK and dV go to scratch
    // slots ([slot][2][block_k][D]: dK unscaled, then dV), summed in piece order by
    // the reduce kernel (splits: {column, first slot, pieces, 0}).  n_items holds
    // the item and split counts.  The dk/dv grid holds 8 * chunk_k workgroups
    // (chunk_k for the most items a plan can hold); the kernel deals the plan's
    // items to the XCDs in contiguous chunks of ceil(items / 8).
    const int32_t* col_lists;
    const int4* items;
    const int32_t* n_items;
    const int4* splits;
    float* scratch;
    int n_cols, chunk_k, max_slots, max_splits;
    void* dq;
    void* dk;
    void* dv;
    int S, n_q, n_k, block_q, block_k;
    int qsteps_log2;  // log2(block_q / 32)
    int ksteps_log2;  // log2(block_k / 32)
    float c;          // scale * log2(e)
    float scale;
    // Element-level masks (the ELEM kernels only): block states [B][H][n_q][n_k]
    // (0 empty, 1 full, else partial), the bit tile of each partial block, and the
    // tiles [n_tiles][block_q][block_k / 32].
    const uint8_t* states;
    const int32_t* pidx;
    const uint32_t* pbits;
    int n_tiles;
};

__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Exchange with the lane 32 positions away (the other half of the wave).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// x[lane] + x[lane ^ 32] with one v_permlane32_swap: it returns (own, partner)
// in the low half-wave and (partner, own) in the high one.
__device__ __forceinline__ float sum_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// NaN-propagating maximum: v_maximum3_f32 on gfx950, with none of the
// canonicalising moves that an IEEE-mode fmaxf needs in front of v_max_f32.
__device__ __forceinline__ float fmax_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// max(x[lane], x[lane ^ 32]) with fmax_nan.
__device__ __forceinline__ float max_halves_nan(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmax_nan(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Maximum of N register values as a tree of three-input maxima (one
// v_maximum3_f32 per node; ceil(log3 N) dependent levels).
template <int N>
__device__ __forceinline__ float max_tree3(const float* v) {
    if constexpr (N == 1) {
        return v[0];
    } else if constexpr (N == 2) {
        return fmax_nan(v[0], v[1]);
    } else {
        constexpr int M = (N + 2) / 3;
        float w[M];
#pragma unroll
        for (int i = 0; i < M; ++i) {
            if (3 * i + 2 < N)
                w[i] = fmax_nan(fmax_nan(v[3 * i], v[3 * i + 1]), v[3 * i + 2]);
            else if (3 * i + 1 < N)
                w[i] = fmax_nan(v[3 * i], v[3 * i + 1]);
            else
                w[i] = v[3 * i];
        }
        return max_tree3<M>(w);
    }
}

// Pairwise (tree) sum of N register values: log2(N) dependent levels instead
// of a serial chain.
template <int N>
__device__ __forceinline__ float tree_sum(float* v) {
#pragma unroll
    for (int w = N / 2; w >= 1; w /= 2)
#pragma unroll
        for (int i = 0; i < w; ++i) v[i] = v[i] + v[i + w];
    return v[0];
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Key block kj of list entry i, clamped into [0, n_k) so a malformed caller list
// can give wrong values but never an out-of-bounds read.
__device__ __forceinline__ int list_entry(const FwdArgs& a, int i) {
    const int kj = wave_uniform(a.list[i]);
    return kj < 0 ? 0 : (kj >= a.n_k ? a.n_k - 1 : kj);
}

// The mask row and sub-tile this block runs; row = -1 for a block with no work
// (uniform across the block).
__device__ __forceinline__ void block_work(const FwdArgs& a, int& row, int& sub) {
    const int b = blockIdx.x;
    const int j = b >> 3;
    const int jr = j >> a.sub_log2;
    int r = -1;
    if (jr < a.chunk) {
        const int slot = (b & 7) * a.chunk + jr;
        r = a.order ? a.order[slot] : slot;
    }
    if (r < 0 || r >= a.nrows) r = -1;
    row = wave_uniform(r);
    sub = wave_uniform(j & (a.sub_per_row - 1));
}

// Resolve the key-block list of mask row r (wave-uniform results).
__device__ __forceinline__ void row_list(const FwdArgs& a, int r, int& beg, int& cnt) {
    if (a.ell_stride > 0) {
        beg = r * a.ell_stride;
        cnt = a.counts[r];
    } else {
        // caller's CSR: keep the span [beg, beg + cnt) inside list[0 .. list_len)
        const int64_t b0 = a.row_ptr[r], e0 = a.row_ptr[r + 1];
        const int64_t b1 = b0 < 0 ? 0 : (b0 > a.list_len ? a.list_len : b0);
        const int64_t e1 = e0 < b1 ? b1 : (e0 > a.list_len ? a.list_len : e0);
        beg = (int)b1;
        cnt = (int)(e1 - b1 > a.n_k ? a.n_k : e1 - b1);
    }
    // A row lists each key block at most once: a larger count is malformed input.
    cnt = cnt < 0 ? 0 : (cnt > a.n_k ? a.n_k : cnt);
    beg = wave_uniform(beg);
    cnt = wave_uniform(cnt);
}

}  // namespace bsattn
