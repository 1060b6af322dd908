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
    void* out;
    float* lse;
    int H, S, n_q, n_k;
    int block_q, block_k;
    int sub_per_row;   // block_q / tile_q: workgroups per mask row
    float c;           // |scale| * log2(e)
    uint32_t qsign;    // 0x80008000 flips the sign of two packed bf16 (scale < 0)
    uint32_t qsign32;  // 0x80000000 flips an fp32 sign (scale < 0)
};

__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Exchange with the lane 32 positions away (the other half of the wave).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Key block kj of list entry i, clamped into [0, n_k) so a malformed caller list
// can give wrong values but never an out-of-bounds read.
__device__ __forceinline__ int list_entry(const FwdArgs& a, int i) {
    const int kj = wave_uniform(a.list[i]);
    return kj < 0 ? 0 : (kj >= a.n_k ? a.n_k - 1 : kj);
}

// Resolve the key-block list of mask row r (wave-uniform results).
__device__ __forceinline__ void row_list(const FwdArgs& a, int r, int& beg, int& cnt) {
    if (a.ell_stride > 0) {
        beg = r * a.ell_stride;
        cnt = a.counts[r];
    } else {
        beg = a.row_ptr[r];
        cnt = a.row_ptr[r + 1] - beg;
    }
    beg = wave_uniform(beg);
    cnt = wave_uniform(cnt);
}

}  // namespace bsattn
