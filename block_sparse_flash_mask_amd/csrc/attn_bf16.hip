// attn_bf16.hip -- fused block-sparse flash-attention forward, bf16 in, fp32
// accumulation, bf16 out + fp32 lse, for gfx950 (CDNA4) MFMA.
//
// What is computed: "Writing Pallas Kernels for JAX" (rajatpandit.com), section
// "Writing the Kernel Logic: Load, Compute, Store" -- scaled Q K^T per tile, scores
// of inactive blocks never contribute (they are -inf), softmax, P V.  Unlike the
// per-tile softmax of that page's listing, the softmax here runs over the whole
// row with a running row max and running row sum, so the result is the exact
// operator ("Pallas-Triton kernels and kernel auto-tuning", section "Flash
// Attention").  Inactive key blocks are not visited at all.
//
// Work decomposition.  One workgroup owns tile_q = 32*WAVES query rows of one mask
// row (b, h, qi); wave w owns 32 of them.  It walks that mask row's list of active
// key blocks in steps of TK keys.  Per step:
//   S^T[key][q] = K Q^T   v_mfma_f32_32x32x16_bf16, A = K (from LDS), B = Q^T
//                         (held in VGPRs for the whole kernel).  Each lane holds
//                         one query column and 16 keys per 32x32 tile, so the row
//                         max is a lane-local max plus one exchange with lane^32.
//   online softmax        m' = max(m, c*rowmax S), alpha = 2^(m - m'),
//                         P = 2^(c*S - m'), l = alpha*l + rowsum P, O *= alpha,
//                         with c = |scale| * log2(e) (a negative scale flips the
//                         sign of Q, which is exact in bf16).
//   O^T[d][q] += V^T P^T  v_mfma_f32_32x32x16_bf16, A = V^T (from LDS), B = P^T
//                         straight from the S^T registers converted to bf16.
// The K rows are fed to the first MFMA in a bit-swapped order (kperm) chosen so
// that the keys each lane holds after it are exactly the keys the second MFMA
// wants in that lane: P never moves between lanes.
//
// LDS.  K tile [TK][D] row-major, V tile transposed [D][TK]; both XOR-swizzled at
// 16-byte granularity so the MFMA operand reads (8 rows x 16 B per LDS cycle) and
// the writes hit distinct banks.  STAGES = 2 keeps two K/V tiles: the next tile is
// fetched into VGPRs before the current tile's MFMAs and written to the other LDS
// buffer after them, one barrier per step.  STAGES = 1 uses one buffer and two
// barriers per step.
#include "common.h"
#include "kernels.h"

namespace bsattn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Row order of K fed to the S^T MFMA: swap bits 2 and 3 of the 5-bit row index.
// After the MFMA, register i of lane (half h) holds key 16*(i/8) + 8*h + i%8 of
// the 32-key tile: keys 8h..8h+7 in registers 0..7 and 16+8h..16+8h+7 in 8..15,
// which is the B-operand layout of two 16-key steps of the P V MFMA.
__device__ __forceinline__ int kperm(int m) { return (m & 0x13) | ((m & 4) << 1) | ((m & 8) >> 1); }

// 16-byte chunk swizzle of a K row: rows read together by 8 lanes (0..3, 8..11 or
// 4..7, 12..15 of each 16) get distinct chunks.
__device__ __forceinline__ int swz_k(int row) { return (row & 3) | ((row >> 1) & 4); }

// 16-byte chunk swizzle of a V^T row (one head-dim index d): consecutive d and
// d 8 apart (the write pattern) get distinct chunks.
template <int TK>
__device__ __forceinline__ int swz_v(int d) {
    return (d ^ (d >> 3)) & (TK / 8 - 1);
}

template <int D, int WAVES, int TK, int STAGES>
__global__ __launch_bounds__(WAVES * 64) void attn_bf16_kernel(FwdArgs a) {
    constexpr int TQ = 32 * WAVES;
    constexpr int NT = 64 * WAVES;
    constexpr int KS = D / 16;   // 16-deep k-steps of the S^T MFMA
    constexpr int MT = TK / 32;  // 32-key tiles of S^T
    constexpr int MD = D / 32;   // 32-wide d tiles of O^T
    constexpr int KROW = D * 2;  // bytes of one K row in LDS
    constexpr int VROW = TK * 2; // bytes of one V^T row in LDS
    constexpr int KTILE = TK * KROW;
    constexpr int VTILE = D * VROW;
    constexpr int KCH = TK * D / 8;  // 16-byte chunks in a K tile
    constexpr int KCH_T = KCH / NT;
    static_assert(KCH % NT == 0, "K tile must split evenly over the workgroup");
    constexpr int VGRP = (TK / 4) * (D / 8);  // (4 keys x 8 d) groups of a V tile
    constexpr int VGRP_T = (VGRP + NT - 1) / NT;

    __shared__ __attribute__((aligned(16))) uint8_t smem[STAGES * (KTILE + VTILE)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;
    const int l32 = lane & 31;

    const int wg = blockIdx.x;
    const int r = wg / a.sub_per_row;
    const int sub = wg - r * a.sub_per_row;
    const int bh = r / a.n_q;
    const int qi = r - bh * a.n_q;
    int beg, cnt;
    row_list(a, r, beg, cnt);
    const int tpb = a.block_k / TK;  // kernel steps per key block
    const int n_steps = cnt * tpb;
    const int q_row = qi * a.block_q + sub * TQ + wave * 32 + l32;
    const size_t head = (size_t)bh * a.S * D;
    const uint16_t* __restrict__ kg = (const uint16_t*)a.k + head;
    const uint16_t* __restrict__ vg = (const uint16_t*)a.v + head;

    // Q^T fragments: lane (h, q) holds Q[q][16*ks + 8*h .. +7] for every ks.
    bf16x8 qf[KS];
    {
        const u32x4* qp = (const u32x4*)((const uint16_t*)a.q + head + (size_t)q_row * D);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 t = qp[2 * ks + h];
            t ^= a.qsign;
            qf[ks] = __builtin_bit_cast(bf16x8, t);
        }
    }

    u32x4 kreg[KCH_T];
    u32x4 vreg[VGRP_T][4];

    auto step_key0 = [&](int t) -> int {
        const int blk_i = t / tpb;
        const int kj = list_entry(a, beg + blk_i);
        return kj * a.block_k + (t - blk_i * tpb) * TK;
    };

    // HBM -> VGPR: K rows as 16-byte chunks; V as 4 keys x 8 d per group.
    auto load_step = [&](int key0) {
        const uint16_t* kt = kg + (size_t)key0 * D;
#pragma unroll
        for (int i = 0; i < KCH_T; ++i) {
            const int c = tid + i * NT;
            const int row = c / (D / 8), cc = c % (D / 8);
            kreg[i] = *(const u32x4*)(kt + row * D + cc * 8);
        }
        const uint16_t* vt = vg + (size_t)key0 * D;
#pragma unroll
        for (int i = 0; i < VGRP_T; ++i) {
            const int g = tid + i * NT;
            if (VGRP % NT == 0 || g < VGRP) {
                const int dc = g % (D / 8), kq = g / (D / 8);
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    vreg[i][u] = *(const u32x4*)(vt + (size_t)(4 * kq + u) * D + dc * 8);
            }
        }
    };

    // VGPR -> LDS buffer st: K as is (swizzled), V transposed to [d][key].
    auto store_step = [&](int st) {
        uint8_t* ks_ = smem + st * (KTILE + VTILE);
        uint8_t* vs_ = ks_ + KTILE;
#pragma unroll
        for (int i = 0; i < KCH_T; ++i) {
            const int c = tid + i * NT;
            const int row = c / (D / 8), cc = c % (D / 8);
            *(u32x4*)(ks_ + row * KROW + ((cc ^ swz_k(row)) << 4)) = kreg[i];
        }
#pragma unroll
        for (int i = 0; i < VGRP_T; ++i) {
            const int g = tid + i * NT;
            if (VGRP % NT == 0 || g < VGRP) {
                const int dc = g % (D / 8), kq = g / (D / 8);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int w = j >> 1;
                    uint32_t e0, e1, e2, e3;
                    if (j & 1) {
                        e0 = vreg[i][0][w] >> 16; e1 = vreg[i][1][w] >> 16;
                        e2 = vreg[i][2][w] >> 16; e3 = vreg[i][3][w] >> 16;
                    } else {
                        e0 = vreg[i][0][w] & 0xffffu; e1 = vreg[i][1][w] & 0xffffu;
                        e2 = vreg[i][2][w] & 0xffffu; e3 = vreg[i][3][w] & 0xffffu;
                    }
                    const int d = 8 * dc + j;
                    u32x2 pk;
                    pk[0] = e0 | (e1 << 16);
                    pk[1] = e2 | (e3 << 16);
                    *(u32x2*)(vs_ + d * VROW + (((kq >> 1) ^ swz_v<TK>(d)) << 4) + ((kq & 1) << 3)) = pk;
                }
            }
        }
    };

    float m_run = -INFINITY;
    float l_run = 0.f;
    f32x16 oacc[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md) oacc[md] = f32x16{};

    if (n_steps > 0) {
        load_step(step_key0(0));
        store_step(0);
        __syncthreads();
        for (int t = 0; t < n_steps; ++t) {
            const int st = (STAGES == 2) ? (t & 1) : 0;
            const bool more = t + 1 < n_steps;
            if (more) load_step(step_key0(t + 1));
            const uint8_t* ks_ = smem + st * (KTILE + VTILE);
            const uint8_t* vs_ = ks_ + KTILE;

            // S^T = K Q^T
            f32x16 sacc[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) sacc[mt] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const int row = 32 * mt + kperm(l32);
                    const bf16x8 kf =
                        *(const bf16x8*)(ks_ + row * KROW + (((2 * ks + h) ^ swz_k(row)) << 4));
                    sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc[mt], 0, 0, 0);
                }
            }

            // online softmax (base 2)
            float mx = sacc[0][0];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = __builtin_fmaxf(mx, sacc[mt][i]);
            mx = __builtin_fmaxf(mx, xor32(mx));
            const float m_new = __builtin_fmaxf(m_run, mx * a.c);
            const float alpha = fast_exp2(m_run - m_new);
            float psum = 0.f;
            bf16x8 pb[MT][2];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = fast_exp2(__builtin_fmaf(sacc[mt][i], a.c, -m_new));
                    psum += p;
                    pb[mt][i >> 3][i & 7] = (__bf16)p;
                }
            l_run = l_run * alpha + psum;
            m_run = m_new;
#pragma unroll
            for (int md = 0; md < MD; ++md) oacc[md] *= alpha;

            // O^T += V^T P^T
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int e = 0; e < 2; ++e)
#pragma unroll
                    for (int md = 0; md < MD; ++md) {
                        const int d = 32 * md + l32;
                        const bf16x8 vf = *(const bf16x8*)(vs_ + d * VROW +
                                                           (((4 * mt + 2 * e + h) ^ swz_v<TK>(d)) << 4));
                        oacc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[mt][e], oacc[md], 0, 0, 0);
                    }

            if (STAGES == 2) {
                if (more) store_step(st ^ 1);
                __syncthreads();
            } else {
                __syncthreads();
                if (more) store_step(0);
                __syncthreads();
            }
        }
    }

    // Epilogue: O / l in bf16 (round to nearest even), lse = ln2 * (m + log2 l).
    const float l_tot = l_run + xor32(l_run);
    const bool any = n_steps > 0;
    const float inv = any ? 1.0f / l_tot : 0.0f;
    uint16_t* og = (uint16_t*)a.out + head + (size_t)q_row * D;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int d0 = 32 * md + 8 * g4 + 4 * h;
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            bf16x4 o;
#pragma unroll
            for (int u = 0; u < 4; ++u) o[u] = (__bf16)(oacc[md][4 * g4 + u] * inv);
            *(bf16x4*)(og + d0) = o;
        }
    if (h == 0) a.lse[(size_t)bh * a.S + q_row] = any ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
}

template <int D, int W, int TK, int ST>
static hipError_t launch_bf16(const FwdArgs& a, unsigned grid, hipStream_t stream) {
    hipLaunchKernelGGL((attn_bf16_kernel<D, W, TK, ST>), dim3(grid), dim3(W * 64), 0, stream, a);
    return hipGetLastError();
}

#define BSATTN_BF16_VARIANT(D, W, TK, ST) {1, D, 32 * W, TK, W, ST, &launch_bf16<D, W, TK, ST>}

static const Variant kBf16Variants[] = {
    BSATTN_BF16_VARIANT(128, 4, 64, 2),  BSATTN_BF16_VARIANT(128, 4, 32, 2),
    BSATTN_BF16_VARIANT(128, 4, 128, 2), BSATTN_BF16_VARIANT(128, 4, 64, 1),
    BSATTN_BF16_VARIANT(128, 4, 32, 1),  BSATTN_BF16_VARIANT(128, 4, 128, 1),
    BSATTN_BF16_VARIANT(128, 2, 64, 2),  BSATTN_BF16_VARIANT(128, 2, 32, 2),
    BSATTN_BF16_VARIANT(128, 2, 64, 1),  BSATTN_BF16_VARIANT(128, 2, 32, 1),
    BSATTN_BF16_VARIANT(64, 4, 64, 2),   BSATTN_BF16_VARIANT(64, 4, 32, 2),
    BSATTN_BF16_VARIANT(64, 4, 128, 2),  BSATTN_BF16_VARIANT(64, 4, 64, 1),
    BSATTN_BF16_VARIANT(64, 4, 32, 1),   BSATTN_BF16_VARIANT(64, 4, 128, 1),
    BSATTN_BF16_VARIANT(64, 2, 64, 2),   BSATTN_BF16_VARIANT(64, 2, 32, 2),
    BSATTN_BF16_VARIANT(64, 2, 128, 2),  BSATTN_BF16_VARIANT(64, 2, 64, 1),
    BSATTN_BF16_VARIANT(64, 2, 32, 1),   BSATTN_BF16_VARIANT(64, 2, 128, 1),
};

const Variant* bf16_variants(int* n) {
    *n = (int)(sizeof(kBf16Variants) / sizeof(kBf16Variants[0]));
    return kBf16Variants;
}

}  // namespace bsattn
