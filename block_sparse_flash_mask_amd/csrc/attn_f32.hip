// attn_f32.hip -- fused block-sparse flash-attention forward in fp32 for gfx950,
// using the fp32 matrix cores (v_mfma_f32_32x32x2_f32, full fp32 products).
//
// Same operator and the same decomposition as the bf16 kernel (one workgroup per
// tile_q query rows of one mask row, 32 rows per wave, a walk over the row's
// active key blocks, S^T = K Q^T, online base-2 softmax, O^T += V^T P^T), kept in
// fp32 end to end: P is never rounded.  The 32x32x2 MFMA takes one element per
// lane per operand, so:
//   * Q^T fragment: lane (h, q) holds Q[q][h*D/2 + s] for s = 0..D/2-1;
//   * S^T step s reads K[row][h*D/2 + s] (LDS rows padded by 16 bytes so the 32
//     rows read together fall in distinct banks);
//   * after the S^T MFMA, register i of lane (h, q) holds key
//     8*(i/4) + 4*h + i%4 of the 32-key tile, and the P V step for that register
//     reads V[that key][d] from a row-major V tile: no transpose is needed.
// Element-level masks (ELEM = 1): the list entry of a partial block carries its bit
// tile (kj | (tile + 1) << 16); after the S^T MFMAs a lane reads one 32-bit word of
// its query row per 32-key tile and sets to -inf the scores whose bit is clear (key
// 8*(i/4) + 4*h + i%4 is bit 8*(i/4) + i%4 of the word shifted by 4*h).  While a
// row has no kept score (m = -inf) the exponent uses m = 0 and the rescale factor
// is 0, so dropped scores give exact zeros; a row that keeps nothing gets 0, -inf.
#include "common.h"
#include "kernels.h"

namespace bsattn {

template <int D, int WAVES, int TK, int ELEM>
__global__ __launch_bounds__(WAVES * 64) void attn_f32_kernel(FwdArgs a) {
    constexpr int TQ = 32 * WAVES;
    constexpr int NT = 64 * WAVES;
    constexpr int HALF = D / 2;
    constexpr int MT = TK / 32;
    constexpr int MD = D / 32;
    constexpr int KLD = D + 4;  // padded K row, in floats
    constexpr int CH = TK * D / 4;  // float4 chunks per K (or V) tile
    static_assert(CH % NT == 0, "tile must split evenly over the workgroup");
    constexpr int CH_T = CH / NT;

    __shared__ __attribute__((aligned(16))) float ks_[TK * KLD];
    __shared__ __attribute__((aligned(16))) float vs_[TK * D];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;
    const int l32 = lane & 31;

    int r, sub;
    block_work(a, r, sub);
    if (r < 0) return;
    const int bh = r / a.n_q;
    const int qi = r - bh * a.n_q;
    int beg, cnt;
    row_list(a, r, beg, cnt);
    const int tpb = a.block_k / TK;
    const int n_steps = cnt * tpb;
    const int q_row = qi * a.block_q + sub * TQ + wave * 32 + l32;
    const size_t head = (size_t)bh * a.S * D;
    const float* __restrict__ kg = (const float*)a.k + head;
    const float* __restrict__ vg = (const float*)a.v + head;

    float qf[HALF];
    {
        const float4* qp = (const float4*)((const float*)a.q + head + (size_t)q_row * D + h * HALF);
#pragma unroll
        for (int s4 = 0; s4 < HALF / 4; ++s4) {
            float4 t = qp[s4];
            qf[4 * s4 + 0] = __uint_as_float(__float_as_uint(t.x) ^ a.qsign32);
            qf[4 * s4 + 1] = __uint_as_float(__float_as_uint(t.y) ^ a.qsign32);
            qf[4 * s4 + 2] = __uint_as_float(__float_as_uint(t.z) ^ a.qsign32);
            qf[4 * s4 + 3] = __uint_as_float(__float_as_uint(t.w) ^ a.qsign32);
        }
    }

    float m_run = -INFINITY;
    float l_run = 0.f;
    f32x16 oacc[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md) oacc[md] = f32x16{};

    for (int t = 0; t < n_steps; ++t) {
        const int blk_i = t / tpb;
        int kj, tile = -1;  // tile: the bit tile of a partial block (element masks)
        if constexpr (ELEM) {
            const int e = wave_uniform(a.list[beg + blk_i]);
            tile = (e >> 16) - 1;
            tile = tile < a.n_tiles ? tile : a.n_tiles - 1;  // (a plan never holds more)
            kj = e & 0xffff;
            kj = kj >= a.n_k ? a.n_k - 1 : kj;
        } else {
            kj = list_entry(a, beg + blk_i);
        }
        const int key0 = kj * a.block_k + (t - blk_i * tpb) * TK;
        float4 kr[CH_T], vr[CH_T];
#pragma unroll
        for (int i = 0; i < CH_T; ++i) {
            const int c = tid + i * NT;
            const int row = c / (D / 4), cc = c % (D / 4);
            kr[i] = *(const float4*)(kg + (size_t)(key0 + row) * D + cc * 4);
            vr[i] = *(const float4*)(vg + (size_t)(key0 + row) * D + cc * 4);
        }
        __syncthreads();  // previous step done with the LDS tiles
#pragma unroll
        for (int i = 0; i < CH_T; ++i) {
            const int c = tid + i * NT;
            const int row = c / (D / 4), cc = c % (D / 4);
            *(float4*)(ks_ + row * KLD + cc * 4) = kr[i];
            *(float4*)(vs_ + row * D + cc * 4) = vr[i];
        }
        __syncthreads();

        f32x16 sacc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) sacc[mt] = f32x16{};
#pragma unroll
        for (int s4 = 0; s4 < HALF / 4; ++s4)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const float4 kf = *(const float4*)(ks_ + (32 * mt + l32) * KLD + h * HALF + 4 * s4);
                sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.x, qf[4 * s4 + 0], sacc[mt], 0, 0, 0);
                sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.y, qf[4 * s4 + 1], sacc[mt], 0, 0, 0);
                sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.z, qf[4 * s4 + 2], sacc[mt], 0, 0, 0);
                sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.w, qf[4 * s4 + 3], sacc[mt], 0, 0, 0);
            }

        if constexpr (ELEM) {
            if (tile >= 0) {
                const int qr = q_row - qi * a.block_q;
                const int ko = (t - blk_i * tpb) * TK;
                const uint32_t* wrow = a.pbits + ((size_t)tile * a.block_q + qr) * (a.block_k >> 5) + (ko >> 5);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const uint32_t w = wrow[mt] >> (4 * h);
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (!((w >> (8 * (i >> 2) + (i & 3))) & 1u)) sacc[mt][i] = -INFINITY;
                }
            }
        }

        float mx = sacc[0][0];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = __builtin_fmaxf(mx, sacc[mt][i]);
        mx = __builtin_fmaxf(mx, xor32(mx));
        const float m_new = __builtin_fmaxf(m_run, mx * a.c);
        // (element masks: no kept score yet leaves m = -inf; 2^(-inf - -inf) would be NaN)
        const float alpha = (ELEM && m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
        const float m_use = (ELEM && m_new == -INFINITY) ? 0.f : m_new;
        float psum = 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = fast_exp2(__builtin_fmaf(sacc[mt][i], a.c, -m_use));
                psum += p;
                sacc[mt][i] = p;
            }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int md = 0; md < MD; ++md) oacc[md] *= alpha;

#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
#pragma unroll
                for (int md = 0; md < MD; ++md) {
                    const float vf = vs_[key * D + 32 * md + l32];
                    oacc[md] = __builtin_amdgcn_mfma_f32_32x32x2f32(vf, sacc[mt][i], oacc[md], 0, 0, 0);
                }
            }
    }

    const float l_tot = l_run + xor32(l_run);
    const bool any = ELEM ? m_run != -INFINITY : n_steps > 0;
    const float inv = any ? 1.0f / l_tot : 0.0f;
    float* og = (float*)a.out + head + (size_t)q_row * D;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int d0 = 32 * md + 8 * g4 + 4 * h;
            float4 o;
            o.x = oacc[md][4 * g4 + 0] * inv;
            o.y = oacc[md][4 * g4 + 1] * inv;
            o.z = oacc[md][4 * g4 + 2] * inv;
            o.w = oacc[md][4 * g4 + 3] * inv;
            *(float4*)(og + d0) = o;
        }
    if (h == 0) a.lse[(size_t)bh * a.S + q_row] = any ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
}

template <int D, int W, int TK, int ELEM>
static hipError_t launch_f32(const FwdArgs& a, unsigned grid, hipStream_t stream) {
    hipLaunchKernelGGL((attn_f32_kernel<D, W, TK, ELEM>), dim3(grid), dim3(W * 64), 0, stream, a);
    return hipGetLastError();
}

#define BSATTN_F32_VARIANT(D, W, TK) {0, D, 32 * W, TK, W, 1, &launch_f32<D, W, TK, 0>}
#define BSATTN_F32_ELEM(D, W, TK) {0, D, 32 * W, TK, W, 1, &launch_f32<D, W, TK, 1>}

static const Variant kF32Variants[] = {
    BSATTN_F32_VARIANT(64, 2, 32),  BSATTN_F32_VARIANT(64, 2, 64),
    BSATTN_F32_VARIANT(64, 4, 32),  BSATTN_F32_VARIANT(64, 4, 64),
    BSATTN_F32_VARIANT(128, 2, 32), BSATTN_F32_VARIANT(128, 2, 64),
    BSATTN_F32_VARIANT(128, 4, 32), BSATTN_F32_VARIANT(128, 4, 64),
};

// The same configs with element-level masks.
static const Variant kF32ElemVariants[] = {
    BSATTN_F32_ELEM(64, 2, 32),  BSATTN_F32_ELEM(64, 2, 64),
    BSATTN_F32_ELEM(64, 4, 32),  BSATTN_F32_ELEM(64, 4, 64),
    BSATTN_F32_ELEM(128, 2, 32), BSATTN_F32_ELEM(128, 2, 64),
    BSATTN_F32_ELEM(128, 4, 32), BSATTN_F32_ELEM(128, 4, 64),
};

const Variant* f32_variants(int* n) {
    *n = (int)(sizeof(kF32Variants) / sizeof(kF32Variants[0]));
    return kF32Variants;
}

const Variant* f32_elem_variants(int* n) {
    *n = (int)(sizeof(kF32ElemVariants) / sizeof(kF32ElemVariants[0]));
    return kF32ElemVariants;
}

}  // namespace bsattn
