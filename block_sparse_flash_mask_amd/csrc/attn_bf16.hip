// attn_bf16.hip -- fused block-sparse flash-attention forward, bf16 in, fp32
// accumulation, bf16 out + fp32 lse, for gfx950 (CDNA4) MFMA.
//
// What is computed: "Writing Pallas Kernels for JAX" (rajatpandit.com), section
// "Writing the Kernel Logic: Load, Compute, Store" -- scaled Q K^T per tile, scores
// of inactive blocks never contribute (they are -inf), softmax, P V.  Unlike the
// per-tile softmax of that page's listing, the softmax here runs over the whole
// row with a running row max and running row sum, so the result is the exact
// operator ("Pallas-Triton kernels and kernel auto-tuning", section "Flash
// Attention").  Inactive key blocks are never visited.
//
// Work decomposition.  One workgroup owns tile_q = 32*WAVES query rows of one mask
// row (b, h, qi); wave w owns 32 of them.  It walks that mask row's list of active
// key blocks in steps of TK keys.  Per step and wave:
//   S^T[key][q] = K Q^T   v_mfma_f32_32x32x16_bf16; A = K from LDS, B = Q^T held
//                         in VGPRs for the whole kernel.  Each lane owns one query
//                         column, so the row max is lane-local plus one exchange
//                         with lane^32.
//   online softmax        base 2 with c = |scale|*log2(e) (a negative scale flips
//                         the sign of Q, exact in bf16).  The reference max m only
//                         moves when the tile max exceeds it by more than 8 (2^8
//                         headroom): then O and l are rescaled by 2^(m-m').  Any
//                         reference <= the true max gives the same exact result,
//                         so most steps skip the rescale.
//   O^T[d][q] += V^T P^T  v_mfma_f32_32x32x16_bf16; A = V^T read from LDS with
//                         the transposing ds_read_b64_tr_b16, B = P^T straight from
//                         the S^T registers converted to bf16.
// K rows enter the first MFMA in a bit-swapped order (kperm) so that the keys a
// lane holds after it are exactly the keys the second MFMA wants in that lane.
//
// Memory path.  K and V tiles go HBM -> LDS by direct DMA (global_load_lds, 16 B
// per lane), no VGPR staging.  Both are stored in LDS in the order the MFMA
// operand reads consume them:
//   K: one 1 KiB block per (32-key tile mt, 16-deep k-step ks); lane l's 16 bytes
//      at l*16 are K[32mt + kperm(l%32)][16ks + 8(l/32) .. +7];
//   V: one 512 B block per (mt, 16-key half e, 4-key quarter r, 32-wide d tile md);
//      lane l's 8 bytes at l*8 are what the 16x4 transpose of its 16-lane group
//      needs: V[32mt + 16e + 8h + 4r + L/4][32md + 16g + 4(L%4) .. +3] with
//      L = l%16, g = (l/16)%2, h = l/32.
// Every LDS read is lane-linear (conflict free) at a per-lane base plus a
// compile-time offset.  Two stages live in distinct LDS arrays: the next step's
// DMA is issued into the other array right after the per-step barrier and
// overlaps the current step's MFMAs.
#include "common.h"
#include "kernels.h"

namespace bsattn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#define BSATTN_LDS __attribute__((address_space(3)))

// Row order of K fed to the S^T MFMA: swap bits 2 and 3 of the 5-bit row index.
// After the MFMA, register i of lane (half h) holds key 16*(i/8) + 8*h + i%8 of
// the 32-key tile: keys 8h..8h+7 in registers 0..7 and 16+8h..16+8h+7 in 8..15,
// which is the B-operand layout of two 16-key steps of the P V MFMA.
__device__ __forceinline__ int kperm(int m) { return (m & 0x13) | ((m & 4) << 1) | ((m & 8) >> 1); }

template <int D, int TK>
struct TileGeom {
    static constexpr int KS = D / 16;               // 16-deep k-steps of S^T
    static constexpr int MT = TK / 32;              // 32-key tiles
    static constexpr int MD = D / 32;               // 32-wide d tiles of O^T
    static constexpr int KBLK = MT * KS;            // 1 KiB K blocks per tile
    static constexpr int VBLK = MT * 2 * 2 * MD;    // 512 B V blocks per tile
    static constexpr int BYTES = TK * D * 2;        // one K (or V) tile
    static_assert(KBLK * 1024 == BYTES, "K layout covers the tile");
    static_assert(VBLK * 512 == BYTES, "V layout covers the tile");
};

// Per-lane global element offsets (relative to the tile's first key) of the DMA
// instructions a wave issues for one tile.
template <int D, int WAVES, int TK>
struct DmaPlan {
    typedef TileGeom<D, TK> G;
    static constexpr int NK = G::KBLK / WAVES;      // K DMA instructions per wave
    static constexpr int NV = G::VBLK / 2 / WAVES;  // V DMA instructions (2 blocks each)
    static_assert(G::KBLK % WAVES == 0 && (G::VBLK / 2) % WAVES == 0, "even DMA split");
    int koff[NK];
    int voff[NV];

    __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int blk = wave + i * WAVES;  // = mt*KS + ks
            const int mt = blk / G::KS, ks = blk % G::KS;
            const int row = 32 * mt + kperm(lane & 31);
            koff[i] = row * D + 16 * ks + 8 * (lane >> 5);
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            // one DMA instruction fills V blocks 2j (lanes 0..31) and 2j+1 (32..63);
            // block index tb = ((mt*2 + e)*2 + r)*MD + md, md even for 2j.
            const int j = wave + i * WAVES;
            const int tb = 2 * j + (lane >> 5);
            const int md = tb % G::MD, r = (tb / G::MD) % 2, e = (tb / G::MD / 2) % 2,
                      mt = tb / G::MD / 4;
            const int u = 2 * (lane & 31);  // first of the two 8-byte units of this lane
            const int L = u & 15, g = (u >> 4) & 1, h = u >> 5;
            const int row = 32 * mt + 16 * e + 8 * h + 4 * r + (L >> 2);
            voff[i] = row * D + 32 * md + 16 * g + 4 * (L & 3);
        }
    }
};

template <int D, int WAVES, int TK, int OCC>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC))) void attn_bf16_kernel(FwdArgs a) {
    typedef TileGeom<D, TK> G;
    typedef DmaPlan<D, WAVES, TK> P;
    constexpr int TQ = 32 * WAVES;
    constexpr int KS = G::KS, MT = G::MT, MD = G::MD;

    __shared__ __attribute__((aligned(1024))) uint8_t k0s[G::BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t v0s[G::BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t k1s[G::BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t v1s[G::BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;
    const int l32 = lane & 31;

    const int wg = block_work(a);
    if (wg < 0) return;
    const int r = wg / a.sub_per_row;
    const int sub = wg - r * a.sub_per_row;
    const int bh = r / a.n_q;
    const int qi = r - bh * a.n_q;
    int beg, cnt;
    row_list(a, r, beg, cnt);
    const int sh = a.steps_log2;  // kernel steps per key block = 1 << sh
    const int n_steps = cnt << sh;
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

    P plan;
    plan.init(wave, lane);

    // List entries are fetched one step before they are needed, so the DMA issue
    // never waits on a global load: `pre` holds the entry of the next issue.
    auto entry_ptr = [&](int t) -> const int32_t* {
        const int i = t >> sh;
        return a.list + beg + (i < cnt ? i : cnt - 1);
    };
    int pre = cnt > 0 ? *entry_ptr(0) : 0;

    // HBM -> LDS DMA of step t's K and V tiles into one stage; prefetch the list
    // entry of step t+1.
    auto issue = [&](int t, uint8_t* ks_, uint8_t* vs_) {
        int kj = wave_uniform(pre);
        kj = kj < 0 ? 0 : (kj >= a.n_k ? a.n_k - 1 : kj);
        const int key0 = kj * a.block_k + (t & ((1 << sh) - 1)) * TK;
        pre = *entry_ptr(t + 1);
        const uint16_t* kt = kg + (size_t)key0 * D;
        const uint16_t* vt = vg + (size_t)key0 * D;
#pragma unroll
        for (int i = 0; i < P::NK; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(kt + plan.koff[i]),
                                             (BSATTN_LDS void*)(ks_ + (wave + i * WAVES) * 1024),
                                             16, 0, 0);
#pragma unroll
        for (int i = 0; i < P::NV; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(vt + plan.voff[i]),
                                             (BSATTN_LDS void*)(vs_ + (wave + i * WAVES) * 1024),
                                             16, 0, 0);
    };

    float m_run = -INFINITY;  // reference max (base-2, scaled units)
    float l_run = 0.f;        // this lane's partial row sum
    f32x16 oacc[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md) oacc[md] = f32x16{};

    auto compute = [&](const uint8_t* ks_, const uint8_t* vs_) {
        // S^T = K Q^T
        f32x16 sacc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) sacc[mt] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const bf16x8 kf = *(const bf16x8*)(ks_ + (mt * KS + ks) * 1024 + lane * 16);
                sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc[mt], 0, 0, 0);
            }

        // online softmax with a lazily moved reference max
        float tmp[16 * MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) tmp[16 * mt + i] = sacc[mt][i];
        const float mx = max_halves(tree_max<16 * MT>(tmp)) * a.c;
        if (__ballot(mx > m_run + 8.0f) != 0) {
            const float m_new = __builtin_fmaxf(m_run, mx);
            const float alpha = fast_exp2(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int md = 0; md < MD; ++md) oacc[md] *= alpha;
            m_run = m_new;
        }
        bf16x8 pb[MT][2];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = fast_exp2(__builtin_fmaf(sacc[mt][i], a.c, -m_run));
                tmp[16 * mt + i] = p;
                pb[mt][i >> 3][i & 7] = (__bf16)p;
            }
        l_run += tree_sum<16 * MT>(tmp);

        // O^T += V^T P^T
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int md = 0; md < MD; ++md) {
                    const uint8_t* vb = vs_ + (((mt * 2 + e) * 2) * MD + md) * 512 + lane * 8;
                    const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BSATTN_LDS bf16x4*)(vb));
                    const bf16x4 v1 =
                        __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BSATTN_LDS bf16x4*)(vb + MD * 512));
                    const bf16x8 vf = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
                    oacc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[mt][e], oacc[md], 0, 0, 0);
                }
    };

    // Two-stage pipeline over distinct LDS arrays (unrolled by two so each body
    // names its arrays statically).  Before computing step t: wait for this
    // wave's DMA of step t, barrier (all waves' DMA landed and all waves are done
    // with step t-1), then start step t+1's DMA into the array step t-1 used.
    if (n_steps > 0) {
        issue(0, k0s, v0s);
        for (int t = 0; t < n_steps; t += 2) {
            __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0)
            __syncthreads();
            if (t + 1 < n_steps) issue(t + 1, k1s, v1s);
            compute(k0s, v0s);
            if (t + 1 < n_steps) {
                __builtin_amdgcn_s_waitcnt(0x3f70);
                __syncthreads();
                if (t + 2 < n_steps) issue(t + 2, k0s, v0s);
                compute(k1s, v1s);
            }
        }
    }

    // Epilogue: O / l in bf16 (round to nearest even), lse = ln2 * (m + log2 l).
    const float l_tot = sum_halves(l_run);
    const bool any = n_steps > 0;
    const float inv = any ? 1.0f / l_tot : 0.0f;
    uint16_t* og = (uint16_t*)a.out + head + (size_t)q_row * D;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int d0 = 32 * md + 8 * g4 + 4 * h;
            bf16x4 o;
#pragma unroll
            for (int u = 0; u < 4; ++u) o[u] = (__bf16)(oacc[md][4 * g4 + u] * inv);
            *(bf16x4*)(og + d0) = o;
        }
    if (h == 0) a.lse[(size_t)bh * a.S + q_row] = any ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
}

template <int D, int W, int TK, int OCC>
static hipError_t launch_bf16(const FwdArgs& a, unsigned grid, hipStream_t stream) {
    hipLaunchKernelGGL((attn_bf16_kernel<D, W, TK, OCC>), dim3(grid), dim3(W * 64), 0, stream, a);
    return hipGetLastError();
}

#define BSATTN_BF16_VARIANT(D, W, TK) {1, D, 32 * W, TK, W, 2, &launch_bf16<D, W, TK, 2>}

static const Variant kBf16Variants[] = {
    BSATTN_BF16_VARIANT(128, 4, 64), BSATTN_BF16_VARIANT(128, 4, 32),
    BSATTN_BF16_VARIANT(128, 4, 128), BSATTN_BF16_VARIANT(128, 2, 64),
    BSATTN_BF16_VARIANT(128, 2, 32), BSATTN_BF16_VARIANT(128, 2, 128),
    BSATTN_BF16_VARIANT(64, 4, 64), BSATTN_BF16_VARIANT(64, 4, 128),
    BSATTN_BF16_VARIANT(64, 2, 64), BSATTN_BF16_VARIANT(64, 2, 32),
    BSATTN_BF16_VARIANT(64, 2, 128),
};

const Variant* bf16_variants(int* n) {
    *n = (int)(sizeof(kBf16Variants) / sizeof(kBf16Variants[0]));
    return kBf16Variants;
}

}  // namespace bsattn
