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
// Memory path.  K and V tiles go HBM -> LDS by direct DMA (buffer loads with the
// LDS flag, 16 B per lane), no VGPR staging.  Both are stored in LDS in the order the MFMA
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
#include <type_traits>

#ifndef BSATTN_SCHED_GROUPS
#define BSATTN_SCHED_GROUPS 0
#endif

#include "bf16_layout.h"
#include "common.h"
#include "kernels.h"

namespace bsattn {

template <int D, int WAVES, int TK, int NQ, int PIPE, int ST, int OCC, int PAIR, int ELEM>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC))) void attn_bf16_kernel(FwdArgs a) {
    typedef TileGeom<D, TK> G;
    typedef DmaPlan<D, WAVES, TK> P;
    constexpr int TQ = 32 * NQ * WAVES;  // query rows per workgroup (both rows of a pair)
    constexpr int KS = G::KS, MT = G::MT, MD = G::MD;
    static_assert(!PAIR || (WAVES == 8 && NQ == 1 && !PIPE), "row pairs: two 4-wave groups");

    static_assert(ST == 2 || (ST == 3 && !PIPE) || (ST == 1 && !PIPE && !PAIR && !ELEM),
                  "three stages use the plain schedule; one stage the 4-wave block-mask kernel");
    static_assert(!ELEM || (!PIPE && NQ == 1), "element masks: plain schedule, one 32-row tile per wave");
    __shared__ __attribute__((aligned(1024))) uint8_t k0s[G::BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t v0s[G::BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t k1s[G::BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t v1s[G::BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t k2s[ST > 2 ? G::BYTES : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t v2s[ST > 2 ? G::BYTES : 16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;
    const int l32 = lane & 31;

    int r, sub;
    block_work(a, r, sub);
    if (r < 0) return;
    const int sh = a.steps_log2;  // kernel steps per key block = 1 << sh
    int bh, qi, qi0, beg = 0, cnt;
    bool row_ok = true;  // this wave's query rows exist (false: second row of a pair past n_q)
    int q_row0;          // this lane's query row in each of the wave's NQ 32-row tiles
    // Row pairs: the workgroup runs over the union of the two rows' key-block lists,
    // built here in LDS as (kj | member bits << 30); group g = wave / 4 owns row 2j + g
    // and computes only the blocks of its own row.
    __shared__ uint32_t pair_bits[PAIR ? 2 * (kPairMaxBlocks / 32) : 1];
    __shared__ uint32_t pair_list[PAIR ? kPairMaxBlocks : 1];
    __shared__ int pair_cnt[1];
    // element masks on row pairs: tile + 1 of each key block of either row (0: full)
    __shared__ uint16_t pair_tile[PAIR && ELEM ? 2 * kPairMaxBlocks : 1];
    const int grp = PAIR ? wave >> 2 : 0;
    // A barrier that orders LDS accesses only (waits for this wave's LDS operations,
    // not for its global loads, which __syncthreads would drain as well).
    auto lds_sync = [&]() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    };
    // Q^T fragments: lane (h, q) holds Q[q][16*ks + 8*h .. +7] for every ks.
    bf16x8 qf[NQ][KS];
    auto load_q = [&](size_t head_q) {
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
            // (a missing row of a row group reads the group's first row, which
            // always exists; those values are never used)
            const int qr = row_ok ? q_row0 + 32 * n : q_row0 - (qi - qi0) * a.block_q;
            const u32x4* qp = (const u32x4*)((const uint16_t*)a.q + head_q + (size_t)qr * D);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                u32x4 t = qp[2 * ks + h];
                t ^= a.qsign;
                qf[n][ks] = __builtin_bit_cast(bf16x8, t);
            }
        }
    };
    if constexpr (PAIR) {
        if (a.n_k > kPairMaxBlocks) return;  // the host rejects such shapes first
        const int hq = (a.n_q + 1) >> 1;
        bh = r / hq;
        const int j = r - bh * hq;
        qi = 2 * j + grp;
        qi0 = 2 * j;
        row_ok = qi < a.n_q;
        const int ra = bh * a.n_q + 2 * j;
        const bool has_b = 2 * j + 1 < a.n_q;
        // The rows' first list entries, then the Q loads: the Q loads do not depend on
        // the list and stay in flight while it is built (its barriers order LDS only,
        // and a wait for the entries, issued first, leaves the later Q loads out).
        // (Padded lists: the entry loads need no count, so they go out first, then
        // the Q loads, then the count loads, which travel the scalar path.)
        int lb[2], lc[2], ent[2];
#pragma unroll
        for (int side = 0; side < 2; ++side) {
            ent[side] = 0;
            if ((side == 0 || has_b) && a.ell_stride > 0 && tid < a.n_k)
                ent[side] = a.list[(size_t)(ra + side) * a.ell_stride + tid];
        }
        q_row0 = qi * a.block_q + (wave & 3) * 32 + l32;
        load_q((size_t)bh * a.S * D);
#pragma unroll
        for (int side = 0; side < 2; ++side) {
            lb[side] = lc[side] = 0;
            if (side == 0 || has_b) {
                row_list(a, ra + side, lb[side], lc[side]);
                if (a.ell_stride == 0 && tid < lc[side]) ent[side] = a.list[lb[side] + tid];
            }
        }
        const int nw = (a.n_k + 31) >> 5;
        for (int w = tid; w < 2 * nw; w += WAVES * 64) pair_bits[(w / nw) * (kPairMaxBlocks / 32) + w % nw] = 0;
        lds_sync();
#pragma unroll
        for (int side = 0; side < 2; ++side) {
            const int b0 = lb[side], c0 = lc[side];
            for (int i = tid; i < c0; i += WAVES * 64) {
                int kj = i == tid ? ent[side] : a.list[b0 + i];
                int tile1 = 0;
                if constexpr (ELEM) {
                    tile1 = kj < 0 ? 0 : kj >> 16;
                    kj &= 0xffff;
                }
                kj = kj < 0 ? 0 : (kj >= a.n_k ? a.n_k - 1 : kj);
                atomicOr(&pair_bits[side * (kPairMaxBlocks / 32) + (kj >> 5)], 1u << (kj & 31));
                if constexpr (ELEM) pair_tile[side * kPairMaxBlocks + kj] = (uint16_t)tile1;
            }
        }
        lds_sync();
        if (wave == 0) {
            // Compact the union bitmap: lane l takes word l of each 64-word chunk.
            int base = 0;
            for (int w0 = 0; w0 < nw; w0 += 64) {
                const int w = w0 + lane;
                const uint32_t ba = w < nw ? pair_bits[w] : 0u;
                const uint32_t bb = w < nw ? pair_bits[(kPairMaxBlocks / 32) + w] : 0u;
                uint32_t u = ba | bb;
                const int c = __popc(u);
                int incl = c;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const int y = __shfl_up(incl, off, 64);
                    if (lane >= off) incl += y;
                }
                int pos = base + incl - c;
                while (u) {
                    const int bit = __builtin_ctz(u);
                    u &= u - 1;
                    const uint32_t m = 1u << bit;
                    pair_list[pos++] = (uint32_t)(w * 32 + bit) | ((ba & m) ? 1u << 30 : 0u) | ((bb & m) ? 1u << 31 : 0u);
                }
                base += __shfl(incl, 63, 64);
            }
            if (lane == 0) pair_cnt[0] = base;
        }
        lds_sync();
        cnt = wave_uniform(pair_cnt[0]);
    } else {
        bh = r / a.n_q;
        qi = r - bh * a.n_q;
        qi0 = qi;
        row_list(a, r, beg, cnt);
        q_row0 = qi * a.block_q + sub * TQ + wave * 32 * NQ + l32;
        load_q((size_t)bh * a.S * D);
    }
    const int n_steps = cnt << sh;
    const size_t head = (size_t)bh * a.S * D;
    const uint16_t* __restrict__ kg = (const uint16_t*)a.k + head;
    const uint16_t* __restrict__ vg = (const uint16_t*)a.v + head;


    P plan;
    plan.init(lane);
    const int wave_s = wave_uniform(wave);

    // Key-block list entries are fetched ahead of use so a DMA issue never waits
    // on a global load.
    auto entry = [&](int t) -> int {
        const int i = t >> sh;
        if constexpr (PAIR)
            return (int)pair_list[i < cnt ? i : cnt - 1];
        else
            return a.list[beg + (i < cnt ? i : cnt - 1)];
    };
    // Does this wave's row own the key block of step t (always, unless paired)?
    auto mine = [&](int t) -> bool {
        if constexpr (PAIR)
            return (pair_list[wave_uniform(t >> sh)] >> (30 + grp)) & 1u;
        else
            return true;
    };
    auto key0_of = [&](int kj_raw, int t) -> int {
        int kj = wave_uniform(kj_raw);
        if constexpr (PAIR) kj &= 0x3fffffff;
        if constexpr (ELEM) kj &= 0xffff;  // element masks: tile + 1 in bits 16..30
        kj = kj < 0 ? 0 : (kj >= a.n_k ? a.n_k - 1 : kj);
        return kj * a.block_k + (t & ((1 << sh) - 1)) * TK;
    };

    // HBM -> LDS DMA of one K tile or one V tile (keys key0 .. key0+TK-1), as raw
    // buffer loads over this head's K (or V): the per-lane byte offset is fixed,
    // the uniform part goes in the scalar offset (no per-step VALU address math).
    const int nrec = a.S * D * 2;
    const int k_voff = plan.k_lane * 2, v_voff = plan.v_lane * 2;
    auto issue_k = [&](int key0, uint8_t* kbuf) {
#pragma unroll
        for (int i = 0; i < P::NK; ++i)
            dma16(kg, nrec, (BSATTN_LDS void*)(kbuf + (wave_s + i * WAVES) * 1024), k_voff,
                  (key0 * D + P::k_uniform(wave_s, i)) * 2);
    };
    auto issue_v = [&](int key0, uint8_t* vbuf) {
#pragma unroll
        for (int i = 0; i < P::NV; ++i)
            dma16(vg, nrec, (BSATTN_LDS void*)(vbuf + (wave_s + i * WAVES) * 1024), v_voff,
                  (key0 * D + P::v_uniform(wave_s, i)) * 2);
    };

    float m_run[NQ];  // reference max per query tile (base-2, scaled units)
    float l_run[NQ];  // this lane's partial row sums
    f32x16 oacc[NQ][MD];
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
        m_run[n] = -INFINITY;
        l_run[n] = 0.f;
#pragma unroll
        for (int md = 0; md < MD; ++md) oacc[n][md] = f32x16{};
    }

    // VALU instructions placed between consecutive S MFMAs of the next tile: the
    // softmax costs ~3.5 VALU instructions per score element (fma, exp, half a
    // cvt, the sum tree), 16 elements per lane per 32-key tile and query tile,
    // spread over the NQ*KS MFMAs of that tile.
    constexpr int SCHED_VALU = 56 / KS;
    using yes = std::integral_constant<bool, true>;
    using no = std::integral_constant<bool, false>;
    struct SAcc { f32x16 v[NQ][MT]; };
    struct PTile { bf16x8 v[NQ][MT][2]; };

    // S^T = K Q^T for the K tile in kbuf; each K fragment read from LDS feeds the
    // NQ query tiles.
    auto qk = [&](const uint8_t* kbuf) -> SAcc {
        SAcc s;
#pragma unroll
        for (int n = 0; n < NQ; ++n)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) s.v[n][mt] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const bf16x8 kf = *(const bf16x8*)(kbuf + (mt * KS + ks) * 1024 + lane * 16);
#pragma unroll
                for (int n = 0; n < NQ; ++n)
                    s.v[n][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[n][ks], s.v[n][mt], 0, 0, 0);
            }
        return s;
    };

    // Row max of S and the lazy move of the reference max (rescaling O and l).
    auto update_max = [&](const SAcc& s) {
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
            float tmp[16 * MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) tmp[16 * mt + i] = s.v[n][mt][i];
            const float mx = max_halves_nan(max_tree3<16 * MT>(tmp)) * a.c;
            if (__ballot(mx > m_run[n] + 8.0f) != 0) {
                const float m_new = fmax_nan(m_run[n], mx);
                // (element masks: a row may still have no kept score, m = -inf;
                // its l and O are zero, and 2^(-inf - -inf) would be NaN)
                const float alpha =
                    (ELEM && m_run[n] == -INFINITY) ? 0.f : fast_exp2(m_run[n] - m_new);
                l_run[n] *= alpha;
#pragma unroll
                for (int md = 0; md < MD; ++md) oacc[n][md] *= alpha;
                m_run[n] = m_new;
            }
        }
    };

    // P = 2^(c S - m) in bf16, and its row sums into l.  (c > 0 always: a zero
    // scale arrives as the smallest normal float, so a dropped element's
    // S = -inf gives -inf, never -inf * 0.)
    auto exps = [&](const SAcc& s) -> PTile {
        PTile p;
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
            float tmp[16 * MT];
            // (element masks: with no kept score yet every S is -inf; use m = 0)
            const float m_use = (ELEM && m_run[n] == -INFINITY) ? 0.f : m_run[n];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float e = fast_exp2(__builtin_fmaf(s.v[n][mt][i], a.c, -m_use));
                    tmp[16 * mt + i] = e;
                    p.v[n][mt][i >> 3][i & 7] = (__bf16)e;
                }
            l_run[n] += tree_sum<16 * MT>(tmp);
        }
        return p;
    };

    // O^T += V^T P^T for the V tile in vbuf; each V fragment feeds NQ MFMAs.
    auto pv = [&](const PTile& p, const uint8_t* vbuf) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int md = 0; md < MD; ++md) {
                    const uint8_t* vb = vbuf + (((mt * 2 + e) * 2) * MD + md) * 512 + lane * 8;
                    const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BSATTN_LDS bf16x4*)(vb));
                    const bf16x4 v1 =
                        __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BSATTN_LDS bf16x4*)(vb + MD * 512));
                    const bf16x8 vf = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                    for (int n = 0; n < NQ; ++n)
                        oacc[n][md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, p.v[n][mt][e], oacc[n][md], 0, 0, 0);
                }
    };

    // Software pipeline.  K runs one step ahead of V: step t's body computes the
    // softmax of S(t) on the VALU while the matrix cores compute S(t+1) = K(t+1)
    // Q^T, then O += P(t) V(t).  Step s's K tile lives in k{s%2}s and its V tile
    // in v{s%2}s (distinct LDS arrays, named statically by unrolling by two).  At
    // the top of step t: wait for this wave's DMA (K(t+1), V(t), issued one step
    // earlier), barrier (everyone's DMA landed; everyone finished reading K(t)
    // and V(t-1)), then start the DMA of K(t+2) and V(t+1) into those buffers.
    auto body = [&](auto has_next, int t, int& kv_next, int& pre, SAcc& s, uint8_t* kfree,
                    uint8_t* vfree, const uint8_t* knext, const uint8_t* vcur) {
        constexpr bool NEXT = decltype(has_next)::value;
        __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0)
        __syncthreads();
        const int k2 = key0_of(pre, t + 2);
        pre = entry(t + 3);
        if (t + 2 < n_steps) issue_k(k2, kfree);
        if (t + 1 < n_steps) issue_v(kv_next, vfree);
        kv_next = k2;
        update_max(s);
        SAcc s_next;
        if constexpr (NEXT) s_next = qk(knext);
        const PTile p = exps(s);
        pv(p, vcur);
        if constexpr (NEXT) {
            s = s_next;
#if BSATTN_SCHED_GROUPS
            // Interleave the next tile's S MFMAs with this tile's exponentials
            // (independent work), then the P V MFMAs with their V reads.
#pragma unroll
            for (int i = 0; i < KS * MT; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);              // LDS read
                __builtin_amdgcn_sched_group_barrier(0x008, NQ, 0);             // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, NQ * SCHED_VALU, 0);  // VALU
            }
#pragma unroll
            for (int i = 0; i < 2 * MT * MD; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, NQ, 0);
            }
#endif
        }
    };

    // Plain schedule: K and V of step t share a stage, ST stages in flight.  The
    // body of step t waits until only the DMA of later steps is outstanding,
    // barriers (everyone's step-t data landed; everyone is done with step t-1's
    // stage), then loads the list entry two issues ahead and starts the DMA of
    // step t+ST-1 into the stage step t-1 used, then runs S, softmax, P V.
    // vmcnt counts in issue order: list-entry load, then the step's DMA, so
    // waiting for "at most NDMA outstanding" (ST = 3) retires step t's DMA and
    // the entry load issued before step t+1's DMA.
    constexpr int NDMA = P::NK + P::NV;
    // Element masks: the list entries of the steps in flight (e1 = this step, e2 =
    // the next with three stages), and the kept-bit test applied to S.
    int e1 = 0, e2 = 0;
    auto apply_tile = [&](SAcc& s, int e, int t) {
        int tile = (e >> 16) - 1;  // -1: full block
        if (tile < 0) return;
        tile = tile < a.n_tiles ? tile : a.n_tiles - 1;  // (a plan never holds more)
        const int qr = q_row0 - qi * a.block_q;  // this lane's row inside the block
        const int ko = (t & ((1 << sh) - 1)) * TK;
        const int wpr = a.block_k >> 5;  // words per tile row
        const uint32_t* wrow = a.pbits + ((size_t)tile * a.block_q + qr) * wpr + (ko >> 5);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            // register i holds key 16*(i/8) + 8h + i%8 of the 32-key tile mt
            const uint32_t w = wrow[mt] >> (8 * h);
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (!((w >> (16 * (i >> 3) + (i & 7))) & 1u)) s.v[0][mt][i] = -INFINITY;
        }
    };
    auto plain = [&](int t, int& pre, uint8_t* kfill, uint8_t* vfill, const uint8_t* kcur,
                     const uint8_t* vcur) {
        if (ST == 3 && t + 1 < n_steps)
            __builtin_amdgcn_s_waitcnt(0x3f70 | (NDMA & 15) | ((NDMA >> 4) << 14));
        else
            __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0)
        __syncthreads();
        const int e_cur = e1;
        if constexpr (ELEM && ST == 3) e1 = e2;
        if (t + ST - 1 < n_steps) {
            const int kn = key0_of(pre, t + ST - 1);
            if constexpr (ELEM) (ST == 3 ? e2 : e1) = wave_uniform(pre);
            pre = entry(t + ST);
            issue_k(kn, kfill);
            issue_v(kn, vfill);
        }
        if (mine(t)) {
            SAcc s = qk(kcur);
            if constexpr (ELEM && PAIR)  // this group's own tile of the block
                apply_tile(s, (int)pair_tile[grp * kPairMaxBlocks + (e_cur & 0xffff)] << 16, t);
            else if constexpr (ELEM)
                apply_tile(s, e_cur, t);
            update_max(s);
            const PTile p = exps(s);
            pv(p, vcur);
        }
    };

    if (n_steps > 0 && ST == 1) {
        // One stage: copy, wait, barrier, compute, then a barrier before the next
        // copy overwrites the stage -- the copy never overlaps the compute.
        int pre = entry(0);
        for (int t = 0; t < n_steps; ++t) {
            const int kn = key0_of(pre, t);
            pre = entry(t + 1);
            if (t > 0) __syncthreads();  // everyone is done reading step t - 1
            issue_k(kn, k0s);
            issue_v(kn, v0s);
            __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0)
            __syncthreads();
            SAcc s = qk(k0s);
            update_max(s);
            const PTile p = exps(s);
            pv(p, v0s);
        }
    } else if (n_steps > 0 && PIPE) {
        const int k0 = key0_of(entry(0), 0);
        const int k1 = key0_of(entry(1), 1);
        int pre = entry(2);
        issue_k(k0, k0s);
        issue_v(k0, v0s);
        if (n_steps > 1) issue_k(k1, k1s);
        int kv_next = k1;
        __builtin_amdgcn_s_waitcnt(0x3f70);
        __syncthreads();
        SAcc s = qk(k0s);
        int t = 0;
        for (; t + 2 < n_steps; t += 2) {
            body(yes{}, t, kv_next, pre, s, k0s, v1s, k1s, v0s);
            body(yes{}, t + 1, kv_next, pre, s, k1s, v0s, k0s, v1s);
        }
        if (t + 1 < n_steps) {
            body(yes{}, t, kv_next, pre, s, k0s, v1s, k1s, v0s);
            body(no{}, t + 1, kv_next, pre, s, k1s, v0s, k0s, v1s);
        } else {
            body(no{}, t, kv_next, pre, s, k0s, v1s, k1s, v0s);
        }
    } else if (n_steps > 0 && ST == 2) {
        e1 = wave_uniform(entry(0));
        const int k0 = key0_of(e1, 0);
        int pre = entry(1);
        issue_k(k0, k0s);
        issue_v(k0, v0s);
        for (int t = 0; t < n_steps; t += 2) {
            plain(t, pre, k1s, v1s, k0s, v0s);
            if (t + 1 < n_steps) plain(t + 1, pre, k0s, v0s, k1s, v1s);
        }
    } else if (n_steps > 0) {
        e1 = wave_uniform(entry(0));
        e2 = wave_uniform(entry(1));
        const int k0 = key0_of(e1, 0);
        const int k1 = key0_of(e2, 1);
        int pre = entry(2);
        issue_k(k0, k0s);
        issue_v(k0, v0s);
        if (n_steps > 1) {
            issue_k(k1, k1s);
            issue_v(k1, v1s);
        }
        for (int t = 0; t < n_steps; t += 3) {
            plain(t, pre, k2s, v2s, k0s, v0s);
            if (t + 1 < n_steps) plain(t + 1, pre, k0s, v0s, k1s, v1s);
            if (t + 2 < n_steps) plain(t + 2, pre, k1s, v1s, k2s, v2s);
        }
    }

    // Epilogue: O / l in bf16 (round to nearest even), lse = ln2 * (m + log2 l).
    // A row that saw no key block (m never left -inf) gets 0 and -inf.
    // A lane holds 8 bytes of its row per (md, g4), so storing straight from the
    // registers writes 32 rows x 16 bytes per instruction (a quarter of each line).
    // Where the stage arrays can hold every wave's 32 x D tile, the tile goes
    // through LDS instead (16-byte units XOR-swizzled by row) and leaves as whole
    // rows, 64 / (D / 8) rows per instruction.
    constexpr int CPR = D / 8;                     // 16-byte units per output row
    constexpr int REG = 32 * D * 2;                // one wave's tile
    constexpr int WPA = G::BYTES / REG;            // tiles per stage array
    constexpr int NARR = ST > 2 ? 6 : 4;           // k0s v0s k1s v1s (k2s v2s)
    constexpr bool STAGED = NQ == 1 && WPA >= 1 && WAVES <= WPA * NARR;
    if constexpr (STAGED) {
        __syncthreads();  // every wave is done with the last step's stage
        if (!row_ok) return;
        const bool any = (PAIR || ELEM) ? m_run[0] != -INFINITY : n_steps > 0;
        const float l_tot = sum_halves(l_run[0]);
        const float inv = any ? 1.0f / l_tot : 0.0f;
        const int arr = wave / (WPA > 0 ? WPA : 1);
        uint8_t* const arrs[6] = {k0s, v0s, k1s, v1s, k2s, v2s};
        uint8_t* tile = arrs[arr] + (wave % (WPA > 0 ? WPA : 1)) * REG;
#pragma unroll
        for (int md = 0; md < MD; ++md)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                // d = 32 md + 8 g4 + 4 h .. +3: unit 4 md + g4, half h
                const int c = 4 * md + g4;
                bf16x4 o;
#pragma unroll
                for (int u = 0; u < 4; ++u) o[u] = (__bf16)(oacc[0][md][4 * g4 + u] * inv);
                *(bf16x4*)(tile + l32 * (2 * D) + ((c ^ (l32 & (CPR - 1))) << 4) + 8 * h) = o;
            }
        constexpr int RPI = 64 / CPR;  // rows per store instruction
        const int row0 = q_row0 - l32;
        uint16_t* og = (uint16_t*)a.out + head + (size_t)row0 * D;
#pragma unroll
        for (int i = 0; i < 32 / RPI; ++i) {
            const int rr = RPI * i + lane / CPR, c = lane % CPR;
            const u32x4 v = *(const u32x4*)(tile + rr * (2 * D) + ((c ^ (rr & (CPR - 1))) << 4));
            *(u32x4*)(og + (size_t)rr * D + 8 * c) = v;
        }
        if (h == 0)
            a.lse[(size_t)bh * a.S + q_row0] = any ? (m_run[0] + log2f(l_tot)) * kLn2 : -INFINITY;
        return;
    }
    if (!row_ok) return;
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
        const bool any = (PAIR || ELEM) ? m_run[n] != -INFINITY : n_steps > 0;
        const int q_row = q_row0 + 32 * n;
        const float l_tot = sum_halves(l_run[n]);
        const float inv = any ? 1.0f / l_tot : 0.0f;
        uint16_t* og = (uint16_t*)a.out + head + (size_t)q_row * D;
#pragma unroll
        for (int md = 0; md < MD; ++md)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d0 = 32 * md + 8 * g4 + 4 * h;
                bf16x4 o;
#pragma unroll
                for (int u = 0; u < 4; ++u) o[u] = (__bf16)(oacc[n][md][4 * g4 + u] * inv);
                *(bf16x4*)(og + d0) = o;
            }
        if (h == 0)
            a.lse[(size_t)bh * a.S + q_row] = any ? (m_run[n] + log2f(l_tot)) * kLn2 : -INFINITY;
    }
}

template <int D, int W, int TK, int NQ, int PIPE, int ST, int OCC, int PAIR = 0, int ELEM = 0>
static hipError_t launch_bf16(const FwdArgs& a, unsigned grid, hipStream_t stream) {
    hipLaunchKernelGGL((attn_bf16_kernel<D, W, TK, NQ, PIPE, ST, OCC, PAIR, ELEM>), dim3(grid), dim3(W * 64), 0,
                       stream, a);
    return hipGetLastError();
}

// {dtype, D, tile_q, tile_k, waves, stages, launcher}.  With no tuning result the
// host prefers the row-pair entries (for 128-row mask blocks), else takes the
// first legal entry in table order.  NQ = 2 (64 query rows per
// wave, each K/V fragment read from LDS feeding two MFMAs) runs one wave per
// SIMD; NQ = 1 runs two to five (OCC): with D = 64 the softmax is as much VALU
// work as with D = 128 against half the MFMA work, and four or five waves per
// SIMD hide it better than two.  PIPE = 1 overlaps the next tile's S MFMAs
// with this tile's softmax inside a wave (two stages); PIPE = 0 runs the steps
// in order with ST K/V stages resident in LDS.
#define BSATTN_BF16_VARIANT(D, W, TK, NQ, PIPE, ST, OCC) \
    {1, D, 32 * NQ * W, TK, W, ST, &launch_bf16<D, W, TK, NQ, PIPE, ST, OCC>}
// Row pairs: 8 waves, two adjacent 128-row mask rows of a head per workgroup
// (tile_q 256), sharing every K/V tile of the union of their block lists.
#define BSATTN_BF16_PAIR(D, TK, ST, OCC) \
    {1, D, 256, TK, 8, ST, &launch_bf16<D, 8, TK, 1, 0, ST, OCC, 1>}

static const Variant kBf16Variants[] = {
    BSATTN_BF16_VARIANT(128, 4, 32, 1, 0, 3, 3), BSATTN_BF16_VARIANT(128, 4, 64, 1, 1, 2, 2),
    BSATTN_BF16_VARIANT(128, 4, 32, 1, 1, 2, 2), BSATTN_BF16_VARIANT(128, 4, 64, 1, 0, 3, 1),
    BSATTN_BF16_VARIANT(128, 2, 64, 2, 0, 2, 1), BSATTN_BF16_VARIANT(128, 2, 32, 2, 0, 3, 1),
    BSATTN_BF16_VARIANT(128, 2, 32, 1, 0, 3, 3), BSATTN_BF16_VARIANT(128, 2, 64, 1, 1, 2, 2),
    BSATTN_BF16_VARIANT(128, 1, 32, 2, 0, 3, 1),
    // the rest of the tuning space (tile_q 64/128, tile_k 32/64/128, 2/4 waves,
    // 1-3 stages) that fits the LDS and the registers
    BSATTN_BF16_VARIANT(128, 2, 32, 1, 0, 2, 3), BSATTN_BF16_VARIANT(128, 2, 64, 1, 0, 3, 1),
    BSATTN_BF16_VARIANT(128, 2, 128, 1, 0, 2, 1), BSATTN_BF16_VARIANT(128, 2, 32, 2, 0, 2, 1),
    BSATTN_BF16_VARIANT(128, 2, 64, 2, 0, 3, 1), BSATTN_BF16_VARIANT(128, 4, 128, 1, 0, 2, 1),
    BSATTN_BF16_VARIANT(128, 4, 32, 1, 0, 1, 3), BSATTN_BF16_VARIANT(128, 4, 64, 1, 0, 1, 2),
    BSATTN_BF16_VARIANT(128, 4, 128, 1, 0, 1, 1), BSATTN_BF16_VARIANT(128, 2, 32, 1, 0, 1, 3),
    BSATTN_BF16_VARIANT(128, 2, 64, 1, 0, 1, 2), BSATTN_BF16_VARIANT(128, 2, 128, 1, 0, 1, 1),
    BSATTN_BF16_VARIANT(128, 2, 32, 2, 0, 1, 1), BSATTN_BF16_VARIANT(128, 2, 64, 2, 0, 1, 1),
    {1, 128, 128, 32, 8, 3, &launch_bf16_pp<128>},
    BSATTN_BF16_PAIR(128, 32, 3, 2), BSATTN_BF16_PAIR(128, 64, 3, 2),
    BSATTN_BF16_PAIR(128, 64, 2, 2), BSATTN_BF16_PAIR(128, 128, 2, 2),
    BSATTN_BF16_VARIANT(64, 4, 64, 1, 0, 2, 4),  BSATTN_BF16_VARIANT(64, 4, 64, 1, 0, 3, 3),
    BSATTN_BF16_VARIANT(64, 4, 32, 1, 0, 2, 5),  BSATTN_BF16_VARIANT(64, 4, 128, 1, 0, 2, 2),
    BSATTN_BF16_VARIANT(64, 2, 64, 2, 0, 2, 1),  BSATTN_BF16_VARIANT(64, 2, 128, 2, 0, 2, 1),
    BSATTN_BF16_VARIANT(64, 2, 64, 1, 0, 3, 2),  BSATTN_BF16_VARIANT(64, 2, 32, 1, 1, 2, 2),
    BSATTN_BF16_VARIANT(64, 1, 64, 2, 0, 2, 1),
    BSATTN_BF16_VARIANT(64, 2, 32, 1, 0, 3, 3), BSATTN_BF16_VARIANT(64, 2, 64, 1, 0, 2, 3),
    BSATTN_BF16_VARIANT(64, 2, 128, 1, 0, 2, 1), BSATTN_BF16_VARIANT(64, 2, 128, 1, 0, 3, 1),
    BSATTN_BF16_VARIANT(64, 2, 32, 2, 0, 2, 1), BSATTN_BF16_VARIANT(64, 2, 32, 2, 0, 3, 1),
    BSATTN_BF16_VARIANT(64, 2, 64, 2, 0, 3, 1), BSATTN_BF16_VARIANT(64, 2, 128, 2, 0, 3, 1),
    BSATTN_BF16_VARIANT(64, 4, 32, 1, 0, 3, 3), BSATTN_BF16_VARIANT(64, 4, 128, 1, 0, 3, 1),
    BSATTN_BF16_VARIANT(64, 4, 32, 1, 0, 1, 4), BSATTN_BF16_VARIANT(64, 4, 64, 1, 0, 1, 3),
    BSATTN_BF16_VARIANT(64, 4, 128, 1, 0, 1, 2), BSATTN_BF16_VARIANT(64, 2, 32, 1, 0, 1, 4),
    BSATTN_BF16_VARIANT(64, 2, 64, 1, 0, 1, 3), BSATTN_BF16_VARIANT(64, 2, 128, 1, 0, 1, 2),
    BSATTN_BF16_VARIANT(64, 2, 32, 2, 0, 1, 1), BSATTN_BF16_VARIANT(64, 2, 64, 2, 0, 1, 1),
    BSATTN_BF16_VARIANT(64, 2, 128, 2, 0, 1, 1),
    {1, 64, 128, 32, 8, 3, &launch_bf16_pp<64>},
    BSATTN_BF16_PAIR(64, 64, 3, 4), BSATTN_BF16_PAIR(64, 64, 2, 4), BSATTN_BF16_PAIR(64, 128, 2, 2),
};

// Element-level masks (plain schedule, one 32-row query tile per wave): the best
// block-mask configs of each D, row pairs included.
#define BSATTN_BF16_ELEM(D, W, TK, ST, OCC) \
    {1, D, 32 * W, TK, W, ST, &launch_bf16<D, W, TK, 1, 0, ST, OCC, 0, 1>}

#define BSATTN_BF16_ELEM_PAIR(D, TK, ST, OCC) \
    {1, D, 256, TK, 8, ST, &launch_bf16<D, 8, TK, 1, 0, ST, OCC, 1, 1>}

static const Variant kBf16ElemVariants[] = {
    BSATTN_BF16_ELEM(128, 4, 32, 3, 3), BSATTN_BF16_ELEM(128, 4, 64, 2, 2), BSATTN_BF16_ELEM(128, 2, 32, 3, 3),
    BSATTN_BF16_ELEM_PAIR(128, 128, 2, 2), BSATTN_BF16_ELEM_PAIR(128, 64, 2, 2),
    BSATTN_BF16_ELEM_PAIR(64, 64, 2, 4), BSATTN_BF16_ELEM_PAIR(64, 128, 2, 2),
    BSATTN_BF16_ELEM(64, 4, 64, 2, 4),  BSATTN_BF16_ELEM(64, 4, 32, 2, 5),  BSATTN_BF16_ELEM(64, 4, 128, 2, 2),
    BSATTN_BF16_ELEM(64, 2, 64, 3, 2),
};

const Variant* bf16_elem_variants(int* n) {
    *n = (int)(sizeof(kBf16ElemVariants) / sizeof(kBf16ElemVariants[0]));
    return kBf16ElemVariants;
}

const Variant* bf16_variants(int* n) {
    *n = (int)(sizeof(kBf16Variants) / sizeof(kBf16Variants[0]));
    return kBf16Variants;
}

}  // namespace bsattn
