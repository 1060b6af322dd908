// attn_bwd.hip -- backward of the block-sparse flash-attention forward for gfx950:
// dq, dk, dv from q, k, v, the forward's out and lse, and the upstream gradient
// dout.  bf16 in, fp32 accumulation, bf16 or fp32 gradients.
//
// What is computed.  "Writing Pallas Kernels for JAX" (rajatpandit.com), section
// "The Empathy of the Void": a hand-written kernel has no automatic gradient, so
// its author writes one.  For the forward of that page (scaled scores, -inf where
// the block mask is 0, row softmax, times V) the chain rule gives, with
// P[r][j] = exp(scale * q_r . k_j - lse_r) on the active keys of row r:
//   dv_j = sum_r P[r][j] dout_r              dP[r][j] = dout_r . v_j
//   delta_r = sum_j P[r][j] dP[r][j] = dout_r . out_r
//   dS[r][j] = P[r][j] (dP[r][j] - delta_r)
//   dq_r = scale sum_j dS[r][j] k_j          dk_j = scale sum_r dS[r][j] q_r
// P is rebuilt exactly from the saved lse, so no running max is needed.
//
// Kernels.
//   bwd_prep_kernel  per row: (lse * log2 e, delta) as a float2 (lse = -inf, a row
//                    that saw no key, becomes +inf so that its P is 0).
//   bwd_cols_kernel  the column form of the block mask: per key block (b, h, kj)
//                    the ascending list of query blocks that see it.
//   bwd_split_kernel the dk/dv work items: one per key block, except that a
//                    block seen by more query blocks than a piece length T is cut
//                    into pieces of T (a few global key blocks seen by every query
//                    block would otherwise be the critical path of the launch).
//                    T is the smallest power of two >= total / 1024 whose pieces
//                    fit the scratch slots.
//   bwd_dkdv_kernel  one workgroup per item (32 keys per wave), walking its
//                    query-block list in 32-query steps.  Per step and wave:
//                      S = Q K^T, dP = dO V^T   (A = Q, dO rows from LDS in the K
//                                               layout, B = the wave's K, V rows
//                                               held in VGPRs; lane = key column)
//                      P = 2^(c S - lse2), dS = P (dP - delta)
//                      dV^T += dO^T P, dK^T += Q^T dS  (A from LDS by the
//                                               transposing read, B = P, dS from
//                                               the S registers)
//                    Q and dO rows enter the first MFMAs in the bit-swapped order
//                    kperm, so the queries a lane holds afterwards are exactly the
//                    k-slots the second MFMAs want (as K rows in the forward).
//   bwd_dq_kernel    one workgroup per query block (32 queries per wave), walking
//                    the mask row's key-block list in 32-key steps:
//                      S^T = K Q^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T.
//   bwd_reduce_kernel  per cut key block: its pieces' fp32 partials summed in
//                    piece order, dK scaled, stored.
// The two main kernels recompute S and dP each (dq is not accumulated across
// workgroups: no atomics, deterministic results).  Tiles stream HBM -> LDS by
// buffer loads with the LDS flag in the operand layouts of bf16_layout.h, two
// stages, one barrier per step.
#include "bf16_layout.h"
#include "common.h"
#include "kernels.h"

namespace bsattn {

namespace {

__device__ __forceinline__ float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// Workgroup -> (slot, sub-tile): slots are dealt to the 8 XCDs in contiguous
// chunks (block b runs on XCD b % 8), so the slots of one head share an L2.
__device__ __forceinline__ int bwd_slot(const BwdArgs& a, const int32_t* order, int chunk, int nslots) {
    const int b = blockIdx.x;
    const int j = b >> 3;
    int r = -1;
    if (j < chunk) {
        const int slot = (b & 7) * chunk + j;
        r = order ? order[slot] : slot;
    }
    if (r < 0 || r >= nslots) r = -1;
    return wave_uniform(r);
}

template <int D>
__device__ __forceinline__ void store4(void* base, size_t idx, const float* x, int out_f32) {
    if (out_f32) {
        *(float4*)((float*)base + idx) = make_float4(x[0], x[1], x[2], x[3]);
    } else {
        bf16x4 o;
#pragma unroll
        for (int u = 0; u < 4; ++u) o[u] = (__bf16)x[u];
        *(bf16x4*)((uint16_t*)base + idx) = o;
    }
}

}  // namespace

template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint16_t* __restrict__ out,
                                                       const uint16_t* __restrict__ dout,
                                                       const float* __restrict__ lse, float2* __restrict__ ld,
                                                       int64_t rows) {
    constexpr int TPR = D / 8;  // threads per row, 16 bytes each
    constexpr int RPB = 256 / TPR;
    const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
    const int part = threadIdx.x % TPR;
    float acc = 0.f;
    if (r < rows) {
        const u32x4 o = *(const u32x4*)(out + r * D + part * 8);
        const u32x4 g = *(const u32x4*)(dout + r * D + part * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc += bf_lo(o[i]) * bf_lo(g[i]) + bf_hi(o[i]) * bf_hi(g[i]);
    }
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (r < rows && part == 0) {
        const float l = lse[r];
        ld[r] = make_float2(l == -INFINITY ? INFINITY : l * kLog2e, acc);
    }
}

// One wave per key block (column): the ascending list of query blocks whose mask
// byte is nonzero.  Lane l tests query block q0 + l; a ballot and a prefix count
// of the lower lanes place each hit.
__global__ __launch_bounds__(256) void bwd_cols_kernel(const uint8_t* __restrict__ mask, int64_t C, int n_q,
                                                       int n_k, int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ lists) {
    const int64_t col = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (col >= C) return;
    const int lane = threadIdx.x & 63;
    const int64_t bh = col / n_k;
    const int kj = (int)(col - bh * n_k);
    const uint8_t* m = mask + bh * n_q * n_k + kj;
    int32_t* lst = lists + col * n_q;
    int cnt = 0;
    for (int q0 = 0; q0 < n_q; q0 += 64) {
        const int qi = q0 + lane;
        const bool hit = qi < n_q && m[(int64_t)qi * n_k] != 0;
        const uint64_t bal = __ballot(hit);
        if (hit) lst[cnt + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u))] = qi;
        cnt += __popcll(bal);
    }
    if (lane == 0) counts[col] = cnt;
}

// Inclusive scan over the 1024 threads of a workgroup (wave scans, then a scan of
// the wave totals).
__device__ __forceinline__ int64_t bwd_block_scan(int64_t x, int64_t* wave_tot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int64_t y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) wave_tot[wave] = x;
    __syncthreads();
    if (wave == 0) {
        int64_t t = lane < 16 ? wave_tot[lane] : 0;
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            const int64_t y = __shfl_up(t, off, 64);
            if (lane >= off) t += y;
        }
        if (lane < 16) wave_tot[lane] = t;
    }
    __syncthreads();
    const int64_t r = x + (wave > 0 ? wave_tot[wave - 1] : 0);
    __syncthreads();
    return r;
}

__device__ __forceinline__ int64_t bwd_block_sum(int64_t x, int64_t* wave_tot) {
    const int64_t incl = bwd_block_scan(x, wave_tot);
    __shared__ int64_t total;
    if (threadIdx.x == 1023) total = incl;
    __syncthreads();
    const int64_t t = total;
    __syncthreads();
    return t;
}

// One workgroup of 1024 threads: the dk/dv work items (header) from the column
// counts.  items holds at most C + max_slots entries, splits at most max_slots / 2.
__global__ __launch_bounds__(1024) void bwd_split_kernel(const int32_t* __restrict__ counts, int64_t C, int n_q,
                                                         int max_slots, int4* __restrict__ items,
                                                         int4* __restrict__ splits, int32_t* __restrict__ n_out) {
    __shared__ int64_t wave_tot[16];
    __shared__ int64_t carry[3];  // items, slots, splits before this chunk
    const int tid = threadIdx.x;
    auto cnt_of = [&](int64_t c) -> int {
        const int x = counts[c];
        return x < 0 ? 0 : (x > n_q ? n_q : x);
    };
    int64_t total = 0;
    for (int64_t c0 = 0; c0 < C; c0 += 1024) total += c0 + tid < C ? cnt_of(c0 + tid) : 0;
    total = bwd_block_sum(total, wave_tot);
    int T = 8;
    while ((int64_t)T * 1024 < total) T <<= 1;
    for (;; T <<= 1) {  // ends: once T >= n_q no column is cut
        int64_t pieces = 0;
        for (int64_t c0 = 0; c0 < C; c0 += 1024)
            if (c0 + tid < C) {
                const int x = cnt_of(c0 + tid);
                pieces += x > T ? (x + T - 1) / T : 0;
            }
        if (bwd_block_sum(pieces, wave_tot) <= max_slots || T >= n_q) break;
    }
    if (tid == 0) carry[0] = carry[1] = carry[2] = 0;
    __syncthreads();
    for (int64_t c0 = 0; c0 < C; c0 += 1024) {
        const int64_t c = c0 + tid;
        const int x = c < C ? cnt_of(c) : 0;
        const bool cut = c < C && x > T;
        const int np = cut ? (x + T - 1) / T : 0;
        const int64_t n_it = c < C ? (cut ? np : 1) : 0;
        const int64_t it_incl = bwd_block_scan(n_it, wave_tot);
        const int64_t sl_incl = bwd_block_scan(np, wave_tot);
        const int64_t sp_incl = bwd_block_scan(cut ? 1 : 0, wave_tot);
        const int64_t it0 = carry[0] + it_incl - n_it, sl0 = carry[1] + sl_incl - np;
        if (c < C) {
            if (cut) {
                for (int p = 0; p < np; ++p) {
                    const int len = x - p * T < T ? x - p * T : T;
                    items[it0 + p] = make_int4((int)c, p * T, len, (int)(sl0 + p));
                }
                splits[carry[2] + sp_incl - 1] = make_int4((int)c, (int)sl0, np, 0);
            } else {
                items[it0] = make_int4((int)c, 0, x, -1);
            }
        }
        __syncthreads();
        if (tid == 1023) {
            carry[0] += it_incl;
            carry[1] += sl_incl;
            carry[2] += sp_incl;
        }
        __syncthreads();
    }
    if (tid == 0) {
        n_out[0] = (int32_t)carry[0];
        n_out[1] = (int32_t)carry[2];
    }
}

// dK and dV of one key block.  WAVES * 32 = block_k keys per workgroup.  The
// register budget is cut for two waves per SIMD with D = 128 (K, V fragments and
// the dK, dV accumulators alone take 192 VGPRs) and three with D = 64.
template <int D, int WAVES, int OUT_F32, int ELEM>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, D == 64 ? 3 : 2))) void bwd_dkdv_kernel(
    BwdArgs a) {
    typedef TileGeom<D, 32> G;  // one 32-row tile of Q or dO
    typedef DmaPlan<D, WAVES, 32> P;
    typedef KRowPlan<D, WAVES, 32> KP;
    // Q and dO tiles for the S and dP MFMAs: row-chunk layout, except with element
    // masks, whose extra registers would then spill; those keep the 1 KiB-per-k-step
    // blocks of DmaPlan.
    constexpr bool RK = !ELEM;
    constexpr int KS = G::KS, MD = G::MD;
    __shared__ __attribute__((aligned(1024))) uint8_t qk0[G::BYTES], qv0[G::BYTES], ok0[G::BYTES], ov0[G::BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t qk1[G::BYTES], qv1[G::BYTES], ok1[G::BYTES], ov1[G::BYTES];
    __shared__ __attribute__((aligned(1024))) float2 ld0[128], ld1[128];

    // items per XCD chunk from the plan's item count (the grid is sized for the
    // most items a plan can hold)
    int n_it = wave_uniform(a.n_items[0]);
    n_it = n_it < a.n_cols + a.max_slots ? n_it : a.n_cols + a.max_slots;
    const int item = bwd_slot(a, nullptr, (n_it + 7) >> 3, n_it);
    if (item < 0) return;
    const int4 it = a.items[item];
    // (fields clamped into range: a malformed plan gives wrong values, never an
    // access out of bounds)
    int col = wave_uniform(it.x), part_slot = wave_uniform(it.w);
    col = col < 0 ? 0 : (col >= a.n_cols ? a.n_cols - 1 : col);
    part_slot = part_slot >= a.max_slots ? a.max_slots - 1 : part_slot;
    int first = wave_uniform(it.y), cnt = wave_uniform(it.z);
    first = first < 0 ? 0 : (first > a.n_q ? a.n_q : first);
    cnt = cnt < 0 ? 0 : (cnt > a.n_q - first ? a.n_q - first : cnt);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
    const int wave_s = wave_uniform(wave);
    const int bh = col / a.n_k;
    const int kj = col - bh * a.n_k;
    const int32_t* lst = a.col_lists + (size_t)col * a.n_q + first;
    const size_t head = (size_t)bh * a.S * D;
    const int key = kj * a.block_k + wave * 32 + l32;

    // B operands: lane (h, key) holds K[key][16ks + 8h .. +7] and the same of V.
    bf16x8 kf[KS], vf[KS];
    {
        const u32x4* kp = (const u32x4*)(a.k + head + (size_t)key * D);
        const u32x4* vp = (const u32x4*)(a.v + head + (size_t)key * D);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            kf[ks] = __builtin_bit_cast(bf16x8, kp[2 * ks + h]);
            vf[ks] = __builtin_bit_cast(bf16x8, vp[2 * ks + h]);
        }
    }

    f32x16 dka[MD], dva[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md) dka[md] = dva[md] = f32x16{};

    const int spb_log2 = a.qsteps_log2;  // 32-query steps per query block
    const int n_steps = cnt << spb_log2;
    auto entry = [&](int i) -> int {
        int qi = wave_uniform(lst[i < cnt ? i : cnt - 1]);
        return qi < 0 ? 0 : (qi >= a.n_q ? a.n_q - 1 : qi);
    };

    P plan;
    plan.init(lane);
    KP kplan;
    kplan.init(lane);
    const int nrec = a.S * D * 2;
    const int v_voff = plan.v_lane * 2;
    const uint16_t* qg = a.q + head;
    const uint16_t* og = a.dout + head;
    const float2* ldg = a.ld + (size_t)bh * a.S;
    auto issue = [&](int q0, uint8_t* qk, uint8_t* qv, uint8_t* ok, uint8_t* ov, float2* ldb) {
#pragma unroll
        for (int i = 0; i < KP::NK; ++i) {
            const int soff = (q0 * D + (RK ? KP::uniform(wave_s, i) : P::k_uniform(wave_s, i))) * 2;
            const int k_voff = (RK ? kplan.dma_off(wave_s, i) : plan.k_lane) * 2;
            dma16(qg, nrec, (BSATTN_LDS void*)(qk + (wave_s + i * WAVES) * 1024), k_voff, soff);
            dma16(og, nrec, (BSATTN_LDS void*)(ok + (wave_s + i * WAVES) * 1024), k_voff, soff);
        }
#pragma unroll
        for (int i = 0; i < P::NV; ++i) {
            const int soff = (q0 * D + P::v_uniform(wave_s, i)) * 2;
            dma16(qg, nrec, (BSATTN_LDS void*)(qv + (wave_s + i * WAVES) * 1024), v_voff, soff);
            dma16(og, nrec, (BSATTN_LDS void*)(ov + (wave_s + i * WAVES) * 1024), v_voff, soff);
        }
        // (lse2, delta) of the 32 queries: 256 bytes; lanes 16..63 repeat lanes
        // 0..15 into the unused rest of the 1 KiB slot.
        if (wave_s == 0)
            dma16(ldg, a.S * 8, (BSATTN_LDS void*)ldb, (lane & 15) * 16, q0 * 8);
    };

    // Element masks: bit i of the result keeps register i's (query, key) pair of
    // the step (32 queries from 32 * rr of query block qb; the lane's key is
    // wave * 32 + l32 of key block kj, bit l32 of word `wave` of a tile row).
    auto keep_bits = [&](int qb, int rr) -> uint32_t {
        if constexpr (!ELEM) return 0xffffu;
        const size_t bi = ((size_t)bh * a.n_q + qb) * a.n_k + kj;
        if (a.states[bi] <= 1) return 0xffffu;
        int tile = a.pidx[bi];
        tile = tile < 0 ? 0 : (tile >= a.n_tiles ? a.n_tiles - 1 : tile);
        const int wpr = a.block_k >> 5;
        const uint32_t* row = a.pbits + ((size_t)tile * a.block_q + rr * 32 + 8 * h) * wpr + wave;
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) m |= ((row[(16 * (i >> 3) + (i & 7)) * wpr] >> l32) & 1u) << i;
        return m;
    };

    auto compute = [&](const uint8_t* qk, const uint8_t* qv, const uint8_t* ok, const uint8_t* ov,
                       const float2* ldb, uint32_t keep) {
        // S = Q K^T and dP = dO V^T: register i of lane (h, key) holds query
        // 16(i/8) + 8h + i%8 of the step.
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int kfo = RK ? KP::frag(0, ks) + kplan.rd_lane[ks & 3] : ks * 1024 + lane * 16;
            const bf16x8 qa = *(const bf16x8*)(qk + kfo);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ks], s, 0, 0, 0);
            const bf16x8 oa = *(const bf16x8*)(ok + kfo);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, vf[ks], dp, 0, 0, 0);
        }
        bf16x8 pb[2], db[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float4* lp = (const float4*)(ldb + 16 * e + 8 * h);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 x = lp[j];  // queries 2j, 2j+1 of the run: (lse2, delta) each
                const int i0 = 8 * e + 2 * j;
                float p0 = fast_exp2(__builtin_fmaf(s[i0], a.c, -x.x));
                float p1 = fast_exp2(__builtin_fmaf(s[i0 + 1], a.c, -x.z));
                if constexpr (ELEM) {
                    p0 = ((keep >> i0) & 1u) ? p0 : 0.f;
                    p1 = ((keep >> (i0 + 1)) & 1u) ? p1 : 0.f;
                }
                pb[e][2 * j] = (__bf16)p0;
                pb[e][2 * j + 1] = (__bf16)p1;
                db[e][2 * j] = (__bf16)(p0 * (dp[i0] - x.y));
                db[e][2 * j + 1] = (__bf16)(p1 * (dp[i0 + 1] - x.w));
            }
        }
        // dV^T += dO^T P and dK^T += Q^T dS (A by the transposing read).
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int md = 0; md < MD; ++md) {
                const int off = ((e * 2) * MD + md) * 512 + lane * 8;
                const bf16x4 o0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BSATTN_LDS bf16x4*)(ov + off));
                const bf16x4 o1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BSATTN_LDS bf16x4*)(ov + off + MD * 512));
                dva[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_shufflevector(o0, o1, 0, 1, 2, 3, 4, 5, 6, 7),
                                                                  pb[e], dva[md], 0, 0, 0);
                const bf16x4 q0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BSATTN_LDS bf16x4*)(qv + off));
                const bf16x4 q1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BSATTN_LDS bf16x4*)(qv + off + MD * 512));
                dka[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7),
                                                                  db[e], dka[md], 0, 0, 0);
            }
    };

    // Query block of the step being issued, and the next one prefetched.
    int blk_cur = 0, blk_pre = 0;
    auto q0_for = [&](int t) -> int {
        const int r = t & ((1 << spb_log2) - 1);
        if (t > 0 && r == 0) {
            blk_cur = blk_pre;
            blk_pre = entry((t >> spb_log2) + 1);
        }
        return blk_cur * a.block_q + r * 32;
    };
    auto step = [&](int t, const uint8_t* qk, const uint8_t* qv, const uint8_t* ok, const uint8_t* ov,
                    const float2* ldb, uint8_t* nqk, uint8_t* nqv, uint8_t* nok, uint8_t* nov, float2* nld) {
        __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this wave's DMA of step t
        __syncthreads();                     // everyone's DMA landed; step t-1 fully read
        const uint32_t keep = keep_bits(blk_cur, t & ((1 << spb_log2) - 1));  // (before q0_for moves on)
        if (t + 1 < n_steps) issue(q0_for(t + 1), nqk, nqv, nok, nov, nld);
        compute(qk, qv, ok, ov, ldb, keep);
    };

    if (n_steps > 0) {
        blk_cur = entry(0);
        blk_pre = entry(1);
        issue(q0_for(0), qk0, qv0, ok0, ov0, ld0);
        for (int t = 0; t < n_steps; t += 2) {
            step(t, qk0, qv0, ok0, ov0, ld0, qk1, qv1, ok1, ov1, ld1);
            if (t + 1 < n_steps) step(t + 1, qk1, qv1, ok1, ov1, ld1, qk0, qv0, ok0, ov0, ld0);
        }
    }

    // dK^T, dV^T: lane (h, key) holds d = 32md + 8g + 4h + u in register 4g + u.
    if (part_slot >= 0) {  // a piece of a cut key block: fp32 partials, dK unscaled
        float* base = a.scratch + (size_t)part_slot * 2 * a.block_k * D + (size_t)(wave * 32 + l32) * D;
#pragma unroll
        for (int md = 0; md < MD; ++md)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d0 = 32 * md + 8 * g4 + 4 * h;
                *(float4*)(base + d0) = make_float4(dka[md][4 * g4], dka[md][4 * g4 + 1], dka[md][4 * g4 + 2],
                                                    dka[md][4 * g4 + 3]);
                *(float4*)(base + (size_t)a.block_k * D + d0) =
                    make_float4(dva[md][4 * g4], dva[md][4 * g4 + 1], dva[md][4 * g4 + 2], dva[md][4 * g4 + 3]);
            }
        return;
    }
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const size_t idx = head + (size_t)key * D + 32 * md + 8 * g4 + 4 * h;
            float xk[4], xv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                xk[u] = dka[md][4 * g4 + u] * a.scale;
                xv[u] = dva[md][4 * g4 + u];
            }
            store4<D>(a.dk, idx, xk, OUT_F32);
            store4<D>(a.dv, idx, xv, OUT_F32);
        }
}

// dQ of one query block.  WAVES * 32 = block_q queries per workgroup.
template <int D, int WAVES, int OUT_F32, int ELEM>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, D == 64 ? 4 : 2))) void bwd_dq_kernel(
    BwdArgs a) {
    typedef TileGeom<D, 32> G;  // one 32-key tile of K or V
    typedef DmaPlan<D, WAVES, 32> P;
    typedef KRowPlan<D, WAVES, 32> KP;
    constexpr int KS = G::KS, MD = G::MD;
    __shared__ __attribute__((aligned(1024))) uint8_t kk0[G::BYTES], kv0[G::BYTES], vk0[G::BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t kk1[G::BYTES], kv1[G::BYTES], vk1[G::BYTES];

    const int r = bwd_slot(a, a.row_order, a.chunk_q, a.n_rows);
    if (r < 0) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
    const int wave_s = wave_uniform(wave);
    const int bh = r / a.n_q;
    const int qi = r - bh * a.n_q;
    int cnt = wave_uniform(a.row_counts[r]);
    cnt = cnt < 0 ? 0 : (cnt > a.n_k ? a.n_k : cnt);
    const int32_t* lst = a.row_lists + (size_t)r * a.n_k;
    const size_t head = (size_t)bh * a.S * D;
    const int q_row = qi * a.block_q + wave * 32 + l32;

    // B operands: lane (h, q) holds Q[q][16ks + 8h .. +7] and the same of dO.
    bf16x8 qf[KS], of[KS];
    {
        const u32x4* qp = (const u32x4*)(a.q + head + (size_t)q_row * D);
        const u32x4* op = (const u32x4*)(a.dout + head + (size_t)q_row * D);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qf[ks] = __builtin_bit_cast(bf16x8, qp[2 * ks + h]);
            of[ks] = __builtin_bit_cast(bf16x8, op[2 * ks + h]);
        }
    }
    const float2 myld = a.ld[(size_t)bh * a.S + q_row];

    f32x16 dqa[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md) dqa[md] = f32x16{};

    const int spb_log2 = a.ksteps_log2;  // 32-key steps per key block
    const int n_steps = cnt << spb_log2;
    auto entry = [&](int i) -> int {
        int kj = wave_uniform(lst[i < cnt ? i : cnt - 1]);
        return kj < 0 ? 0 : (kj >= a.n_k ? a.n_k - 1 : kj);
    };

    P plan;
    plan.init(lane);
    KP kplan;
    kplan.init(lane);
    const int nrec = a.S * D * 2;
    const int v_voff = plan.v_lane * 2;
    const uint16_t* kg = a.k + head;
    const uint16_t* vg = a.v + head;
    auto issue = [&](int k0, uint8_t* kk, uint8_t* kv, uint8_t* vk) {
#pragma unroll
        for (int i = 0; i < KP::NK; ++i) {
            const int soff = (k0 * D + KP::uniform(wave_s, i)) * 2, k_voff = kplan.dma_off(wave_s, i) * 2;
            dma16(kg, nrec, (BSATTN_LDS void*)(kk + (wave_s + i * WAVES) * 1024), k_voff, soff);
            dma16(vg, nrec, (BSATTN_LDS void*)(vk + (wave_s + i * WAVES) * 1024), k_voff, soff);
        }
#pragma unroll
        for (int i = 0; i < P::NV; ++i)
            dma16(kg, nrec, (BSATTN_LDS void*)(kv + (wave_s + i * WAVES) * 1024), v_voff,
                  (k0 * D + P::v_uniform(wave_s, i)) * 2);
    };

    // Element masks: this lane's tile-row word for the step's 32 keys (32 * rr of key
    // block kb), shifted so that bit 16(i/8) + i%8 keeps register i's key.
    auto keep_bits = [&](int kb, int rr) -> uint32_t {
        if constexpr (!ELEM) return 0xffffffffu;
        const size_t bi = (size_t)r * a.n_k + kb;
        if (a.states[bi] <= 1) return 0xffffffffu;
        int tile = a.pidx[bi];
        tile = tile < 0 ? 0 : (tile >= a.n_tiles ? a.n_tiles - 1 : tile);
        const int wpr = a.block_k >> 5;
        return a.pbits[((size_t)tile * a.block_q + wave * 32 + l32) * wpr + rr] >> (8 * h);
    };

    auto compute = [&](const uint8_t* kk, const uint8_t* kv, const uint8_t* vk, uint32_t keep) {
        // S^T = K Q^T, dP^T = V dO^T: register i of lane (h, q) holds key
        // 16(i/8) + 8h + i%8 of the step.
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 ka = *(const bf16x8*)(kk + KP::frag(0, ks) + kplan.rd_lane[ks & 3]);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s, 0, 0, 0);
            const bf16x8 va = *(const bf16x8*)(vk + KP::frag(0, ks) + kplan.rd_lane[ks & 3]);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, of[ks], dp, 0, 0, 0);
        }
        bf16x8 db[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float p = fast_exp2(__builtin_fmaf(s[i], a.c, -myld.x));
            if constexpr (ELEM) p = ((keep >> (16 * (i >> 3) + (i & 7))) & 1u) ? p : 0.f;
            db[i >> 3][i & 7] = (__bf16)(p * (dp[i] - myld.y));
        }
        // dQ^T += K^T dS^T (A by the transposing read of K).
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int md = 0; md < MD; ++md) {
                const int off = ((e * 2) * MD + md) * 512 + lane * 8;
                const bf16x4 k0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BSATTN_LDS bf16x4*)(kv + off));
                const bf16x4 k1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BSATTN_LDS bf16x4*)(kv + off + MD * 512));
                dqa[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_shufflevector(k0, k1, 0, 1, 2, 3, 4, 5, 6, 7),
                                                                  db[e], dqa[md], 0, 0, 0);
            }
    };

    int blk_cur = 0, blk_pre = 0;
    auto k0_for = [&](int t) -> int {
        const int rr = t & ((1 << spb_log2) - 1);
        if (t > 0 && rr == 0) {
            blk_cur = blk_pre;
            blk_pre = entry((t >> spb_log2) + 1);
        }
        return blk_cur * a.block_k + rr * 32;
    };
    auto step = [&](int t, const uint8_t* kk, const uint8_t* kv, const uint8_t* vk, uint8_t* nkk, uint8_t* nkv,
                    uint8_t* nvk) {
        __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0)
        __syncthreads();
        const uint32_t keep = keep_bits(blk_cur, t & ((1 << spb_log2) - 1));  // (before k0_for moves on)
        if (t + 1 < n_steps) issue(k0_for(t + 1), nkk, nkv, nvk);
        compute(kk, kv, vk, keep);
    };

    if (n_steps > 0) {
        blk_cur = entry(0);
        blk_pre = entry(1);
        issue(k0_for(0), kk0, kv0, vk0);
        for (int t = 0; t < n_steps; t += 2) {
            step(t, kk0, kv0, vk0, kk1, kv1, vk1);
            if (t + 1 < n_steps) step(t + 1, kk1, kv1, vk1, kk0, kv0, vk0);
        }
    }

#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const size_t idx = head + (size_t)q_row * D + 32 * md + 8 * g4 + 4 * h;
            float x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) x[u] = dqa[md][4 * g4 + u] * a.scale;
            store4<D>(a.dq, idx, x, OUT_F32);
        }
}

// kReduceParts workgroups per cut key block: dK = scale * sum of its pieces'
// partials and dV = sum of theirs, in piece order (deterministic).
constexpr int kReduceParts = 8;
template <int D, int OUT_F32>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdArgs a) {
    const int sp = blockIdx.x / kReduceParts, part = blockIdx.x % kReduceParts;
    if (sp >= wave_uniform(a.n_items[1]) || sp >= a.max_splits) return;
    const int4 s = a.splits[sp];
    const int col = s.x < 0 ? 0 : (s.x >= a.n_cols ? a.n_cols - 1 : s.x);
    const int slot0 = s.y < 0 ? 0 : (s.y >= a.max_slots ? a.max_slots - 1 : s.y);
    const int np = s.z < 0 ? 0 : (s.z > a.max_slots - slot0 ? a.max_slots - slot0 : s.z);
    const int bh = col / a.n_k, kj = col - bh * a.n_k;
    const size_t out0 = ((size_t)bh * a.S + (size_t)kj * a.block_k) * D;
    const int n4 = a.block_k * D / 4;  // float4 per block; kReduceParts workgroups share them
    for (int i = part * 256 + threadIdx.x; i < n4; i += 256 * kReduceParts) {
        float4 k4 = make_float4(0.f, 0.f, 0.f, 0.f), v4 = k4;
        for (int p = 0; p < np; ++p) {
            const float* base = a.scratch + (size_t)(slot0 + p) * 2 * a.block_k * D;
            const float4 x = ((const float4*)base)[i];
            const float4 y = ((const float4*)(base + (size_t)a.block_k * D))[i];
            k4.x += x.x; k4.y += x.y; k4.z += x.z; k4.w += x.w;
            v4.x += y.x; v4.y += y.y; v4.z += y.z; v4.w += y.w;
        }
        const float xk[4] = {k4.x * a.scale, k4.y * a.scale, k4.z * a.scale, k4.w * a.scale};
        const float xv[4] = {v4.x, v4.y, v4.z, v4.w};
        store4<D>(a.dk, out0 + 4 * (size_t)i, xk, OUT_F32);
        store4<D>(a.dv, out0 + 4 * (size_t)i, xv, OUT_F32);
    }
}

hipError_t launch_bwd_split(const int32_t* counts, int64_t C, int n_q, int max_slots, void* items, void* splits,
                            int32_t* n_out, hipStream_t stream) {
    hipLaunchKernelGGL(bwd_split_kernel, dim3(1), dim3(1024), 0, stream, counts, C, n_q, max_slots, (int4*)items,
                       (int4*)splits, n_out);
    return hipGetLastError();
}

hipError_t launch_bwd_prep(const void* out, const void* dout, const float* lse, void* ld, int64_t rows, int D,
                           hipStream_t stream) {
    const int rpb = 256 / (D / 8);
    const unsigned grid = (unsigned)((rows + rpb - 1) / rpb);
    if (D == 128)
        hipLaunchKernelGGL(bwd_prep_kernel<128>, dim3(grid), dim3(256), 0, stream, (const uint16_t*)out,
                           (const uint16_t*)dout, lse, (float2*)ld, rows);
    else
        hipLaunchKernelGGL(bwd_prep_kernel<64>, dim3(grid), dim3(256), 0, stream, (const uint16_t*)out,
                           (const uint16_t*)dout, lse, (float2*)ld, rows);
    return hipGetLastError();
}

hipError_t launch_bwd_cols(const uint8_t* mask, int64_t C, int n_q, int n_k, int32_t* counts, int32_t* lists,
                           hipStream_t stream) {
    const unsigned grid = (unsigned)((C + 3) / 4);
    hipLaunchKernelGGL(bwd_cols_kernel, dim3(grid), dim3(256), 0, stream, mask, C, n_q, n_k, counts, lists);
    return hipGetLastError();
}

template <int D, int OUT_F32, int ELEM>
static hipError_t launch_main(const BwdArgs& a, bool do_dq, bool do_dkdv, hipStream_t stream) {
    const dim3 gk(8 * a.chunk_k), gq(8 * a.chunk_q);
    if (do_dkdv) {
        if (a.block_k == 128)
            hipLaunchKernelGGL((bwd_dkdv_kernel<D, 4, OUT_F32, ELEM>), gk, dim3(256), 0, stream, a);
        else
            hipLaunchKernelGGL((bwd_dkdv_kernel<D, 2, OUT_F32, ELEM>), gk, dim3(128), 0, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (a.max_splits > 0) {
            hipLaunchKernelGGL((bwd_reduce_kernel<D, OUT_F32>), dim3(a.max_splits * kReduceParts), dim3(256), 0,
                               stream, a);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    if (!do_dq) return hipSuccess;
    if (a.block_q == 128)
        hipLaunchKernelGGL((bwd_dq_kernel<D, 4, OUT_F32, ELEM>), gq, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((bwd_dq_kernel<D, 2, OUT_F32, ELEM>), gq, dim3(128), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_bwd_main(const BwdArgs& a, int D, int out_f32, bool do_dq, bool do_dkdv, hipStream_t stream) {
    if (a.states) {  // element-level masks
        if (D == 128)
            return out_f32 ? launch_main<128, 1, 1>(a, do_dq, do_dkdv, stream)
                           : launch_main<128, 0, 1>(a, do_dq, do_dkdv, stream);
        return out_f32 ? launch_main<64, 1, 1>(a, do_dq, do_dkdv, stream)
                       : launch_main<64, 0, 1>(a, do_dq, do_dkdv, stream);
    }
    if (D == 128)
        return out_f32 ? launch_main<128, 1, 0>(a, do_dq, do_dkdv, stream)
                       : launch_main<128, 0, 0>(a, do_dq, do_dkdv, stream);
    return out_f32 ? launch_main<64, 1, 0>(a, do_dq, do_dkdv, stream) : launch_main<64, 0, 0>(a, do_dq, do_dkdv, stream);
}

}  // namespace bsattn
