// attn_bf16_pp.hip -- fused block-sparse flash-attention forward, bf16 in, fp32
// accumulation, bf16 out + fp32 lse, for gfx950: the two-group ("ping-pong")
// schedule.
//
// What is computed is the same operator as attn_bf16.hip: "Writing Pallas Kernels
// for JAX" (rajatpandit.com), section "Writing the Kernel Logic: Load, Compute,
// Store" (scaled Q K^T per tile, inactive blocks contribute nothing, softmax, P V),
// with the whole-row online softmax of "Pallas-Triton kernels and kernel
// auto-tuning" (robertdyro.com), section "Flash Attention".
//
// Work decomposition.  One workgroup of 8 waves owns the 128 query rows of one
// mask row.  Waves 0-3 (group 0) and 4-7 (group 1) cover the same rows, wave
// w and w+4 the same 32 rows, and split the row's 32-key tiles between them:
// group g takes tiles g, g+2, g+4, ...  Each group keeps its own running max,
// sum and O; at the end group 1 hands (m, l, O) to group 0 through LDS and group
// 0 folds the two into the output (the same rescale-and-add as one online-
// softmax step).
//
// Schedule.  A group's iteration on its tile i has four phases, each closed by a
// workgroup barrier:
//   A  S(i+1) = K(i+1) Q^T (8 MFMAs for D = 128) interleaved with the softmax of
//      S(i): P(i) = 2^(c S(i) - m) in bf16;
//   B  read V(i) from LDS into registers; DMA the K tile four tiles ahead;
//   C  O += V(i)^T P(i) (8 MFMAs) interleaved with the row sums of P(i) (in
//      fp32, before the bf16 rounding) and the row max of S(i+1);
//   D  move the reference max if S(i+1) exceeds it by more than 8 (rescale O, l);
//      read K(i+2) into registers; DMA the V tile three tiles ahead.
// Group 1 runs one phase behind group 0, so on every SIMD one wave is in a
// compute phase (A or C: matrix cores plus VALU) while the other is in a memory
// phase (B or D: LDS reads and DMA issue).  Each group keeps three K and three V
// tiles resident in LDS (distinct arrays, so the compiler can tell the DMA
// targets from the tiles being read); tile layouts are the operand-ordered ones
// of bf16_layout.h.  A tile past the end of the group's share is computed on a
// clamped (real, finite) tile and contributes nothing (its P is 2^-inf = 0), so
// the loop has no data-dependent branches and both groups run the same number
// of barriers.
#include <type_traits>

#include "bf16_layout.h"
#include "common.h"
#include "kernels.h"

namespace bsattn {

namespace {

// vmcnt(N) only (expcnt and lgkmcnt at their maxima: no wait on those).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x3f70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier between phases.  It orders LDS accesses only: this wave's
// LDS reads were consumed (so completed) before it; DMA still in flight is
// waited for explicitly with wait_vm where its data is needed.
__device__ __forceinline__ void phase_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Maximum over a lane's 16 scores of a 32x32 S^T tile.
__device__ __forceinline__ float row_max(const f32x16& s) {
    float t[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) t[u] = s[u];
    return max_tree3<16>(t);
}

}  // namespace

template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_bf16_pp_kernel(FwdArgs a) {
    typedef TileGeom<D, 32> G;
    typedef DmaPlan<D, 4, 32> P;  // the 4 waves of a group split each tile's DMA
    constexpr int KS = G::KS, MD = G::MD, T = G::BYTES;
    constexpr int NB = P::NK;     // DMA instructions per wave per K (or V) tile
    static_assert(P::NK == P::NV, "K and V tiles take the same DMA count");

    __shared__ __attribute__((aligned(1024))) uint8_t k00[T], k01[T], k02[T], v00[T], v01[T], v02[T];
    __shared__ __attribute__((aligned(1024))) uint8_t k10[T], k11[T], k12[T], v10[T], v11[T], v12[T];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;
    const int w4 = wave_uniform(wave & 3);

    int r, sub;
    block_work(a, r, sub);
    if (r < 0) return;
    const int bh = r / a.n_q;
    const int qi = r - bh * a.n_q;
    int beg, cnt;
    row_list(a, r, beg, cnt);
    const int sh = a.steps_log2;  // 32-key tiles per key block = 1 << sh
    const int n_tiles = cnt << sh;
    const int n_iter = (n_tiles + 1) >> 1;
    const int q_row = qi * a.block_q + sub * 128 + w4 * 32 + (lane & 31);
    const size_t head = (size_t)bh * a.S * D;
    const uint16_t* __restrict__ kg = (const uint16_t*)a.k + head;
    const uint16_t* __restrict__ vg = (const uint16_t*)a.v + head;
    const int nrec = a.S * D * 2;
    const float c = a.c;

    auto write_out = [&](const f32x16* o, float l_tot, float m) {
        const bool any = n_tiles > 0;
        const float inv = any ? 1.0f / l_tot : 0.0f;
        uint16_t* og = (uint16_t*)a.out + head + (size_t)q_row * D;
#pragma unroll
        for (int md = 0; md < MD; ++md)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d0 = 32 * md + 8 * g4 + 4 * h;
                bf16x4 ov;
#pragma unroll
                for (int u = 0; u < 4; ++u) ov[u] = (__bf16)(o[md][4 * g4 + u] * inv);
                *(bf16x4*)(og + d0) = ov;
            }
        if (h == 0) a.lse[(size_t)bh * a.S + q_row] = any ? (m + log2f(l_tot)) * kLn2 : -INFINITY;
    };

    if (n_tiles == 0) {
        if (wave < 4) {
            f32x16 z[MD];
#pragma unroll
            for (int md = 0; md < MD; ++md) z[md] = f32x16{};
            write_out(z, 0.f, 0.f);
        }
        return;
    }

    // Merge area (after the loop): wave w's O in arrays 2w and 2w+1 of this list,
    // m and l of all four waves in the ninth.
    auto merge_array = [&](int i) -> uint8_t* {
        switch (i) {
            case 0: return k10;
            case 1: return k11;
            case 2: return k12;
            case 3: return v10;
            case 4: return v11;
            case 5: return v12;
            case 6: return k00;
            case 7: return k01;
            default: return k02;
        }
    };

    auto body = [&](auto group) {
        constexpr int g = decltype(group)::value;
        uint8_t* const kslot[3] = {g ? k10 : k00, g ? k11 : k01, g ? k12 : k02};
        uint8_t* const vslot[3] = {g ? v10 : v00, g ? v11 : v01, g ? v12 : v02};

        // Q^T fragments: lane (h, q) holds Q[q][16ks + 8h .. +7].
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

        // Key-block list entries, 64 at a time in one VGPR (lane e holds entry
        // wbase + e), read back with readlane.  The DMA of K runs at most one key
        // block ahead of the DMA of V, so a window starting one block below the
        // block that overflowed covers both.
        int wbase = 0;
        int win = lane < cnt ? a.list[beg + lane] : 0;
        auto entry = [&](int b) -> int {
            if (b - wbase >= 64) {
                wbase = wave_uniform(b > 0 ? b - 1 : 0);
                win = lane + wbase < cnt ? a.list[beg + wbase + lane] : 0;
                wait_vm<0>();
            }
            int kj = __builtin_amdgcn_readlane(win, b - wbase);
            kj = kj < 0 ? 0 : (kj >= a.n_k ? a.n_k - 1 : kj);
            return kj;
        };
        // First key of this group's tile i (clamped to the group's last tile,
        // so every DMA reads real keys).
        const int my_tiles = (n_tiles - g + 1) >> 1;
        auto tile_key0 = [&](int i) -> int {
            const int ii = i < my_tiles ? i : (my_tiles > 0 ? my_tiles - 1 : 0);
            const int j = wave_uniform(2 * ii + g < n_tiles ? 2 * ii + g : n_tiles - 1);
            return entry(j >> sh) * a.block_k + (j & ((1 << sh) - 1)) * 32;
        };

        // The DMA is issued as inline assembly (dma16_raw): its completion is
        // waited for explicitly below, and the LDS reads of a tile are ordered
        // against the DMA that overwrites it by the phase barriers.
        P plan;
        plan.init(lane);
        const int k_voff = plan.k_lane * 2, v_voff = plan.v_lane * 2;
        const u32x4 krs = make_rsrc(kg, nrec), vrs = make_rsrc(vg, nrec);
        auto dma_k = [&](int i, uint8_t* buf) {
            const int key0 = tile_key0(i);
#pragma unroll
            for (int n = 0; n < P::NK; ++n)
                dma16_raw(krs, lds_addr(buf + (w4 + 4 * n) * 1024), k_voff,
                          wave_uniform((key0 * D + P::k_uniform(w4, n)) * 2));
        };
        auto dma_v = [&](int i, uint8_t* buf) {
            const int key0 = tile_key0(i);
#pragma unroll
            for (int n = 0; n < P::NV; ++n)
                dma16_raw(vrs, lds_addr(buf + (w4 + 4 * n) * 1024), v_voff,
                          wave_uniform((key0 * D + P::v_uniform(w4, n)) * 2));
        };

        bf16x8 kreg[KS];
        auto read_k = [&](const uint8_t* buf) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) kreg[ks] = *(const bf16x8*)(buf + ks * 1024 + lane * 16);
        };
        bf16x8 vreg[2][MD];
        auto read_v = [&](const uint8_t* buf) {
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int md = 0; md < MD; ++md) {
                    const uint8_t* vb = buf + (e * 2 * MD + md) * 512 + lane * 8;
                    const bf16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BSATTN_LDS bf16x4*)(vb));
                    const bf16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BSATTN_LDS bf16x4*)(vb + MD * 512));
                    vreg[e][md] = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
                }
        };
        auto qk = [&]() -> f32x16 {
            f32x16 s = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kreg[ks], qf[ks], s, 0, 0, 0);
            return s;
        };

        f32x16 oacc[MD];
#pragma unroll
        for (int md = 0; md < MD; ++md) oacc[md] = f32x16{};
        float m = -INFINITY;  // reference max (base 2, scaled), per query
        float l = 0.f;        // this lane's partial row sum
        float mx = -INFINITY; // scaled row max of the next tile (-inf if past the end)

        // Move the reference max when the next tile exceeds it by more than 8:
        // any reference at or below the true max gives the same exact result,
        // so most tiles skip the rescale.
        auto rescale = [&]() {
            if (__ballot(mx > m + 8.0f) != 0) {
                const float m_new = fmax_nan(m, mx);
                const float alpha = fast_exp2(m - m_new);
                l *= alpha;
#pragma unroll
                for (int md = 0; md < MD; ++md) oacc[md] *= alpha;
                m = m_new;
            }
        };

        // Prologue: three K and three V tiles in flight, S(0) and K(1).
        dma_k(0, kslot[0]);
        dma_k(1, kslot[1]);
        dma_k(2, kslot[2]);
        dma_v(0, vslot[0]);
        dma_v(1, vslot[1]);
        dma_v(2, vslot[2]);
        wait_vm<0>();
        phase_barrier();
        read_k(kslot[0]);
        f32x16 s_cur = qk();
        read_k(kslot[1]);
        mx = (g < n_tiles) ? max_halves_nan(row_max(s_cur)) * c : -INFINITY;
        rescale();
        phase_barrier();
        dma_k(3, kslot[0]);

        bf16x8 p[2];
        auto iter = [&](int i, auto slot) {
            constexpr int s0 = decltype(slot)::value;  // i % 3
            const bool cur_ok = 2 * i + g < n_tiles;
            const bool next_ok = 2 * (i + 1) + g < n_tiles;

            // Phase A: S(i+1) on the matrix cores, softmax of S(i) on the VALU.
            const f32x16 s_next = qk();
            const float negm = cur_ok ? -m : -INFINITY;
            f32x16 pe;  // P(i) in fp32: its row sums are taken from these
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    pe[8 * e + u] = fast_exp2(__builtin_fmaf(s_cur[8 * e + u], c, negm));
                    p[e][u] = (__bf16)pe[8 * e + u];
                }
#pragma unroll
            for (int n = 0; n < KS; ++n) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x400, 16 / KS, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 24 / KS, 0);
            }
            // Keep P(i) in this phase (the compiler would otherwise sink the
            // softmax next to its uses in phase C).
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                u32x4 pu = __builtin_bit_cast(u32x4, p[e]);
                asm volatile("" : "+v"(pu));
                p[e] = __builtin_bit_cast(bf16x8, pu);
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) asm volatile("" : "+v"(pe[u]));
            wait_vm<4 * NB>();  // V(i) landed (for i >= 3; earlier ones were waited for)
            phase_barrier();

            // Phase B: V(i) into registers, DMA of K(i+4) into the slot K(i+1) left.
            read_v(vslot[s0]);
            dma_k(i + 4, kslot[(s0 + 1) % 3]);
            phase_barrier();

            // Phase C: O += V(i)^T P(i); row sums of P(i); row max of S(i+1).
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int md = 0; md < MD; ++md)
                    oacc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vreg[e][md], p[e], oacc[md], 0, 0, 0);
            {
                float t[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) t[u] = pe[u];
                l += tree_sum<16>(t);
            }
            const float mxn = max_halves_nan(row_max(s_next)) * c;
            mx = next_ok ? mxn : -INFINITY;
#pragma unroll
            for (int n = 0; n < 2 * MD; ++n) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
            }
            if (i == 1)
                wait_vm<3 * NB>();  // K(3) was issued after the prologue's wait
            else
                wait_vm<4 * NB>();  // K(i+2) landed
            phase_barrier();

            // Phase D: lazy rescale, K(i+2) into registers, DMA of V(i+3) into the
            // slot V(i) left.
            rescale();
            read_k(kslot[(s0 + 2) % 3]);
            dma_v(i + 3, vslot[s0]);
            phase_barrier();
            s_cur = s_next;
        };

        if (g == 1) phase_barrier();  // group 1 runs one phase behind
        for (int i = 0; i < n_iter; i += 3) {
            iter(i, std::integral_constant<int, 0>{});
            if (i + 1 < n_iter) iter(i + 1, std::integral_constant<int, 1>{});
            if (i + 2 < n_iter) iter(i + 2, std::integral_constant<int, 2>{});
        }
        if (g == 0) phase_barrier();

        // Fold group 1's (m, l, O) into group 0's.  The DMA of clamped tiles
        // past the end may still be landing: wait before reusing the arrays.
        wait_vm<0>();
        phase_barrier();
        uint8_t* o0 = merge_array(2 * w4);
        uint8_t* o1 = merge_array(2 * w4 + 1);
        float* ml = (float*)merge_array(8) + w4 * 128;
        if constexpr (g == 1) {
#pragma unroll
            for (int md = 0; md < MD; ++md) {
                uint8_t* base = (md < MD / 2 ? o0 : o1) + (md % (MD / 2)) * 4096;
#pragma unroll
                for (int k4 = 0; k4 < 4; ++k4) {
                    const f32x4 v4 = {oacc[md][4 * k4], oacc[md][4 * k4 + 1], oacc[md][4 * k4 + 2], oacc[md][4 * k4 + 3]};
                    *(f32x4*)(base + (k4 * 64 + lane) * 16) = v4;
                }
            }
            ml[lane] = m;
            ml[64 + lane] = l;
            phase_barrier();
        } else {
            phase_barrier();
            const float m1 = ml[lane];
            const float l1 = ml[64 + lane];
            const float mm = fmax_nan(m, m1);
            const float a0 = fast_exp2(m - mm);
            const float a1 = fast_exp2(m1 - mm);
#pragma unroll
            for (int md = 0; md < MD; ++md) {
                const uint8_t* base = (md < MD / 2 ? o0 : o1) + (md % (MD / 2)) * 4096;
#pragma unroll
                for (int k4 = 0; k4 < 4; ++k4) {
                    const f32x4 v4 = *(const f32x4*)(base + (k4 * 64 + lane) * 16);
#pragma unroll
                    for (int u = 0; u < 4; ++u) oacc[md][4 * k4 + u] = oacc[md][4 * k4 + u] * a0 + v4[u] * a1;
                }
            }
            const float lt = sum_halves(l * a0 + l1 * a1);
            write_out(oacc, lt, mm);
        }
    };

    if (wave < 4)
        body(std::integral_constant<int, 0>{});
    else
        body(std::integral_constant<int, 1>{});
}

template <int D>
hipError_t launch_bf16_pp(const FwdArgs& a, unsigned grid, hipStream_t stream) {
    hipLaunchKernelGGL((attn_bf16_pp_kernel<D>), dim3(grid), dim3(512), 0, stream, a);
    return hipGetLastError();
}

template hipError_t launch_bf16_pp<64>(const FwdArgs&, unsigned, hipStream_t);
template hipError_t launch_bf16_pp<128>(const FwdArgs&, unsigned, hipStream_t);

}  // namespace bsattn
