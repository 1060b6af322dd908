// ragged_dot.hip -- ragged dot (grouped matrix multiplication) for gfx950.
//
// What is computed: "Pallas-Triton kernels and kernel auto-tuning" (robertdyro.com),
// section "Ragged Dot (Group Matrix Multiplication)": rhs is a stack of G expert
// matrices [G][K][N]; the rows of lhs [M][K] are assigned to the experts in order,
// group g taking the next group_sizes[g] rows, and output row i is lhs row i times
// its group's matrix.  Rows past the sum of the sizes belong to no group and are
// written as 0.  bf16 in, fp32 accumulation, bf16 or fp32 out.
//
// Plan (ragged_plan_kernel, one workgroup): the groups' row ranges (a scan of the
// sizes, clamped into [0, M]) and the work items: one item per (256-row tile, group)
// pair that share rows, in group order, each with the row range [lo, hi) it owns
// (the compaction idea of the attention path: a tile visits only the groups that
// touch it), then items with group -1 for the rows past the last group, which are
// only zeroed.  A tile that straddles a boundary is visited once per owner and each
// visit stores only its own rows, so no two items write the same row.
//
// Kernels.  ragged_dot256_kernel (N % 256 == 0): one workgroup of 8 waves per
// (item, 256-column tile), a 256 x 256 output tile, waves in a 4 (columns) x 2
// (rows) grid, each 64 columns x 128 rows (each transposing LDS read of W feeds
// four MFMAs).  C^T[n][m] = sum_k W^T[n][k] X^T[k][m] on
// v_mfma_f32_32x32x16_bf16 with both operands from LDS: the expert tile
// W[g][k0..k0+63][n0..n0+255] in the transposed-read layout of bf16_layout.h (the V
// layout, row stride N; A by ds_read_b64_tr_b16) and the lhs rows X[m0..m0+255]
// [k0..k0+63] in 8-row x 128-byte swizzled chunks (B by ds_read_b128), both by
// buffer loads with the LDS flag, two stages (one step of loads in flight).  Per k a
// workgroup moves half the L2 -> LDS bytes per MFMA of the 128 x 128 tile.
// ragged_dot_kernel (any N % 128 == 0): 4 waves per (half item,
// 128-column tile), wave w owns 32 rows, the expert tile in LDS as above (three
// stages) and the wave's own lhs rows loaded straight into VGPRs, two steps ahead
// (in tail mode, below, the lhs rows go through LDS as well).
// The last round.  The 256 x 256 kernel takes the whole rounds of the chip (the
// largest multiple of the CU count of its (item, column tile) units); the rest, a
// partial round that would leave most CUs idle, goes to ragged_dot_kernel in tail
// mode as quarter tiles (two row halves x two 128-column halves of each unit), four
// times as many workgroups, so the last round spreads over all CUs.  Both kernels
// accumulate k in the same order, so the split changes no result.
#include "bf16_layout.h"
#include "common.h"
#include "kernels.h"

namespace bsattn {

constexpr int kRaggedTM = 256;     // rows per work item (tile)
constexpr int kRaggedTN = 128;     // columns per tile
constexpr int kRaggedTK = 64;      // k per step
constexpr int kRaggedThreads = 1024;

// Inclusive scan over the 1024 threads of the plan workgroup (wave scans, then a
// scan of the wave totals).
__device__ __forceinline__ int64_t block_scan(int64_t x, int64_t* wave_tot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int64_t y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) wave_tot[wave] = x;
    __syncthreads();
    if (wave == 0) {
        int64_t t = lane < kRaggedThreads / 64 ? wave_tot[lane] : 0;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int64_t y = __shfl_up(t, off, 64);
            if (lane >= off) t += y;
        }
        if (lane < kRaggedThreads / 64) wave_tot[lane] = t;
    }
    __syncthreads();
    const int64_t r = x + (wave > 0 ? wave_tot[wave - 1] : 0);
    __syncthreads();
    return r;
}

// items[i] = {row tile, group, lo, hi}; *n_items = their number.
__global__ __launch_bounds__(kRaggedThreads) void ragged_plan_kernel(const int32_t* __restrict__ group_sizes,
                                                                     int G, int M, int4* __restrict__ items,
                                                                     int32_t* __restrict__ n_items) {
    __shared__ int64_t wave_tot[kRaggedThreads / 64];
    __shared__ int64_t carry[2];  // rows, items before this chunk
    const int tid = threadIdx.x;
    if (tid == 0) carry[0] = carry[1] = 0;
    __syncthreads();
    for (int g0 = 0; g0 < G; g0 += kRaggedThreads) {
        const int g = g0 + tid;
        const int64_t sz = g < G ? (group_sizes[g] > 0 ? group_sizes[g] : 0) : 0;
        const int64_t rows_incl = block_scan(sz, wave_tot);
        const int64_t r0 = carry[0];
        int64_t start = r0 + rows_incl - sz, end = r0 + rows_incl;
        start = start < M ? start : M;
        end = end < M ? end : M;
        const int64_t cnt = end > start ? (end - 1) / kRaggedTM - start / kRaggedTM + 1 : 0;
        const int64_t items_incl = block_scan(cnt, wave_tot);
        const int64_t pos = carry[1] + items_incl - cnt;
        for (int64_t i = 0; i < cnt; ++i) {
            const int64_t t = start / kRaggedTM + i;
            const int64_t lo = start > t * kRaggedTM ? start : t * kRaggedTM;
            const int64_t hi = end < (t + 1) * kRaggedTM ? end : (t + 1) * kRaggedTM;
            items[pos + i] = make_int4((int)t, g, (int)lo, (int)hi);
        }
        __syncthreads();
        if (tid == kRaggedThreads - 1) {
            carry[0] = r0 + rows_incl;
            carry[1] = carry[1] + items_incl;
        }
        __syncthreads();
    }
    // rows [total, M) of no group: zero-fill items
    const int64_t total = carry[0] < M ? carry[0] : M;
    const int64_t t0 = total / kRaggedTM;
    const int64_t n_tail = total < M ? (M - 1) / kRaggedTM - t0 + 1 : 0;
    for (int64_t i = tid; i < n_tail; i += kRaggedThreads) {
        const int64_t t = t0 + i;
        const int64_t lo = total > t * kRaggedTM ? total : t * kRaggedTM;
        const int64_t hi = M < (t + 1) * kRaggedTM ? M : (t + 1) * kRaggedTM;
        items[carry[1] + i] = make_int4((int)t, -1, (int)lo, (int)hi);
    }
    if (tid == 0) n_items[0] = (int32_t)(carry[1] + n_tail);
}

// TAIL = 1: tail mode (N % 256 == 0, M * K * 2 < 2^31), the units past the whole
// rounds of tail_cu CUs, four workgroups per unit, the lhs rows DMA'd into LDS as
// 8-row x 128-byte chunks (whole lines; the 256 x 256 kernel's layout) instead of
// per-lane loads of 32 rows x 32 bytes (a quarter of the L2 rate), which left the
// tail's lone workgroups waiting on their loads.  TAIL = 0: every (half item, column
// tile), lhs rows straight into VGPRs.
template <int OUT_F32, int TAIL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void ragged_dot_kernel(
    const uint16_t* __restrict__ lhs, const uint16_t* __restrict__ rhs, const int4* __restrict__ items,
    const int32_t* __restrict__ n_items, void* __restrict__ out, int M, int K, int N, int max_items,
    int tail_cu) {
    typedef TileGeom<kRaggedTN, kRaggedTK> G;  // W^T tile: "D" = 128 columns, "keys" = 64 k
    constexpr int KS = kRaggedTK / 16, MT = G::MT, MD = G::MD;
    // Three stages of the expert tile (and in tail mode of the lhs rows) in LDS, and
    // otherwise three register sets of the wave's lhs rows: the loads run two steps
    // ahead.
    constexpr int XB = TAIL ? 128 * kRaggedTK * 2 : 16;  // lhs stage: 128 rows x 64 k
    __shared__ __attribute__((aligned(1024))) uint8_t w0s[G::BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t w1s[G::BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t w2s[G::BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t x0s[XB];
    __shared__ __attribute__((aligned(1024))) uint8_t x1s[XB];
    __shared__ __attribute__((aligned(1024))) uint8_t x2s[XB];

    int n_it = wave_uniform(n_items[0]);
    n_it = n_it < max_items ? n_it : max_items;  // (a plan never holds more)
    int item, half, nt;
    if constexpr (TAIL) {
        const int units = N / 256, total = n_it * units;
        const int gi = total - total % tail_cu + (int)(blockIdx.x >> 2);
        if (gi >= total) return;
        item = gi / units;
        half = (blockIdx.x >> 1) & 1;
        nt = 2 * (gi - item * units) + (blockIdx.x & 1);
    } else {
        const int n_tiles = N / kRaggedTN;
        item = blockIdx.x / (2 * n_tiles);
        const int rem = blockIdx.x - item * 2 * n_tiles;
        half = rem / n_tiles;
        nt = rem - half * n_tiles;
        if (item >= n_it) return;
    }
    const int4 it = items[item];
    const int grp = wave_uniform(it.y);
    const int row0 = wave_uniform(it.x) * kRaggedTM + half * 128;  // this workgroup's 128 rows
    int lo = wave_uniform(it.z), hi = wave_uniform(it.w);
    lo = lo > row0 ? lo : row0;
    hi = hi < row0 + 128 ? hi : row0 + 128;
    if (lo >= hi) return;  // the item has no rows in this half
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
    const int wave_s = wave_uniform(wave);
    const int n0 = nt * kRaggedTN;
    if (grp < 0) {  // rows of no group: zeros
        for (int r = lo + (tid >> 5); r < hi; r += 256 / 32) {
            const int c = n0 + 4 * (tid & 31);
            if constexpr (OUT_F32)
                *(float4*)((float*)out + (size_t)r * N + c) = make_float4(0.f, 0.f, 0.f, 0.f);
            else
                *(uint2*)((uint16_t*)out + (size_t)r * N + c) = make_uint2(0u, 0u);
        }
        return;
    }

    // this lane's lhs row (rows outside [lo, hi) are computed on a valid row and
    // never stored)
    int m = row0 + 32 * wave + l32;
    const bool store = m >= lo && m < hi;
    m = m < M ? m : M - 1;
    const u32x4* xrow = (const u32x4*)(lhs + (size_t)m * K);
    // Tail mode: chunk c = wave + 4 i of a stage holds rows 8c .. 8c + 7 of the 128; lane
    // l fills slot l % 8 of row 8c + l / 8 with unit (l % 8) ^ y(row), y(row) = (row / 2)
    // % 8, so one DMA instruction reads 8 rows x 128 contiguous bytes and the operand
    // reads (16 lanes, 16 consecutive rows, one unit) meet 16 distinct bank groups.
    int x_voff[4] = {0, 0, 0, 0}, x_rd[KS];
    if constexpr (TAIL) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 8 * (wave_s + 4 * i) + lane / 8;
            int xr = row0 + r;
            xr = xr < M ? xr : M - 1;
            x_voff[i] = (xr * K + 8 * ((lane % 8) ^ ((r / 2) % 8))) * 2;
        }
        const int rho = 32 * wave + l32, y = (rho / 2) % 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) x_rd[ks] = (rho / 8) * 1024 + (rho % 8) * 128 + 16 * ((2 * ks + h) ^ y);
    }
    const int xrec = TAIL ? M * K * 2 : 0;  // (tail mode only: the launcher checks it fits)

    // W tile DMA: the V layout of bf16_layout.h with row stride N.  Lane offsets as
    // DmaPlan<128, 4, 64>::init with D replaced by N for the row part.
    const int u = 2 * (lane & 31);
    const int L = u & 15, gg = (u >> 4) & 1, hh = u >> 5;
    const int v_lane = (8 * hh + (L >> 2)) * N + 32 * (lane >> 5) + 16 * gg + 4 * (L & 3);
    constexpr int NV = G::VBLK / 2 / 4;  // DMA instructions per wave per tile
    const uint16_t* wg = rhs + (size_t)grp * K * N + n0;
    const int nrec = (int)((size_t)K * N * 2 - (size_t)n0 * 2);  // bytes from wg to the expert's end
    auto issue = [&](int k0, uint8_t* wbuf, uint8_t* xbuf) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int tb = 2 * (wave_s + i * 4);
            const int md = tb % MD, r = (tb / MD) % 2, e = (tb / MD / 2) % 2, mt = tb / MD / 4;
            const int uni = (k0 + 32 * mt + 16 * e + 4 * r) * N + 32 * md;
            dma16(wg, nrec, (BSATTN_LDS void*)(wbuf + (wave_s + i * 4) * 1024), v_lane * 2, uni * 2);
        }
        if constexpr (TAIL) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dma16(lhs, xrec, (BSATTN_LDS void*)(xbuf + (wave_s + 4 * i) * 1024), x_voff[i], k0 * 2);
        }
    };

    f32x16 acc[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md) acc[md] = f32x16{};
    bf16x8 x0[KS], x1[KS], x2[KS];  // (register-path lhs sets; unused in tail mode)
    auto load_x = [&](int k0, bf16x8 (&dst)[KS]) {
        if constexpr (!TAIL) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) dst[ks] = __builtin_bit_cast(bf16x8, xrow[(k0 + 16 * ks) / 8 + h]);
        }
    };
    auto step = [&](const uint8_t* wbuf, const uint8_t* xbuf, const bf16x8 (&xr)[KS]) {
        bf16x8 xf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if constexpr (TAIL)
                xf[ks] = *(const bf16x8*)(xbuf + x_rd[ks]);
            else
                xf[ks] = xr[ks];
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int md = 0; md < MD; ++md) {
                    const uint8_t* vb = wbuf + (((mt * 2 + e) * 2) * MD + md) * 512 + lane * 8;
                    const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BSATTN_LDS bf16x4*)(vb));
                    const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BSATTN_LDS bf16x4*)(vb + MD * 512));
                    const bf16x8 wf = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
                    acc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, xf[mt * 2 + e], acc[md], 0, 0, 0);
                }
    };

    // Step s uses stage s % 3.  At its top: wait until this wave's loads of step s have
    // landed (each step's loads are NV + KS vector-memory operations -- in tail mode KS
    // lhs DMAs, else KS lhs loads -- in issue order, and those of step s + 1 may stay in
    // flight), barrier (everyone's DMA landed; everyone is done with step s - 1, whose
    // stage the next issue refills), then issue the loads of step s + 2.
    constexpr int PER_STEP = NV + KS;
    static_assert(PER_STEP < 64, "vmcnt range");
    static_assert(!TAIL || KS == 4, "tail mode: four lhs DMAs per wave per stage");
    const int n_steps = K / kRaggedTK;
    issue(0, w0s, x0s);
    load_x(0, x0);
    if (n_steps > 1) {
        issue(kRaggedTK, w1s, x1s);
        load_x(kRaggedTK, x1);
    }
    auto top = [&](int s) {
        if (s + 1 < n_steps)
            __builtin_amdgcn_s_waitcnt(0x3f70 | (PER_STEP & 15) | ((PER_STEP >> 4) << 14));
        else
            __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0)
        __syncthreads();
    };
    for (int t = 0; t < n_steps; t += 3) {
        top(t);
        if (t + 2 < n_steps) {
            issue((t + 2) * kRaggedTK, w2s, x2s);
            load_x((t + 2) * kRaggedTK, x2);
        }
        step(w0s, x0s, x0);
        if (t + 1 >= n_steps) break;
        top(t + 1);
        if (t + 3 < n_steps) {
            issue((t + 3) * kRaggedTK, w0s, x0s);
            load_x((t + 3) * kRaggedTK, x0);
        }
        step(w1s, x1s, x1);
        if (t + 2 >= n_steps) break;
        top(t + 2);
        if (t + 4 < n_steps) {
            issue((t + 4) * kRaggedTK, w1s, x1s);
            load_x((t + 4) * kRaggedTK, x1);
        }
        step(w2s, x2s, x2);
    }

    // C^T[n][m]: lane (h, m) holds n = 32 md + 8 g4 + 4 h + u for u = 0..3
    if (!store) return;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int n = n0 + 32 * md + 8 * g4 + 4 * h;
            if constexpr (OUT_F32) {
                float4 o;
                o.x = acc[md][4 * g4 + 0];
                o.y = acc[md][4 * g4 + 1];
                o.z = acc[md][4 * g4 + 2];
                o.w = acc[md][4 * g4 + 3];
                *(float4*)((float*)out + (size_t)m * N + n) = o;
            } else {
                bf16x4 o;
#pragma unroll
                for (int uu = 0; uu < 4; ++uu) o[uu] = (__bf16)acc[md][4 * g4 + uu];
                *(bf16x4*)((uint16_t*)out + (size_t)m * N + n) = o;
            }
        }
}

// The 256 x 256 kernel walks K in steps of TKS with NST LDS stages of W (TKS x 256)
// and X (256 x TKS) each, NST - 1 steps of loads in flight.  64-deep steps in two
// stages (128 KiB) ran 1.5 % faster on the 8-expert workload than 32-deep steps in
// four stages, and clearly faster than 32-deep steps in two or three.
constexpr int kR256TK = 64;
constexpr int kR256Stages = 2;

template <int OUT_F32, int TKS, int NST>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void ragged_dot256_kernel(
    const uint16_t* __restrict__ lhs, const uint16_t* __restrict__ rhs, const int4* __restrict__ items,
    const int32_t* __restrict__ n_items, void* __restrict__ out, int M, int K, int N, int max_items,
    int tail_cu) {
    typedef TileGeom<256, TKS> GW;      // W^T tile: "D" = 256 columns, "keys" = TKS k
    constexpr int MDW = GW::MD;         // 8 column tiles of 32
    constexpr int KSX = TKS / 16;       // k-steps of 16 per step
    constexpr int WB = GW::BYTES;       // W bytes per stage, then as many of X
    constexpr int NDW = TKS / 16;       // W (and X) DMA instructions per wave per stage
    static_assert(GW::VBLK / 2 == 8 * NDW, "W DMA split over the 8 waves");
    static_assert(NST >= 2 && NST * 2 * WB <= 160 * 1024, "LDS stages");
    // X chunk layout: a 1 KiB chunk holds XR rows x TKS k (XU 16-byte units per
    // row), row r%XR at (r%XR) * 2 TKS and unit u at slot u ^ y(r), y(r) =
    // (r / XP) % XU with XP rows per 256-byte bank period: 16 lanes reading 16
    // consecutive rows at one unit meet 16 distinct 16-byte bank groups.
    constexpr int XU = TKS / 8, XR = 1024 / (2 * TKS), XP = 256 / (2 * TKS);
    static_assert(256 / XR == 8 * NDW, "X DMA split over the 8 waves");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[NST * 2 * WB];

    // Workgroups go to the 8 XCDs round-robin by blockIdx.  XCD x = b % 8 takes the
    // (b / 8)-th (item, column tile) of its own contiguous chunk of the item-major
    // sequence: the column tiles of an item (the same lhs rows) and the neighbouring
    // items of a group (the same expert tiles) then meet in one L2.
    const int n_tiles = N / 256;
    int n_it = wave_uniform(n_items[0]);
    n_it = n_it < max_items ? n_it : max_items;  // (a plan never holds more)
    const int total = n_it * n_tiles;
    // whole rounds of tail_cu CUs here; the rest goes to the tail kernel
    const int whole = tail_cu > 0 ? total - total % tail_cu : total;
    const int chunk = (whole + 7) >> 3;
    const int jx = blockIdx.x >> 3;
    const int gi = (blockIdx.x & 7) * chunk + jx;
    if (jx >= chunk || gi >= whole) return;
    const int item = gi / n_tiles;
    const int nt = gi - item * n_tiles;
    const int4 it = items[item];
    const int tile = wave_uniform(it.x), grp = wave_uniform(it.y);
    const int lo = wave_uniform(it.z), hi = wave_uniform(it.w);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
    const int wave_s = wave_uniform(wave);
    const int n0 = nt * 256, m0 = tile * kRaggedTM;
    if (grp < 0) {  // rows of no group: zeros
        for (int r = lo + (tid >> 6); r < hi; r += 8) {
            const int c = n0 + 4 * (tid & 63);
            if constexpr (OUT_F32)
                *(float4*)((float*)out + (size_t)r * N + c) = make_float4(0.f, 0.f, 0.f, 0.f);
            else
                *(uint2*)((uint16_t*)out + (size_t)r * N + c) = make_uint2(0u, 0u);
        }
        return;
    }
    const int wn = wave & 3, wm = wave >> 2;  // columns 64 wn .., rows 128 wm ..

    // W tile DMA (V layout, row stride N): wave w fills block pairs 2(w + 8 i);
    // lane offsets as the attention kernel's V plan with N for the row.
    const int u = 2 * (lane & 31);
    const int L = u & 15, gg = (u >> 4) & 1, hh = u >> 5;
    const int w_lane = (8 * hh + (L >> 2)) * N + 32 * (lane >> 5) + 16 * gg + 4 * (L & 3);
    const uint16_t* wg = rhs + (size_t)grp * K * N + n0;
    const int wrec = (int)((size_t)K * N * 2 - (size_t)n0 * 2);
    int w_uni[NDW], x_lane[NDW];
#pragma unroll
    for (int i = 0; i < NDW; ++i) {
        const int tb = 2 * (wave_s + 8 * i);
        w_uni[i] = (32 * (tb / MDW / 4) + 16 * ((tb / MDW / 2) % 2) + 4 * ((tb / MDW) % 2)) * N + 32 * (tb % MDW);
        // X tile DMA: chunk c = w + 8 i holds rows m0 + XR c ..; lane l fills slot
        // l % XU of row l / XU, i.e. unit (l % XU) ^ y(row): one instruction reads
        // XR rows x 2 TKS contiguous bytes (whole 128-byte lines at TKS = 64; the
        // 32 rows x 32 bytes of an operand-ordered block run at a quarter of that
        // rate from L2).  Rows past M read row M - 1 (never stored).
        const int c = wave_s + 8 * i;
        const int r = XR * c + lane / XU;
        int xrow = m0 + r;
        xrow = xrow < M ? xrow : M - 1;
        x_lane[i] = (xrow * K + 8 * ((lane % XU) ^ ((r / XP) % XU))) * 2;
    }
    // Read side: lane (h, c) takes X[32 T + kperm(c)][k0 + 16 ks + 8 h ..] (the B
    // operand of 32-row tile T, k-step ks) at T * 32 * 2 TKS + x_rd[ks].
    int x_rd[KSX];
    {
        const int rho = kperm(l32), y = (rho / XP) % XU;
#pragma unroll
        for (int ks = 0; ks < KSX; ++ks)
            x_rd[ks] = (rho / XR) * 1024 + (rho % XR) * 2 * TKS + 16 * ((2 * ks + h) ^ y);
    }
    const int xrec = M * K * 2;  // < 2^31: the launcher checks it
    // Inline-assembly DMA (dma16_raw): with the stage picked at run time the
    // builtin would make the compiler wait for in-flight stages before every LDS
    // read; the explicit vmcnt waits and barriers below order it instead.
    const u32x4 wsrc = make_rsrc(wg, wrec), xsrc = make_rsrc(lhs, xrec);
    auto issue = [&](int t) {
        uint8_t* wbuf = lds + (t % NST) * 2 * WB;
#pragma unroll
        for (int i = 0; i < NDW; ++i) {
            dma16_raw(wsrc, lds_addr(wbuf + (wave_s + 8 * i) * 1024), w_lane * 2, (t * TKS * N + w_uni[i]) * 2);
            dma16_raw(xsrc, lds_addr(wbuf + WB + (wave_s + 8 * i) * 1024), x_lane[i], t * TKS * 2);
        }
    };

    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    auto step = [&](const uint8_t* wbuf, const uint8_t* xbuf) {
#pragma unroll
        for (int ks = 0; ks < KSX; ++ks) {
            bf16x8 xf[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) xf[j] = *(const bf16x8*)(xbuf + (4 * wm + j) * 64 * TKS + x_rd[ks]);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int md = 2 * wn + i;
                const uint8_t* vb = wbuf + ((ks * 2) * MDW + md) * 512 + lane * 8;
                const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BSATTN_LDS bf16x4*)(vb));
                const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BSATTN_LDS bf16x4*)(vb + MDW * 512));
                const bf16x8 wf = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, xf[j], acc[i][j], 0, 0, 0);
            }
        }
    };

    // Stages 0..NST-2 in flight before the loop; step t waits until only the
    // later stages' DMAs (2 NDW instructions each) are outstanding, syncs, issues
    // stage t + NST - 1 into the buffer step t - 1 used, and computes.
    const int n_steps = K / TKS;
    for (int t = 0; t < NST - 1 && t < n_steps; ++t) issue(t);
    for (int t = 0; t < n_steps; ++t) {
        int ahead = n_steps - 1 - t;
        ahead = ahead < NST - 2 ? ahead : NST - 2;
        if constexpr (NST >= 4) {
            if (ahead >= 2)
                __builtin_amdgcn_s_waitcnt(0x3f70 | (4 * NDW));  // vmcnt(2 stages)
            else if (ahead == 1)
                __builtin_amdgcn_s_waitcnt(0x3f70 | (2 * NDW));  // vmcnt(1 stage)
            else
                __builtin_amdgcn_s_waitcnt(0x3f70);              // vmcnt(0)
        } else if constexpr (NST == 3) {
            if (ahead >= 1)
                __builtin_amdgcn_s_waitcnt(0x3f70 | (2 * NDW));
            else
                __builtin_amdgcn_s_waitcnt(0x3f70);
        } else {
            __builtin_amdgcn_s_waitcnt(0x3f70);
        }
        __syncthreads();
        if (t + NST - 1 < n_steps) issue(t + NST - 1);
        const uint8_t* wbuf = lds + (t % NST) * 2 * WB;
        step(wbuf, wbuf + WB);
    }

    // C^T tile (i, j): lane (h, c) holds row m = m0 + 128 wm + 32 j + kperm(c) and
    // columns n = n0 + 64 wn + 32 i + 8 g4 + 4 h + u in register 4 g4 + u.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int m = m0 + 128 * wm + 32 * j + kperm(l32);
        if (m < lo || m >= hi) continue;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int n = n0 + 64 * wn + 32 * i + 8 * g4 + 4 * h;
                if constexpr (OUT_F32) {
                    *(float4*)((float*)out + (size_t)m * N + n) =
                        make_float4(acc[i][j][4 * g4], acc[i][j][4 * g4 + 1], acc[i][j][4 * g4 + 2], acc[i][j][4 * g4 + 3]);
                } else {
                    bf16x4 o;
#pragma unroll
                    for (int uu = 0; uu < 4; ++uu) o[uu] = (__bf16)acc[i][j][4 * g4 + uu];
                    *(bf16x4*)((uint16_t*)out + (size_t)m * N + n) = o;
                }
            }
    }
}

hipError_t launch_ragged_plan(const int32_t* group_sizes, int M, int G, void* workspace, hipStream_t stream) {
    int4* items = (int4*)workspace;
    int32_t* n_items = (int32_t*)(items + ragged_max_items(M, G));
    hipLaunchKernelGGL(ragged_plan_kernel, dim3(1), dim3(kRaggedThreads), 0, stream, group_sizes, G, M, items,
                       n_items);
    return hipGetLastError();
}

hipError_t launch_ragged_planned(const void* lhs, const void* rhs, void* out, int M, int K, int N, int G,
                                 int out_f32, const void* workspace, int n_cu, hipStream_t stream) {
    const int4* items = (const int4*)workspace;
    const int64_t max_items = ragged_max_items(M, G);
    const int32_t* n_items = (const int32_t*)(items + max_items);
    const uint16_t* x = (const uint16_t*)lhs;
    const uint16_t* w = (const uint16_t*)rhs;
    if (N % 256 == 0 && (int64_t)M * K * 2 < ((int64_t)1 << 31)) {  // lhs through one buffer range
        const int64_t units = max_items * (N / 256);
        const int64_t grid = 8 * ((units + 7) / 8);  // 8 XCD chunks
        const int tail_cu = n_cu > 0 ? n_cu : 0;
        if (out_f32)
            hipLaunchKernelGGL((ragged_dot256_kernel<1, kR256TK, kR256Stages>), dim3((unsigned)grid), dim3(512), 0,
                               stream, x, w, items, n_items, out, M, K, N, (int)max_items, tail_cu);
        else
            hipLaunchKernelGGL((ragged_dot256_kernel<0, kR256TK, kR256Stages>), dim3((unsigned)grid), dim3(512), 0,
                               stream, x, w, items, n_items, out, M, K, N, (int)max_items, tail_cu);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || tail_cu == 0) return e;
        // the partial last round: fewer than n_cu units, four workgroups each
        const int64_t tail_grid = 4 * (units < n_cu - 1 ? units : n_cu - 1);
        if (tail_grid == 0) return hipSuccess;
        if (out_f32)
            hipLaunchKernelGGL((ragged_dot_kernel<1, 1>), dim3((unsigned)tail_grid), dim3(256), 0, stream, x, w,
                               items, n_items, out, M, K, N, (int)max_items, tail_cu);
        else
            hipLaunchKernelGGL((ragged_dot_kernel<0, 1>), dim3((unsigned)tail_grid), dim3(256), 0, stream, x, w,
                               items, n_items, out, M, K, N, (int)max_items, tail_cu);
        return hipGetLastError();
    }
    const int64_t grid = max_items * 2 * (N / kRaggedTN);
    if (out_f32)
        hipLaunchKernelGGL((ragged_dot_kernel<1, 0>), dim3((unsigned)grid), dim3(256), 0, stream, x, w, items, n_items,
                           out, M, K, N, (int)max_items, 0);
    else
        hipLaunchKernelGGL((ragged_dot_kernel<0, 0>), dim3((unsigned)grid), dim3(256), 0, stream, x, w, items, n_items,
                           out, M, K, N, (int)max_items, 0);
    return hipGetLastError();
}

}  // namespace bsattn
