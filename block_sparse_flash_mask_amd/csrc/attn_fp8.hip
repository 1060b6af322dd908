// attn_fp8.hip -- block-sparse flash-attention forward with fp8 (e4m3, OCP form)
// q, k, v, fp32 accumulation, bf16 out + fp32 lse, for gfx950.
//
// What is computed: the forward of attn_bf16.hip ("Writing Pallas Kernels for
// JAX", section "Writing the Kernel Logic: Load, Compute, Store"; exact tiled
// softmax, "Pallas-Triton kernels and kernel auto-tuning", section "Flash
// Attention") on fp8 inputs: "JAX Pallas and Blackwell", section "What the
// Tutorial Covers", keeps accumulators in fp32 and uses fp8 only at the
// boundary, in a kernel benchmarked against the fp8 peak.
// Both products run on v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 x e4m3, unit
// scales), twice the bf16 rate; the row max, exponentials and row sums stay fp32
// (so lse is not quantised), and P is rounded to e4m3 for the P V product.
//
// Operand layouts (one step = 64 keys = two 32-key subtiles t):
//   S^T = K Q^T      A = K from LDS, B = Q^T in VGPRs.  Lane (i + 32h) holds 32
//                    bytes of row i at d = 64m + 32h .. +31 in both operands, so
//                    the MFMA pairs equal d whatever its internal k order.
//   O^T += V^T P^T   B = P^T: lane (j + 32h) packs its own S^T registers of both
//                    subtiles (byte 16t + 4g + u = key 32t + 8g + 4h + u, the C
//                    layout of the first product).  A = V^T: lane (d + 32h) needs
//                    V[key][d] for the same 32 keys in the same byte order; a
//                    pre-pass (fp8_vt_kernel) writes V per 64-key tile as
//                    vt[d][64] with byte 32h + 16t + 4g + u = V[32t + 8g + 4h + u][d]
//                    (each lane then reads 32 contiguous bytes), stored in the
//                    order of the LDS image below.
// Element-level masks (ELEM = 1): the list entry of a partial block carries its bit
// tile (kj | (tile + 1) << 16, as in the bf16 kernel); after the S MFMAs each lane
// reads one 32-bit word of its query row per 32-key subtile and sets to -inf the
// scores whose bit is clear (register 4g + u of subtile t is key 8g + 4h + u, so
// the word is shifted by 4h and bit 8g + u tested).  A row may have no kept score
// yet (m = -inf): the exponent then uses m = 0 and the rescale factor is 0, so
// dropped scores give exact zeros; a row that keeps nothing ends with 0 and -inf.
// LDS: a K tile is row-major, 64 rows of D bytes, with the 16-byte unit c of row r
// at slot c ^ x(r), x(r) = (r / (256 / D)) % (D / 16).  Each 1 KiB DMA instruction
// (a buffer load with the LDS flag) then reads 1024 / D whole rows, i.e. whole
// 128-byte lines (the L2 -> CU path serves an instruction that touches 32 rows
// for 32 bytes each at about a quarter of that rate), and an operand read (16
// lanes, 16 consecutive rows, one unit) hits 16 distinct 16-byte bank groups.  A
// V^T tile is D/32 blocks of 2 KiB, block md holding vt[32md + l%32][32(l/32) +
// 16p .. +15] in plane p at p*1024 + l*16 (lane-linear reads); the pre-pass
// stores it in exactly this order, so its DMA is a linear copy.
#include "bf16_layout.h"
#include "common.h"
#include "kernels.h"

namespace bsattn {

typedef int i32x8 __attribute__((ext_vector_type(8)));

namespace {

constexpr int kFp8TK = 64;     // keys per step: the K depth of the fp8 MFMA
constexpr int kFp8Scale = 127;  // E8M0 block scale of 1.0

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, kFp8Scale, 0, kFp8Scale);
}

// 32 bytes of a lane from two 1 KiB planes.
__device__ __forceinline__ i32x8 lds32(const uint8_t* blk, int lane) {
    const u32x4 lo = *(const u32x4*)(blk + lane * 16);
    const u32x4 hi = *(const u32x4*)(blk + 1024 + lane * 16);
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

}  // namespace

// V rearranged per 64-key tile (header).  One workgroup per tile: the tile is
// read into LDS with 16-byte loads, each thread transposes 4x4 byte blocks (keys
// key0 .. key0+3 of output dword w, by d = 4*d4 .. +3) in registers into an LDS
// copy with rows padded to 17 dwords (no bank conflicts on the column writes),
// and the rows go out with 16-byte stores.
template <int D>
__global__ __launch_bounds__(256) void fp8_vt_kernel(const uint8_t* __restrict__ v, uint8_t* __restrict__ vt) {
    constexpr int D4 = D / 4;
    __shared__ uint32_t in[64 * D4];  // [key][d4]
    __shared__ uint32_t tr[D * 17];   // [d][w], 16 of 17 dwords used
    const size_t base = (size_t)blockIdx.x * 64 * D;
    for (int i = threadIdx.x; i < 64 * D / 16; i += 256) ((u32x4*)in)[i] = ((const u32x4*)(v + base))[i];
    __syncthreads();
    for (int i = threadIdx.x; i < 16 * D4; i += 256) {
        const int w = i / D4, d4 = i % D4;
        const int key0 = 32 * ((w >> 2) & 1) + 8 * (w & 3) + 4 * (w >> 3);
        uint32_t x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) x[u] = in[(key0 + u) * D4 + d4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t y = 0;
#pragma unroll
            for (int u = 0; u < 4; ++u) y |= ((x[u] >> (8 * j)) & 0xffu) << (8 * u);
            tr[(4 * d4 + j) * 17 + w] = y;
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * D / 16; i += 256) {  // row d = i / 4, dwords 4q .. +3, q = i % 4
        const int d = i >> 2, q = i & 3;
        const uint32_t* rp = tr + d * 17 + 4 * q;
        // LDS image: block d / 32, plane q % 2, lane 32 (q / 2) + d % 32
        ((u32x4*)(vt + base))[(d >> 5) * 128 + (q & 1) * 64 + (q >> 1) * 32 + (d & 31)] =
            u32x4{rp[0], rp[1], rp[2], rp[3]};
    }
}

template <int D, int WAVES, int OCC, int ELEM>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC))) void attn_fp8_kernel(
    FwdArgs a) {
    constexpr int MQ = D / 64;       // fp8 MFMAs over d per 32x32 score tile
    constexpr int MD = D / 32;       // 32-wide d tiles of O^T
    constexpr int TBYTES = 64 * D;   // one K or V^T tile
    constexpr int NK = 4 * MQ / WAVES;  // K DMA instructions per wave (1 KiB each)
    constexpr int NV = 2 * MD / WAVES;  // V DMA instructions per wave
    static_assert(NK * WAVES == 4 * MQ && NV * WAVES == 2 * MD, "even DMA split");
    __shared__ __attribute__((aligned(1024))) uint8_t k0s[TBYTES], v0s[TBYTES], k1s[TBYTES], v1s[TBYTES];

    int r, sub;
    block_work(a, r, sub);
    if (r < 0) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
    const int wave_s = wave_uniform(wave);
    const int bh = r / a.n_q;
    const int qi = r - bh * a.n_q;
    int beg, cnt;
    row_list(a, r, beg, cnt);
    const int sh = a.steps_log2;  // 64-key steps per key block
    const int n_steps = cnt << sh;
    const size_t head = (size_t)bh * a.S * D;  // bytes
    const int q_row = qi * a.block_q + sub * 32 * WAVES + wave * 32 + l32;

    // Q^T: lane (h, q) holds Q[q][64m + 32h .. +31]; a negative scale flips the
    // sign bit of every byte (c = |scale| log2 e).
    i32x8 qf[MQ];
    {
        const u32x4* qp = (const u32x4*)((const uint8_t*)a.q + head + (size_t)q_row * D);
        const uint32_t sg = a.qsign;
#pragma unroll
        for (int m = 0; m < MQ; ++m) {
            const u32x4 lo = qp[4 * m + 2 * h] ^ sg, hi = qp[4 * m + 2 * h + 1] ^ sg;
            qf[m] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
    }

    const uint8_t* kg = (const uint8_t*)a.k + head;
    const uint8_t* vg = (const uint8_t*)a.v + head;  // the vt copy
    const int nrec = a.S * D;
    // K: instruction i fills rows RPI*i .. of the tile; lane l takes slot l % CPR of
    // row l / CPR, i.e. unit (l % CPR) ^ x(row).  x(RPI*i + l/CPR) depends on i only
    // through its parity (D = 128) or not at all (D = 64), and a wave's i all share
    // the parity of the wave (WAVES is even): one lane offset per wave.
    constexpr int CPR = D / 16, RPI = 1024 / D, XSH = D == 128 ? 1 : 2;
    auto xsw = [](int row) { return (row >> XSH) & (CPR - 1); };
    const int k_row = RPI * (wave_s & 1) + lane / CPR;
    const int k_voff = (lane / CPR) * D + 16 * ((lane % CPR) ^ xsw(k_row));
    // operand reads: lane (h, i) takes units 4m + 2h + p of row 32t + i (x(32t + i) = x(i))
    int k_rd[MQ][2];
#pragma unroll
    for (int m = 0; m < MQ; ++m)
#pragma unroll
        for (int p = 0; p < 2; ++p) k_rd[m][p] = l32 * D + 16 * ((4 * m + 2 * h + p) ^ xsw(l32));
    auto k_frag = [&](const uint8_t* kbuf, int t, int m) -> i32x8 {
        const u32x4 lo = *(const u32x4*)(kbuf + t * 32 * D + k_rd[m][0]);
        const u32x4 hi = *(const u32x4*)(kbuf + t * 32 * D + k_rd[m][1]);
        return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };
    // V: instruction i copies KiB i of the tile's LDS image.
    auto issue = [&](int key0, uint8_t* kbuf, uint8_t* vbuf) {
#pragma unroll
        for (int j = 0; j < NK; ++j) {
            const int i = wave_s + j * WAVES;
            dma16(kg, nrec, (BSATTN_LDS void*)(kbuf + i * 1024), k_voff, (key0 + RPI * i) * D);
        }
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int i = wave_s + j * WAVES;
            dma16(vg, nrec, (BSATTN_LDS void*)(vbuf + i * 1024), lane * 16, key0 * D + i * 1024);
        }
    };

    float m_run = -INFINITY, l_run = 0.f;
    f32x16 oacc[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md) oacc[md] = f32x16{};

    // Element masks: the kept bits of this lane's query row for step st's 64 keys
    // (entry e of the step's key block), applied to S.
    auto apply_tile = [&](f32x16* s, int e, int st) {
        int tile = (e >> 16) - 1;  // -1: full block
        if (tile < 0) return;
        tile = tile < a.n_tiles ? tile : a.n_tiles - 1;  // (a plan never holds more)
        const int qr = q_row - qi * a.block_q;
        const int ko = (st & ((1 << sh) - 1)) * kFp8TK;
        const uint32_t* wrow = a.pbits + ((size_t)tile * a.block_q + qr) * (a.block_k >> 5) + (ko >> 5);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint32_t w = wrow[t] >> (4 * h);
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (!((w >> (8 * g + u)) & 1u)) s[t][4 * g + u] = -INFINITY;
        }
    };

    auto compute = [&](const uint8_t* kbuf, const uint8_t* vbuf, int e, int st) {
        f32x16 s[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            s[t] = f32x16{};
#pragma unroll
            for (int m = 0; m < MQ; ++m) s[t] = mfma_fp8(k_frag(kbuf, t, m), qf[m], s[t]);
        }
        if constexpr (ELEM) apply_tile(s, e, st);
        // row max over the 64 keys and the lazy move of the reference max
        float tmp[32];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            tmp[i] = s[0][i];
            tmp[16 + i] = s[1][i];
        }
        const float mx = max_halves_nan(max_tree3<32>(tmp)) * a.c;
        if (__ballot(mx > m_run + 8.0f) != 0) {
            const float m_new = fmax_nan(m_run, mx);
            // (element masks: a row may still have no kept score, m = -inf)
            const float alpha = (ELEM && m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int md = 0; md < MD; ++md) oacc[md] *= alpha;
            m_run = m_new;
        }
        // P = 2^(c S - m) (<= 2^8, inside e4m3's range); fp32 row sums; P^T in e4m3
        // (element masks: with no kept score yet every S is -inf; use m = 0)
        const float m_use = (ELEM && m_run == -INFINITY) ? 0.f : m_run;
        i32x8 pb;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float e[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    e[u] = fast_exp2(__builtin_fmaf(s[t][4 * g + u], a.c, -m_use));
                    tmp[16 * t + 4 * g + u] = e[u];
                }
                int w = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], 0, false);
                w = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], w, true);
                pb[4 * t + g] = w;
            }
        l_run += tree_sum<32>(tmp);
#pragma unroll
        for (int md = 0; md < MD; ++md) oacc[md] = mfma_fp8(lds32(vbuf + md * 2048, lane), pb, oacc[md]);
    };

    auto entry = [&](int t) -> int {
        const int i = t >> sh;
        return a.list[beg + (i < cnt ? i : cnt - 1)];
    };
    auto key0_of = [&](int kj_raw, int t) -> int {
        int kj = wave_uniform(kj_raw);
        if constexpr (ELEM) kj &= 0xffff;  // element masks: tile + 1 in bits 16..30
        kj = kj < 0 ? 0 : (kj >= a.n_k ? a.n_k - 1 : kj);
        return kj * a.block_k + (t & ((1 << sh) - 1)) * kFp8TK;
    };
    // e_next: the list entry of the step whose DMA was issued last (element masks
    // read its bit tile when that step computes).
    int e_next = 0;
    auto step = [&](int t, int& pre, uint8_t* kfill, uint8_t* vfill, const uint8_t* kcur, const uint8_t* vcur) {
        __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this wave's DMA of step t
        __syncthreads();                     // everyone's landed; step t-1 fully read
        const int e_cur = e_next;
        if (t + 1 < n_steps) {
            const int kn = key0_of(pre, t + 1);
            if constexpr (ELEM) e_next = wave_uniform(pre);
            pre = entry(t + 2);
            issue(kn, kfill, vfill);
        }
        compute(kcur, vcur, e_cur, t);
    };

    if (n_steps > 0) {
        int pre = entry(1);
        e_next = wave_uniform(entry(0));
        issue(key0_of(e_next, 0), k0s, v0s);
        for (int t = 0; t < n_steps; t += 2) {
            step(t, pre, k1s, v1s, k0s, v0s);
            if (t + 1 < n_steps) step(t + 1, pre, k0s, v0s, k1s, v1s);
        }
    }

    // Epilogue: O / l in bf16, lse = ln2 (m + log2 l); a row with no key block
    // gets 0 and -inf.
    const bool any = ELEM ? m_run != -INFINITY : n_steps > 0;
    const float l_tot = sum_halves(l_run);
    const float inv = any ? 1.0f / l_tot : 0.0f;
    uint16_t* og = (uint16_t*)a.out + (size_t)bh * a.S * D + (size_t)q_row * D;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            bf16x4 o;
#pragma unroll
            for (int u = 0; u < 4; ++u) o[u] = (__bf16)(oacc[md][4 * g4 + u] * inv);
            *(bf16x4*)(og + 32 * md + 8 * g4 + 4 * h) = o;
        }
    if (h == 0) a.lse[(size_t)bh * a.S + q_row] = any ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
}

hipError_t launch_fp8_vt(const void* v, void* vt, int64_t tiles, int D, hipStream_t stream) {
    if (D == 128)
        hipLaunchKernelGGL(fp8_vt_kernel<128>, dim3((unsigned)tiles), dim3(256), 0, stream, (const uint8_t*)v,
                           (uint8_t*)vt);
    else
        hipLaunchKernelGGL(fp8_vt_kernel<64>, dim3((unsigned)tiles), dim3(256), 0, stream, (const uint8_t*)v,
                           (uint8_t*)vt);
    return hipGetLastError();
}

template <int D, int W, int OCC, int ELEM = 0>
static hipError_t launch_fp8(const FwdArgs& a, unsigned grid, hipStream_t stream) {
    hipLaunchKernelGGL((attn_fp8_kernel<D, W, OCC, ELEM>), dim3(grid), dim3(W * 64), 0, stream, a);
    return hipGetLastError();
}

// {dtype 2 = fp8, D, tile_q, tile_k, waves, stages, launcher}.  Waves per SIMD:
// three for D = 128 (two measured 2-3 % slower, four spills), four for D = 64
// (its softmax is as much VALU work against half the MFMA work; 2 % faster than
// three on the long-context shape, five spills).
static const Variant kFp8Variants[] = {
    {2, 128, 128, 64, 4, 2, &launch_fp8<128, 4, 3>}, {2, 128, 64, 64, 2, 2, &launch_fp8<128, 2, 3>},
    {2, 64, 128, 64, 4, 2, &launch_fp8<64, 4, 4>},   {2, 64, 64, 64, 2, 2, &launch_fp8<64, 2, 3>},
};

// The same four with element-level masks.
static const Variant kFp8ElemVariants[] = {
    {2, 128, 128, 64, 4, 2, &launch_fp8<128, 4, 3, 1>}, {2, 128, 64, 64, 2, 2, &launch_fp8<128, 2, 3, 1>},
    {2, 64, 128, 64, 4, 2, &launch_fp8<64, 4, 4, 1>},   {2, 64, 64, 64, 2, 2, &launch_fp8<64, 2, 3, 1>},
};

const Variant* fp8_variants(int* n) {
    *n = (int)(sizeof(kFp8Variants) / sizeof(kFp8Variants[0]));
    return kFp8Variants;
}

const Variant* fp8_elem_variants(int* n) {
    *n = (int)(sizeof(kFp8ElemVariants) / sizeof(kFp8ElemVariants[0]));
    return kFp8ElemVariants;
}

}  // namespace bsattn
