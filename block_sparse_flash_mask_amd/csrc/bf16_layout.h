// bf16_layout.h -- operand-ordered LDS layouts of bf16 K and V tiles shared by
// the gfx950 bf16 attention kernels, and the HBM -> LDS DMA plan that fills them.
//
// K tile (TK keys x D): one 1 KiB block per (32-key tile mt, 16-deep k-step ks);
// lane l's 16 bytes at l*16 are K[32mt + kperm(l%32)][16ks + 8(l/32) .. +7], the
// A operand of v_mfma_f32_32x32x16_bf16 for S^T = K Q^T.
// V tile: one 512 B block per (mt, 16-key half e, 4-key quarter r, 32-wide d tile
// md); lane l's 8 bytes at l*8 are what the 16x4 transpose of its 16-lane group
// (ds_read_b64_tr_b16) needs for the A operand V^T of O^T += V^T P^T:
// V[32mt + 16e + 8h + 4r + L/4][32md + 16g + 4(L%4) .. +3], L = l%16,
// g = (l/16)%2, h = l/32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// Global element offsets (relative to the tile's first key) of the DMA
// instructions a wave issues for one tile: a per-lane part shared by all of the
// wave's K (or V) instructions plus a wave-uniform part per instruction, so the
// address is a scalar base plus one 32-bit VGPR offset.
template <int D, int WAVES, int TK>
struct DmaPlan {
    typedef TileGeom<D, TK> G;
    static constexpr int NK = G::KBLK / WAVES;      // K DMA instructions per wave
    static constexpr int NV = G::VBLK / 2 / WAVES;  // V DMA instructions (2 blocks each)
    static_assert(G::KBLK % WAVES == 0 && (G::VBLK / 2) % WAVES == 0, "even DMA split");
    static_assert(G::MD % 2 == 0, "V blocks pair along d");
    int k_lane;  // kperm(l%32) * D + 8 * (l/32)
    int v_lane;  // see v_uniform

    __device__ __forceinline__ void init(int lane) {
        k_lane = kperm(lane & 31) * D + 8 * (lane >> 5);
        // One V DMA instruction fills blocks 2j (lanes 0..31) and 2j+1 (32..63),
        // block index tb = ((mt*2 + e)*2 + r)*MD + md; lane l writes the 8-byte
        // units u = 2(l%32), u+1 of its block, which hold
        // V[32mt + 16e + 8(u/32) + 4r + (u%16)/4][32md + 16((u/16)%2) + 4(u%4) ..].
        const int u = 2 * (lane & 31);
        const int L = u & 15, g = (u >> 4) & 1, hh = u >> 5;
        v_lane = (8 * hh + (L >> 2)) * D + 32 * (lane >> 5) + 16 * g + 4 * (L & 3);
    }
    // K instruction i of wave w: block blk = w + i*WAVES = mt*KS + ks.
    __device__ __forceinline__ static int k_uniform(int w, int i) {
        const int blk = w + i * WAVES;
        return 32 * (blk / G::KS) * D + 16 * (blk % G::KS);
    }
    // V instruction i of wave w: block pair j = w + i*WAVES, first block tb = 2j.
    __device__ __forceinline__ static int v_uniform(int w, int i) {
        const int tb = 2 * (w + i * WAVES);
        const int md = tb % G::MD, r = (tb / G::MD) % 2, e = (tb / G::MD / 2) % 2,
                  mt = tb / G::MD / 4;
        return (32 * mt + 16 * e + 4 * r) * D + 32 * md;
    }
};

// K tile in the row-chunk layout.  The 1 KiB-per-(mt, ks) layout above makes
// every DMA instruction touch 32 rows for 32 bytes each, and the L2 -> CU path
// serves such an instruction at about a quarter of the rate of one that reads
// 8 rows x 128 contiguous bytes (measured on MI355X: ~16 against ~58 bytes per
// clock per CU from L2).  Here a 1 KiB chunk holds 8 consecutive rows x one
// 128-byte segment (64 elements) of each, chunk (r/8)*NSEG + seg, so each DMA
// instruction reads whole 128-byte lines.  Inside a chunk row r%8 sits at
// (r%8)*128 and its 16-byte unit c at slot c ^ x(r), x(r) = (r/2)%8: the
// MFMA operand read (16 lanes reading 16 different rows at one unit) then hits
// 16 distinct 16-byte bank groups.  Rows are stored in natural order; the read
// applies kperm, so the fragment lane l gets is still
// K[32mt + kperm(l%32)][16ks + 8(l/32) .. +7].
template <int D, int WAVES, int TK>
struct KRowPlan {
    static constexpr int NSEG = D / 64;          // 128-byte segments per row
    static constexpr int NCH = TK / 8 * NSEG;    // 1 KiB chunks per tile
    static constexpr int NK = NCH / WAVES;       // DMA instructions per wave
    static_assert(D % 64 == 0 && NCH % WAVES == 0, "even DMA split over whole segments");
    int dma_lane[2];  // element offset of lane l's 16 bytes, chunk row-group parity 0 / 1
    int rd_lane[4];   // byte offset of lane l's fragment for k-step ks with ks % 4 = index

    __device__ __forceinline__ void init(int lane) {
        // DMA: lane l fills slot l%8 of row l/8 of the chunk; that slot holds unit
        // c = (l%8) ^ x(row), and x(8 g + l/8) = (l/16) | 4 (g%2).
#pragma unroll
        for (int p = 0; p < 2; ++p) dma_lane[p] = (lane >> 3) * D + 8 * ((lane & 7) ^ (lane >> 4) ^ (4 * p));
        const int rho = kperm(lane & 31), hh = lane >> 5, x = (rho >> 1) & 7;
        // unit c = 2 (ks%4) + hh of row rho: slot c ^ x = 2 ((ks%4) ^ (x/2)) + (hh ^ x%2)
        const int base = (rho >> 3) * NSEG * 1024 + (rho & 7) * 128 + 16 * (hh ^ (x & 1));
#pragma unroll
        for (int k = 0; k < 4; ++k) rd_lane[k] = base + 32 * (k ^ (x >> 1));
    }
    // DMA instruction i of wave w fills chunk ch = w + i*WAVES: its first element
    // relative to the tile's first key, and the parity of its row group.
    __device__ __forceinline__ static int uniform(int w, int i) {
        const int ch = w + i * WAVES;
        return 8 * (ch / NSEG) * D + (ch % NSEG) * 64;
    }
    __device__ __forceinline__ static int parity(int w, int i) { return ((w + i * WAVES) / NSEG) & 1; }
    __device__ __forceinline__ int dma_off(int w, int i) const { return parity(w, i) ? dma_lane[1] : dma_lane[0]; }
    // Byte offset of fragment (mt, ks) less the lane part rd_lane[ks % 4].
    static constexpr int frag(int mt, int ks) { return mt * 4 * NSEG * 1024 + (ks / 4) * 1024; }
};

// 16-byte HBM -> LDS DMA per lane through a raw buffer resource over
// [base, base + nrec): global byte offset voff (per lane) + soff (uniform); the
// lane's 16 bytes land at lds + 16 * lane.  A buffer load (rather than a global
// one) keeps the compiler's LDS wait counting exact for the reads that follow.
__device__ __forceinline__ void dma16(const void* base, int nrec, BSATTN_LDS void* lds, int voff,
                                      int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, nrec, 0x00020000), lds, 16, voff, soff, 0, 0);
}

// The same DMA issued as inline assembly: the compiler does not see this LDS
// write, so it adds no waits of its own for it.  The caller waits for it with
// an explicit vmcnt and orders the LDS reads of the target with barriers.
// rsrc is a raw buffer descriptor in SGPRs (make_rsrc), lds the LDS byte address.
__device__ __forceinline__ u32x4 make_rsrc(const void* base, int nrec) {
    const uint64_t b = (uint64_t)(uintptr_t)base;
    return u32x4{(uint32_t)b, (uint32_t)(b >> 32) & 0xffffu, (uint32_t)nrec, 0x00020000u};
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const BSATTN_LDS void*)p;
}
__device__ __forceinline__ void dma16_raw(const u32x4& rsrc, uint32_t lds, int voff, int soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
                 : "m0");
}

}  // namespace bsattn
