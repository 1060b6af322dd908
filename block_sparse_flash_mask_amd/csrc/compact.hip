// compact.hip -- block-mask compaction kernels for gfx950.
//
// The forward pass visits only active (query block, key block) pairs.  These
// kernels turn the uint8 block mask [B][H][n_q][n_k] into per-mask-row lists of
// active key blocks, in ascending kj order:
//   rows_kernel   one wave per mask row: a ballot over 64 mask bytes at a time
//                 and a per-lane prefix count (mbcnt) place each active kj; the
//                 row's count and its list (padded to n_k entries) are written.
//   scan_kernel   one workgroup: exclusive scan of the row counts -> row_ptr.
//   pack_kernel   one wave per row: copy each padded list to its CSR slot.
// All integer, so the result is bit-exact and deterministic.
#include "common.h"
#include "kernels.h"

namespace bsattn {

constexpr int kRowsPerBlock = 4;  // one wave per mask row, 4 waves per workgroup

__global__ __launch_bounds__(256) void rows_kernel(const uint8_t* __restrict__ mask, int64_t R,
                                                   int n_k, int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ lists) {
    const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (r >= R) return;  // wave-uniform
    const int lane = threadIdx.x & 63;
    const uint8_t* mrow = mask + r * n_k;
    int32_t* lrow = lists + r * n_k;
    int base = 0;
    for (int s0 = 0; s0 < n_k; s0 += kWave) {
        const int kj = s0 + lane;
        const bool active = kj < n_k && mrow[kj] != 0;
        const uint64_t bal = __ballot(active);
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
        if (active) lrow[base + below] = kj;
        base += __popcll(bal);
    }
    if (lane == 0) counts[r] = base;
}

// Element-level masks: block states (0 empty, 1 full, else partial) and the bit
// tile of each partial block.  Same lists as rows_kernel, with entries
// kj | (tile + 1) << 16 (0 for a full block), the tile index clamped into
// [0, n_tiles) so a malformed index can give wrong values but never an
// out-of-bounds read.
__global__ __launch_bounds__(256) void rows_elem_kernel(const uint8_t* __restrict__ states,
                                                        const int32_t* __restrict__ pidx, int n_tiles,
                                                        int64_t R, int n_k, int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ lists) {
    const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (r >= R) return;  // wave-uniform
    const int lane = threadIdx.x & 63;
    const uint8_t* srow = states + r * n_k;
    const int32_t* prow = pidx + r * n_k;
    int32_t* lrow = lists + r * n_k;
    int base = 0;
    for (int s0 = 0; s0 < n_k; s0 += kWave) {
        const int kj = s0 + lane;
        const int st = kj < n_k ? srow[kj] : 0;
        const bool active = st != 0;
        const uint64_t bal = __ballot(active);
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
        if (active) {
            int tile = 0;
            if (st > 1) {
                tile = prow[kj];
                tile = (tile < 0 ? 0 : (tile >= n_tiles ? n_tiles - 1 : tile)) + 1;
            }
            lrow[base + below] = kj | (tile << 16);
        }
        base += __popcll(bal);
    }
    if (lane == 0) counts[r] = base;
}

constexpr int kScanThreads = 1024;
constexpr int kScanPerThread = 4;

// Inclusive scan across the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

__global__ __launch_bounds__(kScanThreads) void scan_kernel(const int32_t* __restrict__ counts,
                                                            int64_t R,
                                                            int32_t* __restrict__ row_ptr) {
    __shared__ int wave_tot[kScanThreads / kWave];
    __shared__ int carry_s;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) {
        row_ptr[0] = 0;
        carry_s = 0;
    }
    __syncthreads();
    constexpr int64_t kTile = (int64_t)kScanThreads * kScanPerThread;
    for (int64_t t0 = 0; t0 < R; t0 += kTile) {
        const int64_t i0 = t0 + (int64_t)tid * kScanPerThread;
        int v[kScanPerThread];
        int run = 0;
#pragma unroll
        for (int j = 0; j < kScanPerThread; ++j) {
            v[j] = (i0 + j < R) ? counts[i0 + j] : 0;
            run += v[j];
            v[j] = run;  // inclusive within the thread
        }
        const int incl = wave_inclusive_scan(run);
        if (lane == 63) wave_tot[wave] = incl;
        __syncthreads();
        if (wave == 0) {
            int wt = lane < kScanThreads / kWave ? wave_tot[lane] : 0;
            wt = wave_inclusive_scan(wt);
            if (lane < kScanThreads / kWave) wave_tot[lane] = wt;  // inclusive over waves
        }
        __syncthreads();
        const int carry = carry_s;
        const int before = carry + (wave > 0 ? wave_tot[wave - 1] : 0) + (incl - run);
#pragma unroll
        for (int j = 0; j < kScanPerThread; ++j)
            if (i0 + j < R) row_ptr[i0 + j + 1] = before + v[j];
        __syncthreads();
        if (tid == 0) carry_s = carry + wave_tot[kScanThreads / kWave - 1];
        __syncthreads();
    }
}

__global__ __launch_bounds__(256) void pack_kernel(const int32_t* __restrict__ counts,
                                                   const int32_t* __restrict__ lists, int64_t R,
                                                   int n_k, const int32_t* __restrict__ row_ptr,
                                                   int32_t* __restrict__ col_idx) {
    const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (r >= R) return;
    const int lane = threadIdx.x & 63;
    const int cnt = counts[r];
    const int32_t* src = lists + r * n_k;
    int32_t* dst = col_idx + row_ptr[r];
    for (int i = lane; i < cnt; i += kWave) dst[i] = src[i];
}

// Dispatch order of the attention workgroups.  Workgroups go to the 8 XCDs of
// the chip round-robin by blockIdx, so blockIdx b runs on XCD b % 8 and is the
// (b / 8)-th workgroup that XCD receives.  Mask rows are cut into 8 contiguous
// chunks of `chunk` rows, one per XCD, so the query tiles of a head share that
// XCD's L2.  Inside a chunk the rows go head by head, in (b, h) order, and within
// a head longest first: the workgroups in flight on an XCD then read the K and V
// of one or two heads (which stay in its L2), and the short rows come last, which
// evens out the finishing times.  One workgroup per chunk runs a counting sort on
// the key (local head, -count): a histogram in LDS, an exclusive scan of it, then
// a scatter.  If a chunk would need more bins than the histogram holds, the key
// is -count alone (longest first over the whole chunk).  Rows with equal keys land
// in arbitrary order, which cannot change any result (each row is computed on its
// own).  order[x * chunk + j] = mask row, or -1 for padding past the last row.
//
// Within an XCD the dispatcher deals consecutive workgroups to the XCD's four
// shader engines in turn and strictly in order: a workgroup whose engine has no
// free CU holds back every workgroup behind it, even those bound for idle
// engines (measured with per-workgroup timestamps and hardware ids).  Longest
// first within a head would hand the same engine the longest workgroup of every
// group of four, so that engine falls behind and stalls the others.  The sorted
// sequence is therefore laid out in groups of four with every other group
// reversed: each engine alternately gets the longest and the shortest of a
// group, and the four engines' work stays even.
constexpr int kOrderThreads = 1024;
constexpr int kOrderMaxBins = 4096;

__device__ __forceinline__ int order_wave_scan(int x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

// Sort key of a row with c active blocks out of nk1 - 1; hl is its head's index
// within the chunk (0 when the chunk is sorted by count alone).
__device__ __forceinline__ int order_bin(int c, int hl, int nk1) {
    c = c < 0 ? 0 : (c > nk1 - 1 ? nk1 - 1 : c);
    return hl * nk1 + (nk1 - 1 - c);
}

// One sort job: `items` entries (mask rows, or pairs of adjacent mask rows of a
// head) dealt to 8 XCD chunks of `chunk`, each sorted by (head, -count).
struct OrderJob {
    int64_t items;
    int64_t chunk;
    int per_head;   // items per (b, h): n_q rows, or ceil(n_q / 2) pairs
    int pairs;      // 1: item p is rows (b, h, 2j) and (b, h, 2j + 1)
    int by_head;
    int nk1;
    int nbins;
    int32_t* order;
};

// Counting sort of chunk x of a job (one workgroup of kOrderThreads): a
// histogram of the keys in LDS, an exclusive scan of it, then a scatter.
// key_of(k) is the sort key of item r0 + k (it may be called twice per item).
template <class KeyOf>
__device__ void sort_chunk(const OrderJob& job, int64_t r0, int64_t nr, KeyOf key_of, int* hist,
                           int* wave_tot) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int b = tid; b < job.nbins; b += kOrderThreads) hist[b] = 0;
    __syncthreads();
    for (int64_t k = tid; k < nr; k += kOrderThreads) atomicAdd(&hist[key_of(k)], 1);
    __syncthreads();
    // Exclusive scan of hist: each thread owns a run of consecutive bins.
    const int nbins = job.nbins;
    const int per = (nbins + kOrderThreads - 1) / kOrderThreads;
    const int b0 = tid * per;
    int run = 0;
    for (int b = b0; b < b0 + per && b < nbins; ++b) run += hist[b];
    const int incl = order_wave_scan(run);
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        int t = lane < kOrderThreads / kWave ? wave_tot[lane] : 0;
        t = order_wave_scan(t);
        if (lane < kOrderThreads / kWave) wave_tot[lane] = t;
    }
    __syncthreads();
    int pre = (wave > 0 ? wave_tot[wave - 1] : 0) + incl - run;
    for (int b = b0; b < b0 + per && b < nbins; ++b) {
        const int h = hist[b];
        hist[b] = pre;
        pre += h;
    }
    __syncthreads();
    for (int64_t k = tid; k < nr; k += kOrderThreads) {
        int pos = atomicAdd(&hist[key_of(k)], 1);
        // odd groups of four (complete ones only) are reversed
        if (((pos >> 2) & 1) && (int64_t)(pos | 3) < nr) pos ^= 3;
        job.order[r0 + pos] = (int32_t)(r0 + k);
    }
    for (int64_t i = nr + tid; i < job.chunk; i += kOrderThreads) job.order[r0 + i] = -1;
}

// Rows (or pairs) r0 .. r0 + nr - 1 of chunk x of a job.
__device__ __forceinline__ void chunk_range(const OrderJob& job, int x, int64_t& r0, int64_t& nr) {
    r0 = (int64_t)x * job.chunk;
    nr = r0 >= job.items ? 0 : (job.items - r0 < job.chunk ? job.items - r0 : job.chunk);
}

__global__ __launch_bounds__(kOrderThreads) void order_kernel(const int32_t* __restrict__ counts,
                                                              int n_q, OrderJob rows_job,
                                                              OrderJob pairs_job) {
    __shared__ int hist[kOrderMaxBins];
    __shared__ int wave_tot[kOrderThreads / kWave];
    const OrderJob& job = blockIdx.x < 8 ? rows_job : pairs_job;
    int64_t r0, nr;
    chunk_range(job, blockIdx.x & 7, r0, nr);
    const int64_t h0 = r0 / job.per_head;
    auto count_of = [&](int64_t i) -> int {
        if (!job.pairs) return counts[i];
        const int64_t bh = i / job.per_head;
        const int j = (int)(i - bh * job.per_head);
        const int64_t ra = bh * n_q + 2 * j;
        const int ca = counts[ra];
        const int cb = 2 * j + 1 < n_q ? counts[ra + 1] : 0;
        return ca > cb ? ca : cb;
    };
    auto key = [&](int64_t k) {
        const int hl = job.by_head ? (int)((r0 + k) / job.per_head - h0) : 0;
        return order_bin(count_of(r0 + k), hl, job.nk1);
    };
    sort_chunk(job, r0, nr, key, hist, wave_tot);
}

// Nonzero bytes of a 32-bit word: bit 7 of each byte of
// ((x & 0x7f..) + 0x7f..) | x is set iff that byte is nonzero (no carry crosses
// a byte).
__device__ __forceinline__ int nonzero_bytes(uint32_t x) {
    return __popc((((x & 0x7f7f7f7fu) + 0x7f7f7f7fu) | x) & 0x80808080u);
}

// Active blocks of one mask row, counted by one thread: 16-byte loads when the
// rows are 16-byte aligned (vec = 16), 4-byte loads when 4-byte aligned
// (vec = 4), else bytes.  The loads of a row are independent, so they overlap.
__device__ __forceinline__ int mask_row_count(const uint8_t* __restrict__ mrow, int n_k, int vec) {
    int c = 0;
    if (vec == 16) {
        for (int b = 0; b < n_k; b += 16) {
            const uint4 v = *(const uint4*)(mrow + b);
            c += nonzero_bytes(v.x) + nonzero_bytes(v.y) + nonzero_bytes(v.z) + nonzero_bytes(v.w);
        }
    } else if (vec == 4) {
        for (int b = 0; b < n_k; b += 4) c += nonzero_bytes(*(const uint32_t*)(mrow + b));
    } else {
        for (int b = 0; b < n_k; ++b) c += mrow[b] != 0;
    }
    return c;
}

// The whole plan in one launch, for masks small enough that 16 workgroups can
// count their chunks' rows straight from the mask in about the time the row
// lists take.  Workgroups 0-15 run the two sorts (rows, pairs), each thread
// counting the active blocks of one row (or both rows of one pair) of its
// chunk from the mask into an LDS key cache; the others are rows_kernel with
// 16 mask rows (one per wave) each.
// Limits of the single launch: the mask size, and the row length (a thread reads
// a whole row; longer rows than one or two cache lines per thread thrash the L1
// when a wave reads 64 rows at once, and the two launches are faster).
constexpr int kPlanMaxChunk = 8192;
constexpr int64_t kPlanMaxMaskBytes = (int64_t)4 << 20;
constexpr int kPlanMaxRowBytes = 128;

__global__ __launch_bounds__(kOrderThreads) void plan_kernel(const uint8_t* __restrict__ mask,
                                                             int64_t R, int n_q, int n_k, int vec,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ lists,
                                                             OrderJob rows_job, OrderJob pairs_job) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (blockIdx.x >= 16) {
        const int64_t r = (int64_t)(blockIdx.x - 16) * (kOrderThreads / kWave) + wave;
        if (r >= R) return;  // wave-uniform
        const uint8_t* mrow = mask + r * n_k;
        int32_t* lrow = lists + r * n_k;
        int base = 0;
        for (int s0 = 0; s0 < n_k; s0 += kWave) {
            const int kj = s0 + lane;
            const bool active = kj < n_k && mrow[kj] != 0;
            const uint64_t bal = __ballot(active);
            const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                        __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
            if (active) lrow[base + below] = kj;
            base += __popcll(bal);
        }
        if (lane == 0) counts[r] = base;
        return;
    }
    __shared__ int hist[kOrderMaxBins];
    __shared__ int wave_tot[kOrderThreads / kWave];
    __shared__ int keys[kPlanMaxChunk];
    const OrderJob& job = blockIdx.x < 8 ? rows_job : pairs_job;
    int64_t r0, nr;
    chunk_range(job, blockIdx.x & 7, r0, nr);
    const int64_t h0 = r0 / job.per_head;
    for (int64_t k = tid; k < nr; k += kOrderThreads) {
        const int64_t i = r0 + k;
        int c;
        if (!job.pairs) {
            c = mask_row_count(mask + i * n_k, n_k, vec);
        } else {
            const int64_t bh = i / job.per_head;
            const int j = (int)(i - bh * job.per_head);
            const int64_t ra = bh * n_q + 2 * j;
            const int ca = mask_row_count(mask + ra * n_k, n_k, vec);
            const int cb = 2 * j + 1 < n_q ? mask_row_count(mask + (ra + 1) * n_k, n_k, vec) : 0;
            c = ca > cb ? ca : cb;
        }
        const int hl = job.by_head ? (int)(i / job.per_head - h0) : 0;
        keys[k] = order_bin(c, hl, job.nk1);
    }
    __syncthreads();
    sort_chunk(job, r0, nr, [&](int64_t k) { return keys[k]; }, hist, wave_tot);
}

static OrderJob make_job(int64_t items, int64_t chunk, int per_head, int pairs, int n_k,
                         int32_t* order) {
    OrderJob j;
    j.items = items;
    j.chunk = chunk;
    j.per_head = per_head;
    j.pairs = pairs;
    j.order = order;
    // A chunk of `chunk` consecutive items touches at most this many heads.
    const int64_t heads = (chunk + per_head - 1) / per_head + 1;
    j.nk1 = n_k + 1;
    if (heads * j.nk1 <= kOrderMaxBins) {
        j.by_head = 1;
        j.nbins = (int)(heads * j.nk1);
    } else {
        j.by_head = 0;
        j.nk1 = j.nk1 < kOrderMaxBins ? j.nk1 : kOrderMaxBins;
        j.nbins = j.nk1;
    }
    return j;
}

hipError_t launch_compact_order(const int32_t* counts, int64_t R, int n_q, int n_k, int64_t chunk,
                                int32_t* order, int64_t pchunk, int32_t* porder,
                                hipStream_t stream) {
    if (R <= 0 || n_q <= 0 || n_k <= 0 || chunk <= 0 || 8 * chunk < R) return hipErrorInvalidValue;
    const int hq = (n_q + 1) / 2;
    const int64_t P = R / n_q * hq;
    if (pchunk <= 0 || 8 * pchunk < P) return hipErrorInvalidValue;
    const OrderJob rj = make_job(R, chunk, n_q, 0, n_k, order);
    const OrderJob pj = make_job(P, pchunk, hq, 1, n_k, porder);
    hipLaunchKernelGGL(order_kernel, dim3(16), dim3(kOrderThreads), 0, stream, counts, n_q, rj, pj);
    return hipGetLastError();
}

hipError_t launch_plan(const uint8_t* mask, int64_t R, int n_q, int n_k, int32_t* counts,
                       int32_t* lists, int64_t chunk, int32_t* order, int64_t pchunk,
                       int32_t* porder, hipStream_t stream) {
    if (R <= 0 || n_q <= 0 || n_k <= 0 || chunk <= 0 || 8 * chunk < R) return hipErrorInvalidValue;
    const int hq = (n_q + 1) / 2;
    const int64_t P = R / n_q * hq;
    if (pchunk <= 0 || 8 * pchunk < P) return hipErrorInvalidValue;
    if (R * n_k > kPlanMaxMaskBytes || n_k > kPlanMaxRowBytes || chunk > kPlanMaxChunk ||
        pchunk > kPlanMaxChunk) {
        hipError_t e = launch_compact_rows(mask, R, n_k, counts, lists, stream);
        if (e != hipSuccess) return e;
        return launch_compact_order(counts, R, n_q, n_k, chunk, order, pchunk, porder, stream);
    }
    const OrderJob rj = make_job(R, chunk, n_q, 0, n_k, order);
    const OrderJob pj = make_job(P, pchunk, hq, 1, n_k, porder);
    const int64_t row_blocks = (R + kOrderThreads / kWave - 1) / (kOrderThreads / kWave);
    const uintptr_t mbase = (uintptr_t)mask;
    const int vec = (mbase % 16 == 0 && n_k % 16 == 0) ? 16 : (mbase % 4 == 0 && n_k % 4 == 0) ? 4 : 1;
    hipLaunchKernelGGL(plan_kernel, dim3((unsigned)(16 + row_blocks)), dim3(kOrderThreads), 0, stream,
                       mask, R, n_q, n_k, vec, counts, lists, rj, pj);
    return hipGetLastError();
}

hipError_t launch_compact_rows(const uint8_t* mask, int64_t R, int n_k, int32_t* counts,
                               int32_t* lists, hipStream_t stream) {
    const int64_t blocks = (R + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL(rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, mask, R, n_k,
                       counts, lists);
    return hipGetLastError();
}

hipError_t launch_compact_rows_elem(const uint8_t* states, const int32_t* pidx, int n_tiles, int64_t R,
                                    int n_k, int32_t* counts, int32_t* lists, hipStream_t stream) {
    const int64_t blocks = (R + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL(rows_elem_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, states, pidx, n_tiles,
                       R, n_k, counts, lists);
    return hipGetLastError();
}

hipError_t launch_compact_scan(const int32_t* counts, int64_t R, int32_t* row_ptr,
                               hipStream_t stream) {
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, counts, R, row_ptr);
    return hipGetLastError();
}

hipError_t launch_compact_pack(const int32_t* counts, const int32_t* lists, int64_t R, int n_k,
                               const int32_t* row_ptr, int32_t* col_idx, hipStream_t stream) {
    const int64_t blocks = (R + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, counts, lists, R,
                       n_k, row_ptr, col_idx);
    return hipGetLastError();
}

}  // namespace bsattn
