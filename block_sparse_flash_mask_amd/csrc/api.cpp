// api.cpp -- the C ABI of libbsattn.so (declared in include/bsattn.h): argument
// checks, workspace layout, tile-config choice, launches, and the autotuner.
//
// Every check runs on the host before the first HIP call, so a bad argument never
// reaches the device.  Kernels are launched on the caller's stream and nothing is
// allocated on the forward path.
#include <algorithm>
#include <atomic>
#include <cerrno>
#include <cfloat>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "bsattn.h"
#include "kernels.h"

using namespace bsattn;

namespace {

thread_local int g_last_hip = 0;

int hip_fail(hipError_t e) {
    g_last_hip = (int)e;
    return BSATTN_ERR_HIP;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

bool is_aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// Compaction workspace: per-row counts, then per-row lists padded to n_k.
size_t compact_ws_bytes(int64_t R, int64_t n_k) {
    return align_up((size_t)R * 4) + align_up((size_t)(R * n_k) * 4);
}

// Mask rows per XCD chunk.
int64_t xcd_chunk(int64_t R) { return (R + 7) / 8; }

// Forward workspace (the plan): per-row counts, padded lists, the dispatch
// order of the R rows (8 * xcd_chunk(R) slots) and that of the P pairs of
// adjacent rows (8 * xcd_chunk(P) slots), each region 256-byte aligned.
struct PlanLayout {
    int64_t R, P;           // mask rows; pairs of rows (2j, 2j+1) of a head
    int64_t chunk, pchunk;  // rows / pairs per XCD chunk
    size_t lists, order, porder, bytes;
};

PlanLayout plan_layout(int64_t BH, int n_q, int n_k) {
    PlanLayout L;
    L.R = BH * n_q;
    L.P = BH * ((n_q + 1) / 2);
    L.chunk = xcd_chunk(L.R);
    L.pchunk = xcd_chunk(L.P);
    L.lists = align_up((size_t)L.R * 4);
    L.order = L.lists + align_up((size_t)(L.R * n_k) * 4);
    L.porder = L.order + align_up((size_t)(8 * L.chunk) * 4);
    L.bytes = L.porder + align_up((size_t)(8 * L.pchunk) * 4);
    return L;
}

size_t fwd_ws_bytes(int64_t BH, int n_q, int n_k) { return plan_layout(BH, n_q, n_k).bytes; }

// Backward workspace.  Plan part: the forward plan (rows, for dq), per key block
// the count and the query-block list padded to n_q, the dk/dv work items
// (C + max_slots int4), the cut key blocks (max_slots / 2 int4) and the two
// counts.  Scratch part (written by every backward call): the per-row
// (lse * log2 e, dout . out) pairs, and the fp32 partial dK, dV of the pieces of
// cut key blocks (max_slots slots of 2 * block_k * 128 floats).
struct BwdLayout {
    PlanLayout fwd;
    int64_t C;          // key blocks (columns): B * H * n_k
    int64_t max_slots;  // partial slots for pieces of cut key blocks
    size_t ccounts, clists, items, splits, nout, ld, scratch, plan_bytes, bytes;
};

BwdLayout bwd_layout(int64_t BH, int S, int n_q, int n_k, int block_k) {
    BwdLayout L;
    L.fwd = plan_layout(BH, n_q, n_k);
    L.C = BH * n_k;
    L.max_slots = std::max<int64_t>(16, (L.C / 4 + 1) & ~(int64_t)1);
    L.ccounts = L.fwd.bytes;
    L.clists = L.ccounts + align_up((size_t)L.C * 4);
    L.items = L.clists + align_up((size_t)(L.C * n_q) * 4);
    L.splits = L.items + align_up((size_t)(L.C + L.max_slots) * 16);
    L.nout = L.splits + align_up((size_t)(L.max_slots / 2) * 16);
    L.plan_bytes = L.nout + align_up(8);
    L.ld = L.plan_bytes;
    L.scratch = L.ld + align_up((size_t)(BH * S) * 8);
    L.bytes = L.scratch + align_up((size_t)L.max_slots * 2 * block_k * 128 * 4);
    return L;
}

int check_grid(int B, int H, int n_q, int n_k) {
    if (B <= 0 || H <= 0 || n_q <= 0 || n_k <= 0) return BSATTN_ERR_SHAPE;
    // Bound each product before the next one, so no int64 product can overflow.
    const int64_t BH = (int64_t)B * H;  // < 2^62
    if (BH >= ((int64_t)1 << 31)) return BSATTN_ERR_SHAPE;
    const int64_t R = BH * n_q;  // < 2^62
    if (R >= ((int64_t)1 << 31) / 2) return BSATTN_ERR_SHAPE;
    if (R * n_k >= ((int64_t)1 << 31)) return BSATTN_ERR_SHAPE;  // list entries are int32
    return BSATTN_OK;
}

bool block_ok(int b) { return b == 64 || b == 128; }

int check_fwd_shape(int B, int H, int S, int D, int block_q, int block_k, int dtype) {
    if (B <= 0 || H <= 0 || S <= 0 || D <= 0 || block_q <= 0 || block_k <= 0)
        return BSATTN_ERR_SHAPE;
    if (S % block_q != 0 || S % block_k != 0) return BSATTN_ERR_SHAPE;
    if (dtype != BSATTN_F32 && dtype != BSATTN_BF16) return BSATTN_ERR_UNSUPPORTED;
    if (D != 64 && D != 128) return BSATTN_ERR_UNSUPPORTED;
    if (!block_ok(block_q) || !block_ok(block_k)) return BSATTN_ERR_UNSUPPORTED;
    const int rc = check_grid(B, H, S / block_q, S / block_k);
    if (rc) return rc;
    if ((int64_t)B * H * S * D >= ((int64_t)1 << 40)) return BSATTN_ERR_SHAPE;
    // One head of K or V is read through a buffer descriptor with a 32-bit range.
    if ((int64_t)S * D * 4 >= ((int64_t)1 << 31)) return BSATTN_ERR_SHAPE;
    return BSATTN_OK;
}

// Checks shared by every forward entry point that takes q/k/v/out/lse.
// Order: NULL pointers, then shapes, then alignment, scale and aliasing (the
// alias test needs valid sizes).
int check_fwd_buffers(const void* q, const void* k, const void* v, const void* out,
                      const float* lse, int B, int H, int S, int D, int block_q, int block_k,
                      int dtype, float scale) {
    if (!q || !k || !v || !out || !lse) return BSATTN_ERR_NULL;
    const int rc = check_fwd_shape(B, H, S, D, block_q, block_k, dtype);
    if (rc) return rc;
    if (!is_aligned(q, 16) || !is_aligned(k, 16) || !is_aligned(v, 16) || !is_aligned(out, 16) ||
        !is_aligned(lse, 4))
        return BSATTN_ERR_ALIGN;
    if (!std::isfinite(scale)) return BSATTN_ERR_SCALE;
    const size_t esz = dtype == BSATTN_F32 ? 4 : 2;
    const size_t nt = (size_t)B * H * S * D * esz;
    const size_t nl = (size_t)B * H * S * 4;
    if (overlap(out, nt, q, nt) || overlap(out, nt, k, nt) || overlap(out, nt, v, nt) ||
        overlap(lse, nl, q, nt) || overlap(lse, nl, k, nt) || overlap(lse, nl, v, nt) ||
        overlap(lse, nl, out, nt))
        return BSATTN_ERR_ALIAS;
    return BSATTN_OK;
}

// The plan region of a forward workspace (ws_used bytes) must not overlap q, k,
// v, out or lse.  Run after check_fwd_buffers (sizes are valid then).
int check_ws_alias(const void* ws, size_t ws_used, const void* q, const void* k, const void* v,
                   const void* out, const float* lse, int B, int H, int S, int D, int dtype) {
    const size_t esz = dtype == BSATTN_F32 ? 4 : 2;
    const size_t nt = (size_t)B * H * S * D * esz;
    const size_t nl = (size_t)B * H * S * 4;
    if (overlap(ws, ws_used, q, nt) || overlap(ws, ws_used, k, nt) || overlap(ws, ws_used, v, nt) ||
        overlap(ws, ws_used, out, nt) || overlap(ws, ws_used, lse, nl))
        return BSATTN_ERR_ALIAS;
    return BSATTN_OK;
}

const Variant* variants(int dtype, int* n) {
    return dtype == BSATTN_BF16 ? bf16_variants(n) : f32_variants(n);
}

// Row-pair variants: two 128-row mask rows per workgroup.
bool is_pair(const Variant& v) { return v.tile_q == 256; }

bool legal(const Variant& v, int dtype, int D, int block_q, int block_k) {
    const bool rows_ok = is_pair(v) ? block_q == 128 : block_q % v.tile_q == 0;
    return v.dtype == dtype && v.D == D && rows_ok && block_k % v.tile_k == 0;
}

bool matches(const Variant& v, const bsattn_tile_config& c) {
    return (!c.tile_q || c.tile_q == v.tile_q) && (!c.tile_k || c.tile_k == v.tile_k) &&
           (!c.waves || c.waves == v.waves) && (!c.stages || c.stages == v.stages);
}

bool is_auto(const bsattn_tile_config* c) {
    return !c || (!c->tile_q && !c->tile_k && !c->waves && !c->stages);
}

const Variant* first_match(const Variant* t, int n, int dtype, int D, int block_q, int block_k,
                           const bsattn_tile_config& c) {
    for (int i = 0; i < n; ++i)
        if (legal(t[i], dtype, D, block_q, block_k) && matches(t[i], c)) return &t[i];
    return nullptr;
}

const Variant* find(int dtype, int D, int block_q, int block_k, const bsattn_tile_config& c) {
    int n = 0;
    const Variant* t = variants(dtype, &n);
    return first_match(t, n, dtype, D, block_q, block_k, c);
}

// Built-in default of table t when nothing is configured or tuned: for bf16 and
// 128-row mask blocks the row-pair kernel (two mask rows per 8-wave workgroup,
// each K/V tile loaded once for both; the autotuner's pick on every bf16 workload
// measured; rows of at most kPairMaxBlocks key blocks), with the key-tile depth
// in the given order of preference; else the first legal entry of the table.
const Variant* builtin_default(const Variant* t, int n, int dtype, int D, int block_q, int block_k,
                               int n_k, int tk_first, int tk_second) {
    if (dtype == BSATTN_BF16 && block_q == 128 && n_k <= kPairMaxBlocks) {
        for (int tk : {tk_first, tk_second})
            if (const Variant* v = first_match(t, n, dtype, D, block_q, block_k, bsattn_tile_config{256, tk, 8, 2}))
                return v;
    }
    return first_match(t, n, dtype, D, block_q, block_k, bsattn_tile_config{0, 0, 0, 0});
}

// ---- tuning cache -------------------------------------------------------------
// Key: dtype, D, block_q, block_k, S, B*H, and the mask statistic: the mean
// number of active key blocks per mask row in half-octaves,
// round(2 log2(nnz / rows)) (-1 for an empty mask).  Masks of one shape whose
// mean row lengths differ by more than about 41 % tune to separate entries.
typedef std::tuple<int, int, int, int, int, int64_t> ShapeKey;  // dtype, D, bq, bk, S, B*H
typedef std::tuple<int, int, int, int, int, int64_t, int> TuneKey;  // ShapeKey + mask bucket

int mask_bucket(int64_t nnz, int64_t rows) {
    if (nnz <= 0 || rows <= 0) return -1;
    return (int)std::lround(2.0 * std::log2((double)nnz / (double)rows));
}

ShapeKey shape_of(const TuneKey& k) {
    return ShapeKey(std::get<0>(k), std::get<1>(k), std::get<2>(k), std::get<3>(k), std::get<4>(k),
                    std::get<5>(k));
}

struct TuneEntry {
    bsattn_tile_config cfg;
    double t_mean_s;
};

std::mutex g_tune_mu;
std::map<TuneKey, TuneEntry> g_tune;

// A call that does not know its mask statistic (bsattn_fwd with an automatic
// config) takes the shape's entry of the densest mask bucket.  Caller holds
// g_tune_mu.
bool densest_entry(const ShapeKey& k, bsattn_tile_config* out) {
    auto it = g_tune.upper_bound(TuneKey(std::get<0>(k), std::get<1>(k), std::get<2>(k), std::get<3>(k),
                                         std::get<4>(k), std::get<5>(k), INT32_MAX));
    if (it == g_tune.begin()) return false;
    --it;
    if (shape_of(it->first) != k) return false;
    *out = it->second.cfg;
    return true;
}

bool tune_lookup_shape(const ShapeKey& key, bsattn_tile_config* out) {
    std::lock_guard<std::mutex> lk(g_tune_mu);
    return densest_entry(key, out);
}

bool json_number(const std::string& obj, const char* name, double* out) {
    const std::string pat = std::string("\"") + name + "\"";
    size_t p = obj.find(pat);
    if (p == std::string::npos) return false;
    p = obj.find(':', p + pat.size());
    if (p == std::string::npos) return false;
    const char* s = obj.c_str() + p + 1;
    char* end = nullptr;
    errno = 0;
    const double v = std::strtod(s, &end);
    if (end == s || errno) return false;
    *out = v;
    return true;
}

// Parse the entries of a cache file written by write_cache(); returns false if
// the file cannot be opened.
bool read_cache(const char* path, std::map<TuneKey, TuneEntry>* into) {
    FILE* f = std::fopen(path, "rb");
    if (!f) return false;
    std::string text;
    char buf[4096];
    size_t n;
    while ((n = std::fread(buf, 1, sizeof buf, f)) > 0) text.append(buf, n);
    std::fclose(f);
    size_t p = text.find("\"entries\"");
    if (p == std::string::npos) return true;
    while ((p = text.find('{', p + 1)) != std::string::npos) {
        const size_t e = text.find('}', p);
        if (e == std::string::npos) break;
        const std::string obj = text.substr(p, e - p + 1);
        double dt, D, bq, bk, S, BH, mb, tq, tk, w, st, tm = 0.0;
        if (json_number(obj, "dtype", &dt) && json_number(obj, "D", &D) &&
            json_number(obj, "block_q", &bq) && json_number(obj, "block_k", &bk) &&
            json_number(obj, "S", &S) && json_number(obj, "BH", &BH) &&
            json_number(obj, "mask_bucket", &mb) &&
            json_number(obj, "tile_q", &tq) && json_number(obj, "tile_k", &tk) &&
            json_number(obj, "waves", &w) && json_number(obj, "stages", &st)) {
            json_number(obj, "t_mean_s", &tm);
            TuneEntry te;
            te.cfg = bsattn_tile_config{(int)tq, (int)tk, (int)w, (int)st};
            te.t_mean_s = tm;
            (*into)[TuneKey((int)dt, (int)D, (int)bq, (int)bk, (int)S, (int64_t)BH, (int)mb)] = te;
        }
        p = e;
    }
    return true;
}

bool write_cache(const char* path, const std::map<TuneKey, TuneEntry>& m) {
    const std::string tmp = std::string(path) + ".tmp";
    FILE* f = std::fopen(tmp.c_str(), "wb");
    if (!f) return false;
    std::fprintf(f, "{\"bsattn_tune_cache\": 1, \"entries\": [\n");
    size_t i = 0;
    for (const auto& kv : m) {
        const TuneKey& k = kv.first;
        const TuneEntry& e = kv.second;
        std::fprintf(f,
                     "  {\"dtype\": %d, \"D\": %d, \"block_q\": %d, \"block_k\": %d, \"S\": %d, "
                     "\"BH\": %lld, \"mask_bucket\": %d, \"tile_q\": %d, \"tile_k\": %d, \"waves\": %d, "
                     "\"stages\": %d, \"t_mean_s\": %.6e}%s\n",
                     std::get<0>(k), std::get<1>(k), std::get<2>(k), std::get<3>(k),
                     std::get<4>(k), (long long)std::get<5>(k), std::get<6>(k), e.cfg.tile_q, e.cfg.tile_k,
                     e.cfg.waves, e.cfg.stages, e.t_mean_s, (++i < m.size()) ? "," : "");
    }
    std::fprintf(f, "]}\n");
    const bool ok = std::fclose(f) == 0;
    return ok && std::rename(tmp.c_str(), path) == 0;
}

bool env_config(bsattn_tile_config* c, bool* bad) {
    *bad = false;
    const char* s = std::getenv("BSATTN_CONFIG");
    if (!s || !*s) return false;
    int v[4] = {0, 0, 0, 0};
    if (std::sscanf(s, "%d,%d,%d,%d", &v[0], &v[1], &v[2], &v[3]) != 4) {
        *bad = true;
        return false;
    }
    *c = bsattn_tile_config{v[0], v[1], v[2], v[3]};
    return true;
}

// Choose the variant for a call: explicit config, else BSATTN_CONFIG, else the
// tuning cache, else the built-in default (128-key steps first for D = 128, 64-key
// steps first for D = 64: the tuned picks of the dense, causal and sparse shapes
// and of the long-context one).
const Variant* choose(int dtype, int D, int S, int64_t BH, int block_q, int block_k,
                      const bsattn_tile_config* cfg) {
    if (!is_auto(cfg)) return find(dtype, D, block_q, block_k, *cfg);
    bsattn_tile_config c{0, 0, 0, 0};
    bool bad = false;
    if (env_config(&c, &bad)) return find(dtype, D, block_q, block_k, c);
    if (bad) return nullptr;
    if (tune_lookup_shape(ShapeKey(dtype, D, block_q, block_k, S, BH), &c)) {
        const Variant* v = find(dtype, D, block_q, block_k, c);
        if (v) return v;
    }
    int n = 0;
    const Variant* t = variants(dtype, &n);
    return builtin_default(t, n, dtype, D, block_q, block_k, S / block_k, D == 128 ? 128 : 64,
                           D == 128 ? 64 : 128);
}

FwdArgs make_args(const void* q, const void* k, const void* v, void* out, float* lse, int H,
                  int S, int block_q, int block_k, float scale, const Variant& var) {
    FwdArgs a;
    std::memset(&a, 0, sizeof a);
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.lse = lse;
    a.H = H;
    a.S = S;
    a.n_q = S / block_q;
    a.n_k = S / block_k;
    a.block_q = block_q;
    a.block_k = block_k;
    a.sub_per_row = is_pair(var) ? 1 : block_q / var.tile_q;
    a.sub_log2 = 0;
    while ((1 << a.sub_log2) < a.sub_per_row) ++a.sub_log2;
    a.steps_log2 = 0;
    while ((var.tile_k << a.steps_log2) < block_k) ++a.steps_log2;
    const bool neg = std::signbit(scale) && scale != 0.0f;
    a.c = std::fabs(scale) * kLog2e;
    // A zero scale makes every score 0: a uniform softmax over the kept keys.  The
    // kernels get the smallest normal float instead, so an element mask's dropped
    // score (-inf) times c stays -inf rather than NaN, while for any |q . k| < 2^100
    // c * (q . k) stays below 2^-26 and every exponent still rounds to exactly 1.
    if (a.c == 0.0f) a.c = FLT_MIN;
    a.qsign = neg ? 0x80008000u : 0u;
    a.qsign32 = neg ? 0x80000000u : 0u;
    return a;
}

int run_attention(const FwdArgs& a, const Variant& var, hipStream_t stream) {
    const int64_t grid = 8 * (int64_t)a.chunk * a.sub_per_row;
    if (a.nrows <= 0 || (1 << a.sub_log2) != a.sub_per_row || grid >= ((int64_t)1 << 31))
        return BSATTN_ERR_SHAPE;
    const hipError_t e = var.launch(a, (unsigned)grid, stream);
    if (e != hipSuccess) return hip_fail(e);
    return BSATTN_OK;
}

// ---- element-level masks ------------------------------------------------------

// A partial block's tile index travels in bits 16..30 of its list entry (kj in
// bits 0..15), so n_k <= 65536 and 1 <= n_tiles <= 32767.
constexpr int kElemMaxTiles = 32767;

int check_elem_shape(int B, int H, int S, int block_q, int block_k, int n_tiles) {
    if (B <= 0 || H <= 0 || S <= 0 || block_q <= 0 || block_k <= 0) return BSATTN_ERR_SHAPE;
    if (S % block_q != 0 || S % block_k != 0) return BSATTN_ERR_SHAPE;
    if (!block_ok(block_q) || !block_ok(block_k)) return BSATTN_ERR_UNSUPPORTED;
    if (n_tiles < 1 || n_tiles > kElemMaxTiles || S / block_k > 65536) return BSATTN_ERR_SHAPE;
    return check_grid(B, H, S / block_q, S / block_k);
}

// Element masks: an explicit config, else the built-in default (64-key row-pair
// steps first: the pick on the token-causal shape).
const Variant* find_elem(int dtype, int D, int S, int block_q, int block_k, const bsattn_tile_config* cfg) {
    if (dtype != BSATTN_BF16 && dtype != BSATTN_F32) return nullptr;
    int n = 0;
    const Variant* t = dtype == BSATTN_BF16 ? bf16_elem_variants(&n) : f32_elem_variants(&n);
    if (is_auto(cfg)) return builtin_default(t, n, dtype, D, block_q, block_k, S / block_k, 64, 128);
    return first_match(t, n, dtype, D, block_q, block_k, *cfg);
}

// The fp8 workspace: the forward plan, then V rearranged per 64-key tile (B*H*S*D
// bytes, rewritten by every call).
struct Fp8Layout {
    PlanLayout plan;
    size_t vt, bytes;
};

Fp8Layout fp8_layout(int64_t BH, int S, int D, int n_q, int n_k) {
    Fp8Layout L;
    L.plan = plan_layout(BH, n_q, n_k);
    L.vt = L.plan.bytes;
    L.bytes = L.vt + align_up((size_t)(BH * S) * D);
    return L;
}

const Variant* fp8_find(int D, int block_q, bool elem = false) {
    int n = 0;
    const Variant* t = elem ? fp8_elem_variants(&n) : fp8_variants(&n);
    for (int i = 0; i < n; ++i)
        if (t[i].D == D && t[i].tile_q == block_q) return &t[i];
    return nullptr;
}

// Checks of the fp8 forward's tensors (q, k, v e4m3; out bf16; lse fp32).
int check_fp8_buffers(const void* q, const void* k, const void* v, const void* out, const float* lse, int B,
                      int H, int S, int D, int block_q, int block_k, float scale) {
    if (!q || !k || !v || !out || !lse) return BSATTN_ERR_NULL;
    const int rc = check_fwd_shape(B, H, S, D, block_q, block_k, BSATTN_BF16);
    if (rc) return rc;
    if (!is_aligned(q, 16) || !is_aligned(k, 16) || !is_aligned(v, 16) || !is_aligned(out, 16) ||
        !is_aligned(lse, 4))
        return BSATTN_ERR_ALIGN;
    if (!std::isfinite(scale)) return BSATTN_ERR_SCALE;
    const size_t n8 = (size_t)B * H * S * D, no = n8 * 2, nl = (size_t)B * H * S * 4;
    if (overlap(out, no, q, n8) || overlap(out, no, k, n8) || overlap(out, no, v, n8) || overlap(lse, nl, q, n8) ||
        overlap(lse, nl, k, n8) || overlap(lse, nl, v, n8) || overlap(lse, nl, out, no))
        return BSATTN_ERR_ALIAS;
    return BSATTN_OK;
}


// ---- forward with no allocation: the plan in a fixed device array ----------------
// For callers that cannot allocate (graph capture, tight serving loops): the
// forward's plan lives in this file-scope device array instead of a caller
// workspace.  Each GPU the library runs on holds its own copy until the process
// ends.  In host code `scratch` only names the symbol; its device address (one
// per GPU) comes from hipGetSymbolAddress, taken once per device with that device
// current and kept in g_scratch_ptr.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's address on the calling thread's current device.
int scratch_on_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= kMaxDevices) return BSATTN_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e);
        if (!p) return hip_fail(hipErrorInvalidSymbol);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return BSATTN_OK;
}

}  // namespace

extern "C" {

int bsattn_version(void) { return (0 << 16) | (1 << 8) | 0; }

const char* bsattn_status_string(int status) {
    switch (status) {
        case BSATTN_OK: return "BSATTN_OK: success";
        case BSATTN_ERR_NULL: return "BSATTN_ERR_NULL: a required pointer is NULL";
        case BSATTN_ERR_SHAPE:
            return "BSATTN_ERR_SHAPE: a size is <= 0, S is not divisible by a block size, "
                   "or an index would overflow";
        case BSATTN_ERR_UNSUPPORTED:
            return "BSATTN_ERR_UNSUPPORTED: head dim, dtype, block size or tile config not built";
        case BSATTN_ERR_ALIGN:
            return "BSATTN_ERR_ALIGN: q/k/v/out must be 16-byte and lse 4-byte aligned";
        case BSATTN_ERR_WORKSPACE: return "BSATTN_ERR_WORKSPACE: workspace missing or too small";
        case BSATTN_ERR_SCALE: return "BSATTN_ERR_SCALE: scale is not finite";
        case BSATTN_ERR_ALIAS: return "BSATTN_ERR_ALIAS: an output overlaps an input or the other output";
        case BSATTN_ERR_HIP: return "BSATTN_ERR_HIP: a HIP runtime call failed";
        case BSATTN_ERR_IO: return "BSATTN_ERR_IO: a tuning-cache file could not be read or written";
        default: return "BSATTN: unknown status";
    }
}

int bsattn_last_hip_error(void) { return g_last_hip; }

int bsattn_compact_workspace_size(int B, int H, int n_q, int n_k, size_t* bytes) {
    if (!bytes) return BSATTN_ERR_NULL;
    const int rc = check_grid(B, H, n_q, n_k);
    if (rc) return rc;
    *bytes = compact_ws_bytes((int64_t)B * H * n_q, n_k);
    return BSATTN_OK;
}

int bsattn_compact_mask(const uint8_t* block_mask, int B, int H, int n_q, int n_k,
                        int32_t* row_ptr, int32_t* col_idx, void* workspace,
                        size_t workspace_bytes, void* stream) {
    if (!block_mask || !row_ptr || !col_idx) return BSATTN_ERR_NULL;
    int rc = check_grid(B, H, n_q, n_k);
    if (rc) return rc;
    const int64_t R = (int64_t)B * H * n_q;
    if (!workspace || workspace_bytes < compact_ws_bytes(R, n_k)) return BSATTN_ERR_WORKSPACE;
    if (!is_aligned(row_ptr, 4) || !is_aligned(col_idx, 4) || !is_aligned(workspace, 4))
        return BSATTN_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    int32_t* counts = (int32_t*)workspace;
    int32_t* lists = (int32_t*)((char*)workspace + align_up((size_t)R * 4));
    hipError_t e = launch_compact_rows(block_mask, R, n_k, counts, lists, s);
    if (e != hipSuccess) return hip_fail(e);
    e = launch_compact_scan(counts, R, row_ptr, s);
    if (e != hipSuccess) return hip_fail(e);
    e = launch_compact_pack(counts, lists, R, n_k, row_ptr, col_idx, s);
    if (e != hipSuccess) return hip_fail(e);
    return BSATTN_OK;
}

int bsattn_workspace_size(int B, int H, int S, int block_q, int block_k, size_t* bytes) {
    if (!bytes) return BSATTN_ERR_NULL;
    if (B <= 0 || H <= 0 || S <= 0 || block_q <= 0 || block_k <= 0) return BSATTN_ERR_SHAPE;
    if (S % block_q != 0 || S % block_k != 0) return BSATTN_ERR_SHAPE;
    const int rc = check_grid(B, H, S / block_q, S / block_k);
    if (rc) return rc;
    *bytes = fwd_ws_bytes((int64_t)B * H, S / block_q, S / block_k);
    return BSATTN_OK;
}

int bsattn_plan(const uint8_t* block_mask, int B, int H, int S, int block_q, int block_k,
                void* workspace, size_t workspace_bytes, void* stream) {
    if (!block_mask || !workspace) return BSATTN_ERR_NULL;
    if (B <= 0 || H <= 0 || S <= 0 || block_q <= 0 || block_k <= 0) return BSATTN_ERR_SHAPE;
    if (S % block_q != 0 || S % block_k != 0) return BSATTN_ERR_SHAPE;
    if (!block_ok(block_q) || !block_ok(block_k)) return BSATTN_ERR_UNSUPPORTED;
    const int n_q = S / block_q, n_k = S / block_k;
    int rc = check_grid(B, H, n_q, n_k);
    if (rc) return rc;
    const PlanLayout L = plan_layout((int64_t)B * H, n_q, n_k);
    if (workspace_bytes < L.bytes) return BSATTN_ERR_WORKSPACE;
    if (!is_aligned(workspace, 4)) return BSATTN_ERR_ALIGN;
    if (overlap(workspace, L.bytes, block_mask, (size_t)L.R * n_k)) return BSATTN_ERR_ALIAS;
    hipStream_t s = (hipStream_t)stream;
    char* ws = (char*)workspace;
    int32_t* counts = (int32_t*)ws;
    const hipError_t e = launch_plan(block_mask, L.R, n_q, n_k, counts, (int32_t*)(ws + L.lists),
                                     L.chunk, (int32_t*)(ws + L.order), L.pchunk,
                                     (int32_t*)(ws + L.porder), s);
    if (e != hipSuccess) return hip_fail(e);
    return BSATTN_OK;
}

int bsattn_fwd_planned(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                       int H, int S, int D, int block_q, int block_k, float scale, int dtype,
                       const void* workspace, size_t workspace_bytes,
                       const bsattn_tile_config* cfg, void* stream) {
    if (!workspace) return BSATTN_ERR_NULL;
    const int rc = check_fwd_buffers(q, k, v, out, lse, B, H, S, D, block_q, block_k, dtype, scale);
    if (rc) return rc;
    const int n_q = S / block_q, n_k = S / block_k;
    const PlanLayout L = plan_layout((int64_t)B * H, n_q, n_k);
    if (workspace_bytes < L.bytes) return BSATTN_ERR_WORKSPACE;
    if (!is_aligned(workspace, 4)) return BSATTN_ERR_ALIGN;
    if (check_ws_alias(workspace, L.bytes, q, k, v, out, lse, B, H, S, D, dtype))
        return BSATTN_ERR_ALIAS;
    const Variant* var = choose(dtype, D, S, (int64_t)B * H, block_q, block_k, cfg);
    if (!var) return BSATTN_ERR_UNSUPPORTED;
    if (is_pair(*var) && n_k > kPairMaxBlocks) return BSATTN_ERR_UNSUPPORTED;
    FwdArgs a = make_args(q, k, v, out, lse, H, S, block_q, block_k, scale, *var);
    const char* ws = (const char*)workspace;
    a.counts = (const int32_t*)ws;
    a.list = (const int32_t*)(ws + L.lists);
    a.ell_stride = n_k;
    if (is_pair(*var)) {
        a.order = (const int32_t*)(ws + L.porder);
        a.nrows = (int)L.P;
        a.chunk = (int)L.pchunk;
    } else {
        a.order = (const int32_t*)(ws + L.order);
        a.nrows = (int)L.R;
        a.chunk = (int)L.chunk;
    }
    return run_attention(a, *var, (hipStream_t)stream);
}

int bsattn_fwd_config(const void* q, const void* k, const void* v, const uint8_t* block_mask,
                      void* out, float* lse, int B, int H, int S, int D, int block_q,
                      int block_k, float scale, int dtype, void* workspace,
                      size_t workspace_bytes, const bsattn_tile_config* cfg, void* stream) {
    if (!block_mask) return BSATTN_ERR_NULL;
    const int rc = check_fwd_buffers(q, k, v, out, lse, B, H, S, D, block_q, block_k, dtype, scale);
    if (rc) return rc;
    const size_t need = fwd_ws_bytes((int64_t)B * H, S / block_q, S / block_k);
    if (!workspace || workspace_bytes < need) return BSATTN_ERR_WORKSPACE;
    if (!is_aligned(workspace, 4)) return BSATTN_ERR_ALIGN;
    if (check_ws_alias(workspace, need, q, k, v, out, lse, B, H, S, D, dtype))
        return BSATTN_ERR_ALIAS;
    // Resolve the tile config before any device work, so an unsupported one
    // fails with nothing enqueued.
    const Variant* var = choose(dtype, D, S, (int64_t)B * H, block_q, block_k, cfg);
    if (!var || (is_pair(*var) && S / block_k > kPairMaxBlocks)) return BSATTN_ERR_UNSUPPORTED;
    int st = bsattn_plan(block_mask, B, H, S, block_q, block_k, workspace, workspace_bytes, stream);
    if (st) return st;
    return bsattn_fwd_planned(q, k, v, out, lse, B, H, S, D, block_q, block_k, scale, dtype,
                              workspace, workspace_bytes, cfg, stream);
}

int bsattn_fwd(const void* q, const void* k, const void* v, const uint8_t* block_mask,
               void* out, float* lse, int B, int H, int S, int D, int block_q, int block_k,
               float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
    return bsattn_fwd_config(q, k, v, block_mask, out, lse, B, H, S, D, block_q, block_k, scale,
                             dtype, workspace, workspace_bytes, nullptr, stream);
}

size_t bsattn_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

int bsattn_fwd_noalloc(const void* q, const void* k, const void* v, const uint8_t* block_mask,
                       void* out, float* lse, int B, int H, int S, int D, int block_q, int block_k,
                       float scale, int dtype, const bsattn_tile_config* cfg, void* stream) {
    if (!block_mask) return BSATTN_ERR_NULL;
    int rc = check_fwd_buffers(q, k, v, out, lse, B, H, S, D, block_q, block_k, dtype, scale);
    if (rc) return rc;
    if (fwd_ws_bytes((int64_t)B * H, S / block_q, S / block_k) > kNoAllocScratchBytes)
        return BSATTN_ERR_WORKSPACE;
    // Resolve the tile config before any device work.
    const Variant* var = choose(dtype, D, S, (int64_t)B * H, block_q, block_k, cfg);
    if (!var || (is_pair(*var) && S / block_k > kPairMaxBlocks)) return BSATTN_ERR_UNSUPPORTED;
    void* ws = nullptr;
    rc = scratch_on_current_device(&ws);
    if (rc) return rc;
    // The plan launch rewrites every byte the attention launch reads.
    rc = bsattn_plan(block_mask, B, H, S, block_q, block_k, ws, kNoAllocScratchBytes, stream);
    if (rc) return rc;
    return bsattn_fwd_planned(q, k, v, out, lse, B, H, S, D, block_q, block_k, scale, dtype, ws,
                              kNoAllocScratchBytes, cfg, stream);
}

int bsattn_fwd_compacted(const void* q, const void* k, const void* v, const int32_t* row_ptr,
                         const int32_t* col_idx, size_t col_idx_len, void* out, float* lse, int B,
                         int H, int S, int D, int block_q, int block_k, float scale, int dtype,
                         const bsattn_tile_config* cfg, void* stream) {
    if (!row_ptr || !col_idx) return BSATTN_ERR_NULL;
    const int rc = check_fwd_buffers(q, k, v, out, lse, B, H, S, D, block_q, block_k, dtype, scale);
    if (rc) return rc;
    if (!is_aligned(row_ptr, 4) || !is_aligned(col_idx, 4)) return BSATTN_ERR_ALIGN;
    const Variant* var = choose(dtype, D, S, (int64_t)B * H, block_q, block_k, cfg);
    if (!var) return BSATTN_ERR_UNSUPPORTED;
    if (is_pair(*var) && S / block_k > kPairMaxBlocks) return BSATTN_ERR_UNSUPPORTED;
    const PlanLayout L = plan_layout((int64_t)B * H, S / block_q, S / block_k);
    FwdArgs a = make_args(q, k, v, out, lse, H, S, block_q, block_k, scale, *var);
    a.row_ptr = row_ptr;
    a.list = col_idx;
    a.list_len = (int64_t)std::min<size_t>(col_idx_len, (size_t)INT32_MAX);  // row_ptr values are int32
    a.ell_stride = 0;
    a.nrows = (int)(is_pair(*var) ? L.P : L.R);
    a.chunk = (int)xcd_chunk(a.nrows);
    return run_attention(a, *var, (hipStream_t)stream);
}

// ---- element-level masks ------------------------------------------------------

int bsattn_plan_elem(const uint8_t* block_states, const int32_t* partial_index, int n_tiles, int B,
                     int H, int S, int block_q, int block_k, void* workspace,
                     size_t workspace_bytes, void* stream) {
    if (!block_states || !partial_index || !workspace) return BSATTN_ERR_NULL;
    const int rc = check_elem_shape(B, H, S, block_q, block_k, n_tiles);
    if (rc) return rc;
    const int n_q = S / block_q, n_k = S / block_k;
    const PlanLayout L = plan_layout((int64_t)B * H, n_q, n_k);
    if (workspace_bytes < L.bytes) return BSATTN_ERR_WORKSPACE;
    if (!is_aligned(workspace, 4) || !is_aligned(partial_index, 4)) return BSATTN_ERR_ALIGN;
    if (overlap(workspace, L.bytes, block_states, (size_t)L.R * n_k) ||
        overlap(workspace, L.bytes, partial_index, (size_t)L.R * n_k * 4))
        return BSATTN_ERR_ALIAS;
    hipStream_t s = (hipStream_t)stream;
    char* ws = (char*)workspace;
    int32_t* counts = (int32_t*)ws;
    hipError_t e = launch_compact_rows_elem(block_states, partial_index, n_tiles, L.R, n_k, counts,
                                            (int32_t*)(ws + L.lists), s);
    if (e != hipSuccess) return hip_fail(e);
    e = launch_compact_order(counts, L.R, n_q, n_k, L.chunk, (int32_t*)(ws + L.order), L.pchunk,
                             (int32_t*)(ws + L.porder), s);
    if (e != hipSuccess) return hip_fail(e);
    return BSATTN_OK;
}

int bsattn_fwd_planned_elem(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                            int H, int S, int D, int block_q, int block_k, float scale, int dtype,
                            const uint32_t* partial_bits, int n_tiles, const void* workspace,
                            size_t workspace_bytes, const bsattn_tile_config* cfg, void* stream) {
    if (!workspace || !partial_bits) return BSATTN_ERR_NULL;
    int rc = check_fwd_buffers(q, k, v, out, lse, B, H, S, D, block_q, block_k, dtype, scale);
    if (rc) return rc;
    rc = check_elem_shape(B, H, S, block_q, block_k, n_tiles);
    if (rc) return rc;
    const int n_q = S / block_q, n_k = S / block_k;
    const PlanLayout L = plan_layout((int64_t)B * H, n_q, n_k);
    if (workspace_bytes < L.bytes) return BSATTN_ERR_WORKSPACE;
    if (!is_aligned(workspace, 4) || !is_aligned(partial_bits, 4)) return BSATTN_ERR_ALIGN;
    if (check_ws_alias(workspace, L.bytes, q, k, v, out, lse, B, H, S, D, dtype))
        return BSATTN_ERR_ALIAS;
    const size_t nbits = (size_t)n_tiles * block_q * (block_k / 8);
    const size_t nt = (size_t)B * H * S * D * (dtype == BSATTN_F32 ? 4 : 2);
    if (overlap(partial_bits, nbits, out, nt) || overlap(partial_bits, nbits, lse, (size_t)B * H * S * 4) ||
        overlap(partial_bits, nbits, workspace, L.bytes))
        return BSATTN_ERR_ALIAS;
    const Variant* var = find_elem(dtype, D, S, block_q, block_k, cfg);
    if (!var) return BSATTN_ERR_UNSUPPORTED;
    if (is_pair(*var) && n_k > kPairMaxBlocks) return BSATTN_ERR_UNSUPPORTED;
    FwdArgs a = make_args(q, k, v, out, lse, H, S, block_q, block_k, scale, *var);
    const char* ws = (const char*)workspace;
    a.counts = (const int32_t*)ws;
    a.list = (const int32_t*)(ws + L.lists);
    a.ell_stride = n_k;
    if (is_pair(*var)) {
        a.order = (const int32_t*)(ws + L.porder);
        a.nrows = (int)L.P;
        a.chunk = (int)L.pchunk;
    } else {
        a.order = (const int32_t*)(ws + L.order);
        a.nrows = (int)L.R;
        a.chunk = (int)L.chunk;
    }
    a.pbits = partial_bits;
    a.n_tiles = n_tiles;
    return run_attention(a, *var, (hipStream_t)stream);
}

int bsattn_fwd_elem(const void* q, const void* k, const void* v, const uint8_t* block_states,
                    const int32_t* partial_index, const uint32_t* partial_bits, int n_tiles, void* out,
                    float* lse, int B, int H, int S, int D, int block_q, int block_k, float scale,
                    int dtype, void* workspace, size_t workspace_bytes,
                    const bsattn_tile_config* cfg, void* stream) {
    if (!block_states || !partial_index || !partial_bits) return BSATTN_ERR_NULL;
    int rc = check_fwd_buffers(q, k, v, out, lse, B, H, S, D, block_q, block_k, dtype, scale);
    if (rc) return rc;
    rc = check_elem_shape(B, H, S, block_q, block_k, n_tiles);
    if (rc) return rc;
    const size_t need = fwd_ws_bytes((int64_t)B * H, S / block_q, S / block_k);
    if (!workspace || workspace_bytes < need) return BSATTN_ERR_WORKSPACE;
    if (!is_aligned(workspace, 4) || !is_aligned(partial_bits, 4) || !is_aligned(partial_index, 4))
        return BSATTN_ERR_ALIGN;
    if (check_ws_alias(workspace, need, q, k, v, out, lse, B, H, S, D, dtype)) return BSATTN_ERR_ALIAS;
    {
        const size_t nbits = (size_t)n_tiles * block_q * (block_k / 8);
        const size_t nt = (size_t)B * H * S * D * (dtype == BSATTN_F32 ? 4 : 2);
        if (overlap(partial_bits, nbits, out, nt) || overlap(partial_bits, nbits, lse, (size_t)B * H * S * 4) ||
            overlap(partial_bits, nbits, workspace, need))
            return BSATTN_ERR_ALIAS;
    }
    // Resolve the tile config before any device work.
    const Variant* var = find_elem(dtype, D, S, block_q, block_k, cfg);
    if (!var || (is_pair(*var) && S / block_k > kPairMaxBlocks)) return BSATTN_ERR_UNSUPPORTED;
    rc = bsattn_plan_elem(block_states, partial_index, n_tiles, B, H, S, block_q, block_k, workspace,
                          workspace_bytes, stream);
    if (rc) return rc;
    return bsattn_fwd_planned_elem(q, k, v, out, lse, B, H, S, D, block_q, block_k, scale, dtype,
                                   partial_bits, n_tiles, workspace, workspace_bytes, cfg, stream);
}

int bsattn_list_configs_elem(int dtype, int D, int block_q, int block_k, bsattn_tile_config* cfgs,
                             int cap, int* n) {
    if (!n) return BSATTN_ERR_NULL;
    if (dtype != BSATTN_F32 && dtype != BSATTN_BF16) return BSATTN_ERR_UNSUPPORTED;
    int cnt = 0, nv = 0;
    const Variant* t = dtype == BSATTN_BF16 ? bf16_elem_variants(&nv) : f32_elem_variants(&nv);
    for (int i = 0; i < nv; ++i) {
        if (!legal(t[i], dtype, D, block_q, block_k)) continue;
        if (cfgs && cnt < cap) cfgs[cnt] = bsattn_tile_config{t[i].tile_q, t[i].tile_k, t[i].waves, t[i].stages};
        ++cnt;
    }
    *n = cnt;
    return BSATTN_OK;
}

// ---- ragged dot ------------------------------------------------------------------

// Compute units of the current device, cached per device (0 if the query fails:
// the ragged dot then runs in one launch).
int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// The plan's item count is an int32 (and every item index fits one).
static bool ragged_items_ok(int M, int G) { return ragged_max_items(M, G) < ((int64_t)1 << 30); }

int bsattn_ragged_dot_workspace_size(int M, int G, size_t* bytes) {
    if (!bytes) return BSATTN_ERR_NULL;
    if (M <= 0 || G <= 0 || !ragged_items_ok(M, G)) return BSATTN_ERR_SHAPE;
    *bytes = ragged_ws_bytes(M, G);
    return BSATTN_OK;
}

int bsattn_ragged_plan(const int32_t* group_sizes, int M, int G, void* workspace,
                       size_t workspace_bytes, void* stream) {
    if (!group_sizes || !workspace) return BSATTN_ERR_NULL;
    if (M <= 0 || G <= 0 || !ragged_items_ok(M, G)) return BSATTN_ERR_SHAPE;
    if (workspace_bytes < ragged_ws_bytes(M, G)) return BSATTN_ERR_WORKSPACE;
    if (!is_aligned(group_sizes, 4) || !is_aligned(workspace, 16)) return BSATTN_ERR_ALIGN;
    if (overlap(workspace, ragged_ws_bytes(M, G), group_sizes, (size_t)G * 4)) return BSATTN_ERR_ALIAS;
    const hipError_t e = launch_ragged_plan(group_sizes, M, G, workspace, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    return BSATTN_OK;
}

int bsattn_ragged_dot_planned(const void* lhs, const void* rhs, void* out, int M, int K, int N, int G,
                              int dtype, int out_dtype, const void* workspace, size_t workspace_bytes,
                              void* stream) {
    if (!lhs || !rhs || !out || !workspace) return BSATTN_ERR_NULL;
    if (M <= 0 || K <= 0 || N <= 0 || G <= 0) return BSATTN_ERR_SHAPE;
    if (K % 64 != 0 || N % 128 != 0) return BSATTN_ERR_SHAPE;
    if ((int64_t)K * N * 2 >= ((int64_t)1 << 31)) return BSATTN_ERR_SHAPE;  // one expert per buffer
    if (ragged_max_items(M, G) * 2 * (N / 128) >= ((int64_t)1 << 31)) return BSATTN_ERR_SHAPE;
    if (dtype != BSATTN_BF16) return BSATTN_ERR_UNSUPPORTED;
    if (out_dtype != BSATTN_BF16 && out_dtype != BSATTN_F32) return BSATTN_ERR_UNSUPPORTED;
    const size_t nw = ragged_ws_bytes(M, G);
    if (workspace_bytes < nw) return BSATTN_ERR_WORKSPACE;
    if (!is_aligned(lhs, 16) || !is_aligned(rhs, 16) || !is_aligned(out, 16) || !is_aligned(workspace, 16))
        return BSATTN_ERR_ALIGN;
    const size_t nl = (size_t)M * K * 2, nr = (size_t)G * K * N * 2;
    const size_t no = (size_t)M * N * (out_dtype == BSATTN_F32 ? 4 : 2);
    if (overlap(out, no, lhs, nl) || overlap(out, no, rhs, nr) || overlap(out, no, workspace, nw) ||
        overlap(workspace, nw, lhs, nl) || overlap(workspace, nw, rhs, nr))
        return BSATTN_ERR_ALIAS;
    const hipError_t e = launch_ragged_planned(lhs, rhs, out, M, K, N, G, out_dtype == BSATTN_F32, workspace,
                                               device_cu_count(), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    return BSATTN_OK;
}

int bsattn_ragged_dot(const void* lhs, const void* rhs, const int32_t* group_sizes, void* out, int M,
                      int K, int N, int G, int dtype, int out_dtype, void* workspace,
                      size_t workspace_bytes, void* stream) {
    if (!lhs || !rhs || !group_sizes || !out || !workspace) return BSATTN_ERR_NULL;
    if (M <= 0 || K <= 0 || N <= 0 || G <= 0) return BSATTN_ERR_SHAPE;
    if (K % 64 != 0 || N % 128 != 0) return BSATTN_ERR_SHAPE;
    if ((int64_t)K * N * 2 >= ((int64_t)1 << 31)) return BSATTN_ERR_SHAPE;
    if (ragged_max_items(M, G) * 2 * (N / 128) >= ((int64_t)1 << 31)) return BSATTN_ERR_SHAPE;
    if (dtype != BSATTN_BF16) return BSATTN_ERR_UNSUPPORTED;
    if (out_dtype != BSATTN_BF16 && out_dtype != BSATTN_F32) return BSATTN_ERR_UNSUPPORTED;
    const size_t nw = ragged_ws_bytes(M, G);
    if (workspace_bytes < nw) return BSATTN_ERR_WORKSPACE;
    if (!is_aligned(lhs, 16) || !is_aligned(rhs, 16) || !is_aligned(out, 16) ||
        !is_aligned(group_sizes, 4) || !is_aligned(workspace, 16))
        return BSATTN_ERR_ALIGN;
    const size_t no = (size_t)M * N * (out_dtype == BSATTN_F32 ? 4 : 2), ng = (size_t)G * 4;
    if (overlap(out, no, group_sizes, ng)) return BSATTN_ERR_ALIAS;
    const size_t nl = (size_t)M * K * 2, nr = (size_t)G * K * N * 2;
    if (overlap(out, no, lhs, nl) || overlap(out, no, rhs, nr) || overlap(out, no, workspace, nw) ||
        overlap(workspace, nw, lhs, nl) || overlap(workspace, nw, rhs, nr) ||
        overlap(workspace, nw, group_sizes, ng))
        return BSATTN_ERR_ALIAS;
    int rc = bsattn_ragged_plan(group_sizes, M, G, workspace, workspace_bytes, stream);
    if (rc) return rc;
    return bsattn_ragged_dot_planned(lhs, rhs, out, M, K, N, G, dtype, out_dtype, workspace, workspace_bytes,
                                     stream);
}

// ---- fp8 forward -----------------------------------------------------------------

int bsattn_fp8_workspace_size(int B, int H, int S, int D, int block_q, int block_k, size_t* bytes) {
    if (!bytes) return BSATTN_ERR_NULL;
    if (B <= 0 || H <= 0 || S <= 0 || D <= 0 || block_q <= 0 || block_k <= 0) return BSATTN_ERR_SHAPE;
    if (S % block_q != 0 || S % block_k != 0) return BSATTN_ERR_SHAPE;
    const int rc = check_grid(B, H, S / block_q, S / block_k);
    if (rc) return rc;
    *bytes = fp8_layout((int64_t)B * H, S, D, S / block_q, S / block_k).bytes;
    return BSATTN_OK;
}

// Checks shared by the fp8 entry points, all on the host: tensors and shape; with
// bit tiles (element masks) the element-mask shape and the tiles' alignment; then the
// workspace (size, alignment, no overlap with any tensor or with the bit tiles) and
// the config.  Fills *L.
int check_fp8_call(const void* q, const void* k, const void* v, const void* out, const float* lse, int B, int H,
                   int S, int D, int block_q, int block_k, float scale, const void* workspace,
                   size_t workspace_bytes, const uint32_t* bits, int n_tiles, Fp8Layout* L) {
    int rc = check_fp8_buffers(q, k, v, out, lse, B, H, S, D, block_q, block_k, scale);
    if (rc) return rc;
    if (bits) {
        rc = check_elem_shape(B, H, S, block_q, block_k, n_tiles);
        if (rc) return rc;
    }
    *L = fp8_layout((int64_t)B * H, S, D, S / block_q, S / block_k);
    if (workspace_bytes < L->bytes) return BSATTN_ERR_WORKSPACE;
    if (!is_aligned(workspace, 16) || (bits && !is_aligned(bits, 4))) return BSATTN_ERR_ALIGN;
    const size_t n8 = (size_t)B * H * S * D, no = n8 * 2, nl = (size_t)B * H * S * 4;
    const void* ts[] = {q, k, v, out, lse};
    const size_t tn[] = {n8, n8, n8, no, nl};
    for (int i = 0; i < 5; ++i)
        if (overlap(workspace, L->bytes, ts[i], tn[i])) return BSATTN_ERR_ALIAS;
    if (bits) {
        const size_t nbits = (size_t)n_tiles * block_q * (block_k / 8);
        if (overlap(bits, nbits, out, no) || overlap(bits, nbits, lse, nl) || overlap(bits, nbits, workspace, L->bytes))
            return BSATTN_ERR_ALIAS;
    }
    return fp8_find(D, block_q, bits != nullptr) ? BSATTN_OK : BSATTN_ERR_UNSUPPORTED;
}

// The V pre-pass, then the fp8 attention kernel on the plan in the workspace (bit
// tiles: the element-mask kernel).
int run_fp8(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int S, int D,
            int block_q, int block_k, float scale, void* workspace, const Fp8Layout& L, const uint32_t* bits,
            int n_tiles, hipStream_t st) {
    const Variant* var = fp8_find(D, block_q, bits != nullptr);
    char* ws = (char*)workspace;
    const hipError_t e = launch_fp8_vt(v, ws + L.vt, (int64_t)B * H * S / 64, D, st);
    if (e != hipSuccess) return hip_fail(e);
    FwdArgs a = make_args(q, k, ws + L.vt, out, lse, H, S, block_q, block_k, scale, *var);
    a.qsign = a.qsign ? 0x80808080u : 0u;  // the sign bit of each of four e4m3 bytes
    a.counts = (const int32_t*)ws;
    a.list = (const int32_t*)(ws + L.plan.lists);
    a.ell_stride = S / block_k;
    a.order = (const int32_t*)(ws + L.plan.order);
    a.nrows = (int)L.plan.R;
    a.chunk = (int)L.plan.chunk;
    if (bits) {
        a.pbits = bits;
        a.n_tiles = n_tiles;
    }
    return run_attention(a, *var, st);
}

int bsattn_fwd_fp8_planned(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                           int S, int D, int block_q, int block_k, float scale, void* workspace,
                           size_t workspace_bytes, void* stream) {
    if (!workspace) return BSATTN_ERR_NULL;
    Fp8Layout L;
    const int rc = check_fp8_call(q, k, v, out, lse, B, H, S, D, block_q, block_k, scale, workspace,
                                  workspace_bytes, nullptr, 0, &L);
    if (rc) return rc;
    return run_fp8(q, k, v, out, lse, B, H, S, D, block_q, block_k, scale, workspace, L, nullptr, 0,
                   (hipStream_t)stream);
}

int bsattn_fwd_fp8(const void* q, const void* k, const void* v, const uint8_t* block_mask, void* out, float* lse,
                   int B, int H, int S, int D, int block_q, int block_k, float scale, void* workspace,
                   size_t workspace_bytes, void* stream) {
    if (!block_mask || !workspace) return BSATTN_ERR_NULL;
    Fp8Layout L;
    int rc = check_fp8_call(q, k, v, out, lse, B, H, S, D, block_q, block_k, scale, workspace,
                            workspace_bytes, nullptr, 0, &L);
    if (rc) return rc;
    rc = bsattn_plan(block_mask, B, H, S, block_q, block_k, workspace, workspace_bytes, stream);
    if (rc) return rc;
    return run_fp8(q, k, v, out, lse, B, H, S, D, block_q, block_k, scale, workspace, L, nullptr, 0,
                   (hipStream_t)stream);
}

// The fp8 forward with an element-level mask: the plan of bsattn_plan_elem in the
// first part of the fp8 workspace, partial_bits as for bsattn_fwd_planned_elem.
int bsattn_fwd_fp8_planned_elem(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                                int H, int S, int D, int block_q, int block_k, float scale,
                                const uint32_t* partial_bits, int n_tiles, void* workspace,
                                size_t workspace_bytes, void* stream) {
    if (!workspace || !partial_bits) return BSATTN_ERR_NULL;
    Fp8Layout L;
    const int rc = check_fp8_call(q, k, v, out, lse, B, H, S, D, block_q, block_k, scale, workspace,
                                  workspace_bytes, partial_bits, n_tiles, &L);
    if (rc) return rc;
    return run_fp8(q, k, v, out, lse, B, H, S, D, block_q, block_k, scale, workspace, L, partial_bits, n_tiles,
                   (hipStream_t)stream);
}

int bsattn_fwd_fp8_elem(const void* q, const void* k, const void* v, const uint8_t* block_states,
                        const int32_t* partial_index, const uint32_t* partial_bits, int n_tiles, void* out,
                        float* lse, int B, int H, int S, int D, int block_q, int block_k, float scale,
                        void* workspace, size_t workspace_bytes, void* stream) {
    if (!block_states || !partial_index || !partial_bits || !workspace) return BSATTN_ERR_NULL;
    Fp8Layout L;
    int rc = check_fp8_call(q, k, v, out, lse, B, H, S, D, block_q, block_k, scale, workspace,
                            workspace_bytes, partial_bits, n_tiles, &L);
    if (rc) return rc;
    if (!is_aligned(partial_index, 4)) return BSATTN_ERR_ALIGN;
    rc = bsattn_plan_elem(block_states, partial_index, n_tiles, B, H, S, block_q, block_k, workspace,
                          workspace_bytes, stream);
    if (rc) return rc;
    return run_fp8(q, k, v, out, lse, B, H, S, D, block_q, block_k, scale, workspace, L, partial_bits, n_tiles,
                   (hipStream_t)stream);
}

// ---- backward ------------------------------------------------------------------

int bsattn_bwd_workspace_size(int B, int H, int S, int block_q, int block_k, size_t* bytes) {
    if (!bytes) return BSATTN_ERR_NULL;
    if (B <= 0 || H <= 0 || S <= 0 || block_q <= 0 || block_k <= 0) return BSATTN_ERR_SHAPE;
    if (S % block_q != 0 || S % block_k != 0) return BSATTN_ERR_SHAPE;
    const int rc = check_grid(B, H, S / block_q, S / block_k);
    if (rc) return rc;
    *bytes = bwd_layout((int64_t)B * H, S, S / block_q, S / block_k, block_k).bytes;
    return BSATTN_OK;
}

int bsattn_bwd_plan(const uint8_t* block_mask, int B, int H, int S, int block_q, int block_k, void* workspace,
                    size_t workspace_bytes, void* stream) {
    if (!block_mask || !workspace) return BSATTN_ERR_NULL;
    if (B <= 0 || H <= 0 || S <= 0 || block_q <= 0 || block_k <= 0) return BSATTN_ERR_SHAPE;
    if (S % block_q != 0 || S % block_k != 0) return BSATTN_ERR_SHAPE;
    if (!block_ok(block_q) || !block_ok(block_k)) return BSATTN_ERR_UNSUPPORTED;
    const int n_q = S / block_q, n_k = S / block_k;
    const int rc = check_grid(B, H, n_q, n_k);
    if (rc) return rc;
    const BwdLayout L = bwd_layout((int64_t)B * H, S, n_q, n_k, block_k);
    if (workspace_bytes < L.plan_bytes) return BSATTN_ERR_WORKSPACE;
    if (!is_aligned(workspace, 16)) return BSATTN_ERR_ALIGN;
    if (overlap(block_mask, (size_t)L.fwd.R * n_k, workspace, L.plan_bytes)) return BSATTN_ERR_ALIAS;
    hipStream_t st = (hipStream_t)stream;
    char* ws = (char*)workspace;
    hipError_t e = launch_plan(block_mask, L.fwd.R, n_q, n_k, (int32_t*)ws, (int32_t*)(ws + L.fwd.lists),
                               L.fwd.chunk, (int32_t*)(ws + L.fwd.order), L.fwd.pchunk,
                               (int32_t*)(ws + L.fwd.porder), st);
    if (e != hipSuccess) return hip_fail(e);
    e = launch_bwd_cols(block_mask, L.C, n_q, n_k, (int32_t*)(ws + L.ccounts), (int32_t*)(ws + L.clists), st);
    if (e != hipSuccess) return hip_fail(e);
    e = launch_bwd_split((const int32_t*)(ws + L.ccounts), L.C, n_q, (int)L.max_slots, ws + L.items, ws + L.splits,
                         (int32_t*)(ws + L.nout), st);
    if (e != hipSuccess) return hip_fail(e);
    return BSATTN_OK;
}

// bsattn_bwd_planned, and with states != NULL the element-mask kernels (the
// element arguments were checked by the caller).
static int bwd_planned_impl(const void* q, const void* k, const void* v, const void* out, const float* lse,
                            const void* dout, int B, int H, int S, int D, int block_q, int block_k, float scale,
                            int dtype, void* dq, void* dk, void* dv, int grad_dtype, int parts, void* workspace,
                            size_t workspace_bytes, void* stream, const uint8_t* states, const int32_t* pidx,
                            const uint32_t* pbits, int n_tiles) {
    if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv || !workspace) return BSATTN_ERR_NULL;
    if (parts <= 0 || parts > (BSATTN_BWD_PREP | BSATTN_BWD_DQ | BSATTN_BWD_DKDV)) return BSATTN_ERR_UNSUPPORTED;
    int rc = check_fwd_shape(B, H, S, D, block_q, block_k, dtype);
    if (rc) return rc;
    if (dtype != BSATTN_BF16) return BSATTN_ERR_UNSUPPORTED;
    if (grad_dtype != BSATTN_BF16 && grad_dtype != BSATTN_F32) return BSATTN_ERR_UNSUPPORTED;
    const int n_q = S / block_q, n_k = S / block_k;
    const BwdLayout L = bwd_layout((int64_t)B * H, S, n_q, n_k, block_k);
    if (workspace_bytes < L.bytes) return BSATTN_ERR_WORKSPACE;
    const void* al16[] = {q, k, v, out, dout, dq, dk, dv, workspace};
    for (const void* p : al16)
        if (!is_aligned(p, 16)) return BSATTN_ERR_ALIGN;
    if (!is_aligned(lse, 4)) return BSATTN_ERR_ALIGN;
    if (!std::isfinite(scale)) return BSATTN_ERR_SCALE;
    const size_t nt = (size_t)B * H * S * D * 2, nl = (size_t)B * H * S * 4;
    const size_t ng = (size_t)B * H * S * D * (grad_dtype == BSATTN_F32 ? 4 : 2);
    // written: dq, dk, dv and the ld region of the workspace; read: everything else
    const void* wr[] = {dq, dk, dv, (const char*)workspace + L.ld};
    const size_t wn[] = {ng, ng, ng, L.bytes - L.ld};
    const void* rd[] = {q, k, v, out, dout, lse, workspace};
    const size_t rn[] = {nt, nt, nt, nt, nt, nl, L.plan_bytes};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 7; ++j)
            if (overlap(wr[i], wn[i], rd[j], rn[j])) return BSATTN_ERR_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(wr[i], wn[i], wr[j], wn[j])) return BSATTN_ERR_ALIAS;
    }
    hipStream_t st = (hipStream_t)stream;
    char* ws = (char*)workspace;
    hipError_t e = hipSuccess;
    if (parts & BSATTN_BWD_PREP) {
        e = launch_bwd_prep(out, dout, lse, ws + L.ld, L.fwd.R * block_q, D, st);
        if (e != hipSuccess) return hip_fail(e);
    }
    BwdArgs a;
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.dout = (const uint16_t*)dout;
    a.ld = (const float2*)(ws + L.ld);
    a.row_counts = (const int32_t*)ws;
    a.row_lists = (const int32_t*)(ws + L.fwd.lists);
    a.row_order = (const int32_t*)(ws + L.fwd.order);
    a.n_rows = (int)L.fwd.R;
    a.chunk_q = (int)L.fwd.chunk;
    a.col_lists = (const int32_t*)(ws + L.clists);
    a.items = (const int4*)(ws + L.items);
    a.n_items = (const int32_t*)(ws + L.nout);
    a.splits = (const int4*)(ws + L.splits);
    a.scratch = (float*)(ws + L.scratch);
    a.n_cols = (int)L.C;
    a.chunk_k = (int)xcd_chunk(L.C + L.max_slots);
    a.max_slots = (int)L.max_slots;
    a.max_splits = (int)(L.max_slots / 2);
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.S = S;
    a.n_q = n_q;
    a.n_k = n_k;
    a.block_q = block_q;
    a.block_k = block_k;
    a.qsteps_log2 = block_q == 128 ? 2 : 1;
    a.ksteps_log2 = block_k == 128 ? 2 : 1;
    a.c = scale * kLog2e;
    a.scale = scale;
    a.states = states;
    a.pidx = pidx;
    a.pbits = pbits;
    a.n_tiles = n_tiles;
    e = launch_bwd_main(a, D, grad_dtype == BSATTN_F32, (parts & BSATTN_BWD_DQ) != 0,
                        (parts & BSATTN_BWD_DKDV) != 0, st);
    if (e != hipSuccess) return hip_fail(e);
    return BSATTN_OK;
}

int bsattn_bwd_planned(const void* q, const void* k, const void* v, const void* out, const float* lse,
                       const void* dout, int B, int H, int S, int D, int block_q, int block_k, float scale,
                       int dtype, void* dq, void* dk, void* dv, int grad_dtype, int parts, void* workspace,
                       size_t workspace_bytes, void* stream) {
    return bwd_planned_impl(q, k, v, out, lse, dout, B, H, S, D, block_q, block_k, scale, dtype, dq, dk, dv,
                            grad_dtype, parts, workspace, workspace_bytes, stream, nullptr, nullptr, nullptr, 0);
}

// bsattn_bwd; with pidx != NULL block_mask holds block states and the element
// kernels run (bsattn_bwd_elem, which checked the element arguments).
static int bwd_impl(const void* q, const void* k, const void* v, const void* out, const float* lse, const void* dout,
                    const uint8_t* block_mask, int B, int H, int S, int D, int block_q, int block_k, float scale,
                    int dtype, void* dq, void* dk, void* dv, int grad_dtype, void* workspace, size_t workspace_bytes,
                    void* stream, const int32_t* pidx, const uint32_t* pbits, int n_tiles) {
    if (!q || !k || !v || !out || !lse || !dout || !block_mask || !dq || !dk || !dv || !workspace)
        return BSATTN_ERR_NULL;
    int rc = check_fwd_shape(B, H, S, D, block_q, block_k, dtype);
    if (rc) return rc;
    if (dtype != BSATTN_BF16) return BSATTN_ERR_UNSUPPORTED;
    if (grad_dtype != BSATTN_BF16 && grad_dtype != BSATTN_F32) return BSATTN_ERR_UNSUPPORTED;
    const BwdLayout L = bwd_layout((int64_t)B * H, S, S / block_q, S / block_k, block_k);
    if (workspace_bytes < L.bytes) return BSATTN_ERR_WORKSPACE;
    // the plan step writes the workspace: it must not overlap any tensor argument
    const size_t nt = (size_t)B * H * S * D * 2, nl = (size_t)B * H * S * 4;
    const size_t ng = (size_t)B * H * S * D * (grad_dtype == BSATTN_F32 ? 4 : 2);
    const void* ts[] = {q, k, v, out, dout, lse, dq, dk, dv};
    const size_t tn[] = {nt, nt, nt, nt, nt, nl, ng, ng, ng};
    for (int i = 0; i < 9; ++i)
        if (overlap(workspace, L.bytes, ts[i], tn[i])) return BSATTN_ERR_ALIAS;
    // every other check of bsattn_bwd_planned runs before the plan is launched
    const void* al16[] = {q, k, v, out, dout, dq, dk, dv, workspace};
    for (const void* p : al16)
        if (!is_aligned(p, 16)) return BSATTN_ERR_ALIGN;
    if (!is_aligned(lse, 4)) return BSATTN_ERR_ALIGN;
    if (!std::isfinite(scale)) return BSATTN_ERR_SCALE;
    for (int i = 6; i < 9; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlap(ts[i], tn[i], ts[j], tn[j])) return BSATTN_ERR_ALIAS;
        for (int j = i + 1; j < 9; ++j)
            if (overlap(ts[i], tn[i], ts[j], tn[j])) return BSATTN_ERR_ALIAS;
    }
    rc = bsattn_bwd_plan(block_mask, B, H, S, block_q, block_k, workspace, workspace_bytes, stream);
    if (rc) return rc;
    return bwd_planned_impl(q, k, v, out, lse, dout, B, H, S, D, block_q, block_k, scale, dtype, dq, dk, dv,
                            grad_dtype, BSATTN_BWD_ALL, workspace, workspace_bytes, stream,
                            pidx ? block_mask : nullptr, pidx, pbits, n_tiles);
}

int bsattn_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse, const void* dout,
               const uint8_t* block_mask, int B, int H, int S, int D, int block_q, int block_k, float scale,
               int dtype, void* dq, void* dk, void* dv, int grad_dtype, void* workspace, size_t workspace_bytes,
               void* stream) {
    return bwd_impl(q, k, v, out, lse, dout, block_mask, B, H, S, D, block_q, block_k, scale, dtype, dq, dk, dv,
                    grad_dtype, workspace, workspace_bytes, stream, nullptr, nullptr, 0);
}

int bsattn_bwd_planned_elem(const void* q, const void* k, const void* v, const void* out, const float* lse,
                            const void* dout, const uint8_t* block_states, const int32_t* partial_index,
                            const uint32_t* partial_bits, int n_tiles, int B, int H, int S, int D, int block_q,
                            int block_k, float scale, int dtype, void* dq, void* dk, void* dv, int grad_dtype,
                            int parts, void* workspace, size_t workspace_bytes, void* stream) {
    if (!block_states || !partial_index || !partial_bits) return BSATTN_ERR_NULL;
    const int rc = check_elem_shape(B, H, S, block_q, block_k, n_tiles);
    if (rc) return rc;
    if (!is_aligned(partial_index, 4) || !is_aligned(partial_bits, 4)) return BSATTN_ERR_ALIGN;
    return bwd_planned_impl(q, k, v, out, lse, dout, B, H, S, D, block_q, block_k, scale, dtype, dq, dk, dv,
                            grad_dtype, parts, workspace, workspace_bytes, stream, block_states, partial_index,
                            partial_bits, n_tiles);
}

int bsattn_bwd_elem(const void* q, const void* k, const void* v, const void* out, const float* lse,
                    const void* dout, const uint8_t* block_states, const int32_t* partial_index,
                    const uint32_t* partial_bits, int n_tiles, int B, int H, int S, int D, int block_q,
                    int block_k, float scale, int dtype, void* dq, void* dk, void* dv, int grad_dtype,
                    void* workspace, size_t workspace_bytes, void* stream) {
    if (!block_states || !partial_index || !partial_bits) return BSATTN_ERR_NULL;
    int rc = check_elem_shape(B, H, S, block_q, block_k, n_tiles);
    if (rc) return rc;
    if (!is_aligned(partial_index, 4) || !is_aligned(partial_bits, 4)) return BSATTN_ERR_ALIGN;
    // the gradients and the workspace must not overlap the element mask
    const size_t nb = (size_t)B * H * (S / block_q) * (S / block_k);
    const size_t nbits = (size_t)n_tiles * block_q * (block_k / 32) * 4;
    const size_t ng = (size_t)B * H * S * D * (grad_dtype == BSATTN_F32 ? 4 : 2);
    size_t wsb = 0;
    if (bsattn_bwd_workspace_size(B, H, S, block_q, block_k, &wsb) == BSATTN_OK) {
        const void* wr[] = {dq, dk, dv, workspace};
        const size_t wn[] = {ng, ng, ng, wsb};
        for (int i = 0; i < 4; ++i)
            if (wr[i] && (overlap(wr[i], wn[i], block_states, nb) || overlap(wr[i], wn[i], partial_index, nb * 4) ||
                          overlap(wr[i], wn[i], partial_bits, nbits)))
                return BSATTN_ERR_ALIAS;
    }
    return bwd_impl(q, k, v, out, lse, dout, block_states, B, H, S, D, block_q, block_k, scale, dtype, dq, dk, dv,
                    grad_dtype, workspace, workspace_bytes, stream, partial_index, partial_bits, n_tiles);
}

int bsattn_list_configs(int dtype, int D, int block_q, int block_k, bsattn_tile_config* cfgs,
                        int cap, int* n) {
    if (!n) return BSATTN_ERR_NULL;
    if (dtype != BSATTN_F32 && dtype != BSATTN_BF16) return BSATTN_ERR_UNSUPPORTED;
    int nv = 0;
    const Variant* t = variants(dtype, &nv);
    int cnt = 0;
    for (int i = 0; i < nv; ++i) {
        if (!legal(t[i], dtype, D, block_q, block_k)) continue;
        if (cfgs && cnt < cap)
            cfgs[cnt] = bsattn_tile_config{t[i].tile_q, t[i].tile_k, t[i].waves, t[i].stages};
        ++cnt;
    }
    *n = cnt;
    return BSATTN_OK;
}

int bsattn_autotune(const void* q, const void* k, const void* v, const uint8_t* block_mask,
                    void* out, float* lse, int B, int H, int S, int D, int block_q, int block_k,
                    float scale, int dtype, void* workspace, size_t workspace_bytes, int warmup,
                    int iters, bsattn_tile_config* best, bsattn_tune_result* results, int cap,
                    int* n_results, const char* cache_path, void* stream) {
    if (!best || !block_mask) return BSATTN_ERR_NULL;
    const int rc = check_fwd_buffers(q, k, v, out, lse, B, H, S, D, block_q, block_k, dtype, scale);
    if (rc) return rc;
    if (!workspace || workspace_bytes < fwd_ws_bytes((int64_t)B * H, S / block_q, S / block_k))
        return BSATTN_ERR_WORKSPACE;
    if (warmup < 0 || iters < 1) return BSATTN_ERR_SHAPE;

    int nv = 0;
    const Variant* t = variants(dtype, &nv);
    std::vector<bsattn_tune_result> res;
    hipStream_t s = (hipStream_t)stream;
    // The mask statistic of the cache key: active blocks counted on a host copy
    // of the mask, read in stream order (tuning is not on the call path).
    const int64_t R = (int64_t)B * H * (S / block_q), n_k = S / block_k;
    int64_t nnz = 0;
    {
        std::vector<uint8_t> host((size_t)(R * n_k));
        hipError_t he = hipMemcpyAsync(host.data(), block_mask, host.size(), hipMemcpyDeviceToHost, s);
        if (he == hipSuccess) he = hipStreamSynchronize(s);
        if (he != hipSuccess) return hip_fail(he);
        for (uint8_t b : host) nnz += b != 0;
    }
    std::vector<hipEvent_t> ev((size_t)iters + 1);
    for (auto& e : ev) {
        const hipError_t he = hipEventCreate(&e);
        if (he != hipSuccess) return hip_fail(he);
    }
    int status = BSATTN_OK;
    for (int i = 0; i < nv && status == BSATTN_OK; ++i) {
        if (!legal(t[i], dtype, D, block_q, block_k)) continue;
        if (is_pair(t[i]) && S / block_k > kPairMaxBlocks) continue;
        const bsattn_tile_config c{t[i].tile_q, t[i].tile_k, t[i].waves, t[i].stages};
        for (int w = 0; w < warmup && status == BSATTN_OK; ++w)
            status = bsattn_fwd_config(q, k, v, block_mask, out, lse, B, H, S, D, block_q, block_k,
                                       scale, dtype, workspace, workspace_bytes, &c, stream);
        hipError_t he = hipEventRecord(ev[0], s);
        if (he != hipSuccess) { status = hip_fail(he); break; }
        for (int it = 0; it < iters && status == BSATTN_OK; ++it) {
            status = bsattn_fwd_config(q, k, v, block_mask, out, lse, B, H, S, D, block_q, block_k,
                                       scale, dtype, workspace, workspace_bytes, &c, stream);
            he = hipEventRecord(ev[(size_t)it + 1], s);
            if (he != hipSuccess) status = hip_fail(he);
        }
        if (status != BSATTN_OK) break;
        he = hipEventSynchronize(ev[(size_t)iters]);
        if (he != hipSuccess) { status = hip_fail(he); break; }
        double sum = 0.0, sum2 = 0.0, mn = 1e300;
        for (int it = 0; it < iters; ++it) {
            float ms = 0.f;
            he = hipEventElapsedTime(&ms, ev[(size_t)it], ev[(size_t)it + 1]);
            if (he != hipSuccess) { status = hip_fail(he); break; }
            const double sec = ms * 1e-3;
            sum += sec;
            sum2 += sec * sec;
            mn = std::min(mn, sec);
        }
        if (status != BSATTN_OK) break;
        const double mean = sum / iters;
        const double var = std::max(0.0, sum2 / iters - mean * mean);
        bsattn_tune_result r;
        r.id = i;
        r.cfg = c;
        r.t_mean_s = mean;
        r.t_std_s = std::sqrt(var);
        r.t_min_s = mn;
        res.push_back(r);
    }
    for (auto& e : ev) hipEventDestroy(e);
    if (status != BSATTN_OK) return status;
    if (res.empty()) return BSATTN_ERR_UNSUPPORTED;
    std::stable_sort(res.begin(), res.end(), [](const bsattn_tune_result& x,
                                                 const bsattn_tune_result& y) {
        return x.t_mean_s < y.t_mean_s;
    });
    *best = res[0].cfg;
    if (n_results) *n_results = (int)res.size();
    if (results)
        for (int i = 0; i < cap && i < (int)res.size(); ++i) results[i] = res[(size_t)i];
    const TuneKey key(dtype, D, block_q, block_k, S, (int64_t)B * H, mask_bucket(nnz, R));
    {
        std::lock_guard<std::mutex> lk(g_tune_mu);
        g_tune[key] = TuneEntry{res[0].cfg, res[0].t_mean_s};
        if (cache_path) {
            std::map<TuneKey, TuneEntry> merged;
            read_cache(cache_path, &merged);
            merged[key] = g_tune[key];
            if (!write_cache(cache_path, merged)) return BSATTN_ERR_IO;
        }
    }
    return BSATTN_OK;
}

int bsattn_tune_lookup(int dtype, int D, int B, int H, int S, int block_q, int block_k, long long nnz,
                       bsattn_tile_config* cfg) {
    if (!cfg) return BSATTN_ERR_NULL;
    if (B <= 0 || H <= 0 || S <= 0 || block_q <= 0 || block_k <= 0) return BSATTN_ERR_SHAPE;
    if (S % block_q != 0 || S % block_k != 0) return BSATTN_ERR_SHAPE;
    const int64_t R = (int64_t)B * H * (S / block_q);
    std::lock_guard<std::mutex> lk(g_tune_mu);
    if (nnz < 0)
        return densest_entry(ShapeKey(dtype, D, block_q, block_k, S, (int64_t)B * H), cfg) ? BSATTN_OK
                                                                                         : BSATTN_ERR_UNSUPPORTED;
    auto it = g_tune.find(TuneKey(dtype, D, block_q, block_k, S, (int64_t)B * H, mask_bucket(nnz, R)));
    if (it == g_tune.end()) return BSATTN_ERR_UNSUPPORTED;
    *cfg = it->second.cfg;
    return BSATTN_OK;
}

int bsattn_load_tune_cache(const char* cache_path) {
    if (!cache_path) return BSATTN_ERR_NULL;
    std::map<TuneKey, TuneEntry> m;
    if (!read_cache(cache_path, &m)) return BSATTN_ERR_IO;
    std::lock_guard<std::mutex> lk(g_tune_mu);
    for (const auto& kv : m) g_tune[kv.first] = kv.second;
    return BSATTN_OK;
}

void bsattn_clear_tune_cache(void) {
    std::lock_guard<std::mutex> lk(g_tune_mu);
    g_tune.clear();
}

}  // extern "C"
