// gemm_api.cpp -- the C ABI declared in include/gemm.h
//
// Host side of the library: plan creation and validation (no device calls),
// kernel selection from the compiled registry keyed by (element family,
// operand layouts, tile shape, alignment class) -- the role the pages give to
// "KernelsForDataType" and default_operation() ("CUTLASS Python 接口全解析"
// section 3.2) -- the data-parallel / stream-K / hybrid schedule, the
// plan-owned device workspace, and the launches. Errors are reported as
// status codes plus a descriptive thread-local message ("Python packages
// associated with CUTLASS", Overview: descriptive run-time errors).
#include "gemm.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "kernels.hpp"

using namespace mg;

namespace {

thread_local std::string g_err;

gemm_status fail(gemm_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

gemm_status ok() {
    g_err.clear();
    return GEMM_OK;
}

gemm_status hip_fail(hipError_t e, const char *what) {
    return fail(GEMM_HIP_ERROR, "%s failed: %s (%d)", what, hipGetErrorString(e), (int)e);
}

const char *dtype_name(int d) {
    switch (d) {
    case GEMM_F32: return "F32";
    case GEMM_F16: return "F16";
    case GEMM_BF16: return "BF16";
    case GEMM_F8_E4M3: return "F8_E4M3";
    case GEMM_F4_E2M1: return "F4_E2M1";
    }
    return "?";
}

struct Tuple {
    gemm_dtype a, b, c, d, acc;
    int fam;
};
const Tuple kSupported[] = {
    {GEMM_F32, GEMM_F32, GEMM_F32, GEMM_F32, GEMM_F32, FAM_F32},
    {GEMM_F16, GEMM_F16, GEMM_F16, GEMM_F16, GEMM_F32, FAM_F16},
    {GEMM_BF16, GEMM_BF16, GEMM_BF16, GEMM_BF16, GEMM_F32, FAM_BF16},
    {GEMM_F8_E4M3, GEMM_F8_E4M3, GEMM_BF16, GEMM_BF16, GEMM_F32, FAM_F8},
    // FP4 elements exist only under MX block scales (gemm_plan_run_mx)
    {GEMM_F4_E2M1, GEMM_F4_E2M1, GEMM_BF16, GEMM_BF16, GEMM_F32, FAM_MXF4},
};
constexpr int kNumSupported = (int)(sizeof(kSupported) / sizeof(kSupported[0]));

// Bytes per element as the tile engine addresses operands: FP4 operands are
// addressed in bytes (two elements each), with K counted in bytes.
int elem_bytes(int fam) {
    return fam == FAM_F32 ? 4 : (fam == FAM_F8 || fam == FAM_MXF8 || fam == FAM_MXF4) ? 1 : 2;
}
// The kernel family of an MX run on a plan of family `fam`.
int mx_family(int fam) { return fam == FAM_MXF4 ? FAM_MXF4 : FAM_MXF8; }
int out_bytes(int fam) { return fam == FAM_F32 ? 4 : 2; }

// ------------------------------------------------------------------ registry

struct Registry {
    std::vector<KernelEntry> all;
    Registry() {
        const KernelEntry *(*tables[])(int *) = {entries_f32, entries_f16, entries_bf16, entries_f8,
                                                 entries_mxf8, entries_mxf4};
        for (auto t : tables) {
            int n = 0;
            const KernelEntry *e = t(&n);
            all.insert(all.end(), e, e + n);
        }
    }
    const KernelEntry *find(int fam, bool a_kc, bool b_kc, int tile) const {
        for (const auto &e : all)
            if (e.fam == fam && e.a_kc == (int)a_kc && e.b_kc == (int)b_kc && e.tile == tile) return &e;
        return nullptr;
    }
};

const Registry &registry() {
    static Registry r;
    return r;
}

// Per-device facts, and occupancy per kernel (queried once).
struct DeviceInfo {
    int num_cus = 0;
    std::unordered_map<const void *, int> occ;
};
std::mutex g_dev_mu;
std::unordered_map<int, DeviceInfo> g_dev;

gemm_status device_cus(int dev, int *cus) {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    DeviceInfo &di = g_dev[dev];
    if (di.num_cus == 0) {
        int v = 0;
        hipError_t e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(multiprocessor count)");
        di.num_cus = v > 0 ? v : 1;
    }
    *cus = di.num_cus;
    return GEMM_OK;
}

gemm_status kernel_occupancy(int dev, const void *fn, int nt, int *occ) {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    DeviceInfo &di = g_dev[dev];
    auto it = di.occ.find(fn);
    if (it == di.occ.end()) {
        int v = 0;
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, fn, nt, 0);
        if (e != hipSuccess) return hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
        it = di.occ.emplace(fn, v > 0 ? v : 1).first;
    }
    *occ = it->second;
    return GEMM_OK;
}

int static_occupancy(const KernelEntry *e) {
    int occ = (160 * 1024) / e->lds_bytes;
    const int by_waves = 32 / (e->nt / 64);   // 8 waves per SIMD x 4 SIMDs
    if (occ > by_waves) occ = by_waves;
    return occ > 0 ? occ : 1;
}

// ---- configuration cache: JSON text ----------------------------------------
//
// Written by gemm_plan_cache_export, read by gemm_plan_cache_import:
//   {"format": "mi355-gemm-config-cache", "version": 1, "arch": "gfx950",
//    "plan": {"a": "BF16", "b": "BF16", "c": "BF16", "d": "BF16", "acc": "F32",
//             "layout_a": "row", "layout_b": "col", "layout_c": "row"},
//    "entries": [{"m": 4096, "n": 8192, "k": 8192, "mx": 0,
//                 "schedule": "data_parallel", "tile": "256x256", "sk_grid": 0,
//                 "us": 477.8}, ...]}

const char *kCacheFormat = "mi355-gemm-config-cache";

const char *layout_str(gemm_layout l) { return l == GEMM_ROW_MAJOR ? "row" : "col"; }

const char *tile_enum_name(gemm_tile t) {
    switch (t) {
    case GEMM_TILE_256x256: return "256x256";
    case GEMM_TILE_128x128: return "128x128";
    case GEMM_TILE_64x256: return "64x256";
    case GEMM_TILE_32x256: return "32x256";
    case GEMM_TILE_GENERIC: return "generic";
    case GEMM_TILE_WHOLEK: return "wholek";
    default: return "auto";
    }
}

bool parse_tile(const std::string &s, gemm_tile *t) {
    for (int v = GEMM_TILE_AUTO; v <= GEMM_TILE_WHOLEK; ++v)
        if (s == tile_enum_name((gemm_tile)v)) { *t = (gemm_tile)v; return true; }
    return false;
}

const char *sched_name(gemm_schedule s);

bool parse_sched(const std::string &s, gemm_schedule *out) {
    for (int v = GEMM_SCHED_AUTO; v <= GEMM_SCHED_SPLIT_K; ++v)
        if (s == sched_name((gemm_schedule)v)) { *out = (gemm_schedule)v; return true; }
    return false;
}

// A JSON value (only what the cache format needs: objects, arrays, strings,
// numbers, true/false/null).
struct JVal {
    enum Kind { NUL, BOOL, NUM, STR, ARR, OBJ } kind = NUL;
    double num = 0.0;
    bool b = false;
    std::string str;
    std::vector<JVal> arr;
    std::vector<std::pair<std::string, JVal>> obj;
    const JVal *get(const char *key) const {
        for (const auto &kv : obj)
            if (kv.first == key) return &kv.second;
        return nullptr;
    }
};

struct JParser {
    const char *s;
    size_t i = 0, n;
    const char *err = nullptr;
    int depth = 0;
    explicit JParser(const char *t) : s(t), n(strlen(t)) {}
    void ws() {
        while (i < n && (s[i] == ' ' || s[i] == '\t' || s[i] == '\n' || s[i] == '\r')) ++i;
    }
    bool fail_at(const char *m) {
        if (!err) err = m;
        return false;
    }
    bool lit(const char *w) {
        const size_t L = strlen(w);
        if (n - i < L || strncmp(s + i, w, L) != 0) return fail_at("unexpected token");
        i += L;
        return true;
    }
    bool string(std::string *out) {
        if (i >= n || s[i] != '"') return fail_at("expected a string");
        ++i;
        out->clear();
        while (i < n && s[i] != '"') {
            char c = s[i++];
            if (c == '\\') {
                if (i >= n) return fail_at("unterminated escape");
                const char e = s[i++];
                switch (e) {
                case '"': c = '"'; break;
                case '\\': c = '\\'; break;
                case '/': c = '/'; break;
                case 'n': c = '\n'; break;
                case 't': c = '\t'; break;
                case 'r': c = '\r'; break;
                case 'b': c = '\b'; break;
                case 'f': c = '\f'; break;
                default: return fail_at("unsupported string escape");
                }
            } else if ((unsigned char)c < 0x20) {
                return fail_at("control character in a string");
            }
            out->push_back(c);
        }
        if (i >= n) return fail_at("unterminated string");
        ++i;
        return true;
    }
    bool value(JVal *v) {
        if (++depth > 16) return fail_at("nesting too deep");
        ws();
        bool ok_ = false;
        if (i >= n) {
            ok_ = fail_at("unexpected end of text");
        } else if (s[i] == '{') {
            v->kind = JVal::OBJ;
            ++i;
            ws();
            if (i < n && s[i] == '}') {
                ++i;
                ok_ = true;
            } else {
                for (;;) {
                    ws();
                    std::string key;
                    if (!string(&key)) break;
                    ws();
                    if (i >= n || s[i] != ':') { fail_at("expected ':'"); break; }
                    ++i;
                    JVal child;
                    if (!value(&child)) break;
                    v->obj.emplace_back(std::move(key), std::move(child));
                    ws();
                    if (i < n && s[i] == ',') { ++i; continue; }
                    if (i < n && s[i] == '}') { ++i; ok_ = true; }
                    else fail_at("expected ',' or '}'");
                    break;
                }
            }
        } else if (s[i] == '[') {
            v->kind = JVal::ARR;
            ++i;
            ws();
            if (i < n && s[i] == ']') {
                ++i;
                ok_ = true;
            } else {
                for (;;) {
                    JVal child;
                    if (!value(&child)) break;
                    v->arr.push_back(std::move(child));
                    ws();
                    if (i < n && s[i] == ',') { ++i; continue; }
                    if (i < n && s[i] == ']') { ++i; ok_ = true; }
                    else fail_at("expected ',' or ']'");
                    break;
                }
            }
        } else if (s[i] == '"') {
            v->kind = JVal::STR;
            ok_ = string(&v->str);
        } else if (s[i] == 't') {
            v->kind = JVal::BOOL;
            v->b = true;
            ok_ = lit("true");
        } else if (s[i] == 'f') {
            v->kind = JVal::BOOL;
            ok_ = lit("false");
        } else if (s[i] == 'n') {
            ok_ = lit("null");
        } else {
            char *end = nullptr;
            v->kind = JVal::NUM;
            v->num = strtod(s + i, &end);
            if (end == s + i) ok_ = fail_at("unexpected character");
            else {
                i = (size_t)(end - s);
                ok_ = true;
            }
        }
        --depth;
        return ok_;
    }
};

bool json_int(const JVal *v, int64_t lo, int64_t hi, int64_t *out) {
    if (!v || v->kind != JVal::NUM) return false;
    if (!(v->num >= (double)lo && v->num <= (double)hi) || v->num != (double)(int64_t)v->num)
        return false;
    *out = (int64_t)v->num;
    return true;
}

bool json_str(const JVal *v, std::string *out) {
    if (!v || v->kind != JVal::STR) return false;
    *out = v->str;
    return true;
}

}  // namespace

// ------------------------------------------------------------------ plan

struct gemm_plan_s {
    uint32_t magic;
    gemm_dtype a, b, c, d, acc;
    gemm_layout la, lb, lc;
    gemm_epilogue epi;
    int fam;
    gemm_schedule sched;
    gemm_tile tile;
    int sk_grid;
    int device;
    float *partials;
    size_t partial_bytes;
    int *counters;
    size_t counter_count;
    GroupDesc *gdesc;
    size_t gdesc_cap;
    size_t gdesc_count;        // descriptors of the last upload (0: none)
    hipStream_t gdesc_stream;  // the stream that upload went to
    GroupDesc *ghost;
    hipEvent_t gevent;
    bool gevent_pending;
    unsigned int *gqueue;      // grouped launches' tile queues (9 words, zero between launches)
    hipStream_t last_stream;
    bool used;
    // Tuned configurations (from gemm_plan_profile or an imported cache),
    // keyed by (M, N, K, MX); used when the plan has no explicit override.
    struct TunedKey {
        int64_t m, n, k;
        int mx;
        bool operator<(const TunedKey &o) const {
            if (m != o.m) return m < o.m;
            if (n != o.n) return n < o.n;
            if (k != o.k) return k < o.k;
            return mx < o.mx;
        }
    };
    struct Tuned {
        gemm_schedule sched;
        gemm_tile tile;
        int sk_grid;
        float us;
    };
    std::map<TunedKey, Tuned> tuned;
};

namespace {

constexpr uint32_t kMagic = 0x6D473535u;

bool plan_ok(gemm_plan_t p) { return p && p->magic == kMagic; }

// What a run of (M, N, K) will launch.
struct Decision {
    const KernelEntry *e = nullptr;   // null: scalar-load kernel
    gemm_schedule sched = GEMM_SCHED_DATA_PARALLEL;
    int tiles_m = 0, tiles_n = 0, ipt = 0, total = 0, grid = 0, sk_tiles = 0, split = 0;
    int64_t sk_iters = 0;
    int sk_grid = 0;   // workgroups sharing the stream-K iterations (<= grid, <= sk_iters)
    int group_m = 4;
    int vec_cd = 0;
    int wholek = 0;   // > 0: the whole-K kernel, this many MFMA steps per wave (e is null)
    const char *why_generic = "";
};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Vector (16-byte buffer-load) eligibility of one operand for a tile kernel.
// rows: tile rows of this operand; kbytes: bytes of K per k-tile row.
const char *operand_vec_problem(const void *ptr, bool kc, int64_t contig, int64_t rows, int esz,
                                int kbytes) {
    const int vec = 16 / esz;
    if (reinterpret_cast<uintptr_t>(ptr) % 16) return "operand base not 16-byte aligned";
    if (contig % vec) return "contiguous extent not a multiple of 16 bytes";
    // largest in-tile byte offset must stay below the 31-bit buffer range
    const int64_t span = kc ? rows * contig * esz : (int64_t)kbytes * contig;
    if (span + 16 > 0x7FFFFFFFLL) return "operand row stride too large for 32-bit offsets";
    return nullptr;
}

// Why the whole-K kernel cannot take this problem (null: it can). It loads
// K-contiguous operands 16 bytes at a time and addresses every operand with
// 32-bit byte offsets.
const char *wholek_problem(int fam, const void *A, const void *B, bool a_kc, bool b_kc, int64_t M,
                           int64_t N, int64_t K, int64_t batch, bool mx) {
    if (batch != 1 || mx) return "batched or MX-scaled";
    if (K < 1 || wholek_steps(fam, K) == 0) return "K too long or unsupported element type";
    const int esz = elem_bytes(fam);
    if ((a_kc && (reinterpret_cast<uintptr_t>(A) % 16 || (K * esz) % 16)) ||
        (b_kc && (reinterpret_cast<uintptr_t>(B) % 16 || (K * esz) % 16)))
        return "K-contiguous operand not in 16-byte rows";
    if (M * K * esz + 16 > 0x7FFFFFFFLL || N * K * esz + 16 > 0x7FFFFFFFLL)
        return "operand beyond 32-bit offsets";
    return nullptr;
}

// AUTO takes the whole-K kernel when 128x128 tiles would leave most CUs
// idle and K is short enough for it (fp16 1024^3 + ReLU: 64 tiles).
bool wholek_auto(int fam, int64_t M, int64_t N, int64_t K, int cus) {
    return wholek_steps(fam, K) > 0 && cdiv(M, 128) * cdiv(N, 128) < cus;
}

// `batch`: problems of this shape in one launch. The 256x256 tile needs a
// full wave of tiles and a long K: its kernel pays ~20 us per workgroup and
// tile outside the main loop, so on 16 x 1024^3 fp16 batches (one 256x256
// tile per workgroup, 16 k-tiles) 128x128 tiles ran 1.38x faster (44 vs
// 61 us, same box), while the K = 8192 layer GEMMs want 256x256.
gemm_tile pick_tile(int fam, int64_t M, int64_t N, int64_t K, int cus, int64_t batch = 1) {
    if (fam == FAM_F32) return GEMM_TILE_128x128;
    // skinny M streams B once: 64-row tiles matched or beat 32-row ones for
    // every measured M <= 64 (fewer, longer B panels per workgroup)
    if (M <= 64) return GEMM_TILE_64x256;
    const int64_t big = cdiv(M, 256) * cdiv(N, 256) * (batch > 1 ? batch : 1);
    return big >= cus && K >= 2048 ? GEMM_TILE_256x256 : GEMM_TILE_128x128;
}

gemm_tile tile_enum(int id) {
    switch (id) {
    case TILE_256x256: return GEMM_TILE_256x256;
    case TILE_128x128: return GEMM_TILE_128x128;
    case TILE_64x256: return GEMM_TILE_64x256;
    case TILE_32x256: return GEMM_TILE_32x256;
    default: return GEMM_TILE_GENERIC;
    }
}

int tile_id(gemm_tile t) {
    switch (t) {
    case GEMM_TILE_256x256: return TILE_256x256;
    case GEMM_TILE_128x128: return TILE_128x128;
    case GEMM_TILE_64x256: return TILE_64x256;
    case GEMM_TILE_32x256: return TILE_32x256;
    default: return 0;
    }
}

const char *tile_name(const KernelEntry *e) {
    if (!e) return "generic64x64";
    switch (e->tile) {
    case TILE_256x256: return "256x256";
    case TILE_128x128: return "128x128";
    case TILE_64x256: return "64x256";
    case TILE_32x256: return "32x256";
    }
    return "?";
}

const char *sched_name(gemm_schedule s) {
    switch (s) {
    case GEMM_SCHED_DATA_PARALLEL: return "data_parallel";
    case GEMM_SCHED_STREAM_K: return "stream_k";
    case GEMM_SCHED_HYBRID: return "hybrid";
    case GEMM_SCHED_SPLIT_K: return "split_k";
    default: return "auto";
    }
}

// Fewest k-tiles one stream-K or split-K unit takes, so the partial-tile
// fixups stay small next to the work: eight for 16- and 8-bit types (a k-tile
// is 128 bytes of K: 512 MFMA cycles per SIMD on a 128x128 tile), one for
// fp32, whose 32-element k-tile already costs eight times that.
int min_iters(int fam) { return fam == FAM_F32 ? 1 : 8; }

// The schedule / tile / grid a run uses: the plan's explicit override if it
// has one, else a tuned entry for this single (non-batched) shape, else the
// heuristics (AUTO).
struct Cfg {
    gemm_schedule sched;
    gemm_tile tile;
    int sk_grid;
};

Cfg plan_cfg(const gemm_plan_s *pl, int64_t M, int64_t N, int64_t K, int64_t batch, bool mx) {
    Cfg c{pl->sched, pl->tile, pl->sk_grid};
    if (c.sched == GEMM_SCHED_AUTO && c.tile == GEMM_TILE_AUTO && c.sk_grid == 0 && batch == 1) {
        auto it = pl->tuned.find({M, N, K, mx ? 1 : 0});
        if (it != pl->tuned.end()) c = Cfg{it->second.sched, it->second.tile, it->second.sk_grid};
    }
    return c;
}

// `occ_of` gives workgroups per CU for an entry (live query or estimate).
template <class OccFn>
gemm_status decide(const gemm_plan_s *pl, const void *A, const void *B, const void *C, const void *D,
                   const void *bias, int64_t M, int64_t N, int64_t K, float beta, int cus, OccFn occ_of,
                   Decision &d, int64_t batch = 1, const void *mx_a = nullptr,
                   const void *mx_b = nullptr, size_t max_ws = 0) {
    const int fam = mx_a ? mx_family(pl->fam) : pl->fam;
    const Cfg cfg = plan_cfg(pl, M, N, K, batch, mx_a != nullptr);
    const int esz = elem_bytes(fam), osz = out_bytes(fam);
    // the tile kernels count K in their storage units: bytes for FP4
    const int64_t K_el = K;
    if (fam == FAM_MXF4) K = K / 2;
    const bool a_kc = pl->la == GEMM_ROW_MAJOR, b_kc = pl->lb == GEMM_COL_MAJOR;
    d.vec_cd = (pl->lc == GEMM_ROW_MAJOR && N % 4 == 0 &&
                reinterpret_cast<uintptr_t>(D) % (4 * osz) == 0 &&
                (beta == 0.0f || reinterpret_cast<uintptr_t>(C) % (4 * osz) == 0) &&
                reinterpret_cast<uintptr_t>(bias) % (4 * osz) == 0)
                   ? 1 : 0;
    // (AUTO picks it only when the schedule is AUTO too: a pinned schedule
    // asks for the tile kernels)
    const bool want_wk = cfg.tile == GEMM_TILE_WHOLEK ||
                         (cfg.tile == GEMM_TILE_AUTO && cfg.sched == GEMM_SCHED_AUTO && batch == 1 &&
                          !mx_a && wholek_auto(fam, M, N, K, cus));
    if (want_wk && !wholek_problem(fam, A, B, a_kc, b_kc, M, N, K, batch, mx_a != nullptr)) {
        d.wholek = wholek_steps(fam, K);
        d.sched = GEMM_SCHED_DATA_PARALLEL;
        d.tiles_m = (int)cdiv(M, 32);
        d.tiles_n = (int)cdiv(N, 32);
        if ((int64_t)d.tiles_m * d.tiles_n > 0x7FFFFFFFLL)
            return fail(GEMM_UNSUPPORTED, "whole-K kernel: more than 2^31 blocks");
        d.total = d.tiles_m * d.tiles_n;
        d.grid = d.total;
        d.ipt = 1;
        return GEMM_OK;
    }
    if (cfg.tile != GEMM_TILE_GENERIC) {
        // (a whole-K request it cannot take falls back to the heuristic tile)
        gemm_tile t = cfg.tile == GEMM_TILE_AUTO || cfg.tile == GEMM_TILE_WHOLEK
                          ? pick_tile(fam, M, N, K, cus, batch)
                          : cfg.tile;
        const KernelEntry *e = registry().find(fam, a_kc, b_kc, tile_id(t));
        if (!e) e = registry().find(fam, a_kc, b_kc, TILE_128x128);
        const char *why = nullptr;
        if (K > 0) {
            const int kb = e ? e->bk * esz : 128;
            why = operand_vec_problem(A, a_kc, a_kc ? K : M, e ? e->bm : 0, esz, kb);
            if (!why) why = operand_vec_problem(B, b_kc, b_kc ? K : N, e ? e->bn : 0, esz, kb);
        }
        // MX tile kernels copy each row's block scales of a k-tile (128
        // bytes of K: four blocks of e4m3, eight of e2m1) as whole words, at
        // 32-bit offsets
        if (!why && mx_a &&
            (K % 128 != 0 || reinterpret_cast<uintptr_t>(mx_a) % 4 != 0 ||
             reinterpret_cast<uintptr_t>(mx_b) % 4 != 0))
            why = fam == FAM_MXF4 ? "MXFP4 tile kernels need K % 256 == 0 and 4-byte aligned scale arrays"
                                  : "MX tile kernels need K % 128 == 0 and 4-byte aligned scale arrays";
        if (!why && mx_a && (M * (K_el / 32) > 0x7FFFFFFFLL || N * (K_el / 32) > 0x7FFFFFFFLL))
            why = "MX scale arrays beyond 2^31 bytes";
        if (e && !why) d.e = e;
        else d.why_generic = why ? why : "no tile kernel for this layout";
    } else {
        d.why_generic = "scalar-load kernel requested";
    }
    if (!d.e) {
        d.sched = GEMM_SCHED_DATA_PARALLEL;
        d.tiles_m = (int)cdiv(M, 64);
        d.tiles_n = (int)cdiv(N, 64);
        d.total = d.tiles_m * d.tiles_n;
        d.grid = d.total;
        return GEMM_OK;
    }
    const KernelEntry *e = d.e;
    const int64_t tm = cdiv(M, e->bm), tn = cdiv(N, e->bn), ipt = cdiv(K, e->bk);
    if (tm * tn * batch > 0x7FFFFFFFLL || ipt > 0x7FFFFFFFLL || tm * tn * batch * ipt > (1LL << 52))
        return fail(GEMM_UNSUPPORTED, "problem %lldx%lldx%lld (batch %lld) has too many tiles",
                    (long long)M, (long long)N, (long long)K, (long long)batch);
    d.tiles_m = (int)tm;
    d.tiles_n = (int)tn;
    // raster groups of 8 tile rows for 256x256 tiles: a workgroup wave then
    // covers 8 row panels x 32 column panels, which measured 1-2% faster than
    // groups of 4 on the transformer-layer shapes (fewer column-panel re-reads)
    d.group_m = e->tile == TILE_256x256 ? 8 : 4;
    d.ipt = (int)ipt;
    d.total = (int)(tm * tn * batch);
    int occ = 1;
    gemm_status st = occ_of(e, &occ);
    if (st != GEMM_OK) return st;
    int G = cus * occ;
    if (cfg.sk_grid > 0 && cfg.sk_grid < G) G = cfg.sk_grid;
    gemm_schedule s = cfg.sched;
    if (d.ipt == 0) s = GEMM_SCHED_DATA_PARALLEL;
    if (s == GEMM_SCHED_AUTO) {
        if (d.total >= G) {
            const int rem = d.total % G;
            const double eff = (double)d.total / (double)(cdiv(d.total, G) * G);
            s = (rem == 0 || eff >= 0.9 || d.ipt < 4) ? GEMM_SCHED_DATA_PARALLEL : GEMM_SCHED_HYBRID;
        } else {
            // fewer tiles than workgroup slots: nearly full waves run as they
            // are, otherwise stream-K over one workgroup per CU (on the
            // bandwidth-bound skinny shapes it beat split-K and two
            // workgroups per CU, which only add partial-tile traffic)
            if (d.ipt < 4 || (double)d.total >= 0.85 * G) s = GEMM_SCHED_DATA_PARALLEL;
            else s = GEMM_SCHED_STREAM_K;
        }
    }
    if (s == GEMM_SCHED_SPLIT_K && d.total >= G) s = GEMM_SCHED_DATA_PARALLEL;
    if (s == GEMM_SCHED_HYBRID && (d.total < G || d.total % G == 0))
        s = d.total < G ? GEMM_SCHED_STREAM_K : GEMM_SCHED_DATA_PARALLEL;
    d.sched = s;
    switch (s) {
    case GEMM_SCHED_DATA_PARALLEL:
        d.sk_tiles = 0;
        d.grid = d.total < G ? d.total : G;
        break;
    case GEMM_SCHED_STREAM_K: {
        // at least min_iters(fam) MAC iterations per workgroup, so the partial-tile
        // fixups stay small next to the work (an explicit sk_grid overrides)
        const int64_t kMinSkIters = min_iters(fam);
        d.sk_tiles = d.total;
        d.sk_iters = (int64_t)d.total * d.ipt;
        int64_t g = cfg.sk_grid > 0 ? d.sk_iters : d.sk_iters / kMinSkIters;
        if (g > G) g = G;
        if (cfg.sk_grid <= 0 && g > cus) g = cus;   // one stream-K workgroup per CU
        if (g < d.total && cfg.sk_grid <= 0) g = d.total < G ? d.total : G;
        d.grid = (int)(g > 0 ? g : 1);
        d.sk_grid = d.grid;   // g <= sk_iters in every branch above
        break;
    }
    case GEMM_SCHED_SPLIT_K: {
        // `split` interleaved K units per tile, each with >= min_iters(fam) k-tiles
        int S = G / d.total;
        if (S > d.ipt / min_iters(fam)) S = d.ipt / min_iters(fam);
        if (S < 1) S = 1;
        d.split = S;
        d.sk_tiles = d.total;
        d.grid = d.total * S;
        break;
    }
    default:   // hybrid: whole waves data-parallel, the remainder stream-K
        d.sk_tiles = d.total % G;
        d.sk_iters = (int64_t)d.sk_tiles * d.ipt;
        d.grid = G;
        // the remainder's iterations may be fewer than the grid: only as many
        // workgroups as there are iterations share them, so none holds an
        // empty range that its tile's arrival count would wait for
        d.sk_grid = (int)(d.sk_iters < G ? d.sk_iters : G);
        break;
    }
    // a fixed-size workspace (max_ws bytes of partial tiles): the stream-K
    // grid or the split-K factor shrinks until the partials fit; a hybrid
    // remainder that would no longer spread over the grid runs data-parallel
    if (max_ws > 0 && d.sk_tiles > 0 && d.split != 1) {
        const size_t slot = (size_t)e->bm * e->bn * sizeof(float);
        if (d.sched == GEMM_SCHED_SPLIT_K) {
            int S = d.split;
            while (S > 1 && (size_t)d.total * S * slot > max_ws) --S;
            d.split = S;
            d.grid = d.total * S;
            if (S == 1) {   // one unit per tile: a plain data-parallel launch
                d.sched = GEMM_SCHED_DATA_PARALLEL;
                d.split = 0;
                d.sk_tiles = 0;
                d.grid = d.total < G ? d.total : G;
            }
        } else if ((size_t)2 * d.sk_grid * slot > max_ws) {
            const int cap = (int)(max_ws / (2 * slot));
            if (d.sched == GEMM_SCHED_HYBRID || cap < 1) {
                d.sched = GEMM_SCHED_DATA_PARALLEL;
                d.sk_tiles = 0;
                d.sk_iters = 0;
                d.sk_grid = 0;
                d.grid = d.total < G ? d.total : G;
            } else {
                d.grid = cap;
                d.sk_grid = cap;
            }
        }
    }
    if (d.sk_tiles > 0 && d.split == 0 &&
        (d.sk_grid < 1 || d.sk_grid > d.grid || (int64_t)d.sk_grid > d.sk_iters))
        return fail(GEMM_HIP_ERROR, "internal: stream-K grid %d outside [1, min(grid %d, iterations %lld)]",
                    d.sk_grid, d.grid, (long long)d.sk_iters);
    return GEMM_OK;
}

gemm_status check_device(gemm_plan_s *pl, int *dev) {
    hipError_t e = hipGetDevice(dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (pl->device >= 0 && pl->device != *dev)
        return fail(GEMM_UNSUPPORTED, "plan is bound to device %d (first run) but device %d is current",
                    pl->device, *dev);
    pl->device = *dev;
    return GEMM_OK;
}

void note_stream(gemm_plan_s *pl, hipStream_t s) {
    pl->last_stream = s;
    pl->used = true;
}

// Make sure the stream-K workspace covers `slots` partial tiles and `ctr`
// counters; new counters are zeroed on `st` before any kernel that uses them.
gemm_status ensure_workspace(gemm_plan_s *pl, size_t partial_bytes, size_t ctr, hipStream_t st) {
    if (partial_bytes <= pl->partial_bytes && ctr <= pl->counter_count) return GEMM_OK;
    if (pl->used) {
        hipError_t e = hipStreamSynchronize(pl->last_stream);
        if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize (workspace growth)");
    }
    if (partial_bytes > pl->partial_bytes) {
        if (pl->partials) (void)hipFree(pl->partials);
        pl->partials = nullptr;
        pl->partial_bytes = 0;
        hipError_t e = hipMalloc(reinterpret_cast<void **>(&pl->partials), partial_bytes);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(GEMM_OUT_OF_MEMORY, "stream-K workspace of %zu bytes: %s", partial_bytes,
                        hipGetErrorString(e));
        }
        pl->partial_bytes = partial_bytes;
    }
    if (ctr > pl->counter_count) {
        if (pl->counters) (void)hipFree(pl->counters);
        pl->counters = nullptr;
        pl->counter_count = 0;
        const size_t n = ctr < 1024 ? 1024 : ctr;
        hipError_t e = hipMalloc(reinterpret_cast<void **>(&pl->counters), n * sizeof(int));
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(GEMM_OUT_OF_MEMORY, "stream-K counters: %s", hipGetErrorString(e));
        }
        e = launch_zero_u32(reinterpret_cast<uint32_t *>(pl->counters), n, st);
        if (e != hipSuccess) return hip_fail(e, "counter initialisation");
        pl->counter_count = n;
    }
    return GEMM_OK;
}

gemm_status validate_problem(const gemm_plan_s *pl, const void *A, const void *B, const void *C,
                             const void *D, int64_t M, int64_t N, int64_t K, float beta,
                             const char *where) {
    (void)pl;
    if (M < 0 || N < 0 || K < 0)
        return fail(GEMM_INVALID_ARG, "%s: negative size M=%lld N=%lld K=%lld", where, (long long)M,
                    (long long)N, (long long)K);
    if (M == 0 || N == 0) return GEMM_OK;
    if (!D) return fail(GEMM_INVALID_ARG, "%s: D is NULL", where);
    if (K > 0 && (!A || !B)) return fail(GEMM_INVALID_ARG, "%s: A or B is NULL with K > 0", where);
    if (beta != 0.0f && !C) return fail(GEMM_INVALID_ARG, "%s: C is NULL but beta != 0", where);
    if (M > (1LL << 40) || N > (1LL << 40) || K > (1LL << 40))
        return fail(GEMM_UNSUPPORTED, "%s: dimension beyond 2^40", where);
    return GEMM_OK;
}

Prob make_prob(const void *A, const void *B, const void *C, void *D, int64_t M, int64_t N, int64_t K,
               const Decision &d) {
    Prob p;
    p.A = static_cast<const char *>(A);
    p.B = static_cast<const char *>(B);
    p.C = static_cast<const char *>(C);
    p.D = static_cast<char *>(D);
    p.M = M;
    p.N = N;
    p.K = K;
    p.tiles_m = d.tiles_m;
    p.tiles_n = d.tiles_n;
    p.ipt = d.ipt;
    p.vec_cd = d.vec_cd;
    p.batch = 1;
    p.stride_a = p.stride_b = p.stride_c = p.stride_d = 0;
    p.mx_a = p.mx_b = nullptr;
    return p;
}

// Options of one run beyond a single GEMM: a strided batch (a single GEMM is
// batch 1 with zero strides) and MX block scales.
struct RunOpts {
    int64_t count = 1;
    int64_t sa = 0, sb = 0, sc = 0, sd = 0;   // element strides
    const uint8_t *mx_a = nullptr, *mx_b = nullptr;
    // auxiliary tensors of the epilogue (single GEMMs only)
    const void *aux = nullptr;
    void *aux_out = nullptr;
    int aux_op = 0, aux_after = 0;
    // gemm_plan_run_noalloc: partials and counters from the static workspace
    bool noalloc = false;
};

EpiArgs make_epi(const gemm_plan_s *pl, float alpha, float beta, const float *sa, const float *sb,
                 const void *bias, const RunOpts &ro = RunOpts()) {
    EpiArgs e;
    e.alpha = alpha;
    e.beta = beta;
    e.scale_a = sa;
    e.scale_b = sb;
    e.bias = bias;
    e.act = (int)pl->epi;
    e.lc_row = pl->lc == GEMM_ROW_MAJOR ? 1 : 0;
    e.aux = ro.aux;
    e.aux_out = ro.aux_out;
    e.aux_op = ro.aux_op;
    e.aux_after = ro.aux_after;
    return e;
}

gemm_status run_generic(const gemm_plan_s *pl, int fam, const Prob &p, const EpiArgs &ep,
                        hipStream_t st) {
    GenericArgs g;
    g.p = p;
    g.e = ep;
    g.la_row = pl->la == GEMM_ROW_MAJOR;
    g.lb_row = pl->lb == GEMM_ROW_MAJOR;
    hipError_t e = launch_generic(fam, g, st);
    if (e != hipSuccess) return hip_fail(e, "generic kernel launch");
    return GEMM_OK;
}

// ---- the static workspace of gemm_plan_run_noalloc ---------------------------
//
// Stream-K / split-K partial tiles followed by the arrival counters, in a
// file-scope device array: every device the library runs on holds one copy
// for the life of the process, so the entry point allocates nothing. In host
// code `scratch` only names the symbol; its device address on each device
// comes from hipGetSymbolAddress, taken once per device and kept.
constexpr size_t kNoAllocPartialBytes = (size_t)32 << 20;
constexpr size_t kNoAllocCounters = 16384;
static __device__ __align__(256) unsigned char scratch[kNoAllocPartialBytes + kNoAllocCounters * sizeof(int)];

std::mutex g_scratch_mu;
std::unordered_map<int, unsigned char *> g_scratch_ptr;

// The static workspace of device `dev` (current): its address, and on the
// first call its counters cleared (the fill kernel on `st`, then a wait for
// it, so calls on other streams find them clear); afterwards the finishing
// workgroup of every split tile resets its counter.
gemm_status noalloc_workspace(int dev, hipStream_t st, unsigned char **out) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    auto it = g_scratch_ptr.find(dev);
    if (it != g_scratch_ptr.end()) {
        *out = it->second;
        return GEMM_OK;
    }
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(st, &cs);
    if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
    if (cs != hipStreamCaptureStatusNone)
        return fail(GEMM_UNSUPPORTED,
                    "gemm_plan_run_noalloc: the first call on device %d initialises the static workspace "
                    "and must not be captured into a graph; make one uncaptured call first", dev);
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    unsigned char *base = static_cast<unsigned char *>(p);
    e = launch_zero_u32(reinterpret_cast<uint32_t *>(base + kNoAllocPartialBytes), kNoAllocCounters, st);
    if (e != hipSuccess) return hip_fail(e, "static workspace counter initialisation");
    e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize (static workspace initialisation)");
    g_scratch_ptr.emplace(dev, base);
    *out = base;
    return GEMM_OK;
}

gemm_status run_one(gemm_plan_s *pl, const void *A, const void *B, const void *C, void *D, int64_t M,
                    int64_t N, int64_t K, float alpha, float beta, const float *sa, const float *sb,
                    const void *bias, void *stream, const RunOpts &bt = RunOpts()) {
    if (!plan_ok(pl)) return fail(GEMM_NOT_INITIALIZED, "gemm_plan_run: invalid plan handle");
    gemm_status st = validate_problem(pl, A, B, C, D, M, N, K, beta, "gemm_plan_run");
    if (st != GEMM_OK) return st;
    if (pl->fam == FAM_MXF4 && !bt.mx_a && K > 0)
        return fail(GEMM_UNSUPPORTED, "F4_E2M1 elements are defined only under MX block scales: "
                    "use gemm_plan_run_mx");
    if (M == 0 || N == 0 || bt.count == 0) return ok();
    if (beta == 0.0f) C = nullptr;
    const int esz = elem_bytes(pl->fam), osz = out_bytes(pl->fam);
    // batch entries whose operands cannot keep the tile kernel's 16-byte
    // alignment (or whose tile count overflows) run one by one
    const bool batched = bt.count > 1;
    if (batched && ((bt.sa * esz) % 16 != 0 || (bt.sb * esz) % 16 != 0 || bt.sc % 4 != 0 ||
                    bt.sd % 4 != 0 || cdiv(M, 32) * cdiv(N, 32) * bt.count > 0x7FFFFFFFLL)) {
        for (int64_t b = 0; b < bt.count; ++b) {
            st = run_one(pl, static_cast<const char *>(A) + b * bt.sa * esz,
                         static_cast<const char *>(B) + b * bt.sb * esz,
                         C ? static_cast<const char *>(C) + b * bt.sc * osz : nullptr,
                         static_cast<char *>(D) + b * bt.sd * osz, M, N, K, alpha, beta, sa, sb, bias,
                         stream);
            if (st != GEMM_OK) return st;
        }
        return ok();
    }
    int dev = 0;
    if ((st = check_device(pl, &dev)) != GEMM_OK) return st;
    int cus = 0;
    if ((st = device_cus(dev, &cus)) != GEMM_OK) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    Decision d;
    st = decide(pl, A, B, C, D, bias, M, N, K, beta, cus,
                [&](const KernelEntry *e, int *occ) {
                    return kernel_occupancy(dev, e->fn_persistent, e->nt, occ);
                },
                d, bt.count, bt.mx_a, bt.mx_b, bt.noalloc ? kNoAllocPartialBytes : 0);
    if (st != GEMM_OK) return st;
    // the vector epilogue reads and writes the auxiliary tensors like C and D
    if (reinterpret_cast<uintptr_t>(bt.aux) % (4 * osz) != 0 ||
        reinterpret_cast<uintptr_t>(bt.aux_out) % (4 * osz) != 0)
        d.vec_cd = 0;
    const int fam = bt.mx_a ? mx_family(pl->fam) : pl->fam;
    Prob p = make_prob(A, B, C, D, M, N, K, d);
    p.batch = (int)bt.count;
    p.stride_a = bt.sa;
    p.stride_b = bt.sb;
    p.stride_c = bt.sc;
    p.stride_d = bt.sd;
    p.mx_a = bt.mx_a;
    p.mx_b = bt.mx_b;
    const EpiArgs ep = make_epi(pl, alpha, beta, sa, sb, bias, bt);
    if (d.wholek) {
        GenericArgs g;
        g.p = p;
        g.e = ep;
        g.la_row = pl->la == GEMM_ROW_MAJOR;
        g.lb_row = pl->lb == GEMM_ROW_MAJOR;
        hipError_t he = launch_wholek(fam, pl->la == GEMM_ROW_MAJOR, pl->lb == GEMM_COL_MAJOR,
                                      d.wholek, g, hs);
        if (he != hipSuccess) return hip_fail(he, "whole-K kernel launch");
        note_stream(pl, hs);
        return ok();
    }
    if (!d.e) {
        if (batched) {   // the scalar kernel takes one problem per launch
            for (int64_t b = 0; b < bt.count && st == GEMM_OK; ++b) {
                Prob q = make_prob(static_cast<const char *>(A) + b * bt.sa * esz,
                                   static_cast<const char *>(B) + b * bt.sb * esz,
                                   C ? static_cast<const char *>(C) + b * bt.sc * osz : nullptr,
                                   static_cast<char *>(D) + b * bt.sd * osz, M, N, K, d);
                st = run_generic(pl, fam, q, ep, hs);
            }
        } else {
            st = run_generic(pl, fam, p, ep, hs);
        }
        if (st == GEMM_OK) note_stream(pl, hs);
        return st == GEMM_OK ? ok() : st;
    }
    KArgs a;
    a.p = p;
    if (fam == FAM_MXF4) a.p.K = K / 2;   // the tile kernels address FP4 operands in bytes
    a.e = ep;
    a.s.grid = d.grid;
    a.s.total_tiles = d.total;
    a.s.sk_tiles = d.sk_tiles;
    a.s.sk_iters = d.sk_iters;
    a.s.sk_grid = d.sk_grid;
    a.s.group_m = d.group_m;
    a.s.xcd_remap = 1;
    a.s.split = d.split;
    a.s.partials = nullptr;
    a.s.counters = nullptr;
    a.s.gdesc = nullptr;
    a.s.gcount = 0;
    a.s.queue = nullptr;
    if (d.sk_tiles > 0 && d.split != 1) {
        const size_t pbytes = (size_t)2 * d.grid * d.e->bm * d.e->bn * sizeof(float);
        if (bt.noalloc) {
            // the partials the launch writes: 2 slots per stream-K workgroup,
            // one per split-K unit
            const size_t slot = (size_t)d.e->bm * d.e->bn * sizeof(float);
            const size_t need = d.split > 1 ? (size_t)d.grid * slot : (size_t)2 * d.sk_grid * slot;
            if (need > kNoAllocPartialBytes || (size_t)d.sk_tiles > kNoAllocCounters)
                return fail(GEMM_UNSUPPORTED,
                            "gemm_plan_run_noalloc: %s launch needs %zu bytes of partial tiles and %d "
                            "arrival counters; the static workspace holds %zu bytes and %zu counters "
                            "(use gemm_plan_run, or a data-parallel schedule)",
                            sched_name(d.sched), need, d.sk_tiles, kNoAllocPartialBytes, kNoAllocCounters);
            unsigned char *ws = nullptr;
            if ((st = noalloc_workspace(dev, hs, &ws)) != GEMM_OK) return st;
            a.s.partials = reinterpret_cast<float *>(ws);
            a.s.counters = reinterpret_cast<int *>(ws + kNoAllocPartialBytes);
        } else {
            if ((st = ensure_workspace(pl, pbytes, (size_t)d.sk_tiles, hs)) != GEMM_OK) return st;
            a.s.partials = pl->partials;
            a.s.counters = pl->counters;
        }
    }
    hipError_t e = d.e->run(a, d.grid, hs);
    if (e != hipSuccess) return hip_fail(e, "tile kernel launch");
    note_stream(pl, hs);
    return ok();
}

// Output element (kind 0: fp32, 1: fp16, 2: bf16) as a double.
double out_value(const uint8_t *p, int kind) {
    if (kind == 0) {
        float f;
        memcpy(&f, p, 4);
        return f;
    }
    uint16_t h;
    memcpy(&h, p, 2);
    if (kind == 2) {
        const uint32_t w = (uint32_t)h << 16;
        float f;
        memcpy(&f, &w, 4);
        return f;
    }
    const int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v = e == 0 ? std::ldexp((double)m, -24)
               : e == 31 ? (m ? NAN : INFINITY)
                         : std::ldexp((double)(m | 1024), e - 25);
    return sign ? -v : v;
}

// Two launches' outputs agree up to the order of the fp32 sums: the same
// elements are non-finite, and the finite ones differ by at most 4 units of
// the output's precision plus 1 % of the reference's root mean square (a
// stream-K partial that is lost or added twice moves an element by the size
// of a whole k-range's contribution, far beyond that). *bad: first mismatch.
bool outputs_agree(const std::vector<uint8_t> &ref, const std::vector<uint8_t> &got, int kind,
                   int64_t *bad) {
    const int sz = kind == 0 ? 4 : 2;
    const int64_t n = (int64_t)(ref.size() / sz);
    const double rel = kind == 0 ? 0x1p-22 : kind == 1 ? 0x1p-9 : 0x1p-6;   // 4 ulp (relative)
    double ss = 0.0;
    int64_t nf = 0;
    for (int64_t i = 0; i < n; ++i) {
        const double r = out_value(&ref[(size_t)i * sz], kind);
        if (std::isfinite(r)) {
            ss += r * r;
            ++nf;
        }
    }
    const double tol_abs = nf ? 0.01 * std::sqrt(ss / (double)nf) : 0.0;
    for (int64_t i = 0; i < n; ++i) {
        const double r = out_value(&ref[(size_t)i * sz], kind);
        const double g = out_value(&got[(size_t)i * sz], kind);
        const bool fr = std::isfinite(r), fg = std::isfinite(g);
        bool okv = fr == fg;
        if (okv && fr) okv = std::fabs(g - r) <= rel * std::fabs(r) + tol_abs;
        if (okv && !fr) okv = std::isnan(r) == std::isnan(g) && (std::isnan(r) || r == g);
        if (!okv) {
            *bad = i;
            return false;
        }
    }
    return true;
}

}  // namespace

// ------------------------------------------------------------------ C ABI

extern "C" {

gemm_status gemm_plan_create(gemm_plan_t *out, gemm_dtype a, gemm_dtype b, gemm_dtype c, gemm_dtype d,
                             gemm_dtype acc, gemm_layout la, gemm_layout lb, gemm_layout lc,
                             gemm_epilogue epi) {
    if (!out) return fail(GEMM_INVALID_ARG, "gemm_plan_create: out is NULL");
    *out = nullptr;
    auto bad_layout = [](gemm_layout l) { return l != GEMM_ROW_MAJOR && l != GEMM_COL_MAJOR; };
    if (bad_layout(la) || bad_layout(lb) || bad_layout(lc))
        return fail(GEMM_INVALID_ARG, "gemm_plan_create: layout must be ROW_MAJOR or COL_MAJOR");
    if (epi < GEMM_EPI_LINEAR || epi > GEMM_EPI_TANH)
        return fail(GEMM_INVALID_ARG, "gemm_plan_create: epilogue must be LINEAR, RELU, SIGMOID or TANH");
    int fam = -1;
    for (const Tuple &t : kSupported)
        if (t.a == a && t.b == b && t.c == c && t.d == d && t.acc == acc) fam = t.fam;
    if (fam < 0)
        return fail(GEMM_UNSUPPORTED,
                    "gemm_plan_create: element tuple (A=%s, B=%s, C=%s, D=%s, accumulator=%s) is not "
                    "supported; supported: (F32,F32,F32,F32,F32), (F16,F16,F16,F16,F32), "
                    "(BF16,BF16,BF16,BF16,F32), (F8_E4M3,F8_E4M3,BF16,BF16,F32), "
                    "(F4_E2M1,F4_E2M1,BF16,BF16,F32)",
                    dtype_name(a), dtype_name(b), dtype_name(c), dtype_name(d), dtype_name(acc));
    gemm_plan_s *p = new (std::nothrow) gemm_plan_s();
    if (!p) return fail(GEMM_OUT_OF_MEMORY, "gemm_plan_create: host allocation failed");
    p->magic = kMagic;
    p->a = a;
    p->b = b;
    p->c = c;
    p->d = d;
    p->acc = acc;
    p->la = la;
    p->lb = lb;
    p->lc = lc;
    p->epi = epi;
    p->fam = fam;
    p->sched = GEMM_SCHED_AUTO;
    p->tile = GEMM_TILE_AUTO;
    p->sk_grid = 0;
    p->device = -1;
    *out = p;
    return ok();
}

gemm_status gemm_plan_create_simple(gemm_plan_t *out, gemm_dtype element, gemm_layout layout,
                                    gemm_epilogue epi) {
    if (element == GEMM_F8_E4M3)
        return fail(GEMM_UNSUPPORTED,
                    "gemm_plan_create_simple: F8_E4M3 needs BF16 C/D; use gemm_plan_create");
    return gemm_plan_create(out, element, element, element, element, GEMM_F32, layout, layout, layout,
                            epi);
}

gemm_status gemm_plan_destroy(gemm_plan_t p) {
    if (!p) return ok();
    if (!plan_ok(p)) return fail(GEMM_NOT_INITIALIZED, "gemm_plan_destroy: invalid plan handle");
    gemm_status st = GEMM_OK;
    if (p->used || p->gevent_pending) {
        hipError_t e = hipStreamSynchronize(p->last_stream);
        if (e != hipSuccess) st = hip_fail(e, "gemm_plan_destroy: hipStreamSynchronize");
    }
    if (p->partials) (void)hipFree(p->partials);
    if (p->counters) (void)hipFree(p->counters);
    if (p->gdesc) (void)hipFree(p->gdesc);
    if (p->gevent) (void)hipEventDestroy(p->gevent);
    if (p->ghost) (void)hipHostFree(p->ghost);
    if (p->gqueue) (void)hipFree(p->gqueue);
    p->magic = 0;
    delete p;
    return st == GEMM_OK ? ok() : st;
}

gemm_status gemm_plan_set_config(gemm_plan_t p, gemm_schedule s, gemm_tile t, int32_t sk_grid) {
    if (!plan_ok(p)) return fail(GEMM_NOT_INITIALIZED, "gemm_plan_set_config: invalid plan handle");
    if (s < GEMM_SCHED_AUTO || s > GEMM_SCHED_SPLIT_K)
        return fail(GEMM_INVALID_ARG, "gemm_plan_set_config: unknown schedule %d", (int)s);
    if (t < GEMM_TILE_AUTO || t > GEMM_TILE_WHOLEK)
        return fail(GEMM_INVALID_ARG, "gemm_plan_set_config: unknown tile %d", (int)t);
    if (sk_grid < 0) return fail(GEMM_INVALID_ARG, "gemm_plan_set_config: sk_grid < 0");
    p->sched = s;
    p->tile = t;
    p->sk_grid = sk_grid;
    return ok();
}

gemm_status gemm_plan_run(gemm_plan_t p, const void *A, const void *B, const void *C, void *D, int64_t M,
                          int64_t N, int64_t K, float alpha, float beta, void *stream) {
    return run_one(p, A, B, C, D, M, N, K, alpha, beta, nullptr, nullptr, nullptr, stream);
}

gemm_status gemm_plan_run_noalloc(gemm_plan_t p, const void *A, const void *B, const void *C, void *D,
                                  int64_t M, int64_t N, int64_t K, float alpha, float beta,
                                  void *stream) {
    RunOpts ro;
    ro.noalloc = true;
    return run_one(p, A, B, C, D, M, N, K, alpha, beta, nullptr, nullptr, nullptr, stream, ro);
}

gemm_status gemm_plan_run_scaled(gemm_plan_t p, const void *A, const void *B, const void *C, void *D,
                                 int64_t M, int64_t N, int64_t K, float alpha, float beta,
                                 const float *scale_a, const float *scale_b, void *stream) {
    return run_one(p, A, B, C, D, M, N, K, alpha, beta, scale_a, scale_b, nullptr, stream);
}

gemm_status gemm_plan_run_batched(gemm_plan_t p, const void *A, const void *B, const void *C, void *D,
                                  const void *bias, int64_t M, int64_t N, int64_t K,
                                  int64_t batch_count, int64_t stride_a, int64_t stride_b,
                                  int64_t stride_c, int64_t stride_d, float alpha, float beta,
                                  const float *scale_a, const float *scale_b, void *stream) {
    if (!plan_ok(p)) return fail(GEMM_NOT_INITIALIZED, "gemm_plan_run_batched: invalid plan handle");
    if (batch_count < 0 || stride_a < 0 || stride_b < 0 || stride_c < 0 || stride_d < 0)
        return fail(GEMM_INVALID_ARG, "gemm_plan_run_batched: negative batch count or stride");
    if (batch_count > 1 && M > 0 && N > 0 && stride_d < M * N)
        return fail(GEMM_INVALID_ARG,
                    "gemm_plan_run_batched: stride_d = %lld < M*N = %lld makes the outputs overlap",
                    (long long)stride_d, (long long)(M * N));
    if (batch_count > 0x7FFFFFFFLL)
        return fail(GEMM_UNSUPPORTED, "gemm_plan_run_batched: batch count beyond 2^31");
    if (batch_count == 0) {   // nothing to read or write: NULL buffers are fine
        if (M < 0 || N < 0 || K < 0)
            return fail(GEMM_INVALID_ARG, "gemm_plan_run_batched: negative size");
        return ok();
    }
    RunOpts bt;
    bt.count = batch_count;
    bt.sa = stride_a;
    bt.sb = stride_b;
    bt.sc = stride_c;
    bt.sd = stride_d;
    return run_one(p, A, B, C, D, M, N, K, alpha, beta, scale_a, scale_b, bias, stream, bt);
}

gemm_status gemm_plan_run_mx(gemm_plan_t p, const void *A, const void *B, const void *C, void *D,
                             const void *bias, int64_t M, int64_t N, int64_t K, float alpha,
                             float beta, const uint8_t *mx_scale_a, const uint8_t *mx_scale_b,
                             void *stream) {
    if (!plan_ok(p)) return fail(GEMM_NOT_INITIALIZED, "gemm_plan_run_mx: invalid plan handle");
    if (p->fam != FAM_F8 && p->fam != FAM_MXF4)
        return fail(GEMM_UNSUPPORTED,
                    "gemm_plan_run_mx: MX block scaling needs an F8_E4M3 or F4_E2M1 plan");
    if (K % 32 != 0)
        return fail(GEMM_INVALID_ARG, "gemm_plan_run_mx: K = %lld is not a multiple of the "
                    "32-element MX block", (long long)K);
    if (M > 0 && N > 0 && K > 0 && (!mx_scale_a || !mx_scale_b))
        return fail(GEMM_INVALID_ARG, "gemm_plan_run_mx: a block-scale array is NULL");
    RunOpts ro;
    ro.mx_a = mx_scale_a;
    ro.mx_b = mx_scale_b;
    if (K == 0) ro.mx_a = ro.mx_b = nullptr;   // nothing to scale: beta*C (+bias) only
    return run_one(p, A, B, C, D, M, N, K, alpha, beta, nullptr, nullptr, bias, stream, ro);
}

gemm_status gemm_plan_run_aux(gemm_plan_t p, const void *A, const void *B, const void *C, void *D,
                              const void *bias, const void *aux, gemm_aux_op aux_op,
                              gemm_aux_pos aux_pos, void *aux_out, int64_t M, int64_t N, int64_t K,
                              float alpha, float beta, const float *scale_a, const float *scale_b,
                              void *stream) {
    if (!plan_ok(p)) return fail(GEMM_NOT_INITIALIZED, "gemm_plan_run_aux: invalid plan handle");
    if ((int)aux_op < GEMM_AUX_ADD || (int)aux_op > GEMM_AUX_DIV)
        return fail(GEMM_INVALID_ARG, "gemm_plan_run_aux: aux_op %d is not an elementwise op",
                    (int)aux_op);
    if (aux_pos != GEMM_AUX_BEFORE_ACT && aux_pos != GEMM_AUX_AFTER_ACT)
        return fail(GEMM_INVALID_ARG, "gemm_plan_run_aux: aux_pos %d is not a side of the "
                    "activation", (int)aux_pos);
    if (M > 0 && N > 0 && aux_out && aux_out == D)
        return fail(GEMM_INVALID_ARG, "gemm_plan_run_aux: aux_out and D are the same buffer");
    RunOpts ro;
    ro.aux = aux;
    ro.aux_out = aux_out;
    ro.aux_op = (int)aux_op;
    ro.aux_after = aux_pos == GEMM_AUX_AFTER_ACT ? 1 : 0;
    return run_one(p, A, B, C, D, M, N, K, alpha, beta, scale_a, scale_b, bias, stream, ro);
}

gemm_status gemm_plan_run_ex(gemm_plan_t p, const void *A, const void *B, const void *C, void *D,
                             const void *bias, int64_t M, int64_t N, int64_t K, float alpha,
                             float beta, const float *scale_a, const float *scale_b, void *stream) {
    return run_one(p, A, B, C, D, M, N, K, alpha, beta, scale_a, scale_b, bias, stream);
}

gemm_status grouped_gemm_run(gemm_plan_t pl, const gemm_problem *problems, int32_t count, float alpha,
                             float beta, void *stream) {
    if (!plan_ok(pl)) return fail(GEMM_NOT_INITIALIZED, "grouped_gemm_run: invalid plan handle");
    if (count < 0) return fail(GEMM_INVALID_ARG, "grouped_gemm_run: count < 0");
    if (pl->fam == FAM_MXF4)
        return fail(GEMM_UNSUPPORTED, "grouped_gemm_run: F4_E2M1 needs MX block scales, which "
                    "grouped GEMM does not take");
    if (count > 0 && !problems) return fail(GEMM_INVALID_ARG, "grouped_gemm_run: problems is NULL");
    for (int32_t i = 0; i < count; ++i) {
        const gemm_problem &q = problems[i];
        char where[64];
        snprintf(where, sizeof(where), "grouped_gemm_run problem %d", (int)i);
        gemm_status st = validate_problem(pl, q.A, q.B, q.C, q.D, q.M, q.N, q.K, beta, where);
        if (st != GEMM_OK) return st;
    }
    bool any = false;
    for (int32_t i = 0; i < count && !any; ++i) any = problems[i].M > 0 && problems[i].N > 0;
    if (!any) return ok();
    int dev = 0, cus = 0;
    gemm_status st = check_device(pl, &dev);
    if (st != GEMM_OK) return st;
    if ((st = device_cus(dev, &cus)) != GEMM_OK) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const bool a_kc = pl->la == GEMM_ROW_MAJOR, b_kc = pl->lb == GEMM_COL_MAJOR;
    const int esz = elem_bytes(pl->fam), osz = out_bytes(pl->fam);
    const EpiArgs ep = make_epi(pl, alpha, beta, nullptr, nullptr, nullptr);

    // Tile classes, one persistent launch each (256x256 only when the plan
    // pins that tile; problems it cannot take fall back to 128x128).
    struct Class {
        const KernelEntry *e;
        std::vector<GroupDesc> table;
        int64_t total;
    };
    Class cls[2];
    cls[0].e = registry().find(pl->fam, a_kc, b_kc, TILE_256x256);
    cls[1].e = registry().find(pl->fam, a_kc, b_kc, TILE_128x128);
    for (Class &c : cls) c.total = 0;
    const bool generic_only = pl->tile == GEMM_TILE_GENERIC;
    std::vector<int32_t> scalar_path;
    // Workgroups claim tiles in table order as they finish earlier ones;
    // listing the problems by decreasing K (the cost of each of their tiles)
    // hands out the costly tiles first and leaves the cheap ones to even out
    // the finish (longest-first). Results do not depend on the order.
    std::vector<int32_t> order((size_t)count);
    for (int32_t i = 0; i < count; ++i) order[(size_t)i] = i;
    std::stable_sort(order.begin(), order.end(),
                     [&](int32_t x, int32_t y) { return problems[x].K > problems[y].K; });
    for (int32_t i : order) {
        const gemm_problem &q = problems[i];
        if (q.M == 0 || q.N == 0) continue;
        const void *C = beta == 0.0f ? nullptr : q.C;
        // class: 128x128 (two workgroups per CU), which beat 256x256 tiles on
        // grouped problem mixes up to 2048 x 4096 x 4096 (1.47x on the
        // 64-problem fp16 benchmark, same-box); 256x256 when the plan pins it
        const int want = pl->tile == GEMM_TILE_256x256 ? 0 : 1;
        int c = -1;
        for (int k = want; k < 2 && c < 0 && !generic_only; ++k) {
            const KernelEntry *e = cls[k].e;
            if (!e) continue;
            const char *why = nullptr;
            if (q.K > 0) {
                why = operand_vec_problem(q.A, a_kc, a_kc ? q.K : q.M, e->bm, esz, e->bk * esz);
                if (!why) why = operand_vec_problem(q.B, b_kc, b_kc ? q.K : q.N, e->bn, esz, e->bk * esz);
            }
            if (!why) c = k;
        }
        if (c < 0) {
            scalar_path.push_back(i);
            continue;
        }
        const KernelEntry *e = cls[c].e;
        GroupDesc g;
        std::memset(&g, 0, sizeof(g));
        Decision d;
        d.tiles_m = (int)cdiv(q.M, e->bm);
        d.tiles_n = (int)cdiv(q.N, e->bn);
        d.ipt = (int)cdiv(q.K, e->bk);
        d.vec_cd = (pl->lc == GEMM_ROW_MAJOR && q.N % 4 == 0 &&
                    reinterpret_cast<uintptr_t>(q.D) % (4 * osz) == 0 &&
                    (!C || reinterpret_cast<uintptr_t>(C) % (4 * osz) == 0))
                       ? 1 : 0;
        g.p = make_prob(q.A, q.B, C, q.D, q.M, q.N, q.K, d);
        g.tile_start = (int)cls[c].total;
        cls[c].total += (int64_t)d.tiles_m * d.tiles_n;
        if (cls[c].total > 0x7FFFFFFFLL)
            return fail(GEMM_UNSUPPORTED, "grouped_gemm_run: more than 2^31 tiles");
        cls[c].table.push_back(g);
    }
    const size_t n_desc = cls[0].table.size() + cls[1].table.size();
    // A call with the same problem list as the last one on this stream reuses
    // the uploaded descriptors: the upload's completion event need not be
    // waited for (that wait stalled the host until the GPU had reached the
    // previous call, idling the GPU between back-to-back grouped launches).
    const size_t n0 = cls[0].table.size(), n1 = cls[1].table.size();
    const bool reuse = n_desc > 0 && n_desc == pl->gdesc_count && hs == pl->gdesc_stream &&
                       std::memcmp(pl->ghost, cls[0].table.data(), n0 * sizeof(GroupDesc)) == 0 &&
                       std::memcmp(pl->ghost + n0, cls[1].table.data(), n1 * sizeof(GroupDesc)) == 0;
    if (n_desc > 0 && !reuse) {
        const size_t bytes = n_desc * sizeof(GroupDesc);
        if (n_desc > pl->gdesc_cap) {
            if (pl->used || pl->gevent_pending) {
                hipError_t he = hipStreamSynchronize(pl->last_stream);
                if (he != hipSuccess) return hip_fail(he, "hipStreamSynchronize (descriptor growth)");
                pl->gevent_pending = false;
            }
            if (pl->gdesc) (void)hipFree(pl->gdesc);
            if (pl->ghost) (void)hipHostFree(pl->ghost);
            pl->gdesc = nullptr;
            pl->ghost = nullptr;
            pl->gdesc_cap = 0;
            pl->gdesc_count = 0;
            const size_t cap = n_desc < 64 ? 64 : n_desc;
            hipError_t he = hipMalloc(reinterpret_cast<void **>(&pl->gdesc), cap * sizeof(GroupDesc));
            if (he != hipSuccess) {
                (void)hipGetLastError();
                return fail(GEMM_OUT_OF_MEMORY, "grouped descriptor table: %s", hipGetErrorString(he));
            }
            he = hipHostMalloc(reinterpret_cast<void **>(&pl->ghost), cap * sizeof(GroupDesc),
                               hipHostMallocDefault);
            if (he != hipSuccess) {
                (void)hipGetLastError();
                return fail(GEMM_OUT_OF_MEMORY, "grouped pinned staging: %s", hipGetErrorString(he));
            }
            pl->gdesc_cap = cap;
        }
        if (!pl->gevent) {
            hipError_t he = hipEventCreateWithFlags(&pl->gevent, hipEventDisableTiming);
            if (he != hipSuccess) return hip_fail(he, "hipEventCreate");
        }
        if (pl->gevent_pending) {   // the previous upload must finish before reuse
            hipError_t he = hipEventSynchronize(pl->gevent);
            if (he != hipSuccess) return hip_fail(he, "hipEventSynchronize (descriptor staging)");
            pl->gevent_pending = false;
        }
        // one upload: the 256x256 class's descriptors, then the 128x128 class's
        std::memcpy(pl->ghost, cls[0].table.data(), cls[0].table.size() * sizeof(GroupDesc));
        std::memcpy(pl->ghost + cls[0].table.size(), cls[1].table.data(),
                    cls[1].table.size() * sizeof(GroupDesc));
        hipError_t he = hipMemcpyAsync(pl->gdesc, pl->ghost, bytes, hipMemcpyHostToDevice, hs);
        if (he != hipSuccess) return hip_fail(he, "hipMemcpyAsync (descriptor table)");
        he = hipEventRecord(pl->gevent, hs);
        if (he != hipSuccess) return hip_fail(he, "hipEventRecord");
        pl->gevent_pending = true;
        pl->gdesc_count = n_desc;
        pl->gdesc_stream = hs;
    }
    if (n_desc > 0 && !pl->gqueue) {
        // zeroed once here; each launch leaves it zeroed for the next
        hipError_t he = hipMalloc(reinterpret_cast<void **>(&pl->gqueue), 9 * sizeof(unsigned int));
        if (he != hipSuccess) {
            (void)hipGetLastError();
            pl->gqueue = nullptr;
            return fail(GEMM_OUT_OF_MEMORY, "grouped tile queue: %s", hipGetErrorString(he));
        }
        he = launch_zero_u32(pl->gqueue, 9, hs);
        if (he != hipSuccess) return hip_fail(he, "zeroing the grouped tile queue");
    }
    if (n_desc > 0) {
        hipError_t he;
        size_t first = 0;
        for (Class &c : cls) {
            if (c.table.empty()) continue;
            int occ = 1;
            if ((st = kernel_occupancy(dev, c.e->fn_persistent, c.e->nt, &occ)) != GEMM_OK) return st;
            // the persistent kernel with data-parallel tiles only; the kernel's
            // own problem is a placeholder (each tile reads its descriptor)
            KArgs ka;
            std::memset(&ka, 0, sizeof(ka));
            ka.p = c.table[0].p;
            ka.p.batch = 1;
            ka.e = ep;
            const int64_t G = (int64_t)cus * occ;
            ka.s.grid = (int)(c.total < G ? c.total : G);
            ka.s.total_tiles = (int)c.total;
            ka.s.group_m = c.e->bm >= 256 ? 8 : 4;
            ka.s.xcd_remap = 1;
            ka.s.gdesc = pl->gdesc + first;
            ka.s.gcount = (int)c.table.size();
            // Tiles of problems of different K cost different times: a
            // workgroup takes the next unclaimed tile when it is done with
            // one (problems are listed by decreasing K, so the costly tiles
            // go first). When every tile has the same number of k-tiles the
            // static round robin balances as well and saves each tile the
            // claim's device-scope atomic (~3 us a tile: 64 fp16 problems
            // of 1024 x 1024 x 128, 79 -> 58 us).
            bool same_k = true;
            for (const GroupDesc &g : c.table) same_k = same_k && g.p.ipt == c.table[0].p.ipt;
            ka.s.queue = same_k ? nullptr : pl->gqueue;
            he = c.e->run(ka, ka.s.grid, hs);
            if (he != hipSuccess) return hip_fail(he, "grouped kernel launch");
            first += c.table.size();
        }
        note_stream(pl, hs);
    }
    for (int32_t i : scalar_path) {
        const gemm_problem &q = problems[i];
        Decision d;
        d.vec_cd = 0;
        const Prob p = make_prob(q.A, q.B, beta == 0.0f ? nullptr : q.C, q.D, q.M, q.N, q.K, d);
        if ((st = run_generic(pl, pl->fam, p, ep, hs)) != GEMM_OK) return st;
        note_stream(pl, hs);
    }
    return ok();
}

gemm_status gemm_plan_describe(gemm_plan_t pl, int64_t M, int64_t N, int64_t K, int32_t num_cus, char *buf,
                               int32_t len) {
    return gemm_plan_describe_batched(pl, M, N, K, 1, num_cus, buf, len);
}

gemm_status gemm_plan_describe_batched(gemm_plan_t pl, int64_t M, int64_t N, int64_t K,
                                       int64_t batch_count, int32_t num_cus, char *buf,
                                       int32_t len) {
    if (!plan_ok(pl)) return fail(GEMM_NOT_INITIALIZED, "gemm_plan_describe: invalid plan handle");
    if (!buf || len <= 0) return fail(GEMM_INVALID_ARG, "gemm_plan_describe: empty buffer");
    if (M < 0 || N < 0 || K < 0) return fail(GEMM_INVALID_ARG, "gemm_plan_describe: negative size");
    if (batch_count < 1 || batch_count > 0x7FFFFFFFLL)
        return fail(GEMM_INVALID_ARG, "gemm_plan_describe: batch_count outside [1, 2^31)");
    const int cus = num_cus > 0 ? num_cus : 256;
    // aligned stand-in pointers: describes the vector-load path
    const void *fake = reinterpret_cast<const void *>(uintptr_t(1) << 20);
    Decision d;
    gemm_status st = decide(pl, fake, fake, fake, fake, nullptr, M, N, K, 1.0f, cus,
                            [](const KernelEntry *e, int *occ) {
                                *occ = static_occupancy(e);
                                return GEMM_OK;
                            },
                            d, batch_count);
    if (st != GEMM_OK) return st;
    snprintf(buf, (size_t)len,
             "{\"kernel\": \"%s\", \"tile\": \"%s\", \"bk\": %d, \"waves\": %d, \"schedule\": \"%s\", "
             "\"tiles\": %d, \"ipt\": %d, \"sk_tiles\": %d, \"split\": %d, \"grid\": %d, "
             "\"sk_grid\": %d, \"sk_iters\": %lld, \"generic_reason\": \"%s\"}",
             d.wholek ? "wholek" : d.e ? "tile" : "generic", d.wholek ? "wholek32x32" : tile_name(d.e),
             d.wholek ? 8 * d.wholek * (pl->fam == FAM_F32 ? 4 : 8) : d.e ? d.e->bk : 16,
             d.e ? d.e->nt / 64 : d.wholek == 32 ? 8 : 4,
             sched_name(d.sched), d.total, d.ipt, d.sk_tiles, d.split, d.grid, d.sk_grid,
             (long long)d.sk_iters, d.why_generic);
    return ok();
}

gemm_status gemm_plan_profile(gemm_plan_t pl, const void *A, const void *B, const void *C, void *D,
                              int64_t M, int64_t N, int64_t K, float alpha, float beta,
                              int32_t iters, gemm_config *results, int32_t max_results,
                              int32_t *n_results, void *stream) {
    if (!plan_ok(pl)) return fail(GEMM_NOT_INITIALIZED, "gemm_plan_profile: invalid plan handle");
    if (iters < 1 || iters > 100000)
        return fail(GEMM_INVALID_ARG, "gemm_plan_profile: iters = %d outside [1, 100000]", (int)iters);
    if (max_results < 0 || (max_results > 0 && !results))
        return fail(GEMM_INVALID_ARG, "gemm_plan_profile: results array missing");
    gemm_status st = validate_problem(pl, A, B, C, D, M, N, K, beta, "gemm_plan_profile");
    if (st != GEMM_OK) return st;
    if (beta != 0.0f && C == D && M > 0 && N > 0)
        return fail(GEMM_INVALID_ARG, "gemm_plan_profile: D == C with beta != 0 would feed each "
                    "timed run the previous run's output");
    if (n_results) *n_results = 0;
    if (M == 0 || N == 0) return ok();
    int dev = 0, cus = 0;
    if ((st = check_device(pl, &dev)) != GEMM_OK) return st;
    if ((st = device_cus(dev, &cus)) != GEMM_OK) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const Cfg saved{pl->sched, pl->tile, pl->sk_grid};
    struct Cand {
        gemm_config c;
        const KernelEntry *e;
        int sched, grid, split, wholek;
    };
    std::vector<Cand> done;
    hipEvent_t ev[2] = {nullptr, nullptr};
    hipError_t he = hipEventCreate(&ev[0]);
    if (he == hipSuccess) he = hipEventCreate(&ev[1]);
    if (he != hipSuccess) {
        if (ev[0]) (void)hipEventDestroy(ev[0]);
        return hip_fail(he, "gemm_plan_profile: hipEventCreate");
    }
    const int osz = out_bytes(pl->fam);
    std::vector<uint8_t> ref((size_t)(M * N) * osz), got((size_t)(M * N) * osz);
    const gemm_tile tiles[] = {GEMM_TILE_256x256, GEMM_TILE_128x128, GEMM_TILE_64x256,
                               GEMM_TILE_32x256, GEMM_TILE_GENERIC, GEMM_TILE_WHOLEK};
    const gemm_schedule scheds[] = {GEMM_SCHED_DATA_PARALLEL, GEMM_SCHED_STREAM_K,
                                    GEMM_SCHED_HYBRID, GEMM_SCHED_SPLIT_K};
    for (gemm_tile t : tiles) {
        for (gemm_schedule s : scheds) {
            pl->sched = s;
            pl->tile = t;
            pl->sk_grid = 0;
            // what this candidate launches; identical launches are timed once
            Decision d;
            st = decide(pl, A, B, beta == 0.0f ? nullptr : C, D, nullptr, M, N, K, beta, cus,
                        [&](const KernelEntry *e, int *occ) {
                            return kernel_occupancy(dev, e->fn_persistent, e->nt, occ);
                        },
                        d);
            if (st == GEMM_UNSUPPORTED) {   // e.g. too many tiles of this shape: skip it
                st = GEMM_OK;
                continue;
            }
            if (st != GEMM_OK) break;
            bool dup = false;
            for (const Cand &c : done)
                dup |= c.e == d.e && c.sched == (int)d.sched && c.grid == d.grid &&
                       c.split == d.split && c.wholek == d.wholek;
            if (dup) continue;
            // the resolved choice (the registry may fall back to another
            // tile), so the report names what ran and a cached entry
            // reproduces this launch
            pl->sched = d.sched;
            pl->tile = d.wholek ? GEMM_TILE_WHOLEK : d.e ? tile_enum(d.e->tile) : GEMM_TILE_GENERIC;
            // the untimed run writes into a NaN-filled D, and its result must
            // match the first candidate's (up to summation order) before this
            // launch may be timed and cached: an output the launch fails to
            // write, or gets wrong, fails loudly instead of timing fast
            he = hipMemsetAsync(D, 0xFF, (size_t)(M * N) * osz, hs);
            if (he != hipSuccess) break;
            st = run_one(pl, A, B, C, D, M, N, K, alpha, beta, nullptr, nullptr, nullptr, stream);
            if (st == GEMM_OK) {
                he = hipMemcpyAsync(done.empty() ? ref.data() : got.data(), D, (size_t)(M * N) * osz,
                                    hipMemcpyDeviceToHost, hs);
                if (he == hipSuccess) he = hipStreamSynchronize(hs);
                if (he != hipSuccess) break;
                if (!done.empty()) {
                    int64_t bad = -1;
                    if (!outputs_agree(ref, got, osz == 4 ? 0 : pl->d == GEMM_F16 ? 1 : 2, &bad)) {
                        const int64_t i = pl->lc == GEMM_ROW_MAJOR ? bad / N : bad % M;
                        const int64_t j = pl->lc == GEMM_ROW_MAJOR ? bad % N : bad / M;
                        st = fail(GEMM_HIP_ERROR,
                                  "gemm_plan_profile: %s %s (grid %d) disagrees with %s %s at D[%lld][%lld]",
                                  d.wholek ? "wholek32x32" : tile_name(d.e), sched_name(d.sched), d.grid,
                                  done[0].wholek ? "wholek32x32" : tile_name(done[0].e),
                                  sched_name((gemm_schedule)done[0].sched), (long long)i, (long long)j);
                        break;
                    }
                }
            }
            if (st == GEMM_OK) he = hipEventRecord(ev[0], hs);
            for (int32_t r = 0; r < iters && st == GEMM_OK && he == hipSuccess; ++r)
                st = run_one(pl, A, B, C, D, M, N, K, alpha, beta, nullptr, nullptr, nullptr,
                             stream);
            if (st == GEMM_OK && he == hipSuccess) he = hipEventRecord(ev[1], hs);
            if (st == GEMM_OK && he == hipSuccess) he = hipEventSynchronize(ev[1]);
            float ms = 0.0f;
            if (st == GEMM_OK && he == hipSuccess) he = hipEventElapsedTime(&ms, ev[0], ev[1]);
            if (st != GEMM_OK || he != hipSuccess) break;
            Cand c;
            c.c.schedule = pl->sched;
            c.c.tile = pl->tile;
            c.c.sk_grid = 0;
            c.c.grid = d.grid;
            c.c.us = ms * 1000.0f / (float)iters;
            c.e = d.e;
            c.sched = (int)d.sched;
            c.grid = d.grid;
            c.split = d.split;
            c.wholek = d.wholek;
            done.push_back(c);
        }
        if (st != GEMM_OK || he != hipSuccess) break;
    }
    pl->sched = saved.sched;
    pl->tile = saved.tile;
    pl->sk_grid = saved.sk_grid;
    (void)hipEventDestroy(ev[0]);
    (void)hipEventDestroy(ev[1]);
    if (he != hipSuccess) return hip_fail(he, "gemm_plan_profile: timing");
    if (st != GEMM_OK) return st;
    std::stable_sort(done.begin(), done.end(),
                     [](const Cand &x, const Cand &y) { return x.c.us < y.c.us; });
    if (!done.empty()) {
        const gemm_config &b = done.front().c;
        pl->tuned[{M, N, K, 0}] = gemm_plan_s::Tuned{b.schedule, b.tile, b.sk_grid, b.us};
    }
    const int32_t n = (int32_t)std::min<size_t>(done.size(), (size_t)max_results);
    for (int32_t i = 0; i < n; ++i) results[i] = done[i].c;
    if (n_results) *n_results = (int32_t)done.size();
    return ok();
}

gemm_status gemm_plan_cache_export(gemm_plan_t pl, char *buf, int32_t len, int32_t *needed) {
    if (!plan_ok(pl)) return fail(GEMM_NOT_INITIALIZED, "gemm_plan_cache_export: invalid plan handle");
    std::string s;
    char tmp[512];
    snprintf(tmp, sizeof tmp,
             "{\"format\": \"%s\", \"version\": 1, \"arch\": \"gfx950\", \"plan\": {\"a\": \"%s\", "
             "\"b\": \"%s\", \"c\": \"%s\", \"d\": \"%s\", \"acc\": \"%s\", \"layout_a\": \"%s\", "
             "\"layout_b\": \"%s\", \"layout_c\": \"%s\"}, \"entries\": [",
             kCacheFormat, dtype_name(pl->a), dtype_name(pl->b), dtype_name(pl->c),
             dtype_name(pl->d), dtype_name(pl->acc), layout_str(pl->la), layout_str(pl->lb),
             layout_str(pl->lc));
    s += tmp;
    bool first = true;
    for (const auto &kv : pl->tuned) {
        snprintf(tmp, sizeof tmp,
                 "%s\n  {\"m\": %lld, \"n\": %lld, \"k\": %lld, \"mx\": %d, \"schedule\": \"%s\", "
                 "\"tile\": \"%s\", \"sk_grid\": %d, \"us\": %.3f}",
                 first ? "" : ",", (long long)kv.first.m, (long long)kv.first.n,
                 (long long)kv.first.k, kv.first.mx, sched_name(kv.second.sched),
                 tile_enum_name(kv.second.tile), kv.second.sk_grid, (double)kv.second.us);
        s += tmp;
        first = false;
    }
    s += "]}\n";
    const int64_t need = (int64_t)s.size() + 1;
    if (need > 0x7FFFFFFFLL) return fail(GEMM_UNSUPPORTED, "gemm_plan_cache_export: cache too large");
    if (needed) *needed = (int32_t)need;
    if (!buf) return ok();   // size query
    if (len < need)
        return fail(GEMM_INVALID_ARG, "gemm_plan_cache_export: buffer of %d bytes, needs %lld",
                    (int)len, (long long)need);
    memcpy(buf, s.c_str(), (size_t)need);
    return ok();
}

gemm_status gemm_plan_cache_import(gemm_plan_t pl, const char *json) {
    if (!plan_ok(pl)) return fail(GEMM_NOT_INITIALIZED, "gemm_plan_cache_import: invalid plan handle");
    if (!json) return fail(GEMM_INVALID_ARG, "gemm_plan_cache_import: text is NULL");
    JParser jp(json);
    JVal root;
    if (!jp.value(&root))
        return fail(GEMM_INVALID_ARG, "gemm_plan_cache_import: bad JSON at byte %zu: %s", jp.i,
                    jp.err ? jp.err : "?");
    jp.ws();
    if (jp.i != jp.n)
        return fail(GEMM_INVALID_ARG, "gemm_plan_cache_import: text after the JSON value at byte %zu",
                    jp.i);
    std::string fmt;
    int64_t ver = 0;
    if (root.kind != JVal::OBJ || !json_str(root.get("format"), &fmt) || fmt != kCacheFormat ||
        !json_int(root.get("version"), 1, 1, &ver))
        return fail(GEMM_INVALID_ARG, "gemm_plan_cache_import: not a version-1 %s document",
                    kCacheFormat);
    // the cache must come from a plan with the same types and layouts
    const JVal *plan = root.get("plan");
    const char *want[8][2] = {{"a", dtype_name(pl->a)},          {"b", dtype_name(pl->b)},
                              {"c", dtype_name(pl->c)},          {"d", dtype_name(pl->d)},
                              {"acc", dtype_name(pl->acc)},      {"layout_a", layout_str(pl->la)},
                              {"layout_b", layout_str(pl->lb)}, {"layout_c", layout_str(pl->lc)}};
    if (!plan || plan->kind != JVal::OBJ)
        return fail(GEMM_INVALID_ARG, "gemm_plan_cache_import: missing \"plan\" object");
    for (const auto &w : want) {
        std::string v;
        if (!json_str(plan->get(w[0]), &v) || v != w[1])
            return fail(GEMM_UNSUPPORTED,
                        "gemm_plan_cache_import: cache written for %s = %s, this plan has %s",
                        w[0], v.empty() ? "(missing)" : v.c_str(), w[1]);
    }
    const JVal *ents = root.get("entries");
    if (!ents || ents->kind != JVal::ARR)
        return fail(GEMM_INVALID_ARG, "gemm_plan_cache_import: missing \"entries\" array");
    std::map<gemm_plan_s::TunedKey, gemm_plan_s::Tuned> add;
    for (size_t i = 0; i < ents->arr.size(); ++i) {
        const JVal &e = ents->arr[i];
        int64_t m, n, k, mx = 0, skg = 0;
        std::string ss, ts;
        gemm_schedule sc;
        gemm_tile tl;
        const int64_t big = (int64_t)1 << 40;
        const bool good = e.kind == JVal::OBJ && json_int(e.get("m"), 0, big, &m) &&
                          json_int(e.get("n"), 0, big, &n) && json_int(e.get("k"), 0, big, &k) &&
                          (!e.get("mx") || json_int(e.get("mx"), 0, 1, &mx)) &&
                          (!e.get("sk_grid") || json_int(e.get("sk_grid"), 0, 1 << 20, &skg)) &&
                          json_str(e.get("schedule"), &ss) && parse_sched(ss, &sc) &&
                          json_str(e.get("tile"), &ts) && parse_tile(ts, &tl);
        if (!good)
            return fail(GEMM_INVALID_ARG, "gemm_plan_cache_import: entry %zu is malformed (needs "
                        "integer m, n, k, a known schedule and tile)", i);
        float us = 0.0f;
        const JVal *u = e.get("us");
        if (u && u->kind == JVal::NUM) us = (float)u->num;
        add[{m, n, k, (int)mx}] = gemm_plan_s::Tuned{sc, tl, (int)skg, us};
    }
    for (const auto &kv : add) pl->tuned[kv.first] = kv.second;   // later entries win
    return ok();
}

int32_t gemm_plan_cache_size(gemm_plan_t pl) {
    if (!plan_ok(pl)) return -1;
    return (int32_t)std::min<size_t>(pl->tuned.size(), 0x7FFFFFFF);
}

gemm_status gemm_plan_cache_clear(gemm_plan_t pl) {
    if (!plan_ok(pl)) return fail(GEMM_NOT_INITIALIZED, "gemm_plan_cache_clear: invalid plan handle");
    pl->tuned.clear();
    return ok();
}

const char *gemm_last_error(void) { return g_err.c_str(); }

const char *gemm_status_string(gemm_status s) {
    switch (s) {
    case GEMM_OK: return "GEMM_OK";
    case GEMM_INVALID_ARG: return "GEMM_INVALID_ARG";
    case GEMM_UNSUPPORTED: return "GEMM_UNSUPPORTED";
    case GEMM_HIP_ERROR: return "GEMM_HIP_ERROR";
    case GEMM_OUT_OF_MEMORY: return "GEMM_OUT_OF_MEMORY";
    case GEMM_NOT_INITIALIZED: return "GEMM_NOT_INITIALIZED";
    }
    return "GEMM_UNKNOWN_STATUS";
}

int32_t gemm_supported_count(void) { return kNumSupported; }

gemm_status gemm_supported_get(int32_t i, gemm_dtype *a, gemm_dtype *b, gemm_dtype *c, gemm_dtype *d,
                               gemm_dtype *acc) {
    if (i < 0 || i >= kNumSupported) return fail(GEMM_INVALID_ARG, "gemm_supported_get: index %d", (int)i);
    if (a) *a = kSupported[i].a;
    if (b) *b = kSupported[i].b;
    if (c) *c = kSupported[i].c;
    if (d) *d = kSupported[i].d;
    if (acc) *acc = kSupported[i].acc;
    return ok();
}

const char *gemm_version(void) { return "mi355-gemm 0.1.0 (gfx950)"; }

}  // extern "C"
