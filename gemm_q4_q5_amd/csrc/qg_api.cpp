// Host side of libqgemm: the C ABI declared in include/qgemm.h.
//
// Every entry point validates all of its arguments on the host before touching
// the HIP runtime, so a bad call returns a QG_ERR_* code, launches nothing, and
// can be exercised without a GPU.  The arithmetic of a weight row -- its K phases
// and the order their sums are added in -- is a function of (type, m, k) only
// (TandemLLM Kernels page, "Row invariance": tables keyed by the weight's shape,
// never by the row count).  How many waves and workgroups carry those phases, and
// whether x is staged per wave or per workgroup, also follow n: none of it changes
// a row's instructions or their order.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>

#include "qgemm.h"
#include "qg_kernels.h"
#include "qg_prefill.h"
#include "qg_mma_launch.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool known_type(int32_t t) { return t == QG_Q4_K || t == QG_Q5_K || t == QG_Q6_K || t == QG_NVFP4 || t == QG_FP8; }
bool has_scales(int32_t t) { return t == QG_NVFP4 || t == QG_FP8; }

const char *type_name(int32_t t) {
    switch (t) {
    case QG_Q4_K: return "Q4_K";
    case QG_Q5_K: return "Q5_K";
    case QG_Q6_K: return "Q6_K";
    case QG_NVFP4: return "NVFP4";
    case QG_FP8: return "FP8";
    default: return "?";
    }
}

// Largest m * k accepted (keeps every row and element index inside the kernels'
// 32-bit row counters and 64-bit offsets).
constexpr int64_t kMaxM = (int64_t)1 << 30;
constexpr int64_t kMaxK = (int64_t)1 << 20;

int check_weight(const qg_weight *w, const char *name) {
    if (!w) return fail(QG_ERR_NULL, "%s: weight descriptor is NULL", name);
    if (!known_type(w->type)) return fail(QG_ERR_TYPE, "%s: unknown type %d", name, w->type);
    if (w->layout != QG_LAYOUT_ROWS && w->layout != QG_LAYOUT_TILES)
        return fail(QG_ERR_TYPE, "%s: unknown layout %d", name, w->layout);
    if (w->layout == QG_LAYOUT_TILES && has_scales(w->type))
        return fail(QG_ERR_TYPE, "%s: the tiled layout is for the K-quants only", name);
    if (!w->data) return fail(QG_ERR_NULL, "%s: data is NULL", name);
    if (has_scales(w->type) && !w->scales) return fail(QG_ERR_NULL, "%s: %s scales are NULL", name, type_name(w->type));
    if (w->m < 1 || w->m > kMaxM) return fail(QG_ERR_SHAPE, "%s: m = %lld out of range", name, (long long)w->m);
    if (w->k < 256 || w->k > kMaxK || w->k % 256)
        return fail(QG_ERR_SHAPE, "%s: k = %lld must be a positive multiple of 256 (<= %lld)", name,
                    (long long)w->k, (long long)kMaxK);
    if (!aligned(w->data, 16)) return fail(QG_ERR_ALIGN, "%s: data is not 16-byte aligned", name);
    if (has_scales(w->type) && !aligned(w->scales, 16))
        return fail(QG_ERR_ALIGN, "%s: scales are not 16-byte aligned", name);
    return QG_OK;
}

int check_x(const void *x) {
    if (!x) return fail(QG_ERR_NULL, "x is NULL");
    if (!aligned(x, 16)) return fail(QG_ERR_ALIGN, "x is not 16-byte aligned");
    return QG_OK;
}

int check_y(const float *y, const char *name) {
    if (!y) return fail(QG_ERR_NULL, "%s is NULL", name);
    if (!aligned(y, 4)) return fail(QG_ERR_ALIGN, "%s is not 4-byte aligned", name);
    return QG_OK;
}

int check_rows(int32_t n) {
    if (n < 1 || n > QG_MAX_ROWS) return fail(QG_ERR_ROWS, "n = %d outside 1..%d", n, QG_MAX_ROWS);
    return QG_OK;
}

// Waves splitting K for one row tile of 16 rows: a pure function of (type, m, k),
// so a row's partial sums -- and its bits -- never depend on n or on the other
// matrices of a launch.  Doubles (up to 16, while every wave keeps a superblock)
// until each wave's superblocks fit one round of loads in flight (kMmaDepth) and
// the matrix yields at least 256 waves.
int choose_ks(int32_t type, int64_t m, int64_t k) {
    (void)type;
    const int64_t tiles = (m + 15) / 16, nb = k / 256;
    int ks = 1;
    while (ks < 16 && 2 * ks <= nb && ((nb + ks - 1) / ks > qg::kMmaDepth || tiles * ks < 256)) ks *= 2;
    return ks;
}

constexpr size_t kMmaLdsBudget = 65536;   // two workgroups per CU
constexpr size_t kMmaLdsMax = 163840;      // all of a CU's LDS, for grids of at most one workgroup per CU
constexpr size_t kMmaBytesPerTokSb = 4 * 9 * 16;   // staged x per token and superblock (units of 16 B)
constexpr size_t kMmaZeroBytes = 9 * 16;

// Assemble and launch one MFMA-path call over `nseg` matrices sharing x
// (SwiGLU: w[0] gate and w[1] up, served by the same lanes).
int run_mma(const qg_weight *const *w, float *const *y, const float *resid, int nseg, const void *x, int32_t n,
            int mode, void *stream) {
    qg::MmaArgs a;
    memset(&a, 0, sizeof a);
    const int64_t k = w[0]->k;
    const bool sw = mode == qg::MODE_SWIGLU;
    // Every matrix is a segment of one-tile waves, except SwiGLU: one segment whose tile
    // groups come in pairs (gate rows, then the same up rows) in one workgroup, the
    // gate group handing its sums to the up group, which stores silu(g) * u.
    const int pair = sw ? 2 : 1;   // tile groups per block of 16 output rows
    a.x = x;
    a.nmagic = n >= 2 ? (uint32_t)((1ull << 32) / (uint64_t)n + 1) : 0u;
    a.nseg = sw ? 1 : nseg;
    a.k = (int32_t)k;
    a.nb = (int32_t)(k / 256);
    a.n = n;
    a.mode = mode;
    a.nt = 1;
    // K phases of each matrix (fixed by its shape: the arithmetic of every row).
    int ks[3] = {1, 1, 1};
    int ksmax = 1, ksmin = 16;
    for (int s = 0; s < nseg; ++s) {
        ks[s] = choose_ks(w[s]->type, w[s]->m, k);
        ksmax = std::max(ksmax, ks[s]);
        ksmin = std::min(ksmin, ks[s]);
    }
    const int ng = n > 16 ? 2 : 1;
    const size_t per_sb = (size_t)n * kMmaBytesPerTokSb;
    // Decode path (each wave stages its own x, one phase per wave) where a wave's
    // superblocks fit one round of loads and their x (16 items of 32 bytes per
    // superblock and token) kMmaDecRounds rounds of two items per lane.
    const int depth = qg::kMmaDepth;
    auto dec_ok = [&](int s, int wv) {
        const int maxcnt = (a.nb + ks[s] - 1) / ks[s];
        const size_t need = kMmaZeroBytes + (size_t)wv * maxcnt * per_sb;
        return maxcnt <= depth && 16 * n * maxcnt <= 128 * qg::kMmaDecRounds && need <= kMmaLdsBudget;
    };
    bool has_q6 = false;
    for (int s = 0; s < nseg; ++s) has_q6 = has_q6 || w[s]->type == QG_Q6_K;
    bool one_type = true;
    for (int s = 1; s < nseg; ++s) one_type = one_type && w[s]->type == w[0]->type;
    // Several phases per wave take one weight type per launch.
    const int np_max = one_type ? 4 : 1;
    // SwiGLU's paired tile groups need 2 * ks / np <= 16 waves per workgroup.
    const int np_min = sw ? std::max(1, 2 * ksmax / 16) : 1;
    // Rows per workgroup: 16 * wv / (ks / np) / pair for each matrix.
    auto grid_for = [&](int wv, int np) {
        int gr = 0;
        for (int s = 0; s < a.nseg; ++s) {
            const int64_t rows_per_wg = 16 * (wv / (ks[s] / np)) / pair;
            gr += (int)((w[s]->m + rows_per_wg - 1) / rows_per_wg);
        }
        return gr;
    };
    // Phases per wave (np) and waves per workgroup (wv).  Only the number of waves
    // serving a tile changes with np, never a row's arithmetic, so both may follow n.
    // A wave with np phases streams np times the superblocks and a workgroup serves
    // np times the rows, which shares each staged chunk of x among more rows.
    constexpr int kCUs = 256;
    constexpr int kOneRound = 320;
    int np = 1, wv = 0;
    bool any_dec = false;
    for (int s = 0; s < a.nseg; ++s) any_dec = any_dec || dec_ok(s, std::max(4, ksmax));
    if (n < 8) {
        // Below 8 tokens the decode path (np = 1) stays whenever its workgroups are at
        // most 8 waves; otherwise np = 2 or 4 where at least 4096 waves (16 per CU)
        // remain: 16384x8192 FP8 / NVFP4 at one token 38.6 -> 29.8 / 27.1 -> 18.9 us.
        if (!(any_dec && pair * ksmax <= 8)) {
            int64_t waves1 = 0;   // waves at one phase per wave
            for (int s = 0; s < a.nseg; ++s) waves1 += (w[s]->m + 15) / 16 * ks[s] * pair;
            for (int p = np_max; p >= 2; p /= 2)
                if (ksmin >= p && waves1 / p >= 4096) {
                    np = p;
                    break;
                }
        }
        // 16 phases from 3 tokens on: each decode-path wave would stage its x in two
        // rounds, the first waited for before any weight load; two phases per wave in
        // 8-wave workgroups instead (2560x9728 at 3 / 4 / 6 / 7 tokens, Q6_K 12.0 -> 11.6 /
        // 12.3 -> 11.9 / 12.7 -> 12.2 / 12.9 -> 12.5 us, Q5_K at 4 / 6 tokens 12.1 -> 12.0 /
        // 12.7 -> 12.4; at 2 tokens the decode path stays: 9.0 against 11.4).
        if (ksmax >= 16 && n >= 3 && !sw && one_type && ksmin >= 2 && np < 2) np = 2;
        np = std::max(np, np_min);
        if (np > 1) any_dec = false;
        // The general path takes at least eight waves per workgroup and doubles them
        // while that brings the grid to about one workgroup per CU, which then may take
        // all of the CU's LDS for fewer, larger x chunks.
        wv = std::max(sw ? 8 : 4, pair * ksmax / np);
        if (!any_dec) {
            const int wv_max = 16;
            wv = std::max(wv, 8);
            for (int cand = wv; cand <= wv_max; cand *= 2)
                if (grid_for(cand, np) <= kOneRound) {
                    wv = cand;
                    break;
                }
        }
    } else {
        // From 8 tokens on x staging sets the pace: the largest grid of at most one
        // workgroup per CU, preferring (on equal grids) two phases per wave, then
        // 16-wave workgroups (10-wave ones where they give a larger grid).  Without such a grid (large matrices), the most phases
        // per wave and 8-wave workgroups.  Measured at 8 / 16 / 32 tokens (cold rotations, us):
        // the gate/up pair 15.4 -> 13.4 / 15.9 -> 14.4 / 21.0 -> 19.3 (two phases,
        // 16 waves, 152 workgroups) against the next best choices; Wo 2560x4096 keeps
        // 160 workgroups of 8 waves with one phase (11.9; 14.3 with two).
        // Ten-wave workgroups (five tiles of two phases, plain launches) fill more CUs
        // where the tiles do not divide evenly into 8 or 16 per workgroup.
        // With 16 phases and two token groups, one phase per wave in 16-wave workgroups
        // comes before two in 8-wave ones (equal grids): 2560x9728 at 17 / 24 / 32 tokens,
        // Q5_K 17.6 -> 17.0 / 21.0 -> 20.0 / 22.8 -> 21.7 us, Q6_K 16.3 -> 16.0 / 19.4 ->
        // 18.5 / 21.5 -> 20.3 (at 16 tokens and with 4 phases the other way round).
        static const int kPrefA[8][2] = {{16, 2}, {10, 2}, {8, 2}, {16, 4}, {8, 4}, {16, 1}, {8, 1}, {4, 1}};
        static const int kPrefB[8][2] = {{16, 2}, {10, 2}, {16, 1}, {8, 2}, {16, 4}, {8, 4}, {8, 1}, {4, 1}};
        const int(&kPref)[8][2] = (ng == 2 && ksmax >= 16) ? kPrefB : kPrefA;
        bool dec4 = true;   // every matrix takes the decode path in 4-wave workgroups
        for (int s = 0; s < a.nseg; ++s) dec4 = dec4 && dec_ok(s, 4);
        int best = 0;
        for (const auto &c : kPref) {
            const int cw = c[0], p = c[1];
            if (p > np_max || p < np_min || ksmin < p || pair * ksmax / p > cw || (sw && cw < 8) || (cw == 4 && !dec4))
                continue;
            if (cw == 16 && p == 4 && ng == 2 && has_q6) continue;   // not instantiated (registers)
            if (cw == 10) {   // every matrix's waves per tile must divide the workgroup; plain only
                bool fits = !sw;
                for (int s = 0; s < a.nseg; ++s) fits = fits && cw % (ks[s] / p) == 0;
                if (!fits) continue;
            }
            const int gr = grid_for(cw, p);
            if (gr <= kCUs && gr > best) {
                best = gr;
                wv = cw;
                np = p;
            }
        }
        // One phase per wave is all the grid search found: small matrices whose waves
        // all fit the decode path stay there (the QKV triple at 8 tokens 8.0 us, 9.6 in
        // 8-wave workgroups on the general path).
        if (best > 0 && np == 1 && dec4 && pair * ksmax <= 4) wv = 4;
        if (best == 0) {
            np = 1;
            for (int p = np_max; p >= 2; p /= 2)
                if (ksmin >= p) {
                    np = p;
                    break;
                }
            np = std::max(np, np_min);
            wv = std::max(8, pair * ksmax / np);
        }
    }
    a.np = np;
    int kw[3] = {1, 1, 1};   // waves per row tile
    int kwmax = 1;
    for (int s = 0; s < a.nseg; ++s) {
        kw[s] = ks[s] / np;
        kwmax = std::max(kwmax, kw[s]);
    }
    a.wv = wv;
    int grid = 0;
    for (int s = 0; s < a.nseg; ++s) {
        qg::MSeg &g = a.seg[s];
        g.data = (const uint8_t *)w[s]->data;
        g.scales = (const uint8_t *)w[s]->scales;
        g.y = y[s];
        g.resid = s == 0 ? resid : nullptr;
        g.row_bytes = qg_row_bytes(w[s]->type, k);
        g.type = w[s]->type;
        g.m = (int32_t)w[s]->m;
        g.ks = ks[s];
        g.tiled = w[s]->layout == QG_LAYOUT_TILES;
        g.wg_begin = grid;
        if (sw) {
            g.data2 = (const uint8_t *)w[1]->data;
            g.scales2 = (const uint8_t *)w[1]->scales;
        }
        const int64_t rows_per_wg = 16 * (wv / kw[s]) / pair;
        grid += (int)((w[s]->m + rows_per_wg - 1) / rows_per_wg);
    }
    const size_t budget = grid <= kOneRound ? kMmaLdsMax : kMmaLdsBudget;
    // SwiGLU: the hand-over region (a slot per tile-group pair) comes out of the budget.
    const size_t xch_bytes = sw ? (size_t)(wv / kwmax / 2) * ng * 1024 : 0;
    const int kc = (int)std::max<size_t>(1, (budget - kMmaZeroBytes - xch_bytes) / per_sb);
    a.kc = std::min(kc, a.nb);
    size_t lds = kMmaZeroBytes;
    for (int s = 0; s < a.nseg; ++s) {
        if (np == 1 && dec_ok(s, wv)) {
            a.seg[s].dec = 1;
            lds = std::max(lds, kMmaZeroBytes + (size_t)wv * ((a.nb + ks[s] - 1) / ks[s]) * per_sb);
        } else {   // the general path's x chunk
            lds = std::max(lds, kMmaZeroBytes + per_sb * a.kc);
        }
    }
    // Partial sums of the K phases: a slot per phase and tile group, where a tile has
    // more than one wave.
    if (kwmax > 1) lds = std::max(lds, (size_t)wv * np * 1024 * ng);
    if (sw) {   // where the gate groups hand over their sums: after everything else
        lds = (lds + 15) / 16 * 16;
        a.xch = (int32_t)(lds / 16);
        lds += xch_bytes;
    }
    int ts = 0;
    for (int s = 0; s < nseg; ++s) ts |= qg::type_bit(w[s]->type);
    hipError_t e = qg::launch_mma(a, ts, grid, lds, (hipStream_t)stream);
    if (e != hipSuccess) return fail(QG_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
    g_err.clear();
    return QG_OK;
}

int gemv_single(int32_t type, const void *wdata, const void *scales, const void *x, float *y, int64_t m,
                int64_t k, void *stream) {
    qg_weight w = {type, 0, wdata, scales, m, k};
    int rc;
    if ((rc = check_weight(&w, "w")) || (rc = check_x(x)) || (rc = check_y(y, "y"))) return rc;
    const qg_weight *ws[1] = {&w};
    float *ys[1] = {y};
    return run_mma(ws, ys, nullptr, 1, x, 1, qg::MODE_PLAIN, stream);
}

}  // namespace

extern "C" {

int64_t qg_row_bytes(int32_t type, int64_t k) {
    if (k < 256 || k % 256) return -1;
    switch (type) {
    case QG_Q4_K: return k / 256 * 144;
    case QG_Q5_K: return k / 256 * 176;
    case QG_Q6_K: return k / 256 * 210;
    case QG_NVFP4: return k / 2;
    case QG_FP8: return k;
    default: return -1;
    }
}

const char *qg_status_str(int status) {
    switch (status) {
    case QG_OK: return "ok";
    case QG_ERR_NULL: return "null pointer";
    case QG_ERR_SHAPE: return "bad shape";
    case QG_ERR_ROWS: return "row count out of range";
    case QG_ERR_TYPE: return "bad tensor type";
    case QG_ERR_ALIGN: return "misaligned pointer";
    case QG_ERR_LAUNCH: return "launch failed";
    default: return "unknown status";
    }
}

const char *qg_last_error(void) { return g_err.c_str(); }

int qgemv_q4k(const void *w, const void *x, float *y, int64_t m, int64_t k, void *stream) {
    return gemv_single(QG_Q4_K, w, nullptr, x, y, m, k, stream);
}
int qgemv_q5k(const void *w, const void *x, float *y, int64_t m, int64_t k, void *stream) {
    return gemv_single(QG_Q5_K, w, nullptr, x, y, m, k, stream);
}
int qgemv_q6k(const void *w, const void *x, float *y, int64_t m, int64_t k, void *stream) {
    return gemv_single(QG_Q6_K, w, nullptr, x, y, m, k, stream);
}
int qgemv_nvfp4(const void *codes, const void *scales, const void *x, float *y, int64_t m, int64_t k,
                void *stream) {
    return gemv_single(QG_NVFP4, codes, scales, x, y, m, k, stream);
}
int qgemv_fp8(const void *codes, const void *scales, const void *x, float *y, int64_t m, int64_t k,
              void *stream) {
    return gemv_single(QG_FP8, codes, scales, x, y, m, k, stream);
}

int qgemm_rows(const qg_weight *w, const void *x, float *y, int32_t n, void *stream) {
    int rc;
    if ((rc = check_weight(w, "w")) || (rc = check_x(x)) || (rc = check_y(y, "y")) || (rc = check_rows(n)))
        return rc;
    float *ys[1] = {y};
    return run_mma(&w, ys, nullptr, 1, x, n, qg::MODE_PLAIN, stream);
}

int qgemv_add(const qg_weight *w, const void *x, const float *resid, float *y, int32_t n, void *stream) {
    int rc;
    if ((rc = check_weight(w, "w")) || (rc = check_x(x)) || (rc = check_y(y, "y")) ||
        (rc = check_y(resid, "resid")) || (rc = check_rows(n)))
        return rc;
    float *ys[1] = {y};
    return run_mma(&w, ys, resid, 1, x, n, qg::MODE_PLAIN, stream);
}

int qgemv_pair(const qg_weight *w0, const qg_weight *w1, const void *x, float *y0, float *y1, int32_t n,
               void *stream) {
    int rc;
    if ((rc = check_weight(w0, "w0")) || (rc = check_weight(w1, "w1")) || (rc = check_x(x)) ||
        (rc = check_y(y0, "y0")) || (rc = check_y(y1, "y1")) || (rc = check_rows(n)))
        return rc;
    if (w0->k != w1->k) return fail(QG_ERR_SHAPE, "pair: k differs (%lld vs %lld)", (long long)w0->k, (long long)w1->k);
    const qg_weight *ws[2] = {w0, w1};
    float *ys[2] = {y0, y1};
    return run_mma(ws, ys, nullptr, 2, x, n, qg::MODE_PLAIN, stream);
}

int qgemv_triple(const qg_weight *w0, const qg_weight *w1, const qg_weight *w2, const void *x, float *y0,
                 float *y1, float *y2, int32_t n, void *stream) {
    int rc;
    if ((rc = check_weight(w0, "w0")) || (rc = check_weight(w1, "w1")) || (rc = check_weight(w2, "w2")) ||
        (rc = check_x(x)) || (rc = check_y(y0, "y0")) || (rc = check_y(y1, "y1")) || (rc = check_y(y2, "y2")) ||
        (rc = check_rows(n)))
        return rc;
    if (w0->k != w1->k || w0->k != w2->k) return fail(QG_ERR_SHAPE, "triple: k differs between the weights");
    const qg_weight *ws[3] = {w0, w1, w2};
    float *ys[3] = {y0, y1, y2};
    return run_mma(ws, ys, nullptr, 3, x, n, qg::MODE_PLAIN, stream);
}

int qgemv_pair_swiglu(const qg_weight *wg, const qg_weight *wu, const void *x, float *h, int32_t n,
                      void *stream) {
    int rc;
    if ((rc = check_weight(wg, "wg")) || (rc = check_weight(wu, "wu")) || (rc = check_x(x)) ||
        (rc = check_y(h, "h")) || (rc = check_rows(n)))
        return rc;
    if (wg->k != wu->k || wg->m != wu->m)
        return fail(QG_ERR_SHAPE, "swiglu pair: gate and up must have the same m and k");
    if (wg->type != wu->type || wg->layout != wu->layout)
        return fail(QG_ERR_TYPE, "swiglu pair: gate and up must have the same type and layout");
    const qg_weight *ws[2] = {wg, wu};
    float *ys[2] = {h, h};
    return run_mma(ws, ys, nullptr, 2, x, n, qg::MODE_SWIGLU, stream);
}

int64_t qg_tiles_bytes(const qg_weight *w) {
    int rc;
    if ((rc = check_weight(w, "w"))) return rc;
    if (has_scales(w->type)) return fail(QG_ERR_TYPE, "w: the tiled layout is for the K-quants only");
    return (w->m + 15) / 16 * 16 * qg_row_bytes(w->type, w->k);
}

int qg_pack_tiles(const qg_weight *w, void *dst, void *stream) {
    int rc;
    if ((rc = check_weight(w, "w"))) return rc;
    if (w->layout != QG_LAYOUT_ROWS) return fail(QG_ERR_TYPE, "w: the source must be in the row layout");
    if (has_scales(w->type)) return fail(QG_ERR_TYPE, "w: the tiled layout is for the K-quants only");
    if (!dst) return fail(QG_ERR_NULL, "dst is NULL");
    if (!aligned(dst, 16)) return fail(QG_ERR_ALIGN, "dst is not 16-byte aligned");
    const int64_t row_bytes = qg_row_bytes(w->type, w->k);
    const int sbytes = (int)(row_bytes / (w->k / 256));
    hipError_t e = qg::launch_pack_tiles((const uint8_t *)w->data, (uint8_t *)dst, w->m, row_bytes, sbytes,
                                         (hipStream_t)stream);
    if (e != hipSuccess) return fail(QG_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
    g_err.clear();
    return QG_OK;
}

int qgemm_prefill(const qg_weight *w, const void *x, float *y, int64_t n, void *stream) {
    int rc;
    if ((rc = check_weight(w, "w")) || (rc = check_x(x)) || (rc = check_y(y, "y"))) return rc;
    if (n < 1 || n > ((int64_t)1 << 30)) return fail(QG_ERR_SHAPE, "n = %lld out of range", (long long)n);
    qg::PrefillArgs a;
    memset(&a, 0, sizeof a);
    a.data = (const uint8_t *)w->data;
    a.scales = (const uint8_t *)w->scales;
    a.x = x;
    a.y = y;
    a.row_bytes = qg_row_bytes(w->type, w->k);
    a.m = w->m;
    a.n = n;
    a.k = (int32_t)w->k;
    a.type = w->type;
    a.tiled = w->layout == QG_LAYOUT_TILES;
    const int64_t blocks = (w->m + qg::kPrefillBlockN - 1) / qg::kPrefillBlockN *
                           ((n + qg::kPrefillBlockM - 1) / qg::kPrefillBlockM);
    if (blocks > 0x7fffffff)
        return fail(QG_ERR_SHAPE, "m = %lld, n = %lld: more than 2^31 - 1 blocks", (long long)w->m, (long long)n);
    hipError_t e = qg::launch_prefill(a, (hipStream_t)stream);
    if (e != hipSuccess) return fail(QG_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
    g_err.clear();
    return QG_OK;
}

int qdequant(const qg_weight *w, float *out, void *stream) {
    int rc;
    if ((rc = check_weight(w, "w")) || (rc = check_y(out, "out"))) return rc;
    qg::DequantArgs a;
    memset(&a, 0, sizeof a);
    a.data = (const uint8_t *)w->data;
    a.scales = (const uint8_t *)w->scales;
    a.out = out;
    a.row_bytes = qg_row_bytes(w->type, w->k);
    a.m = w->m;
    a.k = (int32_t)w->k;
    a.nb = (int32_t)(w->k / 256);
    a.type = w->type;
    a.tiled = w->layout == QG_LAYOUT_TILES;
    hipError_t e = qg::launch_dequant(a, (hipStream_t)stream);
    if (e != hipSuccess) return fail(QG_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
    g_err.clear();
    return QG_OK;
}

int qg_stream_read(const void *const *ptrs, const int64_t *bytes, int32_t nreg, uint32_t *out, void *stream) {
    if (!ptrs || !bytes || !out) return fail(QG_ERR_NULL, "null argument");
    if (nreg < 1 || nreg > qg::kReadMaxRegions) return fail(QG_ERR_SHAPE, "nreg = %d, need 1..%d", nreg, qg::kReadMaxRegions);
    qg::ReadArgs a;
    memset(&a, 0, sizeof a);
    for (int r = 0; r < nreg; ++r) {
        if (!ptrs[r]) return fail(QG_ERR_NULL, "region %d is null", r);
        if (bytes[r] <= 0 || bytes[r] % 16) return fail(QG_ERR_SHAPE, "region %d: %lld bytes, need a positive multiple of 16", r, (long long)bytes[r]);
        if ((uintptr_t)ptrs[r] % 16) return fail(QG_ERR_ALIGN, "region %d is not 16-byte aligned", r);
        a.p[r] = (const uint4 *)ptrs[r];
        a.n16[r] = bytes[r] / 16;
    }
    if ((uintptr_t)out % 128) return fail(QG_ERR_ALIGN, "out is not 128-byte aligned");
    a.out = out;
    a.nreg = nreg;
    hipError_t e = qg::launch_stream_read(a, (hipStream_t)stream);
    if (e != hipSuccess) return fail(QG_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
    g_err.clear();
    return QG_OK;
}

}  // extern "C"
