// Host-only tactic logic: legality, the tuner's candidate list, the per-M
// table rule, status texts and the thread-local error text.  Nothing here
// calls the HIP runtime, so all of it runs (and is tested) without a GPU.
#include <stdarg.h>

#include <algorithm>
#include <stdio.h>
#include <string.h>

#include "skinny_internal.h"

namespace skinny {

static thread_local char g_error[512];

void set_error(const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_error, sizeof g_error, fmt, ap);
    va_end(ap);
}

size_t tactic_lds_bytes(const skinny_tactic &t, int K8)
{
    (void)K8;
    switch (t.path) {
    case SKINNY_PATH_MFMA:
        return (size_t)t.waves * t.mt * (t.rows + 1) * sizeof(float);
    case SKINNY_PATH_MFMAT:                    // one group's tile of the MFMA kernel
        return (size_t)t.waves * kTokenGroup * (t.rows + 1) * sizeof(float);
    case SKINNY_PATH_MFMAX:
        return mfmax_own_lds_bytes(t.waves, t.mt);
    case SKINNY_PATH_MFMAW:
        return mfmaw_lds_bytes(t.waves, t.rows, t.mt, t.unroll);
    case SKINNY_PATH_MFMA4:
    case SKINNY_PATH_DOT2W:
        return rgs_lds_bytes(t);
    default:
        return 0;
    }
}

const KernelInfo *tactic_kernel(const skinny_tactic &t, int half)
{
    switch (t.path) {
    case SKINNY_PATH_DOT2:
    case SKINNY_PATH_MFMA:
        return find_kernel(t.path, t.mt, t.rows, t.unroll, half);
    case SKINNY_PATH_DOT2R:                    // the DOT2 kernels, another grid
        return find_kernel(SKINNY_PATH_DOT2, t.mt, t.rows, t.unroll, half);
    case SKINNY_PATH_MFMAT:                    // the 16-token MFMA kernels over token groups
        if (t.mt != 2 * kTokenGroup && t.mt != 4 * kTokenGroup)
            return nullptr;
        return find_kernel(SKINNY_PATH_MFMA, kTokenGroup, t.rows, t.unroll, half);
    case SKINNY_PATH_MFMAX:
        if (t.rows != 16 * t.waves || (t.unroll != 1 && t.unroll != 2))
            return nullptr;
        return find_kernel(t.path, t.mt, t.waves, 1, half);   // unroll 2: same kernel, equal row ranges
    case SKINNY_PATH_MFMAW:                    // KernelInfo.rows = 100 waves + row groups
        if (t.rows < 16 || t.rows % 16)
            return nullptr;
        return find_kernel(t.path, t.mt, 100 * t.waves + t.rows / 16, t.unroll, half);
    case SKINNY_PATH_MFMA4:                    // KernelInfo.rows = the most rows of a range
    case SKINNY_PATH_DOT2W:
        return find_kernel(t.path, t.mt, t.rows, t.unroll, half);
    default:
        return nullptr;
    }
}

static bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

}  // namespace skinny

using namespace skinny;

extern "C" {

const char *skinny_status_string(skinny_status s)
{
    switch (s) {
    case SKINNY_OK: return "ok";
    case SKINNY_ERR_INVALID_ARG: return "invalid argument";
    case SKINNY_ERR_SHAPE: return "unsupported shape";
    case SKINNY_ERR_ALIGN: return "misaligned pointer";
    case SKINNY_ERR_UNSUPPORTED_M: return "token count outside 1..64";
    case SKINNY_ERR_DEVICE: return "no gfx950 device";
    case SKINNY_ERR_NOMEM: return "out of memory";
    case SKINNY_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *skinny_last_error(void) { return g_error; }

skinny_status skinny_tactic_check(const skinny_tactic *t, int N, int K)
{
    if (!t) {
        set_error("tactic is NULL");
        return SKINNY_ERR_INVALID_ARG;
    }
    if (N < 1 || K < 8 || K % 8) {
        set_error("bad shape N=%d K=%d (need N >= 1, K >= 8, K %% 8 == 0)", N, K);
        return SKINNY_ERR_INVALID_ARG;
    }
    const int k8 = K / 8;
    if (!is_pow2(t->waves) || t->waves > kMaxWaves) {
        set_error("waves=%d: must be 1, 2, 4 or 8", t->waves);
        return SKINNY_ERR_INVALID_ARG;
    }
    if (t->split < 1 || t->split > 16) {
        set_error("split=%d: must be 1..16", t->split);
        return SKINNY_ERR_INVALID_ARG;
    }
    if (is_retired_path(t->path)) {
        set_error("path=%d: this kernel family was measured and removed; its number stays reserved", t->path);
        return SKINNY_ERR_INVALID_ARG;
    }
    if (t->path == SKINNY_PATH_DOT2 || t->path == SKINNY_PATH_MFMAX || t->path == SKINNY_PATH_DOT2R) {
        if (t->split > k8) {
            set_error("split=%d exceeds the %d 16-byte chunks of a row", t->split, k8);
            return SKINNY_ERR_INVALID_ARG;
        }
    } else if (t->path == SKINNY_PATH_MFMAW) {
        if (t->unroll < 1 || t->unroll > 4) {
            set_error("unroll=%d: for MFMAW 1 or 2 (stages of 8 or 16 chunks, two in flight) or 3 or 4 (the "
                      "same, one in flight)", t->unroll);
            return SKINNY_ERR_INVALID_ARG;
        }
        const int sc = mfmaw_stage_chunks(t->unroll), stages = (k8 + sc - 1) / sc;
        if (t->split > stages) {
            set_error("split=%d exceeds the %d K stages of %d chunks", t->split, stages, sc);
            return SKINNY_ERR_INVALID_ARG;
        }
    } else if (is_rgs_path(t->path)) {
        if (t->unroll != 2 && t->unroll != 3) {
            set_error("unroll=%d: stages of %d chunks in flight, 2 or 3", t->unroll, kRgsChunks);
            return SKINNY_ERR_INVALID_ARG;
        }
        if (t->waves > 4) {
            set_error("waves=%d: MFMA4 and DOT2W workgroups hold at most 4 waves", t->waves);
            return SKINNY_ERR_INVALID_ARG;
        }
        const int stages = (k8 + kRgsChunks - 1) / kRgsChunks;
        if (t->split > 8 || t->split > stages) {
            set_error("split=%d: MFMA4 and DOT2W split K into at most 8 parts and at most their %d stages of %d "
                      "chunks", t->split, stages, kRgsChunks);
            return SKINNY_ERR_INVALID_ARG;
        }
    } else if (t->path == SKINNY_PATH_MFMA || t->path == SKINNY_PATH_MFMAT) {
        if (t->path == SKINNY_PATH_MFMAT && t->mt != 2 * kTokenGroup && t->mt != 4 * kTokenGroup) {
            set_error("mt=%d: MFMAT serves at most 32 or 64 tokens, in groups of %d", t->mt, kTokenGroup);
            return SKINNY_ERR_INVALID_ARG;
        }
        const int steps = (k8 + 3) / 4;
        if (t->split > steps) {
            set_error("split=%d exceeds the %d 32-element K steps of a row", t->split, steps);
            return SKINNY_ERR_INVALID_ARG;
        }
    } else {
        set_error("path=%d: must be 0 (DOT2), 1 (MFMA), 3 (MFMAX), 8 (DOT2R), 9 (MFMAW), 10 (MFMA4), 11 (DOT2W) "
                  "or 12 (MFMAT)", t->path);
        return SKINNY_ERR_INVALID_ARG;
    }
    // the instance first: its fields are then small, so the LDS sizes below
    // cannot overflow
    if (!tactic_kernel(*t)) {
        set_error("no compiled kernel for path=%d mt=%d rows=%d unroll=%d", t->path, t->mt, t->rows,
                  t->unroll);
        return SKINNY_ERR_INVALID_ARG;
    }
    const size_t lds_limit = (t->path == SKINNY_PATH_MFMA || t->path == SKINNY_PATH_MFMAT) ? kMaxLds : kMaxLdsStaged;
    if (tactic_lds_bytes(*t, k8) > lds_limit) {
        set_error("tactic needs %zu bytes of LDS (limit %zu)", tactic_lds_bytes(*t, k8), lds_limit);
        return SKINNY_ERR_INVALID_ARG;
    }
    return SKINNY_OK;
}

int skinny_enumerate_tactics(int N, int K, skinny_tactic *buf, int cap)
{
    return skinny_enumerate_tactics_ex(N, K, 256, buf, cap);
}

int skinny_enumerate_tactics_ex(int N, int K, int cus, skinny_tactic *buf, int cap)
{
    if (N < 1 || K < 8 || K % 8 || cus < 1 || cap < 0 || (cap > 0 && !buf))
        return -1;
    const int k8 = K / 8;
    int count = 0;
    int nk = 0;
    const KernelInfo *ks = kernel_table(&nk);
    static const int kWaves[] = {1, 2, 4, 8};
    static const int kSplits[] = {1, 2, 3, 4, 5, 6, 8};
    // a weight small enough for token groups (MFMAT) to re-read from L2
    const bool small_weight = (long long)N * K * 2 <= kTokenGroupMaxWeightBytes;
    for (int i = 0; i < nk; ++i) {
        const KernelInfo &k = ks[i];
        if (k.half)
            continue;                                    // the same tactics as the BF16 twin
        // the DOT2 kernels also run over equal row ranges (DOT2R); the 16-token
        // MFMA kernels also over 2 or 4 token groups (MFMAT)
        struct { int path, mt; } uses[3] = {{k.path, k.mt}, {-1, 0}, {-1, 0}};
        if (k.path == SKINNY_PATH_DOT2)
            uses[1] = {SKINNY_PATH_DOT2R, k.mt};
        if (k.path == SKINNY_PATH_MFMA && k.mt == kTokenGroup && small_weight) {
            uses[1] = {SKINNY_PATH_MFMAT, 2 * kTokenGroup};
            uses[2] = {SKINNY_PATH_MFMAT, 4 * kTokenGroup};
        }
        for (const auto &use : uses) {
            const int path = use.path;
            if (path < 0)
                continue;
            for (int w : kWaves) {
                for (int s : kSplits) {
                    skinny_tactic t = {path, use.mt, k.rows, w, k.unroll, s};
                    if (path == SKINNY_PATH_MFMAX) {
                        if (w != k.rows)                 // k.rows is the wave count
                            continue;
                        t.rows = 16 * w;
                    }
                    if (path == SKINNY_PATH_MFMAW) {     // k.rows = 100 waves + row groups
                        if (w != k.rows / 100 || s > 4)
                            continue;
                        t.rows = 16 * (k.rows % 100);
                    }
                    if (is_rgs_path(path)) {
                        // the instance whose row groups the equal ranges fill: a range of
                        // ceil(N / ranges) rows leaves none of its 4-row groups empty
                        if (w > 4 || s > 4)
                            continue;
                        const long long per_round = ((long long)cus + s - 1) / s;
                        const long long ranges0 = ((long long)N + k.rows - 1) / k.rows;
                        const long long ranges = ((ranges0 + per_round - 1) / per_round) * per_round;
                        const long long most = ((long long)N + ranges - 1) / std::min<long long>(N, ranges);
                        if (most <= k.rows - 4)
                            continue;
                    }
                    if (skinny_tactic_check(&t, N, K) != SKINNY_OK)
                        continue;
                    const long long tiles = ((long long)N + t.rows - 1) / t.rows, chip = 8LL * cus;
                    if (s > 1 && tiles * token_groups(t) * w >= chip && path != SKINNY_PATH_MFMAW &&
                        !is_rgs_path(path))
                        continue;   // enough waves already; a K split only adds traffic
                    if (path == SKINNY_PATH_DOT2R && tiles * s > chip)
                        continue;   // many workgroups per CU balance themselves
                    if (path == SKINNY_PATH_DOT2) {
                        // each lane of the workgroup should own at least one chunk per
                        // split, and the unrolled loop should run at least once
                        const int per_split = k8 / s;
                        if (per_split < 64 * w * k.unroll && !(w == 1 && s == 1 && k.unroll == 1))
                            continue;
                    } else if (path == SKINNY_PATH_MFMAW) {
                        // every wave should own two stages of its K part at least
                        if (k8 / s < 2 * w * mfmaw_stage_chunks(k.unroll))
                            continue;
                    } else if (is_rgs_path(path)) {
                        // every wave should own a stage of its K part at least
                        if (k8 / s < w * kRgsChunks && !(w == 1 && s == 1))
                            continue;
                    } else if (path == SKINNY_PATH_MFMAX) {
                        if (k8 / s < 2 * kMfmaxChunks)
                            continue;
                    } else if (path == SKINNY_PATH_MFMA || path == SKINNY_PATH_MFMAT) {
                        const int per_split = ((k8 + 3) / 4) / s;
                        if (per_split < w * k.unroll && !(w == 1 && s == 1 && k.unroll == 1))
                            continue;
                    }
                    if (count < cap)
                        buf[count] = t;
                    ++count;
                    if (path == SKINNY_PATH_MFMAX) {     // the same kernel over equal row ranges
                        t.unroll = 2;
                        if (count < cap)
                            buf[count] = t;
                        ++count;
                    }
                }
            }
        }
    }
    return count;
}

skinny_status skinny_select_table(const skinny_tactic *cand, const double *times_us, int count,
                                  skinny_tactic *table)
{
    if (!cand || !times_us || !table || count < 0) {
        set_error("skinny_select_table: NULL argument or negative count");
        return SKINNY_ERR_INVALID_ARG;
    }
    for (int m = 1; m <= SKINNY_MAX_M; ++m) {
        int best = -1;
        for (int i = 0; i < count; ++i) {
            if (times_us[i] < 0 || cand[i].mt < m)
                continue;
            if (best < 0 || times_us[i] < times_us[best] ||
                (times_us[i] == times_us[best] && cand[i].mt < cand[best].mt))
                best = i;
        }
        if (best < 0) {
            set_error("no usable candidate serves M=%d", m);
            return SKINNY_ERR_INVALID_ARG;
        }
        table[m - 1] = cand[best];
    }
    return SKINNY_OK;
}

}  // extern "C"
