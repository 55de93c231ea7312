// Plans: prepare (validate, tune or take a table, warm, allocate the split-K
// workspace) and run (one table lookup, one launch).
//
// This follows the pages' split between install time and forward time: the
// static part of the choice is resolved once into an {M: call} plan so that a
// forward is a single lookup ("vllm.models.kimi_k3.nvidia.low_latency_gemm",
// module docstring), every kernel a plan can use is compiled and warmed before
// graph capture (the warmups registered by enable_kimi_k3_low_latency_gemm
// and Projection.__init__ "compiled before capture"), and the per-part
// measured tables of that page become a table measured on this chip.  Tuned
// tables are shared process-wide per (device, N, K, output type), as the
// split-K projection page's compile cache is shared per shape while weights
// stay private to each prepared object.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <atomic>
#include <map>
#include <mutex>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <tuple>
#include <vector>

#include "skinny_internal.h"

using namespace skinny;

namespace {

struct Entry {
    const void *fn = nullptr;
    unsigned grid = 0, block = 0, lds = 0;
    int n_tiles = 0;
    FastDiv fd_tiles{}, fd_split{};  // see KArgs
    unsigned rows_q = 0, rows_r = 0;
    skinny_tactic t{};
};

}  // namespace

struct skinny_plan {
    int device = -1;
    const void *W = nullptr;
    int N = 0, K = 0;
    int ldw = 0;                     // W row pitch, elements
    int half = 0;                    // 1: FP16 inputs
    skinny_out_dtype od = SKINNY_OUT_BF16;
    float *ws = nullptr;             // split-K exchange nodes (all zero, i.e. empty, between launches)
    KArgs base{};
    Entry e[SKINNY_MAX_M + 1];       // runs without a residual
    Entry er[SKINNY_MAX_M + 1];      // runs with a residual
};

namespace {

using Key = std::tuple<int, int, int, int, int>;   // device, N, K, in dtype, out dtype
using Table = std::array<skinny_tactic, SKINNY_MAX_M>;
struct Tables {
    Table plain;      // runs without a residual
    Table residual;   // runs with a residual
};
std::mutex g_cache_mu;
std::map<Key, Tables> g_cache;

bool env_flag(const char *name)
{
    const char *v = getenv(name);
    return v && *v && strcmp(v, "0") != 0;
}

int env_int(const char *name, int dflt)
{
    const char *v = getenv(name);
    return (v && *v) ? atoi(v) : dflt;
}

double env_double(const char *name, double dflt)
{
    const char *v = getenv(name);
    return (v && *v) ? strtod(v, nullptr) : dflt;
}

skinny_status hip_fail(hipError_t e, const char *what)
{
    set_error("%s: %s", what, hipGetErrorString(e));
    return SKINNY_ERR_HIP;
}

#define HIP_TRY(expr)                                   \
    do {                                                \
        hipError_t e_ = (expr);                         \
        if (e_ != hipSuccess)                           \
            return hip_fail(e_, #expr);                 \
    } while (0)

int device_cus()
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        cus = 1;
    return cus;
}

Entry make_entry(const skinny_tactic &t, int N, int K, int half)
{
    Entry en;
    const KernelInfo *k = tactic_kernel(t, half);
    en.fn = k ? k->fn : nullptr;
    en.n_tiles = tiles_for(t, N);
    if ((t.path == SKINNY_PATH_MFMAX && t.unroll == 2) || t.path == SKINNY_PATH_DOT2R ||
        t.path == SKINNY_PATH_MFMAW || is_rgs_path(t.path)) {
        // equal row ranges, a whole multiple of CUs / split of them, so that
        // every CU gets the same number of (range, K part) workgroups
        const int per_round = (device_cus() + t.split - 1) / t.split;
        const int rounds = (en.n_tiles + per_round - 1) / per_round;
        en.n_tiles = std::min(N, rounds * per_round);
    }
    en.grid = (unsigned)(en.n_tiles * t.split);
    en.block = (unsigned)(64 * t.waves);
    en.lds = (unsigned)tactic_lds_bytes(t, K / 8);
    en.t = t;
    en.fd_tiles = make_fastdiv((uint32_t)en.n_tiles);
    en.fd_split = make_fastdiv((uint32_t)t.split);
    en.rows_q = (unsigned)(N / en.n_tiles);
    en.rows_r = (unsigned)(N % en.n_tiles);
    return en;
}

// Let the LDS-staged kernels use more than the default 64 KiB of dynamic LDS
// (gfx950 has 160 KiB per CU).  Once per process; failures only make the
// largest tactics fail to launch, which the tuner skips.
void raise_lds_limits()
{
    static std::once_flag once;
    std::call_once(once, [] {
        int dev = 0, max_lds = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
            return;
        int nk = 0;
        const KernelInfo *ks = kernel_table(&nk);
        for (int i = 0; i < nk; ++i)
            if (ks[i].path == SKINNY_PATH_MFMAX || ks[i].path == SKINNY_PATH_MFMAW || is_rgs_path(ks[i].path))
                (void)hipFuncSetAttribute(ks[i].fn, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
        (void)hipGetLastError();
    });
}

// Floats of split-K exchange nodes a table entry needs: split - 1 nodes of
// one tile's values per row tile and token group (see swap_exchange in the
// kernels).
size_t ws_floats(const Entry &en)
{
    return en.t.split > 1 ? (size_t)token_groups(en.t) * en.n_tiles * (en.t.split - 1) * tile_values(en.t) : 0;
}

// Static LDS of a kernel plus the device's per-workgroup limit, looked up
// once per kernel.  A dispatch over the limit would abort the queue, so
// launches that would exceed it are refused here instead.
bool lds_fits(const void *fn, unsigned dynamic_bytes)
{
    static std::mutex mu;
    static std::map<const void *, size_t> static_lds;
    static int max_lds = -1;
    std::lock_guard<std::mutex> lock(mu);
    if (max_lds < 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
            max_lds = 64 * 1024;
    }
    auto it = static_lds.find(fn);
    if (it == static_lds.end()) {
        hipFuncAttributes attr{};
        const size_t st = hipFuncGetAttributes(&attr, fn) == hipSuccess ? attr.sharedSizeBytes : kStaticLdsReserve;
        it = static_lds.emplace(fn, st).first;
    }
    return it->second + dynamic_bytes <= (size_t)max_lds;
}

hipError_t launch(const Entry &en, KArgs a, hipStream_t stream)
{
    a.n_tiles = en.n_tiles;
    a.split = en.t.split;
    a.remap = (en.t.split > 1 && a.nxcd > 1) ? 1 : 0;
    a.ranges = (en.t.path == SKINNY_PATH_MFMAX && en.t.unroll == 2) || en.t.path == SKINNY_PATH_DOT2R ||
               en.t.path == SKINNY_PATH_MFMAW || is_rgs_path(en.t.path);
    const int nx = a.nxcd > 1 ? a.nxcd : 1;
    a.fd_tiles = en.fd_tiles;
    a.fd_split = en.fd_split;
    a.fd_nxcd = make_fastdiv((uint32_t)nx);
    a.rows_q = en.rows_q;
    a.rows_r = en.rows_r;
    a.rows_fast = en.n_tiles < (1 << 16);
    a.grid_q = (int)en.grid / nx;
    a.grid_r = (int)en.grid % nx;
    void *params[] = {&a};
    // MFMAT: one grid row per group of 16 of the call's tokens
    const unsigned groups = en.t.path == SKINNY_PATH_MFMAT ? (unsigned)(a.M + kTokenGroup - 1) / kTokenGroup : 1u;
    return hipLaunchKernel(en.fn, dim3(en.grid, groups), dim3(en.block), params, en.lds, stream);
}

// Validation shared by the prepare entry points; no HIP call before it passes.
skinny_status check_prepare_args(const void *W, int N, int K, int ldw, int in_dtype, skinny_out_dtype od,
                                 skinny_plan **plan)
{
    if (!plan) {
        set_error("plan out-pointer is NULL");
        return SKINNY_ERR_INVALID_ARG;
    }
    *plan = nullptr;
    if (!W) {
        set_error("W is NULL");
        return SKINNY_ERR_INVALID_ARG;
    }
    if (N <= 0 || K <= 0) {
        set_error("N=%d K=%d must be positive", N, K);
        return SKINNY_ERR_INVALID_ARG;
    }
    if (od != SKINNY_OUT_BF16 && od != SKINNY_OUT_F32) {
        set_error("out_dtype=%d is not SKINNY_OUT_BF16 or SKINNY_OUT_F32", (int)od);
        return SKINNY_ERR_INVALID_ARG;
    }
    if (in_dtype != SKINNY_IN_BF16 && in_dtype != SKINNY_IN_F16) {
        set_error("in_dtype=%d is not SKINNY_IN_BF16 or SKINNY_IN_F16", in_dtype);
        return SKINNY_ERR_INVALID_ARG;
    }
    if (K % 8) {
        set_error("K=%d is not a multiple of 8 (rows must be whole 16-byte chunks)", K);
        return SKINNY_ERR_SHAPE;
    }
    if (ldw < K || ldw % 8) {
        set_error("ldw=%d must be >= K=%d and a multiple of 8 (a 16-byte row pitch)", ldw, K);
        return SKINNY_ERR_SHAPE;
    }
    // every kernel builds its W buffer resource over at most kMaxTileRows rows
    // and marks a skipped load with the offset kOffOob, which must lie past it
    if ((long long)ldw * 2 * kMaxTileRows >= (long long)kOffOob) {
        set_error("ldw=%d: %d rows of W must span less than %u bytes", ldw, kMaxTileRows, kOffOob);
        return SKINNY_ERR_SHAPE;
    }
    if ((long long)N * K >= (1LL << 31)) {
        set_error("N*K=%lld exceeds 2^31 - 1 elements", (long long)N * K);
        return SKINNY_ERR_SHAPE;
    }
    if ((uintptr_t)W & 15) {
        set_error("W=%p is not 16-byte aligned", W);
        return SKINNY_ERR_ALIGN;
    }
    return SKINNY_OK;
}

// Validation of a run's arguments (x, residual, out, M) for an [N][K]
// weight; no HIP call.
skinny_status check_run_args(int N, int K, skinny_out_dtype od, const void *x, int ldx, const void *residual,
                             int ldr, const void *out, int ldo, int M)
{
    if (M < 1 || M > SKINNY_MAX_M) {
        set_error("M=%d outside 1..%d", M, SKINNY_MAX_M);
        return SKINNY_ERR_UNSUPPORTED_M;
    }
    if (!x || !out) {
        set_error("x or out is NULL");
        return SKINNY_ERR_INVALID_ARG;
    }
    if (ldx < K || ldx % 8 || ldo < N || (residual && ldr < N)) {
        set_error("ldx=%d (>= K=%d, multiple of 8), ldo=%d and ldr=%d (>= N=%d) out of range", ldx, K, ldo,
                  ldr, N);
        return SKINNY_ERR_SHAPE;
    }
    const size_t osz = od == SKINNY_OUT_F32 ? 4 : 2;
    if ((long long)ldx * (SKINNY_MAX_M * 2) >= (long long)kOffOob) {
        set_error("ldx=%d: %d rows of x must span less than %u bytes", ldx, SKINNY_MAX_M, kOffOob);
        return SKINNY_ERR_SHAPE;
    }
    if (((uintptr_t)x & 15) || ((uintptr_t)out & (osz - 1)) || ((uintptr_t)residual & (osz - 1))) {
        set_error("x=%p must be 16-byte aligned, out=%p and residual=%p element aligned", x, out, residual);
        return SKINNY_ERR_ALIGN;
    }
    if (residual && residual != out) {
        // the residual must be out itself or lie apart from it
        const char *o0 = (const char *)out, *o1 = o0 + ((size_t)(M - 1) * ldo + N) * osz;
        const char *r0 = (const char *)residual, *r1 = r0 + ((size_t)(M - 1) * ldr + N) * osz;
        if (r0 < o1 && o0 < r1) {
            set_error("residual=%p overlaps out=%p without being it", residual, out);
            return SKINNY_ERR_INVALID_ARG;
        }
    } else if (residual && ldr != ldo) {
        set_error("residual is out but ldr=%d != ldo=%d", ldr, ldo);
        return SKINNY_ERR_INVALID_ARG;
    }
    return SKINNY_OK;
}

// The weight-side kernel arguments of an [N][K] weight (pitch ldw) whose
// split-K exchange nodes are at ws.
KArgs weight_args(const void *W, int N, int K, int ldw, skinny_out_dtype od, int nxcd, float *ws)
{
    KArgs a{};
    a.W = W;
    a.ws = ws;
    a.N = N;
    a.K8 = K / 8;
    a.out_f32 = od == SKINNY_OUT_F32;
    a.w_pitch = (unsigned)ldw * 2u;
    a.x_pitch = (unsigned)K * 2u;       // per call
    a.ldo = a.ldr = N;                  // per call
    // SKINNY_XCD_REMAP=0 turns off the placement of a tile's split-K
    // workgroups on one XCD (then the partial exchange crosses XCDs).
    a.nxcd = env_int("SKINNY_XCD_REMAP", 1) ? nxcd : 1;
    return a;
}

// The per-call kernel arguments.
void set_call_args(KArgs &a, const void *x, int ldx, const void *residual, int ldr, void *out, int ldo, int M)
{
    a.x = x;
    a.out = out;
    a.res = residual;
    a.M = M;
    a.x_pitch = (unsigned)ldx * 2u;
    a.ldo = ldo;
    a.ldr = residual ? ldr : ldo;
}

skinny_status current_gfx950(int *dev, int *cus)
{
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count == 0) {
        set_error("no HIP device");
        return SKINNY_ERR_DEVICE;
    }
    HIP_TRY(hipGetDevice(dev));
    hipDeviceProp_t prop;
    HIP_TRY(hipGetDeviceProperties(&prop, *dev));
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
        set_error("device %d is %s, not gfx950", *dev, prop.gcnArchName);
        return SKINNY_ERR_DEVICE;
    }
    *cus = prop.multiProcessorCount;
    return SKINNY_OK;
}

struct DevBuf {
    void *p = nullptr;
    ~DevBuf()
    {
        if (p)
            (void)hipFree(p);
    }
};

// Time every candidate on cache-cold copies of W and fill the table.
// Timing harness of the tuner: packed copies of W, rotated per launch so
// that every launch reads its weight from HBM (their total is well past the
// 256 MiB Infinity Cache), x, out and residual buffers of 64 rows, an
// exchange workspace with every node empty, a private stream and two events.
struct Harness {
    DevBuf wcopies, xbuf, obuf, rbuf, wsbuf;
    hipStream_t st = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    size_t wbytes = 0;
    int copies = 1, iters = 8;
    KArgs a{};

    Harness() = default;
    Harness(const Harness &) = delete;
    Harness &operator=(const Harness &) = delete;
    ~Harness()
    {
        if (e0)
            (void)hipEventDestroy(e0);
        if (e1)
            (void)hipEventDestroy(e1);
        if (st)
            (void)hipStreamDestroy(st);
    }

    hipError_t init(const void *W, int N, int K, int ldw, skinny_out_dtype od, int nxcd, size_t max_ws)
    {
        wbytes = (size_t)N * K * 2;
        const size_t cold = (size_t)768 << 20;
        copies = (int)std::min<size_t>(16, std::max<size_t>(1, (cold + wbytes - 1) / wbytes));
        const size_t xb = (size_t)SKINNY_MAX_M * K * 2, ob = (size_t)SKINNY_MAX_M * N * 4;
        const size_t wsb = std::max<size_t>(max_ws, 1) * 4;
        hipError_t e;
        if ((e = hipMalloc(&wcopies.p, wbytes * copies)) != hipSuccess || (e = hipMalloc(&xbuf.p, xb)) != hipSuccess ||
            (e = hipMalloc(&obuf.p, ob)) != hipSuccess || (e = hipMalloc(&rbuf.p, ob)) != hipSuccess ||
            (e = hipMalloc(&wsbuf.p, wsb)) != hipSuccess ||
            (e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking)) != hipSuccess ||
            (e = hipEventCreate(&e0)) != hipSuccess || (e = hipEventCreate(&e1)) != hipSuccess)
            return e;
        // packed copies of W (its pitch does not change the tactic)
        for (int c = 0; c < copies; ++c)
            if ((e = hipMemcpy2DAsync((char *)wcopies.p + wbytes * c, (size_t)K * 2, W, (size_t)ldw * 2,
                                      (size_t)K * 2, N, hipMemcpyDeviceToDevice, st)) != hipSuccess)
                return e;
        if ((e = hipMemsetAsync(xbuf.p, 0, xb, st)) != hipSuccess || (e = hipMemsetAsync(rbuf.p, 0, ob, st)) != hipSuccess ||
            (e = hipMemsetAsync(wsbuf.p, 0, wsb, st)) != hipSuccess)   // every exchange node empty
            return e;
        a.x = xbuf.p;
        a.out = obuf.p;
        a.ws = (float *)wsbuf.p;
        a.N = N;
        a.K8 = K / 8;
        a.out_f32 = od == SKINNY_OUT_F32;
        a.nxcd = nxcd;
        a.w_pitch = a.x_pitch = (unsigned)K * 2u;
        a.ldo = a.ldr = N;
        iters = std::max(1, env_int("SKINNY_TUNE_ITERS", 2 * copies > 8 ? 2 * copies : 8));
        return hipStreamSynchronize(st);
    }

    // Mean time per launch of `iters` launches over the rotated copies at
    // M = a.M, captured in a graph and replayed (the second replay timed, or
    // for a replay shorter than kMinTimedMs enough further replays to fill
    // it), as decode steps run them: launched one by one from the host, a
    // kernel of a few microseconds would be timed at the host's launch rate.
    // -1 if a launch failed.
    hipError_t time_once(const Entry &en, double &us)
    {
        us = -1.0;
        hipGraph_t g = nullptr;
        hipGraphExec_t ge = nullptr;
        hipError_t e = hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal);
        if (e != hipSuccess)
            return e;
        bool ok = true;
        for (int j = 0; j < iters && ok; ++j) {
            a.W = (const char *)wcopies.p + wbytes * ((j + 1) % copies);
            ok = launch(en, a, st) == hipSuccess;
        }
        e = hipStreamEndCapture(st, &g);
        if (!ok || e != hipSuccess) {
            if (g)
                (void)hipGraphDestroy(g);
            (void)hipGetLastError();
            return ok ? e : hipSuccess;        // a launch the device refused: not a candidate
        }
        float ms = 0.f;
        int reps = 1;
        if ((e = hipGraphInstantiate(&ge, g, nullptr, nullptr, 0)) == hipSuccess &&
            (e = hipGraphLaunch(ge, st)) == hipSuccess && (e = hipEventRecord(e0, st)) == hipSuccess &&
            (e = hipGraphLaunch(ge, st)) == hipSuccess && (e = hipEventRecord(e1, st)) == hipSuccess &&
            (e = hipEventSynchronize(e1)) == hipSuccess && (e = hipEventElapsedTime(&ms, e0, e1)) == hipSuccess &&
            ms < kMinTimedMs) {
            // a graph of short kernels: time enough replays to fill kMinTimedMs
            reps = std::min(64, (int)(kMinTimedMs / std::max(ms, 1e-4f)) + 1);
            if ((e = hipEventRecord(e0, st)) == hipSuccess) {
                for (int r = 0; r < reps && e == hipSuccess; ++r)
                    e = hipGraphLaunch(ge, st);
                if (e == hipSuccess && (e = hipEventRecord(e1, st)) == hipSuccess &&
                    (e = hipEventSynchronize(e1)) == hipSuccess)
                    e = hipEventElapsedTime(&ms, e0, e1);
            }
        }
        if (ge)
            (void)hipGraphExecDestroy(ge);
        (void)hipGraphDestroy(g);
        if (e != hipSuccess)
            return e;
        us = 1000.0 * ms / ((double)iters * reps);
        return hipSuccess;
    }
    static constexpr float kMinTimedMs = 0.2f;

    // Entries `ens` at M = m, each timed three times round-robin: best[c] is
    // the best of three of ens[c] (-1 if it did not run).
    hipError_t times_at(int m, const std::vector<const Entry *> &ens, std::vector<double> &best)
    {
        best.assign(ens.size(), -1.0);
        a.M = m;
        for (int round = 0; round < 3; ++round)
            for (size_t c = 0; c < ens.size(); ++c) {
                double us;
                hipError_t e = time_once(*ens[c], us);
                if (e != hipSuccess)
                    return e;
                if (us >= 0 && (best[c] < 0 || us < best[c]))
                    best[c] = us;
            }
        return hipSuccess;
    }
};

skinny_status tune(const void *W, int N, int K, int ldw, int half, skinny_out_dtype od, int nxcd,
                   std::array<skinny_tactic, SKINNY_MAX_M> &table)
{
    const int cus = device_cus();
    const int count = skinny_enumerate_tactics_ex(N, K, cus, nullptr, 0);
    if (count <= 0) {
        set_error("no candidate tactics for N=%d K=%d", N, K);
        return SKINNY_ERR_SHAPE;
    }
    std::vector<skinny_tactic> cand(count);
    skinny_enumerate_tactics_ex(N, K, cus, cand.data(), count);
    size_t max_ws = 0;
    for (const skinny_tactic &t : cand)
        max_ws = std::max(max_ws, ws_floats(make_entry(t, N, K, half)));
    Harness h;
    HIP_TRY(h.init(W, N, K, ldw, od, nxcd, max_ws));
    KArgs &a = h.a;
    const int copies = h.copies;
    auto time_once = [&](const Entry &en, double &us) { return h.time_once(en, us); };

    // First pass: every candidate at its full token tile, best of two, and
    // each candidate of a tile of 16 or more tokens also once at the small-M
    // probe (8 tokens), where those tiles serve most of their token counts.
    constexpr int kProbeM = 8;
    std::vector<double> times(count, -1.0), probe_times(count, -1.0);
    std::vector<Entry> entries(count);
    for (int i = 0; i < count; ++i) {
        entries[i] = make_entry(cand[i], N, K, half);
        const Entry &en = entries[i];
        if (!en.fn || !lds_fits(en.fn, en.lds))
            continue;
        a.M = cand[i].mt;
        a.W = h.wcopies.p;
        if (launch(en, a, h.st) != hipSuccess) {
            (void)hipGetLastError();
            continue;
        }
        double best = -1.0;
        for (int rep = 0; rep < 2; ++rep) {
            double us;
            HIP_TRY(time_once(en, us));
            if (us < 0) {
                best = -1.0;
                break;
            }
            if (best < 0 || us < best)
                best = us;
        }
        times[i] = best;
        if (best >= 0 && cand[i].mt >= 2 * kProbeM) {
            a.M = kProbeM;
            HIP_TRY(time_once(en, probe_times[i]));
        }
    }
    HIP_TRY(hipStreamSynchronize(h.st));
    skinny_status s = skinny_select_table(cand.data(), times.data(), count, table.data());

    // Second pass: for each M, the few fastest candidates of the first pass
    // whose tile serves M, and the two fastest of every token tile >= M, are
    // timed again at M itself (x and out of M rows), round-robin over three
    // rounds, and the fastest is kept; below 16 tokens so are the few fastest
    // at the small-M probe.  First-pass times at the full tile overstate a
    // large tile at small M -- the best 16-token kernel at M = 4 need not be
    // among the fastest at M = 16 -- and single timings differ by a few per
    // cent from run to run.
    const int refine = env_int("SKINNY_TUNE_REFINE", 4);
    // Candidates `top` at M = m, each timed three times round-robin: best[c]
    // is the best of three of top[c] (-1 if it did not run).
    auto times_at = [&](int m, const std::vector<int> &top, std::vector<double> &best) -> hipError_t {
        std::vector<const Entry *> ens;
        for (int i : top)
            ens.push_back(&entries[(size_t)i]);
        return h.times_at(m, ens, best);
    };
    // The fastest of candidates `top` at M = m; -1 if none ran.
    auto fastest_at = [&](int m, const std::vector<int> &top, int &pick) -> hipError_t {
        std::vector<double> best;
        hipError_t e = times_at(m, top, best);
        if (e != hipSuccess)
            return e;
        pick = -1;
        for (size_t c = 0; c < top.size(); ++c)
            if (best[c] >= 0 && (pick < 0 || best[c] < best[(size_t)pick]))
                pick = (int)c;
        pick = pick >= 0 ? top[(size_t)pick] : -1;
        return hipSuccess;
    };
    std::vector<int> chosen(SKINNY_MAX_M, -1);   // candidate index of table[m - 1], once re-timed
    for (int m = 1; s == SKINNY_OK && refine > 1 && m <= SKINNY_MAX_M; ++m) {
        std::vector<int> order;
        for (int i = 0; i < count; ++i)
            if (times[i] >= 0 && cand[i].mt >= m)
                order.push_back(i);
        std::sort(order.begin(), order.end(), [&](int x, int y) { return times[x] < times[y]; });
        std::vector<int> top;
        std::map<int, int> per_tile;
        for (size_t k = 0; k < order.size(); ++k) {
            const int i = order[k];
            if ((int)k < refine || per_tile[cand[i].mt] < 2)
                top.push_back(i);
            ++per_tile[cand[i].mt];
        }
        if (m < 2 * kProbeM) {
            std::vector<int> small;
            for (int i : order)
                if (probe_times[i] >= 0)
                    small.push_back(i);
            std::sort(small.begin(), small.end(), [&](int x, int y) { return probe_times[x] < probe_times[y]; });
            for (size_t k = 0; k < small.size() && (int)k < refine; ++k)
                if (std::find(top.begin(), top.end(), small[k]) == top.end())
                    top.push_back(small[k]);
        }
        if (top.size() < 2)
            continue;
        int pick = -1;
        HIP_TRY(fastest_at(m, top, pick));
        if (pick >= 0) {
            table[m - 1] = cand[pick];
            chosen[m - 1] = pick;
        }
    }
    // Third pass: every kernel the table now uses for some M is timed again
    // at each M its tile serves, and the fastest is kept.  The kernel that
    // wins at M = 8 is often the fastest at M = 4 as well without being among
    // the fastest candidates at its own full tile.
    if (s == SKINNY_OK && refine > 1) {
        std::vector<int> used;
        for (int i : chosen)
            if (i >= 0 && std::find(used.begin(), used.end(), i) == used.end())
                used.push_back(i);
        for (int m = 1; m <= SKINNY_MAX_M; ++m) {
            if (chosen[m - 1] < 0)
                continue;                          // its entry was not re-timed: keep it
            std::vector<int> top;                  // includes chosen[m - 1]
            for (int i : used)
                if (cand[i].mt >= m)
                    top.push_back(i);
            if (top.size() < 2)
                continue;
            int pick = -1;
            HIP_TRY(fastest_at(m, top, pick));
            if (pick >= 0)
                table[m - 1] = cand[pick];
        }
    }
    // Fourth pass: the dot2 paths are the arithmetic meant for token counts
    // up to 8, so at M <= 8 the fastest of the two quickest dot2 candidates
    // (DOT2, DOT2R, DOT2W) that serve M replaces the table's choice when it
    // is within SKINNY_TUNE_DOT2_MARGIN (relative, default 0.02: two timings
    // of one tactic differ by 1-2 % from run to run) of it, both timed again
    // at M.  A negative margin turns the preference off.
    const double margin = env_double("SKINNY_TUNE_DOT2_MARGIN", 0.02);
    if (s == SKINNY_OK && refine > 1 && margin >= 0) {
        for (int m = 1; m <= 8 && m <= SKINNY_MAX_M; ++m) {
            if (is_dot2_path(table[m - 1].path))
                continue;
            int cur = -1;
            for (int i = 0; i < count && cur < 0; ++i)
                if (memcmp(&cand[i], &table[m - 1], sizeof(skinny_tactic)) == 0)
                    cur = i;
            std::vector<int> dots;
            for (int i = 0; i < count; ++i)
                if (times[i] >= 0 && cand[i].mt >= m && is_dot2_path(cand[i].path))
                    dots.push_back(i);
            if (cur < 0 || dots.empty())
                continue;
            std::sort(dots.begin(), dots.end(), [&](int x, int y) { return times[x] < times[y]; });
            std::vector<int> top{cur};
            top.insert(top.end(), dots.begin(), dots.begin() + std::min<size_t>(2, dots.size()));
            std::vector<double> t;
            HIP_TRY(times_at(m, top, t));
            int best = -1;
            for (size_t c = 1; c < top.size(); ++c)
                if (t[c] >= 0 && (best < 0 || t[c] < t[(size_t)best]))
                    best = (int)c;
            if (best < 0 || t[0] < 0)
                continue;
            const bool take = t[(size_t)best] <= (1.0 + margin) * t[0];
            if (env_flag("SKINNY_LOG"))
                fprintf(stderr, "[skinny] N=%d K=%d M=%d: dot2 path %d at %.3f us, path %d at %.3f us, gap %+.1f %%%s\n",
                        N, K, m, cand[top[(size_t)best]].path, t[(size_t)best], table[m - 1].path, t[0],
                        100.0 * (t[(size_t)best] / t[0] - 1.0), take ? ": dot2 taken" : "");
            if (take)
                table[m - 1] = cand[top[(size_t)best]];
        }
    }
    if (env_int("SKINNY_LOG", 0) >= 2) {
        for (int i = 0; i < count; ++i)
            fprintf(stderr, "[skinny] cand N=%d K=%d path=%d mt=%d rows=%d waves=%d unroll=%d split=%d : %.3f us\n",
                    N, K, cand[i].path, cand[i].mt, cand[i].rows,
                    cand[i].waves, cand[i].unroll, cand[i].split, times[i]);
    }
    if (s == SKINNY_OK && env_flag("SKINNY_LOG")) {
        fprintf(stderr, "[skinny] tuned N=%d K=%d out=%s over %d candidates, %d weight copies\n", N, K,
                od == SKINNY_OUT_F32 ? "f32" : "bf16", count, copies);
    }
    return s;
}

// The table for runs with a residual.  The residual is read when a value is
// stored, after the reductions and any split-K exchange, so it lengthens the
// tails of the kernels unequally and can change which of them is fastest at
// an M (the pages' backend choice is keyed on has_residual for the same
// reason).  For each M, every distinct tactic of `table` whose token tile
// serves M is timed at M with a residual, best of three rounds; the fastest
// replaces the plain table's entry only if it beats that entry's own time by
// more than SKINNY_TUNE_RESIDUAL_MARGIN (relative, default 0.01, about the
// spread of two timings of one tactic) -- or, where the entry is a dot2
// kernel at M <= 8, by more than the dot2 margin the plain table was chosen
// with.
skinny_status tune_residual(const void *W, int N, int K, int ldw, int half, skinny_out_dtype od, int nxcd,
                            const Table &table, Table &res_table)
{
    res_table = table;
    std::vector<skinny_tactic> used;
    for (const skinny_tactic &t : table)
        if (std::none_of(used.begin(), used.end(),
                         [&](const skinny_tactic &u) { return memcmp(&u, &t, sizeof t) == 0; }))
            used.push_back(t);
    if (used.size() < 2)
        return SKINNY_OK;
    std::vector<Entry> ens;
    size_t max_ws = 0;
    for (const skinny_tactic &t : used) {
        ens.push_back(make_entry(t, N, K, half));
        max_ws = std::max(max_ws, ws_floats(ens.back()));
    }
    const double margin = std::max(0.0, env_double("SKINNY_TUNE_RESIDUAL_MARGIN", 0.01));
    const double dot2_margin = env_double("SKINNY_TUNE_DOT2_MARGIN", 0.02);
    Harness h;
    HIP_TRY(h.init(W, N, K, ldw, od, nxcd, max_ws));
    h.a.res = h.rbuf.p;
    for (size_t i = 0; i < ens.size(); ++i) {   // warm: load every code object before timing
        if (!ens[i].fn || !lds_fits(ens[i].fn, ens[i].lds))
            continue;
        h.a.M = used[i].mt;
        h.a.W = h.wcopies.p;
        if (launch(ens[i], h.a, h.st) != hipSuccess)
            (void)hipGetLastError();
    }
    HIP_TRY(hipStreamSynchronize(h.st));
    for (int m = 1; m <= SKINNY_MAX_M; ++m) {
        std::vector<const Entry *> top;
        std::vector<size_t> idx;
        for (size_t i = 0; i < used.size(); ++i)
            if (used[i].mt >= m && ens[i].fn && lds_fits(ens[i].fn, ens[i].lds)) {
                top.push_back(&ens[i]);
                idx.push_back(i);
            }
        if (top.size() < 2)
            continue;
        std::vector<double> best;
        HIP_TRY(h.times_at(m, top, best));
        int pick = -1, plain = -1;
        for (size_t c = 0; c < top.size(); ++c) {
            if (best[c] >= 0 && (pick < 0 || best[c] < best[(size_t)pick]))
                pick = (int)c;
            if (memcmp(&used[idx[c]], &table[m - 1], sizeof(skinny_tactic)) == 0)
                plain = (int)c;
        }
        if (pick < 0)
            continue;
        if (plain >= 0 && best[(size_t)plain] >= 0) {
            const bool dot2 = m <= 8 && is_dot2_path(table[m - 1].path) && dot2_margin >= 0;
            const double keep = dot2 ? std::max(margin, dot2_margin) : margin;
            if (best[(size_t)pick] * (1.0 + keep) >= best[(size_t)plain])
                pick = plain;
        }
        res_table[m - 1] = used[idx[(size_t)pick]];
        if (env_flag("SKINNY_LOG") && memcmp(&res_table[m - 1], &table[m - 1], sizeof(skinny_tactic)) != 0)
            fprintf(stderr, "[skinny] N=%d K=%d M=%d with a residual: path %d mt %d split %d at %.3f us\n", N, K,
                    m, res_table[m - 1].path, res_table[m - 1].mt, res_table[m - 1].split, best[(size_t)pick]);
    }
    return SKINNY_OK;
}

skinny_status build_plan(const void *W, int N, int K, int ldw, int half, skinny_out_dtype od, int dev, int nxcd,
                         const skinny_tactic *table, const skinny_tactic *res_table, skinny_plan **out)
{
    for (const skinny_tactic *tb : {table, res_table})
        for (int m = 1; m <= SKINNY_MAX_M; ++m) {
            const skinny_tactic &t = tb[m - 1];
            skinny_status s = skinny_tactic_check(&t, N, K);
            if (s != SKINNY_OK)
                return s;
            if (t.mt < m) {
                set_error("table entry for M=%d has token tile %d < M", m, t.mt);
                return SKINNY_ERR_INVALID_ARG;
            }
        }
    skinny_plan *p = new (std::nothrow) skinny_plan;
    if (!p) {
        set_error("host allocation of the plan failed");
        return SKINNY_ERR_NOMEM;
    }
    p->device = dev;
    p->W = W;
    p->N = N;
    p->K = K;
    p->ldw = ldw;
    p->half = half;
    p->od = od;
    size_t max_ws = 0;
    for (int m = 1; m <= SKINNY_MAX_M; ++m) {
        p->e[m] = make_entry(table[m - 1], N, K, half);
        p->er[m] = make_entry(res_table[m - 1], N, K, half);
        for (const Entry *en : {&p->e[m], &p->er[m]}) {
            if (!en->fn || !lds_fits(en->fn, en->lds)) {
                set_error("table entry for M=%d needs %u bytes of dynamic LDS, more than the device allows "
                          "with the kernel's static LDS", m, en->lds);
                delete p;
                return SKINNY_ERR_INVALID_ARG;
            }
            max_ws = std::max(max_ws, ws_floats(*en));
        }
    }
    auto fail = [&](skinny_status s) {
        skinny_destroy(p);
        return s;
    };
    hipError_t e;
    if (max_ws) {
        if ((e = hipMalloc(&p->ws, max_ws * 4)) != hipSuccess) {
            hip_fail(e, "hipMalloc(split-K workspace)");
            return fail(e == hipErrorOutOfMemory ? SKINNY_ERR_NOMEM : SKINNY_ERR_HIP);
        }
        if ((e = hipMemset(p->ws, 0, max_ws * 4)) != hipSuccess) {   // every exchange node empty
            hip_fail(e, "hipMemset(split-K workspace)");
            return fail(SKINNY_ERR_HIP);
        }
    }
    p->base = weight_args(W, N, K, ldw, od, nxcd, p->ws);
    KArgs &a = p->base;

    // Warm every distinct kernel the tables use, on scratch x/out, so that no
    // code object loads lazily inside a later graph capture.
    void *xs = nullptr, *os = nullptr;
    if ((e = hipMalloc(&xs, (size_t)SKINNY_MAX_M * K * 2)) != hipSuccess) {
        hip_fail(e, "hipMalloc(warm-up x)");
        return fail(SKINNY_ERR_HIP);
    }
    if ((e = hipMalloc(&os, (size_t)SKINNY_MAX_M * N * 4)) != hipSuccess) {
        (void)hipFree(xs);
        hip_fail(e, "hipMalloc(warm-up out)");
        return fail(SKINNY_ERR_HIP);
    }
    e = hipMemset(xs, 0, (size_t)SKINNY_MAX_M * K * 2);
    std::vector<skinny_tactic> warmed;
    for (int m = 1; m <= SKINNY_MAX_M && e == hipSuccess; ++m)
        for (const Entry *en : {&p->e[m], &p->er[m]}) {
            if (e != hipSuccess || std::any_of(warmed.begin(), warmed.end(), [&](const skinny_tactic &t) {
                    return memcmp(&t, &en->t, sizeof t) == 0;
                }))
                continue;
            warmed.push_back(en->t);
            KArgs w = a;
            w.x = xs;
            w.out = os;
            w.M = m;
            e = launch(*en, w, nullptr);
        }
    if (e == hipSuccess)
        e = hipDeviceSynchronize();
    (void)hipFree(xs);
    (void)hipFree(os);
    if (e != hipSuccess) {
        hip_fail(e, "warm-up launch");
        return fail(SKINNY_ERR_HIP);
    }
    if (env_flag("SKINNY_LOG")) {
        for (int m = 1; m <= SKINNY_MAX_M; ++m) {
            char buf[160];
            skinny_describe(p, m, buf, sizeof buf);
            fprintf(stderr, "[skinny] N=%d K=%d M=%d -> %s\n", N, K, m, buf);
        }
    }
    *out = p;
    return SKINNY_OK;
}

// ---------------------------------------------------------------------------
// Allocation-free runs (skinny_run_static): the split-K exchange nodes live in
// a file-scope device array, one copy per device, zero at load and left zero
// (empty) by every launch.  In host code `scratch` only names the symbol; its
// device address is looked up once per device and kept in g_scratch.
// ---------------------------------------------------------------------------
static __device__ __align__(256) float scratch[SKINNY_STATIC_SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's copy of `scratch`, looked up on its first use.
skinny_status scratch_of_device(int dev, float **ptr)
{
    if (dev < 0 || dev >= kMaxDevices) {
        set_error("device %d: the static scratch serves devices 0..%d", dev, kMaxDevices - 1);
        return SKINNY_ERR_DEVICE;
    }
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p)
                return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = static_cast<float *>(p);
    return SKINNY_OK;
}

// The LDS limit check of lds_fits without its cache (which allocates).
bool lds_fits_now(const void *fn, unsigned dynamic_bytes)
{
    int dev = 0, max_lds = 0;
    hipFuncAttributes attr{};
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
        hipFuncGetAttributes(&attr, fn) != hipSuccess)
        return false;
    return attr.sharedSizeBytes + dynamic_bytes <= (size_t)max_lds;
}

}  // namespace

extern "C" {

skinny_status skinny_prepare_ex(const void *W, int N, int K, int ldw, skinny_in_dtype in_dtype,
                                skinny_out_dtype od, skinny_plan **plan)
{
    skinny_status s = check_prepare_args(W, N, K, ldw, (int)in_dtype, od, plan);
    if (s != SKINNY_OK)
        return s;
    // SKINNY_FORCE_TACTIC: one tactic for every M its tile serves and the
    // 64-token MFMA tactic above it, with no tuning and no table file
    const char *force = getenv("SKINNY_FORCE_TACTIC");
    if (force && *force) {
        skinny_tactic ft;
        if (!parse_tactic_text(force, &ft)) {
            set_error("SKINNY_FORCE_TACTIC=\"%.64s\" is not path.mt.rows.waves.unroll.split", force);
            return SKINNY_ERR_INVALID_ARG;
        }
        if ((s = skinny_tactic_check(&ft, N, K)) != SKINNY_OK)
            return s;
        const skinny_tactic above = {SKINNY_PATH_MFMA, SKINNY_MAX_M, 16, 1, 1, 1};
        skinny_tactic table[SKINNY_MAX_M];
        for (int m = 1; m <= SKINNY_MAX_M; ++m)
            table[m - 1] = m <= ft.mt ? ft : above;
        return skinny_prepare_tactics_ex(W, N, K, ldw, in_dtype, od, table, plan);
    }
    const int half = in_dtype == SKINNY_IN_F16;
    int dev = 0, cus = 0;
    if ((s = current_gfx950(&dev, &cus)) != SKINNY_OK)
        return s;
    raise_lds_limits();
    const int nxcd = cus % 8 == 0 ? 8 : 1;
    Tables tb;
    {
        std::lock_guard<std::mutex> lock(g_cache_mu);
        const Key key{dev, N, K, half, (int)od};
        auto it = g_cache.find(key);
        const char *file = getenv("SKINNY_TABLE_CACHE");
        const bool use_file = file && *file;
        if (it != g_cache.end()) {
            tb = it->second;
        } else {
            if (use_file && load_table_file(file, cus, N, K, half, od, 0, tb.plain)) {
                if (env_flag("SKINNY_LOG"))
                    fprintf(stderr, "[skinny] N=%d K=%d: table loaded from %s\n", N, K, file);
            } else {
                if ((s = tune(W, N, K, ldw, half, od, nxcd, tb.plain)) != SKINNY_OK)
                    return s;
                if (use_file)
                    save_table_file(file, cus, N, K, half, od, 0, tb.plain);
            }
            if (use_file && load_table_file(file, cus, N, K, half, od, 1, tb.residual)) {
                if (env_flag("SKINNY_LOG"))
                    fprintf(stderr, "[skinny] N=%d K=%d: residual table loaded from %s\n", N, K, file);
            } else if (env_int("SKINNY_TUNE_RESIDUAL", 1) == 0) {
                tb.residual = tb.plain;
            } else {
                if ((s = tune_residual(W, N, K, ldw, half, od, nxcd, tb.plain, tb.residual)) != SKINNY_OK)
                    return s;
                if (use_file)
                    save_table_file(file, cus, N, K, half, od, 1, tb.residual);
            }
            g_cache[key] = tb;
        }
    }
    return build_plan(W, N, K, ldw, half, od, dev, nxcd, tb.plain.data(), tb.residual.data(), plan);
}

skinny_status skinny_prepare(const void *W, int N, int K, skinny_out_dtype od, skinny_plan **plan)
{
    return skinny_prepare_ex(W, N, K, K, SKINNY_IN_BF16, od, plan);
}

skinny_status skinny_prepare_tactics_ex(const void *W, int N, int K, int ldw, skinny_in_dtype in_dtype,
                                        skinny_out_dtype od, const skinny_tactic *table, skinny_plan **plan)
{
    skinny_status s = check_prepare_args(W, N, K, ldw, (int)in_dtype, od, plan);
    if (s != SKINNY_OK)
        return s;
    if (!table) {
        set_error("table is NULL");
        return SKINNY_ERR_INVALID_ARG;
    }
    for (int m = 1; m <= SKINNY_MAX_M; ++m) {
        if ((s = skinny_tactic_check(&table[m - 1], N, K)) != SKINNY_OK)
            return s;
        if (table[m - 1].mt < m) {
            set_error("table entry for M=%d has token tile %d < M", m, table[m - 1].mt);
            return SKINNY_ERR_INVALID_ARG;
        }
    }
    int dev = 0, cus = 0;
    if ((s = current_gfx950(&dev, &cus)) != SKINNY_OK)
        return s;
    raise_lds_limits();
    // the caller's table serves runs with and without a residual alike
    return build_plan(W, N, K, ldw, in_dtype == SKINNY_IN_F16, od, dev, cus % 8 == 0 ? 8 : 1, table, table, plan);
}

skinny_status skinny_prepare_tactics(const void *W, int N, int K, skinny_out_dtype od,
                                     const skinny_tactic *table, skinny_plan **plan)
{
    return skinny_prepare_tactics_ex(W, N, K, K, SKINNY_IN_BF16, od, table, plan);
}

skinny_status skinny_run_ex(const skinny_plan *p, const void *x, int ldx, const void *residual, int ldr,
                            void *out, int ldo, int M, void *stream)
{
    if (!p) {
        set_error("plan is NULL");
        return SKINNY_ERR_INVALID_ARG;
    }
    skinny_status s = check_run_args(p->N, p->K, p->od, x, ldx, residual, ldr, out, ldo, M);
    if (s != SKINNY_OK)
        return s;
    KArgs a = p->base;
    set_call_args(a, x, ldx, residual, ldr, out, ldo, M);
    hipError_t e = launch(residual ? p->er[M] : p->e[M], a, (hipStream_t)stream);
    if (e != hipSuccess)
        return hip_fail(e, "hipLaunchKernel");
    return SKINNY_OK;
}

skinny_status skinny_run(const skinny_plan *p, const void *x, void *out, int M, void *stream)
{
    return skinny_run_ex(p, x, p ? p->K : 0, nullptr, 0, out, p ? p->N : 0, M, stream);
}

skinny_status skinny_run_static(const void *W, int N, int K, int ldw, skinny_in_dtype in_dtype,
                                skinny_out_dtype out_dtype, const skinny_tactic *tactic, const void *x, int ldx,
                                const void *residual, int ldr, void *out, int ldo, int M, void *stream)
{
    skinny_plan *unused = nullptr;           // check_prepare_args writes through it; nothing is built
    skinny_status s = check_prepare_args(W, N, K, ldw, (int)in_dtype, out_dtype, &unused);
    if (s != SKINNY_OK)
        return s;
    if (!tactic) {
        set_error("tactic is NULL");
        return SKINNY_ERR_INVALID_ARG;
    }
    if ((s = check_run_args(N, K, out_dtype, x, ldx, residual, ldr, out, ldo, M)) != SKINNY_OK)
        return s;
    if ((s = skinny_tactic_check(tactic, N, K)) != SKINNY_OK)
        return s;
    if (tactic->mt < M) {
        set_error("the tactic's token tile %d is smaller than M=%d", tactic->mt, M);
        return SKINNY_ERR_INVALID_ARG;
    }
    int dev = 0, cus = 0;
    if ((s = current_gfx950(&dev, &cus)) != SKINNY_OK)
        return s;
    raise_lds_limits();
    const Entry en = make_entry(*tactic, N, K, in_dtype == SKINNY_IN_F16);
    if (!en.fn || !lds_fits_now(en.fn, en.lds)) {
        set_error("the tactic needs %u bytes of dynamic LDS, more than the device allows with the kernel's "
                  "static LDS", en.lds);
        return SKINNY_ERR_INVALID_ARG;
    }
    const size_t need = ws_floats(en) * sizeof(float);
    if (need > SKINNY_STATIC_SCRATCH_BYTES) {
        set_error("the tactic's split-K exchange needs %zu bytes of scratch; the static scratch holds %d",
                  need, SKINNY_STATIC_SCRATCH_BYTES);
        return SKINNY_ERR_SHAPE;
    }
    float *ws = nullptr;
    if (need && (s = scratch_of_device(dev, &ws)) != SKINNY_OK)
        return s;
    KArgs a = weight_args(W, N, K, ldw, out_dtype, cus % 8 == 0 ? 8 : 1, ws);
    set_call_args(a, x, ldx, residual, ldr, out, ldo, M);
    hipError_t e = launch(en, a, (hipStream_t)stream);
    if (e != hipSuccess)
        return hip_fail(e, "hipLaunchKernel");
    return SKINNY_OK;
}

int skinny_supports(const skinny_plan *p, int M) { return p && M >= 1 && M <= SKINNY_MAX_M; }

skinny_status skinny_plan_tactic_ex(const skinny_plan *p, int M, int has_residual, skinny_tactic *out)
{
    if (!p || !out) {
        set_error("plan or out is NULL");
        return SKINNY_ERR_INVALID_ARG;
    }
    if (M < 1 || M > SKINNY_MAX_M) {
        set_error("M=%d outside 1..%d", M, SKINNY_MAX_M);
        return SKINNY_ERR_UNSUPPORTED_M;
    }
    *out = has_residual ? p->er[M].t : p->e[M].t;
    return SKINNY_OK;
}

skinny_status skinny_plan_tactic(const skinny_plan *p, int M, skinny_tactic *out)
{
    return skinny_plan_tactic_ex(p, M, 0, out);
}

skinny_status skinny_describe(const skinny_plan *p, int M, char *buf, size_t len)
{
    skinny_tactic t;
    skinny_status s = skinny_plan_tactic(p, M, &t);
    if (s != SKINNY_OK)
        return s;
    if (!buf || len == 0) {
        set_error("buf is NULL or empty");
        return SKINNY_ERR_INVALID_ARG;
    }
    const Entry &en = p->e[M];
    static const char *const kNames[] = {"dot2", "mfma16x16x32", "dot2x", "mfmax16x16x32", "mfmad16x16x32",
                                         "mfmas16x16x32", "mfmar16x16x32", "mfmak16x16x32", "dot2r",
                                         "mfmaw16x16x32", "mfma4x4x4", "dot2w", "mfmat16x16x32"};
    constexpr int kPaths = (int)(sizeof(kNames) / sizeof(kNames[0]));
    snprintf(buf, len, "%s mt=%d rows=%d waves=%d unroll=%d split=%d grid=%u block=%u lds=%u",
             (t.path >= 0 && t.path < kPaths) ? kNames[t.path] : "?", t.mt, t.rows, t.waves, t.unroll, t.split,
             en.grid, en.block, en.lds);
    return SKINNY_OK;
}

void skinny_destroy(skinny_plan *p)
{
    if (!p)
        return;
    if (p->ws) {
        int cur = -1;
        (void)hipGetDevice(&cur);
        if (cur != p->device)
            (void)hipSetDevice(p->device);
        (void)hipDeviceSynchronize();
        (void)hipFree(p->ws);
        if (cur != p->device && cur >= 0)
            (void)hipSetDevice(cur);
    }
    delete p;
}

int skinny_probe_read_blocks(void) { return kProbeSinkFloats; }

skinny_status skinny_probe_read(const void *buf, size_t bytes, float *sink, void *stream)
{
    if (!buf || !sink) {
        set_error("buf or sink is NULL");
        return SKINNY_ERR_INVALID_ARG;
    }
    if (((uintptr_t)buf & 15) || (bytes & 15)) {
        set_error("buf must be 16-byte aligned and bytes a multiple of 16");
        return SKINNY_ERR_ALIGN;
    }
    long chunks = (long)(bytes / 16);
    const long blocks = (chunks + 255) / 256;
    if (blocks < 1 || blocks > 0x7FFFFFFF) {
        set_error("probe_read: %zu bytes out of range", bytes);
        return SKINNY_ERR_INVALID_ARG;
    }
    void *params[] = {&buf, &chunks, &sink};
    hipError_t e = hipLaunchKernel(probe_read_fn(), dim3((unsigned)blocks), dim3(64), params, 0,
                                   (hipStream_t)stream);
    return e == hipSuccess ? SKINNY_OK : hip_fail(e, "hipLaunchKernel(probe_read)");
}

skinny_status skinny_probe_empty(void *stream)
{
    hipError_t e = hipLaunchKernel(probe_empty_fn(), dim3(1), dim3(64), nullptr, 0, (hipStream_t)stream);
    return e == hipSuccess ? SKINNY_OK : hip_fail(e, "hipLaunchKernel(probe_empty)");
}

}  // extern "C"
