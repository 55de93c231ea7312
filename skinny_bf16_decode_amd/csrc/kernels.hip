// HIP kernels of the skinny BF16 decode projection for gfx950 (CDNA4).
//
//   out[m][n] = sum_k x[m][k] * W[n][k]     (m < M <= 64, n < N)
//
// the decode-step product "out[M, N] = x[M, K] @ weight[N, K]^T" of class
// PreparedWarpSplitK on the page "vllm.models.kimi_k3.nvidia.specialized_decode.
// cutedsl.gemm.warp_splitk".  At decode sizes the whole cost is streaming W
// once from HBM, so both kernels are organised around the weight stream:
//
//  * Each lane loads 16 bytes (8 BF16 of one row) per load, with the
//    nontemporal bit, so one wave's load is a contiguous 1 KiB run (DOT2) or
//    sixteen 64-byte runs (MFMA).  W is touched once and must not evict x or
//    out from L2 -- the role the page's evict_first L2 policy plays there.
//  * Workgroups own few rows (the page's small 16/32-row output tiles that let
//    many blocks co-reside per SM), and split K across their waves: every
//    wave holds fp32 partials of the same outputs over a different K range
//    (the page's four compute warps that each own a K quarter), reduced at
//    the end through DPP / lane swaps inside the wave and LDS across waves.
//  * Optionally `split` workgroups share one row tile along K; each writes
//    its fp32 partial to a workspace and the last to arrive sums the partials
//    in a fixed order and writes the output (the split-K GEMM of the page
//    "vllm.models.glm5next.nvidia.specialized_decode.gemm", which reduces its
//    split-K partials across a thread-block cluster; here the exchange goes
//    through memory with agent-scope atomic stores and loads and an
//    arrival counter).
//
// DOT2 (token tiles 1..8): v_dot2_f32_bf16, two BF16 products into an fp32
// accumulator per instruction.  MFMA (token tiles 16..64): W rows are the
// 16-row A operand and tokens the 16-column B operand of
// v_mfma_f32_16x16x32_bf16 (the warp split-K page also puts the weight on the
// MMA's row side and the tokens on its column side).
//
// Accumulation is fp32 throughout; BF16 output is rounded to nearest even
// once, from the final fp32 sum.
#include <hip/hip_runtime.h>

#include "skinny_internal.h"

namespace skinny {

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// ---------------------------------------------------------------------------
// Small helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ u32x4 load_stream(const u32x4 *p) { return __builtin_nontemporal_load(p); }

// Reinterpret one 32-bit word as two BF16 values.  The word arrives as a
// by-value argument on purpose: applying __builtin_bit_cast directly to an
// ext-vector component (w.y, w.z, ...) makes this clang extract component 0
// whatever the component named, so components are copied to scalars first.
__device__ __forceinline__ bf16x2 as_bf16x2(unsigned int word) { return __builtin_bit_cast(bf16x2, word); }

typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;

// The same for two FP16 values.
__device__ __forceinline__ f16x2 as_f16x2(unsigned int word) { return __builtin_bit_cast(f16x2, word); }

// 8-element dot product accumulated into acc: 4 x v_dot2_f32_bf16, or
// 4 x v_dot2_f32_f16 for FP16 inputs (H).  Both multiply exactly and add in
// fp32.
template <bool H>
__device__ __forceinline__ float dot8(u32x4 w, u32x4 x, float acc)
{
    const unsigned int w0 = w.x, w1 = w.y, w2 = w.z, w3 = w.w;
    const unsigned int x0 = x.x, x1 = x.y, x2 = x.z, x3 = x.w;
    if constexpr (H) {
        acc = __builtin_amdgcn_fdot2(as_f16x2(w0), as_f16x2(x0), acc, false);
        acc = __builtin_amdgcn_fdot2(as_f16x2(w1), as_f16x2(x1), acc, false);
        acc = __builtin_amdgcn_fdot2(as_f16x2(w2), as_f16x2(x2), acc, false);
        acc = __builtin_amdgcn_fdot2(as_f16x2(w3), as_f16x2(x3), acc, false);
    } else {
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w0), as_bf16x2(x0), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w1), as_bf16x2(x1), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w2), as_bf16x2(x2), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w3), as_bf16x2(x3), acc, false);
    }
    return acc;
}

// One 16x16x32 MFMA step, c += a b, with a and b holding 8 BF16 (or, H,
// FP16) values per lane.
template <bool H>
__device__ __forceinline__ f32x4 mma16(u32x4 a, u32x4 b, f32x4 c)
{
    if constexpr (H)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
}

// Workgroup -> (row tile, K split).  The dispatcher deals consecutive
// workgroup ids round-robin over the XCDs; with `remap`, ids are renumbered
// so that consecutive logical indices -- the `split` workgroups of one row
// tile -- sit on the same XCD (a bijection of [0, gridDim.x)).
// A value the caller knows is the same in every lane, made provably so.  The
// row counts in the kernels come from HIP's min/max, whose results this compiler treats
// as divergent; a buffer resource built from a "divergent" size is then
// re-materialised lane by lane around every load.
__device__ __forceinline__ int uniform_int(int v) { return __builtin_amdgcn_readfirstlane(v); }

// x / d for the divisor whose FastDiv the host made (values shared by every
// lane: scalar multiply-high, add and shifts)
__device__ __forceinline__ unsigned fdiv(unsigned x, const FastDiv &f)
{
    const unsigned t = __umulhi(x, f.mul);
    return (t + ((x - t) >> f.s1)) >> f.s2;
}

__device__ __forceinline__ void block_coords(const KArgs &a, int &tile, int &s)
{
    unsigned idx = blockIdx.x;
    if (a.remap) {
        // gridDim.x = grid_q nxcd + grid_r: XCD x holds grid_q (+ 1 if x < grid_r) ids
        const unsigned j = fdiv(idx, a.fd_nxcd), xcd = idx - j * (unsigned)a.nxcd;
        idx = xcd * (unsigned)a.grid_q + (xcd < (unsigned)a.grid_r ? xcd : (unsigned)a.grid_r) + j;
    }
    const unsigned t = fdiv(idx, a.fd_split);
    tile = (int)t;
    s = (int)(idx - t * (unsigned)a.split);
}

// First row of equal row range t, floor(t N / n_tiles), t <= n_tiles.  With
// N = rows_q n_tiles + rows_r it is t rows_q + floor(t rows_r / n_tiles), in
// 32 bits while n_tiles < 2^16; otherwise the plain 64-bit form.
__device__ __forceinline__ int tile_row(const KArgs &a, int t)
{
    if (a.rows_fast)
        return uniform_int((int)((unsigned)t * a.rows_q + fdiv((unsigned)t * a.rows_r, a.fd_tiles)));
    return uniform_int((int)(((unsigned long long)(unsigned)t * (unsigned)a.N) / (unsigned)a.n_tiles));
}

// First unit of K part s of `split` over `total` units, floor(s total /
// split), s <= split <= 16: s total < 2^32 because K / 8 < 2^28.
__device__ __forceinline__ int split_point(const KArgs &a, int s, int total)
{
    return (int)fdiv((unsigned)s * (unsigned)total, a.fd_split);
}

// out[m][n] = v (+ res[m][n], added in fp32 before the one rounding to BF16)
__device__ __forceinline__ void store_out(const KArgs &a, int m, int n, float v)
{
    const long off = (long)m * a.ldo + n;
    if (a.res) {
        const long roff = (long)m * a.ldr + n;
        v += a.out_f32 ? static_cast<const float *>(a.res)[roff] : (float)static_cast<const __bf16 *>(a.res)[roff];
    }
    if (a.out_f32)
        static_cast<float *>(a.out)[off] = v;
    else
        static_cast<__bf16 *>(a.out)[off] = (__bf16)v;   // v_cvt_pk_bf16_f32: nearest even
}

// ---------------------------------------------------------------------------
// In-wave reduction that also transposes: V fp32 partials per lane (V a power
// of two, V <= 64) are summed over all 64 lanes.  At each of the six steps the
// lanes pair up across one lane-index bit; the lane with the bit clear keeps
// the first half of its vector, the other keeps the second half, and each
// adds its partner's copy of the half it keeps.  Once the vector is down to
// one value the remaining steps are plain butterflies.  Afterwards lane l
// holds the full sum of value index l >> (6 - log2 V).
//   bit 5: v_permlane32_swap    bit 4: v_permlane16_swap
//   bit 3: DPP row_mirror       bit 2: DPP row_half_mirror
//   bit 1: DPP quad_perm xor 2  bit 0: DPP quad_perm xor 1
// (the mirrors pair lane i with 15 - i and 7 - i, which differ in bit 3 and
// bit 2 respectively, so they serve as the pairing for those bits).
// ---------------------------------------------------------------------------

template <int V>
__device__ __forceinline__ void step_swap32(float *v)
{
    if constexpr (V >= 2) {
#pragma unroll
        for (int i = 0; i < V / 2; ++i) {
            auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]),
                                                      __float_as_uint(v[i + V / 2]), false, false);
            v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        }
    } else {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[0]), __float_as_uint(v[0]),
                                                  false, false);
        v[0] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
}

template <int V>
__device__ __forceinline__ void step_swap16(float *v)
{
    if constexpr (V >= 2) {
#pragma unroll
        for (int i = 0; i < V / 2; ++i) {
            auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]),
                                                      __float_as_uint(v[i + V / 2]), false, false);
            v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        }
    } else {
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[0]), __float_as_uint(v[0]),
                                                  false, false);
        v[0] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
}

template <int CTRL>
__device__ __forceinline__ float dpp_read(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

template <int V, int CTRL, int BIT>
__device__ __forceinline__ void step_dpp(float *v, int lane)
{
    if constexpr (V >= 2) {
        const bool hi = (lane & BIT) != 0;
#pragma unroll
        for (int i = 0; i < V / 2; ++i) {
            const float send = hi ? v[i] : v[i + V / 2];
            const float keep = hi ? v[i + V / 2] : v[i];
            v[i] = keep + dpp_read<CTRL>(send);
        }
    } else {
        v[0] = v[0] + dpp_read<CTRL>(v[0]);
    }
}

constexpr int half_of(int v) { return v > 1 ? v / 2 : 1; }

constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]

template <int V>
__device__ __forceinline__ void wave_reduce_transpose(float *v, int lane)
{
    static_assert(V >= 1 && V <= 64 && (V & (V - 1)) == 0, "V must be a power of two <= 64");
    constexpr int V1 = half_of(V), V2 = half_of(V1), V3 = half_of(V2), V4 = half_of(V3),
                  V5 = half_of(V4);
    step_swap32<V>(v);
    step_swap16<V1>(v);
    step_dpp<V2, kDppRowMirror, 8>(v, lane);
    step_dpp<V3, kDppRowHalfMirror, 4>(v, lane);
    step_dpp<V4, kDppQuadXor2, 2>(v, lane);
    step_dpp<V5, kDppQuadXor1, 1>(v, lane);
}

// ---------------------------------------------------------------------------
// Cross-workgroup split-K exchange.
//
// Partials are written with agent-scope atomic stores and read back with
// agent-scope atomic loads; on gfx950 these are the write-through / coherent
// forms of the plain access (sc1), so no L2 writeback is needed to publish
// them.  An agent-scope release fence would add one (buffer_wbl2), and those
// writebacks serialise per XCD.
//
// Every slot of the workspace holds kSlotEmpty, a signalling-NaN pattern that
// no fp32 arithmetic produces, except while a partial is in it.  A workgroup
// publishes its partial and bumps the tile's arrival counter with an
// agent-scope atomic straight away, without waiting for its stores to
// complete: the workgroup that sees split - 1 arrivals before its own knows
// that every partial has been issued, and reads each slot until it no longer
// holds kSlotEmpty (a store in flight always lands; the re-read is bounded
// all the same).  It sums the partials in split order, so the sum is
// deterministic, then empties the slots and resets the counter for the next
// launch.  Against waiting for the stores before the atomic this takes one
// memory round trip off the end of every split launch.
// ---------------------------------------------------------------------------
constexpr unsigned kSlotEmpty = kSlotEmptyBits;
constexpr int kSlotSpinLimit = 1 << 16;

__device__ __forceinline__ void publish_partial(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned read_slot(const float *p)
{
    return __hip_atomic_load(reinterpret_cast<const unsigned *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void empty_slot(float *p)
{
    __hip_atomic_store(reinterpret_cast<unsigned *>(p), kSlotEmpty, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The last arriver's sum of a thread's N output values over the partial
// slots: v[i] = sum over p < parts, in slot order from 0, of slot p at
// offset off[i] (slots `stride` floats apart); off[i] < 0 is no value.  The
// loads of four slots are all issued before the first add, so the reduction
// costs ceil(parts / 4) memory round trips instead of parts x N.  Each slot
// is emptied once read; no two threads may name the same offset.
template <int N>
__device__ __forceinline__ void sum_partials(float *wsp, long stride, int parts, const int (&off)[N],
                                             float (&v)[N])
{
#pragma unroll
    for (int i = 0; i < N; ++i)
        v[i] = 0.f;
    for (int p0 = 0; p0 < parts; p0 += 4) {
        unsigned r[4][N];
        bool empty = false;
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int i = 0; i < N; ++i) {
                r[k][i] = p0 + k < parts && off[i] >= 0 ? read_slot(wsp + (long)(p0 + k) * stride + off[i]) : 0u;
                empty |= r[k][i] == kSlotEmpty;
            }
        // a store still in flight: read the empty slots again, with one
        // bounded budget for the whole batch (past it the sum is a NaN)
        for (int spin = 0; empty && spin < kSlotSpinLimit; ++spin) {
            empty = false;
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int i = 0; i < N; ++i)
                    if (r[k][i] == kSlotEmpty) {
                        r[k][i] = read_slot(wsp + (long)(p0 + k) * stride + off[i]);
                        empty |= r[k][i] == kSlotEmpty;
                    }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (p0 + k < parts)
#pragma unroll
                for (int i = 0; i < N; ++i) {
                    v[i] += __builtin_bit_cast(float, r[k][i]);
                    if (off[i] >= 0)
                        empty_slot(wsp + (long)(p0 + k) * stride + off[i]);
                }
    }
}

// Called by every thread of the workgroup after it issued its partial's stores.
__device__ __forceinline__ bool split_arrive_last(const KArgs &a, int tile, unsigned *flag_lds)
{
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev =
            __hip_atomic_fetch_add(a.ctr + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag_lds = (prev == (unsigned)(a.split - 1)) ? 1u : 0u;
    }
    __syncthreads();
    return *flag_lds != 0;
}

__device__ __forceinline__ void split_reset(const KArgs &a, int tile)
{
    if (threadIdx.x == 0)
        __hip_atomic_store(a.ctr + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Buffer loads.  Each workgroup builds a buffer resource over its own row
// tile of W (num_records = valid rows * row bytes) and one over x
// (num_records = M * row bytes).  A load whose offset falls outside the
// resource returns zeros without touching memory, so rows >= N of a ragged
// last tile and token rows >= M read as zero with no branch, and x rows >= M
// are never read.  Per-lane parts of an address go in the vector offset, the
// workgroup-uniform stage offset in the scalar offset.  A lane whose chunk is
// past the end of its K range uses kOffOob, which is out of range for any
// resource here (tiles are far below 2 GiB).
// ---------------------------------------------------------------------------
constexpr unsigned kOffOob = 0x7FFFFFF0u;
constexpr int kCpolNt = 2;   // nontemporal


// A per-lane offset that is either a real offset or kOffOob.  Passing it
// through an empty asm keeps it a plain select: otherwise this compiler may
// split the load into two branch arms (one per offset), and the branches
// bring their own waits on every load in flight.
__device__ __forceinline__ unsigned lane_off(bool ok, unsigned off)
{
    unsigned r = ok ? off : kOffOob;
    asm volatile("" : "+v"(r));
    return r;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, unsigned bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 load_w(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kCpolNt);
}

__device__ __forceinline__ u32x4 load_x(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}

// ---------------------------------------------------------------------------
// DOT2 kernel: token tile MT <= 8, R rows per workgroup, U chunks per lane
// per pipeline stage.
//
// Lane t of the workgroup (T = blockDim.x lanes) takes chunks kb + t,
// kb + t + T, ... of its K range, for all R rows at once: every wave-wide
// load is 1 KiB of one row, and the MT x chunks a lane loads are reused over
// the R rows.  The K loop is a two-stage register pipeline: the loads of
// stage j + 1 are issued before stage j is multiplied, so every wave keeps
// U * (R + MT) 16-byte loads in flight while it computes.
// ---------------------------------------------------------------------------
template <int MT, int R, int U, bool H>
__global__ __launch_bounds__(512) void k_dot2(KArgs a)
{
    constexpr int V = MT * R;   // partial sums per lane, index m * R + r
    __shared__ float red[kMaxWaves][V];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int nthr = blockDim.x, nwaves = nthr >> 6;
    int tile, s;
    block_coords(a, tile, s);
    // row tile: R aligned rows, or (ranges) the equal range
    // [tile N / n_tiles, (tile + 1) N / n_tiles) of at most R rows
    const int n0 = a.ranges ? tile_row(a, tile) : tile * R;
    const int n_end = a.ranges ? tile_row(a, tile + 1) : a.N;
    const int kb = split_point(a, s, a.K8);
    const int ke = split_point(a, s + 1, a.K8);
    const unsigned row_bytes = a.w_pitch, x_pitch = a.x_pitch;
    const int rows_valid = uniform_int(max(0, min(R, n_end - n0)));
    const auto wres = make_rsrc(static_cast<const char *>(a.W) + (size_t)n0 * row_bytes,
                                (unsigned)rows_valid * row_bytes);
    const auto xres = make_rsrc(a.x, (unsigned)a.M * x_pitch);
    const unsigned lane_off = (unsigned)(kb + tid) * 16u;
    const unsigned pass_bytes = (unsigned)nthr * 16u;

    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i)
        acc[i] = 0.f;

    // passes in which every lane has a chunk; nthr = 64 waves is a power of two
    const int passes = (ke - kb) >> __builtin_ctz((unsigned)nthr);
    const int stages = passes / U;

    u32x4 wa[U][R], xa[U][MT], wb[U][R], xb[U][MT];
    auto load = [&](u32x4(&w)[U][R], u32x4(&x)[U][MT], int j) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const unsigned so = (unsigned)(j * U + u) * pass_bytes;
#pragma unroll
            for (int r = 0; r < R; ++r)
                w[u][r] = load_w(wres, (unsigned)r * row_bytes + lane_off, so);
#pragma unroll
            for (int m = 0; m < MT; ++m)
                x[u][m] = load_x(xres, (unsigned)m * x_pitch + lane_off, so);
        }
        // keep the scheduler from hoisting the previous stage's arithmetic
        // above these loads: they must be in flight while it runs
        __builtin_amdgcn_sched_barrier(0);
    };
    auto compute = [&](const u32x4(&w)[U][R], const u32x4(&x)[U][MT]) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    acc[m * R + r] = dot8<H>(w[u][r], x[u][m], acc[m * R + r]);
    };
    // Loads inside the loop are unconditional: a load under a branch would
    // leave the two paths with different counts of loads in flight, and the
    // wait inserted at the join would then drain the whole pipeline.
    if (stages > 0) {
        load(wa, xa, 0);
        int j = 0;
        for (; j + 2 < stages; j += 2) {
            load(wb, xb, j + 1);
            compute(wa, xa);
            load(wa, xa, j + 2);
            compute(wb, xb);
        }
        if (j + 1 < stages) {
            load(wb, xb, j + 1);
            compute(wa, xa);
            compute(wb, xb);
        } else {
            compute(wa, xa);
        }
    }
    // remaining whole passes, then the partial pass (lanes past ke read zeros)
    for (int p = stages * U; p * nthr < ke - kb; ++p) {
        const bool ok = kb + tid + p * nthr < ke;
        const unsigned so = (unsigned)p * pass_bytes;
        u32x4 w[1][R], x[1][MT];
#pragma unroll
        for (int r = 0; r < R; ++r)
            w[0][r] = load_w(wres, ok ? (unsigned)r * row_bytes + lane_off : kOffOob, so);
#pragma unroll
        for (int m = 0; m < MT; ++m)
            x[0][m] = load_x(xres, ok ? (unsigned)m * x_pitch + lane_off : kOffOob, so);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m)
                acc[m * R + r] = dot8<H>(w[0][r], x[0][m], acc[m * R + r]);
    }

    wave_reduce_transpose<V>(acc, lane);
    constexpr int kLanesPerValue = 64 / V;
    if ((lane & (kLanesPerValue - 1)) == 0)
        red[wave][lane / kLanesPerValue] = acc[0];
    __syncthreads();

    if (wave != 0)
        return;   // V <= 64: wave 0 finishes the tile
    float total = 0.f;
    if (tid < V) {
        for (int w = 0; w < nwaves; ++w)
            total += red[w][tid];
    }
    const int m = tid / R, r = tid - (tid / R) * R, n = n0 + r;
    const bool live = tid < V && m < a.M && n < n_end;
    if (a.split == 1) {
        if (live)
            store_out(a, m, n, total);
        return;
    }
    // split-K: publish this workgroup's partial, the last arriver finalises.
    // Only wave 0 is left and it holds the whole partial, so the arrival is a
    // wave-level one (no workgroup barrier once the other waves have exited).
    float *wsp = a.ws + (long)tile * a.split * V;
    if (live)                                  // exactly the slots the finaliser reads
        publish_partial(wsp + (long)s * V + tid, total);
    unsigned prev = 0;
    if (lane == 0)
        prev = __hip_atomic_fetch_add(a.ctr + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev != (unsigned)(a.split - 1))
        return;
    if (live) {
        const int off[1] = {tid};
        float sum[1];
        sum_partials<1>(wsp, V, a.split, off, sum);
        store_out(a, m, n, sum[0]);
    }
    if (lane == 0)
        __hip_atomic_store(a.ctr + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// MFMA kernel: token tile MT = 16 T (T = 1, 2, 4), rows per workgroup
// NT = 16 RT, U K-steps per wave per pipeline stage.
//
// One K-step is 32 K (4 chunks).  In v_mfma_f32_16x16x32_bf16 lane l = 16 g + i
// supplies A[i][8g .. 8g+7] and B[8g .. 8g+7][i]; here A row i is weight row
// n0 + 16 rt + i and B column i is token 16 t + i, both at chunk 4 step + g,
// so lane l loads 16 bytes of one weight row and 16 bytes of one token row.
// Token columns >= M fall outside the x resource and load zeros.  Wave w of
// the workgroup takes steps sb + w, sb + w + waves, ... (in-workgroup
// split-K) through the same two-stage pipeline as the DOT2 kernel; the 16x16
// fp32 results (lane l holds rows 4 (l / 16) .. +3 of column l % 16) are
// summed over waves in LDS, laid out [wave][token][row] so that the final
// stores of out[token][n0 + row] are row-contiguous.
// ---------------------------------------------------------------------------
template <int T, int RT, int U, bool H>
__global__ __launch_bounds__(512) void k_mfma(KArgs a)
{
    constexpr int MT = 16 * T, NT = 16 * RT, NTP = NT + 1;
    extern __shared__ float lds[];   // [waves][MT][NTP]
    __shared__ unsigned flag;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int nthr = blockDim.x, nwaves = nthr >> 6;
    int tile, s;
    block_coords(a, tile, s);
    const int n0 = tile * NT;
    const int i16 = lane & 15, g = lane >> 4;

    const int steps_full = a.K8 >> 2;              // steps with all 4 chunks in range
    const int steps = (a.K8 + 3) >> 2;
    const int sb = split_point(a, s, steps);
    const int se = split_point(a, s + 1, steps);
    const int se_full = se < steps_full ? se : steps_full;

    const unsigned row_bytes = a.w_pitch, x_pitch = a.x_pitch;
    const int rows_valid = uniform_int(min(NT, a.N - n0));
    const auto wres = make_rsrc(static_cast<const char *>(a.W) + (size_t)n0 * row_bytes,
                                (unsigned)rows_valid * row_bytes);
    const auto xres = make_rsrc(a.x, (unsigned)a.M * x_pitch);
    const unsigned k_off = (unsigned)(4 * (sb + wave) + g) * 16u;   // this lane's first chunk
    const unsigned step_bytes = (unsigned)nwaves * 64u;             // one step of every wave

    f32x4 acc[RT][T];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int t = 0; t < T; ++t)
            acc[rt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // this wave's steps: sb + wave + nwaves * q, q = 0 .. qn - 1 (all full)
    const int first = sb + wave;
    const int qn = first < se_full ? (se_full - first + nwaves - 1) >> __builtin_ctz((unsigned)nwaves) : 0;
    const int stages = qn / U;

    u32x4 aa[U][RT], ba[U][T], ab[U][RT], bb[U][T];
    auto load = [&](u32x4(&av)[U][RT], u32x4(&bv)[U][T], int j) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const unsigned so = (unsigned)(j * U + u) * step_bytes;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                av[u][rt] = load_w(wres, (unsigned)(16 * rt + i16) * row_bytes + k_off, so);
#pragma unroll
            for (int t = 0; t < T; ++t)
                bv[u][t] = load_x(xres, (unsigned)(16 * t + i16) * x_pitch + k_off, so);
        }
        __builtin_amdgcn_sched_barrier(0);   // loads stay ahead of the MFMAs
    };
    auto compute = [&](const u32x4(&av)[U][RT], const u32x4(&bv)[U][T]) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int t = 0; t < T; ++t)
                    acc[rt][t] = mma16<H>(av[u][rt], bv[u][t], acc[rt][t]);
    };
    if (stages > 0) {   // same pipeline shape as the DOT2 kernel
        load(aa, ba, 0);
        int j = 0;
        for (; j + 2 < stages; j += 2) {
            load(ab, bb, j + 1);
            compute(aa, ba);
            load(aa, ba, j + 2);
            compute(ab, bb);
        }
        if (j + 1 < stages) {
            load(ab, bb, j + 1);
            compute(aa, ba);
            compute(ab, bb);
        } else {
            compute(aa, ba);
        }
    }
    // remaining whole steps, then the partial last step when K8 % 4 != 0
    for (int q = stages * U; first + q * nwaves < se; ++q) {
        const bool ok = 4 * (first + q * nwaves) + g < a.K8;
        const unsigned so = (unsigned)q * step_bytes;
        u32x4 av[1][RT], bv[1][T];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            av[0][rt] = load_w(wres, ok ? (unsigned)(16 * rt + i16) * row_bytes + k_off : kOffOob, so);
#pragma unroll
        for (int t = 0; t < T; ++t)
            bv[0][t] = load_x(xres, ok ? (unsigned)(16 * t + i16) * x_pitch + k_off : kOffOob, so);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int t = 0; t < T; ++t)
                acc[rt][t] = mma16<H>(av[0][rt], bv[0][t], acc[rt][t]);
    }

    // accumulator fragments -> LDS [wave][token][row]
    float *mine = lds + (long)wave * MT * NTP;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                mine[(16 * t + i16) * NTP + 16 * rt + 4 * g + q] = acc[rt][t][q];
    __syncthreads();

    constexpr int E = MT * NT;
    const int mlim = a.M < MT ? a.M : MT;
    if (a.split == 1) {
        for (int e = tid; e < E; e += nthr) {
            const int tok = e / NT, row = e - (e / NT) * NT;
            if (tok >= mlim || n0 + row >= a.N)
                continue;
            float v = 0.f;
            for (int w = 0; w < nwaves; ++w)
                v += lds[((long)w * MT + tok) * NTP + row];
            store_out(a, tok, n0 + row, v);
        }
        return;
    }
    float *wsp = a.ws + (long)tile * a.split * E;
    for (int e = tid; e < E; e += nthr) {
        const int tok = e / NT, row = e - (e / NT) * NT;
        if (tok >= mlim)
            continue;
        float v = 0.f;
        for (int w = 0; w < nwaves; ++w)
            v += lds[((long)w * MT + tok) * NTP + row];
        publish_partial(wsp + (long)s * E + e, v);
    }
    if (!split_arrive_last(a, tile, &flag))
        return;
    for (int e0 = tid; e0 < E; e0 += 4 * nthr) {
        int off[4];
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {             // the published values: tokens < mlim
            const int e = e0 + i * nthr;
            off[i] = e < E && e / NT < mlim ? e : -1;
        }
        sum_partials<4>(wsp, E, a.split, off, v);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = e0 + i * nthr;
            const int tok = e / NT, row = e - (e / NT) * NT;
            if (e < E && tok < mlim && n0 + row < a.N)
                store_out(a, tok, n0 + row, v[i]);
        }
    }
    split_reset(a, tile);
}

// ---------------------------------------------------------------------------
// DOT2X kernel: token tile MT <= 8; each wave owns R rows of the workgroup's
// row tile (waves * R rows), and the x slice of the workgroup's K range is
// staged once in LDS, shared by all rows of the workgroup.
//
// Every wave streams its own rows over the whole K range of the split: lane
// l takes chunks kb + l, kb + l + 64, ... of each of its R rows, so a
// wave-wide load is 1 KiB of one row and U loads per row form U KiB
// contiguous runs.  The x operands come from LDS (one ds_read per token and
// chunk, reused over the R rows), which takes them off the vector-memory
// path: only W flows through it.  No cross-wave reduction is needed; the
// in-wave transposing reduction finishes each wave's R x MT outputs.
// ---------------------------------------------------------------------------
template <int MT, int R, int U, bool H>
__global__ __launch_bounds__(512) void k_dot2x(KArgs a)
{
    constexpr int V = MT * R;
    extern __shared__ u32x4 xs[];   // [MT][kr] chunks of x[0..MT)[kb..ke)
    __shared__ unsigned flag;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nthr = blockDim.x, nwaves = nthr >> 6;
    int tile, s;
    block_coords(a, tile, s);
    const int n_wg = tile * nwaves * R;        // first row of the workgroup
    const int n0 = n_wg + wave * R;            // first row of this wave
    const int kb = split_point(a, s, a.K8);
    const int ke = split_point(a, s + 1, a.K8);
    const int kr = ke - kb;
    const unsigned row_bytes = a.w_pitch, x_pitch = a.x_pitch;
    const int rows_valid = uniform_int(max(0, min(R, a.N - n0)));
    const auto wres = make_rsrc(static_cast<const char *>(a.W) + (size_t)(rows_valid ? n0 : 0) * row_bytes,
                                (unsigned)rows_valid * row_bytes);
    const auto xres = make_rsrc(a.x, (unsigned)a.M * x_pitch);
    const unsigned lane_off = (unsigned)(kb + lane) * 16u;
    constexpr unsigned kPass = 64u * 16u;      // one wave-wide pass: 64 chunks

    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i)
        acc[i] = 0.f;

    const int passes = kr / 64;
    const int stages = passes / U;
    u32x4 wa[U][R], wb[U][R];
    auto load = [&](u32x4(&w)[U][R], int j) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const unsigned so = (unsigned)(j * U + u) * kPass;
#pragma unroll
            for (int r = 0; r < R; ++r)
                w[u][r] = load_w(wres, (unsigned)r * row_bytes + lane_off, so);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto compute = [&](const u32x4(&w)[U][R], int j) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = lane + 64 * (j * U + u);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const u32x4 xv = xs[m * kr + c];
#pragma unroll
                for (int r = 0; r < R; ++r)
                    acc[m * R + r] = dot8<H>(w[u][r], xv, acc[m * R + r]);
            }
        }
    };

    // First weight stage in flight before the activations are staged.
    if (stages > 0)
        load(wa, 0);
    {
        const int total = MT * kr;
        for (int q0 = tid; q0 < total; q0 += 8 * nthr) {
            u32x4 v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int q = q0 + i * nthr;
                const int m = q / kr, c = q - (q / kr) * kr;
                v[i] = load_x(xres, q < total ? (unsigned)m * x_pitch + (unsigned)(kb + c) * 16u : kOffOob, 0);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int q = q0 + i * nthr;
                if (q < total)
                    xs[q] = v[i];
            }
        }
    }
    __syncthreads();

    if (stages > 0) {
        int j = 0;
        for (; j + 2 < stages; j += 2) {
            load(wb, j + 1);
            compute(wa, j);
            load(wa, j + 2);
            compute(wb, j + 1);
        }
        if (j + 1 < stages) {
            load(wb, j + 1);
            compute(wa, j);
            compute(wb, j + 1);
        } else {
            compute(wa, j);
        }
    }
    for (int p = stages * U; p * 64 < kr; ++p) {
        const int c = lane + 64 * p;
        const bool ok = c < kr;
        const unsigned so = (unsigned)p * kPass;
        u32x4 w[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            w[r] = load_w(wres, ok ? (unsigned)r * row_bytes + lane_off : kOffOob, so);
        const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const u32x4 xv = ok ? xs[m * kr + (ok ? c : 0)] : zero;   // index kept in range
#pragma unroll
            for (int r = 0; r < R; ++r)
                acc[m * R + r] = dot8<H>(w[r], xv, acc[m * R + r]);
        }
    }

    wave_reduce_transpose<V>(acc, lane);
    constexpr int kLanesPerValue = 64 / V;
    const bool holder = (lane & (kLanesPerValue - 1)) == 0;
    const int idx = lane / kLanesPerValue;     // value index m * R + r
    const int m = idx / R, r = idx - (idx / R) * R;
    if (a.split == 1) {
        if (holder && m < a.M && n0 + r < a.N)
            store_out(a, m, n0 + r, acc[0]);
        return;
    }
    const int E = nwaves * V;                  // partial values of the workgroup
    float *wsp = a.ws + (long)tile * a.split * E;
    if (holder)
        publish_partial(wsp + (long)s * E + wave * V + idx, acc[0]);
    if (!split_arrive_last(a, tile, &flag))
        return;
    for (int e0 = tid; e0 < E; e0 += 4 * nthr) {
        int off[4];
        float v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            off[k] = e0 + k * nthr < E ? e0 + k * nthr : -1;
        sum_partials<4>(wsp, E, a.split, off, v);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int e = e0 + k * nthr;
            const int w = e / V, i = e - (e / V) * V;
            const int mm = i / R, rr = i - (i / R) * R, n = n_wg + w * R + rr;
            if (e < E && mm < a.M && n < a.N)
                store_out(a, mm, n, v[k]);
        }
    }
    split_reset(a, tile);
}

// The last arriver of a tile whose partials are MFMA accumulator fragments
// (value e = ((wave T + t) 4 + q) 64 + lane: token 16 t + lane % 16, row
// n_wg + 16 wave + 4 (lane / 16) + q) sums the slots and stores the rows
// below n_end.
template <int T, int NW>
__device__ __forceinline__ void finalize_mfma_tile(const KArgs &a, float *wsp, int E, int parts, int n_wg,
                                                   int n_end)
{
    constexpr int EPT = 4 * T;                 // values per thread: E = 64 NW EPT
    int off[EPT];
    float v[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i)
        off[i] = (int)threadIdx.x + 64 * NW * i;
    sum_partials<EPT>(wsp, E, parts, off, v);
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = off[i];
        const int ln = e & 63, q = (e >> 6) & 3, wt = e >> 8;
        const int w = wt / T, t = wt - (wt / T) * T;
        const int tok = 16 * t + (ln & 15), n = n_wg + 16 * w + 4 * (ln >> 4) + q;
        if (tok < a.M && n < n_end)
            store_out(a, tok, n, v[i]);
    }
}

// ---------------------------------------------------------------------------
// MFMAX kernel: token tile MT = 16 T; NW waves each own 16 weight rows.
//
// The weight is loaded row-contiguously -- each wave-wide load covers two
// rows x 512 bytes, full 128-byte lines -- into registers, one stage (32
// chunks = 8 K-steps of 32) ahead, and re-laid out through a wave-private LDS
// tile [16 rows][32 chunks] from which each lane reads its A fragment (row i,
// chunk 4 step + g).  The x window [MT tokens][32 chunks] of the same stage is
// loaded cooperatively by the workgroup into a double-buffered LDS tile and
// read as B fragments.  Loading W with the 16-row MFMA pattern directly would
// split every request into 64-byte halves of lines.
//
// Row pitch of both tiles: 34 chunks (544 bytes).  With 16 lanes reading 16
// rows of one 16-byte column, gfx950's LDS served the 128-bit reads without a
// bank conflict only for row pitches of 2 mod 4 chunks (34, 66, 70, 130 ...);
// a pitch of 33 chunks cost 4 conflict cycles per read and 32 chunks 28
// (SQ_LDS_BANK_CONFLICT per SQ_INSTS_LDS, measured).  Writes of whole rows
// were conflict-free at every pitch tried.
// ---------------------------------------------------------------------------
template <int T, int NW, bool H>
__global__ __launch_bounds__(512) void k_mfmax(KArgs a)
{
    constexpr int MT = 16 * T;
    constexpr int KW = kMfmaxChunks;           // chunks per stage
    constexpr int PITCH = KW + 2;              // row pitch in 16-byte chunks (see above)
    constexpr int XL = (MT * KW) / (64 * NW);  // x chunks per thread per stage
    constexpr int NX = mfmax_x_windows(MT);    // x windows in LDS: a barrier per NX / 2 stages
    constexpr int PB = NX / 2;                 // stages per barrier
    static_assert(XL >= 1 && XL * 64 * NW == MT * KW, "x window must split evenly over the waves");
    extern __shared__ u32x4 sm[];              // [NW][16][PITCH] then [NX][MT][PITCH]
    __shared__ unsigned flag;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tile, s;
    block_coords(a, tile, s);
    // row tile: 16 NW aligned rows, or (ranges) the equal range
    // [tile N / n_tiles, (tile + 1) N / n_tiles) of at most 16 NW rows
    const int n_wg = a.ranges ? tile_row(a, tile) : tile * NW * 16;
    const int n_end = a.ranges ? tile_row(a, tile + 1) : a.N;
    const int n0 = n_wg + wave * 16;
    const int kb = split_point(a, s, a.K8);
    const int ke = split_point(a, s + 1, a.K8);
    const int stages = (ke - kb + KW - 1) / KW;
    const unsigned row_bytes = a.w_pitch, x_pitch = a.x_pitch;
    const int rows_valid = uniform_int(max(0, min(16, n_end - n0)));
    const auto wres = make_rsrc(static_cast<const char *>(a.W) + (size_t)(rows_valid ? n0 : 0) * row_bytes,
                                (unsigned)rows_valid * row_bytes);
    const auto xres = make_rsrc(a.x, (unsigned)a.M * x_pitch);
    u32x4 *wl = sm + wave * 16 * PITCH;
    u32x4 *xl = sm + NW * 16 * PITCH;

    // weight loads: instruction q covers rows 2q + (lane >> 5), chunk lane & 31
    const int wrow = lane >> 5, wcol = lane & 31;
    const int i16 = lane & 15, g = lane >> 4;

    f32x4 acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t)
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Two weight register buffers: while stage j is written to LDS and
    // multiplied, the weight loads of stages j + 1 and j + 2 are in flight;
    // the x of the next PB stages is in flight in xr.
    u32x4 wa[8], wb[8], xr[PB][XL];
    auto load_wt = [&](u32x4(&wv)[8], int j) {
        const int c = kb + j * KW + wcol;      // this lane's weight chunk
        const bool wok = j < stages && c < ke;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            wv[q] = load_w(wres, wok ? (unsigned)(2 * q + wrow) * row_bytes + (unsigned)c * 16u : kOffOob, 0);
    };
    auto load_xw = [&](u32x4(&xv)[XL], int j) {
#pragma unroll
        for (int i = 0; i < XL; ++i) {
            const int e = tid + 64 * NW * i;
            const int tok = e / KW, cc = kb + j * KW + (e % KW);
            const bool xok = j < stages && cc < ke;
            xv[i] = load_x(xres, xok ? (unsigned)tok * x_pitch + (unsigned)cc * 16u : kOffOob, 0);
        }
    };
    auto put_w = [&](const u32x4(&wv)[8]) {
#pragma unroll
        for (int q = 0; q < 8; ++q)
            wl[(2 * q + wrow) * PITCH + wcol] = wv[q];
    };
    auto put_x = [&](const u32x4(&xv)[XL], int j) {
        u32x4 *xw = xl + (j % NX) * MT * PITCH;
#pragma unroll
        for (int i = 0; i < XL; ++i) {
            const int e = tid + 64 * NW * i;
            xw[(e / KW) * PITCH + (e % KW)] = xv[i];
        }
    };
    // multiply stage j: A fragments from the wave's W tile, B from x window j
    auto compute = [&](int j) {
        const u32x4 *xw = xl + (j % NX) * MT * PITCH;
        if constexpr (T <= 2) {
            // fragments are read four K-steps at a time, so one LDS round
            // trip feeds 4 T MFMAs
#pragma unroll
            for (int h = 0; h < KW / 16; ++h) {
                u32x4 av[4], bv[4][T];
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    av[s4] = wl[i16 * PITCH + 4 * (4 * h + s4) + g];
#pragma unroll
                    for (int t = 0; t < T; ++t)
                        bv[s4][t] = xw[(16 * t + i16) * PITCH + 4 * (4 * h + s4) + g];
                }
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
                    for (int t = 0; t < T; ++t)
                        acc[t] = mma16<H>(av[s4], bv[s4][t], acc[t]);
            }
        } else {
#pragma unroll
            for (int st = 0; st < KW / 4; ++st) {
                const u32x4 av = wl[i16 * PITCH + 4 * st + g];
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const u32x4 bv = xw[(16 * t + i16) * PITCH + 4 * st + g];
                    acc[t] = mma16<H>(av, bv, acc[t]);
                }
            }
        }
    };
    if constexpr (PB >= 2) {
        // One barrier per PB stages: the x windows of stages j .. j + PB - 1
        // are written, then the barrier, then the PB stages are multiplied.
        // Window j % NX is rewritten PB stages later, after every wave has
        // passed the next barrier, i.e. finished multiplying stage j.  The
        // weight tile is private to the wave and needs no barrier.  Loads are
        // issued in the loop's own order from the start -- the x of PB stages,
        // then the weights stage by stage -- and every pass issues all of
        // them (past the last stage they touch no memory), so every wait in
        // the loop stays partial.
#pragma unroll
        for (int p = 0; p < PB; ++p)
            load_xw(xr[p], p);
        __builtin_amdgcn_sched_barrier(0);
        load_wt(wa, 0);
        __builtin_amdgcn_sched_barrier(0);
        load_wt(wb, 1);
        __builtin_amdgcn_sched_barrier(0);
        for (int j = 0; j < stages; j += PB) {
#pragma unroll
            for (int p = 0; p < PB; ++p)
                put_x(xr[p], j + p);
#pragma unroll
            for (int p = 0; p < PB; ++p)
                load_xw(xr[p], j + PB + p);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
#pragma unroll
            for (int p = 0; p < PB; p += 2) {
                put_w(wa);
                load_wt(wa, j + p + 2);
                __builtin_amdgcn_sched_barrier(0);
                if (j + p < stages)
                    compute(j + p);
                put_w(wb);
                load_wt(wb, j + p + 3);
                __builtin_amdgcn_sched_barrier(0);
                if (j + p + 1 < stages)
                    compute(j + p + 1);
            }
        }
    } else {
        u32x4(&xa)[XL] = xr[0];
        u32x4 xb[XL];
        load_wt(wa, 0);
        load_xw(xa, 0);
        load_wt(wb, 1);
        load_xw(xb, 1);
        auto stage = [&](u32x4(&wv)[8], u32x4(&xv)[XL], int j) {
            put_w(wv);
            put_x(xv, j);
            load_wt(wv, j + 2);                // past the last stage: out of range, no access
            load_xw(xv, j + 2);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            compute(j);
        };
        int j = 0;
        for (; j + 1 < stages; j += 2) {
            stage(wa, xa, j);
            stage(wb, xb, j + 1);
        }
        if (j < stages)
            stage(wa, xa, j);
    }

    // lane (g, i) holds rows 4g .. 4g+3 (of this wave's 16) of token 16 t + i
    if (a.split == 1) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int tok = 16 * t + i16;
            if (tok >= a.M)
                continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + 4 * g + q;
                if (n < n_end)
                    store_out(a, tok, n, acc[t][q]);
            }
        }
        return;
    }
    constexpr int E = NW * T * 4 * 64;         // partial values of the workgroup
    float *wsp = a.ws + (long)tile * a.split * E;
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            publish_partial(wsp + (long)s * E + ((wave * T + t) * 4 + q) * 64 + lane, acc[t][q]);
    if (!split_arrive_last(a, tile, &flag))
        return;
    finalize_mfma_tile<T, NW>(a, wsp, E, a.split, n_wg, n_end);
    split_reset(a, tile);
}

// ---------------------------------------------------------------------------
// MFMAD kernel: token tile MT = 16 T; NW waves each own 16 weight rows; the
// weight and activation tiles stream straight into LDS rings D stages deep.
//
// A stage is 32 K-chunks (512 bytes of a row, 8 MFMA K-steps).  Loads use the
// direct-to-LDS form of the 16-byte buffer load: lane l of a load writes LDS
// bytes [16 l, 16 l + 16) of the load's destination, while its global address
// is free.  Each load covers two rows: lanes 0-31 fill row 2q, lanes 32-63 row
// 2q + 1, and the lane at LDS position p of row r fetches chunk p ^ r (r < 16),
// so that the 16 rows of one K column sit in 16 different bank groups when
// the MFMA fragments are read back (lane (g, i) reads row i, chunk 4 step + g,
// at position (4 step + g) ^ i).  Loads past the end of a row range, of the
// weight (rows >= N) or of x (tokens >= M) are out of the buffer resource and
// write zeros.  The weight ring is private to each wave; the x ring is filled
// cooperatively and shared, so one barrier per stage orders both its fill
// and the reuse of its slots.  The loads of D - 1 stages are in flight while a
// stage is multiplied, and none of it passes through registers.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, u32x4 *lds_dst, unsigned voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds_dst, 16, voff, 0, 0, kCpolNt);
}

template <int T, int NW, int D, bool H>
__global__ __launch_bounds__(512) void k_mfmad(KArgs a)
{
    constexpr int MT = 16 * T;
    constexpr int KW = 32;                       // chunks per stage
    constexpr int XI = MT / (2 * NW);            // x loads per wave per stage
    static_assert(XI >= 1 && XI * 2 * NW == MT, "x tile must split evenly over the waves");
    constexpr int WSLOT = 16 * KW;               // u32x4 per weight slot (8 KiB)
    constexpr int XSLOT = MT * KW;               // u32x4 per x slot
    extern __shared__ u32x4 sm[];                // [NW][D][WSLOT] then [D][XSLOT]
    __shared__ unsigned flag;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tile, s;
    block_coords(a, tile, s);
    const int n_wg = tile * NW * 16;
    const int n0 = n_wg + wave * 16;
    const int kb = split_point(a, s, a.K8);
    const int ke = split_point(a, s + 1, a.K8);
    const int stages = (ke - kb + KW - 1) / KW;
    const unsigned row_bytes = a.w_pitch, x_pitch = a.x_pitch;
    const int rows_valid = uniform_int(max(0, min(16, a.N - n0)));
    const auto wres = make_rsrc(static_cast<const char *>(a.W) + (size_t)(rows_valid ? n0 : 0) * row_bytes,
                                (unsigned)rows_valid * row_bytes);
    const auto xres = make_rsrc(a.x, (unsigned)a.M * x_pitch);
    u32x4 *wring = sm + wave * D * WSLOT;
    u32x4 *xring = sm + NW * D * WSLOT;

    // DMA lane mapping: row (or token) parity from lane >> 5, LDS position from lane & 31
    const int half = lane >> 5, pos = lane & 31;
    const int i16 = lane & 15, g = lane >> 4;

    // Stage j into slot j % D; chunks past the split (or stages past the last)
    // get an out-of-range offset and land as zeros.  Every call issues exactly
    // 8 + XI loads on every lane -- the waits below count on it -- so the
    // validity test is a per-lane select, never a branch.
    auto issue = [&](int j) {
        const int slot = j % D;
        const int cbase = kb + j * KW;
        const int lim = j < stages ? ke : kb;    // no chunk is valid past the last stage
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int r = 2 * q + half;
            const int c = cbase + (pos ^ r);
            const unsigned off = c < lim ? (unsigned)r * row_bytes + (unsigned)c * 16u : kOffOob;
            dma16(wres, wring + slot * WSLOT + 2 * q * KW, off);
        }
#pragma unroll
        for (int i = 0; i < XI; ++i) {
            const int pair = wave + NW * i;        // tokens 2 pair, 2 pair + 1
            const int tok = 2 * pair + half;
            const int c = cbase + (pos ^ (tok & 15));
            const unsigned off = c < lim ? (unsigned)tok * x_pitch + (unsigned)c * 16u : kOffOob;
            dma16(xres, xring + slot * XSLOT + 2 * pair * KW, off);
        }
    };

    f32x4 acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t)
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int j = 0; j < D - 1; ++j)
        issue(j);
    for (int j = 0; j < stages; ++j) {
        // this wave's loads of stage j are done once at most D - 2 stages remain outstanding
        if constexpr (D == 2)
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        else if constexpr (D == 3)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(8 + XI) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * (8 + XI)) : "memory");
        // Every wave's share of stage j has landed once all waves pass here.
        // A bare barrier: __syncthreads would also wait for every load in
        // flight (its release fence), draining the ring.  The asm is a
        // compiler barrier too, so no LDS read moves above it.
        asm volatile("s_barrier" ::: "memory");
        issue(j + D - 1);                        // refills the slot stage j - 1 used
        const u32x4 *wsl = wring + (j % D) * WSLOT;
        const u32x4 *xsl = xring + (j % D) * XSLOT;
#pragma unroll
        for (int st = 0; st < KW / 4; ++st) {
            const int p = (4 * st + g) ^ i16;
            const u32x4 av = wsl[i16 * KW + p];
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const u32x4 bv = xsl[(16 * t + i16) * KW + p];
                acc[t] = mma16<H>(av, bv, acc[t]);
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no load may land after the wave ends

    // lane (g, i) holds rows 4g .. 4g+3 (of this wave's 16) of token 16 t + i
    if (a.split == 1) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int tok = 16 * t + i16;
            if (tok >= a.M)
                continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + 4 * g + q;
                if (n < a.N)
                    store_out(a, tok, n, acc[t][q]);
            }
        }
        return;
    }
    constexpr int E = NW * T * 4 * 64;           // partial values of the workgroup
    float *wsp = a.ws + (long)tile * a.split * E;
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            publish_partial(wsp + (long)s * E + ((wave * T + t) * 4 + q) * 64 + lane, acc[t][q]);
    if (!split_arrive_last(a, tile, &flag))
        return;
    finalize_mfma_tile<T, NW>(a, wsp, E, a.split, n_wg, a.N);
    split_reset(a, tile);
}

// ---------------------------------------------------------------------------
// MFMAS kernel: token tile MT = 16 T, NW waves each own 16 rows of a row
// tile of at most 16 NW rows, under a stream-K schedule, with U weight
// stages in flight in registers.
//
// The work is the flat list of units (row tile t, K stage k), t < n_tiles,
// k < spt = ceil(K / 256), and workgroup g of G takes units [g U / G,
// (g + 1) U / G).  Tile t is the row range [t N / n_tiles, (t + 1) N /
// n_tiles), so tiles differ by at most one row.  With G = the workgroups
// that fit on the chip at once (MFMAS), every workgroup streams the same
// amount of weight and none waits for a second round; with G = n_tiles
// (MFMAR, split 1) each workgroup owns one whole tile, and n_tiles may be
// raised to the CU count so that every CU gets one equal row range and no
// partial sums are exchanged.
//
// A stage is 32 K-chunks (512 bytes of each row).  The weight is loaded
// row-contiguously (each wave-wide load is two rows x 512 bytes) into
// registers U stages ahead, and re-laid out through a wave-private LDS tile
// [16 rows][34 chunks] from which lane (g, i) reads its A fragment (row i,
// chunk 4 step + g); the x window [MT tokens][32 chunks] of a stage is
// loaded by the whole workgroup into a double-buffered LDS tile and read as
// B fragments, so x is fetched once per tile, not once per wave.
//
// A range meets at most two cut tiles: the tile it starts in (unless it
// starts at the tile's first stage) and the tile it ends in (unless it ends
// at the tile's last stage); the tiles between are whole and stored as they
// complete.  A cut tile is shared by consecutive workgroups: each publishes
// its fp32 partial in slot (g - first workgroup of the tile), arrives on the
// tile's counter, and the last to arrive sums the slots in order
// (deterministic) and stores.  The partial of the first cut tile is kept in
// registers until the loop is over, so that every exchange store is issued
// after the last weight load.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int sk_owner(unsigned u, unsigned units, unsigned G)
{
    // the workgroup whose range [g U / G, (g + 1) U / G) contains unit u
    return (int)((((unsigned long long)u + 1) * G - 1) / units);
}

template <int T, int NW, int U, bool H>
__global__ __launch_bounds__(512) void k_mfmas(KArgs a)
{
    constexpr int MT = 16 * T;
    constexpr int KW = kMfmaxChunks;           // chunks per stage
    constexpr int PITCH = KW + 2;              // row pitch in 16-byte chunks (see k_mfmax)
    constexpr int XL = (MT * KW) / (64 * NW);  // x chunks per thread per stage
    static_assert(XL >= 1 && XL * 64 * NW == MT * KW, "x window must split evenly over the waves");
    constexpr int E = NW * T * 4 * 64;         // partial values of a tile
    extern __shared__ u32x4 sm[];              // [NW][16][PITCH] then [2][MT][PITCH]
    __shared__ unsigned last_flag[2];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const unsigned G = gridDim.x, gi = blockIdx.x;
    const unsigned spt = (unsigned)a.sk_spt;
    const unsigned units = (unsigned)a.n_tiles * spt;
    const unsigned u0 = (unsigned)(((unsigned long long)gi * units) / G);
    const unsigned u1 = (unsigned)(((unsigned long long)(gi + 1) * units) / G);
    const int count = (int)(u1 - u0);
    const unsigned row_bytes = a.w_pitch, x_pitch = a.x_pitch;
    const auto xres = make_rsrc(a.x, (unsigned)a.M * x_pitch);
    u32x4 *wl = sm + wave * 16 * PITCH;
    u32x4 *xl = sm + NW * 16 * PITCH;
    const int wrow = lane >> 5, wcol = lane & 31;
    const int i16 = lane & 15, g = lane >> 4;
    // tile t is the row range [t N / n_tiles, (t + 1) N / n_tiles), at most
    // 16 NW rows; wave w multiplies its rows 16 w .. 16 w + 15
    auto tile_row = [&](unsigned t) {
        return skinny::tile_row(a, (int)t);
    };

    // loads: stage j of the range is unit u0 + j
    unsigned ld_tile = u0 / spt, ld_step = u0 - ld_tile * spt;
    int issued = 0;
    auto load = [&](u32x4(&wv)[8], u32x4(&xv)[XL]) {
        const bool live = issued++ < count;
        const int n0 = tile_row(ld_tile) + wave * 16;
        const int rows_valid = uniform_int(live ? max(0, min(16, tile_row(ld_tile + 1) - n0)) : 0);
        const auto wres = make_rsrc(static_cast<const char *>(a.W) + (size_t)(rows_valid ? n0 : 0) * row_bytes,
                                    (unsigned)rows_valid * row_bytes);
        const int cbase = (int)ld_step * KW;
        const int lim = live ? a.K8 : 0;
        const int c = cbase + wcol;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            wv[q] = load_w(wres, lane_off(c < lim, (unsigned)(2 * q + wrow) * row_bytes + (unsigned)c * 16u), 0);
#pragma unroll
        for (int i = 0; i < XL; ++i) {
            const int e = tid + 64 * NW * i;
            const int tok = e / KW, cc = cbase + (e % KW);
            xv[i] = load_x(xres, lane_off(cc < lim, (unsigned)tok * x_pitch + (unsigned)cc * 16u), 0);
        }
        const bool wrap = ld_step + 1 == spt;
        ld_step = wrap ? 0u : ld_step + 1;
        ld_tile = wrap ? ld_tile + 1 : ld_tile;
    };

    f32x4 acc[T], acc_first[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc_first[t] = acc[t];
    }
    unsigned c_tile = ld_tile, c_step = ld_step;   // the unit multiplied next
    bool seg_whole_start = c_step == 0;            // current segment starts at stage 0
    int first_cut = -1;                            // cut tile met first, partial in acc_first

    auto store_tile = [&](int tile, const f32x4(&v)[T]) {
        const int n0 = tile_row((unsigned)tile) + wave * 16, n_end = tile_row((unsigned)tile + 1);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int tok = 16 * t + i16;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + 4 * g + q;
                if (tok < a.M && n < n_end)
                    store_out(a, tok, n, v[t][q]);
            }
        }
    };
    auto publish = [&](int tile, const f32x4(&v)[T]) {
        const int part = (int)gi - sk_owner((unsigned)tile * spt, units, G);
        float *wsp = a.ws + ((long)tile * a.sk_parts + part) * E;
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                publish_partial(wsp + ((wave * T + t) * 4 + q) * 64 + lane, v[t][q]);
    };

    auto stage = [&](u32x4(&wv)[8], u32x4(&xv)[XL], int j) {
        u32x4 *xw = xl + (j & 1) * MT * PITCH;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            wl[(2 * q + wrow) * PITCH + wcol] = wv[q];
#pragma unroll
        for (int i = 0; i < XL; ++i) {
            const int e = tid + 64 * NW * i;
            xw[(e / KW) * PITCH + (e % KW)] = xv[i];
        }
        load(wv, xv);                          // stage j + U (past the range: no memory access)
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        if (j >= count)
            return;
        // fragments are read four K-steps at a time, so one LDS round trip
        // feeds 4 T MFMAs
#pragma unroll
        for (int h = 0; h < KW / 16; ++h) {
            u32x4 av[4], bv[4][T];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                av[s] = wl[i16 * PITCH + 4 * (4 * h + s) + g];
#pragma unroll
                for (int t = 0; t < T; ++t)
                    bv[s][t] = xw[(16 * t + i16) * PITCH + 4 * (4 * h + s) + g];
            }
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int t = 0; t < T; ++t)
                    acc[t] = mma16<H>(av[s], bv[s][t], acc[t]);
        }
        // a segment ends at its tile's last stage or at the range's last
        // stage; the segment of the range's last stage is handled after the
        // loop
        if (j < count - 1 && c_step == spt - 1) {
            if (seg_whole_start) {
                store_tile((int)c_tile, acc);
            } else {                           // the range's first segment, cut
                first_cut = (int)c_tile;
#pragma unroll
                for (int t = 0; t < T; ++t)
                    acc_first[t] = acc[t];
            }
#pragma unroll
            for (int t = 0; t < T; ++t)
                acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            seg_whole_start = true;
        }
        if (j < count - 1) {
            const bool wrap = c_step + 1 == spt;
            c_step = wrap ? 0u : c_step + 1;
            c_tile = wrap ? c_tile + 1 : c_tile;
        }
    };

    // the prologue loads stay in stage order (sched_barrier), so that the
    // loads of the stage multiplied first are the oldest in flight
    u32x4 w0[8], x0[XL], w1[8], x1[XL], w2[8], x2[XL], w3[8], x3[XL];
    load(w0, x0);
    __builtin_amdgcn_sched_barrier(0);
    load(w1, x1);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (U >= 3) {
        load(w2, x2);
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (U >= 4) {
        load(w3, x3);
        __builtin_amdgcn_sched_barrier(0);
    }
    // Whole rounds of U stages, the stages past `count` idle: an exit from
    // the middle of a round would give the loop a path on which the newest
    // loads are not the ones the next round waits for, and every round would
    // then wait for all of its loads.
    for (int j = 0; j < count; j += U) {
        stage(w0, x0, j);
        stage(w1, x1, j + 1);
        if constexpr (U >= 3)
            stage(w2, x2, j + 2);
        if constexpr (U >= 4)
            stage(w3, x3, j + 3);
    }

    // The last segment (c_tile, stages up to c_step) is whole if it started
    // at stage 0 and reached the tile's last stage.
    const bool last_whole = seg_whole_start && c_step == spt - 1;
    const int last_cut = last_whole ? -1 : (int)c_tile;
    if (first_cut >= 0)
        publish(first_cut, acc_first);
    if (last_cut >= 0)
        publish(last_cut, acc);
    __syncthreads();                           // every wave has issued its partial stores
    auto arrive = [&](int t) -> unsigned {
        if (t < 0)
            return 0u;
        const int parts = sk_owner((unsigned)(t + 1) * spt - 1, units, G) - sk_owner((unsigned)t * spt, units, G) + 1;
        const unsigned prev = __hip_atomic_fetch_add(a.ctr + t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return prev == (unsigned)(parts - 1) ? (unsigned)parts : 0u;
    };
    if (tid == 0) {
        last_flag[0] = arrive(first_cut);
        last_flag[1] = arrive(last_cut);
    }
    if (last_whole)
        store_tile((int)c_tile, acc);
    __syncthreads();
    auto finalize = [&](int t, int parts) {
        if (!parts)
            return;
        finalize_mfma_tile<T, NW>(a, a.ws + (long)t * a.sk_parts * E, E, parts, tile_row((unsigned)t),
                                  tile_row((unsigned)t + 1));
        if (tid == 0)
            __hip_atomic_store(a.ctr + t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    finalize(first_cut, (int)last_flag[0]);
    finalize(last_cut, (int)last_flag[1]);
}

// ---------------------------------------------------------------------------
// MFMAK kernel: token tile MT = 16 T; a workgroup owns one row range of at
// most 16 RT rows and the whole of K, with RT x KS waves: wave (rt, ks)
// multiplies rows 16 rt .. 16 rt + 15 of the range over every KS-th K stage
// starting at stage ks, and the KS partial sums of a row group are added in
// LDS at the end (in ks order), so no partial sum leaves the workgroup.
//
// The grid has n_tiles = max(ceil(N / 16 RT), split x CUs) equal row ranges
// [t N / n_tiles, (t + 1) N / n_tiles): with N / 16 RT below the CU count
// every CU gets the same number of rows (6288 rows: 24 or 25 per CU), which
// 16-row MFMA tiles alone cannot do without sharing tiles between
// workgroups.  The weight path is MFMAS's: row-contiguous loads U iterations
// ahead in registers, re-laid out through a wave-private LDS tile; the x
// window of an iteration covers KS stages, [MT tokens][32 KS chunks], loaded
// by the whole workgroup into a double-buffered LDS tile.
// ---------------------------------------------------------------------------
template <int T, int RT, int KS, int U, bool H>
__global__ __launch_bounds__(512) void k_mfmak(KArgs a)
{
    constexpr int MT = 16 * T;
    constexpr int NW = RT * KS;
    constexpr int KW = kMfmaxChunks;           // chunks per wave per iteration
    constexpr int PITCH = KW + 2;
    constexpr int XW = KS * KW;                // x window width, chunks
    constexpr int XP = XW + 2;                 // its row pitch, 2 mod 4 chunks (see k_mfmax)
    constexpr int XL = (MT * XW) / (64 * NW);  // x chunks per thread per iteration
    static_assert(XL >= 1 && XL * 64 * NW == MT * XW, "x window must split evenly over the waves");
    static_assert(U >= 2 && U <= 4, "two to four iterations in flight");
    extern __shared__ u32x4 sm[];              // [NW][16][PITCH] then [2][MT][XP]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rt = wave % RT, ks = wave / RT;
    const unsigned tile = blockIdx.x;
    const int r0 = tile_row(a, (int)tile);
    const int r1 = tile_row(a, (int)tile + 1);
    const int n0 = r0 + 16 * rt;
    const int rows_valid = uniform_int(max(0, min(16, r1 - n0)));
    const unsigned row_bytes = a.w_pitch, x_pitch = a.x_pitch;
    const auto wres = make_rsrc(static_cast<const char *>(a.W) + (size_t)(rows_valid ? n0 : 0) * row_bytes,
                                (unsigned)rows_valid * row_bytes);
    const auto xres = make_rsrc(a.x, (unsigned)a.M * x_pitch);
    const int iters = (a.K8 + XW - 1) / XW;
    u32x4 *wl = sm + wave * 16 * PITCH;
    u32x4 *xl = sm + NW * 16 * PITCH;
    const int wrow = lane >> 5, wcol = lane & 31;
    const int i16 = lane & 15, g = lane >> 4;

    int issued = 0;
    auto load = [&](u32x4(&wv)[8], u32x4(&xv)[XL]) {
        const int j = issued++;
        const int lim = j < iters ? a.K8 : 0;
        const int c = j * XW + ks * KW + wcol;     // this lane's weight chunk
#pragma unroll
        for (int q = 0; q < 8; ++q)
            wv[q] = load_w(wres, lane_off(c < lim, (unsigned)(2 * q + wrow) * row_bytes + (unsigned)c * 16u), 0);
#pragma unroll
        for (int i = 0; i < XL; ++i) {
            const int e = tid + 64 * NW * i;
            const int tok = e / XW, cc = j * XW + (e % XW);
            xv[i] = load_x(xres, lane_off(cc < lim, (unsigned)tok * x_pitch + (unsigned)cc * 16u), 0);
        }
    };

    f32x4 acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t)
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto stage = [&](u32x4(&wv)[8], u32x4(&xv)[XL], int j) {
        u32x4 *xw = xl + (j & 1) * MT * XP;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            wl[(2 * q + wrow) * PITCH + wcol] = wv[q];
#pragma unroll
        for (int i = 0; i < XL; ++i) {
            const int e = tid + 64 * NW * i;
            xw[(e / XW) * XP + (e % XW)] = xv[i];
        }
        load(wv, xv);                          // iteration j + U (past the end: no memory access)
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        if (j >= iters)
            return;
#pragma unroll
        for (int h = 0; h < KW / 16; ++h) {
            u32x4 av[4], bv[4][T];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                av[s] = wl[i16 * PITCH + 4 * (4 * h + s) + g];
#pragma unroll
                for (int t = 0; t < T; ++t)
                    bv[s][t] = xw[(16 * t + i16) * XP + ks * KW + 4 * (4 * h + s) + g];
            }
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int t = 0; t < T; ++t)
                    acc[t] = mma16<H>(av[s], bv[s][t], acc[t]);
        }
    };

    u32x4 w0[8], x0[XL], w1[8], x1[XL], w2[8], x2[XL], w3[8], x3[XL];
    load(w0, x0);
    __builtin_amdgcn_sched_barrier(0);
    load(w1, x1);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (U >= 3) {
        load(w2, x2);
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (U >= 4) {
        load(w3, x3);
        __builtin_amdgcn_sched_barrier(0);
    }
    // whole rounds of U iterations (see the MFMAS kernel)
    for (int j = 0; j < iters; j += U) {
        stage(w0, x0, j);
        stage(w1, x1, j + 1);
        if constexpr (U >= 3)
            stage(w2, x2, j + 2);
        if constexpr (U >= 4)
            stage(w3, x3, j + 3);
    }

    // add the KS partial sums of each row group, in ks order, through LDS
    // (the tiles are free: every wave is past its last fragment read)
    float *red = reinterpret_cast<float *>(sm);
    __syncthreads();
    if constexpr (KS > 1) {
        if (ks > 0) {
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    red[((wave * T + t) * 4 + q) * 64 + lane] = acc[t][q];
        }
        __syncthreads();
        if (ks > 0)
            return;
#pragma unroll
        for (int s = 1; s < KS; ++s)
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    acc[t][q] += red[(((s * RT + rt) * T + t) * 4 + q) * 64 + lane];
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const int tok = 16 * t + i16;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int n = n0 + 4 * g + q;
            if (tok < a.M && n < r1)
                store_out(a, tok, n, acc[t][q]);
        }
    }
}

// ---------------------------------------------------------------------------
// MFMAW kernel: token tile MT = 16 T; a workgroup owns one equal row range of
// at most 16 RG rows and one K part (of `split`), with NW waves that each
// multiply EVERY row group of the range over every NW-th K stage of SC = 8 or
// 16 chunks (SC / 4 MFMA K-steps).  No wave waits for another until the end:
//
//  * the weight and the x of a stage are loaded row-contiguously -- each
//    wave-wide load is 64 / SC rows (or tokens) x 16 SC bytes -- two stages
//    ahead in registers, and re-laid out through the wave's own LDS tiles
//    [16 RG][SC + 2] and [MT][SC + 2] (chunks) into A and B fragments.  The
//    stage width sets the bytes a wave keeps in flight.  A stage's weight
//    registers are refilled as soon as they are in LDS, its x registers only
//    after its MFMAs: x comes from L2, and issuing it with the weight (or
//    three stages ahead) measured slower;
//  * each B fragment feeds the MFMAs of all RG row groups, and the waves take
//    disjoint K stages, so x is read once per workgroup and K stage however
//    many rows the range has, with no x shared between waves;
//  * the NW partial sums are added in LDS once, in wave order, after the
//    stream; with split > 1 the sum goes through the split-K exchange.
//
// A and B take the same chunk (4 st + g) for K-group g of K-step st, so every
// product W[n][k] x[m][k] is formed exactly once.  Row pitch SC + 2 chunks (2
// mod 4): the fragment reads of 16 rows of one column are conflict-free (see
// k_mfmax).  Unlike MFMAX, whose waves share each x window and meet at a
// barrier every two stages, no wave here waits on another's loads.
// ---------------------------------------------------------------------------
template <int T, int RG, int NW, int SC, bool H>
__global__ __launch_bounds__(64 * NW) void k_mfmaw(KArgs a)
{
    static_assert(SC == 8 || SC == 16, "stages of 8 or 16 chunks");
    constexpr int RPL = 64 / SC;               // rows (tokens) per wave-wide load
    constexpr int NL = 16 / RPL;               // loads per 16 rows (tokens)
    constexpr int KS = SC / 4;                 // MFMA K-steps per stage
    constexpr int PITCH = SC + 2;
    constexpr int ROWS = 16 * RG;
    constexpr int MT = 16 * T;
    constexpr int E = RG * T * 4 * 64;         // partial values of one wave (and of the workgroup)
    constexpr int EPT = E / (64 * NW);         // of them per thread in the final sum
    static_assert(EPT >= 1 && EPT * 64 * NW == E, "the final sum must split evenly over the threads");
    static_assert(E * 4 <= (ROWS + MT) * PITCH * 16, "the wave's LDS tiles must hold its partial sums");
    extern __shared__ u32x4 sm[];              // [NW][ROWS + MT][PITCH]; at the end float [NW][E]
    __shared__ unsigned flag;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tile, s;
    block_coords(a, tile, s);
    const int n_wg = tile_row(a, tile), n_end = tile_row(a, tile + 1);
    const int kb = split_point(a, s, a.K8);
    const int ke = split_point(a, s + 1, a.K8);
    const int stages = (ke - kb + SC - 1) / SC;
    const int mine = stages > wave ? (stages - wave + NW - 1) / NW : 0;   // stages wave, wave + NW, ...
    const unsigned row_bytes = a.w_pitch, x_pitch = a.x_pitch;
    const int rows_valid = uniform_int(max(0, min(ROWS, n_end - n_wg)));
    const auto wres = make_rsrc(static_cast<const char *>(a.W) + (size_t)(rows_valid ? n_wg : 0) * row_bytes,
                                (unsigned)rows_valid * row_bytes);
    const auto xres = make_rsrc(a.x, (unsigned)a.M * x_pitch);
    u32x4 *wl = sm + wave * (ROWS + MT) * PITCH;
    u32x4 *xl = wl + ROWS * PITCH;
    const int i16 = lane & 15, g = lane >> 4;
    const int lr = lane / SC, lc = lane % SC;  // row within a load, chunk within the stage

    f32x4 acc[RG][T];
#pragma unroll
    for (int r = 0; r < RG; ++r)
#pragma unroll
        for (int t = 0; t < T; ++t)
            acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Load q of a stage covers weight rows RPL q + lr (x: tokens RPL q + lr),
    // chunk lc of the wave's j-th stage; past the wave's last stage, or past
    // the end of its K part, the offset is out of range and nothing is read.
    const auto lane_chunk = [&](int j, unsigned &off) {
        const int c = kb + (wave + NW * j) * SC + lc;
        off = (unsigned)c * 16u;
        return j < mine && c < ke;
    };
    auto load_wt = [&](u32x4(&wv)[NL * RG], int j) {
        unsigned co;
        const bool ok = lane_chunk(j, co);
#pragma unroll
        for (int q = 0; q < NL * RG; ++q)
            wv[q] = load_w(wres, lane_off(ok, (unsigned)(RPL * q + lr) * row_bytes + co), 0);
    };
    auto load_xt = [&](u32x4(&xv)[NL * T], int j) {
        unsigned co;
        const bool ok = lane_chunk(j, co);
#pragma unroll
        for (int q = 0; q < NL * T; ++q)
            xv[q] = load_x(xres, lane_off(ok, (unsigned)(RPL * q + lr) * x_pitch + co), 0);
    };
    // Stage j.  The tiles are rewritten by the next stage only after these
    // fragment reads, in the wave's own program order.
    auto step = [&](u32x4(&wv)[NL * RG], u32x4(&xv)[NL * T], int j) {
#pragma unroll
        for (int q = 0; q < NL * RG; ++q)
            wl[(RPL * q + lr) * PITCH + lc] = wv[q];
        load_wt(wv, j + 2);
        __builtin_amdgcn_sched_barrier(0);
        if (j < mine) {
#pragma unroll
            for (int q = 0; q < NL * T; ++q)
                xl[(RPL * q + lr) * PITCH + lc] = xv[q];
            u32x4 bv[KS][T];
#pragma unroll
            for (int st = 0; st < KS; ++st)
#pragma unroll
                for (int t = 0; t < T; ++t)
                    bv[st][t] = xl[(16 * t + i16) * PITCH + 4 * st + g];
#pragma unroll
            for (int r = 0; r < RG; ++r) {
                u32x4 av[KS];
#pragma unroll
                for (int st = 0; st < KS; ++st)
                    av[st] = wl[(16 * r + i16) * PITCH + 4 * st + g];
#pragma unroll
                for (int st = 0; st < KS; ++st)
#pragma unroll
                    for (int t = 0; t < T; ++t)
                        acc[r][t] = mma16<H>(av[st], bv[st][t], acc[r][t]);
            }
        }
        load_xt(xv, j + 2);
        __builtin_amdgcn_sched_barrier(0);
    };

    // Two stages in flight; every pass issues all of its loads (past the
    // wave's last stage they touch no memory), so the waits stay partial.
    u32x4 wa[NL * RG], xa[NL * T], wb[NL * RG], xb[NL * T];
    load_wt(wa, 0);
    load_xt(xa, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_wt(wb, 1);
    load_xt(xb, 1);
    __builtin_amdgcn_sched_barrier(0);
    for (int j = 0; j < mine; j += 2) {
        step(wa, xa, j);
        step(wb, xb, j + 1);
    }

    // add the NW partial sums in wave order: value e = ((r T + t) 4 + q) 64 + lane
    float *red = reinterpret_cast<float *>(sm);
    __syncthreads();                           // every wave is past its last fragment read
#pragma unroll
    for (int r = 0; r < RG; ++r)
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                red[wave * E + ((r * T + t) * 4 + q) * 64 + lane] = acc[r][t][q];
    __syncthreads();
    float v[EPT];
    int off[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        off[i] = tid + 64 * NW * i;
        v[i] = red[off[i]];
#pragma unroll
        for (int w = 1; w < NW; ++w)
            v[i] += red[w * E + off[i]];
    }
    // value e: token 16 t + (e % 16), row n_wg + 16 r + 4 ((e / 16) % 4) + q
    auto store_all = [&](const float(&vals)[EPT]) {
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int e = off[i], ln = e & 63, q = (e >> 6) & 3, rt = e >> 8;
            const int r = rt / T, t = rt - (rt / T) * T;
            const int tok = 16 * t + (ln & 15), n = n_wg + 16 * r + 4 * (ln >> 4) + q;
            if (tok < a.M && n < n_end)
                store_out(a, tok, n, vals[i]);
        }
    };
    if (a.split == 1) {
        store_all(v);
        return;
    }
    float *wsp = a.ws + (long)tile * a.split * E;
#pragma unroll
    for (int i = 0; i < EPT; ++i)
        publish_partial(wsp + (long)s * E + off[i], v[i]);
    if (!split_arrive_last(a, tile, &flag))
        return;
    float sum[EPT];
    sum_partials<EPT>(wsp, E, a.split, off, sum);
    store_all(sum);
    split_reset(a, tile);
}

// ---------------------------------------------------------------------------
// Measurement probes: a plain streaming read of a buffer (what the weight
// stream could reach with no arithmetic around it) and an empty launch.
// ---------------------------------------------------------------------------
// Each one-wave workgroup streams one 4 KiB span with its four 1 KiB loads in
// flight at once -- the fastest plain-read shape measured on this chip.
__global__ __launch_bounds__(64) void k_probe_read(const u32x4 *buf, long chunks, float *sink)
{
    const long base = (long)blockIdx.x * 256;          // 256 chunks = 4 KiB per workgroup
    const int lane = threadIdx.x;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    u32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const long c = base + i * 64 + lane;
        v[i] = c < chunks ? load_stream(buf + c) : zero;
    }
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const unsigned int a0 = v[i].x, a3 = v[i].w;
        acc += __uint_as_float(a0 ^ a3);
    }
    for (int off = 32; off > 0; off >>= 1)
        acc += __shfl_xor(acc, off);
    if (lane == 0)
        sink[blockIdx.x & (kProbeSinkFloats - 1)] = acc;
}

__global__ void k_probe_empty() {}

const void *probe_read_fn() { return (const void *)&k_probe_read; }
const void *probe_empty_fn() { return (const void *)&k_probe_empty; }

// ---------------------------------------------------------------------------
// Instance table
// ---------------------------------------------------------------------------

// Every instance is compiled for BF16 (half = 0) and FP16 (half = 1) inputs.
#define SK_PAIR(PATH, MT, ROWS, U, KERNEL, ...)                                                        \
    {PATH, MT, ROWS, U, 0, (const void *)&KERNEL<__VA_ARGS__, false>},                               \
        {PATH, MT, ROWS, U, 1, (const void *)&KERNEL<__VA_ARGS__, true>}
#define SK_DOT2(MT, R, U) SK_PAIR(SKINNY_PATH_DOT2, MT, R, U, k_dot2, MT, R, U)
#define SK_MFMA(T, RT, U) SK_PAIR(SKINNY_PATH_MFMA, 16 * T, 16 * RT, U, k_mfma, T, RT, U)
#define SK_DOT2X(MT, R, U) SK_PAIR(SKINNY_PATH_DOT2X, MT, R, U, k_dot2x, MT, R, U)
#define SK_MFMAX(T, NW) SK_PAIR(SKINNY_PATH_MFMAX, 16 * T, NW, 1, k_mfmax, T, NW)
#define SK_MFMAD(T, NW, D) SK_PAIR(SKINNY_PATH_MFMAD, 16 * T, NW, D, k_mfmad, T, NW, D)
#define SK_MFMAS(T, NW, D) SK_PAIR(SKINNY_PATH_MFMAS, 16 * T, NW, D, k_mfmas, T, NW, D)
// MFMAK: rows field = 100 * KS + RT (row groups and K groups), unroll = iterations in flight
#define SK_MFMAK(T, RT, KS, U) SK_PAIR(SKINNY_PATH_MFMAK, 16 * T, 100 * KS + RT, U, k_mfmak, T, RT, KS, U)
// MFMAW: rows field = 100 * NW + RG (waves and row groups), unroll = stage
// width in 8-chunk units (1: 8 chunks, 2: 16)
#define SK_MFMAW(T, RG, NW, U) SK_PAIR(SKINNY_PATH_MFMAW, 16 * T, 100 * NW + RG, U, k_mfmaw, T, RG, NW, 8 * U)

// Instances whose double-buffered loads, accumulators and offsets fit in 256
// VGPRs without spilling (roughly 8 U (R + MT) + R MT registers).
static const KernelInfo kKernels[] = {
    SK_DOT2(1, 1, 1), SK_DOT2(1, 1, 2), SK_DOT2(1, 1, 4),
    SK_DOT2(1, 2, 1), SK_DOT2(1, 2, 2), SK_DOT2(1, 2, 4),
    SK_DOT2(1, 4, 1), SK_DOT2(1, 4, 2), SK_DOT2(1, 4, 4),
    SK_DOT2(1, 8, 1), SK_DOT2(1, 8, 2),
    SK_DOT2(1, 16, 1),
    SK_DOT2(2, 1, 1), SK_DOT2(2, 1, 2), SK_DOT2(2, 1, 4),
    SK_DOT2(2, 2, 1), SK_DOT2(2, 2, 2), SK_DOT2(2, 2, 4),
    SK_DOT2(2, 4, 1), SK_DOT2(2, 4, 2),
    SK_DOT2(2, 8, 1),
    SK_DOT2(4, 1, 1), SK_DOT2(4, 1, 2), SK_DOT2(4, 1, 4),
    SK_DOT2(4, 2, 1), SK_DOT2(4, 2, 2),
    SK_DOT2(4, 4, 1), SK_DOT2(4, 4, 2),
    SK_DOT2(4, 8, 1),
    SK_DOT2(8, 1, 1), SK_DOT2(8, 1, 2),
    SK_DOT2(8, 2, 1),
    SK_DOT2(8, 4, 1),
    SK_MFMA(1, 1, 1), SK_MFMA(1, 1, 2), SK_MFMA(1, 1, 4),
    SK_MFMA(1, 2, 1), SK_MFMA(1, 2, 2), SK_MFMA(1, 2, 4),
    SK_MFMA(1, 4, 1), SK_MFMA(1, 4, 2),
    SK_MFMA(2, 1, 1), SK_MFMA(2, 1, 2), SK_MFMA(2, 1, 4),
    SK_MFMA(2, 2, 1), SK_MFMA(2, 2, 2), SK_MFMA(2, 2, 4),
    SK_MFMA(2, 4, 1), SK_MFMA(2, 4, 2),
    SK_MFMA(4, 1, 1), SK_MFMA(4, 1, 2),
    SK_MFMA(4, 2, 1), SK_MFMA(4, 2, 2),
    // DOT2X: rows field = rows per wave
    SK_DOT2X(1, 1, 2), SK_DOT2X(1, 1, 4), SK_DOT2X(1, 2, 2), SK_DOT2X(1, 2, 4), SK_DOT2X(1, 4, 2),
    SK_DOT2X(2, 1, 2), SK_DOT2X(2, 1, 4), SK_DOT2X(2, 2, 2), SK_DOT2X(2, 2, 4), SK_DOT2X(2, 4, 2),
    SK_DOT2X(4, 1, 2), SK_DOT2X(4, 1, 4), SK_DOT2X(4, 2, 2), SK_DOT2X(4, 2, 4), SK_DOT2X(4, 4, 2),
    SK_DOT2X(8, 1, 2), SK_DOT2X(8, 1, 4), SK_DOT2X(8, 2, 2), SK_DOT2X(8, 2, 4), SK_DOT2X(8, 4, 2),
    // MFMAX: rows field = waves (16 rows each)
    SK_MFMAX(1, 1), SK_MFMAX(1, 2), SK_MFMAX(1, 4), SK_MFMAX(1, 8),
    SK_MFMAX(2, 2), SK_MFMAX(2, 4), SK_MFMAX(2, 8),
    SK_MFMAX(4, 4), SK_MFMAX(4, 8),
    // MFMAD: rows field = waves (16 rows each), unroll field = pipeline depth
    SK_MFMAD(1, 2, 4), SK_MFMAD(1, 4, 3), SK_MFMAD(1, 8, 2),
    SK_MFMAD(2, 2, 4), SK_MFMAD(2, 4, 2), SK_MFMAD(2, 4, 3),
    SK_MFMAD(4, 2, 3), SK_MFMAD(4, 4, 2),
    // MFMAS: rows field = waves, unroll field = pipeline depth; stream-K grid
    SK_MFMAS(1, 2, 3), SK_MFMAS(1, 4, 2), SK_MFMAS(1, 4, 3), SK_MFMAS(1, 4, 4), SK_MFMAS(1, 8, 2),
    SK_MFMAS(2, 4, 2), SK_MFMAS(2, 4, 3), SK_MFMAS(2, 8, 2),
    SK_MFMAK(1, 1, 4, 2), SK_MFMAK(1, 2, 2, 2), SK_MFMAK(1, 2, 2, 3), SK_MFMAK(1, 2, 4, 2), SK_MFMAK(1, 2, 4, 3),
    SK_MFMAK(2, 2, 2, 2),
    SK_MFMAW(1, 1, 4, 2), SK_MFMAW(1, 2, 1, 2), SK_MFMAW(1, 2, 2, 2), SK_MFMAW(1, 2, 4, 2), SK_MFMAW(1, 4, 4, 2),
    SK_MFMAW(2, 1, 4, 2), SK_MFMAW(2, 2, 1, 2), SK_MFMAW(2, 2, 2, 2), SK_MFMAW(2, 2, 4, 2), SK_MFMAW(2, 2, 8, 2),
    SK_MFMAW(2, 4, 4, 2), SK_MFMAW(4, 1, 4, 2), SK_MFMAW(4, 2, 2, 2), SK_MFMAW(4, 2, 4, 2),
    SK_MFMAW(1, 1, 4, 1), SK_MFMAW(1, 2, 2, 1), SK_MFMAW(1, 2, 4, 1), SK_MFMAW(1, 2, 8, 1), SK_MFMAW(1, 4, 4, 1),
    SK_MFMAW(2, 2, 2, 1), SK_MFMAW(2, 2, 4, 1), SK_MFMAW(2, 2, 8, 1), SK_MFMAW(2, 4, 4, 1),
    SK_MFMAW(4, 2, 2, 1), SK_MFMAW(4, 2, 4, 1),
};

const KernelInfo *kernel_table(int *count)
{
    *count = (int)(sizeof(kKernels) / sizeof(kKernels[0]));
    return kKernels;
}

const KernelInfo *find_kernel(int path, int mt, int rows, int unroll, int half)
{
    for (const KernelInfo &k : kKernels)
        if (k.path == path && k.mt == mt && k.rows == rows && k.unroll == unroll && k.half == half)
            return &k;
    return nullptr;
}

}  // namespace skinny
