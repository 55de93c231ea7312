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
//    through memory with agent-scope release/acquire).
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

// 8-element BF16 dot product accumulated into acc (4 x v_dot2_f32_bf16).
__device__ __forceinline__ float dot8(u32x4 w, u32x4 x, float acc)
{
    const unsigned int w0 = w.x, w1 = w.y, w2 = w.z, w3 = w.w;
    const unsigned int x0 = x.x, x1 = x.y, x2 = x.z, x3 = x.w;
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w0), as_bf16x2(x0), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w1), as_bf16x2(x1), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w2), as_bf16x2(x2), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w3), as_bf16x2(x3), acc, false);
    return acc;
}

// Workgroup -> (row tile, K split).  The dispatcher deals consecutive
// workgroup ids round-robin over the XCDs; with `remap`, ids are renumbered
// so that consecutive logical indices -- the `split` workgroups of one row
// tile -- sit on the same XCD (a bijection of [0, gridDim.x)).
__device__ __forceinline__ void block_coords(const KArgs &a, int &tile, int &s)
{
    int idx = blockIdx.x;
    if (a.remap) {
        const int g = gridDim.x, nx = a.nxcd;
        const int xcd = idx % nx, j = idx / nx;
        const int q = g / nx, r = g % nx;
        idx = xcd * q + (xcd < r ? xcd : r) + j;
    }
    tile = idx / a.split;
    s = idx - tile * a.split;
}

__device__ __forceinline__ void store_out(const KArgs &a, int m, int n, float v)
{
    const long off = (long)m * a.N + n;
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
// Cross-workgroup split-K arrival.  Every thread of the workgroup calls it
// after storing its partials.  Returns true in the workgroup that arrives
// last for this tile; that workgroup then reads all partials.  The counter is
// reset by the last arriver, so it is zero again when the kernel ends.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool split_arrive_last(const KArgs &a, int tile, unsigned *flag_lds)
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");   // own partial stores done, L2 written back
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev =
            __hip_atomic_fetch_add(a.ctr + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag_lds = (prev == (unsigned)(a.split - 1)) ? 1u : 0u;
    }
    __syncthreads();
    const bool last = *flag_lds != 0;
    if (last)
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // see every partial
    return last;
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
template <int MT, int R, int U>
__global__ __launch_bounds__(512) void k_dot2(KArgs a)
{
    constexpr int V = MT * R;   // partial sums per lane, index m * R + r
    __shared__ float red[kMaxWaves][V];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int nthr = blockDim.x, nwaves = nthr >> 6;
    int tile, s;
    block_coords(a, tile, s);
    const int n0 = tile * R;
    const int kb = (int)(((long)s * a.K8) / a.split);
    const int ke = (int)(((long)(s + 1) * a.K8) / a.split);
    const unsigned row_bytes = (unsigned)a.K8 * 16u;
    const int rows_valid = min(R, a.N - n0);
    const auto wres = make_rsrc(static_cast<const char *>(a.W) + (size_t)n0 * row_bytes,
                                (unsigned)rows_valid * row_bytes);
    const auto xres = make_rsrc(a.x, (unsigned)a.M * row_bytes);
    const unsigned lane_off = (unsigned)(kb + tid) * 16u;
    const unsigned pass_bytes = (unsigned)nthr * 16u;

    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i)
        acc[i] = 0.f;

    const int passes = (ke - kb) / nthr;   // passes in which every lane has a chunk
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
                x[u][m] = load_x(xres, (unsigned)m * row_bytes + lane_off, so);
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
                    acc[m * R + r] = dot8(w[u][r], x[u][m], acc[m * R + r]);
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
            x[0][m] = load_x(xres, ok ? (unsigned)m * row_bytes + lane_off : kOffOob, so);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m)
                acc[m * R + r] = dot8(w[0][r], x[0][m], acc[m * R + r]);
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
    const bool live = tid < V && m < a.M && n < a.N;
    if (a.split == 1) {
        if (live)
            store_out(a, m, n, total);
        return;
    }
    // split-K: publish this workgroup's partial, the last arriver finalises
    float *wsp = a.ws + (long)tile * a.split * V;
    if (tid < V)
        wsp[(long)s * V + tid] = total;
    // only wave 0 is left and it holds every partial of the tile, so its own
    // release (wait for its stores, write L2 back) covers the whole partial
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    unsigned prev = 0;
    if (lane == 0)
        prev = __hip_atomic_fetch_add(a.ctr + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev != (unsigned)(a.split - 1))
        return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (live) {
        float sum = 0.f;
        for (int j = 0; j < a.split; ++j)
            sum += __builtin_nontemporal_load(wsp + (long)j * V + tid);
        store_out(a, m, n, sum);
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
template <int T, int RT, int U>
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
    const int sb = (int)(((long)s * steps) / a.split);
    const int se = (int)(((long)(s + 1) * steps) / a.split);
    const int se_full = se < steps_full ? se : steps_full;

    const unsigned row_bytes = (unsigned)a.K8 * 16u;
    const int rows_valid = min(NT, a.N - n0);
    const auto wres = make_rsrc(static_cast<const char *>(a.W) + (size_t)n0 * row_bytes,
                                (unsigned)rows_valid * row_bytes);
    const auto xres = make_rsrc(a.x, (unsigned)a.M * row_bytes);
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
    const int qn = first < se_full ? (se_full - first + nwaves - 1) / nwaves : 0;
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
                bv[u][t] = load_x(xres, (unsigned)(16 * t + i16) * row_bytes + k_off, so);
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
                    acc[rt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, av[u][rt]), __builtin_bit_cast(bf16x8, bv[u][t]),
                        acc[rt][t], 0, 0, 0);
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
            bv[0][t] = load_x(xres, ok ? (unsigned)(16 * t + i16) * row_bytes + k_off : kOffOob, so);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int t = 0; t < T; ++t)
                acc[rt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, av[0][rt]), __builtin_bit_cast(bf16x8, bv[0][t]),
                    acc[rt][t], 0, 0, 0);
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
        wsp[(long)s * E + e] = v;
    }
    if (!split_arrive_last(a, tile, &flag))
        return;
    for (int e = tid; e < E; e += nthr) {
        const int tok = e / NT, row = e - (e / NT) * NT;
        if (tok >= mlim || n0 + row >= a.N)
            continue;
        float v = 0.f;
        for (int j = 0; j < a.split; ++j)
            v += __builtin_nontemporal_load(wsp + (long)j * E + e);
        store_out(a, tok, n0 + row, v);
    }
    split_reset(a, tile);
}

// ---------------------------------------------------------------------------
// Measurement probes: a plain streaming read of a buffer (what the weight
// stream could reach with no arithmetic around it) and an empty launch.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_probe_read(const u32x4 *buf, long chunks, float *sink)
{
    const long stride = (long)gridDim.x * blockDim.x;
    float acc = 0.f;
    long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < chunks; i += 4 * stride) {
        const u32x4 a = load_stream(buf + i), b = load_stream(buf + i + stride);
        const u32x4 c = load_stream(buf + i + 2 * stride), d = load_stream(buf + i + 3 * stride);
        const unsigned int a0 = a.x, b0 = b.y, c0 = c.z, d0 = d.w;
        acc += __uint_as_float(a0 ^ b0) + __uint_as_float(c0 ^ d0);
    }
    for (; i < chunks; i += stride) {
        const u32x4 a = load_stream(buf + i);
        const unsigned int a0 = a.x;
        acc += __uint_as_float(a0);
    }
    __shared__ float part[4];
    for (int off = 32; off > 0; off >>= 1)
        acc += __shfl_xor(acc, off);
    if ((threadIdx.x & 63) == 0)
        part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0)
        sink[blockIdx.x] = part[0] + part[1] + part[2] + part[3];
}

__global__ void k_probe_empty() {}

const void *probe_read_fn() { return (const void *)&k_probe_read; }
const void *probe_empty_fn() { return (const void *)&k_probe_empty; }

// ---------------------------------------------------------------------------
// Instance table
// ---------------------------------------------------------------------------

#define SK_DOT2(MT, R, U) {SKINNY_PATH_DOT2, MT, R, U, (const void *)&k_dot2<MT, R, U>}
#define SK_MFMA(T, RT, U) {SKINNY_PATH_MFMA, 16 * T, 16 * RT, U, (const void *)&k_mfma<T, RT, U>}

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
};

const KernelInfo *kernel_table(int *count)
{
    *count = (int)(sizeof(kKernels) / sizeof(kKernels[0]));
    return kKernels;
}

const KernelInfo *find_kernel(int path, int mt, int rows, int unroll)
{
    for (const KernelInfo &k : kKernels)
        if (k.path == path && k.mt == mt && k.rows == rows && k.unroll == unroll)
            return &k;
    return nullptr;
}

}  // namespace skinny
