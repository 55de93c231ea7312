// HIP kernels of the skinny BF16 decode projection for gfx950 (CDNA4).
//
//   out[m][n] = sum_k x[m][k] * W[n][k]     (m < M <= 64, n < N)
//
// the decode-step product "out[M, N] = x[M, K] @ weight[N, K]^T" of class
// PreparedWarpSplitK on the page "vllm.models.kimi_k3.nvidia.specialized_decode.
// cutedsl.gemm.warp_splitk".  At decode sizes the whole cost is streaming W
// once from HBM, so every kernel is organised around the weight stream:
//
//  * Each lane loads 16 bytes (8 BF16 of one row) per load, with the
//    nontemporal bit, and a wave's load covers whole runs of one or a few
//    rows.  W is touched once and must not evict x or out from L2 -- the role
//    the page's evict_first L2 policy plays there.
//  * Workgroups own few rows (the page's small 16/32-row output tiles that let
//    many blocks co-reside per SM, here equal row ranges sized to the CU
//    count), and split K across their waves: every wave holds fp32 partials
//    of the same outputs over a different K range (the page's four compute
//    warps that each own a K quarter), reduced at the end through DPP / lane
//    swaps inside the wave and LDS across waves.
//  * Optionally `split` workgroups share one row tile along K and exchange
//    their fp32 partials through a workspace (the split-K GEMM of the page
//    "vllm.models.glm5next.nvidia.specialized_decode.gemm", which reduces its
//    split-K partials across a thread-block cluster): here every partial
//    travels inside an agent-scope atomic swap, and whichever part completes
//    a pair adds it (swap_exchange).
//
// DOT2 (token tiles 1..8): v_dot2_f32_bf16, two BF16 products into an fp32
// accumulator per instruction.  MFMA (token tiles 16..64): W rows are the
// 16-row A operand and tokens the 16-column B operand of
// v_mfma_f32_16x16x32_bf16 (the warp split-K page also puts the weight on the
// MMA's row side and the tokens on its column side).  MFMA4 (token tiles
// 4..32): the 16-block v_mfma_f32_4x4x4_16b, whose blocks take sixteen K
// chunks of four rows and four tokens.
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

// A node holds a value v as bits(v) ^ kSlotEmptyBits, so an all-zero node
// (zero-initialised memory, or a node some launch emptied) reads as empty:
// decoding 0 gives the signalling-NaN pattern kSlotEmptyBits, which no fp32
// arithmetic produces.
constexpr unsigned kSlotKey = kSlotEmptyBits;

__device__ __forceinline__ void empty_slot(float *p)
{
    __hip_atomic_store(reinterpret_cast<unsigned *>(p), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Cross-workgroup split-K exchange by atomic swaps.
//
// The `parts` K parts of a row tile meet in a fixed binary tree: at level 0
// parts (0, 1), (2, 3), ... pair up in one node each, an odd part out moves
// up unpaired, and so on until one value is left; a tile has parts - 1 nodes
// of E values, each empty between launches.  A part swaps its value into its
// node with one agent-scope atomic exchange and gets back what was there:
// empty means the partner has not arrived and will carry the pair on, so
// this value is done; anything else is the partner's value, and
// this part empties the node, adds the two and moves up a level.  Whoever
// completes the root holds the whole sum.
//
// Each node adds exactly its two children, and fp32 addition is commutative,
// so the sum is the same bits whatever the arrival order: ((p0 + p1) +
// (p2 + p3)) for four parts.  The value travels inside the atomic itself, so
// nothing is fenced, nothing waits for another workgroup and no counter is
// needed: one memory round trip per level, and a late partner can never be
// missed (the second of two swaps on a node always sees the first).  Every
// node is used by exactly two swaps per launch and left empty, so the next
// launch (graph replays included) finds the workspace as the first did: all
// zero, the state a zeroed allocation and a static device array start in.
// Values no part holds (outputs past N or M) are never swapped, by any part.
// ---------------------------------------------------------------------------
// swaps v into the node and returns what was there, both in the node's
// encoding (bits ^ kSlotKey; 0 = empty)
__device__ __forceinline__ unsigned swap_slot(float *p, float v)
{
    return __hip_atomic_exchange(reinterpret_cast<unsigned *>(p), __float_as_uint(v) ^ kSlotKey, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
}

// v[i] (at value offset off[i] >= 0 of this tile; off[i] < 0: none) is this
// part's partial; on return done[i] says whether this thread now holds the
// whole sum of value i in v[i].  wsp is the tile's node array [parts - 1][E].
template <int N>
__device__ __forceinline__ void swap_exchange(float *wsp, int E, int parts, int part, const int (&off)[N],
                                              float (&v)[N], bool (&done)[N])
{
    bool live[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        live[i] = off[i] >= 0;
        done[i] = false;
    }
    int pos = part, n = parts, node0 = 0;
    while (n > 1) {
        const int pairs = n >> 1;
        if (pos < 2 * pairs) {
            float *node = wsp + (long)(node0 + (pos >> 1)) * E;
            unsigned old[N];
            // all swaps of the level in flight before the first is looked at
#pragma unroll
            for (int i = 0; i < N; ++i)
                old[i] = live[i] ? swap_slot(node + off[i], v[i]) : 0u;
#pragma unroll
            for (int i = 0; i < N; ++i) {
                if (!live[i])
                    continue;
                if (old[i] == 0u) {
                    live[i] = false;           // the partner carries the pair on
                } else {
                    empty_slot(node + off[i]);
                    v[i] += __uint_as_float(old[i] ^ kSlotKey);
                }
            }
        }
        node0 += pairs;
        pos >>= 1;
        n = (n + 1) >> 1;
    }
#pragma unroll
    for (int i = 0; i < N; ++i)
        done[i] = live[i];
}

// The same exchange on value pairs: values 2p and 2p + 1 of a thread travel
// in one 64-bit swap, halving the atomics.  Pair p sits at the 64-bit slot
// pair_off[p] of every node (E / 2 slots); a pair is swapped when either of
// its values is live in this tile -- the same pairs in every K part -- and a
// value that is not live just rides along.
constexpr unsigned long long kPairKey = ((unsigned long long)kSlotKey << 32) | kSlotKey;

template <int N>
__device__ __forceinline__ void swap_exchange_pairs(float *wsp, int E, int parts, int part, const int (&off)[N],
                                                    const int (&pair_off)[N / 2], float (&v)[N], bool (&done)[N])
{
    static_assert(N % 2 == 0, "values go in pairs");
    bool live[N / 2];
#pragma unroll
    for (int p = 0; p < N / 2; ++p)
        live[p] = off[2 * p] >= 0 || off[2 * p + 1] >= 0;
    int pos = part, n = parts, node0 = 0;
    while (n > 1) {
        const int pairs = n >> 1;
        if (pos < 2 * pairs) {
            unsigned long long *node =
                reinterpret_cast<unsigned long long *>(wsp + (long)(node0 + (pos >> 1)) * E);
            unsigned long long old[N / 2];
#pragma unroll
            for (int p = 0; p < N / 2; ++p) {
                const unsigned long long mine = (((unsigned long long)__float_as_uint(v[2 * p + 1]) << 32) |
                                                 __float_as_uint(v[2 * p])) ^ kPairKey;
                old[p] = live[p] ? __hip_atomic_exchange(node + pair_off[p], mine, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT)
                                 : 0ull;
            }
#pragma unroll
            for (int p = 0; p < N / 2; ++p) {
                if (!live[p])
                    continue;
                if (old[p] == 0ull) {
                    live[p] = false;           // the partner carries the pair on
                } else {
                    __hip_atomic_store(node + pair_off[p], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    const unsigned long long theirs = old[p] ^ kPairKey;
                    v[2 * p] += __uint_as_float((unsigned)theirs);
                    v[2 * p + 1] += __uint_as_float((unsigned)(theirs >> 32));
                }
            }
        }
        node0 += pairs;
        pos >>= 1;
        n = (n + 1) >> 1;
    }
#pragma unroll
    for (int i = 0; i < N; ++i)
        done[i] = off[i] >= 0 && live[i / 2];
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
    // split-K: wave 0 holds the workgroup's whole partial; it meets the other
    // K parts' in the swap exchange, and whoever completes a value stores it
    const int off[1] = {live ? tid : -1};
    float sum[1] = {total};
    bool done[1];
    swap_exchange<1>(a.ws + (long)tile * (a.split - 1) * V, V, a.split, s, off, sum, done);
    if (done[0])
        store_out(a, m, n, sum[0]);
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
//
// Token groups (MFMAT): a launch with gridDim.y = ceil(M / MT) gives
// workgroup row y tokens MT y .. MT y + MT - 1; each row tile is then
// multiplied once per group, which re-reads the tile from L2 but gives a
// short-K weight, whose row tiles alone cannot fill the chip, as many
// workgroups as groups times tiles.  Plain launches have gridDim.y = 1.
// ---------------------------------------------------------------------------
template <int T, int RT, int U, bool H>
__global__ __launch_bounds__(512) void k_mfma(KArgs a)
{
    constexpr int MT = 16 * T, NT = 16 * RT, NTP = NT + 1;
    extern __shared__ float lds[];   // [waves][MT][NTP]

    const int group = blockIdx.y;
    if (group > 0) {                 // the launch covers M, so M > MT group here
        const int m0 = MT * group;
        const size_t osz = a.out_f32 ? 4 : 2;
        a.x = static_cast<const char *>(a.x) + (size_t)m0 * a.x_pitch;
        a.out = static_cast<char *>(a.out) + (size_t)m0 * a.ldo * osz;
        if (a.res)
            a.res = static_cast<const char *>(a.res) + (size_t)m0 * a.ldr * osz;
        a.M -= m0;
    }
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
    // each token group's row tiles have nodes of their own
    float *wsp = a.ws + ((long)group * a.n_tiles + tile) * (a.split - 1) * E;
    for (int e0 = tid; e0 < E; e0 += 4 * nthr) {
        int off[4];
        float v[4];
        bool done[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {             // the values every K part holds
            const int e = e0 + i * nthr;
            const int tok = e / NT, row = e - (e / NT) * NT;
            const bool live = e < E && tok < mlim && n0 + row < a.N;
            off[i] = live ? e : -1;
            v[i] = 0.f;
            if (live)
                for (int w = 0; w < nwaves; ++w)
                    v[i] += lds[((long)w * MT + tok) * NTP + row];
        }
        swap_exchange<4>(wsp, E, a.split, s, off, v, done);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = e0 + i * nthr;
            if (done[i])
                store_out(a, e / NT, n0 + e - (e / NT) * NT, v[i]);
        }
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
// split every request into 64-byte halves of lines: a stream of the 6288 x 7168
// weight in that pattern took 25.2 us against 18.4 us for 4 rows x 256 bytes
// per instruction over the same workgroups.
//
// Row pitch of both tiles: 34 chunks (544 bytes).  With 16 lanes reading 16
// rows of one 16-byte column, gfx950's LDS served the 128-bit reads without a
// bank conflict only for row pitches of 2 mod 4 chunks (34, 66, 70, 130 ...);
// a pitch of 33 chunks cost 4 conflict cycles per read and 32 chunks 28
// (SQ_LDS_BANK_CONFLICT per SQ_INSTS_LDS, measured).  Writes of whole rows
// were conflict-free at every pitch tried.
// ---------------------------------------------------------------------------
template <int T, int NW, bool H>
__global__ __launch_bounds__(64 * NW) void k_mfmax(KArgs a)
{
    constexpr int MT = 16 * T;
    constexpr int KW = kMfmaxChunks;           // chunks per stage
    constexpr int PITCH = KW + 2;              // row pitch in 16-byte chunks (see above)
    constexpr int XL = (MT * KW) / (64 * NW);  // x chunks per thread per stage
    constexpr int NX = mfmax_x_windows(MT);    // x windows in LDS: a barrier per NX / 2 stages
    constexpr int PB = NX / 2;                 // stages per barrier
    static_assert(XL >= 1 && XL * 64 * NW == MT * KW, "x window must split evenly over the waves");
    extern __shared__ u32x4 sm[];              // [NW][16][PITCH] then [NX][MT][PITCH]

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
    // split-K: this wave's values ((wave T + t) 4 + q) 64 + lane of the
    // workgroup's partial meet the other K parts' in the swap exchange
    constexpr int E = NW * T * 4 * 64;         // partial values of the workgroup
    int off[4 * T];
    float v[4 * T];
    bool done[4 * T];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const bool live = 16 * t + i16 < a.M && n0 + 4 * g + q < n_end;
            off[t * 4 + q] = live ? ((wave * T + t) * 4 + q) * 64 + lane : -1;
            v[t * 4 + q] = acc[t][q];
        }
    int pair_off[2 * T];                       // the wave's pairs, slot (wave 2T + p) 64 + lane
#pragma unroll
    for (int p = 0; p < 2 * T; ++p)
        pair_off[p] = (wave * 2 * T + p) * 64 + lane;
    swap_exchange_pairs<4 * T>(a.ws + (long)tile * (a.split - 1) * E, E, a.split, s, off, pair_off, v, done);
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (done[t * 4 + q])
                store_out(a, 16 * t + i16, n0 + 4 * g + q, v[t * 4 + q]);
}

// ---------------------------------------------------------------------------
// MFMAW kernel: token tile MT = 16 T; a workgroup owns one equal row range of
// at most 16 RG rows and one K part (of `split`), with NW waves that each
// multiply EVERY row group of the range over every NW-th K stage of SC = 8 or
// 16 chunks (SC / 4 MFMA K-steps).  No wave waits for another until the end:
//
//  * the weight and the x of a stage are loaded row-contiguously -- each
//    wave-wide load is 64 / SC rows (or tokens) x 16 SC bytes -- DEPTH (1 or
//    2) stages ahead in registers, and re-laid out through the wave's own LDS
//    tiles [16 RG][SC + 2] and [MT][SC + 2] (chunks) into A and B fragments.
//    The stage width, the row groups and the depth set the bytes a wave keeps
//    in flight: about 8 KiB of weight per wave (32 KiB per CU) measured
//    best, so four row groups stream one stage ahead and two row groups two.
//    A stage's weight registers are refilled as soon as they are in LDS, its
//    x registers only after its MFMAs: x comes from L2, and issuing it with
//    the weight (or three stages ahead) measured slower;
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
template <int T, int RG, int NW, int SC, int DEPTH, bool H>
__global__ __launch_bounds__(64 * NW) void k_mfmaw(KArgs a)
{
    static_assert(SC == 8 || SC == 16, "stages of 8 or 16 chunks");
    static_assert(DEPTH == 1 || DEPTH == 2, "one or two stages in flight");
    constexpr int RPL = 64 / SC;               // rows (tokens) per wave-wide load
    constexpr int NL = 16 / RPL;               // loads per 16 rows (tokens)
    constexpr int KS = SC / 4;                 // MFMA K-steps per stage
    constexpr int PITCH = SC + 2;
    constexpr int ROWS = 16 * RG;
    constexpr int MT = 16 * T;
    constexpr int E = RG * T * 4 * 64;         // partial values of one wave (and of the workgroup)
    constexpr int EPT = E / (64 * NW);         // of them per thread in the final sum
    static_assert(EPT >= 1 && EPT * 64 * NW == E, "the final sum must split evenly over the threads");
    constexpr int WAVE_LDS = (int)(mfmaw_wave_lds_bytes(ROWS, MT, SC) / 16);   // u32x4 per wave
    static_assert(E * 4 <= WAVE_LDS * 16, "the wave's LDS share must hold its partial sums");
    extern __shared__ u32x4 sm[];              // [NW][WAVE_LDS] (tiles [ROWS + MT][PITCH]); at the end float [NW][E]

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
    u32x4 *wl = sm + wave * WAVE_LDS;
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
        load_wt(wv, j + DEPTH);
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
        load_xt(xv, j + DEPTH);
        __builtin_amdgcn_sched_barrier(0);
    };

    // DEPTH stages in flight; every pass issues all of its loads (past the
    // wave's last stage they touch no memory), so the waits stay partial.
    if constexpr (DEPTH == 2) {
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
    } else {
        u32x4 wa[NL * RG], xa[NL * T];
        load_wt(wa, 0);
        load_xt(xa, 0);
        __builtin_amdgcn_sched_barrier(0);
        for (int j = 0; j < mine; ++j)
            step(wa, xa, j);
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
    // value e: token 16 t + (e % 16), row n_wg + 16 r + 4 ((e / 16) % 4) + q
    auto locate = [&](int e, int &tok, int &n) {
        const int ln = e & 63, q = (e >> 6) & 3, rt = e >> 8;
        const int r = rt / T, t = rt - (rt / T) * T;
        tok = 16 * t + (ln & 15);
        n = n_wg + 16 * r + 4 * (ln >> 4) + q;
    };
    float v[EPT];
    int off[EPT];
    bool done[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = tid + 64 * NW * i;
        int tok, n;
        locate(e, tok, n);
        off[i] = tok < a.M && n < n_end ? e : -1;
        v[i] = red[e];
#pragma unroll
        for (int w = 1; w < NW; ++w)
            v[i] += red[w * E + e];
        done[i] = off[i] >= 0;
    }
    if (a.split > 1) {
        float *wsp = a.ws + (long)tile * (a.split - 1) * E;
        if constexpr (EPT % 2 == 0) {
            int pair_off[EPT / 2];             // the thread's pairs, slot p 64 NW + tid
#pragma unroll
            for (int p = 0; p < EPT / 2; ++p)
                pair_off[p] = p * 64 * NW + tid;
            swap_exchange_pairs<EPT>(wsp, E, a.split, s, off, pair_off, v, done);
        } else {
            swap_exchange<EPT>(wsp, E, a.split, s, off, v, done);
        }
    }
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        if (!done[i])
            continue;
        int tok, n;
        locate(tid + 64 * NW * i, tok, n);
        store_out(a, tok, n, v[i]);
    }
}

// ---------------------------------------------------------------------------
// Row-group stream kernels (MFMA4, DOT2W).  A workgroup owns one equal row
// range of at most 4 RG rows and one K part (of `split`); its NW waves take
// every NW-th stage of 16 K chunks, U stages in flight in registers, with
// nothing shared between waves until their sums are added in LDS at the end.
// Every wave-wide load is the row-contiguous kind: lane l reads chunk l & 15
// of the stage from row (or token) l >> 4 of a 4-row group -- four runs of
// 256 bytes -- so the weight goes HBM -> VGPR -> arithmetic with no LDS.
//
// MFMA4 (token groups T of 4 tokens): v_mfma_f32_4x4x4_16b (BF16, or FP16
// with H) multiplies sixteen independent 4x4x4 blocks: lane 4 b + i gives
// block b its A row i and its B column i (4 values each) and gets back
// D_b[0..3][i].  Block b takes chunk b of the stage, A row i is weight row
// 4 rg + i and B column i token 4 tg + i, so a loaded register becomes an
// operand pair (its low and high 8 bytes) once lane 4 b + i holds what lane
// 16 i + b loaded: one ds_bpermute per dword moves it there (the order the
// operands need, four rows per quad of lanes, loads measurably slower than
// the row-contiguous order).  Each x register serves all RG row groups.
// The blocks hold partial sums over different chunks: after the stream they
// are added by a transposing butterfly over lane bits 5..2.
//
// DOT2W (token tile T = 1, 2, 4 or 8): v_dot2_f32_bf16 (v_dot2_f32_f16),
// lane l multiplies its weight chunk with the same chunk of each token's x,
// loaded per lane (the four lanes of a chunk read the same 16 bytes, which a
// load serves once); each x register serves all RG row groups.  After the
// stream the 16 chunk lanes of a row are added over lane bits 3..0.
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

// c += a b on 4 BF16 (FP16) values per lane, one 4x4x4 block per 4 lanes
template <bool H>
__device__ __forceinline__ f32x4 mma4(unsigned a0, unsigned a1, unsigned b0, unsigned b1, f32x4 c)
{
    const u32x2 av = {a0, a1}, bv = {b0, b1};
    if constexpr (H)
        return __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(f16x4, av), __builtin_bit_cast(f16x4, bv), c,
                                                  0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4, av), __builtin_bit_cast(s16x4, bv),
                                                      c, 0, 0, 0);
}

// lane 4 b + i takes the 16 bytes lane 16 i + b holds (src_addr = 4 x that lane)
__device__ __forceinline__ u32x4 to_block_order(u32x4 v, int src_addr)
{
    const unsigned v0 = v.x, v1 = v.y, v2 = v.z, v3 = v.w;
    return u32x4{(unsigned)__builtin_amdgcn_ds_bpermute(src_addr, (int)v0),
                 (unsigned)__builtin_amdgcn_ds_bpermute(src_addr, (int)v1),
                 (unsigned)__builtin_amdgcn_ds_bpermute(src_addr, (int)v2),
                 (unsigned)__builtin_amdgcn_ds_bpermute(src_addr, (int)v3)};
}

// Transposing steps over single lane bits, exact pairings (lane i with
// i ^ bit): as in wave_reduce_transpose, the lane with the bit clear keeps the
// first half of its vector and adds its partner's copy of that half.
//   bit 3: DPP row_ror:8 (lane i and i ^ 8 of a 16-lane row)
//   bit 2: row_half_mirror (7 - i) then a quad reversal, which brings the
//          partner back to the same quad position: i ^ 4
//   bit 1: quad_perm [2,3,0,1]     bit 0: quad_perm [1,0,3,2]
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppQuadReverse = 0x1B;   // quad_perm [3,2,1,0]

template <int CTRL>
__device__ __forceinline__ float dpp_xor4_read(float x)
{
    return dpp_read<kDppQuadReverse>(dpp_read<kDppRowHalfMirror>(x));
}

template <int V, int BIT>
__device__ __forceinline__ void step_exact(float *v, int lane)
{
    const bool hi = (lane & BIT) != 0;
#pragma unroll
    for (int i = 0; i < V / 2; ++i) {
        const float send = hi ? v[i] : v[i + V / 2];
        const float keep = hi ? v[i + V / 2] : v[i];
        float got;
        if constexpr (BIT == 8)
            got = dpp_read<kDppRowRor8>(send);
        else if constexpr (BIT == 4)
            got = dpp_xor4_read<0>(send);
        else if constexpr (BIT == 2)
            got = dpp_read<kDppQuadXor2>(send);
        else
            got = dpp_read<kDppQuadXor1>(send);
        v[i] = keep + got;
    }
}

constexpr int pow2_at_least(int v, int lo) { return v <= lo ? lo : 2 * pow2_at_least((v + 1) / 2, lo); }

template <bool MFMA, int T, int RG, int U, bool H>
__global__ __launch_bounds__(256) void k_rgs(KArgs a)
{
    constexpr int MT = MFMA ? 4 * T : T;       // token tile
    constexpr int XL = MFMA ? T : T;           // x loads per stage (token groups / tokens)
    constexpr int ROWS = 4 * RG;
    constexpr int V = MFMA ? 4 * RG * T : RG * T;   // sums per lane before the lane reduction
    constexpr int P = pow2_at_least(V, 16);
    constexpr int Q = P / 16;                  // per lane after it
    static_assert(rgs_values_per_lane(MFMA, RG, T) == Q, "host and kernel must agree on the LDS size");
    extern __shared__ float red[];             // [waves][Q][64]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nw = blockDim.x >> 6;
    int tile, s;
    block_coords(a, tile, s);
    const int n_wg = tile_row(a, tile), n_end = tile_row(a, tile + 1);
    const int kb = split_point(a, s, a.K8);
    const int ke = split_point(a, s + 1, a.K8);
    const int stages = (ke - kb + 15) >> 4;
    const int mine = stages > wave ? (stages - wave + nw - 1) / nw : 0;   // stages wave, wave + nw, ...
    const unsigned row_bytes = a.w_pitch, x_pitch = a.x_pitch;
    const int rows_valid = uniform_int(max(0, min(ROWS, n_end - n_wg)));
    const auto wres = make_rsrc(static_cast<const char *>(a.W) + (size_t)(rows_valid ? n_wg : 0) * row_bytes,
                                (unsigned)rows_valid * row_bytes);
    const auto xres = make_rsrc(a.x, (unsigned)a.M * x_pitch);
    const int r4 = lane >> 4, c16 = lane & 15;
    const int perm_src = 4 * (16 * (lane & 3) + (lane >> 2));   // lane 4 b + i <- lane 16 i + b

    f32x4 macc[MFMA ? RG : 1][MFMA ? T : 1];
    float dacc[MFMA ? 1 : RG][MFMA ? 1 : MT];
    if constexpr (MFMA) {
#pragma unroll
        for (int r = 0; r < RG; ++r)
#pragma unroll
            for (int t = 0; t < T; ++t)
                macc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
#pragma unroll
        for (int r = 0; r < RG; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m)
                dacc[r][m] = 0.f;
    }

    // this lane's chunk of the wave's j-th stage; past the wave's last stage,
    // or past the end of its K part, the load is out of range (no memory read)
    auto load = [&](u32x4(&wv)[RG], u32x4(&xv)[XL], int j) {
        const int c = kb + (wave + nw * j) * 16 + c16;
        const bool ok = j < mine && c < ke;
        const unsigned co = (unsigned)c * 16u;
#pragma unroll
        for (int r = 0; r < RG; ++r)
            wv[r] = load_w(wres, lane_off(ok, (unsigned)(4 * r + r4) * row_bytes + co), 0);
#pragma unroll
        for (int t = 0; t < XL; ++t)
            xv[t] = load_x(xres, lane_off(ok, (unsigned)(MFMA ? 4 * t + r4 : t) * x_pitch + co), 0);
        __builtin_amdgcn_sched_barrier(0);   // loads stay ahead of the arithmetic
    };
    auto compute = [&](const u32x4(&wv)[RG], const u32x4(&xv)[XL]) {
        if constexpr (MFMA) {
            u32x4 xb[T];
#pragma unroll
            for (int t = 0; t < T; ++t)
                xb[t] = to_block_order(xv[t], perm_src);
#pragma unroll
            for (int r = 0; r < RG; ++r) {
                const u32x4 wb = to_block_order(wv[r], perm_src);
                const unsigned w0 = wb.x, w1 = wb.y, w2 = wb.z, w3 = wb.w;
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const unsigned x0 = xb[t].x, x1 = xb[t].y, x2 = xb[t].z, x3 = xb[t].w;
                    macc[r][t] = mma4<H>(w0, w1, x0, x1, macc[r][t]);
                    macc[r][t] = mma4<H>(w2, w3, x2, x3, macc[r][t]);
                }
            }
        } else {
#pragma unroll
            for (int r = 0; r < RG; ++r)
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    dacc[r][m] = dot8<H>(wv[r], xv[m], dacc[r][m]);
        }
    };

    // U stages in flight; every pass issues all of its loads (past the wave's
    // last stage they read nothing), so the waits stay partial.
    u32x4 wbuf[U][RG], xbuf[U][XL];
#pragma unroll
    for (int u = 0; u < U; ++u)
        load(wbuf[u], xbuf[u], u);
    for (int j = 0; j < mine; j += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (j + u < mine)
                compute(wbuf[u], xbuf[u]);
            load(wbuf[u], xbuf[u], j + u + U);
        }
    }

    // Lane reduction.  MFMA4: lane bits 5..2 index the block, bits 1..0 the
    // token column; value index (rg T + tg) 4 + row.  DOT2W: lane bits 3..0
    // index the chunk, bits 5..4 the row within a group; value index rg MT + m.
    // Afterwards lane l holds, for q < Q, value (seg Q + q) summed over the
    // reduced lanes, seg = (l >> 2) & 15 (MFMA4) or l & 15 (DOT2W).
    float v[P];
    if constexpr (MFMA) {
#pragma unroll
        for (int r = 0; r < RG; ++r)
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    v[(r * T + t) * 4 + q] = macc[r][t][q];
    } else {
#pragma unroll
        for (int r = 0; r < RG; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m)
                v[r * MT + m] = dacc[r][m];
    }
#pragma unroll
    for (int i = V; i < P; ++i)
        v[i] = 0.f;
    if constexpr (MFMA) {
        step_swap32<P>(v);
        step_swap16<P / 2>(v);
        step_exact<P / 4, 8>(v, lane);
        step_exact<P / 8, 4>(v, lane);
    } else {
        step_exact<P, 8>(v, lane);
        step_exact<P / 2, 4>(v, lane);
        step_exact<P / 4, 2>(v, lane);
        step_exact<P / 8, 1>(v, lane);
    }

    // the waves' sums, added in LDS in wave order
#pragma unroll
    for (int q = 0; q < Q; ++q)
        red[(wave * Q + q) * 64 + lane] = v[q];
    __syncthreads();
    // value e of the workgroup: lane e & 63, q = e >> 6 -> (token, row) or none
    auto locate = [&](int e, int &tok, int &row) {
        const int ln = e & 63, q = e >> 6;
        if constexpr (MFMA) {
            const int idx = ((ln >> 2) & 15) * Q + q, rt = idx >> 2;
            tok = 4 * (rt % T) + (ln & 3);
            row = n_wg + 4 * (rt / T) + (idx & 3);
            return idx < V;
        } else {
            const int idx = (ln & 15) * Q + q;
            tok = idx % MT;
            row = n_wg + 4 * (idx / MT) + (ln >> 4);
            return idx < V;
        }
    };
    float sum[Q];
    int off[Q];
#pragma unroll
    for (int i = 0; i < Q; ++i) {
        const int e = tid + 64 * nw * i;
        off[i] = -1;
        sum[i] = 0.f;
        int tok, row;
        if (e >= Q * 64 || !locate(e, tok, row) || row >= n_end || tok >= a.M)
            continue;
        off[i] = e;
        const int ln = e & 63, q = e >> 6;
        float t = red[q * 64 + ln];
        for (int w = 1; w < nw; ++w)
            t += red[(w * Q + q) * 64 + ln];
        sum[i] = t;
    }
    bool ok[Q];
    if (a.split == 1) {
#pragma unroll
        for (int i = 0; i < Q; ++i)
            ok[i] = off[i] >= 0;
    } else {
        swap_exchange<Q>(a.ws + (long)tile * (a.split - 1) * (Q * 64), Q * 64, a.split, s, off, sum, ok);
    }
#pragma unroll
    for (int i = 0; i < Q; ++i) {
        if (!ok[i])
            continue;
        int tok, row;
        locate(off[i], tok, row);
        store_out(a, tok, row, sum[i]);
    }
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
// instances.def maps each family's parameters to the table fields through
// SK_PAIR(path, mt, rows, unroll, kernel template, template arguments...)
static const KernelInfo kKernels[] = {
#include "instances.def"
};
#undef SK_PAIR

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
