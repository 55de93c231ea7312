// Internal declarations shared by the kernels and the host side of the
// skinny BF16 decode projection library.  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <array>

#include "../../include/skinny.h"

namespace skinny {

// Division of 32-bit unsigned values by a divisor fixed for a launch, as a
// multiply-high, an add and two shifts (Granlund and Montgomery, "Division by
// invariant integers using multiplication", PLDI 1994, section 4): with
// t = (x * mul) >> 32,  x / d = (t + ((x - t) >> s1)) >> s2  for every 32-bit
// x.  The kernels evaluate it on values every lane shares, where a general
// 32- or 64-bit division is a long scalar instruction sequence that would
// delay each workgroup's first load.
struct FastDiv {
    uint32_t mul;
    uint32_t s1;
    uint32_t s2;
};

// d >= 1.  d = 1: t = 0 and x / 1 = x.  Otherwise l = ceil(log2 d) >= 1,
// mul = floor(2^32 (2^l - d) / d) + 1 < 2^32, s1 = 1, s2 = l - 1.
inline FastDiv make_fastdiv(uint32_t d)
{
    if (d <= 1)
        return FastDiv{0u, 0u, 0u};
    const uint32_t l = 32u - (uint32_t)__builtin_clz(d - 1u);
    const uint64_t m = (((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d + 1;
    return FastDiv{(uint32_t)m, 1u, l - 1u};
}

// The same formula on the host, for tests.
inline uint32_t fastdiv_eval(uint32_t x, const FastDiv &f)
{
    const uint32_t t = (uint32_t)(((uint64_t)x * f.mul) >> 32);
    return (t + ((x - t) >> f.s1)) >> f.s2;
}

// Arguments of every kernel, passed by value.  W, x are viewed as rows of
// 16-byte chunks (8 BF16 or FP16 values); K8 = K / 8 chunks per row, rows
// w_pitch / x_pitch bytes apart.
struct KArgs {
    const void *W;      // [N] rows of K8 chunks, w_pitch bytes apart
    const void *x;      // [M] rows of K8 chunks, x_pitch bytes apart
    void *out;          // [M][ldo] BF16 or fp32
    const void *res;    // [M][ldr], the out type, added before the store; or NULL
    float *ws;          // split-K exchange nodes, [tile][split - 1][values of a tile]
    int N;
    int K8;
    int M;
    int n_tiles;        // ceil(N / rows)
    int split;          // workgroups per row tile along K
    int out_f32;        // 1: fp32 output, 0: BF16
    int nxcd;           // XCDs the dispatcher deals workgroups over
    int remap;          // 1: place the split-K workgroups of a tile on one XCD
    int ranges;         // row tile t is [t N / n_tiles, (t + 1) N / n_tiles)
    unsigned w_pitch;   // bytes between rows of W (multiple of 16)
    unsigned x_pitch;   // bytes between rows of x (multiple of 16)
    int ldo;            // elements between rows of out
    int ldr;            // elements between rows of res
    // launch constants for divisions (see FastDiv): by n_tiles, split and
    // nxcd; N = rows_q n_tiles + rows_r, so that with rows_fast (n_tiles <
    // 2^16) t N / n_tiles = t rows_q + (t rows_r) / n_tiles in 32 bits; and
    // gridDim.x = grid_q nxcd + grid_r
    FastDiv fd_tiles, fd_split, fd_nxcd;
    unsigned rows_q, rows_r;
    int rows_fast;
    int grid_q, grid_r;
};

// A compiled kernel instance.
struct KernelInfo {
    int path, mt, rows, unroll;
    int half;           // 0: BF16 inputs, 1: FP16 inputs
    const void *fn;     // host stub address for hipLaunchKernel
};

// All compiled instances (defined next to the kernels).
const KernelInfo *kernel_table(int *count);
const KernelInfo *find_kernel(int path, int mt, int rows, int unroll, int half);

// The compiled instance a tactic runs for BF16 (half = 0) or FP16 inputs
// (KernelInfo.rows is rows per workgroup for DOT2/MFMA, waves for MFMAX,
// 100 waves + row groups for MFMAW, the most rows of a range for MFMA4 and
// DOT2W), or nullptr.  Every instance exists for
// both input types, so a tactic's legality does not depend on it.
const KernelInfo *tactic_kernel(const skinny_tactic &t, int half = 0);

// Measurement probe kernels (host stub addresses).
const void *probe_read_fn();
const void *probe_empty_fn();
constexpr int kProbeSinkFloats = 4096;   // power of two; sink[] size of skinny_probe_read

// Dynamic LDS bytes a tactic needs for rows of K8 16-byte chunks.
size_t tactic_lds_bytes(const skinny_tactic &t, int K8);

// Thread-local error text.
void set_error(const char *fmt, ...);

// Stored tuned tables (tables.cpp): one text line per (chip, N, K, input and
// output type, residual or not: res = 1 for the table of runs that add a
// residual).  parse_table_line fills `table` and returns true only for a
// whole, valid line for this key; load_table_file returns the first such line
// of a file; format_table_line writes one into buf (cap >= 8192 bytes holds
// any table); save_table_file appends one.
bool parse_table_line(const char *line, int cus, int N, int K, int half, skinny_out_dtype od, int res,
                      std::array<skinny_tactic, SKINNY_MAX_M> &table);
// One tactic written as path.mt.rows.waves.unroll.split, the whole string
// (the table lines' field syntax); false for anything else.
bool parse_tactic_text(const char *text, skinny_tactic *t);
bool load_table_file(const char *path, int cus, int N, int K, int half, skinny_out_dtype od, int res,
                     std::array<skinny_tactic, SKINNY_MAX_M> &table);
void format_table_line(int cus, int N, int K, int half, skinny_out_dtype od, int res,
                       const std::array<skinny_tactic, SKINNY_MAX_M> &table, char *buf, size_t cap);
void save_table_file(const char *path, int cus, int N, int K, int half, skinny_out_dtype od, int res,
                     const std::array<skinny_tactic, SKINNY_MAX_M> &table);

// Rows of W per tile and tile count for a tactic.
inline int tiles_for(const skinny_tactic &t, int N) { return (int)(((long long)N + t.rows - 1) / t.rows); }

constexpr int kMaxWaves = 8;
// A buffer load whose offset is at or past its resource's size reads zero and
// touches no memory; kernels pass this offset for a load they skip, so every
// resource (at most kMaxTileRows rows of W, SKINNY_MAX_M rows of x) must be
// smaller than it.
constexpr unsigned kOffOob = 0x7FFFFFF0u;
constexpr int kMaxTileRows = 64;
// A split-K exchange node holds a value as its bits XOR this signalling-NaN
// pattern (no fp32 arithmetic produces it), so an all-zero node is empty:
// the workspace is zeroed when allocated, and every launch leaves it so.
constexpr unsigned kSlotEmptyBits = 0x7FB55AA5u;
constexpr size_t kMaxLds = 60 * 1024;          // in-WG split-K paths (DOT2, MFMA)
// LDS-staged paths (MFMAX, MFMAW) may use a CU's whole 160 KiB, less a
// reserve for the kernels' own static __shared__ variables: a dispatch whose
// static + dynamic LDS exceeds the device limit is not rejected at launch but
// aborts the queue.  Launches are also checked against the exact static size.
constexpr size_t kStaticLdsReserve = 1024;
constexpr size_t kMaxLdsStaged = 160 * 1024 - kStaticLdsReserve;
constexpr int kMfmaxChunks = 32;               // K chunks per MFMAX stage
// MFMAX proper keeps 2 PB x windows, for a barrier per PB stages: PB = 2 for
// token tiles up to 32, 1 for 64 (a barrier per 4 stages measured slower at
// the 16-token tile: 17.6 against 16.3 us on 6288x7168)
constexpr int mfmax_x_windows(int mt) { return mt <= 32 ? 4 : 2; }
inline size_t mfmax_own_lds_bytes(int waves, int mt)
{
    return (size_t)(16 * waves + mfmax_x_windows(mt) * mt) * (kMfmaxChunks + 2) * 16;
}
// MFMAW: unroll 1 and 2 are stages of 8 and 16 chunks two deep, 3 and 4 the
// same one deep; wave tiles [waves][rows + mt][stage + 2 chunks], which the
// waves' partial sums (rows x mt floats a wave) reuse at the end -- the
// larger of the two per wave
inline int mfmaw_stage_chunks(int unroll) { return unroll == 2 || unroll == 4 ? 16 : 8; }
inline int mfmaw_depth(int unroll) { return unroll <= 2 ? 2 : 1; }
constexpr size_t mfmaw_wave_lds_bytes(int rows, int mt, int stage_chunks)
{
    return (size_t)(rows + mt) * (stage_chunks + 2) * 16 > (size_t)rows * mt * 4
               ? (size_t)(rows + mt) * (stage_chunks + 2) * 16
               : (size_t)rows * mt * 4;
}
inline size_t mfmaw_lds_bytes(int waves, int rows, int mt, int unroll)
{
    return (size_t)waves * mfmaw_wave_lds_bytes(rows, mt, mfmaw_stage_chunks(unroll));
}
// Row-group stream kernels (MFMA4, DOT2W): each lane ends with Q = max(16, V
// rounded up to a power of two) / 16 sums, V = 4 RG T (MFMA4, T token groups)
// or RG T (DOT2W, T tokens), added over the waves in LDS [waves][Q][64]
constexpr int rgs_values_per_lane(bool mfma, int rg, int t)
{
    int p = 16;
    while (p < (mfma ? 4 : 1) * rg * t)
        p *= 2;
    return p / 16;
}
inline int rgs_q(const skinny_tactic &t)
{
    const bool mfma = t.path == SKINNY_PATH_MFMA4;
    return rgs_values_per_lane(mfma, t.rows / 4, mfma ? t.mt / 4 : t.mt);
}
inline size_t rgs_lds_bytes(const skinny_tactic &t) { return (size_t)t.waves * rgs_q(t) * 64 * sizeof(float); }
// exchange nodes per tile: split - 1 of Q * 64 values
inline size_t rgs_node_floats(const skinny_tactic &t) { return (size_t)rgs_q(t) * 64; }
// K chunks per row-group stream stage (one per block of the 16-block MFMA)
constexpr int kRgsChunks = 16;
inline bool is_rgs_path(int path) { return path == SKINNY_PATH_MFMA4 || path == SKINNY_PATH_DOT2W; }
// the v_dot2 kernels
inline bool is_dot2_path(int path)
{
    return path == SKINNY_PATH_DOT2 || path == SKINNY_PATH_DOT2R || path == SKINNY_PATH_DOT2W;
}
// Kernel families measured and removed (their path numbers stay reserved, so a
// stored table that names one is refused, not misread).
inline bool is_retired_path(int path)
{
    return path == SKINNY_PATH_DOT2X || path == SKINNY_PATH_MFMAD || path == SKINNY_PATH_MFMAS ||
           path == SKINNY_PATH_MFMAR || path == SKINNY_PATH_MFMAK;
}
// MFMAT: the 16-token MFMA kernel launched over token groups of 16; a launch
// has ceil(M / 16) of them, a table entry at most mt / 16
constexpr int kTokenGroup = 16;
inline int token_groups(const skinny_tactic &t)
{
    return t.path == SKINNY_PATH_MFMAT ? t.mt / kTokenGroup : 1;
}
// MFMAT is enumerated only for weights of at most this many bytes: each
// XCD's 4 MiB L2 then holds its share of the row tiles (an eighth) with
// room to spare, so the groups' re-reads of a tile stay on chip
constexpr long long kTokenGroupMaxWeightBytes = 16LL << 20;
// Values of one row tile's partial (of one token group), the size of one
// exchange node
inline size_t tile_values(const skinny_tactic &t)
{
    if (is_rgs_path(t.path))
        return rgs_node_floats(t);
    return (size_t)(t.path == SKINNY_PATH_MFMAT ? kTokenGroup : t.mt) * t.rows;
}

}  // namespace skinny
