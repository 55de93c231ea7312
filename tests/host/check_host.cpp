// Host-only checks of the tactic logic and the stored-table parser, built with
// g++ -fsanitize=address,undefined (no HIP, no GPU): the kernel instance list
// is expanded into entries without kernels, exactly as the library expands it
// into real ones.  Every check that fails prints its case and the program
// exits non-zero; a sanitizer report aborts it.
#include <limits.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <random>
#include <string>
#include <vector>

#include "skinny_internal.h"

namespace skinny {

#define SK_PAIR(PATH, MT, ROWS, U, KERNEL, ...) {PATH, MT, ROWS, U, 0, nullptr}, {PATH, MT, ROWS, U, 1, nullptr}
static const KernelInfo kKernels[] = {
#include "instances.def"
};
#undef SK_PAIR

// The partial values one workgroup of each instance swaps per split-K
// exchange node, from the kernel's own template arguments: k_dot2<MT, R, U>
// MT R, k_mfma<T, RT, U> (16 T)(16 RT), k_mfmax<T, NW> and k_mfmaw<T, RG, NW,
// SC, DEPTH> 256 T NW and 256 T RG (4 values x 64 lanes per 16x16 tile), and
// k_rgs<MFMA, T, RG, U> 64 lanes x the sums a lane keeps after its lane
// reduction (the power of two >= 16 at least its 4 RG T (MFMA4) or RG T
// (DOT2W) sums, over 16).
constexpr int node_k_dot2(int mt, int r, int) { return mt * r; }
constexpr int node_k_mfma(int t, int rt, int) { return 16 * t * 16 * rt; }
constexpr int node_k_mfmax(int t, int nw) { return 256 * t * nw; }
constexpr int node_k_mfmaw(int t, int rg, int, int, int) { return 256 * t * rg; }
constexpr int node_k_rgs(bool mfma, int t, int rg, int)
{
    int p = 16;
    while (p < (mfma ? 4 : 1) * rg * t)
        p *= 2;
    return p / 16 * 64;
}
#define SK_PAIR(PATH, MT, ROWS, U, KERNEL, ...) node_##KERNEL(__VA_ARGS__), node_##KERNEL(__VA_ARGS__)
static const int kNodeValues[] = {
#include "instances.def"
};
#undef SK_PAIR
static_assert(sizeof(kNodeValues) / sizeof(kNodeValues[0]) == sizeof(kKernels) / sizeof(kKernels[0]),
              "one node size per instance");

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

using namespace skinny;
using Table = std::array<skinny_tactic, SKINNY_MAX_M>;

static int g_failures = 0;

#define CHECK(cond, ...)                                                                                     \
    do {                                                                                                     \
        if (!(cond)) {                                                                                       \
            fprintf(stderr, "FAIL %s:%d: %s: ", __FILE__, __LINE__, #cond);                                 \
            fprintf(stderr, __VA_ARGS__);                                                                    \
            fprintf(stderr, "\n");                                                                           \
            ++g_failures;                                                                                    \
        }                                                                                                    \
    } while (0)

static bool same(const skinny_tactic &a, const skinny_tactic &b) { return memcmp(&a, &b, sizeof a) == 0; }

struct Shape {
    int N, K;
};

// Shapes of the decode projections, tiny ones and the int-range extremes.
static const Shape kShapes[] = {
    {6288, 7168}, {3584, 7168}, {7168, 18432}, {6144, 7168}, {140, 7168}, {1536, 128}, {256, 512},
    {1, 8},       {3, 24},      {17, 1032},    {100000, 8},  {INT_MAX, 8}, {8, INT_MAX - 7},
    {INT_MAX, INT_MAX - 7},
};
static const int kCus[] = {1, 7, 80, 256, 304, 1 << 20, INT_MAX};

static std::vector<skinny_tactic> enumerate(int N, int K, int cus)
{
    const int n = skinny_enumerate_tactics_ex(N, K, cus, nullptr, 0);
    CHECK(n >= 0, "enumerate N=%d K=%d cus=%d returned %d", N, K, cus, n);
    if (n <= 0)
        return {};
    std::vector<skinny_tactic> v((size_t)n);
    const int m = skinny_enumerate_tactics_ex(N, K, cus, v.data(), n);
    CHECK(m == n, "enumerate count changed %d -> %d", n, m);
    // a short buffer takes a prefix and still reports the total
    if (n > 3) {
        std::vector<skinny_tactic> w(3);
        CHECK(skinny_enumerate_tactics_ex(N, K, cus, w.data(), 3) == n, "short buffer count");
        for (int i = 0; i < 3; ++i)
            CHECK(same(w[(size_t)i], v[(size_t)i]), "short buffer prefix %d", i);
    }
    return v;
}

static void check_enumeration()
{
    for (const Shape &s : kShapes) {
        for (int cus : kCus) {
            std::vector<skinny_tactic> v = enumerate(s.N, s.K, cus);
            for (const skinny_tactic &t : v)
                CHECK(skinny_tactic_check(&t, s.N, s.K) == SKINNY_OK, "N=%d K=%d cus=%d path=%d: %s", s.N, s.K,
                      cus, t.path, skinny_last_error());
        }
    }
    // bad arguments
    skinny_tactic one;
    CHECK(skinny_enumerate_tactics_ex(0, 8, 256, &one, 1) == -1, "N=0");
    CHECK(skinny_enumerate_tactics_ex(8, 12, 256, &one, 1) == -1, "K=12");
    CHECK(skinny_enumerate_tactics_ex(8, 8, 0, &one, 1) == -1, "cus=0");
    CHECK(skinny_enumerate_tactics_ex(8, 8, 256, nullptr, 1) == -1, "NULL buffer");
    CHECK(skinny_enumerate_tactics_ex(8, 8, 256, &one, -1) == -1, "cap<0");
    CHECK(skinny_enumerate_tactics(INT_MIN, INT_MIN, nullptr, 0) == -1, "INT_MIN shape");
}

// The host sizes the exchange workspace with tile_values(t) floats per node
// (times token_groups(t) for MFMAT); the kernel a tactic launches indexes
// nodes of its own partial count.  The two must agree for every enumerated
// tactic, or a split launch would swap past the workspace.
static void check_exchange_nodes()
{
    int checked = 0;
    for (const Shape &s : kShapes) {
        if ((long long)s.N * s.K >= (1LL << 31))
            continue;                                    // not a shape a plan accepts
        for (const skinny_tactic &t : enumerate(s.N, s.K, 256)) {
            const KernelInfo *k = tactic_kernel(t);
            CHECK(k != nullptr, "path=%d mt=%d rows=%d: no instance", t.path, t.mt, t.rows);
            if (!k)
                continue;
            const int node = kNodeValues[k - kKernels];
            CHECK(tile_values(t) == (size_t)node, "N=%d K=%d path=%d mt=%d rows=%d waves=%d unroll=%d: host %zu, "
                  "kernel %d values per node", s.N, s.K, t.path, t.mt, t.rows, t.waves, t.unroll, tile_values(t), node);
            if (t.path == SKINNY_PATH_MFMAT)
                CHECK(token_groups(t) * kTokenGroup == t.mt, "MFMAT mt=%d: groups %d", t.mt, token_groups(t));
            else
                CHECK(token_groups(t) == 1, "path=%d: %d token groups", t.path, token_groups(t));
            ++checked;
        }
    }
    CHECK(checked > 1000, "only %d tactics checked", checked);
}

// Tactics of arbitrary fields: the check must answer without undefined
// behaviour, and whatever it accepts must name a compiled instance.
static void check_tactic_fuzz()
{
    std::mt19937_64 rng(12345);
    const int edge[] = {INT_MIN, INT_MIN + 1, -65536, -1, 0, 1, 2, 3, 4, 7, 8, 16, 28, 32, 56, 64, 100, 128,
                        401, 402, 802, 65536, INT_MAX - 1, INT_MAX};
    auto pick = [&]() -> int {
        const unsigned r = (unsigned)(rng() % 4);
        if (r == 0)
            return edge[rng() % (sizeof edge / sizeof edge[0])];
        if (r == 1)
            return (int)(uint32_t)rng();
        return (int)(rng() % 70);
    };
    for (int i = 0; i < 200000; ++i) {
        skinny_tactic t = {(int)(rng() % 14) - 1, pick(), pick(), pick(), pick(), pick()};
        const Shape s = kShapes[rng() % (sizeof kShapes / sizeof kShapes[0])];
        const int N = (rng() % 8) ? s.N : pick(), K = (rng() % 8) ? s.K : pick();
        if (skinny_tactic_check(&t, N, K) == SKINNY_OK)
            CHECK(tactic_kernel(t) != nullptr, "accepted a tactic with no kernel");
        else
            CHECK(skinny_last_error()[0] != 0, "a refusal without a reason");
    }
    CHECK(skinny_tactic_check(nullptr, 8, 8) == SKINNY_ERR_INVALID_ARG, "NULL tactic");
}

static void check_select_table()
{
    std::vector<skinny_tactic> v = enumerate(6288, 7168, 256);
    std::mt19937_64 rng(7);
    std::vector<double> times(v.size());
    for (double &t : times)
        t = (rng() % 5 == 0) ? -1.0 : 10.0 + (double)(rng() % 1000) / 100.0;
    Table table;
    const skinny_status s = skinny_select_table(v.data(), times.data(), (int)v.size(), table.data());
    CHECK(s == SKINNY_OK, "select: %s", skinny_last_error());
    for (int m = 1; m <= SKINNY_MAX_M; ++m)
        CHECK(table[(size_t)m - 1].mt >= m, "table M=%d tile %d", m, table[(size_t)m - 1].mt);
    CHECK(skinny_select_table(nullptr, times.data(), 1, table.data()) == SKINNY_ERR_INVALID_ARG, "NULL cand");
    CHECK(skinny_select_table(v.data(), times.data(), -1, table.data()) == SKINNY_ERR_INVALID_ARG, "count<0");
    CHECK(skinny_select_table(v.data(), times.data(), 0, table.data()) == SKINNY_ERR_INVALID_ARG, "count 0");
}

static void check_status_strings()
{
    for (int s = -100; s <= 100; ++s) {
        const char *p = skinny_status_string((skinny_status)s);
        CHECK(p && p[0], "status %d", s);
    }
}

static void check_fastdiv()
{
    std::mt19937_64 rng(99);
    const uint32_t ds[] = {1u, 2u, 3u, 7u, 255u, 256u, 257u, 3144u, 65535u, 65536u, 0x7FFFFFFFu, 0x80000000u,
                           0x80000001u, 0xFFFFFFFFu};
    for (uint32_t d : ds) {
        const FastDiv f = make_fastdiv(d);
        const uint32_t xs[] = {0u, 1u, d - 1u, d, d + 1u, 0x7FFFFFFFu, 0xFFFFFFFEu, 0xFFFFFFFFu};
        for (uint32_t x : xs)
            CHECK(fastdiv_eval(x, f) == x / d, "x=%u d=%u", x, d);
        for (int i = 0; i < 2000; ++i) {
            const uint32_t x = (uint32_t)rng();
            CHECK(fastdiv_eval(x, f) == x / d, "x=%u d=%u", x, d);
        }
    }
    for (int i = 0; i < 2000; ++i) {
        const uint32_t d = 1u + (uint32_t)(rng() % 0xFFFFFFFFull), x = (uint32_t)rng();
        CHECK(fastdiv_eval(x, make_fastdiv(d)) == x / d, "x=%u d=%u", x, d);
    }
}

static Table a_table(int N, int K)
{
    std::vector<skinny_tactic> v = enumerate(N, K, 256);
    std::vector<double> times(v.size());
    for (size_t i = 0; i < v.size(); ++i)
        times[i] = 10.0 + (double)((i * 7919) % 113);
    Table t;
    skinny_select_table(v.data(), times.data(), (int)v.size(), t.data());
    return t;
}

static std::string line_of(int cus, int N, int K, int half, skinny_out_dtype od, const Table &t, int res = 0)
{
    std::vector<char> buf(8192);
    format_table_line(cus, N, K, half, od, res, t, buf.data(), buf.size());
    return std::string(buf.data());
}

// parse a copy in a buffer of exactly its size, so ASan sees any read past it
static bool parse_exact(const std::string &s, int cus, int N, int K, int half, skinny_out_dtype od, Table &out,
                        int res = 0)
{
    std::vector<char> buf(s.begin(), s.end());
    buf.push_back(0);
    return parse_table_line(buf.data(), cus, N, K, half, od, res, out);
}

static bool valid_table(const Table &t, int N, int K)
{
    for (int m = 1; m <= SKINNY_MAX_M; ++m)
        if (skinny_tactic_check(&t[(size_t)m - 1], N, K) != SKINNY_OK || t[(size_t)m - 1].mt < m)
            return false;
    return true;
}

static void check_table_lines()
{
    const int N = 6288, K = 7168, cus = 256;
    const Table t = a_table(N, K);
    const std::string good = line_of(cus, N, K, 0, SKINNY_OUT_BF16, t);
    Table got;
    CHECK(parse_exact(good, cus, N, K, 0, SKINNY_OUT_BF16, got), "the written line parses");
    for (int m = 0; m < SKINNY_MAX_M; ++m)
        CHECK(same(got[(size_t)m], t[(size_t)m]), "round trip M=%d", m + 1);
    CHECK(parse_exact(good + "\n", cus, N, K, 0, SKINNY_OUT_BF16, got), "newline");
    CHECK(parse_exact(good + "\r\n", cus, N, K, 0, SKINNY_OUT_BF16, got), "CRLF");
    CHECK(parse_exact("  \t" + good + " \t ", cus, N, K, 0, SKINNY_OUT_BF16, got), "spaces and tabs");
    // other keys
    CHECK(!parse_exact(good, cus + 1, N, K, 0, SKINNY_OUT_BF16, got), "other CU count");
    CHECK(!parse_exact(good, cus, N + 8, K, 0, SKINNY_OUT_BF16, got), "other N");
    CHECK(!parse_exact(good, cus, N, K + 8, 0, SKINNY_OUT_BF16, got), "other K");
    CHECK(!parse_exact(good, cus, N, K, 1, SKINNY_OUT_BF16, got), "other input type");
    CHECK(!parse_exact(good, cus, N, K, 0, SKINNY_OUT_F32, got), "other output type");
    // the residual table's line: its own key, and never taken for the other
    const std::string res_line = line_of(cus, N, K, 0, SKINNY_OUT_BF16, t, 1);
    CHECK(res_line.find(" bf16+res ") != std::string::npos, "residual key %s", res_line.substr(0, 60).c_str());
    CHECK(parse_exact(res_line, cus, N, K, 0, SKINNY_OUT_BF16, got, 1), "residual line parses as residual");
    CHECK(!parse_exact(res_line, cus, N, K, 0, SKINNY_OUT_BF16, got, 0), "residual line is not the plain table");
    CHECK(!parse_exact(good, cus, N, K, 0, SKINNY_OUT_BF16, got, 1), "plain line is not the residual table");
    CHECK(!parse_exact(line_of(cus, N, K, 0, SKINNY_OUT_F32, t, 1), cus, N, K, 0, SKINNY_OUT_BF16, got, 1),
          "f32+res is not bf16+res");
    // every prefix of the line is refused (the whole line less trailing blanks aside)
    for (size_t n = 0; n < good.size(); ++n)
        CHECK(!parse_exact(good.substr(0, n), cus, N, K, 0, SKINNY_OUT_BF16, got), "prefix of %zu chars", n);
    // one more or one less tactic, trailing text
    const size_t last = good.rfind(' ');
    CHECK(!parse_exact(good + good.substr(last), cus, N, K, 0, SKINNY_OUT_BF16, got), "65 tactics");
    CHECK(!parse_exact(good.substr(0, last), cus, N, K, 0, SKINNY_OUT_BF16, got), "63 tactics");
    CHECK(!parse_exact(good + " x", cus, N, K, 0, SKINNY_OUT_BF16, got), "trailing word");
    // numbers out of int range, signs, empty fields, other separators
    const char *bad_fields[] = {"99999999999999999999", "2147483648", "-2147483649", "+1", "1e3", "0x10", "",
                                "1..2", ".1", "1.", "-", "--1", "\xff", "1,2"};
    const std::string key = "skinny-table v2 gfx950 256 6288 7168 bf16 bf16";
    CHECK(good.compare(0, key.size(), key) == 0, "line key %s", good.substr(0, key.size()).c_str());
    std::string tail = good.substr(key.size());
    for (const char *b : bad_fields) {
        // in a header number
        CHECK(!parse_exact(std::string("skinny-table v2 gfx950 ") + b + " 6288 7168 bf16 bf16" + tail, cus, N, K,
                           0, SKINNY_OUT_BF16, got),
              "CU field %s", b);
        // as a tactic field
        const size_t first = tail.find('.');
        std::string mutated = key + tail.substr(0, first + 1) + b + tail.substr(tail.find('.', first + 1));
        if (parse_exact(mutated, cus, N, K, 0, SKINNY_OUT_BF16, got))
            CHECK(valid_table(got, N, K), "accepted an invalid table with field %s", b);
    }
    // every single-byte change: whatever parses is a valid table
    const char subs[] = {'x', '.', '-', ' ', '9', '0', '\t', '\n', (char)0x80};
    int accepted = 0;
    for (size_t i = 0; i < good.size(); ++i) {
        for (char c : subs) {
            std::string m = good;
            m[i] = c;
            if (parse_exact(m, cus, N, K, 0, SKINNY_OUT_BF16, got)) {
                ++accepted;
                CHECK(valid_table(got, N, K), "byte %zu -> 0x%02x accepted an invalid table", i, (unsigned char)c);
            }
        }
        std::string d = good;
        d.erase(i, 1);
        if (parse_exact(d, cus, N, K, 0, SKINNY_OUT_BF16, got))
            CHECK(valid_table(got, N, K), "deleting byte %zu accepted an invalid table", i);
    }
    printf("single-byte changes still parsing to valid tables: %d\n", accepted);
    // a table whose M entry has a smaller token tile than M
    Table small = t;
    small[SKINNY_MAX_M - 1] = t[0];
    if (t[0].mt < SKINNY_MAX_M)
        CHECK(!parse_exact(line_of(cus, N, K, 0, SKINNY_OUT_BF16, small), cus, N, K, 0, SKINNY_OUT_BF16, got),
              "token tile below M");
    // a retired kernel family
    Table retired = t;
    retired[0].path = SKINNY_PATH_DOT2X;
    CHECK(!parse_exact(line_of(cus, N, K, 0, SKINNY_OUT_BF16, retired), cus, N, K, 0, SKINNY_OUT_BF16, got),
          "retired path");
    // format into short buffers stays inside them
    for (size_t cap : {(size_t)1, (size_t)10, (size_t)60, (size_t)61, (size_t)200, (size_t)4000}) {
        std::vector<char> buf(cap);
        format_table_line(cus, N, K, 0, SKINNY_OUT_BF16, 0, t, buf.data(), cap);
        CHECK(strlen(buf.data()) < cap, "format cap %zu", cap);
    }
}

// parse_tactic_text (SKINNY_FORCE_TACTIC) on a copy of exactly the string's size
static bool parse_one(const std::string &s, skinny_tactic *t)
{
    std::vector<char> buf(s.begin(), s.end());
    buf.push_back(0);
    return parse_tactic_text(buf.data(), t);
}

static void check_tactic_text()
{
    skinny_tactic t;
    CHECK(parse_one("9.32.64.4.3.2", &t) && same(t, skinny_tactic{9, 32, 64, 4, 3, 2}), "a tactic parses");
    CHECK(parse_one("-1.0.2147483647.-2147483648.0.0", &t) && t.path == -1 && t.rows == INT_MAX &&
              t.waves == INT_MIN,
          "int-range fields parse (legality is skinny_tactic_check's)");
    const char *bad[] = {"", "9", "9.32.64.4.3", "9.32.64.4.3.2.1", "9.32.64.4.3.2 ", " 9.32.64.4.3.2",
                         "9.32.64.4.3.", ".9.32.64.4.3.2", "9..32.64.4.3.2", "9.32.64.4.3.2x", "9,32,64,4,3,2",
                         "9.32.64.4.3.2147483648", "9.32.64.4.3.+2", "9.32.64.4.3.0x2", "9.32.64.4.3.2\n"};
    for (const char *b : bad)
        CHECK(!parse_one(b, &t), "refused \"%s\"", b);
    CHECK(!parse_tactic_text(nullptr, &t) && !parse_tactic_text("1.1.1.1.1.1", nullptr), "NULL arguments");
    // every prefix of a valid tactic but the whole is refused
    const std::string good = "10.16.28.4.3.2";
    for (size_t n = 0; n < good.size(); ++n)
        CHECK(!parse_one(good.substr(0, n), &t), "prefix of %zu chars", n);
}

static void check_table_files(const char *dir)
{
    const int N = 3584, K = 7168, cus = 256;
    const Table t = a_table(N, K);
    const std::string good = line_of(cus, N, K, 0, SKINNY_OUT_F32, t);
    const std::string path = std::string(dir) + "/tables.txt";
    Table got;
    // missing file
    CHECK(!load_table_file((std::string(dir) + "/missing.txt").c_str(), cus, N, K, 0, SKINNY_OUT_F32, 0, got),
          "missing file");
    // garbage around the line, an over-long line holding a valid table after the
    // read buffer (skipped), binary bytes, and the valid line last without a newline
    {
        FILE *f = fopen(path.c_str(), "wb");
        fprintf(f, "\n\n# comment\nskinny-table\nskinny-table v2\n%s", good.substr(0, good.size() / 2).c_str());
        fprintf(f, "\n");
        std::string longline(20000, 'y');
        longline += " " + good;
        fprintf(f, "%s\n", longline.c_str());
        for (int i = 0; i < 300; ++i)
            fputc((i * 37) & 0xFF, f);
        fprintf(f, "\n%s", good.c_str());
        fclose(f);
    }
    CHECK(load_table_file(path.c_str(), cus, N, K, 0, SKINNY_OUT_F32, 0, got), "valid last line without newline");
    for (int m = 0; m < SKINNY_MAX_M; ++m)
        CHECK(same(got[(size_t)m], t[(size_t)m]), "loaded M=%d", m + 1);
    // a file of only malformed content
    {
        FILE *f = fopen(path.c_str(), "wb");
        std::string longline(9000, '7');
        fprintf(f, "%s\n%s\n", longline.c_str(), good.substr(0, good.size() - 3).c_str());
        std::string tailonly = "x" + std::string(8190 - 1, ' ') + good;   // the valid text past the buffer
        fprintf(f, "%s\n", tailonly.c_str());
        fclose(f);
    }
    CHECK(!load_table_file(path.c_str(), cus, N, K, 0, SKINNY_OUT_F32, 0, got), "malformed file");
    // save appends and load takes the first line for the key
    remove(path.c_str());
    save_table_file(path.c_str(), cus, N, K, 0, SKINNY_OUT_F32, 0, t);
    Table other = a_table(N, K);
    other[63] = t[63];
    save_table_file(path.c_str(), cus, N, K, 0, SKINNY_OUT_BF16, 0, other);
    CHECK(load_table_file(path.c_str(), cus, N, K, 0, SKINNY_OUT_F32, 0, got), "saved table loads");
    CHECK(load_table_file(path.c_str(), cus, N, K, 0, SKINNY_OUT_BF16, 0, got), "second saved table loads");
    CHECK(!load_table_file(path.c_str(), cus, N, K, 0, SKINNY_OUT_BF16, 1, got), "no residual table saved yet");
    Table res = t;
    res[0] = t[1].mt >= 1 ? t[1] : t[0];
    save_table_file(path.c_str(), cus, N, K, 0, SKINNY_OUT_BF16, 1, res);
    CHECK(load_table_file(path.c_str(), cus, N, K, 0, SKINNY_OUT_BF16, 1, got) && same(got[0], res[0]),
          "the residual table loads apart from the plain one");
    CHECK(load_table_file(path.c_str(), cus, N, K, 0, SKINNY_OUT_BF16, 0, got) && same(got[0], other[0]),
          "the plain table is unchanged by it");
    remove(path.c_str());
}

int main(int argc, char **argv)
{
    const char *dir = argc > 1 ? argv[1] : ".";
    check_enumeration();
    check_exchange_nodes();
    check_tactic_fuzz();
    check_select_table();
    check_status_strings();
    check_fastdiv();
    check_table_lines();
    check_tactic_text();
    check_table_files(dir);
    if (g_failures) {
        fprintf(stderr, "%d check(s) failed\n", g_failures);
        return 1;
    }
    printf("host checks ok\n");
    return 0;
}
