// Tuned tables stored in a text file (SKINNY_TABLE_CACHE=<file>), keyed like
// the pages' per-part measured tables ("vllm.models.kimi_k3.nvidia.
// low_latency_gemm", the measured {M: call} tables per part) by the chip (arch,
// CU count), the shape and whether the runs add a residual.  One line per table:
//   skinny-table v2 <arch> <cus> <N> <K> <bf16|f16 in> <out> <64 x path.mt.rows.waves.unroll.split>
// with <out> bf16 or f32, followed by +res for the table of runs with a residual.
// The file is input from outside the library: a line is taken only when every
// field parses as a whole decimal number in int range, there are exactly 64
// tactics and nothing after them, every tactic passes skinny_tactic_check and
// the entry for M has a token tile of at least M.  Anything else (a truncated,
// over-long or garbled line) is skipped.  Writers append.  Nothing here calls
// the HIP runtime.
#include <errno.h>
#include <limits.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "skinny_internal.h"

namespace skinny {

namespace {

const char *kTableTag = "skinny-table";
constexpr size_t kMaxLine = 8192;   // 8 header fields + 64 tactics of at most 6 x 11 + 5 chars

// The next whitespace-separated field of *p, as [start, end); false at the end.
bool next_field(const char **p, const char **start, const char **end)
{
    const char *s = *p;
    while (*s == ' ' || *s == '\t' || *s == '\r' || *s == '\n')
        ++s;
    if (!*s)
        return false;
    const char *e = s;
    while (*e && *e != ' ' && *e != '\t' && *e != '\r' && *e != '\n')
        ++e;
    *start = s;
    *end = e;
    *p = e;
    return true;
}

bool field_is(const char *s, const char *e, const char *word)
{
    const size_t n = strlen(word);
    return (size_t)(e - s) == n && !memcmp(s, word, n);
}

const char *out_token(skinny_out_dtype od, int res)
{
    if (od == SKINNY_OUT_F32)
        return res ? "f32+res" : "f32";
    return res ? "bf16+res" : "bf16";
}

// A decimal int (optional '-', at least one digit, in int range) at the start
// of [*s, stop); *s advanced past its digits.
bool parse_int(const char **s, const char *stop, int *v)
{
    const char *q = *s;
    if (q < stop && *q == '-')
        ++q;
    if (q >= stop || *q < '0' || *q > '9')
        return false;
    char buf[24];
    const char *d = q;
    while (d < stop && *d >= '0' && *d <= '9')
        ++d;
    const size_t n = (size_t)(d - *s);
    if (n >= sizeof buf)
        return false;
    memcpy(buf, *s, n);
    buf[n] = 0;
    errno = 0;
    char *endp = nullptr;
    const long long x = strtoll(buf, &endp, 10);
    if (errno || endp != buf + n || x < INT_MIN || x > INT_MAX)
        return false;
    *v = (int)x;
    *s = d;
    return true;
}

bool whole_int(const char *s, const char *e, int *v) { return parse_int(&s, e, v) && s == e; }

// path.mt.rows.waves.unroll.split, exactly
bool parse_tactic(const char *s, const char *e, skinny_tactic *t)
{
    int f[6];
    for (int i = 0; i < 6; ++i) {
        if (!parse_int(&s, e, &f[i]))
            return false;
        if (i < 5) {
            if (s >= e || *s != '.')
                return false;
            ++s;
        }
    }
    if (s != e)
        return false;
    *t = skinny_tactic{f[0], f[1], f[2], f[3], f[4], f[5]};
    return true;
}

}  // namespace

bool parse_tactic_text(const char *text, skinny_tactic *t)
{
    return text && t && parse_tactic(text, text + strlen(text), t);
}

bool parse_table_line(const char *line, int cus, int N, int K, int half, skinny_out_dtype od, int res,
                      std::array<skinny_tactic, SKINNY_MAX_M> &table)
{
    const char *p = line, *s, *e;
    int v;
    if (!next_field(&p, &s, &e) || !field_is(s, e, kTableTag))
        return false;
    if (!next_field(&p, &s, &e) || !field_is(s, e, "v2"))
        return false;
    if (!next_field(&p, &s, &e) || !field_is(s, e, "gfx950"))
        return false;
    const int want[3] = {cus, N, K};
    for (int w : want)
        if (!next_field(&p, &s, &e) || !whole_int(s, e, &v) || v != w)
            return false;
    if (!next_field(&p, &s, &e) || !field_is(s, e, half ? "f16" : "bf16"))
        return false;
    if (!next_field(&p, &s, &e) || !field_is(s, e, out_token(od, res)))
        return false;
    std::array<skinny_tactic, SKINNY_MAX_M> t;
    for (int m = 1; m <= SKINNY_MAX_M; ++m) {
        skinny_tactic &x = t[m - 1];
        if (!next_field(&p, &s, &e) || !parse_tactic(s, e, &x))
            return false;
        if (skinny_tactic_check(&x, N, K) != SKINNY_OK || x.mt < m)
            return false;
    }
    if (next_field(&p, &s, &e))
        return false;
    table = t;
    return true;
}

bool load_table_file(const char *path, int cus, int N, int K, int half, skinny_out_dtype od, int res,
                     std::array<skinny_tactic, SKINNY_MAX_M> &table)
{
    FILE *f = fopen(path, "r");
    if (!f)
        return false;
    char line[kMaxLine];
    bool found = false;
    while (!found && fgets(line, sizeof line, f)) {
        const size_t n = strlen(line);
        if (n + 1 == sizeof line && line[n - 1] != '\n') {
            // longer than any table line: skip the rest of it
            int c;
            while ((c = fgetc(f)) != EOF && c != '\n') {
            }
            continue;
        }
        found = parse_table_line(line, cus, N, K, half, od, res, table);
    }
    fclose(f);
    return found;
}

void format_table_line(int cus, int N, int K, int half, skinny_out_dtype od, int res,
                       const std::array<skinny_tactic, SKINNY_MAX_M> &table, char *buf, size_t cap)
{
    size_t n = (size_t)snprintf(buf, cap, "%s v2 gfx950 %d %d %d %s %s", kTableTag, cus, N, K,
                                half ? "f16" : "bf16", out_token(od, res));
    for (const skinny_tactic &e : table)
        if (n < cap)
            n += (size_t)snprintf(buf + n, cap - n, " %d.%d.%d.%d.%d.%d", e.path, e.mt, e.rows, e.waves,
                                  e.unroll, e.split);
}

void save_table_file(const char *path, int cus, int N, int K, int half, skinny_out_dtype od, int res,
                     const std::array<skinny_tactic, SKINNY_MAX_M> &table)
{
    char line[kMaxLine];
    format_table_line(cus, N, K, half, od, res, table, line, sizeof line);
    FILE *f = fopen(path, "a");
    if (!f)
        return;
    fprintf(f, "%s\n", line);
    fclose(f);
}

}  // namespace skinny
