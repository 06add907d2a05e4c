/*
 * Host sanitizer run of the oracle (oracle/oracle.c), built with
 * -fsanitize=address,undefined and without OpenMP: tagged round trips in
 * both modes and layouts, the one-element form against the element loop,
 * and the rejected arguments.  Exit status 0 when every check holds.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_seq_to_head(int mode, int64_t G, int layout, int64_t N, int64_t B, int64_t S, int64_t H,
                    int64_t d, int64_t es, const void *in, void *out, int64_t *traffic, int threads);
int orc_head_to_seq(int mode, int64_t G, int layout, int64_t N, int64_t B, int64_t S, int64_t H,
                    int64_t d, int64_t es, const void *in, void *out, int64_t *traffic, int threads);
int orc_source_index(int direction, int mode, int64_t G, int layout, int64_t N, int64_t B, int64_t S,
                     int64_t H, int64_t d, const int64_t *dst, int64_t *src, int64_t n);

static int failures = 0;
#define EXPECT(c) do { if (!(c)) { printf("FAIL line %d: %s\n", __LINE__, #c); ++failures; } } while (0)

static void round_trip(int mode, int64_t G, int layout, int64_t N, int64_t B, int64_t S, int64_t H,
                       int64_t d)
{
    const int64_t n = B * S * H * d;
    int32_t *x = malloc(sizeof(int32_t) * n), *y = malloc(sizeof(int32_t) * n),
            *z = malloc(sizeof(int32_t) * n);
    int64_t *dst = malloc(sizeof(int64_t) * n), *src = malloc(sizeof(int64_t) * n);
    int64_t *tm = calloc((size_t)(N * N), sizeof(int64_t));
    for (int64_t i = 0; i < n; ++i) {
        x[i] = (int32_t)i;
        dst[i] = i;
    }
    EXPECT(orc_seq_to_head(mode, G, layout, N, B, S, H, d, 4, x, y, tm, 1) == 0);
    EXPECT(orc_head_to_seq(mode, G, layout, N, B, S, H, d, 4, y, z, NULL, 1) == 0);
    EXPECT(memcmp(x, z, sizeof(int32_t) * n) == 0);
    EXPECT(orc_source_index(0, mode, G, layout, N, B, S, H, d, dst, src, n) == 0);
    for (int64_t i = 0; i < n; ++i)   /* seq -> head: y[i] is read from x[src[i]] = src[i] */
        EXPECT(src[i] == y[i]);
    EXPECT(orc_source_index(1, mode, G, layout, N, B, S, H, d, dst, src, n) == 0);
    for (int64_t i = 0; i < n; ++i)   /* head -> seq: z[i] is read from y[src[i]] */
        EXPECT(z[i] == y[src[i]]);
    int64_t total = 0;
    for (int64_t i = 0; i < N * N; ++i)
        total += tm[i];
    EXPECT(total == n);
    free(x); free(y); free(z); free(dst); free(src); free(tm);
}

int main(void)
{
    for (int layout = 0; layout < 2; ++layout) {
        round_trip(1, 0, layout, 4, 2, 4 * 7, 8, 3);
        round_trip(0, 0, layout, 6, 3, 6 * 5, 12, 2);
        round_trip(1, 0, layout, 8, 16, 5, 4, 2);    /* data-parallel fallback */
        round_trip(1, 0, layout, 1, 1, 9, 3, 5);
        round_trip(2, 2, layout, 6, 4, 3 * 5, 6, 2); /* G groups: 3 members, 2 sequences each */
        round_trip(2, 4, layout, 8, 16, 2 * 3, 4, 3);
    }
    int32_t buf[16];
    int64_t idx = 1 << 30, out;
    EXPECT(orc_seq_to_head(1, 0, 0, 8, 3, 24, 24, 8, 4, buf, buf, NULL, 1) == -1);   /* N % B */
    EXPECT(orc_seq_to_head(0, 0, 0, 4, 1, 6, 8, 8, 4, buf, buf, NULL, 1) == -1);     /* S % P */
    EXPECT(orc_seq_to_head(0, 0, 2, 4, 1, 8, 8, 8, 4, buf, buf, NULL, 1) == -1);     /* layout */
    EXPECT(orc_seq_to_head(2, 3, 0, 8, 6, 24, 24, 8, 4, buf, buf, NULL, 1) == -1);   /* N % G */
    EXPECT(orc_source_index(0, 1, 0, 0, 2, 2, 2, 2, 2, &idx, &out, 1) == -1);       /* outside */
    printf("%s (%d failures)\n", failures ? "FAILED" : "OK", failures);
    return failures ? 1 : 0;
}
