/*
 * oracle.c -- reference oracle for the BASP / Ulysses attention-boundary
 * re-layout.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file.  Only the tests, the smoke check and the benchmark's CPU
 * baseline leg may use it.  It shares no code, header, table or helper with
 * the HIP path.
 *
 * Source: "BASP: Communication-Efficient Batch-Aware Sequence Parallelism
 * for LLM Training" (Ghimire, Calhoun), as described on
 *   [abs]    the fugumt.com abstract page, "Abstract";
 *   [review] the evolve.pub review page, sections "Summary",
 *            "Key claims under review", "Strengths" and
 *            "Frequently asked questions".
 *
 * What the method fixes:
 *   - Ulysses: all N GPUs take part in one N-way all-to-all
 *     [review, Summary].  Before attention each GPU holds a slice of the
 *     sequence dimension; after it, a slice of the head dimension.
 *   - BASP: N = K*B; the N GPUs form B disjoint groups of K = N/B, each
 *     group owns one sequence and runs its own K-way all-to-all; every GPU
 *     still holds B*S/N tokens [review, Summary; Key claims].
 *   - The ranks of a group are consecutive [review, Summary].
 *   - N must be a multiple of B; the heads must split equally over the
 *     members of a group; with more sequences than GPUs the method reverts to
 *     data parallelism [review, Frequently asked questions].
 *
 * What the pages leave open, and the reading taken here (each is also
 * listed with the other readings of this project):
 *   R1  rank r belongs to group g = r / P at position j = r % P (contiguous
 *       ranks).  Group g owns the sequences [g*Bl, (g+1)*Bl).
 *   R2  position j holds the tokens [j*St, (j+1)*St) of each of its
 *       sequences before attention (St = S/P), and the heads
 *       [j*Hl, (j+1)*Hl) after it (Hl = H/P).
 *   R3  a sequence-sharded shard is [Bl][St][H][d] (activation order); a
 *       head-sharded shard is [Bl][Hl][S][d] ("head-major") or, as an
 *       option, [Bl][S][Hl][d] ("token-major").  The buffer of all N
 *       virtual ranks is the concatenation of the shards in rank order.
 *   R4  B > N (data-parallel fallback): each GPU takes B/N whole sequences
 *       (requires B % N == 0), so G = N, P = 1, Bl = B/N.
 *
 * Scheme constants (the general G-group form of [review, Strengths], the
 * per-GPU work equality of the paper's Sec. IV.C):
 *   Ulysses:          G = 1, P = N,   Bl = B
 *   BASP, B <= N:     G = B, P = N/B, Bl = 1
 *   BASP, B >  N:     G = N, P = 1,   Bl = B/N
 *   G groups:         G,     P = N/G, Bl = B/G   (G divides N and B)
 * The last line is the form the work equality is stated for: G groups of
 * P = N/G GPUs, each group holding B/G of the sequences, so that every GPU
 * holds (B/G) sequences x (S*G/N) tokens x H heads x d channels whatever G
 * is.  The two schemes are its cases G = 1 and G = B.
 *
 * The re-layout moves elements without changing them (model accuracy is
 * unchanged, [abs, Abstract]), so the oracle copies raw bytes of es bytes
 * each; no floating point is involved anywhere.
 *
 * Every function walks the destination buffer element by element and reads
 * the one source element the definitions name.  The optional OpenMP pragma
 * only splits the outer destination loops between threads.
 */
#include <stdint.h>
#include <string.h>

enum { ORC_ULYSSES = 0, ORC_BASP = 1, ORC_GROUPS = 2 };
enum { ORC_HEAD_MAJOR = 0, ORC_TOKEN_MAJOR = 1 };

/* Group structure of the schemes, see the header comment.  G_req is the
 * number of groups of ORC_GROUPS (ignored by the other modes).
 * Returns 0, or -1 when the pages' conditions do not hold. */
int orc_groups(int mode, int64_t G_req, int64_t N, int64_t B, int64_t *G, int64_t *P, int64_t *Bl)
{
    if (N <= 0 || B <= 0)
        return -1;
    if (mode == ORC_GROUPS) {
        /* G groups of N/G consecutive ranks, each owning B/G sequences */
        if (G_req <= 0 || N % G_req != 0 || B % G_req != 0)
            return -1;
        *G = G_req;
        *P = N / G_req;
        *Bl = B / G_req;
        return 0;
    }
    if (mode == ORC_ULYSSES) {
        *G = 1;
        *P = N;
        *Bl = B;
        return 0;
    }
    if (mode != ORC_BASP)
        return -1;
    if (B <= N) {
        if (N % B != 0) /* N = K*B */
            return -1;
        *G = B;
        *P = N / B;
        *Bl = 1;
        return 0;
    }
    if (B % N != 0) /* R4 */
        return -1;
    *G = N;
    *P = 1;
    *Bl = B / N;
    return 0;
}

/* Shared argument check: the group structure exists, tokens and heads split
 * evenly over the P members of a group, and sizes are sane. */
static int check(int mode, int64_t G_req, int layout, int64_t N, int64_t B, int64_t S,
                 int64_t H, int64_t d, int64_t es, int64_t *G, int64_t *P, int64_t *Bl)
{
    if (orc_groups(mode, G_req, N, B, G, P, Bl) != 0)
        return -1;
    if (layout != ORC_HEAD_MAJOR && layout != ORC_TOKEN_MAJOR)
        return -1;
    if (S < 0 || H <= 0 || d <= 0)
        return -1;
    if (es != 1 && es != 2 && es != 4 && es != 8)
        return -1;
    if (S % *P != 0 || H % *P != 0)
        return -1;
    return 0;
}

/* R3: element offset of (rank r, local sequence bl, local token t, head h,
 * channel e) in a sequence-sharded buffer. */
static int64_t seq_offset(int64_t r, int64_t bl, int64_t t, int64_t h, int64_t e,
                          int64_t Bl, int64_t St, int64_t H, int64_t d)
{
    return (((r * Bl + bl) * St + t) * H + h) * d + e;
}

/* R3: element offset of (rank r, local sequence bl, local head hl, token s,
 * channel e) in a head-sharded buffer. */
static int64_t head_offset(int layout, int64_t r, int64_t bl, int64_t hl, int64_t s,
                           int64_t e, int64_t Bl, int64_t Hl, int64_t S, int64_t d)
{
    if (layout == ORC_TOKEN_MAJOR)
        return (((r * Bl + bl) * S + s) * Hl + hl) * d + e;
    return (((r * Bl + bl) * Hl + hl) * S + s) * d + e;
}

static void copy_element(void *dst, int64_t di, const void *src, int64_t si, int64_t es)
{
    memcpy((char *)dst + di * es, (const char *)src + si * es, (size_t)es);
}

/*
 * seq -> head for one tensor of H heads (Q, K, V or dO).
 *
 * For destination rank r = (g, j), local sequence bl, local head hl, token s:
 * the head is h = j*Hl + hl (R2), the token s sits on group member s / St at
 * local position s % St (R2), and that member is rank g*P + s/St (R1).
 *
 * traffic, if not NULL, is an N x N row-major matrix of element counts,
 * traffic[src_rank * N + dst_rank]; it is filled with one thread.
 * Returns 0, or -1 on invalid arguments.
 */
int orc_seq_to_head(int mode, int64_t G_req, int layout, int64_t N, int64_t B, int64_t S,
                    int64_t H, int64_t d, int64_t es, const void *in, void *out,
                    int64_t *traffic, int threads)
{
    int64_t G, P, Bl;
    if (check(mode, G_req, layout, N, B, S, H, d, es, &G, &P, &Bl) != 0)
        return -1;
    const int64_t St = S / P, Hl = H / P;
    if (traffic)
        threads = 1;
    if (threads < 1)
        threads = 1;
    (void)G;

#pragma omp parallel for collapse(3) schedule(static) num_threads(threads)
    for (int64_t r = 0; r < N; ++r)
        for (int64_t bl = 0; bl < Bl; ++bl)
            for (int64_t hl = 0; hl < Hl; ++hl) {
                const int64_t g = r / P, j = r % P;
                const int64_t h = j * Hl + hl;
                for (int64_t s = 0; s < S; ++s) {
                    const int64_t src_rank = g * P + s / St;
                    const int64_t t = s % St;
                    for (int64_t e = 0; e < d; ++e)
                        copy_element(out, head_offset(layout, r, bl, hl, s, e, Bl, Hl, S, d),
                                     in, seq_offset(src_rank, bl, t, h, e, Bl, St, H, d), es);
                    if (traffic)
                        traffic[src_rank * N + r] += d;
                }
            }
    return 0;
}

/*
 * head -> seq for one tensor of H heads (O, dQ, dK or dV): the inverse
 * exchange, back to sequence shards.
 *
 * For destination rank r = (g, j), local sequence bl, local token t, head h:
 * the token is s = j*St + t (R2), the head h sits on group member h / Hl at
 * local head h % Hl (R2), and that member is rank g*P + h/Hl (R1).
 */
int orc_head_to_seq(int mode, int64_t G_req, int layout, int64_t N, int64_t B, int64_t S,
                    int64_t H, int64_t d, int64_t es, const void *in, void *out,
                    int64_t *traffic, int threads)
{
    int64_t G, P, Bl;
    if (check(mode, G_req, layout, N, B, S, H, d, es, &G, &P, &Bl) != 0)
        return -1;
    const int64_t St = S / P, Hl = H / P;
    if (traffic)
        threads = 1;
    if (threads < 1)
        threads = 1;
    (void)G;

#pragma omp parallel for collapse(3) schedule(static) num_threads(threads)
    for (int64_t r = 0; r < N; ++r)
        for (int64_t bl = 0; bl < Bl; ++bl)
            for (int64_t t = 0; t < St; ++t) {
                const int64_t g = r / P, j = r % P;
                const int64_t s = j * St + t;
                for (int64_t h = 0; h < H; ++h) {
                    const int64_t src_rank = g * P + h / Hl;
                    const int64_t hl = h % Hl;
                    for (int64_t e = 0; e < d; ++e)
                        copy_element(out, seq_offset(r, bl, t, h, e, Bl, St, H, d),
                                     in, head_offset(layout, src_rank, bl, hl, s, e, Bl, Hl, S, d), es);
                    if (traffic)
                        traffic[src_rank * N + r] += d;
                }
            }
    return 0;
}

/*
 * The same two rules, one destination element at a time: for each of the n
 * destination element offsets dst[i] of a one-tensor call, src[i] receives
 * the source element offset the element is read from.  For checks of sampled
 * outputs where the whole loop is too large.  Returns 0, or -1 on invalid
 * arguments or an offset outside the tensor.
 */
int orc_source_index(int direction, int mode, int64_t G_req, int layout, int64_t N, int64_t B,
                     int64_t S, int64_t H, int64_t d, const int64_t *dst, int64_t *src, int64_t n)
{
    int64_t G, P, Bl;
    if (check(mode, G_req, layout, N, B, S, H, d, 2, &G, &P, &Bl) != 0)
        return -1;
    (void)G;
    const int64_t St = S / P, Hl = H / P, total = B * S * H * d;
    for (int64_t i = 0; i < n; ++i) {
        int64_t x = dst[i];
        if (x < 0 || x >= total)
            return -1;
        const int64_t e = x % d;
        x /= d;
        if (direction == 0) {
            /* seq -> head: x enumerates (r, bl, hl, s) or (r, bl, s, hl) */
            int64_t s, hl;
            if (layout == ORC_TOKEN_MAJOR) {
                hl = x % Hl;
                x /= Hl;
                s = x % S;
                x /= S;
            } else {
                s = x % S;
                x /= S;
                hl = x % Hl;
                x /= Hl;
            }
            const int64_t bl = x % Bl, r = x / Bl;
            const int64_t g = r / P, j = r % P;
            src[i] = seq_offset(g * P + s / St, bl, s % St, j * Hl + hl, e, Bl, St, H, d);
        } else {
            /* head -> seq: x enumerates (r, bl, t, h) */
            const int64_t h = x % H;
            x /= H;
            const int64_t t = x % St;
            x /= St;
            const int64_t bl = x % Bl, r = x / Bl;
            const int64_t g = r / P, j = r % P;
            src[i] = head_offset(layout, g * P + h / Hl, bl, h % Hl, j * St + t, e, Bl, Hl, S, d);
        }
    }
    return 0;
}

/* Number of OpenMP threads a parallel region would get (1 without OpenMP). */
int orc_max_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
