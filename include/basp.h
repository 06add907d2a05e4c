/*
 * basp.h -- C ABI of libbasp: the attention-boundary re-layout of Ulysses
 * sequence parallelism and of BASP (Batch-Aware Sequence Parallelism) for
 * one MI355X (gfx950), with all N virtual ranks in one device allocation.
 *
 * Method: "BASP: Communication-Efficient Batch-Aware Sequence Parallelism
 * for LLM Training" (Ghimire, Calhoun).  Citations below name the evolve.pub
 * review page of the paper ("review") and the fugumt.com abstract page
 * ("abstract"), with the section on that page.
 *
 * ---------------------------------------------------------------------------
 * What is computed
 * ---------------------------------------------------------------------------
 * N ranks share the attention of B sequences of S tokens, H heads, d channels.
 *
 *   Ulysses:  one N-way exchange for the whole batch            [review, Summary]
 *             G = 1 group, P = N members, Bl = B sequences per group.
 *   BASP:     N = K*B ranks in B disjoint groups of K = N/B, each group owns
 *             one sequence and exchanges K-way; every rank keeps B*S/N tokens
 *                                             [review, Summary; Key claims]
 *             G = B, P = K, Bl = 1.  With more sequences than ranks (B > N)
 *             the method reverts to data parallelism [review, Frequently asked
 *             questions]: G = N, P = 1, Bl = B/N (B a multiple of N).
 *   G groups: the general form in which the per-GPU work (B/G)*H*(S*G/N)*d
 *             is the same for every G [review, Strengths; paper Sec. IV.C]:
 *             G groups of P = N/G ranks, each owning Bl = B/G sequences (G
 *             divides N and B).  G = 1 is Ulysses, G = B is BASP, G = N is
 *             the data-parallel fallback.
 *
 * Rank r is member j = r % P of group g = r / P (groups of consecutive ranks,
 * [review, Summary]); group g owns sequences [g*Bl, (g+1)*Bl).  Member j holds
 * the tokens [j*St, (j+1)*St), St = S/P, before attention and the heads
 * [j*Hl, (j+1)*Hl), Hl = H/P, after it (heads split evenly over the members,
 * [review, Frequently asked questions]).
 *
 * Memory layouts (element order; a buffer is the concatenation of the N rank
 * shards in rank order, one allocation):
 *   sequence-sharded   rank shard [Bl][St][H][d]
 *   head-sharded       rank shard [Bl][Hl][S][d]   (BASP_LAYOUT_HEAD_MAJOR)
 *                      rank shard [Bl][S][Hl][d]   (BASP_LAYOUT_TOKEN_MAJOR)
 * For BASP with B <= N the sequence-sharded buffer is exactly the global
 * [B][S][H][d] tensor.
 *
 * The re-layout copies elements bit for bit (model accuracy is unchanged,
 * [abstract, Abstract]): only the element size matters, values are never
 * interpreted, so NaN payloads, signed zeros and subnormals pass unchanged.
 *
 * ---------------------------------------------------------------------------
 * Conventions common to every call
 * ---------------------------------------------------------------------------
 * - Pointers named q, k, v, o, in, out, dq, dk, dv, ws are DEVICE pointers on
 *   the current HIP device; the caller allocates and owns them.  The library
 *   keeps no device memory or pointers after a call.  Only basp_plan_autotune
 *   allocates device memory, for its own duration (below).
 * - stream is a hipStream_t passed as void*; NULL is the null stream.  Every
 *   call that launches work is asynchronous on that stream and does not
 *   synchronise.
 * - A plan is host memory.  The re-layout and query calls only read it and
 *   may use one plan from several threads and streams at once.  The calls
 *   that change its launch shape (basp_plan_set_tuning,
 *   basp_plan_set_direction_tuning, basp_plan_autotune) must not overlap any
 *   other call on the same plan.
 * - Every call returns a basp_status (0 = BASP_OK) and also stores it for
 *   basp_last_error() in the calling thread.  Calls that return a pointer
 *   return NULL on error.
 * - Pointer checks made before any launch: a NULL pointer to a non-empty
 *   buffer is BASP_ERR_INVALID; a pointer not aligned to the element size is
 *   BASP_ERR_ALIGN; an output range overlapping an input range, or another
 *   output range, is BASP_ERR_ALIAS.  Inputs may overlap each other.  A row
 *   size d*elem_size that is a multiple of 16 bytes lets the kernels use
 *   16-byte accesses (8, 4 or 2 bytes otherwise), at any element-aligned
 *   address; buffers that start on a 16-byte boundary are faster, since
 *   their rows do not straddle cache lines.  The result is the same.
 * - A launch failure reported by the HIP runtime is BASP_ERR_HIP.
 * - With S = 0 every buffer is empty: calls check the plan and return
 *   BASP_OK without touching memory (pointers may then be NULL).
 */
#ifndef BASP_H
#define BASP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum basp_status {
    BASP_OK = 0,
    BASP_ERR_INVALID = 1,     /* NULL plan/pointer, size <= 0, unknown enum   */
    BASP_ERR_INDIVISIBLE = 2, /* N % B, B % N (B > N), S % P or H % P != 0    */
    BASP_ERR_UNSUPPORTED = 3, /* sizes beyond the library's index limits     */
    BASP_ERR_ALIGN = 4,       /* pointer not aligned to the element size     */
    BASP_ERR_ALIAS = 5,       /* an output overlaps an input or an output    */
    BASP_ERR_HIP = 6          /* the HIP runtime reported an error           */
} basp_status;

typedef enum basp_dtype {
    BASP_BF16 = 0,  /* 2 bytes */
    BASP_FP16 = 1,  /* 2 bytes */
    BASP_FP32 = 2,  /* 4 bytes */
    BASP_INT32 = 3  /* 4 bytes */
} basp_dtype;

typedef enum basp_mode {
    BASP_MODE_ULYSSES = 0, /* one N-way group                              */
    BASP_MODE_BASP = 1,    /* B groups of K = N/B (or data parallel, B > N) */
    BASP_MODE_GROUPS = 2   /* G groups given explicitly (basp_plan_create_groups;
                              reported by basp_plan_query, not accepted by
                              basp_plan_create / basp_plan_create_ex)       */
} basp_mode;

typedef enum basp_layout {
    BASP_LAYOUT_HEAD_MAJOR = 0, /* head shard [Bl][Hl][S][d] (default)  */
    BASP_LAYOUT_TOKEN_MAJOR = 1 /* head shard [Bl][S][Hl][d]            */
} basp_layout;

typedef struct basp_plan basp_plan;

/* Everything a caller needs to size buffers and to account for traffic.
 * Element counts are in elements, byte counts in bytes.  Where a field is a
 * count the pages state, the passage is named beside it; the others are
 * sizes that follow from the layouts above.
 *
 *   tokens_per_rank     B*S/N tokens stay on every rank in both schemes
 *                       [review, Summary; Frequently asked questions]
 *   peers_per_rank      the ranks a rank exchanges with, itself excluded:
 *                       K-1 under BASP against N-1 under Ulysses
 *                       [review, Summary]
 *   q_elems_per_rank,   the per-rank work (B/G)*H*(S*G/N)*d, equal for every
 *   kv_elems_per_rank   number of groups G [review, Strengths; paper Sec. IV.C]
 *   per_peer_bytes_*    one member's chunk for one other member of its group:
 *                       Bl sequences x St tokens x Hl heads x d channels
 *   cross_rank_bytes_*  bytes that leave their rank in the group exchange
 *                       [review, Summary]: every rank receives P chunks, P-1 of
 *                       them from other ranks, so (P-1)/P of each tensor
 *   tokens_per_rank_foil  tokens per rank of the alternative the pages set
 *                       BASP against, plain Ulysses over groups of N/B ranks
 *                       that each hold the whole micro-batch: B*B*S/N
 *                       [review, Strengths; paper Sec. IV.E, Table I].  0 when
 *                       N/B is not a whole number (no such configuration).
 */
typedef struct basp_plan_info {
    int32_t N, B, Hq, Hkv, d, elem_size;
    int64_t S;
    int32_t mode, layout, dtype;
    int32_t G, P, Bl;             /* groups, members per group, sequences per group */
    int64_t St;                   /* tokens per rank and sequence, S/P             */
    int32_t Hl_q, Hl_kv;          /* heads per rank, Hq/P and Hkv/P                */
    int64_t tokens_per_rank;      /* Bl*St = B*S/N                                 */
    int32_t peers_per_rank;       /* ranks exchanged with, self excluded: P-1      */
    int64_t q_elems, kv_elems;    /* elements of Q (= O) and of K (= V), all ranks */
    int64_t q_elems_per_rank, kv_elems_per_rank;
    int64_t qkv_elems;            /* q_elems + 2*kv_elems: the fused buffer        */
    int64_t qkv_offset_q, qkv_offset_k, qkv_offset_v; /* element offsets in it   */
    int64_t per_peer_bytes_q, per_peer_bytes_kv;   /* Bl*St*Hl*d*elem_size        */
    int64_t cross_rank_bytes_q, cross_rank_bytes_kv; /* (P-1)/P of each tensor    */
    int64_t qkv_bytes_moved;      /* 2*(q_elems + 2*kv_elems)*elem_size            */
    int64_t o_bytes_moved;        /* 2*q_elems*elem_size                           */
    int64_t tokens_per_rank_foil; /* B*B*S/N, or 0 (see above)                     */
} basp_plan_info;

/*
 * Create a plan.  Host only: no device call, no device memory.
 *   N    virtual ranks (>= 1)           B    sequences in the micro-batch (>= 1)
 *   S    tokens per sequence (>= 0)     Hq   query/output heads (>= 1)
 *   Hkv  key/value heads (>= 1; Hkv < Hq is grouped-query attention, each
 *        tensor is re-laid with its own head count, no head replication)
 *   d    channels per head (>= 1)       dtype, mode as above
 * Errors (NULL returned, code in basp_last_error()):
 *   BASP_ERR_INVALID      an argument out of range or an unknown enum
 *   BASP_ERR_INDIVISIBLE  BASP with B <= N and N % B != 0 [review, Summary];
 *                         BASP with B > N and B % N != 0; S % P, Hq % P or
 *                         Hkv % P != 0 [review, Frequently asked questions]
 *   BASP_ERR_UNSUPPORTED  a buffer of more than 2^62 bytes, a tensor of
 *                         2^32 or more (token, head) rows (B*S*max(Hq, Hkv)),
 *                         B above 65535 (the launch grid's z extent), or more
 *                         than 2^31 - 1 work tiles per (group member, batch
 *                         index) in one launch
 * basp_plan_create uses BASP_LAYOUT_HEAD_MAJOR.
 */
basp_plan *basp_plan_create(int N, int B, int64_t S, int Hq, int Hkv, int d,
                            basp_dtype dtype, basp_mode mode);
basp_plan *basp_plan_create_ex(int N, int B, int64_t S, int Hq, int Hkv, int d,
                               basp_dtype dtype, basp_mode mode, basp_layout layout);

/*
 * Create a plan of the general G-group form (see "What is computed"): G
 * groups of N/G consecutive ranks, group g owning the sequences
 * [g*B/G, (g+1)*B/G) [review, Strengths; paper Sec. IV.C].  Other arguments
 * and the host-only contract as for basp_plan_create_ex; the plan's mode is
 * BASP_MODE_GROUPS.  Errors (NULL returned, code in basp_last_error()):
 *   BASP_ERR_INVALID      G < 1, or as for basp_plan_create_ex
 *   BASP_ERR_INDIVISIBLE  N % G or B % G != 0; S, Hq or Hkv not a multiple of
 *                         the group size N/G
 *   BASP_ERR_UNSUPPORTED  as for basp_plan_create_ex
 */
basp_plan *basp_plan_create_groups(int N, int B, int64_t S, int Hq, int Hkv, int d,
                                   basp_dtype dtype, int G, basp_layout layout);

/* Free a plan.  NULL is allowed.  (Host resource management: not a step of
 * the method.) */
void basp_plan_destroy(basp_plan *plan);

/* Fill *info with the plan's group structure, sizes and exchange counts
 * (fields and their passages at basp_plan_info).  Host only.
 * BASP_ERR_INVALID if plan or info is NULL. */
basp_status basp_plan_query(const basp_plan *plan, basp_plan_info *info);

/*
 * Fused Q/K/V seq -> head: the exchange before attention, for the three
 * tensors in one launch [review, Summary; Scope & Claims].
 *   q    sequence-sharded, q_elems elements  (Hq heads)
 *   k, v sequence-sharded, kv_elems elements each (Hkv heads)
 *   out  qkv_elems elements: head-sharded Q, then head-sharded K, then
 *        head-sharded V, at element offsets qkv_offset_q/_k/_v.  The Q part
 *        is itself a valid head-sharded O for basp_head_to_seq.
 */
basp_status basp_seq_to_head(const basp_plan *plan, const void *q, const void *k,
                             const void *v, void *out, void *stream);

/*
 * O head -> seq: the exchange after attention, the inverse of the Q part of
 * basp_seq_to_head [review, Scope & Claims: the attention-phase all-to-all].
 *   o    head-sharded, q_elems elements (Hq heads)
 *   out  sequence-sharded, q_elems elements
 */
basp_status basp_head_to_seq(const basp_plan *plan, const void *o, void *out, void *stream);

/*
 * Backward pass of the same boundary (training, [abstract, Abstract]):
 * the gradient of head -> seq is seq -> head and the reverse.
 *
 * basp_seq_to_head_o: dO sequence-sharded (q_elems, Hq heads) -> head-sharded
 *   (q_elems).  Same mapping as the Q part of basp_seq_to_head.
 * basp_head_to_seq_qkv: fused dQ/dK/dV head -> seq, the exact inverse of
 *   basp_seq_to_head.  in holds qkv_elems elements laid out as that call's
 *   out; dq (q_elems), dk and dv (kv_elems each) receive sequence-sharded
 *   gradients.  dq, dk, dv must not overlap in or each other.
 */
basp_status basp_seq_to_head_o(const basp_plan *plan, const void *dout, void *out,
                               void *stream);
basp_status basp_head_to_seq_qkv(const basp_plan *plan, const void *in, void *dq, void *dk,
                                 void *dv, void *stream);

/*
 * Unfused three-pass seq -> head, kept as an internal baseline: the group
 * all-to-all of the pages [review, Summary] written out as the collective a
 * communication library runs, (1) pack each rank's shard by destination
 * member, (2) exchange the per-peer chunks, (3) unpack into the head-sharded
 * layout.
 * Same inputs and output as basp_seq_to_head (bit-identical result), three
 * times the memory traffic.
 *   ws   device workspace of basp_unfused_workspace_bytes(plan) bytes, owned by
 *        the caller, aligned like the inputs; its contents on return are
 *        unspecified.  It must not overlap any input or out (BASP_ERR_ALIAS).
 * Each tensor must be smaller than 2 GiB here (BASP_ERR_UNSUPPORTED otherwise).
 * basp_unfused_workspace_bytes returns 0 for a NULL plan.
 */
size_t basp_unfused_workspace_bytes(const basp_plan *plan);
basp_status basp_seq_to_head_unfused(const basp_plan *plan, const void *q, const void *k,
                                     const void *v, void *out, void *ws, void *stream);

/*
 * basp_seq_to_head_unfused for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same inputs, output, kernels and result; the workspace is an
 * array of BASP_NOALLOC_SCRATCH_BYTES bytes that the library holds on each
 * device it runs this call on, until the process ends.  The call allocates
 * and frees nothing; on its first call on a device it looks up that device's
 * copy of the array.
 *   Limit: plans with basp_unfused_workspace_bytes(plan) above
 *   BASP_NOALLOC_SCRATCH_BYTES are rejected with BASP_ERR_UNSUPPORTED before
 *   any device call (the Q, K and V together may hold at most half of it).
 *   Sharing: every call on one device uses that device's one array, so calls
 *   that overlap on one device (other streams, other threads) race and give
 *   undefined results; serialise them.  The array keeps the last call's
 *   contents; nothing in it needs to start at zero (every workspace byte a
 *   pass reads was written by the pass before it in the same call).
 * Errors as for basp_seq_to_head_unfused; BASP_ERR_HIP when the runtime cannot
 * name the current device or the array's address on it.
 */
#define BASP_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
basp_status basp_seq_to_head_unfused_noalloc(const basp_plan *plan, const void *q, const void *k,
                                             const void *v, void *out, void *stream);

/*
 * Launch shape of a plan, per direction: BASP_SEQ_TO_HEAD applies to
 * basp_seq_to_head and basp_seq_to_head_o, BASP_HEAD_TO_SEQ to
 * basp_head_to_seq and basp_head_to_seq_qkv (the unfused baseline has a
 * fixed shape).  Zero fields keep the built-in choice, which depends on the
 * row size d*elem_size and on the bytes the call moves (measured on MI355X
 * over the Llama/Qwen attention shapes; listed below the fields).  Results
 * never depend on these values, only the speed does.
 *   vectors_per_thread   1, 2, 4 or 8 (16-byte vectors held in flight per
 *                        lane)
 *   tile_tokens          tokens per work tile (>= 1; built-in: one pass of
 *                        the work-group)
 *   tile_heads           heads per work tile (>= 1, clamped to H/P)
 *   cache_policy         1 = plain loads and stores, 2 = non-temporal stores,
 *                        3 = non-temporal loads and stores, 4 = non-temporal
 *                        loads, non-temporal device-scope stores (gfx950
 *                        NT + SC1; built-in), 5 = non-temporal system-scope
 *                        loads and stores (NT + SC0 + SC1)
 *   max_grid             cap on work-groups along x, the tiles of one
 *                        (group member, batch index) pair (tiles loop beyond it)
 *   lane_order           1 = lanes run along tokens first, 2 = along heads
 *                        first
 *   xcd_remap            1 = tiles in work-group order, 2 = each of the 8
 *                        XCDs takes one contiguous eighth of the tiles of a
 *                        (group member, batch index) pair
 *   tile_order           1 = token blocks fastest (the head-sharded side's
 *                        order), 2 = head blocks fastest (the sequence-sharded
 *                        side's order), 3 = token blocks fastest within one
 *                        source member's token chunk, that member's tiles of
 *                        the neighbouring heads next
 *   stage                1 = rows go straight from load to store registers
 *                        (built-in),
 *                        2 = each tile passes through LDS: loads
 *                        run along the source's contiguous axis, stores along
 *                        the destination's (used with 16-byte vectors and
 *                        tiles of one pass of the work-group)
 *   block_size           threads per work-group: 64, 128 or 256
 *   batch_order          1 = the batch indices one after another (built-in),
 *                        2 = batch indices interleaved with the tiles, so
 *                        that neighbouring work-groups alternate sequences
 * Built-in choices of the fields that depend on the call (a call's bytes
 * being what it reads plus what it writes):
 *   calls above 32 MiB with rows of at most 128 bytes, and above 160 MiB
 *   with longer rows: 256 threads, 1 vector per lane, 8 heads per tile for
 *   rows of at most 128 bytes and 1 for longer ones, tile order 2, lanes
 *   along heads, tiles in work-group order;
 *   smaller calls with rows of at most 128 bytes: 128 threads, 2 vectors
 *   per lane, 4 heads per tile, tile order 3, lanes along tokens, XCD
 *   remap;
 *   smaller calls with longer rows: as for large calls, with tile order 1.
 * vectors_per_thread and block_size apply to 16-byte vectors; rows that
 * need narrower vectors run 256 threads with 4 vectors each.
 * basp_plan_set_tuning sets both directions, basp_plan_set_direction_tuning
 * one; basp_plan_get_tuning reads one.  Errors: BASP_ERR_INVALID on a NULL
 * argument, an unknown direction or an out-of-range field;
 * BASP_ERR_UNSUPPORTED when the shape exceeds the index limits.  A plan's
 * tuning must not change while another thread launches with it.
 */
typedef enum basp_direction {
    BASP_SEQ_TO_HEAD = 0,
    BASP_HEAD_TO_SEQ = 1
} basp_direction;

typedef struct basp_tuning {
    int32_t vectors_per_thread;
    int32_t tile_tokens;
    int32_t tile_heads;
    int32_t cache_policy;
    int32_t max_grid;
    int32_t lane_order;
    int32_t xcd_remap;
    int32_t tile_order;
    int32_t stage;
    int32_t block_size;
    int32_t batch_order;
} basp_tuning;
basp_status basp_plan_set_tuning(basp_plan *plan, const basp_tuning *tuning);
basp_status basp_plan_set_direction_tuning(basp_plan *plan, basp_direction dir,
                                           const basp_tuning *tuning);
basp_status basp_plan_get_tuning(const basp_plan *plan, basp_direction dir, basp_tuning *tuning);

/*
 * Choose the launch shape of both directions by measurement on the caller's
 * buffers (as a planner that times candidates).  A fixed set of launch
 * shapes (larger when the fused seq->head call moves at most 64 MiB: 4 and
 * 8 vectors per lane as well as 1 and 2) is timed for seq->head on
 * (q, k, v -> qkv) and for head->seq on (o -> o_out), in rounds that
 * alternate the two directions, each timed launch right after an untimed
 * launch of the other direction with the plan's shape on entry (as the two
 * run back to back in a step).  The best three shapes of each direction (six
 * on the timing pool described below) are then paired, and every pair is
 * timed as whole back-to-back steps, together with the pair of the plan's
 * shapes on entry.  The pair with the lowest
 * median step time is stored in the plan, replacing its tuning (the shapes
 * on entry stay when they win).  The buffers are those of basp_seq_to_head
 * and basp_head_to_seq, with the same checks, and because the two calls run
 * back to back the six are also checked together: qkv and o_out must not
 * overlap any of q, k, v, o or each other (BASP_ERR_ALIAS, before any
 * launch).  Every candidate computes the
 * same re-layout, so on BASP_OK qkv and o_out hold the results of the two
 * calls.  Runs on stream and waits for it; creates and destroys HIP events.
 * When the six buffers together are smaller than 32 MiB, they fit in the
 * device's caches and the timed launches would run from there, where other
 * shapes win than in a loop of calls that streams from HBM; the timed
 * launches then rotate over buffers of the same sizes in a temporary pool of
 * about 1 GiB (up to 256 sets), allocated with hipMalloc and freed before the
 * call returns, the pairs are timed from HIP graphs on a private stream
 * (created and destroyed in the call; they touch only the pool), and the
 * chosen shapes run once more on the caller's buffers at the end.  If the
 * pool cannot be allocated, the caller's buffers are timed alone.  Larger
 * calls are timed on the caller's buffers, whose placement some shapes'
 * speed depends on.  A pending basp_time_next_call request is
 * dropped.  Errors as for the two calls; on BASP_ERR_HIP the plan keeps its
 * previous tuning.  The plan must not be used by another thread meanwhile.
 */
basp_status basp_plan_autotune(basp_plan *plan, const void *q, const void *k, const void *v,
                               void *qkv, const void *o, void *o_out, void *stream);

/*
 * Kernel timing without extra work on the stream.  The next call of this
 * thread that launches kernels records start_event when its first kernel
 * begins and stop_event when its last kernel ends, from the kernels' own
 * dispatch timestamps (hipExtLaunchKernel).  The events are hipEvent_t
 * handles passed as void*, created by the caller on the current device; either
 * may be NULL.  The request applies to exactly one call (also one that fails
 * or launches nothing) and is then cleared.  Returns BASP_OK.
 */
basp_status basp_time_next_call(void *start_event, void *stop_event);

/*
 * Plain device copy of bytes bytes from src to dst, with the access rules of
 * the re-layout kernels: 16-byte buffer loads and stores, non-temporal loads
 * and non-temporal device-scope stores, one wave of 64 lanes per work-group.
 * It is not part of the method.  It is the simplest kernel that reads every
 * byte once and writes every byte once, so its rate at the same byte count
 * is the ceiling a re-layout call is measured against.
 *   src, dst  device pointers, 16-byte aligned, owned by the caller; they
 *             may be NULL when bytes is 0
 *   bytes     a multiple of 16, at most 2^56
 * Asynchronous on stream, no allocation; basp_time_next_call applies to it.
 * Errors: BASP_ERR_INVALID (NULL pointer with bytes > 0), BASP_ERR_ALIGN
 * (pointer or size not a multiple of 16), BASP_ERR_ALIAS (the two ranges
 * overlap), BASP_ERR_UNSUPPORTED (bytes above 2^56), BASP_ERR_HIP.
 */
basp_status basp_stream_copy(void *dst, const void *src, uint64_t bytes, void *stream);

/* Status of the last call made by this thread, and a static description.
 * (Error reporting: not a step of the method.) */
basp_status basp_last_error(void);
const char *basp_status_str(basp_status status);

#ifdef __cplusplus
}
#endif

#endif /* BASP_H */
