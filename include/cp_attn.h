/*
 * cp_attn.h -- C ABI of the MI355X (gfx950) zigzag ring context-parallel
 * attention library, libcpattn.so.
 *
 * What the library computes.  One context-parallel (CP) rank's exact softmax
 * attention over its share of a long sequence, the core of context parallelism
 * as described in "Sequence Parallelism IV: Megatron Context Parallel and
 * Load-Balanced Rings" (duoan.github.io):
 *   - the sequence of S tokens is cut into 2*cp chunks and rank r owns chunks
 *     r and 2*cp-1-r (zigzag placement, section 3 "Naive Ring Attention Is
 *     Imbalanced Under Causal Masks"), or the contiguous slice
 *     [r*S/cp, (r+1)*S/cp) (naive placement, same section);
 *   - the rank's queries stay resident while the K/V chunks of every rank pass
 *     by, one source rank per ring step (section 4 "What Actually Moves");
 *   - each step's partial result is folded into a running (O, LSE) state by
 *     log-sum-exp correction, which reproduces the unsplit result (section 4);
 *   - sub-blocks that the causal mask puts entirely in the future are skipped
 *     (section 4);
 *   - the next step's K/V is received while the current step computes
 *     (section 5 "Overlap: More Than One Stream").
 * On one GPU the ring is a step schedule: step 0 reads the rank's own K/V in
 * place, and for s >= 1 the K/V of ring source src(r, s) = (r - s) mod cp is
 * copied device-to-device into one of two receive slots on a side HIP stream
 * while step s-1 computes.
 *
 * Attention semantics (the plain definition the result must equal):
 *   causal: key j is valid for query i iff pos(j) <= pos(i) (global token
 *   positions; the diagonal is valid); bidirectional: every key is valid.
 *   s_ij = <q_i, k_j> / sqrt(head_dim);  O_i = sum_j softmax_j(s_ij) v_j;
 *   LSE_i = ln sum_j exp(s_ij)  (natural log, fp32).
 *
 * Tensor layouts (all device memory, row-major, contiguous):
 *   q, k, v, out : [S][heads][head_dim] in natural token order, element type
 *                  set by cp_attn_set_dtype (bf16 by default);
 *   lse          : [heads][S] fp32.
 * Pointers are device pointers and must be 16-byte aligned.  Streams are HIP
 * streams (hipStream_t) passed as void*; NULL means the null stream.
 *
 * Errors: every call returns a status code (CP_ATTN_OK = 0 or a negative
 * error); nothing is enqueued when argument validation fails; no exception or
 * abort crosses the ABI.  cp_attn_last_error() gives a text for the calling
 * thread's last failure.  A plan is not reentrant: keep at most one forward
 * call per plan in flight, and do not destroy a plan while its work is queued.
 */
#ifndef CP_ATTN_H
#define CP_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct cp_attn_plan_s* cp_attn_plan_t;

/* Status codes. */
#define CP_ATTN_OK 0
#define CP_ATTN_EINVAL (-1)       /* bad argument: sizes, divisibility, rank, null or misaligned pointer */
#define CP_ATTN_EUNSUPPORTED (-2) /* valid request this build does not implement (head_dim, cp_size) */
#define CP_ATTN_ENOWORKSPACE (-3) /* caller workspace missing or too small, or allocation failed */
#define CP_ATTN_EHIP (-4)         /* a HIP runtime call or kernel launch failed */

/* Chunk placement. */
#define CP_ATTN_CONTIGUOUS 0 /* rank r owns tokens [r*L, (r+1)*L), L = ceil(S/cp) */
#define CP_ATTN_ZIGZAG 1     /* rank r owns chunks r and 2*cp-1-r of C = ceil(S/(2*cp)) tokens, early chunk first */

/* Element types of q, k, v and out (lse is always fp32). */
#define CP_ATTN_BF16 0
#define CP_ATTN_FP32 1

/* Options for cp_attn_set_option. */
#define CP_ATTN_OPT_MERGE 1       /* 0: merge fused into the attention epilogue (default);
                                     1: separate LSE-merge kernel on the merge stream + finalize kernel */
#define CP_ATTN_OPT_SERIALIZE 2   /* 0: copy/merge on side streams (default); 1: everything on the caller's stream */
#define CP_ATTN_OPT_RECV 3        /* ring receive of step s+1 while step s computes:
                                     0: the library's copy kernel on the copy stream (default):
                                        one-wave workgroups of 16 VGPRs that run beside the
                                        attention kernel in the registers it leaves free;
                                     1: hipMemcpyAsync on the copy stream;
                                     2: inside step s's attention kernel (bf16 with head_dim
                                        128 only, otherwise as 0);
                                     3: as 0 for step 0 (receive of step 1), then as 2: no
                                        cross-stream event after step 1 */
#define CP_ATTN_OPT_POISON 4      /* 1: fill each receive slot / partial buffer with NaN once consumed */
#define CP_ATTN_OPT_STEP_TIMING 5 /* 1: time every ring step's attention kernel with HIP events (a
                                     fused-ring call's one launch per rank under step 0) */
#define CP_ATTN_OPT_RECV_BLOCKS 6 /* grid bound of the ring-receive copy kernel (0: one workgroup
                                     per 128 vectors of 16 bytes); a small grid shares the GPU with
                                     the attention kernel it overlaps.  -1 (default): automatic,
                                     256 beside a per-step launch, 1024 beside the fused ring's
                                     launch (whose later steps wait for the receives).  A receive that
                                     overlaps no attention kernel (serial order, or a ring step
                                     with no valid pair, e.g. under document masks) always takes
                                     the full grid */
#define CP_ATTN_OPT_GRAPH 7       /* 1: graph mode. A forward call is recorded once into a HIP graph
                                     (stream capture on a library stream) and replayed on the
                                     caller's stream while its buffers, rank, workspace, side streams
                                     and options are unchanged; any change records it again. Replays
                                     read the buffers' current contents. Step timing is not recorded
                                     in this mode (cp_attn_last_step_times reports -1). */
#define CP_ATTN_OPT_KSPLIT 8      /* 1 (default): when a step's workgroups would fill at most half
                                     of the GPU (few heads), the bf16 head_dim-128 kernel splits
                                     each full segment's keys in two halves, one workgroup each;
                                     the part that finishes second merges the other's result
                                     (exact LSE merge; no workgroup waits for another).
                                     0: never split. Not used with the separate merge mode.
                                     In the fused ring (CP_ATTN_OPT_FUSED_RING) the split is
                                     decided per rank when the plan's run table is built: where
                                     an estimate of the launch (workgroups in dispatch order, one
                                     per compute unit, slower per unit as more are busy) comes
                                     out at least 5 % shorter, a segment's row tiles take two
                                     workgroups, one the first half of every step's keys, the
                                     other the second halves and the causal diagonal (chunks of a
                                     multiple of 256 rows whose key runs split into whole 64-key
                                     tiles only). */
#define CP_ATTN_OPT_COUNTERS 9    /* 1: the step kernels count the key tiles they compute per (rank,
                                     step) on the device (cp_attn_last_tile_counts) */
#define CP_ATTN_OPT_BWD_KEYS 10   /* backward dK/dV kernel (bf16, head_dim 128): 0 (default): eight
                                     waves, each 32-key column's products split between two waves;
                                     1: four waves, one wave per 32-key column. dK and dV are
                                     bit-identical either way. */
#define CP_ATTN_OPT_LOCKSTEP 12   /* cp_attn_full_forward: 0 (default): the ranks' shares back to
                                     back; 1: the ranks in lockstep, as a CP group runs a ring
                                     step together: per step, every rank's receive on the copy
                                     stream and one launch of the step kernel over every rank's
                                     tiles (no key split).  Each rank gets its own receive slots
                                     and running state in a library-owned buffer (about
                                     cp x (4 x n_loc x H x D x 2 + n_loc x H x (D + 1) x 4) bytes,
                                     allocated by the first such call, freed with the plan;
                                     ENOWORKSPACE if that allocation fails).  Each rank's result is
                                     bit-identical to its back-to-back result without the key
                                     split.  Served for bf16 head_dim 128 with the fused merge,
                                     the copy-kernel or memcpy receive, and no serial, poison or
                                     step-timing mode (and while K/V span at most 4 GiB);
                                     otherwise, and in graph mode, the ranks run back to back. */
#define CP_ATTN_OPT_FUSED_RING 13 /* 0: one launch of the step kernel per ring step, the running
                                     state stored between them; 1 (default): every ring step of a
                                     rank in one launch, where served (cp_attn_fused_ring_active
                                     tells whether the last call was).  Each row tile takes the keys of all its
                                     steps in turn with its running max and sum in registers (the
                                     exact merge of "Sequence Parallelism IV", section 4, carried
                                     across steps) and writes its output once.  The receives of
                                     steps 1 .. cp-1 still go one by one on the copy stream (section
                                     5, "Overlap: More Than One Stream"), each into a slot of its
                                     own, followed by a one-thread kernel that stores the call's
                                     epoch to the step's device flag; a workgroup polls that flag
                                     (a fraction of a second at most) before it loads any key of the step.
                                     The slots (2 x (cp-1) x n_loc x H x D x 2 bytes), flags and
                                     key-run table are a library-owned allocation made by the first
                                     such call and freed with the plan (ENOWORKSPACE if it fails).
                                     A wait that runs out sets a word that
                                     cp_attn_ring_wait_timeouts reports; that call's results are not
                                     valid.  Results agree with mode 0 to rounding (the merge order
                                     differs).  Served for bf16 head_dim 128, the zigzag and the
                                     contiguous layouts, causal or bidirectional, without padding,
                                     with chunks of whole 64-key tiles (a receive no row of the
                                     rank needs is not made), the
                                     fused merge and the copy-kernel receive (CP_ATTN_OPT_RECV 0),
                                     without documents and the serial, counter and poison modes,
                                     while K/V span at most 4 GiB (graph mode included: each call
                                     advances its epoch on the device, so every replay waits for its
                                     own receives); otherwise, and in the no-allocation forward,
                                     mode 0.
                                     2: as 1, but every wait looks for an epoch no signal stores and
                                     gives up after 16 polls: a test of the time-out path (results
                                     not valid).  3 (staged): as 1, but the caller's stream waits
                                     (HIP event) for every receive before the launch, so no wait is
                                     polled and nothing overlaps: for tools that run one kernel at a
                                     time (counter collection), under which mode 1's waits can only
                                     run out.  Results bit-identical to mode 1. */
#define CP_ATTN_OPT_BWD_FUSED 14  /* backward schedule (bf16, head_dim 128, no documents, no padding,
                                     S x H x D x 2 bytes below 2 GiB; elsewhere 0).  0: per ring
                                     step a dK/dV launch and a dQ launch, dQ stored between steps.
                                     1 (default): dQ of every ring step in one launch: a row's keys
                                     over all steps are one prefix of the natural order (the keys
                                     before its chunk, then its chunk's causal part; every key
                                     without the mask), taken in natural order with dQ in
                                     registers and written once; dK/dV per step as in 0.  2: dK/dV
                                     in one launch as well, over the same prefixes: the all-gather
                                     form of "Context Parallelism in MegaDLMs", "Key-Value
                                     Communication Patterns" (every source's K/V present at once).
                                     Results agree with mode 0 to rounding (summation order). */

/*
 * Create a plan (host only: no device memory, no HIP call).
 *   seq_len  S > 0, tokens of the whole sequence (batch 1);
 *   cp_size  number of CP ranks, 1..256;
 *   heads    > 0 (K/V heads equal query heads);
 *   head_dim 64 or 128;
 *   causal   1 causal, 0 bidirectional;
 *   layout   CP_ATTN_ZIGZAG or CP_ATTN_CONTIGUOUS.
 * Per-rank length is S / cp_size ("Context Parallelism in MegaDLMs", section
 * "Sequence Partitioning Across GPUs").  A length that does not divide into
 * the 2*cp_size (zigzag) or cp_size (contiguous) chunks is padded at the end
 * to the next multiple, S_pad ("Context Parallelism for Long-Context
 * Training", section "Test sequence divisibility and padding"): chunk c holds
 * positions [c*C, (c+1)*C) of the padded sequence, of which those below S are
 * real.  A pad position belongs to the rank owning its chunk; pad keys are
 * never attended and pad queries produce no output, so every real token's
 * result equals that of unpadded attention.  A rank's real rows are the first
 * cp_attn_rank_valid_rows of its local buffer.  The natural-order tensors
 * still hold S rows: pad rows exist only in the local layout.
 * Returns EINVAL for non-positive sizes or a bad flag or layout; EUNSUPPORTED
 * for another head_dim, cp_size > 256, (S_pad / cp_size) * heads * head_dim
 * * 4 >= 2^32 (one rank's rows are addressed with 32-bit offsets), or
 * S_pad >= 2^31.  The natural-order tensors may exceed 4 GiB (beyond that,
 * each rank's first ring step reads its own K/V chunks from a receive slot
 * filled by one extra copy instead of in place).
 * On success *out owns the plan; free it with cp_attn_plan_destroy.
 */
int cp_attn_plan(int64_t seq_len, int cp_size, int heads, int head_dim, int causal, int layout,
                 cp_attn_plan_t* out);

/* Free the plan, its library-owned streams, events and workspace.  Waits for
 * the plan's queued work first.  NULL is accepted. */
int cp_attn_plan_destroy(cp_attn_plan_t plan);

/* Element type of q, k, v, out: CP_ATTN_BF16 (default) or CP_ATTN_FP32. */
int cp_attn_set_dtype(cp_attn_plan_t plan, int dtype);

/* Set one of the CP_ATTN_OPT_* options (values as documented above). */
int cp_attn_set_option(cp_attn_plan_t plan, int option, int value);

/* Bytes of device workspace a forward call needs: two K/V receive slots, the
 * fp32 running state (O, LSE), two fp32 partial buffers (separate merge mode,
 * or the two key halves of a split step), (n_loc/256 + 2) * heads int32
 * split counters and the document table (2 int32 per token), each rounded
 * up to 256 bytes.  Everything but the document table is scratch: a call
 * clears what must start at zero (the split counters, with a fill kernel on
 * its own stream before the first step that splits), so the caller may reuse
 * the memory between calls.  The document table is written once per
 * document list (and again after cp_attn_set_workspace); while documents are
 * set, the caller must not write that region between calls. */
int cp_attn_workspace_bytes(cp_attn_plan_t plan, int64_t* bytes);

/* Whether a receive wait of the fused ring (CP_ATTN_OPT_FUSED_RING) ran out
 * of polls since the last query: *timed_out = 1 if so (the results of the
 * calls since then are not valid), else 0; the word is cleared.  The step
 * kernel sets it in host-visible memory: query after synchronizing the
 * calls' stream.  No device call; EINVAL for a null timed_out. */
int cp_attn_ring_wait_timeouts(cp_attn_plan_t plan, int32_t* timed_out);

/* Whether the plan's last forward call (rank or full) ran each rank it
 * computed as one fused launch (CP_ATTN_OPT_FUSED_RING served): *active = 1,
 * or 2 if the last rank it computed split its row tiles' keys in that launch
 * (CP_ATTN_OPT_KSPLIT); 0: one launch per ring step, or no call yet.  Host
 * only; EINVAL for a null active. */
int cp_attn_fused_ring_active(cp_attn_plan_t plan, int32_t* active);

/* Hand the plan caller-owned device memory of at least cp_attn_workspace_bytes
 * bytes (256-byte aligned); the caller keeps ownership and must keep it alive
 * while the plan uses it.  NULL/0 returns to library-allocated workspace
 * (hipMalloc'd on the first forward call, freed by cp_attn_plan_destroy).
 * ENOWORKSPACE if bytes is too small, EINVAL if misaligned. */
int cp_attn_set_workspace(cp_attn_plan_t plan, void* device_ptr, int64_t bytes);

/* Side streams for the ring receive copies and the separate merge (hipStream_t
 * as void*).  NULL lets the library create and own non-blocking streams of
 * default priority on first use. */
int cp_attn_set_streams(cp_attn_plan_t plan, void* copy_stream, void* merge_stream);

/*
 * Document masks ("Context Parallelism for Long-Context Training", section
 * "Prove attention equivalence": causal and document masks).  The S tokens
 * are cut into `count` documents; document d holds the positions
 * [starts[d], starts[d+1]) and the last one runs to S.  A query then attends
 * only to keys of its own document, on top of the plan's causal or
 * bidirectional mask.  starts: host array, strictly increasing, starts[0] =
 * 0, every entry below S; the plan keeps a copy.  count = 0 removes the
 * documents.  Every forward call (ring, all-gather, Ulysses) and the
 * backward calls honour them.  The device table (two int32 per token, in
 * the workspace) is written by the next forward or backward call, which
 * first waits for the device.  A query row that sees no
 * key of a ring step takes nothing from that step; the key split
 * (CP_ATTN_OPT_KSPLIT) is not used while documents are set.
 * EINVAL for an unsorted list, a first start other than 0, a start >= S, a
 * negative count or a null starts with count > 0.  Host-only.
 */
int cp_attn_set_documents(cp_attn_plan_t plan, const int64_t* starts, int64_t count);

/*
 * One rank's share, asynchronous on `stream`: for s = 0..cp_size-1 the rank's
 * queries attend to the K/V chunks of src(rank, s) = (rank - s) mod cp_size,
 * the next source is received into the other slot while step s computes, and
 * partials are merged exactly.  Writes only the rank's rows of out (token
 * positions owned by `rank`) and the matching columns of lse; inputs are read
 * only.  q, k, v, out: [S][heads][head_dim] plan dtype; lse: [heads][S] fp32.
 * EINVAL for rank outside [0, cp_size) or a null/misaligned pointer;
 * ENOWORKSPACE if workspace allocation fails; EHIP if a launch fails.
 */
int cp_attn_rank_forward(cp_attn_plan_t plan, const void* q, const void* k, const void* v, void* out,
                         float* lse, int rank, void* stream);

/* All-gather variant of one rank's share ("Context Parallelism in MegaDLMs",
 * section "Key-Value Communication Patterns": the all_gather communication
 * type, where every rank first collects the K/V of the whole sequence): the
 * rank's rows against the whole natural-order K/V in a single launch of the
 * step kernel, with no ring steps, no receive and no merge; each owned chunk
 * sees the keys before it (causal) or all keys (bidirectional).  Same result
 * as cp_attn_rank_forward up to rounding order.  Same arguments and errors as
 * cp_attn_rank_forward, and EUNSUPPORTED when the K/V tensors exceed 4 GiB.
 * Uses the workspace only for the document table, when documents are set
 * (allocating it on first use unless the caller gave one). */
int cp_attn_allgather_forward(cp_attn_plan_t plan, const void* q, const void* k, const void* v, void* out,
                              float* lse, int rank, void* stream);

/*
 * Ulysses variant ("Sequence Parallelism IV: Megatron Context Parallel and
 * Load-Balanced Rings", section 7 "CP vs Ulysses"): one all-to-all trades
 * token slices for head slices, so that a rank holds all S tokens of
 * heads_per_rank = heads / cp_size heads and runs plain attention on them;
 * a second all-to-all returns the output to the token owners.  The degree
 * cannot exceed the head count: both calls return EUNSUPPORTED unless
 * heads % cp_size == 0.
 *
 * cp_attn_ulysses_a2a: the all-to-all of every rank at once, plan dtype,
 * bit-exact copies.  to_heads = 1: src is the sequence layout
 * [cp][local_rows][heads][head_dim] (as cp_attn_layout_gather writes it),
 * dst the head layout [cp][S][heads_per_rank][head_dim] (rank r: heads
 * r*heads_per_rank .. (r+1)*heads_per_rank-1 of every token, natural order).
 * to_heads = 0: the reverse (pad rows of the sequence layout are not
 * written).  EINVAL for null/misaligned pointers or to_heads outside {0, 1}.
 */
int cp_attn_ulysses_a2a(cp_attn_plan_t plan, const void* src, void* dst, int to_heads, void* stream);

/* One rank's Ulysses attention: q, k, v, out [S][heads_per_rank][head_dim]
 * (that rank's slice of the head layout), lse [heads_per_rank][S] fp32 (4-byte
 * alignment suffices: it may be rows r*heads_per_rank.. of a [heads][S]
 * array); the plan's mask (causal or bidirectional) over all S tokens, one
 * launch of the step kernel.  EUNSUPPORTED also when a slice exceeds 4 GiB. */
int cp_attn_ulysses_forward(cp_attn_plan_t plan, const void* q, const void* k, const void* v, void* out, float* lse,
                            void* stream);

/*
 * cp_attn_rank_forward without any allocation, for callers that cannot
 * allocate device memory or create streams: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments and
 * errors as cp_attn_rank_forward, and its result bit for bit with
 * CP_ATTN_OPT_FUSED_RING 0 (this call runs one launch per ring step; the
 * fused launch agrees with that to rounding), but the workspace
 * is a static device array of the library, CP_ATTN_NOALLOC_SCRATCH_BYTES per
 * GPU, held on every GPU the library runs on until the process ends.  The
 * plan's workspace, side streams, events, graph mode, step timing and work
 * counters are not used: every kernel runs on `stream` (the next ring
 * step's K/V is received inside the step kernel where it supports that,
 * otherwise by a copy kernel before the step), so the call can be captured
 * into a HIP graph.  The array keeps the last call's contents; what must
 * start at zero is cleared by the call itself.  All calls on one GPU share
 * the array: calls in flight on that GPU at the same time (any plan, any
 * stream) race, so the caller must order them.
 * ENOWORKSPACE when cp_attn_workspace_bytes exceeds the array; EUNSUPPORTED
 * while document masks are set; otherwise as cp_attn_rank_forward.
 */
#define CP_ATTN_NOALLOC_SCRATCH_BYTES (128LL << 20)
int cp_attn_rank_forward_noalloc(cp_attn_plan_t plan, const void* q, const void* k, const void* v, void* out,
                                 float* lse, int rank, void* stream);

/* Every rank's share on `stream` (ranks 0..cp_size-1), back to back, or with
 * CP_ATTN_OPT_LOCKSTEP all ranks' ring step s in one launch; fills all rows
 * of out and lse.  In the fused schedule, when a row tile sees at most 192
 * key tiles (short launches), the odd ranks run on a second library-owned
 * stream pair beside the even ones (own receive slots, flags and key-split
 * buffers, allocated on first use); it starts behind the work queued on
 * `stream` before the call, and `stream` waits for it at the end, so the
 * call is ordered on `stream` as a whole.  Same arguments and errors as
 * cp_attn_rank_forward. */
int cp_attn_full_forward(cp_attn_plan_t plan, const void* q, const void* k, const void* v, void* out,
                         float* lse, void* stream);

/*
 * Backward of one rank's share, asynchronous on `stream` ("Context
 * Parallelism for Long-Context Training", section "Prove attention
 * equivalence": gradients must match the unsharded reference).  With the
 * complete forward's out and lse, every step knows the exact softmax of its
 * valid pairs, P_ij = exp(s_ij - lse_i), and adds, over the same ring steps
 * and valid pairs as the forward:
 *   dV_j += P_ij dO_i;  dS_ij = P_ij (<dO_i, v_j> - <dO_i, O_i>);
 *   dQ_i += dS_ij k_j / sqrt(head_dim);  dK_j += dS_ij q_i / sqrt(head_dim).
 * q, k, v, out, dout: [S][heads][head_dim] plan dtype (out and lse as written
 * by a forward call of the same plan); dq, dk, dv: [S][heads][head_dim] fp32.
 * Writes dq at the rank's real rows; ADDS the rank's terms to dk and dv at
 * the rows of every source it sees (on a ring these partial sums travel
 * with the K/V chunks back to their owner), so zero dk and dv before the
 * first rank.  Uses the plan's workspace; ignores the schedule options.
 * Errors as cp_attn_rank_forward.
 */
int cp_attn_rank_backward(cp_attn_plan_t plan, const void* q, const void* k, const void* v, const void* out,
                          const float* lse, const void* dout, float* dq, float* dk, float* dv, int rank,
                          void* stream);

/* Every rank's backward on `stream`: zeroes dk and dv, then runs ranks
 * 0..cp_size-1; dq, dk, dv end as the complete gradients. */
int cp_attn_full_backward(cp_attn_plan_t plan, const void* q, const void* k, const void* v, const void* out,
                          const float* lse, const void* dout, float* dq, float* dk, float* dv, void* stream);

/* ---- host-only introspection (no HIP calls; CPU-testable) ---- */

/* Rows of each rank's local buffer, pad rows included: S_pad/cp. */
int cp_attn_local_rows(cp_attn_plan_t plan, int64_t* rows);

/* Real (non-pad) rows of `rank`: the first *rows rows of its local buffer
 * (S_pad/cp for every rank when S divides; fewer for the ranks owning the
 * tail chunks otherwise, possibly 0).  EINVAL for a bad rank or null rows. */
int cp_attn_rank_valid_rows(cp_attn_plan_t plan, int rank, int64_t* rows);

/* Chunk indices owned by `rank`, local order ("Sequence Parallelism IV:
 * Megatron Context Parallel and Load-Balanced Rings", section 3: rank r holds
 * chunks r and 2cp-1-r under zigzag); *count = 2 (zigzag) or 1 (contiguous,
 * where the chunk index equals the rank).  `count` is an addition to the
 * plain (rank) -> chunk pair: a contiguous plan owns one chunk, and the
 * caller is told so instead of reading an unused second entry. */
int cp_attn_rank_chunks(cp_attn_plan_t plan, int rank, int32_t chunks[2], int32_t* count);

/* Ring source of (rank, step): (rank - step) mod cp_size. */
int cp_attn_step_source(cp_attn_plan_t plan, int rank, int step, int32_t* source);

/*
 * Step descriptor of (rank, step): up to two query-row segments of the rank's
 * local buffer, each row of which attends to a prefix of the source's local
 * K/V buffer.  out[i*7 + 0..6] for segment i = {q_start, q_len, kv_full, diag,
 * first, last, q_global}: local rows [q_start, q_start + q_len), whose local
 * row q_start + t (global token q_global + t) sees local keys
 * [0, kv_full + (diag ? t + 1 : 0)); first/last = 1 when this step is the
 * segment's first/last active step.  Rows in no segment have no valid key in
 * this step (their sub-blocks are skipped).  *count in {0, 1, 2}.
 */
int cp_attn_step_segments(cp_attn_plan_t plan, int rank, int step, int64_t out[14], int32_t* count);

/* Valid (query, key) pairs of one head in (rank, step), and tiles of
 * bm local rows x bn local keys holding at least one valid pair (tiles laid
 * from local index 0, last tile of each axis clipped); document masks
 * included when set. */
int cp_attn_valid_work(cp_attn_plan_t plan, int rank, int step, int bm, int bn, int64_t* tiles,
                       int64_t* pairs);

/* ---- layout kernels (zigzag / contiguous reordering) ---- */

/* src: [S][heads][head_dim] natural order -> dst: [cp][local_rows][heads][head_dim],
 * each rank's rows in its local order.  Plan dtype, bit-exact copy; pad rows
 * (positions >= S of a padded plan) are written as zeros. */
int cp_attn_layout_gather(cp_attn_plan_t plan, const void* src, void* dst, void* stream);

/* Inverse of cp_attn_layout_gather; pad rows of src are not read. */
int cp_attn_layout_scatter(cp_attn_plan_t plan, const void* src, void* dst, void* stream);

/*
 * Exact LSE merge of a partial into a running state, fp32, on `stream`:
 * o_acc, o_s: [rows][heads][head_dim]; lse_acc, lse_s: [heads][rows].
 * Per (row, head): lse_s = -inf leaves the state; lse_acc = -inf takes the
 * partial; otherwise lse' = max + log1p(exp(-|lse_acc - lse_s|)) and
 * O' = exp(lse_acc - lse') O_acc + exp(lse_s - lse') O_s: two partials over
 * disjoint key sets combine into the softmax over their union, so the split
 * result equals the unsplit one ("Sequence Parallelism IV: Megatron Context
 * Parallel and Load-Balanced Rings", section 4 "What Actually Moves").
 * head_dim must be a multiple of 4; pointers 16-byte aligned.
 */
int cp_attn_lse_merge(float* o_acc, float* lse_acc, const float* o_s, const float* lse_s, int64_t rows,
                      int heads, int head_dim, void* stream);

/* Work counters (CP_ATTN_OPT_COUNTERS = 1): counts[rank * cp + step] (n >=
 * cp*cp) = key tiles the step kernels computed for (rank, step) in the last
 * forward call, over all heads, or -1 for pairs that call did not run.  A tile
 * is *tile_rows query rows x *tile_keys keys (32 x 64 for bf16: one wave's
 * rows; the workgroup tile for fp32), laid from each segment's first row and
 * key 0, counted when the kernel computed its scores: with segments starting
 * at multiples of *tile_rows this equals heads x cp_attn_valid_work(rank,
 * step, *tile_rows, *tile_keys).  Waits for the device. */
int cp_attn_last_tile_counts(cp_attn_plan_t plan, int64_t* counts, int n, int32_t* tile_rows, int32_t* tile_keys);

/* Per (rank, step) attention-kernel milliseconds of the last forward call
 * made with CP_ATTN_OPT_STEP_TIMING = 1, row-major [cp][cp]; entries of ranks
 * the call did not run are -1, and a rank run as one fused launch
 * (CP_ATTN_OPT_FUSED_RING) has it under step 0 and -1 for its other steps.
 * Blocks until those events complete.
 * n must be >= cp_size * cp_size. */
int cp_attn_last_step_times(cp_attn_plan_t plan, float* ms, int n);

/* Static text for a status code. */
const char* cp_attn_status_string(int status);

/* Text describing the calling thread's last failed call (empty if none). */
const char* cp_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CP_ATTN_H */
