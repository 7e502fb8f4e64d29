/*
 * dpack.h — C ABI of the deterministic packing library for MI355X (gfx950).
 *
 * The library turns pre-tokenized documents resident in GPU memory into
 * training batches of fixed T-position windows that are byte-identical at any
 * rank count:
 *   hash hold-out → (source, stratum) grouping → counter-based shuffle →
 *   strata merge → window cut (next-fit) → mixture slots → emission of token
 *   ids, position ids, document ids and loss masks → per-window SHA-256.
 *
 * Pages the operations follow (cited per call below):
 *   - NeuronSpark-Trainer README, "Concepts": data lines consumed in cycles,
 *     every token trained once (running out is an error), each update within
 *     two samples of each source's recipe share, strata at their share of the
 *     source's tokens cut at document ends, documents shuffled, 1 % (5 % for
 *     one source) held out by a hash of the text that is the same in every
 *     line; "Training": updates never span a cycle end, a resume with another
 *     sample order is refused.
 *   - Zephon blog post (aixai.ru), resume of a 16-GPU run on 8/32/64 GPUs: the
 *     SHA-256 of every global batch is equal byte for byte; TorchTitan
 *     integration: configuration errors (divisibility) fail at start.
 *   - Linnet "Training" docs, "Supervised fine-tuning": batches of exactly T
 *     positions padded, a prompted example learns only its completion, updates
 *     weighed by the count of learned positions; "Other trainers": a position
 *     id 0 starts a new sequence within a row.
 *
 * Conventions for every call:
 *   - Return 0 (PACK_OK) on success, a negative PACK_E_* code on failure. No
 *     exception or signal crosses the ABI. pack_last_error() gives a message.
 *   - "device" pointers are GPU memory of the current HIP device; "host"
 *     pointers are CPU memory.  Device inputs are borrowed (caller-owned,
 *     read-only, must outlive the context); the context owns its workspace.
 *   - All work is ordered on cfg->stream (NULL = the default stream).
 *   - One context must not be used by two host threads at once.
 *   - No environment variable changes any output byte.
 */
#ifndef DPACK_H
#define DPACK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DPACK_ABI_VERSION 2u

enum {
    PACK_OK = 0,
    PACK_E_ABI = -1,       /* cfg->abi_version differs from DPACK_ABI_VERSION */
    PACK_E_INVAL = -2,     /* an argument or the corpus violates a stated precondition */
    PACK_E_NOMEM = -3,     /* a host or device allocation failed */
    PACK_E_HIP = -4,       /* a HIP runtime call failed (message in pack_last_error) */
    PACK_E_EXHAUSTED = -5, /* a source cannot supply the cycle's windows */
    PACK_E_STATE = -6,     /* calls out of order (cycle skipped, batch before cycle) */
    PACK_E_RANGE = -7,     /* step range beyond the current cycle */
    PACK_E_INTERNAL = -8,  /* a kernel found the plan inconsistent or a bounded wait gave up (a
                              library bug): the call's results are not valid */
};

typedef struct pack_ctx pack_ctx;

/* pack_config.flags: record HIP events around every kernel phase on the
 * context's stream (read with pack_get_timings).  Changes no output byte. */
#define PACK_FLAG_TIMING 1u
/* pack_config.flags: wrap packing instead of next-fit.  "Zephon:
 * deterministic data loading" (aixai.ru), minimal example, packs with
 * pack_flat(max_length, algorithm="wrap"); the page gives only the name.
 * Reading taken: per source, the merged order's tokens are one stream cut
 * every T tokens; a document crossing a cut continues at the next window's
 * first position, its position ids restarting at 0; only each source's last
 * window can be short (padded).  Every other output is as with next-fit. */
#define PACK_FLAG_WRAP 2u
/* pack_config.flags: plan the held-out documents, the validation stream,
 * instead of the training ones.  NeuronSpark-Trainer README, Concepts: each
 * source's validation rows come from its held-out documents of every
 * stratum, and the validation mix weights the sources by the recipe.
 * Reading taken: the same plan (shuffle, strata merge, cut, mixture) over the
 * non-empty held-out documents; the cycle info's kept_* then count the
 * stream's documents, held_* still the documents the hash holds out. */
#define PACK_FLAG_HELDOUT 4u
/* pack_config.flags: read each source's windows of a cycle in a random order.
 * NeuronSpark-Trainer README, Concepts: the trainer reads each source's
 * windows of a segment in a random order.  Reading taken: a segment is a
 * cycle; source s's i-th window of the cycle (i < U·n_s) is ranked by
 * key64 = x1·2^32 + x0 of Philox4x32-10(counter = (i, s, cycle, 0x57494E44),
 * key = seed), ties by i, and update b's k-th window of s is the one of rank
 * b·n_s + k.  Per-update counts, cycle ranges and sums are unchanged. */
#define PACK_FLAG_READ_RANDOM 8u
/* pack_config.flags: per-update window counts from the cycle's cumulative
 * quotas instead of one fixed apportionment.  NeuronSpark-Trainer README,
 * Concepts: every update holds each source within two samples of its recipe
 * share, and every token is trained (max_epochs 1).  Reading taken: after u
 * updates of a cycle, source s has taken A_s(u) windows, floor(u·B·w_s/W) ≤
 * A_s(u) ≤ ceil(u·B·w_s/W), never fewer than after u−1; so every update holds
 * each source within two windows of B·w_s/W and a share below one window per
 * update still gets its windows over the cycle.  Source s's j-th window of
 * the cycle is released in update floor((j−1)·W/(B·w_s)) and due by update
 * ceil(j·W/(B·w_s)) − 1; each update takes the B released windows with the
 * earliest due updates, ties to the lower source (earliest deadline first,
 * which meets every deadline: Balinski and Young's quota method shows a
 * schedule exists).  Each update's slots are in the Sainte-Laguë order of its
 * own counts.  With updates_per_cycle = 0 the cycle is the longest prefix of
 * the schedule no source runs out in.  At most 1024 sources; the table of
 * (updates x sources) is bounded by 2^28 entries at init. */
#define PACK_FLAG_CUMULATIVE 16u
/* pack_config.flags: record HIP events only around the kernels of pack_batch,
 * pack_batch_packed and pack_fingerprint (phases EMIT, LEARNED, DIGEST,
 * FINGERPRINT); pack_init and pack_cycle record none, so their kernels run as
 * in an untimed context (each event costs several microseconds of stream
 * time).  With PACK_FLAG_TIMING as well, every phase is timed.  Changes no
 * output byte. */
#define PACK_FLAG_TIMING_BATCH 32u
/* pack_config.flags: chunked window digests.  Zephon blog post, resume
 * section, fixes only that every global batch's SHA-256 is equal at any rank
 * count; how a window is digested is this library's reading.  Without the
 * flag a window's digest is one SHA-256 over its 13·T-byte record (pack_out),
 * a serial chain of about 13·T/64 compressions.  With it the record is cut
 * into chunks of 4,096 bytes (the last one shorter when 13·T is not a
 * multiple), each chunk is hashed with SHA-256, and the window's digest is
 * the SHA-256 of those chunk digests in record order, 32 bytes each (a
 * record of one chunk, T ≤ 315, gets SHA-256(SHA-256(record))).  The chunks
 * of a window hash side by side, so few windows take far less time; the
 * digests differ from those without the flag, and batch fingerprints are
 * taken over them as before.  Changes no other output byte; the context's
 * device memory grows by at most 16 MiB (the chunk digests of one slice of
 * windows at a time). */
#define PACK_FLAG_DIGEST_CHUNKED 64u

/* Kernel phases timed under PACK_FLAG_TIMING (EMIT to FINGERPRINT also under
 * PACK_FLAG_TIMING_BATCH). */
enum {
    PACK_PHASE_VALIDATE = 0, /* corpus validation kernel */
    PACK_PHASE_HASH,         /* per-document hash and hold-out */
    PACK_PHASE_KEYS,         /* compaction of kept documents and Philox keys */
    PACK_PHASE_SORT,         /* sort by (group, key, document) */
    PACK_PHASE_MERGE,        /* strata merge */
    PACK_PHASE_PIECES,       /* piece counts, prefix sums and piece table */
    PACK_PHASE_CUT,          /* next-fit: next pointers, lifting, windows per source */
    PACK_PHASE_WINDOWS,      /* window table, real and learned positions per window */
    PACK_PHASE_MIXTURE,      /* apportionment, slot table, order checks */
    PACK_PHASE_CYCLE,        /* cycle sums and plan digest */
    PACK_PHASE_EMIT,         /* emission kernel of pack_batch (when not timed under DIGEST) */
    PACK_PHASE_LEARNED,      /* per-update learned counts of pack_batch */
    PACK_PHASE_DIGEST,       /* per-window SHA-256 of pack_batch with digests; the emission runs
                              * inside the same kernel and is timed here */
    PACK_PHASE_FINGERPRINT,  /* pack_fingerprint */
    PACK_N_PHASES
};

typedef struct pack_timings {
    double ms[PACK_N_PHASES];      /* summed event-to-event time of each phase */
    uint64_t calls[PACK_N_PHASES]; /* number of timed intervals summed */
} pack_timings;

/* Configuration of a packing context.  Limits (PACK_E_INVAL otherwise):
 * 1 ≤ n_docs < 2^31; n_tokens < 2^40; every document shorter than 2^32
 * tokens; offsets monotone with doc_offsets[n_docs] ≤ n_tokens;
 * 1 ≤ n_sources ≤ 4096;
 * source < n_sources; stratum < n_strata[source]; Σ n_strata ≤ 65536;
 * Σ share_weight in [1, 2^64); holdout_bp ≤ 10000; 1 ≤ T ≤ 2^20 (any T;
 * with T a multiple of 64 the window digests are computed beside the
 * emission, otherwise from the emitted outputs after it); 1 ≤ B ≤ 2^20; world ≥ 1 divides B; rank < world; with a
 * ramp: n_ramp ≤ 4096, ramp_from[0] = 0 and rising, every ramp_tokens[k] a
 * multiple of T whose batch B_k = ramp_tokens[k]/T world divides, and B the
 * largest B_k.
 *
 * Batch-size ramp (n_ramp > 0).  NeuronSpark-Trainer README, Training,
 * Updates: tokens_per_update is one number or pieces by the tokens trained,
 * and an update's batch is read at the data line's token count (the cycle's
 * start token plus its updates so far).  Reading taken: the count is the
 * positions of every earlier update (B_b·T each), from 0 at cycle 0 and
 * across cycles; an update starting at count t has B_k = ramp_tokens[k]/T
 * windows for the last k with ramp_from[k] ≤ t.  Each update's windows come
 * from the apportionment of its own batch (or, with PACK_FLAG_CUMULATIVE,
 * from quotas at the running count of windows), in the Sainte-Laguë order of
 * its own counts; a cycle still never splits an update.
 *
 * Lanes (n_lanes = L > 1).  Zephon blog post, "lanes instead of ranks": the
 * data are split into a fixed number of logical streams, each with its own
 * ordered samples and packing state, and ranks take whole lanes; the
 * TorchTitan integration checks that the ranks divide the lanes and the
 * lanes every update's batch.  Reading taken: document d belongs to lane
 * d mod L; each (source s, lane l) is a stream s·L + l planned as a source is
 * (shuffle, strata merge, cut); update u gives lane l its B_u/L consecutive
 * slots from l·B_u/L on, apportioned over the sources like a batch of B_u/L
 * (every lane the same counts; with PACK_FLAG_CUMULATIVE one schedule over
 * B_u/L seats that every lane follows).  Limits: L divides B and every ramp
 * batch, world divides L, n_sources·L ≤ 4096, Σ n_strata·L ≤ 65536.  With
 * lanes the per-source arrays of pack_cycle_info and of pack_inspect hold
 * n_sources·L entries, one per stream.
 *
 * Stream starts (start_tokens).  NeuronSpark-Trainer README, Training: every
 * update has one sequence length and updates never span a change of length;
 * a branch forks from the state after a trunk cycle.  Reading taken: a
 * context may cut each stream (source, or source and lane) from a given token
 * of its merged order: documents before it are skipped, the one it falls in
 * contributes its tokens from there on, and next-fit or wrap starts there.
 * pack_cycle_info.stream_next_token reports where each stream's next cycle
 * begins; a context built with those as start_tokens (the same corpus and
 * recipe, any T, first_cycle the next cycle's number, tokens_start the
 * tokens trained so far) goes on from there, and with the same T its cycles
 * are byte for byte the ones the first context would have planned.
 *
 * Streamed corpora (doc_segment, n_segments).  NeuronSpark-Trainer README,
 * Concepts: a data line's cycles are each downloaded, tokenized, trained on
 * and deleted; a file's documents are shuffled at tokenization; files left
 * open give the rest to the next cycles.  Reading taken: a document belongs
 * to the arrival it came with; each stream's documents go arrival by arrival,
 * each arrival shuffled and strata-merged on its own, so the order of the
 * arrivals so far does not change when more arrive.  A context per arrival
 * over the documents so far (appended, so indices stay), with start_tokens
 * from the previous context's stream_next_token, goes on where the previous
 * cycle stopped: the rest of the earlier arrivals first, then the new one.
 * Limit: Σ n_strata · lanes · n_segments ≤ 65536 groups. */
typedef struct pack_config {
    uint32_t abi_version;          /* DPACK_ABI_VERSION */
    uint32_t flags;                /* 0 or an or of PACK_FLAG_TIMING, _TIMING_BATCH, _WRAP, _HELDOUT, _READ_RANDOM,
                                      _CUMULATIVE */
    const uint32_t *tokens;        /* device [n_tokens] token ids */
    uint64_t n_tokens;
    const uint64_t *doc_offsets;   /* device [n_docs+1]: document d is tokens[off[d], off[d+1]) */
    uint64_t n_docs;
    const uint16_t *doc_source;    /* device [n_docs] */
    const uint16_t *doc_stratum;   /* device [n_docs]; NULL = stratum 0 for all */
    const uint32_t *doc_prompt_len;/* device [n_docs]; NULL = no prompt (every token learned) */
    uint32_t n_sources;
    const uint32_t *n_strata;      /* host [n_sources]; NULL = one stratum each */
    const uint64_t *share_weight;  /* host [n_sources] integer recipe weights */
    const uint32_t *holdout_bp;    /* host [n_sources] hold-out rate in basis points */
    uint32_t window_tokens;        /* T: positions per window */
    uint32_t global_batch;         /* B: windows per update (all ranks) */
    uint32_t updates_per_cycle;    /* updates in each cycle; 0 = the most the data support */
    uint32_t pad_token;            /* token id written at padding positions */
    uint64_t seed;                 /* shuffle seed */
    uint32_t rank, world;          /* this context emits slots [rank·B/world, (rank+1)·B/world) */
    void *stream;                  /* hipStream_t for all work; NULL = default stream */
    uint32_t n_ramp;               /* 0: every update has B windows; else the pieces below */
    const uint64_t *ramp_from;     /* host [n_ramp]: tokens trained at which piece k starts */
    const uint64_t *ramp_tokens;   /* host [n_ramp]: tokens per update (B_k·T) within piece k */
    uint32_t n_lanes;              /* 0 or 1: no lanes; L > 1: Zephon lanes (see above) */
    const uint64_t *start_tokens;  /* host [streams] or NULL: first token of each stream to cut (below) */
    uint32_t first_cycle;          /* number of the first cycle (pack_cycle starts there) */
    uint64_t tokens_start;         /* tokens trained before the first cycle (the ramp's count) */
    const uint16_t *doc_segment;   /* device [n_docs] or NULL: the arrival of each document (below) */
    uint32_t n_segments;           /* arrivals: doc_segment < n_segments (0 or 1: one arrival) */
} pack_config;

/* pack_init — build the plan of a corpus (hash and hold-out of every
 * document, grouping, shuffle keys and sort, strata merge, pieces, next-fit
 * windows, per-update apportionment and slot table) on cfg->stream.
 * NeuronSpark-Trainer README, Concepts: documents held out by a hash of their
 * text (the same in every line, each source at its own rate), shuffled, each
 * source's strata at their share of its tokens, windows cut at document
 * ends; Zephon blog post, TorchTitan integration: configuration errors such
 * as a rank count that does not divide the batch fail at start.
 * Synchronous: returns once the plan is on the device; reads back only the
 * per-source window counts and statistics.  The plan is independent of rank
 * and world, which only select the emitted slice.
 * Errors: PACK_E_ABI, PACK_E_INVAL (limits above, checked on the host and,
 * for device arrays, by a validation kernel), PACK_E_NOMEM, PACK_E_HIP,
 * PACK_E_INTERNAL.  On error *out is NULL and nothing is leaked. */
int pack_init(const pack_config *cfg, pack_ctx **out);

/* pack_init_noalloc — pack_init for callers that cannot allocate memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same plan, byte for byte, built without hipMalloc, hipFree,
 * hipHostMalloc or any other allocating HIP call.  The device workspace is a
 * static array of 64 MiB that each GPU the library runs on holds until the
 * process ends; the staging of host<->device copies is a static host buffer of
 * 1 MiB per device (ordinary memory, so the plan's few small copies are
 * pageable).  The context object itself is ordinary host memory.  Limits, on
 * top of pack_init's: the plan's workspace must fit 64 MiB and its staging
 * 1 MiB (PACK_E_INVAL with both sizes in pack_last_error otherwise, checked
 * before any device work; roughly 250,000 documents of a few hundred tokens),
 * no PACK_FLAG_TIMING (PACK_E_INVAL), at most 16 devices.  One context made by
 * pack_init_noalloc may be alive per device at a time: while it is, another
 * pack_init_noalloc on that device returns PACK_E_STATE (pack_destroy frees
 * the slot).  The workspace keeps the previous context's bytes; the plan
 * clears what must start at zero.  The returned context takes every other
 * call as a pack_init context does.  Errors: as pack_init, and PACK_E_STATE. */
int pack_init_noalloc(const pack_config *cfg, pack_ctx **out);

/* Per-cycle information, filled by pack_cycle.  The per-source arrays are
 * optional host buffers of n_sources entries owned by the caller. */
typedef struct pack_cycle_info {
    uint32_t cycle;
    uint32_t n_updates;            /* U of this cycle */
    uint64_t real_tokens;          /* non-padding positions in the cycle (all ranks) */
    uint64_t learned_tokens;       /* positions with loss mask 1 in the cycle (all ranks) */
    uint64_t positions;            /* U·B·T (with a ramp: Σ B_b·T) */
    uint8_t plan_digest[32];       /* SHA-256 identifying recipe, stream sizes, cycle start and order */
    uint64_t *windows_start;       /* first window of the cycle in each source's stream */
    uint64_t *windows_taken;       /* U·n_s (with PACK_FLAG_CUMULATIVE or a ramp: A_s(U)) */
    uint64_t *windows_remaining;   /* windows left after the cycle */
    uint64_t *kept_docs, *kept_tokens, *held_docs, *held_tokens;
    uint32_t *per_update;          /* n_s: windows of each source in every update (the fixed
                                    * apportionment of B; with PACK_FLAG_CUMULATIVE or a ramp the
                                    * counts vary per update: PACK_INSPECT_CUM_TAKEN) */
    uint64_t *stream_next_token;   /* token of each stream's merged order where the next cycle's
                                    * windows begin (its total once used up): start_tokens of a
                                    * context that goes on after this cycle */
} pack_cycle_info;

/* pack_cycle — plan cycle `cycle` (must be first_cycle, then the next, …):
 * U updates, each of B windows of which n_s come from source s, taking the
 * next U·n_s windows of each source's stream.  U = updates_per_cycle, or
 * when that is 0 the most every source with n_s > 0 supports.  With
 * PACK_FLAG_CUMULATIVE update u takes A_s(u+1) − A_s(u) windows of source s
 * (see the flag) and the cycle A_s(U).  NeuronSpark-Trainer README, Concepts
 * and Training: a data line is consumed in cycles, updates never span a
 * cycle end, every token is trained once and running out is an error.
 * Synchronous.  info may be NULL.
 * Errors: PACK_E_STATE (out of order), PACK_E_EXHAUSTED (some source cannot
 * supply its windows of the cycle, or U would be 0: an error, never a second
 * pass), PACK_E_INTERNAL, PACK_E_HIP.  On any error no cycle is current
 * afterwards (pack_batch and the cycle's inspections return PACK_E_STATE)
 * and the same cycle number is the one to plan next. */
int pack_cycle(pack_ctx *ctx, uint32_t cycle, pack_cycle_info *info);

/* Outputs of pack_batch: device buffers owned by the caller, each laid out
 * [n_steps][B/world][T] in slot order (row-major, contiguous); with a
 * batch-size ramp update b contributes B_b/world windows, update after update
 * ([Σ B_b/world][T], PACK_INSPECT_UPDATE_BATCH gives each B_b). */
typedef struct pack_out {
    uint32_t *tokens;    /* token id, pad_token at padding */
    int32_t *pos;        /* offset within the piece (0 starts each piece), 0 at padding */
    int32_t *doc;        /* global input document index, −1 at padding */
    uint8_t *mask;       /* 1 iff the token is learned (at or after the prompt) */
    int64_t *learned;    /* device [n_steps]: global learned positions of each update; NULL = skip */
    uint8_t *digests;    /* device [n_steps][B/world][32]: SHA-256 of each window's record
                            tok‖pos‖doc‖mask (little-endian, 13·T bytes), or of its chunks'
                            digests under PACK_FLAG_DIGEST_CHUNKED; NULL = skip */
} pack_out;

/* pack_batch — emit updates [step, step+n_steps) of the current cycle for
 * this context's rank.  Linnet "Training", Supervised fine-tuning: rows of
 * exactly T positions with the rest padded, loss on completions only, each
 * update weighed by its learned positions; Zephon blog post, resume section:
 * every global batch byte-identical (and its SHA-256 equal) at any rank count.
 * Asynchronous on cfg->stream; a pure function of (corpus, config, cycle,
 * step), so re-emitting a step reproduces it exactly.  A failure inside its
 * kernels (PACK_E_INTERNAL) is reported by the next pack_status.
 * Errors: PACK_E_STATE (no cycle planned), PACK_E_RANGE (step + n_steps > U
 * or n_steps = 0), PACK_E_INVAL (a NULL output array), PACK_E_HIP. */
int pack_batch(pack_ctx *ctx, uint32_t step, uint32_t n_steps, const pack_out *out);

/* Padding-free rows.  Linnet "Training", Supervised fine-tuning (the
 * transformers Trainer path): the padding is removed and a batch's rows are
 * packed into one sequence whose length rounds up to a multiple of a bucket
 * (256) so that few shapes compile; a position id 0 starts each sequence.
 * Device arrays, all required but learned: */
typedef struct pack_out_packed {
    uint32_t *tokens;    /* [n_steps][B/world · T]: update i's row; window jj's real positions
                            (as in pack_batch) at row_start[i][jj] .. row_start[i][jj+1]; with a
                            ramp rows stay B/world·T apart (B the largest batch) */
    int32_t *pos;        /* same layout; 0 starts each piece */
    int32_t *doc;
    uint8_t *mask;
    int64_t *row_start;  /* [n_steps][B/world + 1]: where each window begins; [B/world] = the total
                            (with a ramp entries from [B_i/world] on all hold the total) */
    int64_t *length;     /* [n_steps]: the total rounded up to a multiple of bucket, at most B_i/world · T;
                            positions from the total to the length are padding, later ones are not written */
    int64_t *learned;    /* [n_steps] or NULL: as in pack_batch */
    uint32_t bucket;     /* the rounding multiple (256 in the pages); 0 or 1: none */
} pack_out_packed;

/* pack_batch_packed — pack_batch's windows as padding-free rows (no digests:
 * window digests are defined over the padded records of pack_batch).
 * tokens, pos and doc must be 16-byte aligned, mask 4-byte aligned, row_start,
 * length and learned 8-byte aligned.  Asynchronous on cfg->stream.  Errors as pack_batch. */
int pack_batch_packed(pack_ctx *ctx, uint32_t step, uint32_t n_steps, const pack_out_packed *out);

/* pack_fingerprint — batch fingerprints: for each of n_batches, SHA-256 over
 * its B window digests (B·32 bytes, slot order) from the device array
 * digests [n_batches][B][32], into the device array out [n_batches][32].
 * For world > 1 the caller first gathers every rank's digests in rank order.
 * Asynchronous on the context's stream.  Errors: PACK_E_INVAL (NULL),
 * PACK_E_STATE (a context with a batch-size ramp: use pack_fingerprint_steps),
 * PACK_E_HIP. */
int pack_fingerprint(pack_ctx *ctx, const uint8_t *digests, uint32_t n_batches, uint8_t *out);

/* pack_fingerprint_steps — fingerprints of updates [step, step+n_steps) of
 * the current cycle, each SHA-256 over its own B_b window digests: digests is
 * the device array of those updates' digests one after another (Σ B_b·32
 * bytes; every rank's slice of an update in rank order), out [n_steps][32].
 * Zephon blog post, the 16→8/32/64-GPU resume section: every global batch's
 * SHA-256 equal byte for byte.  Any context (without a ramp it equals
 * pack_fingerprint).  Asynchronous.  Errors: PACK_E_INVAL (NULL),
 * PACK_E_STATE (no cycle), PACK_E_RANGE, PACK_E_HIP. */
int pack_fingerprint_steps(pack_ctx *ctx, uint32_t step, uint32_t n_steps, const uint8_t *digests, uint8_t *out);

/* Plan arrays that pack_inspect copies to the host (for checking the plan
 * against an independent implementation).  Types and lengths: */
enum {
    PACK_INSPECT_HASH = 1,          /* uint64 [n_docs] content hash */
    PACK_INSPECT_KEEP = 2,          /* uint8  [n_docs] 1 = kept */
    PACK_INSPECT_ORDER = 3,         /* uint32 [n_kept] kept docs, source by source, merged order */
    PACK_INSPECT_SRC_DOC_START = 4, /* uint64 [n_sources+1] */
    PACK_INSPECT_PIECE_DOC = 5,     /* uint32 [n_pieces] */
    PACK_INSPECT_PIECE_OFF = 6,     /* uint32 [n_pieces] offset of the piece in its document */
    PACK_INSPECT_PIECE_LEN = 7,     /* uint32 [n_pieces] */
    PACK_INSPECT_PIECE_WOFF = 8,    /* uint32 [n_pieces] offset of the piece in its window */
    PACK_INSPECT_SRC_PIECE_START = 9,  /* uint64 [n_sources+1] */
    PACK_INSPECT_WIN_FIRST = 10,    /* uint64 [n_windows+1] first piece of each window */
    PACK_INSPECT_SRC_WIN_START = 11,/* uint64 [n_sources+1] */
    PACK_INSPECT_WIN_REAL = 12,     /* uint64 [n_windows] real positions */
    PACK_INSPECT_WIN_LEARN = 13,    /* uint64 [n_windows] learned positions */
    PACK_INSPECT_PER_UPDATE = 14,   /* uint32 [n_sources] n_s */
    PACK_INSPECT_SLOT_SRC = 15,     /* uint32 [B] */
    PACK_INSPECT_SLOT_K = 16,       /* uint32 [B] */
    PACK_INSPECT_COUNTS = 17,       /* uint64 [3]: n_kept, n_pieces, n_windows */
    PACK_INSPECT_CUM_TAKEN = 18,    /* uint32 [(U+1)·n_sources]: with PACK_FLAG_CUMULATIVE or a ramp,
                                     * windows of each source taken before each update of the current
                                     * cycle (row U: the cycle's totals); PACK_E_STATE otherwise */
    PACK_INSPECT_UPDATE_BATCH = 19, /* uint32 [U]: windows (all ranks) of each update of the current cycle */
};

/* pack_inspect — copy plan array `what` to host memory (synchronous).
 * *needed receives its size in bytes; nothing is copied when
 * capacity_bytes < *needed.  Errors: PACK_E_INVAL (unknown what, NULL ctx),
 * PACK_E_RANGE (capacity too small), PACK_E_HIP. */
int pack_inspect(const pack_ctx *ctx, uint32_t what, void *host_dst, uint64_t capacity_bytes,
                 uint64_t *needed);

/* pack_status — synchronize the context's stream and report whether a
 * kernel of an asynchronous call made since the last pack_status (the window
 * digests of pack_batch wait, boundedly, for the emission beside them)
 * flagged an internal failure; if so, the outputs of those calls are not
 * valid, and the flag is cleared.  Returns PACK_OK, PACK_E_INTERNAL (message
 * in pack_last_error), PACK_E_INVAL (NULL) or PACK_E_HIP. */
int pack_status(pack_ctx *ctx);

/* Test options for pack_test_option.  They exist so that the error paths
 * above, and code paths that real inputs almost never take, can be exercised
 * on a GPU with every kernel still running to its end; with every option 0
 * (the default) no output byte changes, and PACK_TEST_SORT_INSERTION and
 * PACK_TEST_DIGEST_SLICES change none either. */
enum {
    PACK_TEST_WAIT_GIVE_UP = 1, /* the digest waves' bounded waits give up after one poll:
                                   the batch's digests are invalid, pack_status reports it
                                   (calls of at most 65,536 windows; larger ones have no wait) */
    PACK_TEST_CYCLE_FAULT = 2,  /* a cycle kernel reports an internal failure: pack_cycle fails */
    PACK_TEST_SORT_INSERTION = 3, /* the sort of a cycle's random read order orders every bucket
                                     by insertion, the path of buckets above 16 elements */
    PACK_TEST_DIGEST_SLICES = 4,  /* chunked window digests in slices of 3 windows (many slices
                                     and a partial last one per call); no output byte changes */
};

/* pack_test_option — set test option `what` on (value != 0) or off for the
 * calls that follow.  Errors: PACK_E_INVAL (NULL ctx, unknown option). */
int pack_test_option(pack_ctx *ctx, uint32_t what, uint32_t value);

/* pack_get_timings — synchronize the context's stream and return the phase
 * times recorded since the last reset (all zero unless the context was made
 * with PACK_FLAG_TIMING).  reset != 0 clears them afterwards.
 * Errors: PACK_E_INVAL (NULL), PACK_E_HIP. */
int pack_get_timings(pack_ctx *ctx, pack_timings *out, int reset);

/* pack_destroy — free the context and its device workspace (synchronizes
 * its stream first).  NULL is a no-op. */
void pack_destroy(pack_ctx *ctx);

/* Static description of an error code. */
const char *pack_strerror(int code);

/* Message of the last error on this context (or of the last failed
 * pack_init on this thread when ctx is NULL); never NULL. */
const char *pack_last_error(const pack_ctx *ctx);

#ifdef __cplusplus
}
#endif

#endif /* DPACK_H */
