/*
 * oracle.c — plain, sequential CPU definition of deterministic packing.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this file.  The GPU library
 * never links it, includes it or calls it, and shares no code, header, table
 * or constant generator with it.
 *
 * Each function follows one step of the method, in the order the pages give
 * it, written for a reader to check by eye: one loop per step, no blocking,
 * no fusion, no parallel reformulation.  Where the pages leave a step open,
 * the reading taken is stated at the function.  Pages cited:
 *   [NS]  NeuronSpark-Trainer README — "Concepts" (data lines, mixture,
 *         strata, hold-out, shuffling) and "Training" (updates, cycles,
 *         determinism, checkpoints).
 *   [ZE]  "Zephon: deterministic data loading" (aixai.ru blog) — the 16→8/32/64
 *         GPU resume section (SHA-256 of every global batch), "three
 *         decisions" and the TorchTitan integration section (fail-fast
 *         divisibility checks).
 *   [LI]  Linnet "Training" docs — "Supervised fine-tuning" (pack to exactly
 *         T positions, completion-only loss, learned-position counts),
 *         "Other trainers" (position ids restart at 0 per sequence).
 *   [ZE'] the same Zephon post, its minimal example (a pipeline that packs
 *         with pack_flat(max_length, algorithm="wrap")).
 *
 * Parity status of each part (what pins it is in the test suite):
 *   - doc hash (C1): the pages name no hash function, so the function itself
 *     is our definition.  Pinned by closed forms of the definition and by the
 *     published SplitMix64 output for state 0; "parity unpinned" by the pages.
 *   - Philox4x32-10: Salmon et al., SC'11; pinned against rocRAND's open
 *     implementation.
 *   - SHA-256: FIPS 180-4; pinned against Python's hashlib.
 *   - window digests, whole-record (C8) and chunked: rebuilt from the record
 *     bytes with Python's hashlib; a record of one chunk gives the double
 *     SHA-256 of the record.
 *   - the sort uses the C library's qsort with a total order as comparator.
 *   - cumulative mixture (C6c): pinned by its requirements in exact integers
 *     (quota at every update boundary, monotone, B per update), by exhaustive
 *     enumeration of every valid schedule on tiny cases, and by closed forms
 *     (one source; whole-window shares equal the fixed apportionment).
 *   - batch-size ramp (C6b): batches recomputed from the definition across
 *     cycles; each update's counts equal its batch's apportionment (fixed) or
 *     lie within quota of the running seat count (cumulative, also against
 *     every valid schedule on tiny cases); a one-piece ramp is the plain plan.
 *   - stream starts (C5s): resuming at the reported next tokens with the same T
 *     reproduces the next cycles bit for bit in every mode; with another T
 *     every later token is emitted once, with masks by document offset.
 *
 * All integers are unsigned unless stated; products that can exceed 64 bits
 * are taken in unsigned __int128.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef unsigned __int128 u128;

#if defined(__BYTE_ORDER__) && __BYTE_ORDER__ != __ORDER_LITTLE_ENDIAN__
#error "the oracle writes records in host byte order and assumes little-endian"
#endif

enum {
    OR_OK = 0,
    OR_E_INVAL = -2,
    OR_E_NOMEM = -3,
    OR_E_EXHAUSTED = -5,
    OR_E_STATE = -6,
    OR_E_RANGE = -7,
    OR_E_INTERNAL = -9,  /* a step's own guarantee failed (never expected) */
};

/* ------------------------------------------------------------------------ */
/* C1. Per-document content hash.                                           */
/*                                                                          */
/* [NS] Concepts: documents are held out by a hash of their text that is     */
/* the same in every data line.  Reading: the input is token ids, so hash    */
/* the token sequence and its length; not keyed by seed, cycle or rank.      */
/*                                                                          */
/* Definition: position keys k_i = (i+1)·0x9E3779B1 mod 2^32.  Pair tokens   */
/* (t_{2j}, t_{2j+1}); an odd length gets a virtual t_L = 0 (with its key).  */
/* S = Σ_j ((t_{2j}+k_{2j}) mod 2^32)·((t_{2j+1}+k_{2j+1}) mod 2^32) mod 2^64 */
/* (the NH compression of Black et al., CRYPTO'99, with fixed keys), then    */
/* h = mix64(S xor (L·0x9E3779B97F4A7C15 mod 2^64)), where mix64 is the      */
/* SplitMix64 output function (Steele, Lea & Flood, OOPSLA 2014).            */
/* ------------------------------------------------------------------------ */

uint64_t or_mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static uint32_t position_key(uint64_t i)
{
    return (uint32_t)((i + 1) * 0x9E3779B1ull);
}

uint64_t or_doc_hash(const uint32_t *t, uint64_t L)
{
    uint64_t S = 0;
    for (uint64_t i = 0; i < L; i += 2) {
        uint32_t a = t[i] + position_key(i);
        uint32_t second = (i + 1 < L) ? t[i + 1] : 0u;
        uint32_t b = second + position_key(i + 1);
        S += (uint64_t)a * (uint64_t)b;
    }
    return or_mix64(S ^ (L * 0x9E3779B97F4A7C15ull));
}

/* C2. Hold-out decision: held iff floor(h·10000 / 2^64) < bp, i.e. the hash
 * read as a fraction of 2^64 falls below bp basis points.  [NS] Concepts:
 * 1 % of a file's documents (5 % for one source) by that hash; each source
 * applies its own rate to the same unsalted hash. */
int or_held(uint64_t h, uint32_t bp)
{
    uint64_t q = (uint64_t)(((u128)h * 10000u) >> 64);
    return q < (uint64_t)bp;
}

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon, Moraes, Dror & Shaw, SC'11): ten rounds of the     */
/* 4x32 S-box with multipliers 0xD2511F53 (applied to word 0) and            */
/* 0xCD9E8D57 (word 2), key bumped by the Weyl increments 0x9E3779B9 and     */
/* 0xBB67AE85 between rounds.                                               */
/* ------------------------------------------------------------------------ */

void or_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; round++) {
        if (round > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* C3. Shuffle key of document d: the first two words of
 * Philox4x32-10(counter = (d mod 2^32, d div 2^32, 0x53485546, 0),
 *               key = (seed mod 2^32, seed div 2^32)),
 * key64 = x1·2^32 + x0.  Keyed only by the seed and the input document index,
 * never by rank, world or worker count. */
/* C6r. Read order of a source's windows within a cycle ([NS] Concepts: the
 * trainer reads each source's windows of a segment in a random order).
 * Reading: a segment is a cycle; window i of source s's cycle range (i in
 * [0, U·n_s)) gets key64 = x1·2^32 + x0 of Philox4x32-10(counter =
 * (i, s, cycle, 0x57494E44), key = (seed lo, seed hi)), and the range is read
 * in order of (key64, i). */
uint64_t or_window_key(uint64_t seed, uint32_t s, uint32_t cycle, uint32_t i)
{
    uint32_t ctr[4] = {i, s, cycle, 0x57494E44u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t x[4];
    or_philox4x32_10(ctr, key, x);
    return ((uint64_t)x[1] << 32) | x[0];
}

uint64_t or_shuffle_key(uint64_t seed, uint64_t d)
{
    uint32_t ctr[4] = {(uint32_t)d, (uint32_t)(d >> 32), 0x53485546u, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t x[4];
    or_philox4x32_10(ctr, key, x);
    return ((uint64_t)x[1] << 32) | x[0];
}

/* ------------------------------------------------------------------------ */
/* SHA-256 (FIPS 180-4, section 6.2).                                        */
/* ------------------------------------------------------------------------ */

static const uint32_t SHA_K[64] = {
    0x428a2f98, 0x71374491, 0xb5c0fbcf, 0xe9b5dba5, 0x3956c25b, 0x59f111f1, 0x923f82a4, 0xab1c5ed5,
    0xd807aa98, 0x12835b01, 0x243185be, 0x550c7dc3, 0x72be5d74, 0x80deb1fe, 0x9bdc06a7, 0xc19bf174,
    0xe49b69c1, 0xefbe4786, 0x0fc19dc6, 0x240ca1cc, 0x2de92c6f, 0x4a7484aa, 0x5cb0a9dc, 0x76f988da,
    0x983e5152, 0xa831c66d, 0xb00327c8, 0xbf597fc7, 0xc6e00bf3, 0xd5a79147, 0x06ca6351, 0x14292967,
    0x27b70a85, 0x2e1b2138, 0x4d2c6dfc, 0x53380d13, 0x650a7354, 0x766a0abb, 0x81c2c92e, 0x92722c85,
    0xa2bfe8a1, 0xa81a664b, 0xc24b8b70, 0xc76c51a3, 0xd192e819, 0xd6990624, 0xf40e3585, 0x106aa070,
    0x19a4c116, 0x1e376c08, 0x2748774c, 0x34b0bcb5, 0x391c0cb3, 0x4ed8aa4a, 0x5b9cca4f, 0x682e6ff3,
    0x748f82ee, 0x78a5636f, 0x84c87814, 0x8cc70208, 0x90befffa, 0xa4506ceb, 0xbef9a3f7, 0xc67178f2,
};

static uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

static void sha_block(uint32_t H[8], const uint8_t blk[64])
{
    uint32_t W[64];
    for (int t = 0; t < 16; t++)
        W[t] = ((uint32_t)blk[4 * t] << 24) | ((uint32_t)blk[4 * t + 1] << 16) |
               ((uint32_t)blk[4 * t + 2] << 8) | (uint32_t)blk[4 * t + 3];
    for (int t = 16; t < 64; t++) {
        uint32_t s0 = rotr(W[t - 15], 7) ^ rotr(W[t - 15], 18) ^ (W[t - 15] >> 3);
        uint32_t s1 = rotr(W[t - 2], 17) ^ rotr(W[t - 2], 19) ^ (W[t - 2] >> 10);
        W[t] = W[t - 16] + s0 + W[t - 7] + s1;
    }
    uint32_t a = H[0], b = H[1], c = H[2], d = H[3], e = H[4], f = H[5], g = H[6], h = H[7];
    for (int t = 0; t < 64; t++) {
        uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
        uint32_t ch = (e & f) ^ (~e & g);
        uint32_t T1 = h + S1 + ch + SHA_K[t] + W[t];
        uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
        uint32_t maj = (a & b) ^ (a & c) ^ (b & c);
        uint32_t T2 = S0 + maj;
        h = g; g = f; f = e; e = d + T1;
        d = c; c = b; b = a; a = T1 + T2;
    }
    H[0] += a; H[1] += b; H[2] += c; H[3] += d;
    H[4] += e; H[5] += f; H[6] += g; H[7] += h;
}

void or_sha256(const uint8_t *msg, uint64_t len, uint8_t out[32])
{
    uint32_t H[8] = {0x6a09e667, 0xbb67ae85, 0x3c6ef372, 0xa54ff53a,
                     0x510e527f, 0x9b05688c, 0x1f83d9ab, 0x5be0cd19};
    uint64_t full = len / 64;
    for (uint64_t i = 0; i < full; i++)
        sha_block(H, msg + 64 * i);
    uint8_t tail[128];
    memset(tail, 0, sizeof tail);
    uint64_t rem = len - 64 * full;
    memcpy(tail, msg + 64 * full, rem);
    tail[rem] = 0x80;
    uint64_t tail_len = (rem + 1 + 8 <= 64) ? 64 : 128;
    uint64_t bits = len * 8;
    for (int i = 0; i < 8; i++)
        tail[tail_len - 1 - i] = (uint8_t)(bits >> (8 * i));
    for (uint64_t off = 0; off < tail_len; off += 64)
        sha_block(H, tail + off);
    for (int i = 0; i < 8; i++) {
        out[4 * i] = (uint8_t)(H[i] >> 24);
        out[4 * i + 1] = (uint8_t)(H[i] >> 16);
        out[4 * i + 2] = (uint8_t)(H[i] >> 8);
        out[4 * i + 3] = (uint8_t)H[i];
    }
}

/* ------------------------------------------------------------------------ */
/* C6 (recipe part). Largest-remainder apportionment of the B windows of an  */
/* update over the sources: n_s = floor(B·w_s/W), the B − Σn_s leftover      */
/* seats one each to the largest remainders (B·w_s mod W), ties to the lower */
/* source.  The same n_s holds for every update, so each update holds each   */
/* source within one window of its share ([NS] Concepts asks for two).       */
/* ------------------------------------------------------------------------ */

int or_apportion(uint32_t B, uint32_t S, const uint64_t *w, uint32_t *n)
{
    u128 W = 0;
    for (uint32_t s = 0; s < S; s++) W += w[s];
    if (W == 0 || W >> 64) return OR_E_INVAL;
    uint64_t *rem = (uint64_t *)malloc(sizeof(uint64_t) * (S ? S : 1));
    uint8_t *got = (uint8_t *)calloc(S ? S : 1, 1);
    if (!rem || !got) { free(rem); free(got); return OR_E_NOMEM; }
    uint64_t given = 0;
    for (uint32_t s = 0; s < S; s++) {
        u128 q = (u128)B * w[s];
        n[s] = (uint32_t)(q / W);
        rem[s] = (uint64_t)(q % W);
        given += n[s];
    }
    for (uint64_t left = B - given; left > 0; left--) {
        int best = -1;
        for (uint32_t s = 0; s < S; s++) {
            if (got[s]) continue;
            if (best < 0 || rem[s] > rem[best]) best = (int)s;
        }
        got[best] = 1;
        n[best] += 1;
    }
    free(rem);
    free(got);
    return OR_OK;
}

/* C6 (interleave). The update's slots hold items (s, k), k < n_s, ordered by
 * (2k+1)/(2·n_s) ascending (Sainte-Laguë/Webster order), ties to the lower
 * source: the sources are spread through the update rather than in blocks. */
typedef struct { uint32_t s, k, n; } slot_item;

static int cmp_slot(const void *pa, const void *pb)
{
    const slot_item *a = (const slot_item *)pa, *b = (const slot_item *)pb;
    uint64_t lhs = (2ull * a->k + 1) * (uint64_t)b->n;
    uint64_t rhs = (2ull * b->k + 1) * (uint64_t)a->n;
    if (lhs != rhs) return lhs < rhs ? -1 : 1;
    if (a->s != b->s) return a->s < b->s ? -1 : 1;
    return 0;
}

int or_slot_table(uint32_t B, uint32_t S, const uint32_t *n, uint32_t *slot_src, uint32_t *slot_k)
{
    slot_item *it = (slot_item *)malloc(sizeof(slot_item) * (B ? B : 1));
    if (!it) return OR_E_NOMEM;
    uint32_t m = 0;
    for (uint32_t s = 0; s < S; s++)
        for (uint32_t k = 0; k < n[s]; k++) {
            it[m].s = s; it[m].k = k; it[m].n = n[s];
            m++;
        }
    if (m != B) { free(it); return OR_E_INVAL; }
    qsort(it, m, sizeof(slot_item), cmp_slot);
    for (uint32_t j = 0; j < m; j++) { slot_src[j] = it[j].s; slot_k[j] = it[j].k; }
    free(it);
    return OR_OK;
}

/* C6c. Cumulative mixture of a cycle ([NS] Concepts: every update holds each
 * source within two samples of its recipe share; max_epochs 1, so every
 * source's windows are to be trained, small shares included).  Reading: the
 * cycle's updates are one schedule; after u updates source s has taken
 * A_s(u) windows with floor(u·B·w_s/W) ≤ A_s(u) ≤ ceil(u·B·w_s/W) and
 * A_s(u) ≥ A_s(u−1).  Each update's count A_s(u+1) − A_s(u) is then within
 * two of B·w_s/W, and a source whose share is below one window per update
 * still gets its windows, spread over the cycle.
 * Source s's j-th window of the cycle (j ≥ 1) is released in update
 * floor((j−1)·W/(B·w_s)) (from there on taking it keeps A_s within the upper
 * quota) and is due by update ceil(j·W/(B·w_s)) − 1 (the lower quota at the
 * next boundary needs it).  Update u takes the B released, not yet taken
 * windows with the earliest due updates, ties to the lower source, then the
 * lower j: earliest deadline first.  A seat-by-seat schedule within quota at
 * every house size exists (Balinski and Young's quota method, 1975), so one
 * within quota at every update boundary does, and earliest deadline first
 * meets every deadline of unit jobs whenever some schedule does: a missed
 * deadline or an update with fewer than B released windows is an internal
 * error here, never expected.
 * The cycle has u_cfg updates, or (u_cfg = 0) the most after which no source
 * has taken more than its rem_s remaining windows.  Writes A [(U+1)·S] (A must
 * hold (cap+1)·S entries, cap ≥ the updates it can run) and returns U, or 0
 * when even one update does not fit (the caller reports exhaustion). */
typedef struct { u128 due; uint32_t s; uint32_t j; } due_item;

static int cmp_due(const void *pa, const void *pb)
{
    const due_item *a = (const due_item *)pa, *b = (const due_item *)pb;
    if (a->due != b->due) return a->due < b->due ? -1 : 1;
    if (a->s != b->s) return a->s < b->s ? -1 : 1;
    if (a->j != b->j) return a->j < b->j ? -1 : 1;
    return 0;
}

/* With a batch-size ramp (C6b) each update has its own batch and the quotas
 * are taken at H(u) = seats (windows) before update u.  The batches continue
 * past the cycle (the ramp's last piece forever), so a window's due update is
 * the same whatever the cycle's length: window j of s is released in the first
 * update u with j ≤ ceil(H(u+1)·w_s/W) and due by the first update v with
 * H(v+1)·w_s ≥ j·W.  The batches are given as spans: from update first[k]
 * on, batch[k] windows per update, slot0[k] seats before update first[k]; the
 * last span has no end. */
typedef struct { uint64_t first, slot0; uint32_t batch; } or_span;

static u128 seats_before(const or_span *sp, uint32_t n, u128 v)   /* H(v) */
{
    uint32_t k = 0;
    while (k + 1 < n && sp[k + 1].first <= v) k++;
    return (u128)sp[k].slot0 + (v - sp[k].first) * (u128)sp[k].batch;
}

/* the first update v ≥ from with H(v+1) ≥ X: in span k, H(v+1) = slot0_k +
 * (v + 1 − first_k)·batch_k, so the first such v of the span follows by a
 * ceiling division; spans are tried in order */
static u128 first_reaching(const or_span *sp, uint32_t n, u128 from, u128 X)
{
    for (uint32_t k = 0; k < n; k++) {
        const u128 f = sp[k].first, end = (k + 1 < n) ? (u128)sp[k + 1].first : ~(u128)0;
        if (end <= from) continue;
        u128 v = f;                                              /* H(f+1) = slot0 + batch */
        if (X > (u128)sp[k].slot0 + sp[k].batch) v = f + (X - sp[k].slot0 + sp[k].batch - 1) / sp[k].batch - 1;
        if (v < from) v = from;
        if (v < end) return v;
    }
    return ~(u128)0;
}

int or_cumulative_s(const or_span *sp, uint32_t n_sp, uint32_t S, const uint64_t *w, const uint64_t *rem,
                    uint64_t u_cfg, uint64_t cap, uint32_t *A, uint64_t *U_out)
{
    u128 W = 0;
    for (uint32_t s = 0; s < S; s++) W += w[s];
    if (W == 0 || W >> 64 || n_sp == 0) return OR_E_INVAL;
    *U_out = 0;
    for (uint32_t s = 0; s < S; s++) A[s] = 0;
    uint32_t Bmax = 0;
    for (uint32_t k = 0; k < n_sp; k++) {
        if (sp[k].batch == 0) return OR_E_INVAL;
        if (sp[k].batch > Bmax) Bmax = sp[k].batch;
    }
    due_item *it = (due_item *)malloc(sizeof(due_item) * ((uint64_t)Bmax + S + 1));
    if (!it) return OR_E_NOMEM;
    uint64_t U = 0;
    for (uint64_t u = 0; u < cap && (u_cfg == 0 || u < u_cfg); u++) {
        const uint32_t *a = A + u * S;
        uint32_t *an = A + (u + 1) * S;
        const u128 Hn = seats_before(sp, n_sp, (u128)u + 1);
        const uint64_t Bu = (uint64_t)(Hn - seats_before(sp, n_sp, u));
        /* released, not yet taken windows of every source with their due updates */
        uint64_t m = 0;
        for (uint32_t s = 0; s < S; s++) {
            if (w[s] == 0) continue;
            u128 q = Hn * w[s];
            u128 hi = (q + W - 1) / W;                    /* ceil(H(u+1)·w_s/W) */
            for (u128 j = (u128)a[s] + 1; j <= hi; j++) {
                /* due: the first update v ≥ u with H(v+1)·w_s ≥ j·W, i.e. H(v+1) ≥ ceil(j·W/w_s) */
                it[m].due = first_reaching(sp, n_sp, u, (j * W + w[s] - 1) / w[s]);
                it[m].s = s;
                it[m].j = (uint32_t)j;
                m++;
            }
        }
        if (m < Bu) { free(it); return OR_E_INTERNAL; }
        qsort(it, m, sizeof(due_item), cmp_due);
        for (uint32_t s = 0; s < S; s++) an[s] = a[s];
        for (uint64_t r = 0; r < Bu; r++) an[it[r].s] += 1;
        for (uint64_t r = Bu; r < m; r++)
            if (it[r].due <= u) { free(it); return OR_E_INTERNAL; }  /* deadline missed */
        int fits = 1;
        for (uint32_t s = 0; s < S; s++)
            if (an[s] > rem[s]) fits = 0;
        if (!fits) break;
        U = u + 1;
    }
    free(it);
    *U_out = U;
    return OR_OK;
}

/* B windows in every update: one span. */
int or_cumulative(uint32_t B, uint32_t S, const uint64_t *w, const uint64_t *rem, uint64_t u_cfg,
                  uint64_t cap, uint32_t *A, uint64_t *U_out)
{
    const or_span sp = {0, 0, B};
    return or_cumulative_s(&sp, 1, S, w, rem, u_cfg, cap, A, U_out);
}

/* Bs[0..cap) windows in the first updates, the last batch continuing after them. */
int or_cumulative_b(uint32_t B, const uint32_t *Bs, uint32_t S, const uint64_t *w, const uint64_t *rem,
                    uint64_t u_cfg, uint64_t cap, uint32_t *A, uint64_t *U_out)
{
    if (!Bs) return or_cumulative(B, S, w, rem, u_cfg, cap, A, U_out);
    or_span *sp = (or_span *)malloc(sizeof(or_span) * (cap ? cap : 1));
    if (!sp) return OR_E_NOMEM;
    uint32_t n = 0;
    uint64_t seats = 0;
    for (uint64_t u = 0; u < cap; u++) {
        if (n == 0 || sp[n - 1].batch != Bs[u]) sp[n++] = (or_span){u, seats, Bs[u]};
        seats += Bs[u];
    }
    int rc = n ? or_cumulative_s(sp, n, S, w, rem, u_cfg, cap, A, U_out) : OR_E_INVAL;
    free(sp);
    return rc;
}



/* ------------------------------------------------------------------------ */
/* The plan of a corpus: C1–C6 over every document.                          */
/* ------------------------------------------------------------------------ */

typedef struct {
    const uint32_t *tokens;
    uint64_t n_tokens;
    const uint64_t *offsets;     /* [n_docs+1] */
    uint64_t n_docs;
    const uint16_t *source;      /* [n_docs] */
    const uint16_t *stratum;     /* [n_docs] */
    const uint32_t *prompt_len;  /* [n_docs] or NULL (all 0) */
    uint32_t n_sources;
    const uint32_t *n_strata;    /* [S] */
    const uint64_t *weight;      /* [S] */
    const uint32_t *bp;          /* [S] */
    uint32_t T, B;
    uint64_t seed;
    uint32_t pad_token;
    uint32_t wrap;               /* 0: next-fit cut at document ends; 1: wrap (C5w) */
    uint32_t heldout;            /* 1: the stream is the held-out documents (C2v) */
    uint32_t read_random;        /* 1: each cycle's windows of a source read in a random order (C6r) */
    uint32_t cumulative;         /* 1: per-update counts from the cycle's cumulative quotas (C6c) */
    uint32_t n_ramp;             /* 0: every update has B windows; else pieces of a batch-size ramp (C6b) */
    const uint64_t *ramp_from;   /* [n_ramp] tokens trained at which each piece starts (first 0, rising) */
    const uint64_t *ramp_tokens; /* [n_ramp] tokens per update within the piece (a multiple of T) */
    uint32_t lanes;              /* 0 or 1: no lanes; L > 1: Zephon lanes (C2l) */
    const uint64_t *start_tokens;/* [streams] or NULL: first token of each stream to cut (C5s) */
    uint32_t first_cycle;        /* number of the first cycle planned */
    uint64_t tokens_start;       /* tokens trained before the first cycle (C6b) */
    const uint16_t *segment;     /* [n_docs] or NULL: arrival of each document (C3a) */
    uint32_t n_segments;         /* arrivals (0 or 1: one) */
} or_corpus;

typedef struct {
    or_corpus c;
    uint64_t *hash;              /* [D] */
    uint8_t *keep;               /* [D] */
    uint64_t n_kept;
    uint32_t *order;             /* [n_kept]: source by source, merged order */
    uint64_t *src_doc_start;     /* [S+1] */
    uint64_t n_pieces;
    uint32_t *pc_doc, *pc_off, *pc_len, *pc_woff;   /* [n_pieces] */
    uint64_t *pc_spos;           /* [n_pieces] position of the piece's first token in its source's stream */
    uint64_t *src_piece_start;   /* [S+1] */
    uint64_t n_windows;
    uint64_t *win_first;         /* [n_windows+1] first piece of each window */
    uint64_t *src_win_start;     /* [S+1] */
    uint64_t *win_real;          /* [n_windows] real (non-padding) positions */
    uint64_t *win_learn;         /* [n_windows] learned positions */
    uint32_t *n_upd;             /* [S] windows per update */
    uint32_t *slot_src, *slot_k; /* [B] */
    uint64_t *kept_docs, *kept_tokens, *held_docs, *held_tokens; /* [S] */
    uint64_t order_check, hash_check;
    /* cycle state */
    int64_t cycle;               /* -1 before the first cycle */
    uint32_t U;                  /* updates in the current cycle */
    uint64_t *cyc_start;         /* [S] first window of the current cycle */
    uint64_t *cyc_next;          /* [S] first window of the next cycle */
    uint64_t *perm_start;        /* [S+1] with read_random: start of each source's part of perm */
    uint32_t *perm;              /* [U·B] with read_random: read order within each source's cycle range */
    uint64_t *taken;             /* [S] windows the current cycle takes from each source */
    uint32_t *ramp_n;            /* [n_ramp·S] with a ramp: the fixed apportionment of each piece's batch */
    uint64_t tokens_done;        /* tokens (positions) of every update of the cycles before the current one */
    uint32_t *upd_B;             /* [U] windows of each update of the current cycle */
    uint64_t *upd_slot0;         /* [U+1] first slot of each update (prefix of upd_B) */
    uint32_t *cum_A;             /* [(U+1)·S] tabled: windows of s taken before update u */
    uint32_t *tab_src, *tab_i;   /* [Σ upd_B] tabled: each slot's source and cycle window index */
    /* C2l lanes: the plan runs over V = S·L streams (source s, lane l) = s·L + l;
     * the recipe's own arrays stay for the per-lane mixture */
    uint32_t lanes, S_real;
    const uint64_t *w_real;
    uint16_t *v_source;
    uint32_t *v_strata, *v_bp;
    uint64_t *v_weight;
} or_plan;

/* Cycle mode: per-update tables (a ramp or the cumulative mixture) or the
 * fixed apportionment with one slot table. */
static int tabled(const or_corpus *c) { return c->cumulative || c->n_ramp > 0; }

/* C6b. Batch-size ramp ([NS] Training, Updates: tokens_per_update is one
 * number or pieces by the tokens trained; the batch of an update is read at
 * the data line's token count, the cycle's start token plus its updates so
 * far).  Reading: the tokens trained are the positions (B·T per update) of
 * every earlier update, from 0 at cycle 0; an update starting at count t has
 * the batch of the last piece whose start is ≤ t: tokens/T windows. */
static uint32_t ramp_piece(const or_corpus *c, uint64_t t)
{
    uint32_t k = 0;
    while (k + 1 < c->n_ramp && c->ramp_from[k + 1] <= t) k++;
    return k;
}

typedef struct { uint32_t group; uint32_t d; uint64_t key; } sort_item;

static int cmp_sort(const void *pa, const void *pb)
{
    const sort_item *a = (const sort_item *)pa, *b = (const sort_item *)pb;
    if (a->group != b->group) return a->group < b->group ? -1 : 1;
    if (a->key != b->key) return a->key < b->key ? -1 : 1;
    if (a->d != b->d) return a->d < b->d ? -1 : 1;
    return 0;
}

static uint64_t doc_len(const or_corpus *c, uint64_t d) { return c->offsets[d + 1] - c->offsets[d]; }
static uint32_t doc_prompt(const or_corpus *c, uint64_t d) { return c->prompt_len ? c->prompt_len[d] : 0u; }

void or_plan_free(or_plan *p);

#define ALLOC(ptr, count) do { (ptr) = calloc((count) ? (count) : 1, sizeof(*(ptr))); if (!(ptr)) goto nomem; } while (0)

or_plan *or_plan_build(const or_corpus *cin, int *err)
{
    *err = OR_OK;
    or_plan *p = (or_plan *)calloc(1, sizeof(or_plan));
    if (!p) { *err = OR_E_NOMEM; return NULL; }
    p->c = *cin;
    sort_item *items = NULL;
    uint32_t *gbase = NULL;
    /* C2l. Lanes ([ZE] "lanes instead of ranks": the data are split into a fixed
     * number of logical streams, each with its own ordered samples and its own
     * packing state; a rank takes whole lanes).  Reading: document d belongs to
     * lane d mod L; each (source, lane) is a stream planned as a source is
     * (shuffle, strata merge, cut), numbered s·L + l; each update gives lane l
     * its B/L consecutive slots, l·B/L onwards, apportioned over the sources
     * like a batch of B/L (C6), and the recipe's hold-out rate and weight apply
     * to every lane of a source. */
    p->lanes = cin->lanes > 1 ? cin->lanes : 1;
    p->S_real = cin->n_sources;
    p->w_real = cin->weight;
    if (p->lanes > 1) {
        const uint32_t L = p->lanes, V = cin->n_sources * L;
        if (cin->B % L || V > 65535) { *err = OR_E_INVAL; free(p); return NULL; }
        for (uint32_t k = 0; k < cin->n_ramp; k++)
            if ((cin->ramp_tokens[k] / cin->T) % L) { *err = OR_E_INVAL; free(p); return NULL; }
        p->v_source = calloc(cin->n_docs ? cin->n_docs : 1, sizeof(uint16_t));
        p->v_strata = calloc(V, sizeof(uint32_t));
        p->v_bp = calloc(V, sizeof(uint32_t));
        p->v_weight = calloc(V, sizeof(uint64_t));
        if (!p->v_source || !p->v_strata || !p->v_bp || !p->v_weight) {
            free(p->v_source); free(p->v_strata); free(p->v_bp); free(p->v_weight); free(p);
            *err = OR_E_NOMEM;
            return NULL;
        }
        for (uint64_t d = 0; d < cin->n_docs; d++) p->v_source[d] = (uint16_t)(cin->source[d] * L + d % L);
        for (uint32_t v = 0; v < V; v++) {
            p->v_strata[v] = cin->n_strata[v / L];
            p->v_bp[v] = cin->bp[v / L];
            p->v_weight[v] = cin->weight[v / L];
        }
        p->c.source = p->v_source;
        p->c.n_strata = p->v_strata;
        p->c.bp = p->v_bp;
        p->c.weight = p->v_weight;
        p->c.n_sources = V;
    }
    const or_corpus *c = &p->c;
    const uint64_t D = c->n_docs;
    const uint32_t S = c->n_sources, T = c->T;

    if (T == 0 || c->B == 0 || S == 0) { *err = OR_E_INVAL; or_plan_free(p); return NULL; }
    if (c->cumulative) {   /* C6c: every nonzero share at least 2^-62 of the weights (due updates in 64 bits) */
        u128 Wt = 0;
        for (uint32_t r = 0; r < p->S_real; r++) Wt += p->w_real[r];
        for (uint32_t r = 0; r < p->S_real; r++)
            if (p->w_real[r] && ((u128)p->w_real[r] << 62) <= Wt) { *err = OR_E_INVAL; or_plan_free(p); return NULL; }
    }
    ALLOC(p->hash, D); ALLOC(p->keep, D);
    ALLOC(p->src_doc_start, S + 1); ALLOC(p->src_piece_start, S + 1); ALLOC(p->src_win_start, S + 1);
    ALLOC(p->n_upd, S); ALLOC(p->slot_src, c->B); ALLOC(p->slot_k, c->B);
    ALLOC(p->kept_docs, S); ALLOC(p->kept_tokens, S); ALLOC(p->held_docs, S); ALLOC(p->held_tokens, S);
    ALLOC(p->cyc_start, S); ALLOC(p->cyc_next, S); ALLOC(p->taken, S);

    /* C1 + C2: hash every document, decide hold-out; a kept document is one
     * that is not held out and has at least one token.
     * C2v (heldout): the validation stream.  [NS] Concepts: each source's
     * validation rows come from its held-out documents of every stratum, and
     * the validation mix weights the sources by the recipe.  Reading: the same
     * plan (shuffle, strata merge, cut, mixture) over the non-empty held-out
     * documents instead of the kept ones; kept_* then count the stream's
     * documents, held_* still the documents the hash holds out. */
    p->n_kept = 0;
    for (uint64_t d = 0; d < D; d++) {
        uint64_t L = doc_len(c, d);
        uint32_t s = c->source[d];
        p->hash[d] = or_doc_hash(c->tokens + c->offsets[d], L);
        int held = or_held(p->hash[d], c->bp[s]);
        p->keep[d] = (uint8_t)((c->heldout ? held : !held) && L > 0);
        if (held) { p->held_docs[s]++; p->held_tokens[s] += L; }
        if (p->keep[d]) { p->kept_docs[s]++; p->kept_tokens[s] += L; p->n_kept++; p->hash_check += p->hash[d]; }
    }

    /* C3: per (source, stratum) group, kept documents ordered by
     * (shuffle key, input index).  Groups are numbered source-major.
     * C3a. Streamed corpora ([NS] Concepts: a data line's cycles are each
     * downloaded, tokenized, trained on and deleted; a file's documents are
     * shuffled at tokenization; the files left open give the rest to the next
     * cycles).  Reading: with arrivals (segments), a document belongs to the
     * arrival it came with; each source's documents are ordered arrival by
     * arrival, each arrival shuffled and strata-merged on its own, so the
     * order of the arrivals so far does not change when more arrive, and the
     * stream of a source goes on from one arrival's rest into the next.  Groups
     * are numbered (source, arrival, stratum). */
    const uint32_t NSEG = c->segment && c->n_segments > 1 ? c->n_segments : 1;
#define SEG_OF(d) (NSEG > 1 ? (uint32_t)c->segment[d] : 0u)
    for (uint64_t d = 0; d < D; d++)
        if (SEG_OF(d) >= NSEG) { *err = OR_E_INVAL; goto fail; }
    ALLOC(gbase, (uint64_t)S * NSEG + 1);   /* first group of each (source, arrival) */
    gbase[0] = 0;
    for (uint32_t u = 0; u < S * NSEG; u++) gbase[u + 1] = gbase[u] + c->n_strata[u / NSEG];
    ALLOC(items, p->n_kept);
    {
        uint64_t m = 0;
        for (uint64_t d = 0; d < D; d++) {
            if (!p->keep[d]) continue;
            items[m].group = gbase[c->source[d] * NSEG + SEG_OF(d)] + c->stratum[d];
            items[m].d = (uint32_t)d;
            items[m].key = or_shuffle_key(c->seed, d);
            m++;
        }
        qsort(items, p->n_kept, sizeof(sort_item), cmp_sort);
    }

    /* C4: within each source, interleave its strata by least consumed token
     * fraction.  Sequential greedy: among strata with documents left, take
     * the head of the stratum k with the smallest a_k / A_k (a_k = tokens
     * already taken from k, A_k = kept tokens of k), ties to the smaller k.
     * [NS] Concepts: every segment holds every stratum at its share of the
     * source's tokens, cut at document ends; shares in proportion to sizes. */
    ALLOC(p->order, p->n_kept);
    {
        uint64_t out = 0, gi = 0;
        for (uint32_t u = 0; u < S * NSEG; u++) {   /* (source, arrival) units in order */
            const uint32_t s = u / NSEG;
            uint32_t K = c->n_strata[s];
            uint64_t *head = calloc(K ? K : 1, sizeof(uint64_t));
            uint64_t *end = calloc(K ? K : 1, sizeof(uint64_t));
            uint64_t *a = calloc(K ? K : 1, sizeof(uint64_t));
            uint64_t *A = calloc(K ? K : 1, sizeof(uint64_t));
            if (!head || !end || !a || !A) { free(head); free(end); free(a); free(A); goto nomem; }
            if (u % NSEG == 0) p->src_doc_start[s] = out;
            for (uint32_t k = 0; k < K; k++) {
                head[k] = gi;
                while (gi < p->n_kept && items[gi].group == gbase[u] + k) {
                    A[k] += doc_len(c, items[gi].d);
                    gi++;
                }
                end[k] = gi;
            }
            for (;;) {
                int best = -1;
                for (uint32_t k = 0; k < K; k++) {
                    if (head[k] == end[k]) continue;
                    if (best < 0) { best = (int)k; continue; }
                    /* a_k / A_k < a_best / A_best  <=>  a_k·A_best < a_best·A_k */
                    u128 lhs = (u128)a[k] * A[best];
                    u128 rhs = (u128)a[best] * A[k];
                    if (lhs < rhs) best = (int)k;
                }
                if (best < 0) break;
                uint32_t d = items[head[best]].d;
                p->order[out++] = d;
                a[best] += doc_len(c, d);
                head[best]++;
            }
            free(head); free(end); free(a); free(A);
        }
        p->src_doc_start[S] = out;
    }
    for (uint64_t i = 0; i < p->n_kept; i++)
        p->order_check += or_mix64((i << 32) ^ (uint64_t)p->order[i]);

    /* C5w, wrap packing ([ZE'] pack_flat(..., algorithm="wrap"); the page
     * gives only the name).  Reading: per source, the merged order's tokens
     * are one stream, cut every T tokens into windows; a document that
     * crosses a cut is split there and continues at the next window's first
     * position (its pieces restart position ids at 0, [LI] Other trainers);
     * only the stream's last window can be short, and its rest is padding.
     * A piece is a maximal run of one document inside one window. */
    /* C5s. A stream cut from a later token ([NS] Training: a branch forks from
     * the state after a trunk cycle; every update has one sequence length, so a
     * new length starts a new cut).  Reading: with start_tokens, stream v's
     * first start_tokens[v] tokens (in its merged order) are already consumed:
     * documents wholly before that point are skipped, the one that straddles it
     * contributes its tokens from there on, and the cut (next-fit or wrap)
     * starts there, as if the stream began at that token. */
#define STREAM_START(s) (c->start_tokens ? c->start_tokens[s] : 0)
    if (c->wrap) {
        uint64_t P = 0, M = 0;
        for (uint32_t s = 0; s < S; s++) {
            uint64_t x = 0, y = 0;  /* stream position of the document; of the next token after the start */
            for (uint64_t i = p->src_doc_start[s]; i < p->src_doc_start[s + 1]; i++) {
                uint64_t L = doc_len(c, p->order[i]);
                uint64_t o = STREAM_START(s) > x ? STREAM_START(s) - x : 0;
                for (; o < L;) {
                    uint64_t room = T - y % T, len = (L - o < room) ? (L - o) : room;
                    P++; o += len; y += len;
                }
                x += L;
            }
            M += (y + T - 1) / T;
        }
        p->n_pieces = P;
        p->n_windows = M;
        ALLOC(p->pc_doc, P); ALLOC(p->pc_off, P); ALLOC(p->pc_len, P); ALLOC(p->pc_woff, P); ALLOC(p->pc_spos, P);
        ALLOC(p->win_first, M + 1); ALLOC(p->win_real, M); ALLOC(p->win_learn, M);
        uint64_t q = 0, w = 0;
        for (uint32_t s = 0; s < S; s++) {
            p->src_piece_start[s] = q;
            p->src_win_start[s] = w;
            uint64_t xd = 0, x = 0;   /* stream position of the document; of the next token after the start */
            for (uint64_t i = p->src_doc_start[s]; i < p->src_doc_start[s + 1]; i++) {
                uint32_t d = p->order[i];
                uint64_t L = doc_len(c, d);
                uint64_t o = STREAM_START(s) > xd ? STREAM_START(s) - xd : 0;
                for (; o < L;) {
                    uint64_t room = T - x % T, len = (L - o < room) ? (L - o) : room;
                    if (x % T == 0) p->win_first[w++] = q;  /* the piece opens a window */
                    p->pc_doc[q] = d; p->pc_off[q] = (uint32_t)o; p->pc_len[q] = (uint32_t)len;
                    p->pc_spos[q] = xd + o;
                    p->pc_woff[q] = (uint32_t)(x % T);
                    q++; o += len; x += len;
                }
                xd += L;
            }
        }
        p->src_piece_start[S] = q;
        p->src_win_start[S] = w;
        p->win_first[M] = q;
    } else {
    /* C5a: split documents into pieces: a document of L ≤ T tokens is one
     * piece; a longer one is floor(L/T) pieces of T tokens plus a tail piece
     * of the rest, if any.  Count first, then fill. */
    {   /* with a stream start (C5s), a straddling document's rest is split the same way */
        uint64_t P = 0;
        for (uint32_t s = 0; s < S; s++) {
            uint64_t xd = 0;
            for (uint64_t i = p->src_doc_start[s]; i < p->src_doc_start[s + 1]; i++) {
                uint64_t L = doc_len(c, p->order[i]);
                uint64_t o = STREAM_START(s) > xd ? STREAM_START(s) - xd : 0;
                if (o < L) P += (L - o + T - 1) / T;
                xd += L;
            }
        }
        p->n_pieces = P;
        ALLOC(p->pc_doc, P); ALLOC(p->pc_off, P); ALLOC(p->pc_len, P); ALLOC(p->pc_woff, P); ALLOC(p->pc_spos, P);
        uint64_t q = 0;
        for (uint32_t s = 0; s < S; s++) {
            p->src_piece_start[s] = q;
            uint64_t xd = 0;
            for (uint64_t i = p->src_doc_start[s]; i < p->src_doc_start[s + 1]; i++) {
                uint32_t d = p->order[i];
                uint64_t L = doc_len(c, d);
                for (uint64_t o = STREAM_START(s) > xd ? STREAM_START(s) - xd : 0; o < L; o += T) {
                    uint64_t len = (L - o < T) ? (L - o) : T;
                    p->pc_doc[q] = d; p->pc_off[q] = (uint32_t)o; p->pc_len[q] = (uint32_t)len;
                    p->pc_spos[q] = xd + o;
                    q++;
                }
                xd += L;
            }
        }
        p->src_piece_start[S] = q;
    }

    /* C5b: next-fit, per source, in order: a piece joins the open window if
     * it still fits in T positions, else the window is closed (its rest is
     * padding) and the piece opens a new one.  [LI] Supervised fine-tuning:
     * batches of exactly T positions, padding the rest; [NS] Concepts:
     * windows cut at document ends. */
    {
        uint64_t M = 0;
        for (uint32_t s = 0; s < S; s++) {
            uint64_t fill = 0; int open = 0;
            for (uint64_t q = p->src_piece_start[s]; q < p->src_piece_start[s + 1]; q++) {
                if (!(open && fill + p->pc_len[q] <= T)) { M++; open = 1; fill = 0; }
                fill += p->pc_len[q];
            }
        }
        p->n_windows = M;
        ALLOC(p->win_first, M + 1); ALLOC(p->win_real, M); ALLOC(p->win_learn, M);
        uint64_t w = 0;
        for (uint32_t s = 0; s < S; s++) {
            p->src_win_start[s] = w;
            uint64_t fill = 0; int open = 0;
            for (uint64_t q = p->src_piece_start[s]; q < p->src_piece_start[s + 1]; q++) {
                if (!(open && fill + p->pc_len[q] <= T)) {
                    p->win_first[w] = q; w++; open = 1; fill = 0;
                }
                p->pc_woff[q] = (uint32_t)fill;
                fill += p->pc_len[q];
            }
        }
        p->src_win_start[S] = w;
        p->win_first[M] = p->src_piece_start[S];
    }
    }  /* next-fit */

    /* Real and learned positions of each window.  A position is learned when
     * its token lies at or after the document's prompt ([LI] Supervised
     * fine-tuning: a prompted example learns only its completion). */
    for (uint64_t w = 0; w < p->n_windows; w++) {
        uint64_t real = 0, learn = 0;
        for (uint64_t q = p->win_first[w]; q < p->win_first[w + 1]; q++) {
            uint64_t o = p->pc_off[q], len = p->pc_len[q];
            uint64_t pl = doc_prompt(c, p->pc_doc[q]);
            uint64_t from = o > pl ? o : pl;
            real += len;
            if (o + len > from) learn += o + len - from;
        }
        p->win_real[w] = real;
        p->win_learn[w] = learn;
    }

    /* C6: per-update counts and the slot table (with lanes: every lane's B/L
     * slots apportioned over the sources, lane after lane). */
    {
        const uint32_t L = p->lanes, Sr = p->S_real, BL = c->B / L;
        uint32_t *nr = calloc(Sr, sizeof(uint32_t)), *ts = calloc(BL, sizeof(uint32_t)), *tk = calloc(BL, 4);
        if (!nr || !ts || !tk) { free(nr); free(ts); free(tk); goto nomem; }
        *err = or_apportion(BL, Sr, p->w_real, nr);
        if (!*err) *err = or_slot_table(BL, Sr, nr, ts, tk);
        if (!*err) {
            for (uint32_t v = 0; v < S; v++) p->n_upd[v] = nr[v / L];
            for (uint32_t l = 0; l < L; l++)
                for (uint32_t j = 0; j < BL; j++) {
                    p->slot_src[l * BL + j] = ts[j] * L + l;
                    p->slot_k[l * BL + j] = tk[j];
                }
        }
        free(nr); free(ts); free(tk);
        if (*err) goto fail;
    }
    if (c->n_ramp) {   /* C6b: each piece's batch B_k = tokens/T, world-independent; B is their largest */
        uint32_t Bmax = 0;
        for (uint32_t k = 0; k < c->n_ramp; k++) {
            uint64_t tk = c->ramp_tokens[k];
            if (tk == 0 || tk % T || tk / T > c->B) { *err = OR_E_INVAL; goto fail; }
            if ((k == 0 && c->ramp_from[0] != 0) || (k > 0 && c->ramp_from[k] <= c->ramp_from[k - 1])) {
                *err = OR_E_INVAL; goto fail;
            }
            if (tk / T > Bmax) Bmax = (uint32_t)(tk / T);
        }
        if (Bmax != c->B) { *err = OR_E_INVAL; goto fail; }
        const uint64_t n_ramp_entries = (uint64_t)c->n_ramp * S;
        ALLOC(p->ramp_n, n_ramp_entries);
        uint32_t *nr = calloc(p->S_real, sizeof(uint32_t));
        if (!nr) goto nomem;
        for (uint32_t k = 0; k < c->n_ramp; k++) {   /* each lane's share of the piece's batch */
            *err = or_apportion((uint32_t)(c->ramp_tokens[k] / T / p->lanes), p->S_real, p->w_real, nr);
            if (*err) { free(nr); goto fail; }
            for (uint32_t v = 0; v < S; v++) p->ramp_n[(uint64_t)k * S + v] = nr[v / p->lanes];
        }
        free(nr);
    }

    p->cycle = (int64_t)c->first_cycle - 1;
    p->U = 0;
    free(items);
    free(gbase);
    return p;
nomem:
    *err = OR_E_NOMEM;
fail:
    free(items);
    free(gbase);
    or_plan_free(p);
    return NULL;
}

void or_plan_free(or_plan *p)
{
    if (!p) return;
    free(p->hash); free(p->keep); free(p->order); free(p->src_doc_start);
    free(p->pc_doc); free(p->pc_off); free(p->pc_len); free(p->pc_woff);
    free(p->src_piece_start); free(p->win_first); free(p->src_win_start);
    free(p->win_real); free(p->win_learn); free(p->n_upd); free(p->slot_src); free(p->slot_k);
    free(p->kept_docs); free(p->kept_tokens); free(p->held_docs); free(p->held_tokens);
    free(p->perm); free(p->perm_start);
    free(p->cyc_start); free(p->cyc_next); free(p->taken);
    free(p->cum_A); free(p->tab_src); free(p->tab_i); free(p->ramp_n); free(p->upd_B); free(p->upd_slot0);
    free(p->v_source); free(p->v_strata); free(p->v_bp); free(p->v_weight); free(p->pc_spos);
    free(p);
}

/* ------------------------------------------------------------------------ */
/* C6 (cycles). Cycle c takes U_c·n_s consecutive windows of each source's   */
/* stream, starting where cycle c−1 ended.  U_c is the configured number of  */
/* updates, or (when 0) the most that every source with n_s > 0 supports.    */
/* Running out is an error, not a second pass ([NS] Concepts: max_epochs 1); */
/* a cycle is a whole number of updates ([NS] Training: updates never span a */
/* cycle end).                                                               */
/* ------------------------------------------------------------------------ */

int or_cycle(or_plan *p, uint32_t cyc, uint32_t updates_cfg)
{
    const uint32_t S = p->c.n_sources, B = p->c.B, T = p->c.T;
    if ((int64_t)cyc != p->cycle + 1) return OR_E_STATE;
    uint64_t *start = calloc(S, sizeof(uint64_t)), *take = calloc(S, sizeof(uint64_t));
    uint64_t *rem = calloc(S, sizeof(uint64_t));
    uint32_t *cA = NULL, *tsrc = NULL, *ti = NULL, *cnt = NULL, *Bs = NULL, *srcb = NULL, *kb = NULL;
    uint64_t *slot0 = NULL;
    const int first = (cyc == p->c.first_cycle);
    const uint64_t t0 = first ? p->c.tokens_start
                              : p->tokens_done + (p->upd_slot0 ? p->upd_slot0[p->U] : (uint64_t)p->U * B) * T;
    int rc = OR_OK;
#define CYC_FAIL(code) do { rc = (code); goto out; } while (0)
    if (!start || !take || !rem) CYC_FAIL(OR_E_NOMEM);
    for (uint32_t s = 0; s < S; s++) {
        start[s] = first ? 0 : p->cyc_next[s];
        rem[s] = p->src_win_start[s + 1] - p->src_win_start[s] - start[s];
    }
    uint64_t U;
    if (tabled(&p->c)) {
        /* C6b / C6c: the cycle's updates one by one, each with its own counts */
        uint64_t total = 0;
        for (uint32_t s = 0; s < S; s++) total += rem[s];
        uint32_t Bmin = B;
        for (uint32_t k = 0; k < p->c.n_ramp; k++)
            if (p->c.ramp_tokens[k] / T < Bmin) Bmin = (uint32_t)(p->c.ramp_tokens[k] / T);
        uint64_t cap = total / Bmin;                 /* every update takes at least Bmin windows */
        if (cap == 0) CYC_FAIL(OR_E_EXHAUSTED);
        if (updates_cfg) cap = updates_cfg;
        if (cap > 0xFFFFFFFFull) cap = 0xFFFFFFFFull;
        Bs = malloc(sizeof(uint32_t) * cap);
        cA = malloc(sizeof(uint32_t) * (cap + 1) * S);
        if (!Bs || !cA) CYC_FAIL(OR_E_NOMEM);
        uint64_t t = t0;                             /* C6b: each update's batch at the tokens trained so far */
        for (uint64_t u = 0; u < cap; u++) {
            Bs[u] = p->c.n_ramp ? (uint32_t)(p->c.ramp_tokens[ramp_piece(&p->c, t)] / T) : B;
            t += (uint64_t)Bs[u] * T;
        }
        if (p->c.cumulative) {
            /* every lane runs the same schedule over the sources with B/L windows
             * per update; it must fit the lane with the fewest windows left */
            const uint32_t L = p->lanes, Sr = p->S_real;
            const uint32_t K = p->c.n_ramp ? p->c.n_ramp : 1;
            or_span *sp = malloc(sizeof(or_span) * K);
            uint32_t *Ar = malloc(sizeof(uint32_t) * (cap + 1) * Sr);
            uint64_t *rr = malloc(sizeof(uint64_t) * Sr);
            if (!sp || !Ar || !rr) { free(sp); free(Ar); free(rr); CYC_FAIL(OR_E_NOMEM); }
            /* the batches of one lane from this cycle on, the ramp's last piece forever */
            uint32_t n = 0;
            if (!p->c.n_ramp) {
                sp[n++] = (or_span){0, 0, B / L};
            } else {
                uint64_t u = 0, tt = t0, seats = 0;
                for (;;) {
                    const uint32_t k = ramp_piece(&p->c, tt);
                    const uint64_t tk = p->c.ramp_tokens[k];
                    sp[n++] = (or_span){u, seats / L, (uint32_t)(tk / T / L)};
                    if (k + 1 == p->c.n_ramp) break;
                    const uint64_t cnt_k = (p->c.ramp_from[k + 1] - tt + tk - 1) / tk;  /* updates in piece k */
                    u += cnt_k; tt += cnt_k * tk; seats += cnt_k * (tk / T);
                }
            }
            for (uint32_t r = 0; r < Sr; r++) {
                rr[r] = UINT64_MAX;
                for (uint32_t l = 0; l < L; l++) if (rem[r * L + l] < rr[r]) rr[r] = rem[r * L + l];
            }
            rc = or_cumulative_s(sp, n, Sr, p->w_real, rr, updates_cfg, cap, Ar, &U);
            if (!rc)
                for (uint64_t u = 0; u <= U; u++)
                    for (uint32_t v = 0; v < S; v++) cA[u * S + v] = Ar[u * Sr + v / L];
            free(sp); free(Ar); free(rr);
            if (rc) goto out;
        } else {   /* fixed apportionment of each update's batch, until a source runs out */
            U = 0;
            for (uint32_t s = 0; s < S; s++) cA[s] = 0;
            uint64_t tu = t0;                        /* tokens trained before update u */
            for (uint64_t u = 0; u < cap; u++) {
                const uint32_t *n = p->ramp_n + (uint64_t)ramp_piece(&p->c, tu) * S;
                tu += (uint64_t)Bs[u] * T;
                int fits = 1;
                for (uint32_t s = 0; s < S; s++) {
                    cA[(u + 1) * S + s] = cA[u * S + s] + n[s];
                    if (cA[(u + 1) * S + s] > rem[s]) fits = 0;
                }
                if (!fits) break;
                U = u + 1;
            }
        }
        if (U == 0 || (updates_cfg && U < updates_cfg)) CYC_FAIL(OR_E_EXHAUSTED);
        for (uint32_t s = 0; s < S; s++) take[s] = cA[U * S + s];
        slot0 = malloc(sizeof(uint64_t) * (U + 1));
        if (!slot0) CYC_FAIL(OR_E_NOMEM);
        slot0[0] = 0;
        for (uint64_t u = 0; u < U; u++) slot0[u + 1] = slot0[u] + Bs[u];
        tsrc = malloc(sizeof(uint32_t) * (slot0[U] ? slot0[U] : 1));
        ti = malloc(sizeof(uint32_t) * (slot0[U] ? slot0[U] : 1));
        cnt = malloc(sizeof(uint32_t) * S);
        srcb = malloc(sizeof(uint32_t) * B);
        kb = malloc(sizeof(uint32_t) * B);
        if (!tsrc || !ti || !cnt || !srcb || !kb) CYC_FAIL(OR_E_NOMEM);
        const uint32_t L = p->lanes, Sr = p->S_real;
        for (uint64_t u = 0; u < U; u++) {   /* each update's slots interleaved as in C6, lane after lane */
            const uint32_t BL = Bs[u] / L;
            for (uint32_t l = 0; l < L; l++) {
                for (uint32_t r = 0; r < Sr; r++) cnt[r] = cA[(u + 1) * S + r * L + l] - cA[u * S + r * L + l];
                rc = or_slot_table(BL, Sr, cnt, srcb, kb);
                if (rc) goto out;
                for (uint32_t j = 0; j < BL; j++) {
                    const uint32_t v = srcb[j] * L + l;
                    tsrc[slot0[u] + l * BL + j] = v;
                    ti[slot0[u] + l * BL + j] = cA[u * S + v] + kb[j];
                }
            }
        }
    } else {
        if (updates_cfg > 0) {
            U = updates_cfg;
        } else {
            U = UINT64_MAX;
            for (uint32_t s = 0; s < S; s++) {
                if (p->n_upd[s] == 0) continue;
                uint64_t u = rem[s] / p->n_upd[s];
                if (u < U) U = u;
            }
        }
        int ok = (U > 0 && U <= 0xFFFFFFFFull);
        for (uint32_t s = 0; ok && s < S; s++)
            if ((u128)U * p->n_upd[s] > (u128)rem[s]) ok = 0;
        if (!ok) CYC_FAIL(OR_E_EXHAUSTED);   /* cycle state unchanged */
        for (uint32_t s = 0; s < S; s++) take[s] = U * p->n_upd[s];
    }
    if (p->c.read_random) {
        /* C6r: for each source, its cycle windows ordered by (key64, i) */
        uint64_t total = 0;
        for (uint32_t s = 0; s < S; s++) total += take[s];
        uint64_t *ps = calloc(S + 1, sizeof(uint64_t));
        uint32_t *perm = calloc(total ? total : 1, sizeof(uint32_t));
        sort_item *it = calloc(total ? total : 1, sizeof(sort_item));
        if (!ps || !perm || !it) { free(ps); free(perm); free(it); CYC_FAIL(OR_E_NOMEM); }
        uint64_t e = 0;
        for (uint32_t s = 0; s < S; s++) {
            ps[s] = e;
            for (uint64_t i = 0; i < take[s]; i++, e++) {
                it[e].group = s;
                it[e].d = (uint32_t)i;
                it[e].key = or_window_key(p->c.seed, s, cyc, (uint32_t)i);
            }
        }
        ps[S] = e;
        qsort(it, total, sizeof(sort_item), cmp_sort);  /* by (source, key64, i) */
        for (uint64_t r = 0; r < total; r++) perm[r] = it[r].d;
        free(it);
        free(p->perm); free(p->perm_start);
        p->perm = perm; p->perm_start = ps;
    }
    p->U = (uint32_t)U;
    p->tokens_done = t0;
    for (uint32_t s = 0; s < S; s++) {
        p->cyc_start[s] = start[s];
        p->cyc_next[s] = start[s] + take[s];
        p->taken[s] = take[s];
    }
    if (tabled(&p->c)) {
        free(p->cum_A); free(p->tab_src); free(p->tab_i); free(p->upd_B); free(p->upd_slot0);
        p->cum_A = cA; p->tab_src = tsrc; p->tab_i = ti; p->upd_B = Bs; p->upd_slot0 = slot0;
        cA = tsrc = ti = Bs = NULL;
        slot0 = NULL;
    }
    p->cycle = cyc;
out:
#undef CYC_FAIL
    free(start); free(take); free(rem); free(cA); free(tsrc); free(ti); free(cnt); free(Bs); free(slot0);
    free(srcb); free(kb);
    return rc;
}

/* Windows of update b of the current cycle. */
static uint32_t upd_batch(const or_plan *p, uint64_t b)
{
    return p->upd_B ? p->upd_B[b] : p->c.B;
}

/* Global window index of slot j of update b of the current cycle. */
uint64_t or_window_of(const or_plan *p, uint64_t b, uint32_t j)
{
    uint32_t s;
    uint64_t i;                                    /* the source's i-th window of the cycle */
    if (tabled(&p->c)) {
        const uint64_t x = p->upd_slot0[b] + j;
        s = p->tab_src[x];
        i = p->tab_i[x];
    } else {
        s = p->slot_src[j];
        i = b * p->n_upd[s] + p->slot_k[j];
    }
    if (p->c.read_random) i = p->perm[p->perm_start[s] + i];
    return p->src_win_start[s] + p->cyc_start[s] + i;
}

/* C7. Emission of one window of T positions.  For a position inside piece
 * (d, o, len) placed at window offset f, with u = position − f: the token
 * tokens[off[d] + o + u], position id u (0 starts each piece: [LI] Other
 * trainers), document id d, mask 1 iff o + u ≥ prompt_len(d).  Other
 * positions are padding: pad token, position 0, document −1, mask 0. */
void or_emit_window(const or_plan *p, uint64_t gw, uint32_t *tok, int32_t *pos, int32_t *doc, uint8_t *mask)
{
    const or_corpus *c = &p->c;
    for (uint32_t t = 0; t < c->T; t++) { tok[t] = c->pad_token; pos[t] = 0; doc[t] = -1; mask[t] = 0; }
    for (uint64_t q = p->win_first[gw]; q < p->win_first[gw + 1]; q++) {
        uint32_t d = p->pc_doc[q], o = p->pc_off[q], len = p->pc_len[q], f = p->pc_woff[q];
        uint32_t pl = doc_prompt(c, d);
        for (uint32_t u = 0; u < len; u++) {
            tok[f + u] = c->tokens[c->offsets[d] + o + u];
            pos[f + u] = (int32_t)u;
            doc[f + u] = (int32_t)d;
            mask[f + u] = (uint8_t)((uint64_t)o + u >= pl);
        }
    }
}

/* C8. Window digest: SHA-256 over tok ‖ pos ‖ doc ‖ mask of the window, the
 * first three as 4-byte little-endian words, the mask as bytes.  [ZE] the
 * SHA-256 of every global batch matches byte for byte across GPU counts;
 * reading: hash per window, then the batch as the SHA-256 of its B window
 * digests in slot order, so each rank hashes its own slice. */
void or_window_digest(uint32_t T, const uint32_t *tok, const int32_t *pos, const int32_t *doc,
                      const uint8_t *mask, uint8_t out[32])
{
    uint8_t *rec = (uint8_t *)malloc(13ull * T);
    memcpy(rec, tok, 4ull * T);
    memcpy(rec + 4ull * T, pos, 4ull * T);
    memcpy(rec + 8ull * T, doc, 4ull * T);
    memcpy(rec + 12ull * T, mask, T);
    or_sha256(rec, 13ull * T, out);
    free(rec);
}

/* Chunked window digest (PACK_FLAG_DIGEST_CHUNKED), a second reading of the
 * window digest above, chosen so that one window's hashing is not one serial
 * chain of 13·T/64 blocks: the same 13·T-byte record is cut into chunks of
 * OR_DIGEST_CHUNK bytes (the last one shorter when 13·T is not a multiple),
 * each chunk is hashed with SHA-256, and the window digest is the SHA-256 of
 * the chunk digests concatenated in record order (32 bytes each).  A record
 * of one chunk (T ≤ 315) thus has SHA-256(SHA-256(record)).  Returns OR_OK or
 * OR_E_NOMEM. */
#define OR_DIGEST_CHUNK 4096u

int or_window_digest_chunked(uint32_t T, const uint32_t *tok, const int32_t *pos, const int32_t *doc,
                             const uint8_t *mask, uint8_t out[32])
{
    const uint64_t n = 13ull * T, nc = (n + OR_DIGEST_CHUNK - 1) / OR_DIGEST_CHUNK;
    uint8_t *rec = (uint8_t *)malloc(n ? n : 1);
    uint8_t *cd = (uint8_t *)malloc(32 * (nc ? nc : 1));
    if (!rec || !cd) { free(rec); free(cd); return OR_E_NOMEM; }
    memcpy(rec, tok, 4ull * T);
    memcpy(rec + 4ull * T, pos, 4ull * T);
    memcpy(rec + 8ull * T, doc, 4ull * T);
    memcpy(rec + 12ull * T, mask, T);
    for (uint64_t i = 0; i < nc; i++) {
        const uint64_t at = i * OR_DIGEST_CHUNK;
        or_sha256(rec + at, n - at < OR_DIGEST_CHUNK ? n - at : OR_DIGEST_CHUNK, cd + 32 * i);
    }
    or_sha256(cd, 32 * nc, out);
    free(rec);
    free(cd);
    return OR_OK;
}

/* The chunked digests of n windows laid out [n][T] each array ([n][32] out). */
int or_window_digests_chunked(uint32_t T, uint64_t n, const uint32_t *tok, const int32_t *pos,
                              const int32_t *doc, const uint8_t *mask, uint8_t *out)
{
    for (uint64_t w = 0; w < n; w++) {
        const uint64_t at = w * T;
        const int rc = or_window_digest_chunked(T, tok + at, pos + at, doc + at, mask + at, out + 32 * w);
        if (rc) return rc;
    }
    return OR_OK;
}

/* One call of the batch entry: updates [step, step+n_steps) of the current
 * cycle, rank `rank` of `world` owning slots [rank·B/world, (rank+1)·B/world).
 * Outputs are [n_steps][B/world][T]; learned is the global per-update count;
 * digests (optional) are [n_steps][B/world][32]. */
int or_batch(const or_plan *p, uint32_t step, uint32_t n_steps, uint32_t rank, uint32_t world,
             uint32_t *tok, int32_t *pos, int32_t *doc, uint8_t *mask, int64_t *learned,
             uint8_t *digests)
{
    const uint32_t T = p->c.T;
    if (p->cycle < (int64_t)p->c.first_cycle) return OR_E_STATE;
    if (world == 0 || rank >= world || p->c.B % world) return OR_E_INVAL;
    if ((uint64_t)step + n_steps > p->U) return OR_E_RANGE;
    uint64_t w = 0;   /* this rank's windows, update after update (B_b/world of update b) */
    for (uint32_t i = 0; i < n_steps; i++) {
        uint64_t b = (uint64_t)step + i;
        const uint32_t Bb = upd_batch(p, b);
        if (Bb % world) return OR_E_INVAL;
        const uint32_t per = Bb / world;
        for (uint32_t jj = 0; jj < per; jj++, w++) {
            uint32_t j = rank * per + jj;
            uint64_t gw = or_window_of(p, b, j);
            uint64_t at = w * T;
            or_emit_window(p, gw, tok + at, pos + at, doc + at, mask + at);
            if (digests)
                or_window_digest(T, tok + at, pos + at, doc + at, mask + at, digests + w * 32);
        }
        if (learned) {
            int64_t sum = 0;
            for (uint32_t j = 0; j < Bb; j++) sum += (int64_t)p->win_learn[or_window_of(p, b, j)];
            learned[i] = sum;
        }
    }
    return OR_OK;
}

/* C7p. Padding-free rows ([LI] Supervised fine-tuning, the transformers
 * Trainer path: the padding is removed and the rows are packed into one
 * sequence whose length rounds up to a multiple of bucket, 256, so few shapes
 * compile; a position id 0 starts each sequence).  Reading: for each update,
 * this rank's windows, in slot order, give their real positions (the window's
 * first win_real positions) one after another in one row; row_start[jj] is
 * where window jj begins, row_start[per] their total; the row's length is that
 * total rounded up to a multiple of bucket (none for bucket ≤ 1), at most
 * per·T, and its positions past the total are padding.  Positions of the
 * row buffer past the length are left as padding here (callers use the length).
 * With a batch-size ramp rows are B/world·T positions apart (B the largest
 * batch), row_start rows B/world + 1 long; update b fills its first
 * B_b/world + 1 entries and repeats the total in the rest. */
int or_batch_packed(const or_plan *p, uint32_t step, uint32_t n_steps, uint32_t rank, uint32_t world,
                    uint32_t bucket, uint32_t *tok, int32_t *pos, int32_t *doc, uint8_t *mask,
                    int64_t *row_start, int64_t *length)
{
    const uint32_t B = p->c.B, T = p->c.T;
    if (p->cycle < (int64_t)p->c.first_cycle) return OR_E_STATE;
    if (world == 0 || rank >= world || B % world) return OR_E_INVAL;
    if ((uint64_t)step + n_steps > p->U) return OR_E_RANGE;
    const uint32_t pmax = B / world;               /* row pitch: the largest batch's windows */
    const uint64_t pitch = (uint64_t)pmax * T;
    uint32_t *wt = malloc(4ull * T); int32_t *wp = malloc(4ull * T), *wd = malloc(4ull * T); uint8_t *wm = malloc(T);
    if (!wt || !wp || !wd || !wm) { free(wt); free(wp); free(wd); free(wm); return OR_E_NOMEM; }
    for (uint32_t i = 0; i < n_steps; i++) {
        const uint32_t Bb = upd_batch(p, (uint64_t)step + i);
        if (Bb % world) { free(wt); free(wp); free(wd); free(wm); return OR_E_INVAL; }
        const uint32_t per = Bb / world;
        const uint64_t cap = (uint64_t)per * T;
        uint32_t *rt = tok + i * pitch; int32_t *rp = pos + i * pitch, *rd = doc + i * pitch;
        uint8_t *rm = mask + i * pitch;
        int64_t *rs = row_start + (uint64_t)i * (pmax + 1);
        for (uint64_t x = 0; x < cap; x++) { rt[x] = p->c.pad_token; rp[x] = 0; rd[x] = -1; rm[x] = 0; }
        uint64_t at = 0;
        for (uint32_t jj = 0; jj < per; jj++) {
            uint64_t gw = or_window_of(p, (uint64_t)step + i, rank * per + jj);
            uint64_t real = p->win_real[gw];
            rs[jj] = (int64_t)at;
            or_emit_window(p, gw, wt, wp, wd, wm);
            for (uint64_t t = 0; t < real; t++) {
                rt[at + t] = wt[t]; rp[at + t] = wp[t]; rd[at + t] = wd[t]; rm[at + t] = wm[t];
            }
            at += real;
        }
        for (uint32_t jj = per; jj <= pmax; jj++) rs[jj] = (int64_t)at;
        uint64_t L = at;
        if (bucket > 1) L = (at + bucket - 1) / bucket * bucket;
        if (L > cap) L = cap;
        length[i] = (int64_t)L;
    }
    free(wt); free(wp); free(wd); free(wm);
    return OR_OK;
}

/* Plan digest of the current cycle: SHA-256 over a little-endian header (the
 * mode, the recipe's scalars, the cycle, its updates and two order-free sums
 * that change with the document order and content) followed by the digests of
 * the streams' records, 8 streams to a leaf.  A stream's record (60 bytes):
 * weight, hold-out rate, strata, windows per update, windows in the stream,
 * kept documents and tokens, the cycle's first window, the stream's first
 * token (0 without stream starts).  A resume whose digest differs was planned
 * from another recipe or order ([NS] Training: a resume with another sample
 * order is refused). */
#define OR_DIGEST_RECORD 60u
#define OR_DIGEST_LEAF 8u

static void put(uint8_t **w, uint64_t v, int bytes)
{
    for (int i = 0; i < bytes; i++) *(*w)++ = (uint8_t)(v >> (8 * i));
}

int or_plan_digest(const or_plan *p, uint8_t out[32])
{
    const or_corpus *c = &p->c;
    const uint32_t S = c->n_sources;
    if (p->cycle < (int64_t)p->c.first_cycle) return OR_E_STATE;
    const uint32_t leaves = (S + OR_DIGEST_LEAF - 1) / OR_DIGEST_LEAF;
    uint8_t *rec = (uint8_t *)malloc((uint64_t)S * OR_DIGEST_RECORD + 1), *r = rec;
    uint64_t bytes = 8 + 4 + 4 + (16ull * c->n_ramp + 16) + 8 + 4 + 8 + 4 + 4 + 8 + 4 + 4 + 4 + 4 + 8 + 8 + 32ull * leaves;
    uint8_t *buf = (uint8_t *)malloc(bytes), *w = buf;
    if (!rec || !buf) { free(rec); free(buf); return OR_E_NOMEM; }
    for (uint32_t s = 0; s < S; s++) {
        put(&r, c->weight[s], 8); put(&r, c->bp[s], 4); put(&r, c->n_strata[s], 4);
        put(&r, p->n_upd[s], 4);
        put(&r, p->src_win_start[s + 1] - p->src_win_start[s], 8);
        put(&r, p->kept_docs[s], 8); put(&r, p->kept_tokens[s], 8);
        put(&r, p->cyc_start[s], 8);
        put(&r, c->start_tokens ? c->start_tokens[s] : 0, 8);
    }
    /* the packing mode and the stream (training / held-out) are part of the plan */
    memcpy(w, "DPACKP", 6); w += 6;
    *w++ = c->wrap ? 'W' : 'D';
    *w++ = c->heldout ? 'V' : '1';
    if (c->read_random) put(&w, 0x444E4152u, 4);  /* "RAND": windows read in a random order */
    if (c->cumulative) put(&w, 0x554D5543u, 4);   /* "CUMU": per-update counts from cumulative quotas */
    if (c->n_ramp) {                               /* "RAMP": the pieces and the cycle's first token */
        put(&w, 0x504D4152u, 4);
        put(&w, c->n_ramp, 4);
        for (uint32_t k = 0; k < c->n_ramp; k++) { put(&w, c->ramp_from[k], 8); put(&w, c->ramp_tokens[k], 8); }
        put(&w, p->tokens_done, 8);
    }
    if (p->lanes > 1) { put(&w, 0x454E414Cu, 4); put(&w, p->lanes, 4); }  /* "LANE" and the lane count */
    if (c->start_tokens) put(&w, 0x54525453u, 4);  /* "STRT": streams cut from given tokens (in the records) */
    if (c->segment && c->n_segments > 1) { put(&w, 0x53474553u, 4); put(&w, c->n_segments, 4); }  /* "SEGS" */
    put(&w, c->T, 4); put(&w, c->B, 4); put(&w, c->seed, 8); put(&w, S, 4); put(&w, c->pad_token, 4);
    put(&w, (uint64_t)p->cycle, 4); put(&w, p->U, 4);
    put(&w, p->order_check, 8); put(&w, p->hash_check, 8);
    for (uint32_t j = 0; j < leaves; j++) {  /* the records' digests, 8 streams to a leaf */
        const uint32_t s0 = j * OR_DIGEST_LEAF, s1 = s0 + OR_DIGEST_LEAF < S ? s0 + OR_DIGEST_LEAF : S;
        or_sha256(rec + (uint64_t)s0 * OR_DIGEST_RECORD, (uint64_t)(s1 - s0) * OR_DIGEST_RECORD, w);
        w += 32;
    }
    or_sha256(buf, (uint64_t)(w - buf), out);
    free(rec);
    free(buf);
    return OR_OK;
}

/* ---- accessors for the Python wrapper (sizes, arrays, cycle state) ---- */
uint64_t or_plan_sizes(const or_plan *p, uint64_t *n_kept, uint64_t *n_pieces, uint64_t *n_windows)
{
    *n_kept = p->n_kept; *n_pieces = p->n_pieces; *n_windows = p->n_windows;
    return p->c.n_docs;
}

void or_plan_export(const or_plan *p, uint64_t *hash, uint8_t *keep, uint32_t *order,
                    uint64_t *src_doc_start, uint32_t *pc_doc, uint32_t *pc_off, uint32_t *pc_len,
                    uint32_t *pc_woff, uint64_t *src_piece_start, uint64_t *win_first,
                    uint64_t *src_win_start, uint64_t *win_real, uint64_t *win_learn,
                    uint32_t *n_upd, uint32_t *slot_src, uint32_t *slot_k, uint64_t *stats /*[4][S]*/,
                    uint64_t *checks /*[2]*/)
{
    const uint64_t D = p->c.n_docs, S = p->c.n_sources, B = p->c.B;
    memcpy(hash, p->hash, 8 * D); memcpy(keep, p->keep, D);
    memcpy(order, p->order, 4 * p->n_kept); memcpy(src_doc_start, p->src_doc_start, 8 * (S + 1));
    memcpy(pc_doc, p->pc_doc, 4 * p->n_pieces); memcpy(pc_off, p->pc_off, 4 * p->n_pieces);
    memcpy(pc_len, p->pc_len, 4 * p->n_pieces); memcpy(pc_woff, p->pc_woff, 4 * p->n_pieces);
    memcpy(src_piece_start, p->src_piece_start, 8 * (S + 1));
    memcpy(win_first, p->win_first, 8 * (p->n_windows + 1));
    memcpy(src_win_start, p->src_win_start, 8 * (S + 1));
    memcpy(win_real, p->win_real, 8 * p->n_windows); memcpy(win_learn, p->win_learn, 8 * p->n_windows);
    memcpy(n_upd, p->n_upd, 4 * S); memcpy(slot_src, p->slot_src, 4 * B); memcpy(slot_k, p->slot_k, 4 * B);
    memcpy(stats, p->kept_docs, 8 * S); memcpy(stats + S, p->kept_tokens, 8 * S);
    memcpy(stats + 2 * S, p->held_docs, 8 * S); memcpy(stats + 3 * S, p->held_tokens, 8 * S);
    checks[0] = p->order_check; checks[1] = p->hash_check;
}

uint32_t or_cycle_state(const or_plan *p, int64_t *cycle, uint64_t *start /*[S]*/, uint64_t *taken /*[S]*/)
{
    *cycle = p->cycle;
    memcpy(start, p->cyc_start, 8 * p->c.n_sources);
    memcpy(taken, p->taken, 8 * p->c.n_sources);
    return p->U;
}

/* Batches of the current cycle's updates [U] and the tokens trained before it. */
uint64_t or_cycle_batches(const or_plan *p, uint32_t *Bs)
{
    for (uint32_t u = 0; u < p->U; u++) Bs[u] = upd_batch(p, u);
    return p->tokens_done;
}

/* C5s: each stream's token position where the next cycle's windows begin (the
 * stream's total when it is used up): the start_tokens of a context that goes
 * on from here, with this T or another. */
int or_cycle_stream_next(const or_plan *p, uint64_t *out /*[S]*/)
{
    if (p->cycle < (int64_t)p->c.first_cycle) return OR_E_STATE;
    for (uint32_t s = 0; s < p->c.n_sources; s++) {
        const uint64_t M = p->src_win_start[s + 1] - p->src_win_start[s];
        if (p->cyc_next[s] < M) {
            out[s] = p->pc_spos[p->win_first[p->src_win_start[s] + p->cyc_next[s]]];
        } else {
            uint64_t tot = 0;
            for (uint64_t i = p->src_doc_start[s]; i < p->src_doc_start[s + 1]; i++) tot += doc_len(&p->c, p->order[i]);
            out[s] = tot;
        }
    }
    return OR_OK;
}

/* Tabled cycles (a ramp or the cumulative mixture): A [(U+1)·S] of the current cycle. */
int or_cum_export(const or_plan *p, uint32_t *A)
{
    if (!tabled(&p->c) || p->cycle < (int64_t)p->c.first_cycle) return OR_E_STATE;
    memcpy(A, p->cum_A, sizeof(uint32_t) * ((uint64_t)p->U + 1) * p->c.n_sources);
    return OR_OK;
}
