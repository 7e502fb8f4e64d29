/*
 * sanitize_check.c — TEST INFRASTRUCTURE ONLY: a driver that builds the oracle
 * into one program with AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_oracle_sanitize.py compiles and runs it) and calls every entry
 * point of the oracle over seeded random small corpora in every mode: plain,
 * wrap, held-out stream, random read order, cumulative mixture, batch-size
 * ramp, lanes, arrivals, stream starts, prompts, several cycles, rank slices,
 * padding-free rows, window digests (whole and chunked), plan digests and the
 * exported arrays.  Output buffers are
 * allocated to their exact sizes, so a write one element past any of them is
 * reported.  The driver computes nothing of the method itself: it draws inputs
 * with its own SplitMix64 stream and checks return codes.
 *
 * Usage: sanitize_check [cases]   (exit 0 = every case ran without a report)
 */
#include "oracle.c"

#include <stdio.h>

static uint64_t g_rng;
static uint64_t g_plans, g_cycles, g_batches;  /* coverage counts, printed at the end */
static uint64_t rnd(void) { return or_mix64(g_rng += 0x9E3779B97F4A7C15ull); }
static uint32_t rnd_below(uint32_t n) { return n ? (uint32_t)(rnd() % n) : 0; }

static void *zalloc(uint64_t n, size_t size) { return calloc(n > 0 ? n : 1, size); }
#define NEW(type, n) ((type *)zalloc((uint64_t)(n), sizeof(type)))

static int check_cycle(or_plan *p, uint32_t world, uint32_t lanes)
{
    const or_corpus *c = &p->c;
    const uint32_t S = c->n_sources, T = c->T;
    int64_t cyc;
    int bad = 0;
    uint64_t *start = NEW(uint64_t, S), *taken = NEW(uint64_t, S), *next = NEW(uint64_t, S);
    const uint32_t U = or_cycle_state(p, &cyc, start, taken);
    uint32_t *Bs = NEW(uint32_t, U);
    (void)or_cycle_batches(p, Bs);
    uint8_t dig[32];
    if (or_cycle_stream_next(p, next) != OR_OK || or_plan_digest(p, dig) != OR_OK) bad = 1;
    if (c->cumulative || c->n_ramp) {
        uint32_t *A = NEW(uint32_t, ((uint64_t)U + 1) * S);
        if (or_cum_export(p, A) != OR_OK) bad = 1;
        free(A);
    }
    /* a rank count must divide every update's batch */
    int refused = 0;
    for (uint32_t b = 0; b < U; b++) refused |= Bs[b] % world != 0;
    (void)lanes;
    /* every update, then a sampled sub-range, for this rank count */
    for (uint32_t r = 0; r < world && !bad; r++) {
        uint64_t wins = 0;
        for (uint32_t b = 0; b < U; b++) wins += Bs[b] / world;
        uint32_t *tok = NEW(uint32_t, wins * T);
        int32_t *pos = NEW(int32_t, wins * T), *doc = NEW(int32_t, wins * T);
        uint8_t *mask = NEW(uint8_t, wins * T), *dg = NEW(uint8_t, wins * 32);
        int64_t *learned = NEW(int64_t, U);
        int rc = or_batch(p, 0, U, r, world, tok, pos, doc, mask, learned, dg);
        if (rc != (refused ? OR_E_INVAL : OR_OK)) bad = 1;
        g_batches += rc == OR_OK;
        free(tok); free(pos); free(doc); free(mask); free(dg); free(learned);
        if (!c->n_ramp && U) {  /* padding-free rows of one update, two buckets */
            const uint32_t per = c->B / world;
            for (uint32_t bucket = 1; bucket <= 256; bucket += 255) {
                uint32_t *pt = NEW(uint32_t, (uint64_t)per * T);
                int32_t *pp = NEW(int32_t, (uint64_t)per * T), *pd = NEW(int32_t, (uint64_t)per * T);
                uint8_t *pm = NEW(uint8_t, (uint64_t)per * T);
                int64_t *rs = NEW(int64_t, per + 1), len[1];
                rc = or_batch_packed(p, U - 1, 1, r, world, bucket, pt, pp, pd, pm, rs, len);
                if (rc != (refused ? OR_E_INVAL : OR_OK)) bad = 1;
                free(pt); free(pp); free(pd); free(pm); free(rs);
            }
        }
    }
    /* windows one by one through the window lookup and the single-window emission */
    for (uint32_t b = 0; b < U && b < 3; b++)
        for (uint32_t j = 0; j < Bs[b]; j++) {
            uint32_t *tok = NEW(uint32_t, T);
            int32_t *pos = NEW(int32_t, T), *doc = NEW(int32_t, T);
            uint8_t *mask = NEW(uint8_t, T), d[32];
            or_emit_window(p, or_window_of(p, b, j), tok, pos, doc, mask);
            or_window_digest(T, tok, pos, doc, mask, d);
            if (or_window_digests_chunked(T, 1, tok, pos, doc, mask, d) != OR_OK) bad = 1;
            free(tok); free(pos); free(doc); free(mask);
        }
    free(start); free(taken); free(next); free(Bs);
    return bad;
}

static int run_case(uint32_t seed)
{
    g_rng = 0x5A17u + 1000003ull * seed;
    const uint32_t S = 1 + rnd_below(4), L = (seed % 3 == 0) ? 2 : 1;
    const uint32_t D = 20 + rnd_below(380), T = 64u << rnd_below(2), B = L * (1 + rnd_below(4));
    uint32_t *n_strata = NEW(uint32_t, S);
    uint64_t *weight = NEW(uint64_t, S);
    uint32_t *bp = NEW(uint32_t, S);
    for (uint32_t s = 0; s < S; s++) {
        n_strata[s] = 1 + rnd_below(3);
        weight[s] = 1 + rnd_below(1000);
        bp[s] = rnd_below(3000);
    }
    uint64_t *off = NEW(uint64_t, D + 1);
    uint16_t *src = NEW(uint16_t, D), *str = NEW(uint16_t, D), *seg = NEW(uint16_t, D);
    uint32_t *pl = NEW(uint32_t, D);
    for (uint32_t d = 0; d < D; d++) {  /* documents by (source, stratum), lengths 0 .. 3T */
        src[d] = (uint16_t)((uint64_t)d * S / D);
        str[d] = (uint16_t)rnd_below(n_strata[src[d]]);
        const uint32_t len = rnd_below(8) == 0 ? 0 : 1 + rnd_below(3 * T);
        off[d + 1] = off[d] + len;
        pl[d] = rnd_below(len + 3);
        seg[d] = (uint16_t)rnd_below(3);
    }
    uint32_t *tok = NEW(uint32_t, off[D]);
    for (uint64_t i = 0; i < off[D]; i++) tok[i] = (uint32_t)rnd();
    uint64_t ramp_from[2] = {0, (uint64_t)(1 + rnd_below(20)) * T}, ramp_tok[2] = {(uint64_t)L * T, (uint64_t)B * T};

    or_corpus c;
    memset(&c, 0, sizeof c);
    c.tokens = tok; c.n_tokens = off[D]; c.offsets = off; c.n_docs = D; c.source = src; c.stratum = str;
    c.prompt_len = (seed & 1) ? pl : NULL;
    c.n_sources = S; c.n_strata = n_strata; c.weight = weight; c.bp = bp;
    c.T = T; c.B = B; c.seed = rnd(); c.pad_token = rnd_below(1000);
    c.wrap = (seed >> 1) & 1;
    c.heldout = (seed % 7) == 3;
    c.read_random = (seed >> 2) & 1;
    c.cumulative = (seed >> 3) & 1;
    if ((seed >> 4) & 1 && B > L) { c.n_ramp = 2; c.ramp_from = ramp_from; c.ramp_tokens = ramp_tok; }
    c.lanes = L;
    if ((seed >> 5) & 1) { c.segment = seg; c.n_segments = 3; }

    int err = 0, bad = 0;
    for (int pass = 0; pass < 2 && !bad; pass++) {  /* pass 1: a context resumed at pass 0's stream tokens */
        uint64_t *starts = NULL;
        or_plan *p = or_plan_build(&c, &err);
        if (!p) break;  /* configurations the oracle refuses are fine here */
        g_plans++;
        {   /* the exported arrays, at their exact sizes */
            const uint64_t V = (uint64_t)S * L;
            uint64_t nk, np, nw;
            (void)or_plan_sizes(p, &nk, &np, &nw);
            uint64_t *h = NEW(uint64_t, D), *sds = NEW(uint64_t, V + 1), *sps = NEW(uint64_t, V + 1);
            uint64_t *wf = NEW(uint64_t, nw + 1), *sws = NEW(uint64_t, V + 1), *wr = NEW(uint64_t, nw);
            uint64_t *wl = NEW(uint64_t, nw), *st = NEW(uint64_t, 4 * V), ck[2];
            uint8_t *kp = NEW(uint8_t, D);
            uint32_t *ord = NEW(uint32_t, nk), *pd = NEW(uint32_t, np), *po = NEW(uint32_t, np);
            uint32_t *pln = NEW(uint32_t, np), *pw = NEW(uint32_t, np), *nu = NEW(uint32_t, V);
            uint32_t *ss = NEW(uint32_t, B), *sk = NEW(uint32_t, B);
            or_plan_export(p, h, kp, ord, sds, pd, po, pln, pw, sps, wf, sws, wr, wl, nu, ss, sk, st, ck);
            free(h); free(sds); free(sps); free(wf); free(sws); free(wr); free(wl); free(st); free(kp);
            free(ord); free(pd); free(po); free(pln); free(pw); free(nu); free(ss); free(sk);
        }
        for (uint32_t cyc = c.first_cycle; cyc < c.first_cycle + 3; cyc++) {
            const uint32_t ucfg = rnd_below(4);
            const int rc = or_cycle(p, cyc, ucfg);
            if (rc == OR_E_EXHAUSTED) break;
            if (rc != OR_OK) { bad = 1; break; }
            g_cycles++;
            if (check_cycle(p, 1, L) || (B % 2 == 0 && check_cycle(p, 2, L))) { bad = 1; break; }
            if (pass == 0 && cyc == c.first_cycle) {
                starts = NEW(uint64_t, (uint64_t)S * L);
                if (or_cycle_stream_next(p, starts) != OR_OK) bad = 1;
            }
        }
        if (pass == 0 && starts && !bad) {  /* go on from cycle 0's stream tokens */
            c.start_tokens = starts;
            c.first_cycle = 1;
        } else {
            free(starts);
            starts = NULL;
        }
        or_plan_free(p);
        if (pass == 1) { free((void *)c.start_tokens); c.start_tokens = NULL; }
        if (!c.start_tokens) break;
    }
    free((void *)c.start_tokens);
    free(n_strata); free(weight); free(bp); free(off); free(src); free(str); free(seg); free(pl); free(tok);
    return bad;
}

/* chunked window digests of records of several chunks, the last one partial
 * or whole, over windows laid out back to back */
static int check_chunked_digests(void)
{
    static const uint32_t Ts[] = {315, 316, 1024, 1500, 5000};
    int bad = 0;
    for (uint32_t i = 0; i < sizeof Ts / sizeof Ts[0]; i++) {
        const uint32_t T = Ts[i], n = 3;
        uint32_t *tok = NEW(uint32_t, (uint64_t)n * T);
        int32_t *pos = NEW(int32_t, (uint64_t)n * T), *doc = NEW(int32_t, (uint64_t)n * T);
        uint8_t *mask = NEW(uint8_t, (uint64_t)n * T), *d = NEW(uint8_t, 32 * n);
        for (uint64_t j = 0; j < (uint64_t)n * T; j++) {
            tok[j] = (uint32_t)rnd();
            pos[j] = (int32_t)rnd_below(T);
            doc[j] = (int32_t)rnd_below(1000);
            mask[j] = (uint8_t)rnd_below(2);
        }
        if (or_window_digests_chunked(T, n, tok, pos, doc, mask, d) != OR_OK) bad = 1;
        free(tok); free(pos); free(doc); free(mask); free(d);
    }
    return bad;
}

int main(int argc, char **argv)
{
    const uint32_t cases = argc > 1 ? (uint32_t)strtoul(argv[1], NULL, 10) : 96;
    uint32_t failed = 0;
    g_rng = 0xC4u;
    if (check_chunked_digests()) {
        fprintf(stderr, "chunked window digests: an oracle call returned an unexpected error\n");
        failed++;
    }
    for (uint32_t s = 0; s < cases; s++)
        if (run_case(s)) {
            fprintf(stderr, "case %u: an oracle call returned an unexpected error\n", s);
            failed++;
        }
    printf("%u cases, %u with unexpected errors; %llu plans, %llu cycles, %llu batch calls\n", cases, failed,
           (unsigned long long)g_plans, (unsigned long long)g_cycles, (unsigned long long)g_batches);
    return failed ? 1 : 0;
}
