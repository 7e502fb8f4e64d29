/*
 * abi_host_check.c — drives the C ABI's host-side checks (every error a call
 * returns before any device work) in a library built with host-only
 * AddressSanitizer and UndefinedBehaviorSanitizer; tests/test_sanitize.py
 * builds and runs it on a machine without a GPU.  Exit 0 = every call
 * returned the documented code with no sanitizer report.
 */
#include <stdio.h>
#include <string.h>

#include "dpack.h"

static int expect(int got, int want, const char *what)
{
    if (got != want) {
        fprintf(stderr, "%s: got %d, want %d (%s)\n", what, got, want, pack_last_error(NULL));
        return 1;
    }
    return 0;
}

int main(void)
{
    uint64_t w[2] = {1, 1}, zero_w[2] = {0, 0}, ramp_from[2] = {0, 1000}, ramp_tok[2] = {128 * 4, 128 * 8};
    uint32_t bp[2] = {0, 0}, bad_bp[2] = {0, 10001}, strata[2] = {1, 0};
    pack_config c;
    memset(&c, 0, sizeof c);
    c.abi_version = DPACK_ABI_VERSION;
    c.tokens = (const uint32_t *)16;  /* never dereferenced: every case fails on the host first */
    c.n_tokens = 100;
    c.doc_offsets = (const uint64_t *)16;
    c.n_docs = 3;
    c.doc_source = (const uint16_t *)16;
    c.n_sources = 2;
    c.share_weight = w;
    c.holdout_bp = bp;
    c.window_tokens = 128;
    c.global_batch = 8;
    c.world = 1;
    const pack_config base = c;
    pack_ctx *ctx = NULL;
    int bad = 0;

    c.abi_version = 1; bad |= expect(pack_init(&c, &ctx), PACK_E_ABI, "abi"); c = base;
    c.window_tokens = 0; bad |= expect(pack_init(&c, &ctx), PACK_E_INVAL, "T = 0"); c = base;
    c.window_tokens = (1u << 20) + 1; bad |= expect(pack_init(&c, &ctx), PACK_E_INVAL, "T above 2^20"); c = base;
    c.global_batch = 0; bad |= expect(pack_init(&c, &ctx), PACK_E_INVAL, "B = 0"); c = base;
    c.world = 3; bad |= expect(pack_init(&c, &ctx), PACK_E_INVAL, "world does not divide B"); c = base;
    c.rank = 1; bad |= expect(pack_init(&c, &ctx), PACK_E_INVAL, "rank >= world"); c = base;
    c.share_weight = zero_w; bad |= expect(pack_init(&c, &ctx), PACK_E_INVAL, "weights sum to 0"); c = base;
    c.holdout_bp = bad_bp; bad |= expect(pack_init(&c, &ctx), PACK_E_INVAL, "hold-out above 10000"); c = base;
    c.n_strata = strata; bad |= expect(pack_init(&c, &ctx), PACK_E_INVAL, "a source without strata"); c = base;
    c.n_sources = 5000; bad |= expect(pack_init(&c, &ctx), PACK_E_INVAL, "too many sources"); c = base;
    c.flags = 1u << 20; bad |= expect(pack_init(&c, &ctx), PACK_E_INVAL, "unknown flag"); c = base;
    c.n_ramp = 2; c.ramp_from = ramp_from; c.ramp_tokens = ramp_tok; c.global_batch = 4;
    bad |= expect(pack_init(&c, &ctx), PACK_E_INVAL, "B below the ramp's largest batch"); c = base;
    c.n_lanes = 3; bad |= expect(pack_init(&c, &ctx), PACK_E_INVAL, "lanes do not divide B"); c = base;
    bad |= expect(pack_init(NULL, &ctx), PACK_E_INVAL, "NULL config");
    bad |= expect(pack_init(&c, NULL), PACK_E_INVAL, "NULL out");
    c.n_docs = 1u << 22; c.n_tokens = 1ull << 32;
    bad |= expect(pack_init_noalloc(&c, &ctx), PACK_E_INVAL, "no-alloc workspace limit"); c = base;
    c.flags = PACK_FLAG_TIMING; bad |= expect(pack_init_noalloc(&c, &ctx), PACK_E_INVAL, "no-alloc timing"); c = base;
    c.flags = PACK_FLAG_TIMING_BATCH;
    bad |= expect(pack_init_noalloc(&c, &ctx), PACK_E_INVAL, "no-alloc batch timing"); c = base;
    bad |= ctx != NULL;
    for (int k = -9; k <= 0; ++k) bad |= pack_strerror(k) == NULL || pack_strerror(k)[0] == 0;
    bad |= pack_last_error(NULL) == NULL;
    bad |= expect(pack_cycle(NULL, 0, NULL), PACK_E_INVAL, "cycle NULL");
    bad |= expect(pack_batch(NULL, 0, 1, NULL), PACK_E_INVAL, "batch NULL");
    bad |= expect(pack_batch_packed(NULL, 0, 1, NULL), PACK_E_INVAL, "packed NULL");
    bad |= expect(pack_fingerprint(NULL, NULL, 1, NULL), PACK_E_INVAL, "fingerprint NULL");
    bad |= expect(pack_fingerprint_steps(NULL, 0, 1, NULL, NULL), PACK_E_INVAL, "fingerprint_steps NULL");
    bad |= expect(pack_inspect(NULL, PACK_INSPECT_HASH, NULL, 0, NULL), PACK_E_INVAL, "inspect NULL");
    bad |= expect(pack_get_timings(NULL, NULL, 0), PACK_E_INVAL, "timings NULL");
    bad |= expect(pack_status(NULL), PACK_E_INVAL, "status NULL");
    bad |= expect(pack_test_option(NULL, PACK_TEST_WAIT_GIVE_UP, 1), PACK_E_INVAL, "test option NULL");
    pack_destroy(NULL);
    printf("abi host checks: %s\n", bad ? "FAILED" : "ok");
    return bad;
}
