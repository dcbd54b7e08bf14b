/*
 * Memory and undefined-behaviour check of the CPU oracle (test infrastructure).
 *
 * tests/test_oracle_sanitize.py builds this file together with oracle/oracle.c under AddressSanitizer
 * and UndefinedBehaviorSanitizer (statically linked runtimes) and runs it. It drives every oracle entry
 * point over small seeded inputs at the edge shapes (one env, one step, ragged sizes, every env mode and
 * frame skip, shortened waypoint tables, full respawn rings, padded observation strides, action counts
 * 1 .. 64), with every buffer allocated at exactly the size the entry point is documented to touch, so
 * that a read or write past an array ends the run. A few values that the pages fix are checked on the
 * way (the GAE worked example with gamma = 0.5, lambda = 1; the entropy of uniform logits; the loss at
 * ratio 1). The pins of every result live in the Python tests, which also run against a sanitizer build.
 * Prints "sanitize ok" and returns 0 when every check passed.
 */
#include "../oracle/oracle.c"

#include <stdio.h>

static uint64_t rng_state = 0x243F6A8885A308D3ull;

static uint64_t next_u64(void)   /* xorshift64* (Vigna 2016) */
{
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return rng_state * 0x2545F4914F6CDD1Dull;
}

static int32_t rnd(int32_t lo, int32_t hi) { return lo + (int32_t)(next_u64() % (uint64_t)(hi - lo + 1)); }
static float rnf(void) { return (float)((double)(next_u64() >> 11) * 0x1p-53 * 2.0 - 1.0); }

static void *xalloc(size_t bytes)
{
    void *p = malloc(bytes ? bytes : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    memset(p, 0, bytes ? bytes : 1);
    return p;
}

static int failures = 0;
#define CHECK(cond, ...) do { if (!(cond)) { fprintf(stderr, __VA_ARGS__); fputc('\n', stderr); ++failures; } } while (0)

/* Maps of floor random walks with platforms and freeze tiles above, the spawn on the floor at column 1,
 * checkpoints every 16 columns on the row above the floor, and their standing spots. */
typedef struct {
    int32_t m, h, w, k;
    uint8_t *maps;
    int32_t *ckpts, *spawns, *spots;
} maps_t;

static maps_t make_maps(int32_t m, int32_t h, int32_t w)
{
    maps_t s = {m, h, w, (w - 1) / 16, NULL, NULL, NULL, NULL};
    if (s.k < 1) s.k = 1;
    s.maps = xalloc((size_t)m * h * w);
    s.ckpts = xalloc(sizeof(int32_t) * 2 * (size_t)m * s.k);
    s.spawns = xalloc(sizeof(int32_t) * 2 * (size_t)m);
    s.spots = xalloc(sizeof(int32_t) * 2 * (size_t)m * s.k);
    for (int32_t q = 0; q < m; ++q) {
        uint8_t *g = s.maps + (size_t)q * h * w;
        int32_t top = h - 4;
        int32_t *tops = xalloc(sizeof(int32_t) * (size_t)w);
        for (int32_t c = 0; c < w; ++c) {
            if (c >= 3) top += rnd(-1, 1);
            if (top < 3) top = 3;
            if (top > h - 2) top = h - 2;
            tops[c] = top;
            for (int32_t r = 0; r < h; ++r) {
                uint8_t t = r >= top ? SOLID : AIR;
                if (t == AIR && c >= 3 && r >= 1) {
                    int32_t u = rnd(0, 99);
                    t = u < 10 ? PLATFORM : (u < 12 ? FREEZE : AIR);
                }
                g[(size_t)r * w + c] = t;
            }
        }
        s.spawns[2 * q] = 256;
        s.spawns[2 * q + 1] = tops[1] * 256 - 192;
        for (int32_t r = 0; r < tops[1]; ++r) g[(size_t)r * w + 1] = AIR;   /* a clear column to spawn in */
        for (int32_t j = 0; j < s.k; ++j) {
            int32_t col = 16 * (j + 1) < w ? 16 * (j + 1) : w - 1;
            s.ckpts[(q * s.k + j) * 2] = col;
            s.ckpts[(q * s.k + j) * 2 + 1] = tops[col] - 1;
            s.spots[(q * s.k + j) * 2] = col * 256 + 32;
            s.spots[(q * s.k + j) * 2 + 1] = tops[col] * 256 - 192;
        }
        free(tops);
    }
    return s;
}

static void free_maps(maps_t *s)
{
    free(s->maps); free(s->ckpts); free(s->spawns); free(s->spots);
}

/* A run of one env configuration: resets, steps with observations, a masked reset, a shortened path. */
static void run_env(const maps_t *ms, int32_t n, int32_t offset, int32_t fs, int32_t reward_mode, int32_t respawn,
                    int32_t hook, int32_t steps, int32_t tl, int64_t stride)
{
    oracle_cfg c = {n, offset, ms->m, ms->h, ms->w, ms->k, fs, tl, reward_mode, 0, respawn, hook};
    int32_t *wp = NULL, *wlen = NULL;
    if (reward_mode == 1) {
        int32_t kw = ms->h * ms->w;
        c.max_waypoints = kw;
        wp = xalloc(sizeof(int32_t) * 2 * (size_t)ms->m * kw);
        wlen = xalloc(sizeof(int32_t) * (size_t)ms->m);
        int32_t *scratch = xalloc(sizeof(int32_t) * 2 * (size_t)ms->h * ms->w);
        for (int32_t q = 0; q < ms->m; ++q) {
            const uint8_t *g = ms->maps + (size_t)q * ms->h * ms->w;
            int32_t c0 = (ms->spawns[2 * q] + 96) >> 8, r0 = (ms->spawns[2 * q + 1] + 96) >> 8;
            int32_t c1 = ms->ckpts[(q * ms->k + ms->k - 1) * 2], r1 = ms->ckpts[(q * ms->k + ms->k - 1) * 2 + 1];
            int32_t len = 0;
            int rc = oracle_bfs_path(g, ms->h, ms->w, c0, r0, c1, r1, wp + (size_t)q * kw * 2, kw, &len, scratch);
            if (rc != 0) {   /* unreachable or blocked goal: a one-tile path at the spawn */
                wp[(size_t)q * kw * 2] = c0;
                wp[(size_t)q * kw * 2 + 1] = r0;
                len = 1;
            }
            wlen[q] = len;
        }
        free(scratch);
    }
    int32_t *state = xalloc(sizeof(int32_t) * NF * (size_t)n);
    float *stack = xalloc(sizeof(float) * STACK * FRAME_DIMS * (size_t)n);
    float *obs = xalloc(sizeof(float) * (size_t)stride * (n - 1) + sizeof(float) * OBS_TILES);
    uint8_t *pix = xalloc((size_t)n * STACK * PIX * PIX);
    uint8_t *sprites = xalloc(16 * 64);
    int32_t *actions = xalloc(sizeof(int32_t) * (size_t)n), *aim = xalloc(sizeof(int32_t) * (size_t)n);
    int32_t *ended = xalloc(sizeof(int32_t) * (size_t)n);
    float *rew = xalloc(sizeof(float) * (size_t)n), *done = xalloc(sizeof(float) * (size_t)n);
    uint8_t *mask = xalloc((size_t)n);
    int32_t *ring = xalloc(sizeof(int32_t) * RESPAWN_BUF * (size_t)ms->m);
    int32_t *fill = xalloc(sizeof(int32_t) * (size_t)ms->m), *head = xalloc(sizeof(int32_t) * (size_t)ms->m);
    int32_t *frontier = xalloc(sizeof(int32_t) * (size_t)ms->m);
    for (int i = 0; i < 16 * 64; ++i) sprites[i] = (uint8_t)rnd(0, 255);
    oracle_env_reset(&c, ms->spawns, NULL, state, stack);
    oracle_env_obs_tiles(&c, ms->maps, ms->ckpts, state, stack, obs, stride);
    for (int32_t t = 0; t < steps; ++t) {
        for (int32_t e = 0; e < n; ++e) {
            actions[e] = rnd(0, 9) < 8 ? rnd(0, 11) : rnd(-3, 20);     /* some out-of-range actions */
            aim[e] = (int32_t)(((uint32_t)(uint16_t)rnd(-4096, 4096)) | ((uint32_t)(uint16_t)rnd(-4096, 4096) << 16));
        }
        oracle_env_step(&c, ms->maps, ms->ckpts, ms->spawns, wp, wlen, respawn ? ms->spots : NULL, ring, fill, head,
                        frontier, 77, t, respawn ? ended : NULL, actions, hook ? aim : NULL, state, stack, rew, done);
        for (int32_t e = 0; e < n; ++e) CHECK(done[e] == 0.0f || done[e] == 1.0f, "done is not 0 or 1");
        if (t % 7 == 0) oracle_env_obs_tiles(&c, ms->maps, ms->ckpts, state, stack, obs, stride);
        if (t % 11 == 0) oracle_env_obs_pixels(&c, ms->maps, sprites, stack, pix);
        if (t == steps / 2) {
            for (int32_t e = 0; e < n; ++e) mask[e] = (uint8_t)(e % 3 == 0);
            oracle_env_reset(&c, ms->spawns, mask, state, stack);
            if (wlen)   /* a later, shorter table: the index reached may lie past its end */
                for (int32_t q = 0; q < ms->m; ++q) wlen[q] = wlen[q] > 2 ? 2 : wlen[q];
        }
    }
    free(state); free(stack); free(obs); free(pix); free(sprites); free(actions); free(aim); free(ended);
    free(rew); free(done); free(mask); free(ring); free(fill); free(head); free(frontier); free(wp); free(wlen);
}

static void run_scans(int32_t T, int32_t N)
{
    size_t sz = (size_t)T * N;
    float *r = xalloc(sizeof(float) * sz), *v = xalloc(sizeof(float) * sz), *d = xalloc(sizeof(float) * sz);
    float *lr = xalloc(sizeof(float) * sz), *vl = xalloc(sizeof(float) * (size_t)N);
    double *adv = xalloc(sizeof(double) * sz), *ret = xalloc(sizeof(double) * sz), *nrm = xalloc(sizeof(double) * sz);
    double *vs = xalloc(sizeof(double) * sz), *pg = xalloc(sizeof(double) * sz);
    for (size_t i = 0; i < sz; ++i) {
        r[i] = rnf();
        v[i] = rnf();
        d[i] = rnd(0, 9) == 0 ? 1.0f : 0.0f;
        lr[i] = 0.6f * rnf();
    }
    for (int32_t i = 0; i < N; ++i) vl[i] = rnf();
    oracle_gae(r, v, d, vl, T, N, 0.99, 0.95, adv, ret);
    double mean = 0, std = 0;
    oracle_normalize(adv, (int64_t)sz, 1e-8, nrm, &mean, &std);
    oracle_vtrace(r, v, d, vl, lr, T, N, 0.99, 1.0, 1.0, 1.0, 1.0, vs, pg);
    for (size_t i = 0; i < sz; ++i) CHECK(isfinite(adv[i]) && isfinite(vs[i]) && isfinite(pg[i]), "non-finite scan");
    free(r); free(v); free(d); free(lr); free(vl); free(adv); free(ret); free(nrm); free(vs); free(pg);
}

static void run_loss(int64_t B, int32_t A, int32_t mb, int use_perm)
{
    double *z = xalloc(sizeof(double) * (size_t)B * A), *olp = xalloc(sizeof(double) * (size_t)B);
    double *adv = xalloc(sizeof(double) * (size_t)B), *ret = xalloc(sizeof(double) * (size_t)B);
    double *nv = xalloc(sizeof(double) * (size_t)B);
    int32_t *act = xalloc(sizeof(int32_t) * (size_t)B), *perm = use_perm ? xalloc(sizeof(int32_t) * (size_t)B) : NULL;
    int64_t nmb = B / mb;
    double *out = xalloc(sizeof(double) * 4 * (size_t)nmb), *scale = xalloc(sizeof(double) * 4 * (size_t)nmb);
    double *dl = xalloc(sizeof(double) * (size_t)B * A), *dv = xalloc(sizeof(double) * (size_t)B);
    double *gs = xalloc(sizeof(double) * (size_t)B * A), *vsc = xalloc(sizeof(double) * (size_t)B);
    double *dpg = xalloc(sizeof(double) * (size_t)B * A), *ratio = xalloc(sizeof(double) * (size_t)B);
    for (int64_t i = 0; i < B; ++i) {
        for (int32_t j = 0; j < A; ++j) z[i * A + j] = 2.0 * rnf();
        act[i] = rnd(0, A - 1);
        olp[i] = -1.0 + 0.5 * rnf();
        adv[i] = rnf();
        ret[i] = rnf();
        nv[i] = rnf();
        if (perm) perm[i] = (int32_t)i;
    }
    if (perm)
        for (int64_t i = B - 1; i > 0; --i) {   /* Fisher-Yates */
            int64_t j = (int64_t)(next_u64() % (uint64_t)(i + 1));
            int32_t tmp = perm[i]; perm[i] = perm[j]; perm[j] = tmp;
        }
    oracle_ppo_loss(z, act, olp, adv, ret, nv, perm, B, A, mb, 0.2, 0.5, 0.01, out, scale);
    oracle_ppo_loss_grad(z, act, olp, adv, ret, nv, perm, B, A, mb, 0.2, 0.5, 0.01, dl, dv, gs, vsc, dpg, ratio);
    for (int64_t m = 0; m < 4 * nmb; ++m) CHECK(isfinite(out[m]), "non-finite loss");
    free(z); free(olp); free(adv); free(ret); free(nv); free(act); free(perm); free(out); free(scale);
    free(dl); free(dv); free(gs); free(vsc); free(dpg); free(ratio);
}

static void run_policy(int64_t n, int64_t stride, int64_t offset)
{
    float *obs = xalloc(sizeof(float) * (size_t)(stride * (n > 0 ? n - 1 : 0) + OBS_TILES));
    float *enc = xalloc(sizeof(float) * POLICY_HIDDEN * OBS_TILES), *dec = xalloc(sizeof(float) * POLICY_OUT * POLICY_HIDDEN);
    double *out = xalloc(sizeof(double) * POLICY_OUT * (size_t)(n ? n : 1)), *logp = xalloc(sizeof(double) * (size_t)(n ? n : 1));
    int32_t *act = xalloc(sizeof(int32_t) * (size_t)(n ? n : 1));
    for (int64_t i = 0; i < stride * (n > 0 ? n - 1 : 0) + OBS_TILES; ++i) obs[i] = 4.0f * rnf();
    for (int i = 0; i < POLICY_HIDDEN * OBS_TILES; ++i) enc[i] = 0.01f * rnf();
    for (int i = 0; i < POLICY_OUT * POLICY_HIDDEN; ++i) dec[i] = 0.1f * rnf();
    CHECK(oracle_policy_forward(obs, n, stride, enc, dec, 31, 5, offset, out, act, logp) == 0, "policy rejected");
    for (int64_t e = 0; e < n; ++e) CHECK(act[e] >= 0 && act[e] < POLICY_ACTIONS && logp[e] <= 0.0, "policy action");
    free(obs); free(enc); free(dec); free(out); free(logp); free(act);
}

static void run_bfs(void)
{
    uint8_t one = AIR;
    int32_t path[2 * 4], len = 0, scratch[2];
    CHECK(oracle_bfs_path(&one, 1, 1, 0, 0, 0, 0, path, 1, &len, scratch) == 0 && len == 1, "1x1 bfs");
    uint8_t row[7] = {0, 0, 1, 0, 0, 0, 0};
    int32_t scratch7[14], path7[14];
    CHECK(oracle_bfs_path(row, 1, 7, 0, 0, 6, 0, path7, 7, &len, scratch7) == -1, "blocked row reachable");
    row[2] = FREEZE;
    CHECK(oracle_bfs_path(row, 1, 7, 0, 0, 6, 0, path7, 7, &len, scratch7) == 0 && len == 7, "row path");
    CHECK(oracle_bfs_path(row, 1, 7, 0, 0, 6, 0, path7, 6, &len, scratch7) == -3, "short max_len accepted");
    CHECK(oracle_bfs_path(row, 1, 7, 0, 0, 7, 0, path7, 7, &len, scratch7) == -1, "goal outside accepted");
}

static void check_pinned_values(void)
{
    /* GAE worked example: gamma = 0.5, lambda = 1, r = [1, 0, 0, 1], V = 0, V_T = 0 -> R = [1.125, 0.25, 0.5, 1] */
    float r[4] = {1, 0, 0, 1}, z4[4] = {0, 0, 0, 0}, vl[1] = {0};
    double adv[4], ret[4];
    oracle_gae(r, z4, z4, vl, 4, 1, 0.5, 1.0, adv, ret);
    CHECK(ret[0] == 1.125 && ret[1] == 0.25 && ret[2] == 0.5 && ret[3] == 1.0, "GAE worked example");
    /* uniform logits: entropy ln 12; ratio 1 (old log-probability ln 1/12): pg = -mean(A) */
    double z[2 * 12] = {0}, olp[2] = {-log(12.0), -log(12.0)}, a[2] = {0.5, -1.5}, rt[2] = {0, 0}, nv[2] = {0, 0};
    int32_t act[2] = {3, 11};
    double out[4], scale[4];
    oracle_ppo_loss(z, act, olp, a, rt, nv, NULL, 2, 12, 2, 0.2, 0.5, 0.01, out, scale);
    CHECK(fabs(out[2] - log(12.0)) < 1e-15 && fabs(out[0] - 0.5) < 1e-15 && out[1] == 0.0, "uniform-logit loss");
}

int main(void)
{
    check_pinned_values();
    run_bfs();
    maps_t small = make_maps(2, 12, 40), one = make_maps(1, 8, 20);
    for (int32_t fs = 1; fs <= 5; ++fs)
        for (int32_t mode = 0; mode < 8; ++mode)
            run_env(&small, 37, mode * 5, fs, mode & 1, (mode >> 1) & 1, (mode >> 2) & 1, 60, 45, fs == 2 ? 1400 : OBS_TILES);
    run_env(&one, 1, 0, 3, 1, 1, 1, 200, 30, OBS_TILES);
    free_maps(&small);
    free_maps(&one);
    const int32_t shapes[][2] = {{1, 1}, {1, 9}, {5, 1}, {33, 7}, {128, 3}};
    for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i) run_scans(shapes[i][0], shapes[i][1]);
    const int32_t losses[][3] = {{1, 1, 0}, {8, 3, 1}, {96, 12, 1}, {64, 64, 0}, {30, 5, 1}};
    for (size_t i = 0; i < sizeof losses / sizeof losses[0]; ++i)
        run_loss(losses[i][0] * (int64_t)(i + 1), losses[i][1], losses[i][0], losses[i][2]);
    run_policy(0, OBS_TILES, 0);
    run_policy(1, OBS_TILES, 0);
    run_policy(5, 1408, 1000);
    for (int32_t i = 1; i <= 2; ++i) (void)oracle_respawn_draw(5, 123, 456, i);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("sanitize ok\n");
    return 0;
}
