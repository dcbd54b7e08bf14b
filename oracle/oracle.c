/*
 * CPU oracle of the GPU-resident PPO rollout hot path.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the tests, the smoke check and the bench's CPU-baseline
 * leg may load this library. It shares no source with the HIP path: every constant, table and step
 * below is written out here on its own, from the pages that define the method.
 *
 * Plain, slow, single-threaded C. The environment is all integer arithmetic, so its outputs are exact;
 * GAE, advantage normalisation and the PPO loss are computed in float64 from float32 inputs.
 *
 * Sources (page, then section):
 *   [MARIO]    "Teaching Mario to speedrun" (bigmah.com): s.4 Reward (the return G_t), s.5 (the reverse
 *              return loop), s.6 PPO (GAE, the clipped loss, the collect/judge/learn loop), s.7
 *              PufferLib (the four shared arrays, the vecenv step, the platformer step function), s.8
 *              (PufferLib 5.0's default policy: the shape of the stand-in inference).
 *   [DDNET]    boesch.dev DDNet RL post: "How it works each tick" (frame-skip 3, rewards accumulate
 *              between decisions, contiguous [actions|observations|rewards|dones]), "What the agent
 *              sees and does" (43x31 tile grid, 15-dim player state stacked 4 frames, 4 checkpoint
 *              dims; direction/jump/hook), "Reward Engineering" Version 1 (+10 per checkpoint in
 *              order, high-water-mark progress, time penalty) and Version 2 (+100 finish).
 *   [PLAYTRAIN] "PlayTrain: An Efficient RL Framework for LLM-Generated Adaptable JavaScript Games":
 *              Table 4 (terminated / truncated at 2000), Table 8 (clip 0.2, value 0.5, entropy 0.01),
 *              App. B (frame stack, grayscale observation knobs), Figure 8C and Table 9 (double
 *              buffering: one env group steps while the other's inference runs).
 *
 * The pages never fix the environment's mechanics; every constant and step of the tick below is a
 * reading, stated where it is used.
 *
 * Parity pins: GAE, normalisation and the loss are pinned by closed forms and hand-worked cases. No page
 * gives the environment's outputs, so it is pinned to its stated reading: hand-worked episodes of every
 * rule and invariants over an exhaustive enumeration of decision sequences.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------------------------------------- */
/* Environment constants (readings; units: 1 tile = 256 sub-units, 1 pixel = 32 sub-units).         */
/* ---------------------------------------------------------------------------------------------- */
enum { AIR = 0, SOLID = 1, PLATFORM = 2, FREEZE = 3 };

#define TILE 256            /* sub-units per tile */
#define BOX 192             /* player box side, sub-units */
#define GRAVITY 12          /* sub/tick^2 */
#define MAX_FALL 160        /* sub/tick */
#define JUMP_V 120          /* sub/tick */
#define MAX_VX 48           /* sub/tick */
#define ACC_GROUND 8
#define ACC_AIR 4
#define FREEZE_TICKS 30
#define UNITS_CHECKPOINT 10240   /* +10 reward   (1 reward = 1024 units) */
#define UNITS_FINISH 102400      /* +100 reward */
/* Waypoint-path reward ([DDNET] "Reward Engineering", Version 2; readings): */
#define WP_AHEAD 8               /* the nearest waypoint is searched at the high-water index and 8 past it */
#define UNITS_WAYPOINT 256       /* progress: one tile of path = 256 units, V1's one unit per sub-unit */
#define WP_GRACE 1024            /* the 128-unit (about 4 tile) grace zone, in sub-units */
#define WP_PENALTY_SHIFT 4       /* beyond the grace zone: one unit per 16 sub-units of distance per tick */
/* Adaptive checkpoint respawn ([DDNET] "Checkpoint Respawning"; readings): */
#define RESPAWN_BUF 64           /* the rolling buffer of episode outcomes, per map */
#define RESPAWN_START_U32 858993459u  /* a draw below this (20% of 2^32) starts from the beginning */
/* Grapple hook with a continuous aim ([DDNET] "What the agent sees and does": a hook button and an aim
 * angle with a magnitude). The page gives no hook mechanics; the flight, attachment and pull below, and
 * these constants, are readings: */
#define HOOK_SPEED 256      /* tip speed along the aim, sub-units per tick (one tile, so no tile row or
                               column is stepped over) */
#define HOOK_FLIGHT 10      /* ticks of flight before the tip is lost: a reach of 10 tiles */
#define HOOK_ACCEL 24       /* pull of an attached hook toward its tip, sub/tick^2 (twice gravity) */
#define HOOK_MAX_V 160      /* bound on each velocity component while attached (the fall-speed limit) */
enum { HOOK_IDLE = 0, HOOK_FLYING = 1, HOOK_ATTACHED = 2 };
#define WIN_W 43            /* tile window: 43 columns ... */
#define WIN_H 31            /* ... by 31 rows */
#define WIN_CX 21           /* the player's tile sits at window column 21, row 15 */
#define WIN_CY 15
#define STACK 4
#define FRAME_DIMS 15
#define OBS_TILES (WIN_W * WIN_H + STACK * FRAME_DIMS + 4) /* 1397 */
#define PIX 84              /* pixel frame side */

/* Canonical state layout: int32[N][NF] in this field order. */
enum {
    F_X, F_Y, F_VX, F_VY, F_FACING, F_FREEZE, F_HOOK_TICKS, F_HOOK_HELD, F_JUMP_HELD, F_GROUNDED,
    F_WALL_L, F_WALL_R, F_TICK, F_NEXT, F_BEST_X, F_LAST_ACTION, F_PATH, F_FROM_START,
    F_HOOK_PHASE, F_HOOK_X, F_HOOK_Y, F_HOOK_VX, F_HOOK_VY, F_HOOK_FLIGHT, NF
};

typedef struct {
    int32_t num_envs;    /* envs in the arrays passed to this call */
    int32_t env_offset;  /* global index of the first of them (env n plays map n mod num_maps) */
    int32_t num_maps, map_h, map_w, num_ckpts;
    int32_t frame_skip, time_limit;
    int32_t reward_mode;    /* 0: checkpoint rewards (Version 1); 1: waypoint path (Version 2) */
    int32_t max_waypoints;  /* row length of the waypoint table (reward_mode 1) */
    int32_t respawn_mode;   /* 0: every episode starts at the spawn; 1: adaptive checkpoint respawn */
    int32_t hook_mode;      /* 0: the hook button is only state; 1: grapple hook aimed by the aim input */
} oracle_cfg;

typedef struct {
    int32_t x, y, vx, vy, facing, freeze, hook_ticks, hook_held, jump_held, grounded;
    int32_t wall_l, wall_r, tick, next, best_x, last_action, path, from_start;
    int32_t hook_phase, hook_x, hook_y, hook_vx, hook_vy, hook_flight;   /* hook mode: tip (absolute
                                           sub-units), its velocity while flying, ticks flown */
} env_t;

/* Adaptive respawn state of every map: the ring of the last RESPAWN_BUF episode outcomes (checkpoints
 * passed when the episode ended), how many are filled, the next write position, and the frontier (the
 * most checkpoints an episode that started at the spawn has passed). */
typedef struct {
    const int32_t *ckpt_spawns;   /* [M][K][2] (x, y) standing spot at each checkpoint */
    int32_t *ring;                /* [M][RESPAWN_BUF] */
    int32_t *fill, *head, *frontier;   /* [M] */
    uint64_t seed;
    int64_t counter;              /* the decision counter of this step */
} respawn_t;

/* The waypoint path of every map: waypoints[m][k] = (col, row) of the k-th tile of map m's path,
 * k < lens[m] <= max_waypoints. */
typedef struct {
    const int32_t *waypoints;
    const int32_t *lens;
} path_t;

static void load_env(const int32_t *s, env_t *e)
{
    e->x = s[F_X]; e->y = s[F_Y]; e->vx = s[F_VX]; e->vy = s[F_VY];
    e->facing = s[F_FACING]; e->freeze = s[F_FREEZE]; e->hook_ticks = s[F_HOOK_TICKS];
    e->hook_held = s[F_HOOK_HELD]; e->jump_held = s[F_JUMP_HELD]; e->grounded = s[F_GROUNDED];
    e->wall_l = s[F_WALL_L]; e->wall_r = s[F_WALL_R]; e->tick = s[F_TICK]; e->next = s[F_NEXT];
    e->best_x = s[F_BEST_X]; e->last_action = s[F_LAST_ACTION]; e->path = s[F_PATH];
    e->from_start = s[F_FROM_START];
    e->hook_phase = s[F_HOOK_PHASE]; e->hook_x = s[F_HOOK_X]; e->hook_y = s[F_HOOK_Y];
    e->hook_vx = s[F_HOOK_VX]; e->hook_vy = s[F_HOOK_VY]; e->hook_flight = s[F_HOOK_FLIGHT];
}

static void store_env(const env_t *e, int32_t *s)
{
    s[F_X] = e->x; s[F_Y] = e->y; s[F_VX] = e->vx; s[F_VY] = e->vy;
    s[F_FACING] = e->facing; s[F_FREEZE] = e->freeze; s[F_HOOK_TICKS] = e->hook_ticks;
    s[F_HOOK_HELD] = e->hook_held; s[F_JUMP_HELD] = e->jump_held; s[F_GROUNDED] = e->grounded;
    s[F_WALL_L] = e->wall_l; s[F_WALL_R] = e->wall_r; s[F_TICK] = e->tick; s[F_NEXT] = e->next;
    s[F_BEST_X] = e->best_x; s[F_LAST_ACTION] = e->last_action; s[F_PATH] = e->path;
    s[F_FROM_START] = e->from_start;
    s[F_HOOK_PHASE] = e->hook_phase; s[F_HOOK_X] = e->hook_x; s[F_HOOK_Y] = e->hook_y;
    s[F_HOOK_VX] = e->hook_vx; s[F_HOOK_VY] = e->hook_vy; s[F_HOOK_FLIGHT] = e->hook_flight;
}

/* Mathematical floor of a / b for b > 0 (C's '/' truncates toward zero). */
static int32_t floordiv(int32_t a, int32_t b)
{
    int32_t q = a / b;
    if ((a % b) != 0 && a < 0) q -= 1;
    return q;
}

/* Tile at (row, col) of map m; anything outside the map reads as SOLID (a reading). */
static int tile_at(const oracle_cfg *c, const uint8_t *maps, int m, int32_t row, int32_t col)
{
    if (row < 0 || row >= c->map_h || col < 0 || col >= c->map_w) return SOLID;
    return maps[((size_t)m * c->map_h + row) * c->map_w + col];
}

static int blocks(int t) { return t == SOLID || t == PLATFORM; }

/* Is any blocking tile in column `col` over rows r0..r1? */
static int solid_in_col(const oracle_cfg *c, const uint8_t *maps, int m, int32_t col, int32_t r0, int32_t r1)
{
    for (int32_t r = r0; r <= r1; ++r)
        if (blocks(tile_at(c, maps, m, r, col))) return 1;
    return 0;
}

/* Is any blocking tile in row `row` over columns c0..c1? */
static int solid_in_row(const oracle_cfg *c, const uint8_t *maps, int m, int32_t row, int32_t c0, int32_t c1)
{
    for (int32_t col = c0; col <= c1; ++col)
        if (blocks(tile_at(c, maps, m, row, col))) return 1;
    return 0;
}

static int map_of(const oracle_cfg *c, int n) { return (c->env_offset + n) % c->num_maps; }

/* Spawn state of an env on map m: standing at the map's spawn point, facing right, everything zero. */
static void spawn_env(const int32_t *spawns, int m, env_t *e)
{
    memset(e, 0, sizeof *e);
    e->x = spawns[2 * m + 0];
    e->y = spawns[2 * m + 1];
    e->facing = 1;
    e->grounded = 1;
    e->best_x = e->x;
    e->from_start = 1;
}

/* SplitMix64's output function (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", 2014). */
static uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
#define GOLDEN_GAMMA 0x9E3779B97F4A7C15ull

/* The i-th draw (i = 1, 2) of global env n at decision `counter`: the i-th SplitMix64 output from the
 * state seed + 2 * GOLDEN_GAMMA * (counter * 2^24 + n), i.e. mix64(state + i * GOLDEN_GAMMA). */
static uint64_t respawn_draw(uint64_t seed, int64_t counter, int32_t n, int i)
{
    uint64_t key = (uint64_t)counter * ((uint64_t)1 << 24) + (uint64_t)n;
    return mix64(seed + 2 * GOLDEN_GAMMA * key + (uint64_t)i * GOLDEN_GAMMA);
}

/* The draw above, for the tests. */
uint64_t oracle_respawn_draw(uint64_t seed, int64_t counter, int32_t n, int32_t i)
{
    return respawn_draw(seed, counter, n, i);
}

/* The checkpoint an ended episode of global env n on map m restarts at (0 = the spawn), drawn from the
 * map's outcome buffer as it stood at the start of the step ([DDNET] "Checkpoint Respawning"): 20% of
 * resets, and every reset while the buffer is empty, start at the spawn; otherwise one entry of the top
 * quarter of the buffer (the entries >= the highest outcome v that at least max(1, fill / 4) entries
 * reach) is taken uniformly, capped at the frontier and at the last checkpoint before the finish. */
static int32_t respawn_choice(const oracle_cfg *c, const respawn_t *rs, int m, int32_t n)
{
    int32_t fill = rs->fill[m];
    if (fill == 0) return 0;
    uint64_t u1 = respawn_draw(rs->seed, rs->counter, n, 1);
    if ((uint32_t)(u1 >> 32) < RESPAWN_START_U32) return 0;
    const int32_t *ring = rs->ring + (size_t)m * RESPAWN_BUF;
    int32_t q = fill / 4 > 0 ? fill / 4 : 1;
    int32_t cand = 0, thr = 0;
    for (int32_t v = c->num_ckpts; v >= 0; --v) {
        for (int32_t i = 0; i < fill; ++i) if (ring[i] == v) ++cand;
        if (cand >= q) { thr = v; break; }
    }
    uint64_t u2 = respawn_draw(rs->seed, rs->counter, n, 2);
    int32_t pick = (int32_t)((u2 >> 32) % (uint64_t)cand);
    int32_t chosen = thr;
    for (int32_t v = c->num_ckpts; v >= thr; --v) {
        int32_t cv = 0;
        for (int32_t i = 0; i < fill; ++i) if (ring[i] == v) ++cv;
        if (pick < cv) { chosen = v; break; }
        pick -= cv;
    }
    int32_t k = chosen < rs->frontier[m] ? chosen : rs->frontier[m];
    if (k > c->num_ckpts - 1) k = c->num_ckpts - 1;
    return k > 0 ? k : 0;
}

/* Start a new episode of map m at checkpoint k: the spawn for k = 0, else the standing spot of
 * checkpoint k - 1 with k checkpoints counted as passed. */
static void spawn_at(const oracle_cfg *c, const int32_t *spawns, const respawn_t *rs, int m, int32_t k,
                     env_t *e)
{
    spawn_env(spawns, m, e);
    if (k > 0) {
        const int32_t *p = rs->ckpt_spawns + ((size_t)m * c->num_ckpts + (k - 1)) * 2;
        e->x = p[0];
        e->y = p[1];
        e->best_x = e->x;
        e->next = k;
        e->from_start = 0;
    }
}

/* The 15-dim frame of a state ("What the agent sees and does": position, velocity, hook state,
 * freeze status). Sub-unit quantities are scaled by 2^-8 (tile units), the tick by 2^-11. In hook mode
 * dimension 9 is the hook's phase (idle 0, flying 1, attached 2) instead of the ticks it was held. */
static void make_frame(const oracle_cfg *c, const env_t *e, float *f)
{
    f[0] = (float)e->x * 0x1p-8f;
    f[1] = (float)e->y * 0x1p-8f;
    f[2] = (float)e->vx * 0x1p-8f;
    f[3] = (float)e->vy * 0x1p-8f;
    f[4] = (float)e->grounded;
    f[5] = (float)e->facing;
    f[6] = e->freeze > 0 ? 1.0f : 0.0f;
    f[7] = (float)e->freeze;
    f[8] = (float)e->hook_held;
    f[9] = c->hook_mode ? (float)e->hook_phase : (float)e->hook_ticks;
    f[10] = (float)e->jump_held;
    f[11] = (float)e->wall_l;
    f[12] = (float)e->wall_r;
    f[13] = (float)e->tick * 0x1p-11f;
    f[14] = (float)e->last_action;
}

/* floor(sqrt(v)) for v >= 0, by the digit-by-digit (binary) method. */
static int64_t isqrt64(int64_t v)
{
    uint64_t x = (uint64_t)v, r = 0, bit = (uint64_t)1 << 62;
    while (bit > x) bit >>= 2;
    while (bit != 0) {
        if (x >= r + bit) { x -= r + bit; r = (r >> 1) + bit; }
        else r >>= 1;
        bit >>= 2;
    }
    return (int64_t)r;
}

/* Version 2 progress and distance terms of one tick ([DDNET] "Reward Engineering", Version 2): the
 * waypoint nearest to the box centre among the high-water index and the WP_AHEAD after it (the lowest
 * index on a tie); moving the high-water mark forward pays UNITS_WAYPOINT per waypoint (no backtrack
 * penalty); a distance d beyond the grace zone costs (d - WP_GRACE) >> WP_PENALTY_SHIFT units. */
static int32_t waypoint_units(const oracle_cfg *c, const path_t *pt, int m, env_t *e)
{
    const int32_t *wp = pt->waypoints + (size_t)m * c->max_waypoints * 2;
    int32_t len = pt->lens[m];
    if (e->path > len - 1) e->path = len - 1;   /* a shorter table than the index reached */
    int64_t cx = (int64_t)e->x + BOX / 2, cy = (int64_t)e->y + BOX / 2;
    int32_t best = e->path;
    int64_t best_d2 = -1;
    for (int32_t k = e->path; k <= e->path + WP_AHEAD && k < len; ++k) {
        int64_t dx = cx - ((int64_t)wp[2 * k] * TILE + TILE / 2);
        int64_t dy = cy - ((int64_t)wp[2 * k + 1] * TILE + TILE / 2);
        int64_t d2 = dx * dx + dy * dy;
        if (best_d2 < 0 || d2 < best_d2) { best_d2 = d2; best = k; }
    }
    int32_t units = 0;
    if (best > e->path) { units += (best - e->path) * UNITS_WAYPOINT; e->path = best; }
    int64_t d = isqrt64(best_d2);
    if (d > WP_GRACE) units -= (int32_t)((d - WP_GRACE) >> WP_PENALTY_SHIFT);
    return units;
}

/* Move v toward target by at most acc. */
static int32_t approach(int32_t v, int32_t target, int32_t acc)
{
    if (v < target) return (v + acc > target) ? target : v + acc;
    if (v > target) return (v - acc < target) ? target : v - acc;
    return v;
}

/* One physics tick (all integer). Adds the tick's reward units to *units; returns 1 on the finish. */
static int physics_tick(const oracle_cfg *c, const uint8_t *maps, const int32_t *ckpts, const path_t *pt,
                        int m, env_t *e, int dir, int jump, int hook, int32_t aim_dx, int32_t aim_dy,
                        int32_t *units)
{
    /* 1. a frozen player's input is ignored */
    if (e->freeze > 0) { dir = 0; jump = 0; hook = 0; }

    /* 2. horizontal velocity toward dir * MAX_VX; facing follows the pushed direction */
    int32_t sign = dir == 1 ? -1 : (dir == 2 ? 1 : 0);
    e->vx = approach(e->vx, sign * MAX_VX, e->grounded ? ACC_GROUND : ACC_AIR);
    if (sign != 0) e->facing = sign;

    /* 3-4. jump from the ground, then gravity with a terminal fall speed */
    if (jump && e->grounded) e->vy = -JUMP_V;
    e->vy = e->vy + GRAVITY;
    if (e->vy > MAX_FALL) e->vy = MAX_FALL;

    /* 4h. the grapple hook (hook mode; readings). Letting go retracts it at once. Pressing it while it
     * is idle and was not held on the previous tick, with a non-zero aim (dx, dy), fires the tip from
     * the box centre with velocity HOOK_SPEED * (dx, dy) / floor(|(dx, dy)|), each component truncated
     * toward zero. A flying tip moves once a tick; it attaches where it lands if that tile blocks
     * movement (outside the map included), and is lost after HOOK_FLIGHT ticks in the air. An attached
     * hook adds HOOK_ACCEL * e / floor(|e|) (truncated toward zero) to the velocity, e the offset from
     * the box centre to the tip, and bounds each component by HOOK_MAX_V. */
    if (c->hook_mode) {
        if (!hook) {
            e->hook_phase = HOOK_IDLE;
        } else if (e->hook_phase == HOOK_IDLE && !e->hook_held && (aim_dx != 0 || aim_dy != 0)) {
            int64_t len = isqrt64((int64_t)aim_dx * aim_dx + (int64_t)aim_dy * aim_dy);
            e->hook_vx = (int32_t)((int64_t)aim_dx * HOOK_SPEED / len);
            e->hook_vy = (int32_t)((int64_t)aim_dy * HOOK_SPEED / len);
            e->hook_x = e->x + BOX / 2;
            e->hook_y = e->y + BOX / 2;
            e->hook_flight = 0;
            e->hook_phase = HOOK_FLYING;
        }
        if (e->hook_phase == HOOK_FLYING) {
            e->hook_x += e->hook_vx;
            e->hook_y += e->hook_vy;
            e->hook_flight += 1;
            if (blocks(tile_at(c, maps, m, floordiv(e->hook_y, TILE), floordiv(e->hook_x, TILE))))
                e->hook_phase = HOOK_ATTACHED;
            else if (e->hook_flight >= HOOK_FLIGHT)
                e->hook_phase = HOOK_IDLE;
        }
        if (e->hook_phase == HOOK_ATTACHED) {
            int64_t ex = (int64_t)e->hook_x - (e->x + BOX / 2), ey = (int64_t)e->hook_y - (e->y + BOX / 2);
            int64_t dist = isqrt64(ex * ex + ey * ey);
            if (dist > 0) {
                e->vx += (int32_t)(ex * HOOK_ACCEL / dist);
                e->vy += (int32_t)(ey * HOOK_ACCEL / dist);
            }
            if (e->vx > HOOK_MAX_V) e->vx = HOOK_MAX_V;
            if (e->vx < -HOOK_MAX_V) e->vx = -HOOK_MAX_V;
            if (e->vy > HOOK_MAX_V) e->vy = HOOK_MAX_V;
            if (e->vy < -HOOK_MAX_V) e->vy = -HOOK_MAX_V;
        }
    }

    /* 5. move along x against the rows the box covers before the y move */
    {
        int32_t nx = e->x + e->vx;
        int32_t r0 = floordiv(e->y, TILE), r1 = floordiv(e->y + BOX - 1, TILE);
        if (e->vx > 0) {
            int32_t col = floordiv(nx + BOX - 1, TILE);
            if (solid_in_col(c, maps, m, col, r0, r1)) { nx = col * TILE - BOX; e->vx = 0; }
        } else if (e->vx < 0) {
            int32_t col = floordiv(nx, TILE);
            if (solid_in_col(c, maps, m, col, r0, r1)) { nx = (col + 1) * TILE; e->vx = 0; }
        }
        e->x = nx;
    }

    /* 6. move along y against the columns the box covers after the x move */
    {
        int32_t ny = e->y + e->vy;
        int32_t c0 = floordiv(e->x, TILE), c1 = floordiv(e->x + BOX - 1, TILE);
        if (e->vy > 0) {
            int32_t row = floordiv(ny + BOX - 1, TILE);
            if (solid_in_row(c, maps, m, row, c0, c1)) { ny = row * TILE - BOX; e->vy = 0; }
        } else if (e->vy < 0) {
            int32_t row = floordiv(ny, TILE);
            if (solid_in_row(c, maps, m, row, c0, c1)) { ny = (row + 1) * TILE; e->vy = 0; }
        }
        e->y = ny;
    }

    /* 7. contacts of the final box */
    {
        int32_t c0 = floordiv(e->x, TILE), c1 = floordiv(e->x + BOX - 1, TILE);
        int32_t r0 = floordiv(e->y, TILE), r1 = floordiv(e->y + BOX - 1, TILE);
        e->grounded = solid_in_row(c, maps, m, floordiv(e->y + BOX, TILE), c0, c1);
        e->wall_l = solid_in_col(c, maps, m, floordiv(e->x - 1, TILE), r0, r1);
        e->wall_r = solid_in_col(c, maps, m, floordiv(e->x + BOX, TILE), r0, r1);

        /* 8. freeze: touching a freeze tile (re)arms the counter, otherwise it counts down */
        int touching = 0;
        for (int32_t r = r0; r <= r1; ++r)
            for (int32_t col = c0; col <= c1; ++col)
                if (tile_at(c, maps, m, r, col) == FREEZE) touching = 1;
        if (touching) e->freeze = FREEZE_TICKS;
        else if (e->freeze > 0) e->freeze -= 1;
    }

    /* 9. hook and jump state */
    e->hook_ticks = hook ? (e->hook_ticks + 1 > 255 ? 255 : e->hook_ticks + 1) : 0;
    e->hook_held = hook;
    e->jump_held = jump;

    /* 10. progress reward. Version 1: one unit per sub-unit past the high-water mark of x, no backtrack
     * penalty. Version 2: the waypoint path's progress and distance terms. best_x is kept in both (it is
     * an observation dim). */
    if (c->reward_mode == 1) *units += waypoint_units(c, pt, m, e);
    if (e->x > e->best_x) {
        if (c->reward_mode == 0) *units += e->x - e->best_x;
        e->best_x = e->x;
    }

    /* 11. checkpoints in order (+10 each in Version 1); passing the last one is the finish (+100) */
    int finished = 0;
    if (e->next < c->num_ckpts) {
        const int32_t *ck = ckpts + ((size_t)m * c->num_ckpts + e->next) * 2;
        if (floordiv(e->x + BOX / 2, TILE) >= ck[0]) {
            if (c->reward_mode == 0) *units += UNITS_CHECKPOINT;
            e->next += 1;
            if (e->next == c->num_ckpts) { *units += UNITS_FINISH; finished = 1; }
        }
    }

    /* 12. time: one unit per tick in Version 1 (Version 2 lists no time penalty) */
    e->tick += 1;
    if (c->reward_mode == 0) *units -= 1;
    return finished;
}

/* Reset the envs whose mask byte is non-zero (all when mask is NULL): spawn state, and all STACK
 * frames of the stack set to the spawn frame. */
int oracle_env_reset(const oracle_cfg *c, const int32_t *spawns, const uint8_t *mask,
                     int32_t *state, float *stack)
{
    for (int n = 0; n < c->num_envs; ++n) {
        if (mask && !mask[n]) continue;
        env_t e;
        spawn_env(spawns, map_of(c, n), &e);
        store_env(&e, state + (size_t)n * NF);
        float f[FRAME_DIMS];
        make_frame(c, &e, f);
        for (int k = 0; k < STACK; ++k)
            memcpy(stack + ((size_t)n * STACK + k) * FRAME_DIMS, f, sizeof f);
    }
    return 0;
}

/* One decision of every env ([MARIO] s.7 platformer step; [DDNET] frame-skip 3 with the rewards of
 * the skipped ticks summed): up to frame_skip ticks, stopping after a terminal tick. The reward is
 * the summed units times 2^-10; done = terminated or truncated. A done env is reset in place, so the
 * reward and done describe the episode that ended while the state and stack are the new episode's.
 * Otherwise the new frame is pushed onto the stack (newest first). */
int oracle_env_step(const oracle_cfg *c, const uint8_t *maps, const int32_t *ckpts,
                    const int32_t *spawns, const int32_t *waypoints, const int32_t *wp_lens,
                    const int32_t *ckpt_spawns, int32_t *ring, int32_t *fill, int32_t *head, int32_t *frontier,
                    uint64_t seed, int64_t counter, int32_t *ended,
                    const int32_t *actions, const int32_t *aim, int32_t *state, float *stack, float *rewards,
                    float *dones)
{
    const path_t pt = {waypoints, wp_lens};
    const respawn_t rs = {ckpt_spawns, ring, fill, head, frontier, seed, counter};
    for (int n = 0; n < c->num_envs; ++n) {
        int m = map_of(c, n);
        env_t e;
        load_env(state + (size_t)n * NF, &e);
        int32_t a = actions[n];
        if (a < 0 || a >= 12) a = 0;                   /* out-of-range actions act as no-op */
        int dir = a / 4, jump = (a >> 1) & 1, hook = a & 1;
        /* hook mode's aim: dx in the low 16 bits, dy in the high 16 bits, both signed (NULL: no aim) */
        int32_t aim_dx = aim ? (int16_t)(aim[n] & 0xffff) : 0;
        int32_t aim_dy = aim ? (int16_t)((uint32_t)aim[n] >> 16) : 0;

        int32_t units = 0;
        int terminated = 0, truncated = 0;
        for (int i = 0; i < c->frame_skip && !terminated && !truncated; ++i) {
            terminated = physics_tick(c, maps, ckpts, &pt, m, &e, dir, jump, hook, aim_dx, aim_dy, &units);
            if (e.tick >= c->time_limit) truncated = 1;
        }
        e.last_action = a;
        rewards[n] = (float)units * 0x1p-10f;
        dones[n] = (terminated || truncated) ? 1.0f : 0.0f;

        float *st = stack + (size_t)n * STACK * FRAME_DIMS;
        if (ended) ended[n] = -1;
        if (terminated || truncated) {
            /* the outcome for the respawn buffer: checkpoints passed, and whether the episode began at
             * the spawn; the next episode starts from the buffer as it stood at the start of the step */
            if (ended) ended[n] = e.next | (e.from_start ? (int32_t)1 << 30 : 0);
            int32_t k = c->respawn_mode == 1 ? respawn_choice(c, &rs, m, c->env_offset + n) : 0;
            spawn_at(c, spawns, &rs, m, k, &e);
            float f[FRAME_DIMS];
            make_frame(c, &e, f);
            for (int k = 0; k < STACK; ++k) memcpy(st + k * FRAME_DIMS, f, sizeof f);
        } else {
            memmove(st + FRAME_DIMS, st, (STACK - 1) * FRAME_DIMS * sizeof(float));
            make_frame(c, &e, st);
        }
        store_env(&e, state + (size_t)n * NF);
    }
    /* after every env has stepped: the ended episodes' outcomes enter their map's ring in env order,
     * and those that began at the spawn raise the frontier */
    if (c->respawn_mode == 1)
        for (int n = 0; n < c->num_envs; ++n) {
            if (ended[n] < 0) continue;
            int m = map_of(c, n);
            int32_t outcome = ended[n] & (((int32_t)1 << 30) - 1);
            ring[(size_t)m * RESPAWN_BUF + head[m]] = outcome;
            head[m] = (head[m] + 1) % RESPAWN_BUF;
            if (fill[m] < RESPAWN_BUF) fill[m] += 1;
            if ((ended[n] >> 30) & 1 && outcome > frontier[m]) frontier[m] = outcome;
        }
    return 0;
}

/* Tile path for the waypoint reward ([DDNET] "Reward Engineering", Version 2: a tile-level BFS
 * pathfinder over the map). Breadth-first search over the tiles a box can pass through (not SOLID or
 * PLATFORM, inside the map) with 4-neighbour moves tried in the order right, up, down, left; each tile
 * keeps the first tile that reached it, so the path is the one shortest path this order picks. Writes
 * (col, row) pairs from start to goal inclusive into path[max_len][2] and their count into *len.
 * Returns 0, -1 when start or goal is blocked or outside the map or the goal is unreachable, -3 when
 * the path needs more than max_len tiles. */
int oracle_bfs_path(const uint8_t *map, int32_t h, int32_t w, int32_t c0, int32_t r0, int32_t c1, int32_t r1,
                    int32_t *path, int32_t max_len, int32_t *len, int32_t *scratch)
{
    /* scratch: int32[2 * h * w] = queue, then the parent of every tile (-1 unvisited, -2 start) */
    int32_t *queue = scratch, *parent = scratch + (size_t)h * w;
#define PASSABLE(r, cc) ((r) >= 0 && (r) < h && (cc) >= 0 && (cc) < w && \
                         map[(size_t)(r) * w + (cc)] != SOLID && map[(size_t)(r) * w + (cc)] != PLATFORM)
    if (!PASSABLE(r0, c0) || !PASSABLE(r1, c1)) return -1;
    for (size_t i = 0; i < (size_t)h * w; ++i) parent[i] = -1;
    int32_t head = 0, tail = 0;
    parent[(size_t)r0 * w + c0] = -2;
    queue[tail++] = r0 * w + c0;
    static const int dc[4] = {1, 0, 0, -1}, dr[4] = {0, -1, 1, 0};
    while (head < tail) {
        int32_t cur = queue[head++];
        if (cur == r1 * w + c1) break;
        int32_t r = cur / w, cc = cur % w;
        for (int k = 0; k < 4; ++k) {
            int32_t nr = r + dr[k], nc = cc + dc[k];
            if (!PASSABLE(nr, nc) || parent[(size_t)nr * w + nc] != -1) continue;
            parent[(size_t)nr * w + nc] = cur;
            queue[tail++] = nr * w + nc;
        }
    }
#undef PASSABLE
    if (parent[(size_t)r1 * w + c1] == -1) return -1;
    int32_t n = 0;
    for (int32_t t = r1 * w + c1; t != -2; t = parent[t]) ++n;
    if (n > max_len) return -3;
    *len = n;
    int32_t k = n - 1;
    for (int32_t t = r1 * w + c1; t != -2; t = parent[t], --k) {
        path[2 * k] = t % w;
        path[2 * k + 1] = t / w;
    }
    return 0;
}

/* Tile-mode observation of every env, f32[N][obs_stride] (first 1397 elements written):
 *   [0, 1333)     the 31-row x 43-column tile window around the player's tile, row-major, value =
 *                 tile code, outside the map = SOLID;
 *   [1333, 1393)  the 4 most recent frames of 15 dims, newest first;
 *   [1393, 1397)  next checkpoint dx, dy (tile units, from the box centre to the checkpoint tile's
 *                 centre), checkpoints passed, best x (tile units). */
int oracle_env_obs_tiles(const oracle_cfg *c, const uint8_t *maps, const int32_t *ckpts,
                         const int32_t *state, const float *stack, float *obs, int64_t obs_stride)
{
    for (int n = 0; n < c->num_envs; ++n) {
        int m = map_of(c, n);
        env_t e;
        load_env(state + (size_t)n * NF, &e);
        float *o = obs + (size_t)n * obs_stride;
        int32_t pcol = floordiv(e.x + BOX / 2, TILE), prow = floordiv(e.y + BOX / 2, TILE);
        for (int r = 0; r < WIN_H; ++r)
            for (int col = 0; col < WIN_W; ++col)
                o[r * WIN_W + col] = (float)tile_at(c, maps, m, prow - WIN_CY + r, pcol - WIN_CX + col);
        memcpy(o + WIN_W * WIN_H, stack + (size_t)n * STACK * FRAME_DIMS,
               STACK * FRAME_DIMS * sizeof(float));
        float *ck = o + WIN_W * WIN_H + STACK * FRAME_DIMS;
        if (e.next < c->num_ckpts) {
            const int32_t *p = ckpts + ((size_t)m * c->num_ckpts + e.next) * 2;
            ck[0] = (float)(p[0] * TILE + TILE / 2 - (e.x + BOX / 2)) * 0x1p-8f;
            ck[1] = (float)(p[1] * TILE + TILE / 2 - (e.y + BOX / 2)) * 0x1p-8f;
        } else {
            ck[0] = 0.0f;
            ck[1] = 0.0f;
        }
        ck[2] = (float)e.next;
        ck[3] = (float)e.best_x * 0x1p-8f;
    }
    return 0;
}

/* Pixel-mode observation of every env, u8[N][4][84][84], newest frame first. Each frame is the 84x84
 * grayscale camera view centred on the player's box at that frame's position, drawn from 8x8 sprites
 * (pattern = tile code & 15, outside the map = SOLID), with the player's box drawn as 255. The
 * positions of the older frames are the ones kept in the frame stack. */
int oracle_env_obs_pixels(const oracle_cfg *c, const uint8_t *maps, const uint8_t *sprites,
                          const float *stack, uint8_t *obs)
{
    for (int n = 0; n < c->num_envs; ++n) {
        int m = map_of(c, n);
        for (int k = 0; k < STACK; ++k) {
            const float *f = stack + ((size_t)n * STACK + k) * FRAME_DIMS;
            int32_t x = (int32_t)(f[0] * 256.0f), y = (int32_t)(f[1] * 256.0f);  /* exact */
            int32_t cam_x = floordiv(x + BOX / 2, 32) - PIX / 2;
            int32_t cam_y = floordiv(y + BOX / 2, 32) - PIX / 2;
            int32_t bx0 = floordiv(x, 32), bx1 = floordiv(x + BOX - 1, 32);
            int32_t by0 = floordiv(y, 32), by1 = floordiv(y + BOX - 1, 32);
            uint8_t *o = obs + ((size_t)n * STACK + k) * PIX * PIX;
            for (int py = 0; py < PIX; ++py) {
                for (int px = 0; px < PIX; ++px) {
                    int32_t wx = cam_x + px, wy = cam_y + py;
                    uint8_t v;
                    if (wx >= bx0 && wx <= bx1 && wy >= by0 && wy <= by1) {
                        v = 255;
                    } else {
                        int t = tile_at(c, maps, m, floordiv(wy, 8), floordiv(wx, 8));
                        int sy = wy - 8 * floordiv(wy, 8), sx = wx - 8 * floordiv(wx, 8);
                        v = sprites[((t & 15) * 8 + sy) * 8 + sx];
                    }
                    o[py * PIX + px] = v;
                }
            }
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------------------------- */
/* GAE ([MARIO] s.6 "Better advantages"), written as its definition:                               */
/*   delta_t = r_t + gamma * V_{t+1} * (1 - d_t) - V_t,  V_T = last_values                          */
/*   A_t     = sum_{k>=0} (gamma*lambda)^k * prod_{j<k} (1 - d_{t+j}) * delta_{t+k}                 */
/*   R_t     = A_t + V_t                                                                            */
/* d_t = 1 means the episode ended during step t (dones[t] is what step(actions[t]) returned), so it  */
/* cuts both the bootstrap of delta_t and every later term. O(T^2) per env, float64.                */
/* ---------------------------------------------------------------------------------------------- */
int oracle_gae(const float *rewards, const float *values, const float *dones, const float *last_values,
               int32_t T, int32_t N, double gamma, double lambda, double *adv, double *ret)
{
    for (int32_t n = 0; n < N; ++n) {
        for (int32_t t = 0; t < T; ++t) {
            double a = 0.0, w = 1.0;
            for (int32_t k = t; k < T; ++k) {
                double v_next = (k + 1 < T) ? (double)values[(size_t)(k + 1) * N + n] : (double)last_values[n];
                double d = (double)dones[(size_t)k * N + n];
                double delta = (double)rewards[(size_t)k * N + n] + gamma * v_next * (1.0 - d)
                             - (double)values[(size_t)k * N + n];
                a += w * delta;
                w *= gamma * lambda * (1.0 - d);
            }
            adv[(size_t)t * N + n] = a;
            ret[(size_t)t * N + n] = a + (double)values[(size_t)t * N + n];
        }
    }
    return 0;
}

/* Advantage normalisation over the whole batch: mean and population standard deviation, then
 * (A - mean) / (std + eps). Two passes, float64. */
int oracle_normalize(const double *adv, int64_t n, double eps, double *out, double *mean_out, double *std_out)
{
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) s += adv[i];
    double mean = s / (double)n;
    double q = 0.0;
    for (int64_t i = 0; i < n; ++i) q += (adv[i] - mean) * (adv[i] - mean);
    double std = sqrt(q / (double)n);
    if (out)
        for (int64_t i = 0; i < n; ++i) out[i] = (adv[i] - mean) / (std + eps);
    if (mean_out) *mean_out = mean;
    if (std_out) *std_out = std;
    return 0;
}

/* ---------------------------------------------------------------------------------------------- */
/* PPO loss forward ([MARIO] s.6 "Don't move too far at once"), per minibatch m over the samples      */
/* i = perm[m*mb + k] (k < mb; i = m*mb + k when perm is NULL):                                     */
/*   logp_i  = z_{i,a_i} - logsumexp(z_i)                                                           */
/*   ratio_i = exp(logp_i - old_logp_i)          (new probability over old probability)             */
/*   pg_i    = -min(ratio_i * A_i, clip(ratio_i, 1 - eps, 1 + eps) * A_i)                           */
/*   v_i     = (V_i - R_i)^2                                                                         */
/*   H_i     = entropy of softmax(z_i)                                                               */
/* out[m] = {mean pg, mean v, mean H, mean pg + vf_coef * mean v - ent_coef * mean H}; scale[m] holds */
/* the mean absolute summand of each (the tolerance floor). Inputs are float64 so that the loss can  */
/* also be evaluated at perturbed points (finite differences); float32 data converts exactly.        */
/* ---------------------------------------------------------------------------------------------- */
int oracle_ppo_loss(const double *logits, const int32_t *actions, const double *old_logp, const double *adv,
                    const double *ret, const double *new_values, const int32_t *perm, int64_t B, int32_t A,
                    int32_t mb, double clip_eps, double vf_coef, double ent_coef, double *out, double *scale)
{
    int64_t num_mb = B / mb;
    for (int64_t m = 0; m < num_mb; ++m) {
        double s_pg = 0, s_v = 0, s_h = 0, a_pg = 0, a_h = 0;
        for (int64_t k = 0; k < mb; ++k) {
            int64_t i = perm ? (int64_t)perm[m * mb + k] : m * mb + k;
            const double *z = logits + (size_t)i * A;
            double zmax = z[0];
            for (int j = 1; j < A; ++j) if (z[j] > zmax) zmax = z[j];
            double sum = 0.0;
            for (int j = 0; j < A; ++j) sum += exp(z[j] - zmax);
            double lse = zmax + log(sum);
            double ent = 0.0;  /* -sum p_j log p_j */
            for (int j = 0; j < A; ++j) {
                double lp = z[j] - lse;
                ent -= exp(lp) * lp;
            }
            double logp = z[actions[i]] - lse;
            double ratio = exp(logp - old_logp[i]);
            double clipped = ratio < 1.0 - clip_eps ? 1.0 - clip_eps : (ratio > 1.0 + clip_eps ? 1.0 + clip_eps : ratio);
            double s1 = ratio * adv[i], s2 = clipped * adv[i];
            double pg = -(s1 < s2 ? s1 : s2);
            double dv = new_values[i] - ret[i];
            double v = dv * dv;
            s_pg += pg; s_v += v; s_h += ent;
            a_pg += fabs(pg); a_h += fabs(ent);
        }
        double pg = s_pg / mb, v = s_v / mb, h = s_h / mb;
        out[m * 4 + 0] = pg;
        out[m * 4 + 1] = v;
        out[m * 4 + 2] = h;
        out[m * 4 + 3] = pg + vf_coef * v - ent_coef * h;
        if (scale) {
            scale[m * 4 + 0] = a_pg / mb;
            scale[m * 4 + 1] = v;
            scale[m * 4 + 2] = a_h / mb;
            scale[m * 4 + 3] = a_pg / mb + vf_coef * v + ent_coef * a_h / mb;
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------------------------- */
/* Gradient of each minibatch's total loss L_m = mean pg + vf_coef mean v - ent_coef mean H with     */
/* respect to the logits and the value of every sample i of minibatch m (the step after the loss     */
/* forward in the collect / judge / learn loop of [MARIO] s.6; computing it in the same pass as the  */
/* loss follows the fused loss-and-gradient kernel described in [MARIO] s.8). With p = softmax(z_i),  */
/* a = a_i, r = ratio_i, c = clip(r, 1 - eps, 1 + eps), M = mb:                                       */
/*   d logp / d z_j = [j == a] - p_j,   d r / d z_j = r ([j == a] - p_j)                              */
/*   -min(r A, c A) takes the unclipped term when r A <= c A (inside the band both terms are r A);    */
/*   there its derivative in r is -A, otherwise 0 (c is constant outside the band)                    */
/*   d H / d z_j = -p_j (log p_j + H)                                                                 */
/*   dL_m / d z_j = (1/M) (-[r A <= c A] A r ([j == a] - p_j) + ent_coef p_j (log p_j + H))           */
/*   dL_m / d V_i = (1/M) vf_coef 2 (V_i - R_i)                                                       */
/* Advantages are constants (normalisation statistics included). Extra outputs for the tests:         */
/*   gscale[i][j] = (1/M) (|A| r |[j == a] - p_j| + ent_coef p_j (|log p_j| + H)), vscale[i] =         */
/*   (1/M) vf_coef 2 (|V_i| + |R_i|): the magnitudes of the summands (the tolerance floor);           */
/*   dpg[i][j] = (1/M) (-A r ([j == a] - p_j)): the surrogate's part when the unclipped term is taken;  */
/*   ratio[i] = r. A ratio within rounding of a band edge decides the surrogate's part either way.    */
/* perm must be a permutation of [0, B) (each sample in one minibatch); NULL = contiguous minibatches. */
/* ---------------------------------------------------------------------------------------------- */
int oracle_ppo_loss_grad(const double *logits, const int32_t *actions, const double *old_logp,
                         const double *adv, const double *ret, const double *new_values, const int32_t *perm,
                         int64_t B, int32_t A, int32_t mb, double clip_eps, double vf_coef, double ent_coef,
                         double *dlogits, double *dvalues, double *gscale, double *vscale, double *dpg,
                         double *ratio_out)
{
    const double inv = 1.0 / (double)mb;
    for (int64_t k = 0; k < B; ++k) {
        int64_t i = perm ? (int64_t)perm[k] : k;
        const double *z = logits + (size_t)i * A;
        double zmax = z[0];
        for (int j = 1; j < A; ++j) if (z[j] > zmax) zmax = z[j];
        double sum = 0.0;
        for (int j = 0; j < A; ++j) sum += exp(z[j] - zmax);
        double lse = zmax + log(sum);
        double ent = 0.0;
        for (int j = 0; j < A; ++j) {
            double lp = z[j] - lse;
            ent -= exp(lp) * lp;
        }
        int a = actions[i];
        double logp = z[a] - lse;
        double ratio = exp(logp - old_logp[i]);
        double clipped = ratio < 1.0 - clip_eps ? 1.0 - clip_eps : (ratio > 1.0 + clip_eps ? 1.0 + clip_eps : ratio);
        int unclipped = ratio * adv[i] <= clipped * adv[i];
        for (int j = 0; j < A; ++j) {
            double lp = z[j] - lse;
            double pj = exp(lp);
            double onehot = j == a ? 1.0 : 0.0;
            double g_pg = -adv[i] * ratio * (onehot - pj);
            double g_h = ent_coef * pj * (lp + ent);
            dlogits[(size_t)i * A + j] = inv * ((unclipped ? g_pg : 0.0) + g_h);
            if (gscale) gscale[(size_t)i * A + j] = inv * (fabs(adv[i]) * ratio * fabs(onehot - pj) +
                                                          ent_coef * pj * (fabs(lp) + ent));
            if (dpg) dpg[(size_t)i * A + j] = inv * g_pg;
        }
        dvalues[i] = inv * vf_coef * 2.0 * (new_values[i] - ret[i]);
        if (vscale) vscale[i] = inv * vf_coef * 2.0 * (fabs(new_values[i]) + fabs(ret[i]));
        if (ratio_out) ratio_out[i] = ratio;
    }
    return 0;
}

/* ---------------------------------------------------------------------------------------------- */
/* V-trace targets (the off-policy correction that PlayTrain's IMPALA trainer, App. C.3, takes from   */
/* torchbeast; "Teaching Mario to speedrun" s.8 names it as the alternative to GAE for per-minibatch   */
/* advantages). Restated from its published definition (Espeholt et al., 2018, IMPALA, eq. 1) with    */
/* the done mask read as for GAE: the discount of step t is g_t = gamma (1 - d_t). With V_T = the      */
/* bootstrap values and lr = log(pi / mu) of the taken action:                                         */
/*   rho_t = min(rho_bar, exp(lr_t)),  c_t = lambda min(c_bar, exp(lr_t))                              */
/*   delta_t = rho_t (r_t + g_t V_{t+1} - V_t)                                                         */
/*   vs_s = V_s + sum_{t >= s} (prod_{i = s}^{t-1} g_i c_i) delta_t          (vs_T = V_T)              */
/*   pg_s = min(pg_rho_bar, exp(lr_s)) (r_s + g_s vs_{s+1} - V_s)                                      */
/* The sum is taken as written (O(T^2) per env), in float64.                                           */
/* ---------------------------------------------------------------------------------------------- */
int oracle_vtrace(const float *rewards, const float *values, const float *dones, const float *last_values,
                  const float *log_rhos, int32_t T, int32_t N, double gamma, double lambda, double rho_bar,
                  double c_bar, double pg_rho_bar, double *vs, double *pg_adv)
{
    for (int32_t n = 0; n < N; ++n) {
        for (int32_t s = 0; s < T; ++s) {
            double acc = 0.0, w = 1.0;
            for (int32_t t = s; t < T; ++t) {
                size_t k = (size_t)t * N + n;
                double g = gamma * (1.0 - (double)dones[k]);
                double vnext = t + 1 < T ? (double)values[k + N] : (double)last_values[n];
                double ratio = exp((double)log_rhos[k]);
                double rho = ratio < rho_bar ? ratio : rho_bar;
                double delta = rho * ((double)rewards[k] + g * vnext - (double)values[k]);
                acc += w * delta;
                double c = lambda * (ratio < c_bar ? ratio : c_bar);
                w *= g * c;
                if (w == 0.0) break;
            }
            vs[(size_t)s * N + n] = (double)values[(size_t)s * N + n] + acc;
        }
        for (int32_t s = 0; s < T; ++s) {
            size_t k = (size_t)s * N + n;
            double g = gamma * (1.0 - (double)dones[k]);
            double vs_next = s + 1 < T ? vs[k + N] : (double)last_values[n];
            double ratio = exp((double)log_rhos[k]);
            double rho_pg = ratio < pg_rho_bar ? ratio : pg_rho_bar;
            pg_adv[k] = rho_pg * ((double)rewards[k] + g * vs_next - (double)values[k]);
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------------------------- */
/* Stand-in policy inference, the work one env group's decision needs while the other group steps  */
/* ([PLAYTRAIN] Figure 8C and Table 9: double buffering; App. C.3).                                 */
/* The network's shape follows [MARIO] s.8 (PufferLib 5.0's default policy): a bias-free linear      */
/* encoder from the observation to 128 numbers, and one decoder matrix from those to the logits plus */
/* the value. Its recurrent layers between the two are left out of the stand-in. [MARIO] s.6 gives  */
/* the heads: logits, one per action, sampled through a softmax, and the value.                     */
/* Readings: the encoder reads the observation and its weights rounded to bfloat16 (round to nearest */
/* even), the products summed exactly (float64 here); the decoder is float32 weights on the encoder's */
/* output (float64 here); the sample is the Gumbel-max form of softmax sampling (Gumbel 1954; the    */
/* "Gumbel-max trick"): a = argmax_j (logit_j + g_j), g_j = -ln(-ln u_j), lowest j on a tie, with    */
/* u_j = (2 (x_j >> 41) + 1) / 2^24 and x_j = mix64(seed + GOLDEN_GAMMA (16 (t 2^24 + n) + j + 1)),   */
/* the SplitMix64 output for global env n, decision t, logit j.                                      */
/* ---------------------------------------------------------------------------------------------- */
#define POLICY_HIDDEN 128
#define POLICY_ACTIONS 12
#define POLICY_OUT (POLICY_ACTIONS + 1)

/* Round a float32 to the nearest bfloat16 (ties to even), returned as a float32 (finite inputs). */
static float to_bf16(float x)
{
    uint32_t b;
    memcpy(&b, &x, 4);
    uint32_t lsb = (b >> 16) & 1u;
    b = (b + 0x7FFFu + lsb) & 0xFFFF0000u;
    float r;
    memcpy(&r, &b, 4);
    return r;
}

/* The uniform draw u_j in (0, 1) and its Gumbel variate, for the tests. */
double oracle_policy_gumbel(uint64_t seed, int64_t t, int64_t n, int32_t j, double *u_out)
{
    uint64_t key = (uint64_t)t * ((uint64_t)1 << 24) + (uint64_t)n;
    uint64_t x = mix64(seed + GOLDEN_GAMMA * (16 * key + (uint64_t)j + 1));
    double u = (double)(2 * (x >> 41) + 1) / 16777216.0;
    if (u_out) *u_out = u;
    return -log(-log(u));
}

/* obs float32 [n][stride] (the first OBS_TILES of each row); enc_w float32 [128][OBS_TILES];
 * dec_w float32 [13][128] (rows 0..11 the logits, row 12 the value). Writes out float64 [n][13]
 * (logits then value), the sampled actions and log pi(a) = logit_a - logsumexp(logits). */
int oracle_policy_forward(const float *obs, int64_t n, int64_t stride, const float *enc_w, const float *dec_w,
                          uint64_t seed, int64_t t, int64_t env_offset, double *out, int32_t *actions,
                          double *logp)
{
    if (n < 0 || stride < OBS_TILES || t < 0 || env_offset < 0) return -1;
    double hidden[POLICY_HIDDEN], xq[OBS_TILES];
    double *wq = malloc(sizeof(double) * POLICY_HIDDEN * OBS_TILES);   /* the rounded encoder weights */
    if (!wq) return -1;
    for (size_t i = 0; i < (size_t)POLICY_HIDDEN * OBS_TILES; ++i) wq[i] = (double)to_bf16(enc_w[i]);
    for (int64_t e = 0; e < n; ++e) {
        const float *x = obs + (size_t)e * stride;
        for (int k = 0; k < OBS_TILES; ++k) xq[k] = (double)to_bf16(x[k]);
        for (int h = 0; h < POLICY_HIDDEN; ++h) {
            double s = 0.0;
            for (int k = 0; k < OBS_TILES; ++k) s += xq[k] * wq[(size_t)h * OBS_TILES + k];
            hidden[h] = s;
        }
        double *o = out + (size_t)e * POLICY_OUT;
        for (int j = 0; j < POLICY_OUT; ++j) {
            double s = 0.0;
            for (int h = 0; h < POLICY_HIDDEN; ++h) s += hidden[h] * (double)dec_w[j * POLICY_HIDDEN + h];
            o[j] = s;
        }
        int best = 0;
        double best_score = 0.0, mx = o[0];
        for (int j = 0; j < POLICY_ACTIONS; ++j) {
            double score = o[j] + oracle_policy_gumbel(seed, t, env_offset + e, j, NULL);
            if (j == 0 || score > best_score) { best = j; best_score = score; }
            if (o[j] > mx) mx = o[j];
        }
        double z = 0.0;
        for (int j = 0; j < POLICY_ACTIONS; ++j) z += exp(o[j] - mx);
        actions[e] = best;
        logp[e] = o[best] - (mx + log(z));
    }
    free(wq);
    return 0;
}
