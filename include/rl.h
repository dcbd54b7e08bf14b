/*
 * rl.h -- C ABI of the GPU-resident PPO rollout hot path on AMD Instinct MI355X (gfx950).
 *
 * Three stages, all on one GPU, all data resident in HBM:
 *   1. batched platformer stepping with frame-skip and auto-reset, writing observations, rewards and
 *      dones into caller-owned device buffers (rl_env_*);
 *   2. the GAE reverse scan over a [T][N] rollout with optional whole-batch advantage normalisation
 *      (rl_gae), and the V-trace scan for off-policy targets (rl_vtrace);
 *   3. the PPO clipped-surrogate, value and entropy loss reductions per minibatch (rl_ppo_loss), and
 *      the same reductions with each sample's loss gradient written in the same pass (rl_ppo_loss_grad).
 *
 * Sources (page, then section):
 *   "Teaching Mario to speedrun" (bigmah.com): s.4 the return; s.6 GAE, the clipped loss and the
 *     collect / judge / learn loop; s.7 the four flat arrays shared by trainer and envs (observations
 *     [num_agents][obs_size], actions, rewards, terminals) and the env functions init / reset / step /
 *     close, with a platformer step that runs `frameskip` physics ticks and stops on a terminal tick.
 *   boesch.dev DDNet RL post: "How it works each tick" (frame-skip 3, rewards summed between decisions,
 *     one contiguous [actions | observations | rewards | dones] region), "What the agent sees and does"
 *     (43x31 tile grid, 15-dim player state stacked over 4 frames, 4 checkpoint dims; direction x jump x
 *     hook actions), "Reward Engineering" (+10 per checkpoint in order, high-water-mark progress, time
 *     penalty; +100 finish).
 *   NeSLE article on kongchang.com ("observations never leave VRAM"): observations written by the
 *     kernels into preallocated device buffers that the trainer uses in place, buffers reused across
 *     iterations.
 *   PlayTrain (arXiv 2609.09059): Table 4 (terminated / truncated at a 2000-step limit), Table 8 (clip
 *     0.2, value coefficient 0.5, entropy coefficient 0.01, GAE lambda 0.95), App. B (frame stack,
 *     grayscale observation).
 *
 * Conventions for every function:
 *   - Returns RL_OK (0) or a negative RL_E* code; rl_last_error() then holds a message (thread-local).
 *   - Arguments are validated before any HIP call; a rejected call enqueues nothing.
 *   - Pointers named as device pointers must be device memory the caller owns (for instance torch
 *     tensors); the library never allocates, frees or synchronises device memory, and never copies
 *     between host and device except where stated.
 *   - `stream` is a hipStream_t (NULL = the default stream); all work is enqueued on it in order.
 *     Kernel faults surface at the caller's next synchronisation.
 *   - An env handle may be used from one stream at a time. No C++ exception crosses this ABI.
 */
#ifndef RL_H
#define RL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    RL_OK = 0,
    RL_EINVAL = -1,     /* null pointer, size or enum out of range */
    RL_EALIGN = -2,     /* a pointer or stride breaks the stated alignment */
    RL_ESIZE = -3,      /* a caller buffer (state, workspace) is smaller than required */
    RL_EHIP = -4        /* a HIP launch or API call failed; the HIP message is in rl_last_error() */
};

enum { RL_OBS_TILES = 0, RL_OBS_PIXELS = 1 };
enum { RL_REWARD_CHECKPOINTS = 0, RL_REWARD_WAYPOINTS = 1 };
enum { RL_RESPAWN_OFF = 0, RL_RESPAWN_ADAPTIVE = 1 };
enum { RL_HOOK_OFF = 0, RL_HOOK_GRAPPLE = 1 };

#define RL_STATE_FIELDS 24      /* canonical state fields per env, see rl_env_read_state */
#define RL_RESPAWN_BUF 64       /* episode outcomes kept per map for the adaptive respawn */
#define RL_OBS_TILES_SIZE 1397  /* f32 elements: 31*43 window + 4*15 frames + 4 checkpoint dims */
#define RL_OBS_PIXELS_SIZE 28224 /* u8 elements: 4 frames of 84*84 */
#define RL_MAX_FRAME_SKIP 5

/* Environment configuration. Positions are in sub-units: one tile = 256, the player box is 192 wide
 * and tall. Tile codes: 0 air, 1 solid, 2 platform (solid), 3 freeze (passable; touching it ignores the
 * player's input for 30 ticks). */
typedef struct rl_env_config {
    int32_t num_envs;    /* N >= 1; env n plays map n mod num_maps for its whole life */
    int32_t num_maps;    /* M >= 1 */
    int32_t map_h;       /* rows per map, 1 .. 4096 */
    int32_t map_w;       /* columns per map, 1 .. 65536 */
    int32_t num_ckpts;   /* K >= 0 checkpoints per map; passing the K-th is the finish */
    int32_t frame_skip;  /* physics ticks per decision, 1 .. RL_MAX_FRAME_SKIP (3 on the pages) */
    int32_t time_limit;  /* ticks per episode before truncation, >= 1 (2000) */
    int32_t obs_mode;    /* RL_OBS_TILES (f32 observations) or RL_OBS_PIXELS (u8 observations) */
    int64_t obs_stride;  /* elements from one env's observation to the next, >= the observation size;
                            tiles: a multiple of 1 f32, pixels: a multiple of 4 u8 */
    int32_t reward_mode; /* RL_REWARD_CHECKPOINTS or RL_REWARD_WAYPOINTS (see rl_env_step) */
    int32_t max_waypoints; /* waypoints per map path, 1 .. 2^20, with RL_REWARD_WAYPOINTS (else ignored) */
    int32_t respawn_mode;  /* RL_RESPAWN_OFF or RL_RESPAWN_ADAPTIVE (1 .. 1024 checkpoints; see rl_env_step) */
    uint64_t respawn_seed; /* seed of the adaptive respawn's draws */
    int32_t hook_mode;     /* RL_HOOK_OFF (the hook button is state only) or RL_HOOK_GRAPPLE (a grapple hook
                              aimed by rl_env_step_aim's aims; see there) */
} rl_env_config;

typedef struct rl_env rl_env;   /* opaque host handle */

/* Bytes of device memory the caller must provide as the env state buffer (256-byte aligned). It holds
 * the per-env state in structure-of-arrays form, a ring of the last 4 frames, a padded copy of the maps
 * and the checkpoint, spawn and sprite tables. */
int rl_env_state_bytes(const rl_env_config* cfg, size_t* bytes);

/* Elements in one env's observation (1397 for tiles, 28224 for pixels) and the element size in bytes
 * (4 for f32 tiles, 1 for u8 pixels). */
int rl_env_obs_size(const rl_env_config* cfg, size_t* elems, size_t* elem_bytes);

/* Layout of one contiguous step block [actions int32[N] | observations [N][obs_stride] | rewards f32[N]
 * | dones f32[N]] (the four flat arrays of the pages, each sub-array 256-byte aligned): writes the four
 * byte offsets and the block size. */
int rl_step_layout(const rl_env_config* cfg, size_t offsets[4], size_t* block_bytes);

/* Create an env batch over the caller's state buffer. Copies maps, checkpoints, spawns and sprites into
 * the state buffer with kernels on `stream` (the inputs may be freed once the stream has passed this
 * call) and resets every env.
 *   maps     device u8[M][H][W], row 0 at the top; cells outside the map read as solid.
 *   ckpts    device int32[M][K][2] (column, row) of each map's checkpoints, in the order they must be
 *            passed; may be NULL when K = 0.
 *   spawns   device int32[M][2] (x, y) spawn position of each map in sub-units. The box placed there
 *            must lie inside the map: a step's collision tests read the tiles around the box's starting
 *            tile, which covers every move from a box inside the map; from a box outside it the
 *            physics is unspecified (memory accesses stay inside the state buffer).
 *   sprites  device u8[16][8][8] grayscale patterns (pattern = tile code & 15); required for pixel mode,
 *            ignored (may be NULL) for tiles.
 *   state    device buffer of rl_env_state_bytes() bytes, 256-byte aligned, owned by the caller for the
 *            handle's lifetime; its contents are the whole env state (copying it snapshots the envs).
 * On success *out receives a handle to free with rl_env_destroy. */
int rl_env_create(const rl_env_config* cfg, const uint8_t* maps, const int32_t* ckpts,
                  const int32_t* spawns, const uint8_t* sprites, void* state, size_t state_bytes,
                  void* stream, rl_env** out);

/* Reset the envs whose mask byte is non-zero (mask = device u8[N], or NULL for all) to their spawn
 * state with all 4 stacked frames equal to the spawn frame, then, when obs is not NULL, write every
 * env's observation to obs (device, [N][obs_stride] of the mode's element type). */
int rl_env_reset(rl_env* env, const uint8_t* mask, void* obs, void* stream);

/* The waypoint path of every map, for RL_REWARD_WAYPOINTS ("boesch.dev DDNet RL post", Reward Engineering,
 * Version 2: progress along a path traced through the map, e.g. by rl_waypoint_path). Copies
 *   waypoints  device int32[M][max_waypoints][2] (column, row) of the path's tiles, in order (tiles of
 *              the map: 0 <= column < map_w, 0 <= row < map_h, where the distances are exact), and
 *   lens       device int32[M] path length of each map (values outside 1 .. max_waypoints are clamped)
 * into the state buffer on `stream`; the inputs may be freed once the stream has passed this call. Must
 * be called before the first rl_env_step of a waypoint-reward env (the step fails otherwise); RL_EINVAL
 * for a checkpoint-reward env. */
int rl_env_set_waypoints(rl_env* env, const int32_t* waypoints, const int32_t* lens, void* stream);

/* Standing spots for the adaptive respawn (RL_RESPAWN_ADAPTIVE): copies ckpt_spawns, device
 * int32[M][K][2] = (x, y) in sub-units where an episode restarted at checkpoint k + 1 begins (inside the
 * map, as for rl_env_create's spawns), into the state buffer on `stream` (the input may be freed once the stream has passed this call). Must be called
 * before the first rl_env_step of such an env (the step fails otherwise); RL_EINVAL otherwise. */
int rl_env_set_respawn_spots(rl_env* env, const int32_t* ckpt_spawns, void* stream);

/* The adaptive respawn's per-map state into device outputs: ring int32[M][RL_RESPAWN_BUF] (the buffered
 * outcomes), and int32[M] fill, head (next write position) and frontier. RL_EINVAL without respawn. */
int rl_env_read_respawn(const rl_env* env, int32_t* ring, int32_t* fill, int32_t* head, int32_t* frontier,
                        void* stream);

/* Host helper for the waypoint path: the tile-level BFS pathfinder of the same post. Breadth-first
 * search over the tiles of one map (host u8[h][w]) that a box can pass (not solid or platform) with
 * 4-neighbour moves tried in the order right, up, down, left, each tile keeping the first tile that
 * reached it: the one shortest path from (c0, r0) to (c1, r1) that this order selects. Writes (column,
 * row) pairs from start to goal inclusive to path (host int32[max_len][2]) and the count to *len.
 * RL_EINVAL if an end is blocked or outside the map or the goal is unreachable; RL_ESIZE if the path
 * needs more than max_len tiles. Uses about 8 h w bytes of host memory. */
int rl_waypoint_path(const uint8_t* map, int32_t h, int32_t w, int32_t c0, int32_t r0, int32_t c1, int32_t r1,
                     int32_t* path, int32_t max_len, int32_t* len);

/* One decision of every env (the pages' step: read actions, advance, write observations / rewards /
 * terminals). For env n: decode actions[n] in [0, 12) as direction = a / 4 (none, left, right),
 * jump = bit 1, hook = bit 0 (other values act as 0); run up to frame_skip ticks, stopping after a
 * terminal tick; rewards[n] = the summed reward units times 2^-10. RL_REWARD_CHECKPOINTS (Version 1 of
 * the post's reward): progress past the best x (one unit per sub-unit), +10 per checkpoint in order, +100
 * at the finish, -1 unit per tick. RL_REWARD_WAYPOINTS (Version 2): each tick the waypoint nearest to the
 * box centre among the path's high-water index and the 8 after it (lowest index on a tie); moving the
 * high-water index forward pays 256 units per waypoint, a distance d = floor(sqrt(squared distance in
 * sub-units)) beyond 1024 (the 128-unit grace zone) costs (d - 1024) >> 4 units, +100 at the finish, no
 * checkpoint bonus and no time penalty. dones[n] = 1 if the episode finished (passed its last checkpoint)
 * or hit the time limit, else 0.
 * RL_RESPAWN_ADAPTIVE ("boesch.dev DDNet RL post", Checkpoint Respawning): each map keeps its last
 * RL_RESPAWN_BUF episode outcomes (checkpoints passed when the episode ended) and a frontier (the most
 * checkpoints passed by an episode that began at the spawn). An ended episode of global env n at decision
 * counter c restarts from the buffer as it stood at the start of the step: with the draws
 * u_i = SplitMix64's i-th output from the state seed + 2 * 0x9E3779B97F4A7C15 * (c * 2^24 + n), an empty
 * buffer or (u_1 >> 32) < 858993459 (20%) restarts at the spawn; otherwise the ((u_2 >> 32) mod cand)-th
 * entry, counting from the largest, of the cand entries >= the buffer's max(1, fill / 4)-th largest is
 * taken, capped at the frontier and at K - 1; k > 0 restarts at checkpoint k - 1's standing spot with k
 * checkpoints passed. After the step the ended episodes' outcomes enter their map's buffer in env order,
 * and those that began at the spawn raise its frontier. A done env is reset in place: its reward and done describe the episode that
 * ended, its observation is the new episode's first. Observations (tiles: the 31x43 window around the
 * player's tile, the last 4 frames newest first, next checkpoint dx / dy, checkpoints passed, best x;
 * pixels: 4 frames of 84x84, newest first) go to obs.
 *   actions  device int32[N]; obs device [N][obs_stride]; rewards, dones device f32[N]. */
int rl_env_step(rl_env* env, const int32_t* actions, void* obs, float* rewards, float* dones,
                void* stream);

/* rl_env_step with a continuous aim per env, for RL_HOOK_GRAPPLE ("boesch.dev DDNet RL post", What the
 * agent sees and does: a hook button and an aim given as an angle and a magnitude). aim is device
 * int32[N], (dx & 0xffff) | (dy << 16) with dx, dy int16: the aim as a vector in sub-units (its polar form
 * is the angle and the magnitude); NULL means no aim (the hook never fires); non-NULL with RL_HOOK_OFF is
 * RL_EINVAL. The post gives no hook mechanics; this library's reading, a step of every tick after gravity:
 * releasing the hook retracts it; pressing it while it is idle and was not held on the previous tick,
 * with a non-zero aim, fires the tip from the box centre with velocity 256 (dx, dy) / floor(|(dx, dy)|)
 * per tick (each component truncated toward zero); a flying tip moves once a tick and attaches where it
 * lands if that tile is solid, a platform or outside the map, and is lost after 10 ticks of flight; an
 * attached hook adds 24 e / floor(|e|) (truncated) to the velocity, e the offset from the box centre to
 * the tip, then bounds each velocity component to [-160, 160]. A frozen player's hook input is 0. In hook
 * mode frame dimension 9 of the observation is the hook's phase (0 idle, 1 flying, 2 attached) instead
 * of the ticks the button has been held. */
int rl_env_step_aim(rl_env* env, const int32_t* actions, const int32_t* aim, void* obs, float* rewards,
                    float* dones, void* stream);

/* Decode the state of every env into device int32[N][RL_STATE_FIELDS] with fields in the order
 * x, y, vx, vy, facing (+1/-1), freeze_ticks, hook_ticks, hook_held, jump_held, grounded, wall_left,
 * wall_right, tick, next_ckpt, best_x, last_action, path (the waypoint high-water index; 0 with
 * checkpoint rewards), from_start (1 if the episode began at the spawn), then the grapple hook's phase
 * (0 idle, 1 flying, 2 attached), tip x, tip y, flight velocity x, y and ticks flown (all 0 without
 * RL_HOOK_GRAPPLE). */
int rl_env_read_state(const rl_env* env, int32_t* out, void* stream);

/* The decision counter, whose value mod 4 selects the frame ring's newest slot and which keys the adaptive
 * respawn's draws. Its device copy lives in the state buffer and every step advances it there, so a stream
 * capture of steps (a HIP graph) advances it on every replay. A step launched outside a capture, while the
 * host's count is known to equal the device's (from creation, and from the first step after
 * rl_env_set_step_counter, until a step is recorded into a graph), takes the host's count as an argument
 * and needs no read of the device copy; a step recorded into a graph, and every step after one until the
 * counter is set again, reads the device copy.
 *   rl_env_get_step_counter: the decisions enqueued through rl_env_step / rl_env_step_aim on the host (not
 *     advanced by graph replays; after replays, read the device value or set it).
 *   rl_env_set_step_counter: sets the counter (host and device); the value is applied by the next step,
 *     which must not be inside a stream capture (it returns RL_EINVAL there): set the counter, run one step
 *     outside the capture, then capture. After copying a saved state buffer back in, set the counter to the
 *     saved value (the device value read from the saved buffer), or the host's count goes on.
 *   rl_env_read_step_counter: the device value into out (device int64, 8-byte aligned), on `stream`. */
int rl_env_get_step_counter(const rl_env* env, int64_t* counter);
int rl_env_set_step_counter(rl_env* env, int64_t counter);
int rl_env_read_step_counter(const rl_env* env, int64_t* out, void* stream);

/* Copy of the configuration the env batch was created with. */
int rl_env_get_config(const rl_env* env, rl_env_config* out);

/* Free the host handle (the state buffer stays the caller's). NULL is ignored. */
void rl_env_destroy(rl_env* env);

/* Workspace bytes rl_gae needs for T x N. */
int rl_gae_workspace_bytes(int32_t T, int32_t N, size_t* bytes);

/* GAE over a [T][N] rollout ("Teaching Mario to speedrun", s.6 Better advantages), float32:
 *   delta_t = r_t + gamma * V_{t+1} * (1 - d_t) - V_t  (V_T = last_values)
 *   A_t = delta_t + gamma * lambda * (1 - d_t) * A_{t+1},  A_T = 0;   ret_t = A_t + V_t
 * where dones[t][n] = 1 means env n's episode ended during step t.
 *   rewards, values, dones  device f32[T][N];  last_values device f32[N]
 *   adv, ret                device f32[T][N] outputs (may not alias the inputs)
 *   normalize  0: no statistics; 1: compute the whole-batch mean and population std of A and overwrite
 *              adv with (A - mean) / (std + 1e-8); 2: compute the statistics only (adv stays raw) so that
 *              rl_ppo_loss can normalise on the fly; 3: deferred statistics: as 2, but adv_stats receives
 *              the scan blocks' partial sums (and a header) instead of the finished values, and the
 *              reduction that turns them into the mean and std is left to the consumer (rl_ppo_loss,
 *              rl_ppo_loss_grad, rl_adv_stats_finish), which saves a kernel launch on the rollout path.
 *              ret always uses the raw A.
 *   adv_stats  device f64[3] = {count, mean, std} for normalize 1 and 2; for 3 a device buffer of
 *              rl_gae_stats_bytes(T, N) bytes in the deferred form (first double negative); may be NULL
 *              for 0. 8-byte aligned.
 *   ws         device workspace of rl_gae_workspace_bytes(T, N) bytes, 8-byte aligned (any contents; used
 *              when normalize is 1 or 2, may be NULL otherwise). Calls sharing a workspace must not overlap.
 * Statistics are reduced in a fixed order, so results are identical from run to run, and the mean and std
 * a consumer computes from the deferred form have the same bits as normalize = 2's. */
int rl_gae(const float* rewards, const float* values, const float* dones, const float* last_values,
           int32_t T, int32_t N, float gamma, float lambda, float* adv, float* ret, int32_t normalize,
           double* adv_stats, void* ws, size_t ws_bytes, void* stream);

/* Bytes of adv_stats for rl_gae's deferred statistics (normalize = 3) over T x N. */
int rl_gae_stats_bytes(int32_t T, int32_t N, size_t* bytes);

/* The finished statistics {count, mean, population std} (device f64[3] out) of an adv_stats buffer that
 * rl_gae wrote, in either form: copied when finished, reduced from the partial sums when deferred (the same
 * bits as normalize = 2 gives). One small kernel on `stream`. */
int rl_adv_stats_finish(const double* adv_stats, double* out, void* stream);

/* rl_gae over N columns of wider [T][ld] arrays (ld >= N elements between rows; last_values stays f32[N]
 * contiguous): rewards, values, dones, adv and ret address element [t][n] at t * ld + n, and elements
 * outside the N columns are neither read nor written. This is the per-minibatch form ("Teaching Mario
 * to speedrun", s.8: PufferLib 5.0 computes advantages per minibatch from fresh values): a minibatch of
 * envs n0 .. n0 + N - 1 of a [T][ld] rollout passes its column pointers (base + n0) and its fresh values
 * in the same layout, and normalize = 1 / 2 use that minibatch's own statistics. rl_gae is this call with
 * ld = N; the same kernel runs for the same T and N, so the results are the same bits. */
int rl_gae_strided(const float* rewards, const float* values, const float* dones, const float* last_values,
                   int32_t T, int32_t N, int64_t ld, float gamma, float lambda, float* adv, float* ret,
                   int32_t normalize, double* adv_stats, void* ws, size_t ws_bytes, void* stream);

/* V-trace over a [T][N] rollout: the IMPALA off-policy targets and policy-gradient advantages (PlayTrain
 * App. C.3 takes V-trace from torchbeast for its IMPALA trainer; "Teaching Mario to speedrun" s.8 names it
 * beside GAE for per-minibatch advantages). Restated from the published definition (Espeholt et al. 2018,
 * eq. 1) with the done mask as in rl_gae, g_t = gamma (1 - dones[t]):
 *   ratio_t = exp(log_rhos[t]),  rho_t = min(rho_bar, ratio_t),  c_t = lambda min(c_bar, ratio_t),
 *   vs[t] = V_t + sum_{u >= t} (prod_{i = t}^{u-1} g_i c_i) rho_u (r_u + g_u V_{u+1} - V_u),  V_T = last_values,
 *   pg_adv[t] = min(pg_rho_bar, ratio_t) (r_t + g_t vs[t+1] - V_t),  vs[T] = last_values.
 *   rewards, values, dones, log_rhos   device f32[T][N] (log_rhos = log pi(a_t) - log mu(a_t) of the taken
 *                                      actions); last_values device f32[N];
 *   vs, pg_adv                         device f32[T][N] outputs (may not alias the inputs);
 *   rho_bar, c_bar, pg_rho_bar >= 0 (torchbeast uses 1, 1, 1 and lambda = 1).
 * The scan runs in float32 (the same chunked affine-map scan as rl_gae); no workspace. */
int rl_vtrace(const float* rewards, const float* values, const float* dones, const float* last_values,
              const float* log_rhos, int32_t T, int32_t N, float gamma, float lambda, float rho_bar, float c_bar,
              float pg_rho_bar, float* vs, float* pg_adv, void* stream);

/* rl_vtrace over N columns of [T][ld] arrays (rewards, values, dones, log_rhos, vs, pg_adv), as for
 * rl_gae_strided; rl_vtrace is this call with ld = N. */
int rl_vtrace_strided(const float* rewards, const float* values, const float* dones, const float* last_values,
                      const float* log_rhos, int32_t T, int32_t N, int64_t ld, float gamma, float lambda,
                      float rho_bar, float c_bar, float pg_rho_bar, float* vs, float* pg_adv, void* stream);

/* Workspace bytes rl_ppo_loss needs for B samples in minibatches of mb. */
int rl_ppo_loss_workspace_bytes(int64_t B, int32_t mb, size_t* bytes);

/* PPO loss forward per minibatch ("Teaching Mario to speedrun", s.6 Don't move too far at once; the
 * coefficients of PlayTrain Table 8 are the usual arguments). Minibatch m is a set of mb samples given by
 * one of:
 *   perm      device int32[B], a permutation of 0..B-1: minibatch m = {perm[m*mb + k], k < mb};
 *   mb_index  device u16[B]: sample i belongs to minibatch mb_index[i] (each of 0 .. B/mb - 1 taken
 *             exactly mb times; at most 64 minibatches; values past the last minibatch count as the last);
 *   neither   minibatch m = samples m*mb .. m*mb + mb - 1.
 * (perm and mb_index describe the same split when mb_index[perm[p]] = p / mb.) For each sample i:
 *   logp = logits[i][actions[i]] - logsumexp(logits[i]),  ratio = exp(logp - old_logp[i])
 *   pg = -min(ratio * A, clip(ratio, 1 - clip_eps, 1 + clip_eps) * A),  v = (new_values[i] - ret[i])^2,
 *   H = entropy of softmax(logits[i]),  with A = adv[i], or (adv[i] - mean) / (std + 1e-8) from
 *   adv_stats when adv_stats is not NULL (as rl_gae wrote it with normalize 2, or 3: the deferred partial
 *   sums are then reduced inside the loss, to the same mean and std bits).
 *   out  device f32[B/mb][4] = {mean pg, mean v, mean H, mean pg + vf_coef * mean v - ent_coef * mean H}.
 *   logits device f32[B][A], A in 1..64 (16-byte aligned when A % 4 == 0); actions device int32[B] in
 *   [0, A) (other values act as action 0); old_logp, adv, ret, new_values device f32[B].
 *   B % mb must be 0. ws: device workspace of rl_ppo_loss_workspace_bytes(B, mb) bytes, 8-byte aligned (any
 *   contents); calls sharing it must not overlap. The per-sample terms are float32 (exponentials and
 *   logarithms from the hardware's base-2 instructions, about 1 ulp each) and are reduced in a fixed order
 *   (identical results from run to run): with mb_index (and perm converted to it) each thread first adds
 *   at most 256 of its samples into float32 sums per minibatch (a rounding error of at most 256 * 2^-24,
 *   1.5e-5, of the summed magnitudes), which are then reduced in float64; the gather path adds every term in
 *   float64. With mb_index every input is read once, in storage order. With perm and at most 64 minibatches the perm is first sorted into bins by
 *   destination (in the workspace), each sample's minibatch number is placed from them (in LDS up to 16
 *   minibatches, else in the workspace) and the samples are then read the same way, with the same bits as
 *   the equivalent mb_index; with more minibatches every read is a gather. perm entries outside [0, B) are clamped into it (a permutation
 *   has none). */
int rl_ppo_loss(const float* logits, const int32_t* actions, const float* old_logp, const float* adv,
                const float* ret, const float* new_values, const int32_t* perm, const uint16_t* mb_index,
                const double* adv_stats, int64_t B, int32_t A, int32_t mb, float clip_eps, float vf_coef,
                float ent_coef, float* out, void* ws, size_t ws_bytes, void* stream);

/* rl_ppo_loss for callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same arguments and results (the same kernels, so the same
 * bits) without ws / ws_bytes. Its workspace is a fixed 64 MiB array that the library holds on every device
 * it runs on, from its load until the process ends; the call allocates and frees nothing. The first call
 * on a device looks up that device's copy of the array (the device current at the call; `stream`, if not
 * NULL, must belong to it, else RL_EINVAL). A call whose workspace (rl_ppo_loss_workspace_bytes, less the
 * perm conversion's part when perm is NULL) exceeds 64 MiB returns RL_ESIZE and launches nothing: at
 * 16 minibatches that admits a perm up to 15,630,336 samples (1.86 x 2^23), at 32 or 64 up to about 10.7
 * million; mb_index any size (its partials take at most
 * 1.2 MB); contiguous minibatches while their partials (24 bytes per minibatch and block) fit. Every call on one device shares that device's array and keeps
 * no state in it between calls (nothing in it must start at zero): calls that overlap on one device, on
 * different streams or from different host threads without ordering, race on it. */
int rl_ppo_loss_noalloc(const float* logits, const int32_t* actions, const float* old_logp, const float* adv,
                        const float* ret, const float* new_values, const int32_t* perm, const uint16_t* mb_index,
                        const double* adv_stats, int64_t B, int32_t A, int32_t mb, float clip_eps, float vf_coef,
                        float ent_coef, float* out, void* stream);

/* rl_ppo_loss plus, in the same pass, the gradient of each minibatch's total loss
 * L_m = mean pg + vf_coef * mean v - ent_coef * mean H with respect to the logits and the value of every
 * sample of m (the next step of the learn phase in "Teaching Mario to speedrun", s.6; the loss and its
 * gradient computed in one pass as in the GPU-shader trainer of s.8). With p = softmax(logits[i]),
 * a = actions[i], M = mb and A, ratio as above:
 *   dlogits[i][j] = (1/M) (-u A ratio ([j == a] - p_j) + ent_coef p_j (log p_j + H)),
 *   dvalues[i]    = (1/M) 2 vf_coef (new_values[i] - ret[i]),
 * where u = 1 when ratio * A <= clip(ratio) * A (the minimum takes the unclipped term; inside the clip
 * band both terms are equal) and u = 0 on the clipped side. Advantages (normalised or not) are constants.
 *   dlogits  device f32[B][A] output, row i for sample i in storage order (16-byte aligned when A % 4 == 0);
 *   dvalues  device f32[B] output.
 * Every sample must belong to exactly one minibatch (perm a permutation; mb_index as above), so each
 * row is written once; out-of-range actions act as action 0 in both the loss and its gradient. All other
 * arguments, errors and the workspace are as for rl_ppo_loss; dlogits and dvalues must be non-NULL and
 * may not alias an input. */
int rl_ppo_loss_grad(const float* logits, const int32_t* actions, const float* old_logp, const float* adv,
                     const float* ret, const float* new_values, const int32_t* perm, const uint16_t* mb_index,
                     const double* adv_stats, int64_t B, int32_t A, int32_t mb, float clip_eps, float vf_coef,
                     float ent_coef, float* out, float* dlogits, float* dvalues, void* ws, size_t ws_bytes,
                     void* stream);

/* ---- Stand-in policy inference and the double-buffered rollout ---------------------------------- */

/* The inference a decision needs, standing in for the trainer's policy: the shape of PufferLib 5.0's
 * default policy ("Teaching Mario to speedrun", s.8: a bias-free linear encoder from the observation to
 * 128 numbers, one decoder matrix to the logits plus the value; its recurrent layers are left out) and
 * the heads of s.6 (12 logits sampled through a softmax, and the value). Weights are seeded stand-ins:
 * nothing here is trained. */
#define RL_POLICY_HIDDEN 128
#define RL_POLICY_ACTIONS 12
#define RL_ROLLOUT_MAX_GROUPS 8

/* Bytes of the packed weights rl_policy_pack writes (bfloat16 encoder padded to 1408 columns, float32
 * decoder). */
int rl_policy_weights_bytes(size_t* bytes);

/* Pack float32 weights into the caller's device buffer `packed` (256-byte aligned,
 * rl_policy_weights_bytes bytes), on `stream`:
 *   enc_w  device f32[128][1397]: hidden h = sum_k enc_w[h][k] obs[k] (rounded to bfloat16, nearest even);
 *   dec_w  device f32[13][128]: rows 0..11 the action logits, row 12 the value. */
int rl_policy_pack(const float* enc_w, const float* dec_w, void* packed, void* stream);

/* Inference for envs env_offset .. env_offset + n - 1 (global indices, < 2^24) at decision t >= 0:
 *   hidden = bf16(obs[e]) . bf16(enc_w)^T summed in float32 on the matrix cores; out = hidden . dec_w^T;
 *   actions[e] = argmax_j (out[j] + g_j) over the 12 logits, lowest j on a tie, with the Gumbel variate
 *   g_j = -ln(-ln u_j), u_j = (2 (x_j >> 41) + 1) / 2^24, x_j = SplitMix64 output
 *   mix64(seed + 0x9E3779B97F4A7C15 (16 (t 2^24 + env_offset + e) + j + 1)) (the Gumbel-max form of
 *   sampling from softmax(logits));
 *   logp[e] = out[a] - logsumexp(out[0..11]);  values[e] = out[12].
 *   obs device f32[n][obs_stride] (tile observations, obs_stride >= 1397); actions device int32[n];
 *   logp, values device f32[n]. n = 0 does nothing. */
int rl_policy_forward(const void* packed, const float* obs, int64_t n, int64_t obs_stride, uint64_t seed, int64_t t,
                      int64_t env_offset, int32_t* actions, float* logp, float* values, void* stream);

/* One env group of a rollout: decision t of the group's n envs (the env's num_envs) reads and writes
 *   actions + t*row, logp + t*row, values + t*row, rewards + t*row, dones + t*row   (n elements each),
 *   obs + t*obs_row                                                            (n x obs_stride floats),
 * so two groups can own the two halves of one [T][N] rollout (row = N, obs_row = N * obs_stride, the
 * second group's pointers offset by its first env). obs0 holds the observations decision 0 reads
 * ([n][obs_stride], e.g. the reset's). env_offset is the global index of the group's first env (it keys
 * the action draws). */
typedef struct rl_rollout_group {
    rl_env* env;
    const float* obs0;
    float* obs;
    int32_t* actions;
    float* logp;
    float* values;
    float* rewards;
    float* dones;
    int64_t row;
    int64_t obs_row;
    int64_t env_offset;
    void* stream;
} rl_rollout_group;

/* Rollout decisions t0 .. t0 + steps - 1 of every group ("PlayTrain", Figure 8C and Table 9, double
 * buffering). Per decision and per group, in group order, it enqueues on the group's stream the
 * inference on the group's previous observations (obs0 at t = 0, else obs + (t-1)*obs_row), whose draws
 * are keyed by the envs' decision counter, and then rl_env_step on the actions just written. One group
 * is the single-buffered rollout; with two groups on two streams one group's step runs while the
 * other's inference runs. The buffers must hold rows t0 .. t0 + steps - 1 (the library does not know
 * their length); every check (NULL buffers, 4-byte alignment, row lengths, env offsets, matching decision
 * counters) runs before anything is enqueued. The draws of each decision are keyed on the host (the
 * envs' host decision counter), so a captured rl_rollout replays the same draws: capture rl_env_step
 * loops, not rl_rollout. With `alternate` the groups also take turns at the inference: group g's
 * inference of a decision waits for group g-1's (group 0's waits for the last group's of the decision
 * before), which keeps them out of phase. Every group's env must use tile observations, no grapple hook
 * (the stand-in inference gives no aims) and stand at the same decision counter; env_offset must be a
 * multiple of the group's num_maps (a group's env n plays map n mod num_maps, global env env_offset + n
 * plays map (env_offset + n) mod num_maps); the adaptive respawn (whose outcome buffers and draws belong
 * to one env batch) needs a single group at env_offset 0. RL_EINVAL otherwise. Under these conditions the
 * results equal the single-buffered rollout's for the same envs. */
int rl_rollout(const void* packed, uint64_t seed, const rl_rollout_group* groups, int32_t num_groups, int32_t t0,
               int32_t steps, int32_t alternate);

/* ---- Measurement ------------------------------------------------------------------------------- */

/* A plain store kernel for the rooflines, not part of the rollout path: fills the device buffer `buf`
 * (16-byte aligned, `bytes` bytes, a multiple of 16) with 16-byte stores, each block of 256 threads
 * writing one contiguous chunk of `chunk` bytes (a multiple of 16; the last chunk may be shorter) and
 * exiting. Its bandwidth, timed beside a kernel whose blocks write chunks of the same size, is the write
 * ceiling for that granularity on the same device in the same run. */
int rl_store_probe(void* buf, int64_t bytes, int64_t chunk, void* stream);

/* Plain loads for the same purpose: `bytes` (a multiple of 16) of `buf` (device, 16-byte aligned) read with
 * 16-byte loads, one `chunk`-byte piece (a multiple of 16) per 256-thread block. Each block folds its words
 * by XOR and writes *sink (device uint32) only if the fold equals 0x9E3779B9, which keeps the loads and
 * never happens for a buffer of zeros. Timed beside a read-bound kernel, it is the read ceiling of that
 * granularity in the same run. Errors: RL_EINVAL (NULL, sizes), RL_EALIGN. */
int rl_read_probe(const void* buf, int64_t bytes, int64_t chunk, uint32_t* sink, void* stream);

/* Message for the last non-zero status returned on this thread ("" if none). */
const char* rl_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* RL_H */
