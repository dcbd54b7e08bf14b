// The batched tile platformer: device state layout, map padding, reset, step and observation kernels,
// and the rl_env_* entry points.
//
// What a step computes follows the pages named in rl.h: the platformer step of "Teaching Mario to
// speedrun" s.7 (a frame-skip loop of physics ticks, progress paid on a new best x, a terminal tick ends
// the loop), the DDNet post's tick protocol (frame-skip 3, rewards summed between decisions), its
// observation (43x31 tile window, 15-dim state x 4 frames, 4 checkpoint dims) and its reward (+10 per
// checkpoint in order, high-water-mark progress, time penalty, +100 finish), and PlayTrain's Table 4
// (terminated or truncated at the time limit). The pages leave the mechanics open; the constants and
// the tick order below are the reading used throughout (positions in sub-units of 1/256 tile).
//
// Device layout (inside the caller's state buffer, every region 256-byte aligned, Np = N rounded up to
// 64 so that every array row starts on a 256-byte boundary):
//   slots  int32[4][5][Np]  ring of the last 4 frames; slot s, word w of env n at (s*5 + w)*Np + n.
//                           Words: x, y, (vx & 0xffff) | vy << 16, flags / counters, tick. The newest
//                           slot is the current state; the decision counter mod 4 names it.
//   extra  int32[8][Np]     next checkpoint index, best x, waypoint high-water index, began-at-spawn flag,
//                           the step's ended outcome (checkpoints passed, bit 30 = began at the spawn;
//                           -1 when the env did not end; written in respawn mode only), and in hook mode
//                           the hook tip's x, y and flight velocity ((vx & 0xffff) | vy << 16).
//   map    u8[M][H+32][Wp]  the maps with a 16-row / 32-column solid border, Wp = round_up(W+64, 64),
//                           so that every read of the step and observation kernels stays inside.
//   ckpt   int32[M][K][2], spawn int32[M][2], sprites u8[16][8][8].
//   waypoints int32[M][Kw][2], wplens int32[M]            (waypoint reward only; empty otherwise)
//   spots int32[M][K][2], ring int32[M][64], rmeta int32[M][4] (fill, head, frontier, spare),
//   rhist int32[M][K+1]                                    (adaptive respawn only; empty otherwise)
//   ctr    int64[Np / 16]   the decision counter, one copy per block of a step launch: block b of a step
//                           uses word b (unless the launch carries the value) and writes it back plus one, so
//                           the counter lives on the device (a captured graph of steps advances it on every
//                           replay) with no atomics; every word holds the same value between launches, and
//                           other kernels read word 0.
// Structure-of-arrays keeps the lane-per-env state loads and stores coalesced.

#include <vector>

#include "rl_internal.hpp"

namespace {

constexpr int kTile = 256;
constexpr int kBox = 192;
constexpr int kHalfBox = 96;
constexpr int kGravity = 12;
constexpr int kMaxFall = 160;
constexpr int kJumpV = 120;
constexpr int kMaxVx = 48;
constexpr int kAccGround = 8;
constexpr int kAccAir = 4;
constexpr int kFreezeTicks = 30;
constexpr int kUnitsCkpt = 10240;     // +10 reward, 1024 units per reward
constexpr int kUnitsFinish = 102400;  // +100 reward
constexpr int kNumActions = 12;
// waypoint-path reward ("Reward Engineering", Version 2; readings)
constexpr int kWpAhead = 8;           // the nearest waypoint is searched at the high-water index and 8 past it
constexpr int kUnitsWaypoint = 256;   // one tile of path = 256 units
constexpr int kWpGrace = 1024;        // the 128-unit (about 4 tile) grace zone, sub-units
constexpr int kWpPenaltyShift = 4;    // beyond it: one unit per 16 sub-units of distance per tick
// adaptive checkpoint respawn ("Checkpoint Respawning"; readings)
constexpr int kRespawnBuf = RL_RESPAWN_BUF;          // outcomes kept per map
constexpr uint32_t kRespawnStartU32 = 858993459u;    // a draw below this (20% of 2^32) restarts at the spawn
constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;  // SplitMix64's increment
constexpr int kMaxRespawnCkpts = 1024;
// grapple hook aimed by a continuous aim ("boesch.dev DDNet RL post", What the agent sees and does: a hook
// button and an aim; the mechanics are readings): tip speed one tile a tick along the aim, 10 ticks of
// flight, a pull of twice gravity toward the tip, velocity components bounded by 160 while attached
constexpr int kHookSpeed = 256;
constexpr int kHookFlight = 10;
constexpr int kHookAccel = 24;
constexpr int kHookMaxV = 160;
// the step kernels' variants: bit 0 = the waypoint-path reward, bit 1 = the adaptive respawn, bit 2 = the
// grapple hook, bit 3 (with bit 2) = a frame skip above 3, where a hooked box can leave the 8x8 neighbourhood
constexpr int kModeWaypoints = 1;
constexpr int kModeRespawn = 2;
constexpr int kModeHook = 4;
constexpr int kModeHookFar = 8;

constexpr int kWinW = 43;
constexpr int kWinH = 31;
constexpr int kWinCx = 21;
constexpr int kWinCy = 15;
constexpr int kWinSize = kWinW * kWinH;                       // 1333
constexpr int kStack = 4;
constexpr int kFrameDims = 15;
constexpr int kObsTiles = kWinSize + kStack * kFrameDims + 4;  // 1397
constexpr int kPix = 84;
constexpr int kPixFrame = kPix * kPix;                         // 7056
constexpr int kPixRowDwords = kPix / 4;                        // 21

constexpr int kPadX = 32;
constexpr int kPadY = 16;
constexpr int kSlotWords = 5;
constexpr uint8_t kSolid = 1;
constexpr uint8_t kPlatform = 2;
constexpr uint8_t kFreeze = 3;

// Bits of the flags / counters word.
constexpr uint32_t kFacingRight = 1u << 0;
constexpr uint32_t kGroundedBit = 1u << 1;
constexpr uint32_t kJumpHeldBit = 1u << 2;
constexpr uint32_t kHookHeldBit = 1u << 3;
constexpr uint32_t kWallLBit = 1u << 4;
constexpr uint32_t kWallRBit = 1u << 5;
constexpr int kHookPhaseShift = 6;    // 2 bits, hook mode: idle 0, flying 1, attached 2
constexpr int kFreezeShift = 8;       // 5 bits, 0..30
constexpr int kHookShift = 16;        // 8 bits, 0..255: ticks the hook button has been held
constexpr int kActionShift = 24;      // 4 bits, 0..11
constexpr int kHookFlightShift = 28;  // 4 bits, hook mode: ticks the tip has flown
constexpr int kExtraRows = 8;

struct Layout {
    size_t slots, ctr, extra, map, ckpt, spawn, sprites, waypoints, wplens, spots, ring, rmeta, rhist, total;
    int64_t np, hp, wp;
};

struct EnvDev {
    int32_t* slots;
    int32_t* extra;
    const uint8_t* map;
    const int32_t* ckpt;
    const int32_t* spawn;
    const uint8_t* sprites;
    const int32_t* wpt;     // [M][kw][2] waypoint path (column, row), reward mode 1
    const int32_t* wplen;   // [M]
    const int32_t* spots;   // [M][k][2] respawn standing spots
    int32_t* ring;          // [M][kRespawnBuf] buffered outcomes
    int32_t* rmeta;         // [M][4] fill, head, frontier, -
    int32_t* rhist;         // [M][k + 1] counts of the buffered outcomes
    const int32_t* aim;     // [N] this step's aims (hook mode; NULL: no aim)
    uint64_t seed;          // respawn draws
    int64_t ovr;            // the counter taken from the launch instead of the device words (-1: read them)
    int32_t n, m, h, w, k, fs, time_limit, kw;
    int32_t hook;           // hook mode: frame dimension 9 is the hook's phase
    int64_t np, hp, wp;
    int64_t* ctr;           // [Np / 16] the decision counter, a word per step block
};

int validate_cfg(const rl_env_config* c)
{
    if (!c) return rl::fail(RL_EINVAL, "config is NULL");
    if (c->num_envs < 1 || c->num_envs > (1 << 24))
        return rl::fail(RL_EINVAL, "num_envs %d outside [1, 2^24]", c->num_envs);
    if (c->num_maps < 1 || c->num_maps > 65536)
        return rl::fail(RL_EINVAL, "num_maps %d outside [1, 65536]", c->num_maps);
    if (c->map_h < 1 || c->map_h > 4096) return rl::fail(RL_EINVAL, "map_h %d outside [1, 4096]", c->map_h);
    if (c->map_w < 1 || c->map_w > 65536) return rl::fail(RL_EINVAL, "map_w %d outside [1, 65536]", c->map_w);
    if (c->num_ckpts < 0 || c->num_ckpts > (1 << 20))
        return rl::fail(RL_EINVAL, "num_ckpts %d outside [0, 2^20]", c->num_ckpts);
    if (c->frame_skip < 1 || c->frame_skip > RL_MAX_FRAME_SKIP)
        return rl::fail(RL_EINVAL, "frame_skip %d outside [1, %d]", c->frame_skip, RL_MAX_FRAME_SKIP);
    if (c->time_limit < 1) return rl::fail(RL_EINVAL, "time_limit %d < 1", c->time_limit);
    if (c->obs_mode != RL_OBS_TILES && c->obs_mode != RL_OBS_PIXELS)
        return rl::fail(RL_EINVAL, "obs_mode %d is neither tiles (0) nor pixels (1)", c->obs_mode);
    const int64_t size = c->obs_mode == RL_OBS_TILES ? kObsTiles : kStack * kPixFrame;
    if (c->obs_stride < size)
        return rl::fail(RL_EINVAL, "obs_stride %lld < observation size %lld", (long long)c->obs_stride,
                        (long long)size);
    if (c->obs_mode == RL_OBS_PIXELS && c->obs_stride % 4 != 0)
        return rl::fail(RL_EALIGN, "pixel obs_stride %lld is not a multiple of 4", (long long)c->obs_stride);
    if (c->reward_mode != RL_REWARD_CHECKPOINTS && c->reward_mode != RL_REWARD_WAYPOINTS)
        return rl::fail(RL_EINVAL, "reward_mode %d is neither checkpoints (0) nor waypoints (1)", c->reward_mode);
    if (c->reward_mode == RL_REWARD_WAYPOINTS && (c->max_waypoints < 1 || c->max_waypoints > (1 << 20)))
        return rl::fail(RL_EINVAL, "max_waypoints %d outside [1, 2^20]", c->max_waypoints);
    if (c->respawn_mode != RL_RESPAWN_OFF && c->respawn_mode != RL_RESPAWN_ADAPTIVE)
        return rl::fail(RL_EINVAL, "respawn_mode %d is neither off (0) nor adaptive (1)", c->respawn_mode);
    if (c->respawn_mode == RL_RESPAWN_ADAPTIVE && (c->num_ckpts < 1 || c->num_ckpts > kMaxRespawnCkpts))
        return rl::fail(RL_EINVAL, "the adaptive respawn needs 1 .. %d checkpoints, got %d", kMaxRespawnCkpts,
                        c->num_ckpts);
    if (c->hook_mode != RL_HOOK_OFF && c->hook_mode != RL_HOOK_GRAPPLE)
        return rl::fail(RL_EINVAL, "hook_mode %d is neither off (0) nor grapple (1)", c->hook_mode);
    return RL_OK;
}

Layout layout_of(const rl_env_config* c)
{
    Layout l{};
    l.np = (int64_t)rl::round_up((size_t)c->num_envs, 64);
    l.hp = (int64_t)c->map_h + 2 * kPadY;
    l.wp = (int64_t)rl::round_up((size_t)c->map_w + 2 * kPadX, 64);
    size_t off = 0;
    l.slots = off;
    off = rl::round_up(off + sizeof(int32_t) * kStack * kSlotWords * l.np, 256);
    l.extra = off;   // next checkpoint, best x, path index, from-start flag, the step's ended outcome, hook
    off = rl::round_up(off + sizeof(int32_t) * kExtraRows * l.np, 256);
    l.map = off;
    off = rl::round_up(off + (size_t)c->num_maps * l.hp * l.wp, 256);
    l.ckpt = off;
    off = rl::round_up(off + sizeof(int32_t) * 2 * (size_t)c->num_maps * (c->num_ckpts > 0 ? c->num_ckpts : 1), 256);
    l.spawn = off;
    off = rl::round_up(off + sizeof(int32_t) * 2 * (size_t)c->num_maps, 256);
    l.sprites = off;
    off = rl::round_up(off + 16 * 64, 256);
    const size_t kw = c->reward_mode == RL_REWARD_WAYPOINTS ? (size_t)c->max_waypoints : 0;
    l.waypoints = off;
    off = rl::round_up(off + sizeof(int32_t) * 2 * kw * (size_t)c->num_maps, 256);
    l.wplens = off;
    off = rl::round_up(off + (kw ? sizeof(int32_t) * (size_t)c->num_maps : 0), 256);
    const bool rs = c->respawn_mode == RL_RESPAWN_ADAPTIVE;
    const size_t mm = rs ? (size_t)c->num_maps : 0;
    l.spots = off;
    off = rl::round_up(off + sizeof(int32_t) * 2 * mm * (size_t)c->num_ckpts, 256);
    l.ring = off;
    off = rl::round_up(off + sizeof(int32_t) * kRespawnBuf * mm, 256);
    l.rmeta = off;
    off = rl::round_up(off + sizeof(int32_t) * 4 * mm, 256);
    l.rhist = off;
    off = rl::round_up(off + sizeof(int32_t) * mm * ((size_t)c->num_ckpts + 1), 256);
    l.ctr = off;   // one word per 16 envs covers the tile step's blocks (16 envs) and the pixel step's (64)
    off = rl::round_up(off + sizeof(int64_t) * (size_t)(l.np / 16), 256);
    l.total = off;
    return l;
}

// ------------------------------------------------------------------------------------------------
// Device helpers
// ------------------------------------------------------------------------------------------------

__device__ __forceinline__ int32_t& slot_word(const EnvDev& d, int s, int w, int n)
{
    return d.slots[((int64_t)s * kSlotWords + w) * d.np + n];
}

// The decision counter as a step launch's block b sees it: its own word when the counter is kept on the
// device (DEV: a step recorded into a graph, or any step after one), else the launch's value.
template <bool DEV>
__device__ __forceinline__ int64_t step_counter(const EnvDev& d, int b) { return DEV ? d.ctr[b] : d.ovr; }

// A step launch's last act. On the device every block advances its own word (so no block can see a word
// another block of the launch has advanced); with the launch's value no block reads a word, and block 0
// writes them all, so that a step recorded into a graph later finds them current.
template <bool DEV>
__device__ __forceinline__ void advance_counter(const EnvDev& d, int64_t c)
{
    if constexpr (DEV) {
        if (threadIdx.x == 0) d.ctr[blockIdx.x] = c + 1;
    } else if (blockIdx.x == 0) {
        for (unsigned i = threadIdx.x; i < gridDim.x; i += blockDim.x) d.ctr[i] = c + 1;
    }
}

// The counter as any other kernel sees it: the launch's value, else word 0 (which every step advances).
__device__ __forceinline__ int64_t current_counter(const EnvDev& d) { return d.ovr >= 0 ? d.ovr : d.ctr[0]; }

__device__ __forceinline__ const uint8_t* map_base(const EnvDev& d, int m)
{
    return d.map + (int64_t)m * d.hp * d.wp;
}

// Address of tile (row, col) of padded map m; row/col are map coordinates (may be in the border).
__device__ __forceinline__ const uint8_t* tile_ptr(const EnvDev& d, int m, int row, int col)
{
    return map_base(d, m) + (int64_t)(row + kPadY) * d.wp + (col + kPadX);
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Observation value of frame dimension `dim` from a slot's five words (all conversions exact). In hook
// mode dimension 9 is the hook's phase instead of the ticks the button has been held.
__device__ __forceinline__ float frame_dim(int dim, int32_t x, int32_t y, int32_t vxy, uint32_t misc,
                                           int32_t tick, bool hook)
{
    switch (dim) {
    case 0: return (float)x * 0x1p-8f;
    case 1: return (float)y * 0x1p-8f;
    case 2: return (float)(int16_t)(vxy & 0xffff) * 0x1p-8f;
    case 3: return (float)(vxy >> 16) * 0x1p-8f;
    case 4: return (misc & kGroundedBit) ? 1.0f : 0.0f;
    case 5: return (misc & kFacingRight) ? 1.0f : -1.0f;
    case 6: return ((misc >> kFreezeShift) & 31u) ? 1.0f : 0.0f;
    case 7: return (float)((misc >> kFreezeShift) & 31u);
    case 8: return (misc & kHookHeldBit) ? 1.0f : 0.0f;
    case 9: return hook ? (float)((misc >> kHookPhaseShift) & 3u) : (float)((misc >> kHookShift) & 255u);
    case 10: return (misc & kJumpHeldBit) ? 1.0f : 0.0f;
    case 11: return (misc & kWallLBit) ? 1.0f : 0.0f;
    case 12: return (misc & kWallRBit) ? 1.0f : 0.0f;
    case 13: return (float)tick * 0x1p-11f;
    default: return (float)((misc >> kActionShift) & 15u);
    }
}

// ------------------------------------------------------------------------------------------------
// Set-up kernels
// ------------------------------------------------------------------------------------------------

// Padded map copy, one dword of the destination per thread; cells outside the source map are solid.
__global__ __launch_bounds__(256) void k_pad_maps(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                  int32_t m_count, int32_t h, int32_t w, int64_t hp, int64_t wp)
{
    const int64_t dwords = (int64_t)m_count * hp * wp / 4;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < dwords;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t byte0 = i * 4;
        const int64_t m = byte0 / (hp * wp);
        const int64_t rem = byte0 - m * hp * wp;
        const int64_t row = rem / wp - kPadY;
        const int64_t col0 = rem % wp - kPadX;
        uint32_t word = 0;
        for (int j = 0; j < 4; ++j) {
            const int64_t col = col0 + j;
            uint32_t t = kSolid;
            if (row >= 0 && row < h && col >= 0 && col < w) t = src[(m * h + row) * w + col];
            word |= t << (8 * j);
        }
        reinterpret_cast<uint32_t*>(dst)[i] = word;
    }
}

__device__ __forceinline__ void write_spawn(const EnvDev& d, int n)
{
    const int m = n % d.m;
    const int32_t x = d.spawn[2 * m], y = d.spawn[2 * m + 1];
    for (int s = 0; s < kStack; ++s) {
        slot_word(d, s, 0, n) = x;
        slot_word(d, s, 1, n) = y;
        slot_word(d, s, 2, n) = 0;
        slot_word(d, s, 3, n) = (int32_t)(kFacingRight | kGroundedBit);
        slot_word(d, s, 4, n) = 0;
    }
    d.extra[n] = 0;
    d.extra[d.np + n] = x;
    d.extra[2 * d.np + n] = 0;
    d.extra[3 * d.np + n] = 1;
    d.extra[5 * d.np + n] = 0;
    d.extra[6 * d.np + n] = 0;
    d.extra[7 * d.np + n] = 0;
}

__global__ __launch_bounds__(256) void k_reset(EnvDev d, const uint8_t* __restrict__ mask)
{
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= d.n) return;
    if (mask && !mask[n]) return;
    write_spawn(d, n);
}

// ------------------------------------------------------------------------------------------------
// env_step: one lane per env.
// ------------------------------------------------------------------------------------------------

// Solid / freeze bits of the 8x8 tiles around the player at the start of a decision: bit
// (row - rb) * 8 + (col - cb). With |vx| <= 48 and -108 <= vy <= 160 per tick, up to 5 ticks keep every
// probe of the decision inside rows r0-3 .. r0+4 and columns c0-2 .. c0+5 of the starting box corner.
struct Neighbourhood {
    uint64_t solid, freeze;
    int rb, cb;
    __device__ __forceinline__ uint32_t s(int row, int col) const
    {
        return (uint32_t)(solid >> ((row - rb) * 8 + (col - cb))) & 1u;
    }
    __device__ __forceinline__ uint32_t f(int row, int col) const
    {
        return (uint32_t)(freeze >> ((row - rb) * 8 + (col - cb))) & 1u;
    }
};

// floor(sqrt(v)) for an integer-valued v in [0, 2^53): the rounded square root, then checked exactly.
__device__ __forceinline__ double floor_sqrt(double v)
{
    double r = floor(sqrt(v));
    while (r * r > v) r -= 1.0;
    while ((r + 1.0) * (r + 1.0) <= v) r += 1.0;
    return r;
}

__device__ __forceinline__ Neighbourhood load_neighbourhood(const EnvDev& d, int m, int32_t x, int32_t y)
{
    Neighbourhood nb;
    // Clamping only matters for a spawn placed outside the map; it keeps every read in the border.
    nb.rb = clampi(y >> 8, 0, d.h - 1) - 3;
    nb.cb = clampi(x >> 8, 0, d.w - 1) - 2;
    uint64_t rows[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) __builtin_memcpy(&rows[i], tile_ptr(d, m, nb.rb + i, nb.cb), 8);
    uint64_t s = 0, f = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t t = (uint32_t)(rows[i] >> (8 * j)) & 0xffu;
            s |= (uint64_t)(t == kSolid || t == kPlatform) << (i * 8 + j);
            f |= (uint64_t)(t == kFreeze) << (i * 8 + j);
        }
    }
    nb.solid = s;
    nb.freeze = f;
    return nb;
}

// The five words of one ring slot.
struct SlotWords {
    int32_t x, y, vxy, misc, tick;
};

// Hook mode's inputs of a decision: the tip (x, y), its flight velocity ((vx & 0xffff) | vy << 16) and the
// decision's aim ((dx & 0xffff) | dy << 16).
struct HookIn {
    int32_t x, y, v, aim;
};

template <int MODE>
__device__ __forceinline__ HookIn load_hook(const EnvDev& d, int n)
{
    if constexpr ((MODE & kModeHook) != 0)
        return HookIn{d.extra[5 * d.np + n], d.extra[6 * d.np + n], d.extra[7 * d.np + n], d.aim ? d.aim[n] : 0};
    else
        return HookIn{0, 0, 0, 0};
}

__device__ __forceinline__ SlotWords load_slot(const EnvDev& d, int s, int n)
{
    return SlotWords{slot_word(d, s, 0, n), slot_word(d, s, 1, n), slot_word(d, s, 2, n), slot_word(d, s, 3, n),
                     slot_word(d, s, 4, n)};
}

// The words of the newest ring slot after a decision, plus the extras and whether the env was reset.
struct Decision {
    int32_t x, y, vxy, misc, tick, next, best_x;
    bool done;
};

// The candidates of a tick: the waypoints at the high-water index (clamped to the path's end) and the
// kWpAhead after it, loaded unconditionally with indices clamped to the end so that the loads issue together.
__device__ __forceinline__ void wp_candidates(const EnvDev& d, int m, int32_t path, int2* w)
{
    const int32_t len = clampi(d.wplen[m], 1, d.kw);
    const int32_t p0 = min(path, len - 1);
    const int2* row = reinterpret_cast<const int2*>(d.wpt) + (int64_t)m * d.kw;
#pragma unroll
    for (int j = 0; j <= kWpAhead; ++j) w[j] = row[min(p0 + j, len - 1)];
}

// Reward mode 1's progress and distance terms of one tick: the waypoint nearest to the box centre among
// the high-water index and the kWpAhead after it (the lowest index on a tie); moving the high-water index
// forward pays kUnitsWaypoint per waypoint; a distance d = floor(sqrt(d2)) beyond the grace zone costs
// (d - kWpGrace) >> kWpPenaltyShift units. w holds the candidates, from wp_candidates. Squared distances
// are exact in float64: positions and waypoint centres lie below 2^25 sub-units, so d2 < 2^51 (full-rate
// float64 instead of 64-bit integer multiplies); d = floor(sqrt(d2)) is checked against d2 exactly, and
// needed only past the zone.
__device__ __forceinline__ int32_t waypoint_units(const EnvDev& d, int m, int32_t x, int32_t y, int32_t& path,
                                                  const int2* w)
{
    const int32_t len = clampi(d.wplen[m], 1, d.kw);
    if (path > len - 1) path = len - 1;
    const double cx = (double)(x + kHalfBox), cy = (double)(y + kHalfBox);
    int32_t best = path;
    double best_d2 = 0.0;
#pragma unroll
    for (int j = 0; j <= kWpAhead; ++j) {
        const double dx = cx - (double)(w[j].x * kTile + kTile / 2);
        const double dy = cy - (double)(w[j].y * kTile + kTile / 2);
        const double d2 = fma(dx, dx, dy * dy);
        if (j == 0 || (path + j < len && d2 < best_d2)) {
            best_d2 = d2;
            best = path + j;
        }
    }
    int32_t units = 0;
    if (best > path) {
        units += (best - path) * kUnitsWaypoint;
        path = best;
    }
    if (best_d2 >= (double)((kWpGrace + 1) * (kWpGrace + 1))) {
        units -= (int32_t)(((int64_t)floor_sqrt(best_d2) - kWpGrace) >> kWpPenaltyShift);
    }
    return units;
}

// ------------------------------------------------------------------------------------------------
// Adaptive checkpoint respawn.
// ------------------------------------------------------------------------------------------------

// SplitMix64's output function (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
// 2014).
__device__ __forceinline__ uint64_t splitmix_output(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// The checkpoint an ended episode of env n on map m restarts at (0 = the spawn), from the map's buffer as
// it stood at the start of the step (the buffers change only in k_respawn_append, after the step). The
// draws are SplitMix64's first and second outputs from the state seed + 2 golden (counter 2^24 + n). The
// top quarter of the buffer is read off its histogram: the max(1, fill / 4)-th largest outcome thr, the
// cand outcomes >= thr, and the (pick + 1)-th largest of them.
__device__ int32_t respawn_choice(const EnvDev& d, int m, int n, int64_t counter)
{
    const int32_t* meta = d.rmeta + 4 * m;
    const int32_t fill = meta[0];
    if (fill == 0) return 0;
    const uint64_t key = (uint64_t)counter * ((uint64_t)1 << 24) + (uint64_t)n;
    const uint64_t state = d.seed + 2 * kGolden * key;
    if ((uint32_t)(splitmix_output(state + kGolden) >> 32) < kRespawnStartU32) return 0;
    const int32_t* hist = d.rhist + (int64_t)m * (d.k + 1);
    const int32_t q = max(1, fill / 4);
    int32_t cand = 0, thr = 0;
    for (int32_t v = d.k; v >= 0; --v) {
        cand += hist[v];
        if (cand >= q) {
            thr = v;
            break;
        }
    }
    if (cand == 0) return 0;   // a histogram that disagrees with fill (not produced by this library)
    const uint32_t pick = (uint32_t)(splitmix_output(state + 2 * kGolden) >> 32) % (uint32_t)cand;
    int32_t acc = 0, chosen = thr;
    for (int32_t v = d.k; v >= thr; --v) {
        acc += hist[v];
        if ((int32_t)pick < acc) {
            chosen = v;
            break;
        }
    }
    return max(0, min(min(chosen, meta[2]), d.k - 1));
}

// Start a new episode of env n on map m at checkpoint k in all four ring slots and the extras: the spawn
// for k = 0, else checkpoint k - 1's standing spot with k checkpoints passed. Returns its decision.
template <bool HOOK>
__device__ __forceinline__ Decision spawn_at(const EnvDev& d, int n, int m, int32_t k)
{
    int32_t x = d.spawn[2 * m], y = d.spawn[2 * m + 1];
    if (k > 0) {
        const int32_t* p = d.spots + ((int64_t)m * d.k + (k - 1)) * 2;
        x = p[0];
        y = p[1];
    }
    const int32_t misc = (int32_t)(kFacingRight | kGroundedBit);
    for (int s = 0; s < kStack; ++s) {
        slot_word(d, s, 0, n) = x;
        slot_word(d, s, 1, n) = y;
        slot_word(d, s, 2, n) = 0;
        slot_word(d, s, 3, n) = misc;
        slot_word(d, s, 4, n) = 0;
    }
    d.extra[n] = k;
    d.extra[d.np + n] = x;
    d.extra[2 * d.np + n] = 0;
    d.extra[3 * d.np + n] = k == 0 ? 1 : 0;
    if constexpr (HOOK) {
        d.extra[5 * d.np + n] = 0;
        d.extra[6 * d.np + n] = 0;
        d.extra[7 * d.np + n] = 0;
    }
    return Decision{x, y, 0, misc, 0, k, x, true};
}

// After the step: one block per map appends the step's ended outcomes to the map's ring in env order (only
// the last kRespawnBuf survive), raises the frontier by those that began at the spawn, and recounts the
// ring's histogram.
__global__ __launch_bounds__(256) void k_respawn_append(EnvDev d)
{
    __shared__ int32_t part[256];
    __shared__ int32_t fmax[256];
    __shared__ int32_t hist[kMaxRespawnCkpts + 1];
    const int m = blockIdx.x;
    const int t = threadIdx.x;
    const int cnt = m < d.n ? (d.n - m + d.m - 1) / d.m : 0;   // envs of map m: n = m + M i, i < cnt
    const int per = (cnt + 255) / 256;
    const int i0 = min(cnt, t * per), i1 = min(cnt, i0 + per);
    const int32_t* ended = d.extra + 4 * d.np;
    int32_t mine = 0, front = 0;
    for (int i = i0; i < i1; ++i) {
        const int32_t e = ended[m + (int64_t)d.m * i];
        if (e >= 0) {
            ++mine;
            if ((e >> 30) & 1) front = max(front, e & ((1 << 30) - 1));
        }
    }
    if (!__syncthreads_or(mine)) return;          // uniform: nothing ended on this map this step
    part[t] = mine;
    fmax[t] = front;
    __syncthreads();
    // inclusive scan of the per-thread counts (fixed order), and the frontier candidate
    for (int off = 1; off < 256; off <<= 1) {
        const int32_t a = t >= off ? part[t - off] : 0;
        const int32_t b = t >= off ? fmax[t - off] : 0;
        __syncthreads();
        part[t] += a;
        fmax[t] = max(fmax[t], b);
        __syncthreads();
    }
    const int32_t total = part[255];
    int32_t* meta = d.rmeta + 4 * m;
    int32_t* ring = d.ring + (int64_t)m * kRespawnBuf;
    const int32_t head = meta[1];
    int32_t p = part[t] - mine;                   // this thread's first append position
    for (int i = i0; i < i1; ++i) {
        const int32_t e = ended[m + (int64_t)d.m * i];
        if (e >= 0) {
            if (p >= total - kRespawnBuf) ring[(head + p) % kRespawnBuf] = e & ((1 << 30) - 1);
            ++p;
        }
    }
    for (int v = t; v <= d.k; v += 256) hist[v] = 0;
    __syncthreads();                              // ring writes and the cleared histogram
    const int32_t fill = min(meta[0] + total, kRespawnBuf);
    if (t < fill) atomicAdd(&hist[min(max(ring[t], 0), d.k)], 1);
    __syncthreads();
    int32_t* gh = d.rhist + (int64_t)m * (d.k + 1);
    for (int v = t; v <= d.k; v += 256) gh[v] = hist[v];
    if (t == 0) {
        meta[0] = fill;
        meta[1] = (head + total) % kRespawnBuf;
        meta[2] = max(meta[2], fmax[255]);
    }
}

// Zero the respawn state (create).
__global__ __launch_bounds__(256) void k_zero(int32_t* __restrict__ p, int64_t count)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

template <int MODE>
__device__ __forceinline__ Decision env_decide(const EnvDev& d, int n, int32_t a, const SlotWords& cur, int32_t next,
                                               int32_t best_x, int32_t path, int32_t from_start, const HookIn& hk,
                                               float* __restrict__ rewards, float* __restrict__ dones, int64_t counter)
{
    const int head_new = (int)((counter + 1) & 3);
    constexpr bool kHook = (MODE & kModeHook) != 0;
    const int m = n % d.m;
    int32_t x = cur.x;
    int32_t y = cur.y;
    const int32_t vxy = cur.vxy;
    const uint32_t misc = (uint32_t)cur.misc;
    int32_t tick = cur.tick;
    if (a < 0 || a >= kNumActions) a = 0;

    int32_t vx = (int16_t)(vxy & 0xffff);
    int32_t vy = vxy >> 16;
    int32_t facing = (misc & kFacingRight) ? 1 : -1;
    uint32_t grounded = (misc & kGroundedBit) ? 1u : 0u;
    int32_t freeze = (int32_t)((misc >> kFreezeShift) & 31u);
    int32_t hook_ticks = (int32_t)((misc >> kHookShift) & 255u);
    uint32_t wall_l = (misc & kWallLBit) ? 1u : 0u, wall_r = (misc & kWallRBit) ? 1u : 0u;
    uint32_t jump_held = (misc & kJumpHeldBit) ? 1u : 0u, hook_held = (misc & kHookHeldBit) ? 1u : 0u;
    int32_t phase = kHook ? (int32_t)((misc >> kHookPhaseShift) & 3u) : 0;
    int32_t flight = kHook ? (int32_t)((misc >> kHookFlightShift) & 15u) : 0;
    int32_t hx = hk.x, hy = hk.y;
    int32_t hvx = (int16_t)(hk.v & 0xffff), hvy = hk.v >> 16;
    const int32_t adx = (int16_t)(hk.aim & 0xffff), ady = hk.aim >> 16;

    const Neighbourhood nb = load_neighbourhood(d, m, x, y);
    // A hook can push either velocity component to 160 a tick. Over at most 3 ticks the box (192 wide) then
    // moves at most 480 sub-units, less than two tiles, and every probe stays in rows r0-2..r0+3 and
    // columns c0-2..c0+3, inside the neighbourhood. With 4 or 5 ticks a probe can leave it (by up to 4 tiles
    // in any direction), so the kModeHookFar variants read such a tile from the padded map instead (cached;
    // rare, as it needs a fast swing), clamped into the border, which is solid like everything outside.
    constexpr bool kFar = (MODE & kModeHookFar) != 0;
    const auto tile_at = [&](int row, int col) __attribute__((always_inline)) -> uint32_t {
        return *tile_ptr(d, m, clampi(row, -kPadY, d.h + kPadY - 1), clampi(col, -kPadX, d.w + kPadX - 1));
    };
    const auto solid_at = [&](int row, int col) __attribute__((always_inline)) -> uint32_t {
        if constexpr (kFar) {
            if ((unsigned)(row - nb.rb) >= 8u || (unsigned)(col - nb.cb) >= 8u) {
                const uint32_t t = tile_at(row, col);
                return (t == kSolid || t == kPlatform) ? 1u : 0u;
            }
        }
        return nb.s(row, col);
    };
    const auto freeze_at = [&](int row, int col) __attribute__((always_inline)) -> uint32_t {
        if constexpr (kFar) {
            if ((unsigned)(row - nb.rb) >= 8u || (unsigned)(col - nb.cb) >= 8u) return tile_at(row, col) == kFreeze ? 1u : 0u;
        }
        return nb.f(row, col);
    };
    const int32_t* ck = d.ckpt + (int64_t)m * d.k * 2;
    int32_t ck_col = next < d.k ? ck[2 * next] : 0;

    const int dir = a >> 2;
    const int jump_in = (a >> 1) & 1;
    const int hook_in = a & 1;

    int32_t units = 0;
    bool terminated = false, truncated = false;
    for (int i = 0; i < d.fs && !terminated && !truncated; ++i) {
        // the tick's waypoint candidates depend only on the index the previous tick left, so they are
        // loaded first and the tick's physics runs while they arrive
        int2 wc[kWpAhead + 1];
        if constexpr ((MODE & kModeWaypoints) != 0) wp_candidates(d, m, path, wc);
        // 1. a frozen player's input is ignored
        const bool frozen = freeze > 0;
        const int sign = frozen ? 0 : (dir == 1 ? -1 : (dir == 2 ? 1 : 0));
        const int jump = frozen ? 0 : jump_in;
        const int hook = frozen ? 0 : hook_in;
        // 2. horizontal velocity moves toward sign * MAX_VX without overshoot
        const int32_t target = sign * kMaxVx;
        const int32_t acc = grounded ? kAccGround : kAccAir;
        vx = vx < target ? min(vx + acc, target) : (vx > target ? max(vx - acc, target) : vx);
        if (sign != 0) facing = sign;
        // 3-4. jump from the ground, gravity, terminal fall speed
        if (jump && grounded) vy = -kJumpV;
        vy = min(vy + kGravity, kMaxFall);
        // 4h. the grapple hook: letting go retracts it; a new press with a non-zero aim fires the tip from
        // the box centre at kHookSpeed along the aim (each component truncated toward zero after dividing by
        // the aim's floored length); a flying tip moves once a tick and attaches in the first tile it lands
        // in that blocks movement (the border included), or is lost after kHookFlight ticks; an attached
        // hook adds kHookAccel toward the tip (same rounding) and bounds each velocity component.
        if constexpr (kHook) {
            if (!hook) {
                phase = 0;
            } else if (phase == 0 && !hook_held && (adx | ady) != 0) {
                const int32_t len = (int32_t)floor_sqrt((double)adx * adx + (double)ady * ady);
                hvx = adx * kHookSpeed / len;
                hvy = ady * kHookSpeed / len;
                hx = x + kHalfBox;
                hy = y + kHalfBox;
                flight = 0;
                phase = 1;
            }
            if (phase == 1) {
                hx += hvx;
                hy += hvy;
                flight += 1;
                // the tip never gets past the first border tile, which holds it; the clamp only matters for
                // a spawn placed outside the map
                const uint32_t t = tile_at(hy >> 8, hx >> 8);
                if (t == kSolid || t == kPlatform) phase = 2;
                else if (flight >= kHookFlight) phase = 0;
            }
            if (phase == 2) {
                const int32_t ex = hx - (x + kHalfBox), ey = hy - (y + kHalfBox);
                const int32_t dist = (int32_t)floor_sqrt((double)ex * ex + (double)ey * ey);
                if (dist > 0) {
                    vx += ex * kHookAccel / dist;
                    vy += ey * kHookAccel / dist;
                }
                vx = clampi(vx, -kHookMaxV, kHookMaxV);
                vy = clampi(vy, -kHookMaxV, kHookMaxV);
            }
        }
        // 5. x move against the rows of the box before the y move
        {
            int32_t nx = x + vx;
            const int r0 = y >> 8, r1 = (y + kBox - 1) >> 8;
            if (vx > 0) {
                const int col = (nx + kBox - 1) >> 8;
                if (solid_at(r0, col) | solid_at(r1, col)) { nx = col * kTile - kBox; vx = 0; }
            } else if (vx < 0) {
                const int col = nx >> 8;
                if (solid_at(r0, col) | solid_at(r1, col)) { nx = (col + 1) * kTile; vx = 0; }
            }
            x = nx;
        }
        // 6. y move against the columns of the box after the x move
        {
            int32_t ny = y + vy;
            const int c0 = x >> 8, c1 = (x + kBox - 1) >> 8;
            if (vy > 0) {
                const int row = (ny + kBox - 1) >> 8;
                if (solid_at(row, c0) | solid_at(row, c1)) { ny = row * kTile - kBox; vy = 0; }
            } else if (vy < 0) {
                const int row = ny >> 8;
                if (solid_at(row, c0) | solid_at(row, c1)) { ny = (row + 1) * kTile; vy = 0; }
            }
            y = ny;
        }
        // 7-8. contacts of the final box; touching a freeze tile re-arms the counter
        {
            const int c0 = x >> 8, c1 = (x + kBox - 1) >> 8;
            const int r0 = y >> 8, r1 = (y + kBox - 1) >> 8;
            const int below = (y + kBox) >> 8;
            grounded = solid_at(below, c0) | solid_at(below, c1);
            const int cl = (x - 1) >> 8, cr = (x + kBox) >> 8;
            wall_l = solid_at(r0, cl) | solid_at(r1, cl);
            wall_r = solid_at(r0, cr) | solid_at(r1, cr);
            const uint32_t touching = freeze_at(r0, c0) | freeze_at(r0, c1) | freeze_at(r1, c0) | freeze_at(r1, c1);
            freeze = touching ? kFreezeTicks : (freeze > 0 ? freeze - 1 : 0);
        }
        // 9. hook and jump state
        hook_ticks = hook ? min(hook_ticks + 1, 255) : 0;
        hook_held = (uint32_t)hook;
        jump_held = (uint32_t)jump;
        // 10. progress: past the high-water mark of x (mode 0), or along the waypoint path (mode 1); best x
        // is kept in both (it is an observation dim)
        if constexpr ((MODE & kModeWaypoints) != 0) units += waypoint_units(d, m, x, y, path, wc);
        if (x > best_x) {
            if constexpr ((MODE & kModeWaypoints) == 0) units += x - best_x;
            best_x = x;
        }
        // 11. checkpoints in order (+10 each in mode 0); the last one is the finish
        if (next < d.k && ((x + kHalfBox) >> 8) >= ck_col) {
            if constexpr ((MODE & kModeWaypoints) == 0) units += kUnitsCkpt;
            next += 1;
            if (next == d.k) { units += kUnitsFinish; terminated = true; }
            else ck_col = ck[2 * next];
        }
        // 12. time (a penalty in mode 0 only)
        tick += 1;
        if constexpr ((MODE & kModeWaypoints) == 0) units -= 1;
        if (tick >= d.time_limit) truncated = true;
    }

    rewards[n] = (float)units * 0x1p-10f;
    const bool done = terminated || truncated;
    dones[n] = done ? 1.0f : 0.0f;
    if (done) {
        int32_t k = 0;
        if constexpr ((MODE & kModeRespawn) != 0) {
            d.extra[4 * d.np + n] = next | (from_start ? (1 << 30) : 0);   // the ended episode's outcome
            k = respawn_choice(d, m, n, counter);
        }
        return spawn_at<kHook>(d, n, m, k);
    }
    if constexpr ((MODE & kModeRespawn) != 0) d.extra[4 * d.np + n] = -1;
    const uint32_t new_misc = (facing > 0 ? kFacingRight : 0u) | (grounded ? kGroundedBit : 0u) |
                              (jump_held ? kJumpHeldBit : 0u) | (hook_held ? kHookHeldBit : 0u) |
                              (wall_l ? kWallLBit : 0u) | (wall_r ? kWallRBit : 0u) |
                              ((uint32_t)freeze << kFreezeShift) | ((uint32_t)hook_ticks << kHookShift) |
                              ((uint32_t)a << kActionShift) |
                              (kHook ? ((uint32_t)phase << kHookPhaseShift) | ((uint32_t)flight << kHookFlightShift)
                                     : 0u);
    slot_word(d, head_new, 0, n) = x;
    slot_word(d, head_new, 1, n) = y;
    slot_word(d, head_new, 2, n) = (int32_t)(((uint32_t)vx & 0xffffu) | ((uint32_t)vy << 16));
    slot_word(d, head_new, 3, n) = (int32_t)new_misc;
    slot_word(d, head_new, 4, n) = tick;
    d.extra[n] = next;
    d.extra[d.np + n] = best_x;
    if constexpr ((MODE & kModeWaypoints) != 0) d.extra[2 * d.np + n] = path;
    if constexpr (kHook) {
        d.extra[5 * d.np + n] = hx;
        d.extra[6 * d.np + n] = hy;
        d.extra[7 * d.np + n] = (int32_t)(((uint32_t)hvx & 0xffffu) | ((uint32_t)hvy << 16));
    }
    return Decision{x, y, (int32_t)(((uint32_t)vx & 0xffffu) | ((uint32_t)vy << 16)), (int32_t)new_misc, tick,
                    next, best_x, false};
}

// env_step alone (the pixel path renders in its own kernel): one lane per env, one-wave blocks so that a
// small batch still spreads over every CU (the kernel is latency-bound: a few waves per CU at most).
template <int MODE, bool DEV>
__global__ __launch_bounds__(64) void k_step(EnvDev d, const int32_t* __restrict__ actions,
                                              float* __restrict__ rewards, float* __restrict__ dones)
{
    const int64_t c = step_counter<DEV>(d, blockIdx.x);
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    if (n < d.n)
        env_decide<MODE>(d, n, actions[n], load_slot(d, (int)(c & 3), n), d.extra[n], d.extra[d.np + n],
                     (MODE & kModeWaypoints) != 0 ? d.extra[2 * d.np + n] : 0,
                         (MODE & kModeRespawn) != 0 ? d.extra[3 * d.np + n] : 1, load_hook<MODE>(d, n), rewards,
                         dones, c);
    advance_counter<DEV>(d, c);
}

// ------------------------------------------------------------------------------------------------
// obs_gather, tile mode: one wave per env writes its 1397 floats as 22 fully coalesced 256-byte rows.
// ------------------------------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_obs_tiles(EnvDev d, float* __restrict__ obs, int64_t stride)
{
    const int head = (int)(current_counter(d) & 3);
    const int lane = threadIdx.x & 63;
    const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (n >= d.n) return;
    const int m = n % d.m;
    const int32_t x = slot_word(d, head, 0, n);
    const int32_t y = slot_word(d, head, 1, n);
    const int pcol = clampi((x + kHalfBox) >> 8, 0, d.w - 1);
    const int prow = clampi((y + kHalfBox) >> 8, 0, d.h - 1);
    const uint8_t* win = tile_ptr(d, m, prow - kWinCy, pcol - kWinCx);
    float* o = obs + (int64_t)n * stride;

    // element k = lane + 64 i sits at window row r, column c; stepping k by 64 = 43 + 21 moves one row
    // down and 21 columns right (wrapping into the next row).
    int r = lane >= kWinW ? 1 : 0;
    int c = lane - r * kWinW;
#pragma unroll
    for (int i = 0; i < (kObsTiles + 63) / 64; ++i) {
        const int k = lane + 64 * i;
        if (k < kWinSize) {
            o[k] = (float)win[(int64_t)r * d.wp + c];
        } else if (k < kObsTiles) {
            const int t = k - kWinSize;
            float v;
            if (t < kStack * kFrameDims) {
                const int f = t / kFrameDims, dim = t - f * kFrameDims;
                const int s = (head - f) & 3;
                v = frame_dim(dim, slot_word(d, s, 0, n), slot_word(d, s, 1, n), slot_word(d, s, 2, n),
                              (uint32_t)slot_word(d, s, 3, n), slot_word(d, s, 4, n), d.hook != 0);
            } else {
                const int q = t - kStack * kFrameDims;
                const int32_t next = d.extra[n];
                if (q == 0 || q == 1) {
                    if (next < d.k) {
                        const int32_t* ckp = d.ckpt + ((int64_t)m * d.k + next) * 2;
                        v = q == 0 ? (float)(ckp[0] * kTile + kTile / 2 - (x + kHalfBox)) * 0x1p-8f
                                   : (float)(ckp[1] * kTile + kTile / 2 - (y + kHalfBox)) * 0x1p-8f;
                    } else {
                        v = 0.0f;
                    }
                } else if (q == 2) {
                    v = (float)next;
                } else {
                    v = (float)d.extra[d.np + n] * 0x1p-8f;
                }
            }
            o[k] = v;
        }
        r += 1;
        c += 64 - kWinW;
        if (c >= kWinW) { c -= kWinW; r += 1; }
    }
}

// ------------------------------------------------------------------------------------------------
// env_step + obs_gather fused, tile mode. A block of 256 threads owns E consecutive envs.
//   Phase A (threads 0 .. E-1, one env each): every physics-independent load first (action, current
//   ring slot, the two older slots, extras), then the decision. The env's 64 non-window observation
//   values (4 frames of 15, newest first, and 4 checkpoint dims) and its window's top-left address go
//   to LDS.
//   Phase B (wave w writes the rows of envs w, w+4, ...): the wave first reads every one of its envs'
//   31-row windows from the padded map (11 unaligned dwords per row, about 6 per lane and env) and parks
//   them in LDS as 44-byte rows; only then does it store. Loads and stores share one in-order completion
//   counter, so a load issued after a store could only be waited for together with that store. Each row
//   is written with wave-wide 16-byte stores from its first 16-byte boundary (scalar head and tail
//   elements around them), so any stride works. Four window values come from two LDS dwords and one
//   byte permute, which also skips the spare 44th byte when the four straddle a window row.
// ------------------------------------------------------------------------------------------------

constexpr int kTail = kObsTiles - kWinSize;       // 64
constexpr int kRowBytes = 44;                     // a window row in LDS: 43 tiles + 1 spare byte
constexpr int kRowDwords = kRowBytes / 4;         // 11
constexpr int kWinDwords = kWinH * kRowDwords;    // 341 per env
constexpr int kWinPerLane = (kWinDwords + 63) / 64;   // 6
constexpr int kStepTilesEnvs = 16;                // envs per block of the fused tile kernel

template <bool HOOK>
__device__ __forceinline__ void put_frame(float* t, int32_t x, int32_t y, int32_t vxy, uint32_t misc, int32_t tick)
{
#pragma unroll
    for (int dim = 0; dim < kFrameDims; ++dim) t[dim] = frame_dim(dim, x, y, vxy, misc, tick, HOOK);
}

// Observation element k (< 1397) from a staged window and the staged frame / checkpoint values.
__device__ __forceinline__ float staged_elem(const uint8_t* win, const float* tail, int k)
{
    if (k < kWinSize) {
        const int r = k / kWinW;
        return (float)win[r * kRowBytes + (k - r * kWinW)];
    }
    return tail[k - kWinSize];
}

// One observation row from a staged window (w32, 31 rows of 44 bytes) and staged tail values, written by
// one wave. The float4s that lie wholly in the window take six fixed passes whose LDS reads are all
// issued before the first store; the few that reach into the tail follow in one pass.
__device__ __forceinline__ void write_row(const uint32_t* w32, const float* te, float* row, int lane)
{
    const uint8_t* win = reinterpret_cast<const uint8_t*>(w32);
    const int h = (int)((4 - ((reinterpret_cast<uintptr_t>(row) >> 2) & 3)) & 3);  // scalars before 16 B
    const int nq = (kObsTiles - h) >> 2;                                           // aligned float4s
    const int nwin = (kWinSize - h) >> 2;                                          // ... inside the window
    constexpr int kPasses = (kWinSize / 4 + 63) / 64;                              // 6
    if (lane < h) row[lane] = staged_elem(win, te, lane);
    uint32_t w[kPasses];
#pragma unroll
    for (int j = 0; j < kPasses; ++j) {
        const int k = h + 4 * min(lane + 64 * j, nwin - 1);
        const int r = k / kWinW;
        const int c = k - r * kWinW;
        const int D = k + r;                                  // byte of (r, c) in the staged rows
        uint32_t sel = (uint32_t)(D & 3) * 0x01010101u + 0x03020100u;
        const int avail = kWinW - c;
        if (avail < 4) sel += 0x01010101u << (8 * avail);    // skip the spare byte
        w[j] = __builtin_amdgcn_perm(w32[(D >> 2) + 1], w32[D >> 2], sel);
    }
#pragma unroll
    for (int j = 0; j < kPasses; ++j) {
        const int q = lane + 64 * j;
        if (q < nwin) {
            float4 o;
            o.x = (float)(w[j] & 0xffu);
            o.y = (float)((w[j] >> 8) & 0xffu);
            o.z = (float)((w[j] >> 16) & 0xffu);
            o.w = (float)(w[j] >> 24);
            *reinterpret_cast<float4*>(row + h + 4 * q) = o;
        }
    }
    if (nwin + lane < nq) {
        const int k = h + 4 * (nwin + lane);
        *reinterpret_cast<float4*>(row + k) = make_float4(staged_elem(win, te, k), staged_elem(win, te, k + 1),
                                                          staged_elem(win, te, k + 2), staged_elem(win, te, k + 3));
    }
    const int t0 = h + 4 * nq;
    if (lane < kObsTiles - t0) row[t0 + lane] = staged_elem(win, te, t0 + lane);
}

// This lane's share of an env's window: dwords lane, lane + 64, ... of its 31 rows of 11.
__device__ __forceinline__ void load_window(const EnvDev& d, int64_t base, int lane, uint32_t (&v)[kWinPerLane])
{
#pragma unroll
    for (int j = 0; j < kWinPerLane; ++j) {
        const int i = min(lane + 64 * j, kWinDwords - 1);
        const int r = i / kRowDwords, c4 = i - r * kRowDwords;
        __builtin_memcpy(&v[j], d.map + base + (int64_t)r * d.wp + 4 * c4, 4);
    }
}

// Phase A for env e (< ne) of the group starting at n0: every physics-independent load first, then the
// decision; the 64 non-window observation values go to tail[e] and the window's top-left offset to wbase[e].
template <int E, int MODE>
__device__ __forceinline__ void decide_env(const EnvDev& d, int n0, int e, const int32_t* __restrict__ actions,
                                           float* __restrict__ rewards, float* __restrict__ dones, int64_t counter,
                                           float (*tail)[kTail], int64_t* wbase)
{
    const int head_prev = (int)(counter & 3);
    const int n = n0 + e;
    const int m = n % d.m;
    const int32_t a = actions[n];
    const SlotWords cur = load_slot(d, head_prev, n);
    // the two older slots are only written out; in hook mode they are loaded after the decision, whose
    // state the hook enlarges, to keep the registers within four waves a SIMD
    SlotWords old1{}, old2{};
    if constexpr ((MODE & kModeHook) == 0) {
        old1 = load_slot(d, (head_prev - 1) & 3, n);
        old2 = load_slot(d, (head_prev - 2) & 3, n);
    }
    const int32_t next0 = d.extra[n], best0 = d.extra[d.np + n];
    const int32_t path0 = (MODE & kModeWaypoints) != 0 ? d.extra[2 * d.np + n] : 0;
    const int32_t start0 = (MODE & kModeRespawn) != 0 ? d.extra[3 * d.np + n] : 1;
    const HookIn hk = load_hook<MODE>(d, n);
    const Decision s = env_decide<MODE>(d, n, a, cur, next0, best0, path0, start0, hk, rewards, dones, counter);
    constexpr bool kHook = (MODE & kModeHook) != 0;
    float* t = tail[e];
    put_frame<kHook>(t, s.x, s.y, s.vxy, (uint32_t)s.misc, s.tick);
    if (s.done) {
#pragma unroll
        for (int f = 1; f < kStack; ++f)
#pragma unroll
            for (int dim = 0; dim < kFrameDims; ++dim) t[f * kFrameDims + dim] = t[dim];
    } else {
        if constexpr (kHook) {
            old1 = load_slot(d, (head_prev - 1) & 3, n);
            old2 = load_slot(d, (head_prev - 2) & 3, n);
        }
        put_frame<kHook>(t + kFrameDims, cur.x, cur.y, cur.vxy, (uint32_t)cur.misc, cur.tick);
        put_frame<kHook>(t + 2 * kFrameDims, old1.x, old1.y, old1.vxy, (uint32_t)old1.misc, old1.tick);
        put_frame<kHook>(t + 3 * kFrameDims, old2.x, old2.y, old2.vxy, (uint32_t)old2.misc, old2.tick);
    }
    float* ck = t + kStack * kFrameDims;
    if (s.next < d.k) {
        const int32_t* p = d.ckpt + ((int64_t)m * d.k + s.next) * 2;
        ck[0] = (float)(p[0] * kTile + kTile / 2 - (s.x + kHalfBox)) * 0x1p-8f;
        ck[1] = (float)(p[1] * kTile + kTile / 2 - (s.y + kHalfBox)) * 0x1p-8f;
    } else {
        ck[0] = 0.0f;
        ck[1] = 0.0f;
    }
    ck[2] = (float)s.next;
    ck[3] = (float)s.best_x * 0x1p-8f;
    const int pcol = clampi((s.x + kHalfBox) >> 8, 0, d.w - 1);
    const int prow = clampi((s.y + kHalfBox) >> 8, 0, d.h - 1);
    wbase[e] = tile_ptr(d, m, prow - kWinCy, pcol - kWinCx) - d.map;
}

// Phase B for the group starting at n0 (ne envs), by four waves: wave w owns envs w, w + 4, ... It first
// reads its envs' windows from the padded map into wwin (loads and stores share one in-order completion
// counter, so every load goes before the first store), then writes each env's observation row.
template <int E>
__device__ __forceinline__ void write_group(const EnvDev& d, int n0, int ne, int wave, int lane,
                                            uint32_t (*wwin)[kWinDwords + 1], const float (*tail)[kTail],
                                            const int64_t* wbase, float* __restrict__ obs, int64_t stride)
{
    constexpr int EW = E / 4;                 // envs per wave
    constexpr int EB = EW <= 6 ? EW : 4;      // windows in registers at once
    static_assert(EW % EB == 0, "whole batches");
#pragma unroll 1
    for (int b = 0; b < EW; b += EB) {
        uint32_t v[EB][kWinPerLane];
#pragma unroll
        for (int i = 0; i < EB; ++i)
            if (wave + 4 * (b + i) < ne) load_window(d, wbase[wave + 4 * (b + i)], lane, v[i]);
#pragma unroll
        for (int i = 0; i < EB; ++i)
            if (wave + 4 * (b + i) < ne) {
#pragma unroll
                for (int j = 0; j < kWinPerLane; ++j)
                    if (lane + 64 * j < kWinDwords) wwin[wave + 4 * (b + i)][lane + 64 * j] = v[i][j];
            }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    for (int e = wave; e < ne; e += 4) write_row(wwin[e], tail[e], obs + (int64_t)(n0 + e) * stride, lane);
}

template <int E, int MODE, bool DEV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_step_tiles(EnvDev d, const int32_t* __restrict__ actions,
                                                    float* __restrict__ rewards, float* __restrict__ dones,
                                                    float* __restrict__ obs, int64_t stride)
{
    static_assert(E % 4 == 0 && E <= 64, "whole envs per wave; one lane per env in phase A");
    __shared__ uint32_t wwin[E][kWinDwords + 1];
    __shared__ float tail[E][kTail];
    __shared__ int64_t wbase[E];
    const int n0 = blockIdx.x * E;
    const int ne = min(E, d.n - n0);
    if ((int)threadIdx.x < ne) {
        decide_env<E, MODE>(d, n0, threadIdx.x, actions, rewards, dones, step_counter<DEV>(d, blockIdx.x), tail,
                            wbase);
    } else if (!DEV && blockIdx.x == 0 && threadIdx.x >= 64) {
        // the launch's value: waves 1-3 of block 0, idle while wave 0 decides, write every block's word
        for (unsigned i = threadIdx.x - 64; i < gridDim.x; i += blockDim.x - 64) d.ctr[i] = d.ovr + 1;
    }
    __syncthreads();
    write_group<E>(d, n0, ne, threadIdx.x >> 6, threadIdx.x & 63, wwin, tail, wbase, obs, stride);
    // on the device each block advances its own word, last: a store earlier in the wave would hold up the
    // waits of its window loads, which share the wave's one completion counter with the stores
    if (DEV && threadIdx.x == 0) d.ctr[blockIdx.x] = step_counter<DEV>(d, blockIdx.x) + 1;
}

// ------------------------------------------------------------------------------------------------
// obs_gather, pixel mode: one block per env, one wave per stacked frame. Each frame is re-rendered from
// the position kept in its ring slot (recomputing 7 KB from the cached map is cheaper than storing and
// re-reading it). The wave first stages the frame's camera tiles (at most 12 x 12; 12 rows of 16
// bytes) in LDS beside the block's sprite table. Lanes then own (row offset, pixel dword) pairs, 3 rows
// of 21 dwords per pass, so a lane's tile column, sub-tile shift and player-box column mask are fixed
// for the whole frame. A pixel dword (4 pixels of one row) takes two tile codes and their two 8-pixel
// sprite rows from LDS and one byte-align; the player box is OR-ed in as a byte mask. Each pass stores
// 3 consecutive rows (252 bytes) per wave.
// ------------------------------------------------------------------------------------------------

constexpr int kCamTiles = 12;      // tile rows / columns a camera row / column can touch (84 px span 11-12)
constexpr int kCamTileStride = 16; // bytes per staged tile row

__global__ __launch_bounds__(256) void k_obs_pixels(EnvDev d, uint8_t* __restrict__ obs, int64_t stride)
{
    __shared__ uint2 spr[16 * 8];                                  // sprite rows, 8 pixels each
    __shared__ uint32_t cam[4][kCamTiles * kCamTileStride / 4];    // each frame's camera tiles
    reinterpret_cast<uint32_t*>(spr)[threadIdx.x] = reinterpret_cast<const uint32_t*>(d.sprites)[threadIdx.x];
    const int n = blockIdx.x;
    const int f = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int m = n % d.m;
    const int s = (int)((current_counter(d) - f) & 3);   // the frame's ring slot
    const int32_t x = clampi(slot_word(d, s, 0, n), 0, d.w * kTile - 1);
    const int32_t y = clampi(slot_word(d, s, 1, n), 0, d.h * kTile - 1);
    const int cam_x = ((x + kHalfBox) >> 5) - kPix / 2;
    const int cam_y = ((y + kHalfBox) >> 5) - kPix / 2;
    const int tx0 = cam_x >> 3, ty0 = cam_y >> 3;
    const int bx0 = x >> 5, bx1 = (x + kBox - 1) >> 5;
    const int by0 = y >> 5, by1 = (y + kBox - 1) >> 5;
    // stage tiles: lane < 48 copies 4 bytes of staged row lane / 4 (unaligned map read, in the border)
    if (lane < kCamTiles * kCamTileStride / 4) {
        const int r = lane >> 2, c4 = lane & 3;
        uint32_t w;
        __builtin_memcpy(&w, tile_ptr(d, m, ty0 + r, tx0 + 4 * c4), 4);
        cam[f][lane] = w;
    }
    __syncthreads();
    const uint8_t* tiles = reinterpret_cast<const uint8_t*>(cam[f]);
    uint32_t* o = reinterpret_cast<uint32_t*>(obs + (int64_t)n * stride + (int64_t)f * kPixFrame);

    // lane -> (row offset rl in 0..2, dword jl in 0..20 of the row); lane 63 idles. Everything that
    // depends only on the column is fixed for the frame.
    const int rl = lane / kPixRowDwords, jl = lane - rl * kPixRowDwords;
    if (lane >= 3 * kPixRowDwords) return;
    const int wx = cam_x + 4 * jl;
    const int tc = (wx >> 3) - tx0;                  // 0 .. 10
    const int ofs = wx & 7;                          // first pixel's column inside tile tc
    const bool upper = ofs >= 4;
    const uint32_t shift = (uint32_t)(ofs & 3);
    const int lo_b = max(bx0 - wx, 0), hi_b = min(bx1 - wx, 3);
    const uint32_t boxmask =
        lo_b <= hi_b ? (0xffffffffu >> (8 * (3 - hi_b))) & (0xffffffffu << (8 * lo_b)) : 0u;
    // 28 passes for every lane (84 rows in steps of 3 from its row offset): a fixed count, unrolled, so
    // that the LDS reads of several passes are in flight together
#pragma unroll
    for (int i = 0; i < kPix / 3; ++i) {
        const int py = rl + 3 * i;
        const int wy = cam_y + py;
        const int sy = wy & 7;
        const uint8_t* trow = tiles + ((wy >> 3) - ty0) * kCamTileStride + tc;
        const uint2 a = spr[(trow[0] & 15u) * 8 + sy];
        const uint2 b = spr[(trow[1] & 15u) * 8 + sy];
        uint32_t w = __builtin_amdgcn_alignbyte(upper ? b.x : a.y, upper ? a.y : a.x, shift);
        if (wy >= by0 && wy <= by1) w |= boxmask;
        o[py * kPixRowDwords + jl] = w;
    }
}

// The adaptive respawn's per-map state, one block (64 lanes = the ring) per map.
__global__ __launch_bounds__(64) void k_read_respawn(EnvDev d, int32_t* __restrict__ ring, int32_t* __restrict__ fill,
                                                     int32_t* __restrict__ head, int32_t* __restrict__ frontier)
{
    const int m = blockIdx.x;
    ring[(int64_t)m * kRespawnBuf + threadIdx.x] = d.ring[(int64_t)m * kRespawnBuf + threadIdx.x];
    if (threadIdx.x == 0) {
        fill[m] = d.rmeta[4 * m];
        head[m] = d.rmeta[4 * m + 1];
        frontier[m] = d.rmeta[4 * m + 2];
    }
}

// Decode the newest slot and the extras into the canonical int32[N][RL_STATE_FIELDS] state.
__global__ __launch_bounds__(256) void k_read_state(EnvDev d, int32_t* __restrict__ out)
{
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= d.n) return;
    const int head = (int)(current_counter(d) & 3);
    const int32_t vxy = slot_word(d, head, 2, n);
    const uint32_t misc = (uint32_t)slot_word(d, head, 3, n);
    int32_t* o = out + (int64_t)n * RL_STATE_FIELDS;
    o[0] = slot_word(d, head, 0, n);
    o[1] = slot_word(d, head, 1, n);
    o[2] = (int16_t)(vxy & 0xffff);
    o[3] = vxy >> 16;
    o[4] = (misc & kFacingRight) ? 1 : -1;
    o[5] = (int32_t)((misc >> kFreezeShift) & 31u);
    o[6] = (int32_t)((misc >> kHookShift) & 255u);
    o[7] = (misc & kHookHeldBit) ? 1 : 0;
    o[8] = (misc & kJumpHeldBit) ? 1 : 0;
    o[9] = (misc & kGroundedBit) ? 1 : 0;
    o[10] = (misc & kWallLBit) ? 1 : 0;
    o[11] = (misc & kWallRBit) ? 1 : 0;
    o[12] = slot_word(d, head, 4, n);
    o[13] = d.extra[n];
    o[14] = d.extra[d.np + n];
    o[16] = d.extra[2 * d.np + n];
    o[17] = d.extra[3 * d.np + n];
    o[15] = (int32_t)((misc >> kActionShift) & 15u);
    const int32_t hv = d.extra[7 * d.np + n];
    o[18] = (int32_t)((misc >> kHookPhaseShift) & 3u);
    o[19] = d.extra[5 * d.np + n];
    o[20] = d.extra[6 * d.np + n];
    o[21] = (int16_t)(hv & 0xffff);
    o[22] = hv >> 16;
    o[23] = (int32_t)((misc >> kHookFlightShift) & 15u);
}

// The device decision counter into out.
__global__ void k_read_counter(EnvDev d, int64_t* __restrict__ out) { *out = current_counter(d); }

}  // namespace

struct rl_env {
    rl_env_config cfg;
    Layout lay;
    uint8_t* base;
    int64_t counter;    // decisions enqueued through the entry points (graph replays advance only the device's)
    int64_t pending;    // a value set by rl_env_set_step_counter that no step has applied yet (-1: none)
    bool synced;        // the device words hold `counter` (false from a captured step until a value is set)
    bool waypoints_set;
    bool spots_set;
};

namespace {

EnvDev dev_of(const rl_env* e)
{
    EnvDev d;
    d.slots = reinterpret_cast<int32_t*>(e->base + e->lay.slots);
    d.extra = reinterpret_cast<int32_t*>(e->base + e->lay.extra);
    d.map = e->base + e->lay.map;
    d.ckpt = reinterpret_cast<const int32_t*>(e->base + e->lay.ckpt);
    d.spawn = reinterpret_cast<const int32_t*>(e->base + e->lay.spawn);
    d.sprites = e->base + e->lay.sprites;
    d.wpt = reinterpret_cast<const int32_t*>(e->base + e->lay.waypoints);
    d.wplen = reinterpret_cast<const int32_t*>(e->base + e->lay.wplens);
    d.kw = e->cfg.reward_mode == RL_REWARD_WAYPOINTS ? e->cfg.max_waypoints : 0;
    d.spots = reinterpret_cast<const int32_t*>(e->base + e->lay.spots);
    d.ring = reinterpret_cast<int32_t*>(e->base + e->lay.ring);
    d.rmeta = reinterpret_cast<int32_t*>(e->base + e->lay.rmeta);
    d.rhist = reinterpret_cast<int32_t*>(e->base + e->lay.rhist);
    d.seed = e->cfg.respawn_seed;
    d.ctr = reinterpret_cast<int64_t*>(e->base + e->lay.ctr);
    d.ovr = e->pending;
    d.n = e->cfg.num_envs;
    d.m = e->cfg.num_maps;
    d.h = e->cfg.map_h;
    d.w = e->cfg.map_w;
    d.k = e->cfg.num_ckpts;
    d.fs = e->cfg.frame_skip;
    d.time_limit = e->cfg.time_limit;
    d.hook = e->cfg.hook_mode == RL_HOOK_GRAPPLE ? 1 : 0;
    d.aim = nullptr;
    d.np = e->lay.np;
    d.hp = e->lay.hp;
    d.wp = e->lay.wp;
    return d;
}

// Whether work enqueued on st is being recorded into a graph.
bool capturing(hipStream_t st)
{
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(st, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone;
}

// The counter a launch hands its kernels in place of the device words: a value set on the host and not yet
// applied, else the host's count while it equals the words and the launch is not recorded into a graph (a
// replay must read the words, which earlier replays advanced). -1 makes the kernels read the words.
int64_t launch_counter(const rl_env* e, bool cap)
{
    if (e->pending >= 0) return e->pending;
    return e->synced && !cap ? e->counter : -1;
}

int launch_obs(const rl_env* e, void* obs, hipStream_t st)
{
    EnvDev d = dev_of(e);
    d.ovr = launch_counter(e, capturing(st));
    if (e->cfg.obs_mode == RL_OBS_TILES) {
        hipLaunchKernelGGL(k_obs_tiles, dim3((d.n + 3) / 4), dim3(256), 0, st, d, static_cast<float*>(obs),
                           e->cfg.obs_stride);
    } else {
        hipLaunchKernelGGL(k_obs_pixels, dim3(d.n), dim3(256), 0, st, d, static_cast<uint8_t*>(obs),
                           e->cfg.obs_stride);
    }
    return rl::check_launch("obs_gather");
}

int check_obs_ptr(const rl_env* e, const void* obs)
{
    if (!obs) return rl::fail(RL_EINVAL, "obs is NULL");
    if (!rl::aligned(obs, 4)) return rl::fail(RL_EALIGN, "obs is not 4-byte aligned");
    (void)e;
    return RL_OK;
}

}  // namespace

extern "C" {

int rl_env_state_bytes(const rl_env_config* cfg, size_t* bytes)
{
    if (int rc = validate_cfg(cfg)) return rc;
    if (!bytes) return rl::fail(RL_EINVAL, "bytes is NULL");
    *bytes = layout_of(cfg).total;
    return RL_OK;
}

int rl_env_obs_size(const rl_env_config* cfg, size_t* elems, size_t* elem_bytes)
{
    if (int rc = validate_cfg(cfg)) return rc;
    if (!elems || !elem_bytes) return rl::fail(RL_EINVAL, "output pointer is NULL");
    *elems = cfg->obs_mode == RL_OBS_TILES ? kObsTiles : (size_t)kStack * kPixFrame;
    *elem_bytes = cfg->obs_mode == RL_OBS_TILES ? 4 : 1;
    return RL_OK;
}

int rl_step_layout(const rl_env_config* cfg, size_t offsets[4], size_t* block_bytes)
{
    if (int rc = validate_cfg(cfg)) return rc;
    if (!offsets || !block_bytes) return rl::fail(RL_EINVAL, "output pointer is NULL");
    const size_t n = (size_t)cfg->num_envs;
    const size_t esz = cfg->obs_mode == RL_OBS_TILES ? 4 : 1;
    offsets[0] = 0;
    offsets[1] = rl::round_up(n * 4, 256);
    offsets[2] = rl::round_up(offsets[1] + n * (size_t)cfg->obs_stride * esz, 256);
    offsets[3] = rl::round_up(offsets[2] + n * 4, 256);
    *block_bytes = rl::round_up(offsets[3] + n * 4, 256);
    return RL_OK;
}

int rl_env_create(const rl_env_config* cfg, const uint8_t* maps, const int32_t* ckpts, const int32_t* spawns,
                  const uint8_t* sprites, void* state, size_t state_bytes, void* stream, rl_env** out)
{
    if (int rc = validate_cfg(cfg)) return rc;
    if (!out) return rl::fail(RL_EINVAL, "out is NULL");
    *out = nullptr;
    if (!maps || !spawns || !state) return rl::fail(RL_EINVAL, "maps, spawns and state must be non-NULL");
    if (cfg->num_ckpts > 0 && !ckpts) return rl::fail(RL_EINVAL, "ckpts is NULL with num_ckpts > 0");
    if (cfg->obs_mode == RL_OBS_PIXELS && !sprites) return rl::fail(RL_EINVAL, "pixel mode needs sprites");
    if (!rl::aligned(state, 256)) return rl::fail(RL_EALIGN, "state buffer is not 256-byte aligned");
    if (!rl::aligned(ckpts, 4) || !rl::aligned(spawns, 4))
        return rl::fail(RL_EALIGN, "ckpts / spawns are not 4-byte aligned");
    const Layout lay = layout_of(cfg);
    if (state_bytes < lay.total)
        return rl::fail(RL_ESIZE, "state buffer has %zu bytes, needs %zu", state_bytes, lay.total);

    rl_env* e = new (std::nothrow) rl_env;
    if (!e) return rl::fail(RL_EINVAL, "out of host memory");
    e->cfg = *cfg;
    e->lay = lay;
    e->base = static_cast<uint8_t*>(state);
    e->counter = 0;
    e->pending = -1;
    e->synced = true;
    e->waypoints_set = false;
    e->spots_set = false;
    hipStream_t st = rl::as_stream(stream);
    uint8_t* base = e->base;

    const int64_t dwords = (int64_t)cfg->num_maps * lay.hp * lay.wp / 4;
    const int blocks = (int)std::min<int64_t>((dwords + 255) / 256, 65536);
    hipLaunchKernelGGL(k_pad_maps, dim3(blocks), dim3(256), 0, st, maps, base + lay.map, cfg->num_maps,
                       cfg->map_h, cfg->map_w, lay.hp, lay.wp);
    int rc = rl::check_launch("pad_maps");
    hipError_t he = hipSuccess;
    if (rc == RL_OK && cfg->num_ckpts > 0)
        he = hipMemcpyAsync(base + lay.ckpt, ckpts, sizeof(int32_t) * 2 * (size_t)cfg->num_maps * cfg->num_ckpts,
                            hipMemcpyDeviceToDevice, st);
    if (rc == RL_OK && he == hipSuccess)
        he = hipMemcpyAsync(base + lay.spawn, spawns, sizeof(int32_t) * 2 * (size_t)cfg->num_maps,
                            hipMemcpyDeviceToDevice, st);
    if (rc == RL_OK && he == hipSuccess && cfg->obs_mode == RL_OBS_PIXELS)
        he = hipMemcpyAsync(base + lay.sprites, sprites, 16 * 64, hipMemcpyDeviceToDevice, st);
    if (rc == RL_OK && he != hipSuccess) rc = rl::fail(RL_EHIP, "table copy: %s", hipGetErrorString(he));
    if (rc == RL_OK) {   // the decision counter starts at 0
        const int64_t words = (int64_t)(lay.total - lay.ctr) / 4;
        hipLaunchKernelGGL(k_zero, dim3((unsigned)std::min<int64_t>((words + 255) / 256, 4096)), dim3(256), 0, st,
                           reinterpret_cast<int32_t*>(base + lay.ctr), words);
        rc = rl::check_launch("counter");
    }
    if (rc == RL_OK && cfg->respawn_mode == RL_RESPAWN_ADAPTIVE) {
        // ring, meta and histogram are contiguous: zero them together
        const int64_t words = (int64_t)(lay.total - lay.ring) / 4;
        hipLaunchKernelGGL(k_zero, dim3((unsigned)std::min<int64_t>((words + 255) / 256, 4096)), dim3(256), 0, st,
                           reinterpret_cast<int32_t*>(base + lay.ring), words);
        rc = rl::check_launch("respawn state");
    }
    if (rc == RL_OK) {
        const EnvDev d = dev_of(e);
        hipLaunchKernelGGL(k_reset, dim3((cfg->num_envs + 255) / 256), dim3(256), 0, st, d,
                           static_cast<const uint8_t*>(nullptr));
        rc = rl::check_launch("reset");
    }
    if (rc != RL_OK) {
        delete e;
        return rc;
    }
    *out = e;
    return RL_OK;
}

int rl_env_reset(rl_env* e, const uint8_t* mask, void* obs, void* stream)
{
    if (!e) return rl::fail(RL_EINVAL, "env is NULL");
    if (obs)
        if (int rc = check_obs_ptr(e, obs)) return rc;
    hipStream_t st = rl::as_stream(stream);
    const EnvDev d = dev_of(e);
    hipLaunchKernelGGL(k_reset, dim3((d.n + 255) / 256), dim3(256), 0, st, d, mask);
    if (int rc = rl::check_launch("reset")) return rc;
    if (obs) return launch_obs(e, obs, st);
    return RL_OK;
}

int rl_env_step_aim(rl_env* e, const int32_t* actions, const int32_t* aim, void* obs, float* rewards, float* dones,
                    void* stream)
{
    if (!e) return rl::fail(RL_EINVAL, "env is NULL");
    if (!actions || !rewards || !dones) return rl::fail(RL_EINVAL, "actions, rewards and dones must be non-NULL");
    if (!rl::aligned(actions, 4) || !rl::aligned(rewards, 4) || !rl::aligned(dones, 4) || !rl::aligned(aim, 4))
        return rl::fail(RL_EALIGN, "actions / aim / rewards / dones are not 4-byte aligned");
    const bool hk = e->cfg.hook_mode == RL_HOOK_GRAPPLE;
    if (aim && !hk) return rl::fail(RL_EINVAL, "aims given to an env without the grapple hook");
    if (int rc = check_obs_ptr(e, obs)) return rc;
    const bool wp = e->cfg.reward_mode == RL_REWARD_WAYPOINTS;
    const bool rs = e->cfg.respawn_mode == RL_RESPAWN_ADAPTIVE;
    if (wp && !e->waypoints_set) return rl::fail(RL_EINVAL, "waypoint rewards need rl_env_set_waypoints first");
    if (rs && !e->spots_set) return rl::fail(RL_EINVAL, "the adaptive respawn needs rl_env_set_respawn_spots first");
    hipStream_t st = rl::as_stream(stream);
    const bool cap = capturing(st);
    // a counter set on the host is applied by this launch; inside a capture it would be baked into the graph
    // and reapplied on every replay
    if (cap && e->pending >= 0)
        return rl::fail(RL_EINVAL, "rl_env_set_step_counter was called since the last step: run a step outside the "
                                   "capture first");
    if (cap) e->synced = false;   // replays advance the device words unseen by the host
    EnvDev d = dev_of(e);
    d.ovr = launch_counter(e, cap);
    const bool dev = d.ovr < 0;   // the step kernels read the device words
    d.aim = aim;
    const int mode = (wp ? kModeWaypoints : 0) | (rs ? kModeRespawn : 0) | (hk ? kModeHook : 0) |
                     (hk && e->cfg.frame_skip > 3 ? kModeHookFar : 0);
    if (e->cfg.obs_mode == RL_OBS_TILES) {
        const dim3 grid((d.n + kStepTilesEnvs - 1) / kStepTilesEnvs), block(256);
        float* o = static_cast<float*>(obs);
        const int64_t os = e->cfg.obs_stride;
#define RL_STEP_TILES(M)                                                                                     \
    if (dev) hipLaunchKernelGGL((k_step_tiles<kStepTilesEnvs, M, true>), grid, block, 0, st, d, actions, rewards, \
                                dones, o, os);                                                                \
    else hipLaunchKernelGGL((k_step_tiles<kStepTilesEnvs, M, false>), grid, block, 0, st, d, actions, rewards,    \
                            dones, o, os)
        switch (mode) {
        case 0: RL_STEP_TILES(0); break;
        case 1: RL_STEP_TILES(1); break;
        case 2: RL_STEP_TILES(2); break;
        case 3: RL_STEP_TILES(3); break;
        case 4: RL_STEP_TILES(4); break;
        case 5: RL_STEP_TILES(5); break;
        case 6: RL_STEP_TILES(6); break;
        case 7: RL_STEP_TILES(7); break;
        case 12: RL_STEP_TILES(12); break;
        case 13: RL_STEP_TILES(13); break;
        case 14: RL_STEP_TILES(14); break;
        default: RL_STEP_TILES(15); break;
        }
#undef RL_STEP_TILES
        if (int rc = rl::check_launch("env_step+obs_gather")) return rc;
    } else {
        const dim3 grid((d.n + 63) / 64), block(64);
#define RL_STEP(M)                                                                                           \
    if (dev) hipLaunchKernelGGL((k_step<M, true>), grid, block, 0, st, d, actions, rewards, dones);            \
    else hipLaunchKernelGGL((k_step<M, false>), grid, block, 0, st, d, actions, rewards, dones)
        switch (mode) {
        case 0: RL_STEP(0); break;
        case 1: RL_STEP(1); break;
        case 2: RL_STEP(2); break;
        case 3: RL_STEP(3); break;
        case 4: RL_STEP(4); break;
        case 5: RL_STEP(5); break;
        case 6: RL_STEP(6); break;
        case 7: RL_STEP(7); break;
        case 12: RL_STEP(12); break;
        case 13: RL_STEP(13); break;
        case 14: RL_STEP(14); break;
        default: RL_STEP(15); break;
        }
#undef RL_STEP
        if (int rc = rl::check_launch("env_step")) return rc;
    }
    if (rs) {
        hipLaunchKernelGGL(k_respawn_append, dim3(d.m), dim3(256), 0, st, d);
        if (int rc = rl::check_launch("respawn_append")) return rc;
    }
    e->counter += 1;
    e->pending = -1;        // the step's blocks wrote the counter (the applied value plus one)
    e->synced = d.ovr >= 0;
    if (e->cfg.obs_mode == RL_OBS_TILES) return RL_OK;
    return launch_obs(e, obs, st);
}

int rl_env_step(rl_env* e, const int32_t* actions, void* obs, float* rewards, float* dones, void* stream)
{
    return rl_env_step_aim(e, actions, nullptr, obs, rewards, dones, stream);
}

int rl_env_set_respawn_spots(rl_env* e, const int32_t* ckpt_spawns, void* stream)
{
    if (!e) return rl::fail(RL_EINVAL, "env is NULL");
    if (e->cfg.respawn_mode != RL_RESPAWN_ADAPTIVE) return rl::fail(RL_EINVAL, "the env does not use the adaptive respawn");
    if (!ckpt_spawns) return rl::fail(RL_EINVAL, "ckpt_spawns is NULL");
    if (!rl::aligned(ckpt_spawns, 4)) return rl::fail(RL_EALIGN, "ckpt_spawns is not 4-byte aligned");
    const hipError_t he = hipMemcpyAsync(e->base + e->lay.spots, ckpt_spawns,
                                         sizeof(int32_t) * 2 * (size_t)e->cfg.num_maps * e->cfg.num_ckpts,
                                         hipMemcpyDeviceToDevice, rl::as_stream(stream));
    if (he != hipSuccess) return rl::fail(RL_EHIP, "respawn spot copy: %s", hipGetErrorString(he));
    e->spots_set = true;
    return RL_OK;
}

int rl_env_read_respawn(const rl_env* e, int32_t* ring, int32_t* fill, int32_t* head, int32_t* frontier, void* stream)
{
    if (!e) return rl::fail(RL_EINVAL, "env is NULL");
    if (e->cfg.respawn_mode != RL_RESPAWN_ADAPTIVE) return rl::fail(RL_EINVAL, "the env does not use the adaptive respawn");
    if (!ring || !fill || !head || !frontier) return rl::fail(RL_EINVAL, "outputs must be non-NULL");
    const void* outs[] = {ring, fill, head, frontier};
    for (const void* q : outs)
        if (!rl::aligned(q, 4)) return rl::fail(RL_EALIGN, "an output is not 4-byte aligned");
    hipLaunchKernelGGL(k_read_respawn, dim3(e->cfg.num_maps), dim3(64), 0, rl::as_stream(stream), dev_of(e), ring, fill,
                       head, frontier);
    return rl::check_launch("read_respawn");
}

int rl_env_set_waypoints(rl_env* e, const int32_t* waypoints, const int32_t* lens, void* stream)
{
    if (!e) return rl::fail(RL_EINVAL, "env is NULL");
    if (e->cfg.reward_mode != RL_REWARD_WAYPOINTS) return rl::fail(RL_EINVAL, "the env does not use waypoint rewards");
    if (!waypoints || !lens) return rl::fail(RL_EINVAL, "waypoints and lens must be non-NULL");
    if (!rl::aligned(waypoints, 4) || !rl::aligned(lens, 4))
        return rl::fail(RL_EALIGN, "waypoints / lens are not 4-byte aligned");
    hipStream_t st = rl::as_stream(stream);
    const size_t m = (size_t)e->cfg.num_maps;
    hipError_t he = hipMemcpyAsync(e->base + e->lay.waypoints, waypoints,
                                   sizeof(int32_t) * 2 * (size_t)e->cfg.max_waypoints * m, hipMemcpyDeviceToDevice, st);
    if (he == hipSuccess)
        he = hipMemcpyAsync(e->base + e->lay.wplens, lens, sizeof(int32_t) * m, hipMemcpyDeviceToDevice, st);
    if (he != hipSuccess) return rl::fail(RL_EHIP, "waypoint copy: %s", hipGetErrorString(he));
    e->waypoints_set = true;
    return RL_OK;
}

int rl_waypoint_path(const uint8_t* map, int32_t h, int32_t w, int32_t c0, int32_t r0, int32_t c1, int32_t r1,
                     int32_t* path, int32_t max_len, int32_t* len)
{
    if (!map || !path || !len) return rl::fail(RL_EINVAL, "map, path and len must be non-NULL");
    if (h < 1 || w < 1 || (int64_t)h * w > ((int64_t)1 << 30)) return rl::fail(RL_EINVAL, "map size %d x %d", h, w);
    if (max_len < 1) return rl::fail(RL_EINVAL, "max_len %d < 1", max_len);
    const int64_t cells = (int64_t)h * w;
    auto open = [&](int64_t r, int64_t c) {
        if (r < 0 || r >= h || c < 0 || c >= w) return false;
        const uint8_t t = map[r * w + c];
        return t != kSolid && t != kPlatform;
    };
    if (!open(r0, c0) || !open(r1, c1)) return rl::fail(RL_EINVAL, "start or goal is blocked or outside the map");
    // from[i]: the tile that first reached tile i (row-major), -1 unvisited; the start points to itself
    std::vector<int32_t> from((size_t)cells, -1), frontier;
    frontier.reserve(1024);
    const int32_t start = r0 * w + c0, goal = r1 * w + c1;
    from[(size_t)start] = start;
    frontier.push_back(start);
    static const int step_c[4] = {1, 0, 0, -1}, step_r[4] = {0, -1, 1, 0};   // right, up, down, left
    for (size_t head = 0; head < frontier.size() && from[(size_t)goal] < 0; ++head) {
        const int32_t cur = frontier[head];
        const int32_t r = cur / w, c = cur - r * w;
        for (int k = 0; k < 4; ++k) {
            const int32_t nr = r + step_r[k], nc = c + step_c[k];
            if (!open(nr, nc)) continue;
            const int32_t nxt = nr * w + nc;
            if (from[(size_t)nxt] >= 0) continue;
            from[(size_t)nxt] = cur;
            frontier.push_back(nxt);
        }
    }
    if (from[(size_t)goal] < 0) return rl::fail(RL_EINVAL, "goal unreachable from start");
    int32_t n = 1;
    for (int32_t t = goal; t != start; t = from[(size_t)t]) ++n;
    if (n > max_len) return rl::fail(RL_ESIZE, "path needs %d tiles, max_len is %d", n, max_len);
    int32_t k = n - 1;
    for (int32_t t = goal;; t = from[(size_t)t], --k) {
        path[2 * k] = t % w;
        path[2 * k + 1] = t / w;
        if (t == start) break;
    }
    *len = n;
    return RL_OK;
}

int rl_env_read_state(const rl_env* e, int32_t* out, void* stream)
{
    if (!e || !out) return rl::fail(RL_EINVAL, "env and out must be non-NULL");
    if (!rl::aligned(out, 4)) return rl::fail(RL_EALIGN, "out is not 4-byte aligned");
    const EnvDev d = dev_of(e);
    hipLaunchKernelGGL(k_read_state, dim3((d.n + 255) / 256), dim3(256), 0, rl::as_stream(stream), d, out);
    return rl::check_launch("read_state");
}

int rl_env_get_config(const rl_env* e, rl_env_config* out)
{
    if (!e || !out) return rl::fail(RL_EINVAL, "env and out must be non-NULL");
    *out = e->cfg;
    return RL_OK;
}

int rl_env_get_step_counter(const rl_env* e, int64_t* counter)
{
    if (!e || !counter) return rl::fail(RL_EINVAL, "env and counter must be non-NULL");
    *counter = e->counter;
    return RL_OK;
}

int rl_env_set_step_counter(rl_env* e, int64_t counter)
{
    if (!e) return rl::fail(RL_EINVAL, "env is NULL");
    if (counter < 0) return rl::fail(RL_EINVAL, "counter %lld < 0", (long long)counter);
    e->counter = counter;
    e->pending = counter;
    return RL_OK;
}

int rl_env_read_step_counter(const rl_env* e, int64_t* out, void* stream)
{
    if (!e || !out) return rl::fail(RL_EINVAL, "env and out must be non-NULL");
    if (!rl::aligned(out, 8)) return rl::fail(RL_EALIGN, "out is not 8-byte aligned");
    hipLaunchKernelGGL(k_read_counter, dim3(1), dim3(1), 0, rl::as_stream(stream), dev_of(e), out);
    return rl::check_launch("read_step_counter");
}

void rl_env_destroy(rl_env* e) { delete e; }

}  // extern "C"
