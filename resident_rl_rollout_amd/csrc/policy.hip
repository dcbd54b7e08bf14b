// Stand-in policy inference, and the rollout driver that alternates it with the env step over one or
// more env groups.
//
// The inference is the work one decision needs from a policy of the shape of PufferLib 5.0's default
// ("Teaching Mario to speedrun", s.8): a bias-free linear encoder from the 1397-element tile observation
// to 128 numbers and one decoder matrix to the 12 action logits plus the value (s.6: one network gives
// the logits, sampled through a softmax, and the value). The recurrent layers between encoder and
// decoder are not part of the stand-in. The encoder reads its operands rounded to bfloat16 and sums in
// float32 on the matrix cores; the decoder and the sample are float32. The sample is the Gumbel-max form
// of softmax sampling: a = argmax_j (logit_j + g_j), g_j = -ln(-ln u_j), lowest j on a tie, with
// u_j = (2 (x_j >> 41) + 1) / 2^24 from the SplitMix64 output x_j = mix64(seed + golden (16 (t 2^24 + n)
// + j + 1)) for global env n and decision t.
//
// The driver enqueues, per decision and per group, the inference on the group's last observations and
// then the env step that consumes its actions. Groups on separate streams take turns at the inference
// ("PlayTrain", Figure 8C and Table 9: one env group steps while the other group's inference runs), so
// that one group's HBM-bound step runs beside the other group's matrix-core inference.

#include "rl_internal.hpp"

namespace {

constexpr int kObs = 1397;
constexpr int kK = 1408;                 // encoder row length in the packed weights: 88 k-steps of 16
constexpr int kHidden = 128;
constexpr int kActions = 12;
constexpr int kOut = kActions + 1;
constexpr int kKsUnroll = 4;             // k-steps of a chunk whose fragments are read ahead
constexpr int kKC = 128;                 // k elements per staged chunk
constexpr int kChunks = kK / kKC;        // 11
constexpr int kPitch = kKC + 8;          // LDS row pitch of a staged chunk, bfloat16 elements (272 bytes)
constexpr int kHPitch = kHidden + 4;     // LDS row pitch of the hidden activations, floats
constexpr size_t kEncBytes = sizeof(uint16_t) * kHidden * kK;   // 360,448
constexpr size_t kDecBytes = sizeof(float) * kOut * kHidden;    // 6,656
// LDS of a block of `rows` envs: the staged chunks, reused by the epilogue's hidden values and decoder.
constexpr int lds_bytes(int rows)
{
    return (rows + kHidden) * kPitch * 2 > (rows * kHPitch + kOut * kHidden) * 4 ? (rows + kHidden) * kPitch * 2
                                                                                : (rows * kHPitch + kOut * kHidden) * 4;
}
constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

static_assert(kK % kKC == 0 && kK >= kObs, "chunks cover the padded encoder rows");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// float32 -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_bits(float x)
{
    const uint32_t b = __float_as_uint(x);
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// SplitMix64's output function (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
// 2014).
__device__ __forceinline__ uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// Packed weights: the encoder as bfloat16 [128][1408] (zeros past 1397), then the decoder float32 [13][128].
__global__ __launch_bounds__(256) void k_policy_pack(const float* __restrict__ enc, const float* __restrict__ dec,
                                                     uint16_t* __restrict__ penc, float* __restrict__ pdec)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < kHidden * kK) {
        const int h = i / kK, k = i % kK;
        penc[i] = k < kObs ? (uint16_t)bf16_bits(enc[h * kObs + k]) : (uint16_t)0;
    } else if (i < kHidden * kK + kOut * kHidden) {
        pdec[i - kHidden * kK] = dec[i - kHidden * kK];
    }
}

struct PolicyArgs {
    const uint16_t* enc;   // [128][1408] bfloat16 bits
    const float* dec;      // [13][128]
    const float* obs;      // [n][stride]
    int64_t n, stride;
    uint64_t seed;
    int64_t t, env_offset;
    int32_t* actions;
    float* logp;
    float* values;
};

// One block of 4 ROWS threads (a wave per 16 envs) handles ROWS envs. The encoder product
// [ROWS x 1408] x [1408 x 128] runs on v_mfma_f32_32x32x16_bf16: wave w owns rows 32 (w >> 1) .. +32 and
// columns 64 (w & 1) .. +64 (two 32 x 32 tiles). The observation and weight chunks of 128 k are staged in
// LDS as bfloat16; the next chunk's loads are in flight while the current one multiplies. The epilogue
// parks the ROWS x 128 hidden values in LDS, applies the decoder (four threads per env, each a contiguous
// quarter of the hidden units in order, combined by two exchanges) and draws the action.
// Measured at 65536 envs with 128 rows: 87-94 us. Without the observation loads the kernel still takes
// 63 us and without the weight loads 88 us: it is bound by the latency of its chunk pipeline (one chunk
// of loads in flight per block, two barriers per chunk), not by HBM; 64-k chunks (twice the steps) run
// slower.
template <int ROWS>
__global__ __launch_bounds__(ROWS * 4) void k_policy_forward(PolicyArgs p)
{
    constexpr int kRows = ROWS, kThreads = ROWS * 4;
    static_assert(kRows % 32 == 0 && (kHidden * kKC / 8) % kThreads == 0, "tiles and weight segments divide");
    __shared__ __align__(16) uint8_t lds[lds_bytes(ROWS)];
    uint16_t* As = reinterpret_cast<uint16_t*>(lds);   // [64][kPitch]
    uint16_t* Bs = As + kRows * kPitch;                 // [128][kPitch]
    const int t = threadIdx.x, l = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);   // wave-uniform: row addresses stay scalar
    const int64_t e0 = (int64_t)blockIdx.x * kRows;
    const int rh = w >> 1, ch = w & 1;

    float ra[16][2];   // observation rows 16 w + i, elements k0 + 2 l and k0 + 2 l + 1
    constexpr int kSeg = kHidden * kKC / 8 / kThreads;   // 16-byte weight segments per thread and chunk
    u32x4 rb[kSeg];    // segments t + kThreads i of the weight chunk (column s >> 4, segment s & 15)
    // the wave's 16 rows (clamped to the last env) start at row0 + i * stride, i <= last
    const float* row0 = p.obs + min(e0 + w * 16, p.n - 1) * p.stride;
    const int last = (int)min<int64_t>(15, p.n - 1 - min(e0 + w * 16, p.n - 1));

    auto load_chunk = [&](int c) __attribute__((always_inline)) {
        const int k0 = c * kKC;
        const int k = k0 + 2 * l;
        if (k0 + kKC <= kObs) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float* r = row0 + (int64_t)min(i, last) * p.stride;
                ra[i][0] = r[k];
                ra[i][1] = r[k + 1];
            }
        } else {   // the last chunk: elements past the observation are zero
            const int ka = min(k, kObs - 1), kb = min(k + 1, kObs - 1);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float* r = row0 + (int64_t)min(i, last) * p.stride;
                const float a = r[ka], b = r[kb];
                ra[i][0] = k < kObs ? a : 0.0f;
                ra[i][1] = k + 1 < kObs ? b : 0.0f;
            }
        }
#pragma unroll
        for (int i = 0; i < kSeg; ++i) {
            const int s = i * kThreads + t;
            rb[i] = *reinterpret_cast<const u32x4*>(p.enc + (size_t)(s >> 4) * kK + k0 + (s & 15) * 8);
        }
    };
    auto store_chunk = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            *reinterpret_cast<uint32_t*>(As + (w * 16 + i) * kPitch + 2 * l) =
                bf16_bits(ra[i][0]) | (bf16_bits(ra[i][1]) << 16);
#pragma unroll
        for (int i = 0; i < kSeg; ++i) {
            const int s = i * kThreads + t;
            *reinterpret_cast<u32x4*>(Bs + (s >> 4) * kPitch + (s & 15) * 8) = rb[i];
        }
    };

    f32x16 acc0 = {}, acc1 = {};
    load_chunk(0);
    for (int c = 0; c < kChunks; ++c) {
        __syncthreads();   // the previous chunk's fragments have been read
        store_chunk();
        if (c + 1 < kChunks) load_chunk(c + 1);   // the registers are free: in flight across the barrier
        __syncthreads();
        // A fragment: row 32 rh + (l & 31), k 8 (l >> 5) .. +7 of each 16-step; B: column (l & 31) of
        // each tile, the same k
        const uint16_t* pa = As + (rh * 32 + (l & 31)) * kPitch + 8 * (l >> 5);
        const uint16_t* pb0 = Bs + (ch * 64 + (l & 31)) * kPitch + 8 * (l >> 5);
        const uint16_t* pb1 = pb0 + 32 * kPitch;
#pragma unroll kKsUnroll
        for (int ks = 0; ks < kKC / 16; ++ks) {
            const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(pa + ks * 16));
            const bf16x8 b0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(pb0 + ks * 16));
            const bf16x8 b1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(pb1 + ks * 16));
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, acc1, 0, 0, 0);
        }
    }

    __syncthreads();   // every wave is done with the staged chunks
    float* Hs = reinterpret_cast<float*>(lds);   // [64][kHPitch]
    float* Ds = Hs + kRows * kHPitch;            // [13][128]
    // accumulator r of a 32 x 32 tile: row 8 (r >> 2) + 4 (l >> 5) + (r & 3), column l & 31
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = rh * 32 + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
        Hs[row * kHPitch + ch * 64 + (l & 31)] = acc0[r];
        Hs[row * kHPitch + ch * 64 + 32 + (l & 31)] = acc1[r];
    }
    for (int i = t; i < kOut * kHidden; i += kThreads) Ds[i] = p.dec[i];
    __syncthreads();

    // thread (e, q) sums hidden units 32 q .. 32 q + 31 of env e in order, four at a time (16-byte LDS reads)
    const int e = t >> 2, q = t & 3;
    float o[kOut];
#pragma unroll
    for (int j = 0; j < kOut; ++j) o[j] = 0.0f;
    const float4* hx = reinterpret_cast<const float4*>(Hs + e * kHPitch + 32 * q);
#pragma unroll 2
    for (int i = 0; i < 8; ++i) {
        const float4 x = hx[i];
#pragma unroll
        for (int j = 0; j < kOut; ++j) {
            const float4 wj = reinterpret_cast<const float4*>(Ds + j * kHidden + 32 * q)[i];
            o[j] = fmaf(x.x, wj.x, o[j]);
            o[j] = fmaf(x.y, wj.y, o[j]);
            o[j] = fmaf(x.z, wj.z, o[j]);
            o[j] = fmaf(x.w, wj.w, o[j]);
        }
    }
    // the four quarters: (p0 + p1) + (p2 + p3), the same bits in all four lanes
#pragma unroll
    for (int j = 0; j < kOut; ++j) {
        o[j] += __shfl_xor(o[j], 1, 64);
        o[j] += __shfl_xor(o[j], 2, 64);
    }

    // Gumbel-max: lane q draws logits q, q + 4, q + 8; the best score, lowest logit on a tie
    const int64_t row = e0 + e;
    const uint64_t key = (uint64_t)p.t * (1ull << 24) + (uint64_t)(p.env_offset + row);
    float best = 0.0f;
    int bj = 0;
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        const int j = q + 4 * m;
        const uint64_t x = mix64(p.seed + kGolden * (16 * key + (uint64_t)j + 1));
        const uint32_t kk = (uint32_t)(x >> 41);
        // -ln u = -log1p(-(1 - u)), 1 - u = (2^24 - 1 - 2 kk) / 2^24 exactly
        const float nlu = -log1pf(-(float)(16777215u - 2u * kk) * 0x1p-24f);
        const float g = -logf(nlu);
        float oj = o[0];
#pragma unroll
        for (int jj = 1; jj < kActions; ++jj) oj = jj == j ? o[jj] : oj;
        const float s = oj + g;
        if (m == 0 || s > best) {
            best = s;
            bj = j;
        }
    }
#pragma unroll
    for (int off = 1; off <= 2; off <<= 1) {
        const float ob = __shfl_xor(best, off, 64);
        const int oj = __shfl_xor(bj, off, 64);
        if (ob > best || (ob == best && oj < bj)) {
            best = ob;
            bj = oj;
        }
    }
    if (q == 0 && row < p.n) {
        float mx = o[0], oa = o[0];
#pragma unroll
        for (int j = 1; j < kActions; ++j) {
            mx = fmaxf(mx, o[j]);
            oa = j == bj ? o[j] : oa;
        }
        float z = 0.0f;
#pragma unroll
        for (int j = 0; j < kActions; ++j) z += expf(o[j] - mx);
        p.actions[row] = bj;
        p.logp[row] = oa - (mx + logf(z));
        p.values[row] = o[kActions];
    }
}

int check_packed(const void* packed)
{
    if (!packed) return rl::fail(RL_EINVAL, "packed policy weights are NULL");
    if (!rl::aligned(packed, 256)) return rl::fail(RL_EALIGN, "packed policy weights are not 256-byte aligned");
    return RL_OK;
}

}  // namespace

extern "C" {

int rl_policy_weights_bytes(size_t* bytes)
{
    if (!bytes) return rl::fail(RL_EINVAL, "bytes is NULL");
    *bytes = kEncBytes + kDecBytes;
    return RL_OK;
}

int rl_policy_pack(const float* enc_w, const float* dec_w, void* packed, void* stream)
{
    if (!enc_w || !dec_w) return rl::fail(RL_EINVAL, "enc_w and dec_w must be non-NULL");
    if (!rl::aligned(enc_w, 4) || !rl::aligned(dec_w, 4)) return rl::fail(RL_EALIGN, "weights are not 4-byte aligned");
    if (int rc = check_packed(packed)) return rc;
    uint16_t* penc = static_cast<uint16_t*>(packed);
    float* pdec = reinterpret_cast<float*>(static_cast<uint8_t*>(packed) + kEncBytes);
    const int total = kHidden * kK + kOut * kHidden;
    hipLaunchKernelGGL(k_policy_pack, dim3((total + 255) / 256), dim3(256), 0, rl::as_stream(stream), enc_w, dec_w,
                       penc, pdec);
    return rl::check_launch("policy_pack");
}

int rl_policy_forward(const void* packed, const float* obs, int64_t n, int64_t obs_stride, uint64_t seed, int64_t t,
                      int64_t env_offset, int32_t* actions, float* logp, float* values, void* stream)
{
    if (int rc = check_packed(packed)) return rc;
    if (n < 0 || env_offset < 0 || env_offset + n > ((int64_t)1 << 24))
        return rl::fail(RL_EINVAL, "envs [%lld, %lld) outside [0, 2^24)", (long long)env_offset,
                        (long long)(env_offset + n));
    if (t < 0) return rl::fail(RL_EINVAL, "decision %lld < 0", (long long)t);
    if (obs_stride < kObs) return rl::fail(RL_EINVAL, "obs_stride %lld < %d", (long long)obs_stride, kObs);
    if (n == 0) return RL_OK;
    if (!obs || !actions || !logp || !values)
        return rl::fail(RL_EINVAL, "obs, actions, logp and values must be non-NULL");
    if (!rl::aligned(obs, 4) || !rl::aligned(actions, 4) || !rl::aligned(logp, 4) || !rl::aligned(values, 4))
        return rl::fail(RL_EALIGN, "obs / actions / logp / values are not 4-byte aligned");
    PolicyArgs p;
    p.enc = static_cast<const uint16_t*>(packed);
    p.dec = reinterpret_cast<const float*>(static_cast<const uint8_t*>(packed) + kEncBytes);
    p.obs = obs;
    p.n = n;
    p.stride = obs_stride;
    p.seed = seed;
    p.t = t;
    p.env_offset = env_offset;
    p.actions = actions;
    p.logp = logp;
    p.values = values;
    // 128 envs per block halves the weight re-reads, 64 keeps two blocks per CU in smaller launches (a
    // double-buffered group): 87 against 93 us at 65536 envs, and the 32768-env groups of a double-buffered
    // rollout overlap better with 512 blocks than with 256
    if (n >= 65536)
        hipLaunchKernelGGL(k_policy_forward<128>, dim3((unsigned)((n + 127) / 128)), dim3(512), 0, rl::as_stream(stream), p);
    else
        hipLaunchKernelGGL(k_policy_forward<64>, dim3((unsigned)((n + 63) / 64)), dim3(256), 0, rl::as_stream(stream), p);
    return rl::check_launch("policy_forward");
}

int rl_rollout(const void* packed, uint64_t seed, const rl_rollout_group* groups, int32_t num_groups, int32_t t0,
               int32_t steps, int32_t alternate)
{
    if (int rc = check_packed(packed)) return rc;
    if (!groups || num_groups < 1 || num_groups > RL_ROLLOUT_MAX_GROUPS)
        return rl::fail(RL_EINVAL, "num_groups %d outside [1, %d]", num_groups, RL_ROLLOUT_MAX_GROUPS);
    if (t0 < 0 || steps < 0) return rl::fail(RL_EINVAL, "t0 %d and steps %d must be >= 0", t0, steps);
    rl_env_config cfg[RL_ROLLOUT_MAX_GROUPS];
    int64_t counter0 = 0;
    for (int g = 0; g < num_groups; ++g) {
        const rl_rollout_group& x = groups[g];
        if (int rc = rl_env_get_config(x.env, &cfg[g])) return rc;
        if (cfg[g].obs_mode != RL_OBS_TILES) return rl::fail(RL_EINVAL, "group %d: the inference reads tile observations", g);
        if (cfg[g].hook_mode != RL_HOOK_OFF)
            return rl::fail(RL_EINVAL, "group %d: the stand-in inference gives no aims for the grapple hook", g);
        const int64_t n = cfg[g].num_envs;
        if (!x.actions || !x.logp || !x.values || !x.obs || !x.rewards || !x.dones || (t0 == 0 && !x.obs0))
            return rl::fail(RL_EINVAL, "group %d: a buffer is NULL", g);
        const void* ptrs[] = {x.obs0, x.obs, x.actions, x.logp, x.values, x.rewards, x.dones};
        for (const void* q : ptrs)
            if (q && !rl::aligned(q, 4)) return rl::fail(RL_EALIGN, "group %d: a buffer is not 4-byte aligned", g);
        if (x.row < n || x.obs_row < n * cfg[g].obs_stride)
            return rl::fail(RL_EINVAL, "group %d: row %lld / obs_row %lld shorter than one decision's data", g,
                            (long long)x.row, (long long)x.obs_row);
        if (x.env_offset < 0 || x.env_offset + n > ((int64_t)1 << 24))
            return rl::fail(RL_EINVAL, "group %d: envs outside [0, 2^24)", g);
        // a group's env n plays map n mod M of its own batch; it is global env env_offset + n only when the
        // offset is a multiple of M
        if (x.env_offset % cfg[g].num_maps != 0)
            return rl::fail(RL_EINVAL, "group %d: env_offset %lld is not a multiple of num_maps %d", g,
                            (long long)x.env_offset, cfg[g].num_maps);
        // the adaptive respawn keeps its outcome buffers and draw keys per env batch: split into groups (or
        // offset), its restarts would differ from one batch's
        if (cfg[g].respawn_mode != RL_RESPAWN_OFF && (num_groups > 1 || x.env_offset != 0))
            return rl::fail(RL_EINVAL, "group %d: the adaptive respawn needs a single group at env_offset 0", g);
        int64_t c = 0;
        rl_env_get_step_counter(x.env, &c);
        if (g == 0) counter0 = c;
        else if (c != counter0) return rl::fail(RL_EINVAL, "group %d: decision counter %lld differs from group 0's %lld",
                                                g, (long long)c, (long long)counter0);
    }
    // turn tokens: group g's inference at decision t waits for group g - 1's at t (group 0's for t + 1
    // waits for the last group's at t)
    hipEvent_t ev[RL_ROLLOUT_MAX_GROUPS] = {};
    const bool turns = alternate && num_groups > 1;
    int rc = RL_OK;
    if (turns)
        for (int g = 0; g < num_groups && rc == RL_OK; ++g)
            if (hipEventCreateWithFlags(&ev[g], hipEventDisableTiming) != hipSuccess)
                rc = rl::fail(RL_EHIP, "hipEventCreateWithFlags failed");
    for (int s = 0; s < steps && rc == RL_OK; ++s) {
        const int64_t t = (int64_t)t0 + s;
        for (int g = 0; g < num_groups && rc == RL_OK; ++g) {
            const rl_rollout_group& x = groups[g];
            hipStream_t st = rl::as_stream(x.stream);
            const int64_t n = cfg[g].num_envs, os = cfg[g].obs_stride;
            const float* in = t == 0 ? x.obs0 : x.obs + (t - 1) * x.obs_row;
            if (turns && (g > 0 || s > 0) && hipStreamWaitEvent(st, ev[(g + num_groups - 1) % num_groups], 0) != hipSuccess) {
                rc = rl::fail(RL_EHIP, "hipStreamWaitEvent failed");
                break;
            }
            rc = rl_policy_forward(packed, in, n, os, seed, counter0 + s, x.env_offset, x.actions + t * x.row,
                                   x.logp + t * x.row, x.values + t * x.row, x.stream);
            if (rc) break;
            if (turns && hipEventRecord(ev[g], st) != hipSuccess) {
                rc = rl::fail(RL_EHIP, "hipEventRecord failed");
                break;
            }
            rc = rl_env_step(x.env, x.actions + t * x.row, x.obs + t * x.obs_row, x.rewards + t * x.row,
                             x.dones + t * x.row, x.stream);
        }
    }
    for (int g = 0; g < num_groups; ++g)
        if (ev[g]) (void)hipEventDestroy(ev[g]);
    return rc;
}

}  // extern "C"
