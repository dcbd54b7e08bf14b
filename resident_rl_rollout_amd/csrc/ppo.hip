// PPO loss forward reductions per minibatch ("Teaching Mario to speedrun", s.6 Don't move too far at once):
// for every sample of minibatch m, the log-softmax of its logits, the probability ratio against the
// recorded old log-probability, the clipped surrogate, the squared value error and the policy entropy;
// their minibatch means and the weighted total.
//
// Grid: (blocks per minibatch, minibatches). Each thread accumulates its samples in float64; a block
// reduction (shuffles, then LDS) gives per-block partials, and a finalise kernel with one block per
// minibatch reduces them in block order and writes the four scalars. No floating-point atomics, so
// results are identical from run to run.

#include <algorithm>

#include "rl_internal.hpp"

namespace {

constexpr double kNormEps = 1e-8;
constexpr int kSamplesPerThread = 8;
constexpr int kMaxBlocksPerMb = 4096;

struct LossArgs {
    const float* logits;
    const int32_t* actions;
    const float* old_logp;
    const float* adv;
    const float* ret;
    const float* new_v;
    const int32_t* perm;
    const double* stats;
    int64_t mb;
    int A;
    float clip_lo, clip_hi, vf, ent;
    double* partials;   // [num_mb][bpm][3]
};

__device__ __forceinline__ double block_sum(double v, double* lds)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = v;
    __syncthreads();
    double s = 0.0;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) s += lds[i];
    return s;
}

// Logits row statistics for AC (compile-time action count; 0 = runtime A, read element by element):
// returns log(sum exp(z - max)) in *log_s, (sum e_j (z_j - max)) / S in *mean_u, and z_a - max in *u_a.
template <int AC>
__device__ __forceinline__ void row_stats(const float* __restrict__ row, int A, int a, float* log_s, float* mean_u,
                                          float* u_a)
{
    if constexpr (AC > 0) {
        float z[AC];
        if constexpr (AC % 4 == 0) {
#pragma unroll
            for (int j = 0; j < AC / 4; ++j) {
                const float4 q = reinterpret_cast<const float4*>(row)[j];
                z[4 * j] = q.x;
                z[4 * j + 1] = q.y;
                z[4 * j + 2] = q.z;
                z[4 * j + 3] = q.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < AC; ++j) z[j] = row[j];
        }
        float mx = z[0];
#pragma unroll
        for (int j = 1; j < AC; ++j) mx = fmaxf(mx, z[j]);
        float s = 0.0f, su = 0.0f, ua = z[0] - mx;
#pragma unroll
        for (int j = 0; j < AC; ++j) {
            const float u = z[j] - mx;
            const float ex = expf(u);
            s += ex;
            su += ex * u;
            if (j == a) ua = u;
        }
        *log_s = logf(s);
        *mean_u = su / s;
        *u_a = ua;
    } else {
        float mx = row[0];
        for (int j = 1; j < A; ++j) mx = fmaxf(mx, row[j]);
        float s = 0.0f, su = 0.0f, ua = row[0] - mx;
        for (int j = 0; j < A; ++j) {
            const float u = row[j] - mx;
            const float ex = expf(u);
            s += ex;
            su += ex * u;
            if (j == a) ua = u;
        }
        *log_s = logf(s);
        *mean_u = su / s;
        *u_a = ua;
    }
}

template <int AC>
__global__ __launch_bounds__(256) void k_ppo_loss(LossArgs p)
{
    __shared__ double lds[12];
    const int m = blockIdx.y;
    const int64_t base = (int64_t)m * p.mb;
    float mean = 0.0f, scale = 1.0f;
    if (p.stats) {
        mean = (float)p.stats[1];
        scale = (float)(1.0 / (p.stats[2] + kNormEps));
    }
    double s_pg = 0.0, s_v = 0.0, s_h = 0.0;
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < p.mb; k += step) {
        const int64_t i = p.perm ? (int64_t)p.perm[base + k] : base + k;
        const int a = p.actions[i];
        float log_s, mean_u, u_a;
        row_stats<AC>(p.logits + i * (AC > 0 ? AC : p.A), p.A, a, &log_s, &mean_u, &u_a);
        const float logp = u_a - log_s;
        const float entropy = log_s - mean_u;
        const float ratio = expf(logp - p.old_logp[i]);
        float adv = p.adv[i];
        if (p.stats) adv = (adv - mean) * scale;
        const float clipped = fminf(fmaxf(ratio, p.clip_lo), p.clip_hi);
        const float pg = -fminf(ratio * adv, clipped * adv);
        const float dv = p.new_v[i] - p.ret[i];
        s_pg += (double)pg;
        s_v += (double)(dv * dv);
        s_h += (double)entropy;
    }
    s_pg = block_sum(s_pg, lds);
    s_v = block_sum(s_v, lds + 4);
    s_h = block_sum(s_h, lds + 8);
    if (threadIdx.x == 0) {
        double* part = p.partials + ((int64_t)m * gridDim.x + blockIdx.x) * 3;
        part[0] = s_pg;
        part[1] = s_v;
        part[2] = s_h;
    }
}

// One block per minibatch: reduce its per-block partials in block order and write the four scalars.
__global__ __launch_bounds__(256) void k_ppo_finalize(const double* __restrict__ partials, int bpm, int64_t mb,
                                                      float vf, float ent, float* __restrict__ out)
{
    __shared__ double lds[12];
    const int m = blockIdx.x;
    double a = 0.0, b = 0.0, c = 0.0;
    for (int j = threadIdx.x; j < bpm; j += blockDim.x) {
        const double* part = partials + ((int64_t)m * bpm + j) * 3;
        a += part[0];
        b += part[1];
        c += part[2];
    }
    a = block_sum(a, lds);
    b = block_sum(b, lds + 4);
    c = block_sum(c, lds + 8);
    if (threadIdx.x == 0) {
        const double inv = 1.0 / (double)mb;
        const double pg = a * inv, v = b * inv, h = c * inv;
        out[4 * m + 0] = (float)pg;
        out[4 * m + 1] = (float)v;
        out[4 * m + 2] = (float)h;
        out[4 * m + 3] = (float)(pg + (double)vf * v - (double)ent * h);
    }
}

int blocks_per_mb(int64_t mb)
{
    const int64_t per_block = 256 * kSamplesPerThread;
    return (int)std::max<int64_t>(1, std::min<int64_t>((mb + per_block - 1) / per_block, kMaxBlocksPerMb));
}

}  // namespace

extern "C" {

int rl_ppo_loss_workspace_bytes(int64_t B, int32_t mb, size_t* bytes)
{
    if (B < 1 || mb < 1) return rl::fail(RL_EINVAL, "B %lld and mb %d must be >= 1", (long long)B, mb);
    if (B % mb != 0) return rl::fail(RL_EINVAL, "B %lld is not a multiple of mb %d", (long long)B, mb);
    if (!bytes) return rl::fail(RL_EINVAL, "bytes is NULL");
    const int64_t num_mb = B / mb;
    *bytes = sizeof(double) * 3 * (size_t)num_mb * (size_t)blocks_per_mb(mb);
    return RL_OK;
}

int rl_ppo_loss(const float* logits, const int32_t* actions, const float* old_logp, const float* adv, const float* ret,
                const float* new_values, const int32_t* perm, const double* adv_stats, int64_t B, int32_t A,
                int32_t mb, float clip_eps, float vf_coef, float ent_coef, float* out, void* ws, size_t ws_bytes,
                void* stream)
{
    size_t need = 0;
    if (int rc = rl_ppo_loss_workspace_bytes(B, mb, &need)) return rc;
    if (A < 1 || A > 64) return rl::fail(RL_EINVAL, "A %d outside [1, 64]", A);
    if (B * (int64_t)A > ((int64_t)1 << 40)) return rl::fail(RL_EINVAL, "B*A too large");
    if (!logits || !actions || !old_logp || !adv || !ret || !new_values || !out || !ws)
        return rl::fail(RL_EINVAL, "logits, actions, old_logp, adv, ret, new_values, out and ws must be non-NULL");
    if (!(clip_eps >= 0.0f)) return rl::fail(RL_EINVAL, "clip_eps must be >= 0");
    const void* ptrs[] = {logits, actions, old_logp, adv, ret, new_values, out};
    for (const void* q : ptrs)
        if (!rl::aligned(q, 4)) return rl::fail(RL_EALIGN, "an array is not 4-byte aligned");
    if (perm && !rl::aligned(perm, 4)) return rl::fail(RL_EALIGN, "perm is not 4-byte aligned");
    if (A % 4 == 0 && !rl::aligned(logits, 16)) return rl::fail(RL_EALIGN, "logits must be 16-byte aligned when A %% 4 == 0");
    if (!rl::aligned(ws, 8) || (adv_stats && !rl::aligned(adv_stats, 8)))
        return rl::fail(RL_EALIGN, "ws / adv_stats not 8-byte aligned");
    if (ws_bytes < need) return rl::fail(RL_ESIZE, "workspace has %zu bytes, needs %zu", ws_bytes, need);

    const int64_t num_mb = B / mb;
    if (num_mb > 65535) return rl::fail(RL_EINVAL, "%lld minibatches exceed 65535", (long long)num_mb);
    LossArgs p;
    p.logits = logits;
    p.actions = actions;
    p.old_logp = old_logp;
    p.adv = adv;
    p.ret = ret;
    p.new_v = new_values;
    p.perm = perm;
    p.stats = adv_stats;
    p.mb = mb;
    p.A = A;
    p.clip_lo = 1.0f - clip_eps;
    p.clip_hi = 1.0f + clip_eps;
    p.vf = vf_coef;
    p.ent = ent_coef;
    p.partials = static_cast<double*>(ws);
    const dim3 grid(blocks_per_mb(mb), (unsigned)num_mb), block(256);
    hipStream_t st = rl::as_stream(stream);
    if (A == 12)
        hipLaunchKernelGGL(k_ppo_loss<12>, grid, block, 0, st, p);
    else
        hipLaunchKernelGGL(k_ppo_loss<0>, grid, block, 0, st, p);
    if (int rc = rl::check_launch("ppo_loss")) return rc;
    hipLaunchKernelGGL(k_ppo_finalize, dim3((unsigned)num_mb), block, 0, st, static_cast<const double*>(ws),
                       (int)grid.x, (int64_t)mb, vf_coef, ent_coef, out);
    return rl::check_launch("ppo_finalize");
}

}  // extern "C"
