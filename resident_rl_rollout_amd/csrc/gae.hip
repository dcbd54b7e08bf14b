// GAE reverse scan over a [T][N] rollout, whole-batch advantage statistics and normalisation.
//
// The recurrence ("Teaching Mario to speedrun", s.6 Better advantages; the done mask cuts an episode
// where it ended):
//   delta_t = r_t + gamma * V_{t+1} * (1 - d_t) - V_t,   A_t = delta_t + c_t * A_{t+1},
//   c_t = gamma * lambda * (1 - d_t),  A_T = 0,  R_t = A_t + V_t.
// It is a first-order linear recurrence, so a run of steps composes into one affine map
// A_in = b + c * A_out. The chunked kernel splits T into C chunks per env: each thread loads its chunk
// once into registers, reduces it to (b, c), the C maps are composed through LDS to give every chunk its
// incoming A, and each thread then replays its chunk from registers. Every input is read once and every
// output written once (20 bytes per element), with C times the lane parallelism of one lane per env;
// each row [t][n0 .. n0+E) is a coalesced segment.
//
// Statistics: per-thread float64 sums of A and A^2, a block reduction, per-block partials in the
// workspace, then a one-wave finalise kernel reduces the partials in block order (the kernel boundary
// makes every block's partial visible; no device-wide fence or atomic per block). No floating-point
// atomics: results are identical from run to run. With deferred statistics (normalize = 3) the partials go
// to the caller's adv_stats instead and no finalise runs: the loss kernels reduce them, with the same
// function and so the same bits, when they read the statistics.

#include <algorithm>

#include "rl_internal.hpp"

namespace {

constexpr double kNormEps = 1e-8;

struct StatsOut {
    double* partials;     // [grid][2]: sum A, sum A^2 of each block
    double* header;       // deferred statistics: {-(grid), count} written by block 0; NULL otherwise
    double count;
};

// Sums of two doubles across the block at once, each in the same fixed order on every run (a wave's
// butterfly, then the waves in order), with one barrier. The LDS array must not have been used earlier in
// the kernel.
__device__ __forceinline__ void block_sum2(double& a, double& b, double* lds)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        a += __shfl_xor(a, off, 64);
        b += __shfl_xor(b, off, 64);
    }
    const int w = threadIdx.x >> 6, nw = (int)(blockDim.x >> 6);
    if ((threadIdx.x & 63) == 0) {
        lds[w] = a;
        lds[16 + w] = b;
    }
    __syncthreads();
    a = 0.0;
    b = 0.0;
    for (int i = 0; i < nw; ++i) {
        a += lds[i];
        b += lds[16 + i];
    }
}

// Publish this block's (sum A, sum A^2).
__device__ void publish_stats(double s1, double s2, const StatsOut& so)
{
    __shared__ double lds[32];
    block_sum2(s1, s2, lds);
    if (threadIdx.x == 0) {
        so.partials[2 * blockIdx.x] = s1;
        so.partials[2 * blockIdx.x + 1] = s2;
        if (so.header && blockIdx.x == 0) {
            so.header[0] = -(double)gridDim.x;
            so.header[1] = so.count;
        }
    }
}

// One wave: reduce the per-block partials in block order into {count, mean, population std}.
__global__ __launch_bounds__(64) void k_stats_finalize(const double* __restrict__ partials, int blocks, double count,
                                                       double* __restrict__ stats)
{
    double mean, stdev;
    rl::stats_from_partials(partials, blocks, count, mean, stdev);
    if (threadIdx.x == 0) {
        stats[0] = count;
        stats[1] = mean;
        stats[2] = stdev;
    }
}

// The finished statistics of an adv_stats buffer in either form (finished, or deferred partials).
__global__ __launch_bounds__(64) void k_stats_finish(const double* __restrict__ in, double* __restrict__ out)
{
    const double h = in[0];
    if (h >= 0.0) {
        if (threadIdx.x < 3) out[threadIdx.x] = in[threadIdx.x];
        return;
    }
    double mean, stdev;
    rl::stats_from_partials(in + rl::kDeferredHead, (int)(-h), in[1], mean, stdev);
    if (threadIdx.x == 0) {
        out[0] = in[1];
        out[1] = mean;
        out[2] = stdev;
    }
}

// Block = E envs x (BLOCK / E) chunks of L <= LMAX steps. Thread (e, ch) owns env blockIdx.x*E + e and
// steps [ch*L, min(T, ch*L + L)).
template <int E, int LMAX, int BLOCK>
__global__ __launch_bounds__(BLOCK) void k_gae_chunked(const float* __restrict__ rew, const float* __restrict__ val,
                                                     const float* __restrict__ done, const float* __restrict__ vlast,
                                                     int T, int N, int64_t ld, int L, float gamma, float gl,
                                                     float* __restrict__ adv, float* __restrict__ ret,
                                                     int want_stats, StatsOut so)
{
    constexpr int C = BLOCK / E;
    __shared__ float sb[C][E];
    __shared__ float sc[C][E];
    const int e = threadIdx.x % E;
    const int ch = threadIdx.x / E;
    const int n = blockIdx.x * E + e;
    const bool valid = n < N;
    const int t0 = ch * L;
    const int len = valid ? max(0, min(L, T - t0)) : 0;

    // Loads are unconditional (indices clamped into the arrays) so that all of a thread's loads issue
    // back to back; only the arithmetic and the stores are predicated on the chunk's length. Each input
    // element is read once, so the loads carry the non-temporal hint (they need not displace cached
    // lines).
    const int nn = min(n, N - 1);
    float delta[LMAX], cf[LMAX], vv[LMAX];
#pragma unroll
    for (int j = 0; j < LMAX; ++j) {
        const int64_t idx = (int64_t)min(t0 + j, T - 1) * ld + nn;
        vv[j] = __builtin_nontemporal_load(val + idx);
        delta[j] = __builtin_nontemporal_load(rew + idx);
        cf[j] = 1.0f - __builtin_nontemporal_load(done + idx);
    }
    const float v_after = val[(int64_t)min(t0 + len, T - 1) * ld + nn];
    const float vnext_tail = (t0 + len < T) ? v_after : vlast[nn];

    float b = 0.0f, c = 1.0f;
#pragma unroll
    for (int j = LMAX - 1; j >= 0; --j) {
        if (j < len) {
            const float vn = (j + 1 < len) ? vv[j + 1 < LMAX ? j + 1 : j] : vnext_tail;
            const float notdone = cf[j];
            delta[j] = delta[j] + gamma * vn * notdone - vv[j];
            cf[j] = gl * notdone;
            b = delta[j] + cf[j] * b;
            c = cf[j] * c;
        }
    }
    sb[ch][e] = b;
    sc[ch][e] = c;
    __syncthreads();

    float a = 0.0f;
    for (int k = C - 1; k > ch; --k) a = sb[k][e] + sc[k][e] * a;

    double s1 = 0.0, s2 = 0.0;
#pragma unroll
    for (int j = LMAX - 1; j >= 0; --j) {
        if (j < len) {
            a = delta[j] + cf[j] * a;
            const int64_t idx = (int64_t)(t0 + j) * ld + n;
            adv[idx] = a;
            ret[idx] = a + vv[j];
            s1 += (double)a;
            s2 += (double)a * (double)a;
        }
    }
    if (want_stats) publish_stats(s1, s2, so);
}

// One lane per env walking t = T-1 .. 0: the fallback for horizons longer than the chunked kernels hold.
__global__ __launch_bounds__(256) void k_gae_seq(const float* __restrict__ rew, const float* __restrict__ val,
                                                 const float* __restrict__ done, const float* __restrict__ vlast,
                                                 int T, int N, int64_t ld, float gamma, float gl,
                                                 float* __restrict__ adv, float* __restrict__ ret, int want_stats,
                                                 StatsOut so)
{
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    double s1 = 0.0, s2 = 0.0;
    if (n < N) {
        float a = 0.0f, vn = vlast[n];
        for (int t = T - 1; t >= 0; --t) {
            const int64_t idx = (int64_t)t * ld + n;
            const float v = val[idx];
            const float nd = 1.0f - done[idx];
            const float delta = rew[idx] + gamma * vn * nd - v;
            a = delta + gl * nd * a;
            adv[idx] = a;
            ret[idx] = a + v;
            s1 += (double)a;
            s2 += (double)a * (double)a;
            vn = v;
        }
    }
    if (want_stats) publish_stats(s1, s2, so);
}

__global__ __launch_bounds__(256) void k_normalize(float* __restrict__ adv, int64_t count, const double* __restrict__ stats)
{
    const float mean = (float)stats[1];
    const float scale = (float)(1.0 / (stats[2] + kNormEps));
    const int64_t n4 = count / 4;
    float4* a4 = reinterpret_cast<float4*>(adv);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
        float4 v = a4[i];
        v.x = (v.x - mean) * scale;
        v.y = (v.y - mean) * scale;
        v.z = (v.z - mean) * scale;
        v.w = (v.w - mean) * scale;
        a4[i] = v;
    }
    for (int64_t i = n4 * 4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (int64_t)gridDim.x * blockDim.x)
        adv[i] = (adv[i] - mean) * scale;
}

// The same over a [T][N] block of rows ld elements apart (normalize = 1 on a column range).
__global__ __launch_bounds__(256) void k_normalize_rows(float* __restrict__ adv, int T, int N, int64_t ld,
                                                        const double* __restrict__ stats)
{
    const float mean = (float)stats[1];
    const float scale = (float)(1.0 / (stats[2] + kNormEps));
    const int64_t count = (int64_t)T * N;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (int64_t)gridDim.x * blockDim.x) {
        float* a = adv + (i / N) * ld + i % N;
        *a = (*a - mean) * scale;
    }
}

// ------------------------------------------------------------------------------------------------
// V-trace targets and policy-gradient advantages (the IMPALA off-policy correction that PlayTrain's
// IMPALA trainer takes from torchbeast, App. C.3; "Teaching Mario to speedrun" s.8 names it beside GAE),
// with the done mask read as for GAE: g_t = gamma (1 - d_t). With ratio_t = exp(log_rho_t),
// rho_t = min(rho_bar, ratio_t), c_t = lambda min(c_bar, ratio_t), the TD error e_t = r_t + g_t V_{t+1} - V_t
// and x_t = vs_t - V_t:
//   x_t = rho_t e_t + g_t c_t x_{t+1}   (x_T = 0, V_T = bootstrap),      vs_t = V_t + x_t,
//   pg_t = min(pg_rho_bar, ratio_t) (r_t + g_t vs_{t+1} - V_t) = min(pg_rho_bar, ratio_t) (e_t + g_t x_{t+1}).
// The same first-order linear recurrence as GAE, so the same chunked scan: each thread holds e, ratio,
// 1 - d and V of its chunk in registers, reduces the chunk to an affine map, the maps compose through
// LDS, and the replay writes vs and pg (24 bytes per element: four inputs read, two outputs written).
// ------------------------------------------------------------------------------------------------

struct VtraceCoef {
    float gamma, lambda, rho_bar, c_bar, pg_rho_bar;
};

template <int E, int LMAX, int BLOCK>
__global__ __launch_bounds__(BLOCK) void k_vtrace_chunked(const float* __restrict__ rew, const float* __restrict__ val,
                                                        const float* __restrict__ done, const float* __restrict__ vlast,
                                                        const float* __restrict__ lrho, int T, int N, int64_t ld,
                                                        int L, VtraceCoef k, float* __restrict__ vs,
                                                        float* __restrict__ pg)
{
    constexpr int C = BLOCK / E;
    __shared__ float sb[C][E];
    __shared__ float sc[C][E];
    const int e = threadIdx.x % E;
    const int ch = threadIdx.x / E;
    const int n = blockIdx.x * E + e;
    const bool valid = n < N;
    const int t0 = ch * L;
    const int len = valid ? max(0, min(L, T - t0)) : 0;

    const int nn = min(n, N - 1);
    float td[LMAX], ratio[LMAX], nd[LMAX], vv[LMAX];
#pragma unroll
    for (int j = 0; j < LMAX; ++j) {
        const int64_t idx = (int64_t)min(t0 + j, T - 1) * ld + nn;
        vv[j] = __builtin_nontemporal_load(val + idx);   // read once: non-temporal, as in the GAE scan
        td[j] = __builtin_nontemporal_load(rew + idx);
        nd[j] = 1.0f - __builtin_nontemporal_load(done + idx);
        ratio[j] = __builtin_nontemporal_load(lrho + idx);
    }
    const float v_after = val[(int64_t)min(t0 + len, T - 1) * ld + nn];
    const float vnext_tail = (t0 + len < T) ? v_after : vlast[nn];

    float b = 0.0f, c = 1.0f;
#pragma unroll
    for (int j = LMAX - 1; j >= 0; --j) {
        if (j < len) {
            const float vn = (j + 1 < len) ? vv[j + 1 < LMAX ? j + 1 : j] : vnext_tail;
            const float g = k.gamma * nd[j];
            ratio[j] = expf(ratio[j]);
            td[j] = td[j] + g * vn - vv[j];
            const float rho = fminf(k.rho_bar, ratio[j]);
            const float gc = g * k.lambda * fminf(k.c_bar, ratio[j]);
            b = rho * td[j] + gc * b;
            c = gc * c;
        }
    }
    sb[ch][e] = b;
    sc[ch][e] = c;
    __syncthreads();

    float a = 0.0f;
    for (int q = C - 1; q > ch; --q) a = sb[q][e] + sc[q][e] * a;

#pragma unroll
    for (int j = LMAX - 1; j >= 0; --j) {
        if (j < len) {
            const float g = k.gamma * nd[j];
            const int64_t idx = (int64_t)(t0 + j) * ld + n;
            pg[idx] = fminf(k.pg_rho_bar, ratio[j]) * (td[j] + g * a);
            a = fminf(k.rho_bar, ratio[j]) * td[j] + g * k.lambda * fminf(k.c_bar, ratio[j]) * a;
            vs[idx] = a + vv[j];
        }
    }
}

// One lane per env walking t = T-1 .. 0: V-trace for horizons longer than the chunked kernels hold.
__global__ __launch_bounds__(256) void k_vtrace_seq(const float* __restrict__ rew, const float* __restrict__ val,
                                                    const float* __restrict__ done, const float* __restrict__ vlast,
                                                    const float* __restrict__ lrho, int T, int N, int64_t ld,
                                                    VtraceCoef k, float* __restrict__ vs, float* __restrict__ pg)
{
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N) return;
    float a = 0.0f, vn = vlast[n];
    for (int t = T - 1; t >= 0; --t) {
        const int64_t idx = (int64_t)t * ld + n;
        const float v = val[idx];
        const float g = k.gamma * (1.0f - done[idx]);
        const float ratio = expf(lrho[idx]);
        const float td = rew[idx] + g * vn - v;
        pg[idx] = fminf(k.pg_rho_bar, ratio) * (td + g * a);
        a = fminf(k.rho_bar, ratio) * td + g * k.lambda * fminf(k.c_bar, ratio) * a;
        vs[idx] = a + v;
        vn = v;
    }
}

enum class GaeKernel { C32x8_16, C16x16_8, C16x16_32, C16x16_64, C256x4_32, Seq };

// Shapes by horizon and batch width. Wide batches take 256 envs x 4 chunks (1 KB row segments per block;
// measured fastest at 65536 x 128 against 64 x 4, 32 x 8, 128 x 8, 64 x 16 and float4 variants); narrow
// batches trade row width for more chunks so that enough lanes are busy.
GaeKernel pick(int T, int N)
{
    if (T <= 128 && (N + 255) / 256 >= 128) return GaeKernel::C256x4_32;
    if (T <= 128) {
        if ((N + 31) / 32 >= 512) return GaeKernel::C32x8_16;
        return GaeKernel::C16x16_8;
    }
    if (T <= 512) return GaeKernel::C16x16_32;
    if (T <= 1024) return GaeKernel::C16x16_64;
    return GaeKernel::Seq;
}

int blocks_of(GaeKernel k, int N)
{
    switch (k) {
    case GaeKernel::C32x8_16: return (N + 31) / 32;
    case GaeKernel::C256x4_32: return (N + 255) / 256;
    case GaeKernel::Seq: return (N + 255) / 256;
    default: return (N + 15) / 16;
    }
}

}  // namespace

extern "C" {

int rl_gae_workspace_bytes(int32_t T, int32_t N, size_t* bytes)
{
    if (T < 1 || N < 1) return rl::fail(RL_EINVAL, "T %d and N %d must be >= 1", T, N);
    if (!bytes) return rl::fail(RL_EINVAL, "bytes is NULL");
    *bytes = sizeof(double) * 2 * (size_t)((N + 15) / 16);
    return RL_OK;
}

int rl_gae_stats_bytes(int32_t T, int32_t N, size_t* bytes)
{
    if (T < 1 || N < 1) return rl::fail(RL_EINVAL, "T %d and N %d must be >= 1", T, N);
    if (!bytes) return rl::fail(RL_EINVAL, "bytes is NULL");
    *bytes = sizeof(double) * (rl::kDeferredHead + 2 * (size_t)blocks_of(pick(T, N), N));
    return RL_OK;
}

int rl_adv_stats_finish(const double* adv_stats, double* out, void* stream)
{
    if (!adv_stats || !out) return rl::fail(RL_EINVAL, "adv_stats and out must be non-NULL");
    if (!rl::aligned(adv_stats, 8) || !rl::aligned(out, 8)) return rl::fail(RL_EALIGN, "adv_stats / out not 8-byte aligned");
    hipLaunchKernelGGL(k_stats_finish, dim3(1), dim3(64), 0, rl::as_stream(stream), adv_stats, out);
    return rl::check_launch("adv_stats_finish");
}

int rl_gae_strided(const float* rewards, const float* values, const float* dones, const float* last_values,
                   int32_t T, int32_t N, int64_t ld, float gamma, float lambda, float* adv, float* ret,
                   int32_t normalize, double* adv_stats, void* ws, size_t ws_bytes, void* stream)
{
    if (T < 1 || N < 1) return rl::fail(RL_EINVAL, "T %d and N %d must be >= 1", T, N);
    if (ld < N) return rl::fail(RL_EINVAL, "row stride %lld < N %d", (long long)ld, N);
    if ((T - 1) * ld + N > ((int64_t)1 << 40)) return rl::fail(RL_EINVAL, "(T-1)*ld + N too large");
    if (!rewards || !values || !dones || !last_values || !adv || !ret)
        return rl::fail(RL_EINVAL, "rewards, values, dones, last_values, adv and ret must be non-NULL");
    if (normalize < 0 || normalize > 3) return rl::fail(RL_EINVAL, "normalize %d outside {0, 1, 2, 3}", normalize);
    if (normalize != 0 && !adv_stats) return rl::fail(RL_EINVAL, "normalize %d needs adv_stats", normalize);
    if ((normalize == 1 || normalize == 2) && !ws) return rl::fail(RL_EINVAL, "normalize %d needs ws", normalize);
    const void* ptrs[] = {rewards, values, dones, last_values, adv, ret};
    for (const void* p : ptrs)
        if (!rl::aligned(p, 4)) return rl::fail(RL_EALIGN, "a float array is not 4-byte aligned");
    size_t need = 0;
    rl_gae_workspace_bytes(T, N, &need);
    if (normalize == 1 || normalize == 2) {
        if (!rl::aligned(ws, 8) || !rl::aligned(adv_stats, 8)) return rl::fail(RL_EALIGN, "ws / adv_stats not 8-byte aligned");
        if (ws_bytes < need) return rl::fail(RL_ESIZE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
    }
    if (normalize == 3 && !rl::aligned(adv_stats, 8)) return rl::fail(RL_EALIGN, "adv_stats not 8-byte aligned");
    hipStream_t st = rl::as_stream(stream);
    const float gl = gamma * lambda;
    StatsOut so{};
    so.count = (double)T * (double)N;
    if (normalize == 1 || normalize == 2) so.partials = static_cast<double*>(ws);
    if (normalize == 3) {   // the partials and their header into the caller's adv_stats; no finalise
        so.partials = adv_stats + rl::kDeferredHead;
        so.header = adv_stats;
    }
    const int want = normalize != 0 ? 1 : 0;
    const GaeKernel k = pick(T, N);
    const dim3 grid(blocks_of(k, N)), block(256);
    switch (k) {
    case GaeKernel::C32x8_16:
        hipLaunchKernelGGL((k_gae_chunked<32, 16, 256>), grid, block, 0, st, rewards, values, dones, last_values, T, N, ld,
                           (T + 7) / 8, gamma, gl, adv, ret, want, so);
        break;
    case GaeKernel::C16x16_8:
        hipLaunchKernelGGL((k_gae_chunked<16, 8, 256>), grid, block, 0, st, rewards, values, dones, last_values, T, N, ld,
                           (T + 15) / 16, gamma, gl, adv, ret, want, so);
        break;
    case GaeKernel::C16x16_32:
        hipLaunchKernelGGL((k_gae_chunked<16, 32, 256>), grid, block, 0, st, rewards, values, dones, last_values, T, N, ld,
                           (T + 15) / 16, gamma, gl, adv, ret, want, so);
        break;
    case GaeKernel::C16x16_64:
        hipLaunchKernelGGL((k_gae_chunked<16, 64, 256>), grid, block, 0, st, rewards, values, dones, last_values, T, N, ld,
                           (T + 15) / 16, gamma, gl, adv, ret, want, so);
        break;
    case GaeKernel::C256x4_32:
        hipLaunchKernelGGL((k_gae_chunked<256, 32, 1024>), grid, dim3(1024), 0, st, rewards, values, dones,
                           last_values, T, N, ld, (T + 3) / 4, gamma, gl, adv, ret, want, so);
        break;
    case GaeKernel::Seq:
        hipLaunchKernelGGL(k_gae_seq, grid, block, 0, st, rewards, values, dones, last_values, T, N, ld, gamma, gl,
                           adv, ret, want, so);
        break;
    }
    if (int rc = rl::check_launch("gae_scan")) return rc;
    if (normalize == 1 || normalize == 2) {
        hipLaunchKernelGGL(k_stats_finalize, dim3(1), dim3(64), 0, st, static_cast<const double*>(ws),
                           blocks_of(k, N), (double)T * (double)N, adv_stats);
        if (int rc = rl::check_launch("adv_stats")) return rc;
    }
    if (normalize == 1) {
        const int64_t count = (int64_t)T * N;
        if (ld == N && rl::aligned(adv, 16)) {   // one contiguous block: float4 passes
            const int nb = (int)std::min<int64_t>((count / 4 + 255) / 256 + 1, 8192);
            hipLaunchKernelGGL(k_normalize, dim3(nb), dim3(256), 0, st, adv, count, adv_stats);
        } else {
            const int nb = (int)std::min<int64_t>((count + 255) / 256, 8192);
            hipLaunchKernelGGL(k_normalize_rows, dim3(nb), dim3(256), 0, st, adv, T, N, ld, adv_stats);
        }
        if (int rc = rl::check_launch("adv_normalize")) return rc;
    }
    return RL_OK;
}

int rl_gae(const float* rewards, const float* values, const float* dones, const float* last_values, int32_t T,
           int32_t N, float gamma, float lambda, float* adv, float* ret, int32_t normalize, double* adv_stats,
           void* ws, size_t ws_bytes, void* stream)
{
    return rl_gae_strided(rewards, values, dones, last_values, T, N, N, gamma, lambda, adv, ret, normalize, adv_stats,
                          ws, ws_bytes, stream);
}

int rl_vtrace_strided(const float* rewards, const float* values, const float* dones, const float* last_values,
                      const float* log_rhos, int32_t T, int32_t N, int64_t ld, float gamma, float lambda,
                      float rho_bar, float c_bar, float pg_rho_bar, float* vs, float* pg_adv, void* stream)
{
    if (T < 1 || N < 1) return rl::fail(RL_EINVAL, "T %d and N %d must be >= 1", T, N);
    if (ld < N) return rl::fail(RL_EINVAL, "row stride %lld < N %d", (long long)ld, N);
    if ((T - 1) * ld + N > ((int64_t)1 << 40)) return rl::fail(RL_EINVAL, "(T-1)*ld + N too large");
    if (!rewards || !values || !dones || !last_values || !log_rhos || !vs || !pg_adv)
        return rl::fail(RL_EINVAL, "rewards, values, dones, last_values, log_rhos, vs and pg_adv must be non-NULL");
    if (!(rho_bar >= 0.0f) || !(c_bar >= 0.0f) || !(pg_rho_bar >= 0.0f))
        return rl::fail(RL_EINVAL, "rho_bar, c_bar and pg_rho_bar must be >= 0");
    const void* ptrs[] = {rewards, values, dones, last_values, log_rhos, vs, pg_adv};
    for (const void* p : ptrs)
        if (!rl::aligned(p, 4)) return rl::fail(RL_EALIGN, "a float array is not 4-byte aligned");
    hipStream_t st = rl::as_stream(stream);
    const VtraceCoef k{gamma, lambda, rho_bar, c_bar, pg_rho_bar};
    if (T <= 128 && (N + 127) / 128 >= 256) {
        hipLaunchKernelGGL((k_vtrace_chunked<128, 16, 1024>), dim3((N + 127) / 128), dim3(1024), 0, st, rewards, values,
                           dones, last_values, log_rhos, T, N, ld, (T + 7) / 8, k, vs, pg_adv);
    } else if (T <= 128) {
        hipLaunchKernelGGL((k_vtrace_chunked<16, 8, 256>), dim3((N + 15) / 16), dim3(256), 0, st, rewards, values,
                           dones, last_values, log_rhos, T, N, ld, (T + 15) / 16, k, vs, pg_adv);
    } else if (T <= 256) {
        hipLaunchKernelGGL((k_vtrace_chunked<16, 16, 256>), dim3((N + 15) / 16), dim3(256), 0, st, rewards, values,
                           dones, last_values, log_rhos, T, N, ld, (T + 15) / 16, k, vs, pg_adv);
    } else if (T <= 512) {
        // four per-step arrays of 32 steps would not fit the register file: 32 chunks of up to 16 steps
        hipLaunchKernelGGL((k_vtrace_chunked<8, 16, 256>), dim3((N + 7) / 8), dim3(256), 0, st, rewards, values,
                           dones, last_values, log_rhos, T, N, ld, (T + 31) / 32, k, vs, pg_adv);
    } else {
        hipLaunchKernelGGL(k_vtrace_seq, dim3((N + 255) / 256), dim3(256), 0, st, rewards, values, dones, last_values,
                           log_rhos, T, N, ld, k, vs, pg_adv);
    }
    return rl::check_launch("vtrace");
}

int rl_vtrace(const float* rewards, const float* values, const float* dones, const float* last_values,
              const float* log_rhos, int32_t T, int32_t N, float gamma, float lambda, float rho_bar, float c_bar,
              float pg_rho_bar, float* vs, float* pg_adv, void* stream)
{
    return rl_vtrace_strided(rewards, values, dones, last_values, log_rhos, T, N, N, gamma, lambda, rho_bar, c_bar,
                             pg_rho_bar, vs, pg_adv, stream);
}

}  // extern "C"
