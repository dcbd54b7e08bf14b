// PPO loss forward reductions per minibatch ("Teaching Mario to speedrun", s.6 Don't move too far at once):
// for every sample of minibatch m, the log-softmax of its logits, the probability ratio against the
// recorded old log-probability, the clipped surrogate, the squared value error and the policy entropy;
// their minibatch means and the weighted total.
//
// Two ways to visit the samples, both ending in per-block float64 partials that a finalise kernel (one
// block per minibatch) reduces in block order; no floating-point atomics, so results are identical from
// run to run.
//   Gather (contiguous, or perm with more than 64 minibatches): grid (blocks per minibatch, minibatches);
//   thread k of minibatch m reads sample perm[m*mb + k]. Shuffled indices make every per-sample read a
//   random access.
//   perm with at most 64 minibatches is first sorted by destination into bins (one launch, each block
//   sorting its positions in LDS), then takes the stream pass below: the same sets, summed in storage
//   order instead of perm order. Up to 16 minibatches each stream block's chunk is one bin, whose entries
//   the block places in LDS as 4-bit minibatch numbers before it streams; with more, one block per bin
//   writes 2-byte numbers that the stream pass reads.
//   Stream (mb_index): each minibatch's scalars are means over its set of samples, so one pass over the
//   batch in storage order serves all minibatches at once: every read is coalesced and each sample is
//   read exactly once. Each thread adds its samples' terms into its own per-minibatch slots in LDS
//   (private, so no atomics and a fixed order), and the block then sums the slots thread by thread.
//
// With a gradient (rl_ppo_loss_grad), the same pass also writes each sample's row of dL_m/dlogits and its
// dL_m/dV for the minibatch m that holds it: the fused loss-and-gradient step that the same page (s.8,
// the port of the trainer to GPU shaders) describes. With p = softmax(z), r the ratio, c its clip and
// M the minibatch size:
//   dL/dz_j = (1/M) (-[r A <= c A] A r ([j == a] - p_j) + ent_coef p_j (log p_j + H)),
//   dL/dV   = (1/M) 2 vf_coef (V - R).
// The surrogate's minimum takes the unclipped term whenever r A <= c A (inside the clip band the two
// terms are equal), where its derivative in r is -A; on the clipped side it is constant. Advantages,
// normalised or not, are constants.

#include <algorithm>
#include <mutex>

#include "rl_internal.hpp"

namespace {

constexpr double kNormEps = 1e-8;
constexpr int kSamplesPerThread = 8;
constexpr int kMaxBlocksPerMb = 4096;

// Where the perm conversion's sort left each bin's entries: staging row k (kSortPositions words) holds
// position block k's entries sorted by bin, and starts row k (bins + 1 words) where each bin's run begins.
struct PermRuns {
    const int32_t* starts;
    const uint32_t* staging;
    int rows, bins;
};

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
    double* partials;   // [num_mb][blocks][3]
    const uint16_t* mb_index;
    int64_t B;
    int num_mb;
    float* dlogits;     // [B][A], or NULL without a gradient
    float* dvalues;     // [B]
    float inv_mb;       // 1 / M
    float dv_coef;      // 2 vf / M
    PermRuns runs;      // the sorted perm, for the stream pass that places its own chunk's numbers
};

// The normalisation of the advantages from adv_stats, which holds either the finished statistics
// {count, mean, std} or the scan blocks' deferred partial sums (rl_gae with normalize = 3, header
// adv_stats[0] < 0). Deferred partials are reduced by wave 0 with rl::stats_from_partials, the function the
// scan's own finalise uses, so mean and std have the same bits either way. Every thread calls it; the
// block's barrier follows it, after which norm_read gives mean and the scale 1 / (std + eps).
__device__ __forceinline__ void norm_reduce(const double* __restrict__ stats, double* nrm)
{
    if (stats && stats[0] < 0.0 && threadIdx.x < 64) {
        double mean, stdev;
        rl::stats_from_partials(stats + rl::kDeferredHead, (int)(-stats[0]), stats[1], mean, stdev);
        if (threadIdx.x == 0) {
            nrm[0] = mean;
            nrm[1] = stdev;
        }
    }
}

__device__ __forceinline__ void norm_read(const double* __restrict__ stats, const double* nrm, float& mean, float& scale)
{
    mean = 0.0f;
    scale = 1.0f;
    if (stats) {
        const bool deferred = stats[0] < 0.0;
        const double mu = deferred ? nrm[0] : stats[1];
        const double sd = deferred ? nrm[1] : stats[2];
        mean = (float)mu;
        scale = (float)(1.0 / (sd + kNormEps));
    }
}

// Sums of three doubles across a block of at most 4 waves, each in the same fixed order on every run (a
// wave's butterfly, then the waves in order), with one barrier. The LDS array (12 doubles) must not have
// been used earlier in the kernel.
__device__ __forceinline__ void block_sum3(double& a, double& b, double& c, double* lds)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        a += __shfl_xor(a, off, 64);
        b += __shfl_xor(b, off, 64);
        c += __shfl_xor(c, off, 64);
    }
    const int w = threadIdx.x >> 6, nw = (int)(blockDim.x >> 6);
    if ((threadIdx.x & 63) == 0) {
        lds[w] = a;
        lds[4 + w] = b;
        lds[8 + w] = c;
    }
    __syncthreads();
    a = 0.0;
    b = 0.0;
    c = 0.0;
    for (int i = 0; i < nw; ++i) {
        a += lds[i];
        b += lds[4 + i];
        c += lds[8 + i];
    }
}

// The logits row of a sample in registers (AC = compile-time action count).
template <int AC>
__device__ __forceinline__ void load_row(const float* __restrict__ row, float (&z)[AC])
{
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
}

// e^x and ln x from the hardware's base-2 exponential and logarithm (v_exp_f32 / v_log_f32, about one
// ulp each): e^x = 2^(x log2 e), ln x = log2 x ln 2. The arguments here are u <= 0 (results in (0, 1]),
// ratios' log differences, and sums >= 1, so no denormal scaling is needed.
__device__ __forceinline__ float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }
__device__ __forceinline__ float log_hw(float x) { return __builtin_amdgcn_logf(x) * 0.693147180559945309f; }

// Row statistics with u_j = z_j - max z: log_s = log(S), S = sum e^{u_j}, mean_u = (sum e^{u_j} u_j) / S
// (the entropy is log_s - mean_u), u_a = u of the taken action.
struct RowStats {
    float mx, log_s, mean_u, u_a, inv_s;
};

// AC > 0: the row in registers z; the e^{u_j} stay in ex for the gradient.
template <int AC>
__device__ __forceinline__ RowStats row_stats(const float (&z)[AC], int a, float (&ex)[AC])
{
    float mx = z[0];
#pragma unroll
    for (int j = 1; j < AC; ++j) mx = fmaxf(mx, z[j]);
    float s = 0.0f, su = 0.0f, ua = z[0] - mx;
#pragma unroll
    for (int j = 0; j < AC; ++j) {
        const float u = z[j] - mx;
        ex[j] = exp_hw(u);
        s += ex[j];
        su += ex[j] * u;
        ua = j == a ? u : ua;
    }
    RowStats r;
    r.mx = mx;
    r.inv_s = __builtin_amdgcn_rcpf(s);
    r.log_s = log_hw(s);
    r.mean_u = su * r.inv_s;
    r.u_a = ua;
    return r;
}

// Runtime A: the row is read from memory.
__device__ __forceinline__ RowStats row_stats_mem(const float* __restrict__ row, int A, int a)
{
    float mx = row[0];
    for (int j = 1; j < A; ++j) mx = fmaxf(mx, row[j]);
    float s = 0.0f, su = 0.0f;
    for (int j = 0; j < A; ++j) {
        const float u = row[j] - mx;
        const float ex = exp_hw(u);
        s += ex;
        su += ex * u;
    }
    RowStats r;
    r.mx = mx;
    r.inv_s = __builtin_amdgcn_rcpf(s);
    r.log_s = log_hw(s);
    r.mean_u = su * r.inv_s;
    r.u_a = row[a] - mx;
    return r;
}

// A sample's inputs, loaded ahead of its arithmetic (AC = 0: the logits stay in memory).
template <int AC>
struct SampleIn {
    float z[AC > 0 ? AC : 1];
    int32_t a;
    float old_logp, adv, ret, v;
};

template <int AC>
__device__ __forceinline__ void load_sample(const LossArgs& p, int64_t i, SampleIn<AC>& s)
{
    if constexpr (AC > 0) load_row<AC>(p.logits + i * AC, s.z);
    s.a = p.actions[i];
    s.old_logp = p.old_logp[i];
    s.adv = p.adv[i];
    s.ret = p.ret[i];
    s.v = p.new_v[i];
}

// The three per-sample terms of sample i (inputs s): clipped surrogate, squared value error, entropy;
// with GRAD and `write` also the sample's gradient row and value gradient.
template <int AC, bool GRAD>
__device__ __forceinline__ void terms_of(const LossArgs& p, int64_t i, bool write, const SampleIn<AC>& s, float mean,
                                         float scale, float* pg, float* v, float* h, float* gz_out = nullptr)
{
    const int A = AC > 0 ? AC : p.A;
    int a = s.a;
    if (a < 0 || a >= A) a = 0;   // an out-of-range action reads logit 0
    const float* row = p.logits + i * A;
    float ex[AC > 0 ? AC : 1];
    RowStats r;
    if constexpr (AC > 0) r = row_stats<AC>(s.z, a, ex);
    else r = row_stats_mem(row, A, a);
    const float logp = r.u_a - r.log_s;
    *h = r.log_s - r.mean_u;
    const float ratio = exp_hw(logp - s.old_logp);
    float adv = s.adv;
    if (p.stats) adv = (adv - mean) * scale;
    // clip and minimum by comparisons, which pass a NaN ratio on (fminf / fmaxf would drop it)
    const float clipped = ratio < p.clip_lo ? p.clip_lo : (ratio > p.clip_hi ? p.clip_hi : ratio);
    const float s1 = ratio * adv, s2 = clipped * adv;
    *pg = -(s1 < s2 ? s1 : s2);
    const float dv = s.v - s.ret;
    *v = dv * dv;
    if constexpr (GRAD) {
        if (!write) return;
        // p_j = e^{u_j} / S, and log p_j + H = (u_j - log_s) + (log_s - mean_u) = u_j - mean_u
        const float c_pg = s1 <= s2 ? -adv * ratio * p.inv_mb : 0.0f;   // times ([j == a] - p_j)
        const float c_h = p.ent * p.inv_mb;                               // times p_j (log p_j + H)
        float* g = p.dlogits + i * A;
        if constexpr (AC > 0) {
            float gz[AC];
#pragma unroll
            for (int j = 0; j < AC; ++j) {
                const float pj = ex[j] * r.inv_s;
                gz[j] = c_pg * ((j == a ? 1.0f : 0.0f) - pj) + c_h * pj * ((s.z[j] - r.mx) - r.mean_u);
            }
            if (gz_out) {   // the caller stores the row
#pragma unroll
                for (int j = 0; j < AC; ++j) gz_out[j] = gz[j];
            } else if constexpr (AC % 4 == 0) {
#pragma unroll
                for (int j = 0; j < AC / 4; ++j)
                    reinterpret_cast<float4*>(g)[j] = make_float4(gz[4 * j], gz[4 * j + 1], gz[4 * j + 2], gz[4 * j + 3]);
            } else {
#pragma unroll
                for (int j = 0; j < AC; ++j) g[j] = gz[j];
            }
        } else {
            for (int j = 0; j < A; ++j) {
                const float u = row[j] - r.mx;
                const float pj = exp_hw(u) * r.inv_s;
                g[j] = c_pg * ((j == a ? 1.0f : 0.0f) - pj) + c_h * pj * (u - r.mean_u);
            }
        }
        p.dvalues[i] = p.dv_coef * dv;
    }
}

template <int AC, bool GRAD>
__device__ __forceinline__ void sample_terms(const LossArgs& p, int64_t i, float mean, float scale, float* pg,
                                             float* v, float* h)
{
    SampleIn<AC> s;
    load_sample<AC>(p, i, s);
    terms_of<AC, GRAD>(p, i, true, s, mean, scale, pg, v, h);
}

template <int AC, bool GRAD>
__global__ __launch_bounds__(256) void k_ppo_loss(LossArgs p)
{
    __shared__ double lds[12];
    __shared__ double nrm[2];
    const int m = blockIdx.y;
    const int64_t base = (int64_t)m * p.mb;
    norm_reduce(p.stats, nrm);
    __syncthreads();
    float mean, scale;
    norm_read(p.stats, nrm, mean, scale);
    double s_pg = 0.0, s_v = 0.0, s_h = 0.0;
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < p.mb; k += step) {
        // entries outside [0, B) (never in a permutation) are clamped so that every read stays in bounds
        const int64_t i = p.perm ? min(max((int64_t)p.perm[base + k], (int64_t)0), p.B - 1) : base + k;
        float pg, v, h;
        sample_terms<AC, GRAD>(p, i, mean, scale, &pg, &v, &h);
        s_pg += (double)pg;
        s_v += (double)v;
        s_h += (double)h;
    }
    block_sum3(s_pg, s_v, s_h, lds);
    if (threadIdx.x == 0) {
        double* part = p.partials + ((int64_t)m * gridDim.x + blockIdx.x) * 3;
        part[0] = s_pg;
        part[1] = s_v;
        part[2] = s_h;
    }
}

// Binned perm conversion. perm names, position by position, the sample that minibatch position / mb
// takes; the stream pass wants the inverse, each sample's minibatch. The plain inverse,
// ids[perm[p]] = p / mb, is a random 2-byte scatter (k_perm_to_index below, kept for batches past 2^24
// samples). Binned instead, with destinations in bins of S consecutive samples:
//   sort   one launch over blocks of kSortPositions positions (32 a thread). A block tags its entries
//          with their destination's bin, counts them per bin in LDS, sorts them by bin in LDS and writes
//          them back as one contiguous piece (its staging row), with the start of each bin's run in that
//          row (its starts row: bins + 1 words, the last the row's entry count);
//   place  bin b's entries are the runs [starts[k][b], starts[k][b + 1]) of the staging rows k, placed by
//          destination in LDS. With at most 16 minibatches the stream pass's own blocks do this (block b's
//          chunk is bin b; a 4-bit number per sample, 8 KB for the largest bin), so no minibatch number
//          goes through memory; with 17 to 64, k_perm_place_runs writes 2-byte numbers for the stream
//          kernels of 32 and 64 minibatches (bins of kBinCap samples).
// No global atomics and no scan across blocks: every block's output has a fixed place. A staged entry is
// the destination's offset in its bin (14 bits) and its minibatch (6 bits); inside the sort its bin
// follows (bits 20 and up).
constexpr int kSortPositions = 16384;
constexpr int kSortThreads = 512;
// Words from one staging row to the next: a bin's runs lie at about the same offset in every row, and 256
// bytes more than the row staggers a consumer's reads across rows instead of keeping them 64 KB apart
// (measured: about 1% on the whole perm loss).
constexpr int kStagingStride = kSortPositions + 64;
constexpr int kBinCap = 16384;            // samples a bin holds at most: offsets take 14 bits
constexpr int kMaxBins = 1024;
constexpr int kMapWords = kBinCap / 8;    // a bin's 4-bit minibatch numbers, 8 to a word

// Block-wide exclusive sum over W waves of one value a thread (LDS `sh` of W words); returns the thread's
// prefix and leaves the block total in *total.
template <int W>
__device__ __forceinline__ int32_t block_exclusive_sum(int32_t v, int32_t* sh, int32_t* total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int32_t inc = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t o = __shfl_up(inc, off, 64);
        if (lane >= off) inc += o;
    }
    if (lane == 63) sh[w] = inc;
    __syncthreads();
    int32_t before = 0, all = 0;
#pragma unroll
    for (int k = 0; k < W; ++k) {
        const int32_t s = sh[k];
        before += k < w ? s : 0;
        all += s;
    }
    *total = all;
    __syncthreads();
    return before + inc - v;
}

// x / d for 0 <= x < 2^25 and quotients below 2^12: the float quotient is then within one of the exact
// one (two roundings of relative size 2^-24), and one step corrects it; q * d stays below 2^26.
__device__ __forceinline__ int32_t small_quotient(int32_t x, int32_t d, float inv_d)
{
    int32_t q = (int32_t)((float)x * inv_d);
    if (q * d > x) --q;
    else if ((q + 1) * d <= x) ++q;
    return q;
}

constexpr size_t kSortLdsBytes = sizeof(uint32_t) * kSortPositions + sizeof(int32_t) * (kMaxBins + 1 + kSortThreads / 64);

// The sort. B <= 2^24, bins <= kMaxBins and S <= kBinCap (bins = ceil(B / S)), at most 64 minibatches.
// Positions past the batch's end (the last block's) go to a spare bin, kMaxBins, so that every load and
// every LDS update is unconditional; their sorted slots follow the block's entries and are not written.
__global__ __launch_bounds__(kSortThreads) void k_perm_sort(const int32_t* __restrict__ perm, int32_t B, int32_t mb,
                                                            float inv_mb, int32_t S, float inv_S, int bins,
                                                            int32_t* __restrict__ starts,
                                                            uint32_t* __restrict__ staging)
{
    constexpr int PPT = kSortPositions / kSortThreads;
    constexpr int W = kSortThreads / 64;
    constexpr int BPT = kMaxBins / kSortThreads;    // bins a thread scans
    // LDS from the launch (kSortLdsBytes): the sorted entries, the bins' counts and then their first slots
    // (+ the spare bin), the scan's wave sums
    uint32_t* sorted = reinterpret_cast<uint32_t*>(rl::launch_lds());
    int32_t* cur = reinterpret_cast<int32_t*>(sorted + kSortPositions);
    int32_t* sh = cur + kMaxBins + 1;
    const int t = threadIdx.x;
    const int32_t lo = blockIdx.x * kSortPositions;
    const int32_t hi = min(B, lo + kSortPositions);
    uint32_t e[PPT];
#pragma unroll
    for (int j = 0; j < PPT; ++j) e[j] = (uint32_t)perm[min(lo + t + kSortThreads * j, hi - 1)];
    for (int b = t; b <= kMaxBins; b += kSortThreads) cur[b] = 0;
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        const int32_t p = lo + t + kSortThreads * j;
        const int32_t d = min(max((int32_t)e[j], 0), B - 1);   // a permutation has no entry outside [0, B)
        const int32_t bin = small_quotient(d, S, inv_S);
        const int32_t m = small_quotient(p, mb, inv_mb);
        e[j] = p < hi ? (uint32_t)(d - bin * S) | ((uint32_t)m << 14) | ((uint32_t)bin << 20) : 0xffffffffu;
    }
    __syncthreads();
    // counting gives each entry its rank among the block's entries of its bin (in whatever order the
    // atomics land: a bin's entries are a set, their order within its run does not matter)
    int32_t rank[PPT];
#pragma unroll
    for (int j = 0; j < PPT; ++j) rank[j] = atomicAdd(&cur[e[j] == 0xffffffffu ? kMaxBins : (int)(e[j] >> 20)], 1);
    __syncthreads();
    int32_t c[BPT];
    int32_t own = 0;
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
        const int b = t * BPT + q;
        c[q] = b < bins ? cur[b] : 0;
        own += c[q];
    }
    int32_t total;
    int32_t start = block_exclusive_sum<W>(own, sh, &total);
    int32_t* row = starts + (int64_t)blockIdx.x * (bins + 1);
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
        const int b = t * BPT + q;
        if (b < bins) {
            cur[b] = start;
            row[b] = start;
        }
        start += c[q];
    }
    if (t == 0) {
        cur[kMaxBins] = total;
        row[bins] = total;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PPT; ++j) rank[j] += cur[e[j] == 0xffffffffu ? kMaxBins : (int)(e[j] >> 20)];
#pragma unroll
    for (int j = 0; j < PPT; ++j) sorted[rank[j]] = e[j] & 0xfffffu;
    __syncthreads();
    const int n = hi - lo;
    uint32_t* out = staging + (int64_t)blockIdx.x * kStagingStride;
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        const int i = t + kSortThreads * j;
        if (i < n) out[i] = sorted[i];
    }
}

// Calls put(offset, minibatch) for every staged entry of bin b (for a permutation, each offset of the bin
// exactly once), from THREADS threads. A wave reads one run per load instruction, a lane an entry, so that
// the loads coalesce (a shuffled perm's runs average S * kSortPositions / B entries, 32 at the bench's
// sizes). Wave w takes rows w, w + W, ... 64 at a time: each lane loads one row's run bounds, then the wave
// issues the loads of R runs (each clamped into its row; only their use is masked) before it places any.
// Entries past a run's 64th (only where one position block sends many entries to one bin, as an
// unshuffled perm does) take further passes of the wave.
template <int THREADS, typename Put>
__device__ __forceinline__ void for_bin_entries(const PermRuns& r, int b, Put put)
{
    constexpr int W = THREADS / 64;
    constexpr int R = 32;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int k0 = w; k0 < r.rows; k0 += 64 * W) {
        const int n = min(64, (r.rows - k0 + W - 1) / W);   // rows of this group: k0 + W * j, j < n
        const int k = min(k0 + W * lane, r.rows - 1);
        const int32_t* row = r.starts + (int64_t)k * (r.bins + 1) + b;
        const int32_t beg = row[0];
        const int32_t len = lane < n ? row[1] - beg : 0;
        for (int j0 = 0; j0 < n; j0 += R) {
            uint32_t v[R];
#pragma unroll
            for (int q = 0; q < R; ++q) {
                const int j = min(j0 + q, 63);
                const int32_t bj = __builtin_amdgcn_readlane(beg, j), lj = __builtin_amdgcn_readlane(len, j);
                const int64_t kj = min(k0 + W * j, r.rows - 1);
                v[q] = r.staging[kj * kStagingStride + min(max(bj + min(lane, lj - 1), 0), kSortPositions - 1)];
            }
#pragma unroll
            for (int q = 0; q < R; ++q) {
                const int j = min(j0 + q, 63);
                const int32_t lj = __builtin_amdgcn_readlane(len, j);
                if (j0 + q < n && lane < lj) put((int)(v[q] & (kBinCap - 1)), (int)((v[q] >> 14) & 63));
            }
        }
        for (int j = 0; j < n; ++j) {
            const int32_t bj = __builtin_amdgcn_readlane(beg, j), lj = __builtin_amdgcn_readlane(len, j);
            const int64_t kj = k0 + W * j;
            for (int i = 64 + lane; i < lj; i += 64) {
                const uint32_t e = r.staging[kj * kStagingStride + min(bj + i, kSortPositions - 1)];
                put((int)(e & (kBinCap - 1)), (int)((e >> 14) & 63));
            }
        }
    }
}

// With 17 to 64 minibatches: one block per bin of kBinCap samples places the bin's entries in an LDS
// window (destinations no entry names read 0xffff, past every minibatch, which the stream pass counts as
// the last; a permutation names every destination once), then writes the bin's minibatch numbers as one
// piece with 16-byte stores.
__global__ __launch_bounds__(512) void k_perm_place_runs(PermRuns r, int64_t B, uint16_t* __restrict__ ids)
{
    __shared__ uint4 win4[kBinCap / 8];
    uint16_t* win = reinterpret_cast<uint16_t*>(win4);
    const int b = blockIdx.x;
    const int t = threadIdx.x;
    for (int q = t; q < kBinCap / 8; q += 512) win4[q] = make_uint4(0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu);
    __syncthreads();
    for_bin_entries<512>(r, b, [&](int off, int m) { win[off] = (uint16_t)m; });
    __syncthreads();
    const int64_t lo = (int64_t)b * kBinCap;
    const int n = (int)min((int64_t)kBinCap, B - lo);
    uint4* out4 = reinterpret_cast<uint4*>(ids + lo);     // lo is a multiple of 16384: 32 KB aligned
    for (int q = t; q < n / 8; q += 512) out4[q] = win4[q];
    for (int i = (n / 8) * 8 + t; i < n; i += 512) ids[lo + i] = win[i];
}

// Stream mode: block b visits samples [b*chunk, min(B, (b+1)*chunk)) in storage order. THREADS * NB * 3
// floats of LDS hold each thread's private per-minibatch sums (slot (j*3 + s)*THREADS + thread). A
// thread loads the inputs of its next U samples (indices clamped to the chunk, so the loads issue
// together) before the arithmetic of the first; it still adds its samples in increasing index order.
// The minibatch numbers come from mb_index, or (MAP) from the sorted perm: block b's chunk is then bin b of
// the sort, whose entries the block first places in LDS as 4-bit numbers. Either way the samples, their
// order and the slots are the same, so the two give the same bits.
// LDS bytes of a stream block: the slots, then the 4-bit minibatch numbers (MAP) or two doubles.
constexpr size_t stream_lds_bytes(int NB, int THREADS, bool MAP)
{
    return sizeof(float) * ((size_t)NB * 3 * THREADS + (MAP ? kMapWords : 4));
}

template <int AC, int NB, int THREADS, int U, bool GRAD, bool MAP = false>
__global__ __launch_bounds__(THREADS) void k_ppo_loss_stream(LossArgs p, int64_t chunk)
{
    constexpr int kAcc = NB * 3 * THREADS;
    static_assert(!MAP || NB <= 16, "4-bit minibatch numbers");
    // the slots, then the chunk's minibatch numbers (MAP) or the normalisation's two doubles; with MAP the
    // doubles pass through the last 16 bytes of the slots, which are cleared only after every thread has
    // read them
    float* lds = reinterpret_cast<float*>(rl::launch_lds());   // stream_lds_bytes(NB, THREADS, MAP)
    float* acc = lds;
    uint32_t* map = reinterpret_cast<uint32_t*>(lds + kAcc);
    double* nrm = reinterpret_cast<double*>(MAP ? lds + kAcc - 4 : lds + kAcc);
    const int t = threadIdx.x;
    if constexpr (MAP) {
        for (int j = t; j < kMapWords; j += THREADS) map[j] = 0xffffffffu;
    } else {
        for (int j = t; j < kAcc; j += THREADS) acc[j] = 0.0f;
    }
    norm_reduce(p.stats, nrm);
    __syncthreads();
    float mean, scale;
    norm_read(p.stats, nrm, mean, scale);
    if constexpr (MAP) {
        // a number is set by clearing the bits it lacks: a destination no entry names keeps 15, the last
        for_bin_entries<THREADS>(p.runs, blockIdx.x, [&](int off, int m) {
            atomicAnd(&map[off >> 3], ~((uint32_t)(~m & 15) << ((off & 7) * 4)));
        });
        __syncthreads();
        for (int j = t; j < kAcc; j += THREADS) acc[j] = 0.0f;
        __syncthreads();
    }
    const int64_t lo = (int64_t)blockIdx.x * chunk;
    const int64_t hi = min(p.B, lo + chunk);
    for (int64_t i0 = lo + t; i0 < hi; i0 += (int64_t)THREADS * U) {
        SampleIn<AC> s[U];
        int mbi[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = min(i0 + (int64_t)u * THREADS, hi - 1);
            load_sample<AC>(p, i, s[u]);
            // past the last minibatch counts as the last
            if constexpr (MAP) {
                const int li = (int)(i - lo);
                mbi[u] = min((int)((map[li >> 3] >> ((li & 7) * 4)) & 15u), p.num_mb - 1);
            } else {
                mbi[u] = min((int)p.mb_index[i], p.num_mb - 1);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // every sample's arithmetic runs (a clamped one on a copy of the chunk's last sample, which
            // adds +0 to the sums and writes no gradient), so no load is moved behind a branch
            const int64_t i = i0 + (int64_t)u * THREADS;
            const bool valid = i < hi;
            float pg, v, h;
            if constexpr (GRAD && AC == 12) {
                // the wave's 64 samples are consecutive: when all are in the chunk, its 64 gradient rows
                // (3 KB, contiguous) go out as three 1 KB stores, each lane's 16 bytes gathered from the
                // lanes that own them; else every lane stores its own row
                float gz[12];
                terms_of<AC, GRAD>(p, min(i, hi - 1), valid, s[u], mean, scale, &pg, &v, &h, gz);
                const int L = t & 63;
                const int64_t base = i - L;
                if (base + 63 < hi) {
                    float4* dst = reinterpret_cast<float4*>(p.dlogits + base * 12);
#pragma unroll
                    for (int j = 0; j < 3; ++j) {
                        // float 256 j + 4 L + c of the block is element 4 ((j + L) mod 3) + c of sample
                        // (256 j + 4 L + c) / 12
                        const int sel = (j + L) % 3;
                        float out[4];
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const int src = (256 * j + 4 * L + c) / 12;
                            const float v0 = __shfl(gz[c], src, 64), v1 = __shfl(gz[c + 4], src, 64),
                                        v2 = __shfl(gz[c + 8], src, 64);
                            out[c] = sel == 0 ? v0 : (sel == 1 ? v1 : v2);
                        }
                        dst[64 * j + L] = make_float4(out[0], out[1], out[2], out[3]);
                    }
                } else if (valid) {
                    float4* g4 = reinterpret_cast<float4*>(p.dlogits + i * 12);
#pragma unroll
                    for (int j = 0; j < 3; ++j) g4[j] = make_float4(gz[4 * j], gz[4 * j + 1], gz[4 * j + 2], gz[4 * j + 3]);
                }
            } else {
                terms_of<AC, GRAD>(p, min(i, hi - 1), valid, s[u], mean, scale, &pg, &v, &h);
            }
            float* slot = acc + (mbi[u] * 3) * THREADS + t;
            slot[0] += valid ? pg : 0.0f;
            slot[THREADS] += valid ? v : 0.0f;
            slot[2 * THREADS] += valid ? h : 0.0f;
        }
    }
    __syncthreads();
    // Each slot row j < num_mb * 3 is summed over the threads in order: with enough threads, as four
    // quarter sums (threads 4j .. 4j + 3, consecutive lanes of one wave) added left to right.
    constexpr int Q = THREADS >= 4 * NB * 3 ? 4 : 1;
    if constexpr (Q == 4) {
        const int j = t >> 2, q = t & 3;
        double sum = 0.0;
        if (j < p.num_mb * 3) {
            const float* row = acc + j * THREADS + q * (THREADS / 4);
            for (int u = 0; u < THREADS / 4; ++u) sum += (double)row[u];
        }
        const int first = (t & 63) & ~3;
        const double q0 = __shfl(sum, first, 64), q1 = __shfl(sum, first + 1, 64);
        const double q2 = __shfl(sum, first + 2, 64), q3 = __shfl(sum, first + 3, 64);
        if (j < p.num_mb * 3 && q == 0)
            p.partials[((int64_t)(j / 3) * gridDim.x + blockIdx.x) * 3 + (j % 3)] = ((q0 + q1) + q2) + q3;
    } else {
        for (int j = t; j < p.num_mb * 3; j += THREADS) {
            const float* row = acc + j * THREADS;
            double sum = 0.0;
            for (int u = 0; u < THREADS; ++u) sum += (double)row[u];
            p.partials[((int64_t)(j / 3) * gridDim.x + blockIdx.x) * 3 + (j % 3)] = sum;
        }
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
    block_sum3(a, b, c, lds);
    if (threadIdx.x == 0) {
        const double inv = 1.0 / (double)mb;
        const double pg = a * inv, v = b * inv, h = c * inv;
        out[4 * m + 0] = (float)pg;
        out[4 * m + 1] = (float)v;
        out[4 * m + 2] = (float)h;
        out[4 * m + 3] = (float)(pg + (double)vf * v - (double)ent * h);
    }
}

// Each sample's minibatch number from a permutation: ids[perm[m*mb + k]] = m. Grid (blocks per minibatch,
// minibatches), so the minibatch is the block's. Entries outside [0, B) are clamped into it, so every write
// stays in the array (a permutation writes each entry exactly once).
__global__ __launch_bounds__(256) void k_perm_to_index(const int32_t* __restrict__ perm, int64_t B, int64_t mb,
                                                       uint16_t* __restrict__ ids)
{
    const int64_t base = (int64_t)blockIdx.y * mb;
    const uint16_t m = (uint16_t)blockIdx.y;
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < mb; k += (int64_t)gridDim.x * blockDim.x)
        ids[min(max((int64_t)perm[base + k], (int64_t)0), B - 1)] = m;
}

int blocks_per_mb(int64_t mb)
{
    const int64_t per_block = 256 * kSamplesPerThread;
    return (int)std::max<int64_t>(1, std::min<int64_t>((mb + per_block - 1) / per_block, kMaxBlocksPerMb));
}

constexpr int kStreamMaxMinibatches = 64;
// The stream variants of 32 and 64 minibatches hold 48 KB of LDS per block, so a CU keeps 3 blocks and 768
// blocks are one resident round on 256 CUs: no tail round of partly filled CUs. The 16-minibatch variant
// (384 threads) holds 72 KB, with its chunk's 4-bit minibatch numbers 80 KB: 2 blocks a CU, 512 a round.
constexpr int kStreamBlocks = 768;
constexpr int kStreamBlocks16 = 512;

// Bytes of the per-block partials at the front of the workspace (rounded up to 256, where a perm's
// conversion follows).
size_t partial_bytes(int64_t num_mb, size_t blocks)
{
    return rl::round_up(sizeof(double) * 3 * (size_t)num_mb * blocks, 256);
}

// Each thread adds at most this many samples into its float32 slots (the slot sums are then reduced in
// float64), which bounds their rounding error at kSlotSamples * 2^-24 (1.5e-5) of the summed magnitudes
// at any B.
constexpr int64_t kSlotSamples = 256;

// Threads per stream-mode block: the per-thread slots of 16 / 32 / 64 minibatches fill 72 / 48 / 48 KB of LDS.
int stream_threads(int64_t num_mb) { return num_mb <= 16 ? 384 : (num_mb <= 32 ? 128 : 64); }

// Stream-mode grid: blocks of `chunk` samples. Up to 16 minibatches, whole rounds of kStreamBlocks16
// blocks of at most kBinCap samples (so that a chunk is a bin of the perm conversion, and a thread takes at
// most 43 samples); else kStreamBlocks blocks (one resident round) unless a chunk would give a thread more
// than kSlotSamples samples.
int stream_blocks(int64_t B, int64_t num_mb, int64_t* chunk)
{
    int64_t c;
    if (num_mb <= 16) {
        const int64_t per_round = (int64_t)kStreamBlocks16 * kBinCap;
        const int64_t rounds = (B + per_round - 1) / per_round;
        c = std::max<int64_t>(256, (B + kStreamBlocks16 * rounds - 1) / (kStreamBlocks16 * rounds));
    } else {
        c = std::min<int64_t>(std::max<int64_t>(256, (B + kStreamBlocks - 1) / kStreamBlocks),
                              stream_threads(num_mb) * kSlotSamples);
    }
    *chunk = c;
    return (int)((B + c - 1) / c);
}

// How a perm becomes minibatch numbers (at most 64 minibatches): the sort with the stream pass placing its
// own chunk's numbers (up to 16 minibatches; bins are the stream chunks), the sort and k_perm_place_runs
// (bins of kBinCap), or past 2^24 samples the direct scatter.
enum PermKind { kPermDirect, kPermPlaced, kPermInStream };

struct PermPlan {
    PermKind kind;
    int64_t rows, bins, S;
};

PermPlan perm_plan(int64_t B, int64_t num_mb)
{
    PermPlan q{kPermDirect, (B + kSortPositions - 1) / kSortPositions, 0, 0};
    if (B > ((int64_t)1 << 24)) return q;
    if (num_mb <= 16) {
        q.kind = kPermInStream;
        q.bins = stream_blocks(B, num_mb, &q.S);
    } else {
        q.kind = kPermPlaced;
        q.S = kBinCap;
        q.bins = (B + kBinCap - 1) / kBinCap;
    }
    return q;
}

// Bytes behind the partials for a perm's conversion: the 2-byte minibatch numbers (unless the stream pass
// places them itself), then for the sort its starts rows and staging rows.
size_t perm_bytes(int64_t B, int64_t num_mb)
{
    const PermPlan q = perm_plan(B, num_mb);
    size_t bytes = q.kind == kPermInStream ? 0 : rl::round_up(sizeof(uint16_t) * (size_t)B, 256);
    if (q.kind != kPermDirect)
        bytes += rl::round_up(sizeof(int32_t) * (size_t)(q.rows * (q.bins + 1)), 256) +
                 sizeof(uint32_t) * (size_t)(q.rows * kStagingStride);
    return bytes;
}

}  // namespace

extern "C" {

int rl_ppo_loss_workspace_bytes(int64_t B, int32_t mb, size_t* bytes)
{
    if (B < 1 || mb < 1) return rl::fail(RL_EINVAL, "B %lld and mb %d must be >= 1", (long long)B, mb);
    if (B % mb != 0) return rl::fail(RL_EINVAL, "B %lld is not a multiple of mb %d", (long long)B, mb);
    if (!bytes) return rl::fail(RL_EINVAL, "bytes is NULL");
    const int64_t num_mb = B / mb;
    int64_t chunk = 0;
    const size_t blocks = (size_t)std::max(blocks_per_mb(mb), num_mb <= kStreamMaxMinibatches ? stream_blocks(B, num_mb, &chunk) : 0);
    *bytes = partial_bytes(num_mb, blocks);
    // with at most 64 minibatches, room for turning a perm into minibatch numbers
    if (num_mb <= kStreamMaxMinibatches) *bytes += perm_bytes(B, num_mb);
    return RL_OK;
}

}  // extern "C"

namespace {

template <int AC, int NB, int THREADS, int U, bool GRAD, bool MAP = false>
int launch_stream(const LossArgs& p, int64_t chunk, int nblk, hipStream_t st)
{
    auto* k = &k_ppo_loss_stream<AC, NB, THREADS, U, GRAD, MAP>;
    constexpr size_t bytes = stream_lds_bytes(NB, THREADS, MAP);
    hipLaunchKernelGGL(k, dim3(nblk), dim3(THREADS), bytes, st, p, chunk);
    return RL_OK;
}

template <bool GRAD>
int launch_loss(const LossArgs& p, int64_t num_mb, int A, bool stream_mode, bool map, int64_t chunk, int nblk,
                hipStream_t st)
{
    if (stream_mode) {
        // With 64 minibatches a CU holds 3 one-wave blocks, so each thread loads 4 samples ahead; with
        // 12 waves per CU (16 or 32 minibatches) the loads of one sample per thread already keep HBM busy.
        if (num_mb <= 16) {
            if (map) return A == 12 ? launch_stream<12, 16, 384, 1, GRAD, true>(p, chunk, nblk, st)
                                    : launch_stream<0, 16, 384, 1, GRAD, true>(p, chunk, nblk, st);
            return A == 12 ? launch_stream<12, 16, 384, 1, GRAD>(p, chunk, nblk, st)
                           : launch_stream<0, 16, 384, 1, GRAD>(p, chunk, nblk, st);
        }
        if (num_mb <= 32)
            return A == 12 ? launch_stream<12, 32, 128, 1, GRAD>(p, chunk, nblk, st)
                           : launch_stream<0, 32, 128, 1, GRAD>(p, chunk, nblk, st);
        return A == 12 ? launch_stream<12, 64, 64, 4, GRAD>(p, chunk, nblk, st)
                       : launch_stream<0, 64, 64, 1, GRAD>(p, chunk, nblk, st);
    }
    const dim3 grid(nblk, (unsigned)num_mb);
    if (A == 12) hipLaunchKernelGGL((k_ppo_loss<12, GRAD>), grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL((k_ppo_loss<0, GRAD>), grid, dim3(256), 0, st, p);
    return RL_OK;
}

// Workspace bytes one call needs: the partials, and the perm's conversion only when a perm is given
// (rl_ppo_loss_workspace_bytes covers both).
int call_workspace_bytes(int64_t B, int32_t mb, bool with_perm, size_t* bytes)
{
    if (int rc = rl_ppo_loss_workspace_bytes(B, mb, bytes)) return rc;
    const int64_t num_mb = B / mb;
    if (!with_perm && num_mb <= kStreamMaxMinibatches) *bytes -= perm_bytes(B, num_mb);
    return RL_OK;
}

int ppo_loss_impl(const float* logits, const int32_t* actions, const float* old_logp, const float* adv,
                  const float* ret, const float* new_values, const int32_t* perm, const uint16_t* mb_index,
                  const double* adv_stats, int64_t B, int32_t A, int32_t mb, float clip_eps, float vf_coef,
                  float ent_coef, float* out, float* dlogits, float* dvalues, void* ws, size_t ws_bytes, void* stream)
{
    size_t need = 0;
    if (int rc = call_workspace_bytes(B, mb, perm != nullptr, &need)) return rc;
    if (A < 1 || A > 64) return rl::fail(RL_EINVAL, "A %d outside [1, 64]", A);
    if (B * (int64_t)A > ((int64_t)1 << 40)) return rl::fail(RL_EINVAL, "B*A too large");
    if (!logits || !actions || !old_logp || !adv || !ret || !new_values || !out || !ws)
        return rl::fail(RL_EINVAL, "logits, actions, old_logp, adv, ret, new_values, out and ws must be non-NULL");
    if (!(clip_eps >= 0.0f)) return rl::fail(RL_EINVAL, "clip_eps must be >= 0");
    const void* ptrs[] = {logits, actions, old_logp, adv, ret, new_values, out};
    for (const void* q : ptrs)
        if (!rl::aligned(q, 4)) return rl::fail(RL_EALIGN, "an array is not 4-byte aligned");
    if (perm && !rl::aligned(perm, 4)) return rl::fail(RL_EALIGN, "perm is not 4-byte aligned");
    if (perm && mb_index) return rl::fail(RL_EINVAL, "pass perm or mb_index, not both");
    if (mb_index && !rl::aligned(mb_index, 2)) return rl::fail(RL_EALIGN, "mb_index is not 2-byte aligned");
    if (mb_index && B / mb > kStreamMaxMinibatches)
        return rl::fail(RL_EINVAL, "mb_index supports at most %d minibatches, got %lld", kStreamMaxMinibatches,
                        (long long)(B / mb));
    if (A % 4 == 0 && !rl::aligned(logits, 16)) return rl::fail(RL_EALIGN, "logits must be 16-byte aligned when A %% 4 == 0");
    if (dlogits) {
        if (!rl::aligned(dlogits, 4) || !rl::aligned(dvalues, 4))
            return rl::fail(RL_EALIGN, "dlogits / dvalues are not 4-byte aligned");
        if (A % 4 == 0 && !rl::aligned(dlogits, 16))
            return rl::fail(RL_EALIGN, "dlogits must be 16-byte aligned when A %% 4 == 0");
    }
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
    p.mb_index = mb_index;
    p.B = B;
    p.num_mb = (int)num_mb;
    p.dlogits = dlogits;
    p.dvalues = dvalues;
    p.inv_mb = (float)(1.0 / (double)mb);
    p.dv_coef = (float)(2.0 * (double)vf_coef / (double)mb);
    hipStream_t st = rl::as_stream(stream);
    p.runs = PermRuns{nullptr, nullptr, 0, 0};
    bool map = false;
    if (perm && num_mb <= kStreamMaxMinibatches) {
        // the perm's sets as minibatch numbers (behind the partials), then the stream pass
        int64_t c = 0;
        const size_t blocks = (size_t)std::max(blocks_per_mb(mb), stream_blocks(B, num_mb, &c));
        uint8_t* w = static_cast<uint8_t*>(ws) + partial_bytes(num_mb, blocks);
        const PermPlan q = perm_plan(B, num_mb);
        uint16_t* ids = nullptr;
        if (q.kind != kPermInStream) {
            ids = reinterpret_cast<uint16_t*>(w);
            w += rl::round_up(sizeof(uint16_t) * (size_t)B, 256);
        }
        if (q.kind == kPermDirect) {
            hipLaunchKernelGGL(k_perm_to_index, dim3((unsigned)blocks_per_mb(mb), (unsigned)num_mb), dim3(256), 0, st,
                               perm, B, (int64_t)mb, ids);
        } else {
            int32_t* starts = reinterpret_cast<int32_t*>(w);
            uint32_t* staging = reinterpret_cast<uint32_t*>(w + rl::round_up(sizeof(int32_t) * (size_t)(q.rows * (q.bins + 1)), 256));
            hipLaunchKernelGGL(k_perm_sort, dim3((unsigned)q.rows), dim3(kSortThreads), kSortLdsBytes, st, perm, (int32_t)B,
                               (int32_t)mb, (float)(1.0 / (double)mb), (int32_t)q.S, (float)(1.0 / (double)q.S),
                               (int)q.bins, starts, staging);
            p.runs = PermRuns{starts, staging, (int)q.rows, (int)q.bins};
            if (q.kind == kPermPlaced)
                hipLaunchKernelGGL(k_perm_place_runs, dim3((unsigned)q.bins), dim3(512), 0, st, p.runs, B, ids);
        }
        if (int rc = rl::check_launch("ppo_loss perm")) return rc;
        map = q.kind == kPermInStream;
        mb_index = ids;
        p.mb_index = ids;
        p.perm = nullptr;
    }
    const bool stream_mode = mb_index != nullptr || map;
    int64_t chunk = 0;
    const int nblk = stream_mode ? stream_blocks(B, num_mb, &chunk) : blocks_per_mb(mb);
    if (int rc = dlogits ? launch_loss<true>(p, num_mb, A, stream_mode, map, chunk, nblk, st)
                         : launch_loss<false>(p, num_mb, A, stream_mode, map, chunk, nblk, st))
        return rc;
    if (int rc = rl::check_launch("ppo_loss")) return rc;
    hipLaunchKernelGGL(k_ppo_finalize, dim3((unsigned)num_mb), dim3(256), 0, st, static_cast<const double*>(ws), nblk,
                       (int64_t)mb, vf_coef, ent_coef, out);
    return rl::check_launch("ppo_finalize");
}

// The no-allocation loss's workspace: a fixed array that every device the library runs on holds from the
// library's load until the process ends. Host code never uses the array's name as an address (on the host
// it names a stand-in, not device memory): the first call on each device looks up that device's copy.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch`, looked up once per device with that device current.
int scratch_on_current_device(void** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return rl::fail(RL_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return rl::fail(RL_EINVAL, "device %d outside [0, %d)", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return rl::fail(RL_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return RL_OK;
}

}  // namespace

extern "C" {

int rl_ppo_loss_noalloc(const float* logits, const int32_t* actions, const float* old_logp, const float* adv,
                        const float* ret, const float* new_values, const int32_t* perm, const uint16_t* mb_index,
                        const double* adv_stats, int64_t B, int32_t A, int32_t mb, float clip_eps, float vf_coef,
                        float ent_coef, float* out, void* stream)
{
    size_t need = 0;
    if (int rc = call_workspace_bytes(B, mb, perm != nullptr, &need)) return rc;
    if (need > kScratchBytes)
        return rl::fail(RL_ESIZE, "this loss needs %zu bytes of workspace, more than the %zu bytes of the fixed device "
                                  "array of rl_ppo_loss_noalloc: call rl_ppo_loss with a workspace",
                        need, kScratchBytes);
    void* ws = nullptr;
    if (int rc = scratch_on_current_device(&ws)) return rc;
    if (stream) {   // the array's address is the current device's: the work must run there
        int cur = -1;
        hipDevice_t sdev = -1;
        if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(rl::as_stream(stream), &sdev) != hipSuccess)
            return rl::fail(RL_EHIP, "could not query the current device or the stream's device");
        if (sdev != cur)
            return rl::fail(RL_EINVAL, "stream belongs to device %d, the current device is %d", (int)sdev, cur);
    }
    return ppo_loss_impl(logits, actions, old_logp, adv, ret, new_values, perm, mb_index, adv_stats, B, A, mb, clip_eps,
                         vf_coef, ent_coef, out, nullptr, nullptr, ws, kScratchBytes, stream);
}

int rl_ppo_loss(const float* logits, const int32_t* actions, const float* old_logp, const float* adv, const float* ret,
                const float* new_values, const int32_t* perm, const uint16_t* mb_index, const double* adv_stats,
                int64_t B, int32_t A, int32_t mb, float clip_eps, float vf_coef, float ent_coef, float* out, void* ws,
                size_t ws_bytes, void* stream)
{
    return ppo_loss_impl(logits, actions, old_logp, adv, ret, new_values, perm, mb_index, adv_stats, B, A, mb, clip_eps,
                         vf_coef, ent_coef, out, nullptr, nullptr, ws, ws_bytes, stream);
}

int rl_ppo_loss_grad(const float* logits, const int32_t* actions, const float* old_logp, const float* adv,
                     const float* ret, const float* new_values, const int32_t* perm, const uint16_t* mb_index,
                     const double* adv_stats, int64_t B, int32_t A, int32_t mb, float clip_eps, float vf_coef,
                     float ent_coef, float* out, float* dlogits, float* dvalues, void* ws, size_t ws_bytes,
                     void* stream)
{
    if (!dlogits || !dvalues) return rl::fail(RL_EINVAL, "dlogits and dvalues must be non-NULL");
    return ppo_loss_impl(logits, actions, old_logp, adv, ret, new_values, perm, mb_index, adv_stats, B, A, mb, clip_eps,
                         vf_coef, ent_coef, out, dlogits, dvalues, ws, ws_bytes, stream);
}

}  // extern "C"
