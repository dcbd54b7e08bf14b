// Plain store and load kernels for the rooflines: traffic of a stated granularity whose bandwidth, measured
// in the same run as the path's kernels, is the write or read ceiling for that granularity. Not part of the
// rollout path.
//
// Each block of 256 threads writes one chunk of `chunk` bytes with 16-byte stores (chunk i covers bytes
// [i chunk, (i + 1) chunk) of the buffer), so the chunk is the amount of contiguous output one block
// produces before it exits: the env step's blocks write 16 observation rows of 5588 bytes (89408 bytes),
// a device fill writes a few KB per block. On MI355X the rate depends strongly on this granularity.

#include "rl_internal.hpp"

namespace {

__global__ __launch_bounds__(256) void k_store_chunks(float4* __restrict__ out, int64_t nq, int64_t per)
{
    const int64_t lo = (int64_t)blockIdx.x * per;
    const int64_t hi = lo + per < nq ? lo + per : nq;
    for (int64_t q = lo + threadIdx.x; q < hi; q += 256) out[q] = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
}

// Each block reads one chunk with 16-byte loads, four in flight per thread, and folds the words by XOR. The
// fold goes to *sink only when it equals a fixed constant (so the loads cannot be dropped, and a buffer of
// zeros never writes).
__global__ __launch_bounds__(256) void k_read_chunks(const uint4* __restrict__ in, int64_t nq, int64_t per,
                                                     uint32_t* __restrict__ sink)
{
    const int64_t lo = (int64_t)blockIdx.x * per;
    const int64_t hi = lo + per < nq ? lo + per : nq;
    uint32_t acc = 0;
    int64_t q = lo + threadIdx.x;
    for (; q + 3 * 256 < hi; q += 4 * 256) {
        const uint4 a = in[q], b = in[q + 256], c = in[q + 512], d = in[q + 768];
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; q < hi; q += 256) {
        const uint4 a = in[q];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == 0x9E3779B9u) *sink = acc;
}

}  // namespace

extern "C" int rl_read_probe(const void* buf, int64_t bytes, int64_t chunk, uint32_t* sink, void* stream)
{
    if (!buf || !sink) return rl::fail(RL_EINVAL, "buf and sink must be non-NULL");
    if (!rl::aligned(buf, 16) || !rl::aligned(sink, 4)) return rl::fail(RL_EALIGN, "buf / sink misaligned");
    if (bytes < 16 || bytes % 16 != 0 || chunk < 16 || chunk % 16 != 0)
        return rl::fail(RL_EINVAL, "bytes %lld and chunk %lld must be positive multiples of 16", (long long)bytes,
                        (long long)chunk);
    const int64_t nq = bytes / 16, per = chunk / 16;
    const int64_t blocks = (nq + per - 1) / per;
    if (blocks > (int64_t)1 << 31) return rl::fail(RL_EINVAL, "more than 2^31 chunks");
    hipLaunchKernelGGL(k_read_chunks, dim3((unsigned)blocks), dim3(256), 0, rl::as_stream(stream),
                       static_cast<const uint4*>(buf), nq, per, sink);
    return rl::check_launch("read_probe");
}

extern "C" int rl_store_probe(void* buf, int64_t bytes, int64_t chunk, void* stream)
{
    if (!buf) return rl::fail(RL_EINVAL, "buf is NULL");
    if (!rl::aligned(buf, 16)) return rl::fail(RL_EALIGN, "buf is not 16-byte aligned");
    if (bytes < 16 || bytes % 16 != 0 || chunk < 16 || chunk % 16 != 0)
        return rl::fail(RL_EINVAL, "bytes %lld and chunk %lld must be positive multiples of 16", (long long)bytes,
                        (long long)chunk);
    const int64_t nq = bytes / 16, per = chunk / 16;
    const int64_t blocks = (nq + per - 1) / per;
    if (blocks > (int64_t)1 << 31) return rl::fail(RL_EINVAL, "more than 2^31 chunks");
    hipLaunchKernelGGL(k_store_chunks, dim3((unsigned)blocks), dim3(256), 0, rl::as_stream(stream),
                       static_cast<float4*>(buf), nq, per);
    return rl::check_launch("store_probe");
}
