// Floors of the memory system for the decode workloads, measured beside the attention
// kernels: what a launch of a given grid costs with no work, what a plain read of a
// workload's bytes costs with the same grid, the same read followed by one cross-workgroup
// merge of the split-KV kernel's shape (device-scope partial stores, a wait for their
// completion, an arrival counter, the last workgroup reading every partial back), and a
// read of randomly placed 2 KB blocks through a page table (the paged int8 cache's K and V
// blocks), and the LDS read bandwidth that the forward kernels' fragment reads draw on.
// Measurement probes: they compute nothing of the attention method, and the
// attention library neither links nor calls them.  Built into libattn_floors.so.
//
// Every entry point validates its sizes on the host, and every kernel bounds its accesses
// by the sizes it was given.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 512;
constexpr int kPartFloats = 4 * 130;     // one split partial of the headline decode: 4 heads x (128 + m + l)

__global__ void __launch_bounds__(kThreads) floor_empty_kernel() {}

// Each workgroup reads per_wg 16-byte words starting at blockIdx.x * per_wg, up to sixteen
// loads in flight per thread; one value per wave leaves the kernel so that the loads are kept.
__device__ __forceinline__ uint32_t read_range(const uint4* __restrict__ p, long n) {
    constexpr int U = 16;
    uint32_t a = 0;
    for (long i = threadIdx.x; i < n; i += U * kThreads) {
        uint4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const long j = i + (long)u * kThreads;
            x[u] = j < n ? p[j] : make_uint4(0, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);     // every load issued before the first use
#pragma unroll
        for (int u = 0; u < U; ++u) a ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
    }
    return a;
}

__device__ __forceinline__ uint32_t wave_xor(uint32_t v) {
    for (int m = 32; m >= 1; m >>= 1) v ^= (uint32_t)__shfl_xor((int)v, m, 64);
    return v;
}

__global__ void __launch_bounds__(kThreads) floor_stream_kernel(const uint4* __restrict__ src, long per_wg,
                                                                float* __restrict__ sink) {
    const uint32_t v = wave_xor(read_range(src + (long)blockIdx.x * per_wg, per_wg));
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = (float)(v & 0xffff);
}

// grid (splits, groups): workgroup (s, g) reads range g * splits + s, publishes a partial,
// and the last of the group's splits to arrive sums the group's partials into out[g].
__global__ void __launch_bounds__(kThreads) floor_stream_merge_kernel(const uint4* __restrict__ src, long per_wg,
                                                                      float* __restrict__ part,
                                                                      uint32_t* __restrict__ tickets,
                                                                      float* __restrict__ out) {
    __shared__ uint32_t wsum[kThreads / 64];
    __shared__ int last;
    const int splits = gridDim.x, s = blockIdx.x, g = blockIdx.y;
    const long r = (long)g * splits + s;
    const uint32_t v = wave_xor(read_range(src + r * per_wg, per_wg));
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t t = 0;
    for (int w = 0; w < kThreads / 64; ++w) t ^= wsum[w];
    for (int i = threadIdx.x; i < kPartFloats; i += kThreads)
        __hip_atomic_store(part + r * kPartFloats + i, (float)((t >> (i & 15)) & 1u), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(tickets + g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = prev == (uint32_t)(splits - 1);
        if (last) __hip_atomic_store(tickets + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!last) return;
    // the group's partials, read back with device-scope loads, eight in flight per thread
    for (int i = threadIdx.x; i < kPartFloats; i += kThreads) {
        float a = 0.f;
        int k = 0;
        for (; k + 8 <= splits; k += 8) {
            float x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                x[u] = __hip_atomic_load(part + ((long)g * splits + k + u) * kPartFloats + i, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int u = 0; u < 8; ++u) a += x[u];
        }
        for (; k < splits; ++k)
            a += __hip_atomic_load(part + ((long)g * splits + k) * kPartFloats + i, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        out[(long)g * kPartFloats + i] = a;
    }
}

// Workgroup w reads list entries [w * per_wg, min((w + 1) * per_wg, n)); entry e names the
// 2 KB block blocks[e] (clamped into the pool) of both k and v.  Four blocks per pass:
// thread t reads 16-byte word t % 128 of block t / 128.
__global__ void __launch_bounds__(kThreads) floor_gather_kernel(const uint4* __restrict__ k,
                                                                const uint4* __restrict__ v,
                                                                const uint32_t* __restrict__ blocks, int n,
                                                                int per_wg, uint32_t pool_blocks,
                                                                float* __restrict__ sink) {
    const int e0 = blockIdx.x * per_wg;
    const int e1 = min(n, e0 + per_wg);
    const int word = threadIdx.x & 127, sub = threadIdx.x >> 7;
    uint32_t a = 0;
    for (int e = e0 + sub; e < e1; e += 4) {
        const uint32_t b = min(blocks[e], pool_blocks - 1u);
        const uint4 x = k[(long)b * 128 + word];
        const uint4 y = v[(long)b * 128 + word];
        a ^= x.x ^ x.y ^ x.z ^ x.w ^ y.x ^ y.y ^ y.z ^ y.w;
    }
    a = wave_xor(a);
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = (float)(a & 0xffff);
}

// LDS read bandwidth: each workgroup fills 64 KB of LDS, then every lane reads 16 bytes per
// ds_read_b128 (consecutive lanes at consecutive 16-byte slots: no bank conflicts), four reads
// per iteration, for iters iterations.
template <int NT>
__global__ void __launch_bounds__(NT) floor_lds_kernel(uint32_t* __restrict__ out, int iters) {
    __shared__ __attribute__((aligned(16))) uint4 buf[4096];
    for (int i = threadIdx.x; i < 4096; i += NT) buf[i] = make_uint4(i, i + 1, i + 2, i + 3);
    __syncthreads();
    uint4 a = make_uint4(0, 0, 0, 0), b = a, c = a, d = a;
    const int base = threadIdx.x & 4095;
    for (int it = 0; it < iters; ++it) {
        const int o = (it * 256) & 4095;
        const uint4 x0 = buf[(base + o) & 4095];
        const uint4 x1 = buf[(base + o + 64) & 4095];
        const uint4 x2 = buf[(base + o + 128) & 4095];
        const uint4 x3 = buf[(base + o + 192) & 4095];
        a.x ^= x0.x; a.y ^= x0.y; a.z ^= x0.z; a.w ^= x0.w;
        b.x ^= x1.x; b.y ^= x1.y; b.z ^= x1.z; b.w ^= x1.w;
        c.x ^= x2.x; c.y ^= x2.y; c.z ^= x2.z; c.w ^= x2.w;
        d.x ^= x3.x; d.y ^= x3.y; d.z ^= x3.z; d.w ^= x3.w;
    }
    out[(long)blockIdx.x * NT + threadIdx.x] =
        a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
}

// LDS reads of 8 bytes per lane (the width of the transposing reads that feed the V^T operand
// of the forward kernels' P.V products): TR 0 plain ds_read_b64, TR 1 ds_read_b64_tr_b16.
// Lane l reads the 8 bytes at 8 l of a 512-byte span (no bank conflicts for the plain read),
// four spans per iteration; 512 threads.
template <int TR>
__global__ void __launch_bounds__(512) floor_lds64_kernel(uint32_t* __restrict__ out, int iters) {
    typedef short s4_t __attribute__((ext_vector_type(4)));
    __shared__ __attribute__((aligned(16))) uint4 buf[4096];
    for (int i = threadIdx.x; i < 4096; i += 512) buf[i] = make_uint4(i, i + 1, i + 2, i + 3);
    __syncthreads();
    const char* base = reinterpret_cast<const char*>(buf);
    const int lane = threadIdx.x & 63;
    const int wofs = (threadIdx.x >> 6) * 512;
    uint32_t a = 0, b = 0, c = 0, d = 0;
    for (int it = 0; it < iters; ++it) {
        const int o = (it * 2048 + wofs) & 65535;
        uint2 x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const char* addr = base + ((o + 512 * u) & 65535) + 8 * lane;
            if constexpr (TR == 1) {
                const s4_t w = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s4_t*)(uint32_t)(uintptr_t)addr);
                x[u] = __builtin_bit_cast(uint2, w);
            } else {
                x[u] = *reinterpret_cast<const uint2*>(addr);
            }
        }
        a ^= x[0].x ^ x[0].y;
        b ^= x[1].x ^ x[1].y;
        c ^= x[2].x ^ x[2].y;
        d ^= x[3].x ^ x[3].y;
    }
    out[(long)blockIdx.x * 512 + threadIdx.x] = a ^ b ^ c ^ d;
}

int status(hipError_t e) { return e == hipSuccess ? 0 : -4; }

}  // namespace

extern "C" {

// grid workgroups of kThreads threads that do nothing.
int floor_empty(int grid, void* stream) {
    if (grid < 1 || grid > 65535) return -1;
    hipLaunchKernelGGL(floor_empty_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream);
    return status(hipGetLastError());
}

// A plain read of `bytes` bytes from src (16-byte aligned, bytes a multiple of 16 * grid):
// workgroup w reads the w-th of grid equal ranges.  sink: grid * 8 floats.
int floor_stream(const void* src, long bytes, int grid, float* sink, void* stream) {
    if (!src || !sink || grid < 1 || grid > 65535 || bytes <= 0 || bytes % (16L * grid) != 0) return -1;
    if ((uintptr_t)src % 16 != 0) return -1;
    hipLaunchKernelGGL(floor_stream_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                       (const uint4*)src, bytes / 16 / grid, sink);
    return status(hipGetLastError());
}

// The read of floor_stream over splits * groups workgroups, then one merge per group.
// part: groups * splits * 520 floats; tickets: groups zeroed uint32 (left zeroed);
// out: groups * 520 floats.
int floor_stream_merge(const void* src, long bytes, int splits, int groups, float* part,
                       uint32_t* tickets, float* out, void* stream) {
    const long grid = (long)splits * groups;
    if (!src || !part || !tickets || !out || splits < 1 || groups < 1 || splits > 65535 || groups > 65535)
        return -1;
    if (bytes <= 0 || bytes % (16L * grid) != 0 || (uintptr_t)src % 16 != 0) return -1;
    hipLaunchKernelGGL(floor_stream_merge_kernel, dim3(splits, groups), dim3(kThreads), 0, (hipStream_t)stream,
                       (const uint4*)src, bytes / 16 / grid, part, tickets, out);
    return status(hipGetLastError());
}

// Reads the 2 KB blocks blocks[0 .. n) of k and of v (pools of pool_blocks blocks each);
// workgroup w takes entries [w * per_wg, (w + 1) * per_wg).  sink: grid * 8 floats, with
// grid = ceil(n / per_wg).
int floor_gather(const void* k, const void* v, const uint32_t* blocks, int n, int per_wg, long pool_blocks,
                 float* sink, void* stream) {
    if (!k || !v || !blocks || !sink || n < 1 || per_wg < 1 || pool_blocks < 1 || pool_blocks > 0xffffffffL)
        return -1;
    if ((uintptr_t)k % 16 != 0 || (uintptr_t)v % 16 != 0) return -1;
    const long grid = ((long)n + per_wg - 1) / per_wg;
    if (grid > 65535) return -1;
    hipLaunchKernelGGL(floor_gather_kernel, dim3((unsigned)grid), dim3(kThreads), 0, (hipStream_t)stream,
                       (const uint4*)k, (const uint4*)v, blocks, n, per_wg, (uint32_t)pool_blocks, sink);
    return status(hipGetLastError());
}

// LDS reads of 64 * 8 bytes per wave-instruction, plain (tr 0) or transposing (tr 1): grid
// workgroups of 512 threads, 4 * iters reads per lane.  out: grid * 512 uint32.
int floor_lds_read64(int grid, int tr, int iters, uint32_t* out, void* stream) {
    if (!out || grid < 1 || grid > 65535 || iters < 1 || (tr != 0 && tr != 1)) return -1;
    const hipStream_t st = (hipStream_t)stream;
    if (tr == 1)
        hipLaunchKernelGGL(floor_lds64_kernel<1>, dim3(grid), dim3(512), 0, st, out, iters);
    else
        hipLaunchKernelGGL(floor_lds64_kernel<0>, dim3(grid), dim3(512), 0, st, out, iters);
    return status(hipGetLastError());
}

// LDS reads of 64 * 16 bytes per wave-instruction: grid workgroups of threads (256, 512 or
// 1024) threads, 4 * iters reads per lane.  out: grid * threads uint32.
int floor_lds_read(int grid, int threads, int iters, uint32_t* out, void* stream) {
    if (!out || grid < 1 || grid > 65535 || iters < 1) return -1;
    const hipStream_t st = (hipStream_t)stream;
    if (threads == 256)
        hipLaunchKernelGGL(floor_lds_kernel<256>, dim3(grid), dim3(256), 0, st, out, iters);
    else if (threads == 512)
        hipLaunchKernelGGL(floor_lds_kernel<512>, dim3(grid), dim3(512), 0, st, out, iters);
    else if (threads == 1024)
        hipLaunchKernelGGL(floor_lds_kernel<1024>, dim3(grid), dim3(1024), 0, st, out, iters);
    else
        return -1;
    return status(hipGetLastError());
}

}  // extern "C"
