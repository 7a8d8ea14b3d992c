// Conformer block-local attention with a relative-position term, for gfx950, f32.
//
// The pages give the call (rullama 0.5.0, src/backend/dispatch/attention.rs,
// block_local_attention_chained): Q already projected and scaled per dimension, K and V
// zero padded by pad_left rows in front, a positional projection pos_proj of max_span rows,
// queries grouped in chunks of chunk_size that attend over a context of context_size keys
// (max_past before, max_future after), an optional logit cap, head_dim 128.  The reading
// implemented: query i sees key position t iff i - max_past <= t <= i + max_future and
// 0 <= t < seq; score q_i.k_t + q_i.pos_proj[t - i + max_past], capped c tanh(s / c) when
// c > 0; softmax over the visible keys; rows without a visible key are zeros.  With the
// consistent geometry (context = chunk + past + future, span = past + future + 1, pad_left
// = past) the chunks only decide which rows a kernel stages, so the kernel tiles the
// queries as suits the hardware instead.
//
// Work decomposition: a workgroup owns 32 consecutive query rows of one head (16 when the
// span exceeds 20).  Their keys lie in a window of rows + past + future rows, which is
// staged in LDS once (K and V) with the head's pos_proj rows, every load issued before the
// first LDS write; workgroups are placed so that neighbouring row blocks, whose windows
// overlap, run on one XCD.  A 16-lane group owns one query row (each lane 8 of its 128
// dimensions, the query itself in registers), walks the row's span of offsets computing
// q.(k + pos) with a 16-lane butterfly sum, then the softmax and the weighted V rows.  The
// work is a band of at most span keys per query, a few thousand FLOP per output row: the
// kernel is bound by moving Q, K, V and O, not by arithmetic, so it runs on the vector ALU
// with no matrix products.

#include "device_common.hpp"
#include "launch.hpp"

namespace ta03 {

namespace {

constexpr int kBlD = 128;                 // head_dim (the pages fix it)
constexpr int kBlStride = kBlD + 4;       // LDS row stride in floats (shifts rows across banks)
constexpr int kBlMaxSpan = 29;            // past + future + 1 <= 29: the K and V windows of 16
                                          // queries and the pos_proj rows fit 64 KB of LDS
constexpr int kBlWideSpan = 20;           // spans up to 20 run 32 queries per workgroup

// LDS floats of a workgroup of ROWS query rows
template <int ROWS>
constexpr int bl_lds_floats(int span) { return kBlStride * (2 * (ROWS + span - 1) + span); }

template <int ROWS, bool CAP>
__global__ void __launch_bounds__(16 * ROWS) block_local_kernel(BlockLocalParams a) {
    constexpr int kBlRows = ROWS;                  // query rows per workgroup (one per 16-lane group)
    constexpr int MAXS = ROWS == 32 ? kBlWideSpan : kBlMaxSpan;   // largest span of this shape
    constexpr int NT = 16 * ROWS;
    extern __shared__ __attribute__((aligned(16))) float bl_lds[];
    const int span = a.max_past + a.max_future + 1;
    const int nwin = kBlRows + span - 1;           // window rows of this workgroup
    float* kw = bl_lds;                            // [nwin][stride]
    float* vw = kw + nwin * kBlStride;             // [nwin][stride]
    float* pw = vw + nwin * kBlStride;             // [span][stride]

    // XCD-aware placement: workgroup ids are dealt to the eight XCDs in turn, so give each XCD
    // a contiguous range of (head, row block) items; neighbouring row blocks, whose windows
    // overlap by span - 1 rows, then share an L2
    const int n = gridDim.x;
    const int id = blockIdx.x;
    const int xcd = id & 7, kk = id >> 3, q8 = n >> 3, r8 = n & 7;
    const int item = (xcd < r8 ? xcd * (q8 + 1) : r8 * (q8 + 1) + (xcd - r8) * q8) + kk;
    const int nrb = (a.padded_len + kBlRows - 1) / kBlRows;
    const int head = item / nrb;
    const int i0 = (item % nrb) * kBlRows;
    const int w0 = i0 - a.max_past;                // position of window row 0
    const long hid = (long)a.H * kBlD;             // floats per row of every tensor
    const int tid = threadIdx.x;

    // ---- this lane's query row and dimensions: row g = tid / 16, d in 4 l + {0..3}, 64 + 4 l + {0..3}
    const int g = tid >> 4;
    const int l = tid & 15;
    const int qi = i0 + g;
    const bool live = qi < a.padded_len;
    float4 q0 = {0.f, 0.f, 0.f, 0.f}, q1 = {0.f, 0.f, 0.f, 0.f};
    if (live) {
        const float* qrow = a.q + (long)qi * hid + (long)head * kBlD;
        q0 = *reinterpret_cast<const float4*>(qrow + 4 * l);
        q1 = *reinterpret_cast<const float4*>(qrow + 64 + 4 * l);
    }
    // ---- stage the window's K and V rows and pos_proj: every load of the workgroup's share
    // is issued before the first LDS write, so the staging costs one memory round trip; rows
    // of positions outside [0, seq) are never read from memory and hold zeros in LDS (their
    // scores are masked, and a zero V row keeps the weighted sum finite)
    constexpr int KV_IT = ((kBlRows + MAXS - 1) * (kBlD / 4) + NT - 1) / NT;
    constexpr int P_IT = (MAXS * (kBlD / 4) + NT - 1) / NT;
    float4 kst[KV_IT], vst[KV_IT], pst[P_IT];
#pragma unroll
    for (int u = 0; u < KV_IT; ++u) {
        const int c = tid + u * NT;
        const int r = c / (kBlD / 4), d4 = c % (kBlD / 4);
        const int t = w0 + r;
        kst[u] = float4{0.f, 0.f, 0.f, 0.f};
        vst[u] = kst[u];
        if (r < nwin && t >= 0 && t < a.seq) {
            const long gofs = (long)(t + a.pad_left) * hid + (long)head * kBlD + 4 * d4;
            kst[u] = *reinterpret_cast<const float4*>(a.k + gofs);
            vst[u] = *reinterpret_cast<const float4*>(a.v + gofs);
        }
    }
#pragma unroll
    for (int u = 0; u < P_IT; ++u) {
        const int c = tid + u * NT;
        const int r = c / (kBlD / 4), d4 = c % (kBlD / 4);
        pst[u] = float4{0.f, 0.f, 0.f, 0.f};
        if (r < span) pst[u] = *reinterpret_cast<const float4*>(a.pos + (long)r * hid + (long)head * kBlD + 4 * d4);
    }

#pragma unroll
    for (int u = 0; u < KV_IT; ++u) {
        const int c = tid + u * NT;
        const int r = c / (kBlD / 4), d4 = c % (kBlD / 4);
        if (r < nwin) {
            *reinterpret_cast<float4*>(kw + r * kBlStride + 4 * d4) = kst[u];
            *reinterpret_cast<float4*>(vw + r * kBlStride + 4 * d4) = vst[u];
        }
    }
#pragma unroll
    for (int u = 0; u < P_IT; ++u) {
        const int c = tid + u * NT;
        const int r = c / (kBlD / 4), d4 = c % (kBlD / 4);
        if (r < span) *reinterpret_cast<float4*>(pw + r * kBlStride + 4 * d4) = pst[u];
    }
    __syncthreads();

    // visible offsets j of this row: t = qi - past + j in [0, seq)
    const int j_lo = max(0, a.max_past - qi);
    const int j_hi = min(span - 1, a.seq - 1 - qi + a.max_past);

    // ---- scores, held by every lane of the group (the butterfly leaves the sum everywhere);
    // every offset of the span is computed (a branch per offset would split the groups of a
    // wave) and the invisible ones are masked to -inf ----------------------------------------
    float s[MAXS];
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < MAXS; ++j) {
        s[j] = -INFINITY;
        if (j < span) {
            const float* kr = kw + (g + j) * kBlStride;
            const float* pr = pw + j * kBlStride;
            const float4 k0 = *reinterpret_cast<const float4*>(kr + 4 * l);
            const float4 k1 = *reinterpret_cast<const float4*>(kr + 64 + 4 * l);
            const float4 p0 = *reinterpret_cast<const float4*>(pr + 4 * l);
            const float4 p1 = *reinterpret_cast<const float4*>(pr + 64 + 4 * l);
            float acc = q0.x * k0.x;
            acc = __builtin_fmaf(q0.y, k0.y, acc);
            acc = __builtin_fmaf(q0.z, k0.z, acc);
            acc = __builtin_fmaf(q0.w, k0.w, acc);
            acc = __builtin_fmaf(q1.x, k1.x, acc);
            acc = __builtin_fmaf(q1.y, k1.y, acc);
            acc = __builtin_fmaf(q1.z, k1.z, acc);
            acc = __builtin_fmaf(q1.w, k1.w, acc);
            float pacc = q0.x * p0.x;
            pacc = __builtin_fmaf(q0.y, p0.y, pacc);
            pacc = __builtin_fmaf(q0.z, p0.z, pacc);
            pacc = __builtin_fmaf(q0.w, p0.w, pacc);
            pacc = __builtin_fmaf(q1.x, p1.x, pacc);
            pacc = __builtin_fmaf(q1.y, p1.y, pacc);
            pacc = __builtin_fmaf(q1.z, p1.z, pacc);
            pacc = __builtin_fmaf(q1.w, p1.w, pacc);
            float x = group_sum<16>(acc + pacc);
            if constexpr (CAP) x = a.cap * tanhf(x * a.inv_cap);
            x = (j >= j_lo && j <= j_hi) ? x : -INFINITY;
            s[j] = x;
            m = fmaxf(m, x);
        }
    }
    if (m == -INFINITY) m = 0.f;      // no visible key: every weight is exp(-inf) = 0

    // ---- softmax over the visible offsets, then the weighted sum of V rows --------------
    float lsum = 0.f;
    float4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < MAXS; ++j) {
        if (j < span) {
            const float p = __builtin_amdgcn_exp2f((s[j] - m) * kLog2e);
            lsum += p;
            const float* vr = vw + (g + j) * kBlStride;
            const float4 v0 = *reinterpret_cast<const float4*>(vr + 4 * l);
            const float4 v1 = *reinterpret_cast<const float4*>(vr + 64 + 4 * l);
            o0.x = __builtin_fmaf(p, v0.x, o0.x);
            o0.y = __builtin_fmaf(p, v0.y, o0.y);
            o0.z = __builtin_fmaf(p, v0.z, o0.z);
            o0.w = __builtin_fmaf(p, v0.w, o0.w);
            o1.x = __builtin_fmaf(p, v1.x, o1.x);
            o1.y = __builtin_fmaf(p, v1.y, o1.y);
            o1.z = __builtin_fmaf(p, v1.z, o1.z);
            o1.w = __builtin_fmaf(p, v1.w, o1.w);
        }
    }
    if (live) {
        const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
        float* orow = a.o + (long)qi * hid + (long)head * kBlD;
        *reinterpret_cast<float4*>(orow + 4 * l) = float4{o0.x * inv, o0.y * inv, o0.z * inv, o0.w * inv};
        *reinterpret_cast<float4*>(orow + 64 + 4 * l) = float4{o1.x * inv, o1.y * inv, o1.z * inv, o1.w * inv};
    }
}

}  // namespace

int block_local_max_span() { return kBlMaxSpan; }
int block_local_head_dim() { return kBlD; }

template <int ROWS>
hipError_t launch_rows(const BlockLocalParams& p, hipStream_t st) {
    const dim3 grid(((p.padded_len + ROWS - 1) / ROWS) * p.H);
    const size_t lds = sizeof(float) * (size_t)bl_lds_floats<ROWS>(p.max_past + p.max_future + 1);
    if (p.cap > 0.f)
        hipLaunchKernelGGL((block_local_kernel<ROWS, true>), grid, dim3(16 * ROWS), lds, st, p);
    else
        hipLaunchKernelGGL((block_local_kernel<ROWS, false>), grid, dim3(16 * ROWS), lds, st, p);
    return hipGetLastError();
}

hipError_t launch_block_local(const BlockLocalParams& p, hipStream_t st) {
    // 32 query rows per workgroup where the window fits 64 KB (half the workgroups, each
    // staging 32 + span - 1 key rows instead of 16 + span - 1 for 16 queries, and for the
    // 3000-frame, 8-head workload one round of resident workgroups: 17.8 against 22.1 us)
    if ((long)((p.padded_len + 15) / 16) * p.H > 0x7fffffffL) return hipErrorInvalidValue;
    static_assert(sizeof(float) * bl_lds_floats<32>(kBlWideSpan) <= 65536, "wide windows fit 64 KB");
    static_assert(sizeof(float) * bl_lds_floats<16>(kBlMaxSpan) <= 65536, "windows fit 64 KB");
    if (p.max_past + p.max_future + 1 <= kBlWideSpan) return launch_rows<32>(p, st);
    return launch_rows<16>(p, st);
}

}  // namespace ta03
