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
// overlap, run on one XCD.  A 16-lane group owns two consecutive query rows (each lane 8 of
// their 128 dimensions, both queries in registers): window row 2g + w is offset w of the
// first row and offset w - 1 of the second, and pos_proj row j is offset j of both, so every
// K, V and pos_proj read from LDS serves the two rows.  The lanes' partial dot products are
// summed by a reduce-scatter that leaves the score of offset l with lane l, so the cap, the
// mask and the exponential run once per score; the weights return to every lane of the
// group by row broadcasts for the weighted sum of V rows.  The work is a band of at most
// span keys per query, a few thousand FLOP per output row: no matrix products.

#include "device_common.hpp"
#include "launch.hpp"

namespace ta03 {

namespace {

constexpr int kBlD = 128;                 // head_dim (the pages fix it)
constexpr int kBlStride = kBlD;           // LDS row stride in floats: unpadded rows read without bank
                                          // conflicts here (a group reads a contiguous 256-byte half
                                          // row; the groups of a wave, rows two apart); a 4-float pad
                                          // or a per-group chunk swizzle cost a third of the LDS cycles
constexpr int kBlMaxSpan = 29;            // past + future + 1 <= 29: the K and V windows of 16
                                          // queries and the pos_proj rows fit 64 KB of LDS
constexpr int kBlWideSpan = 20;           // spans up to 20 run 32 queries per workgroup

// LDS floats of a workgroup of ROWS query rows
template <int ROWS>
constexpr int bl_lds_floats(int span) { return kBlStride * (2 * (ROWS + span - 1) + span); }

// Sums over the 16 lanes of a DPP row of 16 values per lane, scattered: lane l gets the sum
// of value l.  Four exchange steps, each pairing a lane with one that differs in the bit being
// settled (lane ^ 15, ^ 7 inside its half, ^ 2, ^ 1); a lane keeps the half of its values whose
// index has that bit of its own lane number and adds its partner's copy of them.
__device__ __forceinline__ float reduce_scatter16(const float* x, int l) {
    float v8[8], v4[4], v2[2];
    const bool b3 = l & 8, b2 = l & 4, b1 = l & 2, b0 = l & 1;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        v8[i] = (b3 ? x[i + 8] : x[i]) + dpp_f<kDppMirror>(b3 ? x[i] : x[i + 8]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        v4[i] = (b2 ? v8[i + 4] : v8[i]) + dpp_f<kDppHalfMirror>(b2 ? v8[i] : v8[i + 4]);
#pragma unroll
    for (int i = 0; i < 2; ++i)
        v2[i] = (b1 ? v4[i + 2] : v4[i]) + dpp_f<kDppXor2>(b1 ? v4[i] : v4[i + 2]);
    return (b0 ? v2[1] : v2[0]) + dpp_f<kDppXor1>(b0 ? v2[0] : v2[1]);
}

// q.k over this lane's 8 dimensions (d in 4 l + {0..3} and 64 + 4 l + {0..3})
__device__ __forceinline__ float dot8(const float4& q0, const float4& q1, const float4& k0, const float4& k1) {
    float acc = q0.x * k0.x;
    acc = __builtin_fmaf(q0.y, k0.y, acc);
    acc = __builtin_fmaf(q0.z, k0.z, acc);
    acc = __builtin_fmaf(q0.w, k0.w, acc);
    acc = __builtin_fmaf(q1.x, k1.x, acc);
    acc = __builtin_fmaf(q1.y, k1.y, acc);
    acc = __builtin_fmaf(q1.z, k1.z, acc);
    return __builtin_fmaf(q1.w, k1.w, acc);
}

// o += p v over this lane's 8 dimensions
__device__ __forceinline__ void fma8(float4& o0, float4& o1, float p, const float4& v0, const float4& v1) {
    o0.x = __builtin_fmaf(p, v0.x, o0.x);
    o0.y = __builtin_fmaf(p, v0.y, o0.y);
    o0.z = __builtin_fmaf(p, v0.z, o0.z);
    o0.w = __builtin_fmaf(p, v0.w, o0.w);
    o1.x = __builtin_fmaf(p, v1.x, o1.x);
    o1.y = __builtin_fmaf(p, v1.y, o1.y);
    o1.z = __builtin_fmaf(p, v1.z, o1.z);
    o1.w = __builtin_fmaf(p, v1.w, o1.w);
}

// this lane's 8 dimensions of an output row, divided by the row's sum of weights (0 for a row
// without a visible key)
__device__ __forceinline__ void store_row(float* orow, int l, const float4& o0, const float4& o1, float lsum) {
    const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
    *reinterpret_cast<float4*>(orow + 4 * l) = float4{o0.x * inv, o0.y * inv, o0.z * inv, o0.w * inv};
    *reinterpret_cast<float4*>(orow + 64 + 4 * l) = float4{o1.x * inv, o1.y * inv, o1.z * inv, o1.w * inv};
}

template <int ROWS, bool CAP>
__global__ void __launch_bounds__(8 * ROWS) block_local_kernel(BlockLocalParams a) {
    constexpr int kBlRows = ROWS;                  // query rows per workgroup (two per 16-lane group)
    constexpr int MAXS = ROWS == 32 ? kBlWideSpan : kBlMaxSpan;   // largest span of this shape
    constexpr int NT = 8 * ROWS;
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

    // ---- this lane's query rows and dimensions: rows 2 g and 2 g + 1 of the block (g = tid / 16),
    // d in 4 l + {0..3} and 64 + 4 l + {0..3}
    const int g = tid >> 4;
    const int l = tid & 15;
    const int qa = i0 + 2 * g, qb = qa + 1;
    const bool live_a = qa < a.padded_len, live_b = qb < a.padded_len;
    float4 qa0 = {0.f, 0.f, 0.f, 0.f}, qa1 = qa0, qb0 = qa0, qb1 = qa0;
    if (live_a) {
        const float* qrow = a.q + (long)qa * hid + (long)head * kBlD;
        qa0 = *reinterpret_cast<const float4*>(qrow + 4 * l);
        qa1 = *reinterpret_cast<const float4*>(qrow + 64 + 4 * l);
    }
    if (live_b) {
        const float* qrow = a.q + (long)qb * hid + (long)head * kBlD;
        qb0 = *reinterpret_cast<const float4*>(qrow + 4 * l);
        qb1 = *reinterpret_cast<const float4*>(qrow + 64 + 4 * l);
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

    // visible offsets j of each row: t = q - past + j in [0, seq)
    const int ja_lo = max(0, a.max_past - qa), ja_hi = min(span - 1, a.seq - 1 - qa + a.max_past);
    const int jb_lo = max(0, a.max_past - qb), jb_hi = min(span - 1, a.seq - 1 - qb + a.max_past);

    // ---- this lane's share (8 of 128 dimensions) of q.(k + pos) for every offset of the span
    // of both rows.  Window row 2 g + w is offset w of row a and offset w - 1 of row b, and
    // pos_proj row j serves offset j of both, so the two rows share every LDS read.  Offsets
    // past the span stay 0 (masked below). --------------------------------------------------
    constexpr int NR = (MAXS + 15) / 16;           // rounds of 16 offsets
    float pa[16 * NR], pb[16 * NR];
#pragma unroll
    for (int j = 0; j < 16 * NR; ++j) pa[j] = pb[j] = 0.f;
#pragma unroll
    for (int w = 0; w <= MAXS; ++w) {
        if (w <= span) {
            const float* kr = kw + (2 * g + w) * kBlStride;
            const float4 k0 = *reinterpret_cast<const float4*>(kr + 4 * l);
            const float4 k1 = *reinterpret_cast<const float4*>(kr + 64 + 4 * l);
            if (w < MAXS && w < span) pa[w] += dot8(qa0, qa1, k0, k1);
            if (w >= 1) pb[w - 1] += dot8(qb0, qb1, k0, k1);
        }
        if (w < MAXS && w < span) {
            const float* pr = pw + w * kBlStride;
            const float4 p0 = *reinterpret_cast<const float4*>(pr + 4 * l);
            const float4 p1 = *reinterpret_cast<const float4*>(pr + 64 + 4 * l);
            pa[w] += dot8(qa0, qa1, p0, p1);
            pb[w] += dot8(qb0, qb1, p0, p1);
        }
    }

    // ---- the group's sums, one offset per lane (lane l: offset 16 r + l of round r), so the
    // cap, the mask and the exponential run once per score instead of on all 16 lanes --------
    float xa[NR], xb[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const bool any = r == 0 || 16 * r < span;
        xa[r] = any ? reduce_scatter16(pa + 16 * r, l) : 0.f;
        xb[r] = any ? reduce_scatter16(pb + 16 * r, l) : 0.f;
    }
    float ma = -INFINITY, mb = -INFINITY;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int j = 16 * r + l;
        float ya = xa[r], yb = xb[r];
        if constexpr (CAP) {
            ya = a.cap * tanh_accurate(ya * a.inv_cap);
            yb = a.cap * tanh_accurate(yb * a.inv_cap);
        }
        xa[r] = (j >= ja_lo && j <= ja_hi) ? ya : -INFINITY;     // j_hi < span
        xb[r] = (j >= jb_lo && j <= jb_hi) ? yb : -INFINITY;
        ma = fmaxf(ma, xa[r]);
        mb = fmaxf(mb, xb[r]);
    }
    ma = group_max16(ma);
    mb = group_max16(mb);
    if (ma == -INFINITY) ma = 0.f;    // no visible key: every weight is exp(-inf) = 0
    if (mb == -INFINITY) mb = 0.f;
    float la = 0.f, lb = 0.f;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        xa[r] = __builtin_amdgcn_exp2f((xa[r] - ma) * kLog2e);
        xb[r] = __builtin_amdgcn_exp2f((xb[r] - mb) * kLog2e);
        la += xa[r];
        lb += xb[r];
    }
    la = group_sum<16>(la);
    lb = group_sum<16>(lb);

    // ---- the weighted sums of V rows (window row 2 g + w: weight w of row a, w - 1 of row b),
    // each weight taken from the lane that holds it -----------------------------------------
    float4 oa0 = {0.f, 0.f, 0.f, 0.f}, oa1 = oa0, ob0 = oa0, ob1 = oa0;
#pragma unroll
    for (int w = 0; w <= MAXS; ++w) {
        if (w <= span) {
            const float* vr = vw + (2 * g + w) * kBlStride;
            const float4 v0 = *reinterpret_cast<const float4*>(vr + 4 * l);
            const float4 v1 = *reinterpret_cast<const float4*>(vr + 64 + 4 * l);
            if (w < MAXS && w < span) {
                const float p = row_bcast16(xa[w / 16], w % 16);
                fma8(oa0, oa1, p, v0, v1);
            }
            if (w >= 1) {
                const float p = row_bcast16(xb[(w - 1) / 16], (w - 1) % 16);
                fma8(ob0, ob1, p, v0, v1);
            }
        }
    }
    const size_t obase = (size_t)head * kBlD;
    if (live_a) store_row(a.o + (long)qa * hid + obase, l, oa0, oa1, la);
    if (live_b) store_row(a.o + (long)qb * hid + obase, l, ob0, ob1, lb);
}

}  // namespace

int block_local_max_span() { return kBlMaxSpan; }
int block_local_head_dim() { return kBlD; }

template <int ROWS>
hipError_t launch_rows(const BlockLocalParams& p, hipStream_t st) {
    const dim3 grid(((p.padded_len + ROWS - 1) / ROWS) * p.H);
    const size_t lds = sizeof(float) * (size_t)bl_lds_floats<ROWS>(p.max_past + p.max_future + 1);
    if (p.cap > 0.f)
        hipLaunchKernelGGL((block_local_kernel<ROWS, true>), grid, dim3(8 * ROWS), lds, st, p);
    else
        hipLaunchKernelGGL((block_local_kernel<ROWS, false>), grid, dim3(8 * ROWS), lds, st, p);
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
