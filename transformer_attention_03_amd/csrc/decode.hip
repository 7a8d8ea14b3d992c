// Split-KV single-token decode for gfx950.
//
// One query token per sequence attends over a KV cache held either as contiguous f16
// rows ([num_kv_heads][kv_len][D], f32 query) or as 16-token pages of symmetric int8 rows
// with one f32 scale per (token, kv head) (doppler gpu/kernels/attention.js: the _f16kv
// decode variants take f32 Q with f16 K/V; executeAttentionTieredQuant reads packed int8
// K/V with separate K and V scale buffers and requires f32 Q; kvLayout "paged" with
// pageSize and a page table; kvLenSource = 1 reads kvLen from a buffer).
//
// Work decomposition (ours, not the pages'): grid (split, kv head x head chunk, batch).
// A workgroup owns GC query heads that share one KV head (the K/V rows are read once for
// all of them) and a contiguous logical token range.  Each of its NW waves streams blocks
// of TB tokens (4 KB of K and 4 KB of V per block), with the loads of the next block
// issued before the current one is processed (register double buffering):
//   K phase: LPT = D/16 lanes per K row, 16 elements per lane, 128-bit loads; the partial
//            dot products for the GC heads are summed across the LPT lanes with DPP.
//   softmax: the block max per head is reduced across the wave; the running maximum is
//            only moved (and the accumulators rescaled) when the block max exceeds it by
//            more than 2^8, so most blocks skip the rescale; exp2 of each (token, head)
//            score is evaluated once, by one lane, and parked in LDS.
//   V phase: V rows are read fully coalesced (one 16-byte chunk per lane), and each lane
//            accumulates p * v for the GC heads over its fixed chunk.
// The waves of a workgroup are merged through LDS; the workgroups of one (sequence, KV
// head) are merged by the last one to arrive (log-sum-exp over the split partials),
// counted with a device-scope atomic that this last workgroup resets to zero.  Partials
// travel through device-scope stores and loads, so no cache-wide fence is needed.
//
// Paged addressing is integer-exact: physical page = page_table[b][t >> 4], slot t & 15,
// row ((page * 16 + slot) * Hkv + kvh) * D.  Rows at or past kv_len are never loaded, so
// poisoned slots of a partial last page cannot reach the result.

#include "device_common.hpp"
#include "launch.hpp"

namespace ta03 {

namespace {

constexpr int kDecodeWaves = 8;
constexpr int kMaxSplits = 256;          // split partials merged per (sequence, head)
constexpr int kMaxSplitTokens = 4096;    // paged: tokens per workgroup (page slice in LDS)
constexpr float kRescaleSlack = 8.0f;    // log2 units: accumulators may grow to 2^8

template <int D, int GC, bool PAGED>
struct DecodeShape {
    static constexpr int ESZ = PAGED ? 1 : 2;          // bytes per K/V element
    static constexpr int LPT = D / 16;                  // K-phase lanes per row
    static constexpr int RPW = 64 / LPT;                // K rows per wave-load
    static constexpr int TB = 4096 / (D * 2);           // tokens per wave block (f16: 4 KB of K)
    static constexpr int U = TB / RPW;                  // K row-sets per block
    static constexpr int KCH = ESZ;                     // 16-byte chunks per lane per K row
    static constexpr int EV = 8;                        // elements per lane per V row
    static constexpr int CPR = D / EV;                  // lanes per V row (8-element chunks)
    static constexpr int VR = 64 / CPR;                 // V rows per wave-load
    static constexpr int NVL = TB / VR;                 // V loads per lane per block
    static_assert(LPT >= 4 && LPT <= 16, "head_dim");
    static_assert(GC <= 4, "heads per workgroup");
    static_assert(U >= 1 && TB % RPW == 0 && TB % VR == 0, "block shape");
};

template <int D, int GC, bool PAGED>
struct BlockRegs {
    using S = DecodeShape<D, GC, PAGED>;
    uint4 k[S::U][S::KCH];
    float ks[S::U];     // K scale of the K-phase row (paged)
    float vs[S::U];     // V scale of the same row (paged)
    // f16: 16-byte chunks (8 halves); int8: 8-byte chunks (8 bytes) in .x, .y
    uint4 v[S::NVL];
};

__device__ __forceinline__ int clamp_page(int p, int num_pages) {
    return p < 0 ? 0 : (p >= num_pages ? num_pages - 1 : p);
}

struct RowCtx {
    const char* kbase;
    const char* vbase;
    const float* kscales;
    const float* vscales;
    const int* pages;      // paged: physical pages of this split, from logical page page0
    int page0;
    int Hkv, kvh, kv_len;
};

// Row index (token t of this KV head) in units of D elements.
template <bool PAGED>
__device__ __forceinline__ size_t row_index(const RowCtx& c, int t) {
    if constexpr (PAGED) {
        const int pg = c.pages[(t >> 4) - c.page0];
        return ((size_t)pg * 16 + (t & 15)) * c.Hkv + c.kvh;
    } else {
        return (size_t)c.kvh * c.kv_len + t;
    }
}

template <int D, int GC, bool PAGED>
__device__ __forceinline__ void load_block(BlockRegs<D, GC, PAGED>& B, const RowCtx& c, int tb,
                                           int t_end, int j, int rg, int vrg, int vc) {
    using S = DecodeShape<D, GC, PAGED>;
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
        const int t = tb + u * S::RPW + rg;
        B.ks[u] = 1.f;
        B.vs[u] = 1.f;
        if (t < t_end) {
            const size_t ri = row_index<PAGED>(c, t);
            const char* kr = c.kbase + ri * D * S::ESZ;
            if constexpr (PAGED) {
                B.k[u][0] = ld_global_b128(kr + 16 * j);
                B.ks[u] = c.kscales[ri];
                B.vs[u] = c.vscales[ri];
            } else {
                B.k[u][0] = ld_global_b128(kr + 16 * j);
                B.k[u][S::KCH - 1] = ld_global_b128(kr + 16 * (j + S::LPT));
            }
        } else {
#pragma unroll
            for (int q = 0; q < S::KCH; ++q) B.k[u][q] = make_uint4(0, 0, 0, 0);
        }
    }
#pragma unroll
    for (int r = 0; r < S::NVL; ++r) {
        const int t = tb + r * S::VR + vrg;
        if (t < t_end) {
            const size_t ri = row_index<PAGED>(c, t);
            const char* vp = c.vbase + ri * D * S::ESZ + S::EV * S::ESZ * vc;
            if constexpr (PAGED) {
                const uint2 x = *reinterpret_cast<const uint2*>(vp);
                B.v[r] = make_uint4(x.x, x.y, 0, 0);
            } else {
                B.v[r] = ld_global_b128(vp);
            }
        } else {
            B.v[r] = make_uint4(0, 0, 0, 0);
        }
    }
}

template <int D, int GC, bool PAGED>
__device__ __forceinline__ void process_block(const BlockRegs<D, GC, PAGED>& B, int tb, int t_end,
                                              const DecodeParams& a, const float (&qr)[GC][16],
                                              float (&m_run)[GC], float (&lsum)[GC],
                                              float (&acc)[GC][DecodeShape<D, GC, PAGED>::EV],
                                              float (*lds_p)[GC], int j, int rg, int vrg) {
    using S = DecodeShape<D, GC, PAGED>;
    // ---- K phase: scores in log2 units -----------------------------------------------
    float sc[S::U][GC];
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
        float kf[16];
        if constexpr (PAGED) {
            i8x16_to_f32(B.k[u][0], kf);
        } else {
            f16x8_to_f32(B.k[u][0], kf);
            f16x8_to_f32(B.k[u][S::KCH - 1], kf + 8);
        }
        const bool valid = (tb + u * S::RPW + rg) < t_end;
#pragma unroll
        for (int g = 0; g < GC; ++g) {
            float d0 = 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e) d0 = __builtin_fmaf(qr[g][e], kf[e], d0);
            float s = group_sum<S::LPT>(d0) * B.ks[u];
            if (a.softcap > 0.f)
                s = a.softcap * tanh_via_exp(s * a.scale * a.inv_softcap) * kLog2e;
            else
                s = s * a.scale_log2;
            sc[u][g] = valid ? s : -INFINITY;
        }
    }

    // ---- block max per head, lazy rescale ----------------------------------------------
#pragma unroll
    for (int g = 0; g < GC; ++g) {
        float mb = sc[0][g];
#pragma unroll
        for (int u = 1; u < S::U; ++u) mb = fmaxf(mb, sc[u][g]);
        mb = strided_max<S::LPT>(mb);
        if (mb > m_run[g] + kRescaleSlack) {
            const float alpha = (m_run[g] == -INFINITY) ? 0.f : fast_exp2(m_run[g] - mb);
            m_run[g] = mb;
            lsum[g] *= alpha;
#pragma unroll
            for (int e = 0; e < S::EV; ++e) acc[g][e] *= alpha;
        }
    }

    // ---- p = exp2(s - m): one lane per (token, head), parked in LDS ----------------------
    if (j < GC) {
#pragma unroll
        for (int u = 0; u < S::U; ++u) {
            float x = sc[u][0], m = m_run[0];
#pragma unroll
            for (int g = 1; g < GC; ++g) {
                x = (j == g) ? sc[u][g] : x;
                m = (j == g) ? m_run[g] : m;
            }
            const float p = (x == -INFINITY) ? 0.f : fast_exp2(x - m);
#pragma unroll
            for (int g = 0; g < GC; ++g) lsum[g] += (j == g) ? p : 0.f;
            lds_p[u * S::RPW + rg][j] = PAGED ? p * B.vs[u] : p;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- V phase -----------------------------------------------------------------------
#pragma unroll
    for (int r = 0; r < S::NVL; ++r) {
        const int tl = r * S::VR + vrg;
        float pg[GC];
#pragma unroll
        for (int g = 0; g < GC; ++g) pg[g] = lds_p[tl][g];
        float vf[S::EV];
        if constexpr (PAGED) i8x8_to_f32(B.v[r].x, B.v[r].y, vf);
        else f16x8_to_f32(B.v[r], vf);
#pragma unroll
        for (int g = 0; g < GC; ++g)
#pragma unroll
            for (int e = 0; e < S::EV; ++e) acc[g][e] = __builtin_fmaf(pg[g], vf[e], acc[g][e]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D, int GC, bool PAGED>
__global__ void __launch_bounds__(64 * kDecodeWaves) decode_split_kernel(DecodeParams a) {
    using S = DecodeShape<D, GC, PAGED>;
    constexpr int NW = kDecodeWaves;
    constexpr int NT = 64 * NW;
    __shared__ float lds_p[NW][S::TB][GC];
    __shared__ float lds_o[NW][GC][D];
    __shared__ float lds_m[NW][GC];
    __shared__ float lds_l[NW][GC];
    __shared__ float lds_w[GC][kMaxSplits];
    __shared__ float lds_L[GC];
    __shared__ int lds_pages[PAGED ? kMaxSplitTokens / 16 + 1 : 1];
    __shared__ int lds_last;
    static_assert(NW * D >= kMaxSplits, "l of the split partials is parked in lds_o");

    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int split = blockIdx.x;
    const int G = a.H / a.Hkv;
    const int nch = G / GC;
    const int kvh = blockIdx.y / nch;
    const int h0 = kvh * G + (blockIdx.y % nch) * GC;
    const int b = blockIdx.z;

    // ---- key range of this sequence, and of this split --------------------------------
    int L = a.kv_len;
    if constexpr (PAGED) {
        L = a.kv_lens[b];
        if (L < 1 || L > a.max_pages * 16) {
            // out of contract: the row becomes NaN; nothing else is read
            if (split == 0)
                for (int i = threadIdx.x; i < GC * D; i += NT)
                    a.o[((size_t)b * a.H + h0 + i / D) * D + (i % D)] = __builtin_nanf("");
            return;
        }
    }
    const int k_lo = (a.window > 0 && L > a.window) ? L - a.window : 0;
    const int n_live = (L - k_lo + a.split_tokens - 1) / a.split_tokens;
    if (split >= n_live) return;
    const int t_begin = k_lo + split * a.split_tokens;
    const int t_end = min(L, t_begin + a.split_tokens);

    // ---- query slice held by this lane for the K phase ----------------------------------
    const int j = lane % S::LPT;          // position inside the row's lane group
    const int rg = lane / S::LPT;         // row within a K row-set
    float qr[GC][16];
#pragma unroll
    for (int g = 0; g < GC; ++g) {
        const float* qh = a.q + ((size_t)b * a.H + h0 + g) * D;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            int d;
            if constexpr (PAGED) d = 16 * j + e;
            else d = (e < 8) ? 8 * j + e : 8 * (j + S::LPT) + (e - 8);
            qr[g][e] = qh[d];
        }
    }

    const int vrg = lane / S::CPR;        // row within a V row-set
    const int vc = lane % S::CPR;         // V chunk owned by this lane

    float m_run[GC], lsum[GC], acc[GC][S::EV];
#pragma unroll
    for (int g = 0; g < GC; ++g) {
        m_run[g] = -INFINITY;
        lsum[g] = 0.f;
#pragma unroll
        for (int e = 0; e < S::EV; ++e) acc[g][e] = 0.f;
    }

    RowCtx c;
    c.kbase = reinterpret_cast<const char*>(a.k);
    c.vbase = reinterpret_cast<const char*>(a.v);
    c.kscales = a.k_scales;
    c.vscales = a.v_scales;
    c.pages = lds_pages;
    c.page0 = t_begin >> 4;
    c.Hkv = a.Hkv;
    c.kvh = kvh;
    c.kv_len = a.kv_len;
    if constexpr (PAGED) {
        // the physical pages of this split, fetched once (clamped into range)
        const int32_t* ptab = a.page_table + (size_t)b * a.max_pages;
        const int np = ((t_end - 1) >> 4) - c.page0 + 1;
        for (int i = threadIdx.x; i < np; i += NT) lds_pages[i] = clamp_page(ptab[c.page0 + i], a.num_pages);
        __syncthreads();
    }

    // ---- stream this wave's blocks, two register buffers in flight ---------------------
    constexpr int STRIDE = NW * S::TB;
    BlockRegs<D, GC, PAGED> A, Bf;
    int tb = t_begin + w * S::TB;
    if (tb < t_end) load_block(A, c, tb, t_end, j, rg, vrg, vc);
    while (tb < t_end) {
        const int t1 = tb + STRIDE;
        if (t1 < t_end) load_block(Bf, c, t1, t_end, j, rg, vrg, vc);
        process_block(A, tb, t_end, a, qr, m_run, lsum, acc, lds_p[w], j, rg, vrg);
        if (t1 >= t_end) break;
        const int t2 = t1 + STRIDE;
        if (t2 < t_end) load_block(A, c, t2, t_end, j, rg, vrg, vc);
        process_block(Bf, t1, t_end, a, qr, m_run, lsum, acc, lds_p[w], j, rg, vrg);
        tb = t2;
    }

    // ---- merge inside the wave --------------------------------------------------------
#pragma unroll
    for (int g = 0; g < GC; ++g) {
        lsum[g] = strided_sum<S::LPT>(lsum[g]);     // lanes j == g held it; others hold 0
        lsum[g] = group_sum<S::LPT>(lsum[g]);
#pragma unroll
        for (int e = 0; e < S::EV; ++e) acc[g][e] = strided_sum<S::CPR>(acc[g][e]);
    }
    if (lane < S::CPR) {
#pragma unroll
        for (int g = 0; g < GC; ++g)
#pragma unroll
            for (int e = 0; e < S::EV; ++e) lds_o[w][g][lane * S::EV + e] = acc[g][e];
    }
    if (lane == 0) {
#pragma unroll
        for (int g = 0; g < GC; ++g) {
            lds_m[w][g] = m_run[g];
            lds_l[w][g] = lsum[g];
        }
    }
    __syncthreads();

    // ---- merge the waves; finish or publish the split partial ---------------------------
    const size_t part_base = (size_t)b * a.H + h0;   // + g, then * n_split_max
    for (int i = threadIdx.x; i < GC * D; i += NT) {
        const int g = i / D, d = i % D;
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, lds_m[ww][g]);
        float os = 0.f, ls = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            const float mw = lds_m[ww][g];
            const float f = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
            os += f * lds_o[ww][g][d];
            ls += f * lds_l[ww][g];
        }
        if (n_live == 1) {
            a.o[(part_base + g) * D + d] = ls != 0.f ? os / ls : 0.f;
        } else {
            const size_t slot = (part_base + g) * a.n_split_max + split;
            store_agent(a.part_o + slot * D + d, os);
            if (d == 0) {
                store_agent(a.part_m + slot, M);
                store_agent(a.part_l + slot, ls);
            }
        }
    }
    if (n_live == 1) return;

    // ---- last-arriving workgroup merges all splits of this (sequence, head chunk) --------
    // The partials are device-scope stores (written through the XCD's L2) and every
    // thread waits for its stores to complete before the barrier, so when the counter is
    // bumped all partials of this workgroup are visible device-wide.  The merging
    // workgroup reads them back with device-scope loads.
    wait_stores_complete();
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t* ticket = a.tickets + (size_t)b * gridDim.y + blockIdx.y;
        const uint32_t prev = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = (prev == (uint32_t)(n_live - 1));
        if (last) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        lds_last = last;
    }
    __syncthreads();
    if (!lds_last) return;

    // (0) start fetching the first partial outputs of this thread's (head, d) pairs
    constexpr int PF = 16;
    constexpr int PER = (GC * D + NT - 1) / NT;     // (head, d) pairs per thread
    float pre[PER][PF];
#pragma unroll
    for (int r = 0; r < PER; ++r) {
        const int i = threadIdx.x + r * NT;
        if (i < GC * D) {
            const size_t row = (part_base + i / D) * a.n_split_max;
#pragma unroll
            for (int s = 0; s < PF; ++s)
                pre[r][s] = s < n_live ? load_agent(a.part_o + (row + s) * D + (i % D)) : 0.f;
        }
    }
    // (1) m and l of every split, one (head, split) pair per thread
    float* lds_ls = &lds_o[0][0][0];      // l of (g, s) at g * n_live + s
    for (int i = threadIdx.x; i < GC * n_live; i += NT) {
        const int g = i / n_live, s = i % n_live;
        const size_t slot = (part_base + g) * a.n_split_max + s;
        lds_w[g][s] = load_agent(a.part_m + slot);
        lds_ls[i] = load_agent(a.part_l + slot);
    }
    __syncthreads();
    // (2) per head: M, weights exp2(m_s - M), L = sum w_s l_s  (one wave per head)
    for (int g = w; g < GC; g += NW) {
        float M = -INFINITY;
        for (int s = lane; s < n_live; s += 64) M = fmaxf(M, lds_w[g][s]);
        M = strided_max<1>(M);
        float Ls = 0.f;
        for (int s = lane; s < n_live; s += 64) {
            const float ms = lds_w[g][s];
            const float f = (ms == -INFINITY) ? 0.f : fast_exp2(ms - M);
            lds_w[g][s] = f;
            Ls += f * lds_ls[g * n_live + s];
        }
        Ls = strided_sum<1>(Ls);
        if (lane == 0) lds_L[g] = Ls;
    }
    __syncthreads();
    // (3) o = sum_s w_s o_s / L, one (head, d) per thread
#pragma unroll
    for (int r = 0; r < PER; ++r) {
        const int i = threadIdx.x + r * NT;
        if (i >= GC * D) break;
        const int g = i / D, d = i % D;
        const size_t row = (part_base + g) * a.n_split_max;
        float os = 0.f;
#pragma unroll
        for (int s = 0; s < PF; ++s) os += (s < n_live ? lds_w[g][s] : 0.f) * pre[r][s];
        int s = PF;
        for (; s + 8 <= n_live; s += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = load_agent(a.part_o + (row + s + u) * D + d);
#pragma unroll
            for (int u = 0; u < 8; ++u) os += lds_w[g][s + u] * v[u];
        }
        for (; s < n_live; ++s) os += lds_w[g][s] * load_agent(a.part_o + (row + s) * D + d);
        const float Ls = lds_L[g];
        a.o[(part_base + g) * D + d] = Ls != 0.f ? os / Ls : 0.f;
    }
}

template <int D, bool PAGED>
hipError_t launch_decode_d(const DecodeParams& p, int gc, dim3 grid, hipStream_t st) {
    const dim3 block(64 * kDecodeWaves);
    switch (gc) {
        case 1: hipLaunchKernelGGL((decode_split_kernel<D, 1, PAGED>), grid, block, 0, st, p); break;
        case 2: hipLaunchKernelGGL((decode_split_kernel<D, 2, PAGED>), grid, block, 0, st, p); break;
        case 4: hipLaunchKernelGGL((decode_split_kernel<D, 4, PAGED>), grid, block, 0, st, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int head_dim, int gc, bool paged, int batch,
                         hipStream_t st) {
    const int nch = (p.H / p.Hkv) / gc;
    dim3 grid(p.n_split_max, p.Hkv * nch, batch);
    if (paged) {
        switch (head_dim) {
            case 64: return launch_decode_d<64, true>(p, gc, grid, st);
            case 128: return launch_decode_d<128, true>(p, gc, grid, st);
            case 256: return launch_decode_d<256, true>(p, gc, grid, st);
        }
    } else {
        switch (head_dim) {
            case 64: return launch_decode_d<64, false>(p, gc, grid, st);
            case 128: return launch_decode_d<128, false>(p, gc, grid, st);
            case 256: return launch_decode_d<256, false>(p, gc, grid, st);
        }
    }
    return hipErrorInvalidValue;
}

int decode_tokens_per_block(int head_dim, bool paged) {
    (void)paged;
    return 4096 / (head_dim * 2);
}

int decode_waves() { return kDecodeWaves; }

int decode_max_splits() { return kMaxSplits; }

int decode_max_split_tokens_paged() { return kMaxSplitTokens; }

}  // namespace ta03
