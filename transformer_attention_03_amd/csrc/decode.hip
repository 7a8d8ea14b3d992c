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
// all of them) and a contiguous logical token range.  Inside, each wave streams blocks of
// TB tokens:
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
// counted with a device-scope atomic that is reset to zero by that last workgroup.
//
// Paged addressing is integer-exact: physical page = page_table[b][t >> 4], slot t & 15,
// row ((page * 16 + slot) * Hkv + kvh) * D.  Rows at or past kv_len are never loaded, so
// poisoned slots of a partial last page cannot reach the result.

#include "device_common.hpp"
#include "launch.hpp"

namespace ta03 {

namespace {

constexpr int kDecodeWaves = 4;
constexpr float kRescaleSlack = 8.0f;   // log2 units: accumulators may grow to 2^8

template <int D, int GC, bool PAGED>
struct DecodeShape {
    static constexpr int ESZ = PAGED ? 1 : 2;          // bytes per K/V element
    static constexpr int LPT = D / 16;                  // K-phase lanes per row
    static constexpr int RPW = 64 / LPT;                // K rows per wave-load
    static constexpr int TB = 8192 / (D * ESZ);         // tokens per wave block (8 KB of K)
    static constexpr int U = TB / RPW;                  // K row-sets per block
    static constexpr int KCH = 16 * ESZ / 16;           // 16-byte chunks per lane per K row
    static constexpr int CPR = D * ESZ / 16;            // 16-byte chunks per V row
    static constexpr int VR = 64 / CPR;                 // V rows per wave-load
    static constexpr int NVL = TB / VR;                 // V loads per lane per block
    static constexpr int EV = 16 / ESZ;                 // elements per V chunk
    static_assert(LPT >= 4 && LPT <= 16, "head_dim");
    static_assert(GC <= 8, "heads per workgroup");
    static_assert(TB % RPW == 0 && TB % VR == 0, "block shape");
};

__device__ __forceinline__ int clamp_page(int p, int num_pages) {
    return p < 0 ? 0 : (p >= num_pages ? num_pages - 1 : p);
}

template <int D, int GC, bool PAGED>
__global__ void __launch_bounds__(256) decode_split_kernel(DecodeParams a) {
    using S = DecodeShape<D, GC, PAGED>;
    constexpr int NW = kDecodeWaves;
    __shared__ float lds_p[NW][S::TB][GC];
    __shared__ float lds_o[NW][GC][D];
    __shared__ float lds_m[NW][GC];
    __shared__ float lds_l[NW][GC];
    __shared__ int lds_last;

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
                for (int i = threadIdx.x; i < GC * D; i += blockDim.x)
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

    const char* kbase = reinterpret_cast<const char*>(a.k);
    const char* vbase = reinterpret_cast<const char*>(a.v);
    const int32_t* ptab = PAGED ? a.page_table + (size_t)b * a.max_pages : nullptr;

    // byte offset of row t of this KV head
    auto row_off = [&](int t, size_t& scale_idx) -> size_t {
        if constexpr (PAGED) {
            const int pg = clamp_page(ptab[t >> 4], a.num_pages);
            scale_idx = ((size_t)pg * 16 + (t & 15)) * a.Hkv + kvh;
            return scale_idx * D;
        } else {
            scale_idx = 0;
            return ((size_t)kvh * a.kv_len + t) * D * 2;
        }
    };

    for (int tb = t_begin + w * S::TB; tb < t_end; tb += NW * S::TB) {
        // ---- issue all loads of the block: K rows (K phase map), V rows (V phase map) --
        uint4 kr[S::U][S::KCH];
        float ks[S::U];
        float vs_own[S::U];
#pragma unroll
        for (int u = 0; u < S::U; ++u) {
            const int t = tb + u * S::RPW + rg;
            ks[u] = 1.f;
            vs_own[u] = 1.f;
            if (t < t_end) {
                size_t si;
                const size_t off = row_off(t, si);
                if constexpr (PAGED) {
                    kr[u][0] = ld_global_b128(kbase + off + 16 * j);
                    ks[u] = a.k_scales[si];
                    vs_own[u] = a.v_scales[si];
                } else {
                    kr[u][0] = ld_global_b128(kbase + off + 16 * j);
                    kr[u][S::KCH - 1] = ld_global_b128(kbase + off + 16 * (j + S::LPT));
                }
            } else {
#pragma unroll
                for (int c = 0; c < S::KCH; ++c) kr[u][c] = make_uint4(0, 0, 0, 0);
            }
        }
        uint4 vr[S::NVL];
#pragma unroll
        for (int r = 0; r < S::NVL; ++r) {
            const int t = tb + r * S::VR + vrg;
            if (t < t_end) {
                size_t si;
                const size_t off = row_off(t, si);
                vr[r] = ld_global_b128(vbase + off + 16 * vc);
            } else {
                vr[r] = make_uint4(0, 0, 0, 0);
            }
        }

        // ---- K phase: scores in log2 units -------------------------------------------
        float sc[S::U][GC];
#pragma unroll
        for (int u = 0; u < S::U; ++u) {
            float kf[16];
            if constexpr (PAGED) {
                i8x16_to_f32(kr[u][0], kf);
            } else {
                f16x8_to_f32(kr[u][0], kf);
                f16x8_to_f32(kr[u][S::KCH - 1], kf + 8);
            }
            const bool valid = (tb + u * S::RPW + rg) < t_end;
#pragma unroll
            for (int g = 0; g < GC; ++g) {
                float d0 = 0.f;
#pragma unroll
                for (int e = 0; e < 16; ++e) d0 = __builtin_fmaf(qr[g][e], kf[e], d0);
                float s = group_sum<S::LPT>(d0) * ks[u];
                if (a.softcap > 0.f)
                    s = a.softcap * tanh_via_exp(s * a.scale * a.inv_softcap) * kLog2e;
                else
                    s = s * a.scale_log2;
                sc[u][g] = valid ? s : -INFINITY;
            }
        }

        // ---- block max per head, lazy rescale --------------------------------------------
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

        // ---- p = exp2(s - m): one lane per (token, head), parked in LDS -------------------
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
                lds_p[w][u * S::RPW + rg][j] = PAGED ? p * vs_own[u] : p;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- V phase -----------------------------------------------------------------
#pragma unroll
        for (int r = 0; r < S::NVL; ++r) {
            const int tl = r * S::VR + vrg;
            float pg[GC];
#pragma unroll
            for (int g = 0; g < GC; ++g) pg[g] = lds_p[w][tl][g];
            float vf[S::EV];
            if constexpr (PAGED) i8x16_to_f32(vr[r], vf);
            else f16x8_to_f32(vr[r], vf);
#pragma unroll
            for (int g = 0; g < GC; ++g)
#pragma unroll
                for (int e = 0; e < S::EV; ++e) acc[g][e] = __builtin_fmaf(pg[g], vf[e], acc[g][e]);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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
    for (int i = threadIdx.x; i < GC * D; i += blockDim.x) {
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
            a.o[(part_base + g) * D + d] = ls > 0.f ? os / ls : 0.f;
        } else {
            const size_t slot = (part_base + g) * a.n_split_max + split;
            a.part_o[slot * D + d] = os;
            if (d == 0) {
                a.part_m[slot] = M;
                a.part_l[slot] = ls;
            }
        }
    }
    if (n_live == 1) return;

    // ---- last-arriving workgroup merges all splits of this (sequence, head chunk) --------
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t* ticket = a.tickets + (size_t)b * gridDim.y + blockIdx.y;
        const uint32_t prev = atomicAdd(ticket, 1u);
        const int last = (prev == (uint32_t)(n_live - 1));
        if (last) atomicExch(ticket, 0u);   // leave the counter zeroed for the next call
        lds_last = last;
    }
    __syncthreads();
    if (!lds_last) return;
    __threadfence();

    for (int i = threadIdx.x; i < GC * D; i += blockDim.x) {
        const int g = i / D, d = i % D;
        const size_t row = (part_base + g) * a.n_split_max;
        float M = -INFINITY;
        for (int s = 0; s < n_live; ++s) M = fmaxf(M, __builtin_nontemporal_load(a.part_m + row + s));
        float os = 0.f, ls = 0.f;
        for (int s = 0; s < n_live; ++s) {
            const float ms = __builtin_nontemporal_load(a.part_m + row + s);
            const float f = (ms == -INFINITY) ? 0.f : fast_exp2(ms - M);
            os += f * __builtin_nontemporal_load(a.part_o + (row + s) * D + d);
            ls += f * __builtin_nontemporal_load(a.part_l + row + s);
        }
        a.o[(part_base + g) * D + d] = ls > 0.f ? os / ls : 0.f;
    }
}

template <int D, bool PAGED>
hipError_t launch_decode_d(const DecodeParams& p, int gc, dim3 grid, hipStream_t st) {
    switch (gc) {
        case 1: hipLaunchKernelGGL((decode_split_kernel<D, 1, PAGED>), grid, dim3(256), 0, st, p); break;
        case 2: hipLaunchKernelGGL((decode_split_kernel<D, 2, PAGED>), grid, dim3(256), 0, st, p); break;
        case 4: hipLaunchKernelGGL((decode_split_kernel<D, 4, PAGED>), grid, dim3(256), 0, st, p); break;
        case 8: hipLaunchKernelGGL((decode_split_kernel<D, 8, PAGED>), grid, dim3(256), 0, st, p); break;
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
    return 8192 / (head_dim * (paged ? 1 : 2));
}

}  // namespace ta03
