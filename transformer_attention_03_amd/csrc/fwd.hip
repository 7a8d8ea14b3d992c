// Prefill and vision attention forward for gfx950: online softmax over K/V tiles held in
// LDS, with both products on the matrix cores.
//
// The pages describe the method for WebGPU (rullama 0.5.0 src/backend/dispatch/attention.rs,
// vision_attention_flash_chained: K and V tiled into workgroup memory in chunks of 32
// patches with an online softmax; the multi-query variants let 4/8/16 queries share one
// K/V load).  Here a workgroup owns a block of query rows of one head and streams K/V
// tiles of BN keys through LDS; each wave owns 16-row query blocks and runs
//   S^T = K Q^T     on v_mfma_f32_16x16x32_f16 (f16) or v_mfma_f32_16x16x4_f32 (f32),
//   online softmax  in f32 registers in the MFMA output layout (exp2 with log2(e) folded
//                   into the scale; the running max only moves, and the accumulator is
//                   only rescaled, when a tile's max exceeds it by more than 2^8),
//   O^T += V^T P^T  with P^T taken straight from the S^T accumulators (f16 for f16 inputs).
// Computing the transposed products means the probabilities never leave registers: the
// S^T output layout (lane = query, 4 consecutive keys) is exactly the B-operand layout the
// PV product needs.  V is written to LDS transposed ([d][key]) so its A-operand fragments
// are 8-byte reads.
//
// Masks: key j is visible to query position p iff j < kv_len, (!causal || j <= p) and
// (W == 0 || p - j < W).  The host-independent tile range skips tiles that no row of the
// workgroup can see; per-element masks run only on tiles that straddle an edge.

#include "device_common.hpp"
#include "launch.hpp"

namespace ta03 {

namespace {

constexpr float kMinit = -1.0e30f;       // finite "minus infinity" for the running max
constexpr float kSlack = 8.0f;           // log2 units

struct TileRange {
    int kt0, kt1;                        // tiles [kt0, kt1)
    int pos_lo, pos_hi;                  // query positions covered by the workgroup
    int k_begin, k_end;                  // visible keys of the workgroup: [k_begin, k_end)
};

__device__ __forceinline__ TileRange tile_range(const FwdParams& a, int q0, int bm, int bn) {
    TileRange r;
    const int last = min(q0 + bm, a.seq_len) - 1;
    r.pos_lo = a.kv_len - a.seq_len + q0;
    r.pos_hi = a.kv_len - a.seq_len + last;
    r.k_end = a.causal ? min(a.kv_len, r.pos_hi + 1) : a.kv_len;
    r.k_begin = a.window > 0 ? max(0, r.pos_lo - a.window + 1) : 0;
    r.kt0 = r.k_begin / bn;
    r.kt1 = (r.k_end + bn - 1) / bn;
    return r;
}

__device__ __forceinline__ bool tile_needs_mask(const FwdParams& a, const TileRange& r, int ks,
                                                int bn) {
    const int ke = ks + bn;
    if (ke > a.kv_len) return true;
    if (a.causal && ke - 1 > r.pos_lo) return true;
    if (a.window > 0 && ks < r.pos_hi - a.window + 1) return true;
    return false;
}

__device__ __forceinline__ bool visible(const FwdParams& a, int key, int pos) {
    return key < a.kv_len && (!a.causal || key <= pos) && (a.window <= 0 || pos - key < a.window);
}

// Work item for this workgroup: XCD-aware (consecutive work ids land on one XCD, so the
// query blocks of a head share that XCD's L2) and heaviest causal blocks first.
__device__ __forceinline__ void work_item(const FwdParams& a, int& head, int& qblock) {
    const int n = gridDim.x;
    int wid = blockIdx.x;
    if ((n & 7) == 0) wid = (wid & 7) * (n >> 3) + (wid >> 3);
    head = wid / a.n_qblocks;
    const int qb = wid % a.n_qblocks;
    qblock = a.causal ? a.n_qblocks - 1 - qb : qb;
}

__device__ __forceinline__ float score_transform(const FwdParams& a, float s) {
    if (a.softcap > 0.f) return a.softcap * tanh_via_exp(s * a.scale * a.inv_softcap) * kLog2e;
    return s * a.scale_log2;
}

// =============================================================================================
// f16 inputs, f32 accumulation: v_mfma_f32_16x16x32_f16
// =============================================================================================

template <int D>
struct F16Shape {
    static constexpr int NW = 4;                  // waves per workgroup
    static constexpr int QB = 2;                  // 16-row query blocks per wave
    static constexpr int BM = NW * QB * 16;       // query rows per workgroup
    static constexpr int BN = 64;                 // keys per tile
    static constexpr int KLD = D + 8;             // K row stride in LDS (halves)
    static constexpr int VLD = BN + 4;            // V^T row stride in LDS (halves)
    static constexpr int KCH = BN * D / 8 / 256;  // 16-byte K chunks per thread per tile
    static constexpr int VGRP = (BN / 4) * (D / 8);        // 4-key x 8-d groups per tile
    static constexpr int VG_PER_T = (VGRP + 255) / 256;    // per thread
    static constexpr int DC = D / 32;             // 32-wide k chunks of the QK^T product
    static constexpr int NDB = D / 16;            // 16-row d blocks of O^T
    static constexpr int NKB = BN / 16;           // 16-key blocks of S^T
};

template <int D>
__global__ void __launch_bounds__(256) fwd_f16_kernel(FwdParams a) {
    using S = F16Shape<D>;
    __shared__ __attribute__((aligned(16))) _Float16 k_lds[S::BN * S::KLD];
    __shared__ __attribute__((aligned(16))) _Float16 vt_lds[D * S::VLD];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int ln = lane & 15;          // query column inside a 16-block / row of an A tile
    const int lg = lane >> 4;          // lane group 0..3

    int head, qblock;
    work_item(a, head, qblock);
    const int kvh = head / (a.H / a.Hkv);
    const int q0 = qblock * S::BM;
    const TileRange tr = tile_range(a, q0, S::BM, S::BN);

    const _Float16* qg = reinterpret_cast<const _Float16*>(a.q) + (long)head * a.q_head;
    const _Float16* kg = reinterpret_cast<const _Float16*>(a.k) + (long)kvh * a.k_head;
    const _Float16* vg = reinterpret_cast<const _Float16*>(a.v) + (long)kvh * a.k_head;

    // ---- Q fragments (B operand of S^T = K Q^T) --------------------------------------------
    half8_t qf[S::QB][S::DC];
    int qpos[S::QB];
#pragma unroll
    for (int qb = 0; qb < S::QB; ++qb) {
        const int row = q0 + (w * S::QB + qb) * 16 + ln;
        qpos[qb] = a.kv_len - a.seq_len + row;
        const int rr = min(row, a.seq_len - 1);
#pragma unroll
        for (int c = 0; c < S::DC; ++c)
            qf[qb][c] = *reinterpret_cast<const half8_t*>(qg + (long)rr * a.q_row + 32 * c + 8 * lg);
    }

    float4_t acc_o[S::NDB][S::QB];
#pragma unroll
    for (int db = 0; db < S::NDB; ++db)
#pragma unroll
        for (int qb = 0; qb < S::QB; ++qb) acc_o[db][qb] = float4_t{0.f, 0.f, 0.f, 0.f};
    float m_run[S::QB], l_part[S::QB];
#pragma unroll
    for (int qb = 0; qb < S::QB; ++qb) {
        m_run[qb] = kMinit;
        l_part[qb] = 0.f;
    }

    // ---- register staging of one K/V tile ------------------------------------------------
    uint4 kst[S::KCH];
    uint4 vst[S::VG_PER_T][4];
    auto load_tile = [&](int kt) {
        const int ks = kt * S::BN;
#pragma unroll
        for (int i = 0; i < S::KCH; ++i) {
            const int ci = tid + 256 * i;
            const int r = ci / (D / 8), c = ci % (D / 8);
            const int key = min(ks + r, a.kv_len - 1);
            kst[i] = *reinterpret_cast<const uint4*>(kg + (long)key * a.k_row + 8 * c);
        }
#pragma unroll
        for (int i = 0; i < S::VG_PER_T; ++i) {
            const int gi = tid + 256 * i;
            if (gi < S::VGRP) {
                const int k4 = gi / (D / 8), c = gi % (D / 8);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int key = min(ks + 4 * k4 + e, a.kv_len - 1);
                    vst[i][e] = *reinterpret_cast<const uint4*>(vg + (long)key * a.k_row + 8 * c);
                }
            }
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < S::KCH; ++i) {
            const int ci = tid + 256 * i;
            const int r = ci / (D / 8), c = ci % (D / 8);
            *reinterpret_cast<uint4*>(&k_lds[r * S::KLD + 8 * c]) = kst[i];
        }
#pragma unroll
        for (int i = 0; i < S::VG_PER_T; ++i) {
            const int gi = tid + 256 * i;
            if (gi < S::VGRP) {
                const int k4 = gi / (D / 8), c = gi % (D / 8);
                const half8_t r0 = __builtin_bit_cast(half8_t, vst[i][0]);
                const half8_t r1 = __builtin_bit_cast(half8_t, vst[i][1]);
                const half8_t r2 = __builtin_bit_cast(half8_t, vst[i][2]);
                const half8_t r3 = __builtin_bit_cast(half8_t, vst[i][3]);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const half4_t col = half4_t{r0[e], r1[e], r2[e], r3[e]};
                    *reinterpret_cast<half4_t*>(&vt_lds[(8 * c + e) * S::VLD + 4 * k4]) = col;
                }
            }
        }
    };

    if (tr.kt0 < tr.kt1) load_tile(tr.kt0);
    for (int kt = tr.kt0; kt < tr.kt1; ++kt) {
        __syncthreads();
        store_tile();
        __syncthreads();
        if (kt + 1 < tr.kt1) load_tile(kt + 1);

        const int ks = kt * S::BN;
        const bool masked = tile_needs_mask(a, tr, ks, S::BN);

        // ---- S^T = K Q^T -----------------------------------------------------------------
        float4_t st[S::NKB][S::QB];
#pragma unroll
        for (int kb = 0; kb < S::NKB; ++kb) {
#pragma unroll
            for (int qb = 0; qb < S::QB; ++qb) st[kb][qb] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < S::DC; ++c) {
                const half8_t kf =
                    *reinterpret_cast<const half8_t*>(&k_lds[(16 * kb + ln) * S::KLD + 32 * c + 8 * lg]);
#pragma unroll
                for (int qb = 0; qb < S::QB; ++qb)
                    st[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[qb][c], st[kb][qb], 0, 0, 0);
            }
        }

        // ---- online softmax in the S^T layout: lane = query (ln), keys 16kb + 4lg + i ----
        half8_t pf[S::QB][S::BN / 32];
#pragma unroll
        for (int qb = 0; qb < S::QB; ++qb) {
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < S::NKB; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float t = score_transform(a, st[kb][qb][i]);
                    if (masked && !visible(a, ks + 16 * kb + 4 * lg + i, qpos[qb])) t = -INFINITY;
                    st[kb][qb][i] = t;
                    mx = fmaxf(mx, t);
                }
            mx = fmaxf(mx, shfl_xor_f(mx, 16));
            mx = fmaxf(mx, shfl_xor_f(mx, 32));
            if (__builtin_amdgcn_ballot_w64(mx > m_run[qb] + kSlack) != 0) {
                const float mnew = fmaxf(m_run[qb], mx);
                const float alpha = fast_exp2(m_run[qb] - mnew);
                m_run[qb] = mnew;
                l_part[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < S::NDB; ++db) acc_o[db][qb] *= alpha;
            }
            float ls = 0.f;
#pragma unroll
            for (int kb = 0; kb < S::NKB; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p = fast_exp2(st[kb][qb][i] - m_run[qb]);
                    st[kb][qb][i] = p;
                    ls += p;
                }
            l_part[qb] += ls;
#pragma unroll
            for (int c = 0; c < S::BN / 32; ++c) {
                half8_t h;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    h[i] = (_Float16)st[2 * c][qb][i];
                    h[4 + i] = (_Float16)st[2 * c + 1][qb][i];
                }
                pf[qb][c] = h;
            }
        }

        // ---- O^T += V^T P^T ---------------------------------------------------------------
#pragma unroll
        for (int db = 0; db < S::NDB; ++db) {
#pragma unroll
            for (int c = 0; c < S::BN / 32; ++c) {
                const _Float16* vrow = &vt_lds[(16 * db + ln) * S::VLD + 32 * c + 4 * lg];
                const half4_t lo = *reinterpret_cast<const half4_t*>(vrow);
                const half4_t hi = *reinterpret_cast<const half4_t*>(vrow + 16);
                const half8_t vf = half8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
                for (int qb = 0; qb < S::QB; ++qb)
                    acc_o[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[qb][c], acc_o[db][qb], 0, 0, 0);
            }
        }
    }

    // ---- epilogue: O = O^T^T / l -----------------------------------------------------------
    _Float16* og = reinterpret_cast<_Float16*>(a.o) + (long)head * a.o_head;
#pragma unroll
    for (int qb = 0; qb < S::QB; ++qb) {
        float l = l_part[qb];
        l += shfl_xor_f(l, 16);
        l += shfl_xor_f(l, 32);
        const float inv = l > 0.f ? 1.0f / l : 0.f;
        const int row = q0 + (w * S::QB + qb) * 16 + ln;
        if (row < a.seq_len) {
#pragma unroll
            for (int db = 0; db < S::NDB; ++db) {
                half4_t h;
#pragma unroll
                for (int i = 0; i < 4; ++i) h[i] = (_Float16)(acc_o[db][qb][i] * inv);
                *reinterpret_cast<half4_t*>(og + (long)row * a.o_row + 16 * db + 4 * lg) = h;
            }
        }
    }
}

// =============================================================================================
// f32 inputs and output, f32 products: v_mfma_f32_16x16x4_f32
// =============================================================================================

template <int D>
struct F32Shape {
    static constexpr int NW = 4;
    static constexpr int BM = NW * 16;            // one 16-row query block per wave
    static constexpr int BN = 32;
    static constexpr int LD = D + 1;              // LDS row stride (floats)
    static constexpr int CH = BN * D / 4 / 256;   // float4 chunks per thread per tile (K or V)
    static constexpr int NKB = BN / 16;
    static constexpr int NDB = D / 16;
    static constexpr int DC = D / 4;
};

template <int D>
__global__ void __launch_bounds__(256) fwd_f32_kernel(FwdParams a) {
    using S = F32Shape<D>;
    __shared__ float k_lds[S::BN * S::LD];
    __shared__ float v_lds[S::BN * S::LD];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int ln = lane & 15;
    const int lg = lane >> 4;

    int head, qblock;
    work_item(a, head, qblock);
    const int kvh = head / (a.H / a.Hkv);
    const int q0 = qblock * S::BM;
    const TileRange tr = tile_range(a, q0, S::BM, S::BN);

    const float* qg = reinterpret_cast<const float*>(a.q) + (long)head * a.q_head;
    const float* kg = reinterpret_cast<const float*>(a.k) + (long)kvh * a.k_head;
    const float* vg = reinterpret_cast<const float*>(a.v) + (long)kvh * a.k_head;

    const int row = q0 + w * 16 + ln;
    const int qpos = a.kv_len - a.seq_len + row;
    float qf[S::DC];
    {
        const int rr = min(row, a.seq_len - 1);
#pragma unroll
        for (int c = 0; c < S::DC; ++c) qf[c] = qg[(long)rr * a.q_row + 4 * c + lg];
    }

    float4_t acc_o[S::NDB];
#pragma unroll
    for (int db = 0; db < S::NDB; ++db) acc_o[db] = float4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = kMinit, l_part = 0.f;

    float4 kst[S::CH], vst[S::CH];
    auto load_tile = [&](int kt) {
        const int ks = kt * S::BN;
#pragma unroll
        for (int i = 0; i < S::CH; ++i) {
            const int ci = tid + 256 * i;
            const int r = ci / (D / 4), c = ci % (D / 4);
            const int key = min(ks + r, a.kv_len - 1);
            kst[i] = *reinterpret_cast<const float4*>(kg + (long)key * a.k_row + 4 * c);
            vst[i] = *reinterpret_cast<const float4*>(vg + (long)key * a.k_row + 4 * c);
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < S::CH; ++i) {
            const int ci = tid + 256 * i;
            const int r = ci / (D / 4), c = ci % (D / 4);
            float* kd = &k_lds[r * S::LD + 4 * c];
            float* vd = &v_lds[r * S::LD + 4 * c];
            kd[0] = kst[i].x; kd[1] = kst[i].y; kd[2] = kst[i].z; kd[3] = kst[i].w;
            vd[0] = vst[i].x; vd[1] = vst[i].y; vd[2] = vst[i].z; vd[3] = vst[i].w;
        }
    };

    if (tr.kt0 < tr.kt1) load_tile(tr.kt0);
    for (int kt = tr.kt0; kt < tr.kt1; ++kt) {
        __syncthreads();
        store_tile();
        __syncthreads();
        if (kt + 1 < tr.kt1) load_tile(kt + 1);
        const int ks = kt * S::BN;
        const bool masked = tile_needs_mask(a, tr, ks, S::BN);

        float4_t st[S::NKB];
#pragma unroll
        for (int kb = 0; kb < S::NKB; ++kb) {
            st[kb] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < S::DC; ++c) {
                const float kf = k_lds[(16 * kb + ln) * S::LD + 4 * c + lg];
                st[kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf, qf[c], st[kb], 0, 0, 0);
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < S::NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float t = score_transform(a, st[kb][i]);
                if (masked && !visible(a, ks + 16 * kb + 4 * lg + i, qpos)) t = -INFINITY;
                st[kb][i] = t;
                mx = fmaxf(mx, t);
            }
        mx = fmaxf(mx, shfl_xor_f(mx, 16));
        mx = fmaxf(mx, shfl_xor_f(mx, 32));
        if (__builtin_amdgcn_ballot_w64(mx > m_run + kSlack) != 0) {
            const float mnew = fmaxf(m_run, mx);
            const float alpha = fast_exp2(m_run - mnew);
            m_run = mnew;
            l_part *= alpha;
#pragma unroll
            for (int db = 0; db < S::NDB; ++db) acc_o[db] *= alpha;
        }
#pragma unroll
        for (int kb = 0; kb < S::NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = fast_exp2(st[kb][i] - m_run);
                st[kb][i] = p;
                l_part += p;
            }
        // O^T += V^T P^T, four keys {16kb + 4g + i : g} per product
#pragma unroll
        for (int db = 0; db < S::NDB; ++db)
#pragma unroll
            for (int kb = 0; kb < S::NKB; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float vf = v_lds[(16 * kb + 4 * lg + i) * S::LD + 16 * db + ln];
                    acc_o[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf, st[kb][i], acc_o[db], 0, 0, 0);
                }
    }

    float l = l_part;
    l += shfl_xor_f(l, 16);
    l += shfl_xor_f(l, 32);
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    float* og = reinterpret_cast<float*>(a.o) + (long)head * a.o_head;
    if (row < a.seq_len) {
#pragma unroll
        for (int db = 0; db < S::NDB; ++db) {
            float4 r;
            r.x = acc_o[db][0] * inv; r.y = acc_o[db][1] * inv;
            r.z = acc_o[db][2] * inv; r.w = acc_o[db][3] * inv;
            *reinterpret_cast<float4*>(og + (long)row * a.o_row + 16 * db + 4 * lg) = r;
        }
    }
}

template <int D>
hipError_t launch_d(const FwdParams& p, int dtype, hipStream_t st) {
    const dim3 grid(p.n_qblocks * p.H);
    if (dtype == 1) hipLaunchKernelGGL(fwd_f16_kernel<D>, grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL(fwd_f32_kernel<D>, grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace

int fwd_block_rows(int head_dim, int dtype) {
    (void)head_dim;
    return dtype == 1 ? F16Shape<64>::BM : F32Shape<64>::BM;
}

hipError_t launch_fwd(const FwdParams& p, int head_dim, int dtype, hipStream_t st) {
    switch (head_dim) {
        case 64: return launch_d<64>(p, dtype, st);
        case 128: return launch_d<128>(p, dtype, st);
        case 256: return launch_d<256>(p, dtype, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace ta03
