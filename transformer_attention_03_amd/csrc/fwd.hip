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

#include <type_traits>

#include "fwd_common.hpp"

namespace ta03 {

namespace {


// Key groups (KS > 1, for grids too small to fill the device): the NW waves form KS groups
// of NW / KS waves; the groups hold the same query rows and each iteration brings in KS
// tiles, one per group, so every wave walks 1 / KS of the keys.  At the end the groups'
// online-softmax states (running max, row sum, unnormalised output) are merged through LDS
// by log-sum-exp and the first group writes the rows.
// CAP: 0 no logit cap; 1 the cap through the exponential identity alone (caps up to
// kFastCapMax, where its absolute score error of about 1.2e-7 c stays below 1e-5); 2 the cap
// through tanh_accurate (larger caps, where that error would grow with c).
template <int D, int QB, int NW, int NS, int BN, int KS, int CAP>
__global__ void __launch_bounds__(64 * NW) fwd_f16_kernel(FwdParams a) {
    using S = F16Shape<D, QB, NW, NS, BN, KS>;
    static_assert(KS == 1 || (NS == 2 && QB == 1 && NW % KS == 0), "key groups: two stages, one row block per wave");
    __shared__ __attribute__((aligned(1024))) char k_lds[NS][KS][S::TILE];
    __shared__ __attribute__((aligned(1024))) char v_lds[NS][KS][S::TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 15;          // query column of the S^T / O^T blocks; A-tile row
    const int lg = lane >> 4;          // lane group 0..3
    const int qw = KS == 1 ? w : w % S::NWQ;     // query block of this wave
    const int kg = KS == 1 ? 0 : w / S::NWQ;     // key group of this wave

    int head, qblock;
    work_item(a, head, qblock);
    const int kvh = head / (a.H / a.Hkv);
    const int q0 = qblock * S::BM;
    if (!resolve_kv_len<_Float16, D>(a, head, q0, S::BM)) return;
    const TileRange tr = tile_range(a, q0, S::BM, S::BN);

    const _Float16* qg = reinterpret_cast<const _Float16*>(a.q) + (long)head * a.q_head;
    const char* kg_ptr = reinterpret_cast<const char*>(reinterpret_cast<const _Float16*>(a.k) + (long)kvh * a.k_head);
    const char* vg = reinterpret_cast<const char*>(reinterpret_cast<const _Float16*>(a.v) + (long)kvh * a.k_head);

    // The tiles of key group kg are loaded by that group's NW / KS waves alone, so a wave
    // forms the address of one tile per iteration instead of KS (scalar arithmetic that all
    // waves of a compute unit otherwise share one scalar unit for).
    constexpr int NWT = NW / KS;
    DmaLane<D, QB, NWT, NS, BN> dl;
    dma_lane_init(dl, a, w % NWT, lane);

    // Tiles are visited from a starting point that depends on the query block, so that the
    // workgroups of one head do not all fetch the same tile at the same moment (each would
    // then wait for the same cold line); any visiting order gives the same softmax.
    const int nt = tr.kt1 - tr.kt0;
    const int rot = nt > 1 ? (int)(((long)qblock * nt) / a.n_qblocks) : 0;
    auto tile_key = [&](int t) { int u = t - tr.kt0 + rot; u -= u >= nt ? nt : 0; return (tr.kt0 + u) * S::BN; };

    // prologue: the tiles of iterations 0 .. NS - 2 in flight (iteration i holds tiles
    // kt0 + i KS + j, j < KS, one per key group)
#pragma unroll
    for (int st0 = 0; st0 < NS - 1; ++st0)
        if (tr.kt0 + st0 * KS + kg < tr.kt1)
            f16_dma_tile<D, QB, NWT, NS, BN>(a, kg_ptr, vg, dl, tile_key(tr.kt0 + st0 * KS + kg), w % NWT, lane,
                                             k_lds[st0][kg], v_lds[st0][kg]);

    // ---- Q fragments (B operand of S^T = K Q^T) --------------------------------------------
    half8_t qf[S::QB][S::DC];
    int qpos[S::QB];
    int vlo[S::QB];
    unsigned vspan[S::QB];
#pragma unroll
    for (int qb = 0; qb < S::QB; ++qb) {
        const int row = q0 + (qw * S::QB + qb) * 16 + ln;
        qpos[qb] = a.kv_len - a.seq_len + row;
        const int hi = a.causal ? min(qpos[qb], a.kv_len - 1) : a.kv_len - 1;
        const int lo = a.window > 0 ? max(0, qpos[qb] - a.window + 1) : 0;
        // an empty interval (padding rows past seq_len only) keeps every key masked
        vlo[qb] = hi >= lo ? lo : 0x40000000;
        vspan[qb] = hi >= lo ? (unsigned)(hi - lo) : 0u;
        const int rr = min(row, a.seq_len - 1);
#pragma unroll
        for (int c = 0; c < S::DC; ++c)
            qf[qb][c] = *reinterpret_cast<const half8_t*>(qg + (long)rr * a.q_row + 32 * c + 8 * lg);
    }
    // Settle the Q loads here: the loop below must not wait on the vector-memory counter,
    // which also counts the in-flight tile DMAs.
#pragma unroll
    for (int qb = 0; qb < S::QB; ++qb)
#pragma unroll
        for (int c = 0; c < S::DC; ++c) asm volatile("" ::"v"(qf[qb][c]));

    float4_t acc_o[S::NDB][S::QB];
#pragma unroll
    for (int db = 0; db < S::NDB; ++db)
#pragma unroll
        for (int qb = 0; qb < S::QB; ++qb) acc_o[db][qb] = float4_t{0.f, 0.f, 0.f, 0.f};
    float m_run[S::QB];
    float4_t acc_l[S::QB];               // row sums of P (all four entries equal)
#pragma unroll
    for (int qb = 0; qb < S::QB; ++qb) {
        m_run[qb] = kMinit;
        acc_l[qb] = float4_t{0.f, 0.f, 0.f, 0.f};
    }
    const half8_t ones = half8_t{1, 1, 1, 1, 1, 1, 1, 1};

    const float sc2 = CAP ? 1.f : a.scale_log2;        // raw score -> log2 units
    // softcap in log2 units: t = C1 - C2 / (2^(s * K1) + 1), C1 = c log2 e, C2 = 2 c log2 e,
    // K1 = 2 scale log2 e / c  (c tanh(scale s / c) = c - 2c / (exp(2 scale s / c) + 1));
    // for large caps t = C1 tanh(s * KX), KX = scale / c
    const float K1 = 2.f * a.scale * kLog2e * a.inv_softcap;
    const float C1 = a.softcap * kLog2e;
    const float C2 = 2.f * C1;
    const float KX = a.scale * a.inv_softcap;

    // Tile-invariant parts of the fragment addresses (the swizzles depend on the row only
    // through bits that the per-block steps 16 kb, 32 c + 16 h do not change).
    //   K:   row 16 kb + ln, logical chunk 4 c + lg
    //   V^T: source lane j = ln of its 16-lane group reads key 32 c + 16 h + 4 lg + ln / 4,
    //        d = 16 db + 4 (ln % 4)
    int koff[S::DC];
#pragma unroll
    for (int c = 0; c < S::DC; ++c) koff[c] = ln * 2 * D + 16 * kswz<D>(ln, 4 * c + lg);
    int voff[S::NDB];
    {
        const int k0 = 4 * lg + (ln >> 2);
        const int d0 = 4 * (ln & 3);
#pragma unroll
        for (int db = 0; db < S::NDB; ++db) {
            const int d = 16 * db + d0;
            voff[db] = k0 * 2 * D + 16 * vswz<D>(k0, d >> 3) + 2 * (d & 7);
        }
    }

    // Keys any row of this wave can see: one interval, since the rows are consecutive.  A tile
    // outside it adds exact zeros to this wave's softmax, so the wave skips its products
    // (it still takes part in the DMA, waits and barriers).
    int wave_lo, wave_hi;
    {
        const int r0 = q0 + qw * S::QB * 16;
        const int r1 = min(r0 + S::QB * 16, a.seq_len) - 1;
        const int p0 = a.kv_len - a.seq_len + r0, p1 = a.kv_len - a.seq_len + r1;
        wave_lo = a.window > 0 ? max(0, p0 - a.window + 1) : 0;
        wave_hi = r1 < r0 ? -1 : (a.causal ? min(p1, a.kv_len - 1) : a.kv_len - 1);
    }
    auto wave_sees = [&](int ks) { return ks <= wave_hi && ks + S::BN - 1 >= wave_lo; };

    // One iteration of the tile loop on LDS stage STG: a run-time int, or a compile-time
    // constant where the loop below is unrolled over the two stages (every LDS address in
    // the body is then a constant offset from one base instead of a per-read computation).
    static_assert(NS == 2, "the tile loop alternates two LDS stages");
    auto iteration = [&](auto STG, int it) {
        const int stage = STG;                 // a constant when STG is an integral_constant
        // this iteration's DMA (issued NS - 1 iterations ago) has landed for every wave, and
        // every wave is done with the stage that the next DMA overwrites
        if constexpr (KS == 1) {
            if (tr.kt0 + it + NS - 2 < tr.kt1) wait_vmem_at_most<2 * S::LI * (NS - 2)>();
            else wait_vmem_at_most<0>();
        } else {
            wait_vmem_at_most<0>();
        }
        __syncthreads();
        {
            const int nxt = it + NS - 1;
            const int sn = (stage + NS - 1) % NS;
            if (tr.kt0 + nxt * KS + kg < tr.kt1)
                f16_dma_tile<D, QB, NWT, NS, BN>(a, kg_ptr, vg, dl, tile_key(tr.kt0 + nxt * KS + kg), w % NWT, lane,
                                                 k_lds[sn][kg], v_lds[sn][kg]);
        }
        const int kt = tr.kt0 + it * KS + kg;
        if ((KS == 1 || kt < tr.kt1) && wave_sees(tile_key(kt))) {
            const char* kl = k_lds[stage][kg];
            const char* vl = v_lds[stage][kg];
            const int ks = tile_key(kt);
            const bool masked = tile_needs_mask(a, tr, ks, S::BN);

            // ---- S^T = K Q^T -----------------------------------------------------------------
            float4_t st[S::NKB][S::QB];
#pragma unroll
            for (int kb = 0; kb < S::NKB; ++kb)
#pragma unroll
                for (int qb = 0; qb < S::QB; ++qb) st[kb][qb] = float4_t{0.f, 0.f, 0.f, 0.f};
            // K fragments are fetched a 32-wide d chunk ahead of their products
            half8_t kf[2][S::NKB];
#pragma unroll
            for (int kb = 0; kb < S::NKB; ++kb)
                kf[0][kb] = *reinterpret_cast<const half8_t*>(kl + koff[0] + 16 * kb * 2 * D);
#pragma unroll
            for (int c = 0; c < S::DC; ++c) {
                if (c + 1 < S::DC) {
#pragma unroll
                    for (int kb = 0; kb < S::NKB; ++kb)
                        kf[(c + 1) & 1][kb] = *reinterpret_cast<const half8_t*>(kl + koff[c + 1] + 16 * kb * 2 * D);
                }
#pragma unroll
                for (int kb = 0; kb < S::NKB; ++kb)
#pragma unroll
                    for (int qb = 0; qb < S::QB; ++qb)
                        st[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[c & 1][kb], qf[qb][c], st[kb][qb], 0, 0, 0);
            }

            // V^T fragments of the tile's first 32 keys, read ahead of the softmax so that their
            // LDS latency overlaps it
            constexpr int NPF = D >= 256 ? S::NDB / 2 : S::NDB;   // register budget
            half8_t vf0[NPF];
#pragma unroll
            for (int db = 0; db < NPF; ++db) {
                const half4_t lo = lds_read_tr16(vl + voff[db]);
                const half4_t hi = lds_read_tr16(vl + voff[db] + 16 * 2 * D);
                vf0[db] = half8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }

            // ---- online softmax in the S^T layout: lane = query (ln), keys 16kb + 4lg + i ----
            // Uncapped scores stay raw (scale > 0 preserves the max); the scale is folded into
            // the exponent: p = 2^(s * scale * log2 e - m).  Capped scores are turned into log2
            // units first.  Masked keys get -inf added.
            half8_t pf[S::QB][S::BN / 32];
#pragma unroll
            for (int qb = 0; qb < S::QB; ++qb) {
                if constexpr (CAP == 1) {
#pragma unroll
                    for (int kb = 0; kb < S::NKB; ++kb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float e2 = fast_exp2(st[kb][qb][i] * K1);
                            st[kb][qb][i] = __builtin_fmaf(-C2, fast_rcp(e2 + 1.f), C1);
                        }
                } else if constexpr (CAP == 2) {
#pragma unroll
                    for (int kb = 0; kb < S::NKB; ++kb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) st[kb][qb][i] = tanh_accurate(st[kb][qb][i] * KX) * C1;
                }
                if (masked) {
                    // visible keys of this row form [vlo, vhi]; key - vlo <= vhi - vlo (unsigned)
                    const int off = ks + 4 * lg - vlo[qb];
#pragma unroll
                    for (int kb = 0; kb < S::NKB; ++kb)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            st[kb][qb][i] = ((unsigned)(off + 16 * kb + i) <= vspan[qb]) ? st[kb][qb][i] : -INFINITY;
                }
                float mx = st[0][qb][0];
#pragma unroll
                for (int kb = 0; kb < S::NKB; ++kb)
#pragma unroll
                    for (int i = (kb == 0 ? 1 : 0); i < 4; ++i) mx = fmaxf(mx, st[kb][qb][i]);
                mx = rows_max(mx);
                const float mxl = mx * sc2;        // in log2 units
                if (__builtin_amdgcn_ballot_w64(mxl > m_run[qb] + kSlack) != 0) {
                    const float mnew = fmaxf(m_run[qb], mxl);
                    const float alpha = fast_exp2(m_run[qb] - mnew);
                    m_run[qb] = mnew;
                    acc_l[qb] *= alpha;
#pragma unroll
                    for (int db = 0; db < S::NDB; ++db) acc_o[db][qb] *= alpha;
                }
                const float mq = m_run[qb];
#pragma unroll
                for (int kb = 0; kb < S::NKB; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) st[kb][qb][i] = fast_exp2(__builtin_fmaf(st[kb][qb][i], sc2, -mq));
#pragma unroll
                for (int c = 0; c < S::BN / 32; ++c) {
                    const half2_t h0 = __builtin_convertvector(float2_t{st[2 * c][qb][0], st[2 * c][qb][1]}, half2_t);
                    const half2_t h1 = __builtin_convertvector(float2_t{st[2 * c][qb][2], st[2 * c][qb][3]}, half2_t);
                    const half2_t h2 = __builtin_convertvector(float2_t{st[2 * c + 1][qb][0], st[2 * c + 1][qb][1]}, half2_t);
                    const half2_t h3 = __builtin_convertvector(float2_t{st[2 * c + 1][qb][2], st[2 * c + 1][qb][3]}, half2_t);
                    pf[qb][c] = half8_t{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
                    // row sums of P on the matrix core: a block of ones times P^T
                    acc_l[qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pf[qb][c], acc_l[qb], 0, 0, 0);
                }
            }

            // ---- O^T += V^T P^T ---------------------------------------------------------------
#pragma unroll
            for (int c = 0; c < S::BN / 32; ++c) {
#pragma unroll
                for (int db = 0; db < S::NDB; ++db) {
                    half8_t vf;
                    if (c == 0 && db < NPF) {
                        vf = vf0[db];
                    } else {
                        const half4_t lo = lds_read_tr16(vl + voff[db] + (32 * c) * 2 * D);
                        const half4_t hi = lds_read_tr16(vl + voff[db] + (32 * c + 16) * 2 * D);
                        vf = half8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    }
#pragma unroll
                    for (int qb = 0; qb < S::QB; ++qb)
                        acc_o[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[qb][c], acc_o[db][qb], 0, 0, 0);
                }
            }
        }
    };
    const int n_it = (tr.kt1 - tr.kt0 + KS - 1) / KS;
    if constexpr (KS > 1) {
        // key groups: unrolled over the two stages (constant LDS offsets; 37 against 43 us
        // for the 512-token chunk after a 3584-token cache)
        for (int it = 0; it < n_it; it += 2) {
            iteration(std::integral_constant<int, 0>{}, it);
            if (it + 1 < n_it) iteration(std::integral_constant<int, 1>{}, it + 1);
        }
    } else {
        // one body with the stage chosen at run time: the unrolled form precomputes an LDS
        // address per fragment read and per stage, which costs these configurations their
        // occupancy (head_dim 256 spills)
        for (int it = 0; it < n_it; ++it) iteration(it & 1, it);
    }

    if constexpr (KS > 1) {
        // ---- merge the key groups: groups 1 .. KS-1 leave (m, l, O^T) in LDS per lane ------
        constexpr int PS = 4 * S::NDB + 2;                       // floats per lane
        static_assert(sizeof(float) * (KS - 1) * S::NWQ * 64 * PS <= sizeof(k_lds), "merge buffer fits");
        float* buf = reinterpret_cast<float*>(&k_lds[0][0][0]);
        __syncthreads();                                         // every wave is done with the tiles
        if (kg > 0) {
            float* mine = buf + (((kg - 1) * S::NWQ + qw) * 64 + lane) * PS;
#pragma unroll
            for (int db = 0; db < S::NDB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) mine[4 * db + i] = acc_o[db][0][i];
            mine[4 * S::NDB] = acc_l[0][0];
            mine[4 * S::NDB + 1] = m_run[0];
        }
        __syncthreads();
        if (kg > 0) return;
        float mx = m_run[0];
#pragma unroll
        for (int g = 1; g < KS; ++g) mx = fmaxf(mx, buf[(((g - 1) * S::NWQ + qw) * 64 + lane) * PS + 4 * S::NDB + 1]);
        const float f0 = fast_exp2(m_run[0] - mx);
        float lsum = acc_l[0][0] * f0;
#pragma unroll
        for (int db = 0; db < S::NDB; ++db) acc_o[db][0] *= f0;
#pragma unroll
        for (int g = 1; g < KS; ++g) {
            const float* other = buf + (((g - 1) * S::NWQ + qw) * 64 + lane) * PS;
            const float fg = fast_exp2(other[4 * S::NDB + 1] - mx);
            lsum += fg * other[4 * S::NDB];
#pragma unroll
            for (int db = 0; db < S::NDB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc_o[db][0][i] += fg * other[4 * db + i];
        }
        acc_l[0] = float4_t{lsum, lsum, lsum, lsum};
    }

    // ---- epilogue: O = (O^T)^T / l ---------------------------------------------------------
    _Float16* og = reinterpret_cast<_Float16*>(a.o) + (long)head * a.o_head;
#pragma unroll
    for (int qb = 0; qb < S::QB; ++qb) {
        const float l = acc_l[qb][0];
        const float inv = l != 0.f ? 1.0f / l : 0.f;
        const int row = q0 + (qw * S::QB + qb) * 16 + ln;
        if (row < a.seq_len) {
#pragma unroll
            for (int db = 0; db < S::NDB; ++db) {
                const half2_t lo = __builtin_convertvector(float2_t{acc_o[db][qb][0] * inv, acc_o[db][qb][1] * inv}, half2_t);
                const half2_t hi = __builtin_convertvector(float2_t{acc_o[db][qb][2] * inv, acc_o[db][qb][3] * inv}, half2_t);
                *reinterpret_cast<half4_t*>(og + (long)row * a.o_row + 16 * db + 4 * lg) =
                    half4_t{lo[0], lo[1], hi[0], hi[1]};
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
    static constexpr int BN = D <= 128 ? 64 : 32; // keys per tile (staging registers bound D 256)
    static constexpr int LD = D + 1;              // LDS row stride (floats)
    static constexpr int CH = BN * D / 4 / 256;   // float4 chunks per thread per tile (K or V)
    static constexpr int NKB = BN / 16;
    static constexpr int NDB = D / 16;
    static constexpr int DC = D / 4;
};

// KG (key groups, for grids too small to fill the device): the four waves share one 16-row
// query block and wave w takes key block w (16 keys) of every tile, so each wave does a
// quarter of the products; the four partial softmaxes are folded by log-sum-exp at the end.
template <int D, bool CAP, bool KG>
__global__ void __launch_bounds__(256) fwd_f32_kernel(FwdParams a) {
    using S = F32Shape<D>;
    constexpr int BM = KG ? 16 : S::BM;
    constexpr int NKBW = KG ? 1 : S::NKB;          // key blocks of a tile per wave
    static_assert(!KG || S::NKB == 4, "key groups take one of the four 16-key blocks of a tile");
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
    const int q0 = qblock * BM;
    if (!resolve_kv_len<float, D>(a, head, q0, BM)) return;
    const TileRange tr = tile_range(a, q0, BM, S::BN);

    const float* qg = reinterpret_cast<const float*>(a.q) + (long)head * a.q_head;
    const float* kg = reinterpret_cast<const float*>(a.k) + (long)kvh * a.k_head;
    const float* vg = reinterpret_cast<const float*>(a.v) + (long)kvh * a.k_head;

    const int row = q0 + (KG ? 0 : w * 16) + ln;
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

        // NKBW independent accumulation chains, interleaved; key block kbi(kb) of the tile
        auto kbi = [&](int kb) { return KG ? w : kb; };
        float4_t st[NKBW];
#pragma unroll
        for (int kb = 0; kb < NKBW; ++kb) st[kb] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < S::DC; ++c)
#pragma unroll
            for (int kb = 0; kb < NKBW; ++kb) {
                const float kf = k_lds[(16 * kbi(kb) + ln) * S::LD + 4 * c + lg];
                st[kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf, qf[c], st[kb], 0, 0, 0);
            }
#pragma unroll
        for (int kb = 0; kb < NKBW; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) st[kb][i] = score_transform<CAP>(a, st[kb][i]);
        if (masked) {
#pragma unroll
            for (int kb = 0; kb < NKBW; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    st[kb][i] = visible(a, ks + 16 * kbi(kb) + 4 * lg + i, qpos) ? st[kb][i] : -INFINITY;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKBW; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, st[kb][i]);
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
        for (int kb = 0; kb < NKBW; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = fast_exp2(st[kb][i] - m_run);
                st[kb][i] = p;
                l_part += p;
            }
        // O^T += V^T P^T, four keys {16kb + 4g + i : g} per product; the NDB output blocks
        // are independent chains, interleaved
#pragma unroll
        for (int kb = 0; kb < NKBW; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int db = 0; db < S::NDB; ++db) {
                    const float vf = v_lds[(16 * kbi(kb) + 4 * lg + i) * S::LD + 16 * db + ln];
                    acc_o[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf, st[kb][i], acc_o[db], 0, 0, 0);
                }
    }

    float l = l_part;
    l += shfl_xor_f(l, 16);
    l += shfl_xor_f(l, 32);
    float* og = reinterpret_cast<float*>(a.o) + (long)head * a.o_head;
    if constexpr (KG) {
        // Fold the four key groups.  The tile buffers are free after the barrier: O^T
        // partials [wave][d][column] go to k_lds for d < D/2 and to v_lds for the rest
        // (4 * D/2 * 16 floats each, within BN * LD), maxima and sums to kg_ml.
        __shared__ float kg_ml[2][4][16];
        auto po = [&](int ww, int d) -> float& {
            return d < D / 2 ? k_lds[(ww * (D / 2) + d) * 16 + ln] : v_lds[(ww * (D / 2) + d - D / 2) * 16 + ln];
        };
        __syncthreads();
#pragma unroll
        for (int db = 0; db < S::NDB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) po(w, 16 * db + 4 * lg + i) = acc_o[db][i];
        if (lg == 0) {
            kg_ml[0][w][ln] = m_run;
            kg_ml[1][w][ln] = l;
        }
        __syncthreads();
        float M = kg_ml[0][0][ln];
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) M = fmaxf(M, kg_ml[0][ww][ln]);
        float f[4], L = 0.f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
            f[ww] = fast_exp2(kg_ml[0][ww][ln] - M);
            L += f[ww] * kg_ml[1][ww][ln];
        }
        const float inv = L != 0.f ? 1.0f / L : 0.f;
        if (row < a.seq_len) {
            // wave w writes the output tiles db = w, w + 4, ...
            for (int db = w; db < S::NDB; db += 4) {
                float r[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float o = 0.f;
#pragma unroll
                    for (int ww = 0; ww < 4; ++ww) o += f[ww] * po(ww, 16 * db + 4 * lg + i);
                    r[i] = o * inv;
                }
                *reinterpret_cast<float4*>(og + (long)row * a.o_row + 16 * db + 4 * lg) = float4{r[0], r[1], r[2], r[3]};
            }
        }
        return;
    }
    const float inv = l != 0.f ? 1.0f / l : 0.f;
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

// Tile configuration per head_dim: 16-row blocks per wave, waves per workgroup, LDS stages,
// keys per tile.  head_dim 64 uses three waves (48 query rows) and 96-key tiles: 48 KB of
// LDS per workgroup, three workgroups per compute unit, and a 2304-row, 16-head vision
// call comes to 768 workgroups, three per compute unit, with no tail.
template <int D> struct F16Cfg;
template <> struct F16Cfg<64> { static constexpr int QB = 1, NW = 3, NS = 2, BN = 96, KS = 1; };
template <> struct F16Cfg<128> { static constexpr int QB = 1, NW = 4, NS = 2, BN = 64, KS = 1; };
template <> struct F16Cfg<256> { static constexpr int QB = 1, NW = 8, NS = 2, BN = 64, KS = 1; };

// Grids of fewer workgroups than compute units (a short chunk, few heads): 32 query rows
// per workgroup and four key groups of two waves, 8 KB tiles (128 KB of LDS, one workgroup
// per compute unit), so each compute unit runs eight waves that each walk a quarter of the
// keys.  head_dim 256 keeps its configuration.
template <int D> struct F16Small;
template <> struct F16Small<64> { static constexpr int QB = 1, NW = 8, NS = 2, BN = 64, KS = 4; };
template <> struct F16Small<128> { static constexpr int QB = 1, NW = 8, NS = 2, BN = 32, KS = 4; };
constexpr int kComputeUnits = 256;

template <int D>
constexpr int std_rows() { return F16Cfg<D>::QB * (F16Cfg<D>::NW / F16Cfg<D>::KS) * 16; }

bool use_small(int head_dim, int dtype, int seq_len, int H) {
    if (dtype != 1 || (head_dim != 64 && head_dim != 128)) return false;
    const int bm = head_dim == 64 ? std_rows<64>() : std_rows<128>();
    return (long)((seq_len + bm - 1) / bm) * H < kComputeUnits;
}

// Largest logit cap taken by the exponential identity alone (kernel CAP mode 1).
constexpr float kFastCapMax = 64.f;

template <int D, typename C>
hipError_t launch_f16(const FwdParams& p, dim3 grid, hipStream_t st) {
    if (p.softcap > kFastCapMax)
        hipLaunchKernelGGL((fwd_f16_kernel<D, C::QB, C::NW, C::NS, C::BN, C::KS, 2>), grid, dim3(64 * C::NW), 0, st, p);
    else if (p.softcap > 0.f)
        hipLaunchKernelGGL((fwd_f16_kernel<D, C::QB, C::NW, C::NS, C::BN, C::KS, 1>), grid, dim3(64 * C::NW), 0, st, p);
    else
        hipLaunchKernelGGL((fwd_f16_kernel<D, C::QB, C::NW, C::NS, C::BN, C::KS, 0>), grid, dim3(64 * C::NW), 0, st, p);
    return hipGetLastError();
}

// f32 grids of fewer than 64 workgroups of 64 rows run key groups (16-row workgroups), where
// a tile holds four 16-key blocks (head_dim 64 and 128: 64-key tiles).
bool use_f32_key_groups(int head_dim, int seq_len, int H) {
    return head_dim <= 128 && (long)((seq_len + 63) / 64) * H < 64;
}

template <int D, bool KG>
hipError_t launch_f32(const FwdParams& p, dim3 grid, hipStream_t st) {
    if (p.softcap > 0.f)
        hipLaunchKernelGGL((fwd_f32_kernel<D, true, KG>), grid, dim3(256), 0, st, p);
    else
        hipLaunchKernelGGL((fwd_f32_kernel<D, false, KG>), grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdParams& p, int dtype, hipStream_t st) {
    const dim3 grid(p.n_qblocks * p.H);
    if (dtype == 1) {
        if constexpr (D != 256) {
            if (use_small(D, dtype, p.seq_len, p.H)) return launch_f16<D, F16Small<D>>(p, grid, st);
        }
        return launch_f16<D, F16Cfg<D>>(p, grid, st);
    }
    if constexpr (F32Shape<D>::NKB == 4) {
        if (use_f32_key_groups(D, p.seq_len, p.H)) return launch_f32<D, true>(p, grid, st);
    }
    return launch_f32<D, false>(p, grid, st);
}

}  // namespace

int fwd_block_rows(int head_dim, int dtype, int seq_len, int H) {
    if (dtype != 1) return use_f32_key_groups(head_dim, seq_len, H) ? 16 : F32Shape<64>::BM;
    if (use_small(head_dim, dtype, seq_len, H))
        return head_dim == 64 ? F16Small<64>::QB * (F16Small<64>::NW / F16Small<64>::KS) * 16
                              : F16Small<128>::QB * (F16Small<128>::NW / F16Small<128>::KS) * 16;
    switch (head_dim) {
        case 64: return std_rows<64>();
        case 128: return std_rows<128>();
        default: return std_rows<256>();
    }
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
