// Split-KV single-token decode for gfx950, on the matrix cores.
//
// One query token per sequence attends over a KV cache held either as contiguous f16
// rows ([num_kv_heads][kv_len][D], f32 query) or as 16-token pages of symmetric int8 rows
// with one f32 scale per (token, kv head) (doppler gpu/kernels/attention.js: the _f16kv
// decode variants take f32 Q with f16 K/V; executeAttentionTieredQuant reads packed int8
// K/V with separate K and V scale buffers and requires f32 Q; kvLayout "paged" with
// pageSize and a page table; kvLenSource = 1 reads kvLen from a buffer).
//
// Work decomposition (ours, not the pages'): grid (split, kv head x head chunk, batch).
// A workgroup owns GC <= 8 query heads that share one KV head (the K/V rows are read once
// for all of them) and a contiguous logical token range.  Each of its NW waves streams
// blocks of 16 tokens through a private ring of RING LDS slots filled by global->LDS DMA
// (every slot is requested at the start and refilled as soon as its block has been
// processed; no staging registers, no barrier between waves).
//
// Both products run as f16 MFMAs with f32 accumulation while keeping f32 accuracy: every
// f32 operand x (the scaled query, and the softmax weight p) is split as
// hi = f16(x), lo = f16(x - hi), and hi and lo occupy two adjacent columns of the 16-wide
// MFMA operand, so column 2g + part of a product holds part of head g.  int8 K/V values
// and f16 K/V values are exact in f16, so each product term is exact and the pair sum
// (one DPP add) restores q.k and p.v to about 2^-22 relative.
//   QK:  S^T[token][col] = K[token][:] . Qx[col][:]       (16x16x32, A = K rows from LDS)
//   PV:  O^T[d][col]    += V^T[d][token] . P^T[token][col] (16x16x16, A = V^T by LDS
//        transposing reads), where P^T comes straight from the S^T accumulator layout.
// The running maximum per head follows the block maxima exactly (every increase rescales),
// so p <= 1.  For int8 V the per-token V scale is folded into p, normalised by a running
// power of two of the largest V scale seen, which keeps the f16 operands in range.
//
// The waves of a workgroup are merged through LDS; the workgroups of one (sequence, KV
// head) are merged by the last one to arrive (log-sum-exp over the split partials),
// counted with a device-scope atomic that this last workgroup resets to zero.  Partials
// travel through device-scope stores and loads, so no cache-wide fence is needed.
//
// Paged addressing is integer-exact: physical page = page_table[b][t >> 4], slot t & 15,
// row ((page * Hkv + kvh) * 16 + slot) * D (pages are head-major, [page][kv head][16][D],
// and so are the scales, [page][kv head][16]: one KV head's block of 16 tokens is one
// contiguous run of rows and of scales).  Rows at or past kv_len are never read: the
// DMA of a block's tail fetches the split's last valid row instead, and those tokens are
// masked, so poisoned slots of a partial last page cannot reach the result.

#include <mutex>

#include "device_common.hpp"
#include "launch.hpp"

namespace ta03 {

namespace {

constexpr int kTB = 16;                  // tokens per block: one MFMA tile
constexpr int kLdsBudget = 136 * 1024;   // ring bytes per workgroup
constexpr int kMaxSplits = 256;          // split partials merged per (sequence, head)
constexpr int kMaxSplitTokens = 4096;    // paged: tokens per workgroup (page slice in LDS)
constexpr int kMergePad = 4;             // floats after each head's row of the wave-merge buffer:
                                         // a wave's writer lanes store the rows of its heads at
                                         // once, and unpadded rows would put them in the same banks

template <int D, bool PAGED>
struct DecShape {
    static constexpr int ESZ = PAGED ? 1 : 2;          // bytes per K/V element
    static constexpr int RB = D * ESZ;                  // bytes per K (or V) row
    static constexpr int TILE = kTB * RB;               // bytes of K (or of V) per block
    static constexpr int SCB = PAGED ? 512 : 0;         // K and V scales of a block
    static constexpr int SLOT = 2 * TILE + SCB;
    // Eight waves with at least two slots each where that fits with room to spare, else
    // four waves; f16: as many slots per wave (up to four) as the budget allows; int8: two
    // slots, so that two workgroups (sixteen waves) share a compute unit.  (At head_dim 256
    // eight int8 waves would fill the budget exactly; four waves with four slots use the
    // same LDS and the block shape of the f16 body, so the tiered kernel can host both.)
    static constexpr int NW = (8 * 2 * SLOT < kLdsBudget) ? 8 : 4;
    static constexpr int RING_FIT = kLdsBudget / (NW * SLOT) >= 4 ? 4 : kLdsBudget / (NW * SLOT);
    static constexpr int RING = PAGED && NW == 8 ? 2 : RING_FIT;
    static constexpr int NT = 64 * NW;
    static constexpr int WAVE_LDS = RING * SLOT;
    static constexpr int TD = TILE / 1024;              // 16-byte DMAs per lane per tile
    static constexpr int NDMA = 2 * TD + (PAGED ? 2 : 0);
    static constexpr int RPL = RB >= 256 ? 1 : 256 / RB;  // rows per 256-byte bank line
    static constexpr int CPR = RB / 16;                 // 16-byte chunks per row
    static constexpr int KC = D / 32;                   // QK MFMA steps
    static constexpr int DT = D / 16;                   // PV output tiles
    static_assert(TILE % 1024 == 0 && CPR >= 4, "tile shape");
    static_assert(RING >= 2, "at least one block in flight while one is processed");
};

// LDS swizzles at 16-byte granularity: chunk c of row r is stored at chunk position
// c ^ sw(r).  K rows are read 16 rows at a time at one chunk, so ksw spreads 16 rows over
// distinct banks; V rows are read in chunk pairs by the transposing loads, so vsw is even
// and keeps each pair adjacent.
template <int RPL>
__device__ __forceinline__ int ksw(int r) {
    if constexpr (RPL == 1) return r & 15;
    else if constexpr (RPL == 2) return (r >> 1) & 7;
    else return (r >> 2) & 3;
}
template <int RPL>
__device__ __forceinline__ int vsw(int r) {
    if constexpr (RPL == 1) return 2 * (r & 7);
    else if constexpr (RPL == 2) return 2 * ((r >> 1) & 3);
    else return 2 * ((r >> 2) & 1);
}

__device__ __forceinline__ int clamp_page(int p, int num_pages) {
    return p < 0 ? 0 : (p >= num_pages ? num_pages - 1 : p);
}

// 16 bytes (dwordx4) or 4 bytes (dword) per lane from global memory straight into LDS, at
// lds_base + size * lane.  Issued as inline asm so that the compiler does not guard later
// LDS reads with full vector-memory waits; completion is tracked per wave with counted
// vmcnt waits.  m0 is written here and is used by nothing else in this kernel.
__device__ __forceinline__ void dma16(const void* gptr, const void* lds_base) {
    const uint32_t off = lds_offset(lds_base);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(off)), "v"(gptr)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* gptr, const void* lds_base) {
    const uint32_t off = lds_offset(lds_base);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(off)), "v"(gptr)
                 : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vmem_at_most() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
// Device-coherent variants (sc1: fetched past the XCD-private L2), for data written by
// workgroups on other XCDs.
__device__ __forceinline__ void dma16_coherent(const void* gptr, const void* lds_base) {
    const uint32_t off = lds_offset(lds_base);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off sc1"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(off)), "v"(gptr)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4_coherent(const void* gptr, const void* lds_base) {
    const uint32_t off = lds_offset(lds_base);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off sc1"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(off)), "v"(gptr)
                 : "memory", "m0");
}
__device__ __forceinline__ void wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// 2^e for integer e (exact); 0 below the normal range.
__device__ __forceinline__ float pow2i(int e) {
    return e < -126 ? 0.f : __int_as_float((min(e, 127) + 127) << 23);
}

// int8 -> f16 for the MFMA operands without any arithmetic: with u = b + 128 (sign bit
// flipped) the f16 bit pattern 0x3C00 | u is exactly 1 + u / 1024.  For such values x a
// product sum obeys  sum y b = 1024 sum y x - 1152 sum y,  so the kernel subtracts the
// second term once per score (K) or once per block and O^T tile (V).  A dword gives the
// f16 pairs (u0, u2) and (u1, u3): the other operand of the product uses the same element
// order.
__device__ __forceinline__ void i8x4_biased(uint32_t w, uint32_t& even, uint32_t& odd) {
    w ^= 0x80808080u;
    even = __builtin_amdgcn_perm(0x3C3C3C3Cu, w, 0x04020400u);
    odd = __builtin_amdgcn_perm(0x3C3C3C3Cu, w, 0x04030401u);
}

struct RowCtx {
    const char* kbase;
    const char* vbase;
    const float* kscales;
    const float* vscales;
    const int* pages;      // paged: physical pages of this split, from logical page page0
    int page0;
    int Hkv, kvh;
    int stride;            // contiguous: rows per KV head
    int ring, ring_base;   // ring: capacity R, and a multiple of R at or below the split's
                           // first token (the split spans at most R tokens)
};

// Row addressing of a cache (or tier): contiguous [Hkv][stride][D], a ring [Hkv][R][D], or
// 16-token pages [P][Hkv][16][D] through a page table.
constexpr int kAddrContig = 0, kAddrRing = 1, kAddrPaged = 2;

// Ring slot of token t (t - ring_base lies in [0, 2R)).
__device__ __forceinline__ int ring_slot(const RowCtx& c, int t) {
    const int tp = t - c.ring_base;
    return tp >= c.ring ? tp - c.ring : tp;
}

// Row index (token t of this KV head) in rows of D elements.
template <int ADDR>
__device__ __forceinline__ size_t row_index(const RowCtx& c, int t) {
    if constexpr (ADDR == kAddrPaged) {
        const int pg = c.pages[(t >> 4) - c.page0];
        return ((size_t)pg * c.Hkv + c.kvh) * 16 + (t & 15);
    } else if constexpr (ADDR == kAddrRing) {
        return (size_t)c.kvh * c.ring + ring_slot(c, t);
    } else {
        return (size_t)c.kvh * c.stride + t;
    }
}

// The same DMAs with a uniform 64-bit base in SGPRs and a 32-bit per-lane offset.
__device__ __forceinline__ uint64_t uniform_ptr(const void* p) {
    const uint64_t b = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, const void* lds_base) {
    const uint32_t off = lds_offset(lds_base);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(off)), "v"(voff), "s"(uniform_ptr(sbase))
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4s(const void* sbase, uint32_t voff, const void* lds_base) {
    const uint32_t off = lds_offset(lds_base);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(off)), "v"(voff), "s"(uniform_ptr(sbase))
                 : "memory", "m0");
}

// Per-lane byte offsets, relative to a block's first row, of the 16-byte chunks this lane
// moves when the block's 16 rows are RS bytes apart in memory (a full block; paged, one
// page; rows are adjacent in every layout).  Slot layout: K tile, V tile, 256 bytes of K scales, 256 bytes of V scales.
template <int D, bool PAGED>
struct DmaLane {
    uint32_t k[DecShape<D, PAGED>::TD];
    uint32_t v[DecShape<D, PAGED>::TD];
    uint32_t sc;           // paged: scale of row lane & 15 (byte offset in the page's run of 16)
};

template <int D, bool PAGED>
__device__ __forceinline__ DmaLane<D, PAGED> dma_lane(int lane, uint32_t rs) {
    using S = DecShape<D, PAGED>;
    DmaLane<D, PAGED> L;
#pragma unroll
    for (int i = 0; i < S::TD; ++i) {
        const int p = 1024 * i + 16 * lane;
        const int r = p / S::RB, cpos = (p % S::RB) / 16;
        L.k[i] = r * rs + 16 * (cpos ^ ksw<S::RPL>(r));
        L.v[i] = r * rs + 16 * (cpos ^ vsw<S::RPL>(r));
    }
    L.sc = (uint32_t)(lane & 15) * 4u;
    return L;
}

// DMA the block of tokens tb .. tb+15 into a ring slot (row r of a tile = token tb + r,
// swizzled chunks; int8: scale areas, row r at 4r).  A full block (and, paged, one whose 16
// tokens share a page; ring, one that does not wrap) takes the uniform-base path; otherwise
// every lane resolves its own row, and tokens at or past t_end fetch the row of token
// t_end - 1.  PAGED is the int8 format (with scales); ADDR the row addressing.
template <int D, bool PAGED, int ADDR>
__device__ __forceinline__ void dma_block(char* slot, const RowCtx& c, const DmaLane<D, PAGED>& L,
                                          int tb, int t_end, int lane) {
    using S = DecShape<D, PAGED>;
    constexpr bool RING = ADDR == kAddrRing;
    const int slot0 = RING ? ring_slot(c, tb) : 0;
    const bool full = tb + kTB <= t_end && (ADDR != kAddrPaged || (tb & 15) == 0) && (!RING || slot0 + kTB <= c.ring);
    if (full) {
        size_t row0;
        if constexpr (ADDR == kAddrPaged) {
            const int pg = __builtin_amdgcn_readfirstlane(c.pages[(tb >> 4) - c.page0]);
            row0 = ((size_t)pg * c.Hkv + c.kvh) * 16;
        } else if constexpr (RING) {
            row0 = (size_t)c.kvh * c.ring + slot0;
        } else {
            row0 = (size_t)c.kvh * c.stride + tb;
        }
        const char* kb = c.kbase + row0 * S::RB;
        const char* vb = c.vbase + row0 * S::RB;
#pragma unroll
        for (int i = 0; i < S::TD; ++i) {
            dma16s(kb, L.k[i], slot + 1024 * i);
            dma16s(vb, L.v[i], slot + S::TILE + 1024 * i);
        }
        if constexpr (PAGED) {
            // 16 lanes carry the block's 16 scales (the instruction still counts once per wave)
            if (lane < 16) {
                dma4s(c.kscales + row0, L.sc, slot + 2 * S::TILE);
                dma4s(c.vscales + row0, L.sc, slot + 2 * S::TILE + 256);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < S::TD; ++i) {
            const int p = 1024 * i + 16 * lane;
            const int r = p / S::RB, cpos = (p % S::RB) / 16;
            const size_t ri = row_index<ADDR>(c, min(tb + r, t_end - 1));
            dma16(c.kbase + ri * S::RB + 16 * (cpos ^ ksw<S::RPL>(r)), slot + 1024 * i);
            dma16(c.vbase + ri * S::RB + 16 * (cpos ^ vsw<S::RPL>(r)), slot + S::TILE + 1024 * i);
        }
        if constexpr (PAGED) {
            if (lane < 16) {
                // a token's scale has the index of its row
                const size_t si = row_index<ADDR>(c, min(tb + lane, t_end - 1));
                dma4(c.kscales + si, slot + 2 * S::TILE);
                dma4(c.vscales + si, slot + 2 * S::TILE + 256);
            }
        }
    }
}

// Per-wave state of the online softmax for the MFMA column this lane holds.
template <int D>
struct WaveAcc {
    float4_t o[D / 16];   // O^T tiles: column lane % 16, d = 16 dt + 4 (lane / 16) + v
    float m;              // running max of the column's head (log2 units)
    float l;              // this lane's share of the running sum of p
    int e;                // paged: running exponent of the largest V scale (wave-uniform)
};

__device__ __forceinline__ uint32_t rows_max_u(uint32_t x) {
    auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = max((uint32_t)a[0], (uint32_t)a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return max((uint32_t)b[0], (uint32_t)b[1]);
}

// f16 operand of the split product: hi in even columns, lo in odd columns.
__device__ __forceinline__ _Float16 split_part(float x, bool odd) {
    const _Float16 hi = (_Float16)x;
    const _Float16 lo = (_Float16)(x - (float)hi);
    return odd ? lo : hi;
}

// One block of 16 tokens.  full: all 16 tokens are below t_end (no masking).
// Splits per chunk of the final merge: outputs [GC][CS][D] plus m and l [GC][CS] in the rings.
template <int D, int GC, bool PAGED>
constexpr int merge_chunk() {
    constexpr int floats = DecShape<D, PAGED>::NW * DecShape<D, PAGED>::WAVE_LDS / 4;
    constexpr int cs = floats / (GC * (D + 2));
    return cs > kMaxSplits ? kMaxSplits : cs;
}

template <int D, bool PAGED, bool CAP>
__device__ __forceinline__ void process_block(const char* slot, int tb, int t_end, bool full,
                                              float cap_log2, float inv_cap, float qbias,
                                              const half8_t (&qx)[D / 32], WaveAcc<D>& A,
                                              int lane) {
    using S = DecShape<D, PAGED>;
    const char* kt = slot;
    const char* vt = slot + S::TILE;
    const int r16 = lane & 15;     // K row (token) of the A operand; MFMA column
    const int g4 = lane >> 4;      // 16-lane row of the wave
    const bool odd = lane & 1;

    // ---- V^T operands, read ahead of the softmax so the LDS latency overlaps it ----------
    // f16: source lane j gives 4 halves of token row 4 g4 + j/4 at d = 16 dt + 4 (j & 3).
    // int8: one transposing byte read feeds two d tiles: source lane j gives 8 bytes of
    // token row 4 g4 + (j/2 & 3), d tile dt + j/8, half j & 1.
    typedef short s4_t __attribute__((ext_vector_type(4)));
    typedef int i2_t __attribute__((ext_vector_type(2)));
    constexpr int NVR = PAGED ? S::DT / 2 : S::DT;
    uint2 vraw[NVR];
    {
        const int j = lane & 15;
#pragma unroll
        for (int i = 0; i < NVR; ++i) {
            if constexpr (PAGED) {
                const int r = 4 * g4 + ((j >> 1) & 3);
                const char* addr = vt + r * S::RB + 16 * ((2 * i + (j >> 3)) ^ vsw<S::RPL>(r)) + 8 * (j & 1);
                const i2_t w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) i2_t*)lds_offset(addr));
                vraw[i] = __builtin_bit_cast(uint2, w);
            } else {
                const int r = 4 * g4 + (j >> 2);
                const char* addr = vt + r * S::RB + 16 * ((2 * i + ((j & 3) >> 1)) ^ vsw<S::RPL>(r)) + 8 * (j & 1);
                const s4_t w = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s4_t*)lds_offset(addr));
                vraw[i] = __builtin_bit_cast(uint2, w);
            }
        }
    }

    // ---- S^T = K Qx^T (two accumulation chains) ---------------------------------------------
    float4_t sacc2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kc = 0; kc < S::KC; ++kc) {
        half8_t a;
        if constexpr (PAGED) {
            const int c = 2 * kc + (g4 >> 1);
            const uint2 w = *reinterpret_cast<const uint2*>(kt + r16 * S::RB + 16 * (c ^ ksw<S::RPL>(r16)) + 8 * (g4 & 1));
            uint32_t e0, o0, e1, o1;
            i8x4_biased(w.x, e0, o0);
            i8x4_biased(w.y, e1, o1);
            a = __builtin_bit_cast(half8_t, u32x4_t{e0, o0, e1, o1});
        } else {
            const int c = 4 * kc + g4;
            a = *reinterpret_cast<const half8_t*>(kt + r16 * S::RB + 16 * (c ^ ksw<S::RPL>(r16)));
        }
        sacc2[kc & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qx[kc], sacc2[kc & 1], 0, 0, 0);
    }
    const float4_t sacc = sacc2[0] + sacc2[1];

    // scores of tokens tb + 4 g4 + v for this lane's column (hi + lo pair summed)
    float4_t ks = {1.f, 1.f, 1.f, 1.f}, vs = {1.f, 1.f, 1.f, 1.f};
    if constexpr (PAGED) {
        ks = *reinterpret_cast<const float4_t*>(slot + 2 * S::TILE + 16 * g4);
        vs = *reinterpret_cast<const float4_t*>(slot + 2 * S::TILE + 256 + 16 * g4);
    }
    float s[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        float x = sacc[v] + dpp_f<kDppXor1>(sacc[v]);
        if constexpr (PAGED) x = __builtin_fmaf(x, 1024.f, -qbias) * ks[v];
        if constexpr (CAP) x = tanh_accurate(x * inv_cap) * cap_log2;
        s[v] = x;
    }
    if (!full) {
#pragma unroll
        for (int v = 0; v < 4; ++v) s[v] = (tb + 4 * g4 + v < t_end) ? s[v] : -INFINITY;
    }
    const float mb = rows_max(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
    int eb = A.e;
    if constexpr (PAGED) {
        // exponent bound of the block's V scales (tokens past t_end repeat a valid row)
        uint32_t vb = max(max(__float_as_uint(vs[0]) & 0x7FFFFFFFu, __float_as_uint(vs[1]) & 0x7FFFFFFFu),
                          max(__float_as_uint(vs[2]) & 0x7FFFFFFFu, __float_as_uint(vs[3]) & 0x7FFFFFFFu));
        vb = rows_max_u(vb);
        eb = (int)(vb >> 23) - 126;   // |vs| < 2^eb
    }

    // ---- move the running max (and the V-scale exponent) when a block exceeds them ---------
    const bool need = mb > A.m || eb > A.e;
    if (__builtin_amdgcn_ballot_w64(need)) {
        const float mn = fmaxf(A.m, mb);
        const int en = max(A.e, eb);
        const float al = fast_exp2(A.m - mn);          // 0 on the first block (m = -inf)
        const float ao = al * pow2i(A.e - en);
        A.l *= al;
#pragma unroll
        for (int dt = 0; dt < S::DT; ++dt) A.o[dt] *= ao;
        A.m = mn;
        A.e = en;
    }

    // ---- p = 2^(s - m), split into the f16 hi (even column) / lo (odd column) operand ------
    const float pe = PAGED ? pow2i(-A.e) : 1.f;
    float xv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const float p = fast_exp2(s[v] - A.m);
        A.l += p;
        xv[v] = PAGED ? p * vs[v] * pe : p;
    }
    // paged: token order (0, 2, 1, 3), the order of the biased int8 V operand
    const half4_t pb = PAGED ? half4_t{split_part(xv[0], odd), split_part(xv[2], odd),
                                       split_part(xv[1], odd), split_part(xv[3], odd)}
                             : half4_t{split_part(xv[0], odd), split_part(xv[1], odd),
                                       split_part(xv[2], odd), split_part(xv[3], odd)};

    // ---- O^T += V^T P^T --------------------------------------------------------------------
    // int8 V enters as (1152 + v) / 1024.  The bias part, 1.125 * sum_t p_t for every row d, is
    // taken out of each O^T tile block by block (one product with a constant -1.125 operand),
    // so the accumulators keep the size of the output and their f32 rounding does not grow
    // with the number of blocks a wave accumulates.
    if constexpr (PAGED) {
        const half4_t nbias = {(_Float16)-1.125f, (_Float16)-1.125f, (_Float16)-1.125f, (_Float16)-1.125f};
        const float4_t nb = __builtin_amdgcn_mfma_f32_16x16x16f16(nbias, pb, float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int dt = 0; dt < S::DT; ++dt) A.o[dt] += nb;
    }
#pragma unroll
    for (int i = 0; i < NVR; ++i) {
        if constexpr (PAGED) {
            uint32_t e0, o0, e1, o1;
            i8x4_biased(vraw[i].x, e0, o0);
            i8x4_biased(vraw[i].y, e1, o1);
            A.o[2 * i] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, uint2{e0, o0}), pb,
                                                              A.o[2 * i], 0, 0, 0);
            A.o[2 * i + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, uint2{e1, o1}), pb,
                                                                  A.o[2 * i + 1], 0, 0, 0);
        } else {
            A.o[i] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, vraw[i]), pb, A.o[i], 0, 0, 0);
        }
    }
}

// Where a split's K/V rows come from: the cache (or tier) pointers, for a ring its capacity
// and index offset (position t lives at row (t + ring_off) mod ring), for a contiguous
// cache its rows per KV head.
struct TierSrc {
    const void* k;
    const void* v;
    const float* ks;
    const float* vs;
    int ring, ring_off;
    int stride;
};

// 16-byte entries per query chunk in the caller's qx buffer: the f16 bodies stage the f32
// query there first (two float4 per lane); the int8 body loads it straight to registers.
template <bool PAGED>
constexpr int qx_entries() { return PAGED ? 64 : 128; }

// One split: stream tokens [t_begin, t_end) of KV head kvh through the waves, merge the
// waves, and either write the output (a single split) or publish the split's partial
// (m, l, o) for the last-arriving workgroup.  LDS is the caller's, so that one kernel can
// host splits of two cache layouts.
template <int D, int GC, bool PAGED, bool CAP, int ADDR>
__device__ __forceinline__ void split_partial(const DecodeParams& a, const TierSrc& src, char* rings,
                                              float (*lds_m)[GC], float (*lds_l)[GC], int* lds_pages,
                                              half8_t* lds_qx, float (*lds_qs)[64], int b,
                                              int split, int n_live, int t_begin, int t_end, int kvh,
                                              int h0) {
    using S = DecShape<D, PAGED>;
    constexpr int NW = S::NW;
    constexpr int NT = S::NT;
    constexpr int QXN = qx_entries<PAGED>();
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    float(*lds_o)[GC][D + kMergePad] = reinterpret_cast<float(*)[GC][D + kMergePad]>(rings);   // [NW][GC][D + pad]

    RowCtx c;
    c.kbase = reinterpret_cast<const char*>(src.k);
    c.vbase = reinterpret_cast<const char*>(src.v);
    c.kscales = src.ks;
    c.vscales = src.vs;
    c.pages = lds_pages;
    c.page0 = t_begin >> 4;
    c.Hkv = a.Hkv;
    c.kvh = kvh;
    c.stride = src.stride;
    constexpr bool RING = ADDR == kAddrRing;
    c.ring = RING ? src.ring : 0;
    c.ring_base = RING ? ((t_begin + src.ring_off) / src.ring) * src.ring - src.ring_off : 0;
    if constexpr (ADDR == kAddrPaged) {
        // the physical pages of this split, fetched once (clamped into range)
        const int32_t* ptab = a.page_table + (size_t)b * a.max_pages;
        const int np = ((t_end - 1) >> 4) - c.page0 + 1;
        for (int i = threadIdx.x; i < np; i += NT) lds_pages[i] = clamp_page(ptab[c.page0 + i], a.num_pages);
        __syncthreads();
    }

    // ---- this wave's blocks start at first + k * NW * 16; fill the ring ------------------
    constexpr int STRIDE = NW * kTB;
    char* ring = rings + w * S::WAVE_LDS;
    const int first = t_begin + w * kTB;
    const int nb = first < t_end ? (t_end - first + STRIDE - 1) / STRIDE : 0;
    const DmaLane<D, PAGED> dl = dma_lane<D, PAGED>(lane, (uint32_t)S::RB);
    const int col = lane & 15;
    const int hq = col >> 1;
    const float* qh = a.q + ((size_t)b * a.H + h0 + min(hq, GC - 1)) * D + 8 * (lane >> 4);
    // f16 bodies: the query chunks this wave converts come in by DMA ahead of the ring, so a
    // counted wait covers them alone and block 0 can be processed while later blocks are in
    // flight (a plain load would be waited for together with every DMA before it).  The two
    // float4 of a lane land in the 2 KB of qx chunk kc, whose first half becomes qx.
    if constexpr (!PAGED)
        for (int kc = w; kc < S::KC; kc += NW) {
            dma16(qh + 32 * kc, lds_qx + kc * QXN);
            dma16(qh + 32 * kc + 4, lds_qx + kc * QXN + 64);
        }
#pragma unroll
    for (int k = 0; k < S::RING; ++k)
        if (k < nb) dma_block<D, PAGED, ADDR>(ring + k * S::SLOT, c, dl, first + k * STRIDE, t_end, lane);

    // ---- Qx: B operand of the QK product.  Column n = lane % 16 holds part n & 1 of head
    // n / 2 (hi, lo); k = d = 32 kc + 8 (lane / 16) + e, with e in the element order of the
    // K operand (int8: 0 2 1 3 4 6 5 7).  The query is pre-multiplied so that the scores come
    // out in log2 units, or, when a cap is set, as scale * q.k, which the block divides by the
    // cap in f32 (folding 1 / c into the query as well would push it into the f16 subnormals
    // for large caps).
    const float qmul = CAP ? a.scale : a.scale_log2;
    const float cap_log2 = a.softcap * kLog2e;
    // Computed once per workgroup: wave w converts the d chunks kc = w, w + NW, ... and
    // every wave reads all of them back from LDS.
    half8_t qx[S::KC];
    float qbias;
    {
        constexpr int kOrder[8] = {0, 2, 1, 3, 4, 6, 5, 7};
        if constexpr (!PAGED) {
            if (w < S::KC) {
                // the query DMAs were issued before the ring's min(nb, RING) blocks
                const int issued = min(nb, S::RING);
                if constexpr (S::RING >= 4) { if (issued == 4) wait_vmem_at_most<4 * S::NDMA>(); }
                if constexpr (S::RING >= 3) { if (issued == 3) wait_vmem_at_most<3 * S::NDMA>(); }
                if (issued == 2) wait_vmem_at_most<2 * S::NDMA>();
                else if (issued == 1) wait_vmem_at_most<S::NDMA>();
                else if (issued == 0) wait_vmem_at_most<0>();
            }
        }
        for (int kc = w; kc < S::KC; kc += NW) {
            float4_t x0, x1;
            if constexpr (PAGED) {
                x0 = *reinterpret_cast<const float4_t*>(qh + 32 * kc);
                x1 = *reinterpret_cast<const float4_t*>(qh + 32 * kc + 4);
            } else {
                x0 = reinterpret_cast<const float4_t*>(lds_qx + kc * QXN)[lane];
                x1 = reinterpret_cast<const float4_t*>(lds_qx + kc * QXN + 64)[lane];
            }
            const float qf[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
            half8_t h;
            float qs = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = hq < GC ? qf[PAGED ? kOrder[e] : e] * qmul : 0.f;
                h[e] = split_part(x, col & 1);
                qs += (float)h[e];
            }
            lds_qx[kc * QXN + lane] = h;
            lds_qs[kc][lane] = qs;
        }
        __syncthreads();
        float qsum = 0.f;
#pragma unroll
        for (int kc = 0; kc < S::KC; ++kc) {
            qx[kc] = lds_qx[kc * QXN + lane];
            qsum += lds_qs[kc][lane];
        }
        // int8 K: the bias term 1152 * sum_d q[d] of the head (hi + lo columns, all rows)
        qsum = rows_sum(qsum);
        qbias = 1152.f * (qsum + dpp_f<kDppXor1>(qsum));
    }

    WaveAcc<D> A;
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) A.o[dt] = float4_t{0.f, 0.f, 0.f, 0.f};
    A.m = -INFINITY;
    A.l = 0.f;
    A.e = PAGED ? -126 : 0;

    for (int k = 0; k < nb; ++k) {
        // block k has landed once no more than (blocks issued after it) * NDMA loads remain
        const int after = min(S::RING - 1, nb - 1 - k);
        if (after >= 3) wait_vmem_at_most<3 * S::NDMA>();
        else if (after == 2) wait_vmem_at_most<2 * S::NDMA>();
        else if (after == 1) wait_vmem_at_most<S::NDMA>();
        else wait_vmem_at_most<0>();
        const int tb = first + k * STRIDE;
        process_block<D, PAGED, CAP>(ring + (k % S::RING) * S::SLOT, tb, t_end, tb + kTB <= t_end,
                                     cap_log2, a.inv_softcap, qbias, qx, A, lane);
        const int kn = k + S::RING;
        if (kn < nb) {
            // the slot of block k is refilled once this wave's reads of it are done
            wait_lds_reads();
            dma_block<D, PAGED, ADDR>(ring + (k % S::RING) * S::SLOT, c, dl, first + kn * STRIDE, t_end, lane);
        }
    }

    // ---- finish the wave: pair sums (hi + lo columns), row sums over the 16-lane rows ------
    const float lw = rows_sum(A.l);
    const float oscale = PAGED ? pow2i(A.e) : 1.f;
    __syncthreads();                      // every wave is done with its ring
    {
        // all pair sums first, then one 16-byte write per O^T tile under a single mask (a
        // masked write per element costs an exec save/restore each)
        const bool writer = (col & 1) == 0 && hq < GC;
        float4_t ov[S::DT];
#pragma unroll
        for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float o = A.o[dt][v] + dpp_f<kDppXor1>(A.o[dt][v]);
                if constexpr (PAGED) o *= 1024.f;
                ov[dt][v] = o * oscale;
            }
        if (writer) {
#pragma unroll
            for (int dt = 0; dt < S::DT; ++dt)
                *reinterpret_cast<float4_t*>(&lds_o[w][hq][16 * dt + 4 * (lane >> 4)]) = ov[dt];
            if (lane < 16) {
                lds_m[w][hq] = A.m;
                lds_l[w][hq] = lw;
            }
        }
    }
    __syncthreads();

    // ---- merge the waves; finish or publish the split partial ---------------------------
    // A wave's 64 (head, d) pairs share one head (D is a multiple of 64): lane ww < NW takes
    // the weight 2^(m_ww - M) of wave ww's partial once, and the fold reads the weights
    // from those lanes.
    static_assert(D % 64 == 0 && NW <= 16, "one head per wave in the wave merge");
    const size_t part_base = (size_t)b * a.H + h0;   // + g, then * n_split_max
    for (int i = threadIdx.x; i < GC * D; i += NT) {
        const int g = __builtin_amdgcn_readfirstlane(i / D), d = i % D;
        const float mw = lane < NW ? lds_m[lane][g] : -INFINITY;
        const float Mx = group_max<NW>(mw);
        const float f = (mw == -INFINITY) ? 0.f : fast_exp2(mw - Mx);
        const float lsx = group_sum<NW>(lane < NW ? f * lds_l[lane][g] : 0.f);
        float os = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww)
            os = __builtin_fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), ww)), lds_o[ww][g][d], os);
        const float M = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Mx), 0));
        const float ls = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lsx), 0));
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
}

// The last-arriving workgroup of a (sequence, head chunk) merges its n_live split partials
// (log-sum-exp), CS splits at a time through LDS.
template <int D, int GC, int NT, int CS>
__device__ __forceinline__ void merge_splits(const DecodeParams& a, char* rings, int* lds_last, int b,
                                             int h0, int n_live) {
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const size_t part_base = (size_t)b * a.H + h0;
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
        *lds_last = last;
    }
    __syncthreads();
    if (!*lds_last) return;

    // The split partials (device-scope data) are pulled into LDS by DMA, CS splits at a
    // time.  Per chunk, one wave per head takes the chunk's maximum and each split's weight
    // 2^(m_s - M) once (a lane per split), and folds the normaliser; then every thread folds
    // its (head, d) pairs with those weights.  Compact loops: this code runs once per
    // (sequence, head chunk), on a compute unit that has not executed it before.
    float* lds_po = reinterpret_cast<float*>(rings);          // [GC][CS][D]
    float* lds_pm = lds_po + GC * CS * D;                      // [GC][CS]: m, then the weights
    float* lds_pl = lds_pm + GC * CS;                          // [GC][CS]
    __shared__ float lds_f[GC];                                // rescale of the running sums
    __shared__ float lds_L[GC];                                // 1 / final normaliser (0 if none)
    constexpr int NWV = NT / 64;
    constexpr int GPW = (GC + NWV - 1) / NWV;                  // heads per wave
    constexpr int PER = (GC * D + NT - 1) / NT;                // (head, d) pairs per thread
    float Mh[GPW], Lh[GPW];                                    // wave-uniform, head w + NWV j
#pragma unroll
    for (int j = 0; j < GPW; ++j) {
        Mh[j] = -INFINITY;
        Lh[j] = 0.f;
    }
    float acc[PER];
#pragma unroll
    for (int r = 0; r < PER; ++r) acc[r] = 0.f;
    for (int s0 = 0; s0 < n_live; s0 += CS) {
        const int cs = min(CS, n_live - s0);
        // outputs: head g's cs * D floats are contiguous in the workspace and in LDS (a loop
        // per head keeps run-time divisions out of the addresses)
        const int npg = cs * (D / 4);                          // 16-byte pieces per head
#pragma unroll
        for (int g = 0; g < GC; ++g) {
            const float* src = a.part_o + ((part_base + g) * a.n_split_max + s0) * D;
            float* dst = lds_po + g * cs * D;
            for (int c0 = w * 64; c0 < npg; c0 += NT)
                if (c0 + lane < npg) dma16_coherent(src + 4 * (c0 + lane), dst + 4 * c0);
        }
        // m and l: a wave per head, a lane per split
        for (int g = w; g < GC; g += NWV) {
            const size_t row = (part_base + g) * a.n_split_max + s0;
            for (int c0 = 0; c0 < cs; c0 += 64)
                if (c0 + lane < cs) {
                    dma4_coherent(a.part_m + row + c0 + lane, lds_pm + g * cs + c0);
                    dma4_coherent(a.part_l + row + c0 + lane, lds_pl + g * cs + c0);
                }
        }
        wait_vmem_at_most<0>();
        __syncthreads();
        // LDS now holds outputs at [g][s][d] with stride cs * D per head, and m, l at [g][s]
#pragma unroll
        for (int j = 0; j < GPW; ++j) {
            const int g = w + NWV * j;
            if (g < GC) {
                float mx = -INFINITY;
                for (int s = lane; s < cs; s += 64) mx = fmaxf(mx, lds_pm[g * cs + s]);
                const float mc = fmaxf(Mh[j], rows_max(group_max16(mx)));
                float ls = 0.f;
                for (int s = lane; s < cs; s += 64) {
                    const float ms = lds_pm[g * cs + s];
                    const float wgt = (ms == -INFINITY) ? 0.f : fast_exp2(ms - mc);
                    ls = __builtin_fmaf(wgt, lds_pl[g * cs + s], ls);
                    lds_pm[g * cs + s] = wgt;
                }
                const float f = (Mh[j] == -INFINITY) ? 0.f : fast_exp2(Mh[j] - mc);
                Lh[j] = __builtin_fmaf(Lh[j], f, rows_sum(group_sum<16>(ls)));
                Mh[j] = mc;
                if (lane == 0) {
                    lds_f[g] = f;
                    lds_L[g] = Lh[j] != 0.f ? 1.f / Lh[j] : 0.f;
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            const int i = min(threadIdx.x + r * NT, GC * D - 1);
            const int g = i / D, d = i % D;
            float o = acc[r] * lds_f[g];
#pragma unroll 4
            for (int s = 0; s < cs; ++s) o = __builtin_fmaf(lds_pm[g * cs + s], lds_po[(g * cs + s) * D + d], o);
            acc[r] = o;
        }
        if (s0 + CS < n_live) __syncthreads();                 // the next chunk reuses the buffers
    }
#pragma unroll
    for (int r = 0; r < PER; ++r) {
        const int i = threadIdx.x + r * NT;
        if (i < GC * D) a.o[(part_base + i / D) * D + (i % D)] = acc[r] * lds_L[i / D];
    }
}

template <int D, int GC, bool PAGED, bool CAP, bool RING>
__global__ void __launch_bounds__((DecShape<D, PAGED>::NT)) decode_split_kernel(DecodeParams a) {
    static_assert(!(PAGED && RING), "a ring cache is contiguous f16");
    using S = DecShape<D, PAGED>;
    constexpr int NW = S::NW;
    constexpr int NT = S::NT;
    static_assert(GC >= 1 && GC <= 8, "heads per workgroup");
    // per-wave DMA rings; the wave-merge buffer lds_o reuses this memory afterwards
    __shared__ __attribute__((aligned(1024))) char rings[NW * S::WAVE_LDS];
    __shared__ float lds_m[NW][GC];
    __shared__ float lds_l[NW][GC];
    __shared__ int lds_pages[PAGED ? kMaxSplitTokens / 16 + 1 : 1];
    __shared__ int lds_last;
    __shared__ __attribute__((aligned(1024))) half8_t lds_qx[S::KC][qx_entries<PAGED>()];
    __shared__ float lds_qs[S::KC][64];
    static_assert(sizeof(float) * NW * GC * (D + kMergePad) <= NW * S::WAVE_LDS, "merge buffer fits in the rings");

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = a.group;
    const int nch = a.nch;
    const int kvh = (int)(((unsigned long long)blockIdx.y * a.nch_inv) >> 32);   // blockIdx.y / nch
    const int h0 = kvh * G + ((int)blockIdx.y - kvh * nch) * GC;

    // ---- key range of this sequence, and of this split --------------------------------
    int b, split, n_live, t_begin, t_end, L;
    if constexpr (PAGED) {
        // Balanced splits over the whole batch: workgroup x of this head chunk takes split s
        // of sequence b, where sequence i gets lb_i = ceil(len_i / kMaxSplitTokens) splits
        // plus its share, by length, of the remaining workgroups (at most one block round per
        // wave less than a split).  Every workgroup derives the same assignment from kv_lens.
        // The lengths are read 64 sequences per load, one per lane (each load is a round trip
        // to memory that is busy with the cache stream, so a per-sequence loop would cost
        // microseconds); sums, the prefix of split counts and the owner search are wave-wide.
        const int max_len = a.max_pages * 16;
        auto eff_of = [&](int li) {
            const bool valid = li >= 1 && li <= max_len;
            return valid ? ((a.window > 0 && li > a.window) ? a.window : li) : 0;
        };
        long tot = 0;
        int lb_sum = 0;
        int len0 = 0;                             // lane's length in the first 64 sequences
        for (int i0 = 0; i0 < a.batch; i0 += 64) {
            const int i = i0 + lane;
            const int li = i < a.batch ? a.kv_lens[i] : 0;
            if (i0 == 0) len0 = li;
            const int e = eff_of(li);             // <= 2^20 (host-checked), so 64 fit an int
            const int lb = i < a.batch ? (e > 0 ? (e + kMaxSplitTokens - 1) / kMaxSplitTokens : 1) : 0;
            tot += wave_sum_i(e);
            lb_sum += wave_sum_i(lb);
        }
        const int extra = max(0, (int)gridDim.x - lb_sum);
        const int p = blockIdx.x;
        int cum = 0, nb_b = 0;
        b = -1;
        L = 0;
        for (int i0 = 0; i0 < a.batch && b < 0; i0 += 64) {
            const int i = i0 + lane;
            const int li = i < a.batch ? (i0 == 0 ? len0 : a.kv_lens[i]) : 0;
            const int e = eff_of(li);
            const int lb = e > 0 ? (e + kMaxSplitTokens - 1) / kMaxSplitTokens : 1;
            int n = lb + (tot > 0 ? (int)((long)extra * e / tot) : 0);
            n = min(n, max(lb, (e + NW * kTB - 1) / (NW * kTB)));
            n = min(n, a.n_split_max);
            if (i >= a.batch) n = 0;
            const int incl = wave_incl_scan_i(n);  // splits of sequences i0 .. i
            // the owner is the first sequence whose splits reach past workgroup p
            const uint64_t hit = __builtin_amdgcn_ballot_w64(i < a.batch && p < cum + incl);
            if (hit) {
                const int j = __builtin_ctzll(hit);
                b = i0 + j;
                nb_b = __builtin_amdgcn_readlane(n, j);
                cum += __builtin_amdgcn_readlane(incl, j) - nb_b;
                L = __builtin_amdgcn_readlane(li, j);
            } else {
                cum += __builtin_amdgcn_readlane(incl, 63);
            }
        }
        if (b < 0) return;                        // more workgroups than splits
        split = p - cum;
        if (L < 1 || L > max_len) {
            // out of contract: the row becomes NaN; nothing else is read
            if (split == 0)
                for (int i = threadIdx.x; i < GC * D; i += NT)
                    a.o[((size_t)b * a.H + h0 + i / D) * D + (i % D)] = __builtin_nanf("");
            return;
        }
        const int k_lo = (a.window > 0 && L > a.window) ? L - a.window : 0;
        const int eff = L - k_lo;
        const int tsplit = (((eff + nb_b - 1) / nb_b) + 15) & ~15;   // <= kMaxSplitTokens
        n_live = (eff + tsplit - 1) / tsplit;
        if (split >= n_live) return;
        t_begin = k_lo + split * tsplit;
        t_end = min(L, t_begin + tsplit);
    } else {
        split = blockIdx.x;
        b = blockIdx.z;
        L = a.kv_len;
        const int k_lo = (a.window > 0 && L > a.window) ? L - a.window : 0;
        n_live = gridDim.x;                       // the host's split count for this length
        t_begin = k_lo + split * a.split_tokens;
        t_end = min(L, t_begin + a.split_tokens);
    }

    const TierSrc src{a.k, a.v, a.k_scales, a.v_scales, RING ? a.ring : 0, 0, a.kv_len};
    constexpr int ADDR = PAGED ? kAddrPaged : (RING ? kAddrRing : kAddrContig);
    split_partial<D, GC, PAGED, CAP, ADDR>(a, src, rings, lds_m, lds_l, lds_pages, &lds_qx[0][0], lds_qs, b, split,
                                           n_live, t_begin, t_end, kvh, h0);
    if (n_live == 1) return;
    merge_splits<D, GC, NT, merge_chunk<D, GC, PAGED>()>(a, rings, &lds_last, b, h0, n_live);
}

// Tiered decode of one sequence: positions [0, cold_len) sit in a cold tier, positions
// [cold_len, kv_len) in an f16 ring (the hot tier).  The cold tier is int8 with per-row
// scales or f16, either in 16-token pages through a page table or contiguous per KV head
// (COLD, one of the kCold* kinds).  Workgroups [0, n_cold) take splits of the cold tier,
// the rest splits of the hot tier with the f16 ring body; all of them publish partials of
// one online softmax and the last to arrive merges them, exactly as for a single-layout
// cache.  LDS is sized for the larger of the two bodies.
constexpr int kColdI8Paged = 0, kColdI8Contig = 1, kColdF16Paged = 2, kColdF16Contig = 3;

template <int D, int COLD>
constexpr int tier_ring_bytes() {
    using SP = DecShape<D, true>;
    using SF = DecShape<D, false>;
    constexpr int p = SP::NW * SP::WAVE_LDS, f = SF::NW * SF::WAVE_LDS;
    return (COLD == kColdI8Paged || COLD == kColdI8Contig) && p > f ? p : f;
}

template <int D, int GC, int COLD, bool CAP>
__global__ void __launch_bounds__((DecShape<D, true>::NT)) decode_tiered_kernel(DecodeParams a) {
    using SP = DecShape<D, true>;
    using SF = DecShape<D, false>;
    static_assert(SP::NT == SF::NT && SP::NW == SF::NW, "one block shape for both tiers");
    constexpr bool COLD_I8 = COLD == kColdI8Paged || COLD == kColdI8Contig;
    constexpr int COLD_ADDR = (COLD == kColdI8Paged || COLD == kColdF16Paged) ? kAddrPaged : kAddrContig;
    constexpr int NT = SP::NT;
    constexpr int RB = tier_ring_bytes<D, COLD>();
    __shared__ __attribute__((aligned(1024))) char rings[RB];
    __shared__ float lds_m[SP::NW][GC];
    __shared__ float lds_l[SP::NW][GC];
    __shared__ int lds_pages[COLD_ADDR == kAddrPaged ? kMaxSplitTokens / 16 + 1 : 1];
    __shared__ int lds_last;
    __shared__ __attribute__((aligned(1024))) half8_t lds_qx[SP::KC][qx_entries<false>()];   // both bodies
    __shared__ float lds_qs[SP::KC][64];
    static_assert(sizeof(float) * SP::NW * GC * (D + kMergePad) <= RB, "merge buffer fits in the rings");
    constexpr int CS = (RB / 4) / (GC * (D + 2)) > kMaxSplits ? kMaxSplits : (RB / 4) / (GC * (D + 2));

    const int G = a.group;
    const int nch = a.nch;
    const int kvh = (int)(((unsigned long long)blockIdx.y * a.nch_inv) >> 32);   // blockIdx.y / nch
    const int h0 = kvh * G + ((int)blockIdx.y - kvh * nch) * GC;
    const int n_live = gridDim.x;
    const int split = blockIdx.x;
    if (split < a.tier_cold_splits) {
        const int t_begin = a.tier_k_lo + split * a.tier_cold_tokens;
        const int t_end = min(a.tier_cold_len, t_begin + a.tier_cold_tokens);
        const TierSrc src{a.k, a.v, a.k_scales, a.v_scales, 0, 0, a.tier_cold_stride};
        split_partial<D, GC, COLD_I8, CAP, COLD_ADDR>(a, src, rings, lds_m, lds_l, lds_pages, &lds_qx[0][0], lds_qs,
                                                      0, split, n_live, t_begin, t_end, kvh, h0);
    } else {
        const int t_begin = max(a.tier_k_lo, a.tier_cold_len) + (split - a.tier_cold_splits) * a.split_tokens;
        const int t_end = min(a.kv_len, t_begin + a.split_tokens);
        const TierSrc src{a.hot_k, a.hot_v, nullptr, nullptr, a.ring, a.ring_off, 0};
        split_partial<D, GC, false, CAP, kAddrRing>(a, src, rings, lds_m, lds_l, lds_pages, &lds_qx[0][0], lds_qs, 0,
                                                    split, n_live, t_begin, t_end, kvh, h0);
    }
    if (n_live == 1) return;
    merge_splits<D, GC, NT, CS>(a, rings, &lds_last, 0, h0, n_live);
}


template <int D, bool PAGED, bool CAP, bool RING>
hipError_t launch_decode_c(const DecodeParams& p, int gc, dim3 grid, hipStream_t st) {
    const dim3 block(DecShape<D, PAGED>::NT);
    switch (gc) {
        case 1: hipLaunchKernelGGL((decode_split_kernel<D, 1, PAGED, CAP, RING>), grid, block, 0, st, p); break;
        case 2: hipLaunchKernelGGL((decode_split_kernel<D, 2, PAGED, CAP, RING>), grid, block, 0, st, p); break;
        case 4: hipLaunchKernelGGL((decode_split_kernel<D, 4, PAGED, CAP, RING>), grid, block, 0, st, p); break;
        case 8: hipLaunchKernelGGL((decode_split_kernel<D, 8, PAGED, CAP, RING>), grid, block, 0, st, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int D, bool PAGED>
hipError_t launch_decode_d(const DecodeParams& p, int gc, dim3 grid, hipStream_t st) {
    if constexpr (!PAGED) {
        if (p.ring > 0)
            return p.softcap > 0.f ? launch_decode_c<D, false, true, true>(p, gc, grid, st)
                                   : launch_decode_c<D, false, false, true>(p, gc, grid, st);
    }
    return p.softcap > 0.f ? launch_decode_c<D, PAGED, true, false>(p, gc, grid, st)
                           : launch_decode_c<D, PAGED, false, false>(p, gc, grid, st);
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int head_dim, int gc, bool paged, int batch,
                         hipStream_t st) {
    const int nch = (p.H / p.Hkv) / gc;
    // paged: n_wg balanced workgroups per head chunk across the batch; contiguous: splits
    dim3 grid(paged ? p.n_wg : p.n_split_max, p.Hkv * nch, paged ? 1 : batch);
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

namespace {

template <int D, int COLD, bool CAP>
hipError_t launch_tiered_c(const DecodeParams& p, int gc, dim3 grid, hipStream_t st) {
    const dim3 block(DecShape<D, true>::NT);
    switch (gc) {
        case 1: hipLaunchKernelGGL((decode_tiered_kernel<D, 1, COLD, CAP>), grid, block, 0, st, p); break;
        case 2: hipLaunchKernelGGL((decode_tiered_kernel<D, 2, COLD, CAP>), grid, block, 0, st, p); break;
        case 4: hipLaunchKernelGGL((decode_tiered_kernel<D, 4, COLD, CAP>), grid, block, 0, st, p); break;
        case 8: hipLaunchKernelGGL((decode_tiered_kernel<D, 8, COLD, CAP>), grid, block, 0, st, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int D, int COLD>
hipError_t launch_tiered_k(const DecodeParams& p, int gc, dim3 grid, hipStream_t st) {
    return p.softcap > 0.f ? launch_tiered_c<D, COLD, true>(p, gc, grid, st)
                           : launch_tiered_c<D, COLD, false>(p, gc, grid, st);
}

template <int D>
hipError_t launch_tiered_d(const DecodeParams& p, int gc, int cold_kind, dim3 grid, hipStream_t st) {
    switch (cold_kind) {
        case kColdI8Paged: return launch_tiered_k<D, kColdI8Paged>(p, gc, grid, st);
        case kColdI8Contig: return launch_tiered_k<D, kColdI8Contig>(p, gc, grid, st);
        case kColdF16Paged: return launch_tiered_k<D, kColdF16Paged>(p, gc, grid, st);
        case kColdF16Contig: return launch_tiered_k<D, kColdF16Contig>(p, gc, grid, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_tiered(const DecodeParams& p, int head_dim, int gc, int n_splits, bool cold_int8,
                                bool cold_paged, hipStream_t st) {
    const int nch = (p.H / p.Hkv) / gc;
    const dim3 grid(n_splits, p.Hkv * nch, 1);
    const int kind = cold_int8 ? (cold_paged ? kColdI8Paged : kColdI8Contig)
                               : (cold_paged ? kColdF16Paged : kColdF16Contig);
    switch (head_dim) {
        case 64: return launch_tiered_d<64>(p, gc, kind, grid, st);
        case 128: return launch_tiered_d<128>(p, gc, kind, grid, st);
        case 256: return launch_tiered_d<256>(p, gc, kind, grid, st);
    }
    return hipErrorInvalidValue;
}

// ---- library-owned scratch, for callers that cannot allocate ---------------------------------
//
// attn_decode_noalloc keeps the split partials and arrival counters in this array instead of
// a caller workspace.  Each GPU the library runs on holds its own copy (loaded with the code
// object) until the process ends.  In host code the name `scratch` is only a host-side
// stand-in: its device address, different on every GPU, comes from hipGetSymbolAddress with
// that GPU current, once per device, and only that address is ever handed to a kernel.

namespace {

constexpr size_t kScratchBytes = size_t(4) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

__global__ void __launch_bounds__(256) zero_u32_kernel(uint32_t* p, int n) {
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}

}  // namespace

size_t decode_scratch_bytes() { return kScratchBytes; }

hipError_t decode_scratch(void** ptr, hipStream_t st) {
    int dev = 0;
    hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

// Clears n uint32 words on the stream with a kernel (no memset node, so the call can also be
// captured into a graph).
hipError_t zero_words(uint32_t* p, int n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    const int blocks = (n + 255) / 256 < 64 ? (n + 255) / 256 : 64;
    hipLaunchKernelGGL(zero_u32_kernel, dim3(blocks), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

int decode_tokens_per_block() { return kTB; }

int decode_waves(int head_dim, bool paged) {
    if (paged) return head_dim == 64 ? DecShape<64, true>::NW : head_dim == 128 ? DecShape<128, true>::NW : DecShape<256, true>::NW;
    return head_dim == 64 ? DecShape<64, false>::NW : head_dim == 128 ? DecShape<128, false>::NW : DecShape<256, false>::NW;
}

int decode_workgroups_per_cu(int head_dim, bool paged) {
    // 160 KB of LDS per compute unit; besides the rings a workgroup holds up to 6 KB more
    auto per = [](int ring_bytes) { return (160 * 1024) / (ring_bytes + 6144); };
    if (paged)
        return head_dim == 64 ? per(DecShape<64, true>::NW * DecShape<64, true>::WAVE_LDS)
             : head_dim == 128 ? per(DecShape<128, true>::NW * DecShape<128, true>::WAVE_LDS)
                               : per(DecShape<256, true>::NW * DecShape<256, true>::WAVE_LDS);
    return head_dim == 64 ? per(DecShape<64, false>::NW * DecShape<64, false>::WAVE_LDS)
         : head_dim == 128 ? per(DecShape<128, false>::NW * DecShape<128, false>::WAVE_LDS)
                           : per(DecShape<256, false>::NW * DecShape<256, false>::WAVE_LDS);
}

int decode_max_splits() { return kMaxSplits; }

int decode_max_split_tokens_paged() { return kMaxSplitTokens; }

int decode_max_heads_per_workgroup() { return 8; }

}  // namespace ta03
