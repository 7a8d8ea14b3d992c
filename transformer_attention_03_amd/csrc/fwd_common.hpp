// Helpers shared by the f16/f32 forward kernels (fwd.hip) and the two-block pipelined f16
// forward kernel (fwd2.hip): tile ranges and masks, the device kv length, the work-item
// map, LDS swizzles and the global->LDS DMA of K/V tiles.
#pragma once

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
    // bitwise, not short-circuit: evaluated for every element of an edge tile
    return (key < a.kv_len) & ((a.causal == 0) | (key <= pos)) & ((a.window <= 0) | (pos - key < a.window));
}

// kv length from device memory (chunked prefill against a cache whose length is only known
// on the device, e.g. under graph replay): a.kv_len then holds the capacity of K/V.  A
// length outside [seq_len, capacity] is out of contract: the workgroup writes NaN to its
// rows and returns false.
template <typename T, int D>
__device__ __forceinline__ bool resolve_kv_len(FwdParams& a, int head, int q0, int bm) {
    if (a.kv_len_dev == nullptr) return true;
    const int L = *a.kv_len_dev;
    if (L >= a.seq_len && L <= a.kv_len) {
        a.kv_len = L;
        return true;
    }
    T* og = reinterpret_cast<T*>(a.o) + (long)head * a.o_head;
    const int rows = min(bm, a.seq_len - q0);
    for (int i = threadIdx.x; i < rows * D; i += blockDim.x)
        og[(long)(q0 + i / D) * a.o_row + i % D] = (T)__builtin_nanf("");
    return false;
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

// Scaled score in log2 units, capped when CAP (a compile-time choice, so the per-element
// code has no branch).
template <bool CAP>
__device__ __forceinline__ float score_transform(const FwdParams& a, float s) {
    if constexpr (CAP) return a.softcap * tanh_accurate(s * a.scale * a.inv_softcap) * kLog2e;
    return s * a.scale_log2;
}

// =============================================================================================
// f16 inputs, f32 accumulation: v_mfma_f32_16x16x32_f16
// =============================================================================================
//
// K and V tiles go from HBM/L2 straight into LDS with global_load_lds_dwordx4 (no staging
// registers, no VALU), into a ring of NS stages so that the loads of the next NS-1 tiles
// are in flight while a tile is computed.  Both tiles keep the natural [key][d] layout;
// their 16-byte chunks are XOR-swizzled by key so that fragment reads hit distinct banks
// (the DMA places lane l of a wave at base + 16 l, so rows cannot be padded).
//   QK^T:  A = K fragment, one ds_read_b128 per lane (16 keys x 32 d),
//   PV:    A = V^T fragment, two ds_read_b64_tr_b16 per lane: within a 16-lane group,
//          lane j points at V[key_0 + j/4][d_0 + 4 (j%4)] and lane i receives
//          V[key_0 + k][d_0 + i] for k = 0..3, which is the transposed operand.

template <int D, int QB_, int NW_, int NS_, int BN_, int KS_ = 1>
struct F16Shape {
    static constexpr int NW = NW_;                // waves per workgroup
    static constexpr int QB = QB_;                // 16-row query blocks per wave
    static constexpr int NS = NS_;                // LDS ring stages
    static constexpr int KS = KS_;                // key groups: waves that share query rows
    static constexpr int NWQ = NW / KS;           // waves per key group
    static constexpr int NT = 64 * NW;
    static constexpr int BM = NWQ * QB * 16;      // query rows per workgroup
    static constexpr int BN = BN_;                // keys per tile (a multiple of 32)
    static constexpr int TILE = BN * D * 2;       // bytes of one K (or V) tile
    static constexpr int LI = TILE / 1024 / NW;   // 1 KB DMA loads per wave per tile, K or V
    static constexpr int DC = D / 32;             // 32-wide k chunks of the QK^T product
    static constexpr int NDB = D / 16;            // 16-row d blocks of O^T
    static constexpr int NKB = BN / 16;           // 16-key blocks of S^T
    static_assert(LI >= 1 && LI * 1024 * NW == TILE && BN % 32 == 0, "tile split");
};

// Physical 16-byte chunk of logical chunk c in K row r / V row r.
template <int D>
__device__ __forceinline__ int kswz(int r, int c) { return c ^ (D >= 128 ? (r & 15) : ((r >> 1) & 7)); }
template <int D>
__device__ __forceinline__ int vswz(int r, int c) {
    // pairs of chunks stay adjacent (the transposing reads take 32 bytes of a row); with
    // 128-byte rows two rows share a 256-byte bank line, so the row's low bit is left out
    return c ^ (D >= 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3));
}

template <int N>
__device__ __forceinline__ void wait_vmem_at_most() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// 16 bytes per lane from global memory straight into LDS at lds_base + 16 * lane.  Issued
// as inline asm so that the compiler does not guard every later LDS read with a full
// vector-memory wait (it cannot tell that the ring stage being filled is not the one being
// read); completion is tracked explicitly with wait_vmem_at_most + a barrier.  m0 is
// written here and is used by nothing else in these kernels.
__device__ __forceinline__ void dma16(const void* gptr, const void* lds_base) {
    const uint32_t off = lds_offset(lds_base);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(off)), "v"(gptr)
                 : "memory", "m0");
}

// Per-lane byte offsets of the DMA loads of one tile: load j of this wave covers LDS bytes
// [(j * NW + w) * 1024, +1024); lane l's 16 bytes hold chunk p of row r of the tile.
template <int D, int QB, int NW, int NS, int BN>
struct DmaLane {
    using S = F16Shape<D, QB, NW, NS, BN>;
    int r[S::LI];            // tile row (key offset) of load j
    uint32_t kg[S::LI];      // byte offset of the K chunk from the tile's first key row
    uint32_t vg[S::LI];      // same for V
};

template <int D, int QB, int NW, int NS, int BN>
__device__ __forceinline__ void dma_lane_init(DmaLane<D, QB, NW, NS, BN>& L, const FwdParams& a, int w,
                                              int lane) {
    using S = F16Shape<D, QB, NW, NS, BN>;
#pragma unroll
    for (int j = 0; j < S::LI; ++j) {
        const int byte = (j * NW + w) * 1024 + 16 * lane;
        const int r = byte / (2 * D), p = (byte % (2 * D)) / 16;
        L.r[j] = r;
        L.kg[j] = (uint32_t)(r * a.k_row * 2 + 16 * kswz<D>(r, p));
        L.vg[j] = (uint32_t)(r * a.k_row * 2 + 16 * vswz<D>(r, p));
    }
}

// DMA one K tile and one V tile (keys ks .. ks+BN-1, clamped to kv_len) into an LDS stage.
template <int D, int QB, int NW, int NS, int BN>
__device__ __forceinline__ void f16_dma_tile(const FwdParams& a, const char* kg, const char* vg,
                                             const DmaLane<D, QB, NW, NS, BN>& L, int ks, int w,
                                             int lane, char* k_dst, char* v_dst) {
    using S = F16Shape<D, QB, NW, NS, BN>;
    const long row_bytes = a.k_row * 2;
    if (ks + S::BN <= a.kv_len) {
        const char* kt = kg + ks * row_bytes;
        const char* vt = vg + ks * row_bytes;
#pragma unroll
        for (int j = 0; j < S::LI; ++j) {
            const int off = (j * NW + w) * 1024;
            dma16(kt + L.kg[j], k_dst + off);
            dma16(vt + L.vg[j], v_dst + off);
        }
    } else {
        // ragged last tile: rows past kv_len repeat the last key (masked out later)
#pragma unroll
        for (int j = 0; j < S::LI; ++j) {
            const int off = (j * NW + w) * 1024;
            const int key = min(ks + L.r[j], a.kv_len - 1);
            const long shift = (long)(key - ks - L.r[j]) * row_bytes;
            dma16(kg + ks * row_bytes + shift + L.kg[j], k_dst + off);
            dma16(vg + ks * row_bytes + shift + L.vg[j], v_dst + off);
        }
    }
}

typedef short short4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half4_t lds_read_tr16(const char* p) {
    const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) short4_t*)lds_offset(p));
    return __builtin_bit_cast(half4_t, v);
}

}  // namespace

}  // namespace ta03
