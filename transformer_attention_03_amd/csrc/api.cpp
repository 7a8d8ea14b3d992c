// C ABI of libattn.so: argument validation, launch planning and error reporting.
// Every argument check runs before the first HIP call, so a rejected call queues nothing.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "attn.h"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";
thread_local int g_split_override = 0;

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return ATTN_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_ptr(const void* p, const char* name) {
    if (!p) return fail(ATTN_ERR_INVALID_ARG, "%s must not be null", name);
    if (!aligned(p, 16)) return fail(ATTN_ERR_INVALID_ARG, "%s must be 16-byte aligned", name);
    return ATTN_OK;
}

int check_heads(int num_heads, int num_kv_heads, int head_dim) {
    if (num_heads < 1 || num_kv_heads < 1)
        return fail(ATTN_ERR_INVALID_ARG, "num_heads (%d) and num_kv_heads (%d) must be >= 1",
                    num_heads, num_kv_heads);
    if (num_heads % num_kv_heads != 0)
        return fail(ATTN_ERR_INVALID_ARG, "num_heads (%d) must be a multiple of num_kv_heads (%d)",
                    num_heads, num_kv_heads);
    if (head_dim < 1) return fail(ATTN_ERR_INVALID_ARG, "head_dim (%d) must be >= 1", head_dim);
    if (head_dim != 64 && head_dim != 128 && head_dim != 256)
        return fail(ATTN_ERR_UNSUPPORTED, "head_dim %d is not built; requires head_dim in {64, 128, 256}",
                    head_dim);
    return ATTN_OK;
}

int check_scalars(int sliding_window, float attn_softcap, float scale) {
    if (sliding_window < 0)
        return fail(ATTN_ERR_INVALID_ARG, "sliding_window (%d) must be >= 0 (0 = off)", sliding_window);
    if (!std::isfinite(attn_softcap) || attn_softcap < 0.f)
        return fail(ATTN_ERR_INVALID_ARG, "attn_softcap must be finite and >= 0 (0 = off)");
    if (!std::isfinite(scale) || !(scale > 0.f))
        return fail(ATTN_ERR_INVALID_ARG, "scale must be finite and > 0");
    return ATTN_OK;
}

#define TRY(x)                      \
    do {                            \
        int _rc = (x);              \
        if (_rc != ATTN_OK) return _rc; \
    } while (0)

constexpr long kMaxElems = 1L << 40;

// q and o hold rows * num_heads * head_dim elements; the split workspace is sized from the
// same product, so capping it keeps every size computation far from overflow.
int check_query_rows(long rows, int num_heads, int head_dim, const char* what) {
    if (rows * num_heads * head_dim > kMaxElems)
        return fail(ATTN_ERR_INVALID_ARG, "%s: %ld query rows of %d heads x %d is too large", what, rows,
                    num_heads, head_dim);
    return ATTN_OK;
}

// ---- decode split plan ----------------------------------------------------------------------

struct DecodePlan {
    int gc;             // query heads per workgroup
    int nch;            // head chunks per KV head
    int split_tokens;   // contiguous: logical tokens per workgroup
    int n_split;        // split partials per (sequence, head): workspace row stride
    int n_wg;           // paged: workgroups per head chunk, balanced over the batch
};

int heads_per_wg(int group) {
    for (int gc : {8, 4, 2, 1})
        if (group % gc == 0) return gc;
    return 1;
}

DecodePlan plan_decode(int batch, int num_heads, int num_kv_heads, int head_dim, int eff_len,
                       bool paged) {
    DecodePlan p;
    const int group = num_heads / num_kv_heads;
    p.gc = heads_per_wg(group);
    p.nch = group / p.gc;
    const int unit = ta03::decode_waves(head_dim, paged) * ta03::decode_tokens_per_block();
    const long resident = 256L * ta03::decode_workgroups_per_cu(head_dim, paged);
    const long chunks = (long)num_kv_heads * p.nch;
    if (paged) {
        // Two rounds of resident workgroups, shared out over the batch by length inside the
        // kernel; every sequence needs at least ceil(len / max split) of them.  An override
        // of the split length asks for about batch * eff_len / override workgroups instead.
        const int max_split = ta03::decode_max_split_tokens_paged();
        const long lbmax = (eff_len + max_split - 1) / max_split;
        long target = (2 * resident + chunks - 1) / chunks;
        if (g_split_override > 0) target = ((long)batch * eff_len + g_split_override - 1) / g_split_override;
        long n_wg = target > (long)batch * lbmax ? target : (long)batch * lbmax;
        if (n_wg > 65535) n_wg = 65535;
        long cap = lbmax + target;
        if (cap > n_wg) cap = n_wg;
        p.n_wg = (int)n_wg;
        p.n_split = (int)cap;
        p.split_tokens = unit;
        return p;
    }
    // Whole rounds of 16-token blocks per wave, at least two; aim for about three waves of
    // workgroups over the resident capacity (256 CUs), which keeps the tail of ragged paged
    // lengths short while the per-workgroup merge stays a small share.
    int t = g_split_override;
    if (t <= 0) {
        const long rows = (long)eff_len * batch * num_kv_heads * p.nch;
        const long want = (rows + 3 * resident - 1) / (3 * resident);
        // short splits: two rounds of blocks per wave; long ones in steps of four rounds
        const long step = want <= 2 * unit ? 2 * unit : 4 * unit;
        t = (int)(((want + step - 1) / step) * step);
    }
    // the merge holds at most decode_max_splits() partials per (sequence, head)
    const int cap = ta03::decode_max_splits();
    if ((eff_len + t - 1) / t > cap) t = (((eff_len + cap - 1) / cap) + 15) / 16 * 16;
    p.split_tokens = t;
    p.n_split = (eff_len + t - 1) / t;
    if (p.n_split < 1) p.n_split = 1;
    p.n_wg = p.n_split;
    return p;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WorkspaceLayout {
    size_t o_off, m_off, l_off, t_off, total;
};

WorkspaceLayout workspace_layout(int batch, int num_heads, int num_kv_heads, int head_dim,
                                 const DecodePlan& p) {
    WorkspaceLayout w;
    const size_t parts = (size_t)batch * num_heads * p.n_split;
    w.o_off = 0;
    w.m_off = w.o_off + align256(parts * head_dim * sizeof(float));
    w.l_off = w.m_off + align256(parts * sizeof(float));
    w.t_off = w.l_off + align256(parts * sizeof(float));
    w.total = w.t_off + align256((size_t)batch * num_kv_heads * p.nch * sizeof(uint32_t));
    return w;
}

// Split partials per (sequence, head) that a workspace sized for max_len holds: the larger
// of the contiguous and paged plans, and at least two (a tiered cache has two tiers).
int workspace_row_splits(int batch, int num_heads, int num_kv_heads, int head_dim, int max_len) {
    int n = 2;
    for (bool paged : {false, true}) {
        const DecodePlan p = plan_decode(batch, num_heads, num_kv_heads, head_dim, max_len, paged);
        if (p.n_split > n) n = p.n_split;
    }
    return n;
}

size_t workspace_bytes_for(int batch, int num_heads, int num_kv_heads, int head_dim, int max_len) {
    DecodePlan p = plan_decode(batch, num_heads, num_kv_heads, head_dim, max_len, false);
    p.n_split = workspace_row_splits(batch, num_heads, num_kv_heads, head_dim, max_len);
    return workspace_layout(batch, num_heads, num_kv_heads, head_dim, p).total;
}

const float kLog2e = 1.4426950408889634f;

void fill_scalars(ta03::DecodeParams& d, int window, float softcap, float scale) {
    d.window = window;
    d.scale = scale;
    d.scale_log2 = scale * kLog2e;
    d.softcap = softcap;
    d.inv_softcap = softcap > 0.f ? 1.0f / softcap : 0.f;
}

int launch_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(ATTN_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

int run_fwd(const void* q, const void* k, const void* v, void* o, int dtype, int seq_len, int kv_len,
            int H, int Hkv, int D, int causal, int window, float softcap, float scale, long q_row,
            long q_head, long k_row, long k_head, long o_row, long o_head, void* stream,
            const char* what, const int32_t* kv_len_dev = nullptr) {
    ta03::FwdParams p;
    p.kv_len_dev = kv_len_dev;
    p.q = q; p.k = k; p.v = v; p.o = o;
    p.q_row = q_row; p.q_head = q_head;
    p.k_row = k_row; p.k_head = k_head;
    p.o_row = o_row; p.o_head = o_head;
    p.seq_len = seq_len; p.kv_len = kv_len;
    p.H = H; p.Hkv = Hkv;
    p.causal = causal; p.window = window;
    p.scale = scale; p.scale_log2 = scale * kLog2e;
    p.softcap = softcap; p.inv_softcap = softcap > 0.f ? 1.0f / softcap : 0.f;
    const int bm = ta03::fwd_block_rows(D, dtype, seq_len, H);
    p.n_qblocks = (seq_len + bm - 1) / bm;
    if ((long)p.n_qblocks * H > 0x7fffffffL)
        return fail(ATTN_ERR_INVALID_ARG, "%s: grid of %ld workgroups exceeds the device limit", what,
                    (long)p.n_qblocks * H);
    return launch_status(ta03::launch_fwd(p, D, dtype, reinterpret_cast<hipStream_t>(stream)), what);
}

// Contiguous or ring f16 decode: kv_len logical tokens (ring: at rows t mod ring), eff of
// them visible (the newest), window as the kernel applies it.
// scratch_owned: the workspace is the library's scratch, whose previous contents are unknown:
// its arrival counters are cleared on the stream before the launch.
int run_decode_contiguous(const float* q, const void* k, const void* v, float* o, int num_heads,
                          int num_kv_heads, int head_dim, int kv_len, int ring, int eff, int window,
                          float attn_softcap, float scale, void* workspace, size_t workspace_bytes,
                          void* stream, const char* what, bool scratch_owned = false) {
    const DecodePlan plan = plan_decode(1, num_heads, num_kv_heads, head_dim, eff, false);
    const WorkspaceLayout wl = workspace_layout(1, num_heads, num_kv_heads, head_dim, plan);
    if (plan.n_split > 1) {
        if (!workspace) return fail(ATTN_ERR_WORKSPACE, "%s: workspace must not be null", what);
        if (!aligned(workspace, 256)) return fail(ATTN_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", what);
        if (workspace_bytes < wl.total)
            return fail(ATTN_ERR_WORKSPACE, "%s: workspace of %zu bytes is smaller than the %zu required", what,
                        workspace_bytes, wl.total);
    }
    if (plan.n_split > 65535 * 32) return fail(ATTN_ERR_INVALID_ARG, "%s: grid too large", what);
    ta03::DecodeParams d{};
    d.q = q; d.k = k; d.v = v; d.o = o;
    char* ws = reinterpret_cast<char*>(workspace);
    d.part_o = reinterpret_cast<float*>(ws + wl.o_off);
    d.part_m = reinterpret_cast<float*>(ws + wl.m_off);
    d.part_l = reinterpret_cast<float*>(ws + wl.l_off);
    d.tickets = reinterpret_cast<uint32_t*>(ws + wl.t_off);
    d.H = num_heads; d.Hkv = num_kv_heads; d.kv_len = kv_len; d.ring = ring;
    d.group = num_heads / num_kv_heads; d.nch = plan.nch;
    d.nch_inv = ((1ull << 32) + plan.nch - 1) / plan.nch;
    d.num_pages = 0; d.max_pages = 0;
    fill_scalars(d, window, attn_softcap, scale);
    d.split_tokens = plan.split_tokens;
    d.n_split_max = plan.n_split;
    if (scratch_owned && plan.n_split > 1) {
        const int n_tickets = (int)((wl.total - wl.t_off) / sizeof(uint32_t));
        const hipError_t e = ta03::zero_words(d.tickets, n_tickets, reinterpret_cast<hipStream_t>(stream));
        if (e != hipSuccess) return launch_status(e, what);
    }
    return launch_status(ta03::launch_decode(d, head_dim, plan.gc, false, 1,
                                             reinterpret_cast<hipStream_t>(stream)),
                         what);
}

}  // namespace

extern "C" {

int attn_prefill(const void* q, const void* k, const void* v, void* o, int dtype, int seq_len,
                 int kv_len, int num_heads, int num_kv_heads, int head_dim, int causal,
                 int sliding_window, float attn_softcap, float scale, void* stream) {
    if (dtype != ATTN_F32 && dtype != ATTN_F16)
        return fail(ATTN_ERR_INVALID_ARG, "attn_prefill: dtype %d is neither ATTN_F32 nor ATTN_F16", dtype);
    TRY(check_ptr(q, "q"));
    TRY(check_ptr(k, "k"));
    TRY(check_ptr(v, "v"));
    TRY(check_ptr(o, "o"));
    if (kv_len < 1) return fail(ATTN_ERR_INVALID_ARG, "attn_prefill: invalid kv_len %d (must be >= 1)", kv_len);
    if (seq_len < 1 || seq_len > kv_len)
        return fail(ATTN_ERR_INVALID_ARG, "attn_prefill: seq_len %d must be in [1, kv_len = %d]", seq_len, kv_len);
    if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID_ARG, "attn_prefill: causal must be 0 or 1");
    TRY(check_heads(num_heads, num_kv_heads, head_dim));
    TRY(check_scalars(sliding_window, attn_softcap, scale));
    if ((long)kv_len * num_kv_heads * head_dim > kMaxElems || (long)seq_len * num_heads * head_dim > kMaxElems)
        return fail(ATTN_ERR_INVALID_ARG, "attn_prefill: tensor too large");
    const long hd = head_dim;
    return run_fwd(q, k, v, o, dtype, seq_len, kv_len, num_heads, num_kv_heads, head_dim, causal,
                   sliding_window, attn_softcap, scale, num_heads * hd, hd, num_kv_heads * hd, hd,
                   num_heads * hd, hd, stream, "attn_prefill");
}

int attn_prefill_device_kv_len(const void* q, const void* k, const void* v, void* o, int dtype,
                               int seq_len, int max_kv_len, const int32_t* kv_len, int num_heads,
                               int num_kv_heads, int head_dim, int causal, int sliding_window,
                               float attn_softcap, float scale, void* stream) {
    if (dtype != ATTN_F32 && dtype != ATTN_F16)
        return fail(ATTN_ERR_INVALID_ARG, "attn_prefill_device_kv_len: dtype %d is neither ATTN_F32 nor ATTN_F16", dtype);
    TRY(check_ptr(q, "q"));
    TRY(check_ptr(k, "k"));
    TRY(check_ptr(v, "v"));
    TRY(check_ptr(o, "o"));
    if (!kv_len) return fail(ATTN_ERR_INVALID_ARG, "attn_prefill_device_kv_len: kv_len must not be null");
    if (!aligned(kv_len, 4)) return fail(ATTN_ERR_INVALID_ARG, "attn_prefill_device_kv_len: kv_len must be 4-byte aligned");
    if (max_kv_len < 1)
        return fail(ATTN_ERR_INVALID_ARG, "attn_prefill_device_kv_len: invalid max_kv_len %d (must be >= 1)", max_kv_len);
    if (seq_len < 1 || seq_len > max_kv_len)
        return fail(ATTN_ERR_INVALID_ARG, "attn_prefill_device_kv_len: seq_len %d must be in [1, max_kv_len = %d]",
                    seq_len, max_kv_len);
    if (causal != 0 && causal != 1)
        return fail(ATTN_ERR_INVALID_ARG, "attn_prefill_device_kv_len: causal must be 0 or 1");
    TRY(check_heads(num_heads, num_kv_heads, head_dim));
    TRY(check_scalars(sliding_window, attn_softcap, scale));
    if ((long)max_kv_len * num_kv_heads * head_dim > kMaxElems || (long)seq_len * num_heads * head_dim > kMaxElems)
        return fail(ATTN_ERR_INVALID_ARG, "attn_prefill_device_kv_len: tensor too large");
    const long hd = head_dim;
    return run_fwd(q, k, v, o, dtype, seq_len, max_kv_len, num_heads, num_kv_heads, head_dim, causal,
                   sliding_window, attn_softcap, scale, num_heads * hd, hd, num_kv_heads * hd, hd,
                   num_heads * hd, hd, stream, "attn_prefill_device_kv_len", kv_len);
}

int attn_vision(const void* q, const void* k, const void* v, void* o, int num_patches, int num_heads,
                int head_dim, float scale, void* stream) {
    TRY(check_ptr(q, "q"));
    TRY(check_ptr(k, "k"));
    TRY(check_ptr(v, "v"));
    TRY(check_ptr(o, "o"));
    if (num_patches < 1) return fail(ATTN_ERR_INVALID_ARG, "attn_vision: num_patches %d must be >= 1", num_patches);
    TRY(check_heads(num_heads, num_heads, head_dim));
    TRY(check_scalars(0, 0.f, scale));
    if ((long)num_patches * num_heads * head_dim > kMaxElems)
        return fail(ATTN_ERR_INVALID_ARG, "attn_vision: tensor too large");
    const long hd = head_dim, ph = (long)num_patches * head_dim;
    return run_fwd(q, k, v, o, ATTN_F16, num_patches, num_patches, num_heads, num_heads, head_dim, 0, 0,
                   0.f, scale, hd, ph, hd, ph, hd, ph, stream, "attn_vision");
}

size_t attn_decode_workspace_bytes(int batch, int num_heads, int num_kv_heads, int head_dim,
                                   int max_kv_len) {
    if (batch < 1 || num_heads < 1 || num_kv_heads < 1 || num_heads % num_kv_heads != 0 ||
        max_kv_len < 1 || (head_dim != 64 && head_dim != 128 && head_dim != 256))
        return 0;
    if ((long)batch * num_heads * head_dim > kMaxElems || (long)max_kv_len * num_kv_heads * head_dim > kMaxElems)
        return 0;
    return workspace_bytes_for(batch, num_heads, num_kv_heads, head_dim, max_kv_len);
}

int attn_set_decode_split(int tokens_per_split) {
    if (tokens_per_split < 0 || tokens_per_split % 16 != 0 || tokens_per_split > (1 << 24))
        return fail(ATTN_ERR_INVALID_ARG,
                    "attn_set_decode_split: %d is not 0 or a positive multiple of 16", tokens_per_split);
    g_split_override = tokens_per_split;
    return ok();
}

int attn_decode(const float* q, const void* k, const void* v, float* o, int num_heads, int num_kv_heads,
                int head_dim, int kv_len, int sliding_window, float attn_softcap, float scale,
                void* workspace, size_t workspace_bytes, void* stream) {
    TRY(check_ptr(q, "q"));
    TRY(check_ptr(k, "k"));
    TRY(check_ptr(v, "v"));
    TRY(check_ptr(o, "o"));
    TRY(check_heads(num_heads, num_kv_heads, head_dim));
    if (kv_len < 1) return fail(ATTN_ERR_INVALID_ARG, "attn_decode: invalid kv_len %d (must be >= 1)", kv_len);
    TRY(check_scalars(sliding_window, attn_softcap, scale));
    if ((long)kv_len * num_kv_heads * head_dim > kMaxElems)
        return fail(ATTN_ERR_INVALID_ARG, "attn_decode: tensor too large");
    TRY(check_query_rows(1, num_heads, head_dim, "attn_decode"));
    const int eff = (sliding_window > 0 && sliding_window < kv_len) ? sliding_window : kv_len;
    return run_decode_contiguous(q, k, v, o, num_heads, num_kv_heads, head_dim, kv_len, 0, eff,
                                 sliding_window, attn_softcap, scale, workspace, workspace_bytes,
                                 stream, "attn_decode");
}

int attn_decode_noalloc(const float* q, const void* k, const void* v, float* o, int num_heads,
                        int num_kv_heads, int head_dim, int kv_len, int sliding_window, float attn_softcap,
                        float scale, void* stream) {
    const char* what = "attn_decode_noalloc";
    TRY(check_ptr(q, "q"));
    TRY(check_ptr(k, "k"));
    TRY(check_ptr(v, "v"));
    TRY(check_ptr(o, "o"));
    TRY(check_heads(num_heads, num_kv_heads, head_dim));
    if (kv_len < 1) return fail(ATTN_ERR_INVALID_ARG, "%s: invalid kv_len %d (must be >= 1)", what, kv_len);
    TRY(check_scalars(sliding_window, attn_softcap, scale));
    if ((long)kv_len * num_kv_heads * head_dim > kMaxElems) return fail(ATTN_ERR_INVALID_ARG, "%s: tensor too large", what);
    TRY(check_query_rows(1, num_heads, head_dim, what));
    const int eff = (sliding_window > 0 && sliding_window < kv_len) ? sliding_window : kv_len;
    // the scratch needed by this call's plan (host arithmetic only, before any HIP call)
    const DecodePlan plan = plan_decode(1, num_heads, num_kv_heads, head_dim, eff, false);
    const size_t need = workspace_layout(1, num_heads, num_kv_heads, head_dim, plan).total;
    if (need > ta03::decode_scratch_bytes())
        return fail(ATTN_ERR_UNSUPPORTED,
                    "%s: this shape needs %zu bytes of split partials, more than the %zu bytes of the "
                    "library's scratch; use attn_decode with a workspace",
                    what, need, ta03::decode_scratch_bytes());
    void* ws = nullptr;
    const hipError_t e = ta03::decode_scratch(&ws, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(ATTN_ERR_LAUNCH, "%s: scratch lookup failed: %s", what, hipGetErrorString(e));
    return run_decode_contiguous(q, k, v, o, num_heads, num_kv_heads, head_dim, kv_len, 0, eff, sliding_window,
                                 attn_softcap, scale, ws, ta03::decode_scratch_bytes(), stream, what, true);
}

int attn_decode_ring(const float* q, const void* k, const void* v, float* o, int num_heads,
                     int num_kv_heads, int head_dim, int ring_len, int total_len, int sliding_window,
                     float attn_softcap, float scale, void* workspace, size_t workspace_bytes,
                     void* stream) {
    TRY(check_ptr(q, "q"));
    TRY(check_ptr(k, "k"));
    TRY(check_ptr(v, "v"));
    TRY(check_ptr(o, "o"));
    TRY(check_heads(num_heads, num_kv_heads, head_dim));
    if (ring_len < 1) return fail(ATTN_ERR_INVALID_ARG, "attn_decode_ring: invalid ring_len %d (must be >= 1)", ring_len);
    if (total_len < 1)
        return fail(ATTN_ERR_INVALID_ARG, "attn_decode_ring: invalid total_len %d (must be >= 1)", total_len);
    TRY(check_scalars(sliding_window, attn_softcap, scale));
    if (sliding_window > ring_len)
        return fail(ATTN_ERR_INVALID_ARG,
                    "attn_decode_ring: sliding_window %d exceeds ring_len %d (the ring holds the newest ring_len tokens)",
                    sliding_window, ring_len);
    if ((long)ring_len * num_kv_heads * head_dim > kMaxElems)
        return fail(ATTN_ERR_INVALID_ARG, "attn_decode_ring: tensor too large");
    TRY(check_query_rows(1, num_heads, head_dim, "attn_decode_ring"));
    // visible keys: the newest E = (W > 0 ? W : ring_len) tokens
    const int span = sliding_window > 0 ? sliding_window : ring_len;
    const int eff = total_len < span ? total_len : span;
    return run_decode_contiguous(q, k, v, o, num_heads, num_kv_heads, head_dim, total_len, ring_len,
                                 eff, span, attn_softcap, scale, workspace, workspace_bytes, stream,
                                 "attn_decode_ring");
}

int attn_decode_paged_q8(const float* q, const int8_t* k_pages, const int8_t* v_pages, const float* k_scales,
                         const float* v_scales, const int32_t* page_table, const int32_t* kv_lens, float* o,
                         int batch, int num_heads, int num_kv_heads, int head_dim, int page_size,
                         int num_pages, int max_pages_per_seq, int sliding_window, float attn_softcap,
                         float scale, void* workspace, size_t workspace_bytes, void* stream) {
    TRY(check_ptr(q, "q"));
    TRY(check_ptr(k_pages, "k_pages"));
    TRY(check_ptr(v_pages, "v_pages"));
    TRY(check_ptr(k_scales, "k_scales"));
    TRY(check_ptr(v_scales, "v_scales"));
    TRY(check_ptr(page_table, "page_table"));
    TRY(check_ptr(kv_lens, "kv_lens"));
    TRY(check_ptr(o, "o"));
    if (batch < 1) return fail(ATTN_ERR_INVALID_ARG, "attn_decode_paged_q8: batch %d must be >= 1", batch);
    TRY(check_heads(num_heads, num_kv_heads, head_dim));
    if (page_size != 16)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_decode_paged_q8: page_size %d is not built; requires page_size 16",
                    page_size);
    if (num_pages < 1 || max_pages_per_seq < 1)
        return fail(ATTN_ERR_INVALID_ARG, "attn_decode_paged_q8: num_pages and max_pages_per_seq must be >= 1");
    TRY(check_scalars(sliding_window, attn_softcap, scale));
    if ((long)num_pages * page_size * num_kv_heads * head_dim > kMaxElems)
        return fail(ATTN_ERR_INVALID_ARG, "attn_decode_paged_q8: cache too large");
    TRY(check_query_rows(batch, num_heads, head_dim, "attn_decode_paged_q8"));
    if ((long)max_pages_per_seq * page_size >
        (long)ta03::decode_max_splits() * ta03::decode_max_split_tokens_paged())
        return fail(ATTN_ERR_UNSUPPORTED,
                    "attn_decode_paged_q8: requires max_pages_per_seq * page_size <= %d",
                    ta03::decode_max_splits() * ta03::decode_max_split_tokens_paged());
    const int max_len = max_pages_per_seq * page_size;
    const int eff = (sliding_window > 0 && sliding_window < max_len) ? sliding_window : max_len;
    const DecodePlan plan = plan_decode(batch, num_heads, num_kv_heads, head_dim, eff, true);
    const WorkspaceLayout wl = workspace_layout(batch, num_heads, num_kv_heads, head_dim, plan);
    if (!workspace) return fail(ATTN_ERR_WORKSPACE, "attn_decode_paged_q8: workspace must not be null");
    if (!aligned(workspace, 256))
        return fail(ATTN_ERR_WORKSPACE, "attn_decode_paged_q8: workspace must be 256-byte aligned");
    if (workspace_bytes < wl.total)
        return fail(ATTN_ERR_WORKSPACE, "attn_decode_paged_q8: workspace of %zu bytes is smaller than the %zu required",
                    workspace_bytes, wl.total);
    if ((long)num_kv_heads * plan.nch > 65535)
        return fail(ATTN_ERR_INVALID_ARG, "attn_decode_paged_q8: grid too large");
    {
        const long per_seq = (eff + ta03::decode_max_split_tokens_paged() - 1) / ta03::decode_max_split_tokens_paged();
        if ((long)plan.n_wg < (long)batch * per_seq)
            return fail(ATTN_ERR_UNSUPPORTED,
                        "attn_decode_paged_q8: batch * ceil(max length / %d) must be <= 65535",
                        ta03::decode_max_split_tokens_paged());
    }
    ta03::DecodeParams d{};
    d.q = q; d.k = k_pages; d.v = v_pages;
    d.k_scales = k_scales; d.v_scales = v_scales;
    d.page_table = page_table; d.kv_lens = kv_lens; d.o = o;
    char* ws = reinterpret_cast<char*>(workspace);
    d.part_o = reinterpret_cast<float*>(ws + wl.o_off);
    d.part_m = reinterpret_cast<float*>(ws + wl.m_off);
    d.part_l = reinterpret_cast<float*>(ws + wl.l_off);
    d.tickets = reinterpret_cast<uint32_t*>(ws + wl.t_off);
    d.H = num_heads; d.Hkv = num_kv_heads; d.kv_len = 0;
    d.group = num_heads / num_kv_heads; d.nch = plan.nch;
    d.nch_inv = ((1ull << 32) + plan.nch - 1) / plan.nch;
    d.num_pages = num_pages; d.max_pages = max_pages_per_seq;
    fill_scalars(d, sliding_window, attn_softcap, scale);
    d.split_tokens = plan.split_tokens;
    d.n_split_max = plan.n_split;
    d.batch = batch;
    d.n_wg = plan.n_wg;
    return launch_status(ta03::launch_decode(d, head_dim, plan.gc, true, batch,
                                             reinterpret_cast<hipStream_t>(stream)),
                         "attn_decode_paged_q8");
}

}  // extern "C"

namespace {

// Tiered decode of one sequence (shared by the three tiered entry points): an f16 ring hot
// tier and a cold tier that is int8 (per-row scales) or f16, paged (16-token pages through
// cold_page_table) or contiguous per KV head (cold_stride rows).
struct ColdTier {
    const void* k;
    const void* v;
    const float* ks;              // int8 only
    const float* vs;
    const int32_t* page_table;    // paged only
    bool int8, paged;
    int page_size, num_pages, max_pages;   // paged
    int stride;                   // contiguous: rows per KV head
};

int run_tiered(const char* what, const float* q, const void* hot_k, const void* hot_v, const ColdTier& ct,
               float* o, int num_heads, int num_kv_heads, int head_dim, int cold_len, int hot_len, int hot_window,
               int hot_start, int sliding_window, float attn_softcap, float scale, void* workspace,
               size_t workspace_bytes, void* stream) {
    TRY(check_ptr(q, "q"));
    TRY(check_ptr(o, "o"));
    TRY(check_heads(num_heads, num_kv_heads, head_dim));
    TRY(check_scalars(sliding_window, attn_softcap, scale));
    if (cold_len < 0 || hot_len < 0)
        return fail(ATTN_ERR_INVALID_ARG, "%s: cold_len (%d) and hot_len (%d) must be >= 0", what, cold_len, hot_len);
    if ((long)cold_len + hot_len < 1 || (long)cold_len + hot_len > 0x7fffffffL - 16)
        return fail(ATTN_ERR_INVALID_ARG, "%s: cold_len + hot_len must be in [1, 2^31 - 17]", what);
    TRY(check_query_rows(1, num_heads, head_dim, what));
    if (hot_len > 0) {
        TRY(check_ptr(hot_k, "hot_k"));
        TRY(check_ptr(hot_v, "hot_v"));
        if (hot_window < hot_len)
            return fail(ATTN_ERR_INVALID_ARG, "%s: hot_len %d exceeds hot_window %d", what, hot_len, hot_window);
        if (hot_start < 0 || hot_start >= hot_window)
            return fail(ATTN_ERR_INVALID_ARG, "%s: hot_start %d must be in [0, hot_window %d)", what, hot_start,
                        hot_window);
        if ((long)hot_window * num_kv_heads * head_dim > kMaxElems)
            return fail(ATTN_ERR_INVALID_ARG, "%s: hot tier too large", what);
    }
    if (cold_len > 0) {
        TRY(check_ptr(ct.k, ct.paged ? "cold_k_pages" : "cold_k"));
        TRY(check_ptr(ct.v, ct.paged ? "cold_v_pages" : "cold_v"));
        if (ct.int8) {
            TRY(check_ptr(ct.ks, "cold_k_scales"));
            TRY(check_ptr(ct.vs, "cold_v_scales"));
        }
        if (ct.paged) {
            TRY(check_ptr(ct.page_table, "cold_page_table"));
            if (ct.page_size != 16)
                return fail(ATTN_ERR_UNSUPPORTED, "%s: page_size %d is not built; requires page_size 16", what,
                            ct.page_size);
            if (ct.num_pages < 1 || ct.max_pages < 1)
                return fail(ATTN_ERR_INVALID_ARG, "%s: num_pages and max_pages must be >= 1", what);
            if ((long)ct.max_pages * ct.page_size < cold_len)
                return fail(ATTN_ERR_INVALID_ARG, "%s: cold_len %d exceeds max_pages * page_size = %ld", what, cold_len,
                            (long)ct.max_pages * ct.page_size);
            if ((long)ct.num_pages * ct.page_size * num_kv_heads * head_dim > kMaxElems)
                return fail(ATTN_ERR_INVALID_ARG, "%s: cold tier too large", what);
        } else {
            if (ct.stride < cold_len)
                return fail(ATTN_ERR_INVALID_ARG, "%s: cold_capacity %d is smaller than cold_len %d", what, ct.stride,
                            cold_len);
            if ((long)ct.stride * num_kv_heads * head_dim > kMaxElems)
                return fail(ATTN_ERR_INVALID_ARG, "%s: cold tier too large", what);
        }
    }
    const int total = cold_len + hot_len;
    const int k_lo = (sliding_window > 0 && total > sliding_window) ? total - sliding_window : 0;
    const int cold_vis = cold_len > k_lo ? cold_len - k_lo : 0;
    const int hot_vis = total - (k_lo > cold_len ? k_lo : cold_len);
    // One split size per tier: about one round of resident workgroups (the kernel's LDS is
    // sized for the larger body), in whole rounds of 16-token blocks per wave, at most the
    // paged page-slice limit; the thread's split override wins.  The split count must fit
    // the workspace row that attn_decode_workspace_bytes(1, ..., cold_len + hot_len) sized.
    DecodePlan plan = plan_decode(1, num_heads, num_kv_heads, head_dim, cold_vis + hot_vis, false);
    const int stride = workspace_row_splits(1, num_heads, num_kv_heads, head_dim, total);
    const int max_split = ta03::decode_max_split_tokens_paged();
    // Split lengths in tokens, cold (tc) and hot (th): equal bytes per split (a cold token
    // carries 2D + 8 bytes in int8 with its scales, 4D in f16; a hot one 4D).
    const long cold_tok_bytes = ct.int8 ? 2L * head_dim + 8 : 4L * head_dim;
    int tc = g_split_override, th = g_split_override;
    if (tc <= 0) {
        int per_cu = ta03::decode_workgroups_per_cu(head_dim, false);
        if (ct.int8) {
            const int per_cu_paged = ta03::decode_workgroups_per_cu(head_dim, true);
            if (per_cu_paged < per_cu) per_cu = per_cu_paged;
        }
        const long chunks = (long)num_kv_heads * plan.nch;
        const long n_target = (256L * per_cu + chunks - 1) / chunks;
        const int unit = ta03::decode_waves(head_dim, true) * ta03::decode_tokens_per_block();
        const long cold_b = (long)cold_vis * cold_tok_bytes, hot_b = (long)hot_vis * 4 * head_dim;
        const long per_b = (cold_b + hot_b + n_target - 1) / n_target;
        auto whole_rounds = [&](long t) { return (int)((((t < 1 ? 1 : t) + unit - 1) / unit) * unit); };
        tc = whole_rounds(per_b / cold_tok_bytes);
        th = whole_rounds(per_b / (4 * head_dim));
    }
    if (tc > max_split) tc = max_split;
    if (th > max_split) th = max_split;
    auto splits = [&]() { return (cold_vis + tc - 1) / tc + (hot_vis + th - 1) / th; };
    while (splits() > stride && (tc < max_split || th < max_split)) {
        if (tc < max_split) tc += 16;
        if (th < max_split) th += 16;
    }
    if (splits() > stride)
        return fail(ATTN_ERR_UNSUPPORTED, "%s: %d splits needed but the workspace row holds %d", what, splits(),
                    stride);
    plan.n_split = stride;
    const WorkspaceLayout wl = workspace_layout(1, num_heads, num_kv_heads, head_dim, plan);
    if (!workspace) return fail(ATTN_ERR_WORKSPACE, "%s: workspace must not be null", what);
    if (!aligned(workspace, 256)) return fail(ATTN_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", what);
    if (workspace_bytes < wl.total)
        return fail(ATTN_ERR_WORKSPACE, "%s: workspace of %zu bytes is smaller than the %zu required", what,
                    workspace_bytes, wl.total);
    if ((long)num_kv_heads * plan.nch > 65535) return fail(ATTN_ERR_INVALID_ARG, "%s: grid too large", what);
    ta03::DecodeParams d{};
    d.q = q;
    d.k = ct.k; d.v = ct.v;
    d.k_scales = ct.ks; d.v_scales = ct.vs;
    d.page_table = ct.page_table; d.o = o;
    char* ws = reinterpret_cast<char*>(workspace);
    d.part_o = reinterpret_cast<float*>(ws + wl.o_off);
    d.part_m = reinterpret_cast<float*>(ws + wl.m_off);
    d.part_l = reinterpret_cast<float*>(ws + wl.l_off);
    d.tickets = reinterpret_cast<uint32_t*>(ws + wl.t_off);
    d.H = num_heads; d.Hkv = num_kv_heads;
    d.group = num_heads / num_kv_heads; d.nch = plan.nch;
    d.nch_inv = ((1ull << 32) + plan.nch - 1) / plan.nch;
    d.kv_len = total;
    d.ring = hot_len > 0 ? hot_window : 1;
    d.num_pages = ct.paged ? ct.num_pages : 0;
    d.max_pages = ct.paged ? ct.max_pages : 0;
    fill_scalars(d, sliding_window, attn_softcap, scale);
    d.split_tokens = th;
    d.n_split_max = stride;
    d.batch = 1;
    d.hot_k = hot_k; d.hot_v = hot_v;
    // position p of the hot tier lives at row (hot_start + p - cold_len) mod hot_window
    d.ring_off = hot_len > 0 ? (int)((((long)hot_start - cold_len) % hot_window + hot_window) % hot_window) : 0;
    d.tier_cold_len = cold_len;
    d.tier_cold_splits = (cold_vis + tc - 1) / tc;
    d.tier_k_lo = k_lo;
    d.tier_cold_tokens = tc;
    d.tier_cold_stride = ct.paged ? 0 : ct.stride;
    return launch_status(ta03::launch_decode_tiered(d, head_dim, plan.gc, splits(), ct.int8, ct.paged,
                                                    reinterpret_cast<hipStream_t>(stream)),
                         what);
}

}  // namespace

extern "C" {

int attn_decode_tiered_q8(const float* q, const void* hot_k, const void* hot_v, const int8_t* cold_k_pages,
                          const int8_t* cold_v_pages, const float* cold_k_scales, const float* cold_v_scales,
                          const int32_t* cold_page_table, float* o, int num_heads, int num_kv_heads, int head_dim,
                          int cold_len, int hot_len, int hot_window, int hot_start, int page_size, int num_pages,
                          int max_pages, int sliding_window, float attn_softcap, float scale, void* workspace,
                          size_t workspace_bytes, void* stream) {
    ColdTier ct{cold_k_pages, cold_v_pages, cold_k_scales, cold_v_scales, cold_page_table, true, true,
                page_size, num_pages, max_pages, 0};
    return run_tiered("attn_decode_tiered_q8", q, hot_k, hot_v, ct, o, num_heads, num_kv_heads, head_dim, cold_len,
                      hot_len, hot_window, hot_start, sliding_window, attn_softcap, scale, workspace, workspace_bytes,
                      stream);
}

int attn_decode_tiered_q8_packed(const float* q, const void* hot_k, const void* hot_v, const int8_t* cold_k,
                                 const int8_t* cold_v, const float* cold_k_scales, const float* cold_v_scales,
                                 float* o, int num_heads, int num_kv_heads, int head_dim, int cold_len, int hot_len,
                                 int hot_window, int hot_start, int cold_capacity, int sliding_window,
                                 float attn_softcap, float scale, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    ColdTier ct{cold_k, cold_v, cold_k_scales, cold_v_scales, nullptr, true, false, 0, 0, 0, cold_capacity};
    return run_tiered("attn_decode_tiered_q8_packed", q, hot_k, hot_v, ct, o, num_heads, num_kv_heads, head_dim,
                      cold_len, hot_len, hot_window, hot_start, sliding_window, attn_softcap, scale, workspace,
                      workspace_bytes, stream);
}

int attn_decode_tiered_f16(const float* q, const void* hot_k, const void* hot_v, const void* cold_k,
                           const void* cold_v, const int32_t* cold_page_table, float* o, int num_heads,
                           int num_kv_heads, int head_dim, int cold_len, int hot_len, int hot_window, int hot_start,
                           int cold_layout, int cold_capacity, int page_size, int num_pages, int sliding_window,
                           float attn_softcap, float scale, void* workspace, size_t workspace_bytes, void* stream) {
    const char* what = "attn_decode_tiered_f16";
    if (cold_layout != ATTN_COLD_CONTIGUOUS && cold_layout != ATTN_COLD_PAGED)
        return fail(ATTN_ERR_INVALID_ARG, "%s: cold_layout %d is neither ATTN_COLD_CONTIGUOUS (0) nor ATTN_COLD_PAGED (2)",
                    what, cold_layout);
    const bool paged = cold_layout == ATTN_COLD_PAGED;
    if (paged && cold_capacity % 16 != 0)
        return fail(ATTN_ERR_INVALID_ARG, "%s: a paged cold tier needs cold_capacity (%d) a multiple of 16", what,
                    cold_capacity);
    if (!paged && cold_page_table != nullptr)
        return fail(ATTN_ERR_INVALID_ARG, "%s: a contiguous cold tier takes no page table", what);
    ColdTier ct{cold_k, cold_v, nullptr, nullptr, cold_page_table, false, paged, page_size, num_pages,
                paged ? cold_capacity / 16 : 0, cold_capacity};
    return run_tiered(what, q, hot_k, hot_v, ct, o, num_heads, num_kv_heads, head_dim, cold_len, hot_len, hot_window,
                      hot_start, sliding_window, attn_softcap, scale, workspace, workspace_bytes, stream);
}

int attn_block_local(const float* q_pad, const float* k_padded, const float* v_padded, const float* pos_proj,
                     float* attn_out, int seq, int padded_len, int kv_rows, int num_heads, int head_dim,
                     int chunk_size, int context_size, int max_span, int max_past, int max_future, int pad_left,
                     float logit_cap, void* stream) {
    const char* what = "attn_block_local";
    TRY(check_ptr(q_pad, "q_pad"));
    TRY(check_ptr(k_padded, "k_padded"));
    TRY(check_ptr(v_padded, "v_padded"));
    TRY(check_ptr(pos_proj, "pos_proj"));
    TRY(check_ptr(attn_out, "attn_out"));
    if (num_heads < 1) return fail(ATTN_ERR_INVALID_ARG, "%s: num_heads %d must be >= 1", what, num_heads);
    if (head_dim != ta03::block_local_head_dim())
        return fail(ATTN_ERR_UNSUPPORTED, "%s: requires head_dim == %d (got %d)", what,
                    ta03::block_local_head_dim(), head_dim);
    if (seq < 1 || padded_len < seq)
        return fail(ATTN_ERR_INVALID_ARG, "%s: requires 1 <= seq (%d) <= padded_len (%d)", what, seq, padded_len);
    if (chunk_size < 1 || padded_len % chunk_size != 0)
        return fail(ATTN_ERR_INVALID_ARG, "%s: padded_len %d must be a positive multiple of chunk_size %d", what,
                    padded_len, chunk_size);
    if (max_past < 0 || max_future < 0)
        return fail(ATTN_ERR_INVALID_ARG, "%s: max_past (%d) and max_future (%d) must be >= 0", what, max_past,
                    max_future);
    if ((long)max_span != (long)max_past + max_future + 1)
        return fail(ATTN_ERR_INVALID_ARG, "%s: requires max_span (%d) == max_past + max_future + 1", what, max_span);
    if ((long)context_size != (long)chunk_size + max_past + max_future)
        return fail(ATTN_ERR_INVALID_ARG, "%s: requires context_size (%d) == chunk_size + max_past + max_future",
                    what, context_size);
    if (pad_left != max_past)
        return fail(ATTN_ERR_INVALID_ARG, "%s: requires pad_left (%d) == max_past (%d)", what, pad_left, max_past);
    if ((long)kv_rows < (long)pad_left + seq)
        return fail(ATTN_ERR_INVALID_ARG, "%s: kv_rows %d must be >= pad_left + seq = %ld", what, kv_rows,
                    (long)pad_left + seq);
    if (max_span > ta03::block_local_max_span())
        return fail(ATTN_ERR_UNSUPPORTED, "%s: requires max_span <= %d (max_past + max_future <= %d)", what,
                    ta03::block_local_max_span(), ta03::block_local_max_span() - 1);
    if (!std::isfinite(logit_cap) || logit_cap < 0.f)
        return fail(ATTN_ERR_INVALID_ARG, "%s: logit_cap must be finite and >= 0 (0 = off)", what);
    const long hidden = (long)num_heads * head_dim;
    if ((long)padded_len * hidden > kMaxElems || (long)kv_rows * hidden > kMaxElems || num_heads > 65535)
        return fail(ATTN_ERR_INVALID_ARG, "%s: tensor too large", what);
    ta03::BlockLocalParams p;
    p.q = q_pad; p.k = k_padded; p.v = v_padded; p.pos = pos_proj; p.o = attn_out;
    p.seq = seq; p.padded_len = padded_len; p.H = num_heads;
    p.max_past = max_past; p.max_future = max_future; p.pad_left = pad_left;
    p.cap = logit_cap; p.inv_cap = logit_cap > 0.f ? 1.0f / logit_cap : 0.f;
    return launch_status(ta03::launch_block_local(p, reinterpret_cast<hipStream_t>(stream)), what);
}

const char* attn_last_error(void) { return g_err; }

}  // extern "C"
