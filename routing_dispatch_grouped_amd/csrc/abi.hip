// The C ABI of librdg (declared in include/rdg.h): argument checks, then
// enqueue.  Nothing here allocates device memory or waits for the stream,
// except rdg_check_status, which is documented to wait.
#include <string.h>

#include "rdg_internal.h"

using namespace rdg;

namespace {

inline int hip_rc(hipError_t e) { return e == hipSuccess ? RDG_OK : RDG_EHIP; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool layout_ok(const rdg_layout* L) {
    if (L == nullptr) return false;
    if (L->n_local < 1 || L->n_local > 1024 || L->m_cap < 0 || L->n_rows < 0) return false;
    if (L->kind == RDG_CONTIGUOUS) {
        if (L->block_m < 16 || L->block_m % 16 != 0) return false;
    } else if (L->kind == RDG_MASKED) {
        if (L->m_max < 1 || (int64_t)L->m_max * L->n_local != L->m_cap) return false;
    } else {
        return false;
    }
    return L->counts && L->offsets && L->masked_m && L->work;
}

// The row tile of the grouped GEMMs for a layout and the kernel family that
// runs it.  The tile grows with the expected rows per expert: 16 (skinny
// split-K kernels, weights streamed once per tile), 32/64 (128-column
// register-tiled kernels), 128 (the LDS-tiled kernels of ffn_tiled.hip, for
// bf16/fp8 in the shapes tiled_supported accepts).  A dense
// one-expert layout of at most 256 rows (a decode batch through the shared
// expert) is weight-streaming work that a 128-row tile would spread over too
// few workgroups: it takes the skinny kernels with up to four 16-row tiles
// per workgroup.  The tile divides the segment alignment, so that every tile
// lies inside one expert and row / tile indexes a unique signal counter (a
// one-expert layout starts at row 0, so any tile fits it).
struct FfnPlan {
    int bt;  // rows per tile
    int nr;  // > 0: skinny kernels with nr 16-row tiles per workgroup
};

FfnPlan plan_ffn(const rdg_layout* L, int dtype, int H, int I) {
    const int64_t rows = L->n_rows;
    if (L->n_local == 1 && rows <= 256) {
        const int nr = rows <= 16 ? 1 : rows <= 32 ? 2 : 4;
        return FfnPlan{16 * nr, nr};
    }
    const int64_t avg = (rows + L->n_local - 1) / L->n_local;
    int want = avg <= 24 ? 16 : avg <= 48 ? 32 : 64;
    if (avg > 48 && tiled_supported(dtype, H, I)) want = 128;
    const int align = L->n_local == 1 ? 128 : L->kind == RDG_CONTIGUOUS ? L->block_m : L->m_max;
    while (want > 16 && align % want != 0) want /= 2;
    return FfnPlan{want, want == 16 ? 1 : 0};
}

int64_t ffn_tiles_max(const rdg_layout* L, int bt) {
    int64_t rows = L->n_rows;
    if (rows > L->m_cap) rows = L->m_cap;
    return (rows + bt - 1) / bt + L->n_local;
}

uint64_t wall_ticks_per_us() {
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 100;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0) return 100;
    return (uint64_t)khz / 1000 > 0 ? (uint64_t)khz / 1000 : 1;
}

}  // namespace

extern "C" {

int rdg_version(void) { return 100; }

const char* rdg_strerror(int code) {
    switch (code) {
        case RDG_OK: return "ok";
        case RDG_EINVAL: return "invalid argument";
        case RDG_ECAPACITY: return "rows exceed the layout's preallocated capacity";
        case RDG_ETIMEOUT: return "a completion signal did not reach its threshold in time";
        case RDG_EHIP: return "HIP runtime error";
        case RDG_EUNSUPPORTED: return "unsupported size or type combination";
        default: return "unknown status";
    }
}

static int route_impl(const float* logits, const float* bias, int B, int N, int n_group, int topk_group, int K,
                      float scale, int32_t* topk_ids, float* topk_w, rdg_stream_t stream) {
    if (B < 0 || N < 1 || N > 1024 || n_group < 1 || N % n_group != 0) return RDG_EINVAL;
    if (topk_group < 1 || topk_group > n_group || K < 1 || K > 32 || K > topk_group * (N / n_group))
        return RDG_EINVAL;
    if (B > 0 && (!logits || !topk_ids || !topk_w)) return RDG_EINVAL;
    return hip_rc(launch_route(logits, bias, B, N, n_group, topk_group, K, scale, topk_ids, topk_w, stream));
}

int rdg_route(const float* logits, int B, int N, int n_group, int topk_group, int K, float scale,
              int32_t* topk_ids, float* topk_w, rdg_stream_t stream) {
    return route_impl(logits, nullptr, B, N, n_group, topk_group, K, scale, topk_ids, topk_w, stream);
}

int rdg_route_biased(const float* logits, const float* bias, int B, int N, int n_group, int topk_group, int K,
                     float scale, int32_t* topk_ids, float* topk_w, rdg_stream_t stream) {
    if (!bias) return RDG_EINVAL;
    return route_impl(logits, bias, B, N, n_group, topk_group, K, scale, topk_ids, topk_w, stream);
}

int rdg_eplb_remap(const int32_t* ids, const int64_t* token_gidx, int T, int K, const int32_t* log2phy,
                   const int32_t* n_replica, int r_max, int n_logical, int phys_begin, int n_local,
                   int32_t* local_ids, rdg_stream_t stream) {
    if (T < 0 || K < 1 || r_max < 1 || n_logical < 1 || n_local < 1 || phys_begin < 0) return RDG_EINVAL;
    if (T > 0 && (!ids || !token_gidx || !log2phy || !n_replica || !local_ids)) return RDG_EINVAL;
    return hip_rc(launch_remap(ids, token_gidx, T, K, log2phy, n_replica, r_max, n_logical, phys_begin, n_local,
                               local_ids, stream));
}

size_t rdg_dispatch_workspace_bytes(int T, int K, int n_local) {
    if (T < 0 || K < 0 || n_local < 1) return 0;
    return ws_tile_off_bytes(n_local) + ws_chunk_bytes(n_local) + align256(sizeof(int32_t) * (size_t)T * K);
}

// Argument checks shared by both dispatch entry points; the element size on
// success (0 on an invalid argument).
static int dispatch_esz(const void* x, const float* x_scales, int dtype, int T, int H, const int32_t* ids, int K,
                        const rdg_layout* L, void* x_perm, float* x_perm_scales) {
    if (!layout_ok(L) || T < 0 || K < 1 || K > 32 || H < 16 || H % 16 != 0) return 0;
    if ((int64_t)T * K != L->n_rows) return 0;
    if (!L->pos || !L->row_src || !L->status) return 0;
    int esz;
    switch (dtype) {
        case RDG_F32: esz = 4; break;
        case RDG_BF16: esz = 2; break;
        case RDG_FP8_E4M3:
        case RDG_FP8_E4M3_UE8M0:
            esz = 1;
            if (H % 128 != 0) return 0;
            if (T > 0 && x_perm && (!x_scales || !x_perm_scales)) return 0;
            break;
        default: return 0;
    }
    // x_perm NULL: the layout only (x, x_scales unused; a gathering GEMM reads the tokens)
    if (!x_perm && x_perm_scales) return 0;
    if (T > 0 && !ids) return 0;
    if (T > 0 && x_perm && (!x || !aligned16(x) || !aligned16(x_perm))) return 0;
    return esz;
}

size_t rdg_layout_tables_bytes(int n_local) {
    if (n_local < 1) return 0;
    return ws_tile_off_bytes(n_local);
}

int rdg_dispatch_noalloc(const void* x, const float* x_scales, int dtype, int T, int H, const int32_t* ids, int K,
                         const rdg_layout* L, void* x_perm, float* x_perm_scales, rdg_stream_t stream) {
    const int esz = dispatch_esz(x, x_scales, dtype, T, H, ids, K, L, x_perm, x_perm_scales);
    if (esz == 0) return RDG_EINVAL;
    if ((int64_t)T * K > kNoallocMaxEntries) return RDG_EUNSUPPORTED;
    return hip_rc(launch_dispatch_noalloc(x, esz == 1 ? x_scales : nullptr, H * esz, T, H, ids, K, *L, x_perm,
                                          x_perm_scales, stream));
}

int rdg_dispatch(const void* x, const float* x_scales, int dtype, int T, int H, const int32_t* ids, int K,
                 const rdg_layout* L, void* x_perm, float* x_perm_scales, rdg_stream_t stream) {
    const int esz = dispatch_esz(x, x_scales, dtype, T, H, ids, K, L, x_perm, x_perm_scales);
    if (esz == 0) return RDG_EINVAL;
    return hip_rc(launch_dispatch(x, esz == 1 ? x_scales : nullptr, H * esz, T, H, ids, K, *L, x_perm,
                                  x_perm_scales, stream));
}

int rdg_layout_dense(int T, const rdg_layout* L, rdg_stream_t stream) {
    if (!layout_ok(L) || T < 0 || L->kind != RDG_CONTIGUOUS || L->n_local != 1 || L->m_cap < T || L->n_rows != T)
        return RDG_EINVAL;
    return hip_rc(launch_layout_dense(T, *L, stream));
}

int rdg_signal_rows(const rdg_layout* L, int dtype, int H, int I) {
    if (!layout_ok(L) || H < 128 || H % 128 != 0 || I < 128 || I % 128 != 0) return RDG_EINVAL;
    return plan_ffn(L, dtype, H, I).bt;
}

int rdg_signal_threshold(int H, int dtype) {
    (void)dtype;
    if (H < 128 || H % 128 != 0) return RDG_EINVAL;
    return H;  // each down-GEMM workgroup adds the number of output columns it stored
}

// gather_k > 0: x holds the dispatched tokens [n_rows / gather_k, H] and
// layout row r reads token row_src[r] / gather_k (the layout must come from
// rdg_dispatch, whose row_src it is); 0: x holds the layout rows.
static int grouped_ffn_impl(const rdg_layout* L, int dtype, int H, int I, const void* x_perm,
                            const float* x_perm_scales, int gather_k, const void* W1, const void* W3, const void* W2,
                            const float* W1_s, const float* W3_s, const float* W2_s, void* h_ws, float* h_scales_ws,
                            void* y, int32_t* signals, int stages, rdg_stream_t stream) {
    if (!layout_ok(L) || H < 128 || H % 128 != 0 || I < 128 || I % 128 != 0) return RDG_EINVAL;
    if (gather_k < 0 || gather_k > 32 || (gather_k > 0 && (!L->row_src || L->n_rows % gather_k != 0)))
        return RDG_EINVAL;
    if (dtype != RDG_F32 && dtype != RDG_BF16 && dtype != RDG_FP8_E4M3 && dtype != RDG_FP8_E4M3_UE8M0)
        return RDG_EINVAL;
    if (L->n_rows == 0) return RDG_OK;  // nothing dispatched: no rows, nothing to launch
    const bool pow2 = dtype == RDG_FP8_E4M3_UE8M0;
    if (pow2) dtype = RDG_FP8_E4M3;
    const bool fp8 = dtype == RDG_FP8_E4M3;
    if (!h_ws || !aligned16(h_ws) || (fp8 && !h_scales_ws)) return RDG_EINVAL;
    if (stages & 1) {
        if (!x_perm || !W1 || !W3 || !aligned16(x_perm) || !aligned16(W1) || !aligned16(W3)) return RDG_EINVAL;
        if (fp8 && (!x_perm_scales || !W1_s || !W3_s)) return RDG_EINVAL;
    }
    if (stages & 2) {
        if (!W2 || !y || !aligned16(W2) || !aligned16(y) || (fp8 && !W2_s)) return RDG_EINVAL;
    }
    const FfnPlan plan = plan_ffn(L, dtype, H, I);
    const int bt = plan.bt;
    // the skinny kernels run tile-major too (row tiles on grid y); they are
    // chosen for at most 24 rows per expert, so this bound is never near
    if (plan.nr > 0 && ffn_tiles_max(L, bt) > 65535) return RDG_EUNSUPPORTED;
    if (signals) {
        const int align = L->n_local == 1 ? 128 : L->kind == RDG_CONTIGUOUS ? L->block_m : L->m_max;
        if (align % bt != 0) return RDG_EUNSUPPORTED;
        if (ffn_tiles_max(L, bt) > 65535) return RDG_EUNSUPPORTED;  // row tiles on grid y
    }
    FfnCall c{};
    c.offsets = L->offsets;
    c.masked_m = L->masked_m;
    c.tile_off = static_cast<const int32_t*>(L->work) + bt_index(bt) * (L->n_local + 1);
    c.n_local = L->n_local;
    c.n_tiles_max = (int)ffn_tiles_max(L, bt);
    c.bt = bt;
    c.skinny_nr = plan.nr;
    c.dtype = dtype;
    c.H = H;
    c.I = I;
    c.x = x_perm;
    c.x_s = x_perm_scales;
    c.gather = gather_k > 0 ? L->row_src : nullptr;
    c.gather_k = gather_k;
    c.W1 = W1;
    c.W3 = W3;
    c.W2 = W2;
    c.W1_s = W1_s;
    c.W3_s = W3_s;
    c.W2_s = W2_s;
    c.h = h_ws;
    c.h_s = h_scales_ws;
    c.y = y;
    c.signals = signals;
    c.stages = stages;
    c.pow2 = pow2;
    return hip_rc(launch_ffn(c, stream));
}

int rdg_grouped_ffn(const rdg_layout* L, int dtype, int H, int I, const void* x_perm, const float* x_perm_scales,
                    const void* W1, const void* W3, const void* W2, const float* W1_s, const float* W3_s,
                    const float* W2_s, void* h_ws, float* h_scales_ws, void* y, int32_t* signals,
                    rdg_stream_t stream) {
    return grouped_ffn_impl(L, dtype, H, I, x_perm, x_perm_scales, 0, W1, W3, W2, W1_s, W3_s, W2_s, h_ws,
                            h_scales_ws, y, signals, 3, stream);
}

int rdg_grouped_ffn_gather(const rdg_layout* L, int dtype, int H, int I, const void* x, const float* x_scales, int K,
                           const void* W1, const void* W3, const void* W2, const float* W1_s, const float* W3_s,
                           const float* W2_s, void* h_ws, float* h_scales_ws, void* y, int32_t* signals,
                           rdg_stream_t stream) {
    if (K < 1) return RDG_EINVAL;
    return grouped_ffn_impl(L, dtype, H, I, x, x_scales, K, W1, W3, W2, W1_s, W3_s, W2_s, h_ws, h_scales_ws, y,
                            signals, 3, stream);
}

int rdg_grouped_gate_up_gather(const rdg_layout* L, int dtype, int H, int I, const void* x, const float* x_scales,
                               int K, const void* W1, const void* W3, const float* W1_s, const float* W3_s,
                               void* h_ws, float* h_scales_ws, rdg_stream_t stream) {
    if (K < 1) return RDG_EINVAL;
    return grouped_ffn_impl(L, dtype, H, I, x, x_scales, K, W1, W3, nullptr, W1_s, W3_s, nullptr, h_ws, h_scales_ws,
                            nullptr, nullptr, 1, stream);
}

int rdg_grouped_gate_up(const rdg_layout* L, int dtype, int H, int I, const void* x_perm, const float* x_perm_scales,
                        const void* W1, const void* W3, const float* W1_s, const float* W3_s, void* h_ws,
                        float* h_scales_ws, rdg_stream_t stream) {
    return grouped_ffn_impl(L, dtype, H, I, x_perm, x_perm_scales, 0, W1, W3, nullptr, W1_s, W3_s, nullptr, h_ws,
                            h_scales_ws, nullptr, nullptr, 1, stream);
}

int rdg_grouped_down(const rdg_layout* L, int dtype, int H, int I, const void* h_ws, const float* h_scales_ws,
                     const void* W2, const float* W2_s, void* y, int32_t* signals, rdg_stream_t stream) {
    return grouped_ffn_impl(L, dtype, H, I, nullptr, nullptr, 0, nullptr, nullptr, W2, nullptr, nullptr, W2_s,
                            const_cast<void*>(h_ws), const_cast<float*>(h_scales_ws), y, signals, 2, stream);
}

int rdg_combine(const void* y, int y_dtype, const rdg_layout* L, const float* topk_w, int T, int K, int H,
                const void* shared_out, void* out, int out_dtype, int32_t* signals, int signal_rows,
                int threshold, int64_t timeout_us, int max_blocks, rdg_stream_t stream) {
    if (!layout_ok(L) || !L->pos || T < 0 || K < 1 || K > 32 || H < 8 || H % 8 != 0) return RDG_EINVAL;
    if ((int64_t)T * K != L->n_rows) return RDG_EINVAL;
    if (!((y_dtype == RDG_BF16 && (out_dtype == RDG_BF16 || out_dtype == RDG_F32)) ||
          (y_dtype == RDG_F32 && out_dtype == RDG_F32)))
        return RDG_EUNSUPPORTED;
    if (T > 0 && (!y || !topk_w || !out || !aligned16(y) || !aligned16(out))) return RDG_EINVAL;
    if (shared_out && !aligned16(shared_out)) return RDG_EINVAL;
    if (max_blocks < 0) return RDG_EINVAL;
    int rows_per_sig = 1;
    uint64_t ticks = 0;
    if (signals) {
        if (threshold < 1 || timeout_us < 0 || !L->status || !L->row_src) return RDG_EINVAL;
        if (signal_rows != 16 && signal_rows != 32 && signal_rows != 64 && signal_rows != 128) return RDG_EINVAL;
        if (L->m_cap + ((int64_t)T + 63) / 64 >= (1 << 30)) return RDG_EUNSUPPORTED;  // unit counter range
        rows_per_sig = signal_rows;
        ticks = (uint64_t)timeout_us * wall_ticks_per_us();
    }
    return hip_rc(launch_combine(y, y_dtype, L->pos, L->row_src, L->m_cap, topk_w, T, K, H, shared_out, out,
                                 out_dtype, signals, rows_per_sig, threshold, ticks, max_blocks, L->status, stream));
}

int rdg_combine_finish(const void* y, int y_dtype, const rdg_layout* L, const float* topk_w, int T, int K, int H,
                       const void* shared_out, void* out, int out_dtype, int32_t* signals, int signal_rows,
                       rdg_stream_t stream) {
    if (!layout_ok(L) || !L->pos || T < 0 || K < 1 || K > 32 || H < 8 || H % 8 != 0) return RDG_EINVAL;
    if ((int64_t)T * K != L->n_rows) return RDG_EINVAL;
    if (!((y_dtype == RDG_BF16 && (out_dtype == RDG_BF16 || out_dtype == RDG_F32)) ||
          (y_dtype == RDG_F32 && out_dtype == RDG_F32)))
        return RDG_EUNSUPPORTED;
    if (!signals) return RDG_EINVAL;
    if (signal_rows != 16 && signal_rows != 32 && signal_rows != 64 && signal_rows != 128) return RDG_EINVAL;
    if (L->m_cap + ((int64_t)T + 63) / 64 >= (1 << 30)) return RDG_EUNSUPPORTED;
    if (T > 0 && (!y || !topk_w || !out || !aligned16(y) || !aligned16(out))) return RDG_EINVAL;
    if (shared_out && !aligned16(shared_out)) return RDG_EINVAL;
    return hip_rc(launch_combine_finish(y, y_dtype, L->pos, L->m_cap, topk_w, T, K, H, shared_out, out, out_dtype,
                                        signals, signal_rows, stream));
}

int rdg_quantize_fp8(const void* src, int src_dtype, int rows, int cols, int block_rows, uint8_t* q,
                     float* scales, rdg_stream_t stream) {
    if (rows < 0 || cols < 128 || cols % 128 != 0 || (block_rows != 1 && block_rows != 128)) return RDG_EINVAL;
    if (src_dtype != RDG_F32 && src_dtype != RDG_BF16) return RDG_EINVAL;
    if (rows > 0 && (!src || !q || !scales)) return RDG_EINVAL;
    return hip_rc(launch_quantize(src, src_dtype, rows, cols, block_rows, false, q, scales, stream));
}

int rdg_quantize_fp8_ue8m0(const void* src, int src_dtype, int rows, int cols, int block_rows, uint8_t* q,
                           float* scales, rdg_stream_t stream) {
    if (rows < 0 || cols < 128 || cols % 128 != 0 || (block_rows != 1 && block_rows != 128)) return RDG_EINVAL;
    if (src_dtype != RDG_F32 && src_dtype != RDG_BF16) return RDG_EINVAL;
    if (rows > 0 && (!src || !q || !scales)) return RDG_EINVAL;
    return hip_rc(launch_quantize(src, src_dtype, rows, cols, block_rows, true, q, scales, stream));
}

size_t rdg_packed_weight_bytes(int dtype, int n_mat, int rows, int cols) {
    if (n_mat < 0 || rows < 0 || cols < 0) return 0;
    const size_t esz = dtype == RDG_F32 ? 4 : dtype == RDG_BF16 ? 2
                     : (dtype == RDG_FP8_E4M3 || dtype == RDG_FP8_E4M3_UE8M0) ? 1 : 0;
    return esz * (size_t)n_mat * rows * cols;
}

int rdg_pack_weights(const void* W, int dtype, int n_mat, int rows, int cols, void* W_packed, rdg_stream_t stream) {
    if (dtype == RDG_FP8_E4M3_UE8M0) dtype = RDG_FP8_E4M3;  // the same codes, packed alike
    if (dtype != RDG_F32 && dtype != RDG_BF16 && dtype != RDG_FP8_E4M3) return RDG_EINVAL;
    if (n_mat < 0 || rows < 0 || cols < 0 || rows % 16 != 0 || cols % 128 != 0) return RDG_EINVAL;
    if ((size_t)n_mat * rows * cols > 0 && (!W || !W_packed || !aligned16(W) || !aligned16(W_packed)))
        return RDG_EINVAL;
    if (W == W_packed) return RDG_EINVAL;
    return hip_rc(launch_pack(W, dtype, n_mat, rows, cols, W_packed, stream));
}

int rdg_fill_i32(int32_t* p, int32_t value, int64_t n, rdg_stream_t stream) {
    if (n < 0 || (n > 0 && !p)) return RDG_EINVAL;
    return hip_rc(launch_fill_i32(p, value, n, stream));
}

int rdg_check_status(const int32_t* status, int32_t* host_status, rdg_stream_t stream) {
    if (!status || !host_status) return RDG_EINVAL;
    if (hipMemcpyAsync(host_status, status, 2 * sizeof(int32_t), hipMemcpyDeviceToHost, stream) != hipSuccess)
        return RDG_EHIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return RDG_EHIP;
    return host_status[0];
}

}  // extern "C"
