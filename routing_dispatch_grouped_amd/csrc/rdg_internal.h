// Internal declarations of librdg: device helpers shared by the kernels and
// the host-side launchers that the C ABI (abi.hip) calls.  gfx950 only.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "rdg.h"

namespace rdg {

constexpr int kWave = 64;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- formats
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16, round to nearest even (finite inputs; NaN -> canonical NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// OCP e4m3fn code -> fp32 (S.EEEE.MMM, bias 7, E=0 subnormal, no infinity).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
    uint32_t e = (c >> 3) & 15u, m = c & 7u;
    float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
    return (c & 0x80u) ? -v : v;
}

// fp32 in [-448, 448] -> e4m3fn code, round to nearest even.  Normal range:
// keep exponent and the top 3 mantissa bits, round on the 20 dropped bits,
// rebias 127 -> 7 (a carry moves into the exponent).  Below 2^-6 the grid is
// 2^-9, and a*2^9 is exact, so rint() rounds it directly.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
    uint32_t u = __float_as_uint(v);
    uint32_t sign = (u >> 24) & 0x80u;
    uint32_t au = u & 0x7fffffffu;
    uint32_t code;
    if (au < 0x3c800000u) {  // |v| < 2^-6
        code = (uint32_t)__builtin_rintf(__uint_as_float(au) * 512.0f);
    } else {
        uint32_t r = au >> 20;
        uint32_t rem = au & 0xfffffu;
        r += (rem > 0x80000u) || (rem == 0x80000u && (r & 1u));
        code = r - (120u << 3);
    }
    return sign | code;
}

// Scale of an fp8 block whose largest magnitude is amax (1 for an all-zero
// block): amax / 448 in fp32, or with pow2 the smallest power of two 2^k with
// 448 * 2^k >= amax, k kept in [-126, 127] (a normal fp32 and a valid 8-bit
// exponent-only scale).  With amax = (1 + m) 2^e the power-of-two form is
// k = e - 8, or e - 7 when m > 0.75 (448 = 1.75 * 2^8): exact bit logic.
__device__ __forceinline__ float fp8_block_scale(float amax, bool pow2) {
    if (!(amax > 0.0f)) return 1.0f;
    if (!pow2) return amax / 448.0f;
    const uint32_t u = __float_as_uint(amax);
    const int be = (int)(u >> 23);  // biased exponent; 0 for subnormal amax
    int k = be - 127 - 8 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0);
    if (be == 0 || k < -126) k = -126;
    return __uint_as_float((uint32_t)(k + 127) << 23);
}

// 8-bit exponent-only (E8M0) encoding of a power-of-two fp32 scale: its
// biased exponent.
__device__ __forceinline__ int e8m0_of(float pow2_scale) { return (int)(__float_as_uint(pow2_scale) >> 23); }

// ---------------------------------------------------------------- waves
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t lo = __shfl_xor((uint32_t)x, off);
        uint32_t hi = __shfl_xor((uint32_t)(x >> 32), off);
        uint64_t o = ((uint64_t)hi << 32) | lo;
        x = o > x ? o : x;
    }
    return x;
}

__device__ __forceinline__ float wave_max_f32(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// The row of the gate/up GEMM's token operand that holds layout row r: r
// itself when the dispatch permuted the rows (x_perm), or, when the GEMM
// gathers from the unpermuted tokens, the token t of row_src[r] = t*K + k.
// gather is a kernel argument, so the branch is uniform.
__device__ __forceinline__ int token_row(const int32_t* gather, int gather_k, int r) {
    return gather ? gather[r] / gather_k : r;
}

// First error wins: code into st[0] (if still 0), then its detail into st[1].
__device__ __forceinline__ void set_status(int32_t* st, int code, int detail) {
    if (st != nullptr && atomicCAS(st, 0, code) == 0) atomicExch(st + 1, detail);
}

// ---------------------------------------------------------------- workspace
// The layout's work area: per-row-tile prefix tables for the GEMM row tiles
// {16, 32, 64, 128} (kNumBT x (n_local+1) int32), the per-chunk counts of the
// counting sort (kMaxChunks x n_local int32), then one int32 per dispatched
// entry (its rank inside its chunk).
constexpr int kNumBT = 4;
constexpr int kBT[kNumBT] = {16, 32, 64, 128};
constexpr int kMaxChunks = 64;

__host__ __device__ inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }
__host__ __device__ inline size_t ws_tile_off_bytes(int n_local) {
    return align256(sizeof(int32_t) * kNumBT * (size_t)(n_local + 1));
}
__host__ __device__ inline size_t ws_chunk_bytes(int n_local) {
    return align256(sizeof(int32_t) * kMaxChunks * (size_t)n_local);
}
// Entries per counting-sort chunk: at most kMaxChunks chunks, and at least
// four 64-entry pieces per chunk so small dispatches scan few chunks.
__host__ __device__ inline int chunk_size_for(int64_t n_rows) {
    int64_t pieces = (n_rows + (int64_t)kWave * kMaxChunks - 1) / ((int64_t)kWave * kMaxChunks);
    if (pieces < 4) pieces = 4;
    return (int)(pieces * kWave);
}
__host__ __device__ inline int bt_index(int bt) { return bt == 16 ? 0 : bt == 32 ? 1 : bt == 64 ? 2 : 3; }

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.  Arguments are validated by
// the ABI layer before these are called.
hipError_t launch_route(const float* logits, const float* bias, int B, int N, int n_group, int topk_group, int K,
                        float scale, int32_t* ids, float* w, hipStream_t s);
hipError_t launch_remap(const int32_t* ids, const int64_t* gidx, int T, int K, const int32_t* log2phy,
                        const int32_t* n_rep, int r_max, int n_logical, int phys_begin, int n_local,
                        int32_t* out, hipStream_t s);
hipError_t launch_dispatch(const void* x, const float* x_scales, int row_bytes, int T, int H, const int32_t* ids,
                           int K, const rdg_layout& L, void* x_perm, float* x_perm_scales, hipStream_t s);
// The same with the scratch in the library's static device array; L.work
// holds only the row-tile tables.  At most kNoallocMaxEntries entries.
constexpr int64_t kNoallocMaxEntries = 1 << 20;
hipError_t launch_dispatch_noalloc(const void* x, const float* x_scales, int row_bytes, int T, int H,
                                   const int32_t* ids, int K, const rdg_layout& L, void* x_perm, float* x_perm_scales,
                                   hipStream_t s);
hipError_t launch_layout_dense(int T, const rdg_layout& L, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t s);
hipError_t launch_pack(const void* W, int dtype, int n_mat, int rows, int cols, void* P, hipStream_t s);

// Output stores of a signalled down GEMM: device scope, so they are written
// through to memory instead of staying dirty in this XCD's L2, where another
// XCD's consumer could not see them.  (Plain stores with a device-scope
// release before the signal would need a write-back of the whole L2 per
// workgroup: the down GEMM ran 20% slower that way.)
template <bool SIGNAL>
__device__ __forceinline__ void store_out8(void* p, uint64_t v) {
    if constexpr (SIGNAL) __hip_atomic_store(static_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *static_cast<uint64_t*>(p) = v;
}
template <bool SIGNAL>
__device__ __forceinline__ void store_out16(void* p, float4 v) {
    if constexpr (SIGNAL) {
        store_out8<true>(p, (uint64_t)__float_as_uint(v.x) | ((uint64_t)__float_as_uint(v.y) << 32));
        store_out8<true>(static_cast<uint8_t*>(p) + 8,
                         (uint64_t)__float_as_uint(v.z) | ((uint64_t)__float_as_uint(v.w) << 32));
    } else {
        *static_cast<float4*>(p) = v;
    }
}

// End of a signalled down-GEMM workgroup: publish `cols` finished output
// columns of its row tile.  Every wave waits for its own output stores to
// complete -- device-scope stores, so they are then in memory, where other
// XCDs' device-scope loads read -- the waves meet at a barrier, and one
// thread adds the column count to the tile's counter (relaxed, device
// scope).  No fence: a device-scope release would also write back this XCD's
// whole L2, and its acquire half would invalidate it, throwing away the
// weight panels the other workgroups on this XCD are re-reading.
__device__ __forceinline__ void signal_done(int32_t* counter, int cols) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(counter, cols, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Column blocks of a signalled (tile-major) down GEMM grid, padded to a
// multiple of the 8 XCDs so that a column block always runs on the same XCD
// (hardware workgroup b runs on XCD b % 8) and its weights stay in that L2.
inline unsigned round8(int n) { return (unsigned)((n + 7) / 8 * 8); }

struct FfnCall {
    const int32_t* offsets;
    const int32_t* masked_m;
    const int32_t* tile_off;  // prefix table for row tile bt
    int n_local, n_tiles_max, bt;
    int skinny_nr;  // > 0: skinny kernel with bt = 16 * skinny_nr (weight streaming)
    int dtype, H, I;
    const void *x, *W1, *W3, *W2;
    const int32_t* gather;  // NULL: x holds layout rows; else x holds tokens and layout row r reads
    int gather_k;           // token gather[r] / gather_k (gather = the layout's row_src, gather_k = K)
    const float *x_s, *W1_s, *W3_s, *W2_s;
    void* h;
    float* h_s;
    void* y;
    int32_t* signals;
    int stages;  // bit 0: gate/up, bit 1: down
    bool pow2;   // fp8 with power-of-two (E8M0) block scales: h re-quantised the same way, and the
                 // 128-row kernels apply the scales inside the scaled MFMA
};
hipError_t launch_ffn(const FfnCall& c, hipStream_t s);
hipError_t launch_quantize(const void* src, int src_dt, int rows, int cols, int block_rows, bool pow2, uint8_t* q,
                           float* scales, hipStream_t s);
hipError_t launch_ffn_tiled(const FfnCall& c, hipStream_t s);  // bt == 128, bf16 / fp8
bool tiled_supported(int dtype, int H, int I);                 // shapes the bt == 128 kernels take

hipError_t launch_combine(const void* y, int y_dt, const int32_t* pos, const int32_t* row_src, int m_cap,
                          const float* w, int T, int K, int H, const void* shared_out, void* out, int out_dt,
                          int32_t* signals, int rows_per_sig, int threshold, uint64_t timeout_ticks,
                          int max_blocks, int32_t* status, hipStream_t s);
// signals: the row tiles' counters, then the polling form's unit counter and
// the finishing form's first unit
hipError_t launch_combine_finish(const void* y, int y_dt, const int32_t* pos, int m_cap, const float* w, int T, int K,
                                 int H, const void* shared_out, void* out, int out_dt, int32_t* signals,
                                 int rows_per_sig, hipStream_t s);

}  // namespace rdg
