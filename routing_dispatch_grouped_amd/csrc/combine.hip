// Combine: routing-weighted unpermute-and-sum.
//
// What it computes (DeepEP deep-dive, EP section: expert outputs are
// summed back to their token weighted by the routing weights; section "why
// is combine slower than dispatch": combine is transfer plus a weighted
// reduction; section "limitations": bf16 pre-reduction loses precision and
// is non-deterministic -- so here the sum is fp32, in slot order, rounded
// once; DeepGEMM single-batch-overlap pull request, section 2: the consumer
// polls a per-row-block counter until it reaches its threshold).
//
//   out[t] = shared_out[t] + sum_{k: pos[t,k] >= 0} w[t,k] * y[pos[t,k]]
//
// Design for CDNA4: one wave per (token, 512-feature slice); each lane owns
// 8 consecutive features (a 16-byte bf16 vector), gathers the K expert rows
// for them, accumulates in fp32 and writes once.  Slicing the row keeps a
// 128-token decode batch from occupying only a handful of CUs.  In the
// polling form, tokens are visited in the order their rows become ready (see
// k_combine), and lane 0 waits (acquire, device scope) on the counter of each
// row tile the token reads; a bounded wait turns a tile that never completes
// into a status code instead of a hang.
#include "rdg_internal.h"

namespace rdg {
namespace {

template <int YDT>
__device__ __forceinline__ void load8(const void* y, size_t row, int H, int v, float* out) {
    if (YDT == RDG_BF16) {
        const uint4 q = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(y) + row * H)[v];
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = bf16_to_f32(w[i] & 0xffffu);
            out[2 * i + 1] = bf16_to_f32(w[i] >> 16);
        }
    } else {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(y) + row * H) + 2 * v;
        const float4 a = p[0], b = p[1];
        out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
        out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
    }
}

// load8 for rows published by a concurrently running producer on another
// XCD: device-scope (relaxed atomic) loads, which read past this CU's L1 and
// any stale line of this XCD's L2 -- so the consumer needs no device-scope
// acquire, whose L2 invalidation would hurt the producer's workgroups here.
template <int YDT>
__device__ __forceinline__ void load8_published(const void* y, size_t row, int H, int v, float* out) {
    if (YDT == RDG_BF16) {
        const uint64_t* p = reinterpret_cast<const uint64_t*>(static_cast<const uint16_t*>(y) + row * H) + 2 * v;
        const uint64_t lo = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t hi = __hip_atomic_load(p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t w[4] = {(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = bf16_to_f32(w[i] & 0xffffu);
            out[2 * i + 1] = bf16_to_f32(w[i] >> 16);
        }
    } else {
        const uint64_t* p = reinterpret_cast<const uint64_t*>(static_cast<const float*>(y) + row * H) + 4 * v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint64_t q = __hip_atomic_load(p + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            out[2 * i] = __uint_as_float((uint32_t)q);
            out[2 * i + 1] = __uint_as_float((uint32_t)(q >> 32));
        }
    }
}

template <int ODT>
__device__ __forceinline__ void store8(void* o, size_t row, int H, int v, const float* acc) {
    if (ODT == RDG_BF16) {
        uint4 q;
        q.x = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
        q.y = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
        q.z = f32_to_bf16(acc[4]) | (f32_to_bf16(acc[5]) << 16);
        q.w = f32_to_bf16(acc[6]) | (f32_to_bf16(acc[7]) << 16);
        reinterpret_cast<uint4*>(static_cast<uint16_t*>(o) + row * H)[v] = q;
    } else {
        float4* p = reinterpret_cast<float4*>(static_cast<float*>(o) + row * H) + 2 * v;
        p[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        p[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
}

// Lane 0 waits for a counter; returns false on timeout.
// Lane 0 waits for a counter; returns false on timeout.  The polls are
// relaxed device-scope loads (they read L2, where the producer's release
// lands, without invalidating this CU's L1 on every poll -- which would slow
// the GEMM waves sharing the CU); the caller issues one acquire fence once
// every counter it needs is complete.  Exponential back-off (64 cycles up to
// about 8k) keeps the polling traffic on the counters' few L2 lines low.
__device__ bool wait_counter(const int32_t* c, int threshold, uint64_t timeout_ticks) {
    if (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= threshold) return true;
    const uint64_t t0 = wall_clock64();
    int backoff = 1;
    while (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < threshold) {
        if (wall_clock64() - t0 > timeout_ticks) return false;
        for (int i = 0; i < backoff; ++i) __builtin_amdgcn_s_sleep(1);
        backoff = backoff < 128 ? backoff * 2 : 128;
    }
    return true;
}

__device__ __forceinline__ int wave_max_i32(int v) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) v = max(v, __shfl_xor(v, o));
    return v;
}

// READY (polling form): tokens are visited in the order their rows become
// ready -- token t at its last layout row max_k pos[t,k], walking the layout
// rows in order, which is the order the signalled down GEMM completes its row
// tiles -- and then the tokens with no row on this GPU.  Otherwise tokens are
// visited in index order.
// Token t's slots into this wave's LDS row: positions (-1: no row, or a row
// whose tile never completed) and weights.  Polling form: lane 0 first waits
// for the counter of every row tile the token reads.
__device__ __forceinline__ void token_slots(const int32_t* __restrict__ pos, const float* __restrict__ w, int t,
                                            int K, const int32_t* signals, int rows_per_sig, int threshold,
                                            uint64_t timeout_ticks, int32_t* status, int* pos_l, float* w_l,
                                            int lane, int& known_tile) {
    int p = -1;
    float wt = 0.0f;
    if (lane < K) {
        p = pos[(size_t)t * K + lane];
        wt = w[(size_t)t * K + lane];
    }
    if (signals != nullptr) {
        for (int k = 0; k < K; ++k) {
            const int pk = __shfl(p, k);
            if (pk < 0) continue;
            const int tile = pk / rows_per_sig;
            if (tile == known_tile) continue;  // confirmed complete for an earlier token
            int ok = 1;
            if (lane == 0) {
                ok = wait_counter(signals + tile, threshold, timeout_ticks) ? 1 : 0;
                if (!ok) set_status(status, RDG_ETIMEOUT, tile);
            }
            ok = __shfl(ok, 0);
            if (ok) known_tile = tile;
            else if (lane == k) p = -1;  // skip the incomplete row
        }
        // the rows are then read with device-scope loads (load8_published);
        // this fence only keeps those loads after the polls
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
    // the feature loop may leave lanes idle: it reads the slots from LDS
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane < K) {
        pos_l[lane] = p;
        w_l[lane] = wt;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One 512-feature slice of token t: lane l owns features [8v, 8v+8), v = 64*slice + l.
template <int YDT, int ODT>
__device__ __forceinline__ void combine_slice(const void* __restrict__ y, const void* __restrict__ shared_out,
                                              void* __restrict__ out, int t, int slice, int K, int H,
                                              const int* pos_l, const float* w_l, int lane) {
    const int v = slice * kWave + lane;
    if (v >= H / 8) return;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < K; ++k) {
        const int pk = pos_l[k];
        const float wk = w_l[k];
        if (pk < 0) continue;
        float yv[8];
        load8<YDT>(y, (size_t)pk, H, v, yv);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += wk * yv[i];
    }
    if (shared_out != nullptr) {
        float sv[8];
        load8<ODT>(shared_out, (size_t)t, H, v, sv);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += sv[i];
    }
    store8<ODT>(out, (size_t)t, H, v, acc);
}

// All slices of token t from published rows, G slices at a time with every
// row load of a group issued before any is used (the device-scope loads go
// to memory; one at a time would leave the wave waiting on each).
template <int YDT, int ODT>
__device__ __forceinline__ void combine_token_published(const void* __restrict__ y, const void* __restrict__ shared_out,
                                                        void* __restrict__ out, int t, int K, int H, const int* pos_l,
                                                        const float* w_l, int lane) {
    constexpr int G = 7;
    const int nvec = H / 8;
    for (int v0 = lane; v0 < nvec; v0 += G * kWave) {
        float acc[G][8];
#pragma unroll
        for (int j = 0; j < G; ++j)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[j][i] = 0.0f;
        for (int k = 0; k < K; ++k) {
            const int pk = pos_l[k];
            const float wk = w_l[k];
            if (pk < 0) continue;
            float yv[G][8];
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const int v = v0 + j * kWave;
                if (v < nvec) load8_published<YDT>(y, (size_t)pk, H, v, yv[j]);
            }
#pragma unroll
            for (int j = 0; j < G; ++j)
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[j][i] += wk * yv[j][i];
        }
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const int v = v0 + j * kWave;
            if (v >= nvec) continue;
            if (shared_out != nullptr) {
                float sv[8];
                load8<ODT>(shared_out, (size_t)t, H, v, sv);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[j][i] += sv[i];
            }
            store8<ODT>(out, (size_t)t, H, v, acc[j]);
        }
    }
}

// Plain form: one wave per (token, 512-feature slice) unit, tokens in index
// order.  Polling form (READY): one wave per token, visited in the order its
// rows become ready -- token t at its last layout row max_k pos[t,k], walking
// the layout rows in order, which is the order the signalled down GEMM
// completes its row tiles -- then the tokens with no row on this GPU; the
// wave polls once for the token and then combines all of its slices.
template <int YDT, int ODT, bool READY>
__global__ __launch_bounds__(256) void k_combine(const void* __restrict__ y, const int32_t* __restrict__ pos,
                                                 const int32_t* __restrict__ row_src, int m_cap,
                                                 const float* __restrict__ w, int T, int K, int H,
                                                 const void* __restrict__ shared_out, void* __restrict__ out,
                                                 const int32_t* signals, int rows_per_sig, int threshold,
                                                 uint64_t timeout_ticks, int32_t* status) {
    __shared__ int pos_lds[4][32];
    __shared__ float w_lds[4][32];
    const int wv = threadIdx.x / kWave, lane = lane_id();
    const int n_slices = (H / 8 + kWave - 1) / kWave;
    const int64_t stride = (int64_t)gridDim.x * 4;
    if (!READY) {
        const int64_t n_units = (int64_t)T * n_slices;
        for (int64_t unit = (int64_t)blockIdx.x * 4 + wv; unit < n_units; unit += stride) {
            const int t = (int)(unit / n_slices), slice = (int)(unit % n_slices);
            int none = -1;
            token_slots(pos, w, t, K, nullptr, rows_per_sig, threshold, timeout_ticks, status, pos_lds[wv],
                        w_lds[wv], lane, none);
            combine_slice<YDT, ODT>(y, shared_out, out, t, slice, K, H, pos_lds[wv], w_lds[wv], lane);
        }
        return;
    }
    // units of RC consecutive layout rows (then of RC tokens without a row
    // here): the tokens completed by neighbouring rows mostly share a row
    // tile, so one confirmed poll serves them all
    constexpr int RC = 16;
    const int64_t row_units = ((int64_t)m_cap + RC - 1) / RC;
    const int64_t n_units = row_units + ((int64_t)T + RC - 1) / RC;
    int known_tile = -1;
    for (int64_t u = (int64_t)blockIdx.x * 4 + wv; u < n_units; u += stride) {
        // lane i < RC looks at row u*RC+i (or token (u-row_units)*RC+i): its
        // token, and whether this unit is where that token gets combined
        int tok = -1;
        bool mine = false;
        if (lane < RC) {
            if (u < row_units) {
                const int64_t r = u * RC + lane;
                const int src = r < m_cap ? row_src[r] : -1;
                if (src >= 0) {
                    tok = src / K;
                    int last = -1;
                    for (int k = 0; k < K; ++k) last = max(last, pos[(size_t)tok * K + k]);
                    mine = last == (int)r;  // the token is combined at its last row
                }
            } else {
                const int64_t tt = (u - row_units) * RC + lane;
                if (tt < T) {
                    tok = (int)tt;
                    int last = -1;
                    for (int k = 0; k < K; ++k) last = max(last, pos[(size_t)tok * K + k]);
                    mine = last < 0;  // no row here: combined in this second pass
                }
            }
        }
        uint64_t todo = __ballot(mine);
        while (todo) {
            const int i = __builtin_ctzll(todo);
            todo &= todo - 1;
            const int t = __shfl(tok, i);
            token_slots(pos, w, t, K, signals, rows_per_sig, threshold, timeout_ticks, status, pos_lds[wv],
                        w_lds[wv], lane, known_tile);
            combine_token_published<YDT, ODT>(y, shared_out, out, t, K, H, pos_lds[wv], w_lds[wv], lane);
        }
    }
}

}  // namespace

hipError_t launch_combine(const void* y, int y_dt, const int32_t* pos, const int32_t* row_src, int m_cap,
                          const float* w, int T, int K, int H, const void* shared_out, void* out, int out_dt,
                          const int32_t* signals, int rows_per_sig, int threshold, uint64_t timeout_ticks,
                          int max_blocks, int32_t* status, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const bool ready = signals != nullptr;
    const int64_t units = ready ? ((int64_t)m_cap + 15) / 16 + ((int64_t)T + 15) / 16
                                : (int64_t)T * ((H / 8 + kWave - 1) / kWave);
    int64_t blocks = (units + 3) / 4;
    if (max_blocks > 0 && blocks > max_blocks) blocks = max_blocks;
    if (ready) {
        // Polling workgroups hold their CU resources while they wait.  A
        // producer workgroup of the down GEMM needs most of a CU, so polling
        // workgroups spread over every CU could leave it nowhere to run until
        // the waits time out: at most a quarter of the CUs' worth of them.
        int dev = 0, n_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return hipErrorInvalidDevice;
        const int64_t cap = n_cu / 4 > 0 ? n_cu / 4 : 1;
        if (blocks > cap) blocks = cap;
    }
#define RDG_COMBINE(YD, OD)                                                                                    \
    do {                                                                                                       \
        if (ready)                                                                                             \
            k_combine<YD, OD, true><<<(unsigned)blocks, 256, 0, s>>>(y, pos, row_src, m_cap, w, T, K, H,        \
                                                                   shared_out, out, signals, rows_per_sig,    \
                                                                   threshold, timeout_ticks, status);         \
        else                                                                                                   \
            k_combine<YD, OD, false><<<(unsigned)blocks, 256, 0, s>>>(y, pos, row_src, m_cap, w, T, K, H,       \
                                                                    shared_out, out, nullptr, rows_per_sig,   \
                                                                    threshold, timeout_ticks, status);        \
    } while (0)
    if (y_dt == RDG_BF16 && out_dt == RDG_BF16) RDG_COMBINE(RDG_BF16, RDG_BF16);
    else if (y_dt == RDG_BF16 && out_dt == RDG_F32) RDG_COMBINE(RDG_BF16, RDG_F32);
    else if (y_dt == RDG_F32 && out_dt == RDG_F32) RDG_COMBINE(RDG_F32, RDG_F32);
    else return hipErrorInvalidValue;
#undef RDG_COMBINE
    return hipGetLastError();
}

}  // namespace rdg
