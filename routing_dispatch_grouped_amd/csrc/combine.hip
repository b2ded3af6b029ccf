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
// for them (eight requests in flight, streamed past the caches: each row is
// read once), accumulates in fp32 in slot order and writes once.  Slicing
// the row keeps a 128-token decode batch from occupying only a handful of
// CUs.  (Requesting the rows one slot at a time took 115 us on the 4096-token
// prefill layer against 96 us, and 12.1 against 9.3 us on the decode layer.)
//
// The polling form (k_combine_poll) runs beside the signalled down GEMM on at
// most a quarter of the CUs.  Each wave claims single layout rows in layout
// order from a counter (the row tiles complete in that order) and combines
// every token whose last row it is, after lane 0 has waited for the counter
// of each row tile the token reads; a bounded wait turns a tile that never
// completes into a status code instead of a hang.  The published rows are
// staged in LDS by device-scope direct loads, many in flight per wave, so that
// a wave is not bound by one memory round trip per 512-feature slice.  The
// finishing form, enqueued after the down GEMM on its stream, closes the
// counter and combines every token the polling waves had not claimed with
// the plain form's parallelism (k_combine_close, then k_combine<.., true>):
// a few polling workgroups take the tokens of the tiles that complete early,
// and the rest no longer waits for them.
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

// Lane 0 waits for a counter; returns false on timeout.  The polls are
// relaxed device-scope loads: they read memory, past this CU's L1 and any
// stale line of this XCD's L2, where the producer's add lands after its
// write-through row stores, without invalidating anything the GEMM waves
// sharing the CU rely on.  Exponential back-off (64 cycles up to about 8k) keeps the polling
// traffic on the counters' few cache lines low.
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

// Token t's slots into this wave's LDS row: positions (-1: no row) and
// weights; the feature loop may leave lanes idle, so it reads them from LDS.
__device__ __forceinline__ void token_slots(const int32_t* __restrict__ pos, const float* __restrict__ w, int t,
                                            int K, int* pos_l, float* w_l, int lane) {
    int p = -1;
    float wt = 0.0f;
    if (lane < K) {
        p = pos[(size_t)t * K + lane];
        wt = w[(size_t)t * K + lane];
    }
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
// The slots' rows are requested eight at a time (streamed: each is read
// once), then summed in slot order.
template <int YDT, int ODT>
__device__ __forceinline__ void combine_slice(const void* __restrict__ y, const void* __restrict__ shared_out,
                                              void* __restrict__ out, int t, int slice, int K, int H,
                                              const int* pos_l, const float* w_l, int lane) {
    const int v = slice * kWave + lane;
    if (v >= H / 8) return;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    constexpr int G = 8;
    constexpr int NQ = YDT == RDG_BF16 ? 1 : 2;  // 16-byte pieces per lane and row
    for (int k0 = 0; k0 < K; k0 += G) {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        u32x4 q[G][NQ];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const int k = k0 + j;
            if (k < K && pos_l[k] >= 0) {
                const u32x4* p = YDT == RDG_BF16
                                     ? reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(y) +
                                                                      (size_t)pos_l[k] * H) + v
                                     : reinterpret_cast<const u32x4*>(static_cast<const float*>(y) +
                                                                      (size_t)pos_l[k] * H) + 2 * v;
#pragma unroll
                for (int i = 0; i < NQ; ++i) q[j][i] = __builtin_nontemporal_load(p + i);
            }
        }
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const int k = k0 + j;
            if (k >= K || pos_l[k] < 0) continue;
            const float wk = w_l[k];
            if (YDT == RDG_BF16) {
                const uint32_t wd[4] = {q[j][0][0], q[j][0][1], q[j][0][2], q[j][0][3]};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] += wk * bf16_to_f32(wd[i] & 0xffffu);
                    acc[2 * i + 1] += wk * bf16_to_f32(wd[i] >> 16);
                }
            } else {
                const uint32_t wd[8] = {q[j][0][0], q[j][0][1], q[j][0][2], q[j][0][3],
                                        q[j][NQ - 1][0], q[j][NQ - 1][1], q[j][NQ - 1][2], q[j][NQ - 1][3]};
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] += wk * __uint_as_float(wd[i]);
            }
        }
    }
    if (shared_out != nullptr) {
        float sv[8];
        load8<ODT>(shared_out, (size_t)t, H, v, sv);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += sv[i];
    }
    store8<ODT>(out, (size_t)t, H, v, acc);
}

// Plain form: one wave per (token, 512-feature slice) unit, tokens in index
// order.  FINISH: only the tokens whose polling unit (see k_combine_poll: the
// token's last layout row, or m_cap + t / 64 without one) is at or past
// *start, the first unit no polling wave claimed.
template <int YDT, int ODT, bool FINISH>
__global__ __launch_bounds__(256) void k_combine(const void* __restrict__ y, const int32_t* __restrict__ pos,
                                                 const float* __restrict__ w, int T, int K, int H,
                                                 const void* __restrict__ shared_out, void* __restrict__ out,
                                                 int m_cap, const int32_t* __restrict__ start) {
    __shared__ int pos_lds[4][32];
    __shared__ float w_lds[4][32];
    const int wv = threadIdx.x / kWave, lane = lane_id();
    const int n_slices = (H / 8 + kWave - 1) / kWave;
    const int64_t stride = (int64_t)gridDim.x * 4;
    const int64_t n_units = (int64_t)T * n_slices;
    const int u0 = FINISH ? *start : 0;
    for (int64_t unit = (int64_t)blockIdx.x * 4 + wv; unit < n_units; unit += stride) {
        const int t = (int)(unit / n_slices), slice = (int)(unit % n_slices);
        token_slots(pos, w, t, K, pos_lds[wv], w_lds[wv], lane);
        if constexpr (FINISH) {
            int last = -1;
            for (int k = 0; k < K; ++k) last = max(last, pos_lds[wv][k]);
            const int64_t u = last >= 0 ? (int64_t)last : (int64_t)m_cap + t / kWave;
            if (u < u0) continue;  // combined by a polling wave (uniform)
        }
        combine_slice<YDT, ODT>(y, shared_out, out, t, slice, K, H, pos_lds[wv], w_lds[wv], lane);
    }
}

// Closes the polling form's unit counter: polling waves that claim after
// this get a unit >= kClaimClosed and stop; every unit below the counter's
// value before the close is theirs, every unit from it on the finishing
// form's.
constexpr int32_t kClaimClosed = 1 << 30;
__global__ void k_combine_close(int32_t* claim, int32_t* start, int n_units) {
    if (threadIdx.x != 0) return;
    const int32_t old = __hip_atomic_fetch_add(claim, kClaimClosed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // closed before (old >= kClaimClosed, or wrapped negative by repeated
    // closes): nothing is left for this call
    *start = old >= 0 && old < n_units ? old : n_units;
}

// Eight features of a published row (device-scope loads: see load8_published),
// as the raw 16 bytes of bf16 (or two 16-byte halves of fp32).
template <int YDT>
struct Raw;
template <>
struct Raw<RDG_BF16> {
    uint64_t a, b;
    __device__ void load(const void* y, size_t row, int H, int v) {
        const uint64_t* p = reinterpret_cast<const uint64_t*>(static_cast<const uint16_t*>(y) + row * H) + 2 * v;
        a = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        b = __hip_atomic_load(p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __device__ void fma_into(float* acc, float wk) const {
        const uint32_t q[4] = {(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32)};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] += wk * bf16_to_f32(q[i] & 0xffffu);
            acc[2 * i + 1] += wk * bf16_to_f32(q[i] >> 16);
        }
    }
};
template <>
struct Raw<RDG_F32> {
    uint64_t q[4];
    __device__ void load(const void* y, size_t row, int H, int v) {
        const uint64_t* p = reinterpret_cast<const uint64_t*>(static_cast<const float*>(y) + row * H) + 4 * v;
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = __hip_atomic_load(p + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __device__ void fma_into(float* acc, float wk) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] += wk * __uint_as_float((uint32_t)q[i]);
            acc[2 * i + 1] += wk * __uint_as_float((uint32_t)(q[i] >> 32));
        }
    }
};

// Device-scope direct load of 16 bytes per lane into LDS (lds + 16 * lane,
// lds wave-uniform): the rows a concurrently running producer on another XCD
// has published are read past this CU's L1 and any stale line of this XCD's
// L2 (device scope), streamed (nt), and land in LDS without occupying
// registers, so a wave can have many of them in flight.  Issued from inline
// assembly; the caller waits for them (vmcnt) before reading the LDS.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16_device_scope(const void* src, const void* lds) {
    typedef __attribute__((address_space(3))) void* lds_ptr_t;
    const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)lds);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off sc1 nt" ::"v"(src), "s"(l) : "memory", "m0");
}
#pragma clang diagnostic pop

// Polling form.  Units: one layout row each (a token is combined at its
// last layout row, max_k pos[t,k]), then units of 64 tokens (the tokens with
// no row here, which get the shared output or zero).  Each wave claims the
// next unit from *claim (a relaxed device-scope add; the row tiles complete
// in layout order, so the claimed units follow the down GEMM) until the
// units run out or the finishing form has closed the counter.  Per token: lane k < K holds
// slot k; lane 0 waits for the counter of each row tile the token reads (the
// last confirmed tile is remembered).  Then the token's rows are staged in
// groups: for bf16 rows, SB 512-feature pieces per wave go through LDS by
// device-scope direct loads, all in flight at once (SB / local rows slices
// of every local row per group), and each slice is summed in slot order in
// fp32 -- the same sum, in the same order, as the plain form.
template <int YDT, int ODT>
__global__ __launch_bounds__(256) void k_combine_poll(const void* __restrict__ y, const int32_t* __restrict__ pos,
                                                      const int32_t* __restrict__ row_src, int m_cap,
                                                      const float* __restrict__ w, int T, int K, int H,
                                                      const void* __restrict__ shared_out, void* __restrict__ out,
                                                      const int32_t* signals, int rows_per_sig, int threshold,
                                                      uint64_t timeout_ticks, int32_t* claim, int32_t* status) {
    constexpr int SB = 8;  // staged pieces of 64 lanes x 16 bytes per wave
    __shared__ __attribute__((aligned(16))) uint8_t stage[4][SB][1024];
    const int lane = lane_id(), wv = threadIdx.x / kWave;
    const int64_t row_units = m_cap;
    const int64_t n_units = row_units + ((int64_t)T + kWave - 1) / kWave;
    const int nvec = H / 8, n_slices = (nvec + kWave - 1) / kWave;
    int known_tile = -1;
    for (;;) {
        int claimed = 0;
        if (lane == 0) claimed = __hip_atomic_fetch_add(claim, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int64_t u = __shfl(claimed, 0);
        if (u < 0 || u >= n_units) break;  // uniform: no units left, or closed (wrapped if closed twice)
        int tok = -1;
        bool mine = false;
        if (u < row_units) {
            if (lane == 0) {
                const int src = row_src[u];
                if (src >= 0) {
                    tok = src / K;
                    int last = -1;
                    for (int k = 0; k < K; ++k) last = max(last, pos[(size_t)tok * K + k]);
                    mine = last == (int)u;
                }
            }
        } else {
            const int64_t tt = (u - row_units) * kWave + lane;
            if (tt < T) {
                tok = (int)tt;
                int last = -1;
                for (int k = 0; k < K; ++k) last = max(last, pos[(size_t)tok * K + k]);
                mine = last < 0;
            }
        }
        uint64_t todo = __ballot(mine);
        while (todo) {
            const int i = __builtin_ctzll(todo);
            todo &= todo - 1;
            const int t = __shfl(tok, i);
            int p = -1;
            float wt = 0.0f;
            if (lane < K) {
                p = pos[(size_t)t * K + lane];
                wt = w[(size_t)t * K + lane];
            }
            for (int k = 0; k < K; ++k) {
                const int pk = __shfl(p, k);
                if (pk < 0) continue;
                const int tile = pk / rows_per_sig;
                if (tile == known_tile) continue;
                int ok = 1;
                if (lane == 0) {
                    ok = wait_counter(signals + tile, threshold, timeout_ticks) ? 1 : 0;
                    if (!ok) set_status(status, RDG_ETIMEOUT, tile);
                }
                ok = __shfl(ok, 0);
                if (ok) known_tile = tile;
                else if (lane == k) p = -1;  // skip the incomplete row
            }
            // the rows are read with device-scope loads; this fence keeps
            // those loads after the polls
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            const uint64_t slots = __ballot(lane < K && p >= 0);
            const int nk = __popcll(slots);
            if constexpr (YDT == RDG_BF16) {
                // G slices of every local row per staging round (rows in
                // rounds of SB when there are more local rows than pieces)
                const int G = nk == 0 ? n_slices : nk >= SB ? 1 : SB / nk;
                for (int g0 = 0; g0 < n_slices; g0 += G) {
                    const int ng = n_slices - g0 < G ? n_slices - g0 : G;
                    if (nk <= SB) {
                        int j = 0;
                        for (uint64_t m = slots; m; m &= m - 1, ++j) {
                            const uint8_t* row =
                                static_cast<const uint8_t*>(y) + (size_t)__shfl(p, __builtin_ctzll(m)) * H * 2;
                            for (int s2 = 0; s2 < ng; ++s2) {
                                const int v = (g0 + s2) * kWave + lane;
                                dma16_device_scope(row + (size_t)(v < nvec ? v : nvec - 1) * 16, stage[wv][j * G + s2]);
                            }
                        }
                        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the pieces are in LDS
                    }
                    for (int s2 = 0; s2 < ng; ++s2) {
                        const int v = (g0 + s2) * kWave + lane;
                        float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                        for (int r0 = 0; r0 < nk; r0 += SB) {
                            uint64_t m = slots;
                            for (int q = 0; q < r0; ++q) m &= m - 1;  // skip the rows of earlier rounds
                            if (nk > SB) {
                                uint64_t mm = m;
                                for (int j = 0; j < SB && mm; ++j, mm &= mm - 1) {
                                    const uint8_t* row =
                                        static_cast<const uint8_t*>(y) + (size_t)__shfl(p, __builtin_ctzll(mm)) * H * 2;
                                    dma16_device_scope(row + (size_t)(v < nvec ? v : nvec - 1) * 16, stage[wv][j]);
                                }
                                __builtin_amdgcn_s_waitcnt(0x0f70);
                            }
                            for (int j = 0; j < SB && m; ++j, m &= m - 1) {
                                const float wk = __shfl(wt, __builtin_ctzll(m));
                                const uint4 q = *reinterpret_cast<const uint4*>(
                                    stage[wv][nk > SB ? j : j * G + s2] + lane * 16);
                                const uint32_t qq[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                                for (int e = 0; e < 4; ++e) {
                                    a[2 * e] += wk * bf16_to_f32(qq[e] & 0xffffu);
                                    a[2 * e + 1] += wk * bf16_to_f32(qq[e] >> 16);
                                }
                            }
                            if (nk > SB) __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0) before restaging
                        }
                        if (v < nvec) {
                            if (shared_out != nullptr) {
                                float sv[8];
                                load8<ODT>(shared_out, (size_t)t, H, v, sv);
#pragma unroll
                                for (int q = 0; q < 8; ++q) a[q] += sv[q];
                            }
                            store8<ODT>(out, (size_t)t, H, v, a);
                        }
                    }
                    // the next group's loads overwrite the pieces: this wave's LDS reads first
                    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
                }
            } else {
#pragma unroll 1
                for (int v = lane; v < nvec; v += kWave) {
                    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                    for (uint64_t m = slots; m; m &= m - 1) {
                        const int k = __builtin_ctzll(m);
                        Raw<YDT> r;
                        r.load(y, (size_t)__shfl(p, k), H, v);
                        r.fma_into(a, __shfl(wt, k));
                    }
                    if (shared_out != nullptr) {
                        float sv[8];
                        load8<ODT>(shared_out, (size_t)t, H, v, sv);
#pragma unroll
                        for (int q = 0; q < 8; ++q) a[q] += sv[q];
                    }
                    store8<ODT>(out, (size_t)t, H, v, a);
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_combine(const void* y, int y_dt, const int32_t* pos, const int32_t* row_src, int m_cap,
                          const float* w, int T, int K, int H, const void* shared_out, void* out, int out_dt,
                          int32_t* signals, int rows_per_sig, int threshold, uint64_t timeout_ticks,
                          int max_blocks, int32_t* status, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const bool ready = signals != nullptr;
    // the unit counter follows the row tiles' counters
    int32_t* claim = ready ? signals + (m_cap + rows_per_sig - 1) / rows_per_sig : nullptr;
    int64_t blocks;
    if (ready) {
        // Polling workgroups hold their CU's resources while they wait, and a
        // down-GEMM workgroup needs most of a CU: at most a quarter of the
        // CUs' worth of them (fewer if max_blocks says so), so that the GEMM
        // always keeps three quarters of the CUs.  (Beside a GEMM workgroup
        // that leaves room for one, a polling workgroup would take no CU;
        // but registers and LDS are allocated in contiguous ranges, and a
        // polling workgroup placed off the gap blocks the CU for the GEMM
        // until it exits -- not a placement the launch can control.)
        int dev = 0, n_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return hipErrorInvalidDevice;
        const int cap = n_cu / 4 > 0 ? n_cu / 4 : 1;
        blocks = max_blocks > 0 && max_blocks < cap ? max_blocks : cap;
        const int64_t units = (int64_t)m_cap + ((int64_t)T + kWave - 1) / kWave;
        if (blocks > (units + 3) / 4) blocks = (units + 3) / 4;
    } else {
        const int64_t units = (int64_t)T * ((H / 8 + kWave - 1) / kWave);
        blocks = (units + 3) / 4;
        if (max_blocks > 0 && blocks > max_blocks) blocks = max_blocks;
    }
#define RDG_COMBINE(YD, OD)                                                                                      \
    do {                                                                                                         \
        if (ready)                                                                                               \
            k_combine_poll<YD, OD><<<(unsigned)blocks, 256, 0, s>>>(y, pos, row_src, m_cap, w, T, K, H,           \
                                                                  shared_out, out, signals, rows_per_sig,       \
                                                                  threshold, timeout_ticks, claim, status);     \
        else                                                                                                     \
            k_combine<YD, OD, false><<<(unsigned)blocks, 256, 0, s>>>(y, pos, w, T, K, H, shared_out, out, 0,     \
                                                                     nullptr);                                  \
    } while (0)
    if (y_dt == RDG_BF16 && out_dt == RDG_BF16) RDG_COMBINE(RDG_BF16, RDG_BF16);
    else if (y_dt == RDG_BF16 && out_dt == RDG_F32) RDG_COMBINE(RDG_BF16, RDG_F32);
    else if (y_dt == RDG_F32 && out_dt == RDG_F32) RDG_COMBINE(RDG_F32, RDG_F32);
    else return hipErrorInvalidValue;
#undef RDG_COMBINE
    return hipGetLastError();
}

hipError_t launch_combine_finish(const void* y, int y_dt, const int32_t* pos, int m_cap, const float* w, int T, int K,
                                 int H, const void* shared_out, void* out, int out_dt, int32_t* signals,
                                 int rows_per_sig, hipStream_t s) {
    if (T == 0) return hipSuccess;
    int32_t* claim = signals + (m_cap + rows_per_sig - 1) / rows_per_sig;
    const int64_t n_units = (int64_t)m_cap + ((int64_t)T + kWave - 1) / kWave;
    k_combine_close<<<1, kWave, 0, s>>>(claim, claim + 1, (int)n_units);
    const int64_t units = (int64_t)T * ((H / 8 + kWave - 1) / kWave);
    const unsigned blocks = (unsigned)((units + 3) / 4);
#define RDG_FINISH(YD, OD) \
    k_combine<YD, OD, true><<<blocks, 256, 0, s>>>(y, pos, w, T, K, H, shared_out, out, m_cap, claim + 1)
    if (y_dt == RDG_BF16 && out_dt == RDG_BF16) RDG_FINISH(RDG_BF16, RDG_BF16);
    else if (y_dt == RDG_BF16 && out_dt == RDG_F32) RDG_FINISH(RDG_BF16, RDG_F32);
    else if (y_dt == RDG_F32 && out_dt == RDG_F32) RDG_FINISH(RDG_F32, RDG_F32);
    else return hipErrorInvalidValue;
#undef RDG_FINISH
    return hipGetLastError();
}

}  // namespace rdg
