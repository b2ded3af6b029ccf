// Dispatch: EPLB remap, the layout builder (a stable counting sort by
// expert) and the payload permutation.
//
// What it computes (SGLang large-scale EP chapter, self-test answer 1 and
// the DeepEP-modes paragraph: the contiguous layout orders tokens by expert
// for the dynamic shapes of prefill, the masked layout keeps fixed shapes
// with a mask of valid rows for decode; H100 deployment article, "DeepEP-
// based EP": overflowing a preallocated fixed buffer is an error; DeepEP
// deep-dive, "normal kernels": a counting pass precedes the transfer, which
// there costs a device-to-host wait -- here the counts stay on the device).
//
// Design for CDNA4, three launches, no host round trip:
//   1. rank:    one wave per chunk of entries; within each 64-entry piece the
//               lanes holding the same expert find each other with one ballot
//               per bit of the expert id, which gives each entry its rank
//               among equal experts in flat order; a per-wave LDS counter
//               carries ranks across pieces.  Writes the chunk histograms.
//   2. scan:    one workgroup turns the chunk histograms into per-chunk bases,
//               counts, padded offsets, masked_m, capacity status and the row
//               tile tables used by the grouped GEMM.
//   3. scatter: one wave per (token, 1 KiB slice of its row) computes the K
//               destinations and copies the slice once from HBM into each of
//               them (16-byte vectors); slicing keeps small batches from
//               leaving most CUs idle.
#include <mutex>

#include "rdg_internal.h"

namespace rdg {
namespace {

__global__ __launch_bounds__(256) void k_remap(const int32_t* __restrict__ ids, const int64_t* __restrict__ gidx,
                                               int T, int K, const int32_t* __restrict__ log2phy,
                                               const int32_t* __restrict__ n_rep, int r_max, int n_logical,
                                               int phys_begin, int n_local, int32_t* out) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)T * K) return;
    int32_t e = ids[i], r = -1;
    if (e >= 0 && e < n_logical) {
        const int32_t nr = n_rep[e];
        if (nr >= 1 && nr <= r_max) {  // a malformed replica count maps the row nowhere
            int64_t g = gidx[i / K] % nr;
            if (g < 0) g += nr;
            const int32_t p = log2phy[(int64_t)e * r_max + g];
            if (p >= phys_begin && p < phys_begin + n_local) r = p - phys_begin;
        }
    }
    out[i] = r;
}

__global__ __launch_bounds__(256) void k_fill_i32(int32_t* p, int32_t v, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// Pass 1.  grid: ceil(n_chunks / 4) workgroups of 4 waves; dynamic LDS: 4 * n_local int32.
__global__ __launch_bounds__(256) void k_rank(const int32_t* __restrict__ ids, int64_t n, int n_local, int chunk,
                                              int n_chunks, int nbits, int32_t* __restrict__ tmp_rank,
                                              int32_t* __restrict__ chunk_counts, int32_t* __restrict__ row_src,
                                              int m_cap, int32_t* __restrict__ status) {
    extern __shared__ int32_t cnt_all[];
    const int wv = threadIdx.x / kWave, lane = lane_id();
    int32_t* cnt = cnt_all + wv * n_local;
    const int c = blockIdx.x * 4 + wv;

    // housekeeping spread over the grid: clear the status word, mark all rows as padding
    if (blockIdx.x == 0 && threadIdx.x == 0 && status) {
        status[0] = 0;
        status[1] = 0;
    }
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < m_cap; i += (int64_t)gridDim.x * blockDim.x)
        row_src[i] = -1;

    if (c >= n_chunks) return;  // per-wave exit; no workgroup barrier follows
    for (int e = lane; e < n_local; e += kWave) cnt[e] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    const uint64_t lt_mask = (1ull << lane) - 1ull;
    for (int p = 0; p < chunk; p += kWave) {
        int64_t i = (int64_t)c * chunk + p + lane;
        int e = -1;
        if (i < n) {
            e = ids[i];
            if (e < 0 || e >= n_local) e = -1;
        }
        const uint32_t key = (uint32_t)(e + 1);
        uint64_t same = ~0ull;
        for (int b = 0; b < nbits; ++b) {
            const uint32_t bit = (key >> b) & 1u;
            const uint64_t bal = __ballot(bit);
            same &= bit ? bal : ~bal;
        }
        if (e >= 0) {
            const int base = cnt[e];
            tmp_rank[i] = base + __popcll(same & lt_mask);
            if (lane == 63 - __clzll(same)) cnt[e] = base + __popcll(same);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    for (int e = lane; e < n_local; e += kWave) chunk_counts[(size_t)c * n_local + e] = cnt[e];
}

// Pass 2 runs as one workgroup of 256 threads (four waves, one per SIMD,
// about 60 registers per lane), so that it can start on a CU where another
// stream's GEMM workgroup (the shared expert's) leaves room beside it; a
// 1024-thread form (four waves per SIMD) needed a whole CU to itself.  (The
// 128-row bf16 GEMM's two waves per SIMD take 480 of the SIMD's 512
// registers, so next to that one it still waits; its own work is 10-16 us
// on a 4096-token batch.)
constexpr int kScanThreads = 256;
constexpr int kScanEPT = 4;  // experts per thread (n_local <= 1024)
static_assert(kScanThreads * kScanEPT >= 1024 && kScanEPT == 4, "the 16-byte loads of k_scan hold four experts");

// Exclusive scan over the pass-2 workgroup (4 waves); lds4: 4 ints.
__device__ int block_exclusive_scan(int v, int* lds4, int* total) {
    const int lane = lane_id(), wv = threadIdx.x / kWave;
    int x = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == kWave - 1) lds4[wv] = x;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kScanThreads / kWave; ++w) {
        const int t = lds4[w];
        before += w < wv ? t : 0;
        tot += t;
    }
    __syncthreads();
    *total = tot;
    return before + x - v;
}

__device__ int block_max(int v, int* lds4) {
    const int lane = lane_id(), wv = threadIdx.x / kWave;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = max(v, __shfl_xor(v, off));
    if (lane == 0) lds4[wv] = v;
    __syncthreads();
    int m = lds4[0];
#pragma unroll
    for (int w = 1; w < kScanThreads / kWave; ++w) m = max(m, lds4[w]);
    __syncthreads();
    return m;
}

// Exclusive scan of the values v[i] of experts kScanEPT*j + i (thread j, in
// expert order): each expert's offset, and the total.
__device__ void experts_exclusive_scan(const int (&v)[kScanEPT], int (&out)[kScanEPT], int* lds4, int* total) {
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kScanEPT; ++i) {
        out[i] = sum;
        sum += v[i];
    }
    const int base = block_exclusive_scan(sum, lds4, total);
#pragma unroll
    for (int i = 0; i < kScanEPT; ++i) out[i] += base;
}

// Pass 2.  Thread j owns experts kScanEPT*j .. +kScanEPT-1: the exclusive
// scan of each expert's per-chunk counts over the chunks (each chunk's base
// row inside the expert), the expert's count, then offsets, masked_m, the
// status and the row-tile tables, all scans in expert order.
__global__ __launch_bounds__(kScanThreads) void k_scan(int32_t* __restrict__ chunk_counts, int n_chunks,
                                                       int n_local, int kind, int block_m, int m_max, int m_cap,
                                                       int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ masked_m,
                                                       int32_t* __restrict__ tile_off, int32_t* __restrict__ status,
                                                       int64_t* __restrict__ expert_load) {
    __shared__ int lds[4];
    __shared__ int cells[1024];
    const int j = threadIdx.x;
    const int e0 = j * kScanEPT;
    int run[kScanEPT];
#pragma unroll
    for (int i = 0; i < kScanEPT; ++i) run[i] = 0;
    const int64_t n_cells = (int64_t)n_local * n_chunks;
    if (n_cells <= 1024) {
        // every (chunk, expert) count in one round of loads; each expert's
        // column scanned from LDS
        for (int c = j; c < n_cells; c += kScanThreads) cells[c] = chunk_counts[c];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kScanEPT; ++i) {
            if (e0 + i >= n_local) continue;
            for (int c = 0; c < n_chunks; ++c) {
                const int v = cells[c * n_local + e0 + i];
                cells[c * n_local + e0 + i] = run[i];
                run[i] += v;
            }
        }
        __syncthreads();
        for (int c = j; c < n_cells; c += kScanThreads) chunk_counts[c] = cells[c];
    } else if (e0 < n_local) {
        if (n_local % kScanEPT == 0) {
            // a row of the chunk table is n_local ints from a 256-byte aligned
            // base: the thread's four experts are one aligned 16-byte vector
            int c = 0;
            for (; c + 8 <= n_chunks; c += 8) {  // eight independent loads, then their scans
                int4 v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    v[u] = *reinterpret_cast<const int4*>(chunk_counts + (size_t)(c + u) * n_local + e0);
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    *reinterpret_cast<int4*>(chunk_counts + (size_t)(c + u) * n_local + e0) =
                        make_int4(run[0], run[1], run[2], run[3]);
                    run[0] += v[u].x;
                    run[1] += v[u].y;
                    run[2] += v[u].z;
                    run[3] += v[u].w;
                }
            }
            for (; c < n_chunks; ++c) {
                int4* p = reinterpret_cast<int4*>(chunk_counts + (size_t)c * n_local + e0);
                const int4 v = *p;
                *p = make_int4(run[0], run[1], run[2], run[3]);
                run[0] += v.x;
                run[1] += v.y;
                run[2] += v.z;
                run[3] += v.w;
            }
        } else {
            for (int c = 0; c < n_chunks; ++c) {
#pragma unroll
                for (int i = 0; i < kScanEPT; ++i) {
                    if (e0 + i >= n_local) continue;
                    int32_t* p = chunk_counts + (size_t)c * n_local + e0 + i;
                    const int v = *p;
                    *p = run[i];
                    run[i] += v;
                }
            }
        }
    }
    int seg[kScanEPT], off[kScanEPT], keep[kScanEPT];
    int worst = 0;
#pragma unroll
    for (int i = 0; i < kScanEPT; ++i) {
        const int e = e0 + i;
        const bool act = e < n_local;
        if (act) {
            counts[e] = run[i];
            // the expert-load recorder: routed rows before any capacity drop
            if (expert_load != nullptr)
                atomicAdd(reinterpret_cast<unsigned long long*>(expert_load + e), (unsigned long long)run[i]);
        }
        seg[i] = !act ? 0 : kind == RDG_MASKED ? m_max : (run[i] + block_m - 1) / block_m * block_m;
        worst = act && run[i] > worst ? run[i] : worst;
    }
    int total;
    experts_exclusive_scan(seg, off, lds, &total);
#pragma unroll
    for (int i = 0; i < kScanEPT; ++i) {
        int k = run[i];
        if (kind == RDG_MASKED && k > m_max) k = m_max;
        if (kind == RDG_CONTIGUOUS) {
            int room = m_cap - off[i];
            if (room < 0) room = 0;
            if (k > room) k = room;
        }
        keep[i] = e0 + i < n_local ? k : 0;
        if (e0 + i < n_local) {
            offsets[e0 + i] = off[i];
            masked_m[e0 + i] = keep[i];
        }
    }
    if (j == 0) offsets[n_local] = total;
    worst = block_max(worst, lds);
    if (j == 0) {
        if (kind == RDG_MASKED && worst > m_max) set_status(status, RDG_ECAPACITY, worst);
        if (kind == RDG_CONTIGUOUS && total > m_cap) set_status(status, RDG_ECAPACITY, total);
    }
    for (int b = 0; b < kNumBT; ++b) {
        int nt[kScanEPT], to[kScanEPT];
#pragma unroll
        for (int i = 0; i < kScanEPT; ++i) nt[i] = (keep[i] + kBT[b] - 1) / kBT[b];
        int tt;
        experts_exclusive_scan(nt, to, lds, &tt);
#pragma unroll
        for (int i = 0; i < kScanEPT; ++i)
            if (e0 + i < n_local) tile_off[b * (n_local + 1) + e0 + i] = to[i];
        if (j == 0) tile_off[b * (n_local + 1) + n_local] = tt;
    }
}

// Pass 3.  One wave per (token, 64-vector slice of its row): the slice-0
// wave also publishes pos and row_src.  Without x_perm (a grouped GEMM that
// gathers its token rows through row_src) only that wave runs per token.
// chunk_base = NULL: pos was published by k_dispatch_small; only the rows
// are copied.  row_bytes: bytes of one x row (a
// multiple of 16); n_slices = ceil(row_bytes / 1024).
__global__ __launch_bounds__(256) void k_scatter(const uint8_t* __restrict__ x, const float* __restrict__ x_s,
                                                 int row_bytes, int n_scales, int n_slices, int T, int K,
                                                 const int32_t* __restrict__ ids, int n_local, int chunk,
                                                 const int32_t* __restrict__ chunk_base,
                                                 const int32_t* __restrict__ tmp_rank,
                                                 const int32_t* __restrict__ offsets,
                                                 const int32_t* __restrict__ masked_m, int32_t* __restrict__ pos,
                                                 int32_t* __restrict__ row_src, uint8_t* __restrict__ x_perm,
                                                 float* __restrict__ x_perm_s) {
    __shared__ int dst_lds[4][32];
    const int wv = threadIdx.x / kWave, lane = lane_id();
    const int64_t unit = (int64_t)blockIdx.x * 4 + wv;
    if (unit >= (int64_t)T * n_slices) return;
    const int t = (int)(unit / n_slices), slice = (int)(unit % n_slices);
    int p = -1;
    if (lane < K) {
        const int64_t i = (int64_t)t * K + lane;
        if (chunk_base == nullptr) {
            p = pos[i];  // published already (small dispatches): the copy only
        } else {
            const int e = ids[i];
            if (e >= 0 && e < n_local) {
                const int r = chunk_base[(size_t)(i / chunk) * n_local + e] + tmp_rank[i];
                if (r < masked_m[e]) p = offsets[e] + r;
            }
            if (slice == 0) {
                pos[i] = p;
                if (p >= 0) row_src[p] = (int32_t)i;
            }
        }
        dst_lds[wv][lane] = p;
    }
    if (x_perm == nullptr) return;  // layout only: the grouped GEMM gathers the rows (uniform)
    // the copy loops below leave lanes idle, so the destinations are read
    // from the wave's LDS slice rather than shuffled from other lanes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int* dst = dst_lds[wv];
    // rows stored past the caches (written once here, read once by the
    // grouped GEMM): 124 -> 112 us for the 4096-token prefill layer
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4* src = reinterpret_cast<const u32x4*>(x + (size_t)t * row_bytes);
    const int v = slice * kWave + lane;
    if (v < row_bytes / 16) {
        const u32x4 val = src[v];
        for (int k = 0; k < K; ++k) {
            const int pk = dst[k];
            if (pk >= 0) __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(x_perm + (size_t)pk * row_bytes) + v);
        }
    }
    if (x_s != nullptr && slice == 0) {
        for (int j = lane; j < n_scales; j += kWave) {
            const float sv = x_s[(size_t)t * n_scales + j];
            for (int k = 0; k < K; ++k) {
                const int pk = dst[k];
                if (pk >= 0) x_perm_s[(size_t)pk * n_scales + j] = sv;
            }
        }
    }
}

// Small dispatches (at most kSmallEntries entries over at most kSmallExperts
// experts: the decode batches and the decode rank share) in one workgroup of
// 16 waves: the three passes above with the per-chunk counters in LDS
// instead of memory and one launch instead of three.  Wave w ranks the
// entries [w*chunk, (w+1)*chunk) as pass 1 does, the waves' counts are
// scanned per expert in wave order (the chunk scan of pass 2), then the
// experts' segments, and every wave publishes its entries' positions.
// Padding rows are marked first; the workgroup barriers order those stores
// before the positions' own.
constexpr int kSmallWaves = 16;
constexpr int kSmallSteps = 8;  // 64-entry steps per wave
constexpr int kSmallEntries = kSmallWaves * kSmallSteps * kWave;  // 8192
constexpr int kSmallExperts = 512;
static_assert(kSmallWaves * kWave >= kSmallExperts && kSmallWaves <= 16,
              "one thread per expert; the scans' wave totals at lds[0..15], the maxima at lds[16..31]");

// Exclusive scan over a 1024-thread workgroup (16 waves); lds: 32 ints.
__device__ int block_scan1024(int v, int* lds, int* total) {
    const int lane = lane_id(), wv = threadIdx.x / kWave;
    int x = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == kWave - 1) lds[wv] = x;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kSmallWaves; ++w) {
        const int t = lds[w];
        before += w < wv ? t : 0;
        tot += t;
    }
    __syncthreads();
    *total = tot;
    return before + x - v;
}

__global__ __launch_bounds__(1024) void k_dispatch_small(const int32_t* __restrict__ ids, int n, int n_local,
                                                         int nbits, int kind, int block_m, int m_max, int m_cap,
                                                         int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ masked_m, int32_t* __restrict__ pos,
                                                         int32_t* __restrict__ row_src,
                                                         int32_t* __restrict__ tile_off, int32_t* __restrict__ status,
                                                         int64_t* __restrict__ expert_load) {
    __shared__ int cnt[kSmallWaves][kSmallExperts];  // per-wave counts, then each wave's base
    __shared__ int s_off[kSmallExperts], s_keep[kSmallExperts];
    __shared__ int lds[32];
    const int wv = threadIdx.x / kWave, lane = lane_id();
    if (threadIdx.x == 0 && status) {
        status[0] = 0;
        status[1] = 0;
    }
    // every row starts as padding (the decode layer's masked layout clears
    // 256 KiB here: 16-byte stores where row_src is 16-byte aligned)
    int i0 = 0;
    if ((reinterpret_cast<uintptr_t>(row_src) & 15) == 0) {
        i0 = m_cap & ~3;
        typedef int i32x4 __attribute__((ext_vector_type(4)));
        const i32x4 pad = {-1, -1, -1, -1};
        for (int i = threadIdx.x * 4; i < i0; i += blockDim.x * 4) *reinterpret_cast<i32x4*>(row_src + i) = pad;
    }
    for (int i = i0 + threadIdx.x; i < m_cap; i += blockDim.x) row_src[i] = -1;
    for (int e = lane; e < n_local; e += kWave) cnt[wv][e] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // pass 1: stable ranks inside each wave's chunk
    const int chunk = (n + kSmallWaves * kWave - 1) / (kSmallWaves * kWave) * kWave;  // <= kSmallSteps * 64
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    int my_e[kSmallSteps], my_r[kSmallSteps];
#pragma unroll
    for (int p = 0; p < kSmallSteps; ++p) {
        my_e[p] = -1;
        my_r[p] = 0;
        if (p * kWave >= chunk) continue;  // uniform
        const int i = wv * chunk + p * kWave + lane;
        int e = -1;
        if (i < n) {
            e = ids[i];
            if (e < 0 || e >= n_local) e = -1;
        }
        const uint32_t key = (uint32_t)(e + 1);
        uint64_t same = ~0ull;
        for (int b = 0; b < nbits; ++b) {
            const uint32_t bit = (key >> b) & 1u;
            const uint64_t bal = __ballot(bit);
            same &= bit ? bal : ~bal;
        }
        if (e >= 0) {
            const int base = cnt[wv][e];
            my_r[p] = base + __popcll(same & lt_mask);
            if (lane == 63 - __clzll(same)) cnt[wv][e] = base + __popcll(same);
        }
        my_e[p] = e;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    __syncthreads();

    // pass 2: expert e's count and each wave's base (thread e), the segments
    const int e = threadIdx.x;
    const bool act = e < n_local;
    int run = 0;
    if (act) {
#pragma unroll
        for (int w = 0; w < kSmallWaves; ++w) {
            const int v = cnt[w][e];
            cnt[w][e] = run;
            run += v;
        }
        counts[e] = run;
        if (expert_load != nullptr)
            atomicAdd(reinterpret_cast<unsigned long long*>(expert_load + e), (unsigned long long)run);
    }
    const int seg = !act ? 0 : kind == RDG_MASKED ? m_max : (run + block_m - 1) / block_m * block_m;
    int total;
    const int off = block_scan1024(seg, lds, &total);
    int keep = run;
    if (kind == RDG_MASKED && keep > m_max) keep = m_max;
    if (kind == RDG_CONTIGUOUS) {
        int room = m_cap - off;
        if (room < 0) room = 0;
        if (keep > room) keep = room;
    }
    if (!act) keep = 0;
    if (act) {
        offsets[e] = off;
        masked_m[e] = keep;
        s_off[e] = off;
        s_keep[e] = keep;
    }
    if (e == 0) offsets[n_local] = total;
    int worst = act ? run : 0;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) worst = max(worst, __shfl_xor(worst, o));
    if (lane == 0) lds[16 + wv] = worst;
    __syncthreads();
    if (threadIdx.x == 0) {
        int m = 0;
        for (int w = 0; w < kSmallWaves; ++w) m = max(m, lds[16 + w]);
        if (kind == RDG_MASKED && m > m_max) set_status(status, RDG_ECAPACITY, m);
        if (kind == RDG_CONTIGUOUS && total > m_cap) set_status(status, RDG_ECAPACITY, total);
    }
    for (int b = 0; b < kNumBT; ++b) {
        const int nt = (keep + kBT[b] - 1) / kBT[b];
        int tt;
        const int to = block_scan1024(nt, lds, &tt);
        if (act) tile_off[b * (n_local + 1) + e] = to;
        if (e == 0) tile_off[b * (n_local + 1) + n_local] = tt;
    }
    __syncthreads();

    // pass 3: positions
#pragma unroll
    for (int p = 0; p < kSmallSteps; ++p) {
        if (p * kWave >= chunk) continue;  // uniform
        const int i = wv * chunk + p * kWave + lane;
        if (i >= n) continue;
        int P = -1;
        const int ee = my_e[p];
        if (ee >= 0) {
            const int r = cnt[wv][ee] + my_r[p];
            if (r < s_keep[ee]) P = s_off[ee] + r;
        }
        pos[i] = P;
        if (P >= 0) row_src[P] = i;
    }
}

__global__ void k_layout_dense(int T, int32_t* counts, int32_t* offsets, int32_t* masked_m, int32_t* tile_off,
                               int32_t* status) {
    if (threadIdx.x != 0) return;
    counts[0] = T;
    masked_m[0] = T;
    offsets[0] = 0;
    offsets[1] = T;
    for (int b = 0; b < kNumBT; ++b) {
        tile_off[b * 2 + 0] = 0;
        tile_off[b * 2 + 1] = (T + kBT[b] - 1) / kBT[b];
    }
    if (status) {
        status[0] = 0;
        status[1] = 0;
    }
}

}  // namespace

hipError_t launch_remap(const int32_t* ids, const int64_t* gidx, int T, int K, const int32_t* log2phy,
                        const int32_t* n_rep, int r_max, int n_logical, int phys_begin, int n_local,
                        int32_t* out, hipStream_t s) {
    int64_t n = (int64_t)T * K;
    if (n == 0) return hipSuccess;
    k_remap<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(ids, gidx, T, K, log2phy, n_rep, r_max, n_logical,
                                                        phys_begin, n_local, out);
    return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    k_fill_i32<<<(unsigned)blocks, 256, 0, s>>>(p, v, n);
    return hipGetLastError();
}

// The three passes.  tile_off: the layout's row-tile tables (an output the
// grouped GEMMs read); chunk_counts [kMaxChunks x n_local] and tmp_rank [T*K]:
// scratch, every element read written first by the same dispatch (k_rank
// writes each used chunk's counts and each routed entry's rank; k_scan and
// k_scatter read only those), so nothing needs clearing between calls.
static hipError_t dispatch_passes(const void* x, const float* x_scales, int row_bytes, int T, int H,
                                  const int32_t* ids, int K, const rdg_layout& L, void* x_perm,
                                  float* x_perm_scales, int32_t* tile_off, int32_t* chunk_counts, int32_t* tmp_rank,
                                  hipStream_t s) {
    const int64_t n = (int64_t)T * K;
    const int chunk = chunk_size_for(n);
    const int n_chunks = n > 0 ? (int)((n + chunk - 1) / chunk) : 0;
    int nbits = 1;
    while ((1 << nbits) < L.n_local + 1) ++nbits;
    const int n_scales = x_scales && x_perm ? H / 128 : 0;

    if (n <= kSmallEntries && L.n_local <= kSmallExperts) {
        k_dispatch_small<<<1, kSmallWaves * kWave, 0, s>>>(ids, (int)n, L.n_local, nbits, L.kind, L.block_m, L.m_max,
                                                           L.m_cap, L.counts, L.offsets, L.masked_m, L.pos,
                                                           L.row_src, tile_off, L.status, L.expert_load);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess || T == 0 || x_perm == nullptr) return err;
        const int n_slices = (row_bytes + 16 * kWave - 1) / (16 * kWave);
        const int64_t units = (int64_t)T * n_slices;
        k_scatter<<<(unsigned)((units + 3) / 4), 256, 0, s>>>(
            static_cast<const uint8_t*>(x), x_scales, row_bytes, n_scales, n_slices, T, K, ids, L.n_local, chunk,
            nullptr, nullptr, L.offsets, L.masked_m, L.pos, L.row_src, static_cast<uint8_t*>(x_perm), x_perm_scales);
        return hipGetLastError();
    }

    // pass 1 (also clears status and marks rows as padding)
    int blocks1 = (n_chunks + 3) / 4;
    int fill_blocks = (int)((L.m_cap + 255) / 256);
    if (blocks1 < fill_blocks) blocks1 = fill_blocks < 1024 ? fill_blocks : 1024;
    if (blocks1 < 1) blocks1 = 1;
    k_rank<<<blocks1, 256, 4 * L.n_local * sizeof(int32_t), s>>>(ids, n, L.n_local, chunk, n_chunks, nbits,
                                                                   tmp_rank, chunk_counts, L.row_src, L.m_cap,
                                                                   L.status);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    k_scan<<<1, kScanThreads, 0, s>>>(chunk_counts, n_chunks, L.n_local, L.kind, L.block_m, L.m_max, L.m_cap, L.counts,
                              L.offsets, L.masked_m, tile_off, L.status, L.expert_load);
    err = hipGetLastError();
    if (err != hipSuccess || T == 0) return err;
    // without x_perm only pos and row_src are published: one wave per token
    const int n_slices = x_perm ? (row_bytes + 16 * kWave - 1) / (16 * kWave) : 1;
    const int64_t units = (int64_t)T * n_slices;
    k_scatter<<<(unsigned)((units + 3) / 4), 256, 0, s>>>(static_cast<const uint8_t*>(x), x_scales, row_bytes, n_scales,
                                                          n_slices, T, K, ids, L.n_local, chunk, chunk_counts,
                                                          tmp_rank, L.offsets, L.masked_m, L.pos, L.row_src,
                                                          static_cast<uint8_t*>(x_perm), x_perm_scales);
    return hipGetLastError();
}

hipError_t launch_dispatch(const void* x, const float* x_scales, int row_bytes, int T, int H, const int32_t* ids,
                           int K, const rdg_layout& L, void* x_perm, float* x_perm_scales, hipStream_t s) {
    uint8_t* ws = static_cast<uint8_t*>(L.work);
    int32_t* tile_off = reinterpret_cast<int32_t*>(ws);
    int32_t* chunk_counts = reinterpret_cast<int32_t*>(ws + ws_tile_off_bytes(L.n_local));
    int32_t* tmp_rank = reinterpret_cast<int32_t*>(ws + ws_tile_off_bytes(L.n_local) + ws_chunk_bytes(L.n_local));
    return dispatch_passes(x, x_scales, row_bytes, T, H, ids, K, L, x_perm, x_perm_scales, tile_off, chunk_counts,
                           tmp_rank, s);
}

// ---------------------------------------------------------------- no allocation
// The allocation-free dispatch keeps its scratch (per-chunk counts for up to
// kMaxChunks x 1024 experts, one rank per dispatched entry for up to
// kNoallocMaxEntries entries) in this file-scope device array: 4.25 MiB,
// held by every GPU the library runs on until the process ends.  Host code
// never passes the array's name to a kernel (in host code it is a stand-in,
// not a device address): the device address comes from hipGetSymbolAddress,
// once per device, with that device current.
namespace {
constexpr size_t kNoallocChunkBytes = sizeof(int32_t) * kMaxChunks * 1024;
constexpr size_t kScratchBytes = kNoallocChunkBytes + sizeof(int32_t) * (size_t)kNoallocMaxEntries;
static_assert(kNoallocChunkBytes % 256 == 0, "rank area aligned");
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}
}  // namespace

hipError_t launch_dispatch_noalloc(const void* x, const float* x_scales, int row_bytes, int T, int H,
                                   const int32_t* ids, int K, const rdg_layout& L, void* x_perm, float* x_perm_scales,
                                   hipStream_t s) {
    void* base = nullptr;
    hipError_t e = scratch_address(&base);
    if (e != hipSuccess) return e;
    int32_t* chunk_counts = static_cast<int32_t*>(base);
    int32_t* tmp_rank = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(base) + kNoallocChunkBytes);
    return dispatch_passes(x, x_scales, row_bytes, T, H, ids, K, L, x_perm, x_perm_scales,
                           static_cast<int32_t*>(L.work), chunk_counts, tmp_rank, s);
}

hipError_t launch_layout_dense(int T, const rdg_layout& L, hipStream_t s) {
    k_layout_dense<<<1, 64, 0, s>>>(T, L.counts, L.offsets, L.masked_m, static_cast<int32_t*>(L.work), L.status);
    return hipGetLastError();
}

}  // namespace rdg
