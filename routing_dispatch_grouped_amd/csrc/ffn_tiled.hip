// Grouped expert FFN for row tiles of 128 rows (prefill, rank shares, the
// shared expert): the same two stages as ffn.hip -- gate/up GEMM with the
// SiLU-gated product (and fp8 re-quantisation of h) in its epilogue, then the
// down GEMM, optionally signalling each finished row tile -- with the
// operand reuse a 128 x 128 output tile needs to approach the MFMA rate.
//
// What it computes: see ffn.hip (DeepEP deep-dive, EP section; H100
// deployment article, "DeepGEMM integration"; DeepGEMM single-batch-overlap
// pull request, sections 2-3).
//
// Design for CDNA4.  A workgroup (8 waves, two per SIMD) owns 128 output
// columns of one expert (128 rows of W1 and of W3 when gated) and a tile of
// 128 layout rows.  Gated, wave w accumulates W1 (w < 4) or W3 for columns
// [32(w%4), +32) over all 128 rows, and the W3 waves hand their sums to the
// W1 waves through LDS for the SiLU-gated product; otherwise wave w covers
// columns [32(w%4), +32) for rows [64(w/4), +64).  Weight operand tiles are
// private to a wave and are loaded straight from the packed weights into
// registers ahead of use (bf16: a chunk ahead; fp8: a step ahead).  The 128-row token tile is
// shared by the eight waves, so it goes through LDS: each chunk (256 bytes of every row) is
// fetched with direct global->LDS loads into a double buffer, and the slot of
// 16-byte piece c of row r is c ^ (r % 16) (chosen through each lane's source
// address), which makes the MFMA-layout LDS reads conflict-free.  Workgroups
// are renumbered so that the token tiles sharing one weight panel run back to
// back on the same XCD and re-read the panel from that XCD's L2.
#include "rdg_internal.h"

namespace rdg {
namespace {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;
typedef int i32x4_t __attribute__((ext_vector_type(4)));

constexpr int TB = 128;          // rows per tile
constexpr int CB = 256;          // bytes of each row per staged chunk
constexpr int CHUNK_LDS = TB * CB;

template <int DT>
struct TOp;

template <>
struct TOp<RDG_BF16> {
    using op_t = bf16x8_t;
    static constexpr int KS = 32, ESZ = 2, BLK = 1024, STEPS = CB / (KS * ESZ);  // 4 steps per chunk
    __device__ static op_t load_w(const uint8_t* tile, int lane) {
        return *reinterpret_cast<const bf16x8_t*>(tile + lane * 16);
    }
    // token operand of step s for local row r, lane group g: 16-byte piece 4s+g
    __device__ static op_t load_x(const uint8_t* buf, int r, int s, int g) {
        const int c = s * 4 + g;
        return *reinterpret_cast<const bf16x8_t*>(buf + r * CB + ((c ^ (r & 15)) << 4));
    }
    __device__ static f32x4_t mma(f32x4_t c, op_t a, op_t b) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <>
struct TOp<RDG_FP8_E4M3> {
    using op_t = i32x8_t;
    static constexpr int KS = 128, ESZ = 1, BLK = 2048, STEPS = CB / KS;  // 2 steps per chunk
    __device__ static op_t load_w(const uint8_t* tile, int lane) {
        const i32x4_t a = *reinterpret_cast<const i32x4_t*>(tile + lane * 16);
        const i32x4_t b = *reinterpret_cast<const i32x4_t*>(tile + 1024 + lane * 16);
        op_t r;
        r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
        r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
        return r;
    }
    // 32 bytes: pieces 8s+2g and 8s+2g+1
    __device__ static op_t load_x(const uint8_t* buf, int r, int s, int g) {
        const int c = s * 8 + g * 2;
        const i32x4_t a = *reinterpret_cast<const i32x4_t*>(buf + r * CB + ((c ^ (r & 15)) << 4));
        const i32x4_t b = *reinterpret_cast<const i32x4_t*>(buf + r * CB + (((c + 1) ^ (r & 15)) << 4));
        op_t o;
        o[0] = a[0]; o[1] = a[1]; o[2] = a[2]; o[3] = a[3];
        o[4] = b[0]; o[5] = b[1]; o[6] = b[2]; o[7] = b[3];
        return o;
    }
    __device__ static f32x4_t mma(f32x4_t c, op_t a, op_t b) {
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
    }
};

struct TArgs {
    const int32_t* offsets;
    const int32_t* masked_m;
    const int32_t* tile_off;  // BT = 128 prefix table
    int n_local, Kdim, Nout, n_tiles_max;
    const uint8_t* X;
    const float* Xs;
    const uint8_t* Wa;
    const uint8_t* Wb;
    const float* Was;
    const float* Wbs;
    uint8_t* O;
    float* Os;
    int32_t* signals;
};

constexpr int NW = 8;            // waves per workgroup

// Stage chunk kc of the tile's rows into an LDS buffer: 32 direct loads of
// one KiB (4 rows x 256 bytes) per workgroup, 4 per wave.  Rows past the
// tile's valid rows re-read the last valid row (in bounds; never stored).
__device__ __forceinline__ void stage_chunk(const uint8_t* X, size_t xstride, int row0, int nvalid, int kc,
                                            uint8_t* buf, int wv, int lane) {
#pragma unroll
    for (int i = 0; i < 32 / NW; ++i) {
        const int q = wv * (32 / NW) + i;  // instruction index: LDS bytes [q*1024, q*1024+1024)
        const int r = q * 4 + lane / 16;   // tile row of this lane's 16 bytes
        const int slot = lane % 16;
        const int c = slot ^ (r & 15);     // source piece for this slot
        const int rr = r < nvalid ? r : nvalid - 1;
        const uint8_t* src = X + (size_t)(row0 + rr) * xstride + (size_t)kc * CB + c * 16;
        __builtin_amdgcn_global_load_lds((gbl_ptr_t)src, (lds_ptr_t)(buf + q * 1024), 16, 0, 0);
    }
}

// Wave roles: gated -- wave w accumulates matrix w/4 (W1 for the gate, W3 for
// the up projection) for columns [32(w%4), +32) over all 128 tile rows;
// not gated -- wave w covers columns [32(w%4), +32) for tile rows [64(w/4), +64).
template <int DT, bool GATED, bool SIGNAL>
__global__ __launch_bounds__(NW * 64, 1) void k_ffn_tiled(TArgs a) {
    using O = TOp<DT>;
    using op_t = typename O::op_t;
    constexpr int S = O::STEPS;
    constexpr int NCT = GATED ? 8 : 4;  // 16-row column tiles per wave
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][CHUNK_LDS];

    // XCD-aware renumbering: hardware block b runs on XCD b % 8, which gets
    // ceil((total - x) / 8) blocks; give XCD x the contiguous logical range
    // starting at x*(total/8) + min(x, total%8) (a bijection for any total), so
    // consecutive row tiles of one weight panel share an L2
    const int gx = a.n_tiles_max, total = gx * gridDim.y;
    const int b = blockIdx.y * gx + blockIdx.x;
    const int xcd = b % 8, q8 = total / 8, r8 = total % 8;
    const int logical = xcd * q8 + (xcd < r8 ? xcd : r8) + b / 8;
    const int fb = logical / gx, tile = logical % gx;

    const int n_tiles = a.tile_off[a.n_local];
    if (tile >= n_tiles) return;  // workgroup-uniform
    int lo = 0, hi = a.n_local;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.tile_off[mid] <= tile) lo = mid;
        else hi = mid;
    }
    const int e = lo;
    const int row0 = a.offsets[e] + (tile - a.tile_off[e]) * TB;
    const int row_end = a.offsets[e] + a.masked_m[e];
    const int nvalid = row_end - row0 < TB ? row_end - row0 : TB;
    const int f0 = fb * 128;
    const int wv = threadIdx.x / kWave, lane = lane_id();
    const int fq = wv % 4;                      // column group
    const int mat = GATED ? wv / 4 : 0;         // 0: W1 / W2, 1: W3
    const int tr0 = GATED ? 0 : (wv / 4) * 64;  // first tile row of this wave
    const int fw = f0 + fq * 32;
    const size_t xstride = (size_t)a.Kdim * O::ESZ;
    const int nks = a.Kdim / O::KS;
    const int nchunks = (int)(xstride / CB);

    const uint8_t* wt[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const size_t grp = (size_t)e * (a.Nout / 16) + (fw + rt * 16) / 16;
        wt[rt] = (mat == 0 ? a.Wa : a.Wb) + grp * nks * O::BLK;
    }
    f32x4_t acc[2][NCT];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) acc[rt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int nkb = a.Kdim / 128;
    const float* wsc = nullptr;  // this wave's weight block scales along K
    if (DT == RDG_FP8_E4M3) wsc = (mat == 0 ? a.Was : a.Wbs) + ((size_t)e * (a.Nout / 128) + f0 / 128) * nkb;

    // prologue: chunk 0 into buffer 0; weights into registers (bf16: the whole
    // first chunk, fp8: the first step)
    stage_chunk(a.X, xstride, row0, nvalid, 0, lds[0], wv, lane);
    constexpr int WS = DT == RDG_FP8_E4M3 ? 1 : S;  // weight steps held per register set
    op_t wreg[WS][2];
#pragma unroll
    for (int s = 0; s < WS; ++s)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) wreg[s][rt] = O::load_w(wt[rt] + (size_t)s * O::BLK, lane);

    for (int kc = 0; kc < nchunks; ++kc) {
        uint8_t* cur = lds[kc & 1];
        __builtin_amdgcn_s_waitcnt(0);  // this wave's share of chunk kc (and its weights) have landed
        __syncthreads();                // ... and every wave's share; buffer kc+1 is free again
        if (kc + 1 < nchunks) stage_chunk(a.X, xstride, row0, nvalid, kc + 1, lds[(kc + 1) & 1], wv, lane);
        op_t wnext[WS][2];
        if (DT != RDG_FP8_E4M3 && kc + 1 < nchunks) {
#pragma unroll
            for (int s = 0; s < WS; ++s)
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) wnext[s][rt] = O::load_w(wt[rt] + (size_t)((kc + 1) * S + s) * O::BLK, lane);
        }
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int ws = DT == RDG_FP8_E4M3 ? 0 : s;
            const int t = kc * S + s;  // global step
            float sw = 0.0f;
            if (DT == RDG_FP8_E4M3) {
                if (t + 1 < nks) {  // next step's weights while this step computes
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt) wnext[0][rt] = O::load_w(wt[rt] + (size_t)(t + 1) * O::BLK, lane);
                }
                sw = wsc[t];
            }
            // one column tile's token operand at a time
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const op_t xo = O::load_x(cur, tr0 + ct * 16 + (lane & 15), s, lane >> 4);
                if (DT != RDG_FP8_E4M3) {
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt) acc[rt][ct] = O::mma(acc[rt][ct], wreg[ws][rt], xo);
                } else {
                    // one MFMA per 128-long block, promoted with its activation and weight scales
                    const int r = tr0 + ct * 16 + (lane & 15);
                    const float sx = a.Xs[(size_t)(row0 + (r < nvalid ? r : nvalid - 1)) * nkb + t];
                    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt) acc[rt][ct] += O::mma(z, wreg[0][rt], xo) * (sx * sw);
                }
            }
            if (DT == RDG_FP8_E4M3 && t + 1 < nks) {
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) wreg[0][rt] = wnext[0][rt];
            }
        }
        if (DT != RDG_FP8_E4M3 && kc + 1 < nchunks) {
#pragma unroll
            for (int s = 0; s < WS; ++s)
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) wreg[s][rt] = wnext[s][rt];
        }
    }

    // ---------------------------------------------------------------- epilogue
    // 16x16 accumulator tile: lane l holds column (row of the layout) l % 16 and
    // rows (output features) 4*(l/16) .. +3
    const int fl = fw + (lane >> 4) * 4;
    if (GATED) {
        // the up-projection waves hand their accumulators to the gate waves
        __syncthreads();  // every wave is done with the staging buffers
        f32x4_t* xch = reinterpret_cast<f32x4_t*>(lds[0]);  // [4 column groups][2][8][64 lanes] = 64 KiB
        if (mat == 1) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) xch[((fq * 2 + rt) * 8 + ct) * kWave + lane] = acc[rt][ct];
        }
        __syncthreads();
        if (mat == 0) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    const f32x4_t u = xch[((fq * 2 + rt) * 8 + ct) * kWave + lane];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float g = acc[rt][ct][r];
                        acc[rt][ct][r] = g / (1.0f + __expf(-g)) * u[r];
                    }
                }
        }
        __syncthreads();  // the exchange area is free again
    }
    if (DT == RDG_FP8_E4M3 && GATED) {
        // h re-quantised with one fp32 scale per row and 128 columns: amax over
        // the four gate waves' 32 columns each
        float* red = reinterpret_cast<float*>(lds[0]);  // [4 column groups][128 rows]
        if (mat == 0) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                float m = 0.0f;
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(acc[rt][ct][r]));
                m = fmaxf(m, __shfl_xor(m, 16));
                m = fmaxf(m, __shfl_xor(m, 32));
                if (lane < 16) red[fq * TB + ct * 16 + lane] = m;
            }
        }
        __syncthreads();
        if (mat == 0) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const int c = ct * 16 + (lane & 15);
                const float amax = fmaxf(fmaxf(red[c], red[TB + c]), fmaxf(red[2 * TB + c], red[3 * TB + c]));
                if (c >= nvalid) continue;
                const int row = row0 + c;
                const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
                const float inv = 1.0f / sc;
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    uint32_t q = 0;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float tq = fminf(fmaxf(acc[rt][ct][r] * inv, -448.0f), 448.0f);
                        q |= f32_to_e4m3(tq) << (8 * r);
                    }
                    *reinterpret_cast<uint32_t*>(a.O + (size_t)row * a.Nout + fl + rt * 16) = q;
                }
                if (fq == 0 && lane < 16) a.Os[(size_t)row * (a.Nout / 128) + f0 / 128] = sc;
            }
        }
    } else if (mat == 0) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const int c = tr0 + ct * 16 + (lane & 15);
            if (c >= nvalid) continue;
            const int row = row0 + c;
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                uint2 o;
                o.x = f32_to_bf16(acc[rt][ct][0]) | (f32_to_bf16(acc[rt][ct][1]) << 16);
                o.y = f32_to_bf16(acc[rt][ct][2]) | (f32_to_bf16(acc[rt][ct][3]) << 16);
                *reinterpret_cast<uint2*>(a.O + ((size_t)row * a.Nout + fl + rt * 16) * 2) = o;
            }
        }
    }
    if (SIGNAL) {
        __threadfence();
        __syncthreads();
        if (threadIdx.x == 0)
            __hip_atomic_fetch_add(a.signals + row0 / TB, 128, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int DT>
hipError_t launch_dt(const FfnCall& c, hipStream_t s) {
    dim3 block(NW * 64);
    if (c.stages & 1) {
        TArgs g{c.offsets, c.masked_m, c.tile_off, c.n_local, c.H, c.I, c.n_tiles_max,
                static_cast<const uint8_t*>(c.x), c.x_s, static_cast<const uint8_t*>(c.W1),
                static_cast<const uint8_t*>(c.W3), c.W1_s, c.W3_s, static_cast<uint8_t*>(c.h), c.h_s, nullptr};
        k_ffn_tiled<DT, true, false><<<dim3(c.n_tiles_max, c.I / 128), block, 0, s>>>(g);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (c.stages & 2) {
        TArgs d{c.offsets, c.masked_m, c.tile_off, c.n_local, c.I, c.H, c.n_tiles_max,
                static_cast<const uint8_t*>(c.h), c.h_s, static_cast<const uint8_t*>(c.W2), nullptr, c.W2_s,
                nullptr, static_cast<uint8_t*>(c.y), nullptr, c.signals};
        if (c.signals)
            k_ffn_tiled<DT, false, true><<<dim3(c.n_tiles_max, c.H / 128), block, 0, s>>>(d);
        else
            k_ffn_tiled<DT, false, false><<<dim3(c.n_tiles_max, c.H / 128), block, 0, s>>>(d);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_tiled(const FfnCall& c, hipStream_t s) {
    if (c.n_tiles_max <= 0) return hipSuccess;
    if (c.dtype == RDG_BF16) return launch_dt<RDG_BF16>(c, s);
    if (c.dtype == RDG_FP8_E4M3) return launch_dt<RDG_FP8_E4M3>(c, s);
    return hipErrorInvalidValue;
}

}  // namespace rdg
