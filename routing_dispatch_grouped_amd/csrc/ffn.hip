// Grouped expert FFN: gate/up GEMM with the SiLU-gated product fused into
// its epilogue, then the down GEMM (optionally signalling each finished row
// tile).
//
// What it computes (DeepEP deep-dive, EP section: each selected expert runs
// its FFN on the token; H100 deployment article, "DeepGEMM integration": a
// grouped GEMM over a contiguous layout for prefill and over a masked
// fixed-shape layout for decode; DeepGEMM single-batch-overlap pull request,
// section 3: the fp8 masked grouped GEMM with 1-D activation and 2-D weight
// block scales, and a release-ordered counter per block of rows written once
// the rows are stored; section 2: the counter is polled by the combine).
//
// Design for CDNA4.  A workgroup is four 64-wide waves and owns one row tile
// (BT rows of one expert) times 128 output columns; wave w owns columns
// [32w, 32w + 32) as two 16-row MFMA tiles, so the weight rows it streams
// are read exactly once per row tile, straight from HBM into registers (no
// LDS: nothing else in the workgroup reuses them).  Weights arrive packed
// (pack.hip): each MFMA operand tile is one contiguous KiB in lane order, so
// every weight load instruction is a fully contiguous KiB, which HBM serves
// far better than 64-byte pieces of 16 different rows.  The token rows are
// the MFMA's second operand, BT/16 column tiles, shared by the four waves
// through L2, loaded from their natural K-major rows.  MFMA: 16x16x4 f32, 16x16x32 bf16, and
// 16x16x128 fp8 e4m3 (one instruction per 128-long scale block, then the
// partial sum is promoted into the fp32 accumulator with its activation and
// weight block scales).  The row-tile -> expert mapping comes from the prefix
// table the dispatch built, so no host sync is needed for dynamic shapes.
#include <type_traits>

#include "rdg_internal.h"

namespace rdg {
namespace {

template <int DT>
struct Mma;

// Per type: the MFMA step KS (reduction elements), element size, unroll U,
// the packed weight tile size BLK (see pack.hip), and operand loads from a
// natural K-major row (tokens) or from a packed weight tile.  Weight tiles
// are read once per call, so they are loaded non-temporally (streamed past
// the caches), which leaves L2 to the token rows that every column block
// re-reads; measured on the decode layer this lifts the weight stream from
// ~5.8 to ~6.4 TB/s.
template <>
struct Mma<RDG_F32> {
    using op_t = float;
    static constexpr int KS = 4, ESZ = 4, U = 8, BLK = 256;
    __device__ static op_t load_tile(const uint8_t* tile, int lane) {
        return __builtin_nontemporal_load(reinterpret_cast<const float*>(tile) + lane);
    }
    __device__ static op_t load_tile_cached(const uint8_t* tile, int lane) {
        return reinterpret_cast<const float*>(tile)[lane];
    }
    __device__ static op_t load(const uint8_t* row, int k0, int lane) {
        return reinterpret_cast<const float*>(row)[k0 + (lane >> 4)];
    }
    __device__ static op_t zero() { return 0.0f; }
    __device__ static f32x4_t mma(f32x4_t c, op_t a, op_t b) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

template <>
struct Mma<RDG_BF16> {
    using op_t = bf16x8_t;
    static constexpr int KS = 32, ESZ = 2, U = 4, BLK = 1024;
    __device__ static op_t load_tile(const uint8_t* tile, int lane) {
        return __builtin_nontemporal_load(reinterpret_cast<const bf16x8_t*>(tile + lane * 16));
    }
    __device__ static op_t load_tile_cached(const uint8_t* tile, int lane) {
        return *reinterpret_cast<const bf16x8_t*>(tile + lane * 16);
    }
    __device__ static op_t load(const uint8_t* row, int k0, int lane) {
        return *reinterpret_cast<const bf16x8_t*>(row + (size_t)(k0 + (lane >> 4) * 8) * 2);
    }
    __device__ static op_t zero() { return op_t{}; }
    __device__ static f32x4_t mma(f32x4_t c, op_t a, op_t b) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <>
struct Mma<RDG_FP8_E4M3> {
    using op_t = i32x8_t;
    static constexpr int KS = 128, ESZ = 1, U = 1, BLK = 2048;
    __device__ static op_t load_tile(const uint8_t* tile, int lane) {
        typedef int i32x4_t __attribute__((ext_vector_type(4)));
        const i32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const i32x4_t*>(tile + lane * 16));
        const i32x4_t b = __builtin_nontemporal_load(reinterpret_cast<const i32x4_t*>(tile + 1024 + lane * 16));
        op_t r;
        r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
        r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
        return r;
    }
    __device__ static op_t load_tile_cached(const uint8_t* tile, int lane) {
        const uint4 a = *reinterpret_cast<const uint4*>(tile + lane * 16);
        const uint4 b = *reinterpret_cast<const uint4*>(tile + 1024 + lane * 16);
        op_t r;
        r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
        r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
        return r;
    }
    __device__ static op_t load(const uint8_t* row, int k0, int lane) {
        const uint4* p = reinterpret_cast<const uint4*>(row + k0 + (lane >> 4) * 32);
        uint4 a = p[0], b = p[1];
        op_t r;
        r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
        r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
        return r;
    }
    __device__ static op_t zero() { return op_t{}; }
    // e4m3 x e4m3 (format code 0 for both), unit block exponents (127 = 2^0)
    __device__ static f32x4_t mma(f32x4_t c, op_t a, op_t b) {
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
    }
};

struct KArgs {
    const int32_t* offsets;
    const int32_t* masked_m;
    const int32_t* tile_off;
    int n_local, Kdim, Nout;
    const uint8_t* X;     // [rows, Kdim] layout rows, or tokens read through gather
    const float* Xs;      // fp8: [rows, Kdim/128]
    const int32_t* gather;  // NULL, or the layout's row_src: row r's operand is token gather[r] / gather_k
    int gather_k;
    const uint8_t* Wa;    // [n_local, Nout, Kdim]  (W1, or W2)
    const uint8_t* Wb;    // [n_local, Nout, Kdim]  (W3 when gated)
    const float* Was;     // fp8: [n_local, Nout/128, Kdim/128]
    const float* Wbs;
    uint8_t* O;           // [rows, Nout]  (h, or y)
    float* Os;            // fp8 h scales [rows, Nout/128]
    int32_t* signals;     // [rows / BT]
    int pow2;             // fp8: h re-quantised with power-of-two scales
};

template <int DT, int BT, bool GATED, bool SIGNAL>
__global__ __launch_bounds__(256) void k_ffn(KArgs a) {
    using M = Mma<DT>;
    using op_t = typename M::op_t;
    constexpr int NCT = BT / 16;
    constexpr int KS = M::KS, U = M::U, ESZ = M::ESZ;
    static_assert(128 % (KS * U) == 0, "the K loop steps by KS*U over a multiple of 128");
    // output storage: fp32 layer -> fp32; bf16 -> bf16; fp8: h in e4m3, y in bf16
    constexpr int OUT_KIND = DT == RDG_F32 ? 0 : (DT == RDG_FP8_E4M3 && GATED) ? 2 : 1;

    // signalled: tile-major order (grid x = column block), so that row tiles
    // complete in layout order for the polling consumer
    const int tile = SIGNAL ? blockIdx.y : blockIdx.x;
    const int n_tiles = a.tile_off[a.n_local];
    if (tile >= n_tiles) return;  // workgroup-uniform
    int lo = 0, hi = a.n_local;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.tile_off[mid] <= tile) lo = mid;
        else hi = mid;
    }
    const int e = lo;
    const int row0 = a.offsets[e] + (tile - a.tile_off[e]) * BT;
    const int row_end = a.offsets[e] + a.masked_m[e];
    const int f0 = (SIGNAL ? blockIdx.x : blockIdx.y) * 128;
    if (f0 >= a.Nout) return;  // signalled grids are padded to a multiple of 8 column blocks (uniform)
    const int wv = threadIdx.x / kWave, lane = lane_id();
    const int fw = f0 + wv * 32;
    const size_t wstride = (size_t)a.Kdim * ESZ;

    // packed weights: the tiles of one 16-row group are contiguous along K
    const int nks = a.Kdim / KS;
    const uint8_t* arow[2];
    const uint8_t* brow[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const size_t grp = (size_t)e * (a.Nout / 16) + (fw + rt * 16) / 16;
        arow[rt] = a.Wa + grp * nks * M::BLK;
        brow[rt] = GATED ? a.Wb + grp * nks * M::BLK : nullptr;
    }
    const uint8_t* xrow[NCT];
    int xr[NCT];  // the operand row (layout row, or gathered token) of each token tile
    bool xv[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        const int r = row0 + ct * 16 + (lane & 15);
        xv[ct] = r < row_end;
        xr[ct] = token_row(a.gather, a.gather_k, xv[ct] ? r : row0);
        xrow[ct] = a.X + (size_t)xr[ct] * wstride;
    }

    f32x4_t accA[2][NCT], accB[2][NCT];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            accA[rt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            accB[rt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }

    const int nkb = a.Kdim / 128;
    const float* was = nullptr;
    const float* wbs = nullptr;
    if (DT == RDG_FP8_E4M3) {
        was = a.Was + ((size_t)e * (a.Nout / 128) + f0 / 128) * nkb;
        if (GATED) wbs = a.Wbs + ((size_t)e * (a.Nout / 128) + f0 / 128) * nkb;
    }

    for (int k0 = 0; k0 < a.Kdim; k0 += KS * U) {
        op_t ra[U][2], rb[U][2], rx[U][NCT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const size_t t_off = (size_t)(k0 / KS + u) * M::BLK;
                ra[u][rt] = M::load_tile(arow[rt] + t_off, lane);
                if (GATED) rb[u][rt] = M::load_tile(brow[rt] + t_off, lane);
            }
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) rx[u][ct] = xv[ct] ? M::load(xrow[ct], k0 + u * KS, lane) : M::zero();
        }
        if (DT != RDG_FP8_E4M3) {
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        accA[rt][ct] = M::mma(accA[rt][ct], ra[u][rt], rx[u][ct]);
                        if (GATED) accB[rt][ct] = M::mma(accB[rt][ct], rb[u][rt], rx[u][ct]);
                    }
        } else {
            const int kb = k0 / 128;
            const float sa_w = was[kb];
            const float sb_w = GATED ? wbs[kb] : 0.0f;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const float sx = xv[ct] ? a.Xs[(size_t)xr[ct] * nkb + kb] : 0.0f;
                const float fa = sx * sa_w, fb = sx * sb_w;
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
                    const f32x4_t pa = M::mma(z, ra[0][rt], rx[0][ct]);
                    accA[rt][ct] += pa * fa;
                    if (GATED) {
                        const f32x4_t pb = M::mma(z, rb[0][rt], rx[0][ct]);
                        accB[rt][ct] += pb * fb;
                    }
                }
            }
        }
    }

    // ---------------------------------------------------------------- epilogue
    // accumulator layout of a 16x16 MFMA tile: lane l holds column (token)
    // l % 16 and rows (features) 4*(l/16) .. 4*(l/16)+3
    const int fl = fw + (lane >> 4) * 4;  // + rt*16 + r
    float val[2][NCT][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float g = accA[rt][ct][r];
                if (GATED) {
                    const float u = accB[rt][ct][r];
                    val[rt][ct][r] = g / (1.0f + __expf(-g)) * u;
                } else {
                    val[rt][ct][r] = g;
                }
            }

    if (OUT_KIND == 2) {
        __shared__ float red[4][BT];
        float amax[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            float m = 0.0f;
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(val[rt][ct][r]));
            m = fmaxf(m, __shfl_xor(m, 16));
            m = fmaxf(m, __shfl_xor(m, 32));
            if (lane < 16) red[wv][ct * 16 + lane] = m;
        }
        __syncthreads();
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const int c = ct * 16 + (lane & 15);
            amax[ct] = fmaxf(fmaxf(red[0][c], red[1][c]), fmaxf(red[2][c], red[3][c]));
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const int row = row0 + ct * 16 + (lane & 15);
            if (row >= row_end) continue;
            const float s = fp8_block_scale(amax[ct], a.pow2 != 0);
            const float inv = 1.0f / s;
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                uint32_t q = 0;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float t = fminf(fmaxf(val[rt][ct][r] * inv, -448.0f), 448.0f);
                    q |= f32_to_e4m3(t) << (8 * r);
                }
                *reinterpret_cast<uint32_t*>(a.O + (size_t)row * a.Nout + fl + rt * 16) = q;
            }
            if (wv == 0 && lane < 16) a.Os[(size_t)row * (a.Nout / 128) + f0 / 128] = s;
        }
    } else {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const int row = row0 + ct * 16 + (lane & 15);
            if (row >= row_end) continue;
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const size_t idx = (size_t)row * a.Nout + fl + rt * 16;
                if (OUT_KIND == 0) {
                    store_out16<SIGNAL>(a.O + idx * 4,
                                        make_float4(val[rt][ct][0], val[rt][ct][1], val[rt][ct][2], val[rt][ct][3]));
                } else {
                    store_out8<SIGNAL>(a.O + idx * 2,
                                       (uint64_t)(f32_to_bf16(val[rt][ct][0]) | (f32_to_bf16(val[rt][ct][1]) << 16)) |
                                           ((uint64_t)(f32_to_bf16(val[rt][ct][2]) |
                                                       (f32_to_bf16(val[rt][ct][3]) << 16))
                                            << 32));
                }
            }
        }
    }

    if (SIGNAL) signal_done(a.signals + row0 / BT, 128);
}


// ---------------------------------------------------------------------------
// Skinny variant for weight-streaming row tiles (decode: a few tokens per
// expert; a dense expert of up to a few hundred tokens).  Each workgroup owns
// 16*FPW weight rows of one expert and NR consecutive 16-row tiles of its
// tokens (BT = 16*NR rows); its four waves split the reduction dimension by
// 128-wide blocks, interleaved (wave w takes blocks w, w+4, ...), so that
// the workgroup's loads run through each weight stream in order, and the
// partial sums are added in LDS in wave order (so the result does not depend
// on timing).  The grid is tile-major: the column blocks of one row tile are
// consecutive workgroups, which stream neighbouring weight panels of one
// expert and share its token rows in L2 (and signalled row tiles complete in
// layout order).  Many short workgroups instead of few long ones keep the
// last round of the grid from idling most of the GPU.  An expert's weights
// are read once per row tile: streamed past the caches when its rows fit one
// tile; when they span several (NR > 1, or a busy expert of a decode batch),
// the loads stay cacheable, and the sibling tiles -- consecutive rows of the
// grid, so on the same XCD at about the same time -- find them in L2.  Used for every
// type except the fp8 gate/up stage, whose 1x128 re-quantisation of h needs
// 128 columns in one workgroup.
template <int DT, bool GATED, bool SIGNAL, int FPW, int NR>
__global__ __launch_bounds__(256) void k_ffn_skinny(KArgs a) {
    using M = Mma<DT>;
    using op_t = typename M::op_t;
    constexpr int KS = M::KS, ESZ = M::ESZ;
    // fewer K steps in flight as the token operand grows (register budget)
    constexpr int U = DT == RDG_FP8_E4M3 ? 1 : NR <= 2 ? M::U : M::U / 2 > 0 ? M::U / 2 : 1;
    constexpr int G = GATED ? 2 : 1;
    constexpr int BT = 16 * NR;
    constexpr int OUT_KIND = DT == RDG_F32 ? 0 : 1;
    // each wave walks whole 128-element blocks of the reduction dimension in
    // steps of KS*U, so a step must never run past the end of its block
    static_assert(DT == RDG_FP8_E4M3 || 128 % (KS * U) == 0, "KS * U must divide 128");
    __shared__ f32x4_t part[4][FPW * G * NR][kWave];

    // tile-major order (grid x = column block)
    const int tile = blockIdx.y;
    const int n_tiles = a.tile_off[a.n_local];
    if (tile >= n_tiles) return;  // workgroup-uniform
    int lo = 0, hi = a.n_local;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.tile_off[mid] <= tile) lo = mid;
        else hi = mid;
    }
    const int e = lo;
    const int row0 = a.offsets[e] + (tile - a.tile_off[e]) * BT;
    const int row_end = a.offsets[e] + a.masked_m[e];
    const int f0 = blockIdx.x * (16 * FPW);
    if (f0 >= a.Nout) return;  // signalled grids are padded to a multiple of 8 column blocks (uniform)
    const int wv = threadIdx.x / kWave, lane = lane_id();
    const size_t wstride = (size_t)a.Kdim * ESZ;

    const int nks = a.Kdim / KS;
    const uint8_t* arow[FPW];
    const uint8_t* brow[FPW];
#pragma unroll
    for (int rt = 0; rt < FPW; ++rt) {
        const size_t grp = (size_t)e * (a.Nout / 16) + (f0 + rt * 16) / 16;
        arow[rt] = a.Wa + grp * nks * M::BLK;
        brow[rt] = GATED ? a.Wb + grp * nks * M::BLK : nullptr;
    }
    int xr[NR];
    bool xv[NR];
    const uint8_t* xrow[NR];
#pragma unroll
    for (int nr = 0; nr < NR; ++nr) {
        const int r = row0 + nr * 16 + (lane & 15);
        xv[nr] = r < row_end;
        xr[nr] = token_row(a.gather, a.gather_k, xv[nr] ? r : row0);  // the operand row
        xrow[nr] = a.X + (size_t)xr[nr] * wstride;
    }
    // weights of an expert whose rows span several row tiles are read by
    // each of them: then cacheable loads, so that the sibling tiles (run
    // side by side on the same XCD) find them in L2; otherwise streamed
    const bool shared_panel = NR > 1 || a.masked_m[e] > BT;

    f32x4_t accA[FPW][NR], accB[FPW][NR];
#pragma unroll
    for (int rt = 0; rt < FPW; ++rt)
#pragma unroll
        for (int nr = 0; nr < NR; ++nr) {
            accA[rt][nr] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            accB[rt][nr] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    const int nkb = a.Kdim / 128;
    const float* was = nullptr;
    const float* wbs = nullptr;
    if (DT == RDG_FP8_E4M3) {
        was = a.Was + ((size_t)e * (a.Nout / 128) + f0 / 128) * nkb;
        if (GATED) wbs = a.Wbs + ((size_t)e * (a.Nout / 128) + f0 / 128) * nkb;
    }
    auto kloop = [&](auto cached) {
        auto wload = [&](const uint8_t* t) {
            if constexpr (decltype(cached)::value) return M::load_tile_cached(t, lane);
            else return M::load_tile(t, lane);
        };
        for (int kb = wv; kb < nkb; kb += 4) {
            if (DT != RDG_FP8_E4M3) {
#pragma unroll
                for (int k0 = kb * 128; k0 < kb * 128 + 128; k0 += KS * U) {
                    op_t ra[U][FPW], rb[U][FPW], rx[U][NR];
#pragma unroll
                    for (int u = 0; u < U; ++u) {
#pragma unroll
                        for (int rt = 0; rt < FPW; ++rt) {
                            const size_t t_off = (size_t)(k0 / KS + u) * M::BLK;
                            ra[u][rt] = wload(arow[rt] + t_off);
                            if (GATED) rb[u][rt] = wload(brow[rt] + t_off);
                        }
#pragma unroll
                        for (int nr = 0; nr < NR; ++nr) rx[u][nr] = xv[nr] ? M::load(xrow[nr], k0 + u * KS, lane) : M::zero();
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u)
#pragma unroll
                        for (int rt = 0; rt < FPW; ++rt)
#pragma unroll
                            for (int nr = 0; nr < NR; ++nr) {
                                accA[rt][nr] = M::mma(accA[rt][nr], ra[u][rt], rx[u][nr]);
                                if (GATED) accB[rt][nr] = M::mma(accB[rt][nr], rb[u][rt], rx[u][nr]);
                            }
                }
            } else {
                op_t ra[FPW], rb[FPW];
#pragma unroll
                for (int rt = 0; rt < FPW; ++rt) {
                    ra[rt] = wload(arow[rt] + (size_t)kb * M::BLK);
                    if (GATED) rb[rt] = wload(brow[rt] + (size_t)kb * M::BLK);
                }
                const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int nr = 0; nr < NR; ++nr) {
                    const op_t rx = xv[nr] ? M::load(xrow[nr], kb * 128, lane) : M::zero();
                    const float sx = xv[nr] ? a.Xs[(size_t)xr[nr] * nkb + kb] : 0.0f;
                    const float fa = sx * was[kb], fb = GATED ? sx * wbs[kb] : 0.0f;
#pragma unroll
                    for (int rt = 0; rt < FPW; ++rt) {
                        accA[rt][nr] += M::mma(z, ra[rt], rx) * fa;
                        if (GATED) accB[rt][nr] += M::mma(z, rb[rt], rx) * fb;
                    }
                }
            }
        }
    };
    if (shared_panel) kloop(std::true_type{});
    else kloop(std::false_type{});
    // reduce the four K ranges in wave order
#pragma unroll
    for (int rt = 0; rt < FPW; ++rt)
#pragma unroll
        for (int nr = 0; nr < NR; ++nr) {
            part[wv][(rt * NR + nr) * G][lane] = accA[rt][nr];
            if (GATED) part[wv][(rt * NR + nr) * G + 1][lane] = accB[rt][nr];
        }
    __syncthreads();
    // wave w finishes row tiles nr = w, w+4, ... (every wave when NR >= 4)
    const int fl = (lane >> 4) * 4;
#pragma unroll
    for (int nr = 0; nr < NR; ++nr) {
        if (nr % 4 != wv) continue;
        const int row = row0 + nr * 16 + (lane & 15);
#pragma unroll
        for (int rt = 0; rt < FPW; ++rt) {
            const int slot = (rt * NR + nr) * G;
            f32x4_t g = part[0][slot][lane];
            f32x4_t u = GATED ? part[0][slot + 1][lane] : g;
#pragma unroll
            for (int w = 1; w < 4; ++w) {
                g += part[w][slot][lane];
                if (GATED) u += part[w][slot + 1][lane];
            }
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = GATED ? g[r] / (1.0f + __expf(-g[r])) * u[r] : g[r];
            if (row < row_end) {
                const size_t idx = (size_t)row * a.Nout + f0 + fl + rt * 16;
                if (OUT_KIND == 0) {
                    store_out16<SIGNAL>(a.O + idx * 4, make_float4(v[0], v[1], v[2], v[3]));
                } else {
                    store_out8<SIGNAL>(a.O + idx * 2, (uint64_t)(f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16)) |
                                                          ((uint64_t)(f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16))
                                                           << 32));
                }
            }
        }
    }
    if (SIGNAL) signal_done(a.signals + row0 / BT, 16 * FPW);
}


KArgs gate_up_args(const FfnCall& c) {
    KArgs g{};
    g.offsets = c.offsets;
    g.masked_m = c.masked_m;
    g.tile_off = c.tile_off;
    g.n_local = c.n_local;
    g.Kdim = c.H;  // gate/up: Kdim = H, Nout = I
    g.Nout = c.I;
    g.X = static_cast<const uint8_t*>(c.x);
    g.Xs = c.x_s;
    g.gather = c.gather;
    g.gather_k = c.gather_k;
    g.Wa = static_cast<const uint8_t*>(c.W1);
    g.Wb = static_cast<const uint8_t*>(c.W3);
    g.Was = c.W1_s;
    g.Wbs = c.W3_s;
    g.O = static_cast<uint8_t*>(c.h);
    g.Os = c.h_s;
    g.signals = nullptr;
    g.pow2 = c.pow2;
    return g;
}

KArgs down_args(const FfnCall& c) {
    KArgs d{};
    d.offsets = c.offsets;
    d.masked_m = c.masked_m;
    d.tile_off = c.tile_off;
    d.n_local = c.n_local;
    d.Kdim = c.I;  // down: Kdim = I, Nout = H, input h
    d.Nout = c.H;
    d.X = static_cast<const uint8_t*>(c.h);  // h is in layout order
    d.Xs = c.h_s;
    d.gather = nullptr;
    d.Wa = static_cast<const uint8_t*>(c.W2);
    d.Wb = nullptr;
    d.Was = c.W2_s;
    d.Wbs = nullptr;
    d.O = static_cast<uint8_t*>(c.y);
    d.Os = nullptr;
    d.signals = c.signals;
    return d;
}

// Row tiles of BT = 16*NR rows through the skinny kernel (the fp8 gate/up
// stage through k_ffn, see above).  Gate/up: 32 weight rows per matrix and
// workgroup for single 16-row tiles, 16 for NR > 1 (twice the workgroups, so
// that a dense expert of a few row groups still fills the GPU); down: 32.
template <int DT, int NR>
hipError_t launch_skinny(const FfnCall& c, hipStream_t s) {
    constexpr int BT = 16 * NR;
    dim3 block(256);
    if (c.stages & 1) {
        const KArgs g = gate_up_args(c);
        if constexpr (DT == RDG_FP8_E4M3) {
            k_ffn<DT, BT, true, false><<<dim3(c.n_tiles_max, c.I / 128), block, 0, s>>>(g);
        } else if constexpr (NR == 1) {
            k_ffn_skinny<DT, true, false, 2, NR><<<dim3(c.I / 32, c.n_tiles_max), block, 0, s>>>(g);
        } else {
            k_ffn_skinny<DT, true, false, 1, NR><<<dim3(c.I / 16, c.n_tiles_max), block, 0, s>>>(g);
        }
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (c.stages & 2) {
        const KArgs d = down_args(c);
        if (c.signals)
            k_ffn_skinny<DT, false, true, 2, NR><<<dim3(round8(c.H / 32), c.n_tiles_max), block, 0, s>>>(d);
        else
            k_ffn_skinny<DT, false, false, 2, NR><<<dim3(c.H / 32, c.n_tiles_max), block, 0, s>>>(d);
    }
    return hipGetLastError();
}

// Row tiles of 32 or 64 rows through k_ffn (register-resident token tiles).
template <int DT, int BT>
hipError_t launch_bt(const FfnCall& c, hipStream_t s) {
    dim3 block(256);
    if (c.stages & 1) {
        k_ffn<DT, BT, true, false><<<dim3(c.n_tiles_max, c.I / 128), block, 0, s>>>(gate_up_args(c));
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (c.stages & 2) {
        const KArgs d = down_args(c);
        if (c.signals)
            k_ffn<DT, BT, false, true><<<dim3(round8(c.H / 128), c.n_tiles_max), block, 0, s>>>(d);
        else
            k_ffn<DT, BT, false, false><<<dim3(c.n_tiles_max, c.H / 128), block, 0, s>>>(d);
    }
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const FfnCall& c, hipStream_t s) {
    if (c.skinny_nr > 0) {
        if (c.bt != 16 * c.skinny_nr) return hipErrorInvalidValue;
        switch (c.skinny_nr) {
            case 1: return launch_skinny<DT, 1>(c, s);
            case 2: return launch_skinny<DT, 2>(c, s);
            case 4: return launch_skinny<DT, 4>(c, s);
            default: return hipErrorInvalidValue;
        }
    }
    switch (c.bt) {
        case 32: return launch_bt<DT, 32>(c, s);
        case 64: return launch_bt<DT, 64>(c, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_ffn(const FfnCall& c, hipStream_t s) {
    if (c.n_tiles_max <= 0) return hipSuccess;
    if (c.bt == 128) return launch_ffn_tiled(c, s);
    switch (c.dtype) {
        case RDG_F32: return launch_dt<RDG_F32>(c, s);
        case RDG_BF16: return launch_dt<RDG_BF16>(c, s);
        case RDG_FP8_E4M3: return launch_dt<RDG_FP8_E4M3>(c, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace rdg
