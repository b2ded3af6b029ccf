// Grouped expert FFN for row tiles of 128 rows (prefill, rank shares, the
// shared expert of a prefill batch): the same two stages as ffn.hip -- gate/up
// GEMM with the SiLU-gated product (and fp8 re-quantisation of h) in its
// epilogue, then the down GEMM, optionally signalling each finished row tile
// -- with the operand reuse and the load pipeline a 128-row tile needs to
// approach the MFMA rate.
//
// What it computes: see ffn.hip (DeepEP deep-dive, EP section; H100
// deployment article, "DeepGEMM integration"; DeepGEMM single-batch-overlap
// pull request, sections 2-3).
//
// Design for CDNA4.  A workgroup is 8 waves (two per SIMD) and owns a tile of
// 128 layout rows of one expert and a panel of 256 weight rows: gated, rows
// [f0, f0+128) of W1 (waves 0-3) and of W3 (waves 4-7); down, rows [f0,
// f0+256) of W2.  Wave w owns 32 weight rows (two 16-row MFMA tiles) against
// all 128 token rows (eight 16-row MFMA tiles), so each token operand read
// from LDS feeds two MFMAs and each weight operand eight.
//
// The reduction dimension is walked in chunks of CB bytes per row.  The
// token tile is shared by the eight waves, so its chunks go through a
// two-slot LDS ring filled by direct global->LDS loads; the slot of 16-byte
// piece c of row r is c ^ (r % 16) (chosen through each lane's source
// address), which makes the MFMA-layout LDS reads conflict-free.  Weight
// operand tiles are private to a wave and arrive packed (pack.hip: one
// contiguous KiB per load instruction) straight into one of two register
// sets; a weight panel is re-read by every row tile of its expert, mostly
// from L2.  While chunk k is multiplied, chunk k+1's token rows (into the
// other ring slot) and weights (into the other register set) are in flight;
// the loop is unrolled by two so that slots and register sets are named at
// compile time (no register copies that would wait for a load in flight, and
// the compiler can tell the slots apart), with one wait and one barrier per
// chunk.
// fp8 tiles also stage each chunk's activation scales (two 1x128 blocks per
// row) through the ring; every 128-long block's MFMA partial is promoted into
// the fp32 accumulator with its activation and weight scales.
//
// Workgroups are renumbered so that the token tiles sharing one weight panel
// run back to back on the same XCD and re-read the panel from its L2; the
// signalled down stage instead runs tile-major, so that row tiles complete in
// layout order while a combine polls them.
#include "rdg_internal.h"

namespace rdg {
namespace {

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;

constexpr int NW = 8;                 // waves per workgroup
constexpr int TB = 128;               // rows per tile
constexpr int NCT = TB / 16;          // 16-row token tiles per wave
constexpr int NRT = 2;                // 16-row weight tiles per wave
constexpr int PANEL = NW * NRT * 16;  // weight rows per workgroup

template <int DT>
struct TOp;

// Per type: the chunk CB (bytes of each row per chunk: two chunks of token
// rows and of weights in flight must fit the register budget of two waves per
// SIMD), the MFMA step KS (reduction elements), element size, the packed
// weight tile size BLK (see pack.hip), MFMA steps per chunk, and the weight
// load instructions per chunk.
template <>
struct TOp<RDG_BF16> {
    using op_t = bf16x8_t;
    static constexpr int CB = 512;
    static constexpr int KS = 32, ESZ = 2, BLK = 1024, STEPS = CB / (KS * ESZ);
    static constexpr int WLOADS = NRT * STEPS;                                   // load instructions
    __device__ static void load_w(op_t (&w)[STEPS][NRT], const uint8_t* const (&wt)[NRT], int t0, int lane) {
#pragma unroll
        for (int s = 0; s < STEPS; ++s)
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt)
                w[s][rt] = *reinterpret_cast<const bf16x8_t*>(wt[rt] + (size_t)(t0 + s) * BLK + lane * 16);
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
    static constexpr int CB = 256;
    static constexpr int KS = 128, ESZ = 1, BLK = 2048, STEPS = CB / KS;  // steps = 1x128 scale blocks
    static constexpr int WLOADS = NRT * STEPS * 2;
    __device__ static void load_w(op_t (&w)[STEPS][NRT], const uint8_t* const (&wt)[NRT], int t0, int lane) {
#pragma unroll
        for (int s = 0; s < STEPS; ++s)
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                const uint8_t* tile = wt[rt] + (size_t)(t0 + s) * BLK;
                const i32x4_t a = *reinterpret_cast<const i32x4_t*>(tile + lane * 16);
                const i32x4_t b = *reinterpret_cast<const i32x4_t*>(tile + 1024 + lane * 16);
                op_t r;
                r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
                r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
                w[s][rt] = r;
            }
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

// s_waitcnt immediate (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8) that waits until at most N vector-memory instructions
// are outstanding and leaves the other counters alone.
template <int N>
constexpr int vmcnt_imm() {
    static_assert(N >= 0 && N < 64, "vmcnt is six bits");
    return (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
}

// Workgroup barrier for the ring.  __syncthreads() (and even an LDS-only
// fence) makes the compiler drain every load in flight -- the next chunk's
// included -- at each barrier.  Here each wave has already waited for its
// own direct loads (counted vmcnt) and for its own LDS reads (their values
// feed MFMAs issued before the barrier), so the bare barrier suffices; the
// scheduling barriers keep the compiler from moving memory operations across.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS reads are done
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

struct Ring {
    uint8_t* x;  // 128 * CB bytes: the token chunk
    float* s;    // fp8: [128 rows][SPB blocks] activation scales of the chunk
};

// Request chunk kc of the tile's token rows: 16 * CB / 1024 direct KiB loads per wave
// (rows past the tile's valid rows re-read the last valid row: in bounds,
// never stored); fp8: one load of 32 activation scales per wave.
template <int DT>
__device__ __forceinline__ void stage_chunk(const TArgs& a, size_t xstride, int nkb, int row0, int nvalid, int kc,
                                            const Ring& ring, int wv, int lane) {
    constexpr int CB = TOp<DT>::CB, XLOADS = TB * CB / 1024 / NW, SPB = CB / 128;
    static_assert(SPB * 16 <= 64 && 1024 % CB == 0, "chunk shape");
    constexpr int PPR = CB / 16;          // 16-byte pieces per row
#pragma unroll
    for (int i = 0; i < XLOADS; ++i) {
        const int q = wv * XLOADS + i;             // LDS bytes [q*1024, q*1024+1024)
        const int r = q * (1024 / CB) + lane / PPR;  // tile row of this lane's 16 bytes
        const int slot = lane % PPR;
        const int c = slot ^ (r & 15);             // source piece for this slot
        const int rr = r < nvalid ? r : nvalid - 1;
        const uint8_t* src = a.X + (size_t)(row0 + rr) * xstride + (size_t)kc * CB + c * 16;
        __builtin_amdgcn_global_load_lds((gbl_ptr_t)src, (lds_ptr_t)(ring.x + q * 1024), 16, 0, 0);
    }
    if (DT == RDG_FP8_E4M3) {
        // lanes 0..16*SPB-1 of wave w: row 16w + l/SPB, scale block SPB*kc + l%SPB
        const int l = lane % (16 * SPB);
        const int r = wv * 16 + l / SPB;
        const int rr = r < nvalid ? r : nvalid - 1;
        const float* src = a.Xs + (size_t)(row0 + rr) * nkb + SPB * kc + l % SPB;
        if (lane < 16 * SPB)
            __builtin_amdgcn_global_load_lds((gbl_ptr_t)src, (lds_ptr_t)(ring.s + wv * 16 * SPB), 4, 0, 0);
    }
}

template <int DT, bool GATED, bool SIGNAL>
__global__ __launch_bounds__(NW * 64, 1) void k_ffn_tiled(TArgs a) {
    using O = TOp<DT>;
    using op_t = typename O::op_t;
    constexpr int S = O::STEPS;
    constexpr bool FP8 = DT == RDG_FP8_E4M3;
    constexpr int CB = O::CB, CHUNK_LDS = TB * CB, SPB = CB / 128;
    __shared__ __attribute__((aligned(16))) uint8_t lx0[CHUNK_LDS];
    __shared__ __attribute__((aligned(16))) uint8_t lx1[CHUNK_LDS];
    __shared__ __attribute__((aligned(16))) float ls0[FP8 ? TB * SPB : 4];
    __shared__ __attribute__((aligned(16))) float ls1[FP8 ? TB * SPB : 4];
    const Ring ring[2] = {{lx0, ls0}, {lx1, ls1}};

    int fb, tile;
    if (SIGNAL) {
        // tile-major in dispatch order (grid x = column panel, padded to a
        // multiple of 8): row tiles complete in layout order for the polling
        // consumer, and XCD x runs the panels fb = x (mod 8) of every tile and
        // keeps them in its L2
        fb = blockIdx.x;
        tile = blockIdx.y;
        if (fb * PANEL >= a.Nout) return;  // padding workgroup (uniform)
    } else {
        // XCD-aware renumbering: hardware block b runs on XCD b % 8, which
        // gets ceil((total - x) / 8) blocks; give XCD x the contiguous logical
        // range starting at x*(total/8) + min(x, total%8) (a bijection for any
        // total), so consecutive row tiles of one weight panel share an L2
        const int gx = a.n_tiles_max, total = gx * gridDim.y;
        const int b = blockIdx.y * gx + blockIdx.x;
        const int xcd = b % 8, q8 = total / 8, r8 = total % 8;
        const int logical = xcd * q8 + (xcd < r8 ? xcd : r8) + b / 8;
        fb = logical / gx;
        tile = logical % gx;
    }

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
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
    const int lane = lane_id();
    // gated: 128 output features per workgroup, wave w: matrix w/4, features
    // [f0 + 32(w%4), +32); down: 256 output columns, wave w: [f0 + 32w, +32)
    const int f0 = fb * (GATED ? PANEL / 2 : PANEL);
    const int mat = GATED ? wv / 4 : 0;
    const int fw = f0 + (GATED ? (wv % 4) : wv) * 32;
    const size_t xstride = (size_t)a.Kdim * O::ESZ;
    const int nks = a.Kdim / O::KS;
    const int nkb = a.Kdim / 128;
    const int nchunks = (int)(xstride / CB);

    const uint8_t* wt[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        const size_t grp = (size_t)e * (a.Nout / 16) + (fw + rt * 16) / 16;
        wt[rt] = (mat == 0 ? a.Wa : a.Wb) + grp * nks * O::BLK;
    }
    // fp8: this wave's weight block scales along K (its 32 rows lie in one 128-row block)
    const float* wsc = nullptr;
    if (FP8) wsc = (mat == 0 ? a.Was : a.Wbs) + ((size_t)e * (a.Nout / 128) + fw / 128) * nkb;

    f32x4_t acc[NRT][NCT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) acc[rt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // two weight register sets (chunk k's and k+1's), three ring slots
    op_t w[2][S][NRT];
    float sw[2][S];

    auto request_w = [&](int kc, op_t (&wr)[S][NRT], float (&swr)[S]) {
        O::load_w(wr, wt, kc * S, lane);
        if (FP8) {
#pragma unroll
            for (int s = 0; s < S; ++s) swr[s] = wsc[kc * S + s];
        }
    };
    // One chunk: items i = (step s, token tile ct) in order.  The token
    // operand of item i+2 is read from LDS while item i's MFMAs run (a
    // three-deep register ring), and fp8 promotes item i-1's block partials
    // behind item i's MFMAs; the scheduling barrier after each item keeps the
    // compiler from hoisting a chunk's worth of LDS reads (registers).
    auto compute = [&](const Ring& rg, const op_t (&wr)[S][NRT], const float (&swr)[S]) {
        constexpr int NI = S * NCT;
        op_t xb[3];
        float fb[4];
        f32x4_t p[2][NRT];
        const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
        auto fetch = [&](int i) {
            const int si = i / NCT, r = (i % NCT) * 16 + (lane & 15);
            xb[i % 3] = O::load_x(rg.x, r, si, lane >> 4);
            if (FP8) fb[i % 4] = rg.s[r * SPB + si] * swr[si];
        };
        fetch(0);
        fetch(1);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int si = i / NCT, ct = i % NCT;
            if (i + 2 < NI) fetch(i + 2);
            if (!FP8) {
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt) acc[rt][ct] = O::mma(acc[rt][ct], wr[si][rt], xb[i % 3]);
            } else {
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt) p[i % 2][rt] = O::mma(z, wr[si][rt], xb[i % 3]);
                if (i > 0) {
                    const int cp = (i - 1) % NCT;
#pragma unroll
                    for (int rt = 0; rt < NRT; ++rt) acc[rt][cp] += p[(i - 1) % 2][rt] * fb[(i - 1) % 4];
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (FP8) {
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) acc[rt][NCT - 1] += p[(NI - 1) % 2][rt] * fb[(NI - 1) % 4];
        }
    };

    // Chunk k+1's token rows and weights are requested once chunk k has
    // arrived, and are in flight while chunk k is multiplied.
    stage_chunk<DT>(a, xstride, nkb, row0, nvalid, 0, ring[0], wv, lane);
    request_w(0, w[0], sw[0]);
    for (int kc0 = 0; kc0 < nchunks; kc0 += 2) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int kc = kc0 + j;
            if (kc >= nchunks) break;
            // this wave's loads of chunk kc have landed, then every wave's; past
            // the barrier every wave is also done with chunk kc-1, whose ring
            // slot and weight set are refilled next
            __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
            lds_barrier();
            if (kc + 1 < nchunks) {
                stage_chunk<DT>(a, xstride, nkb, row0, nvalid, kc + 1, ring[(j + 1) % 2], wv, lane);
                request_w(kc + 1, w[(j + 1) % 2], sw[(j + 1) % 2]);
            }
            compute(ring[j], w[j], sw[j]);
        }
    }

    // ---------------------------------------------------------------- epilogue
    // 16x16 accumulator tile: lane l holds column (row of the layout) l % 16 and
    // rows (output features) 4*(l/16) .. +3
    const int fl = fw + (lane >> 4) * 4;
    __syncthreads();  // every wave is done with the ring
    if (GATED) {
        // the up-projection waves hand their accumulators to the gate waves,
        // weight tile rt through ring slot rt: [4 feature groups][8][64 lanes]
        if (mat == 1) {
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                f32x4_t* xch = reinterpret_cast<f32x4_t*>(rt == 0 ? lx0 : lx1);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) xch[((wv % 4) * NCT + ct) * kWave + lane] = acc[rt][ct];
            }
        }
        __syncthreads();
        if (mat == 0) {
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                const f32x4_t* xch = reinterpret_cast<const f32x4_t*>(rt == 0 ? lx0 : lx1);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    const f32x4_t u = xch[((wv % 4) * NCT + ct) * kWave + lane];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float g = acc[rt][ct][r];
                        acc[rt][ct][r] = g / (1.0f + __expf(-g)) * u[r];
                    }
                }
            }
        }
    }
    if (FP8 && GATED) {
        // h re-quantised with one fp32 scale per row and 128 features: amax
        // over the four gate waves' 32 features each
        __syncthreads();                              // the exchange area is read
        float* red = reinterpret_cast<float*>(lx0);  // [4 feature groups][128 rows]
        if (mat == 0) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                float m = 0.0f;
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(acc[rt][ct][r]));
                m = fmaxf(m, __shfl_xor(m, 16));
                m = fmaxf(m, __shfl_xor(m, 32));
                if (lane < 16) red[(wv % 4) * TB + ct * 16 + lane] = m;
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
                for (int rt = 0; rt < NRT; ++rt) {
                    uint32_t q = 0;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float tq = fminf(fmaxf(acc[rt][ct][r] * inv, -448.0f), 448.0f);
                        q |= f32_to_e4m3(tq) << (8 * r);
                    }
                    *reinterpret_cast<uint32_t*>(a.O + (size_t)row * a.Nout + fl + rt * 16) = q;
                }
                if (wv == 0 && lane < 16) a.Os[(size_t)row * (a.Nout / 128) + f0 / 128] = sc;
            }
        }
    } else if (mat == 0) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const int c = ct * 16 + (lane & 15);
            if (c >= nvalid) continue;
            const int row = row0 + c;
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                uint2 o;
                o.x = f32_to_bf16(acc[rt][ct][0]) | (f32_to_bf16(acc[rt][ct][1]) << 16);
                o.y = f32_to_bf16(acc[rt][ct][2]) | (f32_to_bf16(acc[rt][ct][3]) << 16);
                *reinterpret_cast<uint2*>(a.O + ((size_t)row * a.Nout + fl + rt * 16) * 2) = o;
            }
        }
    }
    if (SIGNAL) signal_done(a.signals + row0 / TB, PANEL);
}

template <int DT>
hipError_t launch_dt(const FfnCall& c, hipStream_t s) {
    dim3 block(NW * 64);
    if (c.stages & 1) {
        TArgs g{c.offsets, c.masked_m, c.tile_off, c.n_local, c.H, c.I, c.n_tiles_max,
                static_cast<const uint8_t*>(c.x), c.x_s, static_cast<const uint8_t*>(c.W1),
                static_cast<const uint8_t*>(c.W3), c.W1_s, c.W3_s, static_cast<uint8_t*>(c.h), c.h_s, nullptr};
        k_ffn_tiled<DT, true, false><<<dim3(c.n_tiles_max, c.I / (PANEL / 2)), block, 0, s>>>(g);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (c.stages & 2) {
        TArgs d{c.offsets, c.masked_m, c.tile_off, c.n_local, c.I, c.H, c.n_tiles_max,
                static_cast<const uint8_t*>(c.h), c.h_s, static_cast<const uint8_t*>(c.W2), nullptr, c.W2_s,
                nullptr, static_cast<uint8_t*>(c.y), nullptr, c.signals};
        if (c.signals)
            k_ffn_tiled<DT, false, true><<<dim3(round8(c.H / PANEL), c.n_tiles_max), block, 0, s>>>(d);
        else
            k_ffn_tiled<DT, false, false><<<dim3(c.n_tiles_max, c.H / PANEL), block, 0, s>>>(d);
    }
    return hipGetLastError();
}

}  // namespace

// bf16 / fp8 with I a multiple of 128 (the gate/up feature panel) and H a
// multiple of 256 (the down column panel); both reduction dimensions in whole
// chunks (512 bytes bf16, 256 bytes fp8).
bool tiled_supported(int dtype, int H, int I) {
    const int esz = dtype == RDG_BF16 ? 2 : dtype == RDG_FP8_E4M3 ? 1 : 0;
    const int cb = dtype == RDG_BF16 ? TOp<RDG_BF16>::CB : TOp<RDG_FP8_E4M3>::CB;
    return esz > 0 && I % (PANEL / 2) == 0 && H % PANEL == 0 && ((int64_t)H * esz) % cb == 0 &&
           ((int64_t)I * esz) % cb == 0;
}

hipError_t launch_ffn_tiled(const FfnCall& c, hipStream_t s) {
    if (c.n_tiles_max <= 0) return hipSuccess;
    if (!tiled_supported(c.dtype, c.H, c.I)) return hipErrorInvalidValue;
    if (c.dtype == RDG_BF16) return launch_dt<RDG_BF16>(c, s);
    if (c.dtype == RDG_FP8_E4M3) return launch_dt<RDG_FP8_E4M3>(c, s);
    return hipErrorInvalidValue;
}

}  // namespace rdg
