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
// 128 layout rows of one expert and a panel of weight rows.  Wave w owns NRT
// 16-row weight tiles against all 128 token rows (eight 16-row MFMA tiles), so
// each token operand read from LDS feeds NRT MFMAs and each weight operand
// eight.  Gated, a wave's first NRT/2 tiles are rows of W1 and the others the
// same rows of W3: the gate and up values of one feature meet in one lane, and
// the SiLU-gated product needs no exchange between waves.  Down, a wave's
// tiles are consecutive rows of W2 (output columns).
//
// The reduction dimension is walked in chunks of CB bytes per row.  The
// token tile is shared by the eight waves, so its chunks go through an LDS
// ring of NSLOT slots filled by direct global->LDS loads; each 16-byte piece
// is stored at a row-dependent XOR of its index (chosen through each lane's
// source address) that makes the MFMA-layout LDS reads conflict-free.  Weight
// operand tiles are private to a wave and arrive packed (pack.hip: one
// contiguous KiB per load instruction) straight into one of NSLOT register
// sets; a weight panel is re-read by every row tile of its expert, mostly
// from L2 (bf16: an expert of one row tile streams its weights past the
// caches with non-temporal loads, 4% faster on the prefill layer's gate/up;
// non-temporal loads for every expert were 12% slower, its sibling tiles
// then missing L2).  While chunk k is multiplied, the next NSLOT-1 chunks'
// token rows and weights are in flight (bf16: three slots of 64 bytes per row, which
// keeps twice as many bytes in flight per CU as two slots of 128 for the
// same registers; fp8: two slots, whose larger chunks halve the barriers of
// its LDS-bound loop); the loop is unrolled by NSLOT so that slots and
// register sets are named at compile time (no register copies that would
// wait for a load in flight, and the compiler can tell the slots apart),
// with one wait and one barrier per chunk.
// fp8 tiles also stage each chunk's activation scales (two 1x128 blocks per
// row) through the ring; every 128-long block's MFMA partial is promoted into
// the fp32 accumulator with its activation and weight scales.
//
// Workgroups are renumbered so that the token tiles sharing one weight panel
// run back to back on the same XCD and re-read the panel from its L2; the
// signalled down stage takes the row tiles in small groups in layout order,
// so that they complete in that order while a combine polls them.
#include <type_traits>

#include "rdg_internal.h"

namespace rdg {
namespace {

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;

constexpr int NW = 8;         // waves per workgroup
constexpr int TB = 128;       // rows per tile
constexpr int NCT = TB / 16;  // 16-row token tiles per wave

template <int DT>
struct TOp;

// LDS slot of 16-byte piece c of tile row r in a chunk of CB bytes per row.
// One MFMA operand read touches one piece of 16 consecutive rows, and the
// XOR spreads those pieces over the LDS banks.  Rows of 256 bytes or more:
// by r % 16, conflict-free.  Rows of 128 bytes (the wide fp8 tile): by r % 8,
// flipped by bit 3 of r, conflict-free; an XOR by (r / 2) % 8 left 43% of the
// LDS's active cycles stalled on bank conflicts (1% slower).  Rows of 64 bytes
// (bf16): by (r / 4) % 4; on this part every placement of 64-byte rows tried
// (other XORs, none) costs a second pass per read, half the LDS cycles, which
// the MFMAs hide (a conflict-free piece-major layout was 5% slower, its
// direct loads touching four times as many rows per instruction).  An
// involution for each row, so it also maps slots back to pieces.
template <int CB>
__device__ __forceinline__ int piece_slot(int r, int c) {
    static_assert(CB == 64 || CB == 128 || CB % 256 == 0, "chunk of 64, 128 or a multiple of 256 bytes per row");
    return CB >= 256   ? (c ^ (r & 15))
           : CB == 128 ? (c ^ ((r & 7) ^ ((r >> 3) & 1)))
                       : (c ^ ((r >> 2) & 3));
}

// Per type: the MFMA step KS (reduction elements), element size, the packed
// weight tile size BLK (see pack.hip), and the operand loads for a chunk of
// S steps and CB bytes per row.
template <int DT>
struct TOp;

template <>
struct TOp<RDG_BF16> {
    using op_t = bf16x8_t;
    static constexpr int KS = 32, ESZ = 2, BLK = 1024;
    template <int S, int NRT, bool NT>
    __device__ static void load_w(op_t (&w)[S][NRT], const uint8_t* const (&wt)[NRT], int t0, int lane) {
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                const bf16x8_t* p = reinterpret_cast<const bf16x8_t*>(wt[rt] + (size_t)(t0 + s) * BLK + lane * 16);
                if constexpr (NT) w[s][rt] = __builtin_nontemporal_load(p);
                else w[s][rt] = *p;
            }
    }
    // token operand of step s for the lane's row l = lane % 16 of a 16-row
    // token tile, lane group g: 16-byte piece 4s+g.  The swizzle depends on
    // l only, so the lane's offset is fixed per step and the token tile and
    // ring slot add a constant (the LDS instruction's immediate offset).
    static constexpr int XH = 1;  // 16-byte pieces per lane and step
    template <int CB>
    __device__ static int x_off(int l, int s, int g, int h) {
        return l * CB + (piece_slot<CB>(l, s * 4 + g) << 4);
    }
    __device__ static op_t load_x(const uint8_t* p, const int (&xo)[XH]) {
        return *reinterpret_cast<const bf16x8_t*>(p + xo[0]);
    }
    __device__ static f32x4_t mma(f32x4_t c, op_t a, op_t b) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <>
struct TOp<RDG_FP8_E4M3> {
    using op_t = i32x8_t;
    static constexpr int KS = 128, ESZ = 1, BLK = 2048;  // a step is one 1x128 scale block
    template <int S, int NRT, bool NT>  // NT unused: the fp8 loop has one load policy (cacheable)
    __device__ static void load_w(op_t (&w)[S][NRT], const uint8_t* const (&wt)[NRT], int t0, int lane) {
#pragma unroll
        for (int s = 0; s < S; ++s)
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
    // 32 bytes: pieces 8s+2g and 8s+2g+1 (lane offsets as for bf16)
    static constexpr int XH = 2;
    template <int CB>
    __device__ static int x_off(int l, int s, int g, int h) {
        return l * CB + (piece_slot<CB>(l, s * 8 + g * 2 + h) << 4);
    }
    __device__ static op_t load_x(const uint8_t* p, const int (&xo)[XH]) {
        const i32x4_t a = *reinterpret_cast<const i32x4_t*>(p + xo[0]);
        const i32x4_t b = *reinterpret_cast<const i32x4_t*>(p + xo[1]);
        op_t o;
        o[0] = a[0]; o[1] = a[1]; o[2] = a[2]; o[3] = a[3];
        o[4] = b[0]; o[5] = b[1]; o[6] = b[2]; o[7] = b[3];
        return o;
    }
    __device__ static f32x4_t mma(f32x4_t c, op_t a, op_t b) {
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
    }
    // with block scales as 8-bit exponents: each lane's scale applies to the
    // 32 reduction elements it holds of its row of a (weights) / column of b
    // (tokens) -- here the lanes of one row or column carry the same scale
    __device__ static f32x4_t mma_scaled(f32x4_t c, op_t a, op_t b, int ea, int eb) {
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, ea, 0, eb);
    }
};

// Tile shape: NRT 16-row weight tiles per wave, the chunk CB (bytes of each
// row per chunk) and the ring depth NSLOT, sized so that NSLOT chunks of
// weights in registers, the accumulators and the operand pipeline fit two
// waves per SIMD.  WIDE: 64
// weight rows per wave, so each token operand read from LDS feeds four MFMAs
// (bf16, and fp8 with power-of-two scales when the grid still fills the
// chip); otherwise 32 rows (fp8 with fp32 scales keeps registers for the
// block partials it promotes).
template <int DT, bool WIDE>
struct TShape;
template <>
struct TShape<RDG_BF16, true> {
    static constexpr int NRT = 4, CB = 64, NSLOT = 3;
};
template <>
struct TShape<RDG_FP8_E4M3, false> {
    static constexpr int NRT = 2, CB = 256, NSLOT = 2;
};
template <>
struct TShape<RDG_FP8_E4M3, true> {
    static constexpr int NRT = 4, CB = 128, NSLOT = 2;
};

template <int DT, bool WIDE>
constexpr int panel_rows() { return NW * TShape<DT, WIDE>::NRT * 16; }  // weight rows per workgroup

struct TArgs {
    const int32_t* offsets;
    const int32_t* masked_m;
    const int32_t* tile_off;  // BT = 128 prefix table
    int n_local, Kdim, Nout, n_tiles_max;
    const uint8_t* X;        // layout rows, or tokens read through gather
    const float* Xs;
    const int32_t* gather;   // NULL, or the layout's row_src: row r's operand is token gather[r] / gather_k
    int gather_k;
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

// Direct global->LDS loads of 16 or 4 bytes per lane (to lds + 16 * lane or
// lds + 4 * lane; lds wave-uniform).  The compiler treats a builtin direct
// load in flight as an LDS operation of unknown order and then waits for
// every LDS read (lgkmcnt(0)) before each use of one: in the fp8 loop a
// token operand prefetched two items ahead was waited for at once.  Issued
// from inline assembly (ASM) the loads are invisible to its counters, so it
// counts the LDS reads again (lgkmcnt(7) there); the loops wait for the
// loads themselves (counted vmcnt waits before each barrier), and any vmcnt
// wait the compiler adds can only wait longer, as loads complete in order.
// fp8 tiles use the assembly form (gate/up and down 3% faster); bf16 tiles,
// whose chunk is one MFMA step deep, keep the builtin (1% faster there).
// The kernels use m0 for nothing else (clang warns about clobbering it).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <bool ASM>
__device__ __forceinline__ void dma16(const void* src, const void* lds) {
    if constexpr (ASM) {
        const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)lds);
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(l) : "memory", "m0");
    } else {
        __builtin_amdgcn_global_load_lds((gbl_ptr_t)src, (lds_ptr_t)lds, 16, 0, 0);
    }
}
__device__ __forceinline__ void dma4(const void* src, const void* lds) {
    const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)lds);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(l) : "memory", "m0");
}
#pragma clang diagnostic pop

struct Ring {
    uint8_t* x;  // 128 * CB bytes: the token chunk
    float* s;    // fp8: [128 rows][SPB blocks] activation scales of the chunk
    float* w;    // fp8: [NW waves][2][STEPS] the chunk's weight block scales of each wave (W1 / W2, W3)
};

// The operand rows this lane stages, found once per workgroup: rows past
// the tile's valid rows re-read the last valid row (in bounds, never
// stored); with a gather, each row's token.  xr[i]: the 16 bytes of x-load
// i (see stage_chunk); sr: fp8, the activation scales of row 16 wv + l / SPB.
template <int CB>
struct StageRows {
    static constexpr int XLOADS = TB * CB / 1024 / NW, PPR = CB / 16, SPB = CB / 128;
    int xr[XLOADS];
    int sr;
    __device__ StageRows(const TArgs& a, int row0, int nvalid, int wv, int lane) {
#pragma unroll
        for (int i = 0; i < XLOADS; ++i) {
            const int r = (wv * XLOADS + i) * (1024 / CB) + lane / PPR;
            xr[i] = token_row(a.gather, a.gather_k, row0 + (r < nvalid ? r : nvalid - 1));
        }
        sr = 0;
        if constexpr (SPB > 0) {
            const int r = wv * 16 + (lane % (16 * SPB)) / SPB;
            sr = token_row(a.gather, a.gather_k, row0 + (r < nvalid ? r : nvalid - 1));
        }
    }
};

// Request chunk kc of the tile's token rows: 128 * CB / 1024 / NW direct KiB
// loads per wave; fp8: one load of the chunk's activation scales of 16 rows
// per wave.
template <int DT, int CB>
__device__ __forceinline__ void stage_chunk(const TArgs& a, size_t xstride, int nkb, const StageRows<CB>& rows,
                                            int kc, const Ring& ring, int wv, int lane) {
    constexpr int XLOADS = StageRows<CB>::XLOADS, SPB = CB / 128;
    constexpr int PPR = CB / 16;  // 16-byte pieces per row
    static_assert(XLOADS >= 1 && 1024 % CB == 0 && XLOADS * NW * 1024 == TB * CB, "chunk shape");
#pragma unroll
    for (int i = 0; i < XLOADS; ++i) {
        const int q = wv * XLOADS + i;               // LDS bytes [q*1024, q*1024+1024)
        const int r = q * (1024 / CB) + lane / PPR;  // tile row of this lane's 16 bytes
        const int c = piece_slot<CB>(r, lane % PPR);  // source piece of this lane's slot
        const uint8_t* src = a.X + (size_t)rows.xr[i] * xstride + (size_t)kc * CB + c * 16;
        dma16<DT == RDG_FP8_E4M3>(src, ring.x + q * 1024);
    }
    if constexpr (DT == RDG_FP8_E4M3) {
        // lanes 0..16*SPB-1 of wave w: row 16w + l/SPB, scale block SPB*kc + l%SPB
        static_assert(TB == 16 * NW && SPB * 16 <= 64, "one load of scales per wave");
        const int l = lane % (16 * SPB);
        const float* src = a.Xs + (size_t)rows.sr * nkb + SPB * kc + l % SPB;
        if (lane < 16 * SPB)
            dma4(src, ring.s + wv * 16 * SPB);
    }
}

// Work order of the plain down GEMM (a tile's output columns in panels of
// PANEL, gridDim.y panels).  Row tiles of experts with several tiles ("busy")
// keep the order above: XCD x runs a contiguous share of the (panel, tile)
// pairs, panel-major, so one weight panel serves consecutive row tiles from
// its L2.  The tile of an expert with one tile has no sibling to share its
// weights with, but every panel of it reads the same h rows (a quarter of
// its bytes at I = 2048): its panels run back to back on one XCD, which then
// fetches those rows once instead of every XCD fetching them.  Each XCD's
// busy and one-tile items are interleaved in proportion (busy items alone
// leave HBM idle, one-tile items alone the matrix cores), and the XCDs get
// equal shares of both.  On the prefill layer's down GEMM: 1.77 -> 1.69 ms
// (balanced layer 1.81 -> 1.66 ms); the gate/up GEMM, whose tokens are 6% of
// a one-tile expert's bytes, was slower this way (3.03 -> 3.10 ms) and keeps
// the plain order, and so does the fp8 down GEMM (the decode rank share's
// step 0.158 -> 0.164 ms this way: its 308 workgroups need a second round).
// Returns false (plain order) when some XCD would get more items than
// workgroups; sets tile = -1 for a workgroup with no item.
__device__ bool down_split(const TArgs& a, int& fb, int& tile) {
    const int gx = a.n_tiles_max, gy = gridDim.y, total = gx * gy;
    const int b = blockIdx.y * gx + blockIdx.x;
    const int xcd = b % 8, q8 = total / 8, r8 = total % 8;
    // exclusive prefixes over the experts of their busy tiles and of their
    // one-tile counts (n_local <= 1024), built by the first wave
    __shared__ int s_busy[1025], s_one[1025];
    if (threadIdx.x < kWave) {
        const int l = threadIdx.x, per = (a.n_local + kWave - 1) / kWave;
        const int e0 = l * per, e1 = e0 + per < a.n_local ? e0 + per : a.n_local;
        int bs = 0, os = 0;
        for (int e = e0; e < e1; ++e) {
            const int nt = a.tile_off[e + 1] - a.tile_off[e];
            bs += nt >= 2 ? nt : 0;
            os += nt == 1 ? 1 : 0;
        }
        int bx = bs, ox = os;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int y = __shfl_up(bx, off), z = __shfl_up(ox, off);
            if (l >= off) {
                bx += y;
                ox += z;
            }
        }
        int bb = bx - bs, ob = ox - os;
        for (int e = e0; e < e1; ++e) {
            s_busy[e] = bb;
            s_one[e] = ob;
            const int nt = a.tile_off[e + 1] - a.tile_off[e];
            bb += nt >= 2 ? nt : 0;
            ob += nt == 1 ? 1 : 0;
        }
        if (l == kWave - 1) {
            s_busy[a.n_local] = bx;
            s_one[a.n_local] = ox;
        }
    }
    __syncthreads();
    const int NB = s_busy[a.n_local], NO = s_one[a.n_local];
    const int busy_items = NB * gy, bq = busy_items / 8, br = busy_items % 8;
    const int oq = NO / 8, orr = NO % 8;
    for (int x = 0; x < 8; ++x)  // every XCD's items must fit its workgroups
        if (bq + (x < br ? 1 : 0) + (oq + (x < orr ? 1 : 0)) * gy > q8 + (x < r8 ? 1 : 0)) return false;
    const int busy_n = bq + (xcd < br ? 1 : 0), busy_start = xcd * bq + (xcd < br ? xcd : br);
    const int one_n = oq + (xcd < orr ? 1 : 0), one_start = xcd * oq + (xcd < orr ? xcd : orr);
    const int n_x = busy_n + one_n * gy, pos = b / 8;
    tile = -1;
    if (pos >= n_x) return true;
    // item pos of the XCD is busy item floor(pos * busy_n / n_x) when that
    // count steps at pos, else one-tile item pos - (busy items before it)
    const int b0 = (int)((int64_t)pos * busy_n / n_x), b1 = (int)((int64_t)(pos + 1) * busy_n / n_x);
    int lo = 0, hi = a.n_local;
    if (b1 > b0) {
        const int item = busy_start + b0;
        fb = item / NB;
        const int h = item % NB;
        while (hi - lo > 1) {  // the last expert whose busy prefix is <= h
            const int mid = (lo + hi) >> 1;
            if (s_busy[mid] <= h) lo = mid;
            else hi = mid;
        }
        tile = a.tile_off[lo] + (h - s_busy[lo]);
    } else {
        const int j = pos - b0;
        const int c = one_start + j / gy;
        fb = j % gy;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_one[mid] <= c) lo = mid;
            else hi = mid;
        }
        tile = a.tile_off[lo];
    }
    return true;
}

// Work order of the signalled down GEMM: the row tiles in groups of G
// (G = 4, raised until G * P is a multiple of 8 for P column panels), in
// layout order, so that the tiles complete group by group in the order the
// polling consumer takes them.  Within a group the G * P items are
// panel-major and split into 8 equal contiguous shares, XCD x (hardware block
// b runs on XCD b % 8 as its (b / 8)-th block) taking share x: a few adjacent
// weight panels against the group's tiles.  The last, partial group is split
// as in the plain order.  On the prefill rank share the signalled down GEMM
// takes 0.397 ms this way against 0.436 ms tile-major (panels fb = x mod 8 of
// every tile on XCD x), 0.399 / 0.409 / 0.418 ms with groups of 2 / 8 / 16
// tiles, and 0.401 ms in the plain order, where tiles complete only at the
// end.  Returns false for a block without an item.  The grid has
// n_tiles_max x (P + 1) blocks, at least tiles x (P + 1): every XCD then has
// at least as many blocks as items.
__device__ bool signal_order(const TArgs& a, int cols, int& fb, int& tile) {
    const int P = a.Nout / cols, nt = a.tile_off[a.n_local];
    int G = 4;
    while ((G * P) % 8) ++G;
    const int b = blockIdx.y * gridDim.x + blockIdx.x, xcd = b % 8, pos = b / 8;
    const int F = nt / G, qg = G * P / 8;  // whole groups; items per XCD and group
    if (pos < F * qg) {
        const int i = xcd * qg + pos % qg;  // item within group pos / qg
        fb = i / G;
        tile = pos / qg * G + i % G;
        return true;
    }
    const int L = nt - F * G, p2 = pos - F * qg;  // the partial group
    const int q8 = L * P / 8, r8 = L * P % 8;
    if (p2 >= q8 + (xcd < r8 ? 1 : 0)) return false;
    const int logical = xcd * q8 + (xcd < r8 ? xcd : r8) + p2;
    fb = logical / L;
    tile = F * G + logical % L;
    return true;
}

// PW2 (fp8 with power-of-two block scales): the scales go into the scaled
// MFMA as 8-bit exponents and the matrix core accumulates across blocks; no
// per-block promotion.  WIDE: see TShape.
template <int DT, bool GATED, bool SIGNAL, bool PW2, bool WIDE>
__global__ __launch_bounds__(NW * 64, 1) void k_ffn_tiled(TArgs a) {
    using O = TOp<DT>;
    using op_t = typename O::op_t;
    constexpr int NRT = TShape<DT, WIDE>::NRT, CB = TShape<DT, WIDE>::CB;
    constexpr int S = CB / (O::KS * O::ESZ);  // MFMA steps per chunk
    constexpr int PANEL = panel_rows<DT, WIDE>();
    constexpr int COLS = GATED ? PANEL / 2 : PANEL;  // output columns per workgroup
    constexpr int NOT = GATED ? NRT / 2 : NRT;       // 16-column output tiles per wave
    constexpr bool FP8 = DT == RDG_FP8_E4M3;
    constexpr int CHUNK_LDS = TB * CB, SPB = CB / 128;
    constexpr int NSLOT = TShape<DT, WIDE>::NSLOT;
    static_assert(NSLOT == 2 || (NSLOT == 3 && !FP8), "two slots, or three without scale slots");
    static_assert(!GATED || NRT % 2 == 0, "a gated wave holds its W1 and W3 tiles in pairs");
    __shared__ __attribute__((aligned(16))) uint8_t lx0[CHUNK_LDS];
    __shared__ __attribute__((aligned(16))) uint8_t lx1[CHUNK_LDS];
    __shared__ __attribute__((aligned(16))) uint8_t lx2[NSLOT > 2 ? CHUNK_LDS : 16];
    __shared__ __attribute__((aligned(16))) float ls0[FP8 ? TB * SPB : 4];
    __shared__ __attribute__((aligned(16))) float ls1[FP8 ? TB * SPB : 4];
    __shared__ __attribute__((aligned(16))) float lw0[FP8 ? NW * 2 * S : 4];
    __shared__ __attribute__((aligned(16))) float lw1[FP8 ? NW * 2 * S : 4];
    const Ring ring[3] = {{lx0, ls0, lw0}, {lx1, ls1, lw1}, {lx2, ls0, lw0}};

    int fb, tile;
    if (SIGNAL) {
        if (!signal_order(a, COLS, fb, tile)) return;  // no item (workgroup-uniform)
    } else if (GATED || FP8 || !down_split(a, fb, tile)) {
        // XCD-aware renumbering over the layout's row tiles: hardware block b
        // runs on XCD b % 8 as its (b / 8)-th block.  XCD x takes the
        // contiguous share starting at x*(n/8) + min(x, n%8) of the n = tiles
        // x panels items, panel-major, so consecutive row tiles of one weight
        // panel share an L2; its blocks past that share have no item.  The
        // grid is sized from the dispatched slots, several times the tiles
        // that arrive on a rank's share: numbering the items over the tiles
        // themselves puts the blocks without one at the end of every XCD's
        // sequence, where they exit beside the last items, instead of between
        // the items.  (The share fits: n <= blocks, so every XCD has at least
        // as many blocks as items.)
        const int gx = a.n_tiles_max, b = blockIdx.y * gx + blockIdx.x;
        const int nt = a.tile_off[a.n_local], n = nt * (int)gridDim.y;
        const int xcd = b % 8, q8 = n / 8, r8 = n % 8;
        if (b / 8 >= q8 + (xcd < r8 ? 1 : 0)) return;  // no item (workgroup-uniform)
        const int logical = xcd * q8 + (xcd < r8 ? xcd : r8) + b / 8;
        fb = logical / nt;
        tile = logical % nt;
    }
    if (tile < 0) return;  // no item for this workgroup (uniform)

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
    // output columns [fw, fw + 16 NOT) of this wave
    const int f0 = fb * COLS;
    const int fw = f0 + wv * NOT * 16;
    const size_t xstride = (size_t)a.Kdim * O::ESZ;
    const int nks = a.Kdim / O::KS;
    const int nkb = a.Kdim / 128;
    const int nchunks = (int)(xstride / CB);
    const StageRows<CB> srows(a, row0, nvalid, wv, lane);

    // weight tile rt: rows fw + 16 (rt % NOT) of W1 (gated, rt < NOT) or W3
    // (gated, rt >= NOT) or W2 (down)
    const uint8_t* wt[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        const size_t grp = (size_t)e * (a.Nout / 16) + fw / 16 + rt % NOT;
        wt[rt] = (rt < NOT ? a.Wa : a.Wb) + grp * nks * O::BLK;
    }
    // fp8: the block scales along K of the wave's W1 / W2 rows and W3 rows
    // (all within one 128-row block)
    const float* wsa = nullptr;
    const float* wsb = nullptr;
    if (FP8) {
        const size_t blk = ((size_t)e * (a.Nout / 128) + fw / 128) * nkb;
        wsa = a.Was + blk;
        wsb = GATED ? a.Wbs + blk : wsa;
    }

    f32x4_t acc[NRT][NCT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) acc[rt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // two weight register sets (chunk k's and k+1's); fp8: the chunk's
    // weight block scales travel with the token chunk's ring slot (direct
    // loads into LDS: a register load of them would make the compiler wait
    // for the chunk in flight to copy it)
    op_t w[NSLOT][S][NRT];

    auto request_w = [&](int kc, op_t (&wr)[S][NRT], const Ring& rg, auto nt) {
        O::template load_w<S, NRT, decltype(nt)::value>(wr, wt, kc * S, lane);
        if (FP8) {
            constexpr int NSC = GATED ? 2 * S : S;
            const float* src = (lane < S ? wsa : wsb) + kc * S + lane % S;
            if (lane < NSC)
                dma4(src, rg.w + wv * 2 * S);
        }
    };
    // the lane's LDS offsets of its token operand pieces, per step
    int xo[S][O::XH];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int h = 0; h < O::XH; ++h) xo[s][h] = O::template x_off<CB>(lane & 15, s, lane >> 4, h);

    // One chunk over the first NV 16-row token tiles: items i = (step s,
    // token tile ct) in order.  The token operand of item i+2 is read from
    // LDS while item i's MFMAs run (a three-deep register ring), and fp8
    // promotes item i-1's block partials behind item i's MFMAs (with
    // power-of-two scales the MFMA applies them and accumulates itself); the
    // scheduling barrier after each item keeps the compiler from hoisting a
    // chunk's worth of LDS reads (registers).
    auto compute = [&](const Ring& rg, const op_t (&wr)[S][NRT], auto nv) {
        constexpr int NV = decltype(nv)::value;
        constexpr int NI = S * NV;
        op_t xb[3];
        float sx[4];
        float swr[S][2];  // fp8: weight block scales of each step (W1 / W2, W3)
        if (FP8) {
#pragma unroll
            for (int s = 0; s < S; ++s) {
                swr[s][0] = rg.w[wv * 2 * S + s];
                swr[s][1] = GATED ? rg.w[wv * 2 * S + S + s] : swr[s][0];
            }
        }
        int ew[S][2];  // PW2: the weight scales as 8-bit exponents
        if (PW2) {
#pragma unroll
            for (int s = 0; s < S; ++s) {
                ew[s][0] = e8m0_of(swr[s][0]);
                ew[s][1] = e8m0_of(swr[s][1]);
            }
        }
        f32x4_t p[2][NRT];
        const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
        auto fetch = [&](int i) {
            const int si = i / NV, ct = i % NV;
            xb[i % 3] = O::load_x(rg.x + ct * 16 * CB, xo[si]);
            if (FP8) sx[i % 4] = rg.s[(ct * 16 + (lane & 15)) * SPB + si];
        };
        auto promote = [&](int i) {  // fp8: item i's block partials into the accumulators
            const int si = i / NV, ct = i % NV;
            const float fa = sx[i % 4] * swr[si][0];
            const float fb3 = sx[i % 4] * swr[si][1];
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) acc[rt][ct] += p[i % 2][rt] * (rt < NOT ? fa : fb3);
        };
        fetch(0);
        fetch(1);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int si = i / NV, ct = i % NV;
            if (i + 2 < NI) fetch(i + 2);
            if constexpr (!FP8) {
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt) acc[rt][ct] = O::mma(acc[rt][ct], wr[si][rt], xb[i % 3]);
            } else if constexpr (PW2) {
                const int eb = e8m0_of(sx[i % 4]);  // this lane's token row
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt)
                    acc[rt][ct] = O::mma_scaled(acc[rt][ct], wr[si][rt], xb[i % 3], ew[si][rt < NOT ? 0 : 1], eb);
            } else {
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt) p[i % 2][rt] = O::mma(z, wr[si][rt], xb[i % 3]);
                // issued behind this item's MFMAs, so that the promotion runs
                // while they execute (item i-1's partials are complete once
                // the MFMA unit starts on item i's)
                __builtin_amdgcn_sched_barrier(0);
                if (i > 0) promote(i - 1);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (FP8 && !PW2) promote(NI - 1);
    };

    // Two slots: chunk k+1's token rows and weights are requested once chunk
    // k has arrived, and are in flight while chunk k is multiplied.  A tile
    // with fewer valid rows (an expert's last tile) only stages and
    // multiplies the 16-row token tiles that hold them: wave w stages rows
    // [16w, 16w+16).
    auto main_loop2 = [&](auto nv) {
        constexpr int NV = decltype(nv)::value;
        if (wv < NV) stage_chunk<DT, CB>(a, xstride, nkb, srows, 0, ring[0], wv, lane);
        request_w(0, w[0], ring[0], std::false_type{});
        for (int kc0 = 0; kc0 < nchunks; kc0 += 2) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int kc = kc0 + j;
                if (kc >= nchunks) break;
                // this wave's loads of chunk kc have landed, then every wave's;
                // past the barrier every wave is also done with chunk kc-1, whose
                // ring slot and weight set are refilled next
                __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
                lds_barrier();
                if (kc + 1 < nchunks) {
                    if (wv < NV)
                        stage_chunk<DT, CB>(a, xstride, nkb, srows, kc + 1, ring[(j + 1) % 2], wv, lane);
                    request_w(kc + 1, w[(j + 1) % 2], ring[(j + 1) % 2], std::false_type{});
                }
                compute(ring[j], w[j], nv);
            }
        }
    };
    // Three slots: chunk k+2 is requested while chunk k is multiplied, so
    // chunk k+1's loads stay in flight across the wait for chunk k.  Every
    // wave issues the same LPC loads for every chunk (all rows of the tile,
    // the clamped ones re-reading the last valid row; past the last chunk it
    // re-reads that chunk into the free slot), so that one count, "at most
    // LPC loads outstanding", means chunk k has landed.  Every slot of an
    // iteration issues its loads and the loop exits only at its latch: the
    // compiler's own wait counts stay exact (an early exit would make it
    // assume the latest loads may still write the next iteration's first
    // register set).  The last loads are drained before the epilogue.
    auto main_loop3 = [&](auto nv, auto nt) {
        constexpr int LPC = TB * CB / 1024 / NW + S * NRT;  // vector-memory loads per chunk and wave
        stage_chunk<DT, CB>(a, xstride, nkb, srows, 0, ring[0], wv, lane);
        request_w(0, w[0], ring[0], nt);
        const int c1 = nchunks > 1 ? 1 : 0;
        stage_chunk<DT, CB>(a, xstride, nkb, srows, c1, ring[1], wv, lane);
        request_w(c1, w[1], ring[1], nt);
        for (int kc0 = 0; kc0 < nchunks; kc0 += 3) {
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                const int kc = kc0 + j;
                __builtin_amdgcn_s_waitcnt(vmcnt_imm<LPC>());
                lds_barrier();
                const int kn = kc + 2 < nchunks ? kc + 2 : nchunks - 1;
                stage_chunk<DT, CB>(a, xstride, nkb, srows, kn, ring[(j + 2) % 3], wv, lane);
                request_w(kn, w[(j + 2) % 3], ring[(j + 2) % 3], nt);
                if (kc < nchunks) compute(ring[j], w[j], nv);
            }
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
    };
    auto main_loop = [&](auto nv) {
        if constexpr (NSLOT == 3) {
            // an expert's only row tile reads its weights once: streamed past
            // the caches; an expert of several tiles keeps them cacheable for
            // its sibling tiles
            if (a.masked_m[e] <= TB) main_loop3(nv, std::true_type{});
            else main_loop3(nv, std::false_type{});
        } else {
            main_loop2(nv);
        }
    };
    // (fp8: the full tile only -- a second copy of the loop does not fit its
    // registers)
    if (nvalid > 64 || FP8) main_loop(std::integral_constant<int, 8>{});
    else if (nvalid > 32) main_loop(std::integral_constant<int, 4>{});
    else if (nvalid > 16) main_loop(std::integral_constant<int, 2>{});
    else main_loop(std::integral_constant<int, 1>{});

    // ---------------------------------------------------------------- epilogue
    // 16x16 accumulator tile: lane l holds column (row of the layout) l % 16 and
    // rows (output features) 4*(l/16) .. +3; gated, the SiLU-gated product of
    // tile ot is formed from W1 tile ot and W3 tile ot + NOT in place
    if (GATED) {
#pragma unroll
        for (int ot = 0; ot < NOT; ++ot)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float g = acc[ot][ct][r];
                    acc[ot][ct][r] = g / (1.0f + __expf(-g)) * acc[ot + NOT][ct][r];
                }
    }
    const int fl = fw + (lane >> 4) * 4;
    if (FP8 && GATED) {
        // h re-quantised with one scale per row and 128 features: the
        // workgroup's waves hold 16 NOT features each, WPB consecutive waves
        // one 128-feature block
        constexpr int WPB = 128 / (NOT * 16);  // waves per 128-feature block
        static_assert(128 % (NOT * 16) == 0 && NW % WPB == 0, "whole 1x128 blocks of h per workgroup");
        __syncthreads();                              // every wave is done with the ring
        float* red = reinterpret_cast<float*>(lx0);  // [NW waves][128 rows]
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            float m = 0.0f;
#pragma unroll
            for (int ot = 0; ot < NOT; ++ot)
#pragma unroll
                for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(acc[ot][ct][r]));
            m = fmaxf(m, __shfl_xor(m, 16));
            m = fmaxf(m, __shfl_xor(m, 32));
            if (lane < 16) red[wv * TB + ct * 16 + lane] = m;
        }
        __syncthreads();
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const int c = ct * 16 + (lane & 15);
            const int w0 = wv / WPB * WPB;
            float amax = red[w0 * TB + c];
#pragma unroll
            for (int q = 1; q < WPB; ++q) amax = fmaxf(amax, red[(w0 + q) * TB + c]);
            if (c >= nvalid) continue;
            const int row = row0 + c;
            const float sc = fp8_block_scale(amax, PW2);
            const float inv = 1.0f / sc;
#pragma unroll
            for (int ot = 0; ot < NOT; ++ot) {
                uint32_t q = 0;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float tq = fminf(fmaxf(acc[ot][ct][r] * inv, -448.0f), 448.0f);
                    q |= f32_to_e4m3(tq) << (8 * r);
                }
                *reinterpret_cast<uint32_t*>(a.O + (size_t)row * a.Nout + fl + ot * 16) = q;
            }
            if (wv == w0 && lane < 16) a.Os[(size_t)row * (a.Nout / 128) + fw / 128] = sc;
        }
    } else {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const int c = ct * 16 + (lane & 15);
            if (c >= nvalid) continue;
            const int row = row0 + c;
#pragma unroll
            for (int ot = 0; ot < NOT; ++ot) {
                const uint64_t o = (uint64_t)(f32_to_bf16(acc[ot][ct][0]) | (f32_to_bf16(acc[ot][ct][1]) << 16)) |
                                   ((uint64_t)(f32_to_bf16(acc[ot][ct][2]) | (f32_to_bf16(acc[ot][ct][3]) << 16))
                                    << 32);
                store_out8<SIGNAL>(a.O + ((size_t)row * a.Nout + fl + ot * 16) * 2, o);
            }
        }
    }
    if (SIGNAL) signal_done(a.signals + row0 / TB, COLS);
}

template <int DT, bool PW2, bool WIDE>
hipError_t launch_dt(const FfnCall& c, hipStream_t s) {
    constexpr int PANEL = panel_rows<DT, WIDE>();
    dim3 block(NW * 64);
    if (c.stages & 1) {
        TArgs g{c.offsets, c.masked_m, c.tile_off, c.n_local, c.H, c.I, c.n_tiles_max,
                static_cast<const uint8_t*>(c.x), c.x_s, c.gather, c.gather_k, static_cast<const uint8_t*>(c.W1),
                static_cast<const uint8_t*>(c.W3), c.W1_s, c.W3_s, static_cast<uint8_t*>(c.h), c.h_s, nullptr};
        k_ffn_tiled<DT, true, false, PW2, WIDE><<<dim3(c.n_tiles_max, c.I / (PANEL / 2)), block, 0, s>>>(g);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (c.stages & 2) {
        TArgs d{c.offsets, c.masked_m, c.tile_off, c.n_local, c.I, c.H, c.n_tiles_max,
                static_cast<const uint8_t*>(c.h), c.h_s, nullptr, 0, static_cast<const uint8_t*>(c.W2), nullptr,
                c.W2_s, nullptr, static_cast<uint8_t*>(c.y), nullptr, c.signals};
        if (c.signals)
            k_ffn_tiled<DT, false, true, PW2, WIDE><<<dim3(c.n_tiles_max, c.H / PANEL + 1), block, 0, s>>>(d);
        else
            k_ffn_tiled<DT, false, false, PW2, WIDE><<<dim3(c.n_tiles_max, c.H / PANEL), block, 0, s>>>(d);
    }
    return hipGetLastError();
}

template <int DT, bool WIDE>
bool shapes_ok(int H, int I) {
    constexpr int PANEL = panel_rows<DT, WIDE>(), CB = TShape<DT, WIDE>::CB, ESZ = TOp<DT>::ESZ;
    return I % (PANEL / 2) == 0 && H % PANEL == 0 && ((int64_t)H * ESZ) % CB == 0 && ((int64_t)I * ESZ) % CB == 0;
}

}  // namespace

// bf16 / fp8 with I a multiple of the gate/up feature panel (bf16 256, fp8
// 128) and H of the down column panel (bf16 512, fp8 256); both reduction
// dimensions in whole chunks.
bool tiled_supported(int dtype, int H, int I) {
    if (dtype == RDG_BF16) return shapes_ok<RDG_BF16, true>(H, I);
    if (dtype == RDG_FP8_E4M3 || dtype == RDG_FP8_E4M3_UE8M0) return shapes_ok<RDG_FP8_E4M3, false>(H, I);
    return false;
}

// power-of-two scales: 64 weight rows per wave when the row tiles times the
// wider gate/up panels fill the CUs several times over, else 32.  n_tiles_max
// bounds the tiles from the dispatched slots, which can be several times the
// rows that arrive (a rank's share), hence the margin.
static bool pow2_wide(const FfnCall& c) {
    return shapes_ok<RDG_FP8_E4M3, true>(c.H, c.I) &&
           (int64_t)c.n_tiles_max * (c.I / (panel_rows<RDG_FP8_E4M3, true>() / 2)) >= 4 * 256;
}

hipError_t launch_ffn_tiled(const FfnCall& c, hipStream_t s) {
    if (c.n_tiles_max <= 0) return hipSuccess;
    if (!tiled_supported(c.dtype, c.H, c.I)) return hipErrorInvalidValue;
    if (c.dtype == RDG_BF16) return launch_dt<RDG_BF16, false, true>(c, s);
    if (c.dtype != RDG_FP8_E4M3) return hipErrorInvalidValue;
    if (!c.pow2) return launch_dt<RDG_FP8_E4M3, false, false>(c, s);
    return pow2_wide(c) ? launch_dt<RDG_FP8_E4M3, true, true>(c, s) : launch_dt<RDG_FP8_E4M3, true, false>(c, s);
}

}  // namespace rdg
