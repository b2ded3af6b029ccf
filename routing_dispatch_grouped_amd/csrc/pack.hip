// Weight packing: natural K-major matrices -> MFMA-operand tile order.
//
// HBM on MI355X streams a wavefront load best when the 64 lanes' 16-byte
// pieces form one contiguous KiB; the MFMA operand layout instead wants lane
// l to hold row l % 16 of a 16-row tile.  Packing the (static) weights once
// puts every 16-row x KS tile into lane order, so the grouped GEMMs load each
// operand with a single contiguous KiB per instruction straight into
// registers.  Within a tile, lane l = 16*g + r holds row r and the g-th
// quarter of the tile's KS reduction elements (4/32/128 for fp32/bf16/fp8);
// an fp8 lane holds 32 bytes, stored as two KiB halves (the lanes' first 16
// bytes, then their second 16 bytes).
#include "rdg_internal.h"

namespace rdg {
namespace {

// One thread per 16-byte piece (bf16 / fp8) or per element (fp32) of the input.
template <int DT>
__global__ __launch_bounds__(256) void k_pack(const uint8_t* __restrict__ W, int rows, int cols, int64_t n_units,
                                              uint8_t* __restrict__ P) {
    constexpr int ESZ = DT == RDG_F32 ? 4 : DT == RDG_BF16 ? 2 : 1;
    constexpr int KS = DT == RDG_F32 ? 4 : DT == RDG_BF16 ? 32 : 128;
    constexpr int UNIT = DT == RDG_F32 ? 4 : 16;         // bytes moved per thread
    constexpr int BLK = 64 * KS / 4 * ESZ;               // tile bytes: 256 / 1024 / 2048
    const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (u >= n_units) return;
    const int per_row = cols * ESZ / UNIT;
    const int64_t row_all = u / per_row;                 // matrix * rows + row
    const int k = (int)(u % per_row) * UNIT / ESZ;       // first element of this piece
    const int64_t mat = row_all / rows;
    const int row = (int)(row_all % rows);
    const int rg = row / 16, r = row % 16;
    const int ks = k / KS, kk = k % KS;
    const int g = kk / (KS / 4);                         // lane group
    const int j = kk % (KS / 4);                         // element inside the lane's chunk
    const int lane = g * 16 + r;
    int64_t off = ((mat * (rows / 16) + rg) * (int64_t)(cols / KS) + ks) * BLK;
    if (DT == RDG_FP8_E4M3) off += (j / 16) * 1024 + lane * 16;  // j is 0 or 16: which KiB half
    else off += (int64_t)lane * (KS / 4) * ESZ + j * ESZ;
    if (DT == RDG_F32)
        *reinterpret_cast<uint32_t*>(P + off) = *reinterpret_cast<const uint32_t*>(W + u * 4);
    else
        *reinterpret_cast<uint4*>(P + off) = *reinterpret_cast<const uint4*>(W + u * 16);
}

}  // namespace

hipError_t launch_pack(const void* W, int dtype, int n_mat, int rows, int cols, void* P, hipStream_t s) {
    const int esz = dtype == RDG_F32 ? 4 : dtype == RDG_BF16 ? 2 : 1;
    const int unit = dtype == RDG_F32 ? 4 : 16;
    const int64_t n_units = (int64_t)n_mat * rows * cols * esz / unit;
    if (n_units == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((n_units + 255) / 256);
    const uint8_t* w = static_cast<const uint8_t*>(W);
    uint8_t* p = static_cast<uint8_t*>(P);
    if (dtype == RDG_F32) k_pack<RDG_F32><<<blocks, 256, 0, s>>>(w, rows, cols, n_units, p);
    else if (dtype == RDG_BF16) k_pack<RDG_BF16><<<blocks, 256, 0, s>>>(w, rows, cols, n_units, p);
    else k_pack<RDG_FP8_E4M3><<<blocks, 256, 0, s>>>(w, rows, cols, n_units, p);
    return hipGetLastError();
}

}  // namespace rdg
