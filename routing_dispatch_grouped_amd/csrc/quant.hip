// fp8 e4m3 block quantiser: the 1x128 activation scales and 128x128 weight
// scales of the block-scaled ("1d2d") grouped GEMM named in the DeepGEMM
// single-batch-overlap pull request, section 3.  Scale = amax / 448 in fp32,
// or the smallest power of two not below it (fp8_block_scale), 1 for an
// all-zero block; code = RNE(clamp(v / scale, -448, 448)) with an IEEE fp32
// division, so the codes are reproducible bit for bit.
#include "rdg_internal.h"

namespace rdg {
namespace {

template <bool BF16>
__device__ __forceinline__ float load_src(const void* p, size_t i) {
    if (BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
    return static_cast<const float*>(p)[i];
}

__device__ __forceinline__ uint32_t quant_one(float v, float s) {
    float t = v / s;
    t = fminf(fmaxf(t, -448.0f), 448.0f);
    return f32_to_e4m3(t);
}

// 1 x 128 blocks: one wave per (row, block), two elements per lane.
template <bool BF16, bool POW2>
__global__ __launch_bounds__(256) void k_quant_rows(const void* __restrict__ src, int rows, int cols,
                                                    uint8_t* __restrict__ q, float* __restrict__ scales) {
    const int nb = cols / 128;
    const int64_t blk = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
    if (blk >= (int64_t)rows * nb) return;
    const int lane = lane_id();
    const int64_t r = blk / nb;
    const int b = (int)(blk % nb);
    const size_t base = (size_t)r * cols + (size_t)b * 128 + 2 * lane;
    const float v0 = load_src<BF16>(src, base), v1 = load_src<BF16>(src, base + 1);
    const float amax = wave_max_f32(fmaxf(fabsf(v0), fabsf(v1)));
    const float s = fp8_block_scale(amax, POW2);
    const uint32_t c = quant_one(v0, s) | (quant_one(v1, s) << 8);
    reinterpret_cast<uint16_t*>(q + base)[0] = (uint16_t)c;
    if (lane == 0) scales[blk] = s;
}

// 128 x 128 blocks: one workgroup per block; thread t covers row t/2, 64 columns.
template <bool BF16, bool POW2>
__global__ __launch_bounds__(256) void k_quant_w(const void* __restrict__ src, int rows, int cols,
                                                 uint8_t* __restrict__ q, float* __restrict__ scales) {
    __shared__ float red[4];
    const int nb = cols / 128;
    const int br = blockIdx.x / nb, bc = blockIdx.x % nb;
    const int r = br * 128 + threadIdx.x / 2;
    const int c0 = bc * 128 + (threadIdx.x & 1) * 64;
    const bool ok = r < rows;
    float amax = 0.0f;
    if (ok)
        for (int j = 0; j < 64; ++j) amax = fmaxf(amax, fabsf(load_src<BF16>(src, (size_t)r * cols + c0 + j)));
    amax = wave_max_f32(amax);
    if (lane_id() == 0) red[threadIdx.x / kWave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = fp8_block_scale(amax, POW2);
    if (threadIdx.x == 0) scales[blockIdx.x] = s;
    if (!ok) return;
    for (int j = 0; j < 64; j += 4) {
        uint32_t c = 0;
        for (int u = 0; u < 4; ++u) c |= quant_one(load_src<BF16>(src, (size_t)r * cols + c0 + j + u), s) << (8 * u);
        *reinterpret_cast<uint32_t*>(q + (size_t)r * cols + c0 + j) = c;
    }
}

template <bool POW2>
hipError_t launch_quantize_t(const void* src, bool bf, int rows, int cols, int block_rows, uint8_t* q, float* scales,
                             hipStream_t s) {
    if (block_rows == 1) {
        int64_t blocks = ((int64_t)rows * (cols / 128) + 3) / 4;
        if (bf)
            k_quant_rows<true, POW2><<<(unsigned)blocks, 256, 0, s>>>(src, rows, cols, q, scales);
        else
            k_quant_rows<false, POW2><<<(unsigned)blocks, 256, 0, s>>>(src, rows, cols, q, scales);
    } else {
        int64_t blocks = (int64_t)((rows + 127) / 128) * (cols / 128);
        if (bf)
            k_quant_w<true, POW2><<<(unsigned)blocks, 256, 0, s>>>(src, rows, cols, q, scales);
        else
            k_quant_w<false, POW2><<<(unsigned)blocks, 256, 0, s>>>(src, rows, cols, q, scales);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const void* src, int src_dt, int rows, int cols, int block_rows, bool pow2, uint8_t* q,
                           float* scales, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    const bool bf = src_dt == RDG_BF16;
    return pow2 ? launch_quantize_t<true>(src, bf, rows, cols, block_rows, q, scales, s)
                : launch_quantize_t<false>(src, bf, rows, cols, block_rows, q, scales, s);
}

}  // namespace rdg
