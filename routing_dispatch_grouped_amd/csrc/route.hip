// Group-limited top-k gating, one wavefront per token.
//
// What it computes (DeepEP deep-dive, section on DeepSeek-V3's
// group-limited gating: the router keeps the best expert groups first and
// then the top-K experts inside them; same page, EP section: the token's
// output is the routing-weighted sum over its K experts).  Scores are
// sigmoids of the logits, a group's score is the sum of its two best scores,
// the K weights are renormalised to sum to `scale`, and every tie goes to the
// lower index.
//
// With a selection bias (a variant not on the pages: a per-expert correction
// added for the choice only), groups and experts are chosen by the fp32 sums
// score + bias, and the weights still renormalise the plain scores.
//
// Design for CDNA4: a token's N <= 1024 choosing scores sit in LDS (one
// wave's private slice) and in registers (N/64 per lane, expert e on lane
// e % 64).  Group g's score is computed by lane g % 64; each of the
// topk_group + K selection rounds is one 64-lane max-reduction of a 64-bit
// key (ordered score bits << 32 | ~index) -- the fp32 bits mapped so that
// unsigned order is numeric order, and ~index makes the lower index win a
// tie.
#include "rdg_internal.h"

#pragma clang fp contract(off)

namespace rdg {
namespace {

// The score: sigmoid in fp64, rounded once to fp32.  Every step is one IEEE
// double operation so the value is identical wherever it is evaluated:
//   x clamped to [-87, 87]; z = -x; n = rint(z * log2(e));
//   r = z - n*ln2 with ln 2 split in a 42-bit head (exact products) and a tail;
//   e^r by its degree-13 Taylor series (Horner, fma, 1/k! rounded to double);
//   e^z = e^r * 2^n exactly; score = (float)(1 / (1 + e^z)).
// The truncation error of the series for |r| <= ln2/2 is below 2^-55.
constexpr double kLog2e = 0x1.71547652b82fep+0;   // double nearest 1/ln 2
constexpr double kLn2Hi = 0x1.62e42fefa3800p-1;   // double ln 2, 42 significant bits
constexpr double kLn2Lo = 0x1.ef00000000000p-45;  // double ln 2 minus the head
constexpr double kInvFact[14] = {
    0x1.0000000000000p+0,  0x1.0000000000000p+0,  0x1.0000000000000p-1,  0x1.5555555555555p-3,
    0x1.5555555555555p-5,  0x1.1111111111111p-7,  0x1.6c16c16c16c17p-10, 0x1.a01a01a01a01ap-13,
    0x1.a01a01a01a01ap-16, 0x1.71de3a556c734p-19, 0x1.27e4fb7789f5cp-22, 0x1.ae64567f544e4p-26,
    0x1.1eed8eff8d898p-29, 0x1.6124613a86d09p-33};

__device__ __forceinline__ float score_sigmoid(float xf) {
    xf = fminf(fmaxf(xf, -87.0f), 87.0f);
    double z = -(double)xf;
    double n = __builtin_rint(z * kLog2e);
    double r = __builtin_fma(-n, kLn2Hi, z);
    r = __builtin_fma(-n, kLn2Lo, r);
    double p = kInvFact[13];
#pragma unroll
    for (int k = 12; k >= 0; --k) p = __builtin_fma(p, r, kInvFact[k]);
    double e = __builtin_ldexp(p, (int)n);
    return (float)(1.0 / (1.0 + e));
}

// fp32 -> uint32 whose unsigned order is the numeric order (negative values
// have every bit flipped, non-negative ones the sign bit); never 0 for a
// finite value
__device__ __forceinline__ uint32_t ordered_bits(float v) {
    const uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint64_t make_key(float score, int idx) {
    return ((uint64_t)ordered_bits(score) << 32) | (uint32_t)(0xffffffffu - (uint32_t)idx);
}
__device__ __forceinline__ int key_index(uint64_t key) { return (int)(0xffffffffu - (uint32_t)key); }

template <int VPL>
__global__ __launch_bounds__(256) void k_route(const float* __restrict__ logits, const float* __restrict__ bias,
                                               int B, int N, int n_group, int topk_group, int K, float scale,
                                               int32_t* __restrict__ ids, float* __restrict__ w) {
    __shared__ float lds[4][64 * VPL];   // choosing scores
    __shared__ float plain_lds[4][64 * VPL];  // plain scores (weights), with a bias
    __shared__ uint8_t gsel_lds[4][64 * VPL];
    const int wv = threadIdx.x / kWave, lane = lane_id();
    const int t = blockIdx.x * 4 + wv;
    if (t >= B) return;  // the wave is idle; nothing below synchronises across waves
    float* s_lds = lds[wv];
    float* p_lds = plain_lds[wv];
    const float* row = logits + (size_t)t * N;

    float s[VPL];  // choosing scores
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        int e = lane + kWave * v;
        const float plain = e < N ? score_sigmoid(row[e]) : 0.0f;
        s[v] = bias && e < N ? plain + bias[e] : plain;
        if (e < N) {
            s_lds[e] = s[v];
            if (bias) p_lds[e] = plain;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // group score: sum of the group's two largest scores (with multiplicity);
    // lane l owns groups l, l+64, ... (n_group <= N <= 64*VPL, so VPL slots suffice)
    const int gs = N / n_group;
    uint64_t gkey[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
        const int g = lane + kWave * j;
        gkey[j] = 0ull;
        if (g < n_group) {
            float a = -__builtin_inff(), b = -__builtin_inff();
            for (int i = g * gs; i < (g + 1) * gs; ++i) {
                const float v = s_lds[i];
                if (v > a) {
                    b = a;
                    a = v;
                } else if (v > b) {
                    b = v;
                }
            }
            gkey[j] = make_key(gs >= 2 ? a + b : a, g);
        }
    }
    // keep topk_group groups; the kept set is a byte per group in LDS
    uint8_t* gsel = gsel_lds[wv];
    for (int g = lane; g < n_group; g += kWave) gsel[g] = 0;
    for (int r = 0; r < topk_group; ++r) {
        uint64_t best = 0;
#pragma unroll
        for (int j = 0; j < VPL; ++j) best = gkey[j] > best ? gkey[j] : best;
        const int g = key_index(wave_max_u64(best));
#pragma unroll
        for (int j = 0; j < VPL; ++j)
            if (lane + kWave * j == g) gkey[j] = 0ull;
        if (lane == 0) gsel[g] = 1;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // top-K experts of the kept groups
    uint64_t key[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        int e = lane + kWave * v;
        bool cand = e < N && gsel[e / gs];
        key[v] = cand ? make_key(s[v], e) : 0ull;
    }
    float my_s = 0.0f;
    int my_id = 0;
    for (int k = 0; k < K; ++k) {
        uint64_t best = 0;
#pragma unroll
        for (int v = 0; v < VPL; ++v) best = key[v] > best ? key[v] : best;
        uint64_t m = wave_max_u64(best);
        int e = key_index(m);
#pragma unroll
        for (int v = 0; v < VPL; ++v)
            if (lane + kWave * v == e) key[v] = 0ull;
        if (lane == k) my_id = e;
    }
    // renormalise the plain scores: fp32 sum in slot order, then
    // w_k = s_k / sum * scale
    if (lane < K) my_s = bias ? p_lds[my_id] : s_lds[my_id];
    float sum = 0.0f;
    for (int k = 0; k < K; ++k) sum += __shfl(my_s, k);
    if (lane < K) {
        ids[(size_t)t * K + lane] = my_id;
        w[(size_t)t * K + lane] = (my_s / sum) * scale;
    }
}

}  // namespace

hipError_t launch_route(const float* logits, const float* bias, int B, int N, int n_group, int topk_group, int K,
                        float scale, int32_t* ids, float* w, hipStream_t s) {
    if (B == 0) return hipSuccess;
    dim3 grid((B + 3) / 4), block(256);
    if (N <= 64)
        k_route<1><<<grid, block, 0, s>>>(logits, bias, B, N, n_group, topk_group, K, scale, ids, w);
    else if (N <= 256)
        k_route<4><<<grid, block, 0, s>>>(logits, bias, B, N, n_group, topk_group, K, scale, ids, w);
    else
        k_route<16><<<grid, block, 0, s>>>(logits, bias, B, N, n_group, topk_group, K, scale, ids, w);
    return hipGetLastError();
}

}  // namespace rdg
