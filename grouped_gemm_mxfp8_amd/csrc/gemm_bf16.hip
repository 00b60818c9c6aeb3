// BF16 GroupedLinear for gfx950: Y[rows of e] = X[rows of e] . W_e^T for all
// experts in one launch (German page, the paragraph on fragmented expert
// execution: one call over all experts, given the tokens per expert).
//
// 64 x 64 output tile per workgroup of 4 waves (2 x 2, 32 x 32 each as 2 x 2
// v_mfma_f32_16x16x32_bf16 blocks).  Fragments are read straight from global
// memory (each lane reads 16 contiguous bytes along K) -- the shapes this
// path serves are small and launch-bound, so there is no LDS staging.  The
// y grid dimension walks M tiles of all experts: each workgroup finds its
// expert from a prefix of per-expert tile counts built in LDS.
#include "internal.h"
#include "mx_device.h"

namespace mx {
namespace {

constexpr int TM = 64, TN = 64;

__global__ void __launch_bounds__(256)
bf16_grouped_kernel(const uint16_t* __restrict__ x, const int64_t* __restrict__ offs,
                    int G, const uint16_t* __restrict__ w, int64_t N, int64_t K,
                    const float* __restrict__ rscale, uint16_t* __restrict__ y) {
    __shared__ int s_prefix[kMaxGroups + 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (wave == 0) {
        int cnt[16], local = 0;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int g = lane * 16 + u;
            int c = 0;
            if (g < G) {
                const int64_t n = offs[g + 1] - offs[g];
                c = n > 0 ? (int)((n + TM - 1) / TM) : 0;
            }
            cnt[u] = c;
            local += c;
        }
        int incl = local;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int o = __shfl_up(incl, d);
            if (lane >= d) incl += o;
        }
        int run = incl - local;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int g = lane * 16 + u;
            if (g < G) { s_prefix[g] = run; run += cnt[u]; }
        }
        if (lane == 63) s_prefix[G] = incl;
    }
    __syncthreads();
    const int t = blockIdx.y;
    if (t >= s_prefix[G]) return;
    int lo = 0, hi = G - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_prefix[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int g = lo;
    const int64_t mbeg = offs[g] + (int64_t)(t - s_prefix[g]) * TM;
    const int64_t mend = offs[g + 1];
    const int64_t n0 = (int64_t)blockIdx.x * TN;
    const uint16_t* wg = w + (int64_t)g * N * K;

    const int wm = wave >> 1, wn = wave & 1;
    const int r16 = lane & 15, q = lane >> 4;
    v4f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    int64_t arow[2], brow[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        int64_t r = mbeg + wm * 32 + i * 16 + r16;
        arow[i] = r < mend ? r : mend - 1;           // clamp; results masked
        int64_t c = n0 + wn * 32 + i * 16 + r16;
        brow[i] = c < N ? c : N - 1;
    }
    for (int64_t k0 = 0; k0 < K; k0 += 32) {
        bf16x8 a[2], b[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            a[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(x + arow[i] * K + k0 + q * 8));
            b[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(wg + brow[i] * K + k0 + q * 8));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t row = mbeg + wm * 32 + i * 16 + 4 * q + v;
            if (row >= mend) continue;
            const float sc = rscale ? rscale[row] : 1.0f;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int64_t col = n0 + wn * 32 + j * 16 + r16;
                if (col < N) y[row * N + col] = (uint16_t)f32_to_bf16(acc[i][j][v] * sc);
            }
        }
}

}  // namespace

hipError_t launch_bf16_grouped(const uint16_t* x, const int64_t* offs, int G,
                               int64_t M, const uint16_t* w, int64_t N,
                               int64_t K, const float* rscale, uint16_t* y,
                               hipStream_t s) {
    const int64_t mt_bound = (M + (int64_t)G * (TM - 1)) / TM;
    if (mt_bound == 0 || N == 0) return hipSuccess;
    dim3 grid((unsigned)((N + TN - 1) / TN), (unsigned)mt_bound);
    hipLaunchKernelGGL(bf16_grouped_kernel, grid, dim3(256), 0, s, x, offs, G, w, N, K,
                       rscale, y);
    return hipGetLastError();
}

}  // namespace mx
