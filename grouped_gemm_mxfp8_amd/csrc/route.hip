// The steps on either side of the expert path, for gfx950: the sorted-row
// plan of a top-k routing (each expert's rows gathered together, the German
// page's paragraph on GroupedLinear: per-expert token counts handed over and
// the expert inputs gathered), and the combine that brings expert outputs
// back to token order with its backward (the Portuguese page, third
// paragraph: routing weights send each token to its experts).
//
// Router: one wave per token picks its k largest logits one at a time (a
// wave-wide arg-max over the lanes' remaining logits, the lower expert index
// among equal values) and turns them into the softmax weights.
//
// Plan: three launches, no host synchronisation and no global atomics.
//  * route_hist: one workgroup per chunk of 256 routing slots counts its
//    slots per expert (LDS counters).
//  * route_scan: one workgroup turns the per-chunk counts into each chunk's
//    first rank per expert and the expert offsets.
//  * route_scatter: every slot's rank among the earlier slots of its chunk
//    with the same expert (an LDS scan of at most 255 entries) gives its
//    sorted row: rows are sorted stably by (expert, token, slot).
// Combine and its backward are HBM-bound gathers: one lane moves 8
// consecutive bf16 values (16 bytes) of a row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "internal.h"
#include "mx_device.h"

namespace mx {

// Library-owned scratch of the plan for callers that cannot allocate
// (moe_route_plan_noalloc): the per-chunk expert counts, kPlanScratchInts
// int32.  Each GPU holds its own copy for the life of the process; in host
// code this name is only a stand-in for the device symbol, so kernels are
// given the address route_plan_scratch() looks up.
static __device__ __align__(256) int32_t scratch[kPlanScratchInts];

namespace {

constexpr int kChunk = 256;   // routing slots per workgroup in the plan
constexpr int kRouterPer = kMaxGroups / 64;   // logits per lane in the router

// (v, i) before (v', i'): larger value, or equal value and lower index
__device__ __forceinline__ bool better(float v, int i, float v2, int i2) {
    return v > v2 || (v == v2 && i < i2);
}

__global__ void __launch_bounds__(256)
router_kernel(const float* __restrict__ logits, int64_t T, int E, int k,
              int32_t* __restrict__ ids, float* __restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;                             // the whole wave
    float v[kRouterPer];
#pragma unroll
    for (int i = 0; i < kRouterPer; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < E ? logits[t * E + e] : 0.f;
    }
    uint32_t taken = 0;
    float my_v = 0.f;
    int my_i = 0;
    for (int p = 0; p < k; ++p) {
        // this lane's best remaining logit (its experts ascend with i)
        float bv = 0.f;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < kRouterPer; ++i) {
            const int e = lane + 64 * i;
            if (e < E && !(taken >> i & 1u) && (bi == 0x7fffffff || v[i] > bv)) {
                bv = v[i];
                bi = e;
            }
        }
        // wave-wide best: a strict total order, so every lane ends with it
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) {
            const float ov = __shfl_xor(bv, d);
            const int oi = __shfl_xor(bi, d);
            if (oi != 0x7fffffff && (bi == 0x7fffffff || better(ov, oi, bv, bi))) {
                bv = ov;
                bi = oi;
            }
        }
        if (lane == p) {
            my_v = bv;
            my_i = bi;
        }
        if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    }
    // softmax of the k selected logits (lane p holds selection p; lane 0 the max)
    const float m = __shfl(my_v, 0);
    const float ex = lane < k ? expf(my_v - m) : 0.f;
    float s = ex;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d);
    if (lane < k) {
        ids[t * k + lane] = my_i;
        w[t * k + lane] = ex / s;
    }
}

__global__ void __launch_bounds__(kChunk)
route_hist_kernel(const int32_t* __restrict__ ids, int64_t n, int E, int32_t* __restrict__ hist) {
    __shared__ int cnt[kMaxGroups];
    for (int e = threadIdx.x; e < E; e += kChunk) cnt[e] = 0;
    __syncthreads();
    const int64_t i = (int64_t)blockIdx.x * kChunk + threadIdx.x;
    if (i < n) {
        const int e = ids[i];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kChunk) hist[(int64_t)blockIdx.x * E + e] = cnt[e];
}

// hist [nchunk][E] counts in, each chunk's first rank per expert out (in
// place); offsets[E+1] = exclusive prefix of the expert totals.
__global__ void __launch_bounds__(kMaxGroups)
route_scan_kernel(int32_t* __restrict__ hist, int64_t nchunk, int E, int64_t* __restrict__ offsets) {
    __shared__ int64_t tot[kMaxGroups];
    const int e = threadIdx.x;
    if (e < E) {
        int64_t run = 0;
        for (int64_t c = 0; c < nchunk; ++c) {
            const int64_t idx = c * E + e;
            const int v = hist[idx];
            hist[idx] = (int32_t)run;
            run += v;
        }
        tot[e] = run;
    }
    __syncthreads();
    if (e == 0) {
        int64_t s = 0;
        for (int g = 0; g < E; ++g) {
            offsets[g] = s;
            s += tot[g];
        }
        offsets[E] = s;
    }
}

__global__ void __launch_bounds__(kChunk)
route_scatter_kernel(const int32_t* __restrict__ ids, int64_t n, int k, int E,
                     const int32_t* __restrict__ base, const int64_t* __restrict__ offsets,
                     const float* __restrict__ w, int32_t* __restrict__ row_of,
                     int32_t* __restrict__ tok_of, float* __restrict__ r_sorted) {
    __shared__ int sid[kChunk];
    const int tid = threadIdx.x;
    const int64_t i = (int64_t)blockIdx.x * kChunk + tid;
    const int e = i < n ? ids[i] : -1;
    const bool ok = e >= 0 && e < E;
    sid[tid] = ok ? e : -1;
    __syncthreads();
    if (i >= n) return;
    if (!ok) {
        row_of[i] = -1;
        return;
    }
    int rank = 0;
    for (int j = 0; j < tid; ++j) rank += sid[j] == e;
    const int64_t row = offsets[e] + base[(int64_t)blockIdx.x * E + e] + rank;
    row_of[i] = (int32_t)row;
    tok_of[row] = (int32_t)(i / k);
    if (w) r_sorted[row] = w[i];
}

__device__ __forceinline__ void unpack8_bf16(const uint4& u, float* v) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

__device__ __forceinline__ uint4 pack8_bf16(const float* v) {
    return make_uint4(bf16x2(v[0], v[1]), bf16x2(v[2], v[3]), bf16x2(v[4], v[5]),
                      bf16x2(v[6], v[7]));
}

// out[t][c..c+8) = sum_j c_tj * y[row_of[t][j]][c..c+8), fp32, j ascending,
// one rounding to bf16; rows outside [0, M) (unrouted slots) are skipped.
__global__ void __launch_bounds__(256)
combine_kernel(const uint16_t* __restrict__ y, const int32_t* __restrict__ row_of,
               const float* __restrict__ w, int64_t T, int k, int64_t H, int64_t M,
               uint16_t* __restrict__ out) {
    const int64_t n8 = H / 8;
    const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (item >= T * n8) return;
    const int64_t t = item / n8, c = (item - t * n8) * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
        const int32_t row = row_of[t * k + j];
        if (row < 0 || row >= M) continue;
        const float cw = w ? w[t * k + j] : 1.0f;
        float v[8];
        unpack8_bf16(*reinterpret_cast<const uint4*>(y + (int64_t)row * H + c), v);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(cw, v[q], acc[q]);
    }
    *reinterpret_cast<uint4*>(out + t * H + c) = pack8_bf16(acc);
}

// dy[row_of[t][j]][c..c+8) = c_tj * dout[t][c..c+8) (bf16; a plain copy of
// the bits when unweighted, which makes this the token -> sorted-row permute).
__global__ void __launch_bounds__(256)
combine_bwd_kernel(const uint16_t* __restrict__ dout, const int32_t* __restrict__ row_of,
                   const float* __restrict__ w, int64_t T, int k, int64_t H, int64_t M,
                   uint16_t* __restrict__ dy) {
    const int64_t n8 = H / 8;
    const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (item >= T * k * n8) return;
    const int64_t s = item / n8, c = (item - s * n8) * 8;
    const int32_t row = row_of[s];
    if (row < 0 || row >= M) return;
    const uint4 u = *reinterpret_cast<const uint4*>(dout + (s / k) * H + c);
    uint4 o = u;
    if (w) {
        const float cw = w[s];
        float v[8];
        unpack8_bf16(u, v);
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] *= cw;
        o = pack8_bf16(v);
    }
    *reinterpret_cast<uint4*>(dy + (int64_t)row * H + c) = o;
}

// dw[t][j] = <dout[t], y[row_of[t][j]]>: one wave per slot, each lane sums
// its columns in order, then a fixed butterfly over the 64 lanes.
__global__ void __launch_bounds__(256)
combine_dw_kernel(const uint16_t* __restrict__ dout, const uint16_t* __restrict__ y,
                  const int32_t* __restrict__ row_of, int64_t T, int k, int64_t H, int64_t M,
                  float* __restrict__ dw) {
    const int lane = threadIdx.x & 63;
    const int64_t s = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (s >= T * k) return;
    const int32_t row = row_of[s];
    float acc = 0.f;
    if (row >= 0 && row < M) {
        const uint16_t* a = dout + (s / k) * H;
        const uint16_t* b = y + (int64_t)row * H;
        for (int64_t c = (int64_t)lane * 8; c < H; c += 512) {
            float va[8], vb[8];
            unpack8_bf16(*reinterpret_cast<const uint4*>(a + c), va);
            unpack8_bf16(*reinterpret_cast<const uint4*>(b + c), vb);
#pragma unroll
            for (int q = 0; q < 8; ++q) acc = __builtin_fmaf(va[q], vb[q], acc);
        }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) acc += __shfl_xor(acc, d);
    if (lane == 0) dw[s] = acc;
}

}  // namespace

int64_t route_chunks(int64_t n) { return (n + kChunk - 1) / kChunk; }

hipError_t route_plan_scratch(int32_t** out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static int32_t* ptrs[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        // once per device, with that device current: this GPU's copy
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        ptrs[dev] = static_cast<int32_t*>(p);
    }
    *out = ptrs[dev];
    return hipSuccess;
}

hipError_t launch_router(const float* logits, int64_t T, int E, int k, int32_t* ids, float* w,
                         hipStream_t s) {
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(router_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, logits, T, E,
                       k, ids, w);
    return hipGetLastError();
}

hipError_t launch_route_plan(const int32_t* ids, int64_t T, int k, int E, const float* w,
                             int64_t* offsets, int32_t* row_of, int32_t* tok_of,
                             float* r_sorted, int32_t* hist, hipStream_t s) {
    const int64_t n = T * k;
    const int64_t nchunk = route_chunks(n);
    if (nchunk > 0) {
        hipLaunchKernelGGL(route_hist_kernel, dim3((unsigned)nchunk), dim3(kChunk), 0, s, ids, n,
                           E, hist);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(kMaxGroups), 0, s, hist, nchunk, E,
                       offsets);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || nchunk == 0) return e;
    hipLaunchKernelGGL(route_scatter_kernel, dim3((unsigned)nchunk), dim3(kChunk), 0, s, ids, n, k,
                       E, hist, offsets, w, row_of, tok_of, r_sorted);
    return hipGetLastError();
}

hipError_t launch_combine(const uint16_t* y, const int32_t* row_of, const float* w, int64_t T,
                          int k, int64_t H, int64_t M, uint16_t* out, hipStream_t s) {
    const int64_t items = T * (H / 8);
    if (items == 0) return hipSuccess;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, s, y,
                       row_of, w, T, k, H, M, out);
    return hipGetLastError();
}

hipError_t launch_combine_bwd(const uint16_t* dout, const int32_t* row_of, const float* w,
                              const uint16_t* y, int64_t T, int k, int64_t H, int64_t M,
                              uint16_t* dy, float* dw, hipStream_t s) {
    const int64_t items = T * k * (H / 8);
    if (items > 0) {
        hipLaunchKernelGGL(combine_bwd_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0,
                           s, dout, row_of, w, T, k, H, M, dy);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (dw && T * k > 0) {
        hipLaunchKernelGGL(combine_dw_kernel, dim3((unsigned)((T * k + 3) / 4)), dim3(256), 0, s,
                           dout, y, row_of, T, k, H, M, dw);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace mx
