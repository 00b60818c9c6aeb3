// Per-tensor scaled FP8 (E4M3) quantizer for gfx950: the plain FP8 format
// that the German page's paragraph on activation memory names beside MXFP8.
// The page gives no recipe; here every expert's slice of a grouped operand
// (a row group of the token-sorted activations, one matrix of the stacked
// weights) is one tensor with one fp32 scale, scale = 448 / amax (an IEEE
// division; amax 0 gives 1, an overflowing quotient the largest finite
// fp32), and a code is the E4M3 rounding (nearest even, saturating) of the
// fp32 product x * scale.  scale_inv = 1 / scale is what the GEMM multiplies
// its fp32 accumulators by.
//
// Three launches:
//  * amax_init -- amax[g] = 0;
//  * amax      -- about two workgroups per CU, each streaming one contiguous
//                 range of rows; the range is cut at group boundaries and each
//                 piece (contiguous bytes) is reduced to one atomic max on its
//                 group (fp32 bit patterns of non-negative values order like
//                 unsigned integers).  Device-scope atomics on one cache line
//                 serialize (about 12 ns each here), so their number is kept
//                 to about the number of workgroups plus the number of groups;
//  * cast      -- 128-row x 64-column tiles (lane t reads 16 bytes, chunk
//                 t & 7, of rows t >> 3 + 32 i, so every load instruction
//                 moves 32 full 128-byte row segments): codes of every row from
//                 its group's scale; the first workgroup also writes scale_inv
//                 of every group.
// The input is read twice (the scale needs the amax of the whole tensor
// first): 5 bytes per element moved against 4 + 1/16 for the MXFP8 tiles.
#include <float.h>

#include "internal.h"
#include "mx_device.h"

namespace mx {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2 /* nt */);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void unpack8(const uint4& u, float* v) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

// Group of a row: row / R for a batch of matrices (offs == nullptr), else the
// g with offs[g] <= row < offs[g+1] (the last g with offs[g] <= row, which
// skips empty groups), or -1 outside [offs[0], offs[G]).
__device__ __forceinline__ int group_of(int64_t row, const int64_t* offs, int G, int64_t R) {
    if (!offs) return (int)(row / R);
    if (row < offs[0] || row >= offs[G]) return -1;
    int lo = 0, hi = G - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (offs[mid] <= row) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// scale = 448 / amax in fp32 (amax as its bit pattern)
__device__ __forceinline__ float tensor_scale(uint32_t amax_bits) {
    const float a = __uint_as_float(amax_bits);
    if (a == 0.0f) return 1.0f;
    const float s = __fdiv_rn(448.0f, a);
    return s > FLT_MAX ? FLT_MAX : s;
}

// The tile's four 16-byte loads (rows past `rows` and columns past C read
// as zeros), issued back to back.
struct TileLoad {
    uint4 w[4];
    int64_t row0, col;
    bool colok;
};
__device__ __forceinline__ TileLoad load_tile(const uint16_t* x, int64_t rows, int64_t C) {
    TileLoad L;
    const int t = threadIdx.x;
    L.row0 = (int64_t)blockIdx.x * 128;
    L.col = (int64_t)blockIdx.y * 64 + (t & 7) * 8;
    L.colok = L.col < C;                               // C % 32 == 0: whole chunks
    const int64_t valid = min((int64_t)128, rows - L.row0);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(x + L.row0 * C), (short)0, (int)(valid * C * 2), 0x00020000);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (t >> 3) + 32 * i;
        const uint32_t off =
            L.colok ? ((uint32_t)r * (uint32_t)C + (uint32_t)L.col) * 2u : 0x7ffffff0u;
        L.w[i] = load_nt(xr, off);
    }
    return L;
}

__global__ void __launch_bounds__(1024)
amax_init_kernel(uint32_t* __restrict__ amax, int G) {
    if ((int)threadIdx.x < G) amax[threadIdx.x] = 0u;
}

// First row of group g (g <= G): offs[g], or g * R for matrices.
__device__ __forceinline__ int64_t group_start(int g, const int64_t* offs, int64_t R) {
    return offs ? offs[g] : (int64_t)g * R;
}

__global__ void __launch_bounds__(256)
amax_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t C,
            const int64_t* __restrict__ offs, int G, int64_t R, int64_t rows_per_block,
            uint32_t* __restrict__ amax) {
    __shared__ uint32_t red[4];
    const int t = threadIdx.x;
    // this workgroup's rows, clipped to the rows the groups cover
    const int64_t lo = max((int64_t)blockIdx.x * rows_per_block, group_start(0, offs, R));
    const int64_t hi = min(min((int64_t)(blockIdx.x + 1) * rows_per_block, rows),
                           group_start(G, offs, R));
    if (lo >= hi) return;                                   // the whole workgroup
    const int g_lo = group_of(lo, offs, G, R), g_hi = group_of(hi - 1, offs, G, R);
    for (int g = g_lo; g <= g_hi; ++g) {
        const int64_t a = max(lo, group_start(g, offs, R));
        const int64_t b = min(hi, group_start(g + 1, offs, R));
        if (a >= b) continue;                               // empty group (uniform)
        // rows [a, b) are (b - a) * C contiguous values: 16-byte chunks,
        // four loads in flight per lane
        const uint4* src = reinterpret_cast<const uint4*>(x + a * C);
        const int64_t n = (b - a) * C / 8;
        uint32_t m = 0u;
        int64_t i = t;
        for (; i + 3 * 256 < n; i += 4 * 256) {
            uint4 w[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) w[u] = load_nt(src + i + u * 256);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float v[8];
                unpack8(w[u], v);
#pragma unroll
                for (int j = 0; j < 8; ++j) m = max(m, abs_bits(v[j]));
            }
        }
        for (; i < n; i += 256) {
            float v[8];
            unpack8(load_nt(src + i), v);
#pragma unroll
            for (int j = 0; j < 8; ++j) m = max(m, abs_bits(v[j]));
        }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, d));
        if ((t & 63) == 0) red[t >> 6] = m;
        __syncthreads();
        if (t == 0) atomicMax(&amax[g], max(max(red[0], red[1]), max(red[2], red[3])));
        __syncthreads();                                    // red is reused by the next group
    }
}

__global__ void __launch_bounds__(256)
cast_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t C,
            const int64_t* __restrict__ offs, int G, int64_t R,
            const uint32_t* __restrict__ amax, uint8_t* __restrict__ codes,
            float* __restrict__ scale_inv) {
    const TileLoad L = load_tile(x, rows, C);
    const int t = threadIdx.x;
    if (blockIdx.x == 0 && blockIdx.y == 0)
        for (int g = t; g < G; g += 256) scale_inv[g] = __fdiv_rn(1.0f, tensor_scale(amax[g]));
    if (!L.colok || L.row0 >= rows) return;
    // one group for the whole tile (the usual case): one lookup, one scale
    const int gf = group_of(L.row0, offs, G, R);
    const int gl = group_of(min(L.row0 + 127, rows - 1), offs, G, R);
    const bool one = gf == gl && gf >= 0;
    const float s_one = one ? tensor_scale(amax[gf]) : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t row = L.row0 + (t >> 3) + 32 * i;
        if (row >= rows) break;
        const int g = one ? gf : group_of(row, offs, G, R);
        if (g < 0) continue;
        const float s = one ? s_one : tensor_scale(amax[g]);
        float v[8];
        unpack8(L.w[i], v);
        store_nt(codes + row * C + L.col, make_uint2(e4m3x4(v[0], v[1], v[2], v[3], s),
                                                     e4m3x4(v[4], v[5], v[6], v[7], s)));
    }
}

}  // namespace

hipError_t launch_fp8_tensor_quant(const uint16_t* x, int64_t rows, int64_t C,
                                   const int64_t* offs, int G, int64_t R, uint32_t* amax,
                                   uint8_t* codes, float* scale_inv, hipStream_t s) {
    hipLaunchKernelGGL(amax_init_kernel, dim3(1), dim3(1024), 0, s, amax, G);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (rows > 0 && C > 0) {
        // about two workgroups per CU, each with at least 16 KiB of input
        int64_t nb = min((int64_t)2 * device_cu_count(), (rows * C + 8191) / 8192);
        nb = max(nb, (int64_t)1);
        const int64_t rpb = (rows + nb - 1) / nb;
        nb = (rows + rpb - 1) / rpb;
        hipLaunchKernelGGL(amax_kernel, dim3((unsigned)nb), dim3(256), 0, s, x, rows, C, offs, G,
                           R, rpb, amax);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const dim3 grid((unsigned)((rows + 127) / 128), (unsigned)((C + 63) / 64));
        hipLaunchKernelGGL(cast_kernel, grid, dim3(256), 0, s, x, rows, C, offs, G, R,
                           (const uint32_t*)amax, codes, scale_inv);
    } else {
        // nothing to cast: scale_inv of every (empty) group from its zero amax
        hipLaunchKernelGGL(cast_kernel, dim3(1, 1), dim3(256), 0, s, x, (int64_t)0, C, offs, G,
                           R, (const uint32_t*)amax, codes, scale_inv);
    }
    return hipGetLastError();
}

}  // namespace mx
