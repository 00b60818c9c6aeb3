// MXFP8 block quantizer for gfx950: bf16 -> E4M3 codes + E8M0 scales, one
// scale per 32 values (the MXFP8 paragraphs of the German page and of the
// Portuguese page's third paragraph).  Memory-bound: each element is read
// once (2 bytes) and written once or twice (1 byte + 1/32 byte per copy).
//
// Three kernels:
//  * quant_rows_kernel  -- flat rowwise copy.  A lane converts 16 contiguous
//    values (two 16-byte loads); two neighbouring lanes hold one 32-block and
//    combine their amax with one lane swap.  Codes leave as one 16-byte store
//    per lane, so a wave moves 2 KiB in and 1 KiB out contiguously.
//  * quant_tiles_kernel -- 128-row x 64-column tile per workgroup producing
//    the rowwise copy (from registers) and the columnwise copy (through an
//    LDS transpose of bf16 row pairs) from one read of the input.  The
//    columnwise copy is transposed ([C][ld], blocks of 32 rows); row groups
//    (experts) start new blocks and are padded with zero codes to a multiple
//    of 128 rows, so every tile lies inside one group.
//  * quant_tiles128_kernel -- the same on 128 x 128 tiles (C % 128 == 0, every
//    operand of the MLP path), computing on the bf16 pairs as loaded.
#include "internal.h"
#include "mx_device.h"

namespace mx {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (the source is read exactly once)
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
// The same through a buffer descriptor: offsets at or past the range read
// zeros, so a masked load needs no branch.
__device__ __forceinline__ uint4 load_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2 /* nt */);
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

__device__ __forceinline__ uint4 encode16(const float* v, float inv) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        w[i] = e4m3x4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3], inv);
    return make_uint4(w[0], w[1], w[2], w[3]);
}

__global__ void __launch_bounds__(1024)
padded_offsets_kernel(const int64_t* __restrict__ offs, int G,
                      int64_t* __restrict__ poff) {
    __shared__ int64_t s[1024];
    const int t = threadIdx.x;
    int64_t v = 0;
    if (t < G) {
        int64_t n = offs[t + 1] - offs[t];
        n = n < 0 ? 0 : n;
        v = (n + kTokenAlign - 1) / kTokenAlign * kTokenAlign;
    }
    s[t] = v;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {       // inclusive Hillis-Steele scan
        int64_t add = t >= d ? s[t - d] : 0;
        __syncthreads();
        s[t] += add;
        __syncthreads();
    }
    if (t == 0) poff[0] = 0;
    if (t < G) poff[t + 1] = s[t];
}

__global__ void __launch_bounds__(256)
quant_rows_kernel(const uint16_t* __restrict__ x, int64_t nchunk, int64_t C, bool tiled,
                  uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nchunk; i += stride) {
        const uint4* src = reinterpret_cast<const uint4*>(x + i * 16);
        uint4 a = load_stream(src);
        uint4 b = load_stream(src + 1);
        float v[16];
        unpack8(a, v);
        unpack8(b, v + 8);
        uint32_t m = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) m = max(m, abs_bits(v[j]));
        // chunks 2k and 2k+1 (one 32-block) sit in neighbouring lanes
        m = max(m, (uint32_t)__shfl_xor((int)m, 1));
        const uint32_t sc = scale_code_from_amax_bits(m);
        const float inv = inv_scale_from_code(sc);
        store_nt(reinterpret_cast<uint4*>(codes) + i, encode16(v, inv));
        if (!(i & 1)) {
            const int64_t blk = i >> 1, bpr = C / 32;       // block index, blocks per row
            scales[tiled ? tiled_scale_offset(blk / bpr, blk % bpr, C) : blk] = (uint8_t)sc;
        }
    }
}

// DPP helpers: lane i of a quad reads lane (pattern) of the same quad
#define MXQ_DPP(x, ctrl) ((uint32_t)__builtin_amdgcn_update_dpp(0, (int)(x), (ctrl), 0xF, 0xF, false))

__device__ __forceinline__ uint2 encode8(const float* v, float inv) {
    return make_uint2(e4m3x4(v[0], v[1], v[2], v[3], inv), e4m3x4(v[4], v[5], v[6], v[7], inv));
}

// ---- bf16 pairs, two values per dword ---------------------------------------
// The 128-column tile kernel works on the input's bf16 pairs as they are
// loaded, never widening them to fp32: a finite bf16 magnitude (the pattern
// with the sign cleared) orders like an unsigned integer, so the block amax is
// a packed 16-bit max, and its bf16 exponent field is the fp32 one (code =
// max(exp - 8, 0), as for fp32).  448 * 2^X is the bf16 pattern
// ((c + 8) << 7) | 0x60 (1.75 * 2^(c - 119)), so the saturation is a packed
// 16-bit min on magnitudes with the sign put back, and v_cvt_scalef32_pk_fp8_bf16
// divides by the block scale 2^X (exact) and rounds to nearest even.  Equal,
// code for code, to the fp32 path of the other kernels (x * 2^-X clamped to
// +-448, v_cvt_pk_fp8_f32), checked on the device for every finite bf16
// pattern at every scale code 0 .. 246.
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(v2u16, a),
                                                                  __builtin_bit_cast(v2u16, b)));
}
__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(v2u16, a),
                                                                  __builtin_bit_cast(v2u16, b)));
}
// Largest magnitude of the 2N bf16 values in w[0 .. N), as a 15-bit pattern.
template <int N>
__device__ __forceinline__ uint32_t bf16_amax(const uint32_t* w) {
    uint32_t m = w[0] & 0x7fff7fffu;
#pragma unroll
    for (int i = 1; i < N; ++i) m = pk_max_u16(m, w[i] & 0x7fff7fffu);
    return max(m & 0xffffu, m >> 16);
}
// Scale of a block from its amax pattern m: code c, the limit 448 * 2^X as a
// bf16 pattern in both halves of lim2, and 2^X as fp32.
struct Bf16Scale {
    uint32_t code, lim2;
    float scale;
};
__device__ __forceinline__ Bf16Scale bf16_scale(uint32_t m) {
    const uint32_t e = max(m >> 7, 8u);           // biased exponent, floored at X = -127
    const uint32_t lim = (e << 7) | 0x60u;
    return {e - 8u, lim | (lim << 16), scale_from_code(e - 8u)};
}
// E4M3 codes of the four values in dwords w0, w1 (bytes in element order).
// The first conversion writes the low half and leaves the rest of its first
// operand, w0's clamped bits, to the second.
__device__ __forceinline__ uint32_t bf16_e4m3x4(uint32_t w0, uint32_t w1, const Bf16Scale& s) {
    const uint32_t c0 = (w0 & 0x80008000u) | pk_min_u16(w0 & 0x7fff7fffu, s.lim2);
    const uint32_t c1 = (w1 & 0x80008000u) | pk_min_u16(w1 & 0x7fff7fffu, s.lim2);
    v2s16 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(__builtin_bit_cast(v2s16, c0),
                                                        __builtin_bit_cast(v2bf16, c0), s.scale,
                                                        false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(v2bf16, c1), s.scale, true);
    return __builtin_bit_cast(uint32_t, r);
}

// 128 rows x 64 columns per workgroup of 256 lanes.  Loads: lane t reads the
// 16-byte chunk (t & 7) of row pair (t >> 3), so every load instruction moves
// eight full 128-byte row segments.  Rowwise blocks of 32 columns are four
// neighbouring lanes (a DPP quad).  The columnwise copy goes through an LDS
// tile that holds bf16 row pairs transposed, [column][row pair] with a row
// stride of 65 dwords: both the writes (eight columns x eight row pairs per
// instruction) and the reads (16 columns x 4 blocks) hit 64 distinct banks.
__global__ void __launch_bounds__(256)
quant_tiles_kernel(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                   const int64_t* __restrict__ offs,
                   const int64_t* __restrict__ poff, int G,
                   uint8_t* __restrict__ rc, uint8_t* __restrict__ rs,
                   uint8_t* __restrict__ cc, uint8_t* __restrict__ cs,
                   int64_t ld, bool tiled, const int32_t* __restrict__ gather,
                   int64_t src_rows) {
    constexpr int kStride = 65;                      // dwords per column of the tile
    __shared__ uint32_t tile[64 * kStride];
    const int64_t b = blockIdx.z;
    const int64_t p0 = (int64_t)blockIdx.y * 128;    // start in the padded axis
    int64_t src0, valid;
    if (offs) {
        if (p0 >= poff[G]) return;
        // last group g < G with poff[g] <= p0 (skips empty groups)
        int lo = 0, hi = G - 1;
        while (lo < hi) {
            int mid = (lo + hi + 1) >> 1;
            if (poff[mid] <= p0) lo = mid; else hi = mid - 1;
        }
        src0 = offs[lo] + (p0 - poff[lo]);
        valid = offs[lo + 1] - src0;
    } else {
        src0 = p0;
        valid = R - p0;
    }
    valid = valid < 0 ? 0 : (valid > 128 ? 128 : valid);

    const int t = threadIdx.x;
    const int c8 = t & 7, rp = t >> 3;
    const int64_t col0 = (int64_t)blockIdx.x * 64;
    const int64_t ccol = col0 + c8 * 8;               // this lane's 8 columns
    const bool colok = ccol < C;                      // C % 32 == 0: whole chunk in or out
    // the tile's valid rows as one buffer: rows at or past `valid` and
    // columns past C read as zeros (the caller keeps 256 * C below 2^31, so
    // the byte offsets fit 32 bits).  With a gather map, row r of the
    // tile is source row gather[src0 + r] of x (src_rows rows, whose bytes
    // the caller keeps below 2^31).
    const __amdgpu_buffer_rsrc_t xr = gather
        ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), (short)0,
                                            (int)(src_rows * C * 2), 0x00020000)
        : __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x + (b * R + src0) * C),
                                            (short)0, (int)(valid * C * 2), 0x00020000);

    // All four row loads first, without branches: issued back to back, they
    // are in flight together instead of each pair waiting behind the previous
    // pair's stores.
    uint4 wl[2][2];
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = it * 64 + 2 * rp + h;
            uint32_t off;
            if (gather) {
                const int32_t sr = r < valid ? gather[src0 + r] : -1;
                off = colok && sr >= 0 && sr < src_rows
                          ? ((uint32_t)sr * (uint32_t)C + (uint32_t)ccol) * 2u : 0x7ffffff0u;
            } else {
                off = colok ? ((uint32_t)r * (uint32_t)C + (uint32_t)ccol) * 2u : 0x7ffffff0u;
            }
            wl[it][h] = load_stream(xr, off);
        }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int r0 = it * 64 + 2 * rp;
        uint4 w[2];
        float v[2][8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            w[h] = wl[it][h];
            unpack8(w[h], v[h]);
        }
        if (rc) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t m = 0;
#pragma unroll
                for (int j = 0; j < 8; ++j) m = max(m, abs_bits(v[h][j]));
                m = max(m, MXQ_DPP(m, 0xB1));         // quad_perm [1,0,3,2]
                m = max(m, MXQ_DPP(m, 0x4E));         // quad_perm [2,3,0,1]
                const uint32_t sc = scale_code_from_amax_bits(m);
                const uint32_t sc_hi = MXQ_DPP(sc, 0x104);   // row_shl:4 -- the next block's
                const int64_t row = b * R + src0 + r0 + h;
                if (colok && r0 + h < valid) {
                    store_nt(rc + row * C + ccol, encode8(v[h], inv_scale_from_code(sc)));
                    if (c8 == 0) {
                        // the row's two scale bytes; one 16-bit store when aligned
                        // (always in the tiled layout: col0 / 32 is even)
                        uint8_t* d = rs + (tiled ? tiled_scale_offset(row, col0 / 32, C)
                                                 : row * (C / 32) + col0 / 32);
                        const bool two = col0 + 64 <= C;
                        if (two && (tiled || !((C / 32) & 1))) {
                            *reinterpret_cast<uint16_t*>(d) = (uint16_t)(sc | (sc_hi << 8));
                        } else {
                            d[0] = (uint8_t)sc;
                            if (two) d[1] = (uint8_t)sc_hi;
                        }
                    }
                }
            }
        }
        if (cc) {
            const uint32_t a4[4] = {w[0].x, w[0].y, w[0].z, w[0].w};
            const uint32_t b4[4] = {w[1].x, w[1].y, w[1].z, w[1].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                tile[(c8 * 8 + 2 * i) * kStride + it * 32 + rp] = __builtin_amdgcn_perm(b4[i], a4[i], 0x05040100u);
                tile[(c8 * 8 + 2 * i + 1) * kStride + it * 32 + rp] = __builtin_amdgcn_perm(b4[i], a4[i], 0x07060302u);
            }
        }
    }
    if (!cc) return;
    __syncthreads();

    const int col = t >> 2, blk = t & 3;
    float v[32];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t d = tile[col * kStride + blk * 16 + i];
        v[2 * i] = __uint_as_float(d << 16);
        v[2 * i + 1] = __uint_as_float(d & 0xffff0000u);
    }
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) m = max(m, abs_bits(v[i]));
    const uint32_t sc = scale_code_from_amax_bits(m);
    const float inv = inv_scale_from_code(sc);
    // the four blocks of a column sit in one quad: gather their scales
    const uint32_t s1 = MXQ_DPP(sc, 0x55), s2 = MXQ_DPP(sc, 0xAA), s3 = MXQ_DPP(sc, 0xFF);
    if (col0 + col >= C) return;
    const int64_t crow = b * C + col0 + col;
    uint4* dst = reinterpret_cast<uint4*>(cc + crow * ld + p0 + blk * 32);
    store_nt(dst, encode16(v, inv));
    store_nt(dst + 1, encode16(v + 16, inv));
    if (blk == 0)
        *reinterpret_cast<uint32_t*>(cs + (tiled ? tiled_scale_offset(crow, p0 / 32, ld)
                                                 : crow * (ld / 32) + p0 / 32)) =
            sc | (s1 << 8) | (s2 << 16) | (s3 << 24);
}

// 128 rows x 128 columns per workgroup of 256 lanes, for C % 128 == 0 (every
// operand of the MLP path): twice the bytes of quant_tiles_kernel's tile.
// Lane t reads the 16-byte chunk (t & 15) of rows 2 (t >> 4) + h of each of
// four 32-row slabs, so each load instruction moves 16 whole 256-byte row
// segments and every lane has eight loads in flight; its 8-byte rowwise code
// stores cover whole 128-byte lines (16 lanes per row).  A row's four 32-blocks
// sit in lanes c16 = 0, 4, 8, 12 of its 16-lane row: one dword of scale codes
// per row.  The columnwise copy goes through the same kind of LDS transpose,
// [column][row pair] with a row stride of 65 dwords.  Codes leave by ordinary
// stores, not nontemporal ones: the GEMM that reads them next then finds
// part of them in the caches (measured in the MLP step: the token-sized
// launches 0.118 -> 0.096 ms, the weight launches unchanged).
__global__ void __launch_bounds__(256)
quant_tiles128_kernel(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                      const int64_t* __restrict__ offs,
                      const int64_t* __restrict__ poff, int G,
                      uint8_t* __restrict__ rc, uint8_t* __restrict__ rs,
                      uint8_t* __restrict__ cc, uint8_t* __restrict__ cs,
                      int64_t ld, bool tiled, const int32_t* __restrict__ gather,
                      int64_t src_rows) {
    constexpr int kStride = 65;
    __shared__ uint32_t tile[128 * kStride];
    const int64_t b = blockIdx.z;
    const int64_t p0 = (int64_t)blockIdx.y * 128;
    int64_t src0, valid;
    if (offs) {
        if (p0 >= poff[G]) return;
        int lo = 0, hi = G - 1;
        while (lo < hi) {
            int mid = (lo + hi + 1) >> 1;
            if (poff[mid] <= p0) lo = mid; else hi = mid - 1;
        }
        src0 = offs[lo] + (p0 - poff[lo]);
        valid = offs[lo + 1] - src0;
    } else {
        src0 = p0;
        valid = R - p0;
    }
    valid = valid < 0 ? 0 : (valid > 128 ? 128 : valid);

    const int t = threadIdx.x;
    const int c16 = t & 15, rg = t >> 4;
    const int64_t col0 = (int64_t)blockIdx.x * 128;
    // The tiled scale layout pads the rows to a multiple of 32: the first row
    // tile of each column tile writes code 0 (2^-127, a finite scale) into the
    // padding rows R .. of its four K blocks, so that a GEMM tile reading
    // rows past R (their codes read as zero through the range checks)
    // accumulates exact zeros there.
    // (one batch only: batched copies continue in the next batch's rows)
    if (tiled && rc && gridDim.z == 1 && blockIdx.y == 0 && t < (int)((32 - (R & 31)) & 31))
        *reinterpret_cast<uint32_t*>(rs + tiled_scale_offset(R + t, col0 / 32, C)) = 0u;
    const int64_t ccol = col0 + c16 * 8;              // this lane's 8 columns (all < C)
    const __amdgpu_buffer_rsrc_t xr = gather
        ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), (short)0,
                                            (int)(src_rows * C * 2), 0x00020000)
        : __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x + (b * R + src0) * C),
                                            (short)0, (int)(valid * C * 2), 0x00020000);
    uint4 wl[4][2];
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = it * 32 + 2 * rg + h;
            uint32_t off;
            if (gather) {
                const int32_t sr = r < valid ? gather[src0 + r] : -1;
                off = sr >= 0 && sr < src_rows ? ((uint32_t)sr * (uint32_t)C + (uint32_t)ccol) * 2u
                                               : 0x7ffffff0u;
            } else {
                off = ((uint32_t)r * (uint32_t)C + (uint32_t)ccol) * 2u;
            }
            wl[it][h] = load_stream(xr, off);
        }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int r0 = it * 32 + 2 * rg;
        if (rc) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t w[4] = {wl[it][h].x, wl[it][h].y, wl[it][h].z, wl[it][h].w};
                uint32_t m = bf16_amax<4>(w);
                m = max(m, MXQ_DPP(m, 0xB1));         // quad_perm [1,0,3,2]
                m = max(m, MXQ_DPP(m, 0x4E));         // quad_perm [2,3,0,1]
                const Bf16Scale bs = bf16_scale(m);
                const uint32_t sc = bs.code;
                // the row's other three blocks: lanes c16 + 4, + 8, + 12
                const uint32_t s1 = MXQ_DPP(sc, 0x104), s2 = MXQ_DPP(sc, 0x108),
                               s3 = MXQ_DPP(sc, 0x10C);   // row_shl:4, 8, 12
                const int64_t row = b * R + src0 + r0 + h;
                if (r0 + h < valid) {
                    *reinterpret_cast<uint2*>(rc + row * C + ccol) =
                        make_uint2(bf16_e4m3x4(w[0], w[1], bs), bf16_e4m3x4(w[2], w[3], bs));
                    if (c16 == 0) {
                        const uint32_t w4 = sc | (s1 << 8) | (s2 << 16) | (s3 << 24);
                        if (tiled) {
                            *reinterpret_cast<uint32_t*>(rs + tiled_scale_offset(row, col0 / 32, C)) = w4;
                        } else {
                            uint8_t* d = rs + row * (C / 32) + col0 / 32;
                            d[0] = (uint8_t)sc; d[1] = (uint8_t)s1;
                            d[2] = (uint8_t)s2; d[3] = (uint8_t)s3;
                        }
                    }
                }
            }
        }
        if (cc) {
            const uint4 w0 = wl[it][0], w1 = wl[it][1];
            const uint32_t a4[4] = {w0.x, w0.y, w0.z, w0.w};
            const uint32_t b4[4] = {w1.x, w1.y, w1.z, w1.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                tile[(c16 * 8 + 2 * i) * kStride + it * 16 + rg] = __builtin_amdgcn_perm(b4[i], a4[i], 0x05040100u);
                tile[(c16 * 8 + 2 * i + 1) * kStride + it * 16 + rg] = __builtin_amdgcn_perm(b4[i], a4[i], 0x07060302u);
            }
        }
    }
    if (!cc) return;
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        const int col = pass * 64 + (t >> 2), blk = t & 3;
        uint32_t d[16];                      // rows 2i, 2i + 1 of the block in dword i
#pragma unroll
        for (int i = 0; i < 16; ++i) d[i] = tile[col * kStride + blk * 16 + i];
        const Bf16Scale bs = bf16_scale(bf16_amax<16>(d));
        const uint32_t sc = bs.code;
        const uint32_t s1 = MXQ_DPP(sc, 0x55), s2 = MXQ_DPP(sc, 0xAA), s3 = MXQ_DPP(sc, 0xFF);
        const int64_t crow = b * C + col0 + col;
        uint4* dst = reinterpret_cast<uint4*>(cc + crow * ld + p0 + blk * 32);
        u32x4 o0 = {bf16_e4m3x4(d[0], d[1], bs), bf16_e4m3x4(d[2], d[3], bs),
                    bf16_e4m3x4(d[4], d[5], bs), bf16_e4m3x4(d[6], d[7], bs)};
        u32x4 o1 = {bf16_e4m3x4(d[8], d[9], bs), bf16_e4m3x4(d[10], d[11], bs),
                    bf16_e4m3x4(d[12], d[13], bs), bf16_e4m3x4(d[14], d[15], bs)};
        // Both halves of the lane's 32 bytes are computed before either store
        // issues, so the two stores leave back to back and the block's four
        // lanes fill each 128-byte line at once; with the second half computed
        // between them (the compiler's order) each store wrote half lines and
        // the kernel took a quarter longer (measured).
        asm volatile("" : "+v"(o0), "+v"(o1));
        dst[0] = make_uint4(o0.x, o0.y, o0.z, o0.w);
        dst[1] = make_uint4(o1.x, o1.y, o1.z, o1.w);
        if (blk == 0)
            *reinterpret_cast<uint32_t*>(cs + (tiled ? tiled_scale_offset(crow, p0 / 32, ld)
                                                     : crow * (ld / 32) + p0 / 32)) =
                sc | (s1 << 8) | (s2 << 16) | (s3 << 24);
    }
}

// Row padding: rows of n bytes (stride n) become rows of np bytes (stride np),
// bytes n .. np - 1 set to fill.  One thread per 16 output bytes: one 16-byte
// copy where both strides are multiples of 16 and the chunk lies within the
// source row, else byte by byte (scale rows, the chunk at the seam).
__global__ void __launch_bounds__(256) pad_rows_kernel(const uint8_t* __restrict__ src,
                                                       int64_t rows, int64_t n,
                                                       uint8_t* __restrict__ dst, int64_t np,
                                                       uint32_t fill) {
    const int64_t chunks = (np + 15) / 16;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= rows * chunks) return;
    const int64_t row = i / chunks, c = (i - row * chunks) * 16;
    const uint8_t* sr = src + row * n;
    uint8_t* dr = dst + row * np + c;
    if (n % 16 == 0 && np % 16 == 0 && c + 16 <= n) {
        *reinterpret_cast<uint4*>(dr) = *reinterpret_cast<const uint4*>(sr + c);
        return;
    }
    for (int b = 0; b < 16 && c + b < np; ++b) dr[b] = c + b < n ? sr[c + b] : (uint8_t)fill;
}

}  // namespace

hipError_t launch_padded_offsets(const int64_t* offs, int G, int64_t* poff,
                                 hipStream_t s) {
    hipLaunchKernelGGL(padded_offsets_kernel, dim3(1), dim3(1024), 0, s, offs, G, poff);
    return hipGetLastError();
}

hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int64_t C,
                             uint8_t* codes, uint8_t* scales, bool tiled, hipStream_t s) {
    const int64_t nchunk = rows * C / 16;
    if (nchunk == 0) return hipSuccess;
    int64_t blocks = (nchunk + 255) / 256;
    const int64_t cap = (int64_t)device_cu_count() * 16;
    if (blocks > cap) blocks = cap;
    hipLaunchKernelGGL(quant_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       x, nchunk, C, tiled, codes, scales);
    return hipGetLastError();
}

hipError_t launch_quant_tiles(const uint16_t* x, int64_t batch, int64_t R,
                              int64_t C, const int64_t* offs,
                              const int64_t* poff, int G, int64_t row_bound,
                              uint8_t* rc, uint8_t* rs, uint8_t* cc,
                              uint8_t* cs, int64_t ld, bool tiled, hipStream_t s,
                              const int32_t* gather, int64_t src_rows) {
    const int64_t ytiles = offs ? row_bound / 128 : (R + 127) / 128;
    if (ytiles == 0 || C == 0 || batch == 0) return hipSuccess;
    if (C % 128 == 0) {
        dim3 grid((unsigned)(C / 128), (unsigned)ytiles, (unsigned)batch);
        hipLaunchKernelGGL(quant_tiles128_kernel, grid, dim3(256), 0, s, x, R, C, offs,
                           poff, G, rc, rs, cc, cs, ld, tiled, gather, src_rows);
        return hipGetLastError();
    }
    dim3 grid((unsigned)((C + 63) / 64), (unsigned)ytiles, (unsigned)batch);
    hipLaunchKernelGGL(quant_tiles_kernel, grid, dim3(256), 0, s, x, R, C, offs,
                       poff, G, rc, rs, cc, cs, ld, tiled, gather, src_rows);
    return hipGetLastError();
}

hipError_t launch_pad_rows(const uint8_t* src, int64_t rows, int64_t n, uint8_t* dst, int64_t np,
                           uint8_t fill, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    const int64_t threads = rows * ((np + 15) / 16);
    hipLaunchKernelGGL(pad_rows_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                       src, rows, n, dst, np, (uint32_t)fill);
    return hipGetLastError();
}

}  // namespace mx
