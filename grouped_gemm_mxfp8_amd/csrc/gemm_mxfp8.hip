// Persistent grouped GEMM on gfx950 block-scaled FP8 MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4, E4M3 operands, one E8M0 scale per 32
// values along K on both sides).
//
// This one kernel body runs every GEMM of the MoE expert path (GroupedLinear:
// all experts in one launch driven by per-expert token counts -- German page,
// the paragraph on fragmented expert execution; the GroupedMLP forward and
// backward with MXFP8 in both passes -- Portuguese page, third and fourth
// paragraphs):
//   * row-grouped  (forward and data gradients): group g owns output rows
//     [off[g], off[g+1]) and its own B (expert weights); K is shared.
//   * k-grouped    (weight gradients): group g contracts over its own padded
//     token range [poff[g], poff[g+1]) and owns its own output matrix.
// Both operands are K-major MXFP8 (codes [rows][ld], scales [rows][ld/32]);
// the columnwise (transposed) copies make the data- and weight-gradient GEMMs
// the same "A . B^T" form.
//
// Tiling: 256 x 256 output tile per workgroup of 4 waves (2 x 2), each wave
// 128 x 128 = 8 x 8 MFMA blocks of 16 x 16 with fp32 accumulators; K step 128
// (one MFMA deep).  Operand tiles are staged through LDS in two buffers with
// one barrier per K step; 16-byte chunks of each 128-byte LDS row are XOR
// swizzled by (row & 7) so the fragment reads of 8 neighbouring rows hit
// distinct banks.  Global reads use buffer resources whose range check
// returns zeros past the last valid row, which handles ragged expert tails
// without branches.  The grid is persistent (one workgroup per CU); tiles are
// walked in bands of 8 M-tiles so that the 32 tiles one XCD runs at a time
// share 8 A panels and 4 B panels in that XCD's L2, and weight-gradient
// groups run longest-K first.  Plain-store tiles run as a chain per
// workgroup: a tile's last two K steps load the next tile's first two, and
// its output leaves straight from the registers (whole 128-byte lines per
// store) while those land, so neither the first loads nor the output stores
// of a tile stand between two tiles' MFMAs.
#include <utility>

#include "internal.h"
#include "mx_device.h"

namespace mx {
namespace {

constexpr int BM = 256, BN = 256, BK = 128, NTHREADS = 256;
constexpr int BAND = 8;
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer, dword format

struct GemmSmem {
    uint8_t a[2][BM * BK];
    uint8_t b[2][BN * BK];
    uint32_t as[2][BM];
    uint32_t bs[2][BN];
};

typedef int v4i __attribute__((ext_vector_type(4)));

// Raw buffer resource (no stride, dword format): base address, byte range
// (accesses at or past it read as zero).
__device__ __forceinline__ v4i make_rsrc(const void* p, int64_t bytes) {
    const int32_t n = bytes > 0x7fffffff ? 0x7fffffff : (int32_t)(bytes < 0 ? 0 : bytes);
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    return v4i{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), n, (int)kRsrcWord3};
}

// Scale source of one operand for one tile: descriptor, this lane's offset
// (its row), and the scalar offset of K step ks = s0 + ks * sstep.  Row-major
// scales put the tile's K range in the descriptor; K-step tiled scales (one
// 128-byte line per 32 rows and K step) start the descriptor at the row group
// of the first row and reach the step through the scalar offset.
struct ScaleSrc {
    v4i rsrc;
    uint32_t voff, s0, sstep;
};
// Four E8M0 codes 127 (scale 1): the scale source of an operand without
// block scales.  Every lane reads this one dword at every K step.
__device__ const uint32_t kUnitScales = 0x7f7f7f7fu;

// UNIT: the plain-store kernel, whose operands may come without block
// scales (scales == nullptr); the fused kernels always have them.
template <bool UNIT>
__device__ __forceinline__ ScaleSrc scale_src(const uint8_t* scales, int64_t ld, bool tiled,
                                              int64_t row0, int64_t rvalid, int64_t lane_row,
                                              int64_t klo, int64_t K) {
    if constexpr (UNIT) {
        if (!scales) return {make_rsrc(&kUnitScales, 4), 0u, 0u, 0u};
    }
    if (!tiled) {
        const int64_t lds = ld / 32;
        return {make_rsrc(scales + row0 * lds + klo / 32, (rvalid - 1) * lds + K / 32),
                (uint32_t)(lane_row * lds), 0u, 4u};
    }
    const int64_t r0 = row0 & 31, last = r0 + rvalid - 1, rel = r0 + lane_row;
    return {make_rsrc(scales + (row0 >> 5) * ld, ((last >> 5) + 1) * ld),
            (uint32_t)((rel >> 5) * ld + (rel & 31) * 4), (uint32_t)(klo >> 7) * 128u, 128u};
}

// LDS byte address of a __shared__ location.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// LDS byte address of byte off of stage st of one GemmSmem member, from the
// region's LDS base taken once per tile: casting a generic pointer to LDS
// per load costs a 64-bit add and a null test each, which in the main loops
// adds some 70 scalar instructions per step.
enum SmemPart { kPartA, kPartB, kPartAs, kPartBs };
template <SmemPart PART>
__device__ __forceinline__ uint32_t stage_lds(uint32_t smb, int st, int off) {
    constexpr uint32_t kOff = PART == kPartA ? offsetof(GemmSmem, a)
                            : PART == kPartB ? offsetof(GemmSmem, b)
                            : PART == kPartAs ? offsetof(GemmSmem, as) : offsetof(GemmSmem, bs);
    constexpr uint32_t kStage = PART == kPartA ? sizeof(GemmSmem::a[0])
                              : PART == kPartB ? sizeof(GemmSmem::b[0])
                              : PART == kPartAs ? sizeof(GemmSmem::as[0]) : sizeof(GemmSmem::bs[0]);
    return smb + kOff + (uint32_t)st * kStage + (uint32_t)off;
}

// Global -> LDS load of 16 (or 4) bytes per lane: lane l's bytes land at LDS
// address lds + OFF + 16*l (4*l).  Issued through inline asm so that the
// compiler does not track it: the kernel waits for these loads itself with
// vmcnt.  M0 carries the LDS address (declared clobbered: no other
// instruction in these kernels reads M0); one wait state separates the M0
// write from the load.  OFF, a constant, is added into M0 by the same scalar
// instruction that writes it, so that the loads of one stage share one base
// register instead of each keeping its own address live in a scalar register.
template <uint32_t OFF = 0>
__device__ __forceinline__ void dma_b128(const v4i& rsrc, uint32_t lds, uint32_t voff,
                                         uint32_t soff) {
    if constexpr (OFF == 0)
        asm volatile(
            "s_mov_b32 m0, %0\n\t"
            "s_nop 0\n\t"
            "buffer_load_dwordx4 %1, %2, %3 offen lds"
            :
            : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
            : "memory", "m0");
    else
        asm volatile(
            "s_add_u32 m0, %0, %4\n\t"
            "s_nop 0\n\t"
            "buffer_load_dwordx4 %1, %2, %3 offen lds"
            :
            : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff), "n"(OFF)
            : "memory", "m0", "scc");
}
template <uint32_t OFF = 0>
__device__ __forceinline__ void dma_b32(const v4i& rsrc, uint32_t lds, uint32_t voff,
                                        uint32_t soff) {
    if constexpr (OFF == 0)
        asm volatile(
            "s_mov_b32 m0, %0\n\t"
            "s_nop 0\n\t"
            "buffer_load_dword %1, %2, %3 offen lds"
            :
            : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
            : "memory", "m0");
    else
        asm volatile(
            "s_add_u32 m0, %0, %4\n\t"
            "s_nop 0\n\t"
            "buffer_load_dword %1, %2, %3 offen lds"
            :
            : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff), "n"(OFF)
            : "memory", "m0", "scc");
}

// Compile-time loop: f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>),
// so that register arrays are only ever indexed by constants.
template <class Fn, int... I>
__device__ __forceinline__ void static_for_impl(Fn&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Workgroup barrier after this wave's LDS reads and writes have completed;
// global loads and stores still in flight (including loads into LDS, which
// the caller waits for with vmcnt) are not waited for.  The memory clobber
// keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Tile coordinates are wave-uniform but come from LDS reads; moving them to
// scalar registers keeps buffer descriptors and LDS-DMA addresses scalar.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uni64(int64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// The lane index, computed where it is used: a volatile computation is not
// hoisted, so no per-lane value has to stay live across the tile loops (where
// it would take a register, or a scratch slot whose reload waits with vmcnt
// for every store and load in flight).
__device__ __forceinline__ int lane_now() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

__device__ __forceinline__ float silu_sig(float a, float& sg) {
    sg = __builtin_amdgcn_rcpf(1.0f + __expf(-a));
    return a * sg;
}

// Cross-lane reductions with single VALU ops (no LDS traffic): DPP quad
// permutes and row rotations within a 16-lane row, v_permlane16/32_swap
// across rows.  A swap of x with itself returns, per lane, x and the value
// of the partner lane 16 (32) away in some order, so max/sum of the pair is
// the pairwise reduction.
#define MX_DPP(x, ctrl) ((uint32_t)__builtin_amdgcn_update_dpp(0, (int)(x), (ctrl), 0xF, 0xF, false))
#define MX_DPPF(x, ctrl) __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), (ctrl), 0xF, 0xF, false))

// max over the 16 lanes that share (lane >> 4)
__device__ __forceinline__ uint32_t max16(uint32_t m) {
    m = max(m, MX_DPP(m, 0xB1));     // quad_perm [1,0,3,2]
    m = max(m, MX_DPP(m, 0x4E));     // quad_perm [2,3,0,1]
    m = max(m, MX_DPP(m, 0x124));    // row_ror:4
    m = max(m, MX_DPP(m, 0x128));    // row_ror:8
    return m;
}
// max over the 4 lanes that share (lane & 15)
__device__ __forceinline__ uint32_t max4q(uint32_t m) {
    auto a = __builtin_amdgcn_permlane16_swap(m, m, false, false);
    m = max(a[0], a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(m, m, false, false);
    return max(b[0], b[1]);
}
// sum over the 4 lanes that share (lane & 15); the pairwise sums are formed
// in the same order on every lane, so all four lanes hold the same value
__device__ __forceinline__ float sum4q(float v) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// (Quad permutes and row rotations with full row and bank masks give every lane
// a source, so the plain DPP move needs no old value to start from.)
// 4 x 4 byte transpose across the 4 lanes that share (lane >> 2): lane u
// holds bytes B[u][0..3] and receives B[0..3][u].  Two rounds: swap 16-bit
// halves with lane u^2, then bytes with lane u^1 (DPP quad permutes + v_perm).
__device__ __forceinline__ uint32_t transpose4x4_bytes(uint32_t x, int u) {
    const uint32_t y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);
    const uint32_t t = (u & 2) ? __builtin_amdgcn_perm(y, x, 0x03020706u)
                               : __builtin_amdgcn_perm(y, x, 0x05040100u);
    const uint32_t w = (uint32_t)__builtin_amdgcn_mov_dpp((int)t, 0xB1, 0xF, 0xF, false);
    return (u & 1) ? __builtin_amdgcn_perm(w, t, 0x03070105u)
                   : __builtin_amdgcn_perm(w, t, 0x06020400u);
}

__device__ __forceinline__ uint2 pack4_bf16(const float (&v)[4]) {
    return make_uint2(bf16x2(v[0], v[1]), bf16x2(v[2], v[3]));
}

__device__ __forceinline__ void unpack4_bf16(uint2 w, float (&v)[4]) {
    v[0] = __uint_as_float(w.x << 16);
    v[1] = __uint_as_float(w.x & 0xffff0000u);
    v[2] = __uint_as_float(w.y << 16);
    v[3] = __uint_as_float(w.y & 0xffff0000u);
}

// The gate-up pre-activation h saved for the backward is stored in 16 x 16
// blocks in the MFMA output layout: block (padded row / 16, column / 16) of
// the [Mp, F] grid holds 1 KiB, 16 bytes per lane l = (q, r16): the four gate
// values then the four up values of row r16, columns 4q..4q+3.  Forward and
// backward tiles share that lane mapping, so both move h with one coalesced
// 16-byte access per lane per block.  Rows are padded per expert (multiples of
// 128), so a block never straddles two experts.
// The block's base is wave-uniform; the lane adds a 32-bit offset.
__device__ __forceinline__ uint4* h_block(uint16_t* h, int64_t prow16, int64_t col16,
                                          int64_t F, int lane) {
    uint8_t* const blk = reinterpret_cast<uint8_t*>(h) + ((prow16 >> 4) * (F >> 4) + (col16 >> 4)) * 1024;
    return reinterpret_cast<uint4*>(blk + (uint32_t)(lane * 16));
}

// Requantized outputs (z in the forward, dh in the backward) are staged per
// wave in LDS and leave as full 16-byte chunks: rowwise codes one 32-row
// slice at a time, token-axis codes kTok tokens (one or two slices) at a
// time, token-axis scales once per tile.  A wave's output columns [0, C) map
// to global columns through colmap (one run of C, or two runs of C/2 at cw
// and F + cw for dh = [da | db]).  The backward (C = 256) flushes token-axis
// codes every slice so that its LDS slot also holds the h ring.
template <int C>
struct QStage {
    static constexpr int kTok = C >= 256 ? 32 : 64;   // tokens per token-axis flush
    static constexpr int kRcStride = C + 16;    // 16-byte aligned rows, conflict-free dword writes
    static constexpr int kCcStride = kTok + 16;
    static constexpr int kRc = 0;
    static constexpr int kRs = kRc + 32 * kRcStride;
    static constexpr int kCc = kRs + 32 * (C / 32);
    static constexpr int kCs = kCc + C * kCcStride;
    static constexpr int kBytes = kCs + C * 4;
};

// LDS of one workgroup: the operand stages of the main loop, reused by the
// fused epilogues as four per-wave slots.  The backward's slot adds a ring of
// four h units (4 x 4 KiB) after its staging area.
constexpr int kHRing = 4 * 4 * 1024;
// The recompute backward's slot adds the stash of the wave's last 32-row
// slice of [a | b] (16 x 1 KiB: 64 floats per lane).
constexpr int kStash = 16 * 1024;
template <Epi EPI>
struct Slot {
    static constexpr int kBytes = EPI == Epi::kDSwiglu ? QStage<256>::kBytes + kHRing
                                                       : (int)sizeof(GemmSmem) / 4;
    static constexpr int kSmem = 4 * kBytes > (int)sizeof(GemmSmem) ? 4 * kBytes
                                                                     : (int)sizeof(GemmSmem);
    static_assert(EPI != Epi::kSwiglu || QStage<64>::kBytes <= kBytes, "staging fits the slot");
    static_assert(EPI != Epi::kDSwigluR || QStage<128>::kBytes + kStash <= kBytes,
                  "staging and stash fit the slot");
    static_assert(EPI != Epi::kStoreBf16 || 4 * 32768 <= kSmem, "output quadrants fit the stages");
    static_assert(kBytes % 16 == 0 && QStage<256>::kBytes % 16 == 0, "16-byte aligned regions");
};

struct QDest {
    uint8_t* qr; uint8_t* qrs; int64_t ldqr;    // rowwise codes [rows][ldqr] + scales
    uint8_t* qc; uint8_t* qcs; int64_t ldqc;    // token-axis codes [cols][ldqc] + scales
    int64_t cw, F;                              // global column of local column 0; F
    bool split;                                 // local columns [C/2, C) go to F + cw
    bool tiled;                                 // K-step tiled scales (Kp = ldqr / ldqc)
};

template <int C>
__device__ __forceinline__ int64_t colmap(const QDest& d, int lc) {
    return (d.split && lc >= C / 2) ? d.F + d.cw + (lc - C / 2) : d.cw + lc;
}

// Quantize a 32 x 32 unit held as u[ii][jj][v] in the transposed MFMA output
// layout (lane (r16, q): row ii*16 + r16 of the slice, columns lc + jj*16 +
// 4q + v) rowwise (32 consecutive columns) and columnwise (the slice's 32
// tokens of a column), writing codes and scales into the wave's staging area.
template <int C>
__device__ __forceinline__ void quant_unit(const float (&u)[2][2][4], int lc, int ip,
                                           uint8_t* st, int lane) {
    using S = QStage<C>;
    const int r16 = lane & 15, q = lane >> 4;
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
        uint32_t m = 0;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int v = 0; v < 4; ++v) m = max(m, abs_bits(u[ii][jj][v]));
        m = max4q(m);
        const uint32_t sc = scale_code_from_amax_bits(m);
        const float scl = scale_from_code(sc), lim = e4m3_limit_from_code(sc);
        uint8_t* row = st + S::kRc + (ii * 16 + r16) * S::kRcStride + lc + 4 * q;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
            *reinterpret_cast<uint32_t*>(row + 16 * jj) = e4m3x4_scaled(
                u[ii][jj][0], u[ii][jj][1], u[ii][jj][2], u[ii][jj][3], lim, scl);
        // the 4 lanes of a row hold the same code and all store it: no
        // divergent branch to split the unit's code for the scheduler
        st[S::kRs + (ii * 16 + r16) * (C / 32) + lc / 32] = (uint8_t)sc;
    }
    const int u4 = r16 & 3, m4 = r16 >> 2;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        uint32_t scv[4];
        // column v's two rows (ii = 0, 1) share its scale: one scaled
        // conversion per column, byte pairs (ii0, ii1) regrouped by row below
        // (the even column's conversion writes the low half, the odd one's the
        // high half, so the even one starts from any bits: its input's)
        uint32_t pr[2];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            uint32_t m = max(abs_bits(u[0][jj][v]), abs_bits(u[1][jj][v]));
            m = max16(m);
            scv[v] = scale_code_from_amax_bits(m);
            pr[v >> 1] = e4m3x2_scaled((v & 1) ? pr[v >> 1] : __float_as_uint(u[0][jj][v]),
                                       u[0][jj][v], u[1][jj][v], e4m3_limit_from_code(scv[v]),
                                       scale_from_code(scv[v]), (v & 1) != 0);
        }
        // pr[0] = [v0 of ii0, v0 of ii1, v1 of ii0, v1 of ii1], pr[1] likewise
        // for v2, v3; row ii's dword holds its v0..v3
        const uint32_t wrow[2] = {__builtin_amdgcn_perm(pr[1], pr[0], 0x06040200u),
                                  __builtin_amdgcn_perm(pr[1], pr[0], 0x07050301u)};
        const int col = lc + jj * 16 + 4 * q + u4;      // this lane's column after the transpose
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            const uint32_t t = transpose4x4_bytes(wrow[ii], u4);    // tokens 4*m4 .. 4*m4+3
            *reinterpret_cast<uint32_t*>(st + S::kCc + col * S::kCcStride +
                                         (ip % (S::kTok / 32)) * 32 + ii * 16 + 4 * m4) = t;
        }
        // the 4 lanes of a column (m4 = 0..3) store the same code, picked
        // from the four with a byte extract rather than a branch
        const uint32_t sc4 = scv[0] | (scv[1] << 8) | (scv[2] << 16) | (scv[3] << 24);
        st[S::kCs + col * 4 + ip] = (uint8_t)(sc4 >> (8 * u4));
    }
}

// The flushes address global memory as a wave-uniform base (scalar
// registers) plus one 32-bit per-lane offset that is the same for every pass,
// so each store is a single instruction with no per-lane 64-bit arithmetic.

// Rowwise codes and scales of slice ip (rows rbase + ip*32 + [0, 32)) to
// global memory; rows at or past rows_valid (relative to the wave) are not
// written.  NT: nontemporal code stores (measured: faster for the forward's
// z copies, slower for the backward's dh copies, whose epilogue waits on
// vmcnt while its stores are in flight).
template <int C, bool NT>
__device__ __forceinline__ void flush_rows(const uint8_t* st, const QDest& d, int64_t rbase,
                                           int ip, int rows_valid, int lane) {
    using S = QStage<C>;
    constexpr int kCpr = C / 16;                  // 16-byte chunks per row
    constexpr int kRpp = 64 / kCpr;               // rows per pass of 64 lanes
    const int rl = lane / kCpr, lc = (lane % kCpr) * 16;
    const uint32_t coff = (d.split && lc >= C / 2) ? (uint32_t)(d.F - C / 2 + lc) : (uint32_t)lc;
    const uint32_t loff = (uint32_t)rl * (uint32_t)d.ldqr + coff;
    uint8_t* const base = d.qr + (rbase + ip * 32) * d.ldqr + d.cw;
#pragma unroll
    for (int t = 0; t < 32 / kRpp; ++t) {
        if (ip * 32 + t * kRpp + rl < rows_valid) {
            const uint4 v = *reinterpret_cast<const uint4*>(
                st + S::kRc + (t * kRpp + rl) * S::kRcStride + lc);
            uint8_t* const dst = base + (int64_t)(t * kRpp) * d.ldqr + loff;
            if constexpr (NT) store_nt(dst, v);
            else *reinterpret_cast<uint4*>(dst) = v;
        }
    }
    // scales: C/32 bytes per row; a split row is two runs of C/64 bytes
    constexpr int kRun = C >= 256 ? 4 : 2;
    constexpr int kRunsPerRow = (C / 32) / kRun;
    static_assert(32 * kRunsPerRow <= 64, "one pass covers the slice's scale runs");
    const int srow = lane / kRunsPerRow, sblk = (lane % kRunsPerRow) * kRun;
    const int64_t lds = d.ldqr / 32;
    if (srow < 32 && ip * 32 + srow < rows_valid) {
        const int64_t kb = (d.split && sblk >= C / 64) ? (d.F + d.cw) / 32 + (sblk - C / 64)
                                                       : d.cw / 32 + sblk;
        uint8_t* dst;
        if (d.tiled) {
            dst = d.qrs + tiled_scale_offset(rbase + ip * 32 + srow, kb, d.ldqr);
        } else {
            const uint32_t soff = (uint32_t)srow * (uint32_t)lds +
                                  ((d.split && sblk >= C / 64) ? (uint32_t)((d.F - C / 2) / 32 + sblk)
                                                               : (uint32_t)sblk);
            dst = d.qrs + (rbase + ip * 32) * lds + d.cw / 32 + soff;
        }
        const uint8_t* src = st + S::kRs + srow * (C / 32) + sblk;
        if constexpr (kRun == 4)
            *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(src);
        else
            *reinterpret_cast<uint16_t*>(dst) = *reinterpret_cast<const uint16_t*>(src);
    }
}

// Token-axis codes of the staged kTok tokens (padded positions tok0 ..
// tok0 + kTok - 1) to global memory: pass t moves kCpp columns.  NT as for
// flush_rows.
template <int C, bool NT>
__device__ __forceinline__ void flush_cols(const uint8_t* st, const QDest& d, int64_t tok0,
                                           int lane) {
    using S = QStage<C>;
    constexpr int kCh = S::kTok / 16;             // 16-byte chunks per column
    constexpr int kCpp = 64 / kCh;                // columns per pass
    const int cl = lane / kCh, ch = (lane % kCh) * 16;
    const uint32_t loff = (uint32_t)cl * (uint32_t)d.ldqc + (uint32_t)ch;
#pragma unroll
    for (int t = 0; t < C / kCpp; ++t) {
        const int64_t gcol = (d.split && t * kCpp >= C / 2) ? d.F + d.cw + t * kCpp - C / 2
                                                            : d.cw + t * kCpp;
        uint8_t* const base = d.qc + gcol * d.ldqc + tok0;
        const uint4 v = *reinterpret_cast<const uint4*>(
            st + S::kCc + (t * kCpp + cl) * S::kCcStride + ch);
        if constexpr (NT) store_nt(base + loff, v);
        else *reinterpret_cast<uint4*>(base + loff) = v;
    }
}

// Token-axis scales of the wave's four slices (one dword per column).
template <int C>
__device__ __forceinline__ void flush_col_scales(const uint8_t* st, const QDest& d,
                                                 int64_t pbase, int lane) {
    using S = QStage<C>;
    const int64_t lds = d.ldqc / 32;
    const uint32_t loff = (uint32_t)lane * (uint32_t)lds;
#pragma unroll
    for (int k = 0; k < (C + 63) / 64; ++k) {
        if (k * 64 + lane < C) {
            const int64_t gcol = (d.split && k * 64 >= C / 2) ? d.F + d.cw + k * 64 - C / 2
                                                              : d.cw + k * 64;
            uint8_t* const dst = d.tiled ? d.qcs + tiled_scale_offset(gcol + lane, pbase / 32, d.ldqc)
                                         : d.qcs + gcol * lds + pbase / 32 + loff;
            *reinterpret_cast<uint32_t*>(dst) =
                *reinterpret_cast<const uint32_t*>(st + S::kCs + (k * 64 + lane) * 4);
        }
    }
}

// The 2 x 2 accumulator blocks of unit (ip, jp): rows 2ip, 2ip+1 and columns
// J0, J0 + 1, for a wave-uniform runtime ip.  The fused epilogues loop over the
// wave's four 32-row slices at run time so that their code stays small enough
// for the instruction cache; one uniform branch per slice keeps the
// accumulator registers indexed by constants, and the empty asm in each
// branch stops the compiler from turning the branches into selects (which
// would read every candidate out of the accumulators at once).
template <int J0, int NJ>
__device__ __forceinline__ void pick_unit(const v4f (&acc)[8][NJ], int ip, float (&u)[2][2][4]) {
    static_for<4>([&](auto c) {
        constexpr int k = decltype(c)::value;
        if (ip == k) {
#pragma unroll
            for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        float x = acc[2 * k + ii][J0 + jj][v];
                        asm volatile("" : "+v"(x));
                        u[ii][jj][v] = x;
                    }
        }
    });
}

// pick_unit for the recompute backward's [a | b], whose last slice (rows
// 6, 7) was moved to the wave's LDS stash: block (ii, j) of it is 1 KiB at
// ((ii * 8 + j) * 64 + lane) * 16, one v4f per lane.
template <int J0>
__device__ __forceinline__ void pick_unit_stashed(const v4f (&acc)[8][8], int ip,
                                                  float (&u)[2][2][4], const uint8_t* stash,
                                                  int lane) {
    static_for<3>([&](auto c) {
        constexpr int k = decltype(c)::value;
        if (ip == k) {
#pragma unroll
            for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        float x = acc[2 * k + ii][J0 + jj][v];
                        asm volatile("" : "+v"(x));
                        u[ii][jj][v] = x;
                    }
        }
    });
    if (ip == 3) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const v4f x = *reinterpret_cast<const v4f*>(
                    stash + ((ii * 8 + J0 + jj) * 64 + lane) * 16);
#pragma unroll
                for (int v = 0; v < 4; ++v) u[ii][jj][v] = x[v];
            }
    }
}

__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// The plain epilogue straight from the registers, for tiles whose LDS holds
// the next tile's operands.  After the same v_permlane16_swap pairing, lane
// (r16, q) holds 8 consecutive columns of row i*16 + r16 for each jp: with
// jp = 2c and 2c + 1, the four lanes of a row hold the eight 16-byte chunks
// of 128-byte line c of the wave's row.  One DPP rotation by 8 within each
// 16-lane row then hands lane r16 < 8 the jp = 2c chunk of row r16 + 8, and
// lane r16 >= 8 the jp = 2c + 1 chunk of row r16 - 8, so that each store
// instruction writes whole lines: rows (r16 & 7) of the block, then rows 8
// + (r16 & 7), with lanes r16 < 8 on the jp = 2c half of the line and lanes
// r16 >= 8 on the other.  (Stored as the pairs left the swap, each
// instruction would write half lines, and the output would cost more.)
// gs: the tile's per-group output scale; rs: the wave's 128 routing weights
// in LDS (rows wm*128 ..), or null.  Nothing here reads global memory: a
// global load would wait (vmcnt) for every store and load in flight.
// part (a chunk of a split tail tile): the fp32 accumulators go instead, as
// they are, to the wave's blocks of a partial tile there (block (i, j) at
// byte (i * 8 + j) * 1024, lane l's 16 bytes at 16 l).  Both outputs share
// one pass over the row blocks, so the accumulators are read one way only.
// SCALED: the accumulators are multiplied by gs (and the row's rs) before
// the conversion; otherwise gs and rs are not read (the kernel variant for
// launches without output scales).
template <bool SCALED>
__device__ __forceinline__ void store_tile_bf16_regs(v4f (&acc)[8][8], const GemmProblem& p,
                                                     int g, int64_t m0, int64_t mvalid, int64_t n0,
                                                     int wm, int wn, int lane, float gs,
                                                     const float* rs, uint8_t* part = nullptr) {
    const int r16 = lane & 15, q = lane >> 4;
    const bool lo8 = r16 < 8;
    const int64_t rwave = m0 + wm * 128;
    const int rows_valid_w = (int)min((int64_t)128, max((int64_t)0, mvalid - wm * 128));
    uint16_t* C = reinterpret_cast<uint16_t*>(p.C) + (p.kgroup ? (int64_t)g * p.c_gstride : 0);
    const int64_t cw = n0 + wn * 128;
    // addresses: a wave-uniform base plus one 32-bit per-lane byte offset (the
    // lane's row r16 & 7 and its 16-byte chunk of line 0); rows, the second
    // half of a block and further lines only move the uniform base
    uint8_t* const Cw = reinterpret_cast<uint8_t*>(C + rwave * p.ldc + cw);
    const uint32_t ldb = (uint32_t)p.ldc * 2u;
    const int chunk0 = (lo8 ? 0 : 4) + 2 * (q & 1) + (q >> 1);
    const uint32_t loff = (uint32_t)(r16 & 7) * ldb + (uint32_t)chunk0 * 16u;
    // The rotation by 8 lanes of the rows' second halves, written only where
    // it lands: into the lanes r16 >= 8 (banks 2, 3) of s1, which start as
    // d0, and into the lanes r16 < 8 (banks 0, 1) of s2, which start as d1:
    // s1 = lo8 ? d0 : d1 of lane r16 ^ 8, s2 = lo8 ? d0 of lane r16 ^ 8 : d1.
    auto into_hi = [](uint32_t old, uint32_t v) {
        return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, 0x128, 0xf, 0xc, false);
    };
    auto into_lo = [](uint32_t old, uint32_t v) {
        return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, 0x128, 0xf, 0x3, false);
    };
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        // the accumulators live in AGPRs: pinned there at each row block, the
        // block moves to VGPRs only when it is converted (else the compiler
        // may move the whole tile up front and spill)
#pragma unroll
        for (int j = 0; j < 8; ++j) asm volatile("" : "+a"(acc[i][j]));
        if (part) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                *reinterpret_cast<v4f*>(part + (int64_t)(i * 8 + j) * 1024 + (uint32_t)lane * 16u) =
                    acc[i][j];
            __builtin_amdgcn_sched_barrier(0);
            continue;
        }
        const float sc = SCALED ? (rs ? rs[i * 16 + r16] * gs : gs) : 1.0f;
        const int rl1 = i * 16 + (r16 & 7), rl2 = rl1 + 8;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            uint32_t d[2][4];                       // jp = 2c + h, after the swap
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int jp = 2 * c + h;
                float va[4], vb[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    va[v] = SCALED ? acc[i][2 * jp][v] * sc : acc[i][2 * jp][v];
                    vb[v] = SCALED ? acc[i][2 * jp + 1][v] * sc : acc[i][2 * jp + 1][v];
                }
                const uint2 a = pack4_bf16(va), b = pack4_bf16(vb);
                const auto x = __builtin_amdgcn_permlane16_swap(a.x, b.x, false, false);
                const auto y = __builtin_amdgcn_permlane16_swap(a.y, b.y, false, false);
                d[h][0] = x[0];
                d[h][1] = y[0];
                d[h][2] = x[1];
                d[h][3] = y[1];
            }
            uint32_t s1[4], s2[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                s1[v] = into_hi(d[0][v], d[1][v]);
                s2[v] = into_lo(d[1][v], d[0][v]);
            }
            const int chunk = chunk0 + 8 * c;
            if (cw + chunk * 8 < p.N) {
                uint8_t* const b1 = Cw + (int64_t)(i * 16) * ldb + c * 128;
                if (rl1 < rows_valid_w)
                    store_nt(b1 + loff, make_uint4(s1[0], s1[1], s1[2], s1[3]));
                if (rl2 < rows_valid_w)
                    store_nt(b1 + (int64_t)8 * ldb + loff, make_uint4(s2[0], s2[1], s2[2], s2[3]));
            }
        }
        // one row block at a time: the scheduler would otherwise read ahead
        // the accumulators of later blocks into registers the kernel has not
        // got (and spill them, the reload then waiting for every store)
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Tail-split workspace: header, then the partial tiles.  A partial tile keeps
// the MFMA output layout: block (i, j) of wave w is 1 KiB at float offset
// ((w * 64 + i * 8 + j) * 64 + lane) * 4, so every store and load of it is
// one coalesced 1 KiB access.
struct SplitHdr {
    int32_t rem;                 // tail tiles that were split (0: none)
    int32_t S;                   // chunks per tail tile
    int32_t pad[14];
    int64_t meta[kSplitItems / 2][4];   // per tail tile: group, m0, mvalid, n0
};
static_assert(sizeof(SplitHdr) <= kSplitHdrBytes, "split header fits");

__device__ __forceinline__ float* split_part(uint8_t* ws, int item) {
    return reinterpret_cast<float*>(ws + kSplitHdrBytes) + (int64_t)item * (BM * BN);
}

// Sources of one GEMM of a tile: buffer descriptors of the A and B codes
// (ranges end with the last valid row's K range, so rows past the valid
// ones read as zeros whether or not the scalar K offset takes part in the
// range check), each lane's offsets for the direct loads, and the scale
// sources.
struct TileSrc {
    v4i ra, rb;
    ScaleSrc sa, sb;
    uint32_t aoff[8], boff[8];
};

// A: rows m0 .. m0 + mvalid - 1 of A.  B: tile row b is row brow0 + brow(b)
// of B (bvalid rows from brow0 are valid).  The B tile has NJ * 32 rows.
// Direct global->LDS loads move 64 lanes x 16 B = 8 tile rows into 1 KiB of
// LDS per instruction, lane l landing at byte 16*l: lane l fetches row
// (l >> 3) of the 8 and the logical chunk that the swizzle places at
// physical chunk (l & 7).
template <bool UNIT, int NJ, class BRow>
__device__ __forceinline__ TileSrc tile_src(const MxOperand& A, const MxOperand& B, int64_t m0,
                                            int64_t mvalid, int64_t brow0, int64_t bvalid,
                                            int64_t klo, int64_t K, BRow brow, int wave, int lane) {
    TileSrc o;
    const int64_t lda = A.ld, ldb = B.ld;
    o.ra = make_rsrc(A.codes + m0 * lda + klo, (mvalid - 1) * lda + K);
    o.rb = make_rsrc(B.codes + brow0 * ldb + klo, (bvalid - 1) * ldb + K);
    const int dma_row = lane >> 3;
    const int dma_chunk = (lane & 7) ^ (dma_row & 7);
#pragma unroll
    for (int j = 0; j < 8; ++j)
        o.aoff[j] = (uint32_t)(((wave * 8 + j) * 8 + dma_row) * lda + dma_chunk * 16);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
        o.boff[j] = (uint32_t)(brow((wave * NJ + j) * 8 + dma_row) * ldb + dma_chunk * 16);
    o.sa = scale_src<UNIT>(A.scales, lda, A.tiled, m0, mvalid, wave * 64 + lane, klo, K);
    o.sb = scale_src<UNIT>(B.scales, ldb, B.tiled, brow0, bvalid, brow(wave * 64 + lane), klo, K);
    return o;
}

// Placement of one K step's loads (u < 8: A rows, u < 8 + NJ: B rows,
// 8 + NJ: A scales, 9 + NJ: B scales) over the MFMA slots of the two passes
// of a step: a_at(s) / b_at(s) give the load issued after pass-A / pass-B
// slot s, or -1.  kNA loads go into pass A.
template <int NJ> struct Sched;
template <> struct Sched<8> {       // 256 x 256 tile: 18 loads, 64 MFMAs per wave
    static constexpr int kLoads = 18, kNA = 12;
    // 12 after slots 1, 4, 6 of every 8; 6 after slots 5, 9, ..., 25
    static constexpr int a_at(int s) {
        return s % 8 == 1 ? 3 * (s / 8) : s % 8 == 4 ? 3 * (s / 8) + 1
                                        : s % 8 == 6 ? 3 * (s / 8) + 2 : -1;
    }
    static constexpr int b_at(int s) {
        return (s >= 5 && s <= 25 && s % 4 == 1) ? 12 + (s - 5) / 4 : -1;
    }
};
template <> struct Sched<4> {       // 256 x 128 tile: 14 loads, 32 MFMAs per wave
    static constexpr int kLoads = 14, kNA = 9;
    static constexpr int a_at(int s) {
        return s == 0 ? 0 : s == 1 ? 1 : s == 3 ? 2 : s == 5 ? 3 : s == 7 ? 4 : s == 8 ? 5
             : s == 10 ? 6 : s == 12 ? 7 : s == 14 ? 8 : -1;
    }
    static constexpr int b_at(int s) {
        return s == 5 ? 9 : s == 7 ? 10 : s == 9 ? 11 : s == 10 ? 12 : s == 11 ? 13 : -1;
    }
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    if constexpr (N == 18) asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
    else if constexpr (N == 14) asm volatile("s_waitcnt vmcnt(14)" ::: "memory");
    else if constexpr (N == 12) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    else if constexpr (N == 9) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    else static_assert(N < 0, "add the wait count");
}

// acc[8][NJ] += A-tile . B-tile^T over nk K steps of 128.  Wave (wm, wn)
// owns rows wm*128 .. +128 of the 256-row tile and B rows wn*NJ*16 .. +NJ*16;
// B is the MFMA's first operand, so acc[i][j] holds the transposed 16 x 16
// block (lane (r16, q): row i*16 + r16, columns j*16 + 4q .. +3).
//
// Software pipeline over two LDS stages (stage k & 1 holds step k):
//  * S1 (start of step k): every wave has step k's fragments in registers,
//    so stage k is free; the loads of step k+2 go into it, kNA of them
//    spread over pass A and the rest over pass B.
//  * pass A: MFMA rows 0..3 over the NJ columns.
//  * S2: vmcnt(kNA) -- this wave's loads of step k+1 have landed (only the
//    pass-A loads of step k+2 may still be in flight) -- then a barrier,
//    after which stage k+1 is complete for every wave.  The next step's A
//    rows 0..3 are read into the registers pass A freed.
//  * pass B: MFMA rows 4..7; after column j the next step's B fragment j is
//    read, and in the last column each A row i is read as soon as its last
//    MFMA has issued.
// So the LDS reads overlap the MFMAs and use no extra registers, and each
// load has about one and a half steps to land.  Every MFMA sits in its own
// slot so that its execution hides the instructions issued after it.
// Barriers fence LDS only (a workgroup fence would also wait for loads in
// flight).  Output stores of an earlier tile may still be in flight: loads
// complete in order among themselves, so the vmcnt waits stay sufficient
// with older stores outstanding (they only make them stricter).  Steps at
// or past nk use zero-range descriptors: they write zeros into a stage
// nobody reads, so every step issues the same instructions and the vmcnt
// counts hold without branches; the caller waits for those trailing loads
// before it reuses the stages.  A Tail other than ZeroTail replaces those
// trailing loads: tail(slot, stage, kn) issues load slot u (same count per
// pass) of step kn = 0, 1 of whatever runs next on the stages.  The steps
// whose loads fall inside the K range run a loop body without the
// zero-range selects.
struct ZeroTail {};
struct ZeroTailMaker {
    __device__ ZeroTail operator()() const { return {}; }
};

template <int NJ, class MakeTail = ZeroTailMaker>
__device__ __forceinline__ void tile_gemm(v4f (&acc)[8][NJ], GemmSmem& sm, const TileSrc& o,
                                          int nk, int wave, int wm, int wn, int lane,
                                          MakeTail make_tail = {}) {
    using SC = Sched<NJ>;
    const int r16 = lane & 15, q = lane >> 4;
    const int swz = r16 & 7;
    const uint32_t smb = uni((int)lds_addr(&sm));
    // load slot u of step ks into stage st; LIVE: the step is known to be
    // inside the K range, else it is checked
    auto dma_u = [&](auto uc, auto livec, int st, int ks) {
        constexpr int u = decltype(uc)::value;
        const bool live = decltype(livec)::value || ks < nk;
        const uint32_t k0 = (uint32_t)ks * BK;
        auto rng = [&](const v4i& r) { return live ? r : v4i{r.x, r.y, 0, r.w}; };
        if constexpr (u < 8) {
            dma_b128<u * 1024>(rng(o.ra), stage_lds<kPartA>(smb, st, wave * 8 * 1024), o.aoff[u], k0);
        } else if constexpr (u < 8 + NJ) {
            dma_b128<(u - 8) * 1024>(rng(o.rb), stage_lds<kPartB>(smb, st, wave * NJ * 1024),
                                     o.boff[u - 8], k0);
        } else if constexpr (u == 8 + NJ) {
            dma_b32(rng(o.sa.rsrc), stage_lds<kPartAs>(smb, st, wave * 64 * 4), o.sa.voff,
                    o.sa.s0 + ks * o.sa.sstep);
        } else {
            dma_b32(rng(o.sb.rsrc), stage_lds<kPartBs>(smb, st, wave * 64 * 4), o.sb.voff,
                    o.sb.s0 + ks * o.sb.sstep);
        }
    };
    // the loads of a step: within the K range, or past its end (the tail)
    using Tail = decltype(make_tail());
    auto load = [&](auto uc, auto tailc, const Tail* tail, int st, int ks) {
        if constexpr (!decltype(tailc)::value || std::is_same<Tail, ZeroTail>::value)
            dma_u(uc, std::integral_constant<bool, !decltype(tailc)::value>{}, st, ks);
        else
            (*tail)(uc, st, ks - nk);
    };

    // Fragments of stage st into registers.  The scaled 16x16x128 MFMA reads
    // a lane's 32 operand bytes as two 16-byte runs of K, [16q, 16q+16) and
    // [64+16q, 64+16q+16), and the scale byte of lane (r, q) as that of K
    // block q of row r (pinned on the device by per-block scale probes).
    v8i af[8], bfr[NJ];
    int asc[8], bsc[NJ];
    // Per-lane byte offsets of the lane's first fragment row (row i adds
    // i * 16 rows, a constant): the reads of one stage then share one base
    // per kind and differ only in their immediate offsets.
    const int a_row0 = wm * 128 + r16, b_row0 = wn * (NJ * 16) + r16;
    const int a_lo = a_row0 * BK + ((q ^ swz) << 4), a_hi = a_row0 * BK + (((q + 4) ^ swz) << 4);
    const int b_lo = b_row0 * BK + ((q ^ swz) << 4), b_hi = b_row0 * BK + (((q + 4) ^ swz) << 4);
    const int a_s = a_row0 * 4 + q, b_s = b_row0 * 4 + q;
    auto read_a = [&](auto ic, int st) {
        constexpr int i = decltype(ic)::value;
        const uint8_t* stg = sm.a[st];
        const uint4 lo = *reinterpret_cast<const uint4*>(stg + a_lo + i * 16 * BK);
        const uint4 hi = *reinterpret_cast<const uint4*>(stg + a_hi + i * 16 * BK);
        af[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                    (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        asc[i] = (reinterpret_cast<const uint8_t*>(sm.as[st]) + a_s)[i * 16 * 4];
    };
    auto read_b = [&](auto jc, int st) {
        constexpr int j = decltype(jc)::value;
        const uint8_t* stg = sm.b[st];
        const uint4 lo = *reinterpret_cast<const uint4*>(stg + b_lo + j * 16 * BK);
        const uint4 hi = *reinterpret_cast<const uint4*>(stg + b_hi + j * 16 * BK);
        bfr[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        bsc[j] = (reinterpret_cast<const uint8_t*>(sm.bs[st]) + b_s)[j * 16 * 4];
    };
    auto mfma = [&](auto ic, auto jc) {
        constexpr int i = decltype(ic)::value, j = decltype(jc)::value;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            bfr[j], af[i], acc[i][j], 0, 0, 0, bsc[j], 0, asc[i]);
    };
    auto step = [&](int ks, auto tailc, const Tail* tail) {
        const int cur = ks & 1, nxt = cur ^ 1;
        lds_barrier();                                  // S1: stage cur is free
        // pass A: slot s is column j = s / 4, row i = s % 4
        static_for<4 * NJ>([&](auto sc) {
            constexpr int s = decltype(sc)::value;
            mfma(std::integral_constant<int, s % 4>{}, std::integral_constant<int, s / 4>{});
            __builtin_amdgcn_sched_barrier(0);
            constexpr int u = SC::a_at(s);
            if constexpr (u >= 0) load(std::integral_constant<int, u>{}, tailc, tail, cur, ks + 2);
            __builtin_amdgcn_sched_barrier(0);
        });
        wait_vmcnt<SC::kNA>();
        lds_barrier();                                  // S2: stage nxt complete
        // pass B: slot s is column j = s / 4, row i = 4 + s % 4
        static_for<4 * NJ>([&](auto sc) {
            constexpr int s = decltype(sc)::value, j = s / 4, i = 4 + s % 4;
            mfma(std::integral_constant<int, i>{}, std::integral_constant<int, j>{});
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (s < 4) read_a(std::integral_constant<int, s>{}, nxt);
            if constexpr (s >= 4 * NJ - 4) read_a(std::integral_constant<int, i>{}, nxt);
            if constexpr (s % 4 == 3) read_b(std::integral_constant<int, j>{}, nxt);
            constexpr int u = SC::b_at(s);
            if constexpr (u >= 0) load(std::integral_constant<int, u>{}, tailc, tail, cur, ks + 2);
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    static_for<SC::kLoads>([&](auto uc) { dma_u(uc, std::false_type{}, 0, 0); });
    static_for<SC::kLoads>([&](auto uc) { dma_u(uc, std::false_type{}, 1, 1); });
    wait_vmcnt<SC::kLoads>();                           // step 0 (this wave)
    lds_barrier();                                      // step 0 (every wave)
    static_for<8>([&](auto ic) { read_a(ic, 0); });
    static_for<NJ>([&](auto jc) { read_b(jc, 0); });
    int ks = 0;
    for (; ks + 2 < nk; ++ks) step(ks, std::false_type{}, nullptr);
    if (ks < nk) {
        const Tail tail = make_tail();
        for (; ks < nk; ++ks) step(ks, std::true_type{}, &tail);
    }
}

// The per-tile part of a plain tile's sources: its lane offsets of the code
// loads depend only on the wave, the lane and the leading dimensions, which
// every tile of a launch shares, so the next tile needs only its buffer
// descriptors, its scale offsets and its K-step count.
struct TileNext {
    v4i ra, rb, sar, sbr;
    uint32_t sav, sbv, sa0, sb0;
    int nk;                      // K steps (0: no next tile)
};

// (the scalar fields pass through readfirstlane: values that came from LDS
// reads are not known to be wave-uniform, and buffer descriptors and scalar
// offsets must sit in scalar registers)
__device__ __forceinline__ v4i uni4(const v4i& v) { return v4i{uni(v.x), uni(v.y), uni(v.z), uni(v.w)}; }
__device__ __forceinline__ TileNext tile_next(const TileSrc& o, int nk) {
    return TileNext{uni4(o.ra), uni4(o.rb), uni4(o.sa.rsrc), uni4(o.sb.rsrc), o.sa.voff, o.sb.voff,
                    (uint32_t)uni((int)o.sa.s0), (uint32_t)uni((int)o.sb.s0), uni(nk)};
}

// tile_gemm<8> for a chain of plain tiles, one after another on one
// workgroup: the loads that tile_gemm spends on zero-range steps past the
// end (steps nk and nk + 1) fetch the next tile's steps 0 and 1 instead, so
// that tile's first operands arrive while this one finishes and while its
// epilogue runs (which must then leave LDS alone).  Stage parity runs on
// across tiles: step ks of this tile lives in stage (base + ks) & 1.
//  * pre: steps 0 and 1 of this tile were issued by the previous tile, and
//    step 0 is complete for every wave (the previous tile's last S2 wait and
//    barrier); otherwise this tile issues them itself, after waiting for any
//    loads still in flight into the stages.
//  * Steps 0 .. nk - 3 load steps 2 .. nk - 1 of this tile, all of them
//    within its K range, so that loop carries no zero-range selects.  The
//    last two steps load from next_src(): steps 0 and 1 of the next tile, or
//    zero-range loads where it has no such step (nk = 0 when there is no
//    next tile).  It is called after the first loop, so that the next
//    tile's sources take the registers of this tile's.
// The waits of the main loop stay sufficient with the previous tile's
// output stores in flight between the loads: loads complete in order among
// themselves, and every vmcnt wait here leaves only loads younger than the
// ones it waits for, so a pending older load would keep the count above the
// wait's bound (stores complete whenever they do; nothing waits for them).
template <class NextSrc>
__device__ __forceinline__ void tile_gemm_chain(v4f (&acc)[8][8], GemmSmem& sm, const TileSrc& o,
                                                NextSrc next_src, int nk, int base, bool pre,
                                                int wave, int wm, int wn, int lane) {
    using SC = Sched<8>;
    constexpr int NJ = 8;
    const int r16 = lane & 15, q = lane >> 4;
    const int swz = r16 & 7;
    const int b0 = uni(base);    // stage addresses stay scalar
    const uint32_t smb = uni((int)lds_addr(&sm));
    // loads of step ks of source s into stage st; LIVE: within its K range
    auto dma_u = [&](auto uc, auto livec, const TileNext& src, int st, int ks) {
        constexpr int u = decltype(uc)::value;
        constexpr bool kLive = decltype(livec)::value;
        const bool live = kLive || ks < src.nk;
        const uint32_t k0 = (uint32_t)ks * BK;
        auto rng = [&](const v4i& r) { return live ? r : v4i{r.x, r.y, 0, r.w}; };
        if constexpr (u < 8) {
            dma_b128<u * 1024>(rng(src.ra), stage_lds<kPartA>(smb, st, wave * 8 * 1024), o.aoff[u], k0);
        } else if constexpr (u < 8 + NJ) {
            dma_b128<(u - 8) * 1024>(rng(src.rb), stage_lds<kPartB>(smb, st, wave * NJ * 1024),
                                     o.boff[u - 8], k0);
        } else if constexpr (u == 8 + NJ) {
            dma_b32(rng(src.sar), stage_lds<kPartAs>(smb, st, wave * 64 * 4), src.sav,
                    src.sa0 + ks * o.sa.sstep);
        } else {
            dma_b32(rng(src.sbr), stage_lds<kPartBs>(smb, st, wave * 64 * 4), src.sbv,
                    src.sb0 + ks * o.sb.sstep);
        }
    };

    v8i af[8], bfr[NJ];
    int asc[8], bsc[NJ];
    // per-lane offsets of the first fragment row, as in tile_gemm
    const int a_row0 = wm * 128 + r16, b_row0 = wn * (NJ * 16) + r16;
    const int a_lo = a_row0 * BK + ((q ^ swz) << 4), a_hi = a_row0 * BK + (((q + 4) ^ swz) << 4);
    const int b_lo = b_row0 * BK + ((q ^ swz) << 4), b_hi = b_row0 * BK + (((q + 4) ^ swz) << 4);
    const int a_s = a_row0 * 4 + q, b_s = b_row0 * 4 + q;
    auto read_a = [&](auto ic, int st) {
        constexpr int i = decltype(ic)::value;
        const uint8_t* stg = sm.a[st];
        const uint4 lo = *reinterpret_cast<const uint4*>(stg + a_lo + i * 16 * BK);
        const uint4 hi = *reinterpret_cast<const uint4*>(stg + a_hi + i * 16 * BK);
        af[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                    (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        asc[i] = (reinterpret_cast<const uint8_t*>(sm.as[st]) + a_s)[i * 16 * 4];
    };
    auto read_b = [&](auto jc, int st) {
        constexpr int j = decltype(jc)::value;
        const uint8_t* stg = sm.b[st];
        const uint4 lo = *reinterpret_cast<const uint4*>(stg + b_lo + j * 16 * BK);
        const uint4 hi = *reinterpret_cast<const uint4*>(stg + b_hi + j * 16 * BK);
        bfr[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        bsc[j] = (reinterpret_cast<const uint8_t*>(sm.bs[st]) + b_s)[j * 16 * 4];
    };
    // FIRST: the tile's first K step, whose MFMAs take a zero accumulator
    // input instead of acc (no per-tile zeroing of the 256 accumulators)
    auto mfma = [&](auto ic, auto jc, auto firstc) {
        constexpr int i = decltype(ic)::value, j = decltype(jc)::value;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            bfr[j], af[i], decltype(firstc)::value ? v4f{0.f, 0.f, 0.f, 0.f} : acc[i][j], 0, 0, 0,
            bsc[j], 0, asc[i]);
    };
    // one K step: the MFMAs of step ks, the loads of step kl of src
    auto step = [&](int ks, auto livec, const TileNext& src, int kl, auto firstc) {
        const int cur = (b0 + ks) & 1, nxt = cur ^ 1;
        lds_barrier();                                  // S1: stage cur is free
        static_for<4 * NJ>([&](auto sc) {
            constexpr int s = decltype(sc)::value;
            mfma(std::integral_constant<int, s % 4>{}, std::integral_constant<int, s / 4>{}, firstc);
            __builtin_amdgcn_sched_barrier(0);
            constexpr int u = SC::a_at(s);
            if constexpr (u >= 0) dma_u(std::integral_constant<int, u>{}, livec, src, cur, kl);
            __builtin_amdgcn_sched_barrier(0);
        });
        wait_vmcnt<SC::kNA>();
        lds_barrier();                                  // S2: stage nxt complete
        static_for<4 * NJ>([&](auto sc) {
            constexpr int s = decltype(sc)::value, j = s / 4, i = 4 + s % 4;
            mfma(std::integral_constant<int, i>{}, std::integral_constant<int, j>{}, firstc);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (s < 4) read_a(std::integral_constant<int, s>{}, nxt);
            if constexpr (s >= 4 * NJ - 4) read_a(std::integral_constant<int, i>{}, nxt);
            if constexpr (s % 4 == 3) read_b(std::integral_constant<int, j>{}, nxt);
            constexpr int u = SC::b_at(s);
            if constexpr (u >= 0) dma_u(std::integral_constant<int, u>{}, livec, src, cur, kl);
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    const TileNext own = tile_next(o, nk);
    if (!pre) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();                                  // no load in flight, stages free
        static_for<SC::kLoads>([&](auto uc) { dma_u(uc, std::false_type{}, own, b0, 0); });
        static_for<SC::kLoads>([&](auto uc) { dma_u(uc, std::false_type{}, own, b0 ^ 1, 1); });
        wait_vmcnt<SC::kLoads>();
        lds_barrier();
    }
    static_for<8>([&](auto ic) { read_a(ic, b0); });
    static_for<NJ>([&](auto jc) { read_b(jc, b0); });
    // Step 0 starts the accumulation from zero when it is followed by two
    // or more steps (its loads then stay within the tile); a tile of one or
    // two K steps (or none) zeroes acc first and runs every step as usual.
    int ks = 0;
    if (nk >= 3) {
        step(0, std::true_type{}, own, 2, std::true_type{});
        ks = 1;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    for (; ks + 2 < nk; ++ks) step(ks, std::true_type{}, own, ks + 2, std::false_type{});
    if (ks < nk) {
        const TileNext nx = next_src();
        for (; ks < nk; ++ks) step(ks, std::false_type{}, nx, ks + 2 - nk, std::false_type{});
    }
}

// tile_gemm with only four A fragments in registers (rows 0..3 of the wave's
// eight, then rows 4..7 in the same registers), for a tile GEMM that runs
// while other accumulators stay live.  Changes to the schedule of tile_gemm:
//  * pass A reads rows 4..7 of the current step from stage cur as soon as
//    the matching row 0..3 has issued its last MFMA, so the part of stage
//    cur that holds rows 4..7 (rows 64..127 and 192..255 of the tile) and
//    the A scales are still in use after S1;
//  * hence the loads of step k+2 into those regions (4 A loads per wave and
//    the A scales) are issued in pass B, after the S2 barrier, by which every
//    wave has read them; the 4 other A loads (rows 0..63 and 128..191), the
//    B loads and the B scales go into pass A as before.
// Load u of wave w: u < 4 A rows of region R0, u < 8 A rows of region R1,
// u < 8 + NJ B rows, 8 + NJ B scales, 9 + NJ A scales.  Region R0 is tile rows
// 0..63 and 128..191, R1 the other half; each is 16 loads of 8 rows, load
// t = 4w + (u & 3) of a region covering its rows 8t .. 8t + 7 (t < 8) or
// 128 + 8(t - 8) .. (t >= 8), offset by 64 for R1.
template <int NJ> struct LeanSched;
template <> struct LeanSched<4> {   // 256 x 128 tile: 14 loads, 32 MFMAs per wave
    static constexpr int kLoads = 14, kNA = 9;
    // pass A: R0 A loads 0..3, B loads 8..11, B scales 12
    static constexpr int a_at(int s) {
        return s == 0 ? 0 : s == 2 ? 8 : s == 3 ? 1 : s == 5 ? 9 : s == 6 ? 2 : s == 8 ? 10
             : s == 9 ? 3 : s == 11 ? 11 : s == 13 ? 12 : -1;
    }
    // pass B: R1 A loads 4..7, A scales 13
    static constexpr int b_at(int s) {
        return s == 1 ? 4 : s == 4 ? 5 : s == 6 ? 6 : s == 8 ? 7 : s == 10 ? 13 : -1;
    }
};

// lean_arow(w, u) = lean_arow_base(w) + (u >= 4 ? 64 : 0) + 8 * (u & 3)
__device__ __forceinline__ constexpr int lean_arow_base(int w) { return w < 2 ? 32 * w : 64 + 32 * w; }
__device__ __forceinline__ constexpr int lean_arow(int w, int u) {
    return ((u >= 4) ? 64 : 0) + ((4 * w + (u & 3)) < 8 ? 8 * (4 * w + (u & 3))
                                                       : 128 + 8 * (4 * w + (u & 3) - 8));
}

// The loads of one K step of tile_gemm_lean<NJ>: load u of step ks into
// stage st (the region layout above; steps at or past nk are zero-range).
// Also the tail of the GEMM that runs before it on the same stages.
template <int NJ>
struct LeanLoads {
    TileSrc o;                   // o.aoff is not used: A rows follow the regions
    uint32_t aoffl[8];
    uint32_t smb;
    int wave, nk;
    __device__ LeanLoads(const TileSrc& o_, int64_t lda, uint32_t smb_, int wave_, int lane,
                         int nk_)
        : o(o_), smb(smb_), wave(wave_), nk(nk_) {
        const int dma_row = lane >> 3;
        const int dma_chunk = (lane & 7) ^ (dma_row & 7);
#pragma unroll
        for (int u = 0; u < 8; ++u)
            aoffl[u] = (uint32_t)((lean_arow(wave, u) + dma_row) * lda + dma_chunk * 16);
    }
    template <int u, bool LIVE = false>     // LIVE: ks is known to be < nk
    __device__ __forceinline__ void load(int st, int ks) const {
        const bool live = LIVE || ks < nk;
        const uint32_t k0 = (uint32_t)ks * BK;
        auto rng = [&](const v4i& r) { return live ? r : v4i{r.x, r.y, 0, r.w}; };
        if constexpr (u < 8) {
            dma_b128<(uint32_t)(((u >= 4 ? 64 : 0) + 8 * (u & 3)) * BK)>(
                rng(o.ra), stage_lds<kPartA>(smb, st, lean_arow_base(wave) * BK), aoffl[u], k0);
        } else if constexpr (u < 8 + NJ) {
            dma_b128<(u - 8) * 1024>(rng(o.rb), stage_lds<kPartB>(smb, st, wave * NJ * 1024),
                                     o.boff[u - 8], k0);
        } else if constexpr (u == 8 + NJ) {
            dma_b32(rng(o.sb.rsrc), stage_lds<kPartBs>(smb, st, wave * 64 * 4), o.sb.voff,
                    o.sb.s0 + ks * o.sb.sstep);
        } else {
            dma_b32(rng(o.sa.rsrc), stage_lds<kPartAs>(smb, st, wave * 64 * 4), o.sa.voff,
                    o.sa.s0 + ks * o.sa.sstep);
        }
    }
};

// pre: steps 0 and 1 were issued by the GEMM before it (its tail) into
// stages base and base ^ 1, and step 0 is complete for every wave; step ks
// lives in stage (base + ks) & 1.
template <int NJ>
__device__ __forceinline__ void tile_gemm_lean(v4f (&acc)[8][NJ], GemmSmem& sm, const TileSrc& o,
                                               int nk, int wave, int wm, int wn, int lane,
                                               int64_t lda, int base = 0, bool pre = false) {
    using SC = LeanSched<NJ>;
    const int r16 = lane & 15, q = lane >> 4;
    const int swz = r16 & 7;
    const int b0 = uni(base);
    const LeanLoads<NJ> L(o, lda, uni((int)lds_addr(&sm)), wave, lane, nk);
    auto dma_u = [&](auto uc, int st, int ks) { L.template load<decltype(uc)::value>(st, ks); };
    // the loads of a step known to be inside the K range
    auto dma_live = [&](auto uc, int st, int ks) {
        L.template load<decltype(uc)::value, true>(st, ks);
    };
    v8i af[4], bfr[NJ];
    int asc[4], bsc[NJ];
    // per-lane offsets of the first fragment row, as in tile_gemm
    const int a_row0 = wm * 128 + r16, b_row0 = wn * (NJ * 16) + r16;
    const int a_lo = a_row0 * BK + ((q ^ swz) << 4), a_hi = a_row0 * BK + (((q + 4) ^ swz) << 4);
    const int b_lo = b_row0 * BK + ((q ^ swz) << 4), b_hi = b_row0 * BK + (((q + 4) ^ swz) << 4);
    const int a_s = a_row0 * 4 + q, b_s = b_row0 * 4 + q;
    // row i (0..7) of the wave into register slot i & 3
    auto read_a = [&](auto ic, int st) {
        constexpr int i = decltype(ic)::value;
        const uint8_t* stg = sm.a[st];
        const uint4 lo = *reinterpret_cast<const uint4*>(stg + a_lo + i * 16 * BK);
        const uint4 hi = *reinterpret_cast<const uint4*>(stg + a_hi + i * 16 * BK);
        af[i & 3] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                        (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        asc[i & 3] = (reinterpret_cast<const uint8_t*>(sm.as[st]) + a_s)[i * 16 * 4];
    };
    auto read_b = [&](auto jc, int st) {
        constexpr int j = decltype(jc)::value;
        const uint8_t* stg = sm.b[st];
        const uint4 lo = *reinterpret_cast<const uint4*>(stg + b_lo + j * 16 * BK);
        const uint4 hi = *reinterpret_cast<const uint4*>(stg + b_hi + j * 16 * BK);
        bfr[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        bsc[j] = (reinterpret_cast<const uint8_t*>(sm.bs[st]) + b_s)[j * 16 * 4];
    };
    auto mfma = [&](auto ic, auto jc) {     // ic: wave row 0..7 (register slot ic & 3)
        constexpr int i = decltype(ic)::value, j = decltype(jc)::value;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            bfr[j], af[i & 3], acc[i][j], 0, 0, 0, bsc[j], 0, asc[i & 3]);
    };

    if (!pre) {
        static_for<SC::kLoads>([&](auto uc) { dma_u(uc, b0, 0); });
        static_for<SC::kLoads>([&](auto uc) { dma_u(uc, b0 ^ 1, 1); });
        wait_vmcnt<SC::kLoads>();                       // step 0 (this wave)
        lds_barrier();                                  // step 0 (every wave)
    }
    static_for<4>([&](auto ic) { read_a(ic, b0); });
    static_for<NJ>([&](auto jc) { read_b(jc, b0); });
    auto step = [&](int ks, auto ld) {
        const int cur = (b0 + ks) & 1, nxt = cur ^ 1;
        lds_barrier();                                  // S1: B, R0 and B scales of cur are free
        // pass A: rows 0..3; in the last column row i + 4 replaces row i
        static_for<4 * NJ>([&](auto sc) {
            constexpr int s = decltype(sc)::value;
            mfma(std::integral_constant<int, s % 4>{}, std::integral_constant<int, s / 4>{});
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (s >= 4 * NJ - 4) read_a(std::integral_constant<int, 4 + s % 4>{}, cur);
            constexpr int u = SC::a_at(s);
            if constexpr (u >= 0) ld(std::integral_constant<int, u>{}, cur, ks + 2);
            __builtin_amdgcn_sched_barrier(0);
        });
        wait_vmcnt<SC::kNA>();
        lds_barrier();                                  // S2: stage nxt complete; R1 of cur read
        // pass B: rows 4..7; the next step's B column j after its last MFMA
        // here, row i (0..3) after row i + 4's last MFMA
        static_for<4 * NJ>([&](auto sc) {
            constexpr int s = decltype(sc)::value, j = s / 4, i = 4 + s % 4;
            mfma(std::integral_constant<int, i>{}, std::integral_constant<int, j>{});
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (s % 4 == 3) read_b(std::integral_constant<int, j>{}, nxt);
            if constexpr (s >= 4 * NJ - 4) read_a(std::integral_constant<int, s % 4>{}, nxt);
            constexpr int u = SC::b_at(s);
            if constexpr (u >= 0) ld(std::integral_constant<int, u>{}, cur, ks + 2);
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    int ks = 0;
    for (; ks + 2 < nk; ++ks) step(ks, dma_live);
    for (; ks < nk; ++ks) step(ks, dma_u);
}

// Position of one tile (or split-tail chunk) of a launch.
struct TileLoc {
    int g, chunk;
    int64_t m0, mvalid, n0, klo, K;
};

// One workgroup of four waves (one per SIMD) per CU, persistent over tiles.
// SPLIT (plain store, row-grouped only): the tail-split schedule below.
// TILED (plain store only): both operands carry block scales in the K-step
// tiled layout and the output has no row scale and no group factors, checked
// on the host; the tile sources then test neither for missing scales nor for
// the layout (runtime flags the plain kernel would otherwise keep live across
// its tile loop, at the cost of spilled registers), and the epilogue converts
// the accumulators without a multiply.
template <Epi EPI, bool SPLIT = false, bool TILED = false>
__global__ void __launch_bounds__(NTHREADS, 1)
mx_gemm_kernel(GemmProblem p) {
    static_assert(!TILED || EPI == Epi::kStoreBf16, "TILED: plain tiles only");
    constexpr int kThreads = NTHREADS;
    __shared__ __attribute__((aligned(16))) uint8_t smem[Slot<EPI>::kSmem];
    GemmSmem& sm = *reinterpret_cast<GemmSmem*>(smem);
    __shared__ int s_prefix[kMaxGroups + 1];
    // weight-gradient (k-grouped) launches are plain-store only
    constexpr bool kKgOk = EPI == Epi::kStoreBf16;
    const bool kgroup = kKgOk && p.kgroup;
    __shared__ int s_perm[kKgOk ? kMaxGroups : 1];
    // the plain kernel keeps the offsets in LDS: a global load while its
    // operand loads and output stores are in flight would wait for all of them
    constexpr bool kOffsLds = EPI == Epi::kStoreBf16;
    __shared__ int64_t s_offs[kOffsLds ? kMaxGroups + 1 : 1];
    // likewise its per-group output scales (per-tensor FP8 operands) and
    // each wave's routing weights of its 128 tile rows, for the epilogue
    __shared__ float s_gs[kOffsLds ? kMaxGroups : 1];
    __shared__ float s_rsw[kOffsLds ? 4 * 128 : 1];
    const bool has_gs = p.gsa || p.gsb;
    // the fused epilogues read the tile's routing weights from LDS: a global
    // load in the epilogue would wait (vmcnt) for the output stores in flight
    constexpr bool kRsLds = EPI != Epi::kStoreBf16;
    __shared__ float s_rs[kRsLds ? BM : 1];

    const int tid = threadIdx.x;
    const int lane_id = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int G = p.G;

    // output columns per tile: the gate-up tile pairs 128 gate with 128 up
    // rows of W1 and produces 128 columns of z;
    // columns of F per tile: the recompute backward pairs 128 gate, 128 up
    // and 128 dz columns
    constexpr int TN_OUT = (EPI == Epi::kSwiglu || EPI == Epi::kDSwigluR) ? BN / 2 : BN;
    const int64_t n_out = (EPI == Epi::kSwiglu || EPI == Epi::kDSwigluR) ? p.F : p.N;
    const int ntn = (int)((n_out + TN_OUT - 1) / TN_OUT);
    const int mtn_k = (int)((p.M + BM - 1) / BM);     // k-grouped: M tiles

    // ---- tile table: prefix of tile counts per group (wave 0) ----
    if (wave == 0) {
        int cnt[16];
        int local = 0;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int g = lane_id * 16 + u;
            int c = 0;
            if (g < G) {
                if (kgroup) {
                    c = mtn_k * ntn;
                } else {
                    const int64_t n = p.offs[g + 1] - p.offs[g];
                    c = n > 0 ? (int)((n + BM - 1) / BM) * ntn : 0;
                }
            }
            cnt[u] = c;
            local += c;
        }
        int incl = local;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int o = __shfl_up(incl, d);
            if (lane_id >= d) incl += o;
        }
        int run = incl - local;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int g = lane_id * 16 + u;
            if (g < G) {
                s_prefix[g] = run;
                run += cnt[u];
            }
        }
        if (lane_id == 63) s_prefix[G] = incl;
    }
    if constexpr (kOffsLds) {
        for (int g = tid; g <= G; g += kThreads) s_offs[g] = p.offs[g];
        if (has_gs)
            for (int g = tid; g < G; g += kThreads)
                s_gs[g] = (p.gsa ? p.gsa[g] : 1.0f) * (p.gsb ? p.gsb[g] : 1.0f);
    }
    auto offs_of = [&](int g) -> int64_t {
        if constexpr (kOffsLds) return s_offs[g];
        else return p.offs[g];
    };
    if (kgroup) {
        // longest contraction first (ties: lower group first)
        for (int g = tid; g < G; g += kThreads) {
            int rank = g;
            if (G <= 256) {
                const int64_t kg = p.offs[g + 1] - p.offs[g];
                rank = 0;
                for (int h = 0; h < G; ++h) {
                    const int64_t kh = p.offs[h + 1] - p.offs[h];
                    rank += (kh > kg) || (kh == kg && h < g);
                }
            }
            s_perm[rank] = g;
        }
    }
    __syncthreads();
    const int total = uni(s_prefix[G]);

    // XCD-aware order: workgroup b runs on XCD b % 8; give each XCD a
    // contiguous run of tiles per round.
    const int grid = gridDim.x;
    const int bid = blockIdx.x;
    const int slot = (grid % 8 == 0) ? (bid % 8) * (grid / 8) + bid / 8 : bid;

    // Tail split (plain store, row-grouped): tiles [0, full) run whole; each
    // of the last round's rem tiles runs as S chunks of its K steps, so that
    // round keeps rem * S workgroups busy instead of rem.  full is a multiple
    // of the grid, so the chunks form the last round on their own.
    int full = total, S = 1;
    if constexpr (SPLIT) {
        {
            const int rem = total % grid;
            const int nk_all = (int)(p.K / BK);
            if (rem > 0 && 2 * rem <= grid) {
                S = min(min(grid / rem, kSplitMax), nk_all);
                if (S < 2 || rem * S > kSplitItems) S = 1;
                else full = total - rem;
            }
            if (bid == 0 && tid == 0) {
                SplitHdr* hdr = reinterpret_cast<SplitHdr*>(p.split_ws);
                hdr->rem = S > 1 ? rem : 0;
                hdr->S = S;
            }
        }
    }
    const int items = full + (total - full) * S;

    // Tile w of the launch: its group, first row, valid rows, first output
    // column and K range; chunk >= 0 for a chunk of a split tail tile.
    auto locate = [&](int w) -> TileLoc {
        int t = w, chunk = -1;
        if constexpr (SPLIT) {
            if (w >= full) {
                t = full + (w - full) / S;
                chunk = (w - full) % S;
            }
        }
        int g;
        int64_t m0, mvalid, n0, klo, K;
        int local, mtiles;
        if (kgroup) {
            const int per = mtn_k * ntn;
            const int gi = t / per;
            g = s_perm[gi];
            local = t - gi * per;
            mtiles = mtn_k;
        } else {
            int lo = 0, hi = G - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (s_prefix[mid] <= t) lo = mid; else hi = mid - 1;
            }
            g = lo;
            local = t - s_prefix[g];
            mtiles = (s_prefix[g + 1] - s_prefix[g]) / ntn;
        }
        const int bandsz = BAND * ntn;
        const int band = local / bandsz;
        const int rem = local - band * bandsz;
        const int bm = min(BAND, mtiles - band * BAND);
        const int mt = band * BAND + rem % bm;
        const int nt = rem / bm;
        n0 = (int64_t)nt * TN_OUT;
        if (kgroup) {
            m0 = (int64_t)mt * BM;
            mvalid = min((int64_t)BM, p.M - m0);
            klo = offs_of(g);
            K = offs_of(g + 1) - klo;
        } else {
            const int64_t lo_row = offs_of(g);
            m0 = lo_row + (int64_t)mt * BM;
            mvalid = min((int64_t)BM, offs_of(g + 1) - m0);
            klo = 0;
            K = p.K;
            if constexpr (SPLIT) {
                if (chunk >= 0) {           // K steps [c0, c1) of the tile
                    const int nk_all = (int)(p.K / BK);
                    const int c0 = chunk * nk_all / S, c1 = (chunk + 1) * nk_all / S;
                    klo = (int64_t)c0 * BK;
                    K = (int64_t)(c1 - c0) * BK;
                }
            }
        }
        return TileLoc{uni(g), uni(chunk), uni64(m0), uni64(mvalid), uni64(n0), uni64(klo),
                       uni64(K)};
    };
    auto brow_plain = [](int b) -> int64_t { return b; };

    if constexpr (EPI == Epi::kStoreBf16) {
        // Plain tiles run as one chain per workgroup (tile_gemm_chain): the
        // last two K steps of a tile fetch the next tile's first two, and the
        // epilogue stores from the registers while they land.
        int w = slot;
        if (w < items) {
            TileLoc L = locate(w);
            bool pre = false;
            int base = 0;
            for (;;) {
                const int wnext = w + grid;
                const bool has_next = wnext < items;
                // per-lane offsets from the lane index computed here, so that
                // they are not kept live through the epilogue
                int lane = lane_now();
                const int nk = (int)(L.K / BK);
                auto src_of = [&](const TileLoc& T) {
                    const int64_t bg = kgroup ? 0 : (int64_t)T.g * p.B.gstride;
                    if constexpr (TILED) {
                        MxOperand A = p.A, B = p.B;
                        A.tiled = true;
                        B.tiled = true;
                        return tile_src<false, 8>(A, B, T.m0, T.mvalid, bg + T.n0, p.N - T.n0,
                                                  T.klo, T.K, brow_plain, wave, lane);
                    } else {
                        return tile_src<true, 8>(p.A, p.B, T.m0, T.mvalid, bg + T.n0, p.N - T.n0,
                                                 T.klo, T.K, brow_plain, wave, lane);
                    }
                };
                // this wave's routing weights (its 128 rows; rows past the
                // tile read as 0) into LDS; the main loop's waits cover the
                // loads (every step waits for all but its own newest loads)
                const bool use_rs = !TILED && p.rscale && (!SPLIT || L.chunk < 0);
                if (use_rs) {
                    const int64_t nrw = min((int64_t)128, max((int64_t)0, L.mvalid - wm * 128));
                    const v4i rr = make_rsrc(p.rscale + L.m0 + wm * 128, nrw * 4);
                    const uint32_t la = (uint32_t)uni((int)lds_addr(&s_rsw[wave * 128]));
                    dma_b32(rr, la, (uint32_t)lane * 4u, 0u);
                    dma_b32(rr, la + 256u, (uint32_t)lane * 4u + 256u, 0u);
                }
                v4f acc[8][8];    // written by tile_gemm_chain's first step
                // the next tile's position, found once (while this tile's
                // last K steps run) and kept for the next iteration
                TileLoc Ln{};
                bool have_ln = false;
                const TileSrc o = src_of(L);
                auto next_src = [&]() -> TileNext {
                    if (!has_next) return tile_next(o, 0);
                    Ln = locate(wnext);
                    have_ln = true;
                    return tile_next(src_of(Ln), (int)(Ln.K / BK));
                };
                tile_gemm_chain(acc, sm, o, next_src, nk, base, pre, wave, wm, wn, lane);
                // a chunk of a split tail tile leaves an fp32 partial tile in
                // the workspace, in the four-wave block order (block (i, j)
                // of wave (wm, wn4) holds rows wm*128 + i*16 .., columns
                // wn4*128 + j*16 ..); chunk 0 also records the tile's
                // coordinates
                uint8_t* part = nullptr;
                if (SPLIT && L.chunk >= 0)
                    part = reinterpret_cast<uint8_t*>(split_part(p.split_ws, w - full)) +
                           (int64_t)wave * 64 * 1024;
                if (use_rs && nk == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                store_tile_bf16_regs<!TILED>(acc, p, L.g, L.m0, L.mvalid, L.n0, wm, wn, lane,
                                         has_gs ? s_gs[L.g] : 1.0f,
                                         use_rs ? &s_rsw[wave * 128] : nullptr, part);
                if (SPLIT && L.chunk >= 0) {
                    if (L.chunk == 0 && wave == 0 && lane == 0) {
                        int64_t* meta = reinterpret_cast<SplitHdr*>(p.split_ws)->meta[(w - full) / S];
                        meta[0] = L.g;
                        meta[1] = L.m0;
                        meta[2] = L.mvalid;
                        meta[3] = L.n0;
                    }
                }
                if (!has_next) break;
                pre = nk >= 2;               // tile_gemm_chain switched to the next tile
                base = uni(pre ? (base + nk) & 1 : 0);
                w = wnext;
                L = have_ln ? Ln : locate(w);
            }
        }
        // no load may still be landing in LDS when the workgroup ends
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
        for (int t0 = 0; t0 < items; t0 += grid) {
            const int w = t0 + slot;
            if (w >= items) break;
            // Per-lane offsets are derived per tile from the lane index computed
            // here: hoisted out of the tile loop they would stay live through
            // the epilogue, which needs every register it can get.
            int lane = lane_now();
            const int r16 = lane & 15, q = lane >> 4;
            const int swz = r16 & 7;
            const TileLoc L = locate(w);
            const int g = L.g;
            const int64_t m0 = L.m0, mvalid = L.mvalid, n0 = L.n0, klo = L.klo, K = L.K;
            const int nk = (int)(K / BK);

            // ---- main loop(s) ----
            // The fused gate-up tile pairs 128 gate with 128 up rows of W1 (gate
            // and up halves are F rows apart): B row b of the tile is W1 row
            // half * F + n0 + (b >> 7) * 64 + (b & 63), half = (b >> 6) & 1, so
            // wave wn's 128 B rows are the gate then the up rows of its 64 output
            // columns.  Plain tiles read B rows n0 + b.
            auto brow_gu = [&](int b) -> int64_t {
                return ((b >> 6) & 1) * p.F + n0 + (b >> 7) * 64 + (b & 63);
            };
            const int64_t bg = kgroup ? 0 : (int64_t)g * p.B.gstride;
            constexpr bool kGU = EPI == Epi::kSwiglu || EPI == Epi::kDSwigluR;
            // the routing weights of rows m0 .. m0 + 255 (zero past mvalid) into
            // s_rs, ahead of the first operand loads, so the main loop's first
            // wait covers them; the previous tile's epilogue has left s_rs
            // (its closing barrier)
            if constexpr (kRsLds) {
                const v4i rr = make_rsrc(p.rscale + m0, mvalid * 4);
                dma_b32(rr, uni((int)lds_addr(&s_rs[wave * 64])), (uint32_t)(wave * 64 + lane) * 4u,
                        0u);
            }
            v4f acc[8][8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
            // the recompute backward's dz GEMM (A2: dY rowwise, B2: W2
            // columnwise, K = H) for the tile's rows and 128 columns of F
            auto dz_src = [&](int ln) {
                return tile_src<false, 4>(p.A2, p.B2, m0, mvalid, (int64_t)g * p.B2.gstride + n0,
                                          p.F - n0, 0, K, brow_plain, wave, ln);
            };
            if constexpr (EPI == Epi::kDSwigluR) {
                // [a | b]'s last two K steps fetch the dz GEMM's first two (its
                // loads 0..13 in the slots of loads 0..13, the 4 slots left as
                // zero-range loads into the half of the B stage the dz GEMM
                // does not use), so that GEMM starts without a prologue
                const TileSrc o = tile_src<false, 8>(p.A, p.B, m0, mvalid, bg, 2 * p.F, klo, K,
                                                     brow_gu, wave, lane);
                const uint32_t smb = uni((int)lds_addr(&sm));
                auto make_tail = [&]() {
                    int lane3 = lane_now();
                    const LeanLoads<4> L(dz_src(lane3), p.A2.ld, smb, wave, lane3, nk);
                    return [L, smb, wave](auto uc, int st, int kn) {
                        constexpr int u = decltype(uc)::value;
                        if constexpr (u < LeanSched<4>::kLoads) {
                            L.template load<u>(st, kn);
                        } else {
                            const v4i z{L.o.rb.x, L.o.rb.y, 0, L.o.rb.w};
                            dma_b128(z, stage_lds<kPartB>(smb, st, (16 + wave * 4 + (u - 14)) * 1024),
                                     0u, 0u);
                        }
                    };
                };
                static_assert(Sched<8>::kLoads == LeanSched<4>::kLoads + 4, "tail slots");
                tile_gemm<8>(acc, sm, o, nk, wave, wm, wn, lane, make_tail);
            } else if constexpr (kGU) {
                const TileSrc o = tile_src<false, 8>(p.A, p.B, m0, mvalid, bg, 2 * p.F, klo, K,
                                                     brow_gu, wave, lane);
                tile_gemm<8>(acc, sm, o, nk, wave, wm, wn, lane);
            } else {
                const TileSrc o = tile_src<false, 8>(p.A, p.B, m0, mvalid, bg + n0, p.N - n0, klo,
                                                     K, brow_plain, wave, lane);
                tile_gemm<8>(acc, sm, o, nk, wave, wm, wn, lane);
            }
            // The fused epilogues stage their outputs in LDS, which overlaps every
            // wave's operand stages: wait until the trailing (zero-range) loads of
            // all waves have landed (before the dz GEMM only if [a | b] did not
            // chain into it).
            const bool chained = EPI == Epi::kDSwigluR && nk >= 2;
            if (!chained) {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                lds_barrier();
            }
            // Recompute backward: the second GEMM of the tile, dz = dY . W2 for
            // the same rows and the tile's 128 columns of F, while acc keeps the
            // recomputed [a | b].
            v4f dacc[8][4];
            if constexpr (EPI == Epi::kDSwigluR) {
                // each block its own zero: one zero shared by all of them (as
                // the compiler would make it) keeps the loop-carried blocks
                // from getting their own registers, and the dz loop then
                // moves accumulators around every step
#pragma unroll
                for (int i = 0; i < 8; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        dacc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
                        asm volatile("" : "+a"(dacc[i][j]));
                    }
                int lane2 = lane_now();
                tile_gemm_lean<4>(dacc, sm, dz_src(lane2), nk, wave, wm, wn, lane2, p.A2.ld,
                                  nk & 1, chained);
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                lds_barrier();
            }

            // ---- epilogue ----
            // B is the MFMA's first operand, so acc[i][j] holds the transposed
            // 16 x 16 block: lane (r16, q) has row i*16 + r16 of the wave tile and
            // its 4 consecutive columns j*16 + 4q + v.
            const int64_t rwave = m0 + wm * 128;          // first row of this wave
            const int rows_valid_w = (int)min((int64_t)128, max((int64_t)0, mvalid - wm * 128));

            if constexpr (EPI == Epi::kSwiglu) {
                // acc[i][j], j < 4: gate; acc[i][j+4]: up, same output columns
                const int64_t F = p.F;
                const int64_t glo = p.offs[g];
                const int64_t prow = p.poff[g] + (rwave - glo);       // padded position
                const int64_t npad = p.poff[g + 1] - p.poff[g];
                const int rows_pad_w = (int)min((int64_t)128, max((int64_t)0, npad - (rwave - glo)));
                const int64_t cw = n0 + wn * 64;                       // wave's first z column
                const QDest d{p.qr, p.qrs, p.ldqr, p.qc, p.qcs, p.ldqc, cw, F, false, p.qtiled};
                uint8_t* st = smem + wave * Slot<EPI>::kBytes;
#pragma nounroll
                for (int ip = 0; ip < 4; ++ip) {
                    // Lane-derived values are re-derived from the lane index in
                    // every slice: hoisted out of the tile loop they would stay
                    // live through the main loop and crowd out the accumulators.
                    int lane = lane_now();
                    const int r16 = lane & 15, q = lane >> 4;
                    float rr[2];
#pragma unroll
                    for (int ii = 0; ii < 2; ++ii) {
                        const int rl = (2 * ip + ii) * 16 + r16;
                        rr[ii] = rl < rows_valid_w ? s_rs[wm * 128 + rl] : 0.0f;
                    }
                    static_for<2>([&](auto jpc) {
                        constexpr int jp = decltype(jpc)::value;
                        float gu[2][2][4], uu[2][2][4], z[2][2][4];
                        pick_unit<2 * jp>(acc, ip, gu);
                        pick_unit<2 * jp + 4>(acc, ip, uu);
                        // Rows past the expert's valid rows (they take part in
                        // the token-axis blocks) hold exact zeros: their codes
                        // read as zero through the range checks and their scales
                        // are finite (the quantizer writes the tiled layout's
                        // padding rows), and their routing weights are zero.
#pragma unroll
                        for (int ii = 0; ii < 2; ++ii) {
                            const int i = 2 * ip + ii;
#pragma unroll
                            for (int jj = 0; jj < 2; ++jj) {
                                const int j = 2 * jp + jj;
                                if (p.h && rows_pad_w > 0) {
                                    const uint2 g2 = pack4_bf16(gu[ii][jj]), u2 = pack4_bf16(uu[ii][jj]);
                                    store_nt(h_block(p.h, prow + i * 16, cw + j * 16, F, lane),
                                             make_uint4(g2.x, g2.y, u2.x, u2.y));
                                }
#pragma unroll
                                for (int v = 0; v < 4; ++v) {
                                    float sg;
                                    z[ii][jj][v] = rr[ii] * (silu_sig(gu[ii][jj][v], sg) * uu[ii][jj][v]);
                                }
                            }
                        }
                        quant_unit<64>(z, 2 * jp * 16, ip, st, lane);
                    });
                    lds_wait();
                    flush_rows<64, true>(st, d, rwave, ip, rows_valid_w, lane);
                    if ((ip & 1) && rows_pad_w > 0) flush_cols<64, true>(st, d, prow + (ip >> 1) * 64, lane);
                    lds_wait();
                }
                if (rows_pad_w > 0) flush_col_scales<64>(st, d, prow, lane);
            } else if constexpr (EPI == Epi::kDSwiglu) {
                const int64_t F = p.F;
                const int64_t glo = p.offs[g];
                const int64_t prow = p.poff[g] + (rwave - glo);
                const int64_t npad = p.poff[g + 1] - p.poff[g];
                const int rows_pad_w = (int)min((int64_t)128, max((int64_t)0, npad - (rwave - glo)));
                const int64_t cw = n0 + wn * 128;
                const QDest d{p.qr, p.qrs, p.ldqr, p.qc, p.qcs, p.ldqc, cw, F, true, p.qtiled};
                uint8_t* st = smem + wave * Slot<EPI>::kBytes;
                const int part = (int)(n0 / BN) * 2 + wn;
                // h = [a | b] of unit (ip, jp) (32 rows x 32 columns) is four 1 KiB
                // blocks, each moved by one global->LDS load into the unit's buffer
                // of the ring.  While slice ip is processed, unit jp's buffer is
                // refilled with unit (ip + 1, jp), so each load has a whole slice
                // to land.  Blocks past F or past the padded rows use a zero-range
                // descriptor (zeros, masked); the last slice loads nothing.
                uint8_t* const ring = st + QStage<256>::kBytes;
                auto dma_unit = [&](int ipn, auto jpc, int lane) {
                    constexpr int jp = decltype(jpc)::value;
#pragma unroll
                    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                        for (int jj = 0; jj < 2; ++jj) {
                            const int64_t col = cw + (2 * jp + jj) * 16;
                            const bool in = rows_pad_w > 0 && col < F && ipn < 4;
                            const uint8_t* blk = reinterpret_cast<const uint8_t*>(p.h) +
                                (((prow >> 4) + 2 * ipn + ii) * (F >> 4) + (col >> 4)) * 1024;
                            const v4i rs = make_rsrc(in ? blk : reinterpret_cast<const uint8_t*>(p.h),
                                                     in ? 1024 : 0);
                            dma_b128(rs, uni(lds_addr(ring + ((jp * 2 + ii) * 2 + jj) * 1024)),
                                     (uint32_t)lane * 16, 0);
                        }
                };
                static_for<4>([&](auto jpc) { dma_unit(0, jpc, lane); });
#pragma nounroll
                for (int ip = 0; ip < 4; ++ip) {
                    // Lane-derived values are re-derived from the lane index in
                    // every slice: hoisted out of the tile loop they would stay
                    // live through the main loop and crowd out the accumulators.
                    int lane = lane_now();
                    const int r16 = lane & 15, q = lane >> 4;
                    float rr[2], drs[2];
#pragma unroll
                    for (int ii = 0; ii < 2; ++ii) {
                        const int rl = (2 * ip + ii) * 16 + r16;
                        rr[ii] = rl < rows_valid_w ? s_rs[wm * 128 + rl] : 0.0f;
                        drs[ii] = 0.f;
                    }
                    static_for<4>([&](auto jpc) {
                        constexpr int jp = decltype(jpc)::value;
                        float dzu[2][2][4], da[2][2][4], db[2][2][4];
                        uint4 hb[2][2];
                        // this unit's ring loads: 12 younger ring loads follow them,
                        // except in the last slice, which issues none
                        if (ip < 3) {
                            asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
                        } else {
                            if constexpr (jp == 0) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
                            if constexpr (jp == 1) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
                            if constexpr (jp == 2) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
                            if constexpr (jp == 3) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                        }
#pragma unroll
                        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                            for (int jj = 0; jj < 2; ++jj)
                                hb[ii][jj] = *reinterpret_cast<const uint4*>(
                                    ring + ((jp * 2 + ii) * 2 + jj) * 1024 + lane * 16);
                        lds_wait();                 // the buffer is free for the next slice's unit
                        if (ip < 3) dma_unit(ip + 1, jpc, lane);
                        pick_unit<2 * jp>(acc, ip, dzu);
                        // Rows past the expert's valid rows get dz = 0 by a select
                        // (rows past M read never-written scale bytes, so their
                        // accumulators may be anything, NaN included); their h is
                        // 0 (the forward stores 0 there), so da = db = 0 in the
                        // token-axis blocks they share with valid rows.  A wave's
                        // columns are all below F or all past it (dz = 0 from
                        // zero-filled B rows, h loads of zero range).
#pragma unroll
                        for (int ii = 0; ii < 2; ++ii) {
                            const bool rv = (2 * ip + ii) * 16 + r16 < rows_valid_w;
#pragma unroll
                            for (int jj = 0; jj < 2; ++jj) {
                                float a[4], b[4];
                                const uint4 hv = hb[ii][jj];
                                unpack4_bf16(make_uint2(hv.x, hv.y), a);
                                unpack4_bf16(make_uint2(hv.z, hv.w), b);
#pragma unroll
                                for (int v = 0; v < 4; ++v) {
                                    const float av = a[v], bv = b[v];
                                    const float dz = rv ? dzu[ii][jj][v] : 0.f;
                                    float sg;
                                    const float sl_ = silu_sig(av, sg);
                                    drs[ii] += dz * (sl_ * bv);
                                    const float ds = rr[ii] * dz;
                                    da[ii][jj][v] = ds * bv * sg * (1.0f + av * (1.0f - sg));
                                    db[ii][jj][v] = ds * sl_;
                                }
                            }
                        }
                        quant_unit<256>(da, 2 * jp * 16, ip, st, lane);
                        quant_unit<256>(db, 128 + 2 * jp * 16, ip, st, lane);
                    });
#pragma unroll
                    for (int ii = 0; ii < 2; ++ii) {
                        const float sum = sum4q(drs[ii]);
                        const int rl = (2 * ip + ii) * 16 + r16;
                        if (q == 0 && rl < rows_valid_w) p.drp[(int64_t)part * p.lddrp + rwave + rl] = sum;
                    }
                    // the wave's 128 columns are all below F or all at or past it
                    lds_wait();
                    if (cw < F) flush_rows<256, false>(st, d, rwave, ip, rows_valid_w, lane);
                    if (cw < F && rows_pad_w > 0) flush_cols<256, false>(st, d, prow + ip * 32, lane);
                    lds_wait();
                }
                if (cw < F && rows_pad_w > 0) flush_col_scales<256>(st, d, prow, lane);
            } else {   // kDSwigluR
                // acc holds the recomputed [a | b] (acc[i][j], j < 4: gate; j + 4:
                // up, same columns) and dacc the dz of the wave's 64 columns of F
                // (cw .. cw + 63, all below F since F % 128 == 0).  dh = [da | db]
                // leaves as rowwise codes (da at columns cw.., db at F + cw..) and
                // token-axis codes; dr partial part = the wave's column block.
                const int64_t F = p.F;
                const int64_t glo = p.offs[g];
                const int64_t prow = p.poff[g] + (rwave - glo);
                const int64_t npad = p.poff[g + 1] - p.poff[g];
                const int rows_pad_w = (int)min((int64_t)128, max((int64_t)0, npad - (rwave - glo)));
                const int64_t cw = n0 + wn * 64;
                const QDest d{p.qr, p.qrs, p.ldqr, p.qc, p.qcs, p.ldqc, cw, F, true, p.qtiled};
                uint8_t* st = smem + wave * Slot<EPI>::kBytes;
                const int part = (int)(n0 / 128) * 2 + wn;
                // the last slice's [a | b] to the stash: 384 accumulators plus the
                // epilogue's working set would not fit the registers
                uint8_t* const stash = st + QStage<128>::kBytes;
                static_for<2>([&](auto iic) {
                    constexpr int ii = decltype(iic)::value;
                    static_for<8>([&](auto jc) {
                        constexpr int j = decltype(jc)::value;
                        *reinterpret_cast<v4f*>(stash + ((ii * 8 + j) * 64 + lane) * 16) = acc[6 + ii][j];
                    });
                });
#pragma nounroll
                for (int ip = 0; ip < 4; ++ip) {
                    // lane-derived values re-derived per slice (see the forward)
                    int lane = lane_now();
                    const int r16 = lane & 15, q = lane >> 4;
                    float rr[2], drs[2];
#pragma unroll
                    for (int ii = 0; ii < 2; ++ii) {
                        const int rl = (2 * ip + ii) * 16 + r16;
                        rr[ii] = rl < rows_valid_w ? s_rs[wm * 128 + rl] : 0.0f;
                        drs[ii] = 0.f;
                    }
                    static_for<2>([&](auto jpc) {
                        constexpr int jp = decltype(jpc)::value;
                        float ga[2][2][4], ua[2][2][4], dzu[2][2][4], da[2][2][4], db[2][2][4];
                        pick_unit_stashed<2 * jp>(acc, ip, ga, stash, lane);
                        pick_unit_stashed<2 * jp + 4>(acc, ip, ua, stash, lane);
                        pick_unit<2 * jp>(dacc, ip, dzu);
                        // Rows past the expert's valid rows (they take part in
                        // the token-axis blocks) hold exact zeros in a, b and dz,
                        // as in the forward, and zero routing weights.
#pragma unroll
                        for (int ii = 0; ii < 2; ++ii) {
#pragma unroll
                            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                                for (int v = 0; v < 4; ++v) {
                                    const float av = ga[ii][jj][v];
                                    const float bv = ua[ii][jj][v];
                                    const float dz = dzu[ii][jj][v];
                                    float sg;
                                    const float sl_ = silu_sig(av, sg);
                                    drs[ii] += dz * (sl_ * bv);
                                    const float ds = rr[ii] * dz;
                                    da[ii][jj][v] = ds * bv * sg * (1.0f + av * (1.0f - sg));
                                    db[ii][jj][v] = ds * sl_;
                                }
                        }
                        quant_unit<128>(da, 2 * jp * 16, ip, st, lane);
                        quant_unit<128>(db, 64 + 2 * jp * 16, ip, st, lane);
                    });
#pragma unroll
                    for (int ii = 0; ii < 2; ++ii) {
                        const float sum = sum4q(drs[ii]);
                        const int rl = (2 * ip + ii) * 16 + r16;
                        if (q == 0 && rl < rows_valid_w) p.drp[(int64_t)part * p.lddrp + rwave + rl] = sum;
                    }
                    lds_wait();
                    flush_rows<128, false>(st, d, rwave, ip, rows_valid_w, lane);
                    if ((ip & 1) && rows_pad_w > 0) flush_cols<128, false>(st, d, prow + (ip >> 1) * 64, lane);
                    lds_wait();
                }
                if (rows_pad_w > 0) flush_col_scales<128>(st, d, prow, lane);
            }
            // the next tile's loads overwrite other waves' staging areas
            lds_barrier();
        }
    }
}

// The partials are part-major ([nparts][M]), so each part's loads are
// coalesced across the rows of a wave; the sum runs over j in ascending order.
__global__ void __launch_bounds__(256)
dr_reduce_kernel(const float* __restrict__ drp, int64_t M, int64_t nparts,
                 float* __restrict__ dr) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= M) return;
    float s = 0.f;
#pragma unroll 32
    for (int64_t j = 0; j < nparts; ++j) s += drp[j * M + i];
    dr[i] = s;
}

// Sum of the S partial tiles of each split tail tile (chunk order fixed),
// with the plain epilogue's scaling and bf16 rounding.  One thread per 4
// consecutive outputs (one v4f of the partial layout: lane (r16, q) of block
// (i, j) of wave w holds row wm*128 + i*16 + r16, columns wn*128 + j*16 + 4q
// .. +3), 64 workgroups per tail tile; the grid covers the largest possible
// tail and workgroups past the recorded count exit.
__global__ void __launch_bounds__(256)
split_fixup_kernel(GemmProblem p) {
    const SplitHdr* hdr = reinterpret_cast<const SplitHdr*>(p.split_ws);
    const int rem = hdr->rem, S = hdr->S;
    const int tb = blockIdx.x >> 6;
    if (tb >= rem) return;
    const int f4 = (blockIdx.x & 63) * 256 + threadIdx.x;     // v4f index in the tile
    const int lane = f4 & 63, blk = f4 >> 6;                   // blk = w * 64 + i * 8 + j
    const int w = blk >> 6, i = (blk >> 3) & 7, j = blk & 7;
    const int64_t* meta = hdr->meta[tb];
    const int g = (int)meta[0];
    const int64_t m0 = meta[1], mvalid = meta[2], n0 = meta[3];
    const int rl = (w >> 1) * 128 + i * 16 + (lane & 15);
    const int64_t col = n0 + (w & 1) * 128 + j * 16 + 4 * (lane >> 4);
    if (rl >= mvalid || col >= p.N) return;
    const float* part = split_part(p.split_ws, tb * S) + (int64_t)f4 * 4;
    v4f sum = *reinterpret_cast<const v4f*>(part);
    for (int c = 1; c < S; ++c) sum += *reinterpret_cast<const v4f*>(part + (int64_t)c * (BM * BN));
    const int64_t row = m0 + rl;
    const float gs = (p.gsa ? p.gsa[g] : 1.0f) * (p.gsb ? p.gsb[g] : 1.0f);
    const float sc = p.rscale ? p.rscale[row] * gs : gs;
    float v[4] = {sum[0] * sc, sum[1] * sc, sum[2] * sc, sum[3] * sc};
    uint16_t* C = reinterpret_cast<uint16_t*>(p.C);
    *reinterpret_cast<uint2*>(C + row * p.ldc + col) = pack4_bf16(v);
}

}  // namespace

hipError_t launch_split_fixup(const GemmProblem& p, hipStream_t s) {
    if (!p.split_ws || p.kgroup) return hipSuccess;
    hipLaunchKernelGGL(split_fixup_kernel, dim3(64 * (kSplitItems / 2)), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_mx_gemm(const GemmProblem& p, Epi epi, hipStream_t s) {
    int grid = device_cu_count();
    grid = grid < 8 ? 8 : grid / 8 * 8;
    switch (epi) {
        case Epi::kStoreBf16: {
            const bool split = p.split_ws && !p.kgroup;
            const bool tiled = p.A.scales && p.B.scales && p.A.tiled && p.B.tiled && !p.rscale &&
                               !p.gsa && !p.gsb;
            auto go = [&](auto kern) {
                hipLaunchKernelGGL(kern, dim3(grid), dim3(NTHREADS), 0, s, p);
            };
            if (tiled) {
                if (split) go(mx_gemm_kernel<Epi::kStoreBf16, true, true>);
                else go(mx_gemm_kernel<Epi::kStoreBf16, false, true>);
            } else {
                if (split) go(mx_gemm_kernel<Epi::kStoreBf16, true, false>);
                else go(mx_gemm_kernel<Epi::kStoreBf16, false, false>);
            }
            break;
        }
        case Epi::kSwiglu:
            hipLaunchKernelGGL(mx_gemm_kernel<Epi::kSwiglu>, dim3(grid), dim3(NTHREADS), 0, s, p);
            break;
        case Epi::kDSwiglu:
            hipLaunchKernelGGL(mx_gemm_kernel<Epi::kDSwiglu>, dim3(grid), dim3(NTHREADS), 0, s, p);
            break;
        case Epi::kDSwigluR:
            hipLaunchKernelGGL(mx_gemm_kernel<Epi::kDSwigluR>, dim3(grid), dim3(NTHREADS), 0, s, p);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_dr_reduce(const float* drp, int64_t M, int64_t nparts,
                            float* dr, hipStream_t s) {
    if (M == 0) return hipSuccess;
    hipLaunchKernelGGL(dr_reduce_kernel, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, s,
                       drp, M, nparts, dr);
    return hipGetLastError();
}

}  // namespace mx
