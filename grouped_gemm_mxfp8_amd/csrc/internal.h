// Internal launchers shared by the kernel files and the C-ABI layer.  Every
// launcher enqueues on `stream`, returns the hipError_t of the launch, and
// assumes the C-ABI layer has validated its arguments.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

constexpr int kTokenAlign = 128;   // padding of token groups in columnwise copies
constexpr int kMaxGroups = 1024;   // largest expert count the kernels accept

// Scale layouts of a K-major MXFP8 operand with rows r and Kp codes per row
// (one E8M0 scale per 32 codes, block kb = k / 32):
//  * row-major:     byte r * (Kp / 32) + kb.
//  * K-step tiled:  the 4 scales of one GEMM K step (128 codes) of 32
//    consecutive rows form one 128-byte line, so a K step of a 256-row tile
//    reads 8 lines instead of 256:
//      byte ((r / 32) * (Kp / 128) + kb / 4) * 128 + (r % 32) * 4 + kb % 4,
//    Kp % 128 == 0, rows padded to a multiple of 32.  The tile quantizer
//    writes code 0 (2^-127) into the padding rows' scale bytes, so that the
//    fused GEMMs, whose token-axis outputs take in rows past the last valid
//    one, accumulate exact zeros for them (their codes read as zero through
//    the range checks); other kernels' padding scale bytes are not written,
//    and the GEMM rows that read them are not stored.
__host__ __device__ inline int64_t tiled_scale_offset(int64_t r, int64_t kb, int64_t Kp) {
    return ((r >> 5) * (Kp >> 7) + (kb >> 2)) * 128 + (r & 31) * 4 + (kb & 3);
}
inline int64_t tiled_scale_bytes(int64_t rows, int64_t Kp) {
    return (rows + 31) / 32 * 32 * (Kp / 32);
}

// ---- quantizer --------------------------------------------------------------
// Padded offsets of token groups: poff[g] = sum_{j<g} ceil(n_j/128)*128.
hipError_t launch_padded_offsets(const int64_t* offs, int G, int64_t* poff,
                                 hipStream_t s);
// Rowwise copy only, over a flat [rows][C] tensor (tiled: K-step tiled
// scales, C % 128 == 0).
hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int64_t C,
                             uint8_t* codes, uint8_t* scales, bool tiled, hipStream_t s);
// Copy rows of n bytes into rows of np bytes (np >= n), the bytes past n set
// to fill; 16-byte aligned src and dst.
hipError_t launch_pad_rows(const uint8_t* src, int64_t rows, int64_t n, uint8_t* dst, int64_t np,
                           uint8_t fill, hipStream_t s);
// Tile pass: rowwise (optional) and columnwise (optional) copies of
// x[batch][R][C].  Grouped mode (offs != nullptr, batch == 1) needs poff
// already computed; row_bound is the padded-length bound (multiple of 128).
// tiled: both copies get K-step tiled scales (rowwise: rows = batch*R, Kp = C,
// needs C % 128 == 0 and R % 32 == 0 when batch > 1; columnwise: rows =
// batch*C, Kp = ld).
// gather (optional, batch == 1): row i of the tiled tensor is source row
// gather[i] of x (src_rows rows; negative entries read as zeros).
hipError_t launch_quant_tiles(const uint16_t* x, int64_t batch, int64_t R,
                              int64_t C, const int64_t* offs,
                              const int64_t* poff, int G, int64_t row_bound,
                              uint8_t* rc, uint8_t* rs, uint8_t* cc,
                              uint8_t* cs, int64_t ld, bool tiled, hipStream_t s,
                              const int32_t* gather = nullptr, int64_t src_rows = 0);

// ---- grouped GEMMs ------------------------------------------------------------
// Operand of a K-major MXFP8 GEMM: codes [rows][ld], scales row-major
// [rows][ld/32] or K-step tiled (Kp = ld).  scales == nullptr: every block
// scale is 1 (code 127), for FP8 operands that carry one scale per group.
struct MxOperand {
    const uint8_t* codes;
    const uint8_t* scales;
    int64_t ld;          // bytes between rows of codes
    int64_t gstride;     // rows between consecutive groups (0: shared)
    bool tiled = false;  // scale layout
};

enum class Epi : int {
    kStoreBf16 = 0,   // C = acc (* row scale) -> bf16
    kSwiglu = 1,      // gate-up: h -> bf16, z = r silu(a) b -> MXFP8 row+col
    kDSwiglu = 2,     // dz -> dr partials, dh = [da|db] -> MXFP8 row+col (h read)
    kDSwigluR = 3,    // [a|b] = X W1^T recomputed, dz = dY W2 (A2, B2) in the
                      //   same tile -> dr partials, dh -> MXFP8 row+col
};

struct GemmProblem {
    // row-grouped (fprop/dgrad): groups split M via offs; B of group g at
    //   rows g*gstride.  k-grouped (wgrad): groups split K via offs; C of
    //   group g at c + g*c_gstride; A and B shared.
    bool kgroup;
    const int64_t* offs;
    int G;
    int64_t M, N, K;            // K unused when kgroup
    MxOperand A, B;
    void* C;                    // bf16
    int64_t ldc, c_gstride;
    const float* rscale;        // kStoreBf16 and fused: per-row routing weight
    // fused epilogues
    int64_t F;
    uint16_t* h;                // kSwiglu writes (if set), kDSwiglu reads: bf16 [M][2F]
    uint8_t* qr; uint8_t* qrs; int64_t ldqr;   // rowwise MXFP8 output
    uint8_t* qc; uint8_t* qcs; int64_t ldqc;   // columnwise MXFP8 output
    bool qtiled;                // fused outputs: K-step tiled scales
    const int64_t* poff;        // padded token offsets of the column copy
    float* drp; int64_t lddrp;  // kDSwiglu(R): dr partials, part j of row i at drp[j * lddrp + i]
    const float* gsa;           // kStoreBf16: per-group factors of A and of B
    const float* gsb;           //   (scale_inv of per-tensor FP8), or nullptr
    uint8_t* split_ws;          // kStoreBf16, row-grouped: tail-split workspace
                                //   of kSplitWsBytes, or nullptr (no split)
    // kDSwigluR: operands of the tile's second GEMM, dz = A2 . B2^T (A2
    // row-grouped like A, B2 of group g at rows g * B2.gstride; K = K)
    MxOperand A2, B2;
};

// Tail split of the plain-store row-grouped GEMM.  When the last round of
// output tiles would leave more than half of the persistent workgroups idle,
// each of its tiles is cut along K into S <= kSplitMax chunks, one workgroup
// per chunk; the chunks' fp32 partial tiles go to split_ws and
// launch_split_fixup (same stream, right after the GEMM) adds them in chunk
// order and stores the tiles.  Workspace: a header (tail tile count, S and
// each tail tile's coordinates) and kSplitItems partial tiles of 256 x 256
// fp32.
constexpr int kSplitMax = 4;
constexpr int kSplitItems = 256;
constexpr size_t kSplitHdrBytes = 8192;
constexpr size_t kSplitWsBytes = kSplitHdrBytes + (size_t)kSplitItems * 256 * 256 * 4;

hipError_t launch_mx_gemm(const GemmProblem& p, Epi epi, hipStream_t s);
hipError_t launch_split_fixup(const GemmProblem& p, hipStream_t s);

// Sum of dr partials: dr[i] = sum_j drp[j * M + i], j ascending.
hipError_t launch_dr_reduce(const float* drp, int64_t M, int64_t nparts,
                            float* dr, hipStream_t s);

// BF16 grouped GEMM (row-grouped): y = x w_e^T (* rscale).
hipError_t launch_bf16_grouped(const uint16_t* x, const int64_t* offs, int G,
                               int64_t M, const uint16_t* w, int64_t N,
                               int64_t K, const float* rscale, uint16_t* y,
                               hipStream_t s);

// ---- routing: sorted-row plan, combine ---------------------------------------
// Plan of a top-k routing ids [T][k] (values in [0, E); others are skipped:
// row_of = -1 and no row): offsets [E+1], row_of [T*k], tok_of [M], and
// r_sorted [M] = w of each row when w is given.  hist: route_chunks(T*k) * E
// int32 of scratch.
int64_t route_chunks(int64_t n);
// The library-owned plan scratch of the no-allocation entry point:
// kPlanScratchInts int32 per GPU (4 MiB); *out = its device address on the
// current device (looked up once per device).
constexpr int64_t kPlanScratchInts = (int64_t)1 << 20;
hipError_t route_plan_scratch(int32_t** out);
// Top-k of logits [T][E] (E <= kMaxGroups, 1 <= k <= min(E, 64)) and the
// softmax of the k selected: ids [T][k] in selection order, w [T][k].
hipError_t launch_router(const float* logits, int64_t T, int E, int k, int32_t* ids, float* w,
                         hipStream_t s);
hipError_t launch_route_plan(const int32_t* ids, int64_t T, int k, int E, const float* w,
                             int64_t* offsets, int32_t* row_of, int32_t* tok_of,
                             float* r_sorted, int32_t* hist, hipStream_t s);
// out [T][H] = sum_j c_tj y[row_of[t][j]] (c = w, or 1 when w is null); H % 8 == 0.
hipError_t launch_combine(const uint16_t* y, const int32_t* row_of, const float* w, int64_t T,
                          int k, int64_t H, int64_t M, uint16_t* out, hipStream_t s);
// dy[row_of[t][j]] = c_tj dout[t]; dw [T][k] = <dout[t], y[row_of[t][j]]> when
// dw is given (y then needed).
hipError_t launch_combine_bwd(const uint16_t* dout, const int32_t* row_of, const float* w,
                              const uint16_t* y, int64_t T, int k, int64_t H, int64_t M,
                              uint16_t* dy, float* dw, hipStream_t s);

// ---- per-tensor FP8 ------------------------------------------------------------
// Codes [rows][C] of x [rows][C] (C % 32 == 0, 256 * C < 2^31) with one scale
// per group: row groups offs [G+1], or matrices of R rows when offs is null
// (rows = G * R).  amax [G] (fp32 bits) and scale_inv [G] are written.
hipError_t launch_fp8_tensor_quant(const uint16_t* x, int64_t rows, int64_t C,
                                   const int64_t* offs, int G, int64_t R, uint32_t* amax,
                                   uint8_t* codes, float* scale_inv, hipStream_t s);

int device_cu_count();

}  // namespace mx
