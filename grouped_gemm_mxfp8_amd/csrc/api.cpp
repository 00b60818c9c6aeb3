// C-ABI layer of the MXFP8 MoE expert path: argument validation (host only,
// before any HIP call), layout of the saved-for-backward context and of the
// workspaces, and the launch sequence of each entry point on the caller's
// stream.  Nothing on the compute path allocates, frees or synchronises; only
// the opt-in launch-timing calls (mx_profile_*) create and wait on events.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "../../include/mxmoe.h"
#include "internal.h"

namespace {

thread_local std::string g_err;

mx_status fail(mx_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

mx_status ok() {
    g_err.clear();
    return MX_OK;
}

mx_status launched(hipError_t e, const char* what) {
    if (e != hipSuccess)
        return fail(MX_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

// ---- launch timing (mx_profile_*) ------------------------------------------
struct ProfRec {
    const char* name;
    double work;
    int unit;
    hipEvent_t a, b;
};
struct Profiler {
    bool on = false;
    int cap = 0;
    std::vector<hipEvent_t> pool;
    std::vector<ProfRec> recs;
    void release() {
        for (hipEvent_t e : pool) (void)hipEventDestroy(e);
        pool.clear();
        recs.clear();
        cap = 0;
    }
};
thread_local Profiler g_prof;

// Run one launch, bracketed by events when timing is on.
template <class Fn>
hipError_t timed(const char* name, double work, int unit, hipStream_t s, Fn&& fn) {
    Profiler& P = g_prof;
    if (!P.on || (int)P.recs.size() >= P.cap) return fn();
    const size_t i = P.recs.size();
    hipEvent_t a = P.pool[2 * i], b = P.pool[2 * i + 1];
    (void)hipEventRecord(a, s);
    const hipError_t e = fn();
    (void)hipEventRecord(b, s);
    P.recs.push_back(ProfRec{name, work, unit, a, b});
    return e;
}

double quant_bytes(int64_t rows, int64_t C, bool row, bool col) {
    const double n = (double)rows * (double)C;
    return 2.0 * n + (row ? n * (1.0 + 1.0 / 32) : 0.0) + (col ? n * (1.0 + 1.0 / 32) : 0.0);
}

constexpr int64_t kI32Max = 0x7fffffffLL;
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Sequential carve-out of a buffer into 256-byte aligned regions.
struct Carver {
    size_t off = 0;
    size_t take(size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes);
        return o;
    }
};

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ---- MX_CHECK: validation of device-side offsets --------------------------
// The offsets arrays live on the device, so the host validation above cannot
// see them; a bad array (decreasing, or not ending at the row count) is
// undefined behaviour for the kernels.  With MX_CHECK=1 in the environment,
// every entry point that takes device offsets copies them to the host on its
// stream, waits for the copy, and checks them before it launches anything.
// Off (the default) the library never synchronises.
bool check_enabled() {
    const char* v = std::getenv("MX_CHECK");
    return v && v[0] == '1' && v[1] == '\0';
}

// offsets [G+1] in host memory: non-decreasing; from_zero: offsets[0] == 0;
// end >= 0: offsets[G] == end; else 0 <= offsets[0] and offsets[G] <= -end - 1
mx_status check_offsets_host(const char* fn, const int64_t* h, int32_t G, int64_t end,
                             bool from_zero) {
    if (from_zero ? h[0] != 0 : h[0] < 0)
        return fail(MX_ERR_INVALID_ARG, "%s: offsets[0] = %lld, expected %s", fn, (long long)h[0],
                    from_zero ? "0" : ">= 0");
    for (int32_t g = 0; g < G; ++g)
        if (h[g + 1] < h[g])
            return fail(MX_ERR_INVALID_ARG, "%s: offsets decrease at group %d (%lld > %lld)", fn, g,
                        (long long)h[g], (long long)h[g + 1]);
    if (end >= 0 && h[G] != end)
        return fail(MX_ERR_INVALID_ARG, "%s: offsets[%d] = %lld, expected the row count %lld", fn,
                    G, (long long)h[G], (long long)end);
    if (end < 0 && h[G] > -end - 1)
        return fail(MX_ERR_INVALID_ARG, "%s: offsets[%d] = %lld past the %lld rows", fn, G,
                    (long long)h[G], (long long)(-end - 1));
    return MX_OK;
}

mx_status check_device_offsets(const char* fn, const int64_t* d_offsets, int32_t G, int64_t end,
                               bool from_zero, hipStream_t s) {
    if (!check_enabled()) return MX_OK;
    std::vector<int64_t> h((size_t)G + 1);
    hipError_t e = hipMemcpyAsync(h.data(), d_offsets, h.size() * sizeof(int64_t),
                                  hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess)
        return fail(MX_ERR_LAUNCH, "%s: MX_CHECK could not read the offsets: %s", fn,
                    hipGetErrorString(e));
    return check_offsets_host(fn, h.data(), G, end, from_zero);
}

int64_t padded_bound(int64_t M, int64_t G, int64_t align) {
    return (M + G * (align - 1)) / align * align;
}

// ---- layouts ----------------------------------------------------------------
struct MlpDims {
    int64_t M, H, F, E, Mp;
};

// Saved-for-backward mode: recompute (default) keeps the X rowwise copy and
// recomputes h = X W1^T in the backward; save-h (MX_MLP_SAVE_H) stores h as
// bf16 in the forward and reads it back.
bool save_h_mode(uint32_t flags) { return (flags & MX_MLP_SAVE_H) != 0; }

struct CtxLayout {
    size_t w1c, w1c_s, w2c, w2c_s, w1r, w1r_s, w2r, w2r_s;   // weight copies
    size_t h;                                                // save-h only
    size_t xr, xr_s;                                         // recompute only
    size_t xcol, xcol_s, zcol, zcol_s, poff, total;
};
CtxLayout ctx_layout(const MlpDims& d, uint32_t flags) {
    Carver c;
    CtxLayout L{};
    // the four weight copies made by the forward's weight pass come first,
    // so that their offsets do not depend on M (a forward that reuses them
    // may have another M): rowwise for the forward GEMMs and the backward's
    // recompute, columnwise for the backward's data gradients
    L.w1c = c.take((size_t)d.E * d.H * 2 * d.F);
    L.w1c_s = c.take((size_t)d.E * d.H * 2 * d.F / 32);
    L.w2c = c.take((size_t)d.E * d.F * d.H);
    L.w2c_s = c.take((size_t)d.E * d.F * d.H / 32);
    L.w1r = c.take((size_t)d.E * 2 * d.F * d.H);
    L.w1r_s = c.take((size_t)d.E * 2 * d.F * d.H / 32);
    L.w2r = c.take((size_t)d.E * d.H * d.F);
    L.w2r_s = c.take((size_t)d.E * d.H * d.F / 32);
    if (save_h_mode(flags)) {
        L.h = c.take((size_t)d.Mp * d.F * 4);     // blocked [Mp/16][F/16] x 1 KiB
    } else {
        L.xr = c.take((size_t)d.M * d.H);
        L.xr_s = c.take((size_t)mx::tiled_scale_bytes(d.M, d.H));
    }
    L.xcol = c.take((size_t)d.H * d.Mp);
    L.xcol_s = c.take((size_t)d.H * d.Mp / 32);
    L.zcol = c.take((size_t)d.F * d.Mp);
    L.zcol_s = c.take((size_t)d.F * d.Mp / 32);
    L.poff = c.take((size_t)(d.E + 1) * 8);
    L.total = c.off;
    return L;
}

struct FwdWs {
    size_t xr, xr_s, zr, zr_s, split, total;
};
FwdWs fwd_ws_layout(const MlpDims& d, uint32_t flags) {
    Carver c;
    FwdWs L{};
    if (save_h_mode(flags)) {     // the recompute mode keeps this copy in ctx
        L.xr = c.take((size_t)d.M * d.H);
        L.xr_s = c.take((size_t)mx::tiled_scale_bytes(d.M, d.H));
    }
    L.zr = c.take((size_t)d.M * d.F);
    L.zr_s = c.take((size_t)mx::tiled_scale_bytes(d.M, d.F));
    L.split = c.take(mx::kSplitWsBytes);      // tail split of the down GEMM
    L.total = c.off;
    return L;
}

// dr partial sums per row: one per 128 columns of F handled by one wave
// (save-h: waves of 128 columns in 256-column tiles; recompute: waves of 64
// columns in 128-column tiles)
int64_t dr_parts(int64_t F, uint32_t flags) {
    return save_h_mode(flags) ? (F + 255) / 256 * 2 : F / 128 * 2;
}

struct BwdWs {
    size_t dyr, dyr_s, dycol, dycol_s, dhr, dhr_s, dhc, dhc_s, drp, split, total;
};
BwdWs bwd_ws_layout(const MlpDims& d, uint32_t flags) {
    Carver c;
    BwdWs L;
    L.dyr = c.take((size_t)d.M * d.H);
    L.dyr_s = c.take((size_t)mx::tiled_scale_bytes(d.M, d.H));
    L.dycol = c.take((size_t)d.H * d.Mp);
    L.dycol_s = c.take((size_t)d.H * d.Mp / 32);
    L.dhr = c.take((size_t)d.M * 2 * d.F);
    L.dhr_s = c.take((size_t)mx::tiled_scale_bytes(d.M, 2 * d.F));
    L.dhc = c.take((size_t)2 * d.F * d.Mp);
    L.dhc_s = c.take((size_t)2 * d.F * d.Mp / 32);
    L.drp = c.take((size_t)d.M * dr_parts(d.F, flags) * 4);
    L.split = c.take(mx::kSplitWsBytes);      // tail split of the gate-up dgrad
    L.total = c.off;
    return L;
}

mx_status check_mlp_dims(int64_t M, int64_t H, int64_t F, int32_t E, MlpDims* out) {
    if (M < 0 || H <= 0 || F <= 0 || E <= 0)
        return fail(MX_ERR_INVALID_ARG, "bad sizes M=%lld H=%lld F=%lld E=%d", (long long)M,
                    (long long)H, (long long)F, E);
    if (E > mx::kMaxGroups)
        return fail(MX_ERR_UNSUPPORTED, "E=%d exceeds %d experts", E, mx::kMaxGroups);
    if (H % 128 || F % 128)
        return fail(MX_ERR_UNSUPPORTED, "H=%lld and F=%lld must be multiples of 128",
                    (long long)H, (long long)F);
    const int64_t Mp = padded_bound(M, E, mx::kTokenAlign);
    // Buffer descriptors are rebased per tile, so only one expert's weight
    // matrix (2F x H) and one tile's rows need 32-bit offsets; the largest
    // per-tile range, 256 rows of a token-axis copy (256 * Mp bytes in the
    // weight-gradient GEMMs), stays below 2^31 with the padded-row bound below
    // (also the quantizer's grid limit of 65535 row tiles).
    if (2 * F * H > kI32Max || 2 * F * 256 > kI32Max)
        return fail(MX_ERR_UNSUPPORTED, "an expert's weights (2F x H = %lld) exceed 2^31 - 1 bytes",
                    (long long)(2 * F * H));
    if (Mp / 128 > 65535)
        return fail(MX_ERR_UNSUPPORTED, "M=%lld too large: %lld padded rows exceed 65535 x 128",
                    (long long)M, (long long)Mp);
    *out = MlpDims{M, H, F, E, Mp};
    return MX_OK;
}

const char* epi_name(mx::Epi e) {
    switch (e) {
        case mx::Epi::kStoreBf16: return "mx_gemm<store_bf16>";
        case mx::Epi::kSwiglu: return "mx_gemm<swiglu_quant>";
        case mx::Epi::kDSwiglu: return "mx_gemm<dswiglu_quant>";
        case mx::Epi::kDSwigluR: return "mx_gemm<dswiglu_recompute>";
    }
    return "mx_gemm";
}

hipError_t gemm(const mx::GemmProblem& p, mx::Epi e, double flops, hipStream_t s) {
    const hipError_t err =
        timed(epi_name(e), flops, MX_WORK_FLOP, s, [&] { return mx::launch_mx_gemm(p, e, s); });
    if (err != hipSuccess || e != mx::Epi::kStoreBf16 || !p.split_ws || p.kgroup) return err;
    // the split tail's partial tiles, added and stored (no-op without a split)
    return timed("split_fixup", 0.0, MX_WORK_BYTES, s,
                 [&] { return mx::launch_split_fixup(p, s); });
}

// Host validation shared by the two plan entry points.
mx_status check_route_plan(const char* fn, const int32_t* d_ids, int64_t T, int32_t k, int32_t E,
                           const float* d_w, int64_t* d_offsets, int32_t* d_row_of,
                           int32_t* d_tok_of, float* d_r_sorted) {
    if (T < 0 || k < 1 || k > 64 || E < 1)
        return fail(MX_ERR_INVALID_ARG, "%s: bad sizes T=%lld k=%d E=%d", fn, (long long)T, k, E);
    if (E > mx::kMaxGroups)
        return fail(MX_ERR_UNSUPPORTED, "%s: E=%d exceeds %d", fn, E, mx::kMaxGroups);
    if (T * k > kI32Max)
        return fail(MX_ERR_UNSUPPORTED, "%s: T*k=%lld rows exceed int32", fn,
                    (long long)(T * k));
    if (!d_offsets || (T > 0 && (!d_ids || !d_row_of || !d_tok_of)))
        return fail(MX_ERR_INVALID_ARG, "%s: NULL argument", fn);
    if ((d_w == nullptr) != (d_r_sorted == nullptr))
        return fail(MX_ERR_INVALID_ARG, "%s: d_w and d_r_sorted go together", fn);
    return MX_OK;
}

mx_status launch_plan(const int32_t* d_ids, int64_t T, int32_t k, int32_t E, const float* d_w,
                      int64_t* d_offsets, int32_t* d_row_of, int32_t* d_tok_of,
                      float* d_r_sorted, int32_t* hist, hipStream_t s) {
    return launched(timed("route_plan", 16.0 * T * k, MX_WORK_BYTES, s,
                          [&] {
                              return mx::launch_route_plan(d_ids, T, k, E, d_w, d_offsets,
                                                           d_row_of, d_tok_of, d_r_sorted, hist,
                                                           s);
                          }),
                    "route_plan");
}

}  // namespace

// ---- misc -------------------------------------------------------------------
namespace mx {
int device_cu_count() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    const bool cacheable = dev >= 0 && dev < 64;
    int v = cacheable ? __atomic_load_n(&cache[dev], __ATOMIC_RELAXED) : 0;
    if (v <= 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            v <= 0)
            v = 256;
        if (cacheable) __atomic_store_n(&cache[dev], v, __ATOMIC_RELAXED);
    }
    return v;
}
}  // namespace mx

extern "C" {

const char* mx_last_error(void) { return g_err.c_str(); }

const char* mx_version(void) { return "mxmoe 0.1 gfx950"; }

int64_t mx_padded_rows_bound(int64_t M, int32_t G, int32_t align) {
    if (M < 0 || G <= 0 || align <= 0) return -1;
    return padded_bound(M, G, align);
}

mx_status mxfp8_quantize(const void* x, int64_t batch, int64_t R, int64_t C,
                         uint8_t* row_codes, uint8_t* row_scales,
                         const int64_t* d_offsets, int32_t G,
                         uint8_t* col_codes, uint8_t* col_scales,
                         int64_t col_ld, int64_t* d_padded_offsets,
                         mx_stream_t stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (!x) return fail(MX_ERR_INVALID_ARG, "mxfp8_quantize: x is NULL");
    if (batch < 1 || R < 0 || C < 0)
        return fail(MX_ERR_INVALID_ARG, "mxfp8_quantize: bad sizes batch=%lld R=%lld C=%lld",
                    (long long)batch, (long long)R, (long long)C);
    if (C % 32)
        return fail(MX_ERR_UNSUPPORTED, "mxfp8_quantize: C=%lld is not a multiple of 32",
                    (long long)C);
    const bool want_row = row_codes || row_scales;
    const bool want_col = col_codes || col_scales;
    if (want_row && !(row_codes && row_scales))
        return fail(MX_ERR_INVALID_ARG, "mxfp8_quantize: row_codes and row_scales go together");
    if (want_col && !(col_codes && col_scales))
        return fail(MX_ERR_INVALID_ARG, "mxfp8_quantize: col_codes and col_scales go together");
    if (!want_row && !want_col)
        return fail(MX_ERR_INVALID_ARG, "mxfp8_quantize: no output requested");
    if (want_col && 256 * C > kI32Max)
        return fail(MX_ERR_UNSUPPORTED, "mxfp8_quantize: C=%lld too large for 32-bit tile offsets",
                    (long long)C);
    if (!aligned(x, 16) || (row_codes && !aligned(row_codes, 16)) ||
        (col_codes && !aligned(col_codes, 16)))
        return fail(MX_ERR_INVALID_ARG, "mxfp8_quantize: x and codes must be 16-byte aligned");
    if ((row_scales && !aligned(row_scales, 4)) || (col_scales && !aligned(col_scales, 4)))
        return fail(MX_ERR_INVALID_ARG, "mxfp8_quantize: scales must be 4-byte aligned");
    if (d_offsets) {
        if (batch != 1)
            return fail(MX_ERR_INVALID_ARG, "mxfp8_quantize: row groups need batch == 1");
        if (G < 1 || G > mx::kMaxGroups)
            return fail(MX_ERR_UNSUPPORTED, "mxfp8_quantize: G=%d outside [1, %d]", G,
                        mx::kMaxGroups);
    }
    int64_t bound = 0;
    if (want_col) {
        bound = d_offsets ? padded_bound(R, G, mx::kTokenAlign)
                          : padded_bound(R, 1, mx::kTokenAlign);
        if (col_ld % 128 || col_ld < bound)
            return fail(MX_ERR_INVALID_ARG,
                        "mxfp8_quantize: col_ld=%lld must be a multiple of 128 and >= %lld",
                        (long long)col_ld, (long long)bound);
        if (d_offsets && !d_padded_offsets)
            return fail(MX_ERR_INVALID_ARG, "mxfp8_quantize: d_padded_offsets is NULL");
        if (bound / 128 > 65535 || batch > 65535)
            return fail(MX_ERR_UNSUPPORTED, "mxfp8_quantize: too many rows for one launch");
    }
    if (d_offsets) {
        const mx_status cs = check_device_offsets("mxfp8_quantize", d_offsets, G, R, true, s);
        if (cs != MX_OK) return cs;
    }
    if (batch * R == 0 || C == 0) {
        if (want_col && d_offsets)
            return launched(timed("padded_offsets", 16.0 * (G + 1), MX_WORK_BYTES, s,
                                  [&] { return mx::launch_padded_offsets(d_offsets, G, d_padded_offsets, s); }),
                            "padded_offsets");
        return ok();
    }
    const uint16_t* xs = static_cast<const uint16_t*>(x);
    if (!want_col)
        return launched(timed("quant_rows", quant_bytes(batch * R, C, true, false), MX_WORK_BYTES,
                              s,
                              [&] {
                                  return mx::launch_quant_rows(xs, batch * R, C, row_codes,
                                                               row_scales, false, s);
                              }),
                        "quant_rows");
    if (d_offsets) {
        hipError_t e = timed("padded_offsets", 16.0 * (G + 1), MX_WORK_BYTES, s, [&] {
            return mx::launch_padded_offsets(d_offsets, G, d_padded_offsets, s);
        });
        if (e != hipSuccess) return launched(e, "padded_offsets");
    }
    return launched(timed("quant_tiles", quant_bytes(batch * R, C, want_row, true), MX_WORK_BYTES,
                          s,
                          [&] {
                              return mx::launch_quant_tiles(xs, batch, R, C, d_offsets,
                                                            d_padded_offsets, d_offsets ? G : 1,
                                                            bound, row_codes, row_scales,
                                                            col_codes, col_scales, col_ld, false,
                                                            s);
                          }),
                    "quant_tiles");
}

// K not a multiple of the GEMM's K step (128) but of the MX block (32): the
// operands are copied into rows of Kp = K rounded up to 128, the codes past K
// set to 0 and (with block scales) their scales to 2^0, so the padding adds
// exact zeros.  The copies live in one device allocation, made and freed in
// stream order around the GEMM.
struct PaddedOperands {
    uint8_t* buf = nullptr;
    const uint8_t *x = nullptr, *xs = nullptr, *w = nullptr, *ws = nullptr;
    hipStream_t s = nullptr;
    ~PaddedOperands() {
        if (buf) (void)hipFreeAsync(buf, s);
    }
};
static int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
static mx_status pad_operands(const char* fn, const uint8_t* x, const uint8_t* x_scales, int64_t M,
                              const uint8_t* w, const uint8_t* w_scales, int64_t EN, int64_t K,
                              int64_t Kp, hipStream_t s, PaddedOperands& out) {
    const bool scaled = x_scales != nullptr;
    const int64_t xb = round_up(M * Kp, 256), wb = round_up(EN * Kp, 256);
    const int64_t xsb = scaled ? round_up(M * (Kp / 32), 256) : 0;
    const int64_t wsb = scaled ? round_up(EN * (Kp / 32), 256) : 0;
    out.s = s;
    hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&out.buf), (size_t)(xb + wb + xsb + wsb), s);
    if (e != hipSuccess) {
        out.buf = nullptr;
        return fail(MX_ERR_LAUNCH, "%s: padded copies (K %% 128 != 0): %s", fn, hipGetErrorString(e));
    }
    uint8_t* xp = out.buf;
    uint8_t* wp = xp + xb;
    uint8_t* xsp = wp + wb;
    uint8_t* wsp = xsp + xsb;
    e = mx::launch_pad_rows(x, M, K, xp, Kp, 0, s);
    if (e == hipSuccess) e = mx::launch_pad_rows(w, EN, K, wp, Kp, 0, s);
    if (scaled && e == hipSuccess) e = mx::launch_pad_rows(x_scales, M, K / 32, xsp, Kp / 32, 127, s);
    if (scaled && e == hipSuccess) e = mx::launch_pad_rows(w_scales, EN, K / 32, wsp, Kp / 32, 127, s);
    if (e != hipSuccess) return launched(e, "pad_rows");
    out.x = xp;
    out.w = wp;
    out.xs = scaled ? xsp : nullptr;
    out.ws = scaled ? wsp : nullptr;
    return MX_OK;
}

mx_status grouped_linear_fwd(int32_t dtype, const void* x, const uint8_t* x_scales,
                             const int64_t* d_offsets, int32_t E, int64_t M,
                             const void* w, const uint8_t* w_scales, int64_t N,
                             int64_t K, const float* d_row_scale, void* y,
                             mx_stream_t stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (!x || !d_offsets || !w || !y)
        return fail(MX_ERR_INVALID_ARG, "grouped_linear_fwd: NULL x, offsets, w or y");
    if (E < 1 || E > mx::kMaxGroups || M < 0 || N <= 0 || K <= 0)
        return fail(MX_ERR_INVALID_ARG, "grouped_linear_fwd: bad sizes E=%d M=%lld N=%lld K=%lld",
                    E, (long long)M, (long long)N, (long long)K);
    if (!aligned(x, 16) || !aligned(w, 16))
        return fail(MX_ERR_INVALID_ARG, "grouped_linear_fwd: x and w must be 16-byte aligned");
    if (dtype == MX_DTYPE_BF16 || dtype == MX_DTYPE_MXFP8) {
        const mx_status cs = check_device_offsets("grouped_linear_fwd", d_offsets, E, M, true, s);
        if (cs != MX_OK) return cs;
    }
    if (dtype == MX_DTYPE_BF16) {
        if (x_scales || w_scales)
            return fail(MX_ERR_INVALID_ARG, "grouped_linear_fwd: bf16 takes no scales");
        if (K % 32)
            return fail(MX_ERR_UNSUPPORTED, "grouped_linear_fwd: bf16 needs K %% 32 == 0");
        if ((M + (int64_t)E * 63) / 64 > 65535)
            return fail(MX_ERR_UNSUPPORTED, "grouped_linear_fwd: M too large for bf16 path");
        if (M == 0) return ok();
        return launched(timed("bf16_grouped", 2.0 * M * N * K, MX_WORK_FLOP, s,
                              [&] {
                                  return mx::launch_bf16_grouped(
                                      static_cast<const uint16_t*>(x), d_offsets, E, M,
                                      static_cast<const uint16_t*>(w), N, K, d_row_scale,
                                      static_cast<uint16_t*>(y), s);
                              }),
                        "bf16_grouped");
    }
    if (dtype != MX_DTYPE_MXFP8)
        return fail(MX_ERR_INVALID_ARG, "grouped_linear_fwd: unknown dtype %d", dtype);
    if (!x_scales || !w_scales)
        return fail(MX_ERR_INVALID_ARG, "grouped_linear_fwd: MXFP8 needs x_scales and w_scales");
    if (K % 32 || N % 32)
        return fail(MX_ERR_UNSUPPORTED, "grouped_linear_fwd: MXFP8 needs K %% 32 == 0 and N %% 32 == 0");
    const int64_t Kp = round_up(K, 128);
    if (N * Kp > kI32Max || 256 * Kp > kI32Max)
        return fail(MX_ERR_UNSUPPORTED, "grouped_linear_fwd: operand too large");
    if (M == 0) return ok();
    PaddedOperands pad;
    const uint8_t *xa = static_cast<const uint8_t*>(x), *xsa = x_scales;
    const uint8_t *wa = static_cast<const uint8_t*>(w), *wsa = w_scales;
    if (Kp != K) {
        const mx_status ps = pad_operands("grouped_linear_fwd", xa, xsa, M, wa, wsa, (int64_t)E * N,
                                          K, Kp, s, pad);
        if (ps != MX_OK) return ps;
        xa = pad.x; xsa = pad.xs; wa = pad.w; wsa = pad.ws;
    }
    mx::GemmProblem p{};
    p.kgroup = false;
    p.offs = d_offsets;
    p.G = E;
    p.M = M; p.N = N; p.K = Kp;
    p.A = mx::MxOperand{xa, xsa, Kp, 0};
    p.B = mx::MxOperand{wa, wsa, Kp, N};
    p.C = y; p.ldc = N; p.c_gstride = 0;
    p.rscale = d_row_scale;
    return launched(gemm(p, mx::Epi::kStoreBf16, 2.0 * M * N * K, s), "mx_gemm");
}

// ---- per-tensor FP8 ------------------------------------------------------------
mx_status fp8_tensor_quantize(const void* x, int64_t batch, int64_t R, int64_t C,
                              const int64_t* d_offsets, int32_t G, uint8_t* codes, float* d_amax,
                              float* d_scale_inv, mx_stream_t stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (batch < 1 || R < 0 || C < 0 || G < 1)
        return fail(MX_ERR_INVALID_ARG,
                    "fp8_tensor_quantize: bad sizes batch=%lld R=%lld C=%lld G=%d",
                    (long long)batch, (long long)R, (long long)C, G);
    if (G > mx::kMaxGroups)
        return fail(MX_ERR_UNSUPPORTED, "fp8_tensor_quantize: G=%d above %d", G, mx::kMaxGroups);
    if (d_offsets ? batch != 1 : G != batch)
        return fail(MX_ERR_INVALID_ARG,
                    "fp8_tensor_quantize: row groups need batch == 1, matrices need G == batch");
    if (C % 32)
        return fail(MX_ERR_UNSUPPORTED, "fp8_tensor_quantize: C=%lld is not a multiple of 32",
                    (long long)C);
    if (256 * C > kI32Max || (batch * R + 127) / 128 > kI32Max || (C + 63) / 64 > 65535)
        return fail(MX_ERR_UNSUPPORTED, "fp8_tensor_quantize: tensor too large");
    if (!d_amax || !d_scale_inv || (batch * R * C > 0 && (!x || !codes)))
        return fail(MX_ERR_INVALID_ARG, "fp8_tensor_quantize: NULL argument");
    if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(d_amax, 4) || !aligned(d_scale_inv, 4))
        return fail(MX_ERR_INVALID_ARG,
                    "fp8_tensor_quantize: x and codes must be 16-byte aligned, amax and "
                    "scale_inv 4-byte aligned");
    const int64_t rows = batch * R;
    if (d_offsets) {
        const mx_status cs = check_device_offsets("fp8_tensor_quantize", d_offsets, G, -rows - 1,
                                                  false, s);
        if (cs != MX_OK) return cs;
    }
    return launched(timed("fp8_tensor_quant", 5.0 * rows * C, MX_WORK_BYTES, s,
                          [&] {
                              return mx::launch_fp8_tensor_quant(
                                  static_cast<const uint16_t*>(x), rows, C, d_offsets, G, R,
                                  reinterpret_cast<uint32_t*>(d_amax), codes, d_scale_inv, s);
                          }),
                    "fp8_tensor_quant");
}

mx_status grouped_linear_fwd_fp8(const uint8_t* x, const float* d_x_scale_inv,
                                 const int64_t* d_offsets, int32_t E, int64_t M, const uint8_t* w,
                                 const float* d_w_scale_inv, int64_t N, int64_t K,
                                 const float* d_row_scale, void* y, mx_stream_t stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (!x || !d_x_scale_inv || !d_offsets || !w || !d_w_scale_inv || !y)
        return fail(MX_ERR_INVALID_ARG, "grouped_linear_fwd_fp8: NULL argument");
    if (E < 1 || E > mx::kMaxGroups || M < 0 || N <= 0 || K <= 0)
        return fail(MX_ERR_INVALID_ARG,
                    "grouped_linear_fwd_fp8: bad sizes E=%d M=%lld N=%lld K=%lld", E,
                    (long long)M, (long long)N, (long long)K);
    if (!aligned(x, 16) || !aligned(w, 16))
        return fail(MX_ERR_INVALID_ARG, "grouped_linear_fwd_fp8: x and w must be 16-byte aligned");
    if (K % 32 || N % 32)
        return fail(MX_ERR_UNSUPPORTED,
                    "grouped_linear_fwd_fp8: needs K %% 32 == 0 and N %% 32 == 0");
    const int64_t Kp = round_up(K, 128);
    if (N * Kp > kI32Max || 256 * Kp > kI32Max)
        return fail(MX_ERR_UNSUPPORTED, "grouped_linear_fwd_fp8: operand too large");
    {
        const mx_status cs = check_device_offsets("grouped_linear_fwd_fp8", d_offsets, E, M, true, s);
        if (cs != MX_OK) return cs;
    }
    if (M == 0) return ok();
    PaddedOperands pad;
    const uint8_t *xa = x, *wa = w;
    if (Kp != K) {
        const mx_status ps = pad_operands("grouped_linear_fwd_fp8", x, nullptr, M, w, nullptr,
                                          (int64_t)E * N, K, Kp, s, pad);
        if (ps != MX_OK) return ps;
        xa = pad.x; wa = pad.w;
    }
    mx::GemmProblem p{};
    p.kgroup = false;
    p.offs = d_offsets;
    p.G = E;
    p.M = M; p.N = N; p.K = Kp;
    p.A = mx::MxOperand{xa, nullptr, Kp, 0};         // no block scales: one per group
    p.B = mx::MxOperand{wa, nullptr, Kp, N};
    p.C = y; p.ldc = N; p.c_gstride = 0;
    p.rscale = d_row_scale;
    p.gsa = d_x_scale_inv;
    p.gsb = d_w_scale_inv;
    return launched(gemm(p, mx::Epi::kStoreBf16, 2.0 * M * N * K, s), "mx_gemm");
}

constexpr uint32_t kFwdFlags = MX_FWD_REUSE_WEIGHTS | MX_MLP_SAVE_H;

size_t grouped_mlp_ctx_bytes(int64_t M, int64_t H, int64_t F, int32_t E, uint32_t flags) {
    MlpDims d;
    if ((flags & ~(uint32_t)MX_MLP_SAVE_H) || check_mlp_dims(M, H, F, E, &d) != MX_OK) return 0;
    return ctx_layout(d, flags).total;
}
size_t grouped_mlp_fwd_ws_bytes(int64_t M, int64_t H, int64_t F, int32_t E, uint32_t flags) {
    MlpDims d;
    if ((flags & ~(uint32_t)MX_MLP_SAVE_H) || check_mlp_dims(M, H, F, E, &d) != MX_OK) return 0;
    return fwd_ws_layout(d, flags).total;
}
size_t grouped_mlp_bwd_ws_bytes(int64_t M, int64_t H, int64_t F, int32_t E, uint32_t flags) {
    MlpDims d;
    if ((flags & ~(uint32_t)MX_MLP_SAVE_H) || check_mlp_dims(M, H, F, E, &d) != MX_OK) return 0;
    return bwd_ws_layout(d, flags).total;
}

int64_t grouped_mlp_ctx_offset(int32_t which, int64_t M, int64_t H, int64_t F, int32_t E,
                               uint32_t flags) {
    MlpDims d;
    if (flags & ~(uint32_t)MX_MLP_SAVE_H) {
        fail(MX_ERR_INVALID_ARG, "grouped_mlp_ctx_offset: unknown flags 0x%x", flags);
        return -1;
    }
    if (check_mlp_dims(M, H, F, E, &d) != MX_OK) return -1;
    const bool sh = save_h_mode(flags);
    const CtxLayout L = ctx_layout(d, flags);
    switch (which) {
        case MX_CTX_H: if (sh) return (int64_t)L.h; break;
        case MX_CTX_XROW: if (!sh) return (int64_t)L.xr; break;
        case MX_CTX_XCOL: return (int64_t)L.xcol;
        case MX_CTX_ZCOL: return (int64_t)L.zcol;
        case MX_CTX_POFF: return (int64_t)L.poff;
        case MX_CTX_W1COL: return (int64_t)L.w1c;
        case MX_CTX_W2COL: return (int64_t)L.w2c;
        case MX_CTX_W1ROW: return (int64_t)L.w1r;
        case MX_CTX_W2ROW: return (int64_t)L.w2r;
        default: break;
    }
    fail(MX_ERR_INVALID_ARG, "grouped_mlp_ctx_offset: region %d not in a ctx of this mode", which);
    return -1;
}

int64_t grouped_mlp_ws_offset(int32_t which, int64_t M, int64_t H, int64_t F, int32_t E,
                              uint32_t flags) {
    MlpDims d;
    if (flags & ~(uint32_t)MX_MLP_SAVE_H) {
        fail(MX_ERR_INVALID_ARG, "grouped_mlp_ws_offset: unknown flags 0x%x", flags);
        return -1;
    }
    if (check_mlp_dims(M, H, F, E, &d) != MX_OK) return -1;
    switch (which) {
        case MX_WS_ZROW: return (int64_t)fwd_ws_layout(d, flags).zr;
        case MX_WS_DHROW: return (int64_t)bwd_ws_layout(d, flags).dhr;
        case MX_WS_DHCOL: return (int64_t)bwd_ws_layout(d, flags).dhc;
        case MX_WS_DYROW: return (int64_t)bwd_ws_layout(d, flags).dyr;
        case MX_WS_DYCOL: return (int64_t)bwd_ws_layout(d, flags).dycol;
        default: break;
    }
    fail(MX_ERR_INVALID_ARG, "grouped_mlp_ws_offset: unknown region %d", which);
    return -1;
}

mx_status grouped_mlp_fwd(const void* x, const int64_t* d_offsets, int32_t E, int64_t M,
                          int64_t H, int64_t F, const void* w1, const void* w2,
                          const float* d_r, void* y, void* ctx, size_t ctx_bytes, void* ws,
                          size_t ws_bytes, mx_stream_t stream) {
    return grouped_mlp_fwd_ex(x, d_offsets, E, M, H, F, w1, w2, d_r, y, ctx, ctx_bytes, ws,
                              ws_bytes, 0u, stream);
}

mx_status grouped_mlp_fwd_ex(const void* x, const int64_t* d_offsets, int32_t E, int64_t M,
                             int64_t H, int64_t F, const void* w1, const void* w2,
                             const float* d_r, void* y, void* ctx, size_t ctx_bytes, void* ws,
                             size_t ws_bytes, uint32_t flags, mx_stream_t stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const bool reuse = (flags & MX_FWD_REUSE_WEIGHTS) != 0;
    const bool sh = save_h_mode(flags);
    if (flags & ~kFwdFlags)
        return fail(MX_ERR_INVALID_ARG, "grouped_mlp_fwd: unknown flags 0x%x", flags);
    // the [M, *] tensors may be NULL when M == 0
    if (!d_offsets || (!reuse && (!w1 || !w2)) || !ctx || !ws || (M > 0 && (!x || !d_r || !y)))
        return fail(MX_ERR_INVALID_ARG, "grouped_mlp_fwd: NULL argument");
    MlpDims d;
    mx_status st = check_mlp_dims(M, H, F, E, &d);
    if (st != MX_OK) return st;
    const CtxLayout C = ctx_layout(d, flags);
    const FwdWs W = fwd_ws_layout(d, flags);
    if (ctx_bytes < C.total)
        return fail(MX_ERR_WORKSPACE, "grouped_mlp_fwd: ctx needs %zu bytes, got %zu", C.total,
                    ctx_bytes);
    if (ws_bytes < W.total)
        return fail(MX_ERR_WORKSPACE, "grouped_mlp_fwd: ws needs %zu bytes, got %zu", W.total,
                    ws_bytes);
    if (!aligned(x, 16) || !aligned(w1, 16) || !aligned(w2, 16) || !aligned(ctx, kAlign) ||
        !aligned(ws, kAlign))
        return fail(MX_ERR_INVALID_ARG,
                    "grouped_mlp_fwd: tensors must be 16-byte and ctx/ws 256-byte aligned");
    {
        const mx_status cs = check_device_offsets("grouped_mlp_fwd", d_offsets, E, M, true, s);
        if (cs != MX_OK) return cs;
    }
    // with reuse the weight copies in ctx are the previous call's
    uint8_t* cb = static_cast<uint8_t*>(ctx);
    uint8_t* wb = static_cast<uint8_t*>(ws);
    int64_t* poff = reinterpret_cast<int64_t*>(cb + C.poff);
    // rowwise X: in ctx for the recompute backward, else forward scratch
    uint8_t* xr = sh ? wb + W.xr : cb + C.xr;
    uint8_t* xr_s = sh ? wb + W.xr_s : cb + C.xr_s;
    const int64_t M2 = 2 * F;
    hipError_t e;

    // (1) X: rowwise copy for the gate-up GEMM, token-axis copy saved for dW1
    e = timed("padded_offsets", 16.0 * (E + 1), MX_WORK_BYTES, s,
              [&] { return mx::launch_padded_offsets(d_offsets, E, poff, s); });
    if (e != hipSuccess) return launched(e, "padded_offsets");
    if (M > 0) {
        e = timed("quant_tiles", quant_bytes(M, H, true, true), MX_WORK_BYTES, s, [&] {
            return mx::launch_quant_tiles(static_cast<const uint16_t*>(x), 1, M, H, d_offsets,
                                          poff, E, d.Mp, xr, xr_s, cb + C.xcol,
                                          cb + C.xcol_s, d.Mp, true, s);
        });
        if (e != hipSuccess) return launched(e, "quant_tiles(x)");
    }
    // (2) weights, one pass each: rowwise copies for the forward GEMMs (W1
    // blocks along H, W2 along F) and the columnwise copies the backward's
    // data gradients use (W1 blocks along 2F, W2 along H), all kept in ctx.
    // Skipped when the caller reuses the copies of an earlier call.
    if (!reuse) {
        e = timed("quant_tiles", quant_bytes((int64_t)E * M2, H, true, true), MX_WORK_BYTES, s,
                  [&] {
                      return mx::launch_quant_tiles(static_cast<const uint16_t*>(w1), E, M2, H,
                                                    nullptr, nullptr, 1, 0, cb + C.w1r,
                                                    cb + C.w1r_s, cb + C.w1c, cb + C.w1c_s, M2,
                                                    true, s);
                  });
        if (e != hipSuccess) return launched(e, "quant_tiles(w1)");
        e = timed("quant_tiles", quant_bytes((int64_t)E * H, F, true, true), MX_WORK_BYTES, s,
                  [&] {
                      return mx::launch_quant_tiles(static_cast<const uint16_t*>(w2), E, H, F,
                                                    nullptr, nullptr, 1, 0, cb + C.w2r,
                                                    cb + C.w2r_s, cb + C.w2c, cb + C.w2c_s, H,
                                                    true, s);
                  });
        if (e != hipSuccess) return launched(e, "quant_tiles(w2)");
    }
    if (M == 0) return ok();

    // (3) gate-up GEMM with the SwiGLU / routing-scale / requantize epilogue;
    // h leaves the chip only in the save-h mode
    mx::GemmProblem p{};
    p.kgroup = false;
    p.offs = d_offsets;
    p.G = E;
    p.M = M; p.N = M2; p.K = H;
    p.A = mx::MxOperand{xr, xr_s, H, 0, true};
    p.B = mx::MxOperand{cb + C.w1r, cb + C.w1r_s, H, M2, true};
    p.rscale = d_r;
    p.F = F;
    p.h = sh ? reinterpret_cast<uint16_t*>(cb + C.h) : nullptr;
    p.qr = wb + W.zr; p.qrs = wb + W.zr_s; p.ldqr = F;
    p.qc = cb + C.zcol; p.qcs = cb + C.zcol_s; p.ldqc = d.Mp;
    p.qtiled = true;
    p.poff = poff;
    e = gemm(p, mx::Epi::kSwiglu, 2.0 * M * M2 * H, s);
    if (e != hipSuccess) return launched(e, "mx_gemm(gate-up)");

    // (4) down projection
    mx::GemmProblem q{};
    q.kgroup = false;
    q.offs = d_offsets;
    q.G = E;
    q.M = M; q.N = H; q.K = F;
    q.A = mx::MxOperand{wb + W.zr, wb + W.zr_s, F, 0, true};
    q.B = mx::MxOperand{cb + C.w2r, cb + C.w2r_s, F, H, true};
    q.C = y; q.ldc = H;
    q.split_ws = wb + W.split;
    return launched(gemm(q, mx::Epi::kStoreBf16, 2.0 * M * H * F, s), "mx_gemm(down)");
}

mx_status grouped_mlp_bwd(const void* dy, const int64_t* d_offsets, int32_t E, int64_t M,
                          int64_t H, int64_t F, const void* w1, const void* w2,
                          const float* d_r, const void* ctx, size_t ctx_bytes, void* dx,
                          void* dw1, void* dw2, float* d_dr, void* ws, size_t ws_bytes,
                          mx_stream_t stream) {
    return grouped_mlp_bwd_ex(dy, d_offsets, E, M, H, F, w1, w2, d_r, ctx, ctx_bytes, dx, dw1,
                              dw2, d_dr, ws, ws_bytes, 0u, stream);
}

mx_status grouped_mlp_bwd_ex(const void* dy, const int64_t* d_offsets, int32_t E, int64_t M,
                             int64_t H, int64_t F, const void* w1, const void* w2,
                             const float* d_r, const void* ctx, size_t ctx_bytes, void* dx,
                             void* dw1, void* dw2, float* d_dr, void* ws, size_t ws_bytes,
                             uint32_t flags, mx_stream_t stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (flags & ~(uint32_t)MX_MLP_SAVE_H)
        return fail(MX_ERR_INVALID_ARG, "grouped_mlp_bwd: unknown flags 0x%x", flags);
    const bool sh = save_h_mode(flags);
    // the [M, *] tensors may be NULL when M == 0
    if (!d_offsets || !w1 || !w2 || !ctx || !dw1 || !dw2 || !ws ||
        (M > 0 && (!dy || !d_r || !dx || !d_dr)))
        return fail(MX_ERR_INVALID_ARG, "grouped_mlp_bwd: NULL argument");
    MlpDims d;
    mx_status st = check_mlp_dims(M, H, F, E, &d);
    if (st != MX_OK) return st;
    const CtxLayout C = ctx_layout(d, flags);
    const BwdWs W = bwd_ws_layout(d, flags);
    if (ctx_bytes < C.total)
        return fail(MX_ERR_WORKSPACE, "grouped_mlp_bwd: ctx needs %zu bytes, got %zu", C.total,
                    ctx_bytes);
    if (ws_bytes < W.total)
        return fail(MX_ERR_WORKSPACE, "grouped_mlp_bwd: ws needs %zu bytes, got %zu", W.total,
                    ws_bytes);
    if (!aligned(dy, 16) || !aligned(w1, 16) || !aligned(w2, 16) || !aligned(ctx, kAlign) ||
        !aligned(ws, kAlign))
        return fail(MX_ERR_INVALID_ARG,
                    "grouped_mlp_bwd: tensors must be 16-byte and ctx/ws 256-byte aligned");
    {
        const mx_status cs = check_device_offsets("grouped_mlp_bwd", d_offsets, E, M, true, s);
        if (cs != MX_OK) return cs;
    }
    const uint8_t* cb = static_cast<const uint8_t*>(ctx);
    uint8_t* wb = static_cast<uint8_t*>(ws);
    const int64_t* poff = reinterpret_cast<const int64_t*>(cb + C.poff);
    const int64_t M2 = 2 * F;
    const int64_t nparts = dr_parts(F, flags);
    hipError_t e;

    // (1) dY: rowwise for the data gradient, token-axis for dW2
    if (M > 0) {
        e = timed("quant_tiles", quant_bytes(M, H, true, true), MX_WORK_BYTES, s, [&] {
            return mx::launch_quant_tiles(static_cast<const uint16_t*>(dy), 1, M, H, d_offsets,
                                          poff, E, d.Mp, wb + W.dyr, wb + W.dyr_s, wb + W.dycol,
                                          wb + W.dycol_s, d.Mp, true, s);
        });
        if (e != hipSuccess) return launched(e, "quant_tiles(dy)");
    }
    // (2) the weights' copies were made by the forward (ctx)

    if (M > 0) {
        // (3) dz = dY W2 with the SwiGLU-backward / dr / requantize epilogue;
        // the recompute mode also recomputes h = X W1^T in the same tile
        mx::GemmProblem p{};
        p.kgroup = false;
        p.offs = d_offsets;
        p.G = E;
        p.M = M; p.K = H;
        p.rscale = d_r;
        p.F = F;
        p.qr = wb + W.dhr; p.qrs = wb + W.dhr_s; p.ldqr = M2;
        p.qc = wb + W.dhc; p.qcs = wb + W.dhc_s; p.ldqc = d.Mp;
        p.qtiled = true;
        p.poff = poff;
        p.drp = reinterpret_cast<float*>(wb + W.drp); p.lddrp = M;   // part-major partials
        const mx::MxOperand dyr{wb + W.dyr, wb + W.dyr_s, H, 0, true};
        const mx::MxOperand w2c{cb + C.w2c, cb + C.w2c_s, H, F, true};
        if (sh) {
            p.N = F;
            p.A = dyr;
            p.B = w2c;
            p.h = const_cast<uint16_t*>(reinterpret_cast<const uint16_t*>(cb + C.h));
            e = gemm(p, mx::Epi::kDSwiglu, 2.0 * M * F * H, s);
        } else {
            p.N = M2;
            p.A = mx::MxOperand{cb + C.xr, cb + C.xr_s, H, 0, true};
            p.B = mx::MxOperand{cb + C.w1r, cb + C.w1r_s, H, M2, true};
            p.A2 = dyr;
            p.B2 = w2c;
            e = gemm(p, mx::Epi::kDSwigluR, 2.0 * M * F * H, s);
        }
        if (e != hipSuccess) return launched(e, "mx_gemm(dgrad-down)");
        e = timed("dr_reduce", 4.0 * M * (nparts + 1), MX_WORK_BYTES, s, [&] {
            return mx::launch_dr_reduce(reinterpret_cast<const float*>(wb + W.drp), M, nparts,
                                        d_dr, s);
        });
        if (e != hipSuccess) return launched(e, "dr_reduce");

        // (4) dX = dh W1
        mx::GemmProblem q{};
        q.kgroup = false;
        q.offs = d_offsets;
        q.G = E;
        q.M = M; q.N = H; q.K = M2;
        q.A = mx::MxOperand{wb + W.dhr, wb + W.dhr_s, M2, 0, true};
        q.B = mx::MxOperand{cb + C.w1c, cb + C.w1c_s, M2, H, true};
        q.C = dx; q.ldc = H;
        q.split_ws = wb + W.split;
        e = gemm(q, mx::Epi::kStoreBf16, 2.0 * M * H * M2, s);
        if (e != hipSuccess) return launched(e, "mx_gemm(dgrad-gate-up)");
    }

    // (5) weight gradients over each expert's padded token range
    mx::GemmProblem w{};
    w.kgroup = true;
    w.offs = poff;
    w.G = E;
    w.M = H; w.N = F;
    w.A = mx::MxOperand{wb + W.dycol, wb + W.dycol_s, d.Mp, 0, true};
    w.B = mx::MxOperand{cb + C.zcol, cb + C.zcol_s, d.Mp, 0, true};
    w.C = dw2; w.ldc = F; w.c_gstride = H * F;
    e = gemm(w, mx::Epi::kStoreBf16, 2.0 * H * F * M, s);
    if (e != hipSuccess) return launched(e, "mx_gemm(wgrad-down)");

    mx::GemmProblem v{};
    v.kgroup = true;
    v.offs = poff;
    v.G = E;
    v.M = M2; v.N = H;
    v.A = mx::MxOperand{wb + W.dhc, wb + W.dhc_s, d.Mp, 0, true};
    v.B = mx::MxOperand{cb + C.xcol, cb + C.xcol_s, d.Mp, 0, true};
    v.C = dw1; v.ldc = H; v.c_gstride = M2 * H;
    return launched(gemm(v, mx::Epi::kStoreBf16, 2.0 * M2 * H * M, s), "mx_gemm(wgrad-gate-up)");
}

// ---- routing: router, sorted-row plan, permute + quantize, combine ------------
mx_status moe_router(const float* d_logits, int64_t T, int32_t E, int32_t k, int32_t* d_ids,
                     float* d_w, mx_stream_t stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (T < 0 || E < 1 || k < 1 || k > E)
        return fail(MX_ERR_INVALID_ARG, "moe_router: bad sizes T=%lld E=%d k=%d", (long long)T,
                    E, k);
    if (E > mx::kMaxGroups || k > 64)
        return fail(MX_ERR_UNSUPPORTED, "moe_router: E=%d or k=%d unsupported", E, k);
    if (T * k > kI32Max) return fail(MX_ERR_UNSUPPORTED, "moe_router: T*k above 2^31-1");
    if (T > 0 && (!d_logits || !d_ids || !d_w))
        return fail(MX_ERR_INVALID_ARG, "moe_router: NULL argument");
    return launched(timed("router", 4.0 * T * E + 8.0 * T * k, MX_WORK_BYTES, s,
                          [&] { return mx::launch_router(d_logits, T, E, k, d_ids, d_w, s); }),
                    "router");
}

size_t moe_route_ws_bytes(int64_t T, int32_t k, int32_t E) {
    if (T < 0 || k < 1 || E < 1 || E > mx::kMaxGroups) return 0;
    const int64_t n = mx::route_chunks(T * k);
    return (size_t)(n > 0 ? n : 1) * (size_t)E * 4;
}

mx_status moe_route_plan(const int32_t* d_ids, int64_t T, int32_t k, int32_t E, const float* d_w,
                         int64_t* d_offsets, int32_t* d_row_of, int32_t* d_tok_of,
                         float* d_r_sorted, void* ws, size_t ws_bytes, mx_stream_t stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    mx_status st = check_route_plan("moe_route_plan", d_ids, T, k, E, d_w, d_offsets, d_row_of,
                                    d_tok_of, d_r_sorted);
    if (st != MX_OK) return st;
    if (!ws) return fail(MX_ERR_INVALID_ARG, "moe_route_plan: NULL argument");
    if (ws_bytes < moe_route_ws_bytes(T, k, E))
        return fail(MX_ERR_WORKSPACE, "moe_route_plan: ws needs %zu bytes, got %zu",
                    moe_route_ws_bytes(T, k, E), ws_bytes);
    if (!aligned(ws, 4))
        return fail(MX_ERR_INVALID_ARG, "moe_route_plan: ws must be 4-byte aligned");
    return launch_plan(d_ids, T, k, E, d_w, d_offsets, d_row_of, d_tok_of, d_r_sorted,
                       static_cast<int32_t*>(ws), s);
}

mx_status moe_route_plan_noalloc(const int32_t* d_ids, int64_t T, int32_t k, int32_t E,
                                 const float* d_w, int64_t* d_offsets, int32_t* d_row_of,
                                 int32_t* d_tok_of, float* d_r_sorted, mx_stream_t stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    mx_status st = check_route_plan("moe_route_plan_noalloc", d_ids, T, k, E, d_w, d_offsets,
                                    d_row_of, d_tok_of, d_r_sorted);
    if (st != MX_OK) return st;
    const int64_t need = mx::route_chunks(T * k) * E;
    if (need > mx::kPlanScratchInts)
        return fail(MX_ERR_UNSUPPORTED,
                    "moe_route_plan_noalloc: ceil(T*k/256)*E = %lld counters exceed the "
                    "library's scratch of %lld (use moe_route_plan with a workspace)",
                    (long long)need, (long long)mx::kPlanScratchInts);
    int32_t* scratch = nullptr;
    const hipError_t e = mx::route_plan_scratch(&scratch);
    if (e != hipSuccess)
        return fail(MX_ERR_LAUNCH, "moe_route_plan_noalloc: scratch lookup failed: %s",
                    hipGetErrorString(e));
    return launch_plan(d_ids, T, k, E, d_w, d_offsets, d_row_of, d_tok_of, d_r_sorted, scratch,
                       s);
}

mx_status moe_permute_quantize(const void* x, int64_t T, int64_t H, const int32_t* d_tok_of,
                               int64_t M, const int64_t* d_offsets, int32_t E,
                               uint8_t* row_codes, uint8_t* row_scales, uint8_t* col_codes,
                               uint8_t* col_scales, int64_t col_ld, int64_t* d_padded_offsets,
                               mx_stream_t stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (!x || !d_tok_of || !d_offsets || !d_padded_offsets)
        return fail(MX_ERR_INVALID_ARG, "moe_permute_quantize: NULL argument");
    if (T < 0 || M < 0 || H <= 0 || E < 1)
        return fail(MX_ERR_INVALID_ARG, "moe_permute_quantize: bad sizes T=%lld M=%lld H=%lld E=%d",
                    (long long)T, (long long)M, (long long)H, E);
    if (E > mx::kMaxGroups || H % 32)
        return fail(MX_ERR_UNSUPPORTED, "moe_permute_quantize: E=%d or H=%lld unsupported", E,
                    (long long)H);
    if (T * H * 2 > kI32Max || 256 * H > kI32Max || M > kI32Max)
        return fail(MX_ERR_UNSUPPORTED, "moe_permute_quantize: too large for 32-bit offsets");
    const bool want_row = row_codes || row_scales, want_col = col_codes || col_scales;
    if (want_row && !(row_codes && row_scales))
        return fail(MX_ERR_INVALID_ARG, "moe_permute_quantize: row_codes and row_scales go together");
    if (want_col && !(col_codes && col_scales))
        return fail(MX_ERR_INVALID_ARG, "moe_permute_quantize: col_codes and col_scales go together");
    if (!want_row && !want_col)
        return fail(MX_ERR_INVALID_ARG, "moe_permute_quantize: no output requested");
    if (!aligned(x, 16) || (row_codes && !aligned(row_codes, 16)) ||
        (col_codes && !aligned(col_codes, 16)) || (row_scales && !aligned(row_scales, 4)) ||
        (col_scales && !aligned(col_scales, 4)))
        return fail(MX_ERR_INVALID_ARG,
                    "moe_permute_quantize: x and codes 16-byte, scales 4-byte aligned");
    const int64_t bound = padded_bound(M, E, mx::kTokenAlign);
    const int64_t ld = want_col ? col_ld : bound;
    if (want_col && (col_ld % 128 || col_ld < bound))
        return fail(MX_ERR_INVALID_ARG,
                    "moe_permute_quantize: col_ld=%lld must be a multiple of 128 and >= %lld",
                    (long long)col_ld, (long long)bound);
    if (bound / 128 > 65535)
        return fail(MX_ERR_UNSUPPORTED, "moe_permute_quantize: too many rows for one launch");
    {
        const mx_status cs = check_device_offsets("moe_permute_quantize", d_offsets, E, M, true, s);
        if (cs != MX_OK) return cs;
    }
    hipError_t e = timed("padded_offsets", 16.0 * (E + 1), MX_WORK_BYTES, s, [&] {
        return mx::launch_padded_offsets(d_offsets, E, d_padded_offsets, s);
    });
    if (e != hipSuccess) return launched(e, "padded_offsets");
    if (M == 0) return ok();
    return launched(timed("quant_tiles", quant_bytes(M, H, want_row, want_col), MX_WORK_BYTES, s,
                          [&] {
                              return mx::launch_quant_tiles(
                                  static_cast<const uint16_t*>(x), 1, M, H, d_offsets,
                                  d_padded_offsets, E, bound, row_codes, row_scales, col_codes,
                                  col_scales, ld, false, s, d_tok_of, T);
                          }),
                    "quant_tiles(permute)");
}

mx_status moe_combine(const void* y, int64_t M, int64_t H, const int32_t* d_row_of, int64_t T,
                      int32_t k, const float* d_w, void* out, mx_stream_t stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (T < 0 || M < 0 || H <= 0 || k < 1)
        return fail(MX_ERR_INVALID_ARG, "moe_combine: bad sizes");
    if (H % 8)
        return fail(MX_ERR_UNSUPPORTED, "moe_combine: H=%lld is not a multiple of 8", (long long)H);
    if (T > 0 && (!y || !d_row_of || !out))
        return fail(MX_ERR_INVALID_ARG, "moe_combine: NULL argument");
    if (!aligned(y, 16) || !aligned(out, 16))
        return fail(MX_ERR_INVALID_ARG, "moe_combine: y and out must be 16-byte aligned");
    return launched(timed("combine", 2.0 * H * (T * k + T), MX_WORK_BYTES, s,
                          [&] {
                              return mx::launch_combine(static_cast<const uint16_t*>(y), d_row_of,
                                                        d_w, T, k, H, M,
                                                        static_cast<uint16_t*>(out), s);
                          }),
                    "combine");
}

mx_status moe_combine_bwd(const void* dout, int64_t T, int64_t H, int32_t k,
                          const int32_t* d_row_of, const float* d_w, const void* y, int64_t M,
                          void* dy, float* d_dw, mx_stream_t stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (T < 0 || M < 0 || H <= 0 || k < 1)
        return fail(MX_ERR_INVALID_ARG, "moe_combine_bwd: bad sizes");
    if (H % 8)
        return fail(MX_ERR_UNSUPPORTED, "moe_combine_bwd: H=%lld is not a multiple of 8",
                    (long long)H);
    if (T > 0 && (!dout || !d_row_of || !dy))
        return fail(MX_ERR_INVALID_ARG, "moe_combine_bwd: NULL argument");
    if (d_dw && (!d_w || !y))
        return fail(MX_ERR_INVALID_ARG, "moe_combine_bwd: d_dw needs d_w and y");
    if (!aligned(dout, 16) || !aligned(dy, 16) || !aligned(y, 16))
        return fail(MX_ERR_INVALID_ARG, "moe_combine_bwd: dout, y and dy must be 16-byte aligned");
    return launched(timed("combine_bwd", 2.0 * H * (T * k + T), MX_WORK_BYTES, s,
                          [&] {
                              return mx::launch_combine_bwd(
                                  static_cast<const uint16_t*>(dout), d_row_of, d_w,
                                  static_cast<const uint16_t*>(y), T, k, H, M,
                                  static_cast<uint16_t*>(dy), d_dw, s);
                          }),
                    "combine_bwd");
}

mx_status mx_validate_offsets(const int64_t* h_offsets, int32_t G, int64_t M) {
    if (!h_offsets || G < 1 || M < 0)
        return fail(MX_ERR_INVALID_ARG, "mx_validate_offsets: NULL offsets or bad sizes G=%d M=%lld",
                    G, (long long)M);
    const mx_status st = check_offsets_host("mx_validate_offsets", h_offsets, G, M, true);
    return st == MX_OK ? ok() : st;
}

mx_status mx_profile_begin(int32_t capacity) {
    if (capacity < 1 || capacity > (1 << 20))
        return fail(MX_ERR_INVALID_ARG, "mx_profile_begin: capacity %d outside [1, 2^20]", capacity);
    Profiler& P = g_prof;
    P.release();
    P.pool.resize((size_t)capacity * 2);
    for (size_t i = 0; i < P.pool.size(); ++i) {
        if (hipEventCreate(&P.pool[i]) != hipSuccess) {
            P.pool.resize(i);
            P.release();
            return fail(MX_ERR_LAUNCH, "mx_profile_begin: hipEventCreate failed");
        }
    }
    P.recs.reserve((size_t)capacity);
    P.cap = capacity;
    P.on = true;
    return ok();
}

mx_status mx_profile_end(void) {
    g_prof.on = false;
    return ok();
}

int32_t mx_profile_count(void) { return (int32_t)g_prof.recs.size(); }

mx_status mx_profile_get(int32_t i, const char** name, float* ms, double* work, int32_t* unit) {
    Profiler& P = g_prof;
    if (i < 0 || i >= (int32_t)P.recs.size())
        return fail(MX_ERR_INVALID_ARG, "mx_profile_get: no record %d", i);
    const ProfRec& r = P.recs[(size_t)i];
    float t = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess)
        return fail(MX_ERR_LAUNCH, "mx_profile_get: event query failed");
    if (name) *name = r.name;
    if (ms) *ms = t;
    if (work) *work = r.work;
    if (unit) *unit = r.unit;
    return ok();
}

}  // extern "C"
