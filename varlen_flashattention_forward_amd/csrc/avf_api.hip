// C ABI of the packed variable-length attention forward and backward:
// argument checks, the exact tile plans, and the launches. Declarations and contracts are in
// include/attn_varlen.h.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <climits>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/attn_varlen.h"
#include "avf_bwd_plan.h"
#include "avf_plan.h"
#include "avf_quant.h"

namespace {

thread_local std::string g_last_error;

int32_t fail(int32_t code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// (extent, stride) pairs of a tensor: true if no two elements share an
// address (each stride, in increasing order, spans everything below it). A
// tensor without elements never overlaps; otherwise a dimension of extent > 1
// with a stride below 1 (0 repeats one address) always does.
struct Dim { int64_t extent, stride; };
bool non_overlapping_dims(std::vector<Dim> in) {
    for (const Dim& x : in)
        if (x.extent <= 0) return true;
    std::vector<Dim> dims;
    for (const Dim& x : in) {
        if (x.extent <= 1) continue;
        if (x.stride < 1) return false;
        dims.push_back(x);
    }
    std::sort(dims.begin(), dims.end(), [](const Dim& x, const Dim& y) { return x.stride < y.stride; });
    for (size_t i = 1; i < dims.size(); ++i) {
        const __int128 span = (__int128)dims[i - 1].extent * dims[i - 1].stride;
        if ((__int128)dims[i].stride < span) return false;
    }
    return true;
}
// [rows, heads, d] with the innermost dimension contiguous
bool non_overlapping(int64_t rows, int64_t row_stride, int64_t heads, int64_t head_stride,
                     int64_t d) {
    return non_overlapping_dims({{d, 1}, {rows, row_stride}, {heads, head_stride}});
}

int32_t check_flags(uint32_t flags) {
    if (flags & ~ATTN_VARLEN_CAUSAL)
        return fail(ATTN_VARLEN_EINVAL, "unknown option flags 0x%x", (unsigned)(flags & ~ATTN_VARLEN_CAUSAL));
    return ATTN_VARLEN_OK;
}

// Per-segment base offsets of batched tensors (all zero for varlen ones).
struct SegStrides {
    int64_t q, k, v, o, lse;
};

int32_t check_scalars(const void* q, const void* k, const void* v, int32_t B, int32_t H,
                      int32_t D, int32_t max_q, int32_t max_k, const attn_varlen_layout* st,
                      float scale, const void* out, const float* lse) {
    if (B < 0) return fail(ATTN_VARLEN_EINVAL, "num_segments must be >= 0 (got %d)", B);
    if (H <= 0) return fail(ATTN_VARLEN_EINVAL, "num_heads must be >= 1 (got %d)", H);
    if (max_q < 0 || max_k < 0)
        return fail(ATTN_VARLEN_EINVAL, "max_seqlen_q/k must be >= 0 (got %d, %d)", max_q, max_k);
    if (!st) return fail(ATTN_VARLEN_ENULL, "layout is NULL");
    if (st->q_tokens < 0 || st->k_tokens < 0 || st->q_tokens > INT32_MAX || st->k_tokens > INT32_MAX)
        return fail(ATTN_VARLEN_EINVAL, "q_tokens/k_tokens must be in [0, 2^31) (got %lld, %lld)",
                    (long long)st->q_tokens, (long long)st->k_tokens);
    if (avf_block_m(D) <= 0)
        return fail(ATTN_VARLEN_EUNSUPPORTED, "head_dim %d not supported (64, 96 or 128)", D);
    if (!std::isfinite(scale) || !(scale > 0.f))
        return fail(ATTN_VARLEN_EINVAL, "softmax_scale must be finite and > 0 (got %g)", (double)scale);
    if (B == 0) return ATTN_VARLEN_OK;
    // tensors with no token rows may be NULL (nothing is read from or written to them)
    if (st->q_tokens > 0 && (!q || !out)) return fail(ATTN_VARLEN_ENULL, "q and out must be non-NULL");
    if (st->k_tokens > 0 && (!k || !v)) return fail(ATTN_VARLEN_ENULL, "k and v must be non-NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(ATTN_VARLEN_EALIGN, "q, k, v and out must be 16-byte aligned");
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u))
        return fail(ATTN_VARLEN_EALIGN, "lse must be 4-byte aligned");
    const int64_t rows[4] = {st->q_row, st->k_row, st->v_row, st->o_row};
    const int64_t heads[4] = {st->q_head, st->k_head, st->v_head, st->o_head};
    const char* names = "qkvo";
    for (int i = 0; i < 4; ++i) {
        if (rows[i] < 1 || heads[i] < 0)
            return fail(ATTN_VARLEN_EINVAL, "%c strides must be row >= 1, head >= 0 (got %lld, %lld)",
                        names[i], (long long)rows[i], (long long)heads[i]);
        if ((rows[i] & 7) || (heads[i] & 7))
            return fail(ATTN_VARLEN_EALIGN, "%c strides must be multiples of 8 elements (got %lld, %lld)",
                        names[i], (long long)rows[i], (long long)heads[i]);
        if (rows[i] > ATTN_VARLEN_MAX_ROW_STRIDE)
            return fail(ATTN_VARLEN_EUNSUPPORTED, "%c row stride %lld exceeds the limit %lld", names[i],
                        (long long)rows[i], (long long)ATTN_VARLEN_MAX_ROW_STRIDE);
    }
    if (lse && st->lse_head < 0) return fail(ATTN_VARLEN_EINVAL, "lse_head must be >= 0");
    return ATTN_VARLEN_OK;
}

int32_t check_cu(const int32_t* cu_q, const int32_t* cu_k, int32_t B, int32_t max_q,
                 int32_t max_k, const attn_varlen_layout* st) {
    if (!cu_q || !cu_k) return fail(ATTN_VARLEN_ENULL, "cu_seqlens_q/k must be non-NULL");
    if (cu_q[0] != 0 || cu_k[0] != 0)
        return fail(ATTN_VARLEN_ECU, "cu_seqlens must start at 0 (got %d, %d)", cu_q[0], cu_k[0]);
    for (int32_t b = 0; b < B; ++b) {
        const int64_t lq = (int64_t)cu_q[b + 1] - cu_q[b];
        const int64_t lk = (int64_t)cu_k[b + 1] - cu_k[b];
        if (lq < 0 || lk < 0)
            return fail(ATTN_VARLEN_ECU, "cu_seqlens decrease at segment %d (q %lld, k %lld)", b,
                        (long long)lq, (long long)lk);
        if (lq > max_q || lk > max_k)
            return fail(ATTN_VARLEN_EMAXSEQ,
                        "segment %d has %lld query / %lld key rows, over max_seqlen %d / %d", b,
                        (long long)lq, (long long)lk, max_q, max_k);
    }
    if (cu_q[B] > st->q_tokens || cu_k[B] > st->k_tokens)
        return fail(ATTN_VARLEN_ECU, "cu_seqlens end at %d / %d tokens, past q_tokens %lld / k_tokens %lld",
                    cu_q[B], cu_k[B], (long long)st->q_tokens, (long long)st->k_tokens);
    return ATTN_VARLEN_OK;
}

// Checks that need the cu values: output overlap and the LSE head stride.
int32_t check_with_cu(const int32_t* cu_q, int32_t B, int32_t H, int32_t D,
                      const attn_varlen_layout* st, const float* lse) {
    const int64_t total_q = cu_q[B];
    if (!non_overlapping(total_q, st->o_row, H, st->o_head, D))
        return fail(ATTN_VARLEN_EINVAL, "out strides (row %lld, head %lld) make elements overlap",
                    (long long)st->o_row, (long long)st->o_head);
    if (lse && H > 1) {
        const int64_t lh = st->lse_head ? st->lse_head : st->q_tokens;
        if (lh < total_q)
            return fail(ATTN_VARLEN_EINVAL, "lse_head %lld is smaller than total_q %lld", (long long)lh,
                        (long long)total_q);
    }
    return ATTN_VARLEN_OK;
}

// Device cu_seqlens (B+1 entries each) copied to the host on `s` and waited
// for: the one synchronisation of the entry points that take device cu.
int32_t read_cu(const int32_t* cu_q_dev, const int32_t* cu_k_dev, int32_t B, hipStream_t s, std::vector<int32_t>& cu) {
    if (!cu_q_dev || !cu_k_dev) return fail(ATTN_VARLEN_ENULL, "cu_seqlens_q/k must be non-NULL");
    cu.assign((size_t)2 * (B + 1), 0);
    hipError_t e = hipMemcpyAsync(cu.data(), cu_q_dev, sizeof(int32_t) * (B + 1), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(cu.data() + B + 1, cu_k_dev, sizeof(int32_t) * (B + 1), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(ATTN_VARLEN_EHIP, "reading cu_seqlens failed: %s", hipGetErrorString(e));
    return ATTN_VARLEN_OK;
}

int32_t validate_all(const void* q, const void* k, const void* v, const int32_t* cu_q,
                     const int32_t* cu_k, int32_t B, int32_t H, int32_t D, int32_t max_q,
                     int32_t max_k, const attn_varlen_layout* st, float scale, const void* out,
                     const float* lse) {
    int32_t rc = check_scalars(q, k, v, B, H, D, max_q, max_k, st, scale, out, lse);
    if (rc != ATTN_VARLEN_OK || B == 0) return rc;
    rc = check_cu(cu_q, cu_k, B, max_q, max_k, st);
    if (rc != ATTN_VARLEN_OK) return rc;
    return check_with_cu(cu_q, B, H, D, st, lse);
}

// Exact tile count of segments [b0, b1).
int64_t tiles_of(const int32_t* cu_q, int32_t b0, int32_t b1, int32_t H, int32_t bm) {
    int64_t t = 0;
    for (int32_t b = b0; b < b1; ++b) {
        const int64_t lq = (int64_t)cu_q[b + 1] - cu_q[b];
        t += (lq + bm - 1) / bm;
    }
    return t * H;
}

// Fill the launch plan for segments [b0, b1); returns the tile count.
int64_t fill_plan(AvfLaunchArgs& a, const int32_t* cu_q, const int32_t* cu_k, int32_t b0,
                  int32_t b1, int32_t H, int32_t bm) {
    int64_t t = 0;
    a.num_segs = b1 - b0;
    for (int32_t s = 0; s <= b1 - b0; ++s) {
        a.tile_start[s] = (int32_t)t;
        a.q_start[s] = cu_q[b0 + s];
        a.k_start[s] = cu_k[b0 + s];
        if (s < b1 - b0) {
            const int64_t lq = (int64_t)cu_q[b0 + s + 1] - cu_q[b0 + s];
            t += H * ((lq + bm - 1) / bm);
        }
    }
    a.num_tiles = (int32_t)t;
    return t;
}

// Largest tile count one launch may have: the grid size in work-items must
// stay below 2^32 (HSA dispatch limit) with the largest workgroup any tile
// kernel uses, 512 threads (the forward's eight waves).
constexpr int64_t kMaxTilesPerLaunch = ((int64_t)1 << 32) / 512 - 1;

// Every segment of `tiled` (cut into blocks of `bm` rows, times H heads) must
// fit one launch. Checked over all segments before the first HIP call of an
// entry point, so a segment that is too large never leaves earlier launches
// (or the fp8 quantization, or the backward's preprocessing) queued.
int32_t check_launch_limits(const int32_t* tiled, int32_t B, int32_t H, int32_t bm) {
    for (int32_t b = 0; b < B; ++b) {
        const int64_t tb = tiles_of(tiled, b, b + 1, H, bm);
        if (tb > kMaxTilesPerLaunch)
            return fail(ATTN_VARLEN_EUNSUPPORTED, "segment %d needs %lld tiles (limit %lld per launch)", b,
                        (long long)tb, (long long)kMaxTilesPerLaunch);
    }
    return ATTN_VARLEN_OK;
}

// Forward configuration from the call's max_seqlen_k (which bounds every key
// segment: checked against cu_seqlens on the host, or by the device planner):
// one-stage (one 128-key K/V stage), short-stage (64-key stages), or the
// general one. Both small ones run 4-wave, 128-row workgroups two per CU; the
// 8-bit forward always takes the general configuration.
enum class FwdCfg { general, one_stage, short_stage };

FwdCfg fwd_config(int32_t max_k, bool low_precision) {
    if (low_precision) return FwdCfg::general;
    if (max_k <= avf_one_stage_keys()) return FwdCfg::one_stage;
    if (max_k <= avf_short_stage_keys()) return FwdCfg::short_stage;
    return FwdCfg::general;
}

int32_t fwd_block_m(int32_t D, FwdCfg c) { return c == FwdCfg::general ? avf_block_m(D) : avf_block_m_one(D); }

// max_k: the call's validated max_seqlen_k; q8/k8/amax8: the 8-bit score
// operands (NULL for the bf16 path)
int32_t run(const void* q, const void* k, const void* v, const int32_t* cu_q, const int32_t* cu_k,
            int32_t B, int32_t H, int32_t D, const attn_varlen_layout* st, float scale, void* out,
            float* lse, hipStream_t stream, uint32_t flags, int32_t max_k, const SegStrides& seg,
            const uint8_t* q8 = nullptr, const uint8_t* k8 = nullptr, const uint32_t* amax8 = nullptr) {
    const FwdCfg cfg = fwd_config(max_k, q8 != nullptr);
    const int32_t bm = fwd_block_m(D, cfg);
    AvfLaunchArgs a;
    std::memset(&a, 0, sizeof a);
    a.q = q; a.k = k; a.v = v; a.o = out; a.lse = lse;
    a.q_row = st->q_row; a.q_head = st->q_head;
    a.k_row = st->k_row; a.k_head = st->k_head;
    a.v_row = st->v_row; a.v_head = st->v_head;
    a.o_row = st->o_row; a.o_head = st->o_head;
    a.lse_head = st->lse_head ? st->lse_head : st->q_tokens;
    a.scale = scale;
    a.scale_log2e = scale * 1.4426950408889634f;
    a.num_heads = H;
    a.causal = (flags & ATTN_VARLEN_CAUSAL) ? 1 : 0;
    a.q_seg = seg.q; a.k_seg = seg.k; a.v_seg = seg.v; a.o_seg = seg.o; a.lse_seg = seg.lse;
    a.q8 = q8; a.k8 = k8; a.amax8 = amax8;
    a.one_stage = cfg == FwdCfg::one_stage;
    a.short_stage = cfg == FwdCfg::short_stage;
    const int32_t rc = check_launch_limits(cu_q, B, H, bm);
    if (rc != ATTN_VARLEN_OK) return rc;
    for (int32_t b0 = 0; b0 < B;) {
        // segments of this launch: at most AVF_SEGS_PER_LAUNCH and at most
        // kMaxTilesPerLaunch tiles (every single segment fits: checked above)
        int32_t b1 = b0;
        int64_t t = 0;
        while (b1 < B && b1 - b0 < AVF_SEGS_PER_LAUNCH) {
            const int64_t tb = tiles_of(cu_q, b1, b1 + 1, H, bm);
            if (t + tb > kMaxTilesPerLaunch && b1 > b0) break;
            t += tb;
            ++b1;
        }
        const int64_t tiles = fill_plan(a, cu_q, cu_k, b0, b1, H, bm);
        a.seg0 = b0;
        if (tiles > 0) {
            const hipError_t e = avf_launch(a, D, stream);
            if (e != hipSuccess)
                return fail(ATTN_VARLEN_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
        }
        b0 = b1;
    }
    return ATTN_VARLEN_OK;
}

}  // namespace

extern "C" {

int32_t attn_varlen_validate_ex(const void* q, const void* k, const void* v, const int32_t* cu_q,
                                const int32_t* cu_k, int32_t B, int32_t H, int32_t D, int32_t max_q,
                                int32_t max_k, const attn_varlen_layout* st, float scale,
                                uint32_t flags, const void* out, const float* lse) {
    g_last_error.clear();
    int32_t rc = check_flags(flags);
    if (rc != ATTN_VARLEN_OK) return rc;
    rc = validate_all(q, k, v, cu_q, cu_k, B, H, D, max_q, max_k, st, scale, out, lse);
    if (rc != ATTN_VARLEN_OK || B == 0) return rc;
    return check_launch_limits(cu_q, B, H, fwd_block_m(D, fwd_config(max_k, false)));
}

int32_t attn_varlen_validate(const void* q, const void* k, const void* v, const int32_t* cu_q,
                             const int32_t* cu_k, int32_t B, int32_t H, int32_t D, int32_t max_q,
                             int32_t max_k, const attn_varlen_layout* st, float scale,
                             const void* out, const float* lse) {
    return attn_varlen_validate_ex(q, k, v, cu_q, cu_k, B, H, D, max_q, max_k, st, scale, 0u, out, lse);
}

int32_t attn_varlen_fwd_hostcu_ex(const void* q, const void* k, const void* v, const int32_t* cu_q,
                                  const int32_t* cu_k, int32_t B, int32_t H, int32_t D, int32_t max_q,
                                  int32_t max_k, const attn_varlen_layout* st, float scale, uint32_t flags,
                                  void* out, float* lse, void* stream) {
    g_last_error.clear();
    int32_t rc = check_flags(flags);
    if (rc != ATTN_VARLEN_OK) return rc;
    rc = validate_all(q, k, v, cu_q, cu_k, B, H, D, max_q, max_k, st, scale, out, lse);
    if (rc != ATTN_VARLEN_OK || B == 0) return rc;
    return run(q, k, v, cu_q, cu_k, B, H, D, st, scale, out, lse, static_cast<hipStream_t>(stream), flags,
               max_k, SegStrides{0, 0, 0, 0, 0});
}

int32_t attn_varlen_fwd_hostcu(const void* q, const void* k, const void* v, const int32_t* cu_q,
                               const int32_t* cu_k, int32_t B, int32_t H, int32_t D, int32_t max_q,
                               int32_t max_k, const attn_varlen_layout* st, float scale, void* out,
                               float* lse, void* stream) {
    return attn_varlen_fwd_hostcu_ex(q, k, v, cu_q, cu_k, B, H, D, max_q, max_k, st, scale, 0u, out, lse,
                                     stream);
}

int32_t attn_varlen_fwd_ex(const void* q, const void* k, const void* v, const int32_t* cu_q_dev,
                           const int32_t* cu_k_dev, int32_t B, int32_t H, int32_t D, int32_t max_q,
                           int32_t max_k, const attn_varlen_layout* st, float scale, uint32_t flags,
                           void* out, float* lse, void* stream) {
    g_last_error.clear();
    int32_t rc = check_flags(flags);
    if (rc != ATTN_VARLEN_OK) return rc;
    rc = check_scalars(q, k, v, B, H, D, max_q, max_k, st, scale, out, lse);
    if (rc != ATTN_VARLEN_OK || B == 0) return rc;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    std::vector<int32_t> cu;
    if ((rc = read_cu(cu_q_dev, cu_k_dev, B, s, cu)) != ATTN_VARLEN_OK) return rc;
    const int32_t* cq = cu.data();
    const int32_t* ck = cu.data() + B + 1;
    rc = check_cu(cq, ck, B, max_q, max_k, st);
    if (rc != ATTN_VARLEN_OK) return rc;
    rc = check_with_cu(cq, B, H, D, st, lse);
    if (rc != ATTN_VARLEN_OK) return rc;
    return run(q, k, v, cq, ck, B, H, D, st, scale, out, lse, s, flags, max_k, SegStrides{0, 0, 0, 0, 0});
}

int32_t attn_varlen_fwd(const void* q, const void* k, const void* v, const int32_t* cu_q_dev,
                        const int32_t* cu_k_dev, int32_t B, int32_t H, int32_t D, int32_t max_q,
                        int32_t max_k, const attn_varlen_layout* st, float scale, void* out,
                        float* lse, void* stream) {
    return attn_varlen_fwd_ex(q, k, v, cu_q_dev, cu_k_dev, B, H, D, max_q, max_k, st, scale, 0u, out, lse,
                              stream);
}

}  // extern "C"

namespace {

// Batched [W, S, H, D] tensors as W uniform segments: the varlen layout with
// the row and head strides, host cu_seqlens b*S, and per-segment base offsets
// that move segment b's token rows from b*S*row to b*batch.
int32_t batched_plan(const void* q, const void* k, const void* v, int32_t W, int32_t Sq, int32_t Sk,
                     int32_t H, int32_t D, const attn_batched_layout* bl, float scale, uint32_t flags,
                     const void* out, const float* lse, attn_varlen_layout* st, SegStrides* seg,
                     std::vector<int32_t>* cu_q, std::vector<int32_t>* cu_k) {
    int32_t rc = check_flags(flags);
    if (rc != ATTN_VARLEN_OK) return rc;
    if (!bl) return fail(ATTN_VARLEN_ENULL, "layout is NULL");
    if (W < 0 || Sq < 0 || Sk < 0)
        return fail(ATTN_VARLEN_EINVAL, "batch, seqlen_q and seqlen_k must be >= 0 (got %d, %d, %d)", W, Sq, Sk);
    if ((int64_t)W * Sq > INT32_MAX || (int64_t)W * Sk > INT32_MAX)
        return fail(ATTN_VARLEN_EUNSUPPORTED, "batch * seqlen must stay below 2^31");
    const int64_t batch[4] = {bl->q_batch, bl->k_batch, bl->v_batch, bl->o_batch};
    for (int i = 0; i < 4; ++i) {
        if (batch[i] < 0) return fail(ATTN_VARLEN_EINVAL, "batch strides must be >= 0");
        if (batch[i] & 7) return fail(ATTN_VARLEN_EALIGN, "batch strides must be multiples of 8 elements");
    }
    std::memset(st, 0, sizeof *st);
    st->q_row = bl->q_row; st->q_head = bl->q_head;
    st->k_row = bl->k_row; st->k_head = bl->k_head;
    st->v_row = bl->v_row; st->v_head = bl->v_head;
    st->o_row = bl->o_row; st->o_head = bl->o_head;
    st->q_tokens = (int64_t)W * Sq;
    st->k_tokens = (int64_t)W * Sk;
    st->lse_head = bl->lse_head;
    rc = check_scalars(q, k, v, W, H, D, Sq, Sk, st, scale, out, lse);
    if (rc != ATTN_VARLEN_OK) return rc;
    if (!non_overlapping_dims({{D, 1}, {Sq, bl->o_row}, {H, bl->o_head}, {W, bl->o_batch}}))
        return fail(ATTN_VARLEN_EINVAL, "out strides make elements overlap");
    if (lse) {
        if (bl->lse_head < 0 || bl->lse_batch < 0) return fail(ATTN_VARLEN_EINVAL, "lse strides must be >= 0");
        if (!non_overlapping_dims({{Sq, 1}, {H, bl->lse_head}, {W, bl->lse_batch}}))
            return fail(ATTN_VARLEN_EINVAL, "lse strides make elements overlap");
    }
    seg->q = bl->q_batch - (int64_t)Sq * bl->q_row;
    seg->k = bl->k_batch - (int64_t)Sk * bl->k_row;
    seg->v = bl->v_batch - (int64_t)Sk * bl->v_row;
    seg->o = bl->o_batch - (int64_t)Sq * bl->o_row;
    seg->lse = bl->lse_batch - Sq;
    cu_q->resize((size_t)W + 1);
    cu_k->resize((size_t)W + 1);
    for (int32_t b = 0; b <= W; ++b) {
        (*cu_q)[b] = b * Sq;
        (*cu_k)[b] = b * Sk;
    }
    return ATTN_VARLEN_OK;
}

}  // namespace

extern "C" {

int32_t attn_fwd_batched_validate(const void* q, const void* k, const void* v, int32_t W, int32_t Sq,
                                  int32_t Sk, int32_t H, int32_t D, const attn_batched_layout* bl,
                                  float scale, uint32_t flags, const void* out, const float* lse) {
    g_last_error.clear();
    attn_varlen_layout st;
    SegStrides seg;
    std::vector<int32_t> cq, ck;
    return batched_plan(q, k, v, W, Sq, Sk, H, D, bl, scale, flags, out, lse, &st, &seg, &cq, &ck);
}

int32_t attn_fwd_batched(const void* q, const void* k, const void* v, int32_t W, int32_t Sq, int32_t Sk,
                         int32_t H, int32_t D, const attn_batched_layout* bl, float scale, uint32_t flags,
                         void* out, float* lse, void* stream) {
    g_last_error.clear();
    attn_varlen_layout st;
    SegStrides seg;
    std::vector<int32_t> cq, ck;
    const int32_t rc = batched_plan(q, k, v, W, Sq, Sk, H, D, bl, scale, flags, out, lse, &st, &seg, &cq, &ck);
    if (rc != ATTN_VARLEN_OK || W == 0 || Sq == 0) return rc;
    return run(q, k, v, cq.data(), ck.data(), W, H, D, &st, scale, out, lse, static_cast<hipStream_t>(stream),
               flags, Sk, seg);
}

int32_t attn_varlen_block_m(int32_t head_dim) {
    const int32_t bm = avf_block_m(head_dim);
    return bm > 0 ? bm : ATTN_VARLEN_EUNSUPPORTED;
}

int32_t attn_varlen_block_m_for(int32_t head_dim, int32_t max_seqlen_k) {
    g_last_error.clear();
    if (max_seqlen_k < 0) return fail(ATTN_VARLEN_EINVAL, "max_seqlen_k must be >= 0 (got %d)", max_seqlen_k);
    const int32_t bm = fwd_block_m(head_dim, fwd_config(max_seqlen_k, false));
    return bm > 0 ? bm : ATTN_VARLEN_EUNSUPPORTED;
}

int32_t attn_varlen_one_stage_keys(void) { return avf_one_stage_keys(); }

int32_t attn_varlen_short_stage_keys(void) { return avf_short_stage_keys(); }

int64_t attn_varlen_count_tiles(const int32_t* cu_q, int32_t B, int32_t H, int32_t block_m) {
    g_last_error.clear();
    if (!cu_q) return fail(ATTN_VARLEN_ENULL, "cu_seqlens_q is NULL");
    if (B < 0 || H <= 0 || block_m <= 0) return fail(ATTN_VARLEN_EINVAL, "bad counts");
    if (B > 0 && cu_q[0] != 0) return fail(ATTN_VARLEN_ECU, "cu_seqlens_q must start at 0");
    for (int32_t b = 0; b < B; ++b)
        if (cu_q[b + 1] < cu_q[b]) return fail(ATTN_VARLEN_ECU, "cu_seqlens_q decreases at %d", b);
    return tiles_of(cu_q, 0, B, H, block_m);
}

int32_t attn_varlen_segments_per_launch(void) { return AVF_SEGS_PER_LAUNCH; }

int32_t attn_varlen_grid_plan(const int32_t* cu_q, int32_t B, int32_t H, int32_t D, int32_t max_k,
                              int64_t* launches, int64_t* workgroups) {
    g_last_error.clear();
    if (!cu_q || !launches || !workgroups) return fail(ATTN_VARLEN_ENULL, "NULL argument");
    if (max_k < 0) return fail(ATTN_VARLEN_EINVAL, "max_seqlen_k must be >= 0 (got %d)", max_k);
    const int32_t bm = fwd_block_m(D, fwd_config(max_k, false));
    if (bm <= 0) return fail(ATTN_VARLEN_EUNSUPPORTED, "head_dim %d not supported", D);
    if (B < 0 || H <= 0) return fail(ATTN_VARLEN_EINVAL, "bad counts");
    int64_t nl = 0, nw = 0;
    for (int32_t b0 = 0; b0 < B;) {
        int32_t b1 = b0;
        int64_t t = 0;
        while (b1 < B && b1 - b0 < AVF_SEGS_PER_LAUNCH) {
            const int64_t tb = tiles_of(cu_q, b1, b1 + 1, H, bm);
            if (t + tb > kMaxTilesPerLaunch && b1 > b0) break;
            if (tb > kMaxTilesPerLaunch)
                return fail(ATTN_VARLEN_EUNSUPPORTED, "segment %d needs %lld tiles (limit %lld per launch)",
                            b1, (long long)tb, (long long)kMaxTilesPerLaunch);
            t += tb;
            ++b1;
        }
        if (t > 0) ++nl;
        nw += t;
        b0 = b1;
    }
    *launches = nl;
    *workgroups = nw;
    return ATTN_VARLEN_OK;
}

int64_t attn_varlen_num_tiles(const int32_t* cu_q, int32_t B, int32_t H, int32_t D, int32_t max_k) {
    g_last_error.clear();
    if (!cu_q) return fail(ATTN_VARLEN_ENULL, "cu_seqlens_q is NULL");
    if (B < 0 || H <= 0) return fail(ATTN_VARLEN_EINVAL, "bad counts");
    if (B > 0 && cu_q[0] != 0) return fail(ATTN_VARLEN_ECU, "cu_seqlens_q must start at 0");
    for (int32_t b = 0; b < B; ++b)
        if (cu_q[b + 1] < cu_q[b]) return fail(ATTN_VARLEN_ECU, "cu_seqlens_q decreases at %d", b);
    int64_t launches = 0, workgroups = 0;
    const int32_t rc = attn_varlen_grid_plan(cu_q, B, H, D, max_k, &launches, &workgroups);
    return rc != ATTN_VARLEN_OK ? rc : workgroups;
}

int32_t attn_varlen_decode_tile(const int32_t* cu_q, int32_t B, int32_t H, int32_t block_m,
                                int64_t wg, int32_t* segment, int32_t* q_block, int32_t* head) {
    g_last_error.clear();
    if (!cu_q || !segment || !q_block || !head) return fail(ATTN_VARLEN_ENULL, "NULL argument");
    if (B <= 0 || B > AVF_SEGS_PER_LAUNCH || H <= 0 || block_m <= 0)
        return fail(ATTN_VARLEN_EINVAL, "bad counts");
    AvfLaunchArgs a;
    std::memset(&a, 0, sizeof a);
    const int64_t t = fill_plan(a, cu_q, cu_q, 0, B, H, block_m);
    if (wg < 0 || wg >= t) return fail(ATTN_VARLEN_EINVAL, "workgroup %lld outside grid of %lld", (long long)wg, (long long)t);
    const int32_t lin = avf_linear_tile((int32_t)wg, a.num_tiles);
    const AvfTile tile = avf_decode(lin, a.tile_start, a.q_start, a.num_segs, H, block_m);
    *segment = tile.seg;
    *q_block = tile.mblk;
    *head = tile.head;
    return ATTN_VARLEN_OK;
}

int64_t attn_varlen_element_offset(int64_t row, int64_t row_stride, int64_t head,
                                   int64_t head_stride) {
    return avf_elem_offset(row, row_stride, head, head_stride);
}

const char* attn_varlen_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

// ---------------------------------------------------------------------------
// Backward

namespace {

// Token-row / head strides of one bf16 [rows, H, D] tensor.
int32_t check_strides(const char* name, int64_t row, int64_t head) {
    if (row < 1 || head < 0)
        return fail(ATTN_VARLEN_EINVAL, "%s strides must be row >= 1, head >= 0 (got %lld, %lld)", name,
                    (long long)row, (long long)head);
    if ((row & 7) || (head & 7))
        return fail(ATTN_VARLEN_EALIGN, "%s strides must be multiples of 8 elements (got %lld, %lld)", name,
                    (long long)row, (long long)head);
    if (row > ATTN_VARLEN_MAX_ROW_STRIDE)
        return fail(ATTN_VARLEN_EUNSUPPORTED, "%s row stride %lld exceeds the limit %lld", name, (long long)row,
                    (long long)ATTN_VARLEN_MAX_ROW_STRIDE);
    return ATTN_VARLEN_OK;
}

int32_t check_fp32_head(const char* name, int64_t head, int64_t rows, int32_t H) {
    if (head < 0) return fail(ATTN_VARLEN_EINVAL, "%s_head must be >= 0", name);
    if (H > 1 && head < rows)
        return fail(ATTN_VARLEN_EINVAL, "%s_head %lld is smaller than the %lld rows", name, (long long)head,
                    (long long)rows);
    return ATTN_VARLEN_OK;
}

int32_t bwd_check_scalars(const void* q, const void* k, const void* v, const void* o, const void* g,
                          const float* lse, int32_t B, int32_t H, int32_t D, int32_t max_q, int32_t max_k,
                          const attn_varlen_bwd_layout* st, float scale, uint32_t flags, const float* delta,
                          const void* dq, const void* dk, const void* dv) {
    int32_t rc = check_flags(flags);
    if (rc != ATTN_VARLEN_OK) return rc;
    if (B < 0) return fail(ATTN_VARLEN_EINVAL, "num_segments must be >= 0 (got %d)", B);
    if (H <= 0) return fail(ATTN_VARLEN_EINVAL, "num_heads must be >= 1 (got %d)", H);
    if (max_q < 0 || max_k < 0)
        return fail(ATTN_VARLEN_EINVAL, "max_seqlen_q/k must be >= 0 (got %d, %d)", max_q, max_k);
    if (!st) return fail(ATTN_VARLEN_ENULL, "layout is NULL");
    if (st->q_tokens < 0 || st->k_tokens < 0 || st->q_tokens > INT32_MAX || st->k_tokens > INT32_MAX)
        return fail(ATTN_VARLEN_EINVAL, "q_tokens/k_tokens must be in [0, 2^31) (got %lld, %lld)",
                    (long long)st->q_tokens, (long long)st->k_tokens);
    if (avf_bwd_block_n(D) <= 0)
        return fail(ATTN_VARLEN_EUNSUPPORTED, "head_dim %d not supported (64, 96 or 128)", D);
    if (!std::isfinite(scale) || !(scale > 0.f))
        return fail(ATTN_VARLEN_EINVAL, "softmax_scale must be finite and > 0 (got %g)", (double)scale);
    if (B == 0) return ATTN_VARLEN_OK;
    if (st->q_tokens > 0 && (!q || !o || !g || !dq || !lse || !delta))
        return fail(ATTN_VARLEN_ENULL, "q, out, dout, dq, lse and delta must be non-NULL");
    if (st->k_tokens > 0 && (!k || !v || !dk || !dv))
        return fail(ATTN_VARLEN_ENULL, "k, v, dk and dv must be non-NULL");
    const void* bf[8] = {q, k, v, o, g, dq, dk, dv};
    for (const void* p : bf)
        if (!aligned16(p)) return fail(ATTN_VARLEN_EALIGN, "q, k, v, out, dout, dq, dk and dv must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(delta) & 3u))
        return fail(ATTN_VARLEN_EALIGN, "lse and delta must be 4-byte aligned");
    const struct { const char* n; int64_t r, h; } t[8] = {
        {"q", st->q_row, st->q_head},    {"k", st->k_row, st->k_head},    {"v", st->v_row, st->v_head},
        {"out", st->o_row, st->o_head},  {"dout", st->do_row, st->do_head}, {"dq", st->dq_row, st->dq_head},
        {"dk", st->dk_row, st->dk_head}, {"dv", st->dv_row, st->dv_head}};
    for (const auto& x : t)
        if ((rc = check_strides(x.n, x.r, x.h)) != ATTN_VARLEN_OK) return rc;
    return ATTN_VARLEN_OK;
}

// Checks that need the cu values (host arrays).
int32_t bwd_check_cu(const int32_t* cu_q, const int32_t* cu_k, int32_t B, int32_t H, int32_t D, int32_t max_q,
                     int32_t max_k, const attn_varlen_bwd_layout* st) {
    attn_varlen_layout ext;
    std::memset(&ext, 0, sizeof ext);
    ext.q_tokens = st->q_tokens;
    ext.k_tokens = st->k_tokens;
    int32_t rc = check_cu(cu_q, cu_k, B, max_q, max_k, &ext);
    if (rc != ATTN_VARLEN_OK) return rc;
    const int64_t tq = cu_q[B], tk = cu_k[B];
    if (!non_overlapping(tq, st->dq_row, H, st->dq_head, D))
        return fail(ATTN_VARLEN_EINVAL, "dq strides make elements overlap");
    if (!non_overlapping(tk, st->dk_row, H, st->dk_head, D))
        return fail(ATTN_VARLEN_EINVAL, "dk strides make elements overlap");
    if (!non_overlapping(tk, st->dv_row, H, st->dv_head, D))
        return fail(ATTN_VARLEN_EINVAL, "dv strides make elements overlap");
    if ((rc = check_fp32_head("lse", st->lse_head ? st->lse_head : st->q_tokens, tq, H)) != ATTN_VARLEN_OK)
        return rc;
    return check_fp32_head("delta", st->delta_head ? st->delta_head : st->q_tokens, tq, H);
}

// Rows of the preprocessing pass per launch: H * rows items, 16 per
// 256-thread workgroup, keep the grid below 2^32 work-items.
constexpr int64_t kPreItemsPerLaunch = (int64_t)1 << 27;

hipError_t preprocess(const void* o, const void* g, int64_t rows, int32_t H, int32_t D, int64_t o_row,
                      int64_t o_head, int64_t do_row, int64_t do_head, float* delta, int64_t delta_head,
                      hipStream_t s) {
    const int64_t chunk = std::max<int64_t>(1, kPreItemsPerLaunch / H);
    for (int64_t r0 = 0; r0 < rows; r0 += chunk) {
        AvfPreArgs p;
        p.o = (const char*)o + 2 * r0 * o_row;
        p.dout = (const char*)g + 2 * r0 * do_row;
        p.delta = delta + r0;
        p.o_row = o_row; p.o_head = o_head; p.do_row = do_row; p.do_head = do_head;
        p.delta_head = delta_head;
        p.rows = std::min(chunk, rows - r0);
        p.num_heads = H;
        const hipError_t e = avf_bwd_preprocess_launch(p, D, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Launches of one tile kernel over all segments; `tiled` is the cu array
// whose segment lengths are cut into blocks of `bm` (keys for dK/dV, query
// rows for dQ). Each launch carries at most AVF_SEGS_PER_LAUNCH segments and
// kMaxTilesPerLaunch tiles. With `count` set only counts, launching nothing.
template <typename Launch>
int32_t for_each_launch(AvfBwdArgs& a, const int32_t* cu_q, const int32_t* cu_k, const int32_t* tiled, int32_t B,
                        int32_t H, int32_t bm, Launch&& launch, int64_t* launches, int64_t* workgroups) {
    for (int32_t b0 = 0; b0 < B;) {
        int32_t b1 = b0;
        int64_t t = 0;
        while (b1 < B && b1 - b0 < AVF_SEGS_PER_LAUNCH) {
            const int64_t tb = tiles_of(tiled, b1, b1 + 1, H, bm);
            if (t + tb > kMaxTilesPerLaunch && b1 > b0) break;
            if (tb > kMaxTilesPerLaunch)
                return fail(ATTN_VARLEN_EUNSUPPORTED, "segment %d needs %lld tiles (limit %lld per launch)", b1,
                            (long long)tb, (long long)kMaxTilesPerLaunch);
            t += tb;
            ++b1;
        }
        int64_t acc = 0;
        a.num_segs = b1 - b0;
        for (int32_t s = 0; s <= b1 - b0; ++s) {
            a.tile_start[s] = (int32_t)acc;
            a.q_start[s] = cu_q[b0 + s];
            a.k_start[s] = cu_k[b0 + s];
            if (s < b1 - b0) acc += tiles_of(tiled, b0 + s, b0 + s + 1, H, bm);
        }
        a.num_tiles = (int32_t)acc;
        if (acc > 0) {
            if (launches) ++*launches;
            if (workgroups) *workgroups += acc;
            const hipError_t e = launch(a);
            if (e != hipSuccess) return fail(ATTN_VARLEN_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
        }
        b0 = b1;
    }
    return ATTN_VARLEN_OK;
}

AvfBwdArgs bwd_args(const void* q, const void* k, const void* v, const void* g, const float* lse, const float* delta,
                    void* dq, void* dk, void* dv, int32_t H, const attn_varlen_bwd_layout* st, float scale,
                    uint32_t flags) {
    AvfBwdArgs a;
    std::memset(&a, 0, sizeof a);
    a.q = q; a.k = k; a.v = v; a.dout = g; a.lse = lse; a.delta = delta; a.dq = dq; a.dk = dk; a.dv = dv;
    a.q_row = st->q_row; a.q_head = st->q_head; a.k_row = st->k_row; a.k_head = st->k_head;
    a.v_row = st->v_row; a.v_head = st->v_head; a.do_row = st->do_row; a.do_head = st->do_head;
    a.dq_row = st->dq_row; a.dq_head = st->dq_head; a.dk_row = st->dk_row; a.dk_head = st->dk_head;
    a.dv_row = st->dv_row; a.dv_head = st->dv_head;
    a.lse_head = st->lse_head ? st->lse_head : st->q_tokens;
    a.delta_head = st->delta_head ? st->delta_head : st->q_tokens;
    a.scale = scale;
    a.scale_log2e = scale * 1.4426950408889634f;
    a.causal = (flags & ATTN_VARLEN_CAUSAL) ? 1 : 0;
    a.num_heads = H;
    return a;
}

int32_t bwd_run(const void* q, const void* k, const void* v, const void* o, const void* g, const float* lse,
                const int32_t* cu_q, const int32_t* cu_k, int32_t B, int32_t H, int32_t D,
                const attn_varlen_bwd_layout* st, float scale, uint32_t flags, float* delta, void* dq, void* dk,
                void* dv, hipStream_t s) {
    int32_t rc = check_launch_limits(cu_k, B, H, avf_bwd_block_n(D));
    if (rc == ATTN_VARLEN_OK) rc = check_launch_limits(cu_q, B, H, avf_bwd_block_m(D));
    if (rc != ATTN_VARLEN_OK) return rc;
    const int64_t delta_head = st->delta_head ? st->delta_head : st->q_tokens;
    hipError_t e = preprocess(o, g, cu_q[B], H, D, st->o_row, st->o_head, st->do_row, st->do_head, delta,
                              delta_head, s);
    if (e != hipSuccess) return fail(ATTN_VARLEN_EHIP, "preprocessing launch failed: %s", hipGetErrorString(e));
    AvfBwdArgs a = bwd_args(q, k, v, g, lse, delta, dq, dk, dv, H, st, scale, flags);
    rc = for_each_launch(a, cu_q, cu_k, cu_k, B, H, avf_bwd_block_n(D),
                                 [&](const AvfBwdArgs& x) { return avf_bwd_dkdv_launch(x, D, s); }, nullptr, nullptr);
    if (rc != ATTN_VARLEN_OK) return rc;
    return for_each_launch(a, cu_q, cu_k, cu_q, B, H, avf_bwd_block_m(D),
                           [&](const AvfBwdArgs& x) { return avf_bwd_dq_launch(x, D, s); }, nullptr, nullptr);
}

}  // namespace

extern "C" {

int32_t attn_varlen_bwd_preprocess(const void* out, const void* dout, int64_t rows, int32_t H, int32_t D,
                                   int64_t o_row, int64_t o_head, int64_t do_row, int64_t do_head, float* delta,
                                   int64_t delta_head, void* stream) {
    g_last_error.clear();
    if (rows < 0 || rows > INT32_MAX) return fail(ATTN_VARLEN_EINVAL, "rows must be in [0, 2^31) (got %lld)", (long long)rows);
    if (H <= 0) return fail(ATTN_VARLEN_EINVAL, "num_heads must be >= 1 (got %d)", H);
    if (avf_bwd_block_n(D) <= 0)
        return fail(ATTN_VARLEN_EUNSUPPORTED, "head_dim %d not supported (64, 96 or 128)", D);
    if (rows == 0) return ATTN_VARLEN_OK;
    if (!out || !dout || !delta) return fail(ATTN_VARLEN_ENULL, "out, dout and delta must be non-NULL");
    if (!aligned16(out) || !aligned16(dout)) return fail(ATTN_VARLEN_EALIGN, "out and dout must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(delta) & 3u) return fail(ATTN_VARLEN_EALIGN, "delta must be 4-byte aligned");
    int32_t rc = check_strides("out", o_row, o_head);
    if (rc == ATTN_VARLEN_OK) rc = check_strides("dout", do_row, do_head);
    if (rc == ATTN_VARLEN_OK) rc = check_fp32_head("delta", delta_head, rows, H);
    if (rc != ATTN_VARLEN_OK) return rc;
    const hipError_t e = preprocess(out, dout, rows, H, D, o_row, o_head, do_row, do_head, delta, delta_head,
                                    static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(ATTN_VARLEN_EHIP, "preprocessing launch failed: %s", hipGetErrorString(e));
    return ATTN_VARLEN_OK;
}

int32_t attn_varlen_bwd_validate(const void* q, const void* k, const void* v, const void* o, const void* g,
                                 const float* lse, const int32_t* cu_q, const int32_t* cu_k, int32_t B, int32_t H,
                                 int32_t D, int32_t max_q, int32_t max_k, const attn_varlen_bwd_layout* st,
                                 float scale, uint32_t flags, const float* delta, const void* dq, const void* dk,
                                 const void* dv) {
    g_last_error.clear();
    int32_t rc = bwd_check_scalars(q, k, v, o, g, lse, B, H, D, max_q, max_k, st, scale, flags, delta, dq, dk, dv);
    if (rc != ATTN_VARLEN_OK || B == 0) return rc;
    return bwd_check_cu(cu_q, cu_k, B, H, D, max_q, max_k, st);
}

int32_t attn_varlen_bwd_hostcu(const void* q, const void* k, const void* v, const void* o, const void* g,
                               const float* lse, const int32_t* cu_q, const int32_t* cu_k, int32_t B, int32_t H,
                               int32_t D, int32_t max_q, int32_t max_k, const attn_varlen_bwd_layout* st,
                               float scale, uint32_t flags, float* delta, void* dq, void* dk, void* dv,
                               void* stream) {
    const int32_t rc =
        attn_varlen_bwd_validate(q, k, v, o, g, lse, cu_q, cu_k, B, H, D, max_q, max_k, st, scale, flags, delta, dq,
                                 dk, dv);
    if (rc != ATTN_VARLEN_OK || B == 0) return rc;
    return bwd_run(q, k, v, o, g, lse, cu_q, cu_k, B, H, D, st, scale, flags, delta, dq, dk, dv,
                   static_cast<hipStream_t>(stream));
}

int32_t attn_varlen_bwd(const void* q, const void* k, const void* v, const void* o, const void* g, const float* lse,
                        const int32_t* cu_q_dev, const int32_t* cu_k_dev, int32_t B, int32_t H, int32_t D,
                        int32_t max_q, int32_t max_k, const attn_varlen_bwd_layout* st, float scale, uint32_t flags,
                        float* delta, void* dq, void* dk, void* dv, void* stream) {
    g_last_error.clear();
    int32_t rc = bwd_check_scalars(q, k, v, o, g, lse, B, H, D, max_q, max_k, st, scale, flags, delta, dq, dk, dv);
    if (rc != ATTN_VARLEN_OK || B == 0) return rc;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    std::vector<int32_t> cu;
    if ((rc = read_cu(cu_q_dev, cu_k_dev, B, s, cu)) != ATTN_VARLEN_OK) return rc;
    const int32_t* cq = cu.data();
    const int32_t* ck = cu.data() + B + 1;
    rc = bwd_check_cu(cq, ck, B, H, D, max_q, max_k, st);
    if (rc != ATTN_VARLEN_OK) return rc;
    return bwd_run(q, k, v, o, g, lse, cq, ck, B, H, D, st, scale, flags, delta, dq, dk, dv, s);
}

int32_t attn_varlen_bwd_grid_plan(const int32_t* cu_q, const int32_t* cu_k, int32_t B, int32_t H, int32_t D,
                                  int64_t* pre_workgroups, int64_t* dkdv_workgroups, int64_t* dq_workgroups,
                                  int64_t* launches) {
    g_last_error.clear();
    if (!cu_q || !cu_k || !pre_workgroups || !dkdv_workgroups || !dq_workgroups || !launches)
        return fail(ATTN_VARLEN_ENULL, "NULL argument");
    if (avf_bwd_block_n(D) <= 0) return fail(ATTN_VARLEN_EUNSUPPORTED, "head_dim %d not supported", D);
    if (B < 0 || H <= 0) return fail(ATTN_VARLEN_EINVAL, "bad counts");
    *pre_workgroups = *dkdv_workgroups = *dq_workgroups = *launches = 0;
    if (B == 0) return ATTN_VARLEN_OK;
    const int64_t items = (int64_t)cu_q[B] * H;
    const int64_t chunk_rows = std::max<int64_t>(1, kPreItemsPerLaunch / H);
    for (int64_t r0 = 0; r0 < cu_q[B]; r0 += chunk_rows)
        *pre_workgroups += (std::min<int64_t>(chunk_rows, cu_q[B] - r0) * H + 15) / 16;
    (void)items;
    AvfBwdArgs a;
    std::memset(&a, 0, sizeof a);
    auto none = [](const AvfBwdArgs&) { return hipSuccess; };
    int32_t rc = for_each_launch(a, cu_q, cu_k, cu_k, B, H, avf_bwd_block_n(D), none, launches, dkdv_workgroups);
    if (rc != ATTN_VARLEN_OK) return rc;
    return for_each_launch(a, cu_q, cu_k, cu_q, B, H, avf_bwd_block_m(D), none, launches, dq_workgroups);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Sync-free forward: device planner + bounded, looping grid

namespace {

// Workgroups of a device-planned launch: at most this many (a multiple of 8;
// larger problems loop), and never more than the bound on the tile count.
constexpr int64_t kAsyncMaxGrid = 8192;

int64_t async_workspace_bytes(int32_t B) {
    const int64_t bytes = 4 * ((int64_t)AVF_PLAN_HEADER_WORDS + B + 1);
    return (bytes + 255) / 256 * 256;
}

// Upper bound on H * sum_b ceil(Lq_b / bm) from host-known values only:
// sum_b ceil(Lq_b / bm) <= ceil((total_q + B * (bm - 1)) / bm) with
// total_q <= q_tokens (the SM120 page's grid formula), and <= B * ceil(max_q / bm).
int64_t async_tile_bound(int64_t q_tokens, int32_t B, int32_t H, int32_t bm, int32_t max_q) {
    const int64_t a = (q_tokens + (int64_t)B * (bm - 1) + bm - 1) / bm;
    const int64_t b = (int64_t)B * ((max_q + bm - 1) / bm);
    return (int64_t)H * std::min(a, b);
}

int64_t async_grid(int64_t bound) {
    const int64_t g = std::min(bound, kAsyncMaxGrid);
    return (g + AVF_NUM_XCD - 1) / AVF_NUM_XCD * AVF_NUM_XCD;
}

// Host-side checks of the sync-free forward (every value the host knows; the
// cu values are checked by the planner on the device).
int32_t async_check(const void* q, const void* k, const void* v, const int32_t* cu_q_dev, const int32_t* cu_k_dev,
                    int32_t B, int32_t H, int32_t D, int32_t max_q, int32_t max_k, const attn_varlen_layout* st,
                    float scale, uint32_t flags, const void* out, const float* lse) {
    int32_t rc = check_flags(flags);
    if (rc != ATTN_VARLEN_OK) return rc;
    rc = check_scalars(q, k, v, B, H, D, max_q, max_k, st, scale, out, lse);
    if (rc != ATTN_VARLEN_OK || B == 0) return rc;
    if (!cu_q_dev || !cu_k_dev) return fail(ATTN_VARLEN_ENULL, "cu_seqlens_q/k must be non-NULL");
    // the checks that need cu, with q_tokens standing in for the unknown total_q
    if (!non_overlapping(st->q_tokens, st->o_row, H, st->o_head, D))
        return fail(ATTN_VARLEN_EINVAL, "out strides (row %lld, head %lld) make elements overlap",
                    (long long)st->o_row, (long long)st->o_head);
    if (lse && H > 1 && st->lse_head != 0 && st->lse_head < st->q_tokens)
        return fail(ATTN_VARLEN_EINVAL, "lse_head %lld is smaller than q_tokens %lld", (long long)st->lse_head,
                    (long long)st->q_tokens);
    return ATTN_VARLEN_OK;
}

// The planner kernel into `ws` (a plan buffer of at least
// async_workspace_bytes(B) bytes), then the attention kernel on the host
// bound of the tile count, both on stream `s`.
int32_t async_launch(const void* q, const void* k, const void* v, const int32_t* cu_q_dev, const int32_t* cu_k_dev,
                     int32_t B, int32_t H, int32_t D, int32_t max_q, int32_t max_k, const attn_varlen_layout* st,
                     float scale, uint32_t flags, int32_t* ws, void* out, float* lse, hipStream_t s) {
    // the planner rejects any segment over max_k, so max_k may pick the one-stage configuration
    const FwdCfg cfg = fwd_config(max_k, false);
    const int32_t bm = fwd_block_m(D, cfg);
    hipError_t e = avf_plan_launch(cu_q_dev, cu_k_dev, B, H, bm, 0, max_q, max_k, st->q_tokens, st->k_tokens, ws, s);
    if (e != hipSuccess) return fail(ATTN_VARLEN_EHIP, "planner launch failed: %s", hipGetErrorString(e));
    const int64_t grid = async_grid(async_tile_bound(st->q_tokens, B, H, bm, max_q));
    if (grid == 0) return ATTN_VARLEN_OK;
    AvfLaunchArgs a;
    std::memset(&a, 0, sizeof a);
    a.q = q; a.k = k; a.v = v; a.o = out; a.lse = lse;
    a.q_row = st->q_row; a.q_head = st->q_head;
    a.k_row = st->k_row; a.k_head = st->k_head;
    a.v_row = st->v_row; a.v_head = st->v_head;
    a.o_row = st->o_row; a.o_head = st->o_head;
    a.lse_head = st->lse_head ? st->lse_head : st->q_tokens;
    a.scale = scale;
    a.scale_log2e = scale * 1.4426950408889634f;
    a.num_heads = H;
    a.causal = (flags & ATTN_VARLEN_CAUSAL) ? 1 : 0;
    a.dev_plan = ws;
    a.cu_q = cu_q_dev;
    a.cu_k = cu_k_dev;
    a.num_segs = B;
    a.num_tiles = (int32_t)grid;
    a.one_stage = cfg == FwdCfg::one_stage;
    a.short_stage = cfg == FwdCfg::short_stage;
    e = avf_launch(a, D, s);
    if (e != hipSuccess) return fail(ATTN_VARLEN_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ATTN_VARLEN_OK;
}

}  // namespace

extern "C" {

int64_t attn_varlen_async_workspace_bytes(int32_t B) {
    g_last_error.clear();
    if (B < 0) return fail(ATTN_VARLEN_EINVAL, "num_segments must be >= 0 (got %d)", B);
    return async_workspace_bytes(B);
}

int32_t attn_varlen_async_grid(int64_t q_tokens, int32_t B, int32_t H, int32_t D, int32_t max_q, int32_t max_k,
                               int64_t* workgroups) {
    g_last_error.clear();
    if (!workgroups) return fail(ATTN_VARLEN_ENULL, "NULL argument");
    if (B < 0 || H <= 0 || q_tokens < 0 || max_q < 0 || max_k < 0) return fail(ATTN_VARLEN_EINVAL, "bad counts");
    const int32_t bm = fwd_block_m(D, fwd_config(max_k, false));
    if (bm <= 0) return fail(ATTN_VARLEN_EUNSUPPORTED, "head_dim %d not supported", D);
    *workgroups = async_grid(async_tile_bound(q_tokens, B, H, bm, max_q));
    return ATTN_VARLEN_OK;
}

int32_t attn_varlen_fwd_async(const void* q, const void* k, const void* v, const int32_t* cu_q_dev,
                              const int32_t* cu_k_dev, int32_t B, int32_t H, int32_t D, int32_t max_q,
                              int32_t max_k, const attn_varlen_layout* st, float scale, uint32_t flags,
                              void* workspace, int64_t workspace_bytes, void* out, float* lse, void* stream) {
    g_last_error.clear();
    const int32_t rc = async_check(q, k, v, cu_q_dev, cu_k_dev, B, H, D, max_q, max_k, st, scale, flags, out, lse);
    if (rc != ATTN_VARLEN_OK || B == 0) return rc;
    if (!workspace) return fail(ATTN_VARLEN_ENULL, "workspace must be non-NULL");
    if (reinterpret_cast<uintptr_t>(workspace) & 15u) return fail(ATTN_VARLEN_EALIGN, "workspace must be 16-byte aligned");
    if (workspace_bytes < async_workspace_bytes(B))
        return fail(ATTN_VARLEN_EINVAL, "workspace of %lld bytes is smaller than the %lld needed",
                    (long long)workspace_bytes, (long long)async_workspace_bytes(B));
    return async_launch(q, k, v, cu_q_dev, cu_k_dev, B, H, D, max_q, max_k, st, scale, flags,
                        static_cast<int32_t*>(workspace), out, lse, static_cast<hipStream_t>(stream));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Sync-free forward without any allocation: the plan lives in a static
// device array of the library, one copy per GPU.

namespace {

// Largest segment count of one call of the no-allocation entry point; the
// plan needs AVF_PLAN_HEADER_WORDS + B + 1 words.
constexpr int32_t kNoAllocMaxSegments = 65536;
constexpr int64_t kScratchWords = ((int64_t)AVF_PLAN_HEADER_WORDS + kNoAllocMaxSegments + 1 + 63) / 64 * 64;
static_assert(kScratchWords * 4 >= 4 * ((int64_t)AVF_PLAN_HEADER_WORDS + kNoAllocMaxSegments + 1),
              "the static plan holds the largest accepted call");
constexpr int kMaxDevices = 64;

}  // namespace

// The plan buffer of attn_varlen_fwd_async_noalloc (about 256 KiB). Each GPU
// the library runs on holds its own copy until the process ends. In host
// code this name only stands in for the device array: its device address,
// per GPU, comes from hipGetSymbolAddress and is the only way host code
// refers to it.
static __device__ __align__(256) int32_t scratch[kScratchWords];

namespace {

std::mutex g_scratch_mutex;
int32_t* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each GPU

// Device address of `scratch` on the current GPU, looked up once per GPU
// (with that GPU current) and kept.
int32_t scratch_on_current_device(int32_t** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ATTN_VARLEN_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(ATTN_VARLEN_EUNSUPPORTED, "device %d is past the %d GPUs the static plan serves", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(ATTN_VARLEN_EHIP, "hipGetSymbolAddress of the static plan failed: %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = static_cast<int32_t*>(p);
    }
    *ptr = g_scratch_ptr[dev];
    return ATTN_VARLEN_OK;
}

}  // namespace

extern "C" {

int32_t attn_varlen_fwd_async_noalloc(const void* q, const void* k, const void* v, const int32_t* cu_q_dev,
                                      const int32_t* cu_k_dev, int32_t B, int32_t H, int32_t D, int32_t max_q,
                                      int32_t max_k, const attn_varlen_layout* st, float scale, uint32_t flags,
                                      void* out, float* lse, void* stream, const void** plan) {
    g_last_error.clear();
    if (plan) *plan = nullptr;
    int32_t rc = async_check(q, k, v, cu_q_dev, cu_k_dev, B, H, D, max_q, max_k, st, scale, flags, out, lse);
    if (rc != ATTN_VARLEN_OK || B == 0) return rc;
    if (B > kNoAllocMaxSegments)
        return fail(ATTN_VARLEN_EUNSUPPORTED, "num_segments %d exceeds the static plan's limit of %d segments", B,
                    kNoAllocMaxSegments);
    int32_t* ws = nullptr;
    if ((rc = scratch_on_current_device(&ws)) != ATTN_VARLEN_OK) return rc;
    if (plan) *plan = ws;
    return async_launch(q, k, v, cu_q_dev, cu_k_dev, B, H, D, max_q, max_k, st, scale, flags, ws, out, lse,
                        static_cast<hipStream_t>(stream));
}

int32_t attn_varlen_async_status(const void* workspace, void* stream, int32_t* status) {
    g_last_error.clear();
    if (!workspace || !status) return fail(ATTN_VARLEN_ENULL, "workspace and status must be non-NULL");
    const hipStream_t s = static_cast<hipStream_t>(stream);
    int32_t word = 0;
    hipError_t e = hipMemcpyAsync(&word, workspace, sizeof word, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(ATTN_VARLEN_EHIP, "reading the workspace status failed: %s", hipGetErrorString(e));
    *status = word;
    return ATTN_VARLEN_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Low-precision forward: per-head E4M3 Q and K, 8-bit score product

namespace {

struct Fp8Layout {
    int64_t q8, k8, bytes;  // byte offsets in the workspace (amax words at 0)
};

int64_t round256(int64_t x) { return (x + 255) / 256 * 256; }

Fp8Layout fp8_layout(int64_t total_q, int64_t total_k, int32_t H, int32_t D) {
    Fp8Layout l;
    l.q8 = round256(8 * (int64_t)H);
    l.k8 = l.q8 + round256(total_q * H * D);
    l.bytes = l.k8 + round256(total_k * H * D);
    return l;
}

bool fp8_dim(int32_t D) { return D == 64 || D == 128; }

int32_t fp8_run(const void* q, const void* k, const void* v, const int32_t* cu_q, const int32_t* cu_k, int32_t B,
                int32_t H, int32_t D, const attn_varlen_layout* st, float scale, uint32_t flags, void* workspace,
                int64_t workspace_bytes, void* out, float* lse, hipStream_t s) {
    const Fp8Layout l = fp8_layout(cu_q[B], cu_k[B], H, D);
    if (workspace_bytes < l.bytes)
        return fail(ATTN_VARLEN_EINVAL, "workspace of %lld bytes is smaller than the %lld needed",
                    (long long)workspace_bytes, (long long)l.bytes);
    const int32_t rc = check_launch_limits(cu_q, B, H, fwd_block_m(D, FwdCfg::general));
    if (rc != ATTN_VARLEN_OK) return rc;
    char* ws = static_cast<char*>(workspace);
    AvfQuantArgs qa;
    qa.q = q; qa.k = k;
    qa.q_rows = cu_q[B]; qa.k_rows = cu_k[B];
    qa.q_row = st->q_row; qa.q_head = st->q_head; qa.k_row = st->k_row; qa.k_head = st->k_head;
    qa.num_heads = H; qa.head_dim = D;
    qa.amax = reinterpret_cast<uint32_t*>(ws);
    qa.q8 = reinterpret_cast<uint8_t*>(ws + l.q8);
    qa.k8 = reinterpret_cast<uint8_t*>(ws + l.k8);
    const hipError_t e = avf_fp8_quantize(qa, s);
    if (e != hipSuccess) return fail(ATTN_VARLEN_EHIP, "quantization launch failed: %s", hipGetErrorString(e));
    return run(q, k, v, cu_q, cu_k, B, H, D, st, scale, out, lse, s, flags, INT32_MAX, SegStrides{0, 0, 0, 0, 0},
               qa.q8, qa.k8,
               qa.amax);
}

int32_t fp8_check(int32_t D, const void* workspace) {
    if (!fp8_dim(D)) return fail(ATTN_VARLEN_EUNSUPPORTED, "head_dim %d not supported by the 8-bit path (64 or 128)", D);
    if (!workspace) return fail(ATTN_VARLEN_ENULL, "workspace must be non-NULL");
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(ATTN_VARLEN_EALIGN, "workspace must be 256-byte aligned");
    return ATTN_VARLEN_OK;
}

}  // namespace

extern "C" {

int64_t attn_varlen_fp8_workspace_bytes(int64_t total_q, int64_t total_k, int32_t H, int32_t D) {
    g_last_error.clear();
    if (total_q < 0 || total_k < 0 || H <= 0) return fail(ATTN_VARLEN_EINVAL, "bad sizes");
    if (!fp8_dim(D)) return fail(ATTN_VARLEN_EUNSUPPORTED, "head_dim %d not supported by the 8-bit path", D);
    return fp8_layout(total_q, total_k, H, D).bytes;
}

int32_t attn_varlen_fp8_workspace_offsets(int64_t total_q, int64_t total_k, int32_t H, int32_t D, int64_t* q8_offset,
                                          int64_t* k8_offset) {
    g_last_error.clear();
    if (!q8_offset || !k8_offset) return fail(ATTN_VARLEN_ENULL, "NULL argument");
    const int64_t b = attn_varlen_fp8_workspace_bytes(total_q, total_k, H, D);
    if (b < 0) return (int32_t)b;
    const Fp8Layout l = fp8_layout(total_q, total_k, H, D);
    *q8_offset = l.q8;
    *k8_offset = l.k8;
    return ATTN_VARLEN_OK;
}

int32_t attn_varlen_fwd_fp8_hostcu(const void* q, const void* k, const void* v, const int32_t* cu_q, const int32_t* cu_k,
                                   int32_t B, int32_t H, int32_t D, int32_t max_q, int32_t max_k,
                                   const attn_varlen_layout* st, float scale, uint32_t flags, void* workspace,
                                   int64_t workspace_bytes, void* out, float* lse, void* stream) {
    g_last_error.clear();
    int32_t rc = check_flags(flags);
    if (rc != ATTN_VARLEN_OK) return rc;
    rc = validate_all(q, k, v, cu_q, cu_k, B, H, D, max_q, max_k, st, scale, out, lse);
    if (rc != ATTN_VARLEN_OK || B == 0) return rc;
    if ((rc = fp8_check(D, workspace)) != ATTN_VARLEN_OK) return rc;
    return fp8_run(q, k, v, cu_q, cu_k, B, H, D, st, scale, flags, workspace, workspace_bytes, out, lse,
                   static_cast<hipStream_t>(stream));
}

int32_t attn_varlen_fwd_fp8(const void* q, const void* k, const void* v, const int32_t* cu_q_dev, const int32_t* cu_k_dev,
                            int32_t B, int32_t H, int32_t D, int32_t max_q, int32_t max_k, const attn_varlen_layout* st,
                            float scale, uint32_t flags, void* workspace, int64_t workspace_bytes, void* out, float* lse,
                            void* stream) {
    g_last_error.clear();
    int32_t rc = check_flags(flags);
    if (rc != ATTN_VARLEN_OK) return rc;
    rc = check_scalars(q, k, v, B, H, D, max_q, max_k, st, scale, out, lse);
    if (rc != ATTN_VARLEN_OK || B == 0) return rc;
    if ((rc = fp8_check(D, workspace)) != ATTN_VARLEN_OK) return rc;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    std::vector<int32_t> cu;
    if ((rc = read_cu(cu_q_dev, cu_k_dev, B, s, cu)) != ATTN_VARLEN_OK) return rc;
    const int32_t* cq = cu.data();
    const int32_t* ck = cu.data() + B + 1;
    rc = check_cu(cq, ck, B, max_q, max_k, st);
    if (rc != ATTN_VARLEN_OK) return rc;
    rc = check_with_cu(cq, B, H, D, st, lse);
    if (rc != ATTN_VARLEN_OK) return rc;
    return fp8_run(q, k, v, cq, ck, B, H, D, st, scale, flags, workspace, workspace_bytes, out, lse, s);
}

}  // extern "C"
