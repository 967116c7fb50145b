// Packed variable-length attention forward for gfx950 (MI355X, CDNA4).
//
// One workgroup computes one tile: BM query rows of one head of one segment,
// streaming that segment's K/V in stages of BN keys through rings of LDS
// buffers. K and V reach LDS by buffer loads that write LDS directly (no
// registers, no LDS store instructions), one stage ahead of the compute.
// Three configurations share this code (chosen on the host from max_seqlen_k):
// the general one (8 waves, BM = 256, 128-key stages, one workgroup per CU),
// and for short key segments, where the work is bound by memory latency
// rather than MFMA, 4-wave workgroups (BM = 128) that share a CU in pairs:
// one 128-key stage with one K and one V buffer (ONE, up to 128 keys) or
// 64-key stages in 80 KiB rings (up to 512 keys).
// The operation is the flash-attention varlen forward with its LSE
// (the (out, lse) return of flash_attn_varlen_func on the "[FA4] cute varlen
// backward: int32 overflow in _bwd_preprocess ..." page); the online softmax
// keeps a running row maximum m and sum l and rescales the accumulator when m
// grows, so the result equals softmax(scale * Q K^T) V exactly up to rounding.
//
// Matrix layout on the MFMA (v_mfma_f32_32x32x16_bf16, wave64):
//   S^T = K * Q^T:  A = 32 keys x 16 dims of K (from LDS, one 16-byte read per
//                   lane), B = Q^T (kept in registers for the whole tile; with
//                   64-key stages it arrives through LDS by whole-row loads).
//                   The 32x32 result puts ONE query row per lane pair
//                   (lane l and l+32, 16 keys each), so the row max needs one
//                   cross-half exchange and the row sum none until the end.
//   O^T += V^T P^T: A = 32 dims x 16 keys of V^T, B = P^T, which is the S^T
//                   result itself rounded to bf16 in place. V stays row-major
//                   in LDS; two transposing reads (ds_read_b64_tr_b16) per
//                   MFMA deliver V^T in exactly the key order of the S^T
//                   result, so P never leaves registers.
//   O^T accumulates with one query row per lane pair too, so the rescale by
//   exp2(m_old - m_new) is a per-lane scalar. At the end O goes through LDS,
//   so that every store instruction writes whole rows.
// Offsets: every tensor base is formed in int64 (row * row_stride + head *
// head_stride, as the "Suggested kernel-side fix" of the _bwd_preprocess page
// asks) and rebased per tile; the per-lane buffer offsets inside a tile are
// bounded by BM * row_stride bytes < 2^31, checked on the host. Buffer
// resources clip every load and store to the tile's valid rows, so a tail
// tile reads zeros past the segment instead of a neighbour's or unmapped memory.
// Validity: the grid is exactly the tile count, so every workgroup decodes to a
// real tile before it forms any address (the SM120 page's memcheck findings
// show the opposite order, prefetching from garbage coordinates).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "avf_device.h"
#include "avf_plan.h"

namespace {

using namespace avf;

// Largest per-lane partial row sum of softmax weights accepted before the
// reference max is moved (bounds every weight by 2^16).
constexpr float kPsumMax = 65536.0f;

// LDS rows of K and V are unpadded (2*D bytes); the 16-byte chunks of a row are
// permuted by XOR with a function of the key so that the MFMA fragment reads
// hit all 64 banks (256 bytes) of gfx950's LDS in every phase:
//  K (ds_read_b128: 16 lanes per phase, 16 consecutive keys, same chunk):
//    D = 128 (16 chunks/row): chunk ^= key % 16;
//    D = 64 (8 chunks, rows alternate bank halves): chunk ^= (key / 2) % 8;
//    D = 96 (12 chunks, 192 B rows cycle through 4 bank offsets): chunk ^= (key / 4) % 4.
//  V (ds_read_b64_tr_b16: 32 lanes per phase, 4 consecutive keys x 4 chunks):
//    D = 128: chunk ^= 4 * (key % 4); D = 64: chunk ^= 4 * ((key / 2) % 2);
//    D = 96: none needed (the 192-byte pitch already spreads the 4 rows).
// The XOR never leaves the row (it only flips low chunk-index bits).
template <int D>
__device__ constexpr int k_swz(int key) {
    return D == 128 ? key & 15 : D == 64 ? (key >> 1) & 7 : (key >> 2) & 3;
}
template <int D>
__device__ constexpr int v_swz(int key) {
    return D == 128 ? (key & 3) << 2 : D == 64 ? ((key >> 1) & 1) << 2 : 0;
}
// 8-bit K rows (D bytes; ds_read_b128, 16 consecutive keys per phase):
//   D = 128 (8 chunks, two rows per 256 bytes): chunk ^= (key / 2) % 8;
//   D = 64 (4 chunks, four rows per 256 bytes): chunk ^= (key / 4) % 4.
template <int D>
__device__ constexpr int k8_swz(int key) {
    return D == 128 ? (key >> 1) & 7 : (key >> 2) & 3;
}

// Device-plan tile decode: segment = the largest s with tile_start[s] <=
// linear (empty segments repeat their successor's start and are never
// chosen), found by a 64-way search. Each lane probes one prefix entry per
// step and a ballot picks the last probe at or below `linear`, so a step
// costs one global round trip and shrinks the candidates 64-fold (one step
// for up to 64 segments) where a binary search pays one round trip per
// halving. Every probe index stays below num_segs; every wave of the
// workgroup computes the same result.
__device__ inline AvfTile decode_wave(int32_t linear, const int32_t* tile_start, const int32_t* cu_q,
                                      int32_t num_segs, int32_t block_m, int lane) {
    int32_t lo = 0, n = num_segs;  // candidates [lo, lo + n); tile_start[lo] <= linear
    int32_t start = 0;             // tile_start[lo]
    for (;;) {
        const int32_t stride = n > 64 ? (n + 63) / 64 : 1;
        const int32_t off = lane * stride;
        const bool probe = off < n;
        const int32_t v = probe ? tile_start[lo + off] : INT32_MAX;
        const uint64_t below = __ballot(probe && v <= linear);  // bit 0 always set
        const int last = 63 - __clzll((long long)below);
        start = __shfl(v, last);
        lo += last * stride;
        if (stride == 1) break;
        n = min(stride, n - last * stride);
    }
    const int32_t lq = cu_q[lo + 1] - cu_q[lo];
    const int32_t mtiles = (lq + block_m - 1) / block_m;
    const int32_t r = linear - start;
    AvfTile t;
    t.seg = lo;
    t.head = r / mtiles;
    t.mblk = r - t.head * mtiles;
    return t;
}

// LDS holds a ring of KBUF K stages followed by a ring of VBUF V stages. V
// lives one stage longer than K because each wave's P.V product trails its
// Q.K^T product by one 32-key sub-block, across stage boundaries. ONE: every
// segment has at most BN keys, so a tile has one stage and one buffer each.
template <int D, int QB, int NW, int BN, bool F8 = false, bool ONE = false>
struct Tile {
    static constexpr int NT = NW * 64;          // threads per workgroup
    static constexpr int BM = QB * 32 * NW;     // query rows per tile
    static constexpr int KS = D / 16;           // MFMA k-steps over D
    static constexpr int DB = D / 32;           // 32-wide column blocks of O
    static constexpr int KB = BN / 32;          // 32-key sub-blocks per K/V stage
    static constexpr int ROWB = D * 2;          // bytes per K/V row in LDS
    static constexpr int SBYTES = BN * ROWB;    // one stage of K (or of V)
    static constexpr int KBUF = ONE ? 1 : 2, VBUF = ONE ? 1 : 3;
    // K stages hold bf16 rows, or with F8 the E4M3 codes (D bytes per row)
    static constexpr int KROWB = F8 ? D : 2 * D;
    static constexpr int KSBYTES = BN * KROWB;
    static constexpr int KQ = D / 64;           // F8: depth-64 Q.K^T MFMAs per sub-block
    static constexpr int NIK = KSBYTES / 1024;  // 1 KiB direct loads per K stage
    static constexpr int LDS_BYTES = KBUF * KSBYTES + VBUF * SBYTES;
    static constexpr int NI = SBYTES / 1024;    // 1 KiB direct loads per array and stage
    static_assert(D % 32 == 0 && BN % 32 == 0 && SBYTES % 1024 == 0, "tile shape");
    static_assert(KB >= 2 && KB % 2 == 0, "an even number of sub-blocks per stage (parity repeats every stage)");
    // Two sub-blocks per stage: the barrier sits at sub-block 0, where V of
    // the previous stage is still being read, so V stages load one stage
    // behind K (see `stage`).
    static constexpr bool VLAG = KB == 2;
    // Waves that issue the stage loads: with 8 waves only the first four
    // (one per SIMD, the older wave of each SIMD's pair; see load_stage).
    static constexpr int NL = NW == 8 ? NW / 2 : NW;
    static_assert(NI % NL == 0 && (!F8 || NIK % NL == 0), "every loading wave issues the same number of loads");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS rings");
    static_assert(!F8 || (D % 64 == 0 && NIK % NW == 0), "8-bit K stages: depth-64 steps, whole loads per wave");
};

// CAUSAL (compile-time): apply the causal mask. A separate instantiation, so
// the unmasked kernel carries none of its per-row limits or extra stage loop.
// DEVPLAN (compile-time): the tile plan was built on the device (no host
// read-back of cu_seqlens); the grid is a bound, every workgroup loops over
// tiles and leaves the loop at the plan's real tile count (below).
// F8 (compile-time): S^T = K Q^T from per-head E4M3 codes of q and k with the
// depth-64 8-bit MFMA (v_mfma_f32_32x32x64_f8f6f4); P.V stays bf16.
// ONE (compile-time): every segment of the call has at most BN keys (the host
// checked max_seqlen_k against cu_seqlens, or the device planner does): one
// K/V stage per tile, LDS for one stage only, so that two workgroups of NW
// waves share a CU and one's loads overlap the other's arithmetic.
template <int D, int QB, int NW, int BN, bool CAUSAL, bool DEVPLAN, bool F8, bool ONE>
__global__ void __launch_bounds__(NW * 64, 8 / NW) avf_fwd_kernel(const AvfLaunchArgs a) {
    using T = Tile<D, QB, NW, BN, F8, ONE>;
    constexpr int BM = T::BM;
    __shared__ __attribute__((aligned(16))) char lds[T::LDS_BYTES];
    // LDS byte address of the array (M0 operand of the direct loads)
    const uint32_t lds_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;

    const int tid = threadIdx.x;
    int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int l32 = lane & 31;
    int hf = lane >> 5;

    // One tile: query block tile_mblk (in dispatch order) of head h of the
    // launch's segment seg, whose query rows are [qs0, qs1) and key rows
    // [ks0, ks1) of the packed tensors.
    auto run_tile = [&](const int32_t seg, const int32_t tile_mblk, const int32_t h, const int32_t qs0,
                        const int32_t qs1, const int32_t ks0, const int32_t ks1) {
    const int32_t lq = qs1 - qs0;
    const int32_t lk = ks1 - ks0;
    // a one-stage tile has LDS for BN keys only (never reached: the host and
    // the device planner reject longer segments before choosing it)
    if (ONE && lk > BN) return;
    // Causal: later query blocks see more keys, so they are dispatched first
    // (the block order within a (segment, head) is reversed).
    const int32_t mblk = CAUSAL ? (lq + BM - 1) / BM - 1 - tile_mblk : tile_mblk;
    const int32_t row0 = mblk * BM;
    const int32_t rows_here = min(BM, lq - row0);
    const int64_t q_tok0 = (int64_t)qs0 + row0;
    const int64_t k_tok0 = (int64_t)ks0;
    const int64_t gseg = (int64_t)a.seg0 + seg;  // batched tensors: per-segment base offsets
    // Keys the tile needs: all of the segment, or with the causal mask (row r
    // sees keys j <= r + lk - lq) those up to its last row's limit. Keys below
    // kfull are visible to every row of the tile, so only stages from
    // kfull / BN on need the per-row mask.
    const int32_t coff = lk - lq;
    const int32_t k_end = CAUSAL ? max(0, min(lk, row0 + rows_here + coff)) : lk;
    const int32_t kfull = CAUSAL ? max(0, min(k_end, row0 + 1 + coff)) : k_end;

    // ---- Q^T fragments (B operand), resident for the whole tile ----
    const uint32_t q_rs = (uint32_t)(a.q_row * 2);
    const char* qptr = (const char*)a.q + 2 * (avf_elem_offset(q_tok0, a.q_row, h, a.q_head) + gseg * a.q_seg);
    const auto qrs = make_rsrc(qptr, (uint32_t)(rows_here - 1) * q_rs + 2 * D);
    const int wrow0 = wave * QB * 32;
    // A lane's Q fragments are 16-byte pieces of one row, so loading them
    // straight into registers makes every load instruction touch 32 rows a
    // token stride apart. With 64-key stages (short segments, a few stages
    // per tile) the tile's Q rows instead arrive by whole-row direct loads
    // into V buffers 1 and 2, which hold nothing until stage 0's barrier,
    // and the fragments are read from there (QLDS); rows past the tile read 0.
    constexpr bool QLDS = T::VLAG && !F8;
    constexpr int QOFF = T::KBUF * T::KSBYTES + T::SBYTES;
    static_assert(!QLDS || (QB == 1 && BM * 2 * D <= 2 * T::SBYTES && (BM * 2 * D / 1024) % NW == 0),
                  "Q rows fit V buffers 1 and 2");
    auto load_q_lds = [&]() {
        const i32x4 qw = rsrc_words(qptr, (uint32_t)(rows_here - 1) * q_rs + 2 * D);
#pragma unroll
        for (int m = 0; m < BM * 2 * D / 1024 / NW; ++m) {
            const int i = wave + NW * m;
            const int pos = i * 1024 + 16 * lane;
            const int r = pos / (2 * D);
            const int slot = (pos % (2 * D)) >> 4;
            load_lds16(qw, lds_addr + QOFF + i * 1024, (uint32_t)r * q_rs + ((slot ^ k_swz<D>(r)) << 4));
        }
    };
    bf16x8 qf[QB][F8 ? 1 : T::KS];
    i32x8 qf8[QB][F8 ? T::KQ : 1];  // F8: lane holds dims 64t + 32*hf .. +32 of its row
    if constexpr (F8) {
        const uint32_t q8_rs = (uint32_t)(a.num_heads * D);
        const uint8_t* q8p = a.q8 + (q_tok0 * a.num_heads + h) * D;
        const auto q8rs = make_rsrc(q8p, (uint32_t)(rows_here - 1) * q8_rs + D);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int t = 0; t < T::KQ; ++t) {
                const uint32_t off = (uint32_t)(wrow0 + qb * 32 + l32) * q8_rs + 64 * t + 32 * hf;
                const i32x4 lo = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(q8rs, off, 0, 0));
                const i32x4 hi = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(q8rs, off + 16, 0, 0));
                qf8[qb][t] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
    } else if constexpr (!QLDS) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int ks = 0; ks < T::KS; ++ks) {
                const uint32_t off = (uint32_t)(wrow0 + qb * 32 + l32) * q_rs + (ks * 16 + hf * 8) * 2;
                qf[qb][ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0));
            }
    }

    f32x16 o[QB][T::DB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int db = 0; db < T::DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[qb][db][e] = 0.f;
    // m_i: the row's softmax reference (a row maximum of the raw scores seen
    // at some block, -inf before the first); mc_i = m_i * c; l_i: this lane's
    // partial row sum of weights against that reference.
    float m_i[QB], mc_i[QB], l_i[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_i[qb] = -INFINITY;
        mc_i[qb] = -INFINITY;
        l_i[qb] = 0.f;
    }
    float c = a.scale_log2e;  // weights are exp2(c * (s - m))
    float lse_scale = a.scale;
    if constexpr (F8) {
        // s is the product of codes: true scores are s * (amax_q/448) * (amax_k/448)
        const float aq = __uint_as_float(a.amax8[h]);
        const float ak = __uint_as_float(a.amax8[a.num_heads + h]);
        const float sqk = (aq > 0.f ? aq / 448.f : 1.f) * (ak > 0.f ? ak / 448.f : 1.f);
        c *= sqk;
        lse_scale *= sqk;
    }

    // ---- K/V staging: buffer loads straight into LDS ----
    // Stage j covers keys [j*BN, j*BN + BN) of the segment. Each wave issues
    // 1 KiB loads; lane l of load i fills LDS bytes [i*1024 + 16*l, +16), which
    // is chunk `slot` of row `key` of the stage, so it fetches chunk
    // slot ^ swz(key) of that key's row. Rows past the segment end re-read its
    // last row (finite data; they are masked out of the softmax).
    const int32_t nkt = (k_end + BN - 1) / BN;
    const int32_t jmask = kfull / BN;  // first stage that needs the per-row causal mask
    const uint32_t k_rs = (uint32_t)(a.k_row * 2);
    const uint32_t v_rs = (uint32_t)(a.v_row * 2);
    auto load_stage = [&](int32_t j, int kbuf, int vbuf, bool do_k = true, bool do_v = true) {
        const int32_t key0 = j * BN;
        const int32_t nk = min(BN, k_end - key0);
        const char* kp = (const char*)a.k + 2 * (avf_elem_offset(k_tok0 + key0, a.k_row, h, a.k_head) + gseg * a.k_seg);
        const char* vp = (const char*)a.v + 2 * (avf_elem_offset(k_tok0 + key0, a.v_row, h, a.v_head) + gseg * a.v_seg);
        const i32x4 vrs = rsrc_words(vp, (uint32_t)(nk - 1) * v_rs + 2 * D);
        const uint32_t kl = lds_addr + kbuf * T::KSBYTES;
        const uint32_t vl = lds_addr + T::KBUF * T::KSBYTES + vbuf * T::SBYTES;
        // Only waves 0 .. NL-1 issue loads. The two waves of a SIMD do the
        // same MFMA and softmax work per stage, and the older one wins
        // every tie for the MFMA pipe, reaches the stage barrier first and
        // waits there; giving it all of the pair's load issue (addresses,
        // M0, the buffer loads) shortens the partner's path to the barrier:
        // +2.8% on dense_77k, +2.3% on strided_9728, +3% on varlen_cross
        // against all eight waves loading (the younger four loading: +0.5-1.3%).
        if (wave >= T::NL) return;
        if constexpr (F8) {
            const uint32_t k8_rs = (uint32_t)(a.num_heads * D);
            const uint8_t* k8p = a.k8 + ((k_tok0 + key0) * a.num_heads + h) * D;
            const i32x4 k8rs = rsrc_words(k8p, (uint32_t)(nk - 1) * k8_rs + D);
#pragma unroll
            for (int m = 0; m < T::NIK / T::NL; ++m) {
                const int i = wave + T::NL * m;
                const int pos = i * 1024 + 16 * lane;
                const int key = pos / T::KROWB;
                const int slot = (pos % T::KROWB) >> 4;
                const uint32_t kc = (uint32_t)min(key, nk - 1);
                load_lds16(k8rs, kl + i * 1024, kc * k8_rs + ((slot ^ k8_swz<D>(key)) << 4));
            }
#pragma unroll
            for (int m = 0; m < T::NI / T::NL; ++m) {
                const int i = wave + T::NL * m;
                const int pos = i * 1024 + 16 * lane;
                const int key = pos / T::ROWB;
                const int slot = (pos % T::ROWB) >> 4;
                const uint32_t kc = (uint32_t)min(key, nk - 1);
                load_lds16(vrs, vl + i * 1024, kc * v_rs + ((slot ^ v_swz<D>(key)) << 4));
            }
            return;
        }
        const i32x4 krs = rsrc_words(kp, (uint32_t)(nk - 1) * k_rs + 2 * D);
        // A full stage at D = 64 or 128: load m of a lane fetches key
        // key0 + m * KSTEP at the same chunk slot, and both swizzles depend on
        // the key only modulo KSTEP, so one lane offset per array serves every
        // load and the per-load step goes into the wave-uniform soffset.
        constexpr int KSTEP = T::NL * 1024 / T::ROWB;
        constexpr bool AFFINE = 1024 % T::ROWB == 0 && KSTEP % 16 == 0;
        if (AFFINE && nk == BN) {
            const int key0 = (wave * 1024 + 16 * lane) / T::ROWB;
            const int slot = ((16 * lane) % T::ROWB) >> 4;
            const uint32_t ko = (uint32_t)key0 * k_rs + ((slot ^ k_swz<D>(key0)) << 4);
            const uint32_t vo = (uint32_t)key0 * v_rs + ((slot ^ v_swz<D>(key0)) << 4);
#pragma unroll
            for (int m = 0; m < T::NI / T::NL; ++m) {
                const int i = wave + T::NL * m;
                if (do_k) load_lds16_so(krs, kl + i * 1024, ko, (uint32_t)(m * KSTEP) * k_rs);
                if (do_v) load_lds16_so(vrs, vl + i * 1024, vo, (uint32_t)(m * KSTEP) * v_rs);
            }
            return;
        }
#pragma unroll
        for (int m = 0; m < T::NI / T::NL; ++m) {
            const int i = wave + T::NL * m;
            const int pos = i * 1024 + 16 * lane;
            const int key = pos / T::ROWB;
            const int slot = (pos % T::ROWB) >> 4;
            const uint32_t kc = (uint32_t)min(key, nk - 1);
            if (do_k) load_lds16(krs, kl + i * 1024, kc * k_rs + ((slot ^ k_swz<D>(key)) << 4));
            if (do_v) load_lds16(vrs, vl + i * 1024, kc * v_rs + ((slot ^ v_swz<D>(key)) << 4));
        }
    };

    // ---- per-sub-block steps (32 keys each) ----
    // MFMA A-operand fragments from LDS: K rows (32 keys x 16 dims per MFMA)
    // and V^T rows (32 dims x 16 keys per MFMA).
    // K: lane reads chunk (2*ks + hf) of key sub*32 + l32 (16 bytes). The
    // swizzle depends on the key only modulo 32, so within a buffer the
    // per-lane byte offsets are fixed; kcur holds them for K buffer 0, and a
    // read adds the buffer's and the sub-block's offsets. In the stages of
    // the hot loop the buffer is known at compile time (the loop runs them in
    // pairs), so every fragment read there is one LDS instruction with an
    // immediate offset.
    constexpr int SUB = 32 * T::ROWB;    // bytes per 32-key sub-block of V (and of bf16 K)
    constexpr int SUBK = 32 * T::KROWB;  // ... of K
    // F8: depth-64 fragment t of the lane is chunks 4t + 2*hf and 4t + 2*hf + 1
    // of its key's row (kcur[2t], kcur[2t + 1])
    constexpr int NKC = F8 ? 2 * T::KQ : T::KS;
    int kcur[NKC];
#pragma unroll
    for (int u = 0; u < NKC; ++u) {
        if constexpr (F8)
            kcur[u] = l32 * T::KROWB + (((4 * (u >> 1) + 2 * hf + (u & 1)) ^ k8_swz<D>(l32)) << 4);
        else
            kcur[u] = l32 * T::ROWB + (((2 * u + hf) ^ k_swz<D>(l32)) << 4);
    }
    // V^T fragment for keys [kb*32 + 16*k2, +16) and dims [db*32, +32): two
    // transposing 8-byte reads. In each 16-lane group, lane j receives element
    // j%4 of the 8-byte rows read by lanes 4t + j/4 (t = 0..3); reading key
    // kb*32 + 16*k2 + 8*r + 4*hf + (lane/4)%4 at dims db*32 + 16*((lane/16)%2)
    // + 4*(lane%4) therefore hands lane l the dims l%32 of the keys that its
    // P operand slots 4r..4r+3 hold.
    const int vkey = 4 * hf + ((lane >> 2) & 3);        // key offset within 8 (per lane)
    const int vdim = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    // The V swizzle depends on the key only modulo 8: fixed per-lane offsets
    // within a buffer; vcur holds them for the V buffer being read now (the
    // V ring starts after the K ring) and moves once per stage.
    int vcur[T::DB];
#pragma unroll
    for (int db = 0; db < T::DB; ++db) {
        const int d = db * 32 + vdim;
        vcur[db] = T::KBUF * T::KSBYTES + vkey * T::ROWB + (((d >> 3) ^ v_swz<D>(vkey)) << 4) + (d & 4) * 2;
    }
    // S^T for 32 keys x (QB*32) query rows
    auto qk = [&](const bf16x8 (&ka)[T::KS], f32x16 (&sc)[QB]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int e = 0; e < 16; ++e) sc[qb][e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                sc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qf[qb][ks], sc[qb], 0, 0, 0);
    };
    // keys of the stage at or past the lane's limit lim[qb] (the segment or
    // tile end, or the row's causal limit) get -inf; element e of a lane
    // holds key kb*32 + 8*(e/4) + 4*hf + e%4 of the stage
    auto mask = [&](int kb, const int32_t (&lim)[QB], f32x16 (&sc)[QB]) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int key = kb * 32 + 8 * (e >> 2) + 4 * hf + (e & 3);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) sc[qb][e] = key >= lim[qb] ? -INFINITY : sc[qb][e];
        }
    };
    // Online softmax against a lazily moved reference m_i: the weights are
    // p = exp2(c*s - c*m_i). Every p is bounded by its lane's partial row sum,
    // so while each lane's sum stays <= kPsumMax nothing can overflow and the
    // reference may stay where it is. Otherwise (the first block, m_i = -inf;
    // or a row max that grew by more than log2(kPsumMax) base-2 units) the wave
    // takes this block's row maximum, moves m_i up to it, rescales O and l by
    // exp2(c*(m_old - m_new)) and recomputes p (fix_reference). Same softmax;
    // the common path has neither a max reduction nor an accumulator rescale.
    auto weights = [&](const f32x16 (&sc)[QB], bf16x8 (&pk)[QB][2], float (&psum)[QB]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[qb][e], c, -mc_i[qb]));
                if (e & 1)
                    acc1 += p;
                else
                    acc0 += p;
                pk[qb][e >> 3][e & 7] = (__bf16)p;
            }
            psum[qb] = acc0 + acc1;
        }
    };
    auto over_limit = [&](const float (&psum)[QB]) {
        bool over = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) over |= !(psum[qb] <= kPsumMax);  // NaN counts as over
        return __builtin_amdgcn_ballot_w64(over) != 0;
    };
    auto fix_reference = [&](const f32x16 (&sc)[QB], bf16x8 (&pk)[QB][2], float (&psum)[QB]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float v = sc[qb][0];
#pragma unroll
            for (int e = 1; e < 16; ++e) v = fmaxf(v, sc[qb][e]);
            const float mnew = fmaxf(m_i[qb], fmaxf(v, __shfl_xor(v, 32)));
            // a row that has seen no key yet (every score -inf, causal rows
            // above the diagonal) keeps m = -inf, l = 0, O = 0 and gets
            // weights exp2(-inf) = 0 from the finite offset 0
            const bool none = CAUSAL && mnew == -INFINITY;
            const float alpha = none ? 1.f : __builtin_amdgcn_exp2f((m_i[qb] - mnew) * c);
            l_i[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < T::DB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) o[qb][db][e] *= alpha;
            m_i[qb] = mnew;
            mc_i[qb] = none ? 0.f : mnew * c;
        }
        weights(sc, pk, psum);
    };
    // O^T += V^T P^T over 32 keys: two 16-key MFMA steps per column block
    auto pv = [&](const bf16x8 (&va)[2][T::DB], const bf16x8 (&pk)[QB][2]) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
            for (int db = 0; db < T::DB; ++db)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[k2][db], pk[qb][k2], o[qb][db], 0, 0, 0);
    };

    // Software pipeline inside the wave, continuous over the whole key
    // sequence. Iteration g (32-key sub-block g) issues the MFMAs of Q.K^T for
    // sub-block g+1 and of P.V for sub-block g-1 while its VALU work is the
    // softmax of sub-block g, whose scores Q.K^T(g) finished during iteration
    // g-1; so neither product waits for the softmax and the softmax never
    // waits for a product. The iteration is written slot by slot with a
    // scheduling fence between slots: slot t issues one MFMA and a share of
    // the softmax, so every MFMA has independent VALU work behind it and the
    // MFMA pipe, shared by the SIMD's waves, stays fed.
    // Fragments rotate through one set of KS registers (Q.K^T and P.V both
    // take KS = D/16 MFMAs per sub-block): slot t < KS consumes K fragment t
    // and refills its register with the V^T fragment that slot t + KS
    // consumes; slot KS + u consumes that V^T fragment and refills the
    // register with K fragment u of the next iteration. Every LDS read thus
    // has KS slots to land. At D = 64 and 96 the general configuration has
    // registers to spare (SPLIT): K and V^T fragments then have a set each,
    // slot t refills K fragment t for the next iteration and slot KS + u the
    // V^T fragment u of sub-block g (multiplied in the next iteration), so
    // every read has a whole iteration to land.
    // The rare reference move (fix_reference) rescales O after the P.V(g-1)
    // MFMAs, so O then holds all earlier sub-blocks against the old reference.
    //
    // Staging: stage j (BN keys) sits in K buffer j % 2 and V buffer j % 3.
    // The one barrier per stage is at the top of its sub-block KB-2, the
    // first iteration that reads K fragments of stage j+1: there each wave
    // first waits for its share of stage j+1 (loaded one stage earlier), and
    // after it every wave is past its last read of K stage j (during
    // sub-block KB-3) and of V stage j-1 (during sub-block 0 of stage j), so
    // stage j+2 is loaded into exactly those two buffers.
    f32x16 sc[2][QB];      // scores of sub-blocks with even / odd index
    bf16x8 pk[2][QB][2];   // their weights as bf16 P^T operands
    bf16x8 fr[F8 ? 1 : T::KS];      // rotating K / V^T fragment registers
    i32x8 kf8[F8 ? T::KQ : 1];      // F8: K fragments (refilled one iteration ahead)
    constexpr bool SPLIT = !F8 && !ONE && !T::VLAG && D < 128;
    bf16x8 vfr[(F8 || SPLIT) ? T::KS : 1];  // F8, SPLIT: V^T fragments (refilled one iteration ahead)
    // K fragment u of sub-block `sub` of the K buffer at byte offset kbo
    auto read_k = [&](int kbo, int sub, int u) {
        return *reinterpret_cast<const bf16x8*>(lds + kcur[u] + kbo + sub * SUB);
    };
    // F8: depth-64 K fragment t of sub-block `sub`
    auto read_k8 = [&](int kbo, int sub, int t) {
        const i32x4 lo = *reinterpret_cast<const i32x4*>(lds + kcur[2 * t] + kbo + sub * SUBK);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(lds + kcur[2 * t + 1] + kbo + sub * SUBK);
        return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    auto mfma8 = [](const i32x8& ka, const i32x8& qa, const f32x16& acc) {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qa, acc, 0, 0, 0, 0, 0, 0);
    };
    // V^T fragment u = k2 * DB + db of sub-block `sub` of the V buffer being read
    auto read_v = [&](int sub, int u) {
        const int k2 = u / T::DB, db = u % T::DB;
        const char* p = lds + vcur[db] + sub * SUB + k2 * 16 * T::ROWB;
        return read_tr8(p, p + 8 * T::ROWB);
    };
    // vsub: V sub-block g-1 (SPLIT: g); ksub: K sub-block g+2 (refill_k false
    // when there is none), each in the buffer its address set points at
    auto iterate = [&](const f32x16 (&sv)[QB], f32x16 (&snext)[QB], bool do_qk, const bf16x8 (&pprev)[QB][2],
                       bf16x8 (&pcur)[QB][2], float (&psum)[QB], int vsub, int kbo, int ksub, bool refill_k) {
        constexpr int NSLOT = 2 * T::KS;
        // Softmax element e (of the lane's 16 scores) belongs to slot
        // e * (NSLOT - 2) / 16; its three dependent steps run one slot apart:
        // the scaled exponent in its slot, exp2 in the next, the row-sum add
        // (and the bf16 packing of an element pair) in the one after. No VALU
        // instruction then waits on a result of its own slot, and the last
        // element's add lands in the last MFMA slot, so the iteration ends
        // without VALU-only slots (with two such slots it measured 0.2% slower).
        float x[QB][16], pw[QB][16], acc[QB][2];
#pragma unroll
        for (int t = 0; t < NSLOT; ++t) {
            if (t < T::KS) {
                if (do_qk) {
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) {
                        const f32x16 zero = {};
                        snext[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[t], qf[qb][t], t == 0 ? zero : snext[qb],
                                                                            0, 0, 0);
                    }
                }
                if constexpr (SPLIT) {
                    if (refill_k) fr[t] = read_k(kbo, ksub, t);
                } else {
                    fr[t] = read_v(vsub, t);
                }
            } else if (t < NSLOT) {
                const int u = t - T::KS, k2 = u / T::DB, db = u % T::DB;
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(SPLIT ? vfr[u] : fr[u], pprev[qb][k2],
                                                                        o[qb][db], 0, 0, 0);
                if constexpr (SPLIT)
                    vfr[u] = read_v(vsub, u);
                else if (refill_k)
                    fr[u] = read_k(kbo, ksub, u);
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int te = e * (NSLOT - 2) / 16;
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    if (t == te) {
                        x[qb][e] = __builtin_fmaf(sv[qb][e], c, -mc_i[qb]);
                        pin(x[qb][e]);
                    } else if (t == te + 1) {
                        pw[qb][e] = __builtin_amdgcn_exp2f(x[qb][e]);
                        pin(pw[qb][e]);
                    } else if (t == te + 2) {
                        // elements 0 and 1 open the two partial sums with
                        // elements 2 and 3 (no copy into the accumulator)
                        if (e >= 2) {
                            acc[qb][e & 1] = (e < 4 ? pw[qb][e - 2] : acc[qb][e & 1]) + pw[qb][e];
                            pin(acc[qb][e & 1]);
                        }
                        if (e & 1) {
                            bf16x2 w = {(__bf16)pw[qb][e - 1], (__bf16)pw[qb][e]};
                            pin(w);
                            pcur[qb][e >> 3][(e & 7) - 1] = w[0];
                            pcur[qb][e >> 3][e & 7] = w[1];
                        }
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) psum[qb] = acc[qb][0] + acc[qb][1];
    };

    // F8 iteration g: KQ slots of 8-bit Q.K^T(g+1) (each refills its K
    // fragment with sub-block g+2), then KS slots of bf16 P.V(g-1) (each
    // refills its V^T fragment with sub-block g, which iteration g+1
    // multiplies); the softmax of sub-block g spreads over all KQ + KS slots
    // as in `iterate`. vsub: sub-block g in the current V buffer.
    auto iterate8 = [&](const f32x16 (&sv)[QB], f32x16 (&snext)[QB], bool do_qk, const bf16x8 (&pprev)[QB][2],
                        bf16x8 (&pcur)[QB][2], float (&psum)[QB], int vsub, int kbo, int ksub, bool refill_k) {
        constexpr int NSLOT = T::KQ + T::KS;
        float x[QB][16], pw[QB][16], acc[QB][2];
#pragma unroll
        for (int t = 0; t < NSLOT + 2; ++t) {
            if (t < T::KQ) {
                if (do_qk) {
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) {
                        const f32x16 zero = {};
                        snext[qb] = mfma8(kf8[t], qf8[qb][t], t == 0 ? zero : snext[qb]);
                    }
                }
                if (refill_k) kf8[t] = read_k8(kbo, ksub, t);
            } else if (t < NSLOT) {
                const int u = t - T::KQ, k2 = u / T::DB, db = u % T::DB;
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[u], pprev[qb][k2], o[qb][db], 0, 0, 0);
                vfr[u] = read_v(vsub, u);
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int te = e * NSLOT / 16;
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    if (t == te) {
                        x[qb][e] = __builtin_fmaf(sv[qb][e], c, -mc_i[qb]);
                        pin(x[qb][e]);
                    } else if (t == te + 1) {
                        pw[qb][e] = __builtin_amdgcn_exp2f(x[qb][e]);
                        pin(pw[qb][e]);
                    } else if (t == te + 2) {
                        // elements 0 and 1 open the two partial sums with
                        // elements 2 and 3 (no copy into the accumulator)
                        if (e >= 2) {
                            acc[qb][e & 1] = (e < 4 ? pw[qb][e - 2] : acc[qb][e & 1]) + pw[qb][e];
                            pin(acc[qb][e & 1]);
                        }
                        if (e & 1) {
                            bf16x2 w = {(__bf16)pw[qb][e - 1], (__bf16)pw[qb][e]};
                            pin(w);
                            pcur[qb][e >> 3][(e & 7) - 1] = w[0];
                            pcur[qb][e >> 3][e & 7] = w[1];
                        }
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) psum[qb] = acc[qb][0] + acc[qb][1];
    };

    // `last` (compile-time) marks the segment's final stage: keys past the
    // segment end are masked and there is no next stage. kp is stage j's K
    // buffer, a compile-time constant in the hot loop; vnext is the V buffer
    // stage j+2 is loaded into. K reads of sub-blocks of stage j+1 (from the
    // barrier on) use the other K buffer; at sub-block 1 the V reads move
    // from stage j-1's buffer to stage j's (vcur += vdelta).
    // `masked` (compile-time) applies the per-row key limit: the last stage
    // (segment or tile end) and, with the causal mask, the stages that cross
    // the tile's diagonal.
    auto stage = [&](int32_t j, auto kp, int vnext, int vdelta, auto last, auto masked) {
        const int kbuf = kp;
        constexpr bool LAST = decltype(last)::value;
        constexpr bool MASKED = decltype(masked)::value || LAST;
        int32_t lim[QB];
        if (MASKED) {
            const int32_t key0 = j * BN;
            const int32_t nk = LAST ? k_end - key0 : BN;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                lim[qb] = CAUSAL ? min(nk, row0 + wrow0 + qb * 32 + l32 + coff + 1 - key0) : nk;
        }
#pragma unroll
        for (int kb = 0; kb < T::KB; ++kb) {
            // With two sub-blocks per stage (VLAG) the barrier is at sub-block
            // 0, where V of stage j-1 is still read, so V stage j+1 (not j+2)
            // is loaded there into the third V buffer; the last stage then
            // needs its barrier too, to see its own V.
            if (kb == T::KB - 2 && (!LAST || T::VLAG)) {
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
                __syncthreads();
                if (!LAST) {
                    if constexpr (T::VLAG) {
                        if (j + 2 < nkt) load_stage(j + 2, kbuf, 0, true, false);
                        load_stage(j + 1, 0, (j + 1) % 3, false, true);
                    } else {
                        if (j + 2 < nkt) load_stage(j + 2, kbuf, vnext);
                    }
                }
            }
            // V reads move to stage j's buffer where they first read it: at
            // sub-block 1 (P.V(g-1) reads V of sub-block g-1), with F8 and
            // SPLIT at sub-block 0 (fragments of sub-block g are read ahead)
            if (kb == ((F8 || SPLIT) ? 0 : 1)) {
#pragma unroll
                for (int db = 0; db < T::DB; ++db) vcur[db] += vdelta;
            }
            if (MASKED) mask(kb, lim, sc[kb & 1]);
            float psum[QB];
            // sub-block g-1 has the other parity
            // K sub-block g+2 lies in this stage's buffer or in the next one's
            const int kbo = (T::KBUF == 1 || kb + 2 < T::KB ? kbuf : kbuf ^ 1) * T::KSBYTES;
            if constexpr (F8)
                iterate8(sc[kb & 1], sc[(kb + 1) & 1], !(LAST && kb == T::KB - 1), pk[(kb + 1) & 1], pk[kb & 1], psum,
                         kb, kbo, (kb + 2) % T::KB, kb + 2 < T::KB || !LAST);
            else
                iterate(sc[kb & 1], sc[(kb + 1) & 1], !(LAST && kb == T::KB - 1), pk[(kb + 1) & 1], pk[kb & 1], psum,
                        SPLIT ? kb : (kb > 0 ? kb - 1 : T::KB - 1), kbo, (kb + 2) % T::KB, kb + 2 < T::KB || !LAST);
            if (over_limit(psum)) fix_reference(sc[kb & 1], pk[kb & 1], psum);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) l_i[qb] += psum[qb];
        }
        if (LAST) {
            // P.V of the segment's final sub-block (F8, SPLIT: its V^T fragments are in vfr)
            if constexpr (F8 || SPLIT) {
#pragma unroll
                for (int u = 0; u < T::KS; ++u)
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
                        o[qb][u % T::DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            vfr[u], pk[(T::KB - 1) & 1][qb][u / T::DB], o[qb][u % T::DB], 0, 0, 0);
            } else {
#pragma unroll
                for (int u = 0; u < T::KS; ++u) fr[u] = read_v(T::KB - 1, u);
#pragma unroll
                for (int u = 0; u < T::KS; ++u)
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
                        o[qb][u % T::DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            fr[u], pk[(T::KB - 1) & 1][qb][u / T::DB], o[qb][u % T::DB], 0, 0, 0);
            }
        }
    };

    if (nkt > 0) {
        if constexpr (QLDS) load_q_lds();
        load_stage(0, 0, 0);
        if (!ONE && nkt > 1) load_stage(1, 1, 1, true, !T::VLAG);
        // Wait for everything issued so far (Q fragments and the first two
        // stages), once per tile: the compiler does not see the stage loads,
        // so only a full vmcnt(0) tells it that the Q fragments have landed;
        // otherwise it would hold the loop's MFMAs on in-flight stage loads.
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __syncthreads();
        // QLDS: the wave's Q fragments (row wrow0 + l32, chunk 2ks + hf, with
        // the K swizzle); read before stage 0's barrier reloads V buffer 1
        if constexpr (QLDS) {
#pragma unroll
            for (int ks = 0; ks < T::KS; ++ks)
                qf[0][ks] = *reinterpret_cast<const bf16x8*>(lds + QOFF + (wrow0 + l32) * 2 * D +
                                                             (((2 * ks + hf) ^ k_swz<D>(l32)) << 4));
        }
        // S(0), then the K fragments of sub-block 1 for the first iteration
        if constexpr (F8) {
#pragma unroll
            for (int t = 0; t < T::KQ; ++t) kf8[t] = read_k8(0, 0, t);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const f32x16 zero = {};
#pragma unroll
                for (int t = 0; t < T::KQ; ++t) sc[0][qb] = mfma8(kf8[t], qf8[qb][t], t == 0 ? zero : sc[0][qb]);
            }
#pragma unroll
            for (int t = 0; t < T::KQ; ++t) kf8[t] = read_k8(0, 1, t);
            // finite V rows for the zero-weight P.V of sub-block -1
#pragma unroll
            for (int u = 0; u < T::KS; ++u) vfr[u] = read_v(0, u);
        } else {
#pragma unroll
            for (int u = 0; u < T::KS; ++u) fr[u] = read_k(0, 0, u);
            qk(fr, sc[0]);
#pragma unroll
            for (int u = 0; u < T::KS; ++u) fr[u] = read_k(0, 1, u);
            // SPLIT: finite V rows for the zero-weight P.V of sub-block -1
            if constexpr (SPLIT) {
#pragma unroll
                for (int u = 0; u < T::KS; ++u) vfr[u] = read_v(0, u);
            }
        }
        // Sub-block 0 has no predecessor: its P.V slots multiply zero
        // weights with loaded (finite) V rows instead, which keeps one
        // branch-free body for every stage.
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pk[1][qb][0][e] = (__bf16)0.f;
                pk[1][qb][1][e] = (__bf16)0.f;
            }
        // buffers of stage j: K j % 2, V j % 3; stage j-1's V (stage 0: its
        // own) and stage j+2's target (j+2) % 3
        int kbuf = 0, vbuf = 0, vprev = 0, vnext = 2;
        auto advance = [&]() {
            kbuf ^= 1;
            vprev = vnext = vbuf;
            vbuf = vbuf == 2 ? 0 : vbuf + 1;
        };
        // stages every row sees whole (in pairs, so that each one's K buffer
        // is a compile-time constant), then the ones crossing the causal
        // diagonal, then the last
        const int32_t nfree = ONE ? 0 : min(jmask, nkt - 1);
        int32_t j = 0;
        using K0 = std::integral_constant<int, 0>;
        using K1 = std::integral_constant<int, 1>;
        // A wave none of whose rows lie in the segment (the last query block
        // of a segment can hold a few rows only) skips the arithmetic and
        // keeps the stages' barriers and its share of the loads, so its SIMD
        // partner runs alone on the MFMA pipe. Nothing of it is stored.
        if (wrow0 >= rows_here) {
            for (; j < nkt; ++j) {
                if (j + 1 < nkt || T::VLAG) {
                    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
                    __syncthreads();
                    if (j + 1 < nkt) {
                        if constexpr (T::VLAG) {
                            if (j + 2 < nkt) load_stage(j + 2, j & 1, 0, true, false);
                            load_stage(j + 1, 0, (j + 1) % 3, false, true);
                        } else {
                            if (j + 2 < nkt) load_stage(j + 2, j & 1, (j + 2) % 3);
                        }
                    }
                }
            }
        } else {
            for (; j + 1 < nfree; j += 2) {
                stage(j, K0{}, vnext, (vbuf - vprev) * T::SBYTES, std::false_type{}, std::false_type{});
                advance();
                stage(j + 1, K1{}, vnext, (vbuf - vprev) * T::SBYTES, std::false_type{}, std::false_type{});
                advance();
            }
            if (j < nfree) {
                stage(j, K0{}, vnext, (vbuf - vprev) * T::SBYTES, std::false_type{}, std::false_type{});
                advance();
                ++j;
            }
            if constexpr (CAUSAL && !ONE) {
                for (; j + 1 < nkt; ++j) {
                    stage(j, kbuf, vnext, (vbuf - vprev) * T::SBYTES, std::false_type{}, std::true_type{});
                    advance();
                }
            }
            stage(nkt - 1, kbuf, vnext, (vbuf - vprev) * T::SBYTES, std::true_type{}, std::true_type{});
        }
    }

    // ---- epilogue: O = O_acc / l (bf16), LSE = ln sum exp(scale * s) ----
    // A lane holds 8-byte pieces of one O row, so storing them directly
    // makes every store instruction touch 32 rows (a head's D elements of a
    // token row, rows a full token stride apart). The rows go through LDS
    // instead: each wave writes its rows into a slot of its own (pitch 2D +
    // 16 bytes), reads them back as whole 16-byte chunks and stores them so
    // that consecutive lanes cover consecutive bytes of a row (short
    // segments, whose tiles are a few stages long: 7-10% faster). One barrier
    // first: the slots overlap the K/V ring, which other waves may still be
    // reading.
    constexpr int OP = 2 * D + 16;
    static_assert(NW * QB * 32 * OP <= T::LDS_BYTES, "O staging fits in the ring");
    __syncthreads();
    char* ow = lds + wave * (QB * 32 * OP);
    const uint32_t o_rs = (uint32_t)(a.o_row * 2);
    char* optr = (char*)a.o + 2 * (avf_elem_offset(q_tok0, a.o_row, h, a.o_head) + gseg * a.o_seg);
    const auto ors = make_rsrc(optr, (uint32_t)(rows_here - 1) * o_rs + 2 * D);
    // the tile's LSE rows (fp32, contiguous per head): stores are clipped to
    // them like the O stores
    float* lptr = a.lse ? a.lse + ((int64_t)h * a.lse_head + q_tok0 + gseg * a.lse_seg) : nullptr;
    const auto lrs = make_rsrc(lptr, (uint32_t)rows_here * 4);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l_tot = l_i[qb] + __shfl_xor(l_i[qb], 32);
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        const int row = wrow0 + qb * 32 + l32;
#pragma unroll
        for (int db = 0; db < T::DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 ov;
#pragma unroll
                for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(o[qb][db][4 * g + e] * inv);
                *reinterpret_cast<bf16x4*>(ow + (qb * 32 + l32) * OP + (db * 32 + 8 * g + 4 * hf) * 2) = ov;
            }
        if (row < rows_here && hf == 0 && a.lse != nullptr) {
            // natural-log LSE: m*scale + ln l (any reference m gives the same value)
            const float lse = l_tot > 0.f ? m_i[qb] * lse_scale + __logf(l_tot) : -INFINITY;
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, lse), lrs, (uint32_t)row * 4, 0, 0);
        }
    }
    // chunk f = 64 i + lane of the wave's rows: row f / (D/8), chunk f % (D/8)
    constexpr int CPR = D / 8;
    static_assert((QB * 32 * CPR) % 64 == 0, "whole store instructions");
#pragma unroll
    for (int i = 0; i < QB * 32 * CPR / 64; ++i) {
        const int f = 64 * i + lane;
        const int r = f / CPR, ch = f % CPR;
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(ow + r * OP + ch * 16);
        if (wrow0 + r < rows_here)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), ors,
                                                   (uint32_t)(wrow0 + r) * o_rs + ch * 16, 0, 0);
    }
    };

    if constexpr (!DEVPLAN) {
        // the grid is exact: every workgroup owns a real tile
        const int32_t linear = avf_linear_tile((int32_t)blockIdx.x, a.num_tiles);
        const AvfTile tile = avf_decode(linear, a.tile_start, a.q_start, a.num_segs, a.num_heads, BM);
        run_tile(tile.seg, tile.mblk, tile.head, a.q_start[tile.seg], a.q_start[tile.seg + 1], a.k_start[tile.seg],
                 a.k_start[tile.seg + 1]);
    } else {
        // Device plan (workspace written by the planner kernel earlier on the
        // stream): word 0 the status of its cu_seqlens check, word 1 the tile
        // count, then the tile prefix. Invalid cu_seqlens: no workgroup forms
        // any address. Otherwise workgroup w takes tiles w, w + G, ... below
        // the count (G = gridDim.x, a multiple of 8, so a workgroup stays on
        // its XCD's contiguous run of tiles).
        const int32_t* plan = a.dev_plan;
        if (plan[0] != 0) return;
        const int32_t nt = plan[1];
        for (int32_t idx = (int32_t)blockIdx.x; idx < nt; idx += (int32_t)gridDim.x) {
            // The lane indices are made opaque to the optimizer once per tile,
            // so the per-lane LDS and buffer offsets derived from them are
            // recomputed for each tile (a few VALU instructions) instead of
            // being kept live across tiles, where they spill (D = 128: 52
            // spill accesses, 19 of them in the stage loop, against 6 and 3).
            // The causal instantiations spill more with it and keep the
            // hoisted offsets.
            if constexpr (!CAUSAL) {
                pin(lane);
                pin(l32);
                pin(hf);
            }
            const int32_t linear = avf_linear_tile(idx, nt);
            // (the causal instantiations keep the binary search: with the
            // 64-way search their stage loop measured 16% slower)
            const AvfTile tile =
                CAUSAL ? avf_decode(linear, plan + AVF_PLAN_HEADER_WORDS, a.cu_q, a.num_segs, a.num_heads, BM)
                       : decode_wave(linear, plan + AVF_PLAN_HEADER_WORDS, a.cu_q, a.num_segs, BM, lane);
            run_tile(tile.seg, tile.mblk, tile.head, a.cu_q[tile.seg], a.cu_q[tile.seg + 1], a.cu_k[tile.seg],
                     a.cu_k[tile.seg + 1]);
            // the next tile's first loads overwrite LDS buffers this one read
            __syncthreads();
        }
    }
}

template <int D, int QB, int NW, int BN, bool ONE>
hipError_t launch_cfg(const AvfLaunchArgs& a, hipStream_t stream) {
    // grid: the exact tile count, or with a device plan the host's bound
    const dim3 grid((uint32_t)a.num_tiles), block(NW * 64);
    if (a.q8) {
        if constexpr (D % 64 == 0 && !ONE && BN >= 128) {  // the 8-bit path runs the general configuration
            if (a.causal)
                hipLaunchKernelGGL((avf_fwd_kernel<D, QB, NW, BN, true, false, true, false>), grid, block, 0, stream, a);
            else
                hipLaunchKernelGGL((avf_fwd_kernel<D, QB, NW, BN, false, false, true, false>), grid, block, 0, stream,
                                   a);
            return hipGetLastError();
        } else {
            return hipErrorInvalidValue;
        }
    }
    if (a.dev_plan) {
        if (a.causal)
            hipLaunchKernelGGL((avf_fwd_kernel<D, QB, NW, BN, true, true, false, ONE>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((avf_fwd_kernel<D, QB, NW, BN, false, true, false, ONE>), grid, block, 0, stream, a);
    } else {
        if (a.causal)
            hipLaunchKernelGGL((avf_fwd_kernel<D, QB, NW, BN, true, false, false, ONE>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((avf_fwd_kernel<D, QB, NW, BN, false, false, false, ONE>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

// Per head_dim tile configuration: (QB query blocks of 32 rows per wave,
// NW waves, BN keys per K/V stage). BM = QB * 32 * NW. Overridable at build
// time (-DAVF_CFG_D128=QB,NW,BN) for tuning sweeps.
#ifndef AVF_CFG_D64
#define AVF_CFG_D64 1, 8, 128
#endif
#ifndef AVF_CFG_D96
#define AVF_CFG_D96 1, 8, 128
#endif
#ifndef AVF_CFG_D128
#define AVF_CFG_D128 1, 8, 128
#endif
template <int QB_, int NW_, int BN_>
struct CfgOf { static constexpr int QB = QB_, NW = NW_, BN = BN_; };
template <int D> struct Cfg;
template <> struct Cfg<64> : CfgOf<AVF_CFG_D64> {};
template <> struct Cfg<96> : CfgOf<AVF_CFG_D96> {};
template <> struct Cfg<128> : CfgOf<AVF_CFG_D128> {};

template <int D>
constexpr int block_m_of() { return Cfg<D>::QB * 32 * Cfg<D>::NW; }

// One-stage configuration (segments of at most kOneStageKeys keys): 4 waves,
// 128 query rows, one 128-key K/V stage; two workgroups per CU.
constexpr int kOneNW = 4, kOneStageKeys = 128;
constexpr int kOneBlockM = 32 * kOneNW;
// Short-stage configuration (segments of at most kShortStageKeys keys): 4
// waves, 128 query rows, 64-key stages in rings of 2 K and 3 V buffers (80 KiB
// at D = 128); two workgroups per CU.
constexpr int kShortNW = 4, kShortBN = 64;
// Measured against the general configuration on 56-head, D = 128 segments
// of S keys: +26% at S = 256, +31% at 384, +4% at 512, even at 768-1024,
// 2-3% slower from 2048 on (more barriers per key).
constexpr int kShortStageKeys = 512;

template <int D>
hipError_t launch_d(const AvfLaunchArgs& a, hipStream_t stream) {
    if (a.one_stage) return launch_cfg<D, 1, kOneNW, kOneStageKeys, true>(a, stream);
    if (a.short_stage) return launch_cfg<D, 1, kShortNW, kShortBN, false>(a, stream);
    return launch_cfg<D, Cfg<D>::QB, Cfg<D>::NW, Cfg<D>::BN, false>(a, stream);
}

}  // namespace

int32_t avf_block_m(int32_t head_dim) {
    switch (head_dim) {
        case 64: return block_m_of<64>();
        case 96: return block_m_of<96>();
        case 128: return block_m_of<128>();
        default: return -1;
    }
}

int32_t avf_block_m_one(int32_t head_dim) {
    return (head_dim == 64 || head_dim == 96 || head_dim == 128) ? kOneBlockM : -1;
}

int32_t avf_one_stage_keys() { return kOneStageKeys; }

int32_t avf_short_stage_keys() { return kShortStageKeys; }

hipError_t avf_launch(const AvfLaunchArgs& a, int32_t head_dim, hipStream_t stream) {
    switch (head_dim) {
        case 64: return launch_d<64>(a, stream);
        case 96: return launch_d<96>(a, stream);
        case 128: return launch_d<128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}
