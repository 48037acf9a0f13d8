// Chunked Gated DeltaNet prefill for bf16 inputs with d_k = d_v = 128 and
// 64-token chunks: one workgroup per (segment, head) covering all 128 state
// columns, long sequences cut into segments.
//
// "Inference for linear attention and hybrid architectures", section "Two
// ways to write the same computation": DeltaNet's update
// (I - b_t k_t^T k_t) S + b_t k_t^T v_t with a decay gate multiplied in, and
// the remark that the in-chunk corrections must first be written in matrix
// form.  The matrix form used here (derived; the page poses it as an
// exercise): inside a chunk entered with state S, with g the running log
// decay, T = (I + A)^-1 for A_tj = b_t exp(g_t - g_j) (k_t . k_j), j < t,
//   X = K S,  Y = V - diag(exp g) X,  U = T diag(b) Y,
//   O = diag(exp g) Q S + ((Q K^T) .* D) U,
//   S <- exp(g_last) S + K^T diag(exp(g_last - g)) U.
// T diag(b) does not depend on S; gdn_prep computes it for every chunk
// beforehand and leaves it in the workspace as bf16 hi / lo planes.
//
// Layout of the work.  Each of the 8 waves owns 16 columns of the 128 x 128
// fp32 state, all rows, as MFMA accumulator tiles.  For the 16x16x32 MFMA a
// pair of those tiles (rows 32s .. 32s + 31) is, as it stands, the B operand
// of X = K S and the A operand of O^T = S^T Q^T, with the contraction index
// in the "split" order {4g .. 4g + 3} u {16 + 4g .. 16 + 4g + 3} per lane
// group g.  Y and U come out of their products in the same accumulator
// layout, so they are in turn the B operand of U = T diag(b) Y and of the
// state update, and (transposed) the A operand of O^T += U^T P^T.  The whole
// chain is therefore local to a wave: only q, k, v, T diag(b) and
// P = (Q K^T) .* D are shared, through LDS.  P is formed once per chunk by
// all waves (10 lower-triangle tiles).  Outputs come out transposed, lane =
// token, 4 consecutive columns each, and go through LDS to whole-row stores.
//
// Operand format: every MFMA takes fp16 operands (v_mfma_f32_16x16x32_f16,
// fp32 accumulation).  q and k are converted to fp16 as they are staged
// (exact for bf16 values below 2^15 in magnitude); v stays bf16 (it only
// enters Y on the vector unit).  The fp32-derived operands S, Y and U are
// rounded to fp16 after scaling each wave's slice by a power of two that
// keeps its largest magnitude below 2^15, undone exactly on the fp32
// results; gdn_seg_prep does the same for T diag(b), per (chunk, head).
// P needs |q_i| |k_j| < 2^15 (always true for L2-normalised q and k).
// A bf16 hi + lo pair would keep about 16 significant bits per operand at
// two MFMAs per product; fp16 keeps 11 at one, which puts the result about
// 5e-4 from the exact one on L2-normalised inputs (a simulation of this
// chunked form in numpy), against 1e-5 for hi + lo.  The scan multiplies
// the transitions with hi + lo pairs: it runs once per segment.
//
// Segments ("Chunked prefill comes for free": a prompt cut into pieces is
// processed the same way when only the state is handed on; here the pieces
// of one prompt run side by side).  The update is affine in the state that
// enters a segment: S_out = M S_in + dS, where dS is the segment's state
// from S_in = 0 and M (d_k x d_k) its transition, the product of the chunks'
// exp(g_last) I - K^T diag(exp(g_last - g)) T diag(b) diag(exp g) K.  So:
//   phase A: every segment but the last of a sequence cut into several runs
//     pass 1 (gdn_seg_state): dS and M, by running the state update alone
//     on [S | M] from [0 | I] (M takes no values: its Y is
//     -diag(exp g) K M).  In batches of many (sequence, head) pairs the
//     first segment runs pass 2 here instead (it needs no M: its entry
//     state is the pool's), and its end state S_in(1) goes to the workspace;
//   scan (gdn_seg_scan): per (sequence, head),
//     S_in(j + 1) = M_j S_in(j) + dS_j, written over dS_j, from S_in(0) =
//     the pool state (copied to a slot of its own) or from S_in(1);
//   phase B: pass 2 for the remaining segments from their S_in; the last one
//     writes the final state to the pool.
// A sequence of one segment is handled by pass 2 alone, reading and writing
// the pool, in phase A.  State slots in the workspace are tile-major (a wave reads or
// writes one accumulator tile as one contiguous 1 KiB); M is stored as the
// scan's A operand fragments.
#include <algorithm>

#include "chunk_common.h"
#include "launch.h"

namespace gla {
namespace {

constexpr int NWV = 8;             // waves
constexpr int NTH = NWV * 64;      // threads
constexpr int D = 128;             // d_k = d_v
constexpr int CH = 64;             // chunk
// LDS row strides: 16-byte operand reads (16 lanes on 16 rows) and the
// transpose read run at full rate with rows 72 dwords (or 40) apart, half
// rate 68 dwords apart.
constexpr int LQ = D + 16;         // q
constexpr int LK = D + 16;         // k, v
constexpr int LP = CH + 16;        // P and T diag(beta), keys in p_col() order
constexpr int LO = D + 8;          // outputs: 8-byte writes (16 rows x 4 lane groups), row reads
constexpr int kTargetBlocks = 256; // about one workgroup per compute unit
constexpr int kPlaneElems = CH * CH;       // T diag(beta) (fp16) per (chunk, head)

// One chunk of the global inputs in registers: 2 x 16 bytes per thread of
// each 64 x 128 bf16 tile, 16 bytes of the 8 KiB fp16 T diag(beta) plane,
// and the gate of token `lane` (wave 0).
template <bool WQ, bool WV>
struct GPrefetch {
    u32x4 q[WQ ? 2 : 1], k[2], v[2], t;
    float a;
    float tinv;        // the inverse scale of this chunk's T diag(beta)
    int n;
};

// Buffer resources over one segment's rows of q, k, v, alpha and its T
// planes, built once; chunk c is then reached through a scalar offset.
// Rows past the segment read as zero, and so does a chunk past its last
// one (its offset is the resource's size).
struct SegSrc {
    BufRsrc q, k, v, a, t;
    uint32_t q_end, a_end, t_end;
    uint32_t q_step, a_step, t_step;     // bytes per chunk
    const float* tinv;
    long ti0;                            // tinv index of chunk 0
    int nch, H;
};

template <bool WQ, bool WV>
__device__ __forceinline__ SegSrc seg_src(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* alpha,
                                          const uint16_t* planes, const float* tinv, long t0, int rows, long ci0,
                                          int nch, int h, int H) {
    const long stride = static_cast<long>(H) * D;
    const uint32_t ext = rows_extent(rows, stride * 2, D * 2);
    const bool w0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0;
    const uint32_t aext = rows_extent(rows, static_cast<long>(H) * 4, 4);
    const uint32_t text = static_cast<uint32_t>(nch > 0 ? ((nch - 1) * static_cast<long>(H) + 1) * kPlaneElems * 2 : 0);
    SegSrc r{BufRsrc(q + t0 * stride + h * D, WQ ? ext : 0u), BufRsrc(k + t0 * stride + h * D, ext),
             BufRsrc(v + t0 * stride + h * D, WV ? ext : 0u), BufRsrc(alpha + t0 * H + h, w0 ? aext : 0u),
             BufRsrc(planes + (ci0 * H + h) * kPlaneElems, text),
             ext, aext, text,
             static_cast<uint32_t>(CH * stride * 2), static_cast<uint32_t>(CH * H * 4),
             static_cast<uint32_t>(static_cast<long>(H) * kPlaneElems * 2),
             tinv, ci0 * H + h, nch, H};
    return r;
}

// Global -> registers for chunk c of the segment.
template <bool WQ, bool WV>
__device__ __forceinline__ void g_fetch(GPrefetch<WQ, WV>& pf, const SegSrc& sr, int c, int n) {
    const bool in = c < sr.nch;
    const uint32_t so = in ? c * sr.q_step : sr.q_end;
    const uint32_t sa = in ? c * sr.a_step : sr.a_end;
    const uint32_t st = in ? c * sr.t_step : sr.t_end;
    const int tid = threadIdx.x;
    const long stride = static_cast<long>(sr.H) * D;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int x = tid + u * NTH;
        const uint32_t offb = static_cast<uint32_t>(((x / (D / 8)) * stride + (x % (D / 8)) * 8) * 2);
        pf.k[u] = sr.k.load16_nt(offb, so);
        if constexpr (WV) pf.v[u] = sr.v.load16_nt(offb, so);
        if constexpr (WQ) pf.q[u] = sr.q.load16_nt(offb, so);
    }
    // T plane: vector tid of 512 (row tid / 8, 8 columns (tid % 8) * 8);
    // rows 0..31 x columns 32..63 are never used
    pf.t = sr.t.load16((tid >> 3) < 32 && (tid & 7) >= 4 ? sr.t_end : static_cast<uint32_t>(tid * 16), st);
    pf.tinv = in ? sr.tinv[sr.ti0 + static_cast<long>(c) * sr.H] : 0.f;
    pf.a = sr.a.loadf_nt(static_cast<uint32_t>((tid & 63) * sr.H * 4), sa);
    pf.n = n;
}

// Gate tables of a chunk from wave 0's prefetched gates (rows past n:
// alpha = 1): running log2 decay, 2^g2, 2^(g2_last - g2), 2^g2_last.
template <class PF>
__device__ __forceinline__ void g_stage_gates(float* g2, float* eg, float* dec, float* gamma, const PF& pf) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    if (__builtin_amdgcn_readfirstlane(tid >> 6) == 0) {
        const float a = lane < pf.n ? pf.a : 1.f;
        const float x = wave_inclusive_sum(__log2f(fmaxf(a, kMinDecay)));
        const float glast = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), CH - 1));
        if (g2) g2[lane] = x;
        if (eg) eg[lane] = hw_exp2(x);
        dec[lane] = hw_exp2(glast - x);
        if (lane == 0) *gamma = hw_exp2(glast);
    }
}

// fp16 operands: two fp32 values -> packed fp16 (round to nearest even)
__device__ __forceinline__ uint32_t pk_f16(float a, float b) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const f16x2 hv = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
    return __builtin_bit_cast(uint32_t, hv);
}
// 8 bf16 values (one 16-byte vector) -> 8 fp16 values
__device__ __forceinline__ u32x4 bf16x8_to_f16(u32x4 w) {
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = pk_f16(__uint_as_float(w[e] << 16), __uint_as_float(w[e] & 0xffff0000u));
    return r;
}
__device__ __forceinline__ f32x4 mfma_f16(const bf16x8& a, const bf16x8& b, f32x4 c) {
    typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
}
// A pair of accumulator tiles times s as one fp16 operand fragment (split k order).
__device__ __forceinline__ bf16x8 f16_pair(const f32x4& a, const f32x4& b, float sc) {
    return as_bf16x8(u32x4{pk_f16(a.x * sc, a.y * sc), pk_f16(a.z * sc, a.w * sc), pk_f16(b.x * sc, b.y * sc),
                           pk_f16(b.z * sc, b.w * sc)});
}
// The same for a wave-uniform power of two s: x s is exact, and written as an
// fma with a zero addend it compiles to the mixed-precision fma that rounds
// to fp16 into one half of the packed register (one instruction per value
// instead of a multiply per value and a pack per two).  Only the sign of a
// zero product can differ (+0 for -0), which changes no MFMA product.
__device__ __forceinline__ bf16x8 f16_pair_scaled(const f32x4& a, const f32x4& b, float sc) {
    auto m = [sc](float x) { return __builtin_fmaf(x, sc, 0.f); };
    return as_bf16x8(u32x4{pk_f16(m(a.x), m(a.y)), pk_f16(m(a.z), m(a.w)), pk_f16(m(b.x), m(b.y)),
                           pk_f16(m(b.z), m(b.w))});
}
// Range guard: a power of two s with (largest |x| of the wave) * s < 2^15,
// and 1 / s (both exact; s is capped at 2^126 for tiny or zero slices).
struct Scale {
    float s, inv;
};
// Maximum of a non-negative float over the wave, as a wave-uniform value:
// integer maxima of the bit patterns (the same order for x >= 0) within each
// row of 16 lanes by DPP, then over the four rows' lanes 0, 16, 32, 48.
__device__ __forceinline__ float wave_max_nonneg(float x) {
    int v = __float_as_int(x);
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0xb1, 0xf, 0xf, false));    // quad_perm [1,0,3,2]
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x4e, 0xf, 0xf, false));    // quad_perm [2,3,0,1]
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x124, 0xf, 0xf, false));   // row_ror:4
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x128, 0xf, 0xf, false));   // row_ror:8
    const int r = max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
                      max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
    return __int_as_float(r);
}
__device__ __forceinline__ Scale range_scale(float local_max) {
    const float m = wave_max_nonneg(local_max);
    const int eb = static_cast<int>((__float_as_uint(m) >> 23) & 0xffu);   // m < 2^(eb - 126)
    const int sf = clampi(268 - eb, 1, 253);                               // s = 2^(141 - eb)
    return {__uint_as_float(static_cast<uint32_t>(sf) << 23), __uint_as_float(static_cast<uint32_t>(254 - sf) << 23)};
}
// max(m, |a|, |b|) as two medians against +inf (v_med3_f32 with the
// absolute values as source modifiers): fmaxf would first quiet each |x|
// against signalling NaN, one more instruction per value
__device__ __forceinline__ float absmax3(float m, float a, float b) {
    constexpr float inf = __builtin_inff();
    return __builtin_amdgcn_fmed3f(__builtin_amdgcn_fmed3f(fabsf(a), fabsf(b), inf), m, inf);
}
__device__ __forceinline__ float absmax4(const f32x4& v, float m) {
    return absmax3(absmax3(m, v.x, v.y), v.z, v.w);
}

// Registers -> LDS: a 64 x 128 tile, as it is (bf16) or converted to fp16.
template <bool TO_F16>
__device__ __forceinline__ void g_stage_tile(uint16_t* dst, int ld, const u32x4 (&w)[2], uint16_t* dst2 = nullptr,
                                             int ld2 = 0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int x = threadIdx.x + u * NTH;
        const u32x4 val = TO_F16 ? bf16x8_to_f16(w[u]) : w[u];
        *reinterpret_cast<u32x4*>(dst + (x / (D / 8)) * ld + (x % (D / 8)) * 8) = val;
        if (dst2) *reinterpret_cast<u32x4*>(dst2 + (x / (D / 8)) * ld2 + (x % (D / 8)) * 8) = val;
    }
}
__device__ __forceinline__ void g_stage_plane(uint16_t (*t)[LP], const u32x4& w) {
    *reinterpret_cast<u32x4*>(&t[threadIdx.x >> 3][(threadIdx.x & 7) * 8]) = w;
}

// A state slot of the workspace, tile-major: accumulator tile (row block mt,
// column block cb) is 1 KiB, lane l's 4 values at ((cb * 8 + mt) * 64 + l) * 4,
// so every access of a wave to one tile is one contiguous 1 KiB.
__device__ __forceinline__ long g_tile(int cb, int mt, int lane) { return ((cb * 8 + mt) * 64 + lane) * 4; }
// this wave's column block (8 tiles) of a slot
__device__ __forceinline__ float* g_slot(float* ws, long slot) {
    return ws + slot * D * D + g_tile(threadIdx.x >> 6, 0, threadIdx.x & 63);
}
__device__ __forceinline__ void g_slot_load(f32x4 (&S)[8], const float* p) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) S[mt] = *reinterpret_cast<const f32x4*>(p + mt * 256);
}
__device__ __forceinline__ void g_slot_store(float* p, const f32x4 (&S)[8]) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) *reinterpret_cast<f32x4*>(p + mt * 256) = S[mt];
}
// M in the layout the scan reads it in: the A operand fragments of row
// block rb, 32-deep block s and half h2 (columns 32 s + 16 h2 .. + 15), lane
// l holding M[16 rb + l % 16][32 s + 16 h2 + 4 (l / 16) + e], e = 0..3, at
// (((rb * 4 + s) * 2 + h2) * 64 + l) * 4; each fragment is 1 KiB.
__device__ __forceinline__ long g_mfrag(int rb, int s, int h2, int lane) { return (((rb * 4 + s) * 2 + h2) * 64 + lane) * 4; }
// This wave's 8 tiles of a row-major [d][n] state (columns col .. col + 15).
__device__ __forceinline__ void g_rowmajor_load(f32x4 (&S)[8], const float* src, int col) {
    const AccPos ap;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[mt][r] = src[(srow(mt, ap.row0) + r) * D + col + ap.col];
}

// Split a pair of accumulator tiles into bf16 hi / lo operand fragments
// (the scan's products).
__device__ __forceinline__ void split_pair(const f32x4& a, const f32x4& b, bf16x8& hi, bf16x8& lo) {
    s16x4 h0, l0, h1, l1;
    split4(a, h0, l0);
    split4(b, h1, l1);
    hi = cat8(h0, h1);
    lo = cat8(l0, l1);
}

// The fp16 operand fragments of this wave's state slice (tiles 2s, 2s + 1
// for the d_k block s) and the scale they carry.
__device__ __forceinline__ Scale state_operand(bf16x8 (&sf)[4], const f32x4 (&S)[8]) {
    float m = 0.f;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) m = absmax4(S[mt], m);
    const Scale sc = range_scale(m);
#pragma unroll
    for (int s = 0; s < 4; ++s) sf[s] = f16_pair_scaled(S[2 * s], S[2 * s + 1], sc.s);
    return sc;
}

// Y = V - diag(eg) X xinv for this wave's columns (V^T fragments vf hold
// tokens 32ks + 4g + {0..3} (first half) and 32ks + 16 + 4g + {0..3}; xinv
// undoes the state operand's scale), as fp16 operand fragments by 32-token
// half; returns their scale.  NEG_ONLY: Y = -diag(eg) X xinv.
template <bool NEG_ONLY>
__device__ __forceinline__ Scale form_y(bf16x8 (&yf)[2], const f32x4 (&X)[4], const bf16x8 (&vf)[2], const float* eg,
                                        float xinv) {
    const int g4 = ((threadIdx.x & 63) >> 4) * 4;
    f32x4 y[4];
    float m = 0.f;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const f32x4 e = *reinterpret_cast<const f32x4*>(eg + it * 16 + g4) * xinv;
        if constexpr (NEG_ONLY) {
            y[it] = -(e * X[it]);
        } else {
            const u32x4 vw = __builtin_bit_cast(u32x4, vf[it >> 1]);
            const uint32_t w0 = (it & 1) ? vw.z : vw.x, w1 = (it & 1) ? vw.w : vw.y;
            const f32x4 vv = {__uint_as_float(w0 << 16), __uint_as_float(w0 & 0xffff0000u),
                              __uint_as_float(w1 << 16), __uint_as_float(w1 & 0xffff0000u)};
            y[it] = vv - e * X[it];
        }
        m = absmax4(y[it], m);
    }
    const Scale sc = range_scale(m);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) yf[ks] = f16_pair_scaled(y[2 * ks], y[2 * ks + 1], sc.s);
    return sc;
}

// U = T diag(beta) Y (lower triangular: row block it uses token halves
// ks <= it / 2; uinv undoes the scales of T diag(beta) and Y), then
// diag(dec) U and (WANT_U) U as fp16 operand fragments under one scale,
// which is returned.
template <bool WANT_U = true>
__device__ __forceinline__ Scale form_u(bf16x8 (&uf)[2], bf16x8 (&df)[2], const bf16x8 (&yf)[2], const uint16_t (*t)[LP],
                                        const float* dec, float uinv) {
    f32x4 U[4];
    float m = 0.f;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        U[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks <= (it >> 1); ++ks) U[it] = mfma_f16(frag_kc(&t[0][0], LP, it * 16, 32 * ks), yf[ks], U[it]);
        m = absmax4(U[it], m);
    }
    // the scale is taken on the true U = uinv U[it]; dec <= 1, so the same
    // scale serves diag(dec) U
    Scale sc = range_scale(m * uinv);
    const float f = uinv * sc.s;
    const int g4 = ((threadIdx.x & 63) >> 4) * 4;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const f32x4 u0 = U[2 * ks] * f, u1 = U[2 * ks + 1] * f;
        if constexpr (WANT_U) uf[ks] = f16_pair(u0, u1, 1.f);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(dec + 32 * ks + g4);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(dec + 32 * ks + 16 + g4);
        df[ks] = f16_pair(u0 * d0, u1 * d1, 1.f);
    }
    return sc;
}

// A float that is the same on every lane, in a scalar register.
__device__ __forceinline__ float uniform_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// The state may be held as S = sigma Shat, sigma a running product of the
// chunks' decays gamma: the update S <- gamma S + X is then
// Shat <- Shat + X / (gamma sigma) with sigma <- gamma sigma, no pass over
// the state, while gamma sigma stays at or above kFoldMin; a chunk that
// would take it lower scales Shat by gamma sigma first and restarts sigma
// at 1.  Shat stays within 2^30 |S|.  fold_scale() applies that rule (to S
// and, if given, M) and returns the factor of X.
constexpr float kFoldMin = 0x1p-30f;
__device__ __forceinline__ float fold_scale(f32x4 (&S)[8], f32x4* M, float gam, float& sigma) {
    const float gs = uniform_f(gam * sigma);
    const bool fold = gs >= kFoldMin;
    if (!fold) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            S[mt] *= gs;
            if (M) M[mt] *= gs;
        }
    }
    sigma = fold ? gs : 1.f;
    return fold ? __builtin_amdgcn_rcpf(gs) : 1.f;
}

// S (this wave's columns) <- gamma S + K^T diag(dec) U (df carries dinv);
// FOLD: S held as sigma Shat (fold_scale).
template <bool FOLD>
__device__ __forceinline__ void state_update(f32x4 (&S)[8], const uint16_t* kbase, float gam, const bf16x8 (&df)[2],
                                             float dinv, float& sigma) {
    float dm = dinv;
    if constexpr (FOLD) dm *= fold_scale(S, nullptr, gam, sigma);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) acc = mfma_f16(frag_kt_pair(kbase, LK, mt, 32 * ks), df[ks], acc);
        S[mt] = FOLD ? S[mt] + dm * acc : gam * S[mt] + dm * acc;
    }
}

// X = K S (rows of the chunk x this wave's columns, times the state
// operand's scale); O^T = S^T Q^T (same scale) too when WQ.
template <bool WQ>
__device__ __forceinline__ void k_times_s(f32x4 (&X)[4], f32x4* ot, const bf16x8 (&sf)[4], const uint16_t* kbase,
                                          const uint16_t* qbase) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        X[it] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (WQ) ot[it] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            X[it] = mfma_f16(frag_kc(kbase, LK, it * 16, 32 * s), sf[s], X[it]);
            if constexpr (WQ) ot[it] = mfma_f16(sf[s], frag_kc(qbase, LQ, it * 16, 32 * s), ot[it]);
        }
    }
}

// Pass 1's two products with K, for the state columns S and the transition
// columns M of this wave at once, so each K fragment is read once.
__device__ __forceinline__ void k_times_sm(f32x4 (&XS)[4], f32x4 (&XM)[4], const bf16x8 (&sf)[4], const bf16x8 (&mf)[4],
                                           const uint16_t* kbase) {
#pragma unroll
    for (int it = 0; it < 4; ++it) XS[it] = XM[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const bf16x8 kf = frag_kc(kbase, LK, it * 16, 32 * s);
            XS[it] = mfma_f16(kf, sf[s], XS[it]);
            XM[it] = mfma_f16(kf, mf[s], XM[it]);
        }
    }
}
// Pass 1's update of [S | M], both held with the same sigma.
__device__ __forceinline__ void state_update_sm(f32x4 (&S)[8], f32x4 (&M)[8], const uint16_t* kbase, float gam,
                                                const bf16x8 (&sdf)[2], float sinv, const bf16x8 (&mdf)[2], float minv,
                                                float& sigma) {
    const float f = fold_scale(S, M, gam, sigma);
    const float sd = sinv * f, md = minv * f;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
        f32x4 as = {0.f, 0.f, 0.f, 0.f}, am = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const bf16x8 kt = frag_kt_pair(kbase, LK, mt, 32 * ks);
            as = mfma_f16(kt, sdf[ks], as);
            am = mfma_f16(kt, mdf[ks], am);
        }
        S[mt] += sd * as;
        M[mt] += md * am;
    }
}

// Which sequence, segment and slot a block works on.
struct GSeg {
    int b, g, nseg, slot, t0, t1;
    long ci0;          // global chunk index of the segment's first chunk
    long jsplit;       // index of the sequence's first split segment
};

// false (for the whole block) if the slot is invalid, or if a malformed
// cu_seqlens gives the sequence split segments beyond the workspace's
// nsplit_max.
__device__ __forceinline__ bool seg_bounds(GSeg& sg, int b, int g, int nseg, const int32_t* cu, int n_tokens,
                                           const int32_t* coff, const int32_t* soff, const int32_t* slot_idx,
                                           int n_slots, int lseg, long nsplit_max) {
    const int slot = slot_idx[b];
    if (slot < 0 || slot >= n_slots) return false;
    if (nseg > 1 && static_cast<long>(soff[b]) + nseg - 1 > nsplit_max) return false;
    const int s0 = clampi(cu[b], 0, n_tokens);
    const int s1 = clampi(cu[b + 1], s0, n_tokens);
    sg.b = b;
    sg.g = g;
    sg.nseg = nseg;
    sg.slot = slot;
    sg.t0 = min(s0 + g * lseg, s1);
    sg.t1 = min(sg.t0 + lseg, s1);
    sg.ci0 = static_cast<long>(coff[b]) + static_cast<long>(g) * (lseg / CH);
    sg.jsplit = soff[b];
    return true;
}

// ------------------------------------------------------------------ prep
// T diag(beta) for every (chunk, head), one wave per item, the items strided
// over a persistent grid.  A = strictly-lower(diag(beta) (K K^T .* D)) comes
// from the MFMA on K fragments loaded straight from HBM; T = (I + A)^-1 by
// 16 x 16 blocks (forward substitution on the diagonal blocks, the fp32
// MFMA for the others); then lane j takes column j of T, scales it by
// beta_j and the item by a power of two (range guard; its inverse goes to
// tinv), and the item is written as one fp16 plane, one 128-byte row per
// store instruction.  Rows 0..31 x columns 32..63 are zero and never read:
// not written.
constexpr int PW = 4;              // waves per prep workgroup
constexpr int LA = CH + 4;         // fp32 row stride of A in LDS
constexpr int kPlRow = CH + 8;     // fp16 row stride of a plane staged in A's place
constexpr int kPrepGroups = 512;   // 2 resident workgroups per compute unit

__global__ void __launch_bounds__(PW * 64, 2)
gdn_seg_prep(const uint16_t* __restrict__ k, const float* __restrict__ alpha, const float* __restrict__ beta,
             const int32_t* __restrict__ cu, int n_seqs, int n_tokens, int H, const int32_t* __restrict__ coff,
             uint16_t* __restrict__ planes, float* __restrict__ tinv) {
    __shared__ alignas(16) float As[PW][CH][LA];
    __shared__ alignas(16) float gs[PW][CH];
    __shared__ alignas(16) float bs[PW][CH];
    __shared__ float Ws[PW][16][17];      // one 16 x 16 product on its way to an MFMA operand
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const AccPos ap;
    const long n_items = static_cast<long>(coff[n_seqs]) * H;
    const long stride = static_cast<long>(H) * D;
    auto wave_sync = []() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    };
    // an item's rows: k from row tok0 of head h, n of them valid (none past
    // the last item: its loads read nothing)
    struct Item {
        long tok0;
        int h, n;
    };
    auto locate = [&](long item) {
        Item it{0, 0, 0};
        if (item < n_items) {
            it.h = static_cast<int>(item % H);
            const int ci = static_cast<int>(item / H);
            const int b = find_span_owner(coff, n_seqs, ci);
            const int s0 = clampi(cu[b], 0, n_tokens);
            const int s1 = clampi(cu[b + 1], s0, n_tokens);
            const int c0 = (ci - coff[b]) * CH;
            it.n = max(0, min(CH, s1 - s0 - c0));
            it.tok0 = s0 + max(c0, 0);
        }
        return it;
    };
    u32x4 kf[4][4];
    float a, bt;
    auto fetch = [&](const Item& it) {
        const BufRsrc rk(k + it.tok0 * stride + it.h * D, rows_extent(it.n, stride * 2, D * 2));
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                kf[tt][ks] = rk.load16_nt(static_cast<uint32_t>(
                    ((tt * 16 + (lane & 15)) * stride + 32 * ks + (lane >> 4) * 8) * 2));
        const uint32_t gext = rows_extent(it.n, static_cast<long>(H) * 4, 4);
        a = BufRsrc(alpha + it.tok0 * H + it.h, gext).loadf_nt(static_cast<uint32_t>(lane * H * 4));
        bt = BufRsrc(beta + it.tok0 * H + it.h, gext).loadf_nt(static_cast<uint32_t>(lane * H * 4));
    };
    const long step = static_cast<long>(gridDim.x) * PW;
    long item = static_cast<long>(blockIdx.x) * PW + wave;
    Item cur = locate(item);
    fetch(cur);
    // the next item's loads are issued as soon as this item's A is formed,
    // so they are in flight during the inversion and the plane stores
    for (; item < n_items; item += step) {
        const int n = cur.n;
        gs[wave][lane] = wave_inclusive_sum(__log2f(fmaxf(lane < n ? a : 1.f, kMinDecay)));
        bs[wave][lane] = lane < n ? bt : 0.f;
        wave_sync();
        // A, the 10 tiles on and below the diagonal (entries j >= i are 0)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
            for (int jt = 0; jt <= tt; ++jt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) acc = mfma_bf16(as_bf16x8(kf[tt][ks]), as_bf16x8(kf[jt][ks]), acc);
                const int j = jt * 16 + ap.col;
                const float gj = gs[wave][j];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = tt * 16 + ap.row0 + r;
                    As[wave][i][j] = (j < i) ? bs[wave][i] * hw_exp2(gs[wave][i] - gj) * acc[r] : 0.f;
                }
            }
        }
        const float bj = bs[wave][lane];        // read before the next item's beta lands
        const Item nxt = locate(item + step);
        fetch(nxt);
        wave_sync();
        // T = (I + A)^-1 (A strictly lower triangular, so I + A is unit lower
        // triangular) by 16 x 16 blocks: the diagonal blocks
        // T_bb = (I + A_bb)^-1 by forward substitution, lane c of lane group
        // b solving for column c of T_bb; then, for i > j in order of i - j,
        //   T_ij = -T_ii (sum over j <= k < i of A_ik T_kj)
        // on the fp32 MFMA.  A's blocks below the diagonal stay in place;
        // T goes transposed into the upper half, T[r][c] at As[c][r] for r
        // in c's block row or below, over A's diagonal blocks once those are
        // solved.  One wave owns As[wave]: its LDS operations complete in
        // order, and wave_sync() keeps the compiler from reordering them.
        {
            const int bb = lane >> 4, c = lane & 15;
            float* Ab = &As[wave][16 * bb][16 * bb];
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
                for (int m = 0; m < r; m += 4) {
                    const f32x4 a4 = *reinterpret_cast<const f32x4*>(Ab + r * LA + m);
                    acc -= a4.x * x[m];
                    if (m + 1 < r) acc -= a4.y * x[m + 1];
                    if (m + 2 < r) acc -= a4.z * x[m + 2];
                    if (m + 3 < r) acc -= a4.w * x[m + 3];
                }
                x[r] = acc;
            }
            wave_sync();
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<f32x4*>(Ab + c * LA + 4 * q) = f32x4{x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]};
        }
        wave_sync();
        {
            float* Aw = &As[wave][0][0];
            float* Wt = &Ws[wave][0][0];
            const int i16 = lane & 15, kg = lane >> 4;
#pragma unroll
            for (int d = 1; d < 4; ++d) {
#pragma unroll
                for (int bi = d; bi < 4; ++bi) {
                    const int bj = bi - d;
                    // W = sum_k A_ik T_kj: A_ik[i16][4 s + kg] in place, T_kj[4 s + kg][i16] transposed
                    f32x4 w = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int bk = bj; bk < bi; ++bk)
#pragma unroll
                        for (int s4 = 0; s4 < 4; ++s4)
                            w = mfma_f32(Aw[(16 * bi + i16) * LA + 16 * bk + 4 * s4 + kg],
                                         Aw[(16 * bj + i16) * LA + 16 * bk + 4 * s4 + kg], w);
                    // W (lane: column i16, rows 4 kg .. + 3) through LDS into the B layout
#pragma unroll
                    for (int r = 0; r < 4; ++r) Wt[(4 * kg + r) * 17 + i16] = w[r];
                    wave_sync();
                    // T_ii W: T_ii[i16][4 s + kg] transposed, W[4 s + kg][i16]
                    f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4)
                        t = mfma_f32(Aw[(16 * bi + 4 * s4 + kg) * LA + 16 * bi + i16], Wt[(4 * s4 + kg) * 17 + i16], t);
                    // T_ij[4 kg + r][i16] = -t[r], transposed into block (j, i)
                    *reinterpret_cast<f32x4*>(&Aw[(16 * bj + i16) * LA + 16 * bi + 4 * kg]) = -t;
                    wave_sync();
                }
            }
        }
        // column `me` of T (the lane index, recomputed per item so the
        // selects below are not hoisted out of the item loop): row me of As
        // from me's block on, zero above it
        const int me = opaque(lane);
        float x[CH];
        {
            const float* Tc = &As[wave][me][0];
            const int b0 = me >> 4;
#pragma unroll
            for (int q = 0; q < CH / 4; ++q) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(Tc + 4 * q);
                const bool keep = (q >> 2) >= b0;
                x[4 * q] = keep ? v.x : 0.f;
                x[4 * q + 1] = keep ? v.y : 0.f;
                x[4 * q + 2] = keep ? v.z : 0.f;
                x[4 * q + 3] = keep ? v.w : 0.f;
            }
        }
        // T diag(beta) -> an fp16 plane scaled by a power of two (its
        // inverse kept per item): column me into LDS (over A, all of which
        // has been read), then whole rows out, 16 bytes a lane
        float mloc = 0.f;
#pragma unroll
        for (int r = 0; r < CH; ++r) mloc = fmaxf(mloc, fabsf(x[r] * bj));
        const Scale sc = range_scale(mloc);
        if (lane == 0) tinv[item] = sc.inv;
        // column me of the plane sits at p_col() order (columns 32..63 stay in 32..63)
        const int pos = p_col(me >> 4, (me >> 2) & 3) + (me & 3);
        uint16_t* pl = reinterpret_cast<uint16_t*>(&As[wave][0][0]);
        wave_sync();
#pragma unroll
        for (int r = 0; r < CH; r += 2) {
            const uint32_t hv = pk_f16(x[r] * bj * sc.s, x[r + 1] * bj * sc.s);
            pl[r * kPlRow + pos] = static_cast<uint16_t>(hv & 0xffffu);
            pl[(r + 1) * kPlRow + pos] = static_cast<uint16_t>(hv >> 16);
        }
        wave_sync();
        const BufRsrc rp(planes + item * kPlaneElems, kPlaneElems * 2u);
#pragma unroll
        for (int u = 0; u < CH * CH / 8 / 64; ++u) {
            const int vix = lane + 64 * u, row = vix >> 3, cb = vix & 7;
            // rows 0..31 x columns 32..63 are never read: not written
            const bool skip = row < 32 && cb >= 4;
            rp.store_b128(*reinterpret_cast<const u32x4*>(pl + row * kPlRow + 8 * cb),
                          skip ? 0x80000000u : static_cast<uint32_t>((row * CH + 8 * cb) * 2));
        }
        cur = nxt;
        wave_sync();       // this wave's A and gate tables are rewritten by its next item
    }
}

// ------------------------------------------------------------------ passes
// Arguments shared by the two passes.
struct SegArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* alpha;
    const int32_t* cu;
    int n_seqs, n_tokens, H;
    float* pool;
    int n_slots;
    const int32_t* slot_idx;
    int zero_init, lseg;
    const int32_t* coff;          // first global chunk of every sequence
    const int32_t* seg_off;       // first segment of every sequence
    const int32_t* split_off;     // first split segment (every segment but the last of a split sequence)
    const int32_t* splitseg_off;  // first segment among those of split sequences (all their segments)
    const uint16_t* planes;       // T diag(beta) per (chunk, head), fp16
    const float* tinv;            // their inverse scales
    long n_chunks_max, nsplit_max;
    float* wsS;                   // per (split segment, head): dS, then the entry state of the next segment
    float* wsM;                   // per (split segment, head): M, as the scan's operand fragments
    float* wsI;                   // per split sequence (at its first split segment) and head: S_in(0)
    int first_in_a;               // the first segment of a split sequence runs in phase A (see launch_gdn_seg)
    Ckpt ck;
    void* o;
};

// ------------------------------------------------------------------ pass 1
struct StateBuf {
    alignas(16) uint16_t k[CH][LK];      // fp16
    alignas(16) uint16_t v[CH][LK];      // bf16
    alignas(16) uint16_t t[CH][LP];      // T diag(beta), fp16, scaled
    alignas(16) float eg[CH];
    alignas(16) float dec[CH];
    float gamma;
    float tinv;
};

// Pass 1 for split segment j of head h (block work item bid = j * H + h).
__device__ __forceinline__ void seg_state_body(StateBuf (&buf)[2], int bid, const SegArgs& a) {
    const int H = a.H;
    const int h = bid % H;
    const int j = bid / H;
    if (j >= a.split_off[a.n_seqs]) return;
    const int b = find_span_owner(a.split_off, a.n_seqs, j);
    const int g = j - a.split_off[b];
    GSeg sg;
    if (!seg_bounds(sg, b, g, a.seg_off[b + 1] - a.seg_off[b], a.cu, a.n_tokens, a.coff, a.split_off, a.slot_idx,
                    a.n_slots, a.lseg, a.nsplit_max))
        return;
    const int nch = (sg.t1 - sg.t0 + CH - 1) / CH;
    if (sg.ci0 < 0 || sg.ci0 + nch > a.n_chunks_max) return;     // malformed cu_seqlens only

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const AccPos ap;
    const int col = wave * 16;

    // [S | M] from [0 | I]: this wave's columns of both
    f32x4 S[8], M[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
        S[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r) M[mt][r] = (mt * 16 + ap.row0 + r == col + ap.col) ? 1.f : 0.f;
    }
    float sigma = 1.f;          // [S | M] = sigma [Shat | Mhat]

    auto rows = [&](int c) { return c < nch ? min(CH, sg.t1 - sg.t0 - c * CH) : 0; };
    auto tok = [&](int c) { return static_cast<long>(sg.t0) + static_cast<long>(c < nch ? c : 0) * CH; };
    GPrefetch<false, true> pf;
    const SegSrc src = seg_src<false, true>(nullptr, a.k, a.v, a.alpha, a.planes, a.tinv, sg.t0, sg.t1 - sg.t0, sg.ci0,
                                            nch, h, H);
    auto fetch = [&](int c) { g_fetch(pf, src, c, rows(c)); };
    auto stage = [&](StateBuf& bb) {
        g_stage_gates(nullptr, bb.eg, bb.dec, &bb.gamma, pf);
        g_stage_tile<true>(&bb.k[0][0], LK, pf.k);
        g_stage_tile<false>(&bb.v[0][0], LK, pf.v);
        g_stage_plane(bb.t, pf.t);
        if (threadIdx.x == 0) bb.tinv = pf.tinv;
    };
    fetch(0);
    stage(buf[0]);
    fetch(1);
    lds_barrier();
    for (int c = 0; c < nch; ++c) {
        const StateBuf& bb = buf[c & 1];
        bf16x8 vf[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) vf[ks] = frag_km_split(&bb.v[0][0], LK, col, 32 * ks);
        // the segment's own state contribution S (with values) and its
        // transition M (no values: Y = -diag(eg) K M)
        bf16x8 sf[4], mf[4];
        const Scale ss = state_operand(sf, S);
        const Scale sm = state_operand(mf, M);
        f32x4 XS[4], XM[4];
        k_times_sm(XS, XM, sf, mf, &bb.k[0][0]);
        bf16x8 yf[2], un[2], sdf[2], mdf[2];
        const Scale sy = form_y<false>(yf, XS, vf, bb.eg, ss.inv * sigma);
        const Scale su = form_u<false>(un, sdf, yf, bb.t, bb.dec, bb.tinv * sy.inv);
        const Scale my = form_y<true>(yf, XM, vf, bb.eg, sm.inv * sigma);
        const Scale mu = form_u<false>(un, mdf, yf, bb.t, bb.dec, bb.tinv * my.inv);
        state_update_sm(S, M, &bb.k[0][0], uniform_f(bb.gamma), sdf, su.inv, mdf, mu.inv, sigma);
        stage(buf[(c + 1) & 1]);
        fetch(c + 2);
        lds_barrier();
    }
    const long slot = (sg.jsplit + g) * H + h;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
        S[mt] *= sigma;
        M[mt] *= sigma;
    }
    g_slot_store(g_slot(a.wsS, slot), S);
    // M[16 mt + row0 + r][col + ap.col] -> row block mt, column k = col + ap.col
    // (s = wave / 2, h2 = wave % 2), fragment lane row0 + r + 16 (ap.col / 4)
    float* mfr = a.wsM + slot * D * D;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            mfr[g_mfrag(mt, wave >> 1, wave & 1, ap.row0 + r + 16 * (ap.col >> 2)) + (ap.col & 3)] = M[mt][r];
}

// ------------------------------------------------------------------ scan
// Per (split sequence, head): S_in(j + 1) = M_j S_in(j) + dS_j over the split
// segments, from S_in(1) in the sequence's first split slot when phase A ran
// the first segment (from_first), else from S_in(0) = the pool state (or
// 0), which also goes to the sequence's slot in wsI.  The state's columns
// are independent, so
// kScanGroups workgroups share a (sequence, head), each with kScanCols
// 16-column blocks, at equal blockIdx % 8 (one XCD, so M_j is fetched into
// one L2).  Wave w forms rows 16 w .. 16 w + 15 of its workgroup's blocks:
// its A operand, rows of M_j, is read from the fragment-major slot into
// registers two steps ahead and serves every block; the B operands, the
// blocks' S_in(j), go round through LDS, one barrier a step.  Every
// workgroup reads all of M_j each step: wider workgroups move fewer bytes
// from L2 and lengthen each step's LDS reads and MFMA chains.
// The products take bf16 hi + lo pairs (three MFMAs per 32-deep block).
// S_in(j + 1) overwrites dS_j (each word by the lane that read it).
// kScanCols: 16-column blocks per workgroup (1 or 2, the latter when there
// are many (sequence, head) pairs; kScanGroups = 8 / kScanCols workgroups
// per pair).
template <int kScanCols>
__global__ void __launch_bounds__(NTH)
gdn_seg_scan(int n_seqs, int H, const float* __restrict__ pool, int n_slots, const int32_t* __restrict__ slot_idx,
             int zero_init, const int32_t* __restrict__ split_off, long nsplit_max, float* __restrict__ wsS,
             const float* __restrict__ wsM, float* __restrict__ wsI, int from_first) {
    constexpr int kScanGroups = 8 / kScanCols;
    const int x = blockIdx.x;
    const int part = (x >> 3) % kScanGroups;         // which kScanCols column blocks
    const long grp = static_cast<long>(x / (8 * kScanGroups)) * 8 + (x & 7);   // split segment * H + head
    if (grp >= nsplit_max * H) return;
    const int h = static_cast<int>(grp % H);
    const int j = static_cast<int>(grp / H);
    if (j >= split_off[n_seqs]) return;
    const int b = find_span_owner(split_off, n_seqs, j);
    if (j != split_off[b]) return;                  // the first split segment stands for the sequence
    const int nsplit = split_off[b + 1] - split_off[b];
    if (static_cast<long>(j) + nsplit > nsplit_max) return;      // malformed cu_seqlens only
    const int slot = slot_idx[b];
    if (slot < 0 || slot >= n_slots) return;        // a sequence skipped by the passes
    const int s0 = from_first ? 1 : 0;              // the first split segment stepped over
    const int nsteps = nsplit - s0;
    if (nsteps <= 0) return;

    __shared__ f32x4 xs[2][kScanCols][NWV][64];      // S_in by column block and row block
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const AccPos ap;
    // this lane's words of a state slot in column block c of the workgroup
    auto lofs = [&](int c) { return g_tile(part * kScanCols + c, wave, lane); };
    f32x4 S[kScanCols];
    if (from_first) {
        const float* s1 = wsS + (static_cast<long>(j) * H + h) * D * D;
#pragma unroll
        for (int c = 0; c < kScanCols; ++c) S[c] = *reinterpret_cast<const f32x4*>(s1 + lofs(c));
    } else {
        // position 16 wave + row0 + r of the pair-order slot is state row srow(wave, row0) + r
        const float* src = pool + (static_cast<long>(slot) * H + h) * D * D;
        float* si = wsI + (static_cast<long>(j) * H + h) * D * D;
#pragma unroll
        for (int c = 0; c < kScanCols; ++c) {
            S[c] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (!zero_init) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    S[c][r] = src[(srow(wave, ap.row0) + r) * D + (part * kScanCols + c) * 16 + ap.col];
            }
            *reinterpret_cast<f32x4*>(si + lofs(c)) = S[c];
        }
    }

    // M_j row 16 wave + lane % 16 at columns 32 s + 4 g + (0..3) and
    // 32 s + 16 + 4 g + (0..3): the split order of the B operand's tile pairs
    struct Pf {
        f32x4 m[8];
        f32x4 d[kScanCols];
    };
    // step s is split segment j + s0 + s
    auto load = [&](Pf& p, int step) {
        const long sl = (static_cast<long>(j) + s0 + step) * H + h;
        const float* mp = wsM + sl * D * D;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            p.m[2 * s] = *reinterpret_cast<const f32x4*>(mp + g_mfrag(wave, s, 0, lane));
            p.m[2 * s + 1] = *reinterpret_cast<const f32x4*>(mp + g_mfrag(wave, s, 1, lane));
        }
#pragma unroll
        for (int c = 0; c < kScanCols; ++c) p.d[c] = *reinterpret_cast<const f32x4*>(wsS + sl * D * D + lofs(c));
        __builtin_amdgcn_sched_barrier(0);     // sets complete in the order they were issued
    };
    auto run = [&](const Pf& p, int step) {
        // fences keep the scheduler from converting a later step's M early,
        // which would wait for the loads issued for that step
        __builtin_amdgcn_sched_barrier(0);
        const int buf = step & 1;       // LDS buffers alternate, so one barrier a step suffices
#pragma unroll
        for (int c = 0; c < kScanCols; ++c) xs[buf][c][wave][lane] = S[c];
        lds_barrier();
        f32x4 acc[kScanCols];
#pragma unroll
        for (int c = 0; c < kScanCols; ++c) acc[c] = p.d[c];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 ah, al;
            split_pair(p.m[2 * s], p.m[2 * s + 1], ah, al);
#pragma unroll
            for (int c = 0; c < kScanCols; ++c) {
                bf16x8 bh, bl;
                split_pair(xs[buf][c][2 * s][lane], xs[buf][c][2 * s + 1][lane], bh, bl);
                acc[c] = mfma_bf16(ah, bh, acc[c]);
                acc[c] = mfma_bf16(ah, bl, acc[c]);
                acc[c] = mfma_bf16(al, bh, acc[c]);
            }
        }
        float* dst = wsS + ((static_cast<long>(j) + s0 + step) * H + h) * D * D;
#pragma unroll
        for (int c = 0; c < kScanCols; ++c) {
            S[c] = acc[c];
            *reinterpret_cast<f32x4*>(dst + lofs(c)) = S[c];
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // three register sets, each reloaded right after use (a clamped step
    // instead of a branch past the end); the loop body has a single path,
    // so the load-counter wait before each step covers only that step's set
    Pf pa, pb, pc;
    load(pa, 0);
    load(pb, min(1, nsteps - 1));
    load(pc, min(2, nsteps - 1));
    int step = 0;
    for (; step + 2 < nsteps; step += 3) {
        run(pa, step);
        load(pa, min(step + 3, nsteps - 1));
        run(pb, step + 1);
        load(pb, min(step + 4, nsteps - 1));
        run(pc, step + 2);
        load(pc, min(step + 5, nsteps - 1));
    }
    if (step < nsteps) run(pa, step);
    if (step + 1 < nsteps) run(pb, step + 1);
}

// ------------------------------------------------------------------ pass 2
struct KGate {
    alignas(16) uint16_t k[CH][LK];      // fp16
    alignas(16) float g2[CH];
    alignas(16) float eg[CH];
    alignas(16) float dec[CH];
    float gamma;
    float tinv;
};

struct OutSmem {
    KGate kb[2];
    alignas(16) uint16_t sq[CH][LQ];      // fp16
    alignas(16) uint16_t sv[CH][LK];      // bf16
    alignas(16) uint16_t st[CH][LP];      // T diag(beta), fp16, scaled
    alignas(16) uint16_t sp[CH][LP];      // P, fp16
    alignas(16) uint16_t obuf[CH][LO];    // bf16 outputs of the previous chunk
};

// Which segments a pass-2 call takes: those of sequences that are not cut
// (the pool in and out), the first segment of a cut sequence run in phase A
// (the pool in, its end state out to the workspace slot the scan starts
// from), or the segments of a cut sequence after the scan (its entry state
// in, the pool out after the last one; the first segment among them when it
// did not run in phase A).
enum SegMode { kWhole = 0, kFirst = 1, kLater = 2 };

// Pass 2 for segment si of head h (bid = si * H + h) if it is of kind MODE.
template <class TO, bool CKPT, int MODE>
__device__ __forceinline__ void seg_out_body(OutSmem& sm, int bid, const SegArgs& a) {
    const int H = a.H;
    const int h = bid % H;
    const int si = bid / H;
    if (si >= a.seg_off[a.n_seqs]) return;
    const int b = find_span_owner(a.seg_off, a.n_seqs, si);
    const int g = si - a.seg_off[b];
    const int nseg = a.seg_off[b + 1] - a.seg_off[b];
    const int mode = nseg <= 1 ? kWhole : (g == 0 && a.first_in_a ? kFirst : kLater);
    if (mode != MODE) return;
    GSeg sg;
    if (!seg_bounds(sg, b, g, nseg, a.cu, a.n_tokens, a.coff, a.split_off, a.slot_idx, a.n_slots, a.lseg,
                    a.nsplit_max))
        return;
    const int nch = (sg.t1 - sg.t0 + CH - 1) / CH;
    if (sg.ci0 < 0 || sg.ci0 + nch > a.n_chunks_max) return;     // malformed cu_seqlens only
    const int lseg = a.lseg;
    const int n_slots = a.n_slots;
    const Ckpt ck = a.ck;
    float* pool = a.pool;
    typename TO::T* o = static_cast<typename TO::T*>(a.o);
    KGate (&kb)[2] = sm.kb;
    uint16_t (&sq)[CH][LQ] = sm.sq;
    uint16_t (&sv)[CH][LK] = sm.sv;
    uint16_t (&st)[CH][LP] = sm.st;
    uint16_t (&sp)[CH][LP] = sm.sp;
    uint16_t (&obuf)[CH][LO] = sm.obuf;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const AccPos ap;
    const int col = wave * 16;
    const long stride = static_cast<long>(H) * D;

    auto rows = [&](int c) { return c < nch ? min(CH, sg.t1 - sg.t0 - c * CH) : 0; };
    auto tok = [&](int c) { return static_cast<long>(sg.t0) + static_cast<long>(c < nch ? c : 0) * CH; };
    GPrefetch<true, true> pf;
    const SegSrc src = seg_src<true, true>(a.q, a.k, a.v, a.alpha, a.planes, a.tinv, sg.t0, sg.t1 - sg.t0, sg.ci0,
                                           nch, h, H);
    auto fetch = [&](int c) { g_fetch(pf, src, c, rows(c)); };
    fetch(0);

    // entry state, held as S = sigma Shat (fold_scale)
    f32x4 S[8];
    float sigma = 1.f;
    float* Sg = pool + (static_cast<long>(sg.slot) * H + h) * D * D;
    if (MODE != kLater) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) S[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (!a.zero_init) g_rowmajor_load(S, Sg, col);
    } else {
        const float* src = g == 0 ? g_slot(a.wsI, sg.jsplit * H + h) : g_slot(a.wsS, (sg.jsplit + g - 1) * H + h);
        g_slot_load(S, src);
    }
    // P tiles above the diagonal that the products still read (rows 0-15 x
    // keys 16-31, rows 32-47 x keys 48-63) stay zero
    for (int idx = tid; idx < 2 * 256; idx += NTH) {
        const int t = idx >> 8, e = idx & 255;
        const int row = (t ? 32 : 0) + (e >> 4), cx = p_col(t ? 3 : 1, (e >> 2) & 3) + (e & 3);
        sp[row][cx] = 0;
    }
    auto stage = [&](KGate& kk) {
        g_stage_gates(kk.g2, kk.eg, kk.dec, &kk.gamma, pf);
        g_stage_tile<true>(&kk.k[0][0], LK, pf.k);
        g_stage_tile<true>(&sq[0][0], LQ, pf.q);
        g_stage_tile<false>(&sv[0][0], LK, pf.v);
        g_stage_plane(st, pf.t);
        if (threadIdx.x == 0) kk.tinv = pf.tinv;
    };
    stage(kb[0]);
    fetch(1);
    lds_barrier();

    // P tile t of (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) (3,1) (3,2) (3,3)
    auto p_tile = [&](const KGate& kk, int t) {
        const int it = t < 1 ? 0 : (t < 3 ? 1 : (t < 6 ? 2 : 3));
        const int jt = t - it * (it + 1) / 2;
        f32x4 pt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
            pt = mfma_f16(frag_kc(&kk.k[0][0], LK, jt * 16, 32 * ks), frag_kc(&sq[0][0], LQ, it * 16, 32 * ks), pt);
        const int i = it * 16 + ap.col;
        const float gi = kk.g2[i];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int jj = jt * 16 + ap.row0 + r;
            pt[r] = (jj <= i) ? pt[r] * hw_exp2(gi - kk.g2[jj]) : 0.f;
        }
        *reinterpret_cast<u32x2*>(&sp[i][p_col(jt, ap.row0 >> 2)]) = u32x2{pk_f16(pt[0], pt[1]), pk_f16(pt[2], pt[3])};
    };
    // chunk cc's bf16 outputs: LDS -> HBM, 16 lanes per 256-byte row
    auto flush_o = [&](int cc) {
        if constexpr (TO::bytes == 2) {
            const BufRsrc ro(o + tok(cc) * stride + h * D, rows_extent(rows(cc), stride * 2, D * 2));
#pragma unroll
            for (int u = 0; u < CH * D / 8 / NTH; ++u) {
                const int x = tid + u * NTH, row = x / (D / 8), vc = (x % (D / 8)) * 8;
                ro.store_b128(*reinterpret_cast<const u32x4*>(&obuf[row][vc]),
                              static_cast<uint32_t>((row * stride + vc) * 2));
            }
        }
    };

    for (int c = 0; c < nch; ++c) {
        const KGate& kk = kb[c & 1];
        const int n = rows(c);
        const long tok0 = tok(c);
        if (c > 0) flush_o(c - 1);

        // ---- phase 1: P tiles -> LDS; X = K S, O^T = S^T Q^T; Y; U
        p_tile(kk, wave);
        if (wave + NWV < 10) p_tile(kk, wave + NWV);
        bf16x8 sf[4];
        const Scale ss = state_operand(sf, S);
        f32x4 X[4], ot[4];
        k_times_s<true>(X, ot, sf, &kk.k[0][0], &sq[0][0]);
        bf16x8 vf[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) vf[ks] = frag_km_split(&sv[0][0], LK, col, 32 * ks);
        bf16x8 yf[2], uf[2], df[2];
        const Scale sy = form_y<false>(yf, X, vf, kk.eg, ss.inv * sigma);
        const Scale su = form_u(uf, df, yf, st, kk.dec, kk.tinv * sy.inv);
#pragma unroll
        for (int it = 0; it < 4; ++it) ot[it] *= kk.eg[it * 16 + ap.col] * (ss.inv * sigma);
        lds_barrier();

        // ---- phase 2: O^T += U^T P^T; outputs; state update; next chunk
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            f32x4 pu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks <= (it >> 1); ++ks) pu = mfma_f16(uf[ks], frag_kc(&sp[0][0], LP, it * 16, 32 * ks), pu);
            ot[it] += su.inv * pu;
        }
        // lane: token it*16 + (lane % 16), columns col + 4 (lane / 16) .. +3
        if constexpr (TO::bytes == 2) {
#pragma unroll
            for (int it = 0; it < 4; ++it)
                *reinterpret_cast<u32x2*>(&obuf[it * 16 + ap.col][col + ap.row0]) =
                    u32x2{pack_bf16x2(ot[it][0], ot[it][1]), pack_bf16x2(ot[it][2], ot[it][3])};
        } else {
            const BufRsrc ro(o + tok0 * stride + h * D, rows_extent(n, stride * 4, D * 4));
#pragma unroll
            for (int it = 0; it < 4; ++it)
                ro.store_b128(__builtin_bit_cast(u32x4, ot[it]),
                              static_cast<uint32_t>(((it * 16 + ap.col) * stride + col + ap.row0) * 4));
        }
        state_update<true>(S, &kk.k[0][0], uniform_f(kk.gamma), df, su.inv, sigma);
        stage(kb[(c + 1) & 1]);
        fetch(c + 2);
        // checkpoint: this wave's columns of the state after chunk c
        const int cs = CKPT && n == CH ? ckpt_slot(ck, sg.b, sg.g * lseg + (c + 1) * CH, n_slots) : -1;
        if (CKPT && cs >= 0) {
            float* Sc = pool + (static_cast<long>(cs) * H + h) * D * D + opaque(2 * ap.row0 * D + col + ap.col);
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
                for (int r = 0; r < 4; ++r) Sc[(srow(mt, 0) + r) * D] = S[mt][r] * sigma;
            }
        }
        lds_barrier();
    }
    if (nch > 0) flush_o(nch - 1);

    if (MODE == kFirst) {
        // S_in of the second segment, where the scan starts
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) S[mt] *= sigma;
        g_slot_store(g_slot(a.wsS, sg.jsplit * H + h), S);
    } else if (sg.g == sg.nseg - 1) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) Sg[(srow(mt, ap.row0) + r) * D + col + ap.col] = S[mt][r] * sigma;
        }
    }
}

// Pass 2 for batches of short prompts: `items` heads h0 .. h0 + items - 1
// (items divides H) of one unsplit sequence's segment (bid0 = segment * H +
// h0), their chunks one stream, item after item, so the next head's loads
// are in flight while the current head's last chunk runs.  Between heads
// the final state of one goes to the pool through buffer stores with scalar
// row offsets.  The output flush and the state stores are issued on every
// path (empty ranges where there is nothing to write), so that the loop's
// load-counter waits for the prefetched rows leave younger stores in flight.
template <class TO, bool ZERO>
__device__ __forceinline__ void seg_out_multi(OutSmem& sm, int bid0, int items, const SegArgs& a) {
    const int H = a.H;
    const int h0 = bid0 % H;
    const int si = bid0 / H;
    if (si >= a.seg_off[a.n_seqs]) return;
    const int b = find_span_owner(a.seg_off, a.n_seqs, si);
    const int g = si - a.seg_off[b];
    const int nseg = a.seg_off[b + 1] - a.seg_off[b];
    if (nseg > 1) return;
    GSeg sg;
    if (!seg_bounds(sg, b, g, nseg, a.cu, a.n_tokens, a.coff, a.split_off, a.slot_idx, a.n_slots, a.lseg,
                    a.nsplit_max))
        return;
    const int nch = (sg.t1 - sg.t0 + CH - 1) / CH;
    if (sg.ci0 < 0 || sg.ci0 + nch > a.n_chunks_max) return;     // malformed cu_seqlens only
    float* pool = a.pool;
    typename TO::T* o = static_cast<typename TO::T*>(a.o);
    KGate (&kb)[2] = sm.kb;
    uint16_t (&sq)[CH][LQ] = sm.sq;
    uint16_t (&sv)[CH][LK] = sm.sv;
    uint16_t (&st)[CH][LP] = sm.st;
    uint16_t (&sp)[CH][LP] = sm.sp;
    uint16_t (&obuf)[CH][LO] = sm.obuf;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const AccPos ap;
    const int col = wave * 16;
    const long stride = static_cast<long>(H) * D;

    auto rows = [&](int c) { return c < nch ? min(CH, sg.t1 - sg.t0 - c * CH) : 0; };
    auto tok = [&](int c) { return static_cast<long>(sg.t0) + static_cast<long>(c < nch ? c : 0) * CH; };
    GPrefetch<true, true> pf;
    // chunk c of item it (nothing past the last item: a chunk past the end)
    auto fetch = [&](int c, int it) {
        const SegSrc src = seg_src<true, true>(a.q, a.k, a.v, a.alpha, a.planes, a.tinv, sg.t0, sg.t1 - sg.t0,
                                               sg.ci0, nch, h0 + min(it, items - 1), H);
        const int cc = it < items ? c : nch;
        g_fetch(pf, src, cc, rows(cc));
    };
    // the position `ahead` chunks after chunk c of item it
    auto step = [&](int c, int it, int ahead, int& c2, int& it2) {
        c2 = c + ahead;
        it2 = it;
        if (nch <= 0) {
            c2 = 0;
            it2 = items;
            return;
        }
        while (c2 >= nch) {
            c2 -= nch;
            ++it2;
        }
    };
    fetch(0, 0);

    // pool states through buffer resources: the lane's offset in one
    // register, each of its 32 rows a scalar offset
    const uint32_t lane_off = static_cast<uint32_t>((2 * ap.row0 * D + col + ap.col) * 4);
    auto pool_state = [&](int it, bool live) {
        return BufRsrc(pool + (static_cast<long>(sg.slot) * H + h0 + it) * D * D, live ? D * D * 4 : 0u);
    };
    f32x4 S[8];
    float sigma = 1.f;           // the update here keeps S itself (no running scale)
    auto entry = [&](int it) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) S[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (!ZERO) {
            const BufRsrc rs = pool_state(it, true);
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) S[mt][r] = rs.loadf(lane_off, (srow(mt, 0) + r) * D * 4);
        }
    };
    auto final_state = [&](int it, bool live) {
        const BufRsrc rs = pool_state(it, live);
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) rs.storef(S[mt][r], lane_off, (srow(mt, 0) + r) * D * 4);
    };
    entry(0);
    if (nch == 0) {
        // empty sequence: every head's state goes back as it came in
        for (int it = 0; it < items; ++it) {
            if (it > 0) entry(it);
            final_state(it, true);
        }
        return;
    }
    // P tiles above the diagonal that the products still read (rows 0-15 x
    // keys 16-31, rows 32-47 x keys 48-63) stay zero
    for (int idx = tid; idx < 2 * 256; idx += NTH) {
        const int t = idx >> 8, e = idx & 255;
        const int row = (t ? 32 : 0) + (e >> 4), cx = p_col(t ? 3 : 1, (e >> 2) & 3) + (e & 3);
        sp[row][cx] = 0;
    }
    auto stage = [&](KGate& kk) {
        g_stage_gates(kk.g2, kk.eg, kk.dec, &kk.gamma, pf);
        g_stage_tile<true>(&kk.k[0][0], LK, pf.k);
        g_stage_tile<true>(&sq[0][0], LQ, pf.q);
        g_stage_tile<false>(&sv[0][0], LK, pf.v);
        g_stage_plane(st, pf.t);
        if (threadIdx.x == 0) kk.tinv = pf.tinv;
    };
    stage(kb[0]);
    {
        int c1, i1;
        step(0, 0, 1, c1, i1);
        fetch(c1, i1);
    }
    lds_barrier();

    auto p_tile = [&](const KGate& kk, int t) {
        const int it = t < 1 ? 0 : (t < 3 ? 1 : (t < 6 ? 2 : 3));
        const int jt = t - it * (it + 1) / 2;
        f32x4 pt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
            pt = mfma_f16(frag_kc(&kk.k[0][0], LK, jt * 16, 32 * ks), frag_kc(&sq[0][0], LQ, it * 16, 32 * ks), pt);
        const int i = it * 16 + ap.col;
        const float gi = kk.g2[i];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int jj = jt * 16 + ap.row0 + r;
            pt[r] = (jj <= i) ? pt[r] * hw_exp2(gi - kk.g2[jj]) : 0.f;
        }
        *reinterpret_cast<u32x2*>(&sp[i][p_col(jt, ap.row0 >> 2)]) = u32x2{pk_f16(pt[0], pt[1]), pk_f16(pt[2], pt[3])};
    };
    // bf16 outputs of chunk cc of item it: LDS -> HBM, 16 lanes per 256-byte row
    auto flush_o = [&](int cc, int it, bool live) {
        if constexpr (TO::bytes == 2) {
            const BufRsrc ro(o + tok(cc) * stride + (h0 + it) * D,
                             live ? rows_extent(rows(cc), stride * 2, D * 2) : 0u);
#pragma unroll
            for (int u = 0; u < CH * D / 8 / NTH; ++u) {
                const int x = tid + u * NTH, row = x / (D / 8), vc = (x % (D / 8)) * 8;
                ro.store_b128(*reinterpret_cast<const u32x4*>(&obuf[row][vc]),
                              static_cast<uint32_t>((row * stride + vc) * 2));
            }
        }
    };

    const int total = items * nch;
    int c = 0, item = 0;              // chunk and item of stream position vc
    int pc = 0, pitem = 0;            // those of the position before
    for (int vc = 0; vc < total; ++vc) {
        const KGate& kk = kb[vc & 1];
        const int n = rows(c);
        const long tok0 = tok(c);
        const int hk = h0 + item;
        flush_o(pc, pitem, vc > 0);

        // ---- phase 1: P tiles -> LDS; X = K S, O^T = S^T Q^T; Y; U
        p_tile(kk, wave);
        if (wave + NWV < 10) p_tile(kk, wave + NWV);
        bf16x8 sf[4];
        const Scale ss = state_operand(sf, S);
        f32x4 X[4], ot[4];
        k_times_s<true>(X, ot, sf, &kk.k[0][0], &sq[0][0]);
        bf16x8 vf[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) vf[ks] = frag_km_split(&sv[0][0], LK, col, 32 * ks);
        bf16x8 yf[2], uf[2], df[2];
        const Scale sy = form_y<false>(yf, X, vf, kk.eg, ss.inv * sigma);
        const Scale su = form_u(uf, df, yf, st, kk.dec, kk.tinv * sy.inv);
#pragma unroll
        for (int it = 0; it < 4; ++it) ot[it] *= kk.eg[it * 16 + ap.col] * (ss.inv * sigma);
        lds_barrier();

        // ---- phase 2: O^T += U^T P^T; outputs; state update; next chunk
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            f32x4 pu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks <= (it >> 1); ++ks) pu = mfma_f16(uf[ks], frag_kc(&sp[0][0], LP, it * 16, 32 * ks), pu);
            ot[it] += su.inv * pu;
        }
        if constexpr (TO::bytes == 2) {
#pragma unroll
            for (int it = 0; it < 4; ++it)
                *reinterpret_cast<u32x2*>(&obuf[it * 16 + ap.col][col + ap.row0]) =
                    u32x2{pack_bf16x2(ot[it][0], ot[it][1]), pack_bf16x2(ot[it][2], ot[it][3])};
        } else {
            const BufRsrc ro(o + tok0 * stride + hk * D, rows_extent(n, stride * 4, D * 4));
#pragma unroll
            for (int it = 0; it < 4; ++it)
                ro.store_b128(__builtin_bit_cast(u32x4, ot[it]),
                              static_cast<uint32_t>(((it * 16 + ap.col) * stride + col + ap.row0) * 4));
        }
        state_update<false>(S, &kk.k[0][0], kk.gamma, df, su.inv, sigma);
        stage(kb[(vc + 1) & 1]);
        {
            int c2, i2;
            step(c, item, 2, c2, i2);
            fetch(c2, i2);
        }
        // between heads: this head's final state out, the next head's entry
        // state in (zeros with ZERO, which then waits for nothing; loaded
        // otherwise, and used here so that the wait for it falls in this
        // chunk, not at the top of the loop)
        const bool item_end = c == nch - 1;
        final_state(item, item_end);
        if (item_end && item + 1 < items) entry(item + 1);
        if constexpr (!ZERO) {
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
                asm volatile("" ::"v"(S[mt][0]), "v"(S[mt][1]), "v"(S[mt][2]), "v"(S[mt][3]));
        }
        pc = c;
        pitem = item;
        if (item_end) {
            c = 0;
            ++item;
        } else {
            ++c;
        }
        lds_barrier();
    }
    flush_o(pc, pitem, true);
}

union SegSmem {
    StateBuf st[2];
    OutSmem out;
};

// Phase A block bid < n1: split segment j = bid / H (every segment but the
// last of a cut sequence).  With first_in_a, the first segment of a cut
// sequence, which needs no transition (its entry state is the pool's), runs
// pass 2 here and its end state seeds the scan; the others run pass 1.
template <class TO, bool CKPT>
__device__ __forceinline__ void phase_a_split(SegSmem& sm, int bid, const SegArgs& a) {
    const int j = bid / a.H;
    if (j >= a.split_off[a.n_seqs]) return;
    const int b = find_span_owner(a.split_off, a.n_seqs, j);
    if (a.first_in_a && j == a.split_off[b])
        seg_out_body<TO, CKPT, kFirst>(sm.out, a.seg_off[b] * a.H + bid % a.H, a);
    else
        seg_state_body(sm.st, bid, a);
}

// Phase A: the split segments (blocks [0, n1)), which the scan waits for,
// and next to them pass 2 for sequences that are not split, which depend
// on nothing else (blocks [n1, ...)).
template <class TO, bool CKPT>
__global__ void __launch_bounds__(NTH)
gdn_seg_a(SegArgs a, int n1) {
    __shared__ SegSmem sm;
    if (static_cast<int>(blockIdx.x) < n1) phase_a_split<TO, CKPT>(sm, blockIdx.x, a);
    else seg_out_body<TO, CKPT, kWhole>(sm.out, blockIdx.x - n1, a);
}

// Phase A for batches of short prompts: the split segments as above, and
// pass 2 for unsplit sequences with `items` heads per block.
template <class TO, bool ZERO>
__global__ void __launch_bounds__(NTH)
gdn_seg_a_multi(SegArgs a, int n1, int items) {
    __shared__ SegSmem sm;
    if (static_cast<int>(blockIdx.x) < n1) phase_a_split<TO, false>(sm, blockIdx.x, a);
    else seg_out_multi<TO, ZERO>(sm.out, (blockIdx.x - n1) * items, items, a);
}

// Phase B (after the scan): pass 2 for the segments of split sequences
// that phase A did not run (a batch of short prompts launches no idle
// blocks here).  With first_in_a, block j is split segment j / H, whose
// i-th of a sequence stands for its segment i + 1; otherwise block j is
// segment j / H of the split sequences' concatenated segment lists.
template <class TO, bool CKPT>
__global__ void __launch_bounds__(NTH)
gdn_seg_b(SegArgs a) {
    __shared__ SegSmem sm;
    const int h = blockIdx.x % a.H;
    const int j = blockIdx.x / a.H;
    const int32_t* off = a.first_in_a ? a.split_off : a.splitseg_off;
    if (j >= off[a.n_seqs]) return;
    const int b = find_span_owner(off, a.n_seqs, j);
    const int si = a.seg_off[b] + (j - off[b]) + (a.first_in_a ? 1 : 0);
    seg_out_body<TO, CKPT, kLater>(sm.out, si * a.H + h, a);
}

// Segment length: whole chunks, at least 4 of them, such that the call
// has about kTargetBlocks (segment, head) workgroups when it is long enough.
// With many (sequence, head) pairs the batch fills the GPU without cutting,
// and segments only bound the longest chain: pass 1 of a split segment and
// pass 2 after the scan run one after the other, so the segments are made
// half as long (about 2 kTargetBlocks of them) to keep that path short.
int g_seg_len(int n_seqs, int n_tokens, int n_heads) {
    const long blocks = static_cast<long>(n_seqs) * n_heads >= 2 * kTargetBlocks ? 2 * kTargetBlocks : kTargetBlocks;
    const long target = n_heads >= blocks ? 1 : blocks / n_heads;
    long L = (n_tokens + target - 1) / target;
    L = ((L + CH - 1) / CH) * CH;
    return static_cast<int>(L < 4 * CH ? 4 * CH : L);
}

// Heads of one segment per phase-A pass-2 block: 1 unless the batch is
// short sequences (at most 4 chunks on average); then the largest divisor
// of H up to 16 that still launches at least kTargetBlocks such blocks.
int g_seg_items(int n_seqs, int n_tokens, int n_heads, long maxseg) {
    if (n_seqs <= 0 || static_cast<long>(n_tokens) > static_cast<long>(n_seqs) * 4 * CH) return 1;
    int best = 1;
    for (int k = 2; k <= 16 && k <= n_heads; ++k)
        if (n_heads % k == 0 && maxseg * n_heads / k >= kTargetBlocks) best = k;
    return best;
}

__host__ __device__ constexpr size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

// Workspace of the segmented path beyond the chunk offsets and T planes:
// segment offsets, split-segment offsets, offsets among the segments of
// split sequences, and three 64 KiB state slots per (split segment, head):
// dS (then S_in of the next segment), M and (at a sequence's first)
// S_in(0).  A sequence of s >= 2 segments is longer than (s - 1) * lseg
// tokens, so split segments number at most n_tokens / lseg.
size_t gdn_seg_workspace(int n_seqs, int n_tokens, int n_heads) {
    const long nsplit = n_tokens / g_seg_len(n_seqs, n_tokens, n_heads);
    return 3 * al256(sizeof(int32_t) * (n_seqs + 1)) +
           3 * static_cast<size_t>(nsplit) * n_heads * D * D * sizeof(float);
}

// The fp16 T planes take the first n_chunks_max * H * 8 KiB of the plane
// region; their inverse scales (one float per (chunk, head)) follow.
float* plane_scales(const uint16_t* planes, long n_chunks_max, int H) {
    return const_cast<float*>(reinterpret_cast<const float*>(planes + n_chunks_max * H * kPlaneElems));
}

// The chunk offsets (coff, ahead of gdn_seg_prep) and the segment,
// split-segment and split-sequence-segment offsets of launch_gdn_seg, in
// one launch.
hipError_t launch_gdn_seg_offsets(const ChunkArgs& a, int32_t* coff, void* seg_ws, hipStream_t s) {
    const int lseg = g_seg_len(a.n_seqs, a.n_tokens, a.n_heads);
    char* ws = static_cast<char*>(seg_ws);
    const size_t oa = al256(sizeof(int32_t) * (a.n_seqs + 1));
    int32_t* seg_off = reinterpret_cast<int32_t*>(ws);
    int32_t* split_off = reinterpret_cast<int32_t*>(ws + oa);
    int32_t* splitseg_off = reinterpret_cast<int32_t*>(ws + 2 * oa);
    const SpanScans sc{{SpanScan{CH, 0, 0, 0, coff}, SpanScan{lseg, 1, 0, 0, seg_off},
                        SpanScan{lseg, 0, 1, 0, split_off}, SpanScan{lseg, 0, 0, 2, splitseg_off}}};
    hipLaunchKernelGGL(span_offsets_multi, dim3(4), dim3(1024), 0, s, a.cu_seqlens, a.n_seqs, a.n_tokens, sc);
    return hipGetLastError();
}

hipError_t launch_gdn_seg_prep(const ChunkArgs& a, const int32_t* coff, uint16_t* planes, long n_chunks_max,
                               hipStream_t s) {
    const long groups = std::min<long>((n_chunks_max * a.n_heads + PW - 1) / PW, kPrepGroups);
    if (groups <= 0) return hipSuccess;
    hipLaunchKernelGGL(gdn_seg_prep, dim3(static_cast<unsigned>(groups)), dim3(PW * 64), 0, s,
                       static_cast<const uint16_t*>(a.k), a.alpha, a.beta, a.cu_seqlens, a.n_seqs, a.n_tokens,
                       a.n_heads, coff, planes, plane_scales(planes, n_chunks_max, a.n_heads));
    return hipGetLastError();
}

hipError_t launch_gdn_seg(const ChunkArgs& a, const int32_t* coff, const uint16_t* planes, long n_chunks_max,
                          void* seg_ws, hipStream_t s) {
    const int lseg = g_seg_len(a.n_seqs, a.n_tokens, a.n_heads);
    const long nsplit = a.n_tokens / lseg;
    const long maxseg = nsplit + a.n_seqs;
    char* ws = static_cast<char*>(seg_ws);
    int32_t* seg_off = reinterpret_cast<int32_t*>(ws);
    ws += al256(sizeof(int32_t) * (a.n_seqs + 1));
    int32_t* split_off = reinterpret_cast<int32_t*>(ws);
    ws += al256(sizeof(int32_t) * (a.n_seqs + 1));
    int32_t* splitseg_off = reinterpret_cast<int32_t*>(ws);
    ws += al256(sizeof(int32_t) * (a.n_seqs + 1));
    float* wsS = reinterpret_cast<float*>(ws);
    float* wsM = wsS + static_cast<size_t>(nsplit) * a.n_heads * D * D;
    float* wsI = wsM + static_cast<size_t>(nsplit) * a.n_heads * D * D;
    // The first segment of a split sequence needs no pass 1 (its entry
    // state is the pool's): run in phase A as pass 2 it saves that work, but
    // puts a pass-2 chain (slower per chunk than pass 1) into phase A.  That
    // pays when the phases are throughput-bound (many (sequence, head) pairs,
    // more workgroups than compute units), not for a few long prompts, where
    // each phase is one segment's chain.
    const int first_in_a = static_cast<long>(a.n_seqs) * a.n_heads >= 2 * kTargetBlocks;
    const SegArgs sa{static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), a.alpha, a.cu_seqlens, a.n_seqs, a.n_tokens, a.n_heads,
                     a.pool, a.n_slots, a.slot_idx, a.zero_init, lseg, coff, seg_off, split_off, splitseg_off,
                     planes, plane_scales(planes, n_chunks_max, a.n_heads), n_chunks_max, nsplit, wsS, wsM, wsI,
                     first_in_a,
                     Ckpt{a.ckpt_slots, a.ckpt_interval, a.ckpt_stride}, a.o};
    const int n1 = static_cast<int>(nsplit * a.n_heads);
    const dim3 grid_a(static_cast<unsigned>(n1 + maxseg * a.n_heads));
    // phase B: with first_in_a the later segments of split sequences, one
    // per split segment (at most nsplit); otherwise all their segments (a
    // sequence of k >= 2 segments is longer than (k - 1) lseg tokens and
    // k <= 2 (k - 1): at most 2 nsplit)
    const dim3 grid_b(static_cast<unsigned>((first_in_a ? nsplit : std::min(maxseg, 2 * nsplit)) * a.n_heads));
    // several heads per block for batches of short prompts (no checkpoints)
    const int items = sa.ck.slots ? 1 : g_seg_items(a.n_seqs, a.n_tokens, a.n_heads, maxseg);
    auto passes = [&](auto ka, auto kb) {
        if (items > 1) {
            const dim3 grid_m(static_cast<unsigned>(n1 + maxseg * a.n_heads / items));
            auto multi = [&](auto kern) { hipLaunchKernelGGL(kern, grid_m, dim3(NTH), 0, s, sa, n1, items); };
            if (a.zero_init) {
                if (a.out_bf16) multi(gdn_seg_a_multi<BF16, true>);
                else multi(gdn_seg_a_multi<F32, true>);
            } else {
                if (a.out_bf16) multi(gdn_seg_a_multi<BF16, false>);
                else multi(gdn_seg_a_multi<F32, false>);
            }
        } else {
            hipLaunchKernelGGL(ka, grid_a, dim3(NTH), 0, s, sa, n1);
        }
        if (nsplit > 0) {
            // one column block per scan workgroup while that leaves the GPU
            // mostly idle, two once there are many (sequence, head) pairs
            auto scan = [&](auto kern, int groups) {
                hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>((n1 + 7) / 8 * 8 * groups)), dim3(NTH), 0, s,
                                   a.n_seqs, a.n_heads, a.pool, a.n_slots, a.slot_idx, a.zero_init, split_off,
                                   nsplit, wsS, wsM, wsI, first_in_a);
            };
            if (static_cast<long>(a.n_seqs) * a.n_heads <= 32) scan(gdn_seg_scan<1>, 8);
            else scan(gdn_seg_scan<2>, 4);
            hipLaunchKernelGGL(kb, grid_b, dim3(NTH), 0, s, sa);
        }
    };
    if (sa.ck.slots) {
        if (a.out_bf16) passes(gdn_seg_a<BF16, true>, gdn_seg_b<BF16, true>);
        else passes(gdn_seg_a<F32, true>, gdn_seg_b<F32, true>);
    } else {
        if (a.out_bf16) passes(gdn_seg_a<BF16, false>, gdn_seg_b<BF16, false>);
        else passes(gdn_seg_a<F32, false>, gdn_seg_b<F32, false>);
    }
    return hipGetLastError();
}

}  // namespace gla
