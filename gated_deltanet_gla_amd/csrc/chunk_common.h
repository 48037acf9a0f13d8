// Building blocks of the chunked prefill kernels (GLA and Gated DeltaNet).
//
// MFMA operands are read from LDS matrices stored "k-contiguous": the
// element (line, k) of an operand sits at base[line * ld + k].  An A
// operand's lines are its rows, a B operand's lines are its columns (the
// matrix is kept transposed).  With that single convention every 16x16
// output tile is one call of mma() whatever the contraction.
//
// Two operand formats:
//  * bf16 inputs: matrices are bf16.  Inputs q, k, v are exact in bf16;
//    every fp32-derived operand (decay-masked scores, the state, decayed or
//    beta-scaled values, the inverse T, ...) is stored as a hi + lo pair of
//    bf16 matrices and contracted with two (or three) MFMAs, which keeps the
//    product accurate to about 2^-16 relative instead of bf16's 2^-8.
//  * fp32 inputs: matrices are fp32 and the 16x16x4 fp32 MFMA is used;
//    there is no lo part.
//
// Lines are padded by 16 bytes, so the 16 lines a ds_read_b128 wave touches
// start in 16 different 4-bank groups (no bank conflicts).
#pragma once

#include "common.h"

namespace gla {

template <bool F32> struct Op;

template <> struct Op<false> {               // bf16 operands
    using E = uint16_t;
    static constexpr int PAD = 8;
    static constexpr bool kHasLo = true;

    __device__ __forceinline__ static void mma(f32x4& acc, const E* A, int lda, const E* B, int ldb,
                                               int K) {
        const int lane = threadIdx.x & 63;
        const int line = lane & 15;
        const int grp = lane >> 4;
        const E* a = A + line * lda + grp * 8;
        const E* b = B + line * ldb + grp * 8;
        int k0 = 0;
        for (; k0 + 32 <= K; k0 += 32) {
            const u32x4 av = *reinterpret_cast<const u32x4*>(a + k0);
            const u32x4 bv = *reinterpret_cast<const u32x4*>(b + k0);
            acc = mfma_bf16(as_bf16x8(av), as_bf16x8(bv), acc);
        }
        if (k0 < K) {   // 16-wide tail: 16x16x16 MFMA, 4 k-values per lane
            typedef __attribute__((ext_vector_type(4))) short s16x4;
            const E* a4 = A + line * lda + k0 + grp * 4;
            const E* b4 = B + line * ldb + k0 + grp * 4;
            const u32x2 av = *reinterpret_cast<const u32x2*>(a4);
            const u32x2 bv = *reinterpret_cast<const u32x2*>(b4);
            acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, av),
                                                            __builtin_bit_cast(s16x4, bv), acc, 0, 0, 0);
        }
    }

    // Store 4 consecutive values (v.x..v.w at p[0..3]) as hi (+ lo).
    __device__ __forceinline__ static void store4(E* hi, E* lo, f32x4 v) {
        uint32_t h0, h1, l0, l1;
        split_bf16x2(v.x, v.y, h0, l0);
        split_bf16x2(v.z, v.w, h1, l1);
        *reinterpret_cast<u32x2*>(hi) = u32x2{h0, h1};
        *reinterpret_cast<u32x2*>(lo) = u32x2{l0, l1};
    }
    __device__ __forceinline__ static void store1(E* hi, E* lo, float x) {
        uint16_t h, l;
        split_bf16(x, h, l);
        *hi = h;
        *lo = l;
    }
    __device__ __forceinline__ static void store1_exact(E* p, float x) { *p = f32_to_bf16_bits(x); }
    __device__ __forceinline__ static float load1(const E* p) { return bf16_bits_to_f32(*p); }
};

template <> struct Op<true> {                // fp32 operands
    using E = float;
    static constexpr int PAD = 4;
    static constexpr bool kHasLo = false;

    __device__ __forceinline__ static void mma(f32x4& acc, const E* A, int lda, const E* B, int ldb,
                                               int K) {
        const int lane = threadIdx.x & 63;
        const int line = lane & 15;
        const int grp = lane >> 4;
        const E* a = A + line * lda + grp * 4;
        const E* b = B + line * ldb + grp * 4;
        for (int k0 = 0; k0 < K; k0 += 16) {
            const f32x4 av = *reinterpret_cast<const f32x4*>(a + k0);
            const f32x4 bv = *reinterpret_cast<const f32x4*>(b + k0);
            acc = mfma_f32(av.x, bv.x, acc);
            acc = mfma_f32(av.y, bv.y, acc);
            acc = mfma_f32(av.z, bv.z, acc);
            acc = mfma_f32(av.w, bv.w, acc);
        }
    }
    __device__ __forceinline__ static void store4(E* hi, E*, f32x4 v) {
        *reinterpret_cast<f32x4*>(hi) = v;
    }
    __device__ __forceinline__ static void store1(E* hi, E*, float x) { *hi = x; }
    __device__ __forceinline__ static void store1_exact(E* p, float x) { *p = x; }
    __device__ __forceinline__ static float load1(const E* p) { return *p; }
};

// acc += A_hi.B (+ A_lo.B): A fp32-derived (hi/lo), B exact.
template <bool F32>
__device__ __forceinline__ void mma_sx(f32x4& acc, const typename Op<F32>::E* Ahi,
                                       const typename Op<F32>::E* Alo, int lda,
                                       const typename Op<F32>::E* B, int ldb, int K) {
    Op<F32>::mma(acc, Ahi, lda, B, ldb, K);
    if constexpr (!F32) Op<F32>::mma(acc, Alo, lda, B, ldb, K);
}
// acc += A.B_hi (+ A.B_lo): A exact, B fp32-derived.
template <bool F32>
__device__ __forceinline__ void mma_xs(f32x4& acc, const typename Op<F32>::E* A, int lda,
                                       const typename Op<F32>::E* Bhi,
                                       const typename Op<F32>::E* Blo, int ldb, int K) {
    Op<F32>::mma(acc, A, lda, Bhi, ldb, K);
    if constexpr (!F32) Op<F32>::mma(acc, A, lda, Blo, ldb, K);
}
// acc += (A_hi + A_lo)(B_hi + B_lo) without the lo.lo term.
template <bool F32>
__device__ __forceinline__ void mma_ss(f32x4& acc, const typename Op<F32>::E* Ahi,
                                       const typename Op<F32>::E* Alo, int lda,
                                       const typename Op<F32>::E* Bhi,
                                       const typename Op<F32>::E* Blo, int ldb, int K) {
    Op<F32>::mma(acc, Ahi, lda, Bhi, ldb, K);
    if constexpr (!F32) {
        Op<F32>::mma(acc, Ahi, lda, Blo, ldb, K);
        Op<F32>::mma(acc, Alo, lda, Bhi, ldb, K);
    }
}

// Lane position inside a 16x16 accumulator tile: column (lane % 16), rows
// 4 * (lane / 16) + {0..3}.
struct AccPos {
    int col, row0;
    __device__ __forceinline__ AccPos() {
        const int lane = threadIdx.x & 63;
        col = lane & 15;
        row0 = (lane >> 4) * 4;
    }
};

// ------------------------------------------------------------------ staging
// Copy rows [0, n) of a [rows x W] slice of a token-major tensor (row j at
// src + j * stride) into LDS, natural layout dst[j * ld + c]; rows >= n are
// zero.  16-byte vectors; TI is the input storage type (F32 or BF16) and the
// LDS element has the same width.
template <class TI, int ROWS, int W, int NT>
__device__ __forceinline__ void stage_natural(typename TI::T* dst, int ld, const typename TI::T* src,
                                              long stride, int n) {
    constexpr int VE = 16 / TI::bytes;
    constexpr int VPR = W / VE;
    for (int idx = threadIdx.x; idx < ROWS * VPR; idx += NT) {
        const int row = idx / VPR;
        const int vc = idx % VPR;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (row < n) val = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + row * stride + vc * VE));
        *reinterpret_cast<u32x4*>(dst + row * ld + vc * VE) = val;
    }
}

// Same source, transposed into LDS: dst[c * ld + j] = src[j][c].  Optionally
// also the natural copy (natural != nullptr).
template <class TI, int ROWS, int W, int NT>
__device__ __forceinline__ void stage_transposed(typename TI::T* dst, int ld, typename TI::T* natural,
                                                 int ldn, const typename TI::T* src, long stride,
                                                 int n) {
    using T = typename TI::T;
    constexpr int VE = 16 / TI::bytes;
    constexpr int VPR = W / VE;
    for (int idx = threadIdx.x; idx < ROWS * VPR; idx += NT) {
        const int row = idx / VPR;
        const int vc = idx % VPR;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (row < n) val = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + row * stride + vc * VE));
        if (natural) *reinterpret_cast<u32x4*>(natural + row * ldn + vc * VE) = val;
        const T* e = reinterpret_cast<const T*>(&val);
#pragma unroll
        for (int i = 0; i < VE; ++i) dst[(vc * VE + i) * ld + row] = e[i];
    }
}

// ------------------------------------------------------------------ decay scan
// Wave 0 computes, for the chunk rows j < C (rows >= n behave as alpha = 1):
//   g[j]   = sum_{r <= j} log alpha_r   (inclusive, restarted at the chunk)
//   eg[j]  = exp(g[j]),  dec[j] = exp(g[C-1] - g[j]),  *gamma = exp(g[C-1]).
// Every exponent is <= 0.  Requires C <= 64.
template <int C>
__device__ __forceinline__ void decay_scan(const float* alpha, long astride, int n, float* g,
                                           float* eg, float* dec, float* gamma) {
    const int lane = threadIdx.x;
    if (lane >= 64) return;
    float x = 0.f;
    if (lane < n && lane < C) x = __logf(fmaxf(__builtin_nontemporal_load(alpha + lane * astride), kMinDecay));
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    const float last = __shfl(x, C - 1, 64);
    if (lane < C) {
        g[lane] = x;
        eg[lane] = __expf(x);
        dec[lane] = __expf(last - x);
    }
    if (lane == 0) *gamma = __expf(last);
}

// The running log-decay alone: g[j] = sum_{i <= j} ln a_i (rows past n: a = 1).
template <int C>
__device__ __forceinline__ void log_decay_scan(const float* alpha, long astride, int n, float* g) {
    const int lane = threadIdx.x;
    if (lane >= 64) return;
    float x = 0.f;
    if (lane < n && lane < C) x = __logf(fmaxf(__builtin_nontemporal_load(alpha + lane * astride), kMinDecay));
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane < C) g[lane] = x;
}

// Workgroup barrier that orders LDS only.  __syncthreads() also fences
// global memory, which makes every wave drain its outstanding global loads
// (the next chunk's prefetch) and stores at each barrier; the chunk loops
// exchange data between waves through LDS alone.
// 2^x by the hardware instruction alone (exp2f adds a rescaling for results
// below 2^-126; the decay factors formed here are as good as zero there).
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// State checkpoints ("Prefix caching has to be redone": a prefix can be
// reused only where a whole state was saved, so an engine saves states at
// block boundaries while it prefills).  Checkpoint j of sequence b is the
// state after (j + 1) * interval tokens of the sequence in this call and
// goes to pool slot slots[b * stride + j]; interval is a multiple of the
// chunk, so every checkpoint falls on the end of a full chunk.
struct Ckpt {
    const int32_t* slots;   // [n_seqs, stride] or NULL (no checkpoints)
    int interval;           // tokens
    int stride;             // checkpoint entries per sequence
};

// Pool slot of the checkpoint after `pos` tokens of sequence b, or -1 (no
// checkpoints, not a checkpoint position, beyond the stride, or a slot
// outside the pool).  Uniform over the workgroup.
__device__ __forceinline__ int ckpt_slot(const Ckpt& ck, int b, int pos, int n_slots) {
    if (ck.slots == nullptr || pos <= 0 || pos % ck.interval != 0) return -1;
    const int j = pos / ck.interval - 1;
    if (j >= ck.stride) return -1;
    const int s = ck.slots[static_cast<long>(b) * ck.stride + j];
    return (s >= 0 && s < n_slots) ? s : -1;
}

// An opaque copy of x: code that uses the copy cannot be hoisted above this
// point.  Checkpoint stores use it for their per-lane offsets, which are
// otherwise loop-invariant and would be computed once and held in registers
// across the whole chunk loop.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// blockIdx -> logical work id, grouping consecutive logical ids on one XCD
// (blocks are dealt to the 8 XCDs round-robin) so that work sharing inputs
// through L2 lands on the same XCD.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
    if ((nblocks & 7) != 0) return bid;
    const int per = nblocks >> 3;
    return (bid & 7) * per + (bid >> 3);
}

}  // namespace gla

namespace gla {

// ------------------------------------------------------------------ operand fragments (bf16)
// A 16x16x32 operand fragment: 8 bf16 per lane.  "KC" storage keeps k
// contiguous along a line (line = operand row for A, column for B); "KM"
// storage is k-major (row = k, the 16 operand lines contiguous), which is
// the natural token-major layout of q/k/v chunks when the contraction runs
// over tokens.  KM fragments are read with ds_read_b64_tr_b16: within each
// 16-lane group, lane i points at row (k0 + i/4) and 4 consecutive lines
// starting at m0 + 4 (i % 4); lane j then receives line m0 + j of the 4
// consecutive rows.  Two such reads give the 8 k-values of a lane group.
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ s16x4 ld_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}
__device__ __forceinline__ bf16x8 cat8(s16x4 a, s16x4 b) {
    typedef __attribute__((ext_vector_type(8))) short s16x8;
    s16x8 r = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, r);
}
// KC: line (lane % 16) of the 16 lines starting at `line0`, k-values
// k0 + 8 g .. k0 + 8 g + 7 (g = lane / 16).
__device__ __forceinline__ bf16x8 frag_kc(const uint16_t* base, int ld, int line0, int k0) {
    const int lane = threadIdx.x & 63;
    const u32x4 v = *reinterpret_cast<const u32x4*>(base + (line0 + (lane & 15)) * ld + k0 + (lane >> 4) * 8);
    return as_bf16x8(v);
}
// KC with the split k order {k0 + 4g .. +3} u {k0 + 16 + 4g .. +3}.
__device__ __forceinline__ bf16x8 frag_kc_split(const uint16_t* base, int ld, int line0, int k0) {
    const int lane = threadIdx.x & 63;
    const uint16_t* p = base + (line0 + (lane & 15)) * ld + k0 + (lane >> 4) * 4;
    const u32x2 a = *reinterpret_cast<const u32x2*>(p);
    const u32x2 b = *reinterpret_cast<const u32x2*>(p + 16);
    return cat8(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b));
}
// KM: lines m0 .. m0 + 15 (contiguous within a row), k-values k0 + 8 g .. +7.
__device__ __forceinline__ bf16x8 frag_km(const uint16_t* base, int ld, int m0, int k0) {
    const int lane = threadIdx.x & 63;
    const int i = lane & 15;
    const uint16_t* p = base + (k0 + (lane >> 4) * 8 + (i >> 2)) * ld + m0 + 4 * (i & 3);
    return cat8(ld_tr16(p), ld_tr16(p + 4 * ld));
}
// KM with the split k order {k0 + 4g .. +3} u {k0 + 16 + 4g .. +3}.
__device__ __forceinline__ bf16x8 frag_km_split(const uint16_t* base, int ld, int m0, int k0) {
    const int lane = threadIdx.x & 63;
    const int i = lane & 15;
    const uint16_t* p = base + (k0 + (lane >> 4) * 4 + (i >> 2)) * ld + m0 + 4 * (i & 3);
    return cat8(ld_tr16(p), ld_tr16(p + 16 * ld));
}
// A 128-row state held as 8 accumulator tiles in "pair" order: tile mt
// gives lane group g (tile rows 4g..4g+3) the state rows
// srow(mt, 4g) + r = 32 (mt / 2) + 8 g + 4 (mt % 2) + r.  Tiles 2s and 2s + 1
// then hand each lane the 8 consecutive rows 32 s + 8 g .. + 7, so the
// state as an MFMA operand (S^T Q^T, K S) meets the other operand's
// fragment in natural order, one 16-byte LDS read per lane; a split order
// would take two 8-byte reads, which the LDS serves at a quarter of the
// 16-byte rate.
__device__ __forceinline__ int srow(int mt, int row0) { return 32 * (mt >> 1) + 2 * row0 + 4 * (mt & 1); }

// K^T operand of the update of pair-order tile mt (lines = its state rows,
// tokens k0 + {4g .. 4g + 3} u {16 + 4g .. 16 + 4g + 3}): the transpose read
// with each lane group's 4 columns where srow() puts them.
__device__ __forceinline__ bf16x8 frag_kt_pair(const uint16_t* base, int ld, int mt, int k0) {
    const int lane = threadIdx.x & 63;
    const int i = lane & 15;
    const uint16_t* p = base + (k0 + (lane >> 4) * 4 + (i >> 2)) * ld + 32 * (mt >> 1) + 8 * (i & 3) + 4 * (mt & 1);
    return cat8(ld_tr16(p), ld_tr16(p + 16 * ld));
}

// Where a 64-key matrix (P, T diag(beta)) keeps keys 16 jt + 4 g .. + 3 (key
// tile jt, lane group g) along its LDS row: at 32 (jt / 2) + 8 g + 4 (jt % 2),
// so that one 16-byte read at 32 ks + 8 g returns keys
// {32 ks + 4 g .. + 3} u {32 ks + 16 + 4 g .. + 3}, the split k order in
// which token-indexed operands come out of the transpose read and of
// accumulator tile pairs.
__device__ __forceinline__ int p_col(int jt, int g) { return 32 * (jt >> 1) + 8 * g + 4 * (jt & 1); }

// 16-wide k tail (16x16x16 MFMA, 4 k-values k0 + 4 g .. +3 per lane).
__device__ __forceinline__ s16x4 frag_kc4(const uint16_t* base, int ld, int line0, int k0) {
    const int lane = threadIdx.x & 63;
    const u32x2 v = *reinterpret_cast<const u32x2*>(base + (line0 + (lane & 15)) * ld + k0 + (lane >> 4) * 4);
    return __builtin_bit_cast(s16x4, v);
}
__device__ __forceinline__ s16x4 frag_km4(const uint16_t* base, int ld, int m0, int k0) {
    const int lane = threadIdx.x & 63;
    const int i = lane & 15;
    return ld_tr16(base + (k0 + (lane >> 4) * 4 + (i >> 2)) * ld + m0 + 4 * (i & 3));
}
__device__ __forceinline__ f32x4 mfma_bf16_k16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// fp32 values -> packed bf16 hi and lo halves (4 values -> 2 dwords each)
__device__ __forceinline__ void split4(f32x4 v, s16x4& hi, s16x4& lo) {
    uint32_t h0, h1, l0, l1;
    split_bf16x2(v.x, v.y, h0, l0);
    split_bf16x2(v.z, v.w, h1, l1);
    hi = __builtin_bit_cast(s16x4, u32x2{h0, h1});
    lo = __builtin_bit_cast(s16x4, u32x2{l0, l1});
}

}  // namespace gla

namespace gla {

// Raw buffer resource over [base, base + nbytes): loads past the end return
// zero and stores past the end are dropped by the hardware.  Used to guard
// partial chunks without branches, so every loop iteration issues the same
// sequence of memory instructions (which keeps the compiler's waits on the
// shared load/store counter precise across iterations).
struct BufRsrc {
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ BufRsrc(const void* base, uint32_t nbytes)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(nbytes), 0x00020000)) {}
    __device__ __forceinline__ u32x4 load16(uint32_t off) const {
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    }
    __device__ __forceinline__ float loadf(uint32_t off) const {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
    }
    __device__ __forceinline__ void store_b16(uint16_t v, uint32_t off) const {
        __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
    }
    __device__ __forceinline__ void store_b32(uint32_t v, uint32_t off) const {
        __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0);
    }
    __device__ __forceinline__ void store_b64(u32x2 v, uint32_t off) const {
        __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
    }
    __device__ __forceinline__ void store_b128(u32x4 v, uint32_t off) const {
        __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
    }
    // Streaming (nontemporal) variants for data touched once per pass: on
    // this memory system they sustain about twice the bandwidth of the
    // default policy for the strided token-major tiles read here.
    static constexpr int kNT = 2;
    __device__ __forceinline__ u32x4 load16_nt(uint32_t off) const {
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNT));
    }
    __device__ __forceinline__ float loadf_nt(uint32_t off) const {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kNT));
    }
    // with a wave-uniform byte offset soff added to the per-lane one
    __device__ __forceinline__ u32x4 load16(uint32_t off, uint32_t soff) const {
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0));
    }
    __device__ __forceinline__ u32x4 load16_nt(uint32_t off, uint32_t soff) const {
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, kNT));
    }
    __device__ __forceinline__ float loadf_nt(uint32_t off, uint32_t soff) const {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, kNT));
    }
    __device__ __forceinline__ float loadf(uint32_t off, uint32_t soff) const {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0));
    }
    __device__ __forceinline__ void storef(float v, uint32_t off, uint32_t soff) const {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, soff, 0);
    }
    __device__ __forceinline__ void store_b128(u32x4 v, uint32_t off, uint32_t soff) const {
        __builtin_amdgcn_raw_buffer_store_b128(v, r, off, soff, 0);
    }
    __device__ __forceinline__ void store_b16_nt(uint16_t v, uint32_t off) const {
        __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, kNT);
    }
    __device__ __forceinline__ void store_b32_nt(uint32_t v, uint32_t off) const {
        __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, kNT);
    }
    __device__ __forceinline__ void store_b64_nt(u32x2 v, uint32_t off) const {
        __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kNT);
    }
    __device__ __forceinline__ void store_b128_nt(u32x4 v, uint32_t off) const {
        __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kNT);
    }
};

// Inclusive prefix sum over the 64 lanes with DPP moves: shifts by 1, 2, 4, 8
// inside each row of 16 lanes, then row 0's total broadcast into row 1 (and
// row 2's into row 3), then rows 0-1's total into rows 2-3.  Lanes without a
// source read 0.
__device__ __forceinline__ float wave_inclusive_sum(float v) {
    auto dpp = [](float a, int ctrl_sel) {
        const int ai = __builtin_bit_cast(int, a);
        int r = 0;
        switch (ctrl_sel) {
            case 1: r = __builtin_amdgcn_update_dpp(0, ai, 0x111, 0xf, 0xf, true); break;   // row_shr:1
            case 2: r = __builtin_amdgcn_update_dpp(0, ai, 0x112, 0xf, 0xf, true); break;   // row_shr:2
            case 4: r = __builtin_amdgcn_update_dpp(0, ai, 0x114, 0xf, 0xf, true); break;   // row_shr:4
            case 8: r = __builtin_amdgcn_update_dpp(0, ai, 0x118, 0xf, 0xf, true); break;   // row_shr:8
            case 15: r = __builtin_amdgcn_update_dpp(0, ai, 0x142, 0xa, 0xf, false); break; // row_bcast:15
            default: r = __builtin_amdgcn_update_dpp(0, ai, 0x143, 0xc, 0xf, false); break; // row_bcast:31
        }
        return __builtin_bit_cast(float, r);
    };
    v += dpp(v, 1);
    v += dpp(v, 2);
    v += dpp(v, 4);
    v += dpp(v, 8);
    v += dpp(v, 15);
    v += dpp(v, 31);
    return v;
}

// Bytes covered by rows [0, n) of a row-strided slice whose rows are
// `width` bytes wide, `stride` bytes apart (0 when n <= 0).
__device__ __forceinline__ uint32_t rows_extent(int n, long stride, int width) {
    return n > 0 ? static_cast<uint32_t>((n - 1) * stride + width) : 0u;
}

}  // namespace gla

namespace gla {
namespace {

// Integer form of wave_inclusive_sum.
__device__ __forceinline__ int wave_inclusive_sum_i(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}

// Up to this many sequences get a longest-first order (rank by a pairwise
// count in LDS); larger batches keep their own order.
constexpr int kOrderMax = 1024;

// Exclusive scan of max(min_count, ceil(L_b / span) - sub) over the
// sequences (L_b from the clamped cu_seqlens): off[b] = first span index of
// sequence b, off[n_seqs] = total.  One workgroup of 1024 threads; each thread sums a
// contiguous range of sequences, then wave scans and a scan of the 16 wave
// totals.  With order != nullptr also writes the sequences by decreasing
// length (ties by index): order[r] = sequence of rank r.
__device__ __forceinline__ void span_offsets_body(const int32_t* __restrict__ cu, int n_seqs, int n_tokens,
                                                  int span, int min_count, int sub, int32_t* __restrict__ off,
                                                  int32_t* __restrict__ order, int* wsum, int* lens,
                                                  int min_keep = 0) {
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    auto length = [&](int b) {
        const int s = clampi(cu[b], 0, n_tokens);
        return clampi(cu[b + 1], s, n_tokens) - s;
    };
    auto count = [&](int b) {
        const int c = max(min_count, (length(b) + span - 1) / span - sub);
        return c < min_keep ? 0 : c;
    };
    const int per = (n_seqs + 1023) / 1024;
    const int b0 = min(t * per, n_seqs), b1 = min(b0 + per, n_seqs);
    int sum = 0;
    for (int b = b0; b < b1; ++b) sum += count(b);
    const int incl = wave_inclusive_sum_i(sum);
    if (lane == 63) wsum[wave] = incl;
    lds_barrier();
    int run = incl - sum;
    for (int w = 0; w < wave; ++w) run += wsum[w];
    for (int b = b0; b < b1; ++b) {
        off[b] = run;
        run += count(b);
    }
    if (b1 == n_seqs && b0 < b1) off[n_seqs] = run;
    if (n_seqs == 0 && t == 0) off[0] = 0;
    if (order == nullptr) return;
    if (n_seqs <= kOrderMax) {
        for (int b = t; b < n_seqs; b += 1024) lens[b] = length(b);
        lds_barrier();
        for (int b = t; b < n_seqs; b += 1024) {
            const int lb = lens[b];
            int r = 0;
            for (int j = 0; j < n_seqs; ++j) {
                const int lj = lens[j];
                r += (lj > lb || (lj == lb && j < b)) ? 1 : 0;
            }
            order[r] = b;
        }
    } else {
        for (int b = t; b < n_seqs; b += 1024) order[b] = b;
    }
}

__global__ void __launch_bounds__(1024)
span_offsets(const int32_t* __restrict__ cu, int n_seqs, int n_tokens, int span, int min_count,
             int sub, int32_t* __restrict__ off, int32_t* __restrict__ order) {
    __shared__ int wsum[16];
    __shared__ int lens[kOrderMax];
    span_offsets_body(cu, n_seqs, n_tokens, span, min_count, sub, off, order, wsum, lens);
}

// Several such scans over the same sequences in one launch, workgroup i
// doing scan i (no order); a count below min_keep counts as 0.
struct SpanScan {
    int span, min_count, sub, min_keep;
    int32_t* off;
};
struct SpanScans {
    SpanScan s[4];
};
__global__ void __launch_bounds__(1024)
span_offsets_multi(const int32_t* __restrict__ cu, int n_seqs, int n_tokens, SpanScans sc) {
    __shared__ int wsum[16];
    const SpanScan& x = sc.s[blockIdx.x];
    span_offsets_body(cu, n_seqs, n_tokens, x.span, x.min_count, x.sub, x.off, nullptr, wsum, nullptr, x.min_keep);
}

// Largest b in [0, n_seqs) with off[b] <= idx (off non-decreasing).
__device__ __forceinline__ int find_span_owner(const int32_t* off, int n_seqs, int idx) {
    int lo = 0, hi = n_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= idx) lo = mid; else hi = mid - 1;
    }
    return lo;
}

}  // namespace
}  // namespace gla
