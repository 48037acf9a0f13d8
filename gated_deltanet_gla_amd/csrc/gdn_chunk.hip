// Chunked Gated DeltaNet prefill on gfx950.
//
// "Inference for linear attention and hybrid architectures", section "Two
// ways to write the same computation": DeltaNet's update
// (I - b_t k_t^T k_t) S + b_t k_t^T v_t with a decay gate a_t multiplied in
// (on the old state), and the remark that the in-chunk error-correcting
// updates must first be written in matrix form.  That matrix form is not on
// the page; the one used here is derived from the update itself:
//
//   u_t = b_t (v_t - a_t k_t S_{t-1})  makes every step a GLA step with
//   value u_t:  S_t = a_t S_{t-1} + k_t^T u_t.
//
// Inside a chunk entered with state S, with g the running sum of log a,
//   (I + A) U = diag(b) (V - diag(exp g) K S),
//   A_tj = b_t exp(g_t - g_j) (k_t . k_j)  for j < t, 0 otherwise,
// so U = T diag(b) Y with T = (I + A)^-1 and Y = V - diag(exp g) (K S).
// Then the GLA chunk formulas apply with U in place of V:
//   O = diag(exp g) Q S + ((Q K^T) .* D) U
//   S <- exp(g_last) S + K^T diag(exp(g_last - g)) U.
//
// Kernels:
//  1. span_offsets: exclusive scan of ceil(L_b / C) -> first chunk of every
//     sequence (one workgroup).
//  2. gdn_prep: one workgroup per (chunk, head), all chunks at once: A from
//     K K^T on MFMA, then the unit-lower-triangular inverse T in fp32
//     (16x16 diagonal blocks by forward substitution, off-diagonal blocks
//     T_ij = -T_ii sum_k A_ik T_kj along successive block diagonals).  T does
//     not depend on the state, so this latency-heavy step runs fully
//     parallel instead of on the serial chain.  Written to the workspace.
//  3. the serial chunk loop with the state slice in MFMA accumulators, one
//     workgroup per (sequence, head, d_v tile): gdn_fast_kernel for bf16
//     inputs with chunks of 32/64 and d_k >= 32 (the prep kernel then also
//     emits T diag(beta) and P as bf16 hi/lo planes), gdn_chunk_kernel for
//     the rest (fp32 inputs, 16-wide shapes).
#include <algorithm>

#include "chunk_common.h"
#include "launch.h"

namespace gla {
namespace {

constexpr int NW = 4;
constexpr int NT = NW * 64;
constexpr long kPrepBlocks = 768;    // 256 compute units x 3 resident prep workgroups
constexpr long kWideMin = 1024;      // 16-column serial workgroups above which 32-column ones run

__host__ __device__ constexpr size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ constexpr long max_chunks(int n_seqs, int n_tokens, int C) {
    return static_cast<long>(n_tokens) / C + n_seqs;
}

// ------------------------------------------------------------------ 2. prep
// LDS: the staged k (and q) and the fp32 A / T tiles are never live at the
// same time, so they share one region; with the per-wave scratch and the
// gate tables a workgroup fits in 40 KiB and four of them share a compute
// unit, which overlaps one workgroup's loads with the others' arithmetic.
template <int DK, int C, bool F32, bool TP>
struct PrepSmem {
    using E = typename Op<F32>::E;
    static constexpr int LQ = DK + Op<F32>::PAD;
    static constexpr int LA = C + 4;           // fp32 lines of A and T (16-byte aligned)
    struct In {
        alignas(16) E k[C][LQ];
        alignas(16) E q[TP ? C : 1][LQ];
    };
    struct Tri {
        alignas(16) float a[C][LA];
        alignas(16) float t[C][LA];
    };
    union {
        In in;
        Tri tri;
    };
    alignas(16) float x[NW][16][20];           // per-wave 16x16 scratch (padded)
    float g[C], beta[C];
};

// One work item = one (chunk, head).  The kernel is persistent: a fixed grid
// of workgroups strides over the items, and while one item's arithmetic runs
// (latency-bound: the triangular inverse), the k / q rows and gates of the
// workgroup's next item are already loading into registers.
struct PrepItem {
    int ci, h, n;      // chunk (global index), head, valid rows
    long tok0;         // first token
    bool ok;
};

template <class TI, int C, int DK, bool TP>
struct PrepPrefetch {
    static constexpr int VE = 16 / TI::bytes;          // elements per 16-byte vector
    static constexpr int NV = (C * DK / VE + NT - 1) / NT;
    u32x4 k[NV];
    u32x4 q[TP ? NV : 1];
    float a;           // gate (wave 0) / beta (wave 1) of token `lane`, raw
};

// PL = 0: write T (fp32, C x C) per (chunk, head).
// PL = 4 (bf16 inputs): write four bf16 C x C planes per (chunk, head):
//   T diag(beta) hi, lo, and P = (Q K^T) .* D (lower, decayed) hi, lo.
// PL = 2 (bf16 inputs): T diag(beta) hi, lo only.
template <int DK, int C, class TI, int PL>
__global__ void __launch_bounds__(NT, 3)       // three resident workgroups per compute unit
gdn_prep(const typename TI::T* __restrict__ k, const typename TI::T* __restrict__ q,
         const float* __restrict__ alpha, const float* __restrict__ beta,
         const int32_t* __restrict__ cu, int n_seqs, int n_tokens, int H,
         const int32_t* __restrict__ off, void* __restrict__ Tws) {
    constexpr bool F32 = (TI::bytes == 4);
    constexpr bool TP = PL > 0;          // bf16 planes
    constexpr bool WP = PL == 4;         // ... including P
    static_assert(!(TP && F32), "planes are bf16");
    using O = Op<F32>;
    using Sm = PrepSmem<DK, C, F32, WP>;
    using PF = PrepPrefetch<TI, C, DK, WP>;
    constexpr int LQ = Sm::LQ;
    constexpr int NB = C / 16;
    constexpr int TPW = (NB * NB + NW - 1) / NW;   // 16x16 tiles per wave
    constexpr int VE = PF::VE;
    constexpr int VPR = DK / VE;                   // vectors per row
    __shared__ Sm sm;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const long tstride = static_cast<long>(H) * DK;
    const long n_items = static_cast<long>(off[n_seqs]) * H;

    auto locate = [&](long item) {
        PrepItem it{0, 0, 0, 0, false};
        if (item >= n_items) return it;
        it.h = static_cast<int>(item % H);
        it.ci = static_cast<int>(item / H);
        // sequence of this chunk: largest b with off[b] <= ci
        int lo = 0, hi = n_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (off[mid] <= it.ci) lo = mid; else hi = mid - 1;
        }
        const int s0 = clampi(cu[lo], 0, n_tokens);
        const int s1 = clampi(cu[lo + 1], s0, n_tokens);
        const int c0 = (it.ci - off[lo]) * C;
        it.n = min(C, s1 - s0 - c0);
        it.ok = c0 >= 0 && it.n > 0;      // false only with a malformed cu_seqlens
        if (!it.ok) it.n = 0;
        it.tok0 = s0 + max(c0, 0);
        return it;
    };
    // item rows -> registers; rows past n (and items that do not exist) read
    // as zero through the buffer resource
    auto fetch = [&](PF& pf, const PrepItem& it) {
        const uint32_t ext = rows_extent(it.n, tstride * TI::bytes, DK * TI::bytes);
        const BufRsrc rk(k + it.tok0 * tstride + it.h * DK, ext);
        const BufRsrc rq(q + it.tok0 * tstride + it.h * DK, WP ? ext : 0u);
#pragma unroll
        for (int u = 0; u < PF::NV; ++u) {
            const int x = threadIdx.x + u * NT;
            const uint32_t offb = static_cast<uint32_t>(((x / VPR) * tstride + (x % VPR) * VE) * TI::bytes);
            pf.k[u] = rk.load16_nt(offb);
            if constexpr (WP) pf.q[u] = rq.load16_nt(offb);
        }
        const float* gsrc = wave == 0 ? alpha : beta;
        const BufRsrc rg(gsrc + it.tok0 * H + it.h, wave < 2 ? rows_extent(it.n, static_cast<long>(H) * 4, 4) : 0u);
        pf.a = rg.loadf_nt(static_cast<uint32_t>(lane * H * 4));
    };
    auto stage = [&](const PF& pf, const PrepItem& it) {
#pragma unroll
        for (int u = 0; u < PF::NV; ++u) {
            const int x = threadIdx.x + u * NT;
            if (C * DK / VE == PF::NV * NT || x < C * DK / VE) {
                const int row = x / VPR, vc = x % VPR;
                *reinterpret_cast<u32x4*>(&sm.in.k[row][vc * VE]) = pf.k[u];
                if constexpr (WP) *reinterpret_cast<u32x4*>(&sm.in.q[row][vc * VE]) = pf.q[u];
            }
        }
        if (wave == 0) {
            // running log-decay g_j = sum_{i <= j} ln a_i (rows past n: a = 1)
            float x = lane < it.n ? __logf(fmaxf(pf.a, kMinDecay)) : 0.f;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const float y = __shfl_up(x, o, 64);
                if (lane >= o) x += y;
            }
            if (lane < C) sm.g[lane] = x;
        } else if (wave == 1) {
            if (lane < C) sm.beta[lane] = lane < it.n ? pf.a : 0.f;
        }
    };

    PF pf;
    long item = blockIdx.x;
    PrepItem cur = locate(item);
    fetch(pf, cur);
    for (; item < n_items; item += gridDim.x) {
    stage(pf, cur);
    lds_barrier();
    const PrepItem nxt = locate(item + gridDim.x);
    fetch(pf, nxt);                      // in flight during this item's arithmetic
    if (cur.ok) {
    const int h = cur.h;
    const int ci = cur.ci;
    const int n = cur.n;
    (void)n;
    const AccPos ap;
    uint16_t* planes = static_cast<uint16_t*>(Tws) + (static_cast<long>(ci) * H + h) * (TP ? PL : 1) * C * C;
    // A = strictly-lower(diag(beta) (K K^T .* D)), fp32, held in registers
    // until k (and q) are no longer read; P = (Q K^T) .* D as P^T tiles (lane:
    // 4 consecutive j of row i) straight to planes 2, 3
    f32x4 areg[TPW];
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
        const int t = wave + NW * m;
        areg[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (t < NB * NB) {
            const int tt = t / NB, jt = t % NB;
            if (jt <= tt) {
                O::mma(areg[m], &sm.in.k[tt * 16][0], LQ, &sm.in.k[jt * 16][0], LQ, DK);
                const int j = jt * 16 + ap.col;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = tt * 16 + ap.row0 + r;
                    areg[m][r] = (j < i) ? sm.beta[i] * __expf(sm.g[i] - sm.g[j]) * areg[m][r] : 0.f;
                }
            }
            if constexpr (WP) {
                const int pj = t / NB, pi = t % NB;
                const int i = pi * 16 + ap.col;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                if (pj <= pi) {
                    O::mma(acc, &sm.in.k[pj * 16][0], LQ, &sm.in.q[pi * 16][0], LQ, DK);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = pj * 16 + ap.row0 + r;
                        acc[r] = (j <= i) ? acc[r] * __expf(sm.g[i] - sm.g[j]) : 0.f;
                    }
                }
                // 32-column blocks wholly above the diagonal are never read
                if ((pj * 16) / 32 * 32 <= pi * 16 + 15)
                    O::store4(planes + 2 * C * C + i * C + pj * 16 + ap.row0,
                              planes + 3 * C * C + i * C + pj * 16 + ap.row0, acc);
            }
        }
    }
    lds_barrier();                       // k, q dead: their space becomes A and T
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
        const int t = wave + NW * m;
        if (t < NB * NB) {
            const int tt = t / NB, jt = t % NB;
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.tri.a[tt * 16 + ap.row0 + r][jt * 16 + ap.col] = areg[m][r];
        }
    }
    // blocks above the diagonal of T are zero
    for (int idx = threadIdx.x; idx < C * C; idx += NT) {
        const int r = idx / C, c = idx % C;
        if ((c >> 4) > (r >> 4)) sm.tri.t[r][c] = 0.f;
    }
    lds_barrier();

    // diagonal blocks: forward substitution, one column per lane
    if (wave < NB && lane < 16) {
        const int base = wave * 16;
        const int c = lane;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < r; ++m) acc -= sm.tri.a[base + r][base + m] * x[m];
            x[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sm.tri.t[base + r][base + c] = x[r];
    }
    lds_barrier();

    // off-diagonal blocks, one block diagonal at a time: T_ij = -T_ii sum_k A_ik T_kj,
    // each 16x16x16 product on the fp32 MFMA (16x16x4: A lane = row, B lane =
    // column, k = lane / 16 within each group of 4; C lane = column, rows
    // 4 (lane / 16) .. +3)
    const int l16 = lane & 15, lg = lane >> 4;
    for (int d = 1; d < NB; ++d) {
        const int i = d + wave;        // this wave's block row (block column i - d)
        if (i < NB) {
            const int j = i - d;
            f32x4 xs = {0.f, 0.f, 0.f, 0.f};
            for (int kb = j; kb < i; ++kb) {
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4)
                    xs = mfma_f32(sm.tri.a[i * 16 + l16][kb * 16 + 4 * s4 + lg],
                                  sm.tri.t[kb * 16 + 4 * s4 + lg][j * 16 + l16], xs);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.x[wave][4 * lg + r][l16] = xs[r];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4)
                y = mfma_f32(sm.tri.t[i * 16 + l16][i * 16 + 4 * s4 + lg], sm.x[wave][4 * s4 + lg][l16], y);
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.tri.t[i * 16 + 4 * lg + r][j * 16 + l16] = -y[r];
        }
        lds_barrier();
    }

    if constexpr (!TP) {
        // T -> workspace, row-major C x C
        float* dst = static_cast<float*>(Tws) + (static_cast<long>(ci) * H + h) * C * C;
        for (int idx = threadIdx.x; idx < C * C / 4; idx += NT) {
            const int r = (idx * 4) / C, c = (idx * 4) % C;
            *reinterpret_cast<f32x4*>(dst + r * C + c) = *reinterpret_cast<const f32x4*>(&sm.tri.t[r][c]);
        }
    } else {
        // T diag(beta) -> planes 0 (hi), 1 (lo); 32-column blocks wholly
        // above the diagonal of a 16-row block are never read
        for (int idx = threadIdx.x; idx < C * C / 4; idx += NT) {
            const int r = (idx * 4) / C, c = (idx * 4) % C;
            if (c / 32 * 32 > (r / 16) * 16 + 15) continue;
            f32x4 tv = *reinterpret_cast<const f32x4*>(&sm.tri.t[r][c]);
#pragma unroll
            for (int e = 0; e < 4; ++e) tv[e] *= sm.beta[c + e];
            O::store4(planes + r * C + c, planes + C * C + r * C + c, tv);
        }
    }
    }  // cur.ok
    lds_barrier();                       // T read out: the next item may restage
    cur = nxt;
    }  // items
}

// ------------------------------------------------------------------ 3. serial chunk loop
template <int DK, int BV, int C, bool F32>
struct GdnSmem {
    using E = typename Op<F32>::E;
    static constexpr int PAD = Op<F32>::PAD;
    static constexpr int LQ = DK + PAD;
    static constexpr int LT = C + PAD;
    static constexpr int HL = F32 ? 1 : 2;      // hi (+ lo) planes
    alignas(16) E q[C][LQ];
    alignas(16) E k[C][LQ];
    alignas(16) E kt[DK][LT];
    alignas(16) E p[HL][C][LT];
    alignas(16) E st[HL][BV][LQ];
    alignas(16) E t1[HL][C][LT];      // T diag(beta)
    alignas(16) E yt[HL][BV][LT];     // (V - diag(exp g) K S)^T
    alignas(16) E ut[HL][BV][LT];     // U^T
    alignas(16) E udt[HL][BV][LT];    // (diag(exp(g_last - g)) U)^T
    float g[C], eg[C], dec[C], beta[C];
    float gamma;
};

template <int DK, int DV, int BV, int C, class TI, class TO>
__global__ void __launch_bounds__(NT)
gdn_chunk_kernel(const typename TI::T* __restrict__ q, const typename TI::T* __restrict__ k,
                 const typename TI::T* __restrict__ v, const float* __restrict__ alpha,
                 const float* __restrict__ beta, const int32_t* __restrict__ cu, int n_seqs,
                 int n_tokens, int H, float* __restrict__ pool, int n_slots,
                 const int32_t* __restrict__ slot_idx, int zero_init,
                 const int32_t* __restrict__ off, long n_chunks_max, const float* __restrict__ Tws,
                 Ckpt ck, typename TO::T* __restrict__ o) {
    constexpr bool F32 = (TI::bytes == 4);
    using O = Op<F32>;
    using Sm = GdnSmem<DK, BV, C, F32>;
    constexpr int LQ = Sm::LQ, LT = Sm::LT;
    constexpr int LO = F32 ? 0 : 1;              // index of the lo plane
    constexpr int NVT = DV / BV;
    constexpr int CT = C / 16;
    constexpr int BT = BV / 16;
    constexpr int ST = (DK / 16) * BT;
    constexpr int SPW = (ST + NW - 1) / NW;
    static_assert(DV % BV == 0 && BV % 16 == 0 && C % 16 == 0 && C <= 64, "tiling");

    __shared__ Sm sm;

    const int work = xcd_remap(blockIdx.x, gridDim.x);
    const int vt = work % NVT;
    const int bh = work / NVT;
    const int h = bh % H;
    const int b = bh / H;
    if (b >= n_seqs) return;
    const int slot = slot_idx[b];
    if (slot < 0 || slot >= n_slots) return;
    const int s0 = clampi(cu[b], 0, n_tokens);
    const int s1 = clampi(cu[b + 1], s0, n_tokens);
    const int L = s1 - s0;
    const int chunk_base = off[b];

    const int wave = threadIdx.x >> 6;
    const AccPos ap;
    const int col0 = vt * BV;

    float* Sg = pool + (static_cast<long>(slot) * H + h) * DK * DV;
    f32x4 S[SPW];
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int t = wave + NW * i;
        const int mt = t / BT, nt = t % BT;
        S[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (t < ST && !zero_init) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[i][r] = Sg[(mt * 16 + ap.row0 + r) * DV + col0 + nt * 16 + ap.col];
        }
    }

    const long tstride = static_cast<long>(H) * DK;
    const long vstride = static_cast<long>(H) * DV;
    for (int c0 = 0, ci = chunk_base; c0 < L; c0 += C, ++ci) {
        const int n = min(C, L - c0);
        const long tok0 = s0 + c0;
        if (ci < 0 || ci >= n_chunks_max) break;   // only reachable with a malformed cu_seqlens
        lds_barrier();

        // ---- phase 0: stage inputs, decay scan, state slice -> st
        stage_natural<TI, C, DK, NT>(&sm.q[0][0], LQ, q + tok0 * tstride + h * DK, tstride, n);
        stage_transposed<TI, C, DK, NT>(&sm.kt[0][0], LT, &sm.k[0][0], LQ,
                                        k + tok0 * tstride + h * DK, tstride, n);
        decay_scan<C>(alpha + tok0 * H + h, H, n, sm.g, sm.eg, sm.dec, &sm.gamma);
        for (int j = threadIdx.x; j < C; j += NT) sm.beta[j] = j < n ? beta[(tok0 + j) * H + h] : 0.f;
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int t = wave + NW * i;
            if (t < ST) {
                const int mt = t / BT, nt = t % BT;
                const int ln = nt * 16 + ap.col;
                O::store4(&sm.st[0][ln][mt * 16 + ap.row0], &sm.st[LO][ln][mt * 16 + ap.row0], S[i]);
            }
        }
        lds_barrier();

        // ---- phase 1: T diag(beta); P; X = K S -> Y = V - diag(exp g) X
        {
            const float* Tc = Tws + (static_cast<long>(ci) * H + h) * C * C;
            for (int idx = threadIdx.x; idx < C * C / 4; idx += NT) {
                const int r = (idx * 4) / C, m = (idx * 4) % C;
                f32x4 tv = *reinterpret_cast<const f32x4*>(Tc + r * C + m);
                tv.x *= sm.beta[m];
                tv.y *= sm.beta[m + 1];
                tv.z *= sm.beta[m + 2];
                tv.w *= sm.beta[m + 3];
                O::store4(&sm.t1[0][r][m], &sm.t1[LO][r][m], tv);
            }
        }
        for (int t = wave; t < CT * CT; t += NW) {
            const int jt = t / CT, it = t % CT;
            const int i = it * 16 + ap.col;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (jt <= it) {
                O::mma(acc, &sm.k[jt * 16][0], LQ, &sm.q[it * 16][0], LQ, DK);
                const float gi = sm.g[i];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = jt * 16 + ap.row0 + r;
                    acc[r] = (j <= i) ? acc[r] * __expf(gi - sm.g[j]) : 0.f;
                }
            }
            O::store4(&sm.p[0][i][jt * 16 + ap.row0], &sm.p[LO][i][jt * 16 + ap.row0], acc);
        }
        for (int t = wave; t < CT * BT; t += NW) {
            const int tt = t / BT, nt = t % BT;
            const int ln = nt * 16 + ap.col;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mma_xs<F32>(acc, &sm.k[tt * 16][0], LQ, &sm.st[0][nt * 16][0], &sm.st[LO][nt * 16][0], LQ, DK);
            f32x4 y;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = tt * 16 + ap.row0 + r;
                const float vv = row < n ? TI::load(v, (tok0 + row) * vstride + h * DV + col0 + ln) : 0.f;
                y[r] = vv - sm.eg[row] * acc[r];
            }
            O::store4(&sm.yt[0][ln][tt * 16 + ap.row0], &sm.yt[LO][ln][tt * 16 + ap.row0], y);
        }
        lds_barrier();

        // ---- phase 2: U = T diag(beta) Y
        for (int t = wave; t < CT * BT; t += NW) {
            const int tt = t / BT, nt = t % BT;
            const int ln = nt * 16 + ap.col;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mma_ss<F32>(acc, &sm.t1[0][tt * 16][0], &sm.t1[LO][tt * 16][0], LT, &sm.yt[0][nt * 16][0],
                        &sm.yt[LO][nt * 16][0], LT, C);
            O::store4(&sm.ut[0][ln][tt * 16 + ap.row0], &sm.ut[LO][ln][tt * 16 + ap.row0], acc);
            f32x4 ud;
#pragma unroll
            for (int r = 0; r < 4; ++r) ud[r] = acc[r] * sm.dec[tt * 16 + ap.row0 + r];
            O::store4(&sm.udt[0][ln][tt * 16 + ap.row0], &sm.udt[LO][ln][tt * 16 + ap.row0], ud);
        }
        lds_barrier();

        // ---- phase 3: outputs and state hand-off
        for (int t = wave; t < CT * BT; t += NW) {
            const int it = t / BT, nt = t % BT;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mma_xs<F32>(acc, &sm.q[it * 16][0], LQ, &sm.st[0][nt * 16][0], &sm.st[LO][nt * 16][0], LQ, DK);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] *= sm.eg[it * 16 + ap.row0 + r];
            mma_ss<F32>(acc, &sm.p[0][it * 16][0], &sm.p[LO][it * 16][0], LT, &sm.ut[0][nt * 16][0],
                        &sm.ut[LO][nt * 16][0], LT, C);
            const int colg = col0 + nt * 16 + ap.col;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = it * 16 + ap.row0 + r;
                if (row < n) TO::store(o, (tok0 + row) * vstride + h * DV + colg, acc[r]);
            }
        }
        const float gam = sm.gamma;
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int t = wave + NW * i;
            if (t < ST) {
                const int mt = t / BT, nt = t % BT;
                S[i] *= gam;
                mma_xs<F32>(S[i], &sm.kt[mt * 16][0], LT, &sm.udt[0][nt * 16][0],
                            &sm.udt[LO][nt * 16][0], LT, C);
            }
        }
        // checkpoint: this wave's tiles of the state after the chunk
        const int cs = c0 + C <= L ? ckpt_slot(ck, b, c0 + C, n_slots) : -1;
        if (cs >= 0) {
            float* Sc = pool + (static_cast<long>(cs) * H + h) * DK * DV +
                        opaque(ap.row0 * DV + col0 + ap.col);
#pragma unroll
            for (int i = 0; i < SPW; ++i) {
                const int t = wave + NW * i;
                if (t < ST) {
                    const int mt = t / BT, nt = t % BT;
#pragma unroll
                    for (int r = 0; r < 4; ++r) Sc[(mt * 16 + r) * DV + nt * 16] = S[i][r];
                }
            }
        }
    }

#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int t = wave + NW * i;
        if (t < ST) {
            const int mt = t / BT, nt = t % BT;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Sg[(mt * 16 + ap.row0 + r) * DV + col0 + nt * 16 + ap.col] = S[i][r];
        }
    }
}

// ------------------------------------------------------------------ 3b. serial chunk loop, bf16
// The bf16 path for chunks of 32 or 64 tokens and d_k >= 32.  One
// workgroup (8 waves) per (sequence, head, 16-column d_v tile).  Waves 0-3
// own a 16-row block of the chunk for X, Y and U, waves 4-7 the same blocks
// for Q S and the outputs, and wave w owns state tile w (rows 16w..16w+15),
// which halves each wave's MFMA chain on the serial path.  T diag(beta) and P come precomputed from
// gdn_prep as bf16 hi/lo planes and are read straight from HBM/L2 into MFMA
// operand registers one chunk ahead, so the serial chain only carries the
// state-dependent work:
//   A: X = K S and Q S (state slice from LDS), Y = V - diag(exp g) X  -> LDS
//   B: U = T diag(beta) Y                                             -> LDS
//   C: O = diag(exp g) Q S + P U; S <- gamma S + K^T diag(dec) U; the new
//      state slice -> LDS for the next chunk.
// q, k, v are double-buffered in LDS and prefetched into registers two
// chunks ahead; three LDS-only barriers per chunk.
constexpr int FW = 8;                 // waves of the bf16 serial kernel
constexpr int FT = FW * 64;

template <int DK, int C, int BV_>
struct GdnFastSmem {
    static constexpr int BV = BV_;
    // rows of the v tile buffer: every thread stages one dword per 16
    // columns (FT / 8 rows), so the staging has no thread-dependent branch
    static constexpr int VR = FT / 8 > C ? FT / 8 : C;
    static constexpr int LQ = DK + 8;
    static constexpr int LV = BV + 8;
    static constexpr int LT = C + 8;
    struct Buf {
        alignas(16) uint16_t q[C][LQ];
        alignas(16) uint16_t k[C][LQ];
        alignas(16) uint16_t v[VR][LV];
        float eg[C];
        float dec[C];
        float gamma;
    };
    Buf buf[2];
    alignas(16) uint16_t st[2][BV][LQ];    // state slice: line = column, k = d (hi, lo)
    alignas(16) uint16_t yt[2][BV][LT];    // Y^T (hi, lo)
    alignas(16) uint16_t ut[2][BV][LT];    // U^T (hi, lo)
    alignas(16) uint16_t udt[2][BV][LT];   // (diag(dec) U)^T (hi, lo)
};

template <int C, int DK, int BV>
struct GdnFastPrefetch {
    static constexpr int NQ = (C * DK / 8 + FT - 1) / FT;
    u32x4 q[NQ], k[NQ];
    uint32_t v[BV / 16];   // two values of row tid / 8 in each 16-column tile of v
    float a;           // raw gate of token `lane`; only the first n are valid
    int n;
};

template <int DK, int DV, int C, class TO, bool CKPT, int BV_>
__global__ void __launch_bounds__(FT)
gdn_fast_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                const uint16_t* __restrict__ v, const float* __restrict__ alpha,
                const int32_t* __restrict__ cu, int n_seqs, int n_tokens, int H,
                float* __restrict__ pool, int n_slots, const int32_t* __restrict__ slot_idx,
                int zero_init, const int32_t* __restrict__ off, const int32_t* __restrict__ order,
                long n_chunks_max, const uint16_t* __restrict__ TP, Ckpt ck,
                typename TO::T* __restrict__ o) {
    using Sm = GdnFastSmem<DK, C, BV_>;
    using PF = GdnFastPrefetch<C, DK, BV_>;
    using O = Op<false>;
    constexpr int BV = Sm::BV, LQ = Sm::LQ, LT = Sm::LT;
    constexpr int NVT = DV / BV;
    constexpr int NTL = BV / 16;                 // 16-column tiles of this workgroup
    constexpr int CT = C / 16;                   // 16-row blocks per chunk
    constexpr int KSD = DK / 32;                 // k steps over d_k
    constexpr int KSC = C / 32;                  // k steps over the chunk
    constexpr int KT = DK / 16;                  // state tiles (one column tile), at most FW
    static_assert(C >= 32 && DK >= 32 && DV % BV == 0 && KT <= FW && CT <= 4, "fast path shapes");

    __shared__ Sm sm;

    // (sequence, head) groups in longest-first order, dealt round-robin to
    // the 8 XCDs (blockIdx mod 8 picks the XCD); the d_v tiles of one group
    // are consecutive blocks of one XCD, so they share q and k through its L2
    const int xcd = blockIdx.x & 7, pos = blockIdx.x >> 3;
    const int vt = pos % NVT;
    const int gi = (pos / NVT) * 8 + xcd;
    if (gi >= n_seqs * H) return;
    const int h = gi % H;
    const int b = order[gi / H];
    if (b < 0 || b >= n_seqs) return;
    const int slot = slot_idx[b];
    if (slot < 0 || slot >= n_slots) return;
    const int s0 = clampi(cu[b], 0, n_tokens);
    const int s1 = clampi(cu[b + 1], s0, n_tokens);
    const int L = s1 - s0;
    int nchunks = (L + C - 1) / C;
    const long cbase = off[b];
    if (cbase < 0) nchunks = 0;                                  // malformed cu_seqlens only
    if (cbase + nchunks > n_chunks_max) nchunks = static_cast<int>(max(0L, n_chunks_max - cbase));

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const AccPos ap;
    const int col0 = vt * BV;
    const long tstride = static_cast<long>(H) * DK;
    const long vstride = static_cast<long>(H) * DV;
    // roles: waves 0..3 own row block `it` for X, Y and U; waves 4..7 own row
    // block `it` for Q S and the outputs; every wave owns state tile `wave`
    const bool xrole = wave < 4 && wave < CT;
    const bool qrole = wave >= 4 && wave - 4 < CT;
    const int it = wave & 3;
    const bool has_tile = wave < KT;

    float* Sg = pool + (static_cast<long>(slot) * H + h) * DK * DV;
    f32x4 S[NTL];
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt) {
        S[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (has_tile && !zero_init) {
#pragma unroll
            for (int r = 0; r < 4; ++r) S[nt][r] = Sg[(wave * 16 + ap.row0 + r) * DV + col0 + nt * 16 + ap.col];
        }
    }

    // rows of chunk c that belong to the sequence (<= 0 past its end)
    auto chunk_rows = [&](int c) { return c < nchunks ? min(C, L - c * C) : 0; };
    PF pf;
    // Global -> registers for chunk c, with no branches: rows past the
    // chunk's valid ones (or chunks past the end) read as zero.
    auto fetch = [&](int c) {
        const int n = chunk_rows(c);
        const long tok0 = s0 + static_cast<long>(c < nchunks ? c : 0) * C;
        const BufRsrc rq(q + tok0 * tstride + h * DK, rows_extent(n, tstride * 2, DK * 2));
        const BufRsrc rk(k + tok0 * tstride + h * DK, rows_extent(n, tstride * 2, DK * 2));
        const BufRsrc rv(v + tok0 * vstride + h * DV + col0, rows_extent(n, vstride * 2, BV * 2));
        const BufRsrc ra(alpha + tok0 * H + h, wave == 0 ? rows_extent(n, static_cast<long>(H) * 4, 4) : 0u);
#pragma unroll
        for (int u = 0; u < PF::NQ; ++u) {
            const int x = tid + u * FT;
            const int row = x / (DK / 8), vc = x % (DK / 8);
            const uint32_t offb = static_cast<uint32_t>((row * tstride + vc * 8) * 2);
            pf.q[u] = rq.load16_nt(offb);
            pf.k[u] = rk.load16_nt(offb);
        }
#pragma unroll
        for (int j = 0; j < NTL; ++j)
            pf.v[j] = __float_as_uint(
                rv.loadf_nt(static_cast<uint32_t>(((tid >> 3) * vstride + j * 16 + (tid & 7) * 2) * 2)));
        // rows past n get a gate of 1 when staged: a select on the loaded
        // value here would make the wave wait for this load right away
        pf.a = ra.loadf_nt(static_cast<uint32_t>(lane * H * 4));
        pf.n = n;
    };
    auto stage = [&](typename Sm::Buf& bb) {
        if (wave == 0) {
            const float a = lane < pf.n ? pf.a : 1.f;
            const float x = wave_inclusive_sum(__log2f(fmaxf(a, kMinDecay)));
            const float glast =
                __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), C - 1));
            if (lane < C) {
                bb.eg[lane] = exp2f(x);
                bb.dec[lane] = exp2f(glast - x);
            }
            if (lane == 0) bb.gamma = exp2f(glast);
        }
#pragma unroll
        for (int u = 0; u < PF::NQ; ++u) {
            const int xx = tid + u * FT;
            // (a constant condition when the threads cover the tile exactly;
            // a branch here would blur the compiler's load-counter waits)
            if (C * DK / 8 == PF::NQ * FT || xx < C * DK / 8) {
                const int row = xx / (DK / 8), vc = xx % (DK / 8);
                *reinterpret_cast<u32x4*>(&bb.q[row][vc * 8]) = pf.q[u];
                *reinterpret_cast<u32x4*>(&bb.k[row][vc * 8]) = pf.k[u];
            }
        }
#pragma unroll
        for (int j = 0; j < NTL; ++j) *reinterpret_cast<uint32_t*>(&bb.v[tid >> 3][j * 16 + (tid & 7) * 2]) = pf.v[j];
    };
    auto write_state = [&]() {
        if (has_tile) {
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt)
                O::store4(&sm.st[0][nt * 16 + ap.col][wave * 16 + ap.row0],
                          &sm.st[1][nt * 16 + ap.col][wave * 16 + ap.row0], S[nt]);
        }
    };
    // This wave's rows of T diag(beta) (x role) or P (q role), hi and lo, for
    // chunk c, as MFMA A operands; zero past the end.  The planes were just
    // written by gdn_prep and are shared by the d_v tiles of the group, so
    // they are read with the default policy (kept in L2).
    const int plane0 = qrole ? 2 : 0;
    // two register sets used alternately (even / odd chunks): each is
    // reloaded for chunk c + 2 right after chunk c used it, so no copy ever
    // waits on a load that was just issued
    u32x4 tpa[2][KSC], tpb[2][KSC];
    auto load_tp = [&](u32x4 (&dst)[2][KSC], int c) {
        const bool ok = c < nchunks && (xrole || qrole);
        const BufRsrc rt(TP + (cbase + (ok ? c : 0)) * static_cast<long>(H) * 4 * C * C +
                             static_cast<long>(h) * 4 * C * C,
                         ok ? 4u * C * C * 2u : 0u);
#pragma unroll
        for (int pl = 0; pl < 2; ++pl) {
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) {
                // columns 32ks.. lie wholly above the diagonal of this row
                // block: never used, so the offset points past the resource
                // (reads zero, moves no bytes) and prep does not write them
                const uint32_t offb = static_cast<uint32_t>(
                    ((plane0 + pl) * C * C + (it * 16 + (lane & 15)) * C + 32 * ks + (lane >> 4) * 8) * 2);
                dst[pl][ks] = rt.load16(32 * ks <= it * 16 + 15 ? offb : 0x80000000u);
            }
        }
    };

    fetch(0);
    stage(sm.buf[0]);
    write_state();
    load_tp(tpa, 0);
    fetch(1);
    load_tp(tpb, 1);
    lds_barrier();

    auto chunk_step = [&](int c, u32x4 (&tpc)[2][KSC]) {
        typename Sm::Buf& bb = sm.buf[c & 1];
        const int n = chunk_rows(c);
        const long tok0 = s0 + static_cast<long>(c) * C;
        f32x4 qs[NTL];
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt) qs[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

        // ---- phase A: X = K S, Y = V - diag(exp g) X (x role); Q S (q role);
        // stage chunk c+1
        if (xrole) {
            f32x4 xs[NTL];
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) xs[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) {
                const bf16x8 kf = frag_kc(&bb.k[0][0], LQ, it * 16, 32 * ks);
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt) {
                    const bf16x8 sh = frag_kc(&sm.st[0][0][0], LQ, nt * 16, 32 * ks);
                    const bf16x8 sl = frag_kc(&sm.st[1][0][0], LQ, nt * 16, 32 * ks);
                    xs[nt] = mfma_bf16(kf, sh, xs[nt]);
                    xs[nt] = mfma_bf16(kf, sl, xs[nt]);
                }
            }
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                f32x4 y;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = it * 16 + ap.row0 + r;
                    y[r] = bf16_bits_to_f32(bb.v[row][nt * 16 + ap.col]) - bb.eg[row] * xs[nt][r];
                }
                O::store4(&sm.yt[0][nt * 16 + ap.col][it * 16 + ap.row0],
                          &sm.yt[1][nt * 16 + ap.col][it * 16 + ap.row0], y);
            }
        } else if (qrole) {
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) {
                const bf16x8 qf = frag_kc(&bb.q[0][0], LQ, it * 16, 32 * ks);
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt) {
                    const bf16x8 sh = frag_kc(&sm.st[0][0][0], LQ, nt * 16, 32 * ks);
                    const bf16x8 sl = frag_kc(&sm.st[1][0][0], LQ, nt * 16, 32 * ks);
                    qs[nt] = mfma_bf16(qf, sh, qs[nt]);
                    qs[nt] = mfma_bf16(qf, sl, qs[nt]);
                }
            }
        }
        stage(sm.buf[(c + 1) & 1]);
        fetch(c + 2);
        lds_barrier();

        // ---- phase B: U = T diag(beta) Y (x role)
        if (xrole) {
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KSC; ++ks) {
                    if (32 * ks <= it * 16 + 15) {
                        const bf16x8 yh = frag_kc(&sm.yt[0][0][0], LT, nt * 16, 32 * ks);
                        const bf16x8 yl = frag_kc(&sm.yt[1][0][0], LT, nt * 16, 32 * ks);
                        u = mfma_bf16(as_bf16x8(tpc[0][ks]), yh, u);
                        u = mfma_bf16(as_bf16x8(tpc[0][ks]), yl, u);
                        u = mfma_bf16(as_bf16x8(tpc[1][ks]), yh, u);
                    }
                }
                O::store4(&sm.ut[0][nt * 16 + ap.col][it * 16 + ap.row0],
                          &sm.ut[1][nt * 16 + ap.col][it * 16 + ap.row0], u);
                f32x4 ud;
#pragma unroll
                for (int r = 0; r < 4; ++r) ud[r] = u[r] * bb.dec[it * 16 + ap.row0 + r];
                O::store4(&sm.udt[0][nt * 16 + ap.col][it * 16 + ap.row0],
                          &sm.udt[1][nt * 16 + ap.col][it * 16 + ap.row0], ud);
            }
        }
        lds_barrier();

        // ---- phase C: outputs (q role) and the state hand-off (every wave)
        if (qrole) {
            // rows past the chunk's valid ones fall outside the resource
            const BufRsrc ro(o + tok0 * vstride + h * DV + col0, rows_extent(n, vstride * TO::bytes, BV * TO::bytes));
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                f32x4 acc;
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] = qs[nt][r] * bb.eg[it * 16 + ap.row0 + r];
#pragma unroll
                for (int ks = 0; ks < KSC; ++ks) {
                    if (32 * ks <= it * 16 + 15) {
                        const bf16x8 uh = frag_kc(&sm.ut[0][0][0], LT, nt * 16, 32 * ks);
                        const bf16x8 ul = frag_kc(&sm.ut[1][0][0], LT, nt * 16, 32 * ks);
                        acc = mfma_bf16(as_bf16x8(tpc[0][ks]), uh, acc);
                        acc = mfma_bf16(as_bf16x8(tpc[0][ks]), ul, acc);
                        acc = mfma_bf16(as_bf16x8(tpc[1][ks]), uh, acc);
                    }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = it * 16 + ap.row0 + r;
                    const uint32_t offb = static_cast<uint32_t>((row * vstride + nt * 16 + ap.col) * TO::bytes);
                    if constexpr (TO::bytes == 2) ro.store_b16(f32_to_bf16_bits(acc[r]), offb);
                    else ro.store_b32(__float_as_uint(acc[r]), offb);
                }
            }
        }
        if (has_tile) {
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) S[nt] *= bb.gamma;
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) {
                const bf16x8 a = frag_km_split(&bb.k[0][0], LQ, wave * 16, 32 * ks);
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt) {
                    S[nt] = mfma_bf16(a, frag_kc_split(&sm.udt[0][0][0], LT, nt * 16, 32 * ks), S[nt]);
                    S[nt] = mfma_bf16(a, frag_kc_split(&sm.udt[1][0][0], LT, nt * 16, 32 * ks), S[nt]);
                }
            }
        }
        // checkpoint: this wave's state tile after chunk c (block-uniform test)
        const int cs = CKPT && (c + 1) * C <= L ? ckpt_slot(ck, b, (c + 1) * C, n_slots) : -1;
        if (CKPT && cs >= 0 && has_tile) {
            float* Sc = pool + (static_cast<long>(cs) * H + h) * DK * DV +
                        opaque((wave * 16 + ap.row0) * DV + col0 + ap.col);
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
#pragma unroll
                for (int r = 0; r < 4; ++r) Sc[r * DV + nt * 16] = S[nt][r];
            }
        }
        write_state();
        load_tp(tpc, c + 2);
        lds_barrier();
    };
    // pairs of chunks with no path that skips the odd one, so the compiler
    // sees the same load sequence on every trip round the loop
    int c = 0;
    for (; c + 1 < nchunks; c += 2) {
        chunk_step(c, tpa);
        chunk_step(c + 1, tpb);
    }
    if (c < nchunks) chunk_step(c, tpa);

    if (has_tile) {
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) Sg[(wave * 16 + ap.row0 + r) * DV + col0 + nt * 16 + ap.col] = S[nt][r];
        }
    }
}

// ------------------------------------------------------------------ dispatch
template <int DK, int DV, int C, class TI, class TO>
hipError_t launch_inst(const ChunkArgs& a, hipStream_t s) {
    using T = typename TI::T;
    constexpr bool F32 = (TI::bytes == 4);
    // bf16, d_k = d_v = 128, 64-token chunks: the segmented path (gdn_seg.hip)
    constexpr bool SEG = !F32 && DK == 128 && DV == 128 && C == 64;
    constexpr bool FAST = !F32 && !SEG && C >= 32 && DK >= 32;
    constexpr int PL = SEG ? 2 : (FAST ? 4 : 0);   // planes per (chunk, head); 0: fp32 T
    constexpr int BV = F32 ? 16 : (DV >= 32 ? 32 : DV);
    char* ws = static_cast<char*>(a.workspace);
    int32_t* off = reinterpret_cast<int32_t*>(ws);
    ws += align256(sizeof(int32_t) * (a.n_seqs + 1));
    int32_t* order = reinterpret_cast<int32_t*>(ws);
    ws += align256(sizeof(int32_t) * a.n_seqs);
    float* Tws = reinterpret_cast<float*>(ws);
    const long mc = max_chunks(a.n_seqs, a.n_tokens, C);
    ws += static_cast<size_t>(mc) * a.n_heads * C * C * 8;        // T / planes (8 C^2 bytes each)
    hipError_t e = hipSuccess;
    // phase 1 (state-independent): chunk offsets, order, inverses / planes
    if (a.gdn_phases != 2) {
    if constexpr (SEG) {
        e = launch_gdn_seg_offsets(a, off, ws, s);
    } else {
        hipLaunchKernelGGL(span_offsets, dim3(1), dim3(1024), 0, s, a.cu_seqlens, a.n_seqs,
                           a.n_tokens, C, 0, 0, off, FAST ? order : nullptr);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    if (a.n_tokens > 0 && SEG) {
        // one wave per (chunk, head) item (gdn_seg.hip)
        e = launch_gdn_seg_prep(a, off, reinterpret_cast<uint16_t*>(Tws), mc, s);
        if (e != hipSuccess) return e;
    } else if (a.n_tokens > 0) {
        // persistent: as many workgroups as are resident at once, striding over
        // the (chunk, head) items
        const long prep_blocks = std::min<long>(mc * a.n_heads, kPrepBlocks);
        hipLaunchKernelGGL((gdn_prep<DK, C, TI, PL>), dim3(static_cast<unsigned>(prep_blocks)),
                           dim3(NT), 0, s, static_cast<const T*>(a.k), static_cast<const T*>(a.q),
                           a.alpha, a.beta, a.cu_seqlens, a.n_seqs, a.n_tokens, a.n_heads, off,
                           static_cast<void*>(Tws));
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    }
    if (a.gdn_phases == 1) return hipSuccess;
    // phase 2: the serial chunk loop
    if constexpr (SEG) {
        return launch_gdn_seg(a, off, reinterpret_cast<const uint16_t*>(Tws), mc, ws, s);
    } else if constexpr (FAST) {
        const long groups = (static_cast<long>(a.n_seqs) * a.n_heads + 7) / 8 * 8;
        // 32 state columns per workgroup when there are workgroups to spare
        // (at least four per compute unit at 16 columns): the per-chunk work
        // that does not depend on the columns (staging q and k, the T / P
        // planes, the barriers) is then shared by twice the columns
        const bool wide = DV % 32 == 0 && groups * (DV / 16) >= kWideMin;
        const long blocks = groups * (DV / (wide ? 32 : 16));
        const Ckpt ck{a.ckpt_slots, a.ckpt_interval, a.ckpt_stride};
        auto serial = [&](auto kern) {
            hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(FT), 0, s,
                               static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                               static_cast<const uint16_t*>(a.v), a.alpha, a.cu_seqlens, a.n_seqs,
                               a.n_tokens, a.n_heads, a.pool, a.n_slots, a.slot_idx, a.zero_init, off,
                               order, mc, reinterpret_cast<const uint16_t*>(Tws), ck,
                               static_cast<typename TO::T*>(a.o));
        };
        // the checkpoint stores are compiled in only where they are asked for
        if constexpr (DV % 32 == 0) {
            if (wide) {
                if (ck.slots) serial(gdn_fast_kernel<DK, DV, C, TO, true, 32>);
                else serial(gdn_fast_kernel<DK, DV, C, TO, false, 32>);
                return hipGetLastError();
            }
        }
        if (ck.slots) serial(gdn_fast_kernel<DK, DV, C, TO, true, 16>);
        else serial(gdn_fast_kernel<DK, DV, C, TO, false, 16>);
        return hipGetLastError();
    } else {
        const long blocks = static_cast<long>(a.n_seqs) * a.n_heads * (DV / BV);
        hipLaunchKernelGGL((gdn_chunk_kernel<DK, DV, BV, C, TI, TO>), dim3(static_cast<unsigned>(blocks)),
                           dim3(NT), 0, s, static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                           static_cast<const T*>(a.v), a.alpha, a.beta, a.cu_seqlens, a.n_seqs, a.n_tokens,
                           a.n_heads, a.pool, a.n_slots, a.slot_idx, a.zero_init, off, mc, Tws,
                           Ckpt{a.ckpt_slots, a.ckpt_interval, a.ckpt_stride},
                           static_cast<typename TO::T*>(a.o));
        return hipGetLastError();
    }
}

template <int DK, int DV, class TI, class TO>
hipError_t launch_c(const ChunkArgs& a, hipStream_t s) {
    switch (a.chunk) {
        case 16: return launch_inst<DK, DV, 16, TI, TO>(a, s);
        case 32: return launch_inst<DK, DV, 32, TI, TO>(a, s);
        case 64: return launch_inst<DK, DV, 64, TI, TO>(a, s);
    }
    return hipErrorInvalidValue;
}

template <int DK, int DV>
hipError_t launch_dt(const ChunkArgs& a, hipStream_t s) {
    if (a.in_bf16) return a.out_bf16 ? launch_c<DK, DV, BF16, BF16>(a, s) : launch_c<DK, DV, BF16, F32>(a, s);
    return a.out_bf16 ? launch_c<DK, DV, F32, BF16>(a, s) : launch_c<DK, DV, F32, F32>(a, s);
}

template <int DK>
hipError_t launch_dv(const ChunkArgs& a, hipStream_t s) {
    switch (a.dv) {
        case 16: return launch_dt<DK, 16>(a, s);
        case 32: return launch_dt<DK, 32>(a, s);
        case 64: return launch_dt<DK, 64>(a, s);
        case 128: return launch_dt<DK, 128>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

size_t gdn_chunk_workspace(int n_seqs, int n_tokens, int n_heads, int dk, int dv, int chunk) {
    // per (chunk, head): T in fp32 (generic path) or four bf16 planes (bf16 path): 8 C^2 bytes
    // plus chunk offsets and the longest-first sequence order
    // (and, for the segmented path at d_k = d_v = 128 and chunk 64, its segment bookkeeping and states)
    const size_t seg = (dk == 128 && dv == 128 && chunk == 64) ? gdn_seg_workspace(n_seqs, n_tokens, n_heads) : 0;
    return align256(sizeof(int32_t) * (n_seqs + 1)) + align256(sizeof(int32_t) * n_seqs) +
           static_cast<size_t>(max_chunks(n_seqs, n_tokens, chunk)) * n_heads * chunk * chunk * 8 + seg;
}

hipError_t launch_gdn_chunk(const ChunkArgs& a, hipStream_t s) {
    switch (a.dk) {
        case 16: return launch_dv<16>(a, s);
        case 32: return launch_dv<32>(a, s);
        case 64: return launch_dv<64>(a, s);
        case 128: return launch_dv<128>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gla
