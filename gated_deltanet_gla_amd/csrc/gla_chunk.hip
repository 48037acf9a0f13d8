// Chunked GLA prefill on gfx950.
//
// "Inference for linear attention and hybrid architectures", section "Two
// ways to write the same computation", the chunked form: inside a chunk of
// C tokens, with g the running sum of log alpha restarted at the chunk,
//   O = ((Q K^T) .* D) V + diag(exp g) Q S,   D_ij = exp(g_i - g_j) [j <= i]
//   S <- exp(g_last) S + (diag(exp(g_last - g)) K)^T V
// and only the state is handed from one chunk to the next (and, through the
// pool, from one call to the next).
//
// Work split: one workgroup per (sequence, head, d_v tile of BV columns).
// State columns evolve independently under this update, so tiling d_v is
// exact; the tiles of one (sequence, head) re-read the same q/k chunk, which
// the XCD-aware block order keeps in one L2.  The BV-column slice of the
// fp32 state stays in MFMA accumulators for the whole sequence.
//
// Eight waves with two roles, one of each per SIMD, so that the VALU work of
// one role overlaps the MFMA work of the other:
//  * output waves 0..3: wave w owns chunk rows 16w..16w+15.  It forms
//    P^T = K Q^T for its rows in accumulators, decays and masks it; the P^T
//    accumulator tile already has the lane layout of an MFMA A operand
//    (lane = row, 4 consecutive tokens), so P never goes through LDS.  Then
//    O = diag(exp g) (Q S) + P V for its rows, stored straight to HBM.
//  * state waves 4..7: each owns a share of the state tiles (weighted so
//    every SIMD gets about the same MFMA count) and applies
//    S = exp(g_last) S + K^T (diag(exp(g_last - g)) V); then they write the
//    updated slice for the next chunk's Q S, stage the next chunk (already
//    in registers) into the other LDS buffer and prefetch the one after.
// q, k, v sit in LDS in their natural token-major layout; contractions over
// tokens read them with the LDS transpose read.  One LDS-only barrier per
// chunk (fp32 inputs use a single buffer and two).
//
// NORM = true is normalised kernelised linear attention (page "Long
// context, fast inference, smart decoding, and life beyond attention",
// section "Linear attention: removing softmax entirely", and its
// running-state listing): phi(x) = elu(x) + 1 is applied to q and k as they
// are staged, there is no gate (alpha = 1), and the output is divided by
// phi(q_i) . z_i + eps with z_i = z_in + sum_{j<=i} phi(k_j).  Inside a chunk
// that normaliser is the row sum of the masked score tile P (which the
// output waves hold anyway) plus phi(q_i) . z_in; the state waves carry z
// from chunk to chunk in a double-buffered LDS vector.
#include <algorithm>

#include "chunk_common.h"
#include "launch.h"

namespace gla {
namespace {

constexpr int NW = 8;
constexpr int NT = NW * 64;
constexpr int NO = 4;            // output waves
constexpr int NS = NW - NO;      // state waves

template <int DK, int BV, int C, bool F32>
struct GlaBuf {
    using E = typename Op<F32>::E;
    static constexpr int PAD = Op<F32>::PAD;
    static constexpr int LQ = DK + PAD;   // q, k rows (token-major) and st lines
    static constexpr int LV = BV + PAD;   // v, vd rows (token-major)
    static constexpr int HL = F32 ? 1 : 2;
    alignas(16) E q[C][LQ];
    alignas(16) E k[C][LQ];
    alignas(16) E v[C][LV];
    alignas(16) E vd[HL][C][LV];    // diag(exp(g_last - g)) V  (hi, lo)
    alignas(16) E st[HL][BV][LQ];   // state slice, line = column n, k = d (hi, lo)
    float g2[C];                    // log2 of the cumulative decay
    float eg[C];                    // exp(g)
    float gamma;                    // exp(g_last)
};

// Split of the state tiles over the state waves.  State wave s shares a SIMD
// with output wave s, whose MFMA count grows with its row block; tiles go
// greedily to the SIMD with the least work.
template <int DK, int BV, int C>
struct StateSplit {
    static constexpr int KT = DK / 16, BT = BV / 16, CT = C / 16, ST = KT * BT;
    struct Tab { int beg[NS + 1]; int maxcnt; };
    static constexpr Tab make() {
        Tab t{};
        int load[NS] = {};
        int cnt[NS] = {};
        const int kd = DK >= 32 ? DK / 32 : 1;
        const int kc = C >= 32 ? C / 32 : 1;
        for (int s = 0; s < NS; ++s) {
            if (s < CT) load[s] = (s + 1) * kd + BT * 2 * kd + BT * 2 * (s / 2 + 1);
        }
        for (int i = 0; i < ST; ++i) {
            int best = 0;
            for (int s = 1; s < NS; ++s)
                if (load[s] < load[best]) best = s;
            load[best] += 2 * kc;
            cnt[best] += 1;
        }
        t.beg[0] = 0;
        t.maxcnt = 0;
        for (int s = 0; s < NS; ++s) {
            t.beg[s + 1] = t.beg[s] + cnt[s];
            if (cnt[s] > t.maxcnt) t.maxcnt = cnt[s];
        }
        return t;
    }
    static constexpr Tab tab = make();
};

template <class TI, int C, int DK, int BV>
struct Prefetch {
    static constexpr int NTS = NS * 64;                  // staging threads
    static constexpr int VE = 16 / TI::bytes;            // elements per 16-byte vector
    static constexpr int NQ = (C * DK / VE + NTS - 1) / NTS;
    static constexpr int NV = (C * BV / VE + NTS - 1) / NTS;
    u32x4 q[NQ], k[NQ], v[NV];
    float a;   // alpha of row (lane) in every state wave; 1 for rows >= n
    int n;     // valid rows of the fetched chunk

    template <bool GATED>
    __device__ __forceinline__ void load(int st, const typename TI::T* qg, const typename TI::T* kg,
                                         const typename TI::T* vg, const float* ag, long tstride,
                                         long vstride, long astride, int n) {
        this->n = n;
#pragma unroll
        for (int u = 0; u < NQ; ++u) {
            const int x = st + u * NTS;
            const int row = x / (DK / VE), vc = x % (DK / VE);
            q[u] = u32x4{0u, 0u, 0u, 0u};
            k[u] = u32x4{0u, 0u, 0u, 0u};
            if (x < C * DK / VE && row < n) {
                q[u] = *reinterpret_cast<const u32x4*>(qg + row * tstride + vc * VE);
                k[u] = *reinterpret_cast<const u32x4*>(kg + row * tstride + vc * VE);
            }
        }
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int x = st + u * NTS;
            const int row = x / (BV / VE), vc = x % (BV / VE);
            v[u] = u32x4{0u, 0u, 0u, 0u};
            if (x < C * BV / VE && row < n) v[u] = *reinterpret_cast<const u32x4*>(vg + row * vstride + vc * VE);
        }
        const int lane = st & 63;
        a = (GATED && lane < n && lane < C) ? ag[lane * astride] : 1.f;
    }
};

// phi(x) = elu(x) + 1 on one 16-byte vector of staged elements
__device__ __forceinline__ float elu1(float x) { return x > 0.f ? x + 1.f : expf(x); }
template <class TI> __device__ __forceinline__ u32x4 phi_vec(u32x4 w);
template <> __device__ __forceinline__ u32x4 phi_vec<F32>(u32x4 w) {
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = __float_as_uint(elu1(__uint_as_float(w[e])));
    return r;
}
template <> __device__ __forceinline__ u32x4 phi_vec<BF16>(u32x4 w) {
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        r[e] = pack_bf16x2(elu1(__uint_as_float(w[e] << 16)), elu1(__uint_as_float(w[e] & 0xffff0000u)));
    return r;
}

template <int DK, int DV, int BV, int C, class TI, class TO, bool NORM>
__global__ void __launch_bounds__(NT)
gla_chunk_kernel(const typename TI::T* __restrict__ q, const typename TI::T* __restrict__ k,
                 const typename TI::T* __restrict__ v, const float* __restrict__ alpha,
                 const int32_t* __restrict__ cu, int n_seqs, int n_tokens, int H,
                 float* __restrict__ pool, int n_slots, const int32_t* __restrict__ slot_idx,
                 int zero_init, Ckpt ck, float* __restrict__ zpool, const float* __restrict__ zsnap,
                 float eps, typename TO::T* __restrict__ o) {
    constexpr bool F32 = (TI::bytes == 4);
    using O = Op<F32>;
    using E = typename O::E;
    using Buf = GlaBuf<DK, BV, C, F32>;
    using PF = Prefetch<TI, C, DK, BV>;
    using SS = StateSplit<DK, BV, C>;
    constexpr int NBUF = F32 ? 1 : 2;
    constexpr int LQ = Buf::LQ, LV = Buf::LV;
    constexpr int LO = F32 ? 0 : 1;
    constexpr int NVT = DV / BV;
    constexpr int CT = C / 16;                   // 16-row tiles per chunk
    constexpr int BT = BV / 16;                  // 16-col tiles per d_v tile
    constexpr int KSD = DK / 32;                 // 32-wide k steps over d_k (0 when DK = 16)
    constexpr int SMAX = SS::tab.maxcnt > 0 ? SS::tab.maxcnt : 1;
    constexpr int VE = PF::VE;
    static_assert(DV % BV == 0 && BV % 16 == 0 && C % 16 == 0 && C <= 64 && CT <= NO, "tiling");

    __shared__ Buf buf[NBUF];
    __shared__ float zb[NORM ? 2 : 1][NORM ? DK : 1];   // normaliser z, by chunk parity

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
    const int nchunks = (L + C - 1) / C;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const bool is_state = wave >= NO;
    const int sw = wave - NO;                    // state wave index
    const int stid = tid - NO * 64;              // staging thread index
    const AccPos ap;
    const int col0 = vt * BV;
    const long tstride = static_cast<long>(H) * DK;
    const long vstride = static_cast<long>(H) * DV;

    // ---- this state wave's tiles; initial state slice -> accumulators
    const int tbeg = is_state ? SS::tab.beg[sw] : 0;
    const int tcnt = is_state ? SS::tab.beg[sw + 1] - SS::tab.beg[sw] : 0;
    float* Sg = pool + (static_cast<long>(slot) * H + h) * DK * DV;
    f32x4 S[SMAX];
#pragma unroll
    for (int i = 0; i < SMAX; ++i) {
        S[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (i < tcnt && !zero_init) {
            const int t = tbeg + i;
            const int mt = t / BT, nt = t % BT;
#pragma unroll
            for (int r = 0; r < 4; ++r) S[i][r] = Sg[(mt * 16 + ap.row0 + r) * DV + col0 + nt * 16 + ap.col];
        }
    }

    PF pf;
    auto fetch = [&](int c) {
        const long tok0 = s0 + static_cast<long>(c) * C;
        pf.template load<!NORM>(stid, q + tok0 * tstride + h * DK, k + tok0 * tstride + h * DK,
                v + tok0 * vstride + h * DV + col0, alpha + tok0 * H + h, tstride, vstride, H,
                min(C, L - c * C));
    };
    // State waves: write the prefetched chunk and the current state slice into bb.
    auto stage = [&](Buf& bb) {
        float x = __log2f(fmaxf(pf.a, kMinDecay));   // in-wave scan, log2 domain
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        const float glast = __shfl(x, C - 1, 64);
        if (sw == 0 && lane < C) {
            bb.g2[lane] = x;
            bb.eg[lane] = exp2f(x);
        }
        if (stid == 0) bb.gamma = exp2f(glast);
#pragma unroll
        for (int u = 0; u < PF::NQ; ++u) {
            const int xx = stid + u * PF::NTS;
            if (xx < C * DK / VE) {
                const int row = xx / (DK / VE), vc = xx % (DK / VE);
                u32x4 qv = pf.q[u], kv = pf.k[u];
                if constexpr (NORM) {
                    // rows past the sequence stay zero (phi(0) = 1 would count them)
                    if (row < pf.n) {
                        qv = phi_vec<TI>(qv);
                        kv = phi_vec<TI>(kv);
                    }
                }
                *reinterpret_cast<u32x4*>(&bb.q[row][vc * VE]) = qv;
                *reinterpret_cast<u32x4*>(&bb.k[row][vc * VE]) = kv;
            }
        }
#pragma unroll
        for (int u = 0; u < PF::NV; ++u) {
            const int xx = stid + u * PF::NTS;
            const int row = xx / (BV / VE), vc = xx % (BV / VE);
            const float dec = exp2f(glast - __shfl(x, row & 63, 64));
            if (xx < C * BV / VE) {
                *reinterpret_cast<u32x4*>(&bb.v[row][vc * VE]) = pf.v[u];
                const E* e = reinterpret_cast<const E*>(&pf.v[u]);
#pragma unroll
                for (int j = 0; j < VE; j += 4) {
                    f32x4 y;
#pragma unroll
                    for (int r = 0; r < 4; ++r) y[r] = O::load1(e + j + r) * dec;
                    O::store4(&bb.vd[0][row][vc * VE + j], &bb.vd[LO][row][vc * VE + j], y);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < SMAX; ++i) {
            if (i < tcnt) {
                const int t = tbeg + i;
                const int mt = t / BT, nt = t % BT;
                const int ln = nt * 16 + ap.col;
                O::store4(&bb.st[0][ln][mt * 16 + ap.row0], &bb.st[LO][ln][mt * 16 + ap.row0], S[i]);
            }
        }
    };

    if (is_state && nchunks > 0) {
        fetch(0);
        stage(buf[0]);
        if (nchunks > 1) fetch(1);
    }
    const long zoff = (static_cast<long>(slot) * H + h) * DK;
    if constexpr (NORM) {
        // with several d_v tiles per head, the entry z comes from a copy
        // taken before the launch: tile 0 writes the final z to norm_pool,
        // possibly before another tile of the same head has started
        const float* zsrc = zsnap ? zsnap + (static_cast<long>(b) * H + h) * DK : zpool + zoff;
        for (int d = tid; d < DK; d += NT) zb[0][d] = zero_init ? 0.f : zsrc[d];
    }
    lds_barrier();

    for (int c = 0; c < nchunks; ++c) {
        Buf& bb = buf[c % NBUF];
        const int n = min(C, L - c * C);
        const long tok0 = s0 + static_cast<long>(c) * C;

        if (!is_state) {
            const int it = wave;
            if (it < CT) {
                const int i = it * 16 + ap.col;       // row held by this lane in the P^T tiles
                const float gi = bb.g2[i];
                // ---- P^T tiles (rows j, cols i) and Q S for this wave's rows
                f32x4 pt[CT];
                f32x4 ov[BT];
                if constexpr (F32) {
#pragma unroll
                    for (int jt = 0; jt < CT; ++jt) {
                        pt[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
                        if (jt <= it) O::mma(pt[jt], &bb.k[jt * 16][0], LQ, &bb.q[it * 16][0], LQ, DK);
                    }
#pragma unroll
                    for (int nt = 0; nt < BT; ++nt) {
                        ov[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
                        O::mma(ov[nt], &bb.q[it * 16][0], LQ, &bb.st[0][nt * 16][0], LQ, DK);
                    }
                } else if constexpr (KSD == 0) {
                    const s16x4 qf = frag_kc4(&bb.q[0][0], LQ, it * 16, 0);
#pragma unroll
                    for (int jt = 0; jt < CT; ++jt) {
                        pt[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
                        if (jt <= it) pt[jt] = mfma_bf16_k16(frag_kc4(&bb.k[0][0], LQ, jt * 16, 0), qf, pt[jt]);
                    }
#pragma unroll
                    for (int nt = 0; nt < BT; ++nt) {
                        ov[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
                        ov[nt] = mfma_bf16_k16(qf, frag_kc4(&bb.st[0][0][0], LQ, nt * 16, 0), ov[nt]);
                        ov[nt] = mfma_bf16_k16(qf, frag_kc4(&bb.st[LO][0][0], LQ, nt * 16, 0), ov[nt]);
                    }
                } else {
                    bf16x8 qf[KSD];                   // this wave's q rows: B of P^T, A of Q S
#pragma unroll
                    for (int ks = 0; ks < KSD; ++ks) qf[ks] = frag_kc(&bb.q[0][0], LQ, it * 16, 32 * ks);
#pragma unroll
                    for (int jt = 0; jt < CT; ++jt) {
                        pt[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
                        if (jt <= it) {
#pragma unroll
                            for (int ks = 0; ks < KSD; ++ks)
                                pt[jt] = mfma_bf16(frag_kc(&bb.k[0][0], LQ, jt * 16, 32 * ks), qf[ks], pt[jt]);
                        }
                    }
#pragma unroll
                    for (int nt = 0; nt < BT; ++nt) {
                        ov[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < KSD; ++ks) {
                            ov[nt] = mfma_bf16(qf[ks], frag_kc(&bb.st[0][0][0], LQ, nt * 16, 32 * ks), ov[nt]);
                            ov[nt] = mfma_bf16(qf[ks], frag_kc(&bb.st[LO][0][0], LQ, nt * 16, 32 * ks), ov[nt]);
                        }
                    }
                }
                // decay exp(g_i - g_j) on tiles below the diagonal; mask j > i on the diagonal one
#pragma unroll
                for (int jt = 0; jt < CT; ++jt) {
                    if (jt < it) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) pt[jt][r] *= exp2f(gi - bb.g2[jt * 16 + ap.row0 + r]);
                    } else if (jt == it) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int j = jt * 16 + ap.row0 + r;
                            pt[jt][r] = (j <= i) ? pt[jt][r] * exp2f(gi - bb.g2[j]) : 0.f;
                        }
                    }
                }
                // ---- normaliser of this wave's rows: row sums of P (rows j are
                // spread over the 4 lane groups) + phi(q_i) . z_in, then moved
                // to the output tile layout (lane holds rows row0 .. row0 + 3)
                float rden[4] = {1.f, 1.f, 1.f, 1.f};
                if constexpr (NORM) {
                    float ps = 0.f;
#pragma unroll
                    for (int jt = 0; jt < CT; ++jt) {
                        if (jt <= it) {
#pragma unroll
                            for (int r = 0; r < 4; ++r) ps += pt[jt][r];
                        }
                    }
                    const float* zin = zb[c & 1];
                    for (int d = lane >> 4; d < DK; d += 4) ps += O::load1(&bb.q[i][d]) * zin[d];
                    ps += __shfl_xor(ps, 16, 64);
                    ps += __shfl_xor(ps, 32, 64);
                    const float den = ps + eps;
#pragma unroll
                    for (int r = 0; r < 4; ++r) rden[r] = 1.f / __shfl(den, ap.row0 + r, 64);
                }
                // ---- O = diag(exp g) Q S + P V
#pragma unroll
                for (int nt = 0; nt < BT; ++nt) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) ov[nt][r] *= bb.eg[it * 16 + ap.row0 + r];
                    if constexpr (F32) {
#pragma unroll
                        for (int jt = 0; jt < CT; ++jt) {
                            if (jt <= it) {
#pragma unroll
                                for (int r = 0; r < 4; ++r)
                                    ov[nt] = mfma_f32(pt[jt][r], bb.v[jt * 16 + ap.row0 + r][nt * 16 + ap.col], ov[nt]);
                            }
                        }
                    } else if constexpr (CT == 1) {
                        s16x4 hi, lo;
                        split4(pt[0], hi, lo);
                        const s16x4 bv = frag_km4(&bb.v[0][0], LV, nt * 16, 0);
                        ov[nt] = mfma_bf16_k16(hi, bv, ov[nt]);
                        ov[nt] = mfma_bf16_k16(lo, bv, ov[nt]);
                    } else {
#pragma unroll
                        for (int s = 0; s < CT / 2; ++s) {
                            if (2 * s <= it) {
                                s16x4 h0, l0, h1, l1;
                                split4(pt[2 * s], h0, l0);
                                split4(pt[2 * s + 1], h1, l1);
                                const bf16x8 bv = frag_km_split(&bb.v[0][0], LV, nt * 16, 32 * s);
                                ov[nt] = mfma_bf16(cat8(h0, h1), bv, ov[nt]);
                                ov[nt] = mfma_bf16(cat8(l0, l1), bv, ov[nt]);
                            }
                        }
                    }
                    const int colg = col0 + nt * 16 + ap.col;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = it * 16 + ap.row0 + r;
                        if (row < n) TO::store(o, (tok0 + row) * vstride + h * DV + colg, ov[nt][r] * rden[r]);
                    }
                }
            }
        } else {
            // ---- state hand-off for this wave's tiles
            const float gam = bb.gamma;
#pragma unroll
            for (int si = 0; si < SMAX; ++si) {
                if (si < tcnt) {
                    const int t = tbeg + si;
                    const int mt = t / BT, nt = t % BT;
                    S[si] *= gam;
                    if constexpr (F32) {
#pragma unroll
                        for (int jb = 0; jb < C; jb += 16) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const int j = jb + (lane >> 4) * 4 + e;
                                S[si] = mfma_f32(bb.k[j][mt * 16 + (lane & 15)], bb.vd[0][j][nt * 16 + (lane & 15)], S[si]);
                            }
                        }
                    } else if constexpr (C == 16) {
                        const s16x4 a = frag_km4(&bb.k[0][0], LQ, mt * 16, 0);
                        S[si] = mfma_bf16_k16(a, frag_km4(&bb.vd[0][0][0], LV, nt * 16, 0), S[si]);
                        S[si] = mfma_bf16_k16(a, frag_km4(&bb.vd[LO][0][0], LV, nt * 16, 0), S[si]);
                    } else {
#pragma unroll
                        for (int k0 = 0; k0 < C; k0 += 32) {
                            const bf16x8 a = frag_km_split(&bb.k[0][0], LQ, mt * 16, k0);
                            S[si] = mfma_bf16(a, frag_km_split(&bb.vd[0][0][0], LV, nt * 16, k0), S[si]);
                            S[si] = mfma_bf16(a, frag_km_split(&bb.vd[LO][0][0], LV, nt * 16, k0), S[si]);
                        }
                    }
                }
            }
            // normaliser after chunk c: z += sum over its rows of phi(k)
            if constexpr (NORM) {
                for (int d = stid; d < DK; d += NS * 64) {
                    float zacc = zb[c & 1][d];
                    for (int j = 0; j < C; ++j) zacc += O::load1(&bb.k[j][d]);
                    zb[(c + 1) & 1][d] = zacc;
                }
            }
            // checkpoint: this wave's tiles of the state after chunk c
            const int cs = (c + 1) * C <= L ? ckpt_slot(ck, b, (c + 1) * C, n_slots) : -1;
            if (cs >= 0) {
                float* Sc = pool + (static_cast<long>(cs) * H + h) * DK * DV +
                            opaque(ap.row0 * DV + col0 + ap.col);
#pragma unroll
                for (int i = 0; i < SMAX; ++i) {
                    if (i < tcnt) {
                        const int t = tbeg + i;
                        const int mt = t / BT, nt = t % BT;
#pragma unroll
                        for (int r = 0; r < 4; ++r) Sc[(mt * 16 + r) * DV + nt * 16] = S[i][r];
                    }
                }
            }
            if (c + 1 < nchunks && NBUF == 2) {
                stage(buf[(c + 1) % NBUF]);
                if (c + 2 < nchunks) fetch(c + 2);
            }
        }
        if constexpr (NBUF == 1) {
            if (c + 1 < nchunks) {
                lds_barrier();                 // everyone done with the single buffer
                if (is_state) {
                    stage(buf[0]);
                    if (c + 2 < nchunks) fetch(c + 2);
                }
            }
        }
        lds_barrier();
    }

    if constexpr (NORM) {
        if (vt == 0) {
            for (int d = tid; d < DK; d += NT) zpool[zoff + d] = zb[nchunks & 1][d];
        }
    }
    // ---- final state slice -> pool (zeros for an empty sequence with zero-init)
#pragma unroll
    for (int i = 0; i < SMAX; ++i) {
        if (i < tcnt) {
            const int t = tbeg + i;
            const int mt = t / BT, nt = t % BT;
#pragma unroll
            for (int r = 0; r < 4; ++r) Sg[(mt * 16 + ap.row0 + r) * DV + col0 + nt * 16 + ap.col] = S[i][r];
        }
    }
}

// Copy of every sequence's entry normaliser z (norm_pool[slot_idx[b]], all
// heads) into snap[b][h][:], for the chunk kernel's d_v tiles to read.
__global__ void __launch_bounds__(256)
z_snapshot(const float* __restrict__ zpool, int n_slots, const int32_t* __restrict__ slot_idx, int n_seqs,
           int H, int dk, float* __restrict__ snap) {
    const long n = static_cast<long>(n_seqs) * H * dk;
    for (long i = blockIdx.x * 256L + threadIdx.x; i < n; i += gridDim.x * 256L) {
        const long bh = i / dk;
        const int b = static_cast<int>(bh / H);
        const int slot = slot_idx[b];
        snap[i] = (slot >= 0 && slot < n_slots) ? zpool[(static_cast<long>(slot) * H + bh % H) * dk + i % dk] : 0.f;
    }
}

template <int DK, int DV, int BV, int C, class TI, class TO, bool NORM>
hipError_t launch_inst(const ChunkArgs& a, hipStream_t s) {
    using T = typename TI::T;
    const long blocks = static_cast<long>(a.n_seqs) * a.n_heads * (DV / BV);
    const float* zsnap = nullptr;
    if (NORM && DV / BV > 1 && !a.zero_init) {
        // the workspace holds the entry z of every (sequence, head)
        float* snap = static_cast<float*>(a.workspace);
        const long n = static_cast<long>(a.n_seqs) * a.n_heads * DK;
        hipLaunchKernelGGL(z_snapshot, dim3(static_cast<unsigned>(std::min<long>((n + 255) / 256, 1024))),
                           dim3(256), 0, s, a.zpool, a.n_slots, a.slot_idx, a.n_seqs, a.n_heads, DK, snap);
        zsnap = snap;
    }
    hipLaunchKernelGGL((gla_chunk_kernel<DK, DV, BV, C, TI, TO, NORM>), dim3(static_cast<unsigned>(blocks)),
                       dim3(NT), 0, s, static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), a.alpha, a.cu_seqlens, a.n_seqs, a.n_tokens,
                       a.n_heads, a.pool, a.n_slots, a.slot_idx, a.zero_init,
                       Ckpt{a.ckpt_slots, a.ckpt_interval, a.ckpt_stride}, a.zpool, zsnap, a.eps,
                       static_cast<typename TO::T*>(a.o));
    return hipGetLastError();
}

template <int DK, int DV, int C, class TI, class TO, bool NORM>
hipError_t launch_bv(const ChunkArgs& a, hipStream_t s) {
    constexpr int BV = DV >= 32 ? 32 : DV;
    return launch_inst<DK, DV, BV, C, TI, TO, NORM>(a, s);
}

template <int DK, int DV, class TI, class TO, bool NORM>
hipError_t launch_c(const ChunkArgs& a, hipStream_t s) {
    switch (a.chunk) {
        case 16: return launch_bv<DK, DV, 16, TI, TO, NORM>(a, s);
        case 32: return launch_bv<DK, DV, 32, TI, TO, NORM>(a, s);
        case 64: return launch_bv<DK, DV, 64, TI, TO, NORM>(a, s);
    }
    return hipErrorInvalidValue;
}

template <int DK, int DV, bool NORM>
hipError_t launch_dt(const ChunkArgs& a, hipStream_t s) {
    if (a.in_bf16)
        return a.out_bf16 ? launch_c<DK, DV, BF16, BF16, NORM>(a, s) : launch_c<DK, DV, BF16, F32, NORM>(a, s);
    return a.out_bf16 ? launch_c<DK, DV, F32, BF16, NORM>(a, s) : launch_c<DK, DV, F32, F32, NORM>(a, s);
}

template <int DK, bool NORM>
hipError_t launch_dv(const ChunkArgs& a, hipStream_t s) {
    switch (a.dv) {
        case 16: return launch_dt<DK, 16, NORM>(a, s);
        case 32: return launch_dt<DK, 32, NORM>(a, s);
        case 64: return launch_dt<DK, 64, NORM>(a, s);
        case 128: return launch_dt<DK, 128, NORM>(a, s);
    }
    return hipErrorInvalidValue;
}

template <bool NORM>
hipError_t launch_dk(const ChunkArgs& a, hipStream_t s) {
    switch (a.dk) {
        case 16: return launch_dv<16, NORM>(a, s);
        case 32: return launch_dv<32, NORM>(a, s);
        case 64: return launch_dv<64, NORM>(a, s);
        case 128: return launch_dv<128, NORM>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

size_t gla_chunk_workspace(int n_seqs, int n_tokens, int n_heads, int dk, int dv, int chunk) {
    // the segmented bf16 path (d_k = d_v = 128, chunk 64) keeps per-segment
    // states in the workspace; the dtype is not known here, so the bound
    // covers both dtypes
    if (dk == 128 && dv == 128 && chunk == 64) return gla_seg_workspace(n_seqs, n_tokens, n_heads);
    return 0;
}

hipError_t launch_gla_chunk(const ChunkArgs& a, hipStream_t s) {
    if (gla_seg_supported(a)) return launch_gla_seg(a, s);
    return launch_dk<false>(a, s);
}

// The generic path splits d_v into 32-column tiles; with more than one per
// head it needs the entry normalisers copied to the workspace first.
size_t lin_attn_chunk_workspace(int n_seqs, int n_tokens, int n_heads, int dk, int dv, int chunk) {
    const size_t snap = dv > 32 ? static_cast<size_t>(n_seqs) * n_heads * dk * sizeof(float) : 0;
    return std::max(snap, gla_chunk_workspace(n_seqs, n_tokens, n_heads, dk, dv, chunk));
}

hipError_t launch_lin_attn_chunk(const ChunkArgs& a, hipStream_t s) {
    // bf16, d_k = d_v = 128, chunk 64 with a workspace: the segmented passes
    if (gla_seg_supported(a) && a.workspace != nullptr) return launch_lin_attn_seg(a, s);
    return launch_dk<true>(a, s);
}

}  // namespace gla
