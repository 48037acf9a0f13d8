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
// Work split: one workgroup (4 waves) per (sequence, head, d_v tile of BV
// columns).  Columns of the state evolve independently under this update,
// so tiling d_v is exact; the tiles of one (sequence, head) re-read the same
// q/k chunk, which the XCD-aware block order keeps in one L2.  The BV-column
// slice of the fp32 state stays in MFMA accumulators for the whole sequence.
//
// Per chunk, wave w owns the 16 output rows 16w..16w+15:
//   P^T = K Q^T for its rows (accumulators), masked and decayed; the P^T
//         accumulator tile already has the lane layout of an MFMA A operand
//         (lane = row i, 4 consecutive j), so P never goes through LDS;
//   O   = diag(exp g) (Q S) + P V  for its rows, stored straight to HBM;
// and a share of the state tiles:
//   S   = exp(g_last) S + K^T (diag(exp(g_last - g)) V).
// q, k, v are staged in LDS in their natural token-major layout; the
// contractions over tokens read them with the LDS transpose read, so
// nothing is transposed on the way in.  Chunk c+1 is fetched from HBM into
// registers while chunk c computes, and written to the second LDS buffer
// after it; one barrier per chunk (fp32 inputs use one buffer and two).
#include "chunk_common.h"
#include "launch.h"

namespace gla {
namespace {

constexpr int NW = 4;
constexpr int NT = NW * 64;

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
    float g[C];
    float eg[C];
    float gamma;
};

template <class TI, int C, int DK, int BV>
struct Prefetch {
    static constexpr int VE = 16 / TI::bytes;            // elements per 16-byte vector
    static constexpr int NQ = (C * DK / VE + NT - 1) / NT;
    static constexpr int NV = (C * BV / VE + NT - 1) / NT;
    u32x4 q[NQ], k[NQ], v[NV];
    float a;   // alpha of row (lane) in every wave; 1 for rows >= n

    __device__ __forceinline__ void load(const typename TI::T* qg, const typename TI::T* kg,
                                         const typename TI::T* vg, const float* ag, long tstride,
                                         long vstride, long astride, int n) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int u = 0; u < NQ; ++u) {
            const int x = tid + u * NT;
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
            const int x = tid + u * NT;
            const int row = x / (BV / VE), vc = x % (BV / VE);
            v[u] = u32x4{0u, 0u, 0u, 0u};
            if (x < C * BV / VE && row < n) v[u] = *reinterpret_cast<const u32x4*>(vg + row * vstride + vc * VE);
        }
        const int lane = tid & 63;
        a = (lane < n && lane < C) ? ag[lane * astride] : 1.f;
    }
};

template <int DK, int DV, int BV, int C, class TI, class TO>
__global__ void __launch_bounds__(NT)
gla_chunk_kernel(const typename TI::T* __restrict__ q, const typename TI::T* __restrict__ k,
                 const typename TI::T* __restrict__ v, const float* __restrict__ alpha,
                 const int32_t* __restrict__ cu, int n_seqs, int n_tokens, int H,
                 float* __restrict__ pool, int n_slots, const int32_t* __restrict__ slot_idx,
                 int zero_init, typename TO::T* __restrict__ o) {
    constexpr bool F32 = (TI::bytes == 4);
    using O = Op<F32>;
    using E = typename O::E;
    using Buf = GlaBuf<DK, BV, C, F32>;
    using PF = Prefetch<TI, C, DK, BV>;
    constexpr int NBUF = F32 ? 1 : 2;
    constexpr int LQ = Buf::LQ, LV = Buf::LV;
    constexpr int LO = F32 ? 0 : 1;
    constexpr int NVT = DV / BV;
    constexpr int CT = C / 16;                   // 16-row tiles per chunk
    constexpr int BT = BV / 16;                  // 16-col tiles per d_v tile
    constexpr int ST = (DK / 16) * BT;           // state tiles
    constexpr int SPW = (ST + NW - 1) / NW;      // state tiles per wave
    constexpr int VE = PF::VE;
    static_assert(DV % BV == 0 && BV % 16 == 0 && C % 16 == 0 && C <= 64 && CT <= NW, "tiling");

    __shared__ Buf buf[NBUF];

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
    const AccPos ap;
    const int col0 = vt * BV;
    const long tstride = static_cast<long>(H) * DK;
    const long vstride = static_cast<long>(H) * DV;

    // ---- initial state slice -> accumulators
    float* Sg = pool + (static_cast<long>(slot) * H + h) * DK * DV;
    f32x4 S[SPW];
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int t = wave + NW * i;
        const int mt = t / BT, nt = t % BT;
        S[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (t < ST && !zero_init) {
#pragma unroll
            for (int r = 0; r < 4; ++r) S[i][r] = Sg[(mt * 16 + ap.row0 + r) * DV + col0 + nt * 16 + ap.col];
        }
    }

    PF pf;
    auto fetch = [&](int c) {
        const long tok0 = s0 + static_cast<long>(c) * C;
        pf.load(q + tok0 * tstride + h * DK, k + tok0 * tstride + h * DK, v + tok0 * vstride + h * DV + col0,
                alpha + tok0 * H + h, tstride, vstride, H, min(C, L - c * C));
    };
    // Write the prefetched chunk and the current state slice into buffer bb.
    auto stage = [&](Buf& bb) {
        // in-wave scan of log alpha (every wave keeps its own copy)
        float x = __logf(pf.a);
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        const float glast = __shfl(x, C - 1, 64);
        if (wave == 0 && lane < C) {
            bb.g[lane] = x;
            bb.eg[lane] = __expf(x);
        }
        if (tid == 0) bb.gamma = __expf(glast);
#pragma unroll
        for (int u = 0; u < PF::NQ; ++u) {
            const int xx = tid + u * NT;
            if (xx < C * DK / VE) {
                const int row = xx / (DK / VE), vc = xx % (DK / VE);
                *reinterpret_cast<u32x4*>(&bb.q[row][vc * VE]) = pf.q[u];
                *reinterpret_cast<u32x4*>(&bb.k[row][vc * VE]) = pf.k[u];
            }
        }
#pragma unroll
        for (int u = 0; u < PF::NV; ++u) {
            const int xx = tid + u * NT;
            const int row = xx / (BV / VE), vc = xx % (BV / VE);
            const float dec = __expf(glast - __shfl(x, row & 63, 64));
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
        // state slice as the B operand of Q S: st[n][d]
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int t = wave + NW * i;
            if (t < ST) {
                const int mt = t / BT, nt = t % BT;
                const int ln = nt * 16 + ap.col;
                O::store4(&bb.st[0][ln][mt * 16 + ap.row0], &bb.st[LO][ln][mt * 16 + ap.row0], S[i]);
            }
        }
    };

    if (nchunks > 0) {
        fetch(0);
        stage(buf[0]);
        if (nchunks > 1) fetch(1);
    }
    lds_barrier();

    for (int c = 0; c < nchunks; ++c) {
        Buf& bb = buf[c % NBUF];
        const int n = min(C, L - c * C);
        const long tok0 = s0 + static_cast<long>(c) * C;
        const float gam = bb.gamma;

        f32x4 ov[BT];                             // this wave's output tiles, stored after staging
        if (wave < CT) {
            const int it = wave;                  // this wave's 16 rows of the chunk
            const int i = it * 16 + ap.col;       // row index held by this lane in P^T tiles
            // ---- P^T tiles (rows j, cols i), masked and decayed
            f32x4 pt[CT];
#pragma unroll
            for (int jt = 0; jt < CT; ++jt) {
                pt[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (jt <= it) {
                    O::mma(pt[jt], &bb.k[jt * 16][0], LQ, &bb.q[it * 16][0], LQ, DK);
                    const float gi = bb.g[i];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = jt * 16 + ap.row0 + r;
                        pt[jt][r] = (j <= i) ? pt[jt][r] * __expf(gi - bb.g[j]) : 0.f;
                    }
                }
            }
            // ---- O tiles of this wave's rows
#pragma unroll
            for (int nt = 0; nt < BT; ++nt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                mma_xs<F32>(acc, &bb.q[it * 16][0], LQ, &bb.st[0][nt * 16][0], &bb.st[LO][nt * 16][0], LQ, DK);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] *= bb.eg[it * 16 + ap.row0 + r];
                if constexpr (F32) {
#pragma unroll
                    for (int jt = 0; jt < CT; ++jt) {
                        if (jt <= it) {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                acc = mfma_f32(pt[jt][r], bb.v[jt * 16 + ap.row0 + r][nt * 16 + ap.col], acc);
                        }
                    }
                } else if constexpr (CT == 1) {
                    s16x4 hi, lo;
                    split4(pt[0], hi, lo);
                    const s16x4 bv = frag_km4(&bb.v[0][0], LV, nt * 16, 0);
                    acc = mfma_bf16_k16(hi, bv, acc);
                    acc = mfma_bf16_k16(lo, bv, acc);
                } else {
#pragma unroll
                    for (int s = 0; s < CT / 2; ++s) {
                        if (2 * s <= it) {
                            s16x4 h0, l0, h1, l1;
                            split4(pt[2 * s], h0, l0);
                            split4(pt[2 * s + 1], h1, l1);
                            const bf16x8 bv = frag_km_split(&bb.v[0][0], LV, nt * 16, 32 * s);
                            acc = mfma_bf16(cat8(h0, h1), bv, acc);
                            acc = mfma_bf16(cat8(l0, l1), bv, acc);
                        }
                    }
                }
                ov[nt] = acc;
            }
        }
        // ---- state hand-off for this wave's state tiles
#pragma unroll
        for (int si = 0; si < SPW; ++si) {
            const int t = wave + NW * si;
            if (t < ST) {
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
                        const bf16x8 a = frag_km(&bb.k[0][0], LQ, mt * 16, k0);
                        S[si] = mfma_bf16(a, frag_km(&bb.vd[0][0][0], LV, nt * 16, k0), S[si]);
                        S[si] = mfma_bf16(a, frag_km(&bb.vd[LO][0][0], LV, nt * 16, k0), S[si]);
                    }
                }
            }
        }

        if (c + 1 < nchunks) {
            if constexpr (NBUF == 1) lds_barrier();   // everyone done with the single buffer
            stage(buf[(c + 1) % NBUF]);
            if (c + 2 < nchunks) fetch(c + 2);
        }
        // Outputs go out after the prefetch is issued: loads and stores share
        // one counter, so stores issued earlier would make the staging of the
        // next chunk wait for them.
        if (wave < CT) {
#pragma unroll
            for (int nt = 0; nt < BT; ++nt) {
                const int colg = col0 + nt * 16 + ap.col;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = wave * 16 + ap.row0 + r;
                    if (row < n) TO::store(o, (tok0 + row) * vstride + h * DV + colg, ov[nt][r]);
                }
            }
        }
        lds_barrier();
    }

    // ---- final state slice -> pool (zeros for an empty sequence with zero-init)
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int t = wave + NW * i;
        if (t < ST) {
            const int mt = t / BT, nt = t % BT;
#pragma unroll
            for (int r = 0; r < 4; ++r) Sg[(mt * 16 + ap.row0 + r) * DV + col0 + nt * 16 + ap.col] = S[i][r];
        }
    }
}

template <int DK, int DV, int BV, int C, class TI, class TO>
hipError_t launch_inst(const ChunkArgs& a, hipStream_t s) {
    using T = typename TI::T;
    const long blocks = static_cast<long>(a.n_seqs) * a.n_heads * (DV / BV);
    hipLaunchKernelGGL((gla_chunk_kernel<DK, DV, BV, C, TI, TO>), dim3(static_cast<unsigned>(blocks)),
                       dim3(NT), 0, s, static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), a.alpha, a.cu_seqlens, a.n_seqs, a.n_tokens,
                       a.n_heads, a.pool, a.n_slots, a.slot_idx, a.zero_init,
                       static_cast<typename TO::T*>(a.o));
    return hipGetLastError();
}

template <int DK, int DV, int C, class TI, class TO>
hipError_t launch_bv(const ChunkArgs& a, hipStream_t s) {
    constexpr int BV = DV >= 32 ? 32 : DV;
    return launch_inst<DK, DV, BV, C, TI, TO>(a, s);
}

template <int DK, int DV, class TI, class TO>
hipError_t launch_c(const ChunkArgs& a, hipStream_t s) {
    switch (a.chunk) {
        case 16: return launch_bv<DK, DV, 16, TI, TO>(a, s);
        case 32: return launch_bv<DK, DV, 32, TI, TO>(a, s);
        case 64: return launch_bv<DK, DV, 64, TI, TO>(a, s);
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

hipError_t launch_gla_chunk(const ChunkArgs& a, hipStream_t s) {
    switch (a.dk) {
        case 16: return launch_dv<16>(a, s);
        case 32: return launch_dv<32>(a, s);
        case 64: return launch_dv<64>(a, s);
        case 128: return launch_dv<128>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gla
