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
// so tiling d_v is exact and multiplies the number of independent chains;
// the d_v tiles of one (sequence, head) re-read the same q/k chunk, which
// the XCD-aware block order keeps in one L2.  The BV-column slice of the
// fp32 state stays in MFMA accumulators for the whole sequence.
//
// Per chunk: stage q, k (natural and transposed) and the v tile
// (transposed) in LDS; wave 0 scans log alpha; the state slice is written to
// LDS as a hi/lo bf16 B operand; then
//   P^T = K Q^T (lower tiles only, masked and decayed)    -> P  (hi/lo)
//   O   = diag(exp g) (Q S) + P V                          -> o  (global)
//   S   = exp(g_last) S + K^T (diag(exp(g_last - g)) V)    (accumulators)
// All four contractions run on MFMA with fp32 accumulation.
#include "chunk_common.h"
#include "launch.h"

namespace gla {
namespace {

constexpr int NW = 4;
constexpr int NT = NW * 64;

template <int DK, int BV, int C, bool F32>
struct GlaSmem {
    using E = typename Op<F32>::E;
    static constexpr int PAD = Op<F32>::PAD;
    static constexpr int LQ = DK + PAD;   // lines of length DK (k = d)
    static constexpr int LT = C + PAD;    // lines of length C  (k = token)
    static constexpr int NLO = F32 ? 1 : 0;   // lo arrays collapse to 1 line in fp32 mode
    alignas(16) E q[C][LQ];
    alignas(16) E k[C][LQ];
    alignas(16) E kt[DK][LT];
    alignas(16) E vt[BV][LT];
    alignas(16) E vd_hi[BV][LT];
    alignas(16) E vd_lo[NLO ? 1 : BV][LT];
    alignas(16) E p_hi[C][LT];
    alignas(16) E p_lo[NLO ? 1 : C][LT];
    alignas(16) E st_hi[BV][LQ];
    alignas(16) E st_lo[NLO ? 1 : BV][LQ];
    float g[C];
    float eg[C];
    float dec[C];
    float gamma;
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
    using Sm = GlaSmem<DK, BV, C, F32>;
    constexpr int LQ = Sm::LQ, LT = Sm::LT;
    constexpr int NVT = DV / BV;
    constexpr int CT = C / 16;                   // 16-row tiles per chunk
    constexpr int BT = BV / 16;                  // 16-col tiles per d_v tile
    constexpr int ST = (DK / 16) * BT;           // state tiles
    constexpr int SPW = (ST + NW - 1) / NW;      // state tiles per wave
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

    const int wave = threadIdx.x >> 6;
    const AccPos ap;
    const int col0 = vt * BV;

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
            for (int r = 0; r < 4; ++r)
                S[i][r] = Sg[(mt * 16 + ap.row0 + r) * DV + col0 + nt * 16 + ap.col];
        }
    }

    const long tstride = static_cast<long>(H) * DK;     // q/k token stride
    const long vstride = static_cast<long>(H) * DV;
    for (int c0 = 0; c0 < L; c0 += C) {
        const int n = min(C, L - c0);
        const long tok0 = s0 + c0;
        __syncthreads();   // previous chunk finished with LDS

        stage_natural<TI, C, DK, NT>(&sm.q[0][0], LQ, q + tok0 * tstride + h * DK, tstride, n);
        stage_transposed<TI, C, DK, NT>(&sm.kt[0][0], LT, &sm.k[0][0], LQ,
                                        k + tok0 * tstride + h * DK, tstride, n);
        stage_transposed<TI, C, BV, NT>(&sm.vt[0][0], LT, nullptr, 0,
                                        v + tok0 * vstride + h * DV + col0, vstride, n);
        decay_scan<C>(alpha + tok0 * H + h, H, n, sm.g, sm.eg, sm.dec, &sm.gamma);
        // state slice as the B operand of Q S: st[n][d] (hi/lo)
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int t = wave + NW * i;
            if (t < ST) {
                const int mt = t / BT, nt = t % BT;
                const int ln = nt * 16 + ap.col;
                O::store4(&sm.st_hi[ln][mt * 16 + ap.row0], &sm.st_lo[F32 ? 0 : ln][mt * 16 + ap.row0], S[i]);
            }
        }
        __syncthreads();

        // ---- P = (Q K^T) .* D, computed as P^T tiles (rows j, cols i) so that
        //      each lane writes 4 consecutive j of row i of P.
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
            O::store4(&sm.p_hi[i][jt * 16 + ap.row0], &sm.p_lo[F32 ? 0 : i][jt * 16 + ap.row0], acc);
        }
        // ---- decayed values for the state update: vd[n][j] = dec[j] v[j][n]
        for (int idx = threadIdx.x; idx < BV * C; idx += NT) {
            const int ln = idx / C, j = idx % C;
            const float x = O::load1(&sm.vt[ln][j]) * sm.dec[j];
            O::store1(&sm.vd_hi[ln][j], &sm.vd_lo[F32 ? 0 : ln][j], x);
        }
        __syncthreads();

        // ---- outputs of this chunk
        for (int t = wave; t < CT * BT; t += NW) {
            const int it = t / BT, nt = t % BT;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mma_xs<F32>(acc, &sm.q[it * 16][0], LQ, &sm.st_hi[nt * 16][0],
                        &sm.st_lo[F32 ? 0 : nt * 16][0], LQ, DK);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] *= sm.eg[it * 16 + ap.row0 + r];
            mma_sx<F32>(acc, &sm.p_hi[it * 16][0], &sm.p_lo[F32 ? 0 : it * 16][0], LT,
                        &sm.vt[nt * 16][0], LT, C);
            const int colg = col0 + nt * 16 + ap.col;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = it * 16 + ap.row0 + r;
                if (row < n) TO::store(o, (tok0 + row) * vstride + h * DV + colg, acc[r]);
            }
        }
        // ---- state hand-off
        const float gam = sm.gamma;
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int t = wave + NW * i;
            if (t < ST) {
                const int mt = t / BT, nt = t % BT;
                S[i] *= gam;
                mma_xs<F32>(S[i], &sm.kt[mt * 16][0], LT, &sm.vd_hi[nt * 16][0],
                            &sm.vd_lo[F32 ? 0 : nt * 16][0], LT, C);
            }
        }
    }

    // ---- final state slice -> pool (zeros for an empty sequence with zero-init)
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
