// Chunked GLA prefill, segmented, for bf16 inputs with d_k = d_v = 128 and
// 64-token chunks.
//
// "Inference for linear attention and hybrid architectures", section "Two
// ways to write the same computation": the chunked form hands only the state
// from chunk to chunk, and a prompt cut into segments is processed the same
// way by handing the state from segment to segment.  Here that hand-off is
// used inside one call to get parallelism along the sequence: every
// sequence is cut into segments of whole chunks, and
//
//   pass 1 (gla_seg_state): for each segment but the last, its local state
//     contribution dS_g = sum over its tokens of exp(G_end - G_t) k_t^T v_t
//     (the state it would produce from S = 0) and its total log-decay
//     Lambda_g; the last segment's slot receives a copy of the initial state;
//   pass 2 (gla_seg_out): each segment folds its entry state
//     S_in(g) = 2^Lambda_{g-1} S_in(g-1) + dS_{g-1} from those, then runs the
//     chunked form over its chunks; the last segment writes the final state
//     back to the pool.
//
// Within a workgroup (8 waves) each wave owns 16 columns of the 128x128
// fp32 state (held in MFMA accumulators).  Q S, P V and the state update are
// then column-local; only P = (Q K^T) .* D is shared, computed once per
// chunk by all waves and passed through LDS.  Per chunk:
//   phase 1: P tiles (split over the waves) -> LDS; this wave's columns of
//            Q S (state operand straight from its accumulators);
//   phase 2: + P V; outputs; S <- exp(g_last) S + K^T (diag(dec) V); stage
//            the next chunk (prefetched into registers) into the other LDS
//            buffer and prefetch the one after.
// q, k, v stay token-major in LDS; contractions over tokens use the LDS
// transpose read.  Global accesses go through buffer resources sized to the
// valid rows, so the loop has no guarded memory instructions.
#include "chunk_common.h"
#include "launch.h"

namespace gla {
namespace {

constexpr int SW = 8;              // waves
constexpr int ST = SW * 64;        // threads
constexpr int SD = 128;            // d_k = d_v
constexpr int SC = 64;             // chunk
constexpr int SL = SD + 8;         // LDS line of a q/k/v row (16-byte pad)
constexpr int SP = SC + 8;         // LDS line of a P row

struct SegBuf {
    alignas(16) uint16_t q[SC][SL];
    alignas(16) uint16_t k[SC][SL];
    alignas(16) uint16_t v[SC][SL];
    alignas(16) float g2[SC];      // running log2 decay
    alignas(16) float eg[SC];      // 2^g2
    alignas(16) float dec[SC];     // 2^(g2_last - g2)
    float gamma;                   // 2^g2_last
};

struct SegPrefetch {
    static constexpr int NV = SC * SD / 8 / ST;    // 16-byte vectors per thread per tensor
    u32x4 q[NV], k[NV], v[NV];
    float a;
};

struct SegGeom {
    int b, g, nseg, h, slot;
    int t0, t1;        // token range of this segment
    long ws_slot;      // this segment's state slot in the workspace
    long ws_first;     // slot of the sequence's first segment
};

// Which (sequence, segment, head) this block works on; false if none.
__device__ __forceinline__ bool seg_geometry(SegGeom& sg, const int32_t* cu, int n_seqs, int n_tokens,
                                             int H, int lseg, const int32_t* soff, const int32_t* slot_idx,
                                             int n_slots) {
    const int h = blockIdx.x % H;
    const int si = blockIdx.x / H;
    const int maxseg = gridDim.x / H;
    if (si >= soff[n_seqs]) return false;
    const int b = find_span_owner(soff, n_seqs, si);
    const int g = si - soff[b];
    const int nseg = soff[b + 1] - soff[b];
    if (g < 0 || g >= nseg) return false;
    // cu_seqlens that are not non-decreasing can claim more segments than
    // the workspace holds; such sequences are skipped rather than overrun it
    if (soff[b + 1] > maxseg) return false;
    const int slot = slot_idx[b];
    if (slot < 0 || slot >= n_slots) return false;
    const int s0 = clampi(cu[b], 0, n_tokens);
    const int s1 = clampi(cu[b + 1], s0, n_tokens);
    sg.b = b;
    sg.g = g;
    sg.nseg = nseg;
    sg.h = h;
    sg.slot = slot;
    sg.t0 = min(s0 + g * lseg, s1);
    sg.t1 = min(sg.t0 + lseg, s1);
    sg.ws_first = static_cast<long>(soff[b]) * H + h;
    sg.ws_slot = static_cast<long>(si) * H + h;
    return true;
}

// One chunk's global slices (rows past n read as zero) into registers.
__device__ __forceinline__ void seg_fetch(SegPrefetch& pf, const uint16_t* q, const uint16_t* k,
                                          const uint16_t* v, const float* alpha, long tok0, int n, int h,
                                          int H, bool with_q) {
    const long stride = static_cast<long>(H) * SD;
    const uint32_t ext = rows_extent(n, stride * 2, SD * 2);
    const BufRsrc rq(q + tok0 * stride + h * SD, with_q ? ext : 0u);
    const BufRsrc rk(k + tok0 * stride + h * SD, ext);
    const BufRsrc rv(v + tok0 * stride + h * SD, ext);
    const BufRsrc ra(alpha + tok0 * H + h, rows_extent(n, static_cast<long>(H) * 4, 4));
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < SegPrefetch::NV; ++u) {
        const int x = tid + u * ST;
        const uint32_t offb = static_cast<uint32_t>(((x / (SD / 8)) * stride + (x % (SD / 8)) * 8) * 2);
        if (with_q) pf.q[u] = rq.load16(offb);
        pf.k[u] = rk.load16(offb);
        pf.v[u] = rv.load16(offb);
    }
    const int lane = tid & 63;
    const float a = ra.loadf(static_cast<uint32_t>(lane * H * 4));
    pf.a = (lane < n && lane < SC) ? a : 1.f;
}

// Registers -> LDS buffer; every wave scans log2(alpha) itself and returns
// the chunk's total log2 decay.
__device__ __forceinline__ float seg_stage(SegBuf& bb, const SegPrefetch& pf, bool with_q) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    float x = __log2f(pf.a);
#pragma unroll
    for (int offs = 1; offs < 64; offs <<= 1) {
        const float y = __shfl_up(x, offs, 64);
        if (lane >= offs) x += y;
    }
    const float glast = __shfl(x, SC - 1, 64);
    if ((tid >> 6) == 0) {
        bb.g2[lane] = x;
        bb.eg[lane] = exp2f(x);
        bb.dec[lane] = exp2f(glast - x);
    }
    if (tid == 0) bb.gamma = exp2f(glast);
#pragma unroll
    for (int u = 0; u < SegPrefetch::NV; ++u) {
        const int xx = tid + u * ST;
        const int row = xx / (SD / 8), vc = (xx % (SD / 8)) * 8;
        if (with_q) *reinterpret_cast<u32x4*>(&bb.q[row][vc]) = pf.q[u];
        *reinterpret_cast<u32x4*>(&bb.k[row][vc]) = pf.k[u];
        *reinterpret_cast<u32x4*>(&bb.v[row][vc]) = pf.v[u];
    }
    return glast;
}

// S (this wave's 16 columns, all 8 row tiles) <- gamma S + K^T diag(dec) V.
__device__ __forceinline__ void seg_state_update(f32x4 (&S)[8], const SegBuf& bb, int col) {
    const int lane = threadIdx.x & 63;
    const float gam = bb.gamma;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) S[mt] *= gam;
#pragma unroll
    for (int ks = 0; ks < SC / 32; ++ks) {
        // decayed values for tokens {32ks + 4g + e} u {32ks + 16 + 4g + e}
        const bf16x8 vf = frag_km_split(&bb.v[0][0], SL, col, 32 * ks);
        const u32x4 vw = __builtin_bit_cast(u32x4, vf);
        const int g = lane >> 4;
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(&bb.dec[32 * ks + 4 * g]);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(&bb.dec[32 * ks + 16 + 4 * g]);
        uint32_t hw[4], lw[4];
        split_bf16x2(__uint_as_float(vw.x << 16) * d0.x, __uint_as_float(vw.x & 0xffff0000u) * d0.y, hw[0], lw[0]);
        split_bf16x2(__uint_as_float(vw.y << 16) * d0.z, __uint_as_float(vw.y & 0xffff0000u) * d0.w, hw[1], lw[1]);
        split_bf16x2(__uint_as_float(vw.z << 16) * d1.x, __uint_as_float(vw.z & 0xffff0000u) * d1.y, hw[2], lw[2]);
        split_bf16x2(__uint_as_float(vw.w << 16) * d1.z, __uint_as_float(vw.w & 0xffff0000u) * d1.w, hw[3], lw[3]);
        const bf16x8 vh = as_bf16x8(u32x4{hw[0], hw[1], hw[2], hw[3]});
        const bf16x8 vl = as_bf16x8(u32x4{lw[0], lw[1], lw[2], lw[3]});
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const bf16x8 kf = frag_km_split(&bb.k[0][0], SL, mt * 16, 32 * ks);
            S[mt] = mfma_bf16(kf, vh, S[mt]);
            S[mt] = mfma_bf16(kf, vl, S[mt]);
        }
    }
}

// ------------------------------------------------------------------ pass 1
__global__ void __launch_bounds__(ST)
gla_seg_state(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
              const float* __restrict__ alpha, const int32_t* __restrict__ cu, int n_seqs,
              int n_tokens, int H, const float* __restrict__ pool, int n_slots,
              const int32_t* __restrict__ slot_idx, int zero_init, int lseg,
              const int32_t* __restrict__ soff, float* __restrict__ wstate, float* __restrict__ wlam) {
    SegGeom sg;
    if (!seg_geometry(sg, cu, n_seqs, n_tokens, H, lseg, soff, slot_idx, n_slots)) return;
    if (sg.nseg <= 1) return;                      // no split: pass 2 reads the pool itself
    const int wave = threadIdx.x >> 6;
    const AccPos ap;
    const int col = wave * 16;
    float* dst = wstate + sg.ws_slot * SD * SD;
    if (sg.g == sg.nseg - 1) {                     // last segment's slot: copy of the initial state
        const float* src = pool + (static_cast<long>(sg.slot) * H + sg.h) * SD * SD;
        for (int i = threadIdx.x; i < SD * SD / 4; i += ST) {
            const f32x4 x = zero_init ? f32x4{0.f, 0.f, 0.f, 0.f} : reinterpret_cast<const f32x4*>(src)[i];
            reinterpret_cast<f32x4*>(dst)[i] = x;
        }
        return;
    }

    __shared__ SegBuf buf[2];
    f32x4 S[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) S[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nch = (sg.t1 - sg.t0 + SC - 1) / SC;
    auto rows = [&](int c) { return c < nch ? min(SC, sg.t1 - sg.t0 - c * SC) : 0; };
    auto tok = [&](int c) { return static_cast<long>(sg.t0) + static_cast<long>(c < nch ? c : 0) * SC; };
    SegPrefetch pf;
    float lam = 0.f;
    seg_fetch(pf, nullptr, k, v, alpha, tok(0), rows(0), sg.h, H, false);
    lam += seg_stage(buf[0], pf, false);
    seg_fetch(pf, nullptr, k, v, alpha, tok(1), rows(1), sg.h, H, false);
    lds_barrier();
    for (int c = 0; c < nch; ++c) {
        seg_state_update(S, buf[c & 1], col);
        const float gl = seg_stage(buf[(c + 1) & 1], pf, false);
        if (c + 1 < nch) lam += gl;
        seg_fetch(pf, nullptr, k, v, alpha, tok(c + 2), rows(c + 2), sg.h, H, false);
        lds_barrier();
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(mt * 16 + ap.row0 + r) * SD + col + ap.col] = S[mt][r];
    }
    if (threadIdx.x == 0) wlam[sg.ws_slot] = lam;
}

// ------------------------------------------------------------------ pass 2
template <class TO>
__global__ void __launch_bounds__(ST)
gla_seg_out(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
            const float* __restrict__ alpha, const int32_t* __restrict__ cu, int n_seqs, int n_tokens,
            int H, float* __restrict__ pool, int n_slots, const int32_t* __restrict__ slot_idx,
            int zero_init, int lseg, const int32_t* __restrict__ soff, const float* __restrict__ wstate,
            const float* __restrict__ wlam, typename TO::T* __restrict__ o) {
    SegGeom sg;
    if (!seg_geometry(sg, cu, n_seqs, n_tokens, H, lseg, soff, slot_idx, n_slots)) return;
    __shared__ SegBuf buf[2];
    __shared__ uint16_t pbuf[2][SC][SP];           // P = (Q K^T) .* D, hi and lo planes

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const AccPos ap;
    const int col = wave * 16;
    const long stride = static_cast<long>(H) * SD;

    // ---- entry state of this segment
    f32x4 S[8];
    float* Sg = pool + (static_cast<long>(sg.slot) * H + sg.h) * SD * SD;
    auto load_tile = [&](const float* base, int mt) {
        f32x4 x;
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = base[(mt * 16 + ap.row0 + r) * SD + col + ap.col];
        return x;
    };
    if (sg.nseg <= 1) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) S[mt] = zero_init ? f32x4{0.f, 0.f, 0.f, 0.f} : load_tile(Sg, mt);
    } else {
        const float* s0 = wstate + (sg.ws_first + static_cast<long>(sg.nseg - 1) * H) * SD * SD;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) S[mt] = load_tile(s0, mt);
        for (int j = 0; j < sg.g; ++j) {
            const long sj = sg.ws_first + static_cast<long>(j) * H;
            const float dcy = exp2f(wlam[sj]);
            const float* dS = wstate + sj * SD * SD;
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) S[mt] = dcy * S[mt] + load_tile(dS, mt);
        }
    }

    const int nch = (sg.t1 - sg.t0 + SC - 1) / SC;
    auto rows = [&](int c) { return c < nch ? min(SC, sg.t1 - sg.t0 - c * SC) : 0; };
    auto tok = [&](int c) { return static_cast<long>(sg.t0) + static_cast<long>(c < nch ? c : 0) * SC; };
    // P tiles above the diagonal that P V still reads (rows 0-15 x cols 16-31,
    // rows 32-47 x cols 48-63) stay zero; the others are rewritten each chunk.
    for (int idx = tid; idx < 2 * 256; idx += ST) {
        const int t = idx >> 8, e = idx & 255;
        const int row = (t ? 32 : 0) + (e >> 4), cx = (t ? 48 : 16) + (e & 15);
        pbuf[0][row][cx] = 0;
        pbuf[1][row][cx] = 0;
    }
    SegPrefetch pf;
    seg_fetch(pf, q, k, v, alpha, tok(0), rows(0), sg.h, H, true);
    seg_stage(buf[0], pf, true);
    seg_fetch(pf, q, k, v, alpha, tok(1), rows(1), sg.h, H, true);
    lds_barrier();

    for (int c = 0; c < nch; ++c) {
        SegBuf& bb = buf[c & 1];
        const int n = rows(c);
        const long tok0 = tok(c);

        // ---- phase 1: P tiles (lower triangle, split over the waves) -> LDS
        for (int t = wave; t < 10; t += SW) {
            // tile t of (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) (3,1) (3,2) (3,3)
            const int it = t < 1 ? 0 : (t < 3 ? 1 : (t < 6 ? 2 : 3));
            const int jt = t - it * (it + 1) / 2;
            f32x4 pt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < SD / 32; ++ks)
                pt = mfma_bf16(frag_kc(&bb.k[0][0], SL, jt * 16, 32 * ks), frag_kc(&bb.q[0][0], SL, it * 16, 32 * ks), pt);
            const int i = it * 16 + ap.col;
            const float gi = bb.g2[i];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = jt * 16 + ap.row0 + r;
                pt[r] = (j <= i) ? pt[r] * exp2f(gi - bb.g2[j]) : 0.f;
            }
            Op<false>::store4(&pbuf[0][i][jt * 16 + ap.row0], &pbuf[1][i][jt * 16 + ap.row0], pt);
        }
        // ---- this wave's columns of Q S, the state operand from its accumulators
        f32x4 oacc[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) oacc[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < SD / 32; ++s) {
            s16x4 h0, l0, h1, l1;
            split4(S[2 * s], h0, l0);
            split4(S[2 * s + 1], h1, l1);
            const bf16x8 sh = cat8(h0, h1), sl = cat8(l0, l1);
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const bf16x8 qf = frag_kc_split(&bb.q[0][0], SL, it * 16, 32 * s);
                oacc[it] = mfma_bf16(qf, sh, oacc[it]);
                oacc[it] = mfma_bf16(qf, sl, oacc[it]);
            }
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const f32x4 e = *reinterpret_cast<const f32x4*>(&bb.eg[it * 16 + ap.row0]);
            oacc[it] *= e;
        }
        lds_barrier();

        // ---- phase 2: + P V, outputs, state update, next chunk
#pragma unroll
        for (int it = 0; it < 4; ++it) {
#pragma unroll
            for (int s = 0; s < SC / 32; ++s) {
                if (32 * s <= it * 16 + 15) {
                    const bf16x8 vf = frag_km(&bb.v[0][0], SL, col, 32 * s);
                    oacc[it] = mfma_bf16(frag_kc(&pbuf[0][0][0], SP, it * 16, 32 * s), vf, oacc[it]);
                    oacc[it] = mfma_bf16(frag_kc(&pbuf[1][0][0], SP, it * 16, 32 * s), vf, oacc[it]);
                }
            }
        }
        {
            const BufRsrc ro(o + tok0 * stride + sg.h * SD, rows_extent(n, stride * TO::bytes, SD * TO::bytes));
#pragma unroll
            for (int it = 0; it < 4; ++it) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t offb =
                        static_cast<uint32_t>(((it * 16 + ap.row0 + r) * stride + col + ap.col) * TO::bytes);
                    if constexpr (TO::bytes == 2) ro.store_b16(f32_to_bf16_bits(oacc[it][r]), offb);
                    else ro.store_b32(__float_as_uint(oacc[it][r]), offb);
                }
            }
        }
        seg_state_update(S, bb, col);
        seg_stage(buf[(c + 1) & 1], pf, true);
        seg_fetch(pf, q, k, v, alpha, tok(c + 2), rows(c + 2), sg.h, H, true);
        lds_barrier();
    }

    if (sg.g == sg.nseg - 1) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) Sg[(mt * 16 + ap.row0 + r) * SD + col + ap.col] = S[mt][r];
        }
    }
    (void)lane;
}

// Every sequence gets at least one segment (an empty one still writes its
// state back).  Segment length: whole chunks, at least 4 of them, about 256 workgroups in
// total (one per compute unit; LDS allows one workgroup per CU).
int seg_len(int n_tokens, int n_heads) {
    const long target = n_heads >= 256 ? 1 : 256 / n_heads;
    long L = (n_tokens + target - 1) / target;
    L = ((L + SC - 1) / SC) * SC;
    return static_cast<int>(L < 4 * SC ? 4 * SC : L);
}

__host__ __device__ constexpr size_t align256s(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

bool gla_seg_supported(const ChunkArgs& a) {
    return a.in_bf16 && a.dk == SD && a.dv == SD && a.chunk == SC;
}

size_t gla_seg_workspace(int n_seqs, int n_tokens, int n_heads) {
    const long lseg = seg_len(n_tokens, n_heads);
    const long maxseg = n_tokens / lseg + n_seqs;
    return align256s(sizeof(int32_t) * (n_seqs + 1)) + align256s(sizeof(float) * maxseg * n_heads) +
           static_cast<size_t>(maxseg) * n_heads * SD * SD * sizeof(float);
}

hipError_t launch_gla_seg(const ChunkArgs& a, hipStream_t s) {
    const int lseg = seg_len(a.n_tokens, a.n_heads);
    const long maxseg = a.n_tokens / lseg + a.n_seqs;
    char* ws = static_cast<char*>(a.workspace);
    int32_t* soff = reinterpret_cast<int32_t*>(ws);
    ws += align256s(sizeof(int32_t) * (a.n_seqs + 1));
    float* wlam = reinterpret_cast<float*>(ws);
    ws += align256s(sizeof(float) * maxseg * a.n_heads);
    float* wstate = reinterpret_cast<float*>(ws);
    hipLaunchKernelGGL(span_offsets, dim3(1), dim3(1024), 0, s, a.cu_seqlens, a.n_seqs, a.n_tokens, lseg, 1, soff);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid(static_cast<unsigned>(maxseg * a.n_heads));
    hipLaunchKernelGGL(gla_seg_state, grid, dim3(ST), 0, s, static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), a.alpha, a.cu_seqlens, a.n_seqs, a.n_tokens,
                       a.n_heads, a.pool, a.n_slots, a.slot_idx, a.zero_init, lseg, soff, wstate, wlam);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.out_bf16) {
        hipLaunchKernelGGL((gla_seg_out<BF16>), grid, dim3(ST), 0, s, static_cast<const uint16_t*>(a.q),
                           static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v), a.alpha,
                           a.cu_seqlens, a.n_seqs, a.n_tokens, a.n_heads, a.pool, a.n_slots, a.slot_idx,
                           a.zero_init, lseg, soff, wstate, wlam, static_cast<uint16_t*>(a.o));
    } else {
        hipLaunchKernelGGL((gla_seg_out<F32>), grid, dim3(ST), 0, s, static_cast<const uint16_t*>(a.q),
                           static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v), a.alpha,
                           a.cu_seqlens, a.n_seqs, a.n_tokens, a.n_heads, a.pool, a.n_slots, a.slot_idx,
                           a.zero_init, lseg, soff, wstate, wlam, static_cast<float*>(a.o));
    }
    return hipGetLastError();
}

}  // namespace gla
