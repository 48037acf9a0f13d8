// Recurrent (decode) step of GLA and Gated DeltaNet on a slot-indexed fp32
// state pool, in place.
//
// "Inference for linear attention and hybrid architectures", section "Two
// ways to write the same computation": decode reads the state once and
// applies one rank-one update, so each step costs the same whatever the
// context length.  Section "Speculative decoding and PD disaggregation":
// each request owns a fixed slot of the state pool and batched kernels read
// and write by slot index.
//
// The step is HBM-bound (about 0.5 flop per byte): each workgroup owns one
// (request, head), streams its d_k x d_v fp32 state from HBM exactly once
// into registers, updates it there and streams it back.  Threads own 4
// adjacent columns (one 16-byte vector) of RPT rows; the rows of a wave are
// contiguous in memory, so every load and store is a full, coalesced
// 16-byte-per-lane access.  The only cross-thread step is the reduction over
// d_k for the outputs (and, for Gated DeltaNet, for p = k S), done in LDS.
//
// Gated DeltaNet uses the identity (exact in real arithmetic)
//   o = q S_new = alpha (q S) + (q . k) u,   u = beta (v - alpha k S),
// so q S, k S and q . k come out of ONE reduction over the old state and the
// state is still touched once.
#include "common.h"
#include "launch.h"

namespace gla {
namespace {

template <int DK, int DV>
struct DecodeShape {
    static constexpr int NT_RAW = DK * DV / 64;
    static constexpr int NT = NT_RAW < 64 ? 64 : (NT_RAW > 256 ? 256 : NT_RAW);  // threads
    static constexpr int CG = DV / 4;          // 16-byte column groups per row
    static constexpr int RG = NT / CG;         // row groups
    static constexpr int RPT = DK / RG;        // rows per thread
    static_assert(RG * CG == NT && RPT * RG == DK && RPT >= 1, "decode tiling");
};

template <int DK, int DV, class TI, class TO, bool GDN>
__global__ void __launch_bounds__((DecodeShape<DK, DV>::NT))
decode_kernel(const typename TI::T* __restrict__ q, const typename TI::T* __restrict__ k,
              const typename TI::T* __restrict__ v, const float* __restrict__ alpha,
              const float* __restrict__ beta, float* __restrict__ pool, int n_heads,
              int n_slots, const int32_t* __restrict__ slot_idx, typename TO::T* __restrict__ o) {
    using Sh = DecodeShape<DK, DV>;
    constexpr int NT = Sh::NT, CG = Sh::CG, RG = Sh::RG, RPT = Sh::RPT;
    constexpr int NRED = GDN ? 2 : 1;          // reduced vectors: (q S) [, k S]

    const int h = blockIdx.x % n_heads;
    const int r = blockIdx.x / n_heads;
    const int t = threadIdx.x;
    const int cg = t % CG;
    const int rg = t / CG;

    const int slot = slot_idx[r];
    if (slot < 0 || slot >= n_slots) return;   // invalid slot: skip, never fault

    __shared__ float s_q[DK];
    __shared__ float s_k[DK];
    __shared__ f32x4 s_red[NRED][RG][CG];
    __shared__ float s_qk[RG];

    float* __restrict__ S = pool + (static_cast<long>(slot) * n_heads + h) * (DK * DV);

    // Issue the whole state tile first: RPT independent 16-byte loads/thread.
    f32x4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + RG * i;
        s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + row * DV + cg * 4));
    }

    const long tok = static_cast<long>(r) * n_heads + h;
    for (int i = t; i < DK; i += NT) {
        s_q[i] = TI::load(q, tok * DK + i);
        s_k[i] = TI::load(k, tok * DK + i);
    }
    const f32x4 v4 = Vec4<TI>::load(v + tok * DV + cg * 4);
    const float a = alpha[tok];
    __syncthreads();

    if constexpr (!GDN) {
        // S <- a S + k^T v ; partial (q S) over own rows
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int row = rg + RG * i;
            s[i] = a * s[i] + s_k[row] * v4;
            acc += s_q[row] * s[i];
            __builtin_nontemporal_store(s[i], reinterpret_cast<f32x4*>(S + row * DV + cg * 4));
        }
        s_red[0][rg][cg] = acc;
        __syncthreads();
        if (rg == 0) {
            f32x4 tot = s_red[0][0][cg];
#pragma unroll
            for (int j = 1; j < RG; ++j) tot += s_red[0][j][cg];
            Vec4<TO>::store(o + tok * DV + cg * 4, tot);
        }
    } else {
        const float b = beta[tok];
        f32x4 accq = {0.f, 0.f, 0.f, 0.f}, acck = {0.f, 0.f, 0.f, 0.f};
        float qk = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int row = rg + RG * i;
            accq += s_q[row] * s[i];
            acck += s_k[row] * s[i];
            qk += s_q[row] * s_k[row];
        }
        s_red[0][rg][cg] = accq;
        s_red[1][rg][cg] = acck;
        if (cg == 0) s_qk[rg] = qk;
        __syncthreads();
        f32x4 p = s_red[1][0][cg];
#pragma unroll
        for (int j = 1; j < RG; ++j) p += s_red[1][j][cg];
        const f32x4 u = b * (v4 - a * p);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int row = rg + RG * i;
            s[i] = a * s[i] + s_k[row] * u;
            __builtin_nontemporal_store(s[i], reinterpret_cast<f32x4*>(S + row * DV + cg * 4));
        }
        if (rg == 0) {
            f32x4 qs = s_red[0][0][cg];
            float qkt = s_qk[0];
#pragma unroll
            for (int j = 1; j < RG; ++j) {
                qs += s_red[0][j][cg];
                qkt += s_qk[j];
            }
            Vec4<TO>::store(o + tok * DV + cg * 4, a * qs + qkt * u);
        }
    }
}

// Several consecutive tokens per request (the draft tokens that one
// speculative-decoding verification step scores), with the state after
// every position kept.  Section "Speculative decoding and PD
// disaggregation": a rejected draft token must not leave its update in the
// request's state, so each position's state goes to a slot of its own
// (pos_slots[r * n_tok + j]; negative = not kept) and the request's own slot
// is only read.  The state is streamed in once, stays in registers across
// the n_tok steps and is streamed out once per kept position.
//
// q/k staging and the reduction buffers are double-buffered by token
// parity, so each token needs two barriers: one after its q/k land in LDS,
// one after the partial sums of the reduction are written.
template <int DK, int DV, class TI, class TO, bool GDN>
__global__ void __launch_bounds__((DecodeShape<DK, DV>::NT))
decode_multi_kernel(const typename TI::T* __restrict__ q, const typename TI::T* __restrict__ k,
                    const typename TI::T* __restrict__ v, const float* __restrict__ alpha,
                    const float* __restrict__ beta, float* __restrict__ pool, int n_heads,
                    int n_tok, int n_slots, const int32_t* __restrict__ slot_idx,
                    const int32_t* __restrict__ pos_slots, typename TO::T* __restrict__ o) {
    using Sh = DecodeShape<DK, DV>;
    constexpr int NT = Sh::NT, CG = Sh::CG, RG = Sh::RG, RPT = Sh::RPT;
    constexpr int NRED = GDN ? 2 : 1;

    const int h = blockIdx.x % n_heads;
    const int r = blockIdx.x / n_heads;
    const int t = threadIdx.x;
    const int cg = t % CG;
    const int rg = t / CG;

    const int slot = slot_idx[r];
    if (slot < 0 || slot >= n_slots) return;

    __shared__ float s_q[2][DK];
    __shared__ float s_k[2][DK];
    __shared__ f32x4 s_red[2][NRED][RG][CG];
    __shared__ float s_qk[2][RG];

    const long head_elems = static_cast<long>(DK) * DV;
    const float* __restrict__ S_in = pool + (static_cast<long>(slot) * n_heads + h) * head_elems;

    f32x4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + RG * i;
        s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S_in + row * DV + cg * 4));
    }

    for (int j = 0; j < n_tok; ++j) {
        const int par = j & 1;
        const long tok = (static_cast<long>(r) * n_tok + j) * n_heads + h;
        for (int i = t; i < DK; i += NT) {
            s_q[par][i] = TI::load(q, tok * DK + i);
            s_k[par][i] = TI::load(k, tok * DK + i);
        }
        const f32x4 v4 = Vec4<TI>::load(v + tok * DV + cg * 4);
        const float a = alpha[tok];
        const int ps = pos_slots[static_cast<long>(r) * n_tok + j];
        const bool keep = ps >= 0 && ps < n_slots;
        float* __restrict__ S_out = pool + (static_cast<long>(keep ? ps : 0) * n_heads + h) * head_elems;
        __syncthreads();

        if constexpr (!GDN) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int row = rg + RG * i;
                s[i] = a * s[i] + s_k[par][row] * v4;
                acc += s_q[par][row] * s[i];
            }
            if (keep) {
#pragma unroll
                for (int i = 0; i < RPT; ++i) {
                    const int row = rg + RG * i;
                    __builtin_nontemporal_store(s[i], reinterpret_cast<f32x4*>(S_out + row * DV + cg * 4));
                }
            }
            s_red[par][0][rg][cg] = acc;
            __syncthreads();
            if (rg == 0) {
                f32x4 tot = s_red[par][0][0][cg];
#pragma unroll
                for (int jj = 1; jj < RG; ++jj) tot += s_red[par][0][jj][cg];
                Vec4<TO>::store(o + tok * DV + cg * 4, tot);
            }
        } else {
            const float b = beta[tok];
            f32x4 accq = {0.f, 0.f, 0.f, 0.f}, acck = {0.f, 0.f, 0.f, 0.f};
            float qk = 0.f;
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int row = rg + RG * i;
                accq += s_q[par][row] * s[i];
                acck += s_k[par][row] * s[i];
                qk += s_q[par][row] * s_k[par][row];
            }
            s_red[par][0][rg][cg] = accq;
            s_red[par][1][rg][cg] = acck;
            if (cg == 0) s_qk[par][rg] = qk;
            __syncthreads();
            f32x4 p = s_red[par][1][0][cg];
#pragma unroll
            for (int jj = 1; jj < RG; ++jj) p += s_red[par][1][jj][cg];
            const f32x4 u = b * (v4 - a * p);
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int row = rg + RG * i;
                s[i] = a * s[i] + s_k[par][row] * u;
            }
            if (keep) {
#pragma unroll
                for (int i = 0; i < RPT; ++i) {
                    const int row = rg + RG * i;
                    __builtin_nontemporal_store(s[i], reinterpret_cast<f32x4*>(S_out + row * DV + cg * 4));
                }
            }
            if (rg == 0) {
                f32x4 qs = s_red[par][0][0][cg];
                float qkt = s_qk[par][0];
#pragma unroll
                for (int jj = 1; jj < RG; ++jj) {
                    qs += s_red[par][0][jj][cg];
                    qkt += s_qk[par][jj];
                }
                Vec4<TO>::store(o + tok * DV + cg * 4, a * qs + qkt * u);
            }
        }
    }
}

// Normalised kernelised linear attention, one token per request (page "Long
// context, fast inference, smart decoding, and life beyond attention",
// section "Linear attention: removing softmax entirely", running-state
// listing), in place on pool[slot] and zpool[slot]:
//   S <- S + phi(k)^T v;  z <- z + phi(k);  o = phi(q) S / (phi(q) . z + eps)
// with phi(x) = elu(x) + 1.  Same tiling as decode_kernel; phi(q) . z_new
// is reduced over d_k with one wave sum per wave.
__device__ __forceinline__ float elu1(float x) { return x > 0.f ? x + 1.f : expf(x); }

template <int DK, int DV, class TI, class TO>
__global__ void __launch_bounds__((DecodeShape<DK, DV>::NT))
lin_attn_decode_kernel(const typename TI::T* __restrict__ q, const typename TI::T* __restrict__ k,
                       const typename TI::T* __restrict__ v, float* __restrict__ pool,
                       float* __restrict__ zpool, int n_heads, int n_slots,
                       const int32_t* __restrict__ slot_idx, float eps,
                       typename TO::T* __restrict__ o) {
    using Sh = DecodeShape<DK, DV>;
    constexpr int NT = Sh::NT, CG = Sh::CG, RG = Sh::RG, RPT = Sh::RPT;
    constexpr int NWV = NT / 64;

    const int h = blockIdx.x % n_heads;
    const int r = blockIdx.x / n_heads;
    const int t = threadIdx.x;
    const int cg = t % CG;
    const int rg = t / CG;

    const int slot = slot_idx[r];
    if (slot < 0 || slot >= n_slots) return;

    __shared__ float s_q[DK];
    __shared__ float s_k[DK];
    __shared__ f32x4 s_red[RG][CG];
    __shared__ float s_den[NWV];

    const long head = static_cast<long>(slot) * n_heads + h;
    float* __restrict__ S = pool + head * (DK * DV);
    float* __restrict__ z = zpool + head * DK;

    f32x4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + RG * i;
        s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + row * DV + cg * 4));
    }

    const long tok = static_cast<long>(r) * n_heads + h;
    float qz = 0.f;
    for (int i = t; i < DK; i += NT) {
        const float pq = elu1(TI::load(q, tok * DK + i));
        const float pk = elu1(TI::load(k, tok * DK + i));
        s_q[i] = pq;
        s_k[i] = pk;
        const float zn = z[i] + pk;
        z[i] = zn;
        qz += pq * zn;
    }
    qz = wave_sum(qz);
    if ((t & 63) == 0) s_den[t >> 6] = qz;
    const f32x4 v4 = Vec4<TI>::load(v + tok * DV + cg * 4);
    __syncthreads();

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + RG * i;
        s[i] = s[i] + s_k[row] * v4;
        acc += s_q[row] * s[i];
        __builtin_nontemporal_store(s[i], reinterpret_cast<f32x4*>(S + row * DV + cg * 4));
    }
    s_red[rg][cg] = acc;
    __syncthreads();
    if (rg == 0) {
        f32x4 tot = s_red[0][cg];
#pragma unroll
        for (int j = 1; j < RG; ++j) tot += s_red[j][cg];
        float den = eps;
#pragma unroll
        for (int w = 0; w < NWV; ++w) den += s_den[w];
        Vec4<TO>::store(o + tok * DV + cg * 4, tot / den);
    }
}

// Plain copy of whole slots of a slot-strided buffer (a state pool, a
// normaliser pool, a conv cache): dst_slots[i] <- src_slots[i].  One
// workgroup per (pair, 16 KiB piece); 16-byte loads and stores.  A pair with
// either slot out of range, or with src == dst, is skipped.
__global__ void __launch_bounds__(256)
slot_copy_kernel(u32x4* __restrict__ buf, long slot_vec4, int pieces, int n_slots,
                 const int32_t* __restrict__ src_slots, const int32_t* __restrict__ dst_slots) {
    const int pair = blockIdx.x / pieces;
    const int piece = blockIdx.x % pieces;
    const int src = src_slots[pair];
    const int dst = dst_slots[pair];
    if (src < 0 || src >= n_slots || dst < 0 || dst >= n_slots || src == dst) return;
    const u32x4* __restrict__ from = buf + src * slot_vec4;
    u32x4* __restrict__ to = buf + dst * slot_vec4;
    constexpr int kPer = 4;     // 4 vectors per thread: 16 KiB per workgroup
    const long base = static_cast<long>(piece) * (256 * kPer) + threadIdx.x;
    u32x4 x[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const long e = base + i * 256;
        x[i] = e < slot_vec4 ? __builtin_nontemporal_load(from + e) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const long e = base + i * 256;
        if (e < slot_vec4) __builtin_nontemporal_store(x[i], to + e);
    }
}

// Measurement helper: the decode step's HBM footprint without its
// arithmetic.  Item (request r, head h) is the 64 KiB block at
// pool + (slot_idx[r] * n_heads + h) * 64 KiB, accessed like decode_kernel
// does (256 threads, 16 independent 16-byte accesses each, thread t
// touching vectors t + 256 i).  OP 0 reads every block; 1 writes zeros to
// it; 2 reads it and writes the same bytes back in place; 3 does 2 for two
// items per workgroup, both blocks read before either is written.  Loads
// and stores use the nontemporal policy unless LDEF / SDEF ask for the
// default one.  The values read are folded into a test that holds only if
// every word read is all ones (a NaN pattern), so the loads stay.
template <int OP, bool LDEF, bool SDEF>
__global__ void __launch_bounds__(256)
hbm_probe_kernel(u32x4* __restrict__ pool, int n_heads, int n_items, int n_slots,
                 const int32_t* __restrict__ slot_idx, uint32_t salt, u32x4* __restrict__ sink) {
    constexpr int PER = OP == 3 ? 2 : 1;
    constexpr int NV = 16;
    const int t = threadIdx.x;
    u32x4* base[PER];
    bool ok[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) {
        const int wi = blockIdx.x * PER + p;
        const int h = wi % n_heads, r = wi / n_heads;
        const int slot = wi < n_items ? slot_idx[r] : -1;
        ok[p] = slot >= 0 && slot < n_slots;
        base[p] = pool + (static_cast<long>(ok[p] ? slot : 0) * n_heads + h) * (256 * NV);
    }
    u32x4 x[PER][NV];
    if constexpr (OP != 1) {
#pragma unroll
        for (int p = 0; p < PER; ++p)
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const u32x4* src = base[p] + t + 256 * i;
                x[p][i] = !ok[p] ? u32x4{0u, 0u, 0u, 0u}
                                 : (LDEF ? *src : __builtin_nontemporal_load(src));
            }
    }
    if constexpr (OP == 0) {
        u32x4 acc = {~0u, ~0u, ~0u, ~0u};
#pragma unroll
        for (int i = 0; i < NV; ++i) acc &= x[0][i];
        if ((acc.x & acc.y & acc.z & acc.w) == 0xffffffffu) sink[0] = acc;
    } else {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            if (!ok[p]) continue;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const u32x4 y = OP == 1 ? u32x4{salt, salt, salt, salt} : (x[p][i] ^ salt);
                u32x4* dst = base[p] + t + 256 * i;
                if constexpr (SDEF) *dst = y;
                else __builtin_nontemporal_store(y, dst);
            }
        }
    }
}

template <int DK, int DV, class TI, class TO, bool GDN>
hipError_t launch4(const DecodeArgs& a, hipStream_t s) {
    using Sh = DecodeShape<DK, DV>;
    dim3 grid(a.n_heads * a.n_req);
    hipLaunchKernelGGL((decode_kernel<DK, DV, TI, TO, GDN>), grid, dim3(Sh::NT), 0, s,
                       static_cast<const typename TI::T*>(a.q), static_cast<const typename TI::T*>(a.k),
                       static_cast<const typename TI::T*>(a.v), a.alpha, a.beta, a.pool, a.n_heads,
                       a.n_slots, a.slot_idx, static_cast<typename TO::T*>(a.o));
    return hipGetLastError();
}

template <int DK, int DV, class TI, class TO, bool GDN>
hipError_t launch4_multi(const DecodeArgs& a, hipStream_t s) {
    using Sh = DecodeShape<DK, DV>;
    dim3 grid(a.n_heads * a.n_req);
    hipLaunchKernelGGL((decode_multi_kernel<DK, DV, TI, TO, GDN>), grid, dim3(Sh::NT), 0, s,
                       static_cast<const typename TI::T*>(a.q), static_cast<const typename TI::T*>(a.k),
                       static_cast<const typename TI::T*>(a.v), a.alpha, a.beta, a.pool, a.n_heads,
                       a.n_tok, a.n_slots, a.slot_idx, a.pos_slots, static_cast<typename TO::T*>(a.o));
    return hipGetLastError();
}

template <int DK, int DV, class TI, class TO, bool GDN>
hipError_t launch_io(const DecodeArgs& a, hipStream_t s) {
    return a.pos_slots ? launch4_multi<DK, DV, TI, TO, GDN>(a, s) : launch4<DK, DV, TI, TO, GDN>(a, s);
}

template <int DK, int DV, bool GDN>
hipError_t launch_dt(const DecodeArgs& a, hipStream_t s) {
    if (a.in_bf16) {
        return a.out_bf16 ? launch_io<DK, DV, BF16, BF16, GDN>(a, s) : launch_io<DK, DV, BF16, F32, GDN>(a, s);
    }
    return a.out_bf16 ? launch_io<DK, DV, F32, BF16, GDN>(a, s) : launch_io<DK, DV, F32, F32, GDN>(a, s);
}

template <int DK, bool GDN>
hipError_t launch_dv(const DecodeArgs& a, hipStream_t s) {
    switch (a.dv) {
        case 16: return launch_dt<DK, 16, GDN>(a, s);
        case 32: return launch_dt<DK, 32, GDN>(a, s);
        case 64: return launch_dt<DK, 64, GDN>(a, s);
        case 128: return launch_dt<DK, 128, GDN>(a, s);
    }
    return hipErrorInvalidValue;
}

template <bool GDN>
hipError_t launch(const DecodeArgs& a, hipStream_t s) {
    if (a.n_req == 0 || a.n_heads == 0 || a.n_tok == 0) return hipSuccess;
    switch (a.dk) {
        case 16: return launch_dv<16, GDN>(a, s);
        case 32: return launch_dv<32, GDN>(a, s);
        case 64: return launch_dv<64, GDN>(a, s);
        case 128: return launch_dv<128, GDN>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gla_decode(const DecodeArgs& a, hipStream_t s) { return launch<false>(a, s); }
hipError_t launch_gdn_decode(const DecodeArgs& a, hipStream_t s) { return launch<true>(a, s); }

template <int DK, int DV, class TI, class TO>
hipError_t launch_lin4(const LinDecodeArgs& a, hipStream_t s) {
    using Sh = DecodeShape<DK, DV>;
    hipLaunchKernelGGL((lin_attn_decode_kernel<DK, DV, TI, TO>), dim3(a.n_heads * a.n_req), dim3(Sh::NT),
                       0, s, static_cast<const typename TI::T*>(a.q),
                       static_cast<const typename TI::T*>(a.k), static_cast<const typename TI::T*>(a.v),
                       a.pool, a.zpool, a.n_heads, a.n_slots, a.slot_idx, a.eps,
                       static_cast<typename TO::T*>(a.o));
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_lin_dt(const LinDecodeArgs& a, hipStream_t s) {
    if (a.in_bf16) return a.out_bf16 ? launch_lin4<DK, DV, BF16, BF16>(a, s) : launch_lin4<DK, DV, BF16, F32>(a, s);
    return a.out_bf16 ? launch_lin4<DK, DV, F32, BF16>(a, s) : launch_lin4<DK, DV, F32, F32>(a, s);
}

template <int DK>
hipError_t launch_lin_dv(const LinDecodeArgs& a, hipStream_t s) {
    switch (a.dv) {
        case 16: return launch_lin_dt<DK, 16>(a, s);
        case 32: return launch_lin_dt<DK, 32>(a, s);
        case 64: return launch_lin_dt<DK, 64>(a, s);
        case 128: return launch_lin_dt<DK, 128>(a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_lin_attn_decode(const LinDecodeArgs& a, hipStream_t s) {
    if (a.n_req == 0) return hipSuccess;
    switch (a.dk) {
        case 16: return launch_lin_dv<16>(a, s);
        case 32: return launch_lin_dv<32>(a, s);
        case 64: return launch_lin_dv<64>(a, s);
        case 128: return launch_lin_dv<128>(a, s);
    }
    return hipErrorInvalidValue;
}

template <int OP, bool LDEF, bool SDEF>
void probe_launch(int items, u32x4* p, int n_heads, int n_slots, const int32_t* slot_idx, u32x4* sk,
                  hipStream_t s) {
    const int blocks = OP == 3 ? (items + 1) / 2 : items;
    hipLaunchKernelGGL((hbm_probe_kernel<OP, LDEF, SDEF>), dim3(blocks), dim3(256), 0, s, p, n_heads, items,
                       n_slots, slot_idx, 0u, sk);
}

template <int OP>
void probe_policy(int policy, int items, u32x4* p, int n_heads, int n_slots, const int32_t* slot_idx,
                  u32x4* sk, hipStream_t s) {
    switch (policy) {
        case 0: probe_launch<OP, false, false>(items, p, n_heads, n_slots, slot_idx, sk, s); break;
        case 1: probe_launch<OP, true, false>(items, p, n_heads, n_slots, slot_idx, sk, s); break;
        case 2: probe_launch<OP, false, true>(items, p, n_heads, n_slots, slot_idx, sk, s); break;
        default: probe_launch<OP, true, true>(items, p, n_heads, n_slots, slot_idx, sk, s); break;
    }
}

// mode: bits 0-1 the operation (read, write, read + write, read + write
// with two items per workgroup); bit 2 default-policy loads; bit 3
// default-policy stores.
hipError_t launch_hbm_probe(int mode, float* pool, int n_req, int n_heads, int n_slots,
                            const int32_t* slot_idx, void* sink, hipStream_t s) {
    const int items = n_req * n_heads;
    if (items == 0) return hipSuccess;
    u32x4* p = reinterpret_cast<u32x4*>(pool);
    u32x4* sk = static_cast<u32x4*>(sink);
    const int policy = (mode >> 2) & 3;
    switch (mode & 3) {
        case 0: probe_policy<0>(policy, items, p, n_heads, n_slots, slot_idx, sk, s); break;
        case 1: probe_policy<1>(policy, items, p, n_heads, n_slots, slot_idx, sk, s); break;
        case 2: probe_policy<2>(policy, items, p, n_heads, n_slots, slot_idx, sk, s); break;
        default: probe_policy<3>(policy, items, p, n_heads, n_slots, slot_idx, sk, s); break;
    }
    return hipGetLastError();
}

hipError_t launch_slot_copy(const CopyArgs& a, hipStream_t s) {
    if (a.n_copy == 0) return hipSuccess;
    const long slot_vec4 = a.slot_bytes / 16;
    const int pieces = static_cast<int>((slot_vec4 + 1023) / 1024);
    hipLaunchKernelGGL(slot_copy_kernel, dim3(a.n_copy * pieces), dim3(256), 0, s,
                       static_cast<u32x4*>(a.buf), slot_vec4, pieces, a.n_slots, a.src_slots,
                       a.dst_slots);
    return hipGetLastError();
}

}  // namespace gla
