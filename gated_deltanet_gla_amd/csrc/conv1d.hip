// Depthwise causal convolution (width <= 4) over packed variable-length
// tokens with a per-request cache of the last width-1 inputs.
//
// "Inference for linear attention and hybrid architectures", section "Two
// ways to write the same computation", last paragraph: a short causal
// convolution precedes the linear-attention layer and keeps, per request,
// the inputs of the last few tokens.  Section "The real model's ledger": an
// engine needs only width-1 of them.
//
// y[t, c] = sum_{i<W} w[c, i] * xx[t + i, c], xx = [cache rows ; sequence].
//
// HBM-bound (one read of x, one write of y).  Kernel 1: each thread owns 8
// adjacent channels (a 16-byte bf16 vector) of a run of RUN consecutive
// tokens and slides a register window along them, so x is read once (plus
// W-1 halo rows per run); a wave covers 64 x 8 consecutive channels of one
// token row (fully coalesced).  For bf16 runs that lie inside one sequence
// every row load of the run is issued before the first output is formed.  Runs may cross sequence boundaries; the window is refilled
// from the sequence's cache slot at each sequence start.  Kernel 2 then
// writes each sequence's new cache rows; it runs after kernel 1 on the same
// stream, so no thread reads a cache row that is being replaced.
#include "common.h"
#include "launch.h"

namespace gla {
namespace {

constexpr int VEC = 8;     // channels per thread
constexpr int RUN = 16;    // tokens per thread
constexpr int NT = 256;

template <class TS>
struct Row8 {
    float v[VEC];
};

template <class TS>
__device__ __forceinline__ void load8(const typename TS::T* p, float* out) {
    const f32x4 a = Vec4<TS>::load(p);
    const f32x4 b = Vec4<TS>::load(p + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

template <class TS>
__device__ __forceinline__ void store8(typename TS::T* p, const float* x) {
    Vec4<TS>::store(p, f32x4{x[0], x[1], x[2], x[3]});
    Vec4<TS>::store(p + 4, f32x4{x[4], x[5], x[6], x[7]});
}

// sequence containing token t: largest b with cu[b] <= t (cu non-decreasing)
__device__ __forceinline__ int find_seq(const int32_t* cu, int n_seqs, int t) {
    int lo = 0, hi = n_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

template <class TS, int W>
__global__ void __launch_bounds__(NT)
conv_kernel(const typename TS::T* __restrict__ x, const float* __restrict__ w,
            const int32_t* __restrict__ cu, int n_seqs, int n_tokens, int channels,
            const typename TS::T* __restrict__ cache, int n_slots,
            const int32_t* __restrict__ slot_idx, int zero_init, typename TS::T* __restrict__ y) {
    const int groups = channels / VEC;
    const long gid = static_cast<long>(blockIdx.x) * NT + threadIdx.x;
    const int cgi = static_cast<int>(gid % groups);
    const long run = gid / groups;
    const int t0 = static_cast<int>(run * RUN);
    if (t0 >= n_tokens) return;
    const int c0 = cgi * VEC;
    const int t1 = min(t0 + RUN, n_tokens);

    float wt[W][VEC];
#pragma unroll
    for (int i = 0; i < W; ++i)
#pragma unroll
        for (int j = 0; j < VEC; ++j) wt[i][j] = w[(c0 + j) * W + i];

    int b = find_seq(cu, n_seqs, t0);
    int s = clampi(cu[b], 0, n_tokens);
    int e = clampi(cu[b + 1], s, n_tokens);
    while (e <= t0 && b + 1 < n_seqs) {   // skip empty sequences that start at t0
        ++b;
        s = clampi(cu[b], 0, n_tokens);
        e = clampi(cu[b + 1], s, n_tokens);
    }
    float win[W][VEC];   // win[W-1] is the current token, win[0] the oldest

    if constexpr (TS::bytes == 2) {
        // Common case: a whole run inside one sequence, its W-1 predecessors
        // in the sequence too.  All RUN + W - 1 rows are loaded up front (one
        // 16-byte load each, all in flight together), then the outputs are
        // formed from a sliding window and stored; the same arithmetic as the
        // general path below.
        const int slot = slot_idx[b];
        if (t1 - t0 == RUN && t0 - (W - 1) >= s && t1 <= e && slot >= 0 && slot < n_slots) {
            u32x4 raw[RUN + W - 1];
#pragma unroll
            for (int i = 0; i < RUN + W - 1; ++i)
                raw[i] = *reinterpret_cast<const u32x4*>(x + static_cast<long>(t0 - (W - 1) + i) * channels + c0);
            auto unpack = [](u32x4 r, float* out) {
                const uint32_t wv[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    out[2 * j] = __uint_as_float(wv[j] << 16);
                    out[2 * j + 1] = __uint_as_float(wv[j] & 0xffff0000u);
                }
            };
#pragma unroll
            for (int i = 0; i < W - 1; ++i) unpack(raw[i], win[i]);
#pragma unroll
            for (int t = 0; t < RUN; ++t) {
                unpack(raw[t + W - 1], win[W - 1]);
                float acc[VEC];
#pragma unroll
                for (int j = 0; j < VEC; ++j) {
                    float a = 0.f;
#pragma unroll
                    for (int i = 0; i < W; ++i) a += wt[i][j] * win[i][j];
                    acc[j] = a;
                }
                *reinterpret_cast<u32x4*>(y + static_cast<long>(t0 + t) * channels + c0) =
                    u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                          pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
#pragma unroll
                for (int i = 0; i < W - 1; ++i)
#pragma unroll
                    for (int j = 0; j < VEC; ++j) win[i][j] = win[i + 1][j];
            }
            return;
        }
    }

    auto refill = [&](int t) {
        // the W-1 inputs before token t of sequence b
        const int slot = slot_idx[b];
        const bool ok = slot >= 0 && slot < n_slots;
#pragma unroll
        for (int i = 0; i < W - 1; ++i) {
            const int rel = t - s - (W - 1) + i;         // position relative to sequence start
            if (rel >= 0) {
                load8<TS>(x + static_cast<long>(s + rel) * channels + c0, win[i]);
            } else if (!zero_init && ok) {
                load8<TS>(cache + (static_cast<long>(slot) * (W - 1) + (W - 1) + rel) * channels + c0,
                          win[i]);
            } else {
#pragma unroll
                for (int j = 0; j < VEC; ++j) win[i][j] = 0.f;
            }
        }
    };
    refill(t0);
    for (int t = t0; t < t1; ++t) {
        while (t >= e && b + 1 < n_seqs) {   // entering the next (non-empty) sequence
            ++b;
            s = clampi(cu[b], 0, n_tokens);
            e = clampi(cu[b + 1], s, n_tokens);
            if (t >= s && t < e) refill(t);
        }
        const int slot = slot_idx[b];
        load8<TS>(x + static_cast<long>(t) * channels + c0, win[W - 1]);
        if (slot >= 0 && slot < n_slots && t >= s && t < e) {
            float acc[VEC];
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                float a = 0.f;
#pragma unroll
                for (int i = 0; i < W; ++i) a += wt[i][j] * win[i][j];
                acc[j] = a;
            }
            store8<TS>(y + static_cast<long>(t) * channels + c0, acc);
        }
#pragma unroll
        for (int i = 0; i < W - 1; ++i)
#pragma unroll
            for (int j = 0; j < VEC; ++j) win[i][j] = win[i + 1][j];
    }
}

template <class TS, int W>
__global__ void __launch_bounds__(NT)
conv_cache_kernel(const typename TS::T* __restrict__ x, const int32_t* __restrict__ cu, int n_seqs,
                  int n_tokens, int channels, typename TS::T* __restrict__ cache, int n_slots,
                  const int32_t* __restrict__ slot_idx, int zero_init) {
    const int groups = channels / VEC;
    const long gid = static_cast<long>(blockIdx.x) * NT + threadIdx.x;
    if (gid >= static_cast<long>(n_seqs) * groups) return;
    const int b = static_cast<int>(gid / groups);
    const int c0 = static_cast<int>(gid % groups) * VEC;
    const int slot = slot_idx[b];
    if (slot < 0 || slot >= n_slots) return;
    const int s = clampi(cu[b], 0, n_tokens);
    const int e = clampi(cu[b + 1], s, n_tokens);
    const int L = e - s;
    typename TS::T* c = cache + static_cast<long>(slot) * (W - 1) * channels + c0;
    float rows[W - 1][VEC];
#pragma unroll
    for (int i = 0; i < W - 1; ++i) {
        const int rel = L - (W - 1) + i;
        if (rel >= 0) {
            load8<TS>(x + static_cast<long>(s + rel) * channels + c0, rows[i]);
        } else if (!zero_init) {
            load8<TS>(c + static_cast<long>((W - 1) + rel) * channels, rows[i]);
        } else {
#pragma unroll
            for (int j = 0; j < VEC; ++j) rows[i][j] = 0.f;
        }
    }
#pragma unroll
    for (int i = 0; i < W - 1; ++i) store8<TS>(c + static_cast<long>(i) * channels, rows[i]);
}

template <class TS, int W>
hipError_t launch_w(const ConvArgs& a, hipStream_t s) {
    using T = typename TS::T;
    const long groups = a.channels / VEC;
    if (a.n_tokens > 0) {
        const long runs = (a.n_tokens + RUN - 1) / RUN;
        const long threads = runs * groups;
        const long blocks = (threads + NT - 1) / NT;
        hipLaunchKernelGGL((conv_kernel<TS, W>), dim3(static_cast<unsigned>(blocks)), dim3(NT), 0, s,
                           static_cast<const T*>(a.x), a.w, a.cu_seqlens, a.n_seqs, a.n_tokens,
                           a.channels, static_cast<const T*>(a.cache), a.n_slots, a.slot_idx,
                           a.zero_init, static_cast<T*>(a.y));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const long threads = static_cast<long>(a.n_seqs) * groups;
    const long blocks = (threads + NT - 1) / NT;
    hipLaunchKernelGGL((conv_cache_kernel<TS, W>), dim3(static_cast<unsigned>(blocks)), dim3(NT), 0, s,
                       static_cast<const T*>(a.x), a.cu_seqlens, a.n_seqs, a.n_tokens, a.channels,
                       static_cast<T*>(a.cache), a.n_slots, a.slot_idx, a.zero_init);
    return hipGetLastError();
}

template <class TS>
hipError_t launch_t(const ConvArgs& a, hipStream_t s) {
    switch (a.width) {
        case 2: return launch_w<TS, 2>(a, s);
        case 3: return launch_w<TS, 3>(a, s);
        case 4: return launch_w<TS, 4>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_conv1d(const ConvArgs& a, hipStream_t s) {
    return a.bf16 ? launch_t<BF16>(a, s) : launch_t<F32>(a, s);
}

}  // namespace gla
