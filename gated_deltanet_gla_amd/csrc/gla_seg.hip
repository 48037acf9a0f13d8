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
//     Lambda_g; the first segment starts from the initial state instead, so
//     its slot holds the entry state of the second, S_in(1), and it leaves a
//     copy of the initial state in the last segment's slot (not for a zero
//     initial state);
//   pass 2 (gla_seg_out): each later segment folds its entry state
//     S_in(g) = 2^Lambda_{g-1} S_in(g-1) + dS_{g-1} from those (g slot reads;
//     one, where a scan between the passes has formed the entry states),
//     the first reads the copy (the pool slot itself is rewritten by the
//     last segment in the same pass); then each runs the chunked form over
//     its chunks; the last segment writes the final state back to the pool.
//
// Within a workgroup (8 waves) each wave owns 16 columns of the 128x128
// fp32 state (held in MFMA accumulators).  Q S, P V and the state update are
// then column-local; only P = (Q K^T) .* D is shared, computed once per
// chunk by all waves and passed through LDS.  Outputs are formed transposed
// (O^T = S^T Q^T + V^T P^T): the state accumulator tile is already an MFMA
// operand in that orientation, and each lane ends up holding 4 consecutive
// columns of one token, stored as one 8-byte write.
//
// One workgroup per compute unit; chunks are double-buffered in LDS and the
// chunk after next is prefetched into registers, so each chunk costs two
// barriers.  Pass 2, per chunk:
//   phase 1: P tiles (split over the waves) -> LDS; this wave's Q S;
//   phase 2: + P V; outputs; S <- exp(g_last) S + K^T (diag(dec) V);
//            stage the prefetched chunk into the other buffer, prefetch the
//            one after.
// Pass 1 runs the state update alone.  q, k, v stay token-major in LDS;
// contractions over tokens use the LDS transpose read.  Each step issues all
// of its LDS operand reads first, so the read latency is hidden behind the
// VALU work that does not depend on them (splits, decays); that VALU work is
// placed next to MFMAs it does not feed (the state update's split before
// the P V products, the next chunk's LDS writes between the update's
// products), so the matrix and vector units run side by side.
// NORM = true runs normalised kernelised linear attention on the same two
// passes (page "Long context, fast inference, smart decoding, and life
// beyond attention", section "Linear attention: removing softmax
// entirely"): phi(x) = elu(x) + 1 is applied to q and k as they are staged,
// the gate is 1, pass 1 also sums phi(k) over each segment (one MFMA per
// half chunk against a ones operand: wave w owns rows 16w..16w+15 of the
// normaliser z) and pass 2 divides each output row by
// phi(q_i) . z_in + (row sum of P) + eps, carrying z from chunk to chunk.
// Global accesses go through buffer resources sized to the valid rows, so
// the loops have no guarded memory instructions; the output pass streams
// q, k, v with the nontemporal policy (pass 1 reads k, v with the default
// one, which leaves them in the last-level cache for pass 2).
#include <algorithm>

#include "chunk_common.h"
#include "launch.h"

namespace gla {
namespace {

constexpr int SW = 8;              // waves
constexpr int ST = SW * 64;        // threads
constexpr int SD = 128;            // d_k = d_v
constexpr int SC = 64;             // chunk
// LDS row strides (bf16 elements).  Operand fragments are read as one
// 16-byte read per lane (16 lanes on 16 rows, 8 consecutive values each)
// or with the transpose read (8 rows of 32 bytes at once); the LDS serves
// both at full rate when a row starts 8 banks (72 dwords) or 40 banks
// (40 dwords) after the one before, and at half rate at 4 banks.  Split
// 8-byte pairs are avoided altogether: the LDS serves 8-byte reads at a
// quarter of the 16-byte rate.
constexpr int LQ = SD + 16;        // 72 dwords
constexpr int LK = SD + 16;        // 72 dwords
constexpr int SP = SC + 16;        // LDS line of a P row (40 dwords)
// The output rows are written 8 bytes a lane (16 rows x 4 lane groups) and
// read back as whole rows: rows 68 dwords apart keep the 8-byte writes at
// their best rate, which 72 would halve.
constexpr int LO = SD + 8;
constexpr int kSegBlocks = 256;    // one workgroup on each of the 256 compute units
constexpr int kShortChunks = 4;    // batches of sequences this short (mean chunks) ...
constexpr int kMaxItems = 16;      // ... put up to this many heads in one output-pass block
constexpr int kScanMinSegs = 6;    // mean segments per sequence from which the entry states are scanned

// Gate tables of a chunk (seg_stage_gates): dec, the update's weights;
// smul, what the held state is multiplied by before the update (1: not
// at all); sig, the state's scale after the update.
struct KVBuf {                     // pass 1 staging
    alignas(16) uint16_t k[SC][LK];
    alignas(16) uint16_t v[SC][LK];
    alignas(16) float dec[SC];
    float smul, sig;
};

struct QKVBuf {                    // pass 2 staging
    alignas(16) uint16_t q[SC][LQ];
    alignas(16) uint16_t k[SC][LK];
    alignas(16) uint16_t v[SC][LK];
    alignas(16) float g2[SC];      // running log2 decay inside the chunk
    alignas(16) float eg[SC];      // 2^g2 times the entry state's scale
    alignas(16) float dec[SC];
    float smul, sig;
};

template <bool WQ>
struct SegPrefetch {
    static constexpr int NV = SC * SD / 8 / ST;    // 16-byte vectors per thread per tensor
    u32x4 q[WQ ? NV : 1], k[NV], v[NV];
    float a;           // raw gate of token `lane`; only the first n are valid
    int n;
};

struct SegGeom {
    int b, g, nseg, h, slot;
    int t0, t1;        // token range of this segment
    long ws_slot;      // this segment's state slot in the workspace
    long ws_first;     // slot of the sequence's first segment
};

// Which (sequence, segment, head) work item bid = segment * H + head is;
// false (for the whole block) if none.  Segment s of the call belongs to the sequence b whose
// exclusive prefix sum of max(1, ceil(L_b / lseg)) covers s; the block
// computes that prefix sum itself (threads sum contiguous ranges of
// sequences, then a wave scan and a scan of the wave totals).
__device__ __forceinline__ bool seg_geometry(SegGeom& sg, const int32_t* cu, int n_seqs, int n_tokens,
                                             int H, int lseg, const int32_t* slot_idx, int n_slots,
                                             int* sh, int bid, int maxseg) {
    const int h = bid % H;
    const int si = bid / H;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    auto count = [&](int b) {
        const int s = clampi(cu[b], 0, n_tokens);
        const int e = clampi(cu[b + 1], s, n_tokens);
        return max(1, (e - s + lseg - 1) / lseg);
    };
    const int per = (n_seqs + ST - 1) / ST;
    const int b0 = min(t * per, n_seqs), b1 = min(b0 + per, n_seqs);
    int sum = 0;
    for (int b = b0; b < b1; ++b) sum += count(b);
    int x = sum;
#pragma unroll
    for (int offs = 1; offs < 64; offs <<= 1) {
        const int y = __shfl_up(x, offs, 64);
        if (lane >= offs) x += y;
    }
    if (lane == 63) sh[wave] = x;
    if (t == 0) sh[SW] = -1;
    lds_barrier();
    int run = x - sum;
    for (int w = 0; w < wave; ++w) run += sh[w];
    if (sum > 0 && run <= si && si < run + sum) {
        for (int b = b0; b < b1; ++b) {
            const int c = count(b);
            if (si < run + c) {
                sh[SW] = b;
                sh[SW + 1] = run;
                sh[SW + 2] = c;
                break;
            }
            run += c;
        }
    }
    lds_barrier();
    // block-uniform from here on: keep it in scalar registers
    const int b = __builtin_amdgcn_readfirstlane(sh[SW]);
    if (b < 0) return false;
    const int first = __builtin_amdgcn_readfirstlane(sh[SW + 1]);
    const int nseg = __builtin_amdgcn_readfirstlane(sh[SW + 2]);
    // cu_seqlens that are not non-decreasing can claim more segments than
    // the workspace holds; such sequences are skipped rather than overrun it
    if (first + nseg > maxseg) return false;
    const int slot = slot_idx[b];
    if (slot < 0 || slot >= n_slots) return false;
    const int s0 = clampi(cu[b], 0, n_tokens);
    const int s1 = clampi(cu[b + 1], s0, n_tokens);
    const int g = si - first;
    sg.b = b;
    sg.g = g;
    sg.nseg = nseg;
    sg.h = h;
    sg.slot = slot;
    sg.t0 = min(s0 + g * lseg, s1);
    sg.t1 = min(sg.t0 + lseg, s1);
    sg.ws_first = static_cast<long>(first) * H + h;
    sg.ws_slot = static_cast<long>(si) * H + h;
    return true;
}

// Pass 1 has work only in sequences cut into two or more segments, so its
// blocks index the segments of those sequences alone (a sequence of one
// segment counts zero): a batch of short prompts launches no idle blocks.
// Block s of pass 1 is segment s of the concatenated segment lists of the
// split sequences; its workspace slot is still that segment's place among
// all segments of the call (exclusive prefix of max(1, ceil(L_b / lseg))),
// so both prefix sums are scanned together.  maxseg bounds all segments.
__device__ __forceinline__ bool split_geometry(SegGeom& sg, const int32_t* cu, int n_seqs, int n_tokens,
                                               int H, int lseg, const int32_t* slot_idx, int n_slots,
                                               int maxseg, int* sh) {
    const int h = blockIdx.x % H;
    const int si = blockIdx.x / H;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    auto count = [&](int b) {
        const int s = clampi(cu[b], 0, n_tokens);
        const int e = clampi(cu[b + 1], s, n_tokens);
        return max(1, (e - s + lseg - 1) / lseg);
    };
    const int per = (n_seqs + ST - 1) / ST;
    const int b0 = min(t * per, n_seqs), b1 = min(b0 + per, n_seqs);
    int sum_all = 0, sum_split = 0;
    for (int b = b0; b < b1; ++b) {
        const int c = count(b);
        sum_all += c;
        sum_split += c >= 2 ? c : 0;
    }
    int xa = sum_all, xs = sum_split;
#pragma unroll
    for (int offs = 1; offs < 64; offs <<= 1) {
        const int ya = __shfl_up(xa, offs, 64);
        const int ys = __shfl_up(xs, offs, 64);
        if (lane >= offs) {
            xa += ya;
            xs += ys;
        }
    }
    if (lane == 63) {
        sh[wave] = xa;
        sh[SW + wave] = xs;
    }
    if (t == 0) sh[2 * SW] = -1;
    lds_barrier();
    int run_all = xa - sum_all, run_split = xs - sum_split;
    for (int w = 0; w < wave; ++w) {
        run_all += sh[w];
        run_split += sh[SW + w];
    }
    if (sum_split > 0 && run_split <= si && si < run_split + sum_split) {
        for (int b = b0; b < b1; ++b) {
            const int c = count(b);
            const int cs = c >= 2 ? c : 0;
            if (si < run_split + cs) {
                sh[2 * SW] = b;
                sh[2 * SW + 1] = run_all;
                sh[2 * SW + 2] = c;
                sh[2 * SW + 3] = si - run_split;
                break;
            }
            run_split += cs;
            run_all += c;
        }
    }
    lds_barrier();
    const int b = __builtin_amdgcn_readfirstlane(sh[2 * SW]);
    if (b < 0) return false;
    const int first = __builtin_amdgcn_readfirstlane(sh[2 * SW + 1]);
    const int nseg = __builtin_amdgcn_readfirstlane(sh[2 * SW + 2]);
    const int g = __builtin_amdgcn_readfirstlane(sh[2 * SW + 3]);
    // the same guard as the output pass: never past the workspace
    if (first + nseg > maxseg) return false;
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
    sg.ws_first = static_cast<long>(first) * H + h;
    sg.ws_slot = static_cast<long>(first + g) * H + h;
    return true;
}

// A state slot in the workspace holds the 128x128 state as the MFMA
// accumulator fragments of the 8 waves, tile-major: tile mt of lane l of
// wave w (4 values) at ((w * 8 + mt) * 64 + l) * 4, so a wave reads or
// writes one tile as one contiguous 1 KiB (16 bytes a lane); tile mt is
// kSlotTile * mt floats after tile 0.
constexpr int kSlotTile = 64 * 4;
// This lane's 8 tiles of a slot, through a buffer resource: the tile
// offsets (up to 7 KiB) go in the scalar offset, so the eight loads share
// one address register.
struct SlotReader {
    BufRsrc rs;
    uint32_t lo;
    __device__ __forceinline__ SlotReader(const float* ws, long slot)
        : rs(ws + slot * SD * SD, SD * SD * 4),
          lo(static_cast<uint32_t>(((threadIdx.x >> 6) * 8 * 64 + (threadIdx.x & 63)) * 16)) {}
    __device__ __forceinline__ f32x4 tile(int mt) const {
        return __builtin_bit_cast(f32x4, rs.load16(lo, static_cast<uint32_t>(mt * kSlotTile * 4)));
    }
};

// The output pass holds the state in the accumulator row order srow()
// (tiles 2s and 2s + 1 give each lane 8 consecutive state rows, which meet
// q fragments in natural order).  Pass 1, which never multiplies S by q,
// keeps the plain order (tile mt, rows 16 mt + 4 g + r), in which its
// transpose reads of K run at full rate, and reorders its tiles only as it
// writes them to the workspace.
// This wave's 8 state tiles read from a row-major [d][n] state (OUT: the
// output pass's row order).
template <bool OUT>
__device__ __forceinline__ void load_state_rowmajor(f32x4 (&S)[8], const float* src, int col) {
    const AccPos ap;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
        const int r0 = OUT ? srow(mt, ap.row0) : mt * 16 + ap.row0;
#pragma unroll
        for (int r = 0; r < 4; ++r) S[mt][r] = src[(r0 + r) * SD + col + ap.col];
    }
}

// Pass 1's tiles (plain row order) into a workspace slot in the output
// pass's order: plain tile mt', group g', row r is state row
// 16 mt' + 4 g' + r, which the output pass holds in tile 2 (mt' / 2) + g' % 2
// of lane group 2 (mt' % 2) + g' / 2 (same column, same wave).
__device__ __forceinline__ void store_slot_out_order(float* ws, long slot, const f32x4 (&S)[8]) {
    const int t = threadIdx.x, lane = t & 63, g = lane >> 4;
    float* base = ws + slot * SD * SD + (t >> 6) * 8 * kSlotTile;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
        const int dl = (lane & 15) + 16 * (2 * (mt & 1) + (g >> 1));
        *reinterpret_cast<f32x4*>(base + (2 * (mt >> 1) + (g & 1)) * kSlotTile + dl * 4) = S[mt];
    }
}

// One chunk's global slices (rows past n read as zero) into registers;
// GATED = false (no gate) loads no alpha.
template <bool WQ, bool GATED = true>
__device__ __forceinline__ void seg_fetch(SegPrefetch<WQ>& pf, const uint16_t* q, const uint16_t* k,
                                          const uint16_t* v, const float* alpha, long tok0, int n, int h,
                                          int H) {
    const long stride = static_cast<long>(H) * SD;
    const uint32_t ext = rows_extent(n, stride * 2, SD * 2);
    const BufRsrc rk(k + tok0 * stride + h * SD, ext);
    const BufRsrc rv(v + tok0 * stride + h * SD, ext);
    // only wave 0 scans the decays: the other waves' alpha loads are out of
    // range (no memory traffic) and read as zero
    const bool w0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0;
    const BufRsrc ra(alpha + tok0 * H + h, (GATED && w0) ? rows_extent(n, static_cast<long>(H) * 4, 4) : 0u);
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < SegPrefetch<WQ>::NV; ++u) {
        const int x = tid + u * ST;
        const uint32_t offb = static_cast<uint32_t>(((x / (SD / 8)) * stride + (x % (SD / 8)) * 8) * 2);
        if constexpr (WQ) {
            pf.q[u] = BufRsrc(q + tok0 * stride + h * SD, ext).load16_nt(offb);
            pf.k[u] = rk.load16_nt(offb);
            pf.v[u] = rv.load16_nt(offb);
        } else {
            pf.k[u] = rk.load16(offb);
            pf.v[u] = rv.load16(offb);
        }
    }
    const int lane = tid & 63;
    // The gates of rows past n are replaced by 1 when staged, not here: a
    // select on the loaded value would make this wave wait for the load now.
    pf.a = ra.loadf_nt(static_cast<uint32_t>(lane * H * 4));
    pf.n = n;
}

// phi(x) = elu(x) + 1 on 8 packed bf16 values (the hardware exp: the result
// is rounded to bf16 right after)
__device__ __forceinline__ float elu1(float x) { return x > 0.f ? x + 1.f : __expf(x); }
__device__ __forceinline__ u32x4 phi8(u32x4 w) {
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        r[e] = pack_bf16x2(elu1(__uint_as_float(w[e] << 16)), elu1(__uint_as_float(w[e] & 0xffff0000u)));
    return r;
}

// Registers -> LDS: the q, k, v rows (NORM: phi(q), phi(k); rows past the
// sequence stay zero, since phi(0) = 1 would count them).
template <bool WQ, bool NORM = false, class Buf>
__device__ __forceinline__ void seg_stage_rows(Buf& bb, const SegPrefetch<WQ>& pf) {
    // NORM compares rows with n: keep that row index from being held across
    // the chunk loop
    const int tid = NORM ? opaque(static_cast<int>(threadIdx.x)) : static_cast<int>(threadIdx.x);
#pragma unroll
    for (int u = 0; u < SegPrefetch<WQ>::NV; ++u) {
        const int xx = tid + u * ST;
        const int row = xx / (SD / 8), vc = (xx % (SD / 8)) * 8;
        u32x4 kv = pf.k[u];
        if constexpr (NORM) {
            if (row < pf.n) kv = phi8(kv);
        }
        if constexpr (WQ) {
            u32x4 qv = pf.q[u];
            if constexpr (NORM) {
                if (row < pf.n) qv = phi8(qv);
            }
            *reinterpret_cast<u32x4*>(&bb.q[row][vc]) = qv;
        }
        *reinterpret_cast<u32x4*>(&bb.k[row][vc]) = kv;
        *reinterpret_cast<u32x4*>(&bb.v[row][vc]) = pf.v[u];
    }
}

// The state is held as S = sigma Shat, sigma a running product of the
// chunks' total decays gamma = 2^g2_last: the update
// S <- gamma S + K^T diag(2^(g2_last - g2)) V is then
// Shat <- Shat + K^T diag(2^(-g2 - log2 sigma)) V with sigma <- gamma sigma, no
// pass over the state, as long as gamma sigma stays at or above
// 2^kFoldFloor; a chunk that would take it lower scales Shat by gamma sigma
// before its update and restarts sigma at 1.  That bounds Shat by
// 2^-kFoldFloor |S| and the weights by 2^(-2 kFoldFloor).
constexpr float kFoldFloor = -30.f;

// Wave 0 scans log2(alpha), writes the per-token tables and gets the chunk's
// total log2 decay back (other waves get 0).  lsig: log2 sigma of the state
// entering the chunk on wave 0, updated to the state leaving it; reset: the
// chunk starts a new state (sigma = 1).
template <bool WQ, bool NORM = false, class Buf>
__device__ __forceinline__ float seg_stage_gates(Buf& bb, const SegPrefetch<WQ>& pf, float& lsig, bool reset = false) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    float glast = 0.f;
    if (__builtin_amdgcn_readfirstlane(tid >> 6) == 0) {
        const float a = (!NORM && lane < pf.n) ? pf.a : 1.f;
        const float x = wave_inclusive_sum(__log2f(fmaxf(a, kMinDecay)));
        glast = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), SC - 1));
        const float l0 = reset ? 0.f : lsig;
        const bool fold = l0 + glast >= kFoldFloor;
        if constexpr (WQ) {
            bb.g2[lane] = x;
            bb.eg[lane] = hw_exp2(x + l0);
        }
        bb.dec[lane] = hw_exp2(fold ? -x - l0 : glast - x);
        if (lane == 0) {
            bb.smul = fold ? 1.f : hw_exp2(l0 + glast);
            bb.sig = fold ? hw_exp2(l0 + glast) : 1.f;
        }
        // wave-uniform: kept in a scalar register across the chunk loop
        lsig = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, fold ? l0 + glast : 0.f)));
    }
    return glast;
}

// Registers -> LDS (rows and gate tables); returns the chunk's total log2
// decay on wave 0.
template <bool WQ, bool NORM = false, class Buf>
__device__ __forceinline__ float seg_stage(Buf& bb, const SegPrefetch<WQ>& pf, float& lsig) {
    const float glast = seg_stage_gates<WQ, NORM>(bb, pf, lsig);
    seg_stage_rows<WQ, NORM>(bb, pf);
    return glast;
}

// z rows 16w..16w+15 (wave w) += sum over the chunk's tokens of phi(k): the
// k^T fragments of those rows times a ones operand (every column of the
// accumulator tile holds the same sums).
template <class Buf>
__device__ __forceinline__ void seg_z_update(f32x4& z, const Buf& bb, int wave) {
    const bf16x8 ones = as_bf16x8(u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
    const int m0 = opaque(wave * 16);     // recomputed per chunk, not held across the loop
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) z = mfma_bf16(frag_km_split(&bb.k[0][0], LK, m0, 32 * ks), ones, z);
}

// V^T operand of this wave's 16 columns for the two 32-token halves of the
// chunk (split k order, so the same registers serve P V and the state update).
template <class Buf>
__device__ __forceinline__ void load_vt(bf16x8 (&vf)[2], const Buf& bb, int col) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) vf[ks] = frag_km_split(&bb.v[0][0], LK, col, 32 * ks);
}

// State update Shat (this wave's 16 columns, all 8 row tiles) <- smul Shat +
// K^T diag(dec) V, in two parts: the operand reads and the VALU work
// (decayed, split values; the smul scaling), then the MFMAs.
struct SegUpd {
    bf16x8 kf[2][8];
    bf16x8 vh[2], vl[2];
};
// SKIP: a block-uniform branch skips the multiply when smul is 1 (where
// the branch would make the loop's register allocation spill, the multiply
// by 1 is done instead).
template <bool OUT, bool SKIP, class Buf>
__device__ __forceinline__ void seg_update_prep(SegUpd& up, f32x4 (&S)[8], const Buf& bb, const bf16x8 (&vf)[2]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
            up.kf[ks][mt] = OUT ? frag_kt_pair(&bb.k[0][0], LK, mt, 32 * ks)
                                : frag_km_split(&bb.k[0][0], LK, mt * 16, 32 * ks);
    __builtin_amdgcn_sched_barrier(0);
    // decayed values for tokens {32ks + 4g + e} u {32ks + 16 + 4g + e}, split
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const u32x4 vw = __builtin_bit_cast(u32x4, vf[ks]);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(&bb.dec[32 * ks + 4 * g]);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(&bb.dec[32 * ks + 16 + 4 * g]);
        uint32_t hw[4], lw[4];
        split_bf16x2(__uint_as_float(vw.x << 16) * d0.x, __uint_as_float(vw.x & 0xffff0000u) * d0.y, hw[0], lw[0]);
        split_bf16x2(__uint_as_float(vw.y << 16) * d0.z, __uint_as_float(vw.y & 0xffff0000u) * d0.w, hw[1], lw[1]);
        split_bf16x2(__uint_as_float(vw.z << 16) * d1.x, __uint_as_float(vw.z & 0xffff0000u) * d1.y, hw[2], lw[2]);
        split_bf16x2(__uint_as_float(vw.w << 16) * d1.z, __uint_as_float(vw.w & 0xffff0000u) * d1.w, hw[3], lw[3]);
        up.vh[ks] = as_bf16x8(u32x4{hw[0], hw[1], hw[2], hw[3]});
        up.vl[ks] = as_bf16x8(u32x4{lw[0], lw[1], lw[2], lw[3]});
    }
    const float sm = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, bb.smul)));
    if (!SKIP || sm != 1.f) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) S[mt] *= sm;
    }
}
__device__ __forceinline__ void seg_update_mfma_half(f32x4 (&S)[8], const SegUpd& up, int ks) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
        S[mt] = mfma_bf16(up.kf[ks][mt], up.vh[ks], S[mt]);
        S[mt] = mfma_bf16(up.kf[ks][mt], up.vl[ks], S[mt]);
    }
}
__device__ __forceinline__ void seg_update_mfma(f32x4 (&S)[8], const SegUpd& up) {
    seg_update_mfma_half(S, up, 0);
    seg_update_mfma_half(S, up, 1);
}
template <class Buf>
__device__ __forceinline__ void seg_state_update(f32x4 (&S)[8], const Buf& bb, const bf16x8 (&vf)[2]) {
    SegUpd up;
    seg_update_prep<false, true>(up, S, bb, vf);
    __builtin_amdgcn_sched_barrier(0);
    seg_update_mfma(S, up);
}

// ------------------------------------------------------------------ pass 1
template <bool NORM>
__global__ void __launch_bounds__(ST)
gla_seg_state(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
              const float* __restrict__ alpha, const int32_t* __restrict__ cu, int n_seqs,
              int n_tokens, int H, const float* __restrict__ pool, int n_slots,
              const int32_t* __restrict__ slot_idx, int zero_init, int lseg,
              float* __restrict__ wstate, float* __restrict__ wlam, const float* __restrict__ zpool,
              float* __restrict__ wz, int maxseg) {
    __shared__ int sh[2 * SW + 4];
    SegGeom sg;
    if (!split_geometry(sg, cu, n_seqs, n_tokens, H, lseg, slot_idx, n_slots, maxseg, sh)) return;
    // no split: pass 2 reads the pool itself; the last segment's local
    // state is never used
    if (sg.nseg <= 1 || sg.g == sg.nseg - 1) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const AccPos ap;
    const int col = wave * 16;
    f32x4 S[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) S[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 zacc = {0.f, 0.f, 0.f, 0.f};
    // The first segment runs from the initial state (sigma = 1), so that its
    // slot holds the second segment's entry state S_in(1); it also copies
    // the initial state to the last segment's slot, from which pass 2's
    // first segment reads it.
    if (sg.g == 0 && !zero_init) {
        const long pslot = static_cast<long>(sg.slot) * H + sg.h;
        const long last = sg.ws_first + static_cast<long>(sg.nseg - 1) * H;
        load_state_rowmajor<false>(S, pool + pslot * SD * SD, col);
        store_slot_out_order(wstate, last, S);
        if constexpr (NORM) {
            zacc = *reinterpret_cast<const f32x4*>(zpool + pslot * SD + wave * 16 + ap.row0);
            if (threadIdx.x < SD) wz[last * SD + threadIdx.x] = zpool[pslot * SD + threadIdx.x];
        }
    }

    __shared__ KVBuf buf[2];
    const int nch = (sg.t1 - sg.t0 + SC - 1) / SC;
    auto rows = [&](int c) { return c < nch ? min(SC, sg.t1 - sg.t0 - c * SC) : 0; };
    auto tok = [&](int c) { return static_cast<long>(sg.t0) + static_cast<long>(c < nch ? c : 0) * SC; };
    SegPrefetch<false> pf;
    float lam = 0.f, lsig = 0.f;
    seg_fetch<false, !NORM>(pf, nullptr, k, v, alpha, tok(0), rows(0), sg.h, H);
    lam += seg_stage<false, NORM>(buf[0], pf, lsig);
    seg_fetch<false, !NORM>(pf, nullptr, k, v, alpha, tok(1), rows(1), sg.h, H);
    lds_barrier();
    for (int c = 0; c < nch; ++c) {
        bf16x8 vf[2];
        load_vt(vf, buf[c & 1], col);
        seg_state_update(S, buf[c & 1], vf);
        if constexpr (NORM) seg_z_update(zacc, buf[c & 1], wave);
        const float gl = seg_stage<false, NORM>(buf[(c + 1) & 1], pf, lsig);
        if (c + 1 < nch) lam += gl;
        seg_fetch<false, !NORM>(pf, nullptr, k, v, alpha, tok(c + 2), rows(c + 2), sg.h, H);
        lds_barrier();
    }
    // dS = sigma Shat (sigma after the last chunk; the loop's last staging
    // went to the other buffer)
    const float sgl = nch > 0 ? buf[(nch - 1) & 1].sig : 1.f;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) S[mt] *= sgl;
    store_slot_out_order(wstate, sg.ws_slot, S);
    if (threadIdx.x == 0) wlam[sg.ws_slot] = lam;
    if constexpr (NORM) {
        if (ap.col == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) wz[sg.ws_slot * SD + wave * 16 + ap.row0 + r] = zacc[r];
        }
    }
}

// ------------------------------------------------------------------ scan
// Entry states by a scan over pass 1's slots, for calls whose sequences
// have many segments: folded in pass 2 instead, segment g would read g
// slots, a number of reads quadratic in the segments.  Slot j >= 1 of a
// split sequence becomes S_in(j + 1) = 2^Lambda_j S_in(j) + dS_j, from
// slot 0 = S_in(1), so pass 2's segment g >= 1 reads slot g - 1 alone
// (and z_in likewise, without decay).  Block (s, c) runs on pass 1's
// geometry (s as there; only a sequence's first segment does the scan) and
// takes floats [c * 2048, (c + 1) * 2048) of every slot, 4 per thread: the
// scan is elementwise, so any split of a slot will do.  Slot loads are
// issued kScanBatch at a time ahead of the chained multiply-adds.
constexpr int kScanCols = 8;       // blocks per sequence and head
constexpr int kScanBatch = 8;
template <bool NORM>
__global__ void __launch_bounds__(ST)
gla_seg_scan(const int32_t* __restrict__ cu, int n_seqs, int n_tokens, int H, int lseg,
             const int32_t* __restrict__ slot_idx, int n_slots, int maxseg, float* __restrict__ wstate,
             const float* __restrict__ wlam, float* __restrict__ wz) {
    __shared__ int sh[2 * SW + 4];
    SegGeom sg;
    if (!split_geometry(sg, cu, n_seqs, n_tokens, H, lseg, slot_idx, n_slots, maxseg, sh)) return;
    if (sg.nseg <= 2 || sg.g != 0) return;        // nothing to scan
    const int n = sg.nseg - 1;                     // slots 0 .. n - 1 of this sequence
    const long off = static_cast<long>(blockIdx.y) * (SD * SD / kScanCols) + threadIdx.x * 4;
    auto slot = [&](int j) { return wstate + (sg.ws_first + static_cast<long>(j) * H) * SD * SD + off; };
    f32x4 S = *reinterpret_cast<const f32x4*>(slot(0));
    for (int j0 = 1; j0 < n; j0 += kScanBatch) {
        f32x4 L[kScanBatch];
        float lam[kScanBatch];
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u) {
            if (j0 + u < n) {
                L[u] = *reinterpret_cast<const f32x4*>(slot(j0 + u));
                lam[u] = wlam[sg.ws_first + static_cast<long>(j0 + u) * H];
            }
        }
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u) {
            if (j0 + u < n) {
                S = hw_exp2(lam[u]) * S + L[u];
                *reinterpret_cast<f32x4*>(slot(j0 + u)) = S;
            }
        }
    }
    if constexpr (NORM) {
        if (blockIdx.y == 0 && threadIdx.x < SD) {
            float* z = wz + sg.ws_first * SD + threadIdx.x;
            float acc = z[0];
            for (int j = 1; j < n; ++j) {
                acc += z[static_cast<long>(j) * H * SD];
                z[static_cast<long>(j) * H * SD] = acc;
            }
        }
    }
}

// ------------------------------------------------------------------ pass 2
template <class TO, bool CKPT, bool NORM>
__global__ void __launch_bounds__(ST)
gla_seg_out(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
            const float* __restrict__ alpha, const int32_t* __restrict__ cu, int n_seqs, int n_tokens,
            int H, float* __restrict__ pool, int n_slots, const int32_t* __restrict__ slot_idx,
            int zero_init, int lseg, const float* __restrict__ wstate, const float* __restrict__ wlam,
            int scanned, Ckpt ck, float* __restrict__ zpool, const float* __restrict__ wz, float eps,
            typename TO::T* __restrict__ o) {
    __shared__ int sh[SW + 4];
    SegGeom sg;
    if (!seg_geometry(sg, cu, n_seqs, n_tokens, H, lseg, slot_idx, n_slots, sh, blockIdx.x, gridDim.x / H)) return;
    __shared__ QKVBuf buf[2];
    __shared__ uint16_t pbuf[2][SC][SP];           // P = (Q K^T) .* D, hi and lo planes
    // bf16 outputs of the previous chunk, stored to HBM as whole rows
    __shared__ uint16_t obuf[TO::bytes == 2 ? SC : 1][LO];
    // NORM: z_in by chunk parity, row sums of the 10 P tiles, phi(q_i) . z_in
    __shared__ alignas(16) float zb[NORM ? 2 : 1][NORM ? SD : 1];
    __shared__ float dpart[NORM ? 10 : 1][16];
    __shared__ float qzb[NORM ? SC : 1];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const AccPos ap;
    const int col = wave * 16;
    const long stride = static_cast<long>(H) * SD;

    const int nch = (sg.t1 - sg.t0 + SC - 1) / SC;
    auto rows = [&](int c) { return c < nch ? min(SC, sg.t1 - sg.t0 - c * SC) : 0; };
    auto tok = [&](int c) { return static_cast<long>(sg.t0) + static_cast<long>(c < nch ? c : 0) * SC; };
    SegPrefetch<true> pf;
    seg_fetch<true, !NORM>(pf, q, k, v, alpha, tok(0), rows(0), sg.h, H);     // in flight during the fold
    const long zoff = (static_cast<long>(sg.slot) * H + sg.h) * SD;

    // ---- entry state of this segment
    f32x4 S[8];
    float* Sg = pool + (static_cast<long>(sg.slot) * H + sg.h) * SD * SD;
    if (sg.nseg <= 1 || (sg.g == 0 && zero_init)) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) S[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (!zero_init) load_state_rowmajor<true>(S, Sg, col);
    } else {
        // first segment: the copy of the initial state in the last
        // segment's slot; later ones: slot 0 holds S_in(1), and after the
        // scan slot g - 1 holds S_in(g)
        const long s_in = sg.g == 0 ? static_cast<long>(sg.nseg - 1) : (scanned ? sg.g - 1 : 0);
        const SlotReader s0(wstate, sg.ws_first + s_in * H);
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) S[mt] = s0.tile(mt);
        for (int j = 1; j < (scanned ? 0 : sg.g); ++j) {
            const long sj = sg.ws_first + static_cast<long>(j) * H;
            const float dcy = hw_exp2(wlam[sj]);
            const SlotReader dS(wstate, sj);
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) S[mt] = dcy * S[mt] + dS.tile(mt);
        }
    }
    if constexpr (NORM) {
        // entry normaliser z_in: rows wave*16 + row0 .. + 3
        const int zr = wave * 16 + ap.row0;
        f32x4 zacc = {0.f, 0.f, 0.f, 0.f};
        if (sg.nseg <= 1 || (sg.g == 0 && zero_init)) {
            if (!zero_init) zacc = *reinterpret_cast<const f32x4*>(zpool + zoff + zr);
        } else {
            const long z_in = sg.g == 0 ? static_cast<long>(sg.nseg - 1) : (scanned ? sg.g - 1 : 0);
            zacc = *reinterpret_cast<const f32x4*>(wz + (sg.ws_first + z_in * H) * SD + zr);
            for (int j = 1; j < (scanned ? 0 : sg.g); ++j)
                zacc += *reinterpret_cast<const f32x4*>(wz + (sg.ws_first + static_cast<long>(j) * H) * SD + zr);
        }
        if (ap.col == 0) *reinterpret_cast<f32x4*>(&zb[0][zr]) = zacc;
    }
    // P tiles above the diagonal that P V still reads (rows 0-15 x keys 16-31,
    // rows 32-47 x keys 48-63) stay zero; the others are rewritten each chunk.
    for (int idx = tid; idx < 2 * 256; idx += ST) {
        const int t = idx >> 8, e = idx & 255;
        const int row = (t ? 32 : 0) + (e >> 4), cx = p_col(t ? 3 : 1, (e >> 2) & 3) + (e & 3);
        pbuf[0][row][cx] = 0;
        pbuf[1][row][cx] = 0;
    }
    float lsig = 0.f;                              // log2 sigma on wave 0
    seg_stage<true, NORM>(buf[0], pf, lsig);
    seg_fetch<true, !NORM>(pf, q, k, v, alpha, tok(1), rows(1), sg.h, H);
    lds_barrier();

    // P tile t of (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) (3,1) (3,2) (3,3):
    // operand reads, then the MFMAs and the decay / mask / split epilogue
    auto tile_it = [](int t) { return t < 1 ? 0 : (t < 3 ? 1 : (t < 6 ? 2 : 3)); };
    auto p_load = [&](const QKVBuf& bb, int t, bf16x8 (&pa)[4], bf16x8 (&pb)[4]) {
        const int it = tile_it(t), jt = t - it * (it + 1) / 2;
#pragma unroll
        for (int ks = 0; ks < SD / 32; ++ks) {
            pa[ks] = frag_kc(&bb.k[0][0], LK, jt * 16, 32 * ks);
            pb[ks] = frag_kc(&bb.q[0][0], LQ, it * 16, 32 * ks);
        }
    };
    auto p_finish = [&](const QKVBuf& bb, int t, const bf16x8 (&pa)[4], const bf16x8 (&pb)[4]) {
        const int it = tile_it(t), jt = t - it * (it + 1) / 2;
        f32x4 pt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < SD / 32; ++ks) pt = mfma_bf16(pa[ks], pb[ks], pt);
        const int i = it * 16 + ap.col;
        const float gi = bb.g2[i];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = jt * 16 + ap.row0 + r;
            pt[r] = (j <= i) ? pt[r] * hw_exp2(gi - bb.g2[j]) : 0.f;
        }
        const int pc = p_col(jt, ap.row0 >> 2);
        Op<false>::store4(&pbuf[0][i][pc], &pbuf[1][i][pc], pt);
        if constexpr (NORM) {
            // row i's sum over this tile's 16 keys (spread over the 4 lane groups)
            float rs = (pt[0] + pt[1]) + (pt[2] + pt[3]);
            rs += __shfl_xor(rs, 16, 64);
            rs += __shfl_xor(rs, 32, 64);
            if ((threadIdx.x & 63) < 16) dpart[t][opaque(ap.col)] = rs;
        }
    };

    // chunk cc's bf16 outputs: LDS -> HBM, 16 lanes per 256-byte row
    auto flush_o = [&](int cc) {
        if constexpr (TO::bytes == 2) {
            const BufRsrc ro(o + tok(cc) * stride + sg.h * SD, rows_extent(rows(cc), stride * 2, SD * 2));
#pragma unroll
            for (int u = 0; u < SC * SD / 8 / ST; ++u) {
                const int x = tid + u * ST, row = x / (SD / 8), vc = (x % (SD / 8)) * 8;
                ro.store_b128(*reinterpret_cast<const u32x4*>(&obuf[row][vc]),
                              static_cast<uint32_t>((row * stride + vc) * 2));
            }
        }
    };

    for (int c = 0; c < nch; ++c) {
        const QKVBuf& bb = buf[c & 1];
        const int n = rows(c);
        const long tok0 = tok(c);
        if (c > 0) flush_o(c - 1);

        // ---- phase 1: P tiles (split over the waves) -> LDS, and
        // O^T = S^T Q^T for this wave's columns (the state accumulator tiles
        // serve as the A operand directly: rows = columns of S)
        bf16x8 pa[4], pb[4], qf[4][4];
        p_load(bb, wave, pa, pb);
#pragma unroll
        for (int s = 0; s < SD / 32; ++s)
#pragma unroll
            for (int it = 0; it < 4; ++it) qf[s][it] = frag_kc(&bb.q[0][0], LQ, it * 16, 32 * s);
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 sh8[4], sl8[4];
#pragma unroll
        for (int s = 0; s < SD / 32; ++s) {
            s16x4 h0, l0, h1, l1;
            split4(S[2 * s], h0, l0);
            split4(S[2 * s + 1], h1, l1);
            sh8[s] = cat8(h0, h1);
            sl8[s] = cat8(l0, l1);
        }
        f32x4 ot[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) ot[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < SD / 32; ++s)
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                ot[it] = mfma_bf16(sh8[s], qf[s][it], ot[it]);
                ot[it] = mfma_bf16(sl8[s], qf[s][it], ot[it]);
            }
        p_finish(bb, wave, pa, pb);
        if (wave + SW < 10) {
            p_load(bb, wave + SW, pa, pb);
            p_finish(bb, wave + SW, pa, pb);
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) ot[it] *= bb.eg[it * 16 + ap.col];
        if constexpr (NORM) {
            // phi(q_i) . z_in: 8 threads per row, 16 dimensions each (the
            // lane offsets are recomputed each chunk, not held across the loop)
            const int tq = opaque(tid);
            const int i = tq >> 3, d0 = (tq & 7) * 16;
            const float* zin = zb[c & 1];
            float acc = 0.f;
#pragma unroll
            for (int h8 = 0; h8 < 2; ++h8) {
                const u32x4 qw = *reinterpret_cast<const u32x4*>(&bb.q[i][d0 + 8 * h8]);
                const f32x4 z0 = *reinterpret_cast<const f32x4*>(zin + d0 + 8 * h8);
                const f32x4 z1 = *reinterpret_cast<const f32x4*>(zin + d0 + 8 * h8 + 4);
                acc += __uint_as_float(qw.x << 16) * z0.x + __uint_as_float(qw.x & 0xffff0000u) * z0.y;
                acc += __uint_as_float(qw.y << 16) * z0.z + __uint_as_float(qw.y & 0xffff0000u) * z0.w;
                acc += __uint_as_float(qw.z << 16) * z1.x + __uint_as_float(qw.z & 0xffff0000u) * z1.y;
                acc += __uint_as_float(qw.w << 16) * z1.z + __uint_as_float(qw.w & 0xffff0000u) * z1.w;
            }
            // sum over the row's 8 lanes by DPP: partners 1 and 2 apart, then
            // the other quad (the half-row mirror; its lanes hold equal sums)
            auto dpp_add = [](float x, int ctrl) {
                const int y = ctrl == 0xb1 ? __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xb1, 0xf, 0xf, false)
                            : ctrl == 0x4e ? __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4e, 0xf, 0xf, false)
                                           : __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xf, 0xf, false);
                return x + __int_as_float(y);
            };
            acc = dpp_add(acc, 0xb1);     // quad_perm [1,0,3,2]
            acc = dpp_add(acc, 0x4e);     // quad_perm [2,3,0,1]
            acc = dpp_add(acc, 0x141);    // row_half_mirror
            if ((tq & 7) == 0) qzb[i] = acc;
        }
        lds_barrier();

        // ---- phase 2: + V^T P^T (split k order on both operands), outputs,
        // state update, next chunk
        bf16x8 vf[2], pp[6][2];
        load_vt(vf, bb, col);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            pp[it][0] = frag_kc(&pbuf[0][0][0], SP, it * 16, 0);
            pp[it][1] = frag_kc(&pbuf[1][0][0], SP, it * 16, 0);
        }
#pragma unroll
        for (int it = 2; it < 4; ++it) {
            pp[it + 2][0] = frag_kc(&pbuf[0][0][0], SP, it * 16, 32);
            pp[it + 2][1] = frag_kc(&pbuf[1][0][0], SP, it * 16, 32);
        }
        __builtin_amdgcn_sched_barrier(0);
        // the state update's operand reads and VALU work go ahead of the
        // P V MFMAs, which do not depend on them, so they can overlap
        SegUpd up;
        seg_update_prep<true, !CKPT>(up, S, bb, vf);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            ot[it] = mfma_bf16(vf[0], pp[it][0], ot[it]);
            ot[it] = mfma_bf16(vf[0], pp[it][1], ot[it]);
        }
#pragma unroll
        for (int it = 2; it < 4; ++it) {
            ot[it] = mfma_bf16(vf[1], pp[it + 2][0], ot[it]);
            ot[it] = mfma_bf16(vf[1], pp[it + 2][1], ot[it]);
        }
        if constexpr (NORM) {
            const int lc = opaque(ap.col);
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int i = it * 16 + lc;
                float den = qzb[i] + eps;
#pragma unroll
                for (int jt = 0; jt <= it; ++jt) den += dpart[it * (it + 1) / 2 + jt][lc];
                ot[it] *= __builtin_amdgcn_rcpf(den);   // hardware reciprocal (1 ulp), not a division
            }
        }
        // lane: token it*16 + (lane % 16), columns col + 4 (lane / 16) .. +3
        if constexpr (TO::bytes == 2) {
#pragma unroll
            for (int it = 0; it < 4; ++it)
                *reinterpret_cast<u32x2*>(&obuf[it * 16 + ap.col][col + ap.row0]) =
                    u32x2{pack_bf16x2(ot[it][0], ot[it][1]), pack_bf16x2(ot[it][2], ot[it][3])};
        } else {
            const BufRsrc ro(o + tok0 * stride + sg.h * SD, rows_extent(n, stride * 4, SD * 4));
#pragma unroll
            for (int it = 0; it < 4; ++it)
                ro.store_b128(__builtin_bit_cast(u32x4, ot[it]),
                              static_cast<uint32_t>(((it * 16 + ap.col) * stride + col + ap.row0) * 4));
        }
        // the next chunk's rows go to LDS between the two halves of the
        // update's MFMAs, the gate scan after them
        seg_update_mfma_half(S, up, 0);
        seg_stage_rows<true, NORM>(buf[(c + 1) & 1], pf);
        seg_update_mfma_half(S, up, 1);
        seg_stage_gates<true, NORM>(buf[(c + 1) & 1], pf, lsig);
        if constexpr (NORM) {
            // z_in of the next chunk = z_in + this chunk's sums of phi(k)
            f32x4 zc = {0.f, 0.f, 0.f, 0.f};
            seg_z_update(zc, bb, wave);
            const int zr = opaque(wave * 16 + ap.row0);
            if (ap.col == 0)
                *reinterpret_cast<f32x4*>(&zb[(c + 1) & 1][zr]) = *reinterpret_cast<const f32x4*>(&zb[c & 1][zr]) + zc;
        }
        seg_fetch<true, !NORM>(pf, q, k, v, alpha, tok(c + 2), rows(c + 2), sg.h, H);
        // checkpoint: this wave's columns of the state after chunk c (the
        // segment starts sg.g * lseg tokens into its sequence)
        const int cs = CKPT && n == SC ? ckpt_slot(ck, sg.b, sg.g * lseg + (c + 1) * SC, n_slots) : -1;
        if (CKPT && cs >= 0) {
            float* Sc = pool + (static_cast<long>(cs) * H + sg.h) * SD * SD +
                        opaque(2 * ap.row0 * SD + col + ap.col);
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
                for (int r = 0; r < 4; ++r) Sc[(srow(mt, 0) + r) * SD] = S[mt][r] * bb.sig;
            }
        }
        lds_barrier();
    }
    if (nch > 0) flush_o(nch - 1);

    if (sg.g == sg.nseg - 1) {
        const float sgl = nch > 0 ? buf[(nch - 1) & 1].sig : 1.f;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) Sg[(srow(mt, ap.row0) + r) * SD + col + ap.col] = S[mt][r] * sgl;
        }
        if constexpr (NORM) {
            // z after the last chunk (the loop ends with a barrier)
            if (tid < SD) zpool[zoff + tid] = zb[nch & 1][tid];
        }
    }
}

// The output pass for batches of short prompts (plain GLA, no checkpoints):
// a block takes `items` work items, heads h0 .. h0 + items - 1 of one
// segment (items divides H).  Their chunks form one stream, item after
// item, so the next item's first loads are in flight while the current
// item's last chunk runs, and a batch of short prompts does not pay a
// block's start-up and drain per (sequence, head).  Between items the
// final state of one goes out and the entry state of the next comes in;
// entry states of split sequences are folded from the workspace there.
template <class TO, bool ZERO>
__global__ void __launch_bounds__(ST)
gla_seg_out_multi(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                  const uint16_t* __restrict__ v, const float* __restrict__ alpha, const int32_t* __restrict__ cu,
                  int n_seqs, int n_tokens, int H, float* __restrict__ pool, int n_slots,
                  const int32_t* __restrict__ slot_idx, int lseg,
                  const float* __restrict__ wstate, const float* __restrict__ wlam, int items,
                  typename TO::T* __restrict__ o) {
    __shared__ int sh[SW + 4];
    SegGeom sg;
    if (!seg_geometry(sg, cu, n_seqs, n_tokens, H, lseg, slot_idx, n_slots, sh, blockIdx.x * items,
                      gridDim.x * items / H))
        return;
    __shared__ QKVBuf buf[2];
    __shared__ uint16_t pbuf[2][SC][SP];           // P = (Q K^T) .* D, hi and lo planes
    // bf16 outputs of the previous chunk, stored to HBM as whole rows
    __shared__ uint16_t obuf[TO::bytes == 2 ? SC : 1][LO];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const AccPos ap;
    const int col = wave * 16;
    const long stride = static_cast<long>(H) * SD;
    const bool last_seg = sg.g == sg.nseg - 1;

    const int nch = (sg.t1 - sg.t0 + SC - 1) / SC;
    auto rows = [&](int c) { return c < nch ? min(SC, sg.t1 - sg.t0 - c * SC) : 0; };
    auto tok = [&](int c) { return static_cast<long>(sg.t0) + static_cast<long>(c < nch ? c : 0) * SC; };
    // the loads of chunk c of item it (nothing past the last item)
    SegPrefetch<true> pf;
    auto fetch = [&](int c, int it) {
        seg_fetch<true, true>(pf, q, k, v, alpha, tok(c), it < items ? rows(c) : 0, sg.h + min(it, items - 1), H);
    };
    // the position `ahead` chunks after chunk c of item it (past the last
    // item when the segment has no chunks: the stream is empty)
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
    fetch(0, 0);     // in flight during the fold

    // ---- entry state of item it
    f32x4 S[8];
    // a pool state through a buffer resource: the lane's offset in one
    // register, each of its 32 rows a scalar offset (no per-row addresses)
    const uint32_t lane_off = static_cast<uint32_t>((2 * ap.row0 * SD + col + ap.col) * 4);
    auto pool_state = [&](int it) {
        return BufRsrc(pool + (static_cast<long>(sg.slot) * H + sg.h + it) * SD * SD, SD * SD * 4);
    };
    auto entry = [&](int it) {
        if (sg.nseg <= 1 || (ZERO && sg.g == 0)) {
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) S[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            if constexpr (!ZERO) {
                const BufRsrc rs = pool_state(it);
#pragma unroll
                for (int mt = 0; mt < 8; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) S[mt][r] = rs.loadf(lane_off, (srow(mt, 0) + r) * SD * 4);
            }
        } else {
            // first segment: the copy of the initial state in the last
            // segment's slot; later ones: slot 0 holds S_in(1)
            const SlotReader s0(wstate, sg.ws_first + it + (sg.g == 0 ? static_cast<long>(sg.nseg - 1) * H : 0L));
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) S[mt] = s0.tile(mt);
            for (int j = 1; j < sg.g; ++j) {
                const long sj = sg.ws_first + it + static_cast<long>(j) * H;
                const float dcy = hw_exp2(wlam[sj]);
                const SlotReader dS(wstate, sj);
#pragma unroll
                for (int mt = 0; mt < 8; ++mt) S[mt] = dcy * S[mt] + dS.tile(mt);
            }
        }
    };
    // P tiles above the diagonal that P V still reads (rows 0-15 x keys 16-31,
    // rows 32-47 x keys 48-63) stay zero; the others are rewritten each chunk.
    auto zero_p_upper = [&]() {
        for (int idx = tid; idx < 2 * 256; idx += ST) {
            const int t = idx >> 8, e = idx & 255;
            const int row = (t ? 32 : 0) + (e >> 4), cx = p_col(t ? 3 : 1, (e >> 2) & 3) + (e & 3);
            pbuf[0][row][cx] = 0;
            pbuf[1][row][cx] = 0;
        }
    };
    // the final state of item it (this wave's columns), last segment only
    auto final_state = [&](int it) {
        const BufRsrc rs = pool_state(it);
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) rs.storef(S[mt][r], lane_off, (srow(mt, 0) + r) * SD * 4);
    };
    // Between item it and item it + 1 (all threads, after a barrier that
    // ends every read of the free chunk buffer fb and of pbuf; ends with the
    // P tiles that must stay zero zeroed again, which the next chunk's P V
    // reads after its own barrier).  The final state of item it (last
    // segment only) goes through LDS into rows (rows 0-95 over fb, 96-127
    // over pbuf, kRow floats a row) and out as whole 512-byte rows, 16 bytes
    // a lane, instead of 32 scattered 4-byte stores per lane.  The next
    // item's entry state is loaded into S before those stores are issued,
    // and S is used (an empty asm) after them: the load-counter wait for it
    // then leaves the stores in flight, and none is needed at the top of
    // the chunk loop, where it would wait for them.  With ZERO (zero_init)
    // a one-segment entry state is zeros: no loads, no wait.
    constexpr int kRow = SD + 4;
    static_assert(96 * kRow * 4 <= sizeof(QKVBuf) && 32 * kRow * 4 <= sizeof(pbuf), "state staging");
    static_assert(offsetof(QKVBuf, sig) >= 96 * kRow * 4, "the staged state leaves sig in place");
    auto next_item = [&](int it, QKVBuf& fb) {
        float* lo = reinterpret_cast<float*>(&fb);
        float* hi = reinterpret_cast<float*>(&pbuf[0][0][0]);
        // lane offsets recomputed here (opaque), not held across the chunk loop
        if (last_seg) {
            const float sgl = fb.sig;          // S = sigma Shat after the item's last chunk
            const int wo = opaque(2 * ap.row0 * kRow + col + ap.col);
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) {
                // state rows srow(mt, .): tiles 0-5 hold rows 0-95, tiles 6 and 7 rows 96-127
                float* base = (mt < 6 ? lo + srow(mt, 0) * kRow : hi + (srow(mt, 0) - 96) * kRow) + wo;
#pragma unroll
                for (int r = 0; r < 4; ++r) base[r * kRow] = S[mt][r] * sgl;
            }
        }
        if (it + 1 < items) entry(it + 1);
        lds_barrier();
        {
            // issued on every path (an empty range when this is not the
            // last segment), for the same reason as the output flush
            const BufRsrc rs(pool + (static_cast<long>(sg.slot) * H + sg.h + it) * SD * SD,
                             last_seg ? SD * SD * 4 : 0u);
            const int t = opaque(tid);
            const int ro = (t >> 5) * kRow + (t & 31) * 4;
            const uint32_t go = static_cast<uint32_t>(((t >> 5) * SD + (t & 31) * 4) * 4);
#pragma unroll
            for (int u = 0; u < SD / (ST / 32); ++u) {
                const float* src = (u < 6 ? lo + u * 16 * kRow : hi + (u - 6) * 16 * kRow) + ro;
                rs.store_b128(*reinterpret_cast<const u32x4*>(src), go, static_cast<uint32_t>(u * 16 * SD * 4));
            }
        }
        if constexpr (!ZERO) {
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
                asm volatile("" ::"v"(S[mt][0]), "v"(S[mt][1]), "v"(S[mt][2]), "v"(S[mt][3]));
        }
        lds_barrier();
        zero_p_upper();
    };
    entry(0);
    zero_p_upper();
    float lsig = 0.f;                              // log2 sigma on wave 0
    seg_stage<true, false>(buf[0], pf, lsig);
    {
        int c1, i1;
        step(0, 0, 1, c1, i1);
        fetch(c1, i1);
    }
    lds_barrier();

    // P tile t of (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) (3,1) (3,2) (3,3):
    // operand reads, then the MFMAs and the decay / mask / split epilogue
    auto tile_it = [](int t) { return t < 1 ? 0 : (t < 3 ? 1 : (t < 6 ? 2 : 3)); };
    auto p_load = [&](const QKVBuf& bb, int t, bf16x8 (&pa)[4], bf16x8 (&pb)[4]) {
        const int it = tile_it(t), jt = t - it * (it + 1) / 2;
#pragma unroll
        for (int ks = 0; ks < SD / 32; ++ks) {
            pa[ks] = frag_kc(&bb.k[0][0], LK, jt * 16, 32 * ks);
            pb[ks] = frag_kc(&bb.q[0][0], LQ, it * 16, 32 * ks);
        }
    };
    auto p_finish = [&](const QKVBuf& bb, int t, const bf16x8 (&pa)[4], const bf16x8 (&pb)[4]) {
        const int it = tile_it(t), jt = t - it * (it + 1) / 2;
        f32x4 pt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < SD / 32; ++ks) pt = mfma_bf16(pa[ks], pb[ks], pt);
        const int i = it * 16 + ap.col;
        const float gi = bb.g2[i];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = jt * 16 + ap.row0 + r;
            pt[r] = (j <= i) ? pt[r] * hw_exp2(gi - bb.g2[j]) : 0.f;
        }
        const int pc = p_col(jt, ap.row0 >> 2);
        Op<false>::store4(&pbuf[0][i][pc], &pbuf[1][i][pc], pt);
    };

    // bf16 outputs of chunk cc of item it: LDS -> HBM, 16 lanes per 256-byte
    // row.  Issued every chunk, before the first with nothing to write (an
    // empty range: no memory traffic), so that every path through the loop
    // has the same vector-memory operations and the load-counter waits for
    // the prefetched rows can leave younger stores in flight.
    auto flush_o = [&](int cc, int it, bool live) {
        if constexpr (TO::bytes == 2) {
            const BufRsrc ro(o + tok(cc) * stride + (sg.h + it) * SD,
                             live ? rows_extent(rows(cc), stride * 2, SD * 2) : 0u);
#pragma unroll
            for (int u = 0; u < SC * SD / 8 / ST; ++u) {
                const int x = tid + u * ST, row = x / (SD / 8), vc = (x % (SD / 8)) * 8;
                ro.store_b128(*reinterpret_cast<const u32x4*>(&obuf[row][vc]),
                              static_cast<uint32_t>((row * stride + vc) * 2));
            }
        }
    };

    const int total = items * nch;
    int c = 0, item = 0;             // chunk and item of stream position vc
    int pc = 0, pitem = 0;           // those of the position before
    for (int vc = 0; vc < total; ++vc) {
        const QKVBuf& bb = buf[vc & 1];
        const int n = rows(c);
        const long tok0 = tok(c);
        const int hk = sg.h + item;
        flush_o(pc, pitem, vc > 0);

        // ---- phase 1: P tiles (split over the waves) -> LDS, and
        // O^T = S^T Q^T for this wave's columns (the state accumulator tiles
        // serve as the A operand directly: rows = columns of S)
        bf16x8 pa[4], pb[4], qf[4][4];
        p_load(bb, wave, pa, pb);
#pragma unroll
        for (int s = 0; s < SD / 32; ++s)
#pragma unroll
            for (int it = 0; it < 4; ++it) qf[s][it] = frag_kc(&bb.q[0][0], LQ, it * 16, 32 * s);
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 sh8[4], sl8[4];
#pragma unroll
        for (int s = 0; s < SD / 32; ++s) {
            s16x4 h0, l0, h1, l1;
            split4(S[2 * s], h0, l0);
            split4(S[2 * s + 1], h1, l1);
            sh8[s] = cat8(h0, h1);
            sl8[s] = cat8(l0, l1);
        }
        f32x4 ot[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) ot[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < SD / 32; ++s)
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                ot[it] = mfma_bf16(sh8[s], qf[s][it], ot[it]);
                ot[it] = mfma_bf16(sl8[s], qf[s][it], ot[it]);
            }
        p_finish(bb, wave, pa, pb);
        if (wave + SW < 10) {
            p_load(bb, wave + SW, pa, pb);
            p_finish(bb, wave + SW, pa, pb);
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) ot[it] *= bb.eg[it * 16 + ap.col];
        lds_barrier();

        // ---- phase 2: + V^T P^T (split k order on both operands), outputs,
        // state update, next chunk
        bf16x8 vf[2], pp[6][2];
        load_vt(vf, bb, col);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            pp[it][0] = frag_kc(&pbuf[0][0][0], SP, it * 16, 0);
            pp[it][1] = frag_kc(&pbuf[1][0][0], SP, it * 16, 0);
        }
#pragma unroll
        for (int it = 2; it < 4; ++it) {
            pp[it + 2][0] = frag_kc(&pbuf[0][0][0], SP, it * 16, 32);
            pp[it + 2][1] = frag_kc(&pbuf[1][0][0], SP, it * 16, 32);
        }
        __builtin_amdgcn_sched_barrier(0);
        // the state update's operand reads and VALU work go ahead of the
        // P V MFMAs, which do not depend on them, so they can overlap
        SegUpd up;
        seg_update_prep<true, false>(up, S, bb, vf);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            ot[it] = mfma_bf16(vf[0], pp[it][0], ot[it]);
            ot[it] = mfma_bf16(vf[0], pp[it][1], ot[it]);
        }
#pragma unroll
        for (int it = 2; it < 4; ++it) {
            ot[it] = mfma_bf16(vf[1], pp[it + 2][0], ot[it]);
            ot[it] = mfma_bf16(vf[1], pp[it + 2][1], ot[it]);
        }
        // lane: token it*16 + (lane % 16), columns col + 4 (lane / 16) .. +3
        if constexpr (TO::bytes == 2) {
#pragma unroll
            for (int it = 0; it < 4; ++it)
                *reinterpret_cast<u32x2*>(&obuf[it * 16 + ap.col][col + ap.row0]) =
                    u32x2{pack_bf16x2(ot[it][0], ot[it][1]), pack_bf16x2(ot[it][2], ot[it][3])};
        } else {
            const BufRsrc ro(o + tok0 * stride + hk * SD, rows_extent(n, stride * 4, SD * 4));
#pragma unroll
            for (int it = 0; it < 4; ++it)
                ro.store_b128(__builtin_bit_cast(u32x4, ot[it]),
                              static_cast<uint32_t>(((it * 16 + ap.col) * stride + col + ap.row0) * 4));
        }
        // the next chunk's rows go to LDS between the two halves of the
        // update's MFMAs, the gate scan after them
        seg_update_mfma_half(S, up, 0);
        seg_stage_rows<true, false>(buf[(vc + 1) & 1], pf);
        seg_update_mfma_half(S, up, 1);
        const bool item_end = c == nch - 1;
        seg_stage_gates<true, false>(buf[(vc + 1) & 1], pf, lsig, item_end);
        {
            int c2, i2;
            step(c, item, 2, c2, i2);
            fetch(c2, i2);
        }
        lds_barrier();
        if (item_end) next_item(item, buf[vc & 1]);
        pc = c;
        pitem = item;
        if (item_end) {
            c = 0;
            ++item;
        } else {
            ++c;
        }
    }
    if (nch > 0) flush_o(pc, pitem, true);
    if (nch == 0) {
        // empty sequence: every item's state goes back as it came in (after
        // the loop, which does not run: placed before it, this code made
        // the loop's register allocation spill)
        for (int it = 0; it < items; ++it) {
            if (it > 0) entry(it);
            if (last_seg) final_state(it);
        }
    }
}

// Every sequence gets at least one segment (an empty one still writes its
// state back).  Segment length: whole chunks, at least 4 of them, about
// kSegBlocks workgroups in total.
int seg_len(int n_tokens, int n_heads) {
    const long target = n_heads >= kSegBlocks ? 1 : kSegBlocks / n_heads;
    long L = (n_tokens + target - 1) / target;
    L = ((L + SC - 1) / SC) * SC;
    return static_cast<int>(L < 4 * SC ? 4 * SC : L);
}

__host__ __device__ constexpr size_t align256s(size_t x) { return (x + 255) & ~size_t(255); }

long seg_count_bound(int n_seqs, int n_tokens, int lseg) { return n_tokens / lseg + n_seqs; }

// Work items (heads of one segment) per output-pass block: 1 unless the
// batch is short sequences (at most kShortChunks chunks on average); then
// the largest divisor of H up to kMaxItems that still launches at least
// kSegBlocks blocks, one per compute unit.
int seg_items(int n_seqs, int n_tokens, int n_heads, long maxseg) {
    if (n_seqs <= 0 || static_cast<long>(n_tokens) > static_cast<long>(n_seqs) * kShortChunks * SC) return 1;
    int best = 1;
    for (int k = 2; k <= kMaxItems && k <= n_heads; ++k)
        if (n_heads % k == 0 && maxseg * n_heads / k >= kSegBlocks) best = k;
    return best;
}

}  // namespace

bool gla_seg_supported(const ChunkArgs& a) {
    return a.in_bf16 && a.dk == SD && a.dv == SD && a.chunk == SC;
}

size_t gla_seg_workspace(int n_seqs, int n_tokens, int n_heads) {
    // per (segment, head): the log2 decay total, a 64 KiB state slot and (for
    // normalised linear attention) a 512-byte normaliser slot
    const long maxseg = seg_count_bound(n_seqs, n_tokens, seg_len(n_tokens, n_heads));
    return align256s(sizeof(float) * maxseg * n_heads) +
           static_cast<size_t>(maxseg) * n_heads * SD * SD * sizeof(float) +
           static_cast<size_t>(maxseg) * n_heads * SD * sizeof(float);
}

namespace {

template <bool NORM>
hipError_t launch_seg(const ChunkArgs& a, hipStream_t s) {
    const int lseg = seg_len(a.n_tokens, a.n_heads);
    const long maxseg = seg_count_bound(a.n_seqs, a.n_tokens, lseg);
    char* ws = static_cast<char*>(a.workspace);
    float* wlam = reinterpret_cast<float*>(ws);
    float* wstate = reinterpret_cast<float*>(ws + align256s(sizeof(float) * maxseg * a.n_heads));
    float* wz = wstate + static_cast<size_t>(maxseg) * a.n_heads * SD * SD;
    const float* alpha = NORM ? nullptr : a.alpha;
    const dim3 grid(static_cast<unsigned>(maxseg * a.n_heads));
    // A sequence of k >= 2 segments is longer than (k - 1) * lseg tokens and
    // k <= 2 (k - 1), so the segments of split sequences number at most
    // 2 * (n_tokens / lseg); pass 1 launches no more blocks than that.
    const long nsplit = std::min(maxseg, 2L * (a.n_tokens / lseg));
    const Ckpt ck{a.ckpt_slots, a.ckpt_interval, a.ckpt_stride};
    // several heads per block for batches of short prompts (plain GLA; the
    // checkpoint and normalised variants keep one)
    const int items = NORM || ck.slots ? 1 : seg_items(a.n_seqs, a.n_tokens, a.n_heads, maxseg);
    // the scan of the entry states pays its launch where sequences have
    // kScanMinSegs segments or more on average (never with several heads
    // per block, which fold: their batches are of short prompts)
    const int scanned =
        items == 1 && nsplit > 0 && a.n_tokens / lseg >= static_cast<long>(kScanMinSegs) * a.n_seqs;
    if (nsplit > 0) {
        hipLaunchKernelGGL(gla_seg_state<NORM>, dim3(static_cast<unsigned>(nsplit * a.n_heads)), dim3(ST), 0,
                           s, static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v), alpha,
                           a.cu_seqlens, a.n_seqs, a.n_tokens, a.n_heads, a.pool, a.n_slots, a.slot_idx,
                           a.zero_init, lseg, wstate, wlam, a.zpool, wz, static_cast<int>(maxseg));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (scanned) {
        hipLaunchKernelGGL(gla_seg_scan<NORM>, dim3(static_cast<unsigned>(nsplit * a.n_heads), kScanCols), dim3(ST),
                           0, s, a.cu_seqlens, a.n_seqs, a.n_tokens, a.n_heads, lseg, a.slot_idx, a.n_slots,
                           static_cast<int>(maxseg), wstate, wlam, wz);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if constexpr (!NORM) {
        if (items > 1) {
            auto multi = [&](auto kern, auto* o) {
                hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(maxseg * a.n_heads / items)), dim3(ST), 0, s,
                                   static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                                   static_cast<const uint16_t*>(a.v), alpha, a.cu_seqlens, a.n_seqs, a.n_tokens,
                                   a.n_heads, a.pool, a.n_slots, a.slot_idx, lseg, wstate, wlam, items, o);
            };
            if (a.zero_init) {
                if (a.out_bf16) multi(gla_seg_out_multi<BF16, true>, static_cast<uint16_t*>(a.o));
                else multi(gla_seg_out_multi<F32, true>, static_cast<float*>(a.o));
            } else {
                if (a.out_bf16) multi(gla_seg_out_multi<BF16, false>, static_cast<uint16_t*>(a.o));
                else multi(gla_seg_out_multi<F32, false>, static_cast<float*>(a.o));
            }
            return hipGetLastError();
        }
    }
    auto out_pass = [&](auto kern, auto* o) {
        hipLaunchKernelGGL(kern, grid, dim3(ST), 0, s, static_cast<const uint16_t*>(a.q),
                           static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v), alpha,
                           a.cu_seqlens, a.n_seqs, a.n_tokens, a.n_heads, a.pool, a.n_slots, a.slot_idx,
                           a.zero_init, lseg, wstate, wlam, scanned, ck, a.zpool, wz, a.eps, o);
    };
    // the checkpoint stores are compiled in only where they are asked for
    if constexpr (!NORM) {
        if (ck.slots) {
            if (a.out_bf16) out_pass(gla_seg_out<BF16, true, false>, static_cast<uint16_t*>(a.o));
            else out_pass(gla_seg_out<F32, true, false>, static_cast<float*>(a.o));
            return hipGetLastError();
        }
    }
    if (a.out_bf16) out_pass(gla_seg_out<BF16, false, NORM>, static_cast<uint16_t*>(a.o));
    else out_pass(gla_seg_out<F32, false, NORM>, static_cast<float*>(a.o));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gla_seg(const ChunkArgs& a, hipStream_t s) { return launch_seg<false>(a, s); }
hipError_t launch_lin_attn_seg(const ChunkArgs& a, hipStream_t s) { return launch_seg<true>(a, s); }

}  // namespace gla
