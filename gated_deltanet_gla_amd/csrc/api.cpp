// Host side of the C ABI declared in include/gla.h: argument validation
// (nothing is enqueued when it fails) and dispatch to the kernel launchers.
#include "gla.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <limits>
#include <mutex>

#include "launch.h"

namespace {

bool is_dim(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool is_chunk(int32_t c) { return c == 16 || c == 32 || c == 64; }
bool is_dtype(int d) { return d == GLA_F32 || d == GLA_BF16; }

// Largest grid the launchers build is (rows of work) x heads x (d_v tiles);
// keep every product comfortably inside int32.
constexpr long kMaxWork = 1L << 26;

int hip_status(hipError_t e) { return e == hipSuccess ? GLA_OK : GLA_EHIP; }

bool is_eps(float eps) { return eps >= 0.f && eps <= 3.0e38f; }

// need_alpha = false for the ungated operation (normalised linear attention).
int check_chunk(const void* q, const void* k, const void* v, const float* alpha, bool need_alpha,
                const float* beta, bool need_beta, const int32_t* cu_seqlens, int32_t n_seqs,
                int32_t n_tokens, int32_t n_heads, int32_t dk, int32_t dv, int32_t chunk,
                int in_dtype, int out_dtype, const float* pool, int32_t n_slots,
                const int32_t* slot_idx, uint32_t flags, const void* o) {
    if (n_seqs < 0 || n_tokens < 0 || n_heads < 1) return GLA_ESHAPE;
    if (!is_dim(dk) || !is_dim(dv)) return GLA_ESHAPE;
    if (!is_chunk(chunk)) return GLA_ECHUNK;
    if (!is_dtype(in_dtype) || !is_dtype(out_dtype)) return GLA_EDTYPE;
    if (flags & ~static_cast<uint32_t>(GLA_ZERO_INIT)) return GLA_ESHAPE;
    if (static_cast<long>(n_seqs) * n_heads > kMaxWork) return GLA_ESHAPE;
    if (static_cast<long>(n_tokens) * n_heads > std::numeric_limits<int32_t>::max() / 128)
        return GLA_ESHAPE;
    if (n_seqs > 0) {
        if (n_slots < 1) return GLA_ESHAPE;
        if (!cu_seqlens || !pool || !slot_idx) return GLA_EPTR;
    }
    if (n_tokens > 0) {
        if (n_seqs < 1) return GLA_ESHAPE;
        if (!q || !k || !v || !o) return GLA_EPTR;
        if ((need_alpha && !alpha) || (need_beta && !beta)) return GLA_EPTR;
    }
    return GLA_OK;
}

// Checkpoint arguments: an interval that is a positive multiple of the
// chunk, a non-negative stride, and a slot table whenever the stride is not 0.
int check_ckpt(int32_t n_seqs, int32_t chunk, int32_t interval, const int32_t* slots,
               int32_t stride) {
    if (stride < 0) return GLA_ESHAPE;
    if (stride == 0) return GLA_OK;
    if (!is_chunk(chunk)) return GLA_ECHUNK;
    if (interval < chunk || interval % chunk != 0) return GLA_ECHUNK;
    if (static_cast<long>(n_seqs) * stride > kMaxWork) return GLA_ESHAPE;
    if (n_seqs > 0 && !slots) return GLA_EPTR;
    return GLA_OK;
}

int check_decode(const void* q, const void* k, const void* v, const float* alpha,
                 bool need_alpha, const float* beta, bool need_beta, int32_t n_req, int32_t n_heads, int32_t dk,
                 int32_t dv, int in_dtype, int out_dtype, const float* pool, int32_t n_slots,
                 const int32_t* slot_idx, const void* o) {
    if (n_req < 0 || n_heads < 1) return GLA_ESHAPE;
    if (!is_dim(dk) || !is_dim(dv)) return GLA_ESHAPE;
    if (!is_dtype(in_dtype) || !is_dtype(out_dtype)) return GLA_EDTYPE;
    if (static_cast<long>(n_req) * n_heads > kMaxWork) return GLA_ESHAPE;
    if (n_req == 0) return GLA_OK;
    if (n_slots < 1) return GLA_ESHAPE;
    if (!q || !k || !v || !pool || !slot_idx || !o) return GLA_EPTR;
    if ((need_alpha && !alpha) || (need_beta && !beta)) return GLA_EPTR;
    return GLA_OK;
}

// Scratch of gla_chunk_fwd_noalloc: a fixed array in each GPU's memory, so
// that entry point allocates nothing.  In host code the name `scratch` is
// only a stand-in for the symbol; its device address (one per GPU) comes
// from hipGetSymbolAddress and is what the kernels receive.
static __device__ __align__(256) unsigned char scratch[GLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_init;

// The scratch array's address on the current device, looked up on the
// first call made with that device current and kept.
int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GLA_EHIP;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_init);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
                (void)hipGetLastError();     // leave no sticky error for the caller's next call
                return GLA_EHIP;
            }
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return GLA_OK;
}

}  // namespace

extern "C" {

const char* gla_version(void) { return "0.2.0"; }

const char* gla_status_string(int status) {
    switch (status) {
        case GLA_OK: return "ok";
        case GLA_EPTR: return "a required pointer is NULL";
        case GLA_ESHAPE: return "a size is negative, unsupported or inconsistent";
        case GLA_EDTYPE: return "unsupported dtype";
        case GLA_ECHUNK: return "unsupported chunk size";
        case GLA_EWORKSPACE: return "workspace missing or too small";
        case GLA_EHIP: return "HIP launch failed";
        case GLA_ESCRATCH: return "the call needs more scratch than gla_chunk_fwd_noalloc's fixed array";
    }
    return "unknown status";
}

size_t gla_chunk_workspace_bytes(int32_t n_seqs, int32_t n_tokens, int32_t n_heads, int32_t dk,
                                 int32_t dv, int32_t chunk) {
    if (n_seqs < 0 || n_tokens < 0 || n_heads < 1 || !is_dim(dk) || !is_dim(dv) || !is_chunk(chunk))
        return 0;
    return gla::gla_chunk_workspace(n_seqs, n_tokens, n_heads, dk, dv, chunk);
}

size_t lin_attn_chunk_workspace_bytes(int32_t n_seqs, int32_t n_tokens, int32_t n_heads,
                                      int32_t dk, int32_t dv, int32_t chunk) {
    if (n_seqs < 0 || n_tokens < 0 || n_heads < 1 || !is_dim(dk) || !is_dim(dv) || !is_chunk(chunk))
        return 0;
    return gla::lin_attn_chunk_workspace(n_seqs, n_tokens, n_heads, dk, dv, chunk);
}

size_t gdn_chunk_workspace_bytes(int32_t n_seqs, int32_t n_tokens, int32_t n_heads, int32_t dk,
                                 int32_t dv, int32_t chunk) {
    if (n_seqs < 0 || n_tokens < 0 || n_heads < 1 || !is_dim(dk) || !is_dim(dv) || !is_chunk(chunk))
        return 0;
    return gla::gdn_chunk_workspace(n_seqs, n_tokens, n_heads, dk, dv, chunk);
}

int gla_chunk_fwd_ckpt(const void* q, const void* k, const void* v, const float* alpha,
                       const int32_t* cu_seqlens, int32_t n_seqs, int32_t n_tokens, int32_t n_heads,
                       int32_t dk, int32_t dv, int32_t chunk, gla_dtype in_dtype,
                       gla_dtype out_dtype, float* state_pool, int32_t n_slots,
                       const int32_t* slot_idx, uint32_t flags, int32_t ckpt_interval,
                       const int32_t* ckpt_slots, int32_t ckpt_stride, void* o, void* workspace,
                       size_t workspace_bytes, void* stream) {
    int st = check_ckpt(n_seqs, chunk, ckpt_interval, ckpt_slots, ckpt_stride);
    if (st != GLA_OK) return st;
    if (ckpt_stride == 0) ckpt_slots = nullptr;
    st = check_chunk(q, k, v, alpha, true, nullptr, false, cu_seqlens, n_seqs, n_tokens, n_heads, dk,
                         dv, chunk, in_dtype, out_dtype, state_pool, n_slots, slot_idx, flags, o);
    if (st != GLA_OK) return st;
    if (n_seqs == 0) return GLA_OK;
    const size_t need = gla::gla_chunk_workspace(n_seqs, n_tokens, n_heads, dk, dv, chunk);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return GLA_EWORKSPACE;
    gla::ChunkArgs a{q, k, v, alpha, nullptr, cu_seqlens, n_seqs, n_tokens, n_heads, dk, dv, chunk,
                     in_dtype == GLA_BF16, out_dtype == GLA_BF16, state_pool, n_slots, slot_idx,
                     (flags & GLA_ZERO_INIT) ? 1 : 0, o, workspace, workspace_bytes,
                     ckpt_slots, ckpt_interval, ckpt_stride};
    return hip_status(gla::launch_gla_chunk(a, static_cast<hipStream_t>(stream)));
}

int gdn_chunk_fwd_ckpt(const void* q, const void* k, const void* v, const float* alpha,
                       const float* beta, const int32_t* cu_seqlens, int32_t n_seqs,
                       int32_t n_tokens, int32_t n_heads, int32_t dk, int32_t dv, int32_t chunk,
                       gla_dtype in_dtype, gla_dtype out_dtype, float* state_pool, int32_t n_slots,
                       const int32_t* slot_idx, uint32_t flags, int32_t ckpt_interval,
                       const int32_t* ckpt_slots, int32_t ckpt_stride, void* o, void* workspace,
                       size_t workspace_bytes, void* stream) {
    int st = check_ckpt(n_seqs, chunk, ckpt_interval, ckpt_slots, ckpt_stride);
    if (st != GLA_OK) return st;
    if (ckpt_stride == 0) ckpt_slots = nullptr;
    st = check_chunk(q, k, v, alpha, true, beta, true, cu_seqlens, n_seqs, n_tokens, n_heads, dk, dv,
                         chunk, in_dtype, out_dtype, state_pool, n_slots, slot_idx, flags, o);
    if (st != GLA_OK) return st;
    if (n_seqs == 0) return GLA_OK;
    const size_t need = gla::gdn_chunk_workspace(n_seqs, n_tokens, n_heads, dk, dv, chunk);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return GLA_EWORKSPACE;
    gla::ChunkArgs a{q, k, v, alpha, beta, cu_seqlens, n_seqs, n_tokens, n_heads, dk, dv, chunk,
                     in_dtype == GLA_BF16, out_dtype == GLA_BF16, state_pool, n_slots, slot_idx,
                     (flags & GLA_ZERO_INIT) ? 1 : 0, o, workspace, workspace_bytes,
                     ckpt_slots, ckpt_interval, ckpt_stride};
    return hip_status(gla::launch_gdn_chunk(a, static_cast<hipStream_t>(stream)));
}

int gla_chunk_fwd(const void* q, const void* k, const void* v, const float* alpha,
                  const int32_t* cu_seqlens, int32_t n_seqs, int32_t n_tokens, int32_t n_heads,
                  int32_t dk, int32_t dv, int32_t chunk, gla_dtype in_dtype, gla_dtype out_dtype,
                  float* state_pool, int32_t n_slots, const int32_t* slot_idx, uint32_t flags,
                  void* o, void* workspace, size_t workspace_bytes, void* stream) {
    return gla_chunk_fwd_ckpt(q, k, v, alpha, cu_seqlens, n_seqs, n_tokens, n_heads, dk, dv, chunk,
                              in_dtype, out_dtype, state_pool, n_slots, slot_idx, flags, chunk,
                              nullptr, 0, o, workspace, workspace_bytes, stream);
}

int gla_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* alpha,
                          const int32_t* cu_seqlens, int32_t n_seqs, int32_t n_tokens,
                          int32_t n_heads, int32_t dk, int32_t dv, int32_t chunk,
                          gla_dtype in_dtype, gla_dtype out_dtype, float* state_pool,
                          int32_t n_slots, const int32_t* slot_idx, uint32_t flags, void* o,
                          void* stream) {
    int st = check_chunk(q, k, v, alpha, true, nullptr, false, cu_seqlens, n_seqs, n_tokens, n_heads,
                         dk, dv, chunk, in_dtype, out_dtype, state_pool, n_slots, slot_idx, flags, o);
    if (st != GLA_OK) return st;
    if (n_seqs == 0) return GLA_OK;
    const size_t need = gla::gla_chunk_workspace(n_seqs, n_tokens, n_heads, dk, dv, chunk);
    if (need > GLA_NOALLOC_SCRATCH_BYTES) return GLA_ESCRATCH;
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != GLA_OK) return st;
    return gla_chunk_fwd(q, k, v, alpha, cu_seqlens, n_seqs, n_tokens, n_heads, dk, dv, chunk, in_dtype,
                         out_dtype, state_pool, n_slots, slot_idx, flags, o, ws,
                         GLA_NOALLOC_SCRATCH_BYTES, stream);
}

int gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* alpha,
                  const float* beta, const int32_t* cu_seqlens, int32_t n_seqs, int32_t n_tokens,
                  int32_t n_heads, int32_t dk, int32_t dv, int32_t chunk, gla_dtype in_dtype,
                  gla_dtype out_dtype, float* state_pool, int32_t n_slots, const int32_t* slot_idx,
                  uint32_t flags, void* o, void* workspace, size_t workspace_bytes, void* stream) {
    return gdn_chunk_fwd_ckpt(q, k, v, alpha, beta, cu_seqlens, n_seqs, n_tokens, n_heads, dk, dv,
                              chunk, in_dtype, out_dtype, state_pool, n_slots, slot_idx, flags,
                              chunk, nullptr, 0, o, workspace, workspace_bytes, stream);
}

int gdn_chunk_prep(const void* q, const void* k, const float* alpha, const float* beta,
                   const int32_t* cu_seqlens, int32_t n_seqs, int32_t n_tokens, int32_t n_heads,
                   int32_t dk, int32_t dv, int32_t chunk, gla_dtype in_dtype, void* workspace,
                   size_t workspace_bytes, void* stream) {
    if (n_seqs < 0 || n_tokens < 0 || n_heads < 1) return GLA_ESHAPE;
    if (!is_dim(dk) || !is_dim(dv)) return GLA_ESHAPE;
    if (!is_chunk(chunk)) return GLA_ECHUNK;
    if (!is_dtype(in_dtype)) return GLA_EDTYPE;
    if (static_cast<long>(n_seqs) * n_heads > kMaxWork) return GLA_ESHAPE;
    if (static_cast<long>(n_tokens) * n_heads > std::numeric_limits<int32_t>::max() / 128)
        return GLA_ESHAPE;
    if (n_tokens > 0 && n_seqs < 1) return GLA_ESHAPE;
    if (n_seqs == 0) return GLA_OK;
    if (!cu_seqlens) return GLA_EPTR;
    if (n_tokens > 0 && (!q || !k || !alpha || !beta)) return GLA_EPTR;
    const size_t need = gla::gdn_chunk_workspace(n_seqs, n_tokens, n_heads, dk, dv, chunk);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return GLA_EWORKSPACE;
    gla::ChunkArgs a{q, k, nullptr, alpha, beta, cu_seqlens, n_seqs, n_tokens, n_heads, dk, dv,
                     chunk, in_dtype == GLA_BF16, 0, nullptr, 0, nullptr, 0, nullptr, workspace,
                     workspace_bytes, nullptr, chunk, 0, nullptr, 0.f, 1};
    return hip_status(gla::launch_gdn_chunk(a, static_cast<hipStream_t>(stream)));
}

int gdn_chunk_run(const void* q, const void* k, const void* v, const float* alpha,
                  const float* beta, const int32_t* cu_seqlens, int32_t n_seqs, int32_t n_tokens,
                  int32_t n_heads, int32_t dk, int32_t dv, int32_t chunk, gla_dtype in_dtype,
                  gla_dtype out_dtype, float* state_pool, int32_t n_slots, const int32_t* slot_idx,
                  uint32_t flags, void* o, void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_chunk(q, k, v, alpha, true, beta, true, cu_seqlens, n_seqs, n_tokens, n_heads,
                         dk, dv, chunk, in_dtype, out_dtype, state_pool, n_slots, slot_idx, flags, o);
    if (st != GLA_OK) return st;
    if (n_seqs == 0) return GLA_OK;
    const size_t need = gla::gdn_chunk_workspace(n_seqs, n_tokens, n_heads, dk, dv, chunk);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return GLA_EWORKSPACE;
    gla::ChunkArgs a{q, k, v, alpha, beta, cu_seqlens, n_seqs, n_tokens, n_heads, dk, dv, chunk,
                     in_dtype == GLA_BF16, out_dtype == GLA_BF16, state_pool, n_slots, slot_idx,
                     (flags & GLA_ZERO_INIT) ? 1 : 0, o, workspace, workspace_bytes, nullptr, chunk,
                     0, nullptr, 0.f, 2};
    return hip_status(gla::launch_gdn_chunk(a, static_cast<hipStream_t>(stream)));
}

int gla_decode_step(const void* q, const void* k, const void* v, const float* alpha, int32_t n_req,
                    int32_t n_heads, int32_t dk, int32_t dv, gla_dtype in_dtype,
                    gla_dtype out_dtype, float* state_pool, int32_t n_slots,
                    const int32_t* slot_idx, void* o, void* stream) {
    int st = check_decode(q, k, v, alpha, true, nullptr, false, n_req, n_heads, dk, dv, in_dtype,
                          out_dtype, state_pool, n_slots, slot_idx, o);
    if (st != GLA_OK || n_req == 0) return st;
    gla::DecodeArgs a{q, k, v, alpha, nullptr, n_req, n_heads, dk, dv, in_dtype == GLA_BF16,
                      out_dtype == GLA_BF16, state_pool, n_slots, slot_idx, o, 1, nullptr};
    return hip_status(gla::launch_gla_decode(a, static_cast<hipStream_t>(stream)));
}

int gdn_decode_step(const void* q, const void* k, const void* v, const float* alpha,
                    const float* beta, int32_t n_req, int32_t n_heads, int32_t dk, int32_t dv,
                    gla_dtype in_dtype, gla_dtype out_dtype, float* state_pool, int32_t n_slots,
                    const int32_t* slot_idx, void* o, void* stream) {
    int st = check_decode(q, k, v, alpha, true, beta, true, n_req, n_heads, dk, dv, in_dtype, out_dtype,
                          state_pool, n_slots, slot_idx, o);
    if (st != GLA_OK || n_req == 0) return st;
    gla::DecodeArgs a{q, k, v, alpha, beta, n_req, n_heads, dk, dv, in_dtype == GLA_BF16,
                      out_dtype == GLA_BF16, state_pool, n_slots, slot_idx, o, 1, nullptr};
    return hip_status(gla::launch_gdn_decode(a, static_cast<hipStream_t>(stream)));
}

int gla_decode_multi(const void* q, const void* k, const void* v, const float* alpha,
                     int32_t n_req, int32_t n_tok, int32_t n_heads, int32_t dk, int32_t dv,
                     gla_dtype in_dtype, gla_dtype out_dtype, float* state_pool, int32_t n_slots,
                     const int32_t* slot_idx, const int32_t* pos_slots, void* o, void* stream) {
    if (n_tok < 0 || (n_tok > 0 && n_req > 0 && !pos_slots)) return n_tok < 0 ? GLA_ESHAPE : GLA_EPTR;
    if (static_cast<long>(n_req) * n_tok * n_heads > kMaxWork) return GLA_ESHAPE;
    int st = check_decode(q, k, v, alpha, true, nullptr, false, n_req, n_heads, dk, dv, in_dtype,
                          out_dtype, state_pool, n_slots, slot_idx, o);
    if (st != GLA_OK || n_req == 0 || n_tok == 0) return st;
    gla::DecodeArgs a{q, k, v, alpha, nullptr, n_req, n_heads, dk, dv, in_dtype == GLA_BF16,
                      out_dtype == GLA_BF16, state_pool, n_slots, slot_idx, o, n_tok, pos_slots};
    return hip_status(gla::launch_gla_decode(a, static_cast<hipStream_t>(stream)));
}

int gdn_decode_multi(const void* q, const void* k, const void* v, const float* alpha,
                     const float* beta, int32_t n_req, int32_t n_tok, int32_t n_heads, int32_t dk,
                     int32_t dv, gla_dtype in_dtype, gla_dtype out_dtype, float* state_pool,
                     int32_t n_slots, const int32_t* slot_idx, const int32_t* pos_slots, void* o,
                     void* stream) {
    if (n_tok < 0 || (n_tok > 0 && n_req > 0 && !pos_slots)) return n_tok < 0 ? GLA_ESHAPE : GLA_EPTR;
    if (static_cast<long>(n_req) * n_tok * n_heads > kMaxWork) return GLA_ESHAPE;
    int st = check_decode(q, k, v, alpha, true, beta, true, n_req, n_heads, dk, dv, in_dtype, out_dtype,
                          state_pool, n_slots, slot_idx, o);
    if (st != GLA_OK || n_req == 0 || n_tok == 0) return st;
    gla::DecodeArgs a{q, k, v, alpha, beta, n_req, n_heads, dk, dv, in_dtype == GLA_BF16,
                      out_dtype == GLA_BF16, state_pool, n_slots, slot_idx, o, n_tok, pos_slots};
    return hip_status(gla::launch_gdn_decode(a, static_cast<hipStream_t>(stream)));
}

int gla_slot_copy(void* buf, size_t slot_bytes, int32_t n_slots, const int32_t* src_slots,
                  const int32_t* dst_slots, int32_t n_copy, void* stream) {
    if (n_copy < 0 || n_slots < 0 || slot_bytes == 0 || slot_bytes % 16 != 0) return GLA_ESHAPE;
    if (slot_bytes > (static_cast<size_t>(1) << 40)) return GLA_ESHAPE;
    if (n_copy == 0) return GLA_OK;
    if (n_slots < 1) return GLA_ESHAPE;
    if (!buf || !src_slots || !dst_slots) return GLA_EPTR;
    if (reinterpret_cast<uintptr_t>(buf) % 16 != 0) return GLA_EPTR;
    const long pieces = (static_cast<long>(slot_bytes / 16) + 1023) / 1024;
    if (static_cast<long>(n_copy) * pieces > kMaxWork) return GLA_ESHAPE;
    gla::CopyArgs a{buf, static_cast<long>(slot_bytes), n_slots, src_slots, dst_slots, n_copy};
    return hip_status(gla::launch_slot_copy(a, static_cast<hipStream_t>(stream)));
}

int gla_state_copy(float* state_pool, int32_t n_slots, int32_t n_heads, int32_t dk, int32_t dv,
                   const int32_t* src_slots, const int32_t* dst_slots, int32_t n_copy,
                   void* stream) {
    if (n_copy < 0 || n_heads < 1 || n_slots < 0 || !is_dim(dk) || !is_dim(dv)) return GLA_ESHAPE;
    return gla_slot_copy(state_pool, static_cast<size_t>(n_heads) * dk * dv * sizeof(float),
                         n_slots, src_slots, dst_slots, n_copy, stream);
}

int gla_hbm_probe(int32_t mode, float* state_pool, int32_t n_req, int32_t n_heads, int32_t dk,
                  int32_t dv, int32_t n_slots, const int32_t* slot_idx, void* sink, void* stream) {
    if (mode < 0 || mode > 15 || n_req < 0 || n_heads < 1 || n_slots < 0) return GLA_ESHAPE;
    if (dk != 128 || dv != 128) return GLA_ESHAPE;
    if (static_cast<long>(n_req) * n_heads > kMaxWork) return GLA_ESHAPE;
    if (n_req == 0) return GLA_OK;
    if (n_slots < 1) return GLA_ESHAPE;
    if (!state_pool || !slot_idx || !sink) return GLA_EPTR;
    return hip_status(gla::launch_hbm_probe(mode, state_pool, n_req, n_heads, n_slots, slot_idx, sink,
                                            static_cast<hipStream_t>(stream)));
}

int lin_attn_chunk_fwd(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                       int32_t n_seqs, int32_t n_tokens, int32_t n_heads, int32_t dk, int32_t dv,
                       int32_t chunk, gla_dtype in_dtype, gla_dtype out_dtype, float* state_pool,
                       float* norm_pool, int32_t n_slots, const int32_t* slot_idx, uint32_t flags,
                       float eps, void* o, void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_chunk(q, k, v, nullptr, false, nullptr, false, cu_seqlens, n_seqs, n_tokens, n_heads,
                         dk, dv, chunk, in_dtype, out_dtype, state_pool, n_slots, slot_idx, flags, o);
    if (st != GLA_OK) return st;
    if (!is_eps(eps)) return GLA_ESHAPE;
    if (n_seqs == 0) return GLA_OK;
    if (!norm_pool) return GLA_EPTR;
    const size_t need = gla::lin_attn_chunk_workspace(n_seqs, n_tokens, n_heads, dk, dv, chunk);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return GLA_EWORKSPACE;
    gla::ChunkArgs a{q, k, v, nullptr, nullptr, cu_seqlens, n_seqs, n_tokens, n_heads, dk, dv, chunk,
                     in_dtype == GLA_BF16, out_dtype == GLA_BF16, state_pool, n_slots, slot_idx,
                     (flags & GLA_ZERO_INIT) ? 1 : 0, o, workspace, workspace_bytes, nullptr, chunk, 0,
                     norm_pool, eps};
    return hip_status(gla::launch_lin_attn_chunk(a, static_cast<hipStream_t>(stream)));
}

int lin_attn_decode_step(const void* q, const void* k, const void* v, int32_t n_req,
                         int32_t n_heads, int32_t dk, int32_t dv, gla_dtype in_dtype,
                         gla_dtype out_dtype, float* state_pool, float* norm_pool, int32_t n_slots,
                         const int32_t* slot_idx, float eps, void* o, void* stream) {
    int st = check_decode(q, k, v, nullptr, false, nullptr, false, n_req, n_heads, dk, dv, in_dtype,
                          out_dtype, state_pool, n_slots, slot_idx, o);
    if (st != GLA_OK) return st;
    if (!is_eps(eps)) return GLA_ESHAPE;
    if (n_req == 0) return GLA_OK;
    if (!norm_pool) return GLA_EPTR;
    gla::LinDecodeArgs a{q, k, v, n_req, n_heads, dk, dv, in_dtype == GLA_BF16, out_dtype == GLA_BF16,
                         state_pool, norm_pool, n_slots, slot_idx, eps, o};
    return hip_status(gla::launch_lin_attn_decode(a, static_cast<hipStream_t>(stream)));
}

int causal_conv1d_fwd(const void* x, const float* w, const int32_t* cu_seqlens, int32_t n_seqs,
                      int32_t n_tokens, int32_t channels, int32_t width, void* conv_cache,
                      int32_t n_slots, const int32_t* slot_idx, uint32_t flags, void* y,
                      gla_dtype dtype, void* stream) {
    if (n_seqs < 0 || n_tokens < 0 || channels < 8 || (channels % 8) != 0) return GLA_ESHAPE;
    if (width < 2 || width > 4) return GLA_ESHAPE;
    if (!is_dtype(dtype)) return GLA_EDTYPE;
    if (flags & ~static_cast<uint32_t>(GLA_ZERO_INIT)) return GLA_ESHAPE;
    if (static_cast<long>(n_tokens) * channels > std::numeric_limits<int32_t>::max())
        return GLA_ESHAPE;
    if (static_cast<long>(n_seqs) * channels > kMaxWork * 8) return GLA_ESHAPE;
    if (n_seqs > 0) {
        if (n_slots < 1) return GLA_ESHAPE;
        if (!cu_seqlens || !conv_cache || !slot_idx || !w) return GLA_EPTR;
    }
    if (n_tokens > 0) {
        if (n_seqs < 1) return GLA_ESHAPE;
        if (!x || !y) return GLA_EPTR;
    }
    if (n_seqs == 0) return GLA_OK;
    gla::ConvArgs a{x, w, cu_seqlens, n_seqs, n_tokens, channels, width, conv_cache, n_slots,
                    slot_idx, (flags & GLA_ZERO_INIT) ? 1 : 0, y, dtype == GLA_BF16};
    return hip_status(gla::launch_conv1d(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
