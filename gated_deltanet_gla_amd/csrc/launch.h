// Internal launch interface between the host-side C ABI (api.cpp) and the
// kernel translation units.  Arguments are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gla {

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const float* beta;       // GDN only
    int n_req, n_heads, dk, dv;
    int in_bf16, out_bf16;
    float* pool;
    int n_slots;
    const int32_t* slot_idx;
    void* o;
    int n_tok;                    // tokens per request (1 for a single step)
    const int32_t* pos_slots;     // [n_req, n_tok] slots for per-position states, or NULL
};

struct LinDecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    int n_req, n_heads, dk, dv;
    int in_bf16, out_bf16;
    float* pool;
    float* zpool;
    int n_slots;
    const int32_t* slot_idx;
    float eps;
    void* o;
};

struct CopyArgs {
    void* buf;               // [n_slots, slot_bytes]
    long slot_bytes;         // a multiple of 16
    int n_slots;
    const int32_t* src_slots;
    const int32_t* dst_slots;
    int n_copy;
};

struct ChunkArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const float* beta;       // GDN only
    const int32_t* cu_seqlens;
    int n_seqs, n_tokens, n_heads, dk, dv, chunk;
    int in_bf16, out_bf16;
    float* pool;
    int n_slots;
    const int32_t* slot_idx;
    int zero_init;
    void* o;
    void* workspace;
    size_t workspace_bytes;
    const int32_t* ckpt_slots;    // [n_seqs, ckpt_stride] or NULL
    int ckpt_interval;            // tokens, a multiple of chunk
    int ckpt_stride;
    float* zpool;                 // normalised linear attention: [n_slots, n_heads, dk]
    float eps;
    int gdn_phases;               // Gated DeltaNet: 0 = prep then run, 1 = prep only, 2 = run only
};

struct ConvArgs {
    const void* x;
    const float* w;
    const int32_t* cu_seqlens;
    int n_seqs, n_tokens, channels, width;
    void* cache;
    int n_slots;
    const int32_t* slot_idx;
    int zero_init;
    void* y;
    int bf16;
};

hipError_t launch_gla_decode(const DecodeArgs& a, hipStream_t s);
hipError_t launch_gdn_decode(const DecodeArgs& a, hipStream_t s);
hipError_t launch_slot_copy(const CopyArgs& a, hipStream_t s);
hipError_t launch_hbm_probe(int mode, float* pool, int n_req, int n_heads, int n_slots,
                            const int32_t* slot_idx, void* sink, hipStream_t s);
hipError_t launch_lin_attn_decode(const LinDecodeArgs& a, hipStream_t s);
hipError_t launch_gla_chunk(const ChunkArgs& a, hipStream_t s);
size_t lin_attn_chunk_workspace(int n_seqs, int n_tokens, int n_heads, int dk, int dv, int chunk);
hipError_t launch_lin_attn_chunk(const ChunkArgs& a, hipStream_t s);
size_t gla_chunk_workspace(int n_seqs, int n_tokens, int n_heads, int dk, int dv, int chunk);
bool gla_seg_supported(const ChunkArgs& a);
size_t gla_seg_workspace(int n_seqs, int n_tokens, int n_heads);
hipError_t launch_gla_seg(const ChunkArgs& a, hipStream_t s);
hipError_t launch_lin_attn_seg(const ChunkArgs& a, hipStream_t s);
hipError_t launch_gdn_chunk(const ChunkArgs& a, hipStream_t s);
size_t gdn_chunk_workspace(int n_seqs, int n_tokens, int n_heads, int dk, int dv, int chunk);
size_t gdn_seg_workspace(int n_seqs, int n_tokens, int n_heads);
hipError_t launch_gdn_seg_offsets(const ChunkArgs& a, int32_t* coff, void* seg_ws, hipStream_t s);
hipError_t launch_gdn_seg_prep(const ChunkArgs& a, const int32_t* chunk_off, uint16_t* planes, long n_chunks_max,
                               hipStream_t s);
hipError_t launch_gdn_seg(const ChunkArgs& a, const int32_t* chunk_off, const uint16_t* planes, long n_chunks_max,
                          void* seg_ws, hipStream_t s);
hipError_t launch_conv1d(const ConvArgs& a, hipStream_t s);

}  // namespace gla
