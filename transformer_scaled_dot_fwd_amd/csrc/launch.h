// launch.h -- host-side launchers of the device kernels (internal to
// libmha.so; the public C ABI is include/mha.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mha {

struct AttnArgs {
    int B, H, Lq, Lk, D;
    int mask;                 // bit 0: key padding, bit 1: causal
    const void* q;
    const void* k;
    const void* v;
    const int32_t* kv_lens;   // device, [B]; only read with key padding
    void* o;
    int window = -1;          // restricted attention half-width; -1: none
};

hipError_t launch_attention_bf16(const AttnArgs& a, hipStream_t stream);
// The streaming kernel for d = 64 (attn_stream.hip): any row length,
// restricted attention included.
hipError_t launch_attention_stream_bf16(const AttnArgs& a, hipStream_t stream);

// Self-attention of every (batch row, head) with the projections fused in:
// x [B, L, DM], w_q/w_k/w_v [DM, H*64], o [B, L, H, 64]; L <= 128.
struct FusedArgs {
    int B, L, DM, H;
    int mask;                 // bit 0: key padding, bit 1: causal
    const void* x;
    const void* w_q;
    const void* w_k;
    const void* w_v;
    const int32_t* kv_lens;   // device, [B]; only read with key padding
    void* o;
};
hipError_t launch_self_attention_fused_bf16(const FusedArgs& a, hipStream_t stream);
hipError_t launch_attention_f32(const AttnArgs& a, hipStream_t stream);

// One decoding step: q [B, H, D] (one query per sequence and head) against
// the caches k, v [B, L, H, D] with lens[b] valid keys (device int32 [B]);
// o [B, H, D]; workspace: decode_workspace_bytes(B, H, L, D) bytes of fp32
// partial states.  D in {64, 128}, bf16.
struct DecodeArgs {
    int B, H, L, D;
    const void* q;
    const void* k;
    const void* v;
    const int32_t* lens;
    void* o;
    void* workspace;
};
size_t decode_workspace_bytes(int B, int H, int L, int D);
// Workgroups along the first grid axis of the partial-state kernel
// (sequences x chunks of the cache); the host keeps it within INT_MAX.
long long decode_partial_workgroups(int B, int L);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream);

// The library's static scratch for the decode step's partial states (for
// callers that cannot allocate): its size, and its device address on the
// stream's device.
constexpr size_t DECODE_SCRATCH_BYTES = (size_t)16 << 20;
hipError_t decode_scratch(hipStream_t stream, void** ptr);

// The attention sub-layer's output with its residual and post-norm:
// out[M, N] = LayerNorm(x[M, N] + o[M, K] w[K, N]) with gain gamma[N], bias
// beta[N]; N in {256, 512, 1024}; bf16 (K % 32 == 0) or fp32.
struct PostNormArgs {
    int M, N, K;
    const void* o;
    const void* w;
    const void* x;
    const void* gamma;
    const void* beta;
    float eps;
    void* out;
};
hipError_t launch_out_proj_post_norm_bf16(const PostNormArgs& a, hipStream_t stream);
hipError_t launch_out_proj_post_norm_f32(const PostNormArgs& a, hipStream_t stream);

// One GEMM problem Y[M, N] = X[M, K] W[K, N] (row-major).
struct GemmProblem {
    const void* x;
    const void* w;
    void* y;
    int M;
};

// Up to three independent problems sharing N and K, in one launch; `qkv`
// only selects the kernel's name (projection of Q/K/V vs. W^O).
hipError_t launch_gemm_bf16(const GemmProblem* probs, int n_probs, int N, int K, bool qkv,
                            hipStream_t stream);
hipError_t launch_gemm_f32(const GemmProblem* probs, int n_probs, int N, int K,
                           hipStream_t stream);

}  // namespace mha
