// mha_api.hip -- the extern "C" boundary of libmha.so (declared in
// include/mha.h): argument validation, dispatch to the compiled kernels and
// launch on the caller's stream.  Validation finishes before the first HIP
// call, so a rejected call touches neither the device nor any buffer.
#include <limits.h>
#include <stdint.h>

#include "launch.h"
#include "mha.h"

static_assert(MHA_DECODE_SCRATCH_BYTES == mha::DECODE_SCRATCH_BYTES,
              "the header states the static scratch's size");

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int launch_status(hipError_t e) { return e == hipSuccess ? MHA_OK : MHA_ERR_LAUNCH; }

}  // namespace

extern "C" {

const char* mha_status_string(int status) {
    switch (status) {
        case MHA_OK: return "ok";
        case MHA_ERR_INVALID_ARG: return "invalid argument";
        case MHA_ERR_UNSUPPORTED: return "unsupported dtype or shape (not compiled)";
        case MHA_ERR_LAUNCH: return "kernel launch failed";
        case MHA_ERR_SCRATCH:
            return "problem needs more scratch than the library's static buffer holds";
        default: return "unknown status";
    }
}

}  // extern "C"

namespace {

// mha_forward and mha_forward_windowed; window < 0: no restriction.
int forward(mha_dtype dt, int B, int h, int Lq, int Lk, int d_k, int d_v, const void* q,
            const void* k, const void* v, int mask_flags, const int32_t* kv_lens, int window,
            void* o, hipStream_t stream) {
    if (dt != MHA_F32 && dt != MHA_BF16) return MHA_ERR_INVALID_ARG;
    if (B < 0 || h < 1 || Lq < 0 || Lk < 0 || d_k < 1 || d_v < 1) return MHA_ERR_INVALID_ARG;
    if (mask_flags & ~(MHA_MASK_KEY_PADDING | MHA_MASK_CAUSAL)) return MHA_ERR_INVALID_ARG;
    if ((mask_flags & MHA_MASK_CAUSAL) && Lq != Lk) return MHA_ERR_INVALID_ARG;
    if (B == 0 || Lq == 0) return MHA_OK;  // empty output: nothing to do
    if (!q || !o) return MHA_ERR_INVALID_ARG;
    if (Lk > 0 && (!k || !v)) return MHA_ERR_INVALID_ARG;
    if ((mask_flags & MHA_MASK_KEY_PADDING) && !kv_lens) return MHA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(o) || (Lk > 0 && (!aligned16(k) || !aligned16(v))))
        return MHA_ERR_INVALID_ARG;
    if (d_k != d_v) return MHA_ERR_UNSUPPORTED;
    if ((long long)B * h > INT_MAX) return MHA_ERR_UNSUPPORTED;
    const long long tiles = (long long)B * h * ((Lq + 63) / 64);
    if (tiles > INT_MAX) return MHA_ERR_UNSUPPORTED;
    // Kernels address one batch row's Q, K or V slab with 32-bit byte
    // offsets below 2^31.
    const long long row_bytes = (long long)h * d_k * (dt == MHA_BF16 ? 2 : 4);
    if ((long long)Lq * row_bytes >= (1LL << 31) || (long long)Lk * row_bytes >= (1LL << 31))
        return MHA_ERR_UNSUPPORTED;

    mha::AttnArgs a{B, h, Lq, Lk, d_k, mask_flags, q, k, v, kv_lens, o};
    // A window of Lk or more restricts nothing; clamping it keeps the
    // kernels' index sums far from overflow.
    a.window = window < 0 ? -1 : (window < Lk ? window : Lk);
    if (dt == MHA_BF16) {
        if (d_k != 16 && d_k != 32 && d_k != 64 && d_k != 128) return MHA_ERR_UNSUPPORTED;
        return launch_status(mha::launch_attention_bf16(a, stream));
    }
    if (d_k != 8 && d_k != 16 && d_k != 32 && d_k != 64) return MHA_ERR_UNSUPPORTED;
    return launch_status(mha::launch_attention_f32(a, stream));
}

}  // namespace

extern "C" {

int mha_forward(mha_dtype dt, int B, int h, int Lq, int Lk, int d_k, int d_v, const void* q,
                const void* k, const void* v, int mask_flags, const int32_t* kv_lens, void* o,
                hipStream_t stream) {
    return forward(dt, B, h, Lq, Lk, d_k, d_v, q, k, v, mask_flags, kv_lens, -1, o, stream);
}

int mha_forward_windowed(mha_dtype dt, int B, int h, int Lq, int Lk, int d_k, int d_v,
                         const void* q, const void* k, const void* v, int mask_flags,
                         const int32_t* kv_lens, int window, void* o, hipStream_t stream) {
    if (window < 0 || Lq != Lk) return MHA_ERR_INVALID_ARG;
    return forward(dt, B, h, Lq, Lk, d_k, d_v, q, k, v, mask_flags, kv_lens, window, o, stream);
}

int mha_project_qkv(mha_dtype dt, int B, int Lq, int Lk, int d_model, int h, int d_k, int d_v,
                    const void* x_q, const void* x_kv, const void* w_q, const void* w_k,
                    const void* w_v, void* q, void* k, void* v, hipStream_t stream) {
    if (dt != MHA_F32 && dt != MHA_BF16) return MHA_ERR_INVALID_ARG;
    if (B < 0 || Lq < 0 || Lk < 0 || d_model < 1 || h < 1 || d_k < 1 || d_v < 1)
        return MHA_ERR_INVALID_ARG;
    const long long Mq = (long long)B * Lq, Mkv = (long long)B * Lk;
    if (Mq == 0 && Mkv == 0) return MHA_OK;
    if (Mq > 0 && (!x_q || !w_q || !q)) return MHA_ERR_INVALID_ARG;
    if (Mkv > 0 && (!x_kv || !w_k || !w_v || !k || !v)) return MHA_ERR_INVALID_ARG;
    const void* ptrs[] = {x_q, x_kv, w_q, w_k, w_v, q, k, v};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MHA_ERR_INVALID_ARG;
    if (d_k != d_v) return MHA_ERR_UNSUPPORTED;
    const long long N = (long long)h * d_k;
    if (d_model % 64 != 0 || N % 64 != 0 || N > INT_MAX) return MHA_ERR_UNSUPPORTED;
    // bf16: a weight matrix and 128 rows of X are addressed with 32-bit byte
    // offsets.
    if (dt == MHA_BF16 &&
        ((long long)d_model * N * 2 >= (1LL << 31) || (long long)d_model * 256 >= (1LL << 31)))
        return MHA_ERR_UNSUPPORTED;
    if (Mq > INT_MAX || Mkv > INT_MAX) return MHA_ERR_UNSUPPORTED;

    mha::GemmProblem probs[3];
    int n = 0;
    if (Mq > 0) probs[n++] = {x_q, w_q, q, (int)Mq};
    if (Mkv > 0) {
        probs[n++] = {x_kv, w_k, k, (int)Mkv};
        probs[n++] = {x_kv, w_v, v, (int)Mkv};
    }
    const hipError_t e = (dt == MHA_BF16)
                             ? mha::launch_gemm_bf16(probs, n, (int)N, d_model, true, stream)
                             : mha::launch_gemm_f32(probs, n, (int)N, d_model, stream);
    return launch_status(e);
}

int mha_out_proj(mha_dtype dt, int B, int Lq, int h, int d_v, int d_model, const void* o,
                 const void* w_o, void* y, hipStream_t stream) {
    if (dt != MHA_F32 && dt != MHA_BF16) return MHA_ERR_INVALID_ARG;
    if (B < 0 || Lq < 0 || h < 1 || d_v < 1 || d_model < 1) return MHA_ERR_INVALID_ARG;
    const long long M = (long long)B * Lq;
    if (M == 0) return MHA_OK;
    if (!o || !w_o || !y) return MHA_ERR_INVALID_ARG;
    if (!aligned16(o) || !aligned16(w_o) || !aligned16(y)) return MHA_ERR_INVALID_ARG;
    const long long K = (long long)h * d_v;
    if (d_model % 64 != 0 || K % 64 != 0 || K > INT_MAX || M > INT_MAX)
        return MHA_ERR_UNSUPPORTED;
    // bf16: W^O and 128 rows of O are addressed with 32-bit byte offsets.
    if (dt == MHA_BF16 && (K * d_model * 2 >= (1LL << 31) || K * 256 >= (1LL << 31)))
        return MHA_ERR_UNSUPPORTED;
    mha::GemmProblem prob{o, w_o, y, (int)M};
    const hipError_t e = (dt == MHA_BF16)
                             ? mha::launch_gemm_bf16(&prob, 1, d_model, (int)K, false, stream)
                             : mha::launch_gemm_f32(&prob, 1, d_model, (int)K, stream);
    return launch_status(e);
}

int mha_out_proj_post_norm(mha_dtype dt, int B, int Lq, int h, int d_v, int d_model,
                           const void* o, const void* w_o, const void* x_res, const void* gamma,
                           const void* beta, float eps, void* y, hipStream_t stream) {
    if (dt != MHA_F32 && dt != MHA_BF16) return MHA_ERR_INVALID_ARG;
    if (B < 0 || Lq < 0 || h < 1 || d_v < 1 || d_model < 1) return MHA_ERR_INVALID_ARG;
    if (!(eps >= 0.0f) || eps > 3.0e38f) return MHA_ERR_INVALID_ARG;  // NaN, negative, inf
    const long long M = (long long)B * Lq;
    if (M == 0) return MHA_OK;
    const void* ptrs[] = {o, w_o, x_res, gamma, beta, y};
    for (const void* p : ptrs)
        if (!p || !aligned16(p)) return MHA_ERR_INVALID_ARG;
    // y may be x_res itself (the residual stream updated in place: each
    // workgroup reads its rows of x_res before it writes them) but must not
    // overlap it otherwise.
    const size_t rows_bytes = (size_t)M * d_model * (dt == MHA_BF16 ? 2 : 4);
    const char* yb = (const char*)y;
    const char* xb = (const char*)x_res;
    if (yb != xb && yb < xb + rows_bytes && xb < yb + rows_bytes) return MHA_ERR_INVALID_ARG;
    const long long K = (long long)h * d_v;
    if (d_model != 256 && d_model != 512 && d_model != 1024) return MHA_ERR_UNSUPPORTED;
    if (K > INT_MAX || M > INT_MAX) return MHA_ERR_UNSUPPORTED;
    mha::PostNormArgs a{(int)M, d_model, (int)K, o, w_o, x_res, gamma, beta, eps, y};
    if (dt == MHA_F32) return launch_status(mha::launch_out_proj_post_norm_f32(a, stream));
    // bf16: the k step is 32, and W^O and 32 rows of o are addressed with
    // 32-bit byte offsets.
    if (K % 32 != 0) return MHA_ERR_UNSUPPORTED;
    if (K * d_model * 2 >= (1LL << 31) || K * 64 >= (1LL << 31)) return MHA_ERR_UNSUPPORTED;
    return launch_status(mha::launch_out_proj_post_norm_bf16(a, stream));
}

size_t mha_decode_workspace_bytes(int B, int h, int L_cache, int d_k) {
    if (B < 0 || h < 1 || L_cache < 0 || d_k < 1) return 0;
    return mha::decode_workspace_bytes(B, h, L_cache, d_k);
}

}  // extern "C"

namespace {

// Validation shared by mha_decode and mha_decode_noalloc (everything but the
// workspace); MHA_OK means "launch".
int decode_check(mha_dtype dt, int B, int h, int L_cache, int d_k, int d_v, const void* q,
                 const void* k_cache, const void* v_cache, const int32_t* cache_lens,
                 const void* o) {
    if (dt != MHA_F32 && dt != MHA_BF16) return MHA_ERR_INVALID_ARG;
    if (B < 0 || h < 1 || L_cache < 0 || d_k < 1 || d_v < 1) return MHA_ERR_INVALID_ARG;
    if (B == 0) return MHA_OK;
    if (!q || !o || !cache_lens) return MHA_ERR_INVALID_ARG;
    if (L_cache > 0 && (!k_cache || !v_cache)) return MHA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(o) ||
        (L_cache > 0 && (!aligned16(k_cache) || !aligned16(v_cache))))
        return MHA_ERR_INVALID_ARG;
    if (dt != MHA_BF16 || d_k != d_v || (d_k != 64 && d_k != 128)) return MHA_ERR_UNSUPPORTED;
    // One sequence's cache rows are addressed with 32-bit byte offsets; one
    // workgroup per (sequence, chunk of the cache).
    if ((long long)L_cache * h * d_k * 2 >= (1LL << 31)) return MHA_ERR_UNSUPPORTED;
    if (mha::decode_partial_workgroups(B, L_cache) > INT_MAX || (long long)B * h > INT_MAX)
        return MHA_ERR_UNSUPPORTED;
    return MHA_OK;
}

}  // namespace

extern "C" {

int mha_decode(mha_dtype dt, int B, int h, int L_cache, int d_k, int d_v, const void* q,
               const void* k_cache, const void* v_cache, const int32_t* cache_lens, void* o,
               void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const int rc = decode_check(dt, B, h, L_cache, d_k, d_v, q, k_cache, v_cache, cache_lens, o);
    if (rc != MHA_OK || B == 0) return rc;
    if (!workspace || !aligned16(workspace)) return MHA_ERR_INVALID_ARG;
    if (workspace_bytes < mha::decode_workspace_bytes(B, h, L_cache, d_k))
        return MHA_ERR_INVALID_ARG;
    mha::DecodeArgs a{B, h, L_cache, d_k, q, k_cache, v_cache, cache_lens, o, workspace};
    return launch_status(mha::launch_decode_bf16(a, stream));
}

int mha_decode_noalloc(mha_dtype dt, int B, int h, int L_cache, int d_k, int d_v,
                       const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* cache_lens, void* o, hipStream_t stream) {
    const int rc = decode_check(dt, B, h, L_cache, d_k, d_v, q, k_cache, v_cache, cache_lens, o);
    if (rc != MHA_OK || B == 0) return rc;
    if (mha::decode_workspace_bytes(B, h, L_cache, d_k) > MHA_DECODE_SCRATCH_BYTES)
        return MHA_ERR_SCRATCH;
    void* ws = nullptr;
    if (mha::decode_scratch(stream, &ws) != hipSuccess) return MHA_ERR_LAUNCH;
    mha::DecodeArgs a{B, h, L_cache, d_k, q, k_cache, v_cache, cache_lens, o, ws};
    return launch_status(mha::launch_decode_bf16(a, stream));
}

int mha_self_attention_fused(mha_dtype dt, int B, int L, int d_model, int h, int d_k,
                             const void* x, const void* w_q, const void* w_k, const void* w_v,
                             int mask_flags, const int32_t* kv_lens, void* o,
                             hipStream_t stream) {
    if (dt != MHA_F32 && dt != MHA_BF16) return MHA_ERR_INVALID_ARG;
    if (B < 0 || L < 1 || d_model < 1 || h < 1 || d_k < 1) return MHA_ERR_INVALID_ARG;
    if (mask_flags & ~(MHA_MASK_KEY_PADDING | MHA_MASK_CAUSAL)) return MHA_ERR_INVALID_ARG;
    if (B == 0) return MHA_OK;
    if (!x || !w_q || !w_k || !w_v || !o) return MHA_ERR_INVALID_ARG;
    if ((mask_flags & MHA_MASK_KEY_PADDING) && !kv_lens) return MHA_ERR_INVALID_ARG;
    const void* ptrs[] = {x, w_q, w_k, w_v, o};
    for (const void* p : ptrs)
        if (!aligned16(p)) return MHA_ERR_INVALID_ARG;
    if (dt != MHA_BF16 || d_k != 64 || L > 128 || d_model % 64 != 0) return MHA_ERR_UNSUPPORTED;
    if ((long long)B * h > INT_MAX || (long long)h * 64 > INT_MAX / 2) return MHA_ERR_UNSUPPORTED;
    // One batch row of X and one weight matrix are addressed with 32-bit
    // byte offsets.
    if ((long long)L * d_model * 2 >= (1LL << 31) || (long long)d_model * h * 64 * 2 >= (1LL << 31))
        return MHA_ERR_UNSUPPORTED;
    mha::FusedArgs a{B, L, d_model, h, mask_flags, x, w_q, w_k, w_v, kv_lens, o};
    return launch_status(mha::launch_self_attention_fused_bf16(a, stream));
}

}  // extern "C"
