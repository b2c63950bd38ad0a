/*
 * mha.h -- C ABI of the MI355X (gfx950) multi-head scaled dot-product
 * attention forward library, libmha.so.
 *
 * The operations are those of "Attention Is All You Need" as stated on the
 * pages this library follows:
 *   [Slides]     "Attention Is All You Need -- A Revolutionary Architecture
 *                for Sequence Transduction" (slide deck)
 *   [Deep]       "Paper Deep Reading: Attention Is All You Need"
 *   [Paperglide] "Attention Is All You Need" explainer (paperglide)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller, contiguous
 *   row-major, 16-byte aligned.  The library never allocates, frees or
 *   synchronises; it keeps no state besides a cached device-property query,
 *   and is safe to call from several host threads.
 * - All work is enqueued on `stream` (a hipStream_t; NULL means the legacy
 *   default stream) and runs asynchronously: a return of MHA_OK means the
 *   arguments were accepted and the kernels launched, not that they finished.
 * - Every tensor of one call has the element type `dt`; arithmetic
 *   accumulates in fp32 and stores round to nearest even.
 * - "BLHD" is the layout [B, L, h, d] (row-major).  It is byte-identical to
 *   the [B*L, h*d] matrix X W with head t in column block t, and to
 *   Concat(head_1, ..., head_h) ([Paperglide] two-head toy example; [Deep]
 *   section 04, MultiHead equations).
 * - Errors: the return value is an mha_status.  Arguments are validated on
 *   the host before any HIP call; a rejected call launches nothing and
 *   leaves every buffer untouched.  MHA_ERR_LAUNCH reports a failed kernel
 *   launch (hipGetLastError after the launch).
 */
#ifndef MHA_H
#define MHA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MHA_OK = 0,
    MHA_ERR_INVALID_ARG = 1, /* a dimension < 1 (or < 0 where 0 is allowed),
                                a NULL pointer, KEY_PADDING without kv_lens,
                                CAUSAL with Lq != Lk, an unknown dtype/mask */
    MHA_ERR_UNSUPPORTED = 2, /* valid but not compiled: d_k != d_v, a head
                                size or GEMM width outside the built set */
    MHA_ERR_LAUNCH = 3,      /* the kernel launch failed */
    MHA_ERR_SCRATCH = 4      /* mha_decode_noalloc: the call needs more than
                                MHA_DECODE_SCRATCH_BYTES of partial states */
} mha_status;

/* The two sentinels give the enum the range of int, so any int a caller
 * passes is a value of the type (an unknown code is rejected with
 * MHA_ERR_INVALID_ARG, not undefined behaviour); they are not dtypes. */
typedef enum {
    MHA_F32 = 0,
    MHA_BF16 = 1,
    MHA_DTYPE_RANGE_MIN_ = -0x7FFFFFFF - 1,
    MHA_DTYPE_RANGE_MAX_ = 0x7FFFFFFF
} mha_dtype;

/* Mask bit flags for M; MHA_MASK_KEY_PADDING | MHA_MASK_CAUSAL is their
 * union (-inf wherever either applies). */
enum {
    MHA_MASK_NONE = 0,
    MHA_MASK_KEY_PADDING = 1, /* key j of batch row b is illegal iff
                                 j >= clamp(kv_lens[b], 0, Lk); the encoder
                                 masks padding ([Deep] section 04) */
    MHA_MASK_CAUSAL = 2       /* key j is illegal for query i iff j > i; the
                                 decoder also masks future positions
                                 ([Deep] section 03 "Decoder layer" and
                                 section 04); requires Lq == Lk */
};

/*
 * mha_forward -- scaled dot-product attention for every (batch row, head):
 *
 *     O = softmax(Q K^T / sqrt(d_k) + M) V
 *
 * ([Deep] section 04, attention equation with M; [Slides] slide "Attention
 * Mechanism").  M is 0 at legal (query, key) pairs and -inf at illegal ones
 * (mask_flags above); the weights of illegal keys are exactly 0.
 *
 *   q  [B, Lq, h, d_k]  BLHD   queries (for cross-attention: decoder side)
 *   k  [B, Lk, h, d_k]  BLHD   keys    (for cross-attention: encoder memory)
 *   v  [B, Lk, h, d_v]  BLHD   values
 *   o  [B, Lq, h, d_v]  BLHD   output, written in full (this IS the concat
 *                              of the heads); must not overlap q, k or v
 *   kv_lens  int32 [B] on the device: valid key count per batch row,
 *            required iff MHA_MASK_KEY_PADDING is set, else ignored (may be
 *            NULL); values outside [0, Lk] are clamped.
 *
 * Rows of K and V at or beyond kv_lens[b] are never read and may hold any
 * bits (NaN included).  Rows below kv_lens[b] must be finite.  A query row
 * with no legal key (kv_lens[b] == 0) outputs exactly 0.  Padded query rows
 * are computed like any other row.
 *
 * Supported: B, Lq, Lk >= 0 and h >= 1 (B == 0 or Lq == 0 is a no-op;
 * Lk == 0 gives O = 0), d_k == d_v, B*h*ceil(Lq/64) < 2^31, and one batch
 * row of Q or of K/V under 2 GiB (L*h*d_k*elem_size < 2^31);
 * MHA_BF16 with d_k in {16, 32, 64, 128} (the head sizes of [Deep] section
 * 08, Table 3, rows (A), besides 512); MHA_F32 with d_k in {8, 16, 32, 64}.
 */
int mha_forward(mha_dtype dt, int B, int h, int Lq, int Lk, int d_k, int d_v,
                const void* q, const void* k, const void* v,
                int mask_flags, const int32_t* kv_lens,
                void* o, hipStream_t stream);

/*
 * mha_forward_windowed -- restricted self-attention: mha_forward with each
 * query i seeing only the keys j with |i - j| <= window, a neighbourhood of
 * r = 2*window + 1 positions centred on the query, so a layer costs
 * O(r n d) instead of O(n^2 d) ([Deep] section 05, the complexity table,
 * "Restricted self-attention"; [Slides] slide "Limitations and Future
 * Work").  The band combines with mask_flags as their union (causal keeps
 * i - window .. i).  Arguments as for mha_forward plus
 *
 *   window   half-width, >= 0 (0: each query sees its own position only);
 *            values >= Lk restrict nothing.
 *
 * K and V rows below kv_lens[b] are data even where they lie outside some
 * query's band, and must be finite, as for causal; rows at or past kv_lens[b]
 * may hold any bits.
 *
 * Errors: MHA_ERR_INVALID_ARG also for window < 0 or Lq != Lk (query and
 * key positions must lie on one axis); otherwise as mha_forward, with the
 * same supported dtypes and head sizes.
 */
int mha_forward_windowed(mha_dtype dt, int B, int h, int Lq, int Lk, int d_k, int d_v,
                         const void* q, const void* k, const void* v,
                         int mask_flags, const int32_t* kv_lens, int window,
                         void* o, hipStream_t stream);

/*
 * mha_project_qkv -- the per-head projections of every head at once:
 *
 *     Q = X_q W^Q,  K = X_kv W^K,  V = X_kv W^V
 *
 * with W^Q = [W_1^Q || ... || W_h^Q] etc., so head t of Q is column block t
 * ([Slides] slide "Multi-Head Attention": head_i = Attention(Q W_i^Q,
 * K W_i^K, V W_i^V); [Paperglide] two-head toy example).  No bias.
 *
 *   x_q   [B, Lq, d_model]           decoder (or self-attention) input
 *   x_kv  [B, Lk, d_model]           key/value source: the same pointer as
 *                                    x_q for self-attention, the encoder
 *                                    memory z for cross-attention
 *   w_q, w_k  [d_model, h*d_k]       row-vector convention: out = x W
 *   w_v       [d_model, h*d_v]
 *   q  [B, Lq, h, d_k], k [B, Lk, h, d_k], v [B, Lk, h, d_v]  BLHD outputs;
 *   outputs must not overlap the inputs or each other.
 *
 * Supported: MHA_BF16 and MHA_F32; d_model % 64 == 0, h*d_k % 64 == 0,
 * d_k == d_v; for MHA_BF16 also d_model * h*d_k < 2^30 and d_model < 2^23
 * (32-bit byte offsets within a weight matrix and 128 rows of X).
 */
int mha_project_qkv(mha_dtype dt, int B, int Lq, int Lk, int d_model, int h,
                    int d_k, int d_v,
                    const void* x_q, const void* x_kv,
                    const void* w_q, const void* w_k, const void* w_v,
                    void* q, void* k, void* v, hipStream_t stream);

/*
 * mha_out_proj -- MultiHead = Concat(head_1, ..., head_h) W^O ([Deep]
 * section 04, MultiHead equation; [Slides] slide "Multi-Head Attention").
 *
 *   o    [B, Lq, h, d_v] = [B*Lq, h*d_v]   the attention output (BLHD)
 *   w_o  [h*d_v, d_model]
 *   y    [B, Lq, d_model]                  output; must not overlap o, w_o
 *
 * Supported: MHA_BF16 and MHA_F32; d_model % 64 == 0, h*d_v % 64 == 0; for
 * MHA_BF16 also h*d_v * d_model < 2^30 and h*d_v < 2^23 (32-bit byte offsets
 * within W^O and 128 rows of o).
 */
int mha_out_proj(mha_dtype dt, int B, int Lq, int h, int d_v, int d_model,
                 const void* o, const void* w_o, void* y, hipStream_t stream);

/*
 * mha_out_proj_post_norm -- the attention sub-layer's output with its
 * residual connection and layer normalisation, in post-norm order:
 *
 *     y = LayerNorm(x_res + Concat(head_1, ..., head_h) W^O)
 *     LayerNorm(z)_j = gamma_j (z_j - mu) / sqrt(var + eps) + beta_j
 *
 * with mu and var the mean and the population variance (divisor d_model) of
 * the row z ([Deep] section 03, residual connection and LayerNorm around each
 * sub-layer, and section 04, MultiHead equation; [Slides] slide "Encoder
 * Architecture").  The pages name the normalisation without its formula;
 * this is the usual per-feature-vector form, eps inside the square root.
 * One kernel: the product, the residual add and the statistics stay in fp32
 * on chip; only y (in the element type dt) is written.
 *
 *   o      [B, Lq, h, d_v] = [B*Lq, h*d_v]   the attention output (BLHD)
 *   w_o    [h*d_v, d_model]
 *   x_res  [B, Lq, d_model]                  the sub-layer's input x
 *   gamma, beta [d_model]                    gain and bias
 *   eps    >= 0, finite (1e-6 is the usual choice); with eps = 0 a row whose
 *          residual sum is constant has var = 0 and normalises to NaN
 *   y      [B, Lq, d_model]                  output: either x_res itself
 *          (in-place update of the residual stream) or memory that overlaps
 *          none of the inputs
 *
 * All pointers device, 16-byte aligned.  Supported: d_model in
 * {256, 512, 1024} and B*Lq, h*d_v < 2^31; MHA_BF16 also needs h*d_v % 32 ==
 * 0 and h*d_v * d_model < 2^30 (one kernel on MFMA); MHA_F32 (fp32
 * products and accumulation on MFMA, the accuracy path) takes any h*d_v.
 * MHA_ERR_UNSUPPORTED otherwise;
 * MHA_ERR_INVALID_ARG for negative sizes, a NaN, negative or infinite eps,
 * a NULL or misaligned pointer, or y partly overlapping x_res.  B*Lq == 0
 * is a no-op.
 */
int mha_out_proj_post_norm(mha_dtype dt, int B, int Lq, int h, int d_v, int d_model,
                           const void* o, const void* w_o, const void* x_res,
                           const void* gamma, const void* beta, float eps, void* y,
                           hipStream_t stream);

/*
 * mha_self_attention_fused -- the Q/K/V projections and the attention of
 * every head of a self-attention layer in one launch, for rows of at most
 * 128 tokens:
 *
 *     O = Concat_t softmax((X W_t^Q)(X W_t^K)^T / sqrt(d_k) + M) (X W_t^V)
 *
 * ([Slides] slide "Multi-Head Attention"; [Deep] section 04, attention
 * equation with M and MultiHead equations).  The result equals
 * mha_project_qkv(x, x, ...) followed by mha_forward(...) on the same
 * arguments; the projected Q, K, V are never written to memory.
 *
 *   x          [B, L, d_model]         the layer input (queries and keys/values)
 *   w_q, w_k, w_v [d_model, h*d_k]     row-vector convention, head t in column
 *                                      block t
 *   mask_flags, kv_lens                as for mha_forward (with Lq = Lk = L)
 *   o          [B, L, h, d_k]  BLHD    output (the concat of the heads); must
 *                                      not overlap the inputs
 *
 * Supported: MHA_BF16, d_k = 64, 1 <= L <= 128, d_model % 64 == 0, B*h <
 * 2^31 (B == 0 is a no-op); MHA_ERR_UNSUPPORTED otherwise, in which case
 * the two-call path computes the same thing.
 */
int mha_self_attention_fused(mha_dtype dt, int B, int L, int d_model, int h, int d_k,
                             const void* x, const void* w_q, const void* w_k, const void* w_v,
                             int mask_flags, const int32_t* kv_lens, void* o,
                             hipStream_t stream);

/*
 * mha_decode -- one decoding step against a key/value cache: for every
 * sequence b and head t, the newest position's query attends to the
 * cache_lens[b] cached keys (positions 0 .. len - 1, which under the
 * decoder's causal mask is every earlier position and itself):
 *
 *     o_b,t = softmax(q_b,t K_b,t^T / sqrt(d_k)) V_b,t
 *
 * ([Deep] section 04, attention equation; section 03 "Decoder layer", one
 * position per step with the causal mask; beam search keeps one cache per
 * beam, so beams are just more sequences).  The result equals mha_forward
 * with Lq = 1, Lk = L_cache and MHA_MASK_KEY_PADDING with kv_lens =
 * cache_lens, computed as a split over the cache (partial softmax states of
 * 1024-key chunks, merged in a fixed order, so it is deterministic) with fp32
 * scores and weights.
 *
 *   q           [B, 1, h, d_k]        the step's queries
 *   k_cache     [B, L_cache, h, d_k]  BLHD, as mha_forward's k; rows at or
 *   v_cache     [B, L_cache, h, d_v]  past cache_lens[b] are never read
 *   cache_lens  device int32 [B], clamped to [0, L_cache]; 0 gives o = 0
 *   o           [B, 1, h, d_v]
 *   workspace   caller-owned device memory of at least
 *               mha_decode_workspace_bytes(B, h, L_cache, d_k) bytes,
 *               16-byte aligned (fp32 partial states; its contents are
 *               scratch, nothing needs clearing); workspace_bytes its size.
 *               Calls that share a workspace must not run at the same time.
 *
 * Supported: MHA_BF16, d_k == d_v in {64, 128}, any h >= 1 (heads are
 * taken 32 at a time per workgroup), L_cache*h*d_k*2 < 2^31 (B == 0 is a
 * no-op); MHA_ERR_UNSUPPORTED otherwise.  A workspace that is
 * NULL, misaligned or too small is MHA_ERR_INVALID_ARG.
 */
size_t mha_decode_workspace_bytes(int B, int h, int L_cache, int d_k);
int mha_decode(mha_dtype dt, int B, int h, int L_cache, int d_k, int d_v,
               const void* q, const void* k_cache, const void* v_cache,
               const int32_t* cache_lens, void* o,
               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mha_decode_noalloc -- mha_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  The same kernels and result (bit for bit) as mha_decode,
 * with the partial states in a static scratch buffer of the library instead
 * of a caller workspace; the call allocates nothing (no hipMalloc, hipFree
 * or allocating library routine).
 *
 * Limit: mha_decode_workspace_bytes(B, h, L_cache, d_k) must not exceed
 * MHA_DECODE_SCRATCH_BYTES (16 MiB: e.g. 64 sequences x 16 heads with caches
 * of up to 32768 positions at d_k = 64, which need 8.7 MB); larger calls
 * return MHA_ERR_SCRATCH and launch nothing.  Each GPU the library runs on holds its own copy of the
 * buffer until the process ends, looked up on the first call on that GPU.
 * Every call on one GPU shares that copy, so calls that overlap in time on
 * one GPU (on different streams, or from different host threads) race and
 * must be ordered by the caller; calls on one stream are ordered already.
 * Nothing in the buffer needs clearing between calls.
 *
 * Arguments, other status codes and support: as mha_decode.
 */
#define MHA_DECODE_SCRATCH_BYTES ((size_t)16 << 20)
int mha_decode_noalloc(mha_dtype dt, int B, int h, int L_cache, int d_k, int d_v,
                       const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* cache_lens, void* o, hipStream_t stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* mha_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MHA_H */
