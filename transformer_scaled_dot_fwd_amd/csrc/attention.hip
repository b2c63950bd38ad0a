// attention.hip -- fused scaled dot-product attention forward for gfx950.
//
//   O = softmax(Q K^T / sqrt(d_k) + M) V        for every (batch row, head)
//
// ("Paper Deep Reading: Attention Is All You Need", section 04, attention
// equation with the mask M; the order MatMul -> Scale -> Mask -> SoftMax ->
// MatMul is that of Figure 2, left.)  M is -inf at illegal pairs: keys at or
// beyond the batch row's length (the encoder masks padding) and, for the
// decoder, keys after the query (section 03 "Decoder layer", section 04).
//
// The softmax is evaluated online over key tiles (a running row maximum m
// and running sum l, rescaling the partial output when m grows), which is
// the exact identity softmax(x) = softmax(x - c) applied tile by tile; the
// score matrix never leaves registers.
#include "device.h"
#include "launch.h"

namespace mha {

// ---------------------------------------------------------------------------
// bf16, d = 64: MFMA path.
//
// Workgroup = 4 waves = one (batch row, head, tile of 128 queries); wave w
// owns queries q0 + 32w .. q0 + 32w + 31, one query per lane column.  Key/
// value tiles of 64 rows are staged through LDS and shared by the 4 waves.
//
//   S^T = K Q^T        v_mfma_f32_32x32x16_bf16, A = K rows (LDS, 16-byte
//                      reads), B = Q (registers, loaded once)
//   O^T += V^T P^T     A = V^T (LDS transpose reads), B = P (registers)
//
// Keeping the query in the lane column makes every per-query quantity (row
// max, row sum, rescale factor) lane-local, with one exchange between the
// two half-waves.  The PV contraction runs over keys in the order the S^T
// accumulator holds them, and the V^T transpose reads fetch V rows in that
// same order.
// ---------------------------------------------------------------------------
namespace {

constexpr int D64 = 64;
constexpr int BM = 128;          // queries per workgroup
constexpr int BN = 64;           // keys per tile
constexpr int KV_STRIDE = D64 + 8;  // LDS row pitch in elements (144 B)
constexpr int THREADS = 256;

template <bool PAD, bool CAUSAL>
__global__ __launch_bounds__(THREADS, 2) void attn_fwd_bf16_d64(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    bf16* __restrict__ o, const int32_t* __restrict__ kv_lens, int B, int H, int Lq, int Lk,
    int n_qtiles, float scale_log2e) {
    __shared__ __attribute__((aligned(16))) bf16 sK[BN * KV_STRIDE];
    __shared__ __attribute__((aligned(16))) bf16 sV[BN * KV_STRIDE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;
    const int l32 = lane & 31;

    // Tile decode.  Causal: the longest query tiles are launched first.
    const int nbh = B * H;
    int bh, qt;
    if (CAUSAL) {
        qt = n_qtiles - 1 - (int)(blockIdx.x / nbh);
        bh = (int)(blockIdx.x % nbh);
    } else {
        bh = (int)(blockIdx.x / n_qtiles);
        qt = (int)(blockIdx.x % n_qtiles);
    }
    const int b = bh / H;
    const int hh = bh - b * H;
    const int q0 = qt * BM;

    int kv_end = Lk;
    if (PAD) kv_end = min(max(kv_lens[b], 0), Lk);
    int key_end = kv_end;
    if (CAUSAL) key_end = min(key_end, min(q0 + BM, Lq));
    const int n_tiles = (key_end + BN - 1) / BN;

    const size_t rs = (size_t)H * D64;  // elements between consecutive positions
    const bf16* qp = q + ((size_t)b * Lq * H + hh) * D64;
    const bf16* kp = k + ((size_t)b * Lk * H + hh) * D64;
    const bf16* vp = v + ((size_t)b * Lk * H + hh) * D64;
    bf16* op = o + ((size_t)b * Lq * H + hh) * D64;

    // Q as the B operand of S^T = K Q^T: lane holds query l32, d = 16kk + 8half .. +7.
    const int wq0 = q0 + 32 * wave;
    const int my_q = wq0 + l32;
    bf16x8 qop[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        qop[kk] = (my_q < Lq) ? *(const bf16x8*)(qp + (size_t)my_q * rs + 16 * kk + 8 * half)
                              : zero_bf16x8();

    f32x16 acc[2];
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;
    float m_run = -INFINITY;  // running max of the raw logits q.k
    float l_part = 0.0f;      // this lane's share of the row sum

    // Cooperative tile load: 64 rows x 128 B of K and of V, 16 B per chunk,
    // 2 chunks of each per thread.  Rows at or past kv_end are zero-filled
    // and never read from memory.
    bf16x8 kreg[2], vreg[2];
    auto gload = [&](int t) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int c = tid + THREADS * u;
            const int row = c >> 3;
            const int col = (c & 7) * 8;
            const int key = t * BN + row;
            if (key < kv_end) {
                kreg[u] = *(const bf16x8*)(kp + (size_t)key * rs + col);
                vreg[u] = *(const bf16x8*)(vp + (size_t)key * rs + col);
            } else {
                kreg[u] = zero_bf16x8();
                vreg[u] = zero_bf16x8();
            }
        }
    };
    auto sstore = [&]() {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int c = tid + THREADS * u;
            const int row = c >> 3;
            const int col = (c & 7) * 8;
            *(bf16x8*)(sK + row * KV_STRIDE + col) = kreg[u];
            *(bf16x8*)(sV + row * KV_STRIDE + col) = vreg[u];
        }
    };

    if (n_tiles > 0) gload(0);
    for (int t = 0; t < n_tiles; ++t) {
        __syncthreads();  // every wave is done reading the previous tile
        sstore();
        __syncthreads();
        if (t + 1 < n_tiles) gload(t + 1);  // in flight while this tile computes

        const int k0 = t * BN;
        if (wq0 >= Lq) continue;                // this wave holds no query rows
        if (CAUSAL && k0 > wq0 + 31) continue;  // the whole tile is in this wave's future

        // ---- S^T = K Q^T for keys k0 .. k0+63 (two 32-key blocks) ----
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const bf16x8 a =
                    *(const bf16x8*)(sK + (32 * kb + l32) * KV_STRIDE + 16 * kk + 8 * half);
                s[kb] = mfma32(a, qop[kk], s[kb]);
            }
        }

        // ---- mask (boundary tiles only): select -inf at illegal keys ----
        const bool need_mask = (k0 + BN > kv_end) || (CAUSAL && k0 + BN - 1 > wq0);
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + 32 * kb + acc_row(r, half);
                    bool legal = key < kv_end;
                    if (CAUSAL) legal = legal && key <= my_q;
                    s[kb][r] = legal ? s[kb][r] : -INFINITY;
                }
        }

        // ---- online softmax ----
        float mx = s[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = max_halves(mx);
        const float m_new = fmaxf(m_run, mx);
        if (m_new > m_run) {
            // m_run = -inf gives alpha = exp2(-inf) = 0: nothing accumulated yet.
            const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2e);
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
            l_part *= alpha;
            m_run = m_new;
        }
        const float mc = (m_run == -INFINITY) ? 0.0f : m_run * scale_log2e;

        // p = exp2(s * c - m * c) = exp(s/sqrt(d) - m/sqrt(d)), rounded to bf16;
        // the row sum accumulates the rounded p, the values PV actually uses.
        bf16x8 pop[4];  // P^T chunk kc = 2*kb + c: registers 8c .. 8c+7 of s[kb]
        const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const float p0 =
                        __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][8 * c + e], scale_log2e, -mc));
                    const float p1 = __builtin_amdgcn_exp2f(
                        __builtin_fmaf(s[kb][8 * c + e + 1], scale_log2e, -mc));
                    const bf16x2 pp = {(bf16)p0, (bf16)p1};
                    pop[2 * kb + c][e] = pp[0];
                    pop[2 * kb + c][e + 1] = pp[1];
                    l_part = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l_part, false);
                }

        // ---- O^T += V^T P^T ----
        // P chunk kc covers keys k0 + 16kc + {0..3, 8..11} (k = 0..7, lanes < 32)
        // and k0 + 16kc + {4..7, 12..15} (k = 8..15, lanes >= 32).  The matching
        // V^T operand: lane group g = lane/16 reads columns 32db + 16(g&1) + j
        // of rows base + 0..3 and base + 8 .. 11, base = 16kc + 4(g>>1).
        const int g = lane >> 4;
        const int i16 = lane & 15;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            const int base = 16 * kc + 4 * (g >> 1) + (i16 >> 2);
#pragma unroll
            for (int db = 0; db < 2; ++db) {
                const int col = 32 * db + 16 * (g & 1) + 4 * (i16 & 3);
                const bf16x4 lo = lds_read_tr(sV + base * KV_STRIDE + col);
                const bf16x4 hi = lds_read_tr(sV + (base + 8) * KV_STRIDE + col);
                acc[db] = mfma32(join(lo, hi), pop[kc], acc[db]);
            }
        }
    }

    // ---- epilogue: O = acc / l, or 0 for a row with no legal key ----
    const float l_tot = sum_halves(l_part);
    const float inv = (l_tot > 0.0f) ? 1.0f / l_tot : 0.0f;
    if (my_q < Lq) {
        bf16* orow = op + (size_t)my_q * rs;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                bf16x4 out;
#pragma unroll
                for (int e = 0; e < 4; ++e) out[e] = (bf16)(acc[db][4 * rg + e] * inv);
                *(bf16x4*)(orow + 32 * db + 8 * rg + 4 * half) = out;
            }
    }
}

// ---------------------------------------------------------------------------
// fp32, d in {8, 16, 32, 64}: the accuracy path (exact fp32 FMAs, accurate
// expf).  One wave per (batch row, head, 64 queries), one query per lane;
// K/V tiles of 64 rows staged in LDS; online softmax one key at a time.
// ---------------------------------------------------------------------------
constexpr int F32_BM = 64;
constexpr int F32_BN = 64;

template <int D, bool PAD, bool CAUSAL>
__global__ __launch_bounds__(64) void attn_fwd_f32(const float* __restrict__ q,
                                                   const float* __restrict__ k,
                                                   const float* __restrict__ v,
                                                   float* __restrict__ o,
                                                   const int32_t* __restrict__ kv_lens, int B,
                                                   int H, int Lq, int Lk, int n_qtiles,
                                                   float scale) {
    __shared__ float sK[F32_BN][D + 1];
    __shared__ float sV[F32_BN][D + 1];
    const int lane = threadIdx.x;
    const int bh = (int)(blockIdx.x / n_qtiles);
    const int qt = (int)(blockIdx.x % n_qtiles);
    const int b = bh / H;
    const int hh = bh - b * H;
    const int q0 = qt * F32_BM;
    int kv_end = Lk;
    if (PAD) kv_end = min(max(kv_lens[b], 0), Lk);
    int key_end = kv_end;
    if (CAUSAL) key_end = min(key_end, min(q0 + F32_BM, Lq));

    const size_t rs = (size_t)H * D;
    const float* qp = q + ((size_t)b * Lq * H + hh) * D;
    const float* kp = k + ((size_t)b * Lk * H + hh) * D;
    const float* vp = v + ((size_t)b * Lk * H + hh) * D;
    const int my_q = q0 + lane;

    float qv[D], acc[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
        qv[c] = (my_q < Lq) ? qp[(size_t)my_q * rs + c] : 0.0f;
        acc[c] = 0.0f;
    }
    float m_run = -INFINITY, l_run = 0.0f;

    for (int k0 = 0; k0 < key_end; k0 += F32_BN) {
        __syncthreads();
        for (int idx = lane; idx < F32_BN * D; idx += 64) {
            const int row = idx / D, col = idx % D;
            const int key = k0 + row;
            const bool in = key < kv_end;
            sK[row][col] = in ? kp[(size_t)key * rs + col] : 0.0f;
            sV[row][col] = in ? vp[(size_t)key * rs + col] : 0.0f;
        }
        __syncthreads();
        const int n = min(F32_BN, key_end - k0);
        for (int j = 0; j < n; ++j) {
            const int key = k0 + j;
            if (key >= kv_end) break;
            if (CAUSAL && key > my_q) break;
            float dot = 0.0f;
#pragma unroll
            for (int c = 0; c < D; ++c) dot = __builtin_fmaf(qv[c], sK[j][c], dot);
            const float s = dot * scale;
            if (s > m_run) {
                const float alpha = expf(m_run - s);  // 0 when m_run = -inf
#pragma unroll
                for (int c = 0; c < D; ++c) acc[c] *= alpha;
                l_run *= alpha;
                m_run = s;
            }
            const float p = expf(s - m_run);
            l_run += p;
#pragma unroll
            for (int c = 0; c < D; ++c) acc[c] = __builtin_fmaf(p, sV[j][c], acc[c]);
        }
    }
    if (my_q < Lq) {
        const float inv = (l_run > 0.0f) ? 1.0f / l_run : 0.0f;
        float* orow = o + ((size_t)b * Lq * H + hh) * D + (size_t)my_q * rs;
#pragma unroll
        for (int c = 0; c < D; ++c) orow[c] = acc[c] * inv;
    }
}

template <int D>
hipError_t launch_f32_d(const AttnArgs& a, hipStream_t stream) {
    const int n_qtiles = (a.Lq + F32_BM - 1) / F32_BM;
    const dim3 grid((unsigned)((long)a.B * a.H * n_qtiles));
    const float scale = (float)(1.0 / sqrt((double)D));
    const float* q = (const float*)a.q;
    const float* k = (const float*)a.k;
    const float* v = (const float*)a.v;
    float* o = (float*)a.o;
    switch (a.mask) {
        case 0:
            hipLaunchKernelGGL((attn_fwd_f32<D, false, false>), grid, dim3(64), 0, stream, q, k, v,
                               o, a.kv_lens, a.B, a.H, a.Lq, a.Lk, n_qtiles, scale);
            break;
        case 1:
            hipLaunchKernelGGL((attn_fwd_f32<D, true, false>), grid, dim3(64), 0, stream, q, k, v,
                               o, a.kv_lens, a.B, a.H, a.Lq, a.Lk, n_qtiles, scale);
            break;
        case 2:
            hipLaunchKernelGGL((attn_fwd_f32<D, false, true>), grid, dim3(64), 0, stream, q, k, v,
                               o, a.kv_lens, a.B, a.H, a.Lq, a.Lk, n_qtiles, scale);
            break;
        default:
            hipLaunchKernelGGL((attn_fwd_f32<D, true, true>), grid, dim3(64), 0, stream, q, k, v,
                               o, a.kv_lens, a.B, a.H, a.Lq, a.Lk, n_qtiles, scale);
            break;
    }
    return hipGetLastError();
}

}  // namespace

int attention_qtile_rows(int dtype) { return dtype == 1 ? BM : F32_BM; }

hipError_t launch_attention_bf16(const AttnArgs& a, hipStream_t stream) {
    const int n_qtiles = (a.Lq + BM - 1) / BM;
    const dim3 grid((unsigned)((long)a.B * a.H * n_qtiles));
    const float sl2e = (float)(1.4426950408889634 / sqrt((double)a.D));
    const bf16* q = (const bf16*)a.q;
    const bf16* k = (const bf16*)a.k;
    const bf16* v = (const bf16*)a.v;
    bf16* o = (bf16*)a.o;
    switch (a.mask) {
        case 0:
            hipLaunchKernelGGL((attn_fwd_bf16_d64<false, false>), grid, dim3(THREADS), 0, stream,
                               q, k, v, o, a.kv_lens, a.B, a.H, a.Lq, a.Lk, n_qtiles, sl2e);
            break;
        case 1:
            hipLaunchKernelGGL((attn_fwd_bf16_d64<true, false>), grid, dim3(THREADS), 0, stream,
                               q, k, v, o, a.kv_lens, a.B, a.H, a.Lq, a.Lk, n_qtiles, sl2e);
            break;
        case 2:
            hipLaunchKernelGGL((attn_fwd_bf16_d64<false, true>), grid, dim3(THREADS), 0, stream,
                               q, k, v, o, a.kv_lens, a.B, a.H, a.Lq, a.Lk, n_qtiles, sl2e);
            break;
        default:
            hipLaunchKernelGGL((attn_fwd_bf16_d64<true, true>), grid, dim3(THREADS), 0, stream,
                               q, k, v, o, a.kv_lens, a.B, a.H, a.Lq, a.Lk, n_qtiles, sl2e);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_attention_f32(const AttnArgs& a, hipStream_t stream) {
    switch (a.D) {
        case 8: return launch_f32_d<8>(a, stream);
        case 16: return launch_f32_d<16>(a, stream);
        case 32: return launch_f32_d<32>(a, stream);
        case 64: return launch_f32_d<64>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mha
