// gemm.hip -- the linear maps of multi-head attention on gfx950:
//
//   Q = X_q W^Q, K = X_kv W^K, V = X_kv W^V     (all heads at once)
//   Y = Concat(head_1, ..., head_h) W^O
//
// ("Attention Is All You Need -- A Revolutionary Architecture for Sequence
// Transduction", slide "Multi-Head Attention"; "Paper Deep Reading", section
// 04, MultiHead equations.)  Every one is Y[M, N] = X[M, K] W[K, N] with
// row-major operands and no bias; the [M, N] result with N = h*d is already
// the BLHD layout (head t in column block t).  Up to three problems with the
// same N and K run in one launch (grid z), which is how the three
// projections share a single launch.
#include "device.h"
#include "launch.h"

namespace mha {
namespace {

struct GemmBatch {
    GemmProblem p[3];
};

// ---------------------------------------------------------------------------
// bf16 MFMA GEMM.  Workgroup tile 128 (m) x 128 (n), k step 64; 4 waves in a
// 2 x 2 arrangement, each owning 64 x 64 of the output as 2 x 2 blocks of
// 32 x 32.  The kernel computes Y^T = W^T X^T so that an accumulator column
// is one row m of Y and each lane stores 4 consecutive n (8 bytes):
//   A = W^T  (32 n x 16 k): LDS transpose reads of the row-major W tile
//   B = X^T  (16 k x 32 m): 16-byte LDS reads of the row-major X tile
// ---------------------------------------------------------------------------
constexpr int GBM = 128;
constexpr int GBN = 128;
constexpr int GBK = 64;
constexpr int XS = GBK + 8;   // LDS pitch of the X tile [m][k], elements (144 B)
constexpr int WS = GBN + 8;   // LDS pitch of the W tile [k][n], elements (272 B)
constexpr int GT = 256;

__global__ __launch_bounds__(GT, 2) void gemm_bf16_kernel(GemmBatch batch, int N, int K) {
    const GemmProblem P = batch.p[blockIdx.z];
    const int M = P.M;
    const int m0 = blockIdx.x * GBM;
    if (m0 >= M) return;  // uniform across the workgroup, before any barrier
    const int n0 = blockIdx.y * GBN;
    const bf16* X = (const bf16*)P.x;
    const bf16* W = (const bf16*)P.w;
    bf16* Y = (bf16*)P.y;

    __shared__ __attribute__((aligned(16))) bf16 sX[GBM * XS];
    __shared__ __attribute__((aligned(16))) bf16 sW[GBK * WS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const int g = lane >> 4;
    const int i16 = lane & 15;
    const int wn = wave & 1;
    const int wm = wave >> 1;

    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][c][r] = 0.0f;

    bf16x8 xr[4], wr[4];
    auto gload = [&](int k0) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = tid + GT * u;
            const int xrow = c >> 3, xcol = (c & 7) * 8;
            xr[u] = (m0 + xrow < M) ? *(const bf16x8*)(X + (size_t)(m0 + xrow) * K + k0 + xcol)
                                    : zero_bf16x8();
            const int wrow = c >> 4, wcol = (c & 15) * 8;
            wr[u] = (n0 + wcol < N) ? *(const bf16x8*)(W + (size_t)(k0 + wrow) * N + n0 + wcol)
                                    : zero_bf16x8();
        }
    };
    auto sstore = [&]() {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = tid + GT * u;
            *(bf16x8*)(sX + (c >> 3) * XS + (c & 7) * 8) = xr[u];
            *(bf16x8*)(sW + (c >> 4) * WS + (c & 15) * 8) = wr[u];
        }
    };

    const int n_k = K / GBK;
    gload(0);
    for (int kt = 0; kt < n_k; ++kt) {
        __syncthreads();
        sstore();
        __syncthreads();
        if (kt + 1 < n_k) gload((kt + 1) * GBK);
#pragma unroll
        for (int k16 = 0; k16 < GBK / 16; ++k16) {
            bf16x8 a[2], bx[2];
            const int krow = 16 * k16 + 8 * (g >> 1) + (i16 >> 2);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const int col = 64 * wn + 32 * nb + 16 * (g & 1) + 4 * (i16 & 3);
                a[nb] = join(lds_read_tr(sW + krow * WS + col),
                             lds_read_tr(sW + (krow + 4) * WS + col));
            }
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
                bx[mb] = *(const bf16x8*)(sX + (64 * wm + 32 * mb + l32) * XS + 16 * k16 +
                                          8 * half);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) acc[nb][mb] = mfma32(a[nb], bx[mb], acc[nb][mb]);
        }
    }

#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int m = m0 + 64 * wm + 32 * mb + l32;
        if (m >= M) continue;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int n = n0 + 64 * wn + 32 * nb + 8 * rg + 4 * half;
                if (n >= N) continue;
                bf16x4 out;
#pragma unroll
                for (int e = 0; e < 4; ++e) out[e] = (bf16)acc[nb][mb][4 * rg + e];
                *(bf16x4*)(Y + (size_t)m * N + n) = out;
            }
    }
}

// ---------------------------------------------------------------------------
// fp32 GEMM (accuracy path): 64 x 64 tile, k step 16, each thread 4 x 4
// outputs with exact fp32 FMAs.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmBatch batch, int N, int K) {
    const GemmProblem P = batch.p[blockIdx.z];
    const int M = P.M;
    const int m0 = blockIdx.x * 64;
    if (m0 >= M) return;
    const int n0 = blockIdx.y * 64;
    const float* X = (const float*)P.x;
    const float* W = (const float*)P.w;
    float* Y = (float*)P.y;
    __shared__ float sX[64][17];
    __shared__ float sW[16][65];
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += 16) {
        __syncthreads();
        for (int u = 0; u < 4; ++u) {
            const int idx = tid + 256 * u;
            const int xr = idx >> 4, xc = idx & 15;
            sX[xr][xc] = (m0 + xr < M) ? X[(size_t)(m0 + xr) * K + k0 + xc] : 0.0f;
            const int wr = idx >> 6, wc = idx & 63;
            sW[wr][wc] = (n0 + wc < N) ? W[(size_t)(k0 + wr) * N + n0 + wc] : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = sX[ty * 4 + i][kk];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = sW[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + ty * 4 + i;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx * 4 + j;
            if (n < N) Y[(size_t)m * N + n] = acc[i][j];
        }
    }
}

GemmBatch make_batch(const GemmProblem* probs, int n, int* max_m) {
    GemmBatch b{};
    *max_m = 0;
    for (int i = 0; i < n; ++i) {
        b.p[i] = probs[i];
        if (probs[i].M > *max_m) *max_m = probs[i].M;
    }
    return b;
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmProblem* probs, int n_probs, int N, int K,
                            hipStream_t stream) {
    int max_m;
    const GemmBatch batch = make_batch(probs, n_probs, &max_m);
    const dim3 grid((unsigned)((max_m + GBM - 1) / GBM), (unsigned)((N + GBN - 1) / GBN),
                    (unsigned)n_probs);
    hipLaunchKernelGGL(gemm_bf16_kernel, grid, dim3(GT), 0, stream, batch, N, K);
    return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmProblem* probs, int n_probs, int N, int K,
                           hipStream_t stream) {
    int max_m;
    const GemmBatch batch = make_batch(probs, n_probs, &max_m);
    const dim3 grid((unsigned)((max_m + 63) / 64), (unsigned)((N + 63) / 64), (unsigned)n_probs);
    hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, stream, batch, N, K);
    return hipGetLastError();
}

}  // namespace mha
