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
    int n_probs;
};

// ---------------------------------------------------------------------------
// bf16 MFMA GEMM.  4 waves in a 2 x 2 arrangement; wave (wm, wn) owns a
// (32 TM) x (32 TN) block of the output as TM x TN accumulators of 32 x 32,
// so the workgroup tile is BM = 64 TM rows by BN = 64 TN columns; k step 64.
// The kernel computes Y^T = W^T X^T so that an accumulator column is one row
// m of Y and each lane stores 4 consecutive n (8 bytes):
//   A = W^T  (32 n x 16 k): LDS transpose reads of the row-major W tile
//   B = X^T  (16 k x 32 m): 16-byte LDS reads of the row-major X tile
// Operand tiles stream through a 3-stage LDS ring filled by direct
// global-to-LDS buffer loads (lane i of a load writes LDS bytes
// base + 16i .. base + 16i + 15), two k steps ahead of the MFMAs.  Both
// tiles are stored with their 16-byte chunks XOR-swizzled by row so the
// row reads of X and the transpose reads of W hit distinct LDS banks.
// ---------------------------------------------------------------------------
constexpr int GT = 256;

// X tile: row r holds BK/8 chunks of 16 B (k = 8c .. 8c+7), chunk c at
// position c ^ x_swz(r), so that the 16-byte row reads of 8 consecutive rows
// hit distinct banks: rows of 128 B (BK = 64) permute by r & 7, rows of 64 B
// (BK = 32) by (r >> 1) & 3.
template <int BK>
__device__ __forceinline__ int x_chunk(int r, int c) {
    return BK == 64 ? c ^ (r & 7) : c ^ ((r >> 1) & 3);
}
// W tile: row k holds BN/8 chunks (n = 8c .. 8c+7) at chunk c ^ w_swz(k).
__device__ __forceinline__ int w_swz(int k) { return (4 * (k & 3)) ^ (8 * ((k >> 3) & 1)); }


template <int TM, int TN, int ST, int BK>
__device__ __forceinline__ void gemm_bf16_body(const GemmBatch& batch, int N, int K, int n_mt,
                                               int n_nt) {
    constexpr int BM = 64 * TM;
    constexpr int BN = 64 * TN;
    static_assert(BK == 32 || BK == 64, "k step");
    constexpr int X_BYTES = BM * BK * 2;           // one X stage
    constexpr int W_BYTES = BK * BN * 2;           // one W stage
    constexpr int X_ROW_CHUNKS = BK / 8;           // 16-byte chunks per X row
    constexpr int X_ROWS_PER_KB = 64 / X_ROW_CHUNKS;
    constexpr int X_INSTR = X_BYTES / 1024 / 4;    // 1 KB loads per wave per stage
    constexpr int W_INSTR = W_BYTES / 1024 / 4;
    constexpr int W_ROW_CHUNKS = BN / 8;
    constexpr int W_ROWS_PER_INSTR = 64 / W_ROW_CHUNKS;
    static_assert(X_INSTR >= 1 && W_INSTR >= 1 && W_ROW_CHUNKS >= 16, "tile shape");

    // Tile order.  Tiles are numbered m-tile major, then problem, then
    // n-tile, so consecutive tiles share their X rows (the three projections
    // of self-attention read the same X).  Workgroups are dispatched to the
    // 8 XCDs round-robin (workgroup w on XCD w % 8); when the tile count
    // divides by 8, XCD x runs the contiguous tile range x*T/8 .. so its L2
    // keeps the X rows of the tiles in flight and the (small) weights.
    const int n_pt = batch.n_probs * n_nt;
    const int T = n_mt * n_pt;
    const int w = (int)blockIdx.x;
    const int t = (T & 7) == 0 ? (w & 7) * (T >> 3) + (w >> 3) : w;
    const int mt = t / n_pt;
    const int prob = (t % n_pt) / n_nt;
    const int nt = t % n_nt;
    const GemmProblem P = batch.p[prob];
    const int M = P.M;
    const int m0 = mt * BM;
    if (m0 >= M) return;  // uniform across the workgroup, before any barrier
    const int n0 = nt * BN;

    static_assert(ST >= 2 && ST <= 4, "ring depth");
    // One LDS allocation: the operand ring (ST X stages, then ST W stages),
    // reused after the main loop for the output tile.
    constexpr int OPITCH = 2 * BN + 16;  // output tile row pitch in bytes
    constexpr int RING_BYTES = ST * (X_BYTES + W_BYTES);
    constexpr int SMEM_BYTES = RING_BYTES > BM * OPITCH ? RING_BYTES : BM * OPITCH;
    __shared__ __attribute__((aligned(1024))) char smem[SMEM_BYTES];
    auto sX = [&](int st) { return smem + st * X_BYTES; };
    auto sW = [&](int st) { return smem + ST * X_BYTES + st * W_BYTES; };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const int g = lane >> 4;
    const int i16 = lane & 15;
    const int wn = wave & 1;
    const int wm = wave >> 1;

    // Buffer resources: X rows m0 .. M-1, W columns n0 .. (rows past the end
    // of W read as zeros; columns past N only feed outputs that are not
    // stored).
    const bf16* X = (const bf16*)P.x + (size_t)m0 * K;
    // (Only the tile's own rows are in range, so the byte range stays below
    // 2^32 whatever M is.)
    const __amdgpu_buffer_rsrc_t xr =
        make_rsrc(X, (uint32_t)((size_t)min(M - m0, BM) * K * 2));
    const bf16* W = (const bf16*)P.w + n0;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(W, (uint32_t)(((size_t)K * N - n0) * 2));

    // Per-lane source offsets of this wave's loads (k step 0), fixed per lane.
    uint32_t xoff[X_INSTR], woff[W_INSTR];
#pragma unroll
    for (int u = 0; u < X_INSTR; ++u) {
        const int t = wave + 4 * u;           // 1 KB slice of the stage
        const int r = X_ROWS_PER_KB * t + lane / X_ROW_CHUNKS;
        const int c = x_chunk<BK>(r, lane % X_ROW_CHUNKS);  // logical chunk at this position
        xoff[u] = (uint32_t)(((size_t)r * K + 8 * c) * 2);
    }
#pragma unroll
    for (int u = 0; u < W_INSTR; ++u) {
        const int t = wave + 4 * u;
        const int r = W_ROWS_PER_INSTR * t + lane / W_ROW_CHUNKS;
        const int c = (lane % W_ROW_CHUNKS) ^ w_swz(r);
        woff[u] = (uint32_t)(((size_t)r * N + 8 * c) * 2);
    }
    auto issue = [&](int kt, int st) {  // direct loads of k step kt into stage st
        const uint32_t xs = lds_addr(sX(st));
        const uint32_t ws = lds_addr(sW(st));
        const uint32_t xk = (uint32_t)kt * BK * 2;
        const uint32_t wk = (uint32_t)((size_t)kt * BK * N * 2);
#pragma unroll
        for (int u = 0; u < X_INSTR; ++u)
            load_lds16(xr, xs + (wave + 4 * u) * 1024, xoff[u] + xk);
#pragma unroll
        for (int u = 0; u < W_INSTR; ++u)
            load_lds16(wr, ws + (wave + 4 * u) * 1024, woff[u] + wk);
    };

    f32x16 acc[TN][TM];
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int c = 0; c < TM; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][c][r] = 0.0f;

    constexpr int PER_STAGE = X_INSTR + W_INSTR;
    const int n_k = K / BK;

    // LDS operand reads of one 16-wide k slice of stage st.
    auto read_ops = [&](int st, int k16, bf16x8 (&a)[TN], bf16x8 (&bx)[TM]) {
        const char* xs = sX(st);
        const char* ws = sW(st);
        const int krow = 16 * k16 + 8 * (g >> 1) + (i16 >> 2);
#pragma unroll
        for (int nb = 0; nb < TN; ++nb) {
            const int n = 32 * TN * wn + 32 * nb + 16 * (g & 1) + 4 * (i16 & 3);
            const int c = n >> 3, byte = (n & 7) * 2;
            const bf16* lo =
                (const bf16*)(ws + krow * (2 * BN) + ((c ^ w_swz(krow)) << 4) + byte);
            const bf16* hi = (const bf16*)(ws + (krow + 4) * (2 * BN) +
                                           ((c ^ w_swz(krow + 4)) << 4) + byte);
            a[nb] = join(lds_read_tr(lo), lds_read_tr(hi));
        }
#pragma unroll
        for (int mb = 0; mb < TM; ++mb) {
            const int r = 32 * TM * wm + 32 * mb + l32;
            bx[mb] = *(const bf16x8*)(xs + r * (2 * BK) + (x_chunk<BK>(r, 2 * k16 + half) << 4));
        }
    };
    auto mfmas = [&](const bf16x8 (&a)[TN], const bf16x8 (&bx)[TM]) {
#pragma unroll
        for (int nb = 0; nb < TN; ++nb)
#pragma unroll
            for (int mb = 0; mb < TM; ++mb) acc[nb][mb] = mfma32(a[nb], bx[mb], acc[nb][mb]);
    };

    // One k step: wait for this wave's loads of step kt (up to ST-2 later
    // steps may still fly), barrier (every wave's loads visible; the stage
    // of step kt-1 is free), start step kt+ST-1 into that stage, then the
    // four k slices with the operand reads of slice i+1 in flight while the
    // MFMAs of slice i run.
    bf16x8 opA[2][TN], opB[2][TM];
    auto step = [&](int kt, int st) {
        const int ahead = min(ST - 2, n_k - 1 - kt);
        if (ahead >= 2) wait_vmcnt<2 * PER_STAGE>();
        else if (ahead == 1) wait_vmcnt<PER_STAGE>();
        else wait_vmcnt<0>();
        barrier_lds();
        if (kt + ST - 1 < n_k) issue(kt + ST - 1, (st + ST - 1) % ST);
        read_ops(st, 0, opA[0], opB[0]);
#pragma unroll
        for (int k16 = 0; k16 < BK / 16; ++k16) {
            __builtin_amdgcn_sched_barrier(0);
            if (k16 + 1 < BK / 16) read_ops(st, k16 + 1, opA[(k16 + 1) & 1], opB[(k16 + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
            mfmas(opA[k16 & 1], opB[k16 & 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

#pragma unroll
    for (int s = 0; s < ST - 1; ++s)
        if (s < n_k) issue(s, s);
    for (int kt = 0; kt < n_k; kt += ST) {
#pragma unroll
        for (int s = 0; s < ST; ++s)
            if (kt + s < n_k) step(kt + s, s);
    }

    // Epilogue: the output tile goes through LDS (reusing the operand ring)
    // so that global stores are whole 16-byte chunks of contiguous row
    // segments rather than 8-byte pieces scattered over 32 rows.  The pitch
    // of 2*BN + 16 bytes spreads a column of 8-byte writes over the banks.
    barrier_lds();  // every wave is done reading the operand ring
    char* so = smem;
#pragma unroll
    for (int mb = 0; mb < TM; ++mb) {
        const int r = 32 * TM * wm + 32 * mb + l32;
#pragma unroll
        for (int nb = 0; nb < TN; ++nb)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int n = 32 * TN * wn + 32 * nb + 8 * rg + 4 * half;
                bf16x4 out;
#pragma unroll
                for (int e = 0; e < 4; ++e) out[e] = (bf16)acc[nb][mb][4 * rg + e];
                *(bf16x4*)(so + r * OPITCH + n * 2) = out;
            }
    }
    barrier_lds();
    bf16* Y = (bf16*)P.y;
    constexpr int ROW_CHUNKS = BN / 8;  // 16-byte chunks per tile row
#pragma unroll
    for (int it = 0; it < BM * ROW_CHUNKS / GT; ++it) {
        const int idx = tid + GT * it;
        const int r = idx / ROW_CHUNKS, c = idx % ROW_CHUNKS;
        const int m = m0 + r, n = n0 + 8 * c;
        if (m < M && n < N)
            store_stream((bf16x8*)(Y + (size_t)m * N + n), *(const bf16x8*)(so + r * OPITCH + c * 16));
    }
}

// The two uses get their own kernel names so traces and counters tell them
// apart.
template <int TM, int TN, int ST, int BK, int OCC>
__global__ __launch_bounds__(GT, OCC) void qkv_projection_gemm(GemmBatch batch, int N, int K,
                                                               int n_mt, int n_nt) {
    gemm_bf16_body<TM, TN, ST, BK>(batch, N, K, n_mt, n_nt);
}

template <int TM, int TN, int ST, int BK, int OCC>
__global__ __launch_bounds__(GT, OCC) void out_projection_gemm(GemmBatch batch, int N, int K,
                                                               int n_mt, int n_nt) {
    gemm_bf16_body<TM, TN, ST, BK>(batch, N, K, n_mt, n_nt);
}

// ---------------------------------------------------------------------------
// fp32 GEMM (accuracy path) on the matrix cores: v_mfma_f32_32x32x2_f32
// (fp32 operands, fp32 accumulation).  64 x 64 output tile per workgroup,
// wave (wm, wn) owning the 32 x 32 block at (32 wm, 32 wn); k step 32.
// At MFMA step s (0..15) lane (i, h = lane / 32) feeds X[m = i][k = 16 h + s]
// (A, 16-byte LDS reads of consecutive k) and W[k = 16 h + s][n = i] (B).
// The next k step's tiles are loaded into registers while the MFMAs of this
// one run, then stored to LDS between two barriers.  Rows past M read as
// zeros and are not stored.
// ---------------------------------------------------------------------------
constexpr int F32G_BK = 32;
constexpr int F32G_XP = F32G_BK + 4;  // X tile row pitch (floats): rows 16 B apart in bank
constexpr int F32G_WP = 64 + 4;       // W tile row pitch (floats)

__global__ __launch_bounds__(256, 2) void gemm_f32_kernel(GemmBatch batch, int N, int K) {
    const GemmProblem P = batch.p[blockIdx.z];
    const int M = P.M;
    const int m0 = blockIdx.x * 64;
    if (m0 >= M) return;  // uniform across the workgroup, before any barrier
    const int n0 = blockIdx.y * 64;
    const float* X = (const float*)P.x;
    const float* W = (const float*)P.w;
    float* Y = (float*)P.y;
    __shared__ __attribute__((aligned(16))) float sX[64 * F32G_XP];
    __shared__ __attribute__((aligned(16))) float sW[F32G_BK * F32G_WP];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int i = lane & 31;
    const int h = lane >> 5;
    const int wm = wave >> 1, wn = wave & 1;

    // Tile loads: X is 64 rows x 8 chunks of 4 floats, W 32 rows x 16 chunks;
    // thread tid takes chunks tid and tid + 256 of each.
    float4 xr[2], wr[2];
    auto load = [&](int k0) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int cx = tid + 256 * u;
            const int row = cx >> 3, c = cx & 7;
            float4 z = {0.0f, 0.0f, 0.0f, 0.0f};
            if (m0 + row < M) z = *(const float4*)(X + (size_t)(m0 + row) * K + k0 + 4 * c);
            xr[u] = z;
            const int cw = tid + 256 * u;
            const int wrow = cw >> 4, wc = cw & 15;
            wr[u] = *(const float4*)(W + (size_t)(k0 + wrow) * N + n0 + 4 * wc);
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int cx = tid + 256 * u;
            *(float4*)(sX + (cx >> 3) * F32G_XP + 4 * (cx & 7)) = xr[u];
            *(float4*)(sW + (cx >> 4) * F32G_WP + 4 * (cx & 15)) = wr[u];
        }
    };

    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    load(0);
    for (int k0 = 0; k0 < K; k0 += F32G_BK) {
        __syncthreads();  // every wave is done with the previous tiles
        store();
        __syncthreads();
        if (k0 + F32G_BK < K) load(k0 + F32G_BK);
        const float* xa = sX + (32 * wm + i) * F32G_XP + 16 * h;
        const float* wb = sW + (16 * h) * F32G_WP + 32 * wn + i;
#pragma unroll
        for (int s = 0; s < 16; s += 4) {
            const float4 a = *(const float4*)(xa + s);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, wb[s * F32G_WP], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, wb[(s + 1) * F32G_WP], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, wb[(s + 2) * F32G_WP], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, wb[(s + 3) * F32G_WP], acc, 0, 0, 0);
        }
    }
    // Lane (i, h) holds Y[m0 + 32 wm + acc_row(r, h)][n0 + 32 wn + i] in
    // register r: each store writes 32 consecutive floats of a row.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int m = m0 + 32 * wm + acc_row(r, h);
        if (m < M) Y[(size_t)m * N + n0 + 32 * wn + i] = acc[r];
    }
}

GemmBatch make_batch(const GemmProblem* probs, int n, int* max_m) {
    GemmBatch b{};
    b.n_probs = n;
    *max_m = 0;
    for (int i = 0; i < n; ++i) {
        b.p[i] = probs[i];
        if (probs[i].M > *max_m) *max_m = probs[i].M;
    }
    return b;
}

}  // namespace

template <int TM, int TN, int ST, int BK, int OCC>
hipError_t launch_bf16_tiles(const GemmBatch& batch, int max_m, int N, int K, bool qkv,
                             hipStream_t stream) {
    const int n_mt = (max_m + 64 * TM - 1) / (64 * TM);
    const int n_nt = (N + 64 * TN - 1) / (64 * TN);
    const dim3 grid((unsigned)((long)n_mt * n_nt * batch.n_probs));
    if (qkv)
        hipLaunchKernelGGL((qkv_projection_gemm<TM, TN, ST, BK, OCC>), grid, dim3(GT), 0, stream,
                           batch, N, K, n_mt, n_nt);
    else
        hipLaunchKernelGGL((out_projection_gemm<TM, TN, ST, BK, OCC>), grid, dim3(GT), 0, stream,
                           batch, N, K, n_mt, n_nt);
    return hipGetLastError();
}

hipError_t launch_gemm_bf16(const GemmProblem* probs, int n_probs, int N, int K, bool qkv,
                            hipStream_t stream) {
    int max_m;
    const GemmBatch batch = make_batch(probs, n_probs, &max_m);
    // 128 x 128 tiles.  With more than one tile per CU, a k step of 32 and a
    // 3-stage ring (48 KB of LDS) let three workgroups share a CU, so up to
    // 768 tiles run in a single round and hide each other's load latency;
    // otherwise one workgroup per CU streams k steps of 64.
    const long tiles = (long)((max_m + 127) / 128) * ((N + 127) / 128) * n_probs;
    if (tiles > 256) return launch_bf16_tiles<2, 2, 3, 32, 3>(batch, max_m, N, K, qkv, stream);
    return launch_bf16_tiles<2, 2, 3, 64, 1>(batch, max_m, N, K, qkv, stream);
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
