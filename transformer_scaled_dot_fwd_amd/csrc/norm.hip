// norm.hip -- the attention sub-layer's output with its residual connection
// and post-norm in one kernel:
//
//   out = LayerNorm(x + Concat(head_1, ..., head_h) W^O)
//
// ("Paper Deep Reading", section 03, residual + LayerNorm in post-norm
// order, and section 04, MultiHead equation; slide "Encoder Architecture".
// Layer normalisation per row over the d_model features: population
// variance, gain gamma, bias beta, eps inside the square root.)
//
// A workgroup of 8 waves owns 32 whole output rows (all d_model columns), so
// the row statistics never leave it: wave w computes features
// 32 NB w .. 32 NB w + 32 NB - 1 of the rows as NB accumulators of 32 x 32
// (Y^T = W^T X^T as in the projection GEMM: A = W^T by LDS transpose reads of
// the shared W tile, B = X^T by 16-byte LDS reads of the X tile; both tiles
// stream through an LDS ring filled by direct global-to-LDS loads).  The
// product stays in fp32 through the residual add; each wave takes the mean
// and the squared deviations of its share of every row, the eight shares are
// merged through LDS, and the normalised tile is staged in LDS and written
// as whole rows.  The residual rows are fetched at the start, with the
// first operand tiles.
#include "device.h"
#include "launch.h"

namespace mha {
namespace {

constexpr int NM_BM = 32;   // rows per workgroup
constexpr int NM_BK = 32;   // k step
constexpr int NM_WAVES = 8;

// X tile: row r (64 bytes, 4 chunks of 16) holds chunk c at c ^ ((r >> 1) & 3).
__device__ __forceinline__ int nm_x_chunk(int r, int c) { return c ^ ((r >> 1) & 3); }
// W tile: row k holds its chunks (8 features each) at chunk c ^ nm_w_swz(k).
__device__ __forceinline__ int nm_w_swz(int k) { return (4 * (k & 3)) ^ (8 * ((k >> 3) & 1)); }

template <int NB>
constexpr int nm_stages() { return NB >= 4 ? 2 : 3; }
template <int NB>
constexpr int nm_smem() {
    constexpr int N = 256 * NB;
    constexpr int ring = nm_stages<NB>() * (NM_BM * NM_BK * 2 + NM_BK * N * 2);
    constexpr int stage_out = NM_BM * (2 * N + 16);
    return ring > stage_out ? ring : stage_out;
}

// xres and out may be the same buffer (the residual stream updated in
// place), so neither is declared __restrict__; each workgroup reads its rows
// of xres before it writes them.
template <int NB>
__global__ __launch_bounds__(64 * NM_WAVES, 1) void out_proj_post_norm_bf16(
    const bf16* __restrict__ o, const bf16* __restrict__ w, const bf16* xres,
    const bf16* __restrict__ gamma, const bf16* __restrict__ beta, bf16* out, int M, int K,
    float eps) {
    constexpr int N = 256 * NB;                     // d_model
    constexpr int ST = nm_stages<NB>();
    constexpr int X_BYTES = NM_BM * NM_BK * 2;      // 2 KB
    constexpr int W_BYTES = NM_BK * N * 2;          // 16 KB per NB
    constexpr int X_INSTR = X_BYTES / 1024;         // issued by wave 0
    constexpr int W_INSTR = W_BYTES / 1024 / NM_WAVES;
    constexpr int OPITCH = 2 * N + 16;              // output staging pitch (bytes)
    static_assert(W_INSTR >= 1 && W_INSTR * 1024 * NM_WAVES == W_BYTES, "W load split");
    __shared__ __attribute__((aligned(1024))) char smem[nm_smem<NB>()];
    __shared__ float2 red[NM_WAVES][NM_BM];
    constexpr int GB_BYTES = 2 * N > 1024 ? 2 * N : 1024;  // gamma, then beta, in LDS
    __shared__ __attribute__((aligned(1024))) char s_gb[2 * GB_BYTES];
    __shared__ __attribute__((aligned(16))) float s_gbf[2][N];  // the same in fp32

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const int g = lane >> 4;
    const int i16 = lane & 15;
    const int m0 = (int)blockIdx.x * NM_BM;

    auto sX = [&](int st) { return smem + st * X_BYTES; };
    auto sW = [&](int st) { return smem + ST * X_BYTES + st * W_BYTES; };

    // Buffer resources: the tile's rows of O (rows past M read as zeros) and
    // the whole of W^O.
    const bf16* X = o + (size_t)m0 * K;
    const __amdgpu_buffer_rsrc_t xr =
        make_rsrc(X, (uint32_t)((size_t)min(M - m0, NM_BM) * K * 2));
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, (uint32_t)((size_t)K * N * 2));
    uint32_t xoff[X_INSTR], woff[W_INSTR];
#pragma unroll
    for (int u = 0; u < X_INSTR; ++u) {
        const int r = 16 * u + (lane >> 2);
        xoff[u] = (uint32_t)((r * K + 8 * nm_x_chunk(r, lane & 3)) * 2);
    }
#pragma unroll
    for (int u = 0; u < W_INSTR; ++u) {
        const int t = wave + NM_WAVES * u;  // 1 KB slice of the stage
        const int byte = 1024 * t + 16 * lane;
        const int r = byte / (2 * N);
        const int c = (byte % (2 * N)) / 16;
        woff[u] = (uint32_t)(((size_t)r * N + 8 * (c ^ nm_w_swz(r))) * 2);
    }
    auto issue = [&](int kt, int st) {
        if (wave == 0) {
            const uint32_t xs = lds_addr(sX(st));
#pragma unroll
            for (int u = 0; u < X_INSTR; ++u)
                load_lds16(xr, xs + 1024 * u, xoff[u] + (uint32_t)kt * NM_BK * 2);
        }
        const uint32_t ws = lds_addr(sW(st));
        const uint32_t wk = (uint32_t)((size_t)kt * NM_BK * N * 2);
#pragma unroll
        for (int u = 0; u < W_INSTR; ++u)
            load_lds16(wr, ws + 1024 * (wave + NM_WAVES * u), woff[u] + wk);
    };

    // Gain and bias go to LDS by direct loads of wave 0, issued before any
    // other load, so the first ring wait (and its barrier) covers them and
    // the epilogue does not wait on global memory for them.
    if (wave == 0) {
        const __amdgpu_buffer_rsrc_t gr = make_rsrc(gamma, (uint32_t)(N * 2));
        const __amdgpu_buffer_rsrc_t br = make_rsrc(beta, (uint32_t)(N * 2));
#pragma unroll
        for (int u = 0; u < GB_BYTES / 1024; ++u) {
            load_lds16(gr, lds_addr(s_gb) + 1024 * u, (uint32_t)(1024 * u + 16 * lane));
            load_lds16(br, lds_addr(s_gb + GB_BYTES) + 1024 * u,
                       (uint32_t)(1024 * u + 16 * lane));
        }
    }

    // The residual rows, prefetched whole (16 bytes per lane, consecutive
    // lanes along a row) while the product runs; rows past M read as zeros
    // (range-checked buffer loads: no branch, so nothing waits for them
    // before the product's loads are issued).
    constexpr int ROW_CHUNKS = N / 8;                          // 16-byte chunks per row
    constexpr int X_PER_LANE = NM_BM * ROW_CHUNKS / (64 * NM_WAVES);
    const __amdgpu_buffer_rsrc_t xrr = make_rsrc(
        xres + (size_t)m0 * N, (uint32_t)((size_t)min(M - m0, NM_BM) * N * 2));
    bf16x8 xres_v[X_PER_LANE];
#pragma unroll
    for (int it = 0; it < X_PER_LANE; ++it) {
        const int idx = tid + 64 * NM_WAVES * it;
        xres_v[it] = buffer_load16(xrr, (uint32_t)(16 * idx));
    }

    f32x16 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[nb][r] = 0.0f;

    auto read_ops = [&](int st, int k16, bf16x8 (&a)[NB], bf16x8& bx) {
        const char* ws = sW(st);
        const char* xs = sX(st);
        const int krow = 16 * k16 + 8 * (g >> 1) + (i16 >> 2);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int n = 32 * NB * wave + 32 * nb + 16 * (g & 1) + 4 * (i16 & 3);
            const int c = n >> 3, byte = (n & 7) * 2;
            const bf16* lo =
                (const bf16*)(ws + krow * (2 * N) + ((c ^ nm_w_swz(krow)) << 4) + byte);
            const bf16* hi = (const bf16*)(ws + (krow + 4) * (2 * N) +
                                           ((c ^ nm_w_swz(krow + 4)) << 4) + byte);
            a[nb] = join(lds_read_tr(lo), lds_read_tr(hi));
        }
        bx = *(const bf16x8*)(xs + l32 * (2 * NM_BK) + (nm_x_chunk(l32, 2 * k16 + half) << 4));
    };

    // k steps: wait for this wave's loads of step kt (later steps may fly),
    // barrier (every wave's loads visible; step kt-1's stage is free), start
    // step kt + ST - 1, then the two 16-wide slices.
    const int n_k = K / NM_BK;
    auto step = [&](int kt, int st) {
        const int ahead = min(ST - 2, n_k - 1 - kt);
        if (ahead >= 1) {
            if (wave == 0) wait_vmcnt<X_INSTR + W_INSTR>();
            else wait_vmcnt<W_INSTR>();
        } else {
            wait_vmcnt<0>();
        }
        barrier_lds();
        if (kt + ST - 1 < n_k) issue(kt + ST - 1, (st + ST - 1) % ST);
        bf16x8 a0[NB], a1[NB], b0, b1;
        read_ops(st, 0, a0, b0);
        read_ops(st, 1, a1, b1);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = mfma32(a0[nb], b0, acc[nb]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = mfma32(a1[nb], b1, acc[nb]);
    };
#pragma unroll
    for (int s = 0; s < ST - 1; ++s)
        if (s < n_k) issue(s, s);
    for (int kt = 0; kt < n_k; kt += ST) {
#pragma unroll
        for (int s = 0; s < ST; ++s)
            if (kt + s < n_k) step(kt + s, s);
    }

    // ---- residual, row statistics, normalisation ----
    // Lane (l32, half) holds row m0 + l32 and features
    // f(nb, r) = 32 NB wave + 32 nb + 8 (r / 4) + 4 half + r % 4.  The
    // residual tile goes through LDS (row layout, pitch OPITCH; the ring is
    // free once every wave has passed the barrier) to the accumulator
    // layout.
    const int f0 = 32 * NB * wave + 4 * half;
    char* so = smem;
    barrier_lds();
#pragma unroll
    for (int it = 0; it < X_PER_LANE; ++it) {
        const int idx = tid + 64 * NM_WAVES * it;
        const int r = idx / ROW_CHUNKS, c = idx % ROW_CHUNKS;
        *(bf16x8*)(so + r * OPITCH + 16 * c) = xres_v[it];
    }
    // Gain and bias are converted to fp32 once per workgroup (a lane then
    // reads its features' values, the same for all 32 rows, as float4s).
    for (int f = tid; f < N; f += 64 * NM_WAVES) {
        s_gbf[0][f] = (float)((const bf16*)s_gb)[f];
        s_gbf[1][f] = (float)((const bf16*)(s_gb + GB_BYTES))[f];
    }
    barrier_lds();
    // acc += x, one exact dot step per element: x * 1 + x' * 0 + acc.  The
    // selectors are kept in registers: as an operand constant, bf16 (1, 0)
    // would be encoded as the inline constant 1.0, which this instruction
    // reads as the fp32 bit pattern, i.e. as (0, 1).
    bf16x2 pick_lo = {(bf16)1.0f, (bf16)0.0f}, pick_hi = {(bf16)0.0f, (bf16)1.0f};
    asm volatile("" : "+v"(pick_lo), "+v"(pick_hi));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const bf16x4 xv = *(const bf16x4*)(so + l32 * OPITCH + 2 * (f0 + 32 * nb + 8 * rg));
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
                const bf16x2 xp = {xv[e], xv[e + 1]};
                acc[nb][4 * rg + e] =
                    __builtin_amdgcn_fdot2_f32_bf16(xp, pick_lo, acc[nb][4 * rg + e], false);
                acc[nb][4 * rg + e + 1] =
                    __builtin_amdgcn_fdot2_f32_bf16(xp, pick_hi, acc[nb][4 * rg + e + 1], false);
            }
        }
    // Row statistics.  Each wave takes the mean and the sum of squared
    // deviations of its 32 NB features of the row (two passes over
    // registers, the row's lane pair combined by a half swap); the eight
    // partial results are merged through LDS with the pairwise update of
    // Chan, Golub and LeVeque (equal counts n_w):
    //   mu = mean of the mu_w,  M2 = sum M2_w + n_w sum (mu_w - mu)^2.
    constexpr float inv_nw = 1.0f / (32 * NB);
    float s1 = 0.0f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s1 += acc[nb][r];
    const float mu_w = sum_halves(s1) * inv_nw;
    float s2 = 0.0f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float dz = acc[nb][r] - mu_w;
            s2 = __builtin_fmaf(dz, dz, s2);
        }
    const float m2_w = sum_halves(s2);
    if (half == 0) red[wave][l32] = make_float2(mu_w, m2_w);
    barrier_lds();
    float2 part[NM_WAVES];
    float mu = 0.0f;
#pragma unroll
    for (int ww = 0; ww < NM_WAVES; ++ww) {
        part[ww] = red[ww][l32];
        mu += part[ww].x;
    }
    mu *= 1.0f / NM_WAVES;
    float m2 = 0.0f, dev = 0.0f;
#pragma unroll
    for (int ww = 0; ww < NM_WAVES; ++ww) {
        m2 += part[ww].y;
        const float dm = part[ww].x - mu;
        dev = __builtin_fmaf(dm, dm, dev);
    }
    const float var = __builtin_fmaf(dev, 32.0f * NB, m2) * (1.0f / N);
    const float inv = 1.0f / sqrtf(var + eps);

    // Each lane overwrites the residual elements it read with its outputs.
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const int f = f0 + 32 * nb + 8 * rg;
            const float4 gf = *(const float4*)&s_gbf[0][f];
            const float4 bf = *(const float4*)&s_gbf[1][f];
            const float gg[4] = {gf.x, gf.y, gf.z, gf.w}, bb[4] = {bf.x, bf.y, bf.z, bf.w};
            bf16x4 y;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                y[e] = (bf16)__builtin_fmaf(gg[e], (acc[nb][4 * rg + e] - mu) * inv, bb[e]);
            *(bf16x4*)(so + l32 * OPITCH + 2 * (f0 + 32 * nb + 8 * rg)) = y;
        }
    barrier_lds();
#pragma unroll
    for (int it = 0; it < X_PER_LANE; ++it) {
        const int idx = tid + 64 * NM_WAVES * it;
        const int r = idx / ROW_CHUNKS, c = idx % ROW_CHUNKS;
        if (m0 + r < M)
            store_stream((bf16x8*)(out + (size_t)(m0 + r) * N + 8 * c),
                         *(const bf16x8*)(so + r * OPITCH + 16 * c));
    }
}

template <int NB>
hipError_t launch_post_norm_d(const PostNormArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)((a.M + NM_BM - 1) / NM_BM));
    hipLaunchKernelGGL((out_proj_post_norm_bf16<NB>), grid, dim3(64 * NM_WAVES), 0, stream,
                       (const bf16*)a.o, (const bf16*)a.w, (const bf16*)a.x,
                       (const bf16*)a.gamma, (const bf16*)a.beta, (bf16*)a.out, a.M, a.K,
                       a.eps);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp32 (accuracy path): the same computation on the matrix cores
// (v_mfma_f32_32x32x2_f32: fp32 products and accumulation), for any h*d_v.
// A workgroup of 4 waves owns 32 whole rows; wave w holds columns
// w N/4 .. (w+1) N/4 - 1 as N/128 accumulators of 32 x 32 (lane (i, h =
// lane / 32) holds column i of each block, rows (r % 4) + 8 (r / 4) + 4h).
// k steps of 8 through LDS: at MFMA step s lane half h feeds k = 4h + s of
// the step, O[row i][k] (A) and W^O[k][column i] (B); past K both tiles
// hold zeros.  The next step's tiles are loaded into registers while the
// MFMAs of this one run.  The row statistics are two passes (mean, then
// squared deviations), reduced over each half-wave's 32 lanes and then
// over the four waves through LDS.
// ---------------------------------------------------------------------------
constexpr int NF_R = 32;   // rows per workgroup
constexpr int NF_KS = 8;   // k step
constexpr int NF_OP = NF_KS + 4;  // O tile row pitch (floats)

template <int NPT>
__global__ __launch_bounds__(256) void out_proj_post_norm_f32(
    const float* __restrict__ o, const float* __restrict__ w, const float* xres,
    const float* __restrict__ gamma, const float* __restrict__ beta, float* out, int M, int K,
    float eps) {
    constexpr int N = 256 * NPT;
    constexpr int NB = N / 128;       // 32-column blocks per wave
    constexpr int WP = N + 4;         // W tile row pitch (floats)
    constexpr int WC = NF_KS * N / 4 / 256;  // float4 chunks of the W tile per thread
    __shared__ __attribute__((aligned(16))) float so[NF_R * NF_OP];
    __shared__ __attribute__((aligned(16))) float sw[NF_KS * WP];
    __shared__ float red[4][NF_R];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int i = lane & 31;
    const int h = lane >> 5;
    const int m0 = (int)blockIdx.x * NF_R;
    const int rows = min(NF_R, M - m0);
    const int c0 = wave * (N / 4);    // this wave's first column

    // Tile loads of k step k0: thread t takes O[m0 + t / 8][k0 + t % 8] and
    // the W^O chunks t, t + 256, ... (row c / (N / 4), 4 floats each).
    float oreg;
    float4 wreg[WC];
    auto load = [&](int k0) {
        const int r = tid >> 3, kk = k0 + (tid & 7);
        oreg = (r < rows && kk < K) ? o[(size_t)(m0 + r) * K + kk] : 0.0f;
#pragma unroll
        for (int u = 0; u < WC; ++u) {
            const int c = tid + 256 * u;
            const int wr = c / (N / 4), wc = c % (N / 4);
            float4 z = {0.0f, 0.0f, 0.0f, 0.0f};
            if (k0 + wr < K) z = *(const float4*)(w + (size_t)(k0 + wr) * N + 4 * wc);
            wreg[u] = z;
        }
    };
    auto store = [&]() {
        so[(tid >> 3) * NF_OP + (tid & 7)] = oreg;
#pragma unroll
        for (int u = 0; u < WC; ++u) {
            const int c = tid + 256 * u;
            *(float4*)(sw + (c / (N / 4)) * WP + 4 * (c % (N / 4))) = wreg[u];
        }
    };

    f32x16 acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[b][r] = 0.0f;
    load(0);
    for (int k0 = 0; k0 < K; k0 += NF_KS) {
        __syncthreads();  // every wave is done with the previous tiles
        store();
        __syncthreads();
        if (k0 + NF_KS < K) load(k0 + NF_KS);
        const f32x4 a = *(const f32x4*)(so + i * NF_OP + 4 * h);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float* wb = sw + (4 * h) * WP + c0 + 32 * b + i;
#pragma unroll
            for (int s = 0; s < 4; ++s)
                acc[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[s], wb[s * WP], acc[b], 0, 0, 0);
        }
    }

    // Residual (rows past M stay zero and are never stored).  Register r of
    // block b holds row acc_row(r, h), column c0 + 32 b + i.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = acc_row(r, h);
        if (row < rows)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                acc[b][r] += xres[(size_t)(m0 + row) * N + c0 + 32 * b + i];
    }

    // Sum of v[r] over each row: the 32 lanes of the half-wave, then the
    // four waves.  tot[r] is the total of row acc_row(r, h).
    auto row_sums = [&](const float (&v)[16], float (&tot)[16]) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float x = v[r];
#pragma unroll
            for (int off = 16; off >= 1; off >>= 1) x += __shfl_xor(x, off);
            if (i == 0) red[wave][acc_row(r, h)] = x;
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = acc_row(r, h);
            tot[r] = red[0][row] + red[1][row] + red[2][row] + red[3][row];
        }
        __syncthreads();
    };
    float part[16], mu[16], var[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        part[r] = 0.0f;
#pragma unroll
        for (int b = 0; b < NB; ++b) part[r] += acc[b][r];
    }
    row_sums(part, mu);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        mu[r] *= 1.0f / N;
        part[r] = 0.0f;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float dz = acc[b][r] - mu[r];
            part[r] = __builtin_fmaf(dz, dz, part[r]);
        }
    }
    row_sums(part, var);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = acc_row(r, h);
        if (row >= rows) continue;
        const float inv = 1.0f / sqrtf(var[r] * (1.0f / N) + eps);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int col = c0 + 32 * b + i;
            out[(size_t)(m0 + row) * N + col] =
                __builtin_fmaf(gamma[col], (acc[b][r] - mu[r]) * inv, beta[col]);
        }
    }
}

template <int NPT>
hipError_t launch_post_norm_f32_d(const PostNormArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)((a.M + NF_R - 1) / NF_R));
    hipLaunchKernelGGL((out_proj_post_norm_f32<NPT>), grid, dim3(256), 0, stream,
                       (const float*)a.o, (const float*)a.w, (const float*)a.x,
                       (const float*)a.gamma, (const float*)a.beta, (float*)a.out, a.M, a.K,
                       a.eps);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_out_proj_post_norm_f32(const PostNormArgs& a, hipStream_t stream) {
    switch (a.N) {
        case 256: return launch_post_norm_f32_d<1>(a, stream);
        case 512: return launch_post_norm_f32_d<2>(a, stream);
        default: return launch_post_norm_f32_d<4>(a, stream);
    }
}

hipError_t launch_out_proj_post_norm_bf16(const PostNormArgs& a, hipStream_t stream) {
    switch (a.N) {
        case 256: return launch_post_norm_d<1>(a, stream);
        case 512: return launch_post_norm_d<2>(a, stream);
        default: return launch_post_norm_d<4>(a, stream);
    }
}

}  // namespace mha
