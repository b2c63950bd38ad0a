// fused.hip -- the self-attention of one (batch row, head) in one kernel,
// for rows of at most 128 tokens:
//
//   [Q | K | V] = X_b [W_t^Q | W_t^K | W_t^V]        (L x 192, kept in LDS)
//   O_t = softmax(Q K^T / sqrt(d_k) + M) V           (written, BLHD)
//
// ("Attention Is All You Need -- A Revolutionary Architecture for Sequence
// Transduction", slide "Multi-Head Attention": head_i = Attention(Q W_i^Q,
// K W_i^K, V W_i^V); "Paper Deep Reading", section 04, attention equation
// with the mask M and the MultiHead equations.)  The projected Q, K and V
// of a head never reach HBM: the projection's accumulators are rounded to
// bf16 straight into the LDS tiles the attention reads.  The arithmetic is
// that of the projection GEMM followed by the short-row attention kernel,
// in the same order, so the output equals that of the two-kernel path.
#include "device.h"
#include "launch.h"

namespace mha {
namespace {

constexpr int FL = 128;                               // rows (tokens) per batch row, at most
constexpr int FKT = 32;                               // keys per attention tile
constexpr int FBK = 32;                               // k step of the projection
constexpr int FST = 3;                                // projection ring depth
constexpr int FX_ROW = FBK * 2;                       // bytes of an X stage row
constexpr int FX_BYTES = FL * FX_ROW;                 // X stage: 128 rows
constexpr int FW_MAT = FBK * 64 * 2;                  // one weight slab: FBK rows of 128 bytes
constexpr int FW_BYTES = 3 * FW_MAT;                  // W stage: the head's slabs of W^Q, W^K, W^V
constexpr int FRING = FST * (FX_BYTES + FW_BYTES);
constexpr int FTILE = FL * 64 * 2;                    // one of Q, K, V in LDS: 16 KB
constexpr int FSMEM = FRING > 3 * FTILE ? FRING : 3 * FTILE;
constexpr int FX_INSTR = FX_BYTES / 1024 / 4;         // 1 KB direct loads per wave: X
constexpr int FW_INSTR = FW_MAT / 1024 / 4;           //   and each weight slab
constexpr int F_PER_STAGE = FX_INSTR + 3 * FW_INSTR;  // direct loads per wave per stage
static_assert((FBK == 32 || FBK == 64) && (FST == 2 || FST == 3), "projection pipeline");

// X stage: row r holds FBK/8 chunks of 16 bytes (k = 8c .. 8c+7), chunk c at
// c ^ ((r >> 1) & 3) for rows of 64 bytes, c ^ (r & 7) for rows of 128
// bytes, so the 16-byte row reads of consecutive rows spread over the banks.
__device__ __forceinline__ int fx_chunk(int r, int c) {
    return FBK == 32 ? c ^ ((r >> 1) & 3) : c ^ (r & 7);
}

template <bool PAD, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void self_attention_fused_bf16(
    const bf16* __restrict__ x, const bf16* __restrict__ wq, const bf16* __restrict__ wk,
    const bf16* __restrict__ wv, const int32_t* __restrict__ kv_lens, bf16* __restrict__ o,
    int B, int L, int DM, int H, float scale_log2e) {
    __shared__ __attribute__((aligned(1024))) char smem[FSMEM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const int g = lane >> 4;
    const int i16 = lane & 15;

    // Workgroup -> (batch row, head).  Workgroups are dispatched to the 8
    // XCDs round-robin (workgroup w on XCD w % 8); when B*H divides by 8,
    // XCD x gets the pairs x*nbh/8 .. (x+1)*nbh/8 - 1, so the heads of a
    // batch row share one L2 for X_b.
    const int nbh = B * H;
    const int w = (int)blockIdx.x;
    const int bh = (nbh & 7) == 0 ? (w & 7) * (nbh >> 3) + (w >> 3) : w;
    const int b = bh / H;
    const int hh = bh - b * H;
    const int N = H * 64;  // row length of each weight matrix
    // The row's length is read first, so its latency hides under the
    // projection's loads.
    int kv_end = L;
    if (PAD) kv_end = min(max(kv_lens[b], 0), L);

    // ---- projection: D^T = W^T X^T, 192 features x 128 tokens ----
    // Wave (wm, wn) owns tokens 64 wm .. +63 (two 32-blocks) and features
    // 96 wn .. +95 (three 32-blocks: feature block f lies in matrix f / 2).
    const int wm = wave >> 1, wn = wave & 1;
    const __amdgpu_buffer_rsrc_t xr =
        make_rsrc(x + (size_t)b * L * DM, (uint32_t)((size_t)L * DM * 2));
    const bf16* wbase[3] = {wq + hh * 64, wk + hh * 64, wv + hh * 64};
    const uint32_t w_bytes = (uint32_t)(((size_t)(DM - 1) * N + 64) * 2);
    // Direct loads in slices of 1 KB: wave w loads slices w, w + 4, ... of
    // the X stage (1024 / FX_ROW rows each) and of each weight slab (8 rows
    // of 128 bytes each).
    constexpr int XC = FX_ROW / 16;  // chunks per X row
    uint32_t xoff[FX_INSTR], woff[FW_INSTR];
#pragma unroll
    for (int u = 0; u < FX_INSTR; ++u) {
        const int r = (1024 / FX_ROW) * (wave + 4 * u) + lane / XC;
        xoff[u] = (uint32_t)(r * DM + 8 * fx_chunk(r, lane % XC)) * 2;
    }
#pragma unroll
    for (int u = 0; u < FW_INSTR; ++u) {
        const int r = 8 * (wave + 4 * u) + (lane >> 3);
        woff[u] = (uint32_t)(r * N + 8 * ((lane & 7) ^ v_swz(r))) * 2;
    }
    auto sX = [&](int st) { return smem + st * FX_BYTES; };
    auto sW = [&](int st) { return smem + FST * FX_BYTES + st * FW_BYTES; };
    auto issue = [&](int kt, int st) {
        const uint32_t xs = lds_addr(sX(st)), ws = lds_addr(sW(st));
        const uint32_t xk = (uint32_t)kt * FBK * 2;
        const uint32_t wk_ = (uint32_t)((size_t)kt * FBK * N * 2);
#pragma unroll
        for (int u = 0; u < FX_INSTR; ++u)
            load_lds16(xr, xs + (wave + 4 * u) * 1024, xoff[u] + xk);
#pragma unroll
        for (int m = 0; m < 3; ++m)
#pragma unroll
            for (int u = 0; u < FW_INSTR; ++u)
                load_lds16(make_rsrc(wbase[m], w_bytes), ws + m * FW_MAT + (wave + 4 * u) * 1024,
                           woff[u] + wk_);
    };

    f32x16 acc[3][2];
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[j][mb][r] = 0.0f;

    // Operands of one 16-wide k slice.  A = W^T (32 features x 16 k) by
    // transpose reads of the weight slab; B = X^T (16 k x 32 tokens) by
    // 16-byte reads of the X stage.
    auto read_ops = [&](int st, int k16, bf16x8 (&a)[3], bf16x8 (&bx)[2]) {
        const char* ws = sW(st);
        const char* xs = sX(st);
        const int krow = 16 * k16 + 8 * (g >> 1) + (i16 >> 2);
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int fb = 3 * wn + j;  // feature block 0..5
            const char* slab = ws + (fb >> 1) * FW_MAT;
            const int n = 32 * (fb & 1) + 16 * (g & 1) + 4 * (i16 & 3);
            const int c = n >> 3, byte = (n & 7) * 2;
            const bf16* lo = (const bf16*)(slab + krow * 128 + ((c ^ v_swz(krow)) << 4) + byte);
            const bf16* hi =
                (const bf16*)(slab + (krow + 4) * 128 + ((c ^ v_swz(krow + 4)) << 4) + byte);
            a[j] = join(lds_read_tr(lo), lds_read_tr(hi));
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int r = 64 * wm + 32 * mb + l32;
            bx[mb] = *(const bf16x8*)(xs + r * FX_ROW + (fx_chunk(r, 2 * k16 + half) << 4));
        }
    };
    const int n_k = DM / FBK;
    bf16x8 opA[2][3], opB[2][2];
    auto step = [&](int kt, int st) {
        const int ahead = min(FST - 2, n_k - 1 - kt);
        if (ahead >= 1) wait_vmcnt<F_PER_STAGE>();
        else wait_vmcnt<0>();
        barrier_lds();  // step kt visible everywhere; the stage of step kt-1 is free
        if (kt + FST - 1 < n_k) issue(kt + FST - 1, (st + FST - 1) % FST);
        // operands of slice i + 1 are read while the MFMAs of slice i run
        read_ops(st, 0, opA[0], opB[0]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k16 = 0; k16 < FBK / 16; ++k16) {
            if (k16 + 1 < FBK / 16) read_ops(st, k16 + 1, opA[(k16 + 1) & 1], opB[(k16 + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < 3; ++j)
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
                    acc[j][mb] = mfma32(opA[k16 & 1][j], opB[k16 & 1][mb], acc[j][mb]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
#pragma unroll
    for (int s = 0; s < FST - 1; ++s)
        if (s < n_k) issue(s, s);
    for (int kt = 0; kt < n_k; kt += FST) {
#pragma unroll
        for (int s = 0; s < FST; ++s)
            if (kt + s < n_k) step(kt + s, s);
    }

    // ---- Q, K, V to LDS as bf16, in the layouts the attention reads ----
    // Register group q (r = 4q .. 4q+3) of feature block fb holds features
    // 32 (fb & 1) + 8q + 4 half .. +3 of matrix fb / 2 for this lane's token.
    // A half swap between lanes l and l + 32 (same token) gathers whole
    // 16-byte chunks: groups 2p and 2p + 1 become chunk 4 (fb & 1) + 2p +
    // half, written by one 16-byte store.  K and V rows at or past the row's
    // length are stored as zeros: like the rows the attention kernels never
    // load, whatever X holds there cannot reach the output.
    barrier_lds();  // every wave is done with the projection ring
    char* const sQ = smem;
    char* const sK = smem + FTILE;
    char* const sV = smem + 2 * FTILE;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int fb = 3 * wn + j;
        const int mat = fb >> 1;
        char* const dst = mat == 0 ? sQ : (mat == 1 ? sK : sV);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int m0 = 64 * wm + 32 * mb;  // the block's first token (wave-uniform)
            const int m = m0 + l32;
            const int swz = mat == 2 ? v_swz(m) : k_swz(m);
            // Only a K or V block that reaches the length needs the zeroing.
            const bool clip = mat != 0 && m0 + 32 > kv_end;
            const bool keep = m < kv_end;
#pragma unroll
            for (int p2 = 0; p2 < 2; ++p2) {
                bf16x4 v4[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int q4 = 2 * p2 + u;
                    const f32x4 f = {acc[j][mb][4 * q4], acc[j][mb][4 * q4 + 1],
                                     acc[j][mb][4 * q4 + 2], acc[j][mb][4 * q4 + 3]};
                    v4[u] = __builtin_convertvector(f, bf16x4);
                    if (clip && !keep) v4[u] = bf16x4{};
                }
                // Swap the upper half of group 2p with the lower half of
                // group 2p + 1: lane l < 32 then holds group 2p of lanes l and
                // l + 32 (the low and high 8 bytes of chunk 2p), lane l + 32
                // group 2p + 1 of both (chunk 2p + 1).
                const auto lo = __builtin_bit_cast(uint2, v4[0]);
                const auto hi = __builtin_bit_cast(uint2, v4[1]);
                const auto s0 = __builtin_amdgcn_permlane32_swap(lo.x, hi.x, false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(lo.y, hi.y, false, false);
                const uint4 c = {s0[0], s1[0], s0[1], s1[1]};
                const int chunk = 4 * (fb & 1) + 2 * p2 + half;
                *(uint4*)(dst + m * 128 + ((chunk ^ swz) << 4)) = c;
            }
        }
    }
    barrier_lds();

    // ---- attention: wave w owns queries 32w .. 32w+31, one per lane ----
    const int n_tiles = (kv_end + FKT - 1) / FKT;
    const int wq0 = 32 * wave;
    int n_mine = (wq0 < L) ? n_tiles : 0;
    if (CAUSAL) n_mine = min(n_mine, wave + 1);

    bf16x8 qop[4];
    {
        const int r = wq0 + l32;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            qop[kk] = *(const bf16x8*)(sQ + r * 128 + (((2 * kk + half) ^ k_swz(r)) << 4));
    }
    uint32_t k_rd[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) k_rd[kk] = l32 * 128 + 16 * ((2 * kk + half) ^ k_swz(l32));
    uint32_t v_rd[2];
    {
        const int row = 4 * half + (i16 >> 2);
#pragma unroll
        for (int db = 0; db < 2; ++db) {
            const int chunk = 4 * db + 2 * (g & 1) + ((i16 & 3) >> 1);
            v_rd[db] = row * 128 + 16 * (chunk ^ v_swz(row)) + 8 * (i16 & 1);
        }
    }
    f32x16 oacc[2];
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
    float m_run = -INFINITY, l_part = 0.0f;
    const f32x16 zero16 = {};
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};

    for (int t = 0; t < n_mine; ++t) {
        const char* kb = sK + t * FKT * 128;
        const char* vb = sV + t * FKT * 128;
        bf16x8 ka[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) ka[kk] = *(const bf16x8*)(kb + k_rd[kk]);
        bf16x8 va[2][2];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int db = 0; db < 2; ++db)
                va[c][db] = join(lds_read_tr((const bf16*)(vb + 2048 * c + v_rd[db])),
                                 lds_read_tr((const bf16*)(vb + 2048 * c + v_rd[db] + 1024)));
        f32x16 S = mfma32(ka[0], qop[0], zero16);
#pragma unroll
        for (int kk = 1; kk < 4; ++kk) S = mfma32(ka[kk], qop[kk], S);

        const int k0 = t * FKT;
        if ((k0 + FKT > kv_end) || (CAUSAL && k0 + FKT - 1 > wq0)) {
            int lim = kv_end - k0;
            if (CAUSAL) lim = min(lim, wq0 + l32 + 1 - k0);
            lim -= 4 * half;
#pragma unroll
            for (int r = 0; r < 16; ++r) S[r] = acc_row(r, 0) < lim ? S[r] : -INFINITY;
        }
        float mx = S[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S[r]);
        mx = max_halves(mx);
        const bool grow = (mx - m_run) * scale_log2e > 8.0f;
        if (__builtin_amdgcn_ballot_w64(grow)) {
            const float m_new = grow ? mx : m_run;
            const float alpha = grow ? __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2e) : 1.0f;
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            l_part *= alpha;
            m_run = m_new;
        }
        const float mc = (m_run == -INFINITY) ? 0.0f : m_run * scale_log2e;
        bf16x8 pop[2];
#pragma unroll
        for (int pr = 0; pr < 8; ++pr) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[2 * pr], scale_log2e, -mc));
            const float p1 =
                __builtin_amdgcn_exp2f(__builtin_fmaf(S[2 * pr + 1], scale_log2e, -mc));
            const bf16x2 pp = {(bf16)p0, (bf16)p1};
            pop[pr >> 2][2 * (pr & 3)] = pp[0];
            pop[pr >> 2][2 * (pr & 3) + 1] = pp[1];
            l_part = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l_part, false);
        }
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int db = 0; db < 2; ++db) oacc[db] = mfma32(va[c][db], pop[c], oacc[db]);
    }

    // ---- O = acc / l (0 without a legal key), staged over this wave's Q
    // rows and written as whole rows.  Only this wave reads or writes
    // those rows, and one wave's LDS accesses take effect in program
    // order, so the staging needs no barrier. ----
    const float l_tot = sum_halves(l_part);
    const float inv = (l_tot > 0.0f) ? 1.0f / l_tot : 0.0f;
    char* stg = sQ + wq0 * 128;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            bf16x4 out;
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e] = (bf16)(oacc[db][4 * rg + e] * inv);
            const int chunk = (4 * db + rg) ^ (l32 & 7);
            *(bf16x4*)(stg + l32 * 128 + 16 * chunk + 8 * half) = out;
        }
    bf16* op = o + ((size_t)b * L * H + hh) * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 8 * i + (lane >> 3), c = lane & 7;
        const int qi = wq0 + r;
        if (qi < L)
            store_stream((bf16x8*)(op + (size_t)qi * N + 8 * c),
                         *(const bf16x8*)(stg + r * 128 + 16 * (c ^ (r & 7))));
    }
}

}  // namespace

hipError_t launch_self_attention_fused_bf16(const FusedArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)((long)a.B * a.H));
    const float sl2e = (float)(1.4426950408889634 / sqrt(64.0));
    const bf16* x = (const bf16*)a.x;
    const bf16* wq = (const bf16*)a.w_q;
    const bf16* wk = (const bf16*)a.w_k;
    const bf16* wv = (const bf16*)a.w_v;
    bf16* o = (bf16*)a.o;
    switch (a.mask) {
        case 0:
            hipLaunchKernelGGL((self_attention_fused_bf16<false, false>), grid, dim3(256), 0, stream,
                               x, wq, wk, wv, a.kv_lens, o, a.B, a.L, a.DM, a.H, sl2e);
            break;
        case 1:
            hipLaunchKernelGGL((self_attention_fused_bf16<true, false>), grid, dim3(256), 0, stream,
                               x, wq, wk, wv, a.kv_lens, o, a.B, a.L, a.DM, a.H, sl2e);
            break;
        case 2:
            hipLaunchKernelGGL((self_attention_fused_bf16<false, true>), grid, dim3(256), 0, stream,
                               x, wq, wk, wv, a.kv_lens, o, a.B, a.L, a.DM, a.H, sl2e);
            break;
        default:
            hipLaunchKernelGGL((self_attention_fused_bf16<true, true>), grid, dim3(256), 0, stream,
                               x, wq, wk, wv, a.kv_lens, o, a.B, a.L, a.DM, a.H, sl2e);
            break;
    }
    return hipGetLastError();
}

}  // namespace mha
