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

namespace {

constexpr int D64 = 64;
constexpr int KT = 32;             // keys per tile

// ---------------------------------------------------------------------------
// bf16, d = 64, rows of at most 256 keys (8 tiles): every K/V row of the
// (batch row, head) fits in LDS, so it is loaded at once.
//
// Workgroup = 4 waves = one (batch row, head, block of 128 queries); wave w
// owns 32 consecutive queries, one per lane column.  All K/V tiles go to
// LDS by direct global-to-LDS loads issued together (one memory round trip)
// behind a single barrier; each wave then runs its tiles with no further
// synchronisation: S^T = K Q^T (4 MFMAs), mask, online softmax (a running
// row maximum, the partial output rescaled only when the maximum grows by
// more than 2^8, exact because numerator and denominator share the stale
// maximum), O^T += V^T P^T (4 MFMAs).  The output block is staged through
// LDS so that each 128-byte (query, head) row is written whole.
//
// LDS tiles here are 32 rows of 128 bytes without padding (a direct load
// writes 16 contiguous bytes per lane); the eight 16-byte chunks of a row
// are permuted by row so both read patterns spread over the banks:
//   K (16-byte row reads):               chunk c of row r at c ^ (r & 7)
//   V (transpose reads of 8 rows x 64 B): chunk c of row r at c ^ 4((r >> 1) & 1)
// ---------------------------------------------------------------------------
constexpr int SHORT_TILE_BYTES = KT * D64 * 2;  // one K (or V) tile
constexpr int SHORT_BM = 128;                   // queries per workgroup

template <int NT, bool PAD, bool CAUSAL>
__global__ __launch_bounds__(256, NT <= 4 ? 4 : 2) void attn_short_bf16_d64(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    bf16* __restrict__ o, const int32_t* __restrict__ kv_lens, int B, int H, int Lq, int Lk,
    int n_qtiles, float scale_log2e) {
    static_assert(NT >= 4 && 2 * NT * SHORT_TILE_BYTES >= 4 * 32 * 128, "LDS for the output");
    __shared__ __attribute__((aligned(1024))) char smem[NT * 2 * SHORT_TILE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const int g = lane >> 4;
    const int i16 = lane & 15;

    // Tile decode: as for long rows (all query blocks of a (batch row, head)
    // on one XCD; causal: longest blocks first).
    const int nbh = B * H;
    const int w = (int)blockIdx.x;
    int bh, qt;
    if ((nbh & 7) == 0) {
        const int x = w & 7, slot = w >> 3, per = nbh >> 3;
        if (CAUSAL) {
            qt = n_qtiles - 1 - slot / per;
            bh = x * per + slot % per;
        } else {
            bh = x * per + slot / n_qtiles;
            qt = slot % n_qtiles;
        }
    } else if (CAUSAL) {
        qt = n_qtiles - 1 - w / nbh;
        bh = w % nbh;
    } else {
        bh = w / n_qtiles;
        qt = w % n_qtiles;
    }
    const int b = bh / H;
    const int hh = bh - b * H;
    const int q0 = qt * SHORT_BM;

    int kv_end = Lk;
    if (PAD) kv_end = min(max(kv_lens[b], 0), Lk);
    int key_end = kv_end;
    if (CAUSAL) key_end = min(key_end, min(q0 + SHORT_BM, Lq));
    const int n_tiles = (key_end + KT - 1) / KT;  // <= NT: Lk <= 32 NT
    const int wq0 = q0 + 32 * wave;
    int n_mine = (wq0 < Lq) ? n_tiles : 0;
    if (CAUSAL) n_mine = min(n_mine, (wq0 + 32 + KT - 1) / KT);

    const size_t rs = (size_t)H * D64;
    const uint32_t rsb = (uint32_t)(rs * sizeof(bf16));
    const bf16* qp = q + ((size_t)b * Lq * H + hh) * D64;
    const bf16* kp = k + ((size_t)b * Lk * H + hh) * D64;
    const bf16* vp = v + ((size_t)b * Lk * H + hh) * D64;
    bf16* op = o + ((size_t)b * Lq * H + hh) * D64;

    // Q (B operand of S^T = K Q^T): lane holds query wq0 + l32, d = 16kk +
    // 8half .. +7.  Rows past Lq read as zeros.
    const __amdgpu_buffer_rsrc_t qrsrc =
        make_rsrc(qp, (uint32_t)(((size_t)(Lq - 1) * rs + D64) * sizeof(bf16)));
    bf16x8 qop[4];
    {
        const int qi = wq0 + l32;
        const uint32_t qoff = qi < Lq ? (uint32_t)qi * rsb + 16 * half : OOB_OFFSET;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) qop[kk] = buffer_load16(qrsrc, qoff + 32 * kk);
    }

    // Every K/V tile of the row into LDS: thread tid fills chunk position
    // tid of tile t's K and V (row tid / 8); rows at or past kv_end land as
    // zeros without a memory access.
    {
        const uint32_t kv_bytes = kv_end > 0 ? (uint32_t)(kv_end - 1) * rsb + D64 * 2 : 0u;
        const __amdgpu_buffer_rsrc_t krsrc = make_rsrc(kp, kv_bytes);
        const __amdgpu_buffer_rsrc_t vrsrc = make_rsrc(vp, kv_bytes);
        const int pr = tid >> 3, pc = tid & 7;
        const uint32_t k_dma = (uint32_t)pr * rsb + 16 * (pc ^ k_swz(pr));
        const uint32_t v_dma = (uint32_t)pr * rsb + 16 * (pc ^ v_swz(pr));
        const uint32_t tile_gbytes = (uint32_t)KT * rsb;
        const uint32_t lds_wave = lds_addr(smem) + 1024 * wave;
        for (int t = 0; t < n_tiles; ++t) {
            const uint32_t st = lds_wave + (uint32_t)t * 2 * SHORT_TILE_BYTES;
            load_lds16(krsrc, st, (uint32_t)t * tile_gbytes + k_dma);
            load_lds16(vrsrc, st + SHORT_TILE_BYTES, (uint32_t)t * tile_gbytes + v_dma);
        }
    }
    wait_vmcnt<0>();
    barrier_lds();

    // LDS operand reads (the lane patterns of the streaming kernel in
    // attn_stream.hip).
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

    f32x16 acc[2];
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;
    float m_run = -INFINITY, l_part = 0.0f;
    const f32x16 zero16 = {};
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};

    for (int t = 0; t < n_mine; ++t) {
        const char* kb = smem + t * 2 * SHORT_TILE_BYTES;
        const char* vb = kb + SHORT_TILE_BYTES;
        bf16x8 ka[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) ka[kk] = *(const bf16x8*)(kb + k_rd[kk]);
        bf16x8 va[2][2];  // [16-key chunk][d block]
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int db = 0; db < 2; ++db)
                va[c][db] = join(lds_read_tr((const bf16*)(vb + 2048 * c + v_rd[db])),
                                 lds_read_tr((const bf16*)(vb + 2048 * c + v_rd[db] + 1024)));
        f32x16 S = mfma32(ka[0], qop[0], zero16);
#pragma unroll
        for (int kk = 1; kk < 4; ++kk) S = mfma32(ka[kk], qop[kk], S);

        // Mask the boundary tiles: key k0 + acc_row(r, half) is legal iff
        // acc_row(r, 0) < lim.
        const int k0 = t * KT;
        if ((k0 + KT > kv_end) || (CAUSAL && k0 + KT - 1 > wq0)) {
            int lim = kv_end - k0;
            if (CAUSAL) lim = min(lim, wq0 + l32 + 1 - k0);
            lim -= 4 * half;
#pragma unroll
            for (int r = 0; r < 16; ++r) S[r] = acc_row(r, 0) < lim ? S[r] : -INFINITY;
        }

        // Running maximum with the lazy rescale (a row moves to a new
        // maximum only when it exceeds the old one by more than 2^8).
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
                for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
            l_part *= alpha;
            m_run = m_new;
        }
        const float mc = (m_run == -INFINITY) ? 0.0f : m_run * scale_log2e;

        // p = exp2(s c - m c), rounded to bf16 for PV; the row sum adds the
        // rounded pairs.
        bf16x8 pop[2];
#pragma unroll
        for (int pr2 = 0; pr2 < 8; ++pr2) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[2 * pr2], scale_log2e, -mc));
            const float p1 =
                __builtin_amdgcn_exp2f(__builtin_fmaf(S[2 * pr2 + 1], scale_log2e, -mc));
            const bf16x2 pp = {(bf16)p0, (bf16)p1};
            pop[pr2 >> 2][2 * (pr2 & 3)] = pp[0];
            pop[pr2 >> 2][2 * (pr2 & 3) + 1] = pp[1];
            l_part = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l_part, false);
        }
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int db = 0; db < 2; ++db) acc[db] = mfma32(va[c][db], pop[c], acc[db]);
    }

    // Epilogue: O = acc / l (0 for a row with no legal key), staged in LDS
    // (wave w: rows of its 32 queries, 128 B each, chunks permuted by row)
    // and written back as whole rows, 16 bytes per lane.
    barrier_lds();  // every wave is done with the K/V tiles
    const float l_tot = sum_halves(l_part);
    const float inv = (l_tot > 0.0f) ? 1.0f / l_tot : 0.0f;
    char* stg = smem + wave * 32 * 128;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            bf16x4 out;
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e] = (bf16)(acc[db][4 * rg + e] * inv);
            const int chunk = (4 * db + rg) ^ (l32 & 7);
            *(bf16x4*)(stg + l32 * 128 + 16 * chunk + 8 * half) = out;
        }
    // The staged rows are this wave's own, and one wave's LDS accesses take
    // effect in program order: no barrier before reading them back.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 8 * i + (lane >> 3), c = lane & 7;
        const int qi = wq0 + r;
        if (qi < Lq)
            store_stream((bf16x8*)(op + (size_t)qi * rs + 8 * c),
                         *(const bf16x8*)(stg + r * 128 + 16 * (c ^ (r & 7))));
    }
}

// ---------------------------------------------------------------------------
// fp32, d in {8, 16, 32, 64}: the accuracy path, on the matrix cores
// (v_mfma_f32_32x32x2_f32: fp32 products, fp32 accumulation), with exact
// fp32 scaling and accurate expf.
//
// Workgroup = 4 waves = one (batch row, head, block of 128 queries); wave w
// owns 32 consecutive queries, one per lane column.  K/V tiles of 32 rows
// are staged in LDS as fp32 (rows at or past the length as zeros, so no
// value stored there can reach the output), loaded into registers one tile
// ahead.  Per tile a wave computes
//   S^T = K Q^T      D/2 MFMAs: lane (i, h = lane / 32) feeds K[key i][d]
//                    and Q[query i][d] for d = h D/2 + s at step s
//   scale, mask, online softmax with a running maximum (the partial output
//                    rescaled whenever the maximum grows)
//   O^T += V^T P^T   16 MFMAs per 32-row block of d: step s takes the
//                    weight of accumulator register s, i.e. key
//                    (s % 4) + 8 (s / 4) + 4 h, which is the one the lane
//                    already holds, so P never moves between lanes.
// For d < 32 the unused rows of the d block read zeros and are not stored.
// ---------------------------------------------------------------------------
constexpr int F32_BM = 128;  // queries per workgroup
constexpr int F32_KT = 32;   // keys per tile

template <int D, bool PAD, bool CAUSAL, bool WIN>
__global__ __launch_bounds__(256, 2) void attn_mfma_f32(const float* __restrict__ q,
                                                        const float* __restrict__ k,
                                                        const float* __restrict__ v,
                                                        float* __restrict__ o,
                                                        const int32_t* __restrict__ kv_lens,
                                                        int B, int H, int Lq, int Lk,
                                                        int n_qtiles, float scale, int window) {
    static_assert(D == 8 || D == 16 || D == 32 || D == 64, "head size");
    constexpr int DH = D / 2;               // d values each half-wave feeds to S^T
    constexpr int PITCH = D + 4;            // LDS row pitch in floats (rows 16 B apart in bank)
    constexpr int DB = D < 32 ? 1 : D / 32; // 32-row blocks of O^T
    constexpr int C4 = D / 4;               // float4 chunks per row
    __shared__ __attribute__((aligned(16))) float sK[F32_KT * PITCH];
    __shared__ __attribute__((aligned(16))) float sV[F32_KT * PITCH];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5;
    const int i = lane & 31;
    const int bh = (int)(blockIdx.x / n_qtiles);
    const int qt = (int)(blockIdx.x % n_qtiles);
    const int b = bh / H;
    const int hh = bh - b * H;
    const int q0 = qt * F32_BM;

    int kv_end = Lk;
    if (PAD) kv_end = min(max(kv_lens[b], 0), Lk);
    int key_end = kv_end;
    if (CAUSAL) key_end = min(key_end, min(q0 + F32_BM, Lq));
    int t_first = 0;  // restricted attention: the workgroup's band only
    if (WIN) {
        key_end = min(key_end, q0 + F32_BM + window);
        t_first = max(q0 - window, 0) / F32_KT;
    }
    const int n_tiles = (key_end + F32_KT - 1) / F32_KT;
    // This wave's tiles: none without a query row; causal stops at the tile
    // of its last query; a band starts and stops a window away.
    const int wq0 = q0 + 32 * wave;
    int n_mine = (wq0 < Lq) ? n_tiles : 0;
    if (CAUSAL) n_mine = min(n_mine, (wq0 + 32 + F32_KT - 1) / F32_KT);
    int w_first = t_first;
    if (WIN) {
        n_mine = min(n_mine, (min(kv_end, wq0 + 32 + window) + F32_KT - 1) / F32_KT);
        w_first = max(wq0 - window, 0) / F32_KT;
    }

    const size_t rs = (size_t)H * D;
    const float* qp = q + ((size_t)b * Lq * H + hh) * D;
    const float* kp = k + ((size_t)b * Lk * H + hh) * D;
    const float* vp = v + ((size_t)b * Lk * H + hh) * D;
    float* op = o + ((size_t)b * Lq * H + hh) * D;

    // Q as the B operand of S^T: query wq0 + i, d = h DH .. h DH + DH - 1.
    const int qi = wq0 + i;
    float qr[DH];
#pragma unroll
    for (int s = 0; s < DH; s += 4) {
        float4 x = {0.0f, 0.0f, 0.0f, 0.0f};
        if (qi < Lq) x = *(const float4*)(qp + (size_t)qi * rs + h * DH + s);
        qr[s] = x.x;
        qr[s + 1] = x.y;
        qr[s + 2] = x.z;
        qr[s + 3] = x.w;
    }

    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;
    float m_run = -INFINITY, l_part = 0.0f;

    // Tile t's K and V rows reach registers one tile ahead (thread tid
    // takes chunks tid, tid + 256, ... of 4 floats: row chunk / (d/4)) and
    // LDS between two barriers.
    constexpr int NPF = (F32_KT * C4 + 255) / 256;
    float4 kpre[NPF], vpre[NPF];
    auto fetch = [&](int t) {
#pragma unroll
        for (int u = 0; u < NPF; ++u) {
            const int idx = tid + 256 * u;
            const int row = idx / C4, c = idx % C4;
            const int key = t * F32_KT + row;
            float4 kx = {0.0f, 0.0f, 0.0f, 0.0f}, vx = {0.0f, 0.0f, 0.0f, 0.0f};
            if (idx < F32_KT * C4 && key < kv_end) {
                kx = *(const float4*)(kp + (size_t)key * rs + 4 * c);
                vx = *(const float4*)(vp + (size_t)key * rs + 4 * c);
            }
            kpre[u] = kx;
            vpre[u] = vx;
        }
    };
    if (t_first < n_tiles) fetch(t_first);
    for (int t = t_first; t < n_tiles; ++t) {
        __syncthreads();  // every wave is done with the previous tile
#pragma unroll
        for (int u = 0; u < NPF; ++u) {
            const int idx = tid + 256 * u;
            if (idx < F32_KT * C4) {
                const int row = idx / C4, c = idx % C4;
                *(float4*)(sK + row * PITCH + 4 * c) = kpre[u];
                *(float4*)(sV + row * PITCH + 4 * c) = vpre[u];
            }
        }
        __syncthreads();
        if (t + 1 < n_tiles) fetch(t + 1);
        if (t < w_first || t >= n_mine) continue;  // wave-uniform

        // S^T = K Q^T: lane (i, h) holds key t*32 + (r % 4) + 8 (r / 4) + 4h
        // of query qi in register r.
        f32x16 S;
#pragma unroll
        for (int r = 0; r < 16; ++r) S[r] = 0.0f;
#pragma unroll
        for (int s = 0; s < DH; s += 4) {
            const float4 kx = *(const float4*)(sK + i * PITCH + h * DH + s);
            S = __builtin_amdgcn_mfma_f32_32x32x2f32(kx.x, qr[s], S, 0, 0, 0);
            S = __builtin_amdgcn_mfma_f32_32x32x2f32(kx.y, qr[s + 1], S, 0, 0, 0);
            S = __builtin_amdgcn_mfma_f32_32x32x2f32(kx.z, qr[s + 2], S, 0, 0, 0);
            S = __builtin_amdgcn_mfma_f32_32x32x2f32(kx.w, qr[s + 3], S, 0, 0, 0);
        }
        // Scale (after the product, as the attention equation orders them),
        // then -inf at illegal pairs.
        float x[16];
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = t * F32_KT + acc_row(r, h);
            bool legal = key < kv_end;
            if (CAUSAL) legal = legal && key <= qi;
            if (WIN) legal = legal && key >= qi - window && key <= qi + window;
            x[r] = legal ? S[r] * scale : -INFINITY;
            mx = fmaxf(mx, x[r]);
        }
        mx = max_halves(mx);
        const float m_new = fmaxf(m_run, mx);
        // No legal key yet (m_new = -inf): weights 0, nothing rescaled.
        const bool none = m_new == -INFINITY;
        const float alpha = none ? 1.0f : expf(m_run - m_new);  // 0 while m_run = -inf
        float p[16];
        float lt = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            p[r] = none ? 0.0f : expf(x[r] - m_new);
            lt += p[r];
        }
        l_part = l_part * alpha + lt;
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
            // O^T[dd][q] += sum over keys of V[key][dd] P[q][key]; lane (i, h)
            // feeds V[key (s % 4) + 8 (s / 4) + 4h][dd = 32 db + i].
            const int dd = 32 * db + i;
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const float a = dd < D ? sV[acc_row(s, h) * PITCH + dd] : 0.0f;
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, p[s], acc[db], 0, 0, 0);
            }
        }
    }

    // O = acc / l (0 for a row with no legal key).  Lane (i, h) holds
    // O[qi][32 db + 8 j + 4 h .. + 3] in registers 4 j .. 4 j + 3.
    const float l_tot = sum_halves(l_part);
    const float inv = (l_tot > 0.0f) ? 1.0f / l_tot : 0.0f;
    if (qi < Lq) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d0 = 32 * db + 8 * j + 4 * h;
                if (d0 >= D) continue;
                const float4 out = {acc[db][4 * j] * inv, acc[db][4 * j + 1] * inv,
                                    acc[db][4 * j + 2] * inv, acc[db][4 * j + 3] * inv};
                *(float4*)(op + (size_t)qi * rs + d0) = out;
            }
    }
}

template <int D, bool WIN>
hipError_t launch_f32_dw(const AttnArgs& a, hipStream_t stream) {
    const int n_qtiles = (a.Lq + F32_BM - 1) / F32_BM;
    const dim3 grid((unsigned)((long)a.B * a.H * n_qtiles));
    const float scale = (float)(1.0 / sqrt((double)D));
    const float* q = (const float*)a.q;
    const float* k = (const float*)a.k;
    const float* v = (const float*)a.v;
    float* o = (float*)a.o;
    switch (a.mask) {
        case 0:
            hipLaunchKernelGGL((attn_mfma_f32<D, false, false, WIN>), grid, dim3(256), 0, stream,
                               q, k, v, o, a.kv_lens, a.B, a.H, a.Lq, a.Lk, n_qtiles, scale,
                               a.window);
            break;
        case 1:
            hipLaunchKernelGGL((attn_mfma_f32<D, true, false, WIN>), grid, dim3(256), 0, stream,
                               q, k, v, o, a.kv_lens, a.B, a.H, a.Lq, a.Lk, n_qtiles, scale,
                               a.window);
            break;
        case 2:
            hipLaunchKernelGGL((attn_mfma_f32<D, false, true, WIN>), grid, dim3(256), 0, stream,
                               q, k, v, o, a.kv_lens, a.B, a.H, a.Lq, a.Lk, n_qtiles, scale,
                               a.window);
            break;
        default:
            hipLaunchKernelGGL((attn_mfma_f32<D, true, true, WIN>), grid, dim3(256), 0, stream,
                               q, k, v, o, a.kv_lens, a.B, a.H, a.Lq, a.Lk, n_qtiles, scale,
                               a.window);
            break;
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_f32_d(const AttnArgs& a, hipStream_t stream) {
    return a.window >= 0 ? launch_f32_dw<D, true>(a, stream) : launch_f32_dw<D, false>(a, stream);
}

template <int NT>
hipError_t launch_short_bf16(const AttnArgs& a, hipStream_t stream) {
    const int n_qtiles = (a.Lq + SHORT_BM - 1) / SHORT_BM;
    const dim3 grid((unsigned)((long)a.B * a.H * n_qtiles));
    const float sl2e = (float)(1.4426950408889634 / sqrt((double)a.D));
    const bf16* q = (const bf16*)a.q;
    const bf16* k = (const bf16*)a.k;
    const bf16* v = (const bf16*)a.v;
    bf16* o = (bf16*)a.o;
    switch (a.mask) {
        case 0:
            hipLaunchKernelGGL((attn_short_bf16_d64<NT, false, false>), grid, dim3(256), 0, stream,
                               q, k, v, o, a.kv_lens, a.B, a.H, a.Lq, a.Lk, n_qtiles, sl2e);
            break;
        case 1:
            hipLaunchKernelGGL((attn_short_bf16_d64<NT, true, false>), grid, dim3(256), 0, stream,
                               q, k, v, o, a.kv_lens, a.B, a.H, a.Lq, a.Lk, n_qtiles, sl2e);
            break;
        case 2:
            hipLaunchKernelGGL((attn_short_bf16_d64<NT, false, true>), grid, dim3(256), 0, stream,
                               q, k, v, o, a.kv_lens, a.B, a.H, a.Lq, a.Lk, n_qtiles, sl2e);
            break;
        default:
            hipLaunchKernelGGL((attn_short_bf16_d64<NT, true, true>), grid, dim3(256), 0, stream,
                               q, k, v, o, a.kv_lens, a.B, a.H, a.Lq, a.Lk, n_qtiles, sl2e);
            break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_bf16(const AttnArgs& a, hipStream_t stream) {
    // d = 64: rows of at most 128 (256) keys hold the whole K/V row in LDS
    // at once; longer rows and restricted attention stream through the
    // kernel of attn_stream.hip, as the other head sizes do at every length.
    if (a.window >= 0 || a.D != 64) return launch_attention_stream_bf16(a, stream);
    if (a.Lk <= 128) return launch_short_bf16<4>(a, stream);
    if (a.Lk <= 256) return launch_short_bf16<8>(a, stream);
    return launch_attention_stream_bf16(a, stream);
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
