// attn_stream.hip -- streaming scaled dot-product attention forward for
// gfx950: head sizes 16, 32 and 128 at every length, and d = 64 rows longer
// than the whole-row-in-LDS kernel takes:
//
//   O = softmax(Q K^T / sqrt(d_k) + M) V        for every (batch row, head)
//
// ("Paper Deep Reading: Attention Is All You Need", section 04, attention
// equation with the mask M; MatMul -> Scale -> Mask -> SoftMax -> MatMul as
// in Figure 2, left.)  M is -inf at illegal pairs: keys at or beyond the
// batch row's length, keys after the query (decoder), and, for restricted
// self-attention (section 05, complexity table), keys more than `window`
// positions from the query.
//
// The softmax runs over 32-key tiles against a reference value m per query
// row: p = exp2((s - m) log2(e) / sqrt(d)), acc += p v, l += p, and O = acc
// / l at the end.  This is the exact identity softmax(x) = softmax(x - c)
// for any c; m only has to keep p inside the fp32/bf16 range.  m is the
// row maximum over the wave's first tile (its first two under restricted
// attention, where a row's band may start a tile in), found exactly, and
// then stays fixed: a later key would have to exceed it by
// more than ~88 scaled-logit units (2^127 in p) to overflow.  A row whose
// sum or output is not finite at the end (that overflow, or a row with no
// legal key in its first tiles) is recomputed by the wave with a running
// maximum that moves every tile.  The common path thereby carries no
// per-tile row maximum and no per-tile data-dependent branch (a branch on
// a VALU compare waits for the wave's MFMAs in flight): only the scale and
// offset, the exponential, the rounding and the row-sum step per value,
// which with the MFMAs is the work this kernel is bound by at d = 64 (at
// d = 16 and 32 the softmax alone; at d = 16 the row sum is taken by the
// PV MFMA's otherwise unused half block).
//
// Workgroup = 4 waves = one (batch row, head, block of 256 or 128 queries);
// wave w owns QB blocks of 32 queries (QB = 2 or 1, one query per lane
// column).  K/V tiles of 32 rows reach LDS by direct global-to-LDS loads
// into a 6-stage ring, two tiles at a time behind a barrier every other
// tile (at d = 128 a 4-stage ring, a tile at a time behind a barrier per
// tile).  Per tile j a wave issues
//
//   O^T += V_{j-1}^T P_{j-1}^T   2 QB max(d/32, 1) MFMAs (the previous
//                                tile's weights)
//   S_{j+1}^T = K_{j+1} Q^T      QB d/16 MFMAs (the next tile's scores)
//
// beside the steps of the softmax of S_j, so the matrix core runs while the
// VALU does the softmax.
#include "device.h"
#include "launch.h"

namespace mha {
namespace {

constexpr int SKT = 32;                // keys per tile
constexpr int SNW = 4;                 // waves per workgroup
// Tuning switches (the defaults are the measured best): a barrier every
// other tile with a 6-stage ring; the slots' priority raise with one query
// block per wave.
#ifndef STREAM_BAR2
#define STREAM_BAR2 1
#endif
#ifndef STREAM_PRIO_QB1
#define STREAM_PRIO_QB1 0
#endif
constexpr float L_LIMIT = 1.0e30f;    // a finite row sum at most this is not an overflow

// Sizes that follow from the head size D (16, 32, 64 or 128).
template <int D>
struct StreamDims {
    static constexpr int TILE = SKT * D * 2;      // bytes of one K (or V) tile
    // d = 16: the PV MFMA's 32-wide d block is half used; its upper 16 rows
    // take V^T rows of ones from a 1 KB block after the V tile, so that
    // those accumulator rows sum the rounded weights (the row sum l).
    static constexpr bool LSUM = D == 16;
    static constexpr int STAGE = 2 * TILE + (LSUM ? 1024 : 0);  // K tile, V tile (, ones)
    static constexpr int NS = D == 128 ? 4 : 6;   // ring stages
    static constexpr int CPR = D / 8;             // 16-byte chunks per row
    static constexpr int SWZ = CPR < 8 ? CPR : 8; // chunks permuted together
    static constexpr int KK = D / 16;             // k slices of a score MFMA
    static constexpr int DB = D < 32 ? 1 : D / 32;  // 32-wide d blocks of a PV MFMA
    // Tiles of at least 4 KB: every thread loads LPT chunks of K and of V.
    // Smaller ones (D = 16, 32): waves 0 and 1 load K, waves 2 and 3 V, as
    // many as the tile needs, one chunk per thread.
    static constexpr bool SMALL = TILE < 64 * SNW * 16;
    static constexpr int LPT = SMALL ? 1 : TILE / (64 * SNW * 16);
    static constexpr int DMA = SMALL ? 1 : 2 * LPT;  // loads per loading thread per tile
    static_assert(NS >= 4 && NS % 2 == 0, "ring: two tiles read, two in flight at least");
    static_assert(D == 16 || D == 32 || D == 64 || D == 128, "head size");
    static_assert(!SMALL || TILE <= 2048, "a small tile takes at most two waves");
};

// Tiles from a wave's first whose rows set their reference exactly: the
// first tile holds every row's first legal key (key 0), except under
// restricted attention, where the band of the wave's last row (31 rows on
// with one query block, 63 with two) starts up to one (two) tiles later.
template <bool WIN, int QB>
constexpr int stream_init_tiles() {
    return WIN ? 1 + QB : 1;
}

// Query blocks of 32 per wave (QB = 1 or 2) and the workgroups per CU the
// register budget then allows.
template <int D, int QB>
constexpr int stream_occupancy() {
    return D <= 32 ? (QB == 1 ? 4 : 3) : (D == 64 && QB == 1) ? 3 : 2;
}

template <int D, int QB, bool PAD, bool CAUSAL, bool WIN>
__global__ __launch_bounds__(64 * SNW, (stream_occupancy<D, QB>())) void attn_stream_bf16(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    bf16* __restrict__ o, const int32_t* __restrict__ kv_lens, int B, int H, int Lq, int Lk,
    int n_qtiles, float scale_log2e, int window) {
    using Dm = StreamDims<D>;
    constexpr int SD = D;
    constexpr int SNS = Dm::NS;
    constexpr int STILE = Dm::TILE;
    constexpr int SSTAGE = Dm::STAGE;
    constexpr int SDMA = Dm::DMA;
    constexpr int CPR = Dm::CPR;
    constexpr int KK = Dm::KK;
    constexpr int DB = Dm::DB;
    constexpr int ROWB = CPR * 16;  // bytes of a K, V or O row in LDS
    // Chunk permutations of a row: K rows by row & 7 (by row & 1 or row & 3
    // for rows of 2 or 4 chunks), V rows by 4 ((row >> 1) & 1) for rows of 8
    // chunks or more and not at all for shorter ones.
    auto kswz = [](int r) { return r & (Dm::SWZ - 1); };
    auto vswz = [](int r) { return Dm::SWZ == 8 ? v_swz(r) : 0; };
    // the ring; the recomputation after it takes one stage per wave
    __shared__ __attribute__((aligned(1024))) char smem[(SNS > SNW ? SNS : SNW) * SSTAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const int g = lane >> 4;
    const int i16 = lane & 15;

    // Workgroup -> (batch row, head, query block).  Workgroups go to the 8
    // XCDs round-robin (workgroup w on XCD w % 8); when B*H divides by 8,
    // XCD x gets the (batch row, head) pairs x*nbh/8 .. (x+1)*nbh/8 - 1
    // whole, so every query block of a pair shares that XCD's L2 for its
    // K/V.  Causal: within each XCD the longest query blocks start first.
    // A causal band keeps the pair-major order: its workgroups carry about
    // equal work, and neighbouring query blocks, which share most of their
    // keys, then run together while those keys are in L2 (longest-first
    // spreads a pair's blocks over the whole launch, and K/V is fetched
    // again from HBM).
    constexpr int SQB = QB;                // 32-query blocks per wave
    constexpr int SWQ = 32 * SQB;          // queries per wave
    constexpr int SBM = SWQ * SNW;         // queries per workgroup
    constexpr int NPV = 2 * DB * SQB;      // PV MFMAs per tile (two 16-key chunks)
    constexpr int NSL = NPV + KK * SQB;    // MFMAs per tile
    constexpr int NPR = 8 * SQB;           // pairs of scores per lane per tile
    // At least one MFMA per pair (d >= 64): a slot per MFMA, RAT slots per
    // pair (1 at d = 64, 2 at d = 128).  Fewer (d = 16, 32): a slot per
    // pair, the MFMAs spread over them.
    constexpr bool DENSE = NSL >= NPR;
    constexpr int RAT = DENSE ? NSL / NPR : 1;
    static_assert(!DENSE || (NSL == RAT * NPR && (RAT == 1 || RAT == 2)), "slots per pair");
    constexpr int SNI = stream_init_tiles<WIN, SQB>();
    // a barrier every other tile (six ring stages), else every tile
    constexpr bool BAR2 = STREAM_BAR2 && Dm::NS >= 6;
    // The slots raise the wave's priority with two query blocks per wave
    // (two waves per SIMD, 1% faster); with one block (three or four waves
    // per SIMD) the waves keep equal priority (3% faster on causal rows).
    constexpr bool PRIO = STREAM_PRIO_QB1 || SQB == 2;
    const int nbh = B * H;
    const int w = (int)blockIdx.x;
    int bh, qt;
    if ((nbh & 7) == 0) {
        const int x = w & 7, slot = w >> 3, per = nbh >> 3;
        if (CAUSAL && !WIN) {
            qt = n_qtiles - 1 - slot / per;
            bh = x * per + slot % per;
        } else {
            bh = x * per + slot / n_qtiles;
            qt = slot % n_qtiles;
        }
    } else if (CAUSAL && !WIN) {
        qt = n_qtiles - 1 - w / nbh;
        bh = w % nbh;
    } else {
        bh = w / n_qtiles;
        qt = w % n_qtiles;
    }
    const int b = bh / H;
    const int hh = bh - b * H;
    const int q0 = qt * SBM;

    int kv_end = Lk;
    if (PAD) kv_end = min(max(kv_lens[b], 0), Lk);
    int key_end = kv_end;
    if (CAUSAL) key_end = min(key_end, min(q0 + SBM, Lq));
    // The workgroup streams tiles t_first .. n_tiles - 1 (a band around its
    // queries when WIN; window < Lk, so no sum below overflows).
    int t_first = 0;
    if (WIN) {
        key_end = min(key_end, q0 + SBM + window);
        t_first = max(q0 - window, 0) / SKT;
    }
    const int n_tiles = (key_end + SKT - 1) / SKT;
    const int n_loop = max(n_tiles - t_first, 0);

    // Tiles this wave computes, w_first .. n_mine - 1: none if it holds no
    // query row; causal stops at the tile holding the wave's last query; a
    // band starts and stops a window away from the wave's queries.
    const int wq0 = q0 + SWQ * wave;
    int n_mine = (wq0 < Lq) ? n_tiles : 0;
    if (CAUSAL) n_mine = min(n_mine, (wq0 + SWQ + SKT - 1) / SKT);
    int w_first = t_first;
    if (WIN) {
        n_mine = min(n_mine, (min(kv_end, wq0 + SWQ + window) + SKT - 1) / SKT);
        w_first = max(wq0 - window, 0) / SKT;
    }

    const size_t rs = (size_t)H * SD;  // elements between consecutive positions
    const uint32_t rsb = (uint32_t)(rs * sizeof(bf16));
    const bf16* qp = q + ((size_t)b * Lq * H + hh) * SD;
    const bf16* kp = k + ((size_t)b * Lk * H + hh) * SD;
    const bf16* vp = v + ((size_t)b * Lk * H + hh) * SD;
    bf16* op = o + ((size_t)b * Lq * H + hh) * SD;

    bf16x8 qop[SQB][KK];  // Q as the B operand of S^T = K Q^T (loaded in the prologue)

    // Direct global-to-LDS tile loads: thread tid fills chunk positions
    // tid + 256u of a tile (row position / CPR), fetching the chunk the
    // swizzle puts there; rows at or past kv_end land as zeros without a
    // memory access.
    const uint32_t kv_bytes = kv_end > 0 ? (uint32_t)(kv_end - 1) * rsb + SD * 2 : 0u;
    const __amdgpu_buffer_rsrc_t krsrc = make_rsrc(kp, kv_bytes);
    const __amdgpu_buffer_rsrc_t vrsrc = make_rsrc(vp, kv_bytes);
    uint32_t k_dma[Dm::LPT], v_dma[Dm::LPT];
    // Small tiles: this wave's 1 KB piece of the K (waves 0, 1) or V (waves
    // 2, 3) tile, if the tile has one.
    const int sub = wave & 1;
    const bool small_v = wave >= 2;
    const bool loads = !Dm::SMALL || 1024 * sub < STILE;
#pragma unroll
    for (int u = 0; u < Dm::LPT; ++u) {
        const int pos = Dm::SMALL ? 64 * sub + lane : tid + 256 * u;
        const int pr = pos / CPR, pc = pos % CPR;
        k_dma[u] = (uint32_t)pr * rsb + 16 * (pc ^ kswz(pr));
        v_dma[u] = (uint32_t)pr * rsb + 16 * (pc ^ vswz(pr));
    }
    const uint32_t tile_gbytes = (uint32_t)SKT * rsb;
    // A wave's 1 KB piece of each 4 KB of a stage (small tiles: of its tile).
    const uint32_t lds_wave = Dm::SMALL ? lds_addr(smem) + (small_v ? STILE : 0) + 1024 * sub
                                        : lds_addr(smem) + 1024 * wave;
    // Tile t (of the workgroup's stream, jr = t - t_first) into `stage`
    // (jr % SNS).
    auto dma = [&](int jr, int stage) {
        const int t = t_first + jr;
        const uint32_t base = t < n_tiles ? (uint32_t)t * tile_gbytes : OOB_OFFSET;
        const uint32_t st = lds_wave + (uint32_t)stage * SSTAGE;
        if (Dm::SMALL) {
            if (loads) {
                if (small_v) load_lds16(vrsrc, st, base + v_dma[0]);
                else load_lds16(krsrc, st, base + k_dma[0]);
            }
            return;
        }
#pragma unroll
        for (int u = 0; u < Dm::LPT; ++u) {
            load_lds16(krsrc, st + 4096u * u, base + k_dma[u]);
            load_lds16(vrsrc, st + STILE + 4096u * u, base + v_dma[u]);
        }
    };

    // LDS operand offsets inside a stage (same lane patterns as the
    // whole-row kernel): K rows for S^T, V^T by transpose reads.
    // (Chunks 8 and on of a d = 128 row sit 128 bytes after chunks 0 .. 7,
    // the swizzle permuting only within each group of eight.)
    uint32_t k_rd[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        k_rd[kk] = l32 * ROWB + 16 * (((2 * kk + half) & (CPR - 1)) ^ kswz(l32));
    uint32_t v_rd[DB];
    {
        const int row = 4 * half + (i16 >> 2);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int chunk = (4 * db + 2 * (g & 1) + ((i16 & 3) >> 1)) & (CPR - 1);
            v_rd[db] = STILE + row * ROWB + 16 * (chunk ^ vswz(row)) + 8 * (i16 & 1);
            // d = 16: lanes 16-31 and 48-63 hold the block's upper rows;
            // they read the ones (every read of read_vt lands in the block:
            // offsets below 64, plus at most 512 + 256 + 8)
            if (Dm::LSUM && (g & 1)) v_rd[db] = 2 * STILE + 8 * (i16 & 7);
        }
    }
    auto read_k = [&](int stage, bf16x8 (&ka)[KK]) {
        const char* base = smem + stage * SSTAGE;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) ka[kk] = *(const bf16x8*)(base + k_rd[kk & 3] + 128 * (kk >> 2));
    };
    // V^T operands [16-key chunk][d block] of the tile in `stage`.
    auto read_vt = [&](int stage, bf16x8 (&va)[2][DB]) {
        const char* base = smem + stage * SSTAGE;
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int db = 0; db < DB; ++db)
                va[c][db] = join(lds_read_tr((const bf16*)(base + 16 * ROWB * c + v_rd[db])),
                                 lds_read_tr((const bf16*)(base + 16 * ROWB * c + v_rd[db] + 8 * ROWB)));
    };

    f32x16 acc[SQB][DB];
#pragma unroll
    for (int qb = 0; qb < SQB; ++qb)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[qb][db][r] = 0.0f;
    // Per query row (this lane's column): the reference m (raw logit units),
    // m * scale_log2e, and this lane's share of the row sum.
    float m_run[SQB], mc[SQB], l_part[SQB];
#pragma unroll
    for (int qb = 0; qb < SQB; ++qb) {
        m_run[qb] = -INFINITY;
        mc[qb] = -INFINITY;
        l_part[qb] = 0.0f;
    }
    const f32x16 zero16 = {};
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};

    // Mask S_j (boundary tiles only): -inf at illegal pairs.
    auto mask_tile = [&](int j, f32x16 (&S)[SQB]) {
        const int k0 = j * SKT;
        const bool need = (k0 + SKT > kv_end) || (CAUSAL && k0 + SKT - 1 > wq0) ||
                          (WIN && (k0 < wq0 + SWQ - 1 - window || k0 + SKT - 1 > wq0 + window));
        if (!need) return;
#pragma unroll
        for (int qb = 0; qb < SQB; ++qb) {
            const int qi = wq0 + 32 * qb + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = k0 + acc_row(r, half);
                bool legal = key < kv_end;
                if (CAUSAL) legal = legal && key <= qi;
                if (WIN) legal = legal && key >= qi - window && key <= qi + window;
                S[qb][r] = legal ? S[qb][r] : -INFINITY;
            }
        }
    };

    // The reference of tile j's rows when it moves (the wave's first tiles,
    // and every tile of the recomputation): the running maximum over the
    // tile's legal values; acc and l are rescaled by exp2(m_old - m_new)
    // (0 while nothing has accumulated; 1 while a row has no legal key).
    // Returns the factors, which the caller applies to acc once the
    // previous tile's PV has landed in it.
    auto move_reference = [&](const f32x16 (&S)[SQB], float (&alpha)[SQB]) {
#pragma unroll
        for (int qb = 0; qb < SQB; ++qb) {
            float mx = S[qb][0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S[qb][r]);
            mx = max_halves(mx);
            const float m_new = fmaxf(m_run[qb], mx);
            alpha[qb] = (m_new == -INFINITY || m_new == m_run[qb])
                            ? 1.0f
                            : __builtin_amdgcn_exp2f((m_run[qb] - m_new) * scale_log2e);
            m_run[qb] = m_new;
            mc[qb] = m_new * scale_log2e;
        }
    };
    auto rescale = [&](const float (&alpha)[SQB]) {
#pragma unroll
        for (int qb = 0; qb < SQB; ++qb) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[qb][db][r] *= alpha[qb];
            l_part[qb] *= alpha[qb];
        }
    };

    // One tile j of the pipeline: NSL slots, each issuing one MFMA, and
    // beside them the softmax of S_j, a pair of values at a time.  Pair n
    // is values 2(n%8), 2(n%8)+1 of query block n/8; its four steps --
    // scale and offset (two FMAs), two exponentials, the rounding to a
    // packed bf16 pair in Pcur, the row-sum step -- run one slot apart
    // (slots n-2 .. n+1 at d = 64, one pair per slot) or two apart (slots
    // 2n-3 .. 2n at d = 128, where a tile has twice the MFMAs), so no
    // instruction waits for the one just before it.  The MFMAs: the first
    // NPV slots the PV of tile j-1 from Pprev and the V^T operands in va
    // (16-key chunk, query block, d block); the rest the scores of tile
    // j+1 (k slice, query block), by when its K rows have arrived from
    // LDS.  Between the two the V^T reads of tile j (for its PV in the next
    // tile) are issued, so they land before the tile ends and the barrier
    // does not wait for them.  The wave's first SNI tiles (`exact`, a
    // wave-uniform flag) move the reference first.
    auto tile_step = [&](bool exact, int j, int stage_cur, f32x16 (&Scur)[SQB],
                         f32x16 (&Snext)[SQB], const bf16x8 (&Pprev)[SQB][2],
                         bf16x8 (&Pcur)[SQB][2], bf16x8 (&va)[2][DB]) {
        const int stage_next = (stage_cur + 1) % SNS;
        bf16x8 ka[KK];
        read_k(stage_next, ka);
        mask_tile(j, Scur);
        float alpha[SQB], off[SQB];
        if (exact) move_reference(Scur, alpha);
        // Rows with no reference yet (no legal key so far) keep mc = -inf,
        // which in the common path turns any value they meet into inf or
        // NaN, so such a row ends non-finite and is recomputed; the exact
        // tiles give them weight 0 (all their values are -inf) instead.
#pragma unroll
        for (int qb = 0; qb < SQB; ++qb)
            off[qb] = (exact && m_run[qb] == -INFINITY) ? 0.0f : mc[qb];
        float lt[SQB];
        float xs[NPR][2], ex[NPR][2];
        bf16x2 pk[NPR];
        auto step_fma = [&](int n) {
            if (n < 0 || n >= NPR) return;
            const int qb = n >> 3, i = n & 7;
            xs[n][0] = __builtin_fmaf(Scur[qb][2 * i], scale_log2e, -off[qb]);
            xs[n][1] = __builtin_fmaf(Scur[qb][2 * i + 1], scale_log2e, -off[qb]);
        };
        auto step_exp = [&](int n) {
            if (n < 0 || n >= NPR) return;
            ex[n][0] = __builtin_amdgcn_exp2f(xs[n][0]);
            ex[n][1] = __builtin_amdgcn_exp2f(xs[n][1]);
        };
        auto step_round = [&](int n) {
            if (n < 0 || n >= NPR) return;
            const int qb = n >> 3, i = n & 7;
            pk[n] = bf16x2{(bf16)ex[n][0], (bf16)ex[n][1]};
            Pcur[qb][i >> 2][2 * (i & 3)] = pk[n][0];
            Pcur[qb][i >> 2][2 * (i & 3) + 1] = pk[n][1];
        };
        auto step_sum = [&](int n) {
            if (Dm::LSUM || n < 0 || n >= NPR) return;
            const int qb = n >> 3, i = n & 7;
            lt[qb] = __builtin_amdgcn_fdot2_f32_bf16(pk[n], ones, i == 0 ? 0.0f : lt[qb], false);
        };
        // The softmax steps beside slot s (negative: before the first MFMA).
        auto slot_steps = [&](int s) {
            if (RAT == 1) {
                step_fma(s + 2);
                step_exp(s + 1);
                step_round(s);
                step_sum(s - 1);
            } else if ((s & 1) != 0) {
                step_fma((s + 3) / 2);
                step_round((s + 1) / 2);
            } else {
                step_exp((s + 2) / 2);
                step_sum(s / 2);
            }
        };
#pragma unroll
        for (int s = -RAT - 1; s < 0; ++s) slot_steps(s);
        __builtin_amdgcn_sched_barrier(0);
        if (PRIO) __builtin_amdgcn_s_setprio(1);
        constexpr int NSLOT = DENSE ? NSL : NPR;  // slots with an MFMA or a pair's step
#pragma unroll
        for (int s = 0; s < NSLOT + (RAT == 1 ? 1 : 0); ++s) {
            __builtin_amdgcn_sched_barrier(0);
            // the MFMA of slot s: MFMA s, or (sparse) MFMA m in the first
            // slot s with s NSL / NPR >= m
            const int m = DENSE ? (s < NSL ? s : -1)
                                : (s < NPR && (s * NSL) % NPR < NSL ? (s * NSL) / NPR : -1);
            if (m >= 0 && m < NPV) {
                const int c = m / (DB * SQB), qb = (m / DB) % SQB, db = m % DB;
                acc[qb][db] = mfma32(va[c][db], Pprev[qb][c], acc[qb][db]);
            } else if (m >= NPV) {
                if (m == NPV) read_vt(stage_cur, va);  // V^T of tile j, for the next tile
                const int mm = m - NPV, kk = mm / SQB, qb = mm % SQB;
                Snext[qb] = mfma32(ka[kk], qop[qb][kk], kk == 0 ? zero16 : Snext[qb]);
            }
            slot_steps(s);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (PRIO) __builtin_amdgcn_s_setprio(0);
        if (exact) rescale(alpha);  // acc now holds tile j-1's PV
        if (!Dm::LSUM) {
#pragma unroll
            for (int qb = 0; qb < SQB; ++qb) l_part[qb] += lt[qb];
        }
    };

    // ---- prologue: tiles 0 .. SNS-3 and Q in flight together, then all
    // of them waited for.  (The tile loads are inline asm, invisible to the
    // compiler's wait bookkeeping; with Q's loads retired before the loop,
    // the waits it places for them stay out of the loop, where they would
    // also wait for the tile loads in flight.)
    if (Dm::LSUM) {  // the ones blocks of every stage (read after the first barrier)
        const bf16x2 one2 = {(bf16)1.0f, (bf16)1.0f};
        const uint32_t o = __builtin_bit_cast(uint32_t, one2);
        const uint4 ones4 = {o, o, o, o};
        for (int i = tid; i < SNS * 64; i += 64 * SNW)
            *(uint4*)(smem + (i >> 6) * SSTAGE + 2 * STILE + 16 * (i & 63)) = ones4;
    }
#pragma unroll
    for (int jr = 0; jr < SNS - 2; ++jr) dma(jr, jr);
    // Q as the B operand of S^T = K Q^T: block qb, lane holds query
    // wq0 + 32qb + l32, d = 16kk + 8half .. +7.  Rows past Lq read zeros.
    const __amdgpu_buffer_rsrc_t qrsrc =
        make_rsrc(qp, (uint32_t)(((size_t)(Lq - 1) * rs + SD) * sizeof(bf16)));
#pragma unroll
    for (int qb = 0; qb < SQB; ++qb) {
        const int qi = wq0 + 32 * qb + l32;
        const uint32_t qoff = qi < Lq ? (uint32_t)qi * rsb + 16 * half : OOB_OFFSET;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qop[qb][kk] = buffer_load16(qrsrc, qoff + 32 * kk);
    }
    // Q's values are consumed here, so the compiler's own wait for them
    // (which also covers the tile loads issued before them) lands here.
#pragma unroll
    for (int qb = 0; qb < SQB; ++qb)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) asm volatile("" ::"v"(qop[qb][kk]));

    f32x16 SA[SQB], SB[SQB];
    // Weights of alternate tiles (the previous tile's wait for their PV);
    // V^T of tile j-1.
    bf16x8 PA[SQB][2], PB[SQB][2], va[2][DB];
#pragma unroll
    for (int qb = 0; qb < SQB; ++qb)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            PA[qb][c] = zero_bf16x8();
            PB[qb][c] = zero_bf16x8();
        }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int db = 0; db < DB; ++db) va[c][db] = zero_bf16x8();

    // Iteration jr (tile j = t_first + jr, stage jr % SNS) reads tile j's
    // V and tile j + 1's K.  With a 4-stage ring it first waits for tile
    // j + 1 (each thread for its own loads of it, the barrier for
    // everyone's), after which every wave is done with tile j - 2's stage,
    // which the load of tile j + 2 then takes.  With six stages the waves
    // meet every other tile: at even jr each waits for all of its loads
    // (tiles up to j + 3, issued two iterations before), and after the
    // barrier tiles j + 4 and j + 5 go to the stages of tiles j - 2 and
    // j - 1, which every wave has left; odd iterations neither wait nor
    // load.  The loop body is unrolled over the ring so every LDS offset is
    // an immediate (and jr's parity is that of the stage); the score and
    // weight register sets alternate with the tile's parity.
    auto iteration = [&](int jr, f32x16 (&Scur)[SQB], f32x16 (&Snext)[SQB],
                         const bf16x8 (&Pprev)[SQB][2], bf16x8 (&Pcur)[SQB][2], int stage) {
        if (!BAR2) {
            wait_vmcnt<SDMA * (SNS - 4)>();
            barrier_lds();
            dma(jr + SNS - 2, (stage + SNS - 2) % SNS);
        } else if ((stage & 1) == 0) {
            wait_vmcnt<0>();
            barrier_lds();
            dma(jr + SNS - 2, (stage + SNS - 2) % SNS);
            dma(jr + SNS - 1, (stage + SNS - 1) % SNS);
        }
        const int j = t_first + jr;
        const bool active = j >= w_first && j < n_mine;
        if (j == w_first && j < n_mine) {
            // the wave's first tile: its scores straight from the ring
            bf16x8 ka[KK];
            read_k(stage, ka);
#pragma unroll
            for (int qb = 0; qb < SQB; ++qb) {
                Scur[qb] = mfma32(ka[0], qop[qb][0], zero16);
#pragma unroll
                for (int kk = 1; kk < KK; ++kk) Scur[qb] = mfma32(ka[kk], qop[qb][kk], Scur[qb]);
            }
        }
        if (active) {
            tile_step(j < w_first + SNI, j, stage, Scur, Snext, Pprev, Pcur, va);
        }
    };
    // Unrolled over the ring (twice when SNS is odd, so the register sets
    // alternate in step): stage u % SNS of copy u is a constant.
    constexpr int UNR = SNS % 2 == 0 ? SNS : 2 * SNS;
    for (int jr = 0; jr < n_loop; jr += UNR) {
#pragma unroll
        for (int u = 0; u < UNR; u += 2) {
            if (jr + u < n_loop) iteration(jr + u, SA, SB, PB, PA, u % SNS);
            if (jr + u + 1 < n_loop) iteration(jr + u + 1, SB, SA, PA, PB, (u + 1) % SNS);
        }
    }
    // Drain: the PV of the wave's last tile (zero weights if it had none),
    // whose weights sit in the set of that tile's parity.
    wait_vmcnt<0>();
    const bool last_odd = n_mine > w_first && ((n_mine - 1 - t_first) & 1) != 0;
#pragma unroll
    for (int qb = 0; qb < SQB; ++qb)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const bf16x8 pl = last_odd ? PB[qb][c] : PA[qb][c];
#pragma unroll
            for (int db = 0; db < DB; ++db) acc[qb][db] = mfma32(va[c][db], pl, acc[qb][db]);
        }

    // Every wave is done with the ring (its loads landed, its reads
    // retired): from here on each wave has its own stage to itself.
    barrier_lds();

    // ---- epilogue: O = acc / l, or 0 for a row with no legal key.  A row
    // whose sum or outputs are not finite (or whose sum exceeds L_LIMIT) is
    // not stored here but recomputed below; `bad` has bit l (and l + 32) set
    // for such a row l of the block, the two lanes holding it decide
    // together.  The 32 x D block goes through the wave's stage (chunks
    // swizzled by row within each group of eight) so that each store writes
    // whole rows (eight of 128 bytes, or four of 256): a lane holds a
    // query's column, a store wants its row.  The first pass
    // (again = false) stores the good rows and returns `bad`; the second
    // stores the rows `first_bad` marks.  Called with every lane active.
    char* const stg = smem + wave * SSTAGE;
    auto finish = [&](int qb, bool again, uint64_t first_bad) -> uint64_t {
        // (d = 16: accumulator row 16 + 4 half, element 8, holds l)
        const float l_tot = Dm::LSUM ? acc[qb][0][8] : sum_halves(l_part[qb]);
        const float inv = (l_tot > 0.0f) ? 1.0f / l_tot : 0.0f;
        bool ok = l_tot <= L_LIMIT;  // false for inf and NaN
        char* const blk = stg + 64 * SD * qb;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                if (4 * db + rg >= CPR) continue;  // d = 16: the block's unused half
                bf16x4 out;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x = acc[qb][db][4 * rg + e] * inv;
                    ok = ok && __builtin_fabsf(x) <= 3.0e38f;
                    out[e] = (bf16)x;
                }
                // d = 32db + 8rg + 4half .. +3: chunk 4db + rg, half of it
                *(bf16x4*)(blk + l32 * ROWB + 16 * ((4 * db + rg) ^ kswz(l32)) + 8 * half) = out;
            }
        const uint64_t bad = __builtin_amdgcn_ballot_w64(!ok);
        const uint64_t marked = again ? first_bad : bad;
        const int cc = lane % CPR;
#pragma unroll
        for (int k = 0; k < CPR / 2; ++k) {
            const int r = lane / CPR + (64 / CPR) * k;
            const bf16x8 row = *(const bf16x8*)(blk + r * ROWB + 16 * (cc ^ kswz(r)));
            const int qi = wq0 + 32 * qb + r;
            const bool r_marked = ((marked >> r) | (marked >> (r + 32))) & 1;
            if (qi < Lq && r_marked == again) *(bf16x8*)(op + (size_t)qi * rs + 8 * cc) = row;
        }
        return bad;
    };
    uint64_t redo[SQB];
#pragma unroll
    for (int qb = 0; qb < SQB; ++qb) redo[qb] = finish(qb, false, 0);

    // ---- recomputation of the rows that overflowed (rare: a key more than
    // ~88 scaled-logit units above the row's first tiles), with a reference
    // that moves every tile.  The wave streams its tiles alone through its
    // own stage, one tile at a time, and stores only the recomputed rows
    // (the block's staged reads above are retired: their rows were stored).
    bool any_redo = false;
#pragma unroll
    for (int qb = 0; qb < SQB; ++qb) any_redo = any_redo || redo[qb] != 0;
    if (any_redo) {
        // the staged reads retire before loads into the stage are issued
        __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));
        asm volatile("" ::: "memory");
#pragma unroll
        for (int qb = 0; qb < SQB; ++qb) {
            m_run[qb] = -INFINITY;
            mc[qb] = -INFINITY;
            l_part[qb] = 0.0f;
#pragma unroll
            for (int db = 0; db < DB; ++db) acc[qb][db] = zero16;
        }
        const uint32_t st = lds_addr(smem) + (uint32_t)wave * SSTAGE;
        for (int j = w_first; j < n_mine; ++j) {
            const uint32_t base = (uint32_t)j * tile_gbytes;
#pragma unroll
            for (int u = 0; u < STILE / 1024; ++u) {
                const int c = lane + 64 * u, r = c / CPR, cc = c % CPR;
                load_lds16(krsrc, st + 1024u * u, base + (uint32_t)r * rsb + 16 * (cc ^ kswz(r)));
                load_lds16(vrsrc, st + STILE + 1024u * u,
                           base + (uint32_t)r * rsb + 16 * (cc ^ vswz(r)));
            }
            wait_vmcnt<0>();
            f32x16 S[SQB];
            bf16x8 ka[KK], vt[2][DB], P[SQB][2];
            read_k(wave, ka);
#pragma unroll
            for (int qb = 0; qb < SQB; ++qb) {
                S[qb] = mfma32(ka[0], qop[qb][0], zero16);
#pragma unroll
                for (int kk = 1; kk < KK; ++kk) S[qb] = mfma32(ka[kk], qop[qb][kk], S[qb]);
            }
            mask_tile(j, S);
            float alpha[SQB];
            move_reference(S, alpha);
            rescale(alpha);
#pragma unroll
            for (int qb = 0; qb < SQB; ++qb) {
                const float o = m_run[qb] == -INFINITY ? 0.0f : mc[qb];
                float lt = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[qb][2 * i], scale_log2e, -o));
                    const float p1 =
                        __builtin_amdgcn_exp2f(__builtin_fmaf(S[qb][2 * i + 1], scale_log2e, -o));
                    const bf16x2 pp = {(bf16)p0, (bf16)p1};
                    P[qb][i >> 2][2 * (i & 3)] = pp[0];
                    P[qb][i >> 2][2 * (i & 3) + 1] = pp[1];
                    lt = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, lt, false);
                }
                l_part[qb] += lt;
            }
            read_vt(wave, vt);
#pragma unroll
            for (int qb = 0; qb < SQB; ++qb)
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int db = 0; db < DB; ++db)
                        acc[qb][db] = mfma32(vt[c][db], P[qb][c], acc[qb][db]);
            // this tile's LDS reads are done before the next tile's loads
            // overwrite the stage
            __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));
            asm volatile("" ::: "memory");
        }
#pragma unroll
        for (int qb = 0; qb < SQB; ++qb)
            if (redo[qb] != 0) finish(qb, true, redo[qb]);
    }
}

template <int D, int QB, bool WIN>
hipError_t launch_stream(const AttnArgs& a, hipStream_t stream) {
    const int bm = 32 * QB * SNW;
    const dim3 block(64 * SNW);
    const int n_qtiles = (a.Lq + bm - 1) / bm;
    const dim3 grid((unsigned)((long)a.B * a.H * n_qtiles));
    const float sl2e = (float)(1.4426950408889634 / sqrt((double)D));
    const bf16* q = (const bf16*)a.q;
    const bf16* k = (const bf16*)a.k;
    const bf16* v = (const bf16*)a.v;
    bf16* o = (bf16*)a.o;
    switch (a.mask) {
        case 0:
            hipLaunchKernelGGL((attn_stream_bf16<D, QB, false, false, WIN>), grid, block, 0,
                               stream, q, k, v, o, a.kv_lens, a.B, a.H, a.Lq, a.Lk, n_qtiles,
                               sl2e, a.window);
            break;
        case 1:
            hipLaunchKernelGGL((attn_stream_bf16<D, QB, true, false, WIN>), grid, block, 0,
                               stream, q, k, v, o, a.kv_lens, a.B, a.H, a.Lq, a.Lk, n_qtiles,
                               sl2e, a.window);
            break;
        case 2:
            hipLaunchKernelGGL((attn_stream_bf16<D, QB, false, true, WIN>), grid, block, 0,
                               stream, q, k, v, o, a.kv_lens, a.B, a.H, a.Lq, a.Lk, n_qtiles,
                               sl2e, a.window);
            break;
        default:
            hipLaunchKernelGGL((attn_stream_bf16<D, QB, true, true, WIN>), grid, block, 0,
                               stream, q, k, v, o, a.kv_lens, a.B, a.H, a.Lq, a.Lk, n_qtiles,
                               sl2e, a.window);
            break;
    }
    return hipGetLastError();
}

}  // namespace

// Workgroups of 128 queries (one block of 32 per wave, three workgroups per
// CU) where work per workgroup is short or uneven: restricted attention,
// whose workgroup streams its queries' span plus the window, so a narrower
// span wastes fewer keys; and causal rows up to 2048 queries, where the
// spread of workgroup lengths and the diagonal tiles some waves sit out
// weigh most.  Workgroups of 256 queries otherwise.
// At d = 128 a wave holds one block of 32 queries (two workgroups per CU);
// at d = 16 and 32 likewise (four workgroups per CU; two blocks per wave ran
// slower).
hipError_t launch_attention_stream_bf16(const AttnArgs& a, hipStream_t stream) {
    switch (a.D) {
        case 16:
            return a.window >= 0 ? launch_stream<16, 1, true>(a, stream)
                                 : launch_stream<16, 1, false>(a, stream);
        case 32:
            return a.window >= 0 ? launch_stream<32, 1, true>(a, stream)
                                 : launch_stream<32, 1, false>(a, stream);
        case 128:
            return a.window >= 0 ? launch_stream<128, 1, true>(a, stream)
                                 : launch_stream<128, 1, false>(a, stream);
        case 64: break;
        default: return hipErrorInvalidValue;
    }
    if (a.window >= 0) return launch_stream<64, 1, true>(a, stream);
    const bool causal = (a.mask & 2) != 0;
    return causal && a.Lq <= 2048 ? launch_stream<64, 1, false>(a, stream)
                                  : launch_stream<64, 2, false>(a, stream);
}

}  // namespace mha
