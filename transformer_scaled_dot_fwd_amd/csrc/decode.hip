// decode.hip -- one decoding step of attention against a key/value cache:
//
//   o_b,t = softmax(q_b,t K_b,t^T / sqrt(d_k)) V_b,t     keys 0 .. len_b - 1
//
// ("Paper Deep Reading", section 04, attention equation; the decoder
// produces one position per step and attends to every earlier one, section
// 03 "Decoder layer" with the causal mask: for the newest position that is
// the whole cache, so the only mask left is the cache length.)  One query
// per (sequence, head) makes this HBM-bound: each cached key costs 4 d bytes
// of K and V for 4 d FLOPs.  The key range is therefore split over many
// workgroups (split-K) that each stream a chunk of K/V at full bandwidth and
// leave a partial softmax state (running max m, sum l, unnormalised acc),
// and a second kernel merges a (sequence, head)'s partial states in a fixed
// order (deterministic), the exact identity softmax(x) = softmax(x - c)
// applied chunk by chunk.
//
// Arithmetic is fp32 on the VALU: the scores stay in fp32 (no bf16 rounding
// of p), and exp2 with log2(e) / sqrt(d_k) folded into q.
#include "device.h"
#include "launch.h"

namespace mha {
namespace {

constexpr int DEC_CHUNK = 256;   // keys per workgroup
constexpr int DEC_WAVES = 4;

// One lane group of 8 lanes holds one key; lane s of the group holds d
// elements E s .. E s + E - 1 (E = D / 8) of q, of that key's K and V rows,
// and of the group's accumulator.
template <int D>
struct DecState {
    float m, l;
    float acc[D / 8];
};

// Combine two partial softmax states of the same query (log2 units).
template <int D>
__device__ __forceinline__ void dec_merge(DecState<D>& a, float m2, float l2, const float* acc2) {
    const float m = fmaxf(a.m, m2);
    if (m == -INFINITY) return;  // both empty
    const float sa = __builtin_amdgcn_exp2f(a.m - m);  // 0 when a is empty
    const float sb = __builtin_amdgcn_exp2f(m2 - m);
    a.l = a.l * sa + l2 * sb;
#pragma unroll
    for (int e = 0; e < D / 8; ++e) a.acc[e] = a.acc[e] * sa + acc2[e] * sb;
    a.m = m;
}

// Partial state of (sequence b, head t, chunk s) into part[((b H + t) S + s)
// (D + 2) ..]: acc[0 .. D-1], m, l.
template <int D>
__global__ __launch_bounds__(64 * DEC_WAVES) void decode_partial_bf16(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const int32_t* __restrict__ lens, float* __restrict__ part, int H, int L, int n_split,
    float scale_log2e) {
    constexpr int E = D / 8;            // elements per lane
    constexpr int NL = E / 8;           // 16-byte loads per lane per row
    static_assert(D == 64 || D == 128, "head size");
    __shared__ float red[DEC_WAVES][D + 2];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 3;            // key group: one key per round
    const int sl = lane & 7;            // d slice
    const int w = (int)blockIdx.x;
    const int s = w % n_split;
    const int bt = w / n_split;
    const int b = bt / H, t = bt - (bt / H) * H;

    const int len = min(max(lens[b], 0), L);
    const int k0 = s * DEC_CHUNK;
    const int k1 = min(k0 + DEC_CHUNK, len);

    // q slice, pre-scaled to log2 units
    float qv[E];
    {
        const bf16* qp = q + ((size_t)b * H + t) * D + E * sl;
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const bf16x8 x = *(const bf16x8*)(qp + 8 * u);
#pragma unroll
            for (int e = 0; e < 8; ++e) qv[8 * u + e] = (float)x[e] * scale_log2e;
        }
    }

    // Key rows of (b, t): row j at byte j * H * D * 2; rows past the cache
    // length read as zeros (never used).
    const size_t rs = (size_t)H * D;
    const bf16* kb = k + ((size_t)b * L * H + t) * D;
    const bf16* vb = v + ((size_t)b * L * H + t) * D;
    const uint32_t bytes = len > 0 ? (uint32_t)(((size_t)(len - 1) * rs + D) * 2) : 0u;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kb, bytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vb, bytes);

    DecState<D> st;
    st.m = -INFINITY;
    st.l = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) st.acc[e] = 0.0f;

    // Round r: this lane group's key k0 + 32 r + 8 wave + g.  K/V rows of the
    // next two rounds are in flight while a round is computed.
    const int n_rounds = k1 > k0 ? (k1 - k0 + 31) / 32 : 0;
    auto key_of = [&](int r) { return k0 + 32 * r + 8 * wave + g; };
    auto offset = [&](int r) {
        const int j = key_of(r);
        return j < k1 ? (uint32_t)(((size_t)j * rs + E * sl) * 2) : OOB_OFFSET;
    };
    bf16x8 kbuf[3][NL], vbuf[3][NL];
    auto fetch = [&](int r, int slot) {
        const uint32_t off = offset(r);
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            kbuf[slot][u] = buffer_load16(kr, off + 16 * u);
            vbuf[slot][u] = buffer_load16(vr, off + 16 * u);
        }
    };
    fetch(0, 0);
    fetch(1, 1);
    for (int r = 0; r < n_rounds; ++r) {
        const int slot = r % 3;
        fetch(r + 2, (r + 2) % 3);
        float sc = 0.0f;
#pragma unroll
        for (int u = 0; u < NL; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) sc = __builtin_fmaf(qv[8 * u + e], (float)kbuf[slot][u][e], sc);
        // the full dot product in all 8 lanes of the group
        sc += __shfl_xor(sc, 1);
        sc += __shfl_xor(sc, 2);
        sc += __shfl_xor(sc, 4);
        if (key_of(r) < k1) {  // the same in the 8 lanes of a group
            const float m = fmaxf(st.m, sc);
            const float alpha = __builtin_amdgcn_exp2f(st.m - m);  // 0 while empty
            const float p = __builtin_amdgcn_exp2f(sc - m);
            st.l = st.l * alpha + p;
#pragma unroll
            for (int u = 0; u < NL; ++u)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    st.acc[8 * u + e] =
                        __builtin_fmaf(p, (float)vbuf[slot][u][e], st.acc[8 * u + e] * alpha);
            st.m = m;
        }
    }

    // The 8 key groups of the wave (lanes sl, sl + 8, ..., same d slice),
    // then the 4 waves through LDS, merged in a fixed order.
#pragma unroll
    for (int x = 8; x < 64; x <<= 1) {
        const float m2 = __shfl_xor(st.m, x), l2 = __shfl_xor(st.l, x);
        float a2[E];
#pragma unroll
        for (int e = 0; e < E; ++e) a2[e] = __shfl_xor(st.acc[e], x);
        dec_merge<D>(st, m2, l2, a2);
    }
    if (lane < 8) {
#pragma unroll
        for (int e = 0; e < E; ++e) red[wave][E * sl + e] = st.acc[e];
        if (lane == 0) {
            red[wave][D] = st.m;
            red[wave][D + 1] = st.l;
        }
    }
    __syncthreads();
    if (wave == 0 && lane < 8) {
        for (int ww = 1; ww < DEC_WAVES; ++ww) dec_merge<D>(st, red[ww][D], red[ww][D + 1], &red[ww][E * sl]);
        float* out = part + (size_t)w * (D + 2);
#pragma unroll
        for (int e = 0; e < E; ++e) out[E * sl + e] = st.acc[e];
        if (lane == 0) {
            out[D] = st.m;
            out[D + 1] = st.l;
        }
    }
}

// o_b,t from the n_split partial states of (b, t): one wave per (b, t), lane
// e holding d elements e (and e + 64 for D = 128).  A sequence with no cached
// key outputs 0.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_bf16(const float* __restrict__ part,
                                                         bf16* __restrict__ o, int n_split) {
    constexpr int PER = D / 64;
    const int lane = threadIdx.x;
    const int bt = (int)blockIdx.x;
    const float* p = part + (size_t)bt * n_split * (D + 2);
    float mx = -INFINITY;
    for (int s = 0; s < n_split; ++s) mx = fmaxf(mx, p[(size_t)s * (D + 2) + D]);
    float l = 0.0f, acc[PER] = {};
    if (mx != -INFINITY) {
        for (int s = 0; s < n_split; ++s) {
            const float* ps = p + (size_t)s * (D + 2);
            const float sc = __builtin_amdgcn_exp2f(ps[D] - mx);  // 0 for an empty chunk
            l = __builtin_fmaf(ps[D + 1], sc, l);
#pragma unroll
            for (int c = 0; c < PER; ++c) acc[c] = __builtin_fmaf(ps[64 * c + lane], sc, acc[c]);
        }
    }
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
    for (int c = 0; c < PER; ++c) o[(size_t)bt * D + 64 * c + lane] = (bf16)(acc[c] * inv);
}

// Chunks per (sequence, head); at least one, so an empty cache still writes
// (zero) outputs.
int n_splits(int L) { return L > DEC_CHUNK ? (L + DEC_CHUNK - 1) / DEC_CHUNK : 1; }

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t stream) {
    const int n_split = n_splits(a.L);
    const float sl2e = (float)(1.4426950408889634 / sqrt((double)D));
    float* part = (float*)a.workspace;
    hipLaunchKernelGGL(decode_partial_bf16<D>, dim3((unsigned)((long)a.B * a.H * n_split)),
                       dim3(64 * DEC_WAVES), 0, stream, (const bf16*)a.q, (const bf16*)a.k,
                       (const bf16*)a.v, a.lens, part, a.H, a.L, n_split, sl2e);
    hipLaunchKernelGGL(decode_merge_bf16<D>, dim3((unsigned)((long)a.B * a.H)), dim3(64), 0,
                       stream, (const float*)part, (bf16*)a.o, n_split);
    return hipGetLastError();
}

}  // namespace

size_t decode_workspace_bytes(int B, int H, int L, int D) {
    return (size_t)B * H * n_splits(L) * (D + 2) * sizeof(float);
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
    return a.D == 128 ? launch_decode_d<128>(a, stream) : launch_decode_d<64>(a, stream);
}

}  // namespace mha
