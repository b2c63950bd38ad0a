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
// workgroups (split-K): each streams one chunk of one sequence's cache, whole
// key rows (every head of a position is contiguous in the cache, so a wave
// reads one row as one contiguous block; per-head pieces of 128 bytes at the
// row stride ran at a sixth of the rate), and leaves a partial softmax state
// per head (running max m, sum l, unnormalised acc); a second kernel merges a
// (sequence, head)'s partial states in a fixed order (deterministic), the
// exact identity softmax(x) = softmax(x - c) applied chunk by chunk.
//
// Arithmetic is fp32 on the VALU: the scores stay in fp32 (no bf16 rounding
// of p), and exp2 with log2(e) / sqrt(d_k) folded into q.
#include <atomic>

#include "device.h"
#include "launch.h"

namespace mha {
namespace {

// Keys per workgroup and waves per workgroup: each wave streams every
// DEC_WAVES-th key of its chunk (128 keys), two rows ahead.  A workgroup's
// rate is bound by the bytes it has in flight, so eight waves per chunk of
// 1024 keys beat four per chunk of 512 on mixed cache lengths (fewer partial
// tail chunks, the same waves per key) and on short caches, and tie on full
// ones; chunks of 256 to 2048 keys at four or eight waves were measured.
constexpr int DEC_CHUNK = 1024;
constexpr int DEC_WAVES = 8;

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

// Partial states of (sequence b, chunk s) for heads t0 .. t0 + 8 HPL - 1
// (t0 = 8 HPL blockIdx.y), into part[((b H + t) S + s) (D + 2) ..]:
// acc[0 .. D-1], m, l.
//
// A cached key's row holds all H heads contiguously (H * D * 2 bytes), so a
// wave reads whole rows (or, past 8 HPL heads, a contiguous 8 HPL-head
// slice of them): lane group g (8 lanes) takes heads t0 + g, t0 + g + 8,
// ... (HPL of them), lane sl of the group d elements E sl .. E sl + E - 1.
// Wave w streams keys k0 + w, k0 + w + DEC_WAVES, ... of the chunk, two
// rows ahead.
template <int D, int HPL>
__global__ __launch_bounds__(64 * DEC_WAVES) void decode_partial_bf16(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const int32_t* __restrict__ lens, float* __restrict__ part, int H, int L, int n_split,
    float scale_log2e) {
    constexpr int E = D / 8;            // elements per lane
    constexpr int NL = E / 8;           // 16-byte loads per lane per head row
    static_assert(D == 64 || D == 128, "head size");
    __shared__ float red[DEC_WAVES][8 * HPL][D + 2];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 3;            // lane group: heads g + 8u
    const int sl = lane & 7;            // d slice
    const int w = (int)blockIdx.x;
    const int s = w % n_split;
    const int b = w / n_split;
    const int t0 = 8 * HPL * (int)blockIdx.y;

    const int len = min(max(lens[b], 0), L);
    const int k0 = s * DEC_CHUNK;
    const int k1 = min(k0 + DEC_CHUNK, len);

    // q slices of this lane's heads, pre-scaled to log2 units (heads past H
    // read zeros and are never stored)
    float qv[HPL][E];
#pragma unroll
    for (int u = 0; u < HPL; ++u) {
        const int t = t0 + g + 8 * u;
        const bf16* qp = q + ((size_t)b * H + min(t, H - 1)) * D + E * sl;
#pragma unroll
        for (int c = 0; c < NL; ++c) {
            const bf16x8 x = *(const bf16x8*)(qp + 8 * c);
#pragma unroll
            for (int e = 0; e < 8; ++e) qv[u][8 * c + e] = t < H ? (float)x[e] * scale_log2e : 0.0f;
        }
    }

    // Rows of sequence b: key j at byte j * H * D * 2; rows at or past the
    // cache length read as zeros (never used).
    const size_t rs = (size_t)H * D;
    const bf16* kb = k + (size_t)b * L * rs;
    const bf16* vb = v + (size_t)b * L * rs;
    const uint32_t bytes = (uint32_t)((size_t)len * rs * 2);
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kb, bytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vb, bytes);

    DecState<D> st[HPL];
#pragma unroll
    for (int u = 0; u < HPL; ++u) {
        st[u].m = -INFINITY;
        st[u].l = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) st[u].acc[e] = 0.0f;
    }

    const int n_rounds = k1 > k0 ? (k1 - k0 - wave + DEC_WAVES - 1) / DEC_WAVES : 0;
    auto key_of = [&](int r) { return k0 + wave + DEC_WAVES * r; };
    bf16x8 kbuf[3][HPL][NL], vbuf[3][HPL][NL];
    auto fetch = [&](int r, int slot) {
        const int j = key_of(r);
        const bool in = r < n_rounds;
#pragma unroll
        for (int u = 0; u < HPL; ++u) {
            const int t = t0 + g + 8 * u;
            const uint32_t off = in && t < H ? (uint32_t)(((size_t)j * rs + (size_t)t * D + E * sl) * 2)
                                             : OOB_OFFSET;
#pragma unroll
            for (int c = 0; c < NL; ++c) {
                kbuf[slot][u][c] = buffer_load16(kr, off + 16 * c);
                vbuf[slot][u][c] = buffer_load16(vr, off + 16 * c);
            }
        }
    };
    auto round = [&](int slot) {
#pragma unroll
        for (int u = 0; u < HPL; ++u) {
            float sc = 0.0f;
#pragma unroll
            for (int c = 0; c < NL; ++c)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    sc = __builtin_fmaf(qv[u][8 * c + e], (float)kbuf[slot][u][c][e], sc);
            sc += __shfl_xor(sc, 1);  // the full dot product in the group's 8 lanes
            sc += __shfl_xor(sc, 2);
            sc += __shfl_xor(sc, 4);
            const float m = fmaxf(st[u].m, sc);
            const float alpha = __builtin_amdgcn_exp2f(st[u].m - m);  // 0 while empty
            const float p = __builtin_amdgcn_exp2f(sc - m);
            st[u].l = __builtin_fmaf(st[u].l, alpha, p);
#pragma unroll
            for (int c = 0; c < NL; ++c)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    st[u].acc[8 * c + e] =
                        __builtin_fmaf(p, (float)vbuf[slot][u][c][e], st[u].acc[8 * c + e] * alpha);
            st[u].m = m;
        }
    };
    // Rounds three at a time so the register slots are fixed.
    fetch(0, 0);
    fetch(1, 1);
    for (int r = 0; r < n_rounds; r += 3) {
        fetch(r + 2, 2);
        round(0);
        if (r + 1 >= n_rounds) break;
        fetch(r + 3, 0);
        round(1);
        if (r + 2 >= n_rounds) break;
        fetch(r + 4, 1);
        round(2);
    }

    // The waves' states through LDS, merged in a fixed order by wave 0.
#pragma unroll
    for (int u = 0; u < HPL; ++u) {
#pragma unroll
        for (int e = 0; e < E; ++e) red[wave][g + 8 * u][E * sl + e] = st[u].acc[e];
        if (sl == 0) {
            red[wave][g + 8 * u][D] = st[u].m;
            red[wave][g + 8 * u][D + 1] = st[u].l;
        }
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int u = 0; u < HPL; ++u) {
            const int tl = g + 8 * u;  // the head's slot in this workgroup
            const int t = t0 + tl;
            for (int ww = 1; ww < DEC_WAVES; ++ww)
                dec_merge<D>(st[u], red[ww][tl][D], red[ww][tl][D + 1], &red[ww][tl][E * sl]);
            if (t < H) {
                float* out = part + (((size_t)b * H + t) * n_split + s) * (D + 2);
#pragma unroll
                for (int e = 0; e < E; ++e) out[E * sl + e] = st[u].acc[e];
                if (sl == 0) {
                    out[D] = st[u].m;
                    out[D + 1] = st[u].l;
                }
            }
        }
    }
}

// o_b,t from the n_split partial states of (b, t): one wave per (b, t), lane
// e holding d elements e (and e + 64 for D = 128).  Lane s first reads chunk
// s's (m, l) (64 chunks per pass), so the maximum and the chunk weights take
// one memory round trip rather than one per chunk; the weighted sum then
// walks the chunks in order (a fixed order: deterministic), its loads issued
// eight chunks at a time.  A sequence with no cached key outputs 0.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_bf16(const float* __restrict__ part,
                                                         bf16* __restrict__ o, int n_split) {
    constexpr int PER = D / 64;
    const int lane = threadIdx.x;
    const int bt = (int)blockIdx.x;
    const float* p = part + (size_t)bt * n_split * (D + 2);
    float mx = -INFINITY;
    for (int s0 = 0; s0 < n_split; s0 += 64) {
        const int s = s0 + lane;
        mx = fmaxf(mx, s < n_split ? p[(size_t)s * (D + 2) + D] : -INFINITY);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float l = 0.0f, acc[PER] = {};
    if (mx != -INFINITY) {
        for (int s0 = 0; s0 < n_split; s0 += 64) {
            const int s = s0 + lane;
            const float* ps = p + (size_t)s * (D + 2);
            // this lane's chunk weight (0 for an empty chunk or past the end)
            const float sc = s < n_split ? __builtin_amdgcn_exp2f(ps[D] - mx) : 0.0f;
            l = s < n_split ? __builtin_fmaf(ps[D + 1], sc, l) : l;
            const int n = min(64, n_split - s0);
            for (int j0 = 0; j0 < n; j0 += 8) {
                float v[8][PER];
#pragma unroll
                for (int j = 0; j < 8; ++j)
#pragma unroll
                    for (int c = 0; c < PER; ++c)
                        v[j][c] = j0 + j < n ? p[(size_t)(s0 + j0 + j) * (D + 2) + 64 * c + lane]
                                             : 0.0f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float w = __shfl(sc, j0 + j);  // weight of chunk s0 + j0 + j
#pragma unroll
                    for (int c = 0; c < PER; ++c) acc[c] = __builtin_fmaf(v[j][c], w, acc[c]);
                }
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
    for (int c = 0; c < PER; ++c) o[(size_t)bt * D + 64 * c + lane] = (bf16)(acc[c] * inv);
}

// Chunks per sequence; at least one, so an empty cache still writes (zero)
// outputs.
int n_splits(int L) { return L > DEC_CHUNK ? (L + DEC_CHUNK - 1) / DEC_CHUNK : 1; }

// Heads per lane group: 8 groups cover 8 HPL heads per workgroup; above 32
// heads, further workgroups (grid axis y) take the next 32.
int heads_per_group(int H) { return H <= 8 ? 1 : (H <= 16 ? 2 : 4); }

template <int D, int HPL>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t stream) {
    const int n_split = n_splits(a.L);
    const float sl2e = (float)(1.4426950408889634 / sqrt((double)D));
    float* part = (float*)a.workspace;
    const unsigned head_groups = (unsigned)((a.H + 8 * HPL - 1) / (8 * HPL));
    hipLaunchKernelGGL((decode_partial_bf16<D, HPL>),
                       dim3((unsigned)((long)a.B * n_split), head_groups), dim3(64 * DEC_WAVES),
                       0, stream, (const bf16*)a.q, (const bf16*)a.k,
                       (const bf16*)a.v, a.lens, part, a.H, a.L, n_split, sl2e);
    hipLaunchKernelGGL(decode_merge_bf16<D>, dim3((unsigned)((long)a.B * a.H)), dim3(64), 0,
                       stream, (const float*)part, (bf16*)a.o, n_split);
    return hipGetLastError();
}

}  // namespace

size_t decode_workspace_bytes(int B, int H, int L, int D) {
    return (size_t)B * H * n_splits(L) * (D + 2) * sizeof(float);
}

long long decode_partial_workgroups(int B, int L) { return (long long)B * n_splits(L); }

// Scratch for callers that cannot allocate (mha_decode_noalloc): the fp32
// partial states of one call, DECODE_SCRATCH_BYTES at most.  Each device
// the library runs on holds its own copy until the process ends, and every
// call on that device shares it.  Nothing in it needs clearing: the
// partial-state kernel writes every state the merge reads.
static __device__ __align__(256) float scratch[DECODE_SCRATCH_BYTES / sizeof(float)];

// Device address of `scratch` on the stream's device, looked up with that
// device current on the first call there and kept per device (the array's
// host-side name is not a device address).  A lost race repeats the
// lookup, which returns the same address.
hipError_t decode_scratch(hipStream_t stream, void** ptr) {
    static std::atomic<void*> addr[64];
    int dev = 0;
    hipError_t e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    void* p = addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t back = (cur != dev) ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess) return e;
        if (back != hipSuccess) return back;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
    const int hpl = heads_per_group(a.H);
    if (a.D == 128) {
        if (hpl == 1) return launch_decode_d<128, 1>(a, stream);
        if (hpl == 2) return launch_decode_d<128, 2>(a, stream);
        return launch_decode_d<128, 4>(a, stream);
    }
    if (hpl == 1) return launch_decode_d<64, 1>(a, stream);
    if (hpl == 2) return launch_decode_d<64, 2>(a, stream);
    return launch_decode_d<64, 4>(a, stream);
}

}  // namespace mha
