// Multi-k cumulative calibration ("Top-Theta Attention: Sparsifying
// Transformers by Compensated Thresholding", Appendix D, Algorithm 2, Eq. 8).
//
// For every (head, row) MKC merges the sorted rows of all S calibration
// samples into kbar(theta), the mean effective k over the samples whose range
// (v_0, v_{m-1}] contains theta (a sample keeps #{v >= theta} elements), and
// returns theta(k) = max{theta : kbar(theta) >= k}, which is a sample value.
//
// Walking the pooled values of a (head, row) from the largest down, at a
// distinct value x with P = #{pooled >= x}, Mx = #{samples whose max >= x}
// and Nl = #{samples whose min >= x}:
//   the covering samples number C = Mx - Nl, and they keep T = P - m * Nl
//   elements in all (a sample above x keeps nothing, one entirely >= x keeps
//   all m), so kbar(x) >= k  <=>  C > 0 and T >= k * C.
// theta(k) is the value at the first such position.  The kernels therefore
//   1. compute each sample row's values (post-softmax, or the scores) and
//      its min and max (one workgroup per sample row, scores in LDS); for
//      bf16 the same pass counts them into step 3's first histogram;
//   2. sort each (head, row)'s sample maxima and minima (one workgroup each);
//   3. find a bound below which no theta of the (head, row) lies: the
//      highest boundary of a two-level histogram of the pooled keys at which
//      the condition holds for the largest target below m;
//   4. move the pooled values at or above the bound to the front of the
//      other buffer, and sort those in descending order: a stable LSD radix
//      sort of the order-preserving 32-bit keys, 8 bits per pass, spread over
//      workgroups of 4096 values (per pass: a histogram per chunk, a scan
//      per (head, row) into every chunk's output positions, then a stable
//      scatter of every chunk);
//   5. walk the sorted positions, chunk by chunk, each thread evaluating the
//      condition at its own positions with binary searches in the sorted
//      maxima and minima, and keep for every target k the smallest
//      qualifying position (a global atomic min); then read theta there.
// Integer counts and the sort make the result exact for the values computed:
// the same values give the same theta on any launch.
#include "topth_internal.h"

#include <math.h>
#include <limits.h>

#include <type_traits>

namespace topth {

constexpr int kMkcValThreads = 256;
constexpr int kMkcSelThreads = 1024;
constexpr int kMkcChunk = 4096;          // sorted values per workgroup of the sort passes
constexpr int kMkcWalkChunk = 2048;      // sorted positions per workgroup of the walk
constexpr int kMkcCompThreads = 1024;    // bound histograms and compaction: 32 values per thread
constexpr int kMkcCompItems = 32;
constexpr int kMkcCompChunk = kMkcCompThreads * kMkcCompItems;   // pooled values per workgroup there
// The sort passes and the walk loop over (chunk, segment) work items, chunk
// first, on at most this many workgroups: only the items below a segment's
// compacted count do work, and they come first.
constexpr int kMkcLoopGrid = 2048;
constexpr int kMkcMaxSamples = 4096;
constexpr int kMkcMaxTargets = 64;
constexpr int kMkcMaxKeys = 32768;

struct MkcArgs {
    const void* q; const void* k;
    int S, Hq, Hkv, Lq, Lk, q_pos0, n_rows, pre;
    float xscale;            // scale * log2(e): scores in the exp2 domain
    float scale;
    float* pool;             // [Hq][Lq] segments of S * m values (sample s at s * m)
    float* pool2;            // second buffer of the radix sort, same layout
    float* smin; float* smax;  // [Hq][Lq][S], ascending after mkc_sortmm_kernel
    int* hist;               // [Hq * Lq][256][wps]: counts per (digit, chunk), then output positions
    int* best;               // [Hq * Lq][n_k]: first qualifying sorted position per target
    unsigned* h1;            // [Hq * Lq][512]: pooled values per bin of the top 9 key bits
    unsigned* h2;            // [Hq * Lq][256]: those of the selected bin per bin of the next 8 bits
    int* sel;                // [Hq * Lq][2]: the selected top-9-bit bin (-1: none), values in the bins above it
    uint32_t* lb;            // [Hq * Lq]: key bound: every theta of the segment is at or above it, or -inf
    int* cnt;                // [Hq * Lq]: pooled values at or above lb, moved to the front of pool2
    int wps;                 // sort chunks per (head, row): ceil(S * m_max / kMkcChunk)
    int wpc;                 // chunks of the bound histograms and the compaction: ceil(S * m_max / kMkcCompChunk)
    int n_k;
    int ks[kMkcMaxTargets];
    float* theta;            // [n_k][Hq][n_rows]
};

// elements of the segments of rows 0..i-1 of one head, per sample
__host__ __device__ __forceinline__ long long mkc_row_prefix(int q_pos0, int i) {
    return (long long)i * (q_pos0 + 1) + (long long)i * (i - 1) / 2;
}

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float w = __shfl_xor(v, o);
        v = is_max ? fmaxf(v, w) : v + w;
    }
    const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    __syncthreads();                       // red may still be read by the previous reduction
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
    for (int w = 1; w < nw; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
    return r;
}

// ---------------------------------------------------------------- values
// One workgroup per (sample s, HPW query heads h0.. of one KV group, row i):
// the scores of keys 0..p of every head go to LDS (s_sc[u * m + j], exp2
// domain unless pre), then mkc_emit_rows writes each head's values to the
// pool with the row's min and max.

// after every score of the HPW heads is in s_sc: per head, the row max, the
// log-sum-exp and the values s_j = exp2(x_j - lse2) (or the scores), then
// the min and max of the written values
template <int HPW>
__device__ __forceinline__ void mkc_emit_rows(const MkcArgs& a, const float* s_sc, float* s_red, int s, int h0,
                                              int i, int m) {
    __syncthreads();                           // every score is in LDS
#pragma unroll 1
    for (int u = 0; u < HPW; ++u) {
        const int h = h0 + u;
        const float* sc = s_sc + u * m;
        float out_min = INFINITY, out_max = -INFINITY;
        float* dst = a.pool + (size_t)h * a.S * mkc_row_prefix(a.q_pos0, a.Lq) +
                     (size_t)a.S * mkc_row_prefix(a.q_pos0, i) + (size_t)s * m;
        if (a.pre) {
            for (int j = threadIdx.x; j < m; j += kMkcValThreads) {
                const float v = sc[j] + 0.0f;  // -0 becomes +0: one key per value
                dst[j] = v;
                out_min = fminf(out_min, v);
                out_max = fmaxf(out_max, v);
            }
        } else {
            float mx = -INFINITY;
            for (int j = threadIdx.x; j < m; j += kMkcValThreads) mx = fmaxf(mx, sc[j]);
            mx = block_reduce(mx, s_red, true);
            float l = 0.f;
            for (int j = threadIdx.x; j < m; j += kMkcValThreads) l += exp2f(sc[j] - mx);
            l = block_reduce(l, s_red, false);
            const float lse2 = mx + log2f(l);
            for (int j = threadIdx.x; j < m; j += kMkcValThreads) {
                const float v = exp2f(sc[j] - lse2);
                dst[j] = v;
                out_min = fminf(out_min, v);
                out_max = fmaxf(out_max, v);
            }
        }
        out_min = -block_reduce(-out_min, s_red, true);
        out_max = block_reduce(out_max, s_red, true);
        if (threadIdx.x == 0) {
            const size_t o = ((size_t)h * a.Lq + i) * a.S + s;
            a.smin[o] = out_min;
            a.smax[o] = out_max;
        }
    }
}

// (m, l) pairs of an online exp2 sum: l is relative to m; m = -inf: empty
__device__ __forceinline__ void mkc_lse_merge(float& m, float& l, float m2, float l2) {
    const float M = fmaxf(m, m2);
    if (M == -INFINITY) return;
    l = l * __builtin_amdgcn_exp2f(m - M) + l2 * __builtin_amdgcn_exp2f(m2 - M);
    m = M;
}

// As mkc_emit_rows, from statistics the lanes gathered while storing the
// scores (lane statistics of head u = 4 kq + r, kq = lane / 16): one merge
// per head, then one pass that writes every head's values.  The written
// minimum and maximum are the value function at the score minimum and
// maximum (it is monotone in the score).  The same pass counts the values
// into the bound's level-1 histogram (top 9 key bits), first in LDS, then
// one global add per nonzero bin: no separate pass over the pool for it.
template <int HPW>
__device__ __forceinline__ void mkc_emit_rows_stats(const MkcArgs& a, const float* s_sc, const float (&st_m)[4],
                                                    const float (&st_l)[4], const float (&st_n)[4], int s, int h0,
                                                    int i, int m) {
    constexpr int NW = kMkcValThreads / 64;
    __shared__ float s_pm[NW][16], s_pl[NW][16], s_pn[NW][16];
    __shared__ float s_off[16];                   // per head: lse2 (0 for pre)
    __shared__ unsigned s_h1[HPW * 512];          // per head: the bound's level-1 histogram of the values
    for (int b = threadIdx.x; b < HPW * 512; b += kMkcValThreads) s_h1[b] = 0u;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float mm = st_m[r], ll = st_l[r], nn = st_n[r];
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {        // the 16 lanes of the group
            const float m2 = __shfl_xor(mm, o), l2 = __shfl_xor(ll, o);
            mkc_lse_merge(mm, ll, m2, l2);
            nn = fminf(nn, __shfl_xor(nn, o));
        }
        const int u = 4 * kq + r;
        if (col == 0 && u < HPW) { s_pm[wave][u] = mm; s_pl[wave][u] = ll; s_pn[wave][u] = nn; }
    }
    __syncthreads();                              // every score is in LDS, every partial too
    if (threadIdx.x < HPW) {
        const int u = threadIdx.x;
        float mm = s_pm[0][u], ll = s_pl[0][u], nn = s_pn[0][u];
        for (int w = 1; w < NW; ++w) {
            mkc_lse_merge(mm, ll, s_pm[w][u], s_pl[w][u]);
            nn = fminf(nn, s_pn[w][u]);
        }
        float off = 0.f, vmin, vmax;
        if (a.pre) {
            vmin = nn + 0.0f;
            vmax = mm + 0.0f;
        } else {
            off = mm + log2f(ll);
            vmin = exp2f(nn - off);
            vmax = exp2f(mm - off);
        }
        s_off[u] = off;
        const size_t o = ((size_t)(h0 + u) * a.Lq + i) * a.S + s;
        a.smin[o] = vmin;
        a.smax[o] = vmax;
    }
    __syncthreads();
    // 16-byte stores where the row of every head starts 16-byte aligned
    // (m a multiple of 4 and the row's pool offset too), else 4-byte ones
    const float* dst0 = a.pool + (size_t)a.S * mkc_row_prefix(a.q_pos0, i) + (size_t)s * m;
    const bool vec = (m & 3) == 0 && (((uintptr_t)dst0 & 15u) == 0) &&
                     ((((size_t)a.S * mkc_row_prefix(a.q_pos0, a.Lq)) & 3u) == 0);
    const bool pre = a.pre != 0;
    auto val0 = [&](float x, float off) { return pre ? x + 0.0f : exp2f(x - off); };   // -0 becomes +0
#pragma unroll 1
    for (int u = 0; u < HPW; ++u) {
        const float* sc = s_sc + u * m;
        const float off = s_off[u];
        unsigned* const hu = s_h1 + u * 512;
        auto val = [&](float x, float o) {
            const float y = val0(x, o);
            atomicAdd(&hu[float_to_ordered(y) >> 23], 1u);
            return y;
        };
        float* dst = a.pool + (size_t)(h0 + u) * a.S * mkc_row_prefix(a.q_pos0, a.Lq) +
                     (size_t)a.S * mkc_row_prefix(a.q_pos0, i) + (size_t)s * m;
        // nontemporal stores: the pool is only read back by later kernels
        if (vec) {
            typedef float f32x4v __attribute__((ext_vector_type(4)));
            for (int j = 4 * threadIdx.x; j < m; j += 4 * kMkcValThreads) {
                const f32x4v x = *(const f32x4v*)(sc + j);
                const f32x4v y = {val(x[0], off), val(x[1], off), val(x[2], off), val(x[3], off)};
                __builtin_nontemporal_store(y, (f32x4v*)(dst + j));
            }
        } else {
            for (int j = threadIdx.x; j < m; j += kMkcValThreads) __builtin_nontemporal_store(val(sc[j], off), dst + j);
        }
    }
    // this sample's counts join the row's histogram (nonzero bins only)
    __syncthreads();
    for (int b = threadIdx.x; b < HPW * 512; b += kMkcValThreads) {
        const unsigned c = s_h1[b];
        if (c != 0u) atomicAdd(&a.h1[((size_t)(h0 + b / 512) * a.Lq + i) * 512 + (b % 512)], c);
    }
}

// float32: a group of lanes per key reads its K row in 16-byte chunks once
// for all HPW heads and reduces the HPW dot products across the group
template <int D, int HPW>
__global__ __launch_bounds__(kMkcValThreads) void mkc_values_f32_kernel(MkcArgs a) {
    extern __shared__ float s_sc[];            // [HPW][m]
    __shared__ float s_red[kMkcValThreads / 64];
    constexpr int EPC = 4;                     // floats per 16-byte chunk
    constexpr int LPR = D / EPC;               // lanes per key row
    constexpr int RPW = 64 / LPR;              // key rows per wave step
    const int nhb = a.Hq / HPW;                // head blocks
    const int row = blockIdx.x;                // ((s * nhb) + hb) * Lq + i
    const int i = row % a.Lq;
    const int hb = (row / a.Lq) % nhb;
    const int s = row / (a.Lq * nhb);
    const int g = a.Hq / a.Hkv;
    const int h0 = hb * HPW;                   // HPW divides g: one KV head
    const int m = a.q_pos0 + i + 1;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % LPR, grp = lane / LPR;
    const float mul = a.pre ? a.scale : a.xscale;

    const float* kg = (const float*)a.k + ((size_t)s * a.Hkv + h0 / g) * (size_t)a.Lk * D;
    float qf[HPW][EPC];
#pragma unroll
    for (int u = 0; u < HPW; ++u) {
        const float* qrow = (const float*)a.q + (((size_t)s * a.Hq + h0 + u) * a.Lq + i) * D;
        const u32x4 w = *(const u32x4*)(qrow + sub * EPC);
#pragma unroll
        for (int e = 0; e < EPC; ++e) qf[u][e] = __uint_as_float(w[e]);
    }
    for (int j0 = wave * RPW; j0 < m; j0 += (kMkcValThreads / 64) * RPW) {
        const int j = j0 + grp;
        float kf[EPC] = {0.f, 0.f, 0.f, 0.f};
        if (j < m) {
            const u32x4 w = *(const u32x4*)(kg + (size_t)j * D + sub * EPC);
#pragma unroll
            for (int e = 0; e < EPC; ++e) kf[e] = __uint_as_float(w[e]);
        }
#pragma unroll
        for (int u = 0; u < HPW; ++u) {
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < EPC; ++e) dot = fmaf(qf[u][e], kf[e], dot);
#pragma unroll
            for (int o = 1; o < LPR; o <<= 1) dot += __shfl_xor(dot, o);
            if (j < m && sub == 0) s_sc[u * m + j] = dot * mul;
        }
    }
    mkc_emit_rows<HPW>(a, s_sc, s_red, s, h0, i, m);
}

// bfloat16: v_mfma_f32_16x16x32_bf16 with the HPW query heads in the A
// operand's rows (rows past HPW are zero) and 16 keys in B's columns.  Every
// lane loads its B fragments (8 elements of one K row per k-step) straight
// from memory, kNtk key tiles at a time, so that 4 * kNtk (d = 128) 16-byte
// loads per lane are in flight before the MFMAs that consume them; lanes
// 0..15 (and 16..31 for HPW = 8) then hold 4 heads' scores of their key.
constexpr int kMkcNtk = 4;
template <int D, int HPW>
__global__ __launch_bounds__(kMkcValThreads) void mkc_values_bf16_kernel(MkcArgs a) {
    extern __shared__ __attribute__((aligned(16))) float s_sc[];   // [HPW][m]
    constexpr int ST = D / 32;                 // k-steps
    constexpr int NW = kMkcValThreads / 64;
    const int nhb = a.Hq / HPW;
    const int row = blockIdx.x;                // ((s * nhb) + hb) * Lq + i
    const int i = row % a.Lq;
    const int hb = (row / a.Lq) % nhb;
    const int s = row / (a.Lq * nhb);
    const int g = a.Hq / a.Hkv;
    const int h0 = hb * HPW;
    const int m = a.q_pos0 + i + 1;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, kq = lane >> 4;
    const float mul = a.pre ? a.scale : a.xscale;

    bf16x8 qa[ST];
    {
        const uint16_t* qrow = (const uint16_t*)a.q + (((size_t)s * a.Hq + h0 + min(col, HPW - 1)) * a.Lq + i) * D;
#pragma unroll
        for (int st = 0; st < ST; ++st) {
            u32x4 w = *(const u32x4*)(qrow + 32 * st + 8 * kq);
            if (col >= HPW) w = u32x4{0u, 0u, 0u, 0u};
            qa[st] = __builtin_bit_cast(bf16x8, w);
        }
    }
    const uint16_t* kg = (const uint16_t*)a.k + ((size_t)s * a.Hkv + h0 / g) * (size_t)a.Lk * D;
    // Each wave takes groups of kMkcNtk 16-key tiles, NW groups apart, with
    // the next group's loads in flight while the current one is scored (two
    // register buffers, the loop unrolled by two so that each is named at
    // compile time).  Keys past the row read its last key, so every load and
    // MFMA is issued unconditionally (a group past the row is scored but not
    // stored): a conditional exit inside the body would make the compiler
    // wait for every load in flight at the top of each trip.
    constexpr int GSTEP = NW * 16 * kMkcNtk;
    auto load = [&](u32x4 (&kb)[kMkcNtk][ST], int t0) {
#pragma unroll
        for (int tk = 0; tk < kMkcNtk; ++tk) {
            const int key = min(t0 + 16 * tk + col, m - 1);
#pragma unroll
            for (int st = 0; st < ST; ++st) kb[tk][st] = *(const u32x4*)(kg + (size_t)key * D + 32 * st + 8 * kq);
        }
    };
    // lane statistics of the scores it stores (head u = 4 kq + r): maximum,
    // sum of exp2 relative to it (online; not needed for pre), minimum
    float st_m[4], st_l[4], st_n[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) { st_m[r] = -INFINITY; st_l[r] = 0.f; st_n[r] = INFINITY; }
    const bool pre = a.pre != 0;
    auto score = [&](const u32x4 (&kb)[kMkcNtk][ST], int t0) {
#pragma unroll
        for (int tk = 0; tk < kMkcNtk; ++tk) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < ST; ++st)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[st], __builtin_bit_cast(bf16x8, kb[tk][st]), acc, 0,
                                                              0, 0);
            const int key = t0 + 16 * tk + col;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int u = 4 * kq + r;
                if (u < HPW && key < m) {
                    const float v = acc[r] * mul;
                    s_sc[u * m + key] = v;
                    const float nm = fmaxf(st_m[r], v);
                    if (!pre)
                        st_l[r] = st_l[r] * __builtin_amdgcn_exp2f(st_m[r] - nm) + __builtin_amdgcn_exp2f(v - nm);
                    st_m[r] = nm;
                    st_n[r] = fminf(st_n[r], v);
                }
            }
        }
    };
    u32x4 k0[kMkcNtk][ST], k1[kMkcNtk][ST];
    const int tw = wave * 16 * kMkcNtk;
    if (tw < m) load(k0, tw);
    for (int t0 = tw; t0 < m; t0 += 2 * GSTEP) {
        load(k1, t0 + GSTEP);
        score(k0, t0);
        load(k0, t0 + 2 * GSTEP);
        score(k1, t0 + GSTEP);
    }
    mkc_emit_rows_stats<HPW>(a, s_sc, st_m, st_l, st_n, s, h0, i, m);
}

// ---------------------------------------------------------------- select
// descending order of values = ascending order of these keys
__device__ __forceinline__ uint32_t mkc_key(float v) { return ~float_to_ordered(v); }

// ascending bitonic sort of n2 (a power of two) floats in LDS, all threads
__device__ void lds_bitonic_asc(float* x, int n2) {
    for (int size = 2; size <= n2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            __syncthreads();
            for (int t = threadIdx.x; t < n2 / 2; t += blockDim.x) {
                const int lo = 2 * t - (t & (stride - 1));
                const int hi = lo + stride;
                const bool up = (lo & size) == 0;
                const float u = x[lo], w = x[hi];
                if ((u > w) == up) { x[lo] = w; x[hi] = u; }
            }
        }
    }
    __syncthreads();
}

// number of entries >= v in an ascending array of n2 floats
__device__ __forceinline__ int count_ge(const float* x, int n2, float v) {
    int lo = 0, hi = n2;                       // first index with x >= v
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (x[mid] < v) lo = mid + 1; else hi = mid;
    }
    return n2 - lo;
}

// the pooled values of (head h, row i) = segment h * Lq + i: offset and count
struct MkcSeg { size_t off; int N; int m; int p; int h; };
__device__ __forceinline__ MkcSeg mkc_seg(const MkcArgs& a, int seg) {
    MkcSeg g;
    const int i = seg % a.Lq;
    g.h = seg / a.Lq;
    g.p = a.q_pos0 + i;
    g.m = g.p + 1;
    g.N = a.S * g.m;
    g.off = (size_t)g.h * a.S * mkc_row_prefix(a.q_pos0, a.Lq) + (size_t)a.S * mkc_row_prefix(a.q_pos0, i);
    return g;
}

// One workgroup per (head, row): its S sample maxima and minima, ascending.
__global__ __launch_bounds__(kMkcSelThreads) void mkc_sortmm_kernel(MkcArgs a) {
    __shared__ float s_x[kMkcMaxSamples];
    const int seg = blockIdx.x;
    int n2 = 1;
    while (n2 < a.S) n2 <<= 1;
    for (int which = 0; which < 2; ++which) {
        float* v = (which ? a.smax : a.smin) + (size_t)seg * a.S;
        __syncthreads();                       // s_x is free
        for (int c = threadIdx.x; c < n2; c += blockDim.x) s_x[c] = c < a.S ? v[c] : -INFINITY;
        lds_bitonic_asc(s_x, n2);              // the -inf padding sorts to the front
        for (int c = threadIdx.x; c < a.S; c += blockDim.x) v[c] = s_x[n2 - a.S + c];
    }
    // the segment's level-2 histogram and compaction count start at zero
    // (the level-1 histogram is cleared before the values kernel)
    for (int c = threadIdx.x; c < 256; c += blockDim.x) a.h2[(size_t)seg * 256 + c] = 0u;
    if (threadIdx.x == 0) a.cnt[seg] = 0;
}

// ---- the bound.  kp is the largest target below m (a target k >= m gives
// -inf).  The Eq. 8 condition for kp at a threshold x only uses P, Mx and Nl
// at x; between x and the smallest pooled value x' >= x lies no pooled value,
// no sample maximum and no minimum, so all three agree there.  If the
// condition holds at x it holds at x', so theta(kp) >= x' >= x, and theta(k)
// >= theta(kp) for every target k <= kp (the condition for kp implies it for
// smaller k).  The highest bin boundary of the pooled values at which the
// condition holds is therefore a bound below which no theta lies: taken
// first over bins of the top 9 bits of the order-preserving keys, then over
// the next 8 bits inside the bin above that boundary.
__device__ __forceinline__ int mkc_kp(const MkcArgs& a, int m) {
    int kp = 0;
    for (int t = 0; t < a.n_k; ++t)
        if (a.ks[t] < m) kp = max(kp, a.ks[t]);
    return kp;
}

// number of entries with key >= k in an ascending array of n floats
__device__ __forceinline__ int count_ge_key(const float* x, int n, uint32_t k) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (float_to_ordered(x[mid]) < k) lo = mid + 1; else hi = mid;
    }
    return n - lo;
}

// Bound, steps 1 and 3: the histogram of one chunk's pooled values by the top
// 9 key bits (LEVEL 1), or of those in the selected bin by the next 8 bits
// (LEVEL 2), added into the segment's counts.
template <int LEVEL>
__global__ __launch_bounds__(kMkcCompThreads) void mkc_phist_kernel(MkcArgs a) {
    // level 1: 16 copies of the histogram, one per lane % 16, 513 words apart
    // (distinct banks): the values crowd into few exponent bins, and lanes
    // adding to one LDS word in one instruction are serialised (level 2 bins
    // the mantissa of one exponent and keeps one copy)
    constexpr int NC = LEVEL == 1 ? 16 : 1, CS = 513;
    __shared__ unsigned s_h[NC * CS];
    const int seg = blockIdx.x / a.wpc, ck = blockIdx.x % a.wpc;
    const MkcSeg g = mkc_seg(a, seg);
    const int j0 = ck * kMkcCompChunk;
    const int sel = LEVEL == 2 ? a.sel[2 * seg] : 0;
    // the whole workgroup: past the segment, no target below m, or no bin selected
    if (j0 >= g.N || mkc_kp(a, g.m) == 0 || sel < 0) return;
    const int tid = threadIdx.x;
    constexpr int NB = LEVEL == 1 ? 512 : 256;
    for (int b = tid; b < NC * CS; b += kMkcCompThreads) s_h[b] = 0u;
    __syncthreads();
    const int end = min(g.N, j0 + kMkcCompChunk);
    const float* sp = a.pool + g.off;
    unsigned* const hc = s_h + (tid & (NC - 1)) * CS;
    float v[kMkcCompItems];
#pragma unroll
    for (int it = 0; it < kMkcCompItems; ++it) v[it] = sp[min(j0 + it * kMkcCompThreads + tid, end - 1)];
#pragma unroll
    for (int it = 0; it < kMkcCompItems; ++it) {
        if (j0 + it * kMkcCompThreads + tid >= end) continue;
        const uint32_t key = float_to_ordered(v[it]);
        if (LEVEL == 1) atomicAdd(&hc[key >> 23], 1u);
        else if ((key >> 23) == (uint32_t)sel) atomicAdd(&hc[(key >> 15) & 255u], 1u);
    }
    __syncthreads();
    unsigned* dst = LEVEL == 1 ? a.h1 + (size_t)seg * 512 : a.h2 + (size_t)seg * 256;
    for (int b = tid; b < NB; b += kMkcCompThreads) {
        unsigned c = 0u;
#pragma unroll
        for (int k = 0; k < NC; ++k) c += s_h[k * CS + b];
        if (c != 0u) atomicAdd(&dst[b], c);
    }
}

// Bound, steps 2 and 4: one workgroup per segment tests the condition at
// every bin boundary (thread t holds the BPT bins below the top NB - BPT t,
// so a prefix over the threads counts the values from the top down) and
// keeps the highest boundary where it holds.
template <int LEVEL>
__global__ __launch_bounds__(256) void mkc_decide_kernel(MkcArgs a) {
    constexpr int NB = LEVEL == 1 ? 512 : 256, BPT = NB / 256;
    __shared__ float s_max[kMkcMaxSamples], s_min[kMkcMaxSamples];
    __shared__ int s_w[4], s_best;
    const int seg = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const MkcSeg g = mkc_seg(a, seg);
    const int kp = mkc_kp(a, g.m);
    const int sel = LEVEL == 2 ? a.sel[2 * seg] : 0;
    if (kp == 0 || sel < 0) {                  // no bound: every pooled value is sorted
        if (tid == 0) {
            if (LEVEL == 1) a.sel[2 * seg] = -1;
            else a.lb[seg] = 0u;
        }
        return;
    }
    const int S = a.S;
    for (int c = tid; c < S; c += 256) {
        s_max[c] = a.smax[(size_t)seg * S + c];
        s_min[c] = a.smin[(size_t)seg * S + c];
    }
    if (tid == 0) s_best = -1;
    const unsigned* h = LEVEL == 1 ? a.h1 + (size_t)seg * 512 : a.h2 + (size_t)seg * 256;
    int cb[BPT], c = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) { cb[i] = (int)h[NB - 1 - BPT * tid - i]; c += cb[i]; }
    int incl = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int w = __shfl_up(incl, d);
        if (lane >= d) incl += w;
    }
    if (lane == 63) s_w[wave] = incl;
    __syncthreads();
    for (int w = 0; w < wave; ++w) incl += s_w[w];
    const long long above = LEVEL == 1 ? 0 : a.sel[2 * seg + 1];   // values in the bins above the selected one
    long long P = above + incl - c;            // values above this thread's bins
    int best = -1;
    long long best_above = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        const int b = NB - 1 - BPT * tid - i;
        P += cb[i];                            // values at or above boundary b
        const uint32_t key = LEVEL == 1 ? (uint32_t)b << 23 : ((uint32_t)sel << 23) | ((uint32_t)b << 15);
        const long long Mx = count_ge_key(s_max, S, key), Nl = count_ge_key(s_min, S, key);
        const long long C = Mx - Nl;
        if (best < 0 && C > 0 && P - (long long)g.m * Nl >= (long long)kp * C) {
            best = b;
            best_above = P - cb[i];
        }
    }
    if (best >= 0) atomicMax(&s_best, best);
    __syncthreads();
    const int b = s_best;
    if (LEVEL == 1) {
        if (tid == 0 && b < 0) a.sel[2 * seg] = -1;
        if (b >= 0 && best == b) {             // the thread that holds it
            a.sel[2 * seg] = b;
            a.sel[2 * seg + 1] = (int)best_above;
        }
    } else if (tid == 0) {
        // the selected bin's lower boundary holds the condition, so b >= 0
        a.lb[seg] = ((uint32_t)sel << 23) | ((uint32_t)max(b, 0) << 15);
    }
}

// The pooled values at or above the segment's bound, moved (in any order)
// to the front of the segment in pool2: per chunk of kMkcCompChunk values, one
// thread takes 32 of them, a prefix over the workgroup places its kept ones,
// and one atomic add on the segment's count reserves the workgroup's range.
__global__ __launch_bounds__(kMkcCompThreads) void mkc_compact_kernel(MkcArgs a) {
    __shared__ int s_w[kMkcCompThreads / 64];
    __shared__ int s_base;
    const int seg = blockIdx.x / a.wpc, ck = blockIdx.x % a.wpc;
    const MkcSeg g = mkc_seg(a, seg);
    const int j0 = ck * kMkcCompChunk;
    if (j0 >= g.N) return;                     // the whole workgroup: past the segment
    const int end = min(g.N, j0 + kMkcCompChunk);
    const uint32_t lb = a.lb[seg];
    const float* sp = a.pool + g.off;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float v[kMkcCompItems];
    uint32_t keep = 0u;
    int c = 0;
#pragma unroll
    for (int it = 0; it < kMkcCompItems; ++it) {
        const int j = j0 + it * kMkcCompThreads + tid;
        v[it] = sp[min(j, end - 1)];
        const bool k = j < end && float_to_ordered(v[it]) >= lb;
        keep |= (uint32_t)k << it;
        c += k ? 1 : 0;
    }
    int incl = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int w = __shfl_up(incl, d);
        if (lane >= d) incl += w;
    }
    if (lane == 63) s_w[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
    for (int w = 0; w < kMkcCompThreads / 64; ++w) {
        before += w < wave ? s_w[w] : 0;
        total += s_w[w];
    }
    if (tid == 0) s_base = total > 0 ? atomicAdd(&a.cnt[seg], total) : 0;
    __syncthreads();
    float* dp = a.pool2 + g.off + s_base + before + incl - c;
#pragma unroll
    for (int it = 0; it < kMkcCompItems; ++it)
        if ((keep >> it) & 1u) *dp++ = v[it];
}

// Sort pass, step 1: the 256-bin histogram of digit (key >> sh) & 255 of one
// chunk, to hist[(seg * 256 + digit) * wps + chunk]; the chunks past the
// segment's compacted count are skipped, and the scan reads none of them.
__global__ __launch_bounds__(256) void mkc_hist_kernel(MkcArgs a, const float* src, int sh) {
    __shared__ int s_h[256];
    const int nseg = a.Hq * a.Lq, items = a.wps * nseg;
    for (int w = blockIdx.x; w < items; w += gridDim.x) {
        const int ck = w / nseg, seg = w % nseg;
        const int n = a.cnt[seg];
        if (ck * kMkcChunk >= n) continue;     // the whole workgroup: no compacted value here
        const MkcSeg g = mkc_seg(a, seg);
        s_h[threadIdx.x] = 0;
        __syncthreads();
        const int end = min(n, (ck + 1) * kMkcChunk);
        const float* sp = src + g.off;
        // 8 loads in flight per thread (indices past the chunk read its last
        // value and are not counted)
        for (int j0 = ck * kMkcChunk + threadIdx.x; j0 < end; j0 += 256 * 8) {
            float v[8];
#pragma unroll
            for (int it = 0; it < 8; ++it) v[it] = sp[min(j0 + it * 256, end - 1)];
#pragma unroll
            for (int it = 0; it < 8; ++it)
                if (j0 + it * 256 < end) atomicAdd(&s_h[(mkc_key(v[it]) >> sh) & 255u], 1);
        }
        __syncthreads();
        a.hist[((size_t)seg * 256 + threadIdx.x) * a.wps + ck] = s_h[threadIdx.x];
        __syncthreads();                       // s_h is read before the next item clears it
    }
}

// Sort pass, step 2: exclusive scan of one segment's counts in (digit,
// chunk) order, in place: the first output position of every (digit, chunk).
__global__ __launch_bounds__(kMkcSelThreads) void mkc_scan_kernel(MkcArgs a) {
    __shared__ int s_w[kMkcSelThreads / 64];
    // only the chunks that hold compacted values have counts: entry f is
    // (digit f / act, chunk f % act)
    int* const xb = a.hist + (size_t)blockIdx.x * 256 * a.wps;
    const int act = (a.cnt[blockIdx.x] + kMkcChunk - 1) / kMkcChunk;
    const int n = 256 * act;
    auto x = [&](int f) -> int& { return xb[(size_t)(f / act) * a.wps + f % act]; };
    const int per = (n + kMkcSelThreads - 1) / kMkcSelThreads;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b0 = min(n, tid * per), b1 = min(n, b0 + per);
    int sum = 0;
    for (int j = b0; j < b1; ++j) sum += x(j);
    int incl = sum;                            // scan of the thread sums: wave, then across waves
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int w = __shfl_up(incl, o);
        if (lane >= o) incl += w;
    }
    if (lane == 63) s_w[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += s_w[w];
    int run = before + incl - sum;
    for (int j = b0; j < b1; ++j) { const int c = x(j); x(j) = run; run += c; }
}

// Sort pass, step 3: stable scatter of one chunk, in tiles of 4096 values
// (8 per thread).  Wave w owns the tile's values w * 512 .. w * 512 + 511
// and ranks them in index order, 64 at a time: lanes with equal digits find
// each other through a per-wave LDS lane mask per digit, and a per-wave LDS
// counter per digit carries the count of the earlier rounds.  A prefix over
// the waves and over the digits then gives every value its place in the tile
// sorted by digit; the tile is staged in LDS in that order and written out in
// order of place, so that each digit's run is written contiguously at the
// position the scan gave this chunk for that digit.
constexpr int kMkcScatThreads = 512;       // two workgroups per CU
constexpr int kMkcScatItems = 8;
constexpr int kMkcScatTile = kMkcScatThreads * kMkcScatItems;
__global__ __launch_bounds__(kMkcScatThreads, 4) void mkc_scatter_kernel(MkcArgs a, const float* src, float* dst,
                                                                         int sh) {
    constexpr int NW = kMkcScatThreads / 64;
    constexpr int PER_WAVE = 64 * kMkcScatItems;
    __shared__ int s_wc[NW][256];              // per-wave counts, then the wave's offset inside the digit
    __shared__ int s_base[256];                // next output position of each digit in this chunk
    __shared__ int s_start[256];               // first place of each digit in the sorted tile
    __shared__ int s_part[4];
    __shared__ float s_out[kMkcScatTile];
    __shared__ unsigned long long s_peer[NW][256];   // lanes per digit of the current round, zero between rounds
    const int nseg = a.Hq * a.Lq, items = a.wps * nseg;
    // one chunk of one segment (the whole workgroup returns where the chunk
    // holds no compacted value); the last tile ends at a barrier, so the next
    // item may set the LDS state up again at once
    auto item = [&](const int seg, const int ck) {
        if (ck * kMkcChunk >= a.cnt[seg]) return;
        const MkcSeg g = mkc_seg(a, seg);
        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
        if (tid < 256) s_base[tid] = a.hist[((size_t)seg * 256 + tid) * a.wps + ck];
        for (int t = tid; t < NW * 256; t += kMkcScatThreads) {
            (&s_wc[0][0])[t] = 0;
            (&s_peer[0][0])[t] = 0ull;
        }
        __syncthreads();
        const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        const int end = min(a.cnt[seg], (ck + 1) * kMkcChunk);
        const float* sp = src + g.off;
        // the next tile's values are loaded while this one is ranked and written;
        // the loads are unconditional (indices past the chunk read its last value,
        // which is never used) so that the wait before ranking counts only the
        // current tile's loads
        auto load_tile = [&](int t0, float (&v)[kMkcScatItems]) {
#pragma unroll
            for (int it = 0; it < kMkcScatItems; ++it) v[it] = sp[min(t0 + wave * PER_WAVE + it * 64 + lane, end - 1)];
        };
        float v[kMkcScatItems], nv[kMkcScatItems];
        if (ck * kMkcChunk < end) load_tile(ck * kMkcChunk, v);
        for (int t0 = ck * kMkcChunk; t0 < end; t0 += kMkcScatTile) {
            const int n = min(kMkcScatTile, end - t0);
            int rk[kMkcScatItems];
            load_tile(t0 + kMkcScatTile, nv);
#pragma unroll
            for (int it = 0; it < kMkcScatItems; ++it) {
                const bool valid = wave * PER_WAVE + it * 64 + lane < n;
                const int dg = (int)((mkc_key(v[it]) >> sh) & 255u);
                // the lanes of this round with the same digit: each sets its bit in
                // the wave's mask of that digit and reads the mask back; the first
                // of them then adds the round's count and clears the mask.  LDS
                // instructions of one wave execute in order, so every lane reads the
                // complete mask and the old count before that lane's writes.
                unsigned long long peers = 0ull;
                int before = 0;
                if (valid) {
                    atomicOr(&s_peer[wave][dg], 1ull << lane);
                    peers = s_peer[wave][dg];
                    before = s_wc[wave][dg];
                }
                const int r = __popcll(peers & lt);
                if (valid && r == 0) {
                    s_wc[wave][dg] = before + __popcll(peers);
                    s_peer[wave][dg] = 0ull;
                }
                rk[it] = before + r;
            }
            __syncthreads();
            int tot = 0;
            if (tid < 256) {                       // prefix over the waves, per digit
#pragma unroll
                for (int w = 0; w < NW; ++w) { const int c = s_wc[w][tid]; s_wc[w][tid] = tot; tot += c; }
            }
            // exclusive scan of the tile's digit counts: places of the digits
            int incl = tot;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int w = __shfl_up(incl, o);
                if (lane >= o) incl += w;
            }
            if (tid < 256 && lane == 63) s_part[wave] = incl;
            __syncthreads();
            if (tid < 256) {
                int before = 0;
                for (int w = 0; w < wave; ++w) before += s_part[w];
                s_start[tid] = before + incl - tot;
            }
            __syncthreads();
#pragma unroll
            for (int it = 0; it < kMkcScatItems; ++it)
                if (wave * PER_WAVE + it * 64 + lane < n) {
                    const int dg = (int)((mkc_key(v[it]) >> sh) & 255u);
                    s_out[s_start[dg] + s_wc[wave][dg] + rk[it]] = v[it];
                }
            __syncthreads();
#pragma unroll
            for (int it = 0; it < kMkcScatItems; ++it) {
                const int pl = it * kMkcScatThreads + tid;
                if (pl < n) {
                    const float x = s_out[pl];
                    const int d = (int)((mkc_key(x) >> sh) & 255u);
                    dst[g.off + s_base[d] + (pl - s_start[d])] = x;
                }
            }
            __syncthreads();
            if (tid < 256) {
                s_base[tid] += tot;
#pragma unroll
                for (int w = 0; w < NW; ++w) s_wc[w][tid] = 0;
            }
            __syncthreads();
#pragma unroll
            for (int it = 0; it < kMkcScatItems; ++it) v[it] = nv[it];
        }
    };
    for (int w = blockIdx.x; w < items; w += gridDim.x) item(w % nseg, w / nseg);
}

// The walk over one chunk of sorted positions: every position that ends a
// run of equal values is tested; the smallest qualifying one per target
// goes to best[seg][t].  Each thread visits its positions in increasing
// order, so its first hit for a target is its smallest: it records that one
// (an LDS atomic min) and stops testing the target; the workgroup then
// makes one global atomic min per target.
__global__ __launch_bounds__(256) void mkc_walk_kernel(MkcArgs a, const float* sorted, int wpw) {
    __shared__ float s_max[kMkcMaxSamples], s_min[kMkcMaxSamples];
    __shared__ int s_best[kMkcMaxTargets];
    const int nseg = a.Hq * a.Lq, items = wpw * nseg;
    for (int w = blockIdx.x; w < items; w += gridDim.x) {
    const int seg = w % nseg, ck = w / nseg;
    if (ck * kMkcWalkChunk >= a.cnt[seg]) continue;   // the whole workgroup: past the sorted values
    const MkcSeg g = mkc_seg(a, seg);
    const int S = a.S;
    for (int c = threadIdx.x; c < S; c += 256) {
        s_max[c] = a.smax[(size_t)seg * S + c];
        s_min[c] = a.smin[(size_t)seg * S + c];
    }
    for (int t = threadIdx.x; t < a.n_k; t += 256) s_best[t] = INT_MAX;
    __syncthreads();
    const float* x = sorted + g.off;
    const int N = a.cnt[seg];                  // the sorted values at or above the bound
    const int end = min(N, (ck + 1) * kMkcWalkChunk);
    const unsigned long long all = a.n_k == 64 ? ~0ull : ((1ull << a.n_k) - 1ull);
    unsigned long long done = 0ull;
    for (int j = ck * kMkcWalkChunk + threadIdx.x; j < end && done != all; j += 256) {
        const float v = x[j];
        if (j + 1 < N && x[j + 1] == v) continue;
        const int Mx = count_ge(s_max, S, v);
        const int Nl = count_ge(s_min, S, v);
        const long long C = (long long)Mx - Nl;
        if (C <= 0) continue;
        const long long T = (long long)(j + 1) - (long long)g.m * Nl;
        for (int t = 0; t < a.n_k; ++t)
            if (!((done >> t) & 1ull) && T >= (long long)a.ks[t] * C) {
                atomicMin(&s_best[t], j);
                done |= 1ull << t;
            }
    }
    __syncthreads();
    for (int t = threadIdx.x; t < a.n_k; t += 256)
        if (s_best[t] != INT_MAX) atomicMin(&a.best[(size_t)seg * a.n_k + t], s_best[t]);
    __syncthreads();   // s_max, s_min and s_best are set up again for the next item
    }
}

// theta at every target's first qualifying position (-inf where none)
__global__ void mkc_theta_kernel(MkcArgs a, const float* sorted) {
    const int seg = blockIdx.x;
    const MkcSeg g = mkc_seg(a, seg);
    if (g.p >= a.n_rows) return;
    for (int t = threadIdx.x; t < a.n_k; t += blockDim.x) {
        const int b = a.best[(size_t)seg * a.n_k + t];
        a.theta[((size_t)t * a.Hq + g.h) * a.n_rows + g.p] = b == INT_MAX ? -INFINITY : sorted[g.off + b];
    }
}

// ------------------------------------------------------------------ host side
// chunks per (head, row) for rows of at most m_max keys
static long long mkc_wps(int S, int m_max) { return ((long long)S * m_max + kMkcChunk - 1) / kMkcChunk; }
// chunks per (head, row) of the bound histograms and the compaction
static long long mkc_wpc(int S, int m_max) { return ((long long)S * m_max + kMkcCompChunk - 1) / kMkcCompChunk; }
// chunks per (head, row) of the walk
static long long mkc_wpw(int S, int m_max) { return ((long long)S * m_max + kMkcWalkChunk - 1) / kMkcWalkChunk; }

size_t mkc_ws_bytes(int S, int Hq, int Lq, int Lk) {
    const size_t seg = (size_t)S * Hq * Lq * Lk;          // bound of the pooled values
    const size_t nseg = (size_t)Hq * Lq;
    const size_t hist = nseg * 256 * (size_t)mkc_wps(S, Lk);
    return 2 * seg * sizeof(float) + 2 * nseg * S * sizeof(float) + hist * sizeof(int) +
           nseg * kMkcMaxTargets * sizeof(int) + nseg * (512 + 256 + 2 + 1 + 1) * sizeof(int) + 4096;
}

int mkc_max_samples() { return kMkcMaxSamples; }
int mkc_max_targets() { return kMkcMaxTargets; }
int mkc_max_keys() { return kMkcMaxKeys; }

template <typename T, int D, int HPW>
static int launch_values_hpw(const MkcArgs& a, hipStream_t s) {
    const void* fn = std::is_same<T, float>::value ? (const void*)mkc_values_f32_kernel<D, HPW>
                                                    : (const void*)mkc_values_bf16_kernel<D, HPW>;
    const int m_max = a.q_pos0 + a.Lq;
    const size_t smem = (size_t)HPW * m_max * sizeof(float);
    if (smem > 65536) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
    }
    const dim3 grid(a.S * (a.Hq / HPW) * a.Lq), block(kMkcValThreads);
    if (std::is_same<T, float>::value)
        hipLaunchKernelGGL((mkc_values_f32_kernel<D, HPW>), grid, block, smem, s, a);
    else
        hipLaunchKernelGGL((mkc_values_bf16_kernel<D, HPW>), grid, block, smem, s, a);
    return hipGetLastError();
}

// heads per workgroup: the largest power of two up to 8 that divides the
// group size and keeps HPW rows of scores within 128 KiB of LDS
template <typename T, int D>
static int launch_values(const MkcArgs& a, hipStream_t s) {
    const int g = a.Hq / a.Hkv;
    const long long m_max = a.q_pos0 + a.Lq;
    int hpw = 8;
    while (hpw > 1 && (g % hpw != 0 || hpw * m_max * 4 > 131072)) hpw >>= 1;
    switch (hpw) {
        case 8: return launch_values_hpw<T, D, 8>(a, s);
        case 4: return launch_values_hpw<T, D, 4>(a, s);
        case 2: return launch_values_hpw<T, D, 2>(a, s);
        default: return launch_values_hpw<T, D, 1>(a, s);
    }
}

int launch_calibrate_mkc(const CalibParams& p, int pre, float* theta, hipStream_t s) {
    MkcArgs a = {};
    a.q = p.q; a.k = p.k; a.S = p.S; a.Hq = p.Hq; a.Hkv = p.Hkv; a.Lq = p.Lq; a.Lk = p.Lk;
    a.q_pos0 = p.q_pos0; a.n_rows = p.n_rows; a.pre = pre;
    a.scale = p.scale; a.xscale = p.scale * kLog2e;
    const size_t seg = (size_t)p.S * p.Hq * mkc_row_prefix(p.q_pos0, p.Lq);
    char* ws = (char*)p.ws;
    a.pool = (float*)ws;
    a.pool2 = a.pool + seg;
    a.smin = a.pool2 + seg;
    a.smax = a.smin + (size_t)p.Hq * p.Lq * p.S;
    a.hist = (int*)(a.smax + (size_t)p.Hq * p.Lq * p.S);
    const long long wps = mkc_wps(p.S, p.q_pos0 + p.Lq);
    const long long nseg = (long long)p.Hq * p.Lq;
    const long long wpw = mkc_wpw(p.S, p.q_pos0 + p.Lq);
    if (wpw * nseg >= (1LL << 31)) return hipErrorInvalidValue;   // the item counts are int
    a.wps = (int)wps;
    a.wpc = (int)mkc_wpc(p.S, p.q_pos0 + p.Lq);
    a.best = a.hist + (size_t)nseg * 256 * (size_t)wps;
    a.h1 = (unsigned*)(a.best + (size_t)nseg * kMkcMaxTargets);
    a.h2 = a.h1 + (size_t)nseg * 512;
    a.sel = (int*)(a.h2 + (size_t)nseg * 256);
    a.lb = (uint32_t*)(a.sel + (size_t)nseg * 2);
    a.cnt = (int*)(a.lb + nseg);
    a.n_k = p.n_k;
    for (int t = 0; t < p.n_k; ++t) a.ks[t] = p.mkc_ks[t];
    a.theta = theta;
    int e = launch_fill_u32(a.h1, (size_t)nseg * 512 * sizeof(unsigned), 0u, s);   // the bf16 values kernel adds to it
    if (e != hipSuccess) return e;
    if (p.dtype == 1) e = p.d == 64 ? launch_values<uint16_t, 64>(a, s) : launch_values<uint16_t, 128>(a, s);
    else e = p.d == 64 ? launch_values<float, 64>(a, s) : launch_values<float, 128>(a, s);
    if (e != hipSuccess) return e;
    e = launch_fill_u32(a.best, (size_t)nseg * p.n_k * sizeof(int), (uint32_t)INT_MAX, s);
    if (e != hipSuccess) return e;
    // the sort passes and the walk loop over (chunk, segment) items, chunk
    // major, on a grid of at most kMkcLoopGrid workgroups: the chunks that
    // hold compacted values are the first ones of every segment
    const unsigned nseg_u = (unsigned)nseg;
    const unsigned nwg = (unsigned)std::min<long long>(wps * nseg, kMkcLoopGrid);
    const unsigned nww = (unsigned)std::min<long long>(wpw * nseg, kMkcLoopGrid);
    hipLaunchKernelGGL(mkc_sortmm_kernel, dim3(nseg_u), dim3(kMkcSelThreads), 0, s, a);
    const unsigned nwc = (unsigned)(a.wpc * nseg);
    if (p.dtype != 1)                          // the bf16 values kernel counted level 1 itself
        hipLaunchKernelGGL(mkc_phist_kernel<1>, dim3(nwc), dim3(kMkcCompThreads), 0, s, a);
    hipLaunchKernelGGL(mkc_decide_kernel<1>, dim3(nseg_u), dim3(256), 0, s, a);
    hipLaunchKernelGGL(mkc_phist_kernel<2>, dim3(nwc), dim3(kMkcCompThreads), 0, s, a);
    hipLaunchKernelGGL(mkc_decide_kernel<2>, dim3(nseg_u), dim3(256), 0, s, a);
    hipLaunchKernelGGL(mkc_compact_kernel, dim3(nwc), dim3(kMkcCompThreads), 0, s, a);
    // four passes of 8 bits over the compacted values; after them they are
    // back in pool2, descending
    float* src = a.pool2;
    float* dst = a.pool;
    for (int sh = 0; sh < 32; sh += 8) {
        hipLaunchKernelGGL(mkc_hist_kernel, dim3(nwg), dim3(256), 0, s, a, (const float*)src, sh);
        hipLaunchKernelGGL(mkc_scan_kernel, dim3(nseg_u), dim3(kMkcSelThreads), 0, s, a);
        hipLaunchKernelGGL(mkc_scatter_kernel, dim3(nwg), dim3(kMkcScatThreads), 0, s, a, (const float*)src, dst, sh);
        float* t = src; src = dst; dst = t;
    }
    hipLaunchKernelGGL(mkc_walk_kernel, dim3(nww), dim3(256), 0, s, a, (const float*)src, (int)wpw);
    hipLaunchKernelGGL(mkc_theta_kernel, dim3(nseg_u), dim3(64), 0, s, a, (const float*)src);
    return hipGetLastError();
}

}  // namespace topth
